// Accepted-path KV compaction after tree verification on gfx950 (page
// "投机解码", section "与调度、KV 的交互", sub-section "SGLang：按最坏情况预留，结束时归还";
// page "Draft sources: draft models, n-gram, suffix decoding", section
// "SGLang's suffix automaton, in tree").
//
// The accepted nodes p_1..p_a of a request (from the root down) hold their
// KV rows wherever the tree put them; for i = 1..a, in order, every layer's
// row at node_slot[p_i] moves to node_slot[i], so the accepted tokens follow
// the committed prefix contiguously (no copy when p_i = i).  Node ids grow
// along a path, so p_i >= i: a copy never reads a slot an earlier copy of
// the request wrote, but it may write the slot an earlier copy read (path
// 2, 3: node 2's slot is read by the first copy and written by the second).
//
// One workgroup per (request, layer, 8 KB piece of the row); each thread
// owns the same 16-byte words of the piece in every copy and does the
// request's copies in path order, kGroup at a time: first the group's loads,
// then its stores.  A copy never reads what an earlier copy wrote (its
// source node p_j > j >= the earlier destinations), and every load of a
// word precedes, in the thread's program order and through the data it
// feeds, the later stores to that word, so moving loads ahead within a
// group is safe.  The bytes moved are the whole cost: HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace svc {

constexpr int kThreads = 256;
constexpr int kWords = 2;                                 // 16-byte words per thread per piece
constexpr int kGroup = 4;                                 // copies whose loads are issued together
constexpr int64_t kPiece = (int64_t)kThreads * kWords * 16;  // bytes of a row per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CompactParams {
  int32_t bs, N, layers, pieces;
  const int32_t* accept_len;
  const int32_t* accept_path;
  const int64_t* node_slot;
  uint8_t* kv;
  int64_t num_slots, slot_stride, layer_stride, row_bytes;
  int32_t* moved;
};

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactParams P) {
  __shared__ int s_ok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t per_req = (int64_t)P.layers * P.pieces;
  const int b = (int)(blockIdx.x / per_req);
  const int rem = (int)(blockIdx.x - (int64_t)b * per_req);
  const int layer = rem / P.pieces, piece = rem - layer * P.pieces;
  const int N = P.N;
  const int len = P.accept_len[b];
  const int32_t* path = P.accept_path + (int64_t)b * N;
  const int64_t* slot = P.node_slot + (int64_t)b * N;
  if (tid < 64) {
    // lane i checks path entry i: node ids grow from i + 1 up, inside the
    // tree, and both slots of its copy lie in the pool
    bool bad = !(len >= 0 && len < N);
    if (!bad && lane < len) {
      const int p = path[lane];
      bad = p < lane + 1 || p >= N || (lane > 0 && p <= path[lane - 1]);
      if (!bad) {
        const int64_t s_src = slot[p], s_dst = slot[lane + 1];
        bad = s_src < 0 || s_src >= P.num_slots || s_dst < 0 || s_dst >= P.num_slots;
      }
    }
    const bool ok = __ballot(bad) == 0;
    if (lane == 0) s_ok = ok;
    if (lane == 0 && layer == 0 && piece == 0 && P.moved) {
      int moved = -1;
      if (ok) {
        moved = 0;
        for (int i = 0; i < len; ++i) moved += path[i] != i + 1;
      }
      P.moved[b] = moved;
    }
  }
  __syncthreads();
  if (!s_ok) return;
  uint8_t* base = P.kv + (int64_t)layer * P.layer_stride;
  const int64_t off0 = (int64_t)piece * kPiece;
  for (int i0 = 0; i0 < len; i0 += kGroup) {
    u32x4 w[kGroup][kWords];
    int src_node[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int i = i0 + g;
      src_node[g] = i < len ? path[i] : i + 1;
      if (src_node[g] == i + 1) continue;
      const uint8_t* src = base + slot[src_node[g]] * P.slot_stride;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const int64_t off = off0 + (int64_t)(k * kThreads + tid) * 16;
        if (off < P.row_bytes) w[g][k] = __builtin_nontemporal_load((const u32x4*)(src + off));
      }
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int i = i0 + g;
      if (src_node[g] == i + 1) continue;
      uint8_t* dst = base + slot[i + 1] * P.slot_stride;
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const int64_t off = off0 + (int64_t)(k * kThreads + tid) * 16;
        if (off < P.row_bytes) __builtin_nontemporal_store(w[g][k], (u32x4*)(dst + off));
      }
    }
  }
}

}  // namespace svc

extern "C" sv_status sv_compact_kv(const sv_compact_desc* d, void* stream) {
  if (d == nullptr) return SV_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->batch > SV_MAX_BATCH || d->num_nodes < 1 || d->num_nodes > SV_MAX_NODES ||
      d->num_layers < 1 || d->num_slots < 1 || d->row_bytes < 16)
    return SV_ERR_INVALID_ARGUMENT;
  if (d->accept_len == nullptr || d->accept_path == nullptr || d->node_slot == nullptr || d->kv == nullptr)
    return SV_ERR_INVALID_ARGUMENT;
  if ((d->row_bytes & 15) || (d->slot_stride & 15) || (d->layer_stride & 15) || ((uintptr_t)d->kv & 15))
    return SV_ERR_UNSUPPORTED;
  if (d->slot_stride < d->row_bytes || (d->num_layers > 1 && d->layer_stride < d->num_slots * d->slot_stride))
    return SV_ERR_INVALID_ARGUMENT;
  svc::CompactParams P;
  P.bs = d->batch;
  P.N = d->num_nodes;
  P.layers = d->num_layers;
  P.pieces = (int32_t)((d->row_bytes + svc::kPiece - 1) / svc::kPiece);
  P.accept_len = d->accept_len;
  P.accept_path = d->accept_path;
  P.node_slot = d->node_slot;
  P.kv = (uint8_t*)d->kv;
  P.num_slots = d->num_slots;
  P.slot_stride = d->slot_stride;
  P.layer_stride = d->layer_stride;
  P.row_bytes = d->row_bytes;
  P.moved = d->moved;
  const int64_t grid = (int64_t)P.bs * P.layers * P.pieces;
  if (grid > INT32_MAX) return SV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(svc::compact_kernel, dim3((unsigned)grid), dim3(svc::kThreads), 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
