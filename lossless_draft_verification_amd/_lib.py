"""ctypes binding of libspecverify (include/specverify.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
layout, their device pointers and the current HIP stream are passed to the C
ABI, and every step of the verification runs in the library's HIP kernels.
There is no fallback: if the library is not built or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

# sv_status
OK, ERR_INVALID_ARGUMENT, ERR_WORKSPACE_TOO_SMALL, ERR_UNSUPPORTED, ERR_LAUNCH = 0, 1, 2, 3, 4
# sv_dtype
F32, BF16 = 0, 1
# sv_draft_kind
DRAFT_PROBS, DRAFT_ONEHOT = 0, 1
# per-request status
REQ_OK, REQ_BAD_DRAFT_ID, REQ_BAD_TREE, REQ_NONFINITE, REQ_BAD_TEMPERATURE, REQ_INTERNAL = 0, 1, 2, 3, 4, 5
# flags
FLAG_PHASED, FLAG_FP64_RACE, FLAG_FUSED, FLAG_STATS_ONLY, FLAG_DECIDE_ONLY, FLAG_BLOCK, FLAG_KF_ROWS = 1, 2, 4, 8, 16, 32, 64

MAX_BATCH, MAX_DRAFT, MAX_NODES, MAX_VOCAB = 65536, 63, 64, 1 << 24
SCRATCH_BYTES, SCRATCH_MAX_BATCH = 8 << 20, 1024
PLAN_MAX_SLOTS = 8192

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t


class ChainDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("max_draft", _I32), ("vocab", _I32), ("logits_dtype", ctypes.c_int),
                ("logits", _P), ("logits_row_stride", _I64), ("draft_kind", ctypes.c_int),
                ("draft_probs", _P), ("q_row_stride", _I64), ("draft_ids", _P), ("temperature", _P),
                ("seed", _P), ("accept_len", _P), ("tokens", _P), ("req_status", _P), ("p_draft", _P),
                ("flags", _U32), ("top_k", _P), ("top_p", _P)]


class TreeDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("num_nodes", _I32), ("vocab", _I32), ("logits_dtype", ctypes.c_int),
                ("logits", _P), ("logits_row_stride", _I64), ("node_tokens", _P), ("parent", _P),
                ("temperature", _P), ("seed", _P), ("accept_len", _P), ("accept_path", _P), ("tokens", _P),
                ("req_status", _P), ("flags", _U32), ("top_k", _P), ("top_p", _P)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("max_steps", _I32), ("confidence", _P), ("num_steps", _P),
                ("max_budget", _I32), ("cost", _P), ("base_tokens", ctypes.c_double),
                ("budget", _P), ("draft_len", _P), ("rate", _P), ("workspace", _P), ("workspace_bytes", _SZ)]


class CompactDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("num_nodes", _I32), ("accept_len", _P), ("accept_path", _P), ("node_slot", _P),
                ("kv", _P), ("num_layers", _I32), ("num_slots", _I64), ("slot_stride", _I64),
                ("layer_stride", _I64), ("row_bytes", _I64), ("moved", _P)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (sv_status {status})")
        self.status = status


_lib = None
_lib_lock = threading.Lock()


def lib():
    """Load libspecverify.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
                L = ctypes.CDLL(LIB_PATH)
                L.sv_abi_version.restype = _I32
                L.sv_abi_version.argtypes = []
                L.sv_status_string.restype = ctypes.c_char_p
                L.sv_status_string.argtypes = [ctypes.c_int]
                L.sv_chain_workspace_bytes.restype = _SZ
                L.sv_chain_workspace_bytes.argtypes = [_I32, _I32, _I32, ctypes.c_int]
                L.sv_tree_workspace_bytes.restype = _SZ
                L.sv_tree_workspace_bytes.argtypes = [_I32, _I32, _I32, ctypes.c_int]
                L.sv_row_stats_workspace_bytes.restype = _SZ
                L.sv_row_stats_workspace_bytes.argtypes = [_I32, _I32, ctypes.c_int]
                L.sv_workspace_init.restype = ctypes.c_int
                L.sv_workspace_init.argtypes = [_P, _SZ, _P]
                L.sv_verify_chain.restype = ctypes.c_int
                L.sv_verify_chain.argtypes = [ctypes.POINTER(ChainDesc), _P, _SZ, _P]
                L.sv_verify_chain_noalloc.restype = ctypes.c_int
                L.sv_verify_chain_noalloc.argtypes = [ctypes.POINTER(ChainDesc), _P]
                L.sv_verify_tree.restype = ctypes.c_int
                L.sv_verify_tree.argtypes = [ctypes.POINTER(TreeDesc), _P, _SZ, _P]
                L.sv_compact_kv.restype = ctypes.c_int
                L.sv_compact_kv.argtypes = [ctypes.POINTER(CompactDesc), _P]
                L.sv_plan_budget.restype = ctypes.c_int
                L.sv_plan_budget.argtypes = [ctypes.POINTER(PlanDesc), _P]
                L.sv_plan_workspace_bytes.restype = _SZ
                L.sv_plan_workspace_bytes.argtypes = [_I32, _I32]
                L.sv_stream_read.restype = ctypes.c_int
                L.sv_stream_read.argtypes = [_P, _SZ, _P, _I32, _P]
                L.sv_row_stats.restype = ctypes.c_int
                L.sv_row_stats.argtypes = [_I32, _I32, ctypes.c_int, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]
                _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sv_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().sv_abi_version())


def chain_workspace_bytes(batch, max_draft, vocab, dtype) -> int:
    return int(lib().sv_chain_workspace_bytes(batch, max_draft, vocab, dtype))


def tree_workspace_bytes(batch, num_nodes, vocab, dtype) -> int:
    return int(lib().sv_tree_workspace_bytes(batch, num_nodes, vocab, dtype))


def row_stats_workspace_bytes(rows, vocab, dtype) -> int:
    return int(lib().sv_row_stats_workspace_bytes(rows, vocab, dtype))


# ------------------------------------------------------------------ workspace
class Workspace:
    """A device workspace (caller-owned memory for one stream at a time).

    Zero-filled once by the library's fill kernel when allocated; the library
    keeps it consistent from call to call.
    """

    def __init__(self, nbytes: int, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.nbytes = 0
        self.buf = None
        self.ensure(nbytes)

    def ensure(self, nbytes: int):
        if nbytes <= self.nbytes:
            return
        nbytes = max(int(nbytes), 1 << 20)
        # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-buf.data_ptr()) % 256
        self.buf = buf
        self.base = buf.data_ptr() + off
        self.nbytes = nbytes
        st = lib().sv_workspace_init(ctypes.c_void_p(self.base), ctypes.c_size_t(nbytes), _stream(self.device))
        if st != OK:
            raise SpecVerifyError(st, "sv_workspace_init")

    def reset(self):
        st = lib().sv_workspace_init(ctypes.c_void_p(self.base), ctypes.c_size_t(self.nbytes), _stream(self.device))
        if st != OK:
            raise SpecVerifyError(st, "sv_workspace_init")


_workspaces: dict = {}
_workspaces_lock = threading.Lock()


def default_workspace(device) -> Workspace:
    """The workspace used when a call passes none: one per (device, current
    stream), so calls on different streams never share scheduling counters
    or partial results.  A workspace only ever serves its own stream, so
    growing it (which returns the old buffer to torch's caching allocator)
    is ordered after every earlier call that used the old buffer.  If a call
    reports REQ_INTERNAL for a request, call reset() on the workspace it used
    (for the default one: default_workspace(device).reset(), on the same
    stream) before the next call."""
    device = torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(index).cuda_stream
    key = (index, stream)
    with _workspaces_lock:
        ws = _workspaces.get(key)
        if ws is None:
            ws = Workspace(1 << 20, torch.device("cuda", index))
            _workspaces[key] = ws
    return ws


_plan_workspaces = {}


def plan_workspace(device, nbytes: int) -> torch.Tensor:
    """The planner's workspace when a call passes none: one buffer per
    (device, current stream), grown to the largest call so far (its contents
    do not matter: each call writes what it reads)."""
    device = torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    with _workspaces_lock:
        ws = _plan_workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 1 << 16), dtype=torch.uint8, device=torch.device("cuda", index))
            _plan_workspaces[key] = ws
    return ws


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ------------------------------------------------------------------ checks
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _rows_view(t: torch.Tensor, lead: int):
    """Rows are indexed by the flattened first `lead` dims.  The library
    needs a contiguous last dim and one common row stride (>= V); other
    layouts are copied to a contiguous tensor.  Returns (tensor, row stride
    in elements)."""
    ok = t.stride(-1) == 1 and t.stride(lead - 1) >= t.shape[-1]
    for d in range(lead - 1):
        if t.shape[d] > 1 and t.stride(d) != t.stride(lead - 1) * _prod(t.shape[d + 1:lead]):
            ok = False
    if not ok:
        t = t.contiguous()
    return t, int(t.stride(lead - 1))


def _prod(xs):
    p = 1
    for x in xs:
        p *= int(x)
    return p


def _on(t: torch.Tensor, device, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.contiguous()


def _seed_tensor(seeds, bs, device):
    s = seeds
    if not torch.is_tensor(s):
        s = torch.as_tensor(s, dtype=torch.int64)
    if s.dtype == torch.uint64:
        s = s.view(torch.int64)
    if s.dtype != torch.int64:
        raise TypeError("seeds must be int64 (raw 64-bit keys) or uint64")
    if s.numel() != bs:
        raise ValueError("need one seed per request")
    return s.to(device).contiguous()


# ------------------------------------------------------------------ calls
def verify_chain(logits, draft_ids, temperature, seeds, draft_probs=None, onehot=False, *, flags=0,
                 return_p_draft=False, workspace=None, top_k=None, top_p=None):
    """Chain verification on the current stream (asynchronous).

    logits [bs, k+1, V] float32/bfloat16; draft_ids [bs, k] int32 (-1 ends a
    chain); temperature [bs] float32 (<= 0: greedy); seeds [bs] int64 (raw
    64-bit Philox keys); draft_probs [bs, k, V] float32, or onehot=True;
    top_k [bs] int32 / top_p [bs] float32 (or None): the stochastic requests'
    target is top-k / top-p filtered.
    Returns a dict of device tensors: accept_len [bs], tokens [bs, k+1],
    status [bs] (int32), and p_draft [bs, k] float64 if requested.
    """
    return _verify_chain(logits, draft_ids, temperature, seeds, draft_probs, onehot, flags, return_p_draft,
                         workspace, top_k, top_p, noalloc=False)


def verify_chain_noalloc(logits, draft_ids, temperature, seeds, draft_probs=None, onehot=False, *, flags=0,
                         return_p_draft=False, top_k=None, top_p=None):
    """verify_chain through sv_verify_chain_noalloc: the library's fixed
    per-GPU scratch array instead of a workspace (the C call allocates
    nothing; this wrapper still allocates the output tensors).  Calls on one
    GPU must not overlap in time."""
    return _verify_chain(logits, draft_ids, temperature, seeds, draft_probs, onehot, flags, return_p_draft,
                         None, top_k, top_p, noalloc=True)


def _verify_chain(logits, draft_ids, temperature, seeds, draft_probs, onehot, flags, return_p_draft, workspace,
                  top_k, top_p, noalloc):
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, k+1, vocab]")
    device = logits.device
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    bs, R, V = (int(x) for x in logits.shape)
    k = R - 1
    code = _dtype_code(logits)
    logits, lstride = _rows_view(logits, 2)
    ids = _on(draft_ids.reshape(bs, k) if k > 0 else torch.empty(bs, 0, dtype=torch.int32, device=device),
              device, torch.int32, "draft_ids")
    temp = _on(temperature.reshape(bs), device, torch.float32, "temperature")
    sd = _seed_tensor(seeds, bs, device)
    q = None
    qstride = 0
    if not onehot:
        if draft_probs is None:
            if k > 0:
                raise ValueError("draft_probs is required unless onehot=True")
        else:
            if tuple(draft_probs.shape) != (bs, k, V):
                raise ValueError("draft_probs must be [batch, k, vocab]")
            q = _on(draft_probs, device, torch.float32, "draft_probs")
            q, qstride = _rows_view(q, 2)
    out = dict(accept_len=torch.empty(bs, dtype=torch.int32, device=device),
               tokens=torch.empty(bs, R, dtype=torch.int32, device=device),
               status=torch.empty(bs, dtype=torch.int32, device=device))
    if return_p_draft:
        out["p_draft"] = torch.empty(bs, k, dtype=torch.float64, device=device)
    tk = None if top_k is None else _on(top_k.reshape(bs), device, torch.int32, "top_k")
    tp = None if top_p is None else _on(top_p.reshape(bs), device, torch.float32, "top_p")
    ws = None
    if not noalloc:
        need = chain_workspace_bytes(bs, k, V, code)
        if need == 0:
            raise SpecVerifyError(ERR_INVALID_ARGUMENT, "sv_chain_workspace_bytes")
        ws = workspace if workspace is not None else default_workspace(device)
        ws.ensure(need)
    d = ChainDesc(bs, k, V, code, logits.data_ptr(), lstride, DRAFT_ONEHOT if onehot else DRAFT_PROBS,
                  q.data_ptr() if q is not None else None, qstride, ids.data_ptr() if k > 0 else None,
                  temp.data_ptr(), sd.data_ptr(), out["accept_len"].data_ptr(), out["tokens"].data_ptr(),
                  out["status"].data_ptr(), out["p_draft"].data_ptr() if return_p_draft else None, int(flags),
                  tk.data_ptr() if tk is not None else None, tp.data_ptr() if tp is not None else None)
    if noalloc:
        st = lib().sv_verify_chain_noalloc(ctypes.byref(d), _stream(device))
        if st != OK:
            raise SpecVerifyError(st, "sv_verify_chain_noalloc")
        return out
    st = lib().sv_verify_chain(ctypes.byref(d), ctypes.c_void_p(ws.base), ctypes.c_size_t(ws.nbytes),
                               _stream(device))
    if st != OK:
        raise SpecVerifyError(st, "sv_verify_chain")
    return out


def verify_tree(logits, node_tokens, parent, temperature, seeds, *, flags=0, workspace=None, top_k=None,
                top_p=None):
    """Target-only tree verification on the current stream (asynchronous).

    logits [bs, N, V]; node_tokens, parent [bs, N] int32; top_k [bs] int32 /
    top_p [bs] float32 (or None) filter the stochastic requests' target.  Returns
    accept_len [bs], accept_path [bs, N], tokens [bs, N], status [bs].
    """
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, nodes, vocab]")
    device = logits.device
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    bs, N, V = (int(x) for x in logits.shape)
    code = _dtype_code(logits)
    logits, lstride = _rows_view(logits, 2)
    nt = _on(node_tokens.reshape(bs, N), device, torch.int32, "node_tokens")
    par = _on(parent.reshape(bs, N), device, torch.int32, "parent")
    temp = _on(temperature.reshape(bs), device, torch.float32, "temperature")
    sd = _seed_tensor(seeds, bs, device)
    out = dict(accept_len=torch.empty(bs, dtype=torch.int32, device=device),
               accept_path=torch.empty(bs, N, dtype=torch.int32, device=device),
               tokens=torch.empty(bs, N, dtype=torch.int32, device=device),
               status=torch.empty(bs, dtype=torch.int32, device=device))
    tk = None if top_k is None else _on(top_k.reshape(bs), device, torch.int32, "top_k")
    tp = None if top_p is None else _on(top_p.reshape(bs), device, torch.float32, "top_p")
    need = tree_workspace_bytes(bs, N, V, code)
    if need == 0:
        raise SpecVerifyError(ERR_INVALID_ARGUMENT, "sv_tree_workspace_bytes")
    ws = workspace if workspace is not None else default_workspace(device)
    ws.ensure(need)
    d = TreeDesc(bs, N, V, code, logits.data_ptr(), lstride, nt.data_ptr(), par.data_ptr(), temp.data_ptr(),
                 sd.data_ptr(), out["accept_len"].data_ptr(), out["accept_path"].data_ptr(),
                 out["tokens"].data_ptr(), out["status"].data_ptr(), int(flags),
                 tk.data_ptr() if tk is not None else None, tp.data_ptr() if tp is not None else None)
    st = lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(ws.base), ctypes.c_size_t(ws.nbytes),
                              _stream(device))
    if st != OK:
        raise SpecVerifyError(st, "sv_verify_tree")
    return out


def compact_kv(kv, accept_len, accept_path, node_slot):
    """Accepted-path KV compaction in place on the current stream.

    kv: device tensor [layers, slots, ...] (contiguous; each slot's trailing
    dimensions are one token's row); accept_len [bs] and accept_path [bs, N]
    int32 as verify_tree returns them; node_slot [bs, N] int64.  Returns
    moved [bs] int32 (rows moved per layer, -1: request left untouched).
    """
    if kv.dim() < 2 or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [layers, slots, ...] tensor")
    dev = kv.device
    L, S = kv.shape[0], kv.shape[1]
    row = kv[0, 0].numel() * kv.element_size()
    al = accept_len.to(device=dev, dtype=torch.int32).contiguous()
    ap = accept_path.to(device=dev, dtype=torch.int32).contiguous()
    ns = node_slot.to(device=dev, dtype=torch.int64).contiguous()
    bs, N = ap.shape
    if al.numel() != bs or ns.shape != ap.shape:
        raise ValueError("accept_len [bs], accept_path and node_slot [bs, N] expected")
    moved = torch.empty(bs, dtype=torch.int32, device=dev)
    d = CompactDesc(bs, N, al.data_ptr(), ap.data_ptr(), ns.data_ptr(), kv.data_ptr(), L, S, row, S * row, row,
                    moved.data_ptr())
    st = lib().sv_compact_kv(ctypes.byref(d), _stream(dev))
    if st != OK:
        raise SpecVerifyError(st, "sv_compact_kv")
    return moved


def plan_budget(confidence, cost, base_tokens, num_steps=None, workspace=None):
    """Survival top-k draft budget on the current stream (asynchronous).

    confidence [bs, K] float32; cost [max_budget + 1] float64 (step cost when
    B draft positions are verified); base_tokens: tokens a step yields with
    none; num_steps [bs] int32 or None; workspace: a uint8 device tensor of
    at least plan_workspace_bytes(bs, K) bytes, any contents (None: one kept
    per device and stream).  Returns device tensors: budget [1] int32, draft_len
    [bs] int32, rate [1] float64.
    """
    p = PreparedPlan(confidence, cost, base_tokens, num_steps, workspace)
    p.launch()
    return p.out


class PreparedPlan:
    """A survival top-k plan with its descriptor built once, for calling
    repeatedly on fixed device buffers.  launch() enqueues one sv_plan_budget
    on the current stream; outputs (self.out) are overwritten in place."""

    def __init__(self, confidence, cost, base_tokens, num_steps=None, workspace=None):
        if confidence.dim() != 2 or confidence.dtype != torch.float32:
            raise ValueError("confidence must be a [batch, K] float32 tensor")
        if cost.dim() != 1 or cost.dtype != torch.float64 or cost.numel() < 1:
            raise ValueError("cost must be a non-empty 1-D float64 tensor")
        dev = confidence.device
        self.conf = confidence.contiguous()
        self.cost = cost.to(dev).contiguous()
        bs, K = self.conf.shape
        self.ns = None
        if num_steps is not None:
            self.ns = num_steps.to(device=dev, dtype=torch.int32).contiguous()
            if self.ns.numel() != bs:
                raise ValueError("need one num_steps entry per request")
        self.out = dict(budget=torch.empty(1, dtype=torch.int32, device=dev),
                        draft_len=torch.empty(bs, dtype=torch.int32, device=dev),
                        rate=torch.empty(1, dtype=torch.float64, device=dev))
        need = int(lib().sv_plan_workspace_bytes(bs, K))
        self.ws = plan_workspace(dev, need) if workspace is None else workspace
        self.device = dev
        self.desc = PlanDesc(bs, K, self.conf.data_ptr(), self.ns.data_ptr() if self.ns is not None else None,
                             self.cost.numel() - 1, self.cost.data_ptr(), float(base_tokens),
                             self.out["budget"].data_ptr(), self.out["draft_len"].data_ptr(),
                             self.out["rate"].data_ptr(), self.ws.data_ptr(), self.ws.numel() * self.ws.element_size())
        self._ref = ctypes.byref(self.desc)
        self._fn = lib().sv_plan_budget

    def launch(self, stream=None):
        s = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream)
        st = self._fn(self._ref, s)
        if st != OK:
            raise SpecVerifyError(st, "sv_plan_budget")


def plan_workspace_bytes(batch: int, max_steps: int) -> int:
    return int(lib().sv_plan_workspace_bytes(int(batch), int(max_steps)))


def row_stats(logits, temperature, *, workspace=None):
    """Row statistics of a [rows, V] tensor with per-row temperature [rows].

    Returns row_max float32, row_argmax int32, row_sumexp float64 (NaN for
    greedy rows), row_status int32.
    """
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    device = logits.device
    if not logits.is_cuda:
        raise ValueError("logits must be a device tensor")
    rows, V = (int(x) for x in logits.shape)
    code = _dtype_code(logits)
    logits, lstride = _rows_view(logits, 1)
    temp = _on(temperature.reshape(rows), device, torch.float32, "temperature")
    out = dict(row_max=torch.empty(rows, dtype=torch.float32, device=device),
               row_argmax=torch.empty(rows, dtype=torch.int32, device=device),
               row_sumexp=torch.empty(rows, dtype=torch.float64, device=device),
               row_status=torch.empty(rows, dtype=torch.int32, device=device))
    need = row_stats_workspace_bytes(rows, V, code)
    if need == 0:
        raise SpecVerifyError(ERR_INVALID_ARGUMENT, "sv_row_stats_workspace_bytes")
    ws = workspace if workspace is not None else default_workspace(device)
    ws.ensure(need)
    st = lib().sv_row_stats(rows, V, code, ctypes.c_void_p(logits.data_ptr()), lstride,
                            ctypes.c_void_p(temp.data_ptr()), ctypes.c_void_p(out["row_max"].data_ptr()),
                            ctypes.c_void_p(out["row_argmax"].data_ptr()),
                            ctypes.c_void_p(out["row_sumexp"].data_ptr()),
                            ctypes.c_void_p(out["row_status"].data_ptr()), ctypes.c_void_p(ws.base),
                            ctypes.c_size_t(ws.nbytes), _stream(device))
    if st != OK:
        raise SpecVerifyError(st, "sv_row_stats")
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None):
    """Enqueue one sv_stream_read of the whole of `src` (a device tensor,
    16-byte aligned, a multiple of 16 bytes) into `sink` (uint32, at least
    `workgroups` entries): the read-bandwidth ceiling measurement."""
    s = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(src.device).cuda_stream)
    st = lib().sv_stream_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(src.numel() * src.element_size()),
                              ctypes.c_void_p(sink.data_ptr()), int(workgroups), s)
    if st != OK:
        raise SpecVerifyError(st, "sv_stream_read")


class PreparedTree:
    """A tree verification with its descriptor built once, for calling
    repeatedly on fixed device buffers.  launch() enqueues one sv_verify_tree
    on the current stream; outputs are overwritten in place."""

    def __init__(self, logits, node_tokens, parent, temperature, seeds, *, flags=0, workspace=None, top_k=None,
                 top_p=None):
        device = logits.device
        bs, N, V = (int(x) for x in logits.shape)
        code = _dtype_code(logits)
        self.logits, lstride = _rows_view(logits, 2)
        self.nt = _on(node_tokens.reshape(bs, N), device, torch.int32, "node_tokens")
        self.par = _on(parent.reshape(bs, N), device, torch.int32, "parent")
        self.temp = _on(temperature.reshape(bs), device, torch.float32, "temperature")
        self.seeds = _seed_tensor(seeds, bs, device)
        self.out = dict(accept_len=torch.empty(bs, dtype=torch.int32, device=device),
                        accept_path=torch.empty(bs, N, dtype=torch.int32, device=device),
                        tokens=torch.empty(bs, N, dtype=torch.int32, device=device),
                        status=torch.empty(bs, dtype=torch.int32, device=device))
        self.top_k = None if top_k is None else _on(top_k.reshape(bs), device, torch.int32, "top_k")
        self.top_p = None if top_p is None else _on(top_p.reshape(bs), device, torch.float32, "top_p")
        self.ws = workspace if workspace is not None else default_workspace(device)
        self.ws.ensure(tree_workspace_bytes(bs, N, V, code))
        self.device = device
        self.desc = TreeDesc(bs, N, V, code, self.logits.data_ptr(), lstride, self.nt.data_ptr(), self.par.data_ptr(),
                             self.temp.data_ptr(), self.seeds.data_ptr(), self.out["accept_len"].data_ptr(),
                             self.out["accept_path"].data_ptr(), self.out["tokens"].data_ptr(),
                             self.out["status"].data_ptr(), int(flags),
                             self.top_k.data_ptr() if self.top_k is not None else None,
                             self.top_p.data_ptr() if self.top_p is not None else None)
        self._fn = lib().sv_verify_tree
        self._phase_descs, self._phase_refs = [], {}

    def launch(self, stream=None, phase_flag=0):
        """Enqueue the call; phase_flag FLAG_STATS_ONLY or FLAG_DECIDE_ONLY
        enqueues only that phase."""
        s = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream)
        d = self.desc
        if phase_flag:
            ref = self._phase_refs.get(phase_flag)
            if ref is None:
                d2 = TreeDesc.from_buffer_copy(self.desc)
                d2.flags = int(self.desc.flags) | int(phase_flag)
                self._phase_descs.append(d2)
                ref = self._phase_refs[phase_flag] = ctypes.byref(d2)
        else:
            ref = ctypes.byref(d)
        st = self._fn(ref, ctypes.c_void_p(self.ws.base), ctypes.c_size_t(self.ws.nbytes), s)
        if st != OK:
            raise SpecVerifyError(st, "sv_verify_tree")


class PreparedChain:
    """A chain verification with its arguments checked and its descriptor
    built once, for calling repeatedly on fixed device buffers (benchmarks,
    serving loops).  launch() enqueues one sv_verify_chain on the current
    stream; outputs are overwritten in place."""

    def __init__(self, logits, draft_ids, temperature, seeds, draft_probs=None, onehot=False, *, flags=0,
                 workspace=None, top_k=None, top_p=None):
        device = logits.device
        bs, R, V = (int(x) for x in logits.shape)
        k = R - 1
        code = _dtype_code(logits)
        self.logits, lstride = _rows_view(logits, 2)
        self.ids = _on(draft_ids.reshape(bs, k), device, torch.int32, "draft_ids")
        self.temp = _on(temperature.reshape(bs), device, torch.float32, "temperature")
        self.seeds = _seed_tensor(seeds, bs, device)
        self.q, qstride = (None, 0)
        if not onehot:
            self.q, qstride = _rows_view(_on(draft_probs, device, torch.float32, "draft_probs"), 2)
        self.out = dict(accept_len=torch.empty(bs, dtype=torch.int32, device=device),
                        tokens=torch.empty(bs, R, dtype=torch.int32, device=device),
                        status=torch.empty(bs, dtype=torch.int32, device=device))
        self.top_k = None if top_k is None else _on(top_k.reshape(bs), device, torch.int32, "top_k")
        self.top_p = None if top_p is None else _on(top_p.reshape(bs), device, torch.float32, "top_p")
        self.ws = workspace if workspace is not None else default_workspace(device)
        self.ws.ensure(chain_workspace_bytes(bs, k, V, code))
        self.device = device
        self.desc = ChainDesc(bs, k, V, code, self.logits.data_ptr(), lstride,
                              DRAFT_ONEHOT if onehot else DRAFT_PROBS,
                              self.q.data_ptr() if self.q is not None else None, qstride,
                              self.ids.data_ptr() if k > 0 else None, self.temp.data_ptr(), self.seeds.data_ptr(),
                              self.out["accept_len"].data_ptr(), self.out["tokens"].data_ptr(),
                              self.out["status"].data_ptr(), None, int(flags),
                              self.top_k.data_ptr() if self.top_k is not None else None,
                              self.top_p.data_ptr() if self.top_p is not None else None)
        self._fn = lib().sv_verify_chain
        self._ref = ctypes.byref(self.desc)
        self._phase_descs, self._phase_refs = [], {}

    def launch(self, stream=None, phase_flag=0):
        """Enqueue the call; phase_flag FLAG_STATS_ONLY or FLAG_DECIDE_ONLY
        enqueues only that phase (the two, in that order on one stream,
        equal a plain launch)."""
        s = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream)
        ref = self._ref
        if phase_flag:
            ref = self._phase_refs.get(phase_flag)
            if ref is None:
                d = ChainDesc.from_buffer_copy(self.desc)
                d.flags = int(self.desc.flags) | int(phase_flag)
                self._phase_descs.append(d)
                ref = self._phase_refs[phase_flag] = ctypes.byref(d)
        st = self._fn(ref, ctypes.c_void_p(self.ws.base), ctypes.c_size_t(self.ws.nbytes), s)
        if st != OK:
            raise SpecVerifyError(st, "sv_verify_chain")
