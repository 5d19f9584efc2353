"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/specverify.h declares, sizes workspaces, and rejects
bad arguments before any HIP call (so no device is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

import lossless_draft_verification_amd as sv
from lossless_draft_verification_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(sv_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for expected in ("sv_verify_chain", "sv_verify_tree", "sv_row_stats", "sv_chain_workspace_bytes",
                     "sv_tree_workspace_bytes", "sv_row_stats_workspace_bytes", "sv_workspace_init",
                     "sv_status_string", "sv_abi_version", "sv_plan_budget", "sv_plan_workspace_bytes", "sv_compact_kv"):
        assert expected in names


def test_library_exports_every_declared_symbol():
    L = sv.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sv.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name


def test_version_and_status_strings():
    assert sv.abi_version() == 3
    assert sv.status_string(0) == "ok"
    assert "workspace" in sv.status_string(2)
    assert sv.status_string(99) == "unknown status"


def test_workspace_sizes():
    a = sv.chain_workspace_bytes(64, 7, 128256, sv.BF16)
    b = sv.chain_workspace_bytes(64, 7, 128256, sv.F32)
    assert a > 0 and b >= a  # fp32 rows have at least as many segments
    assert sv.chain_workspace_bytes(0, 7, 100, sv.F32) == 0
    assert sv.chain_workspace_bytes(1, 64, 100, sv.F32) == 0
    assert sv.chain_workspace_bytes(1, 3, 0, sv.F32) == 0
    assert sv.chain_workspace_bytes(1, 3, 100, 7) == 0
    assert sv.chain_workspace_bytes(sv.MAX_BATCH + 1, 3, 100, sv.F32) == 0
    assert sv.tree_workspace_bytes(48, 8, 128256, sv.F32) > 0
    assert sv.tree_workspace_bytes(1, 65, 10, sv.F32) == 0
    assert sv.row_stats_workspace_bytes(10, 1000, sv.BF16) > 0
    # monotone in batch
    assert sv.chain_workspace_bytes(128, 7, 128256, sv.BF16) > a


def _chain_desc(**kw):
    fake = 0x100000  # a host-side non-null stand-in; validation never dereferences it
    d = dict(batch=2, max_draft=3, vocab=100, logits_dtype=sv.F32, logits=fake, logits_row_stride=100,
             draft_kind=sv.DRAFT_PROBS, draft_probs=fake, q_row_stride=100, draft_ids=fake, temperature=fake,
             seed=fake, accept_len=fake, tokens=fake, req_status=None, p_draft=None, flags=0)
    d.update(kw)
    return _lib.ChainDesc(**d)


def _call_chain(desc, ws_bytes=1 << 30, ws=0x200000):
    return sv.lib().sv_verify_chain(ctypes.byref(desc) if desc is not None else None, ctypes.c_void_p(ws),
                                    ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 1), ("batch", sv.MAX_BATCH + 1, 1), ("max_draft", -1, 1), ("max_draft", 64, 1),
    ("vocab", 0, 1), ("logits_dtype", 5, 3), ("draft_kind", 9, 3), ("flags", 1 << 7, 3), ("flags", 256, 3),
    ("logits", None, 1), ("temperature", None, 1), ("seed", None, 1), ("accept_len", None, 1),
    ("tokens", None, 1), ("draft_ids", None, 1), ("logits_row_stride", 99, 1), ("draft_probs", None, 1),
    ("q_row_stride", 50, 1),
])
def test_chain_argument_validation(field, value, code):
    assert _call_chain(_chain_desc(**{field: value})) == code


def test_schedule_flags_are_exclusive():
    for f in (sv.FLAG_PHASED | sv.FLAG_FUSED, sv.FLAG_PHASED | sv.FLAG_FUSED | sv.FLAG_FP64_RACE,
              sv.FLAG_STATS_ONLY | sv.FLAG_DECIDE_ONLY, sv.FLAG_FUSED | sv.FLAG_STATS_ONLY,
              sv.FLAG_FUSED | sv.FLAG_DECIDE_ONLY):
        assert _call_chain(_chain_desc(flags=f)) == 1
        d = _tree_desc(flags=f)
        assert sv.lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(0x200000), ctypes.c_size_t(1 << 30), None) == 1


def test_block_rule_needs_the_phased_schedule_and_a_chain():
    assert _call_chain(_chain_desc(flags=sv.FLAG_BLOCK | sv.FLAG_FUSED)) == 3
    d = _tree_desc(flags=sv.FLAG_BLOCK)
    assert sv.lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(0x200000), ctypes.c_size_t(1 << 30), None) == 3


def test_filtering_needs_the_phased_schedule():
    fake = 0x300000
    assert _call_chain(_chain_desc(flags=sv.FLAG_FUSED, top_k=fake)) == 3
    assert _call_chain(_chain_desc(flags=sv.FLAG_FUSED, top_p=fake)) == 3
    for kw in (dict(top_k=fake), dict(top_p=fake)):
        d = _tree_desc(flags=sv.FLAG_FUSED, **kw)
        assert sv.lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(0x200000), ctypes.c_size_t(1 << 30), None) == 3


def test_filtered_workspace_holds_a_record_per_row():
    # the thresholds take 16 bytes per row of a chain call (rounded to 256)
    a = sv.chain_workspace_bytes(64, 7, 128256, sv.BF16)
    b = sv.chain_workspace_bytes(65, 7, 128256, sv.BF16)
    assert b > a


def test_chain_null_descriptor_and_workspace_checks():
    assert sv.lib().sv_verify_chain(None, ctypes.c_void_p(0x200000), ctypes.c_size_t(1 << 30), None) == 1
    assert _call_chain(_chain_desc(), ws=0) == 1
    need = sv.chain_workspace_bytes(2, 3, 100, sv.F32)
    assert _call_chain(_chain_desc(), ws_bytes=need - 1) == 2
    assert _call_chain(_chain_desc(), ws=0x200010) == 1  # workspace must be 256-byte aligned
    # one-hot drafts need no q
    assert _call_chain(_chain_desc(draft_kind=sv.DRAFT_ONEHOT, draft_probs=None), ws_bytes=need - 1) == 2
    # k = 0 needs no draft ids
    need0 = sv.chain_workspace_bytes(2, 0, 100, sv.F32)
    assert _call_chain(_chain_desc(max_draft=0, draft_ids=None, draft_probs=None), ws_bytes=need0 - 1) == 2


def _tree_desc(**kw):
    fake = 0x100000
    d = dict(batch=2, num_nodes=8, vocab=100, logits_dtype=sv.BF16, logits=fake, logits_row_stride=100,
             node_tokens=fake, parent=fake, temperature=fake, seed=fake, accept_len=fake, accept_path=fake,
             tokens=fake, req_status=None, flags=0)
    d.update(kw)
    return _lib.TreeDesc(**d)


@pytest.mark.parametrize("field,value,code", [
    ("num_nodes", 0, 1), ("num_nodes", 65, 1), ("parent", None, 1), ("node_tokens", None, 1),
    ("accept_path", None, 1), ("logits_dtype", 3, 3), ("logits_row_stride", 10, 1), ("flags", 128, 3),
])
def test_tree_argument_validation(field, value, code):
    d = _tree_desc(**{field: value})
    assert sv.lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(0x200000), ctypes.c_size_t(1 << 30), None) == code


def test_tree_workspace_too_small():
    d = _tree_desc()
    need = sv.tree_workspace_bytes(2, 8, 100, sv.BF16)
    assert sv.lib().sv_verify_tree(ctypes.byref(d), ctypes.c_void_p(0x200000), ctypes.c_size_t(need - 1), None) == 2


def test_row_stats_validation():
    L = sv.lib()
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    assert L.sv_row_stats(0, 10, sv.F32, fake, 10, fake, None, None, None, None, ws, 1 << 30, None) == 1
    assert L.sv_row_stats(4, 10, sv.F32, None, 10, fake, None, None, None, None, ws, 1 << 30, None) == 1
    assert L.sv_row_stats(4, 10, sv.F32, fake, 9, fake, None, None, None, None, ws, 1 << 30, None) == 1
    assert L.sv_row_stats(4, 10, 4, fake, 10, fake, None, None, None, None, ws, 1 << 30, None) == 3
    need = sv.row_stats_workspace_bytes(4, 10, sv.F32)
    assert L.sv_row_stats(4, 10, sv.F32, fake, 10, fake, None, None, None, None, ws, need - 1, None) == 2


def test_workspace_init_validation():
    L = sv.lib()
    assert L.sv_workspace_init(None, 100, None) == 1
    assert L.sv_workspace_init(ctypes.c_void_p(0x100000), 0, None) == 1
    assert L.sv_workspace_init(ctypes.c_void_p(0x100004), 64, None) == 1


def test_product_path_does_not_touch_the_oracle():
    """The package and the HIP sources never import, link or name the oracle."""
    pkg = os.path.join(ROOT, "lossless_draft_verification_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "svo_" not in text and "oracle/" not in text, f


def _plan_desc(**kw):
    fake = 0x100000
    d = dict(batch=4, max_steps=7, confidence=fake, num_steps=None, max_budget=28, cost=fake, base_tokens=4.0,
             budget=fake, draft_len=fake, rate=None, workspace=fake, workspace_bytes=1 << 20)
    d.update(kw)
    return _lib.PlanDesc(**d)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 1), ("max_steps", 0, 1), ("max_steps", 65, 1), ("max_budget", -1, 1), ("confidence", None, 1),
    ("cost", None, 1), ("budget", None, 1), ("draft_len", None, 1), ("batch", 1171, 3), ("workspace", None, 1),
    ("workspace", 0x100010, 1), ("workspace_bytes", 1024, 2),
])
def test_plan_argument_validation(field, value, code):
    d = _plan_desc(**{field: value})
    assert sv.lib().sv_plan_budget(ctypes.byref(d), None) == code
    assert sv.lib().sv_plan_budget(None, None) == 1


def test_plan_workspace_bytes():
    """One layout for every shape (a workspace serves calls of any shape)."""
    n = sv.plan_workspace_bytes(512, 7)
    assert n >= sv.PLAN_MAX_SLOTS * 8 and n % 256 == 0
    for shape in ((1, 1), (8192, 1), (1024, 8), (3, 64)):
        assert sv.plan_workspace_bytes(*shape) == n
    for bad in ((0, 7), (4, 0), (4, 65), (1171, 7)):
        assert sv.plan_workspace_bytes(*bad) == 0


def _compact_desc(**kw):
    fake = 0x100000
    d = dict(batch=2, num_nodes=8, accept_len=fake, accept_path=fake, node_slot=fake, kv=fake, num_layers=4,
             num_slots=100, slot_stride=4096, layer_stride=409600, row_bytes=4096, moved=None)
    d.update(kw)
    return _lib.CompactDesc(**d)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 1), ("num_nodes", 65, 1), ("num_layers", 0, 1), ("num_slots", 0, 1), ("row_bytes", 8, 1),
    ("accept_len", None, 1), ("accept_path", None, 1), ("node_slot", None, 1), ("kv", None, 1),
    ("row_bytes", 4100, 3), ("slot_stride", 4104, 3), ("kv", 0x100008, 3), ("slot_stride", 2048, 1),
    ("layer_stride", 4096, 1),
])
def test_compact_argument_validation(field, value, code):
    d = _compact_desc(**{field: value})
    assert sv.lib().sv_compact_kv(ctypes.byref(d), None) == code
    assert sv.lib().sv_compact_kv(None, None) == 1


def test_noalloc_entry_point_rejects_before_any_hip_call():
    """sv_verify_chain_noalloc checks the descriptor and the scratch's limits
    on the host first: no device is touched for a bad call."""
    L = sv.lib()
    assert L.sv_verify_chain_noalloc(None, None) == _lib.ERR_INVALID_ARGUMENT
    d = _chain_desc(batch=sv.SCRATCH_MAX_BATCH + 1)
    assert L.sv_verify_chain_noalloc(ctypes.byref(d), None) == _lib.ERR_WORKSPACE_TOO_SMALL
    d = _chain_desc(batch=64, max_draft=0, vocab=1 << 24, logits_row_stride=1 << 24, draft_kind=sv.DRAFT_ONEHOT,
                    draft_probs=None, draft_ids=None)
    assert L.sv_verify_chain_noalloc(ctypes.byref(d), None) == _lib.ERR_WORKSPACE_TOO_SMALL
    d = _chain_desc(vocab=0)
    assert L.sv_verify_chain_noalloc(ctypes.byref(d), None) == _lib.ERR_INVALID_ARGUMENT


def test_stream_read_rejects_bad_arguments_before_any_hip_call():
    L = sv.lib()
    fake = ctypes.c_void_p(0x100000)
    assert L.sv_stream_read(None, 1024, fake, 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sv_stream_read(fake, 1000 + 4, fake, 4, None) == _lib.ERR_INVALID_ARGUMENT   # not a multiple of 16
    assert L.sv_stream_read(ctypes.c_void_p(0x100008), 1024, fake, 4, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sv_stream_read(fake, 1024, fake, 0, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sv_stream_read(fake, 1024, None, 4, None) == _lib.ERR_INVALID_ARGUMENT
