"""CPU checks of the C ABI: the library loads, exports every function sd.h
declares, and rejects invalid arguments on the host before any launch.

Every call below carries at least one argument the host validation rejects,
so no kernel is ever launched (the argument checks run before any HIP call).
The validation cases only run where no GPU is visible, so a validation bug can
never send the fake pointers used here to a real device.
"""
import ctypes
import os
import re

import pytest
import torch

import long_context_kv_split_amd as sd
from long_context_kv_split_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sd.h")

no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="host-validation cases run only where no GPU is visible")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from long_context_kv_split_amd.build import build
        build()
    return sd.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sd_status|size_t|const char \*|int32_t|double)\s*\*?\s*(sd_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    assert names == sorted(binding._SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
    assert sd.version() == 223
    for code in range(5):
        assert sd.status_string(code).startswith("SD_")
    assert "UNKNOWN" in sd.status_string(99)


def test_workspace_sizes_are_host_only_and_consistent(L):
    v = sd.sd_verify_attn_workspace_size(128, 5, 32, 8, 128, 32768)
    assert v > 0 and v % 256 == 0
    # partial outputs stay a small fraction of the 17.2 GB of KV this shape reads
    assert v < 0.03 * 128 * 32768 * 8 * 128 * 2 * 2
    assert sd.sd_verify_attn_workspace_size(0, 5, 32, 8, 128, 32768) == 0
    assert sd.sd_verify_attn_workspace_size(2, 4, 9, 2, 64, 256) == 0   # Hq % Hkv != 0
    assert sd.sd_draft_attn_sparse_workspace_size(32, 1, 32, 8, 128, 512) > 0
    s = sd.sd_snapkv_select_workspace_size(128, 32, 32, 8, 32768)
    assert s >= 2 * 128 * 8 * 32768 * 4          # votes + pooled values
    assert sd.sd_snapkv_select_workspace_size(1, 0, 32, 8, 100) == 0
    a = sd.sd_spec_accept_workspace_size(64, 4, 128256)
    assert a > 0 and sd.sd_spec_accept_workspace_size(64, -1, 10) == 0


def _kv(**over):
    s = binding.sd_kv_cache()
    s.k_pages = 0x1000
    s.v_pages = 0x2000
    s.page_table = 0x3000
    s.kv_lens = 0x4000
    s.num_pages, s.page_size, s.max_pages, s.num_kv_heads, s.head_dim = 10, 16, 4, 2, 128
    s.dtype = binding.SD_BF16
    for k, v in over.items():
        setattr(s, k, v)
    return s


FAKE = ctypes.c_void_p(0x5000)
WS = ctypes.c_void_p(0x6000)


@no_gpu
@pytest.mark.parametrize("over,args,want", [
    ({}, dict(q=None), sd.SD_ERR_INVALID_ARG),
    ({"k_pages": None}, {}, sd.SD_ERR_INVALID_ARG),
    ({"k_pages": 0x1008}, {}, sd.SD_ERR_INVALID_ARG),   # not 16-byte aligned
    ({"v_pages": 0x2002}, {}, sd.SD_ERR_INVALID_ARG),
    ({}, dict(q=ctypes.c_void_p(0x5004)), sd.SD_ERR_INVALID_ARG),
    ({}, dict(out=ctypes.c_void_p(0x5002)), sd.SD_ERR_INVALID_ARG),
    ({"head_dim": 96}, {}, sd.SD_ERR_UNSUPPORTED),
    ({"page_size": 8}, {}, sd.SD_ERR_UNSUPPORTED),
    ({"dtype": 7}, {}, sd.SD_ERR_UNSUPPORTED),
    ({"num_pages": 0}, {}, sd.SD_ERR_INVALID_ARG),
    ({}, dict(hq=9), sd.SD_ERR_INVALID_ARG),          # Hq % Hkv != 0
    ({}, dict(n_q=40), sd.SD_ERR_UNSUPPORTED),        # G * n_q > 64
    ({}, dict(batch=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(max_len=65), sd.SD_ERR_INVALID_ARG),    # > max_pages * page_size
    ({}, dict(ws=None), sd.SD_ERR_WORKSPACE),
    ({}, dict(ws_bytes=1), sd.SD_ERR_WORKSPACE),
    ({}, dict(scale=float("nan")), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=float("inf")), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=0.0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=-0.125), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=3e38), sd.SD_ERR_INVALID_ARG),     # scale * log2(e) overflows
    # batch * ceil(max_len / 16) steps would overflow the schedule's int32 prefix sums
    ({"max_pages": 4096}, dict(batch=1 << 20, max_len=1 << 16), sd.SD_ERR_UNSUPPORTED),
])
def test_verify_rejects_invalid_arguments(L, over, args, want):
    kv = _kv(**over)
    a = dict(q=FAKE, batch=2, n_q=4, hq=8, max_len=64, scale=1.0, out=FAKE, ws=WS, ws_bytes=1 << 30)
    a.update(args)
    st = L.sd_verify_attn(ctypes.byref(kv), a["q"], a["batch"], a["n_q"], a["hq"], a["max_len"],
                          a["scale"], a["out"], None, a["ws"], a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(idx=None), sd.SD_ERR_INVALID_ARG),
    (dict(idx_heads=3), sd.SD_ERR_INVALID_ARG),
    (dict(idx_heads=4), sd.SD_ERR_INVALID_ARG),       # neither 1, Hkv = 2 nor Hq = 8
    (dict(max_sel=0), sd.SD_ERR_INVALID_ARG),
    (dict(ws_bytes=0), sd.SD_ERR_WORKSPACE),
])
def test_draft_rejects_invalid_arguments(L, args, want):
    kv = _kv()
    a = dict(idx=FAKE, idx_heads=1, max_sel=64, ws_bytes=1 << 30)
    a.update(args)
    st = L.sd_draft_attn_sparse(ctypes.byref(kv), FAKE, 2, 1, 8, a["idx"], FAKE, a["idx_heads"],
                                a["max_sel"], 1.0, FAKE, None, WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(lens=None), sd.SD_ERR_INVALID_ARG),
    (dict(sink=-1), sd.SD_ERR_INVALID_ARG),
    (dict(sink=0, recent=0), sd.SD_ERR_INVALID_ARG),
    (dict(batch=0), sd.SD_ERR_INVALID_ARG),
    (dict(sink=2**31 - 1, recent=2**31 - 1), sd.SD_ERR_UNSUPPORTED),
    (dict(sink=1 << 29, recent=1 << 29), sd.SD_ERR_UNSUPPORTED),
])
def test_streaming_rejects_invalid_arguments(L, args, want):
    a = dict(lens=FAKE, batch=2, sink=4, recent=8)
    a.update(args)
    assert L.sd_streaming_select(a["lens"], a["batch"], a["sink"], a["recent"], FAKE, FAKE, None) == want


@no_gpu
@pytest.mark.parametrize("over,args,want", [
    ({}, dict(budget=8), sd.SD_ERR_INVALID_ARG),      # budget <= window
    ({"k_pages": 0x1004}, {}, sd.SD_ERR_INVALID_ARG),   # not 16-byte aligned
    ({}, dict(q=ctypes.c_void_p(0x5008)), sd.SD_ERR_INVALID_ARG),
    ({}, dict(pool=4), sd.SD_ERR_INVALID_ARG),        # even pool kernel
    ({}, dict(pool=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(window=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(window=40, budget=64), sd.SD_ERR_UNSUPPORTED),  # G * window > 128
    ({"dtype": binding.SD_F32}, {}, sd.SD_ERR_UNSUPPORTED),
    ({}, dict(ws_bytes=16), sd.SD_ERR_WORKSPACE),
    ({}, dict(max_len=1000), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=float("nan")), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=float("inf")), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=0.0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=-1.0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(scale=3e38), sd.SD_ERR_INVALID_ARG),
])
def test_snapkv_rejects_invalid_arguments(L, over, args, want):
    kv = _kv(**over)
    a = dict(window=8, pool=7, budget=32, max_len=64, ws_bytes=1 << 30, scale=1.0)
    a.update(args)
    st = L.sd_snapkv_select(ctypes.byref(kv), a.get("q", FAKE), 2, a["window"], 8, a["pool"], a["budget"],
                            a["max_len"], a["scale"], FAKE, FAKE, WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(lse=None), sd.SD_ERR_INVALID_ARG),
    (dict(q=None), sd.SD_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(0x5008)), sd.SD_ERR_INVALID_ARG),
    (dict(window=0), sd.SD_ERR_INVALID_ARG),
    (dict(window=40), sd.SD_ERR_UNSUPPORTED),         # G * window > 128
    (dict(max_len=1000), sd.SD_ERR_INVALID_ARG),
    (dict(scale=0.0), sd.SD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), sd.SD_ERR_INVALID_ARG),
    (dict(ws_bytes=16), sd.SD_ERR_WORKSPACE),
])
def test_snapkv_window_lse_rejects_invalid_arguments(L, args, want):
    kv = _kv()
    a = dict(q=FAKE, lse=FAKE, window=8, max_len=64, ws_bytes=1 << 30, scale=1.0)
    a.update(args)
    st = L.sd_snapkv_window_lse(ctypes.byref(kv), a["q"], 2, a["window"], 8, a["max_len"], a["scale"], a["lse"],
                                WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(lse=None), sd.SD_ERR_INVALID_ARG),
    (dict(idx=None), sd.SD_ERR_INVALID_ARG),
    (dict(budget=8), sd.SD_ERR_INVALID_ARG),          # budget <= window
    (dict(pool=4), sd.SD_ERR_INVALID_ARG),
    (dict(window=40, budget=64), sd.SD_ERR_UNSUPPORTED),
    (dict(scale=-1.0), sd.SD_ERR_INVALID_ARG),
    (dict(ws_bytes=16), sd.SD_ERR_WORKSPACE),
])
def test_snapkv_select_lse_rejects_invalid_arguments(L, args, want):
    kv = _kv()
    a = dict(lse=FAKE, idx=FAKE, window=8, pool=7, budget=32, max_len=64, ws_bytes=1 << 30, scale=1.0)
    a.update(args)
    st = L.sd_snapkv_select_lse(ctypes.byref(kv), FAKE, a["lse"], 2, a["window"], 8, a["pool"], a["budget"],
                                a["max_len"], a["scale"], a["idx"], FAKE, WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("over,args,want", [
    ({}, dict(q=None), sd.SD_ERR_INVALID_ARG),
    ({}, dict(idx=None), sd.SD_ERR_INVALID_ARG),
    ({}, dict(budget=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(hq=9), sd.SD_ERR_INVALID_ARG),          # Hq % Hkv != 0
    ({}, dict(hq=34), sd.SD_ERR_UNSUPPORTED),         # G = 17 > 16
    ({"dtype": binding.SD_F32}, {}, sd.SD_ERR_UNSUPPORTED),
    ({}, dict(max_len=65), sd.SD_ERR_INVALID_ARG),    # > max_pages * page_size
    ({}, dict(ws_bytes=64), sd.SD_ERR_WORKSPACE),
    ({"max_pages": 4096}, dict(batch=1 << 20, max_len=1 << 16), sd.SD_ERR_UNSUPPORTED),
])
def test_topk_select_rejects_invalid_arguments(L, over, args, want):
    kv = _kv(**over)
    a = dict(q=FAKE, idx=FAKE, batch=2, hq=8, budget=16, max_len=64, ws_bytes=1 << 30)
    a.update(args)
    st = L.sd_topk_select(ctypes.byref(kv), a["q"], a["batch"], a["hq"], a["budget"], a["max_len"], a["idx"],
                          FAKE, WS, a["ws_bytes"], None)
    assert st == want


def test_topk_workspace_sizes():
    t = sd.sd_topk_select_workspace_size(128, 32, 8, 32768)
    assert t >= 128 * 32 * 32768 * 4 and t % 256 == 0   # one 32-bit key per (row, position)
    assert sd.sd_topk_select_workspace_size(2, 9, 2, 100) == 0
    assert sd.sd_topk_select_workspace_size(0, 8, 2, 100) == 0
    # the draft workspace also covers one unit per query head
    assert sd.sd_draft_attn_sparse_workspace_size(128, 1, 32, 8, 128, 2048) >= \
        sd.sd_verify_attn_workspace_size(128, 1, 32, 32, 128, 2048)


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(zt=None), sd.SD_ERR_INVALID_ARG),
    (dict(zd=None), sd.SD_ERR_INVALID_ARG),
    (dict(gamma=-1), sd.SD_ERR_INVALID_ARG),
    (dict(gamma=65), sd.SD_ERR_UNSUPPORTED),
    (dict(temp=0.0), sd.SD_ERR_INVALID_ARG),
    (dict(temp=float("inf")), sd.SD_ERR_INVALID_ARG),
    (dict(vocab=0), sd.SD_ERR_INVALID_ARG),
    (dict(ws_bytes=8), sd.SD_ERR_WORKSPACE),
    (dict(batch=1 << 28, gamma=8, vocab=1), sd.SD_ERR_UNSUPPORTED),
])
def test_accept_rejects_invalid_arguments(L, args, want):
    a = dict(zt=FAKE, zd=FAKE, batch=4, gamma=3, vocab=1000, temp=1.0, ws_bytes=1 << 30)
    a.update(args)
    st = L.sd_spec_accept(a["zt"], a["zd"], FAKE, FAKE, FAKE, a["batch"], a["gamma"], a["vocab"], a["temp"],
                          FAKE, FAKE, WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(zt=None), sd.SD_ERR_INVALID_ARG),
    (dict(gamma=65), sd.SD_ERR_UNSUPPORTED),
    (dict(temp=-1.0), sd.SD_ERR_INVALID_ARG),
    # needs more scratch than the library's fixed array holds
    (dict(batch=30000, gamma=4, vocab=1000), sd.SD_ERR_UNSUPPORTED),
    (dict(batch=64, gamma=4, vocab=1 << 24), sd.SD_ERR_UNSUPPORTED),
])
def test_accept_noalloc_rejects_invalid_arguments(L, args, want):
    """Host checks of the allocation-free entry point, including the scratch
    limit, all before any HIP call."""
    a = dict(zt=FAKE, batch=4, gamma=3, vocab=1000, temp=1.0)
    a.update(args)
    st = L.sd_spec_accept_noalloc(a["zt"], FAKE, FAKE, FAKE, FAKE, a["batch"], a["gamma"], a["vocab"],
                                  a["temp"], FAKE, FAKE, None)
    assert st == want


def test_accept_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SD_SPEC_ACCEPT_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.SD_SPEC_ACCEPT_SCRATCH_BYTES
    # the bench-shape acceptance fits; a batch well past it does not
    assert sd.sd_spec_accept_workspace_size(128, 4, 128256) <= binding.SD_SPEC_ACCEPT_SCRATCH_BYTES
    assert sd.sd_spec_accept_workspace_size(2500, 4, 128256) > binding.SD_SPEC_ACCEPT_SCRATCH_BYTES


def test_binding_refuses_host_tensors(L):
    k = torch.zeros((2, 1, 16, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sd.KVCache(k, k, torch.zeros((1, 2), dtype=torch.int32), torch.zeros(1, dtype=torch.int32))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "long_context_kv_split_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


@no_gpu
@pytest.mark.parametrize("args,want", [
    (dict(tail=None), sd.SD_ERR_INVALID_ARG),
    (dict(max_tail=-1), sd.SD_ERR_INVALID_ARG),
    (dict(max_tail=65), sd.SD_ERR_INVALID_ARG),   # > max_pages * page_size
    (dict(ws_bytes=0), sd.SD_ERR_WORKSPACE),
])
def test_draft_tail_rejects_invalid_arguments(L, args, want):
    kv = _kv()
    a = dict(tail=FAKE, max_tail=16, ws_bytes=1 << 30)
    a.update(args)
    st = L.sd_draft_attn_sparse_tail(ctypes.byref(kv), FAKE, 2, 1, 8, FAKE, FAKE, 1, 64, a["tail"],
                                     a["max_tail"], 1.0, FAKE, None, WS, a["ws_bytes"], None)
    assert st == want


@no_gpu
def test_append_and_advance_reject_invalid_arguments(L):
    kv = _kv()
    assert L.sd_kv_append(ctypes.byref(kv), None, FAKE, 2, 1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_append(ctypes.byref(kv), FAKE, FAKE, 0, 1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_append(ctypes.byref(kv), FAKE, FAKE, 2, -1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_append(ctypes.byref(kv), ctypes.c_void_p(0x5004), FAKE, 2, 1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_append(ctypes.byref(_kv(v_pages=None)), FAKE, FAKE, 2, 1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_append(ctypes.byref(kv), FAKE, FAKE, 2, 0, None) == sd.SD_OK  # nothing to write
    assert L.sd_kv_advance(None, None, 2, 1, None) == sd.SD_ERR_INVALID_ARG
    assert L.sd_kv_advance(FAKE, None, 0, 1, None) == sd.SD_ERR_INVALID_ARG


@no_gpu
@pytest.mark.parametrize("over,args,want", [
    ({}, dict(idx=None), sd.SD_ERR_INVALID_ARG),
    ({}, dict(sel_lens=None), sd.SD_ERR_INVALID_ARG),
    ({}, dict(k_out=None), sd.SD_ERR_INVALID_ARG),
    ({}, dict(v_out=ctypes.c_void_p(0x7004)), sd.SD_ERR_INVALID_ARG),   # not 16-byte aligned
    ({"v_pages": None}, {}, sd.SD_ERR_INVALID_ARG),
    ({}, dict(batch=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(max_sel=0), sd.SD_ERR_INVALID_ARG),
    ({}, dict(idx_heads=3), sd.SD_ERR_INVALID_ARG),        # neither 1 nor num_kv_heads
    ({}, dict(max_sel=33, pps=2), sd.SD_ERR_INVALID_ARG),  # 33 entries need 3 pages of 16
    ({}, dict(pps=1 << 26), sd.SD_ERR_UNSUPPORTED),        # 2^32 compact rows
    ({"head_dim": 96}, {}, sd.SD_ERR_UNSUPPORTED),
])
def test_kv_compact_rejects_invalid_arguments(L, over, args, want):
    kv = _kv(**over)
    a = dict(idx=FAKE, sel_lens=FAKE, batch=2, idx_heads=1, max_sel=32, pps=2, k_out=ctypes.c_void_p(0x7000),
             v_out=ctypes.c_void_p(0x8000))
    a.update(args)
    st = L.sd_kv_compact(ctypes.byref(kv), a["idx"], a["sel_lens"], a["batch"], a["idx_heads"], a["max_sel"],
                         a["pps"], a["k_out"], a["v_out"], None)
    assert st == want


@no_gpu
def test_snapkv_budgets_rejects_missing_budgets(L):
    kv = _kv()
    st = L.sd_snapkv_select_budgets(ctypes.byref(kv), FAKE, 2, 8, 8, 7, None, 64, 64, 1.0, FAKE, FAKE, WS,
                                    1 << 30, None)
    assert st == sd.SD_ERR_INVALID_ARG
    st = L.sd_snapkv_select_budgets(ctypes.byref(kv), FAKE, 2, 8, 8, 7, FAKE, 8, 64, 1.0, FAKE, FAKE, WS,
                                    1 << 30, None)
    assert st == sd.SD_ERR_INVALID_ARG  # max_budget <= window


@no_gpu
@pytest.mark.parametrize("args", [
    dict(buf=None),
    dict(checksum=None),
    dict(nbytes=0),
    dict(nbytes=24),                 # not a multiple of 16
    dict(buf=0x5008),                # not 16-byte aligned
    dict(nontemporal=2),
    dict(nontemporal=-1),
    dict(blocks=-1),
    dict(blocks=65537),
])
def test_read_probe_rejects_invalid_arguments(L, args):
    a = dict(buf=FAKE, nbytes=1 << 20, nontemporal=1, blocks=0, checksum=FAKE)
    a.update(args)
    buf = ctypes.c_void_p(a["buf"]) if isinstance(a["buf"], int) else a["buf"]
    st = L.sd_hbm_read_probe(buf, a["nbytes"], a["nontemporal"], a["blocks"], a["checksum"], None)
    assert st == sd.SD_ERR_INVALID_ARG
