"""Guard regions around every output and workspace: no kernel writes outside
the memory its call owns.

Each output tensor and each workspace is a view into a larger buffer whose
leading and trailing 16 KB hold a fixed bit pattern; the workspace view is
exactly the size the library asks for. After the call the guards must be
bit-for-bit unchanged. Shapes are ragged (lengths that end mid-page and mid
step, sequences at or under the draft budget, shuffled pages) so the last
tiles, segments and staged stores of every kernel are exercised. Values are
checked against the oracle by the parity tests; here only the footprint is.
"""
import math

import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
from synth import dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries
from tests.gpu_helpers import ensure_lib, say

pytestmark = pytest.mark.gpu
GUARD_BYTES = 16384
PATTERN = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


class Guarded:
    """A tensor of `shape` and `dtype` inside a byte buffer with guards on both sides."""

    def __init__(self, shape, dtype):
        self.nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((self.nbytes + 2 * GUARD_BYTES,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)

    def intact(self):
        g = self.buf.cpu().numpy()
        return bool((g[:GUARD_BYTES] == PATTERN).all() and (g[GUARD_BYTES + self.nbytes:] == PATTERN).all())


def guarded_ws(nbytes):
    return Guarded((max(1, int(nbytes)),), torch.uint8)


def check(**named):
    torch.cuda.synchronize()
    bad = [k for k, g in named.items() if not g.intact()]
    assert not bad, f"writes outside: {bad}"


LENS = [37, 300, 129, 16, 1000]


def cache(dtype, d, Hkv=2, lens=LENS, spike=0.0):
    return paged_kv(91, lens, Hkv, d, dtype, "cuda", shuffle=True, spike_frac=spike)


@pytest.mark.parametrize("dtype,d,Hq,Hkv,n_q", [
    (torch.bfloat16, 128, 8, 2, 4),   # 16 rows: one tile
    (torch.bfloat16, 128, 16, 2, 5),  # 40 rows: three tiles
    (torch.bfloat16, 64, 4, 2, 1),    # decode
    (torch.float32, 64, 8, 2, 3),
])
def test_verify_writes_only_its_outputs(dtype, d, Hq, Hkv, n_q):
    say(f"guards verify {dtype} d={d} Hq={Hq} n_q={n_q}")
    kv_t = cache(dtype, d, Hkv)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, L = len(LENS), max(LENS)
    q = queries(91, 1, (B, n_q, Hq, d), dtype, "cuda", scale=d ** -0.5)
    out, lse = Guarded((B, n_q, Hq, d), dtype), Guarded((B, n_q, Hq), torch.float32)
    ws = guarded_ws(sd.sd_verify_attn_workspace_size(B, n_q, Hq, Hkv, d, L))
    sd.sd_verify_attn(kv, q, n_q, Hq, L, 1.0, out.t, lse.t, ws.t)
    check(out=out, lse=lse, workspace=ws)


@pytest.mark.parametrize("tail", [False, True])
def test_streaming_select_and_draft_write_only_their_outputs(tail):
    say(f"guards streaming + draft tail={tail}")
    d, Hq, Hkv = 128, 8, 2
    kv_t = cache(torch.bfloat16, d, Hkv)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = len(LENS)
    sink, recent = 16, 48
    idx, sel = Guarded((B, 1, sink + recent), torch.int32), Guarded((B,), torch.int32)
    sd.sd_streaming_select(kv_t.kv_lens, sink, recent, idx.t, sel.t)
    check(idx=idx, sel_lens=sel)
    q = queries(91, 2, (B, 1, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    out, lse = Guarded((B, 1, Hq, d), torch.bfloat16), Guarded((B, 1, Hq), torch.float32)
    ws = guarded_ws(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, sink + recent))
    if tail:
        tb = torch.clamp(kv_t.kv_lens - 5, min=0).to(torch.int32)
        sd.sd_draft_attn_sparse_tail(kv, q, 1, Hq, idx.t, sel.t, 1, sink + recent, tb, 8, 1.0, out.t, lse.t,
                                     ws.t)
    else:
        sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx.t, sel.t, 1, sink + recent, 1.0, out.t, lse.t, ws.t)
    check(out=out, lse=lse, workspace=ws)


@pytest.mark.parametrize("per_sequence", [False, True])
def test_snapkv_and_its_draft_write_only_their_outputs(per_sequence):
    say(f"guards snapkv per_sequence={per_sequence}")
    d, Hq, Hkv, W, budget = 128, 8, 2, 8, 96
    kv_t = cache(torch.bfloat16, d, Hkv, spike=0.1)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, L = len(LENS), max(LENS)
    q_obs = queries(91, 4, (B, W, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    idx, sel = Guarded((B, Hkv, budget), torch.int32), Guarded((B,), torch.int32)
    ws = guarded_ws(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    if per_sequence:
        budgets = torch.tensor([40, 96, 64, 200, 17], dtype=torch.int32, device="cuda")
        sd.sd_snapkv_select_budgets(kv, q_obs, W, Hq, 7, budgets, budget, L, 1.0, idx.t, sel.t, ws.t)
    else:
        sd.sd_snapkv_select(kv, q_obs, W, Hq, 7, budget, L, 1.0, idx.t, sel.t, ws.t)
    check(idx=idx, sel_lens=sel, workspace=ws)
    q = queries(91, 2, (B, 1, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    out, lse = Guarded((B, 1, Hq, d), torch.bfloat16), Guarded((B, 1, Hq), torch.float32)
    wsd = guarded_ws(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, budget))
    sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx.t, sel.t, Hkv, budget, 1.0, out.t, lse.t, wsd.t)
    check(out=out, lse=lse, workspace=wsd)


def test_snapkv_two_calls_write_only_their_outputs():
    """The window normalisers (every sequence scored, short ones included)
    and the selection from them."""
    say("guards snapkv two calls")
    d, Hq, Hkv, W, budget = 128, 8, 2, 8, 96
    kv_t = cache(torch.bfloat16, d, Hkv, spike=0.1)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, L = len(LENS), max(LENS)
    q_obs = queries(91, 4, (B, W, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    lse = Guarded((B, W, Hq), torch.float32)
    ws = guarded_ws(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    sd.sd_snapkv_window_lse(kv, q_obs, W, Hq, L, 1.0, lse.t, ws.t)
    check(lse=lse, workspace=ws)
    idx, sel = Guarded((B, Hkv, budget), torch.int32), Guarded((B,), torch.int32)
    sd.sd_snapkv_select_lse(kv, q_obs, lse.t, W, Hq, 7, budget, L, 1.0, idx.t, sel.t, ws.t)
    check(idx=idx, sel_lens=sel, lse=lse, workspace=ws)


@pytest.mark.parametrize("kind,extra", [("shared", 0), ("per-head", 1)])
def test_kv_compact_writes_only_its_pools(kind, extra):
    """The copy of the selections (ragged, one sequence at or under its
    budget) writes inside its two pools and leaves the source cache as it
    was."""
    say(f"guards kv_compact {kind} extra={extra}")
    d, Hkv, max_sel, P = 128, 2, 96, 16
    kv_t = cache(torch.bfloat16, d, Hkv)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = len(LENS)
    heads = Hkv if kind == "per-head" else 1
    rng = np.random.default_rng(5)
    idx_np = np.full((B, heads, max_sel), -1, dtype=np.int32)
    sel_np = np.array([min(L, max_sel) for L in LENS], dtype=np.int32)
    for b, L in enumerate(LENS):
        for g in range(heads):
            idx_np[b, g, :sel_np[b]] = rng.choice(L, sel_np[b], replace=False)
    idx = torch.tensor(idx_np, device="cuda")
    sel = torch.tensor(sel_np, device="cuda")
    pps = max_sel // P + extra
    k_out = Guarded((B * pps, Hkv, P, d), torch.bfloat16)
    v_out = Guarded((B * pps, Hkv, P, d), torch.bfloat16)
    k_src, v_src = kv_t.k_pages.clone(), kv_t.v_pages.clone()
    sd.sd_kv_compact(kv, idx, sel, heads, max_sel, pps, k_out.t, v_out.t)
    check(k_out=k_out, v_out=v_out)
    assert torch.equal(k_src.view(torch.int16), kv_t.k_pages.view(torch.int16))
    assert torch.equal(v_src.view(torch.int16), kv_t.v_pages.view(torch.int16))


def test_topk_selection_and_per_head_draft_write_only_their_outputs():
    say("guards top-K")
    d, Hq, Hkv, budget = 128, 8, 2, 64
    kv_t = cache(torch.bfloat16, d, Hkv)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, L = len(LENS), max(LENS)
    q = queries(91, 2, (B, 1, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    idx, sel = Guarded((B, Hq, budget), torch.int32), Guarded((B,), torch.int32)
    ws = guarded_ws(sd.sd_topk_select_workspace_size(B, Hq, Hkv, L))
    sd.sd_topk_select(kv, q, Hq, budget, L, idx.t, sel.t, ws.t)
    check(idx=idx, sel_lens=sel, workspace=ws)
    out, lse = Guarded((B, 1, Hq, d), torch.bfloat16), Guarded((B, 1, Hq), torch.float32)
    wsd = guarded_ws(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, budget))
    sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx.t, sel.t, Hq, budget, 1.0, out.t, lse.t, wsd.t)
    check(out=out, lse=lse, workspace=wsd)


@pytest.mark.parametrize("gamma,vocab", [(3, 1000), (0, 5000), (4, 128256)])
def test_accept_writes_only_its_outputs(gamma, vocab):
    say(f"guards accept gamma={gamma} V={vocab}")
    B = 6
    zt = logits(91, 8, (B, gamma + 1, vocab), 2.0, "cuda")
    zd = logits(91, 9, (B, max(gamma, 1), vocab), 0.5, "cuda", base=zt[:, :max(gamma, 1)]).contiguous()
    x = gumbel_tokens(91, zd)
    ua = dyadic_uniforms(91, 11, (B, max(gamma, 1)), "cuda")
    us = dyadic_uniforms(91, 12, (B, gamma + 1), "cuda")
    n_acc, toks = Guarded((B,), torch.int32), Guarded((B, gamma + 1), torch.int32)
    ws = guarded_ws(sd.sd_spec_accept_workspace_size(B, gamma, vocab))
    sd.sd_spec_accept(zt, zd, x, ua, us, gamma, vocab, 1.0, n_acc.t, toks.t, ws.t)
    check(n_accepted=n_acc, out_tokens=toks, workspace=ws)
    assert np.all(toks.t.cpu().numpy()[np.arange(B), n_acc.t.cpu().numpy()] >= 0)


def test_length_advance_writes_only_the_lengths():
    say("guards advance")
    lens = Guarded((5,), torch.int32)
    lens.t.copy_(torch.tensor([10, 0, 7, 100, 3], dtype=torch.int32))
    n = torch.tensor([1, 0, 3, 2, 0], dtype=torch.int32, device="cuda")
    sd.sd_kv_advance(lens.t, n, -3)
    check(kv_lens=lens)
    assert lens.t.cpu().tolist() == [8, 0, 7, 99, 0]
