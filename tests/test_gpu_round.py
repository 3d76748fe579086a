"""GPU parity of a self-speculative round's cache bookkeeping against the CPU
oracle: KV append (bit-exact), length advance (exact), draft attention over the
selection plus the appended tail, and one whole round chained on the device
(select, gamma x [append, draft, sample], append, verify, accept, advance)
checked step by step against the oracle chain. The gamma draft steps are also
captured in a HIP graph and replayed against the eager run.
"""
import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
import oracle
from synth import dyadic_uniforms, logits, paged_kv, queries
from tests.gpu_helpers import check_accept, compare_attn, dirty_workspace, ensure_lib, say

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def _same(a, b):
    """Bitwise equality of float tensors, NaN == NaN."""
    a, b = a.cpu(), b.cpu()
    if a.dtype == BF16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    else:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return torch.equal(a, b)


def _np(t):
    return t.cpu().double().numpy() if t.is_floating_point() else t.cpu().numpy()


def _bits_equal(gpu, ref):
    g = _np(gpu)
    return np.array_equal(np.nan_to_num(g, nan=7.0), np.nan_to_num(ref, nan=7.0))


@pytest.mark.parametrize("dtype,d,P,n_new,shuffle", [
    (BF16, 128, 16, 5, True), (BF16, 64, 32, 3, False), (torch.float32, 64, 16, 1, True),
    (BF16, 128, 48, 17, True)])
def test_kv_append_bit_exact(dtype, d, P, n_new, shuffle):
    lens = [0, 15, 16, 31, 200, 77]
    kv_t = paged_kv(81, [L + n_new for L in lens], 2, d, dtype, "cuda", shuffle=shuffle, page_size=P)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_lens)
    g = torch.Generator(device="cuda").manual_seed(5)
    k_new = torch.randn((len(lens), n_new, 2, d), generator=g, device="cuda").to(dtype)
    v_new = torch.randn((len(lens), n_new, 2, d), generator=g, device="cuda").to(dtype)
    K_ref, V_ref = oracle.kv_append(kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(), lens,
                                    k_new.cpu(), v_new.cpu())
    sd.sd_kv_append(kv, k_new, v_new, n_new)
    torch.cuda.synchronize()
    assert _bits_equal(kv_t.k_pages, K_ref) and _bits_equal(kv_t.v_pages, V_ref)
    assert kv_lens.cpu().tolist() == lens  # append does not move the lengths


def test_kv_advance_exact():
    lens = torch.tensor([10, 5, 0, 3, 2], dtype=torch.int32, device="cuda")
    n_acc = torch.tensor([2, 0, 4, 1, 0], dtype=torch.int32, device="cuda")
    sd.sd_kv_advance(lens, n_acc, -4)
    sd.sd_kv_advance(lens, None, 1)
    torch.cuda.synchronize()
    want = oracle.kv_advance(oracle.kv_advance([10, 5, 0, 3, 2], -4, [2, 0, 4, 1, 0]), 1)
    assert lens.cpu().tolist() == list(want) == [9, 2, 1, 1, 1]  # the last one clamps at 0 first


def _selection(seed, lens, heads, max_sel):
    """Random selections (sorted, or reversed for odd heads) of up to max_sel
    positions per sequence; sequence 1 selects nothing."""
    rng = np.random.default_rng(seed)
    idx = np.full((len(lens), heads, max_sel), -1, dtype=np.int32)
    sel = np.zeros(len(lens), dtype=np.int32)
    for b, L in enumerate(lens):
        n = 0 if b == 1 else int(min(L, rng.integers(1, max_sel + 1)))
        sel[b] = n
        for g in range(heads):
            pos = np.sort(rng.choice(L, size=n, replace=False))
            idx[b, g, :n] = pos[::-1] if g % 2 else pos
    return torch.tensor(idx).cuda(), torch.tensor(sel).cuda()


@pytest.mark.parametrize("dtype,d,P,kind,extra", [
    (BF16, 128, 16, "shared", 0), (BF16, 128, 16, "per-head", 1), (torch.float32, 64, 32, "per-head", 0),
    (BF16, 64, 32, "shared", 2)])
def test_kv_compact_bit_exact_and_its_decode_is_the_draft(dtype, d, P, kind, extra):
    """The compact copy of a selection holds exactly the selected rows in list
    order (bit-exact against the oracle, untouched slots and the page past the
    pool keep their NaN), and a dense decode over it (verify with n_q = 1)
    equals the sparse draft over the original cache."""
    lens = [900, 40, 1300, 17, 600]
    B, Hkv, Hq, max_sel = len(lens), 2, 8, 300
    say(f"kv_compact {dtype} d={d} P={P} {kind} extra={extra}")
    kv_t = paged_kv(31 + d + P, lens, Hkv, d, dtype, "cuda", shuffle=True, page_size=P)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    heads = Hkv if kind == "per-head" else 1
    idx, sel = _selection(d + P, lens, heads, max_sel)
    pps = -(-max_sel // P) + extra
    k_out = torch.full((B * pps + 1, Hkv, P, d), float("nan"), dtype=dtype, device="cuda")
    v_out = torch.full_like(k_out, float("nan"))
    sd.sd_kv_compact(kv, idx, sel, heads, max_sel, pps, k_out, v_out)
    torch.cuda.synchronize()
    Kc, Vc = oracle.kv_compact(kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(), idx.cpu(),
                               sel.cpu(), pps)
    assert _bits_equal(k_out[:-1], Kc) and _bits_equal(v_out[:-1], Vc)
    assert torch.isnan(k_out[-1].float()).all() and torch.isnan(v_out[-1].float()).all()

    table = torch.arange(B * pps, dtype=torch.int32, device="cuda").view(B, pps)
    kvc = sd.KVCache(k_out, v_out, table, sel)
    q = queries(77, 1, (B, 1, Hq, d), dtype, "cuda", scale=d ** -0.5)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, 1, Hq, Hkv, d, max_sel), "cuda")
    sd.sd_verify_attn(kvc, q, 1, Hq, max_sel, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, idx, sel, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, dtype)
    say(f"  compact decode vs draft: max|dO|={err[0]:.3e} norm={err[1]:.3e} lse={err[2]:.3e}")


def test_compact_cache_takes_appended_tokens_like_the_tail_draft():
    """New tokens appended to both the full cache and the compact copy (its
    spare pages): a dense decode over the compact copy is then the draft over
    selection + tail, as the oracle computes it on the full cache."""
    lens0, n_new, max_sel = [700, 260, 333], 3, 96
    B, Hkv, Hq, d, P = len(lens0), 2, 8, 128, 16
    say(f"compact + append: lens={lens0} n_new={n_new}")
    kv_t = paged_kv(85, [L + n_new for L in lens0], Hkv, d, BF16, "cuda", shuffle=True)
    lens_d = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, lens_d)
    idx, sel = _selection(85, lens0, Hkv, max_sel)
    pps = -(-(max_sel + n_new) // P)
    k_c = torch.full((B * pps, Hkv, P, d), float("nan"), dtype=BF16, device="cuda")
    v_c = torch.full_like(k_c, float("nan"))
    sd.sd_kv_compact(kv, idx, sel, Hkv, max_sel, pps, k_c, v_c)
    lens_c = sel.clone()
    kvc = sd.KVCache(k_c, v_c, torch.arange(B * pps, dtype=torch.int32, device="cuda").view(B, pps), lens_c)
    g = torch.Generator(device="cuda").manual_seed(85)
    k_new = torch.randn((B, n_new, Hkv, d), generator=g, device="cuda").to(BF16)
    v_new = torch.randn((B, n_new, Hkv, d), generator=g, device="cuda").to(BF16)
    sd.sd_kv_append(kv, k_new, v_new, n_new)
    sd.sd_kv_append(kvc, k_new, v_new, n_new)
    sd.sd_kv_advance(lens_d, None, n_new)
    sd.sd_kv_advance(lens_c, None, n_new)
    q = queries(85, 1, (B, 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, 1, Hq, Hkv, d, pps * P), "cuda")
    sd.sd_verify_attn(kvc, q, 1, Hq, pps * P, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    lens1 = [L + n_new for L in lens0]
    o_ref, l_ref = oracle.sparse_attn_tail(q.cpu(), kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(),
                                           idx.cpu().numpy(), sel.cpu().numpy(), lens0, lens1, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, BF16)
    say(f"  max|dO|={err[0]:.2e} norm={err[1]:.2e} lse={err[2]:.2e}")


TAIL_CASES = [
    # name, lens, tail_begin, sel width, idx_heads, n_q
    ("streaming+tail", [500, 300], [480, 290], 64, 1, 1),
    ("per-head+tail", [700, 260], [650, 250], 96, 2, 1),
    ("empty-tail", [400, 333], [400, 400], 64, 2, 1),
    ("tail-only", [130, 47], [0, 0], 16, 1, 1),
    ("two-rows-long-tail", [900, 520], [100, 20], 32, 2, 2),
]


@pytest.mark.parametrize("case", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
def test_draft_with_tail_parity(case):
    name, lens, tail_begin, width, idx_heads, n_q = case
    B, Hkv, Hq, d = len(lens), 2, 8, 128
    kv_t = paged_kv(83, lens, Hkv, d, BF16, "cuda", shuffle=True)
    rng = np.random.default_rng(7)
    idx = np.full((B, idx_heads, width), -1, dtype=np.int32)
    sel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        pool = min(tail_begin[b], lens[b])  # selected positions precede the tail and the end
        n = 0 if name == "tail-only" else min(width, pool)
        sel[b] = n
        for gi in range(idx_heads):
            idx[b, gi, :n] = np.sort(rng.choice(pool, n, replace=False))
    idx_d = torch.from_numpy(idx).cuda()
    sel_d = torch.from_numpy(sel).cuda()
    tb = torch.tensor(tail_begin, dtype=torch.int32, device="cuda")
    q = queries(83, 1, (B, n_q, Hq, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, Hq), float("nan"), dtype=torch.float32, device="cuda")
    max_tail = max(max(L - t, 0) for L, t in zip(lens, tail_begin))
    ws = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, n_q, Hq, Hkv, d, width), "cuda")
    sd.sd_draft_attn_sparse_tail(kv, q, n_q, Hq, idx_d, sel_d, idx_heads, width, tb, max_tail, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_attn_tail(q.cpu(), kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(),
                                           idx, sel, tail_begin, lens, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, BF16)
    say(f"  {name}: max|dO|={err[0]:.2e} norm={err[1]:.2e} lse={err[2]:.2e}")


def _round_inputs(B, Hkv, Hq, d, gamma, V, seed):
    """Synthetic per-round tensors: each step's new K/V and query, the draft
    and target logits, and the uniforms (the model around the path is out of
    scope, so its outputs are drawn)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    kv_new = [(torch.randn((B, 1, Hkv, d), generator=g, device="cuda").to(BF16),
               torch.randn((B, 1, Hkv, d), generator=g, device="cuda").to(BF16)) for _ in range(gamma + 1)]
    q_draft = [queries(seed, 100 + i, (B, 1, Hq, d), BF16, "cuda", scale=d ** -0.5) for i in range(gamma)]
    q_verify = queries(seed, 1, (B, gamma + 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    zt = logits(seed, 8, (B, gamma + 1, V), 2.0, "cuda")
    zd = logits(seed, 9, (B, gamma, V), 2.0, "cuda", base=zt[:, :gamma]).contiguous()
    u_draw = dyadic_uniforms(seed, 10, (B, gamma), "cuda")
    u_acc = dyadic_uniforms(seed, 11, (B, gamma), "cuda")
    u_smp = dyadic_uniforms(seed, 12, (B, gamma + 1), "cuda")
    return kv_new, q_draft, q_verify, zt, zd, u_draw, u_acc, u_smp


def test_round_end_to_end_matches_oracle_chain():
    B, Hkv, Hq, d, gamma, V, sink, recent = 4, 2, 8, 128, 3, 1000, 16, 48
    lens0 = [300, 517, 64, 1000]
    extra = gamma + 1
    kv_t = paged_kv(85, [L + extra for L in lens0], Hkv, d, BF16, "cuda", shuffle=True)
    kv_lens = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_lens)
    kv_new, q_draft, q_verify, zt, zd, u_draw, u_acc, u_smp = _round_inputs(B, Hkv, Hq, d, gamma, V, 85)
    # oracle state (float64 copies)
    K = kv_t.k_pages.cpu()
    Vp = kv_t.v_pages.cpu()
    pt = kv_t.page_table.cpu()
    lens = np.array(lens0)

    # selection at "prefill": StreamingLLM on the current lengths; the tail starts there
    cap = sink + recent
    idx = torch.empty((B, 1, cap), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    sd.sd_streaming_select(kv_lens, sink, recent, idx, sel)
    tail_begin = kv_lens.clone()
    idx_ref, sel_ref = oracle.streaming_select(lens, sink, recent)
    ws_d = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, cap), "cuda")
    ws_a = dirty_workspace(sd.sd_spec_accept_workspace_size(B, gamma, V), "cuda")
    ws_s = dirty_workspace(sd.sd_spec_accept_workspace_size(B, 0, V), "cuda")
    n0 = torch.empty((B,), dtype=torch.int32, device="cuda")
    drafted = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
    flagged_any = False
    for i in range(gamma):
        k_i, v_i = kv_new[i]
        sd.sd_kv_append(kv, k_i, v_i, 1)
        sd.sd_kv_advance(kv_lens, None, 1)
        K, Vp = oracle.kv_append(K, Vp, pt, lens, k_i.cpu(), v_i.cpu())
        lens = oracle.kv_advance(lens, 1)
        out = torch.empty_like(q_draft[i])
        lse = torch.empty((B, 1, Hq), dtype=torch.float32, device="cuda")
        sd.sd_draft_attn_sparse_tail(kv, q_draft[i], 1, Hq, idx, sel, 1, cap, tail_begin, gamma + 1, 1.0, out,
                                     lse, ws_d)
        o_ref, l_ref = oracle.sparse_attn_tail(q_draft[i].cpu(), K, Vp, pt, idx_ref, sel_ref, lens0, lens, 1.0)
        torch.cuda.synchronize()
        compare_attn(out, lse, o_ref, l_ref, BF16)
        # draft token i ~ softmax(draft logits i): the accept path with gamma = 0
        tok = torch.empty((B, 1), dtype=torch.int32, device="cuda")
        sd.sd_spec_accept(zd[:, i:i + 1].contiguous(), None, None, None, u_draw[:, i:i + 1].contiguous(), 0, V,
                          1.0, n0, tok, ws_s)
        torch.cuda.synchronize()
        st = check_accept(f"round draft-token draw {i}", np.zeros(B, dtype=np.int32), tok.cpu().numpy(),
                          zd[:, i:i + 1].cpu(), np.zeros((B, 0, V)), np.zeros((B, 0), int),
                          np.zeros((B, 0)), u_draw[:, i:i + 1].cpu())
        flagged_any |= st["flagged"] > 0
        # a flagged draw may differ within its band; the chain continues with the GPU's token on both sides
        drafted[:, i] = tok[:, 0]
    # verification: the last draft's K/V, then gamma + 1 causal queries over the full cache
    k_g, v_g = kv_new[gamma]
    sd.sd_kv_append(kv, k_g, v_g, 1)
    sd.sd_kv_advance(kv_lens, None, 1)
    K, Vp = oracle.kv_append(K, Vp, pt, lens, k_g.cpu(), v_g.cpu())
    lens = oracle.kv_advance(lens, 1)
    assert kv_lens.cpu().tolist() == list(lens) == [L + gamma + 1 for L in lens0]
    assert _bits_equal(kv_t.k_pages, K) and _bits_equal(kv_t.v_pages, Vp)
    out = torch.empty_like(q_verify)
    lse = torch.empty((B, gamma + 1, Hq), dtype=torch.float32, device="cuda")
    ws_v = dirty_workspace(sd.sd_verify_attn_workspace_size(B, gamma + 1, Hq, Hkv, d, max(lens)), "cuda")
    sd.sd_verify_attn(kv, q_verify, gamma + 1, Hq, int(max(lens)), 1.0, out, lse, ws_v)
    o_ref, l_ref = oracle.verify_attn(q_verify.cpu(), K, Vp, pt, lens, 1.0)
    torch.cuda.synchronize()
    compare_attn(out, lse, o_ref, l_ref, BF16)
    # acceptance of the sampled drafts, then the length rollback
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    toks = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    sd.sd_spec_accept(zt, zd, drafted, u_acc, u_smp, gamma, V, 1.0, n_acc, toks, ws_a)
    torch.cuda.synchronize()
    st = check_accept("round acceptance", n_acc.cpu().numpy(), toks.cpu().numpy(), zt.cpu(), zd.cpu(),
                      drafted.cpu(), u_acc.cpu(), u_smp.cpu())
    sd.sd_kv_advance(kv_lens, n_acc, -gamma)
    lens = oracle.kv_advance(lens, -gamma, n_acc.cpu().numpy())
    torch.cuda.synchronize()
    assert kv_lens.cpu().tolist() == list(lens)
    say(f"  accepted {n_acc.cpu().tolist()}, flagged {st['flagged']} + draws {int(flagged_any)}")


def test_draft_steps_graph_replay_matches_eager():
    """The gamma draft steps (append, advance, draft over selection + tail,
    sample) captured in a HIP graph: every replay, from the same starting
    state, reproduces the eager run bit for bit."""
    B, Hkv, Hq, d, gamma, V = 8, 2, 8, 128, 4, 5000
    lens0 = [400, 1500, 64, 999, 2048, 17, 700, 1200]
    kv_t = paged_kv(87, [L + gamma for L in lens0], Hkv, d, BF16, "cuda", shuffle=True)
    kv_lens = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_lens)
    kv_new, q_draft, _, _, zd, u_draw, _, _ = _round_inputs(B, Hkv, Hq, d, gamma, V, 87)
    cap = 512
    idx = torch.empty((B, 1, cap), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    sd.sd_streaming_select(kv_lens, 64, 448, idx, sel)
    tail_begin = kv_lens.clone()
    ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, cap))
    ws_s = sd.workspace(sd.sd_spec_accept_workspace_size(B, 0, V))
    outs = [torch.empty_like(q_draft[i]) for i in range(gamma)]
    toks = torch.empty((B, gamma), dtype=torch.int32, device="cuda")
    tok1 = [torch.empty((B, 1), dtype=torch.int32, device="cuda") for _ in range(gamma)]
    n0 = torch.empty((B,), dtype=torch.int32, device="cuda")
    zd_i = [zd[:, i:i + 1].contiguous() for i in range(gamma)]
    u_i = [u_draw[:, i:i + 1].contiguous() for i in range(gamma)]
    saved = (kv_t.k_pages.clone(), kv_t.v_pages.clone(), kv_lens.clone())

    def steps():
        for i in range(gamma):
            sd.sd_kv_append(kv, kv_new[i][0], kv_new[i][1], 1)
            sd.sd_kv_advance(kv_lens, None, 1)
            sd.sd_draft_attn_sparse_tail(kv, q_draft[i], 1, Hq, idx, sel, 1, cap, tail_begin, gamma, 1.0,
                                         outs[i], None, ws_d)
            sd.sd_spec_accept(zd_i[i], None, None, None, u_i[i], 0, V, 1.0, n0, tok1[i], ws_s)

    def restore():
        kv_t.k_pages.copy_(saved[0])
        kv_t.v_pages.copy_(saved[1])
        kv_lens.copy_(saved[2])

    steps()  # eager (also warms up the occupancy queries before capture)
    torch.cuda.synchronize()
    want = ([o.clone() for o in outs], torch.cat(tok1, 1).clone(), kv_t.k_pages.clone(), kv_lens.clone())
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            steps()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(_same(o, w) for o, w in zip(outs, want[0])), rep
        assert torch.equal(torch.cat(tok1, 1), want[1]), rep
        assert _same(kv_t.k_pages, want[2]) and torch.equal(kv_lens, want[3]), rep
