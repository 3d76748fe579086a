"""GPU parity of the dynamic top-K attention draft (sd_topk_select, then
sd_draft_attn_sparse with one index set per query head) against the oracle.

Selection: rows whose sequence is not longer than the budget must equal
0..L-1 then -1 exactly. Longer rows must hold `budget` distinct ascending
positions below L; a position the GPU and the oracle disagree on must have an
oracle score within SCORE_TOL * max_j sum_i |q_i k_ji| of the cut (the
budget-th largest score): the GPU sums exact bf16 products in fp32, the oracle
in fp64, so two scores that close may be ordered either way. Attention is then
compared with the oracle over the GPU's own sets (the tolerances of
tests/gpu_helpers.py), and with the oracle's own top-K output wherever the
sets agree.
"""
import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
import oracle
from synth import WORKLOADS, paged_kv, queries, workload_lens
from tests.gpu_helpers import compare_attn, dirty_workspace, ensure_lib, gathered_decode, run_draft, say, unit_cache

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
SCORE_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def run_topk(kv_t, q, Hq, budget, max_kv_len=None):
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = kv.batch
    mk = max(1, kv_t.max_kv_len) if max_kv_len is None else max_kv_len
    idx = torch.full((B, Hq, budget), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_topk_select_workspace_size(B, Hq, kv.num_kv_heads, mk), "cuda")
    sd.sd_topk_select(kv, q, Hq, budget, mk, idx, sel, ws)
    torch.cuda.synchronize()
    return idx, sel


def check_row(a, L, budget, scores=None, ref=None):
    """One (sequence, query head) row of the GPU selection; returns 1 if it
    differs from the oracle's set by an explained near-tie, else 0."""
    if L <= budget:
        assert list(a[:L]) == list(range(L)) and (a[L:] == -1).all()
        return 0
    assert len(set(a.tolist())) == budget and (np.diff(a) > 0).all() and a[0] >= 0 and a[-1] < L
    if np.array_equal(a, ref):
        return 0
    s, mag = scores
    thr = np.sort(s)[::-1][budget - 1]
    for t in set(a.tolist()) ^ set(ref.tolist()):
        assert abs(s[t] - thr) <= SCORE_TOL * mag, (t, s[t], thr, mag)
    return 1


def unit_scores(k, table, L, qh):
    """fp64 scores of one query head over a unit cache and the magnitude
    max_j sum_i |q_i k_ji| that bounds their fp32 rounding."""
    s = oracle.topk_scores(qh, k, table, L, 0, 0)
    keys = np.abs(k.double().numpy()[table[0, :]][:, 0].reshape(-1, k.shape[-1])[:int(L[0])])
    return s, float((keys @ np.abs(qh.double().numpy()[0, 0, 0])).max())


def check_selection(kv_t, q, idx, sel, budget, lens, rows):
    Hq = q.shape[2]
    G = Hq // kv_t.k_pages.shape[1]
    idx_c = idx.cpu().numpy()
    assert list(sel.cpu().numpy()) == [min(L, budget) for L in lens]
    near = 0
    for b, h in rows:
        L = lens[b]
        if L <= budget:
            near += check_row(idx_c[b, h], L, budget)
            continue
        k, _, table, Ls = unit_cache(kv_t, b, h // G)
        qh = q[b:b + 1, :, h:h + 1].cpu()
        s, mag = unit_scores(k, table, Ls, qh)
        ref, _ = oracle.topk_select(qh, k, table, Ls, budget)
        near += check_row(idx_c[b, h], L, budget, (s, mag), ref[0, 0])
    return near


TOPK_CASES = [
    # name, Hq, Hkv, d, lens, budget, page_size, shuffle, spike
    ("small-g4", 8, 2, 128, [37, 300, 1000], 64, 16, False, 0.0),
    ("short-rows-kept", 8, 2, 128, [0, 5, 64, 65, 2000], 64, 16, True, 0.0),
    ("g1-d64", 4, 4, 64, [129, 4111, 700], 128, 32, False, 0.1),
    ("g8", 16, 2, 128, [3000, 1500], 256, 16, True, 0.1),
    ("g16", 16, 1, 128, [2500], 100, 48, False, 0.0),
    ("tiles-ragged", 8, 2, 128, [4111, 9000, 16, 8200], 512, 16, True, 0.1),
    ("vpt16", 4, 1, 128, [20000, 12000], 1024, 64, True, 0.1),
    ("budget-1", 8, 2, 128, [50, 333], 1, 16, False, 0.0),
    ("g5-odd", 10, 2, 128, [6000, 2500, 12000], 300, 16, True, 0.1),
    ("g3-d64", 6, 2, 64, [5000, 700, 16384], 256, 32, True, 0.0),
    ("ragged-many", 8, 2, 128, [1000 + 2531 * i for i in range(16)], 512, 16, True, 0.1),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_select_parity(case):
    name, Hq, Hkv, d, lens, budget, P, shuffle, spike = case
    say(f"topk select {name}: Hq={Hq} Hkv={Hkv} d={d} lens={lens} budget={budget} P={P}")
    kv_t = paged_kv(31, lens, Hkv, d, BF16, "cuda", page_size=P, shuffle=shuffle, spike_frac=spike)
    q = queries(31, 2, (len(lens), 1, Hq, d), BF16, "cuda", scale=1.0)
    idx, sel = run_topk(kv_t, q, Hq, budget)
    rows = [(b, h) for b in range(len(lens)) for h in range(Hq)]
    near = check_selection(kv_t, q, idx, sel, budget, lens, rows)
    say(f"  rows={len(rows)} near-tie rows={near}")
    assert near <= max(1, len(rows) // 20)
    idx2, _ = run_topk(kv_t, q, Hq, budget)  # deterministic
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("ramp", [30.0, -30.0])
def test_topk_select_with_trending_scores(ramp):
    """Scores rising (or falling) by 30 over each sequence along one direction
    u of every query: the budget's keys crowd at one end of the sequence, far
    from where a uniform sample of the scores would put the threshold."""
    Hq, Hkv, d, budget = 8, 2, 128, 256
    lens = [6000, 2500]
    say(f"topk select trending scores ramp={ramp}")
    kv_t = paged_kv(78, lens, Hkv, d, BF16, "cuda", shuffle=True)
    g = torch.Generator(device="cuda").manual_seed(78)
    u = torch.randn(d, generator=g, device="cuda")
    u /= u.norm()
    P = kv_t.page_size
    for b, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        page = kv_t.page_table[b].long()[t // P]
        rows = kv_t.k_pages[page, :, t % P, :].float() + (ramp * t / L)[:, None, None] * u
        kv_t.k_pages[page, :, t % P, :] = rows.to(BF16)
    q = (queries(78, 2, (len(lens), 1, Hq, d), torch.float32, "cuda", scale=d ** -0.5) + u).to(BF16)
    idx, sel = run_topk(kv_t, q, Hq, budget)
    rows = [(b, h) for b in range(len(lens)) for h in range(Hq)]
    near = check_selection(kv_t, q, idx, sel, budget, lens, rows)
    say(f"  rows={len(rows)} near-tie rows={near}")
    assert near <= 1


def test_topk_select_max_len_above_lengths_and_exact_ties():
    """max_kv_len larger than every length; a cache whose keys repeat one row
    (every score tied) keeps the lowest positions."""
    lens = [700, 1100]  # the table holds 69 pages of 16: room for 1104 tokens
    kv_t = paged_kv(32, lens, 2, 128, BF16, "cuda")
    kv_t.k_pages[:] = kv_t.k_pages[0:1, :, 0:1, :]
    q = queries(32, 2, (2, 1, 8, 128), BF16, "cuda")
    idx, sel = run_topk(kv_t, q, 8, 300, max_kv_len=1104)
    want = np.array(list(range(300)))
    assert (idx.cpu().numpy() == want).all()


@pytest.mark.parametrize("case", ["sample-grid-spikes", "large-budget", "recompute-by-size"])
def test_topk_select_candidate_paths(case):
    """The selection keeps the keys at or above a sampled threshold as
    candidates. Spikes on exactly the sampled positions push that threshold
    above the budget-th key, so the row is recomputed in full; a large budget
    gives more candidates than the small register path holds; a long row with
    a budget near half its length exceeds every register path."""
    Hq, Hkv, d = 4, 1, 128
    if case == "sample-grid-spikes":
        L, budget = 32768, 2048
    elif case == "large-budget":
        L, budget = 32768, 8192
    else:
        L, budget = 70000, 30000
    kv_t = paged_kv(35, [L], Hkv, d, BF16, "cuda", page_size=16, spike_frac=0.0)
    q = queries(35, 2, (1, 1, Hq, d), BF16, "cuda", scale=1.0)
    grid = None
    if case == "sample-grid-spikes":
        q[:] = q[:, :, :1]  # every head asks the same question
        u = q[0, 0, 0].float()
        # the sampled positions at L = 32768, G = 4: 64 runs of 16 at steps 32k
        grid = (torch.arange(64, device="cuda")[:, None] * 512 + torch.arange(16, device="cuda")).reshape(-1)
        pt = kv_t.page_table[0].long()
        kv_t.k_pages[pt[grid // 16], 0, grid % 16, :] = (4.0 * u / u.norm()).to(BF16)
    idx, sel = run_topk(kv_t, q, Hq, budget)
    near = check_selection(kv_t, q, idx, sel, budget, [L], [(0, h) for h in range(Hq)])
    say(f"  {case}: L={L} budget={budget} near-tie rows={near}")
    if grid is not None:
        ic = idx.cpu().numpy()
        for h in range(Hq):  # every spike is kept
            assert set(grid.tolist()) <= set(ic[0, h].tolist())


def test_topk_select_one_long_sequence_many_segments():
    """One sequence of 200k tokens and one KV head: the scoring schedule splits
    the unit over more segments than the small selection gathers, so the rows
    go through the full-row kernel's candidate path."""
    L, Hq, Hkv, d, budget = 200000, 4, 1, 128, 2048
    kv_t = paged_kv(37, [L], Hkv, d, BF16, "cuda", spike_frac=0.1)
    q = queries(37, 2, (1, 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx, sel = run_topk(kv_t, q, Hq, budget)
    near = check_selection(kv_t, q, idx, sel, budget, [L], [(0, h) for h in range(Hq)])
    say(f"  one sequence L={L}: near-tie rows={near}")
    assert near <= 1


@pytest.mark.parametrize("n_q", [1, 2])
def test_per_query_head_draft_parity(n_q):
    """Draft over one index set per query head (random sets, ragged lengths,
    shuffled pages) against the oracle's per-head sparse attention."""
    Hq, Hkv, d, max_sel = 8, 2, 128, 96
    lens = [500, 97, 3000]
    kv_t = paged_kv(33, lens, Hkv, d, BF16, "cuda", shuffle=True)
    rng = np.random.default_rng(33)
    sel_lens = [min(L, max_sel) for L in lens]
    idx = np.full((len(lens), Hq, max_sel), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        for h in range(Hq):
            idx[b, h, :sel_lens[b]] = np.sort(rng.choice(L, sel_lens[b], replace=False))
    q = queries(33, 3, (len(lens), n_q, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx_t = torch.from_numpy(idx).cuda()
    sel_t = torch.tensor(sel_lens, dtype=torch.int32, device="cuda")
    out, lse = run_draft(kv_t, q, n_q, Hq, idx_t, sel_t)
    o_ref, l_ref = oracle.sparse_attn(q.cpu(), kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(),
                                      idx, sel_lens, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, BF16)
    say(f"  per-head draft n_q={n_q}: max|dO|={err[0]:.2e} lse={err[2]:.2e}")
    # the same sets repeated over each group equal the per-KV-head draft
    shared = np.repeat(idx[:, ::Hq // Hkv][:, :Hkv], Hq // Hkv, axis=1)
    out_a, lse_a = run_draft(kv_t, q, n_q, Hq, torch.from_numpy(shared).cuda(), sel_t)
    out_b, lse_b = run_draft(kv_t, q, n_q, Hq, torch.from_numpy(np.ascontiguousarray(shared[:, ::Hq // Hkv])).cuda(),
                             sel_t)
    assert (out_a.float() - out_b.float()).abs().max() <= 2e-2
    assert (lse_a - lse_b).abs().max() <= 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_per_query_head_draft_fp32(d):
    """The per-query-head draft on fp32 caches, with the appended tail read
    after each head's own set (1e-5 relative bar)."""
    Hq, Hkv, max_sel, tail = 6, 2, 40, 9
    lens = [300, 1200]
    kv_t = paged_kv(38, lens, Hkv, d, torch.float32, "cuda", shuffle=True)
    rng = np.random.default_rng(38)
    tail_begin = [L - tail for L in lens]
    sel_lens = [max_sel, max_sel]
    idx = np.full((len(lens), Hq, max_sel), -1, dtype=np.int32)
    for b in range(len(lens)):
        for h in range(Hq):
            idx[b, h] = np.sort(rng.choice(tail_begin[b], max_sel, replace=False))
    q = queries(38, 3, (len(lens), 1, Hq, d), torch.float32, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((len(lens), 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(len(lens), 1, Hq, Hkv, d, max_sel), "cuda")
    sd.sd_draft_attn_sparse_tail(kv, q, 1, Hq, torch.from_numpy(idx).cuda(),
                                 torch.tensor(sel_lens, dtype=torch.int32, device="cuda"), Hq, max_sel,
                                 torch.tensor(tail_begin, dtype=torch.int32, device="cuda"), tail, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_attn_tail(q.cpu(), kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(),
                                           idx, sel_lens, tail_begin, lens, 1.0)
    compare_attn(out, lse, o_ref, l_ref, torch.float32)


@pytest.mark.parametrize("case", ["small-g4", "tiles-ragged"])
def test_topk_draft_step_parity(case):
    """Select, then draft over the selection: equal to the oracle over the
    GPU's sets, and to the oracle's own top-K attention where the sets agree."""
    _, Hq, Hkv, d, lens, budget, P, shuffle, spike = [c for c in TOPK_CASES if c[0] == case][0]
    kv_t = paged_kv(34, lens, Hkv, d, BF16, "cuda", page_size=P, shuffle=shuffle, spike_frac=spike)
    q = queries(34, 2, (len(lens), 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx, sel = run_topk(kv_t, q, Hq, budget)
    out, lse = run_draft(kv_t, q, 1, Hq, idx, sel)
    kc, vc, tc = kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu()
    o_ref, l_ref = oracle.sparse_attn(q.cpu(), kc, vc, tc, idx.cpu().numpy(), sel.cpu().numpy(), 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, BF16)
    o_top, l_top, idx_top, _ = oracle.topk_attn(q.cpu(), kc, vc, tc, lens, budget, 1.0)
    same = [(b, h) for b in range(len(lens)) for h in range(Hq)
            if np.array_equal(idx_top[b, h], idx.cpu().numpy()[b, h])]
    assert len(same) >= len(lens) * Hq * 0.9
    compare_attn(out, lse, o_top, l_top, BF16, rows=same)
    say(f"  {case}: max|dO|={err[0]:.2e}; rows with the oracle's own set: {len(same)}/{len(lens) * Hq}")


def test_topk_full_size_sampled():
    """Llama-3.1-8B shape B=128, 32k context, budget 2048: sampled rows of the
    selection against the oracle, and the draft over the selection on sampled
    units; every row is checked for structure."""
    w = WORKLOADS["llama8b-b128-l32k-snapkv"]
    lens = workload_lens(w)
    B, Hq, Hkv, d, budget = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.budget
    kv_t = paged_kv(w.seed, lens, Hkv, d, BF16, "cuda", shuffle=w.shuffle, spike_frac=w.spike_frac)
    q = queries(w.seed, 1, (B, 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    say(f"topk full size: B={B} L={max(lens)} Hq={Hq} budget={budget}")
    idx, sel = run_topk(kv_t, q, Hq, budget)
    ic = idx.cpu().numpy()
    assert (np.diff(ic, axis=2) > 0).all() and (ic >= 0).all() and (ic < max(lens)).all()
    rng = np.random.default_rng(5)
    rows = sorted({(0, 0), (B - 1, Hq - 1)} | {(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(4)})
    near = check_selection(kv_t, q, idx, sel, budget, lens, rows)
    say(f"  sampled rows {rows}: near-tie rows={near}")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, budget), "cuda")
    sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx, sel, Hq, budget, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    G = Hq // Hkv
    for b, h in rows:
        k, v, table, L = unit_cache(kv_t, b, h // G)
        o_ref, l_ref = oracle.sparse_attn(q[b:b + 1, :, h:h + 1].cpu(), k, v, table, ic[b:b + 1, h:h + 1],
                                          [int(sel[b])], 1.0)
        compare_attn(out[b:b + 1, :, h:h + 1], lse[b:b + 1, :, h:h + 1], o_ref, l_ref, BF16)
    # every row against a plain PyTorch fp32 reference: scores q . k, stable
    # top-K (ties to the lower position); rows may differ only within
    # SCORE_TOL * max_j sum_i |q_i k_ji| of the cut
    G = Hq // Hkv
    differ = 0
    P = kv_t.k_pages.shape[2]
    for b in range(B):
        L = lens[b]
        if L <= budget:
            continue
        npg = (L + P - 1) // P
        k = kv_t.k_pages[kv_t.page_table[b, :npg].long()].float().permute(1, 0, 2, 3).reshape(Hkv, npg * P, d)[:, :L]
        qb = q[b, 0].float().reshape(Hkv, G, d)
        s = torch.bmm(qb, k.transpose(1, 2).contiguous()).reshape(Hq, L)
        mag = torch.bmm(qb.abs(), k.abs().transpose(1, 2).contiguous()).reshape(Hq, L).max(dim=1).values
        order = torch.sort(-s, dim=1, stable=True).indices[:, :budget]
        thr = torch.gather(s, 1, order[:, -1:])[:, 0]
        ref = torch.sort(order, dim=1).values.cpu().numpy()
        s_np, thr_np, mag_np = s.cpu().numpy(), thr.cpu().numpy(), mag.cpu().numpy()
        for h in range(Hq):
            if np.array_equal(ic[b, h], ref[h]):
                continue
            differ += 1
            for t in set(ic[b, h].tolist()) ^ set(ref[h].tolist()):
                assert abs(s_np[h, t] - thr_np[h]) <= SCORE_TOL * mag_np[h], (b, h, t)
    say(f"  every row vs PyTorch fp32: {differ} of {B * Hq} rows differ, all within the near-tie band")
    # every unit of the per-head draft against a dense decode over its gathered rows
    o_g, l_g = gathered_decode(kv_t, idx, sel, q, Hq)
    err = compare_attn(out, lse, o_g.double().cpu().numpy(), l_g.double().cpu().numpy(), BF16)
    say(f"  per-head draft vs dense decode over its rows (every unit): max|dO|={err[0]:.2e} lse={err[2]:.2e}")


def test_topk_draft_step_graph_replay_matches_eager():
    """Top-K selection and the per-head draft captured in a HIP graph: every
    replay (with eager work between replays) reproduces the eager results bit
    for bit, including a row that takes the full-row path (spikes on the
    sampled positions of sequence 0) and a sequence shorter than the budget."""
    Hq, Hkv, d, budget = 8, 2, 128, 1500  # 1024 spikes < budget: the spiked rows are recomputed
    lens = [32768, 20000, 700, 9000]
    kv_t = paged_kv(36, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=0.1)
    q = queries(36, 2, (len(lens), 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    q[0, 0, :4] = q[0, 0, 0]  # the first group asks one question; spike its sampled positions
    u = q[0, 0, 0].float()
    grid = (torch.arange(64, device="cuda")[:, None] * 512 + torch.arange(16, device="cuda")).reshape(-1)
    pt = kv_t.page_table[0].long()
    kv_t.k_pages[pt[grid // 16], 0, grid % 16, :] = (4.0 * u / u.norm()).to(BF16)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, L = len(lens), max(lens)
    idx = torch.empty((B, Hq, budget), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws_t = sd.workspace(sd.sd_topk_select_workspace_size(B, Hq, Hkv, L))
    ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, budget))

    def step():
        sd.sd_topk_select(kv, q, Hq, budget, L, idx, sel, ws_t)
        sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx, sel, Hq, budget, 1.0, out, None, ws_d)

    step()
    torch.cuda.synchronize()
    want = (idx.clone(), sel.clone(), out.clone())
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        idx.fill_(-7)
        sel.fill_(-7)
        out.fill_(float("nan"))
        ws_t.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want[0]) and torch.equal(sel, want[1]), rep
        assert torch.equal(out.view(torch.int16), want[2].view(torch.int16)), rep
    # the replays agree with the oracle on the spiked row and a short one
    near = check_selection(kv_t, q, idx, sel, budget, lens, [(0, 0), (0, 3), (2, 5), (3, 7)])
    assert near <= 1
