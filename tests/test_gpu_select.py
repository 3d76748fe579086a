"""GPU parity of StreamingLLM and SnapKV selection against the CPU oracle.

Selected index sets must match exactly. The only tolerated difference is a
near-tie: a position the two sides disagree on must have an oracle pooled
value within 1e-5 relative of the threshold value (the budget-W-th largest),
where float32 (GPU) and float64 (oracle) scoring may legitimately order two
distinct values differently. Such cases are counted and reported.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
import oracle
from synth import paged_kv, queries
from tests.gpu_helpers import dirty_workspace, ensure_lib, say
from tests.parity_log import record

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
NEAR_TIE_REL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("sink,recent", [(16, 48), (64, 448), (0, 32), (8, 0)])
def test_streaming_select_parity(sink, recent):
    lens = [0, 1, 15, 16, 63, 64, 65, 100, 511, 512, 513, 8192, 4097]
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx = torch.full((len(lens), 1, sink + recent), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((len(lens),), 7, dtype=torch.int32, device="cuda")
    sd.sd_streaming_select(kv_lens, sink, recent, idx, sel)
    torch.cuda.synchronize()
    idx_ref, sel_ref = oracle.streaming_select(np.array(lens), sink, recent)
    assert (sel.cpu().numpy() == sel_ref).all()
    assert (idx.cpu().numpy() == idx_ref).all()


def run_snapkv(kv_t, q_obs, window, Hq, pool, budget, max_kv_len=None, scale=1.0):
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = kv.batch
    mk = max(1, kv_t.max_kv_len) if max_kv_len is None else max_kv_len
    idx = torch.full((B, kv.num_kv_heads, budget), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, window, Hq, kv.num_kv_heads, mk), "cuda")
    sd.sd_snapkv_select(kv, q_obs, window, Hq, pool, budget, mk, scale, idx, sel, ws)
    torch.cuda.synchronize()
    return idx, sel


def check_selection(idx_gpu, idx_ref, sel_gpu, sel_ref, pooled, window, budget):
    """Exact match except explained near-ties; returns the near-tie count."""
    assert (sel_gpu == sel_ref).all()
    near = 0
    B, H, _ = idx_ref.shape
    for b in range(B):
        for g in range(H):
            a, r = idx_gpu[b, g], idx_ref[b, g]
            if np.array_equal(a, r):
                continue
            n = sel_ref[b]
            assert (a[n:] == -1).all() and len(set(a[:n].tolist())) == n
            assert (np.diff(a[:n]) > 0).all(), "GPU selection not ascending"
            pv = pooled[(b, g)]
            thr = np.sort(pv)[::-1][budget - window - 1]
            diff = set(a[:n].tolist()) ^ set(r[:n].tolist())
            for t in diff:
                assert t < len(pv), f"window position {t} differs"
                assert abs(pv[t] - thr) <= NEAR_TIE_REL * thr, (b, g, t, pv[t], thr)
            near += 1
    return near


SNAP_CASES = [
    # name, Hq, Hkv, d, lens, window, pool, budget, spike_frac
    ("g4-w8-rows32", 8, 2, 128, [700, 1500], 8, 7, 64, 0.0),
    ("g4-w32-rows128-spiky", 32, 8, 128, [3000, 2100], 32, 7, 256, 0.10),
    ("mixed-short", 8, 2, 128, [100, 2000, 200], 8, 7, 200, 0.0),
    ("pool1-w1", 8, 2, 128, [900], 1, 1, 40, 0.0),
    ("d64-pool3", 8, 2, 64, [1234, 517], 4, 3, 100, 0.10),
    ("rows48-ragged-pages", 24, 2, 128, [1111, 4096, 333], 4, 5, 300, 0.05),
    # longer prefixes: 16, 32 and 64 pooled values per top-K thread
    ("prefix-12k", 8, 2, 128, [12000, 5000], 8, 7, 512, 0.10),
    ("prefix-30k-rows128", 32, 1, 128, [30000], 4, 7, 1024, 0.10),
    ("prefix-40k", 8, 2, 64, [40000, 33000], 8, 5, 2048, 0.10),
    # 5..8 row tiles: two waves per block share the K stream
    ("rows80-two-waves", 8, 2, 128, [2500, 1900], 20, 7, 256, 0.10),
    ("rows96-two-waves", 16, 2, 128, [2100, 3300], 12, 5, 300, 0.05),
    ("d64-rows112-two-waves", 16, 2, 64, [3000, 1000], 14, 5, 300, 0.10),
    # a kept share near one half of the prefix
    ("prefix-30k-half-budget", 8, 2, 128, [30000, 24000], 8, 7, 15000, 0.10),
    # radix variant: prefix beyond 64 Ki keys, and a pool kernel wider than 129
    ("prefix-70k-radix", 8, 2, 64, [70000], 4, 3, 1000, 0.10),
    ("pool131-radix", 8, 2, 128, [3000, 2500], 8, 131, 300, 0.0),
    # more sequences than the planning block covers in one pass, most of
    # them at or under the budget
    ("1500-sequences", 8, 2, 128, np.random.default_rng(6).integers(0, 301, 1500).tolist(), 8, 7, 48, 0.10),
]


@pytest.mark.parametrize("case", SNAP_CASES, ids=[c[0] for c in SNAP_CASES])
def test_snapkv_select_parity(case):
    name, Hq, Hkv, d, lens, W, pool, budget, spike = case
    say(f"snapkv {name}: lens={lens} W={W} pool={pool} budget={budget}")
    seed = zlib.crc32(name.encode()) % 10000
    kv_t = paged_kv(seed, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=spike)
    q_obs = queries(seed, 4, (len(lens), W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx, sel = run_snapkv(kv_t, q_obs, W, Hq, pool, budget)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    W, pool, budget, 1.0, return_pooled=True)
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, W, budget)
    say(f"  near-tie (flagged) units: {near}")
    record(f"snapkv {name}", units=len(lens) * Hkv, near_tie=near)
    assert near <= max(1, len(lens) * Hkv // 8)


@pytest.mark.parametrize("ramp", [16.0, -16.0])
def test_snapkv_with_trending_scores(ramp):
    """Scores that rise (or fall) by 16 over each sequence: every window query
    has a component along one direction u that the keys carry with a weight
    growing in the position, so the statistics pass's running maximum keeps
    moving up through the sequence (rising) or is set at its start (falling),
    and the votes span some seven orders of magnitude."""
    Hq, Hkv, d, W, pool, budget = 8, 2, 128, 8, 7, 256
    lens = [3000, 1200]
    say(f"snapkv trending scores ramp={ramp}")
    kv_t = paged_kv(77, lens, Hkv, d, BF16, "cuda", shuffle=True)
    g = torch.Generator(device="cuda").manual_seed(77)
    u = torch.randn(d, generator=g, device="cuda")
    u /= u.norm()
    P = kv_t.page_size
    for b, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        page = kv_t.page_table[b].long()[t // P]
        rows = kv_t.k_pages[page, :, t % P, :].float() + (ramp * t / L)[:, None, None] * u
        kv_t.k_pages[page, :, t % P, :] = rows.to(BF16)
    q_obs = (queries(77, 4, (len(lens), W, Hq, d), torch.float32, "cuda", scale=d ** -0.5) + u).to(BF16)
    idx, sel = run_snapkv(kv_t, q_obs, W, Hq, pool, budget)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    W, pool, budget, 1.0, return_pooled=True)
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, W, budget)
    record(f"snapkv trending scores ramp={ramp}", units=len(lens) * Hkv, near_tie=near)
    assert near <= 1


SCALE_CASES = [
    # name, q_obs scale folded in, softmax_scale passed
    ("unscaled-q-inv-sqrt-d", 1.0, 128 ** -0.5),
    ("scaled-q-0.37", 128 ** -0.5, 0.37),
    ("scaled-q-2.5", 128 ** -0.5, 2.5),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_snapkv_softmax_scale(case):
    """The scale enters both passes (row statistics and the normalised votes):
    the standard 1/sqrt(d) applied by the call to unscaled window queries, and
    two other scales. Each case is checked to be sensitive first: the oracle's
    selection with the scale dropped differs from the one with it."""
    name, q_scale, scale = case
    Hq, Hkv, d, lens, W, pool, budget = 32, 8, 128, [3000, 2100, 4500], 32, 7, 256
    say(f"snapkv scale {name}: q scale {q_scale:.4f}, softmax_scale {scale}")
    kv_t = paged_kv(303, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=0.10)
    q_obs = queries(303, 4, (len(lens), W, Hq, d), BF16, "cuda", scale=q_scale)
    idx, sel = run_snapkv(kv_t, q_obs, W, Hq, pool, budget, scale=scale)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    W, pool, budget, scale, return_pooled=True)
    idx_noscale, _ = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens, W, pool,
                                          budget, 1.0)
    assert (idx_noscale != idx_ref).any(axis=2).sum() >= len(lens) * Hkv // 2
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, W, budget)
    record(f"snapkv scale {name}", units=len(lens) * Hkv, near_tie=near)
    assert near <= 1


@pytest.mark.parametrize("classes", [1, 5, 64])
def test_snapkv_tied_votes(classes):
    """Every key row is one of `classes` vectors, so the votes tie in large
    groups (one value per vector) and the kept set rests on the rule that
    ties go to the lower position. With one vector every prefix vote is equal
    and the kept prefix positions are 0 .. budget - W - 1."""
    lens, W, pool, budget = [20000, 12000], 8, 7, 512
    say(f"snapkv tied votes: classes={classes} lens={lens}")
    kv_t = paged_kv(77, lens, 2, 128, BF16, "cuda", shuffle=True)
    NP, H, P, d = kv_t.k_pages.shape
    g = torch.Generator(device="cpu").manual_seed(700 + classes)
    base = torch.randn(classes, H, d, generator=g).to(BF16)
    cls = (torch.arange(NP * P) * 7919 % classes).view(NP, P)
    kv_t.k_pages.copy_(base[cls].permute(0, 2, 1, 3).contiguous().to("cuda"))
    q_obs = queries(77, 4, (len(lens), W, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    idx, sel = run_snapkv(kv_t, q_obs, W, 8, pool, budget)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    W, pool, budget, 1.0, return_pooled=True)
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, W, budget)
    assert near == 0 if classes == 1 else near <= 1
    if classes == 1:
        for b, L in enumerate(lens):
            want = list(range(budget - W)) + list(range(L - W, L))
            assert (idx[b].cpu().numpy() == np.array(want)).all()


def test_snapkv_is_deterministic():
    kv_t = paged_kv(31, [2500, 1800], 2, 128, BF16, "cuda", shuffle=True, spike_frac=0.1)
    q_obs = queries(31, 4, (2, 16, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    a = run_snapkv(kv_t, q_obs, 16, 8, 7, 128)
    b = run_snapkv(kv_t, q_obs, 16, 8, 7, 128)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_snapkv_then_draft_end_to_end():
    """SnapKV selection feeding the sparse draft kernel equals the oracle chain
    when the selections agree."""
    from tests.gpu_helpers import compare_attn, run_draft

    lens = [1600, 900]
    kv_t = paged_kv(41, lens, 2, 128, BF16, "cuda", shuffle=True, spike_frac=0.1)
    q_obs = queries(41, 4, (2, 8, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    q = queries(41, 1, (2, 1, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    idx, sel = run_snapkv(kv_t, q_obs, 8, 8, 7, 96)
    idx_ref, sel_ref = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens, 8, 7, 96, 1.0)
    if not np.array_equal(idx.cpu().numpy(), idx_ref):
        pytest.skip("selection near-tie; covered by the parity test")
    out, lse = run_draft(kv_t, q, 1, 8, idx, sel)
    o_ref, l_ref = oracle.sparse_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, idx_ref, sel_ref, 1.0)
    compare_attn(out, lse, o_ref, l_ref, BF16)


@pytest.mark.parametrize("lens,pool", [([2000, 1500], 7), ([3000], 131), ([70000], 3)],
                         ids=["register", "radix-wide-pool", "radix-long"])
def test_snapkv_all_ties_take_lowest_positions(lens, pool):
    """All keys zero: every prefix position gets the same vote, bitwise, so the
    kept set is the lowest budget - W positions plus the window."""
    W, budget, Hq, Hkv = 8, 256, 8, 2
    kv_t = paged_kv(57, lens, Hkv, 128 if pool != 3 else 64, BF16, "cuda")
    d = kv_t.k_pages.shape[-1]
    for b, L in enumerate(lens):
        pages = kv_t.page_table[b, :-(-L // kv_t.page_size)].long()
        kv_t.k_pages[pages] = 0
    q_obs = queries(57, 4, (len(lens), W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx, sel = run_snapkv(kv_t, q_obs, W, Hq, pool, budget)
    keep = budget - W
    for b, L in enumerate(lens):
        want = np.concatenate([np.arange(keep), np.arange(L - W, L)])
        assert (idx[b].cpu().numpy() == want).all()
    assert (sel.cpu().numpy() == budget).all()


@pytest.mark.parametrize("page_size", [32, 48])
def test_snapkv_page_sizes(page_size):
    """16-key steps inside larger pages (the K stream's row arithmetic), shuffled."""
    lens = [2000, 3333]
    kv_t = paged_kv(71, lens, 2, 128, BF16, "cuda", shuffle=True, spike_frac=0.1, page_size=page_size)
    q_obs = queries(71, 4, (2, 16, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    idx, sel = run_snapkv(kv_t, q_obs, 16, 8, 7, 256)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    16, 7, 256, 1.0, return_pooled=True)
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, 16, 256)
    assert near <= 1


def test_snapkv_max_len_above_lengths():
    """max_kv_len well above every length: plan, workspace and top-K variant are
    sized from it, the results from the real lengths."""
    lens = [1500, 900]
    kv_t = paged_kv(73, lens, 2, 128, BF16, "cuda", shuffle=True, spike_frac=0.1)
    q_obs = queries(73, 4, (2, 8, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    P = kv_t.page_size
    # let the page table cover max_kv_len: pad it with the spare page
    pad = torch.full((2, 2600 // P), kv_t.spare_page, dtype=torch.int32, device="cuda")
    kv_t = dataclasses.replace(kv_t, page_table=torch.cat([kv_t.page_table, pad], dim=1).contiguous())
    mk = kv_t.page_table.shape[1] * P
    idx, sel = run_snapkv(kv_t, q_obs, 8, 8, 7, 128, max_kv_len=mk)
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    8, 7, 128, 1.0, return_pooled=True)
    near = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, 8, 128)
    assert near <= 1


@pytest.mark.parametrize("name,lens,budgets,Hq,Hkv,W", [
    ("ragged-mixed", [3000, 700, 5000, 1200, 90], [256, 800, 1024, 300, 64], 8, 2, 16),
    ("rows128-mixed", [4100, 2600], [512, 2000], 32, 1, 4),
])
def test_snapkv_per_sequence_budgets(name, lens, budgets, Hq, Hkv, W):
    """A ragged batch with one budget per sequence (some sequences shorter than
    their budget keep everything); then the sparse draft over the per-sequence
    sets."""
    from tests.gpu_helpers import compare_attn, run_draft

    kv_t = paged_kv(91, lens, Hkv, 128, BF16, "cuda", shuffle=True, spike_frac=0.1)
    q_obs = queries(91, 4, (len(lens), W, Hq, 128), BF16, "cuda", scale=128 ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, Kmax = len(lens), max(budgets)
    bud = torch.tensor(budgets, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Hkv, Kmax), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    mk = max(lens)
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, mk), "cuda")
    sd.sd_snapkv_select_budgets(kv, q_obs, W, Hq, 7, bud, Kmax, mk, 1.0, idx, sel, ws)
    torch.cuda.synchronize()
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens, W, 7,
                                                    np.array(budgets), 1.0, return_pooled=True)
    idx_np, sel_np = idx.cpu().numpy(), sel.cpu().numpy()
    assert (sel_np == sel_ref).all()
    near = 0
    for b in range(B):
        K_b = budgets[b]
        assert (idx_np[b, :, min(lens[b], K_b):] == -1).all()
        near += check_selection(idx_np[b:b + 1, :, :K_b], idx_ref[b:b + 1, :, :K_b], sel_np[b:b + 1],
                                sel_ref[b:b + 1], {(0, g): pooled[(b, g)] for g in range(Hkv) if (b, g) in pooled},
                                W, K_b)
    say(f"  {name}: near-tie units {near}")
    assert near <= 1
    q = queries(91, 1, (B, 1, Hq, 128), BF16, "cuda", scale=128 ** -0.5)
    out, lse = run_draft(kv_t, q, 1, Hq, idx, sel)
    if near == 0:
        o_ref, l_ref = oracle.sparse_attn(q.cpu(), kv_t.k_pages.cpu(), kv_t.v_pages.cpu(), kv_t.page_table.cpu(),
                                          idx_ref, sel_ref, 1.0)
        compare_attn(out, lse, o_ref, l_ref, BF16)


LSE_CASES = [
    # name, Hq, Hkv, d, lens, window, pool, budget, spike_frac
    ("g4-w8-rows32", 8, 2, 128, [700, 1500], 8, 7, 64, 0.0),
    ("g4-w32-rows128-spiky", 32, 8, 128, [3000, 2100], 32, 7, 256, 0.10),
    ("short-rows-see-no-key", 8, 2, 128, [5, 0, 2000, 40], 8, 7, 200, 0.0),
    ("d64-pool3", 8, 2, 64, [1234, 517], 4, 3, 100, 0.10),
    ("rows48-ragged-pages", 24, 2, 128, [1111, 4096, 333], 4, 5, 300, 0.05),
    ("prefix-40k", 8, 2, 64, [40000, 33000], 8, 5, 2048, 0.10),
]
LSE_BAR = 3e-5  # fp32 sums of exact bf16 products over up to 40k keys, lse ~ 10


@pytest.mark.parametrize("case", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_snapkv_window_lse_and_select_from_it(case):
    """sd_snapkv_window_lse against the oracle's verify attention of the window
    queries (query w of the window attends to 0 .. L - W + w, exactly step 1
    of the selection), including rows that see no key; then
    sd_snapkv_select_lse fed (a) those values and (b) the oracle's own
    normalisers, each against the oracle's selection, and (a) against
    sd_snapkv_select."""
    name, Hq, Hkv, d, lens, W, pool, budget, spike = case
    say(f"snapkv window lse {name}: lens={lens} W={W}")
    seed = zlib.crc32(("lse-" + name).encode()) % 10000
    kv_t = paged_kv(seed, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=spike)
    q_obs = queries(seed, 4, (len(lens), W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B, mk = len(lens), max(1, max(lens))
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, mk), "cuda")
    lse = torch.full((B, W, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sd.sd_snapkv_window_lse(kv, q_obs, W, Hq, mk, 1.0, lse, ws)
    torch.cuda.synchronize()
    _, l_ref = oracle.verify_attn(q_obs, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens, 1.0)
    l = lse.double().cpu().numpy()
    dead = np.isneginf(l_ref)
    assert (np.isneginf(l) == dead).all(), "rows with no visible key differ"
    lerr = np.abs(l[~dead] - l_ref[~dead]).max() if (~dead).any() else 0.0
    say(f"  window lse: max err {lerr:.2e}, rows without keys {int(dead.sum())}")
    assert lerr <= LSE_BAR, lerr
    idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs, kv_t.k_pages, kv_t.page_table, kv_t.kv_lens,
                                                    W, pool, budget, 1.0, return_pooled=True)
    idx_full, sel_full = run_snapkv(kv_t, q_obs, W, Hq, pool, budget)
    near = {}
    for tag, given in (("own", lse), ("oracle", torch.from_numpy(l_ref).float().cuda())):
        idx = torch.full((B, Hkv, budget), 7, dtype=torch.int32, device="cuda")
        sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
        sd.sd_snapkv_select_lse(kv, q_obs, given, W, Hq, pool, budget, mk, 1.0, idx, sel,
                                dirty_workspace(ws.numel(), "cuda"))
        torch.cuda.synchronize()
        near[tag] = check_selection(idx.cpu().numpy(), idx_ref, sel.cpu().numpy(), sel_ref, pooled, W, budget)
        if tag == "own":
            same = int((idx == idx_full).all(dim=2).sum())
            say(f"  from own lse: {same} of {B * Hkv} units equal sd_snapkv_select's")
            assert torch.equal(sel, sel_full)
    say(f"  near-tie units: {near}")
    record(f"snapkv window lse {name}", rows=int((~dead).sum()), max_lse=float(lerr), near_tie_own=near["own"],
           near_tie_oracle=near["oracle"])
    assert max(near.values()) <= max(1, B * Hkv // 8)
