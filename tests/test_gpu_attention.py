"""GPU parity of verify and sparse draft attention against the CPU oracle.

Small seeded cases that span several 16-token steps, several split-KV chunks,
ragged and shuffled pages, partial last pages (NaN-poisoned tails), every
query-row tile count (NB = 1..4), head_dim 64/128, bf16 and fp32, page size 32,
and the degenerate lengths (kv_len == n_q, kv_len < n_q, empty sequences,
empty selections).
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
from synth import paged_kv, queries
from tests.gpu_helpers import compare_attn, ensure_lib, run_draft, run_verify, say

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


# More sequences than the planning block covers in one pass (1024), and more
# (sequence, KV head) units than resident waves: the schedule's multi-pass
# prefix sums and units that share a wave.
MANY = np.random.default_rng(5).integers(0, 91, 2500).tolist()

VERIFY_CASES = [
    # name, dtype, Hq, Hkv, d, lens, n_q, shuffle, page_size
    ("tiny-f32-b2-l256", F32, 8, 2, 64, [256, 256], 4, False, 16),
    ("bf16-ragged-multichunk", BF16, 8, 2, 128, [37, 300, 1029], 4, True, 16),
    ("bf16-rows20", BF16, 32, 8, 128, [700, 1500], 5, True, 16),
    ("bf16-rows40", BF16, 16, 2, 128, [900, 333], 5, True, 16),
    ("bf16-rows64", BF16, 16, 1, 128, [600], 4, False, 16),
    ("bf16-d64", BF16, 8, 2, 64, [513, 77], 3, True, 16),
    ("f32-d128", F32, 8, 2, 128, [200, 1111], 2, True, 16),
    ("f32-d64-rows40", F32, 16, 2, 64, [450, 97], 5, True, 16),
    ("bf16-page32", BF16, 8, 2, 128, [100, 1000], 4, True, 32),
    ("bf16-short", BF16, 8, 2, 128, [4, 3, 0, 1], 4, False, 16),
    ("bf16-decode-exact-pages", BF16, 8, 2, 128, [512, 1024], 1, True, 16),
    ("bf16-2500-sequences", BF16, 8, 2, 128, MANY, 4, True, 16),
    # one long sequence: each unit spread over about a thousand waves, so the
    # combine merges ~1000 slots per row (its chunked slot loop)
    ("bf16-one-300k-sequence", BF16, 8, 2, 128, [300000], 4, True, 16),
    # 37 sequences x 8 KV heads x 256 steps: shares of 74 steps over 1024
    # resident waves, straddling unit boundaries; segments this short take
    # their steps in order
    ("bf16-37-step-shares", BF16, 32, 8, 128, [4096] * 37, 5, False, 16),
]


@pytest.mark.parametrize("case", VERIFY_CASES, ids=[c[0] for c in VERIFY_CASES])
def test_verify_parity(case):
    name, dtype, Hq, Hkv, d, lens, n_q, shuffle, P = case
    say(f"verify {name}: lens={lens} n_q={n_q} Hq={Hq} Hkv={Hkv} d={d} {dtype}")
    seed = zlib.crc32(name.encode()) % 10000
    kv_t = paged_kv(seed, lens, Hkv, d, dtype, "cuda", shuffle=shuffle, page_size=P)
    q = queries(seed, 1, (len(lens), n_q, Hq, d), dtype, "cuda", scale=d ** -0.5)
    out, lse = run_verify(kv_t, q, n_q, Hq, scale=1.0)
    o_ref, l_ref = oracle.verify_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, dtype)
    say(f"  max|dO|={err[0]:.3e} norm={err[1]:.3e} lse={err[2]:.3e}")


def test_verify_softmax_scale_argument():
    lens = [333, 800]
    kv_t = paged_kv(5, lens, 2, 128, BF16, "cuda", shuffle=True)
    q = queries(5, 1, (2, 4, 8, 128), BF16, "cuda", scale=1.0)
    out, lse = run_verify(kv_t, q, 4, 8, scale=128 ** -0.5)
    o_ref, l_ref = oracle.verify_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens,
                                      128 ** -0.5)
    compare_attn(out, lse, o_ref, l_ref, BF16)


SHARP_CASES = [
    # name, dtype, softmax_scale, ramp (score added linearly from 0 at position 0)
    ("sharp-bf16", BF16, 8.0, 0.0),
    ("sharp-f32", F32, 8.0, 0.0),
    ("rising-bf16", BF16, 1.0, 80.0),
    ("falling-bf16", BF16, 1.0, -80.0),
    ("rising-f32", F32, 1.0, 80.0),
]


@pytest.mark.parametrize("case", SHARP_CASES, ids=[c[0] for c in SHARP_CASES])
def test_attention_with_sharp_or_trending_scores(case):
    """Peaked softmax (scale 8 on unit-variance scores) and scores that rise or
    fall by 80 over each sequence: every query row has a component along one
    direction u that the keys carry with a weight growing in the position, so
    the running maximum moves at nearly every step (rising) or is set by the
    first one (falling). Verify (one sequence long enough for the permuted
    walk) and the draft over every position, in ascending and in descending
    order, against the oracle."""
    name, dtype, scale, ramp = case
    lens = [5000, 700]
    B, Hkv, Hq, d, n_q = len(lens), 2, 8, 128, 4
    say(f"sharp/trending scores {name}")
    kv_t = paged_kv(71, lens, Hkv, d, dtype, "cuda", shuffle=True)
    g = torch.Generator(device="cuda").manual_seed(71)
    u = torch.randn(d, generator=g, device="cuda")
    u /= u.norm()
    P = kv_t.page_size
    for b, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        page = kv_t.page_table[b].long()[t // P]
        for pool in (kv_t.k_pages,):
            rows = pool[page, :, t % P, :].float() + (ramp * t / L)[:, None, None] * u
            pool[page, :, t % P, :] = rows.to(dtype)
    q = (queries(71, 1, (B, n_q, Hq, d), torch.float32, "cuda", scale=d ** -0.5) + u).to(dtype)
    # largest |score| of each (sequence, query row, head) over the sequence's keys
    mag = np.zeros((B, n_q, Hq))
    for b, L in enumerate(lens):
        t = torch.arange(L, device="cuda")
        k = kv_t.k_pages[kv_t.page_table[b].long()[t // P], :, t % P, :].float()      # [L, Hkv, d]
        k = k.repeat_interleave(Hq // Hkv, dim=1)                                    # [L, Hq, d]
        s_ = torch.matmul(q[b].float().permute(1, 0, 2).contiguous(), k.permute(1, 2, 0).contiguous()) * scale
        mag[b] = s_.abs().amax(dim=2).permute(1, 0).cpu().numpy()                   # [n_q, Hq]
    out, lse = run_verify(kv_t, q, n_q, Hq, scale=scale)
    o_ref, l_ref = oracle.verify_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens, scale)
    err = compare_attn(out, lse, o_ref, l_ref, dtype, score_mag=mag)
    say(f"  verify max|dO|={err[0]:.2e} norm={err[1]:.2e} lse/factor={err[2]:.2e}, "
        f"|s|max up to {mag.max():.1f}")
    qd = q[:, :1].contiguous()
    for order in ("ascending", "descending"):
        idx_np = np.full((B, 1, max(lens)), -1, dtype=np.int32)
        for b, L in enumerate(lens):
            idx_np[b, 0, :L] = np.arange(L) if order == "ascending" else np.arange(L)[::-1]
        idx = torch.tensor(idx_np).cuda()
        sel = torch.tensor(lens, dtype=torch.int32).cuda()
        out_d, lse_d = run_draft(kv_t, qd, 1, Hq, idx, sel, scale=scale)
        o_ref, l_ref = oracle.sparse_attn(qd, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, idx, sel, scale)
        err = compare_attn(out_d, lse_d, o_ref, l_ref, dtype, score_mag=mag[:, :1])
        say(f"  draft {order}: max|dO|={err[0]:.2e} norm={err[1]:.2e} lse={err[2]:.2e}")


def test_verify_is_deterministic():
    lens = [2000, 1700, 900]
    kv_t = paged_kv(6, lens, 2, 128, BF16, "cuda", shuffle=True)
    q = queries(6, 1, (3, 4, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    a = run_verify(kv_t, q, 4, 8)
    b = run_verify(kv_t, q, 4, 8)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_verify_page_permutation_invariance():
    """The same tokens under two physical page orders give identical bits."""
    lens = [700, 1200]
    kv1 = paged_kv(7, lens, 2, 128, BF16, "cuda", shuffle=False)
    perm = torch.randperm(kv1.k_pages.shape[0], generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    kv2 = paged_kv(7, lens, 2, 128, BF16, "cuda", shuffle=False)
    kv2.k_pages = kv1.k_pages[perm.cuda()].contiguous()
    kv2.v_pages = kv1.v_pages[perm.cuda()].contiguous()
    kv2.page_table = inv.cuda()[kv1.page_table.long()].to(torch.int32).contiguous()
    q = queries(7, 1, (2, 4, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    a = run_verify(kv1, q, 4, 8)
    b = run_verify(kv2, q, 4, 8)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _random_sets(seed, lens, heads, max_sel, min_frac=0.05):
    rng = np.random.default_rng(seed)
    B = len(lens)
    idx = np.full((B, heads, max_sel), -1, dtype=np.int32)
    sel = np.zeros(B, dtype=np.int32)
    for b, L in enumerate(lens):
        n = int(min(L, rng.integers(max(1, int(min_frac * max_sel)), max_sel + 1)))
        sel[b] = n
        for g in range(heads):
            pos = np.sort(rng.choice(L, size=n, replace=False)) if n else np.zeros(0, np.int64)
            if g % 2 == 1:
                pos = pos[::-1]          # order is irrelevant to the result
            idx[b, g, :n] = pos
    return torch.tensor(idx).cuda(), torch.tensor(sel).cuda()


DRAFT_CASES = [
    # name, dtype, Hq, Hkv, d, lens, n_q, idx_heads ("shared" or "per-head"), max_sel
    ("stream-shared-bf16", BF16, 8, 2, 128, [300, 50, 2000], 1, "streaming", 64),
    ("stream-tiny-f32", F32, 8, 2, 64, [256, 256], 1, "streaming", 64),
    ("per-head-bf16", BF16, 8, 2, 128, [1500, 800, 40], 1, "per-head", 256),
    ("per-head-bf16-nq2", BF16, 32, 8, 128, [3000, 700], 2, "per-head", 600),
    ("shared-bf16-d64", BF16, 8, 2, 64, [999, 1234], 1, "shared", 333),
    ("per-head-f32-d128", F32, 16, 2, 128, [777, 1500], 1, "per-head", 200),
    ("per-head-rows64", BF16, 16, 1, 128, [1800], 4, "per-head", 700),
    # two and three row tiles in the draft (20 and 40 query rows per unit)
    ("per-head-rows20", BF16, 32, 8, 128, [2500, 900], 5, "per-head", 640),
    ("shared-rows40", BF16, 64, 8, 128, [1700, 3100], 5, "shared", 512),
    ("stream-2500-sequences", BF16, 8, 2, 128, MANY, 1, "streaming", 48),
    ("per-head-2500-sequences", BF16, 8, 2, 128, MANY, 1, "per-head", 40),
    # one long selection (up to 120k of 250k positions): many resolved
    # sub-chunks per wave and many slots per unit
    ("shared-bf16-long-selection", BF16, 8, 2, 128, [250000], 1, "shared", 120000),
]


@pytest.mark.parametrize("case", DRAFT_CASES, ids=[c[0] for c in DRAFT_CASES])
def test_draft_parity(case):
    name, dtype, Hq, Hkv, d, lens, n_q, kind, max_sel = case
    say(f"draft {name}: lens={lens} n_q={n_q} {kind} max_sel={max_sel} {dtype}")
    seed = zlib.crc32(name.encode()) % 10000
    kv_t = paged_kv(seed, lens, Hkv, d, dtype, "cuda", shuffle=True)
    q = queries(seed, 1, (len(lens), n_q, Hq, d), dtype, "cuda", scale=d ** -0.5)
    if kind == "streaming":
        idx_np = np.full((len(lens), 1, max_sel), -1, dtype=np.int32)
        sel_np = np.zeros(len(lens), dtype=np.int32)
        for b, L in enumerate(lens):
            keep = sorted(set(range(min(16, L))) | set(range(max(0, L - (max_sel - 16)), L)))
            idx_np[b, 0, :len(keep)] = keep
            sel_np[b] = len(keep)
        idx, sel = torch.tensor(idx_np).cuda(), torch.tensor(sel_np).cuda()
    else:
        idx, sel = _random_sets(seed, lens, Hkv if kind == "per-head" else 1, max_sel)
    out, lse = run_draft(kv_t, q, n_q, Hq, idx, sel)
    o_ref, l_ref = oracle.sparse_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, idx, sel, 1.0)
    err = compare_attn(out, lse, o_ref, l_ref, dtype)
    say(f"  max|dO|={err[0]:.3e} norm={err[1]:.3e} lse={err[2]:.3e}")


def test_draft_empty_selection_and_full_budget_equals_verify_decode():
    lens = [500, 640]
    kv_t = paged_kv(9, lens, 2, 128, BF16, "cuda", shuffle=True)
    q = queries(9, 1, (2, 1, 8, 128), BF16, "cuda", scale=128 ** -0.5)
    idx = torch.full((2, 1, 700), -1, dtype=torch.int32, device="cuda")
    idx[0, 0, :500] = torch.arange(500, dtype=torch.int32)
    idx[1, 0, :640] = torch.arange(640, dtype=torch.int32)
    sel = torch.tensor([500, 0], dtype=torch.int32, device="cuda")
    out, lse = run_draft(kv_t, q, 1, 8, idx, sel)
    assert (out[1] == 0).all() and torch.isneginf(lse[1]).all()
    ref, lref = run_verify(kv_t, q, 1, 8)
    o_ref, l_ref = oracle.verify_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens, 1.0)
    compare_attn(out[:1], lse[:1], o_ref[:1], l_ref[:1], BF16)
    compare_attn(ref, lref, o_ref, l_ref, BF16)


@pytest.mark.parametrize("Hq,Hkv,n_q,draft_heads", [
    (8, 2, 4, "shared"),       # G * n_q = 16 rows: one full tile
    (6, 2, 5, "per-head"),     # G = 3, 15 rows; the draft with one set per query head
])
def test_one_launch_and_split_paths_agree(Hq, Hkv, n_q, draft_heads):
    """Calls whose units all fit one round of the chip and hold at most 1024
    tokens run one workgroup per unit (no split, no combine). The same inputs
    with a length bound above that limit (a wider page table, a longer index
    row) take the persistent split + combine path. Both must meet the oracle
    bars, verify and draft alike."""
    lens = [600, 333, 1000, 17, 0, 1024]
    d = 128
    kv_t = paged_kv(77, lens, Hkv, d, BF16, "cuda", shuffle=True)
    q = queries(77, 1, (len(lens), n_q, Hq, d), BF16, "cuda", scale=d ** -0.5)
    o_ref, l_ref = oracle.verify_attn(q, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens, 1.0)
    spare = kv_t.page_table[4, -1].item()   # the empty sequence's entries point at the spare page
    wide_pt = torch.cat([kv_t.page_table, torch.full((len(lens), 192), spare, dtype=torch.int32,
                                                     device="cuda")], dim=1).contiguous()
    wide = dataclasses.replace(kv_t, page_table=wide_pt)
    one, one_l = run_verify(kv_t, q, n_q, Hq, max_kv_len=1024)
    split, split_l = run_verify(wide, q, n_q, Hq, max_kv_len=4096)
    compare_attn(one, one_l, o_ref, l_ref, BF16)
    compare_attn(split, split_l, o_ref, l_ref, BF16)

    qd = q[:, :1].contiguous()
    if draft_heads == "shared":
        idx_np = np.full((len(lens), 1, 512), -1, dtype=np.int32)
        sel_np = np.zeros(len(lens), dtype=np.int32)
        for b, L in enumerate(lens):
            keep = sorted(set(range(min(64, L))) | set(range(max(0, L - 448), L)))
            idx_np[b, 0, :len(keep)] = keep
            sel_np[b] = len(keep)
        idx, sel = torch.tensor(idx_np).cuda(), torch.tensor(sel_np).cuda()
    else:
        idx, sel = _random_sets(78, lens, Hq, 512)
    idx_wide = torch.full((len(lens), idx.shape[1], 2048), -1, dtype=torch.int32, device="cuda")
    idx_wide[:, :, :512] = idx
    d_ref, dl_ref = oracle.sparse_attn(qd, kv_t.k_pages, kv_t.v_pages, kv_t.page_table, idx, sel, 1.0)
    one, one_l = run_draft(kv_t, qd, 1, Hq, idx, sel)
    split, split_l = run_draft(kv_t, qd, 1, Hq, idx_wide.contiguous(), sel)
    compare_attn(one, one_l, d_ref, dl_ref, BF16)
    compare_attn(split, split_l, d_ref, dl_ref, BF16)
