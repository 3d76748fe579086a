"""Full-size parity: every bf16 workload at its real shape, through the same
entry points and launch plan the benchmark uses, checked against the oracle on
sampled (sequence, KV head) units (the oracle computes one unit at a time from
the unit's pages copied to the host), plus properties that must hold for every
output (finite values, dead-row conventions, selection structure).

Workloads: Llama-3.1-8B shapes B=32 / 8k and B=128 / 32k (SnapKV), the ragged
B=256 batch with 4k-32k lengths on shuffled pages, and Llama-3.1-70B shapes
B=64 / 16k (64/8 heads).
"""
import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
import oracle
from synth import WORKLOADS, dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries, workload_lens
from tests.gpu_helpers import (BF16_LSE, check_accept, compare_attn, dirty_workspace, ensure_lib, gathered_decode,
                               say, unit_cache)
from tests.parity_log import record

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def sample_sequences(lens, Hkv, seed, n_seq=8):
    """Every KV head of n_seq sequences: the first, the last, the shortest, the
    longest and random others (n_seq * Hkv units)."""
    B = len(lens)
    rng = np.random.default_rng(seed)
    seqs = {0, B - 1, int(np.argmin(lens)), int(np.argmax(lens))}
    while len(seqs) < min(n_seq, B):
        seqs.add(int(rng.integers(B)))
    return [(b, g) for b in sorted(seqs) for g in range(Hkv)]


def build(name):
    w = WORKLOADS[name]
    lens = workload_lens(w)
    d = w.head_dim
    kv_t = paged_kv(w.seed, lens, w.num_kv_heads, d, BF16, "cuda", shuffle=w.shuffle, spike_frac=w.spike_frac)
    q = queries(w.seed, 1, (w.batch, w.gamma + 1, w.num_q_heads, d), BF16, "cuda", scale=d ** -0.5)
    return w, lens, kv_t, q


def check_units_verify(w, lens, kv_t, q, out, lse, units, label):
    G = w.num_q_heads // w.num_kv_heads
    worst = np.zeros(3)
    for b, g in units:
        k, v, table, L = unit_cache(kv_t, b, g)
        heads = slice(g * G, (g + 1) * G)
        o_ref, l_ref = oracle.verify_attn(q[b:b + 1, :, heads].cpu(), k, v, table, L, 1.0)
        err = compare_attn(out[b:b + 1, :, heads], lse[b:b + 1, :, heads], o_ref, l_ref, BF16)
        worst = np.maximum(worst, err)
    record(label, units=len(units), max_abs=float(worst[0]), max_norm=float(worst[1]), max_lse=float(worst[2]))
    say(f"  {label}: {len(units)} units, worst max|dO|={worst[0]:.2e} norm={worst[1]:.2e} lse={worst[2]:.2e}")


def check_draft_against_gathered(label, out, lse, kv_t, idx, sel, qd, num_q_heads):
    """Every unit of a full-size draft against the dense decode over its
    gathered rows (different kernels and splits: the bf16 bars)."""
    o_ref, l_ref = gathered_decode(kv_t, idx, sel, qd, num_q_heads)
    err = compare_attn(out, lse, o_ref.double().cpu().numpy(), l_ref.double().cpu().numpy(), BF16)
    record(label, rows=int(out.shape[0] * num_q_heads), max_abs=float(err[0]), max_norm=float(err[1]),
           max_lse=float(err[2]))
    say(f"  {label}: max|dO|={err[0]:.2e} norm={err[1]:.2e} lse={err[2]:.2e}")


@pytest.mark.parametrize("name", ["llama8b-b32-l8k", "llama8b-b128-l32k-snapkv", "ragged-b256-l4k-32k",
                                  "llama70b-b64-l16k"])
def test_verify_full_size_sampled(name):
    w, lens, kv_t, q = build(name)
    say(f"verify {name}: B={w.batch} max L={max(lens)} n_q={w.gamma + 1}")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.batch, w.gamma + 1, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(w.batch, w.gamma + 1, w.num_q_heads, w.num_kv_heads,
                                                          w.head_dim, max(lens)), "cuda")
    sd.sd_verify_attn(kv, q, w.gamma + 1, w.num_q_heads, max(lens), 1.0, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    # |o| is a convex combination of V rows: bounded by the largest |V| entry
    assert out.float().abs().max() <= kv_t.v_pages.float().nan_to_num(0).abs().max() + 1e-2
    check_units_verify(w, lens, kv_t, q, out, lse, sample_sequences(lens, w.num_kv_heads, w.seed),
                       f"verify {name} (full size)")


@pytest.mark.parametrize("L,mult", [(4752, 41), (24288, 43)])
def test_verify_walk_fallback_multipliers(L, mult):
    """Verify takes a segment's unmasked steps in the order (A v + rot) mod n
    with A = 37, or 41 when 37 divides n, or 43 when 41 divides n too. With
    2048 units (B = 256, 8 KV heads) of equal length and 1024 or 2048
    resident waves, every wave owns whole units, whose unmasked steps at
    n_q = 5 number L / 16 - 1: 296 = 37 * 8 (A = 41) at L = 4752 and
    1517 = 37 * 41 (A = 43) at L = 24288. Any unit would show a broken walk
    (a step read twice and another skipped); sampled units are checked
    against the oracle."""
    class W:
        num_q_heads, num_kv_heads = 32, 8
    B, n_q, d = 256, 5, 128
    n = L // 16 - 1
    assert n % 37 == 0 and (mult == 41) == (n % 41 != 0)
    lens = [L] * B
    kv_t = paged_kv(mult, lens, 8, d, BF16, "cuda", shuffle=False)
    q = queries(mult, 1, (B, n_q, 32, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, 32), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, n_q, 32, 8, d, L), "cuda")
    sd.sd_verify_attn(kv, q, n_q, 32, L, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    check_units_verify(W, lens, kv_t, q, out, lse, sample_sequences(lens, 8, mult, n_seq=4),
                       f"verify 2048 units of {n} unmasked steps (walk multiplier {mult})")
    del kv_t, kv, q, out, lse, ws
    torch.cuda.empty_cache()


def test_verify_walk_threshold_boundary():
    """Segments at the walk's length threshold: 256 units (B = 32, 8 KV
    heads) of 1024 steps over 1024 resident waves give shares of exactly 256
    steps, a quarter unit each. The first three quarters have 256 unmasked
    steps (permuted walk), the last 255 and the masked step (in order).
    Sampled units against the oracle."""
    class W:
        num_q_heads, num_kv_heads = 32, 8
    B, L, n_q, d = 32, 16384, 5, 128
    lens = [L] * B
    kv_t = paged_kv(256, lens, 8, d, BF16, "cuda", shuffle=False)
    q = queries(256, 1, (B, n_q, 32, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, 32), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, n_q, 32, 8, d, L), "cuda")
    sd.sd_verify_attn(kv, q, n_q, 32, L, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    check_units_verify(W, lens, kv_t, q, out, lse, sample_sequences(lens, 8, 256, n_seq=4),
                       "verify shares of 256 steps (walk threshold)")


@pytest.mark.parametrize("name", ["llama8b-b128-l32k-snapkv", "ragged-b256-l4k-32k", "llama70b-b64-l16k"])
def test_verify_rows_equal_truncated_decodes_every_unit(name):
    """Every unit at full size, by a property: verify's query row i sees
    positions 0 .. L - n_q + i, so it must equal a decode (n_q = 1) of query i
    over the cache truncated to L - n_q + i + 1 tokens. The two calls split
    the work at different points (other step counts, other wave shares), so a
    slot, schedule or combine error anywhere in the batch shows; they agree to
    rounding. The rounding is not only fp32: the PV product takes P in bf16,
    rounded relative to the running max, which depends on where the work is
    split, so outputs near zero (cancellation) differ by ~1e-4 between two
    correct schedules. The two therefore meet the same bf16 bars as against
    the oracle, on all rows of all units."""
    w, lens, kv_t, q = build(name)
    n_q = w.gamma + 1
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    L = max(lens)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, n_q, Hq, Hkv, d, L), "cuda")
    sd.sd_verify_attn(kv, q, n_q, Hq, L, 1.0, out, lse, ws)
    worst = np.zeros(3)
    wsd = dirty_workspace(sd.sd_verify_attn_workspace_size(B, 1, Hq, Hkv, d, L), "cuda")
    for i in range(n_q):
        lens_i = (kv_t.kv_lens - (n_q - 1 - i)).clamp(min=0).to(torch.int32).contiguous()
        kv_i = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, lens_i)
        qi = q[:, i:i + 1].contiguous()
        oi = torch.full_like(qi, float("nan"))
        li = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
        sd.sd_verify_attn(kv_i, qi, 1, Hq, L, 1.0, oi, li, wsd)
        torch.cuda.synchronize()
        ref_o = oi[:, 0].double().cpu().numpy()[:, None]
        ref_l = li[:, 0].double().cpu().numpy()[:, None]
        err = compare_attn(out[:, i:i + 1], lse[:, i:i + 1], ref_o, ref_l, BF16)
        worst = np.maximum(worst, err)
    record(f"verify rows vs truncated decodes {name} (every unit)", units=B * Hkv, rows=B * n_q * Hq,
           max_abs=float(worst[0]), max_norm=float(worst[1]), max_lse=float(worst[2]))
    say(f"  {name}: all {B * Hkv} units, worst max|dO|={worst[0]:.2e} norm={worst[1]:.2e} lse={worst[2]:.2e}")


@pytest.mark.parametrize("name", ["llama8b-b32-l8k", "ragged-b256-l4k-32k"])
def test_streaming_draft_full_size_sampled(name):
    w, lens, kv_t, q = build(name)
    say(f"streaming draft {name}: sink={w.sink} recent={w.recent}")
    B, cap = w.batch, w.sink + w.recent
    idx = torch.empty((B, 1, cap), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    sd.sd_streaming_select(kv_t.kv_lens, w.sink, w.recent, idx, sel)
    qd = q[:, :1].contiguous()
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, 1, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                                cap), "cuda")
    sd.sd_draft_attn_sparse(kv, qd, 1, w.num_q_heads, idx, sel, 1, cap, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    idx_ref, sel_ref = oracle.streaming_select(np.array(lens), w.sink, w.recent)
    assert (idx.cpu().numpy() == idx_ref).all() and (sel.cpu().numpy() == sel_ref).all()
    assert torch.isfinite(out).all()
    G = w.num_q_heads // w.num_kv_heads
    units = sample_sequences(lens, w.num_kv_heads, w.seed + 1)
    worst = np.zeros(3)
    for b, g in units:
        k, v, table, L = unit_cache(kv_t, b, g)
        heads = slice(g * G, (g + 1) * G)
        o_ref, l_ref = oracle.sparse_attn(qd[b:b + 1, :, heads].cpu(), k, v, table, idx_ref[b:b + 1],
                                          sel_ref[b:b + 1], 1.0)
        err = compare_attn(out[b:b + 1, :, heads], lse[b:b + 1, :, heads], o_ref, l_ref, BF16)
        worst = np.maximum(worst, err)
    record(f"StreamingLLM draft {name} (full size)", units=len(units), max_abs=float(worst[0]),
           max_norm=float(worst[1]), max_lse=float(worst[2]))
    check_draft_against_gathered(f"StreamingLLM draft {name} vs dense decode over its rows (every unit)",
                                 out, lse, kv_t, idx, sel, qd, w.num_q_heads)


def torch_snapkv_pooled(kv_t, q_obs, b, window, pool_kernel, L):
    """Pooled votes of every KV head of sequence b, by plain PyTorch fp32 on
    the GPU (the definition: causal window softmax, votes summed over the
    group's window rows, clipped max pool): [Hkv, L - W]."""
    _, Hkv, P, d = kv_t.k_pages.shape
    Hq = q_obs.shape[2]
    G = Hq // Hkv
    npg = (L + P - 1) // P
    pages = kv_t.page_table[b, :npg].long()
    k = kv_t.k_pages[pages].float().permute(1, 0, 2, 3).reshape(Hkv, npg * P, d)[:, :L]   # [Hkv, L, d]
    qw = q_obs[b].float().reshape(window, Hkv, G, d).permute(1, 0, 2, 3).reshape(Hkv, window * G, d)
    s = torch.bmm(qw, k.transpose(1, 2).contiguous())                                      # [Hkv, W*G, L]
    row_w = torch.arange(window, device="cuda").repeat_interleave(G)                       # window row of each
    lim = (L - window + row_w).view(1, -1, 1)
    s = s.masked_fill(torch.arange(L, device="cuda").view(1, 1, L) > lim, float("-inf"))
    p = torch.softmax(s, dim=-1)
    votes = p[:, :, :L - window].sum(dim=1)                                                  # [Hkv, L - W]
    half = pool_kernel // 2
    return torch.nn.functional.max_pool1d(votes.unsqueeze(1), pool_kernel, stride=1, padding=half).squeeze(1)


def test_snapkv_select_and_draft_full_size_sampled():
    """B=128, 32k context: SnapKV selection (W=32, pool 7, budget 2048) and the
    sparse draft over it, each compared on sampled units; a unit's draft output
    is compared when its selection matches the oracle's exactly."""
    name = "llama8b-b128-l32k-snapkv"
    w, lens, kv_t, q = build(name)
    B, Hkv, G, d = w.batch, w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.head_dim
    q_obs = queries(w.seed, 4, (B, w.window, w.num_q_heads, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    idx = torch.full((B, Hkv, w.budget), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, w.window, w.num_q_heads, Hkv, max(lens)), "cuda")
    sd.sd_snapkv_select(kv, q_obs, w.window, w.num_q_heads, w.pool_kernel, w.budget, max(lens), 1.0, idx, sel, ws)
    qd = q[:, :1].contiguous()
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, 1, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    wsd = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, w.num_q_heads, Hkv, d, w.budget), "cuda")
    sd.sd_draft_attn_sparse(kv, qd, 1, w.num_q_heads, idx, sel, Hkv, w.budget, 1.0, out, lse, wsd)
    torch.cuda.synchronize()
    idx_np, sel_np = idx.cpu().numpy(), sel.cpu().numpy()
    assert (sel_np == w.budget).all() and torch.isfinite(out).all()
    # structure of every selection: ascending, distinct, in range, window kept
    L = lens[0]
    assert (np.diff(idx_np, axis=2) > 0).all() and idx_np.min() >= 0 and idx_np.max() < L
    assert (idx_np[:, :, -w.window:] == np.arange(L - w.window, L)).all()
    near, compared = 0, 0
    worst = np.zeros(3)
    units = sample_sequences(lens, Hkv, w.seed + 2)
    for b, g in units:
        k, v, table, Lb = unit_cache(kv_t, b, g)
        heads = slice(g * G, (g + 1) * G)
        idx_ref, sel_ref, pooled = oracle.snapkv_select(q_obs[b:b + 1, :, heads].cpu(), k, table, Lb, w.window,
                                                        w.pool_kernel, w.budget, 1.0, return_pooled=True)
        got, ref = idx_np[b, g], idx_ref[0, 0]
        if not np.array_equal(got, ref):
            pv = pooled[(0, 0)]
            thr = np.sort(pv)[::-1][w.budget - w.window - 1]
            for t in set(got.tolist()) ^ set(ref.tolist()):
                assert abs(pv[t] - thr) <= 1e-5 * thr, (b, g, t, pv[t], thr)
            near += 1
            continue
        o_ref, l_ref = oracle.sparse_attn(qd[b:b + 1, :, heads].cpu(), k, v, table, idx_ref, sel_ref, 1.0)
        err = compare_attn(out[b:b + 1, :, heads], lse[b:b + 1, :, heads], o_ref, l_ref, BF16)
        worst = np.maximum(worst, err)
        compared += 1
    stats = dict(units=len(units), selection_exact=compared, near_tie=near, draft_max_abs=float(worst[0]),
                 draft_max_norm=float(worst[1]), draft_max_lse=float(worst[2]))
    record("snapkv select + draft B=128 L=32k (full size)", **stats)
    say(f"  {stats}")
    check_draft_against_gathered("snapkv draft B=128 L=32k vs dense decode over its rows (every unit)",
                                 out, lse, kv_t, idx, sel, qd, w.num_q_heads)
    # every unit's selection against a plain PyTorch fp32 reference of the
    # definition: the kept prefix positions are the budget - W largest pooled
    # votes (ties to the lower position); fp32 against fp32 in another order,
    # so positions may differ only within 1e-5 of the cut
    keep = w.budget - w.window
    differ_units = 0
    for b in range(B):
        pooled = torch_snapkv_pooled(kv_t, q_obs, b, w.window, w.pool_kernel, lens[b])     # [Hkv, L - W]
        order = torch.sort(-pooled, dim=1, stable=True).indices[:, :keep]
        thr = torch.gather(pooled, 1, order[:, -1:])
        ref = torch.sort(order, dim=1).values.cpu().numpy()
        pooled_np, thr_np = pooled.cpu().numpy(), thr.cpu().numpy()[:, 0]
        for g in range(Hkv):
            got = idx_np[b, g, :keep]
            if np.array_equal(got, ref[g]):
                continue
            differ_units += 1
            for t in set(got.tolist()) ^ set(ref[g].tolist()):
                assert abs(pooled_np[g, t] - thr_np[g]) <= 1e-5 * thr_np[g], (b, g, t, pooled_np[g, t], thr_np[g])
    record("snapkv select B=128 L=32k vs PyTorch fp32 (every unit)", units=B * Hkv, near_tie_units=differ_units)
    say(f"  every unit vs PyTorch fp32: {differ_units} of {B * Hkv} units differ, all within the near-tie band")
    # fp32 vs fp64 ordering of pooled votes within 1e-5 of the cut: about one
    # unit in a hundred is expected at this shape
    assert len(units) >= 64 and near <= 3, stats

    # the same selection copied into a cache of its own: every row of every
    # unit equals the source row the selection names (a gather by torch
    # indexing), and the dense decode over the copy is the draft
    P = kv_t.page_size
    pps = w.budget // P
    k_c = torch.full((B * pps, Hkv, P, d), float("nan"), dtype=BF16, device="cuda")
    v_c = torch.full_like(k_c, float("nan"))
    sd.sd_kv_compact(kv, idx, sel, Hkv, w.budget, pps, k_c, v_c)
    pos = idx.long()                                                   # [B, Hkv, budget]
    pages = torch.gather(kv_t.page_table.long(), 1, (pos // P).view(B, -1)).view(B, Hkv, w.budget)
    heads_i = torch.arange(Hkv, device="cuda").view(1, Hkv, 1)
    for pool, copy in ((kv_t.k_pages, k_c), (kv_t.v_pages, v_c)):
        want = pool[pages, heads_i, pos % P]                           # [B, Hkv, budget, d]
        got = copy.view(B, pps, Hkv, P, d).permute(0, 2, 1, 3, 4).reshape(B, Hkv, w.budget, d)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    kvc = sd.KVCache(k_c, v_c, torch.arange(B * pps, dtype=torch.int32, device="cuda").view(B, pps), sel)
    out_c = torch.full_like(qd, float("nan"))
    lse_c = torch.full_like(lse, float("nan"))
    wsc = dirty_workspace(sd.sd_verify_attn_workspace_size(B, 1, w.num_q_heads, Hkv, d, w.budget), "cuda")
    sd.sd_verify_attn(kvc, qd, 1, w.num_q_heads, w.budget, 1.0, out_c, lse_c, wsc)
    torch.cuda.synchronize()
    check_draft_against_gathered("snapkv draft as a dense decode over the compact copy (every unit)",
                                 out_c, lse_c, kv_t, idx, sel, qd, w.num_q_heads)


def test_snapkv_two_calls_full_size():
    """B=128, 32k context: sd_snapkv_window_lse on sampled units against the
    oracle's verify attention of the window queries, and the selection from
    those normalisers (sd_snapkv_select_lse) against the one-call selection on
    every unit: equal, or different only at near ties of the plain PyTorch
    fp32 pooled votes (within 1e-5 of the cut)."""
    w, lens, kv_t, _ = build("llama8b-b128-l32k-snapkv")
    B, Hq, Hkv, G, d, W = w.batch, w.num_q_heads, w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.head_dim, w.window
    L = max(lens)
    q_obs = queries(w.seed, 4, (B, W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L), "cuda")
    lse = torch.full((B, W, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sd.sd_snapkv_window_lse(kv, q_obs, W, Hq, L, 1.0, lse, ws)
    idx1 = torch.full((B, Hkv, w.budget), 7, dtype=torch.int32, device="cuda")
    sel1 = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    sd.sd_snapkv_select(kv, q_obs, W, Hq, w.pool_kernel, w.budget, L, 1.0, idx1, sel1, ws)
    idx2 = torch.full_like(idx1, 7)
    sel2 = torch.full_like(sel1, 7)
    sd.sd_snapkv_select_lse(kv, q_obs, lse, W, Hq, w.pool_kernel, w.budget, L, 1.0, idx2, sel2, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.equal(sel1, sel2)
    worst = 0.0
    units = sample_sequences(lens, Hkv, w.seed + 5, n_seq=4)
    for b, g in units:
        k, v, table, Lb = unit_cache(kv_t, b, g)
        heads = slice(g * G, (g + 1) * G)
        _, l_ref = oracle.verify_attn(q_obs[b:b + 1, :, heads].cpu(), k, v, table, Lb, 1.0)
        worst = max(worst, float(np.abs(lse[b:b + 1, :, heads].double().cpu().numpy() - l_ref).max()))
    # the lse bar of every attention output (fp32 sums over 32k keys, some
    # boosted 4x: lse values near 15 carry ~3e-6 relative rounding)
    assert worst <= BF16_LSE, worst
    same = (idx1 == idx2).all(dim=2)
    differ = 0
    for b in (~same).any(dim=1).nonzero().flatten().tolist():
        pooled = torch_snapkv_pooled(kv_t, q_obs, b, W, w.pool_kernel, lens[b])
        keep = w.budget - W
        thr = torch.sort(pooled, dim=1, descending=True).values[:, keep - 1].cpu().numpy()
        pn = pooled.cpu().numpy()
        for g in range(Hkv):
            if bool(same[b, g]):
                continue
            differ += 1
            a, r = idx1[b, g].cpu().numpy(), idx2[b, g].cpu().numpy()
            for t in set(a.tolist()) ^ set(r.tolist()):
                assert abs(pn[g, t] - thr[g]) <= 1e-5 * thr[g], (b, g, t, pn[g, t], thr[g])
    record("snapkv two calls B=128 L=32k", lse_units=len(units), max_lse=worst, units=B * Hkv,
           units_differing_from_one_call=differ)
    say(f"  two calls: window lse worst {worst:.2e} on {len(units)} units; {differ} of {B * Hkv} selections "
        f"differ from the one-call selection (near ties)")


def test_snapkv_per_sequence_budgets_full_size_every_unit():
    """The per-sequence-budget workload at full size (B=256, contexts 4096 to
    32768 on shuffled pages, budget_b = L_b / 16 rounded down to 16, clamped to
    [256, 2048], window 32, pool 7): every unit's selection against the plain
    PyTorch fp32 reference (near-ties within 1e-5 of the cut allowed), rows
    padded with -1 past their own budget, and the draft over the per-sequence
    sets equal to a dense decode over the gathered rows."""
    w = WORKLOADS["ragged-b256-l4k-32k"]
    B, Hq, Hkv, d, W, pool = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, 32, 7
    lens = workload_lens(w)
    kv_t = paged_kv(w.seed, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=0.1)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    budgets = [max(256, min(2048, L // 16 // 16 * 16)) for L in lens]
    Kmax, L = max(budgets), max(lens)
    bud = torch.tensor(budgets, dtype=torch.int32, device="cuda")
    q_obs = queries(w.seed, 4, (B, W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    idx = torch.full((B, Hkv, Kmax), 7, dtype=torch.int32, device="cuda")
    sel = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L), "cuda")
    sd.sd_snapkv_select_budgets(kv, q_obs, W, Hq, pool, bud, Kmax, L, 1.0, idx, sel, ws)
    torch.cuda.synchronize()
    ic, sc = idx.cpu().numpy(), sel.cpu().numpy()
    assert list(sc) == [min(Lb, Kb) for Lb, Kb in zip(lens, budgets)]
    differ = 0
    for b in range(B):
        Kb, Lb = budgets[b], lens[b]
        row = ic[b]
        assert (row[:, Kb:] == -1).all() and (np.diff(row[:, :Kb], axis=1) > 0).all()
        assert (row[:, Kb - W:Kb] == np.arange(Lb - W, Lb)).all()
        pooled = torch_snapkv_pooled(kv_t, q_obs, b, W, pool, Lb)
        keep = Kb - W
        order = torch.sort(-pooled, dim=1, stable=True).indices[:, :keep]
        thr = torch.gather(pooled, 1, order[:, -1:]).cpu().numpy()[:, 0]
        ref = torch.sort(order, dim=1).values.cpu().numpy()
        pn = pooled.cpu().numpy()
        for g in range(Hkv):
            if np.array_equal(row[g, :keep], ref[g]):
                continue
            differ += 1
            for t in set(row[g, :keep].tolist()) ^ set(ref[g].tolist()):
                assert abs(pn[g, t] - thr[g]) <= 1e-5 * thr[g], (b, g, t, pn[g, t], thr[g])
    q = queries(w.seed, 1, (B, 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device="cuda")
    wsd = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, Kmax), "cuda")
    sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx, sel, Hkv, Kmax, 1.0, out, lse, wsd)
    o_g, l_g = gathered_decode(kv_t, idx, sel, q, Hq)
    err = compare_attn(out, lse, o_g.double().cpu().numpy(), l_g.double().cpu().numpy(), BF16)
    record("snapkv per-sequence budgets B=256 ragged (every unit)", units=B * Hkv, near_tie_units=differ,
           draft_vs_gathered_max_abs=float(err[0]))
    say(f"  per-sequence budgets: {differ} of {B * Hkv} units differ from torch fp32 (near ties); "
        f"draft vs gathered decode max|dO|={err[0]:.2e}")


def test_accept_bench_shape():
    """B=128, gamma=4 over the 128256-token vocabulary, as in the benchmark."""
    B, gamma, V, seed = 128, 4, 128256, 3
    zt = logits(seed, 8, (B, gamma + 1, V), 2.0, "cuda")
    zd = logits(seed, 9, (B, gamma, V), 0.5, "cuda", base=zt[:, :gamma]).contiguous()
    x = gumbel_tokens(seed, zd)
    ua = dyadic_uniforms(seed, 11, (B, gamma), "cuda")
    us = dyadic_uniforms(seed, 12, (B, gamma + 1), "cuda")
    n = torch.empty((B,), dtype=torch.int32, device="cuda")
    toks = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_spec_accept_workspace_size(B, gamma, V), "cuda")
    sd.sd_spec_accept(zt, zd, x, ua, us, gamma, V, 1.0, n, toks, ws)
    torch.cuda.synchronize()
    check_accept("accept B=128 gamma=4 V=128256 (bench shape)", n.cpu().numpy(), toks.cpu().numpy(),
                 zt, zd, x, ua, us)
