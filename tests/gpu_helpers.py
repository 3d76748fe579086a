"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, cut single (sequence, KV head) units out of a large cache for the
oracle, and compare results with the stated tolerances.

Tolerances (the 2e-2 absolute bf16 bar and the 1e-5 relative fp32 bar, plus
two readings for bf16 where the absolute bar alone is loose at long context,
where |o| is only ~0.02):
  bf16 attention: max|dO| <= 2e-2, max|dO| / max|O_ref| <= 1e-2, |d lse| <= 1e-4;
  fp32 attention: max|dO| / max|O_ref| <= 1e-5, |d lse| <= 1e-5.
For inputs whose scores reach a magnitude S well past the workloads' (about
4), the lse bars and the fp32 output bar scale by max(1, S / 4): see
compare_attn.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import long_context_kv_split_amd as sd  # noqa: E402
import oracle  # noqa: E402
from long_context_kv_split_amd.binding import LIB_PATH  # noqa: E402
from tests.parity_log import record  # noqa: E402

BF16_ABS, BF16_NORM, BF16_LSE = 2e-2, 1e-2, 1e-4
F32_NORM, F32_LSE = 1e-5, 1e-5
SCORE_REF = 4.0  # largest |score| of unit-variance scores over a few thousand keys


def dirty_workspace(nbytes, device):
    """Workspace pre-filled with 0xFF bytes (NaN as float): a kernel that reads
    scratch it did not write in the same call shows it in the outputs."""
    ws = sd.workspace(nbytes, device)
    ws.fill_(255)
    return ws


def ensure_lib():
    if not os.path.exists(LIB_PATH):
        from long_context_kv_split_amd.build import build
        build()
    sd.lib()


def say(msg):
    print(msg, flush=True)


def run_verify(kv_t, q, n_q, num_q_heads, scale=1.0, max_kv_len=None):
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = kv.batch
    mk = max(1, kv_t.max_kv_len) if max_kv_len is None else max_kv_len
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, num_q_heads), float("nan"), dtype=torch.float32, device=q.device)
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, n_q, num_q_heads, kv.num_kv_heads,
                                                          kv.head_dim, mk), q.device)
    sd.sd_verify_attn(kv, q, n_q, num_q_heads, mk, scale, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def run_draft(kv_t, q, n_q, num_q_heads, idx, sel_lens, scale=1.0):
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    B = kv.batch
    idx_heads, max_sel = int(idx.shape[1]), int(idx.shape[2])
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_q, num_q_heads), float("nan"), dtype=torch.float32, device=q.device)
    ws = dirty_workspace(sd.sd_draft_attn_sparse_workspace_size(B, n_q, num_q_heads, kv.num_kv_heads,
                                                                kv.head_dim, max_sel), q.device)
    sd.sd_draft_attn_sparse(kv, q, n_q, num_q_heads, idx, sel_lens, idx_heads, max_sel, scale, out,
                            lse, ws)
    torch.cuda.synchronize()
    return out, lse


def compare_attn(out, lse, o_ref, l_ref, dtype, rows=None, score_mag=None):
    """Assert parity; `rows` optionally selects (b, query-head) entries to compare.

    score_mag (array of the lse's shape, or a scalar): the largest |score| a
    row's softmax sees, for inputs whose scores go well past the workloads'
    (unit-variance scores, largest |s| about SCORE_REF). A score of magnitude
    S carries an fp32 rounding error that grows with S, and exp turns it into
    a relative error of the softmax weights; so the lse bars, and the fp32
    output bar, are multiplied by max(1, S / SCORE_REF) (per row for the lse,
    the largest for the output).

    Returns (max abs error, normalised error, max lse error divided by its factor)."""
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    if rows is not None:
        o = np.stack([o[b, :, h] for b, h in rows])
        l = np.stack([l[b, :, h] for b, h in rows])
        o_ref = np.stack([o_ref[b, :, h] for b, h in rows])
        l_ref = np.stack([l_ref[b, :, h] for b, h in rows])
    assert np.isfinite(o).all(), "non-finite output"
    dead = np.isneginf(l_ref)
    assert (np.isneginf(l) == dead).all(), "rows with no visible key differ"
    assert (o[dead.nonzero()] == 0).all() if dead.any() else True
    err = np.abs(o - o_ref).max() if o.size else 0.0
    scale = max(np.abs(o_ref).max(), 1e-30)
    mag = (np.ones_like(l_ref) if score_mag is None
           else np.maximum(1.0, np.broadcast_to(score_mag, l_ref.shape) / SCORE_REF))
    lerr = (np.abs(l[~dead] - l_ref[~dead]) / mag[~dead]).max() if (~dead).any() else 0.0
    if dtype == torch.float32:
        assert err / scale <= F32_NORM * mag.max(), (err, scale, mag.max())
        assert lerr <= F32_LSE, lerr
    else:
        assert err <= BF16_ABS, err
        assert err / scale <= BF16_NORM, (err, scale)
        assert lerr <= BF16_LSE, lerr
    return err, err / scale, lerr


def unit_cache(kv_t, b, g):
    """One (sequence b, KV head g) of a paged cache as a standalone CPU cache
    with an identity page table (pages kept in table order)."""
    L = int(kv_t.lens[b])
    P = kv_t.page_size
    npg = max(1, -(-L // P))
    pages = kv_t.page_table[b, :npg].long()
    k = kv_t.k_pages[pages][:, g:g + 1].cpu()
    v = kv_t.v_pages[pages][:, g:g + 1].cpu()
    table = np.arange(npg, dtype=np.int64)[None, :]
    return k, v, table, np.array([L])


def _band_probability(r, eps):
    """Probability over v ~ U[0, 1) that v*Z lies within eps*Z of a boundary of
    the CDF of weights r: the length of the union of the bands around 0, Z and
    the upper end of every interval with mass, in units of Z."""
    c = np.cumsum(r)
    Z = c[-1]
    if Z <= 0:
        return 0.0
    b = np.concatenate(([0.0], c[r > 0] / Z))
    lo, hi = np.clip(b - eps, 0.0, 1.0), np.clip(b + eps, 0.0, 1.0)
    prev = np.maximum.accumulate(np.concatenate(([0.0], hi[:-1])))
    return float(np.clip(hi - np.maximum(lo, prev), 0.0, None).sum())


def expected_draw_flags(zt, zd, n_ref, temperature=1.0, eps=1e-6):
    """Expected number of sequences whose emitted-token draw falls in the flag
    band, from each sequence's drawn weights (residual at n, or the target row
    for the bonus): sum over sequences of the band probability."""
    zt, zd = oracle.f64(zt), oracle.f64(zd)
    gamma = zt.shape[1] - 1
    tot = 0.0
    for b, n in enumerate(n_ref):
        p = oracle.softmax(zt[b, n], temperature)
        r = np.maximum(0.0, p - oracle.softmax(zd[b, n], temperature)) if n < gamma else p
        tot += _band_probability(r if r.sum() > 0 else p, eps)
    return tot


def check_accept(label, n, out, zt, zd, x, ua, us, temperature=1.0, planted=False):
    """Acceptance parity for every sequence of a batch.

    Unflagged sequences must match the oracle exactly. A flagged sequence (a
    uniform within 1e-6 of a decision threshold) must return one of the
    results the oracle lists as correct for it (accept_outcomes: either side
    of an accept test in the band, the prefix unchanged, and a draw whose CDF
    interval meets the band around v*Z); sequences with exactly one correct
    result must return it. The flagged count must stay within 5 standard
    deviations of its expectation from the draws' band probabilities (unless
    the uniforms were planted next to thresholds on purpose). Returns the counts, also recorded for the terminal summary."""
    n = np.asarray(n)
    out = np.asarray(out)
    n_ref, out_ref, flagged = oracle.spec_accept(zt, zd, x, ua, us, temperature=temperature)
    valid, ambiguous = oracle.accept_valid(zt, zd, x, ua, us, n, out, temperature=temperature)
    exact = (n == n_ref) & (out == out_ref).all(axis=1)
    B = int(n.shape[0])
    expect = expected_draw_flags(zt, zd, n_ref, temperature)
    stats = dict(batch=B, flagged=int(flagged.sum()), ambiguous=int(ambiguous.sum()),
                 exact=int(exact.sum()), flagged_exact=int((exact & flagged).sum()),
                 flagged_other_valid=int((valid & ~exact).sum()), invalid=int((~valid).sum()),
                 expected_flagged=round(expect, 2), mean_accepted=float(n.mean()))
    msg = f"{label}: {stats}"
    bad = np.nonzero(~exact & ~flagged)[0]
    assert bad.size == 0, f"{msg}; unflagged mismatch at {bad[:8]}: gpu n {n[bad[:8]]} " \
        f"ref {n_ref[bad[:8]]}, gpu {out[bad[:4]]} ref {out_ref[bad[:4]]}"
    bad = np.nonzero(~valid)[0]
    assert bad.size == 0, f"{msg}; flagged sequences with a result outside the band at {bad[:8]}: " \
        f"gpu {out[bad[:4]]} ref {out_ref[bad[:4]]}"
    assert (exact | ambiguous).all(), msg
    cap = expect + 5.0 * np.sqrt(expect) + 3.0 + 0.002 * B
    assert planted or flagged.sum() <= cap, f"{msg}; more flagged sequences than the band allows ({cap:.1f})"
    record(label, **stats)
    say(msg)
    return stats


def gathered_decode(kv_t, idx, sel, qd, num_q_heads):
    """Dense decode (verify with n_q = 1) over a compact paged cache that holds,
    for every index set, exactly the rows idx[b, h, :sel[b]] in order (the
    gather done by torch indexing, not by the library). idx: [B, H, S] with H
    = 1 (one set for all KV heads), Hkv (one per KV head) or num_q_heads (one
    per query head: the compact cache then has one head per query head, read
    with G = 1)."""
    B, H, S = idx.shape
    _, Hkv, P, d = kv_t.k_pages.shape
    per_q = H == num_q_heads and H != Hkv
    Hc = H if per_q else Hkv
    npg = (S + P - 1) // P
    pos = idx.clamp(min=0).long()
    pos = pos.expand(B, Hc, S) if H == 1 else pos
    pool = torch.arange(Hc, device="cuda") // (num_q_heads // Hkv if per_q else 1)
    page = kv_t.page_table.long().gather(1, (pos // P).reshape(B, -1)).reshape(B, Hc, S)
    heads = pool.view(1, Hc, 1).expand(B, Hc, S)
    k_sel = torch.zeros((B, Hc, npg * P, d), dtype=kv_t.k_pages.dtype, device="cuda")
    v_sel = torch.zeros_like(k_sel)
    k_sel[:, :, :S] = kv_t.k_pages[page, heads, pos % P]
    v_sel[:, :, :S] = kv_t.v_pages[page, heads, pos % P]
    k_c = k_sel.reshape(B, Hc, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hc, P, d).contiguous()
    v_c = v_sel.reshape(B, Hc, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hc, P, d).contiguous()
    pt_c = torch.arange(B * npg, dtype=torch.int32, device="cuda").view(B, npg).contiguous()
    kv_c = sd.KVCache(k_c, v_c, pt_c, sel.to(torch.int32).contiguous())
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, 1, num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ws = dirty_workspace(sd.sd_verify_attn_workspace_size(B, 1, num_q_heads, Hc, d, S), "cuda")
    sd.sd_verify_attn(kv_c, qd, 1, num_q_heads, S, 1.0, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse
