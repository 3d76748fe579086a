"""The parity criteria catch plausible kernel mistakes at full size.

The GPU tests hold bf16 attention to max|dO| <= 2e-2, max|dO| / max|O_ref|
<= 1e-2 and |d lse| <= 1e-4 (tests/gpu_helpers.py). At long context |O| is
only a few hundredths, so those bars are worth something only if a plausible
bug breaks them at the real shapes. Here a mistake is planted in a copy of the
oracle's attention module (the mechanism of test_oracle_mutations.py), the
copy computes verify attention on the Llama-3.1-8B layer shape at context 8192
(two sequences, 32 query / 8 KV heads, head_dim 128, gamma = 3, shuffled
16-token pages), and its output must fail the criteria against the unchanged
oracle. A split-KV combine that forgets the max rescale is emulated directly
(the oracle has no split): eight segments per unit, as the persistent schedule
makes at this shape. Selected indices and emitted tokens must match exactly,
so for them it is enough that a planted mistake changes the result on the
real workloads: the SnapKV tie-break reversed (max-pooling makes plateaus of
equal values, so ties at the threshold are the rule) on the 32k-context
selection, and the bonus token drawn from the last draft position's target
distribution on the 128256-token acceptance workload. CPU only; no GPU code
runs here.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries
from tests.gpu_helpers import BF16_ABS, BF16_LSE, BF16_NORM
from tests.test_oracle_mutations import _install, _planted

B, L, HQ, HKV, D, NQ = 2, 8192, 32, 8, 128, 4
PLANTED = [
    ("drop-last-page", "pos = np.arange(L)", "pos = np.arange(L - 16)"),
    ("causal-hides-own-token", "np.repeat(L - n_q + np.arange(n_q), G)",
     "np.repeat(L - n_q - 1 + np.arange(n_q), G)"),
    ("causal-sees-next-token", "visible = pos[None, :] <= last_visible[:, None]",
     "visible = pos[None, :] <= last_visible[:, None] + 1"),
    ("gqa-interleaved-heads", "        heads = list(range(g * G, (g + 1) * G))\n        # rows ordered",
     "        heads = list(range(g, Hq, Hkv))\n        # rows ordered"),
    ("page-table-of-first-sequence", "pages = page_table[b, positions // P]",
     "pages = page_table[0, positions // P]"),
]


@pytest.fixture(scope="module")
def case():
    kv = paged_kv(21, [L] * B, HKV, D, torch.bfloat16, "cpu", shuffle=True)
    q = queries(21, 1, (B, NQ, HQ, D), torch.bfloat16, "cpu", scale=D ** -0.5)
    o, lse = oracle.verify_attn(q, kv.k_pages, kv.v_pages, kv.page_table, kv.kv_lens, 1.0)
    return kv, q, o, lse


def violations(o, lse, o_ref, lse_ref):
    """Which of the three bf16 criteria an output breaks (the GPU output is
    bf16-rounded; that rounding is far below every bar and is left out)."""
    d = np.abs(o - o_ref).max()
    out = []
    if not d <= BF16_ABS:
        out.append("abs")
    if not d / np.abs(o_ref).max() <= BF16_NORM:
        out.append("norm")
    if lse is not None:
        both = np.isfinite(lse_ref)
        if not (np.array_equal(np.isfinite(lse), both) and np.abs(lse - lse_ref)[both].max() <= BF16_LSE):
            out.append("lse")
    return out


@pytest.mark.parametrize("name,old,new", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_attention_mistake_fails_the_bf16_criteria(case, name, old, new, monkeypatch):
    kv, q, o_ref, lse_ref = case
    mod, copy = _planted("attention", old, new)
    _install(monkeypatch, mod, copy, [oracle, mod])
    o, lse = oracle.verify_attn(q, kv.k_pages, kv.v_pages, kv.page_table, kv.kv_lens, 1.0)
    assert violations(o, lse, o_ref, lse_ref), f"{name} passes every criterion"


def test_dropping_the_last_page_needs_the_normalised_criterion(case, monkeypatch):
    """The absolute bar alone misses this mistake at context 8192."""
    kv, q, o_ref, lse_ref = case
    mod, copy = _planted("attention", *PLANTED[0][1:])
    _install(monkeypatch, mod, copy, [oracle, mod])
    o, _ = oracle.verify_attn(q, kv.k_pages, kv.v_pages, kv.page_table, kv.kv_lens, 1.0)
    v = violations(o, None, o_ref, None)
    assert "abs" not in v and "norm" in v


def test_split_combine_without_max_rescale_fails_the_bf16_criteria(case):
    kv, q, o_ref, _ = case
    K = kv.k_pages.double().numpy()
    V = kv.v_pages.double().numpy()
    pt = kv.page_table.numpy().astype(np.int64)
    qd = q.double().numpy()
    G, segs = HQ // HKV, 8
    o_bad = np.zeros_like(o_ref)
    o_good = np.zeros_like(o_ref)
    for b in range(B):
        pos = np.arange(L)
        for g in range(HKV):
            keys = K[pt[b, pos // 16], g, pos % 16]
            vals = V[pt[b, pos // 16], g, pos % 16]
            for i in range(NQ):
                for h in range(g * G, (g + 1) * G):
                    s = keys[:L - NQ + i + 1] @ qd[b, i, h]
                    parts = []
                    for seg in np.array_split(np.arange(s.shape[0]), segs):
                        m = s[seg].max()
                        e = np.exp(s[seg] - m)
                        parts.append((m, e.sum(), e @ vals[seg] / e.sum()))
                    M = max(p[0] for p in parts)
                    w_good = np.array([l * np.exp(m - M) for m, l, _ in parts])
                    w_bad = np.array([l for _, l, _ in parts])  # rescale by exp(m_s - M) left out
                    os_ = np.stack([p[2] for p in parts])
                    o_good[b, i, h] = w_good @ os_ / w_good.sum()
                    o_bad[b, i, h] = w_bad @ os_ / w_bad.sum()
    assert np.abs(o_good - o_ref).max() < 1e-12   # the emulated split itself is right
    assert violations(o_bad, None, o_ref, None)


def test_reversed_snapkv_tie_break_changes_the_selection_at_full_size(monkeypatch):
    w = WORKLOADS["llama8b-b128-l32k-snapkv"]
    kv = paged_kv(w.seed, [w.context], w.num_kv_heads, w.head_dim, torch.bfloat16, "cpu",
                  spike_frac=w.spike_frac)
    q_obs = queries(w.seed, 4, (1, w.window, w.num_q_heads, w.head_dim), torch.bfloat16, "cpu",
                    scale=w.head_dim ** -0.5)

    def select():
        return oracle.snapkv_select(q_obs, kv.k_pages, kv.page_table, kv.kv_lens, w.window, w.pool_kernel,
                                    w.budget, 1.0)[0]

    ref = select()
    mod, copy = _planted("selection", "np.lexsort((np.arange(v.shape[0]), -v))",
                         "np.lexsort((-np.arange(v.shape[0]), -v))")
    _install(monkeypatch, mod, copy, [oracle, mod])
    bad = select()
    changed = [g for g in range(w.num_kv_heads) if not np.array_equal(ref[0, g], bad[0, g])]
    assert len(changed) >= 4, changed


def test_bonus_from_the_wrong_row_changes_emitted_tokens_at_full_vocab(monkeypatch):
    w = WORKLOADS["llama70b-b64-l16k"]
    B, g, V = w.batch, w.gamma, w.vocab
    zt = logits(w.seed, 8, (B, g + 1, V), w.target_std)
    zd = logits(w.seed, 9, (B, g, V), w.draft_noise_std, base=zt[:, :g]).contiguous()
    x = gumbel_tokens(w.seed, zd)
    ua = dyadic_uniforms(w.seed, 11, (B, g))
    us = dyadic_uniforms(w.seed, 12, (B, g + 1))
    n, out, _ = oracle.spec_accept(zt, zd, x, ua, us)
    mod, copy = _planted("accept", "r = p[gamma].copy()", "r = p[gamma - 1].copy()")
    _install(monkeypatch, mod, copy, [oracle, mod])
    n2, out2, _ = oracle.spec_accept(zt, zd, x, ua, us)
    assert np.array_equal(n, n2)                      # the accept tests are untouched
    full = n == g
    assert full.sum() >= 8                            # ~0.8^4 of the batch accepts every draft
    assert (out[full, g] != out2[full, g]).sum() >= full.sum() // 2
