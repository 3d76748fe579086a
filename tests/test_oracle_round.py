"""Pins for the round-bookkeeping oracle (oracle/round.py).

Each check builds its paged caches here from known dense tensors (test-local
code, not the oracle's paging) and compares with torch's scaled_dot_product_attention
in float64 on the dense tensors, or with hand-worked values.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.round import draft_positions, kv_advance, kv_append, kv_compact, sparse_attn_tail


def build_cache(dense, lens, P, extra_pages, rng):
    """Pools [pages, Hkv, P, d] holding dense[b, :lens[b]] ([B, T, Hkv, d]) on
    shuffled pages; every sequence owns ceil(T / P) pages. Unused slots NaN."""
    B, T, Hkv, d = dense.shape
    per = -(-T // P)
    n_pages = B * per + extra_pages
    perm = rng.permutation(n_pages)
    table = perm[:B * per].reshape(B, per)
    pool = np.full((n_pages, Hkv, P, d), np.nan)
    for b in range(B):
        for t in range(lens[b]):
            pool[table[b, t // P], :, t % P, :] = dense[b, t]
    return pool, table


def sdpa(q_rows, keys, vals, scale, mask=None):
    """torch SDPA in float64: q_rows [R, d], keys/vals [J, d]."""
    q = torch.from_numpy(q_rows)[None, None]
    k = torch.from_numpy(keys)[None, None]
    v = torch.from_numpy(vals)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("P", [16, 32])
def test_append_matches_cache_built_from_concatenation(P):
    rng = np.random.default_rng(5)
    B, Hkv, d, n = 3, 2, 8, 4
    lens = [37, 16, 0]
    T = max(lens) + n
    dense = rng.standard_normal((B, T, Hkv, d))
    new = rng.standard_normal((B, n, Hkv, d))
    K0, table = build_cache(dense, lens, P, 2, np.random.default_rng(1))
    V0 = K0 * 0.5
    K1, V1 = kv_append(K0, V0, table, lens, new, new * 0.5)
    # expected: the same pages, dense sequences extended by the new rows
    want = dense.copy()
    for b in range(B):
        want[b, lens[b]:lens[b] + n] = new[b]
    Kw = K0.copy()
    for b in range(B):
        for t in range(lens[b], lens[b] + n):
            Kw[table[b, t // P], :, t % P, :] = want[b, t]
    assert np.array_equal(np.nan_to_num(K1, nan=7.0), np.nan_to_num(Kw, nan=7.0))
    assert np.array_equal(np.nan_to_num(V1, nan=7.0), np.nan_to_num(Kw * 0.5, nan=7.0))


def test_verify_after_append_is_causal_attention_over_the_extended_sequence():
    """Append the gamma+1 verify tokens, then verify: query i sees the old
    context and new tokens 0..i (torch SDPA with an explicit causal mask)."""
    rng = np.random.default_rng(6)
    B, Hkv, G, d, gamma, P = 2, 2, 2, 16, 3, 16
    n = gamma + 1
    lens = [45, 20]
    dense = rng.standard_normal((B, max(lens) + n, Hkv, d))
    new = rng.standard_normal((B, n, Hkv, d))
    K0, table = build_cache(dense, lens, P, 1, np.random.default_rng(2))
    V0 = -K0
    K1, V1 = kv_append(K0, V0, table, lens, new, -new)
    L1 = kv_advance(lens, n)
    q = rng.standard_normal((B, n, Hkv * G, d))
    o, _ = oracle.verify_attn(q, K1, V1, table, L1, 0.3)
    for b in range(B):
        keys = np.concatenate([dense[b, :lens[b]], new[b]])  # [L1, Hkv, d]
        for g in range(Hkv):
            for h in range(g * G, (g + 1) * G):
                mask = np.zeros((n, L1[b]), dtype=bool)
                for i in range(n):
                    mask[i, :lens[b] + i + 1] = True
                ref = sdpa(q[b, :, h], keys[:, g], -keys[:, g], 0.3, mask)
                assert np.allclose(o[b, :, h], ref, atol=1e-12)


def test_advance_hand_values():
    assert list(kv_advance([10, 5, 0], -4, [2, 0, 4])) == [8, 1, 0]
    assert list(kv_advance([7], 3)) == [10]
    assert list(kv_advance([2, 3], -5, [1, 0])) == [0, 0]  # clamped at zero
    # a round: L tokens, append gamma + 1, accept n -> the first token plus n drafts kept
    L, gamma = 100, 4
    for n in range(gamma + 1):
        assert kv_advance(kv_advance([L], gamma + 1), -gamma, [n])[0] == L + 1 + n


def test_draft_positions_selection_then_tail():
    idx = np.array([[[0, 1, 2, 40, 41, -1]], [[3, 9, -1, -1, -1, -1]]])
    got0 = draft_positions(idx, [5, 2], [64, 10], [67, 10], 0, 0)
    got1 = draft_positions(idx, [5, 2], [64, 10], [67, 10], 1, 0)
    assert list(got0) == [0, 1, 2, 40, 41, 64, 65, 66]
    assert list(got1) == [3, 9]  # empty tail


@pytest.mark.parametrize("idx_heads", [1, 2])
def test_sparse_attn_tail_matches_sdpa_over_gathered_rows(idx_heads):
    rng = np.random.default_rng(7)
    B, Hkv, G, d, P = 2, 2, 3, 16, 16
    lens = [70, 33]
    dense_k = rng.standard_normal((B, max(lens), Hkv, d))
    dense_v = rng.standard_normal((B, max(lens), Hkv, d))
    K, table = build_cache(dense_k, lens, P, 1, np.random.default_rng(3))
    V, _ = build_cache(dense_v, lens, P, 1, np.random.default_rng(3))
    tail_begin = [60, 33]  # second sequence: empty tail
    sel = np.full((B, idx_heads, 8), -1)
    sel_lens = [6, 8]
    for b in range(B):
        for gi in range(idx_heads):
            sel[b, gi, :sel_lens[b]] = np.sort(rng.choice(tail_begin[b], sel_lens[b], replace=False))
    q = rng.standard_normal((B, 1, Hkv * G, d))
    o, lse = sparse_attn_tail(q, K, V, table, sel, sel_lens, tail_begin, lens, 0.25)
    for b in range(B):
        for g in range(Hkv):
            pos = list(sel[b, g if idx_heads > 1 else 0, :sel_lens[b]]) + list(range(tail_begin[b], lens[b]))
            keys, vals = dense_k[b, pos, g], dense_v[b, pos, g]
            for h in range(g * G, (g + 1) * G):
                ref = sdpa(q[b, :, h], keys, vals, 0.25)
                assert np.allclose(o[b, :, h], ref, atol=1e-12)
                s = 0.25 * keys @ q[b, 0, h]
                assert np.isclose(lse[b, 0, h], np.log(np.exp(s - s.max()).sum()) + s.max())


def test_tail_from_zero_without_selection_is_dense_decode():
    rng = np.random.default_rng(8)
    B, Hkv, G, d, P = 2, 1, 4, 8, 16
    lens = [50, 17]
    dense = rng.standard_normal((B, max(lens), Hkv, d))
    K, table = build_cache(dense, lens, P, 0, np.random.default_rng(4))
    q = rng.standard_normal((B, 1, Hkv * G, d))
    sel = np.full((B, 1, 4), -1)
    o_tail, l_tail = sparse_attn_tail(q, K, K, table, sel, [0, 0], [0, 0], lens, 0.5)
    o_dec, l_dec = oracle.verify_attn(q, K, K, table, lens, 0.5)  # n_q = 1: plain decode
    assert np.allclose(o_tail, o_dec, atol=1e-13) and np.allclose(l_tail, l_dec, atol=1e-13)


def test_tail_with_one_set_per_query_head_matches_sdpa():
    """One selection row per query head (top-K attention): head h attends
    over its own positions, then the shared tail (SDPA over gathered rows)."""
    rng = np.random.default_rng(9)
    B, Hkv, G, d, P = 2, 2, 3, 8, 16
    lens = [60, 41]
    dense_k = rng.standard_normal((B, max(lens), Hkv, d))
    dense_v = rng.standard_normal((B, max(lens), Hkv, d))
    K, table = build_cache(dense_k, lens, P, 1, np.random.default_rng(10))
    V, _ = build_cache(dense_v, lens, P, 1, np.random.default_rng(10))
    tail_begin = [52, 41]
    sel = np.full((B, Hkv * G, 6), -1)
    for b in range(B):
        for h in range(Hkv * G):
            sel[b, h, :5] = np.sort(rng.choice(tail_begin[b], 5, replace=False))
    q = rng.standard_normal((B, 1, Hkv * G, d))
    o, _ = sparse_attn_tail(q, K, V, table, sel, [5, 5], tail_begin, lens, 0.3)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            pos = list(sel[b, h, :5]) + list(range(tail_begin[b], lens[b]))
            ref = sdpa(q[b, :, h], dense_k[b, pos, g], dense_v[b, pos, g], 0.3)
            assert np.allclose(o[b, :, h], ref, atol=1e-12)


@pytest.mark.parametrize("idx_heads,P", [(1, 16), (2, 16), (2, 32)])
def test_compact_cache_rows_by_hand(idx_heads, P):
    """Every pool row encodes its own (sequence, position, KV head) as values;
    the compact cache must hold, at page b * pps + t // P, slot t % P of head g,
    the row of position idx[b, g or 0, t], and NaN past the selection."""
    rng = np.random.default_rng(11)
    B, Hkv, d = 2, 2, 4
    lens = [90, 45]
    T = max(lens)
    dense = np.zeros((B, T, Hkv, d))
    for b in range(B):
        for t in range(T):
            for g in range(Hkv):
                dense[b, t, g] = [b, t, g, 1000 * b + 10 * t + g]
    K, table = build_cache(dense, lens, P, 1, np.random.default_rng(5))
    sel_lens = [7, 3]
    sel = np.full((B, idx_heads, 8), -1)
    for b in range(B):
        for gi in range(idx_heads):
            sel[b, gi, :sel_lens[b]] = np.sort(rng.choice(lens[b], sel_lens[b], replace=False))
    pps = 2
    Kc, Vc = kv_compact(K, -K, table, sel, sel_lens, pps)
    assert Kc.shape == (B * pps, Hkv, P, d)
    for b in range(B):
        for g in range(Hkv):
            for t in range(pps * P):
                row = Kc[b * pps + t // P, g, t % P]
                if t < sel_lens[b]:
                    pos = sel[b, g if idx_heads > 1 else 0, t]
                    assert list(row) == [b, pos, g, 1000 * b + 10 * pos + g], (b, g, t)
                    assert np.array_equal(Vc[b * pps + t // P, g, t % P], -row)
                else:
                    assert np.isnan(row).all()


@pytest.mark.parametrize("idx_heads", [1, 2])
def test_decode_over_compact_cache_is_the_sparse_draft(idx_heads):
    """A dense decode (verify with n_q = 1) over the compact cache, with the
    identity page table and lengths sel_lens, equals the draft over the
    selection (SDPA over the gathered rows)."""
    rng = np.random.default_rng(12)
    B, Hkv, G, d, P = 3, 2, 3, 8, 16
    lens = [80, 40, 65]
    dense_k = rng.standard_normal((B, max(lens), Hkv, d))
    dense_v = rng.standard_normal((B, max(lens), Hkv, d))
    K, table = build_cache(dense_k, lens, P, 1, np.random.default_rng(6))
    V, _ = build_cache(dense_v, lens, P, 1, np.random.default_rng(6))
    sel_lens = [20, 9, 33]
    pps = 3
    sel = np.full((B, idx_heads, pps * P), -1)
    for b in range(B):
        for gi in range(idx_heads):
            sel[b, gi, :sel_lens[b]] = np.sort(rng.choice(lens[b], sel_lens[b], replace=False))
    Kc, Vc = kv_compact(K, V, table, sel, sel_lens, pps)
    table_c = np.arange(B * pps).reshape(B, pps)
    q = rng.standard_normal((B, 1, Hkv * G, d))
    o, lse = oracle.verify_attn(q, Kc, Vc, table_c, sel_lens, 0.4)
    for b in range(B):
        for g in range(Hkv):
            pos = list(sel[b, g if idx_heads > 1 else 0, :sel_lens[b]])
            for h in range(g * G, (g + 1) * G):
                ref = sdpa(q[b, :, h], dense_k[b, pos, g], dense_v[b, pos, g], 0.4)
                assert np.allclose(o[b, :, h], ref, atol=1e-12)
