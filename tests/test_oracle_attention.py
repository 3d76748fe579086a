"""Pins for the oracle's attention (verify and sparse draft).

Each test checks the oracle against something other than itself: a library
routine (torch's scaled_dot_product_attention in float64 on the CPU), closed
forms, hand-worked fixtures in tests/golden/attention_cases.json, and
invariants the definition fixes (decode equivalence, truncation, page layout).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scatter_to_pages(dense, lens, page_size, rng, shuffle=True):
    """Independent paging for the tests: dense [B, Lmax, Hkv, d] -> pool, table."""
    B, Lmax, Hkv, d = dense.shape
    npg = [max(1, -(-L // page_size)) for L in lens]
    total = sum(npg) + 1
    phys = rng.permutation(total) if shuffle else np.arange(total)
    pool = np.full((total, Hkv, page_size, d), np.nan)
    table = np.full((B, max(npg)), phys[-1], dtype=np.int64)
    k = 0
    for b in range(B):
        for j in range(npg[b]):
            table[b, j] = phys[k]
            for s in range(page_size):
                t = j * page_size + s
                if t < lens[b]:
                    pool[phys[k], :, s, :] = dense[b, t]
            k += 1
    return pool, table


def _sdpa_verify(q, kd, vd, lens, scale):
    """Reference via torch SDPA: q [B,n_q,Hq,d], kd/vd dense [B,Lmax,Hkv,d]."""
    B, n_q, Hq, d = q.shape
    Hkv = kd.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        L = lens[b]
        k = torch.tensor(kd[b, :L]).repeat_interleave(G, dim=1).permute(1, 0, 2)  # [Hq, L, d]
        v = torch.tensor(vd[b, :L]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        qq = torch.tensor(q[b]).permute(1, 0, 2)                                  # [Hq, n_q, d]
        mask = torch.zeros(n_q, L, dtype=torch.bool)
        for i in range(n_q):
            mask[i, :L - n_q + i + 1] = True
        o = torch.nn.functional.scaled_dot_product_attention(
            qq.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), attn_mask=mask, scale=scale)[0]
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_verify_matches_library_sdpa(seed):
    rng = np.random.default_rng(seed)
    B, n_q, Hq, Hkv, d, P = 3, 3, 6, 2, 8, 4
    lens = [13, 4, 21]
    kd = rng.standard_normal((B, max(lens), Hkv, d))
    vd = rng.standard_normal((B, max(lens), Hkv, d))
    q = rng.standard_normal((B, n_q, Hq, d))
    scale = 0.7
    kp, pt = _scatter_to_pages(kd, lens, P, np.random.default_rng(seed + 50))
    vp, _ = _scatter_to_pages(vd, lens, P, np.random.default_rng(seed + 50))  # same permutation
    o, lse = oracle.verify_attn(q, kp, vp, pt, np.array(lens), scale)
    ref = _sdpa_verify(q, kd, vd, lens, scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # lse against a direct log-sum-exp of the visible scores (torch.logsumexp)
    b, i, h = 2, 1, 5
    g = h // (Hq // Hkv)
    L = lens[b]
    s = torch.tensor(scale * kd[b, :L - n_q + i + 1, g] @ q[b, i, h])
    assert abs(lse[b, i, h] - torch.logsumexp(s, 0).item()) < 1e-12


def test_golden_attention_cases():
    cases = json.load(open(os.path.join(GOLDEN, "attention_cases.json")))["cases"]
    for c in cases:
        if "verify" in c:
            v = c["verify"]
            L, n_q = v["L"], v["n_q"]
            vals = np.array(v["values"])[:, None, :]                 # Hkv=1
            d = vals.shape[-1]
            pool_v = np.zeros((1, 1, 16, d))
            pool_v[0, 0, :L] = vals[:, 0]
            pool_k = np.zeros((1, 1, 16, d))
            q = np.zeros((1, n_q, 1, d))
            o, lse = oracle.verify_attn(q, pool_k, pool_v, np.zeros((1, 1), np.int64),
                                        np.array([L]), 1.0)
            np.testing.assert_allclose(o[0, :, 0], np.array(v["o"]), atol=1e-14)
            np.testing.assert_allclose(lse[0, :, 0], np.array(v["lse"]), atol=1e-14)
        else:
            o, lse = oracle.attend(np.array(c["q"]), np.array(c["keys"]), np.array(c["values"]),
                                   c["scale"])
            np.testing.assert_allclose(o, np.array(c["o"]), rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse, np.array(c["lse"]), atol=1e-13)


def _random_case(seed, lens, n_q=2, Hq=4, Hkv=2, d=8, P=4):
    rng = np.random.default_rng(seed)
    B = len(lens)
    kd = rng.standard_normal((B, max(lens), Hkv, d))
    vd = rng.standard_normal((B, max(lens), Hkv, d))
    q = rng.standard_normal((B, n_q, Hq, d))
    kp, pt = _scatter_to_pages(kd, lens, P, np.random.default_rng(seed + 100))
    vp, _ = _scatter_to_pages(vd, lens, P, np.random.default_rng(seed + 100))
    return q, kp, vp, pt, kd, vd


def test_single_query_verify_is_dense_decode():
    """gamma = 0 (n_q = 1): verify is ordinary decode over every cached token."""
    lens = [9, 17]
    q, kp, vp, pt, _, _ = _random_case(3, lens, n_q=1)
    o, lse = oracle.verify_attn(q, kp, vp, pt, np.array(lens), 0.5)
    idx = np.full((2, 1, 17), -1)
    for b, L in enumerate(lens):
        idx[b, 0, :L] = np.arange(L)
    o2, lse2 = oracle.sparse_attn(q, kp, vp, pt, idx, np.array(lens), 0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_verify_row_equals_decode_on_truncated_cache():
    """Query i of n_q sees exactly the cache truncated to L - n_q + i + 1 tokens."""
    lens = [11, 16]
    n_q = 4
    q, kp, vp, pt, _, _ = _random_case(4, lens, n_q=n_q)
    o, lse = oracle.verify_attn(q, kp, vp, pt, np.array(lens), 1.0)
    for i in range(n_q):
        trunc = np.array([L - n_q + i + 1 for L in lens])
        oi, li = oracle.verify_attn(q[:, i:i + 1], kp, vp, pt, trunc, 1.0)
        np.testing.assert_allclose(o[:, i], oi[:, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, i], li[:, 0], rtol=1e-13)


def test_page_permutation_invariance_is_bitwise():
    lens = [13, 7]
    rng = np.random.default_rng(5)
    kd = rng.standard_normal((2, 13, 2, 8))
    vd = rng.standard_normal((2, 13, 2, 8))
    q = rng.standard_normal((2, 3, 4, 8))
    kp1, pt1 = _scatter_to_pages(kd, lens, 4, np.random.default_rng(1), shuffle=False)
    vp1, _ = _scatter_to_pages(vd, lens, 4, np.random.default_rng(1), shuffle=False)
    kp2, pt2 = _scatter_to_pages(kd, lens, 4, np.random.default_rng(2))
    vp2, _ = _scatter_to_pages(vd, lens, 4, np.random.default_rng(2))
    assert not np.array_equal(pt1, pt2)
    a = oracle.verify_attn(q, kp1, vp1, pt1, np.array(lens), 1.0)
    b = oracle.verify_attn(q, kp2, vp2, pt2, np.array(lens), 1.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_closed_form_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(6)
    L, n_q, d = 10, 3, 4
    key = rng.standard_normal(d)
    kd = np.tile(key, (1, L, 1, 1)).reshape(1, L, 1, d)
    vd = rng.standard_normal((1, L, 1, d))
    q = rng.standard_normal((1, n_q, 1, d))
    kp, pt = _scatter_to_pages(kd, [L], 4, np.random.default_rng(0))
    vp, _ = _scatter_to_pages(vd, [L], 4, np.random.default_rng(0))
    o, lse = oracle.verify_attn(q, kp, vp, pt, np.array([L]), 1.0)
    for i in range(n_q):
        n_vis = L - n_q + i + 1
        np.testing.assert_allclose(o[0, i, 0], vd[0, :n_vis, 0].mean(axis=0), rtol=1e-12)
        s = float(q[0, i, 0] @ key)
        assert abs(lse[0, i, 0] - (s + math.log(n_vis))) < 1e-12


def test_closed_form_dominant_key_returns_its_value():
    L, d = 12, 4
    kd = np.zeros((1, L, 1, d))
    kd[0, 5, 0, 0] = 50.0
    vd = np.random.default_rng(7).standard_normal((1, L, 1, d))
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    kp, pt = _scatter_to_pages(kd, [L], 4, np.random.default_rng(0))
    vp, _ = _scatter_to_pages(vd, [L], 4, np.random.default_rng(0))
    o, _ = oracle.verify_attn(q, kp, vp, pt, np.array([L]), 1.0)
    np.testing.assert_allclose(o[0, 0, 0], vd[0, 5, 0], atol=1e-19 + 1e-18 * 12)


def test_gqa_head_mapping_groups_consecutive_heads():
    """Query head h reads KV head h // G: heads of one group agree with a
    single-KV-head problem built from that KV head alone."""
    lens = [9]
    q, kp, vp, pt, kd, vd = _random_case(8, lens, n_q=2, Hq=6, Hkv=3)
    o, _ = oracle.verify_attn(q, kp, vp, pt, np.array(lens), 1.0)
    for h in range(6):
        g = h // 2
        o1, _ = oracle.verify_attn(q[:, :, h:h + 1], kp[:, g:g + 1], vp[:, g:g + 1], pt,
                                   np.array(lens), 1.0)
        np.testing.assert_array_equal(o[:, :, h], o1[:, :, 0])


def test_scale_folds_into_query():
    lens = [10]
    q, kp, vp, pt, _, _ = _random_case(9, lens)
    a, la = oracle.verify_attn(q, kp, vp, pt, np.array(lens), 0.25)
    b, lb = oracle.verify_attn(q * 0.25, kp, vp, pt, np.array(lens), 1.0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_empty_visible_set_gives_zero_and_minus_inf():
    q = np.ones((1, 1, 1, 4))
    kp = np.zeros((1, 1, 4, 4))
    o, lse = oracle.verify_attn(q, kp, kp, np.zeros((1, 1), np.int64), np.array([0]), 1.0)
    assert np.all(o == 0) and np.isneginf(lse).all()
    o, lse = oracle.sparse_attn(q, kp, kp, np.zeros((1, 1), np.int64), np.zeros((1, 1, 2), np.int64),
                                np.array([0]), 1.0)
    assert np.all(o == 0) and np.isneginf(lse).all()


def test_sparse_index_order_irrelevant_and_subset_matches_sdpa():
    lens = [20]
    q, kp, vp, pt, kd, vd = _random_case(10, lens, n_q=1, Hq=4, Hkv=2)
    sel = np.array([0, 3, 4, 11, 19, 7])
    idx = sel[None, None, :]
    o1, l1 = oracle.sparse_attn(q, kp, vp, pt, idx, np.array([6]), 1.0)
    o2, l2 = oracle.sparse_attn(q, kp, vp, pt, idx[:, :, ::-1].copy(), np.array([6]), 1.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    # library reference on the subset
    for h in range(4):
        g = h // 2
        k = torch.tensor(kd[0, sel, g])[None, None]
        v = torch.tensor(vd[0, sel, g])[None, None]
        qq = torch.tensor(q[0, 0, h])[None, None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=1.0)[0, 0, 0].numpy()
        np.testing.assert_allclose(o1[0, 0, h], ref, rtol=1e-12, atol=1e-13)


def test_per_kv_head_index_sets():
    """idx_heads = Hkv: each KV head reads its own set."""
    lens = [16]
    q, kp, vp, pt, kd, vd = _random_case(11, lens, n_q=1, Hq=4, Hkv=2)
    idx = np.array([[[0, 1, 2, 15], [3, 9, 10, 15]]])
    o, _ = oracle.sparse_attn(q, kp, vp, pt, idx, np.array([4]), 1.0)
    for g in range(2):
        o1, _ = oracle.sparse_attn(q, kp, vp, pt, idx[:, g:g + 1], np.array([4]), 1.0)
        np.testing.assert_array_equal(o[0, 0, 2 * g:2 * g + 2], o1[0, 0, 2 * g:2 * g + 2])
