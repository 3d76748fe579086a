"""Pins for the oracle's draft-KV selection (StreamingLLM, SnapKV).

Checked against hand-worked fixtures (tests/golden/selection_cases.json),
library routines (torch softmax, torch max_pool1d), brute-force loops and
subset enumeration on tiny inputs, and the special cases the definitions fix.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SEL = json.load(open(os.path.join(GOLDEN, "selection_cases.json")))


def _pool_from_dense(dense, P=16):
    """dense [L, Hkv, d] for one sequence -> pool [pages, Hkv, P, d], table [1, pages]."""
    L, Hkv, d = dense.shape
    npg = max(1, -(-L // P))
    pool = np.full((npg, Hkv, P, d), np.nan)
    for t in range(L):
        pool[t // P, :, t % P] = dense[t]
    return pool, np.arange(npg)[None, :]


def test_streaming_golden():
    for c in SEL["streaming"]:
        idx, sel = oracle.streaming_select(np.array([c["L"]]), c["sink"], c["recent"])
        assert sel[0] == len(c["idx"])
        assert idx[0, 0, :sel[0]].tolist() == c["idx"]
        assert (idx[0, 0, sel[0]:] == -1).all()


@pytest.mark.parametrize("L,s,r", [(100, 4, 12), (16, 4, 12), (15, 4, 12), (3, 4, 12), (64, 0, 8), (64, 8, 0)])
def test_streaming_set_properties(L, s, r):
    idx, sel = oracle.streaming_select(np.array([L]), s, r)
    got = idx[0, 0, :sel[0]]
    want = sorted(set(range(min(s, L))) | set(range(max(0, L - r), L)))
    assert got.tolist() == want
    assert sel[0] == min(L, s + r)


def test_full_budget_streaming_equals_dense_decode():
    rng = np.random.default_rng(0)
    lens = [20, 33]
    B, Hq, Hkv, d = 2, 4, 2, 8
    kd = rng.standard_normal((B, 33, Hkv, d))
    vd = rng.standard_normal((B, 33, Hkv, d))
    q = rng.standard_normal((B, 1, Hq, d))
    pools = [_pool_from_dense(kd[b]) for b in range(B)]
    # stack both sequences into one pool with a table
    kp = np.concatenate([pools[0][0], pools[1][0]])
    vp = np.concatenate([_pool_from_dense(vd[0])[0], _pool_from_dense(vd[1])[0]])
    pt = np.array([[0, 1, 1], [2, 3, 4]])   # sequence 0 owns pages 0-1, sequence 1 pages 2-4
    idx, sel = oracle.streaming_select(np.array(lens), 8, 32)   # s + r >= L
    o_s, l_s = oracle.sparse_attn(q, kp, vp, pt, idx, sel, 1.0)
    o_d, l_d = oracle.verify_attn(q, kp, vp, pt, np.array(lens), 1.0)
    np.testing.assert_array_equal(o_s, o_d)
    np.testing.assert_array_equal(l_s, l_d)


def _votes_brute(q_rows, keys, scale, W):
    """Double loop with math.exp, one window row at a time."""
    Wn, G, d = q_rows.shape
    L = keys.shape[0]
    votes = [0.0] * (L - W)
    for w in range(Wn):
        for h in range(G):
            last = L - W + w
            s = [scale * sum(q_rows[w, h, c] * keys[j, c] for c in range(d)) for j in range(last + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for j in range(L - W):
                votes[j] += e[j] / z
    return np.array(votes)


@pytest.mark.parametrize("seed", [0, 1])
def test_votes_match_brute_force_and_library_softmax(seed):
    rng = np.random.default_rng(seed)
    L, W, G, d = 23, 5, 3, 6
    q = rng.standard_normal((W, G, d))
    keys = rng.standard_normal((L, d))
    v = oracle.snapkv_votes(q, keys, 0.8, W)
    np.testing.assert_allclose(v, _votes_brute(q, keys, 0.8, W), rtol=1e-13, atol=1e-15)
    # library softmax, one window row at a time
    ref = np.zeros(L - W)
    for w in range(W):
        s = torch.tensor(0.8 * q[w] @ keys[:L - W + w + 1].T)
        p = torch.softmax(s, dim=-1).numpy()
        ref += p[:, :L - W].sum(axis=0)
    np.testing.assert_allclose(v, ref, rtol=1e-13, atol=1e-15)
    # mass: every window row is a distribution, so prefix votes never exceed W*G
    assert v.sum() <= W * G + 1e-12 and (v >= 0).all()


def test_maxpool_golden_and_library():
    for c in SEL["maxpool"]:
        got = oracle.maxpool1d(np.array(c["values"]), c["kernel"])
        np.testing.assert_array_equal(got, np.array(c["pooled"]))
    rng = np.random.default_rng(3)
    x = rng.random(101)
    for k in (1, 3, 7, 9):
        ref = torch.nn.functional.max_pool1d(torch.tensor(x)[None, None], k, stride=1,
                                             padding=k // 2)[0, 0].numpy()
        np.testing.assert_array_equal(oracle.maxpool1d(x, k), ref)


def test_topk_golden():
    for c in SEL["topk"]:
        assert oracle.topk_lowest_index(np.array(c["values"]), c["k"]).tolist() == c["idx"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_subsets(seed):
    rng = np.random.default_rng(seed)
    n, k = 10, 4
    vals = rng.integers(0, 4, n).astype(float)          # many exact ties
    best = None
    for sub in itertools.combinations(range(n), k):
        key = (-sum(vals[list(sub)]), sub)              # max sum, then lexicographically lowest
        if best is None or key < best:
            best = key
    assert oracle.topk_lowest_index(vals, k).tolist() == list(best[1])


def test_snapkv_golden_one_row():
    c = SEL["snapkv"][0]
    L = c["L"]
    keys = np.array(c["keys"])[:, None, None]            # [L, Hkv=1, d=1]
    pool, pt = _pool_from_dense(keys)
    q = np.full((1, 1, 1, 1), c["q"])
    v = oracle.snapkv_votes(q[0], keys[:, 0, :], 1.0, 1)
    np.testing.assert_allclose(v, np.array(c["votes"]), rtol=1e-14)
    idx1, sel1 = oracle.snapkv_select(q, pool, pt, np.array([L]), 1, 1, c["budget"], 1.0)
    idx3, _ = oracle.snapkv_select(q, pool, pt, np.array([L]), 1, 3, c["budget"], 1.0)
    assert sel1[0] == c["budget"]
    assert idx1[0, 0].tolist() == c["idx_pool1"]
    assert idx3[0, 0].tolist() == c["idx_pool3"]


@pytest.mark.parametrize("seed", range(4))
def test_snapkv_brute_force_selection(seed):
    """Tiny L: the kept prefix set maximises the pooled sum and is lexicographically
    lowest among ties; pooled votes come from an independent brute force."""
    rng = np.random.default_rng(seed)
    L, W, budget, G, d, pk = 12, 2, 6, 2, 4, 3
    keys = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((1, W, G, d))
    pool, pt = _pool_from_dense(keys)
    idx, sel = oracle.snapkv_select(q, pool, pt, np.array([L]), W, pk, budget, 1.0)
    votes = _votes_brute(q[0], keys[:, 0], 1.0, W)
    pooled = np.array([max(votes[max(0, j - 1):j + 2]) for j in range(L - W)])
    best = None
    for sub in itertools.combinations(range(L - W), budget - W):
        key = (-sum(pooled[list(sub)]), sub)
        if best is None or key < best:
            best = key
    want = sorted(list(best[1]) + list(range(L - W, L)))
    assert idx[0, 0].tolist() == want
    assert sel[0] == budget


def test_snapkv_budget_at_least_length_keeps_everything():
    rng = np.random.default_rng(1)
    keys = rng.standard_normal((9, 2, 4))
    pool, pt = _pool_from_dense(keys)
    q = rng.standard_normal((1, 3, 4, 4))
    idx, sel = oracle.snapkv_select(q, pool, pt, np.array([9]), 3, 3, 9, 1.0)
    assert sel[0] == 9
    for g in range(2):
        assert idx[0, g].tolist() == list(range(9))


def test_snapkv_pool_kernel_one_is_plain_topk_of_votes():
    rng = np.random.default_rng(2)
    L, W, budget = 40, 4, 12
    keys = rng.standard_normal((L, 1, 8))
    q = rng.standard_normal((1, W, 2, 8))
    pool, pt = _pool_from_dense(keys)
    idx, _ = oracle.snapkv_select(q, pool, pt, np.array([L]), W, 1, budget, 1.0)
    votes = oracle.snapkv_votes(q[0], keys[:, 0], 1.0, W)
    top = np.argsort(-votes, kind="stable")[:budget - W]
    assert idx[0, 0].tolist() == sorted(top.tolist() + list(range(L - W, L)))


def test_snapkv_planted_key_keeps_its_neighbourhood():
    """A key aligned with every window query dominates the votes; with pool
    kernel 7 its +-3 neighbourhood is selected (the pooling plateau)."""
    rng = np.random.default_rng(4)
    L, W, budget, d = 200, 8, 8 + 7, 16
    keys = rng.standard_normal((L, 1, d)) * 0.1
    q = rng.standard_normal((1, W, 4, d)) * 0.1
    direction = np.ones(d) / math.sqrt(d)
    q[0] += 3.0 * direction
    keys[100, 0] = 5.0 * direction
    pool, pt = _pool_from_dense(keys)
    idx, _ = oracle.snapkv_select(q, pool, pt, np.array([L]), W, 7, budget, 1.0)
    kept = [t for t in idx[0, 0].tolist() if t < L - W]
    assert kept == list(range(97, 104))


def test_snapkv_per_head_sets_differ_and_include_window():
    rng = np.random.default_rng(5)
    L, W, budget = 64, 4, 20
    keys = rng.standard_normal((L, 2, 8))
    q = rng.standard_normal((1, W, 4, 8))
    pool, pt = _pool_from_dense(keys)
    idx, _ = oracle.snapkv_select(q, pool, pt, np.array([L]), W, 3, budget, 1.0)
    for g in range(2):
        s = idx[0, g].tolist()
        assert s == sorted(set(s)) and len(s) == budget
        assert s[-W:] == list(range(L - W, L))
    assert idx[0, 0].tolist() != idx[0, 1].tolist()


def test_snapkv_per_sequence_budgets_brute_force():
    """Per-sequence budgets (ragged batch): each sequence's set is the brute-force
    optimum for its own budget, rows are padded with -1 to the largest budget,
    and a sequence with L <= budget keeps everything."""
    rng = np.random.default_rng(9)
    W, G, d, pk, P = 2, 2, 4, 3, 16
    lens, budgets = [12, 11, 7], [6, 5, 9]
    dense = [rng.standard_normal((L, 1, d)) for L in lens]
    q = rng.standard_normal((3, W, G, d))
    # one pool holding the three sequences on consecutive pages
    pools, tables, base = [], [], 0
    for x in dense:
        pool, pt = _pool_from_dense(x, P)
        pools.append(pool)
        tables.append(pt[0] + base)
        base += pool.shape[0]
    pool = np.concatenate(pools)
    width = max(len(t) for t in tables)
    pt = np.stack([np.pad(t, (0, width - len(t))) for t in tables])
    idx, sel = oracle.snapkv_select(q, pool, pt, np.array(lens), W, pk, np.array(budgets), 1.0)
    assert idx.shape == (3, 1, max(budgets))
    assert sel.tolist() == [min(L, K) for L, K in zip(lens, budgets)]
    for b in range(2):
        L, K = lens[b], budgets[b]
        votes = _votes_brute(q[b], dense[b][:, 0], 1.0, W)
        pooled = np.array([max(votes[max(0, j - 1):j + 2]) for j in range(L - W)])
        best = min((-sum(pooled[list(sub)]), sub) for sub in itertools.combinations(range(L - W), K - W))
        want = sorted(list(best[1]) + list(range(L - W, L)))
        assert idx[b, 0].tolist() == want + [-1] * (max(budgets) - K)
    assert idx[2, 0].tolist() == list(range(7)) + [-1, -1]
