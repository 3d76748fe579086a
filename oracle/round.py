"""Oracle: the cache bookkeeping around the hot path in one self-speculative round.

TEST INFRASTRUCTURE ONLY (see the package header).

The MagicDec notes (papercache.org, §3.1-§3.3 and §4.1) describe a round: the
draft -- the target model reading the static compressed KV cache -- proposes
gamma tokens one at a time, the target scores the candidate positions in one
batched pass over the full cache, and modified rejection sampling keeps a
prefix of the drafts plus one correction or bonus token. The pages leave the
bookkeeping open; the plainest reading, used here:

  * The K/V of new tokens go to the end of the cache: token t of sequence b
    lives at pool[page_table[b, t // P], kv_head, t % P] (kv_append).
  * After acceptance the cache keeps the round's first token and the n accepted
    drafts, dropping the gamma - n rejected ones: kv_len <- kv_len - gamma + n
    (kv_advance with add = -gamma); a length never goes below zero.
  * While drafting, the draft attends to the positions chosen at prefill plus
    every position appended since: the tail [tail_begin, kv_len)
    (sparse_attn_tail).
  * A draft token is drawn from q = softmax(z / T) by inverse CDF, which is
    spec_accept with gamma = 0 (the bonus token from p_0): no separate oracle.
  * The draft's compressed cache may also be materialised once (kv_compact):
    the selected rows, in list order, as a cache of their own, whose dense
    decode is the draft over the selection.
"""
import numpy as np

from oracle.attention import attend, token_rows
from oracle.common import f64, i64


def kv_append(k_pages, v_pages, page_table, kv_lens, k_new, v_new):
    """Copies of the pools with k_new / v_new [B, n, Hkv, d] written at
    positions kv_lens[b] .. kv_lens[b] + n - 1 of each sequence."""
    K = np.array(f64(k_pages))
    V = np.array(f64(v_pages))
    pt = i64(page_table)
    lens = i64(kv_lens)
    kn, vn = f64(k_new), f64(v_new)
    B, n, Hkv, _ = kn.shape
    P = K.shape[2]
    for b in range(B):
        for j in range(n):
            t = int(lens[b]) + j
            page = pt[b, t // P]
            for g in range(Hkv):
                K[page, g, t % P] = kn[b, j, g]
                V[page, g, t % P] = vn[b, j, g]
    return K, V


def kv_advance(kv_lens, add, n_accepted=None):
    """max(0, kv_len + add (+ n_accepted[b])); after a round, add = -gamma.
    A length never goes below zero."""
    lens = i64(kv_lens) + int(add)
    if n_accepted is not None:
        lens = lens + i64(n_accepted)
    return np.maximum(lens, 0)


def draft_positions(idx, sel_lens, tail_begin, kv_lens, b, g):
    """Positions the draft of sequence b reads for idx row g (a KV head, or a
    query head when idx has one row per query head; row 0 when shared): the
    selection idx[b, g or 0, :sel_lens[b]] followed by the tail
    [tail_begin[b], kv_len)."""
    idx = i64(idx)
    gi = g if idx.shape[1] > 1 else 0
    sel = idx[b, gi, :int(i64(sel_lens)[b])]
    tail = np.arange(int(i64(tail_begin)[b]), int(i64(kv_lens)[b]), dtype=np.int64)
    return np.concatenate([sel, tail])


def sparse_attn_tail(q, k_pages, v_pages, page_table, idx, sel_lens, tail_begin, kv_lens, scale,
                     units=None):
    """Draft attention over the selected positions plus the appended tail.

    q: [B, n_q, Hq, d]; every query row sees every position read. idx has one
    row per sequence (shared), per KV head, or per query head (top-K
    attention: head h reads its own selection, then the tail). Returns
    (o [B, n_q, Hq, d], lse [B, n_q, Hq]) in float64.
    """
    q = f64(q)
    K = f64(k_pages)
    V = f64(v_pages)
    pt = i64(page_table)
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, n_q, Hq, d))
    lse = np.full((B, n_q, Hq), -np.inf)
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    per_query_head = i64(idx).shape[1] == Hq and G > 1
    for b, g in todo:
        heads = list(range(g * G, (g + 1) * G))
        for hs in ([[h] for h in heads] if per_query_head else [heads]):
            row = hs[0] if per_query_head else g
            pos = draft_positions(idx, sel_lens, tail_begin, kv_lens, b, row)
            keys = token_rows(K, pt, b, pos, g)
            vals = token_rows(V, pt, b, pos, g)
            rows = q[b][:, hs, :].reshape(n_q * len(hs), d)
            ob, lb = attend(rows, keys, vals, scale)
            o[b][:, hs, :] = ob.reshape(n_q, len(hs), d)
            lse[b][:, hs] = lb.reshape(n_q, len(hs))
    return o, lse


def kv_compact(k_pages, v_pages, page_table, idx, sel_lens, pages_per_seq):
    """The draft's compressed cache as a cache of its own (MagicDec notes, §4.4
    and Appendix A.1: the draft reads a static compressed KV cache built once
    at prefill). For sequence b and KV head g, the K and V rows of the
    positions idx[b, g or 0, :sel_lens[b]] (one row per KV head, or one shared
    row), in list order: list entry t goes to page b * pages_per_seq + t // P,
    slot t % P. Returns float64 pools [B * pages_per_seq, Hkv, P, d]; slots
    past sel_lens[b] hold NaN (nothing reads them)."""
    K = f64(k_pages)
    V = f64(v_pages)
    pt = i64(page_table)
    sel = i64(sel_lens)
    B = pt.shape[0]
    _, Hkv, P, d = K.shape
    Kc = np.full((B * pages_per_seq, Hkv, P, d), np.nan)
    Vc = np.full((B * pages_per_seq, Hkv, P, d), np.nan)
    none = np.zeros(B, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            pos = draft_positions(idx, sel, none, none, b, g)
            keys = token_rows(K, pt, b, pos, g)
            vals = token_rows(V, pt, b, pos, g)
            for t in range(len(pos)):
                Kc[b * pages_per_seq + t // P, g, t % P] = keys[t]
                Vc[b * pages_per_seq + t // P, g, t % P] = vals[t]
    return Kc, Vc
