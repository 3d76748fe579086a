"""Oracle: static draft-KV selection (StreamingLLM window, SnapKV).

TEST INFRASTRUCTURE ONLY (see the package header).

The MagicDec notes (papercache.org, §4.4 and the experimental setup) name
StreamingLLM and SnapKV as the static KV selection algorithms used for the
self-speculative draft, and Appendix A.1 (Fig. 8) says the compressed KV is
built once at prefill and reused for drafting; §4.1 writes the draft cost as a
selection cost plus gamma draft steps over a budget of K tokens. The pages do
not spell either algorithm out, so these readings are taken:

StreamingLLM: keep `sink` leading positions and `recent` trailing ones,
    I = [0, min(s, L)) U [max(s, L - r), L), ascending, no duplicates.

SnapKV, for each (sequence b, KV head g), prompt length L, window W:
  1. the last W positions are the observation window; window row (w, h) for
     query head h in g's group attends causally to keys 0 .. L - W + w;
  2. vote_j = sum over h in the group and w < W of the normalised attention
     weight p[w, h, j], for prefix positions j < L - W;
  3. pooled = 1-D max pool of the votes, odd kernel, stride 1, window clipped
     at both ends of the prefix;
  4. keep the budget - W prefix positions with the largest pooled value, ties
     broken toward the lower position;
  5. the selection is the ascending union of those positions and the window,
     budget positions in all. If L <= budget every position is kept.
"""
import numpy as np

from oracle.attention import token_rows
from oracle.common import f64, i64


def streaming_select(kv_lens, sink, recent):
    """StreamingLLM positions per sequence.

    Returns idx int32 [B, 1, sink + recent] (unused tail = -1) and
    sel_lens int32 [B].
    """
    lens = i64(kv_lens)
    B = lens.shape[0]
    cap = sink + recent
    idx = np.full((B, 1, cap), -1, dtype=np.int32)
    sel = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(lens[b])
        keep = list(range(0, min(sink, L))) + list(range(max(sink, L - recent), L))
        idx[b, 0, :len(keep)] = keep
        sel[b] = len(keep)
    return idx, sel


def snapkv_votes(q_rows, keys, scale, window):
    """Votes of one (sequence, KV head) for its prefix positions.

    q_rows: [W, G, d] observation-window queries of the G query heads of this
    KV head; keys: [L, d] all cached keys of the sequence for this KV head.
    Returns float64 votes [L - W].
    """
    W, G, d = q_rows.shape
    L = keys.shape[0]
    rows = q_rows.reshape(W * G, d)                  # row (w, h) = w * G + h
    s = scale * (rows @ keys.T)                      # [W*G, L]
    last_visible = np.repeat(L - W + np.arange(W), G)
    visible = np.arange(L)[None, :] <= last_visible[:, None]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p[:, :L - W].sum(axis=0)


def maxpool1d(values, kernel):
    """Stride-1 max pool with an odd kernel, window clipped to the array."""
    v = np.asarray(values)
    n = v.shape[0]
    half = kernel // 2
    out = np.empty_like(v)
    for j in range(n):
        out[j] = v[max(0, j - half):min(n, j + half + 1)].max()
    return out


def topk_lowest_index(values, k):
    """Positions of the k largest values, ties toward lower positions; ascending."""
    v = np.asarray(values)
    order = np.lexsort((np.arange(v.shape[0]), -v))   # by value desc, then index asc
    return np.sort(order[:k])


def snapkv_select(q_obs, k_pages, page_table, kv_lens, window, pool_kernel, budget, scale,
                  units=None, return_pooled=False):
    """SnapKV selection per (sequence, KV head).

    q_obs: [B, W, Hq, d] queries of the last W prompt tokens. budget: one KV
    budget for every sequence, or one per sequence (the MagicDec notes, §4.3:
    the best draft budget depends on the context length; with per-sequence
    budgets each sequence is selected on its own budget).
    Returns idx int32 [B, Hkv, max budget] (unused tail = -1), sel_lens int32
    [B] = min(L, budget_b), and with return_pooled=True a dict
    {(b, g): pooled votes} as well.
    """
    q = f64(q_obs)
    K = f64(k_pages)
    pt = i64(page_table)
    lens = i64(kv_lens)
    B, W, Hq, d = q.shape
    assert W == window
    Hkv = K.shape[1]
    G = Hq // Hkv
    budgets = np.broadcast_to(np.asarray(budget, dtype=np.int64), (B,))
    width = int(budgets.max())
    idx = np.full((B, Hkv, width), -1, dtype=np.int32)
    sel = np.array([min(int(L), int(K_b)) for L, K_b in zip(lens, budgets)], dtype=np.int32)
    pooled_out = {}
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if units is None else list(units)
    for b, g in todo:
        L = int(lens[b])
        K_b = int(budgets[b])
        if L <= K_b:
            idx[b, g, :L] = np.arange(L)
            continue
        keys = token_rows(K, pt, b, np.arange(L), g)
        rows = q[b][:, g * G:(g + 1) * G, :]
        votes = snapkv_votes(rows, keys, scale, W)
        pooled = maxpool1d(votes, pool_kernel)
        kept = topk_lowest_index(pooled, K_b - W)
        chosen = np.concatenate([kept, np.arange(L - W, L)])
        idx[b, g, :K_b] = np.sort(chosen)
        pooled_out[(b, g)] = pooled
    if return_pooled:
        return idx, sel, pooled_out
    return idx, sel
