"""Oracle: the dynamic top-K attention draft.

TEST INFRASTRUCTURE ONLY (see the package header).

The MagicDec notes (papercache.org, §4.4, the comparison of KV selection
strategies) set static selection (StreamingLLM, SnapKV: a compressed cache
built once) against dynamic selection, which searches the cache again for
every new query; top-K attention is the exact form of the latter. The notes
say it keeps acceptance high at a small budget but pays a selection cost on
every draft step (§4.1 writes the draft cost as that selection cost plus gamma
draft steps over K tokens). No formula is printed; the textbook reading is
taken:

  for sequence b and query head h, with draft query q_h and the L_b cached keys
  of h's KV head, s_j = <q_h, k_j>; keep the `budget` positions with the
  largest s_j, ties toward the lower position, in ascending order; when
  L_b <= budget every position is kept. The draft attends, per query head,
  over its own kept positions with ordinary softmax attention. A positive
  softmax scale does not change the order, so the selection does not take it.

One draft query per sequence (n_q = 1): drafting proposes one token at a time.
"""
import numpy as np

from oracle.attention import sparse_attn, token_rows
from oracle.common import f64, i64


def topk_scores(q, k_pages, page_table, kv_lens, b, h):
    """s_j = <q[b, 0, h], k_j> for the L_b cached keys of head h's KV head."""
    q = f64(q)
    K = f64(k_pages)
    G = q.shape[2] // K.shape[1]
    L = int(i64(kv_lens)[b])
    keys = token_rows(K, i64(page_table), b, np.arange(L), h // G)
    return keys @ q[b, 0, h]


def topk_select(q, k_pages, page_table, kv_lens, budget, rows=None):
    """Per (sequence, query head) top-`budget` positions by q.k.

    q: [B, 1, Hq, d]. Returns idx int32 [B, Hq, budget] (ascending, -1 past
    the kept positions) and sel_lens int32 [B] = min(L_b, budget). `rows`
    restricts the work to a list of (b, h); other rows stay -1.
    """
    q = f64(q)
    B, n_q, Hq, _ = q.shape
    assert n_q == 1, "one draft query per sequence"
    lens = i64(kv_lens)
    idx = np.full((B, Hq, budget), -1, dtype=np.int32)
    sel = np.minimum(lens, budget).astype(np.int32)
    todo = rows if rows is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        L = int(lens[b])
        if L <= budget:
            idx[b, h, :L] = np.arange(L)
            continue
        s = topk_scores(q, k_pages, page_table, kv_lens, b, h)
        # a stable sort of -s lists equal scores by position: ties go to the lower one
        keep = np.argsort(-s, kind="stable")[:budget]
        idx[b, h] = np.sort(keep)
    return idx, sel


def topk_attn(q, k_pages, v_pages, page_table, kv_lens, budget, scale):
    """Top-K attention draft step: each query head attends over its own kept
    positions. Returns (o [B, 1, Hq, d], lse [B, 1, Hq]) and the selection."""
    idx, sel = topk_select(q, k_pages, page_table, kv_lens, budget)
    o, lse = sparse_attn(q, k_pages, v_pages, page_table, idx, sel, scale)
    return o, lse, idx, sel
