"""Oracle: softmax attention over a paged KV cache (verify and sparse draft).

TEST INFRASTRUCTURE ONLY (see the package header).

The MagicDec notes (papercache.org, §3.2) state that verification and ordinary
decoding read the same KV cache, and §3.3/§4.1 that the self-speculative draft
runs the target model on a compressed (sparse) subset of that cache. Neither
page writes attention out; it is the standard scaled-dot-product softmax
attention, which this module spells out:

    s_j = scale * <q, k_j>,  m = max_j s_j,  l = sum_j exp(s_j - m),
    o   = sum_j exp(s_j - m) v_j / l,          lse = m + ln l.

Readings where the pages are silent:
  * GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
  * Verify: the n_q = gamma + 1 query tokens are the last n_q tokens of the
    cache (their K/V are already in it) and are causal among themselves, so
    query i (0-based) sees positions 0 .. L - n_q + i.
  * A row with no visible key returns o = 0 and lse = -inf.
"""
import numpy as np

from oracle.common import f64, i64


def token_rows(pool, page_table, b, positions, kv_head):
    """Rows of `pool` [num_pages, Hkv, P, d] for token positions of sequence b.

    Token t of sequence b lives at pool[page_table[b, t // P], kv_head, t % P].
    """
    P = pool.shape[2]
    positions = np.asarray(positions, dtype=np.int64)
    pages = page_table[b, positions // P]
    return pool[pages, kv_head, positions % P, :]


def attend(q, keys, values, scale, visible=None):
    """Softmax attention of query rows q [R, d] over keys, values [J, d].

    visible: optional bool [R, J]; hidden pairs get weight 0.
    Returns (o [R, d], lse [R]), lse in natural log.
    """
    R = q.shape[0]
    d = values.shape[1] if values.ndim == 2 else q.shape[1]
    o = np.zeros((R, d))
    lse = np.full(R, -np.inf)
    if keys.shape[0] == 0:
        return o, lse
    s = scale * (q @ keys.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    live = np.isfinite(m[:, 0])
    if not live.any():
        return o, lse
    e = np.exp(s[live] - m[live])
    l = e.sum(axis=1, keepdims=True)
    o[live] = (e @ values) / l
    lse[live] = m[live, 0] + np.log(l[:, 0])
    return o, lse


def _units(B, Hkv, units):
    if units is None:
        return [(b, g) for b in range(B) for g in range(Hkv)]
    return list(units)


def verify_attn(q, k_pages, v_pages, page_table, kv_lens, scale, units=None):
    """Verify attention: gamma+1 causal queries over the full cache.

    q: [B, n_q, Hq, d]. Returns o [B, n_q, Hq, d] and lse [B, n_q, Hq]
    (float64). `units` restricts the work to a list of (b, kv_head) pairs;
    rows of other units are left at 0 / -inf.
    """
    q = f64(q)
    K = f64(k_pages)
    V = f64(v_pages)
    pt = i64(page_table)
    lens = i64(kv_lens)
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, n_q, Hq, d))
    lse = np.full((B, n_q, Hq), -np.inf)
    for b, g in _units(B, Hkv, units):
        L = int(lens[b])
        pos = np.arange(L)
        keys = token_rows(K, pt, b, pos, g)
        vals = token_rows(V, pt, b, pos, g)
        heads = list(range(g * G, (g + 1) * G))
        # rows ordered (i, h): query token i of head h
        rows = q[b][:, heads, :].reshape(n_q * G, d)
        last_visible = np.repeat(L - n_q + np.arange(n_q), G)  # per row
        visible = pos[None, :] <= last_visible[:, None]
        ob, lb = attend(rows, keys, vals, scale, visible)
        o[b][:, heads, :] = ob.reshape(n_q, G, d)
        lse[b][:, heads] = lb.reshape(n_q, G)
    return o, lse


def sparse_attn(q, k_pages, v_pages, page_table, idx, sel_lens, scale, units=None):
    """Draft attention over a selected subset of cached positions.

    idx: [B, idx_heads, max_sel] positions; idx_heads is 1 (one set shared by
    all KV heads, e.g. StreamingLLM), Hkv (one set per KV head, SnapKV) or Hq
    (one set per query head, top-K attention; the same as Hkv when Hq = Hkv).
    Sequence b uses idx[b, g or 0, :sel_lens[b]] (idx[b, h, ...] per query
    head); every query row sees every selected position. q: [B, n_q, Hq, d].
    """
    q = f64(q)
    K = f64(k_pages)
    V = f64(v_pages)
    pt = i64(page_table)
    idx = i64(idx)
    sl = i64(sel_lens)
    B, n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    idx_heads = idx.shape[1]
    o = np.zeros((B, n_q, Hq, d))
    lse = np.full((B, n_q, Hq), -np.inf)
    per_query_head = idx_heads == Hq and G > 1
    for b, g in _units(B, Hkv, units):
        heads = list(range(g * G, (g + 1) * G))
        # one set for the group, or one per query head of it
        groups = [[h] for h in heads] if per_query_head else [heads]
        for hs in groups:
            gi = hs[0] if per_query_head else (g if idx_heads > 1 else 0)
            pos = idx[b, gi, :int(sl[b])]
            keys = token_rows(K, pt, b, pos, g)
            vals = token_rows(V, pt, b, pos, g)
            rows = q[b][:, hs, :].reshape(n_q * len(hs), d)
            ob, lb = attend(rows, keys, vals, scale)
            o[b][:, hs, :] = ob.reshape(n_q, len(hs), d)
            lse[b][:, hs] = lb.reshape(n_q, len(hs))
    return o, lse
