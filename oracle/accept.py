"""Oracle: modified-rejection speculative sampling (accept / correct / bonus).

TEST INFRASTRUCTURE ONLY (see the package header).

The explainer "Wann beschleunigt spekulatives Decoding das LLM-Serving?"
(slavadubrov.com, section "Eine Verifizierungsrunde verstehen") describes the
round: the target model scores all candidate positions in one batched pass;
modified rejection sampling (Chen et al.) accepts candidates left to right
using both distributions; at the first rejection it draws a correction from the
residual target distribution and drops the later candidates; if every
candidate is accepted it may draw one more token from the target. The same
page notes this preserves the target distribution, and that comparing drafts
only with the target's own chosen tokens is a different algorithm.

Written out (float64), per sequence with draft length gamma and temperature t:
  p_i = softmax(z_target[i] / t), i = 0..gamma;  q_i = softmax(z_draft[i] / t)
  for i = 0..gamma-1: accept x_i iff u_i * q_i(x_i) < p_i(x_i)  (u_i < p/q
      without a division; u in [0, 1)), stop at the first rejection; n = count.
  residual r = max(0, p_n - q_n) if n < gamma, else r = p_gamma (bonus);
      if r sums to 0 (p_n == q_n exactly), r = p_n.
  y = smallest token t with sum_{j <= t} r_j > v * Z, Z = sum r, v = u_sample[n];
      if rounding leaves none, the last t with r_t > 0.
  out = [x_0 .. x_{n-1}, y, -1, ...].

A sequence is flagged when a uniform lies within `flag_eps` of a decision
threshold: |u_i - p_i(x_i)/q_i(x_i)| < eps for an evaluated test, or v*Z
within eps*Z of either end of y's CDF interval. Flagged sequences may
legitimately differ between float64 and lower-precision implementations.
"""
import numpy as np

from oracle.common import f64, i64


def softmax(z, temperature=1.0):
    """Row softmax of z / temperature in float64."""
    x = f64(z) / temperature
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def _sample_index(r, v):
    """Inverse-CDF draw from unnormalised weights r >= 0 with uniform v."""
    c = np.cumsum(r)
    Z = c[-1]
    thr = v * Z
    y = int(np.searchsorted(c, thr, side="right"))   # first t with c[t] > thr
    if y >= r.shape[0]:
        y = int(np.nonzero(r > 0)[0][-1])
    lo = c[y - 1] if y > 0 else 0.0
    return y, thr, lo, c[y], Z


def spec_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample,
                temperature=1.0, flag_eps=1e-6):
    """Returns n_accepted int32 [B], out_tokens int32 [B, gamma+1], flagged bool [B].

    target_logits [B, gamma+1, V], draft_logits [B, gamma, V],
    draft_tokens [B, gamma], u_accept [B, gamma], u_sample [B, gamma+1].
    """
    zt = f64(target_logits)
    zd = f64(draft_logits)
    x = i64(draft_tokens)
    ua = f64(u_accept)
    us = f64(u_sample)
    B, g1, V = zt.shape
    gamma = g1 - 1
    n_acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, g1), -1, dtype=np.int32)
    flagged = np.zeros(B, dtype=bool)
    for b in range(B):
        p = softmax(zt[b], temperature)
        q = softmax(zd[b], temperature) if gamma > 0 else np.zeros((0, V))
        n = 0
        for i in range(gamma):
            t = int(x[b, i])
            pi, qi = p[i, t], q[i, t]
            if qi > 0 and abs(ua[b, i] - pi / qi) < flag_eps:
                flagged[b] = True
            if ua[b, i] * qi < pi:
                n += 1
            else:
                break
        if n < gamma:
            r = np.maximum(0.0, p[n] - q[n])
            if r.sum() == 0.0:
                r = p[n].copy()
        else:
            r = p[gamma].copy()
        y, thr, lo, hi, Z = _sample_index(r, us[b, n])
        if abs(thr - lo) < flag_eps * Z or abs(thr - hi) < flag_eps * Z:
            flagged[b] = True
        out[b, :n] = x[b, :n]
        out[b, n] = y
        n_acc[b] = n
    return n_acc, out, flagged
