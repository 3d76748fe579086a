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
legitimately differ between float64 and lower-precision implementations;
`accept_outcomes` lists the results that remain correct for such a sequence
and `accept_valid` checks a result against that list.
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
        r, _ = _residual(p, q, n, gamma)
        y, thr, lo, hi, Z = _sample_index(r, us[b, n])
        if abs(thr - lo) < flag_eps * Z or abs(thr - hi) < flag_eps * Z:
            flagged[b] = True
        out[b, :n] = x[b, :n]
        out[b, n] = y
        n_acc[b] = n
    return n_acc, out, flagged


def _residual(p, q, n, gamma):
    """Weights the emitted token is drawn from at acceptance count n, and
    whether the residual was identically zero (the weights are then p_n)."""
    if n < gamma:
        r = np.maximum(0.0, p[n] - q[n])
        if r.sum() == 0.0:
            return p[n].copy(), True
        return r, False
    r = p[gamma].copy()
    return r, False


def _draws_in_band(r, v, eps, maybe_mass=None):
    """Tokens an inverse-CDF draw with uniform v can return when v*Z may move by
    up to eps*Z: every token with mass whose interval [C_{t-1}, C_t] meets
    [v*Z - eps*Z, v*Z + eps*Z]; `maybe_mass` adds zero-weight tokens whose
    weight a lower-precision evaluation could make positive (their interval is
    the point C_t)."""
    c = np.cumsum(r)
    Z = c[-1]
    lo = np.concatenate(([0.0], c[:-1]))
    thr = v * Z
    live = r > 0
    if maybe_mass is not None:
        live = live | maybe_mass
    hit = live & (lo <= thr + eps * Z) & (c >= thr - eps * Z)
    return set(np.nonzero(hit)[0].tolist())


def accept_outcomes(target_logits, draft_logits, draft_tokens, u_accept, u_sample, b,
                    temperature=1.0, flag_eps=1e-6, zero_eps=1e-5):
    """All results (n, out_tokens row as a tuple) that sequence b may take when
    each decision threshold may move by less than flag_eps (relative), i.e. the
    results an implementation that evaluates p, q, the residual and its CDF to
    about single precision can legitimately return (the explainer's
    verification round, with the flag band of the exactness criterion):

      - accept test i with p_i(x_i) > 0 and q_i(x_i) > 0 can go either way when
        |u_i - p_i(x_i)/q_i(x_i)| < flag_eps; with p_i(x_i) = 0 it rejects and
        with q_i(x_i) = 0 < p_i(x_i) it accepts for every uniform in [0, 1);
      - n is reachable when every test before it can accept and test n can
        reject (or n = gamma);
      - the emitted token at n is any token with mass whose CDF interval meets
        [v Z - eps Z, v Z + eps Z]; a token with zero residual weight counts
        only when p and q agree there to zero_eps relative (single-precision
        evaluation could leave it a sliver of mass); a residual that is zero,
        or whose every weight is such a sliver, may also be replaced by p_n.

    The result the oracle itself returns is always in the set; a sequence the
    oracle does not flag has exactly that one result.
    """
    return _outcomes(f64(target_logits[b]), f64(draft_logits[b]), i64(draft_tokens[b]),
                     f64(u_accept[b]), f64(u_sample[b]), temperature, flag_eps, zero_eps)


def _outcomes(zt, zd, x, ua, us, temperature, flag_eps, zero_eps):
    """accept_outcomes for one sequence's float64 rows."""
    gamma = zt.shape[0] - 1
    p = softmax(zt, temperature)
    q = softmax(zd, temperature) if gamma > 0 else np.zeros((0, zt.shape[1]))
    can_acc, can_rej = [], []
    for i in range(gamma):
        t = int(x[i])
        pi, qi = p[i, t], q[i, t]
        acc = bool(ua[i] * qi < pi)
        band = pi > 0 and qi > 0 and abs(ua[i] - pi / qi) < flag_eps
        can_acc.append(acc or band)
        can_rej.append((not acc) or band)
    results = set()
    for n in range(gamma + 1):
        if not all(can_acc[:n]):
            break
        if n < gamma and not can_rej[n]:
            continue
        r, fallback = _residual(p, q, n, gamma)
        if n == gamma:
            ys = _draws_in_band(r, us[n], flag_eps)
        else:
            close = (p[n] > 0) & (np.abs(p[n] - q[n]) <= zero_eps * np.maximum(p[n], q[n]))
            if fallback or not ((r > 0) & ~close).any():
                # every residual weight is zero or within rounding of zero: a
                # single-precision residual may keep any of them, or none (then
                # the draw is from p_n)
                ys = set(np.nonzero(close)[0].tolist()) | _draws_in_band(p[n], us[n], flag_eps)
            else:
                ys = _draws_in_band(r, us[n], flag_eps, (r == 0) & close)
        for y in ys:
            row = [int(v) for v in x[:n]] + [int(y)] + [-1] * (gamma - n)
            results.add((n, tuple(row)))
    return results


def accept_valid(target_logits, draft_logits, draft_tokens, u_accept, u_sample, n_accepted,
                 out_tokens, temperature=1.0, flag_eps=1e-6, zero_eps=1e-5):
    """Check a computed acceptance result per sequence against accept_outcomes.

    Returns (valid bool [B], ambiguous bool [B]): valid[b] when (n_accepted[b],
    out_tokens[b]) is one of sequence b's correct results, ambiguous[b] when
    that sequence has more than one."""
    n_in = i64(n_accepted)
    out_in = i64(out_tokens)
    zt, zd, x = f64(target_logits), f64(draft_logits), i64(draft_tokens)
    ua, us = f64(u_accept), f64(u_sample)
    B = n_in.shape[0]
    valid = np.zeros(B, dtype=bool)
    ambiguous = np.zeros(B, dtype=bool)
    for b in range(B):
        res = _outcomes(zt[b], zd[b], x[b], ua[b], us[b], temperature, flag_eps, zero_eps)
        valid[b] = (int(n_in[b]), tuple(int(v) for v in out_in[b])) in res
        ambiguous[b] = len(res) > 1
    return valid, ambiguous
