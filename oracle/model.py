"""Oracle: the analytic speedup model of speculative decoding.

TEST INFRASTRUCTURE ONLY (see the package header).

The MagicDec summary (jarxiv.com) prints the speedup of speculative decoding
as T_T * Omega(gamma, alpha) / (gamma * T_D + T_V(gamma)), with T_T and T_D
the target and draft times per decoded token, T_V(gamma) the time to verify
the gamma drafted tokens, and Omega the expected number of tokens one round
produces; with a compressed draft cache, gamma * T_D becomes
T_select(K) + gamma * T_D(K) (MagicDec notes §3.1 and §4.1; their equations
are blank in the extracted text). Readings:

  * Omega(gamma, alpha) = (1 - alpha^(gamma + 1)) / (1 - alpha), the result
    of the cited speculative-decoding paper for a constant per-token
    acceptance rate alpha (gamma + 1 at alpha = 1).
  * T_select(K) is the selection time charged to one round: a static
    selection (SnapKV, StreamingLLM) is made once and charged as a fixed
    share, a dynamic one (top-K attention) is searched at every draft step,
    so a round pays gamma searches: T_select = fixed + gamma * per_step.
  * The objective (Eq. 4, blank) is the expected time per token
    (T_select + gamma * T_D(K) + T_V(gamma)) / Omega, minimised over gamma;
    minimising it maximises the speedup.
"""


def omega(gamma, alpha):
    """Expected tokens per round: (1 - alpha^(gamma+1)) / (1 - alpha)."""
    if not (0.0 <= alpha <= 1.0) or gamma < 0:
        raise ValueError("alpha in [0, 1], gamma >= 0")
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def round_time(t_draft, t_verify, gamma, t_select_fixed=0.0, t_select_step=0.0):
    """Time of one round: T_select + gamma * T_D + T_V(gamma)."""
    return t_select_fixed + gamma * t_select_step + gamma * t_draft + t_verify


def speedup(t_target, t_draft, t_verify, gamma, alpha, t_select_fixed=0.0, t_select_step=0.0):
    """T_T * Omega / (T_select + gamma * T_D + T_V(gamma))."""
    return t_target * omega(gamma, alpha) / round_time(t_draft, t_verify, gamma, t_select_fixed, t_select_step)


def best_gamma(t_target, t_draft, t_verify_by_gamma, alpha, t_select_fixed=0.0, t_select_step=0.0):
    """gamma in 1..len(t_verify_by_gamma) (t_verify_by_gamma[g - 1] = T_V(g))
    with the lowest expected time per token; ties to the smaller gamma.
    Returns (gamma, speedup)."""
    best = None
    for g in range(1, len(t_verify_by_gamma) + 1):
        per_token = round_time(t_draft, t_verify_by_gamma[g - 1], g, t_select_fixed, t_select_step) / omega(g, alpha)
        if best is None or per_token < best[0]:
            best = (per_token, g)
    return best[1], t_target / best[0]
