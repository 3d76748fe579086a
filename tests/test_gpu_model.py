"""The analytic speedup model on kernel times measured on the GPU.

The MagicDec summary page's speedup formula (and MagicDec notes §3.1, §4.1:
with a compressed draft cache the draft's cost is T_select(K) + gamma T_D(K))
evaluated by the library (sd_best_gamma, host code) on attention times measured
here with HIP events: T_T = decode (one query row over the whole cache),
T_V(g) = verify with g + 1 rows, T_D(K) = one draft step over a StreamingLLM
or SnapKV set, T_select = the SnapKV selection (once per prefill, charged as a
fixed share of one round) or nothing. The chosen gamma and the speedup must
equal the oracle's (oracle/model.py) on the same measured times.
"""
import math

import pytest
import torch

import long_context_kv_split_amd as sd
import oracle
from synth import WORKLOADS, paged_kv, queries, workload_lens
from tests.gpu_helpers import ensure_lib, say
from tests.parity_log import record

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def timed(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def test_best_gamma_on_measured_times_matches_oracle():
    w = WORKLOADS["llama8b-b32-l8k"]
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens = workload_lens(w)
    L, max_gamma = max(lens), 6
    kv_t = paged_kv(w.seed, lens, Hkv, d, BF16, "cuda")
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    q_all = queries(w.seed, 1, (B, max_gamma + 1, Hq, d), BF16, "cuda", scale=d ** -0.5)
    ws_v = sd.workspace(sd.sd_verify_attn_workspace_size(B, max_gamma + 1, Hq, Hkv, d, L))
    t_v = []
    for g in range(0, max_gamma + 1):
        qg = q_all[:, :g + 1].contiguous()
        og = torch.empty_like(qg)
        t_v.append(timed(lambda: sd.sd_verify_attn(kv, qg, g + 1, Hq, L, 1.0, og, None, ws_v)))
    t_target, t_verify = t_v[0], t_v[1:]
    q1 = q_all[:, :1].contiguous()
    o1 = torch.empty_like(q1)
    # StreamingLLM-512 draft
    cap = w.sink + w.recent
    s_idx = torch.empty((B, 1, cap), dtype=torch.int32, device="cuda")
    s_sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    sd.sd_streaming_select(kv_t.kv_lens, w.sink, w.recent, s_idx, s_sel)
    ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, 1024))
    t_stream = timed(lambda: sd.sd_draft_attn_sparse(kv, q1, 1, Hq, s_idx, s_sel, 1, cap, 1.0, o1, None, ws_d))
    # SnapKV-1024 draft and its selection
    W, K = 32, 1024
    q_obs = queries(w.seed, 4, (B, W, Hq, d), BF16, "cuda", scale=d ** -0.5)
    k_idx = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
    k_sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws_s = sd.workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    t_select = timed(lambda: sd.sd_snapkv_select(kv, q_obs, W, Hq, 7, K, L, 1.0, k_idx, k_sel, ws_s))
    t_snap = timed(lambda: sd.sd_draft_attn_sparse(kv, q1, 1, Hq, k_idx, k_sel, Hkv, K, 1.0, o1, None, ws_d))
    say(f"T_T {t_target:.4f} ms, T_V {[round(t, 4) for t in t_verify]}, T_D stream {t_stream:.4f}, "
        f"T_D snap {t_snap:.4f}, T_select {t_select:.4f}")
    cases = []
    for alpha in (0.6, 0.8, 0.9):
        cases.append(("streaming-512", t_stream, 0.0, 0.0, alpha))
        cases.append(("snapkv-1024, selection per round", t_snap, t_select, 0.0, alpha))
        cases.append(("snapkv-1024, selection once", t_snap, 0.0, 0.0, alpha))
    for name, t_d, fixed, step, alpha in cases:
        g, s = sd.sd_best_gamma(t_target, t_d, t_verify, alpha, fixed, step)
        g_ref, s_ref = oracle.best_gamma(t_target, t_d, t_verify, alpha, fixed, step)
        assert g == g_ref and math.isclose(s, s_ref, rel_tol=1e-12), (name, alpha, g, g_ref, s, s_ref)
        for gg in range(1, max_gamma + 1):
            got = sd.sd_speedup(t_target, t_d, t_verify[gg - 1], gg, alpha, fixed, step)
            want = oracle.speedup(t_target, t_d, t_verify[gg - 1], gg, alpha, fixed, step)
            assert math.isclose(got, want, rel_tol=1e-12), (name, alpha, gg)
        record(f"speedup model {name} alpha={alpha}", best_gamma=g, speedup=s)
    record("speedup model measured times (ms)", T_T=t_target, T_V1=t_verify[0], T_V6=t_verify[-1],
           T_D_stream512=t_stream, T_D_snap1024=t_snap, T_select_snap1024=t_select)
