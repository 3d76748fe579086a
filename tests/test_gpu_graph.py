"""HIP-graph capture of the prefill-to-accept calls: SnapKV selection (in one
call and in two: the window normalisers, then the selection from them), the
sparse draft over its sets, verify attention and acceptance (gamma = 4),
captured once and replayed several times, with eager library calls and torch
work on the same buffers between the replays. Every replay must reproduce the
eager outputs bit for bit: no call relies on memory cleared by a memset node
or on state kept between calls (the draft-step capture is in
test_gpu_round.py, the top-K one in test_gpu_topk.py).
"""
import pytest
import torch

import long_context_kv_split_amd as sd
from synth import dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries
from tests.gpu_helpers import ensure_lib, say

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def _same(a, b):
    """Bitwise equality, NaN == NaN."""
    if a.dtype == BF16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def test_select_draft_verify_accept_graph_replay_matches_eager():
    say("graph: snapkv + draft + verify + accept")
    B, Hq, Hkv, d, W, budget, gamma, V = 6, 8, 2, 128, 8, 128, 4, 3000
    lens = [2000, 130, 777, 3001, 64, 1500]
    L = max(lens)
    kv_t = paged_kv(97, lens, Hkv, d, BF16, "cuda", shuffle=True, spike_frac=0.1)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    s_ = d ** -0.5
    q_obs = queries(97, 4, (B, W, Hq, d), BF16, "cuda", scale=s_)
    q_d = queries(97, 2, (B, 1, Hq, d), BF16, "cuda", scale=s_)
    q_v = queries(97, 1, (B, gamma + 1, Hq, d), BF16, "cuda", scale=s_)
    zt = logits(97, 8, (B, gamma + 1, V), 2.0, "cuda")
    zd = logits(97, 9, (B, gamma, V), 0.5, "cuda", base=zt[:, :gamma]).contiguous()
    x = gumbel_tokens(97, zd)
    ua = dyadic_uniforms(97, 11, (B, gamma), "cuda")
    us = dyadic_uniforms(97, 12, (B, gamma + 1), "cuda")

    idx = torch.empty((B, Hkv, budget), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    obs_lse = torch.empty((B, W, Hq), dtype=torch.float32, device="cuda")
    idx2 = torch.empty_like(idx)
    sel2 = torch.empty_like(sel)
    o_d = torch.empty_like(q_d)
    o_v, lse_v = torch.empty_like(q_v), torch.empty((B, gamma + 1, Hq), dtype=torch.float32, device="cuda")
    n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    toks = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    ws_s = sd.workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, budget))
    ws_v = sd.workspace(sd.sd_verify_attn_workspace_size(B, gamma + 1, Hq, Hkv, d, L))
    ws_a = sd.workspace(sd.sd_spec_accept_workspace_size(B, gamma, V))
    ws_s2 = sd.workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    # the selection copied into a cache of its own and a dense decode over it;
    # slots past the selections stay NaN in the eager run and every replay
    pps = budget // 16
    k_c = torch.full((B * pps, Hkv, 16, d), float("nan"), dtype=BF16, device="cuda")
    v_c = torch.full_like(k_c, float("nan"))
    kvc = sd.KVCache(k_c, v_c, torch.arange(B * pps, dtype=torch.int32, device="cuda").view(B, pps), sel)
    o_c = torch.empty_like(q_d)
    ws_c = sd.workspace(sd.sd_verify_attn_workspace_size(B, 1, Hq, Hkv, d, budget))
    outs = (idx, sel, o_d, o_v, lse_v, n_acc, toks, obs_lse, idx2, sel2, k_c, v_c, o_c)

    def calls():
        sd.sd_snapkv_select(kv, q_obs, W, Hq, 7, budget, L, 1.0, idx, sel, ws_s)
        sd.sd_snapkv_window_lse(kv, q_obs, W, Hq, L, 1.0, obs_lse, ws_s2)
        sd.sd_snapkv_select_lse(kv, q_obs, obs_lse, W, Hq, 7, budget, L, 1.0, idx2, sel2, ws_s2)
        sd.sd_draft_attn_sparse(kv, q_d, 1, Hq, idx, sel, Hkv, budget, 1.0, o_d, None, ws_d)
        sd.sd_kv_compact(kv, idx, sel, Hkv, budget, pps, k_c, v_c)
        sd.sd_verify_attn(kvc, q_d, 1, Hq, budget, 1.0, o_c, None, ws_c)
        sd.sd_verify_attn(kv, q_v, gamma + 1, Hq, L, 1.0, o_v, lse_v, ws_v)
        sd.sd_spec_accept(zt, zd, x, ua, us, gamma, V, 1.0, n_acc, toks, ws_a)

    calls()  # eager (also warms the occupancy queries before capture)
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]

    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            calls()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: scribble over every output and workspace,
        # and run the library eagerly on other inputs through the same workspaces
        for t in outs:
            t.fill_(-5 if not t.is_floating_point() else float("nan"))
        for w in (ws_s, ws_s2, ws_d, ws_v, ws_a, ws_c):
            w.fill_(0xA5)
        if rep % 2 == 1:
            sd.sd_verify_attn(kv, q_v.flip(0).contiguous(), gamma + 1, Hq, L, 1.0, o_v, lse_v, ws_v)
            sd.sd_spec_accept(zt.flip(0).contiguous(), zd.flip(0).contiguous(), x.flip(0).contiguous(), ua, us,
                              gamma, V, 1.0, n_acc, toks, ws_a)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("idx", "sel_lens", "draft_out", "verify_out", "verify_lse", "n_accepted",
                                   "out_tokens", "window_lse", "idx_from_lse", "sel_lens_from_lse",
                                   "compact_k", "compact_v", "draft_over_compact"), outs, want):
            assert _same(got, ref), f"replay {rep}: {name} differs from the eager run"
