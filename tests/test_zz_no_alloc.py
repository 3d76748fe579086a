"""The allocation-free acceptance entry point (sd_spec_accept_noalloc) against
the workspace entry point (sd_spec_accept): bit-identical outputs on two calls
in a row, the second smaller than the first (the shared per-GPU scratch keeps
the first call's contents), each also held to the oracle's acceptance bar; a
call needing more scratch than the library holds is rejected before any
launch; and the call replays from a HIP graph."""
import pytest
import torch

import long_context_kv_split_amd as sd
from synth import dyadic_uniforms, gumbel_tokens, logits
from tests.gpu_helpers import check_accept, dirty_workspace, ensure_lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def _inputs(seed, B, gamma, V, noise=0.5):
    zt = logits(seed, 8, (B, gamma + 1, V), 2.0, "cuda")
    zd = logits(seed, 9, (B, gamma, V), noise, "cuda", base=zt[:, :gamma]).contiguous()
    x = gumbel_tokens(seed, zd)
    ua = dyadic_uniforms(seed, 11, (B, gamma), "cuda")
    us = dyadic_uniforms(seed, 12, (B, gamma + 1), "cuda")
    return zt, zd, x, ua, us


def _both(zt, zd, x, ua, us, gamma, V):
    B = zt.shape[0]
    n_ws = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    t_ws = torch.full((B, gamma + 1), -7, dtype=torch.int32, device="cuda")
    ws = dirty_workspace(sd.sd_spec_accept_workspace_size(B, gamma, V), "cuda")
    sd.sd_spec_accept(zt, zd, x, ua, us, gamma, V, 1.0, n_ws, t_ws, ws)
    n_na = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    t_na = torch.full((B, gamma + 1), -9, dtype=torch.int32, device="cuda")
    sd.sd_spec_accept_noalloc(zt, zd, x, ua, us, gamma, V, 1.0, n_na, t_na)
    torch.cuda.synchronize()
    return n_ws, t_ws, n_na, t_na


@pytest.mark.parametrize("first,second", [((128, 4, 128256), (16, 2, 5000)),
                                          ((300, 3, 32000), (7, 0, 1000))])
def test_noalloc_matches_workspace_entry_on_two_calls(first, second):
    for i, (B, gamma, V) in enumerate((first, second)):
        assert sd.sd_spec_accept_workspace_size(B, gamma, V) <= sd.SD_SPEC_ACCEPT_SCRATCH_BYTES
        say(f"noalloc call {i}: B={B} gamma={gamma} V={V}")
        zt, zd, x, ua, us = _inputs(40 + i, B, gamma, V)
        n_ws, t_ws, n_na, t_na = _both(zt, zd, x, ua, us, gamma, V)
        assert torch.equal(n_ws, n_na) and torch.equal(t_ws, t_na), (B, gamma, V)
        check_accept(f"noalloc accept B={B} gamma={gamma} V={V}", n_na.cpu().numpy(), t_na.cpu().numpy(),
                     zt, zd, x, ua, us)


def test_noalloc_rejects_more_scratch_than_it_holds():
    B, gamma, V = 30000, 4, 1000
    assert sd.sd_spec_accept_workspace_size(B, gamma, V) > sd.SD_SPEC_ACCEPT_SCRATCH_BYTES
    zt, zd, x, ua, us = _inputs(47, B, gamma, V)
    n = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    t = torch.full((B, gamma + 1), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(sd.SdError) as e:
        sd.sd_spec_accept_noalloc(zt, zd, x, ua, us, gamma, V, 1.0, n, t)
    assert e.value.status == sd.SD_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (n == -5).all() and (t == -5).all()


def test_noalloc_replays_from_a_graph():
    B, gamma, V = 64, 4, 50000
    zt, zd, x, ua, us = _inputs(49, B, gamma, V)
    n_ws, t_ws, _, _ = _both(zt, zd, x, ua, us, gamma, V)
    n = torch.empty((B,), dtype=torch.int32, device="cuda")
    t = torch.empty((B, gamma + 1), dtype=torch.int32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            sd.sd_spec_accept_noalloc(zt, zd, x, ua, us, gamma, V, 1.0, n, t)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for r in range(3):
        n.fill_(-3)
        t.fill_(-3)
        # an eager call of another shape in between overwrites the shared scratch
        zs, zds, xs, uas, uss = _inputs(50 + r, 5, 2, 3000)
        ns = torch.empty((5,), dtype=torch.int32, device="cuda")
        ts = torch.empty((5, 3), dtype=torch.int32, device="cuda")
        sd.sd_spec_accept_noalloc(zs, zds, xs, uas, uss, 2, 3000, 1.0, ns, ts)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(n, n_ws) and torch.equal(t, t_ws), r
