"""GPU check of the streaming-read probe (the attainable-bandwidth ceiling the
bench reports next to the nominal HBM figure).

The probe adds the sum of the buffer's 32-bit words, modulo 2^32, to a
caller-zeroed counter; the host sums the same words with NumPy. Sizes cover a
single 16-byte chunk, partial last rounds, an exact number of full rounds and
a buffer larger than the last-level cache, with and without the nontemporal
hint. This is measurement plumbing, not a step of the method, so no oracle
function is involved.
"""
import numpy as np
import pytest
import torch

import long_context_kv_split_amd as sd
from tests.gpu_helpers import ensure_lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    torch.cuda.set_device(0)


def host_sum(t):
    words = t.cpu().contiguous().view(torch.int32).numpy().view(np.uint32)
    return int(words.astype(np.uint64).sum() % (1 << 32))


def probe(buf, nontemporal, calls=1, blocks=0):
    c = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(calls):
        sd.sd_hbm_read_probe(buf, nontemporal, c, blocks)
    torch.cuda.synchronize()
    return int(c.cpu().numpy().view(np.uint32)[0])


# 16 B (most waves get an empty slice); ragged; 4 MiB = whole 8 KB wave rounds
# at 512 waves; 300 MiB + 48 B exceeds the 256 MB last-level cache. Launch
# sizes: the resident count (0), one workgroup, and 1000 workgroups.
@pytest.mark.parametrize("nbytes", [16, 16 * 1000003, 4 << 20, (300 << 20) + 48])
@pytest.mark.parametrize("nontemporal", [0, 1])
@pytest.mark.parametrize("blocks", [0, 1, 128, 1000])
def test_probe_checksum_matches_host(nbytes, nontemporal, blocks):
    say(f"probe {nbytes} B nontemporal={nontemporal} blocks={blocks}")
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000 + nontemporal)
    buf = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    want = host_sum(buf)
    assert probe(buf.cuda(), nontemporal, blocks=blocks) == want


def test_probe_accumulates_and_reads_any_dtype():
    say("probe accumulate, bf16 buffer")
    g = torch.Generator(device="cpu").manual_seed(7)
    buf = torch.randn((1 << 20) + 8, generator=g).to(torch.bfloat16)  # 2 MiB + 16 B
    want = host_sum(buf)
    assert probe(buf.cuda(), 1, calls=3) == (3 * want) % (1 << 32)


def test_probe_rejects_host_and_ragged_buffers():
    with pytest.raises(ValueError):
        sd.sd_hbm_read_probe(torch.zeros(16, dtype=torch.int32), 1,
                             torch.zeros(1, dtype=torch.int32, device="cuda"))
    with pytest.raises(sd.SdError):
        sd.sd_hbm_read_probe(torch.zeros(6, dtype=torch.int32, device="cuda"), 1,
                             torch.zeros(1, dtype=torch.int32, device="cuda"))
    with pytest.raises(sd.SdError):
        sd.sd_hbm_read_probe(torch.zeros(16, dtype=torch.int32, device="cuda"), 1,
                             torch.zeros(1, dtype=torch.int32, device="cuda"), 70000)
