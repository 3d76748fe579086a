"""Seeded generators and the workload table (shapes and value distributions only).

Tensor ids used in seeds: 1 Q, 2 K, 3 V, 4 observation-window queries,
5 spike set, 6 ragged lengths, 7 page permutation, 8 target logits,
9 draft logits / noise, 10 draft-token noise, 11 accept uniforms,
12 sampling uniforms.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 16


def make_generator(parts, device="cpu") -> torch.Generator:
    """torch.Generator seeded from a tuple of non-negative ints."""
    seed = int(np.random.SeedSequence([int(p) for p in parts]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed & ((1 << 63) - 1))
    return g


@dataclass
class PagedKV:
    """One layer's paged KV cache.

    k_pages, v_pages: [num_pages, num_kv_heads, page_size, head_dim]; each
    (page, head) block is contiguous (page_size * head_dim elements).
    page_table: int32 [batch, max_pages]; entries past a sequence's last page
    point at a spare page filled with NaN.
    kv_lens: int32 [batch].
    """

    k_pages: torch.Tensor
    v_pages: torch.Tensor
    page_table: torch.Tensor
    kv_lens: torch.Tensor
    page_size: int
    spare_page: int
    lens: list = field(default_factory=list)

    @property
    def batch(self):
        return int(self.page_table.shape[0])

    @property
    def max_pages(self):
        return int(self.page_table.shape[1])

    @property
    def num_kv_heads(self):
        return int(self.k_pages.shape[1])

    @property
    def head_dim(self):
        return int(self.k_pages.shape[3])

    @property
    def max_kv_len(self):
        return max(self.lens) if self.lens else 0


def _randn(shape, gen, device, chunk_rows=None):
    """Standard normal fp32 draws, made in slabs along dim 0 to bound peak memory."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    n0 = shape[0]
    if chunk_rows is None or chunk_rows >= n0:
        out.normal_(generator=gen)
        return out
    for s in range(0, n0, chunk_rows):
        out[s:s + chunk_rows].normal_(generator=gen)
    return out


def paged_kv(seed, lens, num_kv_heads, head_dim, dtype=torch.bfloat16, device="cpu",
             shuffle=False, spike_frac=0.0, spike_gain=4.0, poison=True,
             page_size=PAGE_SIZE, extra_pages=1) -> PagedKV:
    """Draw K, V ~ N(0, 1) into a paged pool.

    lens: per-sequence token counts. Sequence b owns ceil(lens[b]/page_size)
    pages; with shuffle=False they are laid out in order, else the physical
    page ids are a seeded permutation. `extra_pages` spare pages are appended
    (NaN-filled when poison=True) and unused page-table entries point at the
    first spare. With poison=True the slots past lens[b] in the last page of b
    hold NaN, so any kernel that lets them reach an output shows it.
    spike_frac > 0 multiplies the K rows of a seeded spike_frac share of the
    positions of every (sequence, kv head) by spike_gain.
    """
    lens = [int(x) for x in lens]
    B = len(lens)
    P = page_size
    npg = [max(1, math.ceil(L / P)) for L in lens]
    max_pages = max(npg)
    used = sum(npg)
    total = used + extra_pages
    if shuffle:
        g = make_generator((seed, 7, 0), "cpu")
        perm = torch.randperm(total, generator=g).to(torch.int64)
    else:
        perm = torch.arange(total, dtype=torch.int64)
    spare = int(perm[used])
    pt = torch.full((B, max_pages), spare, dtype=torch.int64)
    off = 0
    for b in range(B):
        pt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]

    rows_per_slab = max(1, (1 << 27) // (num_kv_heads * P * head_dim))
    shape = (total, num_kv_heads, P, head_dim)
    gk = make_generator((seed, 2, 0), device)
    gv = make_generator((seed, 3, 0), device)
    k = _randn(shape, gk, device, rows_per_slab)
    v = _randn(shape, gv, device, rows_per_slab)

    if spike_frac > 0:
        gs = make_generator((seed, 5, 0), device)
        for b in range(B):
            L = lens[b]
            n_sp = int(round(spike_frac * L))
            if n_sp == 0:
                continue
            keys = torch.rand((num_kv_heads, L), generator=gs, device=device)
            pos = torch.topk(keys, n_sp, dim=1).indices  # [Hkv, n_sp]
            pages = pt[b].to(device)[pos // P]
            slots = pos % P
            heads = torch.arange(num_kv_heads, device=device).unsqueeze(1).expand_as(pos)
            k[pages, heads, slots, :] *= spike_gain

    k = k.to(dtype)
    v = v.to(dtype)
    if poison:
        nan = float("nan")
        for b in range(B):
            tail = lens[b] % P
            if tail:
                last = int(pt[b, npg[b] - 1])
                k[last, :, tail:, :] = nan
                v[last, :, tail:, :] = nan
            if lens[b] == 0:
                k[int(pt[b, 0])] = nan
                v[int(pt[b, 0])] = nan
        for j in range(used, total):
            k[int(perm[j])] = nan
            v[int(perm[j])] = nan
    return PagedKV(k_pages=k, v_pages=v, page_table=pt.to(torch.int32).to(device),
                   kv_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                   page_size=P, spare_page=spare, lens=lens)


def queries(seed, tensor_id, shape, dtype=torch.bfloat16, device="cpu", scale=1.0):
    """N(0,1) * scale, rounded to dtype (round-to-nearest-even for bf16)."""
    g = make_generator((seed, tensor_id, 0), device)
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(generator=g)
    return (x * scale).to(dtype)


def logits(seed, tensor_id, shape, std, device="cpu", base=None):
    """fp32 logits ~ N(0, std^2); with `base`, base + N(0, std^2)."""
    g = make_generator((seed, tensor_id, 0), device)
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(generator=g)
    x *= std
    if base is not None:
        x += base
    return x


def gumbel_tokens(seed, logits_t, temperature=1.0):
    """Draw one token per row of `logits_t` [..., V] by the Gumbel-max trick.

    This stands in for the draft model's own sampling (upstream of the accept
    step); the accept step never sees how the tokens were drawn.
    """
    g = make_generator((seed, 10, 0), logits_t.device)
    u = torch.empty(logits_t.shape, dtype=torch.float64, device=logits_t.device)
    u.uniform_(generator=g)
    u.clamp_(min=1e-300)
    noise = -torch.log(-torch.log(u))
    return torch.argmax(logits_t.double() / temperature + noise, dim=-1).to(torch.int32)


def dyadic_uniforms(seed, tensor_id, shape, device="cpu"):
    """Uniforms k * 2^-24, k in [0, 2^24): exact in fp32 and fp64, always < 1."""
    g = make_generator((seed, tensor_id, 0), device)
    k = torch.randint(0, 1 << 24, shape, generator=g, device=device, dtype=torch.int64)
    return (k.to(torch.float64) * (2.0 ** -24)).to(torch.float32)


@dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""

    name: str
    dtype: str              # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int            # kv_len at verify (fixed-length workloads)
    gamma: int
    ragged: tuple = None    # (lo, hi) inclusive uniform lengths
    shuffle: bool = False
    draft: str = "streaming"  # "streaming" or "snapkv"
    sink: int = 0
    recent: int = 0
    window: int = 0
    pool_kernel: int = 0
    budget: int = 0
    spike_frac: float = 0.0
    vocab: int = 0
    target_std: float = 2.0
    draft_noise_std: float = None   # None: independent draft logits with target_std
    seed: int = 0


WORKLOADS = {
    "tiny-f32": Workload(
        name="tiny-f32", dtype="f32", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64,
        context=256, gamma=3, draft="streaming", sink=16, recent=48, vocab=1000,
        target_std=2.0, draft_noise_std=None, seed=1),
    "llama8b-b32-l8k": Workload(
        name="llama8b-b32-l8k", dtype="bf16", batch=32, num_q_heads=32, num_kv_heads=8,
        head_dim=128, context=8192, gamma=3, draft="streaming", sink=64, recent=448, seed=2),
    "llama8b-b128-l32k-snapkv": Workload(
        name="llama8b-b128-l32k-snapkv", dtype="bf16", batch=128, num_q_heads=32,
        num_kv_heads=8, head_dim=128, context=32768, gamma=4, draft="snapkv", window=32,
        pool_kernel=7, budget=2048, spike_frac=0.10, seed=3),
    "ragged-b256-l4k-32k": Workload(
        name="ragged-b256-l4k-32k", dtype="bf16", batch=256, num_q_heads=32, num_kv_heads=8,
        head_dim=128, context=32768, gamma=3, ragged=(4096, 32768), shuffle=True,
        draft="streaming", sink=64, recent=448, seed=4),
    "llama70b-b64-l16k": Workload(
        name="llama70b-b64-l16k", dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8,
        head_dim=128, context=16384, gamma=4, vocab=128256, target_std=2.0,
        draft_noise_std=0.5, seed=5),
}


def workload_lens(w: Workload):
    """Per-sequence kv_len: fixed, or seeded uniform integers in [lo, hi]."""
    if w.ragged is None:
        return [w.context] * w.batch
    g = make_generator((w.seed, 6, 0), "cpu")
    lo, hi = w.ragged
    return torch.randint(lo, hi + 1, (w.batch,), generator=g).tolist()
