"""Seeded synthetic inputs for the sparse-KV self-speculative decoding hot path.

This package only draws random numbers and lays them out in memory. It holds
none of the method's arithmetic (no attention, no selection, no acceptance):
both the CPU oracle's tests and the HIP path consume exactly the tensors it
returns, so neither side can lean on the other.

Every draw is seeded from a tuple (workload id, tensor id, extra) through
NumPy's SeedSequence, then made with a torch.Generator on the requested device,
so small cases are reproducible on the CPU and the multi-GB workloads are drawn
on the GPU in seconds.
"""
from synth.gen import (  # noqa: F401
    PAGE_SIZE,
    PagedKV,
    WORKLOADS,
    Workload,
    dyadic_uniforms,
    gumbel_tokens,
    logits,
    make_generator,
    paged_kv,
    queries,
    workload_lens,
)
