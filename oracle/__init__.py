"""CPU fp64 oracle for the sparse-KV self-speculative decoding hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this package. The HIP library never
calls it, shares no code, header, table or helper with it, and the product path
fails loudly when its extension is missing instead of falling back here.

What it computes follows the MagicDec pages ("MagicDec: Breaking the
Latency-Throughput Tradeoff for Long Context Generation with Speculative
Decoding", deep notes on papercache.org, and the speculative-decoding explainer
"Wann beschleunigt spekulatives Decoding das LLM-Serving?" on slavadubrov.com),
written plainly in NumPy float64: every bf16 or fp32 input converts to float64
exactly, and each step is the textbook definition or the pages' stated
algorithm, with no blocking or reordering.

Functions and what pins them (tests/test_oracle_*.py):
  attention.verify_attn    library SDPA, pure-Python loops, closed forms,
                           decode/truncation and page-permutation invariants
  attention.sparse_attn    dense equivalence, index-order invariance
  selection.streaming_select  hand-listed sets, dense equivalence
  selection.snapkv_votes   brute-force double loop, column sums of a library softmax
  selection.maxpool1d      brute force, hand fixture
  selection.topk_lowest_index  brute-force subset enumeration
  selection.snapkv_select  brute-force subset search on tiny inputs (one budget,
                           and per-sequence budgets in a ragged batch), special cases
  accept.spec_accept       hand-worked fixtures, Monte Carlo distribution
                           preservation, closed-form acceptance probabilities
                           (with gamma = 0 it is the draft-token sampler)
  round.kv_append          caches built from dense concatenations; verify after
                           append equals SDPA with a causal mask
  round.kv_advance         hand values, the round identity L + 1 + n
  round.sparse_attn_tail   SDPA over explicitly gathered rows; tail-only equals
                           dense decode
  dynamic.topk_select      brute-force subset search on tiny inputs with integer
                           scores (ties), hand-listed per-head sets
  dynamic.topk_attn        budget >= L equals dense decode; the dropped-mass bound
                           against library SDPA over the whole cache; library SDPA
                           over each head's gathered rows
  model.omega / speedup / best_gamma  Monte Carlo of the round process, the
                           explicit sum over acceptance lengths, limits, hand values
No function here is "parity unpinned".
"""
from oracle.attention import attend, sparse_attn, token_rows, verify_attn  # noqa: F401
from oracle.selection import (  # noqa: F401
    maxpool1d,
    snapkv_select,
    snapkv_votes,
    streaming_select,
    topk_lowest_index,
)
from oracle.accept import accept_outcomes, accept_valid, softmax, spec_accept  # noqa: F401
from oracle.round import draft_positions, kv_advance, kv_append, kv_compact, sparse_attn_tail  # noqa: F401
from oracle.dynamic import topk_attn, topk_scores, topk_select  # noqa: F401
from oracle.model import best_gamma, omega, round_time, speedup  # noqa: F401
from oracle.common import f64  # noqa: F401
