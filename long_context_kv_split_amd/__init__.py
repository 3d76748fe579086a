"""MI355X (gfx950) hot path of MagicDec-style sparse-KV self-speculative decoding.

The computation lives in libsdkv.so, a HIP library with the C ABI of
include/sd.h: verify attention over a paged bf16 KV cache (split-KV MFMA
kernel plus combine), sparse draft attention over gathered positions,
StreamingLLM and SnapKV draft-KV selection (one budget, or one per sequence;
or in two calls, the window's softmax normalisers and the selection from
them),
per-step top-K attention selection, modified-rejection speculative acceptance,
the round's cache bookkeeping (KV append, length advance, draft over the
selection plus the appended tail), and the analytic speedup model (host
arithmetic on measured step times). This package is its ctypes binding
(argument marshalling only) and its build script; importing it never computes
anything on the CPU.
"""
from long_context_kv_split_amd.binding import (  # noqa: F401
    KVCache,
    LIB_PATH,
    SD_BF16,
    SD_ERR_HIP,
    SD_ERR_INVALID_ARG,
    SD_ERR_UNSUPPORTED,
    SD_ERR_WORKSPACE,
    SD_F32,
    SD_OK,
    SD_SPEC_ACCEPT_SCRATCH_BYTES,
    SdError,
    lib,
    sd_best_gamma,
    sd_draft_attn_sparse,
    sd_draft_attn_sparse_tail,
    sd_draft_attn_sparse_workspace_size,
    sd_expected_tokens,
    sd_hbm_read_probe,
    sd_kv_advance,
    sd_kv_append,
    sd_kv_cache,
    sd_kv_compact,
    sd_snapkv_select,
    sd_snapkv_select_budgets,
    sd_snapkv_select_lse,
    sd_snapkv_select_workspace_size,
    sd_snapkv_window_lse,
    sd_spec_accept,
    sd_spec_accept_noalloc,
    sd_spec_accept_workspace_size,
    sd_speedup,
    sd_streaming_select,
    sd_topk_select,
    sd_topk_select_workspace_size,
    sd_verify_attn,
    sd_verify_attn_workspace_size,
    status_string,
    version,
    workspace,
)
