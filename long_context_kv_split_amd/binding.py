"""ctypes binding of libsdkv.so, one Python function per C entry point in sd.h.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a non-zero status raises SdError. Every
step of the computation runs in the HIP library; if the library is missing,
loading raises instead of falling back to anything else.

Before handing a tensor to the library the binding checks that it lives on a
GPU, is contiguous, has the expected dtype and holds at least the elements the
C call will touch, so a host pointer or a short buffer never reaches a kernel.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdkv.so")

SD_OK, SD_ERR_INVALID_ARG, SD_ERR_UNSUPPORTED, SD_ERR_WORKSPACE, SD_ERR_HIP = range(5)
SD_BF16, SD_F32 = 0, 1
_DTYPES = {torch.bfloat16: SD_BF16, torch.float32: SD_F32}


class SdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class sd_kv_cache(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("kv_lens", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
_KV = ctypes.POINTER(sd_kv_cache)

_SIGNATURES = {
    "sd_verify_attn": (_I, [_KV, _P, _I, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_verify_attn_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "sd_draft_attn_sparse": (_I, [_KV, _P, _I, _I, _I, _P, _P, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_draft_attn_sparse_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "sd_draft_attn_sparse_tail": (_I, [_KV, _P, _I, _I, _I, _P, _P, _I, _I, _P, _I, _F, _P, _P, _P, _S, _P]),
    "sd_kv_append": (_I, [_KV, _P, _P, _I, _I, _P]),
    "sd_kv_advance": (_I, [_P, _P, _I, _I, _P]),
    "sd_kv_compact": (_I, [_KV, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "sd_streaming_select": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "sd_snapkv_select": (_I, [_KV, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_snapkv_select_workspace_size": (_S, [_I, _I, _I, _I, _I]),
    "sd_snapkv_select_budgets": (_I, [_KV, _P, _I, _I, _I, _I, _P, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_snapkv_window_lse": (_I, [_KV, _P, _I, _I, _I, _I, _F, _P, _P, _S, _P]),
    "sd_snapkv_select_lse": (_I, [_KV, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_topk_select": (_I, [_KV, _P, _I, _I, _I, _I, _P, _P, _P, _S, _P]),
    "sd_topk_select_workspace_size": (_S, [_I, _I, _I, _I]),
    "sd_spec_accept": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "sd_spec_accept_workspace_size": (_S, [_I, _I, _I]),
    "sd_spec_accept_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P]),
    "sd_expected_tokens": (ctypes.c_double, [_I, ctypes.c_double]),
    "sd_speedup": (ctypes.c_double, [ctypes.c_double] * 3 + [_I] + [ctypes.c_double] * 3),
    "sd_best_gamma": (_I, [ctypes.c_double, ctypes.c_double, _P, _I, ctypes.c_double, ctypes.c_double,
                           ctypes.c_double, _P, _P]),
    "sd_hbm_read_probe": (_I, [_P, _S, _I, _I, _P, _P]),
    "sd_status_string": (ctypes.c_char_p, [_I]),
    "sd_version": (_I, []),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m long_context_kv_split_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status):
    return lib().sd_status_string(int(status)).decode()


def version():
    return int(lib().sd_version())


def sd_expected_tokens(gamma, alpha):
    return float(lib().sd_expected_tokens(int(gamma), float(alpha)))


def sd_speedup(t_target, t_draft, t_verify, gamma, alpha, t_select_fixed=0.0, t_select_step=0.0):
    return float(lib().sd_speedup(float(t_target), float(t_draft), float(t_verify), int(gamma), float(alpha),
                                  float(t_select_fixed), float(t_select_step)))


def sd_best_gamma(t_target, t_draft, t_verify_by_gamma, alpha, t_select_fixed=0.0, t_select_step=0.0):
    """(gamma, speedup); t_verify_by_gamma[g - 1] = T_V(g), host floats."""
    n = len(t_verify_by_gamma)
    tv = (ctypes.c_double * max(n, 1))(*[float(t) for t in t_verify_by_gamma])
    g = ctypes.c_int32(0)
    sp = ctypes.c_double(0.0)
    _check(lib().sd_best_gamma(float(t_target), float(t_draft), ctypes.cast(tv, _P), n, float(alpha),
                               float(t_select_fixed), float(t_select_step), ctypes.byref(g), ctypes.byref(sp)),
           "sd_best_gamma")
    return int(g.value), float(sp.value)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _check(status, where):
    if status != SD_OK:
        raise SdError(status, where)


class KVCache:
    """Paged KV cache handed to the library (keeps its tensors alive)."""

    def __init__(self, k_pages, v_pages, page_table, kv_lens):
        if k_pages.dtype not in _DTYPES:
            raise ValueError("k_pages must be bfloat16 or float32")
        if k_pages.dim() != 4:
            raise ValueError("k_pages must be [num_pages, num_kv_heads, page_size, head_dim]")
        self.k_pages, self.v_pages, self.page_table, self.kv_lens = k_pages, v_pages, page_table, kv_lens
        B = page_table.shape[0]
        s = sd_kv_cache()
        s.k_pages = _dev(k_pages, "k_pages")
        s.v_pages = _dev(v_pages, "v_pages", k_pages.dtype, k_pages.numel()) if v_pages is not None else None
        s.page_table = _dev(page_table, "page_table", torch.int32)
        s.kv_lens = _dev(kv_lens, "kv_lens", torch.int32, B)
        s.num_pages, s.num_kv_heads, s.page_size, s.head_dim = (int(x) for x in k_pages.shape)
        s.max_pages = int(page_table.shape[1])
        s.dtype = _DTYPES[k_pages.dtype]
        self.struct = s
        self.dtype = k_pages.dtype
        self.batch = int(B)

    @property
    def num_kv_heads(self):
        return self.struct.num_kv_heads

    @property
    def head_dim(self):
        return self.struct.head_dim

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def sd_verify_attn_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_kv_len):
    return int(lib().sd_verify_attn_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim,
                                                   max_kv_len))


def sd_draft_attn_sparse_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_sel):
    return int(lib().sd_draft_attn_sparse_workspace_size(batch, n_q, num_q_heads, num_kv_heads,
                                                         head_dim, max_sel))


def sd_topk_select_workspace_size(batch, num_q_heads, num_kv_heads, max_kv_len):
    return int(lib().sd_topk_select_workspace_size(batch, num_q_heads, num_kv_heads, max_kv_len))


def sd_snapkv_select_workspace_size(batch, window, num_q_heads, num_kv_heads, max_kv_len):
    return int(lib().sd_snapkv_select_workspace_size(batch, window, num_q_heads, num_kv_heads,
                                                     max_kv_len))


def sd_spec_accept_workspace_size(batch, gamma, vocab):
    return int(lib().sd_spec_accept_workspace_size(batch, gamma, vocab))


def _ws(workspace, need):
    if need == 0:
        return None, 0
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def sd_verify_attn(kv, q, n_q, num_q_heads, max_kv_len, softmax_scale, out, lse=None,
                   workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    n = B * n_q * num_q_heads * d
    qp = _dev(q, "q", kv.dtype, n)
    op = _dev(out, "out", kv.dtype, n)
    lp = _dev(lse, "lse", torch.float32, B * n_q * num_q_heads, allow_none=True)
    need = sd_verify_attn_workspace_size(B, n_q, num_q_heads, kv.num_kv_heads, d, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_verify_attn(kv.ref, qp, B, n_q, num_q_heads, max_kv_len, softmax_scale, op, lp,
                                wp, wb, _stream(stream)), "sd_verify_attn")


def sd_draft_attn_sparse(kv, q, n_q, num_q_heads, idx, sel_lens, idx_heads, max_sel, softmax_scale,
                         out, lse=None, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    n = B * n_q * num_q_heads * d
    qp = _dev(q, "q", kv.dtype, n)
    op = _dev(out, "out", kv.dtype, n)
    lp = _dev(lse, "lse", torch.float32, B * n_q * num_q_heads, allow_none=True)
    ip = _dev(idx, "idx", torch.int32, B * idx_heads * max_sel)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    need = sd_draft_attn_sparse_workspace_size(B, n_q, num_q_heads, kv.num_kv_heads, d, max_sel)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_draft_attn_sparse(kv.ref, qp, B, n_q, num_q_heads, ip, sp, idx_heads, max_sel,
                                      softmax_scale, op, lp, wp, wb, _stream(stream)),
           "sd_draft_attn_sparse")


def sd_draft_attn_sparse_tail(kv, q, n_q, num_q_heads, idx, sel_lens, idx_heads, max_sel, tail_begin,
                              max_tail, softmax_scale, out, lse=None, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    n = B * n_q * num_q_heads * d
    qp = _dev(q, "q", kv.dtype, n)
    op = _dev(out, "out", kv.dtype, n)
    lp = _dev(lse, "lse", torch.float32, B * n_q * num_q_heads, allow_none=True)
    ip = _dev(idx, "idx", torch.int32, B * idx_heads * max_sel)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    tp = _dev(tail_begin, "tail_begin", torch.int32, B)
    need = sd_draft_attn_sparse_workspace_size(B, n_q, num_q_heads, kv.num_kv_heads, d, max_sel)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_draft_attn_sparse_tail(kv.ref, qp, B, n_q, num_q_heads, ip, sp, idx_heads, max_sel, tp,
                                           max_tail, softmax_scale, op, lp, wp, wb, _stream(stream)),
           "sd_draft_attn_sparse_tail")


def sd_kv_append(kv, k_new, v_new, n_new, stream=None):
    B, d = kv.batch, kv.head_dim
    n = B * n_new * kv.num_kv_heads * d
    kp = _dev(k_new, "k_new", kv.dtype, n)
    vp = _dev(v_new, "v_new", kv.dtype, n)
    _check(lib().sd_kv_append(kv.ref, kp, vp, B, n_new, _stream(stream)), "sd_kv_append")


def sd_kv_advance(kv_lens, n_accepted, add, stream=None):
    B = kv_lens.numel()
    lp = _dev(kv_lens, "kv_lens", torch.int32, B)
    np_ = _dev(n_accepted, "n_accepted", torch.int32, B, allow_none=True)
    _check(lib().sd_kv_advance(lp, np_, B, add, _stream(stream)), "sd_kv_advance")


def sd_kv_compact(kv, idx, sel_lens, idx_heads, max_sel, pages_per_seq, k_out, v_out, stream=None):
    B = kv.batch
    n = B * pages_per_seq * kv.num_kv_heads * kv.struct.page_size * kv.head_dim
    ip = _dev(idx, "idx", torch.int32, B * idx_heads * max_sel)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    kp = _dev(k_out, "k_out", kv.dtype, n)
    vp = _dev(v_out, "v_out", kv.dtype, n)
    _check(lib().sd_kv_compact(kv.ref, ip, sp, B, idx_heads, max_sel, pages_per_seq, kp, vp, _stream(stream)),
           "sd_kv_compact")


def sd_streaming_select(kv_lens, sink, recent, idx, sel_lens, stream=None):
    B = kv_lens.numel()
    lp = _dev(kv_lens, "kv_lens", torch.int32, B)
    ip = _dev(idx, "idx", torch.int32, B * (sink + recent))
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    _check(lib().sd_streaming_select(lp, B, sink, recent, ip, sp, _stream(stream)),
           "sd_streaming_select")


def sd_snapkv_select(kv, q_obs, window, num_q_heads, pool_kernel, budget, max_kv_len,
                     softmax_scale, idx, sel_lens, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    qp = _dev(q_obs, "q_obs", kv.dtype, B * window * num_q_heads * d)
    ip = _dev(idx, "idx", torch.int32, B * kv.num_kv_heads * budget)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    need = sd_snapkv_select_workspace_size(B, window, num_q_heads, kv.num_kv_heads, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_snapkv_select(kv.ref, qp, B, window, num_q_heads, pool_kernel, budget, max_kv_len,
                                  softmax_scale, ip, sp, wp, wb, _stream(stream)), "sd_snapkv_select")


def sd_snapkv_window_lse(kv, q_obs, window, num_q_heads, max_kv_len, softmax_scale, lse, workspace=None,
                         stream=None):
    B, d = kv.batch, kv.head_dim
    qp = _dev(q_obs, "q_obs", kv.dtype, B * window * num_q_heads * d)
    lp = _dev(lse, "lse", torch.float32, B * window * num_q_heads)
    need = sd_snapkv_select_workspace_size(B, window, num_q_heads, kv.num_kv_heads, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_snapkv_window_lse(kv.ref, qp, B, window, num_q_heads, max_kv_len, softmax_scale, lp, wp,
                                      wb, _stream(stream)), "sd_snapkv_window_lse")


def sd_snapkv_select_lse(kv, q_obs, obs_lse, window, num_q_heads, pool_kernel, budget, max_kv_len,
                         softmax_scale, idx, sel_lens, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    qp = _dev(q_obs, "q_obs", kv.dtype, B * window * num_q_heads * d)
    lp = _dev(obs_lse, "obs_lse", torch.float32, B * window * num_q_heads)
    ip = _dev(idx, "idx", torch.int32, B * kv.num_kv_heads * budget)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    need = sd_snapkv_select_workspace_size(B, window, num_q_heads, kv.num_kv_heads, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_snapkv_select_lse(kv.ref, qp, lp, B, window, num_q_heads, pool_kernel, budget, max_kv_len,
                                      softmax_scale, ip, sp, wp, wb, _stream(stream)), "sd_snapkv_select_lse")


def sd_snapkv_select_budgets(kv, q_obs, window, num_q_heads, pool_kernel, budgets, max_budget, max_kv_len,
                             softmax_scale, idx, sel_lens, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    qp = _dev(q_obs, "q_obs", kv.dtype, B * window * num_q_heads * d)
    bp = _dev(budgets, "budgets", torch.int32, B)
    ip = _dev(idx, "idx", torch.int32, B * kv.num_kv_heads * max_budget)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    need = sd_snapkv_select_workspace_size(B, window, num_q_heads, kv.num_kv_heads, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_snapkv_select_budgets(kv.ref, qp, B, window, num_q_heads, pool_kernel, bp, max_budget,
                                          max_kv_len, softmax_scale, ip, sp, wp, wb, _stream(stream)),
           "sd_snapkv_select_budgets")


def sd_topk_select(kv, q, num_q_heads, budget, max_kv_len, idx, sel_lens, workspace=None, stream=None):
    B, d = kv.batch, kv.head_dim
    qp = _dev(q, "q", kv.dtype, B * num_q_heads * d)
    ip = _dev(idx, "idx", torch.int32, B * num_q_heads * budget)
    sp = _dev(sel_lens, "sel_lens", torch.int32, B)
    need = sd_topk_select_workspace_size(B, num_q_heads, kv.num_kv_heads, max_kv_len)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_topk_select(kv.ref, qp, B, num_q_heads, budget, max_kv_len, ip, sp, wp, wb, _stream(stream)),
           "sd_topk_select")


SD_SPEC_ACCEPT_SCRATCH_BYTES = 4 << 20


def _accept_args(target_logits, draft_logits, draft_tokens, u_accept, u_sample, gamma, vocab, n_accepted,
                 out_tokens):
    B = target_logits.shape[0]
    tp = _dev(target_logits, "target_logits", torch.float32, B * (gamma + 1) * vocab)
    if gamma > 0:
        dp = _dev(draft_logits, "draft_logits", torch.float32, B * gamma * vocab)
        xp = _dev(draft_tokens, "draft_tokens", torch.int32, B * gamma)
        up = _dev(u_accept, "u_accept", torch.float32, B * gamma)
    else:
        dp = xp = up = None
    us = _dev(u_sample, "u_sample", torch.float32, B * (gamma + 1))
    np_ = _dev(n_accepted, "n_accepted", torch.int32, B)
    op = _dev(out_tokens, "out_tokens", torch.int32, B * (gamma + 1))
    return B, tp, dp, xp, up, us, np_, op


def sd_spec_accept_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample, gamma, vocab,
                           temperature, n_accepted, out_tokens, stream=None):
    """sd_spec_accept without a workspace (the library's fixed per-GPU scratch;
    overlapping calls on one GPU race)."""
    B, tp, dp, xp, up, us, np_, op = _accept_args(target_logits, draft_logits, draft_tokens, u_accept,
                                                  u_sample, gamma, vocab, n_accepted, out_tokens)
    _check(lib().sd_spec_accept_noalloc(tp, dp, xp, up, us, B, gamma, vocab, temperature, np_, op,
                                        _stream(stream)), "sd_spec_accept_noalloc")


def sd_spec_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, gamma, vocab,
                   temperature, n_accepted, out_tokens, workspace=None, stream=None):
    B = target_logits.shape[0]
    tp = _dev(target_logits, "target_logits", torch.float32, B * (gamma + 1) * vocab)
    if gamma > 0:
        dp = _dev(draft_logits, "draft_logits", torch.float32, B * gamma * vocab)
        xp = _dev(draft_tokens, "draft_tokens", torch.int32, B * gamma)
        up = _dev(u_accept, "u_accept", torch.float32, B * gamma)
    else:
        dp = xp = up = None
    us = _dev(u_sample, "u_sample", torch.float32, B * (gamma + 1))
    np_ = _dev(n_accepted, "n_accepted", torch.int32, B)
    op = _dev(out_tokens, "out_tokens", torch.int32, B * (gamma + 1))
    need = sd_spec_accept_workspace_size(B, gamma, vocab)
    wp, wb = _ws(workspace, need)
    _check(lib().sd_spec_accept(tp, dp, xp, up, us, B, gamma, vocab, temperature, np_, op, wp, wb,
                                _stream(stream)), "sd_spec_accept")


def sd_hbm_read_probe(buf, nontemporal, checksum, blocks=0, stream=None):
    """Adds the uint32 word sum of `buf` (mod 2^32) to checksum[0]; the caller
    zeroes it. `buf`: any contiguous GPU tensor of a multiple of 16 bytes;
    `blocks`: 256-thread workgroups (0 = as many as are resident)."""
    bp = _dev(buf, "buf")
    cp = _dev(checksum, "checksum", torch.int32, 1)
    _check(lib().sd_hbm_read_probe(bp, buf.numel() * buf.element_size(), int(nontemporal), int(blocks), cp,
                                   _stream(stream)), "sd_hbm_read_probe")


def workspace(nbytes, device="cuda"):
    """A byte buffer for the `workspace` arguments (allocated through torch)."""
    return torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)
