"""Benchmark of the sparse-KV self-speculative decoding hot path on one MI355X.

Workload (Llama-3.1-8B attention shapes, synthetic bf16 inputs resident in
HBM): batch 128, context 32768, 32 query / 8 KV heads, head_dim 128,
gamma = 4; SnapKV draft set with a 32-query observation window, max-pool 7,
budget 2048 per KV head, keys with 10% of positions boosted 4x; acceptance over
Llama-3.1's 128256-token vocabulary with draft logits = target + N(0, 0.5).

One step = one pass of every kernel of the hot path, in call order:
  sd_snapkv_select, sd_streaming_select (64 + 448), gamma x sd_draft_attn_sparse
  (n_q = 1 over the SnapKV set), sd_verify_attn (n_q = gamma + 1), sd_spec_accept.
`value` = draft+verify KV token reads of one round, B (L + gamma K), over
t_verify + gamma t_draft, both from HIP events around those calls inside the
timed steps (MagicDec notes §4.1: a round costs gamma draft steps plus one
verification; the SnapKV set is built once at prefill, Appendix A.1, so its
selection is reported apart, as is acceptance). `step_kv_tokens_per_s` charges
the same tokens to the whole step. Per-call HIP event times, verify GB/s
against the 8 TB/s HBM peak and against the attainable read bandwidth (the
library's streaming-read probe over the 8.6 GB K pool), and the CPU oracle's
rates on bounded samples are reported beside it.
After that, `round` times one whole self-speculative round at the same shape
(draft steps with KV append and sampling, verify, accept, roll back), eager and
replayed from a HIP graph, and dense decode as the attention-only target step;
`per_sequence_budgets` times SnapKV with one budget per sequence and a draft
step on the ragged B=256 batch; `snapkv_two_calls` times SnapKV split into the
window's softmax normalisers and the selection given them (one K pass: the
cost for a caller whose prefill attention returned them); `compact_draft_cache` copies the SnapKV rows out once (sd_kv_compact) and times
the draft as a dense decode over that copy beside the gathered draft;
`dynamic_topk` times a top-K attention draft
step (selection over the whole cache, then the per-head draft);
`speedup_model` evaluates the analytic speedup model (best speculation length
and attention-side speedup per draft kind and budget) on measured times;
`other_workloads` times verify at the Llama-8B 8k, ragged B=256 and Llama-70B
16k shapes, the StreamingLLM-512 draft step and acceptance over the 128256-token
vocabulary, warm and cold (last-level cache evicted before each call).

python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline] [--no-round]
python bench.py --copy-probe     # plain 4 GiB device copy, for counter scaling
python bench.py --configs-only --steps 5   # only the other workloads (profiling)
python bench.py --compact-only --steps 5   # only the compact draft cache block (profiling)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KV_BYTES_PER_TOKEN = 8 * 128 * 2 * 2       # Hkv * d * (K+V) * bf16
METRIC = "verify-attn KV GB/s and % HBM roofline; draft+verify KV tokens/s at B=128 ctx=32k"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-units", type=int, default=0,
                    help="(sequence, kv head) units the oracle runs (0 = 80 units, about 12 s)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--configs-only", action="store_true",
                    help="time only the other workloads (for their kernel traces and counters)")
    ap.add_argument("--compact-only", action="store_true",
                    help="time only the compact draft cache block (for its kernel trace and counters)")
    ap.add_argument("--no-round", action="store_true",
                    help="skip the round and per-sequence-budget measurements")
    return ap.parse_args()


def copy_probe():
    import torch

    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_bytes_each_way": n, "reps": 5, "ms": dt * 1e3,
                      "read_plus_write_GBps": 2 * n / dt / 1e9}))


def measure_attainable(wl, reps=5, launch_sizes=(0, 256, 512, 1024, 2048)):
    """Attainable streaming-read bandwidth: the library's read probe over the
    K pool (8.6 GB, far beyond the 256 MB last-level cache), with and without
    the nontemporal hint, at several launch sizes (256-thread workgroups; 0 =
    the resident count); median of `reps` timed calls after one warm-up per
    size, best size reported."""
    import torch

    sd = wl.sd
    buf = wl.kv_t.k_pages
    nbytes = buf.numel() * buf.element_size()
    c = torch.zeros(1, dtype=torch.int32, device=buf.device)
    out = {"kernel": "hbm_read_probe_kernel", "buffer_bytes": nbytes, "sweep": {}}
    for nt, key in ((1, "nontemporal_GBps"), (0, "plain_GBps")):
        best = 0.0
        for blocks in launch_sizes:
            sd.sd_hbm_read_probe(buf, nt, c, blocks)
            ms = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                sd.sd_hbm_read_probe(buf, nt, c, blocks)
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            ms.sort()
            gbps = nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9
            out["sweep"][f"{'nt' if nt else 'plain'}_blocks_{blocks}"] = gbps
            best = max(best, gbps)
        out[key] = best
    return out


class Workload:
    """Inputs, outputs and workspaces of one step, allocated once."""

    def __init__(self, dev):
        import torch

        import long_context_kv_split_amd as sd
        from synth import WORKLOADS, dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries, workload_lens

        w = WORKLOADS["llama8b-b128-l32k-snapkv"]
        self.w = w
        B, Hq, Hkv, d, g = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.gamma
        self.B, self.Hq, self.Hkv, self.d, self.gamma = B, Hq, Hkv, d, g
        self.n_q = g + 1
        self.V = 128256
        lens = workload_lens(w)
        self.lens = lens
        self.L = max(lens)
        t0 = time.perf_counter()
        self.kv_t = paged_kv(w.seed, lens, Hkv, d, torch.bfloat16, dev, spike_frac=w.spike_frac)
        self.kv = sd.KVCache(self.kv_t.k_pages, self.kv_t.v_pages, self.kv_t.page_table, self.kv_t.kv_lens)
        s = d ** -0.5
        self.q = queries(w.seed, 1, (B, self.n_q, Hq, d), torch.bfloat16, dev, scale=s)
        self.q_obs = queries(w.seed, 4, (B, w.window, Hq, d), torch.bfloat16, dev, scale=s)
        self.q_draft = [queries(w.seed, 100 + i, (B, 1, Hq, d), torch.bfloat16, dev, scale=s)
                        for i in range(g)]
        self.zt = logits(w.seed, 8, (B, g + 1, self.V), 2.0, dev)
        self.zd = logits(w.seed, 9, (B, g, self.V), 0.5, dev, base=self.zt[:, :g]).contiguous()
        self.x = gumbel_tokens(w.seed, self.zd)
        self.ua = dyadic_uniforms(w.seed, 11, (B, g), dev)
        self.us = dyadic_uniforms(w.seed, 12, (B, g + 1), dev)
        torch.cuda.synchronize()
        log(f"generated inputs in {time.perf_counter() - t0:.1f}s")

        i32 = torch.int32
        self.idx = torch.empty((B, Hkv, w.budget), dtype=i32, device=dev)
        self.sel = torch.empty((B,), dtype=i32, device=dev)
        self.s_idx = torch.empty((B, 1, 512), dtype=i32, device=dev)
        self.s_sel = torch.empty((B,), dtype=i32, device=dev)
        self.o_draft = [torch.empty_like(qd) for qd in self.q_draft]
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, self.n_q, Hq), dtype=torch.float32, device=dev)
        self.n_acc = torch.empty((B,), dtype=i32, device=dev)
        self.toks = torch.empty((B, g + 1), dtype=i32, device=dev)
        self.ws_snap = sd.workspace(sd.sd_snapkv_select_workspace_size(B, w.window, Hq, Hkv, self.L), dev)
        self.ws_draft = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, w.budget), dev)
        self.ws_ver = sd.workspace(sd.sd_verify_attn_workspace_size(B, self.n_q, Hq, Hkv, d, self.L), dev)
        self.ws_acc = sd.workspace(sd.sd_spec_accept_workspace_size(B, g, self.V), dev)
        # the draft's compressed cache as a cache of its own: the SnapKV rows
        # copied out once per prefill, then read by dense decodes
        P = self.kv_t.page_size
        self.pps = -(-w.budget // P)
        self.k_c = torch.empty((B * self.pps, Hkv, P, d), dtype=torch.bfloat16, device=dev)
        self.v_c = torch.empty_like(self.k_c)
        self.table_c = torch.arange(B * self.pps, dtype=i32, device=dev).view(B, self.pps)
        self.kvc = sd.KVCache(self.k_c, self.v_c, self.table_c, self.sel)
        self.ws_dense = sd.workspace(sd.sd_verify_attn_workspace_size(B, 1, Hq, Hkv, d, w.budget), dev)
        self.sd = sd

    def step(self, ev=None):
        """One pass of the hot path; with `ev`, records events between calls."""
        sd, w = self.sd, self.w

        def mark(k):
            if ev is not None:
                ev[k].record()

        mark(0)
        sd.sd_snapkv_select(self.kv, self.q_obs, w.window, self.Hq, w.pool_kernel, w.budget, self.L, 1.0,
                            self.idx, self.sel, self.ws_snap)
        sd.sd_streaming_select(self.kv_t.kv_lens, 64, 448, self.s_idx, self.s_sel)
        mark(1)
        for i in range(self.gamma):
            sd.sd_draft_attn_sparse(self.kv, self.q_draft[i], 1, self.Hq, self.idx, self.sel, self.Hkv,
                                    w.budget, 1.0, self.o_draft[i], None, self.ws_draft)
        mark(2)
        sd.sd_verify_attn(self.kv, self.q, self.n_q, self.Hq, self.L, 1.0, self.o, self.lse, self.ws_ver)
        mark(3)
        sd.sd_spec_accept(self.zt, self.zd, self.x, self.ua, self.us, self.gamma, self.V, 1.0, self.n_acc,
                          self.toks, self.ws_acc)
        mark(4)

    # algorithmic work
    def verify_bytes(self):
        kv = sum(self.lens) * KV_BYTES_PER_TOKEN
        qo = 2 * self.B * self.n_q * self.Hq * self.d * 2
        return kv + qo

    def draft_tokens(self):
        return self.gamma * self.B * self.w.budget

    def verify_tokens(self):
        return sum(self.lens)


def measured_traffic():
    """HBM bytes per verify launch from the committed counter runs, or None if
    the verify kernel's source changed since they were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "verify_attn_b128_l32k_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def profiled_verify():
    """The verify call's kernels as the committed kernel trace of this bench
    command measured them (average duration per launch, and the roofline
    fraction of the whole call from their sum), or None if the attention
    sources changed since the trace was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "verify_attn_b128_l32k_kernel_trace.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    call_ms = sum(k["avg_ms"] for k in rec["kernels"])
    return {"kernels": rec["kernels"], "call_ms": call_ms, "command": rec["command"],
            "frac": rec["algorithmic_bytes_per_launch"] / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def unit_cache(kv_t, b, g):
    """One (sequence b, KV head g) of the paged cache copied to the host, with
    its pages in table order and an identity page table."""
    import numpy as np

    L = int(kv_t.lens[b])
    npg = max(1, -(-L // kv_t.page_size))
    pages = kv_t.page_table[b, :npg].long()
    k = kv_t.k_pages[pages][:, g:g + 1].cpu()
    v = kv_t.v_pages[pages][:, g:g + 1].cpu()
    return k, v, np.arange(npg, dtype=np.int64)[None, :], np.array([L])


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wl, n_units, n_select_units=8, n_accept_seqs=16):
    """Time the oracle on bounded samples of the bench workload: verify + gamma
    sparse drafts on (sequence, KV head) units (the metric's unit, KV tokens/s),
    SnapKV selection on a few units and acceptance on a few sequences (each in
    its own unit, beside it). Host copies are made before each clock starts."""
    import numpy as np

    import oracle

    blas_threads = _blas_threads()
    cores = len(os.sched_getaffinity(0))
    G = wl.Hq // wl.Hkv
    units = [((7 * i) % wl.B, (3 * i) % wl.Hkv) for i in range(n_units)]
    prepared = []
    idx = wl.idx.cpu().numpy()
    sel = wl.sel.cpu().numpy()
    for b, g in units:
        k, v, table, lens = unit_cache(wl.kv_t, b, g)
        heads = slice(g * G, (g + 1) * G)
        q = wl.q[b:b + 1, :, heads].cpu()
        qd = [x[b:b + 1, :, heads].cpu() for x in wl.q_draft]
        prepared.append((k, v, table, lens, q, qd, idx[b:b + 1, g:g + 1], sel[b:b + 1]))
    t0 = time.perf_counter()
    toks = 0
    for k, v, table, lens, q, qd, ix, sl in prepared:
        oracle.verify_attn(q, k, v, table, lens, 1.0)
        toks += int(lens[0])
        for x in qd:
            oracle.sparse_attn(x, k, v, table, ix, sl, 1.0)
            toks += int(sl[0])
    dt = time.perf_counter() - t0

    # SnapKV selection (window scores, pooling, top-K) on a few units
    sel_units = [((11 * i + 5) % wl.B, (5 * i + 1) % wl.Hkv) for i in range(n_select_units)]
    sel_prep = []
    for b, g in sel_units:
        k, v, table, lens = unit_cache(wl.kv_t, b, g)
        sel_prep.append((wl.q_obs[b:b + 1, :, g * G:(g + 1) * G].cpu(), k, table, lens))
    w = wl.w
    t1 = time.perf_counter()
    for qo, k, table, lens in sel_prep:
        oracle.snapkv_select(qo, k, table, lens, w.window, w.pool_kernel, w.budget, 1.0)
    dt_sel = time.perf_counter() - t1
    sel_tokens = sum(int(p[3][0]) for p in sel_prep)

    # acceptance on a few sequences of the 128256-token vocabulary
    zt = wl.zt[:n_accept_seqs].cpu()
    zd = wl.zd[:n_accept_seqs].cpu()
    x, ua, us = (t[:n_accept_seqs].cpu() for t in (wl.x, wl.ua, wl.us))
    t2 = time.perf_counter()
    oracle.spec_accept(zt, zd, x, ua, us)
    dt_acc = time.perf_counter() - t2
    acc_bytes = (zt.numel() + zd.numel()) * 4

    # tokens above are per (sequence, KV head) unit; a KV token of the metric
    # spans all KV heads, so divide by Hkv to use the same unit.
    return {"value": toks / wl.Hkv / dt, "unit": "KV tokens/s", "cores": int(min(cores, max(blas_threads, 1))),
            "host_cores_available": cores, "blas_threads": blas_threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{n_units} (sequence, KV head) units of the same workload: fp64 verify over "
                      f"{wl.L} tokens + {wl.gamma} sparse drafts over {wl.w.budget} SnapKV tokens each",
            "per_op": {
                "snapkv_select": {"units": n_select_units, "seconds": round(dt_sel, 2),
                                  "context_tokens_per_s": sel_tokens / dt_sel,
                                  "K_GBps": sel_tokens * wl.d * 2 / dt_sel / 1e9},
                "spec_accept": {"sequences": n_accept_seqs, "vocab": wl.V, "seconds": round(dt_acc, 3),
                                "sequences_per_s": n_accept_seqs / dt_acc,
                                "logits_GBps": acc_bytes / dt_acc / 1e9}}}


def oracle_verify_rate(kv_t, q, G, units):
    """The oracle's verify rate (KV tokens/s over all KV heads, and GB/s) on a
    few (sequence, KV head) units of a workload."""
    import oracle

    prep = []
    for b, g in units:
        k, v, table, lens = unit_cache(kv_t, b, g)
        prep.append((q[b:b + 1, :, g * G:(g + 1) * G].cpu(), k, v, table, lens))
    t0 = time.perf_counter()
    toks = 0
    for qq, k, v, table, lens in prep:
        oracle.verify_attn(qq, k, v, table, lens, 1.0)
        toks += int(lens[0])
    dt = time.perf_counter() - t0
    Hkv = kv_t.k_pages.shape[1]
    d = kv_t.k_pages.shape[3]
    return {"units": len(units), "seconds": round(dt, 3), "kv_tokens_per_s": toks / Hkv / dt,
            "GBps": toks * d * 2 * 2 / dt / 1e9}


def measure_round(wl, reps=10):
    """One self-speculative round at the bench shape, timed eager and replayed
    from a HIP graph. SnapKV selects once at L0 = L - (gamma + 1); the round is
    gamma x [append the token's K/V, advance, draft over selection + tail,
    sample the next draft token], then append, advance, verify (n_q = gamma + 1
    over L), accept, roll back. The appended K/V are the rows the cache already
    holds at L0 .. L - 1, so the cache is the same after every round. Also
    times, back to back, dense decode (n_q = 1 over L) as the attention-only
    target step T_T, verify, the draft and the draft with its tail."""
    import torch

    sd, w = wl.sd, wl.w
    B, g, Hq, Hkv, V = wl.B, wl.gamma, wl.Hq, wl.Hkv, wl.V
    dev = wl.q.device
    i32 = torch.int32
    L0 = wl.L - (g + 1)
    lens0 = torch.full((B,), L0, dtype=i32, device=dev)
    kv_lens = lens0.clone()
    kv = sd.KVCache(wl.kv_t.k_pages, wl.kv_t.v_pages, wl.kv_t.page_table, kv_lens)
    sd.sd_snapkv_select(kv, wl.q_obs, w.window, Hq, w.pool_kernel, w.budget, L0, 1.0, wl.idx, wl.sel,
                        wl.ws_snap)
    tail_begin = lens0.clone()
    pt = wl.kv_t.page_table.long()
    rows = torch.arange(B, device=dev)
    k_new, v_new = [], []
    for i in range(g + 1):
        pos = L0 + i
        pages = pt[rows, pos // 16]
        k_new.append(wl.kv_t.k_pages[pages, :, pos % 16, :].unsqueeze(1).contiguous())
        v_new.append(wl.kv_t.v_pages[pages, :, pos % 16, :].unsqueeze(1).contiguous())
    zd_i = [wl.zd[:, i:i + 1].contiguous() for i in range(g)]
    u_i = [wl.ua[:, i:i + 1].contiguous() for i in range(g)]
    drafted_t = torch.empty((g, B), dtype=i32, device=dev)  # row i: draft token i of every sequence
    drafted = torch.empty((B, g), dtype=i32, device=dev)
    n0 = torch.empty((B,), dtype=i32, device=dev)
    ws_s = sd.workspace(sd.sd_spec_accept_workspace_size(B, 0, V), dev)

    def one_round():
        for i in range(g):
            sd.sd_kv_append(kv, k_new[i], v_new[i], 1)
            sd.sd_kv_advance(kv_lens, None, 1)
            sd.sd_draft_attn_sparse_tail(kv, wl.q_draft[i], 1, Hq, wl.idx, wl.sel, Hkv, w.budget, tail_begin,
                                         g + 1, 1.0, wl.o_draft[i], None, wl.ws_draft)
            sd.sd_spec_accept(zd_i[i], None, None, None, u_i[i], 0, V, 1.0, n0, drafted_t[i], ws_s)
        sd.sd_kv_append(kv, k_new[g], v_new[g], 1)
        sd.sd_kv_advance(kv_lens, None, 1)
        sd.sd_verify_attn(kv, wl.q, g + 1, Hq, wl.L, 1.0, wl.o, wl.lse, wl.ws_ver)
        drafted.copy_(drafted_t.t())
        sd.sd_spec_accept(wl.zt, wl.zd, drafted, wl.ua, wl.us, g, V, 1.0, wl.n_acc, wl.toks, wl.ws_acc)
        sd.sd_kv_advance(kv_lens, wl.n_acc, -g)

    def timed(fn):
        ts = []
        for _ in range(reps):
            kv_lens.copy_(lens0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sum(ts) / len(ts)

    one_round()
    torch.cuda.synchronize()
    eager_ms = timed(one_round)
    graph = torch.cuda.CUDAGraph()
    kv_lens.copy_(lens0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            one_round()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph_ms = timed(graph.replay)
    mean_acc = float(wl.n_acc.float().mean().item())

    # attention-only step times over the full cache (lengths L)
    q1 = wl.q[:, :1].contiguous()
    o1 = torch.empty_like(q1)

    def decode():
        sd.sd_verify_attn(wl.kv, q1, 1, Hq, wl.L, 1.0, o1, None, wl.ws_ver)

    def verify():
        sd.sd_verify_attn(wl.kv, wl.q, g + 1, Hq, wl.L, 1.0, wl.o, wl.lse, wl.ws_ver)

    def draft():
        sd.sd_draft_attn_sparse(wl.kv, wl.q_draft[0], 1, Hq, wl.idx, wl.sel, Hkv, w.budget, 1.0, wl.o_draft[0],
                                None, wl.ws_draft)

    def draft_tail():
        # the selection made at L0 plus the gamma + 1 positions after it
        sd.sd_draft_attn_sparse_tail(wl.kv, wl.q_draft[0], 1, Hq, wl.idx, wl.sel, Hkv, w.budget, tail_begin,
                                     g + 1, 1.0, wl.o_draft[0], None, wl.ws_draft)

    def back_to_back(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_dec, t_ver, t_dr, t_tail = (back_to_back(f) for f in (decode, verify, draft, draft_tail))
    return {"L0": L0, "eager_ms": eager_ms, "graph_ms": graph_ms, "mean_accepted": mean_acc,
            "decode_ms": t_dec, "verify_ms": t_ver, "draft_ms": t_dr, "draft_tail_ms": t_tail,
            "verify_over_decode": t_ver / t_dec, "draft_over_decode": t_dr / t_dec,
            "budget_over_context": w.budget / wl.L}


def measure_snapkv_lse(wl, reps=10):
    """SnapKV in two calls (MagicDec notes, Appendix A.1: the set is built at
    prefill, whose attention of the window queries yields their softmax
    normalisers): sd_snapkv_window_lse (pass 1 alone) and
    sd_snapkv_select_lse (the selection from given normalisers: one K pass).
    The second is what a caller pays whose prefill attention returned the
    window's log-sum-exp."""
    import torch

    sd, w = wl.sd, wl.w
    B, Hq, Hkv, d, W = wl.B, wl.Hq, wl.Hkv, wl.d, w.window
    dev = wl.q.device
    lse = torch.empty((B, W, Hq), dtype=torch.float32, device=dev)
    idx = torch.empty_like(wl.idx)
    sel = torch.empty_like(wl.sel)

    def window_lse():
        sd.sd_snapkv_window_lse(wl.kv, wl.q_obs, W, Hq, wl.L, 1.0, lse, wl.ws_snap)

    def select_lse():
        sd.sd_snapkv_select_lse(wl.kv, wl.q_obs, lse, W, Hq, w.pool_kernel, w.budget, wl.L, 1.0, idx, sel,
                                wl.ws_snap)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_lse, t_sel = timed(window_lse), timed(select_lse)
    idx1 = torch.empty_like(idx)
    sel1 = torch.empty_like(sel)
    sd.sd_snapkv_select(wl.kv, wl.q_obs, W, Hq, w.pool_kernel, w.budget, wl.L, 1.0, idx1, sel1, wl.ws_snap)
    same = int((idx == idx1).all(dim=2).sum().item())
    k_bytes = B * wl.L * Hkv * d * 2
    return {"window_lse_ms": t_lse, "select_given_lse_ms": t_sel,
            "select_given_lse_K_GBps": k_bytes / (t_sel * 1e-3) / 1e9,
            "units_equal_to_one_call": same, "units": B * Hkv}


def measure_compact(wl, reps=10):
    """The draft over a compact copy of the SnapKV rows (sd_kv_compact once
    per prefill, then dense decodes, sd_verify_attn with n_q = 1) beside the
    step's gathered draft over the same selection in the full cache
    (sd_draft_attn_sparse), with how far the two outputs lie apart at this
    shape. The copy pays for itself after copy / (gathered - dense) draft
    steps."""
    import torch

    sd, w = wl.sd, wl.w
    Hq, Hkv, d, K = wl.Hq, wl.Hkv, wl.d, w.budget
    sd.sd_snapkv_select(wl.kv, wl.q_obs, w.window, Hq, w.pool_kernel, K, wl.L, 1.0, wl.idx, wl.sel, wl.ws_snap)
    q1 = wl.q_draft[0]
    o_dense = torch.empty_like(q1)
    o_gather = torch.empty_like(q1)

    def compact():
        sd.sd_kv_compact(wl.kv, wl.idx, wl.sel, Hkv, K, wl.pps, wl.k_c, wl.v_c)

    def dense():
        sd.sd_verify_attn(wl.kvc, q1, 1, Hq, K, 1.0, o_dense, None, wl.ws_dense)

    def gather():
        sd.sd_draft_attn_sparse(wl.kv, q1, 1, Hq, wl.idx, wl.sel, Hkv, K, 1.0, o_gather, None, wl.ws_draft)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_c, t_dense, t_gather = timed(compact), timed(dense), timed(gather)
    rows = int(wl.sel.sum().item()) * Hkv
    diff = float((o_dense.float() - o_gather.float()).abs().max().item())
    return {"compact_once_per_prefill_ms": t_c,
            "compact_GBps": 4 * rows * d * 2 / (t_c * 1e-3) / 1e9,
            "dense_draft_ms": t_dense, "gathered_draft_ms": t_gather,
            "dense_draft_kv_GBps": 2 * rows * d * 2 / (t_dense * 1e-3) / 1e9,
            "dense_over_gathered": t_dense / t_gather,
            "break_even_draft_steps": t_c / (t_gather - t_dense) if t_gather > t_dense else None,
            "max_abs_diff_dense_vs_gathered": diff}


def measure_topk(wl, reps=10):
    """Dynamic top-K attention draft step at the bench shape (MagicDec notes
    §4.4): per query head, the budget positions with the largest q.k over the
    whole cache (sd_topk_select), then the draft over those positions with one
    index set per query head. The selection is paid again at every step."""
    import torch

    sd, w = wl.sd, wl.w
    B, Hq, Hkv, d, K = wl.B, wl.Hq, wl.Hkv, wl.d, w.budget
    dev = wl.q.device
    idx = torch.empty((B, Hq, K), dtype=torch.int32, device=dev)
    sel = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = sd.workspace(sd.sd_topk_select_workspace_size(B, Hq, Hkv, wl.L), dev)
    q = wl.q_draft[0]
    out = wl.o_draft[0]

    def select():
        sd.sd_topk_select(wl.kv, q, Hq, K, wl.L, idx, sel, ws)

    def attn():
        sd.sd_draft_attn_sparse(wl.kv, q, 1, Hq, idx, sel, Hq, K, 1.0, out, None, wl.ws_draft)

    def step():
        select()
        attn()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_sel, t_att, t_step = timed(select), timed(attn), timed(step)
    k_bytes = B * wl.L * Hkv * d * 2                 # every cached K row, read once
    a_bytes = B * Hq * K * 2 * d * 2                 # K and V of each head's own set
    return {"budget": K, "select_ms": t_sel, "attn_ms": t_att, "step_ms": t_step,
            "select_K_GBps": k_bytes / (t_sel * 1e-3) / 1e9, "attn_GBps": a_bytes / (t_att * 1e-3) / 1e9}


def measure_model(wl, rnd, topk, mean_accepted, reps=5, max_gamma=8, budgets=(256, 512, 1024, 2048, 4096)):
    """The analytic speedup model (sd_best_gamma) evaluated on measured
    attention times at the bench shape: T_T = dense decode (n_q = 1 over L),
    T_V(g) = verify with n_q = g + 1, g = 1..max_gamma; SnapKV drafts at
    several budgets K (T_D(K) one draft step, the selection made once at
    prefill and not charged to rounds) and the top-K attention draft (its
    search charged at every draft step). Attention only: the linear layers
    are not part of the path, so these are attention-side speedups."""
    import torch

    sd, w = wl.sd, wl.w
    B, Hq, Hkv, d, L = wl.B, wl.Hq, wl.Hkv, wl.d, wl.L
    dev = wl.q.device
    from synth import queries

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    q_all = queries(w.seed, 21, (B, max_gamma + 1, Hq, d), torch.bfloat16, dev, scale=d ** -0.5)
    ws_v = sd.workspace(sd.sd_verify_attn_workspace_size(B, max_gamma + 1, Hq, Hkv, d, L), dev)
    t_verify = []
    for g in range(1, max_gamma + 1):
        qg = q_all[:, :g + 1].contiguous()
        og = torch.empty_like(qg)
        t_verify.append(timed(lambda: sd.sd_verify_attn(wl.kv, qg, g + 1, Hq, L, 1.0, og, None, ws_v)))
    t_target = rnd["decode_ms"]

    # alpha of the synthetic logits, from the mean accepted count at gamma:
    # E[n] = alpha + ... + alpha^gamma, increasing in alpha (bisection)
    lo, hi = 0.0, 1.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if sd.sd_expected_tokens(wl.gamma, mid) - 1.0 < mean_accepted:
            lo = mid
        else:
            hi = mid
    alphas = {"synthetic": 0.5 * (lo + hi), "0.90": 0.9}

    def best(t_draft, fixed, step):
        return {k: dict(zip(("best_gamma", "speedup"), sd.sd_best_gamma(t_target, t_draft, t_verify, a, fixed, step)))
                for k, a in alphas.items()}

    rows = []
    q1, o1 = wl.q_draft[0], wl.o_draft[0]
    for K in budgets:
        idx = torch.empty((B, Hkv, K), dtype=torch.int32, device=dev)
        sel = torch.empty((B,), dtype=torch.int32, device=dev)
        ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, K), dev)
        t_sel = timed(lambda: sd.sd_snapkv_select(wl.kv, wl.q_obs, w.window, Hq, w.pool_kernel, K, L, 1.0, idx,
                                                 sel, wl.ws_snap))
        t_d = timed(lambda: sd.sd_draft_attn_sparse(wl.kv, q1, 1, Hq, idx, sel, Hkv, K, 1.0, o1, None, ws_d))
        rows.append({"draft": "snapkv", "K": K, "T_D_ms": t_d, "T_select_once_ms": t_sel, **best(t_d, 0.0, 0.0)})
    if topk is not None:
        rows.append({"draft": "topk", "K": topk["budget"], "T_D_ms": topk["attn_ms"],
                     "T_select_step_ms": topk["select_ms"], **best(topk["attn_ms"], 0.0, topk["select_ms"])})
    return {"attention_only": True, "T_T_ms": t_target, "T_V_ms": t_verify, "alpha": alphas, "rows": rows}


def measure_hetero(reps=5):
    """SnapKV with per-sequence budgets on the ragged batch (B=256, contexts
    4096..32768 on shuffled 16-token pages): budget_b = L_b / 16 rounded down
    to 16 (256..2048, the headline's budget/context ratio), observation window
    32, pool 7; then one draft step over the per-sequence sets."""
    import torch

    import long_context_kv_split_amd as sd
    from synth import WORKLOADS, paged_kv, queries, workload_lens

    w = WORKLOADS["ragged-b256-l4k-32k"]
    B, Hq, Hkv, d, W = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, 32
    lens = workload_lens(w)
    kv_t = paged_kv(w.seed, lens, Hkv, d, torch.bfloat16, "cuda", shuffle=True, spike_frac=0.1)
    kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
    budgets = [max(256, min(2048, L // 16 // 16 * 16)) for L in lens]
    Kmax, L = max(budgets), max(lens)
    bud = torch.tensor(budgets, dtype=torch.int32, device="cuda")
    q_obs = queries(w.seed, 4, (B, W, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    q = queries(w.seed, 1, (B, 1, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
    idx = torch.empty((B, Hkv, Kmax), dtype=torch.int32, device="cuda")
    sel = torch.empty((B,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws_s = sd.workspace(sd.sd_snapkv_select_workspace_size(B, W, Hq, Hkv, L))
    ws_d = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, Kmax))

    def select():
        sd.sd_snapkv_select_budgets(kv, q_obs, W, Hq, 7, bud, Kmax, L, 1.0, idx, sel, ws_s)

    def draft():
        sd.sd_draft_attn_sparse(kv, q, 1, Hq, idx, sel, Hkv, Kmax, 1.0, out, None, ws_d)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_sel = timed(select)
    t_dr = timed(draft)
    k_bytes = sum(lens) * Hkv * d * 2          # K of every token, read by each scoring pass
    d_bytes = sum(budgets) * KV_BYTES_PER_TOKEN
    return {"workload": w.name, "budgets": "L_b/16 rounded down to 16, clamped to [256, 2048]",
            "sum_context": sum(lens), "sum_budget": sum(budgets), "select_ms": t_sel,
            "select_K_GBps": 2 * k_bytes / (t_sel * 1e-3) / 1e9, "draft_ms": t_dr,
            "draft_GBps": d_bytes / (t_dr * 1e-3) / 1e9}


def measure_configs(reps=10, oracle_units=0):
    """The other workloads' timed ops, beside the headline: verify at every
    shape, the StreamingLLM-512 draft step at the Llama-8B 8k and ragged
    shapes, acceptance over the 128256-token vocabulary at the Llama-70B
    shape. Each op is timed warm (back to back, mean of `reps`) and cold
    (median of `reps` single calls, each after writing a 1 GiB buffer that
    evicts the 256 MB last-level cache and L2); GB/s are on algorithmic bytes
    (K/V rows read, logits read). With oracle_units > 0 the oracle's verify
    rate on that many (sequence, KV head) units is reported per workload."""
    import torch

    import long_context_kv_split_amd as sd
    from synth import WORKLOADS, dyadic_uniforms, gumbel_tokens, logits, paged_kv, queries, workload_lens

    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def warm(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def cold(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return ts[len(ts) // 2]

    def timing(fn, nbytes):
        w_ms, c_ms = warm(fn), cold(fn)
        return {"warm_ms": w_ms, "cold_ms": c_ms, "bytes": nbytes,
                "warm_GBps": nbytes / (w_ms * 1e-3) / 1e9, "cold_GBps": nbytes / (c_ms * 1e-3) / 1e9}

    out = {}
    for name in ("llama8b-b32-l8k", "ragged-b256-l4k-32k", "llama70b-b64-l16k"):
        w = WORKLOADS[name]
        B, Hq, Hkv, d, n_q = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.gamma + 1
        lens = workload_lens(w)
        L = max(lens)
        kv_t = paged_kv(w.seed, lens, Hkv, d, torch.bfloat16, "cuda", shuffle=w.shuffle)
        kv = sd.KVCache(kv_t.k_pages, kv_t.v_pages, kv_t.page_table, kv_t.kv_lens)
        q = queries(w.seed, 1, (B, n_q, Hq, d), torch.bfloat16, "cuda", scale=d ** -0.5)
        o = torch.empty_like(q)
        ws = sd.workspace(sd.sd_verify_attn_workspace_size(B, n_q, Hq, Hkv, d, L))
        kv_bytes = sum(lens) * Hkv * d * 2 * 2
        rec = {"batch": B, "q_heads": Hq, "kv_heads": Hkv, "n_q": n_q, "sum_context": sum(lens),
               "pages": "shuffled" if w.shuffle else "in order",
               "verify": timing(lambda: sd.sd_verify_attn(kv, q, n_q, Hq, L, 1.0, o, None, ws), kv_bytes)}
        if oracle_units:
            G = Hq // Hkv
            units = [((13 * i + 3) % B, (5 * i + 2) % Hkv) for i in range(oracle_units)]
            rec["verify"]["oracle"] = oracle_verify_rate(kv_t, q, G, units)
        if w.draft == "streaming" and w.sink + w.recent > 0:
            cap = w.sink + w.recent
            idx = torch.empty((B, 1, cap), dtype=torch.int32, device="cuda")
            sel = torch.empty((B,), dtype=torch.int32, device="cuda")
            sd.sd_streaming_select(kv_t.kv_lens, w.sink, w.recent, idx, sel)
            qd = q[:, :1].contiguous()
            od = torch.empty_like(qd)
            wsd = sd.workspace(sd.sd_draft_attn_sparse_workspace_size(B, 1, Hq, Hkv, d, cap))
            d_bytes = sum(min(x, cap) for x in lens) * Hkv * d * 2 * 2
            rec["draft"] = timing(lambda: sd.sd_draft_attn_sparse(kv, qd, 1, Hq, idx, sel, 1, cap, 1.0, od,
                                                                  None, wsd), d_bytes)
            rec["draft"]["set"] = f"StreamingLLM {w.sink} sink + {w.recent} recent"
        if w.vocab:
            g, V = w.gamma, w.vocab
            zt = logits(w.seed, 8, (B, g + 1, V), w.target_std, "cuda")
            zd = logits(w.seed, 9, (B, g, V), w.draft_noise_std, "cuda", base=zt[:, :g]).contiguous()
            x = gumbel_tokens(w.seed, zd)
            ua = dyadic_uniforms(w.seed, 11, (B, g), "cuda")
            us = dyadic_uniforms(w.seed, 12, (B, g + 1), "cuda")
            n_acc = torch.empty((B,), dtype=torch.int32, device="cuda")
            toks = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
            wsa = sd.workspace(sd.sd_spec_accept_workspace_size(B, g, V))
            rec["accept"] = timing(lambda: sd.sd_spec_accept(zt, zd, x, ua, us, g, V, 1.0, n_acc, toks, wsa),
                                   (zt.numel() + zd.numel()) * 4)
            rec["accept"]["vocab"] = V
            rec["accept"]["mean_accepted"] = float(n_acc.float().mean().item())
        out[name] = rec
        log(f"{name}: verify {rec['verify']['warm_ms']:.3f} ms warm / {rec['verify']['cold_ms']:.3f} cold "
            f"({rec['verify']['cold_GBps']:.0f} GB/s cold)"
            + (f", draft {rec['draft']['cold_ms'] * 1e3:.1f} us cold" if "draft" in rec else "")
            + (f", accept {rec['accept']['cold_ms'] * 1e3:.1f} us cold" if "accept" in rec else ""))
        del kv_t, kv, q, o, ws
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (got --gpus {args.gpus}); "
              "the multi-GPU sharding is a design, not implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe()
        return
    if args.compact_only:
        from __graft_entry__ import _ensure_built

        _ensure_built()
        torch.cuda.set_device(0)
        wl = Workload("cuda:0")
        print(json.dumps({"compact_draft_cache": measure_compact(wl, reps=args.steps)}), flush=True)
        return
    if args.configs_only:
        from __graft_entry__ import _ensure_built

        _ensure_built()
        torch.cuda.set_device(0)
        print(json.dumps({"other_workloads": measure_configs(reps=args.steps)}), flush=True)
        return
    from __graft_entry__ import _ensure_built

    _ensure_built()
    torch.cuda.set_device(0)
    dev = "cuda:0"
    wl = Workload(dev)

    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    # timed region: K steps, with per-call events on the stream the library uses
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(K):
        wl.step(evs[s])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    parts = {"select_ms": [], "draft_ms": [], "verify_ms": [], "accept_ms": []}
    for e in evs:
        parts["select_ms"].append(e[0].elapsed_time(e[1]))
        parts["draft_ms"].append(e[1].elapsed_time(e[2]) / wl.gamma)
        parts["verify_ms"].append(e[2].elapsed_time(e[3]))
        parts["accept_ms"].append(e[3].elapsed_time(e[4]))
    avg = {k: sum(v) / len(v) for k, v in parts.items()}
    log(f"timed {K} steps: {ms_step:.3f} ms/step (host wall {wall * 1e3 / K:.3f} ms/step); " +
        ", ".join(f"{k}={v:.3f}" for k, v in avg.items()))

    v_bytes = wl.verify_bytes()
    v_gbps = v_bytes / (avg["verify_ms"] * 1e-3) / 1e9
    step_tokens = wl.verify_tokens() + wl.draft_tokens()
    round_ms = avg["verify_ms"] + wl.gamma * avg["draft_ms"]
    value = step_tokens / (round_ms * 1e-3)
    draft_gbps = wl.B * wl.w.budget * KV_BYTES_PER_TOKEN / (avg["draft_ms"] * 1e-3) / 1e9
    # SnapKV reads every cached key twice (statistics pass, votes pass); acceptance
    # reads the target and draft logits once
    snap_gbps = 2 * sum(wl.lens) * wl.Hkv * wl.d * 2 / (avg["select_ms"] * 1e-3) / 1e9
    acc_gbps = (2 * wl.gamma + 1) * wl.B * wl.V * 4 / (avg["accept_ms"] * 1e-3) / 1e9

    att = measure_attainable(wl)
    log(f"attainable read bandwidth: {att['nontemporal_GBps']:.0f} GB/s nontemporal, "
        f"{att['plain_GBps']:.0f} GB/s plain")

    cpu = None
    if not args.no_cpu_baseline:
        n_units = args.cpu_sample_units or 80
        log(f"cpu baseline: oracle on {n_units} units ...")
        cpu = cpu_baseline(wl, n_units)
        log(f"cpu baseline {cpu['value']:.3e} KV tokens/s in {cpu['seconds']} s; select "
            f"{cpu['per_op']['snapkv_select']['seconds']} s, accept {cpu['per_op']['spec_accept']['seconds']} s")

    rnd = None
    if not args.no_round:
        rnd = measure_round(wl)
        log(f"round: eager {rnd['eager_ms']:.3f} ms, graph {rnd['graph_ms']:.3f} ms, "
            f"verify/decode {rnd['verify_over_decode']:.3f}, draft/decode {rnd['draft_over_decode']:.3f}")

    topk = None
    if not args.no_round:
        topk = measure_topk(wl)
        topk["step_over_static_draft"] = topk["step_ms"] / avg["draft_ms"]
        if rnd is not None:
            topk["step_over_decode"] = topk["step_ms"] / rnd["decode_ms"]
        log(f"top-K draft step: select {topk['select_ms']:.3f} ms + attention {topk['attn_ms']:.3f} ms "
            f"= {topk['step_ms']:.3f} ms ({topk['step_over_static_draft']:.1f}x the SnapKV draft step)")

    snap2 = None
    if not args.no_round:
        snap2 = measure_snapkv_lse(wl)
        log(f"snapkv in two calls: window lse {snap2['window_lse_ms']:.3f} ms, selection given it "
            f"{snap2['select_given_lse_ms']:.3f} ms ({snap2['units_equal_to_one_call']} of {snap2['units']} "
            f"units as the one-call selection)")

    compact = None
    if not args.no_round:
        compact = measure_compact(wl)
        log(f"compact draft cache: copy {compact['compact_once_per_prefill_ms']:.3f} ms once, dense draft "
            f"{compact['dense_draft_ms']:.3f} ms vs gathered {compact['gathered_draft_ms']:.3f} ms "
            f"(outputs within {compact['max_abs_diff_dense_vs_gathered']:.1e})")

    model = None
    if not args.no_round:
        model = measure_model(wl, rnd, topk, float(wl.n_acc.float().mean().item()))
        for r in model["rows"]:
            log(f"model {r['draft']} K={r['K']}: T_D {r['T_D_ms']:.3f} ms, best gamma / speedup "
                + ", ".join(f"alpha {k}: {v['best_gamma']} / {v['speedup']:.2f}" for k, v in r.items()
                            if isinstance(v, dict)))

    het = None
    if not args.no_round:
        het = measure_hetero()
        log(f"per-sequence budgets: select {het['select_ms']:.3f} ms, draft {het['draft_ms']:.3f} ms")

    cfgs = None
    if not args.no_round:
        cfgs = measure_configs(oracle_units=0 if args.no_cpu_baseline else 4)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.w.name, "batch": wl.B, "context": wl.L, "gamma": wl.gamma,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d, "page_size": 16,
                   "draft": f"snapkv window={wl.w.window} pool={wl.w.pool_kernel} budget={wl.w.budget}",
                   "accept_vocab": wl.V, "parallelism": "single-gpu"},
        "value_definition": "B (L + gamma K) / (t_verify + gamma t_draft), per-call HIP events inside the "
                            "timed steps; SnapKV selection (once per prefill) and acceptance reported apart",
        "roofline": {"bound": "hbm", "kernel": "sd_verify_attn (split + combine)",
                     "achieved": v_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": v_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "attainable": att["nontemporal_GBps"],
                     "frac_attainable": v_gbps / att["nontemporal_GBps"],
                     "algorithmic_bytes_per_launch": v_bytes,
                     "avg_launch_ms": avg["verify_ms"],
                     "kernel_trace": profiled_verify()},
        "verify_kv_GBps": v_gbps,
        "verify_pct_hbm_peak": 100.0 * v_gbps / HBM_PEAK_GBPS,
        "round_kv_tokens_per_s": value,
        "round_ms": round_ms,
        "step_kv_tokens_per_s": step_tokens / (ms_step * 1e-3),
        "snapkv_select_once_per_prefill_ms": avg["select_ms"],
        "draft_kv_GBps": draft_gbps,
        "snapkv_select_K_GBps": snap_gbps,
        "accept_logits_GBps": acc_gbps,
        "attainable_read": att,
        "per_call_ms": avg,
        "mean_accepted": float(wl.n_acc.float().mean().item()),
        "cpu_baseline": cpu,
        "round": rnd,
        "per_sequence_budgets": het,
        "snapkv_two_calls": snap2,
        "compact_draft_cache": compact,
        "dynamic_topk": topk,
        "speedup_model": model,
        "other_workloads": cfgs,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
