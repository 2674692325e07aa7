"""Benchmark of the DSA hot path on one MI355X.

A step is one pass of the whole path (indexer scores -> top-k -> sparse MLA
attention) over one batch of synthetic input already resident in HBM, issued as
one dsa_forward call.  The headline workload is decode at 32K context, batch 32
(one new token per sequence); 4 independent input sets are rotated so the 256 MB
MALL cannot serve a step from the previous one.  The same line carries the other
workloads of the metric: decode at 128K context (batch 8) and the 128K prefill
(16 chunks of 8192 rows through dsa_forward), each with its own roofline object.

Prints one JSON line.  Per-call kernel times come from a second pass that issues
the path as its three C-ABI calls with HIP events recorded around each, on the
stream the library launches on; graph replays of the dsa_forward call are timed
beside the eager calls.

    python bench.py [--steps K] [--warmup W] [--workload decode32k] [--extra]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA decode tokens/s @32K ctx; 128K prefill tokens/s; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0

# Algorithmic work per unit (documented in the design doc):
IDX_BYTES_PER_PAIR = 132          # fp8 key (128 B) + fp32 scale per (row, candidate key)
IDX_FLOP_PER_PAIR = 2 * 64 * 128  # 64 heads x 128-wide fp8 dot per (row, key)
TOPK_BYTES_PER_PAIR = 4           # one fp32 score read per (row, candidate)
ATTN_BYTES_PER_ENTRY = 1152       # one gathered 576-wide bf16 latent row per (row, selected)
ATTN_BYTES_PER_ROW = 128 * 576 * 2 + 128 * 512 * 2  # q in + out
ATTN_FLOP_PER_ENTRY = 2 * 128 * (576 + 512)
PROJ_COLS = 64 * 128 + 128 + 576 + 64   # projection outputs per token (q heads, k, latent, w)
PROJ_OUT_BYTES = 64 * 128 + 64 * 4 + 64 * 4 + 128 + 4 + 576 * 2  # stored per token


# Kernel sources whose digest ties a committed HBM-traffic measurement to the code
# that is built now (a stale measurement is reported as null).
_CALL_SOURCES = {"indexer": ["sparse_attention_fp8_amd/csrc/indexer.hip"],
                 "topk": ["sparse_attention_fp8_amd/csrc/topk.hip"],
                 "attention": ["sparse_attention_fp8_amd/csrc/attention.hip"]}
_COMMON_SOURCES = ["sparse_attention_fp8_amd/csrc/dsa_device.h",
                   "sparse_attention_fp8_amd/csrc/dsa_internal.h", "sparse_attention_fp8_amd/build.py"]


def _sources_digest(call):
    import hashlib

    h = hashlib.sha256()
    for f in _CALL_SOURCES[call] + _COMMON_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, call):
    """HBM bytes per launch of one C-ABI call from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (copy-kernel calibrated), or None when there is none for this
    workload or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    a, b = text.find("```json"), text.rfind("```")
    try:
        entry = json.loads(text[a + 7:b])["calls"][call]
    except (ValueError, KeyError):
        return None
    if entry.get("sources_sha256_16") != _sources_digest(call):
        return None
    return entry["traffic_bytes"], entry["kernels"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode32k")
    p.add_argument("--sets", type=int, default=4)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--headline-only", action="store_true",
                   help="time only the headline step, so that a profiler run sees its kernels "
                        "alone (no graph, paged, long-context, training, projection or MHA "
                        "sections)")
    p.add_argument("--extra", action="store_true",
                   help="also time the 8K prefill")
    p.add_argument("--mha-only", action="store_true",
                   help="only time the masked MHA mode beside the MQA mode (short prefill and "
                        "8K), so that a profiler run sees those kernels alone")
    p.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                   help="only run an fp32 elementwise copy (x * 1) that reads and writes MIB MiB, "
                        "five times: the reference kernel of known traffic that scales the "
                        "FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def _pairs(cfg):
    """(row, candidate key) pairs and (row, selected entry) pairs of one step."""
    seq, pos = cfg.row_seq_pos()
    cand = int((pos.astype("int64") + 1).sum())
    sel = int(sum(min(cfg.topk, int(t) + 1) for t in pos))
    return cand, sel


class Workload:
    """One input set of a workload in device memory and the buffers of its calls.

    run() issues the path as three C-ABI calls per chunk of rows (indexer, top-k,
    attention), optionally bracketing each with HIP events on the library's
    stream; run_forward() issues the same work as one dsa_forward call."""

    def __init__(self, dsa, di, cfg, set_id):
        import torch

        self.cfg = cfg
        self.dsa = dsa
        self.inp = di.make_inputs(cfg, set_id, device="cuda")
        R = cfg.num_rows
        CH = cfg.chunk_rows if 0 < cfg.chunk_rows < R else R
        self.chunk = CH if CH < R else 0
        self.chunks = [(a, min(R, a + CH)) for a in range(0, R, CH)]
        i = self.inp
        self.rows = dsa.rows_struct(i.row_seq, i.row_pos, cfg.num_seqs, cfg.max_ctx, cfg.kv_len - 1)
        self.sub = [dsa.rows_struct(i.row_seq[a:b], i.row_pos[a:b], cfg.num_seqs, cfg.max_ctx,
                                    cfg.kv_len - 1) for a, b in self.chunks]
        self.dims = dsa.Dims.from_config(cfg)
        self.ld = (cfg.kv_len + 63) // 64 * 64
        self.scores = torch.empty(CH, self.ld, dtype=torch.float32, device="cuda")
        self.idx = torch.empty(CH, cfg.topk, dtype=torch.int32, device="cuda")
        self.out = torch.empty(R, cfg.n_heads, cfg.v_dim, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(R, cfg.n_heads, dtype=torch.float32, device="cuda")
        need = max(dsa.sparse_mla_attn_workspace_size(rs, self.dims) for rs in self.sub)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        need = max(dsa.topk_workspace_size(rs, cfg.topk) for rs in self.sub)
        self.tws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.fws = torch.empty(max(dsa.forward_workspace_size(self.rows, self.dims, self.chunk), 1),
                               dtype=torch.uint8, device="cuda")
        self.graph = None

    def make_paged(self, P=64, seed=0):
        """Page pools holding this set's caches, pages scattered in a seeded order."""
        import numpy as np
        import torch

        c, i = self.cfg, self.inp
        B, N = c.num_seqs, c.max_ctx
        pps = N // P
        npg = B * pps
        perm = torch.from_numpy(np.random.default_rng(seed).permutation(npg)).cuda()
        self.table = perm.view(B, pps).to(torch.int32).contiguous()
        self.k_pool = torch.empty(npg, P, c.idx_dim, dtype=torch.uint8, device="cuda")
        self.ks_pool = torch.empty(npg, P, dtype=torch.float32, device="cuda")
        self.lat_pool = torch.empty(npg, P, c.qk_dim, dtype=torch.bfloat16, device="cuda")
        self.k_pool[perm] = i.k_idx.view(npg, P, c.idx_dim)
        self.ks_pool[perm] = i.k_scale.view(npg, P)
        self.lat_pool[perm] = i.latent.view(npg, P, c.qk_dim)
        self.pages = self.dsa.pages_struct(self.table, P, npg)

    def run_paged(self):
        d, i = self.dsa, self.inp
        d.indexer_scores_paged(self.rows, self.dims, self.pages, i.q_idx, i.q_scale, i.w,
                               self.k_pool, self.ks_pool, scores=self.scores)
        d.topk(self.rows, self.cfg.topk, self.scores, indices=self.idx, workspace=self.tws)
        d.sparse_mla_attn_paged(self.rows, self.dims, self.pages, i.q, self.lat_pool, self.idx,
                                self.cfg.scale, out=self.out, lse=self.lse, workspace=self.ws)

    def run(self, ev=None):
        """The three calls per chunk; ev, if given, is a list that receives one
        (call, start event, end event) triple per call."""
        import torch

        d, i, c = self.dsa, self.inp, self.cfg

        def mark(name, fn):
            if ev is None:
                fn()
                return
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev.append((name, e0, e1))

        for rs, (a, b) in zip(self.sub, self.chunks):
            n = b - a
            sc, ix = self.scores[:n], self.idx[:n]
            mark("indexer", lambda: d.indexer_scores(rs, self.dims, i.q_idx[a:b], i.q_scale[a:b],
                                                     i.w[a:b], i.k_idx, i.k_scale, scores=sc))
            mark("topk", lambda: d.topk(rs, c.topk, sc, indices=ix, workspace=self.tws))
            mark("attention", lambda: d.sparse_mla_attn(rs, self.dims, i.q[a:b], i.latent, ix,
                                                        c.scale, out=self.out[a:b],
                                                        lse=self.lse[a:b], workspace=self.ws))

    def run_forward(self):
        i = self.inp
        self.dsa.forward(self.rows, self.dims, i.q_idx, i.q_scale, i.w, i.k_idx, i.k_scale, i.q,
                         i.latent, self.cfg.scale, out=self.out, lse=self.lse,
                         chunk_rows=self.chunk, workspace=self.fws)

    def capture(self):
        """A HIP graph of one dsa_forward call (its kernels only: the library records
        no memset or copy), checked bit for bit against the eager call."""
        import torch

        self.run_forward()
        torch.cuda.synchronize()
        ref = self.out.clone()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run_forward()
        torch.cuda.synchronize()
        self.out.zero_()
        for _ in range(2):
            self.graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(self.out, ref):
                raise RuntimeError("graph replay differs from the eager dsa_forward call")


def time_bare(fn_list, K, W):
    """Wall time per step of K steps (fn_list rotated), after W warm-up steps, with a
    device synchronisation on each side of the timed region."""
    import torch

    for i in range(W):
        fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / K * 1e3


def step_percentiles(fn_list, K):
    """Per-step durations from HIP events recorded between K back-to-back steps (fn_list
    rotated): p10, median and p90 in ms."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(K):
        fn_list[i % len(fn_list)]()
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(K))
    pick = lambda q: d[min(K - 1, int(q * (K - 1) + 0.5))]
    return {"p10": pick(0.1), "median": pick(0.5), "p90": pick(0.9), "steps": K}


def time_calls(sets, K):
    """Per-call event durations (ms per step, summed over a step's chunks) over K
    steps with the sets rotated."""
    import torch

    evs = []
    for i in range(K):
        ev = []
        sets[i % len(sets)].run(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    tot = {}
    for ev in evs:
        for name, e0, e1 in ev:
            tot[name] = tot.get(name, 0.0) + e0.elapsed_time(e1)
    return {k: v / K for k, v in tot.items()}


def kernel_table(cfg, k_ms):
    """Per-call rates against each call's own bound from its algorithmic work."""
    cand, sel = _pairs(cfg)
    R = cfg.num_rows
    idx_b, idx_f = cand * IDX_BYTES_PER_PAIR, cand * IDX_FLOP_PER_PAIR
    topk_b = cand * TOPK_BYTES_PER_PAIR
    att_b, att_f = sel * ATTN_BYTES_PER_ENTRY + R * ATTN_BYTES_PER_ROW, sel * ATTN_FLOP_PER_ENTRY
    t = {"indexer": {"ms": k_ms["indexer"], "bytes": idx_b, "flop": idx_f},
         "topk": {"ms": k_ms["topk"], "bytes": topk_b},
         "attention": {"ms": k_ms["attention"], "bytes": att_b, "flop": att_f}}
    for v in t.values():
        v["gbs"] = v["bytes"] / v["ms"] / 1e6
        if "flop" in v:
            v["tflops"] = v["flop"] / v["ms"] / 1e9
    t["indexer"]["fp8_frac"] = t["indexer"]["tflops"] / FP8_PEAK_TFLOPS
    t["attention"]["bf16_frac"] = t["attention"]["tflops"] / BF16_PEAK_TFLOPS
    return t


def roofline_of(kernels, decode: bool):
    """The roofline object of the dominant call: HBM-bound at decode (algorithmic
    bytes over event time), MFMA-bound at prefill (fp8 peak for the indexer, bf16
    for attention)."""
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    if decode or dom == "topk":
        return {"bound": "hbm", "kernel": dom, "achieved": kd["gbs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kd["gbs"] / HBM_PEAK_GBS,
                "algorithmic_bytes": kd["bytes"], "launch_ms": kd["ms"]}
    peak = FP8_PEAK_TFLOPS if dom == "indexer" else BF16_PEAK_TFLOPS
    return {"bound": "mfma", "kernel": dom, "achieved": kd["tflops"], "peak": peak,
            "unit": "TFLOP/s", "frac": kd["tflops"] / peak, "algorithmic_flop": kd["flop"],
            "launch_ms": kd["ms"]}


def time_decode(dsa, di, cfg, sets, K, W, graphs=True):
    """A decode workload: bare dsa_forward steps (the throughput), HIP-graph replays
    of the same call, and per-call event times."""
    import torch

    print(f"[bench] {cfg.name}: generating {sets} input sets", file=sys.stderr, flush=True)
    ws = [Workload(dsa, di, cfg, s) for s in range(sets)]
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing", file=sys.stderr, flush=True)
    ms = time_bare([w.run_forward for w in ws], K, W)
    calls_ms = time_bare([w.run for w in ws], K, W)
    k_ms = time_calls(ws, K)
    res = {"ms_per_step": ms, "tokens_per_s": cfg.num_rows / (ms * 1e-3),
           "ms_per_step_three_calls": calls_ms,
           # the step's spread (events between steps, input sets rotated: MALL-cold) and
           # the same step repeated on one input set (MALL-warm)
           "step_ms_events": step_percentiles([w.run_forward for w in ws], K),
           "ms_per_step_warm": time_bare([ws[0].run_forward], K, W)}
    if graphs:
        try:
            for w in ws:
                w.capture()
            gms = time_bare([w.graph.replay for w in ws], K, W)
            res["graph"] = {"ms_per_step": gms, "tokens_per_s": cfg.num_rows / (gms * 1e-3)}
        except Exception as e:  # capture unsupported: report and go on
            res["graph"] = {"error": str(e)[:200]}
    cand, sel = _pairs(cfg)
    step_bytes = cand * IDX_BYTES_PER_PAIR + sel * ATTN_BYTES_PER_ENTRY + \
        cfg.num_rows * ATTN_BYTES_PER_ROW
    res["step_hbm_frac"] = step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    res["kernels"] = kernel_table(cfg, k_ms)
    res["roofline"] = roofline_of(res["kernels"], decode=True)
    return res, ws


def time_prefill(dsa, di, cfg, reps):
    """A chunked prefill workload through dsa_forward (tokens/s), per-call event times
    of the same chunks issued as separate calls, and time-weighted MFMA fractions."""
    import torch

    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    w = Workload(dsa, di, cfg, 0)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing", file=sys.stderr, flush=True)
    ms = time_bare([w.run_forward], reps, 1)
    k_ms = time_calls([w], 1)
    cand, sel = _pairs(cfg)
    fp8_tf = cand * IDX_FLOP_PER_PAIR / 1e12
    bf16_tf = sel * ATTN_FLOP_PER_ENTRY / 1e12
    s = ms * 1e-3
    kern = kernel_table(cfg, k_ms)
    res = {"tokens_per_s": cfg.num_rows / s, "ms": ms, "rows": cfg.num_rows, "reps": reps,
           "chunk_rows": w.chunk or cfg.num_rows, "fp8_tflop": fp8_tf, "bf16_tflop": bf16_tf,
           # time-weighted MFMA fraction: ideal time at both peaks over measured time
           "mfma_frac": (fp8_tf / FP8_PEAK_TFLOPS + bf16_tf / BF16_PEAK_TFLOPS) / s,
           "kernels": kern, "roofline": roofline_of(kern, decode=False)}
    del w
    torch.cuda.empty_cache()
    return res


def time_projection(dsa, di, pcfg, reps, sets=3):
    """dsa_project_append on one projection workload: HIP events around each call on
    the library's stream; weight sets rotate so the MALL cannot hold them."""
    import torch

    print(f"[bench] projections {pcfg.name}", file=sys.stderr, flush=True)
    R, d = pcfg.num_tokens, pcfg.d_model
    gens = [di.ProjGenerator(pcfg.cfg_id, d, s) for s in range(sets)]
    W = [g.weights(device="cuda") for g in gens]
    h = gens[0].h(0, R, device="cuda")
    dev = torch.device("cuda")
    k_idx = torch.zeros(pcfg.num_seqs, pcfg.max_ctx, 128, dtype=torch.uint8, device=dev)
    k_scale = torch.zeros(pcfg.num_seqs, pcfg.max_ctx, dtype=torch.float32, device=dev)
    latent = torch.zeros(pcfg.num_seqs, pcfg.max_ctx, 576, dtype=torch.bfloat16, device=dev)
    seq, pos = pcfg.row_seq_pos()
    rows = dsa.rows_struct(torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev),
                           pcfg.num_seqs, pcfg.max_ctx, pcfg.max_ctx - 1)
    q_idx = torch.empty(R, 64, 128, dtype=torch.uint8, device=dev)
    q_scale = torch.empty(R, 64, dtype=torch.float32, device=dev)
    w = torch.empty(R, 64, dtype=torch.float32, device=dev)
    ws = torch.empty(max(dsa.project_append_workspace_size(rows, d), 1), dtype=torch.uint8,
                     device=dev)
    run = lambda i: dsa.project_append(rows, h, *W[i % sets], k_idx, k_scale, latent, q_idx,
                                       q_scale, w, workspace=ws)
    for i in range(2 * sets):
        run(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        run(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[reps]) / reps
    s = ms * 1e-3
    bytes_ = PROJ_COLS * d * 2 + R * d * 2 + R * PROJ_OUT_BYTES
    flop = 2.0 * R * d * PROJ_COLS
    res = {"ms": ms, "tokens": R, "d_model": d, "reps": reps, "weight_sets": sets,
           "algorithmic_bytes": bytes_, "flop": flop, "gbs": bytes_ / s / 1e9,
           "tflops": flop / s / 1e12}
    if flop / bytes_ > BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        res["roofline"] = {"bound": "mfma", "achieved": res["tflops"], "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": res["tflops"] / BF16_PEAK_TFLOPS}
    else:
        res["roofline"] = {"bound": "hbm", "achieved": res["gbs"], "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": res["gbs"] / HBM_PEAK_GBS}
    del W, h, k_idx, k_scale, latent, ws
    torch.cuda.empty_cache()
    return res


def time_training(dsa, st, K):
    """The sparse-stage indexer loss (target, KL, dI) and its backward on one input
    set of the headline workload, each timed with HIP events over K calls."""
    import torch

    c = st.cfg
    R = c.num_rows
    st.run()  # scores, selection, attention lse of this set
    loss = torch.empty(R, dtype=torch.float32, device="cuda")
    dsc = torch.empty(R, c.topk, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dsa.indexer_loss_workspace_size(st.rows), 1), dtype=torch.uint8,
                     device="cuda")
    dq = torch.zeros(R, c.n_idx_heads, c.idx_dim, dtype=torch.float32, device="cuda")
    dw = torch.zeros(R, c.n_idx_heads, dtype=torch.float32, device="cuda")
    dk = torch.zeros(c.num_seqs, c.max_ctx, c.idx_dim, dtype=torch.float32, device="cuda")
    i = st.inp
    fwd = lambda: dsa.indexer_loss(st.rows, i.q, i.latent, st.idx, st.lse, c.scale, st.scores,
                                   loss=loss, dscores=dsc, workspace=ws)
    # one row per sequence: no key is selected twice, so the smallest backward
    # workspace (no fixed-point accumulators) gives the deterministic result
    ws_b = torch.empty(dsa.indexer_backward_workspace_size(st.rows, shared_keys=0),
                       dtype=torch.uint8, device="cuda")
    bwd = lambda: dsa.indexer_backward(st.rows, i.q_idx, i.q_scale, i.w, i.k_idx, i.k_scale,
                                       st.idx, dsc, dq, dw, dk, workspace=ws_b)
    dsc_d = torch.empty_like(st.scores)
    ws_d = torch.empty(max(dsa.indexer_loss_dense_workspace_size(st.rows), 1), dtype=torch.uint8,
                       device="cuda")
    dense = lambda: dsa.indexer_loss_dense(st.rows, i.q, i.latent, c.scale, st.scores, loss=loss,
                                           dscores=dsc_d, workspace=ws_d)
    out = {}
    ws_bd = torch.empty(dsa.indexer_backward_dense_workspace_size(st.rows, shared_keys=0),
                        dtype=torch.uint8, device="cuda")
    bwd_d = lambda: dsa.indexer_backward_dense(st.rows, i.q_idx, i.q_scale, i.w, i.k_idx,
                                               i.k_scale, dsc_d, dq, dw, dk, workspace=ws_bd)
    for name, fn in (("loss", fwd), ("backward", bwd), ("loss_dense", dense),
                     ("backward_dense", bwd_d)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = {"ms": e0.elapsed_time(e1) / K}
    sel = R * c.topk
    # loss: the selected latent rows are gathered again and q.c recomputed (bf16 MFMA)
    lb = sel * ATTN_BYTES_PER_ENTRY
    out["loss"].update({"bytes": lb, "gbs": lb / out["loss"]["ms"] / 1e6,
                        "bf16_tflops": sel * 2 * 128 * 576 / out["loss"]["ms"] / 1e9})
    # backward: two 64 x 128 products per selected key (2 flops per multiply-add),
    # run on the bf16 MFMA with each coefficient in three parts (3x the flops executed)
    fl = sel * 2 * 64 * 128 * 2
    out["backward"].update({"fp32_tflops": fl / out["backward"]["ms"] / 1e9,
                            "bf16_mfma_frac": 3 * fl / out["backward"]["ms"] / 1e9
                            / BF16_PEAK_TFLOPS, "deterministic": True})
    # dense warm-up loss: two passes of q.c over every causal position (bf16 MFMA)
    cand, _ = _pairs(c)
    fl_d = cand * 2 * 2 * 128 * 576
    out["loss_dense"].update({"positions": cand, "bf16_tflops": fl_d / out["loss_dense"]["ms"] / 1e9,
                              "frac_of_bf16_peak": fl_d / out["loss_dense"]["ms"] / 1e9
                              / BF16_PEAK_TFLOPS})
    fl_bd = cand * 2 * 64 * 128 * 2
    out["backward_dense"].update({"fp32_tflops": fl_bd / out["backward_dense"]["ms"] / 1e9,
                                  "bf16_mfma_frac": 3 * fl_bd / out["backward_dense"]["ms"]
                                  / 1e9 / BF16_PEAK_TFLOPS, "deterministic": True})
    del dk, dq, dw, ws, dsc, loss, dsc_d, ws_d, ws_b, ws_bd
    torch.cuda.empty_cache()
    return out


def time_mha(dsa, di, K, name="prefill8k"):
    """The masked MHA mode on a prefill workload (the library's own selections),
    against the MQA mode's sparse attention on the same selection.  Both are timed
    with HIP events over K calls."""
    import torch

    cfg = di.CONFIGS[name]
    print(f"[bench] masked MHA mode {name}", file=sys.stderr, flush=True)
    st = Workload(dsa, di, cfg, 0)
    st.run()
    R = cfg.num_rows
    mg = di.MhaGenerator(cfg.cfg_id, 0)
    q = mg.q(0, R, device="cuda")
    w_uk, w_uv = mg.weights(device="cuda")
    out = torch.empty(R, cfg.n_heads, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, cfg.n_heads, dtype=torch.float32, device="cuda")
    ws = torch.empty(dsa.mha_prefill_workspace_size(st.rows, st.dims), dtype=torch.uint8,
                     device="cuda")
    i = st.inp
    mha = lambda: dsa.mha_prefill(st.rows, q, i.latent, w_uk, w_uv, st.idx, cfg.scale,
                                  dims=st.dims, out=out, lse=lse, workspace=ws)
    mqa = lambda: dsa.sparse_mla_attn(st.rows, st.dims, i.q, i.latent, st.idx, cfg.scale,
                                      out=st.out, lse=st.lse, workspace=st.ws)
    res = {"workload": f"{cfg.name}: {cfg.description}"}
    for nm, fn in (("mha", mha), ("mqa", mqa)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[nm + "_ms"] = e0.elapsed_time(e1) / K
    causal, sel = _pairs(cfg)
    # MHA mode: decompression GEMM (each sequence's positions x 32768 x 512) and,
    # per head, the attention over the causal positions (the mask cuts the
    # selection out of them): 192-wide q.k and 128-wide p.v per (row, position)
    dec_tf = cfg.num_seqs * cfg.kv_len * 2 * 16384 * 512 * 2 / 1e12
    att_tf = causal * cfg.n_heads * 2 * (192 + 128) / 1e12
    res.update({"rows": R, "selected_entries": sel, "causal_pairs": causal,
                "mha_tflop": dec_tf + att_tf,
                "mha_bf16_frac": (dec_tf + att_tf) / (res["mha_ms"] * 1e-3) / BF16_PEAK_TFLOPS,
                "mqa_tflop": sel * ATTN_FLOP_PER_ENTRY / 1e12,
                "mqa_bf16_frac": sel * ATTN_FLOP_PER_ENTRY / 1e12 / (res["mqa_ms"] * 1e-3)
                / BF16_PEAK_TFLOPS,
                "mha_speedup": res["mqa_ms"] / res["mha_ms"]})
    del st, q, w_uk, w_uv, out, lse, ws
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(di, cfg, budget_s=20.0, single_budget_s=6.0):
    """The float64 oracle on a bounded sample of the workload's rows on the host
    cores (BLAS threads as configured), then the same rows on one thread."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    g = di.Generator(cfg, 0)
    seq, pos = cfg.row_seq_pos()
    rows = di.sample_rows(cfg, 64)

    def run(budget):
        done, spent = 0, 0.0
        for r in rows:
            b, t = int(seq[r]), int(pos[r])
            qc, qs = g.q_idx(int(r), int(r) + 1)
            kc, ks = g.k_idx(b, 0, t + 1)
            qv = g.q(int(r), int(r) + 1)[0]
            lat = g.latent(b, 0, t + 1)
            args = (qc[0].numpy(), qs[0].numpy().astype(np.float64),
                    g.w(int(r), int(r) + 1)[0].numpy().astype(np.float64), kc.numpy(),
                    ks.numpy().astype(np.float64), di.bf16_bits(qv), di.bf16_bits(lat))
            t0 = time.perf_counter()
            oracle.dsa_row(*args, t, cfg.topk, cfg.scale, cfg.v_dim, quantised=True)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget:
                break
        return done, spent

    done, spent = run(budget_s)
    res = {"value": done / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": _cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
           "sample": f"{done} of {cfg.num_rows} query rows of {cfg.name} (full indexer, top-k "
                     f"and attention per row, float64 numpy), {spent:.1f} s"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, s1 = run(single_budget_s)
        res["single_thread"] = {"value": d1 / s1, "unit": "tokens/s", "cores": 1,
                                "sample": f"{d1} rows, {s1:.1f} s"}
    return res


def sclk_sample(busy_fn, seconds=1.5):
    """The engine clock while the GPU runs busy_fn in a loop: rocm-smi is started,
    the GPU kept busy until it returns, and its sclk line parsed (MHz; None if
    rocm-smi is unavailable)."""
    import re
    import subprocess

    import torch

    try:
        p = subprocess.Popen(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    while p.poll() is None and time.perf_counter() - t0 < 10.0:
        for _ in range(8):
            busy_fn()
        torch.cuda.synchronize()
    try:
        out, _ = p.communicate(timeout=10)
    except subprocess.TimeoutExpired:
        p.kill()
        return None
    m = re.search(r"sclk.*?\((\d+)\s*Mhz\)", out, re.I)
    return int(m.group(1)) if m else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path is "
              f"single-GPU; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": 4 * n, "copy_calib_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return

    import dsa_inputs as di
    import sparse_attention_fp8_amd as dsa

    if args.mha_only:
        K = max(2, args.steps // 4)
        print(json.dumps({name: time_mha(dsa, di, K, name) for name in ("prefill2k", "prefill8k")}),
              flush=True)
        return

    cfg = di.CONFIGS[args.workload]
    head, sets = time_decode(dsa, di, cfg, args.sets, args.steps, args.warmup,
                             graphs=not args.headline_only)
    kernels = head["kernels"]
    roof = dict(head["roofline"])
    mt = measured_traffic(cfg.name, roof["kernel"])
    roof["traffic"] = mt[0] if mt else None
    roof["traffic_kernels"] = mt[1] if mt else None
    ms = head["ms_per_step"]
    R = cfg.num_rows
    line = {
        "metric": METRIC,
        "value": R / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "batch": cfg.num_seqs,
                   "context": cfg.kv_len, "topk": cfg.topk, "input_sets": args.sets,
                   "timed_call": "dsa_forward, one call per step"},
        "roofline": roof,
        "step_hbm_frac": head["step_hbm_frac"],
        "kernels": kernels,
        "ms_per_step_three_calls": head["ms_per_step_three_calls"],
        "step_ms_events": head["step_ms_events"],
        "ms_per_step_warm": head["ms_per_step_warm"],
    }
    if "graph" in head:
        line["graph"] = head["graph"]
    if not args.headline_only:
        line["sclk_mhz"] = sclk_sample(sets[0].run_forward)
        # the same step over paged caches (64-entry pages in shuffled order)
        P = 64
        for k, st in enumerate(sets):
            st.make_paged(P, seed=k)
        pms = time_bare([st.run_paged for st in sets], args.steps, args.warmup)
        line["paged"] = {"page_size": P, "ms_per_step": pms, "tokens_per_s": R / (pms * 1e-3),
                         "vs_three_contiguous_calls": head["ms_per_step_three_calls"] / pms}
        line["indexer_training"] = time_training(dsa, sets[0], args.steps)
    del sets
    torch.cuda.empty_cache()
    if not args.headline_only:
        # the other two headline workloads of the metric: long decode and 128K prefill
        d128, s128 = time_decode(dsa, di, di.CONFIGS["decode128k"], 3, args.steps, args.warmup)
        del s128
        torch.cuda.empty_cache()
        line["decode128k"] = d128
        line["prefill128k"] = time_prefill(dsa, di, di.CONFIGS["prefill128k"], 2)
        line["prefill128k_tokens_per_s"] = line["prefill128k"]["tokens_per_s"]
        # the step before the path: projections and cache append of the new tokens
        line["projections"] = {name: time_projection(dsa, di, di.PROJ_CONFIGS[name], reps)
                               for name, reps in (("proj_decode32", 30), ("proj_prefill8k", 10))}
        # the masked MHA mode beside the MQA mode: short prefill (every causal set
        # fits in k, where the mode is meant to win) and 8K
        line["mha_prefill2k"] = time_mha(dsa, di, max(2, args.steps // 4), "prefill2k")
        line["mha_prefill8k"] = time_mha(dsa, di, max(2, args.steps // 4), "prefill8k")
    if args.extra:
        line["extra"] = {"prefill8k": time_prefill(dsa, di, di.CONFIGS["prefill8k"], 5)}
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(di, cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
