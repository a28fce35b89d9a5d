"""Benchmark: CSA decode query-tokens/s at 1M and 128K context on one MI355X, with the roofline of
the dominant kernel and the CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--legs main,d128,c32k,hca,flash,append,prefill,compress,oproj]
                    [--mode bench|copy|summarize-trace|summarize-traffic|summarize-mfma|summarize-counters]

One step = one decode pass of the whole hot path over one batch: csa_index_topk (lightning-indexer
scores + top-k) then csa_attend (shared-KV attention over the selected entries + window) for CSA;
hca_attend for HCA.  Inputs are seeded synthetic tensors resident in HBM before timing.  Every
step reads one of several copies of the caches, enough copies that the working set exceeds the
256 MB Infinity Cache by 4x, so each step streams from HBM.  The steps are replayed from a HIP
graph (host launch overhead would otherwise be a large part of the ~50 us step).  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from compressed_sparse_attention_03_amd import inputs as gen  # noqa: E402
from compressed_sparse_attention_03_amd import ops  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA (MI355X, no sparsity)
METRIC = "CSA decode query-tokens/sec at 128K and 1M ctx; % of peak HBM GB/s"
KEY_BYTES = {"fp8": 128 + 4, "mxfp4": 64 + 4}
MALL_BYTES = 256e6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---- algorithmic bytes (each item the method must touch, once per step) ----------------------
def csa_query_bytes(w):
    keys = w.N * KEY_BYTES[w.key_format]
    rows = (w.topk + w.window) * w.d * 2
    q_out = 2 * w.H * w.d * 2
    idx_q = w.H_I * w.D_I * 2 + w.H_I * 4
    sel = w.topk * 4 * 2
    return keys + rows + q_out + idx_q + sel


def hca_query_bytes(w):
    return (w.N + w.window) * w.d * 2 + 2 * w.H * w.d * 2


def index_score_bytes(w):
    return w.B * (w.N * KEY_BYTES[w.key_format] + w.H_I * w.D_I * 2 + w.H_I * 4)


# ---- one workload leg --------------------------------------------------------------------------
class Leg:
    def __init__(self, w: gen.Workload, append: bool = False):
        self.w = w
        self.append = append
        self.step_bytes = w.B * (hca_query_bytes(w) if w.kind == "hca_decode" else csa_query_bytes(w))
        self.ncopies = max(2, math.ceil(4 * MALL_BYTES / self.step_bytes))
        log(f"[{w.name}] generating inputs; {self.ncopies} copies of {self.step_bytes / 1e6:.1f} MB/step")
        t0 = time.time()
        x = gen.decode_inputs(w)
        self.t = dev(x["t"])
        self.win_pos0 = dev(x["win_pos0"])
        self.n_ent = dev(x["n_entries"])
        q, ent, win = dev_bf16(x["q"]), dev_bf16(x["entries"]), dev_bf16(x["win_rows"])
        self.q = [q] + [q.clone() for _ in range(self.ncopies - 1)]
        self.ent = [ent] + [ent.clone() for _ in range(self.ncopies - 1)]
        self.win = [win] + [win.clone() for _ in range(self.ncopies - 1)]
        self.out = [torch.empty_like(q) for _ in range(self.ncopies)]
        if w.kind == "csa_decode":
            qi, wi = dev_bf16(x["q_idx"]), dev(x["w_idx"])
            codes, scales = ops.csa_quantize_keys(dev_bf16(x["k_idx"]), w.key_format)
            self.q_idx = [qi] + [qi.clone() for _ in range(self.ncopies - 1)]
            self.w_idx = [wi] + [wi.clone() for _ in range(self.ncopies - 1)]
            self.codes = [codes] + [codes.clone() for _ in range(self.ncopies - 1)]
            self.scales = [scales] + [scales.clone() for _ in range(self.ncopies - 1)]
            self.sel = [torch.empty((w.B, 1, w.topk), dtype=torch.int32, device="cuda") for _ in range(self.ncopies)]
            self.ws_i = ops.index_topk_workspace(w.B, 1, w.N, w.topk)
            self.ws_a = ops.attend_workspace(w.B, 1, w.H, w.d, w.topk, w.window)
            if append:
                # cache maintenance in front of the step: the new token at t = T-1 closes a group
                # (entry N-1 is rewritten and its key quantised every step); the window rows are
                # read as a ring of W_cap = window rows
                g = torch.Generator(device="cuda").manual_seed(w.cfg)
                bf = lambda *shape, std=1.0: (std * torch.randn(shape, generator=g, device="cuda")).to(torch.bfloat16)
                R = (1 + w.overlap) * w.m
                self.tok_c = [bf(w.B, R, w.d) for _ in range(self.ncopies)]
                self.tok_z = [bf(w.B, R, w.d) for _ in range(self.ncopies)]
                self.c_new = [bf(w.B, w.d) for _ in range(self.ncopies)]
                self.z_new = [bf(w.B, w.d) for _ in range(self.ncopies)]
                self.bias = bf(R, w.d, std=0.1)
                self.n_app = self.n_ent.clone()
                # the indexer stream: its ring, the new token's row and logits, its bias; the
                # closed entry's key is produced by compression and quantised on write
                self.tok_ci = [bf(w.B, R, w.D_I) for _ in range(self.ncopies)]
                self.tok_zi = [bf(w.B, R, w.D_I) for _ in range(self.ncopies)]
                self.c_i_new = [bf(w.B, w.D_I) for _ in range(self.ncopies)]
                self.z_i_new = [bf(w.B, w.D_I) for _ in range(self.ncopies)]
                self.bias_i = bf(R, w.D_I, std=0.1)
        else:
            self.ws_a = ops.hca_workspace(w.B, 1, w.H, w.d, w.N, w.window)
        del x
        torch.cuda.synchronize()
        log(f"[{w.name}] inputs ready in {time.time() - t0:.1f}s")

    def step(self, i):
        w, c = self.w, i % self.ncopies
        if w.kind == "csa_decode" and self.append:
            ops.csa_decode_append_step(self.c_new[c], self.z_new[c], self.t, self.bias, m=w.m, overlap=w.overlap,
                                       rope_dim=w.rope_dim, tok_c=self.tok_c[c], tok_z=self.tok_z[c],
                                       win_ring=self.win[c], entries=self.ent[c], n_entries=self.n_app,
                                       c_i_new=self.c_i_new[c], z_i_new=self.z_i_new[c], bias_i=self.bias_i,
                                       tok_ci=self.tok_ci[c], tok_zi=self.tok_zi[c], key_format=w.key_format,
                                       k_codes=self.codes[c], k_scales=self.scales[c])
            ops.csa_index_topk(self.q_idx[c], self.w_idx[c], self.codes[c], self.scales[c], key_format=w.key_format,
                               n_entries=self.n_app, q_pos0=self.t, m=w.m, topk=w.topk, workspace=self.ws_i,
                               topk_out=self.sel[c])
            ops.csa_attend(self.q[c], self.ent[c], self.sel[c], self.win[c], None, self.t,
                           rope_dim=w.rope_dim, window=w.window, workspace=self.ws_a, out=self.out[c])
        elif w.kind == "csa_decode":
            ops.csa_index_topk(self.q_idx[c], self.w_idx[c], self.codes[c], self.scales[c], key_format=w.key_format,
                               n_entries=self.n_ent, q_pos0=self.t, m=w.m, topk=w.topk, workspace=self.ws_i,
                               topk_out=self.sel[c])
            ops.csa_attend(self.q[c], self.ent[c], self.sel[c], self.win[c], self.win_pos0, self.t,
                           rope_dim=w.rope_dim, window=w.window, workspace=self.ws_a, out=self.out[c])
        else:
            ops.hca_attend(self.q[c], self.ent[c], self.n_ent, self.win[c], self.win_pos0, self.t, m=w.m,
                           rope_dim=w.rope_dim, window=w.window, workspace=self.ws_a, out=self.out[c])

    def kernel_times(self, n=None):
        """Average per-kernel durations (us) from HIP events recorded around each launch."""
        n = self.ncopies * 2 if n is None else n
        for i in range(self.ncopies):
            self.step(i)
        torch.cuda.synchronize()
        ops.timing_enable(True)
        for i in range(n):
            self.step(i)
        torch.cuda.synchronize()
        res = {}
        for k in ("decode_append_step", "decode_append", "decode_append_keys", "index_score", "index_merge", "attend_split",
                  "attend_combine"):
            ms, cnt = ops.timing_read(k)
            if cnt:
                res[k] = 1000.0 * ms / cnt
        ops.timing_enable(False)
        return res

    def run(self, steps, warmup, graph=True):
        """Time exactly `steps` steps after `warmup` steps; returns seconds."""
        G = self.ncopies
        if graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for i in range(G):                      # prime the allocator-free path once
                    self.step(i)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            full = torch.cuda.CUDAGraph()
            with torch.cuda.graph(full):
                for i in range(G):
                    self.step(i)
            singles = []
            for i in range(G):
                g1 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g1):
                    self.step(i)
                singles.append(g1)

            def run_n(n):
                for _ in range(n // G):
                    full.replay()
                for i in range(n % G):
                    singles[i].replay()
        else:
            def run_n(n):
                for i in range(n):
                    self.step(i)
        run_n(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_n(steps)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def free(self):
        for k in list(self.__dict__):
            if k != "w" and k != "step_bytes" and k != "ncopies":
                delattr(self, k)
        torch.cuda.empty_cache()


def profile_traffic(kernel: str, workload: str):
    """HBM bytes per dispatch from a committed rocprofv3 PMC summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    src = os.path.join(ROOT, "compressed_sparse_attention_03_amd", "csrc", vals.get("source", "indexer.hip"))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != vals.get("source_sha256_16"):
        return None
    try:
        return float(vals["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ---- CPU oracle baseline -------------------------------------------------------------------------
def cpu_baseline(w: gen.Workload, budget_s: float = 12.0):
    """The oracle as it stands, on the host cores: one decode query of sequence 0 (its full
    indexer scan, top-k and attention), repeated until the time budget is spent."""
    from oracle import attention as oa
    from oracle import indexer as oi
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    x = gen.decode_inputs(w, 0, 1)
    f = lambda a: gen.bf16_bits_to_f32(a).astype(np.float64)
    kt = np.empty((w.N, w.D_I))
    for i in range(0, w.N, 65536):                       # the stored (quantised) keys: not timed
        codes, sc = oi.quantize_keys(f(x["k_idx"][0, i:i + 65536]), w.key_format)
        kt[i:i + 65536] = oi.dequantize_keys(codes, sc, w.key_format)
    ent = x["entries"][0]
    win = f(x["win_rows"][0])
    t = int(x["t"][0])
    n, t0 = 0, time.perf_counter()
    while True:
        qt = oi.quantize_query(f(x["q_idx"][0, 0]), w.key_format)
        s = oi.index_scores(qt, x["w_idx"][0, 0].astype(np.float64), kt, w.N)
        sel = oi.topk_fast(s, w.topk, w.N)
        oa.csa_attend(f(x["q"][0, 0]), f(ent[sel]), np.arange(w.topk), win, int(x["win_pos0"][0]), t, w.window,
                      w.rope_dim)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 2000:                  # the time budget normally ends it (~12 s)
            break
    return {"value": n / el, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} decode queries of sequence 0 of {w.name} (indexer over all {w.N} entries, "
                      f"top-{w.topk}, attention over {w.topk}+{w.window} rows); keys pre-quantised"}


def stream_floor(nbytes: int, launches: int = 240):
    """The library's plain streaming read (csa_measure_stream_read) of `nbytes`, timed like the
    kernels (events in each dispatch), over enough rotating buffers to miss the 256 MB
    Infinity Cache: the bandwidth a bandwidth-bound kernel of that byte count can reach here."""
    nbytes = (int(nbytes) + 15) // 16 * 16
    nbuf = max(2, math.ceil(2 * MALL_BYTES / nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    for i, b in enumerate(bufs):
        b.fill_(i + 1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for i in range(2 * nbuf):                                  # warm-up
        ops.measure_stream_read(bufs[i % nbuf], sink)
    torch.cuda.synchronize()
    ops.timing_enable(True)
    for i in range(launches):
        ops.measure_stream_read(bufs[i % nbuf], sink)
    torch.cuda.synchronize()
    ms, cnt = ops.timing_read("stream_read")
    ops.timing_enable(False)
    del bufs
    torch.cuda.empty_cache()
    us = 1000.0 * ms / cnt
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "stream_read", "bytes": nbytes, "avg_us": us, "achieved": gbs, "unit": "GB/s",
            "frac_of_peak": gbs / PEAK_HBM_GBS, "buffers": nbuf, "launches": cnt}


COPY_BYTES, COPY_LAUNCHES = 1 << 30, 5


def copy_calibration():
    """Plain device copies of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(COPY_LAUNCHES):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": COPY_LAUNCHES}))


# ---- prefill chunk and compressor legs ------------------------------------------------------------
class PrefillLeg:
    """One prefill chunk: compress 4,096 new tokens (plus the m-token halo) into 1,024 entries
    appended after the 32,768 existing ones (and their prepared window rows), produce the new
    entries' indexer keys by compressing the chunk's per-token indexer stream (quantised on
    write), then csa_index_topk and csa_attend for all 4,096 query tokens."""

    def __init__(self, w: gen.Workload):
        self.w = w
        n, m, d = w.Sq, w.m, w.d
        self.N0, self.Wp = w.N, w.window - 1                # existing entries, earlier window rows
        self.N_cap, self.W_cap = w.N + n // m, w.window - 1 + n
        log(f"[{w.name}] generating inputs")
        t0 = time.time()
        self.c = dev_bf16(gen.normal_bf16(w.cfg, gen.T_C, (n + m, d))).view(1, n + m, d)
        self.z = dev_bf16(gen.normal_bf16(w.cfg, gen.T_Z, (n + m, d))).view(1, n + m, d)
        self.bias = dev_bf16(gen.normal_bf16(w.cfg, gen.T_BIAS, (2 * m, d), std=0.1))
        self.q = dev_bf16(gen.normal_bf16(w.cfg, gen.T_Q, (n * w.H, d))).view(1, n, w.H, d)
        self.q_idx = dev_bf16(gen.normal_bf16(w.cfg, gen.T_QIDX, (n * w.H_I, w.D_I))).view(1, n, w.H_I, w.D_I)
        self.w_idx = dev(gen.uniform_f32(w.cfg, gen.T_W, (n * w.H_I,))).view(1, n, w.H_I)
        self.k_idx = dev_bf16(gen.normal_bf16(w.cfg, gen.T_KIDX, (self.N_cap, w.D_I))).view(1, self.N_cap, w.D_I)
        self.entries = torch.empty((1, self.N_cap, d), dtype=torch.bfloat16, device="cuda")
        self.entries[:, :self.N0] = dev_bf16(gen.normal_bf16(w.cfg, gen.T_ENTRIES, (self.N0, d))).view(1, self.N0, d)
        self.win = torch.empty((1, self.W_cap, d), dtype=torch.bfloat16, device="cuda")
        self.win[:, :self.Wp] = dev_bf16(gen.normal_bf16(w.cfg, gen.T_WIN, (self.Wp, d))).view(1, self.Wp, d)
        self.codes, self.scales = ops.csa_quantize_keys(self.k_idx, w.key_format)   # existing keys
        # the chunk's per-token indexer stream (plus the halo), its logits and position bias
        self.c_i = dev_bf16(gen.normal_bf16(w.cfg, gen.T_KIDX, (n + m, w.D_I), row0=self.N_cap,
                                            nrows=n + m)).view(1, n + m, w.D_I)
        self.z_i = dev_bf16(gen.normal_bf16(w.cfg, gen.T_Z, (n + m, w.D_I))).view(1, n + m, w.D_I)
        self.bias_i = dev_bf16(gen.normal_bf16(w.cfg, gen.T_BIAS, (2 * m, w.D_I), std=0.1))
        self.n_ent = torch.tensor([self.N_cap], dtype=torch.int64, device="cuda")
        self.t = torch.tensor([w.T], dtype=torch.int64, device="cuda")
        self.win_pos0 = torch.tensor([w.T - self.Wp], dtype=torch.int64, device="cuda")
        self.sel = torch.empty((1, n, w.topk), dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.ws_i = ops.index_topk_workspace(1, n, self.N_cap, w.topk)
        self.ws_a = ops.attend_workspace(1, n, w.H, d, w.topk, w.window)
        torch.cuda.synchronize()
        log(f"[{w.name}] inputs ready in {time.time() - t0:.1f}s")
        # work per chunk: indexer scores over every visible entry, attention over k + W rows
        vis = np.minimum(self.N_cap, (w.T + np.arange(n) + 1) // m)
        self.index_flops = float(vis.sum()) * w.H_I * w.D_I * 2
        self.attend_flops = float(n) * w.H * (w.topk + w.window) * d * 4

    def step(self, i=0):
        w = self.w
        ops.csa_compress(self.c, self.z, self.bias, m=w.m, overlap=w.overlap, rope_dim=w.rope_dim, pos0=w.T,
                         win_rows=True, entries_out=self.entries[:, self.N0:], win_rows_out=self.win[:, self.Wp:])
        ops.csa_compress_index_keys(self.c_i, self.z_i, self.bias_i, m=w.m, overlap=w.overlap,
                                    key_format=w.key_format, pos0=w.T, k_codes=self.codes[:, self.N0:],
                                    k_scales=self.scales[:, self.N0:])
        ops.csa_index_topk(self.q_idx, self.w_idx, self.codes, self.scales, key_format=w.key_format,
                           n_entries=self.n_ent, q_pos0=self.t, m=w.m, topk=w.topk, workspace=self.ws_i,
                           topk_out=self.sel)
        ops.csa_attend(self.q, self.entries, self.sel, self.win, self.win_pos0, self.t, rope_dim=w.rope_dim,
                       window=w.window, workspace=self.ws_a, out=self.out)

    def measure(self, steps):
        for _ in range(3):
            self.step()
        torch.cuda.synchronize()
        ops.timing_enable(True)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        kt = {}
        for k in ("compress", "compress_keys", "index_query_prep", "index_score", "index_merge", "attend_split",
                  "attend_combine"):
            ms, cnt = ops.timing_read(k)
            if cnt:
                kt[k] = 1000.0 * ms / cnt
        ops.timing_enable(False)
        # the indexer's time: the shared-tile kernel and the one-time query quantisation before it
        t_index = (kt["index_score"] + kt.get("index_query_prep", 0.0)) * 1e-6
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step()
            with torch.cuda.graph(g, stream=s):
                self.step()
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        w = self.w
        return {"workload": w.name, "value": w.Sq / sec, "unit": "chunk query-tokens/s", "ms_per_step": 1000 * sec,
                "kernel_us": kt,
                "index_mfma": {"bound": "mfma", "dtype": "fp8", "flops": self.index_flops,
                               "achieved_tflops": self.index_flops / t_index / 1e12,
                               "peak_tflops": 5000.0,
                               "frac": self.index_flops / t_index / 5.0e15},
                "attend_mfma": {"bound": "mfma", "dtype": "bf16", "flops": self.attend_flops,
                                "achieved_tflops": self.attend_flops / (kt["attend_split"] * 1e-6) / 1e12,
                                "peak_tflops": 2500.0,
                                "frac": self.attend_flops / (kt["attend_split"] * 1e-6) / 2.5e15}}


def compress_leg(steps: int):
    """The 1M-token HCA compression (8 sequences x 1,048,576 tokens, m = 128, d = 512): HBM-bound
    streaming of c and z.  The 17 GB of inputs are drawn on the GPU with a seeded torch generator
    (N(0,1); bias N(0, 0.1)); the parity tests use the host generator on sampled sequences."""
    w = gen.HCA_DECODE_1M
    gpu = torch.Generator(device="cuda")
    gpu.manual_seed(1000 + w.cfg)
    c = torch.randn((w.B, w.T, w.d), generator=gpu, device="cuda", dtype=torch.bfloat16)
    z = torch.randn((w.B, w.T, w.d), generator=gpu, device="cuda", dtype=torch.bfloat16)
    bias = (0.1 * torch.randn((w.m, w.d), generator=gpu, device="cuda")).to(torch.bfloat16)
    ent = torch.empty((w.B, w.T // w.m, w.d), dtype=torch.bfloat16, device="cuda")
    run = lambda: ops.csa_compress(c, z, bias, m=w.m, overlap=0, rope_dim=w.rope_dim, pos0=0, entries_out=ent)
    run()
    torch.cuda.synchronize()
    ops.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    ms, cnt = ops.timing_read("compress")
    ops.timing_enable(False)
    kus = 1000.0 * ms / max(cnt, 1)
    nbytes = 2 * c.numel() * 2 + ent.numel() * 2
    del c, z
    torch.cuda.empty_cache()
    return {"workload": "hca_compress_1m_b8", "value": w.B * w.T / sec, "unit": "tokens/s", "ms_per_step": 1000 * sec,
            "kernel_us": {"compress": kus},
            "roofline": {"kernel": "compress", "bound": "hbm", "achieved": nbytes / (kus * 1e-6) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": nbytes / (kus * 1e-6) / 1e9 / PEAK_HBM_GBS,
                         "algorithmic_bytes": nbytes},
            "data": "seeded torch generator on the GPU"}


def oproj_leg(steps: int):
    """The grouped output projection after core attention: 64 heads x 512 in 8 groups, each group
    projected to 512 of a 4,096-wide hidden state (synthetic shapes and weights: the pages give
    no sizes).  A decode step of four tokens streams the 32 MiB of weights (HBM roofline); a
    4,096-token prefill chunk is a 137 GFLOP bf16 contraction (MFMA roofline)."""
    H, D, G, N_g = 64, 512, 8, 512
    K_g = H * D // G
    gpu = torch.Generator(device="cuda")
    gpu.manual_seed(77)
    ncopy = max(2, math.ceil(4 * MALL_BYTES / (G * N_g * K_g * 2)))     # weights beyond the cache
    ws = [(torch.randn((G, N_g, K_g), generator=gpu, device="cuda") / math.sqrt(K_g)).to(torch.bfloat16)
          for _ in range(ncopy)]
    res = {"workload": "grouped_output_projection_h64x512_g8_to_4096", "data": "seeded torch generator on the GPU",
           "kernel_us": {}}
    for M, tag in ((4, "decode_m4"), (4096, "prefill_m4096")):
        o = torch.randn((M, H, D), generator=gpu, device="cuda").to(torch.bfloat16)
        y = torch.empty((M, G * N_g), dtype=torch.bfloat16, device="cuda")
        for i in range(ncopy):
            ops.csa_output_projection(o, ws[i], out=y)
        torch.cuda.synchronize()
        n = steps if M == 4 else max(3, steps // 20)
        ops.timing_enable(True)
        for i in range(n):
            ops.csa_output_projection(o, ws[i % ncopy], out=y)
        torch.cuda.synchronize()
        ms, cnt = ops.timing_read("oproj")
        ops.timing_enable(False)
        us = 1000.0 * ms / max(cnt, 1)
        res["kernel_us"][tag] = us
        if M == 4:
            nbytes = G * N_g * K_g * 2 + o.numel() * 2 + y.numel() * 2
            res[tag] = {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes": nbytes}
        else:
            flops = 2.0 * M * K_g * N_g * G
            res[tag] = {"bound": "mfma", "dtype": "bf16", "flops": flops, "achieved_tflops": flops / (us * 1e-6) / 1e12,
                        "peak_tflops": PEAK_BF16_TFLOPS, "frac": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
        del o, y
    del ws
    torch.cuda.empty_cache()
    return res


# ---- rocprofv3 summaries (text for profiles/) -----------------------------------------------------
def _short_kernel(name: str) -> str:
    name = name.replace("void ", "").replace("csa::(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize_trace(db: str, min_calls: int = 3) -> str:
    """Per-kernel duration table of a `rocprofv3 --kernel-trace` database (one row per kernel and
    grid size: launches of one kernel on different workloads differ in grid)."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute("select name, grid_x, grid_y, workgroup_x, count(*), avg(duration), min(duration), "
                       "max(duration) from kernels group by name, grid_x, grid_y order by min(start)").fetchall()
    out = ["| kernel | grid (threads) | block | launches | avg us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for n, gx, gy, wx, c, a, mn, mx in rows:
        if c >= min_calls:
            out.append(f"| {_short_kernel(n)} | {gx}x{gy} | {wx} | {c} | {a / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    return "\n".join(out)


def _counter_stats(db: str, counter: str, kernel_substr: str):
    """(average per dispatch, sum, dispatches) of one counter over the dispatches of a kernel."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    r = cur.execute("select avg(counter_value), sum(counter_value), count(*) from pmc_events "
                    "where counter_name = ? and name like ?", (counter, f"%{kernel_substr}%")).fetchone()
    return (r[0], r[1], r[2]) if r and r[2] else (None, None, 0)


def summarize_traffic(fetch_db: str, write_db: str, copy_fetch_db: str, copy_write_db: str, kernel: str,
                      source: str) -> str:
    """key = value summary of HBM traffic per dispatch of `kernel` (FETCH_SIZE and WRITE_SIZE in KiB,
    each scaled by what the counter reads for a plain copy of known size)."""
    copy_bytes = COPY_BYTES * COPY_LAUNCHES          # every device copy `--mode copy` makes
    _, cf, _ = _counter_stats(copy_fetch_db, "FETCH_SIZE", "copyBuffer")
    _, cw, _ = _counter_stats(copy_write_db, "WRITE_SIZE", "copyBuffer")
    kf, _, nf = _counter_stats(fetch_db, "FETCH_SIZE", kernel)
    kw, _, nw = _counter_stats(write_db, "WRITE_SIZE", kernel)
    ff = copy_bytes / (cf * 1024.0)
    fw = copy_bytes / (cw * 1024.0)
    src = os.path.join(ROOT, "compressed_sparse_attention_03_amd", "csrc", source)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    traffic = kf * 1024.0 * ff + kw * 1024.0 * fw
    return "\n".join([
        f"kernel = {kernel}", f"source = {source}", f"source_sha256_16 = {sha}",
        f"fetch_kib_per_dispatch = {kf:.1f}", f"fetch_dispatches = {nf}",
        f"write_kib_per_dispatch = {kw:.1f}", f"write_dispatches = {nw}",
        f"copy_bytes = {copy_bytes}", f"copy_fetch_kib = {cf:.1f}", f"copy_write_kib = {cw:.1f}",
        f"fetch_factor = {ff:.3f}", f"write_factor = {fw:.3f}",
        f"traffic_bytes_per_dispatch = {traffic:.0f}"])


def summarize_counters(dbs, kernels) -> str:
    """Per-kernel averages per dispatch (summed over the GPU's instances of each counter) of every
    counter in one or more `rocprofv3 --pmc` databases, and the ratios that share a unit: the share
    of wave cycles spent waiting (on anything; on an instruction's dependency), issuing (any
    instruction; VALU; LDS; vector memory), LDS bank-conflict cycles per LDS-active cycle and the
    L2 hit rate."""
    import sqlite3
    vals = {k: {} for k in kernels}
    for db in dbs:
        cur = sqlite3.connect(db).cursor()
        names = [r[0] for r in cur.execute("select distinct counter_name from pmc_events")]
        for k in kernels:
            for c in names:
                r = cur.execute("select avg(v), count(*) from (select sum(counter_value) as v from pmc_events where "
                                "counter_name = ? and name like ? group by dispatch_id)", (c, f"%{k}%")).fetchone()
                if r and r[1]:
                    vals[k][c] = (r[0], r[1])
    out = []
    for k in kernels:
        v = {c: x[0] for c, x in vals[k].items()}
        n = max([x[1] for x in vals[k].values()] + [0])
        out.append(f"{k} ({n} dispatches)")
        for c in sorted(v):
            out.append(f"  {c} = {v[c]:.4g}")
        ratio = lambda a, b: (v[a] / v[b]) if a in v and b in v and v[b] else None
        derived = [("wave cycles waiting (any)", ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
                   ("wave cycles waiting on a dependency", ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
                   ("wave cycles issuing (any)", ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES")),
                   ("wave cycles issuing VALU", ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")),
                   ("wave cycles issuing LDS", ratio("SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES")),
                   ("wave cycles issuing vector memory", ratio("SQ_ACTIVE_INST_VMEM", "SQ_WAVE_CYCLES")),
                   ("LDS bank-conflict cycles per LDS-active cycle", ratio("SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"))]
        if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v and v["TCC_HIT_sum"] + v["TCC_MISS_sum"]:
            derived.append(("L2 hit rate", v["TCC_HIT_sum"] / (v["TCC_HIT_sum"] + v["TCC_MISS_sum"])))
        for name, x in derived:
            if x is not None:
                out.append(f"  [{name}] = {x:.3f}")
    return "\n".join(out)


MFMA_COUNTERS = ("MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16")


def summarize_mfma(db: str, kernels) -> str:
    """Per-kernel MFMA evidence from one `rocprofv3 --pmc` run of MFMA_COUNTERS: MfmaUtil (percent of
    SIMD cycles the matrix unit is busy while the GPU is active) and the MFMA operations counted per
    data type (the counters count add and multiply operations in units of 512), per dispatch."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    out = ["| kernel | dispatches | MfmaUtil % | fp8 GFLOP | fp6/fp4 GFLOP | bf16 GFLOP |", "|---|---|---|---|---|---|"]
    for k in kernels:
        vals = {}
        n = 0
        for c in MFMA_COUNTERS:
            r = cur.execute("select avg(v), count(*) from (select sum(counter_value) as v from pmc_events where "
                            "counter_name = ? and name like ? group by dispatch_id)", (c, f"%{k}%")).fetchone()
            vals[c] = r[0] if r and r[1] else None
            n = max(n, r[1] if r else 0)
        g = lambda c: "-" if vals[c] is None else f"{vals[c] * 512 / 1e9:.1f}"
        u = "-" if vals["MfmaUtil"] is None else f"{vals['MfmaUtil']:.1f}"
        out.append(f"| {k} | {n} | {u} | {g('SQ_INSTS_VALU_MFMA_MOPS_F8')} | {g('SQ_INSTS_VALU_MFMA_MOPS_F6F4')} | "
                   f"{g('SQ_INSTS_VALU_MFMA_MOPS_BF16')} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--legs", default="main,d128,c32k,hca,flash,append,prefill,compress,oproj")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "summarize-trace", "summarize-traffic",
                                                        "summarize-mfma", "summarize-counters"])
    ap.add_argument("--db", nargs="*", default=[], help="rocprofv3 databases for the summarize modes: one "
                    "kernel-trace db; or FETCH, WRITE, copy-FETCH, copy-WRITE dbs")
    ap.add_argument("--kernel", default="index_score_kernel")
    ap.add_argument("--source", default="indexer.hip")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_calibration()
        return
    if args.mode == "summarize-trace":
        print(summarize_trace(args.db[0]))
        return
    if args.mode == "summarize-mfma":
        print(summarize_mfma(args.db[0], args.kernel.split(",")))
        return
    if args.mode == "summarize-traffic":
        print(summarize_traffic(*args.db[:4], kernel=args.kernel, source=args.source))
        return
    if args.mode == "summarize-counters":
        print(summarize_counters(args.db, args.kernel.split(",")))
        return
    legs = args.legs.split(",")
    table = {"main": gen.CSA_DECODE_1M, "d128": gen.CSA_DECODE_128K, "c32k": gen.CSA_DECODE_32K,
             "hca": gen.HCA_DECODE_1M, "append": gen.CSA_DECODE_1M, "flash": gen.CSA_DECODE_1M_FLASH}
    results = {}
    for name in legs:
        if name == "prefill":
            leg = PrefillLeg(gen.CSA_PREFILL_128K)
            results[name] = leg.measure(max(3, min(args.steps // 100, 20)))
            log(json.dumps(results[name]))
            del leg
            torch.cuda.empty_cache()
            continue
        if name == "compress":
            results[name] = compress_leg(max(3, min(args.steps // 200, 10)))
            log(json.dumps(results[name]))
            continue
        if name == "oproj":
            results[name] = oproj_leg(max(20, min(args.steps, 200)))
            log(json.dumps(results[name]))
            continue
        w = table[name]
        leg = Leg(w, append=(name == "append"))
        kt = leg.kernel_times()
        sec = leg.run(args.steps, args.warmup, graph=True)
        sec_eager = leg.run(min(args.steps, 200), min(args.warmup, 20), graph=False)
        ms = 1000 * sec / args.steps
        tok_s = w.B * args.steps / sec
        r = {"workload": w.name + ("+decode_append" if name == "append" else ""), "value": tok_s,
             "unit": "query-tokens/s", "ms_per_step": ms,
             "hbm_frac_step": leg.step_bytes * args.steps / sec / (PEAK_HBM_GBS * 1e9),
             "bytes_per_step": leg.step_bytes, "copies": leg.ncopies,
             "eager_ms_per_step": 1000 * sec_eager / min(args.steps, 200), "kernel_us": kt}
        if w.kind == "csa_decode":
            ab = index_score_bytes(w)
            dur = kt["index_score"] * 1e-6
            r["roofline"] = {"kernel": "index_score", "bound": "hbm", "achieved": ab / dur / 1e9,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ab / dur / 1e9 / PEAK_HBM_GBS,
                             "traffic": profile_traffic("index_score", w.name),
                             "algorithmic_bytes": ab, "avg_us": kt["index_score"]}
        else:
            ab = leg.step_bytes
            dur = (kt.get("attend_split", 0.0) + kt.get("attend_combine", 0.0)) * 1e-6
            ts, tc = profile_traffic("attend_split", w.name), profile_traffic("attend_combine", w.name)
            r["roofline"] = {"kernel": "attend_split+attend_combine", "bound": "hbm", "achieved": ab / dur / 1e9,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ab / dur / 1e9 / PEAK_HBM_GBS,
                             "traffic": None if ts is None or tc is None else ts + tc,
                             "algorithmic_bytes": ab, "avg_us": kt.get("attend_split")}
        results[name] = r
        log(json.dumps(r))
        leg.free()
        del leg
    table_legs = [k for k in legs if k in table and k != "append"]
    if not table_legs:                                           # only side legs were asked for
        return
    main_name = table_legs[0]
    m = results[main_name]
    w = table[main_name]
    line = {
        "metric": METRIC, "value": m["value"], "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+" + w.key_format if w.kind == "csa_decode" else "bf16",
        "data": "synthetic (seeded N(0,1) caches/queries, U(0,1) indexer weights, 16 planted keys)",
        "config": {"workload": w.name, "batch": w.B, "context": w.T, "entries": w.N, "topk": w.topk,
                   "window": w.window, "heads": w.H, "head_dim": w.d, "indexer": f"{w.H_I}x{w.D_I} {w.key_format}",
                   "step": "csa_index_topk + csa_attend, HIP graph"},
        "hbm_frac_step": m["hbm_frac_step"],
        "roofline": m["roofline"],
        "kernel_us": m["kernel_us"],
        "also": [results[k] for k in legs if k != main_name],
    }
    # the plain streaming read of the dominant kernel's byte count, timed the same way
    rf = line["roofline"]
    rf["stream_floor"] = stream_floor(rf["algorithmic_bytes"])
    rf["frac_of_stream_floor"] = rf["achieved"] / rf["stream_floor"]["achieved"]
    log(json.dumps({"stream_floor": rf["stream_floor"]}))
    if not args.no_cpu and w.kind == "csa_decode":
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
