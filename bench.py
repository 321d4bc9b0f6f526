#!/usr/bin/env python3
"""Benchmark of the block-quantized batch-1 decode GEMV on one MI355X.

Headline (the JSON line's ``value``): effective weight GB/s of the Q4_K
batch-1 GEMV on a 14336x4096 matrix (packed bytes / wall time), cold cache:
each step runs on the next of >= 1 GiB of distinct packed copies, so no step
finds its weights in the 256 MB last-level cache.  One step = one GEMV call.
Steps are launched from a HIP graph holding one launch per copy, replayed
back to back, so the figure is the kernels', not the host's launch rate (the
eagerly launched rate is reported next to it).

Also reported (in ``extra``): every GEMV of the four-format comparison
(Q8_0/Q4_0/Q4_1/Q4_K x 4096x4096/14336x4096 x batch 1/8), the low-bit
formats and the RMS-normalising Q4_K GEMV, each timed the same way.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X published HBM3E bandwidth
DENSE_8B_BYTES = 3_925_868_544  # Q4_K bytes of the 8B-class step's linear weights
COLD_BYTES = 1 << 30            # rotate over at least this many bytes of packed copies
COUNTERS_FILE = os.path.join(ROOT, "profiles", "q4k_gemv_14336x4096_counters.txt")
CSRC = os.path.join(ROOT, "block_quantized_decode_qgemv_amd", "csrc")
KERNEL_SOURCES = {"kernel_source_sha256_16": os.path.join(CSRC, "gemv.hip"),
                  "kernel_core_sha256_16": os.path.join(CSRC, "gemv_core.h"),
                  "kernel_dispatch_sha256_16": os.path.join(CSRC, "gemv_dispatch.h")}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    fields = {}
    with open(COUNTERS_FILE, encoding="utf-8") as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if any(fields.get(key) != source_hash(path) for key, path in KERNEL_SOURCES.items()):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Gemv:
    """One GEMV configuration with rotating device copies of its packed weights.

    Launches go straight to the C ABI with precomputed device pointers; timed
    runs replay a HIP graph holding one launch per copy."""

    def __init__(self, torch, qg, fmt, n, k, b, seed, min_bytes, stream, rmsnorm=False):
        import workloads

        self.torch = torch
        self.fmt, self.n, self.k, self.b = fmt, n, k, b
        if fmt == "tern":
            packed = qg.qpack_tern(workloads.ternary_codes(n, k, seed, 1),
                                   workloads.scale_bits_f16((n, k // 128), seed, 2))
        elif fmt in ("bin", "bin8"):
            pack = qg.qpack_bin if fmt == "bin" else qg.qpack_bin8
            packed = pack(workloads.binary_codes(n, k, seed, 1), workloads.scale_bits_f16((n, k // 128), seed, 2))
        else:
            packed = qg.qquant(fmt, workloads.student_t_weights(n, k, seed, n), n_threads=16)
        self.bytes = packed.size
        copies = max(1, -(-min_bytes // self.bytes))
        # the copies are slices of one allocation, 256-byte aligned
        stride = -(-self.bytes // 256) * 256
        self.pool = torch.empty(stride * copies, dtype=torch.uint8, device="cuda")
        src = torch.from_numpy(packed).to("cuda")
        self.w = [self.pool[i * stride:i * stride + self.bytes] for i in range(copies)]
        for t in self.w:
            t.copy_(src)
        del src
        self.x = torch.from_numpy(workloads.normal((b, k), seed, 99)).to("cuda")
        self.y = torch.empty((b, n), device="cuda")
        self.lib = qg.load()
        self.fid = qg.FORMATS[fmt]
        self.wp = [t.data_ptr() for t in self.w]
        self.xp, self.yp = self.x.data_ptr(), self.y.data_ptr()
        # rmsnorm: the same GEMV fed by RMS norm of x (gain gamma, eps 1e-5);
        # "unit": unit gain, the gain folded into the weights (no gamma read)
        self.rmsnorm = rmsnorm
        if rmsnorm:
            self.gamma = torch.from_numpy(1.0 + 0.25 * workloads.normal((k,), seed, 98)).float().to("cuda")
            self.gp = None if rmsnorm == "unit" else self.gamma.data_ptr()
        self.stream = stream
        self.sp = stream.cuda_stream
        self.i = 0
        self.graph = None

    def step(self):
        w = self.wp[self.i % len(self.wp)]
        if self.rmsnorm:
            rc = self.lib.qgemv_rmsnorm(self.fid, w, self.xp, self.gp, 1e-5, self.yp, self.n, self.k, self.b,
                                        self.sp)
        else:
            rc = self.lib.qgemv(self.fid, w, self.xp, self.yp, self.n, self.k, self.b, None, 0, self.sp)
        if rc:
            raise RuntimeError(f"qgemv failed with {rc}")
        self.i += 1

    def capture(self) -> int:
        """A graph with one launch per packed copy, in rotation order."""
        torch = self.torch
        self.i = 0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for _ in range(len(self.wp)):
                self.step()
        self.graph = g
        return len(self.wp)

    def replay(self, reps):
        for _ in range(reps):
            self.graph.replay()

    def timed_replay(self, reps) -> float:
        """Average per-launch time (s) over `reps` graph replays, from HIP events
        recorded on the launch stream."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        self.replay(reps)
        e.record(self.stream)
        e.synchronize()
        return a.elapsed_time(e) * 1e-3 / (reps * len(self.wp))


def graph_time(torch, stream, launches, reps):
    """Capture `launches` (a list of zero-argument callables issuing work on
    `stream`) into one HIP graph; return (seconds per replay, graph)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in launches:
            fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    e.record(stream)
    e.synchronize()
    return a.elapsed_time(e) * 1e-3 / reps, g


def read_probe(torch, qg, stream, head):
    """Streaming-read rate of the library's probe kernel: over the headline's
    rotating copies (same size, same cold cache) and over one 4 GiB buffer."""
    lib = qg.load()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sp = stream.cuda_stream

    def probe(ptr, nbytes):
        return lambda: lib.qg_hbm_read_probe(ptr, nbytes, sink.data_ptr(), sp)

    t, _ = graph_time(torch, stream, [probe(p, head.bytes) for p in head.wp], 20)
    same = head.bytes * len(head.wp) / t / 1e9
    big = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    t_big, _ = graph_time(torch, stream, [probe(big.data_ptr(), big.numel())], 10)
    out = {"same_size_GBps": round(same, 1), "bytes_same_size": head.bytes,
           "large_4GiB_GBps": round(big.numel() / t_big / 1e9, 1)}
    del big
    torch.cuda.empty_cache()
    return out


DENSE_LAYER = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
               ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
DENSE_LAYERS = 32


def dense_step(torch, qg, stream):
    """The 8B-class decode step: 32 layers x 7 Q4_K GEMVs at batch 1, one HIP
    graph.  One layer's weights are drawn and quantized; the 32 layers are
    distinct device copies of it (3.9 GB, far beyond the 256 MB cache, so the
    content repeat does not help the reads).  Also timed with q/k/v and
    gate/up each fused into one matrix (128 launches instead of 224)."""
    import workloads

    lib = qg.load()
    fid = qg.FORMATS["q4_k"]
    sp = stream.cuda_stream
    host = {}
    for j, (name, n, k) in enumerate(DENSE_LAYER):
        host[name] = workloads.student_t_weights_device(n, k, 0, 700 + j).cpu().numpy()
    packed = {name: qg.qquant("q4_k", w, n_threads=16) for name, w in host.items()}
    fused = {"qkv": qg.qquant("q4_k", np.concatenate([host["q"], host["k"], host["v"]]), n_threads=16),
             "gateup": qg.qquant("q4_k", np.concatenate([host["gate"], host["up"]]), n_threads=16)}
    del host
    total = sum(p.size for p in packed.values()) * DENSE_LAYERS
    xs = {4096: workloads.normal_device((1, 4096), 0, 801), 14336: workloads.normal_device((1, 14336), 0, 802)}
    ys = {n: torch.empty((1, n), device="cuda") for n in (1024, 4096, 6144, 14336, 28672)}

    def gemv(w, n, k):
        wp, xp, yp = w.data_ptr(), xs[k].data_ptr(), ys[n].data_ptr()
        return lambda: lib.qgemv(fid, wp, xp, yp, n, k, 1, None, 0, sp)

    dev = [{name: torch.from_numpy(packed[name]).to("cuda") for name, _, _ in DENSE_LAYER} for _ in range(DENSE_LAYERS)]
    launches = [gemv(layer[name], n, k) for layer in dev for name, n, k in DENSE_LAYER]
    t, _ = graph_time(torch, stream, launches, 20)
    del dev, launches
    torch.cuda.empty_cache()
    dev = [{name: torch.from_numpy(p).to("cuda") for name, p in fused.items()} |
           {name: torch.from_numpy(packed[name]).to("cuda") for name in ("o", "down")} for _ in range(DENSE_LAYERS)]
    launches = []
    for layer in dev:
        launches += [gemv(layer["qkv"], 6144, 4096), gemv(layer["o"], 4096, 4096),
                     gemv(layer["gateup"], 28672, 4096), gemv(layer["down"], 4096, 14336)]
    t_fused, _ = graph_time(torch, stream, launches, 20)
    # the same with each layer's two RMS norms folded into the projections
    # they feed (attention norm -> q/k/v, FFN norm -> gate/up)
    gammas = [workloads.normal_device((2, 4096), 0, 900 + j) * 0.25 + 1.0 for j in range(DENSE_LAYERS)]

    def gemv_norm(w, n, k, gamma):
        wp, xp, yp = w.data_ptr(), xs[k].data_ptr(), ys[n].data_ptr()
        gp = None if gamma is None else gamma.data_ptr()
        return lambda: lib.qgemv_rmsnorm(fid, wp, xp, gp, 1e-5, yp, n, k, 1, sp)

    launches = []
    for layer, gm in zip(dev, gammas):
        launches += [gemv_norm(layer["qkv"], 6144, 4096, gm[0]), gemv(layer["o"], 4096, 4096),
                     gemv_norm(layer["gateup"], 28672, 4096, gm[1]), gemv(layer["down"], 4096, 14336)]
    t_norm, _ = graph_time(torch, stream, launches, 20)
    # the gains folded into q/k/v and gate/up (same bytes), unit-gain norms at run time
    launches = []
    for layer in dev:
        launches += [gemv_norm(layer["qkv"], 6144, 4096, None), gemv(layer["o"], 4096, 4096),
                     gemv_norm(layer["gateup"], 28672, 4096, None), gemv(layer["down"], 4096, 14336)]
    t_fold, _ = graph_time(torch, stream, launches, 20)
    del dev, launches, gammas
    torch.cuda.empty_cache()
    return {"layers": DENSE_LAYERS, "bytes": total,
            "launches": DENSE_LAYERS * len(DENSE_LAYER), "step_us": round(t * 1e6, 1),
            "tok_s": round(1.0 / t, 1), "GBps": round(total / t / 1e9, 1),
            "fused_launches": DENSE_LAYERS * 4, "fused_step_us": round(t_fused * 1e6, 1),
            "fused_tok_s": round(1.0 / t_fused, 1), "fused_GBps": round(total / t_fused / 1e9, 1),
            "fused_with_norms_step_us": round(t_norm * 1e6, 1), "fused_with_norms_tok_s": round(1.0 / t_norm, 1),
            "fused_with_folded_norms_step_us": round(t_fold * 1e6, 1),
            "fused_with_folded_norms_tok_s": round(1.0 / t_fold, 1)}


MOE_E, MOE_H, MOE_I, MOE_TOPK, MOE_POOL, MOE_SETS = 512, 4096, 1024, 4, 8, 32


def moe_layer(torch, qg, stream, fmt, t_tokens, norm=False):
    """The MoE layer (512 experts + 1 shared, hidden 4096, intermediate 1024,
    top-4) at T tokens, every expert resident.  Experts are distinct device
    copies of a pool of MOE_POOL drawn experts (the pool repeats every
    MOE_POOL slots; 2-3.6 GB in all, beyond the cache).  MOE_SETS router and
    shared-gate logit sets are drawn; one graph replays a call per set, so
    every call routes anew.  Bytes per call: the distinct experts it touches
    (plus the shared one), gate/up and down.

    norm=True times the layer as a pre-norm block step instead: the router
    projection (Q8_0 [E][H]) fed by the RMS norm of the block input, then the
    expert layer on the normalised input with the block input as residual;
    MOE_SETS input sets, so every call routes anew.  Its bytes add the
    router's."""
    import workloads

    lib = qg.load()
    e_, h_, i_, k_ = MOE_E, MOE_H, MOE_I, MOE_TOPK
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i_, h_), qg.qg_packed_size(fmt, h_, i_)
    gu = torch.empty((e_ + 1) * gu_sz, dtype=torch.uint8, device="cuda")
    dn = torch.empty((e_ + 1) * dn_sz, dtype=torch.uint8, device="cuda")
    pool = []
    for j in range(MOE_POOL):
        wg = workloads.student_t_weights_device(2 * i_, h_, 1, 3 * j).cpu().numpy()
        wd = workloads.student_t_weights_device(h_, i_, 1, 3 * j + 2).cpu().numpy()
        pool.append((torch.from_numpy(qg.qquant(fmt, wg, n_threads=16)).to("cuda"),
                     torch.from_numpy(qg.qquant(fmt, wd, n_threads=16)).to("cuda")))
    for e in range(e_ + 1):
        gu[e * gu_sz:(e + 1) * gu_sz].copy_(pool[e % MOE_POOL][0])
        dn[e * dn_sz:(e + 1) * dn_sz].copy_(pool[e % MOE_POOL][1])
    del pool
    x = workloads.normal_device((t_tokens, h_), 2, 1)
    res = workloads.normal_device((t_tokens, h_), 2, 2)
    logits = [workloads.normal_device((t_tokens, e_), 2, 100 + r) for r in range(MOE_SETS)]
    slog = [workloads.normal_device((t_tokens,), 2, 200 + r) for r in range(MOE_SETS)]
    out = torch.empty((t_tokens, h_), device="cuda")
    ws_bytes = qg.moe_expert_ffn_workspace_size(t_tokens, e_, h_, i_, k_)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    fid, sp = qg.FORMATS[fmt], stream.cuda_stream

    def call(r):
        args = (fid, gu.data_ptr(), dn.data_ptr(), e_, h_, i_, k_, x.data_ptr(), res.data_ptr(),
                logits[r].data_ptr(), slog[r].data_ptr(), t_tokens, 0, out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
        return lambda: lib.moe_expert_ffn(*args)

    router_bytes = 0
    if norm:
        q8 = qg.FORMATS["q8_0"]
        router = torch.from_numpy(qg.qquant("q8_0", workloads.student_t_weights_device(e_, h_, 1, 77).cpu().numpy(),
                                            n_threads=16)).to("cuda")
        router_bytes = router.numel()
        gamma = workloads.normal_device((h_,), 2, 78) * 0.25 + 1.0
        xs = [workloads.normal_device((t_tokens, h_), 2, 300 + r) * 6.0 for r in range(MOE_SETS)]

        gp = None if norm == "unit" else gamma.data_ptr()  # "unit": gains folded into the weights

        def call_norm(r):
            def fn():
                rc = lib.qgemv_rmsnorm(q8, router.data_ptr(), xs[r].data_ptr(), gp, 1e-6,
                                       logits[r].data_ptr(), e_, h_, t_tokens, sp)
                rc = rc or lib.moe_expert_ffn_rmsnorm(fid, gu.data_ptr(), dn.data_ptr(), e_, h_, i_, k_,
                                                      xs[r].data_ptr(), gp, 1e-6, xs[r].data_ptr(),
                                                      logits[r].data_ptr(), slog[r].data_ptr(), t_tokens, 0,
                                                      out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
                if rc:
                    raise RuntimeError(f"MoE block step failed with {rc}")
            return fn

        for r in range(MOE_SETS):
            call_norm(r)()  # the logits the step's routes come from
        torch.cuda.synchronize()
        t, _ = graph_time(torch, stream, [call_norm(r) for r in range(MOE_SETS)], 10)
    else:
        t, _ = graph_time(torch, stream, [call(r) for r in range(MOE_SETS)], 10)
    t /= MOE_SETS
    touched = np.mean([len(set(np.argsort(-lg.cpu().numpy(), axis=1, kind="stable")[:, :k_].ravel().tolist())) + 1
                       for lg in logits])
    nbytes = touched * (gu_sz + dn_sz) + router_bytes
    del gu, dn, ws
    torch.cuda.empty_cache()
    return {"fmt": fmt, "T": t_tokens, "norm_block": {False: False, True: "gain vector", "unit": "gain folded"}[norm],
            "us": round(t * 1e6, 2),
            "experts_touched": round(float(touched), 2),
            "bytes": int(nbytes), "GBps": round(float(nbytes) / t / 1e9, 1)}


def cpu_baseline(seconds=12.0):
    """The oracle (numpy dequant + float64 matvec) on a bounded sample of the
    headline workload: whole 14336x4096 Q4_K GEMVs, repeated for ~seconds."""
    import workloads
    from oracle import formats as OF
    from oracle import gemv as OG

    n, k = 14336, 4096
    w = workloads.student_t_weights(n, k, 0, n)
    packed = OF.quantize_packed("q4_k", w)
    x = workloads.normal((1, k), 0, 99)
    reps = 0
    t_deq = 0.0
    t0 = time.perf_counter()
    while True:
        t1 = time.perf_counter()
        w_deq = OF.dequant_packed("q4_k", packed, n, k)
        t_deq += time.perf_counter() - t1
        OG.gemv_ref(w_deq, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = 1
    try:
        from threadpoolctl import threadpool_info

        threads = max([1] + [int(p.get("num_threads", 1)) for p in threadpool_info()])
    except Exception:
        pass
    return {"value": round(packed.size * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full Q4_K 14336x4096 batch-1 GEMVs (unpack + dequant + float64 matvec), {el:.1f} s; "
                      f"unpack + dequant {100 * t_deq / el:.0f} % of it"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline only, no extra configs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--profile", choices=["gemv", "copy", "probe", "moe", "step", "norm"], default=None,
                    help="run only one part (the headline kernel, a 1 GiB copy, the read probe, the MoE layer, "
                         "the 8B step, or the RMS-norm GEMVs and MoE block step) for rocprofv3")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the GEMV is measured on one GPU's share; no collectives are built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_decode_qgemv_amd as qg

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    qg.load()
    stream = torch.cuda.Stream()  # graphs are captured on a non-default stream
    torch.cuda.set_stream(stream)

    if args.profile == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copied 1 GiB 3 times")
        return

    if args.profile == "moe":
        for fmt in ("q4_k", "q2_k"):
            for t_tokens in (1, 8):
                log(f"moe {moe_layer(torch, qg, stream, fmt, t_tokens)}")
        return
    if args.profile == "norm":
        for n, k in ((14336, 4096), (4096, 4096)):
            for b in (1, 8):
                for norm in (False, True, "unit"):
                    g = Gemv(torch, qg, "q4_k", n, k, b, 0, COLD_BYTES, stream, norm)
                    g.capture()
                    g.replay(2)
                    t = g.timed_replay(max(2, 400 // len(g.wp)))
                    log(f"q4_k {n}x{k} B={b} rmsnorm={norm}: {t * 1e6:.2f} us")
                    del g
                    torch.cuda.empty_cache()
        for t_tokens in (1, 8):
            log(f"moe block {moe_layer(torch, qg, stream, 'q4_k', t_tokens, norm=True)}")
        return
    if args.profile == "step":
        log(f"step {dense_step(torch, qg, stream)}")
        return

    log("setup: Q4_K 14336x4096 batch 1, rotating copies")
    head = Gemv(torch, qg, "q4_k", 14336, 4096, 1, 0, COLD_BYTES, stream)
    if args.profile == "gemv":
        for _ in range(40):
            head.step()
        torch.cuda.synchronize()
        log("ran 40 headline GEMVs")
        return
    if args.profile == "probe":
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        for p in head.wp:
            qg.qg_hbm_read_probe(p, head.bytes, sink, stream)
        torch.cuda.synchronize()
        log(f"ran {len(head.wp)} read probes")
        return

    per = head.capture()
    reps_warm = max(1, args.warmup // per)
    reps = max(1, args.steps // per)
    steps = reps * per
    head.replay(reps_warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    head.replay(reps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = head.bytes * steps / wall / 1e9
    log(f"headline: {value:.1f} GB/s over {steps} steps ({reps} graph replays of {per} launches)")

    t_launch = head.timed_replay(reps)
    achieved = head.bytes / t_launch / 1e9
    # traffic: counter-measured HBM bytes per launch over the same launch time,
    # in the unit of `achieved` (so traffic / achieved = measured / algorithmic bytes)
    hbm_bytes = read_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if hbm_bytes is None else round(hbm_bytes / t_launch / 1e9, 1)}

    # eager launches (host-issued one by one), for reference
    for _ in range(50):
        head.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(500):
        head.step()
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t1) / 500 * 1e6

    extra = {"headline_us_per_launch": round(t_launch * 1e6, 3),
             "headline_eager_us_per_launch": round(eager_us, 3),
             "tok_s_equiv": round(achieved * 1e9 / DENSE_8B_BYTES, 1),
             "headline_algorithmic_bytes": head.bytes,
             "headline_hbm_bytes_counted": hbm_bytes}
    if not args.quick:
        def measure(fmt, n, k, b, rmsnorm=False):
            g = Gemv(torch, qg, fmt, n, k, b, 0, COLD_BYTES, stream, rmsnorm)
            g.capture()
            g.replay(2)
            t = g.timed_replay(max(2, 400 // len(g.wp)))
            nbytes = g.bytes
            del g
            torch.cuda.empty_cache()
            return t, nbytes

        rows = []
        for fmt in ("q8_0", "q4_0", "q4_1", "q4_k"):
            for n, k in ((4096, 4096), (14336, 4096)):
                for b in (1, 8):
                    t, nbytes = measure(fmt, n, k, b)
                    rows.append({"fmt": fmt, "N": n, "K": k, "B": b, "us": round(t * 1e6, 2),
                                 "GBps": round(nbytes / t / 1e9, 1)})
                    log(f"  {fmt} {n}x{k} B={b}: {t*1e6:.2f} us, {nbytes/t/1e9:.1f} GB/s")
        extra["four_formats"] = rows
        rows = []
        for fmt in ("tern", "bin", "bin8", "q2_k"):
            for n, k in ((4096, 4096), (12288, 4096), (4096, 12288)):
                for b in (1, 4):
                    t, nbytes = measure(fmt, n, k, b)
                    rows.append({"fmt": fmt, "N": n, "K": k, "B": b, "us": round(t * 1e6, 2),
                                 "GBps": round(nbytes / t / 1e9, 1), "Gweights_s": round(n * k * b / t / 1e9, 1)})
                    log(f"  {fmt} {n}x{k} B={b}: {t*1e6:.2f} us, {nbytes/t/1e9:.1f} GB/s")
        extra["low_bit"] = rows
        rows = []
        for gain in (True, "unit"):
            for n, k in ((14336, 4096), (4096, 4096)):
                for b in (1, 8):
                    t, nbytes = measure("q4_k", n, k, b, rmsnorm=gain)
                    rows.append({"fmt": "q4_k", "N": n, "K": k, "B": b, "gain": "folded" if gain == "unit" else "vector",
                                 "us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1)})
                    log(f"  rmsnorm ({rows[-1]['gain']} gain) + q4_k {n}x{k} B={b}: {t*1e6:.2f} us, "
                        f"{nbytes/t/1e9:.1f} GB/s")
        extra["rmsnorm_gemv"] = rows
        log("8B decode step (32 layers x 7 Q4_K GEMVs)")
        extra["dense_8b_step"] = dense_step(torch, qg, stream)
        log(f"  {extra['dense_8b_step']}")
        rows = []
        for fmt in ("q4_k", "q2_k"):
            for t_tokens in (1, 8):
                rows.append(moe_layer(torch, qg, stream, fmt, t_tokens))
                log(f"  moe {rows[-1]}")
        for norm in (True, "unit"):
            for t_tokens in (1, 8):
                rows.append(moe_layer(torch, qg, stream, "q4_k", t_tokens, norm=norm))
                log(f"  moe {rows[-1]}")
        extra["moe_layer"] = rows
    extra["hbm_read_probe"] = read_probe(torch, qg, stream, head)
    extra["headline_frac_of_read_probe"] = round(achieved / extra["hbm_read_probe"]["same_size_GBps"], 4)
    log(f"  read probe {extra['hbm_read_probe']}")

    line = {
        "metric": "Q4_K batch-1 GEMV effective weight GB/s and % of HBM peak; tok/s-equiv",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": reps_warm * per,
        "ms_per_step": round(wall / steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Q4_K GEMV 14336x4096, batch 1, Student-t(5)*0.02 weights, N(0,1) x, "
                               "cold cache (rotating >= 1 GiB of packed copies), HIP-graph launches",
                   "format": "q4_k", "N": 14336, "K": 4096, "batch": 1, "parallelism": "none"},
        "roofline": roofline,
        "extra": extra,
    }
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
