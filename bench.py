"""Decode throughput of the staged path on one MI355X.

Workload: the dense 8B-class slice (bf16 weights ~N(0, 0.02), f32 hidden;
8 layers, n_embd 4096, 32 q / 8 kv heads of 128, SwiGLU 14336, vocab 32000),
batch-1 greedy decode with a seeded 4096-row random bf16 KV prefix per layer,
split into N = 4 stages (even split) on one GPU, deferred logits readback.
A step is one token through all four stages and the LM head (+ argmax on the
device, which feeds the next step's embedding).  By default the whole step is
captured once as a graph and replayed (position, step and next id advanced on
the device); --mode eager launches every kernel from the host instead.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--mode graph|eager] [--no-cpu]

Prints one JSON line: decode tokens/s, the algorithmic HBM bytes per token
turned into GB/s and a fraction of MI355X's 8 TB/s, the dominant kernel's
roofline (timed with HIP events on its own stream during a measured pass),
and the float64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import platform
import sys
import time
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, vendor figure
METRIC = "decode tokens/s + achieved HBM GB/s (% of MI355X peak), 1 GPU"


def algorithmic_bytes(cfg, n_rows: int) -> dict:
    """Bytes one decode step must move at context n_rows (rows visible after
    the append): every weight once, every visible K/V row once, the appended
    rows, the embedding row and the logits."""
    d, hd, ff = cfg.d, cfg.hd, cfg.ff
    wb = 2  # bf16
    per_layer_w = ((cfg.nq + 2 * cfg.nkv) * hd * d + d * cfg.nq * hd + 2 * ff * d + d * ff) * wb
    norms = 2 * d * 4
    kv_read = 2 * cfg.nkv * n_rows * hd * 2
    kv_write = 2 * cfg.nkv * hd * 2
    head = cfg.vocab * d * wb + d * 4
    return {
        "weights": cfg.n_layers * (per_layer_w + norms) + head,
        "kv": cfg.n_layers * (kv_read + kv_write),
        "io": d * wb + cfg.vocab * 4,
    }


# HBM traffic of the gate/up GEMVs measured by rocprofv3 PMC counters (FETCH_SIZE,
# WRITE_SIZE, KiB per dispatch, median over the run's dispatches) on
# `python bench.py --no-cpu --mode eager --steps 8 --warmup 2` (dense), `--config pad
# --steps 8` and `--config moe --steps 8`, scaled by what the same counters read for the
# 256 MiB calibration copy (`python bench.py --copy-calibration`: FETCH x 2.0, WRITE x 1.0).
# Valid only for the kernel sources they were taken on (hash below); otherwise null.
GEMV_TRAFFIC = {"src_sha256_16": "90c8c7f3295ba221", "fetch_scale": 2.0, "write_scale": 1.0,
                "dense": (114865.5, 56.4), "pad": (46631.5, 68.3), "moe": (36900.4, 72.0)}
GEMV_SOURCES = ("layer_pipeline_stage_amd/csrc/gemv.hip", "layer_pipeline_stage_amd/csrc/gemv_core.h",
                "layer_pipeline_stage_amd/csrc/dev.h")


def gateup_traffic(which="dense"):
    """Counter-measured HBM bytes of one gate/up launch of the named workload, or None
    when the GEMV sources have changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    t = GEMV_TRAFFIC
    if h.hexdigest()[:16] != t["src_sha256_16"]:
        return None
    fetch, write = t[which]
    return int(1024 * (fetch * t["fetch_scale"] + write * t["write_scale"]))


def gateup_bytes(cfg) -> int:
    """The fused RMSNorm + gate/up GEMV + SwiGLU kernel: its weights once, x and
    the norm gain in, the SwiGLU output out."""
    return 2 * cfg.ff * cfg.d * 2 + 2 * cfg.d * 4 + cfg.ff * 4


KERNEL_BYTES = {
    "qkv": lambda c, n: (c.nq + 2 * c.nkv) * c.hd * c.d * 2 + 2 * c.d * 4 + c.nq * c.hd * 4
    + 2 * c.nkv * c.hd * 2,
    "attn": lambda c, n: 2 * c.nkv * n * c.hd * 2 + 2 * c.nq * c.hd * 4,
    "oproj": lambda c, n: c.d * c.nq * c.hd * 2 + c.nq * c.hd * 4 + 2 * c.d * 4,
    "gateup": lambda c, n: gateup_bytes(c),
    "down": lambda c, n: c.d * c.ff * 2 + c.ff * 4 + 2 * c.d * 4,
    "head": lambda c, n: c.vocab * c.d * 2 + 2 * c.d * 4 + c.vocab * 4,
}


def hbm_achievable_gbs(torch, lps, gib=4, reps=10):
    """Read bandwidth this GPU actually reaches: lps_hbm_stream_read (16-byte
    nontemporal loads, the GEMVs' pattern) over a 4 GiB buffer, 10 launches timed
    with events on the launching stream."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    sink = torch.empty(lps.STREAM_SINK, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    for _ in range(2):
        lps.lps_hbm_stream_read(buf.data_ptr(), n, sink.data_ptr(), st.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        lps.lps_hbm_stream_read(buf.data_ptr(), n, sink.data_ptr(), st.cuda_stream)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    torch.cuda.empty_cache()
    return n / (ms * 1e-3) / 1e9


def cpu_baseline(model, first_token, n_steps=6):
    """The float64 oracle as it is, on this host, on the first n_steps of the
    same greedy run (teacher-forced to the GPU's tokens is not needed: the
    oracle's own greedy steps are the same work)."""
    import threadpoolctl  # noqa: F401  (present in the image; reports BLAS threads)
    from threadpoolctl import threadpool_info

    from oracle.decoder import Decoder
    cores = len(os.sched_getaffinity(0))
    dec = Decoder(model, weight_cache=False)
    t0 = time.perf_counter()
    dec.greedy([first_token], n_steps - 1)
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return {
        "value": round(n_steps / dt, 4), "unit": "tok/s", "cores": int(blas[0]) if blas else cores,
        "kind": "oracle",
        "sample": f"{n_steps} greedy decode steps of the same workload at context 4096 "
                  f"(numpy float64, BLAS threads {blas[0] if blas else '?'} of {cores} host cores, "
                  f"{dt:.1f} s)",
        "cpu": platform.processor() or _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(torch, fn):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def _kernel_times(lps, kind, cap, run):
    """Durations (ms) of every launch of one kind during run(), HIP events on the
    kernels' own stream."""
    lps.lps_timer_start(kind, cap)
    run()
    return lps.timer_stop()


def _roofline(bound, kernel, nbytes_or_flops, avg_us, peak, unit, traffic=None, **extra):
    achieved = nbytes_or_flops / (avg_us * 1e-6) / (1e9 if unit == "GB/s" else 1e12)
    out = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 1), "peak": peak,
           "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
           "avg_us": round(avg_us, 2)}
    out.update(extra)
    return out


def _cpu_info(dt, what):
    from threadpoolctl import threadpool_info
    cores = len(os.sched_getaffinity(0))
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return int(blas[0]) if blas else cores, (f"{what} (numpy float64, BLAS threads "
                                             f"{blas[0] if blas else '?'} of {cores} host cores, "
                                             f"{dt:.1f} s)")


def mx_bytes(n, k):
    """Bytes of an MXFP4 [n, k] matrix: k/2 code bytes and k/32 scale bytes per row."""
    return n * k // 2 + n * k // 32


PAD_KERNEL_BYTES = {
    "qkv": lambda c, n: mx_bytes((c.nq + 2 * c.nkv) * c.hd, c.d) + 2 * c.d * 4 + c.nq * c.hd * 4
    + 2 * c.nkv * c.hd * 2,
    "attn": lambda c, n: 2 * c.nkv * n * c.hd * 2 + 2 * c.nq * c.hd * 4,
    "oproj": lambda c, n: mx_bytes(c.d, c.nq * c.hd) + c.nq * c.hd * 4 + 2 * c.d * 4,
    "gateup": lambda c, n: mx_bytes(2 * c.ff, c.d) + 2 * c.d * 4 + c.ff * 4,
    "down": lambda c, n: mx_bytes(c.d, c.ff) + c.ff * 4 + 2 * c.d * 4,
}


def pad_bench(torch, synth, lps, runtime, steps, cpu=True):
    """Padded-head MXFP4 decode (4 layers, n_embd 5120, 36 q / 6 kv heads of 256 of
    which 12 q and 2 kv are zero dummies, ff 17472, context 8192): `steps` hidden
    rows in and out, device-resident, one stage and two; the gate/up GEMV's
    roofline from a measured pass; the oracle on 4 steps."""
    cfg = replace(synth.PAD, steps=steps)
    model = synth.make_pad(cfg)
    xs = np.asarray(model["x_in"], np.float32)
    c = cfg
    per_tok = c.n_layers * (mx_bytes((c.nq + 2 * c.nkv) * c.hd, c.d) + mx_bytes(c.d, c.nq * c.hd) +
                            mx_bytes(2 * c.ff, c.d) + mx_bytes(c.d, c.ff)) + \
        c.n_layers * 2 * c.nkv * c.hd * 2 * (c.prefix + steps / 2)
    out = {"metric": "decode tokens/s + achieved HBM GB/s (% of MI355X peak), 1 GPU",
           "unit": "tok/s", "n_gpus": 1, "steps": steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "mxfp4 weights, bf16 KV, f32 activations", "data": "synthetic",
           "hbm_bytes_per_token": int(per_tok), "rows": []}
    for fence in ([0, 4], [0, 2, 4]):
        dd = runtime.DeviceDecoder(model, fence=fence, streams="single")
        dd.run_hidden(xs[:4])
        dd.reset()
        dt_eager = _timed(torch, lambda: dd.run_hidden(xs)) / steps
        dd.reset()
        dd.run_hidden_graph(xs[:4])
        dd.reset()
        clock = {}
        dd.run_hidden_graph(xs, timer=lambda start: clock.__setitem__("t0" if start else "t1",
                                                                        time.perf_counter()))
        dt_graph = (clock["t1"] - clock["t0"]) / steps
        dt = dt_eager        # the faster launch form here: the step is kernel-bound
        if len(fence) == 2:
            kernels = {}
            rows = [c.prefix + 1 + i for i in range(steps)]
            for name, kind in lps.KINDS.items():
                if name == "head":
                    continue
                dd.reset()
                ms = _kernel_times(lps, kind, 8 * steps + 8, lambda: dd.run_hidden(xs))
                n_rows = np.repeat(rows, c.n_layers)[:len(ms)]
                byts = np.array([PAD_KERNEL_BYTES[name](c, n) for n in n_rows], np.float64)
                kernels[name] = {"launches": len(ms), "avg_us": round(1e3 * float(np.mean(ms)), 2),
                                 "gbs": round(float(np.sum(byts) / (np.sum(ms) * 1e-3) / 1e9), 1)}
            out["kernels"] = kernels
        dd.close()
        out["rows"].append({"stages": len(fence) - 1, "value": round(1 / dt, 1),
                            "us_per_token": round(1e6 * dt, 2),
                            "hbm_gbs": round(per_tok / dt / 1e9, 1),
                            "hbm_frac": round(per_tok / dt / 1e9 / HBM_PEAK_GBS, 4),
                            "graph_value": round(1 / dt_graph, 1)})
    out["value"] = out["rows"][0]["value"]
    out["ms_per_step"] = round(1e-3 * out["rows"][0]["us_per_token"], 4)
    out["hbm_gbs"] = out["rows"][0]["hbm_gbs"]
    out["hbm_frac"] = out["rows"][0]["hbm_frac"]
    g = out["kernels"]["gateup"]
    out["roofline"] = _roofline("hbm", "rmsnorm + MXFP4 gate/up GEMV + SwiGLU ([34944, 5120], "
                                "e2m1 + e8m0 per 32)", PAD_KERNEL_BYTES["gateup"](c, 0),
                                g["avg_us"], HBM_PEAK_GBS, "GB/s", traffic=gateup_traffic("pad"),
                                bytes_per_launch=PAD_KERNEL_BYTES["gateup"](c, 0))
    out["config"] = {"workload": "padded-head MXFP4 decode: 4 layers, n_embd 5120, 36 q / 6 kv "
                                 "heads of 256 (12 q, 2 kv zero dummies), ff 17472, MXFP4 weights, "
                                 f"context 8192 + {steps} steps, hidden rows in and out "
                                 "(timed including the per-step row copies, excluding the "
                                 "final host readback), eager launches (the whole step as one "
                                 "replayed hipGraph beside it: graph_value), 1 stage (a 2-stage "
                                 "row beside it)",
                     "mode": "eager"}
    if cpu:
        from oracle.decoder import Decoder
        dec = Decoder(model, weight_cache=False)
        n = 4
        t0 = time.perf_counter()
        for t in range(n):
            dec.step(xs[t], c.prefix + t)
        dt = time.perf_counter() - t0
        cores, sample = _cpu_info(dt, f"{n} decode steps of the same padded model at context 8192")
        out["cpu_baseline"] = {"value": round(n / dt, 4), "unit": "tok/s", "cores": cores,
                               "kind": "oracle", "sample": sample}
    return out


def moe_bench(torch, synth, lps, runtime, steps, cpu=True):
    """The MoE layer stack (4 layers, n_embd 2048, 64 experts top-8 + 1 shared, ff
    1024): batch-1 decode of `steps` rows (its expert gate/up GEMV's roofline),
    then the 16,384-token prefill chunk in 8 pieces (both halves of the piece
    transfer; MFMA utilisation of the chunk and of each grouped GEMM launch);
    the oracle on 16 decode steps and a 1,024-token prefill slice."""
    cfg = replace(synth.MOE, steps=steps)
    model = synth.make_moe(cfg)
    st = runtime.DeviceMoEStack(model)
    xs = np.asarray(model["x_in"], np.float32)
    st.decode(xs[:4])
    dt_eager = _timed(torch, lambda: st.decode(xs)) / steps
    st.decode_graph(xs[:4])
    clock = {}
    st.decode_graph(xs, timer=lambda start: clock.__setitem__("t0" if start else "t1",
                                                              time.perf_counter()))
    dt_graph = (clock["t1"] - clock["t0"]) / steps
    dt = dt_eager            # the faster launch form here: the step is kernel-bound
    c = cfg
    k1 = c.top_k + 1
    per_tok = c.n_layers * (k1 * 3 * c.ff * c.d * 2 + c.n_experts * c.d * 2)
    gu_bytes = k1 * 2 * c.ff * c.d * 2 + 2 * c.d * 4 + k1 * c.ff * 4
    dn_bytes = k1 * c.d * c.ff * 2 + k1 * c.ff * 4 + k1 * c.d * 4
    kernels = {}
    for name, kind, nb in (("moe_gateup", 7, gu_bytes), ("moe_down", 8, dn_bytes)):
        ms = _kernel_times(lps, kind, 8 * steps + 8, lambda: st.decode(xs))
        avg = 1e3 * float(np.mean(ms))
        kernels[name] = {"launches": len(ms), "avg_us": round(avg, 2),
                         "gbs": round(nb / (avg * 1e-6) / 1e9, 1)}
    X = np.asarray(model["x_prefill"], np.float32)
    T = X.shape[0]
    xdev = runtime.to_dev(X, "cuda:0")
    st._prefill_scratch(T)
    rs = torch.cuda.Stream()
    times = []
    for _ in range(3):
        x = xdev.clone()
        times.append(_timed(torch, lambda: st.prefill_dev(x, T, 8, rs)))
    tp = min(times[1:])
    flop = 7.44e12 * T / 16384
    # per launch, on one stream (the halves one after the other): algorithmic flops
    # of each grouped GEMM over its launch time
    g1 = _kernel_times(lps, 9, 64, lambda: st.prefill_dev(xdev.clone(), T, 8, st.stream))
    g2 = _kernel_times(lps, 10, 64, lambda: st.prefill_dev(xdev.clone(), T, 8, st.stream))
    gemm_flop = {"moe_gemm1": 2.0 * (T * c.top_k + T) * 2 * c.ff * c.d,
                 "moe_gemm2": 2.0 * (T * c.top_k + T) * c.ff * c.d}
    for name, ms in (("moe_gemm1", g1), ("moe_gemm2", g2)):
        # 2 launches per layer (remote half, then local + shared): their durations
        # summed per layer carry the layer's flops
        per_layer = [ms[i] + ms[i + 1] for i in range(0, len(ms) - 1, 2)]
        avg = 1e3 * float(np.mean(per_layer))
        kernels[name] = {"launches": len(ms), "avg_us_per_layer": round(avg, 2),
                         "tflops": round(gemm_flop[name] / (avg * 1e-6) / 1e12, 1),
                         "mfma_frac": round(gemm_flop[name] / (avg * 1e-6) / 1e12 / 2500.0, 4)}
    out = {"metric": "decode tokens/s + achieved HBM GB/s (% of MI355X peak), 1 GPU",
           "value": round(1 / dt, 1), "unit": "tok/s", "n_gpus": 1, "steps": steps,
           "ms_per_step": round(1e3 * dt, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "us_per_token": round(1e6 * dt, 2),
           "graph_value": round(1 / dt_graph, 1),
           "hbm_bytes_per_token": int(per_tok), "hbm_gbs": round(per_tok / dt / 1e9, 1),
           "hbm_frac": round(per_tok / dt / 1e9 / HBM_PEAK_GBS, 4),
           "roofline": _roofline("hbm", "rmsnorm + gate/up GEMV + SwiGLU of the 8 selected "
                                 "experts and the shared one (9 x [2048, 2048] bf16)", gu_bytes,
                                 kernels["moe_gateup"]["avg_us"], HBM_PEAK_GBS, "GB/s",
                                 traffic=gateup_traffic("moe"), bytes_per_launch=gu_bytes),
           "kernels": kernels,
           "prefill": {"tokens": T, "ms": round(1e3 * tp, 3), "tok_s": round(T / tp, 1),
                       "tflops": round(flop / tp / 1e12, 1),
                       "mfma_frac": round(flop / tp / 1e12 / 2500.0, 4), "pieces": 8,
                       "roofline": {"bound": "mfma", "kernel": "the whole chunk (grouped GEMMs, "
                                    "router, grouping, halves, combine)",
                                    "achieved": round(flop / tp / 1e12, 1), "peak": 2500.0,
                                    "unit": "TFLOP/s", "frac": round(flop / tp / 1e12 / 2500.0, 4),
                                    "traffic": None}},
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "MoE layer stack: 4 layers, n_embd 2048, 64 experts top-8 "
                                  "+ 1 shared, ff 1024, bf16; decode rows device-resident, "
                                  "eager launches (the whole step as one replayed hipGraph "
                                  "beside it: graph_value); prefill chunk 16,384 tokens, FP16 "
                                  "sums and bf16 activations in 8 pieces on a second stream",
                      "mode": "eager"}}
    st.close()
    if cpu:
        from oracle.moe import MoEStack
        ref = MoEStack(model)
        n = 16
        t0 = time.perf_counter()
        for t in range(n):
            ref.forward(xs[t % len(xs)])
        dt_dec = time.perf_counter() - t0
        Tp = 1024
        t0 = time.perf_counter()
        ref.forward(X[:Tp], prefill=True, n_pieces=8)
        dt_pf = time.perf_counter() - t0
        cores, sample = _cpu_info(dt_dec + dt_pf, f"{n} decode steps and a {Tp}-token prefill "
                                  "slice of the same MoE stack")
        out["cpu_baseline"] = {"value": round(n / dt_dec, 4), "unit": "tok/s", "cores": cores,
                               "kind": "oracle", "sample": sample,
                               "prefill_tok_s": round(Tp / dt_pf, 1)}
    return out


def prefill_bench(torch, synth, lps, runtime, T, stages, streams, reps, chunk=None):
    """The dense slice's prompt path: a T-token chunk through the stages (bf16
    GEMMs and causal attention on the matrix cores) after the 4096-row prefix,
    timed from the first embedding to the last stage's output on the device
    (reps runs after one warmup; the caches are reset between runs, untimed)."""
    cfg = replace(synth.DENSE8B, prompt=T, steps=0)
    model = synth.make_dense(cfg)
    dd = runtime.DeviceDecoder(model, fence=lps.stage_plan(cfg.n_layers, stages), streams=streams)
    ids = [int(t) for t in model["prompt"]]
    dd.prefill(ids, chunk=chunk)
    times = []
    for _ in range(reps):
        dd.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dd.prefill(ids, chunk=chunk, hidden=False)   # ends with a device sync and the logits readback
        times.append(time.perf_counter() - t0)
    dd.close()
    dt = min(times)
    c = cfg
    wparams = (c.nq + 2 * c.nkv) * c.hd * c.d + c.d * c.nq * c.hd + 2 * c.ff * c.d + c.d * c.ff
    gemm = 2.0 * T * wparams * c.n_layers
    attn = 4.0 * c.n_layers * c.nq * c.hd * sum(c.prefix + t + 1 for t in range(T))
    return {"metric": "prefill tokens/s (chunked prompt through the stages), 1 GPU",
            "value": round(T / dt, 1), "unit": "tok/s", "ms_per_chunk": round(1e3 * dt, 3),
            "tflops": round((gemm + attn) / dt / 1e12, 1), "gemm_tflop": round(gemm / 1e12, 3),
            "attn_tflop": round(attn / 1e12, 3), "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"dense 8B-class slice prefill: {T}-token prompt "
                                   f"in chunks of {chunk or T} after a "
                                   f"4096-row prefix, {stages} stages ({streams} "
                                   f"stream{'s' if streams == 'per-stage' else ''}), bf16 "
                                   "matrix-core operands, timed from the host to the last "
                                   "row's logits on the host",
                       "prompt": T, "chunk": chunk or T, "stages": stages}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--stages", type=int, default=4)
    ap.add_argument("--streams", choices=("single", "per-stage"), default="single",
                    help="stage streams: one shared stream (the same-stream seam; greedy "
                         "decode cannot overlap stages) or one stream per stage")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: the whole step captured once and replayed, position and "
                         "next id advanced on the device; eager: every launch from the host")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-steps", type=int, default=6)   # about 10 s of oracle work
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB f32 device copy 8 times (reference for HBM counters)")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="T",
                    help="only time the chunked prefill of a T-token prompt through the stages "
                         "(after the 4096-row prefix) and print one JSON line")
    ap.add_argument("--config", choices=("moe", "pad"), default=None,
                    help="only time another workload and print one JSON line: moe = the MoE "
                         "layer stack (batch-1 decode, then the 16,384-token prefill chunk), "
                         "pad = the padded-head MXFP4 decode at context 8192")
    ap.add_argument("--prefill-chunk", type=int, default=0, metavar="C",
                    help="with --prefill-only: feed the prompt in micro-chunks of C rows (on "
                         "per-stage streams a later stage runs chunk k while stage 0 runs k + 1)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: this path runs on one GPU (stages are streams of that GPU); "
              f"--gpus {a.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from layer_pipeline_stage_amd import lps, runtime

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration:
        n = 64 << 20                                   # 256 MiB of f32
        src = torch.randn(n, device="cuda:0")
        dst = torch.empty_like(src)
        st = torch.cuda.current_stream().cuda_stream
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(8):
            lps.lps_copy_f32(src.data_ptr(), dst.data_ptr(), n, st)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 8
        assert torch.equal(src, dst)
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "launches": 8, "gbs": round(8 * n / dt / 1e9, 1)}))
        return
    if a.config:
        fn = moe_bench if a.config == "moe" else pad_bench
        print(json.dumps(fn(torch, synth, lps, runtime, max(8, a.steps), cpu=not a.no_cpu)),
              flush=True)
        return
    if a.prefill_only:
        print(json.dumps(prefill_bench(torch, synth, lps, runtime, a.prefill_only, a.stages,
                                       a.streams, max(1, a.steps), a.prefill_chunk or None)),
              flush=True)
        return
    K, W = a.steps, a.warmup
    cfg = replace(synth.DENSE8B, steps=max(K, W, 128) - 1)
    t0 = time.perf_counter()
    model = synth.make_dense(cfg)
    t_gen = time.perf_counter() - t0
    fence = lps.stage_plan(cfg.n_layers, a.stages)
    dd = runtime.DeviceDecoder(model, fence=fence, streams=a.streams)
    start_tok = [int(model["prompt"][0])]

    # warmup
    dd.reset()
    dd.run_tokens(start_tok, W - 1)
    # timed region: K steps (the start token + K-1 greedy steps), all on the device,
    # through the host-side readback of every step's id and logits
    dd.reset()
    if a.mode == "graph":
        dd.run_tokens_graph(start_tok, W - 1)
        dd.reset()
        clock = {}

        def timer(start):
            clock["t0" if start else "t1"] = time.perf_counter()

        res = dd.run_tokens_graph(start_tok, K - 1, timer=timer)
        dt = clock["t1"] - clock["t0"]
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = dd.run_tokens(start_tok, K - 1)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    tok_s = K / dt
    # the same graph-mode run with one stream per stage: every boundary hop is the
    # event-ordered send / receive (ev_tx / ev_rx) instead of the same-stream seam
    per_stage = None
    if a.mode == "graph" and a.streams == "single" and a.stages > 1:
        dd._streams_mode = "per-stage"
        dd.set_fence(fence)
        dd.reset()
        dd.run_tokens_graph(start_tok, W - 1)
        dd.reset()
        clock2 = {}
        dd.run_tokens_graph(start_tok, K - 1, timer=lambda st_: clock2.__setitem__(
            "t0" if st_ else "t1", time.perf_counter()))
        dt2 = clock2["t1"] - clock2["t0"]
        per_stage = {"value": round(K / dt2, 2), "ms_per_step": round(1e3 * dt2 / K, 4),
                     "streams": "per-stage", "boundary_hops_per_step": a.stages - 1}
        dd._streams_mode = "single"
        dd.set_fence(fence)
    rows = [cfg.prefix + 1 + i for i in range(K)]
    b = [algorithmic_bytes(cfg, n) for n in rows]
    bytes_tok = sum(x["weights"] + x["kv"] + x["io"] for x in b) / K
    gbs = bytes_tok * tok_s / 1e9

    # per-kernel durations, HIP events on each kernel's own stream, one pass each
    kernels = {}
    for name, kind in lps.KINDS.items():
        dd.reset()
        lps.lps_timer_start(kind, 8 * K + 8)
        dd.run_tokens(start_tok, K - 1)
        ms = lps.timer_stop()
        per = KERNEL_BYTES[name]
        launches_per_step = 1 if name == "head" else cfg.n_layers
        n_rows = np.repeat(rows, launches_per_step)[:len(ms)]
        byts = np.array([per(cfg, n) for n in n_rows], dtype=np.float64)
        avg_us = 1e3 * float(np.mean(ms))
        kernels[name] = {"launches": len(ms), "avg_us": round(avg_us, 2),
                         "gbs": round(float(np.sum(byts) / (np.sum(ms) * 1e-3) / 1e9), 1)}
    gk = kernels["gateup"]
    achieved = gateup_bytes(cfg) / (gk["avg_us"] * 1e-6) / 1e9
    achievable = hbm_achievable_gbs(torch, lps)

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(1e3 * dt / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) bf16 KV prefix, device greedy tokens)",
        "config": {
            "workload": "dense 8B-class slice decode: 8 layers, n_embd 4096, 32q/8kv x 128, "
                        "SwiGLU 14336, vocab 32000, bf16 weights, f32 hidden, KV context 4096 + "
                        f"{K} steps, batch 1, {a.stages} stages (even split) on one GPU "
                        f"({a.streams} stream{'s' if a.streams == 'per-stage' else ''}), "
                        + ("the whole step as one replayed hipGraph, " if a.mode == "graph"
                           else "eager launches, ")
                        + ("per-step deferred logits readback (the step's kernels store its "
                           "logits and id into a pinned host ring, drained by the host "
                           "R steps later)" if a.mode == "graph"
                           else "per-step deferred logits readback (a pinned host ring "
                                "filled on its own stream)"),
            "mode": a.mode,
            "global_batch": 1, "seq_len": cfg.prefix + K, "stages": fence,
        },
        "hbm_bytes_per_token": int(bytes_tok),
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "hbm_achievable_gbs": round(achievable, 1),
        "hbm_frac_of_achievable": round(gbs / achievable, 4),
        "roofline": {
            "bound": "hbm", "kernel": "rmsnorm+gate_up GEMV+SwiGLU (bf16 [28672, 4096])",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": gateup_traffic(),
            "frac_of_achievable": round(achieved / achievable, 4),
            "avg_us": gk["avg_us"], "bytes_per_launch": gateup_bytes(cfg),
        },
        "kernels": kernels,
        "per_stage_streams": per_stage,
        "first_tokens": res.fed[:8],
        "gen_s": round(t_gen, 1),
    }
    dd.close()
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(model, start_tok[0], a.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
