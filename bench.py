"""Benchmark: one MLA decode step on one MI355X (gfx950).

A step is one pass of the whole hot path over one batch: one
mla_decode_paged call that first appends the new token of every sequence
(RoPE on its key, in the same launch as the absorb GEMM), then runs the
split-KV flash decode over the latent+RoPE cache, the merge of the splits and
the W_UV projection. Workload: 64 sequences, 128 heads, 4096
cached tokens each (the new one included), DeepSeek-V3 widths, bf16, paged
cache of 64-token blocks placed by a seeded random permutation.

Inputs are resident in HBM before the timed region. Steps cycle over three
independent layers (own weights, queries and cache, ~1 GB in total) so that
a step never finds its cache in the 256 MB last-level cache left by the
previous step, as in a real model where the other layers run in between.

Prints ONE JSON line (see the fields below). Options:
  --steps K --warmup W     timed and untimed steps (defaults 1000 / 300: the
                           GPU reaches its steady-state speed only after a few
                           hundred steps; before, steps run ~15 % slower)
  --gpus N                 only N = 1 is supported (one process, one GPU)
  --no-cpu                 skip the CPU-oracle baseline leg
  --config NAME            3u (default), 3, 4 or 5 (other workloads, for study)
  --separate-append        append with its own mla_cache_append call before the
                           decode call (same work, one more launch)
  --copy-calibration MIB   only run a plain device-to-device copy of MIB MiB
                           five times (the reference kernel that scales the
                           HBM byte counters of a profiler run) and exit
  --length-aware           the decode calls cut the sequences by their actual
                           lengths (mla_decode_options.length_aware)
  --clock SECONDS          after the timed steps, run the same steps for about
                           SECONDS more while a host thread samples the shader
                           clock through amdsmi (reported as "shader_clock")
  --stream-read MIB        only measure the plain streaming-read rate of the
                           device on MIB MiB (calibration kernel) and exit
  --with-projection        the step also computes the new rows from the tokens'
                           hidden states (d_model 7168): mla_project, then the
                           decode call appends from its workspace (with
                           --separate-append: mla_project_append, then a decode
                           call without append)
  --project                only measure mla_project_append (the down-projection
                           of 64 new tokens' hidden states, d_model 7168, bf16,
                           and the append of their rows) and print its own line
  --write-traffic F W CF CW  only turn four rocprofv3 counter CSVs (decode
                           kernel FETCH_SIZE, WRITE_SIZE; copy FETCH_SIZE,
                           WRITE_SIZE, taken with --copy-calibration 1024)
                           into profiles/<kernel>_<config>_traffic.json (with
                           --project: the two kernels of mla_project_append,
                           summed per call)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + latent-cache HBM GB/s (% of peak), B=64 H=128 N=4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
N_LAYERS_CYCLED = 3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--config", default="3u", choices=["1", "2", "3", "3u", "4", "5"])
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--separate-append", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--stream-read", type=int, default=0, metavar="MIB")
    ap.add_argument("--write-traffic", nargs=4, default=None)
    ap.add_argument("--write-mfma", nargs=2, default=None, metavar=("COUNTERS_CSV", "TRACE_CSV"))
    ap.add_argument("--project", action="store_true")
    ap.add_argument("--prefill", action="store_true")
    ap.add_argument("--fused", action="store_true")
    ap.add_argument("--restart", action="store_true")
    ap.add_argument("--with-projection", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from HIP graphs (one per layer)")
    ap.add_argument("--length-aware", action="store_true",
                    help="decode calls use the length-aware split plan (bf16 cache)")
    ap.add_argument("--clock", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, run the same steps for about SECONDS more "
                         "while a host thread samples the GPU's shader clock (amdsmi)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t pairs from libamdhip64 (the decode call records them around
    the split attention kernel on its own stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


# the files whose text defines the split attention kernels (the launch code
# in mla_api.hip only passes them their parameters), and the down-projection's
KERNEL_SOURCES = ("common.hpp", "decode_mfma.hpp")
# sources per attention kernel (the fp8 matrix-core kernel builds on the
# decode kernels' header)
SOURCES_OF = {"mla_decode_fp8mma_kernel": ("common.hpp", "decode_mfma.hpp", "decode_fp8mma.hpp")}


def sources_of(kernel: str):
    return SOURCES_OF.get(kernel, KERNEL_SOURCES)
PROJECT_SOURCES = ("common.hpp", "append.hpp", "kv_project.hpp")
PROJECT_KERNELS = ("mla_kv_project_kernel", "mla_project_append_kernel")
PROJECT_WORKLOAD = "b64_d7168_bf16"


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "head_latent_attention_07_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, per_launch_bytes: float, kernel="mla_decode_bf16_kernel",
                     sources=None):
    """HBM bytes per launch of the measured kernel(s) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(sources or sources_of(kernel)):
        return None
    return t.get("hbm_bytes_per_launch")


def _host_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands (float64, non-absorbed), on a bounded sample of
    the same workload: whole sequences (all heads) until `seconds` elapse."""
    import numpy as np
    import torch
    import synth
    from oracle import mla_oracle as orc
    threads = _host_threads()
    inp = synth.make_inputs(cfg)
    act = "f32" if inp.q_nope.dtype == torch.float32 else "bf16"

    def f64(t, kind):
        return orc.decode_storage(synth.raw_bits(t), kind)

    wuk, wuv = f64(inp.w_uk, act), f64(inp.w_uv, act)
    table = None if inp.block_table is None else inp.block_table.numpy()
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % inp.B
        n = int(inp.lengths[b])
        rows = torch.from_numpy(orc.gather_rows(b, n, seq_capacity=inp.seq_capacity,
                                                block_table=table, block_size=inp.block_size))
        vals = f64(inp.cache[rows], inp.cache_dtype)
        if inp.scales is not None:
            vals = vals * f64(inp.scales[rows], "bf16")[:, None]
        orc.decode(f64(inp.q_nope[b:b + 1], act), f64(inp.q_pe[b:b + 1], act), wuk, wuv,
                   [vals[:, :512]], [vals[:, 512:]], inp.scale)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} sequence(s) x {inp.H} heads of the same workload "
                      f"(N={inp.max_len}), float64 non-absorbed oracle, {dt:.1f} s"}


def cpu_absorbed_f32(cfg, seconds: float):
    """A same-algorithm CPU baseline (not the oracle): the absorbed form in
    float32 on the host cores (torch CPU matrix products, all heads of a
    sequence at once), whole sequences until `seconds` elapse."""
    import torch
    import synth
    inp = synth.make_inputs(cfg)
    threads = torch.get_num_threads()
    wuk, wuv = inp.w_uk.float(), inp.w_uv.float()
    done = 0
    t0 = time.perf_counter()
    while True:
        b = done % inp.B
        n = int(inp.lengths[b])
        if inp.block_table is None:
            rows = b * inp.seq_capacity + torch.arange(n)
        else:
            t = torch.arange(n)
            rows = inp.block_table[b].long()[t // inp.block_size] * inp.block_size + t % inp.block_size
        sel = inp.cache[rows]
        if inp.cache_dtype == "fp8":
            x = sel.view(torch.float8_e4m3fn).float() * inp.scales[rows].float()[:, None]
        else:
            x = sel.float()
        C, R = x[:, :512], x[:, 512:]
        q_lat = torch.einsum("hk,hkc->hc", inp.q_nope[b].float(), wuk)
        S = inp.scale * (C @ q_lat.T + R @ inp.q_pe[b].float().T)
        P = torch.softmax(S, dim=0)
        torch.einsum("hc,hcv->hv", P.T @ C, wuv)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": threads,
            "kind": "absorbed float32 (same algorithm as the GPU path, torch CPU)",
            "sample": f"{done} sequence(s) x {inp.H} heads (N={inp.max_len}), {dt:.1f} s"}


def cpu_baseline_project(seconds: float):
    """The oracle's down-projection and append (float64) on the host cores:
    rows of the --project workload (same shapes, seeds of its first weight
    set) one at a time until `seconds` elapse; the weights are decoded once."""
    import synth
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    h, wd, wk = synth.projection_inputs(9000, 64, "bf16", synth.D_MODEL)

    def f64(t):
        return orc.decode_storage(synth.raw_bits(t), "bf16")

    hh, wdd, wkk = f64(h), f64(wd), f64(wk)
    rows = 0
    t0 = time.perf_counter()
    while True:
        orc.project_append_row(hh[rows % 64], wdd, wkk, 15, "bf16")
        rows += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} rows of the same workload (d_model 7168, bf16 cache), float64 "
                      f"oracle, weights decoded once beforehand, {dt:.1f} s"}


def copy_calibration(mib: int):
    """A plain copy of known size: each launch reads and writes exactly
    mib MiB, so a profiler's HBM read/write counters for it give the factor
    between counted and true bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def stream_read(mib: int):
    """The achievable HBM read rate on this device: a plain streaming read of
    mib MiB (larger than the 256 MB last-level cache) by the calibration
    kernel (libmla_calib.so), timed by events the launch itself records, for
    several grid sizes; 5 untimed then 20 timed launches each. Prints one
    JSON line with the rate per grid and the best."""
    import torch
    from head_latent_attention_07_amd import build as b
    if not os.path.exists(b.CALIB_LIB_PATH):
        raise SystemExit(f"calibration library not built: {b.CALIB_LIB_PATH}")
    lib = ctypes.CDLL(b.CALIB_LIB_PATH)
    lib.mla_calib_stream_read.restype = ctypes.c_int
    lib.mla_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
    n = mib << 20
    buf = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(3)
    grids = (512, 1024, 2048, 4096, 8192)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()
    rates = {}
    for grid in grids:
        for _ in range(5):
            assert lib.mla_calib_stream_read(buf.data_ptr(), n, out.data_ptr(), grid, None, None,
                                             stream) == 0
        pairs = [(ev.create(), ev.create()) for _ in range(20)]
        for a, e in pairs:
            assert lib.mla_calib_stream_read(buf.data_ptr(), n, out.data_ptr(), grid, a, e,
                                             stream) == 0
        torch.cuda.synchronize()
        ms = sorted(ev.elapsed_ms(a, e) for a, e in pairs)
        for a, e in pairs:
            ev.destroy(a)
            ev.destroy(e)
        rates[grid] = {"gbs_mean": n / (sum(ms) / len(ms) * 1e-3) / 1e9,
                       "gbs_median": n / (ms[len(ms) // 2] * 1e-3) / 1e9}
    best = max(r["gbs_mean"] for r in rates.values())
    print(json.dumps({"stream_read_bytes": n, "workgroups_of_256": rates, "best_gbs": best,
                      "frac_of_8000": best / HBM_PEAK_GBS}), flush=True)


def _counter_mean(csv_path: str, kernel_substr: str, counter: str) -> float:
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {csv_path}")
    return sum(vals) / len(vals)


def write_traffic(paths, config: str, kernels, copy_mib: int = 1024, sources=None):
    """HBM bytes per launch of `kernels` (summed: the launches of one call)
    from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    the factor between the true bytes of a plain copy of copy_mib MiB and
    what the same counter reads for it."""
    f, w, cf, cw = paths
    true_kib = copy_mib * 1024.0
    rf = true_kib / _counter_mean(cf, "copyBuffer", "FETCH_SIZE")
    wf = true_kib / _counter_mean(cw, "copyBuffer", "WRITE_SIZE")
    fetch = sum(_counter_mean(f, k, "FETCH_SIZE") for k in kernels) * 1024.0 * rf
    write = sum(_counter_mean(w, k, "WRITE_SIZE") for k in kernels) * 1024.0 * wf
    kernel = kernels[0]
    rec = {"kernel": " + ".join(kernels), "workload": config,
           "kernel_source_hash": kernel_source_hash(sources or sources_of(kernels[0])),
           "read_factor": rf, "write_factor": wf, "hbm_read_bytes_per_launch": fetch,
           "hbm_write_bytes_per_launch": write, "hbm_bytes_per_launch": fetch + write}
    out = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


PROJECT_SETS = 48     # weight sets cycled: ~400 MB, more than the last-level cache


def bench_project(args):
    """Time mla_project_append alone: 64 tokens, d_model 7168, bf16 operands,
    bf16 cache. Each call uses the next of PROJECT_SETS weight/hidden sets so
    that its 8.3 MB of weights come from HBM as in a model whose other layers
    run in between. Algorithmic bytes per call: the weights, the hidden
    states and the written rows."""
    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, D, cap = 64, synth.D_MODEL, 16
    sets = [synth.projection_inputs(9000 + 10 * i, B, "bf16", D, device=dev)
            for i in range(PROJECT_SETS)]
    cache = torch.zeros((B * cap, 576), dtype=torch.bfloat16, device=dev)
    lat, rope = mla.split_cache(cache)
    pos = torch.full((B,), cap - 1, dtype=torch.int32, device=dev)
    ws = torch.empty(mla.project_workspace_size(B, D), dtype=torch.uint8, device=dev)

    def call(i):
        h, wd, wk = sets[i % PROJECT_SETS]
        mla.project_append(h, wd, wk, pos, lat, rope, heads=128, seq_capacity=cap, workspace=ws)

    # A call costs the host more than the GPU, so calls issued one by one
    # leave the GPU idle between them: the calls over all weight sets are
    # captured once in a HIP graph and the graph is replayed (kernels back to
    # back, as in a model's decode step).
    call(PROJECT_SETS - 1)
    torch.cuda.synchronize()
    eager = cache.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(PROJECT_SETS):
            call(i)
    reps = max(1, args.steps // PROJECT_SETS)
    for _ in range(max(1, args.warmup // PROJECT_SETS)):
        graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(cache.view(torch.int16), eager.view(torch.int16)):
        raise RuntimeError("graph replay of mla_project_append differs from the eager call")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    avg_ms = a.elapsed_time(b) / (reps * PROJECT_SETS)
    nbytes = (D_QK_ROWS * D + B * D) * 2 + B * 576 * 2
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    line = {
        "metric": "MLA down-projection + append rows/s (c_KV = W_DKV h, RoPE(W_KR h))",
        "value": B / (avg_ms * 1e-3), "unit": "rows/s", "n_gpus": 1,
        "steps": reps * PROJECT_SETS, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / (reps * PROJECT_SETS),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normals, weights N(0, 1/d_model))",
        "config": {"workload": "mla_project_append_" + PROJECT_WORKLOAD, "B": B, "d_model": D,
                   "weight_sets_cycled": PROJECT_SETS},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(PROJECT_WORKLOAD, nbytes, PROJECT_KERNELS[0],
                                                 PROJECT_SOURCES),
                     "kernel": "mla_kv_project_kernel + mla_project_append_kernel",
                     "bytes_per_launch": nbytes, "avg_launch_us": avg_ms * 1e3},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_project(min(args.cpu_seconds, 10.0))
    print(json.dumps(line), flush=True)


D_QK_ROWS = 576    # rows of W_DKV (512) and W_KR (64)


PREFILL_WORKLOAD = "mla_prefill_b1_t4096_n4096_h128_bf16"


def cpu_baseline_prefill(seconds: float, T: int, heads: int):
    """The oracle's chunked_prefill (float64, recompute form) on the host
    cores: heads of the same 4096-token prompt one at a time until `seconds`
    elapse, scaled to prompt tokens per second (all heads)."""
    import torch
    import synth
    from oracle import mla_oracle as orc
    threads = _host_threads()
    inp = synth.make_inputs(2, B=1, N=T, lengths=torch.tensor([T], dtype=torch.int32))
    qn, qp = synth.prefill_queries(6100, 1, T, heads)

    def f64(t):
        return orc.decode_storage(synth.raw_bits(t), "bf16")

    wuk, wuv, qn64, qp64 = f64(inp.w_uk), f64(inp.w_uv), f64(qn)[0], f64(qp)[0]
    vals = f64(inp.cache[:T])
    C, R = vals[:, :512], vals[:, 512:]
    done = 0
    t0 = time.perf_counter()
    while True:
        h = done % heads
        orc.chunked_prefill(qn64[:, h], qp64[:, h], wuk[h], wuv[h], C, R, inp.scale)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": T / (dt / done * heads), "unit": "prompt tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of the {heads} heads of the same {T}-token prompt, float64 "
                      f"recompute-form oracle, {dt:.1f} s, scaled to all heads"}


def bench_prefill(args):
    """Time mla_prefill on one 4096-token prompt (B=1, T=N=4096, 128 heads,
    bf16): W_UV transpose, decompression of K and V for every head, causal
    attention. The roofline is the attention kernel's against the dense
    matrix-core peak (its operands are fp16, whose peak equals bf16's)."""
    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, H = 1, 4096, 128
    layers = []
    for layer in range(2):
        inp = synth.make_inputs(2, B=B, N=T, H=H, layer=layer,
                                lengths=torch.tensor([T], dtype=torch.int32)).to(dev)
        qn, qp = synth.prefill_queries(6100 + 10 * layer, B, T, H, device=dev)
        lat, rope = mla.split_cache(inp.cache)
        ws = torch.empty(mla.prefill_workspace_size(H, B, T), dtype=torch.uint8, device=dev)
        out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        layers.append(dict(inp=inp, qn=qn, qp=qp, lat=lat, rope=rope, ws=ws, out=out, lse=lse))
    ev = HipEvents()

    def call(L, events=None, expand_events=None):
        inp = L["inp"]
        mla.prefill(L["qn"], L["qp"], inp.w_uk, inp.w_uv, L["lat"], L["rope"], inp.lengths, T,
                    seq_capacity=inp.seq_capacity, out=L["out"], lse=L["lse"], workspace=L["ws"],
                    events=events, expand_events=expand_events)

    for i in range(args.warmup):
        call(layers[i % 2])
    torch.cuda.synchronize()
    pairs = [((ev.create(), ev.create()), (ev.create(), ev.create())) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(layers[i % 2], events=pairs[i][0], expand_events=pairs[i][1])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms = [ev.elapsed_ms(*pr[0]) for pr in pairs]
    exp_ms = [ev.elapsed_ms(*pr[1]) for pr in pairs]
    for pr in pairs:
        for e in pr[0] + pr[1]:
            ev.destroy(e)
    ms = (t1 - t0) * 1e3 / args.steps
    attn_avg = sum(attn_ms) / len(attn_ms)
    exp_avg = sum(exp_ms) / len(exp_ms)
    # causal attention: query i sees i + 1 keys; (192 + 128) x 2 FLOP per
    # (query, key, head); decompression: 2 x 512 x 256 FLOP per (token, head)
    attn_flop = H * (T * (T + 1) // 2) * (192 + 128) * 2
    exp_flop = B * T * H * 512 * 256 * 2
    achieved = attn_flop / (attn_avg * 1e-3) / 1e12
    line = {
        "metric": "MLA prefill prompt tokens/s (recompute mode: decompress K and V, causal attention)",
        "value": B * T / (ms * 1e-3), "unit": "prompt tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (attention operands fp16)",
        "data": "synthetic (seeded normals; random-init weights of the DeepSeek-V3 MLA widths)",
        "config": {"workload": PREFILL_WORKLOAD, "B": B, "T": T, "N": T, "H": H,
                   "d_qk": 192, "d_v": 128},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None, "kernel": "mla_prefill_attn_kernel",
                     "flop_per_launch": attn_flop, "avg_launch_us": attn_avg * 1e3,
                     "launch_us_p10_p50_p90": [percentile(attn_ms, q) * 1e3 for q in (10, 50, 90)]},
        "expand": {"kernel": "mla_prefill_expand_kernel", "flop_per_launch": exp_flop,
                   "avg_launch_us": exp_avg * 1e3,
                   "tflops": exp_flop / (exp_avg * 1e-3) / 1e12,
                   "frac_of_bf16_peak": exp_flop / (exp_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_prefill(min(args.cpu_seconds, 10.0), T, H)
    print(json.dumps(line), flush=True)


def bench_fused(args):
    """Offline absorption decided by measurement: one decode step from the
    tokens' model-width input x (B=64, d_model 7168) to the attention output
    at model width, over the B=64 H=128 N=4096 paged bf16 cache,
      fused:   mla_decode_fused with W_QK = W_UK^T W_Q and W_VO = W_UV W_O
               (mla_fuse_weights, offline);
      unfused: q_nope = x W_Q^T and y = o W_O as library GEMMs (torch.matmul)
               around mla_decode_paged (runtime absorption of W_UK, W_UV).
    Both run in the same process, alternating, on two weight sets each."""
    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, D = 64, 128, synth.D_MODEL
    sets = []
    for layer in range(2):
        inp = synth.make_inputs("3u", layer=layer, gen_device="cuda").to(dev)
        x, w_q, w_o = synth.model_io_inputs(4400 + 10 * layer, B, H, D, device=dev)
        w_qk, w_vo = mla.fuse_weights(w_q, inp.w_uk, inp.w_uv, w_o)
        lat, rope = mla.split_cache(inp.cache)
        ws = torch.empty(mla.decode_fused_workspace_size(H, B, inp.max_len, D), dtype=torch.uint8,
                         device=dev)
        ws_u = torch.empty(mla.workspace_size(H, B, inp.max_len, mla.MLA_BF16, mla.MLA_BF16),
                           dtype=torch.uint8, device=dev)
        sets.append(dict(inp=inp, x=x, wq=w_q.reshape(H * 128, D), wo=w_o.reshape(H * 128, D),
                         w_qk=w_qk, w_vo=w_vo, lat=lat, rope=rope, ws=ws, ws_u=ws_u,
                         y=torch.empty((B, D), dtype=torch.bfloat16, device=dev),
                         o=torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()

    def fused(S):
        inp = S["inp"]
        mla.decode_fused(S["x"], inp.q_pe, S["w_qk"], S["w_vo"], S["lat"], S["rope"], inp.lengths,
                         inp.max_len, block_table=inp.block_table, block_size=inp.block_size,
                         out=S["y"], workspace=S["ws"])

    def unfused(S):
        inp = S["inp"]
        q_nope = torch.matmul(S["x"], S["wq"].t()).view(B, H, 128)
        mla.decode_paged(q_nope, inp.q_pe, inp.w_uk, inp.w_uv, S["lat"], S["rope"], inp.lengths,
                         inp.max_len, block_table=inp.block_table, block_size=inp.block_size,
                         out=S["o"], workspace=S["ws_u"])
        torch.matmul(S["o"].view(B, H * 128), S["wo"], out=S["y"])

    def timed(fn, steps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            fn(sets[i % 2])
            evs[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    for _ in range(max(1, args.warmup // 2)):
        fused(sets[0]); unfused(sets[0]); fused(sets[1]); unfused(sets[1])
    torch.cuda.synchronize()
    tf, tu = [], []
    for _ in range(4):   # alternate in rounds, so both see the same clock history
        tf += timed(fused, args.steps // 4)
        tu += timed(unfused, args.steps // 4)
    fms, ums = sum(tf) / len(tf), sum(tu) / len(tu)
    inp0 = sets[0]["inp"]
    cache_bytes = int(inp0.lengths.sum()) * 1152
    fused_w = 2 * H * 512 * D * 2
    unfused_w = 2 * H * 128 * D * 2 + 2 * H * 128 * 512 * 2
    fb = fused_w + cache_bytes
    line = {
        "metric": "MLA decode step from model-width input, weights fused offline (tokens/s)",
        "value": B / (fms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": len(tf),
        "warmup": args.warmup, "ms_per_step": fms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normals; random-init weights of the DeepSeek-V3 MLA widths)",
        "config": {"workload": "mla_decode_fused_b64_h128_n4096_paged_bf16_d7168", "B": B, "H": H,
                   "N": 4096, "d_model": D},
        "roofline": {"bound": "hbm", "achieved": fb / (fms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": fb / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": None, "kernel": "mla_decode_fused (all launches)",
                     "bytes_per_launch": fb,
                     "launch_us_p10_p50_p90": [percentile(tf, q) * 1e3 for q in (10, 50, 90)]},
        "fused_weight_bytes": fused_w,
        "unfused": {"ms_per_step": ums, "tokens_per_s": B / (ums * 1e-3),
                    "weight_bytes": unfused_w,
                    "step_us_p10_p50_p90": [percentile(tu, q) * 1e3 for q in (10, 50, 90)],
                    "what": "torch.matmul(x, W_Q^T) + mla_decode_paged + torch.matmul(o, W_O)"},
        "fused_over_unfused_time": fms / ums,
    }
    print(json.dumps(line), flush=True)


def bench_restart(args):
    """Worst-case cost of the attention kernel's overflow restart: the B=64
    N=4096 paged bf16 workload with, in every split of every sequence, one row
    set along the part of one head's absorbed query that is orthogonal to the
    other heads', scaled to outscore the split's first tile by far more than
    64 in log2 units. Every workgroup then takes the second pass (scores of
    the whole split for the true maximum, then the split again). Timed against
    the unmodified cache in the same run (decode launches only, no append)."""
    import numpy as np
    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = synth.make_inputs("3u")
    hot = synth.make_inputs("3u")
    B, H = base.B, base.H
    wuk = base.w_uk.double()
    S = 4
    per = base.max_len // S
    table = base.block_table
    for b in range(B):
        qlat = torch.einsum("hn,hnc->hc", base.q_nope[b].double(), wuk).numpy()
        hh = b % H
        others = np.delete(qlat, hh, axis=0)
        coef = np.linalg.lstsq(others.T, qlat[hh], rcond=None)[0]
        qperp = qlat[hh] - others.T @ coef
        x = torch.zeros(576, dtype=torch.float32)
        x[:512] = torch.from_numpy(100.0 / (qperp @ qperp * base.scale * np.log2(np.e)) * qperp)
        for s in range(S):
            t = s * per + per // 2
            row = int(table[b, t // base.block_size]) * base.block_size + t % base.block_size
            hot.cache[row] = x.to(torch.bfloat16)
    ev = HipEvents()
    out = {}
    for name, inp in (("normal", base), ("restart_every_split", hot)):
        d = inp.to(dev)
        ws = torch.empty(mla.workspace_size(H, B, d.max_len, mla.MLA_BF16, mla.MLA_BF16,
                                            num_splits=S), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            mla.decode_inputs(d, workspace=ws, num_splits=S)
        pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
        for i in range(args.steps):
            mla.decode_inputs(d, workspace=ws, num_splits=S, events=pairs[i])
        torch.cuda.synchronize()
        ms = [ev.elapsed_ms(a, b) for a, b in pairs]
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        out[name] = {"attn_us_mean": sum(ms) / len(ms) * 1e3,
                     "attn_us_p10_p50_p90": [percentile(ms, q) * 1e3 for q in (10, 50, 90)]}
        del d
    line = {"metric": "attention kernel time with the overflow restart in every split",
            "workload": "mla_decode_b64_h128_n4096_paged_bf16, 4 splits", "steps": args.steps,
            "warmup": args.warmup, **out,
            "slowdown": out["restart_every_split"]["attn_us_mean"] / out["normal"]["attn_us_mean"]}
    print(json.dumps(line), flush=True)


SIMD_COUNT = 1024            # MI355X: 256 CUs x 4 SIMDs

WORKLOADS = {"1": "mla_decode_b1_h16_n512_f32", "2": "mla_decode_b1_h128_n4096_bf16",
             "3u": "mla_decode_b64_h128_n4096_paged_bf16",
             "3": "mla_decode_b64_h128_ragged1024to4096_paged_bf16",
             "4": "mla_decode_b4_h128_n131072_bf16",
             "5": "mla_decode_b32_h128_n32768_fp8cache_per_layer"}
FULL_STEP_WORKLOAD = "mla_decode_61layer_step_b32_h128_n32768_fp8cache"


# the fp8 cache's attention kernel: the fp8 matrix-core kernel, unless
# MLA_FP8_KERNEL=widen selects the widening one
FP8_KERNEL = ("mla_decode_fp8_kernel" if os.environ.get("MLA_FP8_KERNEL") == "widen"
              else "mla_decode_fp8mma_kernel")


def decode_kernel_name(cache_dtype: str) -> str:
    return {"f32": "mla_decode_f32_kernel", "bf16": "mla_decode_bf16_kernel",
            "fp8": FP8_KERNEL}[cache_dtype]


def write_mfma(counters_csv: str, trace_csv: str, config: str, kernel: str):
    """MFMA evidence for one kernel from a rocprofv3 run with --kernel-trace
    and --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
    GRBM_GUI_ACTIVE: per-dispatch means, the FLOP the matrix cores executed
    (MOPS x 512, rocprofv3's MfmaFlopsBF16), the busy fraction of the
    matrix pipes (MfmaUtil = busy cycles summed over the SIMDs / (the GPU's
    active cycles x SIMDs)), and the GPU clock while the kernel ran (active
    cycles of the busiest counter instance / the traced duration)."""
    import csv
    rows = [r for r in csv.DictReader(open(counters_csv)) if kernel in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no {kernel} rows in {counters_csv}")
    by = {}
    for r in rows:
        by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: sum(v) / len(v) for k, v in by.items()}
    tr = [r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
    durs = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr)
    dur_ns = durs[len(durs) // 2]
    util = mean["MfmaUtil"]
    busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"]
    # MfmaUtil divides by the busiest instance of GRBM_GUI_ACTIVE (one per
    # XCD), so that count follows from the two; the counter window of a
    # dispatch is longer than the kernel, so cycles / duration over-states the
    # clock (an upper bound)
    grbm_max = busy / (util / 100.0 * SIMD_COUNT) if util > 0 else None
    # every matrix-core data type the run counted (bf16 for the bf16 and
    # widening kernels, f8 / f6f4 for the fp8 matrix-core kernel)
    mops = {k: v for k, v in mean.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_")}
    flops = sum(mops.values()) * 512
    rec = {"kernel": kernel, "workload": config,
           "kernel_source_hash": kernel_source_hash(sources_of(kernel)),
           "dispatches": len(rows) // max(1, len(by)), "counters_mean": mean,
           "median_duration_us": dur_ns / 1e3,
           "mfma_util_pct": util,
           "mfma_busy_cycles_per_simd": busy / SIMD_COUNT,
           "mfma_flop_per_dispatch": flops,
           "mfma_flop_by_type": {k[len("SQ_INSTS_VALU_MFMA_MOPS_"):]: v * 512
                                 for k, v in mops.items()},
           "mfma_tflops": flops / dur_ns / 1e3,
           # against the dense peak of the type executed (fp8 twice bf16's)
           "mfma_frac_of_peak": sum(v * 512 / (MFMA_BF16_PEAK_TFLOPS * (2 if k.endswith(("F8", "F6F4"))
                                                                         else 1))
                                    for k, v in mops.items()) / dur_ns / 1e3,
           "gpu_active_cycles_max_instance": grbm_max,
           "clock_ghz_upper_bound": grbm_max / dur_ns if grbm_max else None,
           "mfma_busy_frac_at_2p4ghz": busy / SIMD_COUNT / (dur_ns * 2.4),
           "peak_used": {"bf16_dense_tflops": MFMA_BF16_PEAK_TFLOPS,
                         "fp8_dense_tflops": 2 * MFMA_BF16_PEAK_TFLOPS, "simds": SIMD_COUNT,
                         "clock_ghz": 2.4}}
    out = os.path.join(ROOT, "profiles", f"{kernel}_{config}_mfma.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def measured_mfma(workload: str, kernel: str):
    """The committed MFMA counter record of the kernel on this workload, if it
    was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_mfma.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(sources_of(kernel)):
        return None
    keys = ("mfma_util_pct", "mfma_tflops", "mfma_frac_of_peak", "mfma_flop_per_dispatch",
            "mfma_flop_by_type", "median_duration_us")
    return {k: t[k] for k in keys if k in t}


def percentile(vals, q):
    v = sorted(vals)
    k = (len(v) - 1) * q / 100.0
    i = int(math.floor(k))
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (k - i)


def main():
    args = parse()
    if args.restart:
        args.steps = 200 if args.steps is None else args.steps
        args.warmup = 50 if args.warmup is None else args.warmup
        bench_restart(args)
        return
    if args.fused:
        args.steps = 200 if args.steps is None else args.steps
        args.warmup = 40 if args.warmup is None else args.warmup
        bench_fused(args)
        return
    if args.prefill:
        args.steps = 50 if args.steps is None else args.steps
        args.warmup = 10 if args.warmup is None else args.warmup
        bench_prefill(args)
        return
    if args.project and not args.write_traffic:
        args.steps = 1000 if args.steps is None else args.steps
        args.warmup = 300 if args.warmup is None else args.warmup
        bench_project(args)
        return
    if args.write_traffic:
        if args.project:
            write_traffic(args.write_traffic, PROJECT_WORKLOAD, PROJECT_KERNELS,
                          sources=PROJECT_SOURCES)
        else:
            kern = FP8_KERNEL if args.config == "5" else "mla_decode_bf16_kernel"
            write_traffic(args.write_traffic, args.config, (kern,))
        return
    if args.write_mfma:
        kern = FP8_KERNEL if args.config == "5" else "mla_decode_bf16_kernel"
        write_mfma(*args.write_mfma, args.config, kern)
        return
    if args.stream_read > 0:
        stream_read(args.stream_read)
        return
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this benchmark runs on one GPU only (one process, no collectives); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    cfg_key = args.config
    cfg = cfg_key if cfg_key == "3u" else int(cfg_key)
    # config 5 with --layers 61: a step is the whole 61-layer decode step
    # (every layer resident, one decode call per layer); otherwise a step is
    # one layer's decode call, cycling over a few resident layers so that no
    # step finds its cache in the last-level cache left by the previous one
    full_step = cfg == 5 and args.layers > 1
    n_layers = args.layers if full_step else (args.layers or N_LAYERS_CYCLED)
    per_step = n_layers if full_step else 1
    steps = args.steps if args.steps is not None else (50 if full_step else 1000)
    warmup = args.warmup if args.warmup is not None else (10 if full_step else 300)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (resident in HBM), one set per layer ----
    layers = []
    for layer in range(n_layers):
        gen = "cuda" if cfg == 5 else "cpu"
        inp = synth.make_inputs(cfg, layer=layer, gen_device=gen).to(dev)
        lat, rope = mla.split_cache(inp.cache)
        B, H = inp.B, inp.H
        act = mla.dtype_code(inp.q_nope.dtype)
        # the new token of each sequence sits at position N_b - 1
        c_new, k_new = synth.append_inputs(7000 + layer, B, inp.act, device=dev)
        pos = (inp.lengths - 1).to(dev)
        cdt = mla.dtype_code(inp.cache.dtype)
        ws = torch.empty(mla.workspace_size(H, B, inp.max_len, act, cdt, 0, args.length_aware),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((B, H, 128), dtype=inp.q_nope.dtype, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        L = dict(inp=inp, lat=lat, rope=rope, c=c_new, k=k_new, pos=pos, ws=ws, out=out, lse=lse)
        if args.with_projection:
            L["proj"] = synth.projection_inputs(9100 + 10 * layer, B, inp.act, synth.D_MODEL,
                                                device=dev)
            L["pws"] = torch.empty(mla.project_workspace_size(B, synth.D_MODEL),
                                   dtype=torch.uint8, device=dev)
        layers.append(L)
        if full_step and (layer + 1) % 10 == 0:
            print(f"bench.py: {layer + 1} of {n_layers} layers resident", file=sys.stderr,
                  flush=True)
    torch.cuda.synchronize()
    inp0 = layers[0]["inp"]
    B, H = inp0.B, inp0.H
    tok_rows = int(inp0.lengths.sum())
    row_bytes = mla.cache_bytes_per_token(mla.dtype_code(inp0.cache.dtype))
    cache_bytes = tok_rows * row_bytes                  # algorithmic bytes per launch
    flop_attn = tok_rows * (2 * H * 576 + 2 * H * 512)  # QK^T + PV per launch

    ev = HipEvents()

    def layer_call(L, events=None, stream=None):
        inp = L["inp"]
        new_rows = (L["c"], L["k"], L["pos"])
        if args.with_projection:
            h, wd, wk = L["proj"]
            if args.separate_append:
                mla.project_append(h, wd, wk, L["pos"], L["lat"], L["rope"], heads=H,
                                   scales=inp.scales, seq_capacity=inp.seq_capacity,
                                   block_table=inp.block_table, block_size=inp.block_size,
                                   workspace=L["pws"])
                new_rows = None
            else:
                mla.project(h, wd, wk, L["pws"], heads=H)
                new_rows = (None, None, L["pos"], 10000.0, L["pws"], synth.D_MODEL)
            mla.decode_inputs(inp, out=L["out"], lse=L["lse"], workspace=L["ws"], events=events,
                              append=new_rows, length_aware=args.length_aware)
            return
        if args.separate_append:
            mla.cache_append(*new_rows, L["lat"], L["rope"], heads=H, scales=inp.scales,
                             seq_capacity=inp.seq_capacity, block_table=inp.block_table,
                             block_size=inp.block_size)
            new_rows = None
        if "call" not in L:   # the step's decode call, marshalled once per layer
            L["call"] = mla.prepare_decode_inputs(inp, out=L["out"], lse=L["lse"],
                                                  workspace=L["ws"], append=new_rows,
                                                  length_aware=args.length_aware)
        L["call"].run(events, stream)

    def step(i, events=None, stream=None):
        if full_step:
            for k, L in enumerate(layers):
                layer_call(L, events[k] if events else None, stream)
        else:
            layer_call(layers[i % n_layers], events[0] if events else None, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    pairs = [[(ev.create(), ev.create()) for _ in range(per_step)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, events=pairs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms = [ev.elapsed_ms(a, b) for ps in pairs for a, b in ps]
    for ps in pairs:
        for a, b in ps:
            ev.destroy(a)
            ev.destroy(b)

    ms_per_step = (t1 - t0) * 1e3 / steps
    tokens_per_s = B * steps / (t1 - t0)
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    achieved_gbs = cache_bytes / (attn_avg_ms * 1e-3) / 1e9
    workload = FULL_STEP_WORKLOAD if full_step else WORKLOADS[cfg_key]
    if args.with_projection:
        workload += "_with_down_projection_d7168"
    if args.length_aware:
        workload += "_length_aware"
    kernel = decode_kernel_name(inp0.cache_dtype)
    traffic = measured_traffic(cfg_key, cache_bytes, kernel)
    dtype = {"f32": "f32", "bf16": "bf16", "fp8": "bf16+fp8cache"}[inp0.cache_dtype]
    config = {"workload": workload, "B": B, "H": H, "N_max": inp0.max_len,
              "cache_token_rows": tok_rows, "paged": inp0.paged,
              "block_size": inp0.block_size if inp0.paged else None,
              "d_c": 512, "d_rope": 64, "d_nope": 128, "d_v": 128}
    if full_step:
        config["layers_per_step"] = n_layers
    else:
        config["layers_cycled"] = n_layers
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded normals; random-init weights of the DeepSeek-V3 MLA widths)",
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel, "bytes_per_launch": cache_bytes,
                     "avg_launch_us": attn_avg_ms * 1e3,
                     "launch_us_p10_p50_p90": [percentile(attn_ms, q) * 1e3 for q in (10, 50, 90)]},
        "latent_cache_gbs": achieved_gbs,
        "latent_cache_pct_of_hbm_peak": 100.0 * achieved_gbs / HBM_PEAK_GBS,
        # algorithmic: the attention FLOP of the launch / its event time
        "attention_mfma_algorithmic_tflops": flop_attn / (attn_avg_ms * 1e-3) / 1e12,
        "attention_mfma_algorithmic_frac_of_bf16_peak":
            flop_attn / (attn_avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        # counters: the committed rocprofv3 record of this kernel and workload
        "mfma_counters": measured_mfma(cfg_key, kernel),
        "step_cache_gbs": cache_bytes * per_step / (ms_per_step * 1e-3) / 1e9,
    }
    if full_step:
        step_bytes = cache_bytes * per_step
        step_flop = flop_attn * per_step
        hbm_floor_ms = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        mfma_floor_ms = step_flop / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
        result["full_step"] = {
            "cache_bytes_per_step": step_bytes, "attention_flop_per_step": step_flop,
            "hbm_floor_ms": hbm_floor_ms, "bf16_mfma_floor_ms": mfma_floor_ms,
            "fp8_mfma_floor_ms": mfma_floor_ms / 2,
            "frac_of_hbm_floor": hbm_floor_ms / ms_per_step,
            "frac_of_bf16_mfma_floor": mfma_floor_ms / ms_per_step}
    if args.graph:
        result["hip_graph"] = graph_timing(step, layers, full_step, n_layers, B, steps, warmup)
    if args.clock > 0:
        n_clock = max(steps, int(args.clock / (ms_per_step * 1e-3)))

        def clocked():
            for i in range(n_clock):
                step(i)
            torch.cuda.synchronize()

        result["shader_clock"] = sample_clocks(clocked, n_clock)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
        result["cpu_absorbed_f32"] = cpu_absorbed_f32(cfg, min(args.cpu_seconds, 8.0))
    print(json.dumps(result), flush=True)


def sample_clocks(run, n_steps):
    """The GPU's shader (gfx) clock while run() issues n_steps steps: a host
    thread polls amdsmi's GPU metrics every ~2 ms (the clock fields the
    firmware reports: per-XCD current clocks and the average, N/A values
    dropped) and the GFX clock domain's current frequency. Returns the
    per-field median / p10 / p90 in MHz over the samples taken while the
    steps ran, with the steps' own time for comparison with the timed run."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001 - reported in the line, not fatal
        return {"error": f"amdsmi unavailable: {e!r}"}
    fields, errors = {}, []
    stop = threading.Event()

    def add(name, v):
        if isinstance(v, (list, tuple)):
            vals = [x for x in v if isinstance(x, (int, float)) and 0 < x < 65535]
            if vals:
                fields.setdefault(name + "_mean_over_xcds", []).append(sum(vals) / len(vals))
        elif isinstance(v, (int, float)) and 0 < v < 65535:
            fields.setdefault(name, []).append(float(v))

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                for k, v in m.items():
                    if "gfxclk" in k or "gfx_activity" in k:
                        add("metrics." + k, v)
                c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
                add("clock_info.gfx.clk", c.get("clk"))
            except Exception as e:  # noqa: BLE001
                if len(errors) < 3:
                    errors.append(repr(e))
            time.sleep(0.002)

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    run()
    t1 = time.perf_counter()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    out = {"source": "amdsmi gpu metrics + clock info, polled every ~2 ms from a host thread",
           "steps": n_steps, "ms_per_step": (t1 - t0) * 1e3 / n_steps, "unit": "MHz"}
    for k, v in sorted(fields.items()):
        out[k] = {"samples": len(v), "p10": percentile(v, 10), "median": percentile(v, 50),
                  "p90": percentile(v, 90)}
    if errors:
        out["errors"] = errors
    return out


def graph_timing(step, layers, full_step, n_layers, B, steps, warmup):
    """The same steps replayed from HIP graphs (torch.cuda.CUDAGraph on the
    caller's stream): one graph per cycled layer (the whole step for the
    61-layer mode), captured after a warm-up on a side stream; the step's
    launches then go to the GPU without a host call per kernel."""
    import torch
    n = 1 if full_step else n_layers
    graphs = []
    for k in range(n):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(k, stream=side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(k, stream=torch.cuda.current_stream().cuda_stream)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    return {"ms_per_step": ms, "tokens_per_s": B * steps / (t1 - t0), "graphs": n}


if __name__ == "__main__":
    main()
