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
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--config", default="3u")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--separate-append", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--write-traffic", nargs=4, default=None)
    ap.add_argument("--project", action="store_true")
    ap.add_argument("--with-projection", action="store_true")
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
                     sources=KERNEL_SOURCES):
    """HBM bytes per launch of the measured kernel(s) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, seconds: float):
    """The oracle as it stands (float64, non-absorbed), on a bounded sample of
    the same workload: whole sequences (all heads) until `seconds` elapse."""
    import numpy as np
    import synth
    from oracle import mla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(cfg)

    def f64(t, kind):
        return orc.decode_storage(synth.raw_bits(t), kind)

    wuk, wuv = f64(inp.w_uk, "bf16"), f64(inp.w_uv, "bf16")
    table = None if inp.block_table is None else inp.block_table.numpy()
    done = 0
    tokens = 0
    t0 = time.perf_counter()
    while True:
        b = done % inp.B
        n = int(inp.lengths[b])
        rows = orc.gather_rows(b, n, seq_capacity=inp.seq_capacity, block_table=table,
                               block_size=inp.block_size)
        import torch
        vals = f64(inp.cache[torch.from_numpy(rows)], inp.cache_dtype)
        orc.decode(f64(inp.q_nope[b:b + 1], "bf16"), f64(inp.q_pe[b:b + 1], "bf16"), wuk, wuv,
                   [vals[:, :512]], [vals[:, 512:]], inp.scale)
        done += 1
        tokens += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence(s) x 128 heads of the same workload (N={inp.max_len}), "
                      f"float64 non-absorbed oracle, {dt:.1f} s"}


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


def _counter_mean(csv_path: str, kernel_substr: str, counter: str) -> float:
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {csv_path}")
    return sum(vals) / len(vals)


def write_traffic(paths, config: str, kernels, copy_mib: int = 1024, sources=KERNEL_SOURCES):
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
           "kernel_source_hash": kernel_source_hash(sources),
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


def main():
    args = parse()
    if args.project and not args.write_traffic:
        bench_project(args)
        return
    if args.write_traffic:
        if args.project:
            write_traffic(args.write_traffic, PROJECT_WORKLOAD, PROJECT_KERNELS,
                          sources=PROJECT_SOURCES)
        else:
            write_traffic(args.write_traffic, args.config, ("mla_decode_bf16_kernel",))
        return
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (one process, no collectives); "
              f"--gpus {args.gpus} / WORLD_SIZE={world} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_07_amd as mla
    import synth

    mla.load()
    cfg = args.config if args.config in ("3u", "3", "4", "5") else "3u"
    cfg = cfg if cfg == "3u" else int(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs (resident in HBM), one set per cycled layer ----
    layers = []
    for layer in range(N_LAYERS_CYCLED):
        gen = "cuda" if cfg == 5 else "cpu"
        inp = synth.make_inputs(cfg, layer=layer, gen_device=gen).to(dev)
        lat, rope = mla.split_cache(inp.cache)
        B, H = inp.B, inp.H
        # the new token of each sequence sits at position N_b - 1
        c_new, k_new = synth.append_inputs(7000 + layer, B, "bf16", device=dev)
        pos = (inp.lengths - 1).to(dev)
        cdt = mla.dtype_code(inp.cache.dtype)
        ws = torch.empty(mla.workspace_size(H, B, inp.max_len, mla.MLA_BF16, cdt),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        L = dict(inp=inp, lat=lat, rope=rope, c=c_new, k=k_new, pos=pos, ws=ws, out=out, lse=lse)
        if args.with_projection:
            L["proj"] = synth.projection_inputs(9100 + 10 * layer, B, "bf16", synth.D_MODEL,
                                                device=dev)
            L["pws"] = torch.empty(mla.project_workspace_size(B, synth.D_MODEL),
                                   dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()
    inp0 = layers[0]["inp"]
    B, H = inp0.B, inp0.H
    tok_rows = int(inp0.lengths.sum())
    row_bytes = mla.cache_bytes_per_token(mla.dtype_code(inp0.cache.dtype))
    cache_bytes = tok_rows * row_bytes                  # algorithmic bytes per launch
    flop_attn = tok_rows * (2 * H * 576 + 2 * H * 512)  # QK^T + PV per launch

    ev = HipEvents()

    def step(L, events=None):
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
                              append=new_rows)
            return
        if args.separate_append:
            mla.cache_append(*new_rows, L["lat"], L["rope"], heads=H, scales=inp.scales,
                             seq_capacity=inp.seq_capacity, block_table=inp.block_table,
                             block_size=inp.block_size)
            new_rows = None
        mla.decode_inputs(inp, out=L["out"], lse=L["lse"], workspace=L["ws"], events=events,
                          append=new_rows)

    for i in range(args.warmup):
        step(layers[i % N_LAYERS_CYCLED])
    torch.cuda.synchronize()

    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(layers[i % N_LAYERS_CYCLED], events=pairs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = B * args.steps / (t1 - t0)
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    achieved_gbs = cache_bytes / (attn_avg_ms * 1e-3) / 1e9
    workload = {"3u": "mla_decode_b64_h128_n4096_paged_bf16",
                3: "mla_decode_b64_h128_ragged1024to4096_paged_bf16",
                4: "mla_decode_b4_h128_n131072_bf16",
                5: "mla_decode_b32_h128_n32768_fp8cache_per_layer"}[cfg]
    if args.with_projection:
        workload += "_with_down_projection_d7168"
    traffic = measured_traffic(str(cfg), cache_bytes)
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp0.cache_dtype == "bf16" else "bf16+fp8cache",
        "data": "synthetic (seeded normals; random-init weights of the DeepSeek-V3 MLA widths)",
        "config": {"workload": workload, "B": B, "H": H, "N_max": inp0.max_len,
                   "cache_token_rows": tok_rows, "paged": inp0.paged,
                   "block_size": inp0.block_size if inp0.paged else None,
                   "d_c": 512, "d_rope": 64, "d_nope": 128, "d_v": 128,
                   "layers_cycled": N_LAYERS_CYCLED},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "mla_decode_bf16_kernel" if inp0.cache_dtype == "bf16"
                     else "mla_decode_fp8_kernel",
                     "bytes_per_launch": cache_bytes, "avg_launch_us": attn_avg_ms * 1e3},
        "latent_cache_gbs": achieved_gbs,
        "latent_cache_pct_of_hbm_peak": 100.0 * achieved_gbs / HBM_PEAK_GBS,
        "attention_mfma_tflops": flop_attn / (attn_avg_ms * 1e-3) / 1e12,
        "attention_mfma_frac_of_bf16_peak": flop_attn / (attn_avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "step_cache_gbs": cache_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg if cfg != 5 else 5, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
