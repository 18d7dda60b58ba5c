"""Glue between the synthetic workloads, the CPU oracle and the GPU results
(test-side only)."""

from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import mla_oracle as orc


def to_f64(t: torch.Tensor, kind: str) -> np.ndarray:
    """Decode a CPU tensor's storage bits with the oracle's own decoders."""
    return orc.decode_storage(synth.raw_bits(t), kind)


def act_kind(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]


def gathered_rows(inp, b: int, cache_f64=None, cache_cpu=None):
    """Dequantised latent [N_b, 512] and RoPE-key [N_b, 64] rows of sequence b,
    gathered one token at a time through the oracle's addressing."""
    n = int(inp.lengths[b])
    table = None if inp.block_table is None else inp.block_table.cpu().numpy()
    rows = orc.gather_rows(b, n, seq_capacity=inp.seq_capacity, block_table=table,
                           block_size=inp.block_size)
    cache = inp.cache if cache_cpu is None else cache_cpu
    sel = cache[torch.from_numpy(rows)] if n else cache[:0]
    vals = to_f64(sel, inp.cache_dtype) if n else np.zeros((0, synth.ROW))
    if inp.cache_dtype == "fp8":
        scales = to_f64(inp.scales.cpu()[torch.from_numpy(rows)], "bf16") if n else np.zeros(0)
        vals = vals * scales[:, None]
    return vals[:, :synth.D_C], vals[:, synth.D_C:]


def oracle_decode(inp, batch_ids=None, heads=None, absorbed=False):
    """Oracle outputs for the chosen sequences (all by default).
    Returns (out [len(batch_ids), H, 128], lse [len(batch_ids), H])."""
    cpu = inp.to("cpu")
    bs = list(range(inp.B)) if batch_ids is None else list(batch_ids)
    kind = act_kind(cpu.q_nope)
    qn = to_f64(cpu.q_nope[bs], kind)
    qp = to_f64(cpu.q_pe[bs], kind)
    wuk = to_f64(cpu.w_uk, kind)
    wuv = to_f64(cpu.w_uv, kind)
    lat, rope = [], []
    for b in bs:
        c, r = gathered_rows(cpu, b)
        lat.append(c)
        rope.append(r)
    return orc.decode(qn, qp, wuk, wuv, lat, rope, inp.scale, heads=heads, absorbed=absorbed)


def oracle_decode_seq(inp, batch_ids=None):
    """Oracle outputs for every head of the chosen sequences (all by default)
    through the oracle's all-heads absorbed form, one sequence at a time (the
    affordable form at the full workload sizes). Returns (out [nb, H, 128],
    lse [nb, H])."""
    cpu = inp.to("cpu")
    bs = list(range(inp.B)) if batch_ids is None else list(batch_ids)
    kind = act_kind(cpu.q_nope)
    qn = to_f64(cpu.q_nope[bs], kind)
    qp = to_f64(cpu.q_pe[bs], kind)
    wuk = to_f64(cpu.w_uk, kind)
    wuv = to_f64(cpu.w_uv, kind)
    out = np.empty((len(bs), inp.H, synth.D_V))
    lse = np.empty((len(bs), inp.H))
    for i, b in enumerate(bs):
        c, r = gathered_rows(cpu, b)
        out[i], lse[i] = orc.decode_seq_absorbed(qn[i], qp[i], wuk, wuv, c, r, inp.scale)
    return out, lse


def rel_err_rows(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over (b, h) of ||gpu - ref||_inf / ||ref||_inf (NaN rows of ref skipped)."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    keep = ~np.isnan(r).any(axis=1)
    g, r = g[keep], r[keep]
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return orc.bf16_bits_to_f64(synth.raw_bits(t))
    return t.double().numpy()


TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2}
LSE_TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 1e-2}
