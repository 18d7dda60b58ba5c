"""Seeded synthetic inputs for MLA decode (shared by tests, smoke and bench).

This module only draws random numbers and converts them to storage types with
torch's built-in dtype conversions (round-to-nearest-even). It holds none of
the attention arithmetic, so neither the CPU oracle nor the HIP library
depends on the other through it.

Workloads (DeepSeek-V3-shaped MLA decode: latent 512, decoupled RoPE key 64,
128 heads, no-RoPE query/key 128, value 128):

  cfg 1   fp32,  B=1,  H=16,  N=512,   contiguous
  cfg 2   bf16,  B=1,  H=128, N=4096,  contiguous
  cfg 3   bf16,  B=64, H=128, N_b ~ U[1024, 4096], paged (64-token blocks,
          placed by a seeded random permutation of the block pool)
  cfg 3u  as 3 with every N_b = 4096 (the headline throughput workload)
  cfg 4   bf16,  B=4,  H=128, N=131072, contiguous
  cfg 5   fp8 e4m3 cache + one bf16 scale per row, bf16 activations,
          B=32, H=128, N=32768, 61 independent layers, contiguous

Distributions: q_nope, q_pe, c_KV, k_pe ~ N(0,1); W_UK, W_UV ~ N(0, 1/512)
(standard deviation 1/sqrt(fan_in), fan_in = 512). Seeds:
1000*cfg + 10*tensor_id + 100000*layer, tensor ids q_nope 0, q_pe 1, W_UK 2,
W_UV 3, cache 4 (latent and RoPE key drawn together as one 576-wide row),
lengths 6, block permutation 7. Config 3u reuses config 3's seeds.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

D_C, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128
ROW = D_C + D_ROPE
BLOCK = 64
E4M3_MAX = 448.0

CONFIGS = {
    1: dict(B=1, H=16, N=512, act="f32", cache="f32", paged=False, layers=1),
    2: dict(B=1, H=128, N=4096, act="bf16", cache="bf16", paged=False, layers=1),
    3: dict(B=64, H=128, N=4096, act="bf16", cache="bf16", paged=True, layers=1,
            ragged=(1024, 4096)),
    "3u": dict(B=64, H=128, N=4096, act="bf16", cache="bf16", paged=True, layers=1),
    4: dict(B=4, H=128, N=131072, act="bf16", cache="bf16", paged=False, layers=1),
    5: dict(B=32, H=128, N=32768, act="bf16", cache="fp8", paged=False, layers=61),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


@dataclasses.dataclass
class DecodeInputs:
    cfg: object
    B: int
    H: int
    act: str                      # "f32" or "bf16": queries, weights, output
    cache_dtype: str              # "f32", "bf16" or "fp8"
    q_nope: torch.Tensor          # [B, H, 128]
    q_pe: torch.Tensor            # [B, H, 64] (already rotated)
    w_uk: torch.Tensor            # [H, 128, 512]
    w_uv: torch.Tensor            # [H, 512, 128]
    cache: torch.Tensor           # [rows, 576] latent | RoPE key (uint8 codes for fp8)
    scales: Optional[torch.Tensor]  # [rows] bf16 (fp8 cache only)
    lengths: torch.Tensor         # [B] int32
    max_len: int
    seq_capacity: int             # contiguous: rows per sequence; paged: 0
    block_table: Optional[torch.Tensor]  # [B, max_blocks] int32 (paged)
    block_size: int
    scale: float                  # 1/sqrt(d_nope + d_rope)

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def to(self, device) -> "DecodeInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return dataclasses.replace(
            self, q_nope=mv(self.q_nope), q_pe=mv(self.q_pe), w_uk=mv(self.w_uk),
            w_uv=mv(self.w_uv), cache=mv(self.cache), scales=mv(self.scales),
            lengths=mv(self.lengths), block_table=mv(self.block_table))


def seed_of(cfg, tensor_id: int, layer: int = 0) -> int:
    c = 3 if cfg == "3u" else int(cfg)
    return 1000 * c + 10 * tensor_id + 100000 * layer


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """float32 N(0, std^2) draws from a seeded generator on `device`."""
    t = torch.randn(shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round float32 draws to the storage type (RNE, torch's conversion)."""
    if dtype == "f32":
        return x.contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def fp8_rows(x: torch.Tensor):
    """Synthetic fp8 e4m3fn rows with one bf16 scale per row, spanning the
    code range: scale = bf16(amax/448) (1 for an all-zero row), codes = the
    e4m3fn conversion of x/scale clamped to +-448. Returns (uint8 codes, bf16)."""
    amax = x.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.bfloat16)
    y = (x / s.float().unsqueeze(1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s


def lengths_of(cfg, B: int, N: int) -> torch.Tensor:
    spec = CONFIGS[cfg]
    if "ragged" in spec:
        lo, hi = spec["ragged"]
        return torch.randint(lo, hi + 1, (B,), generator=_gen(seed_of(cfg, 6), "cpu"),
                             dtype=torch.int64).to(torch.int32)
    return torch.full((B,), N, dtype=torch.int32)


def paged_layout(cfg, lengths: torch.Tensor, block_size: int = BLOCK):
    """Block pool of exactly sum(ceil(N_b/bs)) blocks, handed out to the
    sequences in order from one seeded random permutation of the pool.
    Returns (block_table [B, max_blocks] int32 with unused entries 0, num_blocks)."""
    nb = [(int(n) + block_size - 1) // block_size for n in lengths.tolist()]
    num_blocks = sum(nb)
    perm = torch.randperm(num_blocks, generator=_gen(seed_of(cfg, 7), "cpu"))
    max_blocks = max(nb) if nb else 0
    table = torch.zeros((len(nb), max(max_blocks, 1)), dtype=torch.int32)
    off = 0
    for b, k in enumerate(nb):
        table[b, :k] = perm[off:off + k].to(torch.int32)
        off += k
    return table, num_blocks


def make_inputs(cfg, *, device="cpu", layer: int = 0, B: Optional[int] = None,
                N: Optional[int] = None, H: Optional[int] = None,
                lengths: Optional[torch.Tensor] = None, paged: Optional[bool] = None,
                cache_dtype: Optional[str] = None, act: Optional[str] = None,
                seq_capacity: Optional[int] = None, block_size: int = BLOCK,
                gen_device=None) -> DecodeInputs:
    """Seeded inputs of one workload (optionally resized for small tests).

    Random draws happen on `gen_device` (default: the CPU) and the tensors end
    up on `device`."""
    spec = CONFIGS[cfg]
    B = spec["B"] if B is None else B
    H = spec["H"] if H is None else H
    N = spec["N"] if N is None else N
    act = spec["act"] if act is None else act
    cdt = spec["cache"] if cache_dtype is None else cache_dtype
    paged = spec["paged"] if paged is None else paged
    gdev = "cpu" if gen_device is None else gen_device
    if lengths is None:
        lengths = lengths_of(cfg, B, N) if (B == spec["B"] and N == spec["N"]) \
            else torch.full((B,), N, dtype=torch.int32)
    lengths = lengths.to(torch.int32).cpu()
    max_len = int(lengths.max().item()) if B > 0 else 0
    wstd = 1.0 / math.sqrt(D_C)
    q_nope = to_storage(normal((B, H, D_NOPE), seed_of(cfg, 0, layer), gdev), act)
    q_pe = to_storage(normal((B, H, D_ROPE), seed_of(cfg, 1, layer), gdev), act)
    w_uk = to_storage(normal((H, D_NOPE, D_C), seed_of(cfg, 2, layer), gdev, wstd), act)
    w_uv = to_storage(normal((H, D_C, D_V), seed_of(cfg, 3, layer), gdev, wstd), act)
    if paged:
        table, num_blocks = paged_layout(cfg, lengths, block_size)
        rows = num_blocks * block_size
        cap = 0
    else:
        table = None
        cap = max(max_len, 1) if seq_capacity is None else seq_capacity
        rows = B * cap
    x = normal((rows, ROW), seed_of(cfg, 4, layer), gdev)
    if cdt == "fp8":
        cache, scales = fp8_rows(x)
    else:
        cache, scales = to_storage(x, cdt), None
    del x
    inp = DecodeInputs(cfg=cfg, B=B, H=H, act=act, cache_dtype=cdt, q_nope=q_nope,
                       q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, cache=cache, scales=scales,
                       lengths=lengths, max_len=max_len, seq_capacity=cap,
                       block_table=table, block_size=block_size,
                       scale=1.0 / math.sqrt(D_NOPE + D_ROPE))
    return inp.to(device)


def append_inputs(seed: int, B: int, in_dtype: str, device="cpu"):
    """New-token latent c_KV [B, 512] and un-rotated RoPE key k_pe [B, 64]."""
    c = to_storage(normal((B, D_C), seed, device), in_dtype)
    k = to_storage(normal((B, D_ROPE), seed + 1, device), in_dtype)
    return c, k


def prefill_queries(seed: int, B: int, T: int, H: int, act: str = "bf16", device="cpu"):
    """Queries of a prefill chunk: q_nope [B, T, H, 128] and q_pe [B, T, H, 64]
    (already rotated) ~ N(0,1). Seeds: seed, seed + 1."""
    qn = to_storage(normal((B, T, H, D_NOPE), seed, device), act)
    qp = to_storage(normal((B, T, H, D_ROPE), seed + 1, device), act)
    return qn, qp


D_MODEL = 7168    # hidden width of the DeepSeek-V3 setting


def model_io_inputs(seed: int, B: int, H: int, d_model: int = 7168, act: str = "bf16",
                    device="cpu"):
    """Model-width decode inputs: x [B, d_model] ~ N(0,1), query projection
    W_Q [H, 128, d_model] ~ N(0, 1/d_model) and output projection
    W_O [H, 128, d_model] ~ N(0, 1/(128 H)) (standard deviation
    1/sqrt(fan_in): d_model inputs per query, 128 H per output).
    Seeds: seed (x), seed + 1 (W_Q), seed + 2 (W_O)."""
    x = to_storage(normal((B, d_model), seed, device), act)
    w_q = to_storage(normal((H, D_NOPE, d_model), seed + 1, device,
                            std=1.0 / math.sqrt(d_model)), act)
    w_o = to_storage(normal((H, D_V, d_model), seed + 2, device,
                            std=1.0 / math.sqrt(D_V * H)), act)
    return x, w_q, w_o


def projection_inputs(seed: int, B: int, act: str, d_model: int = D_MODEL, device="cpu"):
    """Hidden states h [B, d_model] ~ N(0,1) and the down-projection weights
    W_DKV [512, d_model], W_KR [64, d_model] ~ N(0, 1/d_model) (standard
    deviation 1/sqrt(fan_in), fan_in = d_model), in the activation type.
    Seeds: seed (h), seed+1 (W_DKV), seed+2 (W_KR)."""
    sd = 1.0 / math.sqrt(d_model)
    h = to_storage(normal((B, d_model), seed, device), act)
    w_dkv = to_storage(normal((D_C, d_model), seed + 1, device, std=sd), act)
    w_kr = to_storage(normal((D_ROPE, d_model), seed + 2, device, std=sd), act)
    return h, w_dkv, w_kr


def raw_bits(t: torch.Tensor):
    """Storage bits of a CPU tensor as a numpy integer array (uint16 for bf16,
    uint32 for f32, uint8 for fp8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view("uint32")
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)
