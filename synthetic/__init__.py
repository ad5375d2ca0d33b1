"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the attention arithmetic: it draws random numbers,
rounds them to bf16 storage, and builds the fixed block mask and the row
sample. Both the GPU path and the CPU reference consume what it produces.

Workloads (shapes, masks and value distributions of the five attention
configurations; the pages measure on GPT-2 attention at sequence 1K, on
long-range sequences to 64K and on block-sparse long-range tasks --
lukebest.github.io FlashAttention, "实测摘要" and "Block-Sparse FlashAttention" --
and these seeded inputs stand in for those workloads):

  1 tiny            B=1 H=2  N=128   d=64  dense,   fp32 and bf16
  2 gpt2-small      B=8 H=12 N=1024  d=64  causal
  3 long-causal     B=2 H=16 N=8192  d=128 causal,  Q and K times 2.0
  4 very-long       B=1 H=8  N=65536 d=64  dense,   forward only
  5 block-sparse    B=4 H=8  N=16384 d=64  128x128 block mask

Draw recipe: numpy Generator(PCG64(seed)) with seed = config number; Q, K, V,
dO drawn in that order by standard_normal(float32) with shape [B,H,N,d] in C
order; config 3 multiplies Q and K by 2.0 (exact in binary floating point);
then each tensor is rounded to bf16 with round-to-nearest-even. The block
mask uses its own stream (seed 1005) and the config-4 row sample another
(seed 1004).
"""
from dataclasses import dataclass
import math

import numpy as np

MASK_BLOCK = 128
MASK_SEED = 1005
ROWS_SEED = 1004


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    sparse: bool
    qk_mult: float
    has_bwd: bool

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded once to fp32: both sides receive the same value.
        return float(np.float32(1.0 / math.sqrt(self.d)))


CONFIGS = {
    1: Config(1, "tiny", 1, 2, 128, 64, False, False, 1.0, True),
    2: Config(2, "gpt2-small-causal", 8, 12, 1024, 64, True, False, 1.0, True),
    3: Config(3, "long-causal", 2, 16, 8192, 128, True, False, 2.0, True),
    4: Config(4, "very-long-dense", 1, 8, 65536, 64, False, False, 1.0, False),
    5: Config(5, "block-sparse", 4, 8, 16384, 64, False, True, 1.0, True),
}


def bf16_round_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).
    Returns the bf16 bit patterns as uint16. NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


def draw_qkvdo(B, H, N, d, seed, qk_mult=1.0):
    """Q, K, V, dO as float32 N(0,1) draws in that order, Q and K times qk_mult."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    if qk_mult != 1.0:
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    return q, k, v, do


def config_inputs(cfg: Config, dtype="bf16"):
    """Inputs of one configuration. dtype 'bf16' returns float32 arrays that
    hold bf16-rounded values; 'f32' returns the float32 draws unrounded."""
    q, k, v, do = draw_qkvdo(cfg.B, cfg.H, cfg.N, cfg.d, cfg.cfg_id, cfg.qk_mult)
    if dtype == "bf16":
        q, k, v, do = (bf16_round(t) for t in (q, k, v, do))
    elif dtype != "f32":
        raise ValueError(dtype)
    mask = block_mask(cfg.N // MASK_BLOCK) if cfg.sparse else None
    return q, k, v, do, mask


def block_mask(nb: int, band: int = 1, keep_frac: float = 0.10, seed: int = MASK_SEED):
    """[nb, nb] uint8 block mask: every block with |I - J| <= band kept, plus
    round(keep_frac * #other blocks) other blocks drawn without replacement."""
    I, J = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    m = (np.abs(I - J) <= band).astype(np.uint8)
    off = np.flatnonzero(m.ravel() == 0)
    n_keep = int(round(keep_frac * off.size))
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = rng.choice(off, size=n_keep, replace=False)
    flat = m.ravel()
    flat[pick] = 1
    return flat.reshape(nb, nb)


def row_sample(BH: int, N: int, count: int = 256, seed: int = ROWS_SEED):
    """`count` distinct (head, query) pairs drawn uniformly without replacement
    over BH*N. Returns (row_bh, row_i) int64 arrays, sorted by flat index."""
    rng = np.random.Generator(np.random.PCG64(seed))
    flat = np.sort(rng.choice(BH * N, size=count, replace=False))
    return (flat // N).astype(np.int64), (flat % N).astype(np.int64)


def random_inputs(B, H, N, d, seed, dtype="f32", qk_mult=1.0):
    """Arbitrary-shape seeded inputs for parity cases beyond the five configs."""
    q, k, v, do = draw_qkvdo(B, H, N, d, seed, qk_mult)
    if dtype == "bf16":
        q, k, v, do = (bf16_round(t) for t in (q, k, v, do))
    return q, k, v, do
