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


# ---------------------------------------------------------------- fp8 ---
#
# OCP FP8 E4M3 (the "fn" variant gfx950 uses: bias 7, 3 mantissa bits, no
# infinities, largest finite 448, subnormals down to 2^-9). Inputs of the FP8
# forward are stored in this format with one fp32 scale per tensor: value =
# code * descale, descale = max|x| / 448 so that the largest magnitude maps to
# the largest code.

E4M3_MAX = 448.0


def e4m3_round_bits(x) -> np.ndarray:
    """fp32 -> E4M3 codes (uint8), round to nearest even, magnitudes beyond
    448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    s = np.signbit(x).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade, clamped to the normal range; below 2^-6 the
    # spacing is that of the subnormals (2^-9)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)
    q = np.rint(a / step) * step          # numpy rint: half to even
    q = np.minimum(q, E4M3_MAX)
    # encode q
    out = np.zeros(q.shape, dtype=np.uint8)
    nz = q > 0
    qe = np.floor(np.log2(np.where(nz, q, 1.0)))
    normal = nz & (qe >= -6)
    mant = np.where(normal, q / np.exp2(qe) - 1.0, 0.0)
    code_n = ((qe + 7).astype(np.int64) << 3) + np.rint(mant * 8).astype(np.int64)
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, np.where(nz, code_s, 0))
    out = (code.astype(np.uint8) | s)
    return out


def e4m3_bits_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return sign * val


def fp8_quantize(x):
    """(codes uint8, descale float32) for one tensor: descale = max|x| / 448
    rounded to fp32, codes = E4M3(x / descale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    descale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    codes = e4m3_round_bits(x.astype(np.float64) / np.float64(descale))
    return codes, float(descale)


def fp8_inputs(B, H, N, d, seed, qk_mult=1.0):
    """Q, K, V drawn as in draw_qkvdo, then stored as E4M3 codes with one
    descale each. Returns ((q8, k8, v8), (qs, ks, vs), (q, k, v)) where the
    last triple is the dequantized values (code * descale, exact in fp64)."""
    q, k, v, _ = draw_qkvdo(B, H, N, d, seed, qk_mult)
    codes, scales, deq = [], [], []
    for t in (q, k, v):
        c, s = fp8_quantize(t)
        codes.append(c)
        scales.append(s)
        deq.append(e4m3_bits_to_f64(c) * np.float64(s))
    return tuple(codes), tuple(scales), tuple(deq)
