"""Cases and error bars of the FP8 forward (E4M3 Q, K, V and P, fp32 softmax
statistics), shared by its GPU parity test and by the CPU test that derives
the bars (tests/test_fp8_tolerance.py).

The reference is exact attention of the decoded E4M3 inputs. The one
rounding the kernel adds on top of exact arithmetic and the bf16 store of O
is that of each weight P = 2^(c s - m) to E4M3 (3 mantissa bits) for the P V
product, m the exact running row max of the keys seen so far (so the weight
that sets a new max is exactly 1); S and the row sum stay fp32. The CPU test
replays exactly that on each case below and reports the error it causes; the
bars sit at BAR_MULTIPLE times the worst simulated error over the cases,
which that test asserts.
"""

import numpy as np

import synthetic as syn

# (B, H, N, d, causal, qk_mult)
FP8_CASES = [
    (1, 2, 300, 128, True, 1.0),
    (2, 1, 129, 64, False, 1.0),
    (1, 1, 1031, 128, True, 1.0),
    (1, 2, 64, 64, True, 1.0),
    (1, 2, 2048, 128, True, 2.0),
    (1, 1, 1, 128, False, 1.0),
]


def fp8_seed(N, d):
    """Seed of the inputs of the case with these N and d."""
    return 6000 + N + d


# Multiple of the worst simulated error at which the bars are set: the GPU
# differs from the simulation only where fp32 rounding of S, of the exponent
# or of the sums moves a weight across an E4M3 rounding boundary.
BAR_MULTIPLE = 1.5
# worst simulated over FP8_CASES (O stored in bf16): relative L2 2.02e-2
# (the B=2 N=129 d=64 case), max abs 6.07e-2 (the N=2048 Q,K x 2 case)
FP8_O_REL_L2 = 3.1e-2
FP8_O_MAX_ABS = 9.2e-2


def kernel_c(scale):
    """The kernel's exponent factor: scale * log2(e), rounded to fp32."""
    return float(np.float32(scale) * np.float32(1.4426950408889634))


TILE = 64  # keys per step of the kernel's running max


def e4m3_weight(x):
    return syn.e4m3_bits_to_f64(syn.e4m3_round_bits(x))


def bf16_store(x):
    return syn.bf16_round(np.asarray(x, np.float32)).astype(np.float64)


def simulate(q, k, v, scale, causal, c, round_p=True):
    """Online softmax over 64-key tiles with the reference at the exact
    running row max; P rounded to E4M3 for P V when round_p. Returns O
    (unrounded) and LSE (natural log)."""
    B, H, N, d = q.shape
    O = np.zeros_like(q)
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            S = (q[b, h] @ k[b, h].T) * c  # base-2 exponent units
            if causal:
                S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            o = np.zeros((N, d))
            for t0 in range(0, N, TILE):
                st = S[:, t0:t0 + TILE]
                mn = np.maximum(m, st.max(axis=1))
                fin = np.isfinite(m)
                alpha = np.where(fin, np.exp2(np.where(fin, m, 0.0) - np.where(fin, mn, 0.0)), 0.0)
                ref = np.where(np.isfinite(mn), mn, 0.0)
                p = np.exp2(st - ref[:, None])
                l = alpha * l + p.sum(axis=1)
                o = alpha[:, None] * o + (e4m3_weight(p) if round_p else p) @ v[b, h][t0:t0 + TILE]
                m = mn
            pos = l > 0
            O[b, h] = np.where(pos[:, None], o / np.where(pos, l, 1.0)[:, None], 0.0)
            L[b, h] = np.where(pos, (m + np.log2(np.where(pos, l, 1.0))) * np.log(2.0), -np.inf)
    return O, L
