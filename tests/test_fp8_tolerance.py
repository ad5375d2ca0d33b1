"""Derivation of the FP8 forward's error bars (CPU only).

The FP8 forward computes exact attention of its decoded E4M3 inputs except
for one added rounding: each weight P = 2^(c s - m), m the exact running row
max over the 64-key tiles seen so far, is rounded to E4M3 (round to nearest
even) before the P V product, while S, the row max and the row sum stay
fp32 (lukebest.github.io FlashAttention, lineage table "谱系": the third
generation adds FP8; the pages give no format or tolerance). This test
replays exactly that rounding in numpy (fp64 elsewhere) on the inputs of
every GPU FP8 case, measures the error it causes against the fp64 oracle,
and checks that the bars the GPU test uses sit at BAR_MULTIPLE times the
worst simulated error (and not looser than twice it).
"""
import numpy as np
import pytest

import oracle
import synthetic as syn
from tests.fp8_spec import (BAR_MULTIPLE, FP8_CASES, FP8_O_MAX_ABS, FP8_O_REL_L2, bf16_store,
                            e4m3_weight, fp8_seed, kernel_c, simulate)

def _case(case):
    B, H, N, d, causal, qk = case
    _, _, (q, k, v) = syn.fp8_inputs(B, H, N, d, fp8_seed(N, d), qk)
    scale = float(np.float32(1 / np.sqrt(d)))
    return q, k, v, scale, causal


def _errs(got, ref):
    return float(np.max(np.abs(got - ref))), float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def test_e4m3_rounding_of_weights():
    """The weight rounding the simulation uses: 1 exact, 3 mantissa bits,
    ties to even, subnormal spacing 2^-9 below 2^-6."""
    x = np.array([1.0, 0.9, 0.5 + 1 / 32, 0.5 + 3 / 32, 2.0 ** -7 + 2.0 ** -11, 2.0 ** -11, 0.0])
    want = np.array([1.0, 0.875, 0.5, 0.625, 2.0 ** -7, 0.0, 0.0])
    np.testing.assert_array_equal(e4m3_weight(x), want)


@pytest.mark.parametrize("case", FP8_CASES[:5], ids=str)
def test_simulation_without_rounding_is_exact(case):
    """Without the E4M3 rounding (and with the exact c) the tiled recurrence
    of the simulation reproduces the oracle: the simulation adds nothing but
    the rounding it models."""
    q, k, v, scale, causal = _case(case)
    Or, Lr = oracle.attention(q, k, v, scale, causal=causal)
    O0, L0 = simulate(q, k, v, scale, causal, c=scale / np.log(2.0), round_p=False)
    assert _errs(O0, Or)[1] <= 1e-12
    fin = np.isfinite(Lr)
    assert np.max(np.abs(L0[fin] - Lr[fin])) <= 1e-11


def test_bars_sit_at_the_stated_multiple_of_the_simulated_error():
    worst_abs = worst_rel = 0.0
    for case in FP8_CASES:
        q, k, v, scale, causal = _case(case)
        Or, Lr = oracle.attention(q, k, v, scale, causal=causal)
        Os, Ls = simulate(q, k, v, scale, causal, kernel_c(scale))
        ma, rel = _errs(bf16_store(Os), Or)  # O is stored in bf16
        print(f"{case}: simulated O max_abs={ma:.3e} rel_l2={rel:.3e}", flush=True)
        worst_abs, worst_rel = max(worst_abs, ma), max(worst_rel, rel)
        # LSE is untouched by the rounding of P (S and l stay fp32)
        fin = np.isfinite(Lr)
        assert np.max(np.abs(Ls[fin] - Lr[fin])) <= 1e-5
    print(f"worst: max_abs={worst_abs:.3e} rel_l2={worst_rel:.3e}", flush=True)
    assert BAR_MULTIPLE * worst_rel <= FP8_O_REL_L2 <= 2 * worst_rel
    assert BAR_MULTIPLE * worst_abs <= FP8_O_MAX_ABS <= 2 * worst_abs
