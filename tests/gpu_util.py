"""Helpers for the GPU parity tests: move seeded inputs to the device, call
the library through its C ABI binding, and compare with the CPU reference."""
import numpy as np
import torch

import exact_io_aware_attention_amd as fa

# Tolerances stated for this path: bf16 O max-abs <= 2e-2 and relative L2
# <= 5e-3, dQ/dK/dV relative L2 <= 1e-2; fp32 debug path <= 1e-5.
# LSE is not graded by those; it is held to 1e-3 (bf16) / 1e-5 (fp32).
BF16_O_MAX_ABS = 2e-2
BF16_O_REL_L2 = 5e-3
BF16_GRAD_REL_L2 = 1e-2
BF16_LSE_MAX_ABS = 1e-3
F32_TOL = 1e-5
# FP8 forward: bars derived from a replay of its E4M3 rounding of P on the
# CPU (tests/fp8_spec.py, asserted by tests/test_fp8_tolerance.py).
from tests.fp8_spec import FP8_O_MAX_ABS, FP8_O_REL_L2  # noqa: E402,F401


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_forward(q, k, v, scale, causal, mask, precision="bf16"):
    dt = torch.bfloat16 if precision == "bf16" else torch.float32
    Q, K, V = dev(q, dt), dev(k, dt), dev(v, dt)
    O = torch.empty_like(Q)
    B, H, N, _ = q.shape
    LSE = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    M = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).to("cuda")
    fn = fa.fa_fwd if precision == "bf16" else fa.fa_fwd_f32
    fn(Q, K, V, O, LSE, scale, causal=causal, blockmask=M)
    torch.cuda.synchronize()
    return (Q, K, V, O, LSE, M)


def gpu_forward_backward(q, k, v, do, scale, causal, mask, precision="bf16"):
    dt = torch.bfloat16 if precision == "bf16" else torch.float32
    Q, K, V, O, LSE, M = gpu_forward(q, k, v, scale, causal, mask, precision)
    dO = dev(do, dt)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    fn = fa.fa_bwd if precision == "bf16" else fa.fa_bwd_f32
    fn(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, causal=causal, blockmask=M)
    torch.cuda.synchronize()
    return O, LSE, dQ, dK, dV


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def check(name, got, ref, max_abs=None, rel_l2=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    ma, rl = errors(got, ref)
    print(f"  {name}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    if max_abs is not None:
        assert ma <= max_abs, f"{name}: max abs error {ma:.3e} > {max_abs:.1e}"
    if rel_l2 is not None:
        assert rl <= rel_l2, f"{name}: relative L2 error {rl:.3e} > {rel_l2:.1e}"


def check_lse(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_g, inf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(inf_g, inf_r), f"{name}: -inf pattern differs"
    fin = ~inf_r
    check(name, got[fin], ref[fin], max_abs=tol)


def check_outputs(precision, got, ref, fields=("O", "LSE", "dQ", "dK", "dV")):
    """got/ref: dicts of numpy arrays."""
    for f in fields:
        if f not in ref:
            continue
        if f == "LSE":
            check_lse(f, got[f], ref[f], BF16_LSE_MAX_ABS if precision == "bf16" else F32_TOL)
        elif precision == "f32":
            check(f, got[f], ref[f], max_abs=F32_TOL, rel_l2=F32_TOL)
        elif f == "O":
            check(f, got[f], ref[f], max_abs=BF16_O_MAX_ABS, rel_l2=BF16_O_REL_L2)
        else:
            check(f, got[f], ref[f], rel_l2=BF16_GRAD_REL_L2)
