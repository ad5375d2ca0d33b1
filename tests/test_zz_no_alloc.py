"""The no-allocation backward entry point (fa_bwd_noalloc, scratch in the
library's static device array) against fa_bwd with a caller workspace: the
same kernels on the same inputs, so the outputs must agree bit for bit. Two
calls in a row, the second on a smaller problem (the array then holds the
first call's larger contents), and a check that the call allocates no
device memory."""
import numpy as np
import pytest
import torch

import synthetic as syn

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_io_aware_attention_amd as fa
    from tests import gpu_util as gu

CASES = [  # B, H, N, d, causal, sparse: the second is smaller than the first
    (2, 4, 1000, 128, True, False),
    (1, 2, 300, 64, False, True),
]


def _run_both(B, H, N, d, causal, sparse, seed):
    q, k, v, do = syn.random_inputs(B, H, N, d, seed=seed, dtype="bf16")
    mask = syn.block_mask((N + 127) // 128, seed=seed) if sparse else None
    scale = float(np.float32(1 / np.sqrt(d)))
    Q, K, V, O, LSE, M = gu.gpu_forward(q, k, v, scale, causal, mask)
    dO = gu.dev(do, torch.bfloat16)
    ref = [torch.empty_like(Q) for _ in range(3)]
    fa.fa_bwd(dO, Q, K, V, O, LSE, *ref, scale, causal=causal, blockmask=M)
    torch.cuda.synchronize()
    got = [torch.full_like(Q, float("nan")) for _ in range(3)]
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    fa.fa_bwd_noalloc(dO, Q, K, V, O, LSE, *got, scale, causal=causal, blockmask=M)
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    torch.cuda.synchronize()
    assert after == before, "fa_bwd_noalloc allocated through torch"
    return got, ref


def test_noalloc_backward_matches_workspace_backward():
    for i, (B, H, N, d, causal, sparse) in enumerate(CASES):
        print(f"fa_bwd_noalloc call {i + 1}: B={B} H={H} N={N} d={d} causal={causal} "
              f"sparse={sparse}", flush=True)
        got, ref = _run_both(B, H, N, d, causal, sparse, seed=40 + i)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            gh, rh = gu.host(g), gu.host(r)
            gu.check(name, gh, rh, rel_l2=gu.BF16_GRAD_REL_L2)
            assert torch.equal(g.view(torch.int16), r.view(torch.int16)), f"{name} differs bitwise"
