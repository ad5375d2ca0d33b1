"""The tiled online-softmax recurrence reaches the definition exactly.

mstx.cn/posts/485 §三.2 "Online Softmax" gives the update for a new key/value
block with local statistics (m~, l~, O~):
    m' = max(m, m~);  l' = e^(m - m') l + e^(m~ - m') l~;
    O' = e^(m - m') O + e^(m~ - m') O~,
with O kept unnormalised and divided by l once at the end (the page leaves
the final divide implicit). This test-only numpy routine walks random block
partitions of the keys with that update and must match the CPU reference's
two-pass result in fp64. It pins the method the GPU kernels use to the
definition; it is not the reference.
"""
import numpy as np
import pytest

import oracle


def _online(q, k, v, scale, allowed, cuts):
    N, d = q.shape
    O = np.zeros((N, d))
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = scale * q @ k[a:b].T
        s = np.where(allowed[:, a:b], s, -np.inf)
        mt = s.max(axis=1)
        with np.errstate(invalid="ignore"):
            pt = np.where(np.isfinite(mt)[:, None], np.exp(s - mt[:, None]), 0.0)
        lt = pt.sum(axis=1)
        Ot = pt @ v[a:b]
        mn = np.maximum(m, mt)
        fin = np.isfinite(mn)
        alpha = np.where(fin & np.isfinite(m), np.exp(np.where(fin, m - mn, 0.0)), 0.0)
        beta = np.where(fin & np.isfinite(mt), np.exp(np.where(fin, mt - mn, 0.0)), 0.0)
        l = alpha * l + beta * lt
        O = alpha[:, None] * O + beta[:, None] * Ot
        m = mn
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, O / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("trial", range(4))
def test_block_merge_equals_two_pass(causal, trial):
    rng = np.random.Generator(np.random.PCG64(777 + trial))
    N, d = 50, 6
    q = rng.standard_normal((1, 1, N, d)) * 2
    k = rng.standard_normal((1, 1, N, d)) * 2
    v = rng.standard_normal((1, 1, N, d))
    O, LSE = oracle.attention(q, k, v, 0.45, causal=causal)
    allowed = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    cuts = np.unique(np.r_[0, np.sort(rng.choice(np.arange(1, N), size=6, replace=False)), N])
    Om, Lm = _online(q[0, 0], k[0, 0], v[0, 0], 0.45, allowed, cuts)
    assert np.max(np.abs(Om - O[0, 0])) <= 1e-13
    assert np.max(np.abs(Lm - LSE[0, 0])) <= 1e-13


def test_block_merge_handles_masked_blocks():
    """A block where a row sees no key (local max -inf) must not poison the
    running statistics: the guard alpha = 0 / beta = 0 replaces exp(-inf - -inf)."""
    rng = np.random.Generator(np.random.PCG64(99))
    N, d, blk = 16, 3, 4
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    mask = np.array([[0, 1, 0, 1], [1, 0, 0, 1], [0, 0, 1, 0], [0, 0, 0, 0]], np.uint8)
    O, LSE = oracle.attention(q, k, v, 0.5, blockmask=mask, blk=blk)
    i = np.arange(N)
    allowed = mask[i[:, None] // blk, i[None, :] // blk].astype(bool)
    Om, Lm = _online(q[0, 0], k[0, 0], v[0, 0], 0.5, allowed, np.arange(0, N + 1, blk))
    assert np.max(np.abs(Om - O[0, 0])) <= 1e-13
    fin = np.isfinite(LSE[0, 0])
    assert np.array_equal(fin, np.isfinite(Lm))
    assert np.max(np.abs(Lm[fin] - LSE[0, 0][fin])) <= 1e-13
