"""Pins for the CPU reference: facts fixed by the pages and by mathematics.

Each pin takes an oracle.Oracle instance and raises AssertionError when the
reference disagrees with the fact. The same battery runs against deliberately
broken builds of the reference (test_oracle_mutants.py) to show that a
plausible mistake anywhere in it fails at least one pin.

None of these retypes the reference's formula: they are closed forms,
invariances, brute force on tiny inputs, finite differences, and a library
routine (torch's CPU fp64 scaled_dot_product_attention and its autograd).
"""
import math

import numpy as np
import torch

RNG_SEED = 20221  # fixed seeds: pins are deterministic


def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


def _allowed_matrix(N, causal, mask, blk):
    """Brute-force element mask from the definition: key j visible to query i."""
    A = np.ones((N, N), dtype=bool)
    if causal:
        A &= np.tril(np.ones((N, N), dtype=bool))
    if mask is not None:
        i = np.arange(N)
        A &= mask[i[:, None] // blk, i[None, :] // blk].astype(bool)
    return A


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    worst = float(np.max(err)) if err.size else 0.0
    assert np.all(np.isfinite(err)) and worst <= tol, f"{what}: max err {worst} > {tol}"


# ---------------------------------------------------------------- forward ---

def pin_identical_keys_uniform(orc):
    """All key rows equal -> every allowed key gets the same weight, so O_i is
    the mean of the allowed V rows and LSE_i = scale*q_i.k + ln|A_i|.
    Checked dense, causal (prefix means) and under a block mask."""
    B, H, N, d, blk = 1, 2, 12, 5, 4
    q = _rand((B, H, N, d), RNG_SEED)
    krow = _rand((d,), RNG_SEED + 1)
    k = np.broadcast_to(krow, (B, H, N, d)).copy()
    v = _rand((B, H, N, d), RNG_SEED + 2)
    scale = 0.37
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=np.uint8)
    for causal, bm in ((False, None), (True, None), (False, mask), (True, mask)):
        O, LSE = orc.attention(q, k, v, scale, causal=causal, blockmask=bm, blk=blk)
        A = _allowed_matrix(N, causal, bm, blk)
        for h in range(H):
            for i in range(N):
                js = np.flatnonzero(A[i])
                _close(O[0, h, i], v[0, h, js].mean(axis=0), 1e-13, "uniform O")
                _close(LSE[0, h, i], scale * q[0, h, i] @ krow + math.log(js.size),
                       1e-12, "uniform LSE")


def pin_zero_query(orc):
    """Q = 0 -> all scores 0 -> O is the mean of the allowed V rows, LSE = ln|A_i|."""
    B, H, N, d = 2, 1, 9, 3
    q = np.zeros((B, H, N, d))
    k = _rand((B, H, N, d), RNG_SEED + 3, 3.0)
    v = _rand((B, H, N, d), RNG_SEED + 4)
    for causal in (False, True):
        O, LSE = orc.attention(q, k, v, 0.9, causal=causal)
        for b in range(B):
            for i in range(N):
                n = i + 1 if causal else N
                _close(O[b, 0, i], v[b, 0, :n].mean(axis=0), 1e-13, "Q=0 O")
                _close(LSE[b, 0, i], math.log(n), 1e-13, "Q=0 LSE")


def pin_single_key(orc):
    """N = 1 -> the only weight is 1: O = V and LSE = scale*q.k."""
    q = _rand((3, 2, 1, 7), RNG_SEED + 5)
    k = _rand((3, 2, 1, 7), RNG_SEED + 6)
    v = _rand((3, 2, 1, 7), RNG_SEED + 7)
    O, LSE = orc.attention(q, k, v, 0.25)
    _close(O, v, 1e-15, "N=1 O")
    _close(LSE, 0.25 * np.einsum("bhnd,bhnd->bhn", q, k), 1e-14, "N=1 LSE")


def pin_two_keys_logistic(orc):
    """Two keys, d = 1: the weight of key 0 is the logistic function
    1/(1+exp(s1-s0)) of the score difference, and LSE = log(e^s0 + e^s1)."""
    s0q, s1k = 1.3, -0.4
    q = np.array([s0q, -0.7]).reshape(1, 1, 2, 1)
    k = np.array([0.8, s1k]).reshape(1, 1, 2, 1)
    v = np.array([2.0, -5.0]).reshape(1, 1, 2, 1)
    scale = 0.6
    O, LSE = orc.attention(q, k, v, scale)
    for i in range(2):
        s0 = scale * q[0, 0, i, 0] * k[0, 0, 0, 0]
        s1 = scale * q[0, 0, i, 0] * k[0, 0, 1, 0]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(O[0, 0, i, 0], w0 * 2.0 + (1 - w0) * -5.0, 1e-14, "logistic O")
        _close(LSE[0, 0, i], math.log(math.exp(s0) + math.exp(s1)), 1e-14, "logistic LSE")


def pin_causal_first_row(orc):
    """Causal: query 0 sees only key 0, so O_0 = V_0 and LSE_0 = scale*q0.k0."""
    q = _rand((1, 3, 10, 4), RNG_SEED + 8)
    k = _rand((1, 3, 10, 4), RNG_SEED + 9)
    v = _rand((1, 3, 10, 4), RNG_SEED + 10)
    O, LSE = orc.attention(q, k, v, 0.5, causal=True)
    _close(O[:, :, 0], v[:, :, 0], 1e-15, "causal row 0")
    _close(LSE[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14,
           "causal row 0 LSE")


def pin_identity_values_expose_softmax(orc):
    """With d = N and V = I, O_i is the i-th row of P itself: entries are
    nonnegative, zero off the allowed set, rows sum to 1, and ratios between
    allowed entries are exp(score differences)."""
    N, blk = 8, 2
    q = _rand((1, 1, N, N), RNG_SEED + 11)
    k = _rand((1, 1, N, N), RNG_SEED + 12)
    v = np.eye(N).reshape(1, 1, N, N)
    mask = np.array([[1, 0, 1, 1], [1, 1, 0, 0], [0, 1, 1, 1], [1, 1, 1, 0]], np.uint8)
    scale = 0.8
    for causal, bm in ((False, None), (True, None), (False, mask), (True, mask)):
        P, LSE = orc.attention(q, k, v, scale, causal=causal, blockmask=bm, blk=blk)
        P = P[0, 0]
        A = _allowed_matrix(N, causal, bm, blk)
        S = scale * q[0, 0] @ k[0, 0].T
        for i in range(N):
            js = np.flatnonzero(A[i])
            if js.size == 0:
                continue
            assert np.all(P[i] >= 0.0), "negative weight"
            assert np.all(P[i][~A[i]] == 0.0), "weight on a masked key"
            _close(P[i].sum(), 1.0, 1e-14, "row sum")
            j0 = js[0]
            _close(np.log(P[i, js] / P[i, j0]), S[i, js] - S[i, j0], 1e-12,
                   "log weight ratios")
            _close(LSE[0, 0, i] - S[i, j0], -math.log(P[i, j0]), 1e-12, "LSE vs weight")


def pin_key_shift_invariance(orc):
    """K -> K + 1 u^T leaves P (hence O) unchanged and shifts LSE_i by
    scale * q_i . u."""
    q = _rand((2, 2, 11, 6), RNG_SEED + 13)
    k = _rand((2, 2, 11, 6), RNG_SEED + 14)
    v = _rand((2, 2, 11, 6), RNG_SEED + 15)
    u = _rand((6,), RNG_SEED + 16)
    for causal in (False, True):
        O1, L1 = orc.attention(q, k, v, 0.4, causal=causal)
        O2, L2 = orc.attention(q, k + u, v, 0.4, causal=causal)
        _close(O1, O2, 1e-13, "key shift O")
        _close(L2 - L1, 0.4 * np.einsum("bhnd,d->bhn", q, u), 1e-12, "key shift LSE")


def pin_value_affine(orc):
    """V -> a V + 1 b^T gives O -> a O + 1 b^T (rows of P sum to one)."""
    q = _rand((1, 2, 13, 4), RNG_SEED + 17)
    k = _rand((1, 2, 13, 4), RNG_SEED + 18)
    v = _rand((1, 2, 13, 4), RNG_SEED + 19)
    b = _rand((4,), RNG_SEED + 20)
    for causal in (False, True):
        O1, _ = orc.attention(q, k, v, 0.7, causal=causal)
        O2, _ = orc.attention(q, k, -2.5 * v + b, 0.7, causal=causal)
        _close(O2, -2.5 * O1 + b, 1e-13, "value affine")


def pin_key_permutation(orc):
    """Non-causal dense: permuting key rows and value rows together leaves O
    and LSE unchanged."""
    q = _rand((1, 1, 10, 5), RNG_SEED + 21)
    k = _rand((1, 1, 10, 5), RNG_SEED + 22)
    v = _rand((1, 1, 10, 5), RNG_SEED + 23)
    perm = np.random.Generator(np.random.PCG64(RNG_SEED + 24)).permutation(10)
    O1, L1 = orc.attention(q, k, v, 0.3)
    O2, L2 = orc.attention(q, k[:, :, perm], v[:, :, perm], 0.3)
    _close(O1, O2, 1e-13, "permutation O")
    _close(L1, L2, 1e-13, "permutation LSE")


def pin_scale_folding(orc):
    """Scores are scale * Q K^T: (c Q, scale / c) gives the same result as (Q, scale)."""
    q = _rand((1, 2, 9, 4), RNG_SEED + 25)
    k = _rand((1, 2, 9, 4), RNG_SEED + 26)
    v = _rand((1, 2, 9, 4), RNG_SEED + 27)
    O1, L1 = orc.attention(q, k, v, 0.5, causal=True)
    O2, L2 = orc.attention(4.0 * q, k, v, 0.125, causal=True)
    _close(O1, O2, 1e-13, "scale folding O")
    _close(L1, L2, 1e-13, "scale folding LSE")
    # and the scale is applied: doubling it changes O
    O3, _ = orc.attention(q, k, v, 1.0, causal=True)
    assert np.max(np.abs(O3 - O1)) > 1e-3, "scale has no effect"


def pin_mask_special_cases(orc):
    """All-ones block mask == dense; a lower-triangular block mask combined with
    causal == causal alone; a block row of zeros gives the documented
    masked-row result (O = 0, LSE = -inf, no gradient contribution)."""
    N, d, blk = 12, 3, 4
    nb = N // blk
    q = _rand((1, 2, N, d), RNG_SEED + 28)
    k = _rand((1, 2, N, d), RNG_SEED + 29)
    v = _rand((1, 2, N, d), RNG_SEED + 30)
    do = _rand((1, 2, N, d), RNG_SEED + 31)
    ones = np.ones((nb, nb), np.uint8)
    r_dense = orc.attention(q, k, v, 0.6, do=do)
    r_ones = orc.attention(q, k, v, 0.6, blockmask=ones, blk=blk, do=do)
    for a, b in zip(r_dense, r_ones):
        _close(a, b, 0.0, "all-ones mask")
    tri = np.tril(np.ones((nb, nb), np.uint8))
    r_c = orc.attention(q, k, v, 0.6, causal=True, do=do)
    r_ct = orc.attention(q, k, v, 0.6, causal=True, blockmask=tri, blk=blk, do=do)
    for a, b in zip(r_c, r_ct):
        _close(a, b, 0.0, "tri mask + causal")
    hole = ones.copy()
    hole[1, :] = 0
    O, LSE, dQ, dK, dV = orc.attention(q, k, v, 0.6, blockmask=hole, blk=blk, do=do)
    rows = slice(blk, 2 * blk)
    assert np.all(O[:, :, rows] == 0.0), "masked row O"
    assert np.all(np.isneginf(LSE[:, :, rows])), "masked row LSE"
    assert np.all(dQ[:, :, rows] == 0.0), "masked row dQ"
    # the masked rows contribute nothing to dK, dV: drop them and compare
    keep = np.r_[0:blk, 2 * blk:N]
    _, _, _, dK2, dV2 = orc.attention(q, k, v, 0.6, blockmask=hole, blk=blk,
                                      do=np.where(np.isin(np.arange(N), keep)[None, None, :, None],
                                                  do, 0.0))
    _close(dK, dK2, 1e-13, "masked rows do not feed dK")
    _close(dV, dV2, 1e-13, "masked rows do not feed dV")


def pin_block_mask_brute_force(orc):
    """Block-sparse result equals attention with the element mask built by
    brute force from the block mask (mask[i//blk][j//blk]), evaluated by
    torch's CPU fp64 scaled_dot_product_attention."""
    N, d, blk = 16, 4, 4
    q = _rand((1, 1, N, d), RNG_SEED + 32)
    k = _rand((1, 1, N, d), RNG_SEED + 33)
    v = _rand((1, 1, N, d), RNG_SEED + 34)
    mask = np.array([[1, 0, 0, 1], [1, 1, 0, 0], [0, 1, 1, 0], [1, 0, 1, 1]], np.uint8)
    for causal in (False, True):
        O, _ = orc.attention(q, k, v, 0.5, causal=causal, blockmask=mask, blk=blk)
        A = torch.from_numpy(_allowed_matrix(N, causal, mask, blk))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=A, scale=0.5)
        _close(O, ref.numpy(), 1e-13, "brute-force block mask")


def pin_library_sdpa(orc):
    """Forward and gradients equal torch's CPU fp64 scaled_dot_product_attention
    and its autograd (dense, causal and block-masked)."""
    B, H, N, d, blk = 2, 3, 24, 8, 8
    q = _rand((B, H, N, d), RNG_SEED + 35)
    k = _rand((B, H, N, d), RNG_SEED + 36)
    v = _rand((B, H, N, d), RNG_SEED + 37)
    do = _rand((B, H, N, d), RNG_SEED + 38)
    mask = np.array([[1, 1, 0], [0, 1, 1], [1, 0, 1]], np.uint8)
    for causal, bm in ((False, None), (True, None), (False, mask), (True, mask)):
        O, LSE, dQ, dK, dV = orc.attention(q, k, v, 0.35, causal=causal, blockmask=bm,
                                           blk=blk, do=do)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        A = torch.from_numpy(_allowed_matrix(N, causal, bm, blk))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=A,
                                                               scale=0.35)
        ref.backward(torch.from_numpy(do))
        _close(O, ref.detach().numpy(), 1e-13, "SDPA O")
        _close(dQ, tq.grad.numpy(), 1e-12, "SDPA dQ")
        _close(dK, tk.grad.numpy(), 1e-12, "SDPA dK")
        _close(dV, tv.grad.numpy(), 1e-12, "SDPA dV")
        S = 0.35 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
        S = S.masked_fill(~A, float("-inf"))
        _close(LSE, torch.logsumexp(S, dim=-1).numpy(), 1e-12, "logsumexp")


def pin_finite_differences(orc):
    """Central differences of L = <dO, O> match dQ, dK, dV (N <= 16, d <= 8)."""
    B, H, N, d = 1, 1, 7, 3
    scale = 0.8
    q = _rand((B, H, N, d), RNG_SEED + 39)
    k = _rand((B, H, N, d), RNG_SEED + 40)
    v = _rand((B, H, N, d), RNG_SEED + 41)
    do = _rand((B, H, N, d), RNG_SEED + 42)
    mask = np.array([[1, 0, 1, 1], [1, 1, 0, 1], [0, 1, 1, 0], [1, 1, 0, 1]], np.uint8)
    h = 1e-6
    for causal, bm in ((False, None), (True, None), (False, mask)):
        _, _, dQ, dK, dV = orc.attention(q, k, v, scale, causal=causal, blockmask=bm, blk=2,
                                         do=do)
        grads = {"q": dQ, "k": dK, "v": dV}
        for name in ("q", "k", "v"):
            g = np.zeros_like(q)
            for idx in np.ndindex(q.shape):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[name][idx] += h
                Op, _ = orc.attention(args["q"], args["k"], args["v"], scale, causal=causal,
                                      blockmask=bm, blk=2)
                args[name][idx] -= 2 * h
                Om, _ = orc.attention(args["q"], args["k"], args["v"], scale, causal=causal,
                                      blockmask=bm, blk=2)
                g[idx] = np.sum(do * (Op - Om)) / (2 * h)
            rel = np.linalg.norm(g - grads[name]) / max(np.linalg.norm(g), 1e-30)
            assert rel <= 1e-6, f"finite differences d{name}: rel err {rel}"


def pin_backward_invariants(orc):
    """sum_j dK_j = 0 (O is invariant to a common key shift); identical keys
    give dQ = 0; Q = 0 (dense) gives dV_j = mean_i dO_i."""
    B, H, N, d = 1, 2, 10, 4
    q = _rand((B, H, N, d), RNG_SEED + 43)
    k = _rand((B, H, N, d), RNG_SEED + 44)
    v = _rand((B, H, N, d), RNG_SEED + 45)
    do = _rand((B, H, N, d), RNG_SEED + 46)
    for causal in (False, True):
        _, _, _, dK, _ = orc.attention(q, k, v, 0.5, causal=causal, do=do)
        _close(dK.sum(axis=2), 0.0, 1e-13, "sum of dK")
    kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
    for causal in (False, True):
        _, _, dQ, _, _ = orc.attention(q, kk, v, 0.5, causal=causal, do=do)
        _close(dQ, 0.0, 1e-13, "identical keys dQ")
    _, _, _, _, dV = orc.attention(np.zeros_like(q), k, v, 0.5, do=do)
    _close(dV, np.broadcast_to(do.mean(axis=2, keepdims=True), dV.shape), 1e-14,
           "Q=0 dV")


def pin_rows_match_full(orc):
    """The row-subset forward returns exactly the selected rows of the full forward."""
    B, H, N, d, blk = 2, 2, 16, 4, 4
    q = _rand((B, H, N, d), RNG_SEED + 47)
    k = _rand((B, H, N, d), RNG_SEED + 48)
    v = _rand((B, H, N, d), RNG_SEED + 49)
    mask = np.array([[1, 0, 0, 1], [0, 1, 0, 0], [1, 1, 1, 0], [0, 0, 1, 1]], np.uint8)
    rb = np.array([0, 3, 1, 2, 3])
    ri = np.array([0, 15, 7, 4, 5])
    for causal, bm in ((False, None), (True, mask)):
        O, LSE = orc.attention(q, k, v, 0.5, causal=causal, blockmask=bm, blk=blk)
        Or, Lr = orc.attention_rows(q, k, v, 0.5, rb, ri, causal=causal, blockmask=bm,
                                    blk=blk)
        _close(Or, O.reshape(B * H, N, d)[rb, ri], 0.0, "rows O")
        _close(Lr, LSE.reshape(B * H, N)[rb, ri], 0.0, "rows LSE")


# ------------------------------------------------- decode (Nq != Nk) ---

def _kv_allowed(Nq, Nk, causal):
    """Brute-force visibility for the decode shape: query i sits at position
    Nk - Nq + i and, when causal, sees the keys up to that position."""
    A = np.ones((Nq, Nk), dtype=bool)
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        A &= j <= Nk - Nq + i
    return A


def pin_kv_library_sdpa(orc):
    """Decode-shaped forward equals torch's CPU fp64 scaled_dot_product_attention
    with the visibility matrix built from the definition, and LSE equals
    torch.logsumexp of the masked scores."""
    B, H, d = 2, 2, 8
    for Nq, Nk in ((1, 19), (5, 23), (8, 8), (3, 2)):
        q = _rand((B, H, Nq, d), RNG_SEED + 60 + Nq)
        k = _rand((B, H, Nk, d), RNG_SEED + 70 + Nk)
        v = _rand((B, H, Nk, d), RNG_SEED + 80 + Nk)
        for causal in (False, True):
            O, LSE = orc.attention_kv(q, k, v, 0.45, causal=causal)
            A = torch.from_numpy(_kv_allowed(Nq, Nk, causal))
            S = 0.45 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
            S = S.masked_fill(~A, float("-inf"))
            _close(LSE, torch.logsumexp(S, dim=-1).numpy(), 1e-12, "decode logsumexp")
            rows = A.any(dim=-1).numpy()
            if rows.all():
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                    attn_mask=A, scale=0.45)
                _close(O, ref.numpy(), 1e-13, "decode SDPA O")
            else:  # rows that see no key: O = 0 by convention
                _close(O[:, :, ~rows], 0.0, 0.0, "decode O without keys")


def pin_kv_identical_keys(orc):
    """All key rows equal -> O_i is the mean of the visible V rows, and
    LSE_i = scale*q_i.k + ln(#visible); with the causal rule query i sees
    Nk - Nq + i + 1 keys."""
    B, H, Nq, Nk, d = 1, 2, 4, 11, 5
    q = _rand((B, H, Nq, d), RNG_SEED + 90)
    k = np.broadcast_to(_rand((B, H, 1, d), RNG_SEED + 91), (B, H, Nk, d)).copy()
    v = _rand((B, H, Nk, d), RNG_SEED + 92)
    for causal in (False, True):
        O, LSE = orc.attention_kv(q, k, v, 0.7, causal=causal)
        for i in range(Nq):
            n = Nk - Nq + i + 1 if causal else Nk
            _close(O[:, :, i], v[:, :, :n].mean(axis=2), 1e-14, "decode identical keys O")
            dots = 0.7 * np.einsum("bhd,bhd->bh", q[:, :, i], k[:, :, 0])
            _close(LSE[:, :, i], dots + math.log(n), 1e-13, "decode identical keys LSE")


def pin_kv_square_and_suffix(orc):
    """With Nq = Nk the decode forward is the square forward; with Nq < Nk and
    the causal rule it gives the last Nq rows of the square causal forward
    over the whole sequence (queries at the last Nq positions)."""
    B, H, N, d = 1, 2, 13, 6
    q = _rand((B, H, N, d), RNG_SEED + 93)
    k = _rand((B, H, N, d), RNG_SEED + 94)
    v = _rand((B, H, N, d), RNG_SEED + 95)
    for causal in (False, True):
        O, LSE = orc.attention_kv(q, k, v, 0.6, causal=causal)
        Os, Ls = orc.attention(q, k, v, 0.6, causal=causal)
        _close(O, Os, 1e-14, "decode square O")
        _close(LSE, Ls, 1e-14, "decode square LSE")
    Os, Ls = orc.attention(q, k, v, 0.6, causal=True)
    for nq in (1, 4):
        O, LSE = orc.attention_kv(q[:, :, N - nq:], k, v, 0.6, causal=True)
        _close(O, Os[:, :, N - nq:], 1e-14, "decode suffix O")
        _close(LSE, Ls[:, :, N - nq:], 1e-14, "decode suffix LSE")


def pin_kv_split_merge(orc):
    """Splitting the keys into two chunks and merging the chunk results with
    weights exp(LSE_chunk - LSE) gives the unsplit result (mstx.cn/posts/485
    §三.2 merge of partial softmax sums)."""
    B, H, Nq, Nk, d = 1, 3, 3, 17, 4
    q = _rand((B, H, Nq, d), RNG_SEED + 96)
    k = _rand((B, H, Nk, d), RNG_SEED + 97)
    v = _rand((B, H, Nk, d), RNG_SEED + 98)
    O, LSE = orc.attention_kv(q, k, v, 0.9)
    for a in (1, 8, 16):
        O1, L1 = orc.attention_kv(q, k[:, :, :a], v[:, :, :a], 0.9)
        O2, L2 = orc.attention_kv(q, k[:, :, a:], v[:, :, a:], 0.9)
        L = np.logaddexp(L1, L2)
        Om = np.exp(L1 - L)[..., None] * O1 + np.exp(L2 - L)[..., None] * O2
        _close(L, LSE, 1e-13, "split LSE")
        _close(Om, O, 1e-13, "split O")


# ---------------------------------------------------------------- dropout ---

def pin_philox_known_answers(orc):
    """Philox4x32-10 reproduces the known-answer vectors published with the
    generator (counter, key -> output): zeros, all ones, and the digits of pi."""
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        got = orc.philox4x32_10(ctr, key)
        assert got == want, f"philox {ctr} {key}: {[hex(x) for x in got]}"


def _drop_mask(orc, BH, N, p, seed):
    Z = np.zeros((BH, N, N))
    for bh in range(BH):
        for i in range(N):
            for j in range(N):
                Z[bh, i, j] = orc.dropout_keep(bh, i, j, p, seed)
    return Z


def pin_dropout_zero_is_plain(orc):
    """Dropout probability 0 gives exactly the plain forward and backward."""
    B, H, N, d = 1, 2, 9, 4
    q = _rand((B, H, N, d), RNG_SEED + 100)
    k = _rand((B, H, N, d), RNG_SEED + 101)
    v = _rand((B, H, N, d), RNG_SEED + 102)
    do = _rand((B, H, N, d), RNG_SEED + 103)
    for causal in (False, True):
        a = orc.attention(q, k, v, 0.5, causal=causal, do=do)
        b = orc.attention_dropout(q, k, v, 0.5, 0.0, 77, causal=causal, do=do)
        for x, y, n in zip(a, b, ("O", "LSE", "dQ", "dK", "dV")):
            _close(y, x, 0.0, f"p=0 {n}")


def pin_dropout_torch_autograd(orc):
    """With the mask drawn from the oracle's own rule, forward and gradients
    equal torch's CPU fp64 autograd of O = (softmax(S) o Z / (1 - p)) V
    (dense, causal, block-masked); LSE is that of S without dropout."""
    B, H, N, d, blk = 1, 2, 12, 5, 4
    p, seed = 0.3, 0x1234567890ABCDEF
    q = _rand((B, H, N, d), RNG_SEED + 104)
    k = _rand((B, H, N, d), RNG_SEED + 105)
    v = _rand((B, H, N, d), RNG_SEED + 106)
    do = _rand((B, H, N, d), RNG_SEED + 107)
    Z = torch.from_numpy(_drop_mask(orc, B * H, N, p, seed).reshape(B, H, N, N))
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)
    for causal, bm in ((False, None), (True, None), (False, mask)):
        O, LSE, dQ, dK, dV = orc.attention_dropout(q, k, v, 0.6, p, seed, causal=causal,
                                                   blockmask=bm, blk=blk, do=do)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        A = torch.from_numpy(_allowed_matrix(N, causal, bm, blk))
        S = (0.6 * tq @ tk.transpose(-1, -2)).masked_fill(~A, float("-inf"))
        P = torch.softmax(S, dim=-1)
        ref = (P * Z / (1 - p)) @ tv
        ref.backward(torch.from_numpy(do))
        _close(O, ref.detach().numpy(), 1e-13, "dropout O")
        _close(dQ, tq.grad.numpy(), 1e-12, "dropout dQ")
        _close(dK, tk.grad.numpy(), 1e-12, "dropout dK")
        _close(dV, tv.grad.numpy(), 1e-12, "dropout dV")
        _close(LSE, torch.logsumexp(S, dim=-1).detach().numpy(), 1e-12, "dropout LSE")


def pin_dropout_mask_rule(orc):
    """The keep bit follows the documented rule (a convention of this library,
    stated in include/fa.h): element (i, j) of head bh is dropped iff word
    j % 4 of Philox4x32-10(counter (j // 4, i, bh, 0), key (seed low 32 bits,
    seed high 32 bits)) is below floor(p * 2^32). Checked with the generator
    pinned by its known answers above."""
    seed = 0x0123456789ABCDEF
    for p in (0.2, 0.75):
        t = math.floor(p * 2 ** 32)
        for bh, i, j in ((0, 0, 0), (1, 2, 3), (3, 7, 13), (2, 30, 4), (5, 1, 63)):
            w = orc.philox4x32_10([j // 4, i, bh, 0], [seed & 0xFFFFFFFF, seed >> 32])[j % 4]
            assert orc.dropout_keep(bh, i, j, p, seed) == int(w >= t), (bh, i, j, p)


def pin_dropout_keep_rate(orc):
    """The kept fraction is 1 - p within 5 binomial standard deviations, for
    several p, and different seeds give different masks."""
    n = 64
    for p in (0.1, 0.5, 0.9):
        Z = _drop_mask(orc, 2, n, p, 99)
        m = Z.size
        sd = math.sqrt(m * p * (1 - p))
        assert abs(Z.sum() - m * (1 - p)) <= 5 * sd, f"keep rate {Z.mean()} for p={p}"
    Z1 = _drop_mask(orc, 1, 16, 0.5, 1)
    Z2 = _drop_mask(orc, 1, 16, 0.5, 2)
    assert not np.array_equal(Z1, Z2), "seed has no effect"


ALL_PINS = [
    pin_identical_keys_uniform,
    pin_zero_query,
    pin_single_key,
    pin_two_keys_logistic,
    pin_causal_first_row,
    pin_identity_values_expose_softmax,
    pin_key_shift_invariance,
    pin_value_affine,
    pin_key_permutation,
    pin_scale_folding,
    pin_mask_special_cases,
    pin_block_mask_brute_force,
    pin_library_sdpa,
    pin_finite_differences,
    pin_backward_invariants,
    pin_rows_match_full,
    pin_kv_library_sdpa,
    pin_kv_identical_keys,
    pin_kv_square_and_suffix,
    pin_kv_split_merge,
    pin_philox_known_answers,
    pin_dropout_zero_is_plain,
    pin_dropout_torch_autograd,
    pin_dropout_mask_rule,
    pin_dropout_keep_rate,
]
