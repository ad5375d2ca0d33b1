"""C-ABI boundary on the CPU: the library loads, exports every entry point
that include/fa.h declares, and rejects bad arguments with status codes
before any HIP call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_attention_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "fa.h")

# fake, 256-byte-aligned non-null addresses: never dereferenced, because every
# call below fails validation before reaching HIP
P = 0x100000
MIS = 0x100008  # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED), names
    lib = fa.lib()
    for n in names:
        assert getattr(lib, n) is not None


def _fwd(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H=1, N=128, d=64, scale=0.125, causal=0, mask=None)
    a.update(kw)
    return fa.lib().fa_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"],
                           a["d"], a["scale"], a["causal"], a["mask"], None)


def _bwd(**kw):
    a = dict(dO=P, Q=P, K=P, V=P, O=P, LSE=P, dQ=P, dK=P, dV=P, B=1, H=1, N=128, d=64,
             scale=0.125, causal=0, mask=None, ws=P, wsb=1 << 30)
    a.update(kw)
    return fa.lib().fa_bwd(a["dO"], a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["dQ"], a["dK"],
                           a["dV"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                           a["mask"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("fn", ["fwd", "fwd_f32"])
def test_forward_validation(fn):
    f = {"fwd": fa.lib().fa_fwd, "fwd_f32": fa.lib().fa_fwd_f32}[fn]

    def call(**kw):
        a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H=1, N=128, d=64, scale=0.125, causal=0)
        a.update(kw)
        return f(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"], a["d"],
                 a["scale"], a["causal"], None, None)

    assert call(Q=None) == 1
    assert call(LSE=None) == 1
    assert call(N=-1) == 2
    assert call(B=-3) == 2
    assert call(d=100) == 3                     # head dims: multiples of 8 in [8, 256]
    assert call(d=252) == 3
    assert call(d=264) == 3
    assert call(d=512) == 3
    assert call(d=4) == 3
    assert call(d=0) == 3
    assert call(O=MIS) == 4
    assert call(scale=0.0) == 5
    assert call(scale=-1.0) == 5
    assert call(scale=float("nan")) == 5
    assert call(scale=float("inf")) == 5
    assert call(causal=2) == 5
    assert call(N=1 << 30, d=128) == 2          # per-head slab exceeds 2^30 elements
    assert call(N=1 << 23, d=128) == 2
    assert call(N=(1 << 24) + 8, d=64) == 2
    # empty problems are valid no-ops and touch nothing (even with NULL pointers)
    assert call(B=0, Q=None) == 0
    assert call(H=0) == 0
    assert call(N=0) == 0


def test_backward_validation():
    ws = fa.fa_bwd_workspace_bytes(1, 1, 128, 64)
    assert ws > 0 and ws % 256 == 0
    assert _bwd(dQ=None) == 1
    assert _bwd(d=33) == 3
    assert _bwd(d=252) == 3                       # multiples of 8 up to 256
    assert _bwd(d=264) == 3
    assert _bwd(dV=MIS) == 4
    assert _bwd(scale=0.0) == 5
    assert _bwd(ws=None) == 6
    assert _bwd(wsb=ws - 1) == 6
    assert _bwd(ws=P + 128, wsb=ws) == 6          # workspace must be 256-byte aligned
    assert _bwd(B=0, dO=None) == 0


def test_noalloc_backward_validation():
    """The no-allocation backward checks like fa_bwd (without a workspace)
    and refuses, before any HIP call, a problem whose scratch exceeds its
    static array."""
    lib = fa.lib()

    def call(**kw):
        a = dict(dO=P, Q=P, K=P, V=P, O=P, LSE=P, dQ=P, dK=P, dV=P, B=1, H=1, N=128, d=64,
                 scale=0.125, causal=0)
        a.update(kw)
        return lib.fa_bwd_noalloc(a["dO"], a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["dQ"],
                                  a["dK"], a["dV"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                  a["causal"], None, None)

    assert call(dK=None) == 1
    assert call(d=33) == 3
    assert call(d=264) == 3
    assert call(LSE=MIS) == 4
    assert call(scale=float("inf")) == 5
    assert call(B=0, dO=None) == 0
    # the largest problem whose two scratch vectors fit, and one row more
    rows_max = fa.FA_NOALLOC_SCRATCH_BYTES // 8
    assert fa.fa_bwd_workspace_bytes(1, 1, rows_max, 8) <= fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_bwd_workspace_bytes(1, 1, rows_max + 1, 8) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert call(N=rows_max + 1, d=8) == 8
    assert call(B=4, H=8, N=rows_max // 16, d=8) == 8
    assert "FA_NOALLOC_SCRATCH_BYTES" in lib.fa_status_str(8).decode()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES


def test_backward_phases_head_dims():
    """The phase entry points run only the matrix-core kernels (d <= 128)."""
    lib = fa.lib()
    assert lib.fa_bwd_prep(P, P, P, 1, 1, 128, 136, P, 1 << 30, None) == 3
    assert lib.fa_bwd_dq(P, P, P, P, P, 1, 1, 128, 136, 0.125, 0, None, P, 1 << 30, None) == 3
    assert lib.fa_bwd_dkdv(P, P, P, P, P, P, 1, 1, 128, 256, 0.125, 0, None, P, 1 << 30, None) == 3


def test_f32_backward_head_dims():
    def call(d):
        return fa.lib().fa_bwd_f32(P, P, P, P, P, P, P, P, P, 1, 1, 128, d, 0.125, 0, None, P,
                                   1 << 30, None)

    assert call(252) == 3                         # the fp32 path takes multiples of 8 up to 256
    assert call(264) == 3
    assert call(4) == 3


def test_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(0, 1, 128, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 0, 64) == 0
    # two fp32 vectors per row (D and LSE in base 2), each 256-byte padded
    assert fa.fa_bwd_workspace_bytes(2, 16, 8192, 128) == 2 * 2 * 16 * 8192 * 4
    assert fa.fa_bwd_workspace_bytes(1, 1, 3, 64) == 2 * 256


def test_status_strings():
    lib = fa.lib()
    for s in range(9):
        assert lib.fa_status_str(s)
    assert lib.fa_last_hip_error() is not None
    assert fa.version().startswith("fa-gfx950")


def test_binding_raises_on_bad_status():
    with pytest.raises(fa.FaError) as e:
        fa._check(3)
    assert "FA_ERR_HEADDIM" in str(e.value)


def _dec(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H=2, Nq=4, Nk=1000, d=128, scale=0.1, causal=1,
             ws=P, wsb=1 << 30)
    a.update(kw)
    return fa.lib().fa_decode(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Nq"],
                              a["Nk"], a["d"], a["scale"], a["causal"], a["ws"], a["wsb"], None)


def test_decode_validation():
    ws = fa.fa_decode_workspace_bytes(1, 2, 4, 1000, 128)
    assert ws > 0 and ws % 256 == 0
    assert _dec(Q=None) == 1
    assert _dec(LSE=None) == 1
    assert _dec(K=None) == 1                      # keys present: K and V required
    assert _dec(Nq=-1) == 2
    assert _dec(Nk=-1) == 2
    assert _dec(Nk=1 << 23) == 2                  # key slab exceeds 2^30 elements
    assert _dec(d=100) == 3
    assert _dec(d=264) == 3
    assert _dec(d=252) == 3
    assert _dec(O=MIS) == 4
    assert _dec(scale=0.0) == 5
    assert _dec(causal=3) == 5
    assert _dec(ws=None) == 6
    assert _dec(wsb=ws - 1) == 6
    assert _dec(ws=P + 64, wsb=ws) == 6           # workspace must be 256-byte aligned
    assert _dec(Nq=0, Q=None, O=None) == 0        # empty: nothing done
    assert _dec(B=0) == 0


def test_decode_workspace_bytes():
    assert fa.fa_decode_workspace_bytes(0, 1, 1, 100, 64) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 0, 100, 64) == 0
    # one chunk of a short key range: O part (Nq x d fp32) and LSE part, each
    # 256-byte padded
    assert fa.fa_decode_workspace_bytes(1, 1, 3, 100, 64) == 768 + 256
    assert fa.fa_decode_workspace_bytes(1, 1, 3, 100, 40) == 512 + 256
    # the split count depends on the shape only and grows with Nk
    a = fa.fa_decode_workspace_bytes(1, 8, 1, 4096, 128)
    b = fa.fa_decode_workspace_bytes(1, 8, 1, 65536, 128)
    assert 0 < a < b


def test_dropout_validation():
    lib = fa.lib()

    def fwd(**kw):
        a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H=1, N=128, d=64, scale=0.125, causal=0,
                 mask=None, p=0.1, seed=1)
        a.update(kw)
        return lib.fa_fwd_dropout(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"],
                                  a["N"], a["d"], a["scale"], a["causal"], a["mask"], a["p"],
                                  a["seed"], None)

    def bwd(**kw):
        a = dict(p=0.1, seed=1, ws=P, wsb=1 << 30, N=128, d=64, Q=P)
        a.update(kw)
        return lib.fa_bwd_dropout(P, a["Q"], P, P, P, P, P, P, P, 1, 1, a["N"], a["d"], 0.125, 0,
                                  None, a["p"], a["seed"], a["ws"], a["wsb"], None)

    for f in (fwd, bwd):
        assert f(p=1.0) == 5
        assert f(p=-0.25) == 5
        assert f(p=float("nan")) == 5
        assert f(p=float("inf")) == 5
        assert f(Q=None) == 1
        assert f(d=100) == 3
        assert f(d=136) == 3             # dropout stops at d = 128
        assert f(N=0, p=0.5) == 0        # empty: nothing done
        assert f(N=0, p=2.0) == 5        # but the probability is still checked
    assert bwd(ws=None) == 6


def test_fp8_validation():
    lib = fa.lib()

    def call(**kw):
        a = dict(B=1, H=1, N=128, d=128, qs=0.01, ks=0.01, vs=0.01, ws=P, wsb=1 << 30, Q=P)
        a.update(kw)
        return lib.fa_fwd_fp8(a["Q"], P, P, P, P, a["B"], a["H"], a["N"], a["d"], 0.08, a["qs"],
                              a["ks"], a["vs"], 0, a["ws"], a["wsb"], None)

    assert call(Q=None) == 1
    assert call(d=96) == 3                       # FP8 forward: d = 64 or 128
    assert call(d=32) == 3
    assert call(qs=0.0) == 5
    assert call(vs=float("nan")) == 5
    assert call(ks=-1.0) == 5
    assert call(ws=None) == 6
    assert call(wsb=fa.fa_fwd_fp8_workspace_bytes(1, 1, 128, 128) - 1) == 6
    assert call(N=0) == 0
    # V^T in 64-key tiles: B*H*ceil(N/64)*64*d bytes, 256-byte padded
    assert fa.fa_fwd_fp8_workspace_bytes(2, 3, 100, 64) == 2 * 3 * 2 * 64 * 64
    assert fa.fa_fwd_fp8_workspace_bytes(1, 1, 100, 96) == 0
