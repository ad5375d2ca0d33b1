"""Wait states before inline-asm reads of MFMA results, checked in the
generated gfx950 code (host-side: hipcc cross-compiles, no GPU needed).

The kernels take row maxima of freshly computed scores with v_max3_f32
written as inline asm. The ISA requires a number of wait states between an
MFMA writing a VGPR and a vector ALU instruction reading it; the compiler
inserts them before its own instructions but does not look inside asm. A
read placed too close returns the register's previous contents, which made
the forward's rescale decisions (and its last bits) depend on timing.

The required count is taken from the compiler itself: a probe kernel in
which a compiler-generated VALU instruction reads an MFMA result at once
shows the s_nop the compiler puts in between. Each kernel source is then
compiled to assembly and every asm VALU read of an MFMA-written VGPR is
checked to come at least that many wait states after the MFMA along every
path of the control-flow graph (one wait state per instruction, N + 1 per
s_nop N; a compiler-generated write of the register ends the check for it).
With the waits taken out of the forward and decode sources, the check
reports 12 and 11 wait states missing before their first asm row max.

The reverse order is checked too: an MFMA written as inline asm (the
hand-scheduled backward kernels accumulate into AGPRs that way) reads A and
B operands that vector ALU instructions may have written just before, which
the ISA also separates by wait states the compiler does not insert for asm.
The count again comes from the compiler (a probe whose MFMA reads a freshly
converted operand), and every asm MFMA's A and B registers are checked
against the last vector ALU write along every path.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_io_aware_attention_amd"))
import build  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")

PROBE = r"""
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ void probe_bf16(const bf16x8 *a, float *o) {
  f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], f32x16{}, 0, 0, 0);
  o[threadIdx.x] = s[0] + s[5];
}
__global__ void probe_fp8(const i32x8 *a, float *o) {
  f32x16 s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[threadIdx.x], a[threadIdx.x + 64], f32x16{},
                                                             0, 0, 0, 127, 0, 127);
  o[threadIdx.x] = s[0] + s[5];
}
"""

PROBE_V = r"""
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ void probe_valu_to_mfma(const float *x, const bf16x8 *a, f32x16 *o) {
  const float v = x[threadIdx.x];
  bf16x8 b;
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(v * (float)(i + 1));
  o[threadIdx.x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], b, f32x16{}, 0, 0, 0);
}
"""


def _asm(src, out_dir, name):
    out = os.path.join(out_dir, name + ".s")
    flags = [f for f in build.COMMON_FLAGS if f != "-fPIC"]
    cmd = [build.HIPCC, "-x", "hip", "--cuda-device-only", "-S", *flags,
           "-I" + build.CSRC, src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().splitlines()


def _vgprs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return range(int(m.group(1)), int(m.group(2)) + 1)
    m = re.fullmatch(r"v(\d+)", tok)
    return [int(m.group(1))] if m else []


def _instrs(lines):
    """(opcode, operands, in_asm) for each instruction of the listing."""
    in_asm = False
    for line in lines:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":") or ":" in s.split()[0]:
            continue
        parts = s.split(None, 1)
        ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
        yield parts[0], ops, in_asm


def _wait_states(op, ops):
    return int(ops[0]) + 1 if op == "s_nop" else 1


def _probe_requirements(tmp):
    src = os.path.join(tmp, "probe.hip")
    open(src, "w").write(PROBE)
    lines = _asm(src, tmp, "probe")
    req, kind, dst, since = {}, None, set(), 0
    for op, ops, _ in _instrs(lines):
        if op.startswith("v_mfma"):
            kind, dst, since = op, set(_vgprs(ops[0])), 0
            continue
        if kind is None:
            continue
        if op.startswith("v_") and any(r in dst for t in ops[1:] for r in _vgprs(t)):
            req[kind] = since  # the first instruction that reads the result
            kind = None
            continue
        since += _wait_states(op, ops)
    return req


def _agprs(tok):
    m = re.fullmatch(r"a\[(\d+):(\d+)\]", tok)
    if m:
        return range(int(m.group(1)), int(m.group(2)) + 1)
    m = re.fullmatch(r"a(\d+)", tok)
    return [int(m.group(1))] if m else []


def _check_agprs(lines, req):
    """Largest deficit over accesses to AGPRs that an MFMA is still writing:
    any instruction other than an MFMA taking the register as its own
    accumulator (C operand and destination, which the matrix core chains
    without waits) must come at least the MFMA's result latency after it,
    along every path. The compiler inserts these waits for its own MFMAs; the
    asm ones (the AGPR accumulators of the hand-scheduled loops) rely on the
    code around them."""
    worst = (0, None)
    for blocks in _blocks(lines):
        index = {b[0]: k for k, b in enumerate(blocks) if b[0] is not None}
        entry = [None] * len(blocks)
        entry[0] = {}
        work = [0]
        while work:
            k = work.pop()
            pend = dict(entry[k])
            _, instrs, succ, fall = blocks[k]
            for op, ops, in_asm in instrs:
                if op.startswith("v_mfma"):
                    chained = set(_agprs(ops[0])) if ops else set()
                    touched = [r for t in ops[1:3] for r in _agprs(t)]
                    touched += [r for t in ops[3:4] for r in _agprs(t) if r not in chained]
                else:
                    touched = [r for t in ops for r in _agprs(t)]
                for r in touched:
                    if pend.get(r, 0) > worst[0]:
                        worst = (pend[r], f"{op} {', '.join(ops)}")
                w = _wait_states(op, ops)
                pend = {r: n - w for r, n in pend.items() if n - w > 0}
                if op.startswith("v_mfma") and ops:
                    need = next((n for kk, n in req.items() if op.startswith(kk)), max(req.values()))
                    for r in _agprs(ops[0]):
                        pend[r] = need
            nxt = [index[t] for t in succ if t in index]
            if fall and k + 1 < len(blocks):
                nxt.append(k + 1)
            for n in nxt:
                old = entry[n]
                merged = dict(old or {})
                for r, v in pend.items():
                    merged[r] = max(merged.get(r, 0), v)
                if old is None or merged != old:
                    entry[n] = merged
                    work.append(n)
    return worst


def _probe_valu_to_mfma(tmp):
    """Wait states the compiler puts between the last vector ALU write of an
    MFMA's A or B operand and the MFMA (probe_valu_to_mfma)."""
    src = os.path.join(tmp, "probe_v.hip")
    open(src, "w").write(PROBE_V)
    lines = _asm(src, tmp, "probe_v")
    fn = _blocks(lines)
    for blocks in fn:
        seq = [i for b in blocks for i in b[1]]
        if not any(op.startswith("v_mfma") for op, _, _ in seq):
            continue
        k = next(i for i, (op, _, _) in enumerate(seq) if op.startswith("v_mfma"))
        srcs = {r for t in seq[k][1][1:3] for r in _vgprs(t)}
        since = 0
        for op, ops, _ in reversed(seq[:k]):
            if op.startswith("v_") and not op.startswith("v_mfma") and ops and \
                    any(r in srcs for r in _vgprs(ops[0])):
                return since
            since += _wait_states(op, ops)
    raise AssertionError("no MFMA reading a vector ALU result in the probe")


def _blocks(lines):
    """Functions of the listing as lists of basic blocks: (label, instructions,
    successor labels, falls through)."""
    funcs, blocks, cur, label = [], [], [], None

    def close(fall):
        nonlocal cur, label
        if cur or label is not None:
            blocks.append([label, cur, [], fall])
        cur, label = [], None

    in_asm = False
    for line in lines:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";"):
            continue
        m = re.match(r"([\w.$]+):(\s|;|$)", s)
        if m:
            name = m.group(1)
            if not name.startswith("."):       # a new function
                close(False)
                if blocks:
                    funcs.append(blocks)
                blocks = []
            else:
                close(True)
            label = name
            continue
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        ops = [t.strip() for t in parts[1].split(";")[0].split(",")] if len(parts) > 1 else []
        cur.append((parts[0], ops, in_asm))
        if parts[0].startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            tgt = ops[0] if parts[0].startswith(("s_branch", "s_cbranch")) and ops else None
            close(not parts[0].startswith(("s_branch", "s_endpgm", "s_setpc")))
            blocks[-1][2] = [tgt] if tgt else []
    close(False)
    if blocks:
        funcs.append(blocks)
    return funcs


def _check(lines, req):
    """Largest deficit (wait states missing) over asm VALU reads of
    MFMA-written VGPRs along every control-flow path, and where it occurs.
    State at a block entry: for each VGPR with an MFMA write still in flight,
    the wait states it still needs (the worst over the paths that reach it)."""
    worst = (0, None)
    for blocks in _blocks(lines):
        index = {b[0]: k for k, b in enumerate(blocks) if b[0] is not None}
        entry = [None] * len(blocks)
        entry[0] = {}
        work = [0]
        while work:
            k = work.pop()
            pend = dict(entry[k])
            _, instrs, succ, fall = blocks[k]
            for op, ops, in_asm in instrs:
                if op.startswith("v_") and in_asm and not op.startswith("v_mfma"):
                    for t in ops[1:]:
                        for r in _vgprs(t):
                            if pend.get(r, 0) > worst[0]:
                                worst = (pend[r], f"{op} {', '.join(ops)}")
                w = _wait_states(op, ops)
                pend = {r: n - w for r, n in pend.items() if n - w > 0}
                if op.startswith("v_mfma"):
                    need = next((n for kk, n in req.items() if op.startswith(kk)), max(req.values()))
                    for r in _vgprs(ops[0]):
                        pend[r] = need
                elif ops and op.startswith(("v_", "ds_read", "buffer_load", "global_load")):
                    for r in _vgprs(ops[0]):
                        pend.pop(r, None)
            nxt = [index[t] for t in succ if t in index]
            if fall and k + 1 < len(blocks):
                nxt.append(k + 1)
            for n in nxt:
                old = entry[n]
                merged = dict(old or {})
                for r, v in pend.items():
                    merged[r] = max(merged.get(r, 0), v)
                if old is None or merged != old:
                    entry[n] = merged
                    work.append(n)
    return worst


def _check_operands(lines, need):
    """Largest deficit over the A and B operand reads of asm MFMAs that follow
    a vector ALU write of the register too closely, along every path."""
    worst = (0, None)
    for blocks in _blocks(lines):
        index = {b[0]: k for k, b in enumerate(blocks) if b[0] is not None}
        entry = [None] * len(blocks)
        entry[0] = {}
        work = [0]
        while work:
            k = work.pop()
            pend = dict(entry[k])
            _, instrs, succ, fall = blocks[k]
            for op, ops, in_asm in instrs:
                if op.startswith("v_mfma") and in_asm:
                    for t in ops[1:3]:
                        for r in _vgprs(t):
                            if pend.get(r, 0) > worst[0]:
                                worst = (pend[r], f"{op} {', '.join(ops)}")
                w = _wait_states(op, ops)
                pend = {r: n - w for r, n in pend.items() if n - w > 0}
                if ops and op.startswith("v_") and not op.startswith(("v_mfma", "v_accvgpr_read")):
                    for r in _vgprs(ops[0]):
                        pend[r] = need
                elif ops and op.startswith(("v_mfma", "v_accvgpr_read", "ds_read", "buffer_load",
                                            "global_load")):
                    for r in _vgprs(ops[0]):
                        pend.pop(r, None)
            nxt = [index[t] for t in succ if t in index]
            if fall and k + 1 < len(blocks):
                nxt.append(k + 1)
            for n in nxt:
                old = entry[n]
                merged = dict(old or {})
                for r, v in pend.items():
                    merged[r] = max(merged.get(r, 0), v)
                if old is None or merged != old:
                    entry[n] = merged
                    work.append(n)
    return worst


def test_asm_reads_of_mfma_results_wait_long_enough():
    tmp = tempfile.mkdtemp(prefix="fa_isa_")
    try:
        req = _probe_requirements(tmp)
        assert set(req) == {"v_mfma_f32_32x32x16_bf16", "v_mfma_scale_f32_32x32x64_f8f6f4"}, req
        assert all(n >= 1 for n in req.values()), req
        srcs = ["fa_fwd.hip", "fa_fwd_wide.hip", "fa_decode.hip", "fa_fp8.hip", "fa_bwd.hip", "fa_bwd_wide.hip"]
        with concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
            listings = list(ex.map(lambda s: _asm(os.path.join(build.CSRC, s), tmp, s), srcs))
        need = _probe_valu_to_mfma(tmp)
        assert need >= 1, need
        for name, lines in zip(srcs, listings):
            deficit, where = _check(lines, req)
            print(f"{name}: largest deficit {deficit} ({where})")
            assert deficit == 0, f"{name}: asm read of an MFMA result {deficit} wait states early: {where}"
            deficit, where = _check_operands(lines, need)
            print(f"{name}: asm MFMA operands, largest deficit {deficit} ({where})")
            assert deficit == 0, f"{name}: asm MFMA reads a vector ALU result {deficit} wait states early: {where}"
            deficit, where = _check_agprs(lines, req)
            print(f"{name}: AGPR accumulators, largest deficit {deficit} ({where})")
            assert deficit == 0, f"{name}: access to an AGPR {deficit} wait states before its MFMA is done: {where}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
