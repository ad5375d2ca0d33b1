"""Benchmark: exact attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
fa_fwd, then the backward's three kernels (fa_bwd_prep, fa_bwd_dq,
fa_bwd_dkdv, which together are fa_bwd). The default workload is the
long-context causal configuration B=2, H=16, N=8192, d=128 (Q and K scaled
by 2), bf16 storage, inputs resident in HBM before timing starts.

Throughput uses the algorithmic FLOP count of the method: forward
4*B*H*N^2*d, backward 2.5x that, both halved under the causal mask (and
scaled by the kept-block fraction under a block mask). Per-kernel durations
come from HIP events recorded on the stream the kernels run on.

Prints ONE JSON line. Options: --steps K --warmup W --config {1..5}
--cpu-heads H (heads of the CPU fp64 reference timed as the baseline; 0 skips)
--supp-steps S (the same shape without the causal mask) --dropout-steps S (the
same workload with dropout p=0.1) --decode-steps S (the split-KV decode path on
its own workload, HBM-bound) --fp8-steps S (the FP8 forward on the same
shape) --wide-steps S / --wide-bwd S (the forward and backward at head dim
256 on the same B, H, N) --other-steps S (the GPT-2-shaped, 64K dense and
block-sparse workloads) --sweep-steps S (the block-sparse shape at six mask
densities, with a linear fit of time against kept blocks) --cpu-other 0|1
(the CPU reference also on samples of the other workloads) --padded-steps S
(the headline B, H, N at head dims 64, 72, 96 and 128: dims between the
kernel widths run zero-padded in the next one) --clock-seconds S (the
headline step repeated for S seconds while the GPU's gfx clock and socket
power are sampled through amdsmi: the clock the kernels actually run at
under the board's power limit) --only LIST (run
only these supplementary legs). The supplementary runs are reported beside
the headline and never enter `value`.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
METRIC = "attention fwd+bwd TFLOP/s and % of MFMA bf16 peak at N=8192, d=128, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--supp-steps", type=int, default=10,
                    help="timed steps of the supplementary non-causal run (0: skip)")
    ap.add_argument("--decode-steps", type=int, default=10,
                    help="timed calls of the supplementary split-KV decode run (0: skip)")
    ap.add_argument("--dropout-steps", type=int, default=5,
                    help="timed steps of the supplementary dropout run (0: skip)")
    ap.add_argument("--fp8-steps", type=int, default=10,
                    help="timed calls of the supplementary FP8 forward run (0: skip)")
    ap.add_argument("--wide-steps", type=int, default=10,
                    help="timed calls of the supplementary head-dim-256 forward run (0: skip)")
    ap.add_argument("--wide-bwd", type=int, default=5,
                    help="timed calls of the supplementary head-dim-256 backward (0: skip)")
    ap.add_argument("--other-steps", type=int, default=10,
                    help="timed steps of each of the other workloads (GPT-2 shape, 64K dense "
                         "forward, block-sparse) (0: skip)")
    ap.add_argument("--sweep-steps", type=int, default=3,
                    help="timed steps per density of the block-sparse density sweep (0: skip)")
    ap.add_argument("--padded-steps", type=int, default=3,
                    help="timed steps at head dims 64, 72, 96, 128 on the headline B, H, N "
                         "(0: skip)")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="seconds of repeated headline steps while the gfx clock and socket "
                         "power are sampled (0: skip)")
    ap.add_argument("--cpu-other", type=int, default=1,
                    help="also time the CPU reference on samples of the other workloads (0: skip)")
    ap.add_argument("--only", default="",
                    help="comma-separated subset of supplementary runs to do after the headline "
                         "(supp,dropout,fp8,wide,decode,other,sweep,padded,clock); empty: all; "
                         "'headline': none")
    return ap.parse_args()


# Sources the forward and backward kernels are built from (the decode path
# and the host-side ABI layer do not enter them).
KERNEL_SOURCES = ("csrc/fa_common.h", "csrc/fa_internal.h", "csrc/fa_wide.h", "csrc/fa_fwd.hip",
                  "csrc/fa_bwd.hip", "csrc/fa_bwd_wide.hip", "build.py")


def kernel_source_sha256():
    """sha256 over the forward/backward kernel sources and their build script
    (as recorded in the traffic profile when its counters were taken)."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "exact_io_aware_attention_amd")
    for rel in KERNEL_SOURCES:
        f = os.path.join(pkg, rel)
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload_tag, symbol):
    """HBM bytes per dispatch of `symbol` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when there is none for this
    workload or the kernels changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_tag}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Kernel sources sha256 \([^)]*\): `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_sha256():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if cells and cells[0] == symbol:
            return int(cells[-1])
    return None


def flop_counts(cfg, mask):
    """Algorithmic FLOPs of one forward and of one backward."""
    fwd = 4.0 * cfg.B * cfg.H * cfg.N ** 2 * cfg.d
    if cfg.causal:
        fwd *= 0.5
    if mask is not None:
        fwd *= float(mask.mean())
    return fwd, 2.5 * fwd


# Split-KV decode workload: one new query per sequence against a 32K-token
# cache, 8 sequences x 32 heads, d = 128 (the key/value cache is 4.3 GB, so
# the path is bound by reading it once from HBM).
DECODE_SHAPE = dict(B=8, H=32, Nq=1, Nk=32768, d=128)


def decode_run(steps, d=None):
    """fa_decode on DECODE_SHAPE (head dim d if given) with seeded N(0,1) bf16
    inputs drawn on the device; median of `steps` calls timed with HIP events
    on the stream."""
    import torch
    import exact_io_aware_attention_amd as fa
    B, H, Nq, Nk = (DECODE_SHAPE[x] for x in ("B", "H", "Nq", "Nk"))
    d = DECODE_SHAPE["d"] if d is None else d
    g = torch.Generator(device="cuda")
    g.manual_seed(31337)
    Q = torch.randn((B, H, Nq, d), generator=g, device="cuda").bfloat16()
    K = torch.randn((B, H, Nk, d), generator=g, device="cuda").bfloat16()
    V = torch.randn((B, H, Nk, d), generator=g, device="cuda").bfloat16()
    O = torch.empty_like(Q)
    LSE = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d), dtype=torch.uint8,
                     device="cuda")
    scale = d ** -0.5
    for _ in range(3):
        fa.fa_decode(Q, K, V, O, LSE, scale, causal=True, workspace=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        fa.fa_decode(Q, K, V, O, LSE, scale, causal=True, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    t = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
    # algorithmic bytes: K and V once, Q and O once, LSE
    byts = 2 * B * H * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4
    gbs = byts / t / 1e9
    out = {"workload": "split-KV decode (supplementary)", **DECODE_SHAPE, "d": d, "causal": True,
           "us": round(t * 1e6, 1), "gbs": round(gbs, 1), "bound": "hbm",
           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": byts,
           "steps": steps}
    del Q, K, V, ws
    torch.cuda.empty_cache()
    return out


# Densities of the block-sparse sweep: the band |I - J| <= 1 plus this fraction
# of the other 128 x 128 blocks (the block-sparse workload itself keeps 10%).
SWEEP_KEEP = (0.01, 0.04, 0.10, 0.23, 0.49, 1.0)


def workload_run(cfg, steps, mask=None, seed=None):
    """fa_fwd, and when the workload has a backward fa_bwd's three kernels, on
    cfg's shape with seeded N(0,1) bf16 inputs drawn on the device (Q and K
    times cfg.qk_mult); per-kernel HIP-event averages over `steps` calls
    after one warm-up. mask: a numpy block mask or None."""
    import torch
    import exact_io_aware_attention_amd as fa
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.cfg_id if seed is None else seed)
    shp = (cfg.B, cfg.H, cfg.N, cfg.d)
    Q, K, V, dO = (torch.randn(shp, generator=g, device=dev).mul_(m).to(torch.bfloat16)
                   for m in (cfg.qk_mult, cfg.qk_mult, 1.0, 1.0))
    M = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).to(dev)
    O = torch.empty_like(Q)
    LSE = torch.empty(shp[:3], dtype=torch.float32, device=dev)
    bwd = cfg.has_bwd
    if bwd:
        dQ, dK, dV = (torch.empty_like(Q) for _ in range(3))
        ws = fa.new_workspace(*shp, dev)
    sc, causal = cfg.scale, cfg.causal

    def run(ev=None):
        ev and ev[0].record()
        fa.fa_fwd(Q, K, V, O, LSE, sc, causal=causal, blockmask=M)
        ev and ev[1].record()
        if bwd:
            fa.fa_bwd_prep(dO, O, LSE, ws)
            ev and ev[2].record()
            fa.fa_bwd_dq(dO, Q, K, V, dQ, sc, ws, causal=causal, blockmask=M)
            ev and ev[3].record()
            fa.fa_bwd_dkdv(dO, Q, K, V, dK, dV, sc, ws, causal=causal, blockmask=M)
            ev and ev[4].record()

    run()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    n_ev = 5 if bwd else 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    names = ["fwd", "bwd_prep", "bwd_dq", "bwd_dkdv"][:n_ev - 1]
    us = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps * 1e3 for j, n in enumerate(names)}
    fwd_f, bwd_f = flop_counts(cfg, mask)
    out = {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
           "causal": cfg.causal, "qk_mult": cfg.qk_mult,
           "density": None if mask is None else round(float(mask.mean()), 5),
           "fwd_us": round(us["fwd"], 2), "fwd_flop": fwd_f,
           "fwd_tflops": round(fwd_f / us["fwd"] / 1e6, 2),
           "fwd_frac_of_peak": round(fwd_f / us["fwd"] / 1e6 / PEAK_BF16_TFLOPS, 4),
           "device_bytes_allocated_during_calls": int(extra), "steps": steps}
    if bwd:
        b_us = us["bwd_prep"] + us["bwd_dq"] + us["bwd_dkdv"]
        out.update(bwd_us=round(b_us, 2), bwd_flop=bwd_f,
                   bwd_kernels_us={n: round(us[n], 2) for n in names[1:]},
                   bwd_tflops=round(bwd_f / b_us / 1e6, 2),
                   bwd_frac_of_peak=round(bwd_f / b_us / 1e6 / PEAK_BF16_TFLOPS, 4),
                   dkdv_tflops=round(0.8 * bwd_f / us["bwd_dkdv"] / 1e6, 2))
    del Q, K, V, dO, O, LSE
    if bwd:
        del dQ, dK, dV, ws
    torch.cuda.empty_cache()
    return out


def sparse_sweep(cfg, steps):
    """The block-sparse workload's shape at several mask densities (the band
    plus a growing fraction of the other blocks): forward and backward time
    against kept blocks, with a least-squares line t = a + b * kept and its
    largest relative residual."""
    import synthetic as syn
    nb = (cfg.N + 127) // 128
    rows = []
    for f in SWEEP_KEEP:
        mask = syn.block_mask(nb, keep_frac=f)
        r = workload_run(cfg, steps, mask=mask)
        rows.append({"keep_frac_off_band": f, "kept_blocks": int(mask.sum()),
                     "density": r["density"], "fwd_us": r["fwd_us"], "bwd_us": r["bwd_us"],
                     "fwd_tflops": r["fwd_tflops"], "bwd_tflops": r["bwd_tflops"]})
    kept = np.array([r["kept_blocks"] for r in rows], float)
    fit = {}
    for key in ("fwd_us", "bwd_us"):
        t = np.array([r[key] for r in rows], float)
        b, a = np.polyfit(kept, t, 1)
        res = np.max(np.abs(t - (a + b * kept)) / t)
        fit[key] = {"intercept_us": round(float(a), 2), "us_per_kept_block": round(float(b), 5),
                    "max_rel_residual": round(float(res), 4)}
    return {"workload": cfg.name + " shape, mask density sweep (supplementary)",
            "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d, "points": rows,
            "linear_fit": fit, "steps": steps}


def _smi_handle_for_cuda0(amdsmi, handles):
    """The amdsmi handle of the device torch calls cuda:0, matched by PCI
    address (amdsmi may list devices that HIP does not expose); the first
    handle when the address cannot be read."""
    import torch
    p = torch.cuda.get_device_properties(0)
    want = (getattr(p, "pci_domain_id", None), getattr(p, "pci_bus_id", None),
            getattr(p, "pci_device_id", None))
    if None not in want:
        for h in handles:
            try:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                dev = rest.split(".")[0]
                if (int(dom, 16), int(bus, 16), int(dev, 16)) == want:
                    return h
            except Exception:
                continue
    return handles[0]


def clock_under_load(step, seconds):
    """Repeats `step` (one headline step) for about `seconds` while a
    thread samples the GPU's current gfx clock and socket power through
    amdsmi every 50 ms; the first second (clock ramp) is dropped. Returns
    medians and ranges, the steps' own rate over the sampled window, and
    the bf16 MFMA peak scaled to the sampled clock (the published 2500
    TFLOP/s is at the 2400 MHz peak engine clock); None when amdsmi is not
    usable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        handles = amdsmi.amdsmi_get_processor_handles()
        handle = _smi_handle_for_cuda0(amdsmi, handles)
    except Exception as e:  # monitoring only: the bench goes on without it
        return {"error": f"amdsmi unavailable: {type(e).__name__}: {e}"}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                samples.append((time.perf_counter(), m.get("current_gfxclk"),
                                m.get("current_socket_power")))
            except Exception:
                pass
            stop.wait(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    marks = []
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        marks.append((time.perf_counter(), 20))
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    lo = t0 + 1.0
    win = [s for s in samples if s[0] > lo]
    clk = [s[1] for s in win if isinstance(s[1], (int, float))]
    pw = [s[2] for s in win if isinstance(s[2], (int, float))]
    done = [m for m in marks if m[0] > lo]
    out = {"samples": len(clk), "seconds": round(time.perf_counter() - t0, 2)}
    if clk:
        med = statistics.median(clk)
        out.update(gfxclk_mhz_median=med, gfxclk_mhz_min=min(clk), gfxclk_mhz_max=max(clk),
                   bf16_peak_at_clock_tflops=round(PEAK_BF16_TFLOPS * med / 2400.0, 1))
    if pw:
        out.update(socket_power_w_median=statistics.median(pw), socket_power_w_max=max(pw))
    if len(done) > 1:
        span = done[-1][0] - done[0][0]
        out["step_ms_in_window"] = round(span / sum(m[1] for m in done[1:]) * 1e3, 4)
    return out


def cpu_other(args):
    """The CPU reference (as is) on samples of the other workloads, on the
    same host threads: workloads 1, 2 and the block-sparse one in full
    (fwd+bwd), and the 256 sampled query rows of the
    64K dense forward with a labelled extrapolation to all of its rows.
    Rates use the same algorithmic FLOP counts as the GPU figures."""
    import oracle
    import synthetic as syn
    out = {}
    for cid in (1, 2):
        cfg = syn.CONFIGS[cid]
        q, k, v, do, mask = syn.config_inputs(cfg)
        t1 = time.perf_counter()
        oracle.attention(q, k, v, cfg.scale, causal=cfg.causal, blockmask=mask, do=do)
        dt = time.perf_counter() - t1
        f, b = flop_counts(cfg, mask)
        out[cfg.name] = {"s": round(dt, 3), "tflops": round((f + b) / dt / 1e12, 6),
                         "sample": "all heads, fwd+bwd"}
    cfg = syn.CONFIGS[5]
    q, k, v, do, mask = syn.config_inputs(cfg)
    nh = cfg.B * cfg.H
    hs = lambda x: x.reshape((1, cfg.B * cfg.H) + x.shape[2:])[:, :nh]  # noqa: E731
    t1 = time.perf_counter()
    oracle.attention(hs(q), hs(k), hs(v), cfg.scale, causal=cfg.causal, blockmask=mask, do=hs(do))
    dt = time.perf_counter() - t1
    f, b = flop_counts(cfg, mask)
    out[cfg.name] = {"s": round(dt, 3), "tflops": round(nh * (f + b) / (cfg.B * cfg.H) / dt / 1e12, 6),
                     "sample": f"{nh} of {cfg.B * cfg.H} heads, fwd+bwd"}
    cfg = syn.CONFIGS[4]
    q, k, v, _, _ = syn.config_inputs(cfg)
    rb, ri = syn.row_sample(cfg.B * cfg.H, cfg.N)
    t1 = time.perf_counter()
    oracle.attention_rows(q, k, v, cfg.scale, rb, ri, causal=cfg.causal)
    dt = time.perf_counter() - t1
    f, _ = flop_counts(cfg, None)
    rows = cfg.B * cfg.H * cfg.N
    out[cfg.name] = {"s": round(dt, 3), "tflops": round(f * len(rb) / rows / dt / 1e12, 6),
                     "sample": f"{len(rb)} of {rows} query rows, fwd",
                     "extrapolated_full_fwd_s": round(dt * rows / len(rb), 1)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention "
              "path here is a single-GPU kernel library and has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_attention_amd as fa
    import synthetic as syn

    cfg = syn.CONFIGS[args.config]
    if not cfg.has_bwd:
        raise SystemExit(f"config {cfg.cfg_id} has no backward; pick 1, 2, 3 or 5")
    q, k, v, do, mask = syn.config_inputs(cfg)
    dev = torch.device("cuda:0")

    def t(x):
        return torch.from_numpy(x).to(dev).to(torch.bfloat16)

    Q, K, V, dO = t(q), t(k), t(v), t(do)
    M = None if mask is None else torch.from_numpy(mask).to(dev)
    O = torch.empty_like(Q)
    LSE = torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    ws = fa.new_workspace(cfg.B, cfg.H, cfg.N, cfg.d, dev)
    scale, causal = cfg.scale, cfg.causal

    names = ["fwd", "bwd_prep", "bwd_dq", "bwd_dkdv"]

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        fa.fa_fwd(Q, K, V, O, LSE, scale, causal=causal, blockmask=M)
        if evs is not None:
            evs[1].record()
        fa.fa_bwd_prep(dO, O, LSE, ws)
        if evs is not None:
            evs[2].record()
        fa.fa_bwd_dq(dO, Q, K, V, dQ, scale, ws, causal=causal, blockmask=M)
        if evs is not None:
            evs[3].record()
        fa.fa_bwd_dkdv(dO, Q, K, V, dK, dV, scale, ws, causal=causal, blockmask=M)
        if evs is not None:
            evs[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {n: [ev[j].elapsed_time(ev[j + 1]) * 1e-3 for ev in events]  # seconds
           for j, n in enumerate(names)}
    avg = {n: sum(per[n]) / args.steps for n in names}

    fwd_flops, bwd_flops = flop_counts(cfg, mask)
    step_s = wall / args.steps
    value = (fwd_flops + bwd_flops) / step_s / 1e12
    fwd_s = avg["fwd"]
    bwd_s = avg["bwd_prep"] + avg["bwd_dq"] + avg["bwd_dkdv"]

    # algorithmic work per launch of each kernel: the forward's two
    # contractions; dK/dV's four (S and dP rebuilt, dV, dK); dQ's one
    # (its S and dP rebuild is extra work of this split); prep moves bytes
    E = cfg.B * cfg.H * cfg.N * cfg.d
    rows = cfg.B * cfg.H * cfg.N
    kernel_flops = {"fwd": fwd_flops, "bwd_dkdv": 0.8 * bwd_flops, "bwd_dq": 0.2 * bwd_flops,
                    "bwd_prep": 0.0}
    kernel_bytes = {"fwd": 4 * E * 2 + rows * 4, "bwd_prep": 2 * E * 2 + rows * 4 + 2 * rows * 4,
                    "bwd_dq": 4 * E * 2 + 2 * rows * 4 + E * 2,
                    "bwd_dkdv": 4 * E * 2 + 2 * rows * 4 + 2 * E * 2}
    dominant = max(names, key=lambda n: avg[n])
    ach = kernel_flops[dominant] / avg[dominant] / 1e12
    tf = lambda b: "true" if b else "false"  # noqa: E731
    # kernel template arguments: head width (the forward's: score depth and
    # O column width), causal, block-sparse, dropout
    flags = f"{cfg.d}, {tf(cfg.causal)}, {tf(mask is not None)}, false"
    # the forward's waves per workgroup: 4 for block-sparse masks and for
    # problems with fewer 256-row blocks than two per CU, else 8
    fwd_w = 4 if mask is not None or cfg.B * cfg.H * -(-cfg.N // 256) < 512 else 8
    symbols = {"fwd": f"fwd_bf16_kernel<{cfg.d}, {flags}, {fwd_w}>", "bwd_prep": f"bwd_pre_kernel<{cfg.d}>",
               "bwd_dq": f"bwd_dq_kernel<{flags}>", "bwd_dkdv": f"bwd_dkdv_kernel<{flags}>"}
    # without dropout the slot-scheduled dQ kernel, and at 64 < d <= 128 the
    # slot-scheduled dK/dV kernel (template arguments: row width, [both
    # gradients,] causal, block-sparse)
    bflags = f"{tf(cfg.causal)}, {tf(mask is not None)}"
    symbols["bwd_dq"] = f"bwd_wide_dq_kernel<{cfg.d}, {bflags}>"
    if cfg.d > 64:
        symbols["bwd_dkdv"] = f"bwd_wide_dkdv_kernel<128, 2, {bflags}>"
    tag = f"{cfg.name.replace('-', '_')}_b{cfg.B}h{cfg.H}n{cfg.N}d{cfg.d}"
    roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                # the whole forward, the whole backward (prep + dQ + dK/dV)
                # and the whole step, each on its own algorithmic FLOPs
                "fwd_frac": round(fwd_flops / fwd_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                "bwd_frac": round(bwd_flops / bwd_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                "step_frac": round(value / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(tag, symbols[dominant]),
                "algorithmic_bytes": kernel_bytes[dominant]}

    kernels = {n: {"avg_us": round(avg[n] * 1e6, 2),
                   "median_us": round(statistics.median(per[n]) * 1e6, 2),
                   "min_us": round(min(per[n]) * 1e6, 2),
                   "max_us": round(max(per[n]) * 1e6, 2),
                   "tflops": round(kernel_flops[n] / avg[n] / 1e12, 2) if kernel_flops[n] else None,
                   "gbs": round(kernel_bytes[n] / avg[n] / 1e9, 1)} for n in names}

    # Supplementary: the same shape and inputs without the causal mask (twice
    # the work), forward and backward times only; never part of `value`.
    only = set(x for x in args.only.split(",") if x)
    want = lambda name: not only or name in only  # noqa: E731
    supp = None
    if causal and mask is None and args.supp_steps > 0 and want("supp"):
        def run_nc():
            fa.fa_fwd(Q, K, V, O, LSE, scale, causal=False)
            fa.fa_bwd_prep(dO, O, LSE, ws)
            fa.fa_bwd_dq(dO, Q, K, V, dQ, scale, ws, causal=False)
            fa.fa_bwd_dkdv(dO, Q, K, V, dK, dV, scale, ws, causal=False)
        run_nc()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.supp_steps)]
        for e in ev:
            e[0].record()
            fa.fa_fwd(Q, K, V, O, LSE, scale, causal=False)
            e[1].record()
            fa.fa_bwd_prep(dO, O, LSE, ws)
            fa.fa_bwd_dq(dO, Q, K, V, dQ, scale, ws, causal=False)
            fa.fa_bwd_dkdv(dO, Q, K, V, dK, dV, scale, ws, causal=False)
            e[2].record()
        torch.cuda.synchronize()
        f_s = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
        b_s = statistics.median([e[1].elapsed_time(e[2]) * 1e-3 for e in ev])
        supp = {"workload": cfg.name + " shape without the causal mask (supplementary)",
                "fwd_ms": round(f_s * 1e3, 4), "fwd_tflops": round(2 * fwd_flops / f_s / 1e12, 2),
                "bwd_ms": round(b_s * 1e3, 4), "bwd_tflops": round(2 * bwd_flops / b_s / 1e12, 2),
                "steps": args.supp_steps}

    # Supplementary: the same workload with dropout p = 0.1 on P (fa_fwd_dropout
    # + fa_bwd_dropout); never part of `value`.
    dropout = None
    if args.dropout_steps > 0 and want("dropout"):
        p_drop, seed = 0.1, 1234
        def run_drop():
            fa.fa_fwd_dropout(Q, K, V, O, LSE, scale, p_drop, seed, causal=causal, blockmask=M)
            fa.fa_bwd_dropout(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, p_drop, seed,
                              causal=causal, blockmask=M, workspace=ws)
        run_drop()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(args.dropout_steps)]
        for e in ev:
            e[0].record()
            fa.fa_fwd_dropout(Q, K, V, O, LSE, scale, p_drop, seed, causal=causal, blockmask=M)
            e[1].record()
            fa.fa_bwd_dropout(dO, Q, K, V, O, LSE, dQ, dK, dV, scale, p_drop, seed,
                              causal=causal, blockmask=M, workspace=ws)
            e[2].record()
        torch.cuda.synchronize()
        f_s = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
        b_s = statistics.median([e[1].elapsed_time(e[2]) * 1e-3 for e in ev])
        dropout = {"workload": cfg.name + " with dropout p=0.1 on P (supplementary)",
                   "p_drop": p_drop, "fwd_ms": round(f_s * 1e3, 4),
                   "fwd_tflops": round(fwd_flops / f_s / 1e12, 2),
                   "bwd_ms": round(b_s * 1e3, 4), "bwd_tflops": round(bwd_flops / b_s / 1e12, 2),
                   "steps": args.dropout_steps}

    # Supplementary: the FP8 forward on the same shape (Q, K, V quantized to
    # E4M3 with per-tensor descales); never part of `value`.
    fp8 = None
    if args.fp8_steps > 0 and cfg.d in (64, 128) and mask is None and want("fp8"):
        def q8(t):
            amax = float(t.float().abs().max())
            ds = amax / 448.0
            return (t.float() / ds).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), ds
        (Q8, qd), (K8, kd), (V8, vd) = q8(Q), q8(K), q8(V)
        O8 = torch.empty_like(O)
        ws8 = torch.empty(fa.fa_fwd_fp8_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d),
                          dtype=torch.uint8, device=dev)
        fa.fa_fwd_fp8(Q8, K8, V8, O8, LSE, scale, qd, kd, vd, causal=causal, workspace=ws8)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.fp8_steps)]
        for e in ev:
            e[0].record()
            fa.fa_fwd_fp8(Q8, K8, V8, O8, LSE, scale, qd, kd, vd, causal=causal, workspace=ws8)
            e[1].record()
        torch.cuda.synchronize()
        f_s = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
        fp8 = {"workload": cfg.name + " forward with E4M3 Q, K, V and P (supplementary)",
               "fwd_ms": round(f_s * 1e3, 4), "fwd_tflops": round(fwd_flops / f_s / 1e12, 2),
               "frac_of_fp8_peak": round(fwd_flops / f_s / 1e12 / PEAK_FP8_TFLOPS, 4),
               "steps": args.fp8_steps}
        del Q8, K8, V8, O8, ws8

    # Supplementary: the forward at head dim 256 on the same B, H, N and mask
    # (fresh seeded N(0,1) inputs, Q and K scaled like the workload's);
    # never part of `value`.
    wide = None
    if args.wide_steps > 0 and mask is None and want("wide"):
        g = torch.Generator(device=dev)
        g.manual_seed(256)
        shp = (cfg.B, cfg.H, cfg.N, 256)
        Qw, Kw, Vw = (torch.randn(shp, generator=g, device=dev).mul_(m).to(torch.bfloat16)
                      for m in (cfg.qk_mult, cfg.qk_mult, 1.0))
        Ow = torch.empty_like(Qw)
        sw = float(np.float32(1.0 / np.sqrt(256.0)))
        fa.fa_fwd(Qw, Kw, Vw, Ow, LSE, sw, causal=causal)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.wide_steps)]
        for e in ev:
            e[0].record()
            fa.fa_fwd(Qw, Kw, Vw, Ow, LSE, sw, causal=causal)
            e[1].record()
        torch.cuda.synchronize()
        f_s = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
        wflops = fwd_flops * 256 / cfg.d
        wide = {"workload": cfg.name + " forward at head dim 256 (supplementary)", "d": 256,
                "fwd_ms": round(f_s * 1e3, 4), "fwd_tflops": round(wflops / f_s / 1e12, 2),
                "frac_of_peak": round(wflops / f_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                "mfma_work_factor": 1.0, "steps": args.wide_steps}
        if args.wide_bwd:
            # the backward at d = 256 (dQ, dV and dK passes, S rebuilt in
            # each): one warm-up call, then the median of --wide-bwd timed calls
            dOw = torch.randn(shp, generator=g, device=dev).to(torch.bfloat16)
            dQw, dKw, dVw = (torch.empty_like(Qw) for _ in range(3))
            wsw = fa.new_workspace(cfg.B, cfg.H, cfg.N, 256, dev)
            fa.fa_bwd(dOw, Qw, Kw, Vw, Ow, LSE, dQw, dKw, dVw, sw, causal=causal, workspace=wsw)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.wide_bwd)]
            for e in ev:
                e[0].record()
                fa.fa_bwd(dOw, Qw, Kw, Vw, Ow, LSE, dQw, dKw, dVw, sw, causal=causal, workspace=wsw)
                e[1].record()
            torch.cuda.synchronize()
            b_s = statistics.median([e[0].elapsed_time(e[1]) * 1e-3 for e in ev])
            wide.update(bwd_ms=round(b_s * 1e3, 2), bwd_tflops=round(2.5 * wflops / b_s / 1e12, 3),
                        bwd_mfma_work_factor=1.6, bwd_steps=args.wide_bwd)
            del dOw, dQw, dKw, dVw, wsw
        del Qw, Kw, Vw, Ow

    decode = decode256 = None
    if args.decode_steps > 0 and want("decode"):
        decode = decode_run(args.decode_steps)
        decode256 = decode_run(args.decode_steps, d=256)

    # Supplementary: the pages' other workloads (GPT-2-shaped attention, the
    # 64K dense forward, block-sparse), each with its own algorithmic FLOPs
    # and fraction of peak; never part of `value`.
    other = None
    if args.other_steps > 0 and want("other"):
        other = []
        for c in (2, 4, 5):
            oc = syn.CONFIGS[c]
            om = syn.block_mask((oc.N + 127) // 128) if oc.sparse else None
            other.append(workload_run(oc, args.other_steps, mask=om))
    sweep = None
    if args.sweep_steps > 0 and want("sweep"):
        sweep = sparse_sweep(syn.CONFIGS[5], args.sweep_steps)

    # Supplementary: head dims between the kernel widths (64 and 128) run in
    # the next wider kernel with zero-padded columns, so their algorithmic
    # rate falls with d / width; measured on the headline B, H, N and mask.
    padded = None
    if args.padded_steps > 0 and mask is None and want("padded"):
        from types import SimpleNamespace
        padded = []
        for dd in (64, 72, 96, 128):
            pc = SimpleNamespace(name=f"{cfg.name} shape at d={dd}", cfg_id=cfg.cfg_id, B=cfg.B,
                                 H=cfg.H, N=cfg.N, d=dd, qk_mult=cfg.qk_mult, causal=causal,
                                 scale=dd ** -0.5, has_bwd=True)
            r = workload_run(pc, args.padded_steps)
            r["kernel_width"] = 64 if dd <= 64 else 128
            padded.append(r)

    clock = None
    if args.clock_seconds > 0 and want("clock"):
        clock = clock_under_load(step, args.clock_seconds)
        if clock and "step_ms_in_window" in clock and "bf16_peak_at_clock_tflops" in clock:
            # the step's algorithmic rate in that window against the peak at
            # the sampled clock
            rate = (fwd_flops + bwd_flops) / (clock["step_ms_in_window"] * 1e-3) / 1e12
            clock["step_frac_of_peak_at_clock"] = round(rate / clock["bf16_peak_at_clock_tflops"], 4)

    cpu = None
    if args.cpu_heads > 0:
        import oracle
        nh = min(args.cpu_heads, cfg.B * cfg.H)
        # the first nh (batch, head) pairs, as one batch of nh heads

        def heads(x):
            return x.reshape((1, cfg.B * cfg.H) + x.shape[2:])[:, :nh]
        t1 = time.perf_counter()
        oracle.attention(heads(q), heads(k), heads(v), scale, causal=causal, blockmask=mask, do=heads(do))
        cpu_s = time.perf_counter() - t1
        head_flops = (fwd_flops + bwd_flops) / (cfg.B * cfg.H)
        cpu = {"value": round(nh * head_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{nh} of {cfg.B * cfg.H} heads of the same workload, fwd+bwd, "
                         f"fp64, {cpu_s:.1f} s"}
        if args.cpu_other:
            cpu["other_workloads"] = cpu_other(args)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + " attention fwd+bwd", "B": cfg.B, "H": cfg.H,
                   "N": cfg.N, "d": cfg.d, "causal": cfg.causal,
                   "block_sparse": mask is not None, "qk_mult": cfg.qk_mult,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(fwd_s * 1e3, 4), "tflops": round(fwd_flops / fwd_s / 1e12, 2),
                "frac_of_peak": round(fwd_flops / fwd_s / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_s * 1e3, 4), "tflops": round(bwd_flops / bwd_s / 1e12, 2),
                "frac_of_peak": round(bwd_flops / bwd_s / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "supplementary": supp,
        "dropout": dropout,
        "fp8": fp8,
        "wide_head": wide,
        "decode": decode,
        "decode_d256": decode256,
        "other_workloads": other,
        "sparse_density_sweep": sweep,
        "padded_head_dims": padded,
        "clock_under_load": clock,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
