"""Throughput benchmark of the fused causal long convolution on one MI355X.

Default workload (the headline line): conv_1k, an H3-125M-shaped long
convolution, B=8 x H=768 channels x N=1024, fp16 activations, diagonal-SSM
filter with 64 modes.  One step = one h3conv_fft_conv call over the whole
batch (load u, filter spectrum, forward FFT, pointwise product, inverse FFT,
residual, store y).  The filter f is produced beforehand by h3conv_ssm_filter
and is resident in HBM like the input.

To keep the 256 MB Infinity Cache from serving the inputs, every step uses
the next of several independent input/output sets whose total exceeds 512 MB.

Output: one JSON line with elements/s (B*H*N per second), the roofline of the
dominant kernel against MI355X HBM3E (8 TB/s) measured with HIP events on the
launch stream, and the fp64 CPU oracle timed on this host's cores.  The HBM
traffic and the matrix-core flops of the dominant kernel come from the
committed rocprofv3 counter summary of the workload (profiles/), and are
reported only while the kernel sources still hash to the value recorded
there; the matrix-core utilisation is those flops over the live kernel time
and the dense fp16 peak (2.5 PFLOP/s).  The other workloads, and a sweep of
the sequence length (N = 256 ... 32K, fused up to 8K, state passing above)
timed beside an unfused torch.fft FFT convolution on the same GPU (the
analogue of the pages' cuFFT baseline), are reported under "secondary" and
"sweep".

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-sweep]
    python bench.py --calib-copy    # plain 1 GiB device copy, for counter calibration
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import fft_long_convolution_flashconv_amd as pkg  # noqa: E402
from fft_long_convolution_flashconv_amd import workloads as wl  # noqa: E402

METRIC = "long-conv elements/s (B·H·N) + achieved HBM GB/s vs peak, N=1K–64K, 1 GPU"
HBM_PEAK_GBS = 8000.0
CACHE_BYTES = 512 << 20
ESZ = {"f32": 4, "f16": 2, "bf16": 2}
# dtype the transforms compute in: for 16-bit activations the DFT blocks run
# on the matrix cores with fp16 operands and fp32 accumulation, and twiddles,
# scaling and the spectrum product are packed fp16; fp32 activations use the
# fp32 vector engine
COMPUTE_DTYPE = {"f16": "f16", "bf16": "f16", "f32": "f32"}
MFMA_PEAK_FLOPS = 2.5e15   # dense fp16 matrix-core peak of MI355X
# the kernel sources whose hash a counter summary records
KERNEL_SRC_DIR = "fft_long_convolution_flashconv_amd/csrc"
# counter summary of the dominant kernel of each workload
PROFILES = {"conv_1k": "profiles/k_fft_conv_mfma_conv_1k.md",
            "conv_8k": "profiles/k_fft_conv_mfma_conv_8k.md",
            "state_64k": "profiles/k_sp_block_state_64k.md",
            "h3_mix_2k": "profiles/k_fft_conv_mfma_h3_mix_2k.md",
            "conv_1k_bwd": "profiles/k_fft_bwd_mfma_conv_1k_bwd.md",
            "decode_125m": "profiles/k_ssm_step_decode_125m.md",
            "h3_mix_mh_1k": "profiles/k_fft_conv_mfma_h3_mix_mh_1k.md",
            "bidir_1k": "profiles/k_fft_bidir_mfma_bidir_1k.md"}


def kernel_source_hash() -> str:
    """sha256 (16 hex digits) over every source of the library's kernels."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_SRC_DIR)
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def profiled(workload: str) -> dict:
    """Per-launch HBM traffic (bytes) and matrix-core flops of the dominant
    kernel from the counter summary, if it covers this workload and the
    current kernel sources (else None values)."""
    out = {"traffic": None, "mfma_flops": None, "kernel": None}
    rel = PROFILES.get(workload)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return out
    text = open(os.path.join(ROOT, rel)).read()
    m_hash = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    m_wl = re.search(r"workload: `([a-z0-9_]+)`", text)
    if not (m_hash and m_wl) or m_wl.group(1) != workload or m_hash.group(1) != kernel_source_hash():
        return out
    m_tr = re.search(r"traffic per launch of `([^`]*)`: ([0-9]+) bytes", text)
    m_fl = re.search(r"matrix-core flops per launch of `[^`]*`: ([0-9]+)", text)
    if m_tr:
        out["kernel"], out["traffic"] = m_tr.group(1), int(m_tr.group(2))
    if m_fl:
        out["mfma_flops"] = int(m_fl.group(1))
    return out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w: wl.Workload) -> int:
    """HBM bytes one call must move at least: every input read once, every output written once."""
    e = ESZ[w.dtype]
    if w.kind == "fft_conv":
        return 2 * w.B * w.H * w.N * e + w.H * w.N * 4 + w.H * 4
    if w.kind == "state_pass":
        return 2 * w.B * w.H * w.N * e + w.H * (3 * w.S * 8 + 8)
    if w.kind == "h3_mix":
        return 4 * w.B * w.N * w.Dm * e + w.Dm * (w.L * 4 + w.N * 4 + 4)
    if w.kind == "h3_mix_mh":     # read q, k, v, w, f, D; write out
        return 4 * w.B * w.N * w.Dm * e + w.Dm * w.L * 4 + w.Dm * w.dh * (w.N * 4 + 4)
    if w.kind == "fft_conv_bwd":  # read u, dy, f, D; write du, df, dD
        return 3 * w.B * w.H * w.N * e + 2 * w.H * w.N * 4 + 2 * w.H * 4
    if w.kind == "fft_conv_bidir":  # read u, f, g, D; write y
        return 2 * w.B * w.H * w.N * e + 2 * w.H * w.N * 4 + w.H * 4
    if w.kind == "ssm_step":      # read u, x, parameters; write y, x
        return w.B * w.H * (2 * w.N * e + 2 * w.S * 8) + w.H * (3 * w.S * 8 + 8)
    raise ValueError(w.kind)


class Case:
    """Device-resident inputs for one workload, in several rotating copies."""

    def __init__(self, w: wl.Workload, dev, rotate: bool = True):
        self.w = w
        inp = wl.make_inputs(w)
        d = {k: v.to(dev) for k, v in inp.items()}
        nbytes = algorithmic_bytes(w)
        self.nsets = max(1, -(-CACHE_BYTES // nbytes)) if rotate else 1
        self.sets = []
        for i in range(self.nsets):
            s = {k: (v if i == 0 else v.clone()) for k, v in d.items()}
            if w.kind in ("fft_conv", "h3_mix", "fft_conv_bwd", "h3_mix_mh", "fft_conv_bidir") and "A" in s:
                s["f"] = pkg.ssm_filter(s["A"], s["Bm"], s["C"], s["dt"], w.N)
            if w.kind == "fft_conv_bidir":
                s["g"] = pkg.ssm_filter(s["gA"], s["gBm"], s["gC"], s["gdt"], w.N)
                s["y"] = torch.empty_like(s["u"])
            elif w.kind == "fft_conv":
                s["y"] = torch.empty_like(s["u"])
            elif w.kind == "fft_conv_bwd":
                s["du"] = torch.empty_like(s["u"])
                s["df"] = torch.empty(w.H, w.N, device=dev, dtype=torch.float32)
                s["dD"] = torch.empty(w.H, device=dev, dtype=torch.float32)
            elif w.kind == "ssm_step":
                s["y"] = torch.empty_like(s["u"])
            elif w.kind == "h3_mix_mh":
                s["y"] = torch.empty_like(s["q"])
                s["ws"] = torch.empty(pkg.workspace_size(pkg.OP_H3_MIX_MH, w.B, w.Dm, w.N, w.dh), device=dev,
                                      dtype=torch.uint8)
            elif w.kind == "state_pass":
                s["y"] = torch.empty_like(s["u"])
                s["ws"] = torch.empty(pkg.workspace_size(pkg.OP_STATE_PASS, w.B, w.H, w.N, w.S, w.T),
                                      device=dev, dtype=torch.uint8)
            else:
                s["y"] = torch.empty_like(s["q"])
                s["ws"] = torch.empty(pkg.workspace_size(pkg.OP_H3_MIX, w.B, w.Dm, w.N), device=dev,
                                      dtype=torch.uint8)
            self.sets.append(s)
        torch.cuda.synchronize()

    def step(self, i: int):
        s = self.sets[i % self.nsets]
        w = self.w
        if w.kind == "fft_conv":
            pkg.fft_conv(s["u"], s["f"], s["D"], out=s["y"])
        elif w.kind == "fft_conv_bidir":
            pkg.fft_conv_bidir(s["u"], s["f"], s["g"], s["D"], out=s["y"])
        elif w.kind == "fft_conv_bwd":
            pkg.fft_conv_bwd(s["u"], s["f"], s["D"], s["dy"], du=s["du"], df=s["df"], dD=s["dD"])
        elif w.kind == "ssm_step":
            pkg.ssm_step(s["u"], s["A"], s["Bm"], s["C"], s["dt"], s["D"], s["x"], out=s["y"])
        elif w.kind == "h3_mix_mh":
            pkg.h3_mix_mh(s["q"], s["k"], s["v"], s["w"], s["f"], s["D"], w.dh, out=s["y"], workspace=s["ws"])
        elif w.kind == "state_pass":
            pkg.state_pass(s["u"], s["A"], s["Bm"], s["C"], s["dt"], s["D"], w.T, out=s["y"],
                           workspace=s["ws"])
        else:
            pkg.h3_mix(s["q"], s["k"], s["v"], s["w"], s["f"], s["D"], out=s["y"], workspace=s["ws"])


def time_case(case: Case, steps: int, warmup: int):
    """Warm up, then time exactly `steps` steps.  HIP events on the launch
    stream bracket the whole timed region (launches queue back to back, so
    their elapsed time over `steps` is the average launch duration); the wall
    clock is bracketed by device synchronisations."""
    # no garbage-collection pause of the launching thread inside the timed
    # steps (it would show as the GPU idling between launches); collected
    # before the warm-up, so that no idle gap lets the clocks drop between the
    # warm-up and the timed steps
    gc.collect()
    gc.disable()
    try:
        for i in range(warmup):
            case.step(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            case.step(warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    return wall, e0.elapsed_time(e1) / steps


def time_case_batches(case: Case, steps: int, warmup: int, nb: int = 5):
    """`steps` steps in nb batches, each bracketed by HIP events on the launch
    stream: the mean launch duration of every batch (a one-off stall of the
    box shows in one batch, not in the median)."""
    gc.collect()
    gc.disable()
    try:
        for i in range(warmup):
            case.step(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        per = max(1, steps // nb)
        out, k = [], warmup
        for _ in range(nb):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per):
                case.step(k)
                k += 1
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / per)
    finally:
        gc.enable()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: wl.Workload, budget_s: float = 12.0) -> dict:
    """fp64 oracle on this host's cores over a bounded sample of the workload,
    then on one thread over a smaller sample (both scaled to elements/s)."""
    import numpy as np

    import oracle

    if w.kind != "fft_conv":
        raise ValueError(w.kind)
    inp = wl.make_inputs(w)
    if "A" in inp:
        cp = lambda t: t.double().numpy()[..., 0] + 1j * t.double().numpy()[..., 1]
        f = oracle.ssm_filter(cp(inp["A"]), cp(inp["Bm"]), cp(inp["C"]), inp["dt"].double().numpy(), w.N)
    else:
        f = inp["f"].double().numpy()
    u = inp["u"].double().numpy()
    D = inp["D"].double().numpy()
    H = w.H

    def timed(ua, fa, Da, budget):
        t0 = time.perf_counter()
        oracle.causal_conv(ua, fa, Da)
        t_one = time.perf_counter() - t0
        reps, total = 1, t_one
        while total < budget:
            t0 = time.perf_counter()
            oracle.causal_conv(ua, fa, Da)
            total += time.perf_counter() - t0
            reps += 1
        return reps, total, t_one

    # all cores: whole batch rows of a growing number of channels, then the
    # sample repeated, until about `budget_s` seconds of CPU work
    hs = 16
    while True:
        sel = np.arange(min(hs, H))
        ua, fa, Da = np.ascontiguousarray(u[:, sel]), np.ascontiguousarray(f[sel]), D[sel]
        t0 = time.perf_counter()
        oracle.causal_conv(ua, fa, Da)
        if time.perf_counter() - t0 > budget_s / 4 or hs >= H:
            break
        hs = min(H, hs * 4)
    reps, total, _ = timed(ua, fa, Da, budget_s)
    cores = oracle.max_threads()
    out = {"value": w.B * len(sel) * w.N * reps / total, "unit": "elements/s", "cores": cores,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": "direct O(N^2) causal conv (fp64) of all %d batch rows x %d of %d channels, N=%d, "
                     "%d repetition(s), %.1f s" % (w.B, len(sel), H, w.N, reps, total)}
    # one thread: one batch row of 8 channels
    oracle.set_threads(1)
    try:
        u1, f1, D1 = np.ascontiguousarray(u[:1, :8]), np.ascontiguousarray(f[:8]), D[:8]
        reps1, total1, _ = timed(u1, f1, D1, budget_s / 4)
    finally:
        oracle.set_threads(cores)
    out["one_thread"] = {"value": 8 * w.N * reps1 / total1, "unit": "elements/s", "cores": 1,
                         "sample": "1 batch row x 8 channels, N=%d, %d repetition(s), %.1f s"
                                   % (w.N, reps1, total1)}
    return out


def torch_fftconv(u, f, D):
    """Unfused FFT convolution with torch.fft (rocFFT): rfft of the
    zero-padded input and filter, product, irfft, first N outputs, plus D*u;
    in fp32.  Timing comparison only (the analogue of the pages' cuFFT
    FFTConv baseline)."""
    N = u.shape[-1]
    uf = u.float()
    y = torch.fft.irfft(torch.fft.rfft(uf, n=2 * N) * torch.fft.rfft(f, n=2 * N), n=2 * N)[..., :N]
    return (y + uf * D[:, None]).to(u.dtype)


def torch_fftconv_bwd(u, f, D, dy):
    """Unfused backward of torch_fftconv with torch.fft: du = IDFT(DY conj(F))
    [:N] + D dy, df = IDFT(sum_b conj(U_b) DY_b)[:N], dD = df[..., 0]; in
    fp32.  Timing comparison only."""
    N = u.shape[-1]
    U = torch.fft.rfft(u.float(), n=2 * N)
    DY = torch.fft.rfft(dy.float(), n=2 * N)
    F = torch.fft.rfft(f, n=2 * N)
    du = torch.fft.irfft(DY * F.conj(), n=2 * N)[..., :N] + dy.float() * D[:, None]
    df = torch.fft.irfft((U.conj() * DY).sum(0), n=2 * N)[..., :N]
    return du.to(u.dtype), df, df[..., 0]


def sweep(dev, steps: int, warmup: int) -> list:
    """Sequence-length sweep at the H3-125M width (B=8, H=768, fp16, 64
    modes): fused fft_conv for N <= 16384 (the filter given), state passing
    (T = min(N, 8192); the call builds its channel tables from the SSM
    parameters) for N = 1024 ... 32768, and the backward pass (fft_conv_bwd)
    for N <= 8192, each timed beside its unfused torch.fft counterpart on the
    same inputs."""
    out = []
    pts = [(N, "fft_conv") for N in (256, 512, 1024, 2048, 4096, 8192, 16384)] + \
          [(N, "state_pass") for N in (1024, 4096, 8192, 16384, 32768)] + \
          [(N, "fft_conv_bwd") for N in (256, 512, 1024, 2048, 4096, 8192)]
    for i, (N, kind) in enumerate(pts):
        w = wl.Workload("sweep_%d" % N, kind, "f16", B=8, H=768, N=N, T=min(N, 8192) if kind == "state_pass" else 0,
                        seed=100 + i)
        c = Case(w, dev)
        _, m_ms = time_case(c, steps, warmup)
        s0 = c.sets[0]
        if "f" not in s0:
            s0["f"] = pkg.ssm_filter(s0["A"], s0["Bm"], s0["C"], s0["dt"], N)
        if kind == "fft_conv_bwd":
            ref = lambda: torch_fftconv_bwd(s0["u"], s0["f"], s0["D"], s0["dy"])
        else:
            ref = lambda: torch_fftconv(s0["u"], s0["f"], s0["D"])
        gc.collect()
        gc.disable()
        try:
            for _ in range(warmup):
                ref()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                ref()
            e1.record()
            torch.cuda.synchronize()
        finally:
            gc.enable()
        t_ms = e0.elapsed_time(e1) / steps
        nb = algorithmic_bytes(w)
        out.append({"N": N, "path": kind, "us": m_ms * 1e3, "elements_per_s": w.elements / (m_ms * 1e-3),
                    "frac_hbm": nb / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "torch_fft_us": t_ms * 1e3,
                    "speedup_vs_torch_fft": t_ms / m_ms})
        log("bench: sweep N=%d %s %.1f us (%.1f%% of HBM) torch.fft %.1f us x%.2f"
            % (N, kind, m_ms * 1e3, 100 * out[-1]["frac_hbm"], t_ms * 1e3, t_ms / m_ms))
        del c, s0
        torch.cuda.empty_cache()
    return out


def calib_copy():
    """One plain device-to-device copy of 1 GiB (counter calibration: FETCH/WRITE of a known size)."""
    dev = torch.device("cuda:0")
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="conv_1k", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sequence-length sweep")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash and exit")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(channels shard with no communication; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if a.source_hash:
        print(kernel_source_hash())
        return
    if a.calib_copy:
        calib_copy()
        return
    dev = torch.device("cuda:0")
    pkg.load()

    w = wl.WORKLOADS[a.workload]
    log("bench: workload %s %s" % (w.name, w))
    case = Case(w, dev)
    wall, mean_ms = time_case(case, a.steps, a.warmup)
    ms_per_step = wall * 1e3 / a.steps
    nbytes = algorithmic_bytes(w)
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    prof = profiled(w.name)
    mfma_util = (prof["mfma_flops"] / (mean_ms * 1e-3) / MFMA_PEAK_FLOPS) if prof["mfma_flops"] else None
    out = {
        "metric": METRIC,
        "value": w.elements / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": COMPUTE_DTYPE[w.dtype],
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": w.name, "B": w.B, "H": w.H or w.Dm, "N": w.N, "io_dtype": w.dtype,
                   "kind": w.kind, "input_sets_rotated": case.nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": prof["traffic"],
                     "kernel_mean_us": mean_ms * 1e3, "algorithmic_bytes_per_launch": nbytes,
                     "mfma_util": mfma_util, "mfma_flops_per_launch": prof["mfma_flops"],
                     "mfma_peak_flops": MFMA_PEAK_FLOPS},
    }
    del case
    torch.cuda.empty_cache()
    # side note: the same call with one input set, which stays resident in
    # the 256 MB Infinity Cache and L2 between calls (the line's value and
    # roofline are the rotated, cache-flushed figures above)
    warm = Case(w, dev, rotate=False)
    _, warm_ms = time_case(warm, a.steps, a.warmup)
    out["warm"] = {"kernel_mean_us": warm_ms * 1e3, "GB_s": nbytes / (warm_ms * 1e-3) / 1e9,
                   "note": "one input set, resident in the Infinity Cache / L2 between calls"}
    del warm
    torch.cuda.empty_cache()
    if not a.no_secondary:
        sec = {}
        for name in ("conv_8k", "state_64k", "h3_mix_2k", "conv_1k_bwd", "decode_125m", "h3_mix_mh_1k", "bidir_1k"):
            if name == w.name:
                continue
            ww = wl.WORKLOADS[name]
            c = Case(ww, dev)
            batches = time_case_batches(c, max(10, a.steps), max(3, a.warmup))
            m_ms = sorted(batches)[len(batches) // 2]
            nb = algorithmic_bytes(ww)
            pr = profiled(name)
            sec[name] = {"elements_per_s": ww.elements / (m_ms * 1e-3), "mean_us": m_ms * 1e3,
                         "batches_us": [x * 1e3 for x in batches],
                         "algorithmic_bytes": nb, "GB_s": nb / (m_ms * 1e-3) / 1e9,
                         "frac_hbm": nb / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "sets": c.nsets,
                         "traffic_per_step_kernel": pr["traffic"], "profiled_kernel": pr["kernel"],
                         "mfma_util": (pr["mfma_flops"] / (m_ms * 1e-3) / MFMA_PEAK_FLOPS) if pr["mfma_flops"] else None}
            log("bench: %s mean %.1f us  %.1f GB/s" % (name, m_ms * 1e3, sec[name]["GB_s"]))
            del c
            torch.cuda.empty_cache()
        out["secondary"] = sec
    if not a.no_sweep:
        out["sweep"] = sweep(dev, max(10, a.steps // 2), max(3, a.warmup // 2))
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
