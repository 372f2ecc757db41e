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
traffic of the dominant kernel comes from the committed rocprofv3 counter
summary (profiles/), and is reported only while the kernel sources still hash
to the value recorded there.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --calib-copy    # plain 1 GiB device copy, for counter calibration
"""
from __future__ import annotations

import argparse
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
# sources that define the dominant kernel, and the counter summary of it
KERNEL_SOURCES = ("fft_long_convolution_flashconv_amd/csrc/mfma_engine.h",
                  "fft_long_convolution_flashconv_amd/csrc/fftconv.hip",
                  "fft_long_convolution_flashconv_amd/csrc/h3conv_device.h")
PROFILE = "profiles/k_fft_conv_mfma_conv_1k.md"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str):
    """HBM bytes per launch from the counter summary, if it covers this
    workload and the current kernel sources (else None)."""
    path = os.path.join(ROOT, PROFILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    m_wl = re.search(r"workload: `([a-z0-9_]+)`", text)
    m_tr = re.search(r"traffic per launch(?: of `[^`]*`)?: ([0-9]+) bytes", text)
    if not (m_hash and m_wl and m_tr) or m_wl.group(1) != workload or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_tr.group(1))


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
            if w.kind in ("fft_conv", "h3_mix") and "A" in s:
                s["f"] = pkg.ssm_filter(s["A"], s["Bm"], s["C"], s["dt"], w.N)
            if w.kind == "fft_conv":
                s["y"] = torch.empty_like(s["u"])
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
    return wall, e0.elapsed_time(e1) / steps


def cpu_baseline(w: wl.Workload, budget_s: float = 12.0) -> dict:
    """fp64 oracle on this host's cores over a bounded sample of the workload."""
    import numpy as np

    import oracle

    inp = wl.make_inputs(w)
    g = np.random.default_rng(0)
    if w.kind == "fft_conv":
        f = oracle.ssm_filter(inp["A"].double().numpy()[..., 0] + 1j * inp["A"].double().numpy()[..., 1],
                              inp["Bm"].double().numpy()[..., 0] + 1j * inp["Bm"].double().numpy()[..., 1],
                              inp["C"].double().numpy()[..., 0] + 1j * inp["C"].double().numpy()[..., 1],
                              inp["dt"].double().numpy(), w.N) if "A" in inp else inp["f"].double().numpy()
        u = inp["u"].double().numpy()
        D = inp["D"].double().numpy()
        # sample: whole batch rows of a growing number of channels, then the
        # sample repeated, until about `budget_s` seconds of CPU work
        H = w.H
        hs = 16
        while True:
            sel = np.arange(min(hs, H))
            ua, fa, Da = np.ascontiguousarray(u[:, sel]), np.ascontiguousarray(f[sel]), D[sel]
            t0 = time.perf_counter()
            oracle.causal_conv(ua, fa, Da)
            t_one = time.perf_counter() - t0
            if t_one > budget_s / 4 or hs >= H:
                break
            hs = min(H, hs * 4)
        reps, total = 1, t_one
        while total < budget_s:
            t0 = time.perf_counter()
            oracle.causal_conv(ua, fa, Da)
            total += time.perf_counter() - t0
            reps += 1
        n_el = w.B * len(sel) * w.N * reps
        return {"value": n_el / total, "unit": "elements/s", "cores": oracle.max_threads(), "kind": "oracle",
                "sample": "direct O(N^2) causal conv (fp64) of all %d batch rows x %d of %d channels, N=%d, "
                          "%d repetition(s), %.1f s" % (w.B, len(sel), H, w.N, reps, total)}
    raise ValueError(w.kind)


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
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash and exit")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(channels shard with no communication; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if a.calib_copy:
        calib_copy()
        return
    if a.source_hash:
        print(kernel_source_hash())
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(w.name),
                     "kernel_mean_us": mean_ms * 1e3, "algorithmic_bytes_per_launch": nbytes},
    }
    del case
    torch.cuda.empty_cache()
    if not a.no_secondary:
        sec = {}
        for name in ("conv_8k", "state_64k", "h3_mix_2k"):
            if name == w.name:
                continue
            ww = wl.WORKLOADS[name]
            c = Case(ww, dev)
            _, m_ms = time_case(c, max(5, a.steps // 5), 3)
            nb = algorithmic_bytes(ww)
            sec[name] = {"elements_per_s": ww.elements / (m_ms * 1e-3), "mean_us": m_ms * 1e3,
                         "algorithmic_bytes": nb, "GB_s": nb / (m_ms * 1e-3) / 1e9,
                         "frac_hbm": nb / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "sets": c.nsets}
            log("bench: %s mean %.1f us  %.1f GB/s" % (name, m_ms * 1e3, sec[name]["GB_s"]))
            del c
            torch.cuda.empty_cache()
        out["secondary"] = sec
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
