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
launch stream, and the fp64 CPU oracle timed on this host's cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --calib-copy    # plain 1 GiB device copy, for counter calibration
"""
from __future__ import annotations

import argparse
import json
import os
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
# dtype the convolution arithmetic runs in (activations are stored in the
# workload's I/O dtype; every transform is computed in fp32)
COMPUTE_DTYPE = "f32"


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
    for i in range(warmup):
        case.step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        case.step(warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(per_launch_ms) / len(per_launch_ms)
    return wall, mean_ms, per_launch_ms[len(per_launch_ms) // 2]


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
        # sample: whole batch rows for a growing number of channels until the budget is used
        H = w.H
        t_one = None
        hs = 16
        while True:
            sel = np.arange(min(hs, H))
            t0 = time.perf_counter()
            oracle.causal_conv(np.ascontiguousarray(u[:, sel]), np.ascontiguousarray(f[sel]), D[sel])
            t_one = time.perf_counter() - t0
            if t_one > budget_s / 4 or hs >= H:
                break
            hs = min(H, hs * 4)
        n_el = w.B * len(sel) * w.N
        return {"value": n_el / t_one, "unit": "elements/s", "cores": oracle.max_threads(), "kind": "oracle",
                "sample": "direct O(N^2) causal conv (fp64) of all %d batch rows x %d of %d channels, N=%d "
                          "(%.2f s)" % (w.B, len(sel), H, w.N, t_one)}
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
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(channels shard with no communication; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if a.calib_copy:
        calib_copy()
        return
    dev = torch.device("cuda:0")
    pkg.load()

    w = wl.WORKLOADS[a.workload]
    log("bench: workload %s %s" % (w.name, w))
    case = Case(w, dev)
    wall, mean_ms, med_ms = time_case(case, a.steps, a.warmup)
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
        "dtype": COMPUTE_DTYPE,
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": w.name, "B": w.B, "H": w.H or w.Dm, "N": w.N, "io_dtype": w.dtype,
                   "kind": w.kind, "input_sets_rotated": case.nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel_mean_us": mean_ms * 1e3, "kernel_median_us": med_ms * 1e3,
                     "algorithmic_bytes_per_launch": nbytes},
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
            _, m_ms, md_ms = time_case(c, max(5, a.steps // 5), 3)
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
