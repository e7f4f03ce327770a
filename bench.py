#!/usr/bin/env python3
"""Benchmark of NVFP4 quantized matmul on one MI355X.

Headline (``value``): the decode workload -- qmm with M=1, K=5376, N=21504,
bf16 activations and output, scalar global scale -- as achieved HBM GB/s
of algorithmic bytes.  One step is one nvfp4_qmm call (weight stream, scale
stream, decode, MAC, reduction, epilogue).  The K timed steps are launched
back to back on one stream (the host enqueues ahead of the GPU) and rotate
over 8 independent copies of the weight planes (520 MB > the 256 MB MALL)
so weights come from HBM; the same steps replayed as one HIP graph are
reported beside it.

Also reported, each against its roofline: the prefill GEMM (M=2048,
TFLOP/s), the fused gate/up MLP projection at the same shape, the
multi-row qmv (M=16) and the MoE gather (sorted prefill and unsorted
decode, GB/s); under ``other_configs`` the tiny qmv's latency, multi-row
qmv at every M in f32 and bf16, MoE unsorted decode at B = 1..8,
batched-weight qmm and the load-time transcode / dequantize / quantize.
Kernel durations come from HIP events around back-to-back launches on the
launch stream.  ``stream_ceiling`` is the best plain streaming read of the
decode workload's byte count on the same device, for context.  The CPU oracle is timed on the host
on the full decode workload (cpu_baseline) and on the full prefill workload
(prefill.cpu_baseline).  The prefill is also timed with f16 and float32
activations.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import nvfp4_quantized_matmul_amd as nv  # noqa: E402
import nvfp4_synth as synth  # noqa: E402

METRIC = "NVFP4 qmv HBM GB/s (M=1) and dequant+GEMM TFLOP/s (M=2048), % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
DEV = "cuda:0"
BF16 = 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def words_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def P(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def stream_ptr():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def eager_launch_us(work, n: int, warmup: int = 3):
    """Average duration of one launch over `n` back-to-back launches."""
    ms = timed_eager(work, n, warmup)
    return {"mean_us": ms * 1e3, "launches": n, "source": "HIP events around back-to-back launches"}


def check(status, what):
    if status != 0:
        raise RuntimeError(f"{what}: {nv.status_string(status)}")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

class Decode:
    """qmm M=1, K=5376, N=21504, bf16, scalar gs; `copies` weight planes."""
    M, K, N = 1, 5376, 21504

    def __init__(self, copies: int):
        wl = synth.WORKLOADS["decode_qmv_m1_k5376_n21504_bf16"]
        case = synth.dense_case(wl["seed"], self.M, self.K, self.N, with_gs=True)
        w0, s0 = words_dev(case.w), u8_dev(case.scales)
        self.w = [w0] + [w0.clone() for _ in range(copies - 1)]
        self.s = [s0] + [s0.clone() for _ in range(copies - 1)]
        self.gs = torch.from_numpy(case.gs).to(DEV)
        self.x = torch.from_numpy(case.x).to(torch.bfloat16).to(DEV)
        self.out = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=DEV)
        self.lib = nv.load_library()
        self.copies = copies
        self.bytes = (case.w.nbytes + case.scales.nbytes + 4 + self.x.numel() * 2 + self.out.numel() * 2)
        self.fn = self.lib.nvfp4_qmm
        self.args = None

    def launch(self, i):
        c = i % self.copies
        check(self.lib.nvfp4_qmm(P(self.x), BF16, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]),
                                 P(self.gs), 1, 0, P(self.out), stream_ptr()), "decode qmm")

    def prebuilt(self):
        """Argument tuples for each weight copy, bound to the current stream."""
        st = stream_ptr()
        return [(P(self.x), BF16, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]), P(self.gs), 1, 0,
                 P(self.out), st) for c in range(self.copies)]


DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class Prefill:
    """qmm M=2048, K=5376, N=21504, gs after the matmul; bf16 activations and
    output unless `dtype` says otherwise.  With `workspace` (what the Python
    binding passes) the call is nvfp4_qmm_ws with the workspace
    nvfp4_qmm_workspace_size asks for (none for bf16 and f16 at this size;
    the three-part bf16 copy for float32); without, the one-launch
    nvfp4_qmm."""
    M, K, N = 2048, 5376, 21504

    def __init__(self, decode: Decode, workspace: bool = True, dtype=torch.bfloat16):
        wl = synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]
        g = synth.rng(wl["seed"])
        self.code = DTYPE_CODES[dtype]
        self.x = torch.from_numpy(synth.activations(g, (self.M, self.K))).to(dtype).to(DEV)
        self.w, self.s, self.gs = decode.w, decode.s, decode.gs   # same plane distribution
        self.out = torch.empty((self.M, self.N), dtype=dtype, device=DEV)
        self.lib = decode.lib
        self.flops = 2.0 * self.M * self.N * self.K
        esz = self.x.element_size()
        self.bytes = (decode.w[0].numel() * 4 + decode.s[0].numel() + 4 + self.x.numel() * esz
                      + self.out.numel() * esz)
        nbytes = int(self.lib.nvfp4_qmm_workspace_size(self.M, self.K, self.N, 1, self.code, 0)) if workspace else 0
        self.ws_bytes = nbytes
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes > 0 else None
        self.fn = self.lib.nvfp4_qmm_ws if self.ws is not None else self.lib.nvfp4_qmm

    def prebuilt(self):
        st = stream_ptr()
        if self.ws is not None:
            return [(P(self.x), self.code, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]), P(self.gs), 1, 0,
                     P(self.ws), self.ws_bytes, P(self.out), st) for c in range(len(self.w))]
        return [(P(self.x), self.code, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]), P(self.gs), 1, 0,
                 P(self.out), st) for c in range(len(self.w))]

    def launch(self, i):
        args = self.prebuilt()[i % len(self.w)]
        check(self.fn(*args[:-1], stream_ptr()), "prefill qmm")


class MlpGateUp:
    """Gated MLP projection act(x Wg^T) * (x Wu^T), tanh GELU, at the prefill
    MLP shape M=2048, K=5376, F=21504, bf16, one global scale per plane; the
    gate and up planes of launch c are the weight copies 2c and 2c+1."""
    M, K, F = 2048, 5376, 21504

    def __init__(self, pre: Prefill, decode: Decode, workspace: bool = True):
        self.x = pre.x
        self.w, self.s, self.gs = decode.w, decode.s, decode.gs
        self.out = torch.empty((self.M, self.F), dtype=torch.bfloat16, device=DEV)
        self.lib = decode.lib
        self.flops = 2 * 2.0 * self.M * self.K * self.F
        self.fn = self.lib.nvfp4_qmm_glu
        # the caller-owned workspace that lets the last partial round of tiles
        # split along K (what the Python binding passes)
        nbytes = int(self.lib.nvfp4_qmm_glu_workspace_size(self.M, self.K, self.F, BF16)) if workspace else 0
        self.ws_bytes = nbytes
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes > 0 else None

    def prebuilt(self):
        st = stream_ptr()
        pairs = len(self.w) // 2
        return [(P(self.x), BF16, self.M, self.K, self.F, P(self.w[2 * c]), P(self.s[2 * c]), P(self.gs),
                 P(self.w[2 * c + 1]), P(self.s[2 * c + 1]), P(self.gs), 0, P(self.ws), self.ws_bytes,
                 P(self.out), st) for c in range(pairs)]


class MlpGateUpDecode:
    """The gated projection at the decode MLP shape M=1, K=5376, F=21504,
    bf16, tanh GELU, one global scale per plane: one launch of the decode
    kernel's gated form; gate and up of launch c are weight copies 2c and
    2c+1 (so every launch streams two planes from HBM)."""
    M, K, F = 1, 5376, 21504

    def __init__(self, decode: Decode):
        self.x = decode.x
        self.w, self.s, self.gs = decode.w, decode.s, decode.gs
        self.out = torch.empty((1, self.F), dtype=torch.bfloat16, device=DEV)
        self.lib = decode.lib
        self.bytes = 2 * (decode.w[0].numel() * 4 + decode.s[0].numel() + 4) + self.x.numel() * 2 + self.F * 2
        self.fn = self.lib.nvfp4_qmm_glu

    def prebuilt(self):
        st = stream_ptr()
        return [(P(self.x), BF16, self.M, self.K, self.F, P(self.w[2 * c]), P(self.s[2 * c]), P(self.gs),
                 P(self.w[2 * c + 1]), P(self.s[2 * c + 1]), P(self.gs), 0, None, 0, P(self.out), st)
                for c in range(len(self.w) // 2)]


class MultiRow:
    """qmm M=16, K=4096, N=14336, bf16, gs; 16 weight copies (530 MB)."""
    K, N = 4096, 14336

    def __init__(self, M: int, copies: int):
        wl = synth.WORKLOADS["multirow_qmv_k4096_n14336"]
        case = synth.dense_case(wl["seed"], M, self.K, self.N, with_gs=True)
        w0, s0 = words_dev(case.w), u8_dev(case.scales)
        self.M = M
        self.w = [w0] + [w0.clone() for _ in range(copies - 1)]
        self.s = [s0] + [s0.clone() for _ in range(copies - 1)]
        self.gs = torch.from_numpy(case.gs).to(DEV)
        self.x = torch.from_numpy(case.x).to(torch.bfloat16).to(DEV)
        self.out = torch.empty((M, self.N), dtype=torch.bfloat16, device=DEV)
        self.lib = nv.load_library()
        self.bytes = case.w.nbytes + case.scales.nbytes + 4 + self.x.numel() * 2 + self.out.numel() * 2
        self.flops = 2.0 * M * self.K * self.N
        self.fn = self.lib.nvfp4_qmm

    def prebuilt(self):
        st = stream_ptr()
        return [(P(self.x), BF16, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]), P(self.gs), 1, 0,
                 P(self.out), st) for c in range(len(self.w))]

    def launch(self, i):
        c = i % len(self.w)
        check(self.lib.nvfp4_qmm(P(self.x), BF16, self.M, self.K, self.N, P(self.w[c]), P(self.s[c]),
                                 P(self.gs), 1, 0, P(self.out), stream_ptr()), "multirow qmm")


class Gather:
    """MoE GatherQMM: E=128, N=1536, K=2048, top-8; bf16; per-expert gs."""
    E, N, K, TOPK = 128, 1536, 2048, 8

    def __init__(self, tokens: int, sort: bool, copies: int, seed_off: int = 0):
        wl = synth.WORKLOADS["moe_gather_e128_n1536_k2048_top8"]
        case = synth.gather_case(wl["seed"] + seed_off, tokens=tokens, E=self.E, N=self.N, K=self.K,
                                 top_k=self.TOPK, sort=sort, with_gs=True)
        w0, s0 = words_dev(case.w), u8_dev(case.scales)
        self.w = [w0] + [w0.clone() for _ in range(copies - 1)]
        self.s = [s0] + [s0.clone() for _ in range(copies - 1)]
        self.gs = torch.from_numpy(case.gs).to(DEV)
        self.x = torch.from_numpy(case.x).to(torch.bfloat16).to(DEV)
        self.lhs = torch.from_numpy(case.lhs).to(DEV)
        self.rhs = torch.from_numpy(case.rhs).to(DEV)
        self.R = case.rhs.shape[0]
        self.out = torch.empty((self.R, 1, self.N), dtype=torch.bfloat16, device=DEV)
        self.sort = int(sort)
        self.tokens = tokens
        self.lib = nv.load_library()
        distinct = len(np.unique(case.rhs))
        per_expert = case.w[0].nbytes + case.scales[0].nbytes + 4
        self.distinct = distinct
        self.bytes = (distinct * per_expert + self.x.numel() * 2 + 2 * self.R * 4 + self.out.numel() * 2)
        self.flops = 2.0 * self.R * self.N * self.K
        self.fn = self.lib.nvfp4_gather_qmm

    def prebuilt(self):
        st = stream_ptr()
        return [(P(self.x), BF16, self.tokens, 1, self.K, P(self.lhs), P(self.rhs), self.R, P(self.w[c]),
                 P(self.s[c]), P(self.gs), self.E, self.N, self.sort, P(self.out), st)
                for c in range(len(self.w))]

    def launch(self, i):
        c = i % len(self.w)
        check(self.lib.nvfp4_gather_qmm(P(self.x), BF16, self.tokens, 1, self.K, P(self.lhs), P(self.rhs),
                                        self.R, P(self.w[c]), P(self.s[c]), P(self.gs), self.E, self.N,
                                        self.sort, P(self.out), stream_ptr()), "gather")


# ----------------------------------------------------------------------------
# measurement helpers
# ----------------------------------------------------------------------------

def timed_graph(work, steps: int, warmup: int):
    """Warm up eagerly, capture `steps` launches in one HIP graph, replay it
    once between barriers; returns ms per step."""
    for i in range(warmup):
        work.launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            work.launch(i)
    g.replay()                     # first replay: uploads the graph
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def settle_clocks(work, ms: float = 100.0):
    """Untimed launches of `work` for about `ms` milliseconds before any
    measurement: the device takes tens of milliseconds of sustained load to
    reach its steady clocks, and a process's first few hundred launches
    otherwise run below them."""
    args = work.prebuilt()
    fn, n = work.fn, len(args)
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(64):
            check(fn(*args[i % n]), "settle")
            i += 1
        torch.cuda.synchronize()


def device_state(work, seconds: float = 2.5):
    """Clocks, power and hotspot temperature while `work` runs back to back
    (untimed): one `amd-smi metric --clock --power --temperature --json` sample taken in the middle of
    about `seconds` of launches.  None when the tool is not available."""
    import shutil
    import subprocess
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    args = work.prebuilt()
    fn, n = work.fn, len(args)
    proc = None
    t0 = time.perf_counter()
    i = 0
    try:
        while time.perf_counter() - t0 < seconds:
            for _ in range(16):
                check(fn(*args[i % n]), "device state")
                i += 1
            torch.cuda.synchronize()
            if proc is None and time.perf_counter() - t0 > 0.5:
                proc = subprocess.Popen([tool, "metric", "--clock", "--power", "--temperature", "--json"], stdout=subprocess.PIPE,
                                        stderr=subprocess.DEVNULL, text=True)
        text = proc.communicate(timeout=30)[0] if proc else ""
        gpu = json.loads(text[text.find("{"):])["gpu_data"][0]
        clk = gpu["clock"]
        gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v, dict)]
        return {"gfx_mhz_mean": round(sum(gfx) / len(gfx), 1), "gfx_mhz_min": min(gfx), "gfx_mhz_max": max(gfx),
                "mem_mhz": clk["mem_0"]["clk"]["value"], "socket_power_w": gpu["power"]["socket_power"]["value"],
                "hotspot_c": (gpu.get("temperature") or {}).get("hotspot", {}).get("value"),
                "sampled_during": f"{i} back-to-back launches over {time.perf_counter() - t0:.1f} s"}
    except Exception as exc:  # the measurement is context only
        if proc is not None and proc.poll() is None:
            proc.kill()
        return {"error": f"{type(exc).__name__}: {exc}"[:200]}


def timed_eager(work, steps: int, warmup: int):
    """Warm up, then time `steps` back-to-back launches (prebuilt ctypes
    arguments, so the host stays ahead of the GPU) between HIP events on the
    launch stream, bracketed by synchronizes; returns ms per step."""
    args = work.prebuilt()
    fn, n = work.fn, len(args)
    for i in range(warmup):
        check(fn(*args[i % n]), "warmup")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    bad = 0
    e0.record()
    for i in range(steps):
        bad |= fn(*args[i % n])
    e1.record()
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("a timed launch failed")
    return e0.elapsed_time(e1) / steps


# sources that define the decode kernel and its launch configuration
DECODE_SOURCES = ("decode.hip", "nvfp4_device.hpp")


def kernel_source_sha(files=None) -> str:
    """Digest of the kernel sources (all of them, or the named files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_quantized_matmul_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str):
    """HBM traffic per launch from committed rocprofv3 PMC summaries, if they
    were taken on the current decode sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("decode_source_sha", vals.get("source_sha")) != kernel_source_sha(DECODE_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_us(fn, n: int, warmup: int = 3) -> float:
    """Microseconds per call of fn(i) over n back-to-back calls through the
    Python binding, between events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def measure_library():
    """The benchmark's measurement aid (libnvfp4_measure.so, built beside the
    library but not part of it): nvfp4_stream_read."""
    lib = ctypes.CDLL(os.path.join(ROOT, "nvfp4_quantized_matmul_amd", "libnvfp4_measure.so"))
    lib.nvfp4_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.nvfp4_stream_read.restype = ctypes.c_int
    return lib


def stream_ceiling(nbytes: int, decode_us: float, copies: int = 8, n: int = 100):
    """The best plain streaming read of the decode workload's byte count on
    this device (nvfp4_stream_read over `copies` rotating buffers, a sweep of
    grid sizes), as context for the decode kernel's HBM fraction."""
    lib = measure_library()
    nbytes = nbytes // 16 * 16
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV)
            for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    sweep = {}
    for blocks in (1024, 2048, 4096, 8192, 16384):
        args = [(P(b), nbytes, blocks, P(sink), stream_ptr()) for b in bufs]
        for i in range(8):
            check(lib.nvfp4_stream_read(*args[i % copies]), "stream read")
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            lib.nvfp4_stream_read(*args[i % copies])
        e1.record()
        torch.cuda.synchronize()
        sweep[blocks] = e0.elapsed_time(e1) * 1e3 / n
    best = min(sweep, key=sweep.get)
    us = sweep[best]
    del bufs
    return {"bytes": nbytes, "us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
            "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "blocks": best,
            "sweep_us": {str(k): round(v, 3) for k, v in sweep.items()},
            "decode_frac_of_ceiling": round(us / decode_us, 4),
            "kernel": "stream_read_kernel (grid-stride 16-byte loads, 256 threads)"}


def other_configs():
    """The remaining configurations, each as microseconds per call and the
    rate against its roofline: the tiny qmv (latency), multi-row qmv at every
    M in f32 and bf16, MoE unsorted decode at B = 1, 2, 4, 8, batched-weight
    qmm (all back-to-back C ABI launches with prebuilt arguments), the
    load-time transcode, dequantize and quantize (through the binding), and
    the non-transposed qmm at the prefill shape."""
    out = {}
    lib = nv.load_library()
    # tiny qmv: M=1, K=1024, N=512, f32, no global scale (launch-latency bound)
    wl = synth.WORKLOADS["tiny_qmv_m1_k1024_n512_f32"]
    c = synth.dense_case(wl["seed"], 1, 1024, 512, with_gs=False, code_range=wl["codes"])
    x = torch.from_numpy(c.x).to(DEV)
    w, s = words_dev(c.w), u8_dev(c.scales)
    y = torch.empty((1, 512), dtype=torch.float32, device=DEV)
    targs = (P(x), 0, 1, 1024, 512, P(w), P(s), None, 1, 0, P(y), stream_ptr())
    us = timed_us(lambda i: lib.nvfp4_qmm(*targs), 400, warmup=50)
    binding_us = timed_us(lambda i: nv.qmm(x, w, s, out=y), 200, warmup=20)
    out["tiny_qmv_m1_k1024_n512_f32"] = {"us": round(us, 3), "bytes": 301056, "binding_us": round(binding_us, 3),
                                         "note": "fits in L2; launch latency, not bandwidth, bounds it. us: "
                                                 "back-to-back C ABI launches; binding_us: the same through the "
                                                 "Python binding (host-bound at this size)"}
    # multi-row: one plane, 16 copies (530 MB), every M and dtype
    wl = synth.WORKLOADS["multirow_qmv_k4096_n14336"]
    c = synth.dense_case(wl["seed"], 33, 4096, 14336, with_gs=True)
    w0, s0 = words_dev(c.w), u8_dev(c.scales)
    ws = [w0] + [w0.clone() for _ in range(15)]
    ss = [s0] + [s0.clone() for _ in range(15)]
    gs = torch.from_numpy(c.gs).to(DEV)
    rows = []
    st = stream_ptr()
    for dt, name, size, code in ((torch.bfloat16, "bf16", 2, BF16), (torch.float32, "f32", 4, 0)):
        for M in wl["Ms"]:
            xm = torch.from_numpy(c.x[:M]).to(dt).to(DEV)
            ym = torch.empty((M, 14336), dtype=dt, device=DEV)
            margs = [(P(xm), code, M, 4096, 14336, P(ws[k]), P(ss[k]), P(gs), 1, 0, P(ym), st) for k in range(16)]
            us = timed_us(lambda i: lib.nvfp4_qmm(*margs[i % 16]), 64)
            nbytes = c.w.nbytes + c.scales.nbytes + 4 + M * 4096 * size + M * 14336 * size
            rows.append({"M": M, "dtype": name, "us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
                         "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                         "route": nv.select_route(M, 4096, 14336, dtype=dt)})
    out["multirow_qmv_k4096_n14336"] = rows
    # the gated projection at M = 16 on the same planes (gate and up = copies
    # 2c and 2c + 1): one launch of the multi-row kernel's gated form, beside
    # two multi-row launches and the unfused pipeline
    x16 = torch.from_numpy(c.x[:16]).to(torch.bfloat16).to(DEV)
    y16 = torch.empty((16, 14336), dtype=torch.bfloat16, device=DEV)
    gargs = [(P(x16), BF16, 16, 4096, 14336, P(ws[2 * k]), P(ss[2 * k]), P(gs), P(ws[2 * k + 1]), P(ss[2 * k + 1]),
              P(gs), 0, None, 0, P(y16), st) for k in range(8)]
    glu_us = timed_us(lambda i: lib.nvfp4_qmm_glu(*gargs[i % 8]), 64)
    pair_args = [(P(x16), BF16, 16, 4096, 14336, P(ws[k]), P(ss[k]), P(gs), 1, 0, P(y16), st) for k in range(16)]
    pair_us = 2 * timed_us(lambda i: lib.nvfp4_qmm(*pair_args[i % 16]), 64)
    g16, u16 = torch.empty_like(y16), torch.empty_like(y16)

    def unfused16(i):
        k = i % 8
        nv.qmm(x16, ws[2 * k], ss[2 * k], gs, out=g16)
        nv.qmm(x16, ws[2 * k + 1], ss[2 * k + 1], gs, out=u16)
        torch.nn.functional.gelu(g16, approximate="tanh").mul_(u16)

    unf_us = timed_us(unfused16, 32, warmup=4)
    gbytes = 2 * (c.w.nbytes + c.scales.nbytes + 4) + 16 * 4096 * 2 + 16 * 14336 * 2
    out["mlp_gate_up_multirow_m16_k4096_f14336_bf16"] = {
        "us": round(glu_us, 3), "GB_s": round(gbytes / glu_us / 1e3, 1),
        "frac_hbm": round(gbytes / glu_us / 1e3 / HBM_PEAK_GBS, 4), "bytes": gbytes,
        "separate_pair_us": round(pair_us, 3), "unfused_us": round(unf_us, 3),
        "note": "one launch of the multi-row kernel's gated form (tanh GELU); separate_pair_us = two multi-row "
                "qmm launches; unfused_us = those plus torch's activation and product through the binding"}
    del ws, ss
    # batched weights: two matrices of the multi-row shape at M = 3 (qmv) and 64
    bc = synth.batched_case(3600, B=2, M=64, K=4096, N=14336)
    bw, bs, bg = words_dev(bc.w), u8_dev(bc.scales), torch.from_numpy(bc.gs).to(DEV)
    brow = []
    for M in (3, 64):
        xb = torch.from_numpy(np.ascontiguousarray(bc.x[:, :M])).to(torch.bfloat16).to(DEV)
        yb = torch.empty((2, M, 14336), dtype=torch.bfloat16, device=DEV)
        bargs = (P(xb), BF16, 2, 2, M, 4096, 14336, P(bw), P(bs), P(bg), 1, 0, P(yb), stream_ptr())
        us = timed_us(lambda i: lib.nvfp4_qmm_batched(*bargs), 32)
        nbytes = bc.w.nbytes + bc.scales.nbytes + 8 + xb.numel() * 2 + yb.numel() * 2
        brow.append({"B": 2, "M": M, "dtype": "bf16", "us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
                     "note": "planes fit the MALL (cache-warm); one launch for both matrices"})
    out["batched_qmm_b2_k4096_n14336"] = brow
    # many small matrices (an expert's shape, K = 2048, N = 1536): the
    # batch in one launch beside one call per matrix
    bc = synth.batched_case(3610, B=64, M=8, K=2048, N=1536)
    bw, bs, bg = words_dev(bc.w), u8_dev(bc.scales), torch.from_numpy(bc.gs).to(DEV)
    brow = []
    for M in (1, 8):
        xb = torch.from_numpy(np.ascontiguousarray(bc.x[:, :M])).to(torch.bfloat16).to(DEV)
        yb = torch.empty((64, M, 1536), dtype=torch.bfloat16, device=DEV)
        st = stream_ptr()
        bargs = (P(xb), BF16, 64, 64, M, 2048, 1536, P(bw), P(bs), P(bg), 1, 0, P(yb), st)
        us = timed_us(lambda i: lib.nvfp4_qmm_batched(*bargs), 32)
        per = [(P(xb[b]), BF16, M, 2048, 1536, P(bw[b]), P(bs[b]), P(bg[b:b + 1]), 1, 0, P(yb[b]), st)
               for b in range(64)]
        per_us = timed_us(lambda i: [lib.nvfp4_qmm(*a) for a in per], 8)
        nbytes = bc.w.nbytes + bc.scales.nbytes + 256 + xb.numel() * 2 + yb.numel() * 2
        brow.append({"B": 64, "M": M, "dtype": "bf16", "us": round(us, 3), "GB_s": round(nbytes / us / 1e3, 1),
                     "per_matrix_calls_us": round(per_us, 3),
                     "note": "one launch for the batch beside 64 nvfp4_qmm calls (cache-warm)"})
    out["batched_qmm_b64_k2048_n1536"] = brow
    # MoE unsorted decode at B = 1, 2, 4, 8
    mrow = []
    for B in synth.WORKLOADS["moe_gather_e128_n1536_k2048_top8"]["decode_tokens"]:
        g = Gather(B, False, copies=3, seed_off=B)
        us = eager_launch_us(g, 96)["mean_us"]
        mrow.append({"B": B, "distinct_experts": g.distinct, "us": round(us, 3),
                     "GB_s": round(g.bytes / us / 1e3, 1), "frac_hbm": round(g.bytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del g
    out["moe_unsorted_decode"] = mrow
    # load time at the decode plane's shape [21504, 5376]: transcode (byte move
    # of both planes), dequantize to bf16, quantize from bf16
    gq = synth.rng(6000)
    wu8, wsc, ws2 = synth.modelopt_triplet(gq, 1, 21504, 5376, with_ws2=True)
    tw, tsc, tws2 = torch.from_numpy(wu8[0]).to(DEV), torch.from_numpy(wsc[0]).to(DEV), torch.from_numpy(ws2).to(DEV)
    plane_bytes = wu8[0].nbytes + wsc[0].nbytes
    us = timed_us(lambda i: nv.transcode(tw, tsc, tws2), 16)
    load = {"transcode": {"us": round(us, 2), "GB_s": round(2 * plane_bytes / us / 1e3, 1),
                          "bytes": 2 * plane_bytes}}
    pw, ps, pg = nv.transcode(tw, tsc, tws2)
    us = timed_us(lambda i: nv.dequantize(pw, ps, pg, dtype=torch.bfloat16), 16)
    dq_bytes = plane_bytes + 21504 * 5376 * 2
    load["dequantize_bf16"] = {"us": round(us, 2), "GB_s": round(dq_bytes / us / 1e3, 1), "bytes": dq_bytes}
    dense = nv.dequantize(pw, ps, pg, dtype=torch.bfloat16)
    us = timed_us(lambda i: nv.quantize(dense), 16)
    q_bytes = 2 * 21504 * 5376 * 2 + plane_bytes
    load["quantize_bf16"] = {"us": round(us, 2), "GB_s": round(q_bytes / us / 1e3, 1), "bytes": q_bytes,
                             "note": "two passes over the dense input (matrix maximum, then blocks)"}
    out["load_time_21504x5376"] = load
    # non-transposed plane [K, N/8] at the prefill shape: the dense route
    # (the plane's exact transposed bf16 copy in the workspace, then the
    # matrix-core GEMM), beside the generic kernel (nvfp4_qmm, no workspace)
    M, K, N = 2048, 5376, 21504
    cn = synth.dense_case(synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]["seed"] + 11, 1, K, N,
                          transpose=False, with_gs=True)
    wn, sn, gn = words_dev(cn.w), u8_dev(cn.scales), torch.from_numpy(cn.gs).to(DEV)
    xn = torch.from_numpy(synth.activations(synth.rng(12), (M, K))).to(torch.bfloat16).to(DEV)
    yn = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    need = int(lib.nvfp4_qmm_workspace_size(M, K, N, 0, BF16, 0))
    wsn = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = stream_ptr()
    dargs = (P(xn), BF16, M, K, N, P(wn), P(sn), P(gn), 0, 0, P(wsn), need, P(yn), st)
    gargs = (P(xn), BF16, M, K, N, P(wn), P(sn), P(gn), 0, 0, P(yn), st)
    flops = 2.0 * M * N * K
    dense_us = timed_us(lambda i: lib.nvfp4_qmm_ws(*dargs), 16, warmup=4)
    generic_us = timed_us(lambda i: lib.nvfp4_qmm(*gargs), 2, warmup=1)
    out["non_transposed_gemm_m2048_k5376_n21504_bf16"] = {
        "us": round(dense_us, 2), "TFLOP_s": round(flops / dense_us / 1e6, 2),
        "frac_of_bf16_peak": round(flops / dense_us / 1e6 / BF16_PEAK_TFLOPS, 4), "workspace_bytes": need,
        "generic_us": round(generic_us, 2),
        "note": "us: nvfp4_qmm_ws (dense transposed copy of the plane, then the matrix-core GEMM on it); "
                "generic_us: nvfp4_qmm without a workspace (float32 FMA kernel)"}
    del wsn
    return out


def _host_threads():
    """(BLAS threads, host cores this process may run on)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas = 1
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not on Linux
        host = os.cpu_count() or 1
    return int(blas), int(host)


def _time_oracle(fn, max_reps: int, max_wall: float):
    reps, wall, cpu = 0, 0.0, 0.0
    while reps < max_reps and (reps == 0 or wall < max_wall):
        t0, c0 = time.perf_counter(), time.process_time()
        fn()
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        reps += 1
    return reps, wall / reps, cpu / wall


def cpu_baseline(decode_bytes: float):
    """The oracle, untuned, on the host: the full decode workload (dequantize
    the plane, then the float64 product), passes repeated up to about 10 s.  `cores` is the BLAS thread count
    (the most threads the oracle runs at once: its dequantize runs on one,
    its matmul on all); `host_cores` the cores the process may use."""
    import oracle
    blas, host = _host_threads()
    wl = synth.WORKLOADS["decode_qmv_m1_k5376_n21504_bf16"]
    case = synth.dense_case(wl["seed"], 1, 5376, 21504, with_gs=True)
    x = torch.from_numpy(case.x).to(torch.bfloat16).float().numpy()
    reps, per, busy = _time_oracle(lambda: oracle.qmm(x, case.w, case.scales, case.gs[0]), 16, 10.0)
    return {"value": round(decode_bytes / per / 1e9, 4), "unit": "GB/s", "cores": blas, "host_cores": host,
            "mean_busy_cores": round(busy, 2), "kind": "oracle",
            "sample": f"full decode workload M=1 K=5376 N=21504 (dequantize + float64 matmul), "
                      f"{reps} pass(es), {per:.2f} s per pass"}


def cpu_baseline_prefill(flops: float):
    """The oracle on the whole prefill workload (M=2048, K=5376, N=21504: the
    plane dequantized once per pass, then a float64 product of all 2048
    rows), passes repeated up to about 10 s, as TFLOP/s of the workload's
    2MNK."""
    import oracle
    blas, host = _host_threads()
    wl = synth.WORKLOADS["prefill_gemm_m2048_k5376_n21504_bf16"]
    case = synth.dense_case(wl["seed"], 1, 5376, 21504, with_gs=True)
    x = torch.from_numpy(synth.activations(synth.rng(wl["seed"]), (2048, 5376))).to(torch.bfloat16).float().numpy()
    reps, per, busy = _time_oracle(lambda: oracle.qmm(x, case.w, case.scales, case.gs[0]), 12, 10.0)
    return {"value": round(flops / per / 1e12, 6), "unit": "TFLOP/s", "cores": blas, "host_cores": host,
            "mean_busy_cores": round(busy, 2), "kind": "oracle",
            "sample": f"full prefill workload M=2048 K=5376 N=21504 (dequantize + float64 matmul), "
                      f"{reps} pass(es), {per:.2f} s per pass"}


COPY_BYTES = 256 << 20

# Workloads for hardware-counter runs: the kernel each one times and the
# sources that define it (the digest recorded beside its counter summary).
COUNTER_WORKLOADS = {
    "decode": ("decode.hip", "nvfp4_device.hpp"),
    "prefill": ("gemm.hip", "nvfp4_device.hpp"),
    "multirow16": ("skinny.hip", "nvfp4_device.hpp"),
    "moe_sorted": ("skinny.hip", "nvfp4_device.hpp"),
}


def counters_run(name: str, steps: int):
    """Workload for rocprofv3 PMC passes: one plain device copy of COPY_BYTES
    (it reads and writes exactly that many bytes, so its counter values give
    the scale of the counters), then `steps` launches of the named workload,
    each on a synchronized stream so that every dispatch is counted on its
    own.  Prints the launch count, the algorithmic bytes and flops per
    launch, and the digest of the kernel's sources."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.int32, device=DEV).fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if name == "decode":
        work = Decode(copies=8)
    elif name == "prefill":
        work = Prefill(Decode(copies=8))
    elif name == "multirow16":
        work = MultiRow(16, copies=16)
    else:
        work = Gather(128, True, copies=3)
    args = work.prebuilt()
    torch.cuda.synchronize()
    for i in range(steps):
        check(work.fn(*args[i % len(args)]), name)
        torch.cuda.synchronize()
    print(json.dumps({"workload": name, "copy_bytes": COPY_BYTES, "launches": steps,
                      "bytes_per_launch": getattr(work, "bytes", None),
                      "flops_per_launch": getattr(work, "flops", None),
                      "source_sha": kernel_source_sha(COUNTER_WORKLOADS[name])}), flush=True)


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--counters", choices=sorted(COUNTER_WORKLOADS),
                    help="for hardware-counter runs: a 256 MiB device copy (the calibration of "
                         "FETCH_SIZE/WRITE_SIZE against known bytes), then `steps` launches of the named "
                         "workload; prints the launch count and bytes instead of the JSON line")
    ap.add_argument("--counters-decode", action="store_true", help="the same as --counters decode")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the NVFP4 matmul path here is single-GPU "
              "(sharding across GPUs is described in the design notes, not run).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    nv.load_library()
    if args.counters or args.counters_decode:
        counters_run(args.counters or "decode", steps)
        return

    log("decode: building inputs")
    dec = Decode(copies=8)
    settle_clocks(dec)
    log("decode: timed region")
    ms = timed_eager(dec, steps, warmup)
    graph_ms = timed_graph(dec, steps, warmup)
    value = dec.bytes / (ms * 1e-3) / 1e9
    # the timed region is K back-to-back launches of the one kernel, so its
    # average launch duration is the per-step time
    dur = {"mean_us": ms * 1e3, "launches": steps,
           "source": "HIP events around the timed back-to-back launches"}
    achieved = value
    traffic = traffic_for("decode_qmv")

    log("streaming-read ceiling")
    ceiling = stream_ceiling(dec.bytes, ms * 1e3)

    log("prefill")
    pre = Prefill(dec)
    # the clocks take a few hundred milliseconds of sustained MFMA load to
    # settle (tens of milliseconds still time the ramp): ~300 ms untimed first
    settle_clocks(pre, 300.0)
    pdur = eager_launch_us(pre, 16, warmup=4)
    ptf = pre.flops / (pdur["mean_us"] * 1e-6) / 1e12

    # context, measurement only: the vendor bf16 GEMM (torch linear) on the
    # same shape with a dense bf16 weight matrix, the rate a tuned library
    # reaches here without any dequantization
    wd = torch.randn(pre.N, pre.K, device=DEV).to(torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:            # the same settling as the prefill above
        timed_us(lambda i: torch.nn.functional.linear(pre.x, wd), 16, warmup=0)
    dense_us = timed_us(lambda i: torch.nn.functional.linear(pre.x, wd), 16, warmup=0)
    del wd

    # the same call with f16 activations (the f16 matrix-core GEMM) and with
    # float32 activations (their three-part bf16 copy in the binding's
    # workspace, then the bf16 GEMM over 3K)
    dt_rates = {}
    for name, dt in (("f16", torch.float16), ("f32", torch.float32)):
        pw = Prefill(dec, dtype=dt)
        settle_clocks(pw, 150.0)
        d = eager_launch_us(pw, 16, warmup=2)
        dt_rates[name] = {"value": round(pw.flops / (d["mean_us"] * 1e-6) / 1e12, 2), "unit": "TFLOP/s",
                          "workspace_bytes": pw.ws_bytes, "kernel_duration": d,
                          "frac_of_bf16_peak": round(pw.flops / (d["mean_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del pw

    log("mlp gate/up")
    mlp = MlpGateUp(pre, dec)
    settle_clocks(mlp, 300.0)
    gdur = eager_launch_us(mlp, 16, warmup=2)
    gtf = mlp.flops / (gdur["mean_us"] * 1e-6) / 1e12
    mlp_nows = MlpGateUp(pre, dec, workspace=False)
    settle_clocks(mlp_nows, 100.0)
    nows_us = eager_launch_us(mlp_nows, 16, warmup=2)["mean_us"]
    del mlp_nows
    # the same projection unfused, for comparison: two library qmm launches
    # (gate, up) and the activation and product as torch elementwise ops
    gate_t = torch.empty_like(mlp.out)
    up_t = torch.empty_like(mlp.out)

    def unfused(i):
        c = i % (len(dec.w) // 2)
        nv.qmm(pre.x, dec.w[2 * c], dec.s[2 * c], dec.gs, out=gate_t)
        nv.qmm(pre.x, dec.w[2 * c + 1], dec.s[2 * c + 1], dec.gs, out=up_t)
        torch.nn.functional.gelu(gate_t, approximate="tanh").mul_(up_t)

    unfused_us = timed_us(unfused, 8, warmup=2)
    del gate_t, up_t

    log("mlp gate/up, decode")
    mlpd = MlpGateUpDecode(dec)
    ddur = eager_launch_us(mlpd, 64, warmup=16)
    dgbs = mlpd.bytes / (ddur["mean_us"] * 1e-6) / 1e9
    gate1 = torch.empty((1, 21504), dtype=torch.bfloat16, device=DEV)
    up1 = torch.empty((1, 21504), dtype=torch.bfloat16, device=DEV)

    def unfused_decode(i):
        c = i % (len(dec.w) // 2)
        nv.qmm(dec.x, dec.w[2 * c], dec.s[2 * c], dec.gs, out=gate1)
        nv.qmm(dec.x, dec.w[2 * c + 1], dec.s[2 * c + 1], dec.gs, out=up1)
        torch.nn.functional.gelu(gate1, approximate="tanh").mul_(up1)

    unfused_decode_us = timed_us(unfused_decode, 32, warmup=4)

    log("multi-row qmv")
    mr = MultiRow(16, copies=16)
    mdur = eager_launch_us(mr, 64)
    mgbs = mr.bytes / (mdur["mean_us"] * 1e-6) / 1e9

    log("device state (amd-smi during sustained decode, prefill and gated prefill)")
    state = {"decode": device_state(dec), "prefill": device_state(pre), "mlp_gate_up_prefill": device_state(mlp)}

    log("moe gather")
    gs_sorted = Gather(128, True, copies=3)
    sdur = eager_launch_us(gs_sorted, 24)
    sgbs = gs_sorted.bytes / (sdur["mean_us"] * 1e-6) / 1e9
    gs_dec = Gather(8, False, copies=3, seed_off=8)
    udur = eager_launch_us(gs_dec, 96)
    ugbs = gs_dec.bytes / (udur["mean_us"] * 1e-6) / 1e9

    log("other configurations")
    others = other_configs()

    cpu = cpu_pre = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(dec.bytes)
        cpu_pre = cpu_baseline_prefill(pre.flops)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_qmv_m1_k5376_n21504_bf16", "M": 1, "K": 5376, "N": 21504,
                   "activations": "bf16", "global_scale": True, "weight_copies": 8,
                   "launch": "`steps` back-to-back nvfp4_qmm launches on one stream",
                   "bytes_per_step": dec.bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "qmv1_kernel<bf16,3,1>",
                     "kernel_duration": dur},
        "cpu_baseline": cpu,
        "stream_ceiling": ceiling,
        "device_state": state,
        "graph_ms_per_step": round(graph_ms, 6),
        "prefill": {"workload": "prefill_gemm_m2048_k5376_n21504_bf16", "value": round(ptf, 2),
                    "unit": "TFLOP/s", "flops": pre.flops,
                    "roofline": {"bound": "mfma", "achieved": round(ptf, 2), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ptf / BF16_PEAK_TFLOPS, 4),
                                 "kernel": "gemm_mfma_v3p_kernel (persistent)", "kernel_duration": pdur},
                    "cpu_baseline": cpu_pre,
                    "activations_f16": dt_rates["f16"],
                    "activations_f32": dt_rates["f32"],
                    "dense_bf16_gemm_reference": {"us": round(dense_us, 2),
                                                  "TFLOP_s": round(pre.flops / dense_us / 1e6, 2),
                                                  "note": "torch linear (vendor library) with a dense bf16 "
                                                          "weight of the same shape; context only"}},
        "mlp_gate_up_prefill": {"workload": "mlp_gate_up_m2048_k5376_f21504_bf16_gelu_tanh",
                                "value": round(gtf, 2), "unit": "TFLOP/s", "flops": mlp.flops,
                                "roofline": {"bound": "mfma", "achieved": round(gtf, 2), "peak": BF16_PEAK_TFLOPS,
                                             "unit": "TFLOP/s", "frac": round(gtf / BF16_PEAK_TFLOPS, 4),
                                             "kernel": "gemm_mfma_v3_kernel<glu>", "kernel_duration": gdur},
                                "workspace_bytes": mlp.ws_bytes,
                                "no_workspace_us": round(nows_us, 2),
                                "separate_qmm_pair_us": round(2 * pdur["mean_us"], 2),
                                "unfused_us": round(unfused_us, 2),
                                "note": "the fused kernel with its workspace (the last partial round of tiles "
                                        "split along K, three launches per step); no_workspace_us = the same call "
                                        "without one (one launch); separate_qmm_pair_us = two prefill qmm "
                                        "launches of the same planes; unfused_us = those two launches plus the "
                                        "activation and product as torch elementwise ops (measurement only)"},
        "mlp_gate_up_decode": {"workload": "mlp_gate_up_m1_k5376_f21504_bf16_gelu_tanh", "value": round(dgbs, 2),
                               "unit": "GB/s", "frac_hbm": round(dgbs / HBM_PEAK_GBS, 4), "bytes": mlpd.bytes,
                               "kernel": "qmv1_kernel<bf16,3,2,glu>", "kernel_duration": ddur,
                               "separate_decode_pair_us": round(2 * ms * 1e3, 3),
                               "unfused_us": round(unfused_decode_us, 3),
                               "note": "one launch streaming both planes; separate_decode_pair_us = two decode "
                                       "launches (the headline's per-step time, twice); unfused_us = two qmm calls "
                                       "plus the activation and product as torch elementwise ops, through the "
                                       "binding (measurement only)"},
        "multirow_m16": {"workload": "multirow_qmv_m16_k4096_n14336_bf16", "value": round(mgbs, 2),
                         "unit": "GB/s", "frac_hbm": round(mgbs / HBM_PEAK_GBS, 4),
                         "kernel": "skinny_kernel<bf16,1,16>", "kernel_duration": mdur, "bytes": mr.bytes},
        "moe_sorted_prefill": {"workload": "moe_gather_e128_n1536_k2048_top8_b128_sorted",
                               "value": round(sgbs, 2), "unit": "GB/s",
                               "frac_hbm": round(sgbs / HBM_PEAK_GBS, 4), "distinct_experts": gs_sorted.distinct,
                               "kernel": "gather_mfma_kernel<4>", "kernel_duration": sdur,
                               "bytes": gs_sorted.bytes},
        "moe_unsorted_decode_b8": {"workload": "moe_gather_e128_n1536_k2048_top8_b8_unsorted",
                                   "value": round(ugbs, 2), "unit": "GB/s",
                                   "frac_hbm": round(ugbs / HBM_PEAK_GBS, 4),
                                   "distinct_experts": gs_dec.distinct,
                                   "kernel": "qmv1_gather_kernel<bf16,1>", "kernel_duration": udur,
                                   "bytes": gs_dec.bytes},
        "other_configs": others,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
