"""Helpers for the GPU parity tests: move seeded inputs to the device and
bring results back for comparison with the oracle."""

import numpy as np
import torch

DEV = "cuda:0"

# Tolerances, max |out - ref| / max |ref|: float32 output 1e-5; bf16 and
# f16 output 1e-2 (rounding of the output to 8 or 11 significant bits
# dominates; the contraction itself accumulates in float32).
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2, torch.float16: 1e-2}


def words(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


def u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def activations(x: np.ndarray, dtype):
    """Device activations of `dtype` and the exact float32 values the
    oracle sees (bf16/f16 inputs are rounded once, on the host, by torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.to(DEV), t.float().numpy()


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def guarded(shape, dtype, guard_elems=64, fill=None):
    """An output view surrounded by guard bands filled with a sentinel;
    returns (view, check) where check() asserts the guards are intact."""
    n = int(np.prod(shape)) if len(shape) else 1
    base = torch.empty(n + 2 * guard_elems, dtype=dtype, device=DEV)
    sentinel = fill if fill is not None else (-12345.0 if dtype.is_floating_point else 0x5A)
    base.fill_(sentinel)
    view = base[guard_elems:guard_elems + n].view(shape)

    def check():
        torch.cuda.synchronize()
        lo = base[:guard_elems].float().cpu()
        hi = base[guard_elems + n:].float().cpu()
        want = torch.full_like(lo, float(torch.tensor(sentinel, dtype=dtype).float()))
        assert torch.equal(lo, want) and torch.equal(hi, want), "write outside the output buffer"
    return view, check
