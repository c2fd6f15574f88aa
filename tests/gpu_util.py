"""Helpers of the GPU tests: move seeded problems to the device, run the HIP
path through the binding, and compare with the oracle under the pass
criterion |Y_gpu - Y| <= 2e-3 * sum_k |x*s| + one ulp of the output type."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
BITS_DT = {"f16": torch.int16, "bf16": torch.int16, "f32": torch.int32}
REL_TOL = 2e-3


def device():
    return torch.device("cuda:0")


def bits_to_device(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device()).view(TORCH_DT[dtype])


def problem_to_device(p):
    x = bits_to_device(p.x, p.x_dtype)
    w = torch.from_numpy(np.ascontiguousarray(p.packed)).to(device())
    s = bits_to_device(p.scales, "f16")
    return x, w, s


def out_bits(y: torch.Tensor, dtype: str) -> np.ndarray:
    host = y.view(BITS_DT[dtype]).cpu().numpy()
    return host.view(np.uint32 if dtype == "f32" else np.uint16)


def run(p, path="auto", tensors=None):
    """The product into an output filled with NaN first, so an output the
    kernel fails to write cannot pass on what an earlier call left in the
    same memory."""
    import ternary_weight_matmul_amd as tern
    x, w, s = tensors if tensors is not None else problem_to_device(p)
    y = torch.full((p.shape.M, p.shape.N), float("nan"), dtype=TORCH_DT[p.y_dtype], device=x.device)
    tern.matmul_into(x, w, s, y, path=path)
    torch.cuda.synchronize()
    return y


def run_s8(x, w, q, r, M, N, y_dtype, path="auto"):
    """tern_matmul_s8 into an output filled with NaN first (as run() does)."""
    import ternary_weight_matmul_amd as tern
    y = torch.full((M, N), float("nan"), dtype=TORCH_DT[y_dtype], device=x.device)
    tern.matmul_s8_into(x, w, q, r, y, path=path)
    torch.cuda.synchronize()
    return y


def check(y_bits: np.ndarray, y_dtype: str, Y: np.ndarray, B: np.ndarray, what: str = "") -> float:
    """Assert the pass criterion elementwise; return the worst error / allowance."""
    o = oracle.default()
    got = o.decode(y_bits, y_dtype)
    allow = o.tolerance(Y, B, y_dtype, REL_TOL)
    err = np.abs(got - Y)
    bad = ~(err <= allow)
    if bad.any():
        idx = np.argwhere(bad)[:8]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside tolerance; "
                             f"first {idx.tolist()}: got {got[bad][:8]}, want {Y[bad][:8]}, "
                             f"allow {allow[bad][:8]}")
    return float(np.max(err / allow)) if err.size else 0.0


def sample_indices(M: int, N: int, count: int, seed: int = 0):
    """Sampled (m, n): the four corners, random outputs, and random columns of the last row."""
    rng = np.random.default_rng(seed)
    ms = [0, 0, M - 1, M - 1] + rng.integers(0, M, count).tolist() + [M - 1] * 16
    ns = [0, N - 1, 0, N - 1] + rng.integers(0, N, count).tolist() + rng.integers(0, N, 16).tolist()
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
