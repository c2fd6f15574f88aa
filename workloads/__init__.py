"""Seeded synthetic inputs for the ternary-weight matmul.

This module draws random inputs and nothing else: it holds none of the
method's arithmetic (no decoding, no matmul, no scaling).  Both the CPU oracle
tests and the HIP path's tests and benchmark take their inputs from here, so
the two sides always see the same bytes.

Workloads stand in for the pages' models, none of which is available here:
  * a 27B-class, 48-layer decoder run ternary at 2 bits per weight
    ("Ternary-Bonsai-2-27B" pages on bhfrc.com/news/45317 §1-§2 and
    hotelren.com/news/5173450 §1), hidden size 5120, FFN 17408;
  * a ~0.6B ternary embedding model (2kiu.com/news/5082861 "ternary
    embedding model on vLLM", §1.1), hidden sizes 1024 / 3072.

Packed weight bytes are drawn directly: every byte is four independent 2-bit
codes drawn from the stated code distribution.  Because the codes are drawn
independently, the byte distribution does not depend on the order in which the
four codes sit inside a byte, so no part of the packing layout is encoded
here.  Floating-point values are drawn in float64 and rounded once to the
stored type (round-to-nearest-even).

Seeds: numpy.random.default_rng(SeedSequence([0, cfg_id, tensor_id, shape_id])).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

GROUP = 128  # weights per fp16 scale along K

# Tensor ids inside a seed sequence.
_T_CODES, _T_SCALES, _T_X, _T_OUTLIER = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Shape:
    """One matmul problem Y[M,N] = X[M,K] . W[N,K]^T."""

    M: int
    K: int
    N: int
    label: str = ""


@dataclasses.dataclass(frozen=True)
class Config:
    """A workload: shapes plus the distributions its tensors are drawn from."""

    cfg_id: int
    name: str
    shapes: Tuple[Shape, ...]
    code_probs: Tuple[float, float, float, float]  # P(code 00), P(01), P(10), P(11)
    reserved_rate: float  # after drawing, each code turns into 11 with this probability
    scale_kind: str  # "uniform" or "loguniform"
    scale_lo: float
    scale_hi: float
    x_dtype: str  # "f16" | "bf16"
    x_sigma: float
    outlier_rate: float  # probability that an X element is multiplied by outlier_mult
    outlier_mult: float
    y_dtype: str  # "f32" | "bf16" | "f16"


def _sweep_shapes() -> Tuple[Shape, ...]:
    # 48 layers x 7 projections at M=1 with the 5120/17408 shapes:
    # q, k, v, o as 5120->5120, gate and up 5120->17408, down 17408->5120.
    out: List[Shape] = []
    for layer in range(48):
        for proj in ("q", "k", "v", "o"):
            out.append(Shape(1, 5120, 5120, f"L{layer}.{proj}"))
        out.append(Shape(1, 5120, 17408, f"L{layer}.gate"))
        out.append(Shape(1, 5120, 17408, f"L{layer}.up"))
        out.append(Shape(1, 17408, 5120, f"L{layer}.down"))
    return tuple(out)


CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny", (Shape(1, 512, 256, "tiny"),),
              (1 / 3, 1 / 3, 1 / 3, 0.0), 0.01, "uniform", 0.01, 0.1,
              "f16", 1.0, 0.0, 1.0, "f32"),
    2: Config(2, "attn_decode", (Shape(1, 5120, 5120, "attn"),),
              (0.4, 0.3, 0.3, 0.0), 0.0, "loguniform", 1e-3, 1e-1,
              "bf16", 1.0, 0.0, 1.0, "bf16"),
    3: Config(3, "ffn_decode",
              tuple(Shape(m, k, n, lab) for m in (1, 4, 16)
                    for (k, n, lab) in ((5120, 17408, "up"), (17408, 5120, "down"))),
              (0.4, 0.3, 0.3, 0.0), 0.0, "loguniform", 1e-3, 1e-1,
              "bf16", 0.5, 0.0, 1.0, "bf16"),
    4: Config(4, "prefill",
              tuple(Shape(m, 5120, n, lab) for m in (256, 2048)
                    for (n, lab) in ((7168, "qkv"), (17408, "ffn"))),
              (1 / 3, 1 / 3, 1 / 3, 0.0), 0.0, "uniform", 0.005, 0.05,
              "f16", 1.0, 0.01, 20.0, "f16"),
    5: Config(5, "embedding",
              (Shape(4096, 1024, 1024, "emb_1k_1k"), Shape(4096, 1024, 3072, "emb_1k_3k"),
               Shape(4096, 3072, 1024, "emb_3k_1k")),
              (1 / 3, 1 / 3, 1 / 3, 0.0), 0.0, "uniform", 0.005, 0.05,
              "f16", 1.0, 0.0, 1.0, "f16"),
    6: Config(6, "decode_sweep", _sweep_shapes(),
              (0.4, 0.3, 0.3, 0.0), 0.0, "loguniform", 1e-3, 1e-1,
              "bf16", 1.0, 0.0, 1.0, "bf16"),
}


def rng_for(cfg_id: int, tensor_id: int, shape_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, cfg_id, tensor_id, shape_id]))


def draw_codes(rng: np.random.Generator, n: int, k: int,
               probs=(1 / 3, 1 / 3, 1 / 3, 0.0), reserved_rate: float = 0.0) -> np.ndarray:
    """i.i.d. 2-bit codes, uint8 array [n, k] with values 0..3."""
    p = np.asarray(probs, dtype=np.float64)
    p = p / p.sum()
    codes = rng.choice(4, size=(n, k), p=p).astype(np.uint8)
    if reserved_rate > 0:
        codes[rng.random((n, k)) < reserved_rate] = 3
    return codes


def draw_packed(rng: np.random.Generator, n: int, k: int,
                probs=(1 / 3, 1 / 3, 1 / 3, 0.0), reserved_rate: float = 0.0) -> np.ndarray:
    """Random bytes [n, k//4]; each byte holds four independent codes.

    The four codes of a byte are drawn independently from the same
    distribution, so the result does not depend on where each sits.
    """
    assert k % 4 == 0
    c = draw_codes(rng, n, k, probs, reserved_rate).reshape(n, k // 4, 4).astype(np.uint32)
    b = c[..., 0] + 4 * c[..., 1] + 16 * c[..., 2] + 64 * c[..., 3]
    return np.ascontiguousarray(b.astype(np.uint8))


def to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16))


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, round-to-nearest-even.

    Done in two exact-or-rounded steps: float64 -> float32 (RNE), then the
    float32 bit pattern is rounded to its top 16 bits (RNE).  Double rounding
    can differ from a direct float64 -> bf16 rounding in rare ties; the values
    are random inputs, so any fixed rule serves.
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(f)
    r = np.where(nan, 0x7FC0, r)
    return np.ascontiguousarray(r.astype(np.uint16))


def draw_scales(rng: np.random.Generator, n: int, groups: int, kind: str,
                lo: float, hi: float) -> np.ndarray:
    """fp16 bit patterns [n, groups]."""
    if kind == "uniform":
        v = rng.uniform(lo, hi, size=(n, groups))
    elif kind == "loguniform":
        v = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(n, groups)))
    else:
        raise ValueError(kind)
    return to_f16_bits(v)


def draw_x(rng: np.random.Generator, m: int, k: int, dtype: str, sigma: float = 1.0,
           outlier_rate: float = 0.0, outlier_mult: float = 1.0,
           rng_outlier: Optional[np.random.Generator] = None) -> np.ndarray:
    """Activation bit patterns [m, k] (uint16) of the given dtype."""
    v = rng.normal(0.0, sigma, size=(m, k))
    if outlier_rate > 0:
        r = rng_outlier if rng_outlier is not None else rng
        v = np.where(r.random((m, k)) < outlier_rate, v * outlier_mult, v)
    if dtype == "f16":
        return to_f16_bits(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    raise ValueError(dtype)


@dataclasses.dataclass
class Problem:
    """Host arrays of one problem: X bits, packed W, scale bits."""

    shape: Shape
    x: np.ndarray  # uint16 [M, K]
    x_dtype: str
    packed: np.ndarray  # uint8 [N, K/4]
    scales: np.ndarray  # uint16 [N, K/128]
    y_dtype: str
    group: int = GROUP


def make_problem(cfg_id: int, shape_id: int = 0, shape: Optional[Shape] = None) -> Problem:
    cfg = CONFIGS[cfg_id]
    sh = shape if shape is not None else cfg.shapes[shape_id]
    packed = draw_packed(rng_for(cfg_id, _T_CODES, shape_id), sh.N, sh.K,
                         cfg.code_probs, cfg.reserved_rate)
    scales = draw_scales(rng_for(cfg_id, _T_SCALES, shape_id), sh.N, sh.K // GROUP,
                         cfg.scale_kind, cfg.scale_lo, cfg.scale_hi)
    x = draw_x(rng_for(cfg_id, _T_X, shape_id), sh.M, sh.K, cfg.x_dtype, cfg.x_sigma,
               cfg.outlier_rate, cfg.outlier_mult, rng_for(cfg_id, _T_OUTLIER, shape_id))
    return Problem(sh, x, cfg.x_dtype, packed, scales, cfg.y_dtype)


def make_custom(seed: int, M: int, K: int, N: int, x_dtype: str = "f16", y_dtype: str = "f32",
                probs=(0.4, 0.3, 0.3, 0.0), reserved_rate: float = 0.0,
                scale_lo: float = 1e-3, scale_hi: float = 1e-1, x_sigma: float = 1.0,
                group: int = GROUP) -> Problem:
    """A problem of any shape (tests: ragged tails, edge cases); cfg id 100."""
    sh = Shape(M, K, N, "custom")
    packed = draw_packed(rng_for(100, _T_CODES, seed), N, K, probs, reserved_rate)
    scales = draw_scales(rng_for(100, _T_SCALES, seed), N, K // group, "loguniform",
                         scale_lo, scale_hi)
    x = draw_x(rng_for(100, _T_X, seed), M, K, x_dtype, x_sigma)
    return Problem(sh, x, x_dtype, packed, scales, y_dtype, group)


def draw_ternary(seed: int, n: int, k: int, probs=(0.4, 0.3, 0.3)) -> np.ndarray:
    """int8 [n, k] with values in {-1, 0, +1} (input of the pack step)."""
    rng = rng_for(101, 0, seed)
    p = np.asarray(probs, dtype=np.float64)
    return np.ascontiguousarray(rng.choice(np.array([0, 1, -1], dtype=np.int8), size=(n, k),
                                           p=p / p.sum()))


def draw_block_sparse_packed(rng: np.random.Generator, n: int, k: int, zero_group_rate: float,
                             probs=(0.4, 0.3, 0.3, 0.0), group: int = GROUP) -> np.ndarray:
    """Packed bytes where whole 128-weight groups are all-zero with the given rate.

    An all-zero group is 32 zero bytes whatever the code order, so this, too,
    is layout-free.
    """
    p = draw_packed(rng, n, k, probs)
    zero = rng.random((n, k // group)) < zero_group_rate
    p = p.reshape(n, k // group, group // 4)
    p[zero] = 0
    return np.ascontiguousarray(p.reshape(n, k // 4))


# --- device-side generators (large workloads: the 4.5 GB decode sweep) -------

def draw_packed_device(gen, n: int, k: int, probs=(1 / 3, 1 / 3, 1 / 3, 0.0)):
    """uint8 [n, k//4] on the generator's device: four independent codes per byte."""
    import torch

    p = torch.tensor(probs, dtype=torch.float64)
    cdf = torch.cumsum(p / p.sum(), 0).to(torch.float32).tolist()
    out = torch.zeros((n, k // 4), dtype=torch.int32, device=gen.device)
    for i in range(4):
        u = torch.rand((n, k // 4), generator=gen, device=gen.device)
        code = (u >= cdf[0]).int() + (u >= cdf[1]).int() + (u >= cdf[2]).int()
        out += code << (2 * i)
    return out.to(torch.uint8).contiguous()


def draw_scales_device(gen, n: int, groups: int, lo: float, hi: float):
    """fp16 [n, groups], log-uniform in [lo, hi], on the generator's device."""
    import math

    import torch

    u = torch.rand((n, groups), generator=gen, device=gen.device, dtype=torch.float64)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.float16).contiguous()
