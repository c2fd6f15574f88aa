"""The decode kernels whose sign-select sums run on the matrix cores, against
the CPU oracle, on the GPU: TERN_PATH_GEMV_MFMA (+-2 / 0 16-bit operands of
v_mfma_f32_4x4x4_16b) and TERN_PATH_GEMV_FP4 (e2m1 weight operands, bf16
activations split exactly into two e4m3 terms per 32-block scale; bf16 only).

Outputs must meet |Y_gpu - Y_oracle| <= 2e-3 * sum_k |x*s| + one ulp of the
output type, elementwise, and equal the oracle's value rounded to the output
type bit for bit where the arithmetic is exact.  The cases walk the kernel's
work layout: quads of 4 rows (N off the multiple of 4), 1024-weight steps
(K off the multiple of 1024, down to one 128-weight block), units per wave
from 1 to 8, workgroups of one quad up to many quads with more than one
round of workgroups, staged activations from 1 to 6 blocks per thread (LDS
beyond 64 KB), and every dtype pair.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import (TORCH_DT, bits_to_device, check, device, out_bits, problem_to_device,  # noqa: E402
                      run, run_s8)

tern = pytest.importorskip("ternary_weight_matmul_amd")

PATHS = ["gemv_mfma", "gemv_fp4"]
O = oracle.default


def _paths(x_dtype):
    return PATHS if x_dtype == "bf16" else ["gemv_mfma"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _full(p, path):
    sh = p.shape
    print(f"case {sh.M}x{sh.K}x{sh.N} {p.x_dtype}->{p.y_dtype} {path}", flush=True)
    y = out_bits(run(p, path), p.y_dtype)
    Y, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, sh.M, sh.N, sh.K, threads=8)
    return check(y, p.y_dtype, Y, B, f"{sh} {path}")


def test_tiny_config():
    p = workloads.make_problem(1)
    for path in _paths(p.x_dtype):
        _full(p, path)


@pytest.mark.parametrize("path", PATHS)
def test_attention_decode_config(path):
    _full(workloads.make_problem(2), path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape_id", [0, 1, 2, 3])   # M = 1 and 4, FFN up and down
def test_ffn_decode_config(shape_id, path):
    p = workloads.make_problem(3, shape_id)
    assert p.shape.M <= 4
    _full(p, path)


# (M, K, N): N not a multiple of 4; K not a multiple of 1024 (the last step's
# segments past K read zero activations); one 128-weight block; one quad per
# workgroup; several quads per wave (K <= 1024 with many rows); more rounds
# of workgroups (units per workgroup capped at 128); 6 staged blocks per
# thread (M = 4, K = 17408: 139 KB of activations in LDS)
RAGGED = [(1, 128, 1), (1, 128, 7), (2, 256, 9), (3, 640, 33), (4, 1152, 50), (1, 1920, 17),
          (2, 3200, 29), (3, 5248, 700), (4, 4096, 1021), (1, 17408, 5), (4, 17408, 5123),
          (1, 1024, 40003), (2, 512, 20000), (3, 5120, 34816), (1, 9216, 37), (4, 12288, 45),
          (1, 5120, 1), (2, 7168, 1030), (4, 128, 4097), (3, 17408, 2100), (1, 16384, 300)]


@pytest.mark.parametrize("M,K,N", RAGGED)
@pytest.mark.parametrize("xd,yd", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f16"), ("f16", "f16")])
def test_ragged_shapes(M, K, N, xd, yd):
    p = workloads.make_custom(M * 13 + K + N, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.02)
    for path in _paths(xd):
        _full(p, path)


# The fp4 kernel's own layout: workgroups of 1 to 17 quads (4-row groups;
# the count follows N), 512-weight steps split over up to 16 waves, 1 to 4
# steps per wave (K up to 32768, the images of one step staged at a time), a
# ragged last step (K off the multiple of 512: its blocks past K meet zero
# activations and their scales are dropped), N off the multiple of 4 and of
# the workgroup's rows, and one or many rounds of workgroups.
FP4_LAYOUT = [(1, 128, 1), (2, 640, 17), (3, 1152, 31), (4, 4224, 33), (1, 512, 15), (1, 8320, 70),
              (2, 16512, 48), (1, 24704, 40), (2, 32768, 33), (1, 2048, 8193), (4, 17408, 8195),
              (3, 12416, 8200), (4, 8192, 47), (4, 32768, 1021), (4, 5120, 17407), (1, 5120, 34813),
              (2, 20480, 5119)]


@pytest.mark.parametrize("M,K,N", FP4_LAYOUT)
@pytest.mark.parametrize("yd", ["bf16", "f32", "f16"])
def test_fp4_layout_shapes(M, K, N, yd):
    p = workloads.make_custom(M * 7 + K + N, M, K, N, x_dtype="bf16", y_dtype=yd, reserved_rate=0.02)
    _full(p, "gemv_fp4")


# More ragged fp4 shapes at M <= 2: K off the multiple of 512 and 1024 (the
# blocks of the last step past K meet zero activations, their scales are
# dropped), N odd and off the workgroup's rows, 1 to 4 steps per wave (K up
# to 32768).
FP4_MORE_RAGGED = [(1, 128, 1), (1, 640, 3), (2, 896, 5), (1, 1152, 21), (2, 5120, 5119), (1, 5120, 17409), (2, 17408, 77),
         (1, 16512, 33), (2, 24704, 41), (1, 32768, 10), (2, 1024, 4097), (1, 3200, 257)]


@pytest.mark.parametrize("M,K,N", FP4_MORE_RAGGED)
@pytest.mark.parametrize("yd", ["bf16", "f32"])
def test_fp4_more_ragged_shapes(M, K, N, yd):
    p = workloads.make_custom(M * 11 + K + N, M, K, N, x_dtype="bf16", y_dtype=yd, reserved_rate=0.02)
    _full(p, "gemv_fp4")


@pytest.mark.parametrize("M,K,N", [(1, 1024, 64), (1, 5120, 1100), (2, 2048, 24), (3, 2048, 40), (4, 10240, 16),
                                   (1, 17408, 12), (4, 17408, 77), (2, 640, 4500), (1, 1024, 40001)])
@pytest.mark.parametrize("xd", ["f16", "bf16"])
@pytest.mark.parametrize("yd", ["f32", "bf16", "f16"])
def test_exact_arithmetic_bit_exact(M, K, N, xd, yd):
    """Integer activations in [-8, 8], power-of-two scales: every product and
    partial sum is exact in fp32 in any order, so the output must equal the
    oracle's value rounded to the output type."""
    rng = np.random.default_rng(M * 1000 + K + N)
    xi = rng.integers(-8, 9, (M, K)).astype(np.float64)
    xbits = xi.astype(np.float16).view(np.uint16) if xd == "f16" else workloads.to_bf16_bits(xi)
    P = O().pack(workloads.draw_ternary(K + N + 5, N, K))
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, xd, P, sbits, M, N, K)
    x = bits_to_device(xbits, xd)
    w = torch.from_numpy(P).to(device())
    s = bits_to_device(sbits, "f16")
    want = O().round(Y, yd)
    for path in _paths(xd):
        y = torch.full((M, N), float("nan"), dtype=TORCH_DT[yd], device=device())
        tern.matmul_into(x, w, s, y, path=path)
        got = O().decode(out_bits(y, yd), yd)
        assert np.array_equal(got, want), (path, np.argwhere(got != want)[:5])


def _swap(P):
    out = P.copy()
    for sh in (0, 2, 4, 6):
        f = (P >> sh) & 3
        new = np.where(f == 1, 2, np.where(f == 2, 1, f)).astype(np.uint8)
        out = (out & ~np.uint8(3 << sh)) | (new << sh)
    return out


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_invariants(M, path):
    """Zero codes give 0, reserved codes act as 00, Y(2X) = 2Y and two runs
    agree, bit for bit.  Swapping 01 and 10 negates Y up to the matrix core's
    fp32 rounding: its sums are not rounded symmetrically in sign (measured on
    gfx950: one 4x4x4 MFMA gives D(-A, B, -C) != -D(A, B, C) in the last bit
    for about 30% of inputs with a wide exponent spread), so the negation is
    checked to 1e-6 of the bound sum |x s| instead of bit for bit."""
    p = workloads.make_custom(330 + M, M, 3072, 210, x_dtype="bf16", y_dtype="f32", probs=(0.3, 0.3, 0.3, 0.1))
    x, w, s = problem_to_device(p)

    def y_of(xx, ww, ss):
        return tern.matmul(xx, ww, ss, out_dtype=torch.float32, path=path).cpu().numpy()

    y = y_of(x, w, s)
    assert np.array_equal(y, y_of(x, w, s)), "not deterministic"
    assert not np.any(y_of(x, torch.zeros_like(w), s)), "all-zero codes must give exactly 0"
    assert not np.any(y_of(x, torch.full_like(w, 0xFF), s)), "all-reserved codes must give exactly 0"
    assert np.array_equal(y_of(x * 2, w, s), 2 * y)
    _, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, M, 210, 3072, threads=8)
    ys = y_of(x, torch.from_numpy(_swap(p.packed)).to(device()), s)
    assert np.all(np.abs(ys + y) <= 1e-6 * B), np.max(np.abs(ys + y) / B)


def test_fp4_split_wide_range_within_a_block():
    """Activations spanning 2^-30 .. 2^8 inside each 32-block (the two-term
    e4m3 split is exact only within 2^13 of the block maximum; the rest carry
    an error below 2^-21 of the maximum), with an all-zero and an all-tiny
    block: within the bound."""
    M, K, N = 2, 2048, 300
    rng = np.random.default_rng(5)
    mag = 2.0 ** rng.integers(-30, 9, (M, K))
    x = mag * rng.choice([-1.0, 1.0], (M, K)) * rng.uniform(1, 2, (M, K))
    x[0, 128:160] = 0.0
    x[1, 256:288] = 1e-30
    p = workloads.make_custom(41, M, K, N, x_dtype="bf16", y_dtype="f32")
    p.x = workloads.to_bf16_bits(x)
    _full(p, "gemv_fp4")


def test_fp4_refuses_fp16_activations():
    p = workloads.make_custom(4, 1, 1024, 8, x_dtype="f16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    with pytest.raises(tern.TernError) as err:
        tern.matmul(x, w, s, out_dtype=torch.float32, path="gemv_fp4")
    assert err.value.status == 6


@pytest.mark.parametrize("M,xd", [(1, "bf16"), (3, "f16"), (4, "bf16")])
def test_scales_near_fp16_max_and_negative(M, xd):
    """Every finite fp16 scale, half of them negative: the kernel never forms
    2*s (which overflows past 32752); the halving happens on the fp32 sum."""
    p = workloads.make_custom(910 + M, M, 2048, 98, x_dtype=xd, y_dtype="f32",
                              scale_lo=8192.0, scale_hi=65504.0, x_sigma=1e-3)
    p.scales = p.scales ^ np.where(np.arange(p.scales.size).reshape(p.scales.shape) % 2 == 1,
                                   np.uint16(0x8000), np.uint16(0))
    for path in _paths(xd):
        _full(p, path)


@pytest.mark.parametrize("M,K,N", [(1, 5120, 300), (4, 17408, 77), (2, 1024, 9000), (3, 640, 33)])
def test_int8_scales(M, K, N):
    rng = np.random.default_rng(M + K + N)
    p = workloads.make_custom(M * 17 + K + N, M, K, N, x_dtype="bf16", y_dtype="f32", reserved_rate=0.02)
    s = np.exp(rng.uniform(np.log(1e-4), np.log(1e1), (N, K // 128))) * np.where(rng.random((N, K // 128)) < .3, -1, 1)
    p.scales = s.astype(np.float16).view(np.uint16)
    q, r = O().quantize_scales(p.scales)
    Y, B = O().matmul_s8(p.x, "bf16", p.packed, q, r, M, N, K, threads=8)
    x, w, _ = problem_to_device(p)
    for path in PATHS:
        y = run_s8(x, w, torch.from_numpy(q).to(device()), torch.from_numpy(r).to(device()), M, N, "f32", path)
        check(out_bits(y, "f32"), "f32", Y, B, f"s8 {M}x{K}x{N} {path}")


def test_agrees_with_the_valu_decode_kernel():
    """Both decode kernels are within the bound of the oracle on the same
    inputs (they sum in different orders, so not bit-identical in general)."""
    for M in (1, 2, 4):
        p = workloads.make_custom(520 + M, M, 5120, 5120, x_dtype="bf16", y_dtype="f32")
        assert all(_full(p, path) <= 1 for path in ["gemv"] + PATHS)


@pytest.mark.parametrize("path,M,K", [("gemv_mfma", 4, 20480), ("gemv_fp4", 1, 33280)])
def test_refuses_shapes_beyond_its_layout(path, M, K):
    """The 4x4x4 kernel stages all activations of a workgroup (M = 4, K =
    20480: 160 KB, more than its LDS); the fp4 kernel takes at most 4 steps
    of 512 weights per wave over 16 waves (K <= 32768).  Beyond that the
    forced path is refused before anything runs."""
    p = workloads.make_custom(3, M, K, 8, x_dtype="bf16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    y = torch.full((M, 8), 5.0, dtype=torch.float32, device=device())
    with pytest.raises(tern.TernError) as err:
        tern.matmul_into(x, w, s, y, path=path)
    assert err.value.status == 6
    assert torch.all(y == 5.0).item()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,K,N", [(1, 5120, 5120), (4, 17408, 5120)])
def test_hip_graph_replays_match_eager(M, K, N, path):
    p = workloads.make_custom(710 + M, M, K, N, x_dtype="bf16", y_dtype="bf16")
    x, w, s = problem_to_device(p)
    eager = tern.matmul(x, w, s, out_dtype=torch.bfloat16, path=path).clone()
    y = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tern.matmul_into(x, w, s, y, path=path)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), rep
        tern.matmul(x, w, s, out_dtype=torch.bfloat16, path=path)
