"""The decode kernel for batches of up to 16 rows (TERN_PATH_GEMV_B16: +-2 / 0
weight operands of v_mfma_f32_16x16x32 against activation fragments held in
registers) against the CPU oracle, on the GPU.

Outputs must meet |Y_gpu - Y_oracle| <= 2e-3 * sum_k |x*s| + one ulp of the
output type, elementwise, and equal the oracle's value rounded to the output
type bit for bit where the arithmetic is exact.  The cases walk the kernel's
layout: 1 to 16 activation rows (rows past M read row M - 1 and are never
stored), workgroups of 1 to 4 column blocks of 16 rows (N off the multiple
of 16 and of the workgroup's rows), 512-weight steps split over 1 to 12
waves with 1 to many steps per wave (K up to 34816), a ragged last step (K
off the multiple of 512: its groups past K get a zero scale), one group,
and every dtype pair.
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

PATH = "gemv_b16"
O = oracle.default


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _full(p, path=PATH):
    sh = p.shape
    print(f"case {sh.M}x{sh.K}x{sh.N} {p.x_dtype}->{p.y_dtype} {path}", flush=True)
    y = out_bits(run(p, path), p.y_dtype)
    Y, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, sh.M, sh.N, sh.K, threads=8)
    return check(y, p.y_dtype, Y, B, f"{sh} {path}")


@pytest.mark.parametrize("shape_id", [0, 1, 2, 3, 4, 5])   # M = 1, 4, 16; FFN up and down
def test_ffn_decode_config(shape_id):
    _full(workloads.make_problem(3, shape_id))


def test_attention_decode_shape_at_16_rows():
    p = workloads.make_custom(2016, 16, 5120, 5120, x_dtype="bf16", y_dtype="bf16")
    _full(p)


# (M, K, N): every M from 1 to 16 somewhere; one group (K = 128); K off the
# multiple of 512 (ragged last step: 640, 1152, 3200, 5248, 16512); K of
# 1 to 68 steps (waves taking 1, 2, 3 or more steps); N of one row, off the
# multiple of 16, off the workgroup's rows, and large (many workgroups per CU)
LAYOUT = [(1, 128, 1), (2, 128, 17), (3, 640, 33), (4, 1152, 50), (5, 512, 16), (6, 1024, 31),
          (7, 3200, 300), (8, 5120, 17408), (9, 5248, 1021), (10, 6144, 48), (11, 16512, 95),
          (12, 17408, 5123), (13, 34816, 130), (14, 2048, 8193), (15, 8192, 257), (16, 128, 4097),
          (16, 640, 63), (16, 24576, 700), (16, 12288, 1), (8, 17408, 5120), (5, 5120, 17407)]


@pytest.mark.parametrize("M,K,N", LAYOUT)
@pytest.mark.parametrize("xd,yd", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f16"), ("f16", "f16")])
def test_layout_shapes(M, K, N, xd, yd):
    p = workloads.make_custom(M * 19 + K + N, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.02)
    _full(p)


@pytest.mark.parametrize("M,K,N", [(16, 1024, 64), (5, 5120, 1100), (8, 2048, 24), (16, 17408, 77),
                                   (12, 640, 4500), (1, 1024, 1001), (16, 34816, 40)])
@pytest.mark.parametrize("xd", ["f16", "bf16"])
@pytest.mark.parametrize("yd", ["f32", "bf16", "f16"])
def test_exact_arithmetic_bit_exact(M, K, N, xd, yd):
    """Integer activations in [-8, 8], power-of-two scales: every product and
    partial sum is exact in fp32 in any order, so the output must equal the
    oracle's value rounded to the output type."""
    rng = np.random.default_rng(M * 1000 + K + N)
    xi = rng.integers(-8, 9, (M, K)).astype(np.float64)
    xbits = xi.astype(np.float16).view(np.uint16) if xd == "f16" else workloads.to_bf16_bits(xi)
    P = O().pack(workloads.draw_ternary(K + N + 7, N, K))
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, xd, P, sbits, M, N, K)
    x = bits_to_device(xbits, xd)
    w = torch.from_numpy(P).to(device())
    s = bits_to_device(sbits, "f16")
    want = O().round(Y, yd)
    y = torch.full((M, N), float("nan"), dtype=TORCH_DT[yd], device=device())
    tern.matmul_into(x, w, s, y, path=PATH)
    got = O().decode(out_bits(y, yd), yd)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def _swap(P):
    out = P.copy()
    for sh in (0, 2, 4, 6):
        f = (P >> sh) & 3
        new = np.where(f == 1, 2, np.where(f == 2, 1, f)).astype(np.uint8)
        out = (out & ~np.uint8(3 << sh)) | (new << sh)
    return out


@pytest.mark.parametrize("M", [5, 8, 16])
def test_invariants(M):
    """Zero codes give 0, reserved codes act as 00, Y(2X) = 2Y and two runs
    agree, bit for bit; swapping 01 and 10 negates Y up to the matrix core's
    fp32 rounding (checked to 1e-6 of the bound sum |x s|)."""
    p = workloads.make_custom(430 + M, M, 3072, 210, x_dtype="bf16", y_dtype="f32", probs=(0.3, 0.3, 0.3, 0.1))
    x, w, s = problem_to_device(p)

    def y_of(xx, ww, ss):
        return tern.matmul(xx, ww, ss, out_dtype=torch.float32, path=PATH).cpu().numpy()

    y = y_of(x, w, s)
    assert np.array_equal(y, y_of(x, w, s)), "not deterministic"
    assert not np.any(y_of(x, torch.zeros_like(w), s)), "all-zero codes must give exactly 0"
    assert not np.any(y_of(x, torch.full_like(w, 0xFF), s)), "all-reserved codes must give exactly 0"
    assert np.array_equal(y_of(x * 2, w, s), 2 * y)
    _, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, M, 210, 3072, threads=8)
    ys = y_of(x, torch.from_numpy(_swap(p.packed)).to(device()), s)
    assert np.all(np.abs(ys + y) <= 1e-6 * B), np.max(np.abs(ys + y) / B)


def test_rows_do_not_mix():
    """Row m of Y depends on row m of X alone: the kernel's rows past M read
    row M - 1 again, and each activation row feeds one MFMA row."""
    M, K, N = 11, 2048, 100
    p = workloads.make_custom(77, M, K, N, x_dtype="bf16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    y = tern.matmul(x, w, s, out_dtype=torch.float32, path=PATH)
    for m in (0, 5, 10):
        ym = tern.matmul(x[m:m + 1].contiguous(), w, s, out_dtype=torch.float32, path=PATH)
        assert torch.equal(y[m:m + 1], ym), m


@pytest.mark.parametrize("M,xd", [(5, "bf16"), (16, "f16")])
def test_scales_near_fp16_max_and_negative(M, xd):
    """Every finite fp16 scale, half of them negative: the kernel never forms
    2*s; the halving happens on the fp32 sum."""
    p = workloads.make_custom(990 + M, M, 2048, 98, x_dtype=xd, y_dtype="f32",
                              scale_lo=8192.0, scale_hi=65504.0, x_sigma=1e-3)
    p.scales = p.scales ^ np.where(np.arange(p.scales.size).reshape(p.scales.shape) % 2 == 1,
                                   np.uint16(0x8000), np.uint16(0))
    _full(p)


@pytest.mark.parametrize("M,K,N", [(16, 5120, 300), (8, 17408, 77), (5, 1024, 9000), (13, 640, 33)])
def test_int8_scales(M, K, N):
    rng = np.random.default_rng(M + K + N)
    p = workloads.make_custom(M * 23 + K + N, M, K, N, x_dtype="bf16", y_dtype="f32", reserved_rate=0.02)
    s = np.exp(rng.uniform(np.log(1e-4), np.log(1e1), (N, K // 128))) * np.where(rng.random((N, K // 128)) < .3, -1, 1)
    p.scales = s.astype(np.float16).view(np.uint16)
    q, r = O().quantize_scales(p.scales)
    Y, B = O().matmul_s8(p.x, "bf16", p.packed, q, r, M, N, K, threads=8)
    x, w, _ = problem_to_device(p)
    y = run_s8(x, w, torch.from_numpy(q).to(device()), torch.from_numpy(r).to(device()), M, N, "f32", PATH)
    check(out_bits(y, "f32"), "f32", Y, B, f"s8 {M}x{K}x{N} {PATH}")


def test_longest_k():
    """K = 2^20, the largest K the kernel takes: 2048 steps over 12 waves (171
    each), the code and activation buffer offsets near the top of their
    32-bit range; two column blocks, the second with 4 rows."""
    _full(workloads.make_custom(4242, 16, 1 << 20, 20, x_dtype="bf16", y_dtype="f32"))


@pytest.mark.parametrize("M,K", [(17, 1024), (4, (1 << 20) + 128)])
def test_refuses_shapes_beyond_its_layout(M, K):
    """At most 16 activation rows (one MFMA tile) and K <= 2^20 (32-bit buffer
    offsets); beyond that the forced path is refused before anything runs."""
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=device())
    w = torch.zeros((8, K // 4), dtype=torch.uint8, device=device())
    s = torch.zeros((8, K // 128), dtype=torch.float16, device=device())
    y = torch.full((M, 8), 5.0, dtype=torch.float32, device=device())
    with pytest.raises(tern.TernError) as err:
        tern.matmul_into(x, w, s, y, path=PATH)
    assert err.value.status == 6
    assert torch.all(y == 5.0).item()


@pytest.mark.parametrize("M,K,N", [(16, 5120, 17408), (8, 17408, 5120)])
def test_hip_graph_replays_match_eager(M, K, N):
    p = workloads.make_custom(810 + M, M, K, N, x_dtype="bf16", y_dtype="bf16")
    x, w, s = problem_to_device(p)
    eager = tern.matmul(x, w, s, out_dtype=torch.bfloat16, path=PATH).clone()
    y = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tern.matmul_into(x, w, s, y, path=PATH)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), rep
        tern.matmul(x, w, s, out_dtype=torch.bfloat16, path=PATH)
