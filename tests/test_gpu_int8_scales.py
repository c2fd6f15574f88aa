"""Int8 block scales (the pages' suggested INT8 scale compression), on the GPU.

The codes must equal the oracle's bit for bit (same fp32 decisions); the
product must meet the tern_matmul bound with the effective scales q * r.
Inputs of the oracle come from the seeded generators and the oracle's own
quantiser, never from the device.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import (TORCH_DT, bits_to_device, check, device, out_bits, problem_to_device,  # noqa: E402
                      run_s8, sample_indices)

tern = pytest.importorskip("ternary_weight_matmul_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


O = oracle.default


def _scales(seed, N, G, lo=1e-3, hi=1e-1, negative=True, zero_rows=()):
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), (N, G)))
    if negative:
        s *= np.where(rng.random((N, G)) < 0.3, -1.0, 1.0)
    for n in zero_rows:
        s[n] = 0.0
    return s.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("N,G", [(1, 1), (5, 40), (64, 136), (300, 8), (7, 1000)])
def test_quantize_bit_exact(N, G):
    sb = _scales(N * 7 + G, N, G, lo=1e-5, hi=60000.0, zero_rows=(0,) if N > 1 else ())
    q, r = tern.quantize_scales(bits_to_device(sb, "f16"))
    torch.cuda.synchronize()
    wq, wr = O().quantize_scales(sb)
    assert np.array_equal(q.cpu().numpy(), wq), np.argwhere(q.cpu().numpy() != wq)[:5]
    assert np.array_equal(r.cpu().numpy().view(np.uint32), wr.view(np.uint32))


def _run_s8(p, q, r, path):
    x, w, _ = problem_to_device(p)
    y = run_s8(x, w, torch.from_numpy(q).to(device()), torch.from_numpy(r).to(device()),
               p.shape.M, p.shape.N, p.y_dtype, path)
    return out_bits(y, p.y_dtype)


RAGGED = [(1, 128, 1), (1, 640, 33), (3, 1152, 50), (4, 3200, 29), (1, 17408, 5), (5, 256, 3),
          (17, 640, 100), (130, 384, 257), (64, 128, 512), (257, 640, 300), (1000, 256, 70),
          # small-M MFMA with 8 and 16 staged rows; with fp16 X, 128 x 128 tiles of two K groups
          (8, 4096, 200), (16, 2048, 300), (3000, 384, 1100),
          # M <= 2, K and N <= 5120: the short-step decode kernel at each row count
          (1, 4992, 1025), (1, 2048, 2100), (1, 5120, 3071), (1, 1152, 5120), (2, 5120, 4097), (2, 640, 33),
          # M = 4 with one wave per workgroup: 80 outputs for 64 threads
          (4, 384, 4500), (3, 5120, 2000), (4, 8192, 1500), (2, 7296, 700),
          # M = 2 on layers of 12288 rows or more (several rounds of short-step workgroups)
          (2, 5120, 12289), (2, 8192, 17408)]


@pytest.mark.parametrize("M,K,N", RAGGED)
@pytest.mark.parametrize("xd,yd", [("bf16", "bf16"), ("f16", "f32")])
def test_matmul_s8_ragged(M, K, N, xd, yd):
    p = workloads.make_custom(M * 11 + K + N, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.02)
    p.scales = _scales(M + K + N, N, K // 128, zero_rows=(N - 1,) if N > 2 else ())
    q, r = O().quantize_scales(p.scales)
    Y, B = O().matmul_s8(p.x, xd, p.packed, q, r, M, N, K, threads=8)
    for path in ["auto", "mfma"] + (["gemv", "gemv_mfma"] if M <= tern.GEMV_MAX_M else []):
        check(_run_s8(p, q, r, path), yd, Y, B, f"{M}x{K}x{N} {path}")


@pytest.mark.parametrize("cfg,shape_id", [(2, 0), (3, 0), (3, 1), (3, 2), (3, 5), (4, 0)])
def test_matmul_s8_workloads(cfg, shape_id):
    p = workloads.make_problem(cfg, shape_id)
    sh = p.shape
    q, r = O().quantize_scales(p.scales)
    y = _run_s8(p, q, r, "auto")
    ms, ns = sample_indices(sh.M, sh.N, 2000, shape_id)
    Y = np.empty(len(ms))
    B = np.empty(len(ms))
    # the oracle's column routine over the sampled columns, one row at a time
    for i, (m, n) in enumerate(zip(ms, ns)):
        Yc, Bc = O().matmul_s8(p.x[m:m + 1], p.x_dtype, p.packed[n:n + 1], q[n:n + 1], r[n:n + 1],
                               1, 1, sh.K)
        Y[i], B[i] = Yc[0, 0], Bc[0, 0]
    check(y[ms, ns], p.y_dtype, Y, B, f"cfg{cfg}/{shape_id}")


@pytest.mark.parametrize("M,K,N,xd", [(3, 2048, 72, "bf16"), (200, 1024, 80, "f16"), (3, 2048, 72, "f16"),
                                      (1, 5120, 4500, "bf16"), (1, 640, 33, "f16"), (2, 3072, 1500, "bf16")])
def test_matmul_s8_exact_bit_exact(M, K, N, xd):
    """Integer activations, power-of-two row factors: every product and sum is
    exact in fp32, so the output equals the oracle rounded, bit for bit.
    (M=200 with fp16 activations takes the large-tile kernel.)"""
    rng = np.random.default_rng(99 + M)
    xi = rng.integers(-8, 9, (M, K)).astype(np.float64)
    xbits = workloads.to_bf16_bits(xi) if xd == "bf16" else xi.astype(np.float16).view(np.uint16)
    P = O().pack(workloads.draw_ternary(5, N, K))
    q = rng.integers(-127, 128, (N, K // 128)).astype(np.int8)
    r = (2.0 ** rng.integers(-12, -6, N)).astype(np.float32)
    Y, _ = O().matmul_s8(xbits, xd, P, q, r, M, N, K)
    paths = (("gemv", "f32"), ("mfma", "f32"), ("gemv", "bf16"), ("mfma", "bf16"), ("gemv_mfma", "f32"),
             ("gemv_mfma", "bf16"))
    for path, yd in paths if M <= tern.GEMV_MAX_M else [pp for pp in paths if pp[0] == "mfma"]:
        y = run_s8(bits_to_device(xbits, xd), torch.from_numpy(P).to(device()),
                   torch.from_numpy(q).to(device()), torch.from_numpy(r).to(device()), M, N, yd, path)
        got = O().decode(out_bits(y, yd), yd)
        assert np.array_equal(got, O().round(Y, yd)), (path, yd)


def test_quantized_scales_feed_the_product():
    """Device quantiser -> device product equals oracle quantiser -> oracle product."""
    p = workloads.make_custom(123, 2, 5120, 300, x_dtype="bf16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    dq, dr = tern.quantize_scales(s)
    y = run_s8(x, w, dq, dr, 2, 300, "f32")
    q, r = O().quantize_scales(p.scales)
    Y, B = O().matmul_s8(p.x, "bf16", p.packed, q, r, 2, 300, 5120, threads=8)
    check(out_bits(y, "f32"), "f32", Y, B, "quantised chain")
