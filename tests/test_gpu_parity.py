"""HIP path vs the CPU oracle, on the GPU.

Pack/unpack must be bit-exact.  Matmul outputs must satisfy
|Y_gpu - Y_oracle| <= 2e-3 * sum_k |x[m,k] * s[n,k/128]| + one ulp of the
output type at Y_oracle, elementwise; where the arithmetic is exact
(integer activations, power-of-two scales) the output must equal the
oracle's value rounded to the output type, bit for bit.  Every workload is
seeded and synthetic (see the workloads package).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import (TORCH_DT, bits_to_device, check, device, out_bits, problem_to_device,  # noqa: E402
                      run, sample_indices)

tern = pytest.importorskip("ternary_weight_matmul_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


O = oracle.default


# ---------------------------------------------------------------------------
# pack / unpack: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 4), (3, 12), (7, 36), (64, 1024), (5, 5120), (257, 1028)])
def test_pack_bit_exact(N, K):
    T = workloads.draw_ternary(N * 131 + K, N, K)
    T[0, 0] = 5 if K > 0 else 0           # an invalid value -> reserved code 11
    got = tern.pack(torch.from_numpy(T).to(device())).cpu().numpy()
    want = O().pack(T)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]


@pytest.mark.parametrize("N,K", [(1, 1024), (3, 12), (9, 132), (128, 5120), (2, 4)])
def test_unpack_bit_exact(N, K):
    rng = np.random.default_rng(N + K)
    P = rng.integers(0, 256, (N, K // 4), dtype=np.uint8)
    if P.size >= 256:
        P.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)   # every byte value
    got = tern.unpack(torch.from_numpy(P).to(device()), K).cpu().numpy()
    assert np.array_equal(got, O().unpack(P, N, K))


def test_device_copy_and_roundtrip():
    # the packed bytes on the device equal the host bytes; pack(unpack(P)) is P with 11 -> 00
    rng = np.random.default_rng(5)
    P = rng.integers(0, 256, (33, 80), dtype=np.uint8)
    dP = torch.from_numpy(P).to(device())
    assert np.array_equal(dP.cpu().numpy(), P)
    back = tern.pack(tern.unpack(dP, 320)).cpu().numpy()
    assert np.array_equal(back, O().pack(O().unpack(P, 33, 320)))


# ---------------------------------------------------------------------------
# matmul on the configured workloads
# ---------------------------------------------------------------------------

def _full(p, path):
    sh = p.shape
    y = out_bits(run(p, path), p.y_dtype)
    Y, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, sh.M, sh.N, sh.K, threads=8)
    return check(y, p.y_dtype, Y, B, f"{sh} {path}")


def _sampled(p, path, count=3000, seed=0):
    sh = p.shape
    y = out_bits(run(p, path), p.y_dtype)
    ms, ns = sample_indices(sh.M, sh.N, count, seed)
    Y, B = O().matmul_at(p.x, p.x_dtype, p.packed, p.scales, sh.M, sh.N, sh.K, ms, ns)
    return check(y[ms, ns], p.y_dtype, Y, B, f"{sh} {path}")


@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_tiny_config(path):
    _full(workloads.make_problem(1), path)


@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_attention_decode_config(path):
    _full(workloads.make_problem(2), path)


@pytest.mark.parametrize("shape_id", range(6))
def test_ffn_decode_config(shape_id):
    p = workloads.make_problem(3, shape_id)
    if p.shape.M == 1:
        _full(p, "auto")
    else:
        _sampled(p, "auto", 2000, shape_id)


@pytest.mark.parametrize("shape_id", range(4))
def test_prefill_config(shape_id):
    _sampled(workloads.make_problem(4, shape_id), "auto", 3000, shape_id)


@pytest.mark.parametrize("shape_id", range(3))
def test_embedding_config(shape_id):
    _sampled(workloads.make_problem(5, shape_id), "auto", 3000, shape_id)


@pytest.mark.parametrize("shape_id", [0, 3, 4, 6, 333])
def test_sweep_matrices(shape_id):
    _full(workloads.make_problem(6, shape_id), "auto")


@pytest.mark.parametrize("K,N", [(5120, 3 * 5120), (5120, 2 * 17408)])
def test_sweep_fused_layout_matrices(K, N):
    """The merged projections of the fused-layout decode sweep (q|k|v and
    gate|up stored as one matrix), with the sweep's code and scale
    distributions, compared element by element."""
    _full(workloads.make_problem(6, 0, shape=workloads.Shape(1, K, N, "fused")), "auto")


# ---------------------------------------------------------------------------
# shapes off the tile grid, dtypes, paths
# ---------------------------------------------------------------------------

# (M <= 4 with K > 8192: decode workgroups of 12 rows, two activation rows per
# decode for even M)
RAGGED = [(1, 128, 1), (1, 640, 33), (2, 1152, 50), (3, 384, 17), (4, 3200, 29), (1, 17408, 5),
          (2, 9216, 37), (3, 17408, 21), (4, 12288, 45),
          (5, 256, 3), (17, 640, 100), (130, 384, 257), (129, 1152, 300), (64, 128, 512),
          # small-M MFMA with 4 or 8 staged rows (K <= 8192) and with 16 (K > 8192)
          (6, 4096, 33), (8, 1152, 70), (8, 9216, 40), (16, 8192, 19)]


@pytest.mark.parametrize("M,K,N", RAGGED)
@pytest.mark.parametrize("xd,yd", [("f16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
def test_ragged_shapes(M, K, N, xd, yd):
    p = workloads.make_custom(M * 7 + K + N, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.02)
    paths = ["auto", "mfma"] + (["gemv"] if M <= tern.GEMV_MAX_M else [])
    for path in paths:
        _full(p, path)


# M <= 4, N <= 5120, K <= 5120 (M = 1) or 8192: the short-step decode kernel
# (4 JR rows per workgroup, JR = ceil(N / 1024), 512-weight steps); each JR,
# K off the 512 grid, ragged last workgroups, the size limits and the
# shapes just past them (the 8-row or the MFMA kernel)
SHORT = [(128, 1), (640, 33), (1152, 1023), (4992, 1025), (2048, 2100), (3968, 3071), (5120, 4097),
         (5120, 5120), (384, 5119), (5248, 700), (5120, 5121),
         # from M = 2 up to K = 8192 (16 waves; M = 4 past K = 7168 needs more than 64 KB of LDS)
         (6272, 3000), (8192, 5120), (7296, 129), (8320, 300),
         # M = 2 on layers of 12288 rows or more (several rounds of workgroups)
         (5120, 12289), (2048, 20000), (8192, 12288)]


@pytest.mark.parametrize("K,N", SHORT)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("xd,yd", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f16")])
def test_short_step_decode(M, K, N, xd, yd):
    p = workloads.make_custom(K * 3 + N + M, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.02)
    for path in ("auto", "gemv"):
        _full(p, path)


@pytest.mark.parametrize("K,N,xd,yd", [(5120, 9001, "bf16", "bf16"), (17408, 5121, "f16", "f32"),
                                       (5120, 17408, "bf16", "f32"), (1024, 60003, "f16", "f16")])
def test_decode_rows_beyond_one_round(K, N, xd, yd):
    """M = 1 with more 8-row workgroups than are resident at once (several
    rounds), ragged last workgroup included."""
    p = workloads.make_custom(K + N, 1, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.01)
    for path in ("auto", "gemv"):
        _full(p, path)


@pytest.mark.parametrize("M,K,N,xd,yd", [(1, 36864, 70, "bf16", "bf16"), (2, 40960, 45, "f16", "f32"),
                                         (1, 65536, 9, "f16", "f16")])
def test_decode_beyond_gemv_reach(M, K, N, xd, yd):
    """K too long for the decode kernel's register budget (more than two
    1024-weight steps per wave at M = 1, more than four at M = 2): the
    automatic choice takes the MFMA kernel, and asking for the decode kernel
    is refused before anything is launched."""
    p = workloads.make_custom(M + K + N, M, K, N, x_dtype=xd, y_dtype=yd, reserved_rate=0.01)
    _full(p, "auto")
    _full(p, "mfma")
    with pytest.raises(tern.TernError) as err:
        run(p, "gemv")
    assert err.value.status == 6   # TERN_ERR_UNSUPPORTED


def test_outliers_and_wide_scales():
    # activations with x20 outliers, scales spread over two decades
    p = workloads.make_custom(77, 8, 1024, 96, x_dtype="f16", y_dtype="f32", scale_lo=1e-3, scale_hi=4.0)
    X = p.x.view(np.float16).astype(np.float64)
    X[:, ::37] *= 20
    p.x = X.astype(np.float16).view(np.uint16)
    for path in ("mfma",):
        _full(p, path)
    q = workloads.make_custom(78, 2, 1024, 96, x_dtype="bf16", y_dtype="bf16", scale_lo=1e-3, scale_hi=4.0)
    for path in ("gemv", "mfma"):
        _full(q, path)


@pytest.mark.parametrize("M,path", [(1, "gemv"), (3, "gemv"), (8, "mfma"), (40, "mfma"), (200, "mfma"),
                                    (300, "auto")])
@pytest.mark.parametrize("xd", ["f16", "bf16"])
def test_scales_near_fp16_max_and_negative(M, path, xd):
    """Scales up to the largest fp16 (65504), half of them negative.

    t*s is finite for every finite fp16 scale, so no kernel may form an
    operand that overflows (2*s does, for |s| > 32752)."""
    p = workloads.make_custom(900 + M, M, 1024, 96, x_dtype=xd, y_dtype="f32",
                              scale_lo=8192.0, scale_hi=65504.0, x_sigma=1e-3)
    p.scales = p.scales ^ np.where(np.arange(p.scales.size).reshape(p.scales.shape) % 2 == 1,
                                   np.uint16(0x8000), np.uint16(0))
    _full(p, path)


# ---------------------------------------------------------------------------
# exact arithmetic: bit-exact against the oracle rounded to the output type
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(1, 1024, 64), (3, 2048, 40), (40, 1024, 80), (1, 4096, 16), (200, 1024, 80),
                                   (1, 5120, 1100), (1, 640, 4500), (2, 5120, 2100),
                                   (2, 2048, 24), (2, 9216, 24), (4, 10240, 16), (1, 17408, 12), (8, 3072, 48),
                                   (16, 2048, 40)])
@pytest.mark.parametrize("xd", ["f16", "bf16"])
@pytest.mark.parametrize("yd", ["f32", "bf16", "f16"])
def test_exact_arithmetic_bit_exact(M, K, N, xd, yd):
    rng = np.random.default_rng(M * 1000 + K + N)
    xi = rng.integers(-8, 9, (M, K)).astype(np.float64)
    xbits = (xi.astype(np.float16).view(np.uint16) if xd == "f16"
             else workloads.to_bf16_bits(xi))
    T = workloads.draw_ternary(K + N, N, K)
    P = O().pack(T)
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, xd, P, sbits, M, N, K)
    want = O().round(Y, yd)
    x = bits_to_device(xbits, xd)
    w = torch.from_numpy(P).to(device())
    s = bits_to_device(sbits, "f16")
    for path in ["mfma"] + (["gemv"] if M <= tern.GEMV_MAX_M else []):
        y = tern.matmul(x, w, s, out_dtype=TORCH_DT[yd], path=path)
        got = O().decode(out_bits(y, yd), yd)
        assert np.array_equal(got, want), (path, np.argwhere(got != want)[:5])


@pytest.mark.parametrize("M,K,N,yd", [(2000, 256, 6000, "f16"), (1999, 384, 6001, "f32"), (1000, 128, 17000, "f32"),
                                      (3000, 384, 1100, "f16"), (200, 512, 3000, "f32")])
def test_large_tiles_ragged(M, K, N, yd):
    """Shapes that take the 256 x 256 tiles (the first two), the 192 x 256
    tiles (the third), 128 x 128 tiles with two K groups (the fourth) and
    128 x 64 tiles with two K groups (the last), with ragged row and column
    tails, compared element by element."""
    p = workloads.make_custom(M + N, M, K, N, x_dtype="f16", y_dtype=yd, reserved_rate=0.02)
    _full(p, "auto")


@pytest.mark.parametrize("M,K,N", [(2000, 256, 6000), (3000, 384, 1100)])
def test_large_tiles_exact_bit_exact(M, K, N):
    """Exact arithmetic on the 256 x 256 tiles and on the 128 x 128 tiles with
    two K groups: bit-identical to the oracle."""
    rng = np.random.default_rng(4242 + M)
    xbits = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    P = O().pack(workloads.draw_ternary(77, N, K))
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, "f16", P, sbits, M, N, K, threads=8)
    y = tern.matmul(bits_to_device(xbits, "f16"), torch.from_numpy(P).to(device()),
                    bits_to_device(sbits, "f16"), out_dtype=torch.float32)
    got = O().decode(out_bits(y, "f32"), "f32")
    assert np.array_equal(got, O().round(Y, "f32"))


# The cost model sends M=320, 1024 -> 17408 to the 192 x 256 tiles (136 of
# them; 2 x 68 against 136 tiles of 256 x 256 and 816 of 128 x 64) and M=256,
# 1024 -> 17408 to the plain 128 x 64 tiles with one K group (544 tiles: more
# than the CUs, so no K split; 272 tiles of 128 x 128).  K = 1024 is 16 steps
# of 64, so the steady-state loop that alternates the two register sets of
# staged loads runs many times in both.
FULL_K_TILES = [(320, 1024, 17408), (256, 1024, 17408)]


@pytest.mark.parametrize("M,K,N", FULL_K_TILES)
def test_large_tiles_full_k(M, K, N):
    """Every output of the 192 x 256 and the one-group 128 x 64 tile kernels at
    16 K steps, against the oracle (bf16 output: the rounding epilogue too)."""
    p = workloads.make_custom(M + N + K, M, K, N, x_dtype="f16", y_dtype="bf16", reserved_rate=0.02)
    _full(p, "auto")


@pytest.mark.parametrize("M,K,N", FULL_K_TILES)
def test_large_tiles_full_k_exact_bit_exact(M, K, N):
    """Exact arithmetic (integer activations in [-8, 8], power-of-two scales)
    on the same two tile kernels: bit-identical to the oracle."""
    rng = np.random.default_rng(99 + M)
    xbits = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    P = O().pack(workloads.draw_ternary(78, N, K))
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, "f16", P, sbits, M, N, K, threads=8)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=device())
    tern.matmul_into(bits_to_device(xbits, "f16"), torch.from_numpy(P).to(device()), bits_to_device(sbits, "f16"), y)
    got = O().decode(out_bits(y, "f32"), "f32")
    assert np.array_equal(got, O().round(Y, "f32"))


# ---------------------------------------------------------------------------
# invariants of the method, exact on the GPU
# ---------------------------------------------------------------------------

def _swap(P):
    out = P.copy()
    for s in (0, 2, 4, 6):
        f = (P >> s) & 3
        new = np.where(f == 1, 2, np.where(f == 2, 1, f)).astype(np.uint8)
        out = (out & ~np.uint8(3 << s)) | (new << s)
    return out


def _reserved_to_zero(P):
    out = P.copy()
    for s in (0, 2, 4, 6):
        out = np.where(((P >> s) & 3) == 3, out & ~np.uint8(3 << s), out)
    return out


@pytest.mark.parametrize("M,path", [(1, "gemv"), (4, "gemv"), (1, "mfma"), (4, "mfma"), (8, "mfma"), (96, "mfma")])
def test_invariants_exact(M, path):
    p = workloads.make_custom(300 + M, M, 2048, 200, x_dtype="bf16", y_dtype="f32",
                              probs=(0.3, 0.3, 0.3, 0.1))
    x, w, s = problem_to_device(p)

    def y_of(xx, ww, ss):
        return tern.matmul(xx, ww, ss, out_dtype=torch.float32, path=path).cpu().numpy()

    y = y_of(x, w, s)
    assert np.array_equal(y, y_of(x, w, s)), "not deterministic"
    zero = torch.zeros_like(w)
    assert not np.any(y_of(x, zero, s)), "all-zero codes must give exactly 0"
    ones = torch.full_like(w, 0xFF)
    assert not np.any(y_of(x, ones, s)), "all-reserved codes must give exactly 0"
    ys = y_of(x, torch.from_numpy(_swap(p.packed)).to(device()), s)
    assert np.array_equal(ys, -y), "swapping 01 and 10 must negate Y exactly"
    yr = y_of(x, torch.from_numpy(_reserved_to_zero(p.packed)).to(device()), s)
    assert np.array_equal(yr, y), "code 11 must act as 00"
    y2 = y_of(x * 2, w, s)
    assert np.array_equal(y2, 2 * y), "Y(2X) must be 2Y"


def test_paths_agree_within_tolerance():
    for M in (1, 2, 4):
        p = workloads.make_custom(500 + M, M, 5120, 512, x_dtype="bf16", y_dtype="f32")
        a = _full(p, "gemv")
        b = _full(p, "mfma")
        assert a <= 1 and b <= 1


# ---------------------------------------------------------------------------
# edge cases of the boundary
# ---------------------------------------------------------------------------

def test_k_zero_writes_zeros():
    x = torch.empty((3, 0), dtype=torch.float16, device=device())
    w = torch.empty((5, 0), dtype=torch.uint8, device=device())
    s = torch.empty((5, 0), dtype=torch.float16, device=device())
    y = torch.full((3, 5), 7.0, dtype=torch.float32, device=device())
    tern.matmul_into(x, w, s, y)
    assert not torch.any(y).item()


def test_empty_m_and_n():
    x = torch.empty((0, 256), dtype=torch.float16, device=device())
    w = torch.zeros((4, 64), dtype=torch.uint8, device=device())
    s = torch.ones((4, 2), dtype=torch.float16, device=device())
    assert tern.matmul(x, w, s).shape == (0, 4)
    x1 = torch.ones((2, 256), dtype=torch.float16, device=device())
    w0 = torch.zeros((0, 64), dtype=torch.uint8, device=device())
    s0 = torch.zeros((0, 2), dtype=torch.float16, device=device())
    assert tern.matmul(x1, w0, s0).shape == (2, 0)


def test_rejects_misaligned_and_leaves_output_untouched():
    base = torch.ones((1, 257), dtype=torch.float16, device=device())
    x = base[:, 1:]                        # 2-byte offset: not 16-byte aligned
    w = torch.zeros((8, 64), dtype=torch.uint8, device=device())
    s = torch.ones((8, 2), dtype=torch.float16, device=device())
    y = torch.full((1, 8), 3.0, dtype=torch.float32, device=device())
    with pytest.raises(tern.TernError) as e:
        tern.matmul_into(x, w, s, y)
    assert e.value.status == 5
    assert torch.all(y == 3.0).item()


def test_multiple_calls_on_a_side_stream():
    p = workloads.make_custom(900, 2, 1024, 300, x_dtype="f16", y_dtype="f32")
    x, w, s = problem_to_device(p)
    ref = tern.matmul(x, w, s, out_dtype=torch.float32).cpu()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        outs = [tern.matmul(x, w, s, out_dtype=torch.float32) for _ in range(4)]
    st.synchronize()
    for o in outs:
        assert torch.equal(o.cpu(), ref)


@pytest.mark.parametrize("M,K,N,xd,yd", [(1, 5120, 640, "bf16", "bf16"), (2, 17408, 96, "bf16", "f32"),
                                         (300, 1024, 512, "f16", "f16"), (1, 5120, 17408, "bf16", "bf16")])
def test_hip_graph_replays_match_eager(M, K, N, xd, yd):
    """Captured launches replay to the eager result, every time."""
    p = workloads.make_custom(700 + M, M, K, N, x_dtype=xd, y_dtype=yd)
    x, w, s = problem_to_device(p)
    eager = tern.matmul(x, w, s, out_dtype=TORCH_DT[yd]).clone()
    y = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tern.matmul_into(x, w, s, y)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if yd != "f32" else torch.int32),
                           eager.view(torch.int16 if yd != "f32" else torch.int32)), rep
        tern.matmul(x, w, s, out_dtype=TORCH_DT[yd])   # eager work between replays
