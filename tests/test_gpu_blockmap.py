"""Zero-block skipping (the pages' first proposed extension), on the GPU.

The block map must equal the oracle's bit for bit.  The skipping product must
meet the tern_matmul bound against the oracle (skipping a block whose weights
are all zero changes nothing in the oracle's definition).  With every block
marked it runs the dense kernel's arithmetic in the dense order, so it must
match the dense decode kernel bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads  # noqa: E402
from gpu_util import TORCH_DT, bits_to_device, check, device, out_bits  # noqa: E402

tern = pytest.importorskip("ternary_weight_matmul_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


O = oracle.default


def _sparse_problem(seed, M, K, N, rate, xd="bf16", yd="f32", probs=(0.4, 0.3, 0.3, 0.0)):
    p = workloads.make_custom(seed, M, K, N, x_dtype=xd, y_dtype=yd, probs=probs)
    rng = workloads.rng_for(101, 0, seed)
    p.packed = workloads.draw_block_sparse_packed(rng, N, K, rate, probs)
    return p


def _dev(p):
    return (bits_to_device(p.x, p.x_dtype), torch.from_numpy(p.packed).to(device()),
            bits_to_device(p.scales, "f16"))


def _map_bits(m):
    return m.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("N,K,rate", [(1, 128, 0.0), (3, 128 * 40, 0.5), (17, 128 * 33, 0.9),
                                      (64, 5120, 0.5), (5, 17408, 0.3), (9, 128 * 64, 1.0)])
def test_block_map_bit_exact(N, K, rate):
    p = _sparse_problem(N + K, 1, K, N, rate, probs=(0.5, 0.2, 0.2, 0.1))
    # blocks of reserved codes only are zero blocks too
    if K >= 256:
        p.packed[0, 32:64] = 0xFF
    got = _map_bits(tern.block_map(torch.from_numpy(p.packed).to(device())))
    assert np.array_equal(got, O().block_map(p.packed, N, K))


SHAPES = [(1, 128, 1), (1, 640, 33), (2, 1152, 50), (3, 3200, 29), (4, 1024, 17), (1, 5120, 640),
          (1, 17408, 96), (4, 17408, 40), (2, 5120, 1000)]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("rate", [0.0, 0.5, 0.9, 1.0])
def test_skip_matches_oracle(M, K, N, rate):
    p = _sparse_problem(M * 31 + K + N + int(rate * 10), M, K, N, rate)
    x, w, s = _dev(p)
    bmap = tern.block_map(w)
    y = tern.matmul_blockmap(x, w, s, bmap, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Y, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, M, N, K, threads=8)
    check(out_bits(y, "f32"), "f32", Y, B, f"{M}x{K}x{N} rate {rate}")


# K a multiple of 1024 (whole wave steps): with a partial last step the list
# hands its chunks to other lanes, and the 16-lane sum associates differently.
# K past the short-step kernel's limit (5120 at M = 1, 8192 at M = 2), so the
# dense call takes the decode kernel whose layout the skipping kernel
# follows (the short-step kernel sums in another order).  The skipping
# kernel serves M <= 2; from M = 3 on the call is tern_matmul.
@pytest.mark.parametrize("M,K,N,xd,yd", [(1, 6144, 512, "bf16", "bf16"), (2, 9216, 77, "f16", "f16"),
                                         (1, 17408, 40, "bf16", "f32"), (2, 10240, 50, "f16", "f32")])
def test_all_marked_equals_dense_kernel_bit_for_bit(M, K, N, xd, yd):
    p = _sparse_problem(M + K + N, M, K, N, 0.5, xd=xd, yd=yd)
    x, w, s = _dev(p)
    words = (K // 128 + 31) // 32
    full = torch.full((N, words), -1, dtype=torch.int32, device=device())
    y_skip = tern.matmul_blockmap(x, w, s, full, out_dtype=TORCH_DT[yd])
    y_dense = tern.matmul(x, w, s, out_dtype=TORCH_DT[yd], path="gemv")
    torch.cuda.synchronize()
    assert np.array_equal(out_bits(y_skip, yd), out_bits(y_dense, yd))


@pytest.mark.parametrize("M", [3, 4])
def test_three_or_more_rows_take_the_dense_product(M):
    p = _sparse_problem(80 + M, M, 5120, 300, 0.5)
    x, w, s = _dev(p)
    y_map = tern.matmul_blockmap(x, w, s, tern.block_map(w), out_dtype=torch.float32)
    y = tern.matmul(x, w, s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_map, y)


def test_superset_map_is_harmless():
    p = _sparse_problem(55, 2, 5120, 300, 0.7)
    x, w, s = _dev(p)
    exact = tern.block_map(w)
    extra = exact | torch.randint(0, 2 ** 31 - 1, exact.shape, dtype=torch.int32, device=device())
    Y, B = O().matmul(p.x, p.x_dtype, p.packed, p.scales, 2, 300, 5120, threads=8)
    for m in (exact, extra):
        y = tern.matmul_blockmap(x, w, s, m, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check(out_bits(y, "f32"), "f32", Y, B, "superset map")


def test_exact_arithmetic_bit_exact():
    M, K, N = 3, 4096, 80
    rng = np.random.default_rng(77)
    xbits = rng.integers(-8, 9, (M, K)).astype(np.float16).view(np.uint16)
    T = workloads.draw_ternary(9, N, K)
    T.reshape(N, K // 128, 128)[rng.random((N, K // 128)) < 0.6] = 0
    P = O().pack(T)
    sbits = (2.0 ** rng.integers(-4, 1, (N, K // 128))).astype(np.float16).view(np.uint16)
    Y, _ = O().matmul(xbits, "f16", P, sbits, M, N, K)
    x, w, s = bits_to_device(xbits, "f16"), torch.from_numpy(P).to(device()), bits_to_device(sbits, "f16")
    for yd in ("f32", "bf16", "f16"):
        y = tern.matmul_blockmap(x, w, s, tern.block_map(w), out_dtype=TORCH_DT[yd])
        assert np.array_equal(O().decode(out_bits(y, yd), yd), O().round(Y, yd)), yd


def test_batched_calls_use_the_dense_path():
    p = _sparse_problem(66, 40, 1024, 96, 0.5, xd="f16")
    x, w, s = _dev(p)
    y_map = tern.matmul_blockmap(x, w, s, tern.block_map(w), out_dtype=torch.float32)
    y = tern.matmul(x, w, s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y_map, y)


@pytest.mark.parametrize("cfg,shape_id", [(2, 0), (3, 0), (3, 1), (3, 2)])
def test_decode_workloads_half_zero_blocks(cfg, shape_id):
    base = workloads.make_problem(cfg, shape_id)
    sh = base.shape
    c = workloads.CONFIGS[cfg]
    base.packed = workloads.draw_block_sparse_packed(workloads.rng_for(cfg, 50, shape_id), sh.N, sh.K, 0.5,
                                                     c.code_probs)
    x, w, s = _dev(base)
    y = tern.matmul_blockmap(x, w, s, tern.block_map(w), out_dtype=TORCH_DT[base.y_dtype])
    torch.cuda.synchronize()
    Y, B = O().matmul(base.x, base.x_dtype, base.packed, base.scales, sh.M, sh.N, sh.K, threads=8)
    check(out_bits(y, base.y_dtype), base.y_dtype, Y, B, f"cfg{cfg}/{shape_id}")
