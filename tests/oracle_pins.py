"""Pins that tie the CPU oracle to the pages and to mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with something fixed independently of it: a golden
fixture derived by hand from the packing rule, a numpy or pure-Python
computation written differently, a closed form, or exact rational arithmetic.
The mutation tests run every pin against deliberately broken copies of the
oracle to show that each plausible mistake is caught by at least one pin.

Rule being pinned: 2kiu.com/news/5082861 ("putting a ternary embedding model
into vLLM") §3.1 (2-bit codes 00->0, 01->+1, 10->-1, 11 reserved -> 0; four
per byte, first weight in the lowest bits; one fp16 scale per 128 consecutive
weights along K) and §4.1-§4.2 (sign accumulation inside a block, the scale
applied at the block boundary, x[M,K] times W[N,K] transposed).
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# fixtures
# ---------------------------------------------------------------------------

def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def code_map():
    return {int(a): int(b) for a, b in read_table("code_map.txt")}


def anchor_bytes():
    return [(int(r[0], 16), [int(v) for v in r[1:5]]) for r in read_table("unpack_anchor_bytes.txt")]


def _expand(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out.extend([v] * int(n))
        else:
            out.append(t)
    return out


def worked_examples():
    text = open(os.path.join(GOLDEN, "matmul_worked_examples.txt")).read()
    exs = []
    cur = None
    for raw in text.splitlines():
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "name":
            cur = {"name": rest[0]}
            exs.append(cur)
        elif key == "shape":
            cur["M"], cur["K"], cur["N"], cur["G"] = map(int, rest)
        elif key == "packed":
            cur["packed"] = np.array([int(b, 16) for b in _expand(rest)], dtype=np.uint8)
        else:
            cur[key] = np.array([float(v) for v in _expand(rest)], dtype=np.float64)
    return exs


# ---------------------------------------------------------------------------
# independent helpers (written differently from the oracle on purpose)
# ---------------------------------------------------------------------------

def np_unpack(packed: np.ndarray) -> np.ndarray:
    """Weights from bytes by t = bit0 - bit1 of each 2-bit field (11 -> 1-1 = 0)."""
    p = packed.astype(np.int16)
    fields = np.stack([(p >> s) & 3 for s in (0, 2, 4, 6)], axis=-1)
    t = (fields & 1) - (fields >> 1)
    return t.reshape(packed.shape[0], -1).astype(np.int8)


def np_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    b = np.ascontiguousarray(bits)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return b.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def np_dense_matmul(x_bits, x_dtype, packed, scale_bits, G):
    """Y = X . (T * S)^T by expanding W densely, then one float64 matmul."""
    X = np_decode(x_bits, x_dtype)
    T = np_unpack(packed).astype(np.float64)
    S = np_decode(scale_bits, "f16")
    W = T * np.repeat(S, G, axis=1)
    Y = X @ W.T
    Bnd = np.abs(X) @ np.abs(np.repeat(S, G, axis=1)).T
    return Y, Bnd


# ---------------------------------------------------------------------------
# pins: number formats
# ---------------------------------------------------------------------------

def pin_f16_decode_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decode_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.decode(bits, "bf16")
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_f32_decode_sample(o):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:6] = [0, 0x80000000, 1, 0x7F7FFFFF, 0x7F800000, 0x00800000]
    got = o.decode(bits, "f32")
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _round_cases(rng):
    v = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e4, 5000), rng.normal(0, 1e-5, 5000),
        np.exp(rng.uniform(-120, 120, 5000)) * rng.choice([-1, 1], 5000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e-8, 2.0**-25, 2.0**-24 * 1.5],
    ])
    return v


def pin_round_f16_and_f32(o):
    rng = np.random.default_rng(11)
    v = _round_cases(rng)
    with np.errstate(over="ignore"):
        ref16 = v.astype(np.float16).astype(np.float64)
        ref32 = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(o.round(v, "f16"), ref16)
    assert np.array_equal(o.round(v, "f32"), ref32)
    # exact halfway cases between fp16 neighbours round to the even one
    a = np.arange(1, 2000, dtype=np.float64)
    mid = (np.float16(1.0) + a * 2.0**-10).astype(np.float64) + 2.0**-11
    mid = mid[mid < 2.0]
    assert np.array_equal(o.round(mid, "f16"), mid.astype(np.float16).astype(np.float64))


def pin_round_bf16(o):
    # For values already exact in float32, bf16 rounding is one rounding of the
    # float32 bit pattern to its top 16 bits (ties to even).
    rng = np.random.default_rng(13)
    with np.errstate(over="ignore"):
        f = _round_cases(rng).astype(np.float32)
    f = f[np.isfinite(f)]
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    ref = (r << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(o.round(f.astype(np.float64), "bf16"), ref)


def pin_ulp(o):
    v = np.array([1.0, 1.5, 2.0, 1000.0, 65504.0, 2.0**-14, 2.0**-20, 0.0, -3.0])
    f16 = v.astype(np.float16)
    with np.errstate(over="ignore"):
        nxt = (np.nextafter(np.abs(f16), np.float16(np.inf)).astype(np.float64)
               - np.abs(f16).astype(np.float64))
    nxt[v == 65504.0] = 32.0  # spacing below the largest finite value
    assert np.array_equal(o.ulp(v, "f16"), nxt)
    assert np.array_equal(o.ulp(np.array([1.0, 3.0, 2.0**-126, 0.0]), "bf16"),
                          np.array([2.0**-7, 2.0**-6, 2.0**-133, 2.0**-133]))
    assert np.array_equal(o.ulp(np.array([1.0, 2.0**-126]), "f32"), np.array([2.0**-23, 2.0**-149]))


# ---------------------------------------------------------------------------
# pins: the code, unpack, pack
# ---------------------------------------------------------------------------

def pin_code_map(o):
    for code, val in code_map().items():
        assert o.code_value(code) == val, (code, o.code_value(code), val)


def pin_unpack_anchors(o):
    for byte, weights in anchor_bytes():
        got = o.unpack(np.array([[byte]], dtype=np.uint8), 1, 4)[0].tolist()
        assert got == weights, (hex(byte), got, weights)


def pin_unpack_exhaustive(o):
    bytes_ = np.arange(256, dtype=np.uint8).reshape(1, 256)
    got = o.unpack(bytes_, 1, 1024).reshape(256, 4)
    cm = code_map()
    lut = np.array([cm[c] for c in range(4)], dtype=np.int8)        # the rule as a table
    ref_table = np.stack([lut[(np.arange(256) >> (2 * i)) & 3] for i in range(4)], axis=1)
    assert np.array_equal(got, ref_table)
    assert np.array_equal(got, np_unpack(bytes_).reshape(256, 4))  # the rule as bit arithmetic


def pin_unpack_layout(o):
    # rows are independent and bytes run along K in order
    rng = np.random.default_rng(3)
    P = rng.integers(0, 256, size=(5, 12), dtype=np.uint8)
    got = o.unpack(P, 5, 48)
    assert np.array_equal(got, np_unpack(P))
    for n in range(5):
        assert np.array_equal(got[n], o.unpack(P[n:n + 1], 1, 48)[0])


def pin_pack_all_tuples(o):
    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=4)), dtype=np.int8)  # 81
    P = o.pack(tuples.reshape(1, -1))[0]
    inv = {v: c for c, v in code_map().items() if c != 3}
    for tup, byte in zip(tuples, P):
        want = sum(inv[int(t)] << (2 * i) for i, t in enumerate(tup))
        assert byte == want, (tup, byte, want)
    assert np.array_equal(o.unpack(P.reshape(1, -1), 1, 324).reshape(81, 4), tuples)


def pin_pack_roundtrip(o):
    T = workloads.draw_ternary(5, 7, 256)
    P = o.pack(T)
    assert P.shape == (7, 64)
    assert np.array_equal(o.unpack(P, 7, 256), T)
    assert np.array_equal(np_unpack(P), T)
    # unpack then pack canonicalises the reserved code 11 to 00
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    canon = allb.copy()
    for s in (0, 2, 4, 6):
        f = (allb >> s) & 3
        canon = np.where(f == 3, canon & ~np.uint8(3 << s), canon)
    assert np.array_equal(o.pack(o.unpack(allb, 1, 1024)), canon)


def pin_pack_invalid_values(o):
    T = np.array([[2, -2, 5, 1]], dtype=np.int8)
    P = o.pack(T)
    assert P[0, 0] == (3 | (3 << 2) | (3 << 4) | (1 << 6))
    assert o.unpack(P, 1, 4).tolist() == [[0, 0, 0, 1]]


# ---------------------------------------------------------------------------
# pins: the matmul
# ---------------------------------------------------------------------------

def pin_worked_examples(o):
    for ex in worked_examples():
        M, K, N, G = ex["M"], ex["K"], ex["N"], ex["G"]
        xb = ex["x"].astype(np.float16).view(np.uint16).reshape(M, K)
        sb = ex["scales"].astype(np.float16).view(np.uint16).reshape(N, K // G)
        Y, B = o.matmul(xb, "f16", ex["packed"].reshape(N, K // 4), sb, M, N, K, G)
        assert np.array_equal(Y.ravel(), ex["y"]), (ex["name"], Y.ravel(), ex["y"])
        assert np.array_equal(B.ravel(), ex["b"]), (ex["name"], B.ravel(), ex["b"])


def _problem(seed, M, K, N, x_dtype="f16", G=128):
    return workloads.make_custom(seed, M, K, N, x_dtype=x_dtype, group=G)


def pin_dense_reduction(o):
    for seed, (M, K, N, xd) in enumerate([(3, 256, 40, "f16"), (2, 512, 17, "bf16"),
                                          (5, 384, 9, "f16"), (1, 1024, 33, "bf16")]):
        p = _problem(seed, M, K, N, xd)
        Y, B = o.matmul(p.x, xd, p.packed, p.scales, M, N, K)
        Yr, Br = np_dense_matmul(p.x, xd, p.packed, p.scales, 128)
        assert np.all(np.abs(Y - Yr) <= 1e-12 * Br + 1e-300), np.max(np.abs(Y - Yr) / Br)
        assert np.allclose(B, Br, rtol=1e-12, atol=0)


def pin_dense_reduction_other_groups(o):
    # the oracle takes any block length dividing K; the dense form checks each
    for G in (4, 32, 64, 256):
        p = _problem(40 + G, 2, 512, 6, "f16", G=G)
        Y, B = o.matmul(p.x, "f16", p.packed, p.scales, 2, 6, 512, G)
        Yr, Br = np_dense_matmul(p.x, "f16", p.packed, p.scales, G)
        assert np.all(np.abs(Y - Yr) <= 1e-12 * Br), G


def pin_brute_force_tiny(o):
    # all 3^K ternary rows (the N axis) against a direct pure-Python sum, G=4
    for K in (4, 8):
        G = 4
        rows = list(itertools.product([-1, 0, 1], repeat=K))
        N = len(rows)
        T = np.array(rows, dtype=np.int8)
        P = o.pack(T)
        rng = np.random.default_rng(K)
        xs = rng.normal(0, 1, (2, K)).astype(np.float16)
        ss = rng.uniform(0.1, 2.0, (N, K // G)).astype(np.float16)
        Y, B = o.matmul(xs.view(np.uint16), "f16", P, ss.view(np.uint16), 2, N, K, G)
        for m in range(2):
            for n in range(N):
                y = 0.0
                for k in range(K):
                    y += float(xs[m, k]) * rows[n][k] * float(ss[n, k // G])
                assert abs(Y[m, n] - y) <= 1e-12 * (B[m, n] + 1e-30), (m, n, Y[m, n], y)


def pin_closed_forms(o):
    M, K, N = 3, 512, 8
    p = _problem(9, M, K, N, "f16")
    X = np_decode(p.x, "f16")
    S = np_decode(p.scales, "f16")
    G = 128
    full = lambda byte: np.full((N, K // 4), byte, dtype=np.uint8)
    Yp, _ = o.matmul(p.x, "f16", full(0x55), p.scales, M, N, K)
    want = np.array([[sum(S[n, g] * X[m, g * G:(g + 1) * G].sum() for g in range(K // G))
                      for n in range(N)] for m in range(M)])
    assert np.allclose(Yp, want, rtol=1e-13, atol=1e-13)
    Ym, _ = o.matmul(p.x, "f16", full(0xAA), p.scales, M, N, K)
    assert np.array_equal(Ym, -Yp)
    for byte in (0x00, 0xFF):
        Yz, _ = o.matmul(p.x, "f16", full(byte), p.scales, M, N, K)
        assert np.array_equal(Yz, np.zeros_like(Yz))
    # one nonzero code: +-s*x_k
    P1 = full(0x00)
    P1[2, 37] = 0x01 << 4          # weight k = 4*37 + 2 = 150 of row 2 is +1
    Y1, _ = o.matmul(p.x, "f16", P1, p.scales, M, N, K)
    exp = np.zeros((M, N))
    exp[:, 2] = X[:, 150] * S[2, 150 // G]
    assert np.array_equal(Y1, exp)
    P1[2, 37] = 0x02 << 4
    Y2, _ = o.matmul(p.x, "f16", P1, p.scales, M, N, K)
    assert np.array_equal(Y2, -exp)


def _swap_codes(P):
    out = P.copy()
    for s in (0, 2, 4, 6):
        f = (P >> s) & 3
        new = np.where(f == 1, 2, np.where(f == 2, 1, f)).astype(np.uint8)
        out = (out & ~np.uint8(3 << s)) | (new << s)
    return out


def _reserved_to_zero(P):
    out = P.copy()
    for s in (0, 2, 4, 6):
        f = (P >> s) & 3
        out = np.where(f == 3, out & ~np.uint8(3 << s), out)
    return out


def pin_invariants(o):
    p = workloads.make_custom(12, 4, 640, 24, probs=(0.3, 0.3, 0.3, 0.1))
    args = (4, 24, 640)
    Y, B = o.matmul(p.x, "f16", p.packed, p.scales, *args)
    Ys, _ = o.matmul(p.x, "f16", _swap_codes(p.packed), p.scales, *args)
    assert np.array_equal(Ys, -Y)
    Yr, _ = o.matmul(p.x, "f16", _reserved_to_zero(p.packed), p.scales, *args)
    assert np.array_equal(Yr, Y)
    # Y(2X) = 2Y and Y(2S) = 2Y (powers of two are exact)
    x2 = (np_decode(p.x, "f16") * 2).astype(np.float16).view(np.uint16)
    Y2, B2 = o.matmul(x2, "f16", p.packed, p.scales, *args)
    assert np.array_equal(Y2, 2 * Y) and np.array_equal(B2, 2 * B)
    s2 = (np_decode(p.scales, "f16") * 2).astype(np.float16).view(np.uint16)
    Ys2, _ = o.matmul(p.x, "f16", p.packed, s2, *args)
    assert np.array_equal(Ys2, 2 * Y)
    # block additivity: Y is the sum of Y with all blocks but one zeroed
    acc = np.zeros_like(Y)
    for g in range(640 // 128):
        Pg = np.zeros_like(p.packed)
        Pg[:, g * 32:(g + 1) * 32] = p.packed[:, g * 32:(g + 1) * 32]
        acc += o.matmul(p.x, "f16", Pg, p.scales, *args)[0]
    assert np.allclose(acc, Y, rtol=1e-12, atol=1e-12 * B.max())
    # permuting W's rows (with their scales) permutes Y's columns
    perm = np.random.default_rng(1).permutation(24)
    Yp, _ = o.matmul(p.x, "f16", p.packed[perm], p.scales[perm], *args)
    assert np.array_equal(Yp, Y[:, perm])
    # permuting X's rows permutes Y's rows
    Yq, _ = o.matmul(p.x[::-1].copy(), "f16", p.packed, p.scales, *args)
    assert np.array_equal(Yq, Y[::-1])
    # the bound dominates the value
    assert np.all(np.abs(Y) <= B)


def pin_exact_arithmetic(o):
    # integer x in [-8, 8], power-of-two scales: the exact rational result
    rng = np.random.default_rng(21)
    M, K, N, G = 2, 512, 6, 128
    xi = rng.integers(-8, 9, (M, K))
    T = workloads.draw_ternary(22, N, K)
    P = o.pack(T)
    e = rng.integers(-4, 1, (N, K // G))
    Y, B = o.matmul(xi.astype(np.float16).view(np.uint16), "f16", P,
                    (2.0 ** e).astype(np.float16).view(np.uint16), M, N, K, G)
    for m in range(M):
        for n in range(N):
            y = sum(Fraction(int(xi[m, k]) * int(T[n, k])) * Fraction(2) ** int(e[n, k // G])
                    for k in range(K))
            b = sum(Fraction(abs(int(xi[m, k]))) * Fraction(2) ** int(e[n, k // G]) for k in range(K))
            assert Fraction(Y[m, n]) == y and Fraction(B[m, n]) == b, (m, n)


def pin_bf16_activations(o):
    # bf16 inputs decode through their own format (values beyond fp16 range)
    xb = workloads.to_bf16_bits(np.array([[1e10, -3e-20, 2.5, 7.0] * 32]))
    P = np.full((1, 32), 0x55, dtype=np.uint8)
    s = np.array([[np.float16(0.5)]]).view(np.uint16)
    Y, B = o.matmul(xb, "bf16", P, s, 1, 1, 128)
    X = np_decode(xb, "bf16")
    assert Y[0, 0] == 0.5 * X.sum() or abs(Y[0, 0] - 0.5 * X.sum()) <= 1e-15 * B[0, 0]
    assert X[0, 0] > 9e9


def pin_sampled_matches_full(o):
    p = workloads.make_custom(31, 3, 384, 20, x_dtype="bf16")
    Y, B = o.matmul(p.x, "bf16", p.packed, p.scales, 3, 20, 384, threads=3)
    Y1, B1 = o.matmul(p.x, "bf16", p.packed, p.scales, 3, 20, 384, threads=1)
    assert np.array_equal(Y, Y1) and np.array_equal(B, B1)
    ms = np.array([0, 2, 1, 2])
    ns = np.array([0, 19, 7, 3])
    Ya, Ba = o.matmul_at(p.x, "bf16", p.packed, p.scales, 3, 20, 384, ms, ns)
    assert np.array_equal(Ya, Y[ms, ns]) and np.array_equal(Ba, B[ms, ns])


# ---------------------------------------------------------------------------
# pins: the comparison route, the block map, int8 scales
# ---------------------------------------------------------------------------

def pin_dequant_dense(o):
    p = workloads.make_custom(51, 1, 640, 9, reserved_rate=0.05)
    W = o.dequant(p.packed, p.scales, 9, 640)
    ref = np_unpack(p.packed).astype(np.float64) * np.repeat(np_decode(p.scales, "f16"), 128, axis=1)
    assert np.array_equal(W, ref)


def pin_block_map(o):
    rng = workloads.rng_for(102, 0, 0)
    P = workloads.draw_block_sparse_packed(rng, 7, 128 * 40, 0.5, probs=(0.8, 0.1, 0.1, 0.0))
    P[3, 5 * 32:6 * 32] = 0xFF          # a block of reserved codes only counts as zero
    P[4, 7 * 32 + 3] = 0x40             # a single nonzero weight marks its block
    got = o.block_map(P, 7, 128 * 40)
    nz = (np_unpack(P).reshape(7, 40, 128) != 0).any(axis=2)
    want = np.zeros((7, 2), dtype=np.uint32)
    for n in range(7):
        for g in range(40):
            if nz[n, g]:
                want[n, g // 32] |= np.uint32(1 << (g % 32))
    assert np.array_equal(got, want)
    assert not (got[3, 0] >> 5) & 1 and (got[4, 0] >> 7) & 1


def pin_quantize_scales(o):
    p = workloads.make_custom(52, 1, 128 * 24, 30, scale_lo=1e-4, scale_hi=3.0)
    S = p.scales.copy()
    S[4] = 0                                            # an all-zero row
    S[5, 3] = np.float16(-2.5).view(np.uint16)          # a negative scale
    q, r = o.quantize_scales(S)
    s32 = S.view(np.float16).astype(np.float32)
    r_ref = (np.abs(s32).max(axis=1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q_ref = np.where(r_ref[:, None] > 0, np.rint((s32 / r_ref[:, None]).astype(np.float32)), 0)
    assert np.array_equal(r, r_ref) and np.array_equal(q, q_ref.astype(np.int8))
    assert np.abs(q).max() == 127 and not q[4].any() and q[5, 3] < 0
    rel = np.abs(q * r[:, None].astype(np.float64) - s32) / np.maximum(np.abs(s32).max(axis=1, keepdims=True), 1e-30)
    assert rel.max() <= 0.5 / 127 + 1e-7


def pin_matmul_int8_scales(o):
    p = workloads.make_custom(53, 3, 640, 11, x_dtype="bf16")
    q, r = o.quantize_scales(p.scales)
    Y, B = o.matmul_s8(p.x, "bf16", p.packed, q, r, 3, 11, 640, threads=2)
    S_eff = q.astype(np.float64) * r.astype(np.float64)[:, None]
    W = np_unpack(p.packed).astype(np.float64) * np.repeat(S_eff, 128, axis=1)
    X = np_decode(p.x, "bf16")
    assert np.all(np.abs(Y - X @ W.T) <= 1e-12 * B)
    assert np.allclose(B, np.abs(X) @ np.abs(np.repeat(S_eff, 128, axis=1)).T, rtol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
