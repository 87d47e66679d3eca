"""Pins for the CPU oracle against things other than itself.

Each test checks the oracle (oracle/mole_oracle.c) against an independent
source: numpy/scipy library routines, textbook constants, pure-Python brute
force on tiny inputs, closed forms of the method (softmax special cases,
linearity, direct addressing) and hand-derived NF3 bit patterns.  None of
them re-types the oracle's own formula.

Definitions (MoLE article, "ICML 2025 Spotlight | MoLE" page):
  * inference section: LUT[v,e,:] = FFN_e(Emb[v]); retrieval by token id;
  * training section: all routed experts active, router on contextual h;
  * results section: table compressed to 3 bits, e.g. NF3 (NormalFloat
    construction of QLoRA applied at k = 3, blocks of 64, fp16 absmax scale).
"""
import math
import struct
from fractions import Fraction
from statistics import NormalDist

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from mixture_lookup_experts_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def f32_hex(x):
    return "%08x" % struct.unpack("<I", struct.pack("<f", float(x)))[0]


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_layer(seed, V, D, F, N, std=1.0, dtype="f32"):
    r = rng(seed)
    def draw(shape, s):
        x = (r.standard_normal(shape, dtype=np.float32) * np.float32(s))
        return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    return (draw((V, D), std), draw((N, F, D), std / math.sqrt(D)),
            draw((N, D, F), std / math.sqrt(F)), draw((N, D), std / math.sqrt(D)))


def as_f64(a):
    return (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


# ----------------------------------------------------------------------------
# LUT build
# ----------------------------------------------------------------------------

def numpy_lut(emb, w_up, w_down):
    """Library-routine definition: gelu_erf(Emb @ W_up[e]^T) @ W_down[e]^T."""
    E, U, W = as_f64(emb), as_f64(w_up), as_f64(w_down)
    out = []
    for e in range(U.shape[0]):
        u = E @ U[e].T
        g = 0.5 * u * (1.0 + scipy.special.erf(u / np.sqrt(2.0)))
        out.append(g @ W[e].T)
    return np.stack(out, axis=1)  # [V, N, D]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_build_matches_numpy_scipy(dtype):
    emb, w_up, w_down, _ = rand_layer(11, V=24, D=16, F=40, N=3, std=1.0, dtype=dtype)
    got = oracle.build_lut_rows(emb, w_up, w_down)
    ref = numpy_lut(emb, w_up, w_down)
    assert got.shape == (24, 3, 16)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_build_bruteforce_python_loops():
    emb, w_up, w_down, _ = rand_layer(12, V=3, D=4, F=5, N=2, std=1.0)
    got = oracle.build_lut_rows(emb, w_up, w_down)
    for v in range(3):
        for e in range(2):
            g = []
            for f in range(5):
                u = sum(float(emb[v, d]) * float(w_up[e, f, d]) for d in range(4))
                g.append(u * 0.5 * math.erfc(-u / math.sqrt(2.0)))
            for d in range(4):
                ref = sum(g[f] * float(w_down[e, d, f]) for f in range(5))
                assert got[v, e, d] == pytest.approx(ref, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("u,phi", [(1.0, 0.8413447460685429), (-1.0, 0.15865525393145707),
                                   (2.0, 0.9772498680518208), (0.5, 0.6914624612740131)])
def test_gelu_is_erf_form(u, phi):
    """GELU(u) = u * Phi(u) with textbook Phi values; the tanh approximation
    misses these by ~1e-4 and would fail."""
    emb = np.array([[u]], dtype=np.float32)
    ones = np.ones((1, 1, 1), dtype=np.float32)
    got = oracle.build_lut_rows(emb, ones, ones)[0, 0, 0]
    assert got == pytest.approx(u * phi, rel=1e-14)
    assert oracle.gelu(u) == pytest.approx(u * phi, rel=1e-14)
    tanh_form = 0.5 * u * (1 + math.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))
    assert abs(tanh_form - u * phi) > 1e-5


def test_build_zero_row_is_zero_and_rows_select():
    emb, w_up, w_down, _ = rand_layer(13, V=6, D=8, F=8, N=2)
    emb[4] = 0.0
    full = oracle.build_lut_rows(emb, w_up, w_down)
    assert np.all(full[4] == 0.0)              # no bias, GELU(0) = 0
    sub = oracle.build_lut_rows(emb, w_up, w_down, rows=[5, 0, 5])
    np.testing.assert_array_equal(sub, full[[5, 0, 5]])


def test_build_linear_in_w_down_and_expert_equivariant():
    emb, w_up, w_down, _ = rand_layer(14, V=5, D=8, F=6, N=3)
    base = oracle.build_lut_rows(emb, w_up, w_down)
    np.testing.assert_array_equal(oracle.build_lut_rows(emb, w_up, w_down * np.float32(2)), 2 * base)
    p = [2, 0, 1]
    perm = oracle.build_lut_rows(emb, np.ascontiguousarray(w_up[p]), np.ascontiguousarray(w_down[p]))
    np.testing.assert_array_equal(perm, base[:, p, :])


def test_build_rejects_bad_rows():
    emb, w_up, w_down, _ = rand_layer(15, V=4, D=4, F=4, N=1)
    with pytest.raises(ValueError):
        oracle.build_lut_rows(emb, w_up, w_down, rows=[4])


def test_lut_size_independent_of_hidden_dim():
    """The table is [V][N][D] whatever the expert hidden width F."""
    for F in (8, 32):
        emb, w_up, w_down, _ = rand_layer(16, V=7, D=8, F=F, N=2)
        assert oracle.build_lut_rows(emb, w_up, w_down).shape == (7, 2, 8)


# ----------------------------------------------------------------------------
# Router gates and lookup-combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gates_match_scipy_softmax_and_sum_to_one(dtype):
    r = rng(21)
    h = r.standard_normal((37, 32), dtype=np.float32)
    w_r = r.standard_normal((5, 32), dtype=np.float32) * np.float32(0.3)
    if dtype == "bf16":
        h, w_r = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w_r)
    g = oracle.router_gates(h, w_r)
    ref = scipy.special.softmax(as_f64(h) @ as_f64(w_r).T, axis=1)
    np.testing.assert_allclose(g, ref, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_combine_matches_numpy_einsum():
    r = rng(22)
    V, N, D, T = 40, 4, 24, 50
    lut = r.standard_normal((V, N, D), dtype=np.float32)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = r.standard_normal((N, D), dtype=np.float32) * np.float32(0.2)
    ids = r.integers(0, V, T)
    y = oracle.lookup_combine(ids, h, w_r, lut)
    g = scipy.special.softmax(h.astype(np.float64) @ w_r.astype(np.float64).T, axis=1)
    ref = np.einsum("te,ted->td", g, lut.astype(np.float64)[ids])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_combine_zero_router_gives_slab_mean():
    r = rng(23)
    lut = r.standard_normal((10, 4, 8), dtype=np.float32)
    h = r.standard_normal((6, 8), dtype=np.float32)
    ids = np.array([3, 3, 0, 9, 5, 1])
    y = oracle.lookup_combine(ids, h, np.zeros((4, 8), np.float32), lut)
    np.testing.assert_allclose(y, lut.astype(np.float64)[ids].mean(axis=1), rtol=1e-15, atol=1e-16)


def test_combine_saturated_logits_one_hot_exact():
    r = rng(24)
    lut = r.standard_normal((10, 4, 8), dtype=np.float32)
    h = np.zeros((4, 8), np.float32)
    h[:, 0] = 1.0
    ids = np.array([2, 7, 7, 0])
    for e_star in range(4):
        w_r = np.zeros((4, 8), np.float32)
        w_r[e_star, 0] = 1000.0   # logit gap 1000: exp(-1000) underflows to 0
        y = oracle.lookup_combine(ids, h, w_r, lut)
        np.testing.assert_array_equal(y, lut.astype(np.float64)[ids, e_star])


def test_combine_depends_only_on_own_row_and_is_permutation_invariant():
    r = rng(25)
    V, N, D, T = 12, 4, 16, 5
    lut = r.standard_normal((V, N, D), dtype=np.float32)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = r.standard_normal((N, D), dtype=np.float32)
    ids = np.array([1, 4, 4, 9, 0])
    y = oracle.lookup_combine(ids, h, w_r, lut)
    other = np.setdiff1d(np.arange(V), ids)
    lut2 = lut.copy()
    lut2[other] = r.standard_normal((other.size, N, D), dtype=np.float32)
    np.testing.assert_array_equal(oracle.lookup_combine(ids, h, w_r, lut2), y)
    p = [3, 1, 0, 2]
    yp = oracle.lookup_combine(ids, h, np.ascontiguousarray(w_r[p]), np.ascontiguousarray(lut[:, p]))
    np.testing.assert_allclose(yp, y, rtol=1e-14, atol=1e-15)


def test_combine_uses_every_expert_row_whatever_the_gates():
    """All routed experts are active (no top-k): with every gate positive,
    perturbing any single expert's row of a token's slab moves that token's
    output by exactly gate[e] * delta, so every token reads all N rows and
    the lookup cost is N*D per token however peaked the gates are."""
    r = rng(26)
    V, N, D, T = 9, 6, 16, 7
    lut = r.standard_normal((V, N, D), dtype=np.float32)
    h = r.standard_normal((T, D), dtype=np.float32)
    # peaked but non-zero gates (logit gaps of a few units)
    w_r = r.standard_normal((N, D), dtype=np.float32)
    ids = np.array([0, 3, 3, 8, 5, 1, 0])
    y = oracle.lookup_combine(ids, h, w_r, lut)
    g = oracle.router_gates(h, w_r)
    assert g.min() > 1e-8 and g.max() > 0.9  # peaked, yet every expert weighs in
    for e in range(N):
        lut2 = lut.copy()
        delta = r.standard_normal(D).astype(np.float32)
        lut2[:, e] += delta
        y2 = oracle.lookup_combine(ids, h, w_r, lut2)
        moved = (lut2.astype(np.float64)[ids, e] - lut.astype(np.float64)[ids, e])
        # (fp64: each of y, y2 carries rounding ~1e-16 |y|, hence the absolute bar)
        np.testing.assert_allclose(y2 - y, g[:, e:e + 1] * moved, rtol=1e-9, atol=1e-13)
        assert (np.abs(y2 - y).max(axis=1) > 0).all()


def test_combine_empty_batch_and_bad_id():
    lut = np.zeros((4, 2, 8), np.float32)
    w_r = np.zeros((2, 8), np.float32)
    y = oracle.lookup_combine(np.zeros(0, np.int64), np.zeros((0, 8), np.float32), w_r, lut)
    assert y.shape == (0, 8)
    with pytest.raises(ValueError):
        oracle.lookup_combine(np.array([4]), np.zeros((1, 8), np.float32), w_r, lut)
    with pytest.raises(ValueError):
        oracle.lookup_combine(np.array([-1]), np.zeros((1, 8), np.float32), w_r, lut)


# ----------------------------------------------------------------------------
# NF3
# ----------------------------------------------------------------------------

def nf_levels_stdlib(k):
    """NormalFloat levels at k bits from Python's statistics.NormalDist."""
    nd = NormalDist()
    half = 2 ** (k - 1)
    p = 1 - 0.5 * (1 / (2 * (2 ** k - 1)) + 1 / (2 * 2 ** k))
    pos = [nd.inv_cdf(x) for x in np.linspace(p, 0.5, half + 1)[:-1]]
    neg = [-nd.inv_cdf(x) for x in np.linspace(p, 0.5, half)[:-1]]
    v = sorted(pos + [0.0] + neg)
    return np.array([x / max(v) for x in v], dtype=np.float32)


def test_nf3_codebook_matches_stdlib_construction():
    lv = oracle.nf3_levels()
    np.testing.assert_array_equal(lv, nf_levels_stdlib(3))
    assert [f32_hex(x) for x in lv] == ["bf800000", "bf08f740", "be7cdb98", "00000000",
                                        "3e3bbcd2", "3ec394b6", "3f1f7bfe", "3f800000"]
    assert lv[3] == 0.0 and lv[0] == -1.0 and lv[7] == 1.0


def test_nf_construction_reproduces_nf4_at_four_bits():
    """Sanity of the construction itself: at k = 4 it gives the NF4 table
    (first entries -1, -0.6962, -0.5251, ..., 0.7230, 1)."""
    nf4 = nf_levels_stdlib(4)
    np.testing.assert_allclose(nf4[:4], [-1.0, -0.6961928, -0.5250731, -0.3949175], atol=2e-7)
    np.testing.assert_allclose(nf4[-3:], [0.5626170, 0.7229568, 1.0], atol=2e-7)
    assert nf4[7] == 0.0


def test_nf3_midpoints_are_rne_of_exact_midpoints():
    lv, mid = oracle.nf3_levels(), oracle.nf3_midpoints()
    for j in range(7):
        exact = (Fraction(float(lv[j])) + Fraction(float(lv[j + 1]))) / 2
        cands = [np.float32(float(exact)), np.nextafter(np.float32(float(exact)), np.float32(2)),
                 np.nextafter(np.float32(float(exact)), np.float32(-2))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact),
                                         struct.unpack("<I", struct.pack("<f", float(c)))[0] & 1))
        assert mid[j] == best
    # level 5/6 midpoint is an exact fp32 tie; ties-to-even picks ...2c
    assert f32_hex(mid[5]) == "3f00a32c"


def test_fp16_rne_matches_numpy():
    r = rng(31)
    xs = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * np.float32(1e-3),
        np.abs(r.standard_normal(20000)).astype(np.float32) * np.float32(300),
        (r.random(5000) * 6e-5).astype(np.float32),          # fp16 subnormal range
        np.array([0.0, 65504.0, 65519.0, 6.103515625e-05, 5.960464477539063e-08,
                  2.9802322387695312e-08, 2.98023259e-08, 1.0, 1.00048828125,
                  1.000732421875, 2049.0, 2051.0, 0.333333343], dtype=np.float32),
    ])
    # exact halfway points between fp16 neighbours
    h16 = np.arange(0x0001, 0x7BFF, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0x0001, 0x7BFF, 37, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    xs = np.concatenate([xs, ((h16 + nxt) / 2).astype(np.float32)])
    want = np.abs(xs).astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_rne(abs(float(x))) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    for b in (0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x5640):
        assert oracle.f16_to_f32(b) == float(np.array([b], np.uint16).view(np.float16)[0])


def read_codes_python(row_bytes, D):
    """Independent bit reader: code i = bits [3i, 3i+3) of the little-endian stream."""
    big = int.from_bytes(bytes(row_bytes), "little")
    return [(big >> (3 * i)) & 7 for i in range(D)]


def test_nf3_pack_worked_example_codes_0_to_7():
    """x_i = level[i mod 8] in a block with absmax 1.0: scale fp16(1.0) = 0x3C00
    and codes 0,1,...,7 repeating.  Eight codes 0..7 LSB-first are the octal
    number 76543210 = 0xFAC688, i.e. bytes 88 C6 FA."""
    lv = oracle.nf3_levels()
    x = np.array([lv[i % 8] for i in range(64)], dtype=np.float32).reshape(1, 64)
    codes, scales, nsat = oracle.pack_nf3(x)
    assert nsat == 0
    assert scales.tolist() == [[0x3C00]]
    assert bytes(codes[0]) == bytes([0x88, 0xC6, 0xFA]) * 8
    assert int("76543210", 8) == 0xFAC688


def test_nf3_zero_and_tiny_blocks_give_code_3():
    """code 3 is the zero level; eight 3s are octal 33333333 = 0x6DB6DB."""
    x = np.zeros((2, 128), dtype=np.float32)
    x[1, 64:] = np.float32(1e-9)       # absmax rounds to fp16 zero
    codes, scales, _ = oracle.pack_nf3(x)
    assert scales.tolist() == [[0, 0], [0, 0]]
    assert bytes(codes[0]) == bytes([0xDB, 0xB6, 0x6D]) * 16
    assert bytes(codes[1]) == bytes(codes[0])


def test_nf3_saturation_clamps_scale():
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 5] = -1e6
    x[0, 6] = 70000.0
    codes, scales, nsat = oracle.pack_nf3(x)
    assert nsat == 1 and scales[0, 0] == 0x7BFF
    c = read_codes_python(codes[0], 64)
    assert c[5] == 0 and c[6] == 7 and c[0] == 3


def test_nf3_codes_equal_bruteforce_nearest_level():
    """Away from decision boundaries the threshold code is the nearest level."""
    r = rng(32)
    lv = nf_levels_stdlib(3).astype(np.float64)
    x = (r.standard_normal((64, 128)) * r.choice([1e-3, 0.05, 3.0], size=(64, 1))).astype(np.float32)
    xb = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    codes, scales, _ = oracle.pack_nf3(synth.f32_to_bf16_bits(x))
    s = scales.astype(np.uint16).view(np.float16).astype(np.float64)
    checked = 0
    for row in range(64):
        c = read_codes_python(codes[row], 128)
        for i in range(128):
            si = s[row, i // 64]
            t = float(xb[row, i]) / si
            dist = np.abs(t - lv)
            order = np.argsort(dist)
            if dist[order[1]] - dist[order[0]] < 1e-5:
                continue
            assert c[i] == order[0], (row, i, t)
            checked += 1
    assert checked > 8000


def test_nf3_unpack_roundtrip_and_requantise_fixed_point():
    r = rng(33)
    x = synth.f32_to_bf16_bits(r.standard_normal((9, 4, 192)).astype(np.float32) * np.float32(0.04))
    codes, scales, _ = oracle.pack_nf3(x)
    assert codes.shape == (9, 4, 72) and scales.shape == (9, 4, 3)
    un = oracle.unpack_nf3(codes, 192)
    for v in range(9):
        for e in range(4):
            assert un[v, e].tolist() == read_codes_python(codes[v, e], 192)
    xhat = oracle.dequant_nf3(codes, scales, 192).astype(np.float32)
    codes2, scales2, _ = oracle.pack_nf3(xhat)
    np.testing.assert_array_equal(scales2, scales)
    np.testing.assert_array_equal(codes2, codes)


def test_nf3_error_bound():
    r = rng(34)
    x = r.standard_normal((50, 256)).astype(np.float32)
    codes, scales, _ = oracle.pack_nf3(x)
    xhat = oracle.dequant_nf3(codes, scales, 256)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    a = np.repeat(np.abs(x).reshape(50, 4, 64).max(axis=2), 64, axis=1)
    half_gap = np.max(np.diff(nf_levels_stdlib(3).astype(np.float64))) / 2
    assert half_gap == pytest.approx(0.2324886, abs=1e-6)
    err = np.abs(x.astype(np.float64) - xhat)
    assert np.all(err <= half_gap * s + 2.0 ** -11 * a + 1e-7 * s)


def test_nf3_combine_matches_independent_decode():
    r = rng(35)
    V, N, D, T = 30, 4, 128, 20
    table = synth.f32_to_bf16_bits(r.standard_normal((V, N, D)).astype(np.float32) * np.float32(0.02))
    codes, scales, _ = oracle.pack_nf3(table)
    h = synth.f32_to_bf16_bits(r.standard_normal((T, D)).astype(np.float32))
    w_r = synth.f32_to_bf16_bits(r.standard_normal((N, D)).astype(np.float32) * np.float32(0.05))
    ids = r.integers(0, V, T)
    y = oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)
    lv = nf_levels_stdlib(3).astype(np.float64)
    sc = scales.view(np.float16).astype(np.float64)
    xhat = np.zeros((V, N, D))
    for v in range(V):
        for e in range(N):
            c = read_codes_python(codes[v, e], D)
            xhat[v, e] = lv[c] * np.repeat(sc[v, e], 64)
    g = scipy.special.softmax(as_f64(h) @ as_f64(w_r).T, axis=1)
    ref = np.einsum("te,ted->td", g, xhat[ids])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_nf3_rejects_d_not_multiple_of_64():
    with pytest.raises(ValueError):
        oracle.pack_nf3(np.zeros((2, 96), np.float32))


# ----------------------------------------------------------------------------
# Synthetic inputs (generator module shared by both sides)
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    r = rng(41)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * np.float32(0.02),
                        r.standard_normal(1000).astype(np.float32) * np.float32(1e30),
                        np.array([0.0, -0.0, 1.00390625, 1.01171875], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), want)


def test_zipf_ids_in_range_and_unique_count():
    w = synth.WORKLOADS["410m"]
    perm = synth.rank_permutation(w)
    assert sorted(perm[:5].tolist()) != [0, 1, 2, 3, 4]
    counts = []
    for step in range(6):
        ids = synth.make_ids(w, 1024, step=step, perm=perm)
        assert ids.min() >= 0 and ids.max() < w.V
        counts.append(np.unique(ids).size)
    exp = synth.expected_unique(w.V, 1024)
    assert 400 < exp < 540
    assert abs(np.mean(counts) - exp) < 0.06 * exp
    d = synth.make_ids(w, 4096, kind="distinct")
    assert np.unique(d).size == 4096


# ----------------------------------------------------------------------------
# Shared expert and the full block (training section: shared experts and the
# router read the contextual hidden state; complexity analysis: only the
# shared experts are still computed at inference)
# ----------------------------------------------------------------------------

def numpy_shared(h, w_s_up, w_s_down):
    """Library-routine definition: gelu_erf(h @ W_s_up^T) @ W_s_down^T."""
    u = as_f64(h) @ as_f64(w_s_up).T
    g = 0.5 * u * (1.0 + scipy.special.erf(u / np.sqrt(2.0)))
    return g @ as_f64(w_s_down).T


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_ffn_matches_numpy_scipy(dtype):
    r = rng(301)
    T, D, F = 7, 24, 40
    def draw(shape, s):
        x = r.standard_normal(shape, dtype=np.float32) * np.float32(s)
        return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    h, wu, wd = draw((T, D), 1.0), draw((F, D), 1.0 / math.sqrt(D)), draw((D, F), 1.0 / math.sqrt(F))
    got = oracle.shared_ffn(h, wu, wd)
    assert np.abs(got - numpy_shared(h, wu, wd)).max() <= 1e-12 * max(1.0, np.abs(got).max())


def test_shared_ffn_identity_weights_give_elementwise_gelu():
    # F = D, W_s_up = c I, W_s_down = I  =>  out[t][d] = GELU(c h[t][d]) (closed form,
    # each value from math.erf).
    r = rng(302)
    T, D, c = 5, 12, 1.75
    h = r.standard_normal((T, D), dtype=np.float32)
    wu = (np.eye(D, dtype=np.float32) * np.float32(c))
    wd = np.eye(D, dtype=np.float32)
    got = oracle.shared_ffn(h, wu, wd)
    for t in range(T):
        for d in range(D):
            u = c * float(h[t, d])
            assert got[t, d] == pytest.approx(0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))), abs=1e-14)


def test_shared_ffn_zero_input_is_zero_and_tokens_independent():
    r = rng(303)
    T, D, F = 6, 16, 20
    h = r.standard_normal((T, D), dtype=np.float32)
    h[2] = 0.0
    wu = r.standard_normal((F, D), dtype=np.float32)
    wd = r.standard_normal((D, F), dtype=np.float32)
    got = oracle.shared_ffn(h, wu, wd)
    assert np.all(got[2] == 0.0)                      # no bias, GELU(0) = 0
    one = oracle.shared_ffn(np.ascontiguousarray(h[4:5]), wu, wd)
    assert np.array_equal(one[0], got[4])             # a token sees only its own row


def test_layer_forward_matches_numpy_composition():
    # Residual + shared FFN + router-weighted table rows, each term written with
    # numpy/scipy library routines.
    r = rng(304)
    V, T, D, F, N = 40, 9, 16, 24, 4
    lut = r.standard_normal((V, N, D), dtype=np.float32)
    ids = r.integers(0, V, size=T, dtype=np.int64)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = r.standard_normal((N, D), dtype=np.float32) * np.float32(0.3)
    wu = r.standard_normal((F, D), dtype=np.float32) * np.float32(0.25)
    wd = r.standard_normal((D, F), dtype=np.float32) * np.float32(0.2)
    x = r.standard_normal((T, D), dtype=np.float32)
    got = oracle.layer_forward(ids, h, w_r, lut, wu, wd, x)
    g = scipy.special.softmax(h.astype(np.float64) @ w_r.astype(np.float64).T, axis=1)
    routed = np.einsum("te,ted->td", g, lut.astype(np.float64)[ids])
    ref = x.astype(np.float64) + numpy_shared(h, wu, wd) + routed
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # Without a residual the block output is the two expert terms alone.
    got0 = oracle.layer_forward(ids, h, w_r, lut, wu, wd, None)
    assert np.abs(got0 - (ref - x.astype(np.float64))).max() <= 1e-12 * np.abs(ref).max()


def test_layer_forward_zero_shared_weights_reduce_to_lookup():
    r = rng(305)
    V, T, D, F, N = 30, 5, 16, 8, 3
    lut = r.standard_normal((V, N, D), dtype=np.float32)
    ids = r.integers(0, V, size=T, dtype=np.int64)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = r.standard_normal((N, D), dtype=np.float32)
    zu, zd = np.zeros((F, D), np.float32), np.zeros((D, F), np.float32)
    assert np.array_equal(oracle.layer_forward(ids, h, w_r, lut, zu, zd, None),
                          oracle.lookup_combine(ids, h, w_r, lut))


# ----------------------------------------------------------------------------
# Other table formats (results section: redundancy remains at 3 bits): NF4
# (the NormalFloat construction at 4 bits, same blocks and scales as NF3) and
# int8 with one fp32 scale per (v, e) row.
# ----------------------------------------------------------------------------

def test_nf4_codebook_matches_stdlib_construction_and_published_values():
    lv = oracle.nf4_levels()
    np.testing.assert_array_equal(lv, nf_levels_stdlib(4))
    assert lv[7] == 0.0 and lv[0] == -1.0 and lv[15] == 1.0 and np.all(np.diff(lv) > 0)
    # the NF4 table as published with QLoRA (its probability grid was rounded
    # to fp32, hence agreement to about 2e-7 rather than bit for bit)
    np.testing.assert_allclose(lv[[1, 2, 3, 8, 13, 14]],
                               [-0.6961928, -0.5250731, -0.3949175, 0.0795803, 0.5626170, 0.7229568], atol=2e-7)


def test_nf4_midpoints_are_rne_of_exact_midpoints():
    lv, mid = oracle.nf4_levels(), oracle.nf4_midpoints()
    for j in range(15):
        exact = (Fraction(float(lv[j])) + Fraction(float(lv[j + 1]))) / 2
        assert mid[j] == np.float32(float(exact))  # one rounding of the exact value


def test_nf4_pack_worked_example_codes_0_to_15():
    # s = 1: each element equals a level, codes 0..15 four times; nibbles low
    # first, so a pair (2k, 2k+1) packs into the byte 0x(2k+1)(2k).
    lv = oracle.nf4_levels()
    row = np.tile(lv, 4).astype(np.float32)[None, :]
    codes, scales, nsat = oracle.pack_nf4(row)
    assert nsat == 0 and scales[0, 0] == 0x3C00  # fp16 1.0
    assert bytes(codes[0, :8]).hex() == "1032547698badcfe"
    np.testing.assert_array_equal(oracle.unpack_nf4(codes, 64)[0], np.tile(np.arange(16), 4))
    zero = np.zeros((1, 64), np.float32)
    zc, zs, _ = oracle.pack_nf4(zero)
    assert zs[0, 0] == 0 and np.all(zc == 0x77)  # code 7 = the zero level


def test_nf4_codes_equal_bruteforce_nearest_level():
    """Away from decision boundaries the threshold code is the nearest level
    (levels from the stdlib construction; nibbles read in Python)."""
    r = rng(401)
    lv = nf_levels_stdlib(4).astype(np.float64)
    x = (r.standard_normal((48, 128)) * r.choice([1e-3, 0.05, 3.0], size=(48, 1))).astype(np.float32)
    codes, scales, _ = oracle.pack_nf4(x)
    s = scales.astype(np.uint16).view(np.float16).astype(np.float64)
    checked = 0
    for row in range(48):
        c = [(codes[row, i // 2] >> (4 * (i % 2))) & 15 for i in range(128)]
        for i in range(128):
            t = float(x[row, i]) / s[row, i // 64]
            dist = np.abs(t - lv)
            order = np.argsort(dist)
            if dist[order[1]] - dist[order[0]] < 1e-5:
                continue
            assert c[i] == order[0], (row, i, t)
            checked += 1
    assert checked > 6000


def test_nf4_roundtrip_requantises_and_error_bound():
    r = rng(402)
    x = (r.standard_normal((20, 256)) * 0.05).astype(np.float32)
    codes, scales, _ = oracle.pack_nf4(x)
    xh = oracle.dequant_nf4(codes, scales, 256)
    c2, s2, _ = oracle.pack_nf4(xh.astype(np.float32))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    lv = oracle.nf4_levels().astype(np.float64)
    half_gap = np.max(np.diff(lv)) / 2
    s = np.repeat(np.array([[oracle.f16_to_f32(int(v)) for v in row] for row in scales]), 64, axis=1)
    assert np.all(np.abs(xh - x) <= half_gap * s * (1 + 1e-6) + 1e-12)


def test_int8_pack_worked_example_ties_to_even():
    # absmax 127 -> s = 1 exactly; codes are x rounded half to even
    row = np.array([[127.0, -127.0, 63.5, 62.5, 0.5, 1.5, -2.5, -0.49] + [0.0] * 56], np.float32)
    codes, scales = oracle.pack_int8(row)
    assert scales[0] == 1.0
    assert codes[0, :8].tolist() == [127, -127, 64, 62, 0, 2, -2, 0]
    zc, zs = oracle.pack_int8(np.zeros((2, 64), np.float32))
    assert np.all(zs == 0) and np.all(zc == 0)


def test_int8_pack_matches_numpy_ieee_division():
    r = rng(403)
    x = (r.standard_normal((30, 192)) * 0.04).astype(np.float32)
    codes, scales = oracle.pack_int8(x)
    s_ref = np.abs(x).max(axis=1) / np.float32(127.0)          # float32 IEEE division
    q_ref = np.clip(np.rint(x / s_ref[:, None]), -127, 127)    # float32 division, rint ties to even
    np.testing.assert_array_equal(scales, s_ref.astype(np.float32))
    np.testing.assert_array_equal(codes.astype(np.float64), q_ref)
    xh = oracle.dequant_int8(codes, scales)
    assert np.all(np.abs(xh - x) <= scales[:, None].astype(np.float64) * (0.5 + 1e-6))
    bf = synth.f32_to_bf16_bits(x)
    cb, sb = oracle.pack_int8(bf)                                # bf16 input is upcast exactly
    c32, s32 = oracle.pack_int8(synth.bf16_bits_to_f32(bf))
    np.testing.assert_array_equal(cb, c32)
    np.testing.assert_array_equal(sb, s32)


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_quantised_combine_matches_independent_decode(fmt):
    r = rng(404)
    V, N, D, T = 50, 3, 128, 11
    table = (r.standard_normal((V, N, D)) * 0.05).astype(np.float32)
    ids = r.integers(0, V, size=T, dtype=np.int64)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = (r.standard_normal((N, D)) * 0.1).astype(np.float32)
    g = scipy.special.softmax(as_f64(h) @ as_f64(w_r).T, axis=1)
    if fmt == "nf4":
        codes, scales, _ = oracle.pack_nf4(table)
        lv = oracle.nf4_levels().astype(np.float64)
        nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(V, N, D)   # independent nibble decode
        s = np.array([[[oracle.f16_to_f32(int(v)) for v in row] for row in plane] for plane in scales])
        xh = lv[nib] * np.repeat(s, 64, axis=2)
        got = oracle.lookup_combine_nf4(ids, h, w_r, codes, scales)
    else:
        codes, scales = oracle.pack_int8(table)
        xh = codes.astype(np.float64) * scales[..., None].astype(np.float64)
        got = oracle.lookup_combine_int8(ids, h, w_r, codes, scales)
    ref = np.einsum("te,ted->td", g, xh[ids])
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


# ----------------------------------------------------------------------------
# Training mode (training section: each routed expert reads the token's
# shallow embedding, every expert is active, the router reads h)
# ----------------------------------------------------------------------------

def train_inputs(seed, V=12, D=8, F=10, N=3, T=7):
    r = rng(seed)
    f = lambda shape, s: (r.standard_normal(shape) * s).astype(np.float32)
    return (r.integers(0, V, size=T).astype(np.int64), f((V, D), 1.0), f((N, F, D), 0.4), f((N, D, F), 0.3),
            f((T, D), 1.0), f((N, D), 0.5))


def test_train_forward_matches_numpy_and_the_lookup_path():
    ids, emb, wu, wd, h, wr = train_inputs(501)
    y = oracle.train_forward(ids, emb, wu, wd, h, wr)
    E = emb.astype(np.float64)[ids]
    g = scipy.special.softmax(h.astype(np.float64) @ wr.astype(np.float64).T, axis=1)
    ref = np.zeros_like(y)
    for e in range(wu.shape[0]):
        u = E @ wu[e].astype(np.float64).T
        ref += g[:, e:e + 1] * ((0.5 * u * (1 + scipy.special.erf(u / np.sqrt(2)))) @ wd[e].astype(np.float64).T)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # the inference path: the same function through the reparameterised table
    lut = oracle.build_lut_rows(emb, wu, wd).astype(np.float32)
    y_lut = oracle.lookup_combine(ids, h, wr, lut)
    assert np.abs(y - y_lut).max() <= 1e-6 * np.abs(ref).max()  # the table is stored in fp32 here


def torch_grads(ids, emb, wu, wd, h, wr, dy):
    """Reference gradients from torch.autograd in float64 on the CPU."""
    t = {k: torch.tensor(v.astype(np.float64), requires_grad=True)
         for k, v in dict(emb=emb, wu=wu, wd=wd, h=h, wr=wr).items()}
    x = t["emb"][torch.from_numpy(ids)]
    g = torch.softmax(t["h"] @ t["wr"].T, dim=1)
    y = 0
    for e in range(wu.shape[0]):
        u = x @ t["wu"][e].T
        y = y + g[:, e:e + 1] * (torch.nn.functional.gelu(u) @ t["wd"][e].T)
    (y * torch.from_numpy(dy)).sum().backward()
    return {"d_emb": t["emb"].grad.numpy(), "d_w_up": t["wu"].grad.numpy(), "d_w_down": t["wd"].grad.numpy(),
            "d_h": t["h"].grad.numpy(), "d_w_r": t["wr"].grad.numpy()}


def test_train_backward_matches_torch_autograd():
    ids, emb, wu, wd, h, wr = train_inputs(502)
    ids[3] = ids[1]  # a repeated id: its embedding gradient sums over both tokens
    dy = rng(503).standard_normal((ids.size, emb.shape[1]))
    got = oracle.train_backward(ids, emb, wu, wd, h, wr, dy)
    ref = torch_grads(ids, emb, wu, wd, h, wr, dy)
    for k in ref:
        assert np.abs(got[k] - ref[k]).max() <= 1e-10 * max(1.0, np.abs(ref[k]).max()), k


def test_train_backward_matches_finite_differences():
    """Central differences of the forward on a few coordinates of every input
    (a step of 2^-10 applied to fp32 storage, divided by the step actually
    taken)."""
    ids, emb, wu, wd, h, wr = train_inputs(504, V=6, D=4, F=5, N=2, T=3)
    dy = rng(505).standard_normal((ids.size, emb.shape[1]))
    got = oracle.train_backward(ids, emb, wu, wd, h, wr, dy)
    step = np.float32(2.0 ** -10)
    def loss(**kw):
        a = dict(emb=emb, wu=wu, wd=wd, h=h, wr=wr)
        a.update(kw)
        return float((oracle.train_forward(ids, a["emb"], a["wu"], a["wd"], a["h"], a["wr"]) * dy).sum())
    for name, arr, gkey in (("emb", emb, "d_emb"), ("wu", wu, "d_w_up"), ("wd", wd, "d_w_down"),
                            ("h", h, "d_h"), ("wr", wr, "d_w_r")):
        flat = np.random.Generator(np.random.PCG64(506)).choice(arr.size, size=min(6, arr.size), replace=False)
        if name == "emb":
            flat = np.array([ids[0] * arr.shape[1] + 1, ids[2] * arr.shape[1]])  # rows the batch uses
        for i in flat:
            p, m = arr.copy(), arr.copy()
            p.flat[i] += step
            m.flat[i] -= step
            fd = (loss(**{name: p}) - loss(**{name: m})) / (float(p.flat[i]) - float(m.flat[i]))
            assert abs(fd - got[gkey].flat[i]) <= 1e-5 * max(1.0, abs(fd)), (name, i, fd, got[gkey].flat[i])


def test_train_backward_zero_upstream_and_untouched_rows():
    ids, emb, wu, wd, h, wr = train_inputs(507)
    zero = oracle.train_backward(ids, emb, wu, wd, h, wr, np.zeros((ids.size, emb.shape[1])))
    assert all(np.all(v == 0) for v in zero.values())
    got = oracle.train_backward(ids, emb, wu, wd, h, wr, np.ones((ids.size, emb.shape[1])))
    untouched = np.setdiff1d(np.arange(emb.shape[0]), ids)
    assert np.all(got["d_emb"][untouched] == 0)


# ---------------------------------------------------------------------------
# Exact ties at the decision thresholds (results section: 3-bit table; the
# threshold rule fixed for this build is code = #{j : x > fp32(mid_j * s)},
# strict, so an element equal to a threshold takes the lower code).  Inputs
# and expected bytes are literals: the fp32 bit patterns of the midpoints
# (pinned against exact fractions by the midpoint tests above), of their
# products with the fp16 scale 0x2E66 (= 0.0999755859375) rounded once to
# fp32, and of their fp32 neighbours; the codes follow from the rule by
# hand, and the bytes from packing those codes LSB-first.
# ---------------------------------------------------------------------------
def f32s(*hexes):
    return [struct.unpack("<f", struct.pack("<I", h))[0] for h in hexes]


def next_up(x):
    return float(np.nextafter(np.float32(x), np.float32(np.inf)))


def next_down(x):
    return float(np.nextafter(np.float32(x), np.float32(-np.inf)))


NF3_MID_S1 = f32s(0xbf447ba0, 0xbec82e26, 0xbdfcdb98, 0x3dbbbcd2, 0x3e90b990, 0x3f00a32c, 0x3f4fbdff)
# fp32(mid_j * 0.0999755859375)
NF3_THR_S = f32s(0xbd9d25e0, 0xbd201ae9, 0xbc4a3ca2, 0x3c162745, 0x3ce780d4, 0x3d4dc503, 0x3da62736)
NF4_MID_S1 = f32s(0xbf591cd8, 0xbf1c5270, 0xbeeb847d, 0xbeadea74, 0xbe703cea, 0xbe0d38b9, 0xbd3a7869,
                  0x3d22fb01, 0x3df64860, 0x3e5067dc, 0x3e9582d2, 0x3ec753f6, 0x3f006d02, 0x3f248dac,
                  0x3f5c89d8)
NF4_THR_S = f32s(0xbdada5d2, 0xbd7a0dde, 0xbd3c5e37, 0xbd0b1944, 0xbcc024b8, 0xbc61e63c, 0xbb9523ce,
                 0x3b825a41, 0x3c44fa63, 0x3ca6af11, 0x3cef28c3, 0x3d1f6c67, 0x3d4d6e5f, 0x3d839c4f,
                 0x3db06340)
S_FP16_BITS = 0x2E66  # fp16 nearest to 0.1, exactly 0.0999755859375


def tie_blocks(mid_s1, thr_s):
    """Two 64-element blocks.  Block A: absmax 1.0 (scale 0x3C00, thresholds
    = the midpoints), then for each j: mid_j, its upper and its lower fp32
    neighbour.  Block B: absmax -0.0999755859375 (scale 0x2E66), then for
    each j: the threshold fp32(mid_j * s) and its upper neighbour.  The rest
    are zeros."""
    a = [1.0]
    for m in mid_s1:
        a += [m, next_up(m), next_down(m)]
    b = [-0.0999755859375]
    for t in thr_s:
        b += [t, next_up(t)]
    a += [0.0] * (64 - len(a))
    b += [0.0] * (64 - len(b))
    return np.array([a + b], dtype=np.float32)


def test_nf3_exact_threshold_ties_take_the_lower_code():
    x = tie_blocks(NF3_MID_S1, NF3_THR_S)
    assert x[0, 0] == 1.0 and abs(x[0, 64]) == np.float32(0.0999755859375)
    codes, scales, nsat = oracle.pack_nf3(x)
    assert nsat == 0 and scales.tolist() == [[0x3C00, S_FP16_BITS]]
    c = read_codes_python(codes[0], 128)
    # block A: 1.0 -> 7; (tie, above, below) at mid_j -> (j, j+1, j); zeros -> 3
    assert c[:22] == [7, 0, 1, 0, 1, 2, 1, 2, 3, 2, 3, 4, 3, 4, 5, 4, 5, 6, 5, 6, 7, 6]
    # block B: -s -> 0; (tie, above) at thr_j -> (j, j+1)
    assert c[64:79] == [0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7]
    assert set(c[22:64]) == {3} and set(c[79:]) == {3}
    assert bytes(codes[0]).hex() == (
        "471045d33896757d6fdbb66ddbb66ddbb66ddbb66ddbb66d"
        "40226d646b7fdbb66ddbb66ddbb66ddbb66ddbb66ddbb66d")


def test_nf4_exact_threshold_ties_take_the_lower_code():
    x = tie_blocks(NF4_MID_S1, NF4_THR_S)
    codes, scales, nsat = oracle.pack_nf4(x)
    assert nsat == 0 and scales.tolist() == [[0x3C00, S_FP16_BITS]]
    c = [(int(codes[0, i // 2]) >> (4 * (i % 2))) & 15 for i in range(128)]
    assert c[:46] == [15] + [v for j in range(15) for v in (j, j + 1, j)]
    assert c[64:95] == [0] + [v for j in range(15) for v in (j, j + 1)]
    assert set(c[46:64]) == {7} and set(c[95:]) == {7}
    assert bytes(codes[0]).hex() == (
        "0f01212123434345656567878789a9a9abcbcbcdededef777777777777777777"
        "00112233445566778899aabbccddee7f77777777777777777777777777777777")


def test_tie_literals_are_the_oracles_midpoints_and_products():
    """The literal thresholds above are the midpoints the encoder uses and
    their single-rounding fp32 products with the fp16 scale."""
    s = np.float32(np.array([S_FP16_BITS], np.uint16).view(np.float16)[0])
    for mids, lit_s1, lit_s in ((oracle.nf3_midpoints(), NF3_MID_S1, NF3_THR_S),
                                (oracle.nf4_midpoints(), NF4_MID_S1, NF4_THR_S)):
        np.testing.assert_array_equal(np.asarray(mids, np.float32), np.array(lit_s1, np.float32))
        for m, t in zip(lit_s1, lit_s):
            exact = Fraction(m) * Fraction(float(s))
            assert np.float32(t) == np.float32(float(exact))  # one rounding of the exact product
