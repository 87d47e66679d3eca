"""C-ABI checks that need no GPU: libmole.so loads, exports every function
include/mole.h declares, and rejects bad arguments on the host (no kernel
is launched on any of these paths)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mixture_lookup_experts_amd as mole
from mixture_lookup_experts_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mole.h")

OK, NULL, DIM, DTYPE, ALIGN, WS, UNSUP, HIP, BADID, IO, FORMAT, HOST, MEMORY = (0, -1, -2, -3, -4, -5, -6, -7, -8, -9,
                                                                   -10, -11, -12)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mole_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mole.library()


def test_header_declares_the_hot_path():
    names = declared_functions()
    for fn in ("mole_build_lut", "mole_lookup_combine", "mole_pack_nf3", "mole_lookup_combine_nf3",
               "mole_build_lut_workspace_size", "mole_gather_nf3_host",
               "mole_lookup_combine_nf3_host", "mole_nf3_host_staging_size", "mole_status_string",
               "mole_last_hip_error",
               "mole_nf3_levels", "mole_abi_version", "mole_layer_forward",
               "mole_layer_workspace_size", "mole_nf4_levels", "mole_pack_nf4", "mole_lookup_combine_nf4",
               "mole_pack_int8", "mole_lookup_combine_int8", "mole_train_index", "mole_train_workspace_size",
               "mole_train_forward", "mole_train_backward", "mole_nf3_file_write", "mole_nf3_file_shape",
               "mole_gather_nf3_file", "mole_lookup_combine_nf3_file", "mole_lookup_combine_grouped",
               "mole_lookup_combine_grouped_workspace_size", "mole_check_ids", "mole_release_host_state",
               "mole_nf3_midpoints", "mole_nf4_midpoints", "mole_gelu_phi_coefficients",
               "mole_lookup_combine_nf3_mapped", "mole_lookup_combine_mapped",
               "mole_lookup_combine_grouped_mapped", "mole_lookup_combine_nf3_grouped",
               "mole_lookup_combine_nf3_grouped_mapped"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.mole_abi_version() == 12


def test_every_exported_function_is_declared():
    """The reverse of the export check: the library exports no mole_*
    function that include/mole.h does not declare (nm over the built
    library's dynamic symbol table)."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm is not installed")
    out = subprocess.run(["nm", "-D", "--defined-only", _native.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {f[2] for f in (line.split() for line in out.splitlines())
                if len(f) == 3 and f[1] == "T" and f[2].startswith("mole_")}
    assert exported == set(declared_functions())


def test_status_strings(lib):
    for code in (OK, NULL, DIM, DTYPE, ALIGN, WS, UNSUP, HIP, BADID, IO, FORMAT, HOST, MEMORY):
        assert mole.mole_status_string(code) not in ("", "unknown status")
    assert mole.mole_status_string(12345) == "unknown status"


def nf_levels_stdlib(k):
    """NormalFloat levels at k bits from the stdlib normal quantile: Phi^-1 at
    2^(k-1) evenly spaced probabilities from p* down to 1/2 (1/2 dropped) for
    the positive side, 2^(k-1) - 1 for the negative side, p* = 1 -
    (1/(2(2^k - 1)) + 1/2^(k+1)) / 2, one exact zero, normalised by the
    maximum, fp32."""
    from statistics import NormalDist
    nd = NormalDist()
    half = 2 ** (k - 1)
    p = 1 - 0.5 * (1 / (2 * (2 ** k - 1)) + 1 / (2 * 2 ** k))
    pos = [nd.inv_cdf(x) for x in np.linspace(p, 0.5, half + 1)[:-1]]
    neg = [-nd.inv_cdf(x) for x in np.linspace(p, 0.5, half)[:-1]]
    v = sorted(pos + [0.0] + neg)
    return np.array([x / max(v) for x in v], dtype=np.float32)


def rne_midpoints(levels):
    """fp32 nearest-even rounding of the exact midpoint of neighbouring levels."""
    from fractions import Fraction
    return np.array([float((Fraction(float(a)) + Fraction(float(b))) / 2) for a, b in zip(levels, levels[1:])],
                    dtype=np.float32)


@pytest.mark.parametrize("k", [3, 4])
def test_library_codebooks_are_the_normalfloat_construction(lib, k):
    """The level and threshold tables the kernels read (copied out by the
    host helpers from the same arrays) against the construction done here
    with the stdlib, and the thresholds against exact midpoints."""
    levels = np.array(mole.mole_nf3_levels() if k == 3 else mole.mole_nf4_levels(), np.float32)
    np.testing.assert_array_equal(levels, nf_levels_stdlib(k))
    out = (ctypes.c_float * (2 ** k - 1))()
    fn = lib.mole_nf3_midpoints if k == 3 else lib.mole_nf4_midpoints
    assert fn(ctypes.addressof(out)) == OK
    np.testing.assert_array_equal(np.array(list(out), np.float32), rne_midpoints(levels))
    assert fn(None) == NULL
    import oracle
    np.testing.assert_array_equal(levels, oracle.nf3_levels() if k == 3 else oracle.nf4_levels())


def phi_fit():
    """The least-squares fit behind the bf16 GELU: Phi(u) - 1/2 on 4000
    Chebyshev nodes of [-4, 4] in the odd basis s^(2k+1), s = u/4, k < 10,
    solved in fp64 and rounded to fp32."""
    from scipy.special import ndtr
    x = np.cos(np.pi * (np.arange(4000) + 0.5) / 4000) * 4.0
    s = x / 4.0
    basis = np.stack([s ** (2 * k + 1) for k in range(10)], axis=1)
    c, *_ = np.linalg.lstsq(basis, ndtr(x) - 0.5, rcond=None)
    return c


def phi_poly_f32(u, c, rng_):
    """fp32 evaluation as the kernels do it: clamp, Horner with fused
    multiply-adds (one rounding each: the fp64 product of two fp32 values is
    exact), clamp to [0, 1]."""
    f32 = np.float32
    s = np.clip(np.asarray(u, f32), -rng_, rng_) * f32(1.0 / rng_)
    s2 = (s * s).astype(f32)
    p = np.full_like(s, c[-1])
    for k in range(len(c) - 2, -1, -1):
        p = (p.astype(np.float64) * s2 + np.float64(c[k])).astype(f32)
    return np.clip((s.astype(np.float64) * p + 0.5).astype(f32), 0, 1)


def test_gelu_phi_coefficients_are_the_fit_and_within_bound(lib):
    from scipy.special import ndtr
    c = (ctypes.c_float * 10)()
    r = ctypes.c_float(0)
    assert lib.mole_gelu_phi_coefficients(ctypes.addressof(c), 9, ctypes.byref(r)) == DIM
    assert lib.mole_gelu_phi_coefficients(None, 10, ctypes.byref(r)) == NULL
    assert lib.mole_gelu_phi_coefficients(ctypes.addressof(c), 10, ctypes.byref(r)) == OK
    coef = np.array(list(c), np.float32)
    assert r.value == 4.0
    # every coefficient is the fit's fp32 value, bit for bit
    fit = phi_fit()
    np.testing.assert_array_equal(coef, fit.astype(np.float32))
    u = np.linspace(-4, 4, 400001).astype(np.float32)
    err_in = np.abs(phi_poly_f32(u, coef, 4.0) - ndtr(u.astype(np.float64))).max()
    assert err_in <= 1e-5, err_in
    # outside: the argument is clamped, so the value is the one at +-4
    out = np.concatenate([np.linspace(-30, -4, 1001), np.linspace(4, 30, 1001)]).astype(np.float32)
    v = phi_poly_f32(out, coef, 4.0)
    edge = phi_poly_f32(np.array([-4.0, 4.0], np.float32), coef, 4.0)
    assert np.all(v[:1001] == edge[0]) and np.all(v[1001:] == edge[1])
    assert np.abs(v - ndtr(out.astype(np.float64))).max() <= 3.6e-5  # 1 - Phi(4) + the fit's error at 4
    # GELU = u * Phi(u) at textbook points (Phi(1) = 0.8413447460685429)
    assert abs(float(phi_poly_f32(np.array([1.0], np.float32), coef, 4.0)[0]) - 0.8413447460685429) < 1e-5


def test_release_host_state(lib):
    """The gather pool and staging events are released and re-created on
    use (host-only gathers, no GPU call)."""
    assert lib.mole_release_host_state() == OK
    V, N, D, T = 2048, 4, 256, 900
    r = np.random.default_rng(5)
    codes = r.integers(0, 256, (V, N, 3 * D // 8), dtype=np.uint8)
    scales = r.integers(0, 2 ** 15, (V, N, D // 64), dtype=np.uint16)
    ids = r.integers(0, V, T).astype(np.int64)
    for _ in range(2):
        cs = np.zeros((T, N, 3 * D // 8), np.uint8)
        ss = np.zeros((T, N, D // 64), np.uint16)
        remap = np.zeros(T, np.int64)
        nu = ctypes.c_int64(0)
        rc = lib.mole_gather_nf3_host(ids.ctypes.data, T, codes.ctypes.data, scales.ctypes.data, V, N, D,
                                      cs.ctypes.data, ss.ctypes.data, remap.ctypes.data, ctypes.byref(nu), 8)
        assert rc == OK
        U = nu.value
        uniq = np.array(list(dict.fromkeys(ids.tolist())), np.int64)
        assert U == len(uniq)
        np.testing.assert_array_equal(cs[:U], codes[uniq])
        np.testing.assert_array_equal(ss[:U], scales[uniq])
        np.testing.assert_array_equal(uniq[remap], ids)
        assert lib.mole_release_host_state() == OK


def test_workspace_size(lib):
    mn, rec = mole.mole_build_lut_workspace_size(50304, 1024, 4096, 16)
    assert mn == 256 * 16 * 4096 * 2
    assert rec >= mn and rec % (16 * 4096 * 2) == 0
    mn, rec = mole.mole_build_lut_workspace_size(512, 64, 256, 4, dtype=0)
    assert mn == 0 and rec == 0
    with pytest.raises(mole.MoleError) as e:
        mole.mole_build_lut_workspace_size(0, 64, 256, 4)
    assert e.value.status == DIM
    with pytest.raises(mole.MoleError) as e:
        mole.mole_build_lut_workspace_size(8, 64, 256, 4, dtype=7)
    assert e.value.status == DTYPE


def P(x):
    return ctypes.c_void_p(x)


def test_combine_argument_errors(lib):
    a = 0x1000  # never dereferenced: every case fails validation first
    f = lib.mole_lookup_combine
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, 64, 4, 2, None) == DTYPE
    assert f(None, P(a), P(a), P(a), P(a), 4, 10, 64, 4, 1, None) == NULL
    assert f(P(a), P(a), P(a), P(a), P(a), -1, 10, 64, 4, 1, None) == DIM
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 0, 64, 4, 1, None) == DIM
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, 0, 4, 1, None) == DIM
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, 64, 65, 1, None) == UNSUP
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, (1 << 20) + 8, 4, 1, None) == UNSUP
    assert f(P(a), P(a + 4), P(a), P(a), P(a), 4, 10, 64, 4, 1, None) == ALIGN
    assert f(None, None, None, None, None, 0, 10, 64, 4, 1, None) == OK  # empty batch: no-op


def test_nf3_argument_errors(lib):
    a = 0x1000
    assert lib.mole_pack_nf3(P(a), P(a), P(a), 10, 4, 96, 1, None) == DIM
    assert lib.mole_pack_nf3(None, P(a), P(a), 10, 4, 128, 1, None) == NULL
    assert lib.mole_pack_nf3(P(a), P(a), P(a + 2), 10, 4, 128, 1, None) == ALIGN
    g = lib.mole_lookup_combine_nf3
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, 10, 96, 4, 1, None) == DIM
    assert g(P(a), P(a), P(a), P(a), None, P(a), 4, 10, 128, 4, 1, None) == NULL
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, 10, 128, 4, 5, None) == DTYPE


def test_mapped_nf3_argument_errors(lib):
    """The in-place host-table combine validates like the device one before
    it queries the table's memory (no HIP call on any of these paths)."""
    a = 0x1000
    g = lib.mole_lookup_combine_nf3_mapped
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, 10, 96, 4, 1, None) == DIM
    assert g(P(a), P(a), P(a), None, P(a), P(a), 4, 10, 128, 4, 1, None) == NULL
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, 10, 128, 4, 5, None) == DTYPE
    assert g(P(a), P(a), P(a), P(a + 8), P(a), P(a), 4, 10, 128, 4, 1, None) == ALIGN
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, 10, 128, 65, 1, None) == UNSUP
    assert g(None, None, None, None, None, None, 0, 10, 128, 4, 1, None) == OK  # empty batch: no-op
    f = lib.mole_lookup_combine_mapped
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, 64, 4, 2, None) == DTYPE
    assert f(P(a), P(a), P(a), None, P(a), 4, 10, 64, 4, 1, None) == NULL
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 0, 64, 4, 1, None) == DIM
    assert f(P(a), P(a), P(a), P(a + 8), P(a), 4, 10, 64, 4, 1, None) == ALIGN
    assert f(P(a), P(a), P(a), P(a), P(a), 4, 10, 64, 65, 1, None) == UNSUP
    assert f(None, None, None, None, None, 0, 10, 64, 4, 1, None) == OK
    # a vocabulary whose table byte count would wrap around int64
    huge = 2 ** 62
    assert g(P(a), P(a), P(a), P(a), P(a), P(a), 4, huge, 128, 4, 1, None) == DIM
    assert f(P(a), P(a), P(a), P(a), P(a), 4, huge, 64, 4, 1, None) == DIM


def test_host_staging_size_and_errors(lib):
    """Staging layout of the host-resident combine: remap int64[T], then U
    rows of codes and of fp16 scales, each section 16-byte aligned (sized
    for U = T).  Errors are reported before any GPU call."""
    T, N, D = 7, 3, 128
    want = (T * 8 + 15) // 16 * 16 + (T * N * 3 * D // 8 + 15) // 16 * 16 + T * N * (D // 64) * 2
    assert mole.mole_nf3_host_staging_size(T, N, D) == want
    out = ctypes.c_size_t(0)
    assert lib.mole_nf3_host_staging_size(T, N, 96, ctypes.addressof(out)) == DIM
    assert lib.mole_nf3_host_staging_size(T, N, D, None) == NULL
    a = 0x1000
    f = lib.mole_lookup_combine_nf3_host
    args = lambda stage_bytes, stage=P(a): (P(a), P(a), P(a), P(a), P(a), stage, P(a), stage_bytes, P(a),
                                            T, 100, D, N, 1, 0, None, None)
    assert f(*args(want - 1)) == WS  # too small: rejected before touching the stream
    assert f(*args(want, None)) == NULL
    assert f(*args(want, P(a + 8))) == ALIGN


def test_host_stack_staging_size_and_errors(lib):
    """Layer-stack prefetch: remap int64[T], then per layer U rows of codes
    and of fp16 scales, each section 16-byte aligned (sized for U = T).
    Errors are reported before any GPU call."""
    T, L, N, D = 5, 3, 4, 128
    r16 = lambda x: (x + 15) // 16 * 16
    want = r16(T * 8) + L * (r16(T * N * 3 * D // 8) + r16(T * N * (D // 64) * 2))
    assert mole.mole_nf3_host_stack_staging_size(T, L, N, D) == want
    out = ctypes.c_size_t(0)
    assert lib.mole_nf3_host_stack_staging_size(T, 0, N, D, ctypes.addressof(out)) == DIM
    assert lib.mole_nf3_host_stack_staging_size(T, L, N, 96, ctypes.addressof(out)) == DIM
    a = 0x1000
    tabs = (ctypes.c_void_p * L)(a, a, a)
    nul = (ctypes.c_void_p * L)(a, None, a)
    off = (ctypes.c_size_t * L)()
    f = lib.mole_prefetch_nf3_host_stack
    call = lambda codes=tabs, stage=P(a), nbytes=want, n=N: f(
        P(a), T, ctypes.addressof(codes), ctypes.addressof(tabs), L, 100, n, D, stage, P(a), nbytes,
        ctypes.addressof(off), ctypes.addressof(off), 0, None, None)
    assert call(nbytes=want - 1) == WS
    assert call(codes=nul) == NULL
    assert call(stage=P(a + 4)) == ALIGN
    assert call(n=65) == DIM


def test_build_argument_errors(lib):
    a = 0x1000
    b = lib.mole_build_lut
    assert b(P(a), P(a), P(a), P(a), 8, 64, 256, 4, 1, P(a), 10, None) == WS
    assert b(P(a), P(a), P(a), P(a), 8, 60, 256, 4, 1, P(a), 1 << 40, None) == DIM
    assert b(P(a), P(a), P(a), P(a), 8, 64, 256, 4, 1, None, 1 << 40, None) == NULL
    assert b(P(a), P(a), P(a), P(a + 8), 8, 64, 256, 4, 1, P(a), 1 << 40, None) == ALIGN
    assert b(P(a), P(a), P(a), P(a), 8, 64, 20000, 4, 0, None, 0, None) == UNSUP
    assert b(P(a), P(a), P(a), P(a), 8, 64, 256, 4, 3, None, 0, None) == DTYPE
    # bf16 panels are addressed with 32-bit offsets: N*F or N*D above 2^22 is refused
    assert b(P(a), P(a), P(a), P(a), 8, 64, 1 << 17, 64, 1, P(a), 1 << 40, None) == UNSUP
    assert b(P(a), P(a), P(a), P(a), 8, 1 << 17, 64, 64, 1, P(a), 1 << 40, None) == UNSUP
    assert b(P(a), P(a), P(a), P(a), 8, 64, 1 << 16, 64, 1, P(a), 10, None) == WS  # 2^22 itself is fine


def gather_inputs(seed, V=50, N=3, D=128, T=40):
    r = np.random.Generator(np.random.PCG64(seed))
    codes = r.integers(0, 256, size=(V, N, 3 * D // 8), dtype=np.uint8)
    scales = r.integers(0, 1 << 15, size=(V, N, D // 64), dtype=np.uint16)
    ids = r.integers(0, V, size=T).astype(np.int64)
    return codes, scales, ids


def test_host_gather_dedupes_and_copies_rows(lib):
    import torch
    codes, scales, ids = gather_inputs(7)
    T, (V, N, CB) = ids.size, codes.shape
    cs = torch.zeros(T * N * CB, dtype=torch.uint8)
    ss = torch.zeros(T * N * 2, dtype=torch.int16)
    remap = torch.zeros(T, dtype=torch.int64)
    U = mole.mole_gather_nf3_host(torch.from_numpy(ids), torch.from_numpy(codes),
                                  torch.from_numpy(scales.view(np.int16)), cs, ss, remap)
    uniq = np.unique(ids)
    assert U == uniq.size
    r = remap.numpy()
    cs = cs.numpy().reshape(T, N, CB)
    ss = ss.numpy().view(np.uint16).reshape(T, N, 2)
    # staged row remap[t] is table row ids[t]; first-occurrence order
    for t in range(T):
        np.testing.assert_array_equal(cs[r[t]], codes[ids[t]])
        np.testing.assert_array_equal(ss[r[t]], scales[ids[t]])
    first = [int(x) for x in dict.fromkeys(ids.tolist())]
    assert [int(ids[list(r).index(u)]) for u in range(U)] == first


def test_host_gather_rejects_bad_id(lib):
    import torch
    codes, scales, ids = gather_inputs(8, V=10, T=5)
    ids[3] = 10
    T, (V, N, CB) = ids.size, codes.shape
    with pytest.raises(mole.MoleError) as e:
        mole.mole_gather_nf3_host(torch.from_numpy(ids), torch.from_numpy(codes),
                                  torch.from_numpy(scales.view(np.int16)),
                                  torch.zeros(T * N * CB, dtype=torch.uint8),
                                  torch.zeros(T * N * 2, dtype=torch.int16),
                                  torch.zeros(T, dtype=torch.int64))
    assert e.value.status == BADID


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "_LIB_PATH", str(tmp_path / "libmole.so"))
    with pytest.raises(mole.MoleLibraryMissing):
        _native.library()


def test_layer_workspace_size_and_errors(lib):
    assert mole.mole_layer_workspace_size(0, 1024, 4096) == 0
    # routed y (fp32) + hidden activations (bf16) at least, growing with T
    for T in (1, 37, 256, 4096):
        ws = mole.mole_layer_workspace_size(T, 1024, 4096)
        assert ws >= T * 1024 * 4 + T * 4096 * 2
    assert mole.mole_layer_workspace_size(4096, 1024, 4096) > mole.mole_layer_workspace_size(256, 1024, 4096)
    out = ctypes.c_size_t(0)
    assert lib.mole_layer_workspace_size(-1, 64, 64, ctypes.addressof(out)) == DIM
    assert lib.mole_layer_workspace_size(4, 0, 64, ctypes.addressof(out)) == DIM
    assert lib.mole_layer_workspace_size(4, 64, 64, None) == NULL

    a = 0x1000
    ws = mole.mole_layer_workspace_size(4, 64, 256)

    def call(T=4, V=8, D=64, N=4, F=256, dtype=1, ids=P(a), x=P(a), wsp=P(a), wsb=ws, w_s_up=P(a)):
        return lib.mole_layer_forward(ids, P(a), P(a), P(a), w_s_up, P(a), x, T, V, D, N, F, dtype,
                                      wsp, wsb, None)
    assert call(dtype=0) == UNSUP          # fp32 has no layer path
    assert call(dtype=7) == DTYPE
    assert call(D=60) == DIM               # 16-byte K segments
    assert call(F=250) == DIM
    assert call(F=0) == DIM
    assert call(N=65) == UNSUP
    assert call(D=1 << 23) == UNSUP        # 32-bit panel offsets
    assert call(ids=None) == NULL
    assert call(w_s_up=None) == NULL
    assert call(wsp=None) == NULL
    assert call(x=P(a + 4)) == ALIGN
    assert call(wsb=ws - 1) == WS
    assert call(T=0, ids=None, x=None, wsp=None, wsb=0) == OK   # empty batch: no-op


def test_library_nf4_codebook_is_the_construction(lib):
    import oracle
    np.testing.assert_array_equal(np.array(mole.mole_nf4_levels(), np.float32), oracle.nf4_levels())


@pytest.mark.parametrize("fn", ["mole_pack_nf4", "mole_pack_int8"])
def test_quant_pack_argument_errors(lib, fn):
    a = 0x1000
    f = getattr(lib, fn)
    assert f(P(a), P(a), P(a), 8, 4, 96, 1, None) == DIM
    assert f(P(a), P(a), P(a), 0, 4, 128, 1, None) == DIM
    assert f(P(a), P(a), P(a), 8, 4, 128, 9, None) == DTYPE
    assert f(None, P(a), P(a), 8, 4, 128, 1, None) == NULL
    assert f(P(a), P(a + 4), P(a), 8, 4, 128, 1, None) == ALIGN


@pytest.mark.parametrize("fn", ["mole_lookup_combine_nf4", "mole_lookup_combine_int8"])
def test_quant_combine_argument_errors(lib, fn):
    a = 0x1000
    f = getattr(lib, fn)

    def call(T=4, V=8, D=128, N=4, dt=1, ids=P(a), codes=P(a), y=P(a)):
        return f(ids, P(a), P(a), codes, P(a), y, T, V, D, N, dt, None)
    assert call(D=96) == DIM
    assert call(N=65) == UNSUP
    assert call(dt=5) == DTYPE
    assert call(codes=None) == NULL
    assert call(y=P(a + 4)) == ALIGN
    assert call(T=0, ids=None, codes=None, y=None) == OK


def test_train_index_groups_tokens_by_row():
    import torch
    ids = torch.tensor([5, 2, 5, 9, 2, 5, 0], dtype=torch.int64)
    uniq, remap, row_ptr, tok = mole.mole_train_index(ids, V=10)
    assert uniq.tolist() == [5, 2, 9, 0]                   # first-occurrence order
    assert remap.tolist() == [0, 1, 0, 2, 1, 0, 3]
    assert row_ptr.tolist() == [0, 3, 5, 6, 7]
    assert tok.tolist() == [0, 2, 5, 1, 4, 3, 6]            # each row's tokens, in token order
    with pytest.raises(mole.MoleError):
        mole.mole_train_index(torch.tensor([1, 10], dtype=torch.int64), V=10)
    e_uniq, e_remap, e_ptr, e_tok = mole.mole_train_index(torch.empty(0, dtype=torch.int64), V=10)
    assert e_uniq.numel() == 0 and e_ptr.tolist() == [0]


def test_train_workspace_size_and_errors(lib):
    f, b = mole.mole_train_workspace_size(256, 150, 768, 3072, 4)
    assert f >= 150 * 768 * 2 + 150 * 4 * 3072 * 2 + 150 * 4 * 768 * 2   # X, G, table rows
    assert b > f
    assert mole.mole_train_workspace_size(0, 0, 768, 3072, 4) == (0, 0)
    a = 0x1000
    fwd = lib.mole_train_forward

    def call(T=16, U=8, V=50, D=64, F=128, N=4, dt=1, uniq=P(a), ws=P(a), wsb=1 << 40):
        return fwd(uniq, P(a), P(a), P(a), P(a), P(a), P(a), P(a), T, U, V, D, F, N, dt, ws, wsb, None)
    assert call(dt=0) == UNSUP
    assert call(dt=4) == DTYPE
    assert call(U=17) == DIM              # more rows than tokens
    assert call(U=0) == DIM
    assert call(D=60) == DIM
    assert call(N=65) == UNSUP
    assert call(F=1 << 19, N=4) == UNSUP  # N*F above 2^20
    assert call(uniq=None) == NULL
    assert call(ws=P(a + 8)) == ALIGN
    assert call(wsb=16) == WS
    assert call(T=0, U=0, uniq=None, ws=None, wsb=0) == OK
    bwd = lib.mole_train_backward
    assert bwd(P(a), P(a), P(a), P(a), P(a), P(a), P(a), P(a), P(a), 1 << 40, P(a), 16, P(a), P(a), P(a), P(a),
               P(a), 16, 8, 50, 64, 128, 4, 1, None) == WS
    assert bwd(P(a), P(a), None, P(a), P(a), P(a), P(a), P(a), P(a), 1 << 40, P(a), 1 << 40, P(a), P(a), P(a),
               P(a), P(a), 16, 8, 50, 64, 128, 4, 1, None) == NULL


# ----------------------------------------------------------------------------
# Disk tier: the NF3 table file
# ----------------------------------------------------------------------------

def write_table_file(path, codes, scales):
    import torch
    mole.mole_nf3_file_write(str(path), torch.from_numpy(codes), torch.from_numpy(scales.view(np.int16)))


def test_table_file_layout_is_the_documented_one(tmp_path):
    """The file is the 64-byte header the header file documents followed by
    one record per row (that row's codes, then its scales), byte for byte."""
    import struct
    codes, scales, _ = gather_inputs(11, V=9)
    V, N, CB = codes.shape
    D = CB * 8 // 3
    p = tmp_path / "t.molt"
    write_table_file(p, codes, scales)
    rec = N * CB + N * (D // 64) * 2
    want = struct.pack("<8sII6q", b"MOLENF3\0", 1, 64, V, N, D, rec, 64, 0)
    want += b"".join(codes[v].tobytes() + scales[v].astype("<u2").tobytes() for v in range(V))
    assert p.read_bytes() == want
    fd = os.open(p, os.O_RDONLY)
    try:
        assert mole.mole_nf3_file_shape(fd) == (V, N, D)
    finally:
        os.close(fd)


def test_file_gather_equals_host_gather(tmp_path):
    """Rows read from the file are the rows the host-memory gather copies,
    with the same remap and count, whatever the thread split."""
    import torch
    codes, scales, ids = gather_inputs(12, V=300, T=200)
    T, (V, N, CB) = ids.size, codes.shape
    D = CB * 8 // 3
    p = tmp_path / "t.molt"
    write_table_file(p, codes, scales)
    bufs = lambda: (torch.zeros(T * N * CB, dtype=torch.uint8), torch.zeros(T * N * (D // 64), dtype=torch.int16),
                    torch.zeros(T, dtype=torch.int64))
    hc, hs, hr = bufs()
    Uh = mole.mole_gather_nf3_host(torch.from_numpy(ids), torch.from_numpy(codes),
                                   torch.from_numpy(scales.view(np.int16)), hc, hs, hr)
    fd = os.open(p, os.O_RDONLY)
    try:
        for nthreads in (1, 4):
            fc, fs, fr = bufs()
            Uf = mole.mole_gather_nf3_file(fd, torch.from_numpy(ids), V, N, D, fc, fs, fr, nthreads=nthreads)
            assert Uf == Uh
            assert torch.equal(fr, hr)
            assert torch.equal(fc[:Uf * N * CB], hc[:Uh * N * CB])
            assert torch.equal(fs[:Uf * N * (D // 64)], hs[:Uh * N * (D // 64)])
    finally:
        os.close(fd)


def test_table_file_errors(tmp_path):
    import torch
    codes, scales, ids = gather_inputs(13, V=10, T=5)
    T, (V, N, CB) = ids.size, codes.shape
    D = CB * 8 // 3
    p = tmp_path / "t.molt"
    write_table_file(p, codes, scales)
    bufs = (torch.zeros(T * N * CB, dtype=torch.uint8), torch.zeros(T * N * (D // 64), dtype=torch.int16),
            torch.zeros(T, dtype=torch.int64))

    def status(fd, ids_=ids, V_=V):
        try:
            mole.mole_gather_nf3_file(fd, torch.from_numpy(ids_), V_, N, D, *bufs)
            return OK
        except mole.MoleError as e:
            return e.status

    fd = os.open(p, os.O_RDONLY)
    try:
        assert status(fd) == OK
        assert status(fd, V_=V + 1) == DIM                       # header shape differs
        bad = ids.copy()
        bad[2] = V
        assert status(fd, ids_=bad) == BADID
    finally:
        os.close(fd)
    assert status(-1) == IO                                     # no open file
    raw = bytearray(p.read_bytes())
    raw[0:1] = b"X"
    q = tmp_path / "bad_magic.molt"
    q.write_bytes(bytes(raw))
    fd = os.open(q, os.O_RDONLY)
    try:
        assert status(fd) == FORMAT
    finally:
        os.close(fd)
    r = tmp_path / "short.molt"                                 # records cut off
    r.write_bytes(p.read_bytes()[:64 + 3])
    fd = os.open(r, os.O_RDONLY)
    try:
        ids_last = np.array([V - 1], np.int64)
        assert status(fd, ids_=ids_last) == IO
    finally:
        os.close(fd)
    with pytest.raises(mole.MoleError) as e:
        mole.mole_nf3_file_write(str(tmp_path / "no_such_dir" / "t.molt"), torch.from_numpy(codes),
                                 torch.from_numpy(scales.view(np.int16)))
    assert e.value.status == IO


def test_gathers_from_several_threads_share_the_worker_pool(tmp_path):
    """Host gathers run on one persistent worker pool; calls from several
    threads at once (memory and file sources mixed) each get their own
    rows."""
    import threading
    import torch
    codes, scales, _ = gather_inputs(14, V=400, N=4, D=256, T=10)
    V, N, CB = codes.shape
    D = CB * 8 // 3
    p = tmp_path / "t.molt"
    write_table_file(p, codes, scales)
    fd = os.open(p, os.O_RDONLY)
    errors = []

    def job(k):
        try:
            r = np.random.Generator(np.random.PCG64(100 + k))
            for it in range(20):
                ids = r.integers(0, V, size=600).astype(np.int64)
                T = ids.size
                cs = torch.zeros(T * N * CB, dtype=torch.uint8)
                ss = torch.zeros(T * N * (D // 64), dtype=torch.int16)
                rm = torch.zeros(T, dtype=torch.int64)
                if (k + it) % 2:
                    U = mole.mole_gather_nf3_file(fd, torch.from_numpy(ids), V, N, D, cs, ss, rm, nthreads=8)
                else:
                    U = mole.mole_gather_nf3_host(torch.from_numpy(ids), torch.from_numpy(codes),
                                                  torch.from_numpy(scales.view(np.int16)), cs, ss, rm,
                                                  nthreads=8)
                r_ = rm.numpy()
                c = cs.numpy()[:U * N * CB].reshape(U, N, CB)
                assert U == np.unique(ids).size
                for t in range(0, T, 37):
                    np.testing.assert_array_equal(c[r_[t]], codes[ids[t]])
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=job, args=(k,)) for k in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    os.close(fd)
    assert not any(th.is_alive() for th in threads), "a gather did not return"
    assert not errors, errors


def test_grouped_combine_argument_errors(lib):
    """The grouped combine checks sizes, dtype, its limits and the workspace
    before any launch (no GPU is touched: every call here fails on the host)."""
    dummy = ctypes.c_void_p(16)  # never dereferenced: the calls fail before
    need = mole.mole_lookup_combine_grouped_workspace_size(8)

    def call(T=8, V=100, D=64, N=4, dtype=_native.MOLE_BF16, ptr=dummy, ws=dummy, ws_bytes=need):
        return lib.mole_lookup_combine_grouped(ptr, ptr, ptr, ptr, ptr, T, V, D, N, dtype, ws, ws_bytes, None)

    assert call(dtype=7) == DTYPE
    assert call(D=0) == DIM
    assert call(T=-1) == DIM
    assert call(dtype=_native.MOLE_F32) == UNSUP
    assert call(N=17) == UNSUP
    assert call(D=60) == UNSUP           # D % 8
    assert call(V=2 ** 31) == UNSUP      # rows are held as int32
    assert call(T=0) == OK               # empty batch: no-op
    assert call(ptr=None) == NULL
    assert call(ws=None) == NULL
    assert call(ws_bytes=need - 1) == WS
    assert call(ws=ctypes.c_void_p(24)) == ALIGN


def test_grouped_variant_argument_errors(lib):
    """The grouped read-in-place and grouped NF3 entry points validate like
    the grouped combine before any HIP call (the host-table checks, which
    query the runtime, come only after these)."""
    dummy = ctypes.c_void_p(16)
    need = mole.mole_lookup_combine_grouped_workspace_size(8)

    def gm(T=8, V=100, D=64, N=4, dtype=_native.MOLE_BF16, ptr=dummy, ws=dummy, ws_bytes=need):
        return lib.mole_lookup_combine_grouped_mapped(ptr, ptr, ptr, ptr, ptr, T, V, D, N, dtype, ws, ws_bytes, None)

    assert gm(dtype=7) == DTYPE
    assert gm(dtype=_native.MOLE_F32) == UNSUP
    assert gm(N=17) == UNSUP
    assert gm(T=0) == OK
    assert gm(ptr=None) == NULL
    assert gm(ws=None) == NULL
    assert gm(ws_bytes=need - 1) == WS
    for fn in (lib.mole_lookup_combine_nf3_grouped, lib.mole_lookup_combine_nf3_grouped_mapped):
        def ng(T=8, V=100, D=128, N=4, dtype=_native.MOLE_BF16, ptr=dummy, ws=dummy, ws_bytes=need):
            return fn(ptr, ptr, ptr, ptr, ptr, ptr, T, V, D, N, dtype, ws, ws_bytes, None)

        assert ng(dtype=7) == DTYPE
        assert ng(D=96) == DIM               # D % 64
        assert ng(dtype=_native.MOLE_F32) == UNSUP
        assert ng(N=17) == UNSUP
        assert ng(V=2 ** 31) == UNSUP
        assert ng(T=0) == OK
        assert ng(ptr=None) == NULL
        assert ng(ws=None) == NULL
        assert ng(ws_bytes=need - 1) == WS
        assert ng(ws=ctypes.c_void_p(24)) == ALIGN


def test_grouped_workspace_size():
    """Three sections, each padded to 256 bytes: the grouped token and its
    row (int32 [T] each) and the gates (fp32 [T][16])."""
    r256 = lambda x: (x + 255) // 256 * 256
    assert mole.mole_lookup_combine_grouped_workspace_size(0) == 0
    for T in (1, 64, 65, 4096, 5000):
        assert mole.mole_lookup_combine_grouped_workspace_size(T) == 2 * r256(4 * T) + r256(64 * T)
    with pytest.raises(mole.MoleError):
        mole.mole_lookup_combine_grouped_workspace_size(-1)


def test_check_ids_argument_errors(lib):
    a = ctypes.c_void_p(0x1000)
    assert lib.mole_check_ids(a, -1, 10, a, None) == DIM
    assert lib.mole_check_ids(a, 4, 0, a, None) == DIM
    assert lib.mole_check_ids(None, 4, 10, a, None) == NULL
    assert lib.mole_check_ids(a, 4, 10, None, None) == NULL
    assert lib.mole_check_ids(ctypes.c_void_p(0x1004), 4, 10, a, None) == ALIGN
    assert lib.mole_check_ids(a, 4, 10, ctypes.c_void_p(0x1002), None) == ALIGN
    assert lib.mole_check_ids(None, 0, 10, None, None) == OK
