"""GPU parity: every libmole entry point (through the C ABI) against the CPU
oracle on identical seeded inputs.

Bars (written in each test):
  * lookup-combine (bf16 or fp32 table): per token max_d |y - y_ref| /
    max_d |y_ref| <= 2e-5 (fp32 accumulation vs fp64);
  * NF3 codes and scales: bit-exact;
  * NF3 combine: same 2e-5 bar against the fp64 decode of the same codes;
  * bf16 LUT build: relative L2 error <= 1e-2 vs the fp64 oracle over the
    checked rows; fp32 build: <= 1e-5.
No oracle input or expected value comes from the GPU: tables fed to the
combine and NF3 tests are seeded synthetic arrays (or the oracle's own NF3
encoding), never a GPU-built LUT.
"""
import os

import numpy as np
import pytest
import torch

import mixture_lookup_experts_amd as mole
import oracle
from mixture_lookup_experts_amd import synth
from tests.gpu_util import bf16_to_f64, combine_rel_err, dev, host, rel_l2

pytestmark = pytest.mark.gpu

COMBINE_TOL = 2e-5


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_table(seed, V, N, D, dtype, std=0.05, rows=None):
    """Seeded synthetic table; if `rows` is given only those rows are drawn
    (the rest stay zero), which keeps full-vocabulary tables cheap."""
    r = rng(seed)
    conv = synth.f32_to_bf16_bits if dtype == "bf16" else (lambda a: a)
    if rows is None:
        return conv(r.standard_normal((V, N, D), dtype=np.float32) * np.float32(std))
    out = np.zeros((V, N, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    out[rows] = conv(r.standard_normal((len(rows), N, D), dtype=np.float32) * np.float32(std))
    return out


def rand_hw(seed, T, N, D, dtype, wstd=0.02):
    r = rng(seed)
    h = r.standard_normal((T, D), dtype=np.float32)
    w_r = r.standard_normal((N, D), dtype=np.float32) * np.float32(wstd)
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w_r)
    return h, w_r


def run_combine(ids, h, w_r, lut):
    y = torch.empty((ids.size, lut.shape[2]), dtype=torch.float32, device="cuda")
    mole.mole_lookup_combine(dev(ids), dev(h), dev(w_r), dev(lut), y)
    torch.cuda.synchronize()
    return host(y)


# ----------------------------------------------------------------------------
# lookup-combine, dense table
# ----------------------------------------------------------------------------

COMBINE_CASES = [
    # V, N, D, T, dtype
    (512, 4, 64, 64, "f32"),      # tiny workload
    (512, 4, 64, 1, "f32"),
    (300, 4, 768, 300, "bf16"),   # 160M-class width, ragged token tile
    (300, 16, 1024, 257, "bf16"),
    (200, 16, 2048, 33, "bf16"),
    (100, 1, 128, 17, "bf16"),
    (100, 3, 136, 19, "bf16"),    # N padded to 4, D not a power of two
    (64, 64, 256, 9, "bf16"),     # largest N
    (64, 32, 512, 40, "f32"),
    (50, 5, 60, 21, "bf16"),      # D % 8 != 0: element-wise path
    (50, 2, 30, 7, "f32"),
    (20, 4, 8, 70, "bf16"),       # tiny D: one chunk per row
    # T >= 2048 with several tokens per block: gates from a separate router
    # launch, staged in the output rows
    (300, 16, 1024, 2051, "bf16"),  # ragged last block and router tile
    (200, 5, 256, 3001, "bf16"),    # N padded to 8
    (100, 64, 512, 2048, "bf16"),   # largest N
    # either side of the one-token-per-workgroup limit (T = 1024); from
    # there on, tokens of 128-256 lanes go four to a workgroup of 4 G
    # threads with the matrix-core router
    (300, 16, 1024, 1023, "bf16"),
    (300, 16, 1024, 1024, "bf16"),
    (300, 16, 1024, 1025, "bf16"),  # ragged last workgroup (one token)
    (300, 16, 2048, 1024, "bf16"),  # 1B-class width: 16 wavefronts, one K batch each
    (300, 12, 2048, 1031, "bf16"),  # N padded to 16, ragged
    (300, 16, 1000, 1026, "bf16"),  # D not a multiple of the 32-wide K step
    (300, 16, 1032, 1024, "bf16"),  # 129 chunks in 256 lanes: lanes past the row, direct stores
    (200, 8, 1536, 2050, "bf16"),   # N = 8, 192 chunks per row
    (100, 1, 1024, 1024, "bf16"),   # one expert: every gate 1
    (300, 16, 1024, 4099, "bf16"),  # 410M-class width, large batch
    # rows wider than 256 lanes (D > 2048): one token per workgroup with the
    # vector router over several chunks per lane, at and past T = 1024
    (100, 16, 4096, 1024, "bf16"),
    (64, 12, 8192, 1100, "bf16"),
]


@pytest.mark.parametrize("V,N,D,T,dtype", COMBINE_CASES)
def test_combine_matches_oracle(V, N, D, T, dtype):
    seed = 1000 + V + N + D + T
    lut = rand_table(seed, V, N, D, dtype)
    h, w_r = rand_hw(seed + 1, T, N, D, dtype, wstd=0.3)
    ids = rng(seed + 2).integers(0, V, T).astype(np.int64)
    y = run_combine(ids, h, w_r, lut)
    y_ref = oracle.lookup_combine(ids, h, w_r, lut)
    assert combine_rel_err(y, y_ref) <= COMBINE_TOL


def test_combine_empty_batch_is_noop():
    lut = dev(rand_table(1, 10, 4, 64, "bf16"))
    h = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w_r = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(0, dtype=torch.int64, device="cuda")
    y = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    mole.mole_lookup_combine(ids, h, w_r, lut, y)
    torch.cuda.synchronize()


def test_combine_one_hot_gate_is_exact_row():
    """Logit gap of 1000 makes the softmax exactly one-hot in fp32, so y is
    the selected expert's row bit for bit."""
    V, N, D, T = 40, 4, 256, 12
    lut = rand_table(2, V, N, D, "bf16")
    ids = rng(3).integers(0, V, T).astype(np.int64)
    h = np.zeros((T, D), np.float32)
    h[:, 0] = 1.0
    for e_star in range(N):
        w_r = np.zeros((N, D), np.float32)
        w_r[e_star, 0] = 1000.0
        y = run_combine(ids, synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w_r), lut)
        np.testing.assert_array_equal(y, bf16_to_f64(lut[ids, e_star]).astype(np.float32))


def test_combine_zero_router_is_slab_mean():
    V, N, D, T = 40, 16, 1024, 20
    lut = rand_table(4, V, N, D, "bf16")
    ids = rng(5).integers(0, V, T).astype(np.int64)
    h, _ = rand_hw(6, T, N, D, "bf16")
    y = run_combine(ids, h, np.zeros((N, D), np.uint16), lut)
    assert combine_rel_err(y, bf16_to_f64(lut[ids]).mean(axis=1)) <= COMBINE_TOL


@pytest.mark.parametrize("name,T", [("160m", 1), ("160m", 8), ("160m", 64), ("160m", 256),
                                    ("410m", 256), ("410m", 1024), ("410m", 4096),
                                    ("1b", 1), ("1b", 16), ("1b", 128), ("1b", 1024)])
def test_combine_full_size_zipf(name, T):
    """Full vocabulary, workload widths, Zipf(1.1) ids, every token checked."""
    w = synth.WORKLOADS[name]
    ids = synth.make_ids(w, T, step=0)
    lut = rand_table(77 + w.index, w.V, w.N, w.D, "bf16", rows=np.unique(ids))
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    y = run_combine(ids, h, w_r, lut)
    y_ref = oracle.lookup_combine(ids, h, w_r, lut)
    assert combine_rel_err(y, y_ref) <= COMBINE_TOL


# ----------------------------------------------------------------------------
# NF3 pack
# ----------------------------------------------------------------------------

def run_pack(table):
    lut = dev(table)
    V, N, D = table.shape
    codes = torch.empty((V, N, 3 * D // 8), dtype=torch.uint8, device="cuda")
    scales = torch.empty((V, N, D // 64), dtype=torch.int16, device="cuda")
    mole.mole_pack_nf3(lut, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales)


@pytest.mark.parametrize("V,N,D,dtype,std", [(512, 4, 64, "f32", 0.02), (300, 4, 768, "bf16", 0.02),
                                             (100, 16, 1024, "bf16", 1.0), (33, 3, 2048, "bf16", 1e-3),
                                             (7, 1, 128, "f32", 3.0)])
def test_pack_nf3_bit_exact(V, N, D, dtype, std):
    table = rand_table(10 + D + V, V, N, D, dtype, std=std)
    codes, scales = run_pack(table)
    c_ref, s_ref, _ = oracle.pack_nf3(table)
    np.testing.assert_array_equal(scales, s_ref)
    np.testing.assert_array_equal(codes, c_ref)


def test_pack_nf3_edge_cases_bit_exact():
    """Exact threshold ties (strict compare keeps the lower code), the
    neighbouring float above each tie, zero and tiny blocks (code 3),
    fp16-subnormal scales and saturation at 65504."""
    mid = oracle.nf3_midpoints()
    lv = oracle.nf3_levels()
    rows = []
    tie = np.zeros(64, np.float32)
    tie[0] = 1.0                                   # absmax 1 -> scale exactly 1.0
    tie[1:8] = mid
    tie[8:15] = np.nextafter(mid, np.float32(2))
    tie[15:22] = np.nextafter(mid, np.float32(-2))
    tie[22:30] = lv
    tie[30] = -1.0
    rows.append(tie)
    rows.append(np.zeros(64, np.float32))
    rows.append(np.full(64, 1e-9, np.float32))
    sub = np.linspace(-3e-6, 2e-6, 64).astype(np.float32)
    rows.append(sub)
    sat = np.linspace(-1e5, 7e4, 64).astype(np.float32)
    rows.append(sat)
    half = np.linspace(-1, 1, 64).astype(np.float32) * np.float32(65519.0)
    rows.append(half)
    table = np.stack(rows).reshape(len(rows), 1, 64)
    codes, scales = run_pack(table)
    c_ref, s_ref, nsat = oracle.pack_nf3(table)
    assert nsat == 2
    np.testing.assert_array_equal(scales, s_ref)
    np.testing.assert_array_equal(codes, c_ref)


def test_pack_nf3_full_size_sampled_rows():
    """410M-class table (50304 x 16 x 1024) packed on the GPU in one launch;
    2048 seeded rows plus the first and last are re-encoded by the oracle."""
    w = synth.WORKLOADS["410m"]
    sample = np.unique(np.concatenate([[0, w.V - 1], rng(11).integers(0, w.V, 2048)]))
    table = rand_table(12, w.V, w.N, w.D, "bf16", std=0.02, rows=sample)
    codes, scales = run_pack(table)
    c_ref, s_ref, _ = oracle.pack_nf3(table[sample])
    np.testing.assert_array_equal(scales[sample], s_ref)
    np.testing.assert_array_equal(codes[sample], c_ref)
    other = np.setdiff1d(np.arange(w.V), sample)[:500]   # all-zero rows: scale 0, code 3
    assert np.all(scales[other] == 0)
    assert np.all(codes[other][..., 0::3] == 0xDB)


# ----------------------------------------------------------------------------
# NF3 combine (device table and host-resident table)
# ----------------------------------------------------------------------------

def run_nf3(ids, h, w_r, codes, scales):
    y = torch.empty((ids.size, h.shape[1]), dtype=torch.float32, device="cuda")
    mole.mole_lookup_combine_nf3(dev(ids), dev(h), dev(w_r), dev(codes), dev(scales.view(np.int16)), y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("V,N,D,T,dtype", [(512, 4, 64, 64, "f32"), (300, 4, 768, 200, "bf16"),
                                           (300, 16, 1024, 257, "bf16"), (100, 16, 2048, 33, "bf16"),
                                           (64, 64, 128, 10, "bf16"), (50, 3, 192, 17, "f32"),
                                           (40, 1, 64, 5, "bf16"),
                                           # large batches with several tokens per block
                                           (300, 16, 1024, 2051, "bf16"), (200, 5, 256, 3001, "bf16"),
                                           (100, 64, 512, 2048, "bf16"),
                                           # either side of the one-token-per-workgroup limit
                                           # (from T = 1024: four tokens per workgroup, router
                                           # operands before branch-free code loads)
                                           (300, 16, 1024, 1023, "bf16"), (300, 16, 1024, 1024, "bf16"),
                                           (300, 16, 1024, 1025, "bf16"), (200, 8, 512, 600, "bf16"),
                                           (300, 12, 1024, 1030, "bf16"),  # N padded to 16, ragged
                                           (300, 16, 2048, 1024, "bf16"),  # two batches of code loads
                                           (100, 16, 4096, 1024, "bf16"),  # two chunk rounds per lane
                                           # four wavefronts per token, some without an expert in a round
                                           (300, 12, 1024, 100, "bf16"),
                                           # large batches: four and eight tokens per workgroup with
                                           # ragged last workgroups, rows of 24 chunks in 32-lane groups
                                           (300, 16, 1024, 9001, "bf16"), (300, 4, 768, 5003, "bf16"),
                                           (300, 12, 1024, 2047, "bf16"), (300, 16, 768, 4095, "bf16")])
def test_combine_nf3_matches_oracle(V, N, D, T, dtype):
    seed = 2000 + V + N + D
    table = rand_table(seed, V, N, D, "bf16")
    codes, scales, _ = oracle.pack_nf3(table)
    h, w_r = rand_hw(seed + 1, T, N, D, dtype, wstd=0.3)
    ids = rng(seed + 2).integers(0, V, T).astype(np.int64)
    y = run_nf3(ids, h, w_r, codes, scales)
    y_ref = oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)
    assert combine_rel_err(y, y_ref) <= COMBINE_TOL


# ----------------------------------------------------------------------------
# lookup-combine over a batch grouped by id on the device
# ----------------------------------------------------------------------------

def run_grouped(ids, h, w_r, lut):
    T = ids.size
    y = torch.full((T, lut.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(mole.mole_lookup_combine_grouped_workspace_size(T), 16),), 0xAB, dtype=torch.uint8,
                    device="cuda")  # stale contents: the kernels must not rely on a cleared workspace
    mole.mole_lookup_combine_grouped(dev(ids), dev(h), dev(w_r), dev(lut), y, ws)
    torch.cuda.synchronize()
    return host(y)


def grouped_ids(r, V, T, law):
    if law == "zipf":
        return synth.zipf_ids(r, V, T, r.permutation(V))
    if law == "one":
        return np.full(T, V // 2, np.int64)
    if law == "distinct":
        return r.permutation(V)[:T].astype(np.int64)
    return r.integers(0, V, T).astype(np.int64)


# (V, N, D, T, ids): ragged T and D, N padded to a power of two, one token,
# one 64-lane group (D = 64) and one to four wavefronts per workgroup, a
# single id for every token, distinct ids only, and batches over several
# 4096-token grouping chunks (5000, 8193: a one-token last chunk), with the
# hot Zipf rows spread over many 16-position workgroups.
GROUPED_CASES = [(300, 4, 768, 300, "uniform"), (300, 16, 1024, 257, "zipf"), (200, 16, 2048, 33, "zipf"),
                 (100, 1, 128, 17, "uniform"), (100, 3, 136, 19, "zipf"), (50, 16, 1024, 3000, "zipf"),
                 (20, 8, 64, 5000, "one"), (1000, 16, 1024, 1, "uniform"), (6000, 16, 256, 5000, "distinct"),
                 (3000, 4, 512, 8193, "zipf"), (70, 16, 2048, 4096, "uniform")]


@pytest.mark.parametrize("V,N,D,T,law", GROUPED_CASES)
def test_grouped_combine_matches_oracle(V, N, D, T, law):
    seed = 2000 + V + N + D + T
    lut = rand_table(seed, V, N, D, "bf16")
    h, w_r = rand_hw(seed + 1, T, N, D, "bf16", wstd=0.3)
    ids = grouped_ids(rng(seed + 2), V, T, law)
    y = run_grouped(ids, h, w_r, lut)
    assert np.all(np.isfinite(y))
    assert combine_rel_err(y, oracle.lookup_combine(ids, h, w_r, lut)) <= COMBINE_TOL
    # the per-token combine on the same inputs, up to fp32 summation order
    assert combine_rel_err(y, run_combine(ids, h, w_r, lut).astype(np.float64)) <= COMBINE_TOL


@pytest.mark.parametrize("wl,T", [("410m", 1024), ("410m", 4096), ("1b", 1024), ("1b", 4096)])
def test_grouped_combine_full_size_zipf(wl, T):
    """410M- and 1B-class tables (D = 2048: one workgroup covers all columns),
    full vocabulary, Zipf(1.1) ids, every token checked."""
    w = synth.WORKLOADS[wl]
    ids = synth.make_ids(w, T, step=0)
    lut = rand_table(78, w.V, w.N, w.D, "bf16", rows=np.unique(ids))
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    y = run_grouped(ids, h, w_r, lut)
    assert combine_rel_err(y, oracle.lookup_combine(ids, h, w_r, lut)) <= COMBINE_TOL


def test_check_ids_counts_out_of_range():
    """Direct addressing by id: the optional device check counts the ids
    outside [0, V) (the count accumulates onto the caller's zeroed word)."""
    V = 1000
    ids = np.array([0, 999, 1000, -1, 5, 2 ** 40, 999, -(2 ** 40)] * 1000 + [3], np.int64)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    mole.mole_check_ids(dev(ids), V, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 4000
    mole.mole_check_ids(dev(np.arange(V, dtype=np.int64)), V, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 4000


@pytest.mark.parametrize("T", [256, 1024, 4096])
def test_combine_nf3_full_size_zipf(T):
    w = synth.WORKLOADS["410m-nf3"]
    ids = synth.make_ids(w, T)
    uniq = np.unique(ids)
    table = rand_table(91, w.V, w.N, w.D, "bf16", std=0.02, rows=uniq)
    codes, scales, _ = oracle.pack_nf3(table)
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    y = run_nf3(ids, h, w_r, codes, scales)
    assert combine_rel_err(y, oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)) <= COMBINE_TOL


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_combine_nf3_host_resident(T):
    """Table in pinned host memory; only the distinct requested rows cross
    PCIe.  Equal bit for bit to the device-resident combine, and to the
    oracle within the combine bar."""
    w = synth.WORKLOADS["410m-nf3"]
    V, N, D = w.V, w.N, w.D
    ids = synth.make_ids(w, T, step=3)
    uniq = np.unique(ids)
    table = rand_table(92, V, N, D, "bf16", std=0.02, rows=uniq)
    codes, scales, _ = oracle.pack_nf3(table)
    h = synth.make_hidden(w, T, step=3)
    w_r = synth.make_router(w)
    codes_h = torch.from_numpy(codes).pin_memory()
    scales_h = torch.from_numpy(scales.view(np.int16)).pin_memory()
    nbytes = mole.mole_nf3_host_staging_size(T, N, D)
    stage_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    stage_d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    ref_dev = run_nf3(ids, h, w_r, codes, scales)
    ref = oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)
    # twice in a row through the same staging area (the second call rewrites it)
    for _ in range(2):
        y.fill_(float("nan"))
        U = mole.mole_lookup_combine_nf3_host(torch.from_numpy(ids), dev(h), dev(w_r), codes_h, scales_h,
                                              stage_h, stage_d, y)
        torch.cuda.synchronize()
        assert U == uniq.size
        y_host = host(y)
        np.testing.assert_array_equal(y_host, ref_dev)
        assert combine_rel_err(y_host, ref) <= COMBINE_TOL


@pytest.mark.parametrize("wl,T", [("410m-nf3", 1), ("410m-nf3", 256), ("410m-nf3", 1024), ("410m-nf3", 4096),
                                  ("160m", 64), ("160m", 1500)])
def test_combine_nf3_mapped_host_table(wl, T):
    """Table in page-locked host memory read in place by the kernel (one
    launch, no staging).  Every launch shape of the NF3 combine (one token on
    one or several wavefronts, four and eight tokens per workgroup; the
    160M-class table's N = 4, D = 768) reads the host rows; the codes sit at
    an offset inside their pinned allocation.
    Equal bit for bit to the device-resident combine, and to the oracle
    within the combine bar; twice in a row."""
    w = synth.WORKLOADS[wl]
    V, N, D = w.V, w.N, w.D
    ids = synth.make_ids(w, T, step=5)
    table = rand_table(93, V, N, D, "bf16", std=0.02, rows=np.unique(ids))
    codes, scales, _ = oracle.pack_nf3(table)
    h = synth.make_hidden(w, T, step=5)
    w_r = synth.make_router(w)
    pool = torch.empty(codes.size + 256, dtype=torch.uint8, pin_memory=True)
    codes_h = pool[256:].view(V, N, 3 * D // 8)
    codes_h.copy_(torch.from_numpy(codes))
    scales_h = torch.from_numpy(scales.view(np.int16)).pin_memory()
    ref_dev = run_nf3(ids, h, w_r, codes, scales)
    ref = oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    for _ in range(2):
        y.fill_(float("nan"))
        mole.mole_lookup_combine_nf3_mapped(dev(ids), dev(h), dev(w_r), codes_h, scales_h, y)
        torch.cuda.synchronize()
        y_host = host(y)
        np.testing.assert_array_equal(y_host, ref_dev)
        assert combine_rel_err(y_host, ref) <= COMBINE_TOL


@pytest.mark.parametrize("V,N,D,T,dtype", [(3000, 16, 2048, 1, "bf16"), (3000, 16, 2048, 128, "bf16"),
                                           (3000, 16, 2048, 1030, "bf16"), (2000, 16, 1024, 4100, "bf16"),
                                           (2000, 8, 512, 2100, "bf16"), (300, 4, 96, 70, "f32")])
def test_combine_mapped_host_table(V, N, D, T, dtype):
    """The uncompressed table in page-locked host memory, read in place
    (one token per workgroup, the four-token wide blocks at two widths, the
    staged router's two launches at 64 lanes per token, fp32): bit for bit
    the device-resident combine, and within the oracle's bar."""
    seed = 4000 + V + N + D + T
    table = rand_table(seed, V, N, D, dtype)
    h, w_r = rand_hw(seed + 1, T, N, D, dtype, wstd=0.3)
    ids = rng(seed + 2).integers(0, V, T).astype(np.int64)
    ref_dev = run_combine(ids, h, w_r, table)
    lut_h = dev(table).cpu().pin_memory()
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    for _ in range(2):
        y.fill_(float("nan"))
        mole.mole_lookup_combine_mapped(dev(ids), dev(h), dev(w_r), lut_h, y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), ref_dev)
    assert combine_rel_err(host(y), oracle.lookup_combine(ids, h, w_r, table)) <= COMBINE_TOL
    pageable = lut_h.clone()
    assert not pageable.is_pinned()
    with pytest.raises(mole.MoleError) as e:  # the same table in pageable memory is refused
        mole.mole_lookup_combine_mapped(dev(ids), dev(h), dev(w_r), pageable, y)
    assert e.value.status == -12


@pytest.mark.parametrize("V,N,D,T,law", [(3000, 16, 1024, 4096, "zipf"), (600, 16, 2048, 1030, "zipf"),
                                         (300, 4, 768, 300, "uniform"), (20, 8, 64, 5000, "one")])
def test_grouped_combine_mapped_host_table(V, N, D, T, law):
    """The grouped combine with its bf16 table in page-locked host memory,
    read in place: bit for bit the device-resident grouped combine (each
    token's sum runs over its own gates and slab in a fixed order), and
    within the oracle's bar."""
    seed = 5000 + V + N + D + T
    lut = rand_table(seed, V, N, D, "bf16")
    h, w_r = rand_hw(seed + 1, T, N, D, "bf16", wstd=0.3)
    ids = grouped_ids(rng(seed + 2), V, T, law)
    ref_dev = run_grouped(ids, h, w_r, lut)
    lut_h = dev(lut).cpu().pin_memory()
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    ws = torch.full((max(mole.mole_lookup_combine_grouped_workspace_size(T), 16),), 0xAB, dtype=torch.uint8,
                    device="cuda")
    for _ in range(2):
        y.fill_(float("nan"))
        mole.mole_lookup_combine_grouped_mapped(dev(ids), dev(h), dev(w_r), lut_h, y, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), ref_dev)
    assert combine_rel_err(host(y), oracle.lookup_combine(ids, h, w_r, lut)) <= COMBINE_TOL


@pytest.mark.parametrize("V,N,D,T,law", [(300, 16, 1024, 4096, "zipf"), (300, 4, 768, 300, "uniform"),
                                         (100, 1, 128, 17, "uniform"), (20, 8, 64, 5000, "one"),
                                         (100, 16, 4096, 1024, "zipf"), (50, 3, 192, 2000, "zipf")])
def test_nf3_grouped_combine_matches_oracle(V, N, D, T, law):
    """NF3 combine over the batch grouped by id on the device (ragged T, N
    padded to a power of two, rows of one to 128 chunks with two chunk rounds
    at D = 4096, a single id for 5000 tokens), against the oracle and the
    per-token NF3 combine."""
    seed = 6000 + V + N + D + T
    table = rand_table(seed, V, N, D, "bf16")
    codes, scales, _ = oracle.pack_nf3(table)
    h, w_r = rand_hw(seed + 1, T, N, D, "bf16", wstd=0.3)
    ids = grouped_ids(rng(seed + 2), V, T, law)
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(mole.mole_lookup_combine_grouped_workspace_size(T), 16),), 0xAB, dtype=torch.uint8,
                    device="cuda")
    mole.mole_lookup_combine_nf3_grouped(dev(ids), dev(h), dev(w_r), dev(codes), dev(scales.view(np.int16)), y, ws)
    torch.cuda.synchronize()
    yh = host(y)
    assert np.all(np.isfinite(yh))
    assert combine_rel_err(yh, oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)) <= COMBINE_TOL
    assert combine_rel_err(yh, run_nf3(ids, h, w_r, codes, scales).astype(np.float64)) <= COMBINE_TOL


@pytest.mark.parametrize("T", [1024, 4096])
def test_nf3_grouped_combine_mapped_host_table(T):
    """The grouped NF3 combine with its 410M-class table in page-locked host
    memory, read in place: bit for bit the device-resident grouped NF3
    combine (same gates, same kernel), and within the oracle's bar."""
    w = synth.WORKLOADS["410m-nf3"]
    V, N, D = w.V, w.N, w.D
    ids = synth.make_ids(w, T, step=7)
    table = rand_table(94, V, N, D, "bf16", std=0.02, rows=np.unique(ids))
    codes, scales, _ = oracle.pack_nf3(table)
    h = synth.make_hidden(w, T, step=7)
    w_r = synth.make_router(w)
    ws = torch.empty(mole.mole_lookup_combine_grouped_workspace_size(T), dtype=torch.uint8, device="cuda")
    y_dev = torch.empty((T, D), dtype=torch.float32, device="cuda")
    mole.mole_lookup_combine_nf3_grouped(dev(ids), dev(h), dev(w_r), dev(codes), dev(scales.view(np.int16)), y_dev,
                                         ws)
    codes_h = torch.from_numpy(codes).pin_memory()
    scales_h = torch.from_numpy(scales.view(np.int16)).pin_memory()
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    for _ in range(2):
        y.fill_(float("nan"))
        mole.mole_lookup_combine_nf3_grouped_mapped(dev(ids), dev(h), dev(w_r), codes_h, scales_h, y, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(y_dev))
    assert combine_rel_err(host(y), oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)) <= COMBINE_TOL


def test_combine_nf3_mapped_refuses_unmapped_tables():
    """Pageable host memory and device memory are refused on the host before
    anything is enqueued (a kernel reading pageable memory would fault)."""
    V, N, D, T = 64, 4, 128, 8
    ids = dev(np.arange(T, dtype=np.int64))
    h = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
    w_r = torch.zeros((N, D), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((T, D), dtype=torch.float32, device="cuda")
    codes_p = torch.zeros((V, N, 3 * D // 8), dtype=torch.uint8)     # pageable
    scales_p = torch.zeros((V, N, D // 64), dtype=torch.int16)
    scales_pin = scales_p.pin_memory()
    for c, sc in ((codes_p, scales_pin), (codes_p.pin_memory(), scales_p)):
        with pytest.raises(mole.MoleError) as e:
            mole.mole_lookup_combine_nf3_mapped(ids, h, w_r, c, sc, y)
        assert e.value.status == -12
    # device memory as the "host" table: the binding refuses it, and so does the C ABI
    codes_d = codes_p.cuda()
    rc = mole.library().mole_lookup_combine_nf3_mapped(ids.data_ptr(), h.data_ptr(), w_r.data_ptr(),
                                                       codes_d.data_ptr(), scales_pin.data_ptr(), y.data_ptr(),
                                                       T, V, D, N, 1, None)
    assert rc == -12
    torch.cuda.synchronize()
    # the refused calls left no error behind for the next launch
    mole.mole_lookup_combine_nf3_mapped(ids, h, w_r, codes_p.pin_memory(), scales_pin, y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())


def test_mapped_combines_refuse_a_range_across_two_allocations():
    """A table range whose first byte lies in one page-locked allocation and
    whose last byte lies in another (both ends mapped, the memory between them
    not necessarily) is refused.  The ids touch only rows inside the first
    allocation, so no read could leave it even if a call went through."""
    T = 8
    a = torch.zeros(1 << 20, dtype=torch.uint8).pin_memory()
    b = torch.zeros(1 << 20, dtype=torch.uint8).pin_memory()
    lo, hi = (a, b) if a.data_ptr() < b.data_ptr() else (b, a)
    gap = hi.data_ptr() + 4096 - lo.data_ptr()      # from lo's first byte to a byte inside hi
    ids = dev(np.arange(T, dtype=np.int64))
    lib = mole.library()
    for fmt in ("nf3", "bf16"):
        D, N = 64, 1
        row = N * (3 * D // 8) if fmt == "nf3" else N * D * 2
        V = gap // row + 1                             # the range's last byte: 4096 .. 4096 + row - 1 into hi
        if V * 2 > (1 << 30):
            pytest.skip("the two allocations lie too far apart for a scale table of this size")
        last = lo.data_ptr() + V * row - 1
        assert hi.data_ptr() <= last < hi.data_ptr() + hi.numel()
        h = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
        w_r = torch.zeros((N, D), dtype=torch.bfloat16, device="cuda")
        y = torch.zeros((T, D), dtype=torch.float32, device="cuda")
        if fmt == "nf3":
            scales = torch.zeros((V, N, D // 64), dtype=torch.int16).pin_memory()
            rc = lib.mole_lookup_combine_nf3_mapped(ids.data_ptr(), h.data_ptr(), w_r.data_ptr(), lo.data_ptr(),
                                                    scales.data_ptr(), y.data_ptr(), T, V, D, N, 1, None)
        else:
            rc = lib.mole_lookup_combine_mapped(ids.data_ptr(), h.data_ptr(), w_r.data_ptr(), lo.data_ptr(),
                                                y.data_ptr(), T, V, D, N, 1, None)
        assert rc == -12, (fmt, rc)
    torch.cuda.synchronize()
    # the same first allocation with a range inside it goes through
    V = lo.numel() // (3 * 64 // 8)
    scales = torch.zeros((V, 1, 1), dtype=torch.int16).pin_memory()
    y = torch.full((T, 64), float("nan"), dtype=torch.float32, device="cuda")
    rc = lib.mole_lookup_combine_nf3_mapped(ids.data_ptr(), h.data_ptr(), w_r.data_ptr(), lo.data_ptr(),
                                            scales.data_ptr(), y.data_ptr(), T, V, 64, 1, 1, None)
    torch.cuda.synchronize()
    assert rc == 0 and bool((y == 0).all())


@pytest.mark.parametrize("T", [1, 256, 2048])
def test_combine_nf3_from_table_file(T, tmp_path):
    """Table in a file (the disk tier); only the distinct requested rows are
    read and cross PCIe.  Equal bit for bit to the device-resident combine,
    twice in a row through the same staging area."""
    V, N, D = 4096, 16, 1024
    r = rng(93)
    ids = synth.zipf_ids(r, V, T, r.permutation(V))
    uniq = np.unique(ids)
    table = rand_table(94, V, N, D, "bf16", std=0.02, rows=uniq)
    codes, scales, _ = oracle.pack_nf3(table)
    h, w_r = rand_hw(95, T, N, D, "bf16", wstd=0.3)
    path = tmp_path / "table.molt"
    mole.mole_nf3_file_write(str(path), torch.from_numpy(codes), torch.from_numpy(scales.view(np.int16)))
    nbytes = mole.mole_nf3_host_staging_size(T, N, D)
    stage_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    stage_d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    ref_dev = run_nf3(ids, h, w_r, codes, scales)
    fd = os.open(path, os.O_RDONLY)
    try:
        assert mole.mole_nf3_file_shape(fd) == (V, N, D)
        for _ in range(2):
            y.fill_(float("nan"))
            U = mole.mole_lookup_combine_nf3_file(fd, torch.from_numpy(ids), dev(h), dev(w_r), V, stage_h, stage_d,
                                                  y)
            torch.cuda.synchronize()
            assert U == uniq.size
            np.testing.assert_array_equal(host(y), ref_dev)
    finally:
        os.close(fd)
    assert combine_rel_err(host(y), oracle.lookup_combine_nf3(ids, h, w_r, codes, scales)) <= COMBINE_TOL


def test_nf3_host_stack_prefetch_matches_device_path():
    """Three layers' NF3 tables in host memory, one step's rows prefetched in
    one transfer; every layer's combine on the staged rows equals the
    device-resident NF3 combine bit for bit, and the oracle within the
    combine bar.  Two steps in a row through the same staging area."""
    V, N, D, L = 700, 8, 512, 3
    CB, SB = 3 * D // 8, D // 64
    tabs = []
    for l in range(L):
        codes, scales, _ = oracle.pack_nf3(rand_table(300 + l, V, N, D, "bf16", std=0.02))
        tabs.append((codes, scales))
    codes_h = [torch.from_numpy(c).pin_memory() for c, _ in tabs]
    scales_h = [torch.from_numpy(s.view(np.int16)).pin_memory() for _, s in tabs]
    for step, T in enumerate((97, 40)):
        ids = synth.zipf_ids(rng(400 + step), V, T, rng(401).permutation(V))
        hws = [rand_hw(500 + 10 * step + l, T, N, D, "bf16", wstd=0.3) for l in range(L)]
        nbytes = mole.mole_nf3_host_stack_staging_size(97, L, N, D)
        if step == 0:
            stage_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
            stage_d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        remap, layers = mole.mole_prefetch_nf3_host_stack(torch.from_numpy(ids), codes_h, scales_h,
                                                          stage_h, stage_d)
        U = layers[0][0].shape[0]
        assert U == np.unique(ids).size
        for l in range(L):
            h, w_r = hws[l]
            y = torch.empty((T, D), dtype=torch.float32, device="cuda")
            mole.mole_lookup_combine_nf3(remap, dev(h), dev(w_r), layers[l][0], layers[l][1], y)
            torch.cuda.synchronize()
            got = host(y)
            np.testing.assert_array_equal(got, run_nf3(ids, h, w_r, tabs[l][0], tabs[l][1]))
            ref = oracle.lookup_combine_nf3(ids, h, w_r, tabs[l][0], tabs[l][1])
            assert combine_rel_err(got, ref) <= COMBINE_TOL


# ----------------------------------------------------------------------------
# LUT build
# ----------------------------------------------------------------------------

def run_build(layer, ws_bytes=None):
    emb, w_up, w_down = dev(layer.emb), dev(layer.w_up), dev(layer.w_down)
    V, D = layer.emb.shape
    N, F, _ = layer.w_up.shape
    lut = torch.empty((V, N, D), dtype=emb.dtype, device="cuda")
    ws = None
    if emb.dtype == torch.bfloat16:
        mn, rec = mole.mole_build_lut_workspace_size(V, D, F, N)
        ws = torch.empty(ws_bytes or rec, dtype=torch.uint8, device="cuda")
    mole.mole_build_lut(emb, w_up, w_down, lut, workspace=ws)
    torch.cuda.synchronize()
    return lut


def test_build_tiny_f32_all_rows():
    w = synth.WORKLOADS["tiny"]
    layer = synth.make_layer(w)
    lut = host(run_build(layer))
    ref = oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down)
    assert rel_l2(lut, ref) <= 1e-5


def test_build_tiny_f32_unit_scale_nonlinear():
    """Unit-scale weights put GELU in its nonlinear range (|u| ~ 1), where
    the erf and tanh forms differ by ~1e-4: the 1e-5 bar tells them apart."""
    r = rng(21)
    V, D, F, N = 512, 64, 256, 4
    layer = synth.Layer(r.standard_normal((V, D), dtype=np.float32),
                        (r.standard_normal((N, F, D)) / np.sqrt(D)).astype(np.float32),
                        (r.standard_normal((N, D, F)) / np.sqrt(F)).astype(np.float32),
                        np.zeros((N, D), np.float32))
    lut = host(run_build(layer))
    assert rel_l2(lut, oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down)) <= 1e-5


def bf16_layer(seed, V, D, F, N, std=0.02):
    r = rng(seed)
    f = lambda shape, s: synth.f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(s))
    return synth.Layer(f((V, D), std), f((N, F, D), std), f((N, D, F), std), f((N, D), std))


# The last two cases have LUT rows >= 16 KB apart (N*D*2), which takes the
# LDS-staged output path of the second GEMM; (520, 1000, 136, 9) also has
# ragged row, column and K tiles in both GEMMs.
@pytest.mark.parametrize("V,D,F,N,std", [(600, 256, 512, 2, 0.02), (333, 72, 136, 3, 0.5),
                                         (256, 512, 256, 1, 0.1), (1000, 128, 1024, 4, 0.02),
                                         (700, 1024, 256, 8, 0.03), (520, 1000, 136, 9, 0.1)])
def test_build_bf16_small_all_rows(V, D, F, N, std):
    layer = bf16_layer(V + D + F + N, V, D, F, N, std)
    lut = host(run_build(layer))
    ref = oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down)
    assert rel_l2(bf16_to_f64(lut), ref) <= 1e-2


def test_build_bf16_min_workspace_equals_recommended():
    """Chunking over vocabulary rows does not change the arithmetic."""
    layer = bf16_layer(5, 1300, 256, 512, 2, 0.05)
    mn, _ = mole.mole_build_lut_workspace_size(1300, 256, 512, 2)
    a = host(run_build(layer, ws_bytes=mn))
    b = host(run_build(layer))
    np.testing.assert_array_equal(a, b)
    # and a zero embedding row gives an exactly zero table row
    layer.emb[17] = 0
    assert np.all(host(run_build(layer))[17] == 0)


@pytest.mark.parametrize("name,nrows", [("160m", 48), ("410m", 24), ("1b", 8)])
def test_build_full_size_sampled_rows(name, nrows):
    w = synth.WORKLOADS[name]
    layer = synth.make_layer(w)
    lut = run_build(layer)
    rows = np.unique(np.concatenate([[0, w.V - 1], rng(31).integers(0, w.V, nrows)]))
    got = host(lut[torch.from_numpy(rows).cuda()])
    del lut
    ref = oracle.build_lut_rows(layer.emb, layer.w_up, layer.w_down, rows=rows)
    assert rel_l2(bf16_to_f64(got), ref) <= 1e-2
    per_row = [rel_l2(bf16_to_f64(got[i]), ref[i]) for i in range(len(rows))]
    assert max(per_row) <= 2e-2


# ----------------------------------------------------------------------------
# HIP graph replay: a stack of lookup-combines captured once
# ----------------------------------------------------------------------------

def test_graph_replay_of_layer_stack_matches_eager_and_oracle():
    """Four layers (own table and router each, same ids, own hidden state),
    captured as one HIP graph.  Every replay -- with eager work and
    synchronisations in between -- reproduces the eager outputs bit for bit
    (same kernels, same inputs), and those meet the oracle's 2e-5 bar."""
    V, N, D, T, L = 900, 8, 512, 70, 4
    ids = synth.zipf_ids(rng(91), V, T, rng(92).permutation(V))
    tabs = [rand_table(900 + l, V, N, D, "bf16") for l in range(L)]
    hws = [rand_hw(950 + l, T, N, D, "bf16") for l in range(L)]
    d_ids = dev(ids)
    d_tabs = [dev(t) for t in tabs]
    d_h = [dev(h) for h, _ in hws]
    d_w = [dev(w) for _, w in hws]
    ys = [torch.empty((T, D), dtype=torch.float32, device="cuda") for _ in range(L)]

    def stack(st):
        for l in range(L):
            mole.mole_lookup_combine(d_ids, d_h[l], d_w[l], d_tabs[l], ys[l], stream=st)

    stack(None)
    torch.cuda.synchronize()
    eager = [host(y) for y in ys]
    for l in range(L):
        ref = oracle.lookup_combine(ids, hws[l][0], hws[l][1], tabs[l])
        assert combine_rel_err(eager[l], ref) <= COMBINE_TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack(torch.cuda.current_stream())
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(host(ys[l]), eager[l])
        stack(None)  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_of_mapped_nf3_combines():
    """Two layers whose NF3 tables sit in page-locked host memory, read in
    place, captured as one HIP graph (the pointer checks run at capture
    time; the graph holds only the kernels).  Every replay -- with eager
    work in between -- reproduces the eager outputs bit for bit, and those
    equal the device-resident combine."""
    V, N, D, T, L = 400, 16, 1024, 1100, 2
    ids = rng(93).integers(0, V, T).astype(np.int64)
    layers = []
    for l in range(L):
        codes, scales, _ = oracle.pack_nf3(rand_table(960 + l, V, N, D, "bf16"))
        h, w_r = rand_hw(970 + l, T, N, D, "bf16", wstd=0.3)
        layers.append((codes, scales, h, w_r, torch.from_numpy(codes).pin_memory(),
                       torch.from_numpy(scales.view(np.int16)).pin_memory(), dev(h), dev(w_r)))
    d_ids = dev(ids)
    ys = [torch.empty((T, D), dtype=torch.float32, device="cuda") for _ in range(L)]

    def stack(st):
        for l in range(L):
            _, _, _, _, ch, sh, dh, dw = layers[l]
            mole.mole_lookup_combine_nf3_mapped(d_ids, dh, dw, ch, sh, ys[l], stream=st)

    stack(None)
    torch.cuda.synchronize()
    eager = [host(y) for y in ys]
    for l in range(L):
        codes, scales, h, w_r = layers[l][:4]
        np.testing.assert_array_equal(eager[l], run_nf3(ids, h, w_r, codes, scales))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack(torch.cuda.current_stream())
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            np.testing.assert_array_equal(host(ys[l]), eager[l])
        stack(None)  # eager work between replays
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# The MoLE block: residual + shared expert FFN + routed lookup (training
# section: shared experts read the contextual hidden state; complexity
# analysis: they are the only experts still computed at inference)
# ----------------------------------------------------------------------------

LAYER_TOL = 1e-2  # rel-L2 of the block's update, as for the bf16 build products


def rand_shared(seed, D, F, std_up=0.02, std_down=0.02, zero=False):
    """Shared-expert weights w_s_up [F,D], w_s_down [D,F] as bf16 bits."""
    r = rng(seed)
    if zero:
        return np.zeros((F, D), np.uint16), np.zeros((D, F), np.uint16)
    f = lambda shape, s: synth.f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(s))
    return f((F, D), std_up), f((D, F), std_down)


def run_layer(ids, h, w_r, lut, wu, wd, x0):
    T, D = h.shape
    F = wu.shape[0]
    ws = torch.empty(max(mole.mole_layer_workspace_size(T, D, F), 16), dtype=torch.uint8, device="cuda")
    x = dev(x0)
    mole.mole_layer_forward(dev(ids), dev(h), dev(w_r), dev(lut), dev(wu), dev(wd), x, ws)
    torch.cuda.synchronize()
    return host(x)


# (V, N, D, F, T): every branch of the launch plan --
#   T = 1, 37, 200: one-tile-row MFMA blocks, K splits on both projections (GELU
#     reduction; several partial sums in the final pass); T = 37 has ragged
#     rows, columns and K (D = 264, F = 392) and a ragged last split;
#   T = 512: no splits (GELU in the up-projection's epilogue, one partial sum);
#   T = 2048, F = 8192: both projections on the 256x256 build GEMM (8 equal K
#     splits of fp32 partials for the down-projection), staged router gates;
#   T = 256, F = 4096: two-tile-row blocks with GELU in the epilogue;
#   T = 1024, D = 2048: four-tile-row blocks for the down-projection;
#   T = 1024, F = 8192: four-tile-row blocks with GELU in the epilogue.
LAYER_CASES = [(300, 4, 256, 512, 1), (500, 5, 264, 392, 37), (400, 16, 512, 1024, 200),
               (256, 2, 256, 256, 512), (1000, 8, 128, 8192, 2048), (300, 4, 128, 4096, 256),
               (300, 4, 2048, 512, 1024), (300, 4, 256, 8192, 1024),
               # decode batches (weight-streaming projections): ragged K tails,
               # 1, 2, 4 and 8 tokens per wavefront, a long down-projection
               (500, 5, 264, 392, 3), (400, 16, 1024, 8192, 8), (300, 3, 2048, 200, 5), (200, 4, 64, 136, 2)]


@pytest.mark.parametrize("V,N,D,F,T", LAYER_CASES)
def test_layer_matches_oracle(V, N, D, F, T):
    seed = V + N + D + F + T
    lut = rand_table(seed, V, N, D, "bf16", std=0.05)
    h, w_r = rand_hw(seed + 1, T, N, D, "bf16", wstd=0.05)
    # unit-scale hidden units (|u| ~ 1, where GELU is nonlinear)
    wu, wd = rand_shared(seed + 2, D, F, std_up=1.0 / np.sqrt(D), std_down=1.0 / np.sqrt(F))
    ids = rng(seed + 3).integers(0, V, size=T).astype(np.int64)
    x0 = rng(seed + 4).standard_normal((T, D), dtype=np.float32) * np.float32(3.0)
    got = run_layer(ids, h, w_r, lut, wu, wd, x0)
    upd = oracle.layer_forward(ids, h, w_r, lut, wu, wd, None)
    assert rel_l2(got.astype(np.float64) - x0.astype(np.float64), upd) <= LAYER_TOL
    per_tok = [rel_l2(got[t].astype(np.float64) - x0[t], upd[t]) for t in range(T)]
    assert max(per_tok) <= 2 * LAYER_TOL


@pytest.mark.parametrize("T", [1, 37, 512])
def test_layer_zero_shared_weights_is_the_combine(T):
    """With zero shared weights the block adds exactly the routed lookup, held
    to the combine's 2e-5 bar (the shared path contributes exact zeros)."""
    V, N, D, F = 300, 6, 256, 512
    lut = rand_table(70 + T, V, N, D, "bf16")
    h, w_r = rand_hw(71 + T, T, N, D, "bf16")
    wu, wd = rand_shared(0, D, F, zero=True)
    ids = rng(72 + T).integers(0, V, size=T).astype(np.int64)
    got = run_layer(ids, h, w_r, lut, wu, wd, np.zeros((T, D), np.float32))
    assert combine_rel_err(got, oracle.lookup_combine(ids, h, w_r, lut)) <= COMBINE_TOL


def test_layer_empty_batch_is_noop():
    D, F = 64, 128
    x = torch.full((1, D), 7.0, device="cuda")
    empty = torch.empty((0,), dtype=torch.int64, device="cuda")
    z = torch.zeros((0, D), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, D), dtype=torch.bfloat16, device="cuda")
    lut = torch.zeros((4, 2, D), dtype=torch.bfloat16, device="cuda")
    wu = torch.zeros((F, D), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((D, F), dtype=torch.bfloat16, device="cuda")
    mole.mole_layer_forward(empty, z, w, lut, wu, wd, x[:0], None)
    torch.cuda.synchronize()
    assert torch.all(x == 7.0)


@pytest.mark.parametrize("name,T", [("160m", 1), ("160m", 256), ("410m", 1024), ("410m", 4096),
                                    ("1b", 1024)])
def test_layer_full_size_sampled_tokens(name, T):
    """The block at the benchmark's configurations (shared expert of the
    routed experts' size, Zipf ids): every output row is computed; up to 48
    sampled tokens are checked against the oracle (its cost is per token)."""
    w = synth.WORKLOADS[name]
    D, F, N = w.D, w.F, w.N
    ids = synth.make_ids(w, T)
    lut = rand_table(81, w.V, N, D, "bf16", std=0.05, rows=np.unique(ids))
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    wu, wd = rand_shared(82, D, F)
    x0 = rng(83).standard_normal((T, D), dtype=np.float32)
    got = run_layer(ids, h, w_r, lut, wu, wd, x0)
    assert np.all(np.isfinite(got))
    sample = np.unique(np.concatenate([[0, T - 1], rng(84).integers(0, T, 46)]))
    upd = oracle.layer_forward(ids[sample], np.ascontiguousarray(h[sample]), w_r, lut, wu, wd, None)
    assert rel_l2(got[sample].astype(np.float64) - x0[sample], upd) <= LAYER_TOL


@pytest.mark.parametrize("T", [37, 3])
def test_layer_graph_replay_matches_eager(T):
    """The block (no memset; T = 3 takes the weight-streaming decode path)
    captured once; each replay, after eager work and a reset of the residual
    stream, equals the eager result bit for bit."""
    V, N, D, F = 300, 4, 256, 512
    lut = dev(rand_table(61, V, N, D, "bf16"))
    h, w_r = (dev(a) for a in rand_hw(62, T, N, D, "bf16"))
    wu, wd = (dev(a) for a in rand_shared(63, D, F, std_up=0.05, std_down=0.05))
    ids = dev(rng(64).integers(0, V, size=T).astype(np.int64))
    x0 = dev(rng(65).standard_normal((T, D), dtype=np.float32))
    x = x0.clone()
    ws = torch.empty(mole.mole_layer_workspace_size(T, D, F), dtype=torch.uint8, device="cuda")
    mole.mole_layer_forward(ids, h, w_r, lut, wu, wd, x, ws)
    torch.cuda.synchronize()
    eager = host(x)
    g = torch.cuda.CUDAGraph()
    x.copy_(x0)
    with torch.cuda.graph(g):
        mole.mole_layer_forward(ids, h, w_r, lut, wu, wd, x, ws, stream=torch.cuda.current_stream())
    for rep in range(3):
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(x), eager)
        y = x0.clone()
        mole.mole_layer_forward(ids, h, w_r, lut, wu, wd, y, ws)  # eager work between replays
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# Other table formats: NF4 (NormalFloat at 4 bits) and int8 with one scale per
# row (results section: the table still carries redundancy at 3 bits)
# ----------------------------------------------------------------------------

def run_pack_q(fmt, table):
    lut = dev(table)
    V, N, D = table.shape
    if fmt == "nf4":
        codes = torch.empty((V, N, D // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((V, N, D // 64), dtype=torch.int16, device="cuda")
        mole.mole_pack_nf4(lut, codes, scales)
    else:
        codes = torch.empty((V, N, D), dtype=torch.int8, device="cuda")
        scales = torch.empty((V, N), dtype=torch.float32, device="cuda")
        mole.mole_pack_int8(lut, codes, scales)
    torch.cuda.synchronize()
    return host(codes), host(scales)


def oracle_pack_q(fmt, table):
    if fmt == "nf4":
        c, s, _ = oracle.pack_nf4(table)
        return c, s
    return oracle.pack_int8(table)


def run_combine_q(fmt, ids, h, w_r, codes, scales):
    y = torch.empty((ids.size, h.shape[1]), dtype=torch.float32, device="cuda")
    if fmt == "nf4":
        mole.mole_lookup_combine_nf4(dev(ids), dev(h), dev(w_r), dev(codes), dev(scales.view(np.int16)), y)
    else:
        mole.mole_lookup_combine_int8(dev(ids), dev(h), dev(w_r), dev(codes), dev(scales), y)
    torch.cuda.synchronize()
    return host(y)


def oracle_combine_q(fmt, ids, h, w_r, codes, scales):
    if fmt == "nf4":
        return oracle.lookup_combine_nf4(ids, h, w_r, codes, scales)
    return oracle.lookup_combine_int8(ids, h, w_r, codes, scales)


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
@pytest.mark.parametrize("V,N,D,dtype,std", [(512, 4, 64, "f32", 0.02), (300, 4, 768, "bf16", 0.02),
                                             (100, 16, 1024, "bf16", 1.0), (33, 3, 2048, "bf16", 1e-3),
                                             (7, 1, 128, "f32", 3.0), (20, 2, 4096, "bf16", 0.05)])
def test_pack_q_bit_exact(fmt, V, N, D, dtype, std):
    table = rand_table(20 + D + V, V, N, D, dtype, std=std)
    codes, scales = run_pack_q(fmt, table)
    c_ref, s_ref = oracle_pack_q(fmt, table)
    np.testing.assert_array_equal(scales.view(s_ref.dtype), s_ref)
    np.testing.assert_array_equal(codes.view(c_ref.dtype), c_ref)


def test_pack_nf4_edge_cases_bit_exact():
    """Exact threshold ties (strict compare keeps the lower code) and their
    float neighbours, every level, zero and tiny blocks (code 7), fp16-subnormal
    scales and saturation at 65504."""
    mid, lv = oracle.nf4_midpoints(), oracle.nf4_levels()
    tie = np.zeros(64, np.float32)
    tie[0] = 1.0
    tie[1:16] = mid
    tie[16:31] = np.nextafter(mid, np.float32(2))
    tie[31:46] = np.nextafter(mid, np.float32(-2))
    tie[46:62] = lv
    rows = [tie, np.zeros(64, np.float32), np.full(64, 1e-9, np.float32),
            np.linspace(-3e-6, 2e-6, 64).astype(np.float32), np.linspace(-1e5, 7e4, 64).astype(np.float32)]
    table = np.stack(rows).reshape(len(rows), 1, 64)
    codes, scales = run_pack_q("nf4", table)
    c_ref, s_ref, nsat = oracle.pack_nf4(table)
    assert nsat == 1
    np.testing.assert_array_equal(scales.view(np.uint16), s_ref)
    np.testing.assert_array_equal(codes, c_ref)


def test_pack_int8_edge_cases_bit_exact():
    """Values at exact half-steps (ties to even), the absmax element on both
    signs, an all-zero row, tiny and huge rows."""
    half = (np.arange(64, dtype=np.float32) - 32) + np.float32(0.5)  # absmax 31.5 -> s = 31.5/127
    unit = np.concatenate([[127.0, -127.0], np.arange(-31, 31) + 0.5]).astype(np.float32)  # s = 1 exactly
    rows = [half, unit, np.zeros(64, np.float32), np.full(64, -1e-30, np.float32),
            np.linspace(-3e38, 1e38, 64).astype(np.float32)]
    table = np.stack(rows).reshape(len(rows), 1, 64)
    codes, scales = run_pack_q("int8", table)
    c_ref, s_ref = oracle.pack_int8(table)
    np.testing.assert_array_equal(scales, s_ref)
    np.testing.assert_array_equal(codes.view(np.int8), c_ref)
    assert s_ref[1, 0] == 1.0 and c_ref[1, 0, 2:6].tolist() == [-30, -30, -28, -28]


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
@pytest.mark.parametrize("V,N,D,T,dtype", [(512, 4, 64, 64, "f32"), (300, 4, 768, 200, "bf16"),
                                           (300, 16, 1024, 257, "bf16"), (100, 16, 2048, 33, "bf16"),
                                           (64, 64, 128, 10, "bf16"), (50, 3, 192, 17, "f32"),
                                           (40, 1, 64, 5, "bf16"), (300, 16, 1024, 2051, "bf16"),
                                           (100, 64, 512, 2048, "bf16"), (300, 12, 1024, 100, "bf16"),
                                           (300, 16, 1024, 1023, "bf16"), (300, 16, 1024, 1024, "bf16"),
                                           (300, 12, 2048, 1027, "bf16"), (100, 16, 4096, 1024, "bf16"),
                                           (300, 16, 1024, 9001, "bf16"), (300, 4, 768, 5003, "bf16"),
                                           (300, 12, 1024, 2047, "bf16")])
def test_combine_q_matches_oracle(fmt, V, N, D, T, dtype):
    seed = 3000 + V + N + D
    table = rand_table(seed, V, N, D, "bf16")
    codes, scales = oracle_pack_q(fmt, table)
    h, w_r = rand_hw(seed + 1, T, N, D, dtype, wstd=0.3)
    ids = rng(seed + 2).integers(0, V, T).astype(np.int64)
    y = run_combine_q(fmt, ids, h, w_r, codes, scales)
    assert combine_rel_err(y, oracle_combine_q(fmt, ids, h, w_r, codes, scales)) <= COMBINE_TOL


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
@pytest.mark.parametrize("T", [1, 256, 4096])
def test_combine_q_full_size_zipf(fmt, T):
    """410M-class table (V=50304, N=16, D=1024), Zipf ids: codes from the
    oracle's encoding of the rows the batch touches."""
    w = synth.WORKLOADS["410m"]
    ids = synth.make_ids(w, T)
    uniq = np.unique(ids)
    table = rand_table(92, w.V, w.N, w.D, "bf16", std=0.02, rows=uniq)
    codes, scales = oracle_pack_q(fmt, table)
    h = synth.make_hidden(w, T)
    w_r = synth.make_router(w)
    y = run_combine_q(fmt, ids, h, w_r, codes, scales)
    assert combine_rel_err(y, oracle_combine_q(fmt, ids, h, w_r, codes, scales)) <= COMBINE_TOL


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_pack_q_full_size_sampled_rows(fmt):
    """410M-class table packed on the GPU in one launch; 1024 seeded rows plus
    the first and last are re-encoded by the oracle; untouched rows are zero."""
    w = synth.WORKLOADS["410m"]
    sample = np.unique(np.concatenate([[0, w.V - 1], rng(13).integers(0, w.V, 1024)]))
    table = rand_table(14, w.V, w.N, w.D, "bf16", std=0.02, rows=sample)
    codes, scales = run_pack_q(fmt, table)
    c_ref, s_ref = oracle_pack_q(fmt, table[sample])
    np.testing.assert_array_equal(scales[sample].view(s_ref.dtype), s_ref)
    np.testing.assert_array_equal(codes[sample].view(c_ref.dtype), c_ref)
    other = np.setdiff1d(np.arange(w.V), sample)[:300]
    assert np.all(scales[other] == 0)
    assert np.all(codes[other] == (0x77 if fmt == "nf4" else 0))


# ----------------------------------------------------------------------------
# Training mode: forward (every expert on the token's embedding, dense gates)
# and backward (training section of the MoLE article)
# ----------------------------------------------------------------------------

TRAIN_TOL = 1e-2  # rel-L2, the bf16-product bar of the build


def train_case(seed, V, D, F, N, T, zipf=False):
    r = rng(seed)
    f = lambda shape, s: synth.f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(s))
    emb = f((V, D), 1.0)
    w_up = f((N, F, D), 1.0 / np.sqrt(D))     # unit-scale hidden units: GELU is nonlinear
    w_down = f((N, D, F), 1.0 / np.sqrt(F))
    w_r = f((N, D), 0.3 / np.sqrt(D))
    h = f((T, D), 1.0)
    if zipf:
        ids = synth.zipf_ids(r, V, T, r.permutation(V))
    else:
        ids = r.integers(0, V, size=T).astype(np.int64)
    dy = r.standard_normal((T, D)).astype(np.float32)
    return ids, emb, w_up, w_down, h, w_r, dy


def run_train(ids, emb, w_up, w_down, h, w_r, dy):
    V, D = emb.shape
    N, F, _ = w_up.shape
    T = ids.size
    uniq, remap, row_ptr, tok = mole.mole_train_index(torch.from_numpy(ids), V)
    U = uniq.numel()
    fb, bb = mole.mole_train_workspace_size(T, U, D, F, N)
    fws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    bws = torch.empty(bb, dtype=torch.uint8, device="cuda")
    d_uniq, d_remap, d_ptr, d_tok = (x.cuda() for x in (uniq, remap, row_ptr, tok))
    t_w_up, t_w_down, t_h, t_w_r = dev(w_up), dev(w_down), dev(h), dev(w_r)
    y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    mole.mole_train_forward(d_uniq, d_remap, dev(emb), t_w_up, t_w_down, t_h, t_w_r, y, fws)
    out = {k: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
           for k, s in (("d_w_up", (N, F, D)), ("d_w_down", (N, D, F)), ("d_w_r", (N, D)), ("d_h", (T, D)),
                        ("d_x", (U, D)))}
    mole.mole_train_backward(d_remap, d_ptr, d_tok, U, V, t_w_up, t_w_down, t_h, t_w_r, dev(dy), fws, bws,
                             out["d_w_up"], out["d_w_down"], out["d_w_r"], out["d_h"], out["d_x"])
    torch.cuda.synchronize()
    return host(y), {k: host(v) for k, v in out.items()}, uniq.numpy()


# (V, N, D, F, T, zipf): ragged D/F/T, repeated ids (several tokens per row),
# many experts, a 160M-class width, and long Zipf batches whose head rows run
# over many chunks of the row-gradient walk (64-position chunks at T = 5000;
# 32 experts take its two-columns-per-lane form), D = 1024 (four wavefronts
# per token in the gate backward) and a single token with one expert.
TRAIN_CASES = [(300, 4, 128, 256, 100, False), (50, 3, 136, 200, 37, True), (400, 16, 256, 512, 64, True),
               (40, 64, 64, 64, 20, False), (2000, 4, 768, 3072, 32, True), (500, 16, 64, 64, 5000, True),
               (300, 32, 64, 128, 700, True), (100, 4, 1024, 256, 64, True), (10, 1, 64, 64, 1, False)]


@pytest.mark.parametrize("V,N,D,F,T,zipf", TRAIN_CASES)
def test_train_forward_and_backward_match_oracle(V, N, D, F, T, zipf):
    ids, emb, w_up, w_down, h, w_r, dy = train_case(V + N + D + F + T, V, D, F, N, T, zipf)
    y, grads, uniq = run_train(ids, emb, w_up, w_down, h, w_r, dy)
    y_ref = oracle.train_forward(ids, emb, w_up, w_down, h, w_r)
    assert rel_l2(y, y_ref) <= TRAIN_TOL
    ref = oracle.train_backward(ids, emb, w_up, w_down, h, w_r, dy.astype(np.float64))
    for k in ("d_w_up", "d_w_down", "d_w_r", "d_h"):
        assert np.all(np.isfinite(grads[k])), k
        assert rel_l2(grads[k], ref[k]) <= TRAIN_TOL, (k, rel_l2(grads[k], ref[k]))
    assert rel_l2(grads["d_x"], ref["d_emb"][uniq]) <= TRAIN_TOL


def test_train_one_row_for_every_token():
    """Every token has the same id: one row of the table receives all T
    tokens' gradients, through every chunk of the row-gradient walk."""
    V, N, D, F, T = 30, 4, 64, 128, 700
    ids, emb, w_up, w_down, h, w_r, dy = train_case(5, V, D, F, N, T)
    ids[:] = 7
    y, grads, uniq = run_train(ids, emb, w_up, w_down, h, w_r, dy)
    assert uniq.tolist() == [7]
    assert rel_l2(y, oracle.train_forward(ids, emb, w_up, w_down, h, w_r)) <= TRAIN_TOL
    ref = oracle.train_backward(ids, emb, w_up, w_down, h, w_r, dy.astype(np.float64))
    for k in ("d_w_up", "d_w_down", "d_w_r", "d_h"):
        assert rel_l2(grads[k], ref[k]) <= TRAIN_TOL, (k, rel_l2(grads[k], ref[k]))
    assert rel_l2(grads["d_x"], ref["d_emb"][uniq]) <= TRAIN_TOL


def test_train_matches_the_lookup_path_on_the_built_table():
    """The training forward equals the lookup-combine over the table that
    mole_build_lut makes from the same weights (both round the hidden
    activation and the table to bf16 the same way), up to fp32 summation order."""
    V, N, D, F, T = 500, 4, 256, 512, 90
    ids, emb, w_up, w_down, h, w_r, _ = train_case(77, V, D, F, N, T, zipf=True)
    y, _, _ = run_train(ids, emb, w_up, w_down, h, w_r, np.zeros((T, D), np.float32))
    lut = torch.empty((V, N, D), dtype=torch.bfloat16, device="cuda")
    _, rec = mole.mole_build_lut_workspace_size(V, D, F, N)
    mole.mole_build_lut(dev(emb), dev(w_up), dev(w_down), lut, workspace=torch.empty(rec, dtype=torch.uint8,
                                                                                     device="cuda"))
    y2 = torch.empty((T, D), dtype=torch.float32, device="cuda")
    mole.mole_lookup_combine(dev(ids), dev(h), dev(w_r), lut, y2)
    torch.cuda.synchronize()
    assert combine_rel_err(y, host(y2)) <= COMBINE_TOL
