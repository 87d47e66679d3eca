"""The allocation-free grouped combine (mole_lookup_combine_grouped_noalloc,
workspace in the library's static device array) against the workspace entry
point it shares its kernels with, and against the oracle, through the C ABI:
two calls in a row, the second with a smaller batch (the array keeps the
first call's contents), plus the limit check."""
import ctypes

import numpy as np
import pytest
import torch

import mixture_lookup_experts_amd as mole
import oracle
from mixture_lookup_experts_amd import _native, synth
from tests.gpu_util import combine_rel_err, dev, host

pytestmark = pytest.mark.gpu

COMBINE_TOL = 2e-5


def inputs(seed, V, N, D, T):
    r = np.random.Generator(np.random.PCG64(seed))
    lut = synth.f32_to_bf16_bits(r.standard_normal((V, N, D), dtype=np.float32) * np.float32(0.05))
    h = synth.f32_to_bf16_bits(r.standard_normal((T, D), dtype=np.float32))
    w_r = synth.f32_to_bf16_bits(r.standard_normal((N, D), dtype=np.float32) * np.float32(0.3))
    ids = synth.zipf_ids(r, V, T, r.permutation(V))
    return ids, h, w_r, lut


def with_workspace(ids, h, w_r, lut):
    T = ids.size
    y = torch.full((T, lut.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(mole.mole_lookup_combine_grouped_workspace_size(T), dtype=torch.uint8, device="cuda")
    mole.mole_lookup_combine_grouped(dev(ids), dev(h), dev(w_r), dev(lut), y, ws)
    torch.cuda.synchronize()
    return host(y)


def without_alloc(ids, h, w_r, lut):
    """Direct C-ABI call (ctypes), no workspace argument."""
    lib = mole.library()
    T = ids.size
    V, N, D = lut.shape
    y = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
    ids_d, h_d, w_d, lut_d = dev(ids), dev(h), dev(w_r), dev(lut)
    rc = lib.mole_lookup_combine_grouped_noalloc(ids_d.data_ptr(), h_d.data_ptr(), w_d.data_ptr(), lut_d.data_ptr(),
                                                 y.data_ptr(), T, V, D, N, _native.MOLE_BF16, None)
    assert rc == 0, mole.mole_status_string(rc)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("shape_a,shape_b", [((2000, 16, 1024, 5000), (300, 4, 768, 37)),
                                             ((3000, 16, 2048, 4096), (1000, 16, 2048, 1))])
def test_noalloc_matches_workspace_entry_twice(shape_a, shape_b):
    for k, (V, N, D, T) in enumerate((shape_a, shape_b)):
        ids, h, w_r, lut = inputs(6100 + 10 * k + T, V, N, D, T)
        y0 = without_alloc(ids, h, w_r, lut)
        y1 = with_workspace(ids, h, w_r, lut)
        assert np.all(np.isfinite(y0))
        # same kernels, same workspace layout: identical results
        np.testing.assert_array_equal(y0, y1)
        assert combine_rel_err(y0, oracle.lookup_combine(ids, h, w_r, lut)) <= COMBINE_TOL


def test_noalloc_rejects_batches_past_the_limit():
    lib = mole.library()
    a = ctypes.c_void_p(256)  # never dereferenced: rejected on the host
    T = _native.MOLE_GROUPED_NOALLOC_MAX_T + 1
    rc = lib.mole_lookup_combine_grouped_noalloc(a, a, a, a, a, T, 100, 64, 4, _native.MOLE_BF16, None)
    assert rc == -6  # MOLE_ERR_UNSUPPORTED
    assert lib.mole_lookup_combine_grouped_noalloc(a, a, a, a, a, 0, 100, 64, 4, _native.MOLE_BF16, None) == 0
