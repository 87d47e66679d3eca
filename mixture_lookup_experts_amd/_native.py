"""ctypes marshalling for libmole.so (argument marshalling only).

Each ``mole_*`` function here has the name of the C entry point it calls and
takes torch tensors (device tensors unless the name says host).  Shapes,
dtypes and the stream are read off the tensors; the C library validates
sizes, pointers and alignment and every status other than MOLE_OK raises
MoleError.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libmole.so")

MOLE_F32, MOLE_BF16 = 0, 1
_DTYPE = {torch.float32: MOLE_F32, torch.bfloat16: MOLE_BF16}

_lock = threading.Lock()
_lib = None


class MoleError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = "%s: status %d (%s)" % (fn, status, mole_status_string(status))
        if hip_error:
            msg += ", hipError %d" % hip_error
        super().__init__(msg)


class MoleLibraryMissing(ImportError):
    pass


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libmole.so (once).  Raises MoleLibraryMissing if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise MoleLibraryMissing(
                "libmole.so not found at %s; build it with "
                "`python -m mixture_lookup_experts_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "mole_status_string": (ctypes.c_char_p, [I]),
            "mole_last_hip_error": (I, []),
            "mole_abi_version": (I, []),
            "mole_release_host_state": (I, []),
            "mole_nf3_levels": (I, [P]),
            "mole_nf3_midpoints": (I, [P]),
            "mole_nf4_midpoints": (I, [P]),
            "mole_gelu_phi_coefficients": (I, [P, I, P]),
            "mole_build_lut_workspace_size": (I, [I64, I64, I64, I64, I, P, P]),
            "mole_build_lut": (I, [P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_lookup_combine": (I, [P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_pack_nf3": (I, [P, P, P, I64, I64, I64, I, P]),
            "mole_lookup_combine_nf3": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_lookup_combine_nf3_mapped": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_lookup_combine_mapped": (I, [P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_gather_nf3_host": (I, [P, I64, P, P, I64, I64, I64, P, P, P, P, I]),
            "mole_nf3_host_staging_size": (I, [I64, I64, I64, P]),
            "mole_nf3_host_stack_staging_size": (I, [I64, I64, I64, I64, P]),
            "mole_prefetch_nf3_host_stack": (I, [P, I64, P, P, I64, I64, I64, I64, P, P, SZ, P, P, I, P,
                                                 P]),
            "mole_lookup_combine_nf3_host": (I, [P, P, P, P, P, P, P, SZ, P,
                                                 I64, I64, I64, I64, I, I, P, P]),
            "mole_layer_workspace_size": (I, [I64, I64, I64, P]),
            "mole_nf4_levels": (I, [P]),
            "mole_pack_nf4": (I, [P, P, P, I64, I64, I64, I, P]),
            "mole_lookup_combine_nf4": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_pack_int8": (I, [P, P, P, I64, I64, I64, I, P]),
            "mole_lookup_combine_int8": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_train_index": (I, [P, I64, I64, P, P, P, P, P]),
            "mole_train_workspace_size": (I, [I64, I64, I64, I64, I64, P, P]),
            "mole_train_forward": (I, [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_train_backward": (I, [P, P, P, P, P, P, P, P, P, SZ, P, SZ, P, P, P, P, P,
                                        I64, I64, I64, I64, I64, I64, I, P]),
            "mole_layer_forward": (I, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_lookup_combine_grouped_workspace_size": (I, [I64, P]),
            "mole_check_ids": (I, [P, I64, I64, P, P]),
            "mole_lookup_combine_grouped": (I, [P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_lookup_combine_grouped_noalloc": (I, [P, P, P, P, P, I64, I64, I64, I64, I, P]),
            "mole_lookup_combine_grouped_mapped": (I, [P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_lookup_combine_nf3_grouped": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_lookup_combine_nf3_grouped_mapped": (I, [P, P, P, P, P, P, I64, I64, I64, I64, I, P, SZ, P]),
            "mole_nf3_file_write": (I, [ctypes.c_char_p, P, P, I64, I64, I64]),
            "mole_nf3_file_shape": (I, [I, P, P, P]),
            "mole_gather_nf3_file": (I, [I, P, I64, I64, I64, I64, P, P, P, P, I]),
            "mole_lookup_combine_nf3_file": (I, [I, P, P, P, P, P, SZ, P, I64, I64, I64, I64, I, I, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def mole_status_string(status: int) -> str:
    try:
        return library().mole_status_string(int(status)).decode()
    except MoleLibraryMissing:
        return "library not loaded"


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoleError(fn, rc, library().mole_last_hip_error() if rc == -7 else 0)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        return -1  # rejected by the library as MOLE_ERR_DTYPE


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def mole_nf3_levels() -> list:
    out = (ctypes.c_float * 8)()
    _check("mole_nf3_levels", library().mole_nf3_levels(ctypes.addressof(out)))
    return list(out)


def mole_build_lut_workspace_size(V: int, D: int, F: int, N: int, dtype=torch.bfloat16):
    """(minimum, recommended) workspace bytes for mole_build_lut."""
    mn, rec = ctypes.c_size_t(0), ctypes.c_size_t(0)
    code = _DTYPE.get(dtype, -1) if not isinstance(dtype, int) else dtype
    _check("mole_build_lut_workspace_size",
           library().mole_build_lut_workspace_size(V, D, F, N, code, ctypes.addressof(mn),
                                                   ctypes.addressof(rec)))
    return int(mn.value), int(rec.value)


def mole_build_lut(emb, w_up, w_down, lut, workspace=None, stream=None) -> None:
    """lut[V,N,D] = W_down[e] . GELU(W_up[e] . emb[v]) for all v, e.
    emb [V,D], w_up [N,F,D], w_down [N,D,F]; workspace: a uint8 device tensor
    (bf16 only; see mole_build_lut_workspace_size)."""
    _need(emb.dim() == 2 and w_up.dim() == 3 and w_down.dim() == 3 and lut.dim() == 3,
          "emb [V,D], w_up [N,F,D], w_down [N,D,F], lut [V,N,D]")
    V, D = emb.shape
    N, F, D2 = w_up.shape
    _need(D2 == D and tuple(w_down.shape) == (N, D, F) and tuple(lut.shape) == (V, N, D),
          "inconsistent shapes")
    for t in (emb, w_up, w_down, lut):
        _need(t.is_contiguous() and t.dtype == emb.dtype, "tensors must be contiguous, one dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mole_build_lut", library().mole_build_lut(
        _ptr(emb), _ptr(w_up), _ptr(w_down), _ptr(lut), V, D, F, N, _dtype(emb),
        _ptr(workspace), ws_bytes, _stream(stream)))


def mole_lookup_combine(ids, h, w_r, lut, y, stream=None) -> None:
    """y[t,:] = sum_e softmax(w_r . h[t])[e] * lut[ids[t], e, :] (fp32 y)."""
    V, N, D = lut.shape
    T = ids.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], lut [V,N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32, "ids int64, y float32")
    _need(h.dtype == lut.dtype == w_r.dtype, "h, w_r and lut share one dtype")
    for t in (ids, h, w_r, lut, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine", library().mole_lookup_combine(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut), _ptr(y), T, V, D, N, _dtype(lut),
        _stream(stream)))


def mole_pack_nf3(lut, codes, scales, stream=None) -> None:
    """NF3-encode lut [V,N,D] into codes [V,N,3D/8] (uint8) and scales
    [V,N,D/64] (fp16 bits, int16/uint16 tensor)."""
    V, N, D = lut.shape
    _need(D % 64 == 0, "D must be a multiple of 64")
    _need(tuple(codes.shape) == (V, N, 3 * D // 8) and codes.dtype == torch.uint8, "codes [V,N,3D/8] uint8")
    _need(tuple(scales.shape) == (V, N, D // 64) and scales.element_size() == 2, "scales [V,N,D/64] 16-bit")
    for t in (lut, codes, scales):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_pack_nf3", library().mole_pack_nf3(
        _ptr(lut), _ptr(codes), _ptr(scales), V, N, D, _dtype(lut), _stream(stream)))


def mole_lookup_combine_nf3(ids, h, w_r, codes, scales, y, stream=None) -> None:
    V, N, CB = codes.shape
    D = CB * 8 // 3
    T = ids.numel()
    _need(tuple(scales.shape) == (V, N, D // 64), "scales [V,N,D/64]")
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype,
          "ids int64, y float32, h and w_r one dtype")
    for t in (ids, h, w_r, codes, scales, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_nf3", library().mole_lookup_combine_nf3(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(codes), _ptr(scales), _ptr(y), T, V, D, N,
        _dtype(h), _stream(stream)))


def mole_lookup_combine_mapped(ids, h, w_r, lut_host, y, stream=None) -> None:
    """Lookup-combine reading the table in place from page-locked host memory
    (lut_host: a pinned CPU tensor [V,N,D] of h's dtype); ids, h, w_r, y on the device."""
    V, N, D = lut_host.shape
    T = ids.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype == lut_host.dtype,
          "ids int64, y float32, h, w_r and lut_host one dtype")
    _need(not lut_host.is_cuda, "lut_host in host memory")
    for t in (ids, h, w_r, lut_host, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_mapped", library().mole_lookup_combine_mapped(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut_host), _ptr(y), T, V, D, N, _dtype(h), _stream(stream)))


def mole_lookup_combine_nf3_mapped(ids, h, w_r, codes_host, scales_host, y, stream=None) -> None:
    """NF3 combine reading the table in place from page-locked host memory
    (codes_host / scales_host: pinned CPU tensors); ids, h, w_r, y on the device."""
    V, N, CB = codes_host.shape
    D = CB * 8 // 3
    T = ids.numel()
    _need(tuple(scales_host.shape) == (V, N, D // 64), "scales [V,N,D/64]")
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype,
          "ids int64, y float32, h and w_r one dtype")
    _need(not codes_host.is_cuda and not scales_host.is_cuda, "codes_host and scales_host in host memory")
    for t in (ids, h, w_r, codes_host, scales_host, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_nf3_mapped", library().mole_lookup_combine_nf3_mapped(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(codes_host), _ptr(scales_host), _ptr(y), T, V, D, N,
        _dtype(h), _stream(stream)))


def mole_gather_nf3_host(ids_host, codes_host, scales_host, codes_stage, scales_stage, remap,
                         nthreads: int = 0) -> int:
    """Host-only dedupe + gather of the requested NF3 rows; returns the number
    of distinct ids U (rows 0..U-1 of the staging buffers are written)."""
    V, N, CB = codes_host.shape
    D = CB * 8 // 3
    T = ids_host.numel()
    for t in (ids_host, codes_host, scales_host, codes_stage, scales_stage, remap):
        _need(t.device.type == "cpu" and t.is_contiguous(), "host tensors, contiguous")
    _need(codes_stage.numel() >= T * N * CB and scales_stage.numel() >= T * N * (D // 64)
          and remap.numel() >= T, "staging buffers hold at least T rows")
    u = ctypes.c_int64(0)
    _check("mole_gather_nf3_host", library().mole_gather_nf3_host(
        _ptr(ids_host), T, _ptr(codes_host), _ptr(scales_host), V, N, D, _ptr(codes_stage),
        _ptr(scales_stage), _ptr(remap), ctypes.addressof(u), nthreads))
    return int(u.value)


def mole_nf3_host_staging_size(T: int, N: int, D: int) -> int:
    """Bytes of pinned host staging (and of the device buffer of the same
    size) that mole_lookup_combine_nf3_host needs for up to T tokens."""
    out = ctypes.c_size_t(0)
    _check("mole_nf3_host_staging_size",
           library().mole_nf3_host_staging_size(T, N, D, ctypes.addressof(out)))
    return int(out.value)


def mole_nf3_host_stack_staging_size(T: int, L: int, N: int, D: int) -> int:
    """Bytes of pinned host staging (and of the device buffer of the same
    size) that mole_prefetch_nf3_host_stack needs for T tokens, L layers."""
    out = ctypes.c_size_t(0)
    _check("mole_nf3_host_stack_staging_size",
           library().mole_nf3_host_stack_staging_size(T, L, N, D, ctypes.addressof(out)))
    return int(out.value)


def mole_prefetch_nf3_host_stack(ids_host, codes_host, scales_host, stage_host, stage_dev,
                                 nthreads: int = 0, stream=None):
    """One decode step's NF3 rows for every layer of a stack, gathered on the
    host from the L host tables (lists codes_host[l] [V,N,3D/8] uint8 and
    scales_host[l] [V,N,D/64] int16) and moved to stage_dev (one copy, in up
    to four pieces overlapped with the gather).  Returns (remap [T] int64, [(codes_l [U,N,3D/8], scales_l
    [U,N,D/64]) for each layer]) -- views into stage_dev to hand to
    mole_lookup_combine_nf3 layer by layer on the same stream."""
    L = len(codes_host)
    _need(L > 0 and len(scales_host) == L, "one codes and one scales table per layer")
    V, N, CB = codes_host[0].shape
    D = CB * 8 // 3
    SB = D // 64
    T = ids_host.numel()
    for c, sc in zip(codes_host, scales_host):
        _need(tuple(c.shape) == (V, N, CB) and tuple(sc.shape) == (V, N, SB), "tables [V,N,3D/8] and [V,N,D/64]")
        _need(c.device.type == "cpu" and sc.device.type == "cpu" and c.is_contiguous() and sc.is_contiguous(),
              "host tables, contiguous")
    _need(ids_host.device.type == "cpu" and ids_host.dtype == torch.int64, "ids_host: int64 on the host")
    nbytes = stage_host.numel() * stage_host.element_size()
    _need(stage_dev.numel() * stage_dev.element_size() >= nbytes and stage_dev.dtype == torch.uint8,
          "device staging (uint8) as large as the host one")
    cptrs = (ctypes.c_void_p * L)(*[c.data_ptr() for c in codes_host])
    sptrs = (ctypes.c_void_p * L)(*[sc.data_ptr() for sc in scales_host])
    coff = (ctypes.c_size_t * L)()
    soff = (ctypes.c_size_t * L)()
    u = ctypes.c_int64(0)
    _check("mole_prefetch_nf3_host_stack", library().mole_prefetch_nf3_host_stack(
        _ptr(ids_host), T, ctypes.addressof(cptrs), ctypes.addressof(sptrs), L, V, N, D, _ptr(stage_host),
        _ptr(stage_dev), nbytes, ctypes.addressof(coff), ctypes.addressof(soff), nthreads,
        ctypes.addressof(u), _stream(stream)))
    U = int(u.value)
    remap = stage_dev[:T * 8].view(torch.int64)
    layers = []
    for l in range(L):
        c = stage_dev[coff[l]:coff[l] + U * N * CB].view(U, N, CB)
        sc = stage_dev[soff[l]:soff[l] + U * N * SB * 2].view(torch.int16).view(U, N, SB)
        layers.append((c, sc))
    return remap, layers


def mole_lookup_combine_nf3_host(ids_host, h, w_r, codes_host, scales_host, stage_host, stage_dev, y,
                                 nthreads: int = 0, stream=None) -> int:
    """Host-resident NF3 table: gather the requested rows on the host into
    the pinned staging area, copy its used part to the device buffer in one
    transfer and combine.  Returns U, the number of distinct ids."""
    V, N, CB = codes_host.shape
    D = CB * 8 // 3
    T = ids_host.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "h [T,D], w_r [N,D], y [T,D]")
    nbytes = stage_host.numel() * stage_host.element_size()
    _need(stage_dev.numel() * stage_dev.element_size() >= nbytes, "device staging as large as the host one")
    u = ctypes.c_int64(0)
    _check("mole_lookup_combine_nf3_host", library().mole_lookup_combine_nf3_host(
        _ptr(ids_host), _ptr(h), _ptr(w_r), _ptr(codes_host), _ptr(scales_host),
        _ptr(stage_host), _ptr(stage_dev), nbytes, _ptr(y), T, V, D, N, _dtype(h), nthreads,
        ctypes.addressof(u), _stream(stream)))
    return int(u.value)


def mole_check_ids(ids, V: int, count, stream=None) -> None:
    """Add to count (a one-element int32 device tensor) the number of ids
    outside [0, V)."""
    _need(ids.dtype == torch.int64 and ids.is_contiguous(), "ids int64, contiguous")
    _need(count.dtype == torch.int32 and count.numel() >= 1, "count: int32 device tensor")
    _check("mole_check_ids", library().mole_check_ids(_ptr(ids), ids.numel(), V, _ptr(count), _stream(stream)))


def mole_lookup_combine_grouped_workspace_size(T: int) -> int:
    out = ctypes.c_size_t(0)
    _check("mole_lookup_combine_grouped_workspace_size",
           library().mole_lookup_combine_grouped_workspace_size(T, ctypes.addressof(out)))
    return int(out.value)


def mole_lookup_combine_grouped(ids, h, w_r, lut, y, workspace, stream=None) -> None:
    """The combine with the batch grouped by id on the device: each table
    slab is read once per run of equal ids instead of once per token."""
    V, N, D = lut.shape
    T = ids.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64, "ids int64")
    _need(h.dtype == lut.dtype == w_r.dtype and y.dtype == torch.float32, "h, w_r, lut share one dtype; y float32")
    for t in (ids, h, w_r, lut, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mole_lookup_combine_grouped", library().mole_lookup_combine_grouped(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut), _ptr(y), T, V, D, N, _dtype(lut), _ptr(workspace), ws_bytes,
        _stream(stream)))


def mole_lookup_combine_grouped_mapped(ids, h, w_r, lut_host, y, workspace, stream=None) -> None:
    """The grouped combine reading the table in place from page-locked host
    memory (lut_host: a pinned bf16 CPU tensor [V,N,D]); the rest on the device."""
    V, N, D = lut_host.shape
    T = ids.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64, "ids int64")
    _need(h.dtype == lut_host.dtype == w_r.dtype and y.dtype == torch.float32,
          "h, w_r, lut_host share one dtype; y float32")
    _need(not lut_host.is_cuda, "lut_host in host memory")
    for t in (ids, h, w_r, lut_host, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mole_lookup_combine_grouped_mapped", library().mole_lookup_combine_grouped_mapped(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut_host), _ptr(y), T, V, D, N, _dtype(h), _ptr(workspace),
        ws_bytes, _stream(stream)))


def _nf3_grouped(fn, ids, h, w_r, codes, scales, y, workspace, stream):
    V, N, CB = codes.shape
    D = CB * 8 // 3
    T = ids.numel()
    _need(tuple(scales.shape) == (V, N, D // 64), "scales [V,N,D/64]")
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype,
          "ids int64, y float32, h and w_r one dtype")
    for t in (ids, h, w_r, codes, scales, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn, getattr(library(), fn)(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(codes), _ptr(scales), _ptr(y), T, V, D, N, _dtype(h), _ptr(workspace),
        ws_bytes, _stream(stream)))


def mole_lookup_combine_nf3_grouped(ids, h, w_r, codes, scales, y, workspace, stream=None) -> None:
    """NF3 combine over the batch grouped by id on the device (workspace:
    mole_lookup_combine_grouped_workspace_size(T) bytes on the device)."""
    _nf3_grouped("mole_lookup_combine_nf3_grouped", ids, h, w_r, codes, scales, y, workspace, stream)


def mole_lookup_combine_nf3_grouped_mapped(ids, h, w_r, codes_host, scales_host, y, workspace, stream=None) -> None:
    """The same with the NF3 table in page-locked host memory, read in place."""
    _need(not codes_host.is_cuda and not scales_host.is_cuda, "codes_host and scales_host in host memory")
    _nf3_grouped("mole_lookup_combine_nf3_grouped_mapped", ids, h, w_r, codes_host, scales_host, y, workspace,
                 stream)


def mole_lookup_combine_grouped_noalloc(ids, h, w_r, lut, y, stream=None) -> None:
    """mole_lookup_combine_grouped with the library's static device workspace
    (no allocation; up to MOLE_GROUPED_NOALLOC_MAX_T tokens)."""
    V, N, D = lut.shape
    T = ids.numel()
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64, "ids int64")
    _need(h.dtype == lut.dtype == w_r.dtype and y.dtype == torch.float32, "h, w_r, lut share one dtype; y float32")
    for t in (ids, h, w_r, lut, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_grouped_noalloc", library().mole_lookup_combine_grouped_noalloc(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut), _ptr(y), T, V, D, N, _dtype(lut), _stream(stream)))


MOLE_GROUPED_NOALLOC_MAX_T = 65536


def mole_nf3_file_write(path: str, codes_host, scales_host) -> None:
    """Write a packed NF3 table (codes [V,N,3D/8] uint8, scales [V,N,D/64]
    fp16 bits, host tensors) to `path` as a table file: a 64-byte header,
    then one record (codes, then scales) per vocabulary row."""
    V, N, CB = codes_host.shape
    D = CB * 8 // 3
    for t in (codes_host, scales_host):
        _need(t.device.type == "cpu" and t.is_contiguous(), "host tensors, contiguous")
    _need(tuple(scales_host.shape) == (V, N, D // 64), "scales [V,N,D/64]")
    _check("mole_nf3_file_write", library().mole_nf3_file_write(
        os.fsencode(path), _ptr(codes_host), _ptr(scales_host), V, N, D))


def mole_nf3_file_shape(fd: int):
    """(V, N, D) from the header of an open table file."""
    V, N, D = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check("mole_nf3_file_shape", library().mole_nf3_file_shape(
        int(fd), ctypes.addressof(V), ctypes.addressof(N), ctypes.addressof(D)))
    return int(V.value), int(N.value), int(D.value)


def mole_gather_nf3_file(fd: int, ids_host, V: int, N: int, D: int, codes_stage, scales_stage, remap,
                         nthreads: int = 0) -> int:
    """As mole_gather_nf3_host, with the rows read from the open table file
    `fd`; returns the number of distinct ids U."""
    T = ids_host.numel()
    for t in (ids_host, codes_stage, scales_stage, remap):
        _need(t.device.type == "cpu" and t.is_contiguous(), "host tensors, contiguous")
    _need(codes_stage.numel() >= T * N * (3 * D // 8) and scales_stage.numel() >= T * N * (D // 64)
          and remap.numel() >= T, "staging buffers hold at least T rows")
    u = ctypes.c_int64(0)
    _check("mole_gather_nf3_file", library().mole_gather_nf3_file(
        int(fd), _ptr(ids_host), T, V, N, D, _ptr(codes_stage), _ptr(scales_stage), _ptr(remap),
        ctypes.addressof(u), nthreads))
    return int(u.value)


def mole_lookup_combine_nf3_file(fd: int, ids_host, h, w_r, V: int, stage_host, stage_dev, y,
                                 nthreads: int = 0, stream=None) -> int:
    """Disk-resident NF3 table: read the requested rows from the open table
    file `fd` into the pinned staging area, copy its used part to the device
    buffer in one transfer and combine.  Returns U, the number of distinct
    ids."""
    T, D = h.shape
    N = w_r.shape[0]
    _need(tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D), "h [T,D], w_r [N,D], y [T,D]")
    nbytes = stage_host.numel() * stage_host.element_size()
    _need(stage_dev.numel() * stage_dev.element_size() >= nbytes, "device staging as large as the host one")
    u = ctypes.c_int64(0)
    _check("mole_lookup_combine_nf3_file", library().mole_lookup_combine_nf3_file(
        int(fd), _ptr(ids_host), _ptr(h), _ptr(w_r), _ptr(stage_host), _ptr(stage_dev), nbytes, _ptr(y), T, V,
        D, N, _dtype(h), nthreads, ctypes.addressof(u), _stream(stream)))
    return int(u.value)


def mole_layer_workspace_size(T: int, D: int, F: int) -> int:
    """Workspace bytes mole_layer_forward needs for T tokens (0 for T == 0)."""
    out = ctypes.c_size_t(0)
    _check("mole_layer_workspace_size",
           library().mole_layer_workspace_size(T, D, F, ctypes.addressof(out)))
    return int(out.value)


def mole_layer_forward(ids, h, w_r, lut, w_s_up, w_s_down, x, workspace, stream=None) -> None:
    """The MoLE block in place on the residual stream x [T,D] (fp32):
    x += W_s_down . GELU(W_s_up . h) + sum_e softmax(w_r . h)[e] * lut[ids, e, :].
    h [T,D], w_r [N,D], lut [V,N,D], w_s_up [F,D], w_s_down [D,F] (bf16);
    workspace: a uint8 device tensor of mole_layer_workspace_size(T, D, F) bytes."""
    V, N, D = lut.shape
    T = ids.numel()
    _need(w_s_up.dim() == 2 and w_s_down.dim() == 2, "w_s_up [F,D], w_s_down [D,F]")
    F = w_s_up.shape[0]
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(x.shape) == (T, D)
          and tuple(w_s_up.shape) == (F, D) and tuple(w_s_down.shape) == (D, F),
          "ids [T], h [T,D], w_r [N,D], lut [V,N,D], w_s_up [F,D], w_s_down [D,F], x [T,D]")
    _need(ids.dtype == torch.int64 and x.dtype == torch.float32, "ids int64, x float32")
    _need(h.dtype == w_r.dtype == lut.dtype == w_s_up.dtype == w_s_down.dtype,
          "h, w_r, lut and the shared weights share one dtype")
    for t in (ids, h, w_r, lut, w_s_up, w_s_down, x):
        _need(t.is_contiguous(), "tensors must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mole_layer_forward", library().mole_layer_forward(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(lut), _ptr(w_s_up), _ptr(w_s_down), _ptr(x),
        T, V, D, N, F, _dtype(h), _ptr(workspace), ws_bytes, _stream(stream)))


def mole_nf4_levels() -> list:
    out = (ctypes.c_float * 16)()
    _check("mole_nf4_levels", library().mole_nf4_levels(ctypes.addressof(out)))
    return list(out)


def mole_pack_nf4(lut, codes, scales, stream=None) -> None:
    """NF4-encode lut [V,N,D] into codes [V,N,D/2] (uint8) and scales
    [V,N,D/64] (fp16 bits, int16/uint16 tensor)."""
    V, N, D = lut.shape
    _need(D % 64 == 0, "D must be a multiple of 64")
    _need(tuple(codes.shape) == (V, N, D // 2) and codes.dtype == torch.uint8, "codes [V,N,D/2] uint8")
    _need(tuple(scales.shape) == (V, N, D // 64) and scales.element_size() == 2, "scales [V,N,D/64] 16-bit")
    for t in (lut, codes, scales):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_pack_nf4", library().mole_pack_nf4(
        _ptr(lut), _ptr(codes), _ptr(scales), V, N, D, _dtype(lut), _stream(stream)))


def mole_lookup_combine_nf4(ids, h, w_r, codes, scales, y, stream=None) -> None:
    V, N, CB = codes.shape
    D = CB * 2
    T = ids.numel()
    _need(tuple(scales.shape) == (V, N, D // 64), "scales [V,N,D/64]")
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype,
          "ids int64, y float32, h and w_r one dtype")
    for t in (ids, h, w_r, codes, scales, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_nf4", library().mole_lookup_combine_nf4(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(codes), _ptr(scales), _ptr(y), T, V, D, N,
        _dtype(h), _stream(stream)))


def mole_pack_int8(lut, codes, scales, stream=None) -> None:
    """int8-encode lut [V,N,D] into codes [V,N,D] (int8) and one fp32 scale
    per row, scales [V,N]."""
    V, N, D = lut.shape
    _need(D % 64 == 0, "D must be a multiple of 64")
    _need(tuple(codes.shape) == (V, N, D) and codes.dtype == torch.int8, "codes [V,N,D] int8")
    _need(tuple(scales.shape) == (V, N) and scales.dtype == torch.float32, "scales [V,N] float32")
    for t in (lut, codes, scales):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_pack_int8", library().mole_pack_int8(
        _ptr(lut), _ptr(codes), _ptr(scales), V, N, D, _dtype(lut), _stream(stream)))


def mole_lookup_combine_int8(ids, h, w_r, codes, scales, y, stream=None) -> None:
    V, N, D = codes.shape
    T = ids.numel()
    _need(tuple(scales.shape) == (V, N) and scales.dtype == torch.float32, "scales [V,N] float32")
    _need(codes.dtype == torch.int8, "codes int8")
    _need(tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D) and tuple(y.shape) == (T, D),
          "ids [T], h [T,D], w_r [N,D], y [T,D]")
    _need(ids.dtype == torch.int64 and y.dtype == torch.float32 and h.dtype == w_r.dtype,
          "ids int64, y float32, h and w_r one dtype")
    for t in (ids, h, w_r, codes, scales, y):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_lookup_combine_int8", library().mole_lookup_combine_int8(
        _ptr(ids), _ptr(h), _ptr(w_r), _ptr(codes), _ptr(scales), _ptr(y), T, V, D, N,
        _dtype(h), _stream(stream)))


def mole_train_index(ids_host, V: int):
    """Host-side batch index: (uniq [U], remap [T], row_ptr [U+1], tok [T]) as
    int64 CPU tensors (distinct ids in first-occurrence order, each token's
    row, and the tokens of each row grouped in token order)."""
    ids_host = ids_host.contiguous()
    _need(ids_host.dtype == torch.int64 and not ids_host.is_cuda, "ids_host: int64 CPU tensor")
    T = ids_host.numel()
    uniq = torch.empty(max(T, 1), dtype=torch.int64)
    remap = torch.empty(max(T, 1), dtype=torch.int64)
    row_ptr = torch.empty(T + 1, dtype=torch.int64)
    tok = torch.empty(max(T, 1), dtype=torch.int64)
    U = ctypes.c_int64(0)
    _check("mole_train_index", library().mole_train_index(
        _ptr(ids_host), T, V, _ptr(uniq), _ptr(remap), _ptr(row_ptr), _ptr(tok), ctypes.addressof(U)))
    u = int(U.value)
    return uniq[:u].clone(), remap[:T].clone(), row_ptr[:u + 1].clone(), tok[:T].clone()


def mole_train_workspace_size(T: int, U: int, D: int, F: int, N: int):
    """(forward workspace bytes, backward scratch bytes) for training mode."""
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("mole_train_workspace_size", library().mole_train_workspace_size(
        T, U, D, F, N, ctypes.addressof(f), ctypes.addressof(b)))
    return int(f.value), int(b.value)


def mole_train_forward(uniq, remap, emb, w_up, w_down, h, w_r, y, fwd_ws, stream=None) -> None:
    """Training-mode forward: y[t] = sum_e softmax(w_r . h[t])[e] FFN_e(emb[ids[t]]), with the
    batch given by (uniq, remap) on the device; fwd_ws keeps what the backward pass needs."""
    V, D = emb.shape
    N, F, _ = w_up.shape
    T, U = remap.numel(), uniq.numel()
    _need(tuple(w_down.shape) == (N, D, F) and tuple(h.shape) == (T, D) and tuple(w_r.shape) == (N, D)
          and tuple(y.shape) == (T, D), "emb [V,D], w_up [N,F,D], w_down [N,D,F], h [T,D], w_r [N,D], y [T,D]")
    _need(y.dtype == torch.float32 and uniq.dtype == remap.dtype == torch.int64, "y float32, uniq/remap int64")
    for t in (uniq, remap, emb, w_up, w_down, h, w_r, y, fwd_ws):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_train_forward", library().mole_train_forward(
        _ptr(uniq), _ptr(remap), _ptr(emb), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(w_r), _ptr(y), T, U, V, D, F,
        N, _dtype(emb), _ptr(fwd_ws), fwd_ws.numel() * fwd_ws.element_size(), _stream(stream)))


def mole_train_backward(remap, row_ptr, tok, U: int, V: int, w_up, w_down, h, w_r, dy, fwd_ws, bwd_ws,
                        d_w_up, d_w_down, d_w_r, d_h, d_x, stream=None) -> None:
    """Training-mode backward for the upstream gradient dy [T,D]; outputs are fp32 tensors
    d_w_up [N,F,D], d_w_down [N,D,F], d_w_r [N,D], d_h [T,D], d_x [U,D] (embedding rows)."""
    N, F, D = w_up.shape
    T = remap.numel()
    _need(tuple(d_w_up.shape) == (N, F, D) and tuple(d_w_down.shape) == (N, D, F) and tuple(d_w_r.shape) == (N, D)
          and tuple(d_h.shape) == (T, D) and tuple(d_x.shape) == (U, D) and tuple(dy.shape) == (T, D),
          "gradient shapes")
    for t in (remap, row_ptr, tok, w_up, w_down, h, w_r, dy, fwd_ws, bwd_ws, d_w_up, d_w_down, d_w_r, d_h, d_x):
        _need(t.is_contiguous(), "tensors must be contiguous")
    _check("mole_train_backward", library().mole_train_backward(
        _ptr(remap), _ptr(row_ptr), _ptr(tok), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(w_r), _ptr(dy),
        _ptr(fwd_ws), fwd_ws.numel() * fwd_ws.element_size(), _ptr(bwd_ws), bwd_ws.numel() * bwd_ws.element_size(),
        _ptr(d_w_up), _ptr(d_w_down), _ptr(d_w_r), _ptr(d_h), _ptr(d_x), T, U, V, D, F, N, _dtype(w_up),
        _stream(stream)))
