"""Plain CPU oracle for the MoLE hot path (ctypes wrapper over mole_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares no code with the HIP library.

The arithmetic lives in ``mole_oracle.c`` (fp64, plain loops, OpenMP over
rows/tokens); this module only compiles it with gcc, loads it and marshals
numpy arrays.  bf16 tensors are passed as ``numpy.uint16`` bit patterns.

Definitions followed (MoLE article, the "ICML 2025 Spotlight | MoLE" page):
  * inference section -- LUT[v,e,:] = FFN_e(Emb[v]) over the whole
    vocabulary, then retrieval of each token's rows by id;
  * training section -- all routed experts active, router on the contextual
    hidden state: gates = softmax(W_r h) over all N experts;
  * results section -- the table compressed to 3 bits ("e.g. NF3");
  * results section ("redundancy remains at 3 bits") -- other table formats:
    NF4 (the same construction at 4 bits) and int8 with one scale per row;
  * training section -- the training-mode forward (every expert on the
    token's embedding, dense gates) and its backward pass (``train_forward``,
    ``train_backward``);
  * training section and complexity analysis -- shared experts keep reading
    the contextual hidden state and are the only experts still computed at
    inference, so a MoLE block adds shared FFN + routed lookup to the
    residual stream (``shared_ffn``, ``layer_forward``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mole_oracle.c")
_LIB = os.path.join(_HERE, "libmole_oracle.so")

F32, BF16 = 0, 1

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile mole_oracle.c with gcc (fp64, no fast-math, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "oracle_max_threads": (I, []),
            "oracle_gelu": (D, [D]),
            "oracle_normal_ppf": (D, [D]),
            "oracle_build_lut_rows": (I, [P, P, P, I, I64, I64, I64, I64, P, I64, P, I]),
            "oracle_router_gates": (I, [P, P, I, I64, I64, I64, P, I]),
            "oracle_lookup_combine": (I, [P, P, P, I, P, I, I64, I64, I64, I64, P, I]),
            "oracle_nf3_levels": (None, [P]),
            "oracle_nf3_midpoints": (None, [P]),
            "oracle_f32_to_f16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "oracle_pack_nf3": (I, [P, I, I64, I64, P, P, P, I]),
            "oracle_unpack_nf3": (I, [P, I64, I64, P]),
            "oracle_dequant_nf3": (I, [P, P, I64, I64, P]),
            "oracle_lookup_combine_nf3": (I, [P, P, P, I, P, P, I64, I64, I64, I64, P, I]),
            "oracle_shared_ffn": (I, [P, P, P, I, I64, I64, I64, P, I]),
            "oracle_nf4_levels": (None, [P]),
            "oracle_nf4_midpoints": (None, [P]),
            "oracle_pack_nf4": (I, [P, I, I64, I64, P, P, P, I]),
            "oracle_unpack_nf4": (I, [P, I64, I64, P]),
            "oracle_dequant_nf4": (I, [P, P, I64, I64, P]),
            "oracle_pack_int8": (I, [P, I, I64, I64, P, P, I]),
            "oracle_dequant_int8": (I, [P, P, I64, I64, P]),
            "oracle_lookup_combine_q": (I, [I, P, P, P, I, P, P, I64, I64, I64, I64, P, I]),
            "oracle_train_forward": (I, [P, P, P, P, P, P, I, I64, I64, I64, I64, I64, P, I]),
            "oracle_train_backward": (I, [P, P, P, P, P, P, I, P, I64, I64, I64, I64, I64, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle takes float32 or bf16-as-uint16 arrays, got %s" % a.dtype)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("%s failed with oracle status %d" % (what, rc))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gelu(u: float) -> float:
    return float(_load().oracle_gelu(float(u)))


def normal_ppf(p: float) -> float:
    return float(_load().oracle_normal_ppf(float(p)))


def build_lut_rows(emb, w_up, w_down, rows=None, nthreads: int = 0) -> np.ndarray:
    """LUT rows in fp64: out[r, e, :] = W_down[e] . GELU(W_up[e] . Emb[rows[r]]).

    emb [V,D], w_up [N,F,D], w_down [N,D,F], all float32 or all bf16 (uint16).
    """
    V, D = emb.shape
    N, F, D2 = w_up.shape
    assert D2 == D and w_down.shape == (N, D, F)
    dt = _dtype_code(emb)
    assert _dtype_code(w_up) == dt and _dtype_code(w_down) == dt
    rows = np.arange(V, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, N, D), dtype=np.float64)
    rc = _load().oracle_build_lut_rows(_ptr(emb), _ptr(w_up), _ptr(w_down), dt, V, D, F, N,
                                       _ptr(rows), rows.size, _ptr(out), nthreads)
    _check(rc, "build_lut_rows")
    return out


def router_gates(h, w_r, nthreads: int = 0) -> np.ndarray:
    """gates[t, e] = softmax_e(W_r[e] . h[t]) in fp64.  h [T,D], w_r [N,D]."""
    T, D = h.shape
    N, D2 = w_r.shape
    assert D2 == D
    dt = _dtype_code(h)
    assert _dtype_code(w_r) == dt
    out = np.zeros((T, N), dtype=np.float64)
    _check(_load().oracle_router_gates(_ptr(h), _ptr(w_r), dt, T, D, N, _ptr(out), nthreads),
           "router_gates")
    return out


def lookup_combine(ids, h, w_r, lut, nthreads: int = 0) -> np.ndarray:
    """y[t, :] = sum_e gates[t, e] * lut[ids[t], e, :] in fp64.  lut [V,N,D]."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    T = ids.size
    V, N, D = lut.shape
    assert h.shape == (T, D) and w_r.shape == (N, D)
    dt = _dtype_code(h)
    assert _dtype_code(w_r) == dt
    y = np.zeros((T, D), dtype=np.float64)
    rc = _load().oracle_lookup_combine(_ptr(ids), _ptr(h), _ptr(w_r), dt, _ptr(lut),
                                       _dtype_code(lut), T, V, D, N, _ptr(y), nthreads)
    _check(rc, "lookup_combine")
    return y


def nf3_levels() -> np.ndarray:
    out = np.zeros(8, dtype=np.float32)
    _load().oracle_nf3_levels(_ptr(out))
    return out


def nf3_midpoints() -> np.ndarray:
    out = np.zeros(7, dtype=np.float32)
    _load().oracle_nf3_midpoints(_ptr(out))
    return out


def f32_to_f16_rne(x: float) -> int:
    return int(_load().oracle_f32_to_f16_rne(float(np.float32(x))))


def f16_to_f32(bits: int) -> float:
    return float(_load().oracle_f16_to_f32(int(bits)))


def pack_nf3(table, nthreads: int = 0):
    """Encode a [..., D] table to NF3.  Returns (codes uint8 [..., 3D/8],
    scales uint16 (fp16 bits) [..., D/64], number of saturated blocks)."""
    D = table.shape[-1]
    lead = table.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    t2 = np.ascontiguousarray(table.reshape(rows, D))
    codes = np.zeros((rows, 3 * D // 8), dtype=np.uint8)
    scales = np.zeros((rows, D // 64), dtype=np.uint16)
    nsat = ctypes.c_int64(0)
    rc = _load().oracle_pack_nf3(_ptr(t2), _dtype_code(t2), rows, D, _ptr(codes), _ptr(scales),
                                 ctypes.addressof(nsat), nthreads)
    _check(rc, "pack_nf3")
    return codes.reshape(*lead, 3 * D // 8), scales.reshape(*lead, D // 64), int(nsat.value)


def unpack_nf3(codes, D: int) -> np.ndarray:
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    c2 = np.ascontiguousarray(codes.reshape(rows, 3 * D // 8))
    out = np.zeros((rows, D), dtype=np.uint8)
    _check(_load().oracle_unpack_nf3(_ptr(c2), rows, D, _ptr(out)), "unpack_nf3")
    return out.reshape(*lead, D)


def dequant_nf3(codes, scales, D: int) -> np.ndarray:
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    c2 = np.ascontiguousarray(codes.reshape(rows, 3 * D // 8))
    s2 = np.ascontiguousarray(scales.reshape(rows, D // 64))
    out = np.zeros((rows, D), dtype=np.float64)
    _check(_load().oracle_dequant_nf3(_ptr(c2), _ptr(s2), rows, D, _ptr(out)), "dequant_nf3")
    return out.reshape(*lead, D)


def lookup_combine_nf3(ids, h, w_r, codes, scales, nthreads: int = 0) -> np.ndarray:
    """y[t, d] = sum_e gates[t, e] * level[code] * scale over the NF3 table.
    codes [V,N,3D/8] uint8, scales [V,N,D/64] uint16 (fp16 bits)."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    T = ids.size
    V, N, CB = codes.shape
    D = CB * 8 // 3
    assert scales.shape == (V, N, D // 64)
    assert h.shape == (T, D) and w_r.shape == (N, D)
    dt = _dtype_code(h)
    y = np.zeros((T, D), dtype=np.float64)
    rc = _load().oracle_lookup_combine_nf3(_ptr(ids), _ptr(h), _ptr(w_r), dt, _ptr(codes),
                                           _ptr(scales), T, V, D, N, _ptr(y), nthreads)
    _check(rc, "lookup_combine_nf3")
    return y


def shared_ffn(h, w_s_up, w_s_down, nthreads: int = 0) -> np.ndarray:
    """out[t, :] = W_s_down . GELU(W_s_up . h[t]) in fp64 (exact-form GELU,
    no biases).  h [T,D], w_s_up [F,D], w_s_down [D,F], one dtype."""
    T, D = h.shape
    F, D2 = w_s_up.shape
    assert D2 == D and w_s_down.shape == (D, F)
    dt = _dtype_code(h)
    assert _dtype_code(w_s_up) == dt and _dtype_code(w_s_down) == dt
    out = np.zeros((T, D), dtype=np.float64)
    _check(_load().oracle_shared_ffn(_ptr(h), _ptr(w_s_up), _ptr(w_s_down), dt, T, D, F,
                                     _ptr(out), nthreads), "shared_ffn")
    return out


def layer_forward(ids, h, w_r, lut, w_s_up, w_s_down, x=None, nthreads: int = 0) -> np.ndarray:
    """One MoLE block at inference, in fp64:
        out[t, :] = x[t, :] + shared_ffn(h)[t, :] + lookup_combine(ids, h, w_r, lut)[t, :]
    (the residual stream x, fp32 [T,D], is taken as zero when None).  The
    shared expert and the router read the contextual hidden state h; the
    routed experts are the table lookups."""
    out = shared_ffn(h, w_s_up, w_s_down, nthreads) + lookup_combine(ids, h, w_r, lut, nthreads)
    if x is not None:
        assert x.shape == out.shape and x.dtype == np.float32
        out = out + x.astype(np.float64)
    return out


def nf4_levels() -> np.ndarray:
    out = np.zeros(16, dtype=np.float32)
    _load().oracle_nf4_levels(_ptr(out))
    return out


def nf4_midpoints() -> np.ndarray:
    out = np.zeros(15, dtype=np.float32)
    _load().oracle_nf4_midpoints(_ptr(out))
    return out


def pack_nf4(table, nthreads: int = 0):
    """Encode a [..., D] table to NF4.  Returns (codes uint8 [..., D/2],
    scales uint16 (fp16 bits) [..., D/64], number of saturated blocks)."""
    D = table.shape[-1]
    lead = table.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    t2 = np.ascontiguousarray(table.reshape(rows, D))
    codes = np.zeros((rows, D // 2), dtype=np.uint8)
    scales = np.zeros((rows, D // 64), dtype=np.uint16)
    nsat = ctypes.c_int64(0)
    _check(_load().oracle_pack_nf4(_ptr(t2), _dtype_code(t2), rows, D, _ptr(codes), _ptr(scales),
                                   ctypes.addressof(nsat), nthreads), "pack_nf4")
    return codes.reshape(*lead, D // 2), scales.reshape(*lead, D // 64), int(nsat.value)


def unpack_nf4(codes, D: int) -> np.ndarray:
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    c2 = np.ascontiguousarray(codes.reshape(rows, D // 2))
    out = np.zeros((rows, D), dtype=np.uint8)
    _check(_load().oracle_unpack_nf4(_ptr(c2), rows, D, _ptr(out)), "unpack_nf4")
    return out.reshape(*lead, D)


def dequant_nf4(codes, scales, D: int) -> np.ndarray:
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    c2 = np.ascontiguousarray(codes.reshape(rows, D // 2))
    s2 = np.ascontiguousarray(scales.reshape(rows, D // 64))
    out = np.zeros((rows, D), dtype=np.float64)
    _check(_load().oracle_dequant_nf4(_ptr(c2), _ptr(s2), rows, D, _ptr(out)), "dequant_nf4")
    return out.reshape(*lead, D)


def pack_int8(table, nthreads: int = 0):
    """Encode a [..., D] table to int8 with one fp32 scale per row.
    Returns (codes int8 [..., D], scales float32 [...])."""
    D = table.shape[-1]
    lead = table.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    t2 = np.ascontiguousarray(table.reshape(rows, D))
    codes = np.zeros((rows, D), dtype=np.int8)
    scales = np.zeros(rows, dtype=np.float32)
    _check(_load().oracle_pack_int8(_ptr(t2), _dtype_code(t2), rows, D, _ptr(codes), _ptr(scales),
                                    nthreads), "pack_int8")
    return codes.reshape(*lead, D), scales.reshape(lead)


def dequant_int8(codes, scales) -> np.ndarray:
    D = codes.shape[-1]
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    c2 = np.ascontiguousarray(codes.reshape(rows, D))
    s2 = np.ascontiguousarray(scales.reshape(rows)).astype(np.float32)
    out = np.zeros((rows, D), dtype=np.float64)
    _check(_load().oracle_dequant_int8(_ptr(c2), _ptr(s2), rows, D, _ptr(out)), "dequant_int8")
    return out.reshape(*lead, D)


def _lookup_combine_q(fmt, ids, h, w_r, codes, scales, D, nthreads):
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    T = ids.size
    V, N = codes.shape[:2]
    assert h.shape == (T, D) and w_r.shape == (N, D)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    y = np.zeros((T, D), dtype=np.float64)
    _check(_load().oracle_lookup_combine_q(fmt, _ptr(ids), _ptr(h), _ptr(w_r), _dtype_code(h), _ptr(codes),
                                           _ptr(scales), T, V, D, N, _ptr(y), nthreads),
           "lookup_combine_q")
    return y


def lookup_combine_nf4(ids, h, w_r, codes, scales, nthreads: int = 0) -> np.ndarray:
    """y over the NF4 table: codes [V,N,D/2] uint8, scales [V,N,D/64] uint16 (fp16 bits)."""
    D = codes.shape[2] * 2
    assert scales.shape == codes.shape[:2] + (D // 64,)
    return _lookup_combine_q(4, ids, h, w_r, codes, scales.astype(np.uint16), D, nthreads)


def lookup_combine_int8(ids, h, w_r, codes, scales, nthreads: int = 0) -> np.ndarray:
    """y over the int8 table: codes [V,N,D] int8, scales [V,N] float32."""
    D = codes.shape[2]
    assert scales.shape == codes.shape[:2]
    return _lookup_combine_q(8, ids, h, w_r, codes, scales.astype(np.float32), D, nthreads)


def train_forward(ids, emb, w_up, w_down, h, w_r, nthreads: int = 0) -> np.ndarray:
    """y[t] = sum_e softmax(W_r . h[t])[e] * W_down[e] . GELU(W_up[e] . Emb[ids[t]]), fp64.
    emb [V,D], w_up [N,F,D], w_down [N,D,F], h [T,D], w_r [N,D], one dtype."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    T = ids.size
    V, D = emb.shape
    N, F, _ = w_up.shape
    dt = _dtype_code(emb)
    for a in (w_up, w_down, h, w_r):
        assert _dtype_code(a) == dt
    y = np.zeros((T, D), dtype=np.float64)
    _check(_load().oracle_train_forward(_ptr(ids), _ptr(emb), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(w_r), dt,
                                        T, V, D, F, N, _ptr(y), nthreads), "train_forward")
    return y


def train_backward(ids, emb, w_up, w_down, h, w_r, dy):
    """Gradients of sum(dy * train_forward(...)) in fp64: a dict with
    d_w_up [N,F,D], d_w_down [N,D,F], d_w_r [N,D], d_h [T,D], d_emb [V,D]."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    T = ids.size
    V, D = emb.shape
    N, F, _ = w_up.shape
    dt = _dtype_code(emb)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy.shape == (T, D)
    out = {"d_w_up": np.zeros((N, F, D)), "d_w_down": np.zeros((N, D, F)), "d_w_r": np.zeros((N, D)),
           "d_h": np.zeros((T, D)), "d_emb": np.zeros((V, D))}
    _check(_load().oracle_train_backward(_ptr(ids), _ptr(emb), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(w_r), dt,
                                         _ptr(dy), T, V, D, F, N, _ptr(out["d_w_up"]), _ptr(out["d_w_down"]),
                                         _ptr(out["d_w_r"]), _ptr(out["d_h"]), _ptr(out["d_emb"])),
           "train_backward")
    return out
