"""CPU oracle for the KDA prefill chunk solver (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (``tril_solve_amd``)
never imports, loads or calls it, and it imports nothing from there.

It evaluates the plain definition of what LightLLM PR #1703 ("perf(kda):
parallelize diagonal solves in Prefill", PR description) computes: for every
64-token chunk and head, X = (I + A)^-1 with A the strictly-lower intra-chunk
matrix, by fp64 column forward substitution (``tril_oracle.c``). Inputs in
float32, bfloat16 or binary16 are upcast to float64 exactly before the solve.

For the fused path that first builds A from keys, cumulative log-decays and
write strengths, ``kkt_*`` evaluate A from its definition in float64 and
``kkt_tril_inv_*`` invert that A without rounding it.

``kda_decode`` is one step of the fused KDA decode core (causal convolution
with its state, the KDA recurrent update, gated RMSNorm) from its definition.

Pins (each in ``tests/test_oracle_pins.py``): exact rational Neumann series,
the single-subdiagonal closed form, LAPACK inversion, the residual of
(I + A) X = I, the leading-principal-block property for partial chunks,
hand-derived chunk maps (``tests/golden/``), and the bfloat16 and binary16
roundings against tables worked out by hand (plus torch's bfloat16 cast).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tril_oracle.c")
_LIB = os.path.join(_HERE, "libtril_oracle.so")
CHUNK = 64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP). Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        ci = ctypes.c_int
        lib.oracle_chunks_packed_c.restype = i64
        lib.oracle_chunks_packed_c.argtypes = [p, i64, ci, p, p, p, i64]
        lib.oracle_inv_unit_lower_w.restype = None
        lib.oracle_inv_unit_lower_w.argtypes = [p, i64, ci, ci, p, i64]
        lib.oracle_tril_inv_packed_c.restype = i64
        lib.oracle_tril_inv_packed_c.argtypes = [p, p, p, i64, i64, i32, ci, ci]
        lib.oracle_tril_inv_dense_c.restype = i64
        lib.oracle_tril_inv_dense_c.argtypes = [p, p, i64, i64, i32, ci, ci]
        lib.oracle_kkt_packed.restype = i64
        lib.oracle_kkt_packed.argtypes = [p, p, p, p, p, i64, i64, i32, ci, ci]
        lib.oracle_kkt_dense.restype = i64
        lib.oracle_kkt_dense.argtypes = [p, p, p, p, i64, i64, i32, ci, ci]
        lib.oracle_kda_decode.restype = ctypes.c_int
        lib.oracle_kda_decode.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i32, ci, ci,
                                          ctypes.c_double, ctypes.c_double]
        lib.oracle_rne_bf16.restype = None
        lib.oracle_rne_bf16.argtypes = [p, p, i64]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the OpenMP loops use by default (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a materialised input to float64.

    ``dtype`` is "f32" (a float32 array), "bf16" (a uint16/int16 array of
    bfloat16 bit patterns: the value is those 16 bits followed by 16 zero bits
    of a binary32) or "f16" (IEEE binary16 values or bit patterns).
    """
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.ascontiguousarray(a).view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(a).view(np.float16).astype(np.float64)
    if dtype == "f64":
        return np.ascontiguousarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def chunks_packed(cu_seqlens, chunk: int = CHUNK) -> np.ndarray:
    """Chunks of a packed batch: int64 array of rows (seq, start, length)."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = cu.shape[0] - 1
    lib = _load()
    n = lib.oracle_chunks_packed_c(_ptr(cu), nseq, chunk, None, None, None, 0)
    if n < 0:
        raise ValueError("malformed cu_seqlens")
    seq = np.zeros(n, np.int64)
    start = np.zeros(n, np.int64)
    ln = np.zeros(n, np.int32)
    lib.oracle_chunks_packed_c(_ptr(cu), nseq, chunk, _ptr(seq), _ptr(start), _ptr(ln), n)
    return np.stack([seq, start, ln.astype(np.int64)], axis=1)


def inv_unit_lower(M: np.ndarray, width: int = CHUNK) -> np.ndarray:
    """(I + M)^-1 for one L x L matrix (only the strictly-lower part of M is
    read). Returns an L x width float64 array: full-width output rows of a
    chunk of ``width`` tokens (L <= width <= 64)."""
    M = np.ascontiguousarray(M, dtype=np.float64)
    L = M.shape[0]
    if M.ndim != 2 or M.shape[1] < L or L > width or width > CHUNK:
        raise ValueError("M must be L x >=L with L <= width <= 64")
    X = np.zeros((L, width), np.float64)
    _load().oracle_inv_unit_lower_w(_ptr(M), M.shape[1], L, width, _ptr(X), width)
    return X


def tril_inv_packed(A: np.ndarray, cu_seqlens, dtype: str = "f32", nthreads: int = 0,
                    fill: float = np.nan) -> np.ndarray:
    """Oracle X for a packed [T, H, C] input (chunks of C = A.shape[-1]
    tokens). Rows outside every chunk hold ``fill``."""
    A64 = to_f64(A, dtype)
    T, H, C = A64.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    X = np.full((T, H, C), fill, np.float64)
    r = _load().oracle_tril_inv_packed_c(_ptr(A64), _ptr(X), _ptr(cu), cu.shape[0] - 1, T, H, C,
                                         nthreads)
    if r < 0:
        raise ValueError("malformed packed problem")
    return X


def tril_inv_dense(A: np.ndarray, dtype: str = "f32", nthreads: int = 0) -> np.ndarray:
    """Oracle X for a dense [B, T, H, C] input (chunks of C = A.shape[-1])."""
    A64 = to_f64(A, dtype)
    B, T, H, C = A64.shape
    X = np.full((B, T, H, C), np.nan, np.float64)
    r = _load().oracle_tril_inv_dense_c(_ptr(A64), _ptr(X), B, T, H, C, nthreads)
    if r < 0:
        raise ValueError("malformed dense problem")
    return X


def kkt_packed(k: np.ndarray, g: np.ndarray, beta: np.ndarray, cu_seqlens,
               k_dtype: str = "f32", nthreads: int = 0) -> np.ndarray:
    """The delta-rule matrix A [T, H, 64] (float64) of every 64-token chunk
    and head, from keys k [T, H, K] (``k_dtype``; beta has the same dtype),
    float32 cumulative log-decays g [T, H, K] and write strengths beta [T, H].
    Rows outside every chunk hold NaN."""
    k64 = to_f64(k, k_dtype)
    b64 = to_f64(beta, k_dtype)
    g64 = to_f64(g, "f32")
    T, H, K = k64.shape
    assert g64.shape == (T, H, K) and b64.shape == (T, H)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    A = np.full((T, H, CHUNK), np.nan, np.float64)
    r = _load().oracle_kkt_packed(_ptr(k64), _ptr(g64), _ptr(b64), _ptr(A), _ptr(cu),
                                  cu.shape[0] - 1, T, H, K, nthreads)
    if r < 0:
        raise ValueError("malformed packed problem")
    return A


def kkt_dense(k: np.ndarray, g: np.ndarray, beta: np.ndarray, k_dtype: str = "f32",
              nthreads: int = 0) -> np.ndarray:
    """Dense counterpart of kkt_packed: k, g [B, T, H, K], beta [B, T, H]."""
    k64 = to_f64(k, k_dtype)
    b64 = to_f64(beta, k_dtype)
    g64 = to_f64(g, "f32")
    B, T, H, K = k64.shape
    A = np.full((B, T, H, CHUNK), np.nan, np.float64)
    r = _load().oracle_kkt_dense(_ptr(k64), _ptr(g64), _ptr(b64), _ptr(A), B, T, H, K, nthreads)
    if r < 0:
        raise ValueError("malformed dense problem")
    return A


def kkt_tril_inv_packed(k, g, beta, cu_seqlens, k_dtype: str = "f32",
                        nthreads: int = 0) -> np.ndarray:
    """Oracle of the fused path: A from its definition, kept in float64, then
    X = (I + A)^-1 per chunk-head. Returns X [T, H, 64] (NaN outside chunks)."""
    A = kkt_packed(k, g, beta, cu_seqlens, k_dtype, nthreads)
    return tril_inv_packed(A, cu_seqlens, "f64", nthreads)


def kkt_tril_inv_dense(k, g, beta, k_dtype: str = "f32", nthreads: int = 0) -> np.ndarray:
    A = kkt_dense(k, g, beta, k_dtype, nthreads)
    return tril_inv_dense(A, "f64", nthreads)


def kda_decode(qkv, g, beta, z, wn, cw, slot, S, cs, in_dtype: str = "f32",
               eps_l2: float = 1e-6, eps_norm: float = 1e-6):
    """One step of the fused KDA decode core in float64 (see
    ``oracle_kda_decode`` in tril_oracle.c for the definition and layouts).

    qkv [B, 3, H, d] and z [B, H, d] are in ``in_dtype`` (f32 array, or
    bfloat16 / binary16 bit patterns); g [B, H, d], beta [B, H], wn [d],
    cw [3, W, H, d], S [slots, H, d, d] and cs [slots, 3, H, W - 1, d] are
    float32 (or float64); slot [B] int32 (< 0: padding). Returns
    (out [B, H, d], S_new, cs_new) as float64 arrays; the inputs are not
    modified."""
    qkv64 = to_f64(qkv, in_dtype)
    z64 = to_f64(z, in_dtype)
    g64, b64, wn64, cw64 = (np.ascontiguousarray(a, dtype=np.float64) for a in (g, beta, wn, cw))
    S64 = np.array(S, dtype=np.float64, copy=True, order="C")
    cs64 = np.array(cs, dtype=np.float64, copy=True, order="C")
    sl = np.ascontiguousarray(slot, dtype=np.int32)
    B, three, H, d = qkv64.shape
    W = cw64.shape[1]
    assert three == 3 and cw64.shape == (3, W, H, d) and cs64.shape[1:] == (3, H, W - 1, d)
    assert S64.shape[1:] == (H, d, d) and g64.shape == (B, H, d) and b64.shape == (B, H)
    out = np.zeros((B, H, d), np.float64)
    r = _load().oracle_kda_decode(_ptr(qkv64), _ptr(g64), _ptr(b64), _ptr(z64), _ptr(wn64),
                                  _ptr(cw64), _ptr(sl), _ptr(S64), _ptr(cs64), _ptr(out), B, H, d,
                                  W, eps_l2, eps_norm)
    if r != 0:
        raise ValueError("malformed decode problem")
    return out, S64, cs64


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(bits.shape, np.uint16)
    _load().oracle_rne_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def rne_f16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even,
    overflow to infinity, gradual underflow); returns the uint16 bit
    patterns. numpy's float32 -> float16 conversion is this IEEE rounding;
    it is pinned against a table worked out by hand."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
