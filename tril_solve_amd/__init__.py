"""Python binding of the MI355X KDA chunk solver (libkda_tril.so).

Argument marshalling only: every step of the solve runs in the HIP kernels
behind the C ABI of ``include/kda_tril.h``. torch supplies device memory and
the current stream. There is no CPU fallback: if the library is missing or
fails to load, importing this package raises.

The functions named like the C entry points take torch tensors and forward
their data pointers (the chunk size C is the last dimension of A: 64 goes to
the 64-token entry points, 16 and 32 to the chunk-size ones); ``tril_inv`` is
the convenience form that allocates X (and the split workspace when needed)
with torch.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda_tril.so")

KDA_F32, KDA_BF16, KDA_F16 = 0, 1, 2
KDA_ALGO_AUTO, KDA_ALGO_FUSED, KDA_ALGO_SPLIT, KDA_ALGO_FUSED_VALU = 0, 1, 2, 3
KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = 0, -1, -2, -3, -4

ALGOS = {"auto": KDA_ALGO_AUTO, "fused": KDA_ALGO_FUSED, "split": KDA_ALGO_SPLIT,
         "fused_valu": KDA_ALGO_FUSED_VALU}
ALGO_NAMES = {v: k for k, v in ALGOS.items()}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python tril_solve_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_status_string.argtypes = [ctypes.c_int]
_lib.kda_tril_inv_workspace_size.restype = ctypes.c_int
_lib.kda_tril_inv_workspace_size.argtypes = [_i64, _i64, _i64, _i32, ctypes.c_int,
                                             ctypes.POINTER(_sz), ctypes.POINTER(ctypes.c_int)]
_lib.kda_tril_inv_dense.restype = ctypes.c_int
_lib.kda_tril_inv_dense.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i32, _p, _sz,
                                    ctypes.c_int, _p]
_lib.kda_tril_inv_packed.restype = ctypes.c_int
_lib.kda_tril_inv_packed.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _p, _i64, _i64, _i32, _p,
                                     _i64, _p, _sz, ctypes.c_int, _p]
_lib.kda_tril_auto_plan.restype = ctypes.c_int
_lib.kda_tril_auto_plan.argtypes = [_i64, _i64, _i32, _sz]
_lib.kda_tril_inv_dense_chunk.restype = ctypes.c_int
_lib.kda_tril_inv_dense_chunk.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i32,
                                          _i32, _p, _sz, ctypes.c_int, _p]
_lib.kda_tril_inv_packed_chunk.restype = ctypes.c_int
_lib.kda_tril_inv_packed_chunk.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _p, _i64, _i64,
                                           _i32, _i32, _p, _i64, _p, _sz, ctypes.c_int, _p]

_lib.kda_tril_inv_packed_noalloc.restype = ctypes.c_int
_lib.kda_tril_inv_packed_noalloc.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _p, _i64, _i64,
                                             _i32, _p, _i64, _p]

for _n in ("kda_kkt_tril_inv_packed", "kda_kkt_packed"):
    getattr(_lib, _n).restype = ctypes.c_int
    getattr(_lib, _n).argtypes = [_p, _p, _p, ctypes.c_int, _p, ctypes.c_int, _p, _i64, _i64, _i32,
                                  _i32, _p, _i64, _p]
for _n in ("kda_kkt_tril_inv_dense", "kda_kkt_dense"):
    getattr(_lib, _n).restype = ctypes.c_int
    getattr(_lib, _n).argtypes = [_p, _p, _p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i32,
                                  _i32, _p]

_lib.kda_decode_step.restype = ctypes.c_int
_lib.kda_decode_step.argtypes = [_p, _p, ctypes.c_int, _p, _p, _p, _p, _p, _p, _p, _i64, _p,
                                 ctypes.c_int, _i64, _i32, _i32, _i32, ctypes.c_float,
                                 ctypes.c_float, _p]

EXPORTED = ("kda_tril_inv_workspace_size", "kda_tril_inv_dense", "kda_tril_inv_packed",
            "kda_status_string", "kda_tril_auto_plan", "kda_tril_inv_dense_chunk",
            "kda_tril_inv_packed_chunk", "kda_kkt_tril_inv_packed", "kda_kkt_tril_inv_dense",
            "kda_kkt_packed", "kda_kkt_dense", "kda_decode_step", "kda_tril_inv_packed_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20
CHUNK_SIZES = (16, 32, 64)


class KdaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(kda_status_string(status))


def kda_status_string(status: int) -> str:
    return _lib.kda_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != KDA_OK:
        raise KdaError(status)


def _algo(a) -> int:
    return ALGOS[a] if isinstance(a, str) else int(a)


def kda_tril_inv_workspace_size(total_tokens: int, num_seqs: int, num_chunks: int,
                                num_heads: int, algo="auto"):
    """(workspace bytes, chosen algo name). Host only."""
    b = _sz(0)
    c = ctypes.c_int(0)
    _check(_lib.kda_tril_inv_workspace_size(total_tokens, num_seqs, num_chunks, num_heads,
                                            _algo(algo), ctypes.byref(b), ctypes.byref(c)))
    return int(b.value), ALGO_NAMES[c.value]


def kda_tril_auto_plan(total_tokens: int, num_chunks: int, num_heads: int,
                       workspace_bytes: int) -> str:
    return ALGO_NAMES[_lib.kda_tril_auto_plan(total_tokens, num_chunks, num_heads,
                                              workspace_bytes)]


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float16:
        return KDA_F16
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond, what: str) -> None:
    """Argument check of the binding (kept under python -O, unlike assert)."""
    if not cond:
        raise ValueError(what)


def _ptr(t):
    """Device address of a cuda tensor. Host tensors are refused: the kernels
    would dereference a host address."""
    if t is None:
        return None
    _require(t.is_cuda, f"expected a cuda tensor, got one on {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def _dense_args(A, X, workspace, algo, stream):
    _require(A.is_contiguous() and X.is_contiguous(), "A and X must be contiguous")
    _require(A.dim() == 4 and A.shape == X.shape, "A and X must both be [B, T, H, C]")
    B, T, H, C = A.shape
    _require(C in CHUNK_SIZES, f"chunk size {C} (16, 32 or 64)")
    return (_ptr(A), _dtype_code(A), _ptr(X), _dtype_code(X), B, T, H, C, _ptr(workspace),
            _ws_bytes(workspace), _algo(algo), _stream_ptr(stream))


def _packed_args(A, X, cu_seqlens, chunk_indices, workspace, algo, stream):
    import torch
    _require(A.is_contiguous() and X.is_contiguous(), "A and X must be contiguous")
    _require(A.dim() == 3 and A.shape == X.shape, "A and X must both be [T, H, C]")
    _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous(),
             "cu_seqlens must be contiguous int32")
    T, H, C = A.shape
    _require(C in CHUNK_SIZES, f"chunk size {C} (16, 32 or 64)")
    nch = 0
    if chunk_indices is not None:
        _require(chunk_indices.dtype == torch.int32 and chunk_indices.is_contiguous(),
                 "chunk_indices must be contiguous int32")
        nch = chunk_indices.numel() // 2
    return (_ptr(A), _dtype_code(A), _ptr(X), _dtype_code(X), _ptr(cu_seqlens),
            cu_seqlens.numel() - 1, T, H, C, _ptr(chunk_indices), nch, _ptr(workspace),
            _ws_bytes(workspace), _algo(algo), _stream_ptr(stream))


def _dense_fn(args):
    """The C entry point for marshalled dense arguments, and its argument
    tuple: the 64-token entry point for C = 64, the chunk-size one else."""
    if args[7] == 64:
        return _lib.kda_tril_inv_dense, args[:7] + args[8:]
    return _lib.kda_tril_inv_dense_chunk, args


def _packed_fn(args):
    if args[8] == 64:
        return _lib.kda_tril_inv_packed, args[:8] + args[9:]
    return _lib.kda_tril_inv_packed_chunk, args


def kda_tril_inv_dense(A, X, workspace=None, algo="auto", stream=None) -> None:
    """A [B, T, H, C] -> X [B, T, H, C] (both cuda, contiguous), C = 16, 32
    or 64 (kda_tril_inv_dense for 64, kda_tril_inv_dense_chunk else)."""
    fn, args = _dense_fn(_dense_args(A, X, workspace, algo, stream))
    _check(fn(*args))


def kda_tril_inv_packed(A, X, cu_seqlens, chunk_indices=None, workspace=None, algo="auto",
                        stream=None) -> None:
    """A [T, H, C] -> X [T, H, C] for requests given by int32 cu_seqlens,
    C = 16, 32 or 64."""
    fn, args = _packed_fn(_packed_args(A, X, cu_seqlens, chunk_indices, workspace, algo, stream))
    _check(fn(*args))


def kda_tril_inv_packed_noalloc(A, X, cu_seqlens, chunk_indices=None, stream=None) -> None:
    """kda_tril_inv_packed_noalloc: the split plan with the library's own
    device scratch (no workspace argument, nothing allocated). A, X
    [T, H, 64]."""
    args = _packed_args(A, X, cu_seqlens, chunk_indices, None, "split", stream)
    _require(args[8] == 64, "the allocation-free entry point takes 64-token chunks")
    # drop chunk size, workspace pointer and size, and plan
    _check(_lib.kda_tril_inv_packed_noalloc(*(args[:8] + args[9:11] + args[14:])))


def kda_tril_inv_dense_chunk(A, X, chunk_size, workspace=None, algo="auto", stream=None) -> None:
    """kda_tril_inv_dense_chunk itself (any C, including 64)."""
    args = _dense_args(A, X, workspace, algo, stream)
    _require(args[7] == chunk_size, f"A's last dimension {args[7]} is not chunk_size")
    _check(_lib.kda_tril_inv_dense_chunk(*args))


def kda_tril_inv_packed_chunk(A, X, cu_seqlens, chunk_size, chunk_indices=None, workspace=None,
                              algo="auto", stream=None) -> None:
    """kda_tril_inv_packed_chunk itself (any C, including 64)."""
    args = _packed_args(A, X, cu_seqlens, chunk_indices, workspace, algo, stream)
    _require(args[8] == chunk_size, f"A's last dimension {args[8]} is not chunk_size")
    _check(_lib.kda_tril_inv_packed_chunk(*args))


def _prepared(fn, args):
    def call():
        st = fn(*args)
        if st != KDA_OK:
            raise KdaError(st)
    return call


def prepare_packed(A, X, cu_seqlens, workspace=None, algo="auto", stream=None,
                   chunk_indices=None):
    """Marshal the arguments of one packed call once and return a function
    that issues exactly that call (for launch loops that should not pay the
    per-call Python checks). The tensors must stay alive while it is used."""
    return _prepared(*_packed_fn(_packed_args(A, X, cu_seqlens, chunk_indices, workspace, algo,
                                              stream)))


def prepare_dense(A, X, workspace=None, algo="auto", stream=None):
    """Dense counterpart of prepare_packed: A, X [B, T, H, C]."""
    return _prepared(*_dense_fn(_dense_args(A, X, workspace, algo, stream)))


def _alloc_stream(stream):
    """Context in which torch allocations belong to `stream` (the current
    stream when None)."""
    import contextlib

    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def tril_inv(A, cu_seqlens=None, out_dtype=None, algo="auto", chunk_indices=None, out=None,
             stream=None):
    """X = (I + A)^-1 per chunk of C = A.shape[-1] tokens (16, 32 or 64) and
    head.

    A: cuda tensor, [T, H, C] packed (with int32 ``cu_seqlens``) or
    [B, T, H, C] dense, float32, bfloat16 or float16. Returns X of
    ``out_dtype`` (default float32), same shape. The split workspace, when the
    plan needs one, is allocated here with torch.
    """
    import torch
    out_dtype = out_dtype or torch.float32
    with _alloc_stream(stream):
        X = out if out is not None else torch.empty(A.shape, dtype=out_dtype, device=A.device)
    C = A.shape[-1]
    nbytes = 0
    if C == 64:
        if cu_seqlens is None:
            B, T, H, _ = A.shape
            nbytes, _chosen = kda_tril_inv_workspace_size(B * T, B, B * ((T + 63) // 64), H, algo)
        else:
            T, H, _ = A.shape
            nch = 0 if chunk_indices is None else chunk_indices.numel() // 2
            nbytes, _chosen = kda_tril_inv_workspace_size(T, cu_seqlens.numel() - 1, nch, H, algo)
    # the workspace belongs to the stream the kernels run on: it is freed when
    # this function returns, and torch's caching allocator only reuses a block
    # in the order of the stream it was allocated on
    with _alloc_stream(stream):
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=A.device) if nbytes else None
    if cu_seqlens is None:
        kda_tril_inv_dense(A, X, workspace=ws, algo=algo, stream=stream)
    else:
        kda_tril_inv_packed(A, X, cu_seqlens, chunk_indices=chunk_indices, workspace=ws,
                            algo=algo, stream=stream)
    return X


# ---- A built from keys, decays and write strengths ------------------------

def _kkt_args(k, g, beta, out, cu_seqlens, chunk_indices, stream):
    import torch
    _require(all(t.is_contiguous() for t in (k, g, beta, out)), "inputs must be contiguous")
    _require(g.dtype == torch.float32 and beta.dtype == k.dtype,
             "g must be float32 and beta of k's dtype")
    lead = k.shape[:-1]
    K = k.shape[-1]
    _require(g.shape == k.shape and beta.shape == lead and out.shape == lead + (64,),
             "shapes: k, g [.., H, K], beta [.., H], out [.., H, 64]")
    H = k.shape[-2]
    if cu_seqlens is None:
        _require(k.dim() == 4, "dense inputs are [B, T, H, K]")
        B, T = k.shape[0], k.shape[1]
        return (_ptr(k), _ptr(g), _ptr(beta), _dtype_code(k), _ptr(out), _dtype_code(out), B, T, H,
                K, _stream_ptr(stream))
    _require(k.dim() == 3, "packed inputs are [T, H, K]")
    _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous(),
             "cu_seqlens must be contiguous int32")
    nch = 0
    if chunk_indices is not None:
        _require(chunk_indices.dtype == torch.int32 and chunk_indices.is_contiguous(),
                 "chunk_indices must be contiguous int32")
        nch = chunk_indices.numel() // 2
    return (_ptr(k), _ptr(g), _ptr(beta), _dtype_code(k), _ptr(out), _dtype_code(out),
            _ptr(cu_seqlens), cu_seqlens.numel() - 1, k.shape[0], H, K, _ptr(chunk_indices), nch,
            _stream_ptr(stream))


def kda_kkt_tril_inv(k, g, beta, X, cu_seqlens=None, chunk_indices=None, stream=None) -> None:
    """X = (I + A)^-1 with A built from keys k [.., H, K], FP32 decays g
    [.., H, K] and write strengths beta [.., H] (k's dtype); packed with
    ``cu_seqlens`` ([T, H, *]) or dense ([B, T, H, *]). X [.., H, 64]."""
    args = _kkt_args(k, g, beta, X, cu_seqlens, chunk_indices, stream)
    fn = _lib.kda_kkt_tril_inv_dense if cu_seqlens is None else _lib.kda_kkt_tril_inv_packed
    _check(fn(*args))


def kda_kkt(k, g, beta, A, cu_seqlens=None, chunk_indices=None, stream=None) -> None:
    """The delta-rule matrix A [.., H, 64] itself (same inputs as kda_kkt_tril_inv)."""
    args = _kkt_args(k, g, beta, A, cu_seqlens, chunk_indices, stream)
    fn = _lib.kda_kkt_dense if cu_seqlens is None else _lib.kda_kkt_packed
    _check(fn(*args))


def prepare_kkt(k, g, beta, out, cu_seqlens=None, solve=True, stream=None):
    """Marshalled form of one kda_kkt_tril_inv (solve) or kda_kkt call."""
    args = _kkt_args(k, g, beta, out, cu_seqlens, None, stream)
    if cu_seqlens is None:
        fn = _lib.kda_kkt_tril_inv_dense if solve else _lib.kda_kkt_dense
    else:
        fn = _lib.kda_kkt_tril_inv_packed if solve else _lib.kda_kkt_packed
    return _prepared(fn, args)


def kkt_tril_inv(k, g, beta, cu_seqlens=None, out_dtype=None, chunk_indices=None, stream=None):
    """Convenience form of kda_kkt_tril_inv: allocates X with torch."""
    import torch
    with _alloc_stream(stream):
        X = torch.empty(k.shape[:-1] + (64,), dtype=out_dtype or torch.float32, device=k.device)
    kda_kkt_tril_inv(k, g, beta, X, cu_seqlens, chunk_indices, stream)
    return X


# ---- the fused KDA decode core --------------------------------------------

def _decode_args(qkv, z, g, beta, norm_w, conv_w, slot, state, conv_state, out, eps_l2,
                 eps_norm, stream):
    import torch
    _require(all(t.is_contiguous() for t in (qkv, z, g, beta, norm_w, conv_w, slot, state,
                                              conv_state, out)), "inputs must be contiguous")
    _require(z.dtype == qkv.dtype and slot.dtype == torch.int32,
             "z must have qkv's dtype and slot must be int32")
    _require(all(t.dtype == torch.float32 for t in (g, beta, norm_w, conv_w, state, conv_state)),
             "g, beta, norm_w, conv_w, state and conv_state must be float32")
    _require(qkv.dim() == 4 and conv_w.dim() == 4, "qkv is [B, 3, H, d], conv_w [3, W, H, d]")
    B, three, H, d = qkv.shape
    W = conv_w.shape[1]
    _require(three == 3 and z.shape == (B, H, d) and g.shape == (B, H, d) and
             beta.shape == (B, H) and norm_w.shape == (d,) and slot.shape == (B,),
             "shapes: z, g [B, H, d], beta [B, H], norm_w [d], slot [B]")
    _require(conv_w.shape == (3, W, H, d) and state.dim() == 4 and state.shape[1:] == (H, d, d),
             "shapes: conv_w [3, W, H, d], state [slots, H, d, d]")
    _require(conv_state.shape == (state.shape[0], 3, H, W - 1, d) and out.shape == (B, H, d),
             "shapes: conv_state [slots, 3, H, W - 1, d], out [B, H, d]")
    return (_ptr(qkv), _ptr(z), _dtype_code(qkv), _ptr(g), _ptr(beta), _ptr(norm_w),
            _ptr(conv_w), _ptr(slot), _ptr(state), _ptr(conv_state), state.shape[0], _ptr(out),
            _dtype_code(out), B, H, d, W, float(eps_l2), float(eps_norm), _stream_ptr(stream))


def kda_decode_step(qkv, z, g, beta, norm_w, conv_w, slot, state, conv_state, out,
                    eps_l2=1e-6, eps_norm=1e-6, stream=None) -> None:
    """One decode step of the fused KDA decode core (see include/kda_tril.h);
    state and conv_state are updated in place, out is written."""
    _check(_lib.kda_decode_step(*_decode_args(qkv, z, g, beta, norm_w, conv_w, slot, state,
                                              conv_state, out, eps_l2, eps_norm, stream)))


def prepare_decode(qkv, z, g, beta, norm_w, conv_w, slot, state, conv_state, out, eps_l2=1e-6,
                   eps_norm=1e-6, stream=None):
    """Marshalled form of one kda_decode_step call."""
    return _prepared(_lib.kda_decode_step,
                     _decode_args(qkv, z, g, beta, norm_w, conv_w, slot, state, conv_state, out,
                                  eps_l2, eps_norm, stream))

