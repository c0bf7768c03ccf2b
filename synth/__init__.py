"""Seeded synthetic inputs for the KDA prefill chunk solver.

This module only draws inputs; it holds none of the solver's arithmetic and
imports neither the oracle nor the HIP library, both of which consume what it
makes.

The intra-chunk matrix follows the delta-rule shape that KDA prefill hands to
the solver: for tokens i > j of one chunk (64 tokens, or 16 or 32 for the
smaller branches) and one head,

    A[i, j] = -beta_i * sum_d k[i, d] * k[j, d] * exp(g[i, d] - g[j, d])

with k a Gaussian key row L2-normalised over the key dimension (128),
beta_i = sigmoid(N(0, 1)), and g the within-chunk running sum of
logsigmoid(N(0, 1) + 3) per channel. Since g decreases along the chunk,
exp(g_i - g_j) <= 1 for i > j and |A[i, j]| <= beta_i < 1.

Randomness: chunk number n (counted in packed order over all requests) draws
from ``numpy.random.default_rng([seed, n])``: first k [L, H, K], then the
decay logits [L, H, K], then the beta logits [L, H]. Each chunk is therefore
reproducible on its own, and chunks can be generated in parallel.

The product k_i . k_j weighted by exp(g_i - g_j) is evaluated in float64 as
(k_i * exp(g_i)) . (k_j * exp(-g_j)); with |g| below a few tens this is as
accurate as the direct form, and A is rounded once to float32 at the end.
bfloat16 inputs are rounded from that float32 array by torch's CPU cast.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 64
KEY_DIM = 128

# The workloads, each named by its layout, request lengths, heads, dtypes and
# (when not 64) chunk size. Fields: layout, request lengths (or dense B, T),
# heads, input and output dtypes, data seed, optional chunk size.
CONFIGS = {
    "packed_1x64_h64_f32": dict(layout="packed", lengths=[64], H=64, a_dtype="f32",
                                   x_dtype="f32", seed=0),
    "dense_b4_t512_h16_bf16_f32": dict(layout="dense", B=4, T=512, H=16, a_dtype="bf16",
                                          x_dtype="f32", seed=1),
    "packed_16x512_h64_f32": dict(layout="packed", lengths=[512] * 16, H=64, a_dtype="f32",
                                     x_dtype="f32", seed=2),
    "packed_ragged48_h64_f32_bf16": dict(layout="packed", lengths="ragged48", H=64,
                                            a_dtype="f32", x_dtype="bf16", seed=3),
    "packed_1x131072_h64_f32": dict(layout="packed", lengths=[131072], H=64,
                                       a_dtype="f32", x_dtype="f32", seed=4),
    # the solver's 16- and 32-token branches on the same tokens and heads
    "packed_16x512_h64_c16_f32": dict(layout="packed", lengths=[512] * 16, H=64,
                                         a_dtype="f32", x_dtype="f32", seed=5, chunk=16),
    "packed_16x512_h64_c32_f32": dict(layout="packed", lengths=[512] * 16, H=64,
                                         a_dtype="f32", x_dtype="f32", seed=6, chunk=32),
}

# Workloads of the fused KDA decode core: one decode step for B sequences,
# H = 32 heads of dim 128, conv width 4, bf16 activations in and out, state
# pools with 2 B slots (the batch uses a permutation of half of them).
DECODE_CONFIGS = {
    f"decode_b{B}_h32_d128_w4_bf16": dict(B=B, H=32, d=128, W=4, slots=2 * B, in_dtype="bf16",
                                          out_dtype="bf16", seed=20 + B)
    for B in (2, 4, 8, 16, 32)
}

# Workloads of the path that builds A from keys k, decays g and write
# strengths beta: k and beta in k_dtype, g in float32, X in x_dtype.
KKT_CONFIGS = {
    "packed_16x512_h64_k128_kkt_bf16_f32": dict(layout="packed", lengths=[512] * 16, H=64, K=128,
                                                 k_dtype="bf16", x_dtype="f32", seed=7),
    "packed_16x512_h64_k128_kkt_f32_f32": dict(layout="packed", lengths=[512] * 16, H=64, K=128,
                                                k_dtype="f32", x_dtype="f32", seed=8),
}


def ragged_lengths(n: int = 48, lo: int = 1, hi: int = 1500, seed: int = 0) -> list[int]:
    """Request lengths uniform in [lo, hi] (seed 0 gives T = 33,139 tokens in
    542 chunks for the 48-request workload)."""
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n)]


def config_lengths(cfg: dict) -> list[int]:
    if cfg["layout"] == "dense":
        return [cfg["T"]] * cfg["B"]
    if cfg["lengths"] == "ragged48":
        return ragged_lengths()
    return list(cfg["lengths"])


def cu_seqlens(lengths) -> np.ndarray:
    """Cumulative sequence lengths [0, n0, n0+n1, ...] as int32."""
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def _chunk_rows(lengths, chunk: int = CHUNK):
    """(first token, valid rows) of every chunk, in packed order."""
    out = []
    bos = 0
    for n in lengths:
        for p in range(0, n, chunk):
            out.append((bos + p, min(chunk, n - p)))
        bos += n
    return out


def _chunk_draws(seed: int, idx: int, L: int, H: int, K: int):
    """Keys k [L, H, K] (unit rows), write strengths beta [L, H] and
    within-chunk cumulative log-decays g [L, H, K] of chunk number idx."""
    rng = np.random.default_rng([seed, idx])
    k = rng.standard_normal((L, H, K))
    z = rng.standard_normal((L, H, K))
    b = rng.standard_normal((L, H))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-b))
    g = np.cumsum(-np.logaddexp(0.0, -(z + 3.0)), axis=0)  # logsigmoid(z + 3)
    return k, g, beta


def _one_chunk(seed: int, idx: int, L: int, H: int, K: int, chunk: int) -> np.ndarray:
    k, g, beta = _chunk_draws(seed, idx, L, H, K)
    kq = (k * np.exp(g)).transpose(1, 0, 2)          # [H, L, K]
    kk = (k * np.exp(-g)).transpose(1, 2, 0)         # [H, K, L]
    S = np.matmul(kq, kk)                            # [H, L, L]
    a = -beta.T[:, :, None] * S                      # [H, L, L]
    a = np.tril(a, -1).transpose(1, 0, 2)            # [L, H, L]
    out = np.zeros((L, H, chunk), np.float32)
    out[:, :, :L] = a
    return out


def delta_rule_A(lengths, H: int, seed: int, K: int = KEY_DIM, upper: str = "zero",
                 threads: int | None = None, chunk: int = CHUNK) -> np.ndarray:
    """Packed float32 A [T, H, chunk] for requests of the given lengths.

    ``upper`` fills the entries on and above the diagonal (and the columns past
    a partial chunk's length), which the solver must ignore: "zero", "nan", or
    "garbage" (large finite values, +-inf and NaN mixed)."""
    chunks = _chunk_rows(lengths, chunk)
    T = int(sum(lengths))
    A = np.zeros((T, H, chunk), np.float32)
    nthr = threads or min(16, os.cpu_count() or 1)

    def work(i):
        s, L = chunks[i]
        A[s:s + L] = _one_chunk(seed, i, L, H, K, chunk)

    if len(chunks) > 1 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, range(len(chunks))))
    else:
        for i in range(len(chunks)):
            work(i)
    if upper != "zero":
        _fill_upper(A, chunks, upper, seed)
    return A


def delta_rule_inputs(lengths, H: int, seed: int, K: int = KEY_DIM,
                      threads: int | None = None):
    """Packed float32 keys k [T, H, K], cumulative log-decays g [T, H, K]
    (restarting at every 64-token chunk) and write strengths beta [T, H]:
    the same draws from which delta_rule_A builds A, rounded to float32 once.
    The matrix itself is not formed here."""
    chunks = _chunk_rows(lengths, CHUNK)
    T = int(sum(lengths))
    k = np.zeros((T, H, K), np.float32)
    g = np.zeros((T, H, K), np.float32)
    beta = np.zeros((T, H), np.float32)
    nthr = threads or min(16, os.cpu_count() or 1)

    def work(i):
        s, L = chunks[i]
        kc, gc, bc = _chunk_draws(seed, i, L, H, K)
        k[s:s + L], g[s:s + L], beta[s:s + L] = kc, gc, bc

    if len(chunks) > 1 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, range(len(chunks))))
    else:
        for i in range(len(chunks)):
            work(i)
    return k, g, beta


def _fill_upper(A, chunks, mode, seed):
    rng = np.random.default_rng([seed, 0x5EED])
    col = np.arange(A.shape[-1])
    for s, L in chunks:
        rows = np.arange(L)
        mask = col[None, :] >= rows[:, None]                  # on/above diagonal
        blk = A[s:s + L]
        if mode == "nan":
            fill = np.full(blk.shape, np.nan, np.float32)
        elif mode == "garbage":
            fill = rng.uniform(-1e30, 1e30, blk.shape).astype(np.float32)
            pick = rng.integers(0, 4, blk.shape)
            fill[pick == 0] = np.inf
            fill[pick == 1] = -np.inf
            fill[pick == 2] = np.nan
        else:
            raise ValueError(mode)
        blk[np.broadcast_to(mask[:, None, :], blk.shape)] = fill[
            np.broadcast_to(mask[:, None, :], blk.shape)]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of a float32 array, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) of a float32 array, via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make(name_or_cfg, upper: str = "zero") -> dict:
    """Materialise one workload. Returns a dict with the input ``A`` (float32,
    or uint16 bit patterns when a_dtype is bf16 or f16) in its layout
    ([T, H, C] packed or [B, T, H, C] dense, C = the config's "chunk", default
    64), ``cu_seqlens`` (packed only), the request lengths and the config
    fields."""
    cfg = dict(CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    C = cfg.setdefault("chunk", CHUNK)
    lengths = config_lengths(cfg)
    A = delta_rule_A(lengths, cfg["H"], cfg["seed"], upper=upper, chunk=C)
    if cfg["a_dtype"] == "bf16":
        A = to_bf16_bits(A)
    elif cfg["a_dtype"] == "f16":
        A = to_f16_bits(A)
    out = dict(cfg)
    out["lengths"] = lengths
    out["T_total"] = int(sum(lengths))
    out["num_chunks"] = len(_chunk_rows(lengths, C))
    if cfg["layout"] == "dense":
        out["A"] = A.reshape(cfg["B"], cfg["T"], cfg["H"], C)
    else:
        out["A"] = A
        out["cu_seqlens"] = cu_seqlens(lengths)
    return out


def make_kkt(name_or_cfg) -> dict:
    """Materialise one workload of the build-A-from-keys path: ``k`` [T, H, K]
    and ``beta`` [T, H] (float32, or uint16 bit patterns for bf16 / f16),
    ``g`` [T, H, K] float32, in the packed or dense ([B, T, ...]) layout, plus
    ``cu_seqlens`` (packed), the lengths and the config fields."""
    cfg = dict(KKT_CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    lengths = config_lengths(cfg)
    k, g, beta = delta_rule_inputs(lengths, cfg["H"], cfg["seed"], K=cfg["K"])
    if cfg["k_dtype"] == "bf16":
        k, beta = to_bf16_bits(k), to_bf16_bits(beta)
    elif cfg["k_dtype"] == "f16":
        k, beta = to_f16_bits(k), to_f16_bits(beta)
    out = dict(cfg)
    out["lengths"] = lengths
    out["T_total"] = int(sum(lengths))
    out["num_chunks"] = len(_chunk_rows(lengths, CHUNK))
    if cfg["layout"] == "dense":
        B, T, H, K = cfg["B"], cfg["T"], cfg["H"], cfg["K"]
        k, g, beta = k.reshape(B, T, H, K), g.reshape(B, T, H, K), beta.reshape(B, T, H)
    else:
        out["cu_seqlens"] = cu_seqlens(lengths)
    out["k"], out["g"], out["beta"] = k, g, beta
    return out


def decode_inputs(B: int, H: int, d: int = 128, W: int = 4, slots: int | None = None,
                  seed: int = 0, in_dtype: str = "f32", padding: int = 0) -> dict:
    """Seeded inputs of one decode step: q, k, v and the gate z ~ N(0, 1)
    (float32, or bfloat16 / binary16 bit patterns), log-decays
    g = logsigmoid(N(0, 1) + 3) per key channel, beta = sigmoid(N(0, 1)),
    RMSNorm weights 1 + N(0, 0.1), conv taps U(-0.5, 0.5), FP32 state pools
    (S ~ N(0, 0.05), conv windows ~ N(0, 1)), and the slot of each sequence: a
    random choice of distinct slots, the first ``padding`` entries -1."""
    rng = np.random.default_rng([seed, 0xDEC])
    slots = slots or 2 * B
    qkv = rng.standard_normal((B, 3, H, d)).astype(np.float32)
    z = rng.standard_normal((B, H, d)).astype(np.float32)
    if in_dtype == "bf16":
        qkv, z = to_bf16_bits(qkv), to_bf16_bits(z)
    elif in_dtype == "f16":
        qkv, z = to_f16_bits(qkv), to_f16_bits(z)
    slot = rng.permutation(slots)[:B].astype(np.int32)
    slot[:padding] = -1
    return dict(
        qkv=qkv, z=z,
        g=(-np.logaddexp(0.0, -(rng.standard_normal((B, H, d)) + 3.0))).astype(np.float32),
        beta=(1.0 / (1.0 + np.exp(-rng.standard_normal((B, H))))).astype(np.float32),
        norm_w=(1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32),
        conv_w=rng.uniform(-0.5, 0.5, (3, W, H, d)).astype(np.float32),
        slot=slot,
        state=(0.05 * rng.standard_normal((slots, H, d, d))).astype(np.float32),
        conv_state=rng.standard_normal((slots, 3, H, W - 1, d)).astype(np.float32),
        B=B, H=H, d=d, W=W, slots=slots, in_dtype=in_dtype)

