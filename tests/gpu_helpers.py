"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle to the stated tolerances."""
from __future__ import annotations

import numpy as np

# Tolerances (elementwise, X_ref from the fp64 oracle):
#   fp32 output: |X - X_ref| <= 2e-5 * (1 + |X_ref|)
#   bf16 output: |X - X_ref| <= 1e-2 * |X_ref| + 2e-5 * (1 + |X_ref|)
#   f16 output:  |X - X_ref| <= 1e-3 * |X_ref| + 2e-5 * (1 + |X_ref|)
#                (binary16 rounding is at most 2^-11 relative; subnormal
#                 outputs are within 2^-25 absolute)
#   residual (fp32 outputs): max |(I + A_L) X - I| <= 1e-4
F32_TOL = 2e-5
BF16_REL = 1e-2
F16_REL = 1e-3
RESIDUAL_TOL = 1e-4


def to_torch_input(A_np, a_dtype, device):
    import torch
    if a_dtype in ("bf16", "f16"):
        dt = torch.bfloat16 if a_dtype == "bf16" else torch.float16
        return torch.from_numpy(np.ascontiguousarray(A_np).view(np.int16)).view(dt).to(device)
    return torch.from_numpy(np.ascontiguousarray(A_np, dtype=np.float32)).to(device)


def out_torch_dtype(x_dtype):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16}.get(x_dtype, torch.float32)


def to_numpy_f64(X):
    """Device tensor -> float64 numpy (exact for f32 and bf16)."""
    import torch
    if X.dtype == torch.bfloat16:
        bits = X.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if X.dtype == torch.float16:
        return X.cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)
    return X.cpu().numpy().astype(np.float64)


def bits16(X):
    """uint16 bit patterns of a bfloat16 or float16 tensor."""
    import torch
    assert X.dtype in (torch.bfloat16, torch.float16)
    return X.cpu().view(torch.int16).numpy().view(np.uint16)


def excess(got, ref, x_dtype):
    """Largest amount by which |got - ref| exceeds its bound (<= 0: pass)."""
    diff = np.abs(got - ref)
    bound = F32_TOL * (1.0 + np.abs(ref))
    if x_dtype == "bf16":
        bound = bound + BF16_REL * np.abs(ref)
    elif x_dtype == "f16":
        bound = bound + F16_REL * np.abs(ref)
    e = diff - bound
    e = np.where(np.isnan(got) | np.isnan(ref), np.inf, e)
    return float(e.max()) if e.size else -1.0


def residual_chunks(A64, X64, chunks):
    """max |(I + A_L) X_L - I| over the given (start, len, head) matrices;
    A64, X64 packed [T, H, C] float64."""
    worst = 0.0
    for s, L, h in chunks:
        M = np.tril(A64[s:s + L, h, :L], -1)
        Xm = X64[s:s + L, h, :L]
        r = np.abs((np.eye(L) + M) @ Xm - np.eye(L)).max()
        worst = max(worst, float(r))
    return worst


def all_chunk_heads(lengths, H, C=64):
    out = []
    bos = 0
    for n in lengths:
        for p in range(0, n, C):
            for h in range(H):
                out.append((bos + p, min(C, n - p), h))
        bos += n
    return out


def host_chunk_map(lengths, C=64):
    """(request, chunk-within-request) pairs in packed order, int32 [n, 2]."""
    pairs = []
    for s, n in enumerate(lengths):
        for c in range((n + C - 1) // C):
            pairs.append((s, c))
    return np.asarray(pairs, np.int32).reshape(-1, 2)


def residual_full_chunks(A, X):
    """max |(I + A_c) X_c - I| over every chunk-head of packed [T, H, 64]
    arrays whose chunks are all full and start at multiples of 64 (requests
    of whole chunks); A's entries on and above the diagonal are ignored.
    Batched in float64."""
    T, H, C = A.shape
    assert T % C == 0
    M = np.tril(np.asarray(A, np.float64).reshape(T // C, C, H, C).transpose(0, 2, 1, 3), -1)
    Xm = np.asarray(X, np.float64).reshape(T // C, C, H, C).transpose(0, 2, 1, 3)
    return float(np.abs(M @ Xm + Xm - np.eye(C)).max())
