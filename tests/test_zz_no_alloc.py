"""GPU test of the allocation-free entry point kda_tril_inv_packed_noalloc
(the split plan with the library's own device scratch) against the
workspace-taking entry point kda_tril_inv_packed with the split plan, which
runs the same kernels: X must agree bit for bit, and both must match the fp64
oracle to the fp32 / bf16 tolerances. Two calls in a row, the second on a
smaller input, so the second runs on what the first left in the scratch.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


def _with_workspace(kt, A, cu, x_dtype, cmap=None):
    T, H, _ = A.shape
    nch = 0 if cmap is None else cmap.shape[0]
    nbytes, chosen = kt.kda_tril_inv_workspace_size(T, cu.numel() - 1, nch, H, "split")
    assert chosen == "split"
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    X = torch.empty(A.shape, dtype=x_dtype, device=DEV)
    kt.kda_tril_inv_packed(A, X, cu, chunk_indices=cmap, workspace=ws, algo="split")
    return X


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_noalloc_matches_split_entry_point(kt, x_dtype):
    xt = gh.out_torch_dtype(x_dtype)
    cases = [([512] * 16, 64, 7, False),       # the 16 x 512-token, 64-head batch (36 MiB bound)
             ([100, 64, 1, 17, 300], 8, 8, True)]  # smaller, ragged, with a chunk map
    for lengths, H, seed, use_map in cases:
        print(f"\n[noalloc] lengths={lengths[:3]}.. H={H} x={x_dtype} map={use_map}", flush=True)
        A_np = synth.delta_rule_A(lengths, H, seed=seed, upper="nan")
        cu_np = synth.cu_seqlens(lengths)
        A = torch.from_numpy(A_np).to(DEV)
        cu = torch.from_numpy(cu_np).to(DEV)
        cmap = torch.from_numpy(gh.host_chunk_map(lengths)).to(DEV) if use_map else None
        X = torch.full(A.shape, float("nan"), dtype=xt, device=DEV)
        kt.kda_tril_inv_packed_noalloc(A, X, cu, chunk_indices=cmap)
        Xw = _with_workspace(kt, A, cu, xt, cmap)
        torch.cuda.synchronize()
        assert torch.equal(X, Xw)
        ref = oracle.tril_inv_packed(A_np, cu_np)
        e = gh.excess(gh.to_numpy_f64(X), ref, x_dtype)
        assert e <= 0, f"exceeds tolerance by {e:.3g}"


def test_noalloc_refuses_oversize(kt):
    # 16,385 chunk-heads need 64 MiB + 4 KiB of scratch
    A = torch.zeros((64 * 16385, 1, 64), device=DEV)
    X = torch.empty_like(A)
    cu = torch.tensor([0, 64 * 16385], dtype=torch.int32, device=DEV)
    cmap = torch.from_numpy(gh.host_chunk_map([64 * 16385])).to(DEV)
    with pytest.raises(kt.KdaError) as e:
        kt.kda_tril_inv_packed_noalloc(A, X, cu, chunk_indices=cmap)
    assert e.value.status == kt.KDA_ERR_WORKSPACE
