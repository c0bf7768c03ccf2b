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


def test_noalloc_under_graph_capture(kt, monkeypatch):
    """What the entry point is for: a call captured into a HIP graph (no
    allocation inside the capture), replayed on new inputs with eager work and
    synchronisation between replays; every replay equals the workspace-taking
    split call bit for bit. Run once on the per-wavefront split kernels and
    once on the 4-head ones."""
    lengths = [512, 300, 64, 9]
    H = 6
    T = sum(lengths)
    inputs = [synth.delta_rule_A(lengths, H, seed=s) for s in (121, 122, 123)]
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    for layout in ("wave", "heads4"):
        monkeypatch.setenv("KDA_TRIL_SPLIT_LAYOUT", layout)
        A = torch.from_numpy(inputs[0]).to(DEV)
        X = torch.empty_like(A)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            kt.kda_tril_inv_packed_noalloc(A, X, cu, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            kt.kda_tril_inv_packed_noalloc(A, X, cu)
        for i in range(6):
            A.copy_(torch.from_numpy(inputs[i % 3]))
            X.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ref = _with_workspace(kt, A, cu, torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(X, ref), (layout, i)
    monkeypatch.delenv("KDA_TRIL_SPLIT_LAYOUT")
