"""GPU tests of the solver's 4-head kernels on their edge cases.

Launches of more chunk-heads than the per-wavefront kernels hold at once run
the 4-head kernels (a
workgroup owns one chunk and four adjacent heads, their tiles loaded into
LDS): the fused kernel, and the split plan's diagonal and merge kernels. The
large workloads of the parity tests reach them with 64 heads.
KDA_TRIL_FUSED_LAYOUT=heads4 (fused) and KDA_TRIL_SPLIT_LAYOUT=heads4 (split)
make every launch use them, so these tests reach their edge cases on small
problems: head counts that are not a multiple of four (the last group masks
the missing heads), partial chunks, every input and output type, a caller
chunk map, garbage above the diagonal and malformed cu_seqlens. Every case is
compared with the oracle and, bit for bit, with the per-wavefront kernels
(layout "wave"), which run the same arithmetic.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LENGTHS = [1, 17, 64, 100, 130, 5, 48]  # partial chunks of every block count
PAD = 16
CANARY = -777.0


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


LAYOUT_ENV = {"fused": "KDA_TRIL_FUSED_LAYOUT", "split": "KDA_TRIL_SPLIT_LAYOUT"}


@pytest.fixture(params=sorted(LAYOUT_ENV))
def algo(request):
    return request.param


def _both_layouts(kt, monkeypatch, call, algo):
    """call() under the 4-head layout and under the per-wavefront one."""
    env = LAYOUT_ENV[algo]
    out = {}
    for lay in ("heads4", "wave"):
        monkeypatch.setenv(env, lay)
        out[lay] = call()
        torch.cuda.synchronize()
    monkeypatch.delenv(env)
    return out["heads4"], out["wave"]


@pytest.mark.parametrize("H", [1, 2, 3, 4, 5, 7])
def test_head_counts_and_partial_chunks(kt, monkeypatch, algo, H):
    print(f"\n[heads4] {algo} H={H}", flush=True)
    A = synth.delta_rule_A(LENGTHS, H, seed=300 + H, upper="nan")
    cu = synth.cu_seqlens(LENGTHS)
    T = A.shape[0]
    Ad = torch.from_numpy(np.concatenate([A, np.full((PAD, H, 64), np.nan, np.float32)])).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)

    def run():
        X = torch.full((T + PAD, H, 64), CANARY, device=DEV)
        kt.tril_inv(Ad[:T], cud, algo=algo, out=X[:T])  # allocates the split workspace
        return X

    X4, Xw = _both_layouts(kt, monkeypatch, run, algo)
    assert torch.equal(X4, Xw)
    X = X4.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY), "a row past the last request was written"
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(X[:T], ref, "f32") <= 0


@pytest.mark.parametrize("a_dtype,x_dtype", [("f32", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                             ("bf16", "bf16")])
def test_dtypes(kt, monkeypatch, algo, a_dtype, x_dtype):
    H = 6
    A32 = synth.delta_rule_A(LENGTHS, H, seed=310)
    A = {"f32": A32, "bf16": synth.to_bf16_bits(A32), "f16": synth.to_f16_bits(A32)}[a_dtype]
    cu = synth.cu_seqlens(LENGTHS)
    Ad = gh.to_torch_input(A, a_dtype, DEV)
    cud = torch.from_numpy(cu).to(DEV)
    xt = gh.out_torch_dtype(x_dtype)
    X4, Xw = _both_layouts(kt, monkeypatch,
                           lambda: kt.tril_inv(Ad, cud, out_dtype=xt, algo=algo), algo)
    assert torch.equal(X4, Xw)
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    assert gh.excess(gh.to_numpy_f64(X4), ref, x_dtype) <= 0


def test_dense_layout_and_chunk_map(kt, monkeypatch, algo):
    H = 5
    B, T = 3, 150
    A = synth.delta_rule_A([T] * B, H, seed=320)
    Ad = torch.from_numpy(A).to(DEV)
    X4, Xw = _both_layouts(kt, monkeypatch,
                           lambda: kt.tril_inv(Ad.view(B, T, H, 64), algo=algo), algo)
    assert torch.equal(X4, Xw)
    cu = synth.cu_seqlens([T] * B)
    cud = torch.from_numpy(cu).to(DEV)
    cmap = torch.from_numpy(gh.host_chunk_map([T] * B)).to(DEV)
    Xm, _ = _both_layouts(kt, monkeypatch,
                          lambda: kt.tril_inv(Ad, cud, chunk_indices=cmap, algo=algo), algo)
    assert torch.equal(Xm.view(B, T, H, 64), X4)
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(gh.to_numpy_f64(Xm), ref, "f32") <= 0


@pytest.mark.parametrize("cu,clamped", [([0, 64, 200], [0, 64, 100]),
                                        ([-40, 64, 100], [24, 64, 100]),
                                        ([0, 64, 100, 300], [0, 64, 100, 100])])
def test_malformed_cu_seqlens_clamped(kt, monkeypatch, algo, cu, clamped):
    """Chunks outside rows [0, T) are skipped or cut at T, as for the other
    kernels: nothing past T is read (NaN there) or written (canaries)."""
    H = 3
    A = synth.delta_rule_A([64, 36], H, seed=330)
    T = A.shape[0]
    Ad = torch.from_numpy(np.concatenate([A, np.full((PAD, H, 64), np.nan, np.float32)])).to(DEV)
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)

    def run():
        X = torch.full((T + PAD, H, 64), CANARY, device=DEV)
        kt.tril_inv(Ad[:T], cud, algo=algo, out=X[:T])
        return X

    X4, Xw = _both_layouts(kt, monkeypatch, run, algo)
    assert torch.equal(X4, Xw)
    X = X4.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY)
    ref = np.full(A.shape, np.nan)
    for s, e in zip(clamped[:-1], clamped[1:]):
        if s < e:
            ref[s:e] = oracle.tril_inv_packed(A[s:e], [0, e - s])
    rows = ~np.isnan(ref[:, 0, 0])
    assert gh.excess(X[:T][rows], ref[rows], "f32") <= 0


def test_exact_subdiagonal_bitwise(kt, monkeypatch, algo):
    """A single subdiagonal c: X = (-c)^(i-j), every FP32 operation exact."""
    H, c = 7, -0.5
    lengths = [64, 40, 64]
    T = sum(lengths)
    A = np.zeros((T, H, 64), np.float32)
    bos = 0
    for n in lengths:
        for p0 in range(0, n, 64):
            for i in range(1, min(64, n - p0)):
                A[bos + p0 + i, :, i - 1] = c
        bos += n
    cud = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    Ad = torch.from_numpy(A).to(DEV)
    X4, _ = _both_layouts(kt, monkeypatch, lambda: kt.tril_inv(Ad, cud, algo=algo), algo)
    X = X4.cpu().numpy()
    bos = 0
    for n in lengths:
        L = n
        i = np.arange(L)[:, None]
        j = np.arange(64)[None, :]
        want = np.where(j <= i, np.power(np.float32(-c), (i - j).clip(0)).astype(np.float32), 0)
        for h in range(H):
            assert np.array_equal(X[bos:bos + L, h], want), (bos, h)
        bos += n


@pytest.mark.parametrize("algo_", ["fused", "split"])
def test_graph_capture_replay_heads4(kt, monkeypatch, algo_):
    """The 4-head kernels captured in a HIP graph (launch configuration fixed
    at capture) and replayed on new inputs, with eager work and
    synchronisation between replays: every replay equals the eager result."""
    monkeypatch.setenv(LAYOUT_ENV[algo_], "heads4")
    lengths = [512, 300, 64, 9]
    H = 7
    T = sum(lengths)
    inputs = [synth.delta_rule_A(lengths, H, seed=s) for s in (111, 112, 113)]
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    A = torch.from_numpy(inputs[0]).to(DEV)
    X = torch.empty_like(A)
    nbytes, _ = kt.kda_tril_inv_workspace_size(T, len(lengths), 0, H, algo_)
    ws = torch.empty(max(nbytes // 4, 1), device=DEV) if nbytes else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kt.kda_tril_inv_packed(A, X, cu, workspace=ws, algo=algo_)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kt.kda_tril_inv_packed(A, X, cu, workspace=ws, algo=algo_)
    for i in range(6):
        A.copy_(torch.from_numpy(inputs[i % 3]))
        X.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = kt.tril_inv(A, cu, algo=algo_)
        torch.cuda.synchronize()
        assert torch.equal(X, ref), i
