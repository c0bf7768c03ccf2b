"""GPU parity at the size limits the C ABI accepts (H = 4096 heads, K = 256
key channels) and graph capture of the path that builds A from keys.

At these sizes the kernels' 32-bit buffer offsets come closest to their bound
(a chunk's 64 rows of H x 64 or H x K elements), so every path is checked
there against the oracle: all heads where the oracle is cheap, a sample of
heads otherwise (the oracle then runs on those heads' slices).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
H_MAX = 4096
K_MAX = 256
LENGTHS = [64, 5]  # one full chunk and a partial one


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


@pytest.fixture(scope="module")
def a_max():
    """A [69, 4096, 64] with NaN on and above the diagonal."""
    print("\n[limits] generating H=4096 input", flush=True)
    return synth.delta_rule_A(LENGTHS, H_MAX, seed=90, upper="nan")


@pytest.mark.parametrize("algo", ["fused", "split", "fused_valu"])
def test_max_heads_64(kt, a_max, algo):
    print(f"\n[limits] H=4096 algo={algo}", flush=True)
    cu = synth.cu_seqlens(LENGTHS)
    X = kt.tril_inv(torch.from_numpy(a_max).to(DEV), torch.from_numpy(cu).to(DEV), algo=algo)
    torch.cuda.synchronize()
    got = gh.to_numpy_f64(X)
    ref = oracle.tril_inv_packed(a_max, cu)
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("C", [16, 32])
def test_max_heads_small_chunks(kt, C):
    print(f"\n[limits] H=4096 C={C}", flush=True)
    lengths = [C, 3]
    A = synth.delta_rule_A(lengths, H_MAX, seed=91, chunk=C, upper="nan")
    cu = synth.cu_seqlens(lengths)
    X = kt.tril_inv(torch.from_numpy(A).to(DEV), torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    e = gh.excess(gh.to_numpy_f64(X), oracle.tril_inv_packed(A, cu), "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"


def test_max_heads_and_key_dim_kkt(kt):
    """K = 256 and H = 4096 (k and g of 289 MB each): X for 24 sampled heads
    against the oracle on those heads, and the whole output finite with a unit
    diagonal."""
    print("\n[limits] kkt H=4096 K=256", flush=True)
    T = sum(LENGTHS)
    rng = np.random.default_rng(92)
    k = rng.standard_normal((T, H_MAX, K_MAX), dtype=np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = np.zeros((T, H_MAX, K_MAX), np.float32)
    for s, L in ((0, 64), (64, 5)):  # within-chunk cumulative log-decays
        g[s:s + L] = np.cumsum(-rng.random((L, H_MAX, K_MAX), dtype=np.float32) * 0.05, axis=0)
    beta = rng.random((T, H_MAX), dtype=np.float32)
    cu = synth.cu_seqlens(LENGTHS)
    X = torch.empty((T, H_MAX, 64), device=DEV)
    kt.kda_kkt_tril_inv(torch.from_numpy(k).to(DEV), torch.from_numpy(g).to(DEV),
                        torch.from_numpy(beta).to(DEV), X, torch.from_numpy(cu).to(DEV))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(X).all())
    diag = torch.diagonal(X[:64].permute(1, 0, 2), dim1=1, dim2=2)  # [H, 64]
    assert bool((diag == 1).all())
    got = gh.to_numpy_f64(X)
    heads = np.sort(rng.choice(H_MAX, 24, replace=False))
    heads[-1] = H_MAX - 1  # the last head is always checked
    ref = oracle.kkt_tril_inv_packed(np.ascontiguousarray(k[:, heads]),
                                     np.ascontiguousarray(g[:, heads]),
                                     np.ascontiguousarray(beta[:, heads]), cu)
    e = gh.excess(got[:, heads], ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"


def test_kkt_graph_capture_replay(kt):
    """The build-A call replays correctly from a captured graph several
    times, with eager work and synchronisations between the replays."""
    H, K = 4, 64
    lengths = [64, 37, 100]
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    inputs = [synth.delta_rule_inputs(lengths, H, 93 + i, K=K) for i in range(3)]
    kd, gd, bd = (torch.from_numpy(a).to(DEV) for a in inputs[0])
    X = torch.empty((sum(lengths), H, 64), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kt.kda_kkt_tril_inv(kd, gd, bd, X, cu)  # warm-up outside the graph
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kt.kda_kkt_tril_inv(kd, gd, bd, X, cu)
    torch.cuda.synchronize()
    for rep in range(3):
        for dst, src in zip((kd, gd, bd), inputs[rep]):
            dst.copy_(torch.from_numpy(src).to(DEV))
        X.fill_(5.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = kt.kkt_tril_inv(kd, gd, bd, cu)
        torch.cuda.synchronize()
        assert torch.equal(X, eager), f"replay {rep}"
