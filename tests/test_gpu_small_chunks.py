"""GPU parity of the solver's 16- and 32-token branches (through
kda_tril_inv_{dense,packed}_chunk) against the fp64 oracle.

Same bar as the 64-token path: fp32 output |X - X_ref| <= 2e-5 (1 + |X_ref|),
bf16 / f16 outputs with the relative terms of gpu_helpers, residual
max |(I + A) X - I| <= 1e-4 on fp32 outputs, exact cases bit for bit. Head
counts that do not fill a wavefront's head group (H % 4 for 16-token chunks,
H % 2 for 32-token chunks) and partial chunks are covered explicitly.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SIZES = [16, 32]
# full chunks, one-token requests, partial last chunks, lengths around the
# 16-row block boundary
LENGTHS = [16, 37, 1, 100, 31, 64, 15, 33, 200, 17]


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


def _dev(a, a_dtype="f32"):
    return gh.to_torch_input(a, a_dtype, DEV)


def _solve_packed(kt, A, cu, x_dtype="f32", chunk_indices=None, out=None):
    X = kt.tril_inv(A, torch.from_numpy(cu).to(DEV), out_dtype=gh.out_torch_dtype(x_dtype),
                    chunk_indices=chunk_indices, out=out)
    torch.cuda.synchronize()
    return X


@pytest.mark.parametrize("H", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("C", SIZES)
def test_packed_parity_all_head_counts(kt, C, H):
    print(f"\n[small] packed C={C} H={H}", flush=True)
    A = synth.delta_rule_A(LENGTHS, H, seed=20 + H, chunk=C, upper="nan")
    cu = synth.cu_seqlens(LENGTHS)
    got = gh.to_numpy_f64(_solve_packed(kt, _dev(A), cu))
    ref = oracle.tril_inv_packed(A, cu)
    assert got.shape == (sum(LENGTHS), H, C)
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    A64 = oracle.to_f64(A, "f32")
    assert gh.residual_chunks(A64, got, gh.all_chunk_heads(LENGTHS, H, C)) <= gh.RESIDUAL_TOL


@pytest.mark.parametrize("x_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("a_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("C", SIZES)
def test_dtype_matrix(kt, C, a_dtype, x_dtype):
    print(f"\n[small] dtypes C={C} {a_dtype}->{x_dtype}", flush=True)
    H = 6
    A = synth.delta_rule_A(LENGTHS, H, seed=31, chunk=C)
    if a_dtype == "bf16":
        A = synth.to_bf16_bits(A)
    elif a_dtype == "f16":
        A = synth.to_f16_bits(A)
    cu = synth.cu_seqlens(LENGTHS)
    got = gh.to_numpy_f64(_solve_packed(kt, _dev(A, a_dtype), cu, x_dtype))
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    e = gh.excess(got, ref, x_dtype)
    assert e <= 0, f"exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("C", SIZES)
def test_16bit_outputs_are_rne_of_fp32_output(kt, C):
    H = 5
    A = _dev(synth.delta_rule_A(LENGTHS, H, seed=32, chunk=C))
    cu = synth.cu_seqlens(LENGTHS)
    x32 = _solve_packed(kt, A, cu, "f32").cpu().numpy()
    xb = gh.bits16(_solve_packed(kt, A, cu, "bf16"))
    xh = gh.bits16(_solve_packed(kt, A, cu, "f16"))
    assert np.array_equal(xb, oracle.rne_bf16(x32))
    assert np.array_equal(xh, oracle.rne_f16(x32))


@pytest.mark.parametrize("T", [77, 64, 5])
@pytest.mark.parametrize("C", SIZES)
def test_dense_parity_and_equals_packed(kt, C, T):
    print(f"\n[small] dense C={C} T={T}", flush=True)
    B, H = 3, 5
    A = synth.delta_rule_A([T] * B, H, seed=33, chunk=C, upper="garbage")
    Ad = _dev(A.reshape(B, T, H, C))
    Xd = kt.tril_inv(Ad, None)
    torch.cuda.synchronize()
    ref = oracle.tril_inv_dense(A.reshape(B, T, H, C))
    assert gh.excess(gh.to_numpy_f64(Xd), ref, "f32") <= 0
    Xp = _solve_packed(kt, _dev(A), synth.cu_seqlens([T] * B))
    assert torch.equal(Xd.reshape(B * T, H, C), Xp)


@pytest.mark.parametrize("C", SIZES)
def test_leading_block_of_64_token_result_bitwise(kt, C):
    """Every C-token chunk, solved by its own branch, equals bit for bit the
    leading C x C block of the 64-token kernel's result on the same rows
    (each C-token chunk passed to the 64-token kernel as a request of its
    own, columns C..63 of A zero): the branches share the diagonal solve and
    the first merge level in the same operation order."""
    H = 6
    A = synth.delta_rule_A(LENGTHS, H, seed=34, chunk=C)
    cu = synth.cu_seqlens(LENGTHS)
    XC = _solve_packed(kt, _dev(A), cu)
    pieces = [L for _, _, L in oracle.chunks_packed(cu, C).tolist()]
    A64 = np.zeros((A.shape[0], H, 64), np.float32)
    A64[:, :, :C] = A
    X64 = kt.tril_inv(_dev(A64), torch.from_numpy(synth.cu_seqlens(pieces)).to(DEV),
                      algo="fused")
    torch.cuda.synchronize()
    assert torch.equal(X64[:, :, :C], XC)
    assert bool((X64[:, :, C:] == 0).all())


@pytest.mark.parametrize("H", [3, 4])
@pytest.mark.parametrize("C", SIZES)
def test_rows_outside_chunks_untouched(kt, C, H):
    """X is prefilled with a canary: rows past cu_seqlens[-1] keep it, and no
    row inside a chunk keeps any (every valid row is written in full, for
    every head, also when the last head group is incomplete)."""
    A = synth.delta_rule_A(LENGTHS, H, seed=35, chunk=C)
    extra = 7
    T = A.shape[0] + extra
    Ap = np.zeros((T, H, C), np.float32)
    Ap[:A.shape[0]] = A
    Ap[A.shape[0]:] = np.nan
    cu = synth.cu_seqlens(LENGTHS)
    canary = -12345.0
    out = torch.full((T, H, C), canary, device=DEV)
    X = _solve_packed(kt, _dev(Ap), cu, out=out)
    n = A.shape[0]
    assert bool((X[n:] == canary).all())
    assert not bool((X[:n] == canary).any())
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(gh.to_numpy_f64(X[:n]), ref, "f32") <= 0


@pytest.mark.parametrize("C", SIZES)
def test_chunk_map_matches_device_scan(kt, C):
    H = 4
    A = _dev(synth.delta_rule_A(LENGTHS, H, seed=36, chunk=C))
    cu = synth.cu_seqlens(LENGTHS)
    cmap = torch.from_numpy(gh.host_chunk_map(LENGTHS, C)).to(DEV)
    X0 = _solve_packed(kt, A, cu)
    X1 = _solve_packed(kt, A, cu, chunk_indices=cmap)
    assert torch.equal(X0, X1)


@pytest.mark.parametrize("c", [1.0, -1.0, 0.5, -2.0])
@pytest.mark.parametrize("C", SIZES)
def test_exact_subdiagonal(kt, C, c):
    """A with c on the first subdiagonal only: X_ij = (-c)^(i-j) exactly
    (every sum has one nonzero term, so no rounding occurs)."""
    lengths = [C, C - 3, 2 * C + 1]
    H = 3
    T = sum(lengths)
    A = np.full((T, H, C), np.nan, np.float32)
    ref = np.zeros((T, H, C), np.float64)
    cu = synth.cu_seqlens(lengths)
    for _, s, L in oracle.chunks_packed(cu, C).tolist():
        for i in range(L):
            A[s + i, :, :i] = 0.0  # strictly lower part; the rest stays NaN
            if i > 0:
                A[s + i, :, i - 1] = c
            for j in range(i + 1):
                ref[s + i, :, j] = (-c) ** (i - j)
    got = gh.to_numpy_f64(_solve_packed(kt, _dev(A), cu))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("C", SIZES)
def test_deterministic_and_on_side_stream(kt, C):
    H = 8
    A = _dev(synth.delta_rule_A(LENGTHS, H, seed=37, chunk=C))
    cu = torch.from_numpy(synth.cu_seqlens(LENGTHS)).to(DEV)
    X0 = kt.tril_inv(A, cu)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        X1 = torch.empty_like(A)
        kt.kda_tril_inv_packed_chunk(A, X1, cu, C, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(X0, X1)


@pytest.mark.parametrize("C", SIZES)
def test_rejected_plans_and_empty_calls(kt, C):
    A = torch.zeros((C, 2, C), device=DEV)
    X = torch.empty_like(A)
    cu = torch.tensor([0, C], dtype=torch.int32, device=DEV)
    for algo in ("split", "fused_valu"):
        with pytest.raises(kt.KdaError) as e:
            kt.kda_tril_inv_packed_chunk(A, X, cu, C, algo=algo)
        assert e.value.status == kt.KDA_ERR_UNSUPPORTED
    E = torch.zeros((0, 2, C), device=DEV)
    kt.kda_tril_inv_packed_chunk(E, torch.empty_like(E), torch.zeros(1, dtype=torch.int32,
                                                                      device=DEV), C)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["packed_16x512_h64_c16_f32", "packed_16x512_h64_c32_f32"])
def test_full_workload(kt, name):
    """16 requests x 512 tokens, H = 64, in 16- or 32-token chunks: every
    chunk-head against the oracle, and the residual on a sample."""
    print(f"\n[small] workload {name}", flush=True)
    d = synth.make(name)
    got = gh.to_numpy_f64(_solve_packed(kt, _dev(d["A"]), d["cu_seqlens"]))
    ref = oracle.tril_inv_packed(d["A"], d["cu_seqlens"])
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    ch = gh.all_chunk_heads(d["lengths"], d["H"], d["chunk"])
    rng = np.random.default_rng(0)
    pick = [ch[i] for i in rng.choice(len(ch), 400, replace=False)]
    A64 = oracle.to_f64(d["A"], "f32")
    assert gh.residual_chunks(A64, got, pick) <= gh.RESIDUAL_TOL


@pytest.mark.parametrize("name", ["packed_16x512_h64_c16_f32", "packed_16x512_h64_c32_f32"])
def test_bench_launch_configuration(kt, name):
    """The launch pattern the benchmark times: calls prepared once per buffer
    set and issued back to back over rotating sets with no synchronisation;
    every set's X against the oracle."""
    print(f"\n[small] bench configuration {name}", flush=True)
    cfg = dict(synth.CONFIGS[name])
    sets = []
    for i in range(3):
        c = dict(cfg)
        c["seed"] = cfg["seed"] + 100 * i
        d = synth.make(c)
        A = _dev(d["A"])
        sets.append((d, A, torch.empty_like(A)))
    cu = torch.from_numpy(sets[0][0]["cu_seqlens"]).to(DEV)
    calls = [kt.prepare_packed(A, X, cu) for _, A, X in sets]
    for i in range(9):
        calls[i % 3]()
    torch.cuda.synchronize()
    for d, _, X in sets:
        e = gh.excess(gh.to_numpy_f64(X), oracle.tril_inv_packed(d["A"], d["cu_seqlens"]), "f32")
        assert e <= 0, f"seed {d['seed']}: exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("C", SIZES)
def test_graph_capture_replay(kt, C):
    """A captured call replays correctly several times, with eager work and
    synchronisations between the replays."""
    H = 4
    inputs = [synth.delta_rule_A(LENGTHS, H, seed=40 + i, chunk=C) for i in range(3)]
    cu = torch.from_numpy(synth.cu_seqlens(LENGTHS)).to(DEV)
    A = _dev(inputs[0])
    X = torch.empty_like(A)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kt.kda_tril_inv_packed(A, X, cu)  # warm-up outside the graph
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kt.kda_tril_inv_packed(A, X, cu)
    torch.cuda.synchronize()
    for rep in range(3):
        A.copy_(_dev(inputs[rep]))
        X.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = kt.tril_inv(A, cu)
        torch.cuda.synchronize()
        assert torch.equal(X, eager), f"replay {rep}"


def _both_small_layouts(monkeypatch, call):
    """call() under the 32-token group kernel and under the per-wavefront one."""
    out = {}
    for lay in ("group", "wave"):
        monkeypatch.setenv("KDA_TRIL_SMALL_LAYOUT", lay)
        out[lay] = call()
        torch.cuda.synchronize()
    monkeypatch.delenv("KDA_TRIL_SMALL_LAYOUT")
    return out["group"], out["wave"]


@pytest.mark.parametrize("H", [1, 2, 3, 7, 8, 9, 13])
def test_c32_group_kernel_edge_cases(kt, monkeypatch, H):
    """The 8-head group kernel of the 32-token branch (which launches of
    more than two groups per CU with 32 heads or more run;
    KDA_TRIL_SMALL_LAYOUT=group makes every launch use it):
    head counts that leave a group partly empty (a wavefront with one head
    or none), partial chunks and NaN above the diagonal; X bit for bit that
    of the per-wavefront kernel, within tolerance of the oracle, and rows past
    the requests untouched."""
    print(f"\n[small] c32 group H={H}", flush=True)
    A = synth.delta_rule_A(LENGTHS, H, seed=40 + H, chunk=32, upper="nan")
    cu = synth.cu_seqlens(LENGTHS)
    T = A.shape[0]
    pad = np.full((16, H, 32), np.nan, np.float32)
    Ad = torch.from_numpy(np.concatenate([A, pad])).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)

    def run():
        X = torch.full((T + 16, H, 32), -777.0, device=DEV)
        kt.tril_inv(Ad[:T], cud, out=X[:T])
        return X

    Xg, Xw = _both_small_layouts(monkeypatch, run)
    assert torch.equal(Xg, Xw)
    X = Xg.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == -777.0), "a row past the last request was written"
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(X[:T], ref, "f32") <= 0


@pytest.mark.parametrize("a_dtype,x_dtype", [("bf16", "f32"), ("f16", "f16"), ("f32", "bf16"),
                                             ("bf16", "bf16")])
def test_c32_group_kernel_dtypes_and_dense(kt, monkeypatch, a_dtype, x_dtype):
    H = 10
    A32 = synth.delta_rule_A(LENGTHS, H, seed=50, chunk=32)
    A = {"f32": A32, "bf16": synth.to_bf16_bits(A32), "f16": synth.to_f16_bits(A32)}[a_dtype]
    cu = synth.cu_seqlens(LENGTHS)
    Ad = gh.to_torch_input(A, a_dtype, DEV)
    cud = torch.from_numpy(cu).to(DEV)
    xt = gh.out_torch_dtype(x_dtype)
    Xg, Xw = _both_small_layouts(monkeypatch, lambda: kt.tril_inv(Ad, cud, out_dtype=xt))
    assert torch.equal(Xg, Xw)
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    assert gh.excess(gh.to_numpy_f64(Xg), ref, x_dtype) <= 0
    # dense [B, T, H, 32] through the group kernel equals the packed call
    B, Tn = 3, 70
    Adn = synth.delta_rule_A([Tn] * B, H, seed=51, chunk=32)
    Add = torch.from_numpy(Adn).to(DEV)
    Xd, _ = _both_small_layouts(monkeypatch, lambda: kt.tril_inv(Add.view(B, Tn, H, 32)))
    Xp, _ = _both_small_layouts(
        monkeypatch, lambda: kt.tril_inv(Add, torch.from_numpy(synth.cu_seqlens([Tn] * B)).to(DEV)))
    assert torch.equal(Xd.view(B * Tn, H, 32), Xp)


@pytest.mark.parametrize("C", SIZES)
def test_deterministic_across_grids(kt, monkeypatch, C):
    """The 16 x 512-token, 64-head batch (the 32-token group
    kernel, the 16-token walking kernel) on grids of 1, 2, 3 and 5
    workgroups per CU (KDA_TRIL_BLOCKS_PER_CU, read on every call), 10 calls
    each: X is the same bit for bit as on the default grid."""
    print(f"\n[small] grids C={C}", flush=True)
    name = f"packed_16x512_h64_c{C}_f32"
    d = synth.make(name)
    A = _dev(d["A"])
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    X0 = kt.tril_inv(A, cu)
    torch.cuda.synchronize()
    for bpc in ("1", "2", "3", "5"):
        monkeypatch.setenv("KDA_TRIL_BLOCKS_PER_CU", bpc)
        for _ in range(10):
            X = kt.tril_inv(A, cu)
            torch.cuda.synchronize()
            assert torch.equal(X, X0), bpc
    monkeypatch.delenv("KDA_TRIL_BLOCKS_PER_CU")
