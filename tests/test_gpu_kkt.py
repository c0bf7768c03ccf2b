"""GPU parity of the path that builds the delta-rule matrix A from keys,
decays and write strengths (kda_kkt_tril_inv_*, kda_kkt_*) against the fp64
oracle, which evaluates A from its definition and inverts it without
rounding.

Bar: X as for the solver (fp32 |X - X_ref| <= 2e-5 (1 + |X_ref|), bf16 / f16
with their relative terms, residual of the fp32 X against the oracle's
float64 A <= 1e-4); A from kda_kkt_* to the same elementwise bounds. Exact
zeros and the fused-equals-unfused identity are compared bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# full chunks, partial last chunks, a one-token request, a request of 3 chunks
LENGTHS = [64, 37, 1, 150, 16, 70]


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


def _inputs(lengths, H, K, k_dtype, seed):
    k, g, beta = synth.delta_rule_inputs(lengths, H, seed, K=K)
    if k_dtype == "bf16":
        k, beta = synth.to_bf16_bits(k), synth.to_bf16_bits(beta)
    elif k_dtype == "f16":
        k, beta = synth.to_f16_bits(k), synth.to_f16_bits(beta)
    return k, g, beta


def _dev(k, g, beta, k_dtype):
    return (gh.to_torch_input(k, k_dtype, DEV), torch.from_numpy(g).to(DEV),
            gh.to_torch_input(beta, k_dtype, DEV))


def _solve(kt, kd, gd, bd, cu, x_dtype="f32", solve=True, out=None, chunk_indices=None):
    shape = kd.shape[:-1] + (64,)
    X = out if out is not None else torch.empty(shape, dtype=gh.out_torch_dtype(x_dtype),
                                                device=DEV)
    cud = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).to(DEV)
    if solve:
        kt.kda_kkt_tril_inv(kd, gd, bd, X, cud, chunk_indices=chunk_indices)
    else:
        kt.kda_kkt(kd, gd, bd, X, cud, chunk_indices=chunk_indices)
    torch.cuda.synchronize()
    return X


@pytest.mark.parametrize("K", [16, 64, 128])
@pytest.mark.parametrize("H", [1, 3, 8])
def test_fused_parity(kt, H, K):
    print(f"\n[kkt] fused H={H} K={K}", flush=True)
    k, g, beta = _inputs(LENGTHS, H, K, "f32", seed=50 + H + K)
    cu = synth.cu_seqlens(LENGTHS)
    got = gh.to_numpy_f64(_solve(kt, *_dev(k, g, beta, "f32"), cu))
    A64 = oracle.kkt_packed(k, g, beta, cu)
    ref = oracle.tril_inv_packed(A64, cu, "f64")
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    assert gh.residual_chunks(A64, got, gh.all_chunk_heads(LENGTHS, H)) <= gh.RESIDUAL_TOL


@pytest.mark.parametrize("K", [16, 128])
@pytest.mark.parametrize("H", [2, 5])
def test_matrix_alone_parity_and_exact_zeros(kt, H, K):
    k, g, beta = _inputs(LENGTHS, H, K, "f32", seed=60 + H + K)
    cu = synth.cu_seqlens(LENGTHS)
    A = _solve(kt, *_dev(k, g, beta, "f32"), cu, solve=False)
    got = gh.to_numpy_f64(A)
    ref = oracle.kkt_packed(k, g, beta, cu)
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    for s, L, h in gh.all_chunk_heads(LENGTHS, H):
        blk = got[s:s + L, h]
        assert np.all(np.triu(blk[:, :L]) == 0) and np.all(blk[:, L:] == 0)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("k_dtype", ["f32", "bf16", "f16"])
def test_dtype_matrix(kt, k_dtype, x_dtype):
    print(f"\n[kkt] dtypes {k_dtype}->{x_dtype}", flush=True)
    H, K = 4, 128
    k, g, beta = _inputs(LENGTHS, H, K, k_dtype, seed=70)
    cu = synth.cu_seqlens(LENGTHS)
    dv = _dev(k, g, beta, k_dtype)
    got = gh.to_numpy_f64(_solve(kt, *dv, cu, x_dtype))
    ref = oracle.kkt_tril_inv_packed(k, g, beta, cu, k_dtype)
    e = gh.excess(got, ref, x_dtype)
    assert e <= 0, f"X exceeds tolerance by {e:.3g}"
    gotA = gh.to_numpy_f64(_solve(kt, *dv, cu, x_dtype, solve=False))
    refA = oracle.kkt_packed(k, g, beta, cu, k_dtype)
    e = gh.excess(gotA, refA, x_dtype)
    assert e <= 0, f"A exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("K", [16, 32, 48, 80, 256])
@pytest.mark.parametrize("k_dtype", ["bf16", "f16"])
def test_half_precision_keys_slice_tails(kt, k_dtype, K):
    """16-bit keys (a 32-channel slice is half of each key line, and the
    decays are read with their own cache policy) over K of one half slice,
    one slice, a slice and a half, two and a half slices and eight slices."""
    print(f"\n[kkt] {k_dtype} keys K={K}", flush=True)
    H = 3
    k, g, beta = _inputs(LENGTHS, H, K, k_dtype, seed=80 + K)
    cu = synth.cu_seqlens(LENGTHS)
    dv = _dev(k, g, beta, k_dtype)
    got = gh.to_numpy_f64(_solve(kt, *dv, cu))
    ref = oracle.kkt_tril_inv_packed(k, g, beta, cu, k_dtype)
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"X exceeds tolerance by {e:.3g}"
    gotA = gh.to_numpy_f64(_solve(kt, *dv, cu, solve=False))
    e = gh.excess(gotA, oracle.kkt_packed(k, g, beta, cu, k_dtype), "f32")
    assert e <= 0, f"A exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("k_dtype", ["f32", "bf16"])
def test_fused_equals_unfused_bitwise(kt, k_dtype):
    """X from the fused call equals, bit for bit, the 64-token solver applied
    to the FP32 A that kda_kkt_* stores: both solve the same FP32 values with
    the same code, the fused one without the round trip through memory."""
    H, K = 6, 128
    k, g, beta = _inputs(LENGTHS, H, K, k_dtype, seed=71)
    cu = synth.cu_seqlens(LENGTHS)
    dv = _dev(k, g, beta, k_dtype)
    Xf = _solve(kt, *dv, cu)
    A = _solve(kt, *dv, cu, solve=False)
    Xu = kt.tril_inv(A, torch.from_numpy(cu).to(DEV), algo="fused")
    torch.cuda.synchronize()
    assert torch.equal(Xf, Xu)


def test_dense_equals_packed_and_chunk_map(kt):
    B, T, H, K = 3, 100, 4, 64
    k, g, beta = _inputs([T] * B, H, K, "f32", seed=72)
    cu = synth.cu_seqlens([T] * B)
    dv = _dev(k, g, beta, "f32")
    Xp = _solve(kt, *dv, cu)
    kd, gd, bd = dv
    Xd = _solve(kt, kd.view(B, T, H, K), gd.view(B, T, H, K), bd.view(B, T, H), None)
    assert torch.equal(Xd.view(B * T, H, 64), Xp)
    Ad = _solve(kt, kd.view(B, T, H, K), gd.view(B, T, H, K), bd.view(B, T, H), None, solve=False)
    Ap = _solve(kt, *dv, cu, solve=False)
    assert torch.equal(Ad.view(B * T, H, 64), Ap)
    cmap = torch.from_numpy(gh.host_chunk_map([T] * B)).to(DEV)
    Xm = _solve(kt, *dv, cu, chunk_indices=cmap)
    assert torch.equal(Xm, Xp)


@pytest.mark.parametrize("solve", [True, False])
def test_rows_outside_chunks_untouched(kt, solve):
    H, K = 3, 32
    k, g, beta = _inputs(LENGTHS, H, K, "f32", seed=73)
    n = k.shape[0]
    extra = 9
    kp = np.concatenate([k, np.full((extra, H, K), np.nan, np.float32)])
    gp = np.concatenate([g, np.full((extra, H, K), np.nan, np.float32)])
    bp = np.concatenate([beta, np.full((extra, H), np.nan, np.float32)])
    canary = -777.0
    out = torch.full((n + extra, H, 64), canary, device=DEV)
    X = _solve(kt, *_dev(kp, gp, bp, "f32"), synth.cu_seqlens(LENGTHS), solve=solve, out=out)
    assert bool((X[n:] == canary).all())
    assert not bool((X[:n] == canary).any())
    assert bool(torch.isfinite(X[:n]).all())


def test_zero_keys_give_identity(kt):
    """k = 0 (any decays, beta): A = 0 exactly, so X = I exactly."""
    H, K = 2, 16
    T = sum(LENGTHS)
    rng = np.random.default_rng(3)
    k = np.zeros((T, H, K), np.float32)
    g = np.cumsum(-rng.random((T, H, K)), axis=0).astype(np.float32)
    beta = rng.random((T, H)).astype(np.float32)
    cu = synth.cu_seqlens(LENGTHS)
    X = gh.to_numpy_f64(_solve(kt, *_dev(k, g, beta, "f32"), cu))
    for s, L, h in gh.all_chunk_heads(LENGTHS, H):
        want = np.zeros((L, 64))
        want[:, :L] = np.eye(L)
        assert np.array_equal(X[s:s + L, h], want)


def _decay_inputs(lengths, H, K, mode, seed):
    """Keys and write strengths from the generator, decays chosen per mode:
      fast:    every channel falls by 5.4 per token (within 16 tokens, 86.4:
               the edge of the documented domain), restarting at each chunk;
      mixed:   half the channels fall by 5.4 per token, the others by the
               generator's logsigmoid draws;
      uniform: each (token, channel) falls by U(0, 5.4);
      request: falls U(0, 0.5) summed over the whole request (no restart at
               chunk boundaries) from -3000, so |g| runs into the thousands
               and only the differences within a chunk are small."""
    rng = np.random.default_rng(seed)
    k, g, beta = synth.delta_rule_inputs(lengths, H, seed, K=K)
    T = sum(lengths)
    if mode == "fast":
        fall = np.full((T, H, K), 5.4)
    elif mode == "mixed":
        fall = -np.diff(np.concatenate([np.zeros((1, H, K)), g.astype(np.float64)]), axis=0)
        fall[:, :, ::2] = 5.4
    elif mode in ("uniform", "request"):
        fall = rng.uniform(0.0, 5.4 if mode == "uniform" else 0.5, (T, H, K))
    g = np.zeros((T, H, K))
    bos = 0
    for n in lengths:
        for p in range(0, n, 64):
            hi = min(bos + n, bos + p + 64)
            if mode == "request":
                continue
            g[bos + p:hi] = -np.cumsum(fall[bos + p:hi], axis=0)
        if mode == "request":
            g[bos:bos + n] = -3000.0 - np.cumsum(fall[bos:bos + n], axis=0)
        bos += n
    return k, g.astype(np.float32), beta


@pytest.mark.parametrize("k_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["fast", "mixed", "uniform", "request"])
def test_decay_domain(kt, mode, k_dtype):
    """Parity across the documented decay domain (falls of up to 5.4 per
    token), with full and partial chunks, against the oracle's float64 A."""
    print(f"\n[kkt] decay domain {mode} k={k_dtype}", flush=True)
    lengths = [64, 37, 150, 64]
    H, K = 4, 128
    k, g, beta = _decay_inputs(lengths, H, K, mode, seed=90)
    if k_dtype == "bf16":
        k, beta = synth.to_bf16_bits(k), synth.to_bf16_bits(beta)
    cu = synth.cu_seqlens(lengths)
    X = gh.to_numpy_f64(_solve(kt, *_dev(k, g, beta, k_dtype), cu))
    A64 = oracle.kkt_packed(k, g, beta, cu, k_dtype)
    ref = oracle.tril_inv_packed(A64, cu, "f64")
    assert np.all(np.isfinite(X[~np.isnan(ref)]))
    e = gh.excess(X, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    assert gh.residual_chunks(A64, X, gh.all_chunk_heads(lengths, H)) <= gh.RESIDUAL_TOL
    # the matrix alone to the same bound
    Ag = gh.to_numpy_f64(_solve(kt, *_dev(k, g, beta, k_dtype), cu, solve=False))
    e = gh.excess(Ag, A64, "f32")
    assert e <= 0, f"A exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("name", ["packed_16x512_h64_k128_kkt_bf16_f32",
                                  "packed_16x512_h64_k128_kkt_f32_f32"])
def test_full_workload(kt, name):
    """16 requests x 512 tokens, 64 heads, K = 128 (the benchmark's batch):
    every one of the 8192 chunk-heads against the oracle, the residual of
    every fp32 X against the oracle's float64 A, and every row's unit
    diagonal and zero upper triangle bit for bit."""
    print(f"\n[kkt] workload {name}", flush=True)
    d = synth.make_kkt(name)
    dv = _dev(d["k"], d["g"], d["beta"], d["k_dtype"])
    X = _solve(kt, *dv, d["cu_seqlens"])
    T, H = d["T_total"], d["H"]
    t = X.view(T // 64, 64, H, 64).permute(0, 2, 1, 3)
    assert bool((torch.diagonal(t, dim1=2, dim2=3) == 1).all())
    upper = torch.triu(torch.ones(64, 64, device=DEV, dtype=torch.bool), 1)
    assert bool((t[:, :, upper] == 0).all())
    got = gh.to_numpy_f64(X)
    A64 = oracle.kkt_packed(d["k"], d["g"], d["beta"], d["cu_seqlens"], d["k_dtype"])
    ref = oracle.tril_inv_packed(A64, d["cu_seqlens"], "f64")
    e = gh.excess(got, ref, "f32")
    assert e <= 0, f"exceeds tolerance by {e:.3g}"
    assert gh.residual_full_chunks(A64, got) <= gh.RESIDUAL_TOL


def test_deterministic_across_grids(kt, monkeypatch):
    """The build-A path on the 16 x 512-token, 64-head batch (bf16 keys):
    20 repeats on each of three grids (1, 2 and 3 workgroups per compute
    unit, set per call) equal the default grid's result bit for bit."""
    name = "packed_16x512_h64_k128_kkt_bf16_f32"
    d = synth.make_kkt(name)
    kd, gd, bd = _dev(d["k"], d["g"], d["beta"], d["k_dtype"])
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    monkeypatch.delenv("KDA_TRIL_BLOCKS_PER_CU", raising=False)
    X0 = torch.empty((d["T_total"], d["H"], 64), device=DEV)
    kt.kda_kkt_tril_inv(kd, gd, bd, X0, cu)
    X = torch.empty_like(X0)
    call = kt.prepare_kkt(kd, gd, bd, X, cu)
    for per_cu in ("1", "2", "3"):
        monkeypatch.setenv("KDA_TRIL_BLOCKS_PER_CU", per_cu)
        for rep in range(20):
            X.fill_(float("nan"))
            call()
            assert torch.equal(X, X0), f"{per_cu} per CU, repeat {rep}"
    monkeypatch.delenv("KDA_TRIL_BLOCKS_PER_CU")


def test_bench_launch_configuration(kt):
    """Prepared build-A calls over two rotating buffer sets, issued back to
    back with no synchronisation, as the benchmark times them; each set's X
    checked in full against the oracle."""
    name = "packed_16x512_h64_k128_kkt_bf16_f32"
    cfg = dict(synth.KKT_CONFIGS[name])
    sets = []
    for i in range(2):
        c = dict(cfg)
        c["seed"] = cfg["seed"] + 100 * i
        d = synth.make_kkt(c)
        kd, gd, bd = _dev(d["k"], d["g"], d["beta"], d["k_dtype"])
        X = torch.empty((d["T_total"], d["H"], 64), device=DEV)
        sets.append((d, kd, gd, bd, X))
    cu = torch.from_numpy(sets[0][0]["cu_seqlens"]).to(DEV)
    calls = [kt.prepare_kkt(kd, gd, bd, X, cu) for _, kd, gd, bd, X in sets]
    for i in range(6):
        calls[i % 2]()
    torch.cuda.synchronize()
    for d, _, _, _, X in sets:
        ref = oracle.kkt_tril_inv_packed(d["k"], d["g"], d["beta"], d["cu_seqlens"],
                                         d["k_dtype"])
        e = gh.excess(gh.to_numpy_f64(X), ref, "f32")
        assert e <= 0, f"seed {d['seed']}: exceeds tolerance by {e:.3g}"
