"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 output |X - X_ref| <= 2e-5 (1 + |X_ref|); bf16 output
|X - X_ref| <= 1e-2 |X_ref| + 2e-5 (1 + |X_ref|); residual
max |(I + A) X - I| <= 1e-4 on fp32 outputs. Exact cases are compared bit
for bit. Every input is seeded; every expected value comes from the oracle
or from a closed form.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALGOS = ["fused", "split", "fused_valu"]


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


DEV = "cuda:0"


def _run_cfg(kt, d, algo, x_dtype=None):
    x_dtype = x_dtype or d["x_dtype"]
    A = gh.to_torch_input(d["A"], d["a_dtype"], DEV)
    if d["layout"] == "dense":
        X = kt.tril_inv(A, None, out_dtype=gh.out_torch_dtype(x_dtype), algo=algo)
    else:
        cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
        X = kt.tril_inv(A, cu, out_dtype=gh.out_torch_dtype(x_dtype), algo=algo)
    torch.cuda.synchronize()
    return X


def _oracle_cfg(d):
    if d["layout"] == "dense":
        return oracle.tril_inv_dense(d["A"], d["a_dtype"])
    return oracle.tril_inv_packed(d["A"], d["cu_seqlens"], d["a_dtype"])


_CFG_CACHE = {}


def _cfg(name):
    if name not in _CFG_CACHE:
        d = synth.make(name)
        d["ref"] = _oracle_cfg(d)
        _CFG_CACHE[name] = d
    return _CFG_CACHE[name]


SMALL_CFGS = ["packed_1x64_h64_f32", "dense_b4_t512_h16_bf16_f32",
              "packed_16x512_h64_f32", "packed_ragged48_h64_f32_bf16"]


@pytest.mark.parametrize("algo", ALGOS + ["auto"])
@pytest.mark.parametrize("name", SMALL_CFGS)
def test_config_parity(kt, name, algo):
    print(f"\n[parity] {name} algo={algo}", flush=True)
    d = _cfg(name)
    X = _run_cfg(kt, d, algo)
    got = gh.to_numpy_f64(X)
    ref = d["ref"]
    if d["layout"] == "dense":
        got = got.reshape(-1, d["H"], 64)
        ref = ref.reshape(-1, d["H"], 64)
    e = gh.excess(got, ref, d["x_dtype"])
    assert e <= 0, f"{name}/{algo}: exceeds tolerance by {e:.3g}"
    # residual on an fp32-output run of the same A (bf16 output alone would
    # carry ~1e-3 of rounding)
    if d["x_dtype"] == "f32":
        X32 = got
    else:
        X32 = gh.to_numpy_f64(_run_cfg(kt, d, algo, x_dtype="f32"))
    A64 = oracle.to_f64(d["A"], d["a_dtype"]).reshape(-1, d["H"], 64)
    X32 = X32.reshape(-1, d["H"], 64)
    ch = gh.all_chunk_heads(d["lengths"], d["H"])
    rng = np.random.default_rng(0)
    pick = [ch[i] for i in rng.choice(len(ch), min(len(ch), 400), replace=False)]
    assert gh.residual_chunks(A64, X32, pick) <= gh.RESIDUAL_TOL


C5_PLANS = ["fused", "split", "fused_valu", "auto"]
C5_SLICE = 8192  # tokens per oracle slice: a multiple of 64, so each slice holds whole chunks


@pytest.fixture(scope="module")
def c5(kt):
    """1 request x 131072 tokens, H = 64 (131072 matrices) solved once per
    plan on the GPU, then compared with the oracle slice by slice (8192
    tokens at a time, so host memory stays bounded; chunk boundaries are
    multiples of 64, so a slice solves exactly the chunks it holds). Returns,
    per plan, the largest excess over the fp32 bound, the largest residual,
    and whether the plan equals the fused kernel bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    name = "packed_1x131072_h64_f32"
    print(f"\n[c5] generating {name}", flush=True)
    d = synth.make(name)
    A = torch.from_numpy(d["A"]).to(DEV)
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    T, H = d["T_total"], d["H"]
    outs = {}
    for algo in C5_PLANS:
        print(f"[c5] solving algo={algo}", flush=True)
        outs[algo] = kt.tril_inv(A, cu, algo=algo)
    torch.cuda.synchronize()
    res = {a: {"excess": -1.0, "residual": 0.0, "invariants": True,
               "equals_fused": torch.equal(outs[a], outs["fused"])} for a in C5_PLANS}
    upper = torch.triu(torch.ones(64, 64, device=DEV, dtype=torch.bool), 1)
    for a, X in outs.items():
        t = X.view(T // 64, 64, H, 64).permute(0, 2, 1, 3)
        res[a]["invariants"] = bool((torch.diagonal(t, dim1=2, dim2=3) == 1).all()) and bool(
            (t[:, :, upper] == 0).all())
    cu_slice = np.array([0, C5_SLICE], np.int32)
    with ThreadPoolExecutor(len(C5_PLANS)) as ex:
        for s0 in range(0, T, C5_SLICE):
            A_sl = np.ascontiguousarray(d["A"][s0:s0 + C5_SLICE])
            ref = oracle.tril_inv_packed(A_sl, cu_slice)

            def compare(algo, A_sl=A_sl, ref=ref, s0=s0):
                got = outs[algo][s0:s0 + C5_SLICE].cpu().numpy().astype(np.float64)
                return algo, gh.excess(got, ref, "f32"), gh.residual_full_chunks(A_sl, got)

            for algo, e, r in ex.map(compare, C5_PLANS):
                res[algo]["excess"] = max(res[algo]["excess"], e)
                res[algo]["residual"] = max(res[algo]["residual"], r)
            if s0 % (4 * C5_SLICE) == 0:
                print(f"[c5] compared tokens {s0}..{s0 + C5_SLICE}", flush=True)
    return res


@pytest.mark.parametrize("algo", C5_PLANS)
def test_long_context_full(c5, algo):
    """Every one of C5's 131072 chunk-heads against the oracle, for every
    64-token plan: elementwise fp32 bound, residual, unit diagonal and zero
    upper triangle on every row; split and auto (which picks fused here) equal
    the fused kernel bit for bit (same operations in the same order)."""
    r = c5[algo]
    assert r["invariants"]
    assert r["excess"] <= 0, f"{algo}: exceeds tolerance by {r['excess']:.3g}"
    assert r["residual"] <= gh.RESIDUAL_TOL, f"{algo}: residual {r['residual']:.3g}"
    if algo in ("split", "auto"):
        assert r["equals_fused"]


def _subdiag_input(H, lengths, c):
    T = sum(lengths)
    A = np.zeros((T, H, 64), np.float32)
    bos = 0
    for n in lengths:
        for p in range(0, n, 64):
            L = min(64, n - p)
            for i in range(1, L):
                A[bos + p + i, :, i - 1] = c
        bos += n
    return A


@pytest.mark.parametrize("c", [1.0, -1.0, 0.5, -0.5, 2.0, -2.0])
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_exact_subdiagonal(kt, c, algo, x_dtype):
    """A[i, i-1] = c: X[i, j] = (-c)^(i-j) exactly (one nonzero term per sum)."""
    lengths = [64, 64, 23]
    H = 3
    A = _subdiag_input(H, lengths, c)
    cu = synth.cu_seqlens(lengths)
    X = kt.tril_inv(torch.from_numpy(A).to(DEV), torch.from_numpy(cu).to(DEV),
                    out_dtype=gh.out_torch_dtype(x_dtype), algo=algo)
    got = gh.to_numpy_f64(X)
    bos = 0
    for n in lengths:
        for p in range(0, n, 64):
            L = min(64, n - p)
            want = np.zeros((L, 64))
            for i in range(L):
                for j in range(i + 1):
                    want[i, j] = (-c) ** (i - j)
            for h in range(H):
                assert np.array_equal(got[bos + p:bos + p + L, h, :], want), (n, p, h)
        bos += n


@pytest.mark.parametrize("algo", ALGOS)
def test_zero_and_single_entry(kt, algo):
    H = 2
    A = np.zeros((64, H, 64), np.float32)
    cu = torch.tensor([0, 64], dtype=torch.int32, device=DEV)
    X = kt.tril_inv(torch.from_numpy(A).to(DEV), cu, algo=algo).cpu().numpy()
    for h in range(H):
        assert np.array_equal(X[:, h, :], np.eye(64, dtype=np.float32))
    # one nonzero a at (i, j): (I + a E_ij)^-1 = I - a E_ij, bit for bit
    for (i, j) in [(1, 0), (15, 3), (17, 16), (40, 2), (63, 0), (63, 62), (33, 31), (50, 20)]:
        A = np.zeros((64, H, 64), np.float32)
        A[i, 1, j] = 0.375
        X = kt.tril_inv(torch.from_numpy(A).to(DEV), cu, algo=algo).cpu().numpy()
        want = np.eye(64, dtype=np.float32)
        want[i, j] = -0.375
        assert np.array_equal(X[:, 1, :], want), (i, j)
        assert np.array_equal(X[:, 0, :], np.eye(64, dtype=np.float32))


PARTIAL_LENGTHS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_partial_chunks_and_canaries(kt, algo, x_dtype):
    """Ragged lengths with NaN on and above the diagonal of A. Valid rows
    match the oracle, carry exact 1 on the diagonal and +0 above it; rows past
    cu_seqlens[-1] and guard bands around X stay untouched."""
    H = 4
    lengths = PARTIAL_LENGTHS
    T = sum(lengths)
    tail = 37
    A = np.zeros((T + tail, H, 64), np.float32)
    A[:T] = synth.delta_rule_A(lengths, H, seed=21, upper="nan")
    A[T:] = np.nan
    cu = synth.cu_seqlens(lengths)
    tdt = gh.out_torch_dtype(x_dtype)
    canary = torch.tensor(-1234.5, dtype=tdt)
    pad = 64
    buf = torch.full((T + tail + 2 * pad, H, 64), float(canary), dtype=tdt, device=DEV)
    X = buf[pad:pad + T + tail]
    kt.kda_tril_inv_packed(torch.from_numpy(A).to(DEV), X, torch.from_numpy(cu).to(DEV),
                           workspace=_workspace(kt, T + tail, len(lengths), H, algo), algo=algo)
    torch.cuda.synchronize()
    b = gh.to_numpy_f64(buf)
    assert np.all(b[:pad] == float(canary)) and np.all(b[pad + T + tail:] == float(canary))
    got = b[pad:pad + T + tail]
    assert np.all(got[T:] == float(canary)), "rows past the last request were written"
    ref = oracle.tril_inv_packed(A, cu, fill=np.nan)
    assert gh.excess(got[:T], ref[:T], x_dtype) <= 0
    raw = X.cpu()
    if x_dtype == "bf16":
        bits = raw.view(torch.int16).numpy().view(np.uint16)
        one, zero = 0x3F80, 0
    else:
        bits = raw.view(torch.int32).numpy().view(np.uint32)
        one, zero = 0x3F800000, 0
    for s, L, h in gh.all_chunk_heads(lengths, H):
        blk = bits[s:s + L, h, :]
        for i in range(L):
            assert blk[i, i] == one
            assert np.all(blk[i, i + 1:] == zero)


def _workspace(kt, T, nseq, H, algo, nchunks=0):
    nbytes, _ = kt.kda_tril_inv_workspace_size(T, nseq, nchunks, H, algo)
    if not nbytes:
        return None
    return torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("T", [512, 300])
def test_dense_equals_packed(kt, T):
    B, H = 3, 5
    A = synth.delta_rule_A([T] * B, H, seed=31)
    Ad = torch.from_numpy(A).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens([T] * B)).to(DEV)
    Xp = kt.tril_inv(Ad, cu, algo="fused")
    Xd = kt.tril_inv(Ad.view(B, T, H, 64), None, algo="fused")
    assert torch.equal(Xp.view(B, T, H, 64), Xd)
    Xs = kt.tril_inv(Ad.view(B, T, H, 64), None, algo="split")
    assert torch.equal(Xs, Xd)


def test_dense_equals_packed_multi_round(kt):
    """The dense layout's arithmetic chunk lookup in a launch whose wavefronts
    walk several items (B = 2, T = 5100 with a partial last chunk, 64 heads:
    10,240 work items), against the same data through the packed scan, bit
    for bit, for the fused and the split plans."""
    B, T, H = 2, 5100, 64
    A = synth.delta_rule_A([T] * B, H, seed=37)
    Ad = torch.from_numpy(A).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens([T] * B)).to(DEV)
    Xp = kt.tril_inv(Ad, cu, algo="fused")
    Xd = kt.tril_inv(Ad.view(B, T, H, 64), None, algo="fused")
    assert torch.equal(Xp.view(B, T, H, 64), Xd)
    Xs = kt.tril_inv(Ad.view(B, T, H, 64), None, algo="split")
    assert torch.equal(Xs, Xd)


@pytest.mark.parametrize("algo", ALGOS)
def test_bf16_output_is_rne_of_fp32_output(kt, algo):
    lengths = [512, 300, 64, 7]
    H = 8
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=41)).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    X32 = kt.tril_inv(A, cu, out_dtype=torch.float32, algo=algo)
    X16 = kt.tril_inv(A, cu, out_dtype=torch.bfloat16, algo=algo)
    want = oracle.rne_bf16(X32.cpu().numpy())
    assert np.array_equal(gh.bits16(X16), want)


@pytest.mark.parametrize("algo", ALGOS)
def test_f16_output_is_rne_of_fp32_output(kt, algo):
    lengths = [512, 300, 64, 7]
    H = 8
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=43)).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    X32 = kt.tril_inv(A, cu, out_dtype=torch.float32, algo=algo)
    X16 = kt.tril_inv(A, cu, out_dtype=torch.float16, algo=algo)
    assert np.array_equal(gh.bits16(X16), oracle.rne_f16(X32.cpu().numpy()))


@pytest.mark.parametrize("a_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16", "f16"])
def test_dtype_matrix(kt, a_dtype, x_dtype):
    """Every input x output element type, each plan, against the oracle on
    the materialised (rounded) input."""
    lengths = [300, 64, 17, 1]
    H = 5
    A32 = synth.delta_rule_A(lengths, H, seed=47)
    A = {"f32": A32, "bf16": synth.to_bf16_bits(A32), "f16": synth.to_f16_bits(A32)}[a_dtype]
    cu = synth.cu_seqlens(lengths)
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    Ad = gh.to_torch_input(A, a_dtype, DEV)
    for algo in ALGOS:
        X = kt.tril_inv(Ad, torch.from_numpy(cu).to(DEV), out_dtype=gh.out_torch_dtype(x_dtype),
                        algo=algo)
        assert gh.excess(gh.to_numpy_f64(X), ref, x_dtype) <= 0, algo


_MULTI_ROUND = {}


@pytest.mark.parametrize("a_dtype", ["f32", "bf16", "f16"])
def test_dtype_matrix_multi_round(kt, a_dtype):
    """The fused kernels pick their diagonal-block load layout per launch: one
    row per lane when every work item has its own wavefront, 16 rows per
    instruction plus a lane-swap transpose when wavefronts walk several items.
    The small cases above run in one round; this one has 10,240 tokens x 64
    heads (2.5 rounds of a 256-CU MI355X at 16 wavefronts per CU), ragged
    requests included, through every output type and both merge engines."""
    lengths = [5000, 3000, 2240]
    H = 64
    if "A" not in _MULTI_ROUND:
        _MULTI_ROUND["A"] = synth.delta_rule_A(lengths, H, seed=61)
    A32 = _MULTI_ROUND["A"]
    A = {"f32": A32, "bf16": synth.to_bf16_bits(A32), "f16": synth.to_f16_bits(A32)}[a_dtype]
    cu = synth.cu_seqlens(lengths)
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    Ad = gh.to_torch_input(A, a_dtype, DEV)
    cud = torch.from_numpy(cu).to(DEV)
    for algo in ("fused", "fused_valu"):
        for x_dtype in ("f32", "bf16", "f16"):
            X = kt.tril_inv(Ad, cud, out_dtype=gh.out_torch_dtype(x_dtype), algo=algo)
            e = gh.excess(gh.to_numpy_f64(X), ref, x_dtype)
            assert e <= 0, f"{algo} {a_dtype}->{x_dtype}: exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("algo", ["fused", "fused_valu"])
def test_one_round_equals_multi_round_bitwise(kt, algo):
    """The two diagonal-load layouts differ only in how the diagonal rows reach
    the lanes, so X is the same bit for bit: the first 64-token chunk of every
    head solved alone (one round, one row per lane) against the same rows of
    the 10,240-token call (2.5 rounds, 16-row loads and lane swaps)."""
    lengths = [5000, 3000, 2240]
    H = 64
    if "A" not in _MULTI_ROUND:
        _MULTI_ROUND["A"] = synth.delta_rule_A(lengths, H, seed=61)
    A = _MULTI_ROUND["A"]
    Ad = gh.to_torch_input(A, "f32", DEV)
    X_big = kt.tril_inv(Ad, torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV), algo=algo)
    A_small = Ad[:64].contiguous()
    X_small = kt.tril_inv(A_small, torch.from_numpy(synth.cu_seqlens([64])).to(DEV), algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(X_small, X_big[:64])


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_bf16_input(kt, x_dtype):
    lengths = [200, 64, 1]
    H = 6
    A = synth.to_bf16_bits(synth.delta_rule_A(lengths, H, seed=51))
    cu = synth.cu_seqlens(lengths)
    Ad = gh.to_torch_input(A, "bf16", DEV)
    for algo in ALGOS:
        X = kt.tril_inv(Ad, torch.from_numpy(cu).to(DEV), out_dtype=gh.out_torch_dtype(x_dtype),
                        algo=algo)
        ref = oracle.tril_inv_packed(A, cu, "bf16")
        assert gh.excess(gh.to_numpy_f64(X), ref, x_dtype) <= 0, algo


def test_split_equals_fused_bitwise(kt):
    """The split path runs the same diagonal and merge arithmetic in the same
    order, so it matches the fused kernel bit for bit."""
    d = _cfg("packed_ragged48_h64_f32_bf16")
    A = torch.from_numpy(d["A"]).to(DEV)
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    for dt in (torch.float32, torch.bfloat16):
        Xf = kt.tril_inv(A, cu, out_dtype=dt, algo="fused")
        Xs = kt.tril_inv(A, cu, out_dtype=dt, algo="split")
        assert torch.equal(Xf, Xs)


@pytest.mark.parametrize("algo", ALGOS)
def test_garbage_above_diagonal_is_ignored(kt, algo):
    lengths = [64, 100, 5]
    H = 4
    clean = synth.delta_rule_A(lengths, H, seed=61)
    dirty = synth.delta_rule_A(lengths, H, seed=61, upper="garbage")
    assert np.isnan(dirty).any() and np.isinf(dirty).any()
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    Xc = kt.tril_inv(torch.from_numpy(clean).to(DEV), cu, algo=algo)
    Xd = kt.tril_inv(torch.from_numpy(dirty).to(DEV), cu, algo=algo)
    assert torch.equal(Xc, Xd)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", ["packed_16x512_h64_f32", "packed_ragged48_h64_f32_bf16"])
def test_deterministic_across_grids(kt, name, algo, monkeypatch):
    """100 repeats on each of three grids besides the default one (1, 2 and
    3 workgroups per compute unit, set per call by KDA_TRIL_BLOCKS_PER_CU, so
    wavefronts walk 2 to 8 items each and different wavefronts and compute
    units get each item): every result equals the default grid's bit for
    bit. The split plan launches one wavefront per item whatever the
    setting, and is repeated all the same."""
    print(f"\n[determinism] {name} algo={algo}", flush=True)
    d = _cfg(name)
    A = gh.to_torch_input(d["A"], d["a_dtype"], DEV)
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    xt = gh.out_torch_dtype(d["x_dtype"])
    monkeypatch.delenv("KDA_TRIL_BLOCKS_PER_CU", raising=False)
    X0 = kt.tril_inv(A, cu, out_dtype=xt, algo=algo)
    X = torch.empty_like(X0)
    nbytes, _ = kt.kda_tril_inv_workspace_size(d["T_total"], len(d["lengths"]), 0, d["H"], algo)
    ws = torch.empty(max(nbytes // 4, 1), device=DEV) if nbytes else None
    call = kt.prepare_packed(A, X, cu, workspace=ws, algo=algo)
    for per_cu in ("1", "2", "3"):
        monkeypatch.setenv("KDA_TRIL_BLOCKS_PER_CU", per_cu)
        for rep in range(100):
            X.fill_(float("nan"))
            call()
            assert torch.equal(X, X0), f"{per_cu} per CU, repeat {rep}"
    monkeypatch.delenv("KDA_TRIL_BLOCKS_PER_CU")
    torch.cuda.synchronize()


@pytest.mark.parametrize("algo", ["fused", "split"])
def test_chunk_map_matches_device_scan(kt, algo):
    rng = np.random.default_rng(71)
    lengths = [int(v) for v in rng.integers(0, 300, 200)]  # includes empty requests
    H = 3
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=71)).to(DEV)
    cu_np = synth.cu_seqlens(lengths)
    cu = torch.from_numpy(cu_np).to(DEV)
    cmap = torch.from_numpy(gh.host_chunk_map(lengths)).to(DEV)
    X0 = kt.tril_inv(A, cu, algo=algo)
    X1 = kt.tril_inv(A, cu, algo=algo, chunk_indices=cmap)
    assert torch.equal(X0, X1)
    ref = oracle.tril_inv_packed(A.cpu().numpy(), cu_np)
    assert gh.excess(gh.to_numpy_f64(X0), ref, "f32") <= 0


def test_split_workspace_guard_bands(kt):
    lengths = [512, 77]
    H = 4
    T = sum(lengths)
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=81)).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    nbytes, chosen = kt.kda_tril_inv_workspace_size(T, len(lengths), 0, H, "split")
    assert chosen == "split" and nbytes == (T // 64 + len(lengths)) * H * 4096
    pad = 1024
    wbuf = torch.full((nbytes // 4 + 2 * pad,), 777.0, device=DEV)
    ws = wbuf[pad:pad + nbytes // 4]
    X = torch.empty_like(A)
    kt.kda_tril_inv_packed(A, X, cu, workspace=ws, algo="split")
    torch.cuda.synchronize()
    assert bool((wbuf[:pad] == 777.0).all()) and bool((wbuf[pad + nbytes // 4:] == 777.0).all())
    assert torch.equal(X, kt.tril_inv(A, cu, algo="fused"))


def test_non_default_stream(kt):
    lengths = [512] * 4
    H = 16
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=91)).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    ref = kt.tril_inv(A, cu)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        X = kt.tril_inv(A, cu)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(X, ref)


def test_split_on_a_stream_that_is_not_current(kt, monkeypatch):
    """tril_inv(..., stream=side) with the split plan while `side` is not the
    current stream: the workspace it allocates must belong to `side`, so once
    tril_inv returns and frees it, the caching allocator cannot hand the block
    to work on the current stream while the split kernels may still use it.
    The side stream is held behind a slow computation on a third stream, and
    a same-sized allocation on the current stream is filled meanwhile; X must
    equal the fused result bit for bit, and that allocation must not be the
    workspace's block."""
    lengths = [512] * 8
    H = 16
    A = torch.from_numpy(synth.delta_rule_A(lengths, H, seed=93)).to(DEV)
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    ref = kt.tril_inv(A, cu, algo="fused")
    torch.cuda.synchronize()
    seen = {}
    real = kt.kda_tril_inv_packed

    def spy(A_, X_, cu_, chunk_indices=None, workspace=None, algo="auto", stream=None):
        seen["ws"] = (workspace.data_ptr(), workspace.numel())
        return real(A_, X_, cu_, chunk_indices=chunk_indices, workspace=workspace, algo=algo,
                    stream=stream)

    monkeypatch.setattr(kt, "kda_tril_inv_packed", spy)
    gate, side = torch.cuda.Stream(), torch.cuda.Stream()
    M = torch.randn(2048, 2048, device=DEV)
    gate.wait_stream(torch.cuda.current_stream())
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gate):
        for _ in range(20):
            M = torch.tanh(M @ M)
    side.wait_stream(gate)
    X = kt.tril_inv(A, cu, algo="split", stream=side)
    ptr, n = seen["ws"]
    Y = torch.empty(n, dtype=torch.float32, device=DEV)  # current stream
    Y.fill_(float("nan"))
    assert Y.data_ptr() != ptr
    torch.cuda.synchronize()
    assert torch.equal(X, ref)


def test_empty_problems_are_noops(kt):
    A = torch.zeros((0, 4, 64), device=DEV)
    X = torch.zeros((0, 4, 64), device=DEV)
    kt.kda_tril_inv_packed(A, X, torch.zeros(1, dtype=torch.int32, device=DEV))
    A = torch.zeros((64, 4, 64), device=DEV)
    X = torch.full((64, 4, 64), 5.0, device=DEV)
    kt.kda_tril_inv_packed(A, X, torch.tensor([0, 0, 0], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert bool((X == 5.0).all())
    kt.kda_tril_inv_dense(torch.zeros((0, 64, 4, 64), device=DEV),
                          torch.zeros((0, 64, 4, 64), device=DEV))


def test_forced_split_without_workspace_fails(kt):
    A = torch.zeros((128, 2, 64), device=DEV)
    X = torch.empty_like(A)
    cu = torch.tensor([0, 128], dtype=torch.int32, device=DEV)
    with pytest.raises(kt.KdaError) as e:
        kt.kda_tril_inv_packed(A, X, cu, algo="split")
    assert e.value.status == kt.KDA_ERR_WORKSPACE
    # AUTO without workspace falls back to the fused kernel
    kt.kda_tril_inv_packed(A, X, cu, algo="auto")
    torch.cuda.synchronize()
    assert torch.equal(X[:, 0, :], torch.eye(64, device=DEV).repeat(2, 1))


@pytest.mark.parametrize("algo", ["fused", "split"])
def test_graph_capture_replay(kt, algo):
    """One call captured in a HIP graph with a caller-kept chunk map (as a
    layer loop would reuse it) and a fixed workspace, replayed on new inputs
    with eager work and synchronisation between replays; every replay equals
    the eager result bit for bit."""
    lengths = [512, 300, 64, 9]
    H = 8
    T = sum(lengths)
    inputs = [synth.delta_rule_A(lengths, H, seed=s) for s in (101, 102, 103)]
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    cmap = torch.from_numpy(gh.host_chunk_map(lengths)).to(DEV)
    A = torch.from_numpy(inputs[0]).to(DEV)
    X = torch.empty_like(A)
    nbytes, _ = kt.kda_tril_inv_workspace_size(T, len(lengths), cmap.shape[0], H, algo)
    ws = torch.empty(max(nbytes // 4, 1), device=DEV) if nbytes else None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kt.kda_tril_inv_packed(A, X, cu, chunk_indices=cmap, workspace=ws, algo=algo)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kt.kda_tril_inv_packed(A, X, cu, chunk_indices=cmap, workspace=ws, algo=algo)
    for i in range(6):
        A.copy_(torch.from_numpy(inputs[i % 3]))
        X.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = kt.tril_inv(A, cu, algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(X, ref), i


@pytest.mark.parametrize("name", ["packed_16x512_h64_f32", "packed_ragged48_h64_f32_bf16"])
def test_bench_launch_configuration(kt, name):
    """The launch pattern the benchmark times: calls prepared once per buffer
    set and issued back to back on one stream over rotating sets, with no
    synchronisation in between. Every set's X must still match the oracle."""
    print(f"\n[bench-config] {name}", flush=True)
    cfg = dict(synth.CONFIGS[name])
    sets = []
    for i in range(3):
        c = dict(cfg)
        c["seed"] = cfg["seed"] + 100 * i
        d = synth.make(c)
        A = gh.to_torch_input(d["A"], d["a_dtype"], DEV)
        X = torch.empty(A.shape, dtype=gh.out_torch_dtype(d["x_dtype"]), device=DEV)
        sets.append((d, A, X))
    cu = torch.from_numpy(sets[0][0]["cu_seqlens"]).to(DEV)
    calls = [kt.prepare_packed(A, X, cu, algo="auto") for _, A, X in sets]
    for i in range(9):
        calls[i % 3]()
    torch.cuda.synchronize()
    for d, _, X in sets:
        ref = oracle.tril_inv_packed(d["A"], d["cu_seqlens"], d["a_dtype"])
        e = gh.excess(gh.to_numpy_f64(X), ref, d["x_dtype"])
        assert e <= 0, f"seed {d['seed']}: exceeds tolerance by {e:.3g}"
