"""GPU tests of the fused solver's column kernel.

Launches of at most two chunk-heads per compute unit (a 64-token request over
64 heads, a few short requests) run tril_inv_fused_cols: two wavefronts per
chunk-head (or four) compute two block columns of X each (or one), and after
one barrier they store the block rows; a workgroup holds one chunk-head or
two. KDA_TRIL_FUSED_LAYOUT=cols2, cols2p (two chunk-heads per workgroup) and
cols4 make every launch use one form, so these tests also reach them on
problems that take several rounds. Every case is compared with the oracle
and, bit for bit, with the one-wavefront kernel (layout "wave"), whose
products it runs in the same order. The one-wavefront kernel's one-round
launches (workgroups of one wavefront, or of four past two chunk-heads per
CU) are compared with the 4-head kernel.
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


@pytest.fixture(params=["cols2", "cols2p", "cols4"])
def lay(request):
    return request.param


def _cols_and_wave(monkeypatch, call, lay):
    """call() under the column kernel (layout `lay`) and under the
    one-wavefront one."""
    out = {}
    for name in (lay, "wave"):
        monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", name)
        out[name] = call()
        torch.cuda.synchronize()
    monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT")
    return out[lay], out["wave"]


@pytest.mark.parametrize("H", [1, 3, 4, 7, 64])  # odd item counts leave a half-empty workgroup
def test_head_counts_and_partial_chunks(kt, monkeypatch, lay, H):
    print(f"\n[cols] {lay} H={H}", flush=True)
    A = synth.delta_rule_A(LENGTHS, H, seed=600 + H, upper="nan")
    cu = synth.cu_seqlens(LENGTHS)
    T = A.shape[0]
    Ad = torch.from_numpy(np.concatenate([A, np.full((PAD, H, 64), np.nan, np.float32)])).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)

    def run():
        X = torch.full((T + PAD, H, 64), CANARY, device=DEV)
        kt.tril_inv(Ad[:T], cud, algo="fused", out=X[:T])
        return X

    Xc, Xw = _cols_and_wave(monkeypatch, run, lay)
    assert torch.equal(Xc, Xw)
    X = Xc.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY), "a row past the last request was written"
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(X[:T], ref, "f32") <= 0


@pytest.mark.parametrize("a_dtype,x_dtype", [("f32", "bf16"), ("bf16", "f32"), ("f16", "f16"),
                                             ("bf16", "bf16"), ("f16", "f32")])
def test_dtypes(kt, monkeypatch, lay, a_dtype, x_dtype):
    H = 6
    A32 = synth.delta_rule_A(LENGTHS, H, seed=610)
    A = {"f32": A32, "bf16": synth.to_bf16_bits(A32), "f16": synth.to_f16_bits(A32)}[a_dtype]
    cu = synth.cu_seqlens(LENGTHS)
    Ad = gh.to_torch_input(A, a_dtype, DEV)
    cud = torch.from_numpy(cu).to(DEV)
    xt = gh.out_torch_dtype(x_dtype)
    Xc, Xw = _cols_and_wave(monkeypatch,
                            lambda: kt.tril_inv(Ad, cud, out_dtype=xt, algo="fused"), lay)
    assert torch.equal(Xc, Xw)
    ref = oracle.tril_inv_packed(A, cu, a_dtype)
    assert gh.excess(gh.to_numpy_f64(Xc), ref, x_dtype) <= 0


def test_dense_layout_and_chunk_map(kt, monkeypatch, lay):
    H = 5
    B, T = 3, 150
    A = synth.delta_rule_A([T] * B, H, seed=620)
    Ad = torch.from_numpy(A).to(DEV)
    Xc, Xw = _cols_and_wave(monkeypatch,
                            lambda: kt.tril_inv(Ad.view(B, T, H, 64), algo="fused"), lay)
    assert torch.equal(Xc, Xw)
    cu = synth.cu_seqlens([T] * B)
    cud = torch.from_numpy(cu).to(DEV)
    cmap = torch.from_numpy(gh.host_chunk_map([T] * B)).to(DEV)
    Xm, _ = _cols_and_wave(monkeypatch,
                           lambda: kt.tril_inv(Ad, cud, chunk_indices=cmap, algo="fused"), lay)
    assert torch.equal(Xm.view(B, T, H, 64), Xc)
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(gh.to_numpy_f64(Xm), ref, "f32") <= 0


@pytest.mark.parametrize("cu,clamped", [([0, 64, 200], [0, 64, 100]),
                                        ([-40, 64, 100], [24, 64, 100]),
                                        ([0, 64, 100, 300], [0, 64, 100, 100])])
def test_malformed_cu_seqlens_clamped(kt, monkeypatch, lay, cu, clamped):
    """Chunks outside rows [0, T) are skipped or cut at T: nothing past T is
    read (NaN there) or written (canaries)."""
    H = 3
    A = synth.delta_rule_A([64, 36], H, seed=630)
    T = A.shape[0]
    Ad = torch.from_numpy(np.concatenate([A, np.full((PAD, H, 64), np.nan, np.float32)])).to(DEV)
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)

    def run():
        X = torch.full((T + PAD, H, 64), CANARY, device=DEV)
        kt.tril_inv(Ad[:T], cud, algo="fused", out=X[:T])
        return X

    Xc, Xw = _cols_and_wave(monkeypatch, run, lay)
    assert torch.equal(Xc, Xw)
    X = Xc.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY)
    ref = np.full(A.shape, np.nan)
    for s, e in zip(clamped[:-1], clamped[1:]):
        if s < e:
            ref[s:e] = oracle.tril_inv_packed(A[s:e], [0, e - s])
    rows = ~np.isnan(ref[:, 0, 0])
    assert gh.excess(X[:T][rows], ref[rows], "f32") <= 0


def test_multi_round_problem(kt, monkeypatch, lay):
    """Forced on a problem of many rounds (one workgroup per chunk-head, the
    GPU schedules them in turn): the same X as the 4-head kernel the launch
    would otherwise run."""
    d = synth.make("packed_16x512_h64_f32")
    A = torch.from_numpy(d["A"]).to(DEV)
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    out = {}
    for name in (lay, "heads4"):
        monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", name)
        out[name] = kt.tril_inv(A, cu, algo="fused")
        torch.cuda.synchronize()
    assert torch.equal(out[lay], out["heads4"])


def test_auto_choice_on_small_workloads(kt):
    """Without the variable, a 64-token request over 64 heads (64 chunk-heads,
    the column kernel's size) is solved within tolerance of the oracle."""
    d = synth.make("packed_1x64_h64_f32")
    A = torch.from_numpy(d["A"]).to(DEV)
    cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
    X = kt.tril_inv(A, cu)
    ref = oracle.tril_inv_packed(d["A"], d["cu_seqlens"])
    assert gh.excess(X.cpu().numpy().astype(np.float64), ref, "f32") <= 0


def test_graph_capture_replay(kt, monkeypatch, lay):
    """Captured in a HIP graph and replayed on new inputs, with eager work and
    synchronisation between replays: every replay equals the eager result."""
    monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", lay)
    lengths = [64, 100, 9]
    H = 8
    inputs = [synth.delta_rule_A(lengths, H, seed=s) for s in (641, 642, 643)]
    cu = torch.from_numpy(synth.cu_seqlens(lengths)).to(DEV)
    A = torch.from_numpy(inputs[0]).to(DEV)
    X = torch.empty_like(A)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kt.kda_tril_inv_packed(A, X, cu, algo="fused")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kt.kda_tril_inv_packed(A, X, cu, algo="fused")
    for i in range(6):
        A.copy_(torch.from_numpy(inputs[i % 3]))
        X.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = kt.tril_inv(A, cu, algo="fused")
        torch.cuda.synchronize()
        assert torch.equal(X, eager), f"replay {i}"


@pytest.mark.parametrize("requests", [1, 4, 9, 16, 40])
def test_one_round_workgroup_shapes(kt, monkeypatch, requests):
    """One-round launches of the one-wavefront kernel (64 to 2,560
    chunk-heads: workgroups of one wavefront up to two chunk-heads per CU, of
    four beyond) and the automatic choice: X bit for bit that of the 4-head
    kernel, and within tolerance of the oracle."""
    lengths = [64] * requests
    H = 64
    A = synth.delta_rule_A(lengths, H, seed=650 + requests)
    cu = synth.cu_seqlens(lengths)
    Ad = torch.from_numpy(A).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    out = {}
    for name in ("wave", "heads4", None):
        if name is None:
            monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT", raising=False)
        else:
            monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", name)
        out[name] = kt.tril_inv(Ad, cud, algo="fused")
        torch.cuda.synchronize()
    assert torch.equal(out["wave"], out["heads4"])
    assert torch.equal(out[None], out["heads4"])
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(out[None].cpu().numpy().astype(np.float64), ref, "f32") <= 0


# (seed, requests, longest request, heads): from a few chunk-heads to several
# rounds of the GPU, so that the automatic choice lands on each form: the column
# kernel with one and with two chunk-heads per workgroup, the one-wavefront
# kernel in one round, walking with few heads, and the 4-head kernel; many
# tiny requests, whose chunks ceil(T / 64) undercounts, stay off the column
# kernel
SHAPES = [(0, 12, 400, 5), (1, 9, 130, 32), (2, 30, 250, 16), (3, 150, 800, 5),
          (4, 70, 600, 16), (5, 3, 300, 1), (6, 200, 3, 64)]  # the last: many tiny requests


@pytest.mark.parametrize("seed,requests,longest,H", SHAPES)
def test_random_shapes_every_form_agrees(kt, monkeypatch, seed, requests, longest, H):
    """Random request lengths: X bit for bit the same under the automatic
    choice and under every forced form, and within tolerance of the oracle."""
    rng = np.random.default_rng(700 + seed)
    lengths = [int(x) for x in rng.integers(1, longest + 1, requests)]
    print(f"\n[cols] random seed={seed} requests={requests} tokens={sum(lengths)} H={H}", flush=True)
    A = synth.delta_rule_A(lengths, H, seed=710 + seed, upper="nan")
    cu = synth.cu_seqlens(lengths)
    Ad = torch.from_numpy(A).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    out = {}
    for name in (None, "wave", "heads4", "cols2", "cols2p", "cols4"):
        if name is None:
            monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT", raising=False)
        else:
            monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", name)
        out[name] = kt.tril_inv(Ad, cud, algo="fused")
        torch.cuda.synchronize()
    monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT", raising=False)
    for name, X in out.items():
        assert torch.equal(X, out["heads4"]), name
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(out[None].cpu().numpy().astype(np.float64), ref, "f32") <= 0
    # the VALU merge on the same launch rules (its own products' order)
    Xv = kt.tril_inv(Ad, cud, algo="fused_valu")
    assert gh.excess(Xv.cpu().numpy().astype(np.float64), ref, "f32") <= 0


@pytest.mark.parametrize("name", ["packed_1x64_h64_f32", "dense_b4_t512_h16_bf16_f32"])
def test_repeats_bitwise(kt, name):
    """100 back-to-back calls of the small workloads (column kernel with one
    and with two chunk-heads per workgroup under the automatic choice): every
    result equals the first bit for bit."""
    d = synth.make(name)
    A = gh.to_torch_input(d["A"], d["a_dtype"], DEV)
    xt = gh.out_torch_dtype(d["x_dtype"])
    if d["layout"] == "dense":
        A = A.view(d["B"], d["T"], d["H"], 64)
        X0 = kt.tril_inv(A, out_dtype=xt)
        run = lambda: kt.tril_inv(A, out_dtype=xt)  # noqa: E731
    else:
        cu = torch.from_numpy(d["cu_seqlens"]).to(DEV)
        X0 = kt.tril_inv(A, cu, out_dtype=xt)
        run = lambda: kt.tril_inv(A, cu, out_dtype=xt)  # noqa: E731
    outs = [run() for _ in range(100)]
    torch.cuda.synchronize()
    for i, X in enumerate(outs):
        assert torch.equal(X, X0), f"repeat {i}"


def test_short_chunks_dense_and_chunk_map(kt, monkeypatch):
    """Short chunks that the chunk count cannot reveal: a caller chunk map of
    many short requests, and a dense batch of 100 rows of 10 tokens (the
    automatic choice walks them with the row-per-lane kernel): X bit for bit
    that of the 4-head kernel, and within tolerance of the oracle."""
    H = 64
    rng = np.random.default_rng(660)
    lengths = [int(x) for x in rng.integers(1, 12, 150)]
    A = synth.delta_rule_A(lengths, H, seed=661)
    cu = synth.cu_seqlens(lengths)
    Ad = torch.from_numpy(A).to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    cmap = torch.from_numpy(gh.host_chunk_map(lengths)).to(DEV)
    B, T = 100, 10
    Adn = torch.from_numpy(synth.delta_rule_A([T] * B, H, seed=662)).to(DEV)
    out = {}
    for name in (None, "heads4"):
        if name is None:
            monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT", raising=False)
        else:
            monkeypatch.setenv("KDA_TRIL_FUSED_LAYOUT", name)
        out[name] = (kt.tril_inv(Ad, cud, chunk_indices=cmap, algo="fused"),
                     kt.tril_inv(Adn.view(B, T, H, 64), algo="fused"))
        torch.cuda.synchronize()
    monkeypatch.delenv("KDA_TRIL_FUSED_LAYOUT", raising=False)
    assert torch.equal(out[None][0], out["heads4"][0])
    assert torch.equal(out[None][1], out["heads4"][1])
    ref = oracle.tril_inv_packed(A, cu)
    assert gh.excess(out[None][0].cpu().numpy().astype(np.float64), ref, "f32") <= 0
    refn = oracle.tril_inv_packed(Adn.cpu().numpy(), synth.cu_seqlens([T] * B))
    assert gh.excess(out[None][1].view(B * T, H, 64).cpu().numpy().astype(np.float64), refn,
                     "f32") <= 0
