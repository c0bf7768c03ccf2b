"""GPU parity of the fused KDA decode core (kda_decode_step) against the
fp64 oracle.

Bar: output |out - ref| <= 2e-5 (1 + |ref|) for fp32 output (bf16 / f16
outputs add their relative rounding terms); updated state and conv windows
to the same fp32 bound. Padding entries, untouched slots and closed forms are
compared bit for bit.
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


def _dev(inp):
    """Device tensors of one decode input set."""
    dt = inp["in_dtype"]
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(DEV)
         for k in ("g", "beta", "norm_w", "conv_w", "slot", "state", "conv_state")}
    d["qkv"] = gh.to_torch_input(inp["qkv"], dt, DEV)
    d["z"] = gh.to_torch_input(inp["z"], dt, DEV)
    return d


def _step(kt, d, out_dtype="f32", eps_l2=1e-6, eps_norm=1e-6, out=None):
    B, H = d["beta"].shape
    if out is None:
        out = torch.empty((B, H, 128), dtype=gh.out_torch_dtype(out_dtype), device=DEV)
    kt.kda_decode_step(d["qkv"], d["z"], d["g"], d["beta"], d["norm_w"], d["conv_w"], d["slot"],
                       d["state"], d["conv_state"], out, eps_l2, eps_norm)
    torch.cuda.synchronize()
    return out


def _ref(inp, state=None, conv_state=None, eps_l2=1e-6, eps_norm=1e-6):
    return oracle.kda_decode(inp["qkv"], inp["g"], inp["beta"], inp["z"], inp["norm_w"],
                             inp["conv_w"], inp["slot"],
                             inp["state"] if state is None else state,
                             inp["conv_state"] if conv_state is None else conv_state,
                             inp["in_dtype"], eps_l2, eps_norm)


def _check(kt, inp, d, out, x_dtype="f32"):
    ref_out, ref_S, ref_cs = _ref(inp)
    e = gh.excess(gh.to_numpy_f64(out), ref_out, x_dtype)
    assert e <= 0, f"output exceeds tolerance by {e:.3g}"
    e = gh.excess(d["state"].cpu().numpy().astype(np.float64), ref_S, "f32")
    assert e <= 0, f"state exceeds tolerance by {e:.3g}"
    e = gh.excess(d["conv_state"].cpu().numpy().astype(np.float64), ref_cs, "f32")
    assert e <= 0, f"conv windows exceed tolerance by {e:.3g}"


@pytest.mark.parametrize("layout", [None, "pairs", "cols"])
@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("B,H", [(1, 1), (3, 4), (8, 2), (96, 3)])
def test_step_parity(kt, monkeypatch, B, H, W, layout):
    """One step against the oracle, under the automatic split of the state
    over the wavefronts and under each forced one (KDA_TRIL_DECODE_LAYOUT)."""
    if layout is not None:
        monkeypatch.setenv("KDA_TRIL_DECODE_LAYOUT", layout)
    print(f"\n[decode] B={B} H={H} W={W} layout={layout}", flush=True)
    inp = synth.decode_inputs(B, H, W=W, seed=100 + B * 10 + H + W)
    d = _dev(inp)
    _check(kt, inp, d, _step(kt, d))


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
def test_dtype_matrix(kt, in_dtype, out_dtype):
    inp = synth.decode_inputs(4, 3, seed=120, in_dtype=in_dtype)
    d = _dev(inp)
    _check(kt, inp, d, _step(kt, d, out_dtype), out_dtype)


def test_padding_and_untouched_slots(kt):
    """Padding entries (slot -1, and a slot past the pool) give exact zeros
    and touch no state; slots no entry names keep their bits."""
    inp = synth.decode_inputs(6, 2, seed=121, padding=2)
    inp["slot"][2] = inp["slots"] + 5  # outside the pool: treated as padding
    d = _dev(inp)
    S0, cs0 = d["state"].clone(), d["conv_state"].clone()
    out = _step(kt, d)
    assert bool((out[:3] == 0).all())
    used = set(int(s) for s in inp["slot"][3:])
    for s in range(inp["slots"]):
        same = torch.equal(d["state"][s], S0[s]) and torch.equal(d["conv_state"][s], cs0[s])
        assert same == (s not in used), s
    inp["slot"][2] = -1  # the oracle's view: padding
    _check(kt, inp, d, out)


def test_delta_rule_closed_form(kt):
    """Zero state, g = 0, beta = 1, q = k and taps that pass the new input:
    the step stores k v^T and outputs RMSNorm(silu(v)) * w * sigmoid(z)."""
    B, H = 2, 3
    inp = synth.decode_inputs(B, H, seed=122)
    inp["qkv"][:, 0] = inp["qkv"][:, 1]
    inp["g"][:] = 0.0
    inp["beta"][:] = 1.0
    inp["state"][:] = 0.0
    inp["conv_w"][:] = 0.0
    inp["conv_w"][:, -1] = 1.0
    d = _dev(inp)
    out = gh.to_numpy_f64(_step(kt, d, eps_l2=0.0, eps_norm=0.0))
    v = inp["qkv"][:, 2].astype(np.float64)
    yv = v / (1.0 + np.exp(-v))
    want = (yv / np.sqrt(np.mean(yv ** 2, axis=-1, keepdims=True)) * inp["norm_w"] /
            (1.0 + np.exp(-inp["z"].astype(np.float64))))
    assert gh.excess(out, want, "f32") <= 0
    yk = inp["qkv"][:, 1].astype(np.float64)
    yk = yk / (1.0 + np.exp(-yk))
    k = yk / np.linalg.norm(yk, axis=-1, keepdims=True)
    S = d["state"].cpu().numpy().astype(np.float64)
    for b in range(B):
        want_S = np.einsum("hi,hj->hij", k[b], yv[b])
        assert gh.excess(S[inp["slot"][b]], want_S, "f32") <= 0


def _check_eps(kt, inp, d, out, eps_l2, eps_norm):
    ref_out, ref_S, ref_cs = _ref(inp, eps_l2=eps_l2, eps_norm=eps_norm)
    e = gh.excess(gh.to_numpy_f64(out), ref_out, "f32")
    assert e <= 0, f"output exceeds tolerance by {e:.3g}"
    e = gh.excess(d["state"].cpu().numpy().astype(np.float64), ref_S, "f32")
    assert e <= 0, f"state exceeds tolerance by {e:.3g}"


@pytest.mark.parametrize("eps_l2,eps_norm", [(0.5, 1.0), (0.0, 1.0), (2.0, 0.25)])
def test_large_eps_keeps_q_scale(kt, eps_l2, eps_norm):
    """eps_norm comparable to or above mean(o^2): the gated RMSNorm no longer
    cancels the scale of q, so the 1/sqrt(d) and where eps_l2 enters both
    reach the output (random inputs against the oracle)."""
    inp = synth.decode_inputs(5, 3, seed=126)
    d = _dev(inp)
    out = _step(kt, d, eps_l2=eps_l2, eps_norm=eps_norm)
    _check_eps(kt, inp, d, out, eps_l2, eps_norm)


def test_q_scale_closed_form(kt):
    """Zero state, g = 0, beta = 1, pass-through taps, q and k one-hot in one
    channel before their normalisation, eps_l2 = 0.5, eps_norm = 1: the
    output is (k_m q_m) v / sqrt((k_m q_m)^2 mean(v^2) + 1) * w * sigmoid(z)
    with q_m = silu(xq) / sqrt(silu(xq)^2 + 0.5) / sqrt(128) and
    k_m = silu(xk) / sqrt(silu(xk)^2 + 0.5), worked out here in float64."""
    B, H, eps_l2 = 2, 3, 0.5
    inp = synth.decode_inputs(B, H, seed=127)
    inp["qkv"][:, :2] = 0.0
    m = np.array([[5, 64, 127], [0, 33, 90]])
    xq = np.array([[1.5, -0.5, 2.5], [0.25, 3.0, -1.0]], np.float32)
    xk = np.array([[-2.0, 1.0, 0.5], [1.75, -0.75, 2.0]], np.float32)
    for b in range(B):
        for h in range(H):
            inp["qkv"][b, 0, h, m[b, h]] = xq[b, h]
            inp["qkv"][b, 1, h, m[b, h]] = xk[b, h]
    inp["g"][:] = 0.0
    inp["beta"][:] = 1.0
    inp["state"][:] = 0.0
    inp["conv_w"][:] = 0.0
    inp["conv_w"][:, -1] = 1.0
    d = _dev(inp)
    out = gh.to_numpy_f64(_step(kt, d, eps_l2=eps_l2, eps_norm=1.0))
    silu = lambda x: x / (1.0 + np.exp(-x))  # noqa: E731
    a, bb = silu(xq.astype(np.float64)), silu(xk.astype(np.float64))
    kq = (bb / np.sqrt(bb * bb + eps_l2)) * (a / np.sqrt(a * a + eps_l2) / np.sqrt(128.0))
    v = silu(inp["qkv"][:, 2].astype(np.float64))
    o = kq[:, :, None] * v
    want = (o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + 1.0) * inp["norm_w"] /
            (1.0 + np.exp(-inp["z"].astype(np.float64))))
    assert gh.excess(out, want, "f32") <= 0


def test_eight_steps_carry_state(kt):
    """Eight consecutive steps on the same slots, state kept on the device,
    against the oracle carrying its float64 state."""
    B, H = 4, 2
    base = synth.decode_inputs(B, H, seed=123)
    d = _dev(base)
    S_ref, cs_ref = base["state"].astype(np.float64), base["conv_state"].astype(np.float64)
    for step in range(8):
        inp = synth.decode_inputs(B, H, seed=200 + step)
        inp["slot"] = base["slot"]
        for k in ("qkv", "z", "g", "beta"):
            d[k].copy_(torch.from_numpy(inp[k]).to(DEV))
        for k in ("norm_w", "conv_w"):
            inp[k] = base[k]
        out = _step(kt, d)
        ref_out, S_ref, cs_ref = _ref(inp, S_ref, cs_ref)
        e = gh.excess(gh.to_numpy_f64(out), ref_out, "f32")
        assert e <= 0, f"step {step}: output exceeds tolerance by {e:.3g}"
    e = gh.excess(d["state"].cpu().numpy().astype(np.float64), S_ref, "f32")
    assert e <= 0, f"state after 8 steps exceeds tolerance by {e:.3g}"


def test_graph_capture_replay(kt):
    """A captured decode step replays correctly several times with eager
    work in between; each replay advances the state like an eager call."""
    inp = synth.decode_inputs(3, 2, seed=124)
    d = _dev(inp)
    twin = {k: v.clone() for k, v in d.items()}
    out = torch.empty((3, 2, 128), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the graph (advances d's state once)
        kt.kda_decode_step(d["qkv"], d["z"], d["g"], d["beta"], d["norm_w"], d["conv_w"],
                           d["slot"], d["state"], d["conv_state"], out)
    side.synchronize()
    _step(kt, twin)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kt.kda_decode_step(d["qkv"], d["z"], d["g"], d["beta"], d["norm_w"], d["conv_w"],
                           d["slot"], d["state"], d["conv_state"], out)
    # capture does not run the step; replay it and an eager step on the twin
    for rep in range(3):
        out.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = _step(kt, twin)
        assert torch.equal(out, eager), f"replay {rep}"
        assert torch.equal(d["state"], twin["state"])
        assert torch.equal(d["conv_state"], twin["conv_state"])


@pytest.mark.parametrize("B", [8, 32])
def test_bench_launch_configuration(kt, B):
    """Prepared calls over rotating state pools (one per layer), back to
    back with no synchronisation, as the benchmark times them (B = 32 is the
    benchmark's largest batch)."""
    print(f"\n[decode] bench configuration B={B}", flush=True)
    sets = [synth.decode_inputs(B, 32, seed=130 + B + i, in_dtype="bf16") for i in range(3)]
    devs = [_dev(s) for s in sets]
    outs = [torch.empty((B, 32, 128), dtype=torch.bfloat16, device=DEV) for _ in sets]
    calls = [kt.prepare_decode(d["qkv"], d["z"], d["g"], d["beta"], d["norm_w"], d["conv_w"],
                               d["slot"], d["state"], d["conv_state"], o)
             for d, o in zip(devs, outs)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    for inp, d, o in zip(sets, devs, outs):
        _check(kt, inp, d, o, "bf16")


def test_slots_past_4gib_of_state(kt):
    """A state pool of 2100 slots x 32 heads (4.4 GB): slots near its end,
    whose byte offsets need more than 32 bits, against the oracle on a
    compact pool of the used slots; a slot no entry names keeps its bits."""
    B, H, n_slots = 4, 32, 2100
    print(f"\n[decode] pool of {n_slots} slots x {H} heads", flush=True)
    inp = synth.decode_inputs(B, H, seed=125, slots=B)  # compact pool: slots 0..B-1
    where = np.array([2099, 2050, 1, 2098])  # compact slot c lives in pool slot where[c]
    d = _dev(inp)
    S = torch.zeros((n_slots, H, 128, 128), device=DEV)
    cs = torch.zeros((n_slots, 3, H, 3, 128), device=DEV)
    for c in range(B):
        S[where[c]] = d["state"][c]
        cs[where[c]] = d["conv_state"][c]
    S[2000] = 7.0
    d["state"], d["conv_state"] = S, cs
    d["slot"] = torch.from_numpy(where[inp["slot"]].astype(np.int32)).to(DEV)
    out = _step(kt, d)
    ref_out, ref_S, ref_cs = _ref(inp)
    assert gh.excess(gh.to_numpy_f64(out), ref_out, "f32") <= 0
    idx = torch.from_numpy(where).to(DEV)
    e = gh.excess(S[idx].cpu().numpy().astype(np.float64), ref_S, "f32")
    assert e <= 0, f"state exceeds tolerance by {e:.3g}"
    e = gh.excess(cs[idx].cpu().numpy().astype(np.float64), ref_cs, "f32")
    assert e <= 0, f"conv windows exceed tolerance by {e:.3g}"
    assert bool((S[2000] == 7.0).all())


@pytest.mark.parametrize("layout", ["pairs", "cols"])
def test_repeats_bitwise(kt, monkeypatch, layout):
    """50 steps from the same state pools and inputs, under each split of the
    state over the wavefronts: every output, state and conv window equals the
    first run's bit for bit (the row sums of the row-pair split meet in a
    fixed order)."""
    monkeypatch.setenv("KDA_TRIL_DECODE_LAYOUT", layout)
    inp = synth.decode_inputs(8, 32, seed=131)
    d = _dev(inp)
    S0, C0 = d["state"].clone(), d["conv_state"].clone()
    first = None
    for rep in range(50):
        d["state"].copy_(S0)
        d["conv_state"].copy_(C0)
        out = _step(kt, d)
        got = (out.clone(), d["state"].clone(), d["conv_state"].clone())
        if first is None:
            first = got
            _check(kt, inp, d, out)
        else:
            for a, b in zip(got, first):
                assert torch.equal(a, b), f"repeat {rep}"
