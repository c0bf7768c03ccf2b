"""Malformed device-side chunk descriptions.

The C ABI does not validate cu_seqlens or a chunk map on the device, since
that would need a synchronisation. Instead the kernels clamp every chunk to
rows [0, T) of A and X: a chunk that starts outside them is skipped, and its
end is cut at T. Each case checks three things:
- nothing past row T is written (canary rows);
- nothing past row T is read (NaN rows there);
- the chunks that remain hold the oracle's result for the clamped request bounds.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_helpers as gh

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
H = 3
PAD = 16  # rows past T: NaN in the inputs, a canary in the output
CANARY = -777.0
# (cu_seqlens as passed, the well-formed bounds the kernels clamp it to)
CASES = {
    "end_past_T": ([0, 64, 200], [0, 64, 100]),
    "request_wholly_past_T": ([0, 64, 100, 300], [0, 64, 100, 100]),
    # request 0 claims rows -40..63: its first chunk would start at -40 and
    # is skipped; its second starts at 24 and holds rows 24..63
    "negative_start": ([-40, 64, 100], [24, 64, 100]),
}


@pytest.fixture(scope="module")
def kt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tril_solve_amd
    return tril_solve_amd


def _padded(a, fill=np.nan):
    pad = np.full((PAD,) + a.shape[1:], fill, a.dtype)
    return np.concatenate([a, pad])


def _reference(A, clamped):
    """Oracle X for well-formed request bounds (NaN on rows no chunk covers);
    the chunk size is A.shape[-1]."""
    ref = np.full(A.shape, np.nan)
    for s, e in zip(clamped[:-1], clamped[1:]):
        if s < e:
            ref[s:e] = oracle.tril_inv_packed(A[s:e], [0, e - s])
    return ref


def _check(X_full, T, ref):
    X = X_full.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY), "a row past T was written"
    rows = ~np.isnan(ref[:, 0, 0])
    assert gh.excess(X[:T][rows], ref[rows], "f32") <= 0


@pytest.mark.parametrize("algo", ["fused", "split", "fused_valu"])
@pytest.mark.parametrize("case", list(CASES))
def test_cu_seqlens_clamped_64(kt, case, algo):
    cu, clamped = CASES[case]
    print(f"\n[malformed] C=64 {case} {algo}", flush=True)
    A = synth.delta_rule_A([64, 36], H, seed=140)
    T = A.shape[0]
    Ad = torch.from_numpy(_padded(A)).to(DEV)
    X_full = torch.full((T + PAD, H, 64), CANARY, device=DEV)
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)
    kt.tril_inv(Ad[:T], cud, algo=algo, out=X_full[:T])
    torch.cuda.synchronize()
    _check(X_full, T, _reference(A, clamped))


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("case", ["end_past_T", "request_wholly_past_T"])
def test_cu_seqlens_clamped_small_chunks(kt, case, C):
    cu, clamped = CASES[case]
    print(f"\n[malformed] C={C} {case}", flush=True)
    A = synth.delta_rule_A([64, 36], H, seed=141, chunk=C)
    T = A.shape[0]
    Ad = torch.from_numpy(_padded(A)).to(DEV)
    X_full = torch.full((T + PAD, H, C), CANARY, device=DEV)
    kt.tril_inv(Ad[:T], torch.tensor(cu, dtype=torch.int32, device=DEV), out=X_full[:T])
    torch.cuda.synchronize()
    _check(X_full, T, _reference(A, clamped))


def test_chunk_map_entries_out_of_range_skipped(kt):
    """A caller-supplied chunk map with requests and chunk numbers out of
    range: those entries are skipped, the valid ones solved."""
    A = synth.delta_rule_A([64, 36], H, seed=142)
    T = A.shape[0]
    Ad = torch.from_numpy(_padded(A)).to(DEV)
    X_full = torch.full((T + PAD, H, 64), CANARY, device=DEV)
    cmap = torch.tensor([[0, 0], [5, 0], [-1, 0], [1, 0], [0, -3], [1, 7]], dtype=torch.int32,
                        device=DEV)
    cud = torch.tensor([0, 64, 100], dtype=torch.int32, device=DEV)
    kt.tril_inv(Ad[:T], cud, chunk_indices=cmap, out=X_full[:T])
    torch.cuda.synchronize()
    _check(X_full, T, _reference(A, [0, 64, 100]))


def test_kkt_cu_seqlens_clamped(kt):
    """The path that builds A from keys clamps the same way."""
    lengths = [64, 36]
    k, g, beta = synth.delta_rule_inputs(lengths, H, 143, K=64)
    T = k.shape[0]
    kd, gd, bd = (torch.from_numpy(_padded(a)).to(DEV) for a in (k, g, beta))
    X_full = torch.full((T + PAD, H, 64), CANARY, device=DEV)
    cud = torch.tensor([0, 64, 200], dtype=torch.int32, device=DEV)
    kt.kda_kkt_tril_inv(kd[:T], gd[:T], bd[:T], X_full[:T], cud)
    torch.cuda.synchronize()
    ref = oracle.kkt_tril_inv_packed(k, g, beta, [0, 64, 100])
    X = X_full.cpu().numpy().astype(np.float64)
    assert np.all(X[T:] == CANARY)
    assert gh.excess(X[:T], ref, "f32") <= 0
