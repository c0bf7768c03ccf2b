"""The oracle pinned to facts that do not come from itself (CPU only).

Pins: exact rational Neumann series, the single-subdiagonal closed form, a
hand-derived 4x4 example, LAPACK's inverse, the residual of (I + A) X = I,
the leading-block property of partial chunks, hand-derived chunk maps and
bfloat16 rounding tables, torch's bfloat16 cast. The last test plants
plausible mistakes in copies of the oracle's C source and checks that these
pins reject every one of them.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import pins


def _inv(M):
    return oracle.inv_unit_lower(M)


@pytest.mark.parametrize("name,fn", pins.ALL_INV_CHECKS, ids=[n for n, _ in pins.ALL_INV_CHECKS])
def test_inverse_pins(name, fn):
    assert fn(_inv) is None


@pytest.mark.parametrize("seed", range(4))
def test_neumann_integer_more_seeds(seed):
    assert pins.check_neumann_integer(_inv, n=16, seed=seed + 10) is None
    assert pins.check_neumann_integer(_inv, n=5, seed=seed + 20, density=1.0) is None


def test_delta_rule_matrices_against_lapack():
    """Workload-shaped matrices (the generator's) against LAPACK."""
    import synth
    A = synth.delta_rule_A([64, 37], H=4, seed=7)
    for s, L in ((0, 64), (64, 37)):
        for h in range(4):
            M = A[s:s + L, h, :L].astype(np.float64)
            ref = np.linalg.inv(np.eye(L) + np.tril(M, -1))
            X = oracle.inv_unit_lower(M)
            assert np.abs(X[:, :L] - ref).max() < 1e-13


def test_chunk_map_golden():
    for cu, want in pins.read_chunk_maps():
        got = [tuple(r) for r in oracle.chunks_packed(cu).tolist()]
        assert got == want, cu


def test_chunk_map_rejects_decreasing():
    with pytest.raises(ValueError):
        oracle.chunks_packed([0, 10, 5])


def _packed_case(seed=3, H=3):
    cu = [0, 64, 130, 130, 131, 300]
    T = cu[-1]
    rng = np.random.default_rng(seed)
    A = rng.uniform(-0.5, 0.5, (T, H, 64)).astype(np.float32)
    return cu, A


def test_packed_driver_against_lapack_per_chunk():
    """The packed driver solves every (chunk, head) of the hand-derived chunk
    map; each equals LAPACK on that chunk's strictly-lower L x L block, and
    entries on/above the diagonal (random here) are ignored."""
    cu, A = _packed_case()
    X = oracle.tril_inv_packed(A, cu)
    want = [w for c, w in pins.read_chunk_maps() if c == [0, 64, 130, 130, 131]][0]
    want = want + [(4, 131, 64), (4, 195, 64), (4, 259, 41)]
    assert [tuple(r) for r in oracle.chunks_packed(cu).tolist()] == want
    for _, s, L in want:
        for h in range(A.shape[1]):
            M = np.tril(A[s:s + L, h, :L].astype(np.float64), -1)
            ref = np.linalg.inv(np.eye(L) + M)
            assert np.abs(X[s:s + L, h, :L] - ref).max() < 1e-12
            assert np.all(X[s:s + L, h, L:] == 0)


def test_packed_rows_outside_chunks_untouched():
    cu = [0, 10]
    A = np.zeros((16, 2, 64), np.float32)
    X = oracle.tril_inv_packed(A, cu, fill=-7.0)
    assert np.all(X[10:] == -7.0)
    assert np.array_equal(X[:10, 0, :10], np.eye(10))


def test_dense_driver_against_lapack():
    rng = np.random.default_rng(5)
    B, T, H = 2, 150, 2
    A = rng.uniform(-0.5, 0.5, (B, T, H, 64)).astype(np.float32)
    X = oracle.tril_inv_dense(A)
    for b in range(B):
        for c0 in range(0, T, 64):
            L = min(64, T - c0)
            for h in range(H):
                M = np.tril(A[b, c0:c0 + L, h, :L].astype(np.float64), -1)
                ref = np.linalg.inv(np.eye(L) + M)
                assert np.abs(X[b, c0:c0 + L, h, :L] - ref).max() < 1e-12
                assert np.all(X[b, c0:c0 + L, h, L:] == 0)


def test_dense_equals_packed_with_equal_lengths():
    rng = np.random.default_rng(6)
    B, T, H = 3, 100, 2
    A = rng.uniform(-0.5, 0.5, (B, T, H, 64)).astype(np.float32)
    Xd = oracle.tril_inv_dense(A)
    Xp = oracle.tril_inv_packed(A.reshape(B * T, H, 64), [0, 100, 200, 300])
    assert np.array_equal(Xd.reshape(B * T, H, 64), Xp)


def test_bf16_upcast_is_exact():
    bits = np.array([0x3F80, 0xBF82, 0x0001, 0x7F7F], np.uint16)
    got = oracle.to_f64(bits, "bf16")
    want = np.array([1.0, -(1 + 2 / 128), 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127])
    assert np.array_equal(got, want)


def test_rne_golden():
    table = pins.read_rne_table()
    f = np.array([a for a, _ in table], np.uint32).view(np.float32)
    got = oracle.rne_bf16(f)
    assert [int(v) for v in got] == [b for _, b in table]


def test_f16_rne_golden():
    rows = []
    for line in open(os.path.join(pins.GOLDEN, "f16_rne.txt")):
        t = line.split("#")[0].split()
        if len(t) >= 2:
            rows.append((int(t[0], 16), int(t[1], 16)))
    f = np.array([a for a, _ in rows], np.uint32).view(np.float32)
    with np.errstate(over="ignore"):
        got = oracle.rne_f16(f)
    assert [int(v) for v in got] == [b for _, b in rows]


def test_f16_upcast_is_exact():
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0x0400], np.uint16)
    got = oracle.to_f64(bits, "f16")
    assert np.array_equal(got, np.array([1.0, -2.0, 2.0 ** -24, 65504.0, 2.0 ** -14]))


def test_rne_matches_torch_cast():
    import torch
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(
        -30, 30, 200000).astype(np.float32)
    # add exact ties and neighbours
    ties = (rng.integers(0, 2**31, 5000, dtype=np.int64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.rne_bf16(x), want)


# ---- planted mistakes: each must be rejected by the pins above ----------------

_MUTANTS = {
    "drop_first_term": ("for (int j = c; j < i; ++j) s +=", "for (int j = c + 1; j < i; ++j) s +="),
    "wrong_sign": ("col[i] = -s;", "col[i] = s;"),
    "transposed": ("s += M[(int64_t)i * ldm + j] * col[j];", "s += M[(int64_t)j * ldm + i] * col[j];"),
    "reads_diagonal": ("for (int j = c; j < i; ++j) s +=", "for (int j = c; j <= i; ++j) s +="),
    "global_chunk_alignment": ("for (int64_t p = bos; p < eos; p += C)",
                               "for (int64_t p = bos - bos % C; p < eos; p += C)"),
    "ties_away": ("(rest == 0x8000u && (kept & 1u))", "(rest == 0x8000u)"),
    "dense_row0": ("int64_t row0 = b * T + c * C;",
                   "int64_t row0 = (b * per_b + c) * C;"),
    # the delta-rule matrix A built from keys, decays and write strengths
    "kkt_exp_sign": ("exp(g[(int64_t)i * rs_kg + d] - g[(int64_t)j * rs_kg + d])",
                     "exp(g[(int64_t)j * rs_kg + d] - g[(int64_t)i * rs_kg + d])"),
    "kkt_beta_of_column": ("-beta[(int64_t)i * rs_b] * s", "-beta[(int64_t)j * rs_b] * s"),
    "kkt_keeps_diagonal": ("for (int j = 0; j < i; ++j) {\n            double s = 0.0;",
                           "for (int j = 0; j <= i; ++j) {\n            double s = 0.0;"),
    "kkt_drops_last_channel": ("for (int d = 0; d < K; ++d)", "for (int d = 0; d < K - 1; ++d)"),
    # the decode step
    "dec_conv_window_reversed": ("* st[(int64_t)w * d + c];", "* st[(int64_t)(W - 2 - w) * d + c];"),
    "dec_no_silu": ("y[p][c] = acc / (1.0 + exp(-acc));", "y[p][c] = acc;"),
    "dec_no_beta": ("u[j] = bt * (y[2][j] - r);", "u[j] = (y[2][j] - r);"),
    "dec_decay_sign": ("const double a = exp(gg[i]);", "const double a = exp(-gg[i]);"),
    "dec_silu_gate": ("wn[j] / (1.0 + exp(-zz[j]));", "wn[j] * zz[j] / (1.0 + exp(-zz[j]));"),
    "dec_padding_output": ("for (int j = 0; j < d; ++j) o_out[j] = 0.0;",
                           "for (int j = 0; j < d; ++j) o_out[j] = 1.0;"),
    "dec_no_q_scale": ("/ sqrt(nq + eps_l2) / sqrt((double)d);", "/ sqrt(nq + eps_l2);"),
    "dec_q_eps_outside": ("1.0 / sqrt(nq + eps_l2) / sqrt((double)d);",
                          "1.0 / (sqrt(nq) + eps_l2) / sqrt((double)d);"),
    "dec_k_no_eps": ("const double sk = 1.0 / sqrt(nk + eps_l2);",
                     "const double sk = 1.0 / sqrt(nk);"),
    "dec_q_scale_d_not_sqrt": ("/ sqrt(nq + eps_l2) / sqrt((double)d);",
                               "/ sqrt(nq + eps_l2) / (double)d;"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "tril_oracle.c")).read()
    old, new = _MUTANTS[name]
    assert src.count(old) >= 1, name
    src = src.replace(old, new)
    if name == "reads_diagonal":  # j <= i would read col[i], so make it defined
        src = src.replace("col[c] = 1.0;", "col[c] = 1.0;\n        for (int i = c + 1; i < 64; ++i) col[i] = 0.0;")
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    return _load_lib(c, so)


def _load_lib(c, so):
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o",
                           str(so), str(c), "-lm"])
    lib = ctypes.CDLL(str(so))
    p, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.oracle_inv_unit_lower.argtypes = [p, i64, ci, p, i64]
    lib.oracle_chunks_packed.argtypes = [p, i64, p, p, p, i64]
    lib.oracle_chunks_packed.restype = i64
    lib.oracle_rne_bf16.argtypes = [p, p, i64]
    lib.oracle_tril_inv_dense.argtypes = [p, p, i64, i64, i32, ci]
    lib.oracle_tril_inv_dense.restype = i64
    lib.oracle_kkt_packed.argtypes = [p, p, p, p, p, i64, i64, i32, ci, ci]
    lib.oracle_kkt_packed.restype = i64
    lib.oracle_kda_decode.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i32, ci, ci,
                                      ctypes.c_double, ctypes.c_double]
    lib.oracle_kda_decode.restype = ci
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _pins_fail(lib):
    """True when at least one pin rejects this compiled variant."""
    def inv(M):
        M = np.ascontiguousarray(M, np.float64)
        L = M.shape[0]
        X = np.zeros((L, 64))
        lib.oracle_inv_unit_lower(_ptr(M), M.shape[1], L, _ptr(X), 64)
        return X

    if pins.run_all(inv):
        return True
    for cu, want in pins.read_chunk_maps():
        cu = np.array(cu, np.int32)
        n = lib.oracle_chunks_packed(_ptr(cu), len(cu) - 1, None, None, None, 0)
        if n != len(want):
            return True
        seq, st, ln = np.zeros(n, np.int64), np.zeros(n, np.int64), np.zeros(n, np.int32)
        lib.oracle_chunks_packed(_ptr(cu), len(cu) - 1, _ptr(seq), _ptr(st), _ptr(ln), n)
        if list(zip(seq.tolist(), st.tolist(), ln.tolist())) != want:
            return True
    table = pins.read_rne_table()
    bits = np.array([a for a, _ in table], np.uint32)
    out = np.zeros(len(bits), np.uint16)
    lib.oracle_rne_bf16(_ptr(bits), _ptr(out), len(bits))
    if out.tolist() != [b for _, b in table]:
        return True
    # dense driver on a partial-chunk shape, against LAPACK per matrix
    rng = np.random.default_rng(5)
    B, T, H = 2, 150, 2
    # room past the end so a mutant that indexes rows wrongly stays in bounds
    Abuf = rng.uniform(-0.5, 0.5, (B * T + 4 * 64, H, 64))
    Xbuf = np.full_like(Abuf, np.nan)
    lib.oracle_tril_inv_dense(_ptr(Abuf), _ptr(Xbuf), B, T, H, 1)
    A = Abuf[:B * T].reshape(B, T, H, 64)
    X = Xbuf[:B * T].reshape(B, T, H, 64)
    for b in range(B):
        for c0 in range(0, T, 64):
            L = min(64, T - c0)
            for h in range(H):
                ref = np.linalg.inv(np.eye(L) + np.tril(A[b, c0:c0 + L, h, :L], -1))
                got = X[b, c0:c0 + L, h, :L]
                if not np.all(np.isfinite(got)) or np.abs(got - ref).max() > 1e-12:
                    return True

    def kkt(k, g, beta, cu):
        k, g, beta = (np.ascontiguousarray(a, np.float64) for a in (k, g, beta))
        T, H, K = k.shape
        A = np.full((T, H, 64), np.nan)
        lib.oracle_kkt_packed(_ptr(k), _ptr(g), _ptr(beta), _ptr(A), _ptr(cu), len(cu) - 1, T,
                              H, K, 1)
        return A

    if pins.kkt_all(kkt):
        return True

    def dec(qkv, g, beta, z, wn, cw, slot, S, cs, eps_l2, eps_norm):
        a = [np.ascontiguousarray(t, np.float64) for t in (qkv, g, beta, z, wn, cw)]
        S = np.array(S, np.float64, copy=True)
        cs = np.array(cs, np.float64, copy=True)
        sl = np.ascontiguousarray(slot, np.int32)
        B, _, H, d = a[0].shape
        out = np.zeros((B, H, d))
        lib.oracle_kda_decode(*[_ptr(t) for t in a], _ptr(sl), _ptr(S), _ptr(cs), _ptr(out), B,
                              H, d, a[5].shape[1], eps_l2, eps_norm)
        return out, S, cs

    # the brute force restates the step's formulas, so it does not count as a
    # pin here: every planted mistake must fail a closed-form check
    return bool([n for n in pins.dec_all(dec) if n != "brute_force"])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert _pins_fail(_build_mutant(tmp_path, name)), f"pins accept the mutant {name}"


def test_unpatched_oracle_passes_the_same_gate(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "tril_oracle.c")).read()
    c = tmp_path / "plain.c"
    c.write_text(src)
    assert not _pins_fail(_load_lib(c, tmp_path / "libplain.so"))


# ---- the 16- and 32-token branches -------------------------------------------

def test_chunk_map_golden_16_32():
    for C, cu, want in pins.read_chunk_maps_sized():
        got = [tuple(r) for r in oracle.chunks_packed(cu, C).tolist()]
        assert got == want, (C, cu)


@pytest.mark.parametrize("C", [16, 32])
def test_small_chunk_drivers_against_lapack(C):
    """Packed and dense drivers with C-token chunks: every chunk-head equals
    LAPACK's inverse of its strictly-lower L x L block, columns L..C-1 are 0,
    and entries on/above the diagonal (random here) are ignored."""
    rng = np.random.default_rng(C)
    lengths = [C, C + 5, 1, 3 * C - 1]
    H = 3
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    A = rng.uniform(-0.5, 0.5, (T, H, C)).astype(np.float32)
    X = oracle.tril_inv_packed(A, cu)
    for _, s, L in oracle.chunks_packed(cu, C).tolist():
        for h in range(H):
            M = np.tril(A[s:s + L, h, :L].astype(np.float64), -1)
            ref = np.linalg.inv(np.eye(L) + M)
            assert np.abs(X[s:s + L, h, :L] - ref).max() < 1e-12
            assert np.all(X[s:s + L, h, L:] == 0)
    B, Td = 2, 2 * C + 3
    Ad = rng.uniform(-0.5, 0.5, (B, Td, H, C)).astype(np.float32)
    Xd = oracle.tril_inv_dense(Ad)
    Xp = oracle.tril_inv_packed(Ad.reshape(B * Td, H, C), [0, Td, 2 * Td])
    assert np.array_equal(Xd.reshape(B * Td, H, C), Xp)


def test_small_chunk_is_leading_block_of_64():
    """A 16- or 32-token chunk's inverse is the leading block of the 64-token
    solver's on the same (zero-padded) rows."""
    rng = np.random.default_rng(9)
    M = np.tril(rng.uniform(-0.5, 0.5, (64, 64)), -1)
    full = oracle.inv_unit_lower(M)
    for C in (16, 32):
        X = oracle.inv_unit_lower(M[:C, :C], width=C)
        assert np.array_equal(X, full[:C, :C])


# ---- the delta-rule matrix A (fused "build A, then invert" path) --------------

def _oracle_kkt(k, g, beta, cu):
    return oracle.kkt_packed(k, g, beta, cu, "f64")


def test_kkt_scalar_key_closed_form():
    assert pins.check_kkt_scalar_key(_oracle_kkt)


def test_kkt_uniform_decay_gram():
    assert pins.check_kkt_uniform_decay(_oracle_kkt)


def test_kkt_brute_force():
    assert pins.check_kkt_brute_force(_oracle_kkt)


def test_kkt_dense_equals_packed_and_inverse_composes():
    """Dense driver equals the packed one on the same rows; the fused oracle
    is the inverse (LAPACK) of that float64 A, never rounded in between."""
    rng = np.random.default_rng(7)
    B, T, H, K = 2, 70, 2, 8
    k = rng.standard_normal((B, T, H, K))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)  # unit keys
    g = np.cumsum(-rng.random((B, T, H, K)) * 0.1, axis=1).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    Ad = oracle.kkt_dense(k, g, beta)
    cu = np.array([0, T, 2 * T], np.int32)
    Ap = oracle.kkt_packed(k.reshape(B * T, H, K), g.reshape(B * T, H, K), beta.reshape(B * T, H),
                           cu)
    assert np.array_equal(Ad.reshape(B * T, H, 64), Ap)
    X = oracle.kkt_tril_inv_packed(k.reshape(B * T, H, K), g.reshape(B * T, H, K),
                                   beta.reshape(B * T, H), cu)
    Xd = oracle.kkt_tril_inv_dense(k, g, beta)
    assert np.array_equal(Xd.reshape(B * T, H, 64), X)
    for t0, L in ((0, 64), (64, 6), (70, 64), (134, 6)):
        for h in range(H):
            M = np.tril(Ap[t0:t0 + L, h, :L], -1)
            ref = np.linalg.inv(np.eye(L) + M)
            assert np.abs(X[t0:t0 + L, h, :L] - ref).max() < 1e-12 * max(1.0, np.abs(ref).max())


# ---- the fused KDA decode step -----------------------------------------------

def _oracle_dec(qkv, g, beta, z, wn, cw, slot, S, cs, eps_l2, eps_norm):
    return oracle.kda_decode(qkv, g, beta, z, wn, cw, slot, S, cs, "f64", eps_l2, eps_norm)


@pytest.mark.parametrize("check", ["check_dec_delta_rule", "check_dec_decay_only",
                                   "check_dec_conv_taps", "check_dec_padding_and_slots",
                                   "check_dec_q_scale", "check_dec_brute_force"])
def test_decode_step_pins(check):
    assert getattr(pins, check)(_oracle_dec)


def test_decode_inputs_are_not_modified():
    rng = np.random.default_rng(3)
    B, H, d, W, slots = 2, 2, 8, 4, 2
    S = rng.standard_normal((slots, H, d, d))
    cs = rng.standard_normal((slots, 3, H, W - 1, d))
    S0, cs0 = S.copy(), cs.copy()
    oracle.kda_decode(rng.standard_normal((B, 3, H, d)), -rng.random((B, H, d)),
                      rng.random((B, H)), rng.standard_normal((B, H, d)), np.ones(d),
                      rng.standard_normal((3, W, H, d)), np.array([1, 0], np.int32), S, cs,
                      "f64")
    assert np.array_equal(S, S0) and np.array_equal(cs, cs0)

