"""Pins of the oracle's matrix inverse against facts that do not come from the
oracle itself. Each check takes ``inv(M) -> X``: the (I + M)^-1 of one
L x L matrix (only the strictly-lower part of M is meaningful), returned as
L rows of 64 columns. The same checks run on the real oracle and on copies of
it with a planted mistake, which they must reject.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def neumann_exact(M):
    """X = sum_{k<n} (-M)^k in exact rationals (M strictly lower, so M^n = 0)."""
    n = len(M)
    F = [[Fraction(M[i][j]) if j < i else Fraction(0) for j in range(n)] for i in range(n)]
    X = [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]
    P = [row[:] for row in X]  # (-M)^k
    for _ in range(1, n):
        P = [[-sum(P[i][m] * F[m][j] for m in range(n) if F[m][j] != 0 and P[i][m] != 0)
              for j in range(n)] for i in range(n)]
        for i in range(n):
            for j in range(n):
                X[i][j] += P[i][j]
    return X


def check_neumann_integer(inv, n=12, seed=0, density=0.6):
    """Small integer matrices: every intermediate of a correct substitution is
    an integer below 2^53, so the fp64 result must equal the exact series."""
    rng = np.random.default_rng(seed)
    M = np.tril(rng.integers(-2, 3, (n, n)), -1) * (rng.random((n, n)) < density)
    M = M.astype(np.float64)
    ex = neumann_exact(M.astype(np.int64).tolist())
    X = inv(M)
    for i in range(n):
        for j in range(n):
            if X[i, j] != float(ex[i][j]):
                return f"neumann mismatch at ({i},{j}): {X[i, j]} vs {ex[i][j]}"
        for j in range(n, 64):
            if X[i, j] != 0.0:
                return f"column {j} >= L not zero in row {i}"
    return None


def check_neumann_sparse64(inv, seed=0):
    """Sparse 64 x 64 dyadic matrix (entries +-1/2, +-1): exact series."""
    rng = np.random.default_rng(seed)
    n = 64
    vals = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0]), (n, n))
    M = np.tril(vals * (rng.random((n, n)) < 0.04), -1)
    ex = neumann_exact([[Fraction(v) for v in row] for row in M.tolist()])
    X = inv(M)
    for i in range(n):
        for j in range(n):
            if Fraction(X[i, j]) != ex[i][j]:
                return f"sparse64 mismatch at ({i},{j})"
    return None


def check_subdiagonal(inv, c, n=64):
    """Single subdiagonal M[i, i-1] = c: X[i, j] = (-c)^(i-j) for i >= j."""
    M = np.zeros((n, n))
    for i in range(1, n):
        M[i, i - 1] = c
    X = inv(M)
    want = np.zeros((n, 64))
    for i in range(n):
        for j in range(i + 1):
            want[i, j] = (-c) ** (i - j)
    exact = float(c) in (1.0, -1.0, 0.5, -0.5, 2.0, -2.0)
    if exact:
        if not np.array_equal(X, want):
            return f"subdiagonal c={c}: not bitwise (-c)^(i-j)"
    elif not np.allclose(X, want, rtol=1e-13, atol=0):
        return f"subdiagonal c={c}: off the closed form"
    return None


def check_worked_4x4(inv):
    """Hand-derived 4x4 example in tests/golden/worked_4x4.txt."""
    A, X = [], []
    cur = None
    with open(os.path.join(GOLDEN, "worked_4x4.txt")) as f:
        for line in f:
            s = line.strip()
            if not s or s.startswith("#"):
                continue
            if s in ("A", "X"):
                cur = A if s == "A" else X
                continue
            cur.append([float(v) for v in s.split()])
    got = inv(np.array(A))
    if not np.array_equal(got[:, :4], np.array(X)):
        return "worked 4x4 example mismatch"
    return None


def check_lapack(inv, seed=0, n=64, scale=0.5):
    """Against LAPACK's general inverse of I + M (numpy.linalg.inv)."""
    rng = np.random.default_rng(seed)
    M = np.tril(rng.uniform(-scale, scale, (n, n)), -1)
    X = inv(M)[:, :n]
    ref = np.linalg.inv(np.eye(n) + M)
    err = np.abs(X - ref).max() / max(1.0, np.abs(ref).max())
    if err > 1e-12:
        return f"lapack mismatch {err:.3g}"
    return None


def check_residual(inv, seed=0, n=64):
    rng = np.random.default_rng(seed)
    M = np.tril(rng.uniform(-0.5, 0.5, (n, n)), -1)
    X = inv(M)[:, :n]
    r = np.abs((np.eye(n) + M) @ X - np.eye(n)).max()
    if r > 1e-12:
        return f"residual {r:.3g}"
    return None


def check_upper_ignored(inv, seed=0, n=64):
    """Entries on and above the diagonal of M must not enter the result."""
    rng = np.random.default_rng(seed)
    M = np.tril(rng.uniform(-0.5, 0.5, (n, n)), -1)
    G = M.copy()
    iu = np.triu_indices(n)
    G[iu] = rng.uniform(-1e3, 1e3, len(iu[0]))
    if not np.array_equal(inv(M), inv(G)):
        return "upper triangle leaks into the result"
    # non-finite values on and above the diagonal must not leak either
    G[np.diag_indices(n)] = np.nan
    G[0, 1:] = np.inf
    if not np.array_equal(inv(M), inv(G)):
        return "non-finite diagonal/upper entries leak into the result"
    return None


def check_leading_block(inv, seed=0):
    """For L < 64 the result is the leading L x L block of the zero-padded
    64 x 64 inverse, and matches LAPACK on the L x L matrix."""
    rng = np.random.default_rng(seed)
    M = np.tril(rng.uniform(-0.5, 0.5, (64, 64)), -1)
    full = inv(M)
    for L in (1, 2, 15, 16, 17, 31, 33, 63):
        X = inv(M[:L, :L])
        if not np.array_equal(X[:, :L], full[:L, :L]):
            return f"L={L}: not the leading block"
        if np.any(X[:, L:] != 0):
            return f"L={L}: columns >= L not zero"
        ref = np.linalg.inv(np.eye(L) + M[:L, :L])
        if np.abs(X[:, :L] - ref).max() > 1e-12:
            return f"L={L}: lapack mismatch"
    return None


ALL_INV_CHECKS = [
    ("neumann_integer", check_neumann_integer),
    ("neumann_sparse64", check_neumann_sparse64),
    ("subdiag_1", lambda inv: check_subdiagonal(inv, 1.0)),
    ("subdiag_-0.5", lambda inv: check_subdiagonal(inv, -0.5)),
    ("subdiag_2", lambda inv: check_subdiagonal(inv, 2.0, n=40)),
    ("subdiag_0.3", lambda inv: check_subdiagonal(inv, 0.3)),
    ("worked_4x4", check_worked_4x4),
    ("lapack", check_lapack),
    ("residual", check_residual),
    ("upper_ignored", check_upper_ignored),
    ("leading_block", check_leading_block),
]


def run_all(inv):
    """Names of failed checks (empty when every pin holds)."""
    failed = []
    for name, fn in ALL_INV_CHECKS:
        try:
            msg = fn(inv)
        except Exception as e:  # a broken build may also crash a check
            msg = f"raised {e!r}"
        if msg:
            failed.append((name, msg))
    return failed


def read_chunk_maps():
    cases = []
    cu, chunks = None, []
    with open(os.path.join(GOLDEN, "chunk_map.txt")) as f:
        for line in f:
            s = line.split("#")[0].split()
            if not s:
                continue
            if s[0] == "cu":
                cu, chunks = [int(v) for v in s[1:]], []
            elif s[0] == "chunk":
                chunks.append(tuple(int(v) for v in s[1:]))
            elif s[0] == "end":
                cases.append((cu, chunks))
    return cases


def read_rne_table():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            s = line.split("#")[0].split()
            if len(s) >= 2:
                rows.append((int(s[0], 16), int(s[1], 16)))
    return rows


def read_chunk_maps_sized():
    """(C, cu, chunks) cases of tests/golden/chunk_map_16_32.txt."""
    cases = []
    size, cu, chunks = None, None, []
    with open(os.path.join(GOLDEN, "chunk_map_16_32.txt")) as f:
        for line in f:
            s = line.split("#")[0].split()
            if not s:
                continue
            if s[0] == "size":
                size = int(s[1])
            elif s[0] == "cu":
                cu, chunks = [int(v) for v in s[1:]], []
            elif s[0] == "chunk":
                chunks.append(tuple(int(v) for v in s[1:]))
            elif s[0] == "end":
                cases.append((size, cu, chunks))
    return cases



# ---- the delta-rule matrix A built from keys, decays and write strengths ----
#
# Each check takes ``kkt(k, g, beta, cu) -> A``: float64 inputs k, g [T, H, K],
# beta [T, H], int32 cu_seqlens; A [T, H, 64] for 64-token chunks that
# restart at every request's first token. The decays g are float32 values
# (the solver takes them in float32), so the checks draw them as such.

def kkt_brute_force(k, g, beta, cu):
    """A from its definition with Python floats and math.exp, chunk by chunk:
    A[i][j] = -beta_i sum_d k[i][d] k[j][d] exp(g[i][d] - g[j][d]), j < i."""
    import math
    T, H, K = k.shape
    A = np.full((T, H, 64), np.nan)
    for s in range(len(cu) - 1):
        for c0 in range(int(cu[s]), int(cu[s + 1]), 64):
            L = min(64, int(cu[s + 1]) - c0)
            for h in range(H):
                for i in range(L):
                    row = [0.0] * 64
                    for j in range(i):
                        acc = 0.0
                        for d in range(K):
                            acc += (float(k[c0 + i, h, d]) * float(k[c0 + j, h, d]) *
                                    math.exp(float(g[c0 + i, h, d]) - float(g[c0 + j, h, d])))
                        row[j] = -float(beta[c0 + i, h]) * acc
                    A[c0 + i, h, :] = row
    return A


def check_kkt_scalar_key(kkt, seed=0):
    """K = 1 and g = 0: A[i][j] = -beta_i k_i k_j below the diagonal, 0 on
    and above it (exactly: exp(0) = 1)."""
    rng = np.random.default_rng(seed)
    lengths = [64, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H = int(cu[-1]), 2
    k = rng.standard_normal((T, H, 1))
    g = np.zeros((T, H, 1))
    beta = rng.random((T, H))
    A = kkt(k, g, beta, cu)
    for c0, L in ((0, 64), (64, 20)):
        for h in range(H):
            kv = k[c0:c0 + L, h, 0]
            want = np.tril(-beta[c0:c0 + L, h, None] * (kv[:, None] * kv[None, :]), -1)
            if not np.array_equal(A[c0:c0 + L, h, :L], want) or np.any(A[c0:c0 + L, h, L:] != 0):
                return False
    return True


def check_kkt_uniform_decay(kkt, seed=1):
    """A decay shared by all channels of a token, g[i][d] = gamma_i: then
    A = -diag(beta) (E * K K^T) below the diagonal with E[i][j] =
    exp(gamma_i - gamma_j) (a Gram matrix of the keys, evaluated by numpy)."""
    rng = np.random.default_rng(seed)
    T, H, K = 64, 1, 16
    k = rng.standard_normal((T, H, K))
    gamma = np.cumsum(-rng.random(T) * 0.2).astype(np.float32).astype(np.float64)
    g = np.repeat(gamma[:, None, None], K, axis=2)
    beta = rng.random((T, H))
    A = kkt(k, g, beta, np.array([0, T], np.int32))
    G = k[:, 0, :] @ k[:, 0, :].T
    E = np.exp(gamma[:, None] - gamma[None, :])
    want = np.tril(-beta[:, 0, None] * E * G, -1)
    return bool(np.abs(A[:, 0, :] - want).max() <= 1e-12 * max(1.0, np.abs(want).max()))


def check_kkt_brute_force(kkt, seed=2):
    """Ragged requests (one longer than a chunk) against the brute force."""
    rng = np.random.default_rng(seed)
    lengths = [5, 70, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, K = int(cu[-1]), 2, 3
    k = rng.standard_normal((T, H, K))
    g = np.cumsum(-rng.random((T, H, K)) * 0.3, axis=0).astype(np.float32).astype(np.float64)
    beta = rng.random((T, H))
    A = kkt(k, g, beta, cu)
    want = kkt_brute_force(k, g, beta, cu)
    return bool(np.abs(A - want).max() <= 1e-13)


def kkt_all(kkt):
    """Names of the A-construction checks that fail (empty when all pass)."""
    checks = {"scalar_key": check_kkt_scalar_key, "uniform_decay": check_kkt_uniform_decay,
              "brute_force": check_kkt_brute_force}
    return [n for n, f in checks.items() if not f(kkt)]


# ---- the fused KDA decode step ---------------------------------------------
#
# Each check takes ``dec(qkv, g, beta, z, wn, cw, slot, S, cs, eps_l2,
# eps_norm) -> (out, S_new, cs_new)`` on float64 arrays (layouts of
# oracle.kda_decode).

def _silu(x):
    return x / (1.0 + np.exp(-x))


def _onehot_conv(H, d, W):
    """Taps that pass the newest input through: y = x."""
    cw = np.zeros((3, W, H, d))
    cw[:, W - 1] = 1.0
    return cw


def check_dec_delta_rule(dec, d=16, W=4):
    """Zero state, g = 0, beta = 1, q = k: one step stores k v^T (so the
    output is RMSNorm(v) * wn * sigmoid(z) exactly up to eps), and a second
    step with the same key and a new value replaces it: S = k v'^T."""
    rng = np.random.default_rng(11)
    H = 1
    cw = _onehot_conv(H, d, W)
    x = rng.standard_normal((1, 3, H, d))
    x[:, 0] = x[:, 1]  # q = k
    z = rng.standard_normal((1, H, d))
    wn = rng.random(d) + 0.5
    S = np.zeros((1, H, d, d))
    cs = np.zeros((1, 3, H, W - 1, d))
    out, S1, _ = dec(x, np.zeros((1, H, d)), np.ones((1, H)), z, wn, cw,
                     np.array([0], np.int32), S, cs, 0.0, 0.0)
    yk, yv = _silu(x[0, 1, 0]), _silu(x[0, 2, 0])
    k = yk / np.linalg.norm(yk)
    ok = np.abs(S1[0, 0] - np.outer(k, yv)).max() <= 1e-13
    want = yv / np.sqrt(np.mean(yv ** 2)) * wn / (1.0 + np.exp(-z[0, 0]))
    ok &= np.abs(out[0, 0] - want).max() <= 1e-12
    x2 = x.copy()
    x2[0, 2] = rng.standard_normal((H, d))
    _, S2, _ = dec(x2, np.zeros((1, H, d)), np.ones((1, H)), z, wn, cw,
                   np.array([0], np.int32), S1, np.zeros_like(cs), 0.0, 0.0)
    ok &= np.abs(S2[0, 0] - np.outer(k, _silu(x2[0, 2, 0]))).max() <= 1e-12
    return bool(ok)


def check_dec_decay_only(dec, d=8, W=4):
    """beta = 0: the state only decays, S_new = diag(exp(g)) S."""
    rng = np.random.default_rng(12)
    H, slots = 2, 2
    S = rng.standard_normal((slots, H, d, d))
    g = -rng.random((1, H, d))
    _, S1, _ = dec(rng.standard_normal((1, 3, H, d)), g, np.zeros((1, H)),
                   rng.standard_normal((1, H, d)), np.ones(d), rng.standard_normal((3, W, H, d)),
                   np.array([1], np.int32), S, rng.standard_normal((slots, 3, H, W - 1, d)),
                   1e-6, 1e-6)
    want = S.copy()
    want[1] = np.exp(g[0])[:, :, None] * S[1]
    return bool(np.abs(S1 - want).max() <= 1e-14)


def check_dec_conv_taps(dec, d=8, W=4):
    """A one-hot tap t picks the t-th oldest input of the window (the new
    token for t = W - 1), and the window shifts by one: check both through
    the value path (zero state, q = k, beta = 1, g = 0: the output is the
    normalised silu of the picked input) and the returned conv state."""
    rng = np.random.default_rng(13)
    H = 1
    ok = True
    for t in range(W):
        cw = np.zeros((3, W, H, d))
        cw[0, W - 1] = cw[1, W - 1] = 1.0
        cw[2, t] = 1.0
        x = rng.standard_normal((1, 3, H, d))
        x[:, 0] = x[:, 1]
        cs = rng.standard_normal((1, 3, H, W - 1, d))
        out, _, cs1 = dec(x, np.zeros((1, H, d)), np.ones((1, H)), np.full((1, H, d), 40.0),
                          np.ones(d), cw, np.array([0], np.int32), np.zeros((1, H, d, d)), cs,
                          0.0, 0.0)
        window = np.concatenate([cs[0, 2, 0], x[0, 2]], axis=0)  # oldest first, new last
        yv = _silu(window[t])
        ok &= np.abs(out[0, 0] - yv / np.sqrt(np.mean(yv ** 2))).max() <= 1e-12
        shifted = np.concatenate([cs[0, :, 0, 1:], x[0, :, 0][:, None, :]], axis=1)
        ok &= np.array_equal(cs1[0, :, 0], shifted)
    return bool(ok)


def check_dec_padding_and_slots(dec, d=8, W=4):
    """Batch entries map to state slots; a negative slot is padding (output
    0, no state touched); slots that no entry names are untouched."""
    rng = np.random.default_rng(14)
    H, slots = 2, 4
    S = rng.standard_normal((slots, H, d, d))
    cs = rng.standard_normal((slots, 3, H, W - 1, d))
    slot = np.array([3, -1, 0], np.int32)
    args = (rng.standard_normal((3, 3, H, d)), -rng.random((3, H, d)), rng.random((3, H)),
            rng.standard_normal((3, H, d)), np.ones(d), rng.standard_normal((3, W, H, d)))
    out, S1, cs1 = dec(*args, slot, S, cs, 1e-6, 1e-6)
    ok = np.all(out[1] == 0)
    ok &= np.array_equal(S1[[1, 2]], S[[1, 2]]) and np.array_equal(cs1[[1, 2]], cs[[1, 2]])
    ok &= not np.array_equal(S1[3], S[3]) and not np.array_equal(S1[0], S[0])
    # the same entries alone, each on a fresh copy, give the same result
    for b, s in ((0, 3), (2, 0)):
        one = tuple(a[b:b + 1] for a in args[:4]) + args[4:]
        o1, Sb, _ = dec(*one, np.array([s], np.int32), S, cs, 1e-6, 1e-6)
        ok &= np.array_equal(o1[0], out[b]) and np.array_equal(Sb[s], S1[s])
    return bool(ok)


def check_dec_q_scale(dec, d=16, W=3):
    """The scales of q and k, seen through an output that keeps them: zero
    state, g = 0, beta = 1 and pass-through taps make the step store k v^T
    and return o = (k . q) v; with eps_norm = 1, far above mean(o^2), the
    gated RMSNorm no longer cancels a positive factor on q. Before the
    normalisation q and k are one-hot in channel m of each head,
    y_q = silu(xq) e_m and y_k = silu(xk) e_m, so by hand
        q = e_m silu(xq) / sqrt(silu(xq)^2 + eps_l2) / sqrt(d),
        k = e_m silu(xk) / sqrt(silu(xk)^2 + eps_l2),
        out_j = (k_m q_m) v_j / sqrt((k_m q_m)^2 mean(v^2) + eps_norm) wn_j sigmoid(z_j),
    for two values of eps_l2 (0 and 0.5) and a negative silu(xk), so the
    sign of k . q enters too."""
    rng = np.random.default_rng(16)
    H = 2
    cw = _onehot_conv(H, d, W)
    ok = True
    for eps_l2 in (0.0, 0.5):
        x = np.zeros((1, 3, H, d))
        xq, xk = np.array([1.5, 0.75]), np.array([-2.0, 3.0])
        for h, m in enumerate((3, 10)):
            x[0, 0, h, m] = xq[h]
            x[0, 1, h, m] = xk[h]
        x[0, 2] = rng.standard_normal((H, d))
        z = rng.standard_normal((1, H, d))
        wn = rng.random(d) + 0.5
        out, _, _ = dec(x, np.zeros((1, H, d)), np.ones((1, H)), z, wn, cw,
                        np.array([0], np.int32), np.zeros((1, H, d, d)),
                        np.zeros((1, 3, H, W - 1, d)), eps_l2, 1.0)
        for h in range(H):
            a = xq[h] / (1.0 + np.exp(-xq[h]))
            b = xk[h] / (1.0 + np.exp(-xk[h]))
            qm = a / np.sqrt(a * a + eps_l2) / np.sqrt(d)
            km = b / np.sqrt(b * b + eps_l2)
            v = _silu(x[0, 2, h])
            o = km * qm * v
            want = o / np.sqrt(np.mean(o * o) + 1.0) * wn / (1.0 + np.exp(-z[0, h]))
            ok &= np.abs(out[0, h] - want).max() <= 1e-13
    return bool(ok)


def dec_brute_force(qkv, g, beta, z, wn, cw, slot, S, cs, eps_l2, eps_norm):
    """The decode step with Python floats and loops, entry by entry."""
    import math
    B, _, H, d = qkv.shape
    W = cw.shape[1]
    S = [[[[float(S[s, h, i, j]) for j in range(d)] for i in range(d)] for h in range(H)]
         for s in range(S.shape[0])]
    cs = cs.astype(float).tolist()
    out = [[[0.0] * d for _ in range(H)] for _ in range(B)]
    for b in range(B):
        s = int(slot[b])
        if s < 0:
            continue
        for h in range(H):
            y = []
            for p in range(3):
                row = []
                for c in range(d):
                    win = [cs[s][p][h][w][c] for w in range(W - 1)] + [float(qkv[b, p, h, c])]
                    acc = sum(float(cw[p, w, h, c]) * win[w] for w in range(W))
                    for w in range(W - 1):
                        cs[s][p][h][w][c] = win[w + 1]
                    row.append(acc / (1.0 + math.exp(-acc)))
                y.append(row)
            nq = math.sqrt(sum(t * t for t in y[0]) + eps_l2) * math.sqrt(d)
            nk = math.sqrt(sum(t * t for t in y[1]) + eps_l2)
            q = [t / nq for t in y[0]]
            k = [t / nk for t in y[1]]
            M = S[s][h]
            for i in range(d):
                a = math.exp(float(g[b, h, i]))
                for j in range(d):
                    M[i][j] *= a
            u = [float(beta[b, h]) * (y[2][j] - sum(M[i][j] * k[i] for i in range(d)))
                 for j in range(d)]
            for i in range(d):
                for j in range(d):
                    M[i][j] += k[i] * u[j]
            o = [sum(M[i][j] * q[i] for i in range(d)) for j in range(d)]
            rn = math.sqrt(sum(t * t for t in o) / d + eps_norm)
            out[b][h] = [o[j] / rn * float(wn[j]) / (1.0 + math.exp(-float(z[b, h, j])))
                         for j in range(d)]
    return np.array(out), np.array(S), np.array(cs)


def check_dec_brute_force(dec, d=6, W=3):
    rng = np.random.default_rng(15)
    B, H, slots = 3, 2, 4
    args = (rng.standard_normal((B, 3, H, d)), -rng.random((B, H, d)), rng.random((B, H)),
            rng.standard_normal((B, H, d)), rng.random(d) + 0.5,
            rng.standard_normal((3, W, H, d)) * 0.5, np.array([2, -1, 0], np.int32),
            rng.standard_normal((slots, H, d, d)), rng.standard_normal((slots, 3, H, W - 1, d)))
    got = dec(*args, 1e-6, 1e-3)
    want = dec_brute_force(*args, 1e-6, 1e-3)
    return all(np.abs(a - b).max() <= 1e-12 for a, b in zip(got, want))


def dec_all(dec):
    checks = {"delta_rule": check_dec_delta_rule, "decay_only": check_dec_decay_only,
              "conv_taps": check_dec_conv_taps, "padding_and_slots": check_dec_padding_and_slots,
              "q_scale": check_dec_q_scale, "brute_force": check_dec_brute_force}
    return [n for n, f in checks.items() if not f(dec)]
