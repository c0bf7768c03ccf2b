"""Host-side checks of the C ABI (CPU only: no call here reaches a kernel).

The library must load, export every entry point include/kda_tril.h declares,
size workspaces and choose plans as documented, and reject bad arguments
before any launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda_tril.h")


@pytest.fixture(scope="module")
def kt():
    import tril_solve_amd
    return tril_solve_amd


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol(kt):
    names = declared_functions()
    assert names == sorted(kt.EXPORTED)
    lib = ctypes.CDLL(kt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(kt):
    for code in (0, -1, -2, -3, -4):
        s = kt.kda_status_string(code)
        assert s.startswith("KDA_")
    assert "UNKNOWN" in kt.kda_status_string(7)


def test_workspace_sizes(kt):
    # packed 16 x 512 tokens, 64 heads, exact chunk count: 4 KiB per
    # chunk-head, 32 MiB in all; the FP32 input is 128 MiB, so split fits
    b, c = kt.kda_tril_inv_workspace_size(8192, 16, 128, 64, "split")
    assert (b, c) == (128 * 64 * 4096, "split") and b == 32 * 2**20
    # without the exact count the bound floor(T/64) + N slots is used
    b, _ = kt.kda_tril_inv_workspace_size(8192, 16, 0, 64, "split")
    assert b == (128 + 16) * 64 * 4096
    for algo in ("fused", "fused_valu"):
        assert kt.kda_tril_inv_workspace_size(8192, 16, 128, 64, algo) == (0, algo)


def test_split_budget_is_fp32_input_size(kt):
    # scratch <= FP32 input  <=>  T / slots >= 16
    assert kt.kda_tril_inv_workspace_size(16 * 10, 1, 10, 4, "split")[1] == "split"
    with pytest.raises(kt.KdaError) as e:
        kt.kda_tril_inv_workspace_size(16 * 10 - 1, 1, 10, 4, "split")
    assert e.value.status == kt.KDA_ERR_WORKSPACE
    # many one-token requests: occupancy 1 token per chunk
    with pytest.raises(kt.KdaError):
        kt.kda_tril_inv_workspace_size(100, 100, 100, 8, "split")


def test_auto_plan_rule(kt, monkeypatch):
    # default: no input size where split was measured faster -> fused
    assert kt.kda_tril_auto_plan(8192, 128, 64, 2**40) == "fused"
    monkeypatch.setenv("KDA_TRIL_SPLIT_MIN_TOKENS", "4096")
    assert kt.kda_tril_auto_plan(8192, 128, 64, 2**40) == "split"
    assert kt.kda_tril_auto_plan(4095, 64, 64, 2**40) == "fused"       # below min length
    assert kt.kda_tril_auto_plan(8192, 128, 64, 128 * 64 * 4096 - 1) == "fused"  # short ws
    assert kt.kda_tril_auto_plan(8192, 1000, 64, 2**40) == "fused"     # over budget
    assert kt.kda_tril_inv_workspace_size(8192, 16, 128, 64, "auto") == (32 * 2**20, "split")
    monkeypatch.setenv("KDA_TRIL_SPLIT_MIN_TOKENS", "0")
    assert kt.kda_tril_auto_plan(64, 1, 64, 2**40) == "split"


def test_workspace_query_errors(kt):
    for args in [(-1, 1, 0, 4), (10, -1, 0, 4), (10, 1, -1, 4), (10, 1, 0, 0)]:
        with pytest.raises(kt.KdaError) as e:
            kt.kda_tril_inv_workspace_size(*args, "auto")
        assert e.value.status == kt.KDA_ERR_INVALID_ARG
    with pytest.raises(kt.KdaError) as e:
        kt.kda_tril_inv_workspace_size(2**31, 1, 0, 4, "auto")
    assert e.value.status == kt.KDA_ERR_UNSUPPORTED


# ---- argument validation: every case returns before any launch ------------

P = ctypes.c_void_p


def _packed(kt, A=0x10000, ad=0, X=0x90000000, xd=0, cu=0x2000, nseq=1, T=64, H=2, cmap=None,
            nch=0, ws=None, wsb=0, algo=1):
    return kt._lib.kda_tril_inv_packed(P(A), ad, P(X), xd, P(cu), nseq, T, H, P(cmap), nch, P(ws),
                                       wsb, algo, None)


def _dense(kt, A=0x10000, ad=0, X=0x90000000, xd=0, B=1, T=64, H=2, ws=None, wsb=0, algo=1):
    return kt._lib.kda_tril_inv_dense(P(A), ad, P(X), xd, B, T, H, P(ws), wsb, algo, None)


def test_invalid_arguments_rejected_before_launch(kt):
    E = kt.KDA_ERR_INVALID_ARG
    assert _packed(kt, ad=3) == E                      # unknown input dtype
    assert _packed(kt, xd=-1) == E                     # unknown output dtype
    assert _packed(kt, algo=9) == E                    # unknown plan
    assert _packed(kt, H=0) == E
    assert _packed(kt, A=None) == E
    assert _packed(kt, X=None) == E
    assert _packed(kt, cu=None) == E
    assert _packed(kt, A=0x10008) == E                 # misaligned
    assert _packed(kt, X=0x10000 + 64 * 2 * 64 * 4 - 16) == E  # overlaps A
    assert _packed(kt, cmap=0x3000, nch=0) == E        # map without a length
    assert _packed(kt, cmap=None, nch=5) == E
    assert _packed(kt, nseq=-1) == E
    assert _packed(kt, T=-5) == E
    assert _dense(kt, B=-1) == E
    assert _dense(kt, H=-3) == E
    assert _dense(kt, A=None) == E


def test_unsupported_sizes(kt):
    U = kt.KDA_ERR_UNSUPPORTED
    assert _packed(kt, T=2**31) == U
    assert _dense(kt, B=2**20, T=2**12) == U
    # chunk slots x heads = 2^26 - 1: one wavefront each fits 2^32 threads,
    # but not once rounded up to whole 4-wavefront workgroups
    slots = (2**26 - 1) // 3
    assert _dense(kt, T=64 * slots, H=3, X=1 << 44) == U


def test_forced_split_workspace_errors(kt):
    W = kt.KDA_ERR_WORKSPACE
    assert _packed(kt, algo=2) == W                    # no workspace
    assert _packed(kt, algo=2, ws=0x4000, wsb=1000) == W
    assert _dense(kt, algo=2) == W
    # budget exceeded: 64 one-token requests
    assert _packed(kt, algo=2, nseq=64, T=64, ws=0x4000, wsb=2**40) == W
    # enough workspace but misaligned
    assert _packed(kt, algo=2, ws=0x4004, wsb=2**30) == kt.KDA_ERR_INVALID_ARG


def test_split_workspace_must_not_overlap_a_or_x(kt):
    """The split plan's diagonal kernel writes the workspace before the merge
    kernel reads A, so a workspace that overlaps A (or X) is refused before
    any launch; the fused plans ignore the workspace."""
    E = kt.KDA_ERR_INVALID_ARG
    a_bytes = 64 * 2 * 64 * 4                 # A: 64 tokens x 2 heads x 64 fp32
    need = 1 * 2 * 4096                       # one chunk, two heads
    big = 2**30
    # workspace inside A, straddling A's end, inside X, straddling X's start
    for ws in (0x10000, 0x10000 + a_bytes - 16, 0x90000000, 0x90000000 - need + 16):
        assert _packed(kt, algo=2, ws=ws, wsb=big) == E, hex(ws)
        assert _dense(kt, algo=2, ws=ws, wsb=big) == E, hex(ws)
    # the bytes checked are the ones the split plan uses for these sizes
    assert kt.kda_tril_inv_workspace_size(64, 1, 0, 2, "split") == (need + 2 * 4096, "split")
    assert kt.kda_tril_inv_workspace_size(64, 1, 1, 2, "split") == (need, "split")


def test_algo_override_applies_to_auto_only(kt, monkeypatch):
    """KDA_TRIL_ALGO replaces AUTO's choice (read on every call); calls that
    name a plan keep it, and an ineligible split still falls back to fused."""
    ws = kt.kda_tril_inv_workspace_size
    monkeypatch.setenv("KDA_TRIL_ALGO", "split")
    assert ws(8192, 16, 128, 64, "auto") == (32 * 2**20, "split")
    assert kt.kda_tril_auto_plan(8192, 128, 64, 2**40) == "split"
    assert kt.kda_tril_auto_plan(8192, 128, 64, 100) == "fused"       # workspace short
    assert kt.kda_tril_auto_plan(8192, 1000, 64, 2**40) == "fused"    # over the budget
    assert ws(8192, 16, 128, 64, "fused") == (0, "fused")
    monkeypatch.setenv("KDA_TRIL_ALGO", "fused_valu")
    assert ws(8192, 16, 128, 64, "auto") == (0, "fused_valu")
    assert ws(8192, 16, 128, 64, "split") == (32 * 2**20, "split")
    for v in ("fused", "auto", "", "nonsense"):
        monkeypatch.setenv("KDA_TRIL_ALGO", v)
        assert ws(8192, 16, 128, 64, "auto") == (0, "fused"), v
    monkeypatch.delenv("KDA_TRIL_ALGO")
    assert ws(8192, 16, 128, 64, "auto") == (0, "fused")


def test_empty_problems_are_noops(kt):
    assert _packed(kt, T=0) == kt.KDA_OK
    assert _packed(kt, nseq=0) == kt.KDA_OK
    assert _packed(kt, T=0, A=None, X=None, cu=None) == kt.KDA_OK
    assert _dense(kt, B=0) == kt.KDA_OK
    assert _dense(kt, T=0, A=None, X=None) == kt.KDA_OK


# ---- the 16- and 32-token entry points ---------------------------------------

def _packed_c(kt, C, A=0x10000, ad=0, X=0x90000000, xd=0, cu=0x2000, nseq=1, T=64, H=2,
              cmap=None, nch=0, ws=None, wsb=0, algo=1):
    return kt._lib.kda_tril_inv_packed_chunk(P(A), ad, P(X), xd, P(cu), nseq, T, H, C, P(cmap),
                                             nch, P(ws), wsb, algo, None)


def _dense_c(kt, C, A=0x10000, ad=0, X=0x90000000, xd=0, B=1, T=64, H=2, ws=None, wsb=0,
             algo=1):
    return kt._lib.kda_tril_inv_dense_chunk(P(A), ad, P(X), xd, B, T, H, C, P(ws), wsb, algo,
                                            None)


def test_chunk_size_validation(kt):
    E, U = kt.KDA_ERR_INVALID_ARG, kt.KDA_ERR_UNSUPPORTED
    for C in (0, -16, 8, 48, 128):
        assert _packed_c(kt, C) == E
        assert _dense_c(kt, C) == E
    for C in (16, 32):
        # one kernel per small chunk size: no split, no VALU merge
        assert _packed_c(kt, C, algo=kt.KDA_ALGO_SPLIT) == U
        assert _packed_c(kt, C, algo=kt.KDA_ALGO_FUSED_VALU) == U
        assert _dense_c(kt, C, algo=kt.KDA_ALGO_SPLIT) == U
        assert _packed_c(kt, C, algo=9) == E
        assert _packed_c(kt, C, ad=3) == E
        assert _packed_c(kt, C, A=None) == E
        assert _packed_c(kt, C, cu=None) == E
        assert _packed_c(kt, C, cmap=0x3000, nch=0) == E
        assert _packed_c(kt, C, T=2**31) == U
        # empty problems return before touching the device
        assert _packed_c(kt, C, T=0, A=None, X=None, cu=None) == kt.KDA_OK
        assert _dense_c(kt, C, B=0) == kt.KDA_OK
    # the overlap check uses the row length C: X starting inside the 64 x 2 x C
    # floats of A overlaps, for every C
    for C in (16, 32, 64):
        assert _packed_c(kt, C, X=0x10000 + 64 * 2 * C * 4 - 16) == E
    # C = 64 is the 64-token entry point: forced split without workspace
    assert _packed_c(kt, 64, algo=kt.KDA_ALGO_SPLIT) == kt.KDA_ERR_WORKSPACE


def test_head_limit(kt):
    U = kt.KDA_ERR_UNSUPPORTED
    assert _packed(kt, H=4097) == U
    assert _dense(kt, H=4097) == U
    assert _packed_c(kt, 16, H=4097) == U
    with pytest.raises(kt.KdaError) as e:
        kt.kda_tril_inv_workspace_size(64, 1, 0, 4097, "auto")
    assert e.value.status == U


# ---- A built from keys, decays and write strengths ---------------------------

def _kkt_p(kt, k=0x10000, g=0x20000, beta=0x30000, kd=0, X=0x90000000, xd=0, cu=0x2000, nseq=1,
           T=64, H=2, K=128, cmap=None, nch=0, solve=True):
    fn = kt._lib.kda_kkt_tril_inv_packed if solve else kt._lib.kda_kkt_packed
    return fn(P(k), P(g), P(beta), kd, P(X), xd, P(cu), nseq, T, H, K, P(cmap), nch, None)


def _kkt_d(kt, k=0x10000, g=0x20000, beta=0x30000, kd=0, X=0x90000000, xd=0, B=1, T=64, H=2,
           K=128, solve=True):
    fn = kt._lib.kda_kkt_tril_inv_dense if solve else kt._lib.kda_kkt_dense
    return fn(P(k), P(g), P(beta), kd, P(X), xd, B, T, H, K, None)


def test_kkt_argument_validation(kt):
    E, U = kt.KDA_ERR_INVALID_ARG, kt.KDA_ERR_UNSUPPORTED
    for solve in (True, False):
        for K in (8, 24, 100, 272, 512):       # not a multiple of 16, or too wide
            assert _kkt_p(kt, K=K, solve=solve) == U
        assert _kkt_p(kt, K=0, solve=solve) == E
        assert _kkt_p(kt, kd=3, solve=solve) == E
        assert _kkt_p(kt, xd=7, solve=solve) == E
        assert _kkt_p(kt, H=0, solve=solve) == E
        assert _kkt_p(kt, H=4097, solve=solve) == U
        assert _kkt_p(kt, k=None, solve=solve) == E
        assert _kkt_p(kt, g=None, solve=solve) == E
        assert _kkt_p(kt, beta=None, solve=solve) == E
        assert _kkt_p(kt, cu=None, solve=solve) == E
        assert _kkt_p(kt, k=0x10008, solve=solve) == E      # misaligned keys
        assert _kkt_p(kt, g=0x20004, solve=solve) == E      # misaligned decays
        assert _kkt_p(kt, beta=0x30002, solve=solve) == E   # fp32 beta not 4-byte aligned
        # X starting inside the 64 x 2 x 128 fp32 keys overlaps them
        assert _kkt_p(kt, X=0x10000 + 64 * 2 * 128 * 4 - 16, solve=solve) == E
        assert _kkt_p(kt, X=0x30000 + 64 * 2 * 4 - 16, solve=solve) == E  # overlaps beta
        assert _kkt_p(kt, cmap=0x3000, nch=0, solve=solve) == E
        assert _kkt_p(kt, T=-1, solve=solve) == E
        assert _kkt_p(kt, T=2**31, solve=solve) == U
        assert _kkt_d(kt, B=-1, solve=solve) == E
        assert _kkt_d(kt, K=40, solve=solve) == U
        # empty problems return before touching the device
        assert _kkt_p(kt, T=0, k=None, g=None, beta=None, X=None, cu=None, solve=solve) == kt.KDA_OK
        assert _kkt_d(kt, B=0, solve=solve) == kt.KDA_OK
        assert _kkt_d(kt, T=0, k=None, g=None, beta=None, X=None, solve=solve) == kt.KDA_OK


# ---- the fused KDA decode core -----------------------------------------------

def _dec(kt, qkv=0x10000, z=0x20000, ind=0, g=0x30000, beta=0x40000, wn=0x50000, cw=0x60000,
         slot=0x70000, S=0x1000000, cs=0x80000, ns=4, out=0x90000000, outd=0, B=2, H=2, d=128,
         W=4, e1=1e-6, e2=1e-6):
    return kt._lib.kda_decode_step(P(qkv), P(z), ind, P(g), P(beta), P(wn), P(cw), P(slot), P(S),
                                   P(cs), ns, P(out), outd, B, H, d, W, e1, e2, None)


def test_decode_argument_validation(kt):
    E, U = kt.KDA_ERR_INVALID_ARG, kt.KDA_ERR_UNSUPPORTED
    assert _dec(kt, d=64) == U
    assert _dec(kt, W=1) == U and _dec(kt, W=5) == U
    assert _dec(kt, B=1 << 23, H=2) == U and _dec(kt, B=1 << 24, H=1) == U  # grid past 2^32 threads
    assert _dec(kt, ind=3) == E and _dec(kt, outd=-1) == E
    assert _dec(kt, H=0) == E and _dec(kt, B=-1) == E and _dec(kt, ns=-1) == E
    assert _dec(kt, ns=0) == E
    assert _dec(kt, e1=-1.0) == E and _dec(kt, e2=float("nan")) == E
    assert _dec(kt, e2=float("inf")) == E
    for name in ("qkv", "z", "g", "beta", "wn", "cw", "slot", "S", "cs", "out"):
        assert _dec(kt, **{name: None}) == E, name
    assert _dec(kt, S=0x1000008) == E                # state not 16-byte aligned
    assert _dec(kt, g=0x30002) == E                  # fp32 not 4-byte aligned
    assert _dec(kt, ind=1, qkv=0x10001) == E         # bf16 not 2-byte aligned
    assert _dec(kt, out=0x1000000 + 4 * 2 * 128 * 128 * 4 - 64) == E  # out overlaps state
    assert _dec(kt, B=0) == kt.KDA_OK                # no-op before any pointer is used
    assert _dec(kt, B=0, qkv=None, out=None) == kt.KDA_OK


def test_binding_refuses_host_tensors_and_bad_shapes(kt):
    """The Python binding refuses host (CPU) tensors before any library call,
    since a kernel would dereference their host addresses, and reports
    malformed arguments as ValueError."""
    torch = pytest.importorskip("torch")
    A = torch.zeros((64, 2, 64))
    cu = torch.tensor([0, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="cuda tensor"):
        kt.tril_inv(A, cu)
    with pytest.raises(ValueError, match="cuda tensor"):
        kt.tril_inv(A.view(1, 64, 2, 64))
    with pytest.raises(ValueError, match="chunk size"):
        kt.kda_tril_inv_packed(torch.zeros((64, 2, 48)), torch.zeros((64, 2, 48)), cu)
    with pytest.raises(ValueError, match="int32"):
        kt.kda_tril_inv_packed(A, torch.zeros_like(A), cu.long())
    k = torch.zeros((64, 2, 16))
    with pytest.raises(ValueError, match="cuda tensor"):
        kt.kda_kkt_tril_inv(k, torch.zeros_like(k), torch.zeros((64, 2)),
                            torch.zeros((64, 2, 64)), cu)
    with pytest.raises(ValueError, match="float32"):
        kt.kda_kkt_tril_inv(k, torch.zeros_like(k, dtype=torch.float64), torch.zeros((64, 2)),
                            torch.zeros((64, 2, 64)), cu)
    B, H, d, W, S = 2, 1, 128, 4, 3
    dec = dict(qkv=torch.zeros((B, 3, H, d)), z=torch.zeros((B, H, d)), g=torch.zeros((B, H, d)),
               beta=torch.zeros((B, H)), norm_w=torch.zeros(d), conv_w=torch.zeros((3, W, H, d)),
               slot=torch.zeros(B, dtype=torch.int32), state=torch.zeros((S, H, d, d)),
               conv_state=torch.zeros((S, 3, H, W - 1, d)), out=torch.zeros((B, H, d)))
    with pytest.raises(ValueError, match="cuda tensor"):
        kt.kda_decode_step(**dec)
    with pytest.raises(ValueError, match="norm_w"):
        kt.kda_decode_step(**dict(dec, norm_w=torch.zeros((H, d))))


C_CALLER = r"""
#include <stdio.h>
#include "kda_tril.h"

int main(void) {
    size_t bytes = 0;
    kda_algo chosen = KDA_ALGO_AUTO;
    kda_status s = kda_tril_inv_workspace_size(8192, 16, 0, 64, KDA_ALGO_SPLIT, &bytes, &chosen);
    printf("%d %zu %d %s\n", (int)s, bytes, (int)chosen, kda_status_string(s));
    return s == KDA_OK ? 0 : 1;
}
"""


def test_header_serves_a_plain_c_caller(kt, tmp_path):
    """include/kda_tril.h compiles as C11 (no C++ needed), and a C program
    linked against the library makes a host-only call through it."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are missing")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(kt.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe), "-L", libdir,
                    "-lkda_tril", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == "0" and out[3] == "KDA_OK"
    want_bytes, want_algo = kt.kda_tril_inv_workspace_size(8192, 16, 0, 64, "split")
    assert int(out[1]) == want_bytes
    assert kt.ALGO_NAMES[int(out[2])] == want_algo


# ---- the allocation-free entry point -----------------------------------------

def _noalloc(kt, A=0x10000, ad=0, X=0x90000000, xd=0, cu=0x2000, nseq=1, T=64, H=2, cmap=None,
             nch=0):
    return kt._lib.kda_tril_inv_packed_noalloc(P(A), ad, P(X), xd, P(cu), nseq, T, H, P(cmap),
                                               nch, None)


def test_noalloc_refuses_before_any_device_call(kt):
    """Every refusal of kda_tril_inv_packed_noalloc happens on the host: bad
    arguments, a split workspace past the 64 MiB scratch, or a split past the
    FP32-input budget."""
    E, W = kt.KDA_ERR_INVALID_ARG, kt.KDA_ERR_WORKSPACE
    assert kt.NOALLOC_SCRATCH_BYTES == 64 * 2**20
    assert _noalloc(kt, ad=3) == E and _noalloc(kt, H=0) == E and _noalloc(kt, A=None) == E
    assert _noalloc(kt, cu=None) == E and _noalloc(kt, cmap=0x3000, nch=0) == E
    assert _noalloc(kt, X=0x10000 + 64 * 2 * 64 * 4 - 16) == E
    assert _noalloc(kt, T=2**31) == kt.KDA_ERR_UNSUPPORTED
    # 16,384 chunk-heads fit exactly (with a chunk map giving the exact count);
    # one more head per chunk does not
    mib64 = 64 * 2**20
    assert 256 * 64 * 4096 == mib64
    assert _noalloc(kt, T=256 * 64, nseq=1, H=65, cmap=0x3000, nch=256) == W
    # without a map the slot bound floor(T/64) + num_seqs is what must fit
    assert _noalloc(kt, T=256 * 64, nseq=1, H=64) == W
    # budget: 64 one-token requests, occupancy 1
    assert _noalloc(kt, T=64, nseq=64, H=2) == W
    # empty problems are no-ops that never look up the scratch
    assert _noalloc(kt, T=0, A=None, X=None, cu=None) == kt.KDA_OK
    assert _noalloc(kt, nseq=0) == kt.KDA_OK
