"""Host-only checks of the C ABI: the library loads, exports every function
that include/moe_fp8.h declares, and rejects bad arguments with the
documented codes before launching anything (no GPU needed: every call here
fails validation or is a zero-sized no-op, so no HIP API is reached)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from fp8_block_scaled_bias_amd import _lib as L

HEADER = os.path.join(ROOT, "include", "moe_fp8.h")
FAKE = ctypes.c_void_p(4096)  # never dereferenced: validation fails first


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = header_functions()
    assert "grouped_fp8_gemm" in names and "moe_route" in names and len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, n
    assert set(L.SIGNATURES) == set(names)
    assert L.version().startswith("moe_fp8")


def rc(name, *args):
    return getattr(L.lib(), name)(*args)


def test_quant_validation():
    assert rc("fp8_quant_1x128", FAKE, 4, 100, 100, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert "K=100" in L.last_error()
    assert rc("fp8_quant_1x128", FAKE, 4, 128, 128, 2, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert rc("fp8_quant_1x128", FAKE, 4, 128, 128, 1, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert "ld_in" in L.last_error()
    assert rc("fp8_quant_1x128", None, 4, 128, 128, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert rc("fp8_quant_1x128", ctypes.c_void_p(4100), 4, 128, 128, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert "aligned" in L.last_error()
    assert rc("fp8_quant_1x128", None, 0, 128, 128, 0, None, None, None) == L.MOE_OK
    assert rc("fp8_quant_128x128", FAKE, 2, 100, 128, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert rc("fp8_quant_128x128", None, 0, 128, 128, None, None, None) == L.MOE_OK


def test_transpose_validation():
    def f(G=2, N=256, K=384, w=FAKE, ws=FAKE, wt=ctypes.c_void_p(8192), wts=ctypes.c_void_p(8192 + 64)):
        return rc("fp8_transpose_128x128", w, ws, G, N, K, wt, wts, None)
    assert f(N=100) == L.MOE_ERR_INVALID and "N=100" in L.last_error()
    assert f(K=0) == L.MOE_ERR_INVALID
    assert f(G=-1) == L.MOE_ERR_INVALID and f(G=70000) == L.MOE_ERR_INVALID
    assert f(w=None) == L.MOE_ERR_INVALID and "null" in L.last_error()
    assert f(w=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    assert f(wt=FAKE) == L.MOE_ERR_INVALID and "alias" in L.last_error()
    assert f(G=0, w=None, ws=None, wt=None, wts=None) == L.MOE_OK


def test_wgrad_validation():
    cap = 1 + 4                              # M_total = 100, G = 4
    def q(G=4, M=100, C=256, ld_in=256, cap=cap, out=FAKE, idx=None, in_rows=100):
        return rc("fp8_quant_128x1_grouped", FAKE, ld_in, idx, in_rows, FAKE, G, M, C, out, FAKE, cap,
                  None)
    assert q(C=100) == L.MOE_ERR_INVALID and "C=100" in L.last_error()
    assert q(G=0) == L.MOE_ERR_INVALID
    assert q(G=2000) == L.MOE_ERR_UNSUPPORTED
    assert q(ld_in=128) == L.MOE_ERR_INVALID and "ld_in" in L.last_error()
    assert q(cap=cap - 1) == L.MOE_ERR_INVALID and "chunks_cap" in L.last_error()
    assert q(out=None) == L.MOE_ERR_INVALID
    assert q(out=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    assert q(in_rows=99) == L.MOE_ERR_INVALID and "in_rows" in L.last_error()
    assert q(idx=FAKE, in_rows=0) == L.MOE_ERR_INVALID
    def w(G=4, M=100, N=256, K=384, cap=cap, dW=FAKE):
        return rc("grouped_fp8_wgrad", FAKE, FAKE, FAKE, FAKE, cap, FAKE, G, M, N, K, dW, None)
    assert w(N=200) == L.MOE_ERR_INVALID and "N=200" in L.last_error()
    assert w(G=0) == L.MOE_ERR_INVALID
    assert w(cap=4) == L.MOE_ERR_INVALID and "chunks_cap" in L.last_error()
    assert w(dW=None) == L.MOE_ERR_INVALID
    assert L.wgrad_chunks(100, 4) == cap and L.wgrad_chunks(256, 3) == 5


def test_backward_elementwise_validation():
    def c(T=4, k=2, H=256, ns=1, dD=ctypes.c_void_p(8192)):
        return rc("moe_combine_backward", FAKE, FAKE, FAKE, FAKE, T, k, H, ns, dD, FAKE, None, None,
                  None)
    assert c(k=9) == L.MOE_ERR_INVALID and "k=9" in L.last_error()
    assert c(H=100) == L.MOE_ERR_INVALID
    assert c(ns=2) == L.MOE_ERR_INVALID
    assert c(dD=FAKE) == L.MOE_ERR_INVALID and "alias" in L.last_error()
    assert c(dD=None) == L.MOE_ERR_INVALID
    assert c(T=0, dD=None) == L.MOE_OK
    def g(M=4, I=128, out=FAKE):
        return rc("swiglu_backward", FAKE, FAKE, M, I, out, FAKE, None, None, None)
    assert g(I=100) == L.MOE_ERR_INVALID and "I=100" in L.last_error()
    assert g(out=None) == L.MOE_ERR_INVALID
    assert g(out=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    # the fused 1x128 codes: both or neither, whole 128-column tiles
    assert rc("swiglu_backward", FAKE, FAKE, 4, 128, FAKE, FAKE, FAKE, None, None) == L.MOE_ERR_INVALID
    assert "together" in L.last_error()
    assert rc("swiglu_backward", FAKE, FAKE, 4, 136, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID
    assert "I % 128" in L.last_error()
    assert rc("moe_combine_backward", FAKE, FAKE, FAKE, ctypes.c_void_p(8192), 4, 2, 136, 1, FAKE, FAKE,
              FAKE, FAKE, None) == L.MOE_ERR_INVALID and "H % 128" in L.last_error()
    def sg(G=2, M_=300, I=256, cap=100, out=FAKE, codes=FAKE):
        return rc("swiglu_backward_grouped", FAKE, FAKE, FAKE, G, M_, I, out, FAKE, codes, FAKE, cap,
                  FAKE, FAKE, FAKE, FAKE, None)
    assert sg(I=200) == L.MOE_ERR_INVALID and "I=200" in L.last_error()
    assert sg(G=0) == L.MOE_ERR_INVALID
    assert sg(G=2000) == L.MOE_ERR_UNSUPPORTED
    assert sg(cap=3) == L.MOE_ERR_INVALID and "chunks_cap" in L.last_error()
    assert sg(codes=None) == L.MOE_ERR_INVALID and "null" in L.last_error()
    # the bf16 dGU and h are optional, but only together
    assert sg(out=None) == L.MOE_ERR_INVALID and "together" in L.last_error()
    assert sg(out=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    assert sg(M_=0, out=None) == L.MOE_OK
    assert g(M=0, out=None) == L.MOE_OK
    def r(T=4, H=256, E=16, k=4, dx=FAKE, ts=None):
        return rc("moe_router_backward", FAKE, FAKE, FAKE, FAKE, FAKE, None, T, H, E, k, dx, FAKE, ts,
                  None)
    assert r(k=9) == L.MOE_ERR_INVALID and r(E=2) == L.MOE_ERR_INVALID
    assert r(H=100) == L.MOE_ERR_INVALID and r(dx=None) == L.MOE_ERR_INVALID
    assert r(dx=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    assert r(ts=ctypes.c_void_p(4098)) == L.MOE_ERR_INVALID and "topk_s" in L.last_error()
    assert r(T=0, dx=None) == L.MOE_OK
    def d(E=16, H=256, out=FAKE):
        return rc("moe_router_dcentroids", FAKE, FAKE, FAKE, FAKE, 4, H, E, out, None)
    assert d(E=0) == L.MOE_ERR_INVALID and d(H=12) == L.MOE_ERR_INVALID and d(out=None) == L.MOE_ERR_INVALID


def test_gemm_validation():
    def f(G, M, N, K, A=FAKE, idx=None, A_rows=None):
        A_rows = M if A_rows is None else A_rows
        return rc("grouped_fp8_gemm", A, FAKE, idx, A_rows, FAKE, FAKE, FAKE, G, M, N, K, FAKE, None)
    assert f(0, 10, 128, 128) == L.MOE_ERR_INVALID
    assert f(5000, 10, 128, 128) == L.MOE_ERR_UNSUPPORTED   # more groups than the LDS tables hold
    assert f(4, 10, 100, 128) == L.MOE_ERR_INVALID and "N=100" in L.last_error()
    assert f(4, 10, 128, 200) == L.MOE_ERR_INVALID and "K=200" in L.last_error()
    assert f(4, -1, 128, 128) == L.MOE_ERR_INVALID
    assert f(4, 10, 128, 128, A=None) == L.MOE_ERR_INVALID
    assert f(4, 0, 128, 128, A=None) == L.MOE_OK          # empty problem is a no-op
    # A_rows: at least M_total rows without a row index, at least one with it
    assert f(4, 10, 128, 128, A_rows=9) == L.MOE_ERR_INVALID and "A_rows" in L.last_error()
    assert f(4, 10, 128, 128, idx=FAKE, A_rows=0) == L.MOE_ERR_INVALID
    assert f(4, 10, 128, 128, idx=FAKE, A_rows=1 << 31) == L.MOE_ERR_INVALID


def test_route_validation():
    def f(T=64, H=256, E=16, ng=4, tg=2, k=4, ws=FAKE, wsb=1 << 30, ts=None):
        return rc("moe_route", FAKE, T, H, FAKE, FAKE, E, ng, tg, k, FAKE, FAKE, FAKE, ws, wsb, ts,
                  None)
    assert f(H=200) == L.MOE_ERR_INVALID
    assert f(E=18, ng=4) == L.MOE_ERR_INVALID and "n_group" in L.last_error()
    assert f(tg=5) == L.MOE_ERR_INVALID
    assert f(k=9) == L.MOE_ERR_INVALID                       # k > topk_group * group size
    assert f(E=512, ng=8, tg=4, k=8) == L.MOE_ERR_UNSUPPORTED
    assert f(E=256, ng=8, tg=4, k=16) == L.MOE_ERR_UNSUPPORTED
    assert f(E=24, ng=4, tg=2, k=4) == L.MOE_ERR_UNSUPPORTED  # group size 6
    assert f(E=16, ng=16, tg=2, k=2) == L.MOE_ERR_INVALID      # group size 1: no top-2 sum
    assert f(wsb=16) == L.MOE_ERR_WORKSPACE
    assert f(ws=None) == L.MOE_ERR_WORKSPACE
    assert f(ts=ctypes.c_void_p(4098)) == L.MOE_ERR_INVALID and "topk_s" in L.last_error()


def test_route_scores_and_seq_balance_validation():
    def r(T=64, sc=FAKE, ss=FAKE, k=4):
        return rc("moe_route_scores", FAKE, T, 256, FAKE, FAKE, 16, 4, 2, k, FAKE, FAKE, FAKE, FAKE,
                  1 << 30, sc, ss, None, None)
    assert r(sc=None) == L.MOE_ERR_INVALID and "scores" in L.last_error()
    assert r(ss=None) == L.MOE_ERR_INVALID
    assert r(sc=ctypes.c_void_p(4100)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    assert r(k=9) == L.MOE_ERR_INVALID                       # moe_route's own checks still apply
    # workspace: two [B, chunks of 64 tokens, E] planes, 256-byte rounded
    assert L.moe_seq_balance_workspace_bytes(0, 256, 4096) == 0
    assert L.moe_seq_balance_workspace_bytes(16384, 256, 4096) == 2 * 4 * 64 * 256 * 4
    assert L.moe_seq_balance_workspace_bytes(100, 16, 64) == 2 * 256 * ((2 * 1 * 16 * 4 + 255) // 256)
    def b(T=100, E=16, k=4, L_=64, ws=FAKE, wsb=1 << 20, out=FAKE):
        return rc("moe_seq_balance", FAKE, FAKE, FAKE, T, E, k, L_, 1e-4, out, FAKE, FAKE, ws, wsb,
                  None)
    assert b(E=0) == L.MOE_ERR_INVALID and b(E=257) == L.MOE_ERR_INVALID
    assert b(k=17) == L.MOE_ERR_INVALID and b(k=0) == L.MOE_ERR_INVALID
    assert b(L_=0) == L.MOE_ERR_INVALID and b(L_=65537) == L.MOE_ERR_INVALID
    assert b(out=None) == L.MOE_ERR_INVALID
    assert b(wsb=64) == L.MOE_ERR_WORKSPACE and b(ws=None) == L.MOE_ERR_WORKSPACE
    assert b(T=0, out=None, ws=None) == L.MOE_OK


def test_router_backward_dense_validation():
    def d(T=64, H=256, E=16, k=4, L_=32, dxo=FAKE, dC=FAKE, ws=FAKE, wsb=1 << 30, dxi=None):
        return rc("moe_router_backward_dense", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, H, E, k,
                  L_, 1e-4, dxi, dxo, dC, FAKE, ws, wsb, None)
    assert d(E=24) == L.MOE_ERR_INVALID and d(E=272) == L.MOE_ERR_INVALID
    assert d(k=9) == L.MOE_ERR_INVALID and d(H=192) == L.MOE_ERR_INVALID
    assert d(L_=0) == L.MOE_ERR_INVALID and d(dC=None) == L.MOE_ERR_INVALID
    assert d(dxo=None) == L.MOE_ERR_INVALID
    assert d(dxi=FAKE) == L.MOE_ERR_INVALID and "alias" in L.last_error()
    assert d(dxo=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID and "aligned" in L.last_error()
    # slices of ~1024 tokens, at most 16; one slice needs no workspace
    assert L.moe_router_backward_dense_workspace_bytes(1000, 256, 16) == 0
    assert L.moe_router_backward_dense_workspace_bytes(16384, 7168, 256) == 16 * 256 * 7168 * 4
    assert L.moe_router_backward_dense_workspace_bytes(2000, 256, 16) == 2 * 16 * 256 * 4
    assert d(T=2000, wsb=16) == L.MOE_ERR_WORKSPACE


def test_swiglu_keep_validation():
    def k(I=256, GU=FAKE, M=100):
        return rc("grouped_fp8_gemm_swiglu_keep", FAKE, FAKE, None, M, FAKE, FAKE, FAKE, 4, M, I,
                  1024, FAKE, FAKE, GU, None)
    assert k(I=200) == L.MOE_ERR_INVALID
    assert k(GU=None) == L.MOE_ERR_INVALID and "GU" in L.last_error()
    assert k(GU=ctypes.c_void_p(4104)) == L.MOE_ERR_INVALID
    assert k(M=0, GU=None) == L.MOE_OK


def test_route_group_size_two_is_valid_shape():
    # E=16 in 8 groups has group size 2: valid, but 2 is not 4 * 2^n
    assert rc("moe_route", FAKE, 8, 256, FAKE, FAKE, 16, 8, 2, 4, FAKE, FAKE, FAKE, FAKE, 1 << 30,
              None, None) == L.MOE_ERR_UNSUPPORTED


def test_permute_and_combine_and_bias_validation():
    p = lambda T=10, k=8, E=256, ns=1, ws=FAKE, wsb=1 << 20: rc(
        "moe_permute", FAKE, FAKE, T, k, E, ns, FAKE, FAKE, FAKE, None, None, 7168, None, None,
        ws, wsb, None)
    assert p(k=9) == L.MOE_ERR_INVALID
    assert p(ns=2) == L.MOE_ERR_INVALID
    assert p(E=5000) == L.MOE_ERR_INVALID
    assert p(wsb=8) == L.MOE_ERR_WORKSPACE
    c = lambda T=4, k=8, H=7168: rc("moe_combine", FAKE, FAKE, FAKE, None, T, k, H, FAKE, None)
    assert c(H=7) == L.MOE_ERR_INVALID
    assert c(k=0) == L.MOE_ERR_INVALID
    assert c(T=0) == L.MOE_OK
    assert rc("moe_bias_update", FAKE, FAKE, 0, ctypes.c_float(0.001), None) == L.MOE_ERR_INVALID
    assert rc("moe_bias_update", None, FAKE, 256, ctypes.c_float(0.001), None) == L.MOE_ERR_INVALID


def test_workspace_sizes():
    assert L.moe_permute_workspace_bytes(16384, 8, 256) == 256 * 256 * 4
    assert L.moe_permute_workspace_bytes(0, 8, 256) == 0
    # router: partial logits [splits, T, E] fp32 (256-byte aligned); large
    # batches (4 splits here) also hold the three bf16 planes of the centroids
    assert L.moe_route_workspace_bytes(16384, 7168, 256) == 4 * 16384 * 256 * 4 + 3 * 256 * 7168 * 2
    b = L.moe_route_workspace_bytes(128, 7168, 256)
    assert b % (128 * 256 * 4) == 0 and b >= 128 * 256 * 4
