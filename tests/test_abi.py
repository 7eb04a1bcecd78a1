"""The C-ABI library loads, exports every entry point include/jt.h declares,
and rejects invalid arguments on the host before touching the device (no
compute call happens here; these run without a GPU)."""
import ctypes
import os
import re

import pytest

from tree_causal_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jt.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(jt_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from tree_causal_attention_amd import build
        build.build()
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"jt_build_tree", "jt_tree_meta", "jt_tree_attention", "jt_accept"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SIGNATURES), "binding signatures out of sync with jt.h"


def test_status_strings(lib):
    for s in range(6):
        assert lib.jt_status_string(s)
    assert lib.jt_version() >= 100


N = None


def test_build_tree_validation(lib):
    bt = lib.jt_build_tree
    ok_args = dict(dt=0, b=1, n=4, v=100, w=4, bb=16)

    def call(dt=0, b=1, n=4, v=100, w=4, bb=16, ws_bytes=0, ptr=1):
        p = ctypes.c_void_p(ptr) if ptr else None
        return bt(p, dt, b, n, v, w, bb, p, p, p, p, None, p, None, p, ws_bytes, None)

    assert call(w=101) == B.JT_ERR_INVALID_ARG          # W > V
    assert call(n=0) == B.JT_ERR_INVALID_ARG
    assert call(bb=-1) == B.JT_ERR_INVALID_ARG
    assert call(dt=7) == B.JT_ERR_INVALID_ARG
    assert call(w=17, v=1000) == B.JT_ERR_UNSUPPORTED    # W > 16
    assert call(bb=1024) == B.JT_ERR_UNSUPPORTED         # B + 1 > 1024
    assert call(n=65) == B.JT_ERR_UNSUPPORTED
    # the selection state of 64 levels of up to 300 nodes does not fit one
    # workgroup's LDS; 64 levels of up to 120 do (checked before any launch)
    assert call(n=64, v=500, w=2, bb=300) == B.JT_ERR_UNSUPPORTED
    assert call(n=64, v=500, w=2, bb=120, b=0) == B.JT_OK
    assert call(ptr=0) == B.JT_ERR_INVALID_ARG           # null pointers
    assert call(ws_bytes=0) == B.JT_ERR_WORKSPACE        # workspace too small
    assert call(b=0) == B.JT_OK                          # empty batch: nothing to do
    assert lib.jt_build_tree_workspace(1, 4, 100, 4, 16) > 0


def test_tree_meta_validation(lib):
    f = lib.jt_tree_meta
    p = ctypes.c_void_p(1)
    assert f(p, p, 1, 0, p, None, None) == B.JT_ERR_INVALID_ARG
    assert f(p, p, -1, 4, p, None, None) == B.JT_ERR_INVALID_ARG
    assert f(p, p, 1, 1025, p, None, None) == B.JT_ERR_UNSUPPORTED
    assert f(None, p, 1, 4, p, None, None) == B.JT_ERR_INVALID_ARG
    assert f(None, None, 0, 4, None, None, None) == B.JT_OK


def test_tree_attention_validation(lib):
    f = lib.jt_tree_attention
    p = ctypes.c_void_p(1)

    def call(dt=1, b=1, T=17, hq=32, hkv=8, D=128, maxp=8, npages=10, ps=16, scale=1.0, ws=1 << 40,
             ptr=p):
        return f(ptr, ptr, ptr, dt, b, T, hq, hkv, D, ptr, ptr, ptr, maxp, npages, ps, ptr,
                 scale, ptr, None, None, ptr, ws, None)

    assert call(hkv=7) == B.JT_ERR_INVALID_ARG           # Hq % Hkv != 0
    assert call(D=96) == B.JT_ERR_UNSUPPORTED
    assert call(ps=32) == B.JT_ERR_UNSUPPORTED
    assert call(T=1025) == B.JT_ERR_UNSUPPORTED
    assert call(hq=34, hkv=2) == B.JT_ERR_UNSUPPORTED    # group > 16
    assert call(scale=0.0) == B.JT_ERR_INVALID_ARG
    assert call(scale=float("nan")) == B.JT_ERR_INVALID_ARG
    assert call(npages=0) == B.JT_ERR_INVALID_ARG
    assert call(ptr=None) == B.JT_ERR_INVALID_ARG
    assert call(b=0) == B.JT_OK
    need = lib.jt_tree_attention_workspace(1, 17, 32, 8, 128, 8, 16, 1)
    if need:
        assert call(ws=need - 1) == B.JT_ERR_WORKSPACE


def test_accept_validation(lib):
    f = lib.jt_accept
    p = ctypes.c_void_p(1)

    def call(dt=0, b=1, T=17, V=100, N=8, ws=1 << 40, ptr=p):
        return f(ptr, dt, b, T, V, N, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None, ptr, ws, None)

    assert call(T=0) == B.JT_ERR_INVALID_ARG
    assert call(N=0) == B.JT_ERR_INVALID_ARG
    assert call(T=2000) == B.JT_ERR_UNSUPPORTED
    assert call(ptr=None) == B.JT_ERR_INVALID_ARG
    assert call(ws=0) == B.JT_ERR_WORKSPACE
    assert call(b=0) == B.JT_OK


def test_workspace_queries_are_consistent(lib):
    # bigger problems never need less workspace
    a = lib.jt_accept_workspace(1, 257, 151936)
    b = lib.jt_accept_workspace(8, 257, 151936)
    assert 0 < a <= b
    assert lib.jt_tree_attention_workspace(1, 17, 4, 1, 64, 8, 16, 0) == 0   # fp32: no split


def test_accept_margin_validation(lib):
    f = lib.jt_accept_margin
    p = ctypes.c_void_p(1)

    def call(theta=0.5, temp=1.0, dt=0, b=1, T=17, V=100, N=4, ws=0):
        return f(p, dt, b, T, V, N, p, p, p, p, theta, temp, p, p, p, None, p, ws, None)

    assert call(theta=1.1) == B.JT_ERR_INVALID_ARG            # a ratio above 1
    assert call(theta=0.0) == B.JT_ERR_INVALID_ARG
    assert call(theta=float("nan")) == B.JT_ERR_INVALID_ARG
    assert call(temp=0.0) == B.JT_ERR_INVALID_ARG
    assert call(temp=float("inf")) == B.JT_ERR_INVALID_ARG
    assert call(temp=float("nan")) == B.JT_ERR_INVALID_ARG
    assert call(N=0) == B.JT_ERR_INVALID_ARG
    assert call(T=1025) == B.JT_ERR_UNSUPPORTED
    assert call(ws=0) == B.JT_ERR_WORKSPACE
    assert call(b=0) == B.JT_OK


def test_commit_kv_validation(lib):
    f = lib.jt_commit_kv
    p = ctypes.c_void_p(1)

    def call(dt=1, b=1, hkv=2, D=128, maxp=4, npages=8, ps=16, T=17, N=16):
        return f(p, p, dt, b, hkv, D, p, maxp, npages, ps, p, None, T, N, p, p, p, None, None)

    assert call(ps=32) == B.JT_ERR_UNSUPPORTED
    assert call(D=4) == B.JT_ERR_UNSUPPORTED        # 8-byte rows
    assert call(N=65) == B.JT_ERR_UNSUPPORTED
    assert call(hkv=0) == B.JT_ERR_INVALID_ARG
    assert call(dt=3) == B.JT_ERR_INVALID_ARG
    assert call(b=0) == B.JT_OK


def test_accept_stochastic_validation(lib):
    f = lib.jt_accept_stochastic
    p = ctypes.c_void_p(1)

    need = lib.jt_accept_stochastic_workspace(1, 100)
    # 2 x 100 doubles (et, ed) padded to 256 bytes, then one 4096-entry chunk
    # for each of the two pre-pass rows: sum (8) + max (4) + flag (4) +
    # positive count (4) bytes
    assert need == 1792 + 2 * 20

    def call(temp=0.7, dt=1, b=1, T=17, V=100, N=4, ua=p, ws=need, mode=0, draft=p):
        return f(p, draft, dt, b, T, V, N, p, p, p, p, temp, mode, ua, p, p, p, p, None, p, ws,
                 None)

    assert call(temp=0.0) == B.JT_ERR_INVALID_ARG
    assert call(temp=-1.0) == B.JT_ERR_INVALID_ARG
    assert call(temp=float("inf")) == B.JT_ERR_INVALID_ARG
    assert call(temp=float("nan")) == B.JT_ERR_INVALID_ARG
    assert call(dt=2) == B.JT_ERR_INVALID_ARG
    assert call(N=65) == B.JT_ERR_UNSUPPORTED
    assert call(T=1025) == B.JT_ERR_UNSUPPORTED
    assert call(ua=None) == B.JT_ERR_INVALID_ARG
    assert call(ws=need - 1) == B.JT_ERR_WORKSPACE
    assert call(mode=2) == B.JT_ERR_INVALID_ARG
    assert call(mode=1, draft=None) == B.JT_ERR_INVALID_ARG   # sampled children need the draft
    assert call(b=0) == B.JT_OK


def test_build_tree_variant_validation(lib):
    f = lib.jt_build_tree_variant
    p = ctypes.c_void_p(1)
    need = lib.jt_build_tree_workspace(1, 4, 100, 4, 16)

    def call(mode=0, a=0.5, dt=0, b=1, N=4, V=100, W=4, Bn=16, ws=need):
        return f(p, dt, b, N, V, W, Bn, mode, a, p, p, p, p, None, p, None, p, ws, None)

    assert call(mode=2) == B.JT_ERR_INVALID_ARG
    assert call(a=1.5) == B.JT_ERR_INVALID_ARG
    assert call(a=-0.1) == B.JT_ERR_INVALID_ARG
    assert call(a=float("nan")) == B.JT_ERR_INVALID_ARG
    assert call(W=101) == B.JT_ERR_INVALID_ARG
    assert call(N=65) == B.JT_ERR_UNSUPPORTED
    assert call(Bn=1024) == B.JT_ERR_UNSUPPORTED
    assert call(ws=0) == B.JT_ERR_WORKSPACE
    assert call(b=0) == B.JT_OK
