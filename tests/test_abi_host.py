"""The C ABI on a machine without a GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid calls before touching HIP.

No call here reaches a kernel launch: every call either fails validation or runs with
``fdec_test_fail_launches(1)``, which turns the launch into FDEC_ERR_HIP.  Pointers are
fake device addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import memory_bound_decode_add_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fdec.h")

OK, NULL, SHAPE, ALIGN, ALIAS, WS, UNSUP, HIP, ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8

CW4 = F.CW4

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH), reason="libfdec.so not built")


@pytest.fixture(scope="module")
def L():
    return F.lib()


@pytest.fixture
def inject(L):
    L.fdec_test_fail_launches(1)
    yield
    L.fdec_test_fail_launches(0)


@pytest.fixture
def fake():
    return Fake()


class Fake:
    """Disjoint, 4 KB-aligned fake device addresses."""

    def __init__(self):
        self.next = 0x7F0000000000

    def __call__(self, nbytes=1 << 20):
        p = self.next
        self.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return p


def header_symbols():
    """Every entry point declared in include/*.h (fdec.h and the test-only fdec_test.h)."""
    inc = os.path.dirname(HEADER)
    txt = "".join(open(os.path.join(inc, n)).read() for n in sorted(os.listdir(inc)) if n.endswith(".h"))
    return sorted(set(re.findall(r"FDEC_API\s+[\w\s\*]+?\b(fdec_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported_and_bound(L):
    syms = header_symbols()
    assert len(syms) >= 25
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(F.exported_symbols()) == syms


def test_abi_version_matches_header(L):
    v = int(re.search(r"#define FDEC_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.fdec_abi_version() == v


def test_status_strings(L):
    assert L.fdec_status_str(0) == b"FDEC_OK"
    assert L.fdec_status_str(-5) == b"FDEC_ERR_WORKSPACE"
    assert L.fdec_status_str(-99) == b"FDEC_ERR_UNKNOWN"


def test_workspace_queries(L):
    # the unfused product buffer: exactly M*K*N*4 bytes (about 94 MB at K=9216, N=2560)
    assert L.fdec_unfused_gemv_workspace_bytes(0, 1, 9216, 2560) == 94_371_840
    assert L.fdec_unfused_gemv_workspace_bytes(0, 2, 9216, 2560) == 0     # M > 1 unsupported
    assert L.fdec_unfused_gemv_workspace_bytes(1, 1, 9216, 2560) >= 2 * 9216 * 2
    assert L.fdec_w4_gemv_workspace_bytes(65, 1024, 512) == 0            # invalid shape
    assert L.fdec_w4_gemv_workspace_bytes(0, 1024, 512) == 0
    # 17..64 rows: the matrix-core kernel's partial sums hold 32 or 64 rows per K slice,
    # and its K slices shrink with the rows, so the workspace grows with the row blocks
    w16, w32, w64 = (L.fdec_w4_gemv_workspace_bytes(M, 9216, 2560) for M in (16, 32, 64))
    assert 0 < w16 < w32 < w64
    assert L.fdec_w4_gemv_workspace_bytes(17, 9216, 2560) == w32
    assert L.fdec_w4_gemv_workspace_bytes(33, 9216, 2560) == w64
    assert L.fdec_w4_gemv_workspace_bytes(1, 1000, 512) == 0
    # the fused GEMV's own workspace stays far below the product it avoids
    assert L.fdec_w4_gemv_workspace_bytes(1, 9216, 2560) < 0.02 * 94_371_840
    # the layer's own plans (identity gate_up, SwiGLU down) need no more than the GEMV
    # queries, which cover either prologue, plus (from 5 rows, when the gate_up runs on the
    # row-block kernel) y staged by the norm kernel: M x H fp16 and M x H/128 fp32 scales
    for M in (1, 16):
        need = L.fdec_mlp_workspace_bytes(M, 4096, 14336)
        staged = 0 if M < 5 else M * 4096 * 2 + M * (4096 // 128) * 4
        gemv = max(L.fdec_w4_gemv_workspace_bytes(M, 4096, 28672), L.fdec_w4_gemv_workspace_bytes(M, 14336, 4096))
        assert gemv + staged <= need <= gemv + staged + 512
        assert need >= L.fdec_w4_gemv_workspace_bytes(M, 14336, 4096) or M == 1
    assert L.fdec_unfused_add_rmsnorm_workspace_bytes(8192, 4096) >= 2 * 8192 * 4096 * 4


def _norm(L, fake, x=None, r=None, w=None, eps=1e-6, M=4, H=512, h=None, y=None):
    x = fake() if x is None else x
    r = fake() if r is None else r
    w = fake() if w is None else w
    h = fake() if h is None else h
    y = fake() if y is None else y
    return L.fdec_add_rmsnorm(x, r, w, eps, M, H, h, y, None)


def test_add_rmsnorm_validation(L, inject):
    f = Fake()
    assert _norm(L, f, x=0) == NULL
    assert _norm(L, f, H=12) == SHAPE
    assert _norm(L, f, H=16392) == SHAPE
    assert _norm(L, f, M=-1) == SHAPE
    assert _norm(L, f, eps=-1.0) == ARG
    assert _norm(L, f, eps=float("nan")) == ARG
    assert _norm(L, f, x=f() + 8) == ALIGN
    x = f()
    assert _norm(L, f, x=x, y=x) == ALIAS
    r = f()
    assert _norm(L, f, r=r, h=r + 256) == ALIAS           # partial overlap
    assert _norm(L, f, r=r, h=r) == HIP                    # exact alias allowed -> reaches the launch
    assert b"injected" in L.fdec_last_error()
    assert _norm(L, f) == HIP


def test_add_rmsnorm_empty_batch_enqueues_nothing(L):
    f = Fake()
    assert _norm(L, f, M=0) == OK
    assert L.fdec_add_rmsnorm(0, 0, f(), 1e-6, 0, 512, 0, 0, None) == OK   # empty tensors may be NULL
    assert L.fdec_add_rmsnorm(0, 0, 0, 1e-6, 0, 512, 0, 0, None) == NULL


def _w4(fake, K=1024, N=512, q=None, s=None):
    return F.CW4(fake() if q is None else q, fake() if s is None else s, K, N)


def _gemv(L, fake, W=None, g=None, u=None, ld=None, scale=None, res=None, M=1, y=None, ws=None, wsb=None):
    W = _w4(fake) if W is None else W
    need = L.fdec_w4_gemv_workspace_bytes(M, W.K, W.N)
    g = fake() if g is None else g
    u = fake() if u is None else u
    y = fake() if y is None else y
    ws = fake(max(need, 16)) if ws is None else ws
    wsb = need if wsb is None else wsb
    return L.fdec_swiglu_w4_gemv(g, u, W.K if ld is None else ld, ctypes.byref(W), scale, res, M, y, ws, wsb, None)


def test_gemv_validation(L, inject):
    f = Fake()
    assert L.fdec_swiglu_w4_gemv(f(), f(), 1024, None, None, None, 1, f(), f(), 1 << 20, None) == NULL
    assert _gemv(L, f, W=_w4(f, K=1000)) == SHAPE
    assert _gemv(L, f, W=_w4(f, N=500)) == SHAPE
    assert _gemv(L, f, W=_w4(f, q=0)) == NULL
    assert _gemv(L, f, M=0) == SHAPE
    assert _gemv(L, f, M=65) == SHAPE
    assert _gemv(L, f, ld=1000) == SHAPE
    assert _gemv(L, f, ld=1028) == SHAPE
    assert _gemv(L, f, g=f() + 2) == ALIGN
    assert _gemv(L, f, scale=f() + 2) == ALIGN
    assert _gemv(L, f, g=0) == NULL
    g = f()
    assert _gemv(L, f, g=g, y=g + 16) == ALIAS
    W = _w4(f)
    assert _gemv(L, f, W=W, y=W.scales) == ALIAS
    r = f()
    assert _gemv(L, f, res=r, y=r + 32) == ALIAS
    assert _gemv(L, f, res=r, y=r) == HIP                   # y == residual allowed
    # workspace checks (a split-K shape)
    need = L.fdec_w4_gemv_workspace_bytes(1, 9216, 2560)
    if need:
        assert _gemv(L, f, W=_w4(f, K=9216, N=2560), wsb=need - 1) == WS
        assert _gemv(L, f, W=_w4(f, K=9216, N=2560), ws=0) == NULL
    assert _gemv(L, f) == HIP
    assert _gemv(L, f, M=16, ld=2048) == HIP


def _fp4(f, K=1024, N=512, q=None, s=None):
    return F.CFP4(f(K * N // 2) if q is None else q, f(K * N // 16) if s is None else s, K, N)


def test_fp4_gemv_validation(L, inject):
    f = Fake()

    def call(W=None, g=None, u=None, ld=None, scale=None, res=None, M=1, y=None, ws=None, wsb=None):
        W = _fp4(f) if W is None else W
        need = L.fdec_fp4_gemv_workspace_bytes(M, W.K, W.N)
        return L.fdec_swiglu_fp4_gemv(f() if g is None else g, f() if u is None else u, W.K if ld is None else ld,
                                      ctypes.byref(W), scale, res, M, f() if y is None else y,
                                      f(max(need, 16)) if ws is None else ws, need if wsb is None else wsb, None)

    assert L.fdec_swiglu_fp4_gemv(f(), f(), 1024, None, None, None, 1, f(), 0, 0, None) == NULL
    assert call(W=_fp4(f, K=1000)) == SHAPE              # K % 32
    assert call(W=_fp4(f, N=500)) == SHAPE               # N % 8
    assert call(W=_fp4(f, q=0)) == NULL
    assert call(W=_fp4(f, s=f() + 2)) == ALIGN
    assert call(M=0) == SHAPE
    assert call(M=65) == SHAPE
    assert call(W=_fp4(f, K=16416, N=8)) == UNSUP        # M <= 4 takes K <= 16384
    assert call(M=5, W=_fp4(f, K=96, N=8)) == UNSUP      # M > 4 takes K % 128 == 0
    assert L.fdec_fp4_gemv_workspace_bytes(1, 9216, 2560) == 0
    need = L.fdec_fp4_gemv_workspace_bytes(16, 9216, 2560)
    assert need > 0                                      # the matrix-core kernel's K slices
    W = _fp4(f, K=9216, N=2560)
    assert call(M=16, W=W, ld=9216, wsb=need - 1) == WS
    assert call(M=16, W=W, ld=9216, ws=0) == NULL
    assert call(M=16, W=W, ld=9216, ws=f() + 8) == ALIGN
    assert call(M=16, W=W, ld=9216) == HIP
    assert call(ld=1000) == SHAPE
    assert call(g=f() + 2) == ALIGN
    assert call(u=0) == NULL
    W = _fp4(f)
    assert call(W=W, y=W.scales) == ALIAS
    r = f()
    assert call(res=r, y=r + 32) == ALIAS
    assert call(res=r, y=r) == HIP                       # y == residual allowed
    assert call() == HIP
    assert call(M=4, ld=2048) == HIP
    # identity prologue and the decode hook
    W = _fp4(f, K=96, N=8)
    assert L.fdec_fp4_gemv(f(), ctypes.byref(W), None, None, 1, f(), 0, 0, None) == HIP
    assert L.fdec_fp4_gemv(f(), None, None, None, 1, f(), 0, 0, None) == NULL
    assert L.fdec_fp4_dequant(ctypes.byref(W), 0, None) == NULL
    assert L.fdec_fp4_dequant(ctypes.byref(W), W.qweight + 64, None) == ALIAS
    assert L.fdec_fp4_dequant(ctypes.byref(W), f(), None) == HIP


def test_fp4a4_validation(L, inject):
    f = Fake()
    W = _fp4(f, K=1024, N=512)
    act, y = f(4), f()

    def call(g=None, u=None, a=act, scale=None, res=None, M=1, yy=y, ws=0, wsb=0):
        return L.fdec_swiglu_fp4a4_gemv(f() if g is None else g, f() if u is None else u, W.K, ctypes.byref(W), a,
                                        scale, res, M, yy, ws, wsb, None)

    assert call() == HIP
    assert call(a=0) == NULL                             # the per-tensor scale is required
    assert call(a=act + 2) == ALIGN
    assert call(a=y + 64) == ALIAS                       # y would overwrite it
    assert call(u=0) == NULL
    assert call(M=0) == SHAPE
    assert L.fdec_fp4a4_gemv(f(), ctypes.byref(W), act, None, None, 1, y, 0, 0, None) == HIP
    assert L.fdec_fp4a4_gemv(f(), ctypes.byref(W), 0, None, None, 1, y, 0, 0, None) == NULL
    assert L.fdec_fp4a4_gemv(f(), None, act, None, None, 1, y, 0, 0, None) == NULL
    # the quantiser hook
    x, c, sc = f(), f(), f()
    assert L.fdec_nvfp4_quantize(x, 1024, 4, 1024, act, c, sc, None) == HIP
    assert L.fdec_nvfp4_quantize(x, 1024, 0, 1024, act, c, sc, None) == OK      # nothing to do
    assert L.fdec_nvfp4_quantize(x, 1024, 4, 1000, act, c, sc, None) == SHAPE   # K % 16
    assert L.fdec_nvfp4_quantize(x, 1000, 4, 1024, act, c, sc, None) == SHAPE   # ldx < K
    assert L.fdec_nvfp4_quantize(x, 1028, 4, 1024, act, c, sc, None) == SHAPE   # ldx % 8
    assert L.fdec_nvfp4_quantize(x + 8, 1024, 4, 1024, act, c, sc, None) == ALIGN
    assert L.fdec_nvfp4_quantize(x, 1024, 4, 1024, 0, c, sc, None) == NULL
    assert L.fdec_nvfp4_quantize(x, 1024, 4, 1024, act, x + 64, sc, None) == ALIAS
    assert L.fdec_nvfp4_quantize(x, 1024, 4, 1024, act, c, c + 16, None) == ALIAS


def test_gemv_split_override_changes_only_the_test_queries(L):
    base = L.fdec_w4_gemv_workspace_bytes(1, 9216, 2560)
    mlp = L.fdec_mlp_workspace_bytes(1, 1536, 8960)
    assert L.fdec_test_gemv_workspace_bytes(1, 9216, 2560) == base
    assert L.fdec_test_mlp_workspace_bytes(1, 1536, 8960) == mlp
    try:
        L.fdec_set_gemv_split(18)
        # the production queries are pure functions of the shapes
        assert L.fdec_w4_gemv_workspace_bytes(1, 9216, 2560) == base
        assert L.fdec_mlp_workspace_bytes(1, 1536, 8960) == mlp
        assert L.fdec_test_gemv_workspace_bytes(1, 9216, 2560) > base
        assert L.fdec_test_mlp_workspace_bytes(1, 1536, 8960) > mlp
        # more than 16 rows: only the matrix-core kernel, whatever the override
        assert L.fdec_test_gemv_workspace_bytes(32, 9216, 2560) == L.fdec_w4_gemv_workspace_bytes(32, 9216, 2560)
    finally:
        L.fdec_set_gemv_split(0)
    assert L.fdec_test_gemv_workspace_bytes(1, 9216, 2560) == base


def test_planned_kernel_per_shape(L):
    """The planner's choice (host code, no GPU): one row and the short-K 1536 x 17920 on the
    column kernel; three and four rows at K = 9216 exceed the column kernel's staging slots
    (4 rows x 18 blocks > 64 tasks) and, with the SwiGLU prologue, run on the matrix cores
    with the waves splitting K, as 5..16 rows with at most about 12 MB of weights do (the
    identity prologue there: split-K; at 5..16 rows with K >= 4096 the waves-split-K
    kernel too); more than 12 MB, or identity at short K, on the ring; more than 16 rows
    on row blocks; rejected shapes -1."""
    k = L.fdec_test_gemv_kernel
    assert k(1, 9216, 2560, 1) == 0
    assert k(2, 9216, 2560, 1) == 0
    assert k(1, 1536, 17920, 0) == 0
    assert k(3, 9216, 2560, 1) == 3
    assert k(4, 9216, 2560, 1) == 3
    assert k(4, 9216, 2560, 0) == 1
    assert k(4, 4096, 2560, 1) == 0
    assert k(8, 9216, 2560, 1) == 3
    assert k(16, 9216, 2560, 1) == 3
    assert k(16, 14336, 4096, 1) == 4
    assert k(16, 8960, 1536, 0) == 3          # identity, K >= 4096, <= 12 MB
    assert k(8, 4096, 4096, 0) == 3
    assert k(16, 1536, 17920, 0) == 4         # identity at short K: the ring
    assert k(16, 14336, 4096, 0) == 4         # identity above 12 MB: the ring
    assert k(32, 9216, 2560, 1) == 2
    assert k(64, 9216, 2560, 1) == 2
    assert k(1, 9216, 2555, 1) == -1          # N % 8
    assert k(1, 9200, 2560, 1) == -1          # K % 128
    try:
        L.fdec_set_gemv_split(18)
        assert k(1, 9216, 2560, 1) == 1       # a forced split leaves the column kernel
    finally:
        L.fdec_set_gemv_split(0)
    assert k(1, 9216, 2560, 1) == 0


def test_forced_split_needs_the_larger_workspace(L, fake, inject):
    # planned once at entry: a call under an override is checked against that plan's workspace
    W = CW4(fake(1 << 24), fake(1 << 20), 9216, 2560)
    g, u, y = fake(), fake(), fake()
    try:
        L.fdec_set_gemv_split(18)
        need = L.fdec_test_gemv_workspace_bytes(1, 9216, 2560)
        assert L.fdec_swiglu_w4_gemv(g, u, 9216, ctypes.byref(W), None, None, 1, y, None, 0, None) == -5
        assert L.fdec_swiglu_w4_gemv(g, u, 9216, ctypes.byref(W), None, None, 1, y, fake(need), need, None) == HIP
    finally:
        L.fdec_set_gemv_split(0)
    assert L.fdec_swiglu_w4_gemv(g, u, 9216, ctypes.byref(W), None, None, 1, y, None, 0, None) == HIP


def test_probe_validation(L, fake, inject):
    assert L.fdec_test_empty_kernel(256, 256, None) == HIP
    assert L.fdec_test_empty_kernel(0, 256, None) == SHAPE
    assert L.fdec_test_empty_kernel(1, 96, None) == SHAPE
    wb, gb, sb = 11_796_480, 18_432, 368_640
    args = lambda wbytes=wb, per=2880, rows=72, rowb=5120, pb=20, wgs=256, sink=None: (  # noqa: E731
        fake(wbytes), wbytes, per, fake(gb), fake(gb), gb, fake(sb), sb, rows, rowb, pb, wgs,
        fake() if sink is None else sink, None)
    assert L.fdec_test_read_ceiling(*args()) == HIP
    assert L.fdec_test_read_ceiling(*args(per=2881)) == SHAPE          # past the weights
    assert L.fdec_test_read_ceiling(*args(rows=73)) == SHAPE           # past the scales
    assert L.fdec_test_read_ceiling(*args(pb=21)) == SHAPE             # past a scale row
    assert L.fdec_test_read_ceiling(*args(per=4097, wbytes=4097 * 256 * 16)) == SHAPE   # beyond the probe
    assert L.fdec_test_read_ceiling(*args(rowb=5128)) == ALIGN
    assert L.fdec_test_read_ceiling(*args(sink=0)) == NULL


def test_unfused_validation(L, inject):
    f = Fake()
    W = _w4(f, K=1024, N=512)
    ws = f(1024 * 512 * 4)
    assert L.fdec_unfused_swiglu_w4_gemv(0, f(), f(), 1024, ctypes.byref(W), None, None, 2, f(), ws,
                                         1 << 30, None) == UNSUP
    assert L.fdec_unfused_swiglu_w4_gemv(7, f(), f(), 1024, ctypes.byref(W), None, None, 1, f(), ws,
                                         1 << 30, None) == ARG
    assert L.fdec_unfused_swiglu_w4_gemv(0, f(), f(), 1024, ctypes.byref(W), None, None, 1, f(), ws,
                                         1024 * 512 * 4 - 1, None) == WS
    assert L.fdec_unfused_swiglu_w4_gemv(0, f(), f(), 1024, ctypes.byref(W), None, None, 1, f(), ws,
                                         1024 * 512 * 4, None) == HIP
    need = L.fdec_unfused_add_rmsnorm_workspace_bytes(4, 512)
    assert L.fdec_unfused_add_rmsnorm(f(), f(), f(), 1e-6, 4, 512, f(), f(), f(need), need - 1, None) == WS
    assert L.fdec_unfused_add_rmsnorm(f(), f(), f(), 1e-6, 4, 512, f(), f(), f(need), need, None) == HIP


def _layer(f, H=512, I=1024, **kw):
    return F.CLayer(f(), kw.get("eps", 1e-6), F.CW4(f(), f(), H, 2 * I), F.CW4(f(), f(), I, H),
                    kw.get("scale", f()), kw.get("resid", 1))


def test_layer_validation(L, inject):
    f = Fake()
    M, H, I = 2, 512, 1024
    need = L.fdec_mlp_workspace_bytes(M, H, I)
    lay = _layer(f, H, I)

    def call(layer=lay, x=None, r=None, yn=None, gu=None, out=None, ws=None, wsb=None, m=M):
        x = f() if x is None else x
        return L.fdec_mlp_decode(ctypes.byref(layer), m, x, f() if r is None else r, f() if yn is None else yn,
                                 f() if gu is None else gu, f() if out is None else out,
                                 f(max(16, need)) if ws is None else ws, need if wsb is None else wsb, None)

    assert call() == HIP
    x = f()
    assert call(x=x, out=x) == HIP                      # out == x allowed
    assert call(x=x, out=x + 16) == ALIAS
    bad = F.CLayer(f(), 1e-6, F.CW4(f(), f(), H, 2 * I), F.CW4(f(), f(), I, H + 128), None, 1)
    assert call(layer=bad) == SHAPE
    bad = F.CLayer(0, 1e-6, F.CW4(f(), f(), H, 2 * I), F.CW4(f(), f(), I, H), None, 1)
    assert call(layer=bad) == NULL
    if need:
        assert call(wsb=need - 1) == WS
    assert call(m=17) == SHAPE
    # chains: only the last layer may add the residual
    arr = (F.CLayer * 2)(_layer(f, H, I, resid=1), _layer(f, H, I, resid=0))
    assert L.fdec_mlp_chain(arr, 2, M, f(), f(), f(), f(), f(max(16, need)), need, None) == ARG
    arr = (F.CLayer * 2)(_layer(f, H, I, resid=0), _layer(f, H, I, resid=1))
    assert L.fdec_mlp_chain(arr, 2, M, f(), f(), f(), f(), f(max(16, need)), need, None) == HIP
    g = ctypes.c_void_p()
    assert L.fdec_mlp_graph_create(arr, 2, M, f(), f(), f(), f(), f(max(16, need)), need, None,
                                   ctypes.byref(g)) == ARG      # null stream cannot be captured
    assert L.fdec_mlp_graph_create(arr, 0, M, f(), f(), f(), f(), f(max(16, need)), need, f(),
                                   ctypes.byref(g)) == SHAPE
    # graph updates check the handle first
    assert L.fdec_mlp_graph_update(None, arr, 2, M, f(), f(), f(), f(), f(max(16, need)), need, f()) == NULL
    assert L.fdec_mlp_graph_update2(None, arr, 2, M, f(), f(), f(), f(max(16, need)), need, f()) == NULL


def test_hooks_validation(L, inject):
    f = Fake()
    W = _w4(f)
    assert L.fdec_w4_unpack(ctypes.byref(W), 0, None) == NULL
    assert L.fdec_w4_unpack(ctypes.byref(W), W.qweight + 64, None) == ALIAS
    assert L.fdec_w4_dequant(ctypes.byref(W), f() + 2, None) == ALIGN
    assert L.fdec_w4_dequant(ctypes.byref(W), f(), None) == HIP
    assert L.fdec_workspace_init(0, 64, None) == NULL
    assert L.fdec_workspace_init(0, 0, None) == OK
    assert L.fdec_graph_launch(None, None) == NULL
    assert L.fdec_graph_destroy(None) == OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        F.add_rmsnorm(x, x.clone(), torch.ones(512, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        F.add_rmsnorm(x.float(), x.clone(), torch.ones(512, dtype=torch.bfloat16))


def test_kernel_sources_have_no_inline_asm():
    # The compiler inserts the wait states between an MFMA and a later instruction that
    # writes the registers the MFMA still reads only for instructions it can see; an
    # inline-asm decode next to MFMAs overwrote an accumulator in flight.  Every device
    # source stays asm-free, and the int4 kernels share one compiler-visible decoder.
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "memory_bound_decode_add_amd", "csrc")
    names = [n for n in os.listdir(csrc) if n.endswith((".hip", ".h", ".cpp"))]
    assert "w4_gemv_mfma.hip" in names and "device_common.h" in names
    for n in names:
        code = re.sub(r"//[^\n]*", "", open(os.path.join(csrc, n)).read())
        assert not re.search(r"\basm\b|__asm__", code), f"inline asm in {n}"
    for n in ("w4_gemv.hip", "w4_gemv_mfma.hip", "unfused.hip"):
        code = open(os.path.join(csrc, n)).read()
        assert "decode_int4x8" in code, n
        assert not re.search(r"__device__[^;{]*\bdecode_int4x8", code), f"{n} defines its own int4 decode"
