"""Host-side checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments before any launch.
None of these tests needs a GPU."""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_02_amd as moe
from quantized_moe_expert_02_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", h)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from quantized_moe_expert_02_amd import build
        build.build()
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert set(moe.EXPORTS) == set(names), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for c in (0, -1, -2, -3, -4, 7):
        assert moe.moe_status_string(c)


DIMS = [synth.Dims(6144, 2048, 256, 8, 1, 0), synth.Dims(2048, 512, 256, 8, 1, 1), synth.Dims(256, 128, 8, 2, 1, 0),
        synth.Dims(6144, 2048, 256, 8, 1, 2), synth.Dims(6144, 2048, 256, 8, 1, 3), synth.Dims(256, 128, 8, 2, 1, 3)]


@pytest.mark.parametrize("d", DIMS)
def test_sizes(L, d):
    pb = moe.moe_packed_bytes(d)
    wbytes = d.inter * d.hidden * 3 * synth.code_bits(d.wfmt) // 8
    assert pb >= wbytes and pb % 256 == 0
    if d.wfmt in synth.ROW_SCALED:
        assert pb - wbytes < 2 * (2 * d.inter + d.hidden) + 4 * 256
    if d == DIMS[0]:
        assert wbytes + 2 * (2 * d.inter + d.hidden) == 18_894_848  # ~19 MB per expert
    for T in (1, 8, 16, 17, 2048):
        assert moe.moe_workspace_bytes(d, T) > moe.moe_workspace_sync_bytes(d) > 0
    assert moe.moe_workspace_bytes(d, 0) > 0


@pytest.mark.parametrize("bad,code", [
    (dict(hidden=100), moe.MOE_E_UNSUPPORTED), (dict(inter=96), moe.MOE_E_UNSUPPORTED),
    (dict(top_k=0), moe.MOE_E_INVAL), (dict(top_k=9, n_experts=8), moe.MOE_E_INVAL),
    (dict(n_experts=2048), moe.MOE_E_UNSUPPORTED), (dict(top_k=40, n_experts=64), moe.MOE_E_UNSUPPORTED),
    (dict(wfmt=4), moe.MOE_E_UNSUPPORTED), (dict(wfmt=-1), moe.MOE_E_UNSUPPORTED), (dict(has_shared=2), moe.MOE_E_INVAL),
    (dict(top_p=-0.1), moe.MOE_E_INVAL), (dict(top_p=1.5), moe.MOE_E_INVAL), (dict(top_p=float("nan")), moe.MOE_E_INVAL)])
def test_bad_dims_rejected(L, bad, code):
    base = dict(hidden=256, inter=128, n_experts=8, top_k=2, has_shared=1, wfmt=0, top_p=0.0)
    base.update(bad)
    d = moe.MoeDims(**base)
    assert moe.moe_packed_bytes(d) == 0
    assert moe.moe_workspace_bytes(d, 4) == 0
    w = moe.MoeWeights(16, 256, 16, None)
    rc = L.moe_w4a16_forward(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(16), 4, ctypes.c_void_p(16),
                             None, None, ctypes.c_void_p(16), 1 << 30, None)
    assert rc == code


def _fwd(L, d, w, x=16, T=4, y=16, ws=16, wsb=1 << 40, ti=None, tw=None):
    return L.moe_w4a16_forward(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(x) if x else None, T,
                               ctypes.c_void_p(y) if y else None, ti, tw, ctypes.c_void_p(ws) if ws else None,
                               wsb, None)


def test_forward_argument_errors(L):
    d = moe.MoeDims(256, 128, 8, 2, 1, 0)
    good = moe.MoeWeights(4096, 8192, 4096, None)
    assert _fwd(L, d, good, T=-1) == moe.MOE_E_INVAL
    assert _fwd(L, d, good, T=0) == moe.MOE_OK  # no-op, nothing launched
    assert _fwd(L, d, good, x=0) == moe.MOE_E_INVAL
    assert _fwd(L, d, good, y=0) == moe.MOE_E_INVAL
    assert _fwd(L, d, good, ws=0) == moe.MOE_E_INVAL
    assert _fwd(L, d, good, x=4097) == moe.MOE_E_INVAL  # misaligned
    assert _fwd(L, d, good, wsb=16) == moe.MOE_E_WORKSPACE
    assert _fwd(L, d, moe.MoeWeights(0, 8192, 4096, None)) == moe.MOE_E_INVAL
    assert _fwd(L, d, moe.MoeWeights(4096, None, 4096, None)) == moe.MOE_E_INVAL  # has_shared but no shared
    assert _fwd(L, d, moe.MoeWeights(4096, 8192 + 16, 4096, None)) == moe.MOE_E_INVAL  # shared not 256-aligned
    d0 = moe.MoeDims(256, 128, 8, 2, 0, 0)
    assert _fwd(L, d0, good) == moe.MOE_E_INVAL  # shared given but has_shared == 0
    assert _fwd(L, d, good, T=1 << 21) == moe.MOE_E_UNSUPPORTED


def test_route_and_pack_argument_errors(L):
    d = moe.MoeDims(256, 128, 8, 2, 1, 0)
    w = moe.MoeWeights(4096, 8192, 4096, None)
    P = ctypes.c_void_p
    rc = L.moe_route(ctypes.byref(d), ctypes.byref(w), P(16), 4, P(16), P(16), P(16), P(16), P(16), None,
                     P(16), 1 << 40, None)
    assert rc == moe.MOE_E_INVAL  # pairs missing
    rc = L.moe_route(ctypes.byref(d), ctypes.byref(w), P(16), 4, P(16), P(16), P(16), P(16), P(16), P(16),
                     P(16), 8, None)
    assert rc == moe.MOE_E_WORKSPACE
    rc = L.moe_route(ctypes.byref(d), ctypes.byref(w), P(16), 0, None, None, None, None, None, None, None, 0, None)
    assert rc == moe.MOE_OK
    rc = L.moe_pack(ctypes.byref(d), P(16), P(16), P(16), P(16), P(16), P(16), None, P(16 + 256), None)
    assert rc == moe.MOE_E_INVAL  # packed_out not 256-aligned
    rc = L.moe_pack(ctypes.byref(d), P(16), None, P(16), P(16), P(16), P(16), None, P(256), None)
    assert rc == moe.MOE_E_INVAL


def test_top_p_accepted_range(L):
    """top_p in [0, 1] is valid (0 and 1 keep all slots); sizes do not depend on it."""
    for p in (0.0, 0.5, 1.0):
        d = moe.MoeDims(256, 128, 8, 2, 1, 0, p)
        assert moe.moe_packed_bytes(d) == moe.moe_packed_bytes(moe.MoeDims(256, 128, 8, 2, 1, 0))
        assert moe.moe_workspace_bytes(d, 4) == moe.moe_workspace_bytes(moe.MoeDims(256, 128, 8, 2, 1, 0), 4)


def test_noalloc_rejects_before_any_launch(L):
    """moe_w4a16_forward_noalloc validates like moe_w4a16_forward and
    rejects batches whose workspace would exceed its fixed scratch with
    MOE_E_WORKSPACE, all before touching the device."""
    d = moe.MoeDims(6144, 2048, 256, 8, 1, 0)
    w = moe.MoeWeights(4096, 8192, 4096, None)
    P = ctypes.c_void_p
    big = next(t for t in range(16, 1 << 14, 16) if moe.moe_workspace_bytes(d, t) > moe.MOE_NOALLOC_SCRATCH_BYTES)
    assert moe.moe_workspace_bytes(d, 118) <= moe.MOE_NOALLOC_SCRATCH_BYTES < moe.moe_workspace_bytes(d, 119)
    f = L.moe_w4a16_forward_noalloc
    assert f(ctypes.byref(d), ctypes.byref(w), P(16), big, P(16), None, None, None) == moe.MOE_E_WORKSPACE
    assert f(ctypes.byref(d), ctypes.byref(w), P(16), 0, P(16), None, None, None) == moe.MOE_OK
    assert f(ctypes.byref(d), ctypes.byref(w), P(16), -1, P(16), None, None, None) == moe.MOE_E_INVAL
    assert f(ctypes.byref(d), ctypes.byref(w), None, 4, P(16), None, None, None) == moe.MOE_E_INVAL
    assert f(ctypes.byref(d), ctypes.byref(w), P(16), 4, P(24), None, None, None) == moe.MOE_E_INVAL
    bad = moe.MoeDims(100, 2048, 256, 8, 1, 0)
    assert f(ctypes.byref(bad), ctypes.byref(w), P(16), 4, P(16), None, None, None) == moe.MOE_E_UNSUPPORTED


def test_step_graph_rejects_before_any_launch(L):
    """moe_step_graph_create validates every layer like moe_w4a16_forward,
    and its own arguments, before it touches the device; *out stays
    untouched on failure; destroy(NULL) is a no-op and launch(NULL) an
    error."""
    d = moe.MoeDims(256, 128, 8, 2, 1, 0)
    P = ctypes.c_void_p
    good = moe.MoeWeights(4096, 8192, 4096, None)
    ws_b = moe.moe_workspace_bytes(d, 4)

    def create(n=2, T=4, w=None, x=None, y=None, ws=P(16), wsb=ws_b, dims=d, out=True):
        ws_arr = (moe.MoeWeights * max(n, 1))(*([w or good] * max(n, 1)))
        xa = (P * max(n, 1))(*(x or [P(1 << 20)] * max(n, 1)))
        ya = (P * max(n, 1))(*(y or [P(2 << 20)] * max(n, 1)))
        h = P(12345)
        rc = L.moe_step_graph_create(ctypes.byref(dims), n, ws_arr, xa, T, ya, ws, wsb,
                                     ctypes.byref(h) if out else None)
        assert h.value == 12345  # untouched on every failure below
        return rc

    assert create(out=False) == moe.MOE_E_INVAL
    assert create(n=0) == moe.MOE_E_INVAL
    assert create(n=moe.MOE_STEP_GRAPH_MAX_LAYERS + 1) == moe.MOE_E_INVAL
    assert create(T=0) == moe.MOE_E_INVAL
    assert create(x=[P(1 << 20), P(0)]) == moe.MOE_E_INVAL  # second layer without an input
    assert create(y=[P(2 << 20), P((2 << 20) + 8)]) == moe.MOE_E_INVAL  # misaligned output
    assert create(wsb=16) == moe.MOE_E_WORKSPACE
    assert create(w=moe.MoeWeights(4096, None, 4096, None)) == moe.MOE_E_INVAL  # has_shared without shared
    assert create(dims=moe.MoeDims(256, 100, 8, 2, 1, 0)) == moe.MOE_E_UNSUPPORTED
    assert L.moe_step_graph_destroy(None) == moe.MOE_OK
    assert L.moe_step_graph_launch(None, None) == moe.MOE_E_INVAL


def test_probe_argument_errors(L):
    """The roofline probes reject bad arguments before any launch."""
    P = ctypes.c_void_p
    assert L.moe_probe_stream_read(None, 1 << 20, P(256), 8, None) == moe.MOE_E_INVAL
    assert L.moe_probe_stream_read(P(256), (1 << 20) + 8, P(256), 8, None) == moe.MOE_E_INVAL  # not 16-byte vectors
    assert L.moe_probe_stream_read(P(264), 1 << 20, P(256), 8, None) == moe.MOE_E_INVAL  # misaligned
    assert L.moe_probe_stream_read(P(256), 1 << 20, P(256), 0, None) == moe.MOE_E_INVAL
    assert L.moe_probe_mfma(None, 8, 10, None) == moe.MOE_E_INVAL
    assert L.moe_probe_mfma(P(256), 0, 10, None) == moe.MOE_E_INVAL
    assert L.moe_probe_mfma(P(256), 8, 0, None) == moe.MOE_E_INVAL
