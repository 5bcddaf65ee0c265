"""Host-side checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import quantized_mixture_experts_router_amd as moeq
from quantized_mixture_experts_router_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "moeq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(moeq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_status_strings():
    L = _lib.LIB
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(-4) == b"workspace too small"


def test_workspace_size_empty_and_decode_shapes():
    # T = 0 and every decode shape of the workloads size without error
    for T in (0, 1, 8, 16, 32, 64):
        for (H, I, E, k) in ((4096, 14336, 8, 2), (2048, 512, 256, 6), (8192, 16384, 64, 2), (256, 128, 8, 2)):
            for act in (0, 2):
                assert moeq.workspace_size(T, H, I, E, k, act) >= 256


def test_workspace_size_monotone():
    a = moeq.workspace_size(16, 4096, 14336, 8, 2)
    b = moeq.workspace_size(2048, 4096, 14336, 8, 2)
    c = moeq.workspace_size(2048, 4096, 14336, 8, 2, moeq.ACT_I8_XH)
    assert 0 < a < b < c


def _route(**kw):
    a = dict(x=16, xdt=1, Wr=16, b=None, T=4, H=64, E=8, k=2, ids=16, w=16, logits=None,
             ws=256, ws_bytes=1 << 20)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return _lib.LIB.moe_route(p(a["x"]), a["xdt"], p(a["Wr"]), p(a["b"]), a["T"], a["H"], a["E"],
                              a["k"], p(a["ids"]), p(a["w"]), p(a["logits"]), p(a["ws"]),
                              a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), -1), (dict(k=9), -1), (dict(E=0), -1), (dict(E=257, k=2), -1),
    (dict(H=60), -1), (dict(xdt=7), -1), (dict(x=None), -1), (dict(ids=None), -1),
    (dict(x=17), -3), (dict(T=-1), -1), (dict(k=33, E=64), -1), (dict(ws=None), -1),
    (dict(ws=272), -3), (dict(ws_bytes=0), -4),
])
def test_route_rejects(kw, status):
    assert _route(**kw) == status


def test_route_empty_is_noop():
    assert _route(T=0, x=None, ids=None, w=None, ws=None) == 0


def test_route_workspace_size():
    L = _lib.LIB
    assert L.moe_route_workspace_size(0, 2048, 256) == 0
    for T, H, E in ((1, 4096, 8), (64, 2048, 256), (4096, 2048, 256), (16, 8192, 64), (5, 136, 20)):
        n = L.moe_route_workspace_size(T, H, E)
        # at least the fp64 logits themselves, 256-byte granular
        assert n >= T * E * 8 and n % 256 == 0
        # the layer workspace holds the router's partial logits too
        if H % 128 == 0:
            assert moeq.workspace_size(T, H, 512, E, 2) >= n


def test_permute_workspace_size():
    L = _lib.LIB
    # one block (the flag block only) up to 8192 assignments, then per-block counts
    assert L.moe_permute_workspace_size(4096, 2, 8) == 256
    assert L.moe_permute_workspace_size(8192, 1, 256) == 256
    assert L.moe_permute_workspace_size(8193, 1, 256) > 256
    big = L.moe_permute_workspace_size(4096, 8, 256)
    assert big >= 256 + 16 * 256 * 4
    assert L.moe_permute_workspace_size(-1, 2, 8) == 0
    # the layer workspace holds it (the layer may be driven through the split calls)
    assert moeq.workspace_size(4096, 2048, 512, 256, 8) >= big
    # a workspace big enough for the flag word only is refused above one block
    p = ctypes.c_void_p(256)
    assert L.moe_permute(p, 4096, 8, 256, p, p, p, p, p, 256, None) == -4
    assert L.moe_permute(p, 1 << 20, 1 << 11, 256, p, p, p, p, p, 1 << 30, None) == -1


def _canon(fmt=1, bits=4, group=32, I=256, H=256, codes=256, params=256, down_bits=None,
           up_bits=None, n_out=0, outliers=0):
    q = lambda r, c, b: _lib.QMatC(fmt, b, group, r, c, n_out, codes, params, outliers or None)
    return _lib.ExpertCanonC(q(I, H, bits), q(I, H, up_bits or bits), q(H, I, down_bits or bits))


@pytest.mark.parametrize("kw,ok", [
    (dict(), True), (dict(bits=3), True), (dict(bits=5), False), (dict(group=48), False),
    (dict(fmt=3), False),
    (dict(fmt=2, bits=2), False), (dict(I=100), False), (dict(codes=8), False),
    (dict(params=2), False), (dict(codes=0), False), (dict(fmt=2, group=16), True),
    (dict(bits=2, group=16), True), (dict(down_bits=2), True), (dict(up_bits=3), True),
    (dict(I=65536, H=65536), False),  # beyond 32-bit offsets into a packed matrix
    (dict(n_out=10, outliers=256), True), (dict(n_out=10), False),  # outlier list missing
    (dict(n_out=10, outliers=260), False),                          # misaligned list
    (dict(n_out=256 * 256 + 1, outliers=256), False),               # more than the matrix
])
def test_packed_bytes_validation(kw, ok):
    ec = _canon(**kw)
    n = _lib.LIB.moe_packed_expert_bytes(ctypes.byref(ec))
    assert (n > 0) == ok


def test_packed_bytes_value():
    # asym 4-bit g32: codes 0.5 B/weight; params (s, m) 4 B per 32 weights
    ec = _canon(I=512, H=256)
    n = _lib.LIB.moe_packed_expert_bytes(ctypes.byref(ec))
    w = 3 * 512 * 256
    assert n == w // 2 + w // 32 * 4
    # 3-bit g32: 3/8 B/weight of codes, the same params
    ec = _canon(I=512, H=256, bits=3)
    assert _lib.LIB.moe_packed_expert_bytes(ctypes.byref(ec)) == w * 3 // 8 + w // 32 * 4
    # gate 3-bit, up 2-bit, down 4-bit: separate gate and up streams
    ec = _canon(I=512, H=256, bits=3, up_bits=2, down_bits=4)
    m = 512 * 256
    assert _lib.LIB.moe_packed_expert_bytes(ctypes.byref(ec)) == \
        m * 3 // 8 + m * 2 // 8 + m * 4 // 8 + 3 * (m // 32 * 4)
    # outliers: per matrix group a row-pointer array and 8-byte entries (each
    # part 256-byte aligned)
    al = lambda v: (v + 255) // 256 * 256
    ec = _canon(I=512, H=256, n_out=100, outliers=256)
    assert _lib.LIB.moe_packed_expert_bytes(ctypes.byref(ec)) == \
        w // 2 + w // 32 * 4 + al((2 * 512 + 1) * 4) + al(200 * 8) + al((256 + 1) * 4) + al(100 * 8)


def test_format_mask_split_bit():
    d = (_lib.PackedExpertC * 2)()
    d[0].gu_fmt, d[0].gu_bits, d[0].gu_group = 1, 3, 32
    d[0].up_fmt, d[0].up_bits, d[0].up_group = 1, 2, 16
    d[0].dn_fmt, d[0].dn_bits, d[0].dn_group = 1, 4, 32
    d[0].layout = _lib.PACK_SPLIT_GU
    for x in (d[1],):
        x.gu_fmt, x.gu_bits, x.gu_group = 2, 4, 16
        x.up_fmt, x.up_bits, x.up_group = 2, 4, 16
        x.dn_fmt, x.dn_bits, x.dn_group = 2, 4, 16
    m = _lib.LIB.moe_format_mask(d, 2)
    # ids 4c+g: asym 3-bit c=4 g32 -> 17; asym 2-bit g16 -> 4; asym 4-bit g32 -> 1; e2m1 g16 -> 8
    assert m == (1 << 17) | (1 << 4) | (1 << 1) | (1 << 8) | _lib.MASK_SPLIT_GU | _lib.MASK_NO_FUSE
    # without the split expert: no layout bits
    assert _lib.LIB.moe_format_mask(ctypes.byref(d[1]), 1) == 1 << 8
    # an outlier list (either group) sets the outlier bit and keeps the
    # fused decode kernel away
    d[1].n_out_dn = 3
    assert _lib.LIB.moe_format_mask(ctypes.byref(d[1]), 1) == \
        (1 << 8) | _lib.MASK_OUTLIERS | _lib.MASK_NO_FUSE
    d[1].n_out_dn, d[1].n_out_gu = 0, 7
    assert _lib.LIB.moe_format_mask(ctypes.byref(d[1]), 1) == \
        (1 << 8) | _lib.MASK_OUTLIERS | _lib.MASK_NO_FUSE


def test_ffn_rejects_small_workspace():
    L = _lib.LIB
    p = ctypes.c_void_p(256)
    need = L.moe_workspace_size(8, 256, 256, 4, 2, 0)
    assert L.moe_ffn_gate_up(p, 0, p, 8, 256, 256, 4, 2, 0, p, need - 1, None) == -4
    assert L.moe_ffn_gate_up(p, 0, p, 8, 256, 256, 4, 2, 0, ctypes.c_void_p(260), need, None) == -3
    assert L.moe_ffn_gate_up(p, 0, p, 8, 200, 256, 4, 2, 0, p, need, None) == -1
    assert L.moe_ffn_gate_up(None, 0, p, 8, 256, 256, 4, 2, 0, p, need, None) == -1
    assert L.moe_ffn_gather(p, 1, p, 8, 256, 256, 4, 2, 0, p, need - 1, None) == -4
    assert L.moe_ffn_gather(p, 1, None, 8, 256, 256, 4, 2, 0, p, need, None) == -1
    assert L.moe_ffn_down(p, 0, p, 8, 256, 256, 4, 2, 3, p, p, need, None) == -1
    # expert inputs beyond 32-bit byte offsets: T*k*max(H, I)*2 >= 2^32
    assert L.moe_ffn_gate_up(p, 0, p, 1 << 19, 4096, 4096, 8, 2, 0, p, 1 << 62, None) == -2
    # Y is stored 16 bytes per lane
    assert L.moe_ffn_down(p, 0, p, 8, 256, 256, 4, 2, 0, ctypes.c_void_p(264), p, need, None) == -3
    assert L.moe_ffn_gather(p, 1, None, 0, 256, 256, 4, 2, 0, p, need, None) == 0


def test_layer_forward_rejects():
    L = _lib.LIB
    p = ctypes.c_void_p(256)
    ws = L.moe_workspace_size(4, 256, 256, 8, 2, 0)
    # k > E
    assert L.moe_layer_forward(p, 1, p, None, p, 0, 4, 256, 256, 8, 9, 0, p, 0, None, None, p, ws, None) == -1
    # bad activation mode
    assert L.moe_layer_forward(p, 1, p, None, p, 0, 4, 256, 256, 8, 2, 5, p, 0, None, None, p, ws, None) == -1
    # bad output dtype
    assert L.moe_layer_forward(p, 1, p, None, p, 0, 4, 256, 256, 8, 2, 0, p, 9, None, None, p, ws, None) == -1
    # T = 0 is a no-op
    assert L.moe_layer_forward(p, 1, p, None, p, 0, 0, 256, 256, 8, 2, 0, p, 0, None, None, p, ws, None) == 0


def test_plan_tiers_matches_oracle():
    # host-only entry point: no device work, so it runs here
    import numpy as np
    import oracle
    rng = np.random.default_rng(21)
    for _ in range(300):
        E = int(rng.integers(1, 300))
        nt = int(rng.integers(1, 5))
        tb = sorted((int(b) for b in rng.integers(1, 1 << 30, size=nt)), reverse=True)
        counts = rng.integers(0, int(rng.integers(1, 50)), size=E)
        budget = int(rng.integers(E * tb[-1], E * tb[0] + 2))
        got, used = moeq.plan_tiers(counts, tb, budget)
        want, wused = oracle.plan_tiers(counts, tb, budget)
        np.testing.assert_array_equal(got, want)
        assert used == wused


def test_plan_tiers_rejects():
    import numpy as np
    L = _lib.LIB
    counts = np.array([3, 1, 2], dtype=np.int64)
    out = np.zeros(3, dtype=np.int32)

    def call(c=counts, E=3, tb=(10, 5), budget=30, o=out):
        t = np.ascontiguousarray(np.asarray(tb, dtype=np.uint64))
        return L.moe_plan_tiers(None if c is None else c.ctypes.data, E,
                                None if t.size == 0 else t.ctypes.data, t.size,
                                ctypes.c_uint64(budget), None if o is None else o.ctypes.data, None)

    assert call() == 0
    assert call(c=None) == -1
    assert call(o=None) == -1
    assert call(E=0) == -1
    assert call(tb=()) == -1
    assert call(tb=(5, 10)) == -1                    # not most precise first
    assert call(tb=((1 << 40) + 1, 5)) == -1          # tier too large
    assert call(budget=14) == -1                      # 3 experts at 5 B exceed 14 B
    out[:] = 7
    assert call(budget=14) == -1 and list(out) == [7, 7, 7]  # untouched on failure
    assert call(c=np.array([3, -1, 2], dtype=np.int64)) == -1
    assert call(budget=15) == 0 and list(out) == [1, 1, 1]


def test_expert_histogram_rejects():
    L = _lib.LIB
    p = ctypes.c_void_p
    assert L.moe_expert_histogram(p(16), 4, 2, 8, None, None) == -1
    assert L.moe_expert_histogram(p(16), 4, 0, 8, p(16), None) == -1
    assert L.moe_expert_histogram(p(16), 4, 2, 257, p(16), None) == -1
    assert L.moe_expert_histogram(p(16), -1, 2, 8, p(16), None) == -1
    assert L.moe_expert_histogram(p(16), 4, 2, 8, p(12), None) == -3


def test_router_i8_params_matches_oracle():
    import numpy as np
    import oracle
    rng = np.random.default_rng(41)
    for shared in (False, True):
        for _ in range(50):
            E = int(rng.integers(1, 257))
            lo = rng.uniform(-5, 2, size=E)
            hi = lo + rng.choice([0.0, 1e-3, 1.0, 7.0], size=E)
            s, z = moeq.router_i8_params(lo, hi, shared)
            s0, z0 = oracle.router_i8_params(lo, hi, shared)
            np.testing.assert_array_equal(s, s0)
            np.testing.assert_array_equal(z, z0)


def test_router_i8_rejects():
    import numpy as np
    L = _lib.LIB
    lo = np.zeros(4)
    hi = np.ones(4)
    s = np.zeros(4, dtype=np.float32)
    z = np.zeros(4, dtype=np.int32)
    call = lambda lo_, hi_, E=4: L.moe_router_i8_params(lo_.ctypes.data, hi_.ctypes.data, E, 0,
                                                        s.ctypes.data, z.ctypes.data)
    assert call(lo, hi) == 0
    assert call(hi, lo) == -1                       # lo > hi
    assert call(lo, np.array([1, 1, np.nan, 1.0])) == -1
    assert call(lo, hi, E=0) == -1
    p = ctypes.c_void_p
    # route_i8 / logit range check their arguments like moe_route
    assert L.moe_route_i8(p(16), 1, p(16), None, 4, 64, 8, 0, p(16), p(16), p(16), p(16), None,
                          p(256), 1 << 20, None) == -1          # k = 0
    assert L.moe_route_i8(p(16), 1, p(16), None, 4, 64, 8, 2, None, p(16), p(16), p(16), None,
                          p(256), 1 << 20, None) == -1          # no scale
    assert L.moe_route_i8(p(16), 1, p(16), None, 4, 64, 8, 2, p(16), p(16), p(16), p(16), None,
                          p(256), 0, None) == -4                # workspace
    assert L.moe_router_logit_range(p(16), 1, p(16), None, 4, 64, 8, None, p(16), p(256), 1 << 20,
                                    None) == -1
    assert L.moe_router_logit_range(p(16), 1, p(16), None, 4, 64, 8, p(12), p(16), p(256), 1 << 20,
                                    None) == -3
    assert L.moe_router_logit_range(p(16), 1, p(16), None, 0, 64, 8, None, None, None, 0, None) == 0


def test_package_never_uses_the_oracle():
    """The library and its binding share no code with the oracle: no source
    under the package names it, and importing the package loads no oracle
    module."""
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "quantized_mixture_experts_router_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, f)
    code = ("import sys, quantized_mixture_experts_router_amd as m; "
            "print(any(k == 'oracle' or k.startswith('oracle.') for k in sys.modules))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "False"


def test_package_fails_loudly_without_the_library():
    import subprocess
    import sys
    env = dict(os.environ, MOEQ_LIBRARY=os.path.join(ROOT, "no-such-libmoeq.so"))
    out = subprocess.run([sys.executable, "-c", "import quantized_mixture_experts_router_amd"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert out.returncode != 0
    assert "ImportError" in out.stderr and "no-such-libmoeq.so" in out.stderr


def test_stream_read_shaped_rejects_shapes_on_host():
    """Launch shapes outside the documented ranges are refused before any
    device call (null buffers stand in for device memory); an empty read
    with a valid shape is a no-op; a valid shape with a null buffer is refused."""
    f = _lib.LIB.moe_stream_read_shaped
    vp = ctypes.c_void_p
    bad = [(0, 4, 8, 0), (65537, 4, 8, 0), (8, 0, 8, 0), (8, 17, 8, 0), (8, 4, 3, 0),
           (8, 4, 0, 0), (8, 4, 32, 0), (8, 4, 8, 2), (8, 4, 8, -1)]
    for blocks, waves, inflight, layout in bad:
        assert f(vp(None), 16, 1, blocks, waves, inflight, layout, vp(None), vp(None)) == -1
    assert f(vp(None), 0, 1, 256, 4, 16, 1, vp(None), vp(None)) == 0
    assert f(vp(None), 16, 0, 256, 4, 16, 1, vp(None), vp(None)) == -1
    assert f(vp(16), 24, 0, 256, 4, 16, 1, vp(64), vp(None)) == -1   # bytes % 16
    assert f(vp(8), 16, 0, 256, 4, 16, 1, vp(64), vp(None)) == -3    # src alignment
