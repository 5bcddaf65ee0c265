"""ctypes binding of libmoeq.so: argument marshalling only.

Torch tensors provide device memory and the current HIP stream; every step of
the layer runs in the library's HIP kernels. If the shared library is missing
the import of this module fails loudly (there is no fallback path).
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOEQ_LIBRARY may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("MOEQ_LIBRARY") or os.path.join(_HERE, "libmoeq.so")

MOE_OK = 0
MOE_F32, MOE_BF16 = 0, 1
MOE_W_ASYM, MOE_W_E2M1 = 1, 2
ACT_NONE, ACT_I8_X, ACT_I8_XH = 0, 1, 2
FLAG_BAD_EXPERT_ID, FLAG_NAN_LOGIT, FLAG_FORMAT_NOT_LAUNCHED = 1, 2, 4
FLAG_BAD_SEGMENT, FLAG_EXPERT_SHAPE, FLAG_FP16_RANGE = 8, 16, 32
ID_NAN = -2  # routing id of a token whose router logits include a NaN


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)} ({status})")


class QMatC(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_uint8), ("bits", ctypes.c_uint8), ("group", ctypes.c_uint16),
                ("rows", ctypes.c_uint32), ("cols", ctypes.c_uint32),
                ("n_outliers", ctypes.c_uint32),
                ("codes", ctypes.c_void_p), ("params", ctypes.c_void_p),
                ("outliers", ctypes.c_void_p)]


class ExpertCanonC(ctypes.Structure):
    _fields_ = [("gate", QMatC), ("up", QMatC), ("down", QMatC)]


class PackedExpertC(ctypes.Structure):
    _fields_ = [("gu_fmt", ctypes.c_uint8), ("gu_bits", ctypes.c_uint8), ("gu_group", ctypes.c_uint16),
                ("dn_fmt", ctypes.c_uint8), ("dn_bits", ctypes.c_uint8), ("dn_group", ctypes.c_uint16),
                ("H", ctypes.c_uint32), ("I", ctypes.c_uint32),
                ("up_fmt", ctypes.c_uint8), ("up_bits", ctypes.c_uint8), ("up_group", ctypes.c_uint16),
                ("layout", ctypes.c_uint32), ("n_out_gu", ctypes.c_uint32), ("n_out_dn", ctypes.c_uint32),
                ("gu_codes", ctypes.c_void_p), ("gu_params", ctypes.c_void_p),
                ("dn_codes", ctypes.c_void_p), ("dn_params", ctypes.c_void_p),
                ("up_codes", ctypes.c_void_p), ("up_params", ctypes.c_void_p),
                ("out_gu_rowptr", ctypes.c_void_p), ("out_gu_entries", ctypes.c_void_p),
                ("out_dn_rowptr", ctypes.c_void_p), ("out_dn_entries", ctypes.c_void_p),
                ("reserved", ctypes.c_uint64 * 2)]


assert ctypes.sizeof(QMatC) == 40
assert ctypes.sizeof(PackedExpertC) == 128
DESC_BYTES = 128
PACK_SPLIT_GU = 1
MASK_SPLIT_GU = 1 << 31
MASK_NO_FUSE = 1 << 30
MASK_OUTLIERS = 1 << 29
MASK_INT8_GEMM = 1 << 28
MASK_SHARED_TILE = 1 << 27

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "moe_version": ([], _i),
    "moe_status_string": ([_i], ctypes.c_char_p),
    "moe_packed_expert_bytes": ([ctypes.POINTER(ExpertCanonC)], _sz),
    "moe_pack_expert": ([ctypes.POINTER(ExpertCanonC), _vp, _sz, ctypes.POINTER(PackedExpertC), _vp], _i),
    "moe_workspace_size": ([_i, _i, _i, _i, _i, _i], _sz),
    "moe_route_workspace_size": ([_i, _i, _i], _sz),
    "moe_route": ([_vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_permute_workspace_size": ([_i, _i, _i], _sz),
    "moe_permute": ([_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_format_mask": ([ctypes.POINTER(PackedExpertC), _i], ctypes.c_uint32),
    "moe_grouped_ffn_q": ([_vp, _i, _vp, ctypes.c_uint32, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp], _i),
    "moe_ffn_gather": ([_vp, _i, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "moe_ffn_gate_up": ([_vp, ctypes.c_uint32, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "moe_ffn_down": ([_vp, ctypes.c_uint32, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp], _i),
    "moe_combine": ([_vp, _vp, _vp, _i, _i, _i, _vp, _i, _vp], _i),
    "moe_layer_forward": ([_vp, _i, _vp, _vp, _vp, ctypes.c_uint32, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_stream_read": ([_vp, _sz, _i, _vp, _vp], _i),
    "moe_stream_read_shaped": ([_vp, _sz, _i, _i, _i, _i, _i, _vp, _vp], _i),
    "moe_noalloc_scratch_bytes": ([], _sz),
    "moe_layer_forward_noalloc": ([_vp, _i, _vp, _vp, _vp, ctypes.c_uint32, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp], _i),
    "moe_act_quant_i8": ([_vp, _i, _i, _i, _vp, _vp, _vp], _i),
    "moe_expert_histogram": ([_vp, _i, _i, _i, _vp, _vp], _i),
    "moe_plan_tiers": ([_vp, _i, _vp, _i, ctypes.c_uint64, _vp, _vp], _i),
    "moe_router_logit_range": ([_vp, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp], _i),
    "moe_router_i8_params": ([_vp, _vp, _i, _i, _vp, _vp], _i),
    "moe_route_i8": ([_vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python quantized_mixture_experts_router_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


LIB = _load()
EXPORTED = tuple(_SIGS)


def _status_string(s):
    return LIB.moe_status_string(int(s)).decode()


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def version():
    return LIB.moe_version()


def workspace_size(T, H, I, E, k, act=ACT_NONE):
    return int(LIB.moe_workspace_size(T, H, I, E, k, act))


def workspace(T, H, I, E, k, act=ACT_NONE, device="cuda"):
    n = workspace_size(T, H, I, E, k, act)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def read_flags(ws):
    return int(ws[:4].view(torch.int32).item())


# ---------------------------------------------------------------- weights
class DeviceQMat:
    """A canonical block matrix whose planes live in device memory."""

    def __init__(self, fmt, bits, group, rows, cols, codes, params, outliers=None):
        self.fmt, self.bits, self.group, self.rows, self.cols = fmt, bits, group, rows, cols
        self.codes, self.params, self.outliers = codes, params, outliers

    @classmethod
    def from_host(cls, q, device="cuda"):
        """From a host QMat (codes uint8, params uint16, optional outlier
        records uint32 [n, 2] of (index, fp16 bits))."""
        codes = torch.from_numpy(np.ascontiguousarray(q.codes)).to(device)
        params = torch.from_numpy(np.ascontiguousarray(q.params).view(np.int16)).to(device)
        out = getattr(q, "outliers", None)
        outliers = None
        if out is not None and len(out):
            outliers = torch.from_numpy(np.ascontiguousarray(out, dtype=np.uint32).view(np.int32)).to(device)
        return cls(q.fmt, q.bits, q.group, q.rows, q.cols, codes, params, outliers)

    def c(self):
        n = 0 if self.outliers is None else int(self.outliers.shape[0])
        return QMatC(self.fmt, self.bits, self.group, self.rows, self.cols, n,
                     self.codes.data_ptr(), self.params.data_ptr(),
                     None if self.outliers is None else self.outliers.data_ptr())


class PackedExperts:
    """E experts in the device layout plus the device array of descriptors."""

    def __init__(self, buffers, descs, H, I, device="cuda"):
        self.buffers = buffers
        self.descs = descs
        self.H, self.I = H, I
        raw = bytearray(DESC_BYTES * len(descs))
        for i, d in enumerate(descs):
            ctypes.memmove(ctypes.addressof(ctypes.c_char.from_buffer(raw, i * DESC_BYTES)),
                           ctypes.addressof(d), DESC_BYTES)
        self.dev = torch.frombuffer(raw, dtype=torch.uint8).to(device)
        arr = (PackedExpertC * len(descs))(*descs)
        self.fmt_mask = int(LIB.moe_format_mask(arr, len(descs)))

    @property
    def E(self):
        return len(self.descs)

    def nbytes(self):
        return sum(int(b.numel()) for b in self.buffers if b is not None)


def packed_expert_bytes(gate, up, down):
    ec = ExpertCanonC(gate.c(), up.c(), down.c())
    return int(LIB.moe_packed_expert_bytes(ctypes.byref(ec)))


def pack_expert(gate, up, down, device="cuda"):
    """Pack one expert (DeviceQMat gate/up/down) -> (buffer tensor, descriptor)."""
    ec = ExpertCanonC(gate.c(), up.c(), down.c())
    n = int(LIB.moe_packed_expert_bytes(ctypes.byref(ec)))
    if n == 0:
        raise MoeError(-2, "moe_packed_expert_bytes")
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    view = buf[off:off + n]
    d = PackedExpertC()
    _check(LIB.moe_pack_expert(ctypes.byref(ec), _ptr(view), n, ctypes.byref(d), _stream()),
           "moe_pack_expert")
    return buf, d


def pack_experts(get_expert, E, device="cuda"):
    """get_expert(e) -> {"gate","up","down"} host QMats (canonical). Uploads,
    packs and frees the canonical copies one expert at a time."""
    bufs, descs = [], []
    H = I = None
    for e in range(E):
        ex = get_expert(e)
        g = DeviceQMat.from_host(ex["gate"], device)
        u = DeviceQMat.from_host(ex["up"], device)
        dn = DeviceQMat.from_host(ex["down"], device)
        buf, d = pack_expert(g, u, dn, device)
        torch.cuda.current_stream().synchronize()  # canonical planes may be freed now
        del g, u, dn
        bufs.append(buf)
        descs.append(d)
        I, H = ex["gate"].rows, ex["gate"].cols
    return PackedExperts(bufs, descs, H, I, device)


# ---------------------------------------------------------------- layer steps
def route_workspace_size(T, H, E):
    return int(LIB.moe_route_workspace_size(T, H, E))


def route(x, Wr, b, k, want_logits=False, ws=None):
    x, Wr = _dev(x, "x"), _dev(Wr, "Wr")
    T, H = x.shape
    E = Wr.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    if ws is None:
        ws = torch.empty(max(route_workspace_size(T, H, E), 256), dtype=torch.uint8, device=x.device)
    _check(LIB.moe_route(_ptr(x), _dt(x), _ptr(Wr), _ptr(b), T, H, E, k, _ptr(ids), _ptr(w),
                         _ptr(logits), _ptr(ws), ws.numel(), _stream()), "moe_route")
    return (ids, w, logits) if want_logits else (ids, w)


def permute(ids, E, ws=None):
    ids = _dev(ids, "ids")
    T, k = ids.shape
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(256, int(LIB.moe_permute_workspace_size(T, k, E))), dtype=torch.uint8,
                         device=dev)
    _check(LIB.moe_permute(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
                           _ptr(ws), ws.numel(), _stream()), "moe_permute")
    return counts, offsets, perm[:T * k], inv[:T * k], ws


def grouped_ffn(x, packed, offsets, perm, k, act=ACT_NONE, ws=None, Y=None, I=None):
    """moe_grouped_ffn_q. Y: an fp32 device tensor of at least T*k*H elements
    (a new [T*k, H] one if None); I: the intermediate size passed to the
    library (the packed experts' own if None)."""
    x = _dev(x, "x")
    T, H = x.shape
    I = packed.I if I is None else I
    if Y is None:
        Y = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(T, H, I, packed.E, k, act, x.device)
    _check(LIB.moe_grouped_ffn_q(_ptr(x), _dt(x), _ptr(packed.dev), packed.fmt_mask, _ptr(offsets), _ptr(perm), T, H,
                                 I, packed.E, k, act, _ptr(Y), _ptr(ws), ws.numel(), _stream()),
           "moe_grouped_ffn_q")
    return Y


def ffn_gather(x, perm, k, packed, act, ws):
    T, H = x.shape
    _check(LIB.moe_ffn_gather(_ptr(x), _dt(x), _ptr(perm), T, H, packed.I, packed.E, k, act,
                              _ptr(ws), ws.numel(), _stream()), "moe_ffn_gather")


def ffn_gate_up(T, packed, offsets, k, act, ws):
    _check(LIB.moe_ffn_gate_up(_ptr(packed.dev), packed.fmt_mask, _ptr(offsets), T, packed.H, packed.I, packed.E, k,
                               act, _ptr(ws), ws.numel(), _stream()), "moe_ffn_gate_up")


def ffn_down(T, packed, offsets, k, act, Y, ws):
    _check(LIB.moe_ffn_down(_ptr(packed.dev), packed.fmt_mask, _ptr(offsets), T, packed.H, packed.I, packed.E, k, act,
                            _ptr(Y), _ptr(ws), ws.numel(), _stream()), "moe_ffn_down")


def combine(Y, w, inv, T, k, out_dtype=torch.float32):
    H = Y.shape[1]
    out = torch.empty((T, H), dtype=out_dtype, device=Y.device)
    _check(LIB.moe_combine(_ptr(Y), _ptr(w), _ptr(inv), T, H, k, _ptr(out), _dt(out), _stream()),
           "moe_combine")
    return out


def layer_forward(x, Wr, b, packed, k, act=ACT_NONE, out_dtype=torch.float32, ws=None,
                  out=None, ids=None, w=None):
    x, Wr = _dev(x, "x"), _dev(Wr, "Wr")
    T, H = x.shape
    E = Wr.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(T, H, packed.I, E, k, act, x.device)
    _check(LIB.moe_layer_forward(_ptr(x), _dt(x), _ptr(Wr), _ptr(b), _ptr(packed.dev), packed.fmt_mask, T, H, packed.I,
                                 E, k, act, _ptr(out), _dt(out), _ptr(ids), _ptr(w), _ptr(ws),
                                 ws.numel(), _stream()), "moe_layer_forward")
    return out, ids, w


def noalloc_scratch_bytes():
    return int(LIB.moe_noalloc_scratch_bytes())


def layer_forward_noalloc(x, Wr, b, packed, k, act=ACT_NONE, out_dtype=torch.float32, out=None,
                          ids=None, w=None, flags=None):
    """moe_layer_forward_noalloc: the layer on the library's own device scratch
    array. flags: an int32 device tensor of >= 1 element receiving the flag
    word, or None. Output tensors are created here when not given (the
    library call itself allocates nothing)."""
    x, Wr = _dev(x, "x"), _dev(Wr, "Wr")
    T, H = x.shape
    E = Wr.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(LIB.moe_layer_forward_noalloc(_ptr(x), _dt(x), _ptr(Wr), _ptr(b), _ptr(packed.dev),
                                         packed.fmt_mask, T, H, packed.I, E, k, act, _ptr(out),
                                         _dt(out), _ptr(ids), _ptr(w), _ptr(flags), _stream()),
           "moe_layer_forward_noalloc")
    return out, ids, w


def act_quant_i8(v):
    v = _dev(v, "v")
    rows, cols = v.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=v.device)
    s = torch.empty(rows, dtype=torch.float32, device=v.device)
    _check(LIB.moe_act_quant_i8(_ptr(v), _dt(v), rows, cols, _ptr(q), _ptr(s), _stream()),
           "moe_act_quant_i8")
    return q, s


STREAM_BLOCKS = 4096


def stream_read(buf, nontemporal=True, sink=None):
    """Streaming read of a device buffer (measurement aid); returns the
    per-block XOR words (uint32 as int32 tensor)."""
    buf = _dev(buf, "buf")
    if sink is None:
        sink = torch.empty(STREAM_BLOCKS, dtype=torch.int32, device=buf.device)
    _check(LIB.moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(bool(nontemporal)),
                               _ptr(sink), _stream()), "moe_stream_read")
    return sink


def stream_read_shaped(buf, blocks, waves=4, inflight=8, layout=0, nontemporal=True, sink=None):
    """Streaming read with an explicit launch shape (measurement aid); returns
    the per-block XOR words (uint32 as int32 tensor of `blocks` entries)."""
    buf = _dev(buf, "buf")
    if sink is None:
        sink = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    _check(LIB.moe_stream_read_shaped(_ptr(buf), buf.numel() * buf.element_size(),
                                      int(bool(nontemporal)), int(blocks), int(waves),
                                      int(inflight), int(layout), _ptr(sink), _stream()),
           "moe_stream_read_shaped")
    return sink


def expert_histogram(ids, E, hist=None):
    """Adds the per-expert counts of routing ids [T, k] (device int32) into
    hist (device int64 [E], a new zeroed one if None) and returns hist."""
    ids = _dev(ids, "ids")
    T, k = ids.shape
    if hist is None:
        hist = torch.zeros(E, dtype=torch.int64, device=ids.device)
    _check(LIB.moe_expert_histogram(_ptr(ids), T, k, E, _ptr(hist), _stream()),
           "moe_expert_histogram")
    return hist


def plan_tiers(counts, tier_bytes, budget):
    """Precision tier per expert from a routing profile (host only).
    counts: E non-negative ints; tier_bytes: bytes of one expert per tier, most
    precise first. Returns (tier index per expert as int32 array, bytes used)."""
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int64))
    tb = np.ascontiguousarray(np.asarray(tier_bytes, dtype=np.uint64))
    out = np.empty(c.shape[0], dtype=np.int32)
    used = ctypes.c_uint64(0)
    _check(LIB.moe_plan_tiers(c.ctypes.data, c.shape[0], tb.ctypes.data, tb.shape[0],
                              ctypes.c_uint64(int(budget)), out.ctypes.data, ctypes.byref(used)),
           "moe_plan_tiers")
    return out, used.value


def router_logit_range(x, Wr, b, lo=None, hi=None, ws=None):
    """Per-expert running min / max (device fp64 [E]) of the router logits of
    x, merged into lo / hi (new +inf / -inf ones if None); returns (lo, hi)."""
    x, Wr = _dev(x, "x"), _dev(Wr, "Wr")
    T, H = x.shape
    E = Wr.shape[0]
    if lo is None:
        lo = torch.full((E,), float("inf"), dtype=torch.float64, device=x.device)
    if hi is None:
        hi = torch.full((E,), float("-inf"), dtype=torch.float64, device=x.device)
    if ws is None:
        ws = torch.empty(max(route_workspace_size(T, H, E), 256), dtype=torch.uint8, device=x.device)
    _check(LIB.moe_router_logit_range(_ptr(x), _dt(x), _ptr(Wr), _ptr(b), T, H, E, _ptr(lo), _ptr(hi),
                                      _ptr(ws), ws.numel(), _stream()), "moe_router_logit_range")
    return lo, hi


def router_i8_params(lo, hi, shared=False):
    """int8 scale (fp32) and zero point (int32) per expert from a logit range
    (host arrays or tensors); returns numpy arrays."""
    lo = np.ascontiguousarray(np.asarray(lo.cpu() if hasattr(lo, "cpu") else lo, dtype=np.float64))
    hi = np.ascontiguousarray(np.asarray(hi.cpu() if hasattr(hi, "cpu") else hi, dtype=np.float64))
    E = lo.shape[0]
    scale = np.empty(E, dtype=np.float32)
    zero = np.empty(E, dtype=np.int32)
    _check(LIB.moe_router_i8_params(lo.ctypes.data, hi.ctypes.data, E, int(bool(shared)),
                                    scale.ctypes.data, zero.ctypes.data), "moe_router_i8_params")
    return scale, zero


def route_i8(x, Wr, b, k, scale, zero, want_logits=False, ws=None):
    """moe_route with the int8 round trip of the logits (scale fp32 [E],
    zero int32 [E], device tensors)."""
    x, Wr = _dev(x, "x"), _dev(Wr, "Wr")
    scale, zero = _dev(scale, "scale"), _dev(zero, "zero")
    T, H = x.shape
    E = Wr.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    if ws is None:
        ws = torch.empty(max(route_workspace_size(T, H, E), 256), dtype=torch.uint8, device=x.device)
    _check(LIB.moe_route_i8(_ptr(x), _dt(x), _ptr(Wr), _ptr(b), T, H, E, k, _ptr(scale), _ptr(zero),
                            _ptr(ids), _ptr(w), _ptr(logits), _ptr(ws), ws.numel(), _stream()),
           "moe_route_i8")
    return (ids, w, logits) if want_logits else (ids, w)
