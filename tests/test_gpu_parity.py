"""Parity of the HIP path against the CPU oracle, through the C ABI.

Bars: routing ids bit-exact except near-tie tokens (logit gap < 1e-6,
flagged by the oracle); permutation bit-exact; int8 codes and scales
bit-exact; layer outputs within max per-row relative L2 2e-3 (bf16/fp32
activations) or 1e-2 (int8 activations)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from layer_cases import Workload, prefill_order, rel_l2_rows, tolerance, x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moeq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_router_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- routing
ROUTE_CASES = [
    ("tiny", None, None),
    ("mixtral", 96, None),
    ("fine_e2m1", 300, None),
    ("hotcold", 700, None),
    ("w4a8", 64, None),
]


@pytest.mark.parametrize("name,T,_", ROUTE_CASES)
def test_route_parity(moeq, name, T, _):
    cfg = synth.get_config(name)
    T = cfg.T if T is None else T
    _say(f"[route] {name} T={T} H={cfg.H} E={cfg.E} k={cfg.k}")
    x_np = synth.gen_x(cfg, T)
    Wr, b = synth.gen_router(cfg)
    x = x_to_torch(x_np, cfg.x_dtype)
    bt = torch.from_numpy(b).cuda() if cfg.zipf_alpha > 0 else None
    ids, w, logits = moeq.route(x, torch.from_numpy(Wr).cuda(), bt, cfg.k, want_logits=True)
    torch.cuda.synchronize()
    L = oracle.router_logits(oracle.x_to_f64(x_np, cfg.x_dtype), Wr, b if cfg.zipf_alpha > 0 else None)
    rids, rw, gap, flagged = oracle.topk_softmax(L, cfg.k)
    ids, w, logits = ids.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    ok = ~flagged
    np.testing.assert_array_equal(ids[ok], rids[ok])
    assert np.max(np.abs(w[ok] - rw[ok])) <= 1e-6
    assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-6
    assert np.all(np.abs(logits - L) <= 1e-6 * np.maximum(1.0, np.abs(L)))


# shapes chosen to reach every branch of the router's split plan: expert
# tiles per wave 1..4, one or several waves per block (in-block K split),
# several K blocks (partials summed by the top-k), H % 16 == 8 (half chunk),
# T and E off the 16-row tiles
PLAN_CASES = [
    # T, H, E, k, x dtype, bias
    (1, 4096, 8, 2, "bf16", False),      # 1 tile/wave, 16 waves/block, 4 K blocks
    (5, 136, 20, 3, "f32", True),        # half last chunk, ragged T and E
    (33, 264, 40, 4, "bf16", True),      # 3 expert groups, ragged everything
    (16, 8192, 64, 2, "bf16", False),    # 8 K blocks
    (2100, 1024, 256, 8, "bf16", True),  # 4 tiles/wave, in-block split of 4
    (2048, 256, 48, 4, "f32", False),    # 3 tiles/wave
    (2048, 128, 32, 2, "bf16", True),    # 2 tiles/wave
    (4096, 64, 256, 6, "bf16", False),   # one wave per block, no split at all
]


@pytest.mark.parametrize("T,H,E,k,xdt,with_bias", PLAN_CASES)
def test_route_plan_shapes(moeq, T, H, E, k, xdt, with_bias):
    _say(f"[route-plan] T={T} H={H} E={E} k={k} {xdt} bias={with_bias}")
    rng = np.random.default_rng(T * 7 + H + E)
    x = rng.standard_normal((T, H), dtype=np.float32)
    Wr = (rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    b = (rng.standard_normal(E).astype(np.float32) * np.float32(0.5)) if with_bias else None
    if xdt == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        xt = x_to_torch(bits, "bf16")
        x64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
    else:
        xt = torch.from_numpy(x).cuda()
        x64 = x.astype(np.float64)
    bt = torch.from_numpy(b).cuda() if b is not None else None
    ids, w, logits = moeq.route(xt, torch.from_numpy(Wr).cuda(), bt, k, want_logits=True)
    torch.cuda.synchronize()
    L = oracle.router_logits(x64, Wr, b)
    rids, rw, gap, flagged = oracle.topk_softmax(L, k)
    ids, w, logits = ids.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    ok = ~flagged
    assert ok.sum() >= 0.9 * T
    np.testing.assert_array_equal(ids[ok], rids[ok])
    assert np.max(np.abs(w[ok] - rw[ok])) <= 1e-6
    # fp32 logits are the fp64 sums rounded once (to within an fp32 ulp)
    assert np.all(np.abs(logits - L) <= 2.0 ** -23 * np.abs(L) + 1e-30)


def test_route_ties_and_bias_closed_form(moeq):
    """Zero router weights: all logits tie -> ids 0..k-1, w = 1/k; a ramp bias
    -> ids E-1, E-2, ... with the closed-form softmax."""
    T, H, E, k = 37, 256, 64, 4
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    Wr = torch.zeros(E, H, device="cuda")
    ids, w = moeq.route(x, Wr, None, k)
    assert (ids.cpu().numpy() == np.arange(k)).all()
    assert np.allclose(w.cpu().numpy(), 1.0 / k, atol=1e-7)
    b = torch.arange(E, dtype=torch.float32, device="cuda")
    ids, w = moeq.route(x, Wr, b, k)
    assert (ids.cpu().numpy() == np.arange(E - 1, E - 1 - k, -1)).all()
    z = np.exp(-np.arange(k, dtype=np.float64))
    assert np.allclose(w.cpu().numpy(), z / z.sum(), atol=1e-7)


# --------------------------------------------------------------------------- permutation
PERM_CASES = [
    (1, 2, 8, "random"), (0, 2, 8, "random"), (33, 2, 8, "random"), (1000, 6, 256, "random"),
    (4096, 8, 256, "random"), (2048, 2, 8, "one_expert"), (5000, 8, 64, "skewed"),
    (16384, 2, 64, "random"), (300, 1, 1, "random"), (777, 32, 256, "random"),
    (8192, 1, 8, "random"), (4097, 2, 8, "one_expert"), (100000, 8, 256, "skewed"),
]


@pytest.mark.parametrize("T,k,E,kind", PERM_CASES)
def test_permute_parity(moeq, T, k, E, kind):
    _say(f"[permute] T={T} k={k} E={E} {kind}")
    rng = np.random.default_rng(T * 31 + k)
    if kind == "random":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    elif kind == "one_expert":
        ids = np.tile(np.arange(k), (T, 1))
    else:
        p = 1.0 / np.arange(1, E + 1)
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    ids = ids.astype(np.int32).reshape(T, k)
    counts, offsets, perm, inv, ws = moeq.permute(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rp, ri = oracle.canonical_permute(ids, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    np.testing.assert_array_equal(inv.cpu().numpy(), ri)
    assert moeq.read_flags(ws) == 0


def test_permute_flags_bad_ids(moeq):
    ids = torch.tensor([[0, 1], [2, 9], [-1, 3]], dtype=torch.int32, device="cuda")
    counts, offsets, perm, inv, ws = moeq.permute(ids, 4)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) & moeq.FLAG_BAD_EXPERT_ID
    assert counts.sum().item() == 4


@pytest.mark.parametrize("T,k", [(8193, 1), (3000, 8)])
def test_permute_multiblock_flags_and_drops(moeq, T, k):
    """Above one block's share: bad and NaN ids in different blocks are
    dropped (inv = -1), both flags are raised, the rest sorts as the oracle."""
    E = 64
    rng = np.random.default_rng(T + k)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[5, 0] = E + 3                # bad id in the first block
    ids[T - 2, k - 1] = moeq.ID_NAN  # NaN sentinel in the last block
    counts, offsets, perm, inv, ws = moeq.permute(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    flags = moeq.read_flags(ws)
    assert flags & moeq.FLAG_BAD_EXPERT_ID and flags & moeq.FLAG_NAN_LOGIT
    # dropping an assignment = sorting it into an extra trailing expert E and
    # cutting that segment off: rows of the real experts are unchanged
    bad = (ids < 0) | (ids >= E)
    rc, ro, rp, ri = oracle.canonical_permute(np.where(bad, E, ids), E + 1)
    n = int(ro[E])
    ri = np.where(bad.reshape(-1), -1, ri)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc[:E])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro[:E + 1])
    np.testing.assert_array_equal(perm.cpu().numpy()[:n], rp[:n])
    np.testing.assert_array_equal(inv.cpu().numpy(), ri)


# --------------------------------------------------------------------------- int8
@pytest.mark.parametrize("cols", [1000, 999])  # 8-column vector path / element path
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_act_quant_bit_exact(moeq, dtype, cols):
    rng = np.random.default_rng(5)
    v = rng.standard_normal((67, cols)).astype(np.float32)
    v[3] = 0.0
    v[5, 7] = 37.0
    v[6] *= 1e-30
    v[8] = np.round(v[8] * 40) / 2  # many exact halves
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(v)
        v = synth.bf16_bits_to_f32(bits)
        vt = x_to_torch(bits, "bf16")
    else:
        vt = torch.from_numpy(v).cuda()
    q, s = moeq.act_quant_i8(vt)
    torch.cuda.synchronize()
    rq, rs = oracle.act_quant_i8(v)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


# --------------------------------------------------------------------------- whole layer
LAYER_CASES = [
    # name, T, H, I, E, k   (decode family when T*k < 48*E, else prefill)
    ("tiny", 64, 256, 512, 8, 2),
    ("tiny", 700, 256, 512, 8, 2),
    ("mixtral", 40, 512, 1024, 8, 2),
    ("mixtral", 600, 512, 1024, 8, 2),
    ("fine_e2m1", 70, 256, 256, 256, 6),
    ("fine_e2m1", 2100, 256, 128, 256, 6),
    ("hotcold", 300, 256, 128, 256, 8),
    ("hotcold", 2048, 256, 128, 256, 8),
    ("w4a8", 16, 512, 512, 8, 2),
    ("w4a8", 300, 512, 512, 8, 2),
    # prefill with idle wavefronts: H = 384 leaves two of the last down block's
    # four 64-row units empty, I = 384 gives three gate/up blocks per m-tile
    ("mixtral", 500, 384, 384, 8, 2),
    # small decode batches: the one-block front after the logits kernel
    ("mixtral", 2, 512, 1024, 8, 2),
    # one token
    ("mixtral", 1, 512, 1024, 8, 2),
    ("tiny", 1, 256, 512, 8, 2),            # fp32 activations
    ("w4a8", 1, 512, 512, 16, 2),           # int8 expert inputs, 16 experts
    ("fine_e2m1", 1, 256, 256, 32, 6),
    # few weight rows in flight: K split over more wavefronts (8-tile streams)
    ("fine_e2m1", 1, 2048, 256, 32, 6),
    ("fine_e2m1", 3, 1024, 256, 32, 6),
    # fused decode kernel (one row per touched expert, >= 256 expert-slice
    # blocks): ragged H (6 down row-tile pairs over 4 wavefronts), and 6
    # experts x 256 slices
    ("mixtral", 2, 384, 8192, 8, 2),
    ("mixtral", 3, 256, 16384, 8, 2),
    # expert-major prefill order: 2304 gate/up blocks, at least 4 per block slot
    # of a 256-CU device (the down launch, 72 blocks, takes the four-class order)
    ("mixtral", 4096, 256, 4096, 8, 2),
    # decode gate/up on the shared-token-tile kernel without the mask bit
    # (64 experts x 16 blocks of 4 row groups: two rounds of a 256-CU
    # device's block slots)
    ("mixtral", 64, 256, 4096, 64, 2),
]


def _run_layer_case(moeq, name, T, H, I, E, k, weight_mode="quantize"):
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode=weight_mode,
                              n_hot=min(64, E // 4) if name == "hotcold" else None)
    _say(f"[layer] {name} T={T} H={H} I={I} E={E} k={k} act={cfg.act} "
         f"({prefill_order(T, H, I, E, k)})")
    wl = Workload(cfg)
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, wl.b_np if cfg.zipf_alpha > 0 else None,
                           wl.expert, cfg.E, cfg.k, act=cfg.act)
    return cfg, wl, out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), ref


@pytest.mark.parametrize("name,T,H,I,E,k", LAYER_CASES)
def test_layer_parity(moeq, name, T, H, I, E, k):
    cfg, wl, out, ids, w, ref = _run_layer_case(moeq, name, T, H, I, E, k)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids[ok], ref["ids"][ok])
    err = rel_l2_rows(out[ok], ref["out"][ok])
    _say(f"    max row rel-L2 {err.max():.3e}  mean {err.mean():.3e}  flagged {int((~ok).sum())}")
    assert err.max() <= tolerance(cfg), err.max()


SPLIT_CASES = [
    # name, T, H, I, E, k, n_hot: one case per front-end path of the layer
    ("hotcold", 300, 256, 128, 64, 8, 16),   # separate router/permute/gather kernels
    ("mixtral", 8, 512, 1024, 8, 2, None),   # fused small-batch front
    ("w4a8", 16, 512, 512, 8, 2, None),      # fused front with int8 expert inputs
]


@pytest.mark.parametrize("name,T,H,I,E,k,n_hot", SPLIT_CASES)
def test_split_api_matches_layer_forward(moeq, name, T, H, I, E, k, n_hot):
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize", n_hot=n_hot)
    wl = Workload(cfg)
    act = cfg.act
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=act)
    ids2, w2 = moeq.route(wl.x, wl.Wr, wl.b, cfg.k)
    counts, offsets, perm, inv, _ = moeq.permute(ids2, cfg.E)
    Y = moeq.grouped_ffn(wl.x, wl.packed, offsets, perm, cfg.k, act=act)
    out2 = moeq.combine(Y, w2, inv, cfg.T, cfg.k)
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, act)
    moeq.ffn_gather(wl.x, perm, cfg.k, wl.packed, act, ws)
    moeq.ffn_gate_up(cfg.T, wl.packed, offsets, cfg.k, act, ws)
    Y3 = torch.empty_like(Y)
    moeq.ffn_down(cfg.T, wl.packed, offsets, cfg.k, act, Y3, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y3)
    assert torch.equal(ids, ids2) and torch.equal(w, w2)
    if T <= 32 and cfg.act != 2 and T * k <= min(T * k, E) and min(T * k, E) * I // 64 >= 256:
        # the layer took the fused decode kernel: g and u summed over K in
        # another split, so an fp16 h may round the other way, and Y summed
        # over intermediate slices in another fixed order
        err = rel_l2_rows(out.cpu().numpy(), out2.cpu().numpy())
        assert err.max() <= 1e-3, err.max()
    else:
        assert torch.equal(out, out2)
    # the permutation the layer used is the canonical one of its own ids
    rc, ro, rp, ri = oracle.canonical_permute(ids.cpu().numpy(), cfg.E)
    np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    np.testing.assert_array_equal(inv.cpu().numpy(), ri)


def test_layer_deterministic(moeq):
    cfg = synth.scaled_config("fine_e2m1", T=500, H=256, I=128, E=256, k=6, weight_mode="quantize")
    wl = Workload(cfg)
    a = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k)[0]
    b = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T", [1, 6, 600])  # fused front (one token, a few) / separate kernels
def test_nan_token(moeq, T):
    """A token with a NaN input: its routing is MOE_ID_NAN with weight 0, the
    layer flags MOE_FLAG_NAN_LOGIT and leaves its row 0, and every other
    token's output equals the layer run without that token's values."""
    cfg = synth.scaled_config("tiny", T=T, H=256, I=512, E=8, k=2, weight_mode="quantize")
    wl = Workload(cfg)
    bad = T // 3
    x_nan = wl.x.clone()
    x_nan[bad, 5] = float("nan")
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    out, ids, w = moeq.layer_forward(x_nan, wl.Wr, wl.b, wl.packed, cfg.k, ws=ws)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == moeq.FLAG_NAN_LOGIT
    assert (ids[bad] == moeq.ID_NAN).all() and (w[bad] == 0).all()
    assert (out[bad] == 0).all()
    ref, ids_ref, _ = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, ws=ws)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == 0  # the next call starts its own flag word
    keep = torch.arange(T, device=out.device) != bad
    assert torch.equal(ids[keep], ids_ref[keep])
    assert torch.equal(out[keep], ref[keep])
    ids2, w2 = moeq.route(x_nan, wl.Wr, wl.b, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids) and torch.equal(w2, w)


GRAPH_CASES = [
    ("mixtral", 8, 512, 1024, 8, 2),      # decode: logits + one-block front
    ("hotcold", 2048, 256, 128, 256, 8),  # prefill: multi-block permutation
]


@pytest.mark.parametrize("name,T,H,I,E,k", GRAPH_CASES)
def test_layer_graph_replay(moeq, name, T, H, I, E, k):
    """moe_layer_forward captured once in a HIP graph: every replay, with eager
    layer calls on other inputs in between (they rewrite the workspace),
    equals the eager result bit for bit."""
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize",
                              n_hot=min(64, E // 4) if name == "hotcold" else None)
    _say(f"[graph] {name} T={T} H={H} I={I} E={E} k={k}")
    wl = Workload(cfg)
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.act)
    ref, ids_ref, w_ref = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
    torch.cuda.synchronize()
    ref, ids_ref, w_ref = ref.clone(), ids_ref.clone(), w_ref.clone()
    out, ids, w = torch.empty_like(ref), torch.empty_like(ids_ref), torch.empty_like(w_ref)
    kw = dict(act=cfg.act, ws=ws, out=out, ids=ids, w=w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, **kw)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, **kw)
    other = wl.x.flip(0).contiguous()
    for rep in range(3):
        out.zero_()
        ids.zero_()
        w.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(ids, ids_ref) and torch.equal(w, w_ref), rep
        moeq.layer_forward(other, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
        torch.cuda.synchronize()
    del graph


def test_empty_batch(moeq):
    cfg = synth.scaled_config("tiny", T=4, H=256, I=512, E=8, k=2, weight_mode="quantize")
    wl = Workload(cfg)
    x = wl.x[:0]
    out, ids, w = moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, cfg.k)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)


def test_bf16_output(moeq):
    cfg = synth.scaled_config("mixtral", T=40, H=512, I=1024, E=8, k=2, weight_mode="quantize")
    wl = Workload(cfg)
    o32 = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k)[0]
    o16 = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, out_dtype=torch.bfloat16)[0]
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)


@pytest.mark.parametrize("nbytes", [16, 4096 * 256 * 16 * 8 + 48, 3 << 20])
def test_stream_read_xor(moeq, nbytes):
    """The measurement aid reads every word: the XOR of its per-block words is
    the XOR of the buffer's 32-bit words (remainder loop, 8-deep main loop,
    fewer chunks than threads)."""
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    for nt in (False, True):
        sink = moeq.stream_read(buf, nontemporal=nt)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(words)



@pytest.mark.parametrize("nbytes", [16, 16 * 1000003, 3 << 20])
def test_stream_read_shaped_xor(moeq, nbytes):
    """Every launch shape of the shaped read covers every word once: the XOR
    of its per-block words is the XOR of the buffer's words (both layouts,
    blocks that own no chunk, loads in flight from 1 to 16, tails)."""
    rng = np.random.default_rng(nbytes + 1)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    want = np.bitwise_xor.reduce(words)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    for blocks, waves, inflight, layout, nt in [(1, 1, 1, 0, False), (7, 3, 2, 1, True),
                                                (256, 4, 8, 0, True), (1024, 16, 16, 1, False),
                                                (4096, 4, 4, 1, True), (65536, 2, 16, 0, True)]:
        sink = moeq.stream_read_shaped(buf, blocks, waves, inflight, layout, nt)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == want, (blocks, waves, inflight, layout, nt)


def test_stream_read_shaped_rejects_bad_shapes(moeq):
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for blocks, waves, inflight, layout in [(0, 4, 8, 0), (65537, 4, 8, 0), (8, 0, 8, 0),
                                            (8, 17, 8, 0), (8, 4, 3, 0), (8, 4, 8, 2)]:
        with pytest.raises(moeq.MoeError):
            moeq.stream_read_shaped(buf, blocks, waves, inflight, layout,
                                    sink=torch.empty(max(blocks, 1), dtype=torch.int32, device="cuda"))

# ----------------------------------------------------- routing profile and tiers
@pytest.mark.parametrize("T,k,E", [(1, 2, 8), (1000, 6, 256), (70000, 8, 64), (0, 2, 8)])
def test_expert_histogram(moeq, T, k, E):
    _say(f"[histogram] T={T} k={k} E={E}")
    rng = np.random.default_rng(T + E)
    ids = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    if T:
        ids[0, 0] = moeq.ID_NAN
    d = torch.from_numpy(ids).cuda()
    h = moeq.expert_histogram(d, E)
    h = moeq.expert_histogram(d[: T // 2].contiguous(), E, h)  # accumulates
    torch.cuda.synchronize()
    want = oracle.expert_histogram(ids, E) + oracle.expert_histogram(ids[: T // 2], E)
    np.testing.assert_array_equal(h.cpu().numpy(), want)


@pytest.mark.parametrize("ntiers", [2, 3, 4])
def test_profiled_tiers_layer(moeq, ntiers):
    """Profile the routing of calibration tokens on the device, plan two tiers
    (4-bit g32 hot, 2-bit g16 cold), three (plus 1-bit g16 for the coldest)
    or four (4-, 3-, 2-, 1-bit, group 32), for the budget of n_hot hot experts
    at two tiers, pack by the plan and check the layer against the oracle."""
    from dataclasses import replace
    from synth import FMT_ASYM
    from synth.configs import A1G16, A2G16, A4G32
    n_hot = 16
    three = ntiers == 3
    fmts = {2: (A4G32, A2G16), 3: (A4G32, A2G16, A1G16),
            4: (A4G32, (FMT_ASYM, 3, 32), (FMT_ASYM, 2, 32), (FMT_ASYM, 1, 32))}[ntiers]
    base = synth.scaled_config("hotcold", T=512, H=256, I=128, E=64, k=8,
                               weight_mode="quantize", n_hot=n_hot)
    _say(f"[tiers] hotcold T={base.T} H={base.H} I={base.I} E={base.E} k={base.k}")
    # calibration tokens: the T rows after the layer's own, same router
    x_cal = synth.gen_x(base, 2 * base.T)[base.T:]
    Wr_np, b_np = synth.gen_router(base)
    Wr, b = torch.from_numpy(Wr_np).cuda(), torch.from_numpy(b_np).cuda()
    ids, _ = moeq.route(x_to_torch(x_cal, base.x_dtype), Wr, b, base.k)
    hist = moeq.expert_histogram(ids, base.E)
    torch.cuda.synchronize()
    counts = hist.cpu().numpy()
    np.testing.assert_array_equal(counts, oracle.expert_histogram(ids.cpu().numpy(), base.E))
    # bytes of one expert at each tier, from the library
    sizes = []
    for fmt in fmts:
        ex = synth.gen_expert(replace(base, expert_fmts=(fmt,) * base.E), 0)
        qm = [moeq.DeviceQMat.from_host(ex[r]) for r in ("gate", "up", "down")]
        sizes.append(moeq.packed_expert_bytes(*qm))
    budget = n_hot * sizes[0] + (base.E - n_hot) * sizes[1]
    tiers, used = moeq.plan_tiers(counts, sizes, budget)
    want_t, want_used = oracle.plan_tiers(counts, sizes, budget)
    np.testing.assert_array_equal(tiers, want_t)
    assert used == want_used <= budget
    order = sorted(range(base.E), key=lambda e: (-int(counts[e]), e))
    if ntiers > 2:  # the coarser tiers pay for more 4-bit experts
        assert int((tiers == 0).sum()) > n_hot and int((tiers == ntiers - 1).sum()) > 0
    else:
        assert used == budget
        assert set(np.flatnonzero(tiers == 0).tolist()) == set(order[:n_hot])
    # the profiled hot set covers at least as many calibration slots as the
    # bias-ranked one the workload would pick
    prior = [e for e in range(base.E) if synth.expert_format(base, e) == A4G32]
    assert counts[tiers == 0].sum() >= counts[prior].sum()
    cfg = replace(base, expert_fmts=tuple(fmts[t] for t in tiers))
    wl = Workload(cfg)
    out, ids2, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, wl.b_np, wl.expert, cfg.E, cfg.k,
                           act=cfg.act)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids2.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    _say(f"    hot share {counts[tiers == 0].sum() / counts.sum():.3f} "
         f"(bias-ranked {counts[prior].sum() / counts.sum():.3f}); max row rel-L2 {err.max():.3e}")
    assert err.max() <= tolerance(cfg)


MIXED_TIER_CASES = [
    # name, T, H, I, E, k: decode family (T*k < 48*E), then prefill
    ("hotcold", 40, 256, 256, 32, 4),
    ("hotcold", 600, 256, 256, 32, 4),
    ("hotcold", 1, 1024, 256, 32, 4),
]


@pytest.mark.parametrize("name,T,H,I,E,k", MIXED_TIER_CASES)
def test_layer_parity_one_bit_tiers(moeq, name, T, H, I, E, k):
    """Experts cycle through 4-bit g32, 2-bit g16 and 1-bit g16/g32/g64/g128
    (the sub-2-bit tier), quantised from N(0, 0.02) weights."""
    from dataclasses import replace
    from synth import FMT_ASYM
    cycle = [(FMT_ASYM, 4, 32), (FMT_ASYM, 2, 16), (FMT_ASYM, 1, 16), (FMT_ASYM, 1, 32),
             (FMT_ASYM, 1, 64), (FMT_ASYM, 1, 128)]
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize", n_hot=E // 4)
    cfg = replace(cfg, expert_fmts=tuple(cycle[e % len(cycle)] for e in range(E)))
    _say(f"[one-bit] {name} T={T} H={H} I={I} E={E} k={k}")
    wl = Workload(cfg)
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, wl.b_np, wl.expert, cfg.E, cfg.k,
                           act=cfg.act)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    _say(f"    max row rel-L2 {err.max():.3e}")
    assert err.max() <= tolerance(cfg)


# ------------------------------------------------------------ int8 router logits
@pytest.mark.parametrize("T,H,E,k,shared", [(1, 256, 8, 2, False), (300, 512, 64, 6, False),
                                            (2000, 1024, 256, 8, True), (64, 4096, 8, 2, True)])
def test_router_i8_parity(moeq, T, H, E, k, shared):
    _say(f"[router-i8] T={T} H={H} E={E} k={k} shared={shared}")
    rng = np.random.default_rng(T + E)
    x_np = rng.standard_normal((2 * T, H), dtype=np.float32)
    Wr_np = (rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    b_np = (rng.standard_normal(E) * 0.1).astype(np.float32)
    x = torch.from_numpy(x_np).cuda()
    Wr, b = torch.from_numpy(Wr_np).cuda(), torch.from_numpy(b_np).cuda()
    # calibration range over two calls (the first T rows, then the rest)
    lo, hi = moeq.router_logit_range(x[:T], Wr, b)
    lo, hi = moeq.router_logit_range(x[T:], Wr, b, lo, hi)
    torch.cuda.synchronize()
    L = oracle.router_logits(x_np.astype(np.float64), Wr_np, b_np)
    lo0, hi0 = oracle.router_logit_range(L)
    np.testing.assert_allclose(lo.cpu().numpy(), lo0, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(hi.cpu().numpy(), hi0, rtol=1e-12, atol=1e-15)
    s, z = moeq.router_i8_params(lo0, hi0, shared)  # the same parameters on both sides
    ids, w = moeq.route_i8(x[:T], Wr, b, k, torch.from_numpy(s).cuda(),
                           torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    ids0, w0, amb = oracle.topk_softmax_i8(L[:T], s, z, k)
    ok = ~amb
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ids0[ok])
    np.testing.assert_allclose(w.cpu().numpy()[ok], w0[ok], rtol=0, atol=1e-6)
    # agreement with the exact routing, for the record
    ids_x, _, _, _ = oracle.topk_softmax(L[:T], k)
    same = np.mean([set(a) == set(b2) for a, b2 in zip(ids.cpu().numpy(), ids_x)])
    _say(f"    ambiguous {int(amb.sum())}; same expert set as exact routing {same:.3f}")


# ------------------------------------------------------------ data-dependent flags
@pytest.mark.parametrize("T", [40, 600])  # decode GEMV / prefill GEMM
@pytest.mark.parametrize("scale,where", [(1e5, "input"), (2000.0, "h")])
def test_fp16_range_flag(moeq, T, scale, where):
    """One token scaled so that its fp16 expert input (x 1e5) or its SwiGLU
    output h (x 2000: inputs stay within fp16, h does not) leaves the fp16
    range: MOE_FLAG_FP16_RANGE is raised and every other token still matches
    the oracle."""
    cfg = synth.scaled_config("mixtral", T=T, H=512, I=1024, E=8, k=2, weight_mode="quantize")
    _say(f"[fp16-range] T={T} x{scale:g} ({where})")
    wl = Workload(cfg)
    bad = T // 2
    x32 = synth.bf16_bits_to_f32(wl.x_np).copy()
    x32[bad] *= np.float32(scale)
    xb = synth.f32_to_bf16_bits(x32)
    if where == "h":
        assert np.abs(synth.bf16_bits_to_f32(xb)).max() < 65504
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    out, ids, w = moeq.layer_forward(x_to_torch(xb, "bf16"), wl.Wr, wl.b, wl.packed, cfg.k, ws=ws)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) & moeq.FLAG_FP16_RANGE
    ref = oracle.moe_layer(xb, "bf16", wl.Wr_np, None, wl.expert, cfg.E, cfg.k)
    ok = ~ref["flagged"]
    ok[bad] = False
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    assert err.max() <= tolerance(cfg), err.max()
    # the unscaled batch raises nothing
    moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, ws=ws)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == 0


@pytest.mark.parametrize("T", [40, 600])
def test_bad_offsets_are_clamped(moeq, T):
    """Caller offsets past T*k, or decreasing, are clamped inside the task
    lookups: MOE_FLAG_BAD_SEGMENT is raised, nothing past Y's T*k rows is
    written (a canary tail stays intact), and with offsets[E] just past T*k
    the rows that exist equal those of the correct offsets."""
    cfg = synth.scaled_config("mixtral", T=T, H=512, I=1024, E=8, k=2, weight_mode="quantize")
    _say(f"[bad-offsets] T={T}")
    wl = Workload(cfg)
    R, H = T * cfg.k, cfg.H
    ids, w = moeq.route(wl.x, wl.Wr, wl.b, cfg.k)
    counts, offsets, perm, inv, _ = moeq.permute(ids, cfg.E)
    Y0 = moeq.grouped_ffn(wl.x, wl.packed, offsets, perm, cfg.k)
    torch.cuda.synchronize()
    canary = -12345.0
    for kind in ("past_end", "decreasing", "negative"):
        off = offsets.clone()
        if kind == "past_end":
            off[cfg.E] = R + 7
        elif kind == "decreasing":
            off[3] = off[2] - 5
        else:
            off[0] = -9
        Yb = torch.full(((R + 64) * H,), canary, dtype=torch.float32, device="cuda")
        ws = moeq.workspace(T, H, cfg.I, cfg.E, cfg.k)
        ws[:4].zero_()
        moeq.grouped_ffn(wl.x, wl.packed, off, perm, cfg.k, ws=ws, Y=Yb)
        torch.cuda.synchronize()
        assert moeq.read_flags(ws) & moeq.FLAG_BAD_SEGMENT, kind
        assert (Yb[R * H:] == canary).all(), kind
        if kind == "past_end":
            assert torch.equal(Yb[:R * H].view(R, H), Y0)


def test_expert_shape_mismatch_is_skipped(moeq):
    """Experts packed with I = 256 called with I = 128: MOE_FLAG_EXPERT_SHAPE,
    and no row of Y is written (prefill sizes: the down GEMM writes Y
    directly)."""
    cfg = synth.scaled_config("mixtral", T=600, H=512, I=256, E=8, k=2, weight_mode="quantize")
    wl = Workload(cfg)
    R, H = cfg.T * cfg.k, cfg.H
    ids, w = moeq.route(wl.x, wl.Wr, wl.b, cfg.k)
    counts, offsets, perm, inv, _ = moeq.permute(ids, cfg.E)
    canary = 777.0
    Yb = torch.full((R * H,), canary, dtype=torch.float32, device="cuda")
    ws = moeq.workspace(cfg.T, H, 128, cfg.E, cfg.k)
    ws[:4].zero_()
    moeq.grouped_ffn(wl.x, wl.packed, offsets, perm, cfg.k, ws=ws, Y=Yb, I=128)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) & moeq.FLAG_EXPERT_SHAPE
    assert (Yb == canary).all()


# ------------------------------------------- per-matrix formats, 3-bit, outliers
def _fmt_plan(kind, E):
    """Per-expert (gate, up, down) formats of a parity case."""
    from synth import FMT_ASYM, FMT_E2M1
    A = lambda b, g: (FMT_ASYM, b, g)
    if kind == "three_bit":
        cyc = [(A(3, g),) * 3 for g in (16, 32, 64, 128)]
    elif kind == "split":
        # the "AlphaQ" mix (gate 3-bit, up 2-bit, down 4-bit) and others whose
        # gate and up formats differ, next to experts that keep them equal
        cyc = [(A(3, 32), A(2, 16), A(4, 32)), (A(4, 32), A(3, 64), A(2, 16)),
               (A(2, 16), A(4, 64), A(3, 32)), ((FMT_E2M1, 4, 16), A(4, 32), A(1, 32)),
               (A(4, 32), A(4, 32), A(4, 32))]
    else:
        cyc = [(A(4, 32),) * 3, ((FMT_E2M1, 4, 16),) * 3, (A(2, 16),) * 3, (A(3, 32),) * 3]
    return tuple(cyc[e % len(cyc)] for e in range(E))


NEXT_CASES = [
    # name, T, H, I, E, k, kind, outlier share
    ("mixtral", 40, 512, 512, 8, 2, "three_bit", 0.0),     # decode GEMV
    ("mixtral", 600, 512, 512, 8, 2, "three_bit", 0.0),    # prefill GEMM
    ("mixtral", 40, 512, 512, 8, 2, "split", 0.0),
    ("mixtral", 600, 512, 512, 8, 2, "split", 0.0),
    ("hotcold", 1, 1024, 256, 32, 4, "split", 0.0),        # one token, fused front
    ("mixtral", 40, 512, 512, 8, 2, "mixed", 0.005),       # outliers, decode
    ("mixtral", 600, 512, 512, 8, 2, "mixed", 0.005),      # outliers, prefill
    ("mixtral", 600, 512, 384, 8, 2, "mixed", 0.0005),     # 0.05%: the field notes' share
    ("w4a8", 300, 512, 512, 8, 2, "split", 0.005),         # int8 x and h, split, outliers
    ("w4a8", 16, 512, 512, 8, 2, "split", 0.005),
    ("fine_e2m1", 70, 256, 256, 64, 6, "split", 0.005),
    # Zipf-skewed routing at prefill size: experts with few or no rows in the
    # padded transposed inputs of the outlier corrections
    ("hotcold", 600, 512, 256, 32, 4, "mixed", 0.005),
]


@pytest.mark.parametrize("name,T,H,I,E,k,kind,frac", NEXT_CASES)
def test_layer_parity_matrix_formats_and_outliers(moeq, name, T, H, I, E, k, kind, frac):
    from dataclasses import replace
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize",
                              n_hot=min(64, E // 4) if name == "hotcold" else None)
    cfg = replace(cfg, matrix_fmts=_fmt_plan(kind, E), weight_outlier_frac=frac)
    _say(f"[formats] {name} T={T} H={H} I={I} E={E} k={k} {kind} outliers={frac} act={cfg.act} "
         f"({prefill_order(T, H, I, E, k)})")
    wl = Workload(cfg)
    if kind == "split":
        assert wl.packed.fmt_mask & (1 << 31)
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.act)
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == 0
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, wl.b_np if cfg.zipf_alpha > 0 else None,
                           wl.expert, cfg.E, cfg.k, act=cfg.act)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    _say(f"    max row rel-L2 {err.max():.3e}")
    assert err.max() <= tolerance(cfg), err.max()
    if frac > 0:
        # the side lists matter: the same layer without them is further away
        # same blocks, lists dropped: repack from the workload's own blobs
        def bare(e):
            ex = wl.expert(e)
            return {r: synth.QMat(q.fmt, q.bits, q.group, q.rows, q.cols, q.codes, q.params)
                    for r, q in ex.items()}
        packed0 = moeq.pack_experts(bare, cfg.E)
        out0, _, _ = moeq.layer_forward(wl.x, wl.Wr, wl.b, packed0, cfg.k, act=cfg.act)
        torch.cuda.synchronize()
        err0 = rel_l2_rows(out0.cpu().numpy()[ok], ref["out"][ok])
        _say(f"    without the side lists: max row rel-L2 {err0.max():.3e}")
        assert err0.max() > 4 * err.max()


SHARED_TILE_CASES = [
    # name, T, H, I, E, k, kind (None: the workload's formats), outlier share
    ("mixtral", 40, 640, 1024, 8, 2, None, 0.0),    # 4-bit: 10 K tiles (ring of three, ragged)
    ("fine_e2m1", 70, 640, 512, 32, 6, None, 0.0),  # e2m1
    ("hotcold", 150, 640, 256, 32, 8, None, 0.0),   # 2-bit (two DMAs per wavefront and tile),
                                                    # skewed: several 32-row tiles per hot expert
    ("w4a8", 16, 1024, 512, 8, 2, None, 0.0),       # int8 expert inputs and h
    ("mixtral", 8, 256, 4096, 8, 2, None, 0.0),     # down projection in two K splits
    ("mixtral", 1, 512, 4096, 8, 2, None, 0.0),     # one row: one wavefront loads the tile
    ("mixtral", 40, 640, 512, 8, 2, "mixed", 0.005),  # 3-bit (two code loads), outlier lists
    ("mixtral", 40, 640, 512, 8, 2, "split", 0.005),  # split gate and up roles, 1-bit
]


@pytest.mark.parametrize("name,T,H,I,E,k,kind,frac", SHARED_TILE_CASES)
def test_shared_tile_decode(moeq, name, T, H, I, E, k, kind, frac):
    """The shared-token-tile decode GEMV, forced on every gate/up and down
    launch by MOE_MASK_SHARED_TILE, against the oracle."""
    from dataclasses import replace
    cfg = synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize",
                              n_hot=min(64, E // 4) if name == "hotcold" else None)
    if kind is not None:
        cfg = replace(cfg, matrix_fmts=_fmt_plan(kind, E), weight_outlier_frac=frac)
    order = prefill_order(T, H, I, E, k)
    _say(f"[shared tile] {name} T={T} H={H} I={I} E={E} k={k} {kind} outliers={frac} "
         f"act={cfg.act} ({order})")
    assert "GEMV" in order
    wl = Workload(cfg)
    full = wl.packed.fmt_mask
    ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.act)
    try:
        wl.packed.fmt_mask = full | moeq.MASK_SHARED_TILE
        out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
    finally:
        wl.packed.fmt_mask = full
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == 0
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, wl.b_np if cfg.zipf_alpha > 0 else None,
                           wl.expert, cfg.E, cfg.k, act=cfg.act)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    _say(f"    max row rel-L2 {err.max():.3e}")
    assert err.max() <= tolerance(cfg), err.max()


@pytest.mark.parametrize("T", [40, 600])
def test_outliers_need_mask_bit_at_prefill(moeq, T):
    """Experts with outlier lists and a mask without MOE_MASK_OUTLIERS: at
    prefill sizes the transposed input copy is not made, the flag says so and
    the corrections are missing; decode sizes need no copy and stay exact.
    Mask 0 stands for every bit and matches the oracle."""
    from dataclasses import replace
    cfg = synth.scaled_config("mixtral", T=T, H=512, I=512, E=8, k=2, weight_mode="quantize")
    cfg = replace(cfg, matrix_fmts=_fmt_plan("mixed", 8), weight_outlier_frac=0.005)
    prefill = "GEMV" not in prefill_order(T, cfg.H, cfg.I, cfg.E, cfg.k)
    _say(f"[outlier bit] T={T} prefill={prefill}")
    wl = Workload(cfg)
    full = wl.packed.fmt_mask
    assert full & moeq.MASK_OUTLIERS
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, None, wl.expert, cfg.E, cfg.k,
                           act=cfg.act)
    ok = ~ref["flagged"]
    try:
        for mask, bit in ((0, True), (full & ~moeq.MASK_OUTLIERS, False)):
            wl.packed.fmt_mask = mask
            ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.act)
            out, _, _ = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act, ws=ws)
            torch.cuda.synchronize()
            flags = moeq.read_flags(ws)
            err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok]).max()
            _say(f"    mask bit {bit}: flags {flags}, max row rel-L2 {err:.3e}")
            if bit or not prefill:
                assert flags == 0 and err <= tolerance(cfg), (flags, err)
            else:
                assert flags == moeq.FLAG_FORMAT_NOT_LAUNCHED
                assert err > tolerance(cfg)
    finally:
        wl.packed.fmt_mask = full


@pytest.mark.parametrize("T", [1, 3, 8])
def test_layer_parity_int8_x_fused(moeq, T):
    """int8 x only (MOE_ACT_I8_X): one or three tokens take the fused decode
    kernel with the row scales applied before SwiGLU; eight (two rows per
    expert) the two-launch path."""
    from dataclasses import replace
    cfg = replace(synth.scaled_config("w4a8", T=T, H=512, I=8192, E=8, k=2, weight_mode="quantize"),
                  act=synth.configs.ACT_I8_X)
    _say(f"[int8-x] T={T}")
    wl = Workload(cfg)
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, None, wl.expert, cfg.E, cfg.k, act=cfg.act)
    ok = ~ref["flagged"]
    np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = rel_l2_rows(out.cpu().numpy()[ok], ref["out"][ok])
    _say(f"    max row rel-L2 {err.max():.3e}")
    assert err.max() <= tolerance(cfg), err.max()


I8_CASES = [
    # name, T, H, I, E, k, activation mode, expert formats
    ("w4a8", 300, 512, 512, 8, 2, 2, None),      # ~75 rows per expert: one partial m-tile each
    ("w4a8", 1100, 512, 1024, 8, 2, 2, None),    # ~275 rows: full and partial m-tiles
    ("w4a8", 600, 1024, 512, 8, 2, 1, None),     # int8 x only: int8 gate/up, fp16 down
    ("w4a8", 600, 512, 512, 8, 2, 2, "mixed"),   # beside 2-bit and e2m1 experts: both kernels
    ("w4a8", 900, 512, 512, 32, 2, 2, None),     # 32 experts of about 56 rows
]


@pytest.mark.parametrize("name,T,H,I,E,k,act,kind", I8_CASES)
def test_int8_gemm_path(moeq, name, T, H, I, E, k, act, kind):
    """Prefill with int8 activations on 4-bit group-128 experts, with the
    caller's MOE_MASK_INT8_GEMM bit, runs the int8 MFMA GEMMs (integer group
    sums, scaled in fp32 per group), through moe_layer_forward and
    moe_grouped_ffn_q. They match the oracle, and the default fp16 kernels
    on the same layer."""
    from dataclasses import replace
    from synth import FMT_ASYM, FMT_E2M1
    cfg = replace(synth.scaled_config(name, T=T, H=H, I=I, E=E, k=k, weight_mode="quantize"),
                  act=act)
    if kind == "mixed":
        cyc = [(FMT_ASYM, 4, 128), (FMT_ASYM, 2, 16), (FMT_E2M1, 4, 16)]
        cfg = replace(cfg, expert_fmts=tuple(cyc[e % 3] for e in range(E)))
    _say(f"[int8 gemm] T={T} H={H} I={I} E={E} k={k} act={act} {kind} "
         f"({prefill_order(T, H, I, E, k)})")
    wl = Workload(cfg)
    full = wl.packed.fmt_mask
    assert full & (1 << 3) and not full & (moeq.MASK_SPLIT_GU | moeq.MASK_OUTLIERS)
    assert not full & moeq.MASK_INT8_GEMM  # never set by moe_format_mask
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, None, wl.expert, cfg.E, cfg.k, act=act)
    ok = ~ref["flagged"]
    outs = {}
    try:
        for label, mask in (("int8", full | moeq.MASK_INT8_GEMM), ("fp16", full)):
            wl.packed.fmt_mask = mask
            ws = moeq.workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, act)
            out, ids, _ = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=act, ws=ws)
            torch.cuda.synchronize()
            assert moeq.read_flags(ws) == 0
            np.testing.assert_array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
            outs[label] = out.cpu().numpy()
            err = rel_l2_rows(outs[label][ok], ref["out"][ok])
            _say(f"    {label} kernels: max row rel-L2 {err.max():.3e}")
            assert err.max() <= tolerance(cfg), (label, err.max())
    finally:
        wl.packed.fmt_mask = full
    d = rel_l2_rows(outs["int8"][ok], outs["fp16"][ok])
    _say(f"    int8 against fp16 kernels: max row rel-L2 {d.max():.3e}")
    assert d.max() <= tolerance(cfg)
    # the grouped FFN entry point honours the bit too: same kernels, same Y
    counts, offsets, perm, inv, _ = moeq.permute(torch.from_numpy(ref["ids"]).to("cuda").int(), cfg.E)
    try:
        Ys = {}
        for label, mask in (("int8", full | moeq.MASK_INT8_GEMM), ("fp16", full)):
            wl.packed.fmt_mask = mask
            Ys[label] = moeq.grouped_ffn(wl.x, wl.packed, offsets, perm, cfg.k, act=act).cpu().numpy()
        torch.cuda.synchronize()
    finally:
        wl.packed.fmt_mask = full
    dy = rel_l2_rows(Ys["int8"], Ys["fp16"])
    _say(f"    grouped FFN, int8 against fp16 kernels: max row rel-L2 {dy.max():.3e}")
    assert dy.max() <= tolerance(cfg)
