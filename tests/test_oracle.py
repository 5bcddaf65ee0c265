"""Pins of the CPU oracle against things other than itself: hand-worked blob
examples, the e2m1 code table, closed forms, brute force on tiny inputs,
library routines (torch.nn.functional, torch.softmax, numpy stable argsort)
and the invariants the method fixes. No GPU needed."""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from synth import FMT_ASYM, FMT_E2M1, QMat

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _qmat_from_golden(d):
    codes = np.frombuffer(bytes.fromhex(d["codes_hex"]), dtype=np.uint8).reshape(d["rows"], -1)
    params = np.array(d["params_u16"], dtype=np.uint16).reshape(d["rows"], -1)
    out = np.array(d["outliers"], dtype=np.uint32) if "outliers" in d else None
    return QMat(d["fmt"], d["bits"], d["group"], d["rows"], d["cols"], codes, params, out)


# ---------------------------------------------------------------- blocks
@pytest.mark.parametrize("key", ["asym4_g32", "asym2_g16", "asym1_g16", "e2m1_g16", "asym3_g16",
                                 "asym4_g32_outliers"])
def test_decode_hand_worked_blobs(key):
    d = _golden("blob_examples.json")[key]
    got = oracle.decode_qmat(_qmat_from_golden(d))
    exp = np.array(d["expected"], dtype=np.float32).reshape(d["rows"], d["cols"])
    np.testing.assert_array_equal(got, exp)
    # the sign of zero is part of the e2m1 table
    np.testing.assert_array_equal(np.signbit(got), np.signbit(exp))


def test_e2m1_code_table():
    g = _golden("e2m1_codes.json")
    codes = np.arange(16, dtype=np.uint8)
    packed = np.zeros((1, 16), dtype=np.uint8)
    packed[0, :8] = codes[0::2] | (codes[1::2] << 4)
    qm = QMat(FMT_E2M1, 4, 16, 1, 16, packed, np.array([[0x3C00]], dtype=np.uint16))
    got = oracle.decode_qmat(qm)[0]
    np.testing.assert_array_equal(got, np.array(g["code_to_value"], dtype=np.float32))
    assert np.array_equal(np.signbit(got), np.signbit(np.array(g["code_to_value"])))


@pytest.mark.parametrize("bits,group", [(4, 16), (4, 32), (4, 64), (4, 128), (2, 16), (2, 32), (2, 128),
                                        (1, 16), (1, 32), (1, 128), (3, 16), (3, 32), (3, 64), (3, 128)])
def test_asym_zero_error_roundtrip(bits, group):
    """Weights built exactly representable (s = 2^-j, m = n*2^-j, every group
    using codes 0 and 2^b-1) survive quantise -> decode bit-exactly, and the
    quantiser recovers the codes."""
    rng = np.random.default_rng(7)
    rows, cols = 6, 256
    qmax = (1 << bits) - 1
    q = rng.integers(0, qmax + 1, size=(rows, cols // group, group))
    q[..., 0] = 0
    q[..., -1] = qmax
    j = rng.integers(4, 10, size=(rows, cols // group, 1))
    n = rng.integers(-40, 40, size=(rows, cols // group, 1))
    s = np.ldexp(1.0, -j)
    W = (s * q + n * s).reshape(rows, cols).astype(np.float32)
    qm = synth.quantize_asym(W, bits, group)
    np.testing.assert_array_equal(oracle.decode_qmat(qm), W)
    qm2 = synth.quantize_asym(oracle.decode_qmat(qm), bits, group)
    np.testing.assert_array_equal(qm2.codes, qm.codes)
    np.testing.assert_array_equal(qm2.params, qm.params)


@pytest.mark.parametrize("bits,group", [(4, 32), (3, 64), (2, 16)])
def test_outliers_are_excluded_and_exact(bits, group):
    """Exactly representable groups plus a few planted large values: with the
    side list holding exactly the planted ones, the groups' min and max come
    from the rest, so decode reproduces W bit for bit (a quantiser that kept
    an outlier in its group's range would coarsen that group's step)."""
    rng = np.random.default_rng(9 + bits)
    rows, cols = 8, 256
    qmax = (1 << bits) - 1
    q = rng.integers(0, qmax + 1, size=(rows, cols // group, group))
    q[..., 0] = 0
    q[..., -1] = qmax
    j = rng.integers(6, 10, size=(rows, cols // group, 1))
    n = rng.integers(-20, 20, size=(rows, cols // group, 1))
    s = np.ldexp(1.0, -j)
    W = (s * q + n * s).reshape(rows, cols).astype(np.float32)
    planted = np.sort(rng.choice(rows * cols, size=5, replace=False))
    # planted values are exact in fp16 and beyond every group's range; the
    # planted positions avoid each group's first and last element
    planted = np.unique([p + 1 if p % group == 0 else (p - 1 if p % group == group - 1 else p)
                         for p in planted])
    W.reshape(-1)[planted] = np.array([96.0, -80.5, 70.25, -64.0, 100.0],
                                      dtype=np.float32)[:len(planted)]
    frac = len(planted) / W.size
    qm = synth.quantize_asym(W, bits, group, outlier_frac=frac)
    np.testing.assert_array_equal(qm.outliers[:, 0], np.sort(planted))
    np.testing.assert_array_equal(oracle.decode_qmat(qm), W)
    # the side list replaces exactly those elements: without it they decode
    # to a clipped code of their group
    bare = QMat(qm.fmt, qm.bits, qm.group, qm.rows, qm.cols, qm.codes, qm.params)
    diff = np.flatnonzero(oracle.decode_qmat(bare).reshape(-1) != W.reshape(-1))
    np.testing.assert_array_equal(diff, np.sort(planted))


def test_e2m1_outliers_excluded_from_absmax():
    rng = np.random.default_rng(12)
    rows, cols, group = 4, 64, 16
    code = rng.integers(0, 16, size=(rows, cols // group, group))
    code[..., 0] = 7
    v = oracle.E2M1_TABLE[code & 7] * np.where(code & 8, -1.0, 1.0)
    W = (v * 0.125).reshape(rows, cols).astype(np.float32)
    W[1, 5] = 50.0
    W[3, 60] = -33.0
    qm = synth.quantize_e2m1(W, group, outlier_frac=2 / W.size)
    np.testing.assert_array_equal(qm.outliers[:, 0], [1 * cols + 5, 3 * cols + 60])
    np.testing.assert_array_equal(oracle.decode_qmat(qm), W)


@pytest.mark.parametrize("group", [16, 32])
def test_e2m1_zero_error_roundtrip(group):
    rng = np.random.default_rng(8)
    rows, cols = 5, 128
    code = rng.integers(0, 16, size=(rows, cols // group, group))
    code[..., 0] = 7  # every group reaches |v| = 6, so s = absmax / 6 exactly
    j = rng.integers(2, 9, size=(rows, cols // group, 1))
    v = oracle.E2M1_TABLE[code & 7] * np.where(code & 8, -1.0, 1.0)
    W = (v * np.ldexp(1.0, -j)).reshape(rows, cols).astype(np.float32)
    qm = synth.quantize_e2m1(W, group)
    np.testing.assert_array_equal(oracle.decode_qmat(qm), W)


def test_asym_decode_single_rounding():
    """w = round_fp32(s*q + m): the exact fp64 sum rounded once, i.e. fp32 fma."""
    s = np.float16(0.0123)
    m = np.float16(-0.0917)
    q = np.arange(16)
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, :8] = q[0::2] | (q[1::2] << 4)
    params = np.zeros((1, 2), dtype=np.uint16)
    params[0, 0] = s.view(np.uint16)
    params[0, 1] = m.view(np.uint16)
    got = oracle.decode_qmat(QMat(FMT_ASYM, 4, 16, 1, 16, codes, params))[0]
    exp = [np.float32(float(s) * int(qq) + float(m)) for qq in q]  # python floats are fp64
    np.testing.assert_array_equal(got, np.array(exp, dtype=np.float32))


def test_four_bit_codes_are_quarter_of_fp16():
    f = _golden("pages_figures.json")["four_bit_codes_vs_fp16_bytes"]["value"]
    W = np.zeros((64, 4096), dtype=np.float32)
    qm = synth.quantize_asym(W, 4, 32)
    assert qm.codes.nbytes / (W.size * 2) == f


# ---------------------------------------------------------------- routing
def _brute_topk(L, k):
    """k passes of 'largest value, first index on ties'."""
    T, E = L.shape
    ids = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        taken = set()
        for j in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or L[t, e] > L[t, best]:
                    best = e
            taken.add(best)
            ids[t, j] = best
    return ids


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(3)
    L = rng.integers(-3, 4, size=(200, 8)).astype(np.float64)  # many exact ties
    for k in (1, 2, 3, 8):
        ids, w, gap, flagged = oracle.topk_softmax(L, k)
        np.testing.assert_array_equal(ids, _brute_topk(L, k))


def test_topk_exact_tie_goes_to_lower_index_and_is_flagged():
    L = np.array([[1.0, 3.0, 3.0, 0.0]])
    ids, w, gap, flagged = oracle.topk_softmax(L, 1)
    assert ids[0, 0] == 1 and flagged[0] and gap[0] == 0.0
    L = np.array([[1.0, 3.0, 3.0 - 2e-6, 0.0]])
    ids, w, gap, flagged = oracle.topk_softmax(L, 1)
    assert ids[0, 0] == 1 and not flagged[0]


def test_softmax_closed_form_bias_only_router():
    """Wr = 0, b = [0, 1, ..., E-1]: ids = [E-1, E-2], w = [e/(1+e), 1/(1+e)]."""
    E, H, T = 8, 16, 5
    X = np.random.default_rng(0).standard_normal((T, H))
    L = oracle.router_logits(X, np.zeros((E, H), np.float32), np.arange(E, dtype=np.float32))
    ids, w, gap, flagged = oracle.topk_softmax(L, 2)
    assert (ids == np.array([E - 1, E - 2])).all()
    e = np.e
    np.testing.assert_allclose(w, np.tile([e / (1 + e), 1 / (1 + e)], (T, 1)), rtol=0, atol=1e-15)
    assert not flagged.any()


def test_all_zero_router_ties_to_first_k():
    E, H, T, k = 8, 16, 4, 3
    L = oracle.router_logits(np.ones((T, H)), np.zeros((E, H), np.float32), None)
    ids, w, gap, flagged = oracle.topk_softmax(L, k)
    assert (ids == np.arange(k)).all()
    np.testing.assert_allclose(w, 1.0 / k, rtol=0, atol=1e-15)
    assert flagged.all()


def test_softmax_matches_torch():
    rng = np.random.default_rng(4)
    L = rng.standard_normal((50, 16)) * 3
    ids, w, _, _ = oracle.topk_softmax(L, 4)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    ref = torch.softmax(torch.from_numpy(sel), dim=-1).numpy()
    np.testing.assert_allclose(w, ref, rtol=0, atol=1e-15)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)


@pytest.mark.parametrize("key,E,k", [("activated_fraction_k2_of_128", 128, 2),
                                     ("activated_fraction_k1_of_128", 128, 1)])
def test_activated_fraction(key, E, k):
    frac = _golden("pages_figures.json")[key]["value"]
    rng = np.random.default_rng(5)
    L = rng.standard_normal((64, E))
    ids, *_ = oracle.topk_softmax(L, k)
    for t in range(64):
        assert len(set(ids[t].tolist())) / E == frac


# ---------------------------------------------------------------- permutation
def test_permute_matches_stable_argsort_and_invariants():
    rng = np.random.default_rng(6)
    for (T, k, E) in [(0, 2, 4), (1, 1, 1), (37, 2, 8), (100, 6, 256), (64, 8, 16)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
        counts, offsets, perm, inv = oracle.canonical_permute(ids, E)
        order = np.argsort(ids.reshape(-1), kind="stable")
        np.testing.assert_array_equal(perm, order // k)
        ref_inv = np.empty_like(order)
        ref_inv[order] = np.arange(order.size)
        np.testing.assert_array_equal(inv, ref_inv)
        np.testing.assert_array_equal(counts, np.bincount(ids.reshape(-1), minlength=E))
        assert offsets[0] == 0 and offsets[E] == T * k
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)  # ascending token, each token once
        np.testing.assert_array_equal(np.bincount(perm, minlength=T), np.full(T, k))
        np.testing.assert_array_equal(perm[inv], np.arange(T * k) // k)


# ---------------------------------------------------------------- int8 activations
def test_act_quant_special_cases():
    v = np.array([[0, 0, 0, 0],
                  [127, 2.5, -2.5, 3.5],
                  [-127, 1.5, 0.5, -0.5],
                  [254, 5, -7, 1]], dtype=np.float32)
    q, s = oracle.act_quant_i8(v)
    np.testing.assert_array_equal(s, np.array([0, 1, 1, 2], dtype=np.float32))
    np.testing.assert_array_equal(q, np.array([[0, 0, 0, 0],
                                               [127, 2, -2, 4],
                                               [-127, 2, 0, 0],
                                               [127, 2, -4, 0]], dtype=np.int8))


def test_act_quant_integer_rows_are_exact():
    rng = np.random.default_rng(9)
    v = rng.integers(-127, 128, size=(20, 64)).astype(np.float32)
    v[:, 0] = 127
    q, s = oracle.act_quant_i8(v)
    assert (s == 1).all()
    np.testing.assert_array_equal(q.astype(np.float32), v)
    # requantising dequantised rows is idempotent
    w = rng.standard_normal((20, 64)).astype(np.float32)
    q1, s1 = oracle.act_quant_i8(w)
    q2, s2 = oracle.act_quant_i8((q1.astype(np.float64) * s1[:, None]).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)


# ---------------------------------------------------------------- whole layer
def _tiny_layer(seed, T, H, I, E, k, formats, x_dtype="f32", bias=None):
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    x = synth.f32_to_bf16_bits(x32) if x_dtype == "bf16" else x32
    Wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    b = (rng.standard_normal(E) * bias).astype(np.float32) if bias else None
    experts = []
    for e in range(E):
        f = formats[e % len(formats)]
        # one (fmt, bits, group[, outlier fraction]) for all three matrices,
        # or a (gate, up, down) triple of them
        per_role = f if isinstance(f[0], tuple) else (f, f, f)
        ex = {}
        for (role, (r, c)), rf in zip((("gate", (I, H)), ("up", (I, H)), ("down", (H, I))), per_role):
            fmt, bits, group = rf[:3]
            frac = rf[3] if len(rf) > 3 else 0.0
            W = (rng.standard_normal((r, c)) * 0.1).astype(np.float32)
            ex[role] = (synth.quantize_asym(W, bits, group, frac) if fmt == FMT_ASYM
                        else synth.quantize_e2m1(W, group, frac))
        experts.append(ex)
    return x, Wr, b, experts


def _torch_expert(xt, ex):
    Wg = torch.from_numpy(oracle.decode_qmat(ex["gate"]).astype(np.float64))
    Wu = torch.from_numpy(oracle.decode_qmat(ex["up"]).astype(np.float64))
    Wd = torch.from_numpy(oracle.decode_qmat(ex["down"]).astype(np.float64))
    return F.linear(F.silu(F.linear(xt, Wg)) * F.linear(xt, Wu), Wd)


FORMAT_SETS = [[(FMT_ASYM, 4, 32)], [(FMT_ASYM, 2, 16)], [(FMT_E2M1, 4, 16)],
               [(FMT_ASYM, 4, 32), (FMT_ASYM, 2, 16)], [(FMT_ASYM, 4, 64), (FMT_E2M1, 4, 32)],
               [(FMT_ASYM, 3, 32), (FMT_ASYM, 3, 16)],
               # per-matrix formats: gate 3-bit, up 2-bit, down 4-bit
               [((FMT_ASYM, 3, 32), (FMT_ASYM, 2, 16), (FMT_ASYM, 4, 32))],
               # outlier side lists (2% here, so a 64x64 matrix has some)
               [(FMT_ASYM, 4, 32, 0.02), (FMT_E2M1, 4, 16, 0.02)]]


@pytest.mark.parametrize("fmts", FORMAT_SETS)
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (16, 8, 3), (9, 8, 8), (12, 5, 5)])
def test_layer_equals_dense_brute_force(fmts, T, E, k):
    """Dense MoE: every expert on every token (torch F.linear / F.silu in
    fp64), then the brute-force top-k and a torch softmax over the selected
    logits. Must equal the oracle's sparse path."""
    H, I = 64, 64
    x, Wr, b, experts = _tiny_layer(11 + T + E, T, H, I, E, k, fmts, bias=0.5)
    res = oracle.moe_layer(x, "f32", Wr, b, lambda e: experts[e], E, k)
    xt = torch.from_numpy(x.astype(np.float64))
    dense = torch.stack([_torch_expert(xt, experts[e]) for e in range(E)], dim=1)  # [T,E,H]
    L = xt @ torch.from_numpy(Wr.astype(np.float64)).T + torch.from_numpy(b.astype(np.float64))
    ids = _brute_topk(L.numpy(), k)
    np.testing.assert_array_equal(res["ids"], ids)
    w = torch.softmax(torch.gather(L, 1, torch.from_numpy(ids.astype(np.int64))), dim=-1)
    ref = (w[..., None] * dense[torch.arange(T)[:, None], torch.from_numpy(ids.astype(np.int64))]).sum(1)
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-13)


def test_single_expert_is_plain_swiglu_mlp():
    T, H, I = 6, 64, 96
    x, Wr, b, experts = _tiny_layer(21, T, H, I, 1, 1, [(FMT_ASYM, 4, 32)], x_dtype="bf16")
    res = oracle.moe_layer(x, "bf16", Wr, None, lambda e: experts[e], 1, 1)
    xt = torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64))
    ref = _torch_expert(xt, experts[0])
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-14)
    assert (res["w"] == 1.0).all() and (res["ids"] == 0).all()


def test_k_equals_e_is_full_softmax_mixture():
    T, H, I, E = 5, 32, 48, 4
    x, Wr, b, experts = _tiny_layer(31, T, H, I, E, E, [(FMT_ASYM, 4, 16)])
    res = oracle.moe_layer(x, "f32", Wr, None, lambda e: experts[e], E, E)
    xt = torch.from_numpy(x.astype(np.float64))
    L = xt @ torch.from_numpy(Wr.astype(np.float64)).T
    p = torch.softmax(L, dim=-1)
    ref = sum(p[:, e:e + 1] * _torch_expert(xt, experts[e]) for e in range(E))
    np.testing.assert_allclose(res["out"], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_one_hot_router_forces_routing():
    """Logits e*100*x_0 with x_0 = +-1: positive tokens go to the highest
    experts, negative ones to the lowest."""
    T, H, I, E, k = 6, 32, 32, 6, 2
    x, _, _, experts = _tiny_layer(41, T, H, I, E, k, [(FMT_ASYM, 4, 32)])
    x = x.copy()
    x[:, 0] = np.array([1, -1, 1, -1, 1, -1], dtype=np.float32)
    Wr = np.zeros((E, H), np.float32)
    Wr[:, 0] = np.arange(E) * 100.0
    res = oracle.moe_layer(x, "f32", Wr, None, lambda e: experts[e], E, k)
    for t in range(T):
        exp = [E - 1, E - 2] if x[t, 0] > 0 else [0, 1]
        assert res["ids"][t].tolist() == exp


def test_int8_x_with_integer_inputs_equals_unquantised():
    """x integer with row absmax 127 -> s = 1, q = x, so the int8-x path
    must equal the unquantised path exactly."""
    T, H, I, E, k = 8, 64, 32, 4, 2
    _, Wr, b, experts = _tiny_layer(51, T, H, I, E, k, [(FMT_ASYM, 4, 32)])
    rng = np.random.default_rng(1)
    x = rng.integers(-127, 128, size=(T, H)).astype(np.float32)
    x[:, 3] = -127
    Wr = Wr * np.float32(0.01)
    r0 = oracle.moe_layer(x, "f32", Wr, None, lambda e: experts[e], E, k, act=0)
    r1 = oracle.moe_layer(x, "f32", Wr, None, lambda e: experts[e], E, k, act=1)
    np.testing.assert_array_equal(r0["out"], r1["out"])


def test_int8_xh_mirrors_quantisation_of_h():
    """act = 2 equals the dense expert evaluated with dq8 applied to x and
    to fp32(h), computed here with torch ops."""
    T, H, I, E, k = 6, 64, 32, 3, 1
    x, Wr, b, experts = _tiny_layer(61, T, H, I, E, k, [(FMT_ASYM, 4, 32)])
    res = oracle.moe_layer(x, "f32", Wr, None, lambda e: experts[e], E, k, act=2)

    def tq(v):  # per-row absmax int8 in fp32 torch arithmetic
        v = v.to(torch.float32)
        s = v.abs().amax(dim=1) / 127.0
        q = torch.clamp(torch.round(v / torch.where(s == 0, 1.0, s)[:, None]), -127, 127)
        return (q.double() * s.double()[:, None])

    xt = tq(torch.from_numpy(x))
    for t in range(T):
        e = int(res["ids"][t, 0])
        Wg = torch.from_numpy(oracle.decode_qmat(experts[e]["gate"]).astype(np.float64))
        Wu = torch.from_numpy(oracle.decode_qmat(experts[e]["up"]).astype(np.float64))
        Wd = torch.from_numpy(oracle.decode_qmat(experts[e]["down"]).astype(np.float64))
        h = F.silu(F.linear(xt[t:t + 1], Wg)) * F.linear(xt[t:t + 1], Wu)
        y = F.linear(tq(h), Wd)
        np.testing.assert_allclose(res["out"][t], y[0].numpy(), rtol=1e-12, atol=1e-14)


def test_layer_invariants_on_workload_shapes():
    cfg = synth.scaled_config("hotcold", T=48, H=128, I=64, E=32, k=8, weight_mode="quantize", n_hot=8)
    x = synth.gen_x(cfg)
    Wr, b = synth.gen_router(cfg)
    res = oracle.moe_layer(x, cfg.x_dtype, Wr, b, lambda e: synth.gen_expert(cfg, e), cfg.E, cfg.k)
    assert np.all(np.abs(res["w"].sum(1) - 1) <= 1e-12)
    assert res["counts"].sum() == cfg.T * cfg.k
    np.testing.assert_array_equal(np.bincount(res["perm_token"], minlength=cfg.T), np.full(cfg.T, cfg.k))
    # each token's ids are distinct
    assert all(len(set(r)) == cfg.k for r in res["ids"].tolist())


def test_tokens_subset_matches_full():
    cfg = synth.scaled_config("w4a8", T=24, H=256, I=128, E=8, weight_mode="quantize")
    x = synth.gen_x(cfg)
    Wr, b = synth.gen_router(cfg)
    ge = lambda e: synth.gen_expert(cfg, e)
    full = oracle.moe_layer(x, cfg.x_dtype, Wr, b, ge, cfg.E, cfg.k, act=cfg.act)
    sub = oracle.moe_layer(x, cfg.x_dtype, Wr, b, ge, cfg.E, cfg.k, act=cfg.act, tokens=[3, 17])
    np.testing.assert_array_equal(sub["out"][[3, 17]], full["out"][[3, 17]])


# ---------------------------------------------------------------- generator statistics
def _top32_share(counts):
    c = np.sort(np.asarray(counts))[::-1]
    return c[:32].sum() / c.sum()


def test_hotcold_skew_top32_share():
    """Zipf router bias of the hot/cold workload: the 32 most-routed experts
    take about half of the assignments (expert-aware quantisation digest)."""
    target = _golden("pages_figures.json")["skewed_top32_share_of_256"]["value"]
    cfg = synth.get_config("hotcold")
    x = synth.gen_x(cfg)
    Wr, b = synth.gen_router(cfg)
    L = oracle.router_logits(oracle.x_to_f64(x, cfg.x_dtype), Wr, b)
    ids, *_ = oracle.topk_softmax(L, cfg.k)
    share = _top32_share(np.bincount(ids.reshape(-1), minlength=cfg.E))
    assert abs(share - target) < 0.03, share


def test_uniform_router_top32_share():
    """No bias: the top-32 share is the uniform 12.5% plus sampling noise."""
    target = _golden("pages_figures.json")["uniform_top32_share_of_256"]["value"]
    cfg = synth.get_config("fine_e2m1")
    x = synth.gen_x(cfg)
    Wr, b = synth.gen_router(cfg)
    L = oracle.router_logits(oracle.x_to_f64(x, cfg.x_dtype), Wr, b)
    ids, *_ = oracle.topk_softmax(L, cfg.k)
    share = _top32_share(np.bincount(ids.reshape(-1), minlength=cfg.E))
    assert target <= share < target + 0.04, share


def test_w4a8_outlier_fraction():
    cfg = synth.get_config("w4a8", T=256)
    x = synth.bf16_bits_to_f32(synth.gen_x(cfg))
    frac = np.mean(np.abs(x) > 8.0)  # N(0,1) beyond 8 sigma is ~1e-15; outliers are x20
    assert 0.0006 < frac < 0.0012, frac


# --------------------------------------------------------------------------
# Routing profile and precision tiers (expert-aware quantisation digest)
# --------------------------------------------------------------------------
def test_expert_histogram_hand_example():
    ids = np.array([[0, 3], [3, -2], [7, 0], [3, 1]], dtype=np.int32)
    # 7 and -2 lie outside [0, 4) and are not counted
    np.testing.assert_array_equal(oracle.expert_histogram(ids, 4), [2, 1, 0, 3])


def _lexmin_by_rank(counts, tier_bytes, budget):
    """Brute force: of all tier vectors within the budget, the one whose
    tiers, read hottest first (ties to the lower index), are smallest in
    lexicographic order."""
    E = len(counts)
    order = sorted(range(E), key=lambda e: (-counts[e], e))
    best = None
    for tv in itertools.product(range(len(tier_bytes)), repeat=E):
        if sum(tier_bytes[t] for t in tv) > budget:
            continue
        key = tuple(tv[e] for e in order)
        if best is None or key < best[0]:
            best = (key, tv)
    return None if best is None else np.array(best[1], dtype=np.int32)


def test_plan_tiers_matches_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(200):
        E = int(rng.integers(1, 7))
        nt = int(rng.integers(1, 4))
        tb = sorted((int(b) for b in rng.integers(1, 40, size=nt)), reverse=True)
        counts = [int(c) for c in rng.integers(0, 4, size=E)]  # many ties
        budget = int(rng.integers(0, E * tb[0] + 5))
        got = oracle.plan_tiers(counts, tb, budget)
        want = _lexmin_by_rank(counts, tb, budget)
        if want is None:
            assert got is None
        else:
            np.testing.assert_array_equal(got[0], want)
            assert got[1] == sum(tb[t] for t in want) <= budget


def test_plan_tiers_two_tiers_closed_form():
    # two tiers: the n = (budget - E*lo) // (hi - lo) hottest experts are hot
    rng = np.random.default_rng(12)
    for _ in range(50):
        E = int(rng.integers(1, 300))
        hi, lo = sorted((int(v) for v in rng.integers(1, 10**6, size=2)), reverse=True)
        if hi == lo:
            hi += 1
        counts = rng.integers(0, 50, size=E)
        budget = E * lo + int(rng.integers(0, E * (hi - lo) + 1))
        tiers, used = oracle.plan_tiers(counts, [hi, lo], budget)
        n = min(E, (budget - E * lo) // (hi - lo))
        order = sorted(range(E), key=lambda e: (-int(counts[e]), e))
        assert set(np.flatnonzero(tiers == 0).tolist()) == set(order[:n])
        assert used == n * hi + (E - n) * lo


def test_plan_tiers_digest_configuration():
    # The digest's configuration: 64 of 256 experts hot at 4 bits, 192 cold at
    # 2 bits. Bytes of one hidden-2048, intermediate-512 expert: 3*H*I weights
    # at 0.625 B (4-bit, fp16 scale+min per 32) or 0.5 B (2-bit, per 16).
    H, I, E = 2048, 512, 256
    b4, b2 = 3 * H * I * 5 // 8, 3 * H * I // 2
    rng = np.random.default_rng(13)
    counts = rng.permutation(E) * 7 + 3  # distinct
    tiers, used = oracle.plan_tiers(counts, [b4, b2], 64 * b4 + 192 * b2)
    hot = set(np.argsort(-counts)[:64].tolist())
    assert set(np.flatnonzero(tiers == 0).tolist()) == hot
    assert used == 64 * b4 + 192 * b2
    # one byte less and only 63 fit
    tiers, _ = oracle.plan_tiers(counts, [b4, b2], 64 * b4 + 192 * b2 - 1)
    assert int((tiers == 0).sum()) == 63


def test_plan_tiers_properties():
    rng = np.random.default_rng(14)
    for _ in range(100):
        E = int(rng.integers(1, 100))
        tb = sorted((int(b) for b in rng.integers(1, 1000, size=int(rng.integers(1, 5)))),
                    reverse=True)
        counts = rng.integers(0, 20, size=E)
        budget = int(rng.integers(E * tb[-1], E * tb[0] + 1))
        tiers, used = oracle.plan_tiers(counts, tb, budget)
        assert used <= budget
        order = sorted(range(E), key=lambda e: (-int(counts[e]), e))
        ranked = tiers[order]
        assert np.all(np.diff(ranked) >= 0)  # never more precise for a colder expert
        below = np.flatnonzero(ranked > 0)
        if below.size:  # the first expert below the top tier cannot move up one tier
            t = ranked[below[0]]
            assert used - tb[t] + tb[t - 1] > budget
    assert oracle.plan_tiers([1, 2, 3], [10, 5], 14) is None


# --------------------------------------------------------------------------
# int8 router logits ("AlphaQ" blog, DRAQ)
# --------------------------------------------------------------------------
def test_i8_router_hand_example():
    # s = 0.5, z = 0: L/s = 0.6, 0.4, 2, 0.2 -> codes 1, 0, 2, 0 -> 0.5, 0, 1, 0;
    # experts 1 and 3 tie at 0 and the lower index wins
    ids, w, amb = oracle.topk_softmax_i8([[0.3, 0.2, 1.0, 0.1]], [0.5] * 4, [0] * 4, 3)
    np.testing.assert_array_equal(ids, [[2, 0, 1]])
    e = np.exp([0.0, -0.5, -1.0])
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-15)
    assert not amb[0]


def test_i8_router_exact_on_the_grid():
    """Logits that are codes times the scale survive the round trip exactly,
    so the routing is the unquantised one, weights included."""
    rng = np.random.default_rng(31)
    E, T, k = 16, 200, 4
    s = np.ldexp(1.0, -rng.integers(3, 9, size=E)).astype(np.float32)
    z = rng.integers(-20, 20, size=E)
    codes = rng.integers(-128, 128, size=(T, E))
    L = (codes - z[None, :]) * s.astype(np.float64)[None, :]
    Lq, amb = oracle.quantize_logits_i8(L, s, z)
    np.testing.assert_array_equal(Lq, L)
    ids, w, _ = oracle.topk_softmax_i8(L, s, z, k)
    ids0, w0, _, _ = oracle.topk_softmax(L, k)
    np.testing.assert_array_equal(ids, ids0)
    np.testing.assert_array_equal(w, w0)


def test_i8_router_ambiguity_mask():
    """The mask fires exactly for tokens with some L/s within 1e-9 of a
    half-integer (where the rounding of an fp64 sum could decide the code):
    hand-placed logits at, near and away from a rounding boundary."""
    s = np.array([0.25, 0.5, 0.125], dtype=np.float32)   # exact in fp32
    z = np.array([3, -7, 0])
    sd = s.astype(np.float64)
    L = np.array([
        [2.5 * sd[0], 0.1, 0.3],               # L/s = 2.5 exactly -> ambiguous
        [0.1, (-3.5 + 4e-10) * sd[1], 0.3],    # 4e-10 from -3.5 -> ambiguous
        [0.1, 0.3, (7.5 + 5e-9) * sd[2]],      # 5e-9 away -> not ambiguous
        [0.1, 0.3, 0.77],                      # L/s = 0.4, 0.6, 6.16 -> not
        [(2.5 - 3e-9) * sd[0], 0.3, 0.77],     # 3e-9 below 2.5 -> not
    ])
    _, amb = oracle.quantize_logits_i8(L, s, z)
    np.testing.assert_array_equal(amb, [True, True, False, False, False])
    # an expert whose scale is 0 never makes a token ambiguous
    _, amb0 = oracle.quantize_logits_i8(np.zeros((2, 3)), np.zeros(3, np.float32), z)
    np.testing.assert_array_equal(amb0, [False, False])
    # random logits: a boundary within 1e-9 is a rare event
    rng = np.random.default_rng(34)
    _, ambr = oracle.quantize_logits_i8(rng.standard_normal((2000, 3)), s, z)
    assert ambr.sum() == 0


def test_i8_router_params_map_range_to_codes():
    rng = np.random.default_rng(32)
    for shared in (False, True):
        lo = rng.uniform(-3, 1, size=64)
        hi = lo + rng.uniform(0.01, 4, size=64)
        s, z = oracle.router_i8_params(lo, hi, shared)
        glo, ghi = (np.full(64, lo.min()), np.full(64, hi.max())) if shared else (lo, hi)
        q = lambda v: np.clip(np.rint(v / s.astype(np.float64)) + z, -128, 127)
        np.testing.assert_array_equal(q(glo), -128)
        assert set(np.unique(q(ghi)).tolist()) <= {126.0, 127.0}
        if shared:
            assert np.all(s == s[0]) and np.all(z == z[0])
        # beyond the range the codes saturate
        np.testing.assert_array_equal(q(ghi + 10 * s.astype(np.float64)), 127)


def test_i8_router_shared_codes_rank_like_values():
    """With one scale and zero point the int8 codes themselves give the top-k
    (stable, lower index first): the top-k 'in int8 space'."""
    rng = np.random.default_rng(33)
    L = rng.standard_normal((300, 32)) * 0.8
    s, z = oracle.router_i8_params(*oracle.router_logit_range(L), shared=True)
    ids, _, _ = oracle.topk_softmax_i8(L, s, z, 6)
    codes = np.clip(np.rint(L / s.astype(np.float64)) + z, -128, 127)
    for t in range(L.shape[0]):
        np.testing.assert_array_equal(ids[t], np.argsort(-codes[t], kind="stable")[:6])


def test_logit_range_skips_nan():
    L = np.array([[1.0, np.nan, -2.0], [0.5, np.nan, 3.0], [-1.0, np.nan, 0.0]])
    lo, hi = oracle.router_logit_range(L)
    np.testing.assert_array_equal(lo, [-1.0, np.inf, -2.0])
    np.testing.assert_array_equal(hi, [1.0, -np.inf, 3.0])
