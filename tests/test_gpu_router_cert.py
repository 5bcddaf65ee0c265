"""Parity of the certified prefill router (approximate bf16 matrix-core logits
with an error bound, exact fp64 logits for the experts the bound leaves in
play) against the oracle and against the fp64 router.

moe_route takes the certified path when no fp32 logits are requested and the
batch is large enough (T >= 256, E >= 32); asking for logits selects the fp64
router on the same inputs, so the two can be compared token by token.

Bars: ids bit-exact except near-tie tokens the oracle flags (gap < 1e-6);
weights within 1e-6; against the fp64 router, ids bit-exact on every token
(both rank exact fp64 logits)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from layer_cases import x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moeq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_router_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(rng, T, H, E, xdt, with_bias, wscale=0.02):
    x = rng.standard_normal((T, H), dtype=np.float32)
    Wr = rng.standard_normal((E, H), dtype=np.float32) * np.float32(wscale)
    b = (rng.standard_normal(E).astype(np.float32) * np.float32(0.5)) if with_bias else None
    return x, Wr, b


def _to_dev(x, xdt):
    """(device tensor, exact fp64 copy) of fp32 rows, as bf16 or fp32."""
    if xdt == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        return x_to_torch(bits, "bf16"), synth.bf16_bits_to_f32(bits).astype(np.float64)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda(), x.astype(np.float64)


def _both_routers(moeq, xt, Wr, b, k):
    Wt = torch.from_numpy(Wr).cuda()
    bt = torch.from_numpy(b).cuda() if b is not None else None
    ids, w = moeq.route(xt, Wt, bt, k)                             # certified path
    ids0, w0, _ = moeq.route(xt, Wt, bt, k, want_logits=True)      # fp64 router
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), ids0.cpu().numpy(), w0.cpu().numpy()


def _check_against_oracle(ids, w, x64, Wr, b, k, min_ok=0.9):
    L = oracle.router_logits(x64, Wr, b)
    rids, rw, _, flagged = oracle.topk_softmax(L, k)
    ok = ~flagged
    assert ok.sum() >= min_ok * len(ids)
    np.testing.assert_array_equal(ids[ok], rids[ok])
    assert np.all(np.abs(w[ok] - rw[ok]) <= 1e-6)


# Workloads at full size, then shapes that reach the plan's branches: K splits
# 1..8, ragged token and expert tiles, a hidden size off the 64-column chunk,
# fp32 rows (three products per column), k = 1 and k = 32.
WORKLOAD_CASES = [("fine_e2m1", None), ("hotcold", None), ("w4a8", None), ("w4a8", 300)]


@pytest.mark.parametrize("name,T", WORKLOAD_CASES)
def test_cert_route_workloads(moeq, name, T):
    cfg = synth.get_config(name, T)
    _say(f"[cert-route] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    x_np = synth.gen_x(cfg, cfg.T)
    Wr, b = synth.gen_router(cfg)
    b = b if cfg.zipf_alpha > 0 else None
    xt = x_to_torch(x_np, cfg.x_dtype)
    ids, w, ids0, w0 = _both_routers(moeq, xt, Wr, b, cfg.k)
    _check_against_oracle(ids, w, oracle.x_to_f64(x_np, cfg.x_dtype), Wr, b, cfg.k)
    np.testing.assert_array_equal(ids, ids0)
    assert np.max(np.abs(w - w0)) <= 1e-6


SHAPE_CASES = [
    # T, H, E, k, x dtype, bias
    (256, 64, 32, 1, "bf16", False),     # one chunk, half an expert tile
    (300, 264, 40, 4, "f32", True),      # ragged T, E, and a partial last chunk
    (1000, 1000, 100, 5, "bf16", True),  # H % 64 == 40
    (777, 4104, 256, 32, "f32", False),  # k = 32, K split with a ragged chunk count
    (512, 8192, 32, 2, "bf16", True),    # eight K splits
    (2048, 2048, 64, 8, "f32", True),
]


@pytest.mark.parametrize("T,H,E,k,xdt,with_bias", SHAPE_CASES)
def test_cert_route_shapes(moeq, T, H, E, k, xdt, with_bias):
    _say(f"[cert-shape] T={T} H={H} E={E} k={k} {xdt} bias={with_bias}")
    rng = np.random.default_rng(T + 3 * H + E)
    x, Wr, b = _inputs(rng, T, H, E, xdt, with_bias)
    xt, x64 = _to_dev(x, xdt)
    ids, w, ids0, w0 = _both_routers(moeq, xt, Wr, b, k)
    _check_against_oracle(ids, w, x64, Wr, b, k)
    np.testing.assert_array_equal(ids, ids0)
    assert np.max(np.abs(w - w0)) <= 1e-6


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_cert_route_special_tokens(moeq, xdt):
    """Tokens the bound cannot settle or that leave the finite range: all-zero
    rows (every logit equals the bias), tiny and huge scales, a row whose
    logit overflows the fp32 sums but not fp64, NaN and Inf entries. Every token
    must route as the fp64 router does; NaN tokens get MOE_ID_NAN."""
    T, H, E, k = 512, 1024, 64, 4
    rng = np.random.default_rng(17)
    x, Wr, b = _inputs(rng, T, H, E, xdt, True)
    x[3] = 0.0
    x[10] *= np.float32(1e-30)
    x[11] *= np.float32(1e30)
    # 3e38 with the signs of expert 0's row: that logit (~1e40) overflows the
    # fp32 sums and is finite in fp64
    x[12] = np.float32(3e38) * np.sign(Wr[0])
    x[20, 100] = np.nan
    x[21, 7] = np.inf
    x[22, :] = -np.inf
    xt, x64 = _to_dev(x, xdt)
    ids, w, ids0, w0 = _both_routers(moeq, xt, Wr, b, k)
    np.testing.assert_array_equal(ids, ids0)
    both_nan = np.isnan(w) & np.isnan(w0)
    assert np.all(both_nan | (np.abs(w - w0) <= 1e-6))
    assert (ids[20] == -2).all() and (w[20] == 0).all()
    assert (ids[3] == np.argsort(-b.astype(np.float64), kind="stable")[:k]).all()
    finite = np.isfinite(x64).all(axis=1)
    _check_against_oracle(ids[finite], w[finite], x64[finite], Wr, b, k)


def test_cert_route_many_candidates(moeq):
    """Router rows that are near copies of each other: 16 experts within 1e-7
    relative of one row, 100 experts exactly equal to another. Tokens then
    carry tens to a hundred experts the bound cannot separate, all ranked
    on exact fp64 logits (exact copies tie and go to the lower index)."""
    T, H, E, k = 384, 512, 192, 6
    rng = np.random.default_rng(5)
    x, Wr, _ = _inputs(rng, T, H, E, "bf16", False)
    base = Wr[0].copy()
    for e in range(16):
        Wr[e] = base * np.float32(1.0 + 1e-7 * e) + np.float32(1e-9) * rng.standard_normal(H, dtype=np.float32)
    Wr[40:140] = Wr[40]
    # both groups sit well above the other experts for every token
    b = np.zeros(E, dtype=np.float32)
    b[:16] = 10.0
    b[40:140] = 10.0
    xt, x64 = _to_dev(x, "bf16")
    ids, w, ids0, w0 = _both_routers(moeq, xt, Wr, b, k)
    np.testing.assert_array_equal(ids, ids0)
    assert np.max(np.abs(w - w0)) <= 1e-6
    _check_against_oracle(ids, w, x64, Wr, b, k, min_ok=0.0)
    assert (ids < 16).any() and ((ids >= 40) & (ids < 140)).any()


def _cert_ks(T, H, E, xdt):
    """K splits of the certified router's plan for these sizes (the library's
    own rule: 128-token tiles, 128-expert tiles for bf16 rows and E > 64, else
    64; double the splits while the grid is under 256 blocks and each split
    keeps at least 4 chunks of 64 columns)."""
    bn = 128 if xdt == "bf16" and E > 64 else 64
    tt, et, nc = -(-T // 128), -(-E // bn), -(-H // 64)
    ks = 1
    while tt * et * ks < 256 and nc // (2 * ks) >= 4:
        ks *= 2
    return ks


@pytest.mark.parametrize("xdt,kind", [("bf16", "random"), ("bf16", "cancel"), ("f32", "cancel")])
def test_cert_bound_holds(moeq, xdt, kind):
    """The approximate logits the certified router leaves at the start of its
    workspace ([ks][T][E] fp32 partials) stay within half the bound it uses
    (the bound without its safety factor of 2) of the exact logits, also for
    rows built to cancel: positive token rows against router rows that are
    positive over the first half of every 256 columns and negative over the
    second, so the fp32 running sums climb high and come back near zero."""
    T, H, E, k = 512, 2048, 64, 2
    rng = np.random.default_rng(23)
    x, Wr, _ = _inputs(rng, T, H, E, xdt, False)
    if kind == "cancel":
        # 1 + 2^-9 + ... needs both bf16 parts of an fp32 row
        x = np.float32(1.0 + 2.0 ** -9) + rng.random((T, H)).astype(np.float32) * np.float32(1e-3)
        sign = np.where(np.arange(H) % 256 < 128, 1.0, -1.0).astype(np.float32)
        Wr = (np.float32(1.0) + rng.random((E, H)).astype(np.float32) * np.float32(3.0)) * sign
    xt, x64 = _to_dev(x, xdt)
    ws = torch.zeros(moeq.route_workspace_size(T, H, E), dtype=torch.uint8, device="cuda")
    moeq.route(xt, torch.from_numpy(Wr).cuda(), None, k, ws=ws)
    torch.cuda.synchronize()
    ks = _cert_ks(T, H, E, xdt)
    A = ws[: ks * T * E * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    A = A.reshape(ks, T, E).sum(axis=0)
    L = oracle.router_logits(x64, Wr, None)
    nx = np.linalg.norm(x64, axis=1)
    nw = np.linalg.norm(Wr.astype(np.float64), axis=1)
    n = 4 * 64 * (2 if xdt == "bf16" else 3)
    c = 1.02 * (n - 1) * 2.0 ** -23 + (2.0 ** -16 if xdt == "bf16" else 3.1 * 2.0 ** -16) + 2.0 ** -23
    bound = c * nx[:, None] * nw[None, :] + 2.0 ** -40 * np.abs(L)
    err = np.abs(A - L)
    _say(f"[cert-bound] {xdt} {kind}: max err/bound {np.max(err / bound):.3e}, "
         f"max err {np.max(err):.3e}")
    assert np.all(err <= bound)
