"""Host model of the certified prefill router's candidate count on the
workloads' inputs: how many experts per token the error bound leaves for an
exact fp64 recomputation.

The bound and the threshold follow the library's rule: d = cb |x_t| |w_e| +
2^-40 |A| with cb = 2 (1.02 (n - 1) 2^-23 + 2^-16 + 2^-23 + ...) for bf16
rows (n = 512 products per fp32 run); the threshold is the k-th largest of
the 64 lanes' largest lower ends (lane l holds experts l, l + 64, ...); an
expert is a candidate when its upper end reaches it. The exact logits stand
in for the approximate ones (their difference is far below d)."""
import numpy as np
import pytest

import oracle
import synth


def _cb_bf16(H, ks):
    n = 4 * 64 * 2
    run = 1.02 * (n - 1) * 2.0 ** -23
    rest = 2.0 ** -23 + (H / 64 + ks + 2.0) * 2.0 ** -52
    return 2.0 * (run + 2.0 ** -16 + rest)


def candidates(L, x64, Wr, k, cb):
    nx = np.linalg.norm(x64, axis=1)
    nw = np.linalg.norm(np.asarray(Wr, dtype=np.float64), axis=1)
    d = cb * nx[:, None] * nw[None, :] + 2.0 ** -40 * np.abs(L)
    lo, hi = L - d, L + d
    T, E = L.shape
    pad = (-E) % 64
    lop = np.concatenate([lo, np.full((T, pad), -np.inf)], axis=1)
    lane_max = lop.reshape(T, -1, 64).max(axis=1)           # [T, 64]
    tau = -np.sort(-lane_max, axis=1)[:, k - 1]
    return (hi >= tau[:, None]).sum(axis=1)


@pytest.mark.parametrize("name,T,limit", [("fine_e2m1", 1024, 7.0), ("hotcold", 1024, 9.0),
                                          ("w4a8", 256, 3.0)])
def test_candidates_per_token(name, T, limit):
    cfg = synth.get_config(name, T)
    x64 = oracle.x_to_f64(synth.gen_x(cfg, T), cfg.x_dtype)
    Wr, b = synth.gen_router(cfg)
    b = b if cfg.zipf_alpha > 0 else None
    L = oracle.router_logits(x64, Wr, b)
    c = candidates(L, x64, Wr, cfg.k, _cb_bf16(cfg.H, 4))
    assert c.min() >= cfg.k
    assert c.mean() <= limit, c.mean()


def test_candidates_cover_the_top_k():
    """Brute force on small random cases: the exact top-k always lies inside
    the candidate set, with the logits perturbed by up to d (any values the
    bound allows)."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        T, H, E, k = 8, 64, int(rng.integers(32, 200)), int(rng.integers(1, 9))
        x64 = rng.standard_normal((T, H))
        Wr = rng.standard_normal((E, H)) * 0.02
        L = x64 @ Wr.T
        cb = float(rng.choice([1e-4, 1e-2, 1e-1]))
        nx = np.linalg.norm(x64, axis=1)
        nw = np.linalg.norm(Wr, axis=1)
        d = cb * nx[:, None] * nw[None, :]
        A = L + d * rng.uniform(-1.0, 1.0, L.shape)          # approximations within d
        lo, hi = A - d, A + d
        pad = (-E) % 64
        lane_max = np.concatenate([lo, np.full((T, pad), -np.inf)], axis=1).reshape(T, -1, 64).max(axis=1)
        tau = -np.sort(-lane_max, axis=1)[:, k - 1]
        cand = hi >= tau[:, None]
        top = np.argsort(-L, axis=1, kind="stable")[:, :k]
        assert np.take_along_axis(cand, top, axis=1).all()
