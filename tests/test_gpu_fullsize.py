"""Parity at the workloads' real sizes, in the launch configuration the
benchmark times (moe_layer_forward, one call, device-resident inputs).

Routing is checked on every token (ids bit-exact except oracle-flagged
near-ties) and the permutation on every assignment (bit-exact against the
canonical permutation of the GPU's ids); layer outputs are checked on a
sample of tokens whose experts the oracle decodes one at a time."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from layer_cases import Workload, rel_l2_rows, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moeq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_router_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sample_tokens(ids, flagged, n_tokens, max_experts):
    """Up to n_tokens non-flagged tokens whose experts stay within a set of at
    most max_experts (greedy, in token order)."""
    chosen, experts = [], set()
    for t in range(ids.shape[0]):
        if flagged[t]:
            continue
        new = experts | set(ids[t].tolist())
        if len(new) <= max_experts:
            chosen.append(t)
            experts = new
        if len(chosen) == n_tokens:
            break
    return chosen


CASES = [
    # name, T, sampled tokens, max distinct experts decoded by the oracle
    ("mixtral", 1, 1, 2),
    ("mixtral", 32, 6, 3),
    ("mixtral", 2048, 8, 3),
    ("fine_e2m1", 1, 1, 6),
    ("fine_e2m1", 64, 16, 40),
    ("fine_e2m1", 4096, 24, 40),
    ("hotcold", 4096, 24, 40),
    ("w4a8", 16, 2, 3),
    ("w4a8", 8192, 3, 3),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T,ns,me", CASES)
def test_fullsize_layer(moeq, name, T, ns, me):
    cfg = synth.get_config(name, T=T)
    _say(f"[fullsize] {name} T={T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} act={cfg.act}")
    wl = Workload(cfg)
    out, ids, w = moeq.layer_forward(wl.x, wl.Wr, wl.b, wl.packed, cfg.k, act=cfg.act)
    ids2, w2 = moeq.route(wl.x, wl.Wr, wl.b, cfg.k)
    counts, offsets, perm, inv, ws = moeq.permute(ids2, cfg.E)
    torch.cuda.synchronize()
    assert moeq.read_flags(ws) == 0
    ids_np = ids.cpu().numpy()
    assert np.array_equal(ids_np, ids2.cpu().numpy())

    # routing on every token
    b = wl.b_np if cfg.zipf_alpha > 0 else None
    L = oracle.router_logits(oracle.x_to_f64(wl.x_np, cfg.x_dtype), wl.Wr_np, b)
    rids, rw, gap, flagged = oracle.topk_softmax(L, cfg.k)
    ok = ~flagged
    np.testing.assert_array_equal(ids_np[ok], rids[ok])
    assert np.max(np.abs(w.cpu().numpy()[ok] - rw[ok])) <= 1e-6
    # permutation on every assignment
    rc, ro, rp, ri = oracle.canonical_permute(ids_np, cfg.E)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    np.testing.assert_array_equal(inv.cpu().numpy(), ri)

    # outputs on sampled tokens
    toks = _sample_tokens(ids_np, flagged, ns, me)
    assert toks, "no unflagged token to sample"
    _say(f"    sampled tokens {toks}, experts {sorted(set(ids_np[toks].reshape(-1).tolist()))}")
    ref = oracle.moe_layer(wl.x_np, cfg.x_dtype, wl.Wr_np, b, wl.expert_uncached, cfg.E, cfg.k,
                           act=cfg.act, tokens=toks, ids_override=ids_np)
    got = out.cpu().numpy()[toks]
    err = rel_l2_rows(got, ref["out"][toks])
    _say(f"    max row rel-L2 {err.max():.3e} (flagged tokens {int(flagged.sum())})")
    assert err.max() <= tolerance(cfg), err.max()
