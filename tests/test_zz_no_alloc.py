"""The allocation-free layer entry point (moe_layer_forward_noalloc) against
moe_layer_forward, through the C ABI: two calls in a row on the library's
device scratch array, the second with a smaller batch, each equal bit for bit
to the layer with a caller workspace (same kernels, same order)."""
import sys

import numpy as np
import pytest
import torch

import synth
from layer_cases import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moeq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_mixture_experts_router_amd as m
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,Ts,H,I,E,k", [
    ("mixtral", (600, 8), 512, 1024, 8, 2),    # prefill GEMMs, then the one-block front
    ("w4a8", (300, 16), 512, 512, 8, 2),       # int8 x and h
    ("fine_e2m1", (70, 1), 256, 256, 256, 6),  # 256 experts, decode GEMVs
])
def test_noalloc_matches_layer_forward(moeq, name, Ts, H, I, E, k):
    cfg = synth.scaled_config(name, T=Ts[0], H=H, I=I, E=E, k=k, weight_mode="quantize")
    wl = Workload(cfg)
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for T in Ts:
        _say(f"[noalloc] {name} T={T} H={H} I={I} E={E} k={k} act={cfg.act}")
        assert moeq.workspace_size(T, H, I, E, k, cfg.act) <= moeq.noalloc_scratch_bytes()
        x = wl.x[:T].contiguous()
        ws = moeq.workspace(T, H, I, E, k, cfg.act)
        ref, ids_ref, w_ref = moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, k, act=cfg.act, ws=ws)
        out, ids, w = moeq.layer_forward_noalloc(x, wl.Wr, wl.b, wl.packed, k, act=cfg.act,
                                                 flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(ids, ids_ref) and torch.equal(w, w_ref)
        assert int(flags.item()) == moeq.read_flags(ws) == 0


def test_noalloc_flags_and_limit(moeq):
    """A NaN token raises MOE_FLAG_NAN_LOGIT in the caller's flag word, as in
    the workspace of moe_layer_forward; a batch whose workspace exceeds the
    array is refused before anything runs."""
    cfg = synth.scaled_config("tiny", T=6, H=256, I=512, E=8, k=2, weight_mode="quantize")
    wl = Workload(cfg)
    x = wl.x.clone()
    x[2, 3] = float("nan")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ids, w = moeq.layer_forward_noalloc(x, wl.Wr, wl.b, wl.packed, cfg.k, flags=flags)
    ref, _, _ = moeq.layer_forward(x, wl.Wr, wl.b, wl.packed, cfg.k)
    torch.cuda.synchronize()
    assert int(flags.item()) == moeq.FLAG_NAN_LOGIT
    assert torch.equal(out, ref)
    big = synth.scaled_config("tiny", T=200000, H=256, I=512, E=8, k=2, weight_mode="quantize")
    assert moeq.workspace_size(big.T, big.H, big.I, big.E, big.k) > moeq.noalloc_scratch_bytes()
    xb = torch.zeros((big.T, big.H), dtype=torch.float32, device="cuda")
    with pytest.raises(moeq.MoeError) as ei:
        moeq.layer_forward_noalloc(xb, wl.Wr, wl.b, wl.packed, big.k)
    assert ei.value.status == -4  # MOE_ERR_WORKSPACE
