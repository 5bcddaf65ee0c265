"""Shared helpers for the GPU parity tests and the benchmark: build a workload
on the device through the library, run the oracle on the same seeded inputs,
and compare."""
import numpy as np
import torch

import synth

TOL_F = 2e-3   # max per-row relative L2, bf16 / fp32 activations
TOL_I8 = 1e-2  # max per-row relative L2, int8 activations


def x_to_torch(x_np, x_dtype, device="cuda"):
    if x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_np)).to(device)


class Workload:
    """Seeded inputs of one layer workload, resident on the device."""

    def __init__(self, cfg, T=None, device="cuda", pack=True):
        import quantized_mixture_experts_router_amd as moeq
        self.cfg = cfg
        self.T = cfg.T if T is None else T
        self.x_np = synth.gen_x(cfg, self.T)
        self.Wr_np, self.b_np = synth.gen_router(cfg)
        self.x = x_to_torch(self.x_np, cfg.x_dtype, device)
        self.Wr = torch.from_numpy(self.Wr_np).to(device)
        self.b = torch.from_numpy(self.b_np).to(device) if cfg.zipf_alpha > 0 else None
        self._experts = {}
        self.packed = moeq.pack_experts(self.expert, cfg.E, device) if pack else None
        self._experts.clear()

    def expert(self, e):
        if e not in self._experts:
            self._experts[e] = synth.gen_expert(self.cfg, e)
        return self._experts[e]

    def expert_uncached(self, e):
        return synth.gen_expert(self.cfg, e)


def rel_l2_rows(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.where(den == 0, 1.0, den)


def tolerance(cfg):
    return TOL_I8 if cfg.act != 0 else TOL_F


def prefill_order(T, H, I, E, k, bm=128, blocks_per_cu=2):
    """The kernel family and prefill task order the library picks for these
    sizes (for the test log): decode GEMV below 48 rows per expert, else the
    prefill GEMM in expert-major order (lpt 0) from 4 blocks per block slot,
    longest first below that (lpt 1; the down projection uses four size
    classes below 2 blocks per slot, lpt 2)."""
    R = T * k
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    if R < 48 * E:
        te = min(R, E)
        if T <= 32 and R <= te and te * (I // 64) >= 256:
            return "fused decode kernel (one row per expert)"
        # gate/up on the shared-token-tile kernel from two rounds of its block
        # slots (three blocks per CU), or from one with short K streams
        # (4-bit tiles of 64 columns)
        gu_blocks = te * ((I // 32 + 3) // 4)
        sa = gu_blocks >= 2 * 3 * cus or (H // 64 <= 32 and gu_blocks >= 3 * cus)
        return "decode GEMV" + (", gate/up with a shared token tile" if sa else "")
    slots = cus * blocks_per_cu
    tiles = (R + bm - 1) // bm + min(R, E)
    out = []
    for what, units in (("gate/up", I // 32), ("down", H // 64)):
        nblk = tiles * ((units + 3) // 4)
        lpt = 2 if nblk < 2 * slots else (1 if nblk < 4 * slots else 0)
        if what == "gate/up" and lpt == 2:
            lpt = 1
        out.append(f"{what} {nblk} blocks lpt {lpt}")
    return "prefill GEMM: " + ", ".join(out)
