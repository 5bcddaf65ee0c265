"""Canonical block format of one quantized weight matrix, and the quantisers
that write it (input preparation, not part of the layer's forward pass).

A matrix W[rows, cols] is quantised in groups of `group` consecutive elements
along `cols` (the input / K dimension of the GEMM that uses it).

Codes plane: uint8 [rows, row_bytes(cols, bits)], row-major, each row padded
with zero bytes to a multiple of 16 bytes.
  * 4-bit: element 2i in the low nibble of byte i, element 2i+1 in the high
    nibble.
  * 2-bit: element 4i+j in bits [2j, 2j+1] of byte i.
Params plane: uint16 (IEEE fp16 bit patterns) [rows, n_params], row-major.
  * FMT_ASYM (w = s*q + m, q unsigned b-bit): n_params = 2*cols/group, stored
    as (s, m) pairs per group.
  * FMT_E2M1 (w = e2m1(q) * s): n_params = cols/group, one s per group.

The per-expert bit-width / group-size descriptor follows the per-expert
`{bit_width, group_size}` configuration of the AlphaQ blog (section 4.2); the
4-bit floating-point element follows the OCP microscaling e2m1 encoding
(sign bit 3, two exponent bits with bias 1, one mantissa bit).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

FMT_ASYM = 1
FMT_E2M1 = 2

# e2m1 magnitudes by 3-bit code (OCP MX e2m1).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1_MID = (E2M1_VALUES[1:] + E2M1_VALUES[:-1]) / 2.0


def row_bytes(cols: int, bits: int) -> int:
    """Bytes per code row, padded to 16."""
    raw = (cols * bits + 7) // 8
    return (raw + 15) // 16 * 16


@dataclass
class QMat:
    fmt: int
    bits: int
    group: int
    rows: int
    cols: int
    codes: np.ndarray   # uint8 [rows, row_bytes]
    params: np.ndarray  # uint16 [rows, n_params] (fp16 bits)
    # outlier side list: uint32 [n, 2] of (row * cols + col, fp16 bits),
    # ascending and unique indices; None for none
    outliers: Optional[np.ndarray] = None

    @property
    def n_groups(self) -> int:
        return self.cols // self.group

    def nbytes(self) -> int:
        return int(self.codes.nbytes + self.params.nbytes)

    def payload_bytes(self) -> int:
        """Codes + params (+ outliers, 8 bytes each) without row padding (the
        bytes a kernel must read)."""
        n_out = 0 if self.outliers is None else len(self.outliers)
        return self.rows * (self.cols * self.bits // 8) + self.params.nbytes + 8 * n_out


def _pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    rows, cols = q.shape
    q = q.astype(np.uint8)
    out = np.zeros((rows, row_bytes(cols, bits)), dtype=np.uint8)
    if bits == 4:
        packed = q[:, 0::2] | (q[:, 1::2] << 4)
    elif bits == 2:
        packed = q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6)
    elif bits == 1:
        packed = np.zeros((rows, cols // 8), dtype=np.uint8)
        for j in range(8):
            packed |= q[:, j::8] << j
    elif bits == 3:
        # eight codes per 24-bit little-endian word, code j at bits [3j, 3j+2]
        word = np.zeros((rows, cols // 8), dtype=np.uint32)
        for j in range(8):
            word |= q[:, j::8].astype(np.uint32) << (3 * j)
        packed = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF],
                          axis=-1).astype(np.uint8).reshape(rows, -1)
    else:
        raise ValueError("bits must be 1, 2, 3 or 4")
    out[:, : packed.shape[1]] = packed
    return out


def pick_outliers(W: np.ndarray, frac: float):
    """The ceil(frac * size) elements of largest |w| (ties to the lower flat
    index), as the side list of QMat.outliers and a boolean mask."""
    flat = np.abs(W.astype(np.float64)).reshape(-1)
    n = int(np.ceil(frac * flat.size)) if frac > 0 else 0
    mask = np.zeros(flat.size, dtype=bool)
    if n == 0:
        return None, mask.reshape(W.shape)
    order = np.argsort(-flat, kind="stable")[:n]
    idx = np.sort(order)
    mask[idx] = True
    vals = W.reshape(-1)[idx].astype(np.float16).view(np.uint16)
    out = np.stack([idx.astype(np.uint32), vals.astype(np.uint32)], axis=1)
    return out, mask.reshape(W.shape)


def quantize_asym(W: np.ndarray, bits: int, group: int, outlier_frac: float = 0.0) -> QMat:
    """Asymmetric b-bit group quantisation: m = fp16(min), s = fp16(range/(2^b-1)),
    q = clip(rint((w - m)/s), 0, 2^b - 1) (round half to even); s == 0 gives q = 0.
    With outlier_frac > 0 the largest |w| go to an fp16 side list and are left
    out of their groups' min and max (their codes are the clipped ones)."""
    rows, cols = W.shape
    assert cols % group == 0
    qmax = (1 << bits) - 1
    outliers, omask = pick_outliers(W, outlier_frac)
    Wg = W.astype(np.float64).reshape(rows, cols // group, group)
    Mg = omask.reshape(rows, cols // group, group)
    mn = np.where(Mg, np.inf, Wg).min(axis=-1)
    mx = np.where(Mg, -np.inf, Wg).max(axis=-1)
    allout = ~np.isfinite(mn)          # a group made only of outliers
    mn = np.where(allout, 0.0, mn)
    mx = np.where(allout, 0.0, mx)
    m16 = mn.astype(np.float16)
    s16 = ((mx - mn) / qmax).astype(np.float16)
    s64 = s16.astype(np.float64)[..., None]
    m64 = m16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((Wg - m64) / np.where(s64 == 0, 1.0, s64))
    q = np.where(s64 == 0, 0.0, q)
    q = np.clip(q, 0, qmax).astype(np.uint8).reshape(rows, cols)
    params = np.empty((rows, 2 * (cols // group)), dtype=np.uint16)
    params[:, 0::2] = s16.view(np.uint16)
    params[:, 1::2] = m16.view(np.uint16)
    return QMat(FMT_ASYM, bits, group, rows, cols, _pack_codes(q, bits), params, outliers)


def quantize_e2m1(W: np.ndarray, group: int, outlier_frac: float = 0.0) -> QMat:
    """e2m1 group quantisation with one fp16 scale per group: s = fp16(absmax/6);
    each element goes to the nearest e2m1 value of w/s (ties to the even
    mantissa, saturating at 6); the sign goes to bit 3 (zero magnitude -> +0).
    With outlier_frac > 0 the largest |w| go to an fp16 side list and are left
    out of their groups' absmax."""
    rows, cols = W.shape
    assert cols % group == 0
    outliers, omask = pick_outliers(W, outlier_frac)
    Wg = W.astype(np.float64).reshape(rows, cols // group, group)
    Mg = omask.reshape(rows, cols // group, group)
    amax = np.where(Mg, 0.0, np.abs(Wg)).max(axis=-1)
    s16 = (amax / 6.0).astype(np.float16)
    s64 = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.abs(Wg) / np.where(s64 == 0, 1.0, s64)
    a = np.where(s64 == 0, 0.0, a)
    code = np.searchsorted(_E2M1_MID, a, side="left")
    at_mid = (code < 7) & (a == _E2M1_MID[np.minimum(code, 6)])
    code = np.where(at_mid & (code % 2 == 1), code + 1, code)
    code = np.minimum(code, 7)
    sign = (Wg < 0) & (code > 0)
    q = (code | (sign.astype(np.int64) << 3)).astype(np.uint8).reshape(rows, cols)
    params = s16.view(np.uint16).reshape(rows, cols // group).copy()
    return QMat(FMT_E2M1, 4, group, rows, cols, _pack_codes(q, 4), params, outliers)


def random_qmat(rng: np.random.Generator, rows: int, cols: int, fmt: int,
                bits: int, group: int, sigma: float = 0.02, outlier_frac: float = 0.0) -> QMat:
    """Codes drawn uniformly, per-group parameters drawn so that the decoded
    values span the range a quantisation of N(0, sigma) groups would give.
    With outlier_frac > 0, ceil(frac * size) distinct positions (uniform)
    get fp16 side-list values of magnitude 5-15 sigma, random sign."""
    assert cols % group == 0
    rb = row_bytes(cols, bits)
    used = cols * bits // 8
    codes = np.zeros((rows, rb), dtype=np.uint8)
    codes[:, :used] = rng.integers(0, 256, size=(rows, used), dtype=np.uint8)
    G = cols // group
    if fmt == FMT_ASYM:
        qmax = (1 << bits) - 1
        r = rng.uniform(3.5, 4.5, size=(rows, G))
        s = (sigma * r / qmax).astype(np.float16)
        m = (-sigma * r / 2.0 + 0.1 * sigma * rng.standard_normal((rows, G))).astype(np.float16)
        params = np.empty((rows, 2 * G), dtype=np.uint16)
        params[:, 0::2] = s.view(np.uint16)
        params[:, 1::2] = m.view(np.uint16)
    elif fmt == FMT_E2M1:
        assert bits == 4
        s = (sigma * rng.uniform(2.5, 3.5, size=(rows, G)) / 6.0).astype(np.float16)
        params = s.view(np.uint16).copy()
    else:
        raise ValueError(fmt)
    outliers = None
    n_out = int(np.ceil(outlier_frac * rows * cols)) if outlier_frac > 0 else 0
    if n_out:
        idx = np.sort(rng.choice(rows * cols, size=n_out, replace=False)).astype(np.uint32)
        mag = sigma * rng.uniform(5.0, 15.0, size=n_out)
        val = (mag * rng.choice([-1.0, 1.0], size=n_out)).astype(np.float16).view(np.uint16)
        outliers = np.stack([idx, val.astype(np.uint32)], axis=1)
    return QMat(fmt, bits, group, rows, cols, codes, params, outliers)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = 0x7FFF + ((u >> 16) & 1)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
