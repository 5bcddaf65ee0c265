"""Plain fp64 reference of one quantized MoE FFN layer (test infrastructure).

Sources (pages as titled; sections as numbered on each page):
  [Routing]   Baidu Cloud article on quantized MoE LLM inference, section
              "expert routing": router logits from a linear layer, keep the
              top-k experts, softmax over the selected logits, output is the
              weight-sum of the selected experts applied to the token.
  [TopK]      "Sparse activation in large models: the MoE engineering behind
              GPT-4's 2% activation", section 2.2: the router emits one logit
              per expert and the K highest are kept.
  [Gate]      MoE mixed-precision field notes, section 2.1: gating, softmax,
              top-k, expert compute, weighted sum; the gate stays unquantised
              and the expert inputs are quantised per token dynamically to
              int8 (W8A8).
  [PerExpert] "AlphaQ" blog, section 4.2: per-expert, per-layer
              {bit_width, group_size}, and section 2.2: per-matrix bit
              widths within an expert (a 3-bit gate, 2-bit middle, 4-bit
              output mix); expert-aware quantisation digest: hot experts at
              4-bit, cold experts at 2-bit, ever coarser tiers for colder ones.
  [Outliers]  MoE mixed-precision field notes, section 4.2: isolate the
              largest weights (about 0.05%) in fp16 and quantise the rest.
  [FFN]       "AlphaQ" blog, section 2.2 and the mixed-precision notes,
              section 3.3: each expert is a three-matrix FFN (gate, up/middle,
              down/output); its gated form is SwiGLU.
  [DRAQ]      "AlphaQ" blog, sections 2.2 and 4.1: the router's output
              logits, not its weights, are quantised to int8 with a scale and
              zero point calibrated on real data (range / 255), per output
              channel, and the top-k runs on the quantised values.
  [Tiers]     expert-aware quantisation digest, profiling, results and
              conclusion sections: profile which experts the router uses,
              keep the most used ones precise and the rest at 2 bits, and
              more generally coarser tiers for colder experts.

Readings where the pages are silent (each listed with its reason in the
design notes): ties and near-ties go to the lower expert index; the bias adds
to the logits before selection; segments are ordered by ascending token;
asymmetric blocks decode as w = s*q + m with one fp32 rounding; e2m1 uses the
OCP MX value set; int8 activations are symmetric absmax/127, round half to
even, clamped to +-127; the router sees the unquantised hidden states.

The tier plan is a reading too: experts ranked by routing count (ties to
the lower index), each taking the most precise tier that leaves room in the
byte budget for all experts after it at the cheapest tier.

Parity pins: see tests/test_oracle.py (brute-force dense MoE, invariants,
closed forms, textbook special cases, hand-written golden blobs).
"""
import numpy as np

# Adjacent top-(k+1) logit gaps below this (absolute, fp64) are near-ties: the
# token is flagged and excluded from id / output comparisons.
NEAR_TIE = 1e-6

# e2m1 magnitudes by 3-bit code (OCP microscaling spec): exponent bias 1, one
# mantissa bit, code 1 is the subnormal 0.5.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# --------------------------------------------------------------------------
# Weight blocks [PerExpert]
# --------------------------------------------------------------------------
def _unpack_codes(codes: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """uint8 [rows, row_bytes] -> uint8 [rows, cols]. The codes of a row form
    one little-endian bit stream: element e occupies bits [b*e, b*e + b), bit
    i of the stream being bit i % 8 of byte i // 8. So 4-bit: element 2i is
    the low nibble of byte i; 2-bit: element 4i+j is bits [2j, 2j+1] of byte
    i; 1-bit: element 8i+j is bit j of byte i; 3-bit: elements 8i..8i+7 fill
    the 24 bits of bytes 3i..3i+2 (byte 3i lowest), element 8i+j at bits
    [3j, 3j+2] of that 24-bit word."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows = codes.shape[0]
    mask = (1 << bits) - 1
    out = np.empty((rows, cols), dtype=np.uint8)
    if bits == 3:
        b = codes[:, :cols * 3 // 8].astype(np.uint32).reshape(rows, cols // 8, 3)
        word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        for j in range(8):
            out[:, j::8] = (word >> (3 * j)) & mask
        return out
    per_byte = 8 // bits
    b = codes[:, :cols // per_byte]
    for j in range(per_byte):
        out[:, j::per_byte] = (b >> (bits * j)) & mask
    return out


def decode_qmat(qm) -> np.ndarray:
    """Decode one canonical block matrix to fp32 [rows, cols].

    Asymmetric (fmt 1): w = round_fp32(s*q + m) with fp16 s, m and unsigned
    b-bit q (b = 1, 2, 3 or 4). The exact value s*q + m is formed in fp64
    (both terms are exact there) and rounded once to fp32.
    e2m1 (fmt 2): w = round_fp32(v(q) * s), v from the 3 magnitude bits, bit 3
    the sign, fp16 s per group.
    Each group's parameters apply to its `group` consecutive columns.
    Outliers (MoE mixed-precision field notes, section 4.2: a tiny share of
    the weights kept in fp16, the rest low-bit): when the matrix carries a
    side list, each listed element takes its fp16 value instead.
    """
    rows, cols, g = qm.rows, qm.cols, qm.group
    G = cols // g
    q = _unpack_codes(qm.codes, qm.bits, cols).reshape(rows, G, g)
    p = np.asarray(qm.params, dtype=np.uint16).view(np.float16).astype(np.float64)
    if qm.fmt == 1:
        s = p[:, 0::2][:, :G, None]
        m = p[:, 1::2][:, :G, None]
        w = (s * q + m).astype(np.float32)
    elif qm.fmt == 2:
        s = p[:, :G, None]
        v = E2M1_TABLE[q & 7] * np.where((q & 8) != 0, -1.0, 1.0)
        w = (v * s).astype(np.float32)
    else:
        raise ValueError(f"unknown weight format {qm.fmt}")
    w = w.reshape(rows, cols)
    out = getattr(qm, "outliers", None)
    if out is not None and len(out):
        # outlier side list: these elements are kept as fp16 values and replace
        # the block decode at their positions (index = row * cols + col)
        idx = np.asarray(out[:, 0], dtype=np.int64)
        val = np.asarray(out[:, 1], dtype=np.uint16).view(np.float16).astype(np.float32)
        w.reshape(-1)[idx] = val
    return w


# --------------------------------------------------------------------------
# Router [Routing], [TopK], [Gate]
# --------------------------------------------------------------------------
def x_to_f64(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Hidden states to fp64 (exact): bf16 bit patterns or fp32."""
    if x_dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def router_logits(X: np.ndarray, Wr: np.ndarray, b) -> np.ndarray:
    """L = X Wr^T + b in fp64 (the router linear, with its bias)."""
    L = X @ np.asarray(Wr, dtype=np.float64).T
    if b is not None:
        L = L + np.asarray(b, dtype=np.float64)[None, :]
    return L


def topk_softmax(L: np.ndarray, k: int):
    """Per token: the k largest logits, descending, ties to the lower expert
    index (a stable sort of -L); weights = softmax over those k logits.

    Returns ids [T,k] int32, w [T,k] fp64, gap [T] fp64 (smallest adjacent gap
    among the sorted top min(k+1, E)), flagged [T] bool (gap < NEAR_TIE).
    """
    T, E = L.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = np.argsort(-L[t], kind="stable")
        sel = order[:k]
        ids[t] = sel
        top = L[t, order[:min(k + 1, E)]]
        if top.size > 1:
            gap[t] = np.min(top[:-1] - top[1:])
        z = L[t, sel] - L[t, sel].max()
        e = np.exp(z)
        w[t] = e / e.sum()
    return ids, w, gap, gap < NEAR_TIE


# --------------------------------------------------------------------------
# Permutation by expert (contiguous per-expert segments)
# --------------------------------------------------------------------------
def canonical_permute(ids: np.ndarray, E: int):
    """Stable counting sort of the T*k assignments a = t*k + j by expert.

    counts[e]; offsets = exclusive prefix sum (length E+1);
    perm_token[r] = token of the r-th sorted assignment (ascending token
    inside a segment); inv[a] = r.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    perm_token = np.zeros(T * k, dtype=np.int64)
    inv = np.zeros(T * k, dtype=np.int64)
    for a in range(T * k):
        e = flat[a]
        r = cursor[e]
        cursor[e] += 1
        perm_token[r] = a // k
        inv[a] = r
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm_token.astype(np.int32), inv.astype(np.int32))


# --------------------------------------------------------------------------
# Per-token dynamic int8 activations [Gate]
# --------------------------------------------------------------------------
def act_quant_i8(v: np.ndarray):
    """Per row of fp32 v: s = fp32(absmax)/127 in fp32; q = clamp(rint(v/s),
    -127, 127) with fp32 division and round half to even; zero row -> s = 0,
    q = 0. Returns q int8 [rows, cols], s fp32 [rows]."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    s = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = (v / safe[:, None]).astype(np.float32)
    q = np.clip(np.rint(r), -127, 127)
    q = np.where(s[:, None] == 0, 0, q).astype(np.int8)
    return q, s


def dq8(v32: np.ndarray) -> np.ndarray:
    """fp64 value of the int8 quantisation of fp32 rows: q * s (exact)."""
    q, s = act_quant_i8(v32)
    return q.astype(np.float64) * s.astype(np.float64)[:, None]


# --------------------------------------------------------------------------
# Expert FFN [FFN]
# --------------------------------------------------------------------------
def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u with silu(z) = z / (1 + exp(-z))."""
    return g * u / (1.0 + np.exp(-g))


def expert_ffn(A: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
               act: int) -> np.ndarray:
    """One expert on its rows A (fp64): h = silu(A Wg^T) * (A Wu^T); when both
    expert inputs are int8 (act == 2) h is replaced by dq8(fp32(h));
    Y = h Wd^T."""
    G = A @ Wg.astype(np.float64).T
    U = A @ Wu.astype(np.float64).T
    Hh = swiglu(G, U)
    if act == 2:
        Hh = dq8(Hh.astype(np.float32))
    return Hh @ Wd.astype(np.float64).T


# --------------------------------------------------------------------------
# Weighted combine [Routing]
# --------------------------------------------------------------------------
def combine(Y: np.ndarray, w: np.ndarray, inv: np.ndarray, T: int, k: int) -> np.ndarray:
    """out[t] = sum_j w[t, j] * Y[inv[t*k + j]] in fp64."""
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * Y[inv[t * k + j]]
    return out


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------
def moe_layer(x, x_dtype: str, Wr, b, get_expert, E: int, k: int, act: int = 0,
              tokens=None):
    """Forward pass of the layer.

    get_expert(e) returns {"gate", "up", "down"} canonical block matrices; it
    is called once per expert with assignments, one expert at a time.
    tokens: optional subset of token indices whose outputs are computed (the
    routing and permutation always cover every token).
    act: 0 none; 1 int8 x before gate/up; 2 int8 x and int8 h before down.
    """
    X = x_to_f64(x, x_dtype)
    T = X.shape[0]
    L = router_logits(X, Wr, b)
    ids, w, gap, flagged = topk_softmax(L, k)
    counts, offsets, perm_token, inv = canonical_permute(ids, E)
    A_all = dq8(X.astype(np.float32)) if act in (1, 2) else X

    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    H = X.shape[1]
    Y = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        rows = rows[want[perm_token[rows]]]
        if rows.size == 0:
            continue
        ex = get_expert(e)
        Wg, Wu, Wd = (decode_qmat(ex["gate"]), decode_qmat(ex["up"]),
                      decode_qmat(ex["down"]))
        Y[rows] = expert_ffn(A_all[perm_token[rows]], Wg, Wu, Wd, act)
        del Wg, Wu, Wd
    out = combine(Y, w, inv, T, k)
    return dict(logits=L, ids=ids, w=w, gap=gap, flagged=flagged, counts=counts,
                offsets=offsets, perm_token=perm_token, inv=inv, Y=Y, out=out)


# --------------------------------------------------------------------------
# Routing profile and precision tiers [Tiers]
# --------------------------------------------------------------------------
def expert_histogram(ids: np.ndarray, E: int) -> np.ndarray:
    """Number of routing slots per expert, ids outside [0, E) not counted."""
    ids = np.asarray(ids).reshape(-1)
    out = np.zeros(E, dtype=np.int64)
    for e in ids:
        if 0 <= e < E:
            out[e] += 1
    return out


def plan_tiers(counts, tier_bytes, budget: int):
    """Tier index per expert (0 = most precise) and the bytes they use, or None
    when even every expert at the last tier exceeds the budget. Hottest first
    (count descending, ties to the lower index), each expert takes the first
    tier whose bytes still leave room for all later experts at the last tier."""
    counts = [int(c) for c in counts]
    tier_bytes = [int(b) for b in tier_bytes]
    E, last = len(counts), tier_bytes[-1]
    if E * last > budget:
        return None
    order = sorted(range(E), key=lambda e: (-counts[e], e))
    tiers = [0] * E
    used = 0
    for i, e in enumerate(order):
        rest = (E - 1 - i) * last
        t = next(t for t, b in enumerate(tier_bytes) if used + b + rest <= budget)
        tiers[e] = t
        used += tier_bytes[t]
    return np.array(tiers, dtype=np.int32), used


# --------------------------------------------------------------------------
# int8 router logits [DRAQ]
# --------------------------------------------------------------------------
def router_logit_range(L: np.ndarray):
    """Per expert, the smallest and largest logit over the tokens (NaN logits
    skipped; +inf / -inf when an expert has none)."""
    L = np.asarray(L, dtype=np.float64)
    lo = np.full(L.shape[1], np.inf)
    hi = np.full(L.shape[1], -np.inf)
    for e in range(L.shape[1]):
        col = L[:, e][~np.isnan(L[:, e])]
        if col.size:
            lo[e], hi[e] = col.min(), col.max()
    return lo, hi


def router_i8_params(lo, hi, shared: bool = False):
    """Scale s = fp32((hi - lo) / 255), at least the smallest normal fp32, and
    zero point z = -128 - rint(lo / s) saturated to int32: lo maps to code
    -128. With shared, one pair from the range over all experts."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    if shared:
        lo = np.full_like(lo, lo.min())
        hi = np.full_like(hi, hi.max())
    s = ((hi - lo) / 255.0).astype(np.float32)
    s = np.maximum(s, np.finfo(np.float32).tiny)
    z = -128.0 - np.rint(lo / s.astype(np.float64))
    return s, np.clip(z, -2.0**31, 2.0**31 - 1).astype(np.int64)  # int32, saturated


def quantize_logits_i8(L, scale, zero):
    """Logits after the int8 round trip (clamp(rint(L/s) + z, -128, 127) - z) * s
    (fp64 division, round half to even; experts with s <= 0 give 0), and per
    token whether some L/s lies within 1e-9 of a rounding boundary, where the
    order of an fp64 sum could decide the code."""
    L = np.asarray(L, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :]
    z = np.asarray(zero, dtype=np.float64)[None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = L / s
    q = np.clip(np.rint(r) + z, -128.0, 127.0)
    Lq = np.where(s > 0, (q - z) * s, 0.0)
    with np.errstate(invalid="ignore"):
        amb = (s > 0) & (np.abs(r - np.floor(r) - 0.5) < 1e-9)
    return Lq, amb.any(axis=1)


def topk_softmax_i8(L, scale, zero, k: int):
    """Routing on the int8 round trip of the logits: stable top-k (equal
    values to the lower index) and softmax over the selected quantised
    logits. Returns ids, w, and the tokens to exclude (rounding ambiguous)."""
    L = np.asarray(L, dtype=np.float64)
    nan_row = np.isnan(L).any(axis=1)
    Lq, amb = quantize_logits_i8(np.where(nan_row[:, None], 0.0, L), scale, zero)
    ids, w, _, _ = topk_softmax(Lq, k)
    ids[nan_row] = -2  # undefined routing, as for the unquantised router
    w[nan_row] = 0.0
    return ids, w, amb
