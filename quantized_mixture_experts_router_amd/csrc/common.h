// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "moeq.h"

namespace moeq {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Weight formats handled by the kernels: (element format, bits, group size).
// ---------------------------------------------------------------------------
enum FmtId : int {
  F_A4G16 = 0, F_A4G32, F_A4G64, F_A4G128,
  F_A2G16, F_A2G32, F_A2G64, F_A2G128,
  F_E4G16, F_E4G32, F_E4G64, F_E4G128,
  F_A1G16, F_A1G32, F_A1G64, F_A1G128,
  F_A3G16, F_A3G32, F_A3G64, F_A3G128,
  F_COUNT
};
// bit of a format mask: some expert stores gate and up as separate streams
// (their formats differ), so the split gate and up passes run too
constexpr uint32_t kMaskSplitGU = MOE_MASK_SPLIT_GU;
// bit of a format mask: some expert cannot take the fused decode kernel
// (split gate/up, outlier lists, or a down format other than its gate/up's)
constexpr uint32_t kMaskNoFuse = MOE_MASK_NO_FUSE;
constexpr uint32_t kMaskOutliers = MOE_MASK_OUTLIERS;
constexpr uint32_t kMaskInt8 = MOE_MASK_INT8_GEMM;
constexpr uint32_t kMaskSharedTile = MOE_MASK_SHARED_TILE;
constexpr int kMaxE = 256;  // experts per layer
static_assert(F_COUNT <= 28, "format mask bits");

__host__ __device__ constexpr int fmt_id(int fmt, int bits, int group) {
  int g = group == 16 ? 0 : group == 32 ? 1 : group == 64 ? 2 : group == 128 ? 3 : -1;
  if (g < 0) return -1;
  if (fmt == MOE_W_ASYM && bits == 4) return F_A4G16 + g;
  if (fmt == MOE_W_ASYM && bits == 2) return F_A2G16 + g;
  if (fmt == MOE_W_E2M1 && bits == 4) return F_E4G16 + g;
  if (fmt == MOE_W_ASYM && bits == 1) return F_A1G16 + g;
  if (fmt == MOE_W_ASYM && bits == 3) return F_A3G16 + g;
  return -1;
}

// Roles of a grouped GEMM launch. R_GU: gate and up row tiles interleaved in
// one stream, SwiGLU in the epilogue (an expert whose gate and up share a
// format). R_DN: the down projection. R_GATE / R_UP: gate and up as separate
// streams of their own formats (an expert whose gate and up formats differ):
// the gate pass leaves g in h's buffer, the up pass turns it into
// h = silu(g) * u in place. A wavefront owns a gate/up row-tile pair (R_GU)
// or two consecutive row tiles of one matrix (the other roles).
enum Role : int { R_GU = 0, R_DN = 1, R_GATE = 2, R_UP = 3 };

// Device layout of one packed matrix W[N, K] (N rows = GEMM output columns).
//  - 32-row tiles; one tile spans KT = 2*SPAN columns; lane l = (n = l % 32,
//    kh = l / 32) holds SPAN codes of row n, columns [kt*KT + kh*SPAN, +SPAN).
//    4- and 2-bit: 16 bytes per lane (SPAN = 32, 64), a tile is 1 KiB.
//    1-bit: 8 bytes (SPAN = 64, KT = 128 like 2-bit, so the prefill token tile
//    keeps its size), 512 B. 3-bit: two planes, the low two bits of each code
//    laid out as a 2-bit tile (16 bytes per lane at 16 l) followed by the high
//    bit laid out as a 1-bit tile (8 bytes per lane at 1024 + 8 l): 1536 B.
//  - Inside each 32-bit word the codes are ordered so that (word >> b*i) &
//    mask yields the pair (code 2i, code 2i+1) in the two 16-bit halves.
//  - Tiles are stored row-tile major, then K-tile; interleaved gate/up have
//    row tiles 2j = gate rows 32j.., 2j+1 = up rows 32j...
//  - Params: one "entry" per (row, GE columns) with GE = max(group, SPAN),
//    holding max(1, SPAN/group) params (ASYM: fp16 (s, m) = 4 B each; E2M1:
//    fp16 s = 2 B each). Stored [row tile][entry][32 rows][EB bytes].
struct Codes3 {
  u32x4 lo;  // low two bits of the lane's 64 codes (2-bit layout)
  u32x2 hi;  // their high bit (1-bit layout)
};
template <int FMT, int BITS, int GROUP>
struct Fmt {
  static constexpr int ID = fmt_id(FMT, BITS, GROUP);
  static constexpr int kFmt = FMT;
  static constexpr int kBits = BITS;
  static constexpr int kGroup = GROUP;
  static constexpr int SPAN = (BITS == 1 || BITS == 3) ? 64 : 128 / BITS;  // codes per lane
  static constexpr int CB = BITS == 1 ? 8 : 16;           // bytes per lane, first plane
  static constexpr int TB = BITS == 1 ? 512 : (BITS == 3 ? 1536 : 1024);  // bytes per tile
  static constexpr int HOFF = 1024;                       // 3-bit: the high plane
  using CodeT = typename std::conditional<
      BITS == 3, Codes3, typename std::conditional<CB == 16, u32x4, u32x2>::type>::type;
  static constexpr int KT = 2 * SPAN;                      // K columns per tile
  static constexpr int STEPS = SPAN / 8;                   // 32x32x16 MFMA steps per tile
  static constexpr int GE = GROUP > SPAN ? GROUP : SPAN;   // K columns per param entry
  static constexpr int NP = GROUP < SPAN ? SPAN / GROUP : 1;
  static constexpr int PSZ = FMT == MOE_W_ASYM ? 4 : 2;
  static constexpr int EB = NP * PSZ;                      // entry bytes
};

__host__ __device__ inline int fmt_span(int bits) { return (bits == 1 || bits == 3) ? 64 : 128 / bits; }
__host__ __device__ inline int fmt_kt(int bits) { return 2 * fmt_span(bits); }
__host__ __device__ inline int fmt_tile_bytes(int bits) {
  return bits == 1 ? 512 : (bits == 3 ? 1536 : 1024);
}

inline size_t packed_codes_bytes(int N, int K, int bits) {
  return (size_t)(N / 32) * (size_t)(K / fmt_kt(bits)) * fmt_tile_bytes(bits);
}
inline size_t packed_params_bytes(int N, int K, int fmt, int bits, int group) {
  int span = fmt_span(bits);
  int ge = group > span ? group : span;
  int np = group < span ? span / group : 1;
  int eb = np * (fmt == MOE_W_ASYM ? 4 : 2);
  return (size_t)(N / 32) * (size_t)(K / ge) * 32 * eb;
}
// Outlier side lists, per packed matrix group (gate/up: rows 0..I-1 gate,
// I..2I-1 up; down: rows 0..H-1): rowptr [rows + 1] uint32, then entries
// {uint32 k, float delta} by row, delta = the fp16 outlier value minus the
// fp16 value the kernels decode from the block at (row, k).
struct OutEntry {
  uint32_t k;
  float delta;
};
inline size_t outlier_rowptr_bytes(int rows) { return (size_t)(rows + 1) * 4; }
static_assert(sizeof(moe_packed_expert) == 128, "descriptor size");
static_assert(sizeof(moe_qmat) == 40, "canonical matrix size");
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Workspace layout (byte offsets from the workspace base).
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t flags;    // uint32 flag word (+ pad to 256)
  size_t ids;      // int32 [T*k]
  size_t w;        // f32 [T*k]
  size_t counts;   // int32 [E]
  size_t offsets;  // int32 [E+1]
  size_t perm;     // int32 [T*k]
  size_t inv;      // int32 [T*k]
  size_t a16;      // f16 [T*k, H] expert inputs in sorted-row order
  size_t ascale;   // f32 [T*k] per-row int8 scale of a16 (int8 modes)
  size_t h;        // f16 [T*k, I]  or f32 [T*k, I] under MOE_ACT_I8_XH
  size_t h16;      // f16 [T*k, I] int8 codes of h (MOE_ACT_I8_XH)
  size_t hscale;   // f32 [T*k]
  // int8 prefill GEMM operands (int8 activation modes at prefill sizes):
  // codes in perm8 byte order and tile-major 64-column sums [K/128][T*k][2]
  size_t a8, asum;  // x: int8 [T*k, H], f32 [T*k * H/64]
  size_t h8, hsum;  // h (MOE_ACT_I8_XH): int8 [T*k, I], f32 [T*k * I/64]
  size_t yp;       // f32 [splits, T*k, H] down-projection (partial) sums
  size_t rpart;    // f64 [kb, T, E] router partial logits; aliases yp (routing ends
                   // before the down projection writes it)
  size_t pscratch; // permutation scratch; aliases yp too (the top-k has read the
                   // partial logits before the permutation runs)
  size_t poff;     // int32 [E+1] padded segment starts of the transposed inputs
  // Transposed expert inputs for the prefill outlier corrections (prefill
  // sizes with outliers only): f16 [K][rp], column p of expert e's padded
  // segment at poff[e] + p. The gate/up copy (K = H) takes yp's place when
  // it fits (yp is written only by the down projection); the down copy
  // (K = I) takes the fp32 h of MOE_ACT_I8_XH when it fits (free once its
  // int8 codes are made), else both go to a region at the end.
  size_t at_gu, at_dn;
  int rp;          // row pitch of the transposed copies, 0 when there are none
  size_t total;
  int splits;
  bool decode;
  bool i8;         // the int8 operand regions exist
};

// Choice of kernel family and split-K factor from host-known sizes only.
inline bool use_decode_path(int T, int k, int E) { return (long)T * k < 48L * E; }
#ifndef MOEQ_DEC_TARGET
#define MOEQ_DEC_TARGET 384
#endif
// Down projection at decode sizes: the K range is split over blocks so that
// about MOEQ_DEC_TARGET blocks stream weights (long streams per wavefront),
// at least 8 K tiles per wavefront.
inline int down_splits(int T, int H, int I, int E, int k) {
  if (!use_decode_path(T, k, E)) return 1;
  long rows = (long)T * k;
  long mtiles = rows < E ? rows : E;  // at most one 32-row tile per touched expert
  long blocks = mtiles * (H / 64);    // one block = 2 row tiles of 32
  if (blocks <= 0) return 1;
  int kt_total = I / 64;              // K tiles of a 4-bit matrix
  long s = (MOEQ_DEC_TARGET + blocks / 2) / blocks;
  if (s > kt_total / 32) s = kt_total / 32;
  return s < 1 ? 1 : (int)s;
}

// Fused decode FFN plan (host-known sizes only): used for decode batches of
// at most 32 tokens (one 32-row tile per expert) with one row per touched
// expert on average (MOEQ_FUSED_MAXROWS; with more, the partial planes cost
// more than the second launch saves: measured slower at 2 and 8 rows per
// expert), when the (touched expert, slice) blocks fill the device (at
// least 256; the 256-expert layer's 512-wide experts give too few slices at
// one token and measured slower), and without int8 h (its per-row scale
// needs the whole row of h). The slice width S is the smallest of 64 and the
// multiples of 128 dividing I whose ns = I / S partial planes [ns][T*k][H]
// fp32 stay within ~6% of the touched experts' weight bytes at 0.625 B per
// weight (ns <= 0.028 I / rows), and at most 512 (the h slice stays in 33
// KiB of LDS). A launch may widen S for its formats' K tiles and parameter
// groups (fewer planes, within the workspace).
#ifndef MOEQ_FUSED_MAXROWS
#define MOEQ_FUSED_MAXROWS 1
#endif
#ifndef MOEQ_FUSED_MINBLOCKS
#define MOEQ_FUSED_MINBLOCKS 256
#endif
struct FusedPlan {
  bool use;
  int S, ns;
};
inline FusedPlan fused_plan(int T, int H, int I, int E, int k, int aq) {
  FusedPlan p = {false, 0, 0};
  (void)H;
  if (!use_decode_path(T, k, E) || T > 32 || T <= 0 || aq == MOE_ACT_I8_XH) return p;
  const long R = (long)T * k, te = R < E ? R : E;
  const double rows = (double)R / (double)te;
  if (rows > MOEQ_FUSED_MAXROWS) return p;
  const double nsmax = 0.028125 * I / rows;
  for (int S = 64; S <= I && S <= 512; S = S == 64 ? 128 : S + 128) {
    if (I % S == 0 && I / S <= nsmax) {
      if (te * (I / S) < MOEQ_FUSED_MINBLOCKS) return p;
      p.use = true;
      p.S = S;
      p.ns = I / S;
      return p;
    }
  }
  return p;
}

// Router plan (host-known sizes only). The fp64 logits kernel runs one
// block per (16-token tile, group of ntw 16-expert tiles, K block); the
// block's ks wavefronts split the K block's 16-column chunks, cpw chunks
// each. K is split ks * kb ways in all, as few as give about
// MOEQ_ROUTE_WAVES wavefronts (four per SIMD) with >= 4 chunks per wave;
// expert tiles per wave drop below 4 first when the batch is too small for
// that. kb > 1 leaves kb fp64 partial logits [kb][T][E] for the top-k to add.
#ifndef MOEQ_ROUTE_WAVES
#define MOEQ_ROUTE_WAVES 4096
#endif
struct RoutePlan {
  int ntw, eg, ks, kb, cpw;
  size_t part_bytes;  // workspace of the partial logits
};
inline RoutePlan route_plan(int T, int H, int E) {
  RoutePlan p;
  const long TT = (T + 15) / 16;
  const int NT = (E + 15) / 16, NC = (H + 15) / 16;
  int ntw = NT < 4 ? NT : 4;
  while (ntw > 1 && TT * ((NT + ntw - 1) / ntw) * 16 < MOEQ_ROUTE_WAVES) ntw = (ntw + 1) / 2;
  p.ntw = ntw;
  p.eg = (NT + ntw - 1) / ntw;
  int S = 1;
  while (TT * p.eg * S < MOEQ_ROUTE_WAVES && NC / (2 * S) >= 4) S *= 2;
  int ks = S < 16 ? S : 16;
  while (ks * ntw > 32) ks /= 2;  // LDS of the in-block reduction <= 64 KiB
  p.ks = ks;
  p.kb = S / ks;
  p.cpw = (NC + S - 1) / S;
  p.part_bytes = (size_t)p.kb * (size_t)T * (size_t)E * sizeof(double);
  return p;
}

// Certified router for prefill batches (route_cert.hip): approximate logits
// on the bf16 matrix cores with a proven error bound, then exact fp64 logits
// of the experts that bound cannot rule out of the top-k. The router weights
// are first split into two bf16 planes [2][E][hp] (hp = H rounded up to 64)
// with their rows' fp64 norms [E]; then one block per (128-token
// tile, bn-expert tile, K split), bn = 128 for bf16 tokens and E > 64, else
// 64; ks K splits leave ks fp32 partial logits [ks][T][E] and fp64 partial
// squared norms of the token rows [ks][T]. Used for T >= 256 and E >= 32
// (below, the fp64 logits kernel is as fast) when no fp32 logits are asked
// for, and while every byte offset of x and Wr (as fp32) fits 31 bits.
#ifndef MOEQ_CERT_BLOCKS
#define MOEQ_CERT_BLOCKS 256
#endif
constexpr int kCertTileM = 128;  // tokens per block tile
constexpr int kCertChunk = 64;   // hidden columns per pipeline stage
struct CertPlan {
  bool use;
  int tt, et, bn, ks, cpb, hp;   // tiles, expert tile rows, K splits, chunks per block, padded H
  size_t ap, nx, nw, wp, bytes;  // workspace offsets and size
};
inline CertPlan cert_plan(int T, int H, int E, int xdt) {
  CertPlan p{};
  p.use = T >= 256 && E >= 32 && E <= kMaxE && (size_t)T * H * 4 < (1ull << 31) &&
          (size_t)E * H * 4 < (1ull << 31);
  if (!p.use) return p;
  const int nc = (H + kCertChunk - 1) / kCertChunk;
  p.hp = nc * kCertChunk;
  p.bn = xdt == MOE_BF16 && E > 64 ? 128 : 64;
  p.tt = (T + kCertTileM - 1) / kCertTileM;
  p.et = (E + p.bn - 1) / p.bn;
  p.ks = 1;
  while ((long)p.tt * p.et * p.ks < MOEQ_CERT_BLOCKS && nc / (2 * p.ks) >= 4) p.ks *= 2;
  p.cpb = (nc + p.ks - 1) / p.ks;
  size_t o = 0;
  p.ap = o;
  o = align256(o + (size_t)p.ks * T * E * 4);
  p.nx = o;
  o = align256(o + (size_t)p.ks * T * 8);
  p.nw = o;
  o = align256(o + (size_t)E * 8);
  p.wp = o;
  o = align256(o + (size_t)2 * E * p.hp * 2);
  p.bytes = o;
  return p;
}
inline size_t route_ws_bytes(int T, int H, int E) {
  size_t a = route_plan(T, H, E).part_bytes;
  for (int xdt : {MOE_F32, MOE_BF16}) {
    const CertPlan c = cert_plan(T, H, E, xdt);
    if (c.use && c.bytes > a) a = c.bytes;
  }
  return a;
}

// permutation: one block up to kPermuteSingleMax assignments, else
// histogram / scan / scatter kernels over `blocks` blocks of `chunk`
// assignments with scratch_bytes of device scratch (256-aligned)
constexpr int kPermuteSingleMax = 8192;
struct PermutePlan {
  int blocks, chunk;
  size_t scratch_bytes;
};
PermutePlan permute_plan(int R, int E);

// Columns of the transposed input copies: every expert's segment padded to
// a multiple of 32 rows, rounded up to 64.
inline size_t outlier_pitch(size_t R, int E) {
  const size_t ne = R < (size_t)E ? R : (size_t)E;
  return (R + 31 * ne + 63) / 64 * 64;
}

// outl: room for the transposed input copies of prefill outlier corrections.
// Every offset but at_gu/at_dn and total is the same either way.
inline WsLayout ws_layout(int T, int H, int I, int E, int k, int aq, bool outl = true) {
  WsLayout L;
  size_t R = (size_t)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t p = o; o = align256(o + bytes); return p; };
  L.flags = take(256);
  L.ids = take(R * 4);
  L.w = take(R * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.a16 = take(R * H * 2);
  L.ascale = take(R * 4);
  L.h = take(R * I * (aq == MOE_ACT_I8_XH ? 4 : 2));
  L.h16 = take(aq == MOE_ACT_I8_XH ? R * I * 2 : 0);
  L.hscale = take(R * 4);
  const bool i8 = aq != MOE_ACT_NONE && !use_decode_path(T, k, E);
  L.a8 = take(i8 ? R * H : 0);
  L.asum = take(i8 ? R * (H / 64) * 4 : 0);
  L.h8 = take(i8 && aq == MOE_ACT_I8_XH ? R * I : 0);
  L.hsum = take(i8 && aq == MOE_ACT_I8_XH ? R * (I / 64) * 4 : 0);
  L.i8 = i8;
  L.poff = take((size_t)(E + 1) * 4);
  L.splits = down_splits(T, H, I, E, k);
  L.decode = use_decode_path(T, k, E);
  const FusedPlan fp = fused_plan(T, H, I, E, k, aq);
  const int planes = fp.use && fp.ns > L.splits ? fp.ns : L.splits;
  const size_t yp_bytes = (size_t)planes * R * H * 4;
  const size_t rp_bytes = route_ws_bytes(T, H, E);
  const size_t ps_bytes = permute_plan((int)R, E).scratch_bytes;
  size_t big = yp_bytes > rp_bytes ? yp_bytes : rp_bytes;
  big = big > ps_bytes ? big : ps_bytes;
  L.yp = take(big);
  L.rpart = L.yp;
  L.pscratch = L.yp;
  L.at_gu = L.at_dn = 0;
  L.rp = 0;
  if (outl && !L.decode && R > 0) {
    const size_t rp = outlier_pitch(R, E);
    const size_t gu = (size_t)H * rp * 2, dn = (size_t)I * rp * 2;
    const bool gu_in = gu <= big;
    const bool dn_in = aq == MOE_ACT_I8_XH && dn <= R * I * 4;
    const size_t extra = (gu_in ? 0 : gu) > (dn_in ? 0 : dn) ? gu : (dn_in ? 0 : dn);
    const size_t at = take(extra);
    L.at_gu = gu_in ? L.yp : at;
    L.at_dn = dn_in ? L.h : at;
    L.rp = (int)rp;
  }
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Launchers (defined in the kernel translation units). All return a hip
// error code from the launch.
// ---------------------------------------------------------------------------
// router: fp64 logits (partials P, route_plan(T, H, E).part_bytes), then
// top-k + softmax; launch_route runs both
hipError_t launch_route_logits(const void* x, int xdt, const float* Wr, int T, int H, int E,
                               double* P, hipStream_t s);
hipError_t launch_route_topk(const double* P, int KB, const float* b, int T, int E, int k,
                             int32_t* ids, float* w, float* logits, hipStream_t s);
hipError_t launch_route(const void* x, int xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* logits, double* P,
                        hipStream_t s);
// certified router (cert_plan(T, H, E, xdt).use; ws: route_ws_bytes(T, H, E))
hipError_t launch_route_cert(const void* x, int xdt, const float* Wr, const float* b, int T,
                             int H, int E, int k, int32_t* ids, float* w, void* ws,
                             hipStream_t s);
// fused small-batch front after the logits kernel: top-k, permutation,
// gather (+ int8) in one block
bool front_fits(int T, int H, int E, int k);
hipError_t launch_front(const double* P, int KB, const void* x, int xdt, const float* b, int T,
                        int H, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, uint32_t* flags, int quant,
                        f16* a16, float* ascale, hipStream_t s);
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, uint32_t* flags,
                          void* scratch, hipStream_t s);
// a16 and a8/asum (h16 and h8/hsum) are each optional: the fp16-held codes
// feed the fp16 GEMMs, the byte codes (perm8 order) and their 64-column sums
// (tile-major [K/128][R][2]) the int8 ones
hipError_t launch_gather_a(const void* x, int xdt, const int32_t* perm, int T, int k, int H,
                           int quant, f16* a16, float* ascale, int8_t* a8, float* asum,
                           uint32_t* flags, hipStream_t s);
hipError_t launch_quant_rows_f32(const float* h, int R, int I, f16* h16, float* hscale,
                                 int8_t* h8, float* hsum, hipStream_t s);
hipError_t launch_act_quant_i8(const void* v, int dt, int rows, int cols, int8_t* q, float* sc,
                               hipStream_t s);
// The transposed copy of a prefill GEMM's input rows that its outlier
// corrections read (at == nullptr: none made; experts with outlier lists
// then flag MOE_FLAG_FORMAT_NOT_LAUNCHED at prefill sizes).
struct OutlierInputs {
  const f16* at;        // [K][rp]
  int rp;
  const int32_t* poff;  // [E+1] padded segment starts
};
// at[k][poff[e] + p] = a[lo_e + min(p, count_e - 1)][k] for p < the segment's
// count rounded up to 32, each 32-column group stored in the order the MFMA
// accumulators hold rows: slot 16 h + 4 g + i holds row 8 g + 4 h + i.
// Segments are the clamped [offsets[e], offsets[e+1]) of the GEMMs; poff is
// written too.
hipError_t launch_transpose_pad(const f16* a, int R, int K, const int32_t* offsets, int E,
                                f16* at, int rp, int32_t* poff, hipStream_t s);
// The int8 codes (perm8 byte order) and 64-column sums a prefill GEMM reads
// for the experts of format F_A4G128 (a8 == nullptr: the fp16 kernels take
// every format).
struct I8Inputs {
  const int8_t* a8;
  const float* asum;
};
constexpr uint32_t kI8Formats = 1u << F_A4G128;
hipError_t launch_ffn_gate_up(const moe_packed_expert* experts, const int32_t* offsets,
                              uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E,
                              int k, const f16* a16, const float* ascale, void* h, int h_f32,
                              bool decode, const OutlierInputs& oi, const I8Inputs& i8,
                              hipStream_t s);
hipError_t launch_ffn_down(const moe_packed_expert* experts, const int32_t* offsets,
                           uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                           const f16* ain, const float* ascale, float* yp, int splits,
                           bool decode, const OutlierInputs& oi, const I8Inputs& i8,
                           hipStream_t s);
hipError_t launch_reduce_splits(const float* yp, int splits, size_t n, float* Y, hipStream_t s);
hipError_t launch_combine(const float* yp, int splits, const float* w, const int32_t* inv, int T,
                          int H, int k, void* out, int out_dt, hipStream_t s);
// combine of many partial planes (the fused decode FFN's slices)
hipError_t launch_combine_slices(const float* yp, int ns, const float* w, const int32_t* inv,
                                 int T, int H, int k, void* out, int out_dt, hipStream_t s);
// fused decode FFN over the experts of the mask's formats; S is widened to
// the formats' K tiles and groups (returns hipErrorNotSupported when no
// admissible S fits the plan, before launching anything)
hipError_t launch_ffn_fused(const moe_packed_expert* experts, const int32_t* offsets,
                            uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                            const f16* a16, const float* ascale, float* yp, int S_plan,
                            int ns_plan, int* ns_used, hipStream_t s);
hipError_t launch_stream_read_shaped(const void* src, size_t bytes, int nontemporal, int blocks,
                                     int waves, int inflight, int layout, uint32_t* sink,
                                     hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                              hipStream_t s);
hipError_t launch_pack_matrix(const moe_qmat* a, const moe_qmat* b_or_null, void* codes,
                              void* params, hipStream_t s);
// outlier side lists of a (and, when b is given, of b as rows a.rows..) into
// rowptr [rows(+b.rows) + 1] and entries (OutEntry, n_a + n_b)
hipError_t launch_pack_outliers(const moe_qmat* a, const moe_qmat* b_or_null, uint32_t* rowptr,
                                OutEntry* entries, hipStream_t s);

// The whole layer on a validated workspace (api.hip); flags: where the flag
// word goes (nullptr: the workspace's own). check_layer_sizes validates the
// sizes and gives the workspace layout.
moe_status layer_forward_ws(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                            const moe_packed_expert* experts, uint32_t fmt_mask, int T, int H,
                            int I, int E, int k, moe_actq aq, void* out, moe_dtype out_dt,
                            int32_t* topk_ids, float* topk_w, void* ws, const WsLayout& L,
                            uint32_t* flags, hipStream_t s);
moe_status check_layer_sizes(int T, int H, int I, int E, int k, moe_actq aq, uint32_t fmt_mask,
                             WsLayout& L);

}  // namespace moeq
