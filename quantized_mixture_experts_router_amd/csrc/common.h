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
  F_COUNT
};

__host__ __device__ constexpr int fmt_id(int fmt, int bits, int group) {
  int g = group == 16 ? 0 : group == 32 ? 1 : group == 64 ? 2 : group == 128 ? 3 : -1;
  if (g < 0) return -1;
  if (fmt == MOE_W_ASYM && bits == 4) return F_A4G16 + g;
  if (fmt == MOE_W_ASYM && bits == 2) return F_A2G16 + g;
  if (fmt == MOE_W_E2M1 && bits == 4) return F_E4G16 + g;
  if (fmt == MOE_W_ASYM && bits == 1) return F_A1G16 + g;
  return -1;
}

// Device layout of one packed matrix W[N, K] (N rows = GEMM output columns).
//  - 32-row tiles; one tile spans KT = 2*SPAN columns; lane l = (n = l % 32,
//    kh = l / 32) holds CB bytes = SPAN codes of row n, columns
//    [kt*KT + kh*SPAN, +SPAN). 4- and 2-bit: CB = 16 (SPAN = 32, 64), a tile
//    is 1 KiB. 1-bit: CB = 8 (SPAN = 64, KT = 128 like 2-bit, so the prefill
//    token tile keeps its size), a tile is 512 B.
//  - Inside each 32-bit word the codes are ordered so that (word >> b*i) &
//    mask yields the pair (code 2i, code 2i+1) in the two 16-bit halves.
//  - Tiles are stored row-tile major, then K-tile; gate/up are interleaved
//    as row tiles (2j = gate rows 32j.., 2j+1 = up rows 32j..).
//  - Params: one "entry" per (row, GE columns) with GE = max(group, SPAN),
//    holding max(1, SPAN/group) params (ASYM: fp16 (s, m) = 4 B each; E2M1:
//    fp16 s = 2 B each). Stored [row tile][entry][32 rows][EB bytes].
template <int FMT, int BITS, int GROUP>
struct Fmt {
  static constexpr int ID = fmt_id(FMT, BITS, GROUP);
  static constexpr int kFmt = FMT;
  static constexpr int kBits = BITS;
  static constexpr int kGroup = GROUP;
  static constexpr int SPAN = BITS == 1 ? 64 : 128 / BITS;  // codes per lane per tile
  static constexpr int CB = SPAN * BITS / 8;                // code bytes per lane per tile
  static constexpr int TB = 64 * CB;                        // code bytes per tile
  using CodeT = typename std::conditional<CB == 16, u32x4, u32x2>::type;
  static constexpr int KT = 2 * SPAN;                      // K columns per tile
  static constexpr int STEPS = SPAN / 8;                   // 32x32x16 MFMA steps per tile
  static constexpr int GE = GROUP > SPAN ? GROUP : SPAN;   // K columns per param entry
  static constexpr int NP = GROUP < SPAN ? SPAN / GROUP : 1;
  static constexpr int PSZ = FMT == MOE_W_ASYM ? 4 : 2;
  static constexpr int EB = NP * PSZ;                      // entry bytes
};

__host__ __device__ inline int fmt_span(int bits) { return bits == 1 ? 64 : 128 / bits; }
__host__ __device__ inline int fmt_kt(int bits) { return 2 * fmt_span(bits); }
__host__ __device__ inline int fmt_cb(int bits) { return fmt_span(bits) * bits / 8; }

inline size_t packed_codes_bytes(int N, int K, int bits) {
  return (size_t)(N / 32) * (size_t)(K / fmt_kt(bits)) * 64 * fmt_cb(bits);
}
inline size_t packed_params_bytes(int N, int K, int fmt, int bits, int group) {
  int span = fmt_span(bits);
  int ge = group > span ? group : span;
  int np = group < span ? span / group : 1;
  int eb = np * (fmt == MOE_W_ASYM ? 4 : 2);
  return (size_t)(N / 32) * (size_t)(K / ge) * 32 * eb;
}
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
  size_t yp;       // f32 [splits, T*k, H] down-projection (partial) sums
  size_t rpart;    // f64 [kb, T, E] router partial logits; aliases yp (routing ends
                   // before the down projection writes it)
  size_t pscratch; // permutation scratch; aliases yp too (the top-k has read the
                   // partial logits before the permutation runs)
  size_t total;
  int splits;
  bool decode;
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

// permutation: one block up to kPermuteSingleMax assignments, else
// histogram / scan / scatter kernels over `blocks` blocks of `chunk`
// assignments with scratch_bytes of device scratch (256-aligned)
constexpr int kPermuteSingleMax = 8192;
struct PermutePlan {
  int blocks, chunk;
  size_t scratch_bytes;
};
PermutePlan permute_plan(int R, int E);

inline WsLayout ws_layout(int T, int H, int I, int E, int k, int aq) {
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
  L.splits = down_splits(T, H, I, E, k);
  L.decode = use_decode_path(T, k, E);
  const size_t yp_bytes = (size_t)L.splits * R * H * 4;
  const size_t rp_bytes = route_plan(T, H, E).part_bytes;
  const size_t ps_bytes = permute_plan((int)R, E).scratch_bytes;
  size_t big = yp_bytes > rp_bytes ? yp_bytes : rp_bytes;
  big = big > ps_bytes ? big : ps_bytes;
  L.yp = take(big);
  L.rpart = L.yp;
  L.pscratch = L.yp;
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
hipError_t launch_gather_a(const void* x, int xdt, const int32_t* perm, int T, int k, int H,
                           int quant, f16* a16, float* ascale, hipStream_t s);
hipError_t launch_quant_rows_f32(const float* h, int R, int I, f16* h16, float* hscale,
                                 hipStream_t s);
hipError_t launch_act_quant_i8(const void* v, int dt, int rows, int cols, int8_t* q, float* sc,
                               hipStream_t s);
hipError_t launch_ffn_gate_up(const moe_packed_expert* experts, const int32_t* offsets,
                              uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E,
                              int k, const f16* a16, const float* ascale, void* h, int h_f32,
                              bool decode, hipStream_t s);
hipError_t launch_ffn_down(const moe_packed_expert* experts, const int32_t* offsets,
                           uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                           const f16* ain, const float* ascale, float* yp, int splits,
                           bool decode, hipStream_t s);
hipError_t launch_reduce_splits(const float* yp, int splits, size_t n, float* Y, hipStream_t s);
hipError_t launch_combine(const float* yp, int splits, const float* w, const int32_t* inv, int T,
                          int H, int k, void* out, int out_dt, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                              hipStream_t s);
hipError_t launch_pack_matrix(const moe_qmat* a, const moe_qmat* b_or_null, void* codes,
                              void* params, hipStream_t s);

}  // namespace moeq
