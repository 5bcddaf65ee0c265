// Host side of the C ABI: argument checks, workspace carving and dispatch.
// Every check runs before anything is enqueued; nothing here synchronises.
#include "common.h"
#include "profile.h"

using namespace moeq;

namespace {

constexpr int kMaxK = 32;

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_qmat(const moe_qmat& q, uint32_t rows, uint32_t cols) {
  if (q.rows != rows || q.cols != cols) return MOE_ERR_INVALID_ARG;
  if (!q.codes || !q.params) return MOE_ERR_INVALID_ARG;
  if (fmt_id(q.fmt, q.bits, q.group) < 0) return MOE_ERR_UNSUPPORTED;
  if (rows % 32 != 0 || cols % 128 != 0 || cols % q.group != 0) return MOE_ERR_INVALID_ARG;
  if (!aligned(q.codes, 16) || !aligned(q.params, 4)) return MOE_ERR_ALIGNMENT;
  if (q.n_outliers > 0) {
    if (!q.outliers || (uint64_t)q.n_outliers > (uint64_t)rows * cols) return MOE_ERR_INVALID_ARG;
    if (!aligned(q.outliers, 8)) return MOE_ERR_ALIGNMENT;
  }
  return MOE_OK;
}

moe_status check_canon(const moe_expert_canon* src) {
  if (!src) return MOE_ERR_INVALID_ARG;
  const uint32_t I = src->gate.rows, H = src->gate.cols;
  if (I == 0 || H == 0) return MOE_ERR_INVALID_ARG;
  // packed matrices are addressed with 32-bit byte offsets
  if ((uint64_t)I * H > (1ull << 31)) return MOE_ERR_UNSUPPORTED;
  moe_status s;
  if ((s = check_qmat(src->gate, I, H)) != MOE_OK) return s;
  if ((s = check_qmat(src->up, I, H)) != MOE_OK) return s;
  if ((s = check_qmat(src->down, H, I)) != MOE_OK) return s;
  return MOE_OK;
}

inline bool split_gu(const moe_expert_canon* src) {
  return src->up.fmt != src->gate.fmt || src->up.bits != src->gate.bits ||
         src->up.group != src->gate.group;
}

// byte offsets of the parts of one packed expert (each 256-aligned)
struct PackedSizes {
  size_t gu_codes, gu_params, up_codes, up_params, dn_codes, dn_params;
  size_t gu_rowptr, gu_ent, dn_rowptr, dn_ent, total;
};

PackedSizes packed_sizes(const moe_expert_canon* src) {
  PackedSizes p;
  const int I = (int)src->gate.rows, H = (int)src->gate.cols;
  const bool split = split_gu(src);
  const moe_qmat &g = src->gate, &u = src->up, &d = src->down;
  p.gu_codes = align256(packed_codes_bytes(split ? I : 2 * I, H, g.bits));
  p.gu_params = align256(packed_params_bytes(split ? I : 2 * I, H, g.fmt, g.bits, g.group));
  p.up_codes = split ? align256(packed_codes_bytes(I, H, u.bits)) : 0;
  p.up_params = split ? align256(packed_params_bytes(I, H, u.fmt, u.bits, u.group)) : 0;
  p.dn_codes = align256(packed_codes_bytes(H, I, d.bits));
  p.dn_params = align256(packed_params_bytes(H, I, d.fmt, d.bits, d.group));
  const uint64_t ngu = (uint64_t)g.n_outliers + u.n_outliers, ndn = d.n_outliers;
  p.gu_rowptr = ngu ? align256(outlier_rowptr_bytes(2 * I)) : 0;
  p.gu_ent = ngu ? align256(ngu * sizeof(OutEntry)) : 0;
  p.dn_rowptr = ndn ? align256(outlier_rowptr_bytes(H)) : 0;
  p.dn_ent = ndn ? align256(ndn * sizeof(OutEntry)) : 0;
  p.total = p.gu_codes + p.gu_params + p.up_codes + p.up_params + p.dn_codes + p.dn_params +
            p.gu_rowptr + p.gu_ent + p.dn_rowptr + p.dn_ent;
  return p;
}

moe_status check_sizes(int T, int H, int I, int E, int k) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || E > kMaxE) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > E || k > kMaxK) return MOE_ERR_INVALID_ARG;
  if (H % 128 != 0 || I % 128 != 0) return MOE_ERR_INVALID_ARG;
  if ((long)T * k > (1L << 30)) return MOE_ERR_INVALID_ARG;
  // the expert GEMMs address their fp16 input rows with 32-bit byte offsets
  if ((uint64_t)T * k * (H > I ? H : I) * 2 > 0xFFFFFFFFull) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                          \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

inline char* ws_at(void* ws, size_t off) { return (char*)ws + off; }

// phases of the grouped FFN (workspace already validated)
inline uint32_t effective_mask(uint32_t m) {
  return m ? m : (((1u << F_COUNT) - 1u) | kMaskSplitGU | kMaskNoFuse | kMaskOutliers);
}

// The int8 prefill GEMMs take the W4A8 format (4-bit, groups of 128) when
// the caller asks for them (MOE_MASK_INT8_GEMM), the layout holds their
// operands (int8 activations at prefill sizes) and no expert needs the split
// roles or outlier corrections; the fp16-held codes are still made when
// another format is present.
inline bool use_i8(const WsLayout& L, uint32_t m) {
  return L.i8 && (m & kMaskInt8) && (m & kI8Formats) && !(m & (kMaskSplitGU | kMaskOutliers));
}
inline bool need16(const WsLayout& L, uint32_t m) {
  return !use_i8(L, m) || (m & ((1u << F_COUNT) - 1u) & ~kI8Formats);
}

// the expert inputs: fp16 (or fp16-held int8 codes) when need16, the int8
// GEMMs' operands when i8
moe_status run_gather(const void* x, moe_dtype xdt, const int32_t* perm, int T, int H, int k,
                      moe_actq aq, const WsLayout& L, void* ws, bool want16, bool i8,
                      uint32_t* flags, hipStream_t s) {
  MOE_TRY(launch_gather_a(x, xdt, perm, T, k, H, aq != MOE_ACT_NONE,
                          want16 ? (f16*)ws_at(ws, L.a16) : nullptr, (float*)ws_at(ws, L.ascale),
                          i8 ? (int8_t*)ws_at(ws, L.a8) : nullptr,
                          i8 ? (float*)ws_at(ws, L.asum) : nullptr, flags, s));
  return MOE_OK;
}

// the transposed copy of a prefill GEMM's input (K columns) for its outlier
// corrections, when the layout has room for it (mask with the outlier bit)
moe_status outlier_inputs(const f16* a, int R, int K, const int32_t* offsets, int E,
                          const WsLayout& L, size_t at_off, void* ws, OutlierInputs& oi,
                          hipStream_t s) {
  oi = OutlierInputs{nullptr, 0, nullptr};
  if (!L.rp) return MOE_OK;
  f16* at = (f16*)ws_at(ws, at_off);
  int32_t* poff = (int32_t*)ws_at(ws, L.poff);
  MOE_TRY(launch_transpose_pad(a, R, K, offsets, E, at, L.rp, poff, s));
  oi = OutlierInputs{at, L.rp, poff};
  return MOE_OK;
}

moe_status run_gate_up(const moe_packed_expert* experts, uint32_t mask, const int32_t* offsets,
                       int T, int H, int I, int E, int k, moe_actq aq, const WsLayout& L, void* ws,
                       uint32_t* flags, hipStream_t s) {
  const f16* a16 = (const f16*)ws_at(ws, L.a16);
  OutlierInputs oi;
  moe_status st = outlier_inputs(a16, T * k, H, offsets, E, L, L.at_gu, ws, oi, s);
  if (st != MOE_OK) return st;
  const uint32_t m = effective_mask(mask);
  const I8Inputs i8 = use_i8(L, m) ? I8Inputs{(const int8_t*)ws_at(ws, L.a8),
                                               (const float*)ws_at(ws, L.asum)}
                                    : I8Inputs{nullptr, nullptr};
  MOE_TRY(launch_ffn_gate_up(experts, offsets, m, flags, T, H, I, E, k, a16,
                             aq != MOE_ACT_NONE ? (const float*)ws_at(ws, L.ascale) : nullptr,
                             ws_at(ws, L.h), aq == MOE_ACT_I8_XH, L.decode, oi, i8, s));
  return MOE_OK;
}

moe_status run_down(const moe_packed_expert* experts, uint32_t mask, const int32_t* offsets,
                    int T, int H, int I, int E, int k, moe_actq aq, const WsLayout& L, void* ws,
                    uint32_t* flags, float* yp, hipStream_t s) {
  const int R = T * k;
  const uint32_t m = effective_mask(mask);
  const f16* ain = (const f16*)ws_at(ws, L.h);
  const float* sc = nullptr;
  I8Inputs i8{nullptr, nullptr};
  if (aq == MOE_ACT_I8_XH) {
    // int8 codes of h: fp16-held for the fp16 kernels, bytes and sums for
    // the int8 ones
    const bool q8 = use_i8(L, m);
    f16* h16 = (f16*)ws_at(ws, L.h16);
    float* hs = (float*)ws_at(ws, L.hscale);
    int8_t* h8 = (int8_t*)ws_at(ws, L.h8);
    float* hsum = (float*)ws_at(ws, L.hsum);
    MOE_TRY(launch_quant_rows_f32((const float*)ws_at(ws, L.h), R, I,
                                  need16(L, m) ? h16 : nullptr, hs, q8 ? h8 : nullptr,
                                  q8 ? hsum : nullptr, s));
    ain = h16;
    sc = hs;
    if (q8) i8 = I8Inputs{h8, hsum};
  }
  OutlierInputs oi;
  moe_status st = outlier_inputs(ain, R, I, offsets, E, L, L.at_dn, ws, oi, s);
  if (st != MOE_OK) return st;
  MOE_TRY(launch_ffn_down(experts, offsets, m, flags, T, H, I, E, k, ain, sc, yp, L.splits,
                          L.decode, oi, i8, s));
  return MOE_OK;
}

// layout for a call with format mask `mask`; the transposed copies are
// addressed with 32-bit byte offsets too
moe_status layout_for(int T, int H, int I, int E, int k, moe_actq aq, uint32_t mask,
                      WsLayout& L) {
  L = ws_layout(T, H, I, E, k, aq, (effective_mask(mask) & kMaskOutliers) != 0);
  if (L.rp && (uint64_t)(H > I ? H : I) * (uint64_t)L.rp * 2 > 0xFFFFFFFFull)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_ws(int T, int H, int I, int E, int k, moe_actq aq, uint32_t mask, void* ws,
                    size_t ws_bytes, WsLayout& L) {
  moe_status st = check_sizes(T, H, I, E, k);
  if (st != MOE_OK) return st;
  if (aq < MOE_ACT_NONE || aq > MOE_ACT_I8_XH) return MOE_ERR_INVALID_ARG;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if ((st = layout_for(T, H, I, E, k, aq, mask, L)) != MOE_OK) return st;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status check_experts(const void* experts, const int32_t* offsets) {
  if (!experts || !offsets) return MOE_ERR_INVALID_ARG;
  if (!aligned(experts, 16) || !aligned(offsets, 4)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace

namespace moeq {

// The whole layer on a validated workspace `ws` (layout L). flags: where the
// call's flag word goes (nullptr: the workspace's own).
moe_status layer_forward_ws(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                            const moe_packed_expert* experts, uint32_t fmt_mask, int T, int H,
                            int I, int E, int k, moe_actq aq, void* out, moe_dtype out_dt,
                            int32_t* topk_ids, float* topk_w, void* ws, const WsLayout& L,
                            uint32_t* flags, hipStream_t s) {
  if (!experts) return MOE_ERR_INVALID_ARG;
  if (!aligned(experts, 16)) return MOE_ERR_ALIGNMENT;
  if (xdt != MOE_F32 && xdt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (out_dt != MOE_F32 && out_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !Wr || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(out, out_dt == MOE_F32 ? 16 : 8))
    return MOE_ERR_ALIGNMENT;
  if (!flags) flags = (uint32_t*)ws_at(ws, L.flags);
  int32_t* ids = topk_ids ? topk_ids : (int32_t*)ws_at(ws, L.ids);
  float* w = topk_w ? topk_w : (float*)ws_at(ws, L.w);
  int32_t* counts = (int32_t*)ws_at(ws, L.counts);
  int32_t* offsets = (int32_t*)ws_at(ws, L.offsets);
  int32_t* perm = (int32_t*)ws_at(ws, L.perm);
  int32_t* inv = (int32_t*)ws_at(ws, L.inv);
  float* yp = (float*)ws_at(ws, L.yp);
  double* rpart = (double*)ws_at(ws, L.rpart);
  const int kb = route_plan(T, H, E).kb;
  moe_status st;
  if (L.decode && front_fits(T, H, E, k)) {
    // small batch: top-k, permutation and gather in one block
    MOE_TRY(launch_route_logits(x, xdt, Wr, T, H, E, rpart, s));
    MOE_TRY(launch_front(rpart, kb, x, xdt, b, T, H, E, k, ids, w, counts, offsets, perm, inv,
                         flags, aq != MOE_ACT_NONE, (f16*)ws_at(ws, L.a16),
                         (float*)ws_at(ws, L.ascale), s));
  } else {
    if (cert_plan(T, H, E, xdt).use) {
      MOE_TRY(launch_route_cert(x, xdt, Wr, b, T, H, E, k, ids, w, rpart, s));
    } else {
      MOE_TRY(launch_route_logits(x, xdt, Wr, T, H, E, rpart, s));
      MOE_TRY(launch_route_topk(rpart, kb, b, T, E, k, ids, w, nullptr, s));
    }
    MOE_TRY(launch_permute(ids, T, k, E, counts, offsets, perm, inv, flags,
                           ws_at(ws, L.pscratch), s));
    const uint32_t m = effective_mask(fmt_mask);
    const moe_status sg = run_gather(x, xdt, perm, T, H, k, aq, L, ws, need16(L, m), use_i8(L, m),
                                     flags, s);
    if (sg != MOE_OK) return sg;
  }
  const FusedPlan fp = fused_plan(T, H, I, E, k, aq);
  const uint32_t mask = effective_mask(fmt_mask);
  if (fp.use && !(mask & kMaskNoFuse)) {
    // small decode batch: gate/up, SwiGLU and down in one launch per format,
    // then the sum of its partial planes
    int ns = 0;
    const hipError_t e = launch_ffn_fused(experts, offsets, mask, flags, T, H, I, E, k,
                                          (const f16*)ws_at(ws, L.a16),
                                          aq != MOE_ACT_NONE ? (const float*)ws_at(ws, L.ascale)
                                                             : nullptr,
                                          yp, fp.S, fp.ns, &ns, s);
    if (e == hipSuccess)
      return hip_status(launch_combine_slices(yp, ns, w, inv, T, H, k, out, out_dt, s));
    if (e != hipErrorNotSupported) return MOE_ERR_HIP;
    // no slice width fits these formats: the two-launch path below
  }
  st = run_gate_up(experts, fmt_mask, offsets, T, H, I, E, k, aq, L, ws, flags, s);
  if (st != MOE_OK) return st;
  st = run_down(experts, fmt_mask, offsets, T, H, I, E, k, aq, L, ws, flags, yp, s);
  if (st != MOE_OK) return st;
  return hip_status(launch_combine(yp, L.decode ? L.splits : 1, w, inv, T, H, k, out, out_dt, s));
}

moe_status check_layer_sizes(int T, int H, int I, int E, int k, moe_actq aq, uint32_t fmt_mask,
                             WsLayout& L) {
  moe_status st = check_sizes(T, H, I, E, k);
  if (st != MOE_OK) return st;
  if (aq < MOE_ACT_NONE || aq > MOE_ACT_I8_XH) return MOE_ERR_INVALID_ARG;
  return layout_for(T, H, I, E, k, aq, fmt_mask, L);
}

}  // namespace moeq

extern "C" {

int moe_version(void) { return 20100; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported format";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t moe_packed_expert_bytes(const moe_expert_canon* src) {
  if (check_canon(src) != MOE_OK) return 0;
  return packed_sizes(src).total;
}

moe_status moe_pack_expert(const moe_expert_canon* src, void* dst_dev, size_t dst_bytes,
                           moe_packed_expert* out_desc, void* stream) {
  moe_status st = check_canon(src);
  if (st != MOE_OK) return st;
  if (!dst_dev || !out_desc) return MOE_ERR_INVALID_ARG;
  if (!aligned(dst_dev, 256)) return MOE_ERR_ALIGNMENT;
  PackedSizes p = packed_sizes(src);
  if (dst_bytes < p.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const bool split = split_gu(src);
  char* at = (char*)dst_dev;
  auto take = [&](size_t bytes) -> void* {
    void* r = bytes ? at : nullptr;
    at += bytes;
    return r;
  };
  void* guc = take(p.gu_codes);
  void* gup = take(p.gu_params);
  void* upc = take(p.up_codes);
  void* upp = take(p.up_params);
  void* dnc = take(p.dn_codes);
  void* dnp = take(p.dn_params);
  void* gur = take(p.gu_rowptr);
  void* gue = take(p.gu_ent);
  void* dnr = take(p.dn_rowptr);
  void* dne = take(p.dn_ent);
  if (split) {
    MOE_TRY(launch_pack_matrix(&src->gate, nullptr, guc, gup, s));
    MOE_TRY(launch_pack_matrix(&src->up, nullptr, upc, upp, s));
  } else {
    MOE_TRY(launch_pack_matrix(&src->gate, &src->up, guc, gup, s));
  }
  MOE_TRY(launch_pack_matrix(&src->down, nullptr, dnc, dnp, s));
  const uint32_t ngu = src->gate.n_outliers + src->up.n_outliers, ndn = src->down.n_outliers;
  if (ngu) MOE_TRY(launch_pack_outliers(&src->gate, &src->up, (uint32_t*)gur, (OutEntry*)gue, s));
  if (ndn) MOE_TRY(launch_pack_outliers(&src->down, nullptr, (uint32_t*)dnr, (OutEntry*)dne, s));
  moe_packed_expert d = {};
  d.gu_fmt = src->gate.fmt;
  d.gu_bits = src->gate.bits;
  d.gu_group = src->gate.group;
  d.up_fmt = src->up.fmt;
  d.up_bits = src->up.bits;
  d.up_group = src->up.group;
  d.dn_fmt = src->down.fmt;
  d.dn_bits = src->down.bits;
  d.dn_group = src->down.group;
  d.H = src->gate.cols;
  d.I = src->gate.rows;
  d.layout = split ? MOE_PACK_SPLIT_GU : 0u;
  d.n_out_gu = ngu;
  d.n_out_dn = ndn;
  d.gu_codes = guc;
  d.gu_params = gup;
  d.up_codes = split ? upc : guc;
  d.up_params = split ? upp : gup;
  d.dn_codes = dnc;
  d.dn_params = dnp;
  d.out_gu_rowptr = gur;
  d.out_gu_entries = gue;
  d.out_dn_rowptr = dnr;
  d.out_dn_entries = dne;
  *out_desc = d;
  return MOE_OK;
}

uint32_t moe_format_mask(const moe_packed_expert* descs, int E) {
  if (!descs || E <= 0) return 0;
  uint32_t m = 0;
  for (int e = 0; e < E; ++e) {
    const int a = fmt_id(descs[e].gu_fmt, descs[e].gu_bits, descs[e].gu_group);
    const int u = fmt_id(descs[e].up_fmt, descs[e].up_bits, descs[e].up_group);
    const int b = fmt_id(descs[e].dn_fmt, descs[e].dn_bits, descs[e].dn_group);
    if (a >= 0) m |= 1u << a;
    if (u >= 0) m |= 1u << u;
    if (b >= 0) m |= 1u << b;
    if (descs[e].layout & MOE_PACK_SPLIT_GU) m |= kMaskSplitGU;
    if ((descs[e].layout & MOE_PACK_SPLIT_GU) || descs[e].n_out_gu || descs[e].n_out_dn || a != b)
      m |= kMaskNoFuse;
    if (descs[e].n_out_gu || descs[e].n_out_dn) m |= kMaskOutliers;
  }
  return m;
}

size_t moe_workspace_size(int T, int H, int I, int E, int k, moe_actq aq) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return 0;
  return ws_layout(T, H, I, E, k, aq).total;
}

size_t moe_route_workspace_size(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return align256(route_ws_bytes(T, H, E));
}

moe_status moe_route(const void* x, moe_dtype xdt, const float* Wr, const float* b, int T, int H,
                     int E, int k, int32_t* topk_ids, float* topk_w, float* logits, void* ws,
                     size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return MOE_ERR_INVALID_ARG;
  if (xdt != MOE_F32 && xdt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !Wr || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < moe_route_workspace_size(T, H, E)) return MOE_ERR_WORKSPACE;
  if (!logits && cert_plan(T, H, E, xdt).use)
    return hip_status(launch_route_cert(x, xdt, Wr, b, T, H, E, k, topk_ids, topk_w, ws,
                                        (hipStream_t)stream));
  return hip_status(launch_route(x, xdt, Wr, b, T, H, E, k, topk_ids, topk_w, logits,
                                 (double*)ws, (hipStream_t)stream));
}

static moe_status check_route_args(const void* x, moe_dtype xdt, const float* Wr, int T, int H,
                                   int E, void* ws, size_t ws_bytes) {
  if (T < 0 || H <= 0 || E <= 0 || E > kMaxE) return MOE_ERR_INVALID_ARG;
  if (xdt != MOE_F32 && xdt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !Wr || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < moe_route_workspace_size(T, H, E)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status moe_route_i8(const void* x, moe_dtype xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, const float* scale, const int32_t* zero, int32_t* topk_ids,
                        float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream) {
  if (k < 1 || k > E || k > kMaxK) return MOE_ERR_INVALID_ARG;
  moe_status st = check_route_args(x, xdt, Wr, T, H, E, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!scale || !zero || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(launch_route_logits(x, xdt, Wr, T, H, E, (double*)ws, s));
  return hip_status(launch_route_topk_q((const double*)ws, route_plan(T, H, E).kb, b, T, E, k, scale,
                                        zero, topk_ids, topk_w, logits, s));
}

moe_status moe_router_logit_range(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                                  int T, int H, int E, double* lo, double* hi, void* ws,
                                  size_t ws_bytes, void* stream) {
  moe_status st = check_route_args(x, xdt, Wr, T, H, E, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!lo || !hi) return MOE_ERR_INVALID_ARG;
  if (!aligned(lo, 8) || !aligned(hi, 8)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(launch_route_logits(x, xdt, Wr, T, H, E, (double*)ws, s));
  return hip_status(
      launch_logit_range((const double*)ws, route_plan(T, H, E).kb, b, T, E, lo, hi, s));
}

moe_status moe_router_i8_params(const double* lo, const double* hi, int E, int shared,
                                float* scale, int32_t* zero) {
  if (!lo || !hi || !scale || !zero || E < 1 || E > kMaxE) return MOE_ERR_INVALID_ARG;
  double glo = lo[0], ghi = hi[0];
  for (int e = 0; e < E; ++e) {
    const double a = lo[e], b = hi[e];
    if (!(a <= b) || a < -1e30 || b > 1e30) return MOE_ERR_INVALID_ARG;
    glo = a < glo ? a : glo;
    ghi = b > ghi ? b : ghi;
  }
  for (int e = 0; e < E; ++e) {
    const double a = shared ? glo : lo[e], b = shared ? ghi : hi[e];
    float sc = (float)((b - a) / 255.0);
    if (!(sc >= 1.17549435e-38f)) sc = 1.17549435e-38f;  // smallest normal fp32
    const double z = -128.0 - rint(a / (double)sc);
    scale[e] = sc;
    zero[e] = (int32_t)(z < -2147483648.0 ? -2147483648.0 : (z > 2147483647.0 ? 2147483647.0 : z));
  }
  return MOE_OK;
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E <= 0 || (long)T * k > (1L << 30)) return 0;
  return 256 + permute_plan(T * k, E).scratch_bytes;
}

moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv, void* ws,
                       size_t ws_bytes, void* stream) {
  if (T < 0 || E <= 0 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if ((long)T * k > (1L << 30)) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm_token || !inv)) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < moe_permute_workspace_size(T, k, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* flags = (uint32_t*)ws;
  MOE_TRY(launch_permute(topk_ids, T, k, E, counts, offsets, perm_token, inv, flags,
                         (char*)ws + 256, s));
  return MOE_OK;
}

moe_status moe_ffn_gather(const void* x, moe_dtype xdt, const int32_t* perm_token, int T, int H,
                          int I, int E, int k, moe_actq aq, void* ws, size_t ws_bytes,
                          void* stream) {
  WsLayout L;
  // the gather's regions do not depend on the format mask
  moe_status st = check_ws(T, H, I, E, k, aq, 1u, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  if (xdt != MOE_F32 && xdt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm_token) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16)) return MOE_ERR_ALIGNMENT;
  return run_gather(x, xdt, perm_token, T, H, k, aq, L, ws, true, false,
                    (uint32_t*)ws_at(ws, L.flags), (hipStream_t)stream);
}

moe_status moe_ffn_gate_up(const moe_packed_expert* experts, uint32_t fmt_mask,
                           const int32_t* offsets, int T, int H, int I, int E, int k, moe_actq aq,
                           void* ws, size_t ws_bytes, void* stream) {
  WsLayout L;
  moe_status st = check_ws(T, H, I, E, k, aq, fmt_mask, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  if ((st = check_experts(experts, offsets)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  // the phase entry points keep the fp16 kernels (the gather made no int8
  // operands for them)
  return run_gate_up(experts, fmt_mask & ~kMaskInt8, offsets, T, H, I, E, k, aq, L, ws,
                     (uint32_t*)ws_at(ws, L.flags), (hipStream_t)stream);
}

moe_status moe_ffn_down(const moe_packed_expert* experts, uint32_t fmt_mask,
                        const int32_t* offsets, int T, int H, int I, int E, int k, moe_actq aq,
                        float* Y, void* ws, size_t ws_bytes, void* stream) {
  WsLayout L;
  moe_status st = check_ws(T, H, I, E, k, aq, fmt_mask, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  if ((st = check_experts(experts, offsets)) != MOE_OK) return st;
  if (T > 0 && !Y) return MOE_ERR_INVALID_ARG;
  if (!aligned(Y, 16)) return MOE_ERR_ALIGNMENT;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const size_t n = (size_t)T * k * H;
  if (L.decode && L.splits > 1) {
    float* yp = (float*)ws_at(ws, L.yp);
    st = run_down(experts, fmt_mask & ~kMaskInt8, offsets, T, H, I, E, k, aq, L, ws,
                  (uint32_t*)ws_at(ws, L.flags), yp, s);
    if (st != MOE_OK) return st;
    return hip_status(launch_reduce_splits(yp, L.splits, n, Y, s));
  }
  return run_down(experts, fmt_mask & ~kMaskInt8, offsets, T, H, I, E, k, aq, L, ws,
                  (uint32_t*)ws_at(ws, L.flags), Y, s);
}

moe_status moe_grouped_ffn_q(const void* x, moe_dtype xdt, const moe_packed_expert* experts,
                             uint32_t fmt_mask, const int32_t* offsets, const int32_t* perm_token,
                             int T, int H, int I, int E, int k, moe_actq aq, float* Y, void* ws,
                             size_t ws_bytes, void* stream) {
  WsLayout L;
  moe_status st = check_ws(T, H, I, E, k, aq, fmt_mask, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  if ((st = check_experts(experts, offsets)) != MOE_OK) return st;
  if (xdt != MOE_F32 && xdt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !perm_token || !Y) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(Y, 16)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* flags = (uint32_t*)ws_at(ws, L.flags);
  const uint32_t m = effective_mask(fmt_mask);
  st = run_gather(x, xdt, perm_token, T, H, k, aq, L, ws, need16(L, m), use_i8(L, m), flags, s);
  if (st != MOE_OK) return st;
  st = run_gate_up(experts, fmt_mask, offsets, T, H, I, E, k, aq, L, ws, flags, s);
  if (st != MOE_OK) return st;
  if (L.decode && L.splits > 1) {
    float* yp = (float*)ws_at(ws, L.yp);
    st = run_down(experts, fmt_mask, offsets, T, H, I, E, k, aq, L, ws, flags, yp, s);
    if (st != MOE_OK) return st;
    return hip_status(launch_reduce_splits(yp, L.splits, (size_t)T * k * H, Y, s));
  }
  return run_down(experts, fmt_mask, offsets, T, H, I, E, k, aq, L, ws, flags, Y, s);
}

moe_status moe_combine(const float* Y, const float* topk_w, const int32_t* inv, int T, int H,
                       int k, void* out, moe_dtype out_dt, void* stream) {
  if (T < 0 || H <= 0 || k < 1 || H % 4 != 0) return MOE_ERR_INVALID_ARG;
  if (out_dt != MOE_F32 && out_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!Y || !topk_w || !inv || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(Y, 16) || !aligned(out, out_dt == MOE_F32 ? 16 : 8)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_combine(Y, 1, topk_w, inv, T, H, k, out, out_dt, (hipStream_t)stream));
}

moe_status moe_layer_forward(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                             const moe_packed_expert* experts, uint32_t fmt_mask, int T, int H,
                             int I, int E, int k, moe_actq aq, void* out, moe_dtype out_dt,
                             int32_t* topk_ids,
                             float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  WsLayout L;
  moe_status st = check_ws(T, H, I, E, k, aq, fmt_mask, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  return layer_forward_ws(x, xdt, Wr, b, experts, fmt_mask, T, H, I, E, k, aq, out, out_dt,
                          topk_ids, topk_w, ws, L, nullptr, (hipStream_t)stream);
}

moe_status moe_act_quant_i8(const void* v, moe_dtype dt, int rows, int cols, int8_t* q, float* s,
                            void* stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!v || !q || !s) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_act_quant_i8(v, dt, rows, cols, q, s, (hipStream_t)stream));
}

moe_status moe_expert_histogram(const int32_t* topk_ids, int T, int k, int E, int64_t* hist,
                                void* stream) {
  if (T < 0 || k < 1 || E < 1 || E > kMaxE) return MOE_ERR_INVALID_ARG;
  if ((long)T * k > (1L << 30)) return MOE_ERR_INVALID_ARG;
  if (!hist || (T > 0 && !topk_ids)) return MOE_ERR_INVALID_ARG;
  if (!aligned(hist, 8) || !aligned(topk_ids, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_expert_histogram(topk_ids, (long)T * k, E, hist, (hipStream_t)stream));
}

moe_status moe_plan_tiers(const int64_t* counts, int E, const uint64_t* tier_bytes, int ntiers,
                          uint64_t budget_bytes, int32_t* tier_of, uint64_t* used_bytes) {
  if (!counts || !tier_bytes || !tier_of) return MOE_ERR_INVALID_ARG;
  if (E < 1 || E > (1 << 16) || ntiers < 1 || ntiers > 16) return MOE_ERR_INVALID_ARG;
  for (int t = 0; t < ntiers; ++t) {
    if (tier_bytes[t] > (1ull << 40)) return MOE_ERR_INVALID_ARG;
    if (t > 0 && tier_bytes[t] > tier_bytes[t - 1]) return MOE_ERR_INVALID_ARG;
  }
  for (int e = 0; e < E; ++e)
    if (counts[e] < 0) return MOE_ERR_INVALID_ARG;
  return plan_tiers(counts, E, tier_bytes, ntiers, budget_bytes, tier_of, used_bytes)
             ? MOE_OK
             : MOE_ERR_INVALID_ARG;
}

moe_status moe_stream_read(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                           void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !sink || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_stream_read(src, bytes, nontemporal, sink, (hipStream_t)stream));
}

moe_status moe_stream_read_shaped(const void* src, size_t bytes, int nontemporal, int blocks,
                                  int waves, int inflight, int layout, uint32_t* sink,
                                  void* stream) {
  if (blocks < 1 || blocks > MOE_STREAM_MAX_BLOCKS || waves < 1 || waves > 16 ||
      (inflight != 1 && inflight != 2 && inflight != 4 && inflight != 8 && inflight != 16) ||
      (layout != 0 && layout != 1))
    return MOE_ERR_INVALID_ARG;
  if (bytes == 0) return MOE_OK;
  if (!src || !sink || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_stream_read_shaped(src, bytes, nontemporal, blocks, waves, inflight,
                                              layout, sink, (hipStream_t)stream));
}

}  // extern "C"
