/*
 * moeq.h: C ABI of a quantized Mixture-of-Experts FFN layer (forward pass)
 * for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (Baidu Cloud article on quantized MoE LLM
 * inference, "expert routing" section; MoE mixed-precision field notes,
 * section 2.1): for every token t of the hidden states x[T,H]
 *     L[t,:]   = x[t,:] Wr^T + b                       (router, fp32 in, fp64 accumulate)
 *     ids[t,:] = the k experts with the largest L[t,e], descending, ties to the
 *                lower expert index ("Sparse activation ... GPT-4's 2%
 *                activation", section 2.2: keep the K highest of E logits)
 *     w[t,:]   = softmax of L[t, ids[t,:]]
 *     out[t,:] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t,:])
 *     FFN_e(a) = (silu(a Wg_e^T) * (a Wu_e^T)) Wd_e^T     (SwiGLU expert)
 * Expert weights are block-quantised with a per-expert bit width and group
 * size ("AlphaQ" blog, section 4.2; expert-aware quantisation digest: hot
 * experts 4-bit, cold experts 2-bit) and are decoded on the fly. Optionally
 * the expert inputs are quantised per token to int8 (mixed-precision notes,
 * sections 2.1-2.2); the router always sees the unquantised x.
 *
 * Conventions for every entry point
 *  - Pointers named *_dev or documented "device" are device (HBM) pointers;
 *    everything else is host memory. The caller owns every buffer. The library
 *    keeps no state between calls and never allocates.
 *  - `stream` is a hipStream_t (NULL = the null stream). Compute entry points
 *    only enqueue kernels on it and return; they never synchronise.
 *  - Arguments are checked before anything is enqueued. A failing check
 *    returns a negative moe_status and enqueues nothing. A failed launch
 *    returns MOE_ERR_HIP.
 *  - Data-dependent trouble found on the device (an expert id out of range,
 *    NaN router logits) sets bits of the flag word at the start of the
 *    workspace (MOE_FLAG_*), readable after the stream synchronises.
 *    moe_permute and moe_layer_forward set it (overwriting what a previous
 *    call left); the FFN phases only add bits to it.
 *  - Matrices are row-major; int32 indices; fp32 weights of the router.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, k outside [1,E], ... */
  MOE_ERR_UNSUPPORTED = -2, /* format / bit width / group size not provided */
  MOE_ERR_ALIGNMENT = -3,   /* pointer not aligned as documented */
  MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = -5          /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Element formats of a weight block.
 * MOE_W_ASYM: w = s*q + m, q unsigned b-bit (b in {1,2,3,4}), fp16 s and m
 *             per group; decoded value rounded once to fp32. 1 bit is the
 *             sub-2-bit tier for the coldest experts (expert-aware
 *             quantisation digest, conclusion); 3 bits the gate's width in
 *             the per-matrix mix of the "AlphaQ" blog, section 2.2.
 * MOE_W_E2M1: w = e2m1(q) * s, 4-bit OCP-MX e2m1 element (bit 3 sign, two
 *             exponent bits with bias 1, one mantissa bit: magnitudes
 *             0, .5, 1, 1.5, 2, 3, 4, 6), fp16 s per group (the 4-bit
 *             floating-point weights of the quantized-MoE article). */
typedef enum { MOE_W_ASYM = 1, MOE_W_E2M1 = 2 } moe_wfmt;

/* Per-token dynamic int8 expert inputs (mixed-precision notes, section 2.1):
 * per row, s = fp32(absmax)/127 (fp32 division, correctly rounded),
 * q = clamp(rint(v/s), -127, 127) (round half to even), a zero row gives
 * s = 0, q = 0.
 * MOE_ACT_I8_X: x before gate/up; MOE_ACT_I8_XH: x, and h before down. */
typedef enum { MOE_ACT_NONE = 0, MOE_ACT_I8_X = 1, MOE_ACT_I8_XH = 2 } moe_actq;

enum {
  MOE_FLAG_BAD_EXPERT_ID = 1u << 0, /* an id outside [0,E) reached moe_permute */
  MOE_FLAG_NAN_LOGIT = 1u << 1,     /* a router logit was NaN (routing undefined) */
  MOE_FLAG_FORMAT_NOT_LAUNCHED = 1u << 2, /* an expert with rows has a format outside
                                             fmt_mask: its rows were not computed */
  MOE_FLAG_BAD_SEGMENT = 1u << 3,   /* caller offsets leave [0, T*k] or decrease: each
                                       segment was clamped to [offsets[e], T*k) and
                                       rows outside it were not computed */
  MOE_FLAG_EXPERT_SHAPE = 1u << 4,  /* an expert with rows has a descriptor whose H or
                                       I differs from the call's: its rows were not
                                       computed */
  MOE_FLAG_FP16_RANGE = 1u << 5     /* an expert input (fp16 path) or a SwiGLU output h
                                       stored as fp16 exceeded |v| = 65504: it became
                                       +-inf, and so did the rows it feeds */
};

/* Routing id that moe_route writes in every slot of a token whose router
 * logits include a NaN (the token's weights are 0). moe_permute drops such
 * assignments and raises MOE_FLAG_NAN_LOGIT. */
#define MOE_ID_NAN (-2)

/* One weight matrix W[rows, cols] in the canonical block format.
 * Groups of `group` consecutive elements along cols (the GEMM's K).
 * codes (device): uint8 [rows, row_bytes], row_bytes = cols*bits/8 rounded
 *   up to a multiple of 16 (padding bytes are ignored). A row's codes are one
 *   little-endian bit stream, element e at bits [b*e, b*e + b), bit i of the
 *   stream being bit i % 8 of byte i / 8: 4-bit: element 2i in the low nibble
 *   of byte i, 2i+1 in the high nibble; 2-bit: element 4i+j in bits
 *   [2j, 2j+1] of byte i; 1-bit: element 8i+j in bit j of byte i; 3-bit:
 *   elements 8i..8i+7 in the 24-bit little-endian word of bytes 3i..3i+2,
 *   element 8i+j at bits [3j, 3j+2].
 * params (device): fp16 [rows, cols/group] scales for MOE_W_E2M1, or
 *   [rows, cols/group] (scale, min) pairs for MOE_W_ASYM, row-major.
 * outliers (device, optional; MoE mixed-precision field notes, section 4.2:
 *   the largest ~0.05% of the weights kept in fp16, the rest low-bit):
 *   n_outliers records of 8 bytes {uint32 index = row * cols + col; uint16
 *   fp16 value; uint16 0}, indices strictly ascending. Each listed element
 *   takes its fp16 value instead of its block decode. n_outliers == 0: none
 *   (outliers may be NULL).
 * Supported: ASYM with bits 1, 2, 3 or 4 and group 16/32/64/128; E2M1 with
 * bits 4 and group 16/32/64/128. rows % 32 == 0; cols % 128 == 0; codes
 * 16-byte aligned, params 4-byte aligned, outliers 8-byte aligned. */
typedef struct {
  uint8_t fmt;    /* moe_wfmt */
  uint8_t bits;   /* 1, 2, 3 or 4 */
  uint16_t group; /* 16, 32, 64 or 128 */
  uint32_t rows;
  uint32_t cols;
  uint32_t n_outliers;
  const void* codes;
  const void* params;
  const void* outliers;
} moe_qmat;

/* One expert: gate [I,H], up [I,H], down [H,I], each with its own format
 * (the per-expert, per-matrix bit widths of the "AlphaQ" blog, sections 2.2
 * and 4.2). */
typedef struct {
  moe_qmat gate, up, down;
} moe_expert_canon;

/* Layout bit of a packed expert: gate and up are separate streams (their
 * formats differ); otherwise their 32-row tiles are interleaved in one. */
#define MOE_PACK_SPLIT_GU 1u

/* Device-layout descriptor of one packed expert, filled by moe_pack_expert.
 * The pointed-to layout is private to the library (32-row by 64- or 128-
 * column tiles in matrix-core fragment order; gate and up tiles interleaved
 * when they share a format). An array of E of these, copied to device memory
 * by the caller, is what the FFN entry points take. 128 bytes. */
typedef struct {
  uint8_t gu_fmt, gu_bits; /* gate's format (and up's when interleaved) */
  uint16_t gu_group;
  uint8_t dn_fmt, dn_bits;
  uint16_t dn_group;
  uint32_t H, I;
  uint8_t up_fmt, up_bits; /* up's format */
  uint16_t up_group;
  uint32_t layout;                 /* MOE_PACK_SPLIT_GU or 0 */
  uint32_t n_out_gu, n_out_dn;     /* outliers of gate + up, of down */
  const void* gu_codes;            /* gate (+ up interleaved) */
  const void* gu_params;
  const void* dn_codes;
  const void* dn_params;
  const void* up_codes;            /* split layout only */
  const void* up_params;
  const void* out_gu_rowptr;       /* outlier lists (n_out_* > 0 only) */
  const void* out_gu_entries;
  const void* out_dn_rowptr;
  const void* out_dn_entries;
  uint64_t reserved[2];
} moe_packed_expert;

/* Bytes of device memory moe_pack_expert needs for this expert (0 if the
 * descriptor is invalid or unsupported). Host only. */
size_t moe_packed_expert_bytes(const moe_expert_canon* src);

/* Repack one expert from the canonical format (device planes named in *src)
 * into the device layout at dst_dev (256-byte aligned, dst_bytes >=
 * moe_packed_expert_bytes(src)). Fills *out_desc (host). Enqueues the repack
 * on `stream`; the canonical planes and outlier lists must stay valid until
 * it has run. Gate and up are interleaved when their formats agree, else
 * stored as separate streams (MOE_PACK_SPLIT_GU). Outliers become per-row
 * lists of (column, fp32 difference between the fp16 outlier and the fp16
 * value the kernels decode there), added in the GEMM epilogues.
 * I * H <= 2^31 (else MOE_ERR_UNSUPPORTED: the kernels address a packed
 * matrix with 32-bit byte offsets); n_outliers <= rows * cols. */
moe_status moe_pack_expert(const moe_expert_canon* src, void* dst_dev, size_t dst_bytes,
                           moe_packed_expert* out_desc, void* stream);

/* Bit mask of the block formats used by E packed experts (host array of the
 * descriptors moe_pack_expert filled): bit i is set when some gate, up or
 * down matrix has format i, with i = 4*c + g, c = 0 asym 4-bit, 1 asym 2-bit,
 * 2 e2m1, 3 asym 1-bit, 4 asym 3-bit, and g = 0,1,2,3 for group 16, 32, 64,
 * 128; bit 31 (MOE_MASK_SPLIT_GU) is set when some expert has the split
 * gate/up layout, bit 30 (MOE_MASK_NO_FUSE) when some expert has the split
 * layout, outlier lists or a down format other than its gate/up format (the
 * fused decode kernel of moe_layer_forward then stays unused), bit 29
 * (MOE_MASK_OUTLIERS) when some matrix carries an outlier list (prefill-sized
 * calls then copy each GEMM's input rows into a transposed workspace buffer
 * that the outlier corrections read; without the bit, experts with outlier
 * lists flag MOE_FLAG_FORMAT_NOT_LAUNCHED at prefill sizes and their outputs
 * lack the corrections). The FFN entry points take this mask (fmt_mask) and
 * run one
 * kernel per format (and role) in it; 0 means every supported format
 * (correct for any expert set, but each absent format still costs launches).
 * Experts whose format is missing from a non-zero mask are skipped and flag
 * MOE_FLAG_FORMAT_NOT_LAUNCHED. Host only. */
#define MOE_MASK_SPLIT_GU (1u << 31)
#define MOE_MASK_NO_FUSE (1u << 30)
#define MOE_MASK_OUTLIERS (1u << 29)
/* Bit 28 (MOE_MASK_INT8_GEMM), never set by moe_format_mask: a caller that
 * sets it asks moe_layer_forward, moe_layer_forward_noalloc and
 * moe_grouped_ffn_q to run the prefill GEMMs of asymmetric 4-bit group-128
 * experts on the int8 matrix cores when the activations are int8 (integer
 * group sums scaled into fp32 per group: the same result up to fp32
 * rounding), unless some expert needs the split roles or outlier lists.
 * Measured slightly slower than the default fp16 kernels on this GPU, and
 * closer to the exact result (no fp16 rounding of the decoded weights). The
 * phase entry points (moe_ffn_*) ignore it. */
#define MOE_MASK_INT8_GEMM (1u << 28)
/* Bit 27 (MOE_MASK_SHARED_TILE), never set by moe_format_mask: at decode
 * sizes, run every gate/up and down launch of the two-launch path on the
 * shared-token-tile GEMV (four wavefronts on four row groups over the same K
 * tile, the 32 token rows of that tile loaded into LDS once per block).
 * Without the bit it runs the launches whose wavefront streams are short (at
 * most 32 K tiles) and whose blocks fill a round of the device's block slots,
 * and the gate/up launches whose blocks fill two rounds. The single-launch
 * decode kernel, where moe_layer_forward takes it, is not affected. Same
 * results as without the bit up to fp32 summation order. A kernel-selection
 * control for tuning and tests. */
#define MOE_MASK_SHARED_TILE (1u << 27)
uint32_t moe_format_mask(const moe_packed_expert* descs, int E);

/* Workspace bytes the layer entry points need for these sizes, with any
 * fmt_mask (a mask without MOE_MASK_OUTLIERS needs less: at prefill sizes the
 * transposed copy of the GEMM inputs, up to max(H, I) * (T*k + 31*min(T*k, E))
 * fp16 values, is left out; moe_layer_forward_noalloc uses the smaller size).
 * Host only. */
size_t moe_workspace_size(int T, int H, int I, int E, int k, moe_actq aq);

/* Workspace bytes moe_route needs for these sizes (fp64 partial logits of
 * its split hidden dimension; 0 when T <= 0). Host only. */
size_t moe_route_workspace_size(int T, int H, int E);

/* Router + top-k + softmax (steps 1-2 above).
 * x (device): [T,H] fp32 or bf16 (xdt). Wr (device): fp32 [E,H]. b (device):
 * fp32 [E] or NULL (no bias). Logits are accumulated in fp64 so that the
 * selection matches an exact evaluation except on near-ties; the partial
 * sums of a split hidden dimension are added in a fixed order, so results
 * are the same run to run.
 * Outputs (device): topk_ids int32 [T,k] (descending logit), topk_w fp32
 * [T,k] (softmax over the k selected logits, computed in fp64), logits fp32
 * [T,E] (optional, NULL to skip). A token whose logits include a NaN gets
 * MOE_ID_NAN in every slot and weights 0.
 * ws (device): at least moe_route_workspace_size(T, H, E) bytes, 256-byte
 * aligned; scratch, contents on return unspecified.
 * Constraints: 1 <= k <= min(E, 32), E <= 256, H % 8 == 0, x/Wr 16-byte
 * aligned. T == 0 is a no-op. */
moe_status moe_route(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                     int T, int H, int E, int k, int32_t* topk_ids, float* topk_w,
                     float* logits, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_permute needs: the 256-byte flag block, plus, for
 * more than 8192 assignments, per-block expert counts of the multi-block
 * sort (0 on invalid sizes). Host only. */
size_t moe_permute_workspace_size(int T, int k, int E);

/* Stable counting sort of the T*k assignments a = t*k + j by expert.
 * topk_ids (device) int32 [T,k]. Outputs (device, int32): counts [E],
 * offsets [E+1] (exclusive prefix sum, offsets[E] = T*k), perm_token [T*k]
 * (token of the r-th sorted assignment; ascending token inside each
 * expert's segment), inv [T*k] (inv[a] = r). ws/ws_bytes: at least
 * moe_permute_workspace_size(T, k, E) bytes, 256-byte aligned; its first
 * word is the flag word, the rest scratch.
 * Ids outside [0,E) are dropped (inv = -1): MOE_ID_NAN raises
 * MOE_FLAG_NAN_LOGIT, any other MOE_FLAG_BAD_EXPERT_ID. The flag word is
 * written with exactly the bits this call found. T*k <= 2^30. */
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv, void* ws,
                       size_t ws_bytes, void* stream);

/* Grouped expert FFN over the permuted assignments (steps 3-5):
 * for every sorted row r of expert e (offsets[e] <= r < offsets[e+1]):
 *   Y[r,:] = FFN_e(x[perm_token[r], :]).
 * experts (device): moe_packed_expert [E]; fmt_mask: see moe_format_mask.
 * Y (device): fp32 [T*k, H].
 * Decoded weights and the SwiGLU output h run through fp16 matrix-core
 * operations with fp32 accumulation; with int8 activations the int8 codes
 * enter the matrix cores exactly and the per-row scales are applied in fp32.
 * ws: at least moe_workspace_size(T, H, I, E, k, aq) bytes, 256-aligned.
 * Constraints: H % 128 == 0, I % 128 == 0, every expert packed with these H, I;
 * x and Y 16-byte aligned; T * k * max(H, I) * 2 < 2^32 (else
 * MOE_ERR_UNSUPPORTED: the fp16 expert inputs are addressed with 32-bit byte
 * offsets). */
moe_status moe_grouped_ffn_q(const void* x, moe_dtype xdt, const moe_packed_expert* experts,
                             uint32_t fmt_mask, const int32_t* offsets, const int32_t* perm_token,
                             int T, int H, int I, int E, int k, moe_actq aq, float* Y, void* ws,
                             size_t ws_bytes, void* stream);

/* The three phases of moe_grouped_ffn_q, for callers that time or overlap
 * them; call them in this order on one stream with one workspace (same
 * arguments and workspace size as moe_grouped_ffn_q).
 * moe_ffn_gather: copies the expert input rows x[perm_token[r]] into the
 *   workspace as fp16 (or, under MOE_ACT_I8_*, as their int8 codes plus
 *   per-row scales). One kernel.
 * moe_ffn_gate_up: fused gate/up projection + SwiGLU of every sorted row,
 *   leaving h in the workspace. One kernel.
 * moe_ffn_down: (under MOE_ACT_I8_XH, per-row int8 quantisation of h, then)
 *   the down projection into Y (fp32 [T*k, H], 16-byte aligned); at decode
 *   sizes the K range is split over blocks and a reduction kernel sums the
 *   parts into Y. */
moe_status moe_ffn_gather(const void* x, moe_dtype xdt, const int32_t* perm_token, int T, int H,
                          int I, int E, int k, moe_actq aq, void* ws, size_t ws_bytes,
                          void* stream);
moe_status moe_ffn_gate_up(const moe_packed_expert* experts, uint32_t fmt_mask,
                           const int32_t* offsets, int T, int H, int I, int E, int k,
                           moe_actq aq, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_down(const moe_packed_expert* experts, uint32_t fmt_mask,
                        const int32_t* offsets, int T, int H, int I, int E, int k, moe_actq aq,
                        float* Y, void* ws, size_t ws_bytes, void* stream);

/* Weighted combine (step 5's sum): out[t,:] = sum_j topk_w[t,j] * Y[inv[t*k+j], :],
 * accumulated in fp32 in slot order j = 0..k-1. out (device): [T,H] fp32 or
 * bf16 (round to nearest even). H % 4 == 0. */
moe_status moe_combine(const float* Y, const float* topk_w, const int32_t* inv, int T, int H,
                       int k, void* out, moe_dtype out_dt, void* stream);

/* The whole layer in one call: route, permute, grouped FFN, combine.
 * topk_ids / topk_w (device, optional): receive the routing when non-NULL.
 * ws: at least moe_workspace_size(T, H, I, E, k, aq) bytes. */
moe_status moe_layer_forward(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                             const moe_packed_expert* experts, uint32_t fmt_mask, int T, int H,
                             int I, int E, int k, moe_actq aq, void* out, moe_dtype out_dt,
                             int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): moe_layer_forward
 * with its workspace in a device array inside the library instead of a
 * caller buffer. Each GPU the library runs on holds one such array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) from the first call made with that GPU
 * current until the process ends; the call itself allocates nothing.
 * Sizes whose workspace exceeds it return MOE_ERR_WORKSPACE before
 * anything is enqueued (the workspace moe_layer_forward needs with this
 * fmt_mask: moe_workspace_size, less the transposed input copies when the
 * mask lacks MOE_MASK_OUTLIERS). Decode-size batches fit: the
 * Mixtral-shaped layer up to 314 tokens (191 with outlier lists), the
 * H=8192, I=16384 W4A8 one up to 113.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two host threads)
 * race and must be ordered by the caller. Nothing in the array needs to
 * start at zero; the call writes its flag word itself.
 * flags (device, optional, 4-byte aligned): receives the call's flag word
 * (MOE_FLAG_*) in place of the workspace's first word; NULL keeps it inside
 * the array, where the caller cannot read it.
 * Other arguments, outputs and results as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t moe_noalloc_scratch_bytes(void);
moe_status moe_layer_forward_noalloc(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                                     const moe_packed_expert* experts, uint32_t fmt_mask, int T,
                                     int H, int I, int E, int k, moe_actq aq, void* out,
                                     moe_dtype out_dt, int32_t* topk_ids, float* topk_w,
                                     uint32_t* flags, void* stream);

/* Per-token dynamic int8 quantisation of rows (mixed-precision notes,
 * sections 2.1-2.2), the arithmetic the layer applies to its expert inputs
 * under MOE_ACT_I8_*: per row s = fp32(absmax)/127, q = clamp(rint(v/s),
 * -127, 127) with IEEE fp32 division and round half to even; a zero row gives
 * s = 0 and q = 0. v (device): [rows, cols] fp32 or bf16. q (device): int8
 * [rows, cols]. s (device): fp32 [rows]. */
moe_status moe_act_quant_i8(const void* v, moe_dtype dt, int rows, int cols, int8_t* q, float* s,
                            void* stream);

/* int8 router logits (the "AlphaQ" blog, sections 2.2 and 4.1, DRAQ: leave
 * the router's weights alone and quantise its output logits to int8 with a
 * scale and zero point calibrated on real data). A variant of
 * moe_route that trades routing exactness for int8 logits: it is measured
 * against the exact routing, not used by moe_layer_forward.
 *
 * moe_router_logit_range: the fp64 logits of the T tokens (as moe_route
 *   computes them), merged into the per-expert running minimum lo[E] and
 *   maximum hi[E] (device, double; the caller starts them at +inf / -inf).
 *   NaN logits are skipped. Same arguments, constraints and workspace as
 *   moe_route.
 * moe_router_i8_params (host only): from lo[E] <= hi[E] (host, finite), per
 *   expert (shared == 0; the per-output-channel parameters of the blog's
 *   section 2.2) or for the range over all experts (shared != 0; one scale
 *   and zero point, so the int8 codes themselves rank as the top-k "in int8
 *   space" of section 4.1): scale s = fp32((hi - lo) / 255), at least the
 *   smallest normal fp32, and zero point z = -128 - rint(lo / s) (int32,
 *   saturated), so lo maps to code -128 and hi to 126 or 127.
 * moe_route_i8: as moe_route, except that the top-k and the softmax use
 *   each logit after an int8 round trip, (clamp(rint(L/s) + z, -128, 127) - z)
 *   * s in fp64 (round half to even); experts with s <= 0 get 0. Equal
 *   values go to the lower expert index. scale (device, fp32 [E]) and zero
 *   (device, int32 [E]) as moe_router_i8_params gives them. logits
 *   (optional) receives the logits before the round trip. */
moe_status moe_router_logit_range(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                                  int T, int H, int E, double* lo, double* hi, void* ws,
                                  size_t ws_bytes, void* stream);
moe_status moe_router_i8_params(const double* lo, const double* hi, int E, int shared,
                                float* scale, int32_t* zero);
moe_status moe_route_i8(const void* x, moe_dtype xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, const float* scale, const int32_t* zero, int32_t* topk_ids,
                        float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream);

/* Routing profile for expert-aware precision (expert-aware quantisation
 * digest, profiling and results sections: a profiling run over task data
 * marks the experts the router actually uses as hot and keeps them at higher
 * precision, the rest at 2 bits; its conclusion sketches a gradient of ever
 * coarser tiers for ever colder experts).
 * hist[e] += the number of slots of topk_ids [T,k] (device, int32) equal to e,
 * for e in [0,E); ids outside [0,E) (MOE_ID_NAN included) are not counted.
 * hist (device): int64 [E], accumulated across calls (the caller zeroes it
 * once). Integer adds: the result does not depend on their order.
 * T*k <= 2^30, E <= 256. */
moe_status moe_expert_histogram(const int32_t* topk_ids, int T, int k, int E, int64_t* hist,
                                void* stream);

/* Precision tiers from a routing profile (host only: no device work, no
 * stream). counts [E] (host, >= 0): routing counts, e.g. a
 * moe_expert_histogram profile. tier_bytes [ntiers] (host): the bytes one
 * expert takes at each tier (moe_packed_expert_bytes of its packing), most
 * precise first, non-increasing, each <= 2^40. Experts are ranked by count,
 * descending, ties to the lower index; walking that ranking, each expert
 * gets the most precise tier whose bytes leave room, within budget_bytes,
 * for every expert after it at the last tier. So the tiers never get more
 * precise as the counts fall, and the first expert below the top tier could
 * not be raised one tier without exceeding the budget. tier_of [E] (host,
 * out): the tier index of each expert; *used_bytes (host, out, nullable):
 * their total. MOE_ERR_INVALID_ARG if an argument is out of range or even
 * every expert at the last tier exceeds the budget (tier_of is then left
 * untouched). 1 <= E <= 65536, 1 <= ntiers <= 16. */
moe_status moe_plan_tiers(const int64_t* counts, int E, const uint64_t* tier_bytes, int ntiers,
                          uint64_t budget_bytes, int32_t* tier_of, uint64_t* used_bytes);

/* Measurement aid (not a step of the layer): a plain streaming read of
 * `bytes` bytes at `src` (device, 16-byte aligned, bytes % 16 == 0) by
 * MOE_STREAM_BLOCKS blocks with 16-byte loads, non-temporal when
 * `nontemporal` is non-zero. Each block folds the 32-bit words it read into
 * an XOR and stores it at sink[block] (device, MOE_STREAM_BLOCKS uint32), so
 * the XOR of all sink entries is the XOR of every word of the buffer. Timing
 * it gives the HBM read rate the device reaches, the context for the decode
 * GEMVs' weight-stream rates. */
#define MOE_STREAM_BLOCKS 4096
moe_status moe_stream_read(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                           void* stream);

/* Measurement aid (not a step of the layer): the streaming read above with
 * its launch shape as arguments, to find the read rate the device reaches
 * and the shape that reaches it.
 *   blocks   1..MOE_STREAM_MAX_BLOCKS blocks of 64*waves threads (waves
 *            1..16);
 *   inflight 1, 2, 4, 8 or 16 independent 16-byte loads per thread before
 *            their words are folded;
 *   layout   0: the grid sweeps the buffer as one front (thread t of block b
 *            reads chunk b*nthr + t, then steps by nthr*blocks chunks);
 *            1: block b reads its own contiguous run of ceil(chunks/blocks)
 *            16-byte chunks, nthr chunks at a time.
 * Other values give MOE_ERR_INVALID_ARG. sink (device, `blocks` uint32)
 * receives one XOR word per block, so the XOR of the sink entries is the XOR
 * of every 32-bit word of the buffer, as for moe_stream_read. */
#define MOE_STREAM_MAX_BLOCKS 65536
moe_status moe_stream_read_shaped(const void* src, size_t bytes, int nontemporal, int blocks,
                                  int waves, int inflight, int layout, uint32_t* sink,
                                  void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
