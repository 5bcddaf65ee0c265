// Repack canonical weight blocks into the device tile layout used by the
// grouped GEMMs (see Fmt<> in common.h), and outlier side lists into per-row
// lists the GEMM epilogues add.
//
// The pages describe "expert packing": each expert's weights are cut into
// column blocks quantised independently and laid out as one compact stream so
// that the weight reads are contiguous (MoE mixed-precision notes, sections
// 2.3 and 3.5). Here the stream is cut into 1 KiB tiles of 32 rows that a
// 64-lane wavefront reads with one 16-byte load per lane, already in the
// order the matrix-core B operand consumes them (512 B tiles of 8 bytes per
// lane for 1-bit codes; 1.5 KiB tiles of a 2-bit and a 1-bit plane for
// 3-bit codes). The notes also keep the largest weights (section 4.2) in
// fp16 beside the low-bit blocks: those become per-row lists of (column,
// correction) pairs.
#include "common.h"

namespace moeq {

namespace {

struct PackArgs {
  const uint8_t* src_codes[2];   // canonical code planes (gate, up) or (W, -)
  const uint8_t* src_params[2];
  int nsrc;                      // 2: interleave gate/up row tiles; 1: plain
  int N;                         // rows of one source matrix
  int K;                         // cols
  int fmt, bits, group;
  uint8_t* codes;
  uint8_t* params;
};

// bytes of one canonical code row (padded to 16)
__host__ __device__ inline size_t canon_row_bytes(int K, int bits) {
  return ((size_t)K * bits / 8 + 15) / 16 * 16;
}

// code c of a little-endian bit stream of b-bit codes held in words w
__device__ inline uint32_t stream_code(const uint32_t* w, int c, int bits) {
  const int pos = c * bits, wd = pos >> 5, off = pos & 31;
  uint32_t v = w[wd] >> off;
  if (off + bits > 32) v |= w[wd + 1] << (32 - off);
  return v & ((1u << bits) - 1u);
}

// Words of one plane of `pbits`-bit fields from the lane's codes q[0..span):
// for asymmetric blocks field p of word d holds code per*d + 2p (low half)
// or per*d + 2(p - half) + 1 (high half), so each 16-bit half carries one
// code of every consecutive pair; e2m1 keeps the natural order.
__device__ inline void plane_words(const uint8_t* q, int span, int pbits, bool pairs,
                                   uint32_t* out) {
  const int per = 32 / pbits, half = per / 2, nw = span * pbits / 32;
  for (int d = 0; d < nw; ++d) {
    uint32_t v = 0;
    for (int p = 0; p < per; ++p) {
      const int c = pairs ? per * d + (p < half ? 2 * p : 2 * (p - half) + 1) : per * d + p;
      v |= (uint32_t)q[c] << (p * pbits);
    }
    out[d] = v;
  }
}

// one thread = one lane slot of one tile
__global__ void pack_codes_kernel(PackArgs a) {
  const int span = fmt_span(a.bits), KT = 2 * span, tb = fmt_tile_bytes(a.bits);
  const int KTn = a.K / KT;
  const int NT = a.N / 32;  // row tiles per source
  const long total = (long)NT * a.nsrc * KTn * 64;
  long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  int lane = (int)(gid % 64);
  long t = gid / 64;
  int kt = (int)(t % KTn);
  int vrt = (int)(t / KTn);  // virtual row tile
  int src = a.nsrc == 2 ? (vrt & 1) : 0;
  int rt = a.nsrc == 2 ? (vrt >> 1) : vrt;
  int n = lane % 32, kh = lane / 32;
  int row = rt * 32 + n;
  int k0 = kt * KT + kh * span;  // a multiple of 32: the slice starts on a byte
  const uint32_t* s = reinterpret_cast<const uint32_t*>(
      a.src_codes[src] + (size_t)row * canon_row_bytes(a.K, a.bits) + (size_t)k0 * a.bits / 8);
  uint32_t w[6];
  const int nw_src = span * a.bits / 32;  // 4, 4, 2 or 6 words
  for (int i = 0; i < nw_src; ++i) w[i] = s[i];
  uint8_t q[64];
  for (int c = 0; c < span; ++c) q[c] = (uint8_t)stream_code(w, c, a.bits);
  const bool pairs = a.fmt == MOE_W_ASYM;
  uint8_t* tile = a.codes + ((size_t)vrt * KTn + kt) * tb;
  uint32_t out[4];
  if (a.bits == 3) {
    // low two bits as a 2-bit tile, then the high bit as a 1-bit tile
    uint8_t lo[64], hi[64];
    for (int c = 0; c < 64; ++c) {
      lo[c] = q[c] & 3;
      hi[c] = q[c] >> 2;
    }
    plane_words(lo, 64, 2, pairs, out);
    uint32_t* d = reinterpret_cast<uint32_t*>(tile + lane * 16);
    for (int i = 0; i < 4; ++i) d[i] = out[i];
    plane_words(hi, 64, 1, pairs, out);
    d = reinterpret_cast<uint32_t*>(tile + 1024 + lane * 8);
    for (int i = 0; i < 2; ++i) d[i] = out[i];
  } else {
    plane_words(q, span, a.bits, pairs, out);
    const int nw = span * a.bits / 32;
    uint32_t* d = reinterpret_cast<uint32_t*>(tile + lane * nw * 4);
    for (int i = 0; i < nw; ++i) d[i] = out[i];
  }
}

// one thread = one (row, entry)
__global__ void pack_params_kernel(PackArgs a) {
  const int span = fmt_span(a.bits);
  const int ge = a.group > span ? a.group : span;
  const int np = a.group < span ? span / a.group : 1;
  const int psz = a.fmt == MOE_W_ASYM ? 4 : 2;
  const int eb = np * psz;
  const int NE = a.K / ge;
  const int NT = a.N / 32;
  const long total = (long)NT * a.nsrc * NE * 32;
  long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  int n = (int)(gid % 32);
  long t = gid / 32;
  int ei = (int)(t % NE);
  int vrt = (int)(t / NE);
  int src = a.nsrc == 2 ? (vrt & 1) : 0;
  int rt = a.nsrc == 2 ? (vrt >> 1) : vrt;
  int row = rt * 32 + n;
  const int G = a.K / a.group;
  const uint8_t* srow = a.src_params[src] + (size_t)row * G * psz;
  uint8_t* dst = a.params + (((size_t)vrt * NE + ei) * 32 + n) * eb;
  int g0 = ei * ge / a.group;
  for (int p = 0; p < np; ++p) {
    const uint8_t* sp = srow + (size_t)(g0 + p) * psz;
    for (int b = 0; b < psz; ++b) dst[p * psz + b] = sp[b];
  }
}

// ---------------------------------------------------------------------------
// Outlier side lists
// ---------------------------------------------------------------------------
struct OutSrc {
  const uint32_t* rec;  // n records {index, fp16 value} (two uint32 each)
  uint32_t n;
  int rows, cols, fmt, bits, group;
  const uint8_t* codes;
  const uint16_t* params;
};
struct OutArgs {
  OutSrc s[2];
  int nsrc;
  uint32_t* rowptr;
  OutEntry* entries;
};

// first record of s whose index is >= key (records ascending)
__device__ inline uint32_t lower_bound_idx(const OutSrc& s, uint64_t key) {
  uint32_t lo = 0, hi = s.n;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) / 2;
    if ((uint64_t)s.rec[2 * mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// rowptr[r] for r in [0, rows of all sources]: where row r's entries start
__global__ void pack_outlier_rows_kernel(OutArgs a) {
  const int rows0 = a.s[0].rows, rows = rows0 + (a.nsrc == 2 ? a.s[1].rows : 0);
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r > rows) return;
  uint32_t v;
  if (r == rows) {
    v = a.s[0].n + (a.nsrc == 2 ? a.s[1].n : 0);
  } else if (r < rows0) {
    v = lower_bound_idx(a.s[0], (uint64_t)r * a.s[0].cols);
  } else {
    v = a.s[0].n + lower_bound_idx(a.s[1], (uint64_t)(r - rows0) * a.s[1].cols);
  }
  a.rowptr[r] = v;
}

// The fp16 value the GEMMs decode at (row, k) of a canonical matrix: the
// same fp16 operations as the in-register decode (one packed fp16 fma of the
// exact code for asymmetric blocks, the exact e2m1 value times the scale).
__device__ inline float decoded_f16(const OutSrc& s, int row, int k) {
  // the row's codes as 32-bit words (a row holds cols * bits / 8 bytes, a
  // multiple of 4; a code straddling two words reads both, both in the row)
  const uint32_t* w = reinterpret_cast<const uint32_t*>(
      s.codes + (size_t)row * canon_row_bytes(s.cols, s.bits));
  const uint32_t q = stream_code(w, k, s.bits);
  const int g = k / s.group;
  if (s.fmt == MOE_W_ASYM) {
    const uint16_t* p = s.params + (size_t)row * 2 * (s.cols / s.group) + 2 * g;
    const f16x2 s2 = __builtin_bit_cast(f16x2, (uint32_t)p[0] * 0x10001u);
    const f16x2 m2 = __builtin_bit_cast(f16x2, (uint32_t)p[1] * 0x10001u);
    const f16x2 q2 = f16x2{(f16)(float)q, (f16)(float)q};
    return (float)__builtin_elementwise_fma(q2, s2, m2)[0];
  }
  const uint16_t sc = s.params[(size_t)row * (s.cols / s.group) + g];
  const f16x2 s2 = __builtin_bit_cast(f16x2, (uint32_t)sc * 0x10001u);
  const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * s2;
  return (float)v[0];
}

// one thread = one outlier: (column, fp16 value - decoded fp16 value); an
// index outside the matrix gives a harmless (0, 0) entry
__global__ void pack_outlier_entries_kernel(OutArgs a) {
  const uint32_t n0 = a.s[0].n, n = n0 + (a.nsrc == 2 ? a.s[1].n : 0);
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const OutSrc& s = i < n0 ? a.s[0] : a.s[1];
  const uint32_t j = i < n0 ? i : i - n0;
  const uint64_t idx = s.rec[2 * j];
  OutEntry e = {0u, 0.0f};
  if (idx < (uint64_t)s.rows * s.cols) {
    const int row = (int)(idx / s.cols), k = (int)(idx % s.cols);
    const f16 v = __builtin_bit_cast(f16, (uint16_t)(s.rec[2 * j + 1] & 0xffffu));
    e.k = (uint32_t)k;
    e.delta = (float)v - decoded_f16(s, row, k);
  }
  a.entries[i] = e;
}

OutSrc out_src(const moe_qmat* q) {
  OutSrc s;
  s.rec = (const uint32_t*)q->outliers;
  s.n = q->n_outliers;
  s.rows = (int)q->rows;
  s.cols = (int)q->cols;
  s.fmt = q->fmt;
  s.bits = q->bits;
  s.group = q->group;
  s.codes = (const uint8_t*)q->codes;
  s.params = (const uint16_t*)q->params;
  return s;
}

}  // namespace

hipError_t launch_pack_matrix(const moe_qmat* a, const moe_qmat* b, void* codes, void* params,
                              hipStream_t s) {
  PackArgs pa;
  pa.src_codes[0] = (const uint8_t*)a->codes;
  pa.src_params[0] = (const uint8_t*)a->params;
  pa.src_codes[1] = b ? (const uint8_t*)b->codes : nullptr;
  pa.src_params[1] = b ? (const uint8_t*)b->params : nullptr;
  pa.nsrc = b ? 2 : 1;
  pa.N = (int)a->rows;
  pa.K = (int)a->cols;
  pa.fmt = a->fmt;
  pa.bits = a->bits;
  pa.group = a->group;
  pa.codes = (uint8_t*)codes;
  pa.params = (uint8_t*)params;
  const int span = fmt_span(pa.bits), KT = 2 * span;
  long nc = (long)(pa.N / 32) * pa.nsrc * (pa.K / KT) * 64;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ge = pa.group > span ? pa.group : span;
  long np = (long)(pa.N / 32) * pa.nsrc * (pa.K / ge) * 32;
  hipLaunchKernelGGL(pack_params_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s, pa);
  return hipGetLastError();
}

hipError_t launch_pack_outliers(const moe_qmat* a, const moe_qmat* b, uint32_t* rowptr,
                                OutEntry* entries, hipStream_t s) {
  OutArgs oa;
  oa.s[0] = out_src(a);
  oa.nsrc = b ? 2 : 1;
  if (b) oa.s[1] = out_src(b);
  oa.rowptr = rowptr;
  oa.entries = entries;
  const long rows = (long)a->rows + (b ? (long)b->rows : 0);
  hipLaunchKernelGGL(pack_outlier_rows_kernel, dim3((unsigned)((rows + 1 + 255) / 256)), dim3(256),
                     0, s, oa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n = (long)a->n_outliers + (b ? (long)b->n_outliers : 0);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_outlier_entries_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     s, oa);
  return hipGetLastError();
}

}  // namespace moeq
