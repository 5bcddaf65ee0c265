// Repack canonical weight blocks into the device tile layout used by the
// grouped GEMMs (see Fmt<> in common.h).
//
// The pages describe "expert packing": each expert's weights are cut into
// column blocks quantised independently and laid out as one compact stream so
// that the weight reads are contiguous (MoE mixed-precision notes, sections
// 2.3 and 3.5). Here the stream is cut into 1 KiB tiles of 32 rows that a
// 64-lane wavefront reads with one 16-byte load per lane, already in the
// order the matrix-core B operand consumes them (512 B tiles of 8 bytes per
// lane for 1-bit codes).
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

__device__ inline uint32_t get_field(const uint32_t* w, int idx, int bits) {
  // canonical order: element idx of the 16-byte block, little-endian fields
  int per = 32 / bits;
  return (w[idx / per] >> ((idx % per) * bits)) & ((1u << bits) - 1u);
}

// one thread = one lane slot (16 or 8 bytes) of one tile
__global__ void pack_codes_kernel(PackArgs a) {
  const int span = fmt_span(a.bits), KT = 2 * span, cb = fmt_cb(a.bits);
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
  int k0 = kt * KT + kh * span;
  size_t rb = ((size_t)a.K * a.bits / 8 + 15) / 16 * 16;
  const uint32_t* s =
      reinterpret_cast<const uint32_t*>(a.src_codes[src] + (size_t)row * rb + (size_t)k0 * a.bits / 8);
  const int nw = cb / 4;  // 32-bit words per lane slot
  uint32_t w[4] = {s[0], s[1], 0u, 0u};
  if (nw > 2) {
    w[2] = s[2];
    w[3] = s[3];
  }
  uint32_t out[4];
  const int per = 32 / a.bits;        // codes per word (8, 16 or 32)
  const int half = per / 2;
  const bool pairs = a.fmt == MOE_W_ASYM;  // e2m1 keeps the natural order
  for (int d = 0; d < nw; ++d) {
    uint32_t v = 0;
    for (int p = 0; p < per; ++p) {
      // asymmetric: field p of word d holds code per*d + (p < half ? 2p : 2(p-half)+1),
      // so each 16-bit half carries one code of every consecutive pair
      int c = pairs ? per * d + (p < half ? 2 * p : 2 * (p - half) + 1) : per * d + p;
      v |= get_field(w, c, a.bits) << (p * a.bits);
    }
    out[d] = v;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + ((size_t)vrt * KTn + kt) * 64 * cb + lane * cb);
  for (int d = 0; d < nw; ++d) dst[d] = out[d];
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

}  // namespace moeq
