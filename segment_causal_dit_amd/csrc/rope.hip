// 3D rotary position embedding of video rows, bf16 in and out.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation",
// architecture table, position-encoding row (3D RoPE; 16, 56 and 56 of the
// 128 dimensions for t, h and w; theta 256) and section "Segment-Autoregressive
// Diffusion Transformer" (RoPE encodes video positions). Pair (2i, 2i+1) of a
// slice of width d is rotated by pos_axis * theta^(-2i/d); with even slice
// widths the pair index is simply element / 2 across the whole head.
//
// Rounding: the result is the rotation rounded once to bf16 (nearest, ties to
// even). The fast path rotates in fp32 from fp64 cos/sin; it keeps that result
// only when no bf16 rounding midpoint lies within its error bound
// (2^-21 * (|x0| + |x1|), from the fp32 rounding of cos/sin, of x1*sin and of
// the fused multiply-add). Otherwise the pair is recomputed in fp64 and
// rounded directly from fp64. The output therefore equals the bf16 rounding
// of the fp64 rotation, element for element.
//
// HBM-bound: 512 B per (token, head) moved (read + write of 128 bf16).
#include "internal.h"

namespace segc {
namespace {

constexpr int kTok = 4;          // tokens per workgroup
constexpr int kThreads = 256;    // kTok * 64 pairs for the sin/cos phase

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round an fp64 value to bf16 bits, nearest-even, straight from its bits.
__device__ inline uint32_t bf16_from_f64(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const uint64_t m = b & 0x7FFFFFFFFFFFFFFFull;
  const double a = __longlong_as_double((long long)m);
  if (a != a) return 0x7FC0u;                       // NaN
  if (!(a >= 0x1p-126)) {                           // bf16 subnormal range
    // spacing 2^-133; scaling by a power of two is exact, rint is nearest-even
    return sign | (uint32_t)rint(a * 0x1p133);      // 128 -> 0x0080 = 2^-126
  }
  // drop 45 of the 52 fraction bits with round-to-nearest-even; a carry
  // propagates into the exponent field as it should
  const uint64_t r = (m + ((1ull << 44) - 1) + ((m >> 45) & 1)) >> 45;
  const int64_t e = (int64_t)(r >> 7) - (1023 - 127);
  if (e >= 255) return sign | 0x7F80u;              // overflow -> inf
  return sign | (uint32_t)(r - ((uint64_t)(1023 - 127) << 7));
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};                // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// True when the fp32 value y (error <= 2^-21 * mag) might round to a different
// bf16 than the exact value: a rounding midpoint (low 16 bits 0x8000) lies
// within the error. ulp32(y) >= |y| * 2^-24 turns the bound into
// |lo - 0x8000| * |y| > 8 * mag; one extra ulp of slack is kept.
__device__ inline bool near_midpoint(float y, float mag) {
  const int lo = (int)(__float_as_uint(y) & 0xFFFFu) - 0x8000;
  return fabsf(y) * (fabsf((float)lo) - 1.0f) <= 8.0f * mag;
}

__global__ __launch_bounds__(kThreads) void rope3d_kernel(RopeParams p) {
  __shared__ double cs64[kTok][64][2];
  __shared__ float cs32[kTok][64][2];
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * kTok;

  {  // phase 1: one (token, pair) per thread
    const int tt = tid >> 6, pr = tid & 63;
    const int64_t tok = tok0 + tt;
    if (tok < p.n_tok) {
      const int pt = p.dims[0] >> 1, ph = pt + (p.dims[1] >> 1);
      const int axis = pr < pt ? 0 : (pr < ph ? 1 : 2);
      const double ang = (double)p.pos[tok * 3 + axis] * p.inv_freq[pr];
      double sn, cn;
      sincos(ang, &sn, &cn);
      cs64[tt][pr][0] = cn;
      cs64[tt][pr][1] = sn;
      cs32[tt][pr][0] = (float)cn;
      cs32[tt][pr][1] = (float)sn;
    }
  }
  __syncthreads();

  // phase 2: 16-byte chunks (4 pairs) of every head of the kTok tokens
  const int per_tok = p.n_heads * 16;
  for (int c = tid; c < kTok * per_tok; c += kThreads) {
    const int tt = c / per_tok;
    const int rem = c - tt * per_tok;
    const int head = rem >> 4, d8 = rem & 15;
    const int64_t tok = tok0 + tt;
    if (tok >= p.n_tok) break;
    const int64_t off = tok * p.stride_tok + (int64_t)head * p.stride_head + d8 * 8;
    const u32x4 in = *(const u32x4*)(p.x_in + off);
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pr = d8 * 4 + e;
      const float x0 = bf16_lo(in[e]), x1 = bf16_hi(in[e]);
      const float c32 = cs32[tt][pr][0], s32 = cs32[tt][pr][1];
      const float y0 = fmaf(x0, c32, -(x1 * s32));
      const float y1 = fmaf(x0, s32, x1 * c32);
      const float mag = fabsf(x0) + fabsf(x1);
      uint32_t w = pack_bf16(y0, y1);
      if (near_midpoint(y0, mag) || near_midpoint(y1, mag)) {
        const double c64 = cs64[tt][pr][0], s64 = cs64[tt][pr][1];
        const double z0 = fma((double)x0, c64, -((double)x1 * s64));
        const double z1 = fma((double)x0, s64, (double)x1 * c64);
        w = bf16_from_f64(z0) | (bf16_from_f64(z1) << 16);
      }
      out[e] = w;
    }
    *(u32x4*)(p.x_out + off) = u32x4{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace

hipError_t launch_rope(const RopeParams& p, hipStream_t s) {
  const int64_t blocks = (p.n_tok + kTok - 1) / kTok;
  hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace segc
