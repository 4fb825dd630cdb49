// Expand the selected frames of an INT8 cache into a BF16 cache, in window
// order, so that attention over that window can run on bf16 tiles without
// dequantising inside every query tile's workgroup.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
// "Single-GPU Low-Memory Inference" (keys and values are stored in INT8 while
// attention runs in BF16). The dequantised value is bf16(fp32(code * scale)):
// the product rounded once to fp32, then to bf16 (round to nearest even) --
// the same value the attention kernel forms when it dequantises a tile itself.
//
// Layout: 8 lanes per cache row (token, head), 16 codes each; a workgroup of
// 256 lanes covers 32 consecutive rows of one output frame range. HBM-bound:
// per row 128 code bytes + 4 scale bytes read, 256 bf16 bytes written, for K
// and for V.
#include "internal.h"

namespace segc {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 8;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// code byte b (0..3) of w as a signed value times the row's scale, rounded once to fp32
__device__ inline float dq(uint32_t w, int b, float s) {
  return (float)(int)(int8_t)(w >> (8 * b)) * s;
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantParams p) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 3);   // output row
  if (row >= p.n_rows) return;
  const int part = threadIdx.x & 7;                                  // codes 16 part .. + 15
  const bool isv = blockIdx.y != 0;
  const int f = row / p.rows_per_frame;
  const int64_t src = (int64_t)p.slots[f] * p.rows_per_frame + (row - f * p.rows_per_frame);
  const int8_t* codes = isv ? p.cv : p.ck;
  const float s = (isv ? p.cvs : p.cks)[src];
  const u32x4 w = *(const u32x4*)(codes + src * 128 + 16 * part);
  // packed pairs in a plain array, moved into the stored vectors in one piece
  uint32_t pr[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pr[2 * e] = pack_bf16(dq(w[e], 0, s), dq(w[e], 1, s));
    pr[2 * e + 1] = pack_bf16(dq(w[e], 2, s), dq(w[e], 3, s));
  }
  uint16_t* out = (isv ? p.ov : p.ok) + (int64_t)row * 128 + 16 * part;
  *(u32x4*)out = u32x4{pr[0], pr[1], pr[2], pr[3]};
  *(u32x4*)(out + 8) = u32x4{pr[4], pr[5], pr[6], pr[7]};
}

}  // namespace

hipError_t launch_dequant(const DequantParams& p, hipStream_t s) {
  const unsigned bx = (unsigned)((p.n_rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(dequant_kernel, dim3(bx, 2), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace segc
