// Append the current segment's video K (after RoPE) and V to cache slots,
// quantising to INT8 for an INT8 cache.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
// "Segment-Autoregressive Diffusion Transformer" (cached keys and values
// serve again as generation moves on) and section "Single-GPU Low-Memory
// Inference" (keys and values cached in INT8, attention kept in BF16).
// Quantiser (this library's scheme, per token and head, K and V separately):
//   scale = fp32(max|x| / 127)                       IEEE fp32 division
//   code  = clamp(rint(fp32(x / scale)), -127, 127)  ties to even
// with scale 0 and all-zero codes for an all-zero row.
//
// x / scale + 128 (the biased code before rounding) is first estimated as
// fma(x, rcp(scale), 128) with the hardware reciprocal (within 1 ulp for a
// normal scale): the estimate is within 3.4e-5 of the exact value and the
// IEEE quotient within 2^-18 of x / scale (|x / scale| <= 127), so unless the
// estimate lies within 2^-14 of a half-integer both round to the same
// integer; otherwise the IEEE division decides (an all-zero row, rcp 0, gives
// codes 0). A row whose scale is subnormal (absmax below 127 * 2^-126; bf16
// inputs reach down to 2^-133) has no usable reciprocal (it loses accuracy,
// and overflows to infinity below 2^-128), so every element of such a row
// takes the IEEE division. The division runs in a wave-uniform branch, taken
// by about one wave in eight on unit-scale data.
//
// Layout: a workgroup of 256 lanes handles 16 consecutive tokens of one head;
// 16 lanes per (token, head), 8 elements each. HBM-bound: 776 B per
// (token, head) moved for INT8 (512 read, 256 codes + 8 scale bytes written),
// 1024 B for a BF16 cache.
#include "internal.h"

namespace segc {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 16;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// max over the 16 lanes of a DPP row (quad swaps, then half-row and row mirrors)
__device__ inline float row16_max(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x140, 0xF, 0xF, true)));
  return a;
}

// Quantise 8 bf16 values held by this lane (one of 16 lanes of a row);
// returns the 8 codes packed little-endian and the row's scale.
__device__ inline u32x2 quant_row8(const u32x4 in, float* scale_out) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(in[i]);
    x[2 * i + 1] = bf16_hi(in[i]);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
  a = row16_max(a);
  const float scale = a / 127.0f;                    // IEEE fp32 division
  *scale_out = scale;
  // a subnormal scale: the whole row is divided (same value in all 16 lanes)
  const bool tiny = scale != 0.0f && scale < 0x1p-126f;
  // all-zero row: rcp 0, codes 0
  const float rcp = (scale != 0.0f && !tiny) ? __builtin_amdgcn_rcpf(scale) : 0.0f;
  // |x / scale| <= 127 (1 + 2^-24) < 127.5 for a normal scale = fp32(max|x| /
  // 127), so the biased code rint(x / scale) + 128 lies in [1, 255]. Its
  // estimate v = fma(x, rcp, 128) (one rounding) is within 3.4e-5 of the exact
  // x / scale + 128; away from ties (2^-14) the byte conversion's own
  // round-to-nearest-even of v gives the biased code.
  float v[8];
  bool near = tiny;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = fmaf(x[i], rcp, 128.0f);
    near |= fabsf(v[i] - rintf(v[i])) >= 0.5f - 0x1p-14f;
  }
  if (__builtin_amdgcn_ballot_w64(near)) {
    // (a subnormal scale carries a relative error up to 2^-10, so the clamp
    // to +-127 is kept explicitly here; the biased byte never reaches 0)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (tiny || fabsf(v[i] - rintf(v[i])) >= 0.5f - 0x1p-14f)
        v[i] = fminf(fmaxf(rintf(x[i] / scale), -127.0f), 127.0f) + 128.0f;
  }
  // biased byte written in place, then XOR 0x80 per byte gives the
  // two's-complement code
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wd = __builtin_amdgcn_cvt_pk_u8_f32(v[4 * h + j], j, wd);
    out[h] = wd ^ 0x80808080u;
  }
  return u32x2{out[0], out[1]};
}

__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p) {
  const int tid = threadIdx.x;
  const int head = blockIdx.y;
  const int r = blockIdx.x * kTokPerBlock + (tid >> 4);   // input token
  const int li = tid & 15;                                  // 8-element chunk
  if (r >= p.n_tok) return;        // whole 16-lane groups exit together
  const int f = r / p.G;
  const int g = r - f * p.G;
  const int slot = (p.first_slot + f) % p.n_slots;
  const int64_t row = ((int64_t)slot * p.n_heads + head) * p.G + g;   // cache row
  const u32x4 kin = *(const u32x4*)(p.k + r * p.k_st + head * p.k_sh + li * 8);
  const u32x4 vin = *(const u32x4*)(p.v + r * p.v_st + head * p.v_sh + li * 8);
  if (p.int8) {
    float ks, vs;
    const u32x2 kc = quant_row8(kin, &ks);
    const u32x2 vc = quant_row8(vin, &vs);
    *(u32x2*)((int8_t*)p.ck + row * 128 + li * 8) = kc;
    *(u32x2*)((int8_t*)p.cv + row * 128 + li * 8) = vc;
    if (li == 0) {
      p.cks[row] = ks;
      p.cvs[row] = vs;
    }
  } else {
    *(u32x4*)((uint16_t*)p.ck + row * 128 + li * 8) = kin;
    *(u32x4*)((uint16_t*)p.cv + row * 128 + li * 8) = vin;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  const unsigned bx = (unsigned)((p.n_tok + kTokPerBlock - 1) / kTokPerBlock);
  hipLaunchKernelGGL(append_kernel, dim3(bx, (unsigned)p.n_heads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace segc
