// Per-latent-frame camera cross-attention: each video row attends to the
// camera tokens of its own chunk of latent frames.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation" (model
// card), section "Text and Camera Conditioning": camera extrinsics become one
// 64-dimensional input per latent frame; in each double-stream block, following
// its video MLP, the video tokens cross-attend to the projected camera
// features chunk by chunk, and a one-frame chunk ties each latent frame's
// tokens to its own camera.
//
// Row r (of n_tok video rows) is in chunk c = r / tokens_per_chunk, whose
// camera tokens are rows [c t_cam, (c + 1) t_cam) of k and v. Per head:
//   o_r = sum_j softmax_j(sm_scale q_r . k_j) v_j.
// 16 lanes take one (row, head): 16 bytes of q and o each, so a wave reads
// and writes 1 KB contiguous when heads are contiguous. The chunk's camera
// rows are shared by every row of the chunk and stay in the caches; keys are
// taken four at a time so that their loads overlap. With
// one camera token per chunk (the pages' configuration) the softmax weight
// is exactly 1 (exp2(s - s) = 1, l = 1), so o_r = v of the chunk: that case
// skips q and the products and only writes (the same bits as the general
// path for finite inputs).
#include "internal.h"

namespace segc {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Sum over the 16 lanes of a row with DPP (quad swaps, then the half-row and
// row mirrors): every lane ends with the row's total, without LDS traffic.
__device__ inline float row16_sum(float a) {
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, true));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x140, 0xF, 0xF, true));
  return a;
}

constexpr int kThreads = 256;
constexpr int kPairs = kThreads / 16;     // (row, head) pairs per workgroup

__global__ __launch_bounds__(kThreads) void camera_attn_kernel(CamParams p) {
  const int tid = threadIdx.x;
  const int li = tid & 15;
  const int64_t pair = (int64_t)blockIdx.x * kPairs + (tid >> 4);
  const int64_t row = pair / p.n_heads;
  const int head = (int)(pair - row * p.n_heads);
  if (row >= p.n_tok) return;                 // whole 16-lane groups leave together
  const int64_t chunk = row / p.tpc;
  u32x4* dst = (u32x4*)(p.o + row * p.o_st + (int64_t)head * p.o_sh + 8 * li);
  const int64_t cam0 = chunk * p.t_cam;
  if (p.t_cam == 1) {
    *dst = *(const u32x4*)(p.v + cam0 * p.kv_st + (int64_t)head * p.kv_sh + 8 * li);
    return;
  }
  const u32x4 qv = *(const u32x4*)(p.q + row * p.q_st + (int64_t)head * p.q_sh + 8 * li);
  float qf[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qf[2 * e] = lo_f(qv[e]);
    qf[2 * e + 1] = hi_f(qv[e]);
  }
  // keys in blocks of four: the block's k and v loads go out together (one
  // memory latency per block instead of two per key); indices past t_cam are
  // clamped for the loads and their weights forced to zero
  float m = -INFINITY, l = 0.0f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < p.t_cam; j0 += 4) {
    u32x4 kv[4], vv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t off = (cam0 + min(j0 + u, p.t_cam - 1)) * p.kv_st + (int64_t)head * p.kv_sh + 8 * li;
      kv[u] = *(const u32x4*)(p.k + off);
      vv[u] = *(const u32x4*)(p.v + off);
    }
    float sv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(qf[2 * e], lo_f(kv[u][e]), d);
        d = fmaf(qf[2 * e + 1], hi_f(kv[u][e]), d);
      }
      sv[u] = d;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[u] = row16_sum(sv[u]);
    float mx = m;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[u] = (j0 + u < p.t_cam) ? sv[u] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[u]);
    }
    const float alpha = __builtin_amdgcn_exp2f(m - mx);        // 0 on the first block (m = -inf)
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float pr = __builtin_amdgcn_exp2f(sv[u] - mx);       // 0 for the padded keys
      l += pr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pr, lo_f(vv[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pr, hi_f(vv[u][e]), acc[2 * e + 1]);
      }
    }
    m = mx;
  }
  const float inv = 1.0f / l;
  uint32_t wd[4];                        // plain array first, vector in one piece
#pragma unroll
  for (int e = 0; e < 4; ++e) wd[e] = pack_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *dst = u32x4{wd[0], wd[1], wd[2], wd[3]};
}

}  // namespace

hipError_t launch_camera_attn(const CamParams& p, hipStream_t s) {
  const int64_t pairs = p.n_tok * p.n_heads;
  hipLaunchKernelGGL(camera_attn_kernel, dim3((unsigned)((pairs + kPairs - 1) / kPairs)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace segc
