// Linear layer with INT8 weights and BF16 activations on bf16 MFMA:
//   y[m][n] = bf16( scale[n] * sum_k x[m][k] * code[n][k] + bias[n] )
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation" (model
// card), assets table and section "Single-GPU Low-Memory Inference": the
// quantized DiT stores its weights in INT8 while linear computation stays
// BF16. One fp32 scale per output channel (this library's reading), so the
// scale factors out of the sum: codes (|c| <= 127, exact in bf16) are the
// MFMA operand and the scale is applied once to the fp32 accumulator.
//
// Two kernels per call:
//  * expand: the codes become bf16 in a caller-owned [n][k] workspace, once
//    per call (converting them inside the product instead repeats the work
//    in every row-tile workgroup: 248 times for 63,360 rows);
//  * product: 8 waves (two per SIMD) compute 256-channel x 256-row tiles of
//    y^T = W x^T; wave w owns channels 128 (w & 1) .. + 127 and rows
//    64 (w >> 1) .. + 63 as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16,
//    so each lane stores four consecutive channels of one row at a time.
//    Both operand tiles (64 deep) arrive by direct global -> LDS loads, one
//    stage ahead in two LDS stages (deeper pipelines at 32 deep measured no
//    faster). Tile rows are 128 bytes; chunk c of row r sits at
//    c ^ ((r >> 1) & 7), so an MFMA operand read (16 consecutive rows, one
//    chunk) touches 16 distinct bank groups. The kernel is persistent: one
//    workgroup per CU walks its tiles and starts the next tile's loads right
//    behind the previous tile's stores.
#include "internal.h"
#include "lds_dma.h"

namespace segc {
namespace {

constexpr int TN = 256;                 // output channels per workgroup
constexpr int TM = 256;                 // activation rows per workgroup
constexpr int TK = 64;                  // k per stage
constexpr int NSTG = 2;                 // LDS stages (loads run NSTG - 1 ahead)
constexpr int NTH = 512;
constexpr int CH = TK / 8;              // 16-byte chunks per tile row
constexpr int ROWB = TK * 2;            // bytes per tile row
constexpr int XT_BYTES = TM * ROWB;
constexpr int WT_BYTES = TN * ROWB;
constexpr int STAGE = XT_BYTES + WT_BYTES;
constexpr int G_LDS = NSTG * STAGE;
constexpr int RPL = 64 / CH;            // tile rows per direct load
constexpr int LOADS = 2 * (32 / RPL);   // direct loads per wave per stage
constexpr int GROUP_M = 4;              // row tiles per L2 group

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline int g_swz(int r) { return (r / (16 / CH)) & (CH - 1); }
__device__ inline int g_off(int r, int c) { return r * ROWB + ((c ^ g_swz(r)) << 4); }

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Four signed codes (one dword) -> four bf16, exact.
__device__ inline u32x2 codes_to_bf16(uint32_t d) {
  return u32x2{pack_bf16((float)(int8_t)(d & 0xFF), (float)(int8_t)((d >> 8) & 0xFF)),
               pack_bf16((float)(int8_t)((d >> 16) & 0xFF), (float)(int8_t)(d >> 24))};
}

// 16 codes per thread -> 16 bf16 in the dense [n][k] workspace.
__global__ __launch_bounds__(256) void w8_expand_kernel(W8GemmParams p) {
  const int64_t per_row = p.K / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_row * p.N) return;
  const int64_t n = i / per_row, kc = i - n * per_row;
  const u32x4 c = *(const u32x4*)(p.w + n * p.ldw + 16 * kc);
  u32x4 lo, hi;
  const u32x2 a = codes_to_bf16(c[0]), b = codes_to_bf16(c[1]), d = codes_to_bf16(c[2]), e = codes_to_bf16(c[3]);
  lo = u32x4{a.x, a.y, b.x, b.y};
  hi = u32x4{d.x, d.y, e.x, e.y};
  u32x4* dst = (u32x4*)(p.wbf + n * p.K + 16 * kc);
  dst[0] = lo;
  dst[1] = hi;
}

// Tile of logical index `logical`: groups of GROUP_M row tiles x all channel
// tiles, channel-tile-major inside a group.
__device__ inline void tile_of(const W8GemmParams& p, int logical, int& m0, int& n0) {
  const int per_group = GROUP_M * p.n_tiles;
  const int grp = logical / per_group;
  const int in_grp = logical - grp * per_group;
  const int gm = min(GROUP_M, p.m_tiles - grp * GROUP_M);
  const int ntile = in_grp / gm;
  m0 = (grp * GROUP_M + (in_grp - ntile * gm)) * TM;
  n0 = ntile * TN;
}

// Persistent: the grid holds one workgroup per CU (or one per tile when
// there are fewer tiles). Round i gives workgroup b the logical tile
// i * G + (b % 8) * (G / 8) + b / 8, so the G / 8 workgroups of one XCD
// (dispatched round-robin, b % 8) work on consecutive tiles and share their
// operand tiles in L2. The next tile's first loads are issued right after a
// tile's results are stored.
__global__ __launch_bounds__(NTH, 2) void w8a16_kernel(W8GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  const int wn = w & 1, wm = w >> 1;
  const int G = gridDim.x, b = blockIdx.x;
  const int total = p.m_tiles * p.n_tiles;
  const int slot = (G % 8 == 0) ? (b & 7) * (G / 8) + (b >> 3) : b;
  const int nk = p.K / TK;

  const char* xsrc[32 / RPL];
  const char* wsrc[32 / RPL];
  int m0, n0;
  bool full;                            // every activation row of the tile exists
  // staging: wave w loads tile rows 32 w .. + 31 of both operands, RPL rows
  // per direct load (lane l: row l / CH, physical chunk l % CH). Full tiles
  // use uniform row-group bases and per-lane 32-bit offsets, which depend on
  // the lane and e only; the last, ragged row tile clamps rows per lane.
  uint32_t xoff[32 / RPL], woff[32 / RPL];
#pragma unroll
  for (int e = 0; e < 32 / RPL; ++e) {
    const int row = 32 * w + RPL * e + lane / CH;
    const uint32_t sw = ((lane % CH) ^ g_swz(row)) << 4;
    xoff[e] = (uint32_t)(lane / CH) * (uint32_t)p.ldx * 2 + sw;
    woff[e] = (uint32_t)(lane / CH) * (uint32_t)p.K * 2 + sw;
  }
  auto set_tile = [&](int logical) {
    tile_of(p, logical, m0, n0);
    full = m0 + TM <= p.M;
    if (!full) {
#pragma unroll
      for (int e = 0; e < 32 / RPL; ++e) {
        const int row = 32 * w + RPL * e + lane / CH;
        const int sw = ((lane % CH) ^ g_swz(row)) << 4;
        xsrc[e] = (const char*)(p.x + (int64_t)min(m0 + row, p.M - 1) * p.ldx) + sw;
        wsrc[e] = (const char*)(p.wbf + (int64_t)(n0 + row) * p.K) + sw;
      }
    }
  };
  auto issue = [&](int kt, char* stage) {
    if (full) {
#pragma unroll
      for (int e = 0; e < 32 / RPL; ++e) {
        const int r0 = 32 * w + RPL * e;                 // first tile row of the load
        const uint64_t xb = uniform_addr(p.x + (int64_t)(m0 + r0) * p.ldx + kt * TK);
        const uint64_t wb = uniform_addr(p.wbf + (int64_t)(n0 + r0) * p.K + kt * TK);
        dload16_s(xoff[e], xb, stage + r0 * ROWB);
        dload16_s(woff[e], wb, stage + XT_BYTES + r0 * ROWB);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32 / RPL; ++e) {
        dload16(xsrc[e] + kt * ROWB, stage + (32 * w + RPL * e) * ROWB);
        dload16(wsrc[e] + kt * ROWB, stage + XT_BYTES + (32 * w + RPL * e) * ROWB);
      }
    }
  };
  auto wait_newer = [&](int newer) {
    // leave the `newer` most recently issued stages in flight
    if (NSTG > 3 && newer >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * LOADS) : "memory");
    else if (NSTG > 2 && newer >= 1)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto prologue = [&]() {
#pragma unroll
    for (int i = 0; i < NSTG - 1; ++i)
      if (i < nk) issue(i, smem + i * STAGE);
  };

  int logical = slot;
  if (logical >= total) return;
  set_tile(logical);
  prologue();
  f32x16 acc[4][2];
  while (true) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};
    wait_newer(min(nk - 1, NSTG - 2));
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = smem + (kt % NSTG) * STAGE;
      if (kt + NSTG - 1 < nk) issue(kt + NSTG - 1, smem + ((kt + NSTG - 1) % NSTG) * STAGE);
      const char* xt = cur;
      const char* wt = cur + XT_BYTES;
#pragma unroll
      for (int ks = 0; ks < TK / 16; ++ks) {
        bf16x8 a[4], bb[2];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) a[nb] = *(const bf16x8*)(wt + g_off(128 * wn + 32 * nb + lr, 2 * ks + hh));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) bb[mb] = *(const bf16x8*)(xt + g_off(64 * wm + 32 * mb + lr, 2 * ks + hh));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[nb], bb[mb], acc[nb][mb], 0, 0, 0);
      }
      // tile kt + 1 must have landed; the tiles issued after it stay in flight
      wait_newer(min(nk - 1, kt + NSTG - 1) - (kt + 1));
      __syncthreads();
    }

    // epilogue: lane holds channels n .. n + 3 (n = 8 jq + 4 hh in each
    // 32-channel block) of row m
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nbase = n0 + 128 * wn + 32 * nb + 4 * hh;
      f32x4 sc[4], bi[4];
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        sc[jq] = *(const f32x4*)(p.scale + nbase + 8 * jq);
        bi[jq] = p.bias ? *(const f32x4*)(p.bias + nbase + 8 * jq) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 64 * wm + 32 * mb + lr;
        if (m >= p.M) continue;
        uint16_t* dst = p.y + (int64_t)m * p.ldy + nbase;
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x16& v = acc[nb][mb];
          const u32x2 o = {pack_bf16(fmaf(v[4 * jq], sc[jq][0], bi[jq][0]), fmaf(v[4 * jq + 1], sc[jq][1], bi[jq][1])),
                           pack_bf16(fmaf(v[4 * jq + 2], sc[jq][2], bi[jq][2]), fmaf(v[4 * jq + 3], sc[jq][3], bi[jq][3]))};
          *(u32x2*)(dst + 8 * jq) = o;
        }
      }
    }
    logical += G;
    if (logical >= total) break;
    // the LDS stages are free (every wave passed the last barrier)
    set_tile(logical);
    prologue();
  }
}

}  // namespace

hipError_t launch_w8a16(const W8GemmParams& p0, hipStream_t s) {
  W8GemmParams p = p0;
  p.n_tiles = p.N / TN;
  p.m_tiles = (p.M + TM - 1) / TM;
  const int64_t expand_threads = (int64_t)p.N * (p.K / 16);
  hipLaunchKernelGGL(w8_expand_kernel, dim3((unsigned)((expand_threads + 255) / 256)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  }
  const int64_t nwg = tiles < cus ? tiles : cus;   // one workgroup per CU (LDS allows no second)
  e = hipFuncSetAttribute((const void*)w8a16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, G_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(w8a16_kernel, dim3((unsigned)nwg), dim3(NTH), G_LDS, s, p);
  return hipGetLastError();
}

}  // namespace segc
