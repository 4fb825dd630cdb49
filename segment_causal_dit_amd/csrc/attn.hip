// Segment-wise causal joint attention over a KV cache plus the current
// segment(s), on gfx950 bf16 MFMA.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
// "Segment-Autoregressive Diffusion Transformer" (text and video interact
// through segment-wise causal joint attention; the layer's KV cache supplies
// earlier segments; attention is causal across segments) and section
// "Single-GPU Low-Memory Inference" (INT8 KV storage, BF16 attention);
// architecture table (16 heads x 128).
//
// What is computed: for each query row i and head, softmax over the visible
// keys of sm_scale * q_i . k_j, applied to v_j; keys are the history rows
// (frames listed in hist_slots) followed by the current rows. Visibility:
// history rows are visible to every query; a current key is visible to a
// query of segment s if it lies in segment s and is not a padded text row, or
// if it is a video row of an earlier segment.
//
// Design (one workgroup = 8 waves = 256 query rows of one head, one
// workgroup per CU, two waves per SIMD):
//  * each wave owns 32 query rows; Q stays in registers as MFMA B operands;
//  * waves 0-3 stage the K/V tiles, so each SIMD hosts one staging wave and
//    one compute-only wave and the staging cost is shared by 256 queries;
//  * key tiles of 64 rows are staged through LDS, double buffered: K row-major
//    [key][d] (272-byte rows), V transposed [d][key'] (128-byte rows, 16-byte
//    chunks XOR-swizzled by row) so that both MFMA operands are single
//    16-byte LDS reads without bank conflicts;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys land in accumulator
//    registers and queries across lanes, so a row max needs only one
//    cross-half exchange (v_permlane32_swap); O^T = V^T P^T takes the S^T
//    accumulators as the P operand directly (V^T is stored in the matching
//    key order);
//  * software pipeline: the QK^T MFMAs of tile t+1 are issued before the
//    softmax of tile t, so MFMA and VALU work of one wave overlap; K is
//    prefetched two tiles ahead and V one tile ahead, with one barrier per tile;
//  * each wave stages a 16-row group of a tile: with frames of a multiple of
//    16 tokens a group never straddles a frame, so its base address is
//    wave-uniform and lanes only add 32-bit offsets; rows past the end are
//    clamped to the last valid row (finite data) and masked;
//  * online softmax in base 2 with the rescale of O deferred until the running
//    max grows by more than 2^8 (exact: the final division uses the same
//    reference max);
//  * INT8 history rows are dequantised to bf16(code * scale) while they are
//    written to LDS, so the MFMA path is the same for both cache types;
//  * masks are per tile: only tiles at a ragged end or with segment structure
//    evaluate a per-element predicate from a 64-entry key table in LDS; keys
//    of later segments than the workgroup's last query are never loaded;
//  * workgroup ids are remapped so that each XCD (dispatched round-robin)
//    works through contiguous query tiles of the same head, sharing K/V in L2.
#include "internal.h"

// Tuning switches (compile time): waves per workgroup (4 or 8; waves 0-3
// stage K/V tiles, any further waves only compute), minimum waves per SIMD the
// register allocation must allow, and whether QK^T of the next tile is issued
// ahead of the softmax of the current one.
#ifndef SEGC_ATTN_NW
#define SEGC_ATTN_NW 8
#endif
#ifndef SEGC_ATTN_WAVES_PER_SIMD
#define SEGC_ATTN_WAVES_PER_SIMD 2
#endif
#ifndef SEGC_ATTN_PIPELINE
#define SEGC_ATTN_PIPELINE 0
#endif

namespace segc {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                 // keys per tile
constexpr int NW = SEGC_ATTN_NW;       // waves per workgroup
constexpr int NT = NW * 64;
constexpr int NSTAGE = 4;              // waves that stage tiles (16 rows each)
constexpr int BM = 32 * NW;            // query rows per workgroup
constexpr int KS = 136;                // LDS K row stride (bf16 elements, 272 B)
constexpr int K_BYTES = BN * KS * 2;   // 17408
constexpr int V_BYTES = D * BN * 2;    // 16384: V^T rows of 64 keys
constexpr int INFO_BYTES = BN * 4;
constexpr int KBUF0 = 0;
constexpr int VBUF0 = 2 * K_BYTES;
constexpr int INFO0 = VBUF0 + 2 * V_BYTES;
constexpr int LDS_BYTES = INFO0 + 2 * INFO_BYTES;
constexpr float kTau = 8.0f;           // deferred-rescale threshold (log2 units)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// max / sum of x over lanes l and l ^ 32 (both outputs of the swap hold one
// lane of each half, whichever way the halves move)
__device__ inline float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Segment of current row r (scalar loop over at most kMaxSeg entries).
__device__ inline int seg_of(const AttnParams& p, int r) {
  int s = 0;
  for (int i = 1; i < p.n_seg; ++i) s += (r >= p.seg_start[i]) ? 1 : 0;
  return s;
}

struct Tile {
  int hist;      // 1 = history rows, 0 = current rows
  int j0;        // first row (history row index or current row index)
  int nvalid;    // rows [0, nvalid) exist; later rows are clamped and masked
};

__device__ inline Tile tile_at(const AttnParams& p, int t, int cur_end) {
  Tile tl;
  if (t < p.hist_tiles) {
    tl.hist = 1;
    tl.j0 = t * BN;
    tl.nvalid = min(BN, p.n_hist_rows - tl.j0);
  } else {
    tl.hist = 0;
    tl.j0 = (t - p.hist_tiles) * BN;
    tl.nvalid = min(BN, cur_end - tl.j0);
  }
  return tl;
}

__device__ inline bool tile_masked(const AttnParams& p, const Tile& tl) {
  return tl.nvalid < BN || (!tl.hist && p.needs_mask);
}

// Where a wave's 16-row group of a tile lives. Uniform fields describe the
// group's first row; lanes add row offsets (clamped to `lim`).
struct Group {
  int64_t row0;   // history: cache row index of the group's first row; current: row index
  int lim;        // largest valid local row (0..15)
  bool generic;   // history frames not a multiple of 16 tokens: per-lane rows
  int j;          // first tile row of the group (generic path)
};

__device__ inline Group group_at(const AttnParams& p, const Tile& tl, int w, int head) {
  Group g;
  const int last = tl.j0 + tl.nvalid - 1;            // last valid row of the tile
  const int gs = min(tl.j0 + 16 * w, last & ~15);
  g.lim = last - gs;
  g.generic = false;
  g.j = gs;
  if (tl.hist) {
    if (p.G % 16 == 0) {
      const int f = gs / p.G;
      const int slot = p.hist_slots[f];
      g.row0 = ((int64_t)slot * p.n_heads + head) * p.G + (gs - f * p.G);
    } else {
      g.generic = true;
      g.row0 = 0;
    }
  } else {
    g.row0 = gs;
  }
  return g;
}

// Cache row index of local row lr of a history group (generic path: per lane).
__device__ inline int64_t hist_row_generic(const AttnParams& p, const Group& g, int lr, int head) {
  const int row = g.j + lr;
  const int f = row / p.G;
  const int slot = p.hist_slots[f];
  return ((int64_t)slot * p.n_heads + head) * p.G + (row - f * p.G);
}

struct KStage { u32x4 d[4]; float s[2]; };
struct VStage { u32x4 d[4]; float s[4]; };

// ---- K: 4 instructions x (4 rows x 16 chunks of 16 B) = 16 rows per wave
__device__ inline void load_k(const AttnParams& p, const Tile& tl, int w, int lane, int head,
                              KStage& st) {
  const Group g = group_at(p, tl, w, head);
  if (!tl.hist || !p.hist_int8) {
    const int ch = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = min(4 * r + (lane >> 4), g.lim);
      const char* src;
      if (!tl.hist) {
        const char* base = (const char*)(p.k + g.row0 * p.k_st + head * p.k_sh);
        src = base + (uint32_t)(lr * (int)p.k_st * 2);
      } else if (!g.generic) {
        const char* base = (const char*)p.hk + g.row0 * 256;
        src = base + (uint32_t)(lr * 256);
      } else {
        src = (const char*)p.hk + hist_row_generic(p, g, lr, head) * 256;
      }
      st.d[r] = *(const u32x4*)(src + ch * 16);
    }
  } else {
    const int c16 = lane & 7;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int lr = min(8 * i + (lane >> 3), g.lim);
      const int64_t row = g.generic ? hist_row_generic(p, g, lr, head) : g.row0 + lr;
      st.d[i] = *(const u32x4*)((const char*)p.hk + row * 128 + c16 * 16);
      st.s[i] = p.hks[row];
    }
  }
}

// ---- V: lane holds 4 consecutive rows (quad) x 8 elements (chunk c8)
__device__ inline void load_v(const AttnParams& p, const Tile& tl, int w, int lane, int head,
                              VStage& st) {
  const Group g = group_at(p, tl, w, head);
  const int q4 = 4 * (lane >> 4);
  const int c8 = lane & 15;
  if (!tl.hist || !p.hist_int8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = min(q4 + r, g.lim);
      const char* src;
      if (!tl.hist) {
        const char* base = (const char*)(p.v + g.row0 * p.v_st + head * p.v_sh);
        src = base + (uint32_t)(lr * (int)p.v_st * 2);
      } else if (!g.generic) {
        const char* base = (const char*)p.hv + g.row0 * 256;
        src = base + (uint32_t)(lr * 256);
      } else {
        src = (const char*)p.hv + hist_row_generic(p, g, lr, head) * 256;
      }
      st.d[r] = *(const u32x4*)(src + c8 * 16);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = min(q4 + r, g.lim);
      const int64_t row = g.generic ? hist_row_generic(p, g, lr, head) : g.row0 + lr;
      const u32x2 w2 = *(const u32x2*)((const char*)p.hv + row * 128 + c8 * 8);
      st.d[r].x = w2.x;
      st.d[r].y = w2.y;
      st.s[r] = p.hvs[row];
    }
  }
}

// int8 code bytes (4 per dword) times scale -> fp32; (u - 128) * s in one fma.
__device__ inline void dequant4(uint32_t w, float s, float* out) {
  const uint32_t u = w ^ 0x80808080u;
  const float ms = -128.0f * s;
  out[0] = fmaf((float)(u & 0xFFu), s, ms);
  out[1] = fmaf((float)((u >> 8) & 0xFFu), s, ms);
  out[2] = fmaf((float)((u >> 16) & 0xFFu), s, ms);
  out[3] = fmaf((float)(u >> 24), s, ms);
}

__device__ inline void store_k(const AttnParams& p, const Tile& tl, int w, int lane,
                               const KStage& st, char* kbuf) {
  if (!tl.hist || !p.hist_int8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * w + 4 * r + (lane >> 4);
      *(u32x4*)(kbuf + row * (KS * 2) + (lane & 15) * 16) = st.d[r];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * w + 8 * i + (lane >> 3);
      float f[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) dequant4(st.d[i][e], st.s[i], f + 4 * e);
      u32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = pack_bf16(f[2 * e], f[2 * e + 1]);
        b[e] = pack_bf16(f[8 + 2 * e], f[9 + 2 * e]);
      }
      char* dst = kbuf + row * (KS * 2) + (lane & 7) * 32;
      *(u32x4*)dst = a;
      *(u32x4*)(dst + 16) = b;
    }
  }
}

// V^T byte offset of (row d, keys pos..pos+3) with pos a multiple of 4. Keys
// are stored with bits 2 and 3 of their index inside each 16-key chunk
// swapped (pos), and the row's 16-byte chunks XOR-swizzled by (d ^ d>>3) & 7.
__device__ inline int vt_off(int d, int pos) {
  const int sw = (d ^ (d >> 3)) & 7;
  return d * (BN * 2) + ((((pos >> 3) ^ sw) << 4) | ((pos & 4) << 1));
}

// Position of the 4 keys 4*quad..4*quad+3 inside a V^T row.
__device__ inline int vt_pos(int quad) {
  const int m = quad & 3;
  return (quad >> 2) * 16 + (((m & 1) << 1) | (m >> 1)) * 4;
}

__device__ inline void store_v(const AttnParams& p, const Tile& tl, int w, int lane,
                               const VStage& st, char* vbuf) {
  const int quad = 4 * w + (lane >> 4);
  const int c8 = lane & 15;
  const int pos = vt_pos(quad);
  if (!tl.hist || !p.hist_int8) {
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int e = dd >> 1;
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      u32x2 o2;
      o2.x = __builtin_amdgcn_perm(st.d[1][e], st.d[0][e], sel);
      o2.y = __builtin_amdgcn_perm(st.d[3][e], st.d[2][e], sel);
      *(u32x2*)(vbuf + vt_off(8 * c8 + dd, pos)) = o2;
    }
  } else {
    float f[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dequant4(st.d[r].x, st.s[r], f[r]);
      dequant4(st.d[r].y, st.s[r], f[r] + 4);
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      u32x2 o2;
      o2.x = pack_bf16(f[0][dd], f[1][dd]);
      o2.y = pack_bf16(f[2][dd], f[3][dd]);
      *(u32x2*)(vbuf + vt_off(8 * c8 + dd, pos)) = o2;
    }
  }
}

// Visibility table of the tile's 64 keys: [lo, hi] range of query segments
// that may see the key (lo > hi: nobody).
__device__ inline void store_info(const AttnParams& p, const Tile& tl, int tid, int* info) {
  if (tid >= BN) return;
  int lo = 0xFFFF, hi = 0;
  if (tid < tl.nvalid) {
    if (tl.hist) {
      lo = 0;
      hi = 0xFFFF;
    } else {
      const int jc = tl.j0 + tid;
      const int s = seg_of(p, jc);
      const int ti = jc - p.seg_start[s];
      if (ti >= p.seg_text_len[s]) {
        lo = s;
        hi = 0xFFFF;
      } else if (ti < p.seg_text_valid[s]) {
        lo = s;
        hi = s;
      }
    }
  }
  info[tid] = lo | (hi << 16);
}

// S^T (64 keys x 32 queries) = K Q^T from the K tile in LDS.
__device__ inline void qk_tile(const char* kbuf, const bf16x8 (&qf)[8], int lr, int hh,
                               f32x16 (&s)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const char* row = kbuf + (32 * kb + lr) * (KS * 2) + hh * 16;
    bf16x8 a = *(const bf16x8*)row;
    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int dt = 1; dt < 8; ++dt) {
      a = *(const bf16x8*)(row + dt * 32);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dt], s[kb], 0, 0, 0);
    }
  }
}

struct RowState {
  float m, l;
};

// Softmax of one tile (in place: s becomes p) and O rescale when needed.
__device__ inline void softmax_tile(f32x16 (&s)[2], bool masked, const int* info, int qseg, int hh,
                                    float c, RowState& rs, f32x16 (&o)[4]) {
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const i32x4 inf4 = *(const i32x4*)(info + 32 * kb + 8 * jq + 4 * hh);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int lo = inf4[jj] & 0xFFFF, hi = (inf4[jj] >> 16) & 0xFFFF;
          if (qseg < lo || qseg > hi) s[kb][4 * jq + jj] = -INFINITY;
        }
      }
  }
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
  mx = xhalf_max(mx);
  const float mnew = fmaxf(rs.m, mx);
  const bool need = (mnew - rs.m) * c > kTau;          // false for -inf/-inf (NaN)
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = __builtin_amdgcn_exp2f((rs.m - mnew) * c);
    rs.m = mnew;
    rs.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
  }
  const float mc = (rs.m == -INFINITY) ? 0.0f : rs.m * c;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) s[kb][j] = __builtin_amdgcn_exp2f(fmaf(s[kb][j], c, -mc));
}

// O^T += V^T P^T for one tile; the row sum l accumulates the fp32 P values.
__device__ inline void pv_tile(const char* vbuf, const f32x16 (&s)[2], int lr, int hh,
                               f32x16 (&o)[4], RowState& rs) {
  float ls = 0.0f;
#pragma unroll
  for (int ck = 0; ck < 4; ++ck) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] = pack_bf16(s[ck >> 1][8 * (ck & 1) + 2 * e], s[ck >> 1][8 * (ck & 1) + 2 * e + 1]);
      ls += s[ck >> 1][8 * (ck & 1) + 2 * e] + s[ck >> 1][8 * (ck & 1) + 2 * e + 1];
    }
    const bf16x8 pb = as_bf16x8(u);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + lr;
      const int sw = (d ^ (d >> 3)) & 7;
      const bf16x8 a = *(const bf16x8*)(vbuf + d * (BN * 2) + (((2 * ck + hh) ^ sw) << 4));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
    }
  }
  rs.l += ls;
}

__global__ __launch_bounds__(NT, SEGC_ATTN_WAVES_PER_SIMD) void attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // XCD-aware remap: hardware deals workgroup b to XCD b % 8; give each XCD a
  // contiguous range of (head, query tile) in head-major order.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int qn = nwg >> 3, rn = nwg & 7;
  const int logical = (xcd < rn) ? xcd * (qn + 1) + local : rn * (qn + 1) + (xcd - rn) * qn + local;
  const int head = logical / p.n_qtiles;
  const int qtile = logical - head * p.n_qtiles;

  const int m0 = qtile * BM;
  const int wg_last = min(m0 + BM, p.n_cur) - 1;
  const int cur_end = p.seg_start[seg_of(p, wg_last) + 1];   // later keys are future for all
  const int n_tiles = p.hist_tiles + (cur_end + BN - 1) / BN;

  // Q operands (B of S^T = K Q^T) and the query row's segment
  const int qrow = m0 + 32 * w + lr;
  const bool qok = qrow < p.n_cur;
  const int qseg = seg_of(p, qok ? qrow : p.n_cur - 1);
  bf16x8 qf[8];
  {
    const uint16_t* src = p.q + (int64_t)(qok ? qrow : 0) * p.q_st + head * p.q_sh + hh * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (qok) u = *(const u32x4*)(src + 16 * t);
      qf[t] = as_bf16x8(u);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  RowState rs = {-INFINITY, 0.0f};
  const float c = p.scale_log2;

  const bool stager = w < NSTAGE;
#if SEGC_ATTN_PIPELINE
  // prologue: K(0), V(0) (+ key table), K(1) into LDS
  if (stager) {
    KStage ks;
    VStage vs;
    const Tile t0 = tile_at(p, 0, cur_end);
    load_k(p, t0, w, lane, head, ks);
    load_v(p, t0, w, lane, head, vs);
    store_k(p, t0, w, lane, ks, smem + KBUF0);
    store_v(p, t0, w, lane, vs, smem + VBUF0);
    if (tile_masked(p, t0)) store_info(p, t0, tid, (int*)(smem + INFO0));
    if (n_tiles > 1) {
      const Tile t1 = tile_at(p, 1, cur_end);
      load_k(p, t1, w, lane, head, ks);
      store_k(p, t1, w, lane, ks, smem + KBUF0 + K_BYTES);
    }
  }
  __syncthreads();

  f32x16 sa[2], sb[2];
  qk_tile(smem + KBUF0, qf, lr, hh, sa);

  // one pipelined tile: S(t+1) into s_next while s_cur (tile t) is consumed
  auto step = [&](int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
    const bool has_v1 = t + 1 < n_tiles;
    const bool has_k2 = t + 2 < n_tiles;
    const Tile tt = tile_at(p, t, cur_end);
    KStage ks;
    VStage vs;
    const Tile tk = tile_at(p, t + 2, cur_end);
    const Tile tv = tile_at(p, t + 1, cur_end);
    if (has_k2 && stager) load_k(p, tk, w, lane, head, ks);
    if (has_v1) {
      if (stager) load_v(p, tv, w, lane, head, vs);
      qk_tile(smem + KBUF0 + ((t + 1) & 1) * K_BYTES, qf, lr, hh, s_next);
    }
    softmax_tile(s_cur, tile_masked(p, tt), (const int*)(smem + INFO0 + (t & 1) * INFO_BYTES), qseg,
                 hh, c, rs, o);
    pv_tile(smem + VBUF0 + (t & 1) * V_BYTES, s_cur, lr, hh, o, rs);
    if (stager) {
      if (has_k2) store_k(p, tk, w, lane, ks, smem + KBUF0 + (t & 1) * K_BYTES);
      if (has_v1) {
        store_v(p, tv, w, lane, vs, smem + VBUF0 + ((t + 1) & 1) * V_BYTES);
        if (tile_masked(p, tv))
          store_info(p, tv, tid, (int*)(smem + INFO0 + ((t + 1) & 1) * INFO_BYTES));
      }
    }
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  if (t < n_tiles) step(t, sa, sb);
#else
  // prologue: tile 0 into LDS buffer 0
  if (stager) {
    KStage ks;
    VStage vs;
    const Tile t0 = tile_at(p, 0, cur_end);
    load_k(p, t0, w, lane, head, ks);
    load_v(p, t0, w, lane, head, vs);
    store_k(p, t0, w, lane, ks, smem + KBUF0);
    store_v(p, t0, w, lane, vs, smem + VBUF0);
    if (tile_masked(p, t0)) store_info(p, t0, tid, (int*)(smem + INFO0));
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const bool has_next = t + 1 < n_tiles;
    const Tile tt = tile_at(p, t, cur_end);
    const Tile tn = tile_at(p, t + 1, cur_end);
    KStage ks;
    VStage vs;
    if (has_next && stager) {
      load_k(p, tn, w, lane, head, ks);
      load_v(p, tn, w, lane, head, vs);
    }
    const int b = t & 1;
    f32x16 sc[2];
    qk_tile(smem + KBUF0 + b * K_BYTES, qf, lr, hh, sc);
    softmax_tile(sc, tile_masked(p, tt), (const int*)(smem + INFO0 + b * INFO_BYTES), qseg, hh, c,
                 rs, o);
    pv_tile(smem + VBUF0 + b * V_BYTES, sc, lr, hh, o, rs);
    if (has_next && stager) {
      store_k(p, tn, w, lane, ks, smem + KBUF0 + (b ^ 1) * K_BYTES);
      store_v(p, tn, w, lane, vs, smem + VBUF0 + (b ^ 1) * V_BYTES);
      if (tile_masked(p, tn)) store_info(p, tn, tid, (int*)(smem + INFO0 + (b ^ 1) * INFO_BYTES));
    }
    __syncthreads();
  }
#endif

  // epilogue: O = acc / l, bf16; lse = m * sm_scale + ln l
  const float lt = xhalf_sum(rs.l);
  const float inv = 1.0f / lt;
  if (qok) {
    uint16_t* dst = p.o + (int64_t)qrow * p.o_st + head * p.o_sh + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        u32x2 v2;
        v2.x = pack_bf16(o[db][4 * jq] * inv, o[db][4 * jq + 1] * inv);
        v2.y = pack_bf16(o[db][4 * jq + 2] * inv, o[db][4 * jq + 3] * inv);
        *(u32x2*)(dst + 32 * db + 8 * jq) = v2;
      }
    if (p.lse && hh == 0) p.lse[(int64_t)head * p.n_cur + qrow] = rs.m * p.sm_scale + logf(lt);
  }
}

}  // namespace

hipError_t launch_attn(const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  p.n_qtiles = (p.n_cur + BM - 1) / BM;
  const int64_t nwg = (int64_t)p.n_qtiles * p.n_heads;
  // more than 64 KB of dynamic LDS must be allowed explicitly (gfx950 has 160 KB per CU)
  hipError_t e = hipFuncSetAttribute((const void*)attn_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)nwg), dim3(NT), LDS_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace segc
