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
// Design (one workgroup = 4 waves = one (query tile, head)):
//  * each wave owns 32*QG query rows; Q stays in registers as MFMA B operands;
//  * key tiles of 64 rows are staged through LDS, double buffered: K row-major
//    [key][d] (272-byte rows), V transposed [d][key'] (144-byte rows) so that
//    both MFMA operands are single 16-byte LDS reads; global loads for tile
//    t+1 are issued before tile t is computed;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys land in accumulator
//    registers and queries across lanes, so a row max needs only one
//    cross-half exchange; O^T = V^T P^T reuses the S^T accumulators as the
//    P operand directly (V^T is stored in the matching key order);
//  * online softmax in base 2 with the rescale of O deferred until the running
//    max grows by more than 2^8 (exact: the final division uses the same
//    reference max);
//  * INT8 history rows are dequantised to bf16(code * scale) while they are
//    written to LDS, so the MFMA path is the same for both cache types;
//  * masks are per tile: only tiles at a ragged end or with segment structure
//    evaluate a per-element predicate from a 64-entry key table in LDS; tiles
//    invisible to a whole wave are skipped; keys of later segments than the
//    workgroup's last query are never loaded;
//  * workgroup ids are remapped so that each XCD (dispatched round-robin)
//    works through contiguous query tiles of the same head, sharing K/V in L2.
#include "internal.h"

namespace segc {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                 // keys per tile
constexpr int NW = 4;                  // waves per workgroup
constexpr int NT = NW * 64;
constexpr int KS = 136;                // LDS K row stride (bf16 elements)
constexpr int VS = 72;                 // LDS V^T row stride (bf16 elements)
constexpr int K_ELEMS = BN * KS;
constexpr int V_ELEMS = D * VS;
constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 2 + BN * 4;
constexpr float kTau = 8.0f;           // deferred-rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

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

// Segment of current row r (scalar loop over at most kMaxSeg entries).
__device__ inline int seg_of(const AttnParams& p, int r) {
  int s = 0;
  for (int i = 1; i < p.n_seg; ++i) s += (r >= p.seg_start[i]) ? 1 : 0;
  return s;
}

// Where the rows of one key tile come from (uniform across the workgroup).
struct TileSrc {
  int hist;      // 1 = history rows, 0 = current rows
  int j0;        // first row (history row index or current row index)
  int nvalid;    // rows [0, nvalid) exist; the rest are zero-filled
  int f0, r0;    // history: frame of row j0 and row inside that frame
  int slot0, slot1;
};

__device__ inline TileSrc tile_src(const AttnParams& p, int t, int cur_end) {
  TileSrc ts;
  if (t < p.hist_tiles) {
    ts.hist = 1;
    ts.j0 = t * BN;
    ts.nvalid = min(BN, p.n_hist_rows - ts.j0);
    ts.f0 = ts.j0 / p.G;
    ts.r0 = ts.j0 - ts.f0 * p.G;
    const int n_hist = p.n_hist_rows / p.G;
    ts.slot0 = p.hist_slots[ts.f0];
    ts.slot1 = (ts.f0 + 1 < n_hist) ? p.hist_slots[ts.f0 + 1] : ts.slot0;
  } else {
    ts.hist = 0;
    ts.j0 = (t - p.hist_tiles) * BN;
    ts.nvalid = min(BN, cur_end - ts.j0);
    ts.f0 = ts.r0 = ts.slot0 = ts.slot1 = 0;
  }
  return ts;
}

// Cache row index (in units of 128 elements) of history tile row o.
__device__ inline int64_t hist_row(const AttnParams& p, const TileSrc& ts, int head, int o) {
  int rr = ts.r0 + o;
  int slot;
  if (p.G >= BN) {
    const bool nx = rr >= p.G;
    slot = nx ? ts.slot1 : ts.slot0;
    rr = nx ? rr - p.G : rr;
  } else {
    int f = ts.f0;
    while (rr >= p.G) {
      rr -= p.G;
      ++f;
    }
    slot = p.hist_slots[f];
  }
  return ((int64_t)slot * p.n_heads + head) * p.G + rr;
}

// Registers holding one tile's global loads between issue and LDS write.
struct Stage {
  u32x4 k[4];
  u32x4 v[4];
  float ks[2];
  float vs[4];
};

__device__ inline void issue_loads(const AttnParams& p, const TileSrc& ts, int head, int tid,
                                   Stage& st) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int quad = tid & 15, c8 = tid >> 4;
  if (!ts.hist || !p.hist_int8) {
    // bf16 rows: K as 16-byte chunks (16 lanes per row), V as 4 rows x 8 d
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i;
      const int o = c >> 4, col = c & 15;
      st.k[i] = z;
      if (o < ts.nvalid) {
        const uint16_t* src = ts.hist
            ? (const uint16_t*)p.hk + hist_row(p, ts, head, o) * D
            : p.k + (int64_t)(ts.j0 + o) * p.k_st + head * p.k_sh;
        st.k[i] = *(const u32x4*)(src + col * 8);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = quad * 4 + r;
      st.v[r] = z;
      if (o < ts.nvalid) {
        const uint16_t* src = ts.hist
            ? (const uint16_t*)p.hv + hist_row(p, ts, head, o) * D
            : p.v + (int64_t)(ts.j0 + o) * p.v_st + head * p.v_sh;
        st.v[r] = *(const u32x4*)(src + c8 * 8);
      }
    }
  } else {
    // int8 history rows: K as 16-code chunks (8 lanes per row), V as 4 rows x 8 codes
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + NT * i;
      const int o = c >> 3, col = c & 7;
      st.k[i] = z;
      st.ks[i] = 0.0f;
      if (o < ts.nvalid) {
        const int64_t row = hist_row(p, ts, head, o);
        st.k[i] = *(const u32x4*)((const int8_t*)p.hk + row * D + col * 16);
        st.ks[i] = p.hks[row];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = quad * 4 + r;
      st.v[r] = z;
      st.vs[r] = 0.0f;
      if (o < ts.nvalid) {
        const int64_t row = hist_row(p, ts, head, o);
        const u32x2 w = *(const u32x2*)((const int8_t*)p.hv + row * D + c8 * 8);
        st.v[r].x = w.x;
        st.v[r].y = w.y;
        st.vs[r] = p.hvs[row];
      }
    }
  }
}

// Offset (keys) of the 4 consecutive keys 4*quad..4*quad+3 inside a V^T row.
// Within each 16-key chunk, key bits 2 and 3 are swapped so that the 8 keys a
// lane half feeds to one PV MFMA are contiguous.
__device__ inline int vt_pos(int quad) {
  const int m = quad & 3;
  return (quad >> 2) * 16 + (((m & 1) << 1) | (m >> 1)) * 4;
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

__device__ inline void write_lds(const AttnParams& p, const TileSrc& ts, int tid, const Stage& st,
                                 char* buf, bool need_info, int cur_end) {
  uint16_t* Kl = (uint16_t*)buf;
  uint16_t* Vl = Kl + K_ELEMS;
  int* info = (int*)(Vl + V_ELEMS);
  const int quad = tid & 15, c8 = tid >> 4;
  const int vp = vt_pos(quad);
  if (!ts.hist || !p.hist_int8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i;
      *(u32x4*)(Kl + (c >> 4) * KS + (c & 15) * 8) = st.k[i];
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1;
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      u32x2 o2;
      o2.x = __builtin_amdgcn_perm(st.v[1][w], st.v[0][w], sel);
      o2.y = __builtin_amdgcn_perm(st.v[3][w], st.v[2][w], sel);
      *(u32x2*)(Vl + (c8 * 8 + dd) * VS + vp) = o2;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + NT * i;
      const int o = c >> 3, col = c & 7;
      float f[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) dequant4(st.k[i][w], st.ks[i], f + 4 * w);
      u32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = pack_bf16(f[2 * e], f[2 * e + 1]);
        b[e] = pack_bf16(f[8 + 2 * e], f[8 + 2 * e + 1]);
      }
      *(u32x4*)(Kl + o * KS + col * 16) = a;
      *(u32x4*)(Kl + o * KS + col * 16 + 8) = b;
    }
    float f[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dequant4(st.v[r].x, st.vs[r], f[r]);
      dequant4(st.v[r].y, st.vs[r], f[r] + 4);
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      u32x2 o2;
      o2.x = pack_bf16(f[0][dd], f[1][dd]);
      o2.y = pack_bf16(f[2][dd], f[3][dd]);
      *(u32x2*)(Vl + (c8 * 8 + dd) * VS + vp) = o2;
    }
  }
  if (need_info && tid < BN) {
    // [lo, hi] range of query segments that may see key tid; lo > hi = nobody
    int lo = 0xFFFF, hi = 0;
    if (tid < ts.nvalid) {
      if (ts.hist) {
        lo = 0;
        hi = 0xFFFF;
      } else {
        const int jc = ts.j0 + tid;
        if (jc < cur_end) {
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
    }
    info[tid] = lo | (hi << 16);
  }
}

template <int QG>
__global__ __launch_bounds__(NT, 1) void attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hh = lane >> 5;

  // XCD-aware remap: hardware deals workgroup b to XCD b % 8; give each XCD a
  // contiguous range of (head, query tile) in head-major order.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, local = b >> 3;
  const int qn = nwg >> 3, rn = nwg & 7;
  const int logical = (xcd < rn) ? xcd * (qn + 1) + local : rn * (qn + 1) + (xcd - rn) * qn + local;
  const int head = logical / p.n_qtiles;
  const int qtile = logical - head * p.n_qtiles;

  constexpr int BM = 32 * QG * NW;
  const int m0 = qtile * BM;
  const int wg_last = min(m0 + BM, p.n_cur) - 1;
  const int cur_end = p.seg_start[seg_of(p, wg_last) + 1];   // later keys are future for all
  const int n_tiles = p.hist_tiles + (cur_end + BN - 1) / BN;

  const int w0 = m0 + wave * 32 * QG;
  const bool wave_live = w0 < p.n_cur;
  const int w_last = min(w0 + 32 * QG, p.n_cur) - 1;
  const int w_vis_end = wave_live ? p.seg_start[seg_of(p, w_last) + 1] : 0;

  // Q operands and per-row segment
  bf16x8 qf[QG][8];
  int qs[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int row = w0 + 32 * g + lr;
    const bool ok = row < p.n_cur;
    qs[g] = seg_of(p, ok ? row : p.n_cur - 1);
    const uint16_t* src = p.q + (int64_t)(ok ? row : 0) * p.q_st + head * p.q_sh + hh * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (ok) u = *(const u32x4*)(src + 16 * t);
      qf[g][t] = as_bf16x8(u);
    }
  }

  f32x16 oacc[4][QG];
  float mrow[QG], lrow[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    mrow[g] = -INFINITY;
    lrow[g] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][g][j] = 0.0f;
  }
  const float c = p.scale_log2;

  auto tile_needs_info = [&](const TileSrc& ts) -> bool {
    return ts.nvalid < BN || (!ts.hist && p.needs_mask);
  };

  Stage st;
  TileSrc ts_next = tile_src(p, 0, cur_end);
  issue_loads(p, ts_next, head, tid, st);
  write_lds(p, ts_next, tid, st, smem, tile_needs_info(ts_next), cur_end);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const TileSrc ts = ts_next;
    const bool have_next = t + 1 < n_tiles;
    if (have_next) {
      ts_next = tile_src(p, t + 1, cur_end);
      issue_loads(p, ts_next, head, tid, st);
    }
    char* buf = smem + (t & 1) * BUF_BYTES;
    const bool skip = !wave_live || (!ts.hist && ts.j0 >= w_vis_end);
    if (!skip) {
      const uint16_t* Kl = (const uint16_t*)buf;
      const uint16_t* Vl = Kl + K_ELEMS;
      const int* info = (const int*)(Vl + V_ELEMS);

      f32x16 sacc[2][QG];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < QG; ++g)
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[kb][g][j] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *(const bf16x8*)(Kl + (32 * kb + lr) * KS + 16 * dt + 8 * hh);
#pragma unroll
          for (int g = 0; g < QG; ++g)
            sacc[kb][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[g][dt], sacc[kb][g], 0, 0, 0);
        }
      }

      if (tile_needs_info(ts)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const i32x4 inf4 = *(const i32x4*)(info + 32 * kb + 8 * jq + 4 * hh);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int lo = inf4[jj] & 0xFFFF, hi = (inf4[jj] >> 16) & 0xFFFF;
#pragma unroll
              for (int g = 0; g < QG; ++g)
                if (qs[g] < lo || qs[g] > hi) sacc[kb][g][4 * jq + jj] = -INFINITY;
            }
          }
      }

#pragma unroll
      for (int g = 0; g < QG; ++g) {
        float mx = sacc[0][g][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][g][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow[g], mx);
        const bool need = (mnew - mrow[g]) * c > kTau;   // false for -inf/-inf (NaN)
        if (__ballot(need)) {
          const float alpha = __builtin_amdgcn_exp2f((mrow[g] - mnew) * c);
          mrow[g] = mnew;
          lrow[g] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][g][j] *= alpha;
        }
        const float mc = (mrow[g] == -INFINITY) ? 0.0f : mrow[g] * c;
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][g][j], c, -mc));
            sacc[kb][g][j] = e;
            ls += e;
          }
        lrow[g] += ls;
      }

#pragma unroll
      for (int ck = 0; ck < 4; ++ck) {
        bf16x8 pb[QG];
#pragma unroll
        for (int g = 0; g < QG; ++g) {
          u32x4 u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            u[e] = pack_bf16(sacc[ck >> 1][g][8 * (ck & 1) + 2 * e],
                             sacc[ck >> 1][g][8 * (ck & 1) + 2 * e + 1]);
          pb[g] = as_bf16x8(u);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a = *(const bf16x8*)(Vl + (32 * db + lr) * VS + 16 * ck + 8 * hh);
#pragma unroll
          for (int g = 0; g < QG; ++g)
            oacc[db][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[g], oacc[db][g], 0, 0, 0);
        }
      }
    }
    if (have_next)
      write_lds(p, ts_next, tid, st, smem + ((t + 1) & 1) * BUF_BYTES, tile_needs_info(ts_next),
                cur_end);
    __syncthreads();
  }

  // epilogue: O = acc / l, bf16; lse = m * sm_scale + ln l
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const float lt = lrow[g] + __shfl_xor(lrow[g], 32);
    const float inv = 1.0f / lt;
    const int row = w0 + 32 * g + lr;
    if (row < p.n_cur) {
      uint16_t* dst = p.o + (int64_t)row * p.o_st + head * p.o_sh + 4 * hh;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          u32x2 w;
          w.x = pack_bf16(oacc[db][g][4 * jq] * inv, oacc[db][g][4 * jq + 1] * inv);
          w.y = pack_bf16(oacc[db][g][4 * jq + 2] * inv, oacc[db][g][4 * jq + 3] * inv);
          *(u32x2*)(dst + 32 * db + 8 * jq) = w;
        }
      if (p.lse && hh == 0) p.lse[(int64_t)head * p.n_cur + row] = mrow[g] * p.sm_scale + logf(lt);
    }
  }
}

template <int QG>
hipError_t launch_qg(const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  constexpr int BM = 32 * QG * NW;
  p.n_qtiles = (p.n_cur + BM - 1) / BM;
  const int64_t nwg = (int64_t)p.n_qtiles * p.n_heads;
  // more than 64 KB of dynamic LDS must be allowed explicitly (gfx950 has 160 KB per CU)
  hipError_t e = hipFuncSetAttribute((const void*)attn_kernel<QG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 2 * BUF_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_kernel<QG>, dim3((unsigned)nwg), dim3(NT), 2 * BUF_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  return launch_qg<1>(p, s);
}

}  // namespace segc
