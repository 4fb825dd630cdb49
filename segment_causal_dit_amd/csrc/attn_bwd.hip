// Gradients of segment-wise causal joint attention in the packed training
// form (every segment of the sequence present, no cache), on gfx950 bf16 MFMA.
//
// Source: "Hy-Nomas Explained: How Tencent's Open World Model Runs Steerable
// Video on an RTX 4090", section "The training recipe" (segment-forcing
// training on sequences packed offline, up to 360,000 tokens); the attention
// differentiated is that of the model card's section "Segment-Autoregressive
// Diffusion Transformer" (the same segment-causal mask as the forward).
//
// What is computed, per head, for upstream gradient do of the forward output
// o (p = softmax of sm_scale q.k over visible keys, recomputed from the
// forward's lse):
//   delta_i = do_i . o_i
//   dv_j = sum_i p_ij do_i
//   ds_ij = p_ij (do_i . v_j - delta_i)
//   dq_i = sm_scale sum_j ds_ij k_j,   dk_j = sm_scale sum_i ds_ij q_i
//
// Three kernels:
//  * delta: 16 lanes per (row, head);
//  * dQ: one workgroup = 8 waves = 256 query rows of one head (two waves per
//    SIMD); each wave keeps its 32 rows' q and do as MFMA B operands and
//    walks the key tiles it can see: S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T with K^T from the transposing LDS read;
//  * dK/dV: one workgroup = 8 waves = 128 keys of one head (two waves per
//    SIMD); K and V of the 128 keys sit in LDS and are re-read as B
//    operands, so that the two 128 x 32 fp32 accumulators of a wave fit
//    beside them; wave w owns keys 32 (w mod 4) .. + 31 and query rows
//    32 floor(w / 4) .. + 31 of every 64-row query tile, walks the query
//    tiles that can see its keys: S = Q K^T, dP = dO V^T, then
//    dV^T += dO^T P and dK^T += Q^T dS; the two waves of a key group add
//    their partial dK and dV through LDS at the end.
// 64-row tiles are staged through LDS, double buffered, by direct global->LDS
// loads issued from inline assembly and awaited explicitly once per tile (the
// dK/dV kernel issues the next tile's loads after six of the eight steps of
// the current tile's S and dP products, and fetches its lse and delta in the
// same place). Both kernels order their workgroups XCD-aware and head-major.
// Chunk c of tile row r sits at c ^ (((r & 3) << 2) | ((r >> 2) & 3)): every
// read by rows (16 consecutive rows, one chunk) and every transposing read
// (4 aligned chunks of 4 aligned rows) touches distinct bank groups. Tile
// pairs in which every key is video of a segment no later than the first
// query's segment are fully visible and skip the per-element mask.
#include "internal.h"
#include "lds_dma.h"
#include "segtab.h"

namespace segc {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                     // rows per staged tile
constexpr int TILE_BYTES = BN * D * 2;
constexpr int TAB_BYTES = 3 * BN * 4;      // per-row tables of a staged tile
constexpr int AOFF = 0, BOFF = TILE_BYTES, TOFF = 2 * TILE_BYTES;
constexpr int BUF_BYTES = 2 * TILE_BYTES + TAB_BYTES;
constexpr int LDS_BYTES = 2 * BUF_BYTES;   // double buffered
constexpr int NSTAGE = 4;                  // staging waves, 16 rows each
constexpr int RW = BN / NSTAGE;

constexpr int QW = 8;                      // dQ: waves per workgroup
constexpr int QT = QW * 64;
constexpr int QBM = 32 * QW;               // dQ: query rows per workgroup
constexpr int KW = 8;                      // dK/dV: waves per workgroup
constexpr int KT = KW * 64;
constexpr int KBN = 128;                   // dK/dV: keys per workgroup
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ inline int t_off(int r, int c) { return r * 256 + ((c ^ swz(r)) << 4); }

__device__ inline void dload_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline int seg_of(const AttnBwdParams& p, int r) {
  int s = 0;
  for (int i = 1; i < p.n_seg; ++i) s += (r >= p.seg_start[i]) ? 1 : 0;
  return s;
}

// Logical index of this workgroup in a launch of nwg: workgroup b runs on XCD
// b % 8, and each XCD gets a contiguous range (the first nwg % 8 XCDs one
// more), so the workgroups resident on one XCD take neighbouring indices.
__device__ inline int xcd_head_major(int nwg) {
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int qn = nwg >> 3, rn = nwg & 7;
  return (xcd < rn) ? xcd * (qn + 1) + local : rn * (qn + 1) + (xcd - rn) * qn + local;
}

// no text row (valid or padded) in [a, b)
__device__ inline bool all_video(const AttnBwdParams& p, int a, int b) {
  bool ok = true;
  for (int s = 0; s < p.n_seg; ++s) {
    const int t0 = p.seg_start[s], t1 = t0 + p.seg_text_len[s];
    ok = ok && (t1 <= a || t0 >= b);
  }
  return ok;
}

// Query-segment range [lo, hi] that may see key row j (lo > hi: nobody).
__device__ inline void key_range(const AttnBwdParams& p, int j, int& lo, int& hi) {
  lo = 0xFFFF;
  hi = 0;
  if (j >= p.n) return;
  const int s = seg_of(p, j);
  const int ti = j - p.seg_start[s];
  if (ti >= p.seg_text_len[s]) {
    lo = s;
    hi = 0xFFFF;
  } else if (ti < p.seg_text_valid[s]) {
    lo = s;
    hi = s;
  }
}

// Staging wave w loads rows [16 w, 16 w + 16) of a 64-row tile starting at
// row0 of two row-major tensors (a: head base + row stride; b likewise) into
// the A and B tiles of buf; rows past nvalid repeat the last valid row.
__device__ inline void stage_rows(const uint16_t* a, int64_t a_st, const uint16_t* b, int64_t b_st,
                                  int row0, int nvalid, int w, int lane, char* buf) {
  const char* ar[RW / 4];
  const char* br[RW / 4];
#pragma unroll
  for (int e = 0; e < RW / 4; ++e) {
    const int r = row0 + min(RW * w + 4 * e + (lane >> 4), nvalid - 1);
    ar[e] = (const char*)(a + (int64_t)r * a_st);
    br[e] = (const char*)(b + (int64_t)r * b_st);
  }
#pragma unroll
  for (int e = 0; e < RW / 4; ++e) {
    const int row = RW * w + 4 * e + (lane >> 4);
    const int pc = lane & 15;
    char* dst = buf + (RW * w + 4 * e) * 256;
    dload16(ar[e] + ((pc ^ swz(row)) << 4), dst + AOFF);
    dload16(br[e] + ((pc ^ swz(row)) << 4), dst + BOFF);
  }
}

// acc[kb] = T[32 kb + ..][:] F^T over the 128 columns: rows of the tile in
// the accumulator registers, the lanes' fragment columns across lanes. The
// two 32-row blocks form two interleaved chains; reads run 4 MFMAs ahead.
__device__ inline void rows_x_frag(const char* tile, const bf16x8 (&f)[8], int lr, int hh,
                                   f32x16 (&acc)[2]) {
  bf16x8 a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = *(const bf16x8*)(tile + t_off(32 * (i & 1) + lr, 2 * (i >> 1) + hh));
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], f[0], f32x16{}, 0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], f[0], f32x16{}, 0, 0, 0);
#pragma unroll
  for (int dt = 1; dt < 8; ++dt) {
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * dt], f[dt], acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * dt + 1], f[dt], acc[1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// The 64 accumulator values of x (rows 32 kb + 8 (j / 4) + 4 hh + (j % 4))
// as bf16 B operands over the tile rows: chunk ck holds rows 16 ck + 4 hh +
// 0..3 in slots 0-3 and 16 ck + 8 + 4 hh + 0..3 in slots 4-7.
__device__ inline void pack_rows(const f32x16 (&x)[2], u32x4 (&pk)[4]) {
  // packed words go into a plain array first and into each vector in one
  // piece (element-wise writes of vectors inside unrolled loops have lost
  // values in this compiler's output)
#pragma unroll
  for (int ck = 0; ck < 4; ++ck) {
    uint32_t wd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wd[e] = pack_bf16(x[ck >> 1][8 * (ck & 1) + 2 * e], x[ck >> 1][8 * (ck & 1) + 2 * e + 1]);
    pk[ck] = u32x4{wd[0], wd[1], wd[2], wd[3]};
  }
}

// out[db] += T^T[32 db + ..][rows] pk[rows][lanes]: the tile's columns as
// accumulator rows. T^T comes from the row-major tile through the transposing
// LDS read: inside each 16-lane group, lane j addresses 4 elements of row
// base + j / 4 at column d0 + 4 (j % 4); lane i then holds rows base..base+3
// of column d0 + i. Two reads give the 8 rows a pk chunk holds in this half.
__device__ inline void tileT_x_packed(const char* tile, const u32x4 (&pk)[4], int lane, int hh,
                                      f32x16 (&out)[4]) {
  const int gi = lane & 15;
  const int hb = ((gi & 3) >> 1) | (((lane >> 4) & 1) << 1);
  const int r0 = 4 * hh + (gi >> 2);
  const int sub = 8 * (gi & 1);
#pragma unroll
  for (int ck = 0; ck < 4; ++ck) {
    const bf16x8 pb = as_bf16x8(pk[ck]);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + t_off(16 * ck + r0, 4 * db + hb) + sub));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + t_off(16 * ck + r0 + 8, 4 * db + hb) + sub));
      const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      out[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb, out[db], 0, 0, 0);
    }
  }
}

// 8 B-operand fragments of one row of a row-major tensor (k = columns): lane
// half hh holds columns 16 dt + 8 hh .. + 7 of the row; zeros when !ok.
__device__ inline void load_frags(const uint16_t* row, bool ok, int hh, bf16x8 (&f)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (ok) u = *(const u32x4*)(row + hh * 8 + 16 * t);
    f[t] = as_bf16x8(u);
  }
}

// 128 accumulated columns of this lane's row (x[db][j]: column 32 db + 8 (j / 4)
// + 4 hh + (j % 4)) times `scale`, stored as bf16.
__device__ inline void store_row(uint16_t* row, int hh, const f32x16 (&x)[4], float scale) {
  uint16_t* dst = row + 4 * hh;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const u32x2 v2 = {pack_bf16(x[db][4 * jq] * scale, x[db][4 * jq + 1] * scale),
                        pack_bf16(x[db][4 * jq + 2] * scale, x[db][4 * jq + 3] * scale)};
      *(u32x2*)(dst + 32 * db + 8 * jq) = v2;
    }
}

// ------------------------------------------------------------------ delta ----

constexpr int kDeltaRows = 16;

__global__ __launch_bounds__(256) void delta_kernel(AttnBwdParams p) {
  const int tid = threadIdx.x;
  const int head = blockIdx.y;
  const int r = blockIdx.x * kDeltaRows + (tid >> 4);
  const int li = tid & 15;
  if (r >= p.n) return;                       // whole 16-lane groups leave together
  const u32x4 ov = *(const u32x4*)(p.o + (int64_t)r * p.o_st + (int64_t)head * p.o_sh + li * 8);
  const u32x4 dv = *(const u32x4*)(p.dout + (int64_t)r * p.do_st + (int64_t)head * p.do_sh + li * 8);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(__uint_as_float(ov[e] << 16), __uint_as_float(dv[e] << 16), acc);
    acc = fmaf(__uint_as_float(ov[e] & 0xFFFF0000u), __uint_as_float(dv[e] & 0xFFFF0000u), acc);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (li == 0) p.delta[(int64_t)head * p.n + r] = acc;
}

// --------------------------------------------------------------------- dQ ----

__global__ __launch_bounds__(QT, 2) void dq_kernel(AttnBwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;
  // Workgroup b runs on XCD b % 8; each XCD takes a contiguous head-major
  // range, so the workgroups resident on one XCD walk the same head's key
  // tiles and share them in its L2. Inside a head the heaviest query tiles
  // (the last ones see the most keys) go first.
  const int nwg = gridDim.x;
  const int n_qt = nwg / p.n_heads;
  const int logical = xcd_head_major(nwg);
  const int head = logical / n_qt;
  const int qtile = n_qt - 1 - (logical - head * n_qt);

  const int m0 = qtile * QBM;
  const int wg_last = min(m0 + QBM, p.n) - 1;
  const int cur_end = p.seg_start[seg_of(p, wg_last) + 1];   // later keys are invisible to all
  const int n_tiles = (cur_end + BN - 1) / BN;
  const int qseg_first = seg_of(p, m0);

  const int qrow = m0 + 32 * w + lr;
  const bool qok = qrow < p.n;
  const int qseg = seg_of(p, qok ? qrow : p.n - 1);
  bf16x8 qf[8], df[8];
  load_frags(p.q + (int64_t)(qok ? qrow : 0) * p.q_st + (int64_t)head * p.q_sh, qok, hh, qf);
  load_frags(p.dout + (int64_t)(qok ? qrow : 0) * p.do_st + (int64_t)head * p.do_sh, qok, hh, df);
  // rows past the end: lse = +inf makes their p exactly 0
  const float lse2 = qok ? p.lse[(int64_t)head * p.n + qrow] * kLog2e : INFINITY;
  const float dlt = qok ? p.delta[(int64_t)head * p.n + qrow] : 0.0f;
  // settle these loads here: a wait for them inside the loop would also
  // drain the direct loads in flight there
  __builtin_amdgcn_s_waitcnt(0);

  const uint16_t* kb = p.k + (int64_t)head * p.k_sh;
  const uint16_t* vb = p.v + (int64_t)head * p.v_sh;
  const bool stager = w < NSTAGE;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  const float c = p.scale_log2;

  // mask state of key tile t (decided once per tile, in order) and the key
  // table of a masked tile: [lo, hi] query-segment range per key
  FreeRuns fr;
  fr.init(p, BN, qseg_first);
  SegWalk kw;
  kw.init(p, 0);
  auto tile_masked = [&](int t) {
    const int j0 = t * BN;
    kw.at(p, j0);
    return j0 + BN > cur_end || (p.needs_mask && !fr.free(p, BN, qseg_first, t));
  };
  auto finish = [&](int t, char* buf, bool masked) {
    dload_wait();
    if (masked && tid < BN)
      ((int*)(buf + TOFF))[tid] = key_visibility(p, kw.s, t * BN, BN, t * BN + tid, t * BN + tid < cur_end);
  };
  bool masked = tile_masked(0);
  if (stager) stage_rows(kb, p.k_st, vb, p.v_st, 0, min(BN, cur_end), w, lane, smem);
  finish(0, smem, masked);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    char* const cur = smem + (t & 1) * BUF_BYTES;
    char* const nxt = smem + ((t + 1) & 1) * BUF_BYTES;
    const bool has_next = t + 1 < n_tiles;
    const int j0 = t * BN;
    if (stager && has_next)
      stage_rows(kb, p.k_st, vb, p.v_st, j0 + BN, min(BN, cur_end - j0 - BN), w, lane, nxt);
    f32x16 s[2], dp[2];
    rows_x_frag(cur + AOFF, qf, lr, hh, s);      // S^T = K Q^T
    rows_x_frag(cur + BOFF, df, lr, hh, dp);     // dP^T = V dO^T
    if (masked) {
      const int* info = (const int*)(cur + TOFF);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const i32x4 inf4 = *(const i32x4*)(info + 32 * kb2 + 8 * jq + 4 * hh);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int lo = inf4[jj] & 0xFFFF, hi = (inf4[jj] >> 16) & 0xFFFF;
            if (qseg < lo || qseg > hi) s[kb2][4 * jq + jj] = -INFINITY;
          }
        }
    }
    f32x16 ds[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kb2][j], c, -lse2));
        ds[kb2][j] = pr * (dp[kb2][j] - dlt);
      }
    u32x4 pk[4];
    pack_rows(ds, pk);
    tileT_x_packed(cur + AOFF, pk, lane, hh, acc);   // dQ^T += K^T dS^T
    bool masked_next = false;
    if (has_next) {
      masked_next = tile_masked(t + 1);
      finish(t + 1, nxt, masked_next);
    }
    __syncthreads();
    masked = masked_next;
  }
  if (qok) store_row(p.dq + (int64_t)qrow * p.dq_st + (int64_t)head * p.dq_sh, hh, acc, p.sm_scale);
}

// ------------------------------------------------------------------- dK/dV ----

// Staging wave w of `nwaves` loads rows [rpw w, rpw w + rpw) of a tile of two
// row-major tensors starting at row0 into dstA / dstB (rows past nvalid
// repeat the last valid row).
template <int RPW>
__device__ inline void stage_pair(const uint16_t* a, int64_t a_st, const uint16_t* b, int64_t b_st,
                                  int row0, int nvalid, int w, int lane, char* dstA, char* dstB) {
  if (RPW * w + RPW <= nvalid) {
    // a whole group (no clamping): uniform bases and loop-invariant lane offsets
    const uint64_t ab = uniform_addr(a + (int64_t)(row0 + RPW * w) * a_st);
    const uint64_t bb = uniform_addr(b + (int64_t)(row0 + RPW * w) * b_st);
    const uint32_t lrow = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int e = 0; e < RPW / 4; ++e) {
      const uint32_t r = 4 * e + lrow;
      const uint32_t sw = (pc ^ swz(RPW * w + r)) << 4;
      dload16_s(r * (uint32_t)a_st * 2 + sw, ab, dstA + (RPW * w + 4 * e) * 256);
      dload16_s(r * (uint32_t)b_st * 2 + sw, bb, dstB + (RPW * w + 4 * e) * 256);
    }
    return;
  }
  const char* ar[RPW / 4];
  const char* br[RPW / 4];
#pragma unroll
  for (int e = 0; e < RPW / 4; ++e) {
    const int r = row0 + min(RPW * w + 4 * e + (lane >> 4), nvalid - 1);
    ar[e] = (const char*)(a + (int64_t)r * a_st);
    br[e] = (const char*)(b + (int64_t)r * b_st);
  }
#pragma unroll
  for (int e = 0; e < RPW / 4; ++e) {
    const int row = RPW * w + 4 * e + (lane >> 4);
    const int pc = lane & 15;
    dload16(ar[e] + ((pc ^ swz(row)) << 4), dstA + (RPW * w + 4 * e) * 256);
    dload16(br[e] + ((pc ^ swz(row)) << 4), dstB + (RPW * w + 4 * e) * 256);
  }
}

// out[db] += T^T[32 db + ..][rows rbase + ..] pk[..]: as tileT_x_packed over
// the 32 tile rows from rbase (two 16-row chunks).
__device__ inline void tileT_x_packed32(const char* tile, int rbase, const u32x4 (&pk)[2], int lane, int hh,
                                        f32x16 (&out)[4]) {
  const int gi = lane & 15;
  const int hb = ((gi & 3) >> 1) | (((lane >> 4) & 1) << 1);
  const int r0 = rbase + 4 * hh + (gi >> 2);
  const int sub = 8 * (gi & 1);
#pragma unroll
  for (int ck = 0; ck < 2; ++ck) {
    const bf16x8 pb = as_bf16x8(pk[ck]);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + t_off(16 * ck + r0, 4 * db + hb) + sub));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + t_off(16 * ck + r0 + 8, 4 * db + hb) + sub));
      const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      out[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb, out[db], 0, 0, 0);
    }
  }
}

constexpr int KV_BYTES = 2 * KBN * D * 2;              // K and V rows of the workgroup's keys
constexpr int KLDS_BYTES = KV_BYTES + 2 * BUF_BYTES;
static_assert(KW == 8 && KBN == 128, "dK/dV: 4 key groups x 2 query halves");
static_assert(4 * 2 * 16384 <= KLDS_BYTES, "room for the partial sums of the wave pairs");

// Wave w owns keys 32 (w & 3) .. + 31 of the workgroup and query rows
// 32 (w >> 2) .. + 31 of every 64-row tile; the two waves of a key group add
// their partial dK and dV through LDS at the end.
__global__ __launch_bounds__(KT, 2) void dkdv_kernel(AttnBwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w & 3, qh = w >> 2;
  const int lr = lane & 31, hh = lane >> 5;
  // XCD-aware head-major order as in the dQ kernel; inside a head the first
  // key tiles, seen by the most queries, go first
  const int nwg = gridDim.x;
  const int n_kt = nwg / p.n_heads;
  const int logical = xcd_head_major(nwg);
  const int head = logical / n_kt;
  const int ktile = logical - head * n_kt;

  const int j0 = ktile * KBN;
  const int j1 = min(j0 + KBN, p.n);
  const int q_begin = p.seg_start[seg_of(p, j0)];   // earlier queries see none of these keys
  const int n_qt = (p.n - q_begin + BN - 1) / BN;
  const bool wg_video = all_video(p, j0, j1);
  const int wg_kseg_last = seg_of(p, j1 - 1);

  const int krow = j0 + 32 * kg + lr;
  const bool kok = krow < p.n;
  int klo, khi;
  key_range(p, krow, klo, khi);

  const uint16_t* qb = p.q + (int64_t)head * p.q_sh;
  const uint16_t* db_ = p.dout + (int64_t)head * p.do_sh;
  char* const kv = smem;                      // K rows at 0, V rows at KBN * 256
  char* const stage = smem + KV_BYTES;
  f32x16 dkacc[4], dvacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }
  const float c = p.scale_log2;

  // per-query tables of a tile: lse (log2 units; +inf past the end), delta,
  // segment (sg: the segment of the tile's first row)
  auto finish = [&](int q0, char* buf, int sg) {
    dload_wait();
    if (tid < BN) {
      const int r = q0 + tid;
      const bool ok = r < p.n;
      float* tb = (float*)(buf + TOFF);
      tb[tid] = ok ? p.lse[(int64_t)head * p.n + r] * kLog2e : INFINITY;
      tb[BN + tid] = ok ? p.delta[(int64_t)head * p.n + r] : 0.0f;
      ((int*)tb)[2 * BN + tid] = row_segment(p, sg, q0, BN, r);
    }
  };
  // The next tile's lse and delta are fetched during an iteration, into
  // registers of the lanes that write the table, and stored at its end: a
  // fetch at the end would hold every wave at the barrier for a memory round
  // trip.
  float nl = 0.0f, nd = 0.0f;
  auto fetch_next = [&](int q0) {
    if (tid < BN) {
      const int r = min(q0 + tid, p.n - 1);
      nl = p.lse[(int64_t)head * p.n + r];
      nd = p.delta[(int64_t)head * p.n + r];
    }
  };
  auto finish_next = [&](int q0, char* buf, int sg) {
    dload_wait();
    if (tid < BN) {
      const int r = q0 + tid;
      const bool ok = r < p.n;
      float* tb = (float*)(buf + TOFF);
      tb[tid] = ok ? nl * kLog2e : INFINITY;
      tb[BN + tid] = ok ? nd : 0.0f;
      ((int*)tb)[2 * BN + tid] = row_segment(p, sg, q0, BN, r);
    }
  };
  // the tile needs the mask unless every key here is video of a segment no
  // later than every query in it
  SegWalk qw;
  qw.init(p, q_begin);
  auto tile_masked = [&](int qs) { return p.needs_mask && !(wg_video && wg_kseg_last <= qs); };
  bool masked = tile_masked(qw.s);
  stage_pair<KBN / KW>(p.k + (int64_t)head * p.k_sh, p.k_st, p.v + (int64_t)head * p.v_sh, p.v_st, j0, j1 - j0,
                       w, lane, kv, kv + KBN * 256);
  stage_pair<BN / KW>(qb, p.q_st, db_, p.do_st, q_begin, min(BN, p.n - q_begin), w, lane, stage + AOFF,
                      stage + BOFF);
  finish(q_begin, stage, qw.s);
  __syncthreads();
  const char* const ktile_l = kv + (32 * kg) * 256;
  const char* const vtile_l = kv + (KBN + 32 * kg) * 256;
  for (int t = 0; t < n_qt; ++t) {
    char* const cur = stage + (t & 1) * BUF_BYTES;
    char* const nxt = stage + ((t + 1) & 1) * BUF_BYTES;
    const bool has_next = t + 1 < n_qt;
    const int q0 = q_begin + t * BN;
    // S = Q K^T and dP = dO V^T over this wave's 32 queries and 32 keys:
    // queries in the accumulator rows, keys across lanes
    f32x16 s = f32x16{}, dp = f32x16{};
    const char* qa = cur + AOFF;
    const char* da = cur + BOFF;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 aq = *(const bf16x8*)(qa + t_off(32 * qh + lr, 2 * dt + hh));
      const bf16x8 bk = *(const bf16x8*)(ktile_l + t_off(lr, 2 * dt + hh));
      const bf16x8 ad = *(const bf16x8*)(da + t_off(32 * qh + lr, 2 * dt + hh));
      const bf16x8 bv = *(const bf16x8*)(vtile_l + t_off(lr, 2 * dt + hh));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bv, dp, 0, 0, 0);
      // the next tile's loads go out after six of the eight steps: their
      // writes into LDS then land after the products' operand reads, which
      // keep the LDS busy (issued at the start of the iteration they
      // measured 7 % slower)
      if (dt == 5 && has_next) {
        stage_pair<BN / KW>(qb, p.q_st, db_, p.do_st, q0 + BN, min(BN, p.n - q0 - BN), w, lane, nxt + AOFF,
                            nxt + BOFF);
        fetch_next(q0 + BN);
      }
    }
    const float* tb = (const float*)(cur + TOFF);
    f32x16 pm, ds;
    // exponent arguments; a tile that needs the mask sends invisible pairs to -inf
    float arg[16];
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const f32x4 l4 = *(const f32x4*)(tb + 32 * qh + 8 * jq + 4 * hh);   // tile rows r .. r + 3
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) arg[4 * jq + jj] = fmaf(s[4 * jq + jj], c, -l4[jj]);
    }
    if (masked) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const i32x4 g4 = *(const i32x4*)((const int*)tb + 2 * BN + 32 * qh + 8 * jq + 4 * hh);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (g4[jj] < klo || g4[jj] > khi) arg[4 * jq + jj] = -INFINITY;
      }
    }
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const f32x4 d4 = *(const f32x4*)(tb + BN + 32 * qh + 8 * jq + 4 * hh);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pr = __builtin_amdgcn_exp2f(arg[4 * jq + jj]);
        pm[4 * jq + jj] = pr;
        ds[4 * jq + jj] = pr * (dp[4 * jq + jj] - d4[jj]);
      }
    }
    u32x4 pkp[2], pkd[2];
#pragma unroll
    for (int ck = 0; ck < 2; ++ck) {
      uint32_t wp[4], wd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wp[e] = pack_bf16(pm[8 * ck + 2 * e], pm[8 * ck + 2 * e + 1]);
        wd[e] = pack_bf16(ds[8 * ck + 2 * e], ds[8 * ck + 2 * e + 1]);
      }
      pkp[ck] = u32x4{wp[0], wp[1], wp[2], wp[3]};
      pkd[ck] = u32x4{wd[0], wd[1], wd[2], wd[3]};
    }
    tileT_x_packed32(da, 32 * qh, pkp, lane, hh, dvacc);   // dV^T += dO^T P
    tileT_x_packed32(qa, 32 * qh, pkd, lane, hh, dkacc);   // dK^T += Q^T dS
    bool masked_next = false;
    if (has_next) {
      const int qs = qw.at(p, q0 + BN);
      masked_next = tile_masked(qs);
      finish_next(q0 + BN, nxt, qs);
    }
    __syncthreads();
    masked = masked_next;
  }
  // pair reduction: the second-half wave hands over its dV, the first-half
  // wave its dK; each then finishes one of the two
  float* const red = (float*)(smem + kg * 32768);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) red[(db * 16 + j) * 64 + lane] = dvacc[db][j];
  } else {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) red[4096 + (db * 16 + j) * 64 + lane] = dkacc[db][j];
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) dvacc[db][j] += red[(db * 16 + j) * 64 + lane];
    if (kok) store_row(p.dv + (int64_t)krow * p.dv_st + (int64_t)head * p.dv_sh, hh, dvacc, 1.0f);
  } else {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) dkacc[db][j] += red[4096 + (db * 16 + j) * 64 + lane];
    if (kok) store_row(p.dk + (int64_t)krow * p.dk_st + (int64_t)head * p.dk_sh, hh, dkacc, p.sm_scale);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdParams& p0, hipStream_t s) {
  AttnBwdParams p = p0;
  const unsigned drows = (unsigned)((p.n + kDeltaRows - 1) / kDeltaRows);
  hipLaunchKernelGGL(delta_kernel, dim3(drows, (unsigned)p.n_heads), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)dq_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)dkdv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, KLDS_BYTES);
  if (e != hipSuccess) return e;
  const int64_t nq = (int64_t)((p.n + QBM - 1) / QBM) * p.n_heads;
  hipLaunchKernelGGL(dq_kernel, dim3((unsigned)nq), dim3(QT), LDS_BYTES, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nk = (int64_t)((p.n + KBN - 1) / KBN) * p.n_heads;
  hipLaunchKernelGGL(dkdv_kernel, dim3((unsigned)nk), dim3(KT), KLDS_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace segc
