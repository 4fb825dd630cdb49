// Segment-wise causal joint attention over a KV cache plus the current
// segment(s), on gfx950 bf16 MFMA.
//
// Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
// "Segment-Autoregressive Diffusion Transformer" (one joint attention over
// text and video, causal across segments, with the layer's cache holding the
// earlier segments) and section
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
//  * key tiles of 64 rows are staged through LDS by direct global->LDS
//    loads (no staging registers); waves 0-3 stage, so each SIMD hosts one
//    staging wave and one compute-only wave. Two schedules:
//    - bf16 keys (a BF16 cache, or no history): two tiles per barrier,
//      double buffered -- while tiles 2u and 2u+1 are computed from two
//      tile slots, the loads of tiles 2u+2 and 2u+3 land in the other two
//      (one barrier, one wait and one round of staging bookkeeping per 128
//      keys); the loop body exists once per slot pair, so every operand
//      read takes its slot as an immediate offset; the loads are issued
//      inside the iteration, not at its start, and history groups are
//      found by a running (frame, row) position rather than a division and
//      a slot lookup per tile;
//    - an INT8 history: one tile per barrier, three tile buffers, loads two
//      tiles ahead, and two staging areas for the codes and scales (the
//      128-key buffers and the INT8 staging would not fit the 160 KB LDS);
//    the loads are issued from inline assembly and awaited explicitly, once
//    per barrier, because the compiler, unable to tell the LDS buffers
//    apart, would otherwise drain them before every operand read of another
//    buffer; all slot lookups precede the loads of a tile (a wait for a
//    lookup would drain them too);
//  * tiles are row-major with XOR-swizzled 16-byte chunks, chosen for the
//    gfx950 LDS (16 lanes of a 16-byte read per cycle over 64 banks) so that
//    every operand read is conflict-free and every load instruction moves 4
//    whole rows;
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: keys land in accumulator
//    registers and queries across lanes, so a row max needs only one
//    cross-half exchange (v_permlane32_swap); O^T = V^T P^T takes the S^T
//    accumulators as the P operand directly, and its V^T operand comes from
//    the row-major V tile through the transposing LDS read (ds_read_b64_tr_b16);
//    the QK^T MFMAs run as two interleaved accumulation chains (the two key
//    blocks) with their operand reads scheduled 4 MFMAs ahead;
//  * each staging wave loads a 16-row group of a tile: with frames of a
//    multiple of 16 tokens a group never straddles a frame, so its base
//    address is wave-uniform (SGPRs) and a whole group is loaded in the
//    scalar-base form with loop-invariant 32-bit lane offsets: the staging
//    waves wait at every barrier for each other, so their per-tile address
//    work is on the critical path; rows past the end are clamped to the last
//    valid row (finite data) and masked;
//  * INT8 history rows (codes and scales) are direct-loaded into one of two
//    staging areas and dequantised to bf16(code * scale) into the tile by the
//    wave that loaded them, so the MFMA path is the same for both cache types;
//  * online softmax in base 2 against a per-row reference max that moves
//    only when needed: a tile's exponentials are taken against the current
//    reference, rounded to bf16 as the PV operand and summed from those
//    rounded values (dot products of the packed pairs with (1, 1)), so the
//    row sum weighs every value exactly as the products do; only when that
//    per-lane sum exceeds 2^12 (so some exponential might, or has
//    overflowed) or the row has seen no visible key yet does the wave form
//    the logits again, take the true tile max, rescale O and l and redo the
//    exponentials. No per-tile max reduction remains on the common path,
//    and the result is exact: the final division uses the same reference;
//  * masks are per tile: only tiles at a ragged end, or with text rows, or
//    with video of a segment later than the workgroup's first query evaluate
//    a per-element predicate from a 64-entry key table in LDS; keys of later
//    segments than the workgroup's last query are never loaded;
//  * workgroup ids are remapped so that each XCD (dispatched round-robin)
//    works through contiguous query tiles of the same head, sharing K/V in L2.
#include "internal.h"
#include "lds_dma.h"
#include "segtab.h"

namespace segc {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                 // keys per tile
constexpr int NSTAGE = 4;              // waves that stage tiles
constexpr int RW = BN / NSTAGE;        // tile rows staged per wave (a "group")
constexpr int NW = 8;                  // waves per workgroup: 0-3 stage and compute, 4-7 compute
constexpr int NT = NW * 64;
constexpr int BM = 32 * NW;            // query rows per workgroup
constexpr int TILE_BYTES = BN * D * 2;           // one 64 x 128 bf16 tile
constexpr int INFO_BYTES = BN * 4;               // per-key visibility table
constexpr int KOFF = 0, VOFF = TILE_BYTES, IOFF = 2 * TILE_BYTES;
constexpr int BUF_BYTES = 2 * TILE_BYTES + INFO_BYTES;
constexpr int NBUF = 3;                          // tiles t, t+1 and t+2 are live at once
constexpr int RAW0 = NBUF * BUF_BYTES;           // two INT8 staging areas: codes, then scales
constexpr int RAW_KC = 0, RAW_VC = BN * D, RAW_S = 2 * BN * D;
constexpr int RAW_BYTES = 2 * BN * D + NSTAGE * 256;   // codes + one 64-float scale block per wave
constexpr int LDS_BYTES = RAW0 + 2 * RAW_BYTES;
// two-tile schedule (bf16 keys only): four tile slots (0 and 1 are computed
// while 2 and 3 land, then the reverse); all K tiles lie in the first 64 KB
// and all V tiles in the next, so that every operand read of any slot is a
// per-lane base plus an immediate offset below 64 KB; then the four key tables
constexpr int PK_OFF = 0, PV_OFF = 4 * TILE_BYTES, PI_OFF = 8 * TILE_BYTES;
constexpr int LDS_PAIR_BYTES = PI_OFF + 4 * INFO_BYTES;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

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

// Mask state of the tiles, decided once per tile in ascending order: a tile
// needs the per-element mask at a ragged end, or when it holds current rows
// other than video of segments no later than the workgroup's first query
// segment (segments ascend with rows, so every query of the workgroup sees
// those). `kseg` tracks the segment of each current tile's first row for the
// key table.
struct MaskWalk {
  FreeRuns free;
  SegWalk kseg;
  int qseg_first;
};

// kSeg = false: one unpadded segment (no per-element mask but at a ragged
// end); the walk is compiled out, which keeps the loop's scalar state small.
template <bool kSeg>
__device__ inline bool tile_masked(const AttnParams& p, const Tile& tl, MaskWalk& mw) {
  if constexpr (!kSeg) {
    return tl.nvalid < BN;
  } else {
    if (!tl.hist) mw.kseg.at(p, tl.j0);
    if (tl.nvalid < BN) return true;
    if (tl.hist) return false;
    return !mw.free.free(p, BN, mw.qseg_first, tl.j0 / BN);
  }
}

// Where a staging wave's group of RW consecutive tile rows lives. Uniform
// fields describe the group's first row; lanes add row offsets (clamped to
// `lim`). With frames of a multiple of RW tokens a group never straddles a
// frame, so one slot lookup serves the whole group.
// The slot list is not written while the kernel runs: reading it through the
// constant address space lets a wave-uniform lookup be a scalar load.
__device__ inline int const_load(const int* p) {
  return *(const __attribute__((address_space(4))) int*)p;
}

struct Group {
  int64_t row0;   // history: cache row index of the group's first row; current: row index
  int lim;        // largest valid local row
  bool generic;   // history frames not a multiple of RW tokens: per-lane rows
  int j;          // first tile row of the group (generic path)
};

__device__ inline Group group_at(const AttnParams& p, const Tile& tl, int w, int head) {
  Group g;
  const int last = tl.j0 + tl.nvalid - 1;            // last valid row of the tile
  const int gs = min(tl.j0 + RW * w, last & ~(RW - 1));
  g.lim = last - gs;
  g.generic = false;
  g.j = gs;
  if (tl.hist) {
    if (p.G % RW == 0) {
      const int f = gs / p.G;
      const int slot = const_load(p.hist_slots + f);
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

// Tile layouts: 64 rows of 256 bytes (row-major, so a direct-load
// instruction fills 4 whole rows and reads them coalesced), with the 16-byte
// chunks of each row XOR-swizzled. On gfx950 the LDS serves 16 lanes of a
// 16-byte read (32 lanes of an 8-byte read) per cycle from 64 four-byte
// banks; the swizzles make every operand read conflict-free:
//  * K: chunk c of row r at c ^ (r & 15); an MFMA operand read takes one
//    chunk of 16 consecutive rows per 16 lanes -> 16 distinct bank groups;
//  * V: chunk c of row r at c ^ 5 (r & 3); a 32-lane window of the
//    transposing read takes 4 adjacent chunks (an aligned group of 4) of 4
//    consecutive rows, which the high term 4 (r & 3) sends to 4 distinct
//    groups -> 256 distinct bytes; the low term (r & 3) makes the INT8
//    dequantisation stores conflict-free too (16 lanes store chunks
//    4 q + e, q = 0..3, of 4 consecutive rows: distinct low bits per row).
__device__ inline int k_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ inline int v_off(int r, int c) { return r * 256 + ((c ^ (5 * (r & 3))) << 4); }

// Issue the loads of staging wave w's group of tile tl: bf16 rows go
// straight into the K/V tiles of `buf`; INT8 history rows go into `raw`
// (codes, plus the group's K and V scales) for stage_finish to convert.
// kInt8 = false compiles the INT8 branch out (the pair schedule never sees
// INT8 rows).
template <bool kInt8 = true>
__device__ inline int stage_issue(const AttnParams& p, const Tile& tl, int w, int lane, int head,
                                  char* kt, char* vt, char* raw) {
  const Group g = group_at(p, tl, w, head);
  if (!kInt8 || !tl.hist || !p.hist_int8) {
    if (g.lim >= RW - 1 && !g.generic) {
      // a whole group (no clamping) of consecutive rows of one frame or of the
      // current rows: a uniform base per tensor, and per-lane offsets that only
      // depend on the lane and the row pitch (4 rows per instruction; group row
      // r = 4 e + lane / 16 is also the tile row modulo 16, which sets the swizzle)
      uint64_t kb, vb;
      uint32_t ks, vs;
      if (tl.hist) {
        kb = uniform_addr((const char*)p.hk + g.row0 * 256);
        vb = uniform_addr((const char*)p.hv + g.row0 * 256);
        ks = vs = 256;
      } else {
        kb = uniform_addr(p.k + g.row0 * p.k_st + head * p.k_sh);
        vb = uniform_addr(p.v + g.row0 * p.v_st + head * p.v_sh);
        ks = (uint32_t)p.k_st * 2;
        vs = (uint32_t)p.v_st * 2;
      }
      const uint32_t lrow = lane >> 4, pc = lane & 15;
#pragma unroll
      for (int e = 0; e < RW / 4; ++e) {
        const uint32_t r = 4 * e + lrow;
        const int dst = (RW * w + 4 * e) * 256;
        dload16_s(r * ks + ((pc ^ r) << 4), kb, kt + dst);
        dload16_s(r * vs + ((pc ^ (5 * (lrow & 3))) << 4), vb, vt + dst);
      }
      return 2 * (RW / 4);
    }
    // all addresses first: a per-lane slot lookup (generic path) is an
    // ordinary load, and waiting for it would also drain earlier direct loads
    const char *krow[RW / 4], *vrow[RW / 4];
#pragma unroll
    for (int e = 0; e < RW / 4; ++e) {                     // 4 whole rows per instruction
      const int lr = min(4 * e + (lane >> 4), g.lim);      // group-local row (clamped)
      if (!tl.hist) {
        krow[e] = (const char*)(p.k + g.row0 * p.k_st + head * p.k_sh) + (uint32_t)(lr * (int)p.k_st * 2);
        vrow[e] = (const char*)(p.v + g.row0 * p.v_st + head * p.v_sh) + (uint32_t)(lr * (int)p.v_st * 2);
      } else if (!g.generic) {
        krow[e] = (const char*)p.hk + g.row0 * 256 + (uint32_t)(lr * 256);
        vrow[e] = (const char*)p.hv + g.row0 * 256 + (uint32_t)(lr * 256);
      } else {
        const int64_t cr = hist_row_generic(p, g, lr, head);
        krow[e] = (const char*)p.hk + cr * 256;
        vrow[e] = (const char*)p.hv + cr * 256;
      }
    }
#pragma unroll
    for (int e = 0; e < RW / 4; ++e) {
      const int row = RW * w + 4 * e + (lane >> 4);        // tile row of this lane's slot
      const int pc = lane & 15;                            // physical chunk in the LDS row
      const int dst = (RW * w + 4 * e) * 256;
      dload16(krow[e] + ((pc ^ (row & 15)) << 4), kt + dst);
      dload16(vrow[e] + ((pc ^ (5 * (row & 3))) << 4), vt + dst);
    }
    return 2 * (RW / 4);
  } else {
    int64_t cr[RW / 8];
#pragma unroll
    for (int e = 0; e < RW / 8; ++e) {
      const int lr = min(8 * e + (lane >> 3), g.lim);
      cr[e] = g.generic ? hist_row_generic(p, g, lr, head) : g.row0 + lr;
    }
    // scales: lanes [0, RW) K of the group's rows, [RW, 2 RW) V, the rest repeat
    const int slr = min(lane & (RW - 1), g.lim);
    const int64_t scr = g.generic ? hist_row_generic(p, g, slr, head) : g.row0 + slr;
    const uint64_t sbase = (lane & RW) ? uniform_addr(p.hvs) : uniform_addr(p.hks);
#pragma unroll
    for (int e = 0; e < RW / 8; ++e) {                     // 8 rows of codes per instruction
      const int off = (lane & 7) * 16;
      dload16((const char*)p.hk + cr[e] * 128 + off, raw + RAW_KC + (RW * w + 8 * e) * 128);
      dload16((const char*)p.hv + cr[e] * 128 + off, raw + RAW_VC + (RW * w + 8 * e) * 128);
    }
    dload4((const void*)(sbase + (uint64_t)scr * 4), raw + RAW_S + w * 256);
    return 2 * (RW / 8) + 1;
  }
}

// A whole history group (RW rows of one frame, 256-byte rows) from the
// group's first cache row: the per-lane offsets depend only on the lane.
__device__ inline void stage_hist_group(const AttnParams& p, int64_t row0, int w, int lane, char* kt, char* vt) {
  const uint64_t kb = uniform_addr((const char*)p.hk + row0 * 256);
  const uint64_t vb = uniform_addr((const char*)p.hv + row0 * 256);
  const uint32_t lrow = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int e = 0; e < RW / 4; ++e) {
    const uint32_t r = 4 * e + lrow;
    const int dst = (RW * w + 4 * e) * 256;
    dload16_s(r * 256 + ((pc ^ r) << 4), kb, kt + dst);
    dload16_s(r * 256 + ((pc ^ (5 * (lrow & 3))) << 4), vb, vt + dst);
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

template <bool IS_V>
__device__ inline void convert_group(const char* codes, const float* scales, char* tile, int w,
                                     int lane) {
  const int row = RW * w + (lane >> 2), q = lane & 3;
  const float sc = scales[lane >> 2];
  const u32x4 c0 = *(const u32x4*)(codes + row * 128 + 32 * q);
  const u32x4 c1 = *(const u32x4*)(codes + row * 128 + 32 * q + 16);
  float f[32];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dequant4(c0[e], sc, f + 4 * e);
    dequant4(c1[e], sc, f + 16 + 4 * e);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t wd[4];                      // plain array first, vector in one piece
#pragma unroll
    for (int k = 0; k < 4; ++k) wd[k] = pack_bf16(f[8 * e + 2 * k], f[8 * e + 2 * k + 1]);
    const u32x4 o = {wd[0], wd[1], wd[2], wd[3]};
    const int cc = 4 * q + e;
    *(u32x4*)(tile + (IS_V ? v_off(row, cc) : k_off(row, cc))) = o;
  }
}

// Visibility table of the tile's 64 keys: [lo, hi] range of query segments
// that may see the key (lo > hi: nobody).
template <bool kSeg>
__device__ inline void store_info(const AttnParams& p, const Tile& tl, int tid, int* info, int sg) {
  if (tid >= BN) return;
  int v;
  if (!kSeg || tl.hist)
    v = (tid < tl.nvalid) ? (0xFFFF << 16) : 0xFFFF;
  else
    v = key_visibility(p, sg, tl.j0, BN, tl.j0 + tid, tid < tl.nvalid);
  info[tid] = v;
}

// S^T (64 keys x 32 queries) = K Q^T from the K tile in LDS: the two key
// blocks form two independent accumulation chains, interleaved, with the
// operand reads kept 4 MFMAs ahead of their use.
__device__ inline void qk_tile(const char* kbuf, const bf16x8 (&qf)[8], int lr, int hh,
                               f32x16 (&s)[2]) {
  bf16x8 a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = *(const bf16x8*)(kbuf + k_off(32 * (i & 1) + lr, 2 * (i >> 1) + hh));
  s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], qf[0], f32x16{}, 0, 0, 0);
  s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
  for (int dt = 1; dt < 8; ++dt) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * dt], qf[dt], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2 * dt + 1], qf[dt], s[1], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

struct RowState {
  float m, l;
};

// Exponentials of one tile, in place (s becomes p), against the row's
// reference max m, and their per-lane sum ls. The reference moves only when
// the tile's exponentials would outgrow kPLimit (their per-lane sum says so:
// every term is at most the sum; an infinite or NaN sum fails the test too)
// or while the row has seen no visible key; then the logits are formed again
// from the K tile (still in LDS), the true tile max is taken, O and l are
// rescaled and the exponentials recomputed. Any reference no larger than the
// row max gives the same softmax: the final division uses the same reference.
constexpr float kPLimit = 0x1p12f;

// Exponentials of one tile, packed to bf16 in the PV operand order (word
// 4 ck + e of chunk ck holds accumulator values 8 (ck & 1) + 2 e and + 1 of
// block ck >> 1), and their per-lane sum, taken from the packed values with
// dot products against (1, 1) so that the row sum uses the same rounded
// weights as the products.
__device__ inline float exp_pack_sum(const f32x16 (&s)[2], float c, float mc, uint32_t (&pw)[16]) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int ck = 0; ck < 4; ++ck)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 8 * (ck & 1) + 2 * e;
      const float x0 = __builtin_amdgcn_exp2f(fmaf(s[ck >> 1][j], c, -mc));
      const float x1 = __builtin_amdgcn_exp2f(fmaf(s[ck >> 1][j + 1], c, -mc));
      pw[4 * ck + e] = pack_bf16(x0, x1);
    }
  float acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[e]), ones, 0.0f, false);
#pragma unroll
    for (int ck = 1; ck < 4; ++ck)
      acc[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[4 * ck + e]), ones, acc[e], false);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

__device__ inline void mask_tile(f32x16 (&s)[2], const int* info, int qseg, int hh) {
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

__device__ inline void softmax_tile(f32x16 (&s)[2], bool masked, const int* info, int qseg, int hh,
                                    float c, RowState& rs, f32x16 (&o)[4], float& ls,
                                    const char* kbuf, const bf16x8 (&qf)[8], int lr, uint32_t (&pw)[16]) {
  if (masked) mask_tile(s, info, qseg, hh);
  ls = exp_pack_sum(s, c, (rs.m == -INFINITY) ? 0.0f : rs.m * c, pw);
  const bool need = !(ls <= kPLimit) || rs.m == -INFINITY;
  if (__builtin_amdgcn_ballot_w64(need)) {
    qk_tile(kbuf, qf, lr, hh, s);
    if (masked) mask_tile(s, info, qseg, hh);
    float m1[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a = 3 * i, b = 3 * i + 1, e = 3 * i + 2;
      m1[i] = fmaxf(fmaxf(s[a >> 4][a & 15], s[b >> 4][b & 15]), s[e >> 4][e & 15]);
    }
    m1[10] = fmaxf(s[1][14], s[1][15]);
    const float m2a = fmaxf(fmaxf(m1[0], m1[1]), m1[2]), m2b = fmaxf(fmaxf(m1[3], m1[4]), m1[5]);
    const float m2c = fmaxf(fmaxf(m1[6], m1[7]), m1[8]), m2d = fmaxf(m1[9], m1[10]);
    float mx = fmaxf(fmaxf(m2a, m2b), fmaxf(m2c, m2d));
    mx = xhalf_max(mx);
    const float mnew = fmaxf(rs.m, mx);
    // a row that has seen no visible key yet keeps m = -inf: its factor is 1
    // (exp2 of -inf - -inf would be NaN and poison O and l for good)
    const float alpha = (mnew == rs.m) ? 1.0f : __builtin_amdgcn_exp2f((rs.m - mnew) * c);
    rs.m = mnew;
    rs.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
    ls = exp_pack_sum(s, c, (rs.m == -INFINITY) ? 0.0f : rs.m * c, pw);
  }
}

// O^T += V^T P^T for one tile (p from s, rounded to bf16 as the operand).
// The V^T operand comes from the row-major V tile through the transposing
// LDS read: inside each 16-lane group, lane j addresses 4 elements of row
// base + j/4 at column d0 + 4 (j % 4); lane i then receives rows base..base+3
// at column d0 + i, i.e. 4 keys of its own d. Two reads give the 8 keys the
// P operand holds in this lane half (rows 16 ck + 4 hh + 0..3 and + 8..11).
__device__ inline void pv_tile(const char* vbuf, const uint32_t (&pw)[16], int lane, int hh,
                               f32x16 (&o)[4]) {
  // lane i of 16-lane group g reads row 16 ck + 4 hh + i / 4 and the row 8
  // further down, column 32 db + 16 (g & 1) + 4 (i % 4): chunk 4 db + hb with
  // hb = 2 (g & 1) + (i % 4) / 2, byte 8 (i & 1).
  const int gi = lane & 15;
  const int hb = ((gi & 3) >> 1) | (((lane >> 4) & 1) << 1);
  const int r0 = 4 * hh + (gi >> 2);
  const int sub = 8 * (gi & 1);
#pragma unroll
  for (int ck = 0; ck < 4; ++ck) {
    // the four packed pairs go into a plain array first and into the vector
    // in one piece (writing vector elements one by one inside unrolled loops
    // has been seen to lose some of them in this compiler's output)
    const u32x4 u = {pw[4 * ck], pw[4 * ck + 1], pw[4 * ck + 2], pw[4 * ck + 3]};
    const bf16x8 pb = as_bf16x8(u);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vbuf + v_off(16 * ck + r0, 4 * db + hb) + sub));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vbuf + v_off(16 * ck + r0 + 8, 4 * db + hb) + sub));
      const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb, o[db], 0, 0, 0);
    }
  }
  // V^T reads two products ahead of their use
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// Finish staging wave w's group of tile tl: wait for its direct loads, turn
// INT8 rows into bf16 (each wave converts exactly the rows it loaded), and
// (wave 0) write the tile's key table when the tile needs a mask.
template <bool kSeg>
__device__ inline void stage_finish(const AttnParams& p, const Tile& tl, int w, int lane, int tid,
                                    char* buf, const char* raw, int newer, bool masked, int sg) {
  // the direct loads are invisible to the compiler: wait in asm with a memory
  // clobber so that no read of the landed data is scheduled above the wait.
  // Loads complete in order: leaving the `newer` most recent ones (the next
  // tile's) in flight still waits for every load of this tile.
  if (newer == 2 * (RW / 4))
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * (RW / 4)) : "memory");
  else if (newer == 2 * (RW / 8) + 1)
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * (RW / 8) + 1) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tl.hist && p.hist_int8) {
    const float* sk = (const float*)(raw + RAW_S + w * 256);   // K scales of the group's rows
    convert_group<false>(raw + RAW_KC, sk, buf + KOFF, w, lane);
    convert_group<true>(raw + RAW_VC, sk + RW, buf + VOFF, w, lane);
  }
  if (masked) store_info<kSeg>(p, tl, tid, (int*)(buf + IOFF), sg);
}

template <bool kSeg, bool kPair>
__global__ __launch_bounds__(NT, 2) void attn_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // Workgroups [0, n_full) take whole (head, query tile)s, remapped XCD-aware:
  // hardware deals workgroup b to XCD b % 8; each XCD gets a contiguous range
  // in head-major order. Later workgroups (split > 1) take key range `part`
  // of one of the remaining tiles.
  const int b = blockIdx.x;
  int logical, part = -1;
  if (kSeg || !kPair || b < p.n_full) {     // only the single-segment two-tile kernel splits
    const int nwg = p.n_full;
    const int xcd = b & 7, local = b >> 3;
    const int qn = nwg >> 3, rn = nwg & 7;
    logical = (xcd < rn) ? xcd * (qn + 1) + local : rn * (qn + 1) + (xcd - rn) * qn + local;
  } else {
    // range-major: the split workgroups in flight together (and those dealt to
    // one XCD) cover few key ranges, so they share K/V in L2
    const int rest = p.n_qtiles * p.n_heads - p.n_full;
    const int idx = b - p.n_full;
    part = idx / rest;
    logical = p.n_full + (idx - part * rest);
  }
  const int head = logical / p.n_qtiles;
  const int qtile = logical - head * p.n_qtiles;

  const int m0 = qtile * BM;
  const int wg_last = min(m0 + BM, p.n_cur) - 1;
  const int cur_end = p.seg_start[seg_of(p, wg_last) + 1];   // later keys are future for all
  MaskWalk mw;
  if constexpr (kSeg) {
    mw.qseg_first = seg_of(p, m0);
    mw.free.init(p, BN, mw.qseg_first);
    mw.kseg.init(p, 0);
  } else {
    mw.kseg.s = 0;
  }
  const int n_tiles = p.hist_tiles + (cur_end + BN - 1) / BN;
  // key tiles [tb, te) of this workgroup (a split covers one key range)
  int tb = 0, te = n_tiles;
  if (!kSeg && kPair && part >= 0) {
    tb = (int)((int64_t)part * n_tiles / p.split);
    te = (int)((int64_t)(part + 1) * n_tiles / p.split);
  }

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
  // Settle the Q loads here: a wait for them left inside the loop would also
  // drain the direct loads in flight there.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  RowState rs = {-INFINITY, 0.0f};
  const float c = p.scale_log2;

  const bool stager = w < NSTAGE;
  if constexpr (kPair) {
    // Two tiles per barrier, double buffered: during iteration u every wave
    // computes tiles 2u and 2u+1 from slots 2 (u % 2) and + 1 while the
    // staging waves' direct loads for tiles 2u+2 and 2u+3 land in the other
    // two slots; at the end of the iteration the staging waves wait for those
    // loads and write the key tables of tiles that need a mask. The mask walk
    // visits the tiles in ascending order, once each.
    //
    // One tile: S^T, softmax, O^T += V^T P^T; `mid` runs between the S^T
    // products and the softmax.
    auto half = [&](int slot, bool masked, auto&& mid) __attribute__((always_inline)) {
      const char* kb = smem + PK_OFF + slot * TILE_BYTES;
      const int* info = (const int*)(smem + PI_OFF + slot * INFO_BYTES);
      f32x16 sc[2];
      qk_tile(kb, qf, lr, hh, sc);
      mid();
      float ls;
      uint32_t pw[16];
      softmax_tile(sc, masked, info, qseg, hh, c, rs, o, ls, kb, qf, lr, pw);
      rs.l += ls;
      pv_tile(smem + PV_OFF + slot * TILE_BYTES, pw, lane, hh, o);
    };
    // Staging waves walk the history in whole tiles with a running position
    // of their group (frame hf, row hoff inside it, its cache slot hslot), so
    // the slot list is read once per frame rather than once per tile. Tiles
    // are issued in ascending order. Frames of a multiple of RW tokens only
    // (a group then never straddles a frame); other tiles take the general path.
    const bool hwalk = p.G % RW == 0;
    const int full_hist_tiles = p.n_hist_rows / BN;
    int hf = 0, hoff = 0, hslot = 0;
    if (stager && hwalk && tb < full_hist_tiles) {
      const int g0 = BN * tb + RW * w;
      hf = g0 / p.G;
      hoff = g0 - hf * p.G;
      hslot = const_load(p.hist_slots + hf);
    }
    auto issue = [&](int t, int slot) __attribute__((always_inline)) {
      char* const kt = smem + PK_OFF + slot * TILE_BYTES;
      char* const vt = smem + PV_OFF + slot * TILE_BYTES;
      if (hwalk && t < full_hist_tiles) {
        stage_hist_group(p, ((int64_t)hslot * p.n_heads + head) * p.G + hoff, w, lane, kt, vt);
        hoff += BN;
        if (hoff >= p.G) {
          do { hoff -= p.G; ++hf; } while (hoff >= p.G);
          if (t + 1 < full_hist_tiles) hslot = const_load(p.hist_slots + hf);
        }
      } else {
        stage_issue<false>(p, tile_at(p, t, cur_end), w, lane, head, kt, vt, nullptr);
      }
    };
    auto info_at = [&](int slot) __attribute__((always_inline)) { return (int*)(smem + PI_OFF + slot * INFO_BYTES); };
    // (a split workgroup starts at tile tb > 0 only without segment structure,
    // whose mask walk is stateless)
    bool m0t = tile_masked<kSeg>(p, tile_at(p, tb, cur_end), mw);
    const int s0 = mw.kseg.s;
    bool m1t = tb + 1 < te && tile_masked<kSeg>(p, tile_at(p, tb + 1, cur_end), mw);
    const int s1 = mw.kseg.s;
    if (stager) {
      issue(tb, 0);
      if (tb + 1 < te) issue(tb + 1, 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (m0t) store_info<kSeg>(p, tile_at(p, tb, cur_end), tid, info_at(0), s0);
      if (m1t) store_info<kSeg>(p, tile_at(p, tb + 1, cur_end), tid, info_at(1), s1);
    }
    __syncthreads();
    const int n_pairs = (te - tb + 1) >> 1;
    // the loop body is instantiated once per slot parity, so that every LDS
    // operand address is a loop-invariant per-lane base plus an immediate
    auto pair_iter = [&](int u, int cs) __attribute__((always_inline)) {
      const int ns = 2 - cs;
      __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0) only
      const int t0 = tb + 2 * u;
      // The staging waves issue tile t0+2's loads after the first tile and
      // tile t0+3's between the second tile's S^T products and its softmax:
      // issued all at the start of the iteration (or right after the first
      // tile's S^T products) they held the staging waves back, and every
      // wave waits for those at the barrier.
      auto none = [&]() __attribute__((always_inline)) {};
      auto second = [&]() __attribute__((always_inline)) { if (stager && t0 + 3 < te) issue(t0 + 3, ns + 1); };
      half(cs, m0t, none);
      if (stager && t0 + 2 < te) issue(t0 + 2, ns);
      if (t0 + 1 < te) half(cs + 1, m1t, second);
      const bool n0 = t0 + 2 < te && tile_masked<kSeg>(p, tile_at(p, t0 + 2, cur_end), mw);
      const int sg0 = mw.kseg.s;
      const bool n1 = t0 + 3 < te && tile_masked<kSeg>(p, tile_at(p, t0 + 3, cur_end), mw);
      const int sg1 = mw.kseg.s;
      if (stager && t0 + 2 < te) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (n0) store_info<kSeg>(p, tile_at(p, t0 + 2, cur_end), tid, info_at(ns), sg0);
        if (n1) store_info<kSeg>(p, tile_at(p, t0 + 3, cur_end), tid, info_at(ns + 1), sg1);
      }
      __syncthreads();
      m0t = n0;
      m1t = n1;
    };
    for (int u = 0; u < n_pairs; u += 2) {
      pair_iter(u, 0);
      if (u + 1 < n_pairs) pair_iter(u + 1, 2);
    }
  } else {
    // One tile per barrier (an INT8 history), loads two tiles ahead: during
    // iteration t every wave computes tile t from LDS buffer t % 3 while the
    // staging waves' direct loads for tile t+2 land in buffer (t+2) % 3 (bf16)
    // or INT8 staging area t & 1; at the end of the iteration they wait for
    // tile t+1's loads (issued one iteration earlier) and dequantise it.
    char* const raw0 = smem + RAW0;
    char* const raw1 = smem + RAW0 + RAW_BYTES;
    // every wave walks the mask state (scalar work); the next tile's decision
    // is made after this tile's products are issued
    bool mt = tile_masked<kSeg>(p, tile_at(p, 0, cur_end), mw);
    if (stager) {
      const Tile t0 = tile_at(p, 0, cur_end);
      stage_issue(p, t0, w, lane, head, smem + KOFF, smem + VOFF, raw0);
      stage_finish<kSeg>(p, t0, w, lane, tid, smem, raw0, 0, mt, mw.kseg.s);
      if (n_tiles > 1) stage_issue(p, tile_at(p, 1, cur_end), w, lane, head, smem + BUF_BYTES + KOFF, smem + BUF_BYTES + VOFF, raw1);
    }
    __syncthreads();
    int bc = 0;
    for (int t = 0; t < n_tiles; ++t) {
      char* const cur = smem + bc * BUF_BYTES;
      char* const nx1 = smem + (bc == NBUF - 1 ? 0 : bc + 1) * BUF_BYTES;
      char* const nx2 = smem + (bc == 0 ? NBUF - 1 : bc - 1) * BUF_BYTES;
      const int* info = (const int*)(cur + IOFF);
      // nothing is outstanding here (the barrier drained LDS; scalar loads are
      // consumed where issued), but a scalar load hoisted before the loop would
      // otherwise make the compiler wait for every LDS read ahead of the first
      // product of each tile (scalar and LDS loads share a counter, and scalar
      // loads complete out of order)
      __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0) only
      int issued = 0;
      if (stager && t + 2 < n_tiles)
        issued = stage_issue(p, tile_at(p, t + 2, cur_end), w, lane, head, nx2 + KOFF, nx2 + VOFF, (t & 1) ? raw1 : raw0);
      f32x16 sc[2];
      qk_tile(cur + KOFF, qf, lr, hh, sc);
      float ls;
      uint32_t pw[16];
      softmax_tile(sc, mt, info, qseg, hh, c, rs, o, ls, cur + KOFF, qf, lr, pw);
      rs.l += ls;
      pv_tile(cur + VOFF, pw, lane, hh, o);
      const bool mt_next = t + 1 < n_tiles && tile_masked<kSeg>(p, tile_at(p, t + 1, cur_end), mw);
      if (stager && t + 1 < n_tiles)
        stage_finish<kSeg>(p, tile_at(p, t + 1, cur_end), w, lane, tid, nx1, (t & 1) ? raw0 : raw1, issued, mt_next,
                     mw.kseg.s);
      __syncthreads();
      mt = mt_next;
      bc = (bc == NBUF - 1) ? 0 : bc + 1;
    }
  }

  const float lt = xhalf_sum(rs.l);
  if (part >= 0) {
    // one key range of a split tile: unnormalised O, row max m and row sum l
    if (qok) {
      const int64_t rest = (int64_t)p.n_qtiles * p.n_heads - p.n_full;
      const int64_t row = ((int64_t)(logical - p.n_full) * p.split + part) * BM + 32 * w + lr;
      float* dst = p.ws + row * D + 4 * hh;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x4 v4 = {o[db][4 * jq], o[db][4 * jq + 1], o[db][4 * jq + 2], o[db][4 * jq + 3]};
          *(f32x4*)(dst + 32 * db + 8 * jq) = v4;
        }
      if (hh == 0) {
        float* ml = p.ws + rest * p.split * BM * D + row * 2;
        ml[0] = rs.m;
        ml[1] = lt;
      }
    }
    return;
  }
  // epilogue: O = acc / l, bf16; lse = m * sm_scale + ln l
  const float inv = 1.0f / lt;
  if (qok) {
    uint16_t* dst = p.o + (int64_t)qrow * p.o_st + head * p.o_sh + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x2 v2 = {pack_bf16(o[db][4 * jq] * inv, o[db][4 * jq + 1] * inv),
                          pack_bf16(o[db][4 * jq + 2] * inv, o[db][4 * jq + 3] * inv)};
        *(u32x2*)(dst + 32 * db + 8 * jq) = v2;
      }
    if (p.lse && hh == 0) p.lse[(int64_t)head * p.n_cur + qrow] = rs.m * p.sm_scale + logf(lt);
  }
}

// Merge the key ranges of the split tiles: for each row, M = max m_s,
// O = sum_s 2^((m_s - M) c) O_s / sum_s 2^((m_s - M) c) l_s, lse = M sm_scale +
// ln(that sum), as one workgroup would have produced (up to rounding order).
// 32 lanes per row, 4 columns each; 8 rows per workgroup.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int64_t rest = (int64_t)p.n_qtiles * p.n_heads - p.n_full;
  const int64_t rg = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);   // row among the split tiles
  const int r = (int)(rg / BM), rl = (int)(rg - (int64_t)r * BM);
  if (r >= rest) return;
  const int logical = p.n_full + r;
  const int head = logical / p.n_qtiles;
  const int qrow = (logical - head * p.n_qtiles) * BM + rl;
  if (qrow >= p.n_cur) return;
  const int c4 = 4 * (threadIdx.x & 31);
  const float* ml = p.ws + rest * p.split * BM * D;
  float mx = -INFINITY;
  for (int k = 0; k < p.split; ++k) mx = fmaxf(mx, ml[(((int64_t)r * p.split + k) * BM + rl) * 2]);
  float l = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < p.split; ++k) {
    const int64_t row = ((int64_t)r * p.split + k) * BM + rl;
    const float m = ml[row * 2];
    const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - mx) * p.scale_log2);
    l += f * ml[row * 2 + 1];
    const f32x4 v = *(const f32x4*)(p.ws + row * D + c4);
    acc += f * v;
  }
  const float inv = 1.0f / l;
  const u32x2 v2 = {pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  *(u32x2*)(p.o + (int64_t)qrow * p.o_st + head * p.o_sh + c4) = v2;
  if (p.lse && c4 == 0) p.lse[(int64_t)head * p.n_cur + qrow] = mx * p.sm_scale + logf(l);
}

}  // namespace

int64_t attn_split_plan(AttnParams& p, int n_cu) {
  p.n_qtiles = (p.n_cur + BM - 1) / BM;
  const int64_t nwg = (int64_t)p.n_qtiles * p.n_heads;
  p.n_full = (int32_t)nwg;
  p.split = 1;
  // only the two-tile kernel without segment structure splits: its tiles
  // are independent of where a key range starts
  const bool pair = !(p.hist_tiles > 0 && p.hist_int8);
  if (p.needs_mask || !pair || n_cu <= 0 || nwg < 1) return 0;
  const int64_t full = nwg / n_cu * n_cu, rest = nwg - full;
  // Only long launches split: measured on MI355X, a split of launches of one
  // or two rounds (c2, c3) cost more than it saved, and at c4 (15.6 rounds)
  // it saves about 1 %, well under the idle share of the last round (the
  // clock rises while part of the chip idles, which makes that round cheaper).
  if (rest == 0 || full < 4 * (int64_t)n_cu) return 0;
  const int n_tiles = p.hist_tiles + (p.n_cur + BN - 1) / BN;
  // Cost model: a workgroup takes about 1.7 us per 64-key tile; splitting the
  // last round into s ranges shortens it from one workgroup time to
  // ceil(rest s / n_cu) / s of one, and costs the partial results written and
  // read again (2 x 130 KiB per split workgroup at about 5 TB/s) plus one more
  // launch (about 10 us). At most 8 ranges per tile (16 measured no better).
  const double t_wg = 1.7 * n_tiles;
  double best_gain = 0.0;
  int best = 1;
  for (int sp = 2; sp <= 8 && 4 * sp <= n_tiles; ++sp) {
    const double last = (double)((rest * sp + n_cu - 1) / n_cu) / sp;
    const double gain = (1.0 - last) * t_wg - (double)rest * sp * 2.0 * BM * (D + 2) * 4 / 5.0e6 - 10.0;
    if (gain > best_gain) {
      best_gain = gain;
      best = sp;
    }
  }
  if (best == 1) return 0;
  p.n_full = (int32_t)full;
  p.split = best;
  return rest * best * (int64_t)BM * (D + 2) * 4;
}

hipError_t launch_attn(const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  p.n_qtiles = (p.n_cur + BM - 1) / BM;
  if (p.split <= 1) {
    p.split = 1;
    p.n_full = (int32_t)((int64_t)p.n_qtiles * p.n_heads);
  }
  const int64_t nwg = p.n_full + ((int64_t)p.n_qtiles * p.n_heads - p.n_full) * p.split;
  // more than 64 KB of dynamic LDS must be allowed explicitly (gfx950 has 160 KB per CU)
  const bool pair = !(p.hist_tiles > 0 && p.hist_int8);
  const void* fn = p.needs_mask ? (pair ? (const void*)attn_kernel<true, true> : (const void*)attn_kernel<true, false>)
                                : (pair ? (const void*)attn_kernel<false, true> : (const void*)attn_kernel<false, false>);
  const int lds = pair ? LDS_PAIR_BYTES : LDS_BYTES;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)nwg), block(NT);
  if (p.needs_mask) {
    if (pair) hipLaunchKernelGGL((attn_kernel<true, true>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((attn_kernel<true, false>), grid, block, lds, s, p);
  } else {
    if (pair) hipLaunchKernelGGL((attn_kernel<false, true>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((attn_kernel<false, false>), grid, block, lds, s, p);
  }
  if (p.split > 1) {
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = ((int64_t)p.n_qtiles * p.n_heads - p.n_full) * BM;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace segc
