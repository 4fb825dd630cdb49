// Internal declarations shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "segcausal.h"

namespace segc {

// ------------------------------------------------------------- RoPE ----
struct RopeParams {
  const uint16_t* x_in;
  uint16_t* x_out;
  const int32_t* pos;
  int64_t n_tok;
  int64_t stride_tok, stride_head;   // elements
  int32_t n_heads;
  int32_t dims[3];                   // t, h, w slice widths
  double inv_freq[64];               // theta^(-2i/d) per pair, t pairs then h then w
};
hipError_t launch_rope(const RopeParams& p, hipStream_t s);

// ----------------------------------------------------------- append ----
struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_st, k_sh, v_st, v_sh;    // elements
  void* ck;                          // cache K (int8 codes or bf16)
  void* cv;
  float* cks;                        // cache scales (INT8)
  float* cvs;
  int32_t n_tok;                     // n_frames * G
  int32_t G;
  int32_t n_heads;
  int32_t n_slots;
  int32_t first_slot;
  int32_t int8;
};
hipError_t launch_append(const AppendParams& p, hipStream_t s);

// -------------------------------------------------- window dequantise ----
struct DequantParams {
  const int8_t* ck;                  // INT8 cache codes [n_slots][H][G][128]
  const int8_t* cv;
  const float* cks;                  // INT8 cache scales [n_slots][H][G]
  const float* cvs;
  uint16_t* ok;                      // BF16 output cache [>= n][H][G][128]
  uint16_t* ov;
  const int32_t* slots;              // device [n]: source slot of output frame i
  int32_t rows_per_frame;            // H * G
  int32_t n_rows;                    // n * H * G
};
hipError_t launch_dequant(const DequantParams& p, hipStream_t s);

// -------------------------------------------------------- attention ----
constexpr int kMaxSeg = SEGC_MAX_SEG;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;   // elements
  // history (cache) view
  const void* hk;
  const void* hv;
  const float* hks;
  const float* hvs;
  const int32_t* hist_slots;
  int32_t n_hist_rows;       // n_hist * G
  int32_t hist_tiles;        // ceil(n_hist_rows / 64)
  int32_t G;
  int32_t hist_int8;
  // current segment(s)
  int32_t n_cur;
  int32_t n_heads;
  int32_t n_qtiles;
  int32_t n_seg;
  int32_t needs_mask;        // segment structure beyond one unpadded segment
  float sm_scale;
  float scale_log2;          // sm_scale * log2(e)
  int32_t seg_start[kMaxSeg + 1];
  int32_t seg_text_len[kMaxSeg];
  int32_t seg_text_valid[kMaxSeg];
  // Split of the last partial round (split > 1): workgroups [0, n_full) take
  // whole (head, query tile)s; each later tile is taken by `split` workgroups
  // over key ranges, whose partial results go to ws and are merged after.
  int32_t n_full;
  int32_t split;
  float* ws;
};
// Workspace bytes and split for p on a device with n_cu compute units (fills
// n_full and split in p; split = 1 and 0 bytes when the call does not split).
int64_t attn_split_plan(AttnParams& p, int n_cu);
hipError_t launch_attn(const AttnParams& p, hipStream_t s);

// Gradients of the packed form (no history): delta = rowsum(do * o), then
// dq, and dk with dv, from q, k, v, do and the forward's natural-log lse.
struct AttnBwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const float* lse;          // [n_heads][n]
  float* delta;              // [n_heads][n], written by the first kernel
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;       // elements
  int64_t do_st, do_sh, dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh;
  int32_t n;
  int32_t n_heads;
  int32_t n_seg;
  int32_t needs_mask;        // segment structure beyond one unpadded segment
  float sm_scale;
  float scale_log2;          // sm_scale * log2(e)
  int32_t seg_start[kMaxSeg + 1];
  int32_t seg_text_len[kMaxSeg];
  int32_t seg_text_valid[kMaxSeg];
};
hipError_t launch_attn_bwd(const AttnBwdParams& p, hipStream_t s);

// Host side (api.cpp): the backward's argument checks and launches with the
// delta workspace given separately, and the error reporting of the ABI.
int attn_bwd_checked(const segc_attn_bwd_args* a, float* delta, void* stream);
int report(int code, const char* msg);

// Linear with INT8 weights: y[M][N] = bf16(scale[n] * x[M][K] . code[n][K] + bias[n]).
struct W8GemmParams {
  const uint16_t* x;         // bf16 [M][ldx]
  const int8_t* w;           // int8 [N][ldw]
  const float* scale;        // [N]
  const float* bias;         // [N] or null
  uint16_t* y;               // bf16 [M][ldy]
  uint16_t* wbf;             // workspace: the codes as bf16, dense [N][K]
  int64_t ldx, ldw, ldy;     // elements
  int32_t M, N, K;
  int32_t n_tiles, m_tiles;  // set by the launcher
};
hipError_t launch_w8a16(const W8GemmParams& p, hipStream_t s);

// Camera cross-attention: row r attends to camera rows [c t_cam, (c+1) t_cam),
// c = r / tpc.
struct CamParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_st, q_sh, kv_st, kv_sh, o_st, o_sh;   // elements
  int64_t n_tok;
  int32_t n_heads, tpc, t_cam;
  float scale_log2;          // sm_scale * log2(e)
};
hipError_t launch_camera_attn(const CamParams& p, hipStream_t s);

}  // namespace segc
