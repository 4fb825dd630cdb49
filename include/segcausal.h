/*
 * segcausal.h -- C ABI of libsegcausal.so: segment-wise causal joint attention
 * over a persistent per-layer KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method: inside each dual-stream MMDiT block, the current segment's text
 * and video tokens attend jointly over the layer's KV cache of earlier
 * segments plus the current segment; video positions carry 3D RoPE; the cache
 * may be stored in INT8 while attention is computed in BF16; a single-GPU
 * deployment bounds the history to a window of recent latent frames.
 * Sources: "Hy-Nomas: Towards Free-Form Interactive World Generation" (model
 * card), section "Segment-Autoregressive Diffusion Transformer", its
 * architecture table, and section "Single-GPU Low-Memory Inference";
 * "Hy-Nomas Explained: How Tencent's Open World Model Runs Steerable Video on
 * an RTX 4090", Step 2 "Segment-wise causal joint attention".
 *
 * Conventions for every entry point:
 *  - Tensor pointers are caller-owned DEVICE memory unless marked "host".
 *    The library never allocates, frees or keeps pointers after returning.
 *  - bf16 tensors of rows are laid out [rows][heads][128] with the 128 head
 *    elements contiguous; the token and head strides are given in ELEMENTS and
 *    must be multiples of 8 (16-byte aligned rows) below SEGC_MAX_STRIDE
 *    (the kernels form a row's offset inside a staged group of rows in 32
 *    bits); base pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call is asynchronous on that stream; the library never
 *    synchronises. The caller keeps buffers alive until the stream has run the
 *    work and orders writes and reads of the same memory on its streams.
 *  - All argument checks happen on the host before anything is launched. On a
 *    non-zero status nothing has been written; segcausal_last_error() returns
 *    a message (per calling thread). Device-side bounds (e.g. that a pointer
 *    really spans the stated sizes) cannot be checked: they are preconditions.
 *  - No call prints, exits or throws across the ABI. The library holds no
 *    device state and is reentrant.
 */
#ifndef SEGCAUSAL_H
#define SEGCAUSAL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SEGC_OK           0
#define SEGC_EINVAL       1  /* bad argument: null/misaligned pointer, bad size, stride, slot, segment */
#define SEGC_EUNSUPPORTED 2  /* well-formed but outside what the kernels implement */
#define SEGC_EHIP         3  /* a HIP launch error; the message has hipGetErrorString */

/* cache element types */
#define SEGC_BF16 0
#define SEGC_INT8 1

#define SEGC_HEAD_DIM 128    /* 16 heads x 128 dims per head (model card, architecture table) */
#define SEGC_MAX_SEG  16     /* packed segments per attention call */
#define SEGC_MAX_STRIDE ((int64_t)1 << 26)   /* exclusive bound on every stride, in elements */

/*
 * A per-layer KV cache of latent frames (the keys and values of earlier
 * segments that each layer reuses; model card, section "Segment-Autoregressive
 * Diffusion Transformer"). Holds video tokens only, K after RoPE, V as is.
 *
 * Memory (all caller-owned device memory):
 *   k, v       : [n_slots][n_heads][tokens_per_frame][128], bf16 (SEGC_BF16)
 *                or int8 codes (SEGC_INT8); one slot holds one latent frame,
 *                its tokens in raster (h, w) order.
 *   k_scale,
 *   v_scale    : [n_slots][n_heads][tokens_per_frame] fp32, SEGC_INT8 only
 *                (NULL for SEGC_BF16). Dequantised value = code * scale.
 * The host tracks which latent-frame index t each slot holds (see
 * window_select).
 */
typedef struct segc_cache {
  int32_t dtype;             /* SEGC_BF16 or SEGC_INT8 */
  int32_t n_heads;
  int32_t head_dim;          /* must be 128 */
  int32_t tokens_per_frame;  /* G = grid_h * grid_w, e.g. 22 * 40 = 880 */
  int32_t n_slots;           /* frame capacity */
  int32_t reserved;
  void*  k;
  void*  v;
  float* k_scale;
  float* v_scale;
} segc_cache;

/*
 * rope3d_apply -- 3D rotary position embedding of video rows.
 * Source: model card architecture table, "Position encoding": 3D RoPE with
 * temporal/height/width dimensions [16, 56, 56] and theta 256; section
 * "Segment-Autoregressive Diffusion Transformer": RoPE encodes video positions.
 *
 * For every row r < n_tok and head: the head's 128 elements are split into
 * contiguous slices of widths d_t, d_h, d_w (in that order); inside a slice of
 * width d, the pair (2i, 2i+1) is rotated by the angle pos_axis * theta^(-2i/d)
 *   (x0, x1) <- (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 * The rotation is evaluated in double precision and rounded once to bf16
 * (nearest, ties to even). Text rows take no RoPE: do not pass them.
 *
 * x_in, x_out : bf16 [n_tok] rows with token stride `stride_tok` and head
 *               stride `stride_head` (elements), shared by both; x_out == x_in
 *               is allowed (in place); partial overlap is not.
 * pos         : int32 [n_tok][3] = (t, h, w) integer latent-grid coordinates.
 * Errors: EINVAL on null/misaligned pointers, n_tok < 0, n_heads < 1, bad
 *   strides, theta <= 0; EUNSUPPORTED if head_dim != 128 or the widths are not
 *   even and positive or do not sum to head_dim. n_tok == 0 is a no-op.
 */
int rope3d_apply(const void* x_in, void* x_out, int64_t n_tok, int32_t n_heads,
                 int32_t head_dim, int64_t stride_tok, int64_t stride_head,
                 const int32_t* pos, double theta, int32_t d_t, int32_t d_h,
                 int32_t d_w, void* stream);

/*
 * kv_cache_append -- write the current segment's video K (after RoPE) and V
 * into cache slots, quantising to INT8 when the cache is SEGC_INT8.
 * Source: model card, section "Segment-Autoregressive Diffusion Transformer"
 * (cached keys and values serve again as generation moves on) and section
 * "Single-GPU Low-Memory Inference" (cached keys/values stored in INT8, BF16
 * compute). The INT8 scheme is this library's: per (token, head)
 *   scale = fp32(max|x| / 127)             (IEEE fp32 division)
 *   code  = clamp(rint(fp32(x / scale)), -127, 127)   (ties to even)
 * with scale = 0 and all codes 0 for an all-zero row; K and V separately.
 * BF16 caches receive a plain copy.
 *
 * Frame f (0 <= f < n_frames) = input rows [f*G, (f+1)*G) goes to slot
 * (first_slot + f) mod n_slots, so a ring of slots can wrap.
 * k, v : bf16 [n_frames * G] rows, strides in elements (see conventions).
 * Errors: EINVAL on null/misaligned pointers, a bad cache descriptor,
 *   first_slot outside [0, n_slots), n_frames < 0 or > n_slots, bad strides.
 */
int kv_cache_append(const segc_cache* cache, int32_t first_slot, int32_t n_frames,
                    const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                    const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                    void* stream);

/*
 * kv_window_dequant -- expand selected frames of an INT8 cache into a BF16
 * cache, in window order: output slot i (0 <= i < n_frames) receives source
 * slot slots[i], as bf16(fp32(code * scale)) for every element of K and V.
 * Attention over the window may then read the BF16 cache with hist_slots =
 * 0, 1, ..., n_frames - 1 and gives bit-identical outputs to reading the INT8
 * cache with hist_slots = slots: the values are those the attention forms
 * when it dequantises a tile itself, computed once per window instead of
 * once per query tile.
 * Source: model card, section "Single-GPU Low-Memory Inference" (keys and
 * values stored in INT8, attention in BF16).
 * cache  : SEGC_INT8 source (read only).
 * slots  : device int32 [n_frames]; each entry in [0, cache->n_slots)
 *          (not checked: device memory).
 * out    : SEGC_BF16 cache with the same n_heads and tokens_per_frame and
 *          n_slots >= n_frames; caller-owned, written in slots 0..n_frames-1.
 * Errors: EINVAL on a bad descriptor, a source that is not INT8, an output
 *   that is not BF16 or differs in heads/tokens per frame, n_frames outside
 *   [0, out->n_slots], a null or misaligned slots pointer, more than 2^31
 *   rows. n_frames == 0 is a no-op.
 */
int kv_window_dequant(const segc_cache* cache, const int32_t* slots, int32_t n_frames,
                      const segc_cache* out, void* stream);

/*
 * kv_archive_fetch / kv_archive_store -- move whole frames between a device
 * cache and a history archive in pinned host memory.
 * Source: model card, section "Single-GPU Low-Memory Inference" (up to 18
 * historical frames on the GPU, older history archived on the CPU) and the
 * model card's description of the per-layer cache reused as generation
 * advances.
 *
 * The archive is a segc_cache whose k, v (and k_scale, v_scale for INT8)
 * point to PINNED HOST memory (hipHostMalloc or an equivalent pinned
 * allocation) in the cache layout, n_slots = its frame capacity. fetch copies
 * archive frame archive_frames[i] into cache slot slots[i]; store copies cache
 * slot slots[i] into archive frame archive_frames[i] (codes and scales,
 * byte for byte). archive_frames and slots are HOST int32 arrays of n
 * entries. Copies are asynchronous DMA on `stream` (a copy stream lets them
 * overlap attention on another stream); runs of consecutive frames on both
 * sides go as one copy per tensor. The caller keeps the host lists' contents
 * only until the call returns, and the archive and cache alive and unchanged
 * until the stream has run the copies.
 * Errors: EINVAL on a bad descriptor, descriptors that differ in dtype,
 *   heads or tokens_per_frame, n < 0, NULL lists, an index out of range, a
 *   destination frame listed twice, an archive that is not pinned host
 *   memory or a cache that is not device memory; EHIP if a copy cannot be
 *   queued (earlier copies of the call may then have been queued).
 *   n == 0 is a no-op.
 */
int kv_archive_fetch(const segc_cache* archive, const int32_t* archive_frames, const segc_cache* cache,
                     const int32_t* slots, int32_t n, void* stream);
int kv_archive_store(const segc_cache* cache, const int32_t* slots, const segc_cache* archive,
                     const int32_t* archive_frames, int32_t n, void* stream);

/*
 * w8a16_linear -- linear layer with INT8 weights and BF16 activations.
 * Source: model card, assets table (the quantized distilled DiT stores
 * weights in INT8, DiT linear computation stays BF16) and section
 * "Single-GPU Low-Memory Inference"; Explainer, architecture notes (hidden
 * size 2,048, feed-forward 8,192). This library's weight format: one fp32
 * scale per output channel, weight value = code * scale, codes in
 * [-127, 127].
 *   y[i][j] = bf16( w_scale[j] * sum_t x[i][t] * w[j][t] + bias[j] )
 * computed with bf16 MFMA products (codes are exact in bf16) and fp32
 * accumulation; the scale and bias are applied in fp32, rounded once. The
 * codes are first expanded to bf16 into `workspace` (one pass per call, on
 * the same stream), which the product then reads.
 *
 * x       : bf16 [m][ldx] row-major, first k columns used
 * w       : int8 [n][ldw] row-major codes, first k columns used
 * w_scale : fp32 [n]; bias: fp32 [n] or NULL
 * y       : bf16 [m][ldy] output, first n columns written
 * workspace : caller-owned device memory of 2 * n * k bytes (bf16 [n][k]),
 *           overwritten; it may not overlap x, w or y
 * Errors: EINVAL on m outside [0, 2^31), negative n or k, ldx < k or not a
 *   multiple of 8, ldw < k or not a multiple of 16, ldy < n or not a
 *   multiple of 4, ldx, ldw or ldy at or above SEGC_MAX_STRIDE, NULL or misaligned pointers (x, w, w_scale, bias,
 *   workspace: 16 bytes; y: 8 bytes), y equal to x or w, a workspace
 *   overlapping x, w or y; EUNSUPPORTED unless n is a multiple of 256 and k
 *   a positive multiple of 64. m == 0 or n == 0 is a no-op.
 */
int w8a16_linear(const void* x, int64_t ldx, const int8_t* w, int64_t ldw, const float* w_scale,
                 const float* bias, void* y, int64_t ldy, int64_t m, int32_t n, int32_t k, void* workspace,
                 void* stream);

/*
 * camera_cross_attn -- per-latent-frame camera cross-attention of the video
 * rows.
 * Source: model card, section "Text and Camera Conditioning" (four video
 * frames' camera extrinsics form one 64-dimensional input per latent frame;
 * in each double-stream block, following its video MLP, the video tokens
 * cross-attend to the projected camera features in chunks of one latent
 * frame).
 *
 * Row r (0 <= r < n_tok) belongs to chunk c = r / tokens_per_chunk (e.g.
 * tokens_per_chunk = 880 for one 22x40 latent frame) and attends to camera
 * rows c*t_cam .. c*t_cam + t_cam - 1 of k and v. Per head:
 *   o_r = sum_j softmax_j(sm_scale * q_r . k_j) v_j
 * in fp32 from bf16 inputs, rounded once to bf16. With t_cam == 1 (the pages'
 * configuration, one camera token per latent frame) the weight is exactly 1
 * and o_r = v of the chunk; q is then not read and may be NULL.
 */
typedef struct segc_camera_args {
  const void* q;   /* bf16 [n_tok] rows (video queries) */
  const void* k;   /* bf16 [ceil(n_tok / tokens_per_chunk) * t_cam] rows (camera keys) */
  const void* v;   /* bf16, same rows and strides as k (camera values) */
  void*       o;   /* bf16 [n_tok] rows, output */
  int64_t q_stride_tok, q_stride_head;
  int64_t kv_stride_tok, kv_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t n_tok;
  int32_t n_heads;
  int32_t head_dim;          /* must be 128 */
  int32_t tokens_per_chunk;  /* >= 1 */
  int32_t t_cam;             /* camera tokens per chunk, 1 .. 4096 */
  float   sm_scale;          /* > 0 */
} segc_camera_args;

/*
 * Errors: EINVAL on null/misaligned pointers (q only when t_cam > 1), n_tok
 *   outside [0, 2^31), n_heads outside [1, 1024], n_tok x n_heads >= 2^31
 *   (the launch grid and row indexes are 32-bit), tokens_per_chunk < 1, t_cam
 *   outside [1, 4096], bad strides, sm_scale <= 0 or not finite, o equal to
 *   q, k or v; EUNSUPPORTED if head_dim != 128. n_tok == 0 is a no-op.
 */
int camera_cross_attn(const segc_camera_args* args, void* stream);

/*
 * window_select -- choose the cached frames the attention reads (host only).
 * Source: model card, section "Segment-Autoregressive Diffusion Transformer"
 * (a bounded set of historical latent frames, default budget 18, excluding
 * the current segment; full history when unbounded) and section "Single-GPU
 * Low-Memory Inference" (up to 18 historical frames selected, older ones
 * archived on CPU). This library's policy: the `budget` most recent valid
 * frames by t, returned in ascending t.
 *
 * slot_t    : host int32 [n_slots]; slot_t[s] = latent-frame index held by
 *             slot s, or -1 if the slot is empty.
 * out_slots : host int32 [>= min(budget, n_slots)] receives slot indices.
 * out_n     : host, receives the number written.
 * Errors: EINVAL on null pointers, n_slots < 0, budget < 0, or two valid slots
 *   with the same t.
 */
int window_select(const int32_t* slot_t, int32_t n_slots, int32_t budget,
                  int32_t* out_slots, int32_t* out_n);

/*
 * segcausal_joint_attn -- segment-wise causal joint attention.
 * Source: model card, section "Segment-Autoregressive Diffusion Transformer"
 * (joint text-video attention, the layer's KV cache supplies earlier
 * segments, attention is causal across segments); "Hy-Nomas Explained ...",
 * Step 2 "Segment-wise causal joint attention".
 *
 * Keys = the selected history rows (frames hist_slots[0..n_hist), G rows
 * each) followed by the n_cur current rows. Current rows are n_seg packed
 * segments, segment s spanning rows [seg_start[s], seg_start[s+1]) laid out
 * [text (seg_text_len[s] rows) | video rows]. Query i of segment s sees key j
 * iff j is a history row, or j is in segment s and is not a padded text row
 * (text index >= seg_text_valid[s]), or j is a video row of a segment < s.
 *   o_i   = sum_j softmax_j(sm_scale * q_i . k_j) v_j   over visible j
 *   lse_i = natural log of sum_j exp(sm_scale * q_i . k_j)
 * Computed with bf16 MFMA products and fp32 accumulation and softmax; INT8
 * cache rows are dequantised to bf16 (bf16(code * scale)) as they are loaded.
 */
typedef struct segc_attn_args {
  const void* q;   /* bf16 [n_cur] rows, current segment queries (video rows after RoPE) */
  const void* k;   /* bf16 [n_cur] rows, current keys (video rows after RoPE) */
  const void* v;   /* bf16 [n_cur] rows */
  void*       o;   /* bf16 [n_cur] rows, output */
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head;
  float*  lse;     /* optional fp32 [n_heads][n_cur]; NULL = not written */
  int64_t n_cur;
  int32_t n_heads;
  int32_t head_dim;                /* must be 128 */
  int32_t n_seg;                   /* 1 .. SEGC_MAX_SEG */
  int32_t reserved;
  const int32_t* seg_start;        /* host [n_seg + 1]: 0 = seg_start[0] < ... <= seg_start[n_seg] = n_cur */
  const int32_t* seg_text_len;     /* host [n_seg] */
  const int32_t* seg_text_valid;   /* host [n_seg], <= seg_text_len */
  const segc_cache* cache;         /* NULL = no history */
  const int32_t* hist_slots;       /* device int32 [n_hist], slot indices (e.g. from window_select) */
  int32_t n_hist;                  /* number of history frames, 0 = none */
  float   sm_scale;                /* > 0, e.g. 1/sqrt(128) */
  int32_t reserved2;               /* must be 0 */
  void*   workspace;               /* optional device scratch (see below); NULL = none */
  int64_t workspace_bytes;         /* its size in bytes */
} segc_attn_args;

/*
 * Errors: EINVAL on null/misaligned pointers, n_cur < 0 or > 2^30,
 *   n_heads outside [1, 1024], n_cur x n_heads >= 2^31 (the launch grid and
 *   row indexes are 32-bit), bad strides, bad
 *   segment tables (not starting at 0, not ascending, not ending at n_cur,
 *   text_valid > text_len, text_len longer than its segment), a segment whose
 *   queries would see no key, n_hist < 0 or > n_slots, n_hist > 0 without a
 *   cache, a cache with n_heads different from the call's, sm_scale <= 0 or
 *   not finite, a hist_slots pointer that is NULL (n_hist > 0) or not 4-byte
 *   aligned; EUNSUPPORTED if head_dim != 128 or n_seg outside
 *   [1, SEGC_MAX_SEG]. n_cur == 0 is a no-op. Slot indices in hist_slots are
 *   read on the device and must lie in [0, n_slots) (a precondition).
 */
int segcausal_joint_attn(const segc_attn_args* args, void* stream);

/*
 * Bytes of device workspace with which segcausal_joint_attn(args) splits its
 * last partial round of workgroups: the grid has one workgroup per (head,
 * 256-query tile); when their number is not a multiple of the device's
 * compute units, the last round would leave units idle, so those tiles are
 * split by key range into several workgroups each, whose partial results
 * (fp32 O, row max, row sum) land in the workspace and are merged by lse in
 * one more launch. Returns 0 when the call would not split (it needs one
 * unpadded segment, bf16 keys, at least four whole rounds before the partial
 * one, and a split that pays by a cost model), -1 on a NULL args. n_cu > 0 gives the compute-unit count; 0 asks the current device
 * (-1 if that fails). The result depends only on n_cur, n_heads, the segment
 * tables, n_hist, the cache's tokens_per_frame and dtype, and n_cu.
 * With workspace NULL the call does not split. A non-NULL workspace must be
 * 16-byte aligned and hold at least this many bytes (else EINVAL); it is
 * caller-owned device memory, written and read on the call's stream, so two
 * calls in flight at once need two workspaces.
 */
int64_t segcausal_joint_attn_workspace_bytes(const segc_attn_args* args, int32_t n_cu);

/*
 * segcausal_joint_attn_bwd -- gradients of segcausal_joint_attn in the packed
 * training form (every segment of the sequence present, no history).
 * Source: "Hy-Nomas Explained ...", section "The training recipe" (segment
 * forcing on sequences packed offline, up to 360,000 tokens), differentiating
 * the attention and mask of segcausal_joint_attn above.
 *
 * With p_ij = exp(sm_scale * q_i . k_j - lse_i) over the keys query i sees
 * (the same mask as the forward with n_hist = 0) and do = dL/do:
 *   delta_i = do_i . o_i
 *   dv_j = sum_i p_ij do_i
 *   ds_ij = p_ij * (do_i . v_j - delta_i)
 *   dq_i = sm_scale * sum_j ds_ij k_j,   dk_j = sm_scale * sum_i ds_ij q_i
 * Computed with bf16 MFMA products and fp32 accumulation; p and ds are rounded
 * to bf16 as MFMA operands; dq, dk, dv are written as bf16 (overwritten, not
 * accumulated). Keys no query sees (padded text rows) get dk = dv = 0.
 */
typedef struct segc_attn_bwd_args {
  const void* q;      /* bf16 [n] rows, the forward's q (after RoPE) */
  const void* k;      /* bf16 [n] rows, the forward's k (after RoPE) */
  const void* v;      /* bf16 [n] rows */
  const void* o;      /* bf16 [n] rows, the forward's output */
  const void* dout;   /* bf16 [n] rows, dL/do */
  void*       dq;     /* bf16 [n] rows, output */
  void*       dk;     /* bf16 [n] rows, output */
  void*       dv;     /* bf16 [n] rows, output */
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t do_stride_tok, do_stride_head;
  int64_t dq_stride_tok, dq_stride_head;
  int64_t dk_stride_tok, dk_stride_head;
  int64_t dv_stride_tok, dv_stride_head;
  const float* lse;   /* fp32 [n_heads][n], natural log, as the forward wrote it */
  float* delta;       /* fp32 [n_heads][n], caller-owned workspace, receives delta */
  int64_t n;
  int32_t n_heads;
  int32_t head_dim;                /* must be 128 */
  int32_t n_seg;                   /* 1 .. SEGC_MAX_SEG */
  int32_t reserved;
  const int32_t* seg_start;        /* host [n_seg + 1], as for segcausal_joint_attn */
  const int32_t* seg_text_len;     /* host [n_seg] */
  const int32_t* seg_text_valid;   /* host [n_seg] */
  float   sm_scale;                /* > 0, the forward's */
} segc_attn_bwd_args;

/*
 * Errors: EINVAL on null/misaligned pointers (rows 16-byte aligned, lse and
 *   delta 4-byte aligned), n < 0 or n >= 2^30, n x n_heads >= 2^31 (the
 *   launch grid and row indexes are 32-bit), bad strides, bad segment
 *   tables (as for segcausal_joint_attn, including a segment whose queries
 *   would see no key), sm_scale <= 0 or not finite, an output (dq, dk, dv,
 *   delta) whose base pointer equals another argument's (in-place);
 *   EUNSUPPORTED if head_dim != 128 or n_seg outside [1, SEGC_MAX_SEG].
 *   n == 0 is a no-op. Outputs must not overlap inputs or each other
 *   element-wise (a precondition beyond the base-pointer check; interleaved
 *   views of one buffer are fine).
 */
int segcausal_joint_attn_bwd(const segc_attn_bwd_args* args, void* stream);

/*
 * segcausal_joint_attn_bwd_noalloc -- segcausal_joint_attn_bwd for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). It takes the same
 * arguments and computes the same gradients with the same kernels, but
 * args->delta is ignored (it may be NULL): delta lives in a device array of
 * 2^23 floats (32 MiB) inside the library, which each GPU the library runs on
 * holds until the process ends. The call allocates nothing, does not
 * synchronise, and on the first call on a device looks up that device's
 * address of the array (the device must be current). Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on other streams or
 * from other host threads) race and must be ordered by the caller.
 * Errors: those of segcausal_joint_attn_bwd (delta excepted), and EINVAL when
 *   n x n_heads exceeds 2^23; EHIP if the device or the array's address cannot
 *   be queried.
 */
int segcausal_joint_attn_bwd_noalloc(const segc_attn_bwd_args* args, void* stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* segcausal_last_error(void);

/* ABI version of this header, (major << 16) | minor. */
int segcausal_abi_version(void);
#define SEGC_ABI_VERSION ((1 << 16) | 9)

#ifdef __cplusplus
}
#endif

#endif /* SEGCAUSAL_H */
