// Host side of libsegcausal.so: argument checks, error reporting, window
// selection and kernel launches. Every check runs before anything is
// launched, so a non-zero status means nothing was written.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SEGC_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SEGC_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device, looked up once per device.
int device_cu_count(int* n_cu) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SEGC_EINVAL, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute");
    cache[dev] = v;
  }
  *n_cu = cache[dev];
  return SEGC_OK;
}

// Strides are multiples of 8 elements (16-byte rows) and below
// SEGC_MAX_STRIDE: the kernels form a row's offset inside a staged group of at
// most 16 rows in 32 bits (15 * 2 bytes * 2^26 < 2^31).
bool strides_ok(int64_t st, int64_t sh) {
  return st >= 0 && sh >= 0 && st % 8 == 0 && sh % 8 == 0 && st < SEGC_MAX_STRIDE && sh < SEGC_MAX_STRIDE;
}

// Segment tables: rows [seg_start[s], seg_start[s+1]) are segment s, its first
// seg_text_len[s] rows text, the first seg_text_valid[s] of those unpadded.
int check_segments(int n_seg, const int32_t* start, const int32_t* text_len, const int32_t* text_valid,
                   int64_t n) {
  if (!start || !text_len || !text_valid) return fail(SEGC_EINVAL, "NULL segment table");
  if (start[0] != 0) return fail(SEGC_EINVAL, "seg_start[0] must be 0");
  if (start[n_seg] != n) return fail(SEGC_EINVAL, "seg_start[n_seg] = %d != %lld rows", start[n_seg], (long long)n);
  for (int s = 0; s < n_seg; ++s) {
    const int len = start[s + 1] - start[s];
    if (len < 0) return fail(SEGC_EINVAL, "seg_start not ascending at %d", s);
    if (text_len[s] < 0 || text_len[s] > len)
      return fail(SEGC_EINVAL, "segment %d: text_len %d outside [0, %d]", s, text_len[s], len);
    if (text_valid[s] < 0 || text_valid[s] > text_len[s])
      return fail(SEGC_EINVAL, "segment %d: text_valid %d > text_len %d", s, text_valid[s], text_len[s]);
  }
  return SEGC_OK;
}

// Every query must see at least one key (else its softmax is undefined).
int check_visible(int n_seg, const int32_t* start, const int32_t* text_len, const int32_t* text_valid,
                  int64_t n_hist_rows) {
  int64_t earlier_video = 0;
  for (int s = 0; s < n_seg; ++s) {
    const int len = start[s + 1] - start[s];
    const int64_t visible = n_hist_rows + earlier_video + text_valid[s] + (len - text_len[s]);
    if (len > 0 && visible == 0) return fail(SEGC_EINVAL, "segment %d has no visible key", s);
    earlier_video += len - text_len[s];
  }
  return SEGC_OK;
}


int check_cache(const segc_cache* c) {
  if (!c) return fail(SEGC_EINVAL, "cache descriptor is NULL");
  if (c->dtype != SEGC_BF16 && c->dtype != SEGC_INT8)
    return fail(SEGC_EINVAL, "cache dtype %d is neither SEGC_BF16 nor SEGC_INT8", c->dtype);
  if (c->head_dim != SEGC_HEAD_DIM)
    return fail(SEGC_EUNSUPPORTED, "cache head_dim %d != 128", c->head_dim);
  if (c->n_heads < 1 || c->tokens_per_frame < 1 || c->n_slots < 1)
    return fail(SEGC_EINVAL, "cache n_heads, tokens_per_frame and n_slots must be >= 1");
  if ((int64_t)c->n_slots * c->n_heads * c->tokens_per_frame > ((int64_t)1 << 40))
    return fail(SEGC_EINVAL, "cache is too large");
  if (!c->k || !c->v) return fail(SEGC_EINVAL, "cache k/v pointer is NULL");
  if (!aligned16(c->k) || !aligned16(c->v))
    return fail(SEGC_EINVAL, "cache k/v pointers must be 16-byte aligned");
  if (c->dtype == SEGC_INT8) {
    if (!c->k_scale || !c->v_scale) return fail(SEGC_EINVAL, "INT8 cache needs k_scale and v_scale");
    if (((uintptr_t)c->k_scale & 3u) || ((uintptr_t)c->v_scale & 3u))
      return fail(SEGC_EINVAL, "cache scales must be 4-byte aligned");
  }
  return SEGC_OK;
}

// Memory kind of [p, p + bytes) as HIP reports it at both ends (pinned host
// memory, device memory, or neither).
hipMemoryType memory_kind(const void* p, size_t bytes) {
  hipPointerAttribute_t a, b;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return hipMemoryTypeUnregistered;
  }
  if (bytes > 1 && hipPointerGetAttributes(&b, (const char*)p + bytes - 1) != hipSuccess) {
    (void)hipGetLastError();
    return hipMemoryTypeUnregistered;
  }
  if (bytes > 1 && b.type != a.type) return hipMemoryTypeUnregistered;
  return a.type;
}

// Frame copies between two caches of one layout (one of them a pinned host
// archive): element i moves frame src_idx[i] of src into frame dst_idx[i]
// of dst. Runs of consecutive frames on both sides become one copy per tensor.
int move_frames(const segc_cache* src, const int32_t* src_idx, const segc_cache* dst, const int32_t* dst_idx,
                int32_t n, hipMemcpyKind kind, const char* what, void* stream) {
  int rc = check_cache(src);
  if (rc) return rc;
  rc = check_cache(dst);
  if (rc) return rc;
  if (src->dtype != dst->dtype || src->n_heads != dst->n_heads || src->tokens_per_frame != dst->tokens_per_frame)
    return fail(SEGC_EINVAL, "%s: archive and cache differ in dtype, heads or tokens_per_frame", what);
  if (n < 0) return fail(SEGC_EINVAL, "%s: n < 0", what);
  if (n == 0) return ok();
  if (!src_idx || !dst_idx) return fail(SEGC_EINVAL, "%s: NULL frame list", what);
  std::vector<int32_t> seen;
  seen.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    if (src_idx[i] < 0 || src_idx[i] >= src->n_slots)
      return fail(SEGC_EINVAL, "%s: source frame %d outside [0, %d)", what, src_idx[i], src->n_slots);
    if (dst_idx[i] < 0 || dst_idx[i] >= dst->n_slots)
      return fail(SEGC_EINVAL, "%s: destination frame %d outside [0, %d)", what, dst_idx[i], dst->n_slots);
    seen.push_back(dst_idx[i]);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(SEGC_EINVAL, "%s: a destination frame appears twice", what);
  const size_t rows = (size_t)src->n_heads * src->tokens_per_frame;
  const size_t code_bytes = rows * SEGC_HEAD_DIM * (src->dtype == SEGC_INT8 ? 1 : 2);
  const size_t scale_bytes = rows * sizeof(float);
  const bool int8 = src->dtype == SEGC_INT8;
  const segc_cache* host = kind == hipMemcpyHostToDevice ? src : dst;
  const segc_cache* dev = kind == hipMemcpyHostToDevice ? dst : src;
  const void* hp[4] = {host->k, host->v, host->k_scale, host->v_scale};
  const void* dp[4] = {dev->k, dev->v, dev->k_scale, dev->v_scale};
  const size_t fb[4] = {code_bytes, code_bytes, scale_bytes, scale_bytes};
  for (int t = 0; t < (int8 ? 4 : 2); ++t) {
    if (memory_kind(hp[t], fb[t] * host->n_slots) != hipMemoryTypeHost)
      return fail(SEGC_EINVAL, "%s: the archive must be pinned host memory (hipHostMalloc)", what);
    if (memory_kind(dp[t], fb[t] * dev->n_slots) != hipMemoryTypeDevice)
      return fail(SEGC_EINVAL, "%s: the cache must be device memory", what);
  }
  char* const sp[4] = {(char*)src->k, (char*)src->v, (char*)src->k_scale, (char*)src->v_scale};
  char* const tp[4] = {(char*)dst->k, (char*)dst->v, (char*)dst->k_scale, (char*)dst->v_scale};
  for (int32_t i = 0; i < n;) {
    int32_t j = i + 1;
    while (j < n && src_idx[j] == src_idx[j - 1] + 1 && dst_idx[j] == dst_idx[j - 1] + 1) ++j;
    const size_t frames = (size_t)(j - i);
    for (int t = 0; t < (int8 ? 4 : 2); ++t) {
      const hipError_t e = hipMemcpyAsync(tp[t] + fb[t] * dst_idx[i], sp[t] + fb[t] * src_idx[i], fb[t] * frames,
                                          kind, (hipStream_t)stream);
      if (e != hipSuccess) return hip_status(e, what);
    }
    i = j;
  }
  return ok();
}

}  // namespace

int segc::report(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

const char* segcausal_last_error(void) { return g_err; }

int segcausal_abi_version(void) { return SEGC_ABI_VERSION; }

int rope3d_apply(const void* x_in, void* x_out, int64_t n_tok, int32_t n_heads, int32_t head_dim,
                 int64_t stride_tok, int64_t stride_head, const int32_t* pos, double theta,
                 int32_t d_t, int32_t d_h, int32_t d_w, void* stream) {
  if (head_dim != SEGC_HEAD_DIM) return fail(SEGC_EUNSUPPORTED, "head_dim %d != 128", head_dim);
  if (d_t <= 0 || d_h <= 0 || d_w <= 0 || (d_t | d_h | d_w) & 1 || d_t + d_h + d_w != head_dim)
    return fail(SEGC_EUNSUPPORTED, "RoPE widths (%d, %d, %d) must be even, positive, sum to 128",
                d_t, d_h, d_w);
  if (n_tok < 0 || n_tok > ((int64_t)1 << 32)) return fail(SEGC_EINVAL, "n_tok out of range");
  if (n_heads < 1 || n_heads > 1024) return fail(SEGC_EINVAL, "n_heads out of range");
  if (!(theta > 0.0) || !std::isfinite(theta)) return fail(SEGC_EINVAL, "theta must be > 0");
  if (!strides_ok(stride_tok, stride_head))
    return fail(SEGC_EINVAL, "strides must be non-negative multiples of 8 elements below 2^26");
  if (n_tok == 0) return ok();
  if (!x_in || !x_out || !pos) return fail(SEGC_EINVAL, "NULL pointer");
  if (!aligned16(x_in) || !aligned16(x_out))
    return fail(SEGC_EINVAL, "x_in/x_out must be 16-byte aligned");
  if (((uintptr_t)pos & 3u)) return fail(SEGC_EINVAL, "pos must be 4-byte aligned");
  segc::RopeParams p;
  p.x_in = (const uint16_t*)x_in;
  p.x_out = (uint16_t*)x_out;
  p.pos = pos;
  p.n_tok = n_tok;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.n_heads = n_heads;
  p.dims[0] = d_t;
  p.dims[1] = d_h;
  p.dims[2] = d_w;
  const int widths[3] = {d_t, d_h, d_w};
  int pr = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < widths[a] / 2; ++i)
      p.inv_freq[pr++] = std::pow(theta, -2.0 * (double)i / (double)widths[a]);
  return hip_status(segc::launch_rope(p, (hipStream_t)stream), "rope3d_apply launch");
}

int kv_cache_append(const segc_cache* cache, int32_t first_slot, int32_t n_frames, const void* k,
                    int64_t k_stride_tok, int64_t k_stride_head, const void* v,
                    int64_t v_stride_tok, int64_t v_stride_head, void* stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (first_slot < 0 || first_slot >= cache->n_slots)
    return fail(SEGC_EINVAL, "first_slot %d outside [0, %d)", first_slot, cache->n_slots);
  if (n_frames < 0 || n_frames > cache->n_slots)
    return fail(SEGC_EINVAL, "n_frames %d outside [0, n_slots=%d]", n_frames, cache->n_slots);
  if (!strides_ok(k_stride_tok, k_stride_head) || !strides_ok(v_stride_tok, v_stride_head))
    return fail(SEGC_EINVAL, "strides must be non-negative multiples of 8 elements below 2^26");
  const int64_t n_tok = (int64_t)n_frames * cache->tokens_per_frame;
  if (n_tok > (int64_t)1 << 30) return fail(SEGC_EINVAL, "append too large");
  if (n_frames == 0) return ok();
  if (!k || !v) return fail(SEGC_EINVAL, "NULL k or v");
  if (!aligned16(k) || !aligned16(v)) return fail(SEGC_EINVAL, "k/v must be 16-byte aligned");
  segc::AppendParams p;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.k_st = k_stride_tok;
  p.k_sh = k_stride_head;
  p.v_st = v_stride_tok;
  p.v_sh = v_stride_head;
  p.ck = cache->k;
  p.cv = cache->v;
  p.cks = cache->k_scale;
  p.cvs = cache->v_scale;
  p.n_tok = (int32_t)n_tok;
  p.G = cache->tokens_per_frame;
  p.n_heads = cache->n_heads;
  p.n_slots = cache->n_slots;
  p.first_slot = first_slot;
  p.int8 = cache->dtype == SEGC_INT8;
  return hip_status(segc::launch_append(p, (hipStream_t)stream), "kv_cache_append launch");
}

int kv_window_dequant(const segc_cache* cache, const int32_t* slots, int32_t n_frames,
                      const segc_cache* out, void* stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (cache->dtype != SEGC_INT8) return fail(SEGC_EINVAL, "source cache must be SEGC_INT8");
  rc = check_cache(out);
  if (rc) return rc;
  if (out->dtype != SEGC_BF16) return fail(SEGC_EINVAL, "output cache must be SEGC_BF16");
  if (out->n_heads != cache->n_heads || out->tokens_per_frame != cache->tokens_per_frame)
    return fail(SEGC_EINVAL, "output cache heads/tokens_per_frame differ from the source cache");
  if (n_frames < 0 || n_frames > out->n_slots)
    return fail(SEGC_EINVAL, "n_frames %d outside [0, output n_slots=%d]", n_frames, out->n_slots);
  const int64_t rows_per_frame = (int64_t)cache->n_heads * cache->tokens_per_frame;
  if (rows_per_frame * n_frames >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "window too large");
  if (n_frames == 0) return ok();
  if (!slots) return fail(SEGC_EINVAL, "slots is NULL");
  if ((uintptr_t)slots & 3u) return fail(SEGC_EINVAL, "slots must be 4-byte aligned");
  segc::DequantParams p;
  p.ck = (const int8_t*)cache->k;
  p.cv = (const int8_t*)cache->v;
  p.cks = cache->k_scale;
  p.cvs = cache->v_scale;
  p.ok = (uint16_t*)out->k;
  p.ov = (uint16_t*)out->v;
  p.slots = slots;
  p.rows_per_frame = (int32_t)rows_per_frame;
  p.n_rows = (int32_t)(rows_per_frame * n_frames);
  return hip_status(segc::launch_dequant(p, (hipStream_t)stream), "kv_window_dequant launch");
}

int kv_archive_fetch(const segc_cache* archive, const int32_t* archive_frames, const segc_cache* cache,
                     const int32_t* slots, int32_t n, void* stream) {
  return move_frames(archive, archive_frames, cache, slots, n, hipMemcpyHostToDevice, "kv_archive_fetch",
                     stream);
}

int kv_archive_store(const segc_cache* cache, const int32_t* slots, const segc_cache* archive,
                     const int32_t* archive_frames, int32_t n, void* stream) {
  return move_frames(cache, slots, archive, archive_frames, n, hipMemcpyDeviceToHost, "kv_archive_store",
                     stream);
}

int w8a16_linear(const void* x, int64_t ldx, const int8_t* w, int64_t ldw, const float* w_scale,
                 const float* bias, void* y, int64_t ldy, int64_t m, int32_t n, int32_t k, void* workspace,
                 void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "m out of range");
  if (n < 0 || k < 0) return fail(SEGC_EINVAL, "n and k must be >= 0");
  if (n % 256 || k % 64 || k == 0)
    return fail(SEGC_EUNSUPPORTED, "n must be a multiple of 256 and k a positive multiple of 64 (n=%d, k=%d)", n, k);
  if (ldx < k || ldx % 8) return fail(SEGC_EINVAL, "ldx must be >= k and a multiple of 8");
  if (ldw < k || ldw % 16) return fail(SEGC_EINVAL, "ldw must be >= k and a multiple of 16");
  if (ldy < n || ldy % 4) return fail(SEGC_EINVAL, "ldy must be >= n and a multiple of 4");
  // row offsets inside a staged group (up to 8 rows) are formed in 32 bits
  if (ldx >= SEGC_MAX_STRIDE || ldw >= SEGC_MAX_STRIDE || ldy >= SEGC_MAX_STRIDE)
    return fail(SEGC_EINVAL, "ldx, ldw and ldy must be below 2^26");
  if (m == 0 || n == 0) return ok();
  if (!x || !w || !w_scale || !y || !workspace) return fail(SEGC_EINVAL, "NULL x/w/w_scale/y/workspace");
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & 7u) || !aligned16(w_scale) ||
      (bias && !aligned16(bias)) || !aligned16(workspace))
    return fail(SEGC_EINVAL, "x, w, w_scale, bias, workspace must be 16-byte and y 8-byte aligned");
  if ((int64_t)n * k >= ((int64_t)1 << 36)) return fail(SEGC_EINVAL, "weights too large");
  {
    // the workspace is written while x, w, y are in use: it may overlap none of them
    const uintptr_t ws = (uintptr_t)workspace, we = ws + (uintptr_t)(2 * (int64_t)n * k);
    const uintptr_t spans[3][2] = {
        {(uintptr_t)x, (uintptr_t)x + (uintptr_t)(2 * ((m - 1) * ldx + k))},
        {(uintptr_t)w, (uintptr_t)w + (uintptr_t)((int64_t)(n - 1) * ldw + k)},
        {(uintptr_t)y, (uintptr_t)y + (uintptr_t)(2 * ((m - 1) * ldy + n))}};
    for (int i = 0; i < 3; ++i)
      if (ws < spans[i][1] && spans[i][0] < we) return fail(SEGC_EINVAL, "workspace overlaps x, w or y");
  }
  const int64_t tiles = ((m + 255) / 256) * (int64_t)(n / 256);
  if (tiles >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "problem too large");
  if ((const void*)y == x || (const void*)y == (const void*)w)
    return fail(SEGC_EINVAL, "y must not be x or w (in place)");
  segc::W8GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = (const uint16_t*)x;
  p.w = w;
  p.scale = w_scale;
  p.bias = bias;
  p.y = (uint16_t*)y;
  p.wbf = (uint16_t*)workspace;
  p.ldx = ldx;
  p.ldw = ldw;
  p.ldy = ldy;
  p.M = (int32_t)m;
  p.N = n;
  p.K = k;
  return hip_status(segc::launch_w8a16(p, (hipStream_t)stream), "w8a16_linear launch");
}

int camera_cross_attn(const segc_camera_args* a, void* stream) {
  if (!a) return fail(SEGC_EINVAL, "args is NULL");
  if (a->head_dim != SEGC_HEAD_DIM) return fail(SEGC_EUNSUPPORTED, "head_dim %d != 128", a->head_dim);
  if (a->n_tok < 0 || a->n_tok >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "n_tok out of range");
  if (a->n_heads < 1 || a->n_heads > 1024) return fail(SEGC_EINVAL, "n_heads out of range");
  if (a->n_tok * a->n_heads >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "n_tok x n_heads must be below 2^31");
  if (a->tokens_per_chunk < 1) return fail(SEGC_EINVAL, "tokens_per_chunk must be >= 1");
  if (a->t_cam < 1 || a->t_cam > 4096) return fail(SEGC_EINVAL, "t_cam must be in [1, 4096]");
  if (!(a->sm_scale > 0.0f) || !std::isfinite(a->sm_scale))
    return fail(SEGC_EINVAL, "sm_scale must be finite and > 0");
  if (!strides_ok(a->q_stride_tok, a->q_stride_head) || !strides_ok(a->kv_stride_tok, a->kv_stride_head) ||
      !strides_ok(a->o_stride_tok, a->o_stride_head))
    return fail(SEGC_EINVAL, "strides must be non-negative multiples of 8 elements below 2^26");
  if (a->n_tok == 0) return ok();
  if (!a->k || !a->v || !a->o || (a->t_cam > 1 && !a->q)) return fail(SEGC_EINVAL, "NULL q/k/v/o");
  if ((a->q && !aligned16(a->q)) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(SEGC_EINVAL, "q/k/v/o must be 16-byte aligned");
  if (a->o == a->q || a->o == a->k || a->o == a->v) return fail(SEGC_EINVAL, "o must not be q, k or v (in place)");
  segc::CamParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)a->q;
  p.k = (const uint16_t*)a->k;
  p.v = (const uint16_t*)a->v;
  p.o = (uint16_t*)a->o;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.kv_st = a->kv_stride_tok;
  p.kv_sh = a->kv_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  p.n_tok = a->n_tok;
  p.n_heads = a->n_heads;
  p.tpc = a->tokens_per_chunk;
  p.t_cam = a->t_cam;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  return hip_status(segc::launch_camera_attn(p, (hipStream_t)stream), "camera_cross_attn launch");
}

int window_select(const int32_t* slot_t, int32_t n_slots, int32_t budget, int32_t* out_slots,
                  int32_t* out_n) {
  if (n_slots < 0) return fail(SEGC_EINVAL, "n_slots < 0");
  if (budget < 0) return fail(SEGC_EINVAL, "budget < 0");
  if (!out_n || (n_slots > 0 && !slot_t)) return fail(SEGC_EINVAL, "NULL pointer");
  std::vector<std::pair<int32_t, int32_t>> valid;   // (t, slot)
  valid.reserve(n_slots);
  for (int32_t s = 0; s < n_slots; ++s)
    if (slot_t[s] >= 0) valid.emplace_back(slot_t[s], s);
  std::sort(valid.begin(), valid.end());
  for (size_t i = 1; i < valid.size(); ++i)
    if (valid[i].first == valid[i - 1].first)
      return fail(SEGC_EINVAL, "slots %d and %d both hold t = %d", valid[i - 1].second,
                  valid[i].second, valid[i].first);
  const size_t keep = std::min<size_t>((size_t)budget, valid.size());
  if (keep > 0 && !out_slots) return fail(SEGC_EINVAL, "NULL out_slots");
  const size_t first = valid.size() - keep;
  for (size_t i = 0; i < keep; ++i) out_slots[i] = valid[first + i].second;
  *out_n = (int32_t)keep;
  return ok();
}

int segcausal_joint_attn(const segc_attn_args* a, void* stream) {
  if (!a) return fail(SEGC_EINVAL, "args is NULL");
  if (a->head_dim != SEGC_HEAD_DIM) return fail(SEGC_EUNSUPPORTED, "head_dim %d != 128", a->head_dim);
  if (a->n_seg < 1 || a->n_seg > SEGC_MAX_SEG)
    return fail(SEGC_EUNSUPPORTED, "n_seg %d outside [1, %d]", a->n_seg, SEGC_MAX_SEG);
  if (a->n_cur < 0 || a->n_cur > (int64_t)1 << 30) return fail(SEGC_EINVAL, "n_cur out of range");
  if (a->n_heads < 1 || a->n_heads > 1024) return fail(SEGC_EINVAL, "n_heads out of range");
  // (row, head) pairs index the launch grid and the kernels' 32-bit row math
  if (a->n_cur * a->n_heads >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "n_cur x n_heads must be below 2^31");
  if (!(a->sm_scale > 0.0f) || !std::isfinite(a->sm_scale))
    return fail(SEGC_EINVAL, "sm_scale must be finite and > 0");
  if (a->reserved != 0 || a->reserved2 != 0) return fail(SEGC_EINVAL, "reserved fields must be 0");
  if (a->workspace_bytes < 0) return fail(SEGC_EINVAL, "workspace_bytes < 0");
  if (!strides_ok(a->q_stride_tok, a->q_stride_head) || !strides_ok(a->k_stride_tok, a->k_stride_head) ||
      !strides_ok(a->v_stride_tok, a->v_stride_head) || !strides_ok(a->o_stride_tok, a->o_stride_head))
    return fail(SEGC_EINVAL, "strides must be non-negative multiples of 8 elements below 2^26");
  int rc = check_segments(a->n_seg, a->seg_start, a->seg_text_len, a->seg_text_valid, a->n_cur);
  if (rc) return rc;
  if (a->n_hist < 0) return fail(SEGC_EINVAL, "n_hist < 0");
  int64_t n_hist_rows = 0;
  int hist_int8 = 0;
  if (a->n_hist > 0) {
    if (!a->cache) return fail(SEGC_EINVAL, "n_hist > 0 without a cache");
    rc = check_cache(a->cache);
    if (rc) return rc;
    if (a->cache->n_heads != a->n_heads)
      return fail(SEGC_EINVAL, "cache has %d heads, call has %d", a->cache->n_heads, a->n_heads);
    if (a->n_hist > a->cache->n_slots)
      return fail(SEGC_EINVAL, "n_hist %d > n_slots %d", a->n_hist, a->cache->n_slots);
    if (!a->hist_slots) return fail(SEGC_EINVAL, "NULL hist_slots");
    if ((uintptr_t)a->hist_slots & 3u) return fail(SEGC_EINVAL, "hist_slots must be 4-byte aligned");
    n_hist_rows = (int64_t)a->n_hist * a->cache->tokens_per_frame;
    if (n_hist_rows > (int64_t)1 << 30) return fail(SEGC_EINVAL, "history too long");
    hist_int8 = a->cache->dtype == SEGC_INT8;
  }
  rc = check_visible(a->n_seg, a->seg_start, a->seg_text_len, a->seg_text_valid, n_hist_rows);
  if (rc) return rc;
  if (a->n_cur == 0) return ok();
  if (!a->q || !a->k || !a->v || !a->o) return fail(SEGC_EINVAL, "NULL q/k/v/o");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(SEGC_EINVAL, "q/k/v/o must be 16-byte aligned");
  if (a->lse && ((uintptr_t)a->lse & 3u)) return fail(SEGC_EINVAL, "lse must be 4-byte aligned");

  segc::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)a->q;
  p.k = (const uint16_t*)a->k;
  p.v = (const uint16_t*)a->v;
  p.o = (uint16_t*)a->o;
  p.lse = a->lse;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.k_st = a->k_stride_tok;
  p.k_sh = a->k_stride_head;
  p.v_st = a->v_stride_tok;
  p.v_sh = a->v_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  if (a->n_hist > 0) {
    p.hk = a->cache->k;
    p.hv = a->cache->v;
    p.hks = a->cache->k_scale;
    p.hvs = a->cache->v_scale;
    p.hist_slots = a->hist_slots;
    p.G = a->cache->tokens_per_frame;
    p.n_hist_rows = (int32_t)n_hist_rows;
    p.hist_tiles = (int32_t)((n_hist_rows + 63) / 64);
    p.hist_int8 = hist_int8;
  } else {
    p.G = 1;
  }
  p.n_cur = (int32_t)a->n_cur;
  p.n_heads = a->n_heads;
  p.n_seg = a->n_seg;
  bool needs_mask = a->n_seg > 1;
  for (int s = 0; s <= a->n_seg; ++s) p.seg_start[s] = a->seg_start[s];
  for (int s = 0; s < a->n_seg; ++s) {
    p.seg_text_len[s] = a->seg_text_len[s];
    p.seg_text_valid[s] = a->seg_text_valid[s];
    needs_mask = needs_mask || a->seg_text_valid[s] < a->seg_text_len[s];
  }
  p.needs_mask = needs_mask;
  p.sm_scale = a->sm_scale;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  if (a->workspace) {
    if (!aligned16(a->workspace)) return fail(SEGC_EINVAL, "workspace must be 16-byte aligned");
    int n_cu = 0;
    rc = device_cu_count(&n_cu);
    if (rc) return rc;
    const int64_t need = segc::attn_split_plan(p, n_cu);
    if (a->workspace_bytes < need)
      return fail(SEGC_EINVAL, "workspace holds %lld bytes, this call needs %lld", (long long)a->workspace_bytes,
                  (long long)need);
    p.ws = (float*)a->workspace;
  } else {
    segc::attn_split_plan(p, 0);             // no workspace: no split
  }
  return hip_status(segc::launch_attn(p, (hipStream_t)stream), "segcausal_joint_attn launch");
}

int64_t segcausal_joint_attn_workspace_bytes(const segc_attn_args* a, int32_t n_cu) {
  if (!a) return -1;
  if (a->n_seg < 1 || a->n_seg > SEGC_MAX_SEG || a->n_cur < 0 || a->n_cur > (int64_t)1 << 30 ||
      a->n_heads < 1 || a->n_heads > 1024 || !a->seg_text_len || !a->seg_text_valid)
    return -1;
  segc::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.n_cur = (int32_t)a->n_cur;
  p.n_heads = a->n_heads;
  bool needs_mask = a->n_seg > 1;
  for (int s = 0; s < a->n_seg; ++s) needs_mask = needs_mask || a->seg_text_valid[s] < a->seg_text_len[s];
  p.needs_mask = needs_mask;
  if (a->n_hist > 0 && a->cache) {
    const int64_t rows = (int64_t)a->n_hist * a->cache->tokens_per_frame;
    p.hist_tiles = (int32_t)((rows + 63) / 64);
    p.hist_int8 = a->cache->dtype == SEGC_INT8;
  }
  if (n_cu <= 0 && device_cu_count(&n_cu)) return -1;
  return segc::attn_split_plan(p, n_cu);
}

int segcausal_joint_attn_bwd(const segc_attn_bwd_args* a, void* stream) {
  if (!a) return fail(SEGC_EINVAL, "args is NULL");
  return segc::attn_bwd_checked(a, a->delta, stream);
}

}  // extern "C"

// Checks and launches of the packed-form backward with the delta workspace
// `delta` (the caller's, or the allocation-free entry point's device scratch).
int segc::attn_bwd_checked(const segc_attn_bwd_args* a, float* delta, void* stream) {
  if (a->head_dim != SEGC_HEAD_DIM) return fail(SEGC_EUNSUPPORTED, "head_dim %d != 128", a->head_dim);
  if (a->n_seg < 1 || a->n_seg > SEGC_MAX_SEG)
    return fail(SEGC_EUNSUPPORTED, "n_seg %d outside [1, %d]", a->n_seg, SEGC_MAX_SEG);
  if (a->n < 0 || a->n >= (int64_t)1 << 30) return fail(SEGC_EINVAL, "n out of range");
  if (a->n_heads < 1 || a->n_heads > 1024) return fail(SEGC_EINVAL, "n_heads out of range");
  if (a->n * a->n_heads >= ((int64_t)1 << 31)) return fail(SEGC_EINVAL, "n x n_heads must be below 2^31");
  if (!(a->sm_scale > 0.0f) || !std::isfinite(a->sm_scale))
    return fail(SEGC_EINVAL, "sm_scale must be finite and > 0");
  const int64_t st[8][2] = {{a->q_stride_tok, a->q_stride_head},   {a->k_stride_tok, a->k_stride_head},
                            {a->v_stride_tok, a->v_stride_head},   {a->o_stride_tok, a->o_stride_head},
                            {a->do_stride_tok, a->do_stride_head}, {a->dq_stride_tok, a->dq_stride_head},
                            {a->dk_stride_tok, a->dk_stride_head}, {a->dv_stride_tok, a->dv_stride_head}};
  for (int i = 0; i < 8; ++i)
    if (!strides_ok(st[i][0], st[i][1]))
      return fail(SEGC_EINVAL, "strides must be non-negative multiples of 8 elements below 2^26");
  int rc = check_segments(a->n_seg, a->seg_start, a->seg_text_len, a->seg_text_valid, a->n);
  if (rc) return rc;
  rc = check_visible(a->n_seg, a->seg_start, a->seg_text_len, a->seg_text_valid, 0);
  if (rc) return rc;
  if (a->n == 0) return ok();
  const void* ptr[8] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv};
  for (int i = 0; i < 8; ++i) {
    if (!ptr[i]) return fail(SEGC_EINVAL, "NULL q/k/v/o/dout/dq/dk/dv");
    if (!aligned16(ptr[i])) return fail(SEGC_EINVAL, "q/k/v/o/dout/dq/dk/dv must be 16-byte aligned");
  }
  if (!a->lse || !delta) return fail(SEGC_EINVAL, "NULL lse/delta");
  if (((uintptr_t)a->lse & 3u) || ((uintptr_t)delta & 3u))
    return fail(SEGC_EINVAL, "lse/delta must be 4-byte aligned");
  // outputs are written while inputs are still read: an output that starts
  // where another argument starts is an in-place call, which this computation
  // cannot do (interleaved views, e.g. one [n][3][H][128] buffer, are fine)
  const void* all[10] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv, a->lse, delta};
  const char* names[10] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv", "lse", "delta"};
  const int outs[4] = {5, 6, 7, 9};
  for (int oi = 0; oi < 4; ++oi)
    for (int j = 0; j < 10; ++j)
      if (j != outs[oi] && all[j] == all[outs[oi]])
        return fail(SEGC_EINVAL, "%s and %s share a base pointer (in-place is not supported)",
                    names[outs[oi]], names[j]);

  segc::AttnBwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)a->q;
  p.k = (const uint16_t*)a->k;
  p.v = (const uint16_t*)a->v;
  p.o = (const uint16_t*)a->o;
  p.dout = (const uint16_t*)a->dout;
  p.dq = (uint16_t*)a->dq;
  p.dk = (uint16_t*)a->dk;
  p.dv = (uint16_t*)a->dv;
  p.lse = a->lse;
  p.delta = delta;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.k_st = a->k_stride_tok;
  p.k_sh = a->k_stride_head;
  p.v_st = a->v_stride_tok;
  p.v_sh = a->v_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  p.do_st = a->do_stride_tok;
  p.do_sh = a->do_stride_head;
  p.dq_st = a->dq_stride_tok;
  p.dq_sh = a->dq_stride_head;
  p.dk_st = a->dk_stride_tok;
  p.dk_sh = a->dk_stride_head;
  p.dv_st = a->dv_stride_tok;
  p.dv_sh = a->dv_stride_head;
  p.n = (int32_t)a->n;
  p.n_heads = a->n_heads;
  p.n_seg = a->n_seg;
  bool needs_mask = a->n_seg > 1;
  for (int s = 0; s <= a->n_seg; ++s) p.seg_start[s] = a->seg_start[s];
  for (int s = 0; s < a->n_seg; ++s) {
    p.seg_text_len[s] = a->seg_text_len[s];
    p.seg_text_valid[s] = a->seg_text_valid[s];
    needs_mask = needs_mask || a->seg_text_valid[s] < a->seg_text_len[s];
  }
  p.needs_mask = needs_mask;
  p.sm_scale = a->sm_scale;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  return hip_status(segc::launch_attn_bwd(p, (hipStream_t)stream), "segcausal_joint_attn_bwd launch");
}
