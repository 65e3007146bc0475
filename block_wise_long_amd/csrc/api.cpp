// C-ABI entry points of libblockattn: argument checks on the host, launch
// geometry, and the fp64 noise-schedule coefficients of the block update.
// Every check runs before anything is enqueued; on failure nothing is
// enqueued, no descriptor changes and ba_last_error() says why.
#include <math.h>
#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "blockattn.h"
#include "internal.h"

namespace {

// Split schedule of the bf16 attention kernel: used only when every tail
// workgroup gets at least this many key tiles on average (measured: at 8-32
// tiles per task the split is 10-50 % slower than whole tasks, at 64 equal,
// at the video key sets' ~170 faster).
constexpr int kSplitMinTilesPerWg = 24;
// ... and only when whole tasks would leave at least a quarter of an XCD's
// resident slots idle in their last round (measured at the 480p block shape
// with 16-96 heads: cutting tasks costs about a fifth of a round; with 1/8
// of the slots idle whole tasks were 1.5 % faster, at 3/16 the two tied, at
// 1/4 the split was 0.6 % faster).
constexpr int64_t kSplitIdleNum = 1, kSplitIdleDen = 4;

thread_local char g_err[512] = "";

ba_status fail(ba_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ba_status ok() {
  g_err[0] = '\0';
  return BA_OK;
}

ba_status hip_fail(hipError_t e, const char* what) {
  return fail(BA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int32_t dtype) { return dtype == BA_BF16 ? 2 : (dtype == BA_F32 ? 4 : 0); }

int64_t pad_tokens(int64_t t) {
  return (t + ba::kTokenAlign - 1) / ba::kTokenAlign * ba::kTokenAlign;
}

ba_status check_shape(int32_t n_slots, int32_t slot_tokens, int32_t heads, int32_t head_dim,
                      int32_t dtype) {
  if (dtype != BA_BF16 && dtype != BA_F32) return fail(BA_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(BA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (n_slots < 1 || slot_tokens < 1 || heads < 1)
    return fail(BA_ERR_INVALID_ARG, "n_slots, slot_tokens and heads must be >= 1");
  if (heads > 65535) return fail(BA_ERR_OUT_OF_RANGE, "heads %d > 65535", heads);
  if (slot_tokens > (1 << 30)) return fail(BA_ERR_OUT_OF_RANGE, "slot_tokens too large");
  return BA_OK;
}

ba_status check_ring(const ba_ring* r, const char* name) {
  if (r == nullptr) return fail(BA_ERR_INVALID_ARG, "%s is NULL", name);
  ba_status st = check_shape(r->n_slots, r->slot_tokens, r->heads, r->head_dim, r->dtype);
  if (st != BA_OK) return st;
  if (r->base == nullptr) return fail(BA_ERR_INVALID_ARG, "%s->base is NULL", name);
  if (!aligned(r->base, 256)) return fail(BA_ERR_INVALID_ARG, "%s->base not 256-byte aligned", name);
  if (r->slot_stride_tokens != pad_tokens(r->slot_tokens))
    return fail(BA_ERR_INVALID_ARG, "%s was not set up by ba_ring_init", name);
  if (r->appended < 0) return fail(BA_ERR_INVALID_ARG, "%s->appended < 0", name);
  return BA_OK;
}

void schedule_or_default(const ba_schedule* s, ba_schedule* out) {
  if (s) {
    *out = *s;
  } else {
    out->T = 1000;
    out->stride = 20;
    out->beta_start = 1e-4;
    out->beta_end = 0.02;
    out->kind = BA_SCHED_DDIM;
    out->shift = 1.0;
  }
}

ba_status check_schedule(const ba_schedule& s) {
  if (s.T < 2 || s.T > 100000) return fail(BA_ERR_OUT_OF_RANGE, "schedule T=%d outside [2, 100000]", s.T);
  if (s.stride < 0) return fail(BA_ERR_OUT_OF_RANGE, "schedule stride < 0");
  if (s.kind == BA_SCHED_FLOW) {
    if (!(s.shift > 0.0) || !(s.shift <= 1e6)) return fail(BA_ERR_OUT_OF_RANGE, "need 0 < shift <= 1e6");
    return BA_OK;
  }
  if (s.kind != BA_SCHED_DDIM) return fail(BA_ERR_INVALID_ARG, "schedule kind %d unknown", s.kind);
  if (!(s.beta_start > 0.0) || !(s.beta_end >= s.beta_start) || !(s.beta_end < 1.0))
    return fail(BA_ERR_OUT_OF_RANGE, "need 0 < beta_start <= beta_end < 1");
  return BA_OK;
}

// Flow matching: noise level of timestep t, sigma = shift u / (1 + (shift - 1) u), u = t / T.
double flow_sigma(const ba_schedule& s, int t) {
  const double u = (double)t / (double)s.T;
  return s.shift * u / (1.0 + (s.shift - 1.0) * u);
}

// abar_0..abar_T of the DDPM linear beta schedule, in fp64.
std::vector<double> alpha_bar(const ba_schedule& s) {
  std::vector<double> ab(s.T + 1);
  ab[0] = 1.0;
  double acc = 1.0;
  for (int i = 1; i <= s.T; ++i) {
    const double beta = s.beta_start + (s.beta_end - s.beta_start) * (double)(i - 1) / (double)(s.T - 1);
    acc *= 1.0 - beta;
    ab[i] = acc;
  }
  return ab;
}

// DDIM (eta = 0) from t to t' = max(t - stride, 0), folded into x' = c1 x + c2 eps.
void coefficients(const std::vector<double>& ab, int stride, int t, float* c1, float* c2) {
  const int tp = t - stride > 0 ? t - stride : 0;
  const double at = ab[t], ap = ab[tp];
  *c1 = (float)sqrt(ap / at);
  *c2 = (float)(sqrt(1.0 - ap) - sqrt(ap) * sqrt(1.0 - at) / sqrt(at));
}

// Workgroups of the bf16 attention kernel (launch shape `shape`) the current
// device holds at once.  The answer depends only on the device and the
// kernel, so it is asked once per (device, head dim, shape) and kept.
constexpr int kCachedDevices = 64;
std::atomic<int> g_resident[kCachedDevices][2][3];
std::once_flag g_resident_init;

hipError_t resident_workgroups(int head_dim, int shape, int* n) {
  std::call_once(g_resident_init, [] {
    for (auto& d : g_resident)
      for (auto& h : d)
        for (auto& x : h) x.store(-1, std::memory_order_relaxed);
  });
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *n = 0;
    return e;
  }
  std::atomic<int>* slot =
      dev >= 0 && dev < kCachedDevices && shape >= 0 && shape < 3 ? &g_resident[dev][head_dim == 128][shape] : nullptr;
  if (slot != nullptr) {
    const int v = slot->load(std::memory_order_acquire);
    if (v >= 0) {
      *n = v;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = ba::attention_bf16_resident(head_dim, shape, &per_cu);
  *n = e == hipSuccess ? cus * per_cu : 0;
  if (e == hipSuccess && slot != nullptr) slot->store(*n, std::memory_order_release);
  return e;
}

}  // namespace

extern "C" {

const char* ba_status_string(ba_status s) {
  switch (s) {
    case BA_OK: return "BA_OK";
    case BA_ERR_INVALID_ARG: return "BA_ERR_INVALID_ARG";
    case BA_ERR_UNSUPPORTED: return "BA_ERR_UNSUPPORTED";
    case BA_ERR_OUT_OF_RANGE: return "BA_ERR_OUT_OF_RANGE";
    case BA_ERR_HIP: return "BA_ERR_HIP";
  }
  return "BA_ERR_UNKNOWN";
}

const char* ba_last_error(void) { return g_err; }

int32_t ba_version(void) { return 1 * 10000 + 4 * 100 + 0; }

size_t ba_ring_bytes(int32_t n_slots, int32_t slot_tokens, int32_t heads, int32_t head_dim,
                     int32_t dtype) {
  if (check_shape(n_slots, slot_tokens, heads, head_dim, dtype) != BA_OK) return 0;
  return (size_t)n_slots * 2 * heads * (size_t)pad_tokens(slot_tokens) * head_dim * elem_bytes(dtype);
}

ba_status ba_ring_init(ba_ring* ring, void* base, size_t bytes, int32_t n_slots, int32_t slot_tokens,
                       int32_t heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  if (ring == nullptr) return fail(BA_ERR_INVALID_ARG, "ring is NULL");
  ba_status st = check_shape(n_slots, slot_tokens, heads, head_dim, dtype);
  if (st != BA_OK) return st;
  if (base == nullptr) return fail(BA_ERR_INVALID_ARG, "base is NULL");
  if (!aligned(base, 256)) return fail(BA_ERR_INVALID_ARG, "base not 256-byte aligned");
  const size_t need = ba_ring_bytes(n_slots, slot_tokens, heads, head_dim, dtype);
  if (bytes < need) return fail(BA_ERR_INVALID_ARG, "ring buffer has %zu bytes, needs %zu", bytes, need);
  hipError_t e = ba::launch_zero_fill(base, need, stream);
  if (e != hipSuccess) return hip_fail(e, "zero fill launch");
  ring->base = base;
  ring->n_slots = n_slots;
  ring->slot_tokens = slot_tokens;
  ring->heads = heads;
  ring->head_dim = head_dim;
  ring->dtype = dtype;
  ring->slot_stride_tokens = (int32_t)pad_tokens(slot_tokens);
  ring->appended = 0;
  return ok();
}

static ba_status append_common(const ba_ring* ring, const void* k, const void* v, int32_t n_tokens,
                               const int32_t* slots, int32_t n_blocks, hipStream_t stream) {
  ba_status st = check_ring(ring, "ring");
  if (st != BA_OK) return st;
  if (k == nullptr || v == nullptr) return fail(BA_ERR_INVALID_ARG, "k or v is NULL");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(BA_ERR_INVALID_ARG, "k or v not 16-byte aligned");
  if (n_tokens < 1 || n_tokens > ring->slot_tokens)
    return fail(BA_ERR_OUT_OF_RANGE, "n_tokens %d outside [1, %d]", n_tokens, ring->slot_tokens);
  for (int i = 0; i < n_blocks; ++i) {
    if (slots[i] < 0 || slots[i] >= ring->n_slots)
      return fail(BA_ERR_OUT_OF_RANGE, "slot %d outside [0, %d)", slots[i], ring->n_slots);
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return fail(BA_ERR_INVALID_ARG, "slot %d written twice in one call", slots[i]);
  }
  const int eb = elem_bytes(ring->dtype);
  const int64_t block_elems = (int64_t)n_tokens * ring->heads * ring->head_dim;
  for (int first = 0; first < n_blocks; first += ba::kAppendMaxBlocks) {
    ba::AppendArgs a;
    memset(&a, 0, sizeof(a));
    a.n_blocks = n_blocks - first < ba::kAppendMaxBlocks ? n_blocks - first : ba::kAppendMaxBlocks;
    a.k = static_cast<const char*>(k) + first * block_elems * eb;
    a.v = static_cast<const char*>(v) + first * block_elems * eb;
    a.ring = ring->base;
    a.src_tok = (int64_t)ring->heads * ring->head_dim;   // token-major [n_tokens][heads][head_dim]
    a.src_head = ring->head_dim;
    a.n_tokens = n_tokens;
    a.heads = ring->heads;
    a.t_pad = ring->slot_stride_tokens;
    for (int i = 0; i < a.n_blocks; ++i) a.slot[i] = slots[first + i];
    hipError_t e = ba::launch_append(a, ring->head_dim, eb, stream);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  return ok();
}

ba_status ba_cache_append(ba_ring* ring, const void* k, const void* v, int32_t n_tokens,
                          int32_t* slot_out, hipStream_t stream) {
  ba_status st = check_ring(ring, "ring");
  if (st != BA_OK) return st;
  const int32_t slot = (int32_t)(ring->appended % ring->n_slots);
  st = append_common(ring, k, v, n_tokens, &slot, 1, stream);
  if (st != BA_OK) return st;
  ring->appended += 1;
  if (slot_out) *slot_out = slot;
  return ok();
}

ba_status ba_cache_append_batched(const ba_ring* ring, const void* k, const void* v, int32_t n_tokens,
                                  const int32_t* slots, int32_t n_blocks, hipStream_t stream) {
  if (n_blocks < 0) return fail(BA_ERR_INVALID_ARG, "n_blocks < 0");
  if (n_blocks > 0 && slots == nullptr) return fail(BA_ERR_INVALID_ARG, "slots is NULL");
  if (n_blocks > 4096) return fail(BA_ERR_OUT_OF_RANGE, "n_blocks %d > 4096", n_blocks);
  if (n_blocks == 0) {
    ba_status st = check_ring(ring, "ring");
    return st != BA_OK ? st : ok();
  }
  return append_common(ring, k, v, n_tokens, slots, n_blocks, stream);
}

int32_t ba_attention_query_tile(int32_t head_dim, int32_t dtype, int32_t max_keys) {
  if ((head_dim != 64 && head_dim != 128) || max_keys < 0) return 0;
  if (dtype == BA_BF16)
    return ba::attention_bf16_q_tile(head_dim, ba::attention_bf16_shape(head_dim, max_keys,
                                                                        (max_keys + ba::kKeyTile - 1) / ba::kKeyTile));
  if (dtype == BA_F32) return ba::attention_f32_q_tile();
  return 0;
}

size_t ba_attention_workspace_bytes(int32_t head_dim, int32_t dtype, int32_t n_blocks, int32_t q_stride,
                                    int32_t heads) {
  if (dtype != BA_BF16 || (head_dim != 64 && head_dim != 128) || n_blocks < 1 || q_stride < 1 || heads < 1)
    return 0;
  // two partial results per tail workgroup, one tail workgroup per resident
  // slot; enough for either launch shape
  size_t bytes = 0;
  for (int shape = 0; shape < (head_dim == 64 ? 2 : 1); ++shape) {   // the resident shape takes none
    int wg = 0;
    if (resident_workgroups(head_dim, shape, &wg) != hipSuccess || wg < 1) return 0;
    const size_t b = (size_t)2 * (wg / 8 * 8) * ba::attention_partial_bytes(head_dim, shape);
    if (b > bytes) bytes = b;
  }
  return bytes;
}

}  // extern "C"

namespace {

// Block b's segment table for the kernels: zero-length segments dropped, the
// text last (slot -1 - text_slot).  *keys receives the block's key count (0
// for a block without queries).  The checks of one meta entry.
ba_status block_table(const ba_block_meta& m, int b, int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                      ba::AttnBlock* out, int64_t* keys_out) {
  ba::AttnBlock& B = *out;
  memset(&B, 0, sizeof(B));
  if (m.q_len < 0 || m.q_len > q_stride)
    return fail(BA_ERR_OUT_OF_RANGE, "block %d: q_len %d outside [0, %d]", b, m.q_len, q_stride);
  if (m.n_segs < 0 || m.n_segs > BA_MAX_SEGS)
    return fail(BA_ERR_OUT_OF_RANGE, "block %d: n_segs %d outside [0, %d]", b, m.n_segs, BA_MAX_SEGS);
  B.q_len = m.q_len;
  int64_t keys = 0;
  for (int i = 0; i < m.n_segs; ++i) {
    const ba_seg& sg = m.seg[i];
    if (sg.slot < 0 || sg.slot >= cache->n_slots)
      return fail(BA_ERR_OUT_OF_RANGE, "block %d seg %d: slot %d outside [0, %d)", b, i, sg.slot, cache->n_slots);
    if (sg.len < 0 || sg.len > cache->slot_tokens)
      return fail(BA_ERR_OUT_OF_RANGE, "block %d seg %d: len %d outside [0, %d]", b, i, sg.len, cache->slot_tokens);
    if (sg.len == 0) continue;
    B.slot[B.n_segs] = sg.slot;
    B.len[B.n_segs] = sg.len;
    ++B.n_segs;
    keys += sg.len;
  }
  if (m.text_len != 0) {
    if (text == nullptr) return fail(BA_ERR_INVALID_ARG, "text_len > 0 but text ring is NULL");
    if (m.text_len < 0 || m.text_len > text->slot_tokens)
      return fail(BA_ERR_OUT_OF_RANGE, "block %d: text_len %d outside [0, %d]", b, m.text_len, text->slot_tokens);
    if (m.text_slot < 0 || m.text_slot >= text->n_slots)
      return fail(BA_ERR_OUT_OF_RANGE, "block %d: text_slot %d outside [0, %d)", b, m.text_slot, text->n_slots);
    B.slot[B.n_segs] = -1 - m.text_slot;
    B.len[B.n_segs] = m.text_len;
    ++B.n_segs;
    keys += m.text_len;
  }
  if (m.q_len > 0 && keys == 0) return fail(BA_ERR_INVALID_ARG, "block %d has queries but no keys", b);
  *keys_out = m.q_len > 0 ? keys : 0;
  return BA_OK;
}

// The work of ba_block_attention after the pointer checks.  With plan != NULL
// nothing is launched: *plan receives the most tail workgroups per XCD any of
// the call's launches would use (0: every workgroup runs whole tasks).
ba_status attention_run(const void* q, int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                        const ba_block_meta* meta, int32_t n_blocks, float scale, void* out, float* lse,
                        bool has_workspace, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        int32_t* plan) {
  ba_status st = check_ring(cache, "cache");
  if (st != BA_OK) return st;
  if (n_blocks < 0) return fail(BA_ERR_INVALID_ARG, "n_blocks < 0");
  if (n_blocks > 0 && meta == nullptr) return fail(BA_ERR_INVALID_ARG, "meta is NULL");
  if (q_stride < 1) return fail(BA_ERR_INVALID_ARG, "q_stride < 1");
  if (!isfinite(scale)) return fail(BA_ERR_INVALID_ARG, "scale is not finite");
  if (plan) *plan = 0;
  bool need_text = false;
  for (int b = 0; b < n_blocks; ++b) need_text |= meta[b].text_len != 0;
  if (text != nullptr || need_text) {
    if (need_text && text == nullptr) return fail(BA_ERR_INVALID_ARG, "text_len > 0 but text ring is NULL");
    st = check_ring(text, "text");
    if (st != BA_OK) return st;
    if (text->heads != cache->heads || text->head_dim != cache->head_dim || text->dtype != cache->dtype)
      return fail(BA_ERR_INVALID_ARG, "text ring heads/head_dim/dtype differ from the cache ring");
  }
  const int D = cache->head_dim;
  const int H = cache->heads;
  if ((int64_t)n_blocks * q_stride * H > (int64_t)1 << 40) return fail(BA_ERR_OUT_OF_RANGE, "q too large");
  // the bf16 kernel's per-lane copy offsets within a ring matrix are 32-bit
  if (cache->dtype == BA_BF16) {
    if (cache->slot_stride_tokens >= ba::kAttnMaxSlotStride)
      return fail(BA_ERR_OUT_OF_RANGE, "cache slot stride %d tokens >= %lld (bf16 attention limit)",
                  cache->slot_stride_tokens, (long long)ba::kAttnMaxSlotStride);
    if (text != nullptr && text->slot_stride_tokens >= ba::kAttnMaxSlotStride)
      return fail(BA_ERR_OUT_OF_RANGE, "text slot stride %d tokens >= %lld (bf16 attention limit)",
                  text->slot_stride_tokens, (long long)ba::kAttnMaxSlotStride);
  }

  // every block's segment table is checked before anything is launched
  int32_t q_max = 0;
  for (int b = 0; b < n_blocks; ++b) {
    ba::AttnBlock B;
    int64_t keys = 0;
    st = block_table(meta[b], b, q_stride, cache, text, &B, &keys);
    if (st != BA_OK) return st;
    if (meta[b].q_len > q_max) q_max = meta[b].q_len;
  }
  if (n_blocks == 0 || q_max == 0) return ok();

  const bool bf16 = cache->dtype == BA_BF16;
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
  const int eb = elem_bytes(cache->dtype);
  for (int first = 0; first < n_blocks; first += ba::kAttnMaxBlocks) {
    const int nb = n_blocks - first < ba::kAttnMaxBlocks ? n_blocks - first : ba::kAttnMaxBlocks;
    // this launch's segment tables (checked above); launch shape from its
    // longest key set
    ba::AttnBlock tables[ba::kAttnMaxBlocks];
    int64_t max_keys = 0, max_tiles = 0;
    for (int i = 0; i < nb; ++i) {
      int64_t keys = 0, tiles = 0;
      block_table(meta[first + i], first + i, q_stride, cache, text, &tables[i], &keys);
      if (keys > max_keys) max_keys = keys;
      if (keys > 0)
        for (int sg = 0; sg < tables[i].n_segs; ++sg) tiles += (tables[i].len[sg] + ba::kKeyTile - 1) / ba::kKeyTile;
      if (tiles > max_tiles) max_tiles = tiles;
    }
    int shape = bf16 ? ba::attention_bf16_shape(D, max_keys, max_tiles) : 0;
    if (shape == 2) {
      // the resident shape pays a key-set copy per workgroup up front: with
      // fewer units of 32 queries than the device has wave slots (measured:
      // 1512 and 2256 units on 3072 slots ran 15-19 % slower than the narrow
      // shape, 3072 and more 4-15 % faster) the narrow shape is taken
      int64_t units = 0;
      for (int i = 0; i < nb; ++i) units += (int64_t)H * ((tables[i].q_len + 31) / 32);
      int wg = 0;
      hipError_t e = resident_workgroups(D, shape, &wg);
      if (e != hipSuccess && !plan) return hip_fail(e, "device query");
      if (e == hipSuccess && units < (int64_t)wg * ba::kResWaves) shape = 1;
    }
    const int qtile = bf16 ? ba::attention_bf16_q_tile(D, shape) : ba::attention_f32_q_tile();
    int resident = 0;   // workgroups the device holds at once (split schedule)
    if (bf16 && has_workspace && shape != 2) {
      hipError_t e = resident_workgroups(D, shape, &resident);
      if (e != hipSuccess) return hip_fail(e, "device query");
    }
    ba::AttnArgs a;
    memset(&a, 0, sizeof(a));
    int32_t qm = 0;
    int64_t tasks = 0, work = 0;
    for (int i = 0; i < nb; ++i) {
      ba::AttnBlock& B = a.blk[i];
      B = tables[i];
      if (B.q_len > qm) qm = B.q_len;
      B.nqt = (B.q_len + qtile - 1) / qtile;
      for (int sg = 0; sg < B.n_segs; ++sg) B.n_tiles += (B.len[sg] + ba::kKeyTile - 1) / ba::kKeyTile;
      B.task_start = (int32_t)tasks;
      B.work_start = (int32_t)work;
      tasks += (int64_t)H * B.nqt;
      work += (int64_t)H * B.nqt * B.n_tiles;
      if (work >= ((int64_t)1 << 31) || tasks >= ((int64_t)1 << 30))
        return fail(BA_ERR_OUT_OF_RANGE, "too much attention work in one call");
    }
    if (qm == 0) continue;
    const int64_t blk_elems = (int64_t)q_stride * H * D;
    a.q = q ? static_cast<const char*>(q) + first * blk_elems * eb : nullptr;
    a.out = out ? static_cast<char*>(out) + first * blk_elems * eb : nullptr;
    a.lse = lse ? lse + (int64_t)first * H * q_stride : nullptr;
    a.cache = cache->base;
    a.text = text ? text->base : nullptr;
    a.cache_tpad = cache->slot_stride_tokens;
    a.text_tpad = text ? text->slot_stride_tokens : 0;
    a.q_stride = q_stride;
    a.heads = H;
    a.n_blocks = nb;
    a.qscale = (float)((double)sc * 1.4426950408889634);
    a.scale_ln = sc;
    // fp32 kernel: one workgroup per (block, head, query tile)
    a.n_qtiles = (qm + qtile - 1) / qtile;
    a.total_tasks = nb * H * a.n_qtiles;
    a.tasks_per_xcd = (a.total_tasks + 7) / 8;
    // bf16 kernel: one task per workgroup, or (with a workspace) equal ranges
    // of task tiles over the workgroups the device holds at once
    a.n_tasks = (int32_t)tasks;
    a.total_work = (int32_t)work;
    a.wg_per_xcd = (int32_t)((tasks + 7) / 8);   // default: one whole task per workgroup
    if (resident > 0) {
      const size_t pb = ba::attention_partial_bytes(D, shape);
      int64_t tail = resident / 8;           // tail workgroups per XCD: one per resident slot
      const int64_t fit = (int64_t)(workspace_bytes / (16 * pb));
      // whole tasks alone: the busiest XCD's last round leaves `idle` of its
      // resident slots empty.  Cutting tasks costs about a fifth of a round
      // (partial stores, merge launch), so a nearly full last round is left
      // alone.
      const int64_t slots = resident / 8;
      const int64_t per_xcd = (tasks + 7) / 8;
      const int64_t idle = slots >= 1 ? (per_xcd + slots - 1) / slots * slots - per_xcd : 0;
      const bool worth = slots >= 1 && idle * kSplitIdleDen >= slots * kSplitIdleNum;
      if (tail > fit) tail = fit;
      if (worth && tail >= 1 && tasks >= 8 * tail) {
        a.split = 1;
        a.tail_wg = (int32_t)tail;
        a.partials = static_cast<float*>(workspace);
        int whole_max = 0, tail_tasks_max = 0;
        int64_t tail_tiles_max = 0;
        for (int x = 0; x < 8; ++x) {
          const ba::XcdPlan p = ba::xcd_plan(a, x);
          if (p.whole > whole_max) whole_max = p.whole;
          if (p.t1 - p.t0 - p.whole > tail_tasks_max) tail_tasks_max = p.t1 - p.t0 - p.whole;
          if (p.tail1 - p.tail0 > tail_tiles_max) tail_tiles_max = p.tail1 - p.tail0;
        }
        a.wg_per_xcd = whole_max + a.tail_wg;
        a.merge_per_xcd = tail_tasks_max;
        // short tasks (a text-only key set, a few hundred keys) would be cut
        // into pieces of a few tiles: the partial stores and the merge launch
        // then cost more than the idle end of the last round
        if (tail_tiles_max < (int64_t)kSplitMinTilesPerWg * tail) {
          a.split = 0;
          a.tail_wg = 0;
          a.partials = nullptr;
          a.merge_per_xcd = 0;
          a.wg_per_xcd = (int32_t)((tasks + 7) / 8);
        }
      }
    }
    if (plan) {
      if (a.tail_wg > *plan) *plan = a.tail_wg;
      continue;
    }
    if (shape == 2) {
      // resident key sets: the units (tasks of 32 queries) in equal
      // contiguous ranges, one per workgroup the device holds at once (no
      // workspace)
      int wg = 0;
      hipError_t e = resident_workgroups(D, shape, &wg);
      if (e != hipSuccess) return hip_fail(e, "device query");
      if (wg < 8) wg = 8;
      const int64_t per_xcd = ((tasks < wg ? tasks : wg) + 7) / 8;
      a.wg_per_xcd = (int32_t)per_xcd;
      // Contiguous ranges cross (block, head) boundaries, and a crossing
      // workgroup copies a second key set (~5 us).  When every block has as
      // many units per head, each (block, head) can take two or more whole
      // workgroups, and that needs no more rounds of units per wave than the
      // contiguous ranges, the workgroups are dealt per (block, head)
      // instead (measured at 24 heads x 64, 512 text keys: one block of 5400
      // queries 0.0275 against 0.0317 ms, of 4200 0.0237 against 0.0280; at
      // 8192 queries the rounds rule keeps the contiguous ranges, 2 % faster).
      const int64_t n_wg = 8 * per_xcd, groups = (int64_t)nb * H, nu = a.blk[0].nqt;
      bool same = nu > 0;
      for (int i = 1; i < nb; ++i) same = same && a.blk[i].nqt == nu;
      if (same && n_wg >= 2 * groups) {
        const int64_t contiguous = (tasks + n_wg - 1) / n_wg;          // most units of a workgroup
        const int64_t per_group = n_wg / groups;                        // fewest workgroups of a group
        const int64_t aligned = (nu + per_group - 1) / per_group;
        const int64_t nw = ba::kResWaves;
        if ((aligned + nw - 1) / nw <= (contiguous + nw - 1) / nw) a.res_group_units = (int32_t)nu;
      }
    }
    hipError_t e = bf16 ? ba::launch_attention_bf16(a, D, shape, stream) : ba::launch_attention_f32(a, D, stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
  }
  return ok();
}

}  // namespace

extern "C" {

ba_status ba_block_attention(const void* q, int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                             const ba_block_meta* meta, int32_t n_blocks, float scale, void* out,
                             float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (q == nullptr || out == nullptr) return fail(BA_ERR_INVALID_ARG, "q or out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(BA_ERR_INVALID_ARG, "q or out not 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(BA_ERR_INVALID_ARG, "lse not 4-byte aligned");
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(BA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  return attention_run(q, q_stride, cache, text, meta, n_blocks, scale, out, lse, workspace != nullptr,
                       workspace, workspace_bytes, stream, nullptr);
}

// ---- text K/V as plain arrays -------------------------------------------------

ba_status ba_text_ring_set(const ba_ring* text, int32_t slot, const void* text_k, const void* text_v,
                           int32_t text_cap, int32_t text_len, hipStream_t stream) {
  ba_status st = check_ring(text, "text");
  if (st != BA_OK) return st;
  if (text_k == nullptr || text_v == nullptr) return fail(BA_ERR_INVALID_ARG, "text_k or text_v is NULL");
  if (!aligned(text_k, 16) || !aligned(text_v, 16))
    return fail(BA_ERR_INVALID_ARG, "text_k or text_v not 16-byte aligned");
  if (slot < 0 || slot >= text->n_slots)
    return fail(BA_ERR_OUT_OF_RANGE, "slot %d outside [0, %d)", slot, text->n_slots);
  if (text_cap < 1 || (int64_t)text_cap * text->heads * text->head_dim >= ((int64_t)1 << 40))
    return fail(BA_ERR_OUT_OF_RANGE, "text_cap %d out of range", text_cap);
  if (text_len < 1 || text_len > text_cap || text_len > text->slot_tokens)
    return fail(BA_ERR_OUT_OF_RANGE, "text_len %d outside [1, min(text_cap %d, slot_tokens %d)]", text_len,
                text_cap, text->slot_tokens);
  ba::AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.k = text_k;
  a.v = text_v;
  a.ring = text->base;
  a.src_tok = text->head_dim;                           // head-major [heads][text_cap][head_dim]
  a.src_head = (int64_t)text_cap * text->head_dim;
  a.n_tokens = text_len;
  a.heads = text->heads;
  a.t_pad = text->slot_stride_tokens;
  a.n_blocks = 1;
  a.slot[0] = slot;
  hipError_t e = ba::launch_append(a, text->head_dim, elem_bytes(text->dtype), stream);
  if (e != hipSuccess) return hip_fail(e, "text copy launch");
  return ok();
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ba_attention_text_arrays_workspace_bytes(int32_t head_dim, int32_t dtype, int32_t n_blocks,
                                                int32_t q_stride, int32_t heads, int32_t text_cap) {
  const size_t ring = ba_ring_bytes(1, text_cap, heads, head_dim, dtype);
  if (ring == 0) return 0;
  return round256(ring) + ba_attention_workspace_bytes(head_dim, dtype, n_blocks, q_stride, heads);
}

ba_status ba_block_attention_text_arrays(const void* q, int32_t q_stride, const ba_ring* cache,
                                         const void* text_k, const void* text_v, int32_t text_cap,
                                         const ba_block_meta* meta, int32_t n_blocks, float scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (q == nullptr || out == nullptr) return fail(BA_ERR_INVALID_ARG, "q or out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(BA_ERR_INVALID_ARG, "q or out not 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(BA_ERR_INVALID_ARG, "lse not 4-byte aligned");
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(BA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  ba_status st = check_ring(cache, "cache");
  if (st != BA_OK) return st;
  if (n_blocks > 0 && meta == nullptr) return fail(BA_ERR_INVALID_ARG, "meta is NULL");
  int32_t max_len = 0;
  for (int b = 0; b < n_blocks; ++b)
    if (meta[b].text_len > max_len) max_len = meta[b].text_len;
  if (max_len == 0)   // no block reads the text: plain block attention
    return attention_run(q, q_stride, cache, nullptr, meta, n_blocks, scale, out, lse, workspace != nullptr,
                         workspace, workspace_bytes, stream, nullptr);
  if (text_k == nullptr || text_v == nullptr) return fail(BA_ERR_INVALID_ARG, "text_len > 0 but text_k or text_v is NULL");
  if (!aligned(text_k, 16) || !aligned(text_v, 16))
    return fail(BA_ERR_INVALID_ARG, "text_k or text_v not 16-byte aligned");
  const size_t ring = ba_ring_bytes(1, text_cap, cache->heads, cache->head_dim, cache->dtype);
  if (ring == 0) return fail(BA_ERR_OUT_OF_RANGE, "text_cap %d out of range", text_cap);
  const size_t rb = round256(ring);
  if (workspace == nullptr || workspace_bytes < rb)
    return fail(BA_ERR_INVALID_ARG, "workspace of %zu bytes cannot hold the text ring (%zu bytes)",
                workspace == nullptr ? (size_t)0 : workspace_bytes, rb);
  // the text ring at the start of the workspace, the rest for the split
  // schedule's partial results
  ba_ring tr;
  memset(&tr, 0, sizeof(tr));
  tr.base = workspace;
  tr.n_slots = 1;
  tr.slot_tokens = text_cap;
  tr.heads = cache->heads;
  tr.head_dim = cache->head_dim;
  tr.dtype = cache->dtype;
  tr.slot_stride_tokens = (int32_t)pad_tokens(text_cap);
  void* rest = workspace_bytes > rb ? static_cast<char*>(workspace) + rb : nullptr;
  const size_t rest_bytes = workspace_bytes > rb ? workspace_bytes - rb : 0;
  // every check of the attention call (key sets, text_len <= text_cap,
  // text_slot 0) before anything is launched
  int32_t plan = 0;
  st = attention_run(q, q_stride, cache, &tr, meta, n_blocks, scale, out, lse, rest != nullptr, rest, rest_bytes,
                     stream, &plan);
  if (st != BA_OK) return st;
  st = ba_text_ring_set(&tr, 0, text_k, text_v, text_cap, max_len, stream);
  if (st != BA_OK) return st;
  return attention_run(q, q_stride, cache, &tr, meta, n_blocks, scale, out, lse, rest != nullptr, rest, rest_bytes,
                       stream, nullptr);
}

ba_status ba_attention_plan(int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                            const ba_block_meta* meta, int32_t n_blocks, size_t workspace_bytes,
                            int32_t* tail_workgroups) {
  if (tail_workgroups == nullptr) return fail(BA_ERR_INVALID_ARG, "tail_workgroups is NULL");
  return attention_run(nullptr, q_stride, cache, text, meta, n_blocks, 0.f, nullptr, nullptr,
                       workspace_bytes > 0, nullptr, workspace_bytes, nullptr, tail_workgroups);
}

}  // extern "C"

// ---- block attention without allocation ---------------------------------------
// The split schedule's partial results live in the library's own device array
// (one copy per GPU: a __device__ variable exists on every device the code
// object is loaded on).  72 MiB holds two partial results for every workgroup
// slot of a 256-CU device at either head dim (the most is 66 MiB, head_dim
// 128).  Every call on a GPU shares that GPU's copy.
namespace {
constexpr size_t kScratchBytes = (size_t)72 << 20;
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchMaxDevices];   // device address of `scratch` per device, once known
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// The device address of the current device's `scratch`, looked up with that
// device current on its first use and kept (the array's name in host code is
// not a device address).
ba_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(BA_ERR_UNSUPPORTED, "device %d: the library keeps scratch for devices 0-%d", dev,
                kScratchMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(BA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BA_OK;
}
}  // namespace

extern "C" {

ba_status ba_block_attention_static(const void* q, int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                                    const ba_block_meta* meta, int32_t n_blocks, float scale, void* out,
                                    float* lse, hipStream_t stream) {
  if (q == nullptr || out == nullptr) return fail(BA_ERR_INVALID_ARG, "q or out is NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(BA_ERR_INVALID_ARG, "q or out not 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(BA_ERR_INVALID_ARG, "lse not 4-byte aligned");
  ba_status st = check_ring(cache, "cache");
  if (st != BA_OK) return st;
  if (cache->dtype != BA_BF16)   // the fp32 kernel uses no scratch
    return attention_run(q, q_stride, cache, text, meta, n_blocks, scale, out, lse, false, nullptr, 0, stream,
                         nullptr);
  const size_t need = ba_attention_workspace_bytes(cache->head_dim, cache->dtype, n_blocks > 0 ? n_blocks : 1,
                                                   q_stride > 0 ? q_stride : 1, cache->heads);
  if (need > kScratchBytes)
    return fail(BA_ERR_OUT_OF_RANGE, "this device needs %zu bytes of split-schedule scratch; the library holds %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != BA_OK) return st;
  return attention_run(q, q_stride, cache, text, meta, n_blocks, scale, out, lse, true, ws, kScratchBytes, stream,
                       nullptr);
}

ba_status ba_schedule_coefficients(const ba_schedule* sched, const int32_t* t, int32_t n, float* c1, float* c2) {
  ba_schedule s;
  schedule_or_default(sched, &s);
  ba_status st = check_schedule(s);
  if (st != BA_OK) return st;
  if (n < 0) return fail(BA_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (t == nullptr || c1 == nullptr || c2 == nullptr))
    return fail(BA_ERR_INVALID_ARG, "t, c1 or c2 is NULL");
  for (int i = 0; i < n; ++i)
    if (t[i] < 0 || t[i] > s.T) return fail(BA_ERR_OUT_OF_RANGE, "t[%d] = %d outside [0, %d]", i, t[i], s.T);
  if (s.kind == BA_SCHED_FLOW) {
    // one Euler step of the velocity: x' = x + (sigma(t') - sigma(t)) v
    for (int i = 0; i < n; ++i) {
      const int tp = t[i] - s.stride > 0 ? t[i] - s.stride : 0;
      c1[i] = 1.0f;
      c2[i] = (float)(flow_sigma(s, tp) - flow_sigma(s, t[i]));
    }
    return ok();
  }
  const std::vector<double> ab = alpha_bar(s);
  for (int i = 0; i < n; ++i) coefficients(ab, s.stride, t[i], &c1[i], &c2[i]);
  return ok();
}

ba_status ba_block_update(void* x, const void* eps, int64_t elems_per_block, const int32_t* t_per_block,
                          int32_t n_blocks, const ba_schedule* sched, hipStream_t stream) {
  if (n_blocks < 0) return fail(BA_ERR_INVALID_ARG, "n_blocks < 0");
  if (elems_per_block < 0) return fail(BA_ERR_INVALID_ARG, "elems_per_block < 0");
  // one thread per 8 elements, at most 2^31 - 1 workgroups of 256 threads
  if (elems_per_block > ((int64_t)1 << 40))
    return fail(BA_ERR_OUT_OF_RANGE, "elems_per_block %lld > 2^40", (long long)elems_per_block);
  if (n_blocks > 0 && t_per_block == nullptr) return fail(BA_ERR_INVALID_ARG, "t_per_block is NULL");
  if (x == nullptr || eps == nullptr) return fail(BA_ERR_INVALID_ARG, "x or eps is NULL");
  if (!aligned(x, 16) || !aligned(eps, 16)) return fail(BA_ERR_INVALID_ARG, "x or eps not 16-byte aligned");
  if (n_blocks > 65535) return fail(BA_ERR_OUT_OF_RANGE, "n_blocks %d > 65535", n_blocks);
  std::vector<float> c1(n_blocks), c2(n_blocks);
  ba_status st = ba_schedule_coefficients(sched, t_per_block, n_blocks, c1.data(), c2.data());
  if (st != BA_OK) return st;
  if (n_blocks == 0 || elems_per_block == 0) return ok();
  for (int first = 0; first < n_blocks; first += ba::kUpdateMaxBlocks) {
    ba::UpdateArgs a;
    memset(&a, 0, sizeof(a));
    a.n_blocks = n_blocks - first < ba::kUpdateMaxBlocks ? n_blocks - first : ba::kUpdateMaxBlocks;
    a.x = static_cast<uint16_t*>(x) + first * elems_per_block;
    a.eps = static_cast<const uint16_t*>(eps) + first * elems_per_block;
    a.elems = elems_per_block;
    for (int i = 0; i < a.n_blocks; ++i) {
      a.c1[i] = c1[first + i];
      a.c2[i] = c2[first + i];
    }
    hipError_t e = ba::launch_update(a, stream);
    if (e != hipSuccess) return hip_fail(e, "update launch");
  }
  return ok();
}

// ---- single-GPU FIFO block queue (host bookkeeping) -------------------------

int32_t ba_queue_ring_slots(int32_t n_queue) {
  return n_queue >= 1 && n_queue <= BA_QUEUE_MAX ? 2 * n_queue : 0;
}

ba_status ba_queue_init(ba_queue* q, int32_t n_queue, int32_t T, int32_t block_tokens, int32_t text_len) {
  if (q == nullptr) return fail(BA_ERR_INVALID_ARG, "q is NULL");
  if (n_queue < 1 || n_queue > BA_QUEUE_MAX)
    return fail(BA_ERR_OUT_OF_RANGE, "n_queue %d outside [1, %d]", n_queue, BA_QUEUE_MAX);
  if (T < 2 || T > 100000 || T % n_queue != 0)
    return fail(BA_ERR_OUT_OF_RANGE, "T = %d must be in [2, 100000] and a multiple of n_queue = %d", T, n_queue);
  if (block_tokens < 1) return fail(BA_ERR_OUT_OF_RANGE, "block_tokens < 1");
  if (text_len < 0) return fail(BA_ERR_OUT_OF_RANGE, "text_len < 0");
  q->n_queue = n_queue;
  q->T = T;
  q->block_tokens = block_tokens;
  q->text_len = text_len;
  q->step = 0;
  q->head_id = 0;
  return ok();
}

static ba_status check_queue(const ba_queue* q) {
  if (q == nullptr) return fail(BA_ERR_INVALID_ARG, "q is NULL");
  if (q->n_queue < 1 || q->n_queue > BA_QUEUE_MAX || q->T < 2 || q->T % q->n_queue != 0 ||
      q->block_tokens < 1 || q->text_len < 0 || q->step < 0 || q->head_id < 0)
    return fail(BA_ERR_INVALID_ARG, "q was not set up by ba_queue_init");
  return BA_OK;
}

ba_status ba_queue_plan(const ba_queue* q, int32_t* write_slots, ba_block_meta* meta, int32_t* t,
                        int32_t* stride) {
  ba_status st = check_queue(q);
  if (st != BA_OK) return st;
  if (write_slots == nullptr || meta == nullptr || t == nullptr || stride == nullptr)
    return fail(BA_ERR_INVALID_ARG, "an output array is NULL");
  const int64_t n = q->n_queue, g = q->step;
  const int32_t rung = q->T / q->n_queue;
  for (int64_t m = 0; m < n; ++m) {
    const int64_t i = ((m - q->head_id) % n + n) % n;      // queue position of latent slot m
    const int64_t k = q->head_id + i;                      // its block id
    write_slots[m] = (int32_t)(2 * (k % n) + (g % 2));
    ba_block_meta& b = meta[m];
    memset(&b, 0, sizeof(b));
    b.q_len = q->block_tokens;
    if (g > 0) {   // the neighbour toward the head wrote its K/V at step g - 1
      const int64_t kn = k - 1 + n;                        // k - 1, kept non-negative
      b.seg[b.n_segs].slot = (int32_t)(2 * (kn % n) + ((g - 1) % 2));
      b.seg[b.n_segs].len = q->block_tokens;
      ++b.n_segs;
    }
    b.seg[b.n_segs].slot = write_slots[m];
    b.seg[b.n_segs].len = q->block_tokens;
    ++b.n_segs;
    b.text_slot = 0;
    b.text_len = q->text_len;
    t[m] = (int32_t)((i + 1) * rung);
  }
  *stride = rung;
  return ok();
}

ba_status ba_queue_advance(ba_queue* q) {
  ba_status st = check_queue(q);
  if (st != BA_OK) return st;
  q->head_id += 1;
  q->step += 1;
  return ok();
}

// ---- fused K/V producer -----------------------------------------------------

ba_status ba_qkv_project_batched(const void* x, int32_t n_blocks, int32_t n_tokens, int32_t dim, const void* w,
                                 void* q, const ba_ring* cache, const int32_t* slots, const float* rope,
                                 int64_t rope_block_stride, hipStream_t stream) {
  ba_status st = check_ring(cache, "cache");
  if (st != BA_OK) return st;
  if (cache->dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "the producer writes bf16 rings only");
  if (x == nullptr || w == nullptr || slots == nullptr) return fail(BA_ERR_INVALID_ARG, "x, w or slots is NULL");
  if (!aligned(x, 16) || !aligned(w, 16) || (q && !aligned(q, 16)))
    return fail(BA_ERR_INVALID_ARG, "x, w or q not 16-byte aligned");
  if (rope && !aligned(rope, 8)) return fail(BA_ERR_INVALID_ARG, "rope not 8-byte aligned");
  if (n_blocks < 1 || n_blocks > ba::kProjMaxBlocks)
    return fail(BA_ERR_OUT_OF_RANGE, "n_blocks %d outside [1, %d]", n_blocks, ba::kProjMaxBlocks);
  for (int b = 0; b < n_blocks; ++b) {
    if (slots[b] < 0 || slots[b] >= cache->n_slots)
      return fail(BA_ERR_OUT_OF_RANGE, "slots[%d] = %d outside [0, %d)", b, slots[b], cache->n_slots);
    for (int c = 0; c < b; ++c)
      if (slots[c] == slots[b]) return fail(BA_ERR_INVALID_ARG, "blocks %d and %d share slot %d", c, b, slots[b]);
  }
  if (n_tokens < 1 || n_tokens > cache->slot_tokens)
    return fail(BA_ERR_OUT_OF_RANGE, "n_tokens %d outside [1, %d]", n_tokens, cache->slot_tokens);
  if (dim < 64 || dim % 64 != 0 || (int64_t)n_tokens * dim >= ((int64_t)1 << 30))
    return fail(BA_ERR_OUT_OF_RANGE, "dim %d must be a positive multiple of 64 (n_tokens * dim < 2^30)", dim);
  const int64_t n_ch = 3 * (int64_t)cache->heads * cache->head_dim;
  if (n_ch * dim >= ((int64_t)1 << 30)) return fail(BA_ERR_OUT_OF_RANGE, "weight too large");
  const int64_t table = (int64_t)n_tokens * cache->head_dim;   // floats of one block's table
  if (rope && rope_block_stride != 0 && rope_block_stride < table)
    return fail(BA_ERR_INVALID_ARG, "rope_block_stride %lld is neither 0 nor >= one table (%lld floats)",
                (long long)rope_block_stride, (long long)table);
  ba::ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.q = static_cast<uint16_t*>(q);
  a.ring = static_cast<uint16_t*>(cache->base);
  a.rope = rope;
  a.rope_bstride = rope ? rope_block_stride : 0;
  a.n_tokens = n_tokens;
  a.dim = dim;
  a.heads = cache->heads;
  a.t_pad = cache->slot_stride_tokens;
  a.n_ch = (int32_t)n_ch;
  a.ch_begin = q ? 0 : cache->heads * cache->head_dim;
  a.n_blocks = n_blocks;
  for (int b = 0; b < n_blocks; ++b) a.slot[b] = slots[b];
  hipError_t e = ba::launch_project(a, cache->head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return ok();
}

ba_status ba_qkv_project(const void* x, int32_t n_tokens, int32_t dim, const void* w, void* q,
                         const ba_ring* cache, int32_t slot, const float* rope, hipStream_t stream) {
  return ba_qkv_project_batched(x, 1, n_tokens, dim, w, q, cache, &slot, rope, 0, stream);
}

}  // extern "C"

// ---- coordinated noise initialisation -------------------------------------

namespace {

static_assert(ba::kNoiseMaxFrames == BA_NOISE_MAX_FRAMES, "kernarg frame table");

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): a Weyl sequence with
// increment 0x9E3779B97F4A7C15 whose states pass through a 64-bit finaliser.
struct Mix64 {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // uniform in [0, n): words below 2^64 mod n are rejected (no modulo bias)
  uint64_t below(uint64_t n) {
    const uint64_t threshold = (0 - n) % n;
    for (;;) {
      const uint64_t r = next();
      if (r >= threshold) return r % n;
    }
  }
};

}  // namespace

extern "C" {

ba_status ba_noise_assign(uint64_t seed, int64_t block_id, int32_t pool_frames, int32_t n_exclude,
                          int32_t block_frames, int32_t* frames) {
  if (frames == nullptr) return fail(BA_ERR_INVALID_ARG, "frames is NULL");
  if (block_id < 0) return fail(BA_ERR_OUT_OF_RANGE, "block_id < 0");
  if (pool_frames < 1 || n_exclude < 0 || n_exclude >= pool_frames)
    return fail(BA_ERR_OUT_OF_RANGE, "need pool_frames >= 1 and 0 <= n_exclude < pool_frames");
  const int32_t m = pool_frames - n_exclude;
  if (block_frames < 1 || block_frames > m || block_frames > BA_NOISE_MAX_FRAMES)
    return fail(BA_ERR_OUT_OF_RANGE, "block_frames %d outside [1, min(%d, %d)]", block_frames, m,
                BA_NOISE_MAX_FRAMES);
  // block b's seed: output b of the generator seeded with `seed`; the Weyl
  // state after b + 1 steps is seed + (b + 1) * gamma
  Mix64 root{seed + (uint64_t)block_id * 0x9E3779B97F4A7C15ull};
  Mix64 g{root.next()};
  std::vector<int32_t> a(m);
  for (int32_t i = 0; i < m; ++i) a[i] = i;
  for (int32_t i = 0; i < block_frames; ++i) {
    const int32_t j = i + (int32_t)g.below((uint64_t)(m - i));
    const int32_t t = a[i];
    a[i] = a[j];
    a[j] = t;
  }
  for (int32_t i = 0; i < block_frames; ++i) frames[i] = a[i];
  return ok();
}

ba_status ba_noise_block(const void* pool, int32_t channels, int32_t pool_frames, int64_t frame_bytes,
                         const int32_t* frames, int32_t block_frames, void* out, hipStream_t stream) {
  if (pool == nullptr || out == nullptr || frames == nullptr)
    return fail(BA_ERR_INVALID_ARG, "pool, out or frames is NULL");
  if (!aligned(pool, 16) || !aligned(out, 16)) return fail(BA_ERR_INVALID_ARG, "pool or out not 16-byte aligned");
  if (frame_bytes < 16 || frame_bytes % 16 != 0 || frame_bytes > ((int64_t)1 << 40))
    return fail(BA_ERR_INVALID_ARG, "frame_bytes %lld must be a positive multiple of 16 (<= 2^40)",
                (long long)frame_bytes);
  if (channels < 1 || pool_frames < 1) return fail(BA_ERR_OUT_OF_RANGE, "channels and pool_frames must be >= 1");
  if (block_frames < 1 || block_frames > BA_NOISE_MAX_FRAMES)
    return fail(BA_ERR_OUT_OF_RANGE, "block_frames %d outside [1, %d]", block_frames, BA_NOISE_MAX_FRAMES);
  if ((int64_t)channels * block_frames > 65535)
    return fail(BA_ERR_OUT_OF_RANGE, "channels * block_frames > 65535");
  for (int i = 0; i < block_frames; ++i)
    if (frames[i] < 0 || frames[i] >= pool_frames)
      return fail(BA_ERR_OUT_OF_RANGE, "frames[%d] = %d outside [0, %d)", i, frames[i], pool_frames);
  const uintptr_t p0 = (uintptr_t)pool, p1 = p0 + (uintptr_t)channels * pool_frames * frame_bytes;
  const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (uintptr_t)channels * block_frames * frame_bytes;
  if (o0 < p1 && p0 < o1) return fail(BA_ERR_INVALID_ARG, "out overlaps the pool");
  ba::NoiseArgs a;
  memset(&a, 0, sizeof(a));
  a.pool = static_cast<const unsigned int __attribute__((ext_vector_type(4)))*>(pool);
  a.out = static_cast<unsigned int __attribute__((ext_vector_type(4)))*>(out);
  a.frame_vecs = frame_bytes / 16;
  a.channels = channels;
  a.pool_frames = pool_frames;
  a.block_frames = block_frames;
  for (int i = 0; i < block_frames; ++i) a.frames[i] = frames[i];
  hipError_t e = ba::launch_noise(a, stream);
  if (e != hipSuccess) return hip_fail(e, "noise launch");
  return ok();
}

}  // extern "C"
