/*
 * A plain C caller of libblockattn: HIP runtime and the C ABI only, no
 * Python, no torch.  It builds a two-slot feature cache and a text ring,
 * appends a context block and the current block, runs block attention over
 * [context | current | text] and one DDIM update, and writes every input and
 * output to a binary file for the test that drives it to check against the
 * oracle.
 *
 * usage: abi_demo OUT_FILE
 * file:  int32 header {magic, L, H, D, TXT, E, t} then uint16 arrays q, k_ctx,
 *        v_ctx, k_cur, v_cur, k_txt, v_txt ([tokens][H][D] each), out
 *        ([L][H][D]), x, eps, x_after ([E] each); all bf16 bit patterns.
 *        Then the host bookkeeping, int32: the noise assignment of block 3
 *        (seed 7, pool 21, 3 excluded, 4 frames) and, for a 4-block queue
 *        (T 1000) at its third step, every block's write slot and timestep.
 *        Last, uint16: out2 ([L][H][D]), the same attention through
 *        ba_block_attention_text_arrays with the text given as
 *        [H][TXT][D] arrays.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "blockattn.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                              \
    }                                                                       \
  } while (0)
#define CHECK_BA(x)                                                         \
  do {                                                                      \
    ba_status s_ = (x);                                                     \
    if (s_ != BA_OK) {                                                      \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, ba_status_string(s_), ba_last_error()); \
      exit(3);                                                              \
    }                                                                       \
  } while (0)

/* xorshift64*: the inputs only need to be reproducible and modest in size */
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint16_t rand_bf16(float scale) {
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  const uint64_t r = g_state * 0x2545F4914F6CDD1Dull;
  const float u = (float)((r >> 40) & 0xFFFFFF) / 16777216.0f;   /* [0, 1) */
  const float f = (2.0f * u - 1.0f) * scale;
  uint32_t bits;
  memcpy(&bits, &f, 4);
  bits += 0x7FFFu + ((bits >> 16) & 1u);                           /* round to nearest even */
  return (uint16_t)(bits >> 16);
}

static uint16_t* host_fill(size_t n, float scale) {
  uint16_t* p = (uint16_t*)malloc(n * 2);
  for (size_t i = 0; i < n; ++i) p[i] = rand_bf16(scale);
  return p;
}

static void* to_device(const uint16_t* h, size_t n) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, n * 2));
  CHECK_HIP(hipMemcpy(d, h, n * 2, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
    return 1;
  }
  const int L = 200, H = 2, D = 64, TXT = 40;
  const int64_t E = (int64_t)L * 64;
  const int32_t t = 500;
  const size_t blk = (size_t)L * H * D, tblk = (size_t)TXT * H * D;
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  uint16_t* q = host_fill(blk, 1.0f);
  uint16_t* kc = host_fill(blk, 1.0f);
  uint16_t* vc = host_fill(blk, 1.0f);
  uint16_t* ku = host_fill(blk, 1.0f);
  uint16_t* vu = host_fill(blk, 1.0f);
  uint16_t* kt = host_fill(tblk, 1.0f);
  uint16_t* vt = host_fill(tblk, 1.0f);
  uint16_t* x = host_fill((size_t)E, 1.5f);
  uint16_t* eps = host_fill((size_t)E, 1.5f);

  /* the feature cache (two slots) and the text ring (one slot) */
  const size_t cache_bytes = ba_ring_bytes(2, L, H, D, BA_BF16);
  const size_t text_bytes = ba_ring_bytes(1, TXT, H, D, BA_BF16);
  void *cache_mem = NULL, *text_mem = NULL;
  CHECK_HIP(hipMalloc(&cache_mem, cache_bytes));
  CHECK_HIP(hipMalloc(&text_mem, text_bytes));
  ba_ring cache, text;
  CHECK_BA(ba_ring_init(&cache, cache_mem, cache_bytes, 2, L, H, D, BA_BF16, stream));
  CHECK_BA(ba_ring_init(&text, text_mem, text_bytes, 1, TXT, H, D, BA_BF16, stream));

  void *dq = to_device(q, blk), *dkc = to_device(kc, blk), *dvc = to_device(vc, blk);
  void *dku = to_device(ku, blk), *dvu = to_device(vu, blk);
  void *dkt = to_device(kt, tblk), *dvt = to_device(vt, tblk);
  void *dx = to_device(x, (size_t)E), *deps = to_device(eps, (size_t)E);
  void* dout = NULL;
  CHECK_HIP(hipMalloc(&dout, blk * 2));

  int32_t slot_ctx = -1, slot_cur = -1, slot_txt = -1;
  CHECK_BA(ba_cache_append(&cache, dkc, dvc, L, &slot_ctx, stream));   /* the neighbour's K/V */
  CHECK_BA(ba_cache_append(&cache, dku, dvu, L, &slot_cur, stream));   /* this block's */
  CHECK_BA(ba_cache_append(&text, dkt, dvt, TXT, &slot_txt, stream));

  ba_block_meta meta;
  memset(&meta, 0, sizeof(meta));
  meta.q_len = L;
  meta.n_segs = 2;
  meta.seg[0].slot = slot_ctx;
  meta.seg[0].len = L;
  meta.seg[1].slot = slot_cur;
  meta.seg[1].len = L;
  meta.text_slot = slot_txt;
  meta.text_len = TXT;
  CHECK_BA(ba_block_attention(dq, L, &cache, &text, &meta, 1, 0.0f, dout, NULL, NULL, 0, stream));
  CHECK_BA(ba_block_update(dx, deps, E, &t, 1, NULL, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  uint16_t* out = (uint16_t*)malloc(blk * 2);
  uint16_t* xa = (uint16_t*)malloc((size_t)E * 2);
  CHECK_HIP(hipMemcpy(out, dout, blk * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(xa, dx, (size_t)E * 2, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) {
    perror(argv[1]);
    return 4;
  }
  const int32_t hdr[7] = {0x62616331, L, H, D, TXT, (int32_t)E, t};
  fwrite(hdr, 4, 7, f);
  const uint16_t* arrays[] = {q, kc, vc, ku, vu, kt, vt, out, x, eps, xa};
  const size_t counts[] = {blk, blk, blk, blk, blk, tblk, tblk, blk, (size_t)E, (size_t)E, (size_t)E};
  for (int i = 0; i < 11; ++i) fwrite(arrays[i], 2, counts[i], f);

  /* host bookkeeping through the same ABI: a block's noise frames, a queue plan */
  int32_t frames[4];
  CHECK_BA(ba_noise_assign(7, 3, 21, 3, 4, frames));
  fwrite(frames, 4, 4, f);
  ba_queue q4;
  CHECK_BA(ba_queue_init(&q4, 4, 1000, L, TXT));
  int32_t wslots[4], tq[4], stride = 0;
  ba_block_meta qm[4];
  for (int g = 0; g < 2; ++g) {
    CHECK_BA(ba_queue_plan(&q4, wslots, qm, tq, &stride));
    CHECK_BA(ba_queue_advance(&q4));
  }
  CHECK_BA(ba_queue_plan(&q4, wslots, qm, tq, &stride));
  fwrite(wslots, 4, 4, f);
  fwrite(tq, 4, 4, f);

  /* the same attention with the text as plain head-major arrays: the text
     ring is made in the workspace */
  uint16_t* kt_hm = (uint16_t*)malloc(tblk * 2);
  uint16_t* vt_hm = (uint16_t*)malloc(tblk * 2);
  for (int tk = 0; tk < TXT; ++tk)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        kt_hm[((size_t)h * TXT + tk) * D + d] = kt[((size_t)tk * H + h) * D + d];
        vt_hm[((size_t)h * TXT + tk) * D + d] = vt[((size_t)tk * H + h) * D + d];
      }
  void *dkt_hm = to_device(kt_hm, tblk), *dvt_hm = to_device(vt_hm, tblk);
  const size_t ws_bytes = ba_attention_text_arrays_workspace_bytes(D, BA_BF16, 1, L, H, TXT);
  void *ws = NULL, *dout2 = NULL;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMalloc(&dout2, blk * 2));
  CHECK_BA(ba_block_attention_text_arrays(dq, L, &cache, dkt_hm, dvt_hm, TXT, &meta, 1, 0.0f, dout2, NULL, ws,
                                          ws_bytes, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  uint16_t* out2 = (uint16_t*)malloc(blk * 2);
  CHECK_HIP(hipMemcpy(out2, dout2, blk * 2, hipMemcpyDeviceToHost));
  fwrite(out2, 2, blk, f);
  fclose(f);
  printf("abi_demo ok: slots ctx %d cur %d text %d, library %d\n", slot_ctx, slot_cur, slot_txt, ba_version());
  return 0;
}
