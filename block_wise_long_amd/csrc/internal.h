// Internal launch interfaces between the C-ABI layer (api.cpp) and the HIP
// kernels.  Everything here is validated by the caller before it is called.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace ba {

constexpr int kTokenAlign = 64;          // ring slot stride granularity
constexpr int kKeyTile = 64;             // keys per attention tile (divides kTokenAlign)
constexpr int kAppendMaxBlocks = 64;     // slots per append launch (kernarg)
constexpr int kAttnMaxBlocks = 16;       // blocks per attention launch (kernarg)
constexpr int kAttnMaxSegs = 9;          // 8 cache segments + text
constexpr int kUpdateMaxBlocks = 64;     // blocks per update launch (kernarg)
// The bf16 attention kernel addresses a lane's V^T chunk of a ring matrix by
// a 32-bit byte offset below (32 * T_pad) * 2 from the segment's base: ring
// slot strides (T_pad) of bf16 rings it reads stay below this.
constexpr int64_t kAttnMaxSlotStride = (int64_t)1 << 26;

// ---- ring append -----------------------------------------------------------
struct AppendArgs {
  const void* k;            // block z's token t, head h at z*n_tokens*heads*D + t*src_tok + h*src_head
  const void* v;
  void* ring;               // ring base
  int64_t src_tok;          // elements between tokens: heads*D token-major, D head-major
  int64_t src_head;         // elements between heads: D token-major, cap*D head-major
  int32_t n_tokens;
  int32_t heads;
  int32_t t_pad;            // slot token stride
  int32_t n_blocks;
  int32_t slot[kAppendMaxBlocks];
};
hipError_t launch_append(const AppendArgs& a, int head_dim, int elem_bytes, hipStream_t s);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s);

// ---- block attention --------------------------------------------------------
// A segment with slot >= 0 lives in the cache ring, slot < 0 is text slot
// (-1 - slot) of the text ring.  Zero-length segments were dropped on the host.
struct AttnBlock {
  int32_t q_len;
  int32_t n_segs;
  int32_t slot[kAttnMaxSegs];
  int32_t len[kAttnMaxSegs];
  int32_t n_tiles;          // 64-key tiles of the key set (sum over segments)
  int32_t nqt;              // query tiles of this block (bf16 kernel)
  int32_t task_start;       // first task id of this block in the launch
  int32_t work_start;       // first work unit (task tile) of this block
};

struct AttnArgs {
  const void* q;            // [n_blocks][q_stride][heads][D] (this launch's first block)
  void* out;
  float* lse;               // [n_blocks][heads][q_stride] or null
  const void* cache;        // cache ring base
  const void* text;         // text ring base (may be null if unused)
  int32_t cache_tpad;
  int32_t text_tpad;
  int32_t q_stride;
  int32_t heads;
  int32_t n_qtiles;         // query tiles per (block, head)
  int32_t total_tasks;      // n_blocks * heads * n_qtiles
  int32_t tasks_per_xcd;    // ceil(total_tasks / 8)
  float qscale;             // scale * log2(e)
  float scale_ln;           // scale (fp32 kernel), ln(2) factor for lse
  // bf16 kernel schedule; XCD x (workgroup w runs on XCD w % 8) owns tasks
  // [x*n_tasks/8, (x+1)*n_tasks/8) and takes them in order.  split = 0: one
  // whole task per workgroup.  split = 1: the XCD's tasks but about its last
  // round run as whole-task workgroups; the rest of its task tiles is shared
  // evenly by tail_wg tail workgroups, which write the partial results of the
  // tasks they cut to the workspace; a second kernel merges them.
  float* partials;          // [8 * tail_wg][2][partial floats] (split)
  int32_t total_work;       // task tiles of the launch, < 2^31
  int32_t n_tasks;
  int32_t wg_per_xcd;       // list length per XCD
  int32_t tail_wg;          // tail workgroups per XCD (split)
  int32_t split;
  int32_t n_blocks;
  int32_t merge_per_xcd;    // merge workgroups per XCD (split)
  int32_t res_group_units;  // resident shape: units per (block, head) when each takes whole workgroups, else 0
  AttnBlock blk[kAttnMaxBlocks];
};
hipError_t launch_attention_bf16(const AttnArgs& a, int head_dim, int shape, hipStream_t s);

// ---- split schedule (shared by host and device) ------------------------------
// Even split of n units over k takers: taker j starts at split_start(n, k, j).
__host__ __device__ inline int split_start(int n, int k, int j) {
  const int q = n / k, r = n - (n / k) * k;
  return j * q + (j < r ? j : r);
}
// Taker whose share holds unit u (u < n).
__host__ __device__ inline int split_owner(int n, int k, int u) {
  const int q = n / k, r = n - (n / k) * k;
  const int big = r * (q + 1);
  return u < big ? u / (q + 1) : r + (u - big) / q;
}
// First work unit (task tile) of task t; t = n_tasks gives the total.
__host__ __device__ inline int task_work_start(const AttnArgs& a, int t) {
  if (t >= a.n_tasks) return a.total_work;
  int b = 0;
  while (b + 1 < a.n_blocks && a.blk[b + 1].task_start <= t) ++b;
  return a.blk[b].work_start + (t - a.blk[b].task_start) * a.blk[b].n_tiles;
}
// The task list of XCD x under the split schedule.
struct XcdPlan {
  int t0, t1;          // tasks [t0, t1)
  int whole;           // tasks t0 .. t0 + whole - 1 run whole
  int tail0, tail1;    // work units shared by the tail workgroups
};
__host__ __device__ inline XcdPlan xcd_plan(const AttnArgs& a, int x) {
  XcdPlan p;
  p.t0 = (int)(((int64_t)x * a.n_tasks) >> 3);
  p.t1 = (int)(((int64_t)(x + 1) * a.n_tasks) >> 3);
  const int wpx = a.tail_wg;               // resident workgroups of the XCD
  const int n = p.t1 - p.t0;
  int rounds = n / wpx;
  // the tail takes the part of the last round that does not fill the XCD; a
  // small one takes a whole round more, so no task is cut into many pieces
  if ((n - rounds * wpx) * 4 < wpx && rounds > 0) --rounds;
  p.whole = rounds * wpx;
  p.tail0 = task_work_start(a, p.t0 + p.whole);
  p.tail1 = task_work_start(a, p.t1);
  return p;
}
hipError_t launch_attention_f32(const AttnArgs& a, int head_dim, hipStream_t s);
// Launch shape of the bf16 kernel for a launch whose longest key set has
// max_keys keys and whose key sets span at most max_tiles tiles of 64 keys
// (tiles never straddle segments): 2 (resident: the whole key set held in
// LDS, independent 32-query units) when head_dim is 64 and every key set fits
// kResTiles tiles; 1 (narrow: 4-wave workgroups, several per CU) for other
// short key sets at head_dim 64, where the per-task prologue and epilogue
// weigh most; else 0 (wide: one workgroup per CU sharing each K/V copy among
// the most queries).  Measured at the 480p query shape: narrow 10-20 %
// faster up to 3072 keys, wide 2.5 % faster at 4096.
constexpr int kResTiles = 8;
constexpr int kResWaves = 12;            // waves per workgroup of the resident shape
constexpr int64_t kNarrowMaxKeys = 3072;
inline int attention_bf16_shape(int head_dim, int64_t max_keys, int64_t max_tiles) {
  if (head_dim != 64) return 0;
  if (max_tiles <= kResTiles) return 2;
  return max_keys <= kNarrowMaxKeys ? 1 : 0;
}
int attention_bf16_q_tile(int head_dim, int shape);   // queries per workgroup of the bf16 kernel
size_t attention_partial_bytes(int head_dim, int shape);   // workspace bytes of one partial result
hipError_t attention_bf16_resident(int head_dim, int shape, int* per_cu);   // workgroups per CU
int attention_f32_q_tile();

// ---- fused K/V producer (QKV projection) --------------------------------------
constexpr int kProjMaxBlocks = 64;       // blocks per producer launch (kernarg)
struct ProjArgs {
  const uint16_t* x;        // [n_blocks][n_tokens][dim] bf16
  const uint16_t* w;        // [3 * heads * head_dim][dim] bf16 (rows q | k | v)
  uint16_t* q;              // [n_blocks][n_tokens][heads][head_dim] bf16, or null (q rows skipped)
  uint16_t* ring;           // cache ring base
  const float* rope;        // [head_dim / 2][n_tokens][2] (cos, sin) per block, or null
  int64_t rope_bstride;     // floats between blocks' tables (0: one table for all)
  int32_t n_tokens;
  int32_t dim;              // multiple of 64
  int32_t heads;
  int32_t t_pad;            // ring slot token stride
  int32_t ch_begin;         // first output row computed: 0, or heads * head_dim without q
  int32_t n_ch;             // 3 * heads * head_dim
  int32_t n_blocks;
  int32_t pad_;
  int32_t slot[kProjMaxBlocks];   // ring slot of each block's K and V
};
hipError_t launch_project(const ProjArgs& a, int head_dim, hipStream_t s);
#ifndef BA_PROJ_TOK
#define BA_PROJ_TOK 256
#endif
#ifndef BA_PROJ_CH
#define BA_PROJ_CH 256
#endif
#ifndef BA_PROJ_K
#define BA_PROJ_K 64
#endif
#ifndef BA_PROJ_WPS
#define BA_PROJ_WPS 2
#endif
#ifndef BA_PROJ_WAVES_T
#define BA_PROJ_WAVES_T 4
#endif
#ifndef BA_PROJ_STAGES
#define BA_PROJ_STAGES 2
#endif
#ifndef BA_PROJ_GROUP
#define BA_PROJ_GROUP 8
#endif
constexpr int kProjTokTile = BA_PROJ_TOK;        // tokens per workgroup tile of the producer
constexpr int kProjChTile = BA_PROJ_CH;          // output rows per workgroup tile
constexpr int kProjKStep = BA_PROJ_K;            // input dims per LDS stage

// ---- coordinated noise initialisation ------------------------------------------
constexpr int kNoiseMaxFrames = 64;      // frames per block (kernarg)
struct NoiseArgs {
  const unsigned int __attribute__((ext_vector_type(4)))* pool;   // [channels][pool_frames][frame_vecs]
  unsigned int __attribute__((ext_vector_type(4)))* out;          // [channels][block_frames][frame_vecs]
  int64_t frame_vecs;       // 16-byte vectors per frame
  int32_t channels;
  int32_t pool_frames;
  int32_t block_frames;
  int32_t pad_;
  int32_t frames[kNoiseMaxFrames];
};
hipError_t launch_noise(const NoiseArgs& a, hipStream_t s);

// ---- block update -----------------------------------------------------------
struct UpdateArgs {
  uint16_t* x;              // [n_blocks][elems] bf16
  const uint16_t* eps;
  int64_t elems;
  int32_t n_blocks;
  float c1[kUpdateMaxBlocks];
  float c2[kUpdateMaxBlocks];
};
hipError_t launch_update(const UpdateArgs& a, hipStream_t s);

}  // namespace ba
