// Internal launch interfaces between the C-ABI layer (api.cpp) and the HIP
// kernels.  Everything here is validated by the caller before it is called.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace ba {

constexpr int kTokenAlign = 64;          // ring slot stride granularity
constexpr int kAppendMaxBlocks = 64;     // slots per append launch (kernarg)
constexpr int kAttnMaxBlocks = 16;       // blocks per attention launch (kernarg)
constexpr int kAttnMaxSegs = 9;          // 8 cache segments + text
constexpr int kUpdateMaxBlocks = 64;     // blocks per update launch (kernarg)

// ---- ring append -----------------------------------------------------------
struct AppendArgs {
  const void* k;            // [n_blocks][n_tokens][heads][D]
  const void* v;
  void* ring;               // ring base
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
  AttnBlock blk[kAttnMaxBlocks];
};
hipError_t launch_attention_bf16(const AttnArgs& a, int head_dim, hipStream_t s);
hipError_t launch_attention_f32(const AttnArgs& a, int head_dim, hipStream_t s);
int attention_bf16_q_tile(int head_dim);   // queries per workgroup of the bf16 kernel
int attention_f32_q_tile();

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
