// Cache append: one block's K/V (token-major, as a QKV projection emits them,
// or head-major, as a text prompt's per-head K/V arrays come) into a ring
// slot.  K keeps its token-major rows; V is transposed to the
// dim-major layout the attention kernel streams.  Pure data movement, bound by
// HBM bandwidth: every byte is read once and written once, 16 bytes per lane.
//
// The feature cache it fills is the one of "Minute-Long Videos with Dual
// Parallelisms" (Abstract): a block's K/V are stored once and reused as
// context by the neighbouring block.
#include "internal.h"

namespace ba {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// The block's K/V are read once: streaming loads, which do not keep them in
// the caches (measured with the Infinity Cache flushed, 128-token tiles:
// 4.7-5.1 TB/s from 268 MB to 2 GB against 4.3-4.7 with ordinary loads).
// The ring is written with ordinary stores: the attention that follows reads
// it.
__device__ __forceinline__ u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// E: element storage type (uint16_t for bf16, uint32_t for fp32).  A
// workgroup moves TOK tokens of one head: their K rows (one contiguous run of
// the slot's K matrix) and, through LDS, their V as V^T rows of TOK tokens
// (TOK * sizeof(E) bytes each; the longer the run, the fewer scattered
// pieces).  Tokens past n_tokens are written as zeros; tokens past the slot
// stride are not touched.
template <int D, typename E, int TOK>
__global__ __launch_bounds__(kThreads) void append_kernel(const AppendArgs a) {
  constexpr int EB = sizeof(E);
  constexpr int ROW_CH = D * EB / 16;            // 16-B chunks per token row
  constexpr int K_CH = TOK * ROW_CH;             // chunks in the K tile
  constexpr int K_PER_THREAD = K_CH / kThreads;
  constexpr int PAD = 4 / EB;                    // LDS row padding (elements)
  constexpr int LROW = D + PAD;                  // LDS row stride (elements)
  constexpr int TOK_PER_CH = 16 / EB;            // tokens per 16-B chunk of a V^T row
  constexpr int VT_ROW_CH = TOK / TOK_PER_CH;    // chunks per V^T row in this tile
  constexpr int VT_CH = D * VT_ROW_CH;
  constexpr int VT_PER_THREAD = VT_CH / kThreads;
  static_assert(K_CH % kThreads == 0 && VT_CH % kThreads == 0, "tile shape");

  __shared__ E vt[TOK * LROW];

  const int t0 = blockIdx.x * TOK;
  const int h = blockIdx.y;
  const int z = blockIdx.z;
  const int tid = threadIdx.x;
  const int H = a.heads;
  const int64_t slot = a.slot[z];

  const E* ksrc = static_cast<const E*>(a.k) + (int64_t)z * a.n_tokens * H * D;
  const E* vsrc = static_cast<const E*>(a.v) + (int64_t)z * a.n_tokens * H * D;
  E* kdst = static_cast<E*>(a.ring) + ((slot * 2 + 0) * H + h) * (int64_t)a.t_pad * D;
  E* vdst = static_cast<E*>(a.ring) + ((slot * 2 + 1) * H + h) * (int64_t)a.t_pad * D;

  // K rows: straight copy, zeros past n_tokens.
#pragma unroll
  for (int u = 0; u < K_PER_THREAD; ++u) {
    const int g = tid + u * kThreads;
    const int t = t0 + g / ROW_CH;
    const int c = g % ROW_CH;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (t < a.n_tokens) val = load_stream(ksrc + t * a.src_tok + h * a.src_head + c * (16 / EB));
    if (t < a.t_pad) *reinterpret_cast<u32x4*>(kdst + (int64_t)t * D + c * (16 / EB)) = val;
  }

  // V: stage the [TOK tokens][D] tile in LDS, then write it out dim-major.
#pragma unroll
  for (int u = 0; u < K_PER_THREAD; ++u) {
    const int g = tid + u * kThreads;
    const int tl = g / ROW_CH;
    const int t = t0 + tl;
    const int c = g % ROW_CH;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (t < a.n_tokens) val = load_stream(vsrc + t * a.src_tok + h * a.src_head + c * (16 / EB));
    unsigned int* dst = reinterpret_cast<unsigned int*>(vt + tl * LROW + c * (16 / EB));
    dst[0] = val[0]; dst[1] = val[1]; dst[2] = val[2]; dst[3] = val[3];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < VT_PER_THREAD; ++u) {
    const int g = tid + u * kThreads;
    const int d = g / VT_ROW_CH;
    const int j = g % VT_ROW_CH;
    E e[TOK_PER_CH];
#pragma unroll
    for (int i = 0; i < TOK_PER_CH; ++i) e[i] = vt[(j * TOK_PER_CH + i) * LROW + d];
    u32x4 val;
    if constexpr (EB == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) val[w] = (unsigned)e[2 * w] | ((unsigned)e[2 * w + 1] << 16);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) val[w] = (unsigned)e[w];
    }
    if (t0 + j * TOK_PER_CH < a.t_pad)
      *reinterpret_cast<u32x4*>(vdst + (int64_t)d * a.t_pad + t0 + j * TOK_PER_CH) = val;
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* p, int64_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = z;
}

}  // namespace

// 128-token tiles (V^T pieces of 256 bytes at bf16) unless that leaves fewer
// than four workgroups per CU of a 256-CU device; then 64-token tiles.
template <int D, typename E>
void launch_append_d(const AppendArgs& a, hipStream_t s) {
  const int64_t wg128 = (int64_t)((a.t_pad + 127) / 128) * a.heads * a.n_blocks;
  if (wg128 >= 1024) {
    dim3 grid((a.t_pad + 127) / 128, a.heads, a.n_blocks);
    hipLaunchKernelGGL((append_kernel<D, E, 128>), grid, dim3(kThreads), 0, s, a);
  } else {
    dim3 grid(a.t_pad / 64, a.heads, a.n_blocks);
    hipLaunchKernelGGL((append_kernel<D, E, 64>), grid, dim3(kThreads), 0, s, a);
  }
}

hipError_t launch_append(const AppendArgs& a, int head_dim, int elem_bytes, hipStream_t s) {
  if (elem_bytes == 2) {
    if (head_dim == 64) launch_append_d<64, uint16_t>(a, s);
    else launch_append_d<128, uint16_t>(a, s);
  } else {
    if (head_dim == 64) launch_append_d<64, uint32_t>(a, s);
    else launch_append_d<128, uint32_t>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace ba
