// Fused K/V producer: the QKV projection of one block's tokens on the matrix
// cores, with the optional pair rotation and the cache's own layout in the
// epilogue, so K and V land in their ring slot without a separate append pass
// (the feature cache of "Minute-Long Videos with Dual Parallelisms",
// Abstract, holds the self-attention K/V a block produced).
//
//   Y^T = W X^T, W: [3 H D][dim] (a linear layer's weight), X: [tokens][dim]
//
// Computed transposed (rows = output channels, columns = tokens) with
// v_mfma_f32_32x32x16_bf16, so that a lane holds one token and consecutive
// output channels: the rotation of adjacent pairs stays inside a lane, K rows
// go out as 8-byte stores and V^T columns as one 2-byte store per lane, lanes
// walking consecutive tokens.
#include "internal.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesT = BA_PROJ_WAVES_T;               // waves along the tokens (2 along the rows)
constexpr int kThreads = 128 * kWavesT;
constexpr int kKStep = kProjKStep;                     // input dims per LDS stage
constexpr int kRowChunks = kKStep / 8;                 // 16-byte chunks per LDS row
constexpr int kWRows = kProjChTile;                    // weight rows per stage
constexpr int kXRows = kProjTokTile;                   // token rows per stage
constexpr int kWaveRows = kWRows / 2;                  // rows of a wave's tile
constexpr int kWaveToks = kXRows / kWavesT;            // tokens of a wave's tile
constexpr int kRB = kWaveRows / 32;                    // 32-row MFMA blocks per wave
constexpr int kTB = kWaveToks / 32;                    // 32-token MFMA blocks per wave
constexpr int kStageChunks = (kWRows + kXRows) * kRowChunks;
constexpr int kLoads = kStageChunks / kThreads;        // per thread and stage
constexpr int kWLoads = kWRows * kRowChunks / kThreads;
constexpr int kStages = BA_PROJ_STAGES;
static_assert(kStageChunks % kThreads == 0 && (kWRows * kRowChunks) % kThreads == 0, "tile shape");
static_assert(kRowChunks == 4 || kRowChunks == 8, "row length");

// XOR swizzle of the 16-byte chunks of a row: the lanes of an MFMA operand
// read consecutive rows at one chunk; any 8 of them (16 over 256 bytes) must
// fall on distinct bank groups.  128-byte rows: chunk ^ (r mod 8, flipped by
// bit 3); 64-byte rows (four rows per 256 bytes): chunk ^ (r / 4 mod 4).
__device__ __forceinline__ int swz(int r) {
  return kRowChunks == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}
__device__ __forceinline__ int lds_idx(int r, int c) { return r * kRowChunks + (c ^ swz(r)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, p);
}

// One stage: kWRows weight rows and kXRows token rows, kKStep input dims
// each, straight from global memory into LDS (global_load_lds_dwordx4 issued
// from asm: no register result; the stage is read only after the vmcnt wait
// and barrier that publish it).  Rows past the end are clamped to the last
// row; their results are not stored.
__device__ __forceinline__ void load_stage(const ProjArgs& a, int ch0, int t0, int k0, int tid,
                                           unsigned stage_lds) {
  const int lane = tid & 63;
  const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int p0 = u * kThreads + wave_base;
    const int p = p0 + lane;
    const uint16_t* base;
    unsigned off;
    if (u < kWLoads) {
      const int r = p / kRowChunks, c = (p % kRowChunks) ^ swz(r);
      int row = ch0 + r;
      row = row < a.n_ch ? row : a.n_ch - 1;
      base = a.w;
      off = (unsigned)(row * a.dim + k0 + 8 * c) * 2u;
    } else {
      const int q = p - kWRows * kRowChunks;
      const int r = q / kRowChunks, c = (q % kRowChunks) ^ swz(r);
      int tok = t0 + r;
      tok = tok < a.n_tokens ? tok : a.n_tokens - 1;
      base = a.x;
      off = (unsigned)(tok * a.dim + k0 + 8 * c) * 2u;
    }
    const unsigned lds = stage_lds + 16u * (unsigned)p0;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
  }
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Wait until at most n stages' loads (n * kLoads) are still in flight: loads
// complete in order, so every older stage has landed.  simm16 of s_waitcnt:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 (the latter two left at
// their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  constexpr int v = N * kLoads;
  static_assert(v < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (v & 15) | ((v >> 4) << 14));
}
__device__ __forceinline__ void wait_newer(int n) {   // n in [0, kStages - 2]
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: if constexpr (kStages > 3) wait_vm<2>(); break;
    case 3: if constexpr (kStages > 4) wait_vm<3>(); break;
    case 4: if constexpr (kStages > 5) wait_vm<4>(); break;
    case 5: if constexpr (kStages > 6) wait_vm<5>(); break;
    default: wait_vm<0>(); break;
  }
}
static_assert(kStages >= 2 && kStages <= 7, "stages");

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BA_PROJ_WPS, BA_PROJ_WPS)))
void project_kernel(const ProjArgs a) {
  __shared__ u32x4 lds[kStages][kStageChunks];
  const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)&lds[0][0];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int cw = wave & 1;             // weight rows kWaveRows cw .. of the tile
  const int tw = wave >> 1;            // token rows kWaveToks tw .. of the tile (0 .. kWavesT - 1)
  const int t0 = blockIdx.x * kProjTokTile;
  const int ch0 = a.ch_begin + blockIdx.y * kProjChTile;
  const int n_k = a.dim / kKStep;

  f32x16 acc[kRB][kTB];
#pragma unroll
  for (int cb = 0; cb < kRB; ++cb)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  // kStages buffers: kStages - 1 stages in flight ahead of the one consumed;
  // stage s holds input dims [kKStep s, kKStep (s + 1))
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < n_k) load_stage(a, ch0, t0, s * kKStep, tid, lds_addr + 16u * kStageChunks * s);
  {
    const int issued = n_k < kStages - 1 ? n_k : kStages - 1;
    wait_newer(issued - 1);                             // stage 0 has landed
  }
  __syncthreads();
  for (int kt = 0; kt < n_k; ++kt) {
    const int st = kt % kStages;
    const int ahead = kt + kStages - 1;
    if (ahead < n_k)     // its buffer was last read at kt - 1 (barrier below)
      load_stage(a, ch0, t0, ahead * kKStep, tid, lds_addr + 16u * kStageChunks * (ahead % kStages));
    const u32x4* L = lds[st];
#pragma unroll
    for (int ks = 0; ks < kKStep / 16; ++ks) {
      bf16x8 wa[kRB], xb[kTB];
#pragma unroll
      for (int cb = 0; cb < kRB; ++cb)
        wa[cb] = as_bf16x8(L[lds_idx(kWaveRows * cw + 32 * cb + (lane & 31), 2 * ks + half)]);
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb)
        xb[tb] = as_bf16x8(L[kWRows * kRowChunks + lds_idx(kWaveToks * tw + 32 * tb + (lane & 31), 2 * ks + half)]);
#pragma unroll
      for (int cb = 0; cb < kRB; ++cb)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[cb], xb[tb], acc[cb][tb], 0, 0, 0);
    }
    if (kt + 1 < n_k) {
      // publish stage kt + 1: the stages issued after it may stay in flight
      const int last = ahead < n_k ? ahead : n_k - 1;
      wait_newer(last - (kt + 1));
      __syncthreads();
    }
  }

  // ---- epilogue: lane = token, registers = consecutive output rows --------
  const int HD = a.heads * D;
#pragma unroll
  for (int cb = 0; cb < kRB; ++cb) {
    const int chb = ch0 + kWaveRows * cw + 32 * cb;   // first row of this 32-row block
    if (chb >= a.n_ch) continue;
    const int which = chb / HD;                        // 0 q, 1 k, 2 v (a 32-row block never straddles)
    const int rem = chb - which * HD;
    const int h = rem / D;
    const int d0 = rem - h * D;                        // first dim of the block within the head
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      const int tok = t0 + kWaveToks * tw + 32 * tb + (lane & 31);
      const bool valid = tok < a.n_tokens;
      f32x16 y = acc[cb][tb];
      if (which < 2 && a.rope != nullptr && valid) {
        // pairs (d, d + 1), d even: registers (i, i + 1) with i even
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const int d = d0 + 8 * (i >> 2) + 4 * half + (i & 3);
          const float2 cs = *reinterpret_cast<const float2*>(a.rope + ((int64_t)tok * (D / 2) + d / 2) * 2);
          const float y0 = y[i], y1 = y[i + 1];
          y[i] = y0 * cs.x - y1 * cs.y;
          y[i + 1] = y0 * cs.y + y1 * cs.x;
        }
      }
      if (!valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = 0.f;         // the slot's tail reads as zeros
      }
      if (which == 0) {
        if (!valid || a.q == nullptr) continue;
        uint16_t* qp = a.q + ((int64_t)tok * a.heads + h) * D;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = d0 + 8 * g + 4 * half;
          uint2 v;
          v.x = pack2(y[4 * g], y[4 * g + 1]);
          v.y = pack2(y[4 * g + 2], y[4 * g + 3]);
          *reinterpret_cast<uint2*>(qp + d) = v;
        }
      } else if (tok < a.t_pad) {
        const int64_t mat = (int64_t)a.t_pad * D;
        uint16_t* base = a.ring + ((int64_t)(a.slot * 2 + which - 1) * a.heads + h) * mat;
        if (which == 1) {           // K: token-major [T_pad][D]
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = d0 + 8 * g + 4 * half;
            uint2 v;
            v.x = pack2(y[4 * g], y[4 * g + 1]);
            v.y = pack2(y[4 * g + 2], y[4 * g + 3]);
            *reinterpret_cast<uint2*>(base + (int64_t)tok * D + d) = v;
          }
        } else {                    // V: dim-major [D][T_pad]
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int d = d0 + 8 * (i >> 2) + 4 * half + (i & 3);
            bf16x2 p;
            p[0] = (__bf16)y[i];
            base[(int64_t)d * a.t_pad + tok] = __builtin_bit_cast(uint16_t, p[0]);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_project(const ProjArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid((a.t_pad + kProjTokTile - 1) / kProjTokTile,
                  (a.n_ch - a.ch_begin + kProjChTile - 1) / kProjChTile);
  if (head_dim == 64)
    hipLaunchKernelGGL(project_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(project_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
