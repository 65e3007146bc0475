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
#include <type_traits>

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
// epilogue staging (bf16 elements; pitches padded off the 128-byte bank period)
constexpr int kEpiTokPitch = 64 + 8;                   // [token][64 dims]
constexpr int kEpiDimPitch = kWaveToks + 8;            // [64 dims][tokens]
constexpr int kEpiWaveElems = (kWaveToks * kEpiTokPitch > 64 * kEpiDimPitch ? kWaveToks * kEpiTokPitch
                                                                             : 64 * kEpiDimPitch);
static_assert((kThreads / 64) * kEpiWaveElems * 2 <= kStages * kStageChunks * 16, "epilogue fits the LDS stages");
static_assert(kWaveRows % 64 == 0 && kWaveToks % 32 == 0 && kWaveToks <= 512, "wave tile");
static_assert(kEpiWaveElems % 8 == 0, "16-byte aligned wave regions");
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
// row; their results are not stored.  A lane fetches the same rows and
// chunks in every stage: its byte offsets (stage_offsets) are computed once
// per tile, and a stage only moves the uniform base by its first input dim.
__device__ __forceinline__ void stage_offsets(const ProjArgs& a, int ch0, int t0, int tid,
                                              unsigned (&off)[kLoads]) {
  const int lane = tid & 63;
  const int wave_base = tid & ~63;
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int p = u * kThreads + wave_base + lane;
    if (u < kWLoads) {
      const int r = p / kRowChunks, c = (p % kRowChunks) ^ swz(r);
      int row = ch0 + r;
      row = row < a.n_ch ? row : a.n_ch - 1;
      off[u] = (unsigned)(row * a.dim + 8 * c) * 2u;
    } else {
      const int q = p - kWRows * kRowChunks;
      const int r = q / kRowChunks, c = (q % kRowChunks) ^ swz(r);
      int tok = t0 + r;
      tok = tok < a.n_tokens ? tok : a.n_tokens - 1;
      off[u] = (unsigned)(tok * a.dim + 8 * c) * 2u;
    }
  }
}

__device__ __forceinline__ void load_stage(const ProjArgs& a, const uint16_t* xb, const unsigned (&off)[kLoads],
                                           int k0, int tid, unsigned stage_lds) {
  const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const uint16_t* base = (u < kWLoads ? a.w : xb) + k0;   // uniform
    const unsigned lds = stage_lds + 16u * (unsigned)(u * kThreads + wave_base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off[u]), "s"(base), "s"(lds)
                 : "memory", "m0");
  }
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Workgroup barrier that orders LDS accesses only.  The fence of
// __syncthreads also waits for every global load in flight, which would
// drain the LDS-direct copies of the stages not yet due at every stage.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
__device__ __forceinline__ void wait_newer(int n) {   // n in [0, kStages - 1]
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: if constexpr (kStages > 1) wait_vm<1>(); break;
    case 2: if constexpr (kStages > 2) wait_vm<2>(); break;
    case 3: if constexpr (kStages > 3) wait_vm<3>(); break;
    case 4: if constexpr (kStages > 4) wait_vm<4>(); break;
    case 5: if constexpr (kStages > 5) wait_vm<5>(); break;
    default: wait_vm<0>(); break;
  }
}
static_assert(kStages >= 2 && kStages <= 6, "stages");

// Workgroup -> output tile.  Workgroup w runs on XCD w % 8, whose L2 is its
// own; XCD x takes a contiguous run of tiles in an order that walks bands of
// kGroup token tiles channel tile by channel tile, so the workgroups resident
// on one XCD at a time share most of their input rows and weight rows in
// that XCD's L2.
// Blocks of a batched call come one after the other in that order (they share
// the weight rows).
constexpr int kGroup = BA_PROJ_GROUP;
struct TileXY { int b, tt, ct; };
__device__ __forceinline__ TileXY tile_of(int w, int n_blocks, int n_tt, int n_ct) {
  const int per_block = n_tt * n_ct;
  const int n = n_blocks * per_block;
  const int x = w & 7, j = w >> 3;
  const int q = n >> 3, r = n & 7;
  const int rank = x * q + (x < r ? x : r) + j;     // this XCD's share starts at x*q + min(x, r)
  const int b = rank / per_block;
  const int rb = rank - b * per_block;
  const int band = rb / (kGroup * n_ct);
  const int g = min(kGroup, n_tt - band * kGroup);  // token tiles in this band
  const int local = rb - band * kGroup * n_ct;
  return {b, band * kGroup + local % g, local / g};
}

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
  const TileXY tile = tile_of(blockIdx.x, a.n_blocks, (a.t_pad + kProjTokTile - 1) / kProjTokTile,
                              (a.n_ch - a.ch_begin + kProjChTile - 1) / kProjChTile);
  // this tile's block: its input rows, q rows, rotation table and ring slot
  const uint16_t* xb = a.x + (int64_t)tile.b * a.n_tokens * a.dim;
  uint16_t* qb = a.q ? a.q + (int64_t)tile.b * a.n_tokens * a.heads * D : nullptr;
  const float* ropeb = a.rope ? a.rope + (int64_t)tile.b * a.rope_bstride : nullptr;
  const int slot = a.slot[tile.b];
  const int t0 = tile.tt * kProjTokTile;
  const int ch0 = a.ch_begin + tile.ct * kProjChTile;
  const int n_k = a.dim / kKStep;
  unsigned loff[kLoads];
  stage_offsets(a, ch0, t0, tid, loff);

  f32x16 acc[kRB][kTB];
#pragma unroll
  for (int cb = 0; cb < kRB; ++cb)
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  // kStages LDS buffers; stage s holds input dims [kKStep s, kKStep (s + 1)).
  // Software pipeline inside a wave: the operands of the next 16-dim step are
  // read from LDS while the matrix cores work on the current one (two register
  // sets), and the barrier that publishes the next stage sits between the two,
  // so a wave's MFMA stream never waits on its own LDS reads.
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < n_k) load_stage(a, xb, loff, s * kKStep, tid, lds_addr + 16u * kStageChunks * s);
  {
    const int issued = n_k < kStages ? n_k : kStages;
    wait_newer(issued - 1);                             // stage 0 has landed
  }
  lds_barrier();

  bf16x8 fw[2][kRB], fx[2][kTB];
  auto read_frag = [&](int f, const u32x4* L, int ks) {
#pragma unroll
    for (int cb = 0; cb < kRB; ++cb)
      fw[f][cb] = as_bf16x8(L[lds_idx(kWaveRows * cw + 32 * cb + (lane & 31), 2 * ks + half)]);
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
      fx[f][tb] = as_bf16x8(L[kWRows * kRowChunks + lds_idx(kWaveToks * tw + 32 * tb + (lane & 31), 2 * ks + half)]);
  };
  constexpr int kSub = kKStep / 16;                    // 16-dim steps per stage (even)
  static_assert(kSub % 2 == 0, "register sets alternate by step parity");
  // one stage; the last one has no next stage to publish or read, and is a
  // copy of its own so that no branch joins the two register sets' waits
  auto stage = [&](int kt, auto is_last) {
    const u32x4* L = lds[kt % kStages];
#pragma unroll
    for (int ks = 0; ks < kSub; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < kSub) {
        read_frag(nxt, L, ks + 1);
      } else if constexpr (!decltype(is_last)::value) {
        // publish stage kt + 1 (the stages issued after it may stay in
        // flight); past the barrier every wave's reads of this stage's buffer
        // are done (its last operands are already in registers), so that
        // buffer takes stage kt + kStages
        const int ahead = kt + kStages - 1;               // newest stage issued so far
        wait_newer((ahead < n_k ? ahead : n_k - 1) - (kt + 1));
        lds_barrier();
        if (kt + kStages < n_k)
          load_stage(a, xb, loff, (kt + kStages) * kKStep, tid, lds_addr + 16u * kStageChunks * (kt % kStages));
        read_frag(nxt, lds[(kt + 1) % kStages], 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < kRB; ++cb)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][cb], fx[cur][tb], acc[cb][tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  read_frag(0, lds[0], 0);
  for (int kt = 0; kt + 1 < n_k; ++kt) stage(kt, std::false_type{});
  stage(n_k - 1, std::true_type{});

  // ---- epilogue --------------------------------------------------------------
  // A wave's rows come in units of 64 (one head of 64 dims, or half of one of
  // 128): a unit is all q, all k or all v, of one head.  Lane = token and
  // registers = consecutive rows in the accumulators; the unit is rotated and
  // rounded there, then passed through the wave's own LDS region so that every
  // lane stores 16 contiguous bytes: 8 dims of one token (q, k) or 8 tokens of
  // one dim (v, stored dim-major).
  __syncthreads();                                     // the LDS stages are free
  const int HD = a.heads * D;
  const int tok_w = t0 + kWaveToks * tw;               // first token of the wave's columns
  uint16_t* E = reinterpret_cast<uint16_t*>(&lds[0][0]) + wave * kEpiWaveElems;
  // Rotation table entries of the wave's tokens, all issued together (one
  // memory round trip).  At head dim 64 every unit is a whole head (pairs
  // 0..31), so the wave loads them once; at 128 a unit is half a head and
  // loads its own half.  Tokens past the end read the last token's entry
  // (their results are replaced by zeros).
  float2 cs[2][kTB][8];
  auto load_cs = [&](int dbase) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const int tok = tok_w + 32 * tb + (lane & 31);
        const int tc = tok < a.n_tokens ? tok : a.n_tokens - 1;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const int d = dbase + 32 * c2 + 8 * (i >> 2) + 4 * half + (i & 3);
          cs[c2][tb][i >> 1] = *reinterpret_cast<const float2*>(ropeb + ((int64_t)(d >> 1) * a.n_tokens + tc) * 2);
        }
      }
  };
  if (D == 64 && ropeb != nullptr) load_cs(0);
#pragma unroll
  for (int u = 0; u < kWaveRows / 64; ++u) {
    const int r0 = ch0 + kWaveRows * cw + 64 * u;      // first row of the unit
    if (r0 >= a.n_ch) break;                           // n_ch is a multiple of 64
    const int which = r0 / HD;                         // 0 q, 1 k, 2 v
    const int h = (r0 - which * HD) / D;
    const int dbase = r0 - which * HD - h * D;         // 0, or 64 in a 128-dim head
    if (which == 0 && qb == nullptr) continue;
    const bool rotate = which < 2 && ropeb != nullptr;
    if (D == 128 && rotate) load_cs(dbase);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const int tl = 32 * tb + (lane & 31);          // token within the wave's columns
        const int tok = tok_w + tl;
        const bool valid = tok < a.n_tokens;
        f32x16 y = acc[2 * u + c2][tb];
        if (rotate && valid) {
          // pairs (d, d + 1), d even: registers (i, i + 1), i even; the table
          // is pair-major, so the lanes (consecutive tokens) read one run
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float2 r = cs[c2][tb][i >> 1];
            const float y0 = y[i], y1 = y[i + 1];
            y[i] = y0 * r.x - y1 * r.y;
            y[i + 1] = y0 * r.y + y1 * r.x;
          }
        }
        if (!valid) {
#pragma unroll
          for (int i = 0; i < 16; ++i) y[i] = 0.f;       // the slot's tail reads as zeros
        }
        if (which < 2) {               // E: [token][64 dims], pitch kEpiTokPitch
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 v;
            v.x = pack2(y[4 * g], y[4 * g + 1]);
            v.y = pack2(y[4 * g + 2], y[4 * g + 3]);
            *reinterpret_cast<uint2*>(E + tl * kEpiTokPitch + 32 * c2 + 8 * g + 4 * half) = v;
          }
        } else {                       // E: [64 dims][tokens], pitch kEpiDimPitch
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            bf16x2 pk;
            pk[0] = (__bf16)y[i];
            E[(32 * c2 + 8 * (i >> 2) + 4 * half + (i & 3)) * kEpiDimPitch + tl] = __builtin_bit_cast(uint16_t, pk[0]);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (which < 2) {
      // 8 lanes per token (64 dims), 8 tokens per store instruction
      uint16_t* base;
      int64_t tstride;
      int tlimit;
      if (which == 0) {
        base = qb + (int64_t)h * D + dbase;
        tstride = HD;
        tlimit = a.n_tokens;
      } else {
        base = a.ring + ((int64_t)(slot * 2) * a.heads + h) * ((int64_t)a.t_pad * D) + dbase;
        tstride = D;
        tlimit = a.t_pad;
      }
#pragma unroll
      for (int j = 0; j < kWaveToks / 8; ++j) {
        const int tl = 8 * j + (lane >> 3);
        const int tok = tok_w + tl;
        const u32x4 v = *reinterpret_cast<const u32x4*>(E + tl * kEpiTokPitch + 8 * (lane & 7));
        if (tok < tlimit) *reinterpret_cast<u32x4*>(base + tok * tstride + 8 * (lane & 7)) = v;
      }
    } else {
      // kWaveToks / 8 lanes per dim row, 8 tokens each
      constexpr int kLanesPerRow = kWaveToks / 8;
      constexpr int kRowsPerStore = 64 / kLanesPerRow;
      uint16_t* base = a.ring + ((int64_t)(slot * 2 + 1) * a.heads + h) * ((int64_t)a.t_pad * D);
      const int c = lane % kLanesPerRow;
      const int tok = tok_w + 8 * c;                   // a multiple of 8: the 8 tokens share the bound
#pragma unroll
      for (int j = 0; j < 64 / kRowsPerStore; ++j) {
        const int r = kRowsPerStore * j + lane / kLanesPerRow;
        const u32x4 v = *reinterpret_cast<const u32x4*>(E + r * kEpiDimPitch + 8 * c);
        if (tok < a.t_pad) *reinterpret_cast<u32x4*>(base + (int64_t)(dbase + r) * a.t_pad + tok) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}


}  // namespace

hipError_t launch_project(const ProjArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(a.n_blocks * ((a.t_pad + kProjTokTile - 1) / kProjTokTile) *
                  ((a.n_ch - a.ch_begin + kProjChTile - 1) / kProjChTile));
  if (head_dim == 64)
    hipLaunchKernelGGL(project_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(project_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
