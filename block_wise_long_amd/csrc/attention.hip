// Block attention: the queries of each queued block attend over
// [cache segment ... | text] keys streamed straight from the K/V ring, with no
// concatenated copy of the key set.
//
// What is computed: scaled dot-product attention ("Attention Is All You Need",
// listed among the works the DualParal page builds on), per head, over the key
// set that the feature cache of "Minute-Long Videos with Dual Parallelisms"
// (Abstract) defines: the neighbouring block's cached K/V, the block's own K/V
// and the text-conditioning K/V.
//
// bf16 kernel (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * workgroup = one query tile of one (block, head); wave = 32 queries.
//     All waves of a workgroup share each K/V tile copied to LDS.  Wide
//     shape: 12 waves (384 queries) at head dim 64, 8 waves (256) at 128, one
//     workgroup per CU; narrow shape for short key sets (head dim 64): 4
//     waves, three workgroups per CU (see Shape).  Key sets of at most 8
//     tiles at head dim 64 (a text prompt) take attention_resident_kernel
//     instead: the whole key set in LDS, waves on independent 32-query units.
//   * S^T = K Q^T is computed per 32-key group, so that a lane owns one
//     query column and 16 of its scores: every per-query softmax quantity is
//     lane-local (lanes l and l^32 share a query), and O^T = V^T P^T leaves the
//     output of a query in the lanes that hold its weights.  Q and K enter the
//     MFMA exactly as given; the scale c = scale*log2(e) and the reference
//     maximum are applied to the fp32 scores by one FMA each, so the score
//     error does not grow with the score's magnitude.
//   * Scores are taken relative to a reference maximum m, the chunk's first
//     group's maximum.  Head dim 64 (fast form) never moves it and takes the
//     weight sums on the matrix cores (a 16x16x32 product per 16 keys with a
//     0/1 selector operand), so the vector ALUs spend one FMA, one
//     v_exp_f32 and half a bf16 conversion per score and nothing else; a
//     chunk whose weights overflow is computed again with a per-group check
//     that raises m by whole numbers (exact form).  Head dim 128 sums the
//     weights in fp32 on the vector ALUs and raises m whenever a group's
//     weight sum exceeds 2^12.  Either way the result is exact softmax:
//     out = (sum p v) / (sum p) with a common m.
//   * The weights are rounded to bf16 for the PV product; the row sums are
//     taken from the rounded weights (head dim 64) or in fp32 from the
//     unrounded exponentials (head dim 128).
//   * K and V^T tiles of 64 keys rotate through three LDS buffers with an XOR
//     swizzle of 16-byte chunks (conflict-free ds_read_b128 for the MFMA
//     operands).  The tile after next streams from global memory straight
//     into a free buffer (global_load_lds_dwordx4, no staging registers)
//     while the current tile computes.  One barrier per tile.
//   * Workgroups are mapped to tasks XCD-major: the hardware deals workgroups
//     round-robin to the 8 XCDs, so consecutive tasks (same block and head,
//     neighbouring query tiles, hence the same K/V stream) share an XCD's L2.
//
// fp32 kernel: plain VALU, one query per lane, exact running maximum; used for
// fp32 rings (small shapes, parity at 1e-5).
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKTile = kKeyTile;   // keys per LDS tile
constexpr float kLazyLog2 = 12.0f;          // scaled scores above m + 12 (weights above 2^12) raise m
constexpr float kLazyThreshold = 4096.0f;   // 2^12: the same bound on a group's weight sum
constexpr float kLn2 = 0.693147180559945309f;


// Key of LDS K row r within its 32-row group: bits 2 and 3 swapped.  With it,
// the 16 scores a lane holds for one 32-key group (rows 8(i/4) + 4(l/32) + i%4
// of the MFMA output) are keys 8(l/32) + i and 16 + 8(l/32) + i - 8, i.e. two
// runs of 8 consecutive keys, exactly the B operand of the PV product.
__device__ __forceinline__ int key_of_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Segment cursor: which ring matrix the current key tile comes from.
struct Cursor {
  const uint16_t* k;   // K rows of (slot, head): [T_pad][D]
  const uint16_t* v;   // V^T of (slot, head): [D][T_pad]
  int tpad;
  int len;             // valid keys in the segment
  int off;             // first key of the tile within the segment
  int seg;
};

template <int D>
__device__ __forceinline__ void open_segment(const AttnArgs& a, const AttnBlock& B, int h, Cursor& c) {
  const int s = B.slot[c.seg];
  const uint16_t* base;
  int64_t slot;
  if (s >= 0) {
    base = static_cast<const uint16_t*>(a.cache);
    c.tpad = a.cache_tpad;
    slot = s;
  } else {
    base = static_cast<const uint16_t*>(a.text);
    c.tpad = a.text_tpad;
    slot = -1 - s;
  }
  const int64_t mat = (int64_t)c.tpad * D;
  c.k = base + ((slot * 2 + 0) * a.heads + h) * mat;
  c.v = base + ((slot * 2 + 1) * a.heads + h) * mat;
  c.len = B.len[c.seg];
  c.off = 0;
  // the segment table is read with scalar loads; finish them here so that no
  // step starts with one in flight (the LDS reads of a step are then waited
  // for one by one instead of all at once)
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
}

template <int D>
__device__ __forceinline__ void advance(const AttnArgs& a, const AttnBlock& B, int h, Cursor& c) {
  c.off += kKTile;
  if (c.off >= c.len) {
    ++c.seg;
    if (c.seg < B.n_segs) open_segment<D>(a, B, h, c);
  }
}

// Per-wave state of the online softmax for its 32 queries.
template <int D>
struct WaveState {
  f32x16 o[D / 32];    // O^T accumulator: lane owns query lane%32, 16 dims per block
  float m_ref;         // reference maximum (exp2 domain); equal in lanes l, l^32
  float l_sum;         // this lane's share of the weight sum
  f32x4 l_acc;         // fast path: weight sums on the matrix cores (see row_sums)
};

// Launch shapes: waves per workgroup (32 queries each).  S = 0, the wide
// shape: one workgroup per CU, as many queries as the registers allow sharing
// each K/V tile copy; D = 64: 12 waves, 3 per SIMD; D = 128: 8 waves, 2 per
// SIMD.  S = 1, the narrow shape for short key sets (D = 64 only): 4 waves,
// three workgroups per CU, whose prologues and epilogues overlap.  S = 2,
// the resident shape for key sets held whole in LDS (see
// attention_resident_kernel): one workgroup per CU.  KW of the waves copy the
// K tile, the others the V^T tile (see load_tile).
template <int D, int S = 0> struct Shape;
template <> struct Shape<64, 0> { static constexpr int NW = 12, WAVES_PER_SIMD = 3, KW = 8; };
template <> struct Shape<64, 1> { static constexpr int NW = 4, WAVES_PER_SIMD = 3, KW = 2; };
template <> struct Shape<64, 2> { static constexpr int NW = kResWaves, WAVES_PER_SIMD = 3, KW = 8; };
template <> struct Shape<128, 0> { static constexpr int NW = 8, WAVES_PER_SIMD = 2, KW = 4; };

constexpr int kBuffers = 3;   // LDS tile buffers: in use, being consumed, being filled
// a step's LDS operand reads issued ahead of their MFMA
template <int D> constexpr int kLdsAhead = 3;
// Where a step's weight computation goes.  D = 64 (VALU-bound, three waves
// per SIMD): in chunks after the MFMAs, so every wave keeps both pipes busy.
// D = 128 (two waves per SIMD, twice the MFMAs per weight): all of it after
// the step's last MFMA, so that one wave's MFMA phase overlaps the other's
// VALU phase (measured 4 % faster at the 720p block; the same at D = 64).
template <int D> constexpr bool kSplitPhases = D == 128;
// Weight sums on the matrix cores (see pipe_step): head dim 64 only.
template <int D> constexpr bool kMatrixSums = D == 64;

// Tile<D, S>: the LDS layout (the same for every shape) and the launch shape
template <int D, int S = 0>
struct Tile {
  static constexpr int NW = Shape<D, S>::NW;
  static constexpr int THREADS = NW * 64;
  static constexpr int QTILE = NW * 32;
  static constexpr int KCH = D / 8;                  // 16-B chunks per K row
  static constexpr int K_CH = kKTile * KCH;          // chunks of the K tile
  static constexpr int V_CH = D * (kKTile / 8);      // chunks of the V^T tile
  static constexpr int CH = K_CH + V_CH;
  static constexpr int LOADS = (CH + THREADS - 1) / THREADS;   // zero-fill rounds per buffer
  // copies: KW waves take the K tile in KR rounds of 64 chunks, the other VW
  // waves the V^T tile in VR rounds
  static constexpr int KW = Shape<D, S>::KW, VW = NW - KW;
  static constexpr int KR = K_CH / 64 / KW, VR = V_CH / 64 / VW;
  static constexpr int K_ROWS_STEP = 64 * KW / KCH;  // K rows between a wave's rounds
  static constexpr int V_DIMS_STEP = 8 * VW;         // V^T rows between a wave's rounds
  static_assert(KW > 0 && VW > 0 && KR * KW * 64 == K_CH && VR * VW * 64 == V_CH, "copy rounds");
  // a round's lanes keep the chunk (column) and row-order offsets of the first
  // round: both swizzles and the row order repeat every 16 rows
  static_assert(K_ROWS_STEP % 16 == 0 && V_DIMS_STEP % 16 == 0, "copy round strides");
  // a V lane's chunk sits in V^T rows below VW * 8 and columns below 64 of
  // its tile: its 32-bit byte offset stays below 2 * VW * 8 * T_pad, in range
  // for every slot stride the host accepts
  static_assert(VW * 8 <= 32 && (unsigned long long)2 * 32 * kAttnMaxSlotStride <= (1ull << 32),
                "32-bit copy offsets");

  // XOR swizzle of the 16-byte chunks of a row.  A b128 LDS access is served
  // 8 lanes per 128 bytes or 16 lanes per 256 bytes of banks; consecutive
  // lanes of an MFMA operand read consecutive rows at the same chunk, so the
  // swizzle must spread any 8 (128-byte rows: any 16 over a row pair)
  // consecutive rows over distinct bank groups.
  static __device__ __forceinline__ int row_swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
  static __device__ __forceinline__ int k_idx(int r, int c) {
    return r * KCH + (D == 64 ? (c ^ row_swz128(r)) : (c ^ (r & 15)));
  }
  static __device__ __forceinline__ int v_idx(int d, int c) { return K_CH + d * 8 + (c ^ row_swz128(d)); }
};

// The per-lane part of a wave's copy address, the same for every tile and
// round: a K wave's lane fetches chunk `lo` (in elements) of the K tile; a V
// wave's lane fetches the chunk at column offset `lo` of V^T row `hi`, whose
// pitch is the segment's T_pad.
struct CopyLane {
  unsigned lo, hi;
};

template <int D, int S>
__device__ __forceinline__ CopyLane copy_lane(int wave, int lane) {
  using T = Tile<D, S>;
  CopyLane cl;
  if (wave < T::KW) {
    const int p = wave * 64 + lane;               // LDS chunk of the first round
    const int r = p / T::KCH, pos = p % T::KCH;
    const int ch = D == 64 ? (pos ^ T::row_swz128(r)) : (pos ^ (r & 15));
    cl.lo = (unsigned)(key_of_row(r) * D + ch * 8);
    cl.hi = 0u;
  } else {
    const int pv = (wave - T::KW) * 64 + lane;    // V^T chunk of the first round
    const int d = pv / 8, pos = pv % 8;
    cl.lo = (unsigned)((pos ^ T::row_swz128(d)) * 8);
    cl.hi = (unsigned)d;
  }
  return cl;
}

// Stream one K tile and one V^T tile straight from global memory into the LDS
// buffer at byte address buf_lds (global_load_lds_dwordx4: lane i of a wave
// fills the i-th 16 bytes after the wave's LDS base, held in M0).  The swizzle
// is applied by choosing which global chunk each lane fetches for its fixed
// LDS position.  Each wave copies K only or V^T only, so its lane offsets are
// fixed (CopyLane, one multiply-add per tile for the V^T row pitch) and its
// rounds differ by a uniform step of the base address.  Completion is waited
// for with vmcnt before the barrier that publishes the buffer.
template <int D, int S>
__device__ __forceinline__ void load_tile(const Cursor& c, const CopyLane& cl, int wave, unsigned buf_lds) {
  using T = Tile<D, S>;
  const bool kw = wave < T::KW;                   // wave-uniform
  const unsigned off = (cl.hi * (unsigned)c.tpad + cl.lo) * 2u;   // bytes, per lane
  const uint16_t* base = kw ? c.k + (int64_t)c.off * D : c.v + c.off;
  const int64_t step = kw ? (int64_t)T::K_ROWS_STEP * D : (int64_t)T::V_DIMS_STEP * c.tpad;
  const unsigned lds0 = buf_lds + 16u * (unsigned)(kw ? wave * 64 : T::K_CH + (wave - T::KW) * 64);
  const unsigned lds_step = 16u * 64u * (unsigned)(kw ? T::KW : T::VW);
  const int rounds = kw ? T::KR : T::VR;
#pragma unroll
  for (int r = 0; r < (T::KR > T::VR ? T::KR : T::VR); ++r) {
    if (r >= rounds) break;
    // The copy is an asm statement: it has no register result and lands in
    // LDS, which is read only after the explicit vmcnt wait and barrier that
    // publish the buffer.  Seen by the compiler as an LDS write in flight, it
    // would make every LDS read of the steps wait for all outstanding LDS
    // reads.
    const uint16_t* src = base + r * step;        // uniform
    const unsigned lds = lds0 + (unsigned)r * lds_step;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(src), "s"(lds)
                 : "memory", "m0");
  }
}

// Wait for this wave's outstanding global loads (including the LDS-direct ones).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float exchange_half(float x) {
  return __shfl_xor(x, 32);
}

// In-place select on a register the compiler must keep where it is: the tail
// fix-up modifies live scores without creating a second copy at the join.
// (Only VALU results are touched this way: a value an MFMA writes needs the
// compiler's hazard tracking, so the accumulators are scaled in plain code.)
// `keep` is a wave-uniform lane mask (bit l: lane l keeps its value).
__device__ __forceinline__ float mask_inplace(float x, uint64_t keep) {
  asm volatile("v_cndmask_b32 %0, %1, %0, %2" : "+v"(x) : "v"(-INFINITY), "s"(keep));
  return x;
}

// S^T of one 32-key group (LDS K rows 32g..32g+31) against the wave's queries.
template <int D>
__device__ __forceinline__ f32x16 scores(const u32x4* L, int lane, int g, const bf16x8 (&qf)[D / 16]) {
  using T = Tile<D>;
  const int r = 32 * g + (lane & 31);
  const int half = lane >> 5;
  f32x16 s;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 kf = as_bf16x8(L[T::k_idx(r, 2 * ks + half)]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
  }
  return s;
}

// O^T += V^T P^T for one 32-key group (LDS V^T columns 32g..32g+31).
template <int D>
__device__ __forceinline__ void accumulate(const u32x4* L, int lane, int g, const bf16x8 (&p)[2],
                                           f32x16 (&o)[D / 32]) {
  using T = Tile<D>;
  const int half = lane >> 5;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int ob = 0; ob < D / 32; ++ob) {
      const int d = 32 * ob + (lane & 31);
      const bf16x8 vf = as_bf16x8(L[T::v_idx(d, 4 * g + 2 * k2 + half)]);
      o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[k2], o[ob], 0, 0, 0);
    }
}

// Weight sums on the matrix cores (fast path).  v_mfma_f32_16x16x32_bf16
// reads its B operand as 32 (k) x 16 (n): lane l gives column l % 16, rows
// 8 (l / 16) .. + 7.  Handed the weights of one 16-key k-step in their PV
// layout (lane l: query l % 32, keys 8 (l / 32) .. + 7), lane groups 0 and 2
// hold queries 0-15 and groups 1 and 3 queries 16-31.  With A row 0 = 1 over
// k-groups 0 and 2 and row 1 = 1 over groups 1 and 3 (all else 0), output row 0
// is the k-step's weight sum of queries 0-15 and row 1 that of queries 16-31,
// in register 0 and 1 of lanes 0-15.  The sums are of the bf16 weights the PV
// product multiplies.  The A operand: ones in lanes 0 and 32 (row 0) and 17
// and 49 (row 1).
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
  const bool one = lane == 0 || lane == 32 || lane == 17 || lane == 49;
  const unsigned u = one ? 0x3F803F80u : 0u;   // two bf16 1.0
  const u32x4 v = {u, u, u, u};
  return as_bf16x8(v);
}

// The weight sum of query lane % 32 from the row-sum accumulator, in lanes
// 0-31 (lanes 32-63 get 0, so that l_sum + its other half is the total).
__device__ __forceinline__ float row_sum_of_lane(const f32x4& acc, int lane) {
  const int q = lane & 31;
  const float lo = __shfl(acc[0], q & 15);
  const float hi = __shfl(acc[1], q & 15);
  return lane < 32 ? (q < 16 ? lo : hi) : 0.f;
}

// Scaled scores of one group relative to the reference maximum m:
// score * c - m, one FMA each; keys at or past the group's `valid` count
// (>= 32: all valid) get -inf in a fix-up that only tail groups run.
__device__ __forceinline__ void scale_scores(const f32x16& s_in, float c, float m, int valid, f32x16& sc) {
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(s_in[i], c, -m);
  if (__builtin_expect(valid < 32, 0)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // key of element i: 16(i/8) + i%8 in lanes 0-31, 8 more in lanes 32-63
      const int key = 16 * (i >> 3) + (i & 7);
      const uint64_t keep = (key < valid ? 0xFFFFFFFFull : 0ull) | (key + 8 < valid ? ~0xFFFFFFFFull : 0ull);
      sc[i] = mask_inplace(sc[i], keep);
    }
  }
}

// Weights of one group from its scaled scores, shifted by `shift`: bf16
// exp2 values packed as the B operand of the PV product, and their fp32 sum.
__device__ __forceinline__ float weights(const f32x16& s, float shift, bf16x8 (&p)[2]) {
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(s[8 * k2 + i] - shift);
      const float e1 = __builtin_amdgcn_exp2f(s[8 * k2 + i + 1] - shift);
      bf16x2 pr;
      pr[0] = (__bf16)e0;
      pr[1] = (__bf16)e1;
      p[k2][i] = pr[0];
      p[k2][i + 1] = pr[1];
      la += e0;
      lb += e1;
    }
  return la + lb;
}

// One pipeline step for group k: the matrix cores take S^T of group k+1,
// O^T += V^T P^T of group k-1 and that group's weight sums (two 16x16x32
// products, see row_sum_selector) while the vector ALUs turn the raw scores
// of group k into weights.  P of group k replaces p on exit.  `valid` counts
// the group's keys that lie before its segment's end (see scale_scores).
//
// The scores are taken relative to a reference maximum m that starts as the
// chunk's first group's maximum (first_reference).  The fast form never
// moves m: the vector ALUs spend one FMA, one exponential and half a bf16
// conversion per score, nothing else.  A chunk whose weights overflow is
// detected at its end and computed again with `exact` set: then each group
// first checks for a scaled score more than 12 above m (a weight above
// 2^12; one v_max3 per three scores), and the rare raise moves m by a whole
// number, so that O, the row sums and the pending weights of group k-1 scale
// by an exact power of two, and the group's scores are scaled again.
//
// Head dim 128 has twice the matrix work per score and is bound by the
// matrix cores: there the sums are fp32 additions of the unrounded weights
// on the vector ALUs instead (kMatrixSums), the one form checks every group
// (its weight sum, which bounds its largest weight, against 2^12) after the
// MFMAs, and a raise multiplies O and the sum by exp2(-raise) and recomputes
// the group's weights.
template <int D>
__device__ __forceinline__ void pipe_step(const u32x4* Ls, int gs, const u32x4* Lp, int gp, int lane,
                                          const bf16x8 (&qf)[D / 16], float c, const f32x16& s_in,
                                          f32x16& s_out, bf16x8 (&p)[2], int valid, bool exact,
                                          const bf16x8& sel, WaveState<D>& w) {
  constexpr int NOB = D / 32;
  constexpr bool MS = kMatrixSums<D>;
  f32x16 sc;
  scale_scores(s_in, c, w.m_ref, valid, sc);
  if (MS && __builtin_expect(exact, 0)) {
    // Does any scaled score exceed 12?  Compared as integers (v_max3_i32, no
    // NaN handling): a float above 12 has a larger bit pattern than 12, a
    // negative one (and -inf) a negative pattern.
    int mb[5];
#pragma unroll
    for (int j = 0; j < 5; ++j)
      mb[j] = max(max(__float_as_int(sc[3 * j]), __float_as_int(sc[3 * j + 1])), __float_as_int(sc[3 * j + 2]));
    const int mbits = max(max(max(mb[0], mb[1]), mb[2]), max(max(mb[3], mb[4]), __float_as_int(sc[15])));
    if (__any(mbits > __float_as_int(kLazyLog2))) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      mx = fmaxf(mx, exchange_half(mx));
      const int delta = mx > 0.f ? (int)ceilf(mx) : 0;
      const float alpha = ldexpf(1.0f, -delta);
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[ob][i] *= alpha;
      // lanes 0-15 hold the sums of queries lane (register 0) and lane + 16 (1)
      const float alpha_hi = __shfl(alpha, (lane & 15) + 16);
      w.l_acc[0] *= alpha;
      w.l_acc[1] *= alpha_hi;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int i = 0; i < 8; ++i) p[k2][i] = (__bf16)((float)p[k2][i] * alpha);
      w.m_ref += (float)delta;
      scale_scores(s_in, c, w.m_ref, valid, sc);
    }
  }
  // ---- hot block: matrix cores and vector ALUs work side by side ----------
  // The wave issues in order, so the step is laid out by hand: each MFMA is
  // followed by the LDS read of the operand three MFMAs ahead and, at D = 64,
  // by its share of the weight computation (one of eight chunks: two
  // exponentials and their bf16 pair); at D = 128 the chunks all follow the
  // last MFMA (kSplitPhases).  The two row-sum products follow the first and
  // the next-to-last MFMA.  Scheduling barriers keep the compiler from
  // regrouping them.
  {
    // nothing of the LGKM counter is outstanding here: with that known, each
    // MFMA below waits only for its own operand
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    using T = Tile<D>;
    constexpr int NKS = D / 16;
    constexpr int NM = NKS + 2 * NOB;           // MFMAs of the step reading LDS operands
    constexpr int LA = kLdsAhead<D>;            // LDS reads in flight ahead of use
    const int half = lane >> 5;
    const int r = 32 * gs + (lane & 31);
    // MFMA slot m: QK^T k-step m/2 on even slots while those last, PV
    // products (k2, ob) on the others: two independent accumulator chains
    auto is_qk = [](int m) { return m < 2 * NKS && (m & 1) == 0; };
    auto pv_of = [](int m) { return m < 2 * NKS ? m / 2 : m - NKS; };
    auto operand = [&](int m) {
      if (is_qk(m)) return as_bf16x8(Ls[T::k_idx(r, 2 * (m / 2) + half)]);
      const int pv = pv_of(m), k2 = pv / NOB, ob = pv % NOB;
      return as_bf16x8(Lp[T::v_idx(32 * ob + (lane & 31), 4 * gp + 2 * k2 + half)]);
    };
    bf16x8 fr[NM];
#pragma unroll
    for (int m = 0; m < LA && m < NM; ++m) fr[m] = operand(m);
    bf16x8 pn[2];
    f32x16 s;
    float la, lb;
    // after MFMA m comes the share of the weight computation due by then
    int chunk = 0;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (is_qk(m)) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m], qf[m / 2], m == 0 ? f32x16{} : s, 0, 0, 0);
      } else {
        const int pv = pv_of(m), k2 = pv / NOB, ob = pv % NOB;
        w.o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m], p[k2], w.o[ob], 0, 0, 0);
      }
      if (m + LA < NM) fr[m + LA] = operand(m + LA);
      if constexpr (MS) {
        if (m == 0) w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[0], w.l_acc, 0, 0, 0);
        if (m == NM - 2) w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[1], w.l_acc, 0, 0, 0);
      }
      if (kSplitPhases<D> && m == NM - 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (; chunk < 8 && (kSplitPhases<D> ? m == NM - 1 : chunk * NM < 8 * (m + 1)); ++chunk) {
        const int k2 = chunk / 4, i = 2 * (chunk % 4);
        const float e0 = __builtin_amdgcn_exp2f(sc[8 * k2 + i]);
        const float e1 = __builtin_amdgcn_exp2f(sc[8 * k2 + i + 1]);
        bf16x2 pr;
        pr[0] = (__bf16)e0;
        pr[1] = (__bf16)e1;
        pn[k2][i] = pr[0];
        pn[k2][i + 1] = pr[1];
        if constexpr (!MS) {
          if (chunk == 0) {        // the first pair starts the two chains (0 + x is not folded: -0)
            la = e0;
            lb = e1;
          } else {
            la += e0;
            lb += e1;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s_out = s;
    p[0] = pn[0];
    p[1] = pn[1];
    if constexpr (!MS) {
      float l_g = la + lb;
      // the group's weight sum bounds each weight: raise the reference when large
      if (__builtin_expect(__any(l_g > kLazyThreshold), 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        mx = fmaxf(mx, exchange_half(mx));
        const float delta = fmaxf(mx, 0.f);
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        w.l_sum *= alpha;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
          for (int i = 0; i < 16; ++i) w.o[ob][i] *= alpha;
        w.m_ref += delta;
        l_g = weights(sc, delta, p);
      }
      w.l_sum += l_g;
    }
  }
}

// The reference maximum of a chunk: the largest scaled score of its first
// group among the valid keys (`valid` as in pipe_step), in both lanes of a
// query.  Its weight is exp2(0) = 1, so no sum underflows.
__device__ __forceinline__ float first_reference(const f32x16& s, float c, int valid) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = 16 * (i >> 3) + (i & 7) + 8 * (int)(__lane_id() >> 5);
    mx = key < valid ? fmaxf(mx, s[i] * c) : mx;
  }
  return fmaxf(mx, exchange_half(mx));
}

// Work unit = one 64-key tile of one task (block, head, query tile).
struct Where {
  int b;        // block
  int ti;       // task within the block (head-major, query tile fastest)
  int tile;     // first tile
};

__device__ __forceinline__ Where locate(const AttnArgs& a, int pos) {
  int b = 0;
  while (b + 1 < a.n_blocks && a.blk[b + 1].work_start <= pos) ++b;
  const int r = pos - a.blk[b].work_start;
  const int nt = a.blk[b].n_tiles;
  Where w;
  w.b = b;
  w.ti = r / nt;
  w.tile = r - w.ti * nt;
  return w;
}

template <int D, int S>
struct Partial {
  // [wave][o block][element][lane] accumulators, then [wave][lane] m, then l
  static constexpr int NW = Shape<D, S>::NW;
  static constexpr int O_FLOATS = NW * (D / 32) * 16 * 64;
  static constexpr int FLOATS = O_FLOATS + 2 * NW * 64;
};

template <int D, int S>
__device__ __forceinline__ void store_partial(float* part, int wave, int lane, const WaveState<D>& w) {
  constexpr int NOB = D / 32;
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[((wave * NOB + ob) * 16 + i) * 64 + lane] = w.o[ob][i];
  part[Partial<D, S>::O_FLOATS + wave * 64 + lane] = w.m_ref;
  part[Partial<D, S>::O_FLOATS + Partial<D, S>::NW * 64 + wave * 64 + lane] = w.l_sum;
}

// w <- w merged with the partial result at `part` (same lanes, same queries).
template <int D, int S>
__device__ __forceinline__ void merge_partial(const float* part, int wave, int lane, WaveState<D>& w) {
  constexpr int NOB = D / 32;
  const float m2 = part[Partial<D, S>::O_FLOATS + wave * 64 + lane];
  const float l2 = part[Partial<D, S>::O_FLOATS + Partial<D, S>::NW * 64 + wave * 64 + lane];
  const float m = fmaxf(w.m_ref, m2);
  // (the state being folded into starts at m = -inf: equal maxima scale by 1)
  const float a1 = w.m_ref == m ? 1.f : __builtin_amdgcn_exp2f(w.m_ref - m);
  const float a2 = m2 == m ? 1.f : __builtin_amdgcn_exp2f(m2 - m);
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w.o[ob][i] = w.o[ob][i] * a1 + part[((wave * NOB + ob) * 16 + i) * 64 + lane] * a2;
  w.l_sum = w.l_sum * a1 + l2 * a2;
  w.m_ref = m;
}

template <int D>
__device__ __forceinline__ void store_output(const AttnArgs& a, int b, int h, int qrow, bool row_ok, int half,
                                             const WaveState<D>& w) {
  constexpr int NOB = D / 32;
  const float l_tot = w.l_sum + exchange_half(w.l_sum);
  const float inv = 1.0f / l_tot;
  if (!row_ok) return;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (((int64_t)b * a.q_stride + qrow) * a.heads + h) * D;
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * ob + 8 * g4 + 4 * half;
      bf16x2 p01, p23;
      p01[0] = (__bf16)(w.o[ob][4 * g4 + 0] * inv);
      p01[1] = (__bf16)(w.o[ob][4 * g4 + 1] * inv);
      p23[0] = (__bf16)(w.o[ob][4 * g4 + 2] * inv);
      p23[1] = (__bf16)(w.o[ob][4 * g4 + 3] * inv);
      uint2 pk;
      pk.x = __builtin_bit_cast(unsigned, p01);
      pk.y = __builtin_bit_cast(unsigned, p23);
      *reinterpret_cast<uint2*>(op + d) = pk;
    }
  if (a.lse != nullptr && half == 0)
    a.lse[((int64_t)b * a.heads + h) * a.q_stride + qrow] = (w.m_ref + __log2f(l_tot)) * kLn2;
}

template <int D, int S>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Tile<D, S>::THREADS)))
__attribute__((amdgpu_waves_per_eu(Shape<D, S>::WAVES_PER_SIMD, Shape<D, S>::WAVES_PER_SIMD)))
void attention_bf16_kernel(const AttnArgs a) {
  using T = Tile<D, S>;
  constexpr int NKS = D / 16;        // k-steps of the QK^T product
  constexpr int NOB = D / 32;        // 32-row blocks of O^T
  __shared__ u32x4 lds[kBuffers][T::CH];
  // its LDS byte address, for the copies that name LDS by address
  const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)&lds[0][0];

  // ---- this workgroup's work ------------------------------------------------
  // The hardware deals workgroups round-robin to the 8 XCDs (workgroup w runs
  // on XCD w % 8).  Tasks are dealt so that each XCD works through its own
  // contiguous stretch of tasks (same block and head, neighbouring query
  // tiles, hence the same K/V stream in its L2), and a cut task is shared only
  // by workgroups of one XCD.
  const int wgid = blockIdx.x;
  const int x = wgid & 7;
  const int j_wg = wgid >> 3;                // place in the XCD's list

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const CopyLane cl = copy_lane<D, S>(wave_u, lane);
  const float c = a.qscale;

  // one range of work: a whole task, or (split) a share of the XCD's tail
  XcdPlan plan;
  int pos, end;
  bool first_chunk = true;                    // first chunk of the range
  int tail_j = 0;                             // tail workgroup index within the XCD
  if (!a.split) {
    const int t = x * a.wg_per_xcd + j_wg;
    if (t >= a.n_tasks) return;
    pos = task_work_start(a, t);
    end = pos + a.blk[locate(a, pos).b].n_tiles;
  } else {
    plan = xcd_plan(a, x);
    if (j_wg < plan.whole) {
      pos = task_work_start(a, plan.t0 + j_wg);
      end = pos + a.blk[locate(a, pos).b].n_tiles;
    } else {
      tail_j = j_wg - plan.whole;
      const int n = plan.tail1 - plan.tail0;
      if (tail_j >= a.tail_wg || n <= 0) return;
      pos = plan.tail0 + split_start(n, a.tail_wg, tail_j);
      end = plan.tail0 + split_start(n, a.tail_wg, tail_j + 1);
    }
  }

  const bf16x8 sel = row_sum_selector(lane);
  __shared__ int redo_vote;                   // a fast pass overflowed in some wave
  while (pos < end) {
    if (tid == 0) redo_vote = 0;
    // ---- the chunk: tiles [tile0, tile0 + n_tiles) of one task ----------
    const Where at = locate(a, pos);
    const AttnBlock& B = a.blk[at.b];
    const int b = at.b;
    const int h = at.ti / B.nqt;
    const int qt = at.ti - h * B.nqt;
    const int tile0 = at.tile;
    const int left = end - pos;
    const int n_tiles = B.n_tiles - tile0 < left ? B.n_tiles - tile0 : left;
    const bool whole = tile0 == 0 && n_tiles == B.n_tiles;

    const int q0 = qt * T::QTILE;
    const int qrow = q0 + wave * 32 + (lane & 31);
    const bool row_ok = qrow < B.q_len;
    const int qrow_c = row_ok ? qrow : B.q_len - 1;
    const bool active = q0 + wave * 32 < B.q_len;    // wave has queries (uniform)

    // Q fragment: B operand of S^T = K Q^T, exactly as given
    bf16x8 qf[NKS];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           (((int64_t)b * a.q_stride + qrow_c) * a.heads + h) * D;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * half));
    }

    // The chunk's pass over its key tiles, in the fast form first and, if a
    // wave of the workgroup overflowed, again in the exact one (see
    // pipe_step): the same loop, with a wave-uniform flag.
    for (int exact = 0; exact < 2; ++exact) {
      // cursor at tile0: skip whole segments, then the tiles before it
      Cursor lc;
      {
        int rem = tile0;
        int sg = 0;
        for (; sg + 1 < B.n_segs; ++sg) {
          const int nt = (B.len[sg] + kKTile - 1) / kKTile;
          if (rem < nt) break;
          rem -= nt;
        }
        lc.seg = sg;
        open_segment<D>(a, B, h, lc);
        lc.off = rem * kKTile;
      }
      Cursor cc = lc;                           // cursor of the tile being consumed
      load_tile<D, S>(lc, cl, wave_u, lds_addr);
      if (n_tiles > 1) {
        advance<D>(a, B, h, lc);
        load_tile<D, S>(lc, cl, wave_u, lds_addr + 16u * T::CH);
      }
      {
        // buffer 2 starts as zeros: the first step's deferred PV reads it
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < T::LOADS; ++u)
          if (T::CH % T::THREADS == 0 || u * T::THREADS + tid < T::CH) lds[2][u * T::THREADS + tid] = z;
      }
      WaveState<D> w;
#pragma unroll
      for (int j = 0; j < NOB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[j][i] = 0.f;
      w.m_ref = 0.f;
      w.l_sum = 0.f;
      w.l_acc = f32x4{0.f, 0.f, 0.f, 0.f};
      wait_loads();
      __syncthreads();

      // Software pipeline over 32-key groups (two per tile).  Tile t lives in
      // buffer t % 3; tile t+2 starts loading when tile t+1 is published, after
      // every wave has issued its last read of the buffer it overwrites.  Every
      // step has the same shape: the first step's deferred PV multiplies zero
      // weights with the zero-filled third buffer, and the last step's look-ahead
      // QK^T reads whatever the next buffer holds and is discarded.
      f32x16 sa, sb;                            // raw scores of even / odd groups
      bf16x8 p[2];                              // weights of the previous group
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int i = 0; i < 8; ++i) p[k2][i] = (__bf16)0.0f;
      if (active) {
        sa = scores<D>(lds[0], lane, 0, qf);
        w.m_ref = first_reference(sa, c, cc.len - cc.off);
      }
      // one tile; its buffer index is a compile-time constant so that every LDS
      // address of the steps is a per-lane base plus an immediate offset
      auto tile = [&](auto buf_c, int t) {
        constexpr int buf = decltype(buf_c)::value;
        constexpr int nbuf = buf == 2 ? 0 : buf + 1;
        constexpr int pbuf = buf == 0 ? 2 : buf - 1;
        const int valid = cc.len - cc.off;
        // group 2t: S of group 2t+1 (same tile), PV of group 2t-1 (previous tile)
        if (active)
          pipe_step<D>(lds[buf], 1, lds[pbuf], 1, lane, qf, c, sa, sb, p, valid, exact != 0, sel, w);
        if (t + 1 < n_tiles) {
          // publish tile t+1, start loading tile t+2 into the buffer of tile t-1
          wait_loads();
          __syncthreads();
          if (t + 2 < n_tiles) {
            advance<D>(a, B, h, lc);
            load_tile<D, S>(lc, cl, wave_u, lds_addr + 16u * T::CH * pbuf);
          }
          advance<D>(a, B, h, cc);
        }
        // group 2t+1: S of group 2t+2 (next tile), PV of group 2t (this tile)
        if (active)
          pipe_step<D>(lds[nbuf], 0, lds[buf], 0, lane, qf, c, sb, sa, p, valid - 32, exact != 0, sel, w);
      };
      // Tile t lives in buffer t % 3.  Whole rounds of three tiles, then the
      // remainder: a loop with one exit (with an exit after each tile the
      // compiler kept the accumulators in different registers in each copy
      // and spilled them).
      int t = 0;
      for (; t + 3 <= n_tiles; t += 3) {
        tile(std::integral_constant<int, 0>{}, t);
        tile(std::integral_constant<int, 1>{}, t + 1);
        tile(std::integral_constant<int, 2>{}, t + 2);
      }
      if (t < n_tiles) tile(std::integral_constant<int, 0>{}, t++);
      if (t < n_tiles) tile(std::integral_constant<int, 1>{}, t++);
      // the last group's PV (group 1 of the last tile)
      if (active) {
        accumulate<D>(lds[(n_tiles - 1) % 3], lane, 1, p, w.o);
        if constexpr (kMatrixSums<D>) {
          w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[0], w.l_acc, 0, 0, 0);
          w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[1], w.l_acc, 0, 0, 0);
        }
      }
      // the weight sums from the matrix cores
      if constexpr (kMatrixSums<D>) w.l_sum = row_sum_of_lane(w.l_acc, lane);
      if (kMatrixSums<D> && !exact) {
        // A fast pass overflowed where a sum or an accumulator is not
        // finite, or a sum is past 2^100 (beyond it the accumulators may
        // overflow for large values): then the whole workgroup computes the
        // chunk again in the exact form.
        float chk = w.l_sum;
#pragma unroll
        for (int j = 0; j < NOB; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) chk += w.o[j][i];
        const bool bad = active && !(__builtin_isfinite(chk) && w.l_sum < 0x1p100f);
        // the flag was cleared before this pass's first barrier and is cleared
        // again only after the chunk's closing barrier, when every wave has
        // read it; this barrier also orders every wave's last LDS read before
        // the copies of a second pass
        if (bad) redo_vote = 1;
        __syncthreads();
        if (redo_vote != 0) continue;
      }
      if (whole) {
        store_output<D>(a, b, h, qrow, row_ok, half, w);
      } else {
        // a cut task: the merge kernel combines the pieces after this launch
        store_partial<D, S>(a.partials + ((int64_t)2 * (x * a.tail_wg + tail_j) + (first_chunk ? 0 : 1)) *
                                          Partial<D, S>::FLOATS, wave, lane, w);
      }
      break;
    }
    pos += n_tiles;
    first_chunk = false;
    __syncthreads();                          // LDS buffers are reused by the next chunk
  }
}


// Second pass of the split schedule: every tail task that the tail
// workgroups cut is folded from its pieces (in workgroup order, so the result
// does not depend on timing) and normalised.  Same wave/lane layout as the
// main kernel, so each lane reads back exactly what it wrote.
template <int D, int S>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Tile<D, S>::THREADS))) void attention_merge_kernel(const AttnArgs a) {
  constexpr int NOB = D / 32;
  const int x = blockIdx.x & 7;
  const int u = blockIdx.x >> 3;
  const XcdPlan plan = xcd_plan(a, x);
  const int t = plan.t0 + plan.whole + u;
  if (t >= plan.t1) return;
  const int tstart = task_work_start(a, t);
  const Where at = locate(a, tstart);
  const AttnBlock& B = a.blk[at.b];
  const int n_tail = plan.tail1 - plan.tail0;
  const int j_lo = split_owner(n_tail, a.tail_wg, tstart - plan.tail0);
  const int j_hi = split_owner(n_tail, a.tail_wg, tstart + B.n_tiles - 1 - plan.tail0);
  if (j_lo == j_hi) return;                  // ran whole inside one tail range
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int h = at.ti / B.nqt;
  const int qt = at.ti - h * B.nqt;
  const int qrow = qt * Tile<D, S>::QTILE + wave * 32 + (lane & 31);
  WaveState<D> w;
#pragma unroll
  for (int j = 0; j < NOB; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) w.o[j][i] = 0.f;
  w.m_ref = -INFINITY;
  w.l_sum = 0.f;
  for (int oj = j_lo; oj <= j_hi; ++oj) {
    // the task opens tail workgroup oj's range (slot 0) or follows its first chunk (slot 1)
    const int slot = plan.tail0 + split_start(n_tail, a.tail_wg, oj) >= tstart ? 0 : 1;
    merge_partial<D, S>(a.partials + ((int64_t)2 * (x * a.tail_wg + oj) + slot) * Partial<D, S>::FLOATS, wave,
                     lane, w);
  }
  store_output<D>(a, at.b, h, qrow, qrow < B.q_len, half, w);
}

// ---------------------------------------------------------------------------
// Resident key sets (head dim 64, at most kResTiles tiles of 64 keys): a text
// prompt's K/V (the separate text cross-attention) or any other short key
// set.  A workgroup copies the whole key set of one (block, head) into LDS
// once and its waves then run independent units of 32 queries against it,
// with no barrier inside a unit: the per-tile copies, barriers and pipeline
// refills of the streaming kernel would otherwise recur every few tiles.
//
// Work: the launch's units in (block, head, 32-query unit) order, cut into
// one contiguous range per workgroup; the ranges of XCD x are consecutive, so
// that an XCD's workgroups share few key sets in its L2.  A range that crosses
// a (block, head) boundary runs one phase per key set: barrier, copy, barrier,
// units dealt round-robin to the waves (wave i takes units i, i + NW, ...;
// the hardware places wave i on SIMD i % 4, so the SIMDs get equal shares).
// When that costs no extra round of units per wave, each (block, head) takes
// whole workgroups instead and no range crosses (res_group_units).
// Units are never cut: measured at 5400 queries x 24 heads, sharing the
// left-over units' tiles among groups of waves (partial states folded in LDS
// or through memory) was slower than letting one wave run a unit alone.
// LDS: a zero tile, the key set's tiles, and one more tile that only the
// discarded look-ahead of the last step reads.
// ---------------------------------------------------------------------------
constexpr int kResBufs = kResTiles + 2;

template <int S>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Tile<64, S>::THREADS)))
__attribute__((amdgpu_waves_per_eu(Shape<64, S>::WAVES_PER_SIMD, Shape<64, S>::WAVES_PER_SIMD)))
void attention_resident_kernel(const AttnArgs a) {
  constexpr int D = 64;
  using T = Tile<D, S>;
  constexpr int NKS = D / 16;
  constexpr int NOB = D / 32;
  // res[0]: zeros (the first step's deferred PV); res[1 + t]: tile t
  __shared__ u32x4 res[kResBufs][T::CH];
  static_assert(sizeof(res) <= 160 * 1024, "LDS");
  const unsigned lds_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)&res[0][0];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const CopyLane cl = copy_lane<D, S>(wave_u, lane);
  const float c = a.qscale;
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u)
      if (T::CH % T::THREADS == 0 || u * T::THREADS + tid < T::CH) res[0][u * T::THREADS + tid] = z;
  }
  const int n_wg = 8 * a.wg_per_xcd;
  const int j = (blockIdx.x & 7) * a.wg_per_xcd + (blockIdx.x >> 3);
  int pos, end;
  if (a.res_group_units > 0) {
    // every (block, head) takes whole workgroups (consecutive ones, mostly
    // on one XCD) that split its units evenly: no workgroup copies a second
    // key set
    const int nu = a.res_group_units;
    const int G = a.n_tasks / nu;
    const int g = split_owner(n_wg, G, j);
    const int g0 = split_start(n_wg, G, g);
    const int nk = split_start(n_wg, G, g + 1) - g0;
    pos = g * nu + split_start(nu, nk, j - g0);
    end = g * nu + split_start(nu, nk, j - g0 + 1);
  } else {
    pos = split_start(a.n_tasks, n_wg, j);
    end = split_start(a.n_tasks, n_wg, j + 1);
  }
  const bf16x8 sel = row_sum_selector(lane);

  while (pos < end) {
    // the phase: units [u0, u0 + n) of (block b, head h)
    int b = 0;
    while (b + 1 < a.n_blocks && a.blk[b + 1].task_start <= pos) ++b;
    const AttnBlock& B = a.blk[b];
    const int r = pos - B.task_start;
    const int h = r / B.nqt;
    const int u0 = r - h * B.nqt;
    const int n = end - pos < B.nqt - u0 ? end - pos : B.nqt - u0;
    const int n_tiles = B.n_tiles;

    // copy the key set (every wave's reads of the previous one are done);
    // vt packs each tile's count of keys before its segment's end, capped
    // at 64, in 7 bits
    __syncthreads();
    uint64_t vt = 0;
    {
      Cursor lc;
      lc.seg = 0;
      open_segment<D>(a, B, h, lc);
      for (int t = 0; t < n_tiles; ++t) {
        const int v = lc.len - lc.off;
        vt |= (uint64_t)(v < kKTile ? v : kKTile) << (7 * t);
        load_tile<D, S>(lc, cl, wave_u, lds_addr + 16u * T::CH * (1 + t));
        if (t + 1 < n_tiles) advance<D>(a, B, h, lc);
      }
    }
    wait_loads();
    __syncthreads();

    for (int i = wave_u; i < n; i += T::NW) {
      const int qrow = (u0 + i) * 32 + (lane & 31);
      const bool row_ok = qrow < B.q_len;
      const int qrow_c = row_ok ? qrow : B.q_len - 1;
      bf16x8 qf[NKS];
      {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             (((int64_t)b * a.q_stride + qrow_c) * a.heads + h) * D;
#pragma unroll
        for (int s = 0; s < NKS; ++s)
          qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * half));
      }
      // fast form first; the exact one if this wave's weights overflowed
      for (int exact = 0; exact < 2; ++exact) {
        WaveState<D> w;
#pragma unroll
        for (int jj = 0; jj < NOB; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) w.o[jj][e] = 0.f;
        w.l_sum = 0.f;
        w.l_acc = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x16 sa, sb;
        bf16x8 p[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int e = 0; e < 8; ++e) p[k2][e] = (__bf16)0.0f;
        sa = scores<D>(res[1], lane, 0, qf);
        w.m_ref = first_reference(sa, c, (int)(vt & 127));
        // A run of tiles from `base` = the LDS buffer before the first: the
        // previous, current and next buffers of each tile sit at fixed
        // offsets from it (every operand address is a per-lane base plus an
        // immediate).  Two tiles per round, then the odd one.
        auto tile = [&](const u32x4* base, auto k_c, int t) {
          constexpr int k = decltype(k_c)::value;
          const int valid = (int)((vt >> (7 * t)) & 127);
          pipe_step<D>(base + (k + 1) * T::CH, 1, base + k * T::CH, 1, lane, qf, c, sa, sb, p, valid,
                       exact != 0, sel, w);
          pipe_step<D>(base + (k + 2) * T::CH, 0, base + (k + 1) * T::CH, 0, lane, qf, c, sb, sa, p,
                       valid - 32, exact != 0, sel, w);
        };
        int t = 0;
        for (; t + 2 <= n_tiles; t += 2) {
          const u32x4* base = res[t];
          tile(base, std::integral_constant<int, 0>{}, t);
          tile(base, std::integral_constant<int, 1>{}, t + 1);
        }
        if (t < n_tiles) tile(res[t], std::integral_constant<int, 0>{}, t);
        // the last group's PV (group 1 of the last tile)
        accumulate<D>(res[n_tiles], lane, 1, p, w.o);
        w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[0], w.l_acc, 0, 0, 0);
        w.l_acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p[1], w.l_acc, 0, 0, 0);
        w.l_sum = row_sum_of_lane(w.l_acc, lane);
        if (!exact) {
          // overflow check of the fast form, as in the streaming kernel, but
          // per wave: the key set in LDS is read-only, so a wave can run its
          // unit again alone
          float chk = w.l_sum;
#pragma unroll
          for (int jj = 0; jj < NOB; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) chk += w.o[jj][e];
          const bool bad = !(__builtin_isfinite(chk) && w.l_sum < 0x1p100f);
          if (__builtin_amdgcn_ballot_w64(bad) != 0) continue;
        }
        store_output<D>(a, b, h, qrow, row_ok, half, w);
        break;
      }
    }
    pos += n;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one query per lane, exact running maximum, VALU only.
// ---------------------------------------------------------------------------
constexpr int kF32QTile = 64;

template <int D>
__global__ __launch_bounds__(kF32QTile) void attention_f32_kernel(const AttnArgs a) {
  __shared__ float ks[kKTile][D + 1];
  __shared__ float vs[D][kKTile + 1];
  const int w = blockIdx.x;
  const int task = (w & 7) * a.tasks_per_xcd + (w >> 3);
  if (task >= a.total_tasks) return;
  const int qt = task % a.n_qtiles;
  const int h = (task / a.n_qtiles) % a.heads;
  const int b = task / (a.n_qtiles * a.heads);
  const AttnBlock& B = a.blk[b];
  const int q0 = qt * kF32QTile;
  if (q0 >= B.q_len) return;
  const int tid = threadIdx.x;
  const int qrow = q0 + tid;
  const bool row_ok = qrow < B.q_len;
  const int qrow_c = row_ok ? qrow : B.q_len - 1;

  float q[D], o[D];
  const float* qp = static_cast<const float*>(a.q) + (((int64_t)b * a.q_stride + qrow_c) * a.heads + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qp[d] * a.qscale;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int sg = 0; sg < B.n_segs; ++sg) {
    const int s = B.slot[sg];
    const float* base;
    int tpad;
    int64_t slot;
    if (s >= 0) { base = static_cast<const float*>(a.cache); tpad = a.cache_tpad; slot = s; }
    else { base = static_cast<const float*>(a.text); tpad = a.text_tpad; slot = -1 - s; }
    const float* kp = base + ((slot * 2 + 0) * a.heads + h) * (int64_t)tpad * D;
    const float* vp = base + ((slot * 2 + 1) * a.heads + h) * (int64_t)tpad * D;
    const int len = B.len[sg];
    for (int off = 0; off < len; off += kKTile) {
      __syncthreads();
      for (int e = tid; e < kKTile * D; e += kF32QTile) {
        const int r = e / D, d = e % D;
        ks[r][d] = kp[(int64_t)(off + r) * D + d];
      }
      for (int e = tid; e < kKTile * D; e += kF32QTile) {
        const int d = e / kKTile, t = e % kKTile;
        vs[d][t] = vp[(int64_t)d * tpad + off + t];
      }
      __syncthreads();
      const int valid = len - off < kKTile ? len - off : kKTile;
      for (int t = 0; t < valid; ++t) {
        float sc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) sc = __builtin_fmaf(q[d], ks[t][d], sc);
        if (sc > m) {
          const float alpha = exp2f(m - sc);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] *= alpha;
          m = sc;
        }
        const float p = exp2f(sc - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[d][t], o[d]);
      }
    }
  }
  if (row_ok) {
    float* op = static_cast<float*>(a.out) + (((int64_t)b * a.q_stride + qrow) * a.heads + h) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
    if (a.lse != nullptr)
      a.lse[((int64_t)b * a.heads + h) * a.q_stride + qrow] = (m + log2f(l)) * kLn2;
  }
}

}  // namespace

// shape: 0 wide, 1 narrow, 2 resident (head_dim 64 only)
int attention_bf16_q_tile(int head_dim, int shape) {
  if (head_dim == 128) return Tile<128, 0>::QTILE;
  return shape == 2 ? 32 : shape ? Tile<64, 1>::QTILE : Tile<64, 0>::QTILE;
}
int attention_f32_q_tile() { return kF32QTile; }
size_t attention_partial_bytes(int head_dim, int shape) {
  if (shape == 2) return 0;     // pieces are folded in LDS
  return sizeof(float) *
         (head_dim == 128 ? Partial<128, 0>::FLOATS : shape ? Partial<64, 1>::FLOATS : Partial<64, 0>::FLOATS);
}

hipError_t attention_bf16_resident(int head_dim, int shape, int* per_cu) {
  if (head_dim == 128)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, attention_bf16_kernel<128, 0>, Tile<128, 0>::THREADS, 0);
  if (shape == 2)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, attention_resident_kernel<2>, Tile<64, 2>::THREADS, 0);
  if (shape)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, attention_bf16_kernel<64, 1>, Tile<64, 1>::THREADS, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, attention_bf16_kernel<64, 0>, Tile<64, 0>::THREADS, 0);
}

namespace {
template <int D, int S>
hipError_t launch_shape(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attention_bf16_kernel<D, S>), dim3(8 * a.wg_per_xcd), dim3(Tile<D, S>::THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.split || a.merge_per_xcd == 0) return e;
  hipLaunchKernelGGL((attention_merge_kernel<D, S>), dim3(8 * a.merge_per_xcd), dim3(Tile<D, S>::THREADS), 0, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attention_bf16(const AttnArgs& a, int head_dim, int shape, hipStream_t s) {
  if (head_dim == 128) return launch_shape<128, 0>(a, s);
  if (shape == 2) {
    hipLaunchKernelGGL(attention_resident_kernel<2>, dim3(8 * a.wg_per_xcd), dim3(Tile<64, 2>::THREADS), 0, s, a);
    return hipGetLastError();
  }
  return shape ? launch_shape<64, 1>(a, s) : launch_shape<64, 0>(a, s);
}

hipError_t launch_attention_f32(const AttnArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(8 * a.tasks_per_xcd);
  if (head_dim == 64)
    hipLaunchKernelGGL(attention_f32_kernel<64>, grid, dim3(kF32QTile), 0, s, a);
  else
    hipLaunchKernelGGL(attention_f32_kernel<128>, grid, dim3(kF32QTile), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
