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
//   * workgroup = 4 waves = 128 queries of one (block, head); wave = 32 queries.
//   * S^T = K Q^T is computed per 32-key group, so that a lane owns one
//     query column and 16 of its scores: every per-query softmax quantity is
//     lane-local (lanes l and l^32 share a query), and O^T = V^T P^T leaves the
//     output of a query in the lanes that hold its weights.  Q and K enter the
//     MFMA exactly as given; the scale c = scale*log2(e) and the reference
//     maximum are applied to the fp32 scores by one FMA each, so the score
//     error does not grow with the score's magnitude.
//   * The running maximum is lazy: scores are taken relative to a reference m
//     that is raised only when a tile's weights would exceed 2^12 (checked on
//     the tile's weight sum, which bounds its largest weight), so the common
//     path spends one FMA and one v_exp_f32 per score and no max at all.  The
//     result is exact softmax: out = (sum p v) / (sum p) with a common m.
//   * The weights are rounded to bf16 for the PV product and summed from those
//     rounded values (v_dot2_f32_bf16 against 1.0), so numerator and
//     denominator see the same weights.
//   * K and V^T tiles of 64 keys are double-buffered in LDS with an XOR
//     swizzle of 16-byte chunks (conflict-free ds_read_b128 for the MFMA
//     operands); the next tile's global loads are in flight while the current
//     tile computes.  One barrier per tile.
//   * Workgroups are mapped to tasks XCD-major: the hardware deals workgroups
//     round-robin to the 8 XCDs, so consecutive tasks (same block and head,
//     neighbouring query tiles, hence the same K/V stream) share an XCD's L2.
//
// fp32 kernel: plain VALU, one query per lane, exact running maximum; used for
// fp32 rings (small shapes, parity at 1e-5).
#include <math.h>

#include "internal.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQTile = 128;        // queries per workgroup (4 waves x 32)
constexpr int kKTile = 64;         // keys per LDS tile
constexpr int kThreads = 256;
constexpr float kLazyThreshold = 4096.0f;   // 2^12: bound on a tile's weight sum
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
}

template <int D>
__device__ __forceinline__ void advance(const AttnArgs& a, const AttnBlock& B, int h, Cursor& c) {
  c.off += kKTile;
  if (c.off >= c.len) {
    ++c.seg;
    if (c.seg < B.n_segs) open_segment<D>(a, B, h, c);
  }
}

template <int D>
struct Tile {
  static constexpr int KCH = D / 8;                  // 16-B chunks per K row
  static constexpr int K_CH = kKTile * KCH;          // chunks of the K tile
  static constexpr int V_CH = D * (kKTile / 8);      // chunks of the V^T tile
  static constexpr int CH = K_CH + V_CH;
  static constexpr int K_LOADS = K_CH / kThreads;
  static constexpr int LOADS = CH / kThreads;
  static_assert(K_CH % kThreads == 0 && V_CH % kThreads == 0, "tile shape");

  // LDS chunk index of K row r, chunk c / V^T row d, chunk c (XOR swizzle).
  static __device__ __forceinline__ int k_idx(int r, int c) { return r * KCH + (c ^ (r & 7)); }
  static __device__ __forceinline__ int v_idx(int d, int c) { return K_CH + d * 8 + (c ^ (d & 7)); }
};

template <int D>
__device__ __forceinline__ void load_tile(const Cursor& c, int tid, u32x4 (&st)[Tile<D>::LOADS]) {
  using T = Tile<D>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int g = tid + u * kThreads;
    if (u < T::K_LOADS) {
      const int r = g / T::KCH, ch = g % T::KCH;
      const int key = c.off + key_of_row(r);
      st[u] = *reinterpret_cast<const u32x4*>(c.k + (int64_t)key * D + ch * 8);
    } else {
      const int gv = g - T::K_CH;
      const int d = gv / 8, ch = gv % 8;
      st[u] = *reinterpret_cast<const u32x4*>(c.v + (int64_t)d * c.tpad + c.off + ch * 8);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(u32x4* lds, int tid, const u32x4 (&st)[Tile<D>::LOADS]) {
  using T = Tile<D>;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int g = tid + u * kThreads;
    if (u < T::K_LOADS) {
      const int r = g / T::KCH, ch = g % T::KCH;
      lds[T::k_idx(r, ch)] = st[u];
    } else {
      const int gv = g - T::K_CH;
      const int d = gv / 8, ch = gv % 8;
      lds[T::v_idx(d, ch)] = st[u];
    }
  }
}

__device__ __forceinline__ float exchange_half(float x) {
  return __shfl_xor(x, 32);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attention_bf16_kernel(const AttnArgs a) {
  using T = Tile<D>;
  constexpr int NKS = D / 16;        // k-steps of the QK^T product
  constexpr int NOB = D / 32;        // 32-row blocks of O^T
  __shared__ u32x4 lds[2][T::CH];

  // ---- task (XCD-major order) ---------------------------------------------
  const int w = blockIdx.x;
  const int task = (w & 7) * a.tasks_per_xcd + (w >> 3);
  if (task >= a.total_tasks) return;
  const int qt = task % a.n_qtiles;
  const int h = (task / a.n_qtiles) % a.heads;
  const int b = task / (a.n_qtiles * a.heads);
  const AttnBlock& B = a.blk[b];
  const int q0 = qt * kQTile;
  if (q0 >= B.q_len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = tid >> 6;
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool row_ok = qrow < B.q_len;
  const int qrow_c = row_ok ? qrow : B.q_len - 1;

  // ---- Q fragment: B operand of S^T = K Q^T, exactly as given ---------------
  bf16x8 qf[NKS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)b * a.q_stride + qrow_c) * a.heads + h) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s + 8 * half));
  }
  const float c = a.qscale;

  // ---- key tiles ----------------------------------------------------------
  int n_tiles = 0;
  for (int sg = 0; sg < B.n_segs; ++sg) n_tiles += (B.len[sg] + kKTile - 1) / kKTile;

  Cursor cur;
  cur.seg = 0;
  open_segment<D>(a, B, h, cur);
  u32x4 st[T::LOADS];
  load_tile<D>(cur, tid, st);
  store_tile<D>(lds[0], tid, st);
  __syncthreads();

  f32x16 o[NOB];
#pragma unroll
  for (int j = 0; j < NOB; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[j][i] = 0.f;
  float m_ref = 0.f;     // reference maximum (exp2 domain), same for lanes l, l^32
  float l_sum = 0.f;     // this lane's share of the weight sum

  bf16x2 ones2;
  ones2[0] = (__bf16)1.0f;
  ones2[1] = (__bf16)1.0f;

  Cursor nxt = cur;
  for (int j = 0; j < n_tiles; ++j) {
    const bool has_next = j + 1 < n_tiles;
    if (has_next) {
      advance<D>(a, B, h, nxt);
      load_tile<D>(nxt, tid, st);
    }
    const u32x4* L = lds[j & 1];
    const int valid = cur.len - cur.off;   // >= 1; a full tile when >= 64

    // S^T for the two 32-key groups of the tile
    f32x16 s[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[g][i] = 0.f;
      const int r = 32 * g + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kf = as_bf16x8(L[T::k_idx(r, 2 * ks + half)]);
        s[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[g], 0, 0, 0);
      }
    }
    // scores in the exp2 domain, relative to the reference maximum
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[g][i] = __builtin_fmaf(s[g][i], c, -m_ref);
    if (valid < kKTile) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * g + 16 * (i >> 3) + 8 * half + (i & 7);
          if (key >= valid) s[g][i] = -INFINITY;
        }
    }

    // weights, rounded to bf16, and their sum
    bf16x8 pb[2][2];
    float l_tile = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          bf16x2 pr;
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(s[g][8 * k2 + i]);
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(s[g][8 * k2 + i + 1]);
          pb[g][k2][i] = pr[0];
          pb[g][k2][i + 1] = pr[1];
          l_tile = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_tile, false);
        }

    // raise the reference maximum when the tile's weights got too large
    // (always on the first tile, which sets it)
    const bool need = (j == 0) || (l_tile > kLazyThreshold);
    if (__any(need)) {
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[g][i]);
      mx = fmaxf(mx, exchange_half(mx));
      const float delta = (j == 0) ? mx : fmaxf(mx, 0.f);
      if (j != 0) {
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        l_sum *= alpha;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[ob][i] *= alpha;
      }
      m_ref += delta;
      l_tile = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            bf16x2 pr;
            pr[0] = (__bf16)__builtin_amdgcn_exp2f(s[g][8 * k2 + i] - delta);
            pr[1] = (__bf16)__builtin_amdgcn_exp2f(s[g][8 * k2 + i + 1] - delta);
            pb[g][k2][i] = pr[0];
            pb[g][k2][i + 1] = pr[1];
            l_tile = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_tile, false);
          }
    }
    l_sum += l_tile;

    // O^T += V^T P^T
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) {
          const int d = 32 * ob + (lane & 31);
          const bf16x8 vf = as_bf16x8(L[T::v_idx(d, 4 * g + 2 * k2 + half)]);
          o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[g][k2], o[ob], 0, 0, 0);
        }

    if (has_next) store_tile<D>(lds[(j + 1) & 1], tid, st);
    __syncthreads();
    cur = nxt;
  }

  // ---- epilogue: normalise, round to bf16, store --------------------------
  const float l_tot = l_sum + exchange_half(l_sum);
  const float inv = 1.0f / l_tot;
  if (row_ok) {
    uint16_t* op = static_cast<uint16_t*>(a.out) +
                   (((int64_t)b * a.q_stride + qrow) * a.heads + h) * D;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * ob + 8 * g4 + 4 * half;
        bf16x2 p01, p23;
        p01[0] = (__bf16)(o[ob][4 * g4 + 0] * inv);
        p01[1] = (__bf16)(o[ob][4 * g4 + 1] * inv);
        p23[0] = (__bf16)(o[ob][4 * g4 + 2] * inv);
        p23[1] = (__bf16)(o[ob][4 * g4 + 3] * inv);
        uint2 pk;
        pk.x = __builtin_bit_cast(unsigned, p01);
        pk.y = __builtin_bit_cast(unsigned, p23);
        *reinterpret_cast<uint2*>(op + d) = pk;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[((int64_t)b * a.heads + h) * a.q_stride + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
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

int attention_bf16_q_tile() { return kQTile; }
int attention_f32_q_tile() { return kF32QTile; }

hipError_t launch_attention_bf16(const AttnArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(8 * a.tasks_per_xcd);
  if (head_dim == 64)
    hipLaunchKernelGGL(attention_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attention_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
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
