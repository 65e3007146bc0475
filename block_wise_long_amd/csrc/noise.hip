// Coordinated noise initialisation, device part: a new block's latent frames
// gathered from the noise pool every GPU shares ("Minute-Long Videos with
// Dual Parallelisms", Abstract: initial noise patterns shared across GPUs; the
// pith.science verdict on it, pith_inferences: a full noise pool, shuffled
// assignment, the last few latents excluded).  The assignment itself is host
// bookkeeping (ba_noise_assign); this kernel is a streaming copy bound by HBM
// bandwidth: one 16-byte vector per thread and iteration, nontemporal.
#include "internal.h"

namespace ba {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// grid.y = channel * block_frames + frame; x covers the frame's vectors
__global__ __launch_bounds__(256) void noise_gather_kernel(const NoiseArgs a) {
  const int cf = blockIdx.y;
  const int c = cf / a.block_frames;
  const int f = cf - c * a.block_frames;
  const u32x4* src = a.pool + ((int64_t)c * a.pool_frames + a.frames[f]) * a.frame_vecs;
  u32x4* dst = a.out + (int64_t)cf * a.frame_vecs;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < a.frame_vecs; v += step)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
}

}  // namespace

hipError_t launch_noise(const NoiseArgs& a, hipStream_t s) {
  int64_t bx = (a.frame_vecs + 255) / 256;
  if (bx > 4096) bx = 4096;
  const dim3 grid((unsigned)bx, (unsigned)(a.channels * a.block_frames));
  hipLaunchKernelGGL(noise_gather_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
