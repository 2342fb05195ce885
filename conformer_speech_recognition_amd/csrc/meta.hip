// Batch geometry on the device: clip offsets and row -> clip maps of the packed
// mel (T), first-conv (S) and encoder (U) row spaces, plus the 64-frame tiles (depthwise
// conv, with each tile's clip geometry in one 16-byte record) and 128-frame query tiles
// (attention, numbered longest clip first) of every clip.
// Variable-length clips are packed back to back so every per-frame kernel touches valid
// frames only (batched chunks with masks: "GigaAM MLX port for Mac", section "What is
// inside the model").
#include "kernels.h"

namespace gg {

__device__ __forceinline__ int find_clip(const int* cu, int B, int r) {
  int lo = 0, hi = B - 1;                 // largest b with cu[b] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256) k_meta(MetaArgs a, MetaDev m, int T_tot, int S_tot,
                                              int U_tot) {
  __shared__ int cuQ[kMaxBatch + 1];
  __shared__ int cuQ2[kMaxBatch + 1];     // indexed by clip
  __shared__ int cuQ2s[kMaxBatch + 1];    // indexed by rank
  __shared__ int order[kMaxBatch];        // clips by length, longest first (ties: index)
  // The 128-frame query tiles are numbered clip by clip in that order, so the attention
  // grid (dispatched in tile order) starts the longest clips' work first and ends on the
  // shortest: the last, partly filled round of workgroups is the cheapest.
  for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
    const int Ub = a.cuU[b + 1] - a.cuU[b];
    int r = 0;
    for (int k = 0; k < a.B; ++k) {
      const int Uk = a.cuU[k + 1] - a.cuU[k];
      r += (Uk > Ub) || (Uk == Ub && k < b);
    }
    order[r] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int q = 0, q2 = 0;
    for (int b = 0; b < a.B; ++b) {
      cuQ[b] = q;
      q += (a.cuU[b + 1] - a.cuU[b] + kQTile - 1) / kQTile;
    }
    cuQ[a.B] = q;
    for (int i = 0; i < a.B; ++i) {
      const int b = order[i];
      cuQ2s[i] = q2;
      cuQ2[b] = q2;
      q2 += (a.cuU[b + 1] - a.cuU[b] + kQTile2 - 1) / kQTile2;
    }
    cuQ2s[a.B] = q2;
    cuQ2[a.B] = q2;
  }
  __syncthreads();
  const int nQ = cuQ[a.B], nQ2 = cuQ2[a.B];
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b <= a.B; b += blockDim.x) {
      m.cuT[b] = a.cuT[b]; m.cuS[b] = a.cuS[b]; m.cuU[b] = a.cuU[b]; m.cuQ[b] = cuQ[b];
      m.cuQ2[b] = cuQ2[b];
    }
  }
  const int stride = gridDim.x * blockDim.x;
  for (int r = gid; r < T_tot; r += stride) m.rowT[r] = find_clip(a.cuT, a.B, r);
  for (int r = gid; r < S_tot; r += stride) m.rowS[r] = find_clip(a.cuS, a.B, r);
  for (int r = gid; r < U_tot; r += stride) {
    const int b = find_clip(a.cuU, a.B, r);
    m.rowU[r] = b;
    if (m.posU) m.posU[r] = r - a.cuU[b];
  }
  for (int r = gid; r < nQ; r += stride) {
    const int b = find_clip(cuQ, a.B, r);
    m.tileQ[r] = b;
    if (m.tileG) {
      const int4 g = {a.cuU[b], a.cuU[b + 1] - a.cuU[b], (r - cuQ[b]) * kQTile, b};
      *(int4*)(m.tileG + 4 * r) = g;
    }
  }
  for (int r = gid; r < nQ2; r += stride) m.tileQ2[r] = order[find_clip(cuQ2s, a.B, r)];
}

hipError_t launch_meta(const MetaArgs& a, const MetaDev& m, int T_tot, int S_tot, int U_tot,
                       hipStream_t s) {
  int blocks = (T_tot + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 512 ? 512 : blocks);
  hipLaunchKernelGGL(k_meta, dim3(blocks), dim3(256), 0, s, a, m, T_tot, S_tot, U_tot);
  return hipGetLastError();
}

}  // namespace gg

namespace gg {

// Plain device copy of n floats (the streaming ring's moves and appends); the ranges
// never overlap.
__global__ void __launch_bounds__(256) k_copy_f32(float* __restrict__ dst,
                                                  const float* __restrict__ src, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_copy_f32(float* dst, const float* src, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_copy_f32, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace gg
