// CTC head tail for gfx950: per-frame log-softmax + argmax, and greedy collapse.
// "GigaAM MLX port for Mac" (Russian page), signal path: the CTC layer gives the log of
// each character's probability per step; decoding removes repeats and blank symbols.
// "GigaAM v3 RNNT - MLX" card, Notes: blank = len(vocabulary) = n_classes - 1.
#include "kernels.h"

namespace gg {

// a row of up to 64 * kLsmRegs classes is held in registers
constexpr int kLsmRegs = 8;

// One wave per padded output row (b, t). Rows t >= U_b are zero / -1.

__global__ void __launch_bounds__(256) k_logsoftmax_argmax(const float* __restrict__ logits,
                                                           int C, int B, int U_max,
                                                           const int* __restrict__ cuU,
                                                           float* __restrict__ logp,
                                                           int* __restrict__ frame_ids) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= B * U_max) return;
  const int b = row / U_max, t = row - b * U_max;
  const int Ub = cuU[b + 1] - cuU[b];
  float* out = logp + (long)row * C;
  if (t >= Ub) {
    for (int c = lane; c < C; c += 64) out[c] = 0.f;
    if (lane == 0) frame_ids[row] = -1;
    return;
  }
  const float* z = logits + (long)(cuU[b] + t) * C;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  if (C <= 64 * kLsmRegs) {
    // the row in registers, all its loads issued together (columns past C clamped, unused)
    float zv[kLsmRegs];
#pragma unroll
    for (int j = 0; j < kLsmRegs; ++j) {
      const int c = lane + 64 * j;
      zv[j] = z[c < C ? c : C - 1];
    }
#pragma unroll
    for (int j = 0; j < kLsmRegs; ++j) {
      const int c = lane + 64 * j;
      if (c < C && zv[j] > best) { best = zv[j]; bi = c; }   // ascending c: first max wins per lane
    }
    wave_argmax(best, bi);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kLsmRegs; ++j)
      if (lane + 64 * j < C) s += expf(zv[j] - best);
    s = wave_sum(s);
    const float lse = best + logf(s);
#pragma unroll
    for (int j = 0; j < kLsmRegs; ++j)
      if (lane + 64 * j < C) out[lane + 64 * j] = zv[j] - lse;
  } else {
    for (int c = lane; c < C; c += 64) {
      const float v = z[c];
      if (v > best) { best = v; bi = c; }
    }
    wave_argmax(best, bi);
    float s = 0.f;
    for (int c = lane; c < C; c += 64) s += expf(z[c] - best);
    s = wave_sum(s);
    const float lse = best + logf(s);
    for (int c = lane; c < C; c += 64) out[c] = z[c] - lse;
  }
  if (lane == 0) frame_ids[row] = bi;
}

// One wave per clip: keep frame t if id_t != blank and (t == 0 or id_t != id_{t-1});
// kept ids are compacted in order with a ballot prefix count.
__global__ void __launch_bounds__(64) k_collapse(const int* __restrict__ frame_ids, int U_max,
                                                 const int* __restrict__ cuU, int blank,
                                                 int* __restrict__ tokens,
                                                 int* __restrict__ n_tokens) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int Ub = cuU[b + 1] - cuU[b];
  const int* ids = frame_ids + (long)b * U_max;
  int* out = tokens + (long)b * U_max;
  int n = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int t0 = 0; t0 < Ub; t0 += 64) {
    const int t = t0 + lane;
    bool keep = false;
    int id = blank;
    if (t < Ub) {
      id = ids[t];
      const int prev = t > 0 ? ids[t - 1] : -1;
      keep = (id != blank) && (id != prev);
    }
    const unsigned long long m = __ballot(keep);
    if (keep) out[n + __popcll(m & below)] = id;
    n += __popcll(m);
  }
  for (int t = n + lane; t < U_max; t += 64) out[t] = -1;
  if (lane == 0) n_tokens[b] = n;
}

// Packed [sum U_b][d] -> padded [B][U_max][d], zero rows beyond each clip.
__global__ void __launch_bounds__(256) k_scatter_rows(const float* __restrict__ x, int d, int B,
                                                      int U_max, const int* __restrict__ cuU,
                                                      float* __restrict__ out) {
  const long n4 = (long)B * U_max * (d / 4);
  for (long e = blockIdx.x * 256L + threadIdx.x; e < n4; e += (long)gridDim.x * 256) {
    const long row = e / (d / 4);
    const int c4 = (int)(e - row * (d / 4));
    const int b = (int)(row / U_max), t = (int)(row - (long)b * U_max);
    const int Ub = cuU[b + 1] - cuU[b];
    f32x4 v = f32x4{0, 0, 0, 0};
    if (t < Ub) v = *(const f32x4*)(x + (long)(cuU[b] + t) * d + 4 * c4);
    *(f32x4*)(out + row * d + 4 * c4) = v;
  }
}

hipError_t launch_logsoftmax_argmax(const float* logits, int C, int B, int U_max,
                                    const int* cuU, float* logp, int* frame_ids,
                                    hipStream_t s) {
  const int rows = B * U_max;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_logsoftmax_argmax, dim3((rows + 3) / 4), dim3(256), 0, s, logits, C, B,
                     U_max, cuU, logp, frame_ids);
  return hipGetLastError();
}

hipError_t launch_collapse(const int* frame_ids, int B, int U_max, const int* cuU, int blank,
                           int* tokens, int* n_tokens, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_collapse, dim3(B), dim3(64), 0, s, frame_ids, U_max, cuU, blank, tokens,
                     n_tokens);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* x, int d, int B, int U_max, const int* cuU,
                               float* out, hipStream_t s) {
  const long n4 = (long)B * U_max * (d / 4);
  if (n4 <= 0) return hipSuccess;
  long blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_scatter_rows, dim3((unsigned)blocks), dim3(256), 0, s, x, d, B, U_max, cuU,
                     out);
  return hipGetLastError();
}

}  // namespace gg
