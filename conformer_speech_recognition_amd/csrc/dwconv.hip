// Conformer convolution module, middle part, for gfx950:
//   depthwise Conv1d (kernel K, 'same' zero padding inside each clip) + BatchNorm with
//   running statistics (folded to a per-channel affine in the kernel) + SiLU.
// (The GLU before it is fused into the pointwise-1 GEMM epilogue.) "GigaAM MLX port for
// Mac", section "Where the time goes": the convolution module is ~17% of a block.
//
// Block = 64 frames x 64 channels of one clip. The (64 + K - 1) x 64 input window is
// staged once in LDS in the storage type (zeros outside the clip); each thread then
// slides its channel over 16 consecutive frames with the whole window in fp32
// registers. The taps are stored tap-major so a wave's lanes read consecutive channels.
#include "kernels.h"

namespace gg {

template <typename T, int K>
__global__ void __launch_bounds__(256) k_dw(DwParams p) {
  constexpr int TT = 64, CH = 64, HALF = (K - 1) / 2, R = TT + K - 1, TPT = 16;
  // the window is staged in the storage type (12 KiB for 16-bit types: 8 blocks per CU)
  __shared__ __attribute__((aligned(16))) T sx[R][CH + 16 / sizeof(T)];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x, c0 = blockIdx.y * CH;
  const int b = p.tileQ[tile];
  const int base = p.cuU[b], U = p.cuU[b + 1] - base;
  const int t0 = (tile - p.cuQ[b]) * TT;

  // per-channel taps and folded BatchNorm first, so their loads overlap the staging
  const int c = tid & 63, tg = tid >> 6;
  const int ch = c0 + c;
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) w[j] = p.w[(long)j * p.d + ch];
  const float alpha = p.bn_g[ch] / sqrtf(p.bn_v[ch] + p.eps);
  const float beta = p.bn_b[ch] + (p.b[ch] - p.bn_m[ch]) * alpha;

  typedef T t8 __attribute__((ext_vector_type(8)));
  for (int e = tid; e < R * (CH / 8); e += 256) {
    const int row = e / (CH / 8), c8 = e - row * (CH / 8);
    const int t = t0 - HALF + row;
    t8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (T)0.0f;
    if (t >= 0 && t < U) x = *(const t8*)((const T*)p.in + (long)(base + t) * p.d + c0 + c8 * 8);
    *(t8*)&sx[row][c8 * 8] = x;
  }
  __syncthreads();

  float win[TPT + K - 1];
#pragma unroll
  for (int i = 0; i < TPT + K - 1; ++i) win[i] = (float)sx[tg * TPT + i][c];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = t0 + tg * TPT + i;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) acc = fmaf(w[j], win[i + j], acc);
    if (t < U) ((T*)p.out)[(long)(base + t) * p.d + ch] = from_f32<T>(siluf_(acc * alpha + beta));
  }
}

hipError_t launch_dwconv(DType dt, int kernel, const DwParams& p, hipStream_t s) {
  if (p.n_tiles <= 0) return hipSuccess;
  if (p.d % 64) return hipErrorInvalidValue;
  dim3 grid(p.n_tiles, p.d / 64), blk(256);
#define GG_D(T, KK) hipLaunchKernelGGL((k_dw<T, KK>), grid, blk, 0, s, p)
#define GG_DK(T)                                                   \
  switch (kernel) {                                                \
    case 31: GG_D(T, 31); break;                                   \
    case 15: GG_D(T, 15); break;                                   \
    case 5: GG_D(T, 5); break;                                     \
    default: return hipErrorInvalidValue;                          \
  }
  if (dt == DT_F32) { GG_DK(float) }
  else if (dt == DT_BF16) { GG_DK(bf16) }
  else { GG_DK(f16) }
#undef GG_DK
#undef GG_D
  return hipGetLastError();
}

}  // namespace gg
