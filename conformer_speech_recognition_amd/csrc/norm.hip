// Row LayerNorm (one wave per row, fp32 statistics) with three fused variants:
//   LN_PLAIN : y = LN(x) -> T                      (FFN and conv-module pre-norms)
//   LN_ROPE  : y = LN(x) -> T and r = rope(y) -> T (attention pre-norm; the rotation is
//              applied per head to the raw normed input BEFORE the q/k projections,
//              value uses y unrotated: "GigaAM on MLX: the transcripts matched, but the
//              model was broken", Trap 2)
//   LN_TWO   : x <- LN_out(x) in place (fp32), then y = LN_next(x) -> T (block's final
//              norm fused with the next block's first pre-norm)
// Lane l holds the d/64 contiguous features [l*EPL, (l+1)*EPL); with 16 heads a head is
// 4 lanes, so rotate_half's partner (i +- d_k/2) lives in lane l ^ 2.
#include "kernels.h"

namespace gg {

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c,
                                                          float d) {
  *(f32x4*)dst = f32x4{a, b, c, d};
}
template <> __device__ __forceinline__ void store4<f16>(f16* dst, float a, float b, float c,
                                                        float d) {
  *(f16x4*)dst = f16x4{(f16)a, (f16)b, (f16)c, (f16)d};
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c,
                                                         float d) {
  *(bf16x4*)dst = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}

template <int EPL>
__device__ __forceinline__ void ln_row(float (&v)[EPL], const float* g, const float* b, int lane,
                                       float eps) {
  constexpr int D = EPL * 64;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s += v[i];
  const float mean = wave_sum(s) * (1.0f / D);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    v[i] -= mean;
    ss += v[i] * v[i];
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < EPL; i += 4) {
    const f32x4 gg4 = *(const f32x4*)(g + lane * EPL + i);
    const f32x4 bb4 = *(const f32x4*)(b + lane * EPL + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[i + j] = v[i + j] * rstd * gg4[j] + bb4[j];
  }
}

template <typename T, int EPL, int MODE>
__global__ void __launch_bounds__(256) k_ln(LnParams p) {
  constexpr int D = EPL * 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  float v[EPL];
  float* xr = p.x + (long)row * D + lane * EPL;
#pragma unroll
  for (int i = 0; i < EPL; i += 4) {
    const f32x4 q = *(const f32x4*)(xr + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[i + j] = q[j];
  }
  ln_row<EPL>(v, p.g1, p.b1, lane, p.eps);
  T* yr = (T*)p.y + (long)row * D + lane * EPL;
  if constexpr (MODE == LN_TWO) {
#pragma unroll
    for (int i = 0; i < EPL; i += 4) *(f32x4*)(xr + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
    if (p.g2 == nullptr) {          // last block: x only (optionally a T copy)
      if (p.y != nullptr)
#pragma unroll
        for (int i = 0; i < EPL; i += 4) store4<T>(yr + i, v[i], v[i + 1], v[i + 2], v[i + 3]);
      return;
    }
    ln_row<EPL>(v, p.g2, p.b2, lane, p.eps);
  }
#pragma unroll
  for (int i = 0; i < EPL; i += 4) store4<T>(yr + i, v[i], v[i + 1], v[i + 2], v[i + 3]);
  if constexpr (MODE == LN_ROPE) {
    constexpr int HALF = 2 * EPL;           // d_k / 2
    const int b = p.rowclip[row];
    const int t = row - p.cu[b];
    const float* cr = p.cos_t + (long)t * HALF + (lane & 1) * EPL;
    const float* sr = p.sin_t + (long)t * HALF + (lane & 1) * EPL;
    const float sgn = (lane & 2) ? 1.0f : -1.0f;
    float r[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float partner = __shfl_xor(v[i], 2, 64);
      r[i] = v[i] * cr[i] + sgn * partner * sr[i];
    }
    T* rr = (T*)p.r + (long)row * D + lane * EPL;
#pragma unroll
    for (int i = 0; i < EPL; i += 4) store4<T>(rr + i, r[i], r[i + 1], r[i + 2], r[i + 3]);
  }
}

template <typename T, int EPL>
static hipError_t ln_modes(LnMode mode, const LnParams& p, hipStream_t s) {
  dim3 grid((p.rows + 3) / 4);
  switch (mode) {
    case LN_PLAIN: hipLaunchKernelGGL((k_ln<T, EPL, LN_PLAIN>), grid, dim3(256), 0, s, p); break;
    case LN_ROPE: hipLaunchKernelGGL((k_ln<T, EPL, LN_ROPE>), grid, dim3(256), 0, s, p); break;
    case LN_TWO: hipLaunchKernelGGL((k_ln<T, EPL, LN_TWO>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t ln_widths(LnMode mode, const LnParams& p, hipStream_t s) {
  switch (p.d) {
    case 768: return ln_modes<T, 12>(mode, p, s);
    case 1024: return ln_modes<T, 16>(mode, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm(DType dt, LnMode mode, const LnParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return ln_widths<float>(mode, p, s);
    case DT_F16:
    case DT_W8F16:
    case DT_W6F16:
    case DT_W4F16: return ln_widths<f16>(mode, p, s);
    case DT_BF16: return ln_widths<bf16>(mode, p, s);
  }
  return hipErrorInvalidValue;
}

// cos/sin tables [n_pos][d_k/2]: angle(t, i) = t * base^(-2i/d_k), evaluated in fp64 so the
// fp32 table is correctly rounded ("GigaAM on MLX ...", Trap 1: base 5000 and dim
// d_model / n_heads; the tables are built once per forward pass).
__global__ void k_rope_table(float* cos_t, float* sin_t, int n_pos, int dk, double base) {
  const int half = dk / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_pos * half) return;
  const int t = e / half, i = e - t * half;
  const double ang = (double)t * pow(base, -2.0 * i / dk);
  double sn, cs;
  sincos(ang, &sn, &cs);
  cos_t[e] = (float)cs;
  sin_t[e] = (float)sn;
}

hipError_t launch_rope_table(float* cos_t, float* sin_t, int n_pos, int dk, float base,
                             hipStream_t s) {
  const int n = n_pos * (dk / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, s, cos_t, sin_t, n_pos, dk,
                     (double)base);
  return hipGetLastError();
}

}  // namespace gg
