// Row LayerNorm (one wave per row or per two rows, fp32 statistics) with three fused variants:
//   LN_PLAIN : y = LN(x) -> T                      (FFN and conv-module pre-norms)
//   LN_ROPE  : y = LN(x) -> T and r = rope(y) -> T (attention pre-norm; the rotation is
//              applied per head to the raw normed input BEFORE the q/k projections,
//              value uses y unrotated: "GigaAM on MLX: the transcripts matched, but the
//              model was broken", Trap 2)
//   LN_TWO   : x <- LN_out(x) in place (fp32), then y = LN_next(x) -> T (block's final
//              norm fused with the next block's first pre-norm)
// Lane l holds features 256 i + 4 l + q (i < d / 256, q < 4), so every load and store
// instruction of a wave covers one contiguous 1 KiB (fp32) or 512 B (16-bit) span.
// rotate_half's partner (the feature d_k / 2 away inside the same head) is read back
// from the wave's own copy of the normed row in LDS.
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

// gamma and beta of this lane's features, loaded with the row (the deferred-residual
// variants store x before normalising, and loads written after those stores waited for them)
template <int NI> struct LnAffine { f32x4 g[NI], b[NI]; };
template <int NI>
__device__ __forceinline__ LnAffine<NI> ln_affine(const float* g, const float* b, int lane) {
  LnAffine<NI> a;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    a.g[i] = *(const f32x4*)(g + 256 * i + 4 * lane);
    a.b[i] = *(const f32x4*)(b + 256 * i + 4 * lane);
  }
  return a;
}

// v[4 i + q] = feature 256 i + 4 lane + q
template <int NI>
__device__ __forceinline__ void ln_row(float (&v)[4 * NI], const LnAffine<NI>& ab, int lane,
                                       float eps) {
  constexpr int D = NI * 256;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4 * NI; ++e) s += v[e];
  const float mean = wave_sum(s) * (1.0f / D);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4 * NI; ++e) {
    v[e] -= mean;
    ss += v[e] * v[e];
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) * (1.0f / D) + eps);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) v[4 * i + q] = v[4 * i + q] * rstd * ab.g[i][q] + ab.b[i][q];
}

// normalise one row held in v (the row's loads already issued) and write its outputs
template <typename T, int NI, int MODE>
__device__ __forceinline__ void ln_finish(const LnParams& p, float (&v)[4 * NI], int row, int lane,
                                          float* sr, float cv, float sv, const LnAffine<NI>& a1,
                                          const LnAffine<NI>& a2) {
  constexpr int D = NI * 256;
  constexpr int DK = D / 16, HALF = DK / 2;      // 16 heads
  float* xr = p.x + (long)row * D + 4 * lane;
  ln_row<NI>(v, a1, lane, p.eps);
  T* yr = (T*)p.y + (long)row * D + 4 * lane;
  if constexpr (MODE == LN_TWO) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *(f32x4*)(xr + 256 * i) = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    if (p.g2 == nullptr) {          // last block: x only (optionally a T copy)
      if (p.y != nullptr)
#pragma unroll
        for (int i = 0; i < NI; ++i)
          store4<T>(yr + 256 * i, v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      return;
    }
    ln_row<NI>(v, a2, lane, p.eps);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) store4<T>(yr + 256 * i, v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  if constexpr (MODE == LN_ROPE) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *(f32x4*)(sr + 256 * i + 4 * lane) = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    // this frame's cos / sin rows next to the normed row
    float* cs = sr + D;
    if (lane < HALF) {
      cs[lane] = cv;
      cs[HALF + lane] = sv;
    }
    // the reads below take other lanes' entries: order them after every lane's stores
    // (wavefront-scope release / acquire around a wave barrier, so the compiler may not
    // move an LDS read above the stores it depends on)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // a lane's 4 consecutive features sit in one half of one head (4 divides d_k / 2), so
    // their partners, cosines and sines are 16-byte LDS reads
    float r[4 * NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = 256 * i + 4 * lane;                      // first feature of the group
      const int pos = j % DK;                                // position inside the head
      const bool lo = pos < HALF;
      const int i2 = lo ? pos : pos - HALF;
      const f32x4 pt = *(const f32x4*)(sr + (lo ? j + HALF : j - HALF));
      const f32x4 cc = *(const f32x4*)(cs + i2), sn = *(const f32x4*)(cs + HALF + i2);
#pragma unroll
      for (int q = 0; q < 4; ++q) r[4 * i + q] = v[4 * i + q] * cc[q] + (lo ? -pt[q] : pt[q]) * sn[q];
    }
    T* rr = (T*)p.r + (long)row * D + 4 * lane;
#pragma unroll
    for (int i = 0; i < NI; ++i) store4<T>(rr + 256 * i, r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
  }
}

// One wave per RPW consecutive rows: every row's loads (and, for RoPE, its cos / sin
// entries, two dependent loads: the frame's position, then the table) are issued before the
// first row's statistics, so a wave keeps RPW rows of reads in flight and the grid fits the
// chip in one round. RKS > 0: the preceding residual GEMM left its K sum in RKS slices,
// which are added here (all slice reads issued together: a loop over a run-time slice count
// made the compiler wait for each one, one round trip to memory per slice and feature group).
template <typename T, int NI, int MODE, int RPW, int RKS>
__global__ void __launch_bounds__(256) k_ln(LnParams p) {
  constexpr int D = NI * 256;
  constexpr int DK = D / 16, HALF = DK / 2;
  __shared__ __attribute__((aligned(16))) float srow[MODE == LN_ROPE ? 4 : 1][MODE == LN_ROPE ? D + D / 16 : 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wv) * RPW;
  if (row0 >= p.rows) return;
  float v[RPW][4 * NI];
  float cv[RPW], sv[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r < p.rows ? row0 + r : p.rows - 1;   // past the end: reload the last
    const float* xr = p.x + (long)row * D + 4 * lane;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const f32x4 q = *(const f32x4*)(xr + 256 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r][4 * i + j] = q[j];
    }
  }
  const LnAffine<NI> a1 = ln_affine<NI>(p.g1, p.b1, lane);
  // (pointers selected, not the loads: a load under a branch is waited for at its join)
  const LnAffine<NI> a2 = MODE == LN_TWO ? ln_affine<NI>(p.g2 ? p.g2 : p.g1, p.g2 ? p.b2 : p.b1, lane) : a1;
  if constexpr (RKS > 0) {
    // x += ralpha * (slices in order + bias): the reduce step of that GEMM done here, and x
    // written back unless the LayerNorm overwrites it
    const long slice = (long)p.rows * D;
    f32x4 part[RPW][NI][RKS];
    f32x4 rb[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) rb[i] = *(const f32x4*)(p.rbias + 256 * i + 4 * lane);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row0 + r < p.rows ? row0 + r : p.rows - 1;
      const long off = (long)row * D + 4 * lane;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int k = 0; k < RKS; ++k) part[r][i][k] = *(const f32x4*)(p.rpart + off + 256 * i + k * slice);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        f32x4 a = part[r][i][0];
#pragma unroll
        for (int k = 1; k < RKS; ++k) a += part[r][i][k];
        const f32x4 sum = a + rb[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[r][4 * i + j] = v[r][4 * i + j] + p.ralpha * sum[j];
      }
    if constexpr (MODE != LN_TWO) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (row0 + r >= p.rows) continue;
        const long off = (long)(row0 + r) * D + 4 * lane;
#pragma unroll
        for (int i = 0; i < NI; ++i)
          *(f32x4*)(p.x + off + 256 * i) = f32x4{v[r][4 * i], v[r][4 * i + 1], v[r][4 * i + 2], v[r][4 * i + 3]};
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    cv[r] = 0.f;
    sv[r] = 0.f;
    if constexpr (MODE == LN_ROPE) {
      const int row = row0 + r < p.rows ? row0 + r : p.rows - 1;
      const int t = p.rowpos[row];
      if (lane < HALF) {
        cv[r] = p.cos_t[(long)t * HALF + lane];
        sv[r] = p.sin_t[(long)t * HALF + lane];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    if (row0 + r < p.rows) ln_finish<T, NI, MODE>(p, v[r], row0 + r, lane, srow[wv], cv[r], sv[r], a1, a2);
}

// rows per wave, by timing inside the encode: one (two made the RoPE variant slower, 11.3 ->
// 12.4 us at 8207 rows of 768, and the plain one 8.8 -> 10.0; the two-norm variant, faster with
// two rows while its parameter loads waited for its first row, is now 13.7 -> 13.5 us with one)
template <typename T, int NI, int MODE, int RPW>
static hipError_t ln_launch(const LnParams& p, hipStream_t s) {
  dim3 grid((p.rows + 4 * RPW - 1) / (4 * RPW));
  // each deferred-residual slice count is its own instantiation: its stores to x would
  // otherwise keep the plain kernel's parameter loads from being hoisted
  switch (p.rks) {
    case 0: hipLaunchKernelGGL((k_ln<T, NI, MODE, RPW, 0>), grid, dim3(256), 0, s, p); break;
    case 1: hipLaunchKernelGGL((k_ln<T, NI, MODE, RPW, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_ln<T, NI, MODE, RPW, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((k_ln<T, NI, MODE, RPW, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_ln<T, NI, MODE, RPW, 4>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int NI>
static hipError_t ln_modes(LnMode mode, const LnParams& p, hipStream_t s) {
  switch (mode) {
    case LN_PLAIN: return ln_launch<T, NI, LN_PLAIN, 1>(p, s);
    case LN_ROPE: return ln_launch<T, NI, LN_ROPE, 1>(p, s);
    case LN_TWO: return ln_launch<T, NI, LN_TWO, 1>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t ln_widths(LnMode mode, const LnParams& p, hipStream_t s) {
  switch (p.d) {
    case 768: return ln_modes<T, 3>(mode, p, s);
    case 1024: return ln_modes<T, 4>(mode, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm(DType dt, LnMode mode, const LnParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.rks > 0 && (!p.rpart || !p.rbias)) return hipErrorInvalidValue;
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
