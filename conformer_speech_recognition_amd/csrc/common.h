// Shared device/host definitions for the gfx950 kernels of the Conformer CTC encoder.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef __bf16 bf16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace gg {

// Element storage types of the GEMM/attention operands.
enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_W8F16 = 3, DT_W6F16 = 4, DT_W4F16 = 5 };

// Per-call batch geometry, written into the workspace by the meta kernel.
// Row r of the packed mel / sub / encoder spaces belongs to clip rowclip_X[r];
// clip b owns rows [cu_X[b], cu_X[b+1]).  q-tiles are blocks of 64 encoder frames
// of one clip, numbered clip after clip (cu_Q).
constexpr int kMaxBatch = 256;
constexpr int kQTile = 64;

struct MetaArgs {          // passed by value to the meta kernel (kernarg, < 4 KiB)
  int B;
  int cuT[kMaxBatch + 1];
  int cuS[kMaxBatch + 1];
  int cuU[kMaxBatch + 1];
};

struct MetaDev {           // device view of the meta region
  int* cuT; int* cuS; int* cuU; int* cuQ;
  int* rowT; int* rowS; int* rowU; int* tileQ;
};

template <typename T> struct TypeOf;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Logistic sigmoid and SiLU from the hardware exp2 and reciprocal (about 1 ulp each);
// an IEEE division costs ten dependent instructions per element in the epilogues.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * x));
}
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }

// Wave-wide (64 lanes) butterfly sums.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace gg
