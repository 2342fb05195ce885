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

// Attention works on 128-frame query tiles (cuQ2 / tileQ2; numbered clip by clip, longest
// clip first).
constexpr int kQTile2 = 128;

struct MetaDev {           // device view of the meta region
  int* cuT; int* cuS; int* cuU; int* cuQ;
  int* rowT; int* rowS; int* rowU; int* tileQ;
  int* cuQ2; int* tileQ2;
  int* tileG;              // 4 ints per 64-frame tile: first row, clip length, first frame, clip
  int* posU;               // position of each encoder row inside its clip, or nullptr
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

// Orders LDS accesses across the lanes of one wave (each wave owns its LDS slice): a
// wavefront-scope release/acquire pair around a wave barrier, which, unlike a workgroup
// barrier's fence, waits for no outstanding global access.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane exchanges for butterfly reductions, without the LDS crossbar that a shuffle
// (ds_bpermute) goes through.
//  * lanes 32 / 16 apart: v_permlane32_swap / v_permlane16_swap on two copies of a value
//    return {own, partner} in an order that depends on the lane's half, so the x32 / x16
//    steps combine both results with a symmetric operation (a + b, max, argmax with the
//    lower index on ties): each lane gets exactly combine(v, v[lane ^ o]).
//  * lanes 8 apart: DPP row rotation by 8 inside a 16-lane row is exactly lane ^ 8.
//  * lanes 4 apart: a row rotation by 4 equals lane ^ 4 once the values repeat every 8
//    lanes of a row, which a butterfly run from 8 (or wider) downwards guarantees.
//  * lanes 2 / 1 apart: DPP quad permutations [2,3,0,1] / [1,0,3,2] are exact.
// So a butterfly over o = 32, 16, .., 1 (or 16, .., 1 or 8, .., 1 inside aligned groups)
// computes the same values, in the same order, as one built on __shfl_xor.
__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float ffrom(uint32_t v) { return __builtin_bit_cast(float, v); }
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) { return ffrom(dpp_u<CTRL>(fbits(v))); }
constexpr int kDppRor8 = 0x128, kDppRor4 = 0x124, kDppXor2 = 0x4E, kDppXor1 = 0xB1;

// {own, partner} pairs (order unspecified) for lanes 32 / 16 apart
__device__ __forceinline__ void pair_x32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void pair_x16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

// butterfly sum over aligned groups of G lanes (G = 64, 32, 16, 8, 4, 2 or 1)
template <int G> __device__ __forceinline__ float group_sum(float v) {
  uint32_t a, b;
  if constexpr (G >= 64) { pair_x32(fbits(v), a, b); v = ffrom(a) + ffrom(b); }
  if constexpr (G >= 32) { pair_x16(fbits(v), a, b); v = ffrom(a) + ffrom(b); }
  if constexpr (G >= 16) { v += dpp_f<kDppRor8>(v); v += dpp_f<kDppRor4>(v); }
  else if constexpr (G == 8) { v += __shfl_xor(v, 4, 64); }   // values not 8-periodic yet
  if constexpr (G >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (G >= 2) v += dpp_f<kDppXor1>(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// wave-wide argmax: the larger value wins, the lower index on equal values (the values
// must not be NaN)
__device__ __forceinline__ void argmax_take(float& best, int& bi, float ov, int oi) {
  if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
}
__device__ __forceinline__ void wave_argmax(float& best, int& bi) {
  uint32_t a, b, ia, ib;
  pair_x32(fbits(best), a, b);
  pair_x32((uint32_t)bi, ia, ib);
  best = ffrom(a); bi = (int)ia;
  argmax_take(best, bi, ffrom(b), (int)ib);
  pair_x16(fbits(best), a, b);
  pair_x16((uint32_t)bi, ia, ib);
  best = ffrom(a); bi = (int)ia;
  argmax_take(best, bi, ffrom(b), (int)ib);
  argmax_take(best, bi, dpp_f<kDppRor8>(best), (int)dpp_u<kDppRor8>((uint32_t)bi));
  argmax_take(best, bi, dpp_f<kDppRor4>(best), (int)dpp_u<kDppRor4>((uint32_t)bi));
  argmax_take(best, bi, dpp_f<kDppXor2>(best), (int)dpp_u<kDppXor2>((uint32_t)bi));
  argmax_take(best, bi, dpp_f<kDppXor1>(best), (int)dpp_u<kDppXor1>((uint32_t)bi));
}

}  // namespace gg
