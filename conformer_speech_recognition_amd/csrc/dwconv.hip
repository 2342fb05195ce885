// Conformer convolution module, middle part, for gfx950:
//   depthwise Conv1d (kernel K, 'same' zero padding inside each clip) + BatchNorm with
//   running statistics (folded to a per-channel affine in the kernel) + SiLU.
// (The GLU before it is fused into the pointwise-1 GEMM epilogue.) "GigaAM MLX port for
// Mac", section "Where the time goes": the convolution module is ~17% of a block.
//
// 16-bit types. One work item = 16 frames x 64 channels of one clip, taken by one wave;
// a workgroup holds four independent waves (own LDS slice, no workgroup barrier). The wave
// stages its (16 + K + 1)-frame window in LDS: 16-byte buffer loads against a resource
// that spans the clip, so frames outside it read zero (the padding), and 16-byte LDS
// stores. Lane c then reads its channel's frames as packed pairs of the storage type:
// E[k] = (x[2k], x[2k+1]) from two 16-bit LDS reads, O[k] = (x[2k+1], x[2k+2]) by one
// byte-align of E[k] and E[k+1]. Output i is 16 two-element dot products with fp32
// accumulation (v_dot2_f32_f16 / v_dot2_f32_bf16) of the tap pairs (w[2p], w[2p+1]) (the
// last pair (w[K-1], 0)) with E[i/2 + p] for even i or O[(i-1)/2 + p] for odd i: half the
// vector instructions of one fp32 FMA per tap. The products are exact in fp32 (the taps
// are used at the storage precision, in which the 16-bit checkpoints hold them); only the
// order of the fp32 additions differs from a sequential sum. The 16 x 64 outputs go back
// through LDS so that each lane stores whole 16-byte row segments, against an output
// resource that drops frames past the clip's end. Items are ordered channel group, clip
// tile, frame group, and each XCD takes a contiguous range, so neighbouring items'
// overlapping windows meet in one L2.
//
// fp32: one block = 64 frames x 64 channels; the (64 + K - 1)-frame window is staged in LDS,
// each thread slides its channel over 16 frames with the window in registers (fp32 FMAs).
#include "kernels.h"

namespace gg {

template <typename T, int K>
__global__ void __launch_bounds__(256) k_dw32(DwParams p) {
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


// storage-type pairs as the dot-product instructions take them
template <typename T> struct Pair;
template <> struct Pair<f16> {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c, false);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const v2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <> struct Pair<bf16> {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c,
                                           false);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const v2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

template <typename T, int K>
__global__ void __launch_bounds__(256) k_dw(DwParams p, int n_items, int per_xcd) {
  constexpr int TPT = 16, CH = 64, HALF = (K - 1) / 2;
  constexpr int NE = (TPT + K + 1) / 2, NP = (K + 1) / 2;
  constexpr int RS = (2 * NE + 7) / 8 * 8;            // staged rows: whole 16-byte rounds
  constexpr int NL = RS / 8;                          // 16-byte window loads per lane
  constexpr int PITCH = CH + 8;                       // 144-byte rows
  static_assert(K % 2 == 1 && RS >= TPT, "odd kernel");
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint16_t sxa[4][RS][PITCH];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto& sx = sxa[wv];                                 // this wave's window
  // workgroup i runs on XCD i % 8: give each XCD a contiguous range of items. Nothing
  // branches: a wave past the last item recomputes the last one and stores nothing.
  const int raw = ((int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8)) * 4 + wv;
  const int item = min(raw, n_items - 1);
  const int fg = item & 3, rest = item >> 2;
  const int tile = rest % p.n_tiles, c0 = (rest / p.n_tiles) * CH;
  const int c = threadIdx.x & 63, ch = c0 + c;
  const int d2 = 2 * p.d;                             // bytes per row

  // taps and BatchNorm statistics depend on the channel group only: issued first
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.w, 0, K * p.d * 4, 0x00020000);
  float tr[K];
#pragma unroll
  for (int q = 0; q < K; ++q)
    tr[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, ch * 4, q * p.d * 4, 0));
  const float g = p.bn_g[ch], var = p.bn_v[ch], bb = p.bn_b[ch], cb = p.b[ch], mu = p.bn_m[ch];
  // one load for the clip geometry of the tile: first row, length, first frame
  const int4 geo = *(const int4*)(p.tileG + 4 * tile);
  const int U = geo.y, t0 = geo.z + fg * TPT;

  // window rows r = 0 .. RS-1 hold frames t0 - HALF + r, read through a buffer resource
  // spanning the clip's rows: frames outside the clip (negative offsets wrap past the end)
  // read as zero, which is the convolution's padding
  const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.in + (long)geo.x * p.d), 0, U * d2, 0x00020000);
  u4 stg[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int e = c + 64 * q, row = e >> 3, c8 = e & 7;
    stg[q] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rin, (t0 - HALF + row) * d2 + (c0 + c8 * 8) * 2, 0, 0));
  }
  uint32_t tp[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) tp[q] = Pair<T>::pack(tr[2 * q], 2 * q + 1 < K ? tr[2 * q + 1] : 0.f);
  const float alpha = g / sqrtf(var + p.eps);
  const float beta = bb + (cb - mu) * alpha;
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int e = c + 64 * q, row = e >> 3, c8 = e & 7;
    *(u4*)&sx[row][c8 * 8] = stg[q];
  }
  wave_lds_sync();                                     // the staged rows, to every lane

  uint32_t E[NE], O[NE - 1];
#pragma unroll
  for (int k = 0; k < NE; ++k) E[k] = (uint32_t)sx[2 * k][c] | ((uint32_t)sx[2 * k + 1][c] << 16);
#pragma unroll
  for (int k = 0; k < NE - 1; ++k) O[k] = __builtin_amdgcn_alignbyte(E[k + 1], E[k], 2);
  wave_lds_sync();                                     // window reads before the rows are reused
  // outputs: lane c's 16 frames of channel c go to LDS rows 0..15, which are then copied
  // out a whole 16-byte row segment per lane (frames past the clip's end are dropped by
  // the output resource, which spans the clip's rows)
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) acc = Pair<T>::dot(tp[q], (i & 1) ? O[(i >> 1) + q] : E[(i >> 1) + q], acc);
    const T v = from_f32<T>(siluf_(acc * alpha + beta));
    sx[i][c] = __builtin_bit_cast(uint16_t, v);
  }
  wave_lds_sync();
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((T*)p.out + (long)geo.x * p.d), 0, raw < n_items ? U * d2 : 0, 0x00020000);
#pragma unroll
  for (int q = 0; q < TPT * 8 / 64; ++q) {
    const int e = c + 64 * q, row = e >> 3, c8 = e & 7;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, *(const u4*)&sx[row][c8 * 8]), ro,
                                           (t0 + row) * d2 + (c0 + c8 * 8) * 2, 0, 0);
  }
}

hipError_t launch_dwconv(DType dt, int kernel, const DwParams& p, hipStream_t s) {
  if (p.n_tiles <= 0) return hipSuccess;
  if (p.d % 64) return hipErrorInvalidValue;
  if (dt == DT_F32) {
    dim3 grid(p.n_tiles, p.d / 64), blk(256);
#define GG_D(KK) hipLaunchKernelGGL((k_dw32<float, KK>), grid, blk, 0, s, p)
    switch (kernel) {
      case 31: GG_D(31); break;
      case 15: GG_D(15); break;
      case 5: GG_D(5); break;
      default: return hipErrorInvalidValue;
    }
#undef GG_D
    return hipGetLastError();
  }
  // 16-bit: 4 frame groups of 16 per 64-frame tile, per 64-channel group; four items
  // (waves) per workgroup
  const long items = (long)p.n_tiles * (p.d / 64) * 4;
  if (items > (1L << 30)) return hipErrorInvalidValue;
  const int n = (int)items, per_xcd = ((n + 3) / 4 + 7) / 8;
  dim3 grid(8 * per_xcd), blk(256);
#define GG_D(T, KK) hipLaunchKernelGGL((k_dw<T, KK>), grid, blk, 0, s, p, n, per_xcd)
#define GG_DK(T)                                                   \
  switch (kernel) {                                                \
    case 31: GG_D(T, 31); break;                                   \
    case 15: GG_D(T, 15); break;                                   \
    case 5: GG_D(T, 5); break;                                     \
    default: return hipErrorInvalidValue;                          \
  }
  if (dt == DT_BF16) { GG_DK(bf16) }
  else { GG_DK(f16) }
#undef GG_DK
#undef GG_D
  return hipGetLastError();
}

}  // namespace gg
