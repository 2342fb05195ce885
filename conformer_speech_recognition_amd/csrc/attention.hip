// Flash-style self-attention over packed variable-length clips for gfx950.
// softmax(q k^T / sqrt(d_k)) v per clip and head, keys beyond the clip masked
// (key-padding mask; fused scaled-dot-product attention: "GigaAM MLX port for Mac",
// section "Where the time goes").
//
// Block = 4 waves = 64 queries of one clip and one head; each wave owns 16 queries.
// Per 64-key tile (K and V^T staged in LDS, the next tile prefetched into registers):
//   S^T[key][query] = K . Q^T   with 16x16 MFMAs (A = K rows from LDS, B = the wave's Q
//                               fragment kept in registers)
//   lane l then holds 16 scores of ONE query (l % 16): keys kb*16 + 4*(l/16) + r,
//   so the online-softmax running max / sum / rescale are lane-local (plus a 4-lane
//   max across l/16);
//   O^T[dim][query] += V^T . P^T with the probabilities used straight from the score
//   registers as the B operand (the lane's k slots are exactly its keys).
// Scores, max, sum and the output accumulator are fp32; P is rounded to T for the MFMA.
// d_k = 48 runs the score contraction as two 16x16x32 MFMAs with the top 16 k slots zero.
#include "kernels.h"

namespace gg {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int AT_KV = 64;

template <typename T> struct AttnMma;
template <> struct AttnMma<f16> {
  static __device__ __forceinline__ f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct AttnMma<bf16> {
  static __device__ __forceinline__ f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ u32x4 pack8f(const float* v) {
  typedef T t8 __attribute__((ext_vector_type(8)));
  t8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (T)v[i];
  return __builtin_bit_cast(u32x4, h);
}

// ---------------------------------------------------------------- fp16 / bf16 kernel
// K and V^T tiles are double-buffered in LDS: the next 64-key tile is loaded into
// registers while the current one is consumed, and stored after it (one barrier per
// tile). V is transposed in 4-key x 8-dim register blocks, written as 8-byte LDS stores.
template <typename T, int DK>
__global__ void __launch_bounds__(256) k_attn(AttnParams p) {
  constexpr int KP = DK + 8;         // LDS row pitch (elements) of K: 16 rows -> 16 bank groups
  constexpr int VP = AT_KV + 8;      // LDS row pitch of V^T
  constexpr int NDB = DK / 16;       // 16-wide dim blocks of the output
  constexpr int KCH = AT_KV * DK / 8;          // 16-byte K chunks per tile
  constexpr int VBL = (AT_KV / 4) * (DK / 8);  // 4-key x 8-dim V blocks per tile
  constexpr int KPT = (KCH + 255) / 256;       // K chunks per thread
  static_assert(VBL <= 256, "one V block per thread");
  __shared__ T sK[2][AT_KV][KP];
  __shared__ T sVt[2][DK][VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int b = p.tileQ[tile];
  const int base = p.cuU[b], U = p.cuU[b + 1] - base;
  const int qi = (tile - p.cuQ[b]) * 64 + wave * 16 + c16;
  const int ld = 3 * p.d;
  const T* Qg = (const T*)p.qkv + (long)base * ld + h * DK;
  const T* Kg = Qg + p.d;
  const T* Vg = Qg + 2 * p.d;

  // Q fragment (B operand of S^T): query qi, dims [8g, 8g+8) and the remainder block
  const int qrow = qi < U ? qi : U - 1;
  const T* qp = Qg + (long)qrow * ld;
  // dims 32.. go through a second 16x16x32 MFMA; for d_k = 48 its lanes g >= 2 (dims 48..63)
  // are zero on both operands
  const bool hi_ok = DK == 64 || g < 2;
  const u32x4 qa = *(const u32x4*)(qp + 8 * g);
  const u32x4 qb = hi_ok ? *(const u32x4*)(qp + 32 + 8 * g) : u32x4{0, 0, 0, 0};

  // tile loads into registers
  u32x4 rk[KPT];
  u32x4 rv[4];
  const int vq = tid / (DK / 8), vch = tid - vq * (DK / 8);   // V block: keys 4vq.., dims 8vch..
  auto load = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + 256 * i;
      const int key = e / (DK / 8), ch = e - key * (DK / 8);
      rk[i] = u32x4{0, 0, 0, 0};
      if (e < KCH && kv0 + key < U) rk[i] = *(const u32x4*)(Kg + (long)(kv0 + key) * ld + ch * 8);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kv0 + 4 * vq + j;
      rv[j] = u32x4{0, 0, 0, 0};
      if (tid < VBL && key < U) rv[j] = *(const u32x4*)(Vg + (long)key * ld + vch * 8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = tid + 256 * i;
      if (e < KCH) {
        const int key = e / (DK / 8), ch = e - key * (DK / 8);
        *(u32x4*)&sK[buf][key][ch * 8] = rk[i];
      }
    }
    if (tid < VBL) {
      typedef uint16_t h8 __attribute__((ext_vector_type(8)));
      typedef uint16_t h4 __attribute__((ext_vector_type(4)));
      const h8 v0 = __builtin_bit_cast(h8, rv[0]), v1 = __builtin_bit_cast(h8, rv[1]);
      const h8 v2 = __builtin_bit_cast(h8, rv[2]), v3 = __builtin_bit_cast(h8, rv[3]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(h4*)&sVt[buf][vch * 8 + i][4 * vq] = h4{v0[i], v1[i], v2[i], v3[i]};
    }
  };

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0, 0, 0, 0};

  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int kv0 = 0; kv0 < U; kv0 += AT_KV) {
    const bool more = kv0 + AT_KV < U;
    if (more) load(kv0 + AT_KV);

    // S^T blocks: s[kb][r] = score(key kv0 + kb*16 + 4g + r, query qi)
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const T* kr = &sK[buf][kb * 16 + c16][0];
      f32x4 acc = f32x4{0, 0, 0, 0};
      acc = AttnMma<T>::k32(*(const u32x4*)(kr + 8 * g), qa, acc);
      const u32x4 kh = hi_ok ? *(const u32x4*)(kr + 32 + 8 * g) : u32x4{0, 0, 0, 0};
      acc = AttnMma<T>::k32(kh, qb, acc);
      s[kb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + kb * 16 + 4 * g + r;
        const float v = key < U ? s[kb][r] * p.scale_log2 : -INFINITY;
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float pv[4][4];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[kb][r] = exp2f(s[kb][r] - m_new);
        ls += pv[kb][r];
      }
    l_part = l_part * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;

#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      float pp[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { pp[r] = pv[2 * hk][r]; pp[4 + r] = pv[2 * hk + 1][r]; }
      const u32x4 pb = pack8f<T>(pp);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const T* vr = &sVt[buf][db * 16 + c16][32 * hk + 4 * g];
        const u32x2 lo = *(const u32x2*)vr;
        const u32x2 hi = *(const u32x2*)(vr + 16);
        o[db] = AttnMma<T>::k32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[db]);
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  float l = l_part + __shfl_xor(l_part, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (qi < U) {
    const float inv = 1.0f / l;
    T* op = (T*)p.out + (long)(base + qi) * p.d + h * DK;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      typedef T t4 __attribute__((ext_vector_type(4)));
      t4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (T)(o[db][r] * inv);
      *(t4*)(op + db * 16 + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------- fp32 kernel
// Same dataflow with v_mfma_f32_16x16x4_f32 (one k element per lane group).
template <int DK>
__global__ void __launch_bounds__(256) k_attn_f32(AttnParams p) {
  constexpr int KP = DK + 4, VP = AT_KV + 4, NDB = DK / 16;
  __shared__ float sK[AT_KV][KP];
  __shared__ float sVt[DK][VP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int b = p.tileQ[tile];
  const int base = p.cuU[b], U = p.cuU[b + 1] - base;
  const int qi = (tile - p.cuQ[b]) * 64 + wave * 16 + c16;
  const int ld = 3 * p.d;
  const float* Qg = (const float*)p.qkv + (long)base * ld + h * DK;
  const float* Kg = Qg + p.d;
  const float* Vg = Qg + 2 * p.d;
  const int qrow = qi < U ? qi : U - 1;
  float qf[DK / 4];
#pragma unroll
  for (int s4 = 0; s4 < DK / 4; ++s4) qf[s4] = Qg[(long)qrow * ld + 4 * s4 + g];

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0, 0, 0, 0};

  for (int kv0 = 0; kv0 < U; kv0 += AT_KV) {
    __syncthreads();
    for (int e = tid; e < AT_KV * DK; e += 256) {
      const int key = e / DK, dd = e - key * DK;
      const bool ok = kv0 + key < U;
      sK[key][dd] = ok ? Kg[(long)(kv0 + key) * ld + dd] : 0.f;
      sVt[dd][key] = ok ? Vg[(long)(kv0 + key) * ld + dd] : 0.f;
    }
    __syncthreads();
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s4 = 0; s4 < DK / 4; ++s4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sK[kb * 16 + c16][4 * s4 + g], qf[s4], acc, 0, 0, 0);
      s[kb] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + kb * 16 + 4 * g + r;
        const float v = key < U ? s[kb][r] * p.scale_log2 : -INFINITY;
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] = exp2f(s[kb][r] - m_new);
        ls += s[kb][r];
      }
    l_part = l_part * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      o[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(sVt[db * 16 + c16][kb * 16 + 4 * g + r],
                                                       s[kb][r], o[db], 0, 0, 0);
    }
  }
  float l = l_part + __shfl_xor(l_part, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (qi < U) {
    const float inv = 1.0f / l;
    float* op = (float*)p.out + (long)(base + qi) * p.d + h * DK;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(f32x4*)(op + db * 16 + 4 * g) = o[db] * inv;
  }
}

hipError_t launch_attention(DType dt, int dk, const AttnParams& p, hipStream_t s) {
  if (p.n_tiles <= 0) return hipSuccess;
  dim3 grid(p.n_tiles, p.n_heads), blk(256);
#define GG_A(T, D) hipLaunchKernelGGL((k_attn<T, D>), grid, blk, 0, s, p)
  if (dt == DT_F32) {
    if (dk == 48) hipLaunchKernelGGL(k_attn_f32<48>, grid, blk, 0, s, p);
    else if (dk == 64) hipLaunchKernelGGL(k_attn_f32<64>, grid, blk, 0, s, p);
    else return hipErrorInvalidValue;
  } else if (dt == DT_BF16) {
    if (dk == 48) GG_A(bf16, 48); else if (dk == 64) GG_A(bf16, 64); else return hipErrorInvalidValue;
  } else {
    if (dk == 48) GG_A(f16, 48); else if (dk == 64) GG_A(f16, 64); else return hipErrorInvalidValue;
  }
#undef GG_A
  return hipGetLastError();
}

}  // namespace gg
