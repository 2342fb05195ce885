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

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Inside each group of 16 lanes, lane
// i = 4 s + q names 4 consecutive 16-bit elements (8 bytes); lane j of the group receives
// element (j & 3) of the rows named by lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4, in
// that order (measured on the device: lane j, slot s <- lane 4 s + j / 4, element j & 3).
// So if lane 4 s + q points at V[key_s][d0 + 4 q .. d0 + 4 q + 3] of a row-major V tile,
// lane j gets V[key_0..key_3][d0 + j]: four keys of one dimension, an MFMA A-operand half.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <typename T> __device__ __forceinline__ u32x2 lds_read_tr(const T* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p)));
}

// ---------------------------------------------------------------- fp16 / bf16 kernel
// K and V tiles are double-buffered in LDS, both row-major (key, dim) copies of the global
// rows: the next 64-key tile is loaded into registers while the current one is consumed,
// and stored after it (one barrier per tile). The P.V product reads its V^T operand with
// the transposing LDS read, so V is never transposed in registers.
//
// The softmax is kept in base 2 with the scale folded into one FMA per score:
// p = 2^(s*c - m*c), c = log2(e)/sqrt(d_k), m the running max of the raw scores.  The
// key mask is applied only on a clip's last, partial tile; the accumulator is rescaled
// only when some query's running max moved.
// v_max3_f32 without the NaN-quieting canonicalisation the compiler adds around fmaxf
__device__ __forceinline__ float max3_(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Work order. Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8), each with its own L2. Item w = head * n_tiles + q-tile keeps the q-tiles of
// one clip and head next to each other; giving every XCD a contiguous range of items
// means the K and V blocks of a clip and head are fetched into one L2, not into all.
__device__ __forceinline__ void attn_item(int bid, int n_tiles, int n_heads, int& tile, int& h) {
  const int total = n_tiles * n_heads;
  const int q = total / 8, r = total % 8;
  const int x = bid % 8, j = bid / 8;
  const int w = x * q + (x < r ? x : r) + j;
  h = w / n_tiles;
  tile = w - h * n_tiles;
}

__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return max3_(__uint_as_float(r[0]), __uint_as_float(r[1]), v);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return max3_(__uint_as_float(r[0]), __uint_as_float(r[1]), v);
}

template <typename T, int DK>
__global__ void __launch_bounds__(256) k_attn(AttnParams p) {
  constexpr int KP = DK + 8;         // LDS row pitch (elements) of K: 16 rows -> 16 bank groups
  // LDS row pitch of V: dims, then a column of ones and zeros up to DK + 16; 80 elements
  // put the 8 rows one transposing read pass touches on disjoint banks
  constexpr int VP = 80;
  constexpr int NDB = DK / 16;       // 16-wide dim blocks of the output
  constexpr int NDBX = NDB + 1;      // + one block whose first column is all ones: row sums
  constexpr int CPR = DK / 8;        // 16-byte chunks per K / V row
  constexpr int KCH = AT_KV * CPR;   // 16-byte chunks per tile (each of K and V)
  constexpr int KPT = (KCH + 255) / 256;       // chunks per thread
  static_assert(DK + 16 <= VP, "V row pitch");
  __shared__ T sK[2][AT_KV][KP];
  __shared__ __attribute__((aligned(16))) T sV[2][AT_KV][VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int tile, h;
  attn_item(blockIdx.x, p.n_tiles, p.n_heads, tile, h);
  const int b = p.tileQ[tile];
  const int base = p.cuU[b], U = p.cuU[b + 1] - base;
  const int qi = (tile - p.cuQ[b]) * 64 + wave * 16 + c16;
  const int ld = 3 * p.d;
  const T* Qg = (const T*)p.qkv + (long)base * ld + h * DK;
  const T* Kg = Qg + p.d;
  const T* Vg = Qg + 2 * p.d;
  const float c = p.scale_log2;

  // Q fragment (B operand of S^T): query qi, dims [8g, 8g+8) and the remainder block
  const int qrow = qi < U ? qi : U - 1;
  const T* qp = Qg + (long)qrow * ld;
  // dims 32.. go through a second 16x16x32 MFMA; for d_k = 48 its lanes g >= 2 (dims 48..63)
  // are zero on both operands
  const bool hi_ok = DK == 64 || g < 2;
  const u32x4 qa = *(const u32x4*)(qp + 8 * g);
  const u32x4 qb = hi_ok ? *(const u32x4*)(qp + 32 + 8 * g) : u32x4{0, 0, 0, 0};

  // this thread's tile loads: 16-byte K and V chunks (e = tid + 256 i: key e / CPR, chunk
  // e % CPR), as raw buffer loads against a per-tile resource that ends at the clip's last
  // row: rows past the clip read as zero
  int koff[KPT], kls[KPT], vls[KPT];  // global byte offset in the tile, LDS element offsets
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = tid + 256 * i, key = e / CPR, ch = e - key * CPR;
    koff[i] = (key * ld + ch * 8) * (int)sizeof(T);
    kls[i] = key * KP + ch * 8;
    vls[i] = key * VP + ch * 8;
  }
  u32x4 rk[KPT], rv[KPT];
  auto load = [&](int kv0) {
    const int bytes = (U - kv0) * ld * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rK =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (long)kv0 * ld), 0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + (long)kv0 * ld), 0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (KCH % 256 == 0 || tid + 256 * i < KCH) {
        rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rK, koff[i], 0, 0));
        rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rV, koff[i], 0, 0));
      }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (KCH % 256 == 0 || tid + 256 * i < KCH) {
        *(u32x4*)(&sK[buf][0][0] + kls[i]) = rk[i];
        *(u32x4*)(&sV[buf][0][0] + vls[i]) = rv[i];
      }
  };
  // d_k = 48: the score MFMA's upper 16 k slots read the zero pad columns [48, 56) of the
  // K rows (set once here, never overwritten by the tile stores)
  if (DK == 48 && tid < 2 * AT_KV)
    *(u32x4*)&sK[tid / AT_KV][tid % AT_KV][DK] = u32x4{0, 0, 0, 0};
  const int khi = hi_ok ? 32 + 8 * g : DK;

  // columns DK.. DK+15 of both V buffers: a column of ones then zeros, so that the P.V
  // product also accumulates each query's probability sum (in the rounded P the MFMA uses)
  {
    const int vb = tid >> 7, key = (tid >> 1) & 63, half = tid & 1;
    const uint32_t one = half == 0 ? (uint32_t)__builtin_bit_cast(uint16_t, (T)1.0f) : 0u;
    *(u32x4*)&sV[vb][key][DK + 8 * half] = u32x4{one, 0u, 0u, 0u};
  }
  // this lane's rows for the transposing V reads: lane 4 s + q of its 16-lane group names
  // key 4 g + s (and 16 + 4 g + s) of a 32-key half, dims 4 q .. 4 q + 3 of a dim block
  const int tr_key = 4 * g + (c16 >> 2), tr_dim = 4 * (c16 & 3);
  float m_run = -INFINITY;
  f32x4 o[NDBX];
#pragma unroll
  for (int db = 0; db < NDBX; ++db) o[db] = f32x4{0, 0, 0, 0};

  load(0);
  store(0);
  // every load issued so far (Q fragments, first tile) is complete here, so the loop's
  // wait-count bookkeeping starts clean and only the store waits for the prefetch
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  int buf = 0;
  for (int kv0 = 0; kv0 < U; kv0 += AT_KV) {
    const bool more = kv0 + AT_KV < U;
    if (more) load(kv0 + AT_KV);

    // S^T blocks: s[kb][r] = raw score(key kv0 + kb*16 + 4g + r, query qi)
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const T* kr = &sK[buf][kb * 16 + c16][0];
      f32x4 acc = f32x4{0, 0, 0, 0};
      acc = AttnMma<T>::k32(*(const u32x4*)(kr + 8 * g), qa, acc);
      acc = AttnMma<T>::k32(*(const u32x4*)(kr + khi), qb, acc);
      s[kb] = acc;
    }
    if (!more) {                     // the clip's last tile: keys >= U get probability 0
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kv0 + kb * 16 + 4 * g + r >= U) s[kb][r] = -INFINITY;
    }
    float mx = max3_(s[0][0], s[0][1], s[0][2]);
    mx = max3_(mx, s[0][3], s[1][0]);
    mx = max3_(mx, s[1][1], s[1][2]);
    mx = max3_(mx, s[1][3], s[2][0]);
    mx = max3_(mx, s[2][1], s[2][2]);
    mx = max3_(mx, s[2][3], s[3][0]);
    mx = max3_(mx, s[3][1], s[3][2]);
    mx = max3_(mx, s[3][3], m_run);
    const float m_new = max_xor32(max_xor16(mx));
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
      for (int db = 0; db < NDBX; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
    float pv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));

#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      float pp[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) { pp[r] = pv[2 * hk][r]; pp[4 + r] = pv[2 * hk + 1][r]; }
      const u32x4 pb = pack8f<T>(pp);
#pragma unroll
      for (int db = 0; db < NDBX; ++db) {
        // V^T rows db*16 + c16, keys 32 hk + 4 g + 0..3 and 32 hk + 16 + 4 g + 0..3
        const u32x2 lo = lds_read_tr(&sV[buf][32 * hk + tr_key][db * 16 + tr_dim]);
        const u32x2 hi = lds_read_tr(&sV[buf][32 * hk + 16 + tr_key][db * 16 + tr_dim]);
        o[db] = AttnMma<T>::k32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[db]);
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // the probability sum sits in dim DK of the extra block: lane c16 (g = 0), element 0
  const float l = __shfl(o[NDB][0], c16, 64);
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
  int tile, h;
  attn_item(blockIdx.x, p.n_tiles, p.n_heads, tile, h);
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
  dim3 grid(p.n_tiles * p.n_heads), blk(256);
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
