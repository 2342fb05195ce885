// Flash-style self-attention over packed variable-length clips for gfx950.
// softmax(q k^T / sqrt(d_k)) v per clip and head, keys beyond the clip masked
// (key-padding mask; fused scaled-dot-product attention: "GigaAM MLX port for Mac",
// section "Where the time goes"). Scores, max, sum and the output accumulator are fp32;
// the probabilities are rounded to the operand type for the second product.
#include "kernels.h"

namespace gg {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int AT_KV = 64;

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
// Block = 4 waves = 128 queries (a 128-frame tile) of one clip and one head; wave w owns
// queries 32 w .. 32 w + 31 of the tile (a wave past the clip's end only helps with the
// K / V loads). Per 64-key tile, with 32 x 32 x 16 MFMAs:
//   S^T[key][query] = K . Q^T  (A = 32 K rows from LDS, 16 dims per step; B = the wave's Q
//                               fragment in registers; d_k / 16 steps, no padded dims)
//   lane l then holds 32 scores of ONE query (l % 32): in each 32-key block the keys
//   8 (r / 4) + 4 (l / 32) + r % 4, r < 16; lanes l and l + 32 share a query, so the
//   running max needs one lane swap;
//   O^T[dim][query] += V^T . P^T with 32-dim output blocks; the probabilities go straight
//   from the score registers into the B operand (8 per lane per 16-key step: r = 8 j ..
//   8 j + 7 of a block, i.e. keys 16 j + 4 (l / 32) + {0..3} and 16 j + 8 + 4 (l / 32) +
//   {0..3}); the A operand (V^T) is read in exactly that key order with the transposing LDS
//   read, so V is never transposed in registers.
// V carries a column of ones at dim d_k, so the last output block also accumulates each
// query's probability sum in the rounded P the MFMA uses (for d_k = 48 it sits in the
// second 32-dim block's spare rows).
//
// K and V tiles are double-buffered in LDS as row-major (key, dim) copies of the global
// rows: the next 64-key tile is loaded into registers while the current one is consumed,
// and stored after it (one barrier per tile). The softmax is kept in base 2 with the scale
// folded into one FMA per score: p = 2^(s*c - m*c), c = log2(e)/sqrt(d_k), m the running
// of the raw scores seen so far (a stale one while it is within 2^8, see below). The key mask
// is applied only on a clip's last, partial tile.
//
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

__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return max3_(__uint_as_float(r[0]), __uint_as_float(r[1]), v);
}

template <typename T> struct AttnMma32;
template <> struct AttnMma32<f16> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct AttnMma32<bf16> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// KS2 = 2 (a clip or two: no more 64-query items than CUs): a block takes a 64-frame query tile; waves 0
// and 1 own its two 32-query groups over the even 64-key tiles, waves 2 and 3 the same
// queries over the odd ones, and the pairs' partial results (reference max, unnormalised
// output with its probability-sum row) are merged at the end; twice the blocks, each
// walking half the keys per wave.
template <typename T, int DK, int KS2 = 1>
__global__ void __launch_bounds__(256, KS2 == 1 ? 4 : 2) k_attn(AttnParams p) {
  constexpr int QT = 128 / KS2;      // queries per block
  constexpr int KP = DK + 8;         // K row pitch (elements): 16 rows of a read pass on disjoint banks
  // V row pitch: dims, the ones column, zeros; 96 elements (48 dwords) put the 4 rows of one
  // transposing read pass, 32 dims each, on disjoint banks
  constexpr int VP = 96;
  constexpr int KS = DK / 16;        // 16-dim steps of the score product
  constexpr int NDB = (DK + 1 + 31) / 32;   // 32-dim output blocks, the ones column included
  constexpr int CPR = DK / 8;        // 16-byte chunks per K / V row
  constexpr int KCH = AT_KV * CPR;   // 16-byte chunks per tile (each of K and V)
  constexpr int KPT = (KCH + 255) / 256;    // chunks per thread
  static_assert(DK % 16 == 0 && NDB * 32 <= VP, "head size");
  __shared__ __attribute__((aligned(16))) T sK[2][KS2][AT_KV][KP];
  __shared__ __attribute__((aligned(16))) T sV[2][KS2][AT_KV][VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, c32 = lane & 31;
  const int qg = KS2 == 1 ? wave : (wave & 1);             // the wave's 32-query group
  const int kg = KS2 == 1 ? 0 : (wave >> 1);                // its share of the key tiles
  int tile, h;
  attn_item(blockIdx.x, KS2 == 1 ? p.n_tiles : p.n_tiles64, p.n_heads, tile, h);
  int base, U, q0;                                         // clip's first row, length; wave's first query
  if constexpr (KS2 == 1) {
    const int b = p.tileQ[tile];
    base = p.cuU[b];
    U = p.cuU[b + 1] - base;
    q0 = (tile - p.cuQ[b]) * QT + qg * 32;
  } else {
    // one load for the tile's clip geometry: first row, length, first frame
    const int4 geo = *(const int4*)(p.tileG64 + 4 * tile);
    base = geo.x;
    U = geo.y;
    q0 = geo.z + qg * 32;
  }
  const bool active = q0 < U;                              // wave-uniform
  const int qi = q0 + c32;
  const int ld = 3 * p.d;
  const T* Qg = (const T*)p.qkv + (long)base * ld + h * DK;
  const T* Kg = Qg + p.d;
  const T* Vg = Qg + 2 * p.d;
  const float c = p.scale_log2;

  // Q fragments (B operand of S^T): query qi, dims 16 ks + 8 hf .. + 7
  const int qrow = qi < U ? qi : U - 1;
  const T* qp = Qg + (long)qrow * ld + 8 * hf;
  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4*)(qp + 16 * ks);

  // this thread's tile loads: 16-byte K and V chunks (e = tid + 256 i: key e / CPR, chunk
  // e % CPR), as raw buffer loads against a per-tile resource that ends at the clip's last
  // row: rows past the clip read as zero
  // Chunk e of a tile goes to LDS so that every 16 lanes of one store hit disjoint banks:
  //  K (row pitch 28 dwords): 16 consecutive keys, one chunk column;
  //  V (row pitch 48 dwords): 4 consecutive keys x 4 consecutive chunks (the last
  //    chunks of each row, fewer than 4, take 8 keys x 2 chunks).
  int koff[KPT], voff[KPT], kls[KPT], vls[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = tid + 256 * i;
    {
      const int blk = e / (16 * CPR), r = e - blk * 16 * CPR;
      const int key = 16 * blk + (r & 15), ch = r >> 4;
      koff[i] = (key * ld + ch * 8) * (int)sizeof(T);
      kls[i] = key * KP + ch * 8;
    }
    {
      constexpr int C4 = CPR / 4 * 4;               // chunks placed 4 at a time
      int key, ch;
      if (e < AT_KV * C4) {
        const int g = e >> 4, l = e & 15, cg = g / (AT_KV / 4), kg = g - cg * (AT_KV / 4);
        key = 4 * kg + (l >> 2);
        ch = 4 * cg + (l & 3);
      } else {
        const int r = e - AT_KV * C4, w = CPR - C4;
        key = r / w;
        ch = C4 + r % w;
      }
      voff[i] = (key * ld + ch * 8) * (int)sizeof(T);
      vls[i] = key * VP + ch * 8;
    }
  }
  u32x4 rk[KS2][KPT], rv[KS2][KPT];
  // key tiles kv0 + 64 j, j < KS2 (a tile past the clip reads as zeros: empty resource)
  auto load = [&](int kv0) {
#pragma unroll
    for (int j = 0; j < KS2; ++j) {
      const int kvj = kv0 + AT_KV * j;
      const bool in = j == 0 || kvj < U;       // the first tile is always inside the clip
      const int bytes = in ? (U - kvj) * ld * (int)sizeof(T) : 0;
      const int kvc = in ? kvj : 0;
      const __amdgpu_buffer_rsrc_t rK =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (long)kvc * ld), 0, bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rV =
          __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + (long)kvc * ld), 0, bytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (KCH % 256 == 0 || tid + 256 * i < KCH) {
          rk[j][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rK, koff[i], 0, 0));
          rv[j][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rV, voff[i], 0, 0));
        }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KS2; ++j)
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (KCH % 256 == 0 || tid + 256 * i < KCH) {
          *(u32x4*)(&sK[buf][j][0][0] + kls[i]) = rk[j][i];
          *(u32x4*)(&sV[buf][j][0][0] + vls[i]) = rv[j][i];
        }
  };
  // columns DK .. VP - 1 of both V buffers: one at DK, zeros after it (never overwritten by
  // the tile stores)
  {
    constexpr int XC = (VP - DK) / 8;            // 16-byte chunks per row past the dims
    const uint32_t one = (uint32_t)__builtin_bit_cast(uint16_t, (T)1.0f);
    for (int e = tid; e < 2 * KS2 * AT_KV * XC; e += 256) {
      const int vb = e / (AT_KV * XC), rem = e - vb * AT_KV * XC, key = rem / XC, x = rem - key * XC;
      *(u32x4*)&sV[vb / KS2][vb % KS2][key][DK + 8 * x] = u32x4{x == 0 ? one : 0u, 0u, 0u, 0u};
    }
  }
  // this lane's transposing V reads: lane 4 s + q of its 16-lane group g names key
  // 4 (g / 2) + s (plus 8 for the second read) of a 16-key step, dims 16 (g % 2) + 4 q ..
  // + 3 of a 32-dim block; it receives dim (lane % 32) of keys 4 hf + {0..3} (+ 8)
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_key = 4 * (g16 >> 1) + (i16 >> 2), tr_dim = 16 * (g16 & 1) + 4 * (i16 & 3);
  float m_run = -INFINITY;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  load(0);
  store(0);
  // every load issued so far (Q fragments, first tile) is complete here, so the loop's
  // wait-count bookkeeping starts clean and only the store waits for the prefetch
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  int buf = 0;
  for (int kv0 = 0; kv0 < U; kv0 += AT_KV * KS2) {
    const bool more = kv0 + AT_KV * KS2 < U;
    if (more) load(kv0 + AT_KV * KS2);
    const int kvw = kv0 + AT_KV * kg;                       // this wave's key tile
    if (active && (KS2 == 1 || kvw < U)) {
      // S^T blocks: s[kb][r] = raw score(key kvw + 32 kb + 8 (r / 4) + 4 hf + r % 4, query qi)
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const T* kr = &sK[buf][kg][kb * 32 + c32][8 * hf];
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = AttnMma32<T>::run(*(const u32x4*)(kr + 16 * ks), qf[ks], acc);
        s[kb] = acc;
      }
      if (KS2 == 1 ? !more : kvw + AT_KV > U) {   // the clip's last tile: keys >= U get probability 0
        const int lim = U - kvw - 4 * hf;         // first masked key offset of this lane's rows
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
      }
      float mx = max3_(s[0][0], s[0][1], m_run);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = max3_(mx, s[0][r], s[0][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = max3_(mx, s[1][r], s[1][r + 1]);
      const float m_new = max_xor32(mx);
      // The reference point of the exponentials moves only when some query's maximum rose by
      // more than 8 in base-2 units: until then every probability stays below 2^8, and the
      // numerator and the sum (the ones column) share the same reference, so the result is
      // unchanged while most tiles skip the rescale.
      if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > 8.0f)) {
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        m_run = m_new;
      }
      const float mc = m_run * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float pp[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) pp[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * j + t], c, -mc));
          const u32x4 pb = pack8f<T>(pp);
          const int k0 = 32 * kb + 16 * j + tr_key;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x2 lo = lds_read_tr(&sV[buf][kg][k0][32 * db + tr_dim]);
            const u32x2 hi = lds_read_tr(&sV[buf][kg][k0 + 8][32 * db + tr_dim]);
            o[db] = AttnMma32<T>::run(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, o[db]);
          }
        }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if constexpr (KS2 == 2) {
    // merge the odd-tile waves' results into the even-tile waves' (every wave is past its
    // last LDS read: the loop ended on a barrier): per lane its query's reference max and
    // output rows, scaled to the larger of the two maxima
    constexpr int XW = 1 + NDB * 16;
    float* xo = (float*)&sK[0][0][0][0] + (qg * 64 + lane) * XW;
    if (kg == 1) {
      xo[0] = m_run;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[1 + 16 * db + r] = o[db][r];
    }
    __syncthreads();
    if (kg == 1 || !active) return;
    const float mb = xo[0];
    const float mm = fmaxf(m_run, mb);
    const float fa = __builtin_amdgcn_exp2f((m_run - mm) * c);
    const float fb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mb - mm) * c);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * fa + xo[1 + 16 * db + r] * fb;
  }
  if (!active) return;

  // the probability sum: dim DK of block DK / 32, i.e. row DK % 32 of that block, held by
  // the lanes of half (DK % 32) / 4 % 2 at r = 4 ((DK % 32) / 8) + DK % 4 (DK % 32 is 16 or 0)
  constexpr int LR = DK % 32, LDB = DK / 32;
  constexpr int LHF = (LR >> 2) & 1, LRR = 4 * (LR >> 3) + (LR & 3);
  const float lsum = __shfl(o[LDB][LRR], c32 + 32 * LHF, 64);
  if (qi < U) {
    const float inv = 1.0f / lsum;
    T* op = (T*)p.out + (long)(base + qi) * p.d + h * DK;
    typedef T t4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dim = 32 * db + 8 * rg + 4 * hf;
        if (dim < DK) {
          t4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (T)(o[db][4 * rg + r] * inv);
          *(t4*)(op + dim) = w;
        }
      }
  }
}

// ---------------------------------------------------------------- fp32 kernel
// 64-frame query tiles, 16 queries per wave, v_mfma_f32_16x16x4_f32 (one k element per lane
// group); lane l holds the scores of query l % 16 for keys 16 kb + 4 (l / 16) + r.
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

constexpr long kAttnSplitMax = 256;           // 64-query items: at most one per CU

hipError_t launch_attention(DType dt, int dk, const AttnParams& p, hipStream_t s) {
  if (p.n_tiles <= 0) return hipSuccess;
  dim3 grid(p.n_tiles * p.n_heads), blk(256);
  // a clip or two: 64-query items with the keys split between two wave pairs (one 20 s clip:
  // 64 -> 128 workgroups), as long as every such workgroup gets a CU of its own (beyond that,
  // two of them sharing a CU take as long as one 128-query item, and the merge is extra)
  const bool split = dt != DT_F32 && p.n_tiles64 > 0 && p.tileG64 &&
                     (long)p.n_tiles64 * p.n_heads <= kAttnSplitMax;
  dim3 grid2(split ? p.n_tiles64 * p.n_heads : 1);
#define GG_A(T, D) hipLaunchKernelGGL((k_attn<T, D>), grid, blk, 0, s, p)
#define GG_A2(T, D) hipLaunchKernelGGL((k_attn<T, D, 2>), grid2, blk, 0, s, p)
  if (dt == DT_F32) {
    if (dk == 48) hipLaunchKernelGGL(k_attn_f32<48>, grid, blk, 0, s, p);
    else if (dk == 64) hipLaunchKernelGGL(k_attn_f32<64>, grid, blk, 0, s, p);
    else return hipErrorInvalidValue;
  } else if (split) {
    if (dt == DT_BF16) {
      if (dk == 48) GG_A2(bf16, 48); else if (dk == 64) GG_A2(bf16, 64); else return hipErrorInvalidValue;
    } else {
      if (dk == 48) GG_A2(f16, 48); else if (dk == 64) GG_A2(f16, 64); else return hipErrorInvalidValue;
    }
  } else if (dt == DT_BF16) {
    if (dk == 48) GG_A(bf16, 48); else if (dk == 64) GG_A(bf16, 64); else return hipErrorInvalidValue;
  } else {
    if (dk == 48) GG_A(f16, 48); else if (dk == 64) GG_A(f16, 64); else return hipErrorInvalidValue;
  }
#undef GG_A
#undef GG_A2
  return hipGetLastError();
}

}  // namespace gg
