// MFMA GEMM for gfx950: C = epilogue(A * W^T + bias), A [M][K] and W [N][K] both
// K-contiguous (PyTorch Linear layout), fp32 accumulation.
//
// These are the dense contractions of the encoder (subsampling convs as implicit GEMMs,
// FFN, q/k/v/out projections, pointwise convs, CTC head): "GigaAM MLX port for Mac",
// section "Why parts of the model cannot simply be removed", notes that most of the time
// goes to multiplying large matrices.
//
// Structure: 256 threads = 4 waves on a WGM x WGN grid; block tile BM x BN; k-tile of
// 128 bytes per row (64 fp16/bf16 or 32 fp32 elements); LDS double buffer with register
// staging, one barrier per k-tile. Each wave owns (BM/WGM) x (BN/WGN) built from 32x32
// MFMA blocks: v_mfma_f32_32x32x16_{f16,bf16} (8 elements per lane) or four
// v_mfma_f32_32x32x2_f32 for fp32. A 16-byte LDS fragment per lane feeds either.
// Because the A and B fragments of a lane always carry the same k indices, the sum over
// k is exact whatever order the hardware assigns to the k slots.
#include <cstring>

#include "kernels.h"

namespace gg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;
template <> struct Mma<f16> {
  static __device__ __forceinline__ void run(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16& acc, u32x4 a, u32x4 b) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
  }
};

// 8 floats -> 8 elements of T packed in 16 bytes (round to nearest even).
template <typename T> __device__ __forceinline__ u32x4 pack8(f32x4 lo, f32x4 hi);
template <> __device__ __forceinline__ u32x4 pack8<f16>(f32x4 lo, f32x4 hi) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) { h[i] = (f16)lo[i]; h[4 + i] = (f16)hi[i]; }
  return __builtin_bit_cast(u32x4, h);
}
template <> __device__ __forceinline__ u32x4 pack8<bf16>(f32x4 lo, f32x4 hi) {
  bf16x8 h;
#pragma unroll
  for (int i = 0; i < 4; ++i) { h[i] = (bf16)lo[i]; h[4 + i] = (bf16)hi[i]; }
  return __builtin_bit_cast(u32x4, h);
}

// 16 packed QB-bit weights times one fp16 scale -> 16 fp16 (two 16-byte chunks). The 16
// weights are 2*QB bytes: QB = 8 one byte each; QB = 4 two per byte, low nibble first;
// QB = 6 four per 3 bytes (a little-endian 24-bit word, weight j at bits 6j..6j+5). Every
// value is a two's-complement integer in [-(2^(QB-1) - 1), 2^(QB-1) - 1].
template <int QB> __device__ __forceinline__ int qval(u32x4 q, int i);
template <> __device__ __forceinline__ int qval<8>(u32x4 q, int i) {
  return (int)(int8_t)((q[i >> 2] >> (8 * (i & 3))) & 0xff);
}
template <> __device__ __forceinline__ int qval<4>(u32x4 q, int i) {
  return ((int)(q[i >> 3] << (28 - 4 * (i & 7)))) >> 28;
}
template <> __device__ __forceinline__ int qval<6>(u32x4 q, int i) {
  const int g = i >> 2, j = i & 3;                  // 24-bit group g at byte 3g
  const int bit = 24 * g + 6 * j;                   // bit offset in the 96-bit string
  const int w = bit >> 5, o = bit & 31;
  uint64_t two = (uint64_t)q[w] | ((w + 1 < 3) ? (uint64_t)q[w + 1] << 32 : 0ull);
  return ((int)((uint32_t)(two >> o) << 26)) >> 26;
}
template <int QB>
__device__ __forceinline__ void dequant16(u32x4 q, float s, u32x4& lo, u32x4& hi) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (f16)((float)qval<QB>(q, i) * s);
    b[i] = (f16)((float)qval<QB>(q, 8 + i) * s);
  }
  lo = __builtin_bit_cast(u32x4, a);
  hi = __builtin_bit_cast(u32x4, b);
}

// Tile order. Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8), each XCD with its own L2. Give every XCD a contiguous range of tiles, and
// walk each range in groups of GM tile-rows, so the workgroups that are resident on one
// XCD at the same time share their A rows and W rows through that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(int bid, int nM, int nN, int& tm, int& tn) {
  const int total = nM * nN;
  const int q = total / kXcds, r = total % kXcds;
  const int x = bid % kXcds, j = bid / kXcds;
  const int t = x * q + (x < r ? x : r) + j;          // bijective: XCD x owns a contiguous range
  const int group = kGroupM * nN;
  const int g = t / group, first = g * kGroupM;
  const int rows = (nM - first) < kGroupM ? (nM - first) : kGroupM;
  const int w = t - g * group;
  tm = first + w % rows;
  tn = w / rows;
}

// Epilogue of a wave's (32 MI) x (32 NI) accumulator tile whose first row is rm and first
// column cn. 32x32 MFMA accumulator: lane holds column (lane & 31) and rows
// 8 * (r / 4) + 4 * (lane / 32) + (r % 4), r = 0..15. GLU pairs column block 2q (value)
// with 2q + 1 (gate); their output column starts at cglu / 2.
template <typename T, int MI, int NI, int EP>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16 (&acc)[MI][NI], int rm, int cn,
                                         int cglu, int lane) {
  const int rbase = rm + 4 * (lane >> 5);
  const int cbase = cn + (lane & 31);
  if constexpr (EP == E_GLU) {
#pragma unroll
    for (int q = 0; q < NI / 2; ++q) {
      const int cv = cbase + 2 * q * 32, cg = cv + 32;
      const int co = cglu / 2 + q * 32 + (lane & 31);
      if (cv >= p.N) continue;
      const float bv = p.bias ? p.bias[cv] : 0.f, bg = p.bias ? p.bias[cg] : 0.f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          if (row < p.M) {
            const float v = acc[mi][2 * q][r] + bv, g = acc[mi][2 * q + 1][r] + bg;
            ((T*)p.C)[(long)row * p.ldc + co] = from_f32<T>(v * sigmoidf_(g));
          }
        }
    }
  } else if constexpr (EP == E_RESID) {
    // x += alpha * (acc + b): issue every residual load of the lane first, then the stores,
    // so the read-modify-write costs one memory round trip instead of MI * NI * 16.
    float* X = (float*)p.C;
    float old[MI][NI][16];
    const bool full = rm + 32 * MI <= p.M;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = cbase + ni * 32;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          old[mi][ni][r] = (col < p.N && (full || row < p.M)) ? X[(long)row * p.ldc + col] : 0.f;
        }
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = cbase + ni * 32;
      if (col >= p.N) continue;
      const float bb = p.bias ? p.bias[col] : 0.f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          if (full || row < p.M)
            X[(long)row * p.ldc + col] = old[mi][ni][r] + p.alpha * (acc[mi][ni][r] + bb);
        }
    }
  } else {
    const bool full = rm + 32 * MI <= p.M;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = cbase + ni * 32;
      if (col >= p.N) continue;
      const float bb = p.bias ? p.bias[col] : 0.f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + mi * 32 + 8 * (r >> 2) + (r & 3);
          if (full || row < p.M) {
            const float v = acc[mi][ni][r] + bb;
            const long o = (long)row * p.ldc + col;
            if constexpr (EP == E_STORE) ((T*)p.C)[o] = from_f32<T>(v);
            else if constexpr (EP == E_SILU) ((T*)p.C)[o] = from_f32<T>(siluf_(v));
            else if constexpr (EP == E_RELU) ((T*)p.C)[o] = from_f32<T>(fmaxf(v, 0.f));
            else if constexpr (EP == E_RELU_F32) ((float*)p.C)[o] = fmaxf(v, 0.f);
            else ((float*)p.C)[o] = v;
          }
        }
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, int AM, int QB, int EP>
__global__ void __launch_bounds__(256) k_gemm(GemmParams p) {
  constexpr int ES = sizeof(T);
  constexpr int EPC = 16 / ES;                  // elements per 16-byte chunk
  constexpr int BKE = 128 / ES;                 // elements per k-tile
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int LDR = 9;                        // 16-byte slots per LDS row (8 + pad)
  constexpr int A_CH = BM * 8 / 256;
  constexpr bool Q8 = QB != 0;                 // quantised weights (QB bits each)
  constexpr int B_CH = Q8 ? BN * 4 / 256 : BN * 8 / 256;
  constexpr bool AF = (AM == A_F32 || AM == A_CONV_F32) && ES == 2;   // float source
  constexpr bool CONV = (AM == A_CONV || AM == A_CONV_F32);
  static_assert(WGM * WGN == 4 && MI >= 1 && NI >= 1, "tile");
  static_assert(A_CH >= 1 && B_CH >= 1, "tile");
  static_assert(EP != E_GLU || NI % 2 == 0, "GLU needs value/gate block pairs");

  __shared__ u32x4 sA[2][BM][LDR];
  __shared__ u32x4 sB[2][BN][LDR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // split-K: slice blockIdx.y takes k-tiles [kt0, kt0 + KT) and writes its own fp32 slice
  const int KT = p.K / BKE / (int)gridDim.y, kt0 = (int)blockIdx.y * KT;
  if (gridDim.y > 1) p.C = (float*)p.C + blockIdx.y * (long)p.M * p.ldc;

  const char* Abase = (const char*)((AM == A_DUAL && n0 >= p.nsplit) ? p.A2 : p.A);

  // ---- per-thread A rows
  int a_row[A_CH], a_col[A_CH];
  long a_off[A_CH];
  int a_lo[A_CH], a_hi[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + 256 * i;
    a_row[i] = c >> 3;
    a_col[i] = c & 7;
    int gm = m0 + a_row[i];
    gm = gm < p.M ? gm : p.M - 1;
    if constexpr (CONV) {
      const int b = p.rowclip[gm];
      const int s = gm - p.cu_out[b];
      a_lo[i] = p.cu_in[b];
      a_hi[i] = p.cu_in[b + 1];
      a_off[i] = (long)a_lo[i] + 2 * s - 2;     // source row of tap 0
    } else {
      a_lo[i] = a_hi[i] = 0;
      a_off[i] = (long)gm * p.lda;
    }
  }
  // ---- per-thread W rows
  int b_row[B_CH], b_col[B_CH];
  long b_off[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + 256 * i;
    b_row[i] = Q8 ? (c >> 2) : (c >> 3);
    b_col[i] = Q8 ? (c & 3) : (c & 7);
    int gn = n0 + b_row[i];
    gn = gn < p.N ? gn : p.N - 1;
    b_off[i] = (long)gn * p.ldw;
  }

  u32x4 ra[A_CH][AF ? 2 : 1];
  u32x4 rb[B_CH];
  float rs[B_CH];

  auto load_tile = [&](int kt) {
    const int kk = kt * BKE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      long src;
      bool ok = true;
      if constexpr (CONV) {
        const int j = kk / p.cin, c0 = kk - j * p.cin;
        const long r = a_off[i] + j;
        ok = (r >= a_lo[i]) && (r < a_hi[i]);
        src = (ok ? r : a_lo[i]) * p.cin + c0 + a_col[i] * EPC;
      } else {
        src = a_off[i] + kk + a_col[i] * EPC;
      }
      if constexpr (AF) {
        const f32x4* q = (const f32x4*)((const float*)Abase + src);
        f32x4 lo = q[0], hi = q[1];
        if (!ok) { lo = f32x4{0, 0, 0, 0}; hi = lo; }
        ra[i][0] = __builtin_bit_cast(u32x4, lo);
        ra[i][1] = __builtin_bit_cast(u32x4, hi);
      } else {
        u32x4 v = *(const u32x4*)(Abase + src * ES);
        if (!ok) v = u32x4{0, 0, 0, 0};
        ra[i][0] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if constexpr (Q8) {
        // 16 weights = 2 QB bytes at byte (k * QB / 8) of the packed row
        const uint8_t* q = (const uint8_t*)p.W + (b_off[i] + kk + b_col[i] * 16) * QB / 8;
        if constexpr (QB == 8) rb[i] = *(const u32x4*)q;
        else if constexpr (QB == 4) { const u32x2 v = *(const u32x2*)q; rb[i] = u32x4{v[0], v[1], 0, 0}; }
        else rb[i] = u32x4{((const uint32_t*)q)[0], ((const uint32_t*)q)[1], ((const uint32_t*)q)[2], 0};
        int gn = n0 + b_row[i];
        gn = gn < p.N ? gn : p.N - 1;
        rs[i] = (float)p.Wscale[(long)gn * (p.K / 64) + kt];
      } else {
        rb[i] = *(const u32x4*)((const char*)p.W + (b_off[i] + kk + b_col[i] * EPC) * ES);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if constexpr (AF)
        sA[buf][a_row[i]][a_col[i]] = pack8<T>(__builtin_bit_cast(f32x4, ra[i][0]),
                                               __builtin_bit_cast(f32x4, ra[i][1]));
      else
        sA[buf][a_row[i]][a_col[i]] = ra[i][0];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if constexpr (Q8) {
        u32x4 lo, hi;
        dequant16<QB>(rb[i], rs[i], lo, hi);
        sB[buf][b_row[i]][b_col[i] * 2] = lo;
        sB[buf][b_row[i]][b_col[i] * 2 + 1] = hi;
      } else {
        sB[buf][b_row[i]][b_col[i]] = rb[i];
      }
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  load_tile(kt0);
  store_tile(0);
  __syncthreads();

  const int fr = lane & 31, fk = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt0 + kt + 1);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = sA[cur][wm * WTM + mi * 32 + fr][kc * 2 + fk];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = sB[cur][wn * WTN + ni * 32 + fr][kc * 2 + fk];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) Mma<T>::run(acc[mi][ni], af[mi], bfr[ni]);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  epilogue<T, MI, NI, EP>(p, acc, m0 + wm * WTM, n0 + wn * WTN, n0 + wn * WTN, lane);
}

// ---------------------------------------------------------------------------------------
// Pipelined fp16/bf16 GEMM with direct global->LDS loads (gfx950 global_load_lds_dwordx4):
// one 64-lane load instruction drops 1 KiB straight into LDS (lane i -> bytes 16i..16i+15),
// with no staging registers and no LDS store instructions. S k-tiles are in flight; a
// k-tile is consumed after `s_waitcnt vmcnt` (own loads) and a barrier (everyone's).
// LDS rows hold one k-tile (64 or 32 k-elements); their 16-byte chunks are XOR-swizzled by a
// row key so the fragment reads of 16 consecutive rows hit 16 different bank groups.
//
// The loads are issued from inline asm because the compiler, not knowing which LDS stage
// a DMA targets, waits for all of them (vmcnt(0)) before any LDS read; the waits below
// are exact instead. The asm has no register outputs.

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// (m0 carries the LDS destination. It is a reserved register for the compiler, which sets
// it afresh before every instruction that reads it and never keeps a value in it, so
// overwriting it here cannot disturb compiled code.)
__device__ __forceinline__ void dma16(uint32_t lds, const void* g) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n (uniform, 0 <= n <= MAXN) groups of L loads are still in flight
template <int L, int MAXN> __device__ __forceinline__ void wait_groups(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<MAXN * L>();
    else wait_groups<L, MAXN - 1>(n);
  }
}

// 4 floats -> 4 elements of T in 8 bytes (round to nearest even)
template <typename T> __device__ __forceinline__ u32x2 pack4(f32x4 v);
template <> __device__ __forceinline__ u32x2 pack4<f16>(f32x4 v) {
  f16x4 h = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  return __builtin_bit_cast(u32x2, h);
}
template <> __device__ __forceinline__ u32x2 pack4<bf16>(f32x4 v) {
  bf16x4 h = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  return __builtin_bit_cast(u32x2, h);
}

// ---------------------------------------------------------------------------------------
// The direct-load GEMM, software-pipelined: each wave reads the fragments of the next
// 16-k phase between the MFMAs of the current one, and the k-tile boundary (own loads
// waited, then the barrier) sits before the last phase's MFMAs, whose slots also issue
// the loads of k-tile kt + S into the stage just freed, spread evenly over the MFMAs. A
// wave never waits for an LDS read it issued in the same phase; the second wave on each
// SIMD fills the remaining gaps (and runs its epilogue math while the other computes).
//
// The MFMA operands are swapped (W rows feed the MFMA's rows): a lane's accumulators of
// a 32 x 32 block are one output row and four runs of 4 consecutive output columns, so
// the epilogue stages the tile in LDS with 8-byte (T) or 16-byte (fp32) writes before the
// row-wise 16-byte copy-out (every thread's LDS reads issued before its stores).

// rows per epilogue chunk: the largest power-of-two part of BM that fits the LDS
constexpr int chunk_rows(int BM, int fit) {
  int c = BM;
  while (c > fit && c > 32) c /= 2;
  return c;
}

// 16 zero bytes: the source of every load of a subsampling-conv tap that falls outside its clip
__device__ __align__(16) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

template <typename T, int BM, int BN, int WGM, int WGN, int S, int KB, int AM, int EP, int OCC = 1>
__global__ void __launch_bounds__(64 * WGM * WGN, OCC) k_gemm_p(GemmParams p) {
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int WTM = BM / WGM, WTN = BN / WGN, MI = WTM / 32, NI = WTN / 32;
  constexpr int RB = KB * 2, CPR = RB / 16, RPI = 1024 / RB;
  constexpr int SWS = (RB == 128) ? 1 : 2;
  constexpr int ROWS = BM + BN, STAGE = ROWS * RB;
  constexpr int LPW = ROWS / RPI / NW;                 // loads per wave per k-tile
  constexpr int PH = KB / 16;                          // 16-k phases per k-tile
  constexpr int NM = MI * NI, NR = MI + NI;
  constexpr int R0 = NR >= NM ? 0 : NM - NR;           // first MFMA slot of the boundary reads
  static_assert(KB == 32 || KB == 64, "k-tile");
  static_assert(LPW * RPI * NW == ROWS, "load plan");
  // the prologue leaves up to S - 1 load groups in flight (the vmcnt field is 6 bits)
  static_assert(LPW * (S - 1) <= 63 && S >= 2, "vmcnt range");
  static_assert(EP != E_GLU || NI % 2 == 0, "GLU needs value/gate block pairs");
  static_assert(AM == A_PLAIN || AM == A_DUAL || AM == A_CONV, "A mode");
  constexpr bool CONV = AM == A_CONV;
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  int tm, tn;
  tile_coords(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = p.K / KB;
  const char* Ab = (const char*)((AM == A_DUAL && n0 >= p.nsplit) ? p.A2 : p.A);
  const long koff = (long)blockIdx.y * p.K;            // split-K slice
  if (gridDim.y > 1) p.C = (float*)p.C + blockIdx.y * (long)p.M * p.ldc;

  // The implicit subsampling conv (kernel 5, stride 2, padding 2, clips packed by rows):
  // the A row of output frame s of clip b is source rows r0 .. r0 + 4 (r0 = the clip's
  // first source row + 2s - 2) laid end to end, which is contiguous memory, so it streams
  // like a plain row. A k-tile lies inside one tap (cin is a multiple of KB); a tap outside
  // the clip loads the zero chunk instead. Bit 5i + j of tapok: load i's row has tap j
  // inside its clip (all bits set for weight rows).
  unsigned long long tapok = 0;
  const char* src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int R = RPI * (wave * LPW + i) + lane / CPR;
    const int lc = (lane % CPR) ^ ((R >> SWS) & (CPR - 1));
    if (R < BM) {
      const int gm = m0 + R < p.M ? m0 + R : p.M - 1;
      if constexpr (CONV) {
        const int b = p.rowclip[gm];
        const int lo = p.cu_in[b], hi = p.cu_in[b + 1];
        const long r0 = (long)lo + 2 * (gm - p.cu_out[b]) - 2;
#pragma unroll
        for (int j = 0; j < 5; ++j)
          if (r0 + j >= lo && r0 + j < hi) tapok |= 1ull << (5 * i + j);
        // (r0 is two rows before the clip for its first frame: such a row's taps 0 and 1
        // take the zero chunk, so this address is only dereferenced from tap 2 on)
        src[i] = Ab + (r0 * p.cin + koff + lc * 8) * (long)sizeof(T);
      } else {
        src[i] = Ab + ((long)gm * p.lda + koff + lc * 8) * sizeof(T);
      }
    } else {
      const int gn = n0 + R - BM < p.N ? n0 + R - BM : p.N - 1;
      src[i] = (const char*)p.W + ((long)gn * p.ldw + koff + lc * 8) * sizeof(T);
      tapok |= 31ull << (5 * i);
    }
  }
  // tap of k-tile g: (koff / KB + g) / (cin / KB), by a multiply (exact while the k-tile
  // index times cin / KB stays below 2^20)
  const uint32_t kt_tap = CONV ? (uint32_t)(p.cin / KB) : 1u;
  const uint32_t tap_mul = (1u << 20) / kt_tap + 1u;
  const uint32_t kt0 = (uint32_t)(koff / KB);
  auto asrc = [&](int i, int g) -> const char* {
    const char* a = src[i] + (long)g * RB;
    if constexpr (CONV) {
      const uint32_t j = ((kt0 + (uint32_t)g) * tap_mul) >> 20;
      if (!((tapok >> (5 * i + j)) & 1ull)) a = (const char*)g_zero16;
    }
    return a;
  };
  const uint32_t sbase = lds_u32(smem) + wave * LPW * 1024;

  f32x16 acc[NI][MI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ni][mi][r] = 0.0f;

  const int frow = (lane & 31) * RB;
  const int fkey = ((lane & 31) >> SWS) & (CPR - 1);
  const int arow = (wm * WTM) * RB + frow, brow = (BM + wn * WTN) * RB + frow;
  u32x4 fa[2][MI], fb[2][NI];
  auto rd = [&](int st, int kc, int b, int r) {
    const int off = st * STAGE + ((((kc * 2) + (lane >> 5)) ^ fkey) << 4);
    if (r < MI) fa[b][r] = *(const u32x4*)(smem + off + arow + r * 32 * RB);
    else fb[b][r - MI] = *(const u32x4*)(smem + off + brow + (r - MI) * 32 * RB);
  };

  // epilogue geometry: the output is staged through LDS in chunks of CH rows
  constexpr bool F32OUT = (EP == E_RESID || EP == E_F32 || EP == E_RELU_F32);
  constexpr int OES = F32OUT ? 4 : (int)sizeof(T);
  constexpr int BNO = (EP == E_GLU) ? BN / 2 : BN;
  constexpr int PITCH = BNO * OES + 16;
  constexpr int CH = chunk_rows(BM, (S * STAGE) / PITCH);
  constexpr int NCH = BM / CH;
  constexpr int SEGS = BNO * OES / 16;
  constexpr int PER = (CH * SEGS + NT - 1) / NT;
  constexpr int EPS = 16 / OES;
  static_assert(CH >= 32 && BM % CH == 0 && CH * PITCH <= S * STAGE, "epilogue chunking");
  const int n0o = (EP == E_GLU) ? n0 / 2 : n0;
  const int Nout = (EP == E_GLU) ? p.N / 2 : p.N;
  const bool vec = ((long)p.ldc * OES) % 16 == 0;
  // Residual epilogue, one workgroup per CU: the x segments this thread will update are read
  // now, so that their HBM reads overlap the main loop rather than follow it (every tile of
  // such a launch reaches its epilogue at about the same time). Loads complete in issue
  // order, so these extra ones only make the k-tile waits below stricter, never looser.
  constexpr bool PFX = EP == E_RESID && OCC == 1 && NCH * PER <= 16;
  f32x4 xpre[PFX ? NCH * PER : 1];
  if constexpr (PFX) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + NT * i, rl = e / SEGS, sg = e % SEGS;
        const int row = m0 + c * CH + rl, col = n0o + sg * EPS;
        xpre[c * PER + i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (e < CH * SEGS && row < p.M && vec && col + EPS <= Nout)
          xpre[c * PER + i] = *(const f32x4*)((const char*)p.C + ((long)row * p.ldc + col) * 4);
      }
  }

  // prologue: k-tiles 0 .. S-1 in flight, then k-tile 0 complete
#pragma unroll
  for (int g = 0; g < S; ++g)
    if (g < KT)
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma16(sbase + g * STAGE + i * 1024, asrc(i, g));
  wait_groups<LPW, S - 1>((KT < S ? KT : S) - 1);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) rd(0, 0, 0, r);

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % S, sn = (kt + 1) % S;
#pragma unroll
    for (int kc = 0; kc < PH; ++kc) {
      const int b = kc & 1;
      if (kc < PH - 1) {
#pragma unroll
        for (int j = 0; j < NM; ++j) {
          Mma<T>::run(acc[j % NI][j / NI], fb[b][j % NI], fa[b][j / NI]);
          if (j < NR) rd(st, kc + 1, b ^ 1, j);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NR > NM) {
#pragma unroll
          for (int r = NM; r < NR; ++r) rd(st, kc + 1, b ^ 1, r);
        }
      } else {
        // boundary: k-tile kt + 1 landed (own loads, then everyone's), stage st free
        if (kt + 1 < KT) {
          // groups kt + 2 .. min(kt + S - 1, KT - 1) may stay in flight
          wait_groups<LPW, S - 2>((KT - 2 - kt) < (S - 2) ? (KT - 2 - kt) : (S - 2));
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const bool more = kt + S < KT, next = kt + 1 < KT;
#pragma unroll
        for (int j = 0; j < NM; ++j) {
          Mma<T>::run(acc[j % NI][j / NI], fb[b][j % NI], fa[b][j / NI]);
          if (more) {
#pragma unroll
            for (int i = 0; i < LPW; ++i)          // loads spread evenly over the slots
              if (i * NM / LPW == j) dma16(sbase + st * STAGE + i * 1024, asrc(i, kt + S));
          }
          // the next k-tile's first reads take the last slots (all slots when NR > NM)
          if (next && j >= R0) rd(sn, 0, 0, j - R0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NR > NM) {
          if (next)
#pragma unroll
            for (int r = NM; r < NR; ++r) rd(sn, 0, 0, r);
        }
      }
    }
  }

  // ---- epilogue: stage through LDS in chunks of whole 32-row blocks, copy out rows
  const int lr = lane & 31, h4 = 4 * (lane >> 5);
  // this lane's bias: 4 consecutive columns per (block, g), loaded once
  f32x4 bv[NI][4];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = n0 + wn * WTN + ni * 32 + 8 * g + h4;
      bv[ni][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p.bias) {
        if (col + 4 <= p.N && (p.N & 3) == 0) bv[ni][g] = *(const f32x4*)(p.bias + col);
        else
          for (int j = 0; j < 4; ++j) bv[ni][g][j] = col + j < p.N ? p.bias[col + j] : 0.f;
      }
    }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    __syncthreads();
    const int rb0 = wm * WTM - c * CH;                          // wave's first row in the chunk
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rb = rb0 + mi * 32;
      if (rb >= 0 && rb < CH) {
        char* srow = smem + (rb + lr) * PITCH;
        if constexpr (EP == E_GLU) {
#pragma unroll
          for (int q = 0; q < NI / 2; ++q)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 v;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                v[j] = (acc[2 * q][mi][4 * g + j] + bv[2 * q][g][j]) *
                       sigmoidf_(acc[2 * q + 1][mi][4 * g + j] + bv[2 * q + 1][g][j]);
              *(u32x2*)(srow + (wn * WTN / 2 + q * 32 + 8 * g + h4) * OES) = pack4<T>(v);
            }
        } else {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 v;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float x = acc[ni][mi][4 * g + j] + bv[ni][g][j];
                v[j] = (EP == E_SILU) ? siluf_(x) : (EP == E_RESID) ? p.alpha * x
                       : (EP == E_RELU_F32 || EP == E_RELU) ? fmaxf(x, 0.f) : x;
              }
              const int cs = wn * WTN + ni * 32 + 8 * g + h4;
              if constexpr (F32OUT) *(f32x4*)(srow + cs * 4) = v;
              else *(u32x2*)(srow + cs * OES) = pack4<T>(v);
            }
        }
      }
    }
    __syncthreads();
    u32x4 sv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, rl = e / SEGS, sg = e % SEGS;
      if (e < CH * SEGS) sv[i] = *(const u32x4*)(smem + rl * PITCH + sg * 16);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + NT * i, rl = e / SEGS, sg = e % SEGS;
      const int row = m0 + c * CH + rl, col = n0o + sg * EPS;
      if (e >= CH * SEGS || row >= p.M || col >= Nout) continue;
      char* gd = (char*)p.C + ((long)row * p.ldc + col) * OES;
      if (vec && col + EPS <= Nout) {
        if constexpr (EP == E_RESID) {
          if constexpr (PFX) *(f32x4*)gd = xpre[c * PER + i] + __builtin_bit_cast(f32x4, sv[i]);
          else *(f32x4*)gd = *(const f32x4*)gd + __builtin_bit_cast(f32x4, sv[i]);
        }
        else
          *(u32x4*)gd = sv[i];
      } else {                                      // ragged last segment or unaligned rows
        const char* ls = smem + rl * PITCH + sg * 16;
        for (int j = 0; j < EPS && col + j < Nout; ++j) {
          if constexpr (EP == E_RESID) ((float*)gd)[j] += ((const float*)ls)[j];
          else if constexpr (F32OUT) ((float*)gd)[j] = ((const float*)ls)[j];
          else ((T*)gd)[j] = ((const T*)ls)[j];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// dispatch

template <typename T, int BM, int BN, int WGM, int WGN, int QB>
static hipError_t run_epi(AMode am, Epi ep, const GemmParams& p, hipStream_t s, int ks = 1) {
  dim3 grid(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN), ks);
#define GG_L(AMv, EPv)                                                                   \
  if (am == AMv && ep == EPv) {                                                          \
    hipLaunchKernelGGL((k_gemm<T, BM, BN, WGM, WGN, AMv, QB, EPv>), grid, dim3(256), 0, s, p); \
    return hipGetLastError();                                                            \
  }
  if constexpr (QB != 0) {
    GG_L(A_PLAIN, E_SILU) GG_L(A_PLAIN, E_RESID) GG_L(A_DUAL, E_STORE) GG_L(A_PLAIN, E_GLU)
    GG_L(A_PLAIN, E_F32) GG_L(A_DUAL, E_F32)
  } else {
    GG_L(A_PLAIN, E_STORE) GG_L(A_PLAIN, E_SILU) GG_L(A_PLAIN, E_RESID) GG_L(A_DUAL, E_STORE)
    GG_L(A_PLAIN, E_GLU) GG_L(A_PLAIN, E_F32) GG_L(A_CONV, E_RELU_F32)
    if constexpr (sizeof(T) == 2) {
      GG_L(A_F32, E_F32) GG_L(A_CONV_F32, E_RELU) GG_L(A_DUAL, E_F32) GG_L(A_CONV, E_F32)
      GG_L(A_CONV_F32, E_F32)
    } else {
      GG_L(A_CONV, E_RELU)
    }
  }
#undef GG_L
  return hipErrorInvalidValue;
}

// Split-K: out = epilogue(sum over the KS slices of the fp32 partials + bias), the slices
// summed in order 0, 1, ... (deterministic). Thread = 4 consecutive output columns of one
// row; GLU reads the value columns and their gates 32 columns later (64-column groups). The
// slice count is a template argument so that every slice's load is issued before the first
// add (a loop over a run-time count waited for each load in turn); KS = 0 takes `slices` at
// run time (the fused FFN's f / 256 slices).
template <typename T, int EP, int KS>
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* __restrict__ part, int slices,
                                                       GemmParams p) {
  const int No = (EP == E_GLU) ? p.N / 2 : p.N;
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  const int qpr = No / 4;
  if (q >= (long)p.M * qpr) return;
  const int row = (int)(q / qpr), co = (int)(q % qpr) * 4;
  const long slice = (long)p.M * p.N;
  auto sum4 = [&](int col) {
    const float* src = part + (long)row * p.N + col;
    if constexpr (KS == 0) {
      const f32x4 v = p.bias ? *(const f32x4*)(p.bias + col) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 a = *(const f32x4*)src;
      for (int k = 1; k < slices; ++k) a += *(const f32x4*)(src + k * slice);
      return a + v;
    } else {
      f32x4 a[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) a[k] = *(const f32x4*)(src + k * slice);
      const f32x4 v = p.bias ? *(const f32x4*)(p.bias + col) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 1; k < KS; ++k) a[0] += a[k];
      return a[0] + v;
    }
  };
  if constexpr (EP == E_GLU) {
    const int c = (co / 32) * 64 + co % 32;              // value column; its gate is c + 32
    const f32x4 v = sum4(c), g = sum4(c + 32);
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = v[j] * sigmoidf_(g[j]);
    *(u32x2*)((T*)p.C + (long)row * p.ldc + co) = pack4<T>(o);
  } else {
    f32x4 v = sum4(co);
    if constexpr (EP == E_SILU) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = siluf_(v[j]);
    }
    if constexpr (EP == E_RELU || EP == E_RELU_F32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.f);
    }
    if constexpr (EP == E_STORE || EP == E_SILU || EP == E_RELU) {
      *(u32x2*)((T*)p.C + (long)row * p.ldc + co) = pack4<T>(v);
    } else if constexpr (EP == E_RESID) {
      f32x4* d = (f32x4*)((float*)p.C + (long)row * p.ldc + co);
      *d = *d + p.alpha * v;
    } else {
      *(f32x4*)((float*)p.C + (long)row * p.ldc + co) = v;
    }
  }
}

// Split-K for an fp32 output of any width (the CTC head: 34, 129 or 257 classes): one thread
// per output, the KS slices summed in order, then the bias.
template <int KS>
__global__ void __launch_bounds__(256) k_splitk_reduce_f32(const float* __restrict__ part, GemmParams p) {
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  if (q >= (long)p.M * p.N) return;
  const int row = (int)(q / p.N), col = (int)(q % p.N);
  const long slice = (long)p.M * p.N;
  float a[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) a[k] = part[q + k * slice];
  const float b = p.bias ? p.bias[col] : 0.f;
#pragma unroll
  for (int k = 1; k < KS; ++k) a[0] += a[k];
  ((float*)p.C)[(long)row * p.ldc + col] = a[0] + b;
}

// Residual GEMMs whose split-K sum the next kernel adds (the LayerNorm that reads x):
// launch_gemm's caller passes where to report the slices; the reduce launch is skipped. Only
// up to kDeferMaxSlices: the LayerNorm has one wave per row, and adding 8 slices there was
// slower than the reduce kernel's wider grid (a 20 s clip's FFN-down splits 8 ways).
static thread_local int* g_defer_ks = nullptr;
constexpr int kDeferMaxSlices = 4;

// Slices for a launch of `tiles` workgroups over K (k-tile KB), tiles * slices <= 256, slices
// of at least two k-tiles: at most 8, or kDeferMaxSlices when the next LayerNorm takes them;
// only when the tiles fill less than half the chip, or less than a quarter when K <= 1024
// and a reduce launch would follow (measured on 20 s clips: 1 clip 8.37k -> 9.34k audio-s/s,
// 2 clips 15.4k -> 16.7k, 4 and more unchanged; the quarter rule alone lost 3% at 4 clips,
// where the out-projection's 96 tiles gain from a split the LayerNorm finishes).
static int splitk_slices(const GemmParams& p, long tiles, int KB, Epi ep) {
  // (fp32 outputs of any width have a reduce of their own)
  const bool any_width = ep == E_F32;
  const bool deferred = ep == E_RESID && g_defer_ks;
  const long below = (deferred || p.K > 1024) ? 128 : 64;
  if (!p.part || tiles >= below || (!any_width && (p.N % 4 != 0 || p.ldc % 4 != 0)) ||
      (ep == E_GLU && p.N % 64 != 0))
    return 1;
  int ks = 1;
  const int kmax = deferred ? kDeferMaxSlices : 8;
  while (ks < kmax && tiles * ks * 2 <= 256 && p.K % (ks * 2 * KB) == 0 && p.K / (ks * 2) >= 2 * KB &&
         (long)p.M * p.N * ks * 2 <= p.part_cap)
    ks *= 2;
  return ks;
}

template <typename T>
static hipError_t run_splitk_reduce(Epi ep, int ks, const GemmParams& p, hipStream_t s) {
  if (ep == E_F32 && (p.N % 4 != 0 || p.ldc % 4 != 0)) {
    dim3 grid((unsigned)(((long)p.M * p.N + 255) / 256));
    if (ks == 2) hipLaunchKernelGGL((k_splitk_reduce_f32<2>), grid, dim3(256), 0, s, p.part, p);
    else if (ks == 4) hipLaunchKernelGGL((k_splitk_reduce_f32<4>), grid, dim3(256), 0, s, p.part, p);
    else if (ks == 8) hipLaunchKernelGGL((k_splitk_reduce_f32<8>), grid, dim3(256), 0, s, p.part, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int No = (ep == E_GLU) ? p.N / 2 : p.N;
  const long n = (long)p.M * (No / 4);
  dim3 grid((unsigned)((n + 255) / 256));
#define GG_R(EPv)                                                                                  \
  if (ep == EPv) {                                                                                 \
    if (ks == 2) hipLaunchKernelGGL((k_splitk_reduce<T, EPv, 2>), grid, dim3(256), 0, s, p.part, ks, p); \
    else if (ks == 4) hipLaunchKernelGGL((k_splitk_reduce<T, EPv, 4>), grid, dim3(256), 0, s, p.part, ks, p); \
    else if (ks == 8) hipLaunchKernelGGL((k_splitk_reduce<T, EPv, 8>), grid, dim3(256), 0, s, p.part, ks, p); \
    else hipLaunchKernelGGL((k_splitk_reduce<T, EPv, 0>), grid, dim3(256), 0, s, p.part, ks, p);          \
    return hipGetLastError();                                                                      \
  }
  if constexpr (sizeof(T) == 4) {
    GG_R(E_F32)                        // the fp32 CTC head of the 16-bit models
  } else {
    GG_R(E_STORE) GG_R(E_SILU) GG_R(E_RESID) GG_R(E_GLU) GG_R(E_F32) GG_R(E_RELU) GG_R(E_RELU_F32)
  }
#undef GG_R
  return hipErrorInvalidValue;
}

// The register-staged kernel (fp32, quantised weights, the implicit convs): with few output
// tiles the K sum is split as in the direct path (16-bit models, which bring a workspace).
static void tiles_geometry(Epi ep, const GemmParams& p, int& BM, int& BN) {
  if (p.N <= 512 && ep != E_GLU) { BM = 128; BN = 64; }
  else { BM = 128; BN = 128; }
}

template <typename T, int QB>
static hipError_t run_tiles(AMode am, Epi ep, const GemmParams& p, hipStream_t s) {
  int BM, BN;
  tiles_geometry(ep, p, BM, BN);
  const long tiles = (long)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  auto go = [&](Epi e, const GemmParams& q, int k) {
    if (BN == 64) return run_epi<T, 128, 64, 4, 1, QB>(am, e, q, s, k);
    return run_epi<T, 128, 128, 2, 2, QB>(am, e, q, s, k);
  };
  // 16-bit models (which bring a workspace); their fp32 CTC head too (fp32 models have none)
  if (sizeof(T) == 2 || ep == E_F32) {
    const int ks = splitk_slices(p, tiles, 64, ep);
    if (ks > 1) {
      GemmParams q = p;
      q.C = p.part;
      q.ldc = p.N;
      q.bias = nullptr;
      const hipError_t e = go(E_F32, q, ks);
      if (e != hipSuccess) return e;
      if (g_defer_ks && ep == E_RESID && ks <= kDeferMaxSlices) { *g_defer_ks = ks; return hipSuccess; }
      return run_splitk_reduce<T>(ep, ks, p, s);
    }
  }
  return go(ep, p, 1);
}

template <typename T, int BM, int BN, int WGM, int WGN, int S, int KB, int OCC>
static hipError_t run_dl(AMode am, Epi ep, const GemmParams& p, hipStream_t s) {
  constexpr bool GLU_OK = ((BN / WGN) / 32) % 2 == 0;     // value / gate block pairs per wave
  if (ep == E_GLU && !GLU_OK) return hipErrorInvalidValue;
  if (am == A_DUAL && p.nsplit % BN != 0) return hipErrorInvalidValue;
  if (am == A_CONV && (p.cin % KB != 0 || p.K != 5 * p.cin)) return hipErrorInvalidValue;
  const long tiles = (long)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const int ks = splitk_slices(p, tiles, KB, ep);
  dim3 blk(64 * WGM * WGN);
  if (ks > 1) {
    // each slice's raw sums into part, then the epilogue over their ordered sum
    GemmParams q = p;
    q.K = p.K / ks;
    q.C = p.part;
    q.ldc = p.N;
    q.bias = nullptr;
    dim3 grid((unsigned)tiles, ks);
    if (am == A_DUAL)
      hipLaunchKernelGGL((k_gemm_p<T, BM, BN, WGM, WGN, S, KB, A_DUAL, E_F32, OCC>), grid, blk, 0, s, q);
    else if (am == A_CONV)
      hipLaunchKernelGGL((k_gemm_p<T, BM, BN, WGM, WGN, S, KB, A_CONV, E_F32, OCC>), grid, blk, 0, s, q);
    else
      hipLaunchKernelGGL((k_gemm_p<T, BM, BN, WGM, WGN, S, KB, A_PLAIN, E_F32, OCC>), grid, blk, 0, s, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g_defer_ks && ep == E_RESID && ks <= kDeferMaxSlices) { *g_defer_ks = ks; return hipSuccess; }
    return run_splitk_reduce<T>(ep, ks, p, s);
  }
  dim3 grid((unsigned)tiles);
#define GG_DL(AMv, EPv)                                                                            \
  if (am == AMv && ep == EPv) {                                                                    \
    hipLaunchKernelGGL((k_gemm_p<T, BM, BN, WGM, WGN, S, KB, AMv, EPv, OCC>), grid, blk, 0, s, p); \
    return hipGetLastError();                                                                      \
  }
  GG_DL(A_PLAIN, E_STORE) GG_DL(A_PLAIN, E_SILU) GG_DL(A_PLAIN, E_RESID) GG_DL(A_PLAIN, E_F32)
  GG_DL(A_DUAL, E_STORE) GG_DL(A_CONV, E_RELU_F32) GG_DL(A_CONV, E_RELU)
  if constexpr (GLU_OK) { GG_DL(A_PLAIN, E_GLU) }
#undef GG_DL
  return hipErrorInvalidValue;
}

// Shapes of the direct-load pipeline, 8 waves each, chosen by timing inside the encode
// (operands arriving cold from the previous kernel) at 8207 rows:
//   single-source outputs wider than 1024 (FFN up, pointwise-1): 256 x 256 tiles, 64 x 128
//     per wave, 2 stages of 64 k (128 KiB LDS, one workgroup per CU);
//   the q/k/v projection (two A sources split at a 128-aligned column): 256 x 128 tiles,
//     3 stages of 32 k, two workgroups per CU;
//   outputs of at most 1024 columns with long K (FFN down): 256 x 128 tiles, 3 stages of
//     64 k (144 KiB, one workgroup per CU: half the barriers of 32-k tiles, 59.9 -> 54.5 us);
//   outputs of at most 1024 columns with K <= 1024 (out-proj, pointwise-2): 128 x 128
//     tiles, 2 stages of 64 k, two workgroups per CU.
// With few rows (a clip or two, a streaming window) the large tiles leave most of the chip
// idle: when one of them would give fewer than 128 tiles, the 128 x 128 shape is used
// (then split-K on top when even those are few).
static long tile_count(const GemmParams& p, int BM, int BN) {
  return (long)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
}
constexpr long kNarrowBelow = 160;
constexpr long kFewTiles = 256;     // at most one 128 x 128 workgroup per CU

// Direct-load kernel variants (the GemmShape ids): tile BM x BN, WGM x WGN waves, S stages of
// KB-element k-tiles, OCC workgroups per CU.
struct DlGeom { int id, BM, BN, KB; };
constexpr DlGeom kDlGeom[] = {
  {GEMM_DMA_256x256, 256, 256, 64},     // 8 waves, 2 stages, 1 per CU (128 KiB)
  {GEMM_DMA_256x128_K32, 256, 128, 32}, // 8 waves, 3 stages, 2 per CU
  {GEMM_DMA_256x128_K64, 256, 128, 64}, // 8 waves, 3 stages, 1 per CU (144 KiB)
  {GEMM_DMA_128x128, 128, 128, 64},     // 8 waves, 2 stages, 2 per CU
  {GEMM_DMA_256x192, 256, 192, 64},     // 8 waves (64 x 96 each), 2 stages, 1 per CU (112 KiB)
  {GEMM_DMA_256x128_W4, 256, 128, 32},  // 4 waves of 64 x 128, 3 stages, 2 per CU
  {GEMM_DMA_256x128_W4S, 256, 128, 32}, // 4 waves of 128 x 64, 3 stages, 2 per CU
  {GEMM_DMA_128x256, 128, 256, 32},     // 8 waves (64 x 64 each), 2 stages, 2 per CU
  {GEMM_DMA_128x128_S3, 128, 128, 64},  // 8 waves, 3 stages, 1 per CU (96 KiB): few tiles
};
static const DlGeom* dl_geom(int id) {
  for (const DlGeom& g : kDlGeom) if (g.id == id) return &g;
  return nullptr;
}

// A diagnostic override of the variant (gigaam_debug_gemm_role); 0: the encoder's choice.
static thread_local int g_force_variant = 0;

// The encoder's choice:
//   single-source outputs wider than 1024 (FFN up, pointwise-1): 256 x 256;
//   the q/k/v projection (two A sources split at a column multiple of the tile): 256 x 128,
//     3 stages of 32 k, two workgroups per CU (in isolation with hot operands 128 x 128 is
//     4% faster, 42.3 vs 44.3 us, but inside the encode, its operands arriving from the
//     LayerNorm, it is 8% slower: 51.5 vs 47.7 us);
//   outputs of at most 1024 columns with long K (FFN down): 256 x 128, 3 stages of 64 k
//     (half the barriers of 32-k tiles: 59.9 -> 54.5 us);
//   outputs of at most 1024 columns with K <= 1024 (out-proj, pointwise-2): 128 x 128.
// With few rows (a clip or two, a streaming window) the large tiles leave most of the chip
// idle: when one of them would give fewer than 160 workgroups even split, 128 x 128 is used
// (then split-K on top when even those are few). When the 128 x 128 workgroups (split or
// not) number at most one per CU, the 3-stage form runs instead: with one workgroup per CU
// nothing hides a k-tile's load latency but a deeper prefetch (a 20 s clip: 2.46 -> 2.40 ms).
static int dl_variant(AMode am, const GemmParams& p) {
  if (g_force_variant) return g_force_variant;
  int v = GEMM_DMA_128x128;
  if (p.N > 1024 && am != A_DUAL) v = GEMM_DMA_256x256;
  else if (p.N > 1024) v = GEMM_DMA_256x128_K32;
  else if (p.K > 1024) v = GEMM_DMA_256x128_K64;
  if (v != GEMM_DMA_128x128) {
    const DlGeom* g = dl_geom(v);
    const long t = tile_count(p, g->BM, g->BN);
    if (t * splitk_slices(p, t, g->KB, E_STORE) < kNarrowBelow) v = GEMM_DMA_128x128;
  }
  if (v == GEMM_DMA_128x128) {
    const long t = tile_count(p, 128, 128);
    if (t * splitk_slices(p, t, 64, E_STORE) <= kFewTiles) v = GEMM_DMA_128x128_S3;
  }
  return v;
}
// Geometry {BM, BN, KB} of the chosen variant, for the split-K planning:
static void dl_geometry(AMode am, const GemmParams& p, int& BM, int& BN, int& KB) {
  const DlGeom* g = dl_geom(dl_variant(am, p));
  BM = g->BM; BN = g->BN; KB = g->KB;
}

template <typename T>
static hipError_t run_dl_shape(AMode am, Epi ep, const GemmParams& p, hipStream_t s) {
  switch (dl_variant(am, p)) {
    case GEMM_DMA_256x256: return run_dl<T, 256, 256, 4, 2, 2, 64, 1>(am, ep, p, s);
    case GEMM_DMA_256x128_K32: return run_dl<T, 256, 128, 4, 2, 3, 32, 2>(am, ep, p, s);
    case GEMM_DMA_256x128_K64: return run_dl<T, 256, 128, 4, 2, 3, 64, 1>(am, ep, p, s);
    case GEMM_DMA_128x128: return run_dl<T, 128, 128, 4, 2, 2, 64, 2>(am, ep, p, s);
    case GEMM_DMA_256x192: return run_dl<T, 256, 192, 4, 2, 2, 64, 1>(am, ep, p, s);
    case GEMM_DMA_256x128_W4: return run_dl<T, 256, 128, 4, 1, 3, 32, 2>(am, ep, p, s);
    case GEMM_DMA_256x128_W4S: return run_dl<T, 256, 128, 2, 2, 3, 32, 2>(am, ep, p, s);
    case GEMM_DMA_128x256: return run_dl<T, 128, 256, 2, 4, 2, 32, 2>(am, ep, p, s);
    case GEMM_DMA_128x128_S3: return run_dl<T, 128, 128, 4, 2, 3, 64, 1>(am, ep, p, s);
  }
  return hipErrorInvalidValue;
}

static bool direct_path(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p) {
  if (dt == DT_F32 || qbits != 0 || p.K % 64 != 0) return false;
  if (am == A_CONV) return (ep == E_RELU_F32 || ep == E_RELU) && p.cin % 64 == 0 && p.K == 5 * p.cin;
  if (am == A_DUAL) return ep == E_STORE;
  return am == A_PLAIN &&
         (ep == E_STORE || ep == E_SILU || ep == E_RESID || ep == E_GLU || ep == E_F32);
}


// Quantised weights with many rows of A: the weights are expanded once per call to fp16
// rows [N][K] in the workspace (the fp16(q * s) values the register-staged kernel forms
// while staging, one rounding each), and the LDS-DMA pipeline runs on them. One thread
// per 16 weights of a row.
template <int QB>
__global__ void __launch_bounds__(256) k_dequant(GemmParams p, f16* __restrict__ out) {
  const int cpr = p.K / 16;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)p.N * cpr) return;
  const int n = (int)(e / cpr), k = (int)(e - (long)n * cpr) * 16;
  const uint8_t* q = (const uint8_t*)p.W + ((long)n * p.ldw + k) * QB / 8;
  u32x4 c;
  if constexpr (QB == 8) c = *(const u32x4*)q;
  else if constexpr (QB == 4) { const u32x2 v = *(const u32x2*)q; c = u32x4{v[0], v[1], 0, 0}; }
  else c = u32x4{((const uint32_t*)q)[0], ((const uint32_t*)q)[1], ((const uint32_t*)q)[2], 0};
  const float sc = (float)p.Wscale[(long)n * (p.K / 64) + k / 64];
  u32x4 lo, hi;
  dequant16<QB>(c, sc, lo, hi);
  u32x4* o = (u32x4*)(out + (long)n * p.K + k);
  o[0] = lo;
  o[1] = hi;
}

// rows of A from which expanding the weights first pays (the pipelined tiles then fill the
// chip; below it the register-staged kernel reads the packed weights directly)
constexpr int kDequantMinRows = 2048;

static bool dequant_first(int qbits, AMode am, Epi ep, const GemmParams& p) {
  if (qbits == 0 || !p.part || p.M < kDequantMinRows || p.K % 64 != 0) return false;
  if ((long)p.N * p.K * 2 > p.part_cap * 4) return false;
  return direct_path(DT_F16, 0, am, ep, p);
}

int gemm_split_slices(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p) {
  if (dt == DT_F32 && ep != E_F32) return 1;          // fp32 splits only an fp32-output product
  if (qbits != 0 && dequant_first(qbits, am, ep, p)) return 1;
  if (!direct_path(dt, qbits, am, ep, p)) {           // the register-staged kernel
    int BM, BN;
    tiles_geometry(ep, p, BM, BN);
    return splitk_slices(p, tile_count(p, BM, BN), 64, ep);
  }
  int BM, BN, KB;
  dl_geometry(am, p, BM, BN, KB);
  return splitk_slices(p, tile_count(p, BM, BN), KB, ep);
}

int gemm_shape_id(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p) {
  if (dt == DT_F32) {
    if (am == A_F32) am = A_PLAIN;
    if (am == A_CONV_F32) am = A_CONV;
  }
  bool direct = direct_path(dt, qbits, am, ep, p);
  if (qbits != 0) direct = dequant_first(qbits, am, ep, p);
  if (!direct) {
    int BM, BN;
    tiles_geometry(ep, p, BM, BN);
    return BN == 64 ? GEMM_REG_128x64 : GEMM_REG_128x128;
  }
  GemmParams q = p;
  if (qbits != 0) { q.part = nullptr; q.part_cap = 0; }   // the expanded weights fill it
  return dl_variant(am, q);
}

int gemm_force_variant(int id) {
  if (id != 0 && !dl_geom(id)) return -1;
  const int old = g_force_variant;
  g_force_variant = id;
  return old;
}

static hipError_t launch_gemm_impl(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p,
                                   hipStream_t s);

hipError_t launch_gemm(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p, hipStream_t s,
                       int* deferred_ks) {
  if (deferred_ks) *deferred_ks = 0;
  g_defer_ks = ep == E_RESID ? deferred_ks : nullptr;
  const hipError_t e = launch_gemm_impl(dt, qbits, am, ep, p, s);
  g_defer_ks = nullptr;
  return e;
}

static hipError_t launch_gemm_impl(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p,
                                   hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  if ((dt == DT_W8F16 || dt == DT_W6F16 || dt == DT_W4F16) && dequant_first(qbits, am, ep, p)) {
    f16* wd = (f16*)p.part;
    const long n = (long)p.N * (p.K / 16);
    dim3 grid((unsigned)((n + 255) / 256));
    if (qbits == 8) hipLaunchKernelGGL(k_dequant<8>, grid, dim3(256), 0, s, p, wd);
    else if (qbits == 6) hipLaunchKernelGGL(k_dequant<6>, grid, dim3(256), 0, s, p, wd);
    else if (qbits == 4) hipLaunchKernelGGL(k_dequant<4>, grid, dim3(256), 0, s, p, wd);
    else return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmParams q = p;
    q.W = wd;
    q.ldw = p.K;
    q.Wscale = nullptr;
    q.part = nullptr;                 // the workspace now holds the weights: no split
    q.part_cap = 0;
    return run_dl_shape<f16>(am, ep, q, s);
  }
  // fp32 A sources are native for the fp32 GEMM
  if (dt == DT_F32) {
    if (am == A_F32) am = A_PLAIN;
    if (am == A_CONV_F32) am = A_CONV;
  }
  const bool direct = direct_path(dt, qbits, am, ep, p);
  switch (dt) {
    case DT_F32: return run_tiles<float, 0>(am, ep, p, s);
    case DT_F16: return direct ? run_dl_shape<f16>(am, ep, p, s) : run_tiles<f16, 0>(am, ep, p, s);
    case DT_BF16: return direct ? run_dl_shape<bf16>(am, ep, p, s) : run_tiles<bf16, 0>(am, ep, p, s);
    case DT_W8F16:
    case DT_W6F16:
    case DT_W4F16:
      if (qbits == 8) return run_tiles<f16, 8>(am, ep, p, s);
      if (qbits == 6) return run_tiles<f16, 6>(am, ep, p, s);
      if (qbits == 4) return run_tiles<f16, 4>(am, ep, p, s);
      if (qbits != 0) return hipErrorInvalidValue;
      return direct ? run_dl_shape<f16>(am, ep, p, s) : run_tiles<f16, 0>(am, ep, p, s);
  }
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------------------
// Fused macaron FFN for few rows (a clip or two, a streaming window), a variant that never
// writes the hidden activations (measured against the two GEMMs; the encoder does not use
// it): a workgroup takes 32 WM rows and one 256-unit chunk of the hidden layer.
//   phase 1: h = SiLU(y W1[chunk]^T + b1[chunk]) -> LDS, rounded to T as the unfused path
//            rounds the hidden activations it stores;
//   phase 2: its share of the output, h W2[:, chunk]^T, accumulated over the 256 units in
//            fp32 and written as slice `chunk` of the partial sums [f/256][M][d].
// The split-K reduce then adds the f/256 slices in order with b2 and the residual half step
// (x += alpha (sum + b2)). Register-staged loads (the next k-tile is read into registers
// while the current one is consumed), 32 x 32 x 16 MFMAs, 8 waves as 2 (rows) x 4 (columns).
constexpr int kMlpChunk = 256;

// WM row groups of 32 (BM = 32 WM rows per workgroup), 8 / WM column groups
template <typename T, int D, int WM>
__global__ void __launch_bounds__(512) k_mlp(MlpArgs a) {
  constexpr int BM = 32 * WM, WN = 8 / WM;
  constexpr int NI1 = kMlpChunk / WN / 32;       // phase-1 32-column blocks per wave
  constexpr int NI2 = D / WN / 32;               // phase-2 32-column blocks per wave
  constexpr int LDR1 = 9;                        // phase 1: 64-k rows, 8 slots + pad
  constexpr int LDR2 = 5;                        // phase 2: 32-k rows, 4 slots + pad
  constexpr int HS = kMlpChunk / 8 + 1;          // h rows: 32 slots + pad
  constexpr int ST1 = (BM + kMlpChunk) * LDR1;   // slots per phase-1 stage
  constexpr int ST2 = D * LDR2;                  // slots of the phase-2 stage
  constexpr int SREG = 2 * ST1 > ST2 ? 2 * ST1 : ST2;
  static_assert(NI1 >= 1 && NI2 >= 1 && BM * 8 <= 512, "mlp tile");
  __shared__ u32x4 lds[SREG + BM * HS];
  u32x4* hs = lds + SREG;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 31, fk = lane >> 5;
  const int m0 = blockIdx.x * BM, c0 = blockIdx.y * kMlpChunk;
  const T* Y = (const T*)a.y;
  const T* W1 = (const T*)a.W1;
  const T* W2 = (const T*)a.W2;

  // ---- phase 1: [BM x 256] = y[BM x D] W1[256 x D]^T, k-tiles of 64
  const bool aload = tid < BM * 8;
  const int ar = tid >> 3, ac = tid & 7;
  const int arow = aload ? (m0 + ar < a.M ? m0 + ar : a.M - 1) : 0;
  const T* asrc = Y + (long)arow * D + ac * 8;
  const T* bsrc[4];
  int brow[4], bcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 512 * i;
    brow[i] = e >> 3;
    bcol[i] = e & 7;
    bsrc[i] = W1 + (long)(c0 + brow[i]) * D + bcol[i] * 8;
  }
  u32x4 ra, rb[4];
  auto load1 = [&](int kt) {
    if (aload) ra = *(const u32x4*)(asrc + kt * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *(const u32x4*)(bsrc[i] + kt * 64);
  };
  auto store1 = [&](int buf) {
    u32x4* st = lds + buf * ST1;
    if (aload) st[ar * LDR1 + ac] = ra;
#pragma unroll
    for (int i = 0; i < 4; ++i) st[(BM + brow[i]) * LDR1 + bcol[i]] = rb[i];
  };
  f32x16 acc1[NI1];
#pragma unroll
  for (int ni = 0; ni < NI1; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc1[ni][r] = 0.f;
  constexpr int KT1 = D / 64;
  load1(0);
  store1(0);
  __syncthreads();
  for (int kt = 0; kt < KT1; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT1) load1(kt + 1);
    const u32x4* st = lds + cur * ST1;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const u32x4 af = st[(wm * 32 + fr) * LDR1 + kc * 2 + fk];
#pragma unroll
      for (int ni = 0; ni < NI1; ++ni)
        Mma<T>::run(acc1[ni], af, st[(BM + wn * NI1 * 32 + ni * 32 + fr) * LDR1 + kc * 2 + fk]);
    }
    if (kt + 1 < KT1) store1(cur ^ 1);
    __syncthreads();
  }
  // h = SiLU(acc + b1) in T, into LDS rows [BM][256]
  {
    T* h = (T*)hs;
#pragma unroll
    for (int ni = 0; ni < NI1; ++ni) {
      const int col = wn * NI1 * 32 + ni * 32 + fr;
      const float bb = a.b1 ? a.b1[c0 + col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
        h[row * HS * 8 + col] = from_f32<T>(siluf_(acc1[ni][r] + bb));
      }
    }
  }

  // ---- phase 2: [BM x D] = h[BM x 256] W2[D x chunk]^T, k-tiles of 32, one LDS stage
  constexpr int CH2 = D * 4 / 512;               // 16-byte chunks per thread per k-tile
  const T* wsrc[CH2];
  int wrow[CH2], wcol[CH2];
#pragma unroll
  for (int i = 0; i < CH2; ++i) {
    const int e = tid + 512 * i;
    wrow[i] = e >> 2;
    wcol[i] = e & 3;
    wsrc[i] = W2 + (long)wrow[i] * a.f + c0 + wcol[i] * 8;
  }
  u32x4 rw[CH2];
  auto load2 = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH2; ++i) rw[i] = *(const u32x4*)(wsrc[i] + kt * 32);
  };
  f32x16 acc2[NI2];
#pragma unroll
  for (int ni = 0; ni < NI2; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[ni][r] = 0.f;
  constexpr int KT2 = kMlpChunk / 32;
  load2(0);
  for (int kt = 0; kt < KT2; ++kt) {
    // the stage is free (the previous k-tile consumed; h written before the first)
#pragma unroll
    for (int i = 0; i < CH2; ++i) lds[wrow[i] * LDR2 + wcol[i]] = rw[i];
    __syncthreads();
    if (kt + 1 < KT2) load2(kt + 1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 af = hs[(wm * 32 + fr) * HS + kt * 4 + kc * 2 + fk];
#pragma unroll
      for (int ni = 0; ni < NI2; ++ni)
        Mma<T>::run(acc2[ni], af, lds[(wn * NI2 * 32 + ni * 32 + fr) * LDR2 + kc * 2 + fk]);
    }
    __syncthreads();
  }
  GemmParams q = {};
  q.M = a.M; q.N = D; q.C = a.part + blockIdx.y * (long)a.M * D; q.ldc = D; q.bias = nullptr;
  epilogue<T, 1, NI2, E_F32>(q, (f32x16(&)[1][NI2])acc2, m0 + wm * 32, wn * NI2 * 32, 0, lane);
}

bool mlp_fusable(DType dt, int qbits, int M, int d, int f, long part_cap) {
  return (dt == DT_F16 || dt == DT_BF16) && qbits == 0 && M >= 1 && M <= kMlpMaxRows &&
         (d == 768 || d == 1024) && f % kMlpChunk == 0 &&
         (long)(f / kMlpChunk) * M * d <= part_cap;
}

constexpr int kMlpWM = 1;                  // row groups of 32 per workgroup

hipError_t launch_mlp(DType dt, const MlpArgs& a, const float* b2, float alpha, float* x,
                      hipStream_t s) {
  dim3 grid((a.M + 32 * kMlpWM - 1) / (32 * kMlpWM), a.f / kMlpChunk), blk(512);
  if (dt == DT_F16) {
    if (a.d == 768) hipLaunchKernelGGL((k_mlp<f16, 768, kMlpWM>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_mlp<f16, 1024, kMlpWM>), grid, blk, 0, s, a);
  } else {
    if (a.d == 768) hipLaunchKernelGGL((k_mlp<bf16, 768, kMlpWM>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_mlp<bf16, 1024, kMlpWM>), grid, blk, 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams r;
  std::memset(&r, 0, sizeof r);
  r.M = a.M; r.N = a.d; r.C = x; r.ldc = a.d; r.bias = b2; r.alpha = alpha; r.part = a.part;
  return dt == DT_F16 ? run_splitk_reduce<f16>(E_RESID, a.f / kMlpChunk, r, s)
                      : run_splitk_reduce<bf16>(E_RESID, a.f / kMlpChunk, r, s);
}

}  // namespace gg
