// RNNT greedy decoding for gfx950: one workgroup per clip runs the whole sequential
// loop (frames x emissions) on chip, with the prediction-network state and the joint
// activations in LDS.
//
// "GigaAM on MLX ...", section "What we're porting": the head is a single-layer LSTM of
// size 320 plus a joint; "GigaAM v3 MLX" card, "Long-form stage breakdown": greedy
// decoding is the sequential bottleneck, the joint its largest part. Per step:
//   joint   z = relu(fenc[t] + fpred);  logits = W_out z + b_out;  k = argmax
//   emit    gates = gemb[k] + W_hh h;  (c, h) <- LSTM cell;  fpred = W_pred h + b_pred
// fenc = W_enc e_t + b_enc for every frame and gemb = W_ih embed + b_ih + b_hh for every
// symbol come from two GEMMs before this kernel.
//
// Matrix-vector products read their matrix transposed ([rows][cols], cols padded to a
// multiple of 8), so each thread streams 16-byte column groups; the rows are split over
// as many threads as the 1024 allow, so that many loads are in flight per CU (an
// emission step is bound by how fast one CU pulls W_hh from L2). Every wave takes the
// argmax itself, so a decision costs two workgroup barriers.
#include "kernels.h"

#include <algorithm>

namespace gg {

template <typename T> struct Vec;                 // 16 bytes of T as floats
template <> struct Vec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const void* p, float* out) {
    const f32x4 v = *(const f32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = v[i];
  }
};
template <> struct Vec<f16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const void* p, float* out) {
    const f16x8 v = *(const f16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
  }
};
template <> struct Vec<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const void* p, float* out) {
    const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
  }
};

constexpr int RN_T = 1024;         // threads per workgroup

// y[col] = init[col] + sum_{r < rows} M[r][col] * x[r] for col < cols; M is T
// [rows][ldm] (ldm a multiple of Vec::N), x and y in LDS. Two ways to split the rows:
//  - matvec_lanes: over S consecutive lanes of one wave per 16-byte column group (S a
//    power of two, as large as the threads allow with at least 4 rows per lane), the
//    partial sums meeting through a butterfly of lane shuffles; for narrow matrices
//    (the joint's output layer), where it saves a barrier and a long reduction;
//  - matvec_slices: consecutive lanes take consecutive column groups (1 KiB per wave
//    load) and the rows are cut into slices of at least 8, partial sums reduced through
//    LDS (part: RN_T * Vec::N floats); for the wide W_hh and W_pred.
// Both sum in a fixed order and end with a barrier.
template <typename T>
__device__ void matvec_lanes(const T* __restrict__ M, int ldm, int rows, int cols,
                             const float* x, const float* __restrict__ init, float* y) {
  constexpr int V = Vec<T>::N;
  const int tid = threadIdx.x;
  const int groups = (cols + V - 1) / V;
  int S = 1;
  while (S < 64 && 2 * S * groups <= RN_T && 2 * S * 4 <= rows) S *= 2;
  const int per = (rows + S - 1) / S;
  const int sl = tid & (S - 1);
  for (int gi = tid / S; gi < groups; gi += RN_T / S) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const int r0 = sl * per, r1 = min(rows, r0 + per);
    const T* mp = M + gi * V;
#pragma unroll 8
    for (int r = r0; r < r1; ++r) {
      float w[V];
      Vec<T>::load(mp + (long)r * ldm, w);
      const float xr = x[r];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i], xr, acc[i]);
    }
    // butterfly over the S lanes of the group (same order as lane-xor shuffles)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      switch (S) {
        case 64: acc[i] = group_sum<64>(acc[i]); break;
        case 32: acc[i] = group_sum<32>(acc[i]); break;
        case 16: acc[i] = group_sum<16>(acc[i]); break;
        case 8: acc[i] = group_sum<8>(acc[i]); break;
        case 4: acc[i] = group_sum<4>(acc[i]); break;
        case 2: acc[i] = group_sum<2>(acc[i]); break;
        default: break;
      }
    }
    if (sl == 0)
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (gi * V + i < cols) y[gi * V + i] = acc[i] + (init ? init[gi * V + i] : 0.f);
  }
  __syncthreads();
}

template <typename T>
__device__ void matvec_slices(const T* __restrict__ M, int ldm, int rows, int cols,
                              const float* x, const float* __restrict__ init, float* y,
                              float* part) {
  constexpr int V = Vec<T>::N;
  const int tid = threadIdx.x;
  const int groups = (cols + V - 1) / V;
  const int slices = max(1, min(RN_T / groups, rows / 8));
  const int per = (rows + slices - 1) / slices;
  for (int e = tid; e < groups * slices; e += RN_T) {
    const int gi = e % groups, sl = e / groups;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const int r0 = sl * per, r1 = min(rows, r0 + per);
    const T* mp = M + gi * V;
#pragma unroll 8
    for (int r = r0; r < r1; ++r) {
      float w[V];
      Vec<T>::load(mp + (long)r * ldm, w);
      const float xr = x[r];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i], xr, acc[i]);
    }
    if (slices == 1) {
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (gi * V + i < cols) y[gi * V + i] = acc[i] + (init ? init[gi * V + i] : 0.f);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) part[sl * groups * V + gi * V + i] = acc[i];
    }
  }
  if (slices > 1) {
    __syncthreads();
    for (int col = tid; col < cols; col += RN_T) {
      float s = init ? init[col] : 0.f;
      for (int k = 0; k < slices; ++k) s += part[k * groups * V + col];
      y[col] = s;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <typename T>
__global__ void __launch_bounds__(RN_T) k_rnnt(RnntParams p) {
  extern __shared__ float sm[];
  const int P = p.P, J = p.J, C = p.C, blank = C - 1;
  float* h = sm;
  float* c = h + P;
  float* fpred = c + P;
  float* z = fpred + J;
  float* gates = z + J;
  float* logit = gates + 4 * P;
  float* part = logit + p.Cp;                         // RN_T * Vec::N floats
  T* swo = (T*)(part + RN_T * Vec<T>::N);             // W_out^T in LDS when it fits

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int U = p.frames[b];
  int* tok = p.tokens + (long)b * p.max_tokens;
  int* tfr = p.tframes ? p.tframes + (long)b * p.max_tokens : nullptr;
  const T* whhT = (const T*)p.whhT;
  const T* wpT = (const T*)p.wpT;
  const T* woT = (const T*)p.woT;
  if (p.wo_lds) {                                     // the joint's output matrix is read
    const int n16 = J * p.Cp * (int)sizeof(T) / 16;   // every decision: keep it on chip
    for (int i = tid; i < n16; i += RN_T) ((f32x4*)swo)[i] = ((const f32x4*)woT)[i];
    woT = swo;
  }

  for (int i = tid; i < P; i += RN_T) { h[i] = 0.f; c[i] = 0.f; }
  __syncthreads();

  // prediction network on symbol k: gates, LSTM cell, then the joint's prediction half
  auto predict = [&](int k) {
    matvec_slices<T>(whhT, 4 * P, P, 4 * P, h, p.gemb + (long)k * 4 * P, gates, part);
    for (int u = tid; u < P; u += RN_T) {
      const float ig = sigm(gates[u]), fg = sigm(gates[P + u]);
      const float gg = tanhf(gates[2 * P + u]), og = sigm(gates[3 * P + u]);
      const float cn = fg * c[u] + ig * gg;
      c[u] = cn;
      h[u] = og * tanhf(cn);
    }
    __syncthreads();
    matvec_slices<T>(wpT, J, P, J, h, p.bp, fpred, part);
  };

  predict(blank);
  int n = 0;
  const float* fenc = p.fenc + (long)b * p.stride * J;
  float fe_next = tid < J ? fenc[tid] : 0.f;          // frame t's row, loaded a frame ahead
  for (int t = 0; t < U; ++t) {
    const float fe = fe_next;
    if (t + 1 < U && tid < J) fe_next = fenc[(long)(t + 1) * J + tid];
    for (int sym = 0; sym < p.max_symbols; ++sym) {
      if (tid < J) z[tid] = fmaxf(fe + fpred[tid], 0.f);
      __syncthreads();
      matvec_lanes<T>(woT, p.Cp, J, C, z, p.bo, logit);
      // argmax, lowest index on ties (NaN never wins), taken by every wave on its own
      float best = -INFINITY;
      int bi = C;
      for (int v = lane; v < C; v += 64) {
        const float a = logit[v];
        if (a > best) { best = a; bi = v; }
      }
      wave_argmax(best, bi);
      const int k = bi >= C ? blank : bi;             // all logits NaN: treat as blank
      if (k == blank) break;
      if (tid == 0) {
        if (n < p.max_tokens) { tok[n] = k; if (tfr) tfr[n] = t; }
      }
      ++n;
      predict(k);
    }
  }
  if (n > p.max_tokens) n = p.max_tokens;
  for (int i = n + tid; i < p.max_tokens; i += RN_T) {
    tok[i] = -1;
    if (tfr) tfr[i] = -1;
  }
  if (tid == 0) p.ntok[b] = n;
}

// ---------------------------------------------------------------------------------------
// Clustered decoding: G workgroups per clip, launched cooperatively (all co-resident), each
// holding a 1/G slice of the prediction network and of the joint in LDS, so that no
// emission streams W_hh through one CU. Member g owns LSTM units [g P/G, (g+1) P/G) (their
// four gate rows of W_hh), joint rows [g J/G, (g+1) J/G) (W_pred rows, the matching
// columns of W_out). Per decision the members exchange their partial logits (W_out over
// their joint slice); per emission their slices of the new h. Every member sums the
// partials in member order and takes the same argmax, so all follow the same path.
//
// Exchange: each value travels as one 64-bit word (float bits | sequence number << 32),
// so a reader takes a value exactly when its sequence number is the step it waits for,
// with no fence and no separate flag (see Xch for the cache paths). Slots alternate by the
// step's parity: a member can be at most one step ahead of another (a step ends only when
// every member's value of that step has been read), so a slot is never rewritten before
// all members have read it. The buffers are zeroed before the launch (sequence numbers
// start at 1). The members of a clip are placed on one XCD (workgroups 8 k + x run on XCD
// x) and check it at start. Polls are bounded: a member that waits longer than the limit
// marks its clip failed (n_tokens < 0: -1, -2, -3 for the XCD, h and logits exchanges,
// 16 less on the L2 path) and leaves, and the others in turn.

constexpr int RC_T = 256;          // threads per cluster member

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p) { return to_f32(*p); }

// y[r] = init[r] + sum_k W[r][k] x[k] for r < R (W row-major [R][K] in LDS, K % 64 == 0);
// 8 consecutive lanes per row, each summing K/8 columns, then a fixed-order butterfly
template <typename T>
__device__ void mv_rows8(const T* W, int R, int K, const float* x, const float* init, float* y) {
  constexpr int V = Vec<T>::N;
  const int tid = threadIdx.x, sub = tid & 7, rr = tid >> 3;
  const int KC = K / 8;
  for (int r0 = 0; r0 < R; r0 += RC_T / 8) {
    const int r = r0 + rr;
    float acc = 0.f;
    if (r < R) {
      const T* wr = W + (long)r * K + sub * KC;
      const float* xr = x + sub * KC;
      for (int k = 0; k < KC; k += V) {
        float w[V];
        Vec<T>::load(wr + k, w);
#pragma unroll
        for (int i = 0; i < V; ++i) acc = fmaf(w[i], xr[k + i], acc);
      }
    }
    acc = group_sum<8>(acc);
    if (sub == 0 && r < R) y[r] = acc + (init ? init[r] : 0.f);
  }
}

// One exchange word: float bits | sequence number << 32. Two ways to move it:
//  - agent scope: relaxed agent-scope atomics (coherent across XCDs, through memory);
//  - one XCD's L2, taken when all members of a cluster run on one XCD: stores with sc0 (the
//    L1 is write-through: the word lands in the L2 that every CU of one XCD shares) and
//    loads with sc1 (they miss the CU's L1 and read that L2). Measured on the 6-clip test
//    head: 15.9 ms against 19.9 ms at agent scope; a load with sc0 kept returning a stale
//    L1 copy even with the L1 invalidated between polls.
// A 64-bit aligned access is single-copy atomic either way.
struct Xch {
  unsigned long long* base;
  __amdgpu_buffer_rsrc_t rsrc;
  bool l2;
  __device__ __forceinline__ void put(long i, float v, unsigned seq) const {
    const unsigned long long w = ((unsigned long long)seq << 32) | __float_as_uint(v);
    if (l2) {
      typedef unsigned int u2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, w), rsrc, (int)(i * 8), 0, 1);
    } else {
      __hip_atomic_store(base + i, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __device__ __forceinline__ bool get(long i, unsigned seq, int limit, float& v) const {
    for (int k = 0; k < limit; ++k) {
      const unsigned long long w =
          l2 ? __builtin_bit_cast(unsigned long long,
                                  __builtin_amdgcn_raw_buffer_load_b64(rsrc, (int)(i * 8), 0, 16))
             : __hip_atomic_load(base + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((unsigned)(w >> 32) == seq) {
        v = __uint_as_float((unsigned)w);
        return true;
      }
      __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");
    }
    return false;
  }
};

// floats before the member's weight slices in LDS (a multiple of 4: 16-byte alignment)
__host__ __device__ __forceinline__ int rnnt_cl_floats(int P, int UG, int JG, int Cp, int G) {
  return (P + 5 * UG + 2 * JG + Cp + 4 + G * Cp + 3) / 4 * 4;
}

template <typename T>
__global__ void __launch_bounds__(RC_T) k_rnnt_cl(RnntParams p, RnntCluster q) {
  extern __shared__ float sm[];
  const int G = q.G, P = p.P, J = p.J, C = p.C, Cp = p.Cp, blank = C - 1;
  const int UG = P / G, JG = J / G;
  // workgroup i runs on XCD i % 8: the members of clip b are workgroups
  // 8 (G (b / 8) + g) + b % 8, g < G, all on one XCD (checked below)
  const int x8 = (int)(blockIdx.x % 8), r8 = (int)(blockIdx.x / 8);
  const int b = (r8 / G) * 8 + x8, g = r8 % G;
  if (b >= q.batch) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ug0 = g * UG, jg0 = g * JG;
  // LDS: h[P] c[UG] gates[4UG] fpred[JG] z[JG] logit[Cp] fail; then W_hh rows [4UG][P],
  // W_pred rows [JG][P], W_out columns [JG][Cp] (when they fit)
  float* h = sm;
  float* cs = h + P;
  float* gates = cs + UG;
  float* fpred = gates + 4 * UG;
  float* z = fpred + JG;
  float* logit = z + JG;
  int* fail = (int*)(logit + Cp);
  float* parts = (float*)(fail + 4);                  // [G][Cp] every member's partial logits
  T* whh = (T*)(sm + rnnt_cl_floats(P, UG, JG, Cp, G));   // 16-byte aligned
  T* wp = whh + (long)4 * UG * P;
  T* wo = q.wo_lds ? wp + (long)JG * P : (T*)p.woT + (long)jg0 * Cp;

  const T* whhT = (const T*)p.whhT;
  const T* wpT = (const T*)p.wpT;
  for (int i = tid; i < 4 * UG * P; i += RC_T) {   // consecutive threads: consecutive units
    const int k = i / (4 * UG), r = i - k * 4 * UG, gq = r / UG, u = r - gq * UG;
    whh[(long)r * P + k] = whhT[(long)k * 4 * P + gq * P + ug0 + u];
  }
  for (int i = tid; i < JG * P; i += RC_T) {
    const int k = i / JG, jj = i - k * JG;
    wp[(long)jj * P + k] = wpT[(long)k * J + jg0 + jj];
  }
  if (q.wo_lds)
    for (int i = tid; i < JG * Cp; i += RC_T) wo[i] = ((const T*)p.woT)[(long)jg0 * Cp + i];
  for (int i = tid; i < P; i += RC_T) h[i] = 0.f;
  for (int i = tid; i < UG; i += RC_T) cs[i] = 0.f;
  if (tid == 0) { fail[0] = 0; fail[1] = 1; }
  __syncthreads();

  // which XCD each member runs on: exchanged once at agent scope; the cluster uses the
  // L2 path only if all members share one
  Xch X;
  X.base = q.xl;
  X.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)q.xl, 0, q.xbytes, 0x00020000);
  X.l2 = false;
  {
    const long xc = q.xc - q.xl + (long)b * G;
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 15;   // HW_REG_XCC_ID
    if (tid == 0) X.put(xc + g, (float)xcc, 1);
    for (int m = tid; m < G; m += RC_T) {
      float v;
      if (!X.get(xc + m, 1, q.spin_limit, v)) fail[0] = 1;   // stage 1: the XCD exchange
      else if (v != (float)xcc) fail[1] = 0;
    }
    __syncthreads();
    X.l2 = fail[1] != 0;
  }

  const int U = p.frames[b];
  int* tok = p.tokens + (long)b * p.max_tokens;
  int* tfr = p.tframes ? p.tframes + (long)b * p.max_tokens : nullptr;
  const long xl = (long)b * 2 * G * Cp;               // word offsets from q.xl
  const long xh = (q.xh - q.xl) + (long)b * 2 * P;
  unsigned dseq = 0, eseq = 0;

  // prediction network on symbol k: this member's gate rows, its units' LSTM cell, the
  // exchange of h, then this member's rows of the joint's prediction half
  auto predict = [&](int k) -> bool {
    ++eseq;
    const float* ge = p.gemb + (long)k * 4 * P;
    for (int r = tid; r < 4 * UG; r += RC_T) {     // gemb entries of this member's gate rows
      const int gq = r / UG;
      gates[r] = ge[gq * P + ug0 + r - gq * UG];
    }
    __syncthreads();
    mv_rows8<T>(whh, 4 * UG, P, h, gates, gates);
    __syncthreads();
    const long hs = xh + (eseq & 1) * P;
    for (int u = tid; u < UG; u += RC_T) {
      const float ig = sigm(gates[u]), fg = sigm(gates[UG + u]);
      const float gg = tanhf(gates[2 * UG + u]), og = sigm(gates[3 * UG + u]);
      const float cn = fg * cs[u] + ig * gg;
      cs[u] = cn;
      X.put(hs + ug0 + u, og * tanhf(cn), eseq);
    }
    __syncthreads();                                  // every read of the old h is done
    for (int i = tid; i < P; i += RC_T) {
      float v;
      if (X.get(hs + i, eseq, q.spin_limit, v)) h[i] = v;
      else *fail = 2;                                 // stage 2: the h exchange
    }
    __syncthreads();
    if (*fail) return false;
    mv_rows8<T>(wp, JG, P, h, p.bp + jg0, fpred);
    __syncthreads();
    return true;
  };

  bool ok = fail[0] == 0 && predict(blank);
  int n = 0;
  const float* fenc = p.fenc + (long)b * p.stride * J + jg0;
  for (int t = 0; ok && t < U; ++t) {
    for (int sym = 0; sym < p.max_symbols; ++sym) {
      ++dseq;
      if (tid < JG) z[tid] = fmaxf(fenc[(long)t * J + tid] + fpred[tid], 0.f);
      __syncthreads();
      const long ls = xl + (dseq & 1) * G * Cp;
      for (int v = tid; v < C; v += RC_T) {           // this member's partial logits
        float acc = 0.f;
        for (int jj = 0; jj < JG; ++jj) acc = fmaf(ld_elem(wo + (long)jj * Cp + v), z[jj], acc);
        X.put(ls + g * Cp + v, acc, dseq);
      }
      for (int e = tid; e < G * C; e += RC_T) {       // every member's, gathered in parallel
        const int m = e / C, v = e - m * C;
        float part = 0.f;
        if (!X.get(ls + m * Cp + v, dseq, q.spin_limit, part)) *fail = 3;   // stage 3: logits
        parts[m * Cp + v] = part;
      }
      __syncthreads();
      for (int v = tid; v < C; v += RC_T) {           // summed in member order
        float sum = p.bo[v];
        for (int m = 0; m < G; ++m) sum += parts[m * Cp + v];
        logit[v] = sum;
      }
      __syncthreads();
      if (*fail) { ok = false; break; }
      float best = -INFINITY;
      int bi = C;
      for (int v = lane; v < C; v += 64) {
        const float a = logit[v];
        if (a > best) { best = a; bi = v; }
      }
      wave_argmax(best, bi);
      const int k = bi >= C ? blank : bi;             // all logits NaN: treat as blank
      __syncthreads();                                 // logit reads done before the next step
      if (k == blank) break;
      if (g == 0 && tid == 0 && n < p.max_tokens) { tok[n] = k; if (tfr) tfr[n] = t; }
      ++n;
      if (!predict(k)) { ok = false; break; }
    }
  }
  if (g != 0) return;
  if (!ok) {
    if (tid == 0) p.ntok[b] = -fail[0] - 16 * (int)X.l2;
    return;
  }
  if (n > p.max_tokens) n = p.max_tokens;
  for (int i = n + tid; i < p.max_tokens; i += RC_T) {
    tok[i] = -1;
    if (tfr) tfr[i] = -1;
  }
  if (tid == 0) p.ntok[b] = n;
}

size_t rnnt_cl_lds_bytes(DType dt, int P, int J, int Cp, int G, bool wo_lds) {
  const size_t es = dt == DT_F32 ? 4 : 2;
  const size_t UG = P / G, JG = J / G;
  return (size_t)rnnt_cl_floats(P, (int)UG, (int)JG, Cp, G) * 4 +
         (4 * UG * P + JG * P + (wo_lds ? JG * Cp : 0)) * es;
}

// workgroups of a clustered launch: clips in groups of 8 (one per XCD), G members each
long rnnt_cl_grid(int batch, int G) { return (long)(batch + 7) / 8 * 8 * G; }

__global__ void __launch_bounds__(256) k_zero_u64(unsigned long long* a, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += stride) a[i] = 0ull;
}

hipError_t launch_rnnt_cluster(DType dt, const RnntParams& p, const RnntCluster& q, int batch,
                               hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const long nx = q.xbytes / 8;                                  // xl, xh, xc: contiguous
  hipLaunchKernelGGL(k_zero_u64, dim3((unsigned)std::min<long>((nx + 255) / 256, 1024)), dim3(256), 0, s,
                     q.xl, nx);
  const size_t lds = rnnt_cl_lds_bytes(dt, p.P, p.J, p.Cp, q.G, q.wo_lds != 0);
  RnntParams pp = p;
  RnntCluster qq = q;
  void* args[] = {&pp, &qq};
  const void* fn = dt == DT_F32 ? (const void*)k_rnnt_cl<float>
                   : dt == DT_BF16 ? (const void*)k_rnnt_cl<bf16> : (const void*)k_rnnt_cl<f16>;
  return hipLaunchCooperativeKernel(fn, dim3(rnnt_cl_grid(batch, q.G)), dim3(RC_T), args, (unsigned)lds, s);
}

int rnnt_cluster_size(DType dt, int P, int J, int Cp, int batch, int max_g) {
  int dev = 0, ncu = 0, coop = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return 1;
  for (int G = 64; G >= 2; G /= 2) {
    if (G > max_g || P % G || J % G) continue;
    if (rnnt_cl_lds_bytes(dt, P, J, Cp, G, false) > 160 * 1024) continue;
    const void* fn = dt == DT_F32 ? (const void*)k_rnnt_cl<float>
                     : dt == DT_BF16 ? (const void*)k_rnnt_cl<bf16> : (const void*)k_rnnt_cl<f16>;
    const bool wo = rnnt_cl_lds_bytes(dt, P, J, Cp, G, true) <= 160 * 1024;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, RC_T, rnnt_cl_lds_bytes(dt, P, J, Cp, G, wo)) !=
            hipSuccess || (long)per_cu * ncu < rnnt_cl_grid(batch, G))
      continue;
    return G;
  }
  return 1;
}

size_t rnnt_lds_bytes(DType dt, int P, int J, int Cp, bool wo_lds) {
  const size_t es = dt == DT_F32 ? 4 : 2;
  const int V = dt == DT_F32 ? 4 : 8;
  return (size_t)(2 * P + 2 * J + 4 * P + Cp + RN_T * V) * 4 + (wo_lds ? J * Cp * es : 0);
}

hipError_t launch_rnnt_decode(DType dt, const RnntParams& p, int batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const size_t lds = rnnt_lds_bytes(dt, p.P, p.J, p.Cp, p.wo_lds != 0);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (dt == DT_F32)
    hipLaunchKernelGGL(k_rnnt<float>, dim3(batch), dim3(RN_T), lds, s, p);
  else if (dt == DT_BF16)
    hipLaunchKernelGGL(k_rnnt<bf16>, dim3(batch), dim3(RN_T), lds, s, p);
  else
    hipLaunchKernelGGL(k_rnnt<f16>, dim3(batch), dim3(RN_T), lds, s, p);
  return hipGetLastError();
}

}  // namespace gg
