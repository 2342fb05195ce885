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
