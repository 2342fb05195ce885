// RNNT greedy decoding for gfx950: one workgroup per clip runs the whole sequential
// loop (frames x emissions) on chip, with the prediction-network state, the joint
// activations and all partial sums in LDS.
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
// multiple of 8), so each thread streams 16-byte column groups; when there are fewer
// column groups than threads the rows are split into slices whose partial sums are
// reduced through LDS.
#include "kernels.h"

namespace gg {

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

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

// y[col] = init[col] + sum_{r < rows} M[r][col] * x[r] for col < cols; M is T
// [rows][ldm] (ldm a multiple of Vec::N), x and y in LDS, part = LDS scratch of
// 256 * Vec::N floats. Ends with a barrier.
template <typename T>
__device__ void matvec(const T* __restrict__ M, int ldm, int rows, int cols, const float* x,
                       const float* __restrict__ init, float* y, float* part) {
  constexpr int V = Vec<T>::N;
  const int tid = threadIdx.x;
  const int groups = (cols + V - 1) / V;
  if (groups >= 256) {                               // one column group per thread
    for (int gi = tid; gi < groups; gi += 256) {
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      const T* mp = M + gi * V;
#pragma unroll 4
      for (int r = 0; r < rows; ++r) {
        float w[V];
        Vec<T>::load(mp + (long)r * ldm, w);
        const float xr = x[r];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i], xr, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (gi * V + i < cols) y[gi * V + i] = acc[i] + (init ? init[gi * V + i] : 0.f);
    }
    __syncthreads();
    return;
  }
  const int slices = 256 / groups;                   // rows split into this many slices
  const int per = (rows + slices - 1) / slices;
  const int gi = tid % groups, sl = tid / groups;
  if (sl < slices) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const int r0 = sl * per, r1 = min(rows, r0 + per);
    const T* mp = M + gi * V;
    for (int r = r0; r < r1; ++r) {
      float w[V];
      Vec<T>::load(mp + (long)r * ldm, w);
      const float xr = x[r];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w[i], xr, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) part[sl * groups * V + gi * V + i] = acc[i];
  }
  __syncthreads();
  for (int col = tid; col < cols; col += 256) {
    float s = init ? init[col] : 0.f;
    for (int k = 0; k < slices; ++k) s += part[k * groups * V + col];   // fixed order
    y[col] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <typename T>
__global__ void __launch_bounds__(256) k_rnnt(RnntParams p) {
  extern __shared__ float sm[];
  constexpr int V = Vec<T>::N;
  const int P = p.P, J = p.J, C = p.C, blank = C - 1;
  float* h = sm;
  float* c = h + P;
  float* fpred = c + P;
  float* z = fpred + J;
  float* gates = z + J;
  float* logit = gates + 4 * P;
  float* part = logit + p.Cp;                         // 256 * V floats
  __shared__ float rv[4];
  __shared__ int ri[4];

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int U = p.frames[b];
  int* tok = p.tokens + (long)b * p.max_tokens;
  int* tfr = p.tframes ? p.tframes + (long)b * p.max_tokens : nullptr;
  const T* whhT = (const T*)p.whhT;
  const T* wpT = (const T*)p.wpT;
  const T* woT = (const T*)p.woT;

  for (int i = tid; i < P; i += 256) { h[i] = 0.f; c[i] = 0.f; }
  __syncthreads();

  // prediction network on symbol k: gates, LSTM cell, then the joint's prediction half
  auto predict = [&](int k) {
    matvec<T>(whhT, 4 * P, P, 4 * P, h, p.gemb + (long)k * 4 * P, gates, part);
    for (int u = tid; u < P; u += 256) {
      const float ig = sigm(gates[u]), fg = sigm(gates[P + u]);
      const float gg = tanhf(gates[2 * P + u]), og = sigm(gates[3 * P + u]);
      const float cn = fg * c[u] + ig * gg;
      c[u] = cn;
      h[u] = og * tanhf(cn);
    }
    __syncthreads();
    matvec<T>(wpT, J, P, J, h, p.bp, fpred, part);
  };

  predict(blank);
  int n = 0;
  for (int t = 0; t < U; ++t) {
    const float* fe = p.fenc + ((long)b * p.stride + t) * J;
    for (int sym = 0; sym < p.max_symbols; ++sym) {
      for (int j = tid; j < J; j += 256) z[j] = fmaxf(fe[j] + fpred[j], 0.f);
      __syncthreads();
      matvec<T>(woT, p.Cp, J, C, z, p.bo, logit, part);
      // argmax, lowest index on ties (NaN never wins)
      float best = -INFINITY;
      int bi = C;
      for (int v = tid; v < C; v += 256) {
        const float a = logit[v];
        if (a > best) { best = a; bi = v; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
      }
      if (lane == 0) { rv[wv] = best; ri[wv] = bi; }
      __syncthreads();
      best = rv[0];
      bi = ri[0];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (rv[w] > best || (rv[w] == best && ri[w] < bi)) { best = rv[w]; bi = ri[w]; }
      __syncthreads();
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
  for (int i = n + tid; i < p.max_tokens; i += 256) {
    tok[i] = -1;
    if (tfr) tfr[i] = -1;
  }
  if (tid == 0) p.ntok[b] = n;
  (void)V;
}

size_t rnnt_lds_bytes(DType dt, int P, int J, int Cp) {
  const int V = dt == DT_F32 ? 4 : 8;
  return (size_t)(2 * P + 2 * J + 4 * P + Cp + 256 * V) * 4;
}

hipError_t launch_rnnt_decode(DType dt, const RnntParams& p, int batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const size_t lds = rnnt_lds_bytes(dt, p.P, p.J, p.Cp);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (dt == DT_F32)
    hipLaunchKernelGGL(k_rnnt<float>, dim3(batch), dim3(256), lds, s, p);
  else if (dt == DT_BF16)
    hipLaunchKernelGGL(k_rnnt<bf16>, dim3(batch), dim3(256), lds, s, p);
  else
    hipLaunchKernelGGL(k_rnnt<f16>, dim3(batch), dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace gg
