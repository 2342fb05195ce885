// Log-mel frontend for gfx950.
// "GigaAM v3 MLX" model card, table "Frontend configuration": 16 kHz, window 320,
// FFT 320, hop 160, center false, 64 mel bins, HTK scale, no mel normalisation,
// power 2.0; "GigaAM v3 RNNT - MLX" card, "Notes for other runtimes": the window and
// filterbank are stored model buffers and the features are log(clip(x, 1e-9, 1e9)).
//
// One block turns FE_FT frames into FE_FT x 64 log-mel values entirely on chip. The
// 320-point DFT of each windowed frame is factored as 320 = 16 x 20 (Cooley-Tukey with
// n = 20 n1 + n2, k = k1 + 16 k2):
//   Y[n2][k1] = sum_{n1<16} x[20 n1 + n2] W16^(n1 k1)           (16-point DFTs)
//   Z[n2][k1] = Y[n2][k1] W320^(n2 k1)                           (twiddle)
//   X[k1 + 16 k2] = sum_{n2<20} Z[n2][k1] W20^(n2 k2)            (20-point DFTs)
// evaluated in fp32 with twiddles rounded from fp64, for bins k <= 160 only; then
// power, mel projection and log-clip. The small DFTs keep their twiddles in registers.
// A one-block prologue kernel builds, once per launch, the twiddle table and each mel
// filter's range of nonzero weights; the projection sums over that range only, in the
// same ascending order as the full sum, so the result is the same (the skipped terms
// are exact zeros).
#include "kernels.h"

namespace gg {

constexpr int FE_FT = 12;     // frames per block
constexpr int FE_N = 320;     // FFT size = window length
constexpr int FE_K = 161;     // power bins 0..160
constexpr int FE_M = 64;      // mel bins

// twiddles W320^j = tw[j] - i tw[320 + j] (rounded from fp64) and, per mel filter m, the
// first and last bin with a nonzero weight (melr[2m], melr[2m + 1]; an all-zero filter
// gets an empty range)
__global__ void __launch_bounds__(FE_N) k_frontend_prep(const float* __restrict__ fb,
                                                        float* __restrict__ tw,
                                                        int* __restrict__ melr) {
  __shared__ int lo_s[FE_M], hi_s[FE_M];
  const int i = threadIdx.x;
  if (i < FE_M) {
    lo_s[i] = FE_K;
    hi_s[i] = -1;
  }
  double sn, cs;
  sincospi(2.0 * i / FE_N, &sn, &cs);
  tw[i] = (float)cs;
  tw[FE_N + i] = (float)sn;
  __syncthreads();
  // every filterbank entry once (coalesced, all loads issued before any test); the first
  // and last nonzero bin of each filter by LDS min / max (order-independent)
  constexpr int PER = (FE_K * FE_M + FE_N - 1) / FE_N;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = i + j * FE_N;
    v[j] = e < FE_K * FE_M ? fb[e] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = i + j * FE_N;
    if (v[j] != 0.f) {
      atomicMin(&lo_s[e % FE_M], e / FE_M);
      atomicMax(&hi_s[e % FE_M], e / FE_M);
    }
  }
  __syncthreads();
  if (i < FE_M) {
    melr[2 * i] = lo_s[i];
    melr[2 * i + 1] = hi_s[i];
  }
}

__global__ void __launch_bounds__(256) k_frontend(const float* __restrict__ pcm, int stride,
                                                  const float* __restrict__ window,
                                                  const float* __restrict__ fb,
                                                  const float* __restrict__ tw,
                                                  const int* __restrict__ melr, MetaDev m,
                                                  int T_tot, float* __restrict__ mel) {
  // one LDS region holds, in turn, the windowed frames, the stage-1 outputs and the power
  // spectra (each stage reads its input into registers before the next is written), so
  // four blocks fit on a CU
  constexpr int ZP = 17;                          // row pitch of the stage-1 outputs
  constexpr int ZSZ = FE_FT * 20 * ZP;
  static_assert(FE_FT * FE_N <= 2 * ZSZ && FE_FT * (FE_K + 3) <= 2 * ZSZ, "LDS reuse");
  __shared__ float region[2 * ZSZ];
  __shared__ float tc[FE_N], ts[FE_N];           // W320^j = tc[j] - i ts[j]
  float (*xw)[FE_N] = (float (*)[FE_N])region;
  float (*zr)[20][ZP] = (float (*)[20][ZP])region;
  float (*zi)[20][ZP] = (float (*)[20][ZP])(region + ZSZ);
  float (*P)[FE_K + 3] = (float (*)[FE_K + 3])region;
  __shared__ long foff[FE_FT];                   // each frame's first sample in pcm (-1: none)
  const int tid = threadIdx.x;
  const int f0 = blockIdx.x * FE_FT;
  const int f1 = tid / 20, n21 = tid - f1 * 20;  // stage-1 thread (frame, n2)
  const int mm = tid & (FE_M - 1);               // this thread's mel filter (every pass)

  // Everything that does not depend on the samples is loaded first and independently of
  // them: the frames' clip geometry (one dependent pair of loads per frame, not per
  // sample), the twiddles, this stage-1 thread's 16 window values and this thread's mel
  // filter's nonzero range (its weights are loaded during stage 2).
  if (tid < FE_FT) {
    const int g = f0 + tid;
    long off = -1;
    if (g < T_tot) {
      const int b = m.rowT[g];
      off = (long)b * stride + 160L * (g - m.cuT[b]);
    }
    foff[tid] = off;
  }
  for (int i = tid; i < FE_N; i += 256) {
    tc[i] = tw[i];
    ts[i] = tw[FE_N + i];
  }
  float win[16];
#pragma unroll
  for (int n1 = 0; n1 < 16; ++n1) win[n1] = tid < FE_FT * 20 ? window[20 * n1 + n21] : 0.f;
  const int lo = melr[2 * mm], hi = melr[2 * mm + 1];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < (FE_FT * FE_N + 255) / 256; ++r) {   // independent loads, all in flight
    const int e = tid + 256 * r;
    if (e < FE_FT * FE_N) {
      const int f = e / FE_N, n = e - f * FE_N;
      const long off = foff[f];
      xw[f][n] = off >= 0 ? pcm[off + n] : 0.f;
    }
  }
  __syncthreads();

  // stage 1: thread (f, n2) -> 16-point DFT over n1 of the windowed frame, then the
  // W320^(n2 k1) twiddle
  float x[16];
  if (tid < FE_FT * 20) {
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) x[n1] = xw[f1][20 * n1 + n21] * win[n1];
  }
  __syncthreads();                               // the frames are in registers: reuse
  if (tid < FE_FT * 20) {
    const int f = f1, n2 = n21;
#pragma unroll
    for (int k1 = 0; k1 < 16; ++k1) {
      float yr = 0.f, yi = 0.f;
#pragma unroll
      for (int n1 = 0; n1 < 16; ++n1) {
        const int j = 20 * ((n1 * k1) & 15);      // W16^(n1 k1) = W320^(20 (n1 k1 mod 16))
        yr = fmaf(x[n1], tc[j], yr);
        yi = fmaf(-x[n1], ts[j], yi);
      }
      const int j = (n2 * k1) % FE_N;
      const float c = tc[j], sn = ts[j];           // (yr + i yi)(c - i sn)
      zr[f][n2][k1] = yr * c + yi * sn;
      zi[f][n2][k1] = yi * c - yr * sn;
    }
  }
  __syncthreads();

  // stage 2: thread (f, k1) -> 20-point DFT over n2 for k2 = 0..10, power of bins <= 160
  const int f2 = tid >> 4, k12 = tid & 15;
  float ar[20], ai[20];
  if (tid < FE_FT * 16) {
#pragma unroll
    for (int n2 = 0; n2 < 20; ++n2) { ar[n2] = zr[f2][n2][k12]; ai[n2] = zi[f2][n2][k12]; }
  }
  __syncthreads();                               // stage-1 outputs in registers: reuse
  // this thread's mel filter weights (the HTK filters span at most 13 bins), in flight
  // during stage 2
  constexpr int MW = 16;
  float wts[MW];
#pragma unroll
  for (int j = 0; j < MW; ++j) wts[j] = lo + j <= hi ? fb[(lo + j) * FE_M + mm] : 0.f;
  if (tid < FE_FT * 16) {
    const int f = f2, k1 = k12;
#pragma unroll
    for (int k2 = 0; k2 <= 10; ++k2) {
      const int k = k1 + 16 * k2;
      if (k < FE_K) {
        float xr = 0.f, xi = 0.f;
#pragma unroll
        for (int n2 = 0; n2 < 20; ++n2) {
          const int j = 16 * ((n2 * k2) % 20);    // W20^(n2 k2) = W320^(16 (n2 k2 mod 20))
          const float c = tc[j], sn = ts[j];
          xr = fmaf(ar[n2], c, fmaf(ai[n2], sn, xr));
          xi = fmaf(ai[n2], c, fmaf(-ar[n2], sn, xi));
        }
        P[f][k] = xr * xr + xi * xi;
      }
    }
  }
  __syncthreads();

  // mel projection + log clip: thread (f, m), the filter's weights already in registers
  // (a wider filter continues from the table), summed in ascending bin order
  for (int e = tid; e < FE_FT * FE_M; e += 256) {
    const int f = e >> 6;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < MW; ++j)
      if (lo + j <= hi) acc = fmaf(wts[j], P[f][lo + j], acc);
    for (int k = lo + MW; k <= hi; ++k) acc = fmaf(fb[k * FE_M + mm], P[f][k], acc);
    const int g = f0 + f;
    if (g < T_tot) mel[(long)g * FE_M + mm] = logf(fminf(fmaxf(acc, 1e-9f), 1e9f));
  }
}

hipError_t launch_frontend(const float* pcm, int stride, const float* window, const float* fb,
                           const MetaDev& m, int T_tot, float* mel, float* tw, int* melr,
                           hipStream_t s) {
  if (T_tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_frontend_prep, dim3(1), dim3(FE_N), 0, s, fb, tw, melr);
  hipLaunchKernelGGL(k_frontend, dim3((T_tot + FE_FT - 1) / FE_FT), dim3(256), 0, s, pcm, stride,
                     window, fb, tw, melr, m, T_tot, mel);
  return hipGetLastError();
}

// Default frontend tables, computed in fp64: periodic Hann window and the HTK
// triangular filterbank on [0, 8000] Hz (65 equal mel steps between 66 corner
// frequencies; filter m rises over corners m..m+1 and falls over m+1..m+2).
__global__ void k_default_frontend(float* window, float* fb) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < FE_N) window[i] = (float)(0.5 - 0.5 * cospi(2.0 * i / FE_N));
  if (i < FE_K * FE_M) {
    const int k = i / FE_M, mm = i - k * FE_M;
    const double mel_top = 2595.0 * log10(1.0 + 8000.0 / 700.0);
    double c[3];
    for (int j = 0; j < 3; ++j) {
      const double mj = mel_top * (double)(mm + j) / 65.0;
      c[j] = 700.0 * (pow(10.0, mj / 2595.0) - 1.0);
    }
    const double f = 50.0 * k;
    const double up = (f - c[0]) / (c[1] - c[0]);
    const double dn = (c[2] - f) / (c[2] - c[1]);
    fb[i] = (float)fmax(0.0, fmin(up, dn));
  }
}

hipError_t launch_default_frontend(float* window, float* fb, hipStream_t s) {
  hipLaunchKernelGGL(k_default_frontend, dim3((FE_K * FE_M + 255) / 256), dim3(256), 0, s,
                     window, fb);
  return hipGetLastError();
}

}  // namespace gg
