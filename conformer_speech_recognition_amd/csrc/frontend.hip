// Log-mel frontend for gfx950.
// "GigaAM v3 MLX" model card, table "Frontend configuration": 16 kHz, window 320,
// FFT 320, hop 160, center false, 64 mel bins, HTK scale, no mel normalisation,
// power 2.0; "GigaAM v3 RNNT - MLX" card, "Notes for other runtimes": the window and
// filterbank are stored model buffers and the features are log(clip(x, 1e-9, 1e9)).
//
// One block turns 32 frames into 32 x 64 log-mel values entirely on chip:
//   framing + window (LDS) -> 161-bin DFT power (fp32, twiddles from an fp64 table in
//   LDS, 3 bins x 8 frames per thread) -> mel projection -> log-clip -> one store.
#include "kernels.h"

namespace gg {

constexpr int FE_FT = 32;     // frames per block
constexpr int FE_N = 320;     // FFT size = window length
constexpr int FE_K = 161;     // power bins 0..160
constexpr int FE_M = 64;      // mel bins

__global__ void __launch_bounds__(256) k_frontend(const float* __restrict__ pcm, int stride,
                                                  const float* __restrict__ window,
                                                  const float* __restrict__ fb, MetaDev m,
                                                  int T_tot, float* __restrict__ mel) {
  __shared__ float xw[FE_FT][FE_N];
  __shared__ float tc[FE_N], ts[FE_N];
  __shared__ float P[FE_FT][FE_K];
  const int tid = threadIdx.x;
  const int f0 = blockIdx.x * FE_FT;

  for (int i = tid; i < FE_N; i += 256) {
    double s, c;
    sincospi(2.0 * i / FE_N, &s, &c);
    tc[i] = (float)c;
    ts[i] = (float)s;
  }
  for (int e = tid; e < FE_FT * FE_N; e += 256) {
    const int f = e / FE_N, n = e - f * FE_N, g = f0 + f;
    float v = 0.f;
    if (g < T_tot) {
      const int b = m.rowT[g];
      const int t = g - m.cuT[b];
      v = pcm[(long)b * stride + 160 * t + n] * window[n];
    }
    xw[f][n] = v;
  }
  __syncthreads();

  // power spectrum: lane kl handles bins kl, kl + 64, kl + 128; wave fg frames 8fg..8fg+7
  const int kl = tid & 63, fg = tid >> 6;
  float re[3][8], im[3][8];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int f = 0; f < 8; ++f) re[j][f] = im[j][f] = 0.f;
  int idx[3] = {0, 0, 0};
  const int kk[3] = {kl, kl + 64, kl + 128};
  for (int n = 0; n < FE_N; ++n) {
    float xv[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) xv[f] = xw[fg * 8 + f][n];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const float c = tc[idx[j]], s = ts[idx[j]];
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        re[j][f] = fmaf(xv[f], c, re[j][f]);
        im[j][f] = fmaf(-xv[f], s, im[j][f]);
      }
      idx[j] += kk[j];
      if (idx[j] >= FE_N) idx[j] -= FE_N;
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (kk[j] < FE_K)
#pragma unroll
      for (int f = 0; f < 8; ++f) P[fg * 8 + f][kk[j]] = re[j][f] * re[j][f] + im[j][f] * im[j][f];
  __syncthreads();

  // mel projection + log clip: lane = mel bin, wave fg = frames 8fg..8fg+7
  const int mm = tid & 63;
  float acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = 0.f;
  for (int k = 0; k < FE_K; ++k) {
    const float w = fb[k * FE_M + mm];
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[f] = fmaf(w, P[fg * 8 + f][k], acc[f]);
  }
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int g = f0 + fg * 8 + f;
    if (g < T_tot) mel[(long)g * FE_M + mm] = logf(fminf(fmaxf(acc[f], 1e-9f), 1e9f));
  }
}

hipError_t launch_frontend(const float* pcm, int stride, const float* window, const float* fb,
                           const MetaDev& m, int T_tot, float* mel, hipStream_t s) {
  if (T_tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_frontend, dim3((T_tot + FE_FT - 1) / FE_FT), dim3(256), 0, s, pcm, stride,
                     window, fb, m, T_tot, mel);
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
