// Log-mel frontend for gfx950.
// "GigaAM v3 MLX" model card, table "Frontend configuration": 16 kHz, window 320,
// FFT 320, hop 160, center false, 64 mel bins, HTK scale, no mel normalisation,
// power 2.0; "GigaAM v3 RNNT - MLX" card, "Notes for other runtimes": the window and
// filterbank are stored model buffers and the features are log(clip(x, 1e-9, 1e9)).
//
// One wave turns two frames at a time into 2 x 64 log-mel values, 32 lanes per frame,
// with no workgroup barrier in its loop. The 320-point DFT of the real windowed frame x
// comes from one 160-point complex DFT of z[n] = x[2n] + i x[2n+1] (even samples as the
// real part, odd as the imaginary part), factored as 160 = 5 x 32 (Cooley-Tukey with
// n = 32 n1 + n2, k = k1 + 5 k2):
//   Y[n2][k1] = sum_{n1<5} z[32 n1 + n2] W5^(n1 k1)          lane n2, in registers
//   Y[n2][k1] *= W160^(n2 k1)                                 twiddle
//   Z[k1 + 5 k2] = sum_{n2<32} Y[n2][k1] W32^(n2 k2)          radix-2 across the 32 lanes
// The radix-2 steps are decimation in frequency over lane spans 16, 8, 4, 2, 1 (lane
// exchanges), which leaves Z[k1 + 5 k2] in lane bitreverse(k2). Through the wave's LDS
// slice, the even / odd halves are separated,
//   E[k] = (Z[k] + conj Z[160 - k]) / 2,  O[k] = (Z[k] - conj Z[160 - k]) / 2i,
//   X[k] = E[k] + W320^k O[k]  (k < 160),  X[160] = E[0] - O[0],
// then power |X[k]|^2 for k <= 160, the mel projection and the log-clip. Everything is
// fp32 with twiddles rounded from fp64. A one-block prologue kernel builds, once per
// launch, the twiddle table and each mel filter's range of nonzero weights; the
// projection sums over that range only, in the same ascending order as the full sum, so
// the result is the same (the skipped terms are exact zeros).
#include <type_traits>

#include "kernels.h"

namespace gg {

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

constexpr int FE_WAVES = 4;   // waves per block, each with its own LDS slice

// the value of lane ^ SP (SP = 16, 8, 4, 2, 1: inside the lane's 32-lane half) on vector
// lane operations instead of the LDS crossbar a shuffle takes: a row swap for 16 (whichever
// of the two results is not the lane's own value; equal values make either one right), a row
// rotation by 8, a half-row mirror then a quad reversal for 4, quad permutations for 2 and 1
template <int SP> __device__ __forceinline__ float lane_xor(float v) {
  if constexpr (SP == 16) {
    uint32_t a, b;
    pair_x16(fbits(v), a, b);
    return ffrom(a == fbits(v) ? b : a);
  } else if constexpr (SP == 8) {
    return dpp_f<kDppRor8>(v);
  } else if constexpr (SP == 4) {
    return dpp_f<0x1B>(dpp_f<0x141>(v));
  } else if constexpr (SP == 2) {
    return dpp_f<kDppXor2>(v);
  } else {
    static_assert(SP == 1, "span");
    return dpp_f<kDppXor1>(v);
  }
}

__device__ __forceinline__ float2 cmul(float2 a, float c, float sn) {   // a (c - i sn)
  return make_float2(fmaf(a.x, c, a.y * sn), fmaf(a.y, c, -a.x * sn));
}

__global__ void __launch_bounds__(64 * FE_WAVES) k_frontend(const float* __restrict__ pcm, int stride,
                                                          const float* __restrict__ window,
                                                          const float* __restrict__ fb,
                                                          const float* __restrict__ tw,
                                                          const int* __restrict__ melr, MetaDev m,
                                                          int T_tot, float* __restrict__ mel,
                                                          void* __restrict__ mel_t, int mel_dt) {
  __shared__ float tc[FE_N], ts[FE_N];                  // W320^t = tc[t] - i ts[t]
  __shared__ float2 zs[FE_WAVES][2][164];               // Z of the wave's two frames (padded)
  __shared__ float ps[FE_WAVES][2][FE_K + 3];           // their power spectra
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5, j = lane & 31;               // frame of the pair, n2 / output lane

  for (int i = threadIdx.x; i < FE_N; i += 64 * FE_WAVES) {
    tc[i] = tw[i];
    ts[i] = tw[FE_N + i];
  }
  // per-lane constants, loaded once: this lane's 10 window values (samples 2j + 64 n1 and
  // the next), its two mel filters (j and j + 32: range and up to 16 weights each)
  float wv[5][2];
#pragma unroll
  for (int n1 = 0; n1 < 5; ++n1) {
    wv[n1][0] = window[2 * j + 64 * n1];
    wv[n1][1] = window[2 * j + 64 * n1 + 1];
  }
  constexpr int MW = 16;
  int lo[2], hi[2];
  float wts[2][MW];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int mm = j + 32 * q;
    lo[q] = melr[2 * mm];
    hi[q] = melr[2 * mm + 1];
#pragma unroll
    for (int t = 0; t < MW; ++t) wts[q][t] = lo[q] + t <= hi[q] ? fb[(lo[q] + t) * FE_M + mm] : 0.f;
  }
  __syncthreads();                                      // the twiddle table, once
  // W5^q = W320^(64 q) for q = 1, 2 (the only two the 5-point DFT needs, with conjugates)
  const float c1 = tc[64], s1 = ts[64], c2 = tc[128], s2 = ts[128];
  // stage-1 twiddles W160^(j k1) = W320^(2 j k1), k1 = 1..4
  float t1c[4], t1s[4];
#pragma unroll
  for (int k1 = 1; k1 < 5; ++k1) { t1c[k1 - 1] = tc[2 * j * k1]; t1s[k1 - 1] = ts[2 * j * k1]; }
  // radix-2 steps over spans 16, 8, 4, 2: the lower lane of a pair keeps x + partner, the
  // upper one (partner - x) W_{2s}^(j mod s) = (partner - x) W320^((j mod s) 160 / s)
  float bs[4], bc[4], bn[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int sp = 16 >> st;
    const bool up = (j & sp) != 0;
    const int t = up ? (j & (sp - 1)) * (160 / sp) : 0;
    bs[st] = up ? -1.f : 1.f;
    bc[st] = tc[t];
    bn[st] = ts[t];
  }
  const int br = (int)(__builtin_bitreverse32((uint32_t)j) >> 27);   // k2 held after the steps

  const int n_pairs = (T_tot + 1) >> 1;
  for (int pr = blockIdx.x * FE_WAVES + wave; pr < n_pairs; pr += gridDim.x * FE_WAVES) {
    const int g = 2 * pr + h;                           // this half-wave's frame
    float2 z[5];
    if (g < T_tot) {
      const int b = m.rowT[g];
      const float* x = pcm + (long)b * stride + 160L * (g - m.cuT[b]) + 2 * j;
#pragma unroll
      for (int n1 = 0; n1 < 5; ++n1)
        z[n1] = make_float2(x[64 * n1] * wv[n1][0], x[64 * n1 + 1] * wv[n1][1]);
    } else {
#pragma unroll
      for (int n1 = 0; n1 < 5; ++n1) z[n1] = make_float2(0.f, 0.f);
    }
    // 5-point DFT over n1: y[k] and y[5 - k] share R = sum z[n1] cos, I = sum z[n1] sin
    float2 y[5];
    y[0] = make_float2(z[0].x + z[1].x + z[2].x + z[3].x + z[4].x,
                       z[0].y + z[1].y + z[2].y + z[3].y + z[4].y);
    {
      // k = 1: cos / sin of 2 pi n1 / 5 for n1 = 1..4 are (c1, s1), (c2, s2), (c2, -s2), (c1, -s1)
      const float Rx = fmaf(c1, z[1].x + z[4].x, c2 * (z[2].x + z[3].x));
      const float Ry = fmaf(c1, z[1].y + z[4].y, c2 * (z[2].y + z[3].y));
      const float Ix = fmaf(s1, z[1].x - z[4].x, s2 * (z[2].x - z[3].x));
      const float Iy = fmaf(s1, z[1].y - z[4].y, s2 * (z[2].y - z[3].y));
      y[1] = make_float2(z[0].x + Rx + Iy, z[0].y + Ry - Ix);     // z0 + R - i I
      y[4] = make_float2(z[0].x + Rx - Iy, z[0].y + Ry + Ix);     // z0 + R + i I
    }
    {
      // k = 2: angles 4 pi n1 / 5 -> (c2, s2), (c1, -s1), (c1, s1), (c2, -s2)
      const float Rx = fmaf(c2, z[1].x + z[4].x, c1 * (z[2].x + z[3].x));
      const float Ry = fmaf(c2, z[1].y + z[4].y, c1 * (z[2].y + z[3].y));
      const float Ix = fmaf(s2, z[1].x - z[4].x, -s1 * (z[2].x - z[3].x));
      const float Iy = fmaf(s2, z[1].y - z[4].y, -s1 * (z[2].y - z[3].y));
      y[2] = make_float2(z[0].x + Rx + Iy, z[0].y + Ry - Ix);
      y[3] = make_float2(z[0].x + Rx - Iy, z[0].y + Ry + Ix);
    }
#pragma unroll
    for (int k1 = 1; k1 < 5; ++k1) y[k1] = cmul(y[k1], t1c[k1 - 1], t1s[k1 - 1]);
    // radix-2 steps across the frame's 32 lanes
    auto step = [&](auto spc, int st) {
      constexpr int SP = decltype(spc)::value;
#pragma unroll
      for (int k1 = 0; k1 < 5; ++k1) {
        const float px = lane_xor<SP>(y[k1].x), py = lane_xor<SP>(y[k1].y);
        if constexpr (SP > 1) {
          const float2 d = make_float2(fmaf(bs[st], y[k1].x, px), fmaf(bs[st], y[k1].y, py));
          y[k1] = cmul(d, bc[st], bn[st]);
        } else {
          const float sg = (j & 1) ? -1.f : 1.f;
          y[k1] = make_float2(fmaf(sg, y[k1].x, px), fmaf(sg, y[k1].y, py));
        }
      }
    };
    step(std::integral_constant<int, 16>{}, 0);
    step(std::integral_constant<int, 8>{}, 1);
    step(std::integral_constant<int, 4>{}, 2);
    step(std::integral_constant<int, 2>{}, 3);
    step(std::integral_constant<int, 1>{}, 4);
#pragma unroll
    for (int k1 = 0; k1 < 5; ++k1) zs[wave][h][k1 + 5 * br] = y[k1];
    wave_lds_sync();
    // even / odd separation and power, bins k = j + 32 q; k = 160 from Z[0] (lane 0)
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int k = j + 32 * q;
      const float2 a = zs[wave][h][k];
      float p;
      if (k == 0) {
        const float x0 = a.x + a.y, x160 = a.x - a.y;
        p = x0 * x0;
        ps[wave][h][160] = x160 * x160;
      } else {
        const float2 c = zs[wave][h][160 - k];
        const float Er = 0.5f * (a.x + c.x), Ei = 0.5f * (a.y - c.y);
        const float2 o = cmul(make_float2(0.5f * (a.y + c.y), -0.5f * (a.x - c.x)), tc[k], ts[k]);
        const float Xr = Er + o.x, Xi = Ei + o.y;
        p = fmaf(Xr, Xr, Xi * Xi);
      }
      ps[wave][h][k] = p;
    }
    wave_lds_sync();
    // mel projection (ascending bins of each filter's range) and log clip
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < MW; ++t)
        if (lo[q] + t <= hi[q]) acc = fmaf(wts[q][t], ps[wave][h][lo[q] + t], acc);
      for (int k = lo[q] + MW; k <= hi[q]; ++k) acc = fmaf(fb[k * FE_M + j + 32 * q], ps[wave][h][k], acc);
      if (g < T_tot) {
        const long o = (long)g * FE_M + j + 32 * q;
        const float v = logf(fminf(fmaxf(acc, 1e-9f), 1e9f));
        mel[o] = v;
        if (mel_dt == DT_F16) ((f16*)mel_t)[o] = (f16)v;          // round to nearest even
        else if (mel_dt == DT_BF16) ((bf16*)mel_t)[o] = (bf16)v;
      }
    }
    wave_lds_sync();                                    // spectra read before the next pair
  }
}

hipError_t launch_frontend(const float* pcm, int stride, const float* window, const float* fb,
                           const MetaDev& m, int T_tot, float* mel, void* mel_t, DType mel_dt,
                           float* tw, int* melr, hipStream_t s) {
  if (mel_dt != DT_F32 && mel_dt != DT_F16 && mel_dt != DT_BF16) return hipErrorInvalidValue;
  if (mel_dt != DT_F32 && !mel_t) return hipErrorInvalidValue;
  if (T_tot <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_frontend_prep, dim3(1), dim3(FE_N), 0, s, fb, tw, melr);
  // waves walk frame pairs: one pass over all pairs with four 4-wave blocks per CU
  const int pairs = (T_tot + 1) / 2;
  const int blocks = std::min((pairs + FE_WAVES - 1) / FE_WAVES, 1024);
  hipLaunchKernelGGL(k_frontend, dim3(blocks), dim3(64 * FE_WAVES), 0, s, pcm, stride, window, fb,
                     tw, melr, m, T_tot, mel, mel_t, (int)mel_dt);
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
