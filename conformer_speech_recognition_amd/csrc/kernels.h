// Internal launcher interface between the host orchestration and the kernels.
#pragma once
#include "common.h"

namespace gg {

// ---- GEMM: C[m, n] = epilogue( sum_k A[m, k] * W[n, k] + bias[n] ) -------------------
enum AMode {
  A_PLAIN = 0,     // A: T [M][lda]
  A_F32 = 1,       // A: float [M][lda], rounded to T while staging
  A_DUAL = 2,      // A for output columns < nsplit, A2 for the rest (both T)
  A_CONV = 3,      // implicit Conv1d k5 s2 p2 over packed clips, source T [rows][cin]
  A_CONV_F32 = 4   // same, source float
};
enum Epi {
  E_STORE = 0,     // C (T)      = acc + b
  E_SILU = 1,      // C (T)      = silu(acc + b)
  E_RELU = 2,      // C (T)      = relu(acc + b)
  E_RELU_F32 = 3,  // C (float)  = relu(acc + b)
  E_GLU = 4,       // C (T) [M][N/2]: value/gate pairs of 32-column blocks
  E_RESID = 5,     // C (float) += alpha * (acc + b)
  E_F32 = 6        // C (float)  = acc + b
};

struct GemmParams {
  int M, N, K;
  const void* A; int lda;
  const void* A2; int nsplit;
  const void* W; int ldw;          // [N][ldw] in T, or packed qbits-bit rows (ldw in weights)
  const f16* Wscale;               // quantised weights: [N][K/64] fp16 scales
  const float* bias;               // [N] or nullptr
  void* C; int ldc;
  float alpha;
  const int* rowclip;              // conv modes: clip of each output row
  const int* cu_in;                // conv modes: input row offsets per clip
  const int* cu_out;               // conv modes: output row offsets per clip
  int cin;                         // conv modes: input channels (row length of source)
  float* part;                     // split-K partial sums (fp32), or nullptr: never split
  long part_cap;                   // floats available at part
};

// Floats of split-K partials any launch_gemm call may use (the workspace reserves this
// much for part): a split keeps tiles * slices <= 256, so M * N * slices <= 256 * 256 * 128.
constexpr long kSplitPartFloats = 256L * 256 * 128;

// qbits: 0 = weights stored in the operand type; 8 / 6 / 4 = packed quantised rows with
// fp16 group scales (dequantised to fp16 in the kernel). deferred_ks (E_RESID only, may be
// nullptr): when the K sum is split, the slices are left in p.part, their number is written
// here and the caller's next kernel must add them (LnParams.rks); 0 when nothing is deferred.
hipError_t launch_gemm(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p,
                       hipStream_t s, int* deferred_ks = nullptr);
// K slices launch_gemm uses for these arguments (1: no split)
int gemm_split_slices(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p);
// Kernel shape launch_gemm uses for these arguments (the GIGAAM_GEMM_* ids of gigaam.h)
enum GemmShape {
  GEMM_REG_128x64 = 1, GEMM_REG_128x128 = 2, GEMM_DMA_256x256 = 3, GEMM_DMA_256x128_K32 = 4,
  GEMM_DMA_256x128_K64 = 5, GEMM_DMA_128x128 = 6, GEMM_DMA_256x192 = 7, GEMM_DMA_256x128_W4 = 8,
  GEMM_DMA_256x128_W4S = 9, GEMM_DMA_128x256 = 10,
  GEMM_DMA_128x128_S3 = 11
};
int gemm_shape_id(DType dt, int qbits, AMode am, Epi ep, const GemmParams& p);
// Diagnostics: force the direct-load variant of the following launches on this thread (0:
// the encoder's choice); returns the previous setting, or -1 for an unknown id.
int gemm_force_variant(int id);

// Fused macaron FFN for few rows: x += alpha * (W2 SiLU(W1 y + b1) + b2) without the hidden
// activations in HBM (16-bit weights, d 768 or 1024, f a multiple of 256, at most
// kMlpMaxRows rows; part holds (f / 256) * M * d floats of partial sums).
struct MlpArgs {
  int M, d, f;
  const void* y;                   // T [M][d], the LayerNorm output
  const void* W1; const float* b1; // [f][d], [f]
  const void* W2;                  // [d][f]
  float* part;                     // fp32 scratch
};
constexpr int kMlpMaxRows = 896;
bool mlp_fusable(DType dt, int qbits, int M, int d, int f, long part_cap);
hipError_t launch_mlp(DType dt, const MlpArgs& a, const float* b2, float alpha, float* x,
                      hipStream_t s);

// ---- meta -------------------------------------------------------------------------
hipError_t launch_meta(const MetaArgs& a, const MetaDev& m, int T_tot, int S_tot, int U_tot,
                       hipStream_t s);
// n floats from src to dst (non-overlapping device ranges)
hipError_t launch_copy_f32(float* dst, const float* src, long n, hipStream_t s);

// ---- frontend -----------------------------------------------------------------------
// tw: 640 floats and melr: 128 ints of scratch for the per-launch tables; mel_t (or
// nullptr): a second copy of the log-mel rows rounded to mel_dt (DT_F16 or DT_BF16), the
// operand of the first subsampling conv on 16-bit models
hipError_t launch_frontend(const float* pcm, int stride, const float* window, const float* fb,
                           const MetaDev& m, int T_tot, float* mel, void* mel_t, DType mel_dt,
                           float* tw, int* melr, hipStream_t s);
hipError_t launch_default_frontend(float* window, float* fb, hipStream_t s);

// ---- norms / rotary -----------------------------------------------------------------
enum LnMode { LN_PLAIN = 0, LN_ROPE = 1, LN_TWO = 2 };
struct LnParams {
  int rows, d;
  float* x;                        // [rows][d] fp32 (LN_TWO writes x back in place)
  const float* g1; const float* b1;
  const float* g2; const float* b2;  // LN_TWO: second norm applied to the first's output
  void* y;                         // T out
  void* r;                         // LN_ROPE: rotated copy (T)
  const float* cos_t; const float* sin_t;  // [U_max][d_k/2]
  const int* rowpos;                       // LN_ROPE: position of each row inside its clip
  float eps;
  // a residual GEMM's deferred split-K sum, added to x first: x += ralpha * (sum of the rks
  // slices of rpart [rks][rows][d] in slice order + rbias); rks = 0: none, else 1..4 with
  // rpart and rbias both given
  const float* rpart; const float* rbias; int rks; float ralpha;
};
hipError_t launch_layernorm(DType dt, LnMode mode, const LnParams& p, hipStream_t s);
hipError_t launch_rope_table(float* cos_t, float* sin_t, int n_pos, int dk, float base,
                             hipStream_t s);

// ---- attention ----------------------------------------------------------------------
struct AttnParams {
  const void* qkv;                 // T [rows][3d]: q | k | v
  void* out;                       // T [rows][d]
  // query tiles: 128 frames for the 16-bit kernel (MetaDev cuQ2 / tileQ2), 64 frames for
  // the fp32 kernel (cuQ / tileQ)
  int d, n_heads, n_tiles;
  const int* cuU; const int* cuQ; const int* tileQ;
  float scale_log2;                // log2(e) / sqrt(d_k)
  // 16-bit kernel, a clip or two: the 64-frame tiles, each taken by two wave pairs that split
  // the keys, and their geometry records (MetaDev tileG); n_tiles64 = 0: not used
  int n_tiles64; const int* tileG64;
};
hipError_t launch_attention(DType dt, int dk, const AttnParams& p, hipStream_t s);

// ---- conv module: depthwise + BatchNorm + SiLU --------------------------------------
struct DwParams {
  const void* in; void* out;       // T [rows][d]
  const float* w; const float* b;  // taps [K][d] (tap-major), bias [d]
  const float* bn_g; const float* bn_b; const float* bn_m; const float* bn_v;
  int d, n_tiles;
  const int* cuU; const int* cuQ; const int* tileQ;
  const int* tileG;                // per 64-frame tile: first row, clip length, first frame, clip
  float eps;
};
hipError_t launch_dwconv(DType dt, int kernel, const DwParams& p, hipStream_t s);

// ---- CTC head -----------------------------------------------------------------------
hipError_t launch_logsoftmax_argmax(const float* logits, int C, int B, int U_max,
                                    const int* cuU, float* logp, int* frame_ids,
                                    hipStream_t s);
hipError_t launch_collapse(const int* frame_ids, int B, int U_max, const int* cuU, int blank,
                           int* tokens, int* n_tokens, hipStream_t s);
hipError_t launch_scatter_rows(const float* x, int d, int B, int U_max, const int* cuU,
                               float* out, hipStream_t s);

// ---- RNNT greedy decoding (one workgroup per clip) ---------------------------------
struct RnntParams {
  const float* fenc;               // [batch * stride][J]: W_enc e_t + b_enc per frame
  const float* gemb;               // [C][4P]: W_ih embed[k] + b_ih + b_hh per symbol
  const void* whhT;                // T [P][4P]   (W_hh transposed)
  const void* wpT;                 // T [P][J]    (W_pred transposed)
  const float* bp;                 // [J]
  const void* woT;                 // T [J][Cp]   (W_out transposed, columns padded)
  const float* bo;                 // [C]
  int P, J, C, Cp, max_symbols, stride, max_tokens;
  int wo_lds;                      // W_out^T is copied to LDS (rnnt_lds_bytes counts it)
  int* tokens; int* tframes; int* ntok;
  int frames[kMaxBatch];
};
size_t rnnt_lds_bytes(DType dt, int P, int J, int Cp, bool wo_lds);
hipError_t launch_rnnt_decode(DType dt, const RnntParams& p, int batch, hipStream_t s);

// Clustered decoding (G cooperative workgroups per clip exchanging partial logits and h
// slices through sequence-tagged 64-bit words).
struct RnntCluster {
  unsigned long long* xl;          // [batch][2][G][Cp] partial logits, then
  unsigned long long* xh;          // [batch][2][P] h slices, then
  unsigned long long* xc;          // [batch][G] each member's XCD (contiguous, xbytes in all)
  int xbytes;
  int batch;
  int G;                           // members per clip (P % G == J % G == 0)
  int wo_lds;                      // the member's W_out columns are copied to LDS
  int spin_limit;                  // polls before a member gives up (its clip: n_tokens < 0)
};
long rnnt_cl_grid(int batch, int G);
size_t rnnt_cl_lds_bytes(DType dt, int P, int J, int Cp, int G, bool wo_lds);
// largest usable G <= max_g for this batch on the current device (1: none)
int rnnt_cluster_size(DType dt, int P, int J, int Cp, int batch, int max_g);
hipError_t launch_rnnt_cluster(DType dt, const RnntParams& p, const RnntCluster& q, int batch,
                               hipStream_t s);

}  // namespace gg
