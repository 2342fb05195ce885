/*
 * gigaam.h - C ABI of the MI355X (gfx950) Conformer CTC encoder forward pass.
 *
 * The path (pages cited by title and section):
 *   PCM 16 kHz -> log-mel frontend (window 320, hop 160, FFT 320, 64 HTK mel bins,
 *       no centring, log(clip(x, 1e-9, 1e9)))          ["GigaAM v3 MLX" card, Frontend
 *                                                      configuration; "GigaAM v3 RNNT - MLX"
 *                                                      card, Notes for other runtimes]
 *   -> two Conv1d, kernel 5, stride 2 (4x fewer frames) ["GigaAM on MLX: the transcripts
 *                                                      matched, but the model was broken",
 *                                                      What we're porting]
 *   -> N Conformer blocks: FFN, rotary self-attention with the rotation (base 5000)
 *      applied to the per-head LayerNorm output BEFORE linear_q/linear_k and value not
 *      rotated, convolution module, FFN               [same page, Trap 1 and Trap 2;
 *                                                      "GigaAM MLX port for Mac", What is
 *                                                      inside the model]
 *   -> CTC linear + log-softmax, greedy collapse with blank = n_classes - 1
 *                                                     ["GigaAM v3 RNNT - MLX" card, Notes]
 *
 * Conventions for every entry point
 *   - Returns GIGAAM_OK (0) or a negative error code; no exception crosses the ABI.
 *     gigaam_last_error() then holds a message (thread-local, valid until the next
 *     call on the same thread).
 *   - All argument checks happen before the first GPU launch, so a failed call leaves
 *     every output untouched.
 *   - "dev" pointers are device memory on the current HIP device; "host" pointers are
 *     host memory. The caller allocates and owns every buffer; the library never calls
 *     hipMalloc. A model handle borrows its device pointers: they must outlive it.
 *   - Device work is enqueued on the caller's hip_stream (NULL = default stream) and
 *     is complete when that stream is; host-side outputs are written before return.
 *   - A model handle is immutable after creation: concurrent encodes are allowed when
 *     each uses its own workspace and stream.
 */
#ifndef GIGAAM_H
#define GIGAAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GIGAAM_OK = 0,
  GIGAAM_E_INVAL = -1,       /* bad argument (null pointer, size out of range ...) */
  GIGAAM_E_WORKSPACE = -2,   /* workspace smaller than gigaam_workspace_bytes()     */
  GIGAAM_E_UNSUPPORTED = -3, /* shape/dtype this build has no kernel for            */
  GIGAAM_E_HIP = -4          /* a HIP runtime call or launch failed                  */
};

/* Arithmetic of the encoder GEMMs and attention. Residual stream, norms, soft-max,
 * frontend and the CTC head (its weights, its product with the fp32 encoder output, and
 * the log-softmax) are always fp32.                                                  */
enum {
  GIGAAM_F32 = 0,    /* fp32 weights and operands (fp32 MFMA)                         */
  GIGAAM_F16 = 1,    /* fp16 weights and GEMM/attention operands, fp32 accumulate     */
  GIGAAM_BF16 = 2,   /* bf16 weights and operands, fp32 accumulate                    */
  GIGAAM_W8F16 = 3,  /* FFN, attention and pointwise-conv linears stored as int8 with
                        one fp16 scale per group of 64 input weights, dequantised
                        in-kernel to fp16; everything else as GIGAAM_F16             */
  GIGAAM_W6F16 = 4,  /* as GIGAAM_W8F16 with 6-bit weights in [-31, 31]             */
  GIGAAM_W4F16 = 5   /* as GIGAAM_W8F16 with 4-bit weights in [-7, 7]               */
};
/* Weight-only quantisation ("GigaAM MLX port for Mac", section "How precision affects
 * size and speed": a shared scale per group of 64 weights; INT8, INT6 and INT4 variants).
 * Packed device rows: weight k of a row occupies bits [k*b, k*b + b) of the row's
 * little-endian bit string (b = 8, 6, 4; two's complement), rows of K*b/8 bytes; scales
 * fp16 [N][K/64]. A weight is q * scale[n][k / 64].                                    */

/* Largest batch one gigaam_encode call accepts. */
#define GIGAAM_MAX_BATCH 256

typedef struct gigaam_config {
  int32_t n_layers;     /* Conformer blocks (16 for v3, 24 for the multilingual model) */
  int32_t d_model;      /* 768 or 1024; multiple of 64                                 */
  int32_t n_heads;      /* 16; d_model / n_heads must be 48 or 64                      */
  int32_t d_ff;         /* FFN width (4 d_model); multiple of 64                       */
  int32_t conv_kernel;  /* depthwise kernel, odd, <= 63 (31)                           */
  int32_t n_classes;    /* CTC classes including blank; blank id = n_classes - 1      */
  int32_t n_mels;       /* 64   (fixed)                                                */
  int32_t n_fft;        /* 320  (fixed)                                                */
  int32_t win_length;   /* 320  (fixed)                                                */
  int32_t hop_length;   /* 160  (fixed)                                                */
  int32_t sub_kernel;   /* 5    (fixed; padding 2)                                     */
  int32_t sub_stride;   /* 2    (fixed)                                                */
  int32_t dtype;        /* GIGAAM_F32 ... GIGAAM_W4F16                                 */
  float rope_base;      /* 5000                                                        */
  float ln_eps;         /* LayerNorm epsilon (1e-5)                                    */
  float bn_eps;         /* BatchNorm epsilon (1e-5)                                    */
} gigaam_config;

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t gigaam_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* gigaam_last_error(void);

/* Host arithmetic, no GPU: frame counts of one clip of n_samples samples.
 * mel = floor((n - 320)/160) + 1: window 320, hop 160, no centring ("GigaAM v3 MLX"
 * card, Frontend configuration); sub = floor((mel - 1)/2) + 1 and
 * enc = floor((sub - 1)/2) + 1: each of the two Conv1d (kernel 5, stride 2, padding 2)
 * halves the frames, a subsampling factor of 4 (same section; "GigaAM on MLX: the
 * transcripts matched, but the model was broken", What we're porting). The padding is
 * the one that reproduces the printed shapes: 1 s gives 99 mel frames and 25 encoder
 * frames ("GigaAM v3 MLX" card, Selected validation results), 20 s gives 1,999 and about
 * 500 ("GigaAM MLX port for Mac", Where the time goes). Any output pointer may be NULL.
 * Error: GIGAAM_E_INVAL if n_samples < 320 (no complete window).                     */
int gigaam_frames(int32_t n_samples, int32_t* mel_frames, int32_t* sub_frames,
                  int32_t* enc_frames);

/* Validate a configuration (same checks as gigaam_create). */
int gigaam_check_config(const gigaam_config* cfg);

/* ---------------------------------------------------------------------------------
 * Weights.
 * A checkpoint is handed over as one host float32 "canonical" buffer: the tensors
 * listed by gigaam_canonical_entry, concatenated in that order, each in PyTorch layout
 * (Linear [out, in]; Conv1d [out, in, K]; pointwise convs [out, in]; depthwise
 * [channels, K]), holding the checkpoint values exactly (fp16/bf16 values for those
 * dtypes; for GIGAAM_W8F16 / W6F16 / W4F16 the quantised linears appear as
 * "<name>.weight_q" holding integers in [-(2^(b-1)-1), 2^(b-1)-1] and
 * "<name>.weight_scale" [out, in/64] holding fp16 values; out-of-range or non-integer
 * values make gigaam_pack_weights fail with GIGAAM_E_INVAL).
 * gigaam_pack_weights turns it into the device layout (host -> host); the caller
 * copies the packed bytes to the device and passes that pointer to gigaam_create.
 * ------------------------------------------------------------------------------- */

/* Number of canonical tensors and total float count of the canonical buffer. */
int gigaam_canonical_count(const gigaam_config* cfg, int32_t* n_entries, size_t* n_floats);

/* Entry i: name (NUL-terminated, written to name_buf of name_cap bytes), rank (1..3),
 * shape (up to 3 dims) and float offset in the canonical buffer.                     */
int gigaam_canonical_entry(const gigaam_config* cfg, int32_t i, char* name_buf,
                           int32_t name_cap, int32_t* rank, int32_t* shape,
                           size_t* offset_floats);

/* Size in bytes of the packed device blob. */
int gigaam_packed_bytes(const gigaam_config* cfg, size_t* bytes);

/* Host-side repacking: casts (round-to-nearest-even) to the kernel storage type,
 * transposes subsampling convs to [out, K, in], interleaves the pointwise-1 rows so
 * each 64-row group holds 32 value rows followed by their 32 gate rows, concatenates
 * q/k/v. canonical: host float[n_floats]; packed: host buffer of packed_bytes.
 * Errors: GIGAAM_E_INVAL on size mismatch or an int8 value outside [-127, 127].      */
int gigaam_pack_weights(const gigaam_config* cfg, const float* canonical_host,
                        size_t n_floats, void* packed_host, size_t packed_bytes);

/* ---------------------------------------------------------------------------------
 * Frontend tables. The STFT window [win_length] and mel filterbank
 * [n_fft/2 + 1][n_mels] are model data ("port the matrix": "GigaAM on MLX ...",
 * Trap 3). This fills them on the device with the defaults: periodic Hann and an HTK
 * triangular bank on [0, 8000] Hz without normalisation, computed in fp64 on the GPU.
 * window_dev: float[320]; melfb_dev: float[161 * 64] row-major [bin][mel].           */
int gigaam_default_frontend(float* window_dev, float* melfb_dev, void* hip_stream);

/* ---------------------------------------------------------------------------------
 * Model handle.
 * packed_weights_dev: device copy of the gigaam_pack_weights output (256-B aligned).
 * window_dev, melfb_dev: device frontend tables as above (any values allowed).
 * ------------------------------------------------------------------------------- */
typedef struct gigaam_model gigaam_model;

int gigaam_create(const gigaam_config* cfg, const void* packed_weights_dev,
                  const float* window_dev, const float* melfb_dev, gigaam_model** out);
void gigaam_destroy(gigaam_model* model);

/* Bytes of device workspace one call needs for `batch` clips of at most max_samples
 * samples each (an upper bound over all length mixes).                               */
int gigaam_workspace_bytes(const gigaam_model* model, int32_t batch, int32_t max_samples,
                           size_t* bytes);

/* ---------------------------------------------------------------------------------
 * Encode a padded batch: the whole path of the file header for every clip, log-mel
 * frontend ("GigaAM v3 MLX" card, Frontend configuration), two stride-2 Conv1d and the
 * Conformer blocks ("GigaAM on MLX: the transcripts matched, but the model was broken",
 * What we're porting, Trap 1 and Trap 2; "GigaAM MLX port for Mac", What is inside the
 * model), CTC log-softmax and greedy collapse with blank = n_classes - 1 ("GigaAM v3
 * RNNT - MLX" card, Notes for other runtimes). A clip's outputs are those of the clip
 * encoded alone on its valid samples: padding never reaches a valid output (each time
 * convolution sees zeros outside the clip, attention masks the keys past its end).
 *   pcm_dev      float [batch][pcm_stride] 16 kHz samples; clip b uses its first
 *                lengths_host[b] samples (the rest is never read).
 *   lengths_host int32 [batch], each in [320, pcm_stride].
 *   batch        1 .. GIGAAM_MAX_BATCH.
 *   workspace    device scratch of at least gigaam_workspace_bytes(model, batch,
 *                max(lengths)) bytes, 256-B aligned; contents need no initialisation.
 * Outputs (U_b = encoder frames of clip b, U_max = max_b U_b):
 *   log_probs_dev  float [batch][U_max][n_classes] CTC log-probabilities; rows t >= U_b
 *                  are 0.
 *   token_ids_dev  int32 [batch][U_max] greedy CTC tokens of clip b (argmax per frame,
 *                  lowest index on ties, repeats merged, then blanks removed), -1 padded.
 *   n_tokens_dev   int32 [batch] number of tokens of each clip.
 *   frame_ids_dev  int32 [batch][U_max] per-frame argmax, -1 padded; may be NULL.
 *   enc_out_dev    float [batch][U_max][d_model] encoder output; rows t >= U_b are 0;
 *                  may be NULL.
 *   n_frames_host  int32 [batch] receives U_b; may be NULL.
 * Errors: GIGAAM_E_INVAL (null pointer, batch or a length out of range),
 *         GIGAAM_E_WORKSPACE, GIGAAM_E_HIP.                                          */
int gigaam_encode(gigaam_model* model, const float* pcm_dev, const int32_t* lengths_host,
                  int32_t batch, int32_t pcm_stride, void* workspace, size_t workspace_bytes,
                  float* log_probs_dev, int32_t* token_ids_dev, int32_t* n_tokens_dev,
                  int32_t* frame_ids_dev, float* enc_out_dev, int32_t* n_frames_host,
                  void* hip_stream);

/* Allocation-free variant of gigaam_encode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and outputs without the workspace pair. Its workspace is a fixed
 * scratch array of GIGAAM_NOALLOC_SCRATCH_BYTES in the library's own device memory, one
 * per GPU, held until the process ends (for example one clip of up to 30 s at d_model
 * 1024, or any batch whose gigaam_workspace_bytes is at most that size). Calls needing
 * more are refused with GIGAAM_E_WORKSPACE before any launch. The call allocates nothing.
 * Every call on one GPU uses that GPU's single array: calls that overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller. The array keeps the
 * last call's contents; the encode never reads scratch it has not written in the same
 * call, so nothing needs clearing.                                                     */
#define GIGAAM_NOALLOC_SCRATCH_BYTES (64u << 20)
int gigaam_encode_noalloc(gigaam_model* model, const float* pcm_dev, const int32_t* lengths_host,
                          int32_t batch, int32_t pcm_stride, float* log_probs_dev,
                          int32_t* token_ids_dev, int32_t* n_tokens_dev, int32_t* frame_ids_dev,
                          float* enc_out_dev, int32_t* n_frames_host, void* hip_stream);

/* Stage taps for parity diagnostics: run the path up to `stage` and copy that
 * tensor, packed over clips (rows of clip b follow those of clip b-1), as float32:
 *   GIGAAM_STAGE_MEL     [sum_b T_b][n_mels]     log-mel
 *   GIGAAM_STAGE_SUB     [sum_b U_b][d_model]    subsampling output
 *   GIGAAM_STAGE_LAYER+i [sum_b U_b][d_model]    output of Conformer block i
 * out_dev must hold out_floats floats (at least the tensor size).                    */
enum { GIGAAM_STAGE_MEL = 0, GIGAAM_STAGE_SUB = 1, GIGAAM_STAGE_LAYER = 2 };
int gigaam_encode_stage(gigaam_model* model, const float* pcm_dev, const int32_t* lengths_host,
                        int32_t batch, int32_t pcm_stride, void* workspace,
                        size_t workspace_bytes, int32_t stage, float* out_dev,
                        size_t out_floats, void* hip_stream);

/* ---------------------------------------------------------------------------------
 * Diagnostics: the encoder's GEMM kernel on its own,
 *   C[m][n] = sum_k A[m][k] * W[n][k] + bias[n]      (fp32 accumulate, fp32 out)
 * A_dev [M][K] and W_dev [N][K] in the storage type of `dtype` (GIGAAM_F32: float,
 * GIGAAM_F16: fp16, GIGAAM_BF16: bf16; GIGAAM_W8F16 / W6F16 / W4F16: A fp16, W the
 * packed b-bit rows described above with scale_dev [N][K/64] fp16 scales); bias_dev
 * float[N] or NULL; C_dev float [M][N]. A_dev, W_dev and C_dev must be 16-byte aligned.
 * part_dev: float [part_floats] scratch (16-byte aligned) for split-K partial sums, or
 * NULL. With it the kernel splits the K sum across workgroups when the output tiles
 * alone fill less than half the GPU, as the encoder does for small batches: each slice
 * writes fp32 partials and a second kernel adds the slices in order and applies the
 * epilogue. For the quantised dtypes with at least 2048 rows of A, the scratch instead
 * receives the weights expanded to fp16 (N * K * 2 bytes must fit), and the fp16 kernel
 * runs on them, as the encoder does for large batches. slices_host (may be NULL)
 * receives the number of K slices used (1: none).
 * K must be a multiple of 64 (32 for GIGAAM_F32). Errors: GIGAAM_E_INVAL, GIGAAM_E_HIP. */
int gigaam_debug_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A_dev,
                      const void* W_dev, const void* scale_dev, const float* bias_dev,
                      float* C_dev, float* part_dev, size_t part_floats, int32_t* slices_host,
                      void* hip_stream);

/* Diagnostics: one encoder GEMM role on its own, with the A operand mode and the fused
 * epilogue the encoder launches it with, through the same kernel selection:
 *   P[m][n] = sum_k A'[m][k] * W[n][k] + bias[n]           (fp32 accumulate)
 * a_mode:  GIGAAM_GEMM_A_PLAIN  A' = A_dev [M][K];
 *          GIGAAM_GEMM_A_DUAL   A' row m = A_dev row m for output columns n < nsplit and
 *                               A2_dev row m for the others (the q/k/v projection: q and k
 *                               from the rotated LayerNorm output, v from the plain one);
 *                               nsplit a multiple of 128 in (0, N); epilogue STORE only.
 * epilogue: GIGAAM_GEMM_E_STORE C T [M][N]    = T(P)
 *           GIGAAM_GEMM_E_SILU  C T [M][N]    = T(P * sigmoid(P))              (FFN up)
 *           GIGAAM_GEMM_E_GLU   C T [M][N/2]  = T(value * sigmoid(gate)): W's rows come in
 *                               groups of 64, 32 value rows then their 32 gate rows; the
 *                               output column of value row 64 q + j is 32 q + j (N % 64 == 0)
 *           GIGAAM_GEMM_E_RESID C float [M][N] += alpha * P (in place: the residual stream)
 *           GIGAAM_GEMM_E_F32   C float [M][N] = P
 * T = the storage type of `dtype` (GIGAAM_F32: fp32 everything; GIGAAM_F16 / BF16; the
 * quantised dtypes: fp16 A and C, W the packed rows with scale_dev as in
 * gigaam_debug_gemm). A_dev, A2_dev, W_dev, C_dev 16-byte aligned; bias_dev float [N] or
 * NULL; part_dev / part_floats / slices_host as in gigaam_debug_gemm (a split K sum is
 * always finished by the reduce kernel here). shape_request: 0 = the kernel the encoder
 * would choose for these arguments; otherwise one of the GIGAAM_GEMM_DMA_* variants, run
 * instead (measurement of alternatives: fp16 / bf16 or quantised-with-expansion paths
 * only; GLU needs an even number of 32-column blocks per wave, the dual mode a split at
 * a multiple of the tile width). shape_host (may be NULL) receives the kernel shape
 * used, one of GIGAAM_GEMM_REG_* (register-staged loads, 4 waves) or GIGAAM_GEMM_DMA_*
 * (direct-to-LDS pipeline: tile rows x columns, 8 waves unless _W4*: 4 waves; _S3: three
 * k-tile stages, one workgroup per CU, taken when the tiles are few). K must be
 * a multiple of 64 (32 for GIGAAM_F32). Errors: GIGAAM_E_INVAL, GIGAAM_E_HIP.        */
enum { GIGAAM_GEMM_A_PLAIN = 0, GIGAAM_GEMM_A_DUAL = 2 };
enum { GIGAAM_GEMM_E_STORE = 0, GIGAAM_GEMM_E_SILU = 1, GIGAAM_GEMM_E_GLU = 4,
       GIGAAM_GEMM_E_RESID = 5, GIGAAM_GEMM_E_F32 = 6 };
enum { GIGAAM_GEMM_REG_128x64 = 1, GIGAAM_GEMM_REG_128x128 = 2, GIGAAM_GEMM_DMA_256x256 = 3,
       GIGAAM_GEMM_DMA_256x128_K32 = 4, GIGAAM_GEMM_DMA_256x128_K64 = 5,
       GIGAAM_GEMM_DMA_128x128 = 6, GIGAAM_GEMM_DMA_256x192 = 7, GIGAAM_GEMM_DMA_256x128_W4 = 8,
       GIGAAM_GEMM_DMA_256x128_W4S = 9, GIGAAM_GEMM_DMA_128x256 = 10,
       GIGAAM_GEMM_DMA_128x128_S3 = 11 };
int gigaam_debug_gemm_role(int32_t dtype, int32_t a_mode, int32_t epilogue, int32_t M, int32_t N,
                           int32_t K, const void* A_dev, const void* A2_dev, int32_t nsplit,
                           const void* W_dev, const void* scale_dev, const float* bias_dev,
                           float alpha, void* C_dev, float* part_dev, size_t part_floats,
                           int32_t shape_request, int32_t* slices_host, int32_t* shape_host,
                           void* hip_stream);

/* Diagnostics: a fused variant of the macaron FFN for few rows (hidden activations kept on
 * chip), measured against the encoder's two GEMMs, which the encoder uses instead:
 *   x[m][n] += alpha * (sum_j W2[n][j] h[m][j] + b2[n]),
 *   h[m][j]  = T(SiLU(sum_k W1[j][k] y[m][k] + b1[j]))      (the hidden activations rounded
 *                                                          to T, never stored in HBM)
 * dtype GIGAAM_F16 or GIGAAM_BF16 (T); y_dev [M][d], W1_dev [f][d], W2_dev [d][f] in T;
 * (all three 16-byte aligned); b1_dev float [f] or NULL, b2_dev float [d] or NULL; x_dev
 * float [M][d], 16-byte aligned, updated in place;
 * part_dev float scratch (16-byte aligned) of at least (f / 256) * M * d floats.
 * d = 768 or 1024, f a multiple of 256, 1 <= M <= 896. Errors: GIGAAM_E_INVAL, GIGAAM_E_HIP. */
int gigaam_debug_mlp(int32_t dtype, int32_t M, int32_t d, int32_t f, const void* y_dev,
                     const void* W1_dev, const float* b1_dev, const void* W2_dev,
                     const float* b2_dev, float alpha, float* x_dev, float* part_dev,
                     size_t part_floats, void* hip_stream);

/* Diagnostics: the encoder's attention kernel on its own, over packed clips.
 * frames_host int32 [batch]: frames U_b of each clip (>= 1); qkv_dev [sum U_b][3 d_model]
 * holds q | k | v per frame in the storage type of `dtype` (fp32, fp16, bf16;
 * the quantised dtypes = fp16); out_dev [sum U_b][d_model] the same type. qkv_dev and
 * out_dev must be 16-byte aligned (the kernel moves 16 bytes per access). d_model / n_heads must
 * be 48 or 64. workspace: device memory of at least
 *   20 * (batch + 1) + 36 * sum U_b + 4096 bytes (256-B aligned).
 * Errors: GIGAAM_E_INVAL, GIGAAM_E_WORKSPACE, GIGAAM_E_UNSUPPORTED, GIGAAM_E_HIP.        */
int gigaam_debug_attention(int32_t dtype, int32_t d_model, int32_t n_heads, int32_t batch,
                           const int32_t* frames_host, const void* qkv_dev, void* out_dev,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------------
 * RNNT head ("GigaAM on MLX ...", section "What we're porting": a single-layer LSTM of
 * size 320 plus a joint network; "GigaAM v3 RNNT - MLX" card: character model with 33
 * letters + blank, sequential greedy decoding; "Notes for other runtimes": the LSTM
 * bias is bias_ih + bias_hh and blank = len(vocabulary)). It decodes the encoder output
 * that gigaam_encode writes to enc_out.
 *
 *   prediction network: x = embed[previous symbol] (blank at the start, zero state),
 *                       PyTorch LSTM, gates (i, f, g, o) = W_ih x + W_hh h + b_ih + b_hh
 *   joint:              logits = W_out relu(W_enc e_t + b_enc + W_pred h + b_pred) + b_out
 *   greedy decoding:    per frame, argmax of the joint (lowest index on ties); blank
 *                       moves to the next frame, another symbol is emitted, advances
 *                       the prediction network and stays on the frame, at most
 *                       max_symbols emissions per frame.
 * ------------------------------------------------------------------------------- */
typedef struct gigaam_rnnt_config {
  int32_t d_model;       /* encoder width (768 / 1024); multiple of 64                 */
  int32_t n_classes;     /* vocabulary + blank, blank id = n_classes - 1; 2 .. 8192    */
  int32_t pred_hidden;   /* LSTM width (320); multiple of 64, <= 1024                  */
  int32_t joint_hidden;  /* joint width (320); multiple of 64, <= 1024                 */
  int32_t max_symbols;   /* emissions per encoder frame at most, 1 .. 64               */
  int32_t dtype;         /* GIGAAM_F32 / F16 / BF16: storage of the head's matrices;
                            every product accumulates in fp32, state stays fp32       */
} gigaam_rnnt_config;

typedef struct gigaam_rnnt gigaam_rnnt;

int gigaam_rnnt_check_config(const gigaam_rnnt_config* cfg);

/* Canonical host float32 buffer, as for the encoder, with the tensors (PyTorch layout)
 * "rnnt.embed.weight" [n_classes, P], "rnnt.lstm.weight_ih_l0" [4P, P],
 * "rnnt.lstm.weight_hh_l0" [4P, P], "rnnt.lstm.bias_ih_l0" [4P], "rnnt.lstm.bias_hh_l0"
 * [4P], "rnnt.joint.enc.weight" [J, d], "rnnt.joint.enc.bias" [J],
 * "rnnt.joint.pred.weight" [J, P], "rnnt.joint.pred.bias" [J], "rnnt.joint.out.weight"
 * [n_classes, J], "rnnt.joint.out.bias" [n_classes], in that order.                  */
int gigaam_rnnt_canonical_count(const gigaam_rnnt_config* cfg, int32_t* n_entries,
                                size_t* n_floats);
int gigaam_rnnt_canonical_entry(const gigaam_rnnt_config* cfg, int32_t i, char* name_buf,
                                int32_t name_cap, int32_t* rank, int32_t* shape,
                                size_t* offset_floats);
int gigaam_rnnt_packed_bytes(const gigaam_rnnt_config* cfg, size_t* bytes);
/* Host repacking: casts to the storage type (round-to-nearest-even), sums the two LSTM
 * biases, stores W_hh, W_pred and W_out transposed. Errors: GIGAAM_E_INVAL on sizes.  */
int gigaam_rnnt_pack_weights(const gigaam_rnnt_config* cfg, const float* canonical_host,
                             size_t n_floats, void* packed_host, size_t packed_bytes);

/* packed_dev: device copy of the packed blob (256-B aligned), borrowed by the handle. */
int gigaam_rnnt_create(const gigaam_rnnt_config* cfg, const void* packed_dev,
                       gigaam_rnnt** out);
void gigaam_rnnt_destroy(gigaam_rnnt* head);

/* Device workspace for `batch` clips whose encoder output rows are enc_stride apart. */
int gigaam_rnnt_workspace_bytes(const gigaam_rnnt* head, int32_t batch, int32_t enc_stride,
                                size_t* bytes);

/* Greedy RNNT decoding of a padded batch of encoder outputs.
 *   enc_dev          float [batch][enc_stride][d_model] (gigaam_encode's enc_out with
 *                    enc_stride = U_max); clip b uses its first frames_host[b] rows.
 *   frames_host      int32 [batch], each in [1, enc_stride].
 *   tokens_dev       int32 [batch][max_tokens]: emitted symbols in order, -1 after them.
 *   token_frames_dev int32 [batch][max_tokens]: frame of each symbol, -1 after; or NULL.
 *   n_tokens_dev     int32 [batch]; negative marks a clip whose cluster gave up (below).
 *   max_tokens       >= enc_stride * max_symbols (the most a clip can emit).
 * The whole sequential loop runs on the GPU (the stream is not synchronised). When the
 * batch leaves enough compute units ("GigaAM v3 MLX" card, section "Long-form stage
 * breakdown": the decoding loop is the sequential bottleneck), each clip gets a cluster of
 * G cooperatively launched workgroups (G a power of two, batch * G within the CUs, P and J
 * multiples of G), each holding 1/G of W_hh, W_pred and W_out in LDS; the members exchange
 * partial logits per decision and h slices per emission through the workspace. A member
 * that waits for a partner beyond a fixed bound (tens of milliseconds; a partner that was
 * never scheduled) ends its clip with a negative n_tokens instead of hanging. Otherwise one
 * workgroup per clip. Both give the oracle's decisions within rounding (the sums are
 * taken in a different order). Errors: GIGAAM_E_INVAL, GIGAAM_E_WORKSPACE, GIGAAM_E_HIP. */
int gigaam_rnnt_decode(gigaam_rnnt* head, const float* enc_dev, int32_t enc_stride,
                       const int32_t* frames_host, int32_t batch, void* workspace,
                       size_t workspace_bytes, int32_t* tokens_dev, int32_t* token_frames_dev,
                       int32_t* n_tokens_dev, int32_t max_tokens, void* hip_stream);

/* The cluster size gigaam_rnnt_decode would use for `batch` clips on the current device
 * (1: one workgroup per clip), and a cap on it for this handle (max_members in [1, 64];
 * 1 forces one workgroup per clip; the default cap is 64). Errors: GIGAAM_E_INVAL.      */
int gigaam_rnnt_cluster_size(const gigaam_rnnt* head, int32_t batch, int32_t* members);
int gigaam_rnnt_set_max_cluster(gigaam_rnnt* head, int32_t max_members);

/* ---------------------------------------------------------------------------------
 * Pseudo-streaming ("GigaAM on MLX ...", section "Streaming: honestly, it's
 * pseudo-streaming"): the model is not a streaming model, so a stream keeps a growing
 * buffer of the audio received so far and every step re-encodes all of it, but never
 * more than the last `window` samples (30 s = 480000 in the port); a step costs more as
 * the buffer grows.
 *
 * The caller owns a device ring of `capacity` float samples (capacity >= 2 * window) and
 * a gigaam_stream_state, a plain host struct. gigaam_stream_push appends samples; when the
 * ring has no room after the window, the retained samples are first moved to its start
 * (a device copy of at most `window` samples, once per capacity - window samples pushed).
 * gigaam_stream_step encodes the current window with gigaam_encode (batch 1); its
 * workspace is gigaam_workspace_bytes(model, 1, window) and serves every step.       */
typedef struct gigaam_stream_state {
  int64_t total;      /* samples pushed since gigaam_stream_init                      */
  int32_t window;     /* most samples one step encodes (>= 320)                         */
  int32_t capacity;   /* samples the device ring holds (>= 2 * window)                  */
  int32_t start;      /* ring offset of the window's first sample                       */
  int32_t length;     /* samples in the window: min(total, window)                      */
} gigaam_stream_state;

/* What a push of n samples does to the ring, computed on the host only:
 *   move_len samples at ring offset move_src go to offset 0 (move_len may be 0), then
 *   the last append_len = min(n, window) samples of the pushed chunk go to offset
 *   append_at; the new window is [start, start + length) of the updated state.       */
typedef struct gigaam_stream_plan {
  int32_t move_src, move_len;
  int32_t append_at, append_len, skip;   /* skip = n - append_len leading samples dropped */
  int32_t start, length;                 /* window after the push                          */
  int64_t total;
} gigaam_stream_plan;

/* Initialise a state: window in [320, 2^30 / 2], capacity >= 2 * window.
 * Errors: GIGAAM_E_INVAL.                                                             */
int gigaam_stream_init(gigaam_stream_state* state, int32_t window, int32_t capacity);

/* Plan a push of n >= 0 samples (no device work, state unchanged). Errors: GIGAAM_E_INVAL. */
int gigaam_stream_plan_push(const gigaam_stream_state* state, int32_t n,
                            gigaam_stream_plan* plan);

/* Append n samples from pcm_dev (device, float) to the ring ring_dev (device, float
 * [capacity]) with the library's copy kernel on hip_stream, then update the state (only
 * when every launch succeeded). pcm_dev may be NULL when n == 0.
 * Errors: GIGAAM_E_INVAL, GIGAAM_E_HIP.                                              */
int gigaam_stream_push(gigaam_stream_state* state, float* ring_dev, const float* pcm_dev,
                       int32_t n, void* hip_stream);

/* Encode the current window: gigaam_encode of ring_dev + start with one clip of
 * `length` samples; the outputs are those of gigaam_encode for batch 1 (U = frames of
 * the window). Errors: GIGAAM_E_INVAL (fewer than 320 samples buffered, null pointer),
 * GIGAAM_E_WORKSPACE, GIGAAM_E_HIP.                                                   */
int gigaam_stream_step(gigaam_model* model, const gigaam_stream_state* state,
                       const float* ring_dev, void* workspace, size_t workspace_bytes,
                       float* log_probs_dev, int32_t* token_ids_dev, int32_t* n_tokens_dev,
                       int32_t* frame_ids_dev, float* enc_out_dev, int32_t* n_frames_host,
                       void* hip_stream);

/* Diagnostics: per-kernel timing. Between gigaam_profile_start and _stop every launch
 * of gigaam_encode is bracketed by HIP events recorded on the caller's stream (the
 * events add a little stream overhead). gigaam_profile_report waits for those events
 * and writes a JSON array of {name, launches, total_ms, avg_us, min_us, max_us} per
 * kernel role into buf (cap bytes), then clears the record. Process-wide state, one
 * profiling thread at a time. Errors: GIGAAM_E_INVAL (buffer too small), GIGAAM_E_HIP. */
int gigaam_profile_start(void);
int gigaam_profile_stop(void);
int gigaam_profile_report(char* buf, size_t cap);

#ifdef __cplusplus
}
#endif
#endif /* GIGAAM_H */
