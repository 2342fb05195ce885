// Host side of the RNNT head's C ABI (include/gigaam.h): configuration checks, the
// canonical weight list, repacking, workspace planning and the launch sequence
// (two GEMMs, then the greedy decoding kernel: a cooperative cluster of workgroups per clip
// when the batch leaves enough CUs, else one workgroup per clip) on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "gigaam.h"
#include "host.h"
#include "kernels.h"

using namespace gg;

namespace {

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct RnntLayout {
  size_t emb, wih, bsum, whhT, we, be, wpT, bp, woT, bo, total;
  int Cp;
  int es;
};

RnntLayout rnnt_layout(const gigaam_rnnt_config& c) {
  RnntLayout L;
  L.es = c.dtype == GIGAAM_F32 ? 4 : 2;
  L.Cp = (c.n_classes + 7) / 8 * 8;
  const size_t P = c.pred_hidden, J = c.joint_hidden, C = c.n_classes, d = c.d_model;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  L.emb = take(C * P * L.es);
  L.wih = take(4 * P * P * L.es);
  L.bsum = take(4 * P * 4);
  L.whhT = take(P * 4 * P * L.es);
  L.we = take(J * d * L.es);
  L.be = take(J * 4);
  L.wpT = take(P * J * L.es);
  L.bp = take(J * 4);
  L.woT = take(J * L.Cp * L.es);
  L.bo = take(C * 4);
  L.total = off;
  return L;
}

struct REntry { const char* name; int rank; int s0, s1; };

std::vector<REntry> rnnt_entries(const gigaam_rnnt_config& c) {
  const int P = c.pred_hidden, J = c.joint_hidden, C = c.n_classes, d = c.d_model;
  return {{"rnnt.embed.weight", 2, C, P},      {"rnnt.lstm.weight_ih_l0", 2, 4 * P, P},
          {"rnnt.lstm.weight_hh_l0", 2, 4 * P, P}, {"rnnt.lstm.bias_ih_l0", 1, 4 * P, 0},
          {"rnnt.lstm.bias_hh_l0", 1, 4 * P, 0}, {"rnnt.joint.enc.weight", 2, J, d},
          {"rnnt.joint.enc.bias", 1, J, 0},    {"rnnt.joint.pred.weight", 2, J, P},
          {"rnnt.joint.pred.bias", 1, J, 0},   {"rnnt.joint.out.weight", 2, C, J},
          {"rnnt.joint.out.bias", 1, C, 0}};
}

size_t count_of(const REntry& e) { return (size_t)e.s0 * (e.rank > 1 ? e.s1 : 1); }

}  // namespace

struct gigaam_rnnt {
  gigaam_rnnt_config cfg;
  const char* w;
  RnntLayout L;
  int max_cluster;
};

extern "C" int gigaam_rnnt_check_config(const gigaam_rnnt_config* c) {
  if (!c) return fail(GIGAAM_E_INVAL, "NULL config");
  if (c->d_model < 64 || c->d_model % 64 || c->d_model > 4096)
    return fail(GIGAAM_E_INVAL, "rnnt d_model %d not a multiple of 64 in [64, 4096]", c->d_model);
  if (c->n_classes < 2 || c->n_classes > 8192) return fail(GIGAAM_E_INVAL, "rnnt n_classes %d", c->n_classes);
  if (c->pred_hidden < 64 || c->pred_hidden % 64 || c->pred_hidden > 1024)
    return fail(GIGAAM_E_INVAL, "pred_hidden %d not a multiple of 64 in [64, 1024]", c->pred_hidden);
  if (c->joint_hidden < 64 || c->joint_hidden % 64 || c->joint_hidden > 1024)
    return fail(GIGAAM_E_INVAL, "joint_hidden %d not a multiple of 64 in [64, 1024]", c->joint_hidden);
  if (c->max_symbols < 1 || c->max_symbols > 64) return fail(GIGAAM_E_INVAL, "max_symbols %d", c->max_symbols);
  if (c->dtype != GIGAAM_F32 && c->dtype != GIGAAM_F16 && c->dtype != GIGAAM_BF16)
    return fail(GIGAAM_E_INVAL, "rnnt dtype %d (F32, F16 or BF16)", c->dtype);
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_canonical_count(const gigaam_rnnt_config* cfg, int32_t* n_entries,
                                           size_t* n_floats) {
  int rc = gigaam_rnnt_check_config(cfg);
  if (rc) return rc;
  const auto e = rnnt_entries(*cfg);
  size_t n = 0;
  for (const auto& x : e) n += count_of(x);
  if (n_entries) *n_entries = (int32_t)e.size();
  if (n_floats) *n_floats = n;
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_canonical_entry(const gigaam_rnnt_config* cfg, int32_t i, char* name_buf,
                                           int32_t name_cap, int32_t* rank, int32_t* shape,
                                           size_t* offset_floats) {
  int rc = gigaam_rnnt_check_config(cfg);
  if (rc) return rc;
  const auto e = rnnt_entries(*cfg);
  if (i < 0 || i >= (int32_t)e.size()) return fail(GIGAAM_E_INVAL, "entry %d out of range", i);
  size_t off = 0;
  for (int k = 0; k < i; ++k) off += count_of(e[k]);
  if (name_buf) {
    if ((int32_t)std::strlen(e[i].name) + 1 > name_cap) return fail(GIGAAM_E_INVAL, "name buffer too small");
    std::strcpy(name_buf, e[i].name);
  }
  if (rank) *rank = e[i].rank;
  if (shape) { shape[0] = e[i].s0; shape[1] = e[i].rank > 1 ? e[i].s1 : 0; shape[2] = 0; }
  if (offset_floats) *offset_floats = off;
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_packed_bytes(const gigaam_rnnt_config* cfg, size_t* bytes) {
  int rc = gigaam_rnnt_check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(GIGAAM_E_INVAL, "NULL bytes");
  *bytes = rnnt_layout(*cfg).total;
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_pack_weights(const gigaam_rnnt_config* cfg, const float* canonical,
                                        size_t n_floats, void* packed, size_t packed_bytes) {
  int rc = gigaam_rnnt_check_config(cfg);
  if (rc) return rc;
  const gigaam_rnnt_config& c = *cfg;
  const RnntLayout L = rnnt_layout(c);
  size_t want = 0;
  const auto e = rnnt_entries(c);
  for (const auto& x : e) want += count_of(x);
  if (!canonical || !packed) return fail(GIGAAM_E_INVAL, "NULL buffer");
  if (n_floats != want) return fail(GIGAAM_E_INVAL, "canonical buffer has %zu floats, expected %zu", n_floats, want);
  if (packed_bytes < L.total) return fail(GIGAAM_E_INVAL, "packed buffer %zu < %zu bytes", packed_bytes, L.total);
  char* dst = (char*)packed;
  std::memset(dst, 0, L.total);
  std::vector<const float*> src;
  size_t off = 0;
  for (const auto& x : e) { src.push_back(canonical + off); off += count_of(x); }
  auto put_w = [&](size_t base, size_t idx, float v) {
    if (L.es == 4) { std::memcpy(dst + base + idx * 4, &v, 4); return; }
    const uint16_t hb = c.dtype == GIGAAM_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
    std::memcpy(dst + base + idx * 2, &hb, 2);
  };
  auto put_f = [&](size_t base, size_t idx, float v) { std::memcpy(dst + base + idx * 4, &v, 4); };
  const size_t P = c.pred_hidden, J = c.joint_hidden, C = c.n_classes, d = c.d_model;
  for (size_t i = 0; i < C * P; ++i) put_w(L.emb, i, src[0][i]);
  for (size_t i = 0; i < 4 * P * P; ++i) put_w(L.wih, i, src[1][i]);
  for (size_t i = 0; i < 4 * P; ++i) put_f(L.bsum, i, src[3][i] + src[4][i]);
  for (size_t g = 0; g < 4 * P; ++g)                 // W_hh [4P][P] -> [P][4P]
    for (size_t k = 0; k < P; ++k) put_w(L.whhT, k * 4 * P + g, src[2][g * P + k]);
  for (size_t i = 0; i < J * d; ++i) put_w(L.we, i, src[5][i]);
  for (size_t j = 0; j < J; ++j) put_f(L.be, j, src[6][j]);
  for (size_t j = 0; j < J; ++j)                     // W_pred [J][P] -> [P][J]
    for (size_t k = 0; k < P; ++k) put_w(L.wpT, k * J + j, src[7][j * P + k]);
  for (size_t j = 0; j < J; ++j) put_f(L.bp, j, src[8][j]);
  for (size_t v = 0; v < C; ++v)                     // W_out [C][J] -> [J][Cp]
    for (size_t j = 0; j < J; ++j) put_w(L.woT, j * L.Cp + v, src[9][v * J + j]);
  for (size_t v = 0; v < C; ++v) put_f(L.bo, v, src[10][v]);
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_create(const gigaam_rnnt_config* cfg, const void* packed_dev,
                                  gigaam_rnnt** out) {
  int rc = gigaam_rnnt_check_config(cfg);
  if (rc) return rc;
  if (!packed_dev || !out) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if ((uintptr_t)packed_dev & 255) return fail(GIGAAM_E_INVAL, "packed weights not 256-B aligned");
  const RnntLayout L = rnnt_layout(*cfg);
  if (rnnt_lds_bytes((DType)cfg->dtype, cfg->pred_hidden, cfg->joint_hidden, L.Cp, false) > 160 * 1024)
    return fail(GIGAAM_E_UNSUPPORTED, "RNNT state does not fit the 160 KiB of LDS");
  gigaam_rnnt* h = new gigaam_rnnt;
  h->cfg = *cfg;
  h->w = (const char*)packed_dev;
  h->L = L;
  h->max_cluster = 64;
  *out = h;
  return GIGAAM_OK;
}

extern "C" void gigaam_rnnt_destroy(gigaam_rnnt* head) { delete head; }

namespace {
// cluster members per clip the workspace is sized for: the clustered grid (clips in groups
// of 8) within two workgroups on each of 256 CUs, G <= 64 (the launch itself checks the
// occupancy of the device it runs on)
int rnnt_gmax(int batch) {
  int g = 1;
  while (g < 64 && rnnt_cl_grid(batch, 2 * g) <= 512) g *= 2;
  return g;
}
struct RnntWs { size_t fenc, gemb, xch, total; int gmax; };
RnntWs rnnt_ws(const gigaam_rnnt_config& c, int batch, int stride) {
  RnntWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  const int Cp = (c.n_classes + 7) / 8 * 8;
  w.gmax = rnnt_gmax(batch);
  w.fenc = take((size_t)batch * stride * c.joint_hidden * 4);
  w.gemb = take((size_t)c.n_classes * 4 * c.pred_hidden * 4);
  // the clustered decoder's exchange words: partial logits, then h slices, two slots each
  w.xch = take(w.gmax > 1 ? ((size_t)batch * 2 * ((size_t)w.gmax * Cp + c.pred_hidden) + (size_t)batch * w.gmax) * 8
                          : 0);
  w.total = off;
  return w;
}
}  // namespace

extern "C" int gigaam_rnnt_set_max_cluster(gigaam_rnnt* head, int32_t max_members) {
  if (!head) return fail(GIGAAM_E_INVAL, "head is NULL");
  if (max_members < 1 || max_members > 64) return fail(GIGAAM_E_INVAL, "max_members %d outside [1, 64]", max_members);
  head->max_cluster = max_members;
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_cluster_size(const gigaam_rnnt* head, int32_t batch, int32_t* members) {
  if (!head || !members) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d", batch);
  const gigaam_rnnt_config& c = head->cfg;
  *members = rnnt_cluster_size((DType)c.dtype, c.pred_hidden, c.joint_hidden, head->L.Cp, batch,
                               std::min(head->max_cluster, rnnt_gmax(batch)));
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_workspace_bytes(const gigaam_rnnt* head, int32_t batch, int32_t enc_stride,
                                           size_t* bytes) {
  if (!head || !bytes) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d", batch);
  if (enc_stride < 1) return fail(GIGAAM_E_INVAL, "enc_stride %d", enc_stride);
  *bytes = rnnt_ws(head->cfg, batch, enc_stride).total;
  return GIGAAM_OK;
}

extern "C" int gigaam_rnnt_decode(gigaam_rnnt* head, const float* enc_dev, int32_t enc_stride,
                                  const int32_t* frames_host, int32_t batch, void* workspace,
                                  size_t workspace_bytes, int32_t* tokens_dev,
                                  int32_t* token_frames_dev, int32_t* n_tokens_dev,
                                  int32_t max_tokens, void* hip_stream) {
  if (!head) return fail(GIGAAM_E_INVAL, "head is NULL");
  const gigaam_rnnt_config& c = head->cfg;
  if (!enc_dev || !frames_host || !workspace || !tokens_dev || !n_tokens_dev)
    return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d", batch);
  if (enc_stride < 1) return fail(GIGAAM_E_INVAL, "enc_stride %d", enc_stride);
  for (int b = 0; b < batch; ++b)
    if (frames_host[b] < 1 || frames_host[b] > enc_stride)
      return fail(GIGAAM_E_INVAL, "frames[%d] = %d outside [1, %d]", b, frames_host[b], enc_stride);
  if ((long)max_tokens < (long)enc_stride * c.max_symbols)
    return fail(GIGAAM_E_INVAL, "max_tokens %d < enc_stride * max_symbols", max_tokens);
  if ((uintptr_t)workspace & 255) return fail(GIGAAM_E_INVAL, "workspace not 256-B aligned");
  const RnntWs w = rnnt_ws(c, batch, enc_stride);
  if (workspace_bytes < w.total)
    return fail(GIGAAM_E_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, w.total);
  const DType dt = (DType)c.dtype;
  const RnntLayout& L = head->L;
  const char* Wp = head->w;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)hip_stream;
  const int P = c.pred_hidden, J = c.joint_hidden, C = c.n_classes;

  // fenc = enc W_enc^T + b_enc over every padded row (fp32 encoder output, staged to T)
  GemmParams g1;
  std::memset(&g1, 0, sizeof g1);
  g1.M = batch * enc_stride; g1.N = J; g1.K = c.d_model;
  g1.A = enc_dev; g1.lda = c.d_model; g1.W = Wp + L.we; g1.ldw = c.d_model;
  g1.bias = (const float*)(Wp + L.be); g1.C = ws + w.fenc; g1.ldc = J; g1.alpha = 1.f;
  HIP_TRY(launch_gemm(dt, 0, A_F32, E_F32, g1, s));
  // gemb = embed W_ih^T + (b_ih + b_hh) for every symbol
  GemmParams g2;
  std::memset(&g2, 0, sizeof g2);
  g2.M = C; g2.N = 4 * P; g2.K = P;
  g2.A = Wp + L.emb; g2.lda = P; g2.W = Wp + L.wih; g2.ldw = P;
  g2.bias = (const float*)(Wp + L.bsum); g2.C = ws + w.gemb; g2.ldc = 4 * P; g2.alpha = 1.f;
  HIP_TRY(launch_gemm(dt, 0, A_PLAIN, E_F32, g2, s));

  RnntParams rp;
  std::memset(&rp, 0, sizeof rp);
  rp.fenc = (const float*)(ws + w.fenc);
  rp.gemb = (const float*)(ws + w.gemb);
  rp.whhT = Wp + L.whhT; rp.wpT = Wp + L.wpT; rp.bp = (const float*)(Wp + L.bp);
  rp.woT = Wp + L.woT; rp.bo = (const float*)(Wp + L.bo);
  rp.P = P; rp.J = J; rp.C = C; rp.Cp = L.Cp; rp.max_symbols = c.max_symbols;
  rp.stride = enc_stride; rp.max_tokens = max_tokens;
  // W_out^T stays in LDS when that keeps the workgroup within 96 KiB
  rp.wo_lds = rnnt_lds_bytes(dt, P, J, L.Cp, true) <= 96 * 1024;
  rp.tokens = tokens_dev; rp.tframes = token_frames_dev; rp.ntok = n_tokens_dev;
  for (int b = 0; b < batch; ++b) rp.frames[b] = frames_host[b];
  const int G = rnnt_cluster_size(dt, P, J, L.Cp, batch, std::min(head->max_cluster, w.gmax));
  if (G >= 2) {
    RnntCluster q;
    q.xl = (unsigned long long*)(ws + w.xch);
    q.xh = q.xl + (size_t)batch * 2 * G * L.Cp;
    q.xc = q.xh + (size_t)batch * 2 * P;
    q.xbytes = (int)(((size_t)batch * 2 * ((size_t)G * L.Cp + P) + (size_t)batch * G) * 8);
    q.batch = batch;
    q.G = G;
    q.wo_lds = rnnt_cl_lds_bytes(dt, P, J, L.Cp, G, true) <= 160 * 1024;
    q.spin_limit = 1 << 16;
    HIP_TRY(launch_rnnt_cluster(dt, rp, q, batch, s));
  } else {
    HIP_TRY(launch_rnnt_decode(dt, rp, batch, s));
  }
  return GIGAAM_OK;
}
