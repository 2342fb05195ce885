// Host side of the C ABI declared in include/gigaam.h: argument validation, frame
// arithmetic, weight repacking, workspace planning and the launch sequence of one
// encoder forward pass on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gigaam.h"
#include "host.h"
#include "kernels.h"

using namespace gg;

// --------------------------------------------------------------------------- errors
static thread_local std::string g_err;

int gg::fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// --------------------------------------------------------------------------- profiler
// Diagnostics only: when on, every launch of an encode is bracketed by HIP events on the
// caller's stream; gigaam_profile_report aggregates them per kernel role.
namespace {
struct ProfRec { const char* name; hipEvent_t a, b; };
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<ProfRec> recs;
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Profiler g_prof;
}  // namespace

// Launch `expr` (a hipError_t expression), timing it when the profiler is on.
// (profiling is best effort: a launch whose events fail to record is simply not timed)
#define LAUNCH(name, expr)                                                              \
  do {                                                                                  \
    hipEvent_t a_ = g_prof.on ? g_prof.next() : nullptr;                                \
    if (a_ && hipEventRecord(a_, s) != hipSuccess) a_ = nullptr;                        \
    HIP_TRY(expr);                                                                      \
    if (a_) {                                                                           \
      hipEvent_t b_ = g_prof.next();                                                    \
      if (b_ && hipEventRecord(b_, s) == hipSuccess) g_prof.recs.push_back({name, a_, b_}); \
    }                                                                                   \
  } while (0)

extern "C" int gigaam_profile_start(void) {
  g_prof.used = 0;
  g_prof.recs.clear();
  g_prof.on = true;
  return GIGAAM_OK;
}

extern "C" int gigaam_profile_stop(void) {
  g_prof.on = false;
  return GIGAAM_OK;
}

extern "C" int gigaam_profile_report(char* buf, size_t cap) {
  if (!buf || cap == 0) return fail(GIGAAM_E_INVAL, "NULL report buffer");
  struct Agg { std::string name; int n; double tot, mn, mx; };
  std::vector<Agg> agg;
  for (const ProfRec& r : g_prof.recs) {
    float ms = 0.f;
    HIP_TRY(hipEventSynchronize(r.b));
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    Agg* a = nullptr;
    for (Agg& x : agg) if (x.name == r.name) a = &x;
    if (!a) { agg.push_back({r.name, 0, 0.0, 1e30, 0.0}); a = &agg.back(); }
    a->n += 1; a->tot += ms; a->mn = ms < a->mn ? ms : a->mn; a->mx = ms > a->mx ? ms : a->mx;
  }
  std::string js = "[";
  for (size_t i = 0; i < agg.size(); ++i) {
    char line[256];
    snprintf(line, sizeof line, "%s{\"name\": \"%s\", \"launches\": %d, \"total_ms\": %.6f, "
             "\"avg_us\": %.3f, \"min_us\": %.3f, \"max_us\": %.3f}", i ? ", " : "",
             agg[i].name.c_str(), agg[i].n, agg[i].tot, 1e3 * agg[i].tot / agg[i].n,
             1e3 * agg[i].mn, 1e3 * agg[i].mx);
    js += line;
  }
  js += "]";
  g_prof.used = 0;
  g_prof.recs.clear();
  if (js.size() + 1 > cap) return fail(GIGAAM_E_INVAL, "report needs %zu bytes", js.size() + 1);
  std::memcpy(buf, js.c_str(), js.size() + 1);
  return GIGAAM_OK;
}

extern "C" int32_t gigaam_version(void) { return 100; }
extern "C" const char* gigaam_last_error(void) { return g_err.c_str(); }

// --------------------------------------------------------------------------- casts
// Round-to-nearest-even fp32 -> fp16 / bf16 bit patterns (host packing).
uint16_t gg::f32_to_f16_bits(float v) {
  uint32_t x;
  std::memcpy(&x, &v, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);          // rounds to >= 65520
  if (ax < 0x38800000u) {                                             // fp16 subnormal or 0
    if (ax < 0x33000000u) return (uint16_t)sign;                      // < 2^-25: rounds to 0
    const uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
    const int e = (int)(ax >> 23);                                    // 102..112
    const int shift = 126 - e;                                        // 14..24
    uint32_t r = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u), halfway = 1u << (shift - 1);
    if (rem > halfway || (rem == halfway && (r & 1u))) ++r;
    return (uint16_t)(sign | r);
  }
  uint32_t r = ((ax >> 13) - (112u << 10));
  const uint32_t rem = ax & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  return (uint16_t)(sign | r);
}

uint16_t gg::f32_to_bf16_bits(float v) {
  uint32_t x;
  std::memcpy(&x, &v, 4);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

// --------------------------------------------------------------------------- frames
static void frame_counts(int n, int& T, int& S, int& U) {
  T = (n - 320) / 160 + 1;        // un-centred STFT, window 320, hop 160
  S = (T + 2 * 2 - 5) / 2 + 1;    // Conv1d k5 s2 p2
  U = (S + 2 * 2 - 5) / 2 + 1;
}

extern "C" int gigaam_frames(int32_t n_samples, int32_t* mel, int32_t* sub, int32_t* enc) {
  if (n_samples < 320) return fail(GIGAAM_E_INVAL, "n_samples %d < 320 (one window)", n_samples);
  int T, S, U;
  frame_counts(n_samples, T, S, U);
  if (mel) *mel = T;
  if (sub) *sub = S;
  if (enc) *enc = U;
  return GIGAAM_OK;
}

// --------------------------------------------------------------------------- config
extern "C" int gigaam_check_config(const gigaam_config* c) {
  if (!c) return fail(GIGAAM_E_INVAL, "config is NULL");
  if (c->n_mels != 64 || c->n_fft != 320 || c->win_length != 320 || c->hop_length != 160)
    return fail(GIGAAM_E_UNSUPPORTED, "frontend must be 64 mels, FFT/window 320, hop 160");
  if (c->sub_kernel != 5 || c->sub_stride != 2)
    return fail(GIGAAM_E_UNSUPPORTED, "subsampling must be Conv1d kernel 5 stride 2");
  if (c->n_layers < 1 || c->n_layers > 128) return fail(GIGAAM_E_INVAL, "n_layers %d", c->n_layers);
  if (c->d_model != 768 && c->d_model != 1024)
    return fail(GIGAAM_E_UNSUPPORTED, "d_model %d (kernels built for 768 and 1024)", c->d_model);
  if (c->n_heads != 16) return fail(GIGAAM_E_UNSUPPORTED, "n_heads %d (16 supported)", c->n_heads);
  if (c->d_ff < 128 || c->d_ff % 128) return fail(GIGAAM_E_UNSUPPORTED, "d_ff %d not a multiple of 128", c->d_ff);
  if (c->conv_kernel != 31 && c->conv_kernel != 15 && c->conv_kernel != 5)
    return fail(GIGAAM_E_UNSUPPORTED, "conv_kernel %d (5, 15, 31 built)", c->conv_kernel);
  if (c->n_classes < 2 || c->n_classes > 8192) return fail(GIGAAM_E_INVAL, "n_classes %d", c->n_classes);
  if (c->dtype < GIGAAM_F32 || c->dtype > GIGAAM_W4F16) return fail(GIGAAM_E_INVAL, "dtype %d", c->dtype);
  if (!(c->rope_base > 0.f) || !(c->ln_eps > 0.f) || !(c->bn_eps > 0.f))
    return fail(GIGAAM_E_INVAL, "rope_base / eps must be positive");
  return GIGAAM_OK;
}

// bits of the packed quantised linears of a dtype (0: stored in the operand type)
static int qbits_of(int dtype) {
  return dtype == GIGAAM_W8F16 ? 8 : dtype == GIGAAM_W6F16 ? 6 : dtype == GIGAAM_W4F16 ? 4 : 0;
}

// --------------------------------------------------------------------------- canonical list
namespace {

struct Entry {
  std::string name;
  int rank;
  int shape[3];
  size_t offset;   // floats
  size_t count;
};

const char* kQuantized[] = {"ff1.linear1", "ff1.linear2", "att.linear_q", "att.linear_k",
                            "att.linear_v", "att.linear_out", "conv.pointwise1",
                            "conv.pointwise2", "ff2.linear1", "ff2.linear2"};

std::vector<Entry> canonical(const gigaam_config& c) {
  std::vector<Entry> e;
  size_t off = 0;
  auto add = [&](const std::string& n, int r, int a, int b = 0, int d = 0) {
    Entry x{n, r, {a, b, d}, off, (size_t)a * (r > 1 ? b : 1) * (r > 2 ? d : 1)};
    off += x.count;
    e.push_back(x);
  };
  const bool qd = qbits_of(c.dtype) != 0;
  auto lin = [&](const std::string& pre, const char* local, int N, int K) {
    bool q = false;
    for (const char* s : kQuantized) q |= (std::strcmp(s, local) == 0);
    if (q && qd) {
      add(pre + local + ".weight_q", 2, N, K);
      add(pre + local + ".weight_scale", 2, N, K / 64);
    } else {
      add(pre + local + ".weight", 2, N, K);
    }
    add(pre + local + ".bias", 1, N);
  };
  const int d = c.d_model, f = c.d_ff, k = c.conv_kernel;
  add("pre.conv1.weight", 3, d, c.n_mels, c.sub_kernel);
  add("pre.conv1.bias", 1, d);
  add("pre.conv2.weight", 3, d, d, c.sub_kernel);
  add("pre.conv2.bias", 1, d);
  for (int i = 0; i < c.n_layers; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    add(p + "ff1.norm.weight", 1, d);
    add(p + "ff1.norm.bias", 1, d);
    lin(p, "ff1.linear1", f, d);
    lin(p, "ff1.linear2", d, f);
    add(p + "att.norm.weight", 1, d);
    add(p + "att.norm.bias", 1, d);
    lin(p, "att.linear_q", d, d);
    lin(p, "att.linear_k", d, d);
    lin(p, "att.linear_v", d, d);
    lin(p, "att.linear_out", d, d);
    add(p + "conv.norm.weight", 1, d);
    add(p + "conv.norm.bias", 1, d);
    lin(p, "conv.pointwise1", 2 * d, d);
    add(p + "conv.depthwise.weight", 2, d, k);
    add(p + "conv.depthwise.bias", 1, d);
    add(p + "conv.bn.weight", 1, d);
    add(p + "conv.bn.bias", 1, d);
    add(p + "conv.bn.running_mean", 1, d);
    add(p + "conv.bn.running_var", 1, d);
    lin(p, "conv.pointwise2", d, d);
    add(p + "ff2.norm.weight", 1, d);
    add(p + "ff2.norm.bias", 1, d);
    lin(p, "ff2.linear1", f, d);
    lin(p, "ff2.linear2", d, f);
    add(p + "norm_out.weight", 1, d);
    add(p + "norm_out.bias", 1, d);
  }
  add("head.weight", 2, c.n_classes, d);
  add("head.bias", 1, c.n_classes);
  return e;
}

// --------------------------------------------------------------------------- packed layout
struct Lin { size_t w = 0, s = 0, b = 0; int qb = 0; };   // qb: bits of packed weights, 0 = T
struct LayerOff {
  size_t ff1_g, ff1_b; Lin ff1_1, ff1_2;
  size_t att_g, att_b; Lin qkv, out;
  size_t cv_g, cv_b; Lin pw1; size_t dw_w, dw_b, bn_g, bn_b, bn_m, bn_v; Lin pw2;
  size_t ff2_g, ff2_b; Lin ff2_1, ff2_2;
  size_t no_g, no_b;
};
struct Layout {
  size_t conv1_w, conv1_b, conv2_w, conv2_b, head_w, head_b;
  std::vector<LayerOff> layers;
  size_t total;
  int wsize;   // bytes per element of non-quantised GEMM weights
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(const gigaam_config& c) {
  Layout L;
  const int es = c.dtype == GIGAAM_F32 ? 4 : 2;
  L.wsize = es;
  const int qbits = qbits_of(c.dtype);
  const size_t d = c.d_model, f = c.d_ff;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  auto lin = [&](size_t N, size_t K, bool quant) {
    Lin l;
    l.qb = quant ? qbits : 0;
    if (l.qb) { l.w = take(N * K * l.qb / 8); l.s = take(N * (K / 64) * 2); }
    else l.w = take(N * K * es);
    l.b = take(N * 4);
    return l;
  };
  L.conv1_w = take(d * 5 * c.n_mels * es);
  L.conv1_b = take(d * 4);
  L.conv2_w = take(d * 5 * d * es);
  L.conv2_b = take(d * 4);
  for (int i = 0; i < c.n_layers; ++i) {
    LayerOff o;
    o.ff1_g = take(d * 4); o.ff1_b = take(d * 4);
    o.ff1_1 = lin(f, d, true); o.ff1_2 = lin(d, f, true);
    o.att_g = take(d * 4); o.att_b = take(d * 4);
    o.qkv = lin(3 * d, d, true); o.out = lin(d, d, true);
    o.cv_g = take(d * 4); o.cv_b = take(d * 4);
    o.pw1 = lin(2 * d, d, true);
    o.dw_w = take(d * c.conv_kernel * 4); o.dw_b = take(d * 4);
    o.bn_g = take(d * 4); o.bn_b = take(d * 4); o.bn_m = take(d * 4); o.bn_v = take(d * 4);
    o.pw2 = lin(d, d, true);
    o.ff2_g = take(d * 4); o.ff2_b = take(d * 4);
    o.ff2_1 = lin(f, d, true); o.ff2_2 = lin(d, f, true);
    o.no_g = take(d * 4); o.no_b = take(d * 4);
    L.layers.push_back(o);
  }
  // the CTC head stays fp32 whatever the encoder's type: its logits decide the argmax
  L.head_w = take((size_t)c.n_classes * d * 4);
  L.head_b = take((size_t)c.n_classes * 4);
  L.total = off;
  return L;
}

// ---- host conversions (round to nearest even)

struct Packer {
  const gigaam_config& c;
  const float* src;
  char* dst;
  std::vector<Entry> ents;
  int es;
  int err = 0;
  const Entry* find(const std::string& n) {
    for (const Entry& e : ents) if (e.name == n) return &e;
    return nullptr;
  }
  const float* get(const std::string& n) {
    const Entry* e = find(n);
    return e ? src + e->offset : nullptr;
  }
  void put_w(size_t off, size_t idx, float v) {   // GEMM weight element in storage type
    if (es == 4) std::memcpy(dst + off + idx * 4, &v, 4);
    else {
      const uint16_t h = c.dtype == GIGAAM_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
      std::memcpy(dst + off + idx * 2, &h, 2);
    }
  }
  void put_f(size_t off, size_t idx, float v) { std::memcpy(dst + off + idx * 4, &v, 4); }
  void copy_f(size_t off, const std::string& n, size_t count) {
    const float* s = get(n);
    for (size_t i = 0; i < count; ++i) put_f(off, i, s[i]);
  }
  // Linear weight rows [N][K] from several canonical tensors (row_map gives, for each
  // packed row, the source tensor index and its row).
  void linear(const Lin& l, const std::vector<std::string>& names, size_t K,
              const std::vector<std::pair<int, int>>& row_map) {
    for (size_t r = 0; r < row_map.size(); ++r) {
      const std::string& base = names[row_map[r].first];
      const size_t sr = row_map[r].second;
      if (l.qb) {
        const float* q = get(base + ".weight_q");
        const float* s = get(base + ".weight_scale");
        const float qmax = (float)((1 << (l.qb - 1)) - 1);
        uint8_t* row = (uint8_t*)dst + l.w + r * K * l.qb / 8;
        std::memset(row, 0, K * l.qb / 8);
        for (size_t k = 0; k < K; ++k) {
          const float v = q[sr * K + k];
          if (!(v >= -qmax && v <= qmax) || v != std::nearbyint(v)) err = 1;
          const uint32_t u = (uint32_t)(int)v & ((1u << l.qb) - 1);
          const size_t bit = k * l.qb;               // little-endian bit string of the row
          for (int j = 0; j < l.qb; ++j)
            if (u >> j & 1) row[(bit + j) >> 3] |= (uint8_t)(1u << ((bit + j) & 7));
        }
        for (size_t g = 0; g < K / 64; ++g) {
          const uint16_t h = f32_to_f16_bits(s[sr * (K / 64) + g]);
          std::memcpy(dst + l.s + (r * (K / 64) + g) * 2, &h, 2);
        }
      } else {
        const float* w = get(base + ".weight");
        for (size_t k = 0; k < K; ++k) put_w(l.w, r * K + k, w[sr * K + k]);
      }
      put_f(l.b, r, get(base + ".bias")[sr]);
    }
  }
};

}  // namespace

extern "C" int gigaam_canonical_count(const gigaam_config* cfg, int32_t* n_entries, size_t* n_floats) {
  int rc = gigaam_check_config(cfg);
  if (rc) return rc;
  std::vector<Entry> e = canonical(*cfg);
  if (n_entries) *n_entries = (int32_t)e.size();
  if (n_floats) *n_floats = e.back().offset + e.back().count;
  return GIGAAM_OK;
}

extern "C" int gigaam_canonical_entry(const gigaam_config* cfg, int32_t i, char* name_buf,
                                      int32_t name_cap, int32_t* rank, int32_t* shape,
                                      size_t* offset_floats) {
  int rc = gigaam_check_config(cfg);
  if (rc) return rc;
  std::vector<Entry> e = canonical(*cfg);
  if (i < 0 || i >= (int)e.size()) return fail(GIGAAM_E_INVAL, "entry %d out of range", i);
  const Entry& x = e[i];
  if (name_buf) {
    if (name_cap <= (int)x.name.size()) return fail(GIGAAM_E_INVAL, "name buffer too small");
    std::memcpy(name_buf, x.name.c_str(), x.name.size() + 1);
  }
  if (rank) *rank = x.rank;
  if (shape) for (int j = 0; j < 3; ++j) shape[j] = j < x.rank ? x.shape[j] : 0;
  if (offset_floats) *offset_floats = x.offset;
  return GIGAAM_OK;
}

extern "C" int gigaam_packed_bytes(const gigaam_config* cfg, size_t* bytes) {
  int rc = gigaam_check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(GIGAAM_E_INVAL, "bytes is NULL");
  *bytes = layout(*cfg).total;
  return GIGAAM_OK;
}

extern "C" int gigaam_pack_weights(const gigaam_config* cfg, const float* canonical_host,
                                   size_t n_floats, void* packed_host, size_t packed_bytes) {
  int rc = gigaam_check_config(cfg);
  if (rc) return rc;
  if (!canonical_host || !packed_host) return fail(GIGAAM_E_INVAL, "NULL buffer");
  const gigaam_config& c = *cfg;
  Packer P{c, canonical_host, (char*)packed_host, canonical(c), c.dtype == GIGAAM_F32 ? 4 : 2};
  const size_t need = P.ents.back().offset + P.ents.back().count;
  if (n_floats != need) return fail(GIGAAM_E_INVAL, "canonical buffer has %zu floats, expected %zu", n_floats, need);
  const Layout L = layout(c);
  if (packed_bytes < L.total) return fail(GIGAAM_E_INVAL, "packed buffer %zu < %zu bytes", packed_bytes, L.total);
  std::memset(packed_host, 0, L.total);
  const size_t d = c.d_model, f = c.d_ff, m = c.n_mels;
  // subsampling convs: [out][in][5] -> [out][5][in]
  {
    const float* w1 = P.get("pre.conv1.weight");
    for (size_t o = 0; o < d; ++o)
      for (size_t j = 0; j < 5; ++j)
        for (size_t ci = 0; ci < m; ++ci) P.put_w(L.conv1_w, (o * 5 + j) * m + ci, w1[(o * m + ci) * 5 + j]);
    P.copy_f(L.conv1_b, "pre.conv1.bias", d);
    const float* w2 = P.get("pre.conv2.weight");
    for (size_t o = 0; o < d; ++o)
      for (size_t j = 0; j < 5; ++j)
        for (size_t ci = 0; ci < d; ++ci) P.put_w(L.conv2_w, (o * 5 + j) * d + ci, w2[(o * d + ci) * 5 + j]);
    P.copy_f(L.conv2_b, "pre.conv2.bias", d);
  }
  auto ident = [](int n) {
    std::vector<std::pair<int, int>> v;
    for (int i = 0; i < n; ++i) v.push_back({0, i});
    return v;
  };
  for (int i = 0; i < c.n_layers; ++i) {
    const std::string p = "layers." + std::to_string(i) + ".";
    const LayerOff& o = L.layers[i];
    P.copy_f(o.ff1_g, p + "ff1.norm.weight", d); P.copy_f(o.ff1_b, p + "ff1.norm.bias", d);
    P.linear(o.ff1_1, {p + "ff1.linear1"}, d, ident(f));
    P.linear(o.ff1_2, {p + "ff1.linear2"}, f, ident(d));
    P.copy_f(o.att_g, p + "att.norm.weight", d); P.copy_f(o.att_b, p + "att.norm.bias", d);
    {
      std::vector<std::pair<int, int>> rm;
      for (int s = 0; s < 3; ++s) for (size_t r = 0; r < d; ++r) rm.push_back({s, (int)r});
      P.linear(o.qkv, {p + "att.linear_q", p + "att.linear_k", p + "att.linear_v"}, d, rm);
    }
    P.linear(o.out, {p + "att.linear_out"}, d, ident(d));
    P.copy_f(o.cv_g, p + "conv.norm.weight", d); P.copy_f(o.cv_b, p + "conv.norm.bias", d);
    {
      // pointwise-1 rows: each 64-row group = 32 value rows then their 32 gate rows
      std::vector<std::pair<int, int>> rm;
      for (size_t q = 0; q < d / 32; ++q) {
        for (int r = 0; r < 32; ++r) rm.push_back({0, (int)(32 * q + r)});
        for (int r = 0; r < 32; ++r) rm.push_back({0, (int)(d + 32 * q + r)});
      }
      P.linear(o.pw1, {p + "conv.pointwise1"}, d, rm);
    }
    {   // depthwise taps tap-major [K][d]: a wave's lanes read consecutive channels
      const float* w = P.get(p + "conv.depthwise.weight");
      const int K = c.conv_kernel;
      for (int ch = 0; ch < d; ++ch)
        for (int j = 0; j < K; ++j) P.put_f(o.dw_w, (size_t)j * d + ch, w[(size_t)ch * K + j]);
    }
    P.copy_f(o.dw_b, p + "conv.depthwise.bias", d);
    P.copy_f(o.bn_g, p + "conv.bn.weight", d); P.copy_f(o.bn_b, p + "conv.bn.bias", d);
    P.copy_f(o.bn_m, p + "conv.bn.running_mean", d); P.copy_f(o.bn_v, p + "conv.bn.running_var", d);
    P.linear(o.pw2, {p + "conv.pointwise2"}, d, ident(d));
    P.copy_f(o.ff2_g, p + "ff2.norm.weight", d); P.copy_f(o.ff2_b, p + "ff2.norm.bias", d);
    P.linear(o.ff2_1, {p + "ff2.linear1"}, d, ident(f));
    P.linear(o.ff2_2, {p + "ff2.linear2"}, f, ident(d));
    P.copy_f(o.no_g, p + "norm_out.weight", d); P.copy_f(o.no_b, p + "norm_out.bias", d);
  }
  {
    const float* w = P.get("head.weight");
    for (size_t i = 0; i < (size_t)c.n_classes * d; ++i) P.put_f(L.head_w, i, w[i]);
    P.copy_f(L.head_b, "head.bias", c.n_classes);
  }
  if (P.err) return fail(GIGAAM_E_INVAL, "a quantised weight is not an integer in [-(2^(b-1)-1), 2^(b-1)-1]");
  return GIGAAM_OK;
}

extern "C" int gigaam_default_frontend(float* window_dev, float* melfb_dev, void* hip_stream) {
  if (!window_dev || !melfb_dev) return fail(GIGAAM_E_INVAL, "NULL table pointer");
  HIP_TRY(launch_default_frontend(window_dev, melfb_dev, (hipStream_t)hip_stream));
  return GIGAAM_OK;
}

// --------------------------------------------------------------------------- model
struct gigaam_model {
  gigaam_config cfg;
  const char* w;
  const float* window;
  const float* fb;
  Layout L;
};

extern "C" int gigaam_create(const gigaam_config* cfg, const void* packed_weights_dev,
                             const float* window_dev, const float* melfb_dev, gigaam_model** out) {
  int rc = gigaam_check_config(cfg);
  if (rc) return rc;
  if (!packed_weights_dev || !window_dev || !melfb_dev || !out)
    return fail(GIGAAM_E_INVAL, "NULL pointer argument");
  if ((uintptr_t)packed_weights_dev & 255) return fail(GIGAAM_E_INVAL, "packed weights not 256-B aligned");
  gigaam_model* m = new gigaam_model;
  m->cfg = *cfg;
  m->w = (const char*)packed_weights_dev;
  m->window = window_dev;
  m->fb = melfb_dev;
  m->L = layout(*cfg);
  *out = m;
  return GIGAAM_OK;
}

extern "C" void gigaam_destroy(gigaam_model* m) { delete m; }

// --------------------------------------------------------------------------- workspace
namespace {

struct Ws {
  size_t cuT, cuS, cuU, cuQ, rowT, rowS, rowU, posU, tileQ, cuQ2, tileQ2, tileG;
  size_t mel, melh, h1, x, y, r, qkv, ao, hid, cos_t, sin_t, logits, fids, part, fe;
  size_t total;
};

Ws plan(const gigaam_config& c, int B, int T_tot, int S_tot, int U_tot, int nQ, int U_max) {
  Ws w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t es = c.dtype == GIGAAM_F32 ? 4 : 2, d = c.d_model;
  const size_t hidw = (size_t)c.d_ff > 2 * d ? (size_t)c.d_ff : 2 * d;
  w.cuT = take((B + 1) * 4); w.cuS = take((B + 1) * 4); w.cuU = take((B + 1) * 4); w.cuQ = take((B + 1) * 4);
  w.rowT = take((size_t)T_tot * 4); w.rowS = take((size_t)S_tot * 4); w.rowU = take((size_t)U_tot * 4);
  w.posU = take((size_t)U_tot * 4);
  w.tileQ = take((size_t)nQ * 4);
  w.cuQ2 = take((B + 1) * 4);
  w.tileQ2 = take((size_t)nQ * 4);            // nQ2 <= nQ
  w.tileG = take((size_t)nQ * 16);
  w.mel = take((size_t)T_tot * 64 * 4);
  w.melh = take(es == 2 ? (size_t)T_tot * 64 * 2 : 0);     // 16-bit copy: the conv1 operand
  w.h1 = take((size_t)S_tot * d * es);
  w.x = take((size_t)U_tot * d * 4);
  w.y = take((size_t)U_tot * d * es);
  w.r = take((size_t)U_tot * d * es);
  w.qkv = take((size_t)U_tot * 3 * d * es);
  w.ao = take((size_t)U_tot * d * es);
  w.hid = take((size_t)U_tot * hidw * es);
  w.cos_t = take((size_t)U_max * (d / c.n_heads / 2) * 4);
  w.sin_t = take((size_t)U_max * (d / c.n_heads / 2) * 4);
  w.logits = take((size_t)U_tot * c.n_classes * 4);
  w.fids = take((size_t)B * U_max * 4);
  w.fe = take((640 + 128) * 4);               // frontend twiddles and mel filter ranges
  // split-K partial sums of the 16-bit GEMMs (small batches)
  w.part = take(c.dtype == GIGAAM_F32 ? 0 : (size_t)kSplitPartFloats * 4);
  w.total = off;
  return w;
}

// packed mel rows past this (B clips of the longest length) overflow the row counters
constexpr long long kMaxPackedRows = INT_MAX / 2;

Ws plan_bound(const gigaam_config& c, int B, int max_samples) {
  int T, S, U;
  frame_counts(max_samples, T, S, U);
  if ((long long)B * T > kMaxPackedRows) {       // no such batch fits a GPU: bound = "never"
    Ws w;
    std::memset(&w, 0, sizeof w);
    w.total = SIZE_MAX;
    return w;
  }
  const int nQ = B * ((U + kQTile - 1) / kQTile);
  return plan(c, B, B * T, B * S, B * U, nQ, U);
}

}  // namespace

extern "C" int gigaam_workspace_bytes(const gigaam_model* m, int32_t batch, int32_t max_samples,
                                      size_t* bytes) {
  if (!m || !bytes) return fail(GIGAAM_E_INVAL, "NULL argument");
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d out of [1, %d]", batch, GIGAAM_MAX_BATCH);
  if (max_samples < 320) return fail(GIGAAM_E_INVAL, "max_samples %d < 320", max_samples);
  const size_t total = plan_bound(m->cfg, batch, max_samples).total;
  if (total == SIZE_MAX) return fail(GIGAAM_E_INVAL, "batch %d x %d samples too large", batch, max_samples);
  *bytes = total;
  return GIGAAM_OK;
}

// --------------------------------------------------------------------------- forward
namespace {

enum { STAGE_NONE = -1 };

GemmParams gemm(int M, int N, int K, const void* A, int lda, const void* W, const void* scale,
                const float* bias, void* C, int ldc, float alpha = 1.f) {
  GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.M = M; p.N = N; p.K = K; p.A = A; p.lda = lda; p.W = W; p.ldw = K;
  p.Wscale = (const f16*)scale; p.bias = bias; p.C = C; p.ldc = ldc; p.alpha = alpha;
  return p;
}

int run(gigaam_model* m, const float* pcm, const int32_t* lengths, int32_t B, int32_t stride,
        void* ws, size_t ws_bytes, int stage, float* stage_out, size_t stage_floats,
        float* log_probs, int32_t* token_ids, int32_t* n_tokens, int32_t* frame_ids,
        float* enc_out, int32_t* n_frames, void* stream_v) {
  if (!m) return fail(GIGAAM_E_INVAL, "model is NULL");
  if (!pcm || !lengths || !ws) return fail(GIGAAM_E_INVAL, "NULL pcm / lengths / workspace");
  if (B < 1 || B > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d out of [1, %d]", B, GIGAAM_MAX_BATCH);
  if (stride < 320) return fail(GIGAAM_E_INVAL, "pcm_stride %d < 320", stride);
  if ((uintptr_t)ws & 255) return fail(GIGAAM_E_INVAL, "workspace not 256-B aligned");
  if (stage == STAGE_NONE && (!log_probs || !token_ids || !n_tokens))
    return fail(GIGAAM_E_INVAL, "NULL output pointer");
  const gigaam_config& c = m->cfg;
  const int d = c.d_model, f = c.d_ff, H = c.n_heads, dk = d / H, C = c.n_classes;
  const DType dt = (DType)c.dtype;
  const size_t es = dt == DT_F32 ? 4 : 2;
  hipStream_t s = (hipStream_t)stream_v;

  // ---- geometry (host)
  MetaArgs meta;
  std::memset(&meta, 0, sizeof meta);
  meta.B = B;
  int U_max = 0, nQ = 0, nQ2 = 0, maxlen = 0;
  std::vector<int> Ub(B);
  for (int b = 0; b < B; ++b) {
    const int L = lengths[b];
    if (L < 320 || L > stride)
      return fail(GIGAAM_E_INVAL, "lengths[%d] = %d outside [320, pcm_stride = %d]", b, L, stride);
    int T, S, U;
    frame_counts(L, T, S, U);
    meta.cuT[b + 1] = meta.cuT[b] + T;
    meta.cuS[b + 1] = meta.cuS[b] + S;
    meta.cuU[b + 1] = meta.cuU[b] + U;
    Ub[b] = U;
    U_max = U > U_max ? U : U_max;
    nQ += (U + kQTile - 1) / kQTile;
    nQ2 += (U + kQTile2 - 1) / kQTile2;
    maxlen = L > maxlen ? L : maxlen;
  }
  const int T_tot = meta.cuT[B], S_tot = meta.cuS[B], U_tot = meta.cuU[B];
  const Ws need = plan_bound(c, B, maxlen);
  if (ws_bytes < need.total)
    return fail(GIGAAM_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need.total);
  const Ws w = plan(c, B, T_tot, S_tot, U_tot, nQ, U_max);
  if (stage != STAGE_NONE) {
    size_t n = 0;
    if (stage == GIGAAM_STAGE_MEL) n = (size_t)T_tot * 64;
    else if (stage == GIGAAM_STAGE_SUB || (stage >= GIGAAM_STAGE_LAYER && stage < GIGAAM_STAGE_LAYER + c.n_layers) ||
             (stage >= 1000 && stage < 1000 + 10 * c.n_layers && stage % 10 < 4))
      n = (size_t)U_tot * d;
    else return fail(GIGAAM_E_INVAL, "stage %d out of range", stage);
    if (!stage_out || stage_floats < n) return fail(GIGAAM_E_INVAL, "stage output too small (%zu < %zu)", stage_floats, n);
  }
  if (n_frames) for (int b = 0; b < B; ++b) n_frames[b] = Ub[b];

  char* W = (char*)ws;
  MetaDev md{(int*)(W + w.cuT), (int*)(W + w.cuS), (int*)(W + w.cuU), (int*)(W + w.cuQ),
             (int*)(W + w.rowT), (int*)(W + w.rowS), (int*)(W + w.rowU), (int*)(W + w.tileQ),
             (int*)(W + w.cuQ2), (int*)(W + w.tileQ2), (int*)(W + w.tileG), (int*)(W + w.posU)};
  float* mel = (float*)(W + w.mel);
  char* h1 = W + w.h1;
  float* x = (float*)(W + w.x);
  char* y = W + w.y;
  char* r = W + w.r;
  char* qkv = W + w.qkv;
  char* ao = W + w.ao;
  char* hid = W + w.hid;
  char* hid2 = hid + (size_t)U_tot * d * es;
  float* cos_t = (float*)(W + w.cos_t);
  float* sin_t = (float*)(W + w.sin_t);
  float* logits = (float*)(W + w.logits);
  int* fids = frame_ids ? frame_ids : (int*)(W + w.fids);
  const char* P = m->w;
  const Layout& L = m->L;
  auto copy_out = [&](const float* src, size_t n) -> int {
    HIP_TRY(hipMemcpyAsync(stage_out, src, n * 4, hipMemcpyDeviceToDevice, s));
    return GIGAAM_OK;
  };
  // defer: a residual GEMM whose split-K slices (if it splits) the next LayerNorm adds
  auto G = [&](const char* name, AMode am, Epi ep, int wq, const GemmParams& gp,
               int* defer = nullptr, DType gdt = DT_F32, bool own_type = true) -> int {
    GemmParams q = gp;
    if (c.dtype != GIGAAM_F32) {
      q.part = (float*)(W + w.part);
      q.part_cap = kSplitPartFloats;
    }
    const DType t = own_type ? dt : gdt;
    LAUNCH(name, launch_gemm(t, wq, am, ep, q, s, stage == STAGE_NONE ? defer : nullptr));
    return GIGAAM_OK;
  };
  auto lin = [&](const Lin& l, int M, int N, int K, const void* A, int lda, void* Cp, int ldc,
                 float alpha = 1.f) {
    return gemm(M, N, K, A, lda, P + l.w, l.qb ? P + l.s : nullptr, (const float*)(P + l.b), Cp, ldc, alpha);
  };
  // macaron FFN half step x += 1/2 (W2 SiLU(W1 y + b1) + b2) as two GEMMs; dks reports a
  // split left to the next LayerNorm. (The fused few-row kernel behind gigaam_debug_mlp
  // measured slower than this inside the encode, where each layer's weights come from HBM.)
  auto ffn = [&](const Lin& l1, const Lin& l2, int* dks) -> int {
    int rc2;
    if ((rc2 = G("gemm.ffn_up", A_PLAIN, E_SILU, l1.qb, lin(l1, U_tot, f, d, y, d, hid, f)))) return rc2;
    return G("gemm.ffn_down", A_PLAIN, E_RESID, l2.qb, lin(l2, U_tot, d, f, hid, f, x, d, 0.5f), dks);
  };
  int rc;

  // ---- geometry to the device
  LAUNCH("meta", launch_meta(meta, md, T_tot, S_tot, U_tot, s));
  // ---- frontend (log-mel)
  // activations of the 16-bit models are bf16 for the bf16 dtype, fp16 otherwise
  const DType act = dt == DT_F32 ? DT_F32 : dt == DT_BF16 ? DT_BF16 : DT_F16;
  LAUNCH("frontend", launch_frontend(pcm, stride, m->window, m->fb, md, T_tot, mel,
                                     act == DT_F32 ? nullptr : (void*)(W + w.melh), act,
                                     (float*)(W + w.fe), (int*)(W + w.fe + 640 * 4), s));
  if (stage == GIGAAM_STAGE_MEL) return copy_out(mel, (size_t)T_tot * 64);
  // ---- subsampling: two implicit-GEMM Conv1d k5 s2 p2 + ReLU
  {
    // 16-bit models read the mel copy in their own type (the same rounding the fp32
    // source gets while staging), which the pipelined kernel streams
    const bool mel16 = act != DT_F32;
    GemmParams g1 = gemm(S_tot, d, 5 * 64, mel16 ? (const void*)(W + w.melh) : (const void*)mel, 0,
                         P + L.conv1_w, nullptr, (const float*)(P + L.conv1_b), h1, d);
    g1.rowclip = md.rowS; g1.cu_in = md.cuT; g1.cu_out = md.cuS; g1.cin = 64;
    if ((rc = G("gemm.conv1", mel16 ? A_CONV : A_CONV_F32, E_RELU, false, g1))) return rc;
    GemmParams g2 = gemm(U_tot, d, 5 * d, h1, 0, P + L.conv2_w, nullptr, (const float*)(P + L.conv2_b), x, d);
    g2.rowclip = md.rowU; g2.cu_in = md.cuS; g2.cu_out = md.cuU; g2.cin = d;
    if ((rc = G("gemm.conv2", A_CONV, E_RELU_F32, false, g2))) return rc;
  }
  if (stage == GIGAAM_STAGE_SUB) return copy_out(x, (size_t)U_tot * d);
  // ---- rotary tables for positions 0..U_max-1
  LAUNCH("rope_table", launch_rope_table(cos_t, sin_t, U_max, dk, c.rope_base, s));

  LnParams ln;
  std::memset(&ln, 0, sizeof ln);
  ln.rows = U_tot; ln.d = d; ln.x = x; ln.eps = c.ln_eps;
  ln.cos_t = cos_t; ln.sin_t = sin_t; ln.rowpos = md.posU;
  // ks / rb / ra: a preceding residual GEMM's deferred split-K slices, its bias and scale
  auto LN = [&](LnMode mode, size_t g1, size_t b1, const float* g2, const float* b2, void* yo,
                void* ro, int ks = 0, const float* rb = nullptr, float ra = 1.f) -> int {
    LnParams q = ln;
    q.g1 = (const float*)(P + g1); q.b1 = (const float*)(P + b1);
    q.g2 = g2; q.b2 = b2; q.y = yo; q.r = ro;
    if (ks > 0) { q.rpart = (const float*)(W + w.part); q.rks = ks; q.rbias = rb; q.ralpha = ra; }
    LAUNCH(mode == LN_ROPE ? "layernorm_rope" : mode == LN_TWO ? "layernorm_two" : "layernorm",
           launch_layernorm(dt, mode, q, s));
    return GIGAAM_OK;
  };
  const bool f32 = dt == DT_F32;              // the fp32 kernel works on 64-frame tiles
  AttnParams ap{qkv, ao, d, H, f32 ? nQ : nQ2, md.cuU, f32 ? md.cuQ : md.cuQ2, f32 ? md.tileQ : md.tileQ2,
                (float)(1.4426950408889634 / std::sqrt((double)dk)), f32 ? 0 : nQ, md.tileG};
  DwParams dp;
  dp.in = hid; dp.out = hid2; dp.d = d; dp.n_tiles = nQ; dp.cuU = md.cuU; dp.cuQ = md.cuQ;
  dp.tileQ = md.tileQ; dp.tileG = md.tileG; dp.eps = c.bn_eps;

  if ((rc = LN(LN_PLAIN, L.layers[0].ff1_g, L.layers[0].ff1_b, nullptr, nullptr, y, nullptr))) return rc;
  for (int li = 0; li < c.n_layers; ++li) {
    const LayerOff& o = L.layers[li];
    const int tap = 1000 + 10 * li;
    // first macaron FFN (half step)
    int dks = 0;      // split-K slices of the last residual GEMM left for the next LayerNorm
    if ((rc = ffn(o.ff1_1, o.ff1_2, &dks))) return rc;
    if (stage == tap + 0) return copy_out(x, (size_t)U_tot * d);
    // attention: LN + rope(y) -> [Q|K] from r, V from y -> flash attention -> out proj
    if ((rc = LN(LN_ROPE, o.att_g, o.att_b, nullptr, nullptr, y, r, dks, (const float*)(P + o.ff1_2.b), 0.5f))) return rc;
    {
      GemmParams gq = lin(o.qkv, U_tot, 3 * d, d, r, d, qkv, 3 * d);
      gq.A2 = y; gq.nsplit = 2 * d;
      if ((rc = G("gemm.qkv", A_DUAL, E_STORE, o.qkv.qb, gq))) return rc;
    }
    LAUNCH("attention", launch_attention(dt, dk, ap, s));
    if ((rc = G("gemm.out_proj", A_PLAIN, E_RESID, o.out.qb, lin(o.out, U_tot, d, d, ao, d, x, d), &dks))) return rc;
    if (stage == tap + 1) return copy_out(x, (size_t)U_tot * d);
    // convolution module
    if ((rc = LN(LN_PLAIN, o.cv_g, o.cv_b, nullptr, nullptr, y, nullptr, dks, (const float*)(P + o.out.b)))) return rc;
    if ((rc = G("gemm.pw1_glu", A_PLAIN, E_GLU, o.pw1.qb, lin(o.pw1, U_tot, 2 * d, d, y, d, hid, d)))) return rc;
    dp.w = (const float*)(P + o.dw_w); dp.b = (const float*)(P + o.dw_b);
    dp.bn_g = (const float*)(P + o.bn_g); dp.bn_b = (const float*)(P + o.bn_b);
    dp.bn_m = (const float*)(P + o.bn_m); dp.bn_v = (const float*)(P + o.bn_v);
    LAUNCH("dwconv_bn_silu", launch_dwconv(dt, c.conv_kernel, dp, s));
    if ((rc = G("gemm.pw2", A_PLAIN, E_RESID, o.pw2.qb, lin(o.pw2, U_tot, d, d, hid2, d, x, d), &dks))) return rc;
    if (stage == tap + 2) return copy_out(x, (size_t)U_tot * d);
    // second macaron FFN (half step) + block-final norm fused with the next block's first pre-norm
    if ((rc = LN(LN_PLAIN, o.ff2_g, o.ff2_b, nullptr, nullptr, y, nullptr, dks, (const float*)(P + o.pw2.b)))) return rc;
    if ((rc = ffn(o.ff2_1, o.ff2_2, &dks))) return rc;
    if (stage == tap + 3) return copy_out(x, (size_t)U_tot * d);
    const float* rb2 = (const float*)(P + o.ff2_2.b);
    if (li + 1 < c.n_layers) {
      const LayerOff& nx = L.layers[li + 1];
      if ((rc = LN(LN_TWO, o.no_g, o.no_b, (const float*)(P + nx.ff1_g), (const float*)(P + nx.ff1_b), y, nullptr, dks, rb2, 0.5f))) return rc;
    } else {
      if ((rc = LN(LN_TWO, o.no_g, o.no_b, nullptr, nullptr, nullptr, nullptr, dks, rb2, 0.5f))) return rc;
    }
    if (stage == GIGAAM_STAGE_LAYER + li) return copy_out(x, (size_t)U_tot * d);
  }
  // ---- CTC head + log-softmax + argmax, then greedy collapse
  {
    // fp32 operands and weights for every encoder type (the fp32 residual stream x is
    // read as it is, not rounded to the 16-bit type)
    GemmParams gh = gemm(U_tot, C, d, x, d, P + L.head_w, nullptr, (const float*)(P + L.head_b), logits, C);
    if ((rc = G("gemm.head", A_PLAIN, E_F32, 0, gh, nullptr, DT_F32, false))) return rc;
  }
  LAUNCH("logsoftmax_argmax", launch_logsoftmax_argmax(logits, C, B, U_max, md.cuU, log_probs, fids, s));
  LAUNCH("ctc_collapse", launch_collapse(fids, B, U_max, md.cuU, C - 1, token_ids, n_tokens, s));
  if (enc_out) LAUNCH("scatter_enc_out", launch_scatter_rows(x, d, B, U_max, md.cuU, enc_out, s));
  return GIGAAM_OK;
}

}  // namespace

extern "C" int gigaam_encode(gigaam_model* model, const float* pcm_dev, const int32_t* lengths_host,
                             int32_t batch, int32_t pcm_stride, void* workspace, size_t workspace_bytes,
                             float* log_probs_dev, int32_t* token_ids_dev, int32_t* n_tokens_dev,
                             int32_t* frame_ids_dev, float* enc_out_dev, int32_t* n_frames_host,
                             void* hip_stream) {
  return run(model, pcm_dev, lengths_host, batch, pcm_stride, workspace, workspace_bytes, STAGE_NONE,
             nullptr, 0, log_probs_dev, token_ids_dev, n_tokens_dev, frame_ids_dev, enc_out_dev,
             n_frames_host, hip_stream);
}

extern "C" int gigaam_encode_stage(gigaam_model* model, const float* pcm_dev, const int32_t* lengths_host,
                                   int32_t batch, int32_t pcm_stride, void* workspace,
                                   size_t workspace_bytes, int32_t stage, float* out_dev,
                                   size_t out_floats, void* hip_stream) {
  if (stage < 0) return fail(GIGAAM_E_INVAL, "stage %d out of range", stage);
  return run(model, pcm_dev, lengths_host, batch, pcm_stride, workspace, workspace_bytes, stage,
             out_dev, out_floats, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, hip_stream);
}

// --------------------------------------------------------------------------- fixed scratch
// The workspace of gigaam_encode_noalloc, for callers that cannot allocate device memory:
// a fixed array in the library's own device memory, one copy per GPU, held until the process
// ends. Its name is a host-side stand-in in host code: every host use goes through the
// device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[GIGAAM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// device address of the current device's scratch (looked up once per device)
int scratch_for_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(GIGAAM_E_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr || ((uintptr_t)ptr & 255)) return fail(GIGAAM_E_HIP, "scratch address %p not 256-B aligned", ptr);
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return GIGAAM_OK;
}
}  // namespace

extern "C" int gigaam_encode_noalloc(gigaam_model* model, const float* pcm_dev,
                                     const int32_t* lengths_host, int32_t batch, int32_t pcm_stride,
                                     float* log_probs_dev, int32_t* token_ids_dev, int32_t* n_tokens_dev,
                                     int32_t* frame_ids_dev, float* enc_out_dev, int32_t* n_frames_host,
                                     void* hip_stream) {
  if (!model) return fail(GIGAAM_E_INVAL, "model is NULL");
  if (!lengths_host) return fail(GIGAAM_E_INVAL, "NULL lengths");
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d out of [1, %d]", batch, GIGAAM_MAX_BATCH);
  int maxlen = 320;
  for (int b = 0; b < batch; ++b) {
    if (lengths_host[b] < 320 || lengths_host[b] > pcm_stride)
      return fail(GIGAAM_E_INVAL, "lengths[%d] = %d outside [320, pcm_stride = %d]", b, lengths_host[b], pcm_stride);
    maxlen = lengths_host[b] > maxlen ? lengths_host[b] : maxlen;
  }
  const size_t need = plan_bound(model->cfg, batch, maxlen).total;
  if (need > (size_t)GIGAAM_NOALLOC_SCRATCH_BYTES)
    return fail(GIGAAM_E_WORKSPACE, "this call needs %zu bytes of workspace, more than the %zu-byte fixed "
                "scratch of the allocation-free entry point", need, (size_t)GIGAAM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return run(model, pcm_dev, lengths_host, batch, pcm_stride, ws, GIGAAM_NOALLOC_SCRATCH_BYTES, STAGE_NONE,
             nullptr, 0, log_probs_dev, token_ids_dev, n_tokens_dev, frame_ids_dev, enc_out_dev,
             n_frames_host, hip_stream);
}

extern "C" int gigaam_debug_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A_dev,
                                 const void* W_dev, const void* scale_dev, const float* bias_dev,
                                 float* C_dev, float* part_dev, size_t part_floats,
                                 int32_t* slices_host, void* hip_stream) {
  if (dtype < GIGAAM_F32 || dtype > GIGAAM_W4F16) return fail(GIGAAM_E_INVAL, "dtype %d", dtype);
  if (M < 1 || N < 1 || K < 1) return fail(GIGAAM_E_INVAL, "bad shape %d x %d x %d", M, N, K);
  if (K % (dtype == GIGAAM_F32 ? 32 : 64)) return fail(GIGAAM_E_INVAL, "K %d not a multiple of the k-tile", K);
  const int qb = qbits_of(dtype);
  if (!A_dev || !W_dev || !C_dev || (qb && !scale_dev))
    return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (part_dev && ((uintptr_t)part_dev & 15))
    return fail(GIGAAM_E_INVAL, "partial-sum buffer not 16-byte aligned");
  if (((uintptr_t)A_dev & 15) || ((uintptr_t)W_dev & 15) || ((uintptr_t)C_dev & 15))
    return fail(GIGAAM_E_INVAL, "A / W / C not 16-byte aligned");
  GemmParams p = gemm(M, N, K, A_dev, K, W_dev, scale_dev, bias_dev, C_dev, N);
  p.part = part_dev;
  p.part_cap = part_dev ? (long)part_floats : 0;
  if (slices_host) *slices_host = gemm_split_slices((DType)dtype, qb, A_PLAIN, E_F32, p);
  HIP_TRY(launch_gemm((DType)dtype, qb, A_PLAIN, E_F32, p, (hipStream_t)hip_stream));
  return GIGAAM_OK;
}

extern "C" int gigaam_debug_gemm_role(int32_t dtype, int32_t a_mode, int32_t epilogue, int32_t M,
                                      int32_t N, int32_t K, const void* A_dev, const void* A2_dev,
                                      int32_t nsplit, const void* W_dev, const void* scale_dev,
                                      const float* bias_dev, float alpha, void* C_dev, float* part_dev,
                                      size_t part_floats, int32_t shape_request, int32_t* slices_host,
                                      int32_t* shape_host, void* hip_stream) {
  if (dtype < GIGAAM_F32 || dtype > GIGAAM_W4F16) return fail(GIGAAM_E_INVAL, "dtype %d", dtype);
  if (a_mode != GIGAAM_GEMM_A_PLAIN && a_mode != GIGAAM_GEMM_A_DUAL)
    return fail(GIGAAM_E_INVAL, "a_mode %d", a_mode);
  if (epilogue != GIGAAM_GEMM_E_STORE && epilogue != GIGAAM_GEMM_E_SILU && epilogue != GIGAAM_GEMM_E_GLU &&
      epilogue != GIGAAM_GEMM_E_RESID && epilogue != GIGAAM_GEMM_E_F32)
    return fail(GIGAAM_E_INVAL, "epilogue %d", epilogue);
  if (M < 1 || N < 1 || K < 1) return fail(GIGAAM_E_INVAL, "bad shape %d x %d x %d", M, N, K);
  if (K % (dtype == GIGAAM_F32 ? 32 : 64)) return fail(GIGAAM_E_INVAL, "K %d not a multiple of the k-tile", K);
  if (N % 4) return fail(GIGAAM_E_INVAL, "N %d not a multiple of 4", N);
  const int qb = qbits_of(dtype);
  if (!A_dev || !W_dev || !C_dev || (qb && !scale_dev)) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (a_mode == GIGAAM_GEMM_A_DUAL) {
    if (!A2_dev) return fail(GIGAAM_E_INVAL, "NULL A2 for the dual mode");
    if (nsplit <= 0 || nsplit >= N || nsplit % 128) return fail(GIGAAM_E_INVAL, "nsplit %d", nsplit);
    if (epilogue != GIGAAM_GEMM_E_STORE) return fail(GIGAAM_E_INVAL, "dual mode stores only");
    if ((uintptr_t)A2_dev & 15) return fail(GIGAAM_E_INVAL, "A2 not 16-byte aligned");
  }
  if (epilogue == GIGAAM_GEMM_E_GLU && N % 64) return fail(GIGAAM_E_INVAL, "GLU needs N %% 64 == 0");
  if (part_dev && ((uintptr_t)part_dev & 15))
    return fail(GIGAAM_E_INVAL, "partial-sum buffer not 16-byte aligned");
  if (((uintptr_t)A_dev & 15) || ((uintptr_t)W_dev & 15) || ((uintptr_t)C_dev & 15))
    return fail(GIGAAM_E_INVAL, "A / W / C not 16-byte aligned");
  const int ldc = epilogue == GIGAAM_GEMM_E_GLU ? N / 2 : N;
  GemmParams p = gemm(M, N, K, A_dev, K, W_dev, scale_dev, bias_dev, C_dev, ldc, alpha);
  p.A2 = A2_dev;
  p.nsplit = nsplit;
  p.part = part_dev;
  p.part_cap = part_dev ? (long)std::min(part_floats, (size_t)LONG_MAX) : 0;
  const AMode am = (AMode)a_mode;
  const Epi ep = (Epi)epilogue;
  if (shape_request != 0) {
    if (shape_request < GIGAAM_GEMM_DMA_256x256 || shape_request > GIGAAM_GEMM_DMA_128x128_S3)
      return fail(GIGAAM_E_INVAL, "shape_request %d is not a direct-load variant", shape_request);
    const int natural = gemm_shape_id((DType)dtype, qb, am, ep, p);
    if (natural < GIGAAM_GEMM_DMA_256x256)
      return fail(GIGAAM_E_INVAL, "this dtype / shape runs the register-staged kernel");
    if (epilogue == GIGAAM_GEMM_E_GLU &&
        (shape_request == GIGAAM_GEMM_DMA_256x192))
      return fail(GIGAAM_E_INVAL, "variant %d has odd 32-column blocks per wave (no GLU)", shape_request);
    if (a_mode == GIGAAM_GEMM_A_DUAL) {
      const int bn = shape_request == GIGAAM_GEMM_DMA_256x256 || shape_request == GIGAAM_GEMM_DMA_128x256 ? 256
                     : shape_request == GIGAAM_GEMM_DMA_256x192 ? 192 : 128;
      if (nsplit % bn) return fail(GIGAAM_E_INVAL, "dual split %d not a multiple of tile width %d", nsplit, bn);
    }
  }
  struct Force {                        // the override covers this call only
    int old;
    explicit Force(int id) : old(gemm_force_variant(id)) {}
    ~Force() { gemm_force_variant(old); }
  } force(shape_request);
  if (slices_host) *slices_host = gemm_split_slices((DType)dtype, qb, am, ep, p);
  if (shape_host) *shape_host = gemm_shape_id((DType)dtype, qb, am, ep, p);
  HIP_TRY(launch_gemm((DType)dtype, qb, am, ep, p, (hipStream_t)hip_stream));
  return GIGAAM_OK;
}

extern "C" int gigaam_debug_mlp(int32_t dtype, int32_t M, int32_t d, int32_t f, const void* y_dev,
                                const void* W1_dev, const float* b1_dev, const void* W2_dev,
                                const float* b2_dev, float alpha, float* x_dev, float* part_dev,
                                size_t part_floats, void* hip_stream) {
  if (dtype != GIGAAM_F16 && dtype != GIGAAM_BF16) return fail(GIGAAM_E_INVAL, "dtype %d", dtype);
  if (!y_dev || !W1_dev || !W2_dev || !x_dev || !part_dev) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if (((uintptr_t)part_dev & 15) || ((uintptr_t)x_dev & 15))
    return fail(GIGAAM_E_INVAL, "x / partial-sum buffer not 16-byte aligned");
  if (((uintptr_t)y_dev & 15) || ((uintptr_t)W1_dev & 15) || ((uintptr_t)W2_dev & 15))
    return fail(GIGAAM_E_INVAL, "y / W1 / W2 not 16-byte aligned");
  if (!mlp_fusable((DType)dtype, 0, M, d, f, (long)std::min(part_floats, (size_t)LONG_MAX)))
    return fail(GIGAAM_E_INVAL, "fused MLP shape %d x %d x %d or scratch of %zu floats unsupported",
                M, d, f, part_floats);
  MlpArgs ma{M, d, f, y_dev, W1_dev, b1_dev, W2_dev, part_dev};
  HIP_TRY(launch_mlp((DType)dtype, ma, b2_dev, alpha, x_dev, (hipStream_t)hip_stream));
  return GIGAAM_OK;
}

extern "C" int gigaam_debug_attention(int32_t dtype, int32_t d_model, int32_t n_heads, int32_t batch,
                                      const int32_t* frames_host, const void* qkv_dev, void* out_dev,
                                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (dtype < GIGAAM_F32 || dtype > GIGAAM_W4F16) return fail(GIGAAM_E_INVAL, "dtype %d", dtype);
  if (batch < 1 || batch > GIGAAM_MAX_BATCH) return fail(GIGAAM_E_INVAL, "batch %d", batch);
  if (!frames_host || !qkv_dev || !out_dev || !workspace) return fail(GIGAAM_E_INVAL, "NULL pointer");
  if ((uintptr_t)workspace & 255) return fail(GIGAAM_E_INVAL, "workspace not 256-B aligned");
  if (((uintptr_t)qkv_dev & 15) || ((uintptr_t)out_dev & 15))
    return fail(GIGAAM_E_INVAL, "qkv / out not 16-byte aligned");
  if (n_heads < 1 || d_model % n_heads) return fail(GIGAAM_E_INVAL, "d_model %d / n_heads %d", d_model, n_heads);
  const int dk = d_model / n_heads;
  if (dk != 48 && dk != 64) return fail(GIGAAM_E_UNSUPPORTED, "head size %d", dk);
  MetaArgs meta;
  std::memset(&meta, 0, sizeof meta);
  meta.B = batch;
  int nQ = 0, nQ2 = 0;
  for (int b = 0; b < batch; ++b) {
    if (frames_host[b] < 1) return fail(GIGAAM_E_INVAL, "frames[%d] = %d", b, frames_host[b]);
    meta.cuU[b + 1] = meta.cuU[b] + frames_host[b];
    nQ += (frames_host[b] + kQTile - 1) / kQTile;
    nQ2 += (frames_host[b] + kQTile2 - 1) / kQTile2;
  }
  const int U_tot = meta.cuU[batch];
  std::memcpy(meta.cuT, meta.cuU, sizeof meta.cuU);
  std::memcpy(meta.cuS, meta.cuU, sizeof meta.cuU);
  const size_t need = 20 * (size_t)(batch + 1) + 36 * (size_t)U_tot + 4096;
  if (workspace_bytes < need) return fail(GIGAAM_E_WORKSPACE, "workspace %zu < %zu", workspace_bytes, need);
  int* w = (int*)workspace;
  const int c1 = batch + 1;                    // five clip tables, five row/tile tables, then
  int* rows = w + 5 * c1;                      // the 16-byte tile geometry records
  int* geo = (int*)(((uintptr_t)(rows + 5 * U_tot) + 15) & ~(uintptr_t)15);
  MetaDev md{w, w + c1, w + 2 * c1, w + 3 * c1, rows, rows + U_tot, rows + 2 * U_tot,
             rows + 3 * U_tot, w + 4 * c1, rows + 4 * U_tot, geo, nullptr};
  hipStream_t s = (hipStream_t)hip_stream;
  HIP_TRY(launch_meta(meta, md, U_tot, U_tot, U_tot, s));
  const bool f32 = dtype == GIGAAM_F32;
  AttnParams ap{qkv_dev, out_dev, d_model, n_heads, f32 ? nQ : nQ2, md.cuU, f32 ? md.cuQ : md.cuQ2,
                f32 ? md.tileQ : md.tileQ2, (float)(1.4426950408889634 / std::sqrt((double)dk)),
                f32 ? 0 : nQ, md.tileG};
  HIP_TRY(launch_attention((DType)dtype, dk, ap, s));
  return GIGAAM_OK;
}
