// Host side of the C ABI declared in include/kvq.h: validation, the device
// buffer layout, RoPE tables, split planning and kernel launches on the
// caller's stream. No device memory is allocated here.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvq_status ok() { return KVQ_OK; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static_assert(KVQ_MAX_SPLITS == kvq::kMaxSplits, "split limit");
static_assert(KVQ_MAX_PAGED_BATCH == kvq::kMaxPagedBatch, "paged batch limit");

// Smallest distance between consecutive NUQ codebook entries: with entries at least this far
// apart, fp32 rounding of |u - C_j| (u, C_j in [-1, 1]) can never make an entry tie with or beat
// a nearer one (the spacing of fp32 values up to 2 is at most 2^-22).
constexpr double kMinCodebookGap = 1.0 / (1 << 21);

// Order-preserving map between fp32 values and integers (for a binary search over floats).
int32_t f2key(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (u & 0x80000000u) ? -(int32_t)(u & 0x7fffffffu) : (int32_t)u;
}
float key2f(int32_t k) {
  const uint32_t u = k < 0 ? ((uint32_t)(-k) | 0x80000000u) : (uint32_t)k;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Decision threshold between consecutive NUQ entries lo < hi (KVQuant notes 1.2 and 3.3: the
// code is the argmin of |u - C_j|, ties to the smaller index). The predicate "hi is strictly
// closer than lo" in fp32, P(u) = |RN(u - hi)| < |RN(u - lo)|, is false at u = lo, true at
// u = hi and monotone in u, so it switches at one fp32 value tau. With sorted entries at least
// kMinCodebookGap apart, the first-index argmin over all entries equals the number of
// thresholds tau_j <= u, which the quantize kernel evaluates with a short binary search.
float nuq_threshold(float lo, float hi) {
  auto closer_hi = [&](float u) {
    const float dlo = std::fabs(u - lo), dhi = std::fabs(u - hi);
    return dhi < dlo;
  };
  int32_t a = f2key(lo), b = f2key(hi);   // P(key2f(a)) false, P(key2f(b)) true
  while (b - a > 1) {
    const int32_t m = a + (b - a) / 2;
    if (closer_hi(key2f(m))) b = m; else a = m;
  }
  return key2f(b);
}

float u32_as_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// Code table of one codebook's decision thresholds tau[0..n): the kernel maps u in [-1, 1]
// to bucket floor(RN(u * 512 + 512)) (one fma); RN can move u by at most 2^-23 up across a
// bucket edge, never down, so every u that lands in bucket b lies in [B_b - 2^-23, B_b+1)
// with B_b = -1 + b / 512. Entry b = (number of thresholds below B_b - 2^-22, the one
// threshold in [B_b - 2^-22, B_b+1) or +inf); the code is then that count plus (u >= the
// threshold). The count is stored as the integer's bits. Two thresholds in one such range:
// entry 0's count bits are all ones and the kernel counts the thresholds instead.
void nuq_code_table(const float* tau, int n, float2* lut) {
  const double eps = std::ldexp(1.0, -22);
  bool ok = true;
  for (int b = 0; b <= kvq::kNuqBuckets; ++b) {
    const double lo = -1.0 + (double)b / (kvq::kNuqBuckets / 2);
    const double hi = b == kvq::kNuqBuckets ? 2.0 : -1.0 + (double)(b + 1) / (kvq::kNuqBuckets / 2);
    int below = 0, inside = 0;
    float t_in = INFINITY;
    for (int t = 0; t < n; ++t) {
      if ((double)tau[t] < lo - eps) ++below;
      else if ((double)tau[t] < hi) { ++inside; t_in = tau[t]; }
    }
    if (inside > 1) ok = false;
    lut[b] = make_float2(u32_as_float((uint32_t)below), t_in);   // the count's integer bits
  }
  for (int b = kvq::kNuqBuckets + 1; b < kvq::kNuqLutStride; ++b) lut[b] = make_float2(0.f, INFINITY);
  if (!ok) lut[0].x = u32_as_float(0xFFFFFFFFu);   // unusable: the kernel counts thresholds
}

}  // namespace

namespace kvq {

RecordLayout make_layout(int mode, int bits, int k_out) {
  RecordLayout L{};
  uint32_t pos = 0, payload = 0;
  auto seg = [&](uint32_t size) {
    pos = (uint32_t)align_up(pos, 16);
    const uint32_t at = pos;
    pos += size;
    payload += size;
    return at;
  };
  const uint32_t R = 16u * (uint32_t)bits;
  const uint32_t stat = mode == SYM ? 256u : (mode == ASYM ? 512u : 1024u);
  L.kc = seg(kT * R);
  L.vc = seg(kD * R);
  L.ks = seg(stat);
  L.vs = seg(stat);
  if (mode == KVARN) {
    L.k1 = seg(4 * kT);
    L.v1 = seg(4 * kD);
  }
  if (k_out > 0) {
    const uint32_t n = 128u * (uint32_t)k_out;
    L.ko_val = seg(2 * n);
    L.ko_ptr = seg(2 * 129);
    L.ko_idx = seg(n);
    L.vo_val = seg(2 * n);
    L.vo_ptr = seg(2 * 129);
    L.vo_idx = seg(n);
  }
  L.rec_bytes = (uint32_t)align_up(pos, 256);
  L.payload = payload;
  return L;
}

}  // namespace kvq

struct kvq_cache_s {
  kvq_config cfg;
  kvq::RecordLayout lay;
  uint8_t* base = nullptr;
  size_t bytes = 0;
  int max_blocks = 0;
  size_t off_rec = 0, layer_rec_bytes = 0;
  size_t off_tail = 0, layer_tail_bytes = 0;
  size_t off_cb = 0, off_lut = 0, off_rope_base = 0, off_rope_off = 0, off_work = 0;
  std::vector<int32_t> len;         // [layer]; paged caches: the largest sequence length
  std::vector<int32_t> seq_len;     // paged caches: [layer][batch]
  int pages = 0;                    // paged caches: pages per layer pool
  std::vector<uint8_t> cb_loaded;   // [layer][kv_head][2]
  std::vector<float> cb_host;       // [layer][kv_head][2][kCbStride]
  std::vector<float2> lut_host;     // [layer][kv_head][2][kNuqLutStride]
  std::vector<float> rope_host;     // base table then offset table
  int splits_override = 0;
  bool matrix_cores = true;         // kvq_set_matrix_cores
  int sink = 0, window = 0;         // sink tokens, fp16 window (tokens)
  int ring_rows = kvq::kT;          // fp16 ring of body tokens per tensor: window + 128
  int tail_rows = kvq::kT;          // fp16 rows per tensor: sink + ring
};

namespace {

kvq_status check_codebooks(kvq_cache c, int layer) {
  const kvq_config& cfg = c->cfg;
  if (cfg.mode != KVQ_MODE_NUQ) return KVQ_OK;
  for (int h = 0; h < cfg.n_kv_heads; ++h)
    for (int w = 0; w < 2; ++w)
      if (!c->cb_loaded[((size_t)layer * cfg.n_kv_heads + h) * 2 + w])
        return fail(KVQ_ERR_STATE, "NUQ codebook of layer %d kv head %d (%s) not loaded", layer, h, w ? "V" : "K");
  return KVQ_OK;
}

// Quantizer arguments shared by the unpaged and paged appends.
kvq::QuantArgs quant_args(kvq_cache c, int layer, const void* k_f16, const void* v_f16, int n_rows) {
  const kvq_config& cfg = c->cfg;
  kvq::QuantArgs a{};
  a.lay = c->lay;
  a.k_out = cfg.outliers_per_vec;
  a.varn_iters = cfg.varn_iters;
  a.k_in = static_cast<const __half*>(k_f16);
  a.v_in = static_cast<const __half*>(v_f16);
  a.n_new = n_rows;
  a.sink = c->sink;
  a.ring_rows = c->ring_rows;
  a.tail_rows = c->tail_rows;
  a.Hkv = cfg.n_kv_heads;
  a.max_blocks = c->max_blocks;
  a.rec = c->base + c->off_rec + (size_t)layer * c->layer_rec_bytes;
  a.tail = reinterpret_cast<__half*>(c->base + c->off_tail + (size_t)layer * c->layer_tail_bytes);
  a.cb = reinterpret_cast<const float*>(c->base + c->off_cb) + (size_t)layer * cfg.n_kv_heads * 2 * kvq::kCbStride;
  a.nuq_lut = reinterpret_cast<const float2*>(c->base + c->off_lut) + (size_t)layer * cfg.n_kv_heads * 2 * kvq::kNuqLutStride;
  return a;
}

struct Regions {
  int max_blocks;
  size_t layer_rec, rec, layer_tail, tail, cb, lut, rope_base, rope_off, work, total;
  size_t off_rec, off_tail, off_cb, off_lut, off_rope_base, off_rope_off, off_work;
};

kvq_status validate_config(const kvq_config* c) {
  if (!c) return fail(KVQ_ERR_ARG, "config is NULL");
  if (c->n_layers < 1 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(KVQ_ERR_ARG, "n_layers, batch, n_kv_heads and n_q_heads must be >= 1");
  if (c->head_dim != KVQ_HEAD_DIM) return fail(KVQ_ERR_ARG, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVQ_ERR_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  const int g = c->n_q_heads / c->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return fail(KVQ_ERR_ARG, "query group %d not in {1,2,4,8}", g);
  if (c->max_tokens < KVQ_BLOCK_TOKENS || c->max_tokens % KVQ_BLOCK_TOKENS != 0)
    return fail(KVQ_ERR_ARG, "max_tokens must be a positive multiple of 128 (got %d)", c->max_tokens);
  if (c->mode < KVQ_MODE_RTN || c->mode > KVQ_MODE_ASYM_INT4) return fail(KVQ_ERR_ARG, "unknown mode %d", c->mode);
  if (c->mode == KVQ_MODE_ASYM_INT4 && c->bits != 4) return fail(KVQ_ERR_ARG, "asymmetric int4 requires bits = 4");
  if (c->bits != 2 && c->bits != 3 && c->bits != 4 && c->bits != 8)
    return fail(KVQ_ERR_ARG, "bits must be 2, 3, 4 or 8 (got %d)", c->bits);
  if (c->mode == KVQ_MODE_SYM_INT4 && c->bits != 4 && c->bits != 8)
    return fail(KVQ_ERR_ARG, "symmetric mode requires bits = 4 or 8");
  if (c->mode == KVQ_MODE_NUQ && c->bits == 8) return fail(KVQ_ERR_ARG, "NUQ codebooks have at most 16 entries");
  if (c->outliers_per_vec < 0 || c->outliers_per_vec > KVQ_MAX_OUTLIERS)
    return fail(KVQ_ERR_ARG, "outliers_per_vec must be in 0..8 (got %d)", c->outliers_per_vec);
  if (c->pre_rope != 0 && c->pre_rope != 1) return fail(KVQ_ERR_ARG, "pre_rope must be 0 or 1");
  if (c->pre_rope && !(c->rope_theta > 0.f && std::isfinite(c->rope_theta)))
    return fail(KVQ_ERR_ARG, "rope_theta must be finite and > 0");
  if (c->mode == KVQ_MODE_KVARN) {
    if (c->outliers_per_vec != 0 || c->pre_rope != 0)
      return fail(KVQ_ERR_ARG, "KVARN mode supports neither outliers nor pre-RoPE keys");
    if (c->varn_iters < 0 || c->varn_iters > 64) return fail(KVQ_ERR_ARG, "varn_iters must be in 0..64");
  }
  if (c->sink_tokens < 0 || c->sink_tokens > KVQ_MAX_SINK)
    return fail(KVQ_ERR_ARG, "sink_tokens must be in 0..%d (got %d)", KVQ_MAX_SINK, c->sink_tokens);
  if (c->fp16_window < 0 || c->fp16_window > KVQ_MAX_WINDOW || c->fp16_window % KVQ_BLOCK_TOKENS != 0)
    return fail(KVQ_ERR_ARG, "fp16_window must be a multiple of 128 in 0..%d (got %d)", KVQ_MAX_WINDOW, c->fp16_window);
  const double rec = kvq::make_layout(c->mode, c->bits, c->outliers_per_vec).rec_bytes;
  if (c->paged_pages < 0) return fail(KVQ_ERR_ARG, "paged_pages must be >= 0 (got %d)", c->paged_pages);
  if (c->paged_pages > 0) {
    if (c->batch > KVQ_MAX_PAGED_BATCH)
      return fail(KVQ_ERR_ARG, "a paged cache holds at most %d sequences (got %d)", KVQ_MAX_PAGED_BATCH, c->batch);
    if (c->sink_tokens != 0 || c->fp16_window != 0)
      return fail(KVQ_ERR_ARG, "a paged cache keeps neither sink tokens nor an fp16 window");
    if (rec * c->n_kv_heads * (double)c->paged_pages > (double)KVQ_MAX_POOL_BYTES)
      return fail(KVQ_ERR_ARG, "page pool of %d pages exceeds %llu bytes per layer", c->paged_pages,
                  (unsigned long long)KVQ_MAX_POOL_BYTES);
  }
  const double blocks = c->paged_pages > 0 ? (double)c->paged_pages : c->batch * (c->max_tokens / 128.0);
  const double total = rec * c->n_layers * c->n_kv_heads * blocks;
  if (total > 4.0e12) return fail(KVQ_ERR_ARG, "cache larger than 4 TB requested");
  return KVQ_OK;
}

int ring_rows_of(const kvq_config* c) { return c->fp16_window + KVQ_BLOCK_TOKENS; }
int tail_rows_of(const kvq_config* c) { return c->sink_tokens + ring_rows_of(c); }

Regions regions(const kvq_config* c) {
  Regions r{};
  const kvq::RecordLayout L = kvq::make_layout(c->mode, c->bits, c->outliers_per_vec);
  r.max_blocks = c->max_tokens / KVQ_BLOCK_TOKENS;
  const size_t units = (size_t)c->batch * c->n_kv_heads;
  r.layer_rec = c->paged_pages > 0 ? (size_t)c->paged_pages * c->n_kv_heads * L.rec_bytes
                                    : units * r.max_blocks * L.rec_bytes;
  r.rec = r.layer_rec * c->n_layers;
  r.layer_tail = units * 2 * (size_t)tail_rows_of(c) * kvq::kD * sizeof(__half);
  r.tail = r.layer_tail * c->n_layers;
  r.cb = c->mode == KVQ_MODE_NUQ ? (size_t)c->n_layers * c->n_kv_heads * 2 * kvq::kCbStride * sizeof(float) : 0;
  r.lut = c->mode == KVQ_MODE_NUQ ? (size_t)c->n_layers * c->n_kv_heads * 2 * kvq::kNuqLutStride * sizeof(float2) : 0;
  r.rope_base = c->pre_rope ? (size_t)(r.max_blocks + 1) * 64 * 2 * sizeof(float) : 0;
  r.rope_off = c->pre_rope ? ((size_t)128 * 64 * 2 + 64) * sizeof(float) : 0;   // offsets, then theta_i
  // split partials: up to KVQ_MAX_SPLITS splits plus the fp16 part's partial
  r.work = (size_t)c->batch * c->n_q_heads * (KVQ_MAX_SPLITS + 1) * kvq::kPartStride * sizeof(float);
  size_t pos = 0;
  auto place = [&](size_t size) { pos = align_up(pos, 256); const size_t at = pos; pos += size; return at; };
  r.off_rec = place(r.rec);
  r.off_tail = place(r.tail);
  r.off_cb = place(r.cb);
  r.off_lut = place(r.lut);
  r.off_rope_base = place(r.rope_base);
  r.off_rope_off = place(r.rope_off);
  r.off_work = place(r.work);
  r.total = align_up(pos, 256);
  return r;
}

kvq_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

kvq_status check_layer(kvq_cache c, int layer) {
  if (!c) return fail(KVQ_ERR_ARG, "cache handle is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers)
    return fail(KVQ_ERR_ARG, "layer %d out of range [0, %d)", layer, c->cfg.n_layers);
  return KVQ_OK;
}

}  // namespace

namespace {

// Split partials of kvq_decode_attn_static: a library-owned array, one copy per GPU the
// library runs on, held until the process ends. Every call on a GPU shares its copy.
constexpr size_t kScratchBytes = (size_t)KVQ_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of the scratch array (looked up once per device, with
// that device current). The array's name is a host-side stand-in and is never passed on.
kvq_status scratch_for_current_device(float** out) {
  int dev = -1;
  kvq_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != KVQ_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_HIP, "device %d outside the supported range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != KVQ_OK) return st;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

// Decode over one layer with the split partials in `part` (nullptr: the cache's workspace).
// part_limit: bytes available at `part` (checked against what this call's splits need).
// table: the block table of a paged cache (nullptr for an unpaged one).
kvq_status decode_impl(kvq_cache c, int layer, const void* q_f16, float* out, float softmax_scale,
                       void* stream, float* part, size_t part_limit, const int32_t* table);

}  // namespace

extern "C" {

kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_ARG, "bytes is NULL");
  const kvq_status st = validate_config(cfg);
  if (st != KVQ_OK) return st;
  *bytes = regions(cfg).total;
  return ok();
}

kvq_status kvq_cache_init(const kvq_config* cfg, void* dev_buf, size_t bytes, void* stream,
                          kvq_cache* out) {
  if (!out) return fail(KVQ_ERR_ARG, "out is NULL");
  *out = nullptr;
  kvq_status st = validate_config(cfg);
  if (st != KVQ_OK) return st;
  if (!dev_buf) return fail(KVQ_ERR_ARG, "dev_buf is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256 != 0) return fail(KVQ_ERR_ARG, "dev_buf must be 256-byte aligned");
  const Regions r = regions(cfg);
  if (bytes < r.total) return fail(KVQ_ERR_SIZE, "dev_buf holds %zu bytes, %zu needed", bytes, r.total);

  auto* c = new kvq_cache_s();
  c->cfg = *cfg;
  c->lay = kvq::make_layout(cfg->mode, cfg->bits, cfg->outliers_per_vec);
  c->base = static_cast<uint8_t*>(dev_buf);
  c->bytes = bytes;
  c->max_blocks = r.max_blocks;
  c->off_rec = r.off_rec;
  c->layer_rec_bytes = r.layer_rec;
  c->off_tail = r.off_tail;
  c->layer_tail_bytes = r.layer_tail;
  c->off_cb = r.off_cb;
  c->off_lut = r.off_lut;
  c->off_rope_base = r.off_rope_base;
  c->off_rope_off = r.off_rope_off;
  c->off_work = r.off_work;
  c->sink = cfg->sink_tokens;
  c->window = cfg->fp16_window;
  c->ring_rows = ring_rows_of(cfg);
  c->tail_rows = tail_rows_of(cfg);
  c->len.assign(cfg->n_layers, 0);
  c->pages = cfg->paged_pages;
  if (c->pages > 0) c->seq_len.assign((size_t)cfg->n_layers * cfg->batch, 0);
  c->cb_loaded.assign((size_t)cfg->n_layers * cfg->n_kv_heads * 2, 0);
  c->cb_host.assign((size_t)cfg->n_layers * cfg->n_kv_heads * 2 * kvq::kCbStride, 0.f);
  if (cfg->mode == KVQ_MODE_NUQ)
    c->lut_host.assign((size_t)cfg->n_layers * cfg->n_kv_heads * 2 * kvq::kNuqLutStride, make_float2(0.f, 0.f));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg->pre_rope) {
    // RoPE angles n * theta_i, theta_i = theta^(-2i/128), evaluated in double precision:
    // base rows for n = sink + 128 * block (the first position of body block `block`) and
    // offset rows for n = 0..127 (KVQuant notes 1.3)
    const int nb = r.max_blocks + 1;
    c->rope_host.resize((size_t)nb * 128 + 128 * 128 + 64);
    for (int i = 0; i < 64; ++i) {
      const double th = std::pow((double)cfg->rope_theta, -2.0 * i / 128.0);
      for (int blk = 0; blk < nb; ++blk) {
        const double ang = ((double)cfg->sink_tokens + (double)blk * 128.0) * th;
        c->rope_host[((size_t)blk * 64 + i) * 2] = (float)std::cos(ang);
        c->rope_host[((size_t)blk * 64 + i) * 2 + 1] = (float)std::sin(ang);
      }
      c->rope_host[(size_t)nb * 128 + 128 * 128 + i] = (float)th;
      for (int jj = 0; jj < 128; ++jj) {
        const double ang = (double)jj * th;
        c->rope_host[(size_t)nb * 128 + ((size_t)i * 128 + jj) * 2] = (float)std::cos(ang);
        c->rope_host[(size_t)nb * 128 + ((size_t)i * 128 + jj) * 2 + 1] = (float)std::sin(ang);
      }
    }
    st = hip_check(hipMemcpyAsync(c->base + c->off_rope_base, c->rope_host.data(), (size_t)nb * 128 * sizeof(float),
                                  hipMemcpyHostToDevice, s), "upload RoPE base table");
    if (st == KVQ_OK)
      st = hip_check(hipMemcpyAsync(c->base + c->off_rope_off, c->rope_host.data() + (size_t)nb * 128,
                                    (128 * 128 + 64) * sizeof(float), hipMemcpyHostToDevice, s), "upload RoPE offset table");
    if (st == KVQ_OK) st = hip_check(hipStreamSynchronize(s), "synchronize after init");
    if (st != KVQ_OK) {
      delete c;
      return st;
    }
  }
  *out = c;
  return ok();
}

void kvq_cache_destroy(kvq_cache cache) { delete cache; }

kvq_status kvq_codebook_load(kvq_cache c, int layer, int kv_head, int which, const float* host_codebook,
                             int n_entries, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->cfg.mode != KVQ_MODE_NUQ) return fail(KVQ_ERR_STATE, "codebooks are only used in NUQ mode");
  if (kv_head < 0 || kv_head >= c->cfg.n_kv_heads) return fail(KVQ_ERR_ARG, "kv_head %d out of range", kv_head);
  if (which != 0 && which != 1) return fail(KVQ_ERR_ARG, "which must be 0 (keys) or 1 (values)");
  if (!host_codebook) return fail(KVQ_ERR_ARG, "codebook is NULL");
  if (n_entries != (1 << c->cfg.bits))
    return fail(KVQ_ERR_ARG, "codebook needs %d entries (got %d)", 1 << c->cfg.bits, n_entries);
  for (int i = 0; i < n_entries; ++i) {
    const float v = host_codebook[i];
    if (!std::isfinite(v) || v < -1.f || v > 1.f) return fail(KVQ_ERR_ARG, "codebook entry %d not in [-1, 1]", i);
    if (i > 0 && !((double)v - (double)host_codebook[i - 1] >= kMinCodebookGap))
      return fail(KVQ_ERR_ARG, "codebook entries %d and %d are not ascending by at least 2^-21", i - 1, i);
  }
  const size_t slot = ((size_t)layer * c->cfg.n_kv_heads + kv_head) * 2 + which;
  float* dst = c->cb_host.data() + slot * kvq::kCbStride;
  for (int i = 0; i < kvq::kCbStride; ++i) dst[i] = 0.f;
  for (int i = 0; i < n_entries; ++i) dst[i] = host_codebook[i];
  for (int i = 0; i + 1 < n_entries; ++i) dst[16 + i] = nuq_threshold(host_codebook[i], host_codebook[i + 1]);
  st = hip_check(hipMemcpyAsync(c->base + c->off_cb + slot * kvq::kCbStride * sizeof(float), dst,
                                kvq::kCbStride * sizeof(float), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream)), "upload codebook");
  if (st != KVQ_OK) return st;
  float2* lut = c->lut_host.data() + slot * kvq::kNuqLutStride;
  nuq_code_table(dst + 16, n_entries - 1, lut);
  st = hip_check(hipMemcpyAsync(c->base + c->off_lut + slot * kvq::kNuqLutStride * sizeof(float2), lut,
                                kvq::kNuqLutStride * sizeof(float2), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream)), "upload codebook table");
  if (st != KVQ_OK) return st;
  c->cb_loaded[slot] = 1;
  return ok();
}

kvq_status kvq_quantize_append(kvq_cache c, int layer, const void* k_f16, const void* v_f16, int n_new,
                               void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages > 0) return fail(KVQ_ERR_STATE, "the cache is paged: use kvq_quantize_append_paged");
  if (n_new < 0) return fail(KVQ_ERR_ARG, "n_new must be >= 0");
  if (n_new == 0) return ok();
  if (!k_f16 || !v_f16) return fail(KVQ_ERR_ARG, "k or v is NULL");
  if (reinterpret_cast<uintptr_t>(k_f16) % 16 || reinterpret_cast<uintptr_t>(v_f16) % 16)
    return fail(KVQ_ERR_ARG, "k and v must be 16-byte aligned");
  const kvq_config& cfg = c->cfg;
  const int len = c->len[layer];
  if ((int64_t)len + n_new > cfg.max_tokens)
    return fail(KVQ_ERR_CAPACITY, "layer %d holds %d tokens; %d more exceed max_tokens %d", layer, len, n_new,
                cfg.max_tokens);
  st = check_codebooks(c, layer);
  if (st != KVQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // positions < sink are sink tokens; body token u sits at position sink + u. Body block j
  // is quantized once the body holds at least 128 (j + 1) + window tokens.
  const int S = c->sink, W = c->window;
  const int n_sink = std::max(0, std::min(S - len, n_new));
  const int u_old = std::max(0, len - S), u_new = std::max(0, len + n_new - S);
  const int nq_old = std::max(0, u_old - W) / KVQ_BLOCK_TOKENS;
  const int nq_new = std::max(0, u_new - W) / KVQ_BLOCK_TOKENS;
  const int nb = nq_new - nq_old;
  const int in_row0 = S - len;   // input row of body token u
  __half* tail = reinterpret_cast<__half*>(c->base + c->off_tail + (size_t)layer * c->layer_tail_bytes);
  if (nb > 0) {
    kvq::QuantArgs a = quant_args(c, layer, k_f16, v_f16, n_new);
    a.blk0 = nq_old;
    a.u_old = u_old;
    a.in_row0 = in_row0;
    st = hip_check(kvq::launch_quantize(cfg.mode, cfg.bits, a, nb, cfg.batch, s), "launch quantize");
    if (st != KVQ_OK) return st;
  }
  // new tokens that stay fp16: sink tokens, and body tokens of blocks not quantized now
  kvq::TailArgs ta{};
  ta.k_in = static_cast<const __half*>(k_f16);
  ta.v_in = static_cast<const __half*>(v_f16);
  ta.n_new = n_new;
  ta.Hkv = cfg.n_kv_heads;
  ta.tail = tail;
  ta.n_sink = n_sink;
  ta.sink_row0 = len;
  ta.ring_u0 = std::max(u_old, nq_new * KVQ_BLOCK_TOKENS);
  ta.ring_count = std::max(0, u_new - ta.ring_u0);
  ta.ring_src0 = ta.ring_u0 + in_row0;
  ta.sink = S;
  ta.ring_rows = c->ring_rows;
  ta.tail_rows = c->tail_rows;
  if (ta.n_sink + ta.ring_count > 0) {
    st = hip_check(kvq::launch_tail(ta, cfg.batch, s), "launch tail copy");
    if (st != KVQ_OK) return st;
  }
  c->len[layer] = len + n_new;
  return ok();
}

kvq_status kvq_quantize_append_paged(kvq_cache c, int layer, const void* k_f16, const void* v_f16,
                                     const int32_t* n_new, int max_new, const int32_t* block_table,
                                     void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages == 0) return fail(KVQ_ERR_STATE, "the cache is not paged: use kvq_quantize_append");
  const kvq_config& cfg = c->cfg;
  if (!n_new) return fail(KVQ_ERR_ARG, "n_new is NULL");
  if (max_new < 0) return fail(KVQ_ERR_ARG, "max_new must be >= 0");
  kvq::PagedSeq pg{};
  int total = 0, most = 0, blocks = 0;
  for (int b = 0; b < cfg.batch; ++b) {
    const int n = n_new[b];
    if (n < 0 || n > max_new) return fail(KVQ_ERR_ARG, "n_new[%d] = %d not in 0..%d", b, n, max_new);
    const int len = c->seq_len[(size_t)layer * cfg.batch + b];
    if ((int64_t)len + n > cfg.max_tokens)
      return fail(KVQ_ERR_CAPACITY, "sequence %d of layer %d holds %d tokens; %d more exceed max_tokens %d", b, layer,
                  len, n, cfg.max_tokens);
    pg.len[b] = len;
    pg.n_new[b] = n;
    total += n;
    most = std::max(most, len + n);
    blocks = std::max(blocks, (len + n) / KVQ_BLOCK_TOKENS - len / KVQ_BLOCK_TOKENS);
  }
  if (total == 0) return ok();
  if (!k_f16 || !v_f16) return fail(KVQ_ERR_ARG, "k or v is NULL");
  if (reinterpret_cast<uintptr_t>(k_f16) % 16 || reinterpret_cast<uintptr_t>(v_f16) % 16)
    return fail(KVQ_ERR_ARG, "k and v must be 16-byte aligned");
  if (blocks > 0 && !block_table) return fail(KVQ_ERR_ARG, "block_table is NULL");
  if (reinterpret_cast<uintptr_t>(block_table) % 4) return fail(KVQ_ERR_ARG, "block_table must be 4-byte aligned");
  st = check_codebooks(c, layer);
  if (st != KVQ_OK) return st;
  pg.table = block_table;
  pg.table_stride = c->max_blocks;
  pg.n_pages = c->pages;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the blocks each sequence completes, read partly from its fp16 tail (before the tail
  // copy below overwrites it), then the new tokens of each sequence's open block
  if (blocks > 0) {
    kvq::QuantArgs a = quant_args(c, layer, k_f16, v_f16, max_new);
    a.pg = pg;
    st = hip_check(kvq::launch_quantize(cfg.mode, cfg.bits, a, blocks, cfg.batch, s), "launch quantize");
    if (st != KVQ_OK) return st;
  }
  kvq::TailArgs ta{};
  ta.k_in = static_cast<const __half*>(k_f16);
  ta.v_in = static_cast<const __half*>(v_f16);
  ta.n_new = max_new;
  ta.Hkv = cfg.n_kv_heads;
  ta.tail = reinterpret_cast<__half*>(c->base + c->off_tail + (size_t)layer * c->layer_tail_bytes);
  ta.sink = 0;
  ta.ring_rows = c->ring_rows;
  ta.tail_rows = c->tail_rows;
  ta.pg = pg;
  st = hip_check(kvq::launch_tail(ta, cfg.batch, s), "launch tail copy");
  if (st != KVQ_OK) return st;
  for (int b = 0; b < cfg.batch; ++b) c->seq_len[(size_t)layer * cfg.batch + b] += n_new[b];
  c->len[layer] = most;
  return ok();
}

kvq_status kvq_decode_attn(kvq_cache c, int layer, const void* q_f16, float* out, float softmax_scale,
                           void* stream) {
  return decode_impl(c, layer, q_f16, out, softmax_scale, stream, nullptr, 0, nullptr);
}

kvq_status kvq_decode_attn_paged(kvq_cache c, int layer, const void* q_f16, float* out, float softmax_scale,
                                 const int32_t* block_table, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages == 0) return fail(KVQ_ERR_STATE, "the cache is not paged: use kvq_decode_attn");
  if (!block_table) return fail(KVQ_ERR_ARG, "block_table is NULL");
  if (reinterpret_cast<uintptr_t>(block_table) % 4) return fail(KVQ_ERR_ARG, "block_table must be 4-byte aligned");
  return decode_impl(c, layer, q_f16, out, softmax_scale, stream, nullptr, 0, block_table);
}

kvq_status kvq_decode_attn_static(kvq_cache c, int layer, const void* q_f16, float* out, float softmax_scale,
                                  void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages > 0) return fail(KVQ_ERR_STATE, "the cache is paged: use kvq_decode_attn_paged");
  float* part = nullptr;
  st = scratch_for_current_device(&part);
  if (st != KVQ_OK) return st;
  return decode_impl(c, layer, q_f16, out, softmax_scale, stream, part, kScratchBytes, nullptr);
}

}  // extern "C"

namespace {

kvq_status decode_impl(kvq_cache c, int layer, const void* q_f16, float* out, float softmax_scale,
                       void* stream, float* part, size_t part_limit, const int32_t* table) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages > 0 && !table) return fail(KVQ_ERR_STATE, "the cache is paged: use kvq_decode_attn_paged");
  if (!q_f16 || !out) return fail(KVQ_ERR_ARG, "q or out is NULL");
  if (reinterpret_cast<uintptr_t>(q_f16) % 4 || reinterpret_cast<uintptr_t>(out) % 4)
    return fail(KVQ_ERR_ARG, "q and out must be 4-byte aligned");
  if (!(softmax_scale <= 0.f || std::isfinite(softmax_scale))) return fail(KVQ_ERR_ARG, "softmax_scale not finite");
  const kvq_config& cfg = c->cfg;
  const int L = c->len[layer];
  if (L == 0) return fail(KVQ_ERR_STATE, "layer %d holds no tokens", layer);
  kvq::PagedSeq pg{};
  if (table) {
    pg.table = table;
    pg.table_stride = c->max_blocks;
    pg.n_pages = c->pages;
    for (int b = 0; b < cfg.batch; ++b) {
      pg.len[b] = c->seq_len[(size_t)layer * cfg.batch + b];
      if (pg.len[b] == 0) return fail(KVQ_ERR_STATE, "sequence %d of layer %d holds no tokens", b, layer);
    }
  }
  // quantized blocks and fp16 tokens (see kvq_quantize_append); paged caches: the longest
  // sequence's blocks set the split plan, each sequence stops at its own length
  const int U = std::max(0, L - c->sink);
  const int nblk = std::max(0, U - c->window) / KVQ_BLOCK_TOKENS;
  const int fp16_body = U - nblk * KVQ_BLOCK_TOKENS;
  const bool side = c->sink > 0 || c->window > 0;   // the fp16 part gets its own kernel
  const int tail_n = side ? 0 : fp16_body;
  const int units = cfg.batch * cfg.n_kv_heads;
  const int group = cfg.n_q_heads / cfg.n_kv_heads;
  const bool tab = kvq::tab_supported(cfg.mode, cfg.bits, group, cfg.pre_rope);
  int splits = 1, bps = 0;
  if (nblk > 0) {
    if (c->splits_override > 0) {
      splits = std::min(c->splits_override, nblk);
    } else {
      // about two resident workgroups of four waves per CU (512 on 256 CUs; the table
      // kernel's workgroups have two waves: 1024), each streaming at least 8 blocks, so
      // that per-workgroup set-up and the split merge stay small
      const int target_wgs = tab ? 1024 : 512;
      splits = (target_wgs + units - 1) / units;
      splits = std::min(splits, (nblk + 7) / 8);
      splits = std::max(1, std::min(splits, KVQ_MAX_SPLITS));
    }
    bps = (nblk + splits - 1) / splits;
    splits = (nblk + bps - 1) / bps;
  }
  // the fp16 part (sink tokens and body tokens not yet quantized) in chunks of whole 16-token
  // groups, one workgroup and one partial each, as many as the free partial slots allow
  const int q_slots = nblk > 0 ? splits : 0;
  const int n_fp16 = side ? std::min(L, c->sink) + fp16_body : 0;
  int n_side = 0, side_chunk = 0;
  if (side) {
    int free_slots = KVQ_MAX_SPLITS + 1 - q_slots;
    if (part) {   // a caller-sized partial array (the static entry point): its capacity too
      const size_t row_bytes = (size_t)cfg.batch * cfg.n_q_heads * kvq::kPartStride * sizeof(float);
      free_slots = std::min(free_slots, (int)std::min<size_t>(part_limit / row_bytes, KVQ_MAX_SPLITS + 1) - q_slots);
    }
    n_side = std::max(1, std::min((n_fp16 + kvq::kSideChunk - 1) / kvq::kSideChunk, free_slots));
    side_chunk = std::max(16, ((n_fp16 + n_side - 1) / n_side + 15) / 16 * 16);
    n_side = std::max(1, (n_fp16 + side_chunk - 1) / side_chunk);
  }
  // partial slots per (sequence, query head): the splits, then the fp16 part's
  const int part_slots = side ? q_slots + n_side : splits;
  if (part && part_slots > 1) {
    const size_t need = (size_t)cfg.batch * cfg.n_q_heads * part_slots * kvq::kPartStride * sizeof(float);
    if (need > part_limit)
      return fail(KVQ_ERR_SIZE, "%d splits x %d sequences x %d query heads need %zu bytes of split partials; "
                  "the static scratch holds %zu (lower the split count with kvq_set_decode_splits)",
                  part_slots, cfg.batch, cfg.n_q_heads, need, part_limit);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvq::DecodeArgs a{};
  a.lay = c->lay;
  a.k_out = cfg.outliers_per_vec;
  a.rec = c->base + c->off_rec + (size_t)layer * c->layer_rec_bytes;
  a.tail = reinterpret_cast<const __half*>(c->base + c->off_tail + (size_t)layer * c->layer_tail_bytes);
  a.cb = reinterpret_cast<const float*>(c->base + c->off_cb) + (size_t)layer * cfg.n_kv_heads * 2 * kvq::kCbStride;
  a.rope_base = reinterpret_cast<const float*>(c->base + c->off_rope_base);
  a.rope_off = reinterpret_cast<const float*>(c->base + c->off_rope_off);
  a.q = static_cast<const __half*>(q_f16);
  a.part = part ? part : reinterpret_cast<float*>(c->base + c->off_work);
  a.out = out;
  a.Hkv = cfg.n_kv_heads;
  a.Hq = cfg.n_q_heads;
  a.max_blocks = c->max_blocks;
  a.nblk = nblk;
  a.tail_n = tail_n;
  a.splits = splits;
  a.blocks_per_split = bps;
  a.part_slots = part_slots;
  a.sink_n = std::min(L, c->sink);
  a.fp16_u0 = nblk * KVQ_BLOCK_TOKENS;
  a.fp16_n = side ? fp16_body : 0;
  a.ring_rows = c->ring_rows;
  a.tail_rows = c->tail_rows;
  a.side_slot = part_slots > 1 ? q_slots : -1;
  a.side_chunk = side_chunk;
  a.pg = pg;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(128.0f);
  a.scale_log2 = scale * 1.4426950408889634f;
  if (cfg.outliers_per_vec > 0) {
    // staging for the sparse fix-ups: the outlier segments (table kernel: one copy per
    // workgroup), plus key S/M, value S/M of a half and a RoPE base row (VALU kernel: per wave)
    const uint32_t blob = c->lay.vo_idx + 128u * cfg.outliers_per_vec - c->lay.ko_val;
    // (table kernel: plus one prefix array of the value-outlier corrections per wave and,
    // at 2 bits, one array of folded key-outlier entries per wave)
    const uint32_t pref = 2u * (((128u * cfg.outliers_per_vec + 1u) * 4u + 15u) & ~15u) +
                          (cfg.bits == 2 ? 2u * 128u * 16u * (uint32_t)cfg.outliers_per_vec : 0u);
    a.wave_lds = (int)(((blob + 15u) & ~15u) + (tab ? pref : 1024u + 512u + 512u));
  }
  if (nblk > 0 || !side) {
    if (tab)
      st = hip_check(kvq::launch_decode_tab(cfg.mode, cfg.bits, c->matrix_cores, a, cfg.batch, s), "launch decode");
    else if (c->matrix_cores && kvq::mfma_supported(cfg.mode, cfg.bits, cfg.pre_rope, cfg.outliers_per_vec))
      st = hip_check(kvq::launch_decode_mfma(cfg.mode, cfg.bits, group, a, cfg.batch, s), "launch decode");
    else
      st = hip_check(kvq::launch_decode(cfg.mode, cfg.bits, group, cfg.pre_rope, a, cfg.batch, s), "launch decode");
    if (st != KVQ_OK) return st;
  }
  if (side) {
    st = hip_check(kvq::launch_decode_fp16(group, cfg.pre_rope, a, cfg.batch, n_side, s), "launch fp16 decode");
    if (st != KVQ_OK) return st;
  }
  if (part_slots > 1) {
    st = hip_check(kvq::launch_combine(a.part, out, cfg.n_q_heads, part_slots, cfg.batch, s), "launch split combine");
    if (st != KVQ_OK) return st;
  }
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_error_decomposition(kvq_cache c, int layer, int block0, int n_blocks, const void* k_f16,
                                   const void* v_f16, double* out, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!k_f16 || !v_f16 || !out) return fail(KVQ_ERR_ARG, "k, v or out is NULL");
  if (reinterpret_cast<uintptr_t>(k_f16) % 16 || reinterpret_cast<uintptr_t>(v_f16) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 8)
    return fail(KVQ_ERR_ARG, "k and v must be 16-byte aligned, out 8-byte aligned");
  if (c->pages > 0) return fail(KVQ_ERR_STATE, "the error diagnostic reads unpaged caches only");
  const int U = std::max(0, c->len[layer] - c->sink);
  const int nq = std::max(0, U - c->window) / KVQ_BLOCK_TOKENS;   // quantized blocks
  if (n_blocks <= 0 || block0 < 0 || block0 + n_blocks > nq)
    return fail(KVQ_ERR_ARG, "blocks %d .. %d are not all quantized (layer %d holds %d quantized blocks)", block0,
                block0 + n_blocks - 1, layer, nq);
  kvq::DiagArgs a{};
  a.lay = c->lay;
  a.k_out = c->cfg.outliers_per_vec;
  a.rec = c->base + c->off_rec + (size_t)layer * c->layer_rec_bytes;
  a.cb = reinterpret_cast<const float*>(c->base + c->off_cb) + (size_t)layer * c->cfg.n_kv_heads * 2 * kvq::kCbStride;
  a.k_in = static_cast<const __half*>(k_f16);
  a.v_in = static_cast<const __half*>(v_f16);
  a.block0 = block0;
  a.n_blocks = n_blocks;
  a.Hkv = c->cfg.n_kv_heads;
  a.max_blocks = c->max_blocks;
  a.out = out;
  return hip_check(kvq::launch_diag(c->cfg.mode, c->cfg.bits, a, c->cfg.batch, static_cast<hipStream_t>(stream)),
                   "launch error diagnostic");
}

}  // extern "C"

namespace {

struct CodebookWs {
  int n_ranges;
  int64_t per_range;
  size_t off_assign, off_partials, off_changes, off_state, total;
};

CodebookWs codebook_ws(int64_t n) {
  CodebookWs w{};
  w.n_ranges = (int)std::min<int64_t>(kvq::kCodebookMaxRanges, (n + 4095) / 4096);
  w.per_range = (n + w.n_ranges - 1) / w.n_ranges;
  size_t pos = 0;
  auto place = [&](size_t size) { pos = align_up(pos, 256); const size_t at = pos; pos += size; return at; };
  w.off_assign = place((size_t)n);
  w.off_partials = place((size_t)w.n_ranges * 2 * 16 * sizeof(double));
  w.off_changes = place((size_t)w.n_ranges * sizeof(int));
  w.off_state = place(sizeof(kvq::CodebookState));
  w.total = align_up(pos, 256);
  return w;
}

}  // namespace

extern "C" {

kvq_status kvq_codebook_build_workspace(int64_t n, int bits, size_t* bytes) {
  if (!bytes) return fail(KVQ_ERR_ARG, "bytes is NULL");
  if (n < 1 || n > ((int64_t)1 << 40)) return fail(KVQ_ERR_ARG, "n must be in 1..2^40 (got %lld)", (long long)n);
  if (bits < 2 || bits > 4) return fail(KVQ_ERR_ARG, "bits must be 2, 3 or 4 (got %d)", bits);
  *bytes = codebook_ws(n).total;
  return ok();
}

kvq_status kvq_codebook_build(const float* act, const float* weight, int64_t n, int bits, int max_iters,
                              void* workspace, size_t workspace_bytes, float* codebook, int32_t* iters,
                              void* stream) {
  size_t need = 0;
  kvq_status st = kvq_codebook_build_workspace(n, bits, &need);
  if (st != KVQ_OK) return st;
  if (!act || !workspace || !codebook) return fail(KVQ_ERR_ARG, "act, workspace or codebook is NULL");
  if (max_iters < 1 || max_iters > 1000) return fail(KVQ_ERR_ARG, "max_iters must be in 1..1000 (got %d)", max_iters);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(KVQ_ERR_ARG, "workspace must be 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(act) % 4 || reinterpret_cast<uintptr_t>(weight) % 4 ||
      reinterpret_cast<uintptr_t>(codebook) % 4 || reinterpret_cast<uintptr_t>(iters) % 4)
    return fail(KVQ_ERR_ARG, "act, weight, codebook and iters must be 4-byte aligned");
  if (workspace_bytes < need) return fail(KVQ_ERR_SIZE, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  const CodebookWs w = codebook_ws(n);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  kvq::CodebookArgs a{};
  a.act = act;
  a.weight = weight;
  a.n = n;
  a.per_range = w.per_range;
  a.n_ranges = w.n_ranges;
  a.assign = base + w.off_assign;
  a.partials = reinterpret_cast<double*>(base + w.off_partials);
  a.changes = reinterpret_cast<int*>(base + w.off_changes);
  a.state = reinterpret_cast<kvq::CodebookState*>(base + w.off_state);
  a.out = codebook;
  a.iters_out = iters;
  return hip_check(kvq::launch_codebook_build(bits, a, max_iters, static_cast<hipStream_t>(stream)),
                   "launch codebook builder");
}

kvq_status kvq_cache_length(kvq_cache c, int layer, int32_t* n_tokens) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!n_tokens) return fail(KVQ_ERR_ARG, "n_tokens is NULL");
  *n_tokens = c->len[layer];
  return ok();
}

kvq_status kvq_cache_reset(kvq_cache c, int layer) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  c->len[layer] = 0;
  if (c->pages > 0)
    std::fill(c->seq_len.begin() + (size_t)layer * c->cfg.batch, c->seq_len.begin() + (size_t)(layer + 1) * c->cfg.batch, 0);
  return ok();
}

kvq_status kvq_sequence_length(kvq_cache c, int layer, int b, int32_t* n_tokens) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (b < 0 || b >= c->cfg.batch) return fail(KVQ_ERR_ARG, "sequence %d out of range [0, %d)", b, c->cfg.batch);
  if (!n_tokens) return fail(KVQ_ERR_ARG, "n_tokens is NULL");
  *n_tokens = c->pages > 0 ? c->seq_len[(size_t)layer * c->cfg.batch + b] : c->len[layer];
  return ok();
}

kvq_status kvq_sequence_reset(kvq_cache c, int layer, int b) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (b < 0 || b >= c->cfg.batch) return fail(KVQ_ERR_ARG, "sequence %d out of range [0, %d)", b, c->cfg.batch);
  if (c->pages == 0) return fail(KVQ_ERR_STATE, "the sequences of an unpaged cache keep equal lengths");
  int32_t* l = c->seq_len.data() + (size_t)layer * c->cfg.batch;
  l[b] = 0;
  c->len[layer] = *std::max_element(l, l + c->cfg.batch);
  return ok();
}

kvq_status kvq_page_span(kvq_cache c, int layer, int page, int kv_head, size_t* offset, size_t* bytes) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages == 0) return fail(KVQ_ERR_STATE, "the cache is not paged: use kvq_block_span");
  if (page < 0 || page >= c->pages || kv_head < 0 || kv_head >= c->cfg.n_kv_heads)
    return fail(KVQ_ERR_ARG, "page coordinates out of range");
  if (!offset || !bytes) return fail(KVQ_ERR_ARG, "offset or bytes is NULL");
  *offset = c->off_rec + (size_t)layer * c->layer_rec_bytes + ((size_t)page * c->cfg.n_kv_heads + kv_head) * c->lay.rec_bytes;
  *bytes = c->lay.rec_bytes;
  return ok();
}

kvq_status kvq_set_decode_splits(kvq_cache c, int splits) {
  if (!c) return fail(KVQ_ERR_ARG, "cache handle is NULL");
  if (splits < 0 || splits > KVQ_MAX_SPLITS) return fail(KVQ_ERR_ARG, "splits must be in 0..%d", KVQ_MAX_SPLITS);
  c->splits_override = splits;
  return ok();
}

kvq_status kvq_set_matrix_cores(kvq_cache c, int enable) {
  if (!c) return fail(KVQ_ERR_ARG, "cache handle is NULL");
  if (enable != 0 && enable != 1) return fail(KVQ_ERR_ARG, "enable must be 0 or 1");
  c->matrix_cores = enable == 1;
  return ok();
}

kvq_status kvq_block_span(kvq_cache c, int layer, int b, int kv_head, int block, size_t* offset, size_t* bytes) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->pages > 0) return fail(KVQ_ERR_STATE, "the cache is paged: use kvq_page_span");
  if (b < 0 || b >= c->cfg.batch || kv_head < 0 || kv_head >= c->cfg.n_kv_heads || block < 0 ||
      block >= c->max_blocks)
    return fail(KVQ_ERR_ARG, "block coordinates out of range");
  if (!offset || !bytes) return fail(KVQ_ERR_ARG, "offset or bytes is NULL");
  const size_t unit = (size_t)b * c->cfg.n_kv_heads + kv_head;
  *offset = c->off_rec + (size_t)layer * c->layer_rec_bytes + (unit * c->max_blocks + block) * c->lay.rec_bytes;
  *bytes = c->lay.rec_bytes;
  return ok();
}

kvq_status kvq_tail_span(kvq_cache c, int layer, int b, int kv_head, size_t* offset, size_t* bytes) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (b < 0 || b >= c->cfg.batch || kv_head < 0 || kv_head >= c->cfg.n_kv_heads)
    return fail(KVQ_ERR_ARG, "tail coordinates out of range");
  if (!offset || !bytes) return fail(KVQ_ERR_ARG, "offset or bytes is NULL");
  const size_t unit = (size_t)b * c->cfg.n_kv_heads + kv_head;
  *offset = c->off_tail + (size_t)layer * c->layer_tail_bytes + unit * 2 * (size_t)c->tail_rows * kvq::kD * sizeof(__half);
  *bytes = 2 * (size_t)c->tail_rows * kvq::kD * sizeof(__half);
  return ok();
}

kvq_status kvq_decode_bytes(kvq_cache c, int layer, size_t* bytes) {
  const kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!bytes) return fail(KVQ_ERR_ARG, "bytes is NULL");
  const kvq_config& cfg = c->cfg;
  const size_t units = (size_t)cfg.batch * cfg.n_kv_heads;
  const int L = c->len[layer];
  const int U = std::max(0, L - c->sink);
  const size_t nblk = std::max(0, U - c->window) / KVQ_BLOCK_TOKENS;
  const size_t tail_n = (size_t)(U - (int)nblk * KVQ_BLOCK_TOKENS) + (size_t)std::min(L, c->sink);   // fp16 tokens
  size_t n = 0;
  if (c->pages > 0) {   // each sequence its own blocks (and their block-table entries) and tail
    for (int b = 0; b < cfg.batch; ++b) {
      const size_t lb = (size_t)c->seq_len[(size_t)layer * cfg.batch + b];
      n += cfg.n_kv_heads * ((lb / 128) * c->lay.payload + (lb % 128) * 2 * KVQ_HEAD_DIM * sizeof(__half)) +
           (lb / 128) * sizeof(int32_t);
    }
  } else {
    n = units * (nblk * c->lay.payload + tail_n * 2 * KVQ_HEAD_DIM * sizeof(__half));
  }
  n += (size_t)cfg.batch * cfg.n_q_heads * KVQ_HEAD_DIM * (sizeof(__half) + sizeof(float));
  if (cfg.mode == KVQ_MODE_NUQ) n += (size_t)cfg.n_kv_heads * 2 * (1u << cfg.bits) * sizeof(float);
  if (cfg.pre_rope)
    n += (nblk + ((size_t)(U - (int)nblk * KVQ_BLOCK_TOKENS) + 127) / 128) * 64 * 2 * sizeof(float) +
         128 * 64 * 2 * sizeof(float);
  *bytes = n;
  return ok();
}

const char* kvq_strerror(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_SIZE: return "buffer too small";
    case KVQ_ERR_CAPACITY: return "capacity exceeded";
    case KVQ_ERR_STATE: return "invalid state";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
