// libkvarn C ABI: argument validation (host only, before any HIP call) and launches.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "kvarn_common.h"
#include "kvarn_launch.h"

using namespace kvarn;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The seven fields of kvarn_geom, plus variant and num_pages when the caller passed a
// kvarn_geom_ext (KVARN_GEOM_EXT in bits); then the limits of this library.
kvarn_status resolve_geom(const kvarn_geom* in, Geo* g) {
  if (!in) return KVARN_ERR_NULL;
  *g = Geo{in->batch, in->num_kv_heads, in->head_dim, in->capacity, in->group, in->varn_iters,
           in->bits & ~KVARN_GEOM_EXT, 0, 0};
  if (in->bits & KVARN_GEOM_EXT) {
    const kvarn_geom_ext* e = reinterpret_cast<const kvarn_geom_ext*>(in);
    if (e->size != sizeof(kvarn_geom_ext)) return KVARN_ERR_GEOM;
    g->variant = e->variant;
    g->num_pages = e->num_pages;
  }
  if (g->batch <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0 || g->capacity <= 0 || g->group <= 0 ||
      g->varn_iters < 0 || g->bits <= 0 || g->num_pages < 0)
    return KVARN_ERR_GEOM;
  if (g->head_dim != kD || (g->group != 32 && g->group != 64) || g->bits < 2 || g->bits > 4 || g->varn_iters > 8)
    return KVARN_ERR_UNSUPPORTED;
  if (g->variant & ~(int32_t)(KVARN_VARIANT_NO_ROTATION | KVARN_VARIANT_NO_CHANNEL_PASS | KVARN_VARIANT_NO_TOKEN_PASS |
                              KVARN_VARIANT_CENTERED))
    return KVARN_ERR_UNSUPPORTED;
  if (g->capacity % g->group != 0) return KVARN_ERR_GEOM;
  // keep every element index of a [B][capacity][Hkv][D] tensor and every tile count in range
  if ((long long)g->batch * g->capacity * g->num_kv_heads * kD >= (1LL << 40)) return KVARN_ERR_RANGE;
  if ((long long)g->batch * g->num_kv_heads * (g->capacity / g->group) * 2 >= (1LL << 31)) return KVARN_ERR_RANGE;
  if ((long long)g->num_pages * g->num_kv_heads * 2 >= (1LL << 31)) return KVARN_ERR_RANGE;
  return KVARN_OK;
}

#define RESOLVE(in, g)                              \
  Geo g##_v;                                        \
  {                                                 \
    const kvarn_status rs = resolve_geom(in, &g##_v); \
    if (rs != KVARN_OK) return rs;                  \
  }                                                 \
  const Geo* g = &g##_v

kvarn_status dev(hipError_t e) { return e == hipSuccess ? KVARN_OK : KVARN_ERR_DEVICE; }

kvarn_status check_prefill(const Geo* g, void* cache, const void* k, const void* v, int32_t T) {
  if (!cache || ((!k || !v) && T > 0)) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(k) || !aligned16(v)) return KVARN_ERR_ALIGN;
  if (T < 0 || T > g->capacity) return KVARN_ERR_RANGE;
  return KVARN_OK;
}

// Work-groups of one layer's prefill launch (tile work-groups + tail work-groups), and the
// waves per work-group; a launch's work-items (all layers) must stay below 2^32.
long long prefill_blocks(const Geo* g, int32_t T) {
  const long long nw = g->group / 32;
  return (long long)g->batch * g->num_kv_heads * (T / g->group) * 2 + (2LL * g->batch * g->num_kv_heads + nw - 1) / nw;
}
constexpr long long kMaxWorkItems = (1LL << 32) - 1;

// The fields of a prefill launch shared by every layer of one geometry and token count
PrefillArgs prefill_args(const Geo* g, int32_t T) {
  PrefillArgs a{};
  a.L = make_layout(*g);
  a.T = T;
  a.nfull = T / g->group;
  a.jobs = g->batch * g->num_kv_heads * a.nfull * 2;
  a.dhkv = make_fastdiv((uint32_t)g->num_kv_heads);
  a.dnfull = make_fastdiv((uint32_t)a.nfull);
  return a;
}

kvarn_status prefill_impl(const kvarn_geom* gin, void* cache, const void* k, const void* v, int32_t T,
                          float* wk, float* wv, float* yk, float* yv, void* stream) {
  RESOLVE(gin, g);
  kvarn_status st = check_prefill(g, cache, k, v, T);
  if (st != KVARN_OK) return st;
  for (const float* p : {wk, wv, yk, yv})
    if (p && !aligned16(p)) return KVARN_ERR_ALIGN;
  if (prefill_blocks(g, T) * 64 * (g->group / 32) > kMaxWorkItems) return KVARN_ERR_RANGE;
  PrefillArgs a = prefill_args(g, T);
  a.cache = static_cast<uint8_t*>(cache);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.wk = wk;
  a.wv = wv;
  a.yk = yk;
  a.yv = yv;
  return dev(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int kvarn_format_version(void) { return kVersion; }

const char* kvarn_status_str(kvarn_status s) {
  // a C caller may pass any int: read the argument's bits, not an enum value C++ may assume
  // to lie in the enumeration's range
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case KVARN_OK: return "ok";
    case KVARN_ERR_NULL: return "null pointer";
    case KVARN_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KVARN_ERR_GEOM: return "inconsistent geometry";
    case KVARN_ERR_UNSUPPORTED: return "unsupported geometry (head_dim 128, group 32/64, 2-4 bits, <= 8 VarN iterations, variant bits 1|2|4|8)";
    case KVARN_ERR_RANGE: return "size out of range";
    case KVARN_ERR_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

kvarn_status kvarn_cache_bytes(const kvarn_geom* gin, size_t* bytes) {
  RESOLVE(gin, g);
  if (!bytes) return KVARN_ERR_NULL;
  *bytes = (size_t)make_layout(*g).total;
  return KVARN_OK;
}

kvarn_status kvarn_cache_init(const kvarn_geom* gin, void* cache, const int8_t* signs_host, void* stream) {
  RESOLVE(gin, g);
  if (!cache || !signs_host) return KVARN_ERR_NULL;
  if (!aligned16(cache)) return KVARN_ERR_ALIGN;
  for (int j = 0; j < kD; ++j)
    if (signs_host[j] != 1 && signs_host[j] != -1) return KVARN_ERR_RANGE;
  InitArgs a{};
  a.cache = static_cast<uint8_t*>(cache);
  a.geom[0] = g->batch;
  a.geom[1] = g->num_kv_heads;
  a.geom[2] = g->head_dim;
  a.geom[3] = g->capacity;
  a.geom[4] = g->group;
  a.geom[5] = g->varn_iters;
  a.geom[6] = g->bits;
  a.variant = (uint32_t)g->variant;
  a.num_pages = g->num_pages;
  memcpy(a.sigma, signs_host, kD);
  a.n_len = 2LL * g->batch * g->num_kv_heads;
  const Layout L = make_layout(*g);
  a.hdr_bytes = L.header;
  a.map_off = L.map_off;
  a.map_end = g->num_pages > 0 ? L.map_off + 4LL * g->batch * L.tiles : L.map_off;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const kvarn_status st = dev(launch_init(a, hs));
  if (st != KVARN_OK) return st;
  return dev(hipStreamSynchronize(hs));
}

kvarn_status kvarn_quantize_prefill(const kvarn_geom* g, void* cache, const void* k_bf16, const void* v_bf16,
                                    int32_t num_tokens, void* stream) {
  return prefill_impl(g, cache, k_bf16, v_bf16, num_tokens, nullptr, nullptr, nullptr, nullptr, stream);
}

kvarn_status kvarn_quantize_prefill_layers(const kvarn_geom* gin, int32_t n_layers, void* const* caches,
                                           const void* const* k_bf16, const void* const* v_bf16,
                                           int32_t num_tokens, void* stream) {
  RESOLVE(gin, g);
  if (!caches || !k_bf16 || !v_bf16) return KVARN_ERR_NULL;
  if (n_layers < 1 || n_layers > KVARN_MAX_PREFILL_LAYERS) return KVARN_ERR_RANGE;
  for (int32_t i = 0; i < n_layers; ++i) {
    const kvarn_status st = check_prefill(g, caches[i], k_bf16[i], v_bf16[i], num_tokens);
    if (st != KVARN_OK) return st;
  }
  {  // distinct caches: two entries writing one cache would race
    uintptr_t sorted[KVARN_MAX_PREFILL_LAYERS];
    for (int32_t i = 0; i < n_layers; ++i) sorted[i] = (uintptr_t)caches[i];
    std::sort(sorted, sorted + n_layers);
    for (int32_t i = 1; i < n_layers; ++i)
      if (sorted[i] == sorted[i - 1]) return KVARN_ERR_GEOM;
  }
  // layers per launch: at most kMaxLayersPerLaunch, and fewer work-items than 2^32
  const long long per_layer = prefill_blocks(g, num_tokens) * 64 * (g->group / 32);
  const long long fit = kMaxWorkItems / per_layer;
  if (fit < 1) return KVARN_ERR_RANGE;
  const int32_t step = fit < kMaxLayersPerLaunch ? (int32_t)fit : kMaxLayersPerLaunch;
  const PrefillArgs a = prefill_args(g, num_tokens);
  for (int32_t l0 = 0; l0 < n_layers; l0 += step) {
    const int n = n_layers - l0 < step ? n_layers - l0 : step;
    PrefillLayers ly{};
    for (int i = 0; i < n; ++i) {
      ly.cache[i] = static_cast<uint8_t*>(caches[l0 + i]);
      ly.k[i] = static_cast<const uint16_t*>(k_bf16[l0 + i]);
      ly.v[i] = static_cast<const uint16_t*>(v_bf16[l0 + i]);
    }
    const kvarn_status st = dev(launch_prefill_layers(a, ly, n, static_cast<hipStream_t>(stream)));
    if (st != KVARN_OK) return st;
  }
  return KVARN_OK;
}

kvarn_status kvarn_debug_prefill(const kvarn_geom* g, void* cache, const void* k_bf16, const void* v_bf16,
                                 int32_t num_tokens, float* w_k, float* w_v, float* y_k, float* y_v,
                                 void* stream) {
  return prefill_impl(g, cache, k_bf16, v_bf16, num_tokens, w_k, w_v, y_k, y_v, stream);
}

kvarn_status kvarn_append_decode(const kvarn_geom* gin, void* cache, const void* k_bf16, const void* v_bf16,
                                 void* stream) {
  RESOLVE(gin, g);
  if (!cache || !k_bf16 || !v_bf16) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(k_bf16) || !aligned16(v_bf16)) return KVARN_ERR_ALIGN;
  AppendArgs a{};
  a.L = make_layout(*g);
  a.cache = static_cast<uint8_t*>(cache);
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.v = static_cast<const uint16_t*>(v_bf16);
  return dev(launch_append(a, static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_append_tokens(const kvarn_geom* gin, void* cache, const void* k_bf16, const void* v_bf16,
                                 int32_t num_tokens, const int32_t* counts, void* stream) {
  RESOLVE(gin, g);
  if (!cache || ((!k_bf16 || !v_bf16) && num_tokens > 0)) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(k_bf16) || !aligned16(v_bf16) || ((uintptr_t)counts & 3u)) return KVARN_ERR_ALIGN;
  if (num_tokens < 0 || num_tokens > g->capacity) return KVARN_ERR_RANGE;
  if (num_tokens == 0) return KVARN_OK;
  TokensArgs a{};
  a.L = make_layout(*g);
  a.cache = static_cast<uint8_t*>(cache);
  a.k = static_cast<const uint16_t*>(k_bf16);
  a.v = static_cast<const uint16_t*>(v_bf16);
  a.counts = counts;
  a.T = num_tokens;
  a.max_tiles = (g->group - 1 + num_tokens) / g->group;
  const long long jobs = (long long)g->batch * a.max_tiles * 2 * g->num_kv_heads;
  if (jobs >= (1LL << 31)) return KVARN_ERR_RANGE;
  a.jobs = (int)jobs;
  a.dhkv = make_fastdiv((uint32_t)g->num_kv_heads);
  a.dmt = make_fastdiv((uint32_t)a.max_tiles);
  return dev(launch_tokens(a, static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_cache_set_pages(const kvarn_geom* gin, void* cache, const int32_t* pages, int32_t tile_first,
                                   int32_t num_tiles, void* stream) {
  RESOLVE(gin, g);
  if (g->num_pages == 0) return KVARN_ERR_GEOM;
  if (!cache || (!pages && num_tiles > 0)) return KVARN_ERR_NULL;
  if (!aligned16(cache) || ((uintptr_t)pages & 3u)) return KVARN_ERR_ALIGN;
  const int tiles = g->capacity / g->group;
  if (tile_first < 0 || num_tiles < 0 || tile_first > tiles || num_tiles > tiles - tile_first) return KVARN_ERR_RANGE;
  if (num_tiles == 0) return KVARN_OK;
  SetPagesArgs a{};
  a.L = make_layout(*g);
  a.cache = static_cast<uint8_t*>(cache);
  a.pages = pages;
  a.tile_first = tile_first;
  a.n = num_tiles;
  return dev(launch_set_pages(a, static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_dequantize(const kvarn_geom* gin, const void* cache, void* k_out, void* v_out, int32_t max_tokens,
                              int32_t out_dtype, void* stream) {
  RESOLVE(gin, g);
  if (!cache || ((!k_out || !v_out) && max_tokens > 0)) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(k_out) || !aligned16(v_out)) return KVARN_ERR_ALIGN;
  if (max_tokens < 0 || max_tokens > g->capacity) return KVARN_ERR_RANGE;
  if (out_dtype != KVARN_OUT_F32 && out_dtype != KVARN_OUT_BF16) return KVARN_ERR_UNSUPPORTED;
  if (max_tokens == 0) return KVARN_OK;
  DequantArgs a{};
  a.L = make_layout(*g);
  a.cache = static_cast<const uint8_t*>(cache);
  a.ko = k_out;
  a.vo = v_out;
  a.maxT = max_tokens;
  a.bf16out = out_dtype == KVARN_OUT_BF16;
  a.nblk = (max_tokens + 31) / 32;
  const long long jobs = (long long)g->batch * g->num_kv_heads * 2 * a.nblk;
  if (jobs >= (1LL << 31)) return KVARN_ERR_RANGE;  // defensive: check_geom's bound keeps it below 2^29
  if (((jobs + 3) / 4) * 256 > kMaxWorkItems) return KVARN_ERR_RANGE;  // work-items of the launch
  a.jobs = (int)jobs;
  a.dhkv = make_fastdiv((uint32_t)g->num_kv_heads);
  a.dnblk = make_fastdiv((uint32_t)a.nblk);
  return dev(launch_dequant(a, static_cast<hipStream_t>(stream)));
}

// Work split of attn_decode: a work-group of 4 waves per (batch, kv head, group of up to
// 4 query heads, span), the full tiles of a sequence cut into nspan equal spans. nspan is
// chosen for about KVARN_ATTN_WG_TARGET work-groups, with at most 16 and at least 2 tiles
// per wave at the capacity. Depends only on the geometry, so the workspace size is static.
#ifndef KVARN_ATTN_WG_TARGET
#define KVARN_ATTN_WG_TARGET 2048
#endif
static int attn_split(const Geo* g, int grp) {
  const long long tiles = g->capacity / g->group;
  const long long units = (long long)g->batch * g->num_kv_heads * ((grp + 3) / 4);
  long long ns = (KVARN_ATTN_WG_TARGET + units - 1) / units;
  ns = std::max(ns, (tiles + 63) / 64);
  ns = std::min(ns, std::max(1LL, tiles / 8));
  return (int)ns;
}

// Workspace: the span partials [B][Hq][nspan][4 + D] f32, then len [B][Hkv] i32 as the
// tile pass saw it.
static size_t attn_partial_bytes(const Geo* g, int32_t num_q_heads) {
  const int nspan = attn_split(g, num_q_heads / g->num_kv_heads);
  return (size_t)g->batch * num_q_heads * nspan * (4 + kD) * sizeof(float);
}

static kvarn_status ws_need(const Geo* g, int32_t num_q_heads, size_t* bytes) {
  if (num_q_heads <= 0 || num_q_heads % g->num_kv_heads != 0) return KVARN_ERR_GEOM;
  if ((long long)g->batch * num_q_heads >= (1LL << 31)) return KVARN_ERR_RANGE;
  const size_t lens = ((size_t)g->batch * g->num_kv_heads * sizeof(int32_t) + 15) / 16 * 16;
  *bytes = attn_partial_bytes(g, num_q_heads) + lens;
  return KVARN_OK;
}

kvarn_status kvarn_attn_workspace_bytes(const kvarn_geom* gin, int32_t num_q_heads, size_t* bytes) {
  RESOLVE(gin, g);
  if (!bytes) return KVARN_ERR_NULL;
  return ws_need(g, num_q_heads, bytes);
}

static kvarn_status attn_impl(const kvarn_geom* gin, const void* cache, const void* q_bf16, int32_t num_q_heads,
                              float softmax_scale, uint32_t flags, void* workspace, size_t workspace_bytes,
                              float* out, void* cache_rw, const void* k_bf16, const void* v_bf16, void* stream) {
  RESOLVE(gin, g);
  size_t need = 0;
  kvarn_status st = ws_need(g, num_q_heads, &need);
  if (st != KVARN_OK) return st;
  if (!cache || !q_bf16 || !workspace || !out) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(q_bf16) || !aligned16(workspace) || !aligned16(out)) return KVARN_ERR_ALIGN;
  if (cache_rw && (!k_bf16 || !v_bf16)) return KVARN_ERR_NULL;
  if (cache_rw && (!aligned16(k_bf16) || !aligned16(v_bf16))) return KVARN_ERR_ALIGN;
  if (workspace_bytes < need) return KVARN_ERR_RANGE;
  if ((flags & ~(uint32_t)KVARN_Q_PREROTATED) != 0) return KVARN_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVARN_ERR_RANGE;
  AttnArgs a{};
  a.L = make_layout(*g);
  a.cache = static_cast<const uint8_t*>(cache);
  a.q = static_cast<const uint16_t*>(q_bf16);
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.Hq = num_q_heads;
  a.grp = num_q_heads / g->num_kv_heads;
  a.nqg = (a.grp + 3) / 4;
  a.nspan = attn_split(g, a.grp);
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)kD);
  a.flags = flags;
  a.idr = (g->variant & KVARN_VARIANT_NO_ROTATION) != 0;
  a.lens_ws = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + attn_partial_bytes(g, num_q_heads));
  a.cache_rw = static_cast<uint8_t*>(cache_rw);
  a.kn = static_cast<const uint16_t*>(k_bf16);
  a.vn = static_cast<const uint16_t*>(v_bf16);
  return dev(launch_attn(a, static_cast<hipStream_t>(stream)));
}

kvarn_status kvarn_attn_decode(const kvarn_geom* g, const void* cache, const void* q_bf16, int32_t num_q_heads,
                               float softmax_scale, uint32_t flags, void* workspace, size_t workspace_bytes,
                               float* out, void* stream) {
  return attn_impl(g, cache, q_bf16, num_q_heads, softmax_scale, flags, workspace, workspace_bytes, out, nullptr,
                   nullptr, nullptr, stream);
}

kvarn_status kvarn_append_attn_decode(const kvarn_geom* g, void* cache, const void* k_bf16, const void* v_bf16,
                                      const void* q_bf16, int32_t num_q_heads, float softmax_scale, uint32_t flags,
                                      void* workspace, size_t workspace_bytes, float* out, void* stream) {
  if (!cache) return KVARN_ERR_NULL;
  return attn_impl(g, cache, q_bf16, num_q_heads, softmax_scale, flags, workspace, workspace_bytes, out, cache, k_bf16,
                   v_bf16, stream);
}

kvarn_status kvarn_attn_decode_noalloc(const kvarn_geom* gin, const void* cache, const void* q_bf16,
                                       int32_t num_q_heads, float softmax_scale, uint32_t flags, float* out,
                                       void* stream) {
  RESOLVE(gin, g);
  size_t need = 0;
  kvarn_status st = ws_need(g, num_q_heads, &need);
  if (st != KVARN_OK) return st;
  if (need > kAttnScratchBytes) return KVARN_ERR_RANGE;
  if (!cache || !q_bf16 || !out) return KVARN_ERR_NULL;
  if (!aligned16(cache) || !aligned16(q_bf16) || !aligned16(out)) return KVARN_ERR_ALIGN;
  if ((flags & ~(uint32_t)KVARN_Q_PREROTATED) != 0) return KVARN_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVARN_ERR_RANGE;
  void* ws = nullptr;
  if (attn_scratch(&ws) != hipSuccess) return KVARN_ERR_DEVICE;
  return attn_impl(gin, cache, q_bf16, num_q_heads, softmax_scale, flags, ws, kAttnScratchBytes, out, nullptr,
                   nullptr, nullptr, stream);
}

kvarn_status kvarn_cache_flags(const void* cache, void* stream, uint32_t* flags_host) {
  if (!cache || !flags_host) return KVARN_ERR_NULL;
  if (!aligned16(cache)) return KVARN_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t f = 0;
  if (hipMemcpyAsync(&f, static_cast<const uint8_t*>(cache) + kFlagsOff, 4, hipMemcpyDeviceToHost, st) != hipSuccess)
    return KVARN_ERR_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return KVARN_ERR_DEVICE;
  *flags_host = f;
  return KVARN_OK;
}

}  // extern "C"
