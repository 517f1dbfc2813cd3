// Kernel argument blocks and launchers (internal to libkvarn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvarn_common.h"

namespace kvarn {

struct InitArgs {
  uint8_t* cache;
  int32_t geom[7];
  uint32_t variant;  // header byte 40
  int32_t num_pages;  // header byte 44
  int8_t sigma[kD];
  long long n_len;  // entries of len[]
  long long hdr_bytes;  // header size; everything past byte 512 is zeroed except the page map
  long long map_off, map_end;  // page map bytes (set to -1); empty for per-sequence caches
};

struct SetPagesArgs {
  Layout L;
  uint8_t* cache;
  const int32_t* pages;  // [B][n]
  int tile_first, n;
};

// Multi-token append: counts[b] (or T) tokens of k, v per sequence after its stored ones.
struct TokensArgs {
  Layout L;
  uint8_t* cache;
  const uint16_t* k;       // bf16 [B][T][Hkv][D]
  const uint16_t* v;
  const int32_t* counts;   // [B] or nullptr
  int T;
  int max_tiles;           // groups one sequence can complete: (G - 1 + T) / G
  int jobs;                // B * max_tiles * 2 * Hkv tile jobs
  FastDiv dhkv, dmt;       // division by Hkv and by max_tiles
};

struct PrefillArgs {
  Layout L;
  uint8_t* cache;
  const uint16_t* k;  // bf16 [B][T][Hkv][D]
  const uint16_t* v;
  int T, nfull;       // tokens; full tiles per sequence
  int jobs;           // B * Hkv * nfull * 2 tile-streams (< 2^31, checked on the host)
  FastDiv dhkv, dnfull;  // division by Hkv and by nfull
  float *wk, *wv, *yk, *yv;  // optional fp32 intermediates [B][nfull*G][Hkv][D]
};

// Per-layer pointers of a multi-layer prefill launch (kernel argument, at most
// kMaxLayersPerLaunch layers; the host splits longer lists over several launches).
constexpr int kMaxLayersPerLaunch = 64;
struct PrefillLayers {
  uint8_t* cache[kMaxLayersPerLaunch];
  const uint16_t* k[kMaxLayersPerLaunch];
  const uint16_t* v[kMaxLayersPerLaunch];
  uint32_t blocks;  // work-groups per layer
  FastDiv dblocks;  // division by blocks
};

struct AppendArgs {
  Layout L;
  uint8_t* cache;
  const uint16_t* k;  // bf16 [B][Hkv][D]
  const uint16_t* v;
};

struct DequantArgs {
  Layout L;
  const uint8_t* cache;
  void* ko;
  void* vo;
  int maxT, bf16out, nblk;  // nblk = ceil(maxT / 32)
  int jobs;                 // B * Hkv * 2 * nblk (< 2^31)
  FastDiv dhkv, dnblk;      // division by Hkv and by nblk
};

struct AttnArgs {
  Layout L;
  const uint8_t* cache;
  const uint16_t* q;  // bf16 [B][Hq][D]
  float* ws;          // [B][Hq][nspan][4 + D]: m, l, pad, pad, o_rot
  float* out;         // [B][Hq][D]
  int Hq, grp;        // query heads; query heads per kv head
  int nqg;            // groups of up to 4 query heads per kv head
  int nspan;         // spans per sequence: min(nspan, full tiles) equal spans of the length
  float scale;
  uint32_t flags;
  int idr;            // identity in place of H_D (KVARN_VARIANT_NO_ROTATION)
  int32_t* lens_ws;   // [B][Hkv] len at the tile pass, for the merge of a fused call
  // fused append + attention: the call's new token (bf16 [B][Hkv][D]) and the writable
  // cache; kn == nullptr for a plain attention call
  const uint16_t* kn;
  const uint16_t* vn;
  uint8_t* cache_rw;
};

hipError_t launch_init(const InitArgs& a, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_layers(const PrefillArgs& a, PrefillLayers& ly, int n_layers, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t st);
hipError_t launch_set_pages(const SetPagesArgs& a, hipStream_t st);
hipError_t launch_tokens(const TokensArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

// Size of the file-scope workspace of kvarn_attn_decode_noalloc, and its device address on
// the current device (looked up once per device).
constexpr size_t kAttnScratchBytes = (size_t)32 << 20;
hipError_t attn_scratch(void** ptr);

}  // namespace kvarn
