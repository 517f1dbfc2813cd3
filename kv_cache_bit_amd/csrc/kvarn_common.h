// Shared device/host definitions of libkvarn: cache layout, wave shuffles, number formats.
// gfx950 only: wave64, DPP quad permutes, ds_swizzle for in-row exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvarn.h"

namespace kvarn {

constexpr int kD = 128;                     // the one head_dim the kernels support
constexpr uint32_t kMagic = 0x4E52564Bu;    // 'K' 'V' 'R' 'N'
constexpr int kVersion = 3;
constexpr int kHdrFixed = 512;              // len[] offset
constexpr int kSigmaOff = 64;
constexpr int kSignOff = 192;               // sign words [64]: bit 15 / bit 31 of word d set
                                            // where sigma of channel 2d / 2d + 1 is -1
constexpr int kFlagsOff = 36;
constexpr int kVariantOff = 40;
constexpr int kNumPagesOff = 44;
constexpr float kFp16Max = 65504.0f;
constexpr float kInMax = 65536.0f;                      // inputs saturate at +-2^16
constexpr float kScaleMin = 6.103515625e-05f;          // 2^-14
constexpr float kInvSqrtD = 0.08838834764831845f;      // 1/sqrt(128), fp32-rounded

inline __host__ __device__ long long align256(long long n) { return (n + 255) / 256 * 256; }

// The geometry as the library uses it: kvarn_geom's seven fields (bits without the
// KVARN_GEOM_EXT marker) and the extension's variant and num_pages (0 without it).
struct Geo {
  int32_t batch, num_kv_heads, head_dim, capacity, group, varn_iters, bits, variant, num_pages;
};

// Byte layout of one layer cache (format v3), computed on the host and passed by value.
// Records are stored per sequence ([B][Hkv][tiles][2][TR]) or, for a paged cache
// (num_pages > 0), in a pool of pages [num_pages][Hkv][2][TR] named by the page map
// int32 [B][tiles] at map_off; record_at resolves either.
struct Layout {
  int B, Hkv, cap, G, n_it, tiles;  // tiles = cap / G
  int variant;                      // KVARN_VARIANT_* bits
  int num_pages;                    // 0: per-sequence records
  int bits;                         // code width: 2, 3 or 4
  int tr;                           // tile record bytes
  long long header, map_off, tail_off, total;

  __host__ __device__ long long record_seq(int b, int h, int tile, int s) const {
    return header + ((((long long)b * Hkv + h) * tiles + tile) * 2 + s) * tr;
  }
  __host__ __device__ long long page_record(int page, int h, int s) const {
    return header + (((long long)page * Hkv + h) * 2 + s) * tr;
  }
  __host__ __device__ long long tail_row(int b, int h, int s, int slot) const {
    return tail_off + ((((long long)b * Hkv + h) * 2 + s) * G + slot) * (kD * 2);
  }
  __host__ __device__ long long len_off(int b, int h, int s) const {
    return kHdrFixed + (((long long)b * Hkv + h) * 2 + s) * 4;
  }
};

// Division of a 32-bit unsigned n by a fixed d >= 1 without a divide: with l = ceil(log2 d)
// and m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every n < 2^32
// (Granlund and Montgomery, "Division by invariant integers using multiplication", 1994).
// On uniform operands the device side runs on the scalar unit.
struct FastDiv {
  uint32_t m;
  int l;
  uint32_t d;
};
inline __host__ FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) d = 1;
  int l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{(uint32_t)m, l, d};
}
#if defined(__HIPCC__)
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.l);
}
#endif

inline __host__ Layout make_layout(const Geo& g) {
  Layout L;
  L.B = g.batch;
  L.Hkv = g.num_kv_heads;
  L.cap = g.capacity;
  L.G = g.group;
  L.n_it = g.varn_iters;
  L.variant = g.variant;
  L.num_pages = g.num_pages;
  L.bits = g.bits;
  L.tiles = g.capacity / g.group;
  L.tr = g.group * kD * g.bits / 8 + 2 * g.group + 6 * kD;
  L.map_off = kHdrFixed + 8LL * g.batch * g.num_kv_heads;
  L.header = align256(L.map_off + (g.num_pages > 0 ? 4LL * g.batch * L.tiles : 0));
  const long long pool = g.num_pages > 0 ? (long long)g.num_pages * g.num_kv_heads * 2 * L.tr
                                         : (long long)g.batch * g.num_kv_heads * L.tiles * 2 * L.tr;
  L.tail_off = L.header + align256(pool);
  L.total = L.tail_off + align256((long long)g.batch * g.num_kv_heads * 2 * g.group * kD * 2);
  return L;
}

#if defined(__HIPCC__)
// Byte offset of the record of (b, h, tile, s), or -1 when a paged cache names no valid
// page for that tile (writers then drop the tile, readers skip it).
__device__ __forceinline__ long long record_at(const uint8_t* cache, const Layout& L, int b, int h, int tile,
                                               int s) {
  if (L.num_pages == 0) return L.record_seq(b, h, tile, s);
  const int page = reinterpret_cast<const int32_t*>(cache + L.map_off)[(long long)b * L.tiles + tile];
  if (page < 0 || page >= L.num_pages) return -1;
  return L.page_record(page, h, s);
}

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------------------- lane exchange
// Every control used here reads a valid lane for every lane, so no "old" value is needed.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane ^ 7 within the row), row_mirror (lane ^ 15), row_ror:8 (lane ^ 8),
// row_newbcast:n (lane n of the row to all 16)
constexpr int kQx1 = 0xB1, kQx2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140, kRor8 = 0x128, kNewBcast = 0x150;

// Cross-lane min/max on values the compiler cannot prove canonical (they come
// through DPP / permlane as integers): plain v_min/v_max, no NaN quieting needed
// for the finite values that reach them.
__device__ __forceinline__ float vmin(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Orders LDS traffic of one wave against itself: LDS operations of a wave complete in
// issue order, so a compiler fence at wavefront scope is all a wave-private buffer needs.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// xor-partner exchange inside a wave. Masks 1 and 2 use DPP quad permutes (no LDS
// traffic); 4, 8 and 16 use ds_swizzle's bit-mask mode (within 32 lanes); 32 uses
// ds_bpermute.
template <int M>
__device__ __forceinline__ float xshfl(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4 || M == 8 || M == 16) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F));
  } else {
    static_assert(M == 32, "xor mask");
    return __shfl_xor(v, 32);
  }
}

template <int M>
__device__ __forceinline__ uint32_t xshfl_u(uint32_t v) {
  return (uint32_t)__float_as_int(xshfl<M>(__int_as_float((int)v)));
}

// Sum over the 16 lanes of a row (lanes sharing lane>>4). Each stage adds a lane's
// value to its partner's; addition is commutative, so every lane ends bit-identical.
__device__ __forceinline__ float row16_sum(float v) {
  v += xshfl<1>(v);
  v += xshfl<2>(v);
  v += xshfl<4>(v);
  v += xshfl<8>(v);
  return v;
}
// Sum over the 4 rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float col4_sum(float v) {
  v += xshfl<16>(v);
  v += xshfl<32>(v);
  return v;
}
__device__ __forceinline__ float col4_min(float v) {
  v = fminf(v, xshfl<16>(v));
  return fminf(v, xshfl<32>(v));
}
__device__ __forceinline__ float col4_max(float v) {
  v = fmaxf(v, xshfl<16>(v));
  return fmaxf(v, xshfl<32>(v));
}

// ----------------------------------------------------------------------------- number formats
__device__ __forceinline__ float bf16lo(uint32_t w) { return __int_as_float((int)(w << 16)); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __int_as_float((int)(w & 0xFFFF0000u)); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t f16bits(float x) {  // RNE, x assumed within fp16 range
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }

// Exact product of two fp16 values taken from the same half (low: HI = 0, high: HI = 1)
// of two packed registers, one v_fma_mix_f32 (an fp16 x fp16 product fits fp32 exactly).
template <int HI>
__device__ __forceinline__ float mul_f16(uint32_t a, uint32_t b) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a), "v"(b));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ----------------------------------------------------------------------------- Hadamard
__device__ __forceinline__ void fwht8(float (&a)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float x = a[e], y = a[e + h];
        a[e] = x + y;
        a[e + h] = x - y;
      }
    }
  }
}

// Butterfly across lanes differing in bit M: the lane with the bit clear keeps
// own + partner, the lane with it set keeps partner - own.
template <int M>
__device__ __forceinline__ void xstage(float (&a)[8], int cg) {
  const float sgn = (cg & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = fmaf(a[e], sgn, xshfl<M>(a[e]));
}

// Unnormalized Sylvester-ordered Walsh-Hadamard transform of the 128-vector held by
// the 16 lanes of a row (channel 8*cg + e): out[n] = sum_k in[k] (-1)^popcount(k & n).
__device__ __forceinline__ void fwht128(float (&a)[8], int cg) {
  fwht8(a);
  xstage<1>(a, cg);
  xstage<2>(a, cg);
  xstage<4>(a, cg);
  xstage<8>(a, cg);
}

__device__ __forceinline__ void load_sigma(const uint8_t* hdr, int cg, float (&sg)[8]) {
  const uint2 w = *reinterpret_cast<const uint2*>(hdr + kSigmaOff + 8 * cg);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sg[e] = (float)(int8_t)((w.x >> (8 * e)) & 0xFF);
    sg[e + 4] = (float)(int8_t)((w.y >> (8 * e)) & 0xFF);
  }
}

// Non-temporal 16-byte global accesses, for data a kernel streams exactly once (inputs
// read once, outputs it never reads again): the hint keeps them from displacing cached
// lines that are reused.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ void store8f(float* p, const float (&a)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(a[0], a[1], a[2], a[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(a[4], a[5], a[6], a[7]);
}

#endif  // __HIPCC__

}  // namespace kvarn
