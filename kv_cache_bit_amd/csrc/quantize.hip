// KVarN write path on gfx950: prefill quantization, decode append, dequantization.
//
// Method (KVarN pages, ai-paper-analysis page): rotate tokens by a randomized
// Hadamard matrix along head_dim (section 3.1), then VarN -- token-axis and
// channel-axis variance normalization repeated a few times, Sinkhorn-Knopp style,
// with grouped scales undone at dequantization (section 3.2) -- then uniform 2-bit
// quantization with four codes per byte.
//
// Work mapping. A tile is G consecutive tokens x 128 channels of one (batch, kv head,
// stream) and is handled by G/32 waves. Inside a wave, lane = 16*rg + cg holds tokens
// 8*rg + i (i < 8) of its 32-token block and channels 8*cg + e (e < 8): one 16-byte
// load per token. So:
//   * the Hadamard transform is 3 butterfly stages inside the lane plus 4 across the
//     16 lanes of a row (DPP quad permutes, ds_swizzle);
//   * a token-axis sum is 8 in-lane terms plus a 16-lane row reduction;
//   * a channel-axis sum is 8 in-lane terms plus a 4-row reduction, plus an LDS
//     exchange between the G/32 waves of a G=64 tile.
// Every reduction has a fixed order, so results are bit-identical run to run.
#include "kvarn_common.h"
#include "kvarn_launch.h"

namespace kvarn {

// bf16 x 8 (one uint4) -> canonical fp16 values widened to fp32. `amax` tracks the
// largest magnitude seen, so saturation is flagged once per lane, not per element.
__device__ __forceinline__ void canon8_bf16(const uint4 w, float (&x)[8], float& amax) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = bf16lo(ws[k]), hi = bf16hi(ws[k]);
    amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
    x[2 * k] = round_f16(fminf(fmaxf(lo, -kFp16Max), kFp16Max));
    x[2 * k + 1] = round_f16(fminf(fmaxf(hi, -kFp16Max), kFp16Max));
  }
}
__device__ __forceinline__ uint32_t sat_flag(float amax) {
  return amax > kFp16Max ? (uint32_t)KVARN_FLAG_SATURATED : 0u;
}
__device__ __forceinline__ void widen8_f16(const uint4 w, float (&x)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = f16lo(ws[k]);
    x[2 * k + 1] = f16hi(ws[k]);
  }
}
__device__ __forceinline__ uint4 pack8_f16(const float (&x)[8]) {
  uint4 o;
  o.x = f16bits(x[0]) | (f16bits(x[1]) << 16);
  o.y = f16bits(x[2]) | (f16bits(x[3]) << 16);
  o.z = f16bits(x[4]) | (f16bits(x[5]) << 16);
  o.w = f16bits(x[6]) | (f16bits(x[7]) << 16);
  return o;
}

// LDS used by one tile: the record being assembled and the cross-wave channel partials.
template <int NW>
struct TileLds {
  static constexpr int G = 32 * NW;
  static constexpr int TR = G * kD / 4 + 2 * G + 6 * kD;
  uint8_t rec[TR] __attribute__((aligned(16)));
  float red_a[NW][kD];
  float red_b[NW][kD];
};

template <int NW>
__device__ __forceinline__ void chan_reduce_sum(float (&s)[8], TileLds<NW>& sh, int lane, int sub) {
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = col4_sum(s[e]);
  if constexpr (NW > 1) {
    const int cg = lane & 15;
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sh.red_a[sub][8 * cg + e] = s[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = sh.red_a[0][8 * cg + e];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += sh.red_a[w][8 * cg + e];
      s[e] = t;
    }
    __syncthreads();
  }
}

template <int NW>
__device__ __forceinline__ void chan_reduce_minmax(float (&mn)[8], float (&mx)[8], TileLds<NW>& sh,
                                                   int lane, int sub) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = col4_min(mn[e]);
    mx[e] = col4_max(mx[e]);
  }
  if constexpr (NW > 1) {
    const int cg = lane & 15;
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sh.red_a[sub][8 * cg + e] = mn[e];
        sh.red_b[sub][8 * cg + e] = mx[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = sh.red_a[0][8 * cg + e], b = sh.red_b[0][8 * cg + e];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        a = fminf(a, sh.red_a[w][8 * cg + e]);
        b = fmaxf(b, sh.red_b[w][8 * cg + e]);
      }
      mn[e] = a;
      mx[e] = b;
    }
    __syncthreads();
  }
}

// The tile core: canonical tokens x (this lane's 8 tokens x 8 channels) -> tile record
// assembled in sh.rec. Steps follow the ai-paper-analysis page, sections 3.1-3.2.
// Optional fp32 debug copies of W (rotated) and Y (normalized): dbg_* point at this
// lane's first token row, `dstride` elements between its tokens.
template <int NW>
__device__ void tile_core(float (&x)[8][8], const uint8_t* hdr, int lane, int sub, int stream, int n_it,
                          TileLds<NW>& sh, uint32_t& flags, float* dbg_w, float* dbg_y,
                          long long dstride) {
  constexpr int G = 32 * NW;
  const int rg = lane >> 4, cg = lane & 15;

  // 1. randomized Hadamard rotation: W = (x * sigma) H_syl / sqrt(D)
  float sg[8];
  load_sigma(hdr, cg, sg);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] *= sg[e];
    fwht128(x[i], cg);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] *= kInvSqrtD;
  }
  if (dbg_w) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store8f(dbg_w + i * dstride, x[i]);
  }

  // 2. VarN. With cumulative scales, a token pass sets r_t = sqrt(mean_j W_tj^2 / c_j^2)
  //    and a channel pass c_j = sqrt(mean_t W_tj^2 / r_t^2) (the mean square of
  //    W / (r c) along that axis becomes 1); all-zero lines keep their scale.
  float p[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) p[i][e] = x[i][e] * x[i][e];
  float r[8], c[8], u[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = c[k] = u[k] = 1.0f;
  for (int it = 0; it < n_it; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(p[i][e], u[e], s);
      s = row16_sum(s);
      if (s > 0.0f) r[i] = __builtin_amdgcn_sqrtf(s * (1.0f / kD));
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_rcpf(r[i] * r[i]);
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) t = fmaf(p[i][e], v[i], t);
      s[e] = t;
    }
    chan_reduce_sum<NW>(s, sh, lane, sub);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (s[e] > 0.0f) c[e] = __builtin_amdgcn_sqrtf(s[e] * (1.0f / G));
      u[e] = __builtin_amdgcn_rcpf(c[e] * c[e]);
    }
  }

  // 3. stored scales: fp16, clamped to [2^-14, 65504]; normalize with the stored values
  float ir[8], ic[8], r16[8], c16[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float rc = fminf(fmaxf(r[k], kScaleMin), kFp16Max);
    const float cc = fminf(fmaxf(c[k], kScaleMin), kFp16Max);
    if (rc != r[k] || cc != c[k]) flags |= KVARN_FLAG_SCALE_CLAMPED;
    r16[k] = round_f16(rc);
    c16[k] = round_f16(cc);
    ir[k] = 1.0f / r16[k];
    ic[k] = 1.0f / c16[k];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = (x[i][e] * ir[i]) * ic[e];
  if (dbg_y) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store8f(dbg_y + i * dstride, x[i]);
  }

  // 4. per-channel asymmetric min/max 2-bit grid over the tile's G tokens
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = mx[e] = x[0][e];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn[e] = fminf(mn[e], x[i][e]);
      mx[e] = fmaxf(mx[e], x[i][e]);
    }
  }
  chan_reduce_minmax<NW>(mn, mx, sh, lane, sub);
  float s16[8], z16[8], is[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sr = (mx[e] - mn[e]) / 3.0f;
    const float sc = fminf(sr, kFp16Max);
    const float zc = fminf(fmaxf(mn[e], -kFp16Max), kFp16Max);
    if (sc != sr || zc != mn[e]) flags |= KVARN_FLAG_SCALE_CLAMPED;
    s16[e] = round_f16(sc);
    z16[e] = round_f16(zc);
    is[e] = s16[e] > 0.0f ? 1.0f / s16[e] : 0.0f;
  }

  // 5. codes q = clamp(rne((Y - z) / s), 0, 3), packed four per byte into the record
  //    K: byte t*32 + j/4 (channels fastest); V: byte j*G/4 + t/4 (tokens fastest)
  const int tw0 = sub * 32 + rg * 8;  // first token of this lane inside the tile
  uint32_t hv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t hk = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float uu = (x[i][e] - z16[e]) * is[e];
      const uint32_t q = (uint32_t)fminf(fmaxf(__builtin_rintf(uu), 0.0f), 3.0f);
      hk |= q << (2 * e);
      hv[e] |= q << (2 * i);
    }
    if (stream == 0) *reinterpret_cast<uint16_t*>(sh.rec + (tw0 + i) * 32 + 2 * cg) = (uint16_t)hk;
  }
  if (stream != 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint16_t*>(sh.rec + (8 * cg + e) * (G / 4) + tw0 / 4) = (uint16_t)hv[e];
  }
  constexpr int RO = G * kD / 4, CO = RO + 2 * G, SO = CO + 2 * kD, ZO = SO + 2 * kD;
  if (cg == 0) *reinterpret_cast<uint4*>(sh.rec + RO + 2 * tw0) = pack8_f16(r16);
  if (rg == 0 && sub == 0) {
    *reinterpret_cast<uint4*>(sh.rec + CO + 16 * cg) = pack8_f16(c16);
    *reinterpret_cast<uint4*>(sh.rec + SO + 16 * cg) = pack8_f16(s16);
    *reinterpret_cast<uint4*>(sh.rec + ZO + 16 * cg) = pack8_f16(z16);
  }
  __syncthreads();
}

template <int NW>
__device__ __forceinline__ void copy_record(const TileLds<NW>& sh, uint8_t* dst, int lane, int sub) {
  constexpr int N16 = TileLds<NW>::TR / 16;
  const uint4* s = reinterpret_cast<const uint4*>(sh.rec);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int k = sub * 64 + lane; k < N16; k += 64 * NW) d[k] = s[k];
}

__device__ __forceinline__ void raise_flags(uint8_t* hdr, uint32_t f) {
  if (f) atomicOr(reinterpret_cast<uint32_t*>(hdr + kFlagsOff), f);
}

// ----------------------------------------------------------------------------- prefill
// Work-groups [0, tile_blocks) quantize full tiles, 4/NW tiles per work-group; the
// remaining work-groups write the fp16 tail and len[], one (b, h, s) per wave.
template <int NW, bool DBG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int TPW = 4 / NW;
  __shared__ TileLds<NW> sh_all[TPW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane >> 4, cg = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = a.cache;
  uint32_t flags = 0;
  const long long tile_blocks = (a.jobs + TPW - 1) / TPW;

  if ((long long)blockIdx.x >= tile_blocks) {
    const long long sj = ((long long)blockIdx.x - tile_blocks) * 4 + wave;  // (b, h, s)
    if (sj >= 2LL * L.B * L.Hkv) return;
    const int s = (int)(sj % 2), h = (int)((sj / 2) % L.Hkv), b = (int)(sj / 2 / L.Hkv);
    const uint16_t* src = s ? a.v : a.k;
    for (int t = a.nfull * L.G + rg; t < a.T; t += 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + (((long long)b * a.T + t) * L.Hkv + h) * kD + 8 * cg);
      float x[8], amax = 0.0f;
      canon8_bf16(w, x, amax);
      flags |= sat_flag(amax);
      *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, t % L.G) + 16 * cg) = pack8_f16(x);
    }
    if (lane == 0) *reinterpret_cast<int32_t*>(a.cache + L.len_off(b, h, s)) = a.T;
    raise_flags(hdr, flags);
    return;
  }

  const int tw = wave / NW, sub = wave % NW;
  TileLds<NW>& sh = sh_all[tw];
  long long job = (long long)blockIdx.x * TPW + tw;
  const bool valid = job < a.jobs;
  if (!valid) job = 0;  // keep the barrier sequence uniform; results are discarded
  // job = ((b * nfull + tile) * 2 + s) * Hkv + h : neighbouring waves read neighbouring heads
  const int h = (int)(job % L.Hkv);
  const int s = (int)((job / L.Hkv) % 2);
  const int tile = (int)((job / L.Hkv / 2) % a.nfull);
  const int b = (int)(job / L.Hkv / 2 / a.nfull);
  const uint16_t* src = s ? a.v : a.k;
  const int t0 = tile * L.G + sub * 32 + rg * 8;
  float x[8][8], amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + (((long long)b * a.T + t0 + i) * L.Hkv + h) * kD + 8 * cg);
    canon8_bf16(w, x[i], amax);
  }
  flags |= sat_flag(amax);
  float* dw = s ? a.wv : a.wk;
  float* dy = s ? a.yv : a.yk;
  const long long tfull = (long long)a.nfull * L.G;
  const long long doff = (((long long)b * tfull + t0) * L.Hkv + h) * kD + 8 * cg;
  if constexpr (DBG)
    tile_core<NW>(x, hdr, lane, sub, s, L.n_it, sh, flags, (valid && dw) ? dw + doff : nullptr,
                  (valid && dy) ? dy + doff : nullptr, (long long)L.Hkv * kD);
  else
    tile_core<NW>(x, hdr, lane, sub, s, L.n_it, sh, flags, nullptr, nullptr, 0);
  if (valid) {
    copy_record<NW>(sh, a.cache + L.record(b, h, tile, s), lane, sub);
    raise_flags(hdr, flags);
  }
}

// ----------------------------------------------------------------------------- append
// One work-group (G/32 waves) per (b, h, s). The token goes to tail slot len mod G;
// when it completes a group, the group is quantized into the next tile record.
template <int NW>
__global__ __launch_bounds__(64 * NW) void append_kernel(AppendArgs a) {
  constexpr int G = 32 * NW;
  __shared__ TileLds<NW> sh;
  const int sub = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane >> 4, cg = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = a.cache;
  const int s = blockIdx.x % 2, h = (blockIdx.x / 2) % L.Hkv, b = blockIdx.x / 2 / L.Hkv;
  int32_t* lenp = reinterpret_cast<int32_t*>(a.cache + L.len_off(b, h, s));
  const int pos = *lenp;
  if (pos >= L.cap) {
    if (threadIdx.x == 0) raise_flags(hdr, KVARN_FLAG_CAPACITY);
    return;
  }
  uint32_t flags = 0;
  const uint16_t* src = (s ? a.v : a.k) + ((long long)b * L.Hkv + h) * kD + 8 * cg;
  float xin[8], amax = 0.0f;
  canon8_bf16(*reinterpret_cast<const uint4*>(src), xin, amax);
  flags |= sat_flag(amax);
  if (sub == 0 && rg == 0)
    *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, pos % G) + 16 * cg) = pack8_f16(xin);
  if ((pos + 1) % G == 0) {
    float x[8][8];
    const int t0 = sub * 32 + rg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (t0 + i == G - 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = xin[e];
      } else {
        widen8_f16(*reinterpret_cast<const uint4*>(a.cache + L.tail_row(b, h, s, t0 + i) + 16 * cg), x[i]);
      }
    }
    tile_core<NW>(x, hdr, lane, sub, s, L.n_it, sh, flags, nullptr, nullptr, 0);
    copy_record<NW>(sh, a.cache + L.record(b, h, (pos + 1) / G - 1, s), lane, sub);
  }
  raise_flags(hdr, flags);
  __syncthreads();
  if (threadIdx.x == 0) *lenp = pos + 1;
}

// ----------------------------------------------------------------------------- dequantize
// One wave per 32-token block of one (b, h, s): undo grid and scales, rotate back.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane >> 4, cg = lane & 15;
  const Layout& L = a.L;
  const long long job = (long long)blockIdx.x * 4 + wave;
  if (job >= a.jobs) return;
  // job = ((b * nblk + blk) * 2 + s) * Hkv + h
  const int h = (int)(job % L.Hkv);
  const int s = (int)((job / L.Hkv) % 2);
  const int blk = (int)((job / L.Hkv / 2) % a.nblk);
  const int b = (int)(job / L.Hkv / 2 / a.nblk);
  const int n = *reinterpret_cast<const int32_t*>(a.cache + L.len_off(b, h, s));
  const int nfull = n / L.G;
  const int t0 = blk * 32 + rg * 8;
  void* outp = s ? a.vo : a.ko;
  auto store_row = [&](int t, const float (&y)[8]) {
    if (t >= a.maxT) return;
    const long long off = (((long long)b * a.maxT + t) * L.Hkv + h) * kD + 8 * cg;
    if (a.bf16out) {
      uint4 o;
      o.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
      o.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
      o.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
      o.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(outp) + off) = o;
    } else {
      store8f(reinterpret_cast<float*>(outp) + off, y);
    }
  };
  const int tile = (blk * 32) / L.G;
  if (tile < nfull) {
    const uint8_t* rec = a.cache + L.record(b, h, tile, s);
    const int G = L.G;
    const int ro = G * kD / 4, co = ro + 2 * G, so = co + 2 * kD, zo = so + 2 * kD;
    const int tw0 = (blk * 32) % G + rg * 8;
    float cj[8], sj[8], zj[8], ri[8], sg[8];
    widen8_f16(*reinterpret_cast<const uint4*>(rec + co + 16 * cg), cj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + so + 16 * cg), sj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + zo + 16 * cg), zj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + ro + 2 * tw0), ri);
    load_sigma(a.cache, cg, sg);
    float w[8][8];
    if (s == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t hq = *reinterpret_cast<const uint16_t*>(rec + (tw0 + i) * 32 + 2 * cg);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[i][e] = (float)((hq >> (2 * e)) & 3u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hq = *reinterpret_cast<const uint16_t*>(rec + (8 * cg + e) * (G / 4) + tw0 / 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i][e] = (float)((hq >> (2 * i)) & 3u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[i][e] = (ri[i] * cj[e]) * fmaf(sj[e], w[i][e], zj[e]);
      fwht128(w[i], cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[i][e] *= kInvSqrtD * sg[e];
      store_row(blk * 32 + rg * 8 + i, w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + i;
      float y[8];
      if (t < n) {
        widen8_f16(*reinterpret_cast<const uint4*>(a.cache + L.tail_row(b, h, s, t % L.G) + 16 * cg), y);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.0f;
      }
      store_row(t, y);
    }
  }
}

// ----------------------------------------------------------------------------- header
__global__ void init_kernel(InitArgs a) {
  const int t = threadIdx.x;
  uint32_t* h32 = reinterpret_cast<uint32_t*>(a.cache);
  if (t == 0) {
    h32[0] = kMagic;
    h32[1] = kVersion;
    for (int k = 0; k < 7; ++k) h32[2 + k] = (uint32_t)a.geom[k];
    h32[9] = 0;  // flags
  }
  for (int k = t; k < 128; k += blockDim.x) {  // bytes 40..511: pad, sigma, pad
    const int off = 40 + 4 * k;
    if (off >= kHdrFixed) break;
    uint32_t w = 0;
    for (int q = 0; q < 4; ++q) {
      const int byte = off + q;
      if (byte >= kSigmaOff && byte < kSigmaOff + kD) w |= (uint32_t)(uint8_t)a.sigma[byte - kSigmaOff] << (8 * q);
    }
    h32[off / 4] = w;
  }
  for (long long k = t; k < (long long)a.n_len; k += blockDim.x) h32[kHdrFixed / 4 + k] = 0;
}

// ----------------------------------------------------------------------------- launchers
hipError_t launch_init(const InitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(init_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int tpw = 4 / (a.L.G / 32);
  const long long tile_blocks = (a.jobs + tpw - 1) / tpw;
  const long long tail_blocks = (2LL * a.L.B * a.L.Hkv + 3) / 4;
  const dim3 grid((unsigned)(tile_blocks + tail_blocks));
  const bool dbg = a.wk || a.wv || a.yk || a.yv;
  if (a.L.G == 32) {
    if (dbg)
      hipLaunchKernelGGL((prefill_kernel<1, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<1, false>), grid, dim3(256), 0, st, a);
  } else {
    if (dbg)
      hipLaunchKernelGGL((prefill_kernel<2, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<2, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(2LL * a.L.B * a.L.Hkv));
  if (a.L.G == 32)
    hipLaunchKernelGGL(append_kernel<1>, grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<2>, grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.jobs + 3) / 4));
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
