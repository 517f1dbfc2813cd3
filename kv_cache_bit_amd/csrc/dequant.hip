// KVarN inverse path on gfx950: dequantization of the 2-bit cache, and the header
// writer used by kvarn_cache_init.
//
// Dequantization undoes the grid and both VarN scales (ai-paper-analysis page,
// section 3.2: the grouped scales are restored at dequantization) and rotates back
// by H_D^T = H_syl diag(sigma) / sqrt(D) (section 3.1). One wave per 32-token block;
// lane = 16 rg + cg holds tokens 8 rg + i and channels 8 cg + e, so the inverse
// Walsh-Hadamard transform is 3 in-lane butterfly stages plus 4 across the row.
#include "kvarn_common.h"
#include "kvarn_launch.h"

namespace kvarn {

__device__ __forceinline__ void widen8_f16(const uint4 w, float (&x)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = f16lo(ws[k]);
    x[2 * k + 1] = f16hi(ws[k]);
  }
}

// ----------------------------------------------------------------------------- dequantize
// One wave per 32-token block of one (b, h, s): undo grid and scales, rotate back.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: job math on the SALU
  const int lane = threadIdx.x & 63;
  const int rg = lane >> 4, cg = lane & 15;
  const Layout& L = a.L;
  const uint32_t job = blockIdx.x * 4u + (uint32_t)wave;
  if (job >= (uint32_t)a.jobs) return;
  // job = ((b * nblk + blk) * 2 + s) * Hkv + h
  const uint32_t q1 = fdiv(job, a.dhkv), q2 = q1 >> 1, q3 = fdiv(q2, a.dnblk);
  const int h = (int)(job - q1 * (uint32_t)L.Hkv);
  const int s = (int)(q1 & 1u);
  const int blk = (int)(q2 - q3 * (uint32_t)a.nblk);
  const int b = (int)q3;
  const int n = *reinterpret_cast<const int32_t*>(a.cache + L.len_off(b, h, s));
  const int nfull = n / L.G;
  const int t0 = blk * 32 + rg * 8;
  void* outp = s ? a.vo : a.ko;
  // sgn[d]: sign bits XORed into the output of channels (2d, 2d + 1) of the lane, at bits
  // 15 and 31 (a packed bf16 pair's sign bits): sigma for rotated tokens, 0 otherwise
  // output row of this lane's first token (t0), and the step from one token to the next
  const long long off0 = (((long long)b * a.maxT + t0) * L.Hkv + h) * kD + 8 * cg;
  const long long tstep = (long long)L.Hkv * kD;
  auto store_row = [&](int t, const float (&y)[8], const uint32_t (&sgn)[4]) {
    if (t >= a.maxT) return;
    const long long off = off0 + (t - t0) * tstep;
    if (a.bf16out) {  // round half to even (v_cvt_pk_bf16_f32), then the sign
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){y[2 * d], y[2 * d + 1]}, bf2v)) ^ sgn[d];
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(outp) + off) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      float z[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        z[2 * d] = __int_as_float(__float_as_int(y[2 * d]) ^ (int)(sgn[d] << 16));
        z[2 * d + 1] = __int_as_float(__float_as_int(y[2 * d + 1]) ^ (int)(sgn[d] & 0x80000000u));
      }
      store8f(reinterpret_cast<float*>(outp) + off, z);
    }
  };
  const uint32_t nosign[4] = {0u, 0u, 0u, 0u};
  const int tile = (blk * 32) / L.G;
  const long long roff = tile < nfull ? record_at(a.cache, L, b, h, tile, s) : 0;
  if (tile < nfull && roff < 0) {  // paged cache without a page for this tile: zeros
    const float zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) store_row(blk * 32 + rg * 8 + i, zero, nosign);
  } else if (tile < nfull) {
    const uint8_t* rec = a.cache + roff;
    const int G = L.G;
    const int ro = G * kD * L.bits / 8, co = ro + 2 * G, so = co + 2 * kD, zo = so + 2 * kD;
    const int tw0 = (blk * 32) % G + rg * 8;
    float cj[8], sj[8], zj[8], ri[8];
    widen8_f16(*reinterpret_cast<const uint4*>(rec + co + 16 * cg), cj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + so + 16 * cg), sj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + zo + 16 * cg), zj);
    widen8_f16(*reinterpret_cast<const uint4*>(rec + ro + 2 * tw0), ri);
    float w[8][8];
    if (s == 0) {
      // channel j = 8cg + e = 16m + 2w + d (m = cg/2, w = 4(cg%2) + e/2, d = e%2) sits in
      // word w at slot 4(m/2) + m%2 + 2d
      const int sbase = 2 * (4 * (cg >> 2) + ((cg >> 1) & 1));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 q4 = *reinterpret_cast<const uint4*>(rec + (tw0 + i) * 32 + 16 * (cg & 1));
        const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) w[i][e] = (float)((qw[e >> 1] >> (sbase + 4 * (e & 1))) & 3u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hq = *reinterpret_cast<const uint16_t*>(rec + (8 * cg + e) * (G / 4) + tw0 / 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i][e] = (float)((hq >> (2 * i)) & 3u);
      }
    }
    // plane B of 3- and 4-bit codes (the code is plane A + 4 * plane B)
    const uint8_t* pb = rec + G * kD / 4;
    if (L.bits == 4) {  // the 2-bit layout again
      if (s == 0) {
        const int sbase = 2 * (4 * (cg >> 2) + ((cg >> 1) & 1));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 q4 = *reinterpret_cast<const uint4*>(pb + (tw0 + i) * 32 + 16 * (cg & 1));
          const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) w[i][e] += 4.0f * (float)((qw[e >> 1] >> (sbase + 4 * (e & 1))) & 3u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hq = *reinterpret_cast<const uint16_t*>(pb + (8 * cg + e) * (G / 4) + tw0 / 4);
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i][e] += 4.0f * (float)((hq >> (2 * i)) & 3u);
        }
      }
    } else if (L.bits == 3) {  // the 1-bit layout
      if (s == 0) {
        // channel 8cg + e: 2-bit word wd = 4(cg%2) + e/2, slot k = 4(m/2) + m%2 + 2(e%2) with
        // m = cg/2; its bit: word wd/2 of the token's four, bit 4(k/2) + k%2 + 2(wd%2)
        const int m = cg >> 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 q4 = *reinterpret_cast<const uint4*>(pb + (tw0 + i) * 16);
          const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int wd = 4 * (cg & 1) + (e >> 1), k = 4 * (m >> 1) + (m & 1) + 2 * (e & 1);
            const int bit = 4 * (k >> 1) + (k & 1) + 2 * (wd & 1);
            w[i][e] += 4.0f * (float)((qw[wd >> 1] >> bit) & 1u);
          }
        }
      } else {
        // token t = 8o + 2n + par of channel 16 blk + c (blk = i4 + 4hh, i4 = 2ip + ii): word
        // (16 ip + c) G/8 + o, bit 4(n + 4hh) + par + 2ii; this lane's 8 tokens are one octet
        const int blk = cg >> 1, i4 = blk & 3, hh = blk >> 2, ip = i4 >> 1, ii = i4 & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cc = 8 * (cg & 1) + e;
          const uint32_t word = *reinterpret_cast<const uint32_t*>(pb + 4 * ((16 * ip + cc) * (G / 8) + tw0 / 8));
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i][e] += 4.0f * (float)((word >> (4 * ((i >> 1) + 4 * hh) + (i & 1) + 2 * ii)) & 1u);
        }
      }
    }
    // x = r (c s q + c z) H_syl^T diag(sigma) / sqrt(D): the per-channel factors take
    // 1/sqrt(D) (the transform is linear), sigma is a sign flip at the store
    const bool idr = (L.variant & KVARN_VARIANT_NO_ROTATION) != 0;  // uniform
    const float kf = idr ? 1.0f : kInvSqrtD;
    float csj[8], czj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      csj[e] = cj[e] * sj[e] * kf;
      czj[e] = cj[e] * zj[e] * kf;
    }
    uint32_t sgn[4] = {0u, 0u, 0u, 0u};
    if (!idr) {
      const uint2 sw = *reinterpret_cast<const uint2*>(a.cache + kSigmaOff + 8 * cg);  // int8 sigma
      const uint32_t sb[2] = {sw.x, sw.y};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t x = sb[d >> 1] >> (16 * (d & 1));  // bytes: sigma of channels 2d, 2d + 1
        sgn[d] = ((x << 8) & 0x8000u) | ((x << 16) & 0x80000000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[i][e] = ri[i] * fmaf(csj[e], w[i][e], czj[e]);
      if (!idr) fwht128(w[i], cg);
      store_row(blk * 32 + rg * 8 + i, w[i], sgn);
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
      store_row(t, y, nosign);
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
    h32[kFlagsOff / 4] = 0;  // flags
    h32[kVariantOff / 4] = a.variant;
    h32[kNumPagesOff / 4] = (uint32_t)a.num_pages;
  }
  for (int k = t; k < 128; k += blockDim.x) {  // bytes 48..511: pad, sigma, sign words, pad
    const int off = kNumPagesOff + 4 + 4 * k;
    if (off >= kHdrFixed) break;
    uint32_t w = 0;
    if (off >= kSignOff && off < kSignOff + 2 * kD) {  // word d: signs of channels 2d, 2d + 1
      const int d = (off - kSignOff) / 4;
      w = (a.sigma[2 * d] < 0 ? 0x8000u : 0u) | (a.sigma[2 * d + 1] < 0 ? 0x80000000u : 0u);
    } else {
      for (int q = 0; q < 4; ++q) {
        const int byte = off + q;
        if (byte >= kSigmaOff && byte < kSigmaOff + kD) w |= (uint32_t)(uint8_t)a.sigma[byte - kSigmaOff] << (8 * q);
      }
    }
    h32[off / 4] = w;
  }
  for (long long k = kHdrFixed / 4 + t; k < a.hdr_bytes / 4; k += blockDim.x)  // len[], page map, padding
    h32[k] = (k >= a.map_off / 4 && k < a.map_end / 4) ? 0xFFFFFFFFu : 0u;
}

// ----------------------------------------------------------------------------- page map
// Tiles [tile_first, tile_first + n) of every sequence take the pages given (no check of
// the values: readers and writers check each entry when they use it).
__global__ void set_pages_kernel(SetPagesArgs a) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)a.L.B * a.n) return;
  const long long b = i / a.n, t = i - b * a.n;
  reinterpret_cast<int32_t*>(a.cache + a.L.map_off)[b * a.L.tiles + a.tile_first + t] = a.pages[i];
}

// ----------------------------------------------------------------------------- launchers
hipError_t launch_init(const InitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(init_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_set_pages(const SetPagesArgs& a, hipStream_t st) {
  const long long n = (long long)a.L.B * a.n;
  hipLaunchKernelGGL(set_pages_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.jobs + 3) / 4));
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
