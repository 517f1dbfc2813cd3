// KVarN inverse path on gfx950: dequantization of the 2-bit cache, and the header
// writer used by kvarn_cache_init.
//
// Dequantization undoes the grid and both VarN scales (ai-paper-analysis page,
// section 3.2: the grouped scales are restored at dequantization) and rotates back
// by H_D^T = H_syl diag(sigma) / sqrt(D) (section 3.1). One wave per 32-token block of one
// stream. The lanes are laid out after each stream's code layout: K lanes hold one code
// word (16 channels) of 4 tokens, V lanes 8 channels of 8 tokens; codes become fp32
// through the packed fp4 conversion (3- and 4-bit codes add plane B, brought into the
// same nibble planes by shifts and masks), the inverse Walsh-Hadamard transform runs as
// butterfly stages in registers plus fused DPP stages across lanes, and K's bf16 rows pass
// through LDS so that both streams store whole 256-byte token rows.
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
__device__ __forceinline__ void widen8_bf16(const uint4 w, float (&x)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16lo(ws[k]);
    x[2 * k + 1] = bf16hi(ws[k]);
  }
}

// ----------------------------------------------------------------------------- 2-bit helpers
constexpr uint32_t kNib2 = 0x33333333u;  // bits 0..1 of every nibble
constexpr uint32_t kBit1 = 0x11111111u;  // bit 0 of every nibble

// Two codes from byte BY of a nibble plane as fp32: a 2-bit code zero-extended to a nibble
// is the e2m1 value q/2, which the packed fp4 conversion with scale 2 turns into q.
template <int BY>
__device__ __forceinline__ void cvt2f(uint32_t plane, float& lo, float& hi) {
  const f2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(plane, 2.0f, BY);
  lo = v[0];
  hi = v[1];
}
// The same for plane B of 4-bit codes, worth 4x: scale 8 turns the e2m1 value q_B/2 into 4 q_B.
template <int BY>
__device__ __forceinline__ void cvt2f8(uint32_t plane, float& lo, float& hi) {
  const f2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(plane, 8.0f, BY);
  lo = v[0];
  hi = v[1];
}

// Butterfly stage across lanes in one v_fmac_f32_dpp per element: a <- a + m * a(partner),
// m = +1 where the lane's stage bit is clear and -1 where it is set. A set lane then holds
// own - partner, the negative of its butterfly output; the partner of a lane carries the
// same sign history, so the signs compose into one +-1 per lane, (-1)^(number of set
// stage bits), which the store takes with the sign word. DPP reaches lane ^ 1 and ^ 2
// (quad permutes), ^ 7 (row_half_mirror) and ^ 8 (row_ror:8); with the lane index
// relabelled as T(u) = u ^ (u & 4 ? 3 : 0) (an involution), the partner across ^ 7 is
// T ^ 4, so the four stages are the butterflies on bits 0..3 of T.
//
// The stage is one asm block over 8 registers: its leading s_nop 1 gives the two wait
// states a DPP read needs after a vector ALU write of the same register (the writes before
// the block), and inside the block each register is read long after its last write.
#define KVARN_FMAC_DPP8(CTRL)                                                                           \
  asm volatile("s_nop 1\n"                                                                             \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                       \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                          \
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]) \
               : "v"(m))
template <int CTRL>
__device__ __forceinline__ void xstage_dpp8(float* a, float m) {
  if constexpr (CTRL == kQx1) {
    KVARN_FMAC_DPP8("quad_perm:[1,0,3,2]");
  } else if constexpr (CTRL == kQx2) {
    KVARN_FMAC_DPP8("quad_perm:[2,3,0,1]");
  } else if constexpr (CTRL == kHalfMirror) {
    KVARN_FMAC_DPP8("row_half_mirror");
  } else {
    static_assert(CTRL == kRor8, "DPP control");
    KVARN_FMAC_DPP8("row_ror:8");
  }
}
#undef KVARN_FMAC_DPP8
template <int CTRL, int N>
__device__ __forceinline__ void xstage_dpp(float (&a)[N], float m) {
  static_assert(N % 8 == 0, "stage width");
#pragma unroll
  for (int e = 0; e < N; e += 8) xstage_dpp8<CTRL>(a + e, m);
}
__device__ __forceinline__ int relabel_t(int u) { return u ^ ((u & 4) ? 3 : 0); }

// Unnormalized Walsh-Hadamard transform over the 4 bits of an in-lane index
__device__ __forceinline__ void fwht16(float (&a)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if ((e & h) == 0) {
        const float x = a[e], y = a[e + h];
        a[e] = x + y;
        a[e + h] = x - y;
      }
    }
  }
}

// ----------------------------------------------------------------------------- dequantize
// One wave per 32-token block of one (b, h, s): undo grid and scales, rotate back.
// BITS 2, 3 or 4. Plane A (bits 0..1 of every code) has the 2-bit layout; plane B of
// 4-bit codes repeats it, plane B of 3-bit codes is the 1-bit layout (include/kvarn.h).
// bf16 K rows of a 2-bit block staged in LDS: 32 tokens x 64 dwords, dword column c of
// token row t at t * 64 + (c ^ 8 ((t / 4) % 8)): the lanes of one write (8 token quads x 8
// words) hit 64 distinct banks, and the XOR keeps each aligned 4-dword group together for
// the 16-byte row reads. 32 KB per work-group of 4 waves.
constexpr int kKRow = 64;

__device__ __forceinline__ int kst_col(int t, int c) { return c ^ (8 * ((t >> 2) & 7)); }

template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  constexpr bool PB = BITS > 2;  // with plane B: q = q_A + 4 q_B
  __shared__ uint32_t kst[4][32 * kKRow];
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
      st_nt16(reinterpret_cast<uint16_t*>(outp) + off, make_uint4(o[0], o[1], o[2], o[3]));
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
    const int ro = G * kD * BITS / 8, co = ro + 2 * G, so = co + 2 * kD, zo = so + 2 * kD;
    const uint8_t* recb = rec + G * kD / 4;  // plane B
    const bool idr = (L.variant & KVARN_VARIANT_NO_ROTATION) != 0;  // uniform
    const float kf = idr ? 1.0f : kInvSqrtD;
    const int tb0 = (blk * 32) % G;  // first token of the block inside the tile
    const long long rowstep = (long long)L.Hkv * kD;
    const long long outb = ((long long)b * a.maxT + blk * 32) * rowstep + (long long)h * kD;  // token blk*32, channel 0
    if (s == 0) {
      // K: a token's 128 codes are 8 words; word w holds channels 16 nb + 2 w + d (nb < 8,
      // d < 2) at slot 4 (nb/2) + nb%2 + 2 d. Lane (rg, cg) takes word w = T(cg % 8) of the
      // 4 tokens 4 tq .. 4 tq + 3 (tq = 2 rg + cg/8): its 16 values v[2 nb + d] per token
      // carry channel bits 0 and 4..6 in the lane (4 in-register butterfly stages) and bits
      // 1..3 = w on the lane (3 stages across lanes).
      const int w = relabel_t(cg & 7), tq = 2 * rg + (cg >> 3);
      const int tb = tb0 + 4 * tq;
      uint32_t x[4], xb[PB ? 4 : 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const uint32_t*>(rec + (tb + i) * 32 + 4 * w);
      if constexpr (BITS == 4) {  // word w of the token's plane B
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[i] = *reinterpret_cast<const uint32_t*>(recb + (tb + i) * 32 + 4 * w);
      } else if constexpr (BITS == 3) {
        // one 1-bit word per pair of 2-bit words (w = 2 p + r): the bits of slots 2 n and
        // 2 n + 1 of word w sit at 4 n + 2 r and 4 n + 2 r + 1
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xb[i] = *reinterpret_cast<const uint32_t*>(recb + (tb + i) * 16 + 4 * (w >> 1)) >> (2 * (w & 1));
      }
      const uint2 rw = *reinterpret_cast<const uint2*>(rec + ro + 2 * tb);
      float cs[16], cz[16];  // c s and c z of channel 16 nb + 2 w + d at [2 nb + d]
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(rec + co + 32 * nb + 4 * w);
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(rec + so + 32 * nb + 4 * w);
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(rec + zo + 32 * nb + 4 * w);
        cs[2 * nb] = mul_f16<0>(cw, sw);
        cs[2 * nb + 1] = mul_f16<1>(cw, sw);
        cz[2 * nb] = mul_f16<0>(cw, zw);
        cz[2 * nb + 1] = mul_f16<1>(cw, zw);
      }
      float v[4][16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // nibble plane e: codes of the even channel blocks (byte k: nb = 2k, d = 0 | 1);
        // plane o: the odd blocks
        const uint32_t e = x[i] & kNib2, o = (x[i] >> 2) & kNib2;
        cvt2f<0>(e, v[i][0], v[i][1]);
        cvt2f<0>(o, v[i][2], v[i][3]);
        cvt2f<1>(e, v[i][4], v[i][5]);
        cvt2f<1>(o, v[i][6], v[i][7]);
        cvt2f<2>(e, v[i][8], v[i][9]);
        cvt2f<2>(o, v[i][10], v[i][11]);
        cvt2f<3>(e, v[i][12], v[i][13]);
        cvt2f<3>(o, v[i][14], v[i][15]);
        if constexpr (PB) {  // the code q_A + 4 q_B (exact): plane B converted with scale 8
          const uint32_t eb = BITS == 4 ? xb[i] & kNib2 : xb[i] & kBit1;
          const uint32_t ob = BITS == 4 ? (xb[i] >> 2) & kNib2 : (xb[i] >> 1) & kBit1;
          float u[16];
          cvt2f8<0>(eb, u[0], u[1]);
          cvt2f8<0>(ob, u[2], u[3]);
          cvt2f8<1>(eb, u[4], u[5]);
          cvt2f8<1>(ob, u[6], u[7]);
          cvt2f8<2>(eb, u[8], u[9]);
          cvt2f8<2>(ob, u[10], u[11]);
          cvt2f8<3>(eb, u[12], u[13]);
          cvt2f8<3>(ob, u[14], u[15]);
#pragma unroll
          for (int k = 0; k < 16; ++k) v[i][k] += u[k];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) v[i][k] = fmaf(v[i][k], cs[k], cz[k]);
        if (!idr) fwht16(v[i]);
      }
      uint32_t flip = 0u;  // the lane's butterfly sign as a pair sign mask
      if (!idr) {
        const float m0 = (w & 1) ? -1.0f : 1.0f, m1 = (w & 2) ? -1.0f : 1.0f, m2 = (w & 4) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xstage_dpp<kQx1>(v[i], m0);
          xstage_dpp<kQx2>(v[i], m1);
          xstage_dpp<kHalfMirror>(v[i], m2);
        }
        flip = (__builtin_popcount(w) & 1) ? 0x80008000u : 0u;
      }
      uint32_t sg[8];  // sign words of output channels (16 nb + 2 w, +1), with the lane's sign
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        sg[nb] = idr ? 0u : *reinterpret_cast<const uint32_t*>(a.cache + kSignOff + 32 * nb + 4 * w) ^ flip;
      if (a.bf16out) {
        // bf16 pairs (channels 16 nb + 2 w, +1) into the wave's LDS tile, then each lane
        // stores 16 B of a token row (channels 8 cg .. + 7 of token 8 rg + i): whole
        // 256-byte rows instead of 32-byte pieces
        uint32_t* tile_l = kst[wave];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 4 * tq + i;
          const uint32_t rwi = i < 2 ? rw.x : rw.y;
          const float rk = ((i & 1) ? f16hi(rwi) : f16lo(rwi)) * kf;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            tile_l[tt * kKRow + kst_col(tt, 8 * nb + w)] =
                __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){v[i][2 * nb] * rk, v[i][2 * nb + 1] * rk},
                                                                     bf2v)) ^ sg[nb];
        }
        wave_sync();
        const long long offr = outb + (long long)(rg * 8) * rowstep + 8 * cg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (blk * 32 + rg * 8 + i >= a.maxT) continue;
          const uint4 row = *reinterpret_cast<const uint4*>(&tile_l[(8 * rg + i) * kKRow + kst_col(8 * rg + i, 4 * cg)]);
          st_nt16(reinterpret_cast<uint16_t*>(outp) + offr + i * rowstep, row);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = 4 * tq + i;  // token inside the block
          if (blk * 32 + tt >= a.maxT) continue;
          const uint32_t rwi = i < 2 ? rw.x : rw.y;
          const float rk = ((i & 1) ? f16hi(rwi) : f16lo(rwi)) * kf;
          const long long off = outb + tt * rowstep + 2 * w;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const float z0 = __int_as_float(__float_as_int(v[i][2 * nb] * rk) ^ (int)(sg[nb] << 16));
            const float z1 = __int_as_float(__float_as_int(v[i][2 * nb + 1] * rk) ^ (int)(sg[nb] & 0x80000000u));
            *reinterpret_cast<float2*>(reinterpret_cast<float*>(outp) + off + 16 * nb) = make_float2(z0, z1);
          }
        }
      }
    } else {
      // V: tokens fastest, byte j G/4 + t/4 holds tokens 4 (t/4) .. + 3 of channel j. Lane
      // (rg, cg) takes tokens 8 rg + i and channels 8 T(cg) + e: 3 butterfly stages in the
      // lane, 4 across the row. The two 16-bit words of channels (2k, 2k + 1) give four
      // nibble-plane bytes.
      const int cb = relabel_t(cg);
      const int tw0 = tb0 + rg * 8;
      float cj[8], sj[8], zj[8], ri[8];
      widen8_f16(*reinterpret_cast<const uint4*>(rec + co + 16 * cb), cj);
      widen8_f16(*reinterpret_cast<const uint4*>(rec + so + 16 * cb), sj);
      widen8_f16(*reinterpret_cast<const uint4*>(rec + zo + 16 * cb), zj);
      widen8_f16(*reinterpret_cast<const uint4*>(rec + ro + 2 * tw0), ri);
      float w8[8][8];  // [token i][channel e]
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(rec + (8 * cb + 2 * k) * (G / 4) + tw0 / 4);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(rec + (8 * cb + 2 * k + 1) * (G / 4) + tw0 / 4);
        const uint32_t xx = lo | (hi << 16);
        // byte 0/1: tokens 0..3 / 4..7 of channel 2k, bytes 2/3: of channel 2k + 1; plane e
        // holds tokens 4 m + 0, 2 of byte m's pair, plane o tokens 4 m + 1, 3
        const uint32_t e = xx & kNib2, o = (xx >> 2) & kNib2;
        cvt2f<0>(e, w8[0][2 * k], w8[2][2 * k]);
        cvt2f<0>(o, w8[1][2 * k], w8[3][2 * k]);
        cvt2f<1>(e, w8[4][2 * k], w8[6][2 * k]);
        cvt2f<1>(o, w8[5][2 * k], w8[7][2 * k]);
        cvt2f<2>(e, w8[0][2 * k + 1], w8[2][2 * k + 1]);
        cvt2f<2>(o, w8[1][2 * k + 1], w8[3][2 * k + 1]);
        cvt2f<3>(e, w8[4][2 * k + 1], w8[6][2 * k + 1]);
        cvt2f<3>(o, w8[5][2 * k + 1], w8[7][2 * k + 1]);
        if constexpr (PB) {  // + 4 q_B, in the same nibble planes as e and o, scale 8
          uint32_t eb, ob;
          if constexpr (BITS == 4) {
            const uint32_t lb = *reinterpret_cast<const uint16_t*>(recb + (8 * cb + 2 * k) * (G / 4) + tw0 / 4);
            const uint32_t hb =
                *reinterpret_cast<const uint16_t*>(recb + (8 * cb + 2 * k + 1) * (G / 4) + tw0 / 4);
            const uint32_t xb2 = lb | (hb << 16);
            eb = xb2 & kNib2;
            ob = (xb2 >> 2) & kNib2;
          } else {
            // channel 16 cbk + cc (cbk = 4 hh + 2 ip + ii): the bits of its tokens 8 o + 2 n
            // and 8 o + 2 n + 1 are bits 4 (n + 4 hh) + 2 ii (+1) of 1-bit word
            // (16 ip + cc) G/8 + o; channels 2k and 2k + 1 of this lane share cbk
            const int c0 = 8 * cb + 2 * k, cbk = c0 >> 4, cc = c0 & 15;
            const int sh = 16 * (cbk >> 2) + 2 * (cbk & 1);
            const uint8_t* wp = recb + 4 * ((16 * ((cbk >> 1) & 1) + cc) * (G / 8) + tw0 / 8);
            const uint32_t y0 = *reinterpret_cast<const uint32_t*>(wp) >> sh;
            const uint32_t y1 = *reinterpret_cast<const uint32_t*>(wp + 4 * (G / 8)) >> sh;
            eb = (y0 & 0x1111u) | ((y1 & 0x1111u) << 16);
            ob = ((y0 >> 1) & 0x1111u) | (((y1 >> 1) & 0x1111u) << 16);
          }
          float u[16];  // token i of channel 2k at u[i], of channel 2k + 1 at u[8 + i]
          cvt2f8<0>(eb, u[0], u[2]);
          cvt2f8<0>(ob, u[1], u[3]);
          cvt2f8<1>(eb, u[4], u[6]);
          cvt2f8<1>(ob, u[5], u[7]);
          cvt2f8<2>(eb, u[8], u[10]);
          cvt2f8<2>(ob, u[9], u[11]);
          cvt2f8<3>(eb, u[12], u[14]);
          cvt2f8<3>(ob, u[13], u[15]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            w8[i][2 * k] += u[i];
            w8[i][2 * k + 1] += u[8 + i];
          }
        }
      }
      float csj[8], czj[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        csj[e] = cj[e] * sj[e];
        czj[e] = cj[e] * zj[e];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w8[i][e] = fmaf(w8[i][e], csj[e], czj[e]);
        if (!idr) fwht8(w8[i]);
      }
      uint32_t sgn[4] = {0u, 0u, 0u, 0u};
      if (!idr) {
        const float m0 = (cb & 1) ? -1.0f : 1.0f, m1 = (cb & 2) ? -1.0f : 1.0f;
        const float m2 = (cb & 4) ? -1.0f : 1.0f, m3 = (cb & 8) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xstage_dpp<kQx1>(w8[i], m0);
          xstage_dpp<kQx2>(w8[i], m1);
          xstage_dpp<kHalfMirror>(w8[i], m2);
          xstage_dpp<kRor8>(w8[i], m3);
        }
        const uint32_t flip = (__builtin_popcount(cb) & 1) ? 0x80008000u : 0u;
        const uint4 sw = *reinterpret_cast<const uint4*>(a.cache + kSignOff + 16 * cb);  // sign words 4 cb .. +3
        sgn[0] = sw.x ^ flip; sgn[1] = sw.y ^ flip; sgn[2] = sw.z ^ flip; sgn[3] = sw.w ^ flip;
      }
      const long long offv = outb + (long long)(rg * 8) * rowstep + 8 * cb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (blk * 32 + rg * 8 + i >= a.maxT) continue;
        const float rk = ri[i] * kf;
        const long long off = offv + i * rowstep;
        if (a.bf16out) {
          uint32_t o[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            o[d] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){w8[i][2 * d] * rk, w8[i][2 * d + 1] * rk},
                                                                       bf2v)) ^ sgn[d];
          st_nt16(reinterpret_cast<uint16_t*>(outp) + off, make_uint4(o[0], o[1], o[2], o[3]));
        } else {
          float z[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            z[2 * d] = __int_as_float(__float_as_int(w8[i][2 * d] * rk) ^ (int)(sgn[d] << 16));
            z[2 * d + 1] = __int_as_float(__float_as_int(w8[i][2 * d + 1] * rk) ^ (int)(sgn[d] & 0x80000000u));
          }
          store8f(reinterpret_cast<float*>(outp) + off, z);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + i;
      float y[8];
      if (t < n) {
        widen8_bf16(*reinterpret_cast<const uint4*>(a.cache + L.tail_row(b, h, s, t % L.G) + 16 * cg), y);
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
  if (a.L.bits == 2)
    hipLaunchKernelGGL(dequant_kernel<2>, grid, dim3(256), 0, st, a);
  else if (a.L.bits == 3)
    hipLaunchKernelGGL(dequant_kernel<3>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(dequant_kernel<4>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
