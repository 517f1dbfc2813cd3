// KVarN write path on gfx950: prefill quantization and decode append.
//
// Method (KVarN pages, ai-paper-analysis page): rotate tokens by a randomized
// Hadamard matrix along head_dim (section 3.1), then VarN -- token-axis and
// channel-axis variance normalization repeated a few times, Sinkhorn-Knopp style,
// with grouped scales undone at dequantization (section 3.2) -- then uniform 2-bit
// quantization with four codes per byte.
//
// Work mapping. A tile (G tokens x 128 channels of one batch row, kv head and
// stream) is handled by G/32 waves, one 32-token block each.
//   * Rotation on the matrix cores: the inputs are bf16 values and the Sylvester
//     matrix is +-1, so the products are exact in v_mfma_f32_16x16x32_bf16 with fp32
//     accumulation, and the sign flips of sigma are one XOR per pair of inputs. H_syl of order 128 is H_4 (x) H_32: each 32-channel K step
//     goes through H_32 on the matrix cores (its two 32x16 halves are the register
//     fragments F and G, so no matrix leaves registers), and the four K steps are
//     combined by the 4-point transform H_4 in registers (16 MFMAs and 128 adds per
//     32-token block).
//   * The MFMA output leaves lane (g = lane/16, c = lane%16) with tokens 16mb + 4g + i
//     (mb < 2, i < 4) and channels 16nb + c (nb < 8): a token-axis sum is 8 in-lane
//     terms plus a DPP reduction over the 16 lanes of a row; a channel-axis sum is 8
//     in-lane terms plus permlane16/32 swaps across the 4 rows (and an LDS exchange
//     between the two waves of a G=64 tile).
//   * The 2-bit codes are formed with the magic-number trick: after clamping to
//     [0, 3] the value is added to 1.5 * 2^23, so fp32 round-half-to-even leaves the
//     code in mantissa bits 0..1 (bits 2..21 zero); it is then shifted into its slot.
// Reductions have a fixed order, so results are bit-identical run to run.
//
// This header holds the device code of the write path (rotation, VarN, grid, codes,
// the tile core and the decode append job); quantize.hip instantiates the kernels, and
// the attention merge launch reuses the append job for the fused decode step.
#pragma once

#include <type_traits>

#include "kvarn_common.h"
#include "kvarn_launch.h"

namespace kvarn {

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}): a loop
// whose index is a constant expression (instruction immediates such as a byte select)
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMin { __device__ float operator()(float a, float b) const { return vmin(a, b); } };
struct OpMax { __device__ float operator()(float a, float b) const { return vmax(a, b); } };

// Reduce-scatter of 8 per-token partials over the 16 lanes of a row. Stages pair
// lane c with c^15, c^7, c^2, c^1 (row_mirror, row_half_mirror, quad perms); at each
// stage a lane keeps half of its tokens (chosen by bits 3, 2, 1 of c) and adds the
// partner's partial of the same tokens. Lane c ends with the row total of token
// c/2 (identical in lanes c and c^1). The first two stages choose by lane bits 3 and 2,
// which are bits of the DPP bank (4 lanes): each kept value is two DPP adds that write
// complementary banks, instead of two selects and an add.
__device__ __forceinline__ float row_rs8(const float (&v)[8], int c) {
  const bool b1 = c & 2;
  float a0, a1, a2, a3, bb0, bb1;
  // lanes 0..7 of a row (banks 0, 1) keep tokens 0..3, lanes 8..15 (banks 2, 3) tokens 4..7
  asm("s_nop 1\n"
      "v_add_f32_dpp %0, %4, %4 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %1, %5, %5 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %1, %9, %9 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %2, %6, %6 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %2, %10, %10 row_mirror row_mask:0xf bank_mask:0xc\n"
      "v_add_f32_dpp %3, %7, %7 row_mirror row_mask:0xf bank_mask:0x3\n"
      "v_add_f32_dpp %3, %11, %11 row_mirror row_mask:0xf bank_mask:0xc"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
  // lanes with bit 2 clear (banks 0, 2) keep the first two, the others the last two
  asm("s_nop 1\n"
      "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0xa\n"
      "v_add_f32_dpp %1, %3, %3 row_half_mirror row_mask:0xf bank_mask:0x5\n"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(bb0), "=&v"(bb1)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3));
  const float send = b1 ? bb0 : bb1, keep = b1 ? bb1 : bb0;
  const float d = keep + dppf<kQx2>(send);
  return d + dppf<kQx1>(d);
}
// Token tau's value from its owner lanes (2 tau, 2 tau + 1) to the whole row, through a
// wave-private LDS slot (a wave's LDS operations complete in issue order).
__device__ __forceinline__ void row_gather8(float own, float (&v)[8], float* buf, int g, int c) {
  wave_sync();
  if ((c & 1) == 0) buf[8 * g + (c >> 1)] = own;
  wave_sync();
  const float4 x = *reinterpret_cast<const float4*>(buf + 8 * g);
  const float4 y = *reinterpret_cast<const float4*>(buf + 8 * g + 4);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

// Reduce-scatter of 8 per-channel partials (channel blocks nb) over the 4 rows:
// permlane16_swap of two channel registers leaves rows 0+1 / 2+3 partials of one
// channel in rows 0, 2 and of the other in rows 1, 3; permlane32_swap then combines
// the halves. Row g ends with channel block g in out[0] and 4 + g in out[1].
template <typename Op>
__device__ __forceinline__ void col_rs8(const float (&v)[8], float (&out)[2], Op op) {
  float y[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(v[2 * p]), __float_as_int(v[2 * p + 1]),
                                                    false, false);
    y[p] = op(__int_as_float(s[0]), __int_as_float(s[1]));
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(y[2 * q]), __float_as_int(y[2 * q + 1]),
                                                    false, false);
    out[q] = op(__int_as_float(s[0]), __int_as_float(s[1]));
  }
}
// Inverse of col_rs8: row g holds channel blocks g and 4 + g; every row gets all 8,
// through a wave-private LDS slot laid out [c][g][q].
__device__ __forceinline__ void col_gather8(const float (&own)[2], float (&v)[8], float* buf, int g, int c) {
  wave_sync();
  *reinterpret_cast<float2*>(buf + 8 * c + 2 * g) = make_float2(own[0], own[1]);
  wave_sync();
  const float4 x = *reinterpret_cast<const float4*>(buf + 8 * c);      // (g0,q0) (g0,q1) (g1,q0) (g1,q1)
  const float4 y = *reinterpret_cast<const float4*>(buf + 8 * c + 4);  // (g2,q0) (g2,q1) (g3,q0) (g3,q1)
  v[0] = x.x; v[4] = x.y; v[1] = x.z; v[5] = x.w;
  v[2] = y.x; v[6] = y.y; v[3] = y.z; v[7] = y.w;
}

// ----------------------------------------------------------------------------- Hadamard fragments
// B operand of the 16x16x32 MFMA for K-step ks (channels 32ks..32ks+31) and channel
// block nb: lane (g, c) holds H_syl[32ks + 8g + e][16nb + c], e < 8. With
// popcount((32ks + 8g + e) & (16nb + c)) = pc(e & c%8) + (g%2)(c/8) + (g/2)(nb%2)
// + pc(ks & nb/2), the fragment is F (nb even) or G = F * (-1)^(g/2) (nb odd), times
// the uniform sign (-1)^pc(ks & nb/2), which is H_4[ks][nb/2]: the Hadamard path uses F
// and G (the two halves of H_32) and applies H_4 after the products; the identity
// ablation fills the four slots with its own one-hot fragments.
struct Frags {
  b8v v[4];  // F, -F, G, -G
};
// The four fragments of every lane as bf16 bit patterns, computed at compile time:
// word [lane][4 f + d] holds elements 2d, 2d+1 of fragment f.
struct FragTable {
  uint32_t w[64][16];
};
constexpr FragTable make_frag_table() {
  FragTable t{};
  for (int lane = 0; lane < 64; ++lane) {
    const int g = lane >> 4, c = lane & 15;
    for (int e = 0; e < 8; ++e) {
      int pc = (g & 1) & (c >> 3);
      for (int b = 0; b < 3; ++b) pc += (e >> b) & (c >> b) & 1;
      const uint32_t f = (pc & 1) ? 0xBF80u : 0x3F80u;  // -1 / +1
      const uint32_t gg = (g >> 1) ? f ^ 0x8000u : f;
      const uint32_t vals[4] = {f, f ^ 0x8000u, gg, gg ^ 0x8000u};
      for (int q = 0; q < 4; ++q) t.w[lane][4 * q + e / 2] |= vals[q] << (16 * (e & 1));
    }
  }
  return t;
}
static __device__ const FragTable kFrags = make_frag_table();
__device__ __forceinline__ Frags hadamard_frags(int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(kFrags.w[lane]);
  Frags h;
#pragma unroll
  for (int q = 0; q < 4; ++q) h.v[q] = __builtin_bit_cast(b8v, p[q]);
  return h;
}
// Identity in place of H_syl (the "VarN only" ablation): block nb takes the single K-step
// ks = nb/2, whose B fragment is one-hot: lane (g, c) holds 1 at e = c%8 iff
// 8g + e = 16(nb%2) + c, i.e. g = 2(nb%2) + c/8. v[P] is the fragment for nb%2 = P.
__device__ __forceinline__ Frags identity_frags(int lane) {
  const int g = lane >> 4, c = lane & 15;
  Frags h;
#pragma unroll
  for (int P = 0; P < 2; ++P) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = (g == 2 * P + (c >> 3) && d == ((c & 7) >> 1)) ? 0x3F80u << (16 * (c & 1)) : 0u;
    h.v[P] = __builtin_bit_cast(b8v, make_uint4(w[0], w[1], w[2], w[3]));
  }
  h.v[2] = h.v[0];
  h.v[3] = h.v[1];
  return h;
}

// ----------------------------------------------------------------------------- inputs
typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Sign words of the 8 channels of chunk `chunk` (channels 8 chunk .. +7), from the
// header table written at cache init: bit 15 / bit 31 of m[d] is set where sigma of
// channel 2d / 2d + 1 is -1, i.e. at the sign bits of a packed pair of 16-bit floats.
struct SigMask {
  uint32_t m[4];
};
__device__ __forceinline__ SigMask sigma_masks(const uint8_t* hdr, int chunk) {
  const uint4 s = *reinterpret_cast<const uint4*>(hdr + kSignOff + 16 * chunk);
  return SigMask{{s.x, s.y, s.z, s.w}};
}

// two fp32 -> packed fp16 pair, round half to even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, h2v));
}

// 8 bf16 values times sigma: the sign bits of the pairs flip where the mask words are set
__device__ __forceinline__ b8v sign8(const uint4 w, const SigMask& m) {
  return __builtin_bit_cast(b8v, make_uint4(w.x ^ m.m[0], w.y ^ m.m[1], w.z ^ m.m[2], w.w ^ m.m[3]));
}
// 8 bf16 inputs -> their canonical values (bf16 bits): a NaN becomes +0 (KVARN_FLAG_NAN)
// and a magnitude beyond 2^16 (bf16 0x4780), infinities included, becomes +-2^16
// (KVARN_FLAG_SATURATED); every other value is kept as it is. Integer arithmetic on both
// halves of a word at once, with no per-value compares: for a magnitude m <= 0x7FFF, bit 15
// of m + 0x7F is set iff m > 0x7F80 (NaN) and bit 15 of m + 0x387F iff m > 0x4780.
__device__ __forceinline__ uint32_t canon2(uint32_t w, uint32_t& nan_acc, uint32_t& sat_acc) {
  const uint32_t m = w & 0x7FFF7FFFu;
  const uint32_t nan = (m + 0x007F007Fu) & 0x80008000u;         // no carry leaves a half
  const uint32_t big = (m + 0x387F387Fu) & 0x80008000u & ~nan;
  nan_acc |= nan;
  sat_acc |= big;
  const uint32_t nan_all = nan | (nan - (nan >> 15));            // 0xFFFF in NaN halves
  const uint32_t big_all = big | (big - (big >> 15));            // 0xFFFF in saturated halves
  const uint32_t v = (w & ~big_all) | (big_all & ((w & 0x80008000u) | 0x47804780u));
  return v & ~nan_all;
}
__device__ __forceinline__ uint4 canon8(const uint4 w, uint32_t& flags) {
  uint32_t nan = 0, sat = 0;
  const uint4 o = make_uint4(canon2(w.x, nan, sat), canon2(w.y, nan, sat), canon2(w.z, nan, sat),
                             canon2(w.w, nan, sat));
  flags |= (nan ? (uint32_t)KVARN_FLAG_NAN : 0u) | (sat ? (uint32_t)KVARN_FLAG_SATURATED : 0u);
  return o;
}
// the largest magnitude of 8 bf16 values
__device__ __forceinline__ float maxabs8(const uint4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float m = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) m = fmaxf(m, fmaxf(fabsf(bf16lo(ws[d])), fabsf(bf16hi(ws[d]))));
  return m;
}
// 8 bf16 values times 2^e, exactly (e only scales tokens whose values all lie below 2^-20,
// up to magnitudes below 1, so every result is a bf16 value again)
__device__ __forceinline__ uint4 scale8(const uint4 w, int e) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = (uint32_t)__float_as_int(__builtin_amdgcn_ldexpf(bf16lo(ws[d]), e));
    const uint32_t hi = (uint32_t)__float_as_int(__builtin_amdgcn_ldexpf(bf16hi(ws[d]), e));
    o[d] = (lo >> 16) | (hi & 0xFFFF0000u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// W'[token 16mb + 4g + i][channel 16nb + c] = sum_k A[mb][k] H[k][16nb + c]; with ID the
// identity fragments make W' = A (one MFMA per block).
//
// H_syl of order 128 is H_4 (x) H_32 (channel 32 q + j), so the Hadamard path takes each
// K step's 32 channels through H_32 on the matrix cores (F for output half h = nb % 2,
// G for h = 1: two MFMAs per token block and K step) and combines the four K steps with
// the 4-point transform H_4 in registers, output block nb = 2 nb' + h:
//   nb' = 0: y0 + y1 + y2 + y3   nb' = 1: y0 - y1 + y2 - y3
//   nb' = 2: y0 + y1 - y2 - y3   nb' = 3: y0 - y1 - y2 + y3
// (16 MFMAs and 128 adds per 32-token block instead of 64 MFMAs).
//
// An MFMA whose destination shares registers with its A or B source reads clobbered
// rows on this hardware. After each MFMA (or accumulation chain) an empty asm takes the
// result as read-write and all its A and B fragments as inputs: the data dependency
// pins it after the MFMAs, so every source is still live when each of them issues and
// the register allocator cannot hand a source's registers to the result.
__device__ __forceinline__ void h32_steps(const b8v (&a)[4], const Frags& hf, int h, f4v (&y)[4]) {
  // the wave's priority is raised while it issues these MFMAs, so that they start while
  // the other waves of the SIMD keep the VALU busy
  __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    f4v t = {0.0f, 0.0f, 0.0f, 0.0f};
    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], hf.v[2 * h], t, 0, 0, 0);
    asm volatile("" : "+v"(t) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(hf.v[0]), "v"(hf.v[2]));
    y[ks] = t;
  }
  __builtin_amdgcn_s_setprio(0);
}
// out[nb'] = sum_ks H_4[ks][nb'] y[ks], element by element
__device__ __forceinline__ void h4_combine(const f4v (&y)[4], f4v (&out)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s01 = y[0][i] + y[1][i], d01 = y[0][i] - y[1][i];
    const float s23 = y[2][i] + y[3][i], d23 = y[2][i] - y[3][i];
    out[0][i] = s01 + s23;
    out[1][i] = d01 + d23;
    out[2][i] = s01 - s23;
    out[3][i] = d01 - d23;
  }
}
template <bool ID>
__device__ __forceinline__ void rotate_block(const b8v (&a)[2][4], const Frags& hf, f4v (&acc)[2][8]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if constexpr (ID) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        f4v s = {0.0f, 0.0f, 0.0f, 0.0f};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][nb >> 1], hf.v[nb & 1], s, 0, 0, 0);
        asm volatile("" : "+v"(s) : "v"(a[mb][0]), "v"(a[mb][1]), "v"(a[mb][2]), "v"(a[mb][3]), "v"(hf.v[0]),
                     "v"(hf.v[1]), "v"(hf.v[2]), "v"(hf.v[3]));
        acc[mb][nb] = s;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f4v y[4], w[4];
        h32_steps(a[mb], hf, h, y);
        h4_combine(y, w);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[mb][2 * q + h] = w[q];
      }
    }
  }
}

// ----------------------------------------------------------------------------- butterfly form
// The library built with KVARN_ROTATION_BUTTERFLY=1 (libkvarn_fwht.so, for measurement only)
// rotates on the VALU instead of the matrix cores: a 128-point fast Walsh-Hadamard
// transform. Lane (g, c) holds token 16 mb + c, channels k = 32 ks + 8 g + e: bits 0..2
// and 5..6 of k are in the lane's registers, bits 3..4 are lane bits 4..5. The five stages
// on the register bits are adds; a stage on a lane bit pairs two registers whose channels
// differ in bit 5 or 6 and swaps half of the lanes of each with v_permlane16_swap or
// v_permlane32_swap, which leaves that lane bit and that register bit exchanged. After
// both, register (ks, e) of lane (g, c) holds output channel 32 g + 8 ks + e, and the
// block goes through LDS (xt[token][channel], rows of 132 floats: 16-B aligned writes, and
// the four rows g of one read on different banks) into the layout the MFMA path leaves
// and VarN works on. The token's sum of squares (the first token-axis pass) is summed in
// the input layout, where gram_own finds it.
#ifndef KVARN_ROTATION_BUTTERFLY
#define KVARN_ROTATION_BUTTERFLY 0
#endif
constexpr int kXtRow = 132;
__device__ __forceinline__ float fwht_squares_mb(const b8v (&a)[4], f4v (&w4)[8], float (&p)[8][4], int c,
                                                 float* xt) {
  const int g = (int)(threadIdx.x & 63) >> 4;
  float x[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 u = __builtin_bit_cast(uint4, a[ks]);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x[ks][2 * d] = bf16lo(w[d]);
      x[ks][2 * d + 1] = bf16hi(w[d]);
    }
  }
  float d = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(x[ks][e], x[ks][e], d);
  {  // over the four lanes g that hold the token's channels
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_int(d), __float_as_int(d), false, false);
    d = __int_as_float(s1[0]) + __int_as_float(s1[1]);
    const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_int(d), __float_as_int(d), false, false);
    d = __int_as_float(s2[0]) + __int_as_float(s2[1]);
  }
#pragma unroll
  for (int b = 1; b < 8; b <<= 1)  // channel bits 0..2
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & b)) {
          const float u = x[ks][e], v = x[ks][e | b];
          x[ks][e] = u + v;
          x[ks][e | b] = u - v;
        }
#pragma unroll
  for (int b = 1; b < 4; b <<= 1)  // channel bits 5..6
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      if (!(ks & b))
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float u = x[ks][e], v = x[ks | b][e];
          x[ks][e] = u + v;
          x[ks | b][e] = u - v;
        }
  // channel bit 4 (lane bit 5) against register bit ks/2, then bit 3 (lane bit 4) against ks%2
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto t = __builtin_amdgcn_permlane32_swap(__float_as_int(x[ks][e]), __float_as_int(x[ks + 2][e]),
                                                      false, false);
      x[ks][e] = __int_as_float(t[0]) + __int_as_float(t[1]);
      x[ks + 2][e] = __int_as_float(t[0]) - __int_as_float(t[1]);
    }
#pragma unroll
  for (int ks = 0; ks < 4; ks += 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto t = __builtin_amdgcn_permlane16_swap(__float_as_int(x[ks][e]), __float_as_int(x[ks + 1][e]),
                                                      false, false);
      x[ks][e] = __int_as_float(t[0]) + __int_as_float(t[1]);
      x[ks + 1][e] = __int_as_float(t[0]) - __int_as_float(t[1]);
    }
  // to the MFMA output layout: lane (g, c) takes tokens 4 g + i of channel 16 nb + c
  wave_sync();  // the previous block's reads are issued before these writes
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float* row = xt + c * kXtRow + 32 * g + 8 * ks;
    *reinterpret_cast<float4*>(row) = make_float4(x[ks][0], x[ks][1], x[ks][2], x[ks][3]);
    *reinterpret_cast<float4*>(row + 4) = make_float4(x[ks][4], x[ks][5], x[ks][6], x[ks][7]);
  }
  wave_sync();
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = xt[(4 * g + i) * kXtRow + 16 * nb + c];
      w4[nb][i] = v;
      p[nb][i] = v * v;
    }
  return d;
}

// Rotation fused with the squares: each chain's W' block is squared as soon as it is
// complete, so the fp32 block is never held whole. Returns the first token-axis sum
// (u = 1) of the lane's own token, 16 (c/8) + 4 g + (c/2) % 4 (identical in lanes c and
// c ^ 1), from the Gram diagonal instead of the squares: with H_syl H_syl^T = D I the row
// sum of W'^2 is D times the row sum of x^2 (1 times it for the identity), and diag(X X^T)
// comes exactly from the matrix cores, since the B operand X^T of the 16x16x32 MFMA is
// held in the same registers as the A operand X (lane (g, c): token c, channels 8 g ..
// 8 g + 7 of the K step). Lane (g, c) of the Gram block holds rows 4 g + i at column c:
// the diagonal sits in lanes c = 4 g + j at element j, and the owner lane fetches it.
template <bool ID>
__device__ __forceinline__ float rotate_squares_mb(const b8v (&a)[4], const Frags& hf, f4v (&w4)[8], float (&p)[8][4],
                                                   int c, float* xt) {
  if constexpr (!ID && KVARN_ROTATION_BUTTERFLY) return fwht_squares_mb(a, w4, p, c, xt);
  // the Gram block first: the token block's inputs are dead once its rotation is done
  f4v gm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], a[ks], gm, 0, 0, 0);
  asm volatile("" : "+v"(gm) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
  if constexpr (ID) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f4v s = {0.0f, 0.0f, 0.0f, 0.0f};
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nb >> 1], hf.v[nb & 1], s, 0, 0, 0);
      asm volatile("" : "+v"(s) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(hf.v[0]), "v"(hf.v[1]),
                   "v"(hf.v[2]), "v"(hf.v[3]));
      w4[nb] = s;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[nb][i] = s[i] * s[i];
    }
  } else {  // H_4 (x) H_32, as in rotate_block; each block is squared once combined
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f4v y[4], w[4];
      h32_steps(a, hf, h, y);
      h4_combine(y, w);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w4[2 * q + h] = w[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[2 * q + h][i] = w[q][i] * w[q][i];
      }
    }
  }
  // this lane's diagonal candidate (element c % 4)
  const float lo = (c & 1) ? gm[1] : gm[0], hi = (c & 1) ? gm[3] : gm[2];
  return (c & 2) ? hi : lo;
}
// The owner lane's diagonal element from the candidates of the two token blocks
template <bool ID>
__device__ __forceinline__ float gram_own(float d0, float d1, int c) {
  const int g = (int)(threadIdx.x & 63) >> 4;
  const int src = 4 * (20 * g + ((c >> 1) & 3));  // byte address of lane 16 g + 4 g + (c/2) % 4
  const float x0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(d0)));
  const float x1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(d1)));
  return ((c >> 3) ? x1 : x0) * (ID ? 1.0f : (float)kD);
}
template <bool ID>
__device__ __forceinline__ float rotate_squares(const b8v (&a)[2][4], const Frags& hf, f4v (&w4)[2][8],
                                                float (&p)[2][8][4], int c, float* xt) {
  const float d0 = rotate_squares_mb<ID>(a[0], hf, w4[0], p[0], c, xt);
  const float d1 = rotate_squares_mb<ID>(a[1], hf, w4[1], p[1], c, xt);
  return gram_own<ID>(d0, d1, c);
}

// Dispatch for the ablation build (ABL): the identity rotation is a runtime choice there;
// the standard build compiles the Hadamard path only.
template <bool ABL>
__device__ __forceinline__ float rotate_squares_v(bool idr, const b8v (&a)[2][4], const Frags& hf, f4v (&w4)[2][8],
                                                  float (&p)[2][8][4], int c, float* xt) {
  if constexpr (ABL) {
    if (idr) return rotate_squares<true>(a, hf, w4, p, c, xt);
  }
  return rotate_squares<false>(a, hf, w4, p, c, xt);
}
template <bool ABL>
__device__ __forceinline__ float rotate_squares_mb_v(bool idr, const b8v (&a)[4], const Frags& hf, f4v (&w4)[8],
                                                     float (&p)[8][4], int c, float* xt) {
  if constexpr (ABL) {
    if (idr) return rotate_squares_mb<true>(a, hf, w4, p, c, xt);
  }
  return rotate_squares_mb<false>(a, hf, w4, p, c, xt);
}
template <bool ABL>
__device__ __forceinline__ float gram_own_v(bool idr, float d0, float d1, int c) {
  if constexpr (ABL) {
    if (idr) return gram_own<true>(d0, d1, c);
  }
  return gram_own<false>(d0, d1, c);
}
template <bool ABL>
__device__ __forceinline__ void rotate_block_v(bool idr, const b8v (&a)[2][4], const Frags& hf,
                                               f4v (&acc)[2][8]) {
  if constexpr (ABL) {
    if (idr) {
      rotate_block<true>(a, hf, acc);
      return;
    }
  }
  rotate_block<false>(a, hf, acc);
}
template <bool ABL>
__device__ __forceinline__ SigMask masks_v(bool idr, const uint8_t* hdr, int chunk) {
  if constexpr (ABL) {
    if (idr) return SigMask{};  // no sign flips without the rotation
  }
  return sigma_masks(hdr, chunk);
}
template <bool ABL>
__device__ __forceinline__ Frags frags_v(bool idr, int lane) {
  if constexpr (ABL) {
    if (idr) return identity_frags(lane);
  }
  return hadamard_frags(lane);
}

// ----------------------------------------------------------------------------- checked rotation
// The rotation runs on the bf16 inputs as given. It stands when every token's sum of
// squares lies in [2^-100, 2^32]: then no value exceeds 2^16 in magnitude, none is NaN,
// and the squares that carry a token's mean square do not underflow fp32. st is the
// owner lane's first token-axis sum (D or 1 times the token's sum of squares), so a wave
// checks its 32 tokens with one vote.
__device__ __forceinline__ bool rotation_stands(bool idr, float st) {
  const float k = idr ? 1.0f : (float)kD;
  return st >= 0x1p-100f * k && st <= 0x1p32f * k;
}
// max over the 4 rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float rows_max4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(q[0]), __int_as_float(q[1]));
}
// Otherwise the wave redoes its block from load(mb, ks), the bf16 rows the first pass read
// (token 16 mb + c, channels 8 (4 ks + g) .. +7): the values are made canonical (canon8,
// flags), and a token whose largest magnitude is below 2^-20 is scaled by the power of two
// 2^sx that brings it into [0.5, 1), exactly, so that no square it needs underflows. Every
// step of VarN is invariant under a per-token power of two except r itself and the factor
// that maps W' to Y, which the owner lane corrects with its token's sx (sx_own).
template <bool ABL, typename Load>
__device__ float rotate_checked(bool idr, Load&& load, const uint8_t* hdr, const Frags& hf, b8v (&av)[2][4],
                                f4v (&w4)[2][8], float (&p)[2][8][4], int g, int c, uint32_t& flags, int& sx_own,
                                float* xt) {
  // two passes over the rows (the second reads them again rather than holding them):
  // each token's largest magnitude, then the scaled, signed operands
  float mx[2] = {0.0f, 0.0f};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t counted_below = 0;
      mx[mb] = fmaxf(mx[mb], maxabs8(canon8(load(mb, ks), counted_below)));
    }
  int sx[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const float m = rows_max4(mx[mb]);  // token 16 mb + c has its channels in lanes c + 16 g'
    sx[mb] = (m > 0.0f && m < 0x1p-20f) ? -__builtin_amdgcn_frexp_expf(m) : 0;
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const SigMask m = masks_v<ABL>(idr, hdr, 4 * ks + g);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint4 x = canon8(load(mb, ks), flags);
      av[mb][ks] = sign8(sx[mb] ? scale8(x, sx[mb]) : x, m);
    }
  }
  const float st = rotate_squares_v<ABL>(idr, av, hf, w4, p, c, xt);
  // the owner lane of token 16 (c/8) + 4 g + (c/2) % 4 reads sx where that token is an A row
  const int src = 4 * (20 * g + ((c >> 1) & 3));
  const int s0 = __builtin_amdgcn_ds_bpermute(src, sx[0]), s1 = __builtin_amdgcn_ds_bpermute(src, sx[1]);
  sx_own = (c >> 3) ? s1 : s0;
  return st;
}

// ----------------------------------------------------------------------------- LDS
// A one-wave tile only needs its own LDS writes ordered before its reads (a wave's LDS
// operations complete in order); a two-wave tile needs the work-group barrier.
template <int NW>
__device__ __forceinline__ void tile_sync() {
  if constexpr (NW == 1) {
    wave_sync();
  } else {
    __syncthreads();
  }
}

template <int NW>
struct TileLds {
  static constexpr int G = 32 * NW;
  static constexpr int TR = G * kD / 2 + 2 * G + 6 * kD;  // room for the widest (4-bit) record
  uint8_t rec[TR] __attribute__((aligned(16)));
  float red_a[NW][kD];
  float red_b[NW][kD];
  float gcol[NW][kD] __attribute__((aligned(16)));  // per-wave gather buffers
  float grow[NW][32] __attribute__((aligned(16)));
  float xt[NW][KVARN_ROTATION_BUTTERFLY ? 16 * kXtRow : 1] __attribute__((aligned(16)));  // butterfly form only
};

// Per-channel reduction of a tile: 4-row reduce-scatter inside the wave, then (G=64)
// the partials of the NW waves through LDS in wave order. own[q] is channel
// 16 (4q + g) + c. The trailing barrier lets the next call reuse the LDS slots.
template <int NW, typename Op>
__device__ __forceinline__ void chan_reduce(const float (&v)[8], float (&own)[2], int g, int c, int sub,
                                            float (*red)[kD], Op op) {
  col_rs8(v, own, op);
  if constexpr (NW > 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) red[sub][16 * (4 * q + g) + c] = own[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float t = red[0][16 * (4 * q + g) + c];
#pragma unroll
      for (int w = 1; w < NW; ++w) t = op(t, red[w][16 * (4 * q + g) + c]);
      own[q] = t;
    }
    __syncthreads();
  }
}

// VarN with the centered reading of "variance" (an ablation): explicit cumulative scales,
// y = W / (r c), and per pass var = mean(y^2) - mean(y)^2 along the axis; a pass leaves
// the scale unchanged where the variance is not positive. Needs W itself, so the
// rotation is recomputed here (the ablation build only). r_own, c_own: the owner
// lane's token and channel scales, in units of W.
template <int NW, bool ABL>
__device__ void centered_varn(const b8v (&av)[2][4], const Frags& hf, bool idr, bool tok, bool chp, int n_it,
                              float inv_k, int lane, int sub, TileLds<NW>& sh, float& r_own, float (&c_own)[2]) {
  constexpr int G = 32 * NW;
  const int g = lane >> 4, c = lane & 15;
  f4v w[2][8];
  rotate_block_v<ABL>(idr, av, hf, w);
  float ir[8], ic[8];  // 1/(k r) per lane token, 1/c per lane channel block
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ir[k] = inv_k;
    ic[k] = 1.0f;
  }
  r_own = 1.0f;
  c_own[0] = c_own[1] = 1.0f;
  for (int it = 0; it < n_it; ++it) {
    if (tok) {
      float s1[8], s2[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = 0.0f, b = 0.0f;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const float y = w[mb][nb][i] * ir[4 * mb + i] * ic[nb];
            a += y;
            b = fmaf(y, y, b);
          }
          s1[4 * mb + i] = a;
          s2[4 * mb + i] = b;
        }
      const float m1 = row_rs8(s1, c) * (1.0f / kD), m2 = row_rs8(s2, c) * (1.0f / kD);
      const float vr = m2 - m1 * m1;
      if (vr > 0.0f) r_own *= __builtin_amdgcn_sqrtf(vr);
      row_gather8(inv_k / r_own, ir, sh.grow[sub], g, c);
    }
    if (chp) {
      float s1[8], s2[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float y = w[mb][nb][i] * ir[4 * mb + i] * ic[nb];
            a += y;
            b = fmaf(y, y, b);
          }
        s1[nb] = a;
        s2[nb] = b;
      }
      float m1[2], m2[2];
      chan_reduce<NW>(s1, m1, g, c, sub, sh.red_a, OpAdd());
      chan_reduce<NW>(s2, m2, g, c, sub, sh.red_b, OpAdd());
      float icn[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float mean = m1[q] * (1.0f / G);
        const float vr = m2[q] * (1.0f / G) - mean * mean;
        if (vr > 0.0f) c_own[q] *= __builtin_amdgcn_sqrtf(vr);
        icn[q] = 1.0f / c_own[q];
      }
      col_gather8(icn, ic, sh.gcol[sub], g, c);
    }
  }
}

// ----------------------------------------------------------------------------- codes
// The 2-bit layout of one plane of codes, written into `base` (the record in LDS):
// K: word w = c/2 of token t holds channel 16nb + c in slot 4(nb/2) + nb%2 + 2(c%2).
// V: byte j*G/4 + t/4 holds tokens 4(t/4) .. +3 of channel j, token t%4 in slot t%4.
// code(y, nb) gives the plane's 2-bit value in bits 0..1; bits from 22 up may hold junk
// (they are shifted out of the bytes kept).
template <int NW, typename F>
__device__ __forceinline__ void emit_plane2(const f4v (&acc)[2][8], F code, int stream, int ttile0, int c,
                                            uint8_t* base) {
  constexpr int G = 32 * NW;
  if (stream == 0) {
    // lane c's channel 16nb + c goes to word c/2, slot 4(nb/2) + nb%2 + 2(c%2): the even
    // lane assembles bits 8(nb/2) + 2(nb%2) (blocks 0..3 in bytes 0..1, 4..7 in bytes
    // 2..3, one byte permute), the odd lane's pattern lands 4 bits higher.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          lo |= code(acc[mb][nb][i], nb) << (8 * (nb >> 1) + 2 * (nb & 1));
          hi |= code(acc[mb][nb + 4][i], nb + 4) << (8 * (nb >> 1) + 2 * (nb & 1));
        }
        const uint32_t h = __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // bytes lo.0 lo.1 hi.0 hi.1
        const uint32_t hp = (uint32_t)__builtin_amdgcn_mov_dpp((int)h, kQx1, 0xF, 0xF, true);
        if ((c & 1) == 0)
          *reinterpret_cast<uint32_t*>(base + (ttile0 + 16 * mb + i) * 32 + 2 * c) = h | (hp << 4);
      }
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint32_t h = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) h |= code(acc[mb][nb][i], nb) << (2 * i);
        base[(16 * nb + c) * (G / 4) + (ttile0 + 16 * mb) / 4] = (uint8_t)h;
      }
  }
}

// The 1-bit plane of 3-bit codes (their bit 2), ORed into the zeroed plane at `base`:
// K: channel j of token t sits in the 2-bit layout's word w, slot k; its bit goes to word
//    4t + w/2, bit 4(k/2) + k%2 + 2(w%2). For lane c's channel 16nb + c that is word
//    4t + c/4, bit 8(nb/2) + nb%2 + 4(c%2) + 2((c/2)%2).
// V: token t = 8o + 2n + par of channel 16 blk + c, blk = i + 4hh, i = 2ip + ii: word
//    (16 ip + c) G/8 + o, bit 4(n + 4hh) + par + 2ii. This lane's tokens 4(g%2) + i4 of
//    an octet fill nibbles 2(g%2) + i4/2 (+ 4hh); rows g and g^1 share the word.
template <int NW, typename F>
__device__ __forceinline__ void emit_bit_plane(const f4v (&acc)[2][8], F bit, int stream, int ttile0, int g,
                                               int c, uint8_t* base) {
  constexpr int G = 32 * NW;
  if (stream == 0) {
    const int off = 4 * (c & 1) + 2 * ((c >> 1) & 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) v |= bit(acc[mb][nb][i], nb) << (8 * (nb >> 1) + (nb & 1));
        atomicOr(reinterpret_cast<uint32_t*>(base + (ttile0 + 16 * mb + i) * 16 + 4 * (c >> 2)), v << off);
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        uint32_t v = 0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const int nb = 2 * ip + ii + 4 * hh;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              v |= bit(acc[mb][nb][i4], nb) << (4 * (2 * (g & 1) + (i4 >> 1) + 4 * hh) + (i4 & 1) + 2 * ii);
          }
        const int o = (ttile0 + 16 * mb) / 8;
        atomicOr(reinterpret_cast<uint32_t*>(base + 4 * ((16 * ip + c) * (G / 8) + o)), v);
      }
  }
}

// 2-bit codes through the packed fp4 conversion. v_cvt_scalef32_pk_fp4_f32 rounds two fp32
// values, divided by the power of two of its scale, to e2m1 with round-half-to-even and
// writes them as the two nibbles of a chosen byte. On [0, 1.5] e2m1 is the grid
// {0, 0.5, 1, 1.5}, so the nibble of t / 2 is RNE(t) for t in [0, 3.5): the 2-bit code in
// bits 0..1 of a nibble. Inputs arrive as t / 4 (al4, ga4 = al / 4, ga / 4, exact), clamped to
// [0, 1] by the multiply-add itself, which also keeps the sign bit of the nibble clear; with
// CLAMP (some u may leave (-0.5, 3.5)) the top is cut at 3/4 as well. Two nibble words whose
// nibble k holds codes A and B give A | B << 2: nibble k of the result holds both codes.
//   K: word w of token t, byte k: nibble 0 = lane 2w's codes of channel blocks (2k, 2k + 1),
//      nibble 1 = lane 2w + 1's. A lane converts its tokens t0 = 4g + i and t1 = 16 + 4g + i
//      together (t0 into the low nibble of each byte, t1 into the high one), swaps the
//      result with its partner lane, and each of the two keeps one token's word: the even
//      lane t0's, the odd lane t1's.
//   V: byte of tokens 4g .. 4g + 3 (+ 16 mb) of channel 16 nb + c: codes i = 0 | 1 << 2 |
//      2 << 4 | 3 << 6; the low nibbles take i = 0, 1 and the high ones i = 2, 3.
template <int NW, bool CLAMP>
__device__ __forceinline__ void emit_codes2(const f4v (&acc)[2][8], const float (&al4)[8], const float (&ga4)[8],
                                            int stream, int sub, int g, int c, uint8_t* base) {
  constexpr int G = 32 * NW;
  const int ttile0 = sub * 32 + 4 * g;
  auto q4 = [&](float y, int nb) -> float {
    float t;
    asm("v_fma_f32 %0, %1, %2, %3 clamp" : "=v"(t) : "v"(y), "v"(al4[nb]), "v"(ga4[nb]));
    if constexpr (CLAMP) t = vmin(t, 0.75f);
    return t;
  };
  if (stream == 0) {
    const bool odd = c & 1;
    const uint32_t keep = odd ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
    const uint32_t rot = odd ? 4u : 28u;
    uint8_t* row = base + 2 * (c & ~1);
    // every byte of xa, xb is rewritten in each iteration, so they start undefined and
    // carry the last iteration's (dead) words: no initializing moves
    uint32_t xa = __builtin_nondeterministic_value(0u), xb = __builtin_nondeterministic_value(0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      static_for<4>([&](auto K) {
        constexpr int k = decltype(K)::value;
        xa = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(xa, q4(acc[0][2 * k][i], 2 * k), q4(acc[1][2 * k][i], 2 * k),
                                                      0.5f, k);
        xb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(xb, q4(acc[0][2 * k + 1][i], 2 * k + 1),
                                                      q4(acc[1][2 * k + 1][i], 2 * k + 1), 0.5f, k);
      });
      const uint32_t z = xa | (xb << 2);
      const uint32_t zp = (uint32_t)__builtin_amdgcn_mov_dpp((int)z, kQx1, 0xF, 0xF, true);
      const uint32_t p = __builtin_amdgcn_alignbit(zp, zp, rot);  // even: zp << 4, odd: zp >> 4
      const uint32_t word = (z & keep) | (p & ~keep);
      *reinterpret_cast<uint32_t*>(row + (ttile0 + i + (odd ? 16 : 0)) * 32) = word;
    }
  } else {
    uint32_t x0 = __builtin_nondeterministic_value(0u), x1 = __builtin_nondeterministic_value(0u);
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {  // channel blocks 2 n2 and 2 n2 + 1, both token blocks
      static_for<4>([&](auto BB) {
        constexpr int bb = decltype(BB)::value;
        const int nb = 2 * n2 + (bb >> 1), mb = bb & 1;
        x0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x0, q4(acc[mb][nb][0], nb), q4(acc[mb][nb][2], nb), 0.5f, bb);
        x1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x1, q4(acc[mb][nb][1], nb), q4(acc[mb][nb][3], nb), 0.5f, bb);
      });
      const uint32_t z = x0 | (x1 << 2);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int nb = 2 * n2 + (bb >> 1), mb = bb & 1;
        base[(16 * nb + c) * (G / 4) + (ttile0 + 16 * mb) / 4] = (uint8_t)(z >> (8 * bb));
      }
    }
  }
}

// Writes the codes of this wave's block into the record in LDS: 2-bit codes in the layout
// of emit_plane2; 3- and 4-bit codes as plane A (bits 0..1, that layout) followed by
// plane B (4-bit: bits 2..3 in the same layout; 3-bit: bit 2, emit_bit_plane).
template <int NW, bool CLAMP>
__device__ __forceinline__ void emit_codes(const f4v (&acc)[2][8], const float (&al)[8], const float (&ga)[8],
                                           int stream, int sub, int g, int c, TileLds<NW>& sh, int bits) {
  constexpr int G = 32 * NW;
  const int ttile0 = sub * 32 + 4 * g;  // token of (mb = 0, i = 0) inside the tile
  const float top = bits == 2 ? 3.0f : (float)((1 << bits) - 1);
  auto code = [&](float y, int nb) -> uint32_t {  // the code in bits 0..bits-1
    float t = fmaf(y, al[nb], ga[nb]);
    if constexpr (CLAMP) t = __builtin_amdgcn_fmed3f(t, 0.0f, top);
    return (uint32_t)__float_as_int(t + 12582912.0f);  // 1.5 * 2^23
  };
  if (bits == 2) {  // al, ga arrive divided by 4 (emit_codes2)
    emit_codes2<NW, CLAMP>(acc, al, ga, stream, sub, g, c, sh.rec);
    return;
  }
  uint8_t* pb = sh.rec + G * kD / 4;
  if (bits == 3) {  // plane B is ORed together from several lanes: clear it first
    reinterpret_cast<uint2*>(pb)[sub * 64 + (g * 16 + c)] = make_uint2(0u, 0u);
    tile_sync<NW>();
  }
  emit_plane2<NW>(acc, [&](float y, int nb) { return code(y, nb) & 3u; }, stream, ttile0, c, sh.rec);
  if (bits == 4)
    emit_plane2<NW>(acc, [&](float y, int nb) { return (code(y, nb) >> 2) & 3u; }, stream, ttile0, c, pb);
  else
    emit_bit_plane<NW>(acc, [&](float y, int nb) { return (code(y, nb) >> 2) & 1u; }, stream, ttile0, g, c, pb);
}

// ----------------------------------------------------------------------------- the tile core
// From the rotated block W' = sqrt(D) W (acc), its squares p and the first token-axis
// sum of the lane's own token (u = 1): VarN, stored scales, grid, codes; the record
// is assembled in sh.rec. Steps follow the ai-paper-analysis page, section 3.2.
//
// VarN with cumulative scales (the mean square of W/(r c) along the axis becomes 1):
//   token pass   S'_t = sum_j W'_tj^2 / c_j^2,   r_t = sqrt(S'_t) / D,  v_t = D / S'_t
//   channel pass S'_j = sum_t W'_tj^2 v_t,       c_j = sqrt(S'_j / G),  u_j = G / S'_j
// (with W' = sqrt(D) W these are the oracle's r_t <- r_t sqrt(ms_t), c_j <- c_j sqrt(ms_j));
// an all-zero line keeps its scale. Each lane owns one token (c/2 of its row's 8) and
// two channels (16g + c, 64 + 16g + c): their scalars are computed once, by the owner,
// and broadcast back.
//
// ABL builds the ablation variants (var = KVARN_VARIANT_* bits, uniform): with the
// identity rotation W' = W (k = 1 instead of sqrt(D)): v and u keep their form, only r
// becomes sqrt(S'_t) / (k sqrt(D)) and the start value v = 1/k^2; a dropped pass keeps
// its scale at 1 (the other pass then repeats the same sums every iteration). The
// centered reading of "variance" runs its own loop (centered_varn).
template <int NW, bool DBG, bool ABL>
__device__ __forceinline__ void tile_finish(const b8v (&av)[2][4], const Frags& hf, f4v (&acc)[2][8], float (&p)[2][8][4],
                            float st_own, int sx_own, int lane,
                            int sub, int stream, int n_it, int var, int bits_in, TileLds<NW>& sh, uint32_t& flags,
                            float* dbg_w, float* dbg_y, long long dstride) {
  constexpr int G = 32 * NW;
  const int bits = ABL ? bits_in : 2;  // code width; the standard build has 2
  const int g = lane >> 4, c = lane & 15;
  const int tau_own = c >> 1;  // own token: mb = tau/4, i = tau%4
  const bool idr = ABL && (var & KVARN_VARIANT_NO_ROTATION);
  const bool tok = !ABL || !(var & KVARN_VARIANT_NO_TOKEN_PASS);
  const bool chp = !ABL || !(var & KVARN_VARIANT_NO_CHANNEL_PASS);
  const bool cen = ABL && (var & KVARN_VARIANT_CENTERED);
  const float inv_k = idr ? 1.0f : kInvSqrtD;   // 1/k
  const float r_k = idr ? kInvSqrtD : 1.0f / kD;  // 1/(k sqrt(D))
  const int n_std = cen ? 0 : n_it;              // iterations of the mean-square loop

  float u[8], v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) u[k] = 1.0f;
  float v_own = idr ? 1.0f : 1.0f / kD, s_tok = st_own;
  float u_own[2] = {1.0f, 1.0f}, s_ch[2] = {0.0f, 0.0f};
  for (int it = 0; it < n_std; ++it) {
    if (tok) {
      if (it > 0) {  // token pass (the first one arrives precomputed)
        float tp[8];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float t = 0.0f;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) t = fmaf(p[mb][nb][i], u[nb], t);
            tp[4 * mb + i] = t;
          }
        s_tok = row_rs8(tp, c);
      }
      if (s_tok > 0.0f) v_own = (float)kD * __builtin_amdgcn_rcpf(s_tok);
    }
    if (chp) {
      row_gather8(v_own, v, sh.grow[sub], g, c);
      float cp[8];  // channel pass
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float t = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) t = fmaf(p[mb][nb][i], v[4 * mb + i], t);
        cp[nb] = t;
      }
      chan_reduce<NW>(cp, s_ch, g, c, sub, sh.red_a, OpAdd());
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (s_ch[q] > 0.0f) u_own[q] = (float)G * __builtin_amdgcn_rcpf(s_ch[q]);
      col_gather8(u_own, u, sh.gcol[sub], g, c);
    }
  }

  // stored scales: fp16, clamped to [2^-14, 65504]
  float r_own = (n_std > 0 && tok && s_tok > 0.0f) ? __builtin_amdgcn_sqrtf(s_tok) * r_k : 1.0f;
  float c_own[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    c_own[q] = (n_std > 0 && s_ch[q] > 0.0f) ? __builtin_amdgcn_sqrtf(s_ch[q] * (1.0f / G)) : 1.0f;
  if constexpr (ABL) {
    if (cen) centered_varn<NW, ABL>(av, hf, idr, tok, chp, n_it, inv_k, lane, sub, sh, r_own, c_own);
  }
  r_own = __builtin_amdgcn_ldexpf(r_own, -sx_own);  // the token's scale of the checked rotation undone
  const float rc = fminf(fmaxf(r_own, kScaleMin), kFp16Max);
  if (rc != r_own) flags |= KVARN_FLAG_SCALE_CLAMPED;
  const float r16_own = round_f16(rc);
  float at[8];  // Y = W' / (k r16 c16): per-token factor 1 / (k r16)
  row_gather8(__builtin_amdgcn_ldexpf(inv_k * __builtin_amdgcn_rcpf(r16_own), -sx_own), at, sh.grow[sub], g, c);
  float c16_own[2], ic_own[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float cv = c_own[q];
    const float x = fminf(fmaxf(cv, kScaleMin), kFp16Max);
    if (x != cv) flags |= KVARN_FLAG_SCALE_CLAMPED;
    c16_own[q] = round_f16(x);
    ic_own[q] = __builtin_amdgcn_rcpf(c16_own[q]);
  }
  if constexpr (DBG) {
    float ic[8], ex[8];
    col_gather8(ic_own, ic, sh.gcol[sub], g, c);
    row_gather8(__builtin_amdgcn_ldexpf(1.0f, -sx_own), ex, sh.grow[sub], g, c);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const long long off = (16 * mb + 4 * g + i) * dstride + 16 * nb + c;
          if (dbg_w) dbg_w[off] = acc[mb][nb][i] * inv_k * ex[4 * mb + i];
          if (dbg_y) dbg_y[off] = (acc[mb][nb][i] * at[4 * mb + i]) * ic[nb];
        }
  }
  // Y' = W' / (k r16) = Y c16 (the positive c16 is applied to the channel's min/max)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mb][nb][i] *= at[4 * mb + i];

  // per-channel asymmetric min/max 2-bit grid over the tile's G tokens
  float mnl[8], mxl[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    float lo = acc[0][nb][0], hi = acc[0][nb][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo = fminf(lo, acc[mb][nb][i]);
        hi = fmaxf(hi, acc[mb][nb][i]);
      }
    mnl[nb] = lo;
    mxl[nb] = hi;
  }
  float mn_own[2], mx_own[2];
  chan_reduce<NW>(mnl, mn_own, g, c, sub, sh.red_a, OpMin());
  chan_reduce<NW>(mxl, mx_own, g, c, sub, sh.red_b, OpMax());
  float s16_own[2], z16_own[2], al_own[2], ga_own[2];
  bool need_clamp_own = false;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float lo = mn_own[q] * ic_own[q], hi = mx_own[q] * ic_own[q];
    const float sr = (hi - lo) * (bits == 2 ? (1.0f / 3.0f) : 1.0f / (float)((1 << bits) - 1));
    const float sc = fminf(sr, kFp16Max);
    const float zc = fminf(fmaxf(lo, -kFp16Max), kFp16Max);
    if (sc != sr || zc != lo) {
      flags |= KVARN_FLAG_SCALE_CLAMPED;
      need_clamp_own = true;
    }
    const float big = fmaxf(fabsf(lo), fabsf(hi));
    if (sc != 0.0f && (!(sc >= kScaleMin) || !(big <= 200.0f * sc))) need_clamp_own = true;
    s16_own[q] = round_f16(sc);
    z16_own[q] = round_f16(zc);
    const float is = s16_own[q] > 0.0f ? __builtin_amdgcn_rcpf(s16_own[q]) : 0.0f;
    const float k4 = bits == 2 ? 0.25f : 1.0f;  // the 2-bit emitter takes u / 4
    al_own[q] = ic_own[q] * is * k4;  // u = (Y - z)/s = Y' (ic/s) - z/s
    ga_own[q] = -z16_own[q] * is * k4;
  }
  float al[8], ga[8];
  col_gather8(al_own, al, sh.gcol[sub], g, c);
  col_gather8(ga_own, ga, sh.gcol[sub], g, c);

  // codes, q = clamp(rne(u), 0, 2^bits - 1): 1.5 * 2^23 + u rounds half to even with q left in
  // bits 0..bits-1 and zeros up to bit 21; shifted into its slot, the junk above bit 21
  // falls outside the bytes kept (permute) / the byte stored. The clamp is needed only where u can
  // leave (-0.5, 2^bits - 0.5): with normal s16 and max(|Y|) <= 200 s16 the fp16 rounding of
  // z and s moves u by less than 0.1, so a wave whose channels all satisfy that skips it.
  const bool need_clamp = __any(need_clamp_own);
  if (need_clamp)
    emit_codes<NW, true>(acc, al, ga, stream, sub, g, c, sh, bits);
  else
    emit_codes<NW, false>(acc, al, ga, stream, sub, g, c, sh, bits);
  const int ttile0 = sub * 32 + 4 * g;
  const int RO = G * kD * bits / 8, CO = RO + 2 * G, SO = CO + 2 * kD, ZO = SO + 2 * kD;
  if ((c & 1) == 0) {
    const int t = ttile0 + 16 * (tau_own >> 2) + (tau_own & 3);
    *reinterpret_cast<uint16_t*>(sh.rec + RO + 2 * t) = (uint16_t)f16bits(r16_own);
  }
  if (sub == 0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 16 * (4 * q + g) + c;
      *reinterpret_cast<uint16_t*>(sh.rec + CO + 2 * j) = (uint16_t)f16bits(c16_own[q]);
      *reinterpret_cast<uint16_t*>(sh.rec + SO + 2 * j) = (uint16_t)f16bits(s16_own[q]);
      *reinterpret_cast<uint16_t*>(sh.rec + ZO + 2 * j) = (uint16_t)f16bits(z16_own[q]);
    }
  }
  tile_sync<NW>();
}

// tr: the record's bytes (a multiple of 16 for every supported width and group)
template <int NW>
__device__ __forceinline__ void copy_record(const TileLds<NW>& sh, uint8_t* dst, int lane, int sub, int tr) {
  const int n16 = tr / 16;
  const uint4* s = reinterpret_cast<const uint4*>(sh.rec);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int k = sub * 64 + lane; k < n16; k += 64 * NW) st_nt16(d + k, s[k]);
}

__device__ __forceinline__ void raise_flags(uint8_t* hdr, uint32_t f) {
  if (f) atomicOr(reinterpret_cast<uint32_t*>(hdr + kFlagsOff), f);
}

// ----------------------------------------------------------------------------- append
// Decode append of one (b, h, s) = job (s fastest, then h) by the G/32 waves
// sub = 0 .. NW-1 of a work-group; any further waves of the work-group must have exited
// (the barriers then wait on these waves only). The token goes to tail slot len mod G;
// when it completes a group, the group is quantized into the next tile record.
template <int NW, bool ABL>
__device__ void append_job(const AppendArgs& a, int job, int sub, int lane, TileLds<NW>& sh) {
  constexpr int G = 32 * NW;
  const int g = lane >> 4, c = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = a.cache;
  const int s = job % 2, h = (job / 2) % L.Hkv, b = job / 2 / L.Hkv;
  int32_t* lenp = reinterpret_cast<int32_t*>(a.cache + L.len_off(b, h, s));
  const int pos = *lenp;
  if (pos >= L.cap) {
    if (sub == 0 && lane == 0) raise_flags(hdr, KVARN_FLAG_CAPACITY);
    return;
  }
  uint32_t flags = 0;
  const uint16_t* src = (s ? a.v : a.k) + ((long long)b * L.Hkv + h) * kD;
  if (sub == 0 && g == 0) {  // the new token into the bf16 tail (16 lanes x 8 channels)
    *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, pos % G) + 16 * c) =
        canon8(*reinterpret_cast<const uint4*>(src + 8 * c), flags);
  }
  if ((pos + 1) % G == 0) {
    const bool idr = ABL && (L.variant & KVARN_VARIANT_NO_ROTATION);
    const Frags hf = frags_v<ABL>(idr, lane);
    // token 16 mb + c of this wave's block, channels 8 (4 ks + g) .. +7: the stored tail
    // tokens, and the token just written taken from the input, not from memory
    auto load = [&](int mb, int ks) -> uint4 {
      const int t = sub * 32 + 16 * mb + c;
      if (t == G - 1) {
        uint32_t seen = 0;  // flags of this token were raised with its tail write
        return canon8(*reinterpret_cast<const uint4*>(src + 8 * (4 * ks + g)), seen);
      }
      return *reinterpret_cast<const uint4*>(a.cache + L.tail_row(b, h, s, t) + 16 * (4 * ks + g));
    };
    b8v av[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const SigMask m = masks_v<ABL>(idr, hdr, 4 * ks + g);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) av[mb][ks] = sign8(load(mb, ks), m);
    }
    float p[2][8][4];
    f4v w4[2][8];
    float st = rotate_squares_v<ABL>(idr, av, hf, w4, p, c, sh.xt[sub]);
    int sx_own = 0;
    if (__any(!rotation_stands(idr, st)))
      st = rotate_checked<ABL>(idr, load, hdr, hf, av, w4, p, g, c, flags, sx_own, sh.xt[sub]);
    tile_finish<NW, false, ABL>(av, hf, w4, p, st, sx_own, lane, sub, s, L.n_it, L.variant, L.bits, sh, flags,
                                nullptr, nullptr, 0);
    const long long ro = record_at(a.cache, L, b, h, (pos + 1) / G - 1, s);
    if (ro >= 0)
      copy_record<NW>(sh, a.cache + ro, lane, sub, L.tr);
    else
      flags |= KVARN_FLAG_UNMAPPED;
  }
  raise_flags(hdr, flags);
  __syncthreads();  // every wave has read len before it moves
  if (sub == 0 && lane == 0) *lenp = pos + 1;
}

}  // namespace kvarn
