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
//   * Rotation on the matrix cores: the canonical inputs are exact in fp16 and the
//     Sylvester matrix is +-1, so W' = (x * sigma) H_syl is computed exactly by
//     v_mfma_f32_16x16x32_f16 with fp32 accumulation (2 token blocks x 8 channel
//     blocks x 4 K-steps). H_syl's 32x16 blocks are one of four register fragments
//     (+-F, +-G), so the 32 KiB matrix never leaves registers.
//   * The MFMA output leaves lane (g = lane/16, c = lane%16) with tokens 16mb + 4g + i
//     (mb < 2, i < 4) and channels 16nb + c (nb < 8): a token-axis sum is 8 in-lane
//     terms plus a DPP reduction over the 16 lanes of a row; a channel-axis sum is 8
//     in-lane terms plus permlane16/32 swaps across the 4 rows (and an LDS exchange
//     between the two waves of a G=64 tile).
//   * The 2-bit codes are formed with the magic-number trick: after clamping to
//     [0, 3] the value is added to 1.5 * 2^23, so fp32 round-half-to-even leaves the
//     code in mantissa bits 0..1 (bits 2..21 zero); it is then shifted into its slot.
// Reductions have a fixed order, so results are bit-identical run to run.
#include "kvarn_common.h"
#include "kvarn_launch.h"

namespace kvarn {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- lane exchange
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
constexpr int kQx1 = 0xB1, kQx2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

// All 16 lanes of a row get the row total; the pairing order is the same in every
// lane (commutative adds), so all lanes hold bit-identical values.
__device__ __forceinline__ float row_sum16(float x) {
  x += dppf<kQx1>(x);
  x += dppf<kQx2>(x);
  x += dppf<kHalfMirror>(x);
  x += dppf<kMirror>(x);
  return x;
}

// Combine the 4 rows (lanes c, c+16, c+32, c+48) with permlane swaps: rows 0+1 and
// 2+3, then the two halves.
template <typename Op>
__device__ __forceinline__ float col_reduce4(float x, Op op) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = op(__int_as_float(p[0]), __int_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return op(__int_as_float(q[0]), __int_as_float(q[1]));
}
struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMin { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// ----------------------------------------------------------------------------- Hadamard fragments
// B operand of the 16x16x32 MFMA for K-step ks (channels 32ks..32ks+31) and channel
// block nb: lane (g, c) holds H_syl[32ks + 8g + e][16nb + c], e < 8. With
// popcount((32ks + 8g + e) & (16nb + c)) = pc(e & c%8) + (g%2)(c/8) + (g/2)(nb%2)
// + pc(ks & nb/2), the fragment is F (nb even) or G = F * (-1)^(g/2) (nb odd), times
// the uniform sign (-1)^pc(ks & nb/2).
struct Frags {
  h8v v[4];  // F, -F, G, -G
};
__device__ __forceinline__ Frags hadamard_frags(int g, int c) {
  Frags h;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pc = __builtin_popcount(e & (c & 7)) + ((g & 1) & (c >> 3));
    const float f = (pc & 1) ? -1.0f : 1.0f;
    const float gg = (g >> 1) ? -f : f;
    h.v[0][e] = (_Float16)f;
    h.v[1][e] = (_Float16)(-f);
    h.v[2][e] = (_Float16)gg;
    h.v[3][e] = (_Float16)(-gg);
  }
  return h;
}
__device__ __forceinline__ int frag_index(int ks, int nb) {
  return ((nb & 1) << 1) | (__builtin_popcount(ks & (nb >> 1)) & 1);
}

// ----------------------------------------------------------------------------- inputs
// Sign masks for the 8 channels of chunk `chunk` (channels 8*chunk .. +7): bit 15 / 31
// of dword d flips fp16 halves 2d / 2d+1 where sigma is -1.
__device__ __forceinline__ void sigma_masks(const uint8_t* hdr, int chunk, uint32_t (&m)[4]) {
  const uint2 s = *reinterpret_cast<const uint2*>(hdr + kSigmaOff + 8 * chunk);
  m[0] = ((s.x << 8) & 0x8000u) | ((s.x << 16) & 0x80000000u);
  m[1] = ((s.x >> 8) & 0x8000u) | (s.x & 0x80000000u);
  m[2] = ((s.y << 8) & 0x8000u) | ((s.y << 16) & 0x80000000u);
  m[3] = ((s.y >> 8) & 0x8000u) | (s.y & 0x80000000u);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return f16bits(lo) | (f16bits(hi) << 16);
}

// 8 bf16 -> 8 canonical fp16 (round half to even), times sigma. Without clamping a
// value beyond fp16 becomes inf, which the caller detects and then redoes with CLAMP.
template <bool CLAMP>
__device__ __forceinline__ h8v canon_a(const uint4 w, const uint32_t (&m)[4]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float lo = bf16lo(ws[d]), hi = bf16hi(ws[d]);
    if constexpr (CLAMP) {
      lo = fminf(fmaxf(lo, -kFp16Max), kFp16Max);
      hi = fminf(fmaxf(hi, -kFp16Max), kFp16Max);
    }
    o[d] = pack_f16x2(lo, hi) ^ m[d];
  }
  return __builtin_bit_cast(h8v, make_uint4(o[0], o[1], o[2], o[3]));
}
__device__ __forceinline__ h8v sign_a(const uint4 w, const uint32_t (&m)[4]) {  // fp16 input
  return __builtin_bit_cast(h8v, make_uint4(w.x ^ m[0], w.y ^ m[1], w.z ^ m[2], w.w ^ m[3]));
}

// W'[token 16mb + 4g + i][channel 16nb + c] = sum_k A[mb][k] H[k][16nb + c]
__device__ __forceinline__ void rotate_block(const h8v (&a)[2][4], const Frags& hf, f4v (&acc)[2][8]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f4v s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb][ks], hf.v[frag_index(ks, nb)], s, 0, 0, 0);
      acc[mb][nb] = s;
    }
  }
  // Keep the A fragments allocated until every MFMA has issued: an MFMA whose
  // destination reuses its own A registers reads clobbered rows on this hardware.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(a[mb][ks]));
}

// ----------------------------------------------------------------------------- LDS
template <int NW>
struct TileLds {
  static constexpr int G = 32 * NW;
  static constexpr int TR = G * kD / 4 + 2 * G + 6 * kD;
  uint8_t rec[TR] __attribute__((aligned(16)));
  float red_a[NW][kD];
  float red_b[NW][kD];
};

// channel partials of the NW waves of a tile, combined in wave order
template <int NW, typename Op>
__device__ __forceinline__ void chan_reduce(float (&s)[8], TileLds<NW>& sh, int g, int c, int sub, Op op) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) s[nb] = col_reduce4(s[nb], op);
  if constexpr (NW > 1) {
    if (g == 0) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) sh.red_a[sub][16 * nb + c] = s[nb];
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float t = sh.red_a[0][16 * nb + c];
#pragma unroll
      for (int w = 1; w < NW; ++w) t = op(t, sh.red_a[w][16 * nb + c]);
      s[nb] = t;
    }
    __syncthreads();
  }
}

template <int NW>
__device__ __forceinline__ void chan_minmax(float (&mn)[8], float (&mx)[8], TileLds<NW>& sh, int g, int c,
                                            int sub) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    mn[nb] = col_reduce4(mn[nb], OpMin());
    mx[nb] = col_reduce4(mx[nb], OpMax());
  }
  if constexpr (NW > 1) {
    if (g == 0) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        sh.red_a[sub][16 * nb + c] = mn[nb];
        sh.red_b[sub][16 * nb + c] = mx[nb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float a = sh.red_a[0][16 * nb + c], b = sh.red_b[0][16 * nb + c];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        a = fminf(a, sh.red_a[w][16 * nb + c]);
        b = fmaxf(b, sh.red_b[w][16 * nb + c]);
      }
      mn[nb] = a;
      mx[nb] = b;
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- the tile core
// From the rotated block W' = sqrt(D) W (acc) and its squares p, with st holding the
// first token-axis sums (u = 1): VarN, stored scales, grid, codes; the record is
// assembled in sh.rec. Steps follow the ai-paper-analysis page, section 3.2.
//
// VarN with cumulative scales (the mean square of W/(r c) along the axis becomes 1):
//   token pass   S'_t = sum_j W'_tj^2 / c_j^2,   r_t = sqrt(S'_t) / D,  v_t = D / S'_t
//   channel pass S'_j = sum_t W'_tj^2 v_t,       c_j = sqrt(S'_j / G),  u_j = G / S'_j
// (with W' = sqrt(D) W these are the oracle's r_t <- r_t sqrt(ms_t), c_j <- c_j sqrt(ms_j));
// an all-zero line keeps its scale.
template <int NW, bool DBG>
__device__ void tile_finish(f4v (&acc)[2][8], float (&p)[2][8][4], float (&st)[2][4], int lane, int sub,
                            int stream, int n_it, TileLds<NW>& sh, uint32_t& flags, float* dbg_w,
                            float* dbg_y, long long dstride) {
  constexpr int G = 32 * NW;
  const int g = lane >> 4, c = lane & 15;

  float u[8], v[2][4], rr[2][4], cc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    u[nb] = 1.0f;
    cc[nb] = 1.0f;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[mb][i] = 1.0f / kD;
      rr[mb][i] = 1.0f;
    }
  for (int it = 0; it < n_it; ++it) {
    if (it > 0) {  // token pass (the first one arrives precomputed in st)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = 0.0f;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) s = fmaf(p[mb][nb][i], u[nb], s);
          st[mb][i] = row_sum16(s);
        }
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (st[mb][i] > 0.0f) {
          v[mb][i] = (float)kD * __builtin_amdgcn_rcpf(st[mb][i]);
          rr[mb][i] = __builtin_amdgcn_sqrtf(st[mb][i]) * (1.0f / kD);
        }
    float sj[8];  // channel pass
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float s = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(p[mb][nb][i], v[mb][i], s);
      sj[nb] = s;
    }
    chan_reduce<NW>(sj, sh, g, c, sub, OpAdd());
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      if (sj[nb] > 0.0f) {
        u[nb] = (float)G * __builtin_amdgcn_rcpf(sj[nb]);
        cc[nb] = __builtin_amdgcn_sqrtf(sj[nb] * (1.0f / G));
      }
  }

  // stored scales: fp16, clamped to [2^-14, 65504]
  float r16[2][4], at[2][4], c16[8], ic[8];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = fminf(fmaxf(rr[mb][i], kScaleMin), kFp16Max);
      if (x != rr[mb][i]) flags |= KVARN_FLAG_SCALE_CLAMPED;
      r16[mb][i] = round_f16(x);
      at[mb][i] = kInvSqrtD * __builtin_amdgcn_rcpf(r16[mb][i]);  // Y = W' / (sqrt(D) r16 c16)
    }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const float x = fminf(fmaxf(cc[nb], kScaleMin), kFp16Max);
    if (x != cc[nb]) flags |= KVARN_FLAG_SCALE_CLAMPED;
    c16[nb] = round_f16(x);
    ic[nb] = __builtin_amdgcn_rcpf(c16[nb]);
  }
  if constexpr (DBG) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const long long off = (16 * mb + 4 * g + i) * dstride + 16 * nb + c;
          if (dbg_w) dbg_w[off] = acc[mb][nb][i] * kInvSqrtD;
          if (dbg_y) dbg_y[off] = (acc[mb][nb][i] * at[mb][i]) * ic[nb];
        }
  }
  // Y' = W' a_t = Y c16 (the positive per-channel c16 is applied to the channel's min/max)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mb][nb][i] *= at[mb][i];

  // per-channel asymmetric min/max 2-bit grid over the tile's G tokens
  float mn[8], mx[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    float a = acc[0][nb][0], b = acc[0][nb][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a = fminf(a, acc[mb][nb][i]);
        b = fmaxf(b, acc[mb][nb][i]);
      }
    mn[nb] = a;
    mx[nb] = b;
  }
  chan_minmax<NW>(mn, mx, sh, g, c, sub);
  float s16[8], z16[8], al[8], ga[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const float lo = mn[nb] * ic[nb], hi = mx[nb] * ic[nb];
    const float sr = (hi - lo) * (1.0f / 3.0f);
    const float sc = fminf(sr, kFp16Max);
    const float zc = fminf(fmaxf(lo, -kFp16Max), kFp16Max);
    if (sc != sr || zc != lo) flags |= KVARN_FLAG_SCALE_CLAMPED;
    s16[nb] = round_f16(sc);
    z16[nb] = round_f16(zc);
    const float is = s16[nb] > 0.0f ? __builtin_amdgcn_rcpf(s16[nb]) : 0.0f;
    al[nb] = ic[nb] * is;  // u = (Y - z)/s = Y' (ic/s) - z/s
    ga[nb] = -z16[nb] * is;
  }

  // codes, q = clamp(rne(u), 0, 3): clamp, then 1.5 * 2^23 + u rounds half to even
  // with q left in bits 0..1 and zeros in bits 2..21; shifted into its 2-bit slot,
  // the junk above bit 21 falls outside the masked half-word / byte
  const int ttile0 = sub * 32 + 4 * g;  // token of (mb = 0, i = 0) inside the tile
  if (stream == 0) {  // K: word w = c/2 of token t holds channel 16nb + c in slot 8(c%2) + nb
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h = 0;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          float t = fmaf(acc[mb][nb][i], al[nb], ga[nb]);
          t = __builtin_amdgcn_fmed3f(t, 0.0f, 3.0f);
          h |= (uint32_t)__float_as_int(t + 12582912.0f) << (2 * nb);
        }
        h &= 0xFFFFu;
        const uint32_t hp = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, kQx1, 0xF, 0xF, false);
        if ((c & 1) == 0)
          *reinterpret_cast<uint32_t*>(sh.rec + (ttile0 + 16 * mb + i) * 32 + 2 * c) = h | (hp << 16);
      }
  } else {  // V: byte j*G/4 + t/4 holds tokens 4(t/4) .. +3 of channel j, token t%4 in slot t%4
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint32_t h = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = fmaf(acc[mb][nb][i], al[nb], ga[nb]);
          t = __builtin_amdgcn_fmed3f(t, 0.0f, 3.0f);
          h |= (uint32_t)__float_as_int(t + 12582912.0f) << (2 * i);
        }
        sh.rec[(16 * nb + c) * (G / 4) + (ttile0 + 16 * mb) / 4] = (uint8_t)h;
      }
  }
  constexpr int RO = G * kD / 4, CO = RO + 2 * G, SO = CO + 2 * kD, ZO = SO + 2 * kD;
  if (c == 0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      uint2 w;
      w.x = pack_f16x2(r16[mb][0], r16[mb][1]);
      w.y = pack_f16x2(r16[mb][2], r16[mb][3]);
      *reinterpret_cast<uint2*>(sh.rec + RO + 2 * (ttile0 + 16 * mb)) = w;
    }
  }
  if (g == 0 && sub == 0) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int j = 16 * nb + c;
      *reinterpret_cast<uint16_t*>(sh.rec + CO + 2 * j) = (uint16_t)f16bits(c16[nb]);
      *reinterpret_cast<uint16_t*>(sh.rec + SO + 2 * j) = (uint16_t)f16bits(s16[nb]);
      *reinterpret_cast<uint16_t*>(sh.rec + ZO + 2 * j) = (uint16_t)f16bits(z16[nb]);
    }
  }
  __syncthreads();
}

// squares of the rotated block and their per-token sums (the first token pass, u = 1)
__device__ __forceinline__ void squares_and_token_sums(const f4v (&acc)[2][8], float (&p)[2][8][4],
                                                       float (&st)[2][4]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        p[mb][nb][i] = acc[mb][nb][i] * acc[mb][nb][i];
        s += p[mb][nb][i];
      }
      st[mb][i] = row_sum16(s);
    }
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

__device__ __forceinline__ uint4 pack8_f16(const float (&x)[8]) {
  uint4 o;
  o.x = pack_f16x2(x[0], x[1]);
  o.y = pack_f16x2(x[2], x[3]);
  o.z = pack_f16x2(x[4], x[5]);
  o.w = pack_f16x2(x[6], x[7]);
  return o;
}
// bf16 x 8 -> canonical fp16 values (saturating), largest magnitude into amax
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

// ----------------------------------------------------------------------------- prefill
// Work-groups [0, tile_blocks) quantize full tiles, 4/NW tiles per work-group; the
// remaining work-groups write the fp16 tail and len[], one (b, h, s) per wave.
template <int NW, bool DBG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int TPW = 4 / NW;
  __shared__ TileLds<NW> sh_all[TPW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = a.cache;
  uint32_t flags = 0;
  const long long tile_blocks = (a.jobs + TPW - 1) / TPW;

  if ((long long)blockIdx.x >= tile_blocks) {
    const long long sj = ((long long)blockIdx.x - tile_blocks) * 4 + wave;  // (b, h, s)
    if (sj >= 2LL * L.B * L.Hkv) return;
    const int s = (int)(sj % 2), h = (int)((sj / 2) % L.Hkv), b = (int)(sj / 2 / L.Hkv);
    const uint16_t* src = s ? a.v : a.k;
    for (int t = a.nfull * L.G + g; t < a.T; t += 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + (((long long)b * a.T + t) * L.Hkv + h) * kD + 8 * c);
      float x[8], amax = 0.0f;
      canon8_bf16(w, x, amax);
      flags |= sat_flag(amax);
      *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, t % L.G) + 16 * c) = pack8_f16(x);
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
  const int t0 = tile * L.G + sub * 32;  // first token of this wave's block
  const Frags hf = hadamard_frags(g, c);

  // A rows are tokens t0 + 16mb + c; K chunk 4ks + g holds channels 8(4ks + g) .. +7
  uint4 raw[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      raw[mb][ks] = *reinterpret_cast<const uint4*>(
          src + (((long long)b * a.T + t0 + 16 * mb + c) * L.Hkv + h) * kD + 8 * (4 * ks + g));
  uint32_t msk[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) sigma_masks(hdr, 4 * ks + g, msk[ks]);

  f4v acc[2][8];
  float p[2][8][4], st[2][4];
  {
    h8v av[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[mb][ks] = canon_a<false>(raw[mb][ks], msk[ks]);
    rotate_block(av, hf, acc);
  }
  squares_and_token_sums(acc, p, st);
  bool bad = false;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) bad |= !(st[mb][i] <= 3.0e38f);
  if (__any(bad)) {  // an input beyond fp16 (inf after conversion): redo saturating
    h8v av[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[mb][ks] = canon_a<true>(raw[mb][ks], msk[ks]);
    rotate_block(av, hf, acc);
    squares_and_token_sums(acc, p, st);
    flags |= KVARN_FLAG_SATURATED;
  }

  float* dw = nullptr;
  float* dy = nullptr;
  long long dstride = 0;
  if constexpr (DBG) {
    const long long tfull = (long long)a.nfull * L.G;
    const long long doff = (((long long)b * tfull + t0) * L.Hkv + h) * kD;
    float* pw = s ? a.wv : a.wk;
    float* py = s ? a.yv : a.yk;
    dstride = (long long)L.Hkv * kD;
    dw = (valid && pw) ? pw + doff : nullptr;
    dy = (valid && py) ? py + doff : nullptr;
  }
  tile_finish<NW, DBG>(acc, p, st, lane, sub, s, L.n_it, sh, flags, dw, dy, dstride);
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
  const int g = lane >> 4, c = lane & 15;
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
  const uint16_t* src = (s ? a.v : a.k) + ((long long)b * L.Hkv + h) * kD;
  if (sub == 0 && g == 0) {  // the new token into the fp16 tail (16 lanes x 8 channels)
    float xin[8], amax = 0.0f;
    canon8_bf16(*reinterpret_cast<const uint4*>(src + 8 * c), xin, amax);
    flags |= sat_flag(amax);
    *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, pos % G) + 16 * c) = pack8_f16(xin);
  }
  if ((pos + 1) % G == 0) {
    const Frags hf = hadamard_frags(g, c);
    h8v av[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t m[4];
      sigma_masks(hdr, 4 * ks + g, m);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int t = sub * 32 + 16 * mb + c;  // token of this A row inside the tile
        uint4 w;
        if (t == G - 1) {  // the token just written: take it from the input, not from memory
          float x[8], amax = 0.0f;
          canon8_bf16(*reinterpret_cast<const uint4*>(src + 8 * (4 * ks + g)), x, amax);
          w = pack8_f16(x);
        } else {
          w = *reinterpret_cast<const uint4*>(a.cache + L.tail_row(b, h, s, t) + 16 * (4 * ks + g));
        }
        av[mb][ks] = sign_a(w, m);
      }
    }
    f4v acc[2][8];
    float p[2][8][4], st[2][4];
    rotate_block(av, hf, acc);
    squares_and_token_sums(acc, p, st);
    tile_finish<NW, false>(acc, p, st, lane, sub, s, L.n_it, sh, flags, nullptr, nullptr, 0);
    copy_record<NW>(sh, a.cache + L.record(b, h, (pos + 1) / G - 1, s), lane, sub);
  }
  raise_flags(hdr, flags);
  __syncthreads();
  if (threadIdx.x == 0) *lenp = pos + 1;
}

// ----------------------------------------------------------------------------- launchers
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

}  // namespace kvarn
