// KVarN read path on gfx950: single-query decode attention over the 2-bit cache.
//
// The query takes the same randomized Hadamard rotation as the keys, so scores are
// computed in rotated space without rotating the cache back (ai-paper-analysis page,
// section 3.1: H H^T = I leaves Q K^T unchanged). Dequantization is folded into the
// products: for a K tile with scales r (token), c, s, z (channel) and codes q,
//   score_t = scale * r_t * (sum_j q_tj a_j + b),  a_j = q_rot,j c_j s_j,  b = sum_j q_rot,j c_j z_j,
// and for a V tile with weights w_t = p_t r_t (p the softmax numerators),
//   o_rot,j += c_j s_j sum_t w_t q_tj + c_j z_j sum_t w_t.
// Both sums over codes run on the 16x16x32 f16 MFMA:
//   * codes become exact f16 values 0..3: a 2-bit code zero-extended to a nibble is
//     the fp4 (e2m1) value q/2, and the packed fp4 -> f16 conversion with scale 2
//     turns one byte (two nibbles) into two f16 codes;
//   * the per-tile factors (a_j, w_t) are split into f16 hi + lo parts, held in two
//     MFMA columns / rows and added after the product, so the result keeps about 22
//     bits of each factor; a per-tile power-of-two scale puts the largest factor near
//     2^14 first;
//   * K: A = codes (16 tokens x 32 channels), B = a-values (32 channels x {hi, lo} x
//     4 query heads); V: A = weights ({hi, lo} x 4 query heads x 32 tokens, twice:
//     rows 8..15 hold the same weights against a second channel block), B = codes.
// The K code word layout puts each channel pair (2i, 2i+1) in one byte, so a converted
// byte is one dword of the MFMA operand; the V layout (tokens fastest) gives 8
// consecutive tokens of a channel per 16-bit load.
//
// Work split: a work-group of 4 waves per (batch, kv head, group of up to 4 query heads,
// span); the full tiles of a sequence are cut into min(nspan, tiles) spans of equal size,
// so every work-group of a call has the same work. Wave w takes tiles w, w + 4, ... of its
// span with its own
// online softmax, the 4 wave states are merged in LDS and one partial (m, l, o_rot) per
// query head and span goes to the workspace. The merge kernel combines the spans in
// index order (log-sum-exp), adds the bf16 tail tokens (unrotated, scored in original
// space), rotates the V part back by H_D^T and normalizes. Scores live in log2 units.
//
// Fused decode step (append + attention): the tile pass records each sequence's length
// in the workspace; the merge launch then also runs the append jobs (tail write, group
// quantization, len update) as extra work-groups. Its rows take the call's new token
// from the input, read only tail slots below the recorded length, and never read len
// or tile records, so they do not race with the append jobs of the same launch.
#include <atomic>

#include "kvarn_common.h"
#include "kvarn_launch.h"
#include "quantize_dev.h"

namespace kvarn {

constexpr int kPart = 4 + kD;  // floats per (b, q head, span): m (log2 units), l, 2 pad, o_rot[D]
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kNib = 0x33333333u;

struct WaveLds {
  uint4 bop[128];    // K-side B operand, unit (s, g, n8 ^ swz(s, g)) = 4 dwords
  float vf[16][20];  // V fold factors (c s, c z) of channel 16 blk + n at [n][2 blk], rows
                     // padded to 80 B so the 16 lanes of a row read distinct banks
};
struct AttnLds {
  float qrot[4][kD];
  union {
    WaveLds w[4];
    float oo[4][4][kD];  // wave, query head, channel (after the tile loop)
  } u;
  float mm[4][4], ll[4][4];
};

// ----------------------------------------------------------------------------- helpers
// Two f16 codes from byte BY of a nibble plane (each nibble a 2-bit code, e2m1 = q/2).
template <int BY>
__device__ __forceinline__ uint32_t cvt2(uint32_t plane) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(plane, 2.0f, BY));
}
// The same for plane B of 3- and 4-bit codes, worth 4x: a nibble q_B (0..3, or 0..1 for
// the 1-bit plane) is the e2m1 value q_B/2, converted with scale 8 to 4 q_B.
template <int BY>
__device__ __forceinline__ uint32_t cvt2_hi(uint32_t plane) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(plane, 8.0f, BY));
}
constexpr uint32_t kBit = 0x11111111u;  // bit 0 of each nibble
__device__ __forceinline__ h8v as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(h8v, v);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}

// x - m * (fp16 half HI of h), one v_fma_mix_f32: the residual of an fp16 rounding
// (exact, as x and the rounded value are within a factor of two of each other)
template <int HI>
__device__ __forceinline__ float sub_f16(float x, uint32_t h, float m) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(-m), "v"(x));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(-m), "v"(x));
  return r;
}

// max over the 64 lanes of non-negative floats (compared as integers), wave-uniform
__device__ __forceinline__ uint32_t wave_max_pos(float x) {
  uint32_t u = (uint32_t)__float_as_int(x);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kQx1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kQx2, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kHalfMirror, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, kMirror, 0xF, 0xF, true));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)u, 0), (uint32_t)__builtin_amdgcn_readlane((int)u, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)u, 32), (uint32_t)__builtin_amdgcn_readlane((int)u, 48));
  return max(a, b);
}
// Power-of-two scale 2^(14 - e) for a bound with biased exponent e, and its inverse;
// e is clamped to [15, 254] so both are normal floats.
__device__ __forceinline__ void pow2_scale(uint32_t bound_bits, float& s, float& inv) {
  int e = (int)(bound_bits >> 23);
  e = e < 15 ? 15 : (e > 254 ? 254 : e);
  s = __int_as_float((268 - e) << 23);
  inv = __int_as_float((e - 14) << 23);
}
// across the 4 rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float rows_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = vmax(__int_as_float(p[0]), __int_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return vmax(__int_as_float(q[0]), __int_as_float(q[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(p[0]) + __int_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}
// Sum over the wave of 4 per-lane partials; lane c of every row returns the total of
// partial (c >> 1) & 3. Reduce-scatter: row_half_mirror pairs lanes differing in bit 2
// (each keeps the pair of partials its bit 2 selects), quad xor 2 pairs bit 1, then the
// sets {c, c ^ 1} and the row halves (row_ror:8) and the 4 rows are summed.
__device__ __forceinline__ float reduce4(const float (&v)[4], int c) {
  const bool b2 = (c >> 2) & 1, b1 = (c >> 1) & 1;
  const float k0 = b2 ? v[2] : v[0], k1 = b2 ? v[3] : v[1];
  const float s0 = b2 ? v[0] : v[2], s1 = b2 ? v[1] : v[3];
  const float u0 = k0 + dppf<kHalfMirror>(s0), u1 = k1 + dppf<kHalfMirror>(s1);
  float x = (b1 ? u1 : u0) + dppf<kQx2>(b1 ? u0 : u1);
  x += dppf<kQx1>(x);
  x += dppf<kRor8>(x);
  return rows_sum(x);
}

// ----------------------------------------------------------------------------- main kernel
// Lane roles (g = lane / 16, c = lane % 16, m = lane):
//  * K MFMA, token block mb: lane (c, g) supplies token 32 kb + 8 (c/4) + (c%2) +
//    4 ((c/2)%2) + 2 (mb%2) (kb = mb/2), words 2g, 2g+1; the score output leaves lane
//    (c, g) with tokens 32 kb + 8 g + tau(2 i + mb%2), tau = [0,2,1,3,4,6,5,7], in
//    column c = 2 qh + part (c >= 8 repeats columns 0..7);
//  * MFMA s takes word 2g + s/2, channel blocks nb = 4 (s%2) .. +3, one converted byte
//    per block: element pair (2 (nb%4), +1) = channels (16 nb + 2w, +1);
//  * lane m computes the a-values of channels (16 (m/8) + 2 (m%8), +1) for the 4 query
//    heads and writes them to the B-operand slot (s, g, kk) = (2 (m%2) + m/32, (m%8)/2,
//    (m/8)%4) in LDS; it also owns those channels' V fold factors;
//  * V MFMA i (i < 4): columns = channels 16 i + c (rows 0..7 of A) and 16 (i+4) + c
//    (rows 8..15), lane (c, g) folds rows 4 (g%2) .. +3 of block i + 4 (g/2), i.e. query
//    heads 2 (g%2) + {0, 1} of channel 16 (i + 4 (g/2)) + c.
//
// BITS = 3 or 4: the codes are plane A (bits 0..1, the 2-bit layout) plus 4 x plane B
// (4-bit: the 2-bit layout at PB; 3-bit: the 1-bit layout, whose words give the nibble
// planes of two 2-bit words by shifts and masks). Plane B runs through the same MFMAs
// with codes worth 4 q_B, accumulated into the same sums.
template <int G, int BITS>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int NKB = G / 32;  // 32-token blocks per tile
  constexpr int NMB = 2 * NKB; // 16-token K blocks per tile
  constexpr int PB = G * kD / 4;  // plane B of 3- and 4-bit codes
  constexpr int RO = G * kD * BITS / 8, CO = RO + 2 * G, SO = CO + 2 * kD, ZO = SO + 2 * kD;
  __shared__ AttnLds sh;
  const Layout& L = a.L;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  // Work-group i runs on XCD i % 8, and each XCD has its own L2. The logical job is
  // remapped so that every XCD takes a contiguous range of jobs, and the query-head groups
  // of one span are adjacent in it: work-groups that stream the same K/V records run on
  // one XCD at about the same time and share its L2.
  int bid;
  {
    const int nb = gridDim.x, q = nb >> 3, r = nb & 7, x = blockIdx.x & 7, k = blockIdx.x >> 3;
    bid = x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
  }
  const int qg = bid % a.nqg;  // logical job = ((b Hkv + h) nspan + span) nqg + qg
  bid /= a.nqg;
  const int span = bid % a.nspan;
  bid /= a.nspan;
  const int h = bid % L.Hkv, b = bid / L.Hkv;
  const int n = *reinterpret_cast<const int32_t*>(a.cache + L.len_off(b, h, 0));
  if (span == 0 && qg == 0 && threadIdx.x == 0) a.lens_ws[b * L.Hkv + h] = n;  // for the merge
  // the full tiles split into nsp spans of equal size (within one tile) whatever the length
  const int nfull = n / G, nsp = min(a.nspan, nfull);
  if (span >= nsp) return;  // uniform over the work-group
  const int t0 = (int)((long long)span * nfull / nsp), t1 = (int)((long long)(span + 1) * nfull / nsp);
  const int q0 = qg * 4;
  const float qscale = kLog2e * a.scale;

  // --- query heads q0 .. q0+3 of this kv head, rotated into the cache basis
  if (wave == 0) {
    float qv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (q0 + g < a.grp) {
      const uint4 w = *reinterpret_cast<const uint4*>(a.q + ((long long)b * a.Hq + h * a.grp + q0 + g) * kD + 8 * c);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qv[2 * k] = bf16lo(ws[k]);
        qv[2 * k + 1] = bf16hi(ws[k]);
      }
    }
    if (!(a.flags & KVARN_Q_PREROTATED) && !a.idr) {
      float sg[8];
      load_sigma(a.cache, c, sg);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] *= sg[e];
      fwht128(qv, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] *= kInvSqrtD;
    }
    store8f(&sh.qrot[g][8 * c], qv);
  }
  __syncthreads();

  // --- per-lane constants
  const int nbm = lane >> 3, wm = lane & 7;
  const int j0 = 16 * nbm + 2 * wm;
  float qr[4][2];
  float mql = 0.0f;
#pragma unroll
  for (int qh = 0; qh < 4; ++qh) {
    const float2 v = *reinterpret_cast<const float2*>(&sh.qrot[qh][j0]);
    qr[qh][0] = v.x;
    qr[qh][1] = v.y;
    mql = fmaxf(mql, fmaxf(fabsf(v.x), fabsf(v.y)));
  }
  const float mq = __int_as_float((int)wave_max_pos(mql));
  WaveLds& wl = sh.u.w[wave];
  uint32_t* bop = reinterpret_cast<uint32_t*>(wl.bop);
  const int s_m = 2 * (wm & 1) + (nbm >> 2), g_m = wm >> 1, kk_m = nbm & 3;
  const int wbase = (s_m * 4 + g_m) * 8, wswz = (2 * s_m + (g_m >> 1)) & 7;
  int krow[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
    krow[mb] = 32 * (mb >> 1) + 8 * (c >> 2) + (c & 1) + 4 * ((c >> 1) & 1) + 2 * (mb & 1);
  const float partf = (float)(c & 1);
  const bool rows_lo = c < 8;
  // byte permutes building (even-block token, odd-block token) f16 pairs from this lane's
  // pair `mine` (bytes 0..3) and the partner's `theirs` (bytes 4..7)
  const uint32_t sel_lo = rows_lo ? 0x05040100u : 0x01000504u;
  const uint32_t sel_hi = rows_lo ? 0x07060302u : 0x03020706u;
  const uint32_t sh_g1 = (uint32_t)(g & 1);

  float m_run = -INFINITY, l_run = 0.0f;
  float o[2][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[0][k] = o[1][k] = 0.0f;

  // paged cache: the page map entries of this wave's tiles t0 + wave + 4 i, lane i holding
  // entry i (64 at a time), so that no tile waits on a map read before its record loads
  const int32_t* pmap = reinterpret_cast<const int32_t*>(a.cache + L.map_off) + (long long)b * L.tiles;
  int page_i = -1;
  for (int tile = t0 + wave, it = 0; tile < t1; tile += 4, ++it) {
    long long roff;
    if (L.num_pages == 0) {
      roff = L.record_seq(b, h, tile, 0);
    } else {
      if ((it & 63) == 0) {
        const int tl = tile + 4 * lane;
        page_i = tl < t1 ? pmap[tl] : -1;
      }
      const int page = __builtin_amdgcn_readlane(page_i, it & 63);
      roff = (page < 0 || page >= L.num_pages) ? -1 : L.page_record(page, h, 0);
    }
    if (roff < 0) continue;  // paged cache, no page for this tile: its tokens are left out
    const uint8_t* rk = a.cache + roff;
    const uint8_t* rv = rk + L.tr;
    // ---- loads
    uint2 kc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) kc[mb] = ld_nt8(rk + krow[mb] * 32 + 8 * g);
    uint2 kcb[BITS > 2 ? NMB : 1];  // plane B: two 2-bit words (BITS 4) or one 1-bit word in .x
    if constexpr (BITS == 4) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) kcb[mb] = *reinterpret_cast<const uint2*>(rk + PB + krow[mb] * 32 + 8 * g);
    } else if constexpr (BITS == 3) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
        kcb[mb] = make_uint2(*reinterpret_cast<const uint32_t*>(rk + PB + krow[mb] * 16 + 4 * g), 0u);
    }
    const uint32_t kcs = *reinterpret_cast<const uint32_t*>(rk + CO + 4 * lane);
    const uint32_t kss = *reinterpret_cast<const uint32_t*>(rk + SO + 4 * lane);
    const uint32_t kzs = *reinterpret_cast<const uint32_t*>(rk + ZO + 4 * lane);
    const uint32_t vcs = *reinterpret_cast<const uint32_t*>(rv + CO + 4 * lane);
    const uint32_t vss = *reinterpret_cast<const uint32_t*>(rv + SO + 4 * lane);
    const uint32_t vzs = *reinterpret_cast<const uint32_t*>(rv + ZO + 4 * lane);
    uint4 kr[NKB], vr[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      kr[kb] = ld_nt16(rk + RO + 2 * (32 * kb + 8 * g));
      vr[kb] = ld_nt16(rv + RO + 2 * (32 * kb + 8 * g));
    }
    uint32_t vq[4][NKB];  // channel 16 i + c (low half) and 16 (i + 4) + c (high half)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t lo =
            __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(rv + (16 * i + c) * (G / 4) + 2 * (4 * kb + g)));
        const uint32_t hi = __builtin_nontemporal_load(
            reinterpret_cast<const uint16_t*>(rv + (16 * (i + 4) + c) * (G / 4) + 2 * (4 * kb + g)));
        vq[i][kb] = lo | (hi << 16);
      }
    // plane B of V: BITS 4 as vq; BITS 3 one 1-bit word per channel pair {i, i + 1} (i even)
    uint32_t vqb[BITS > 2 ? 4 : 1][NKB];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(rv + PB + (16 * i + c) * (G / 4) + 2 * (4 * kb + g));
          const uint32_t hi =
              *reinterpret_cast<const uint16_t*>(rv + PB + (16 * (i + 4) + c) * (G / 4) + 2 * (4 * kb + g));
          vqb[i][kb] = lo | (hi << 16);
        }
    } else if constexpr (BITS == 3) {
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          vqb[ip][kb] = *reinterpret_cast<const uint32_t*>(rv + PB + 4 * ((16 * ip + c) * (G / 8) + 4 * kb + g));
    }

    // ---- K-side factors of this lane's channel pair; per-tile scale of the a-values
    const float cs0 = mul_f16<0>(kcs, kss), cs1 = mul_f16<1>(kcs, kss);
    const float cz0 = mul_f16<0>(kcs, kzs), cz1 = mul_f16<1>(kcs, kzs);
    float sB, invSB;
    pow2_scale(wave_max_pos(fmaxf(cs0, cs1) * mq), sB, invSB);
    const float f0 = cs0 * sB, f1 = cs1 * sB;
    wave_sync();  // the previous tile's LDS reads are issued before these writes
#pragma unroll
    for (int qh = 0; qh < 4; ++qh) {
      const float a0 = f0 * qr[qh][0], a1 = f1 * qr[qh][1];
      const uint32_t hv = pack_f16(a0, a1);
      const uint32_t lv = pack_f16(sub_f16<0>(a0, hv, 1.0f), sub_f16<1>(a1, hv, 1.0f));
      bop[(wbase + ((2 * qh) ^ wswz)) * 4 + kk_m] = hv;
      bop[(wbase + ((2 * qh + 1) ^ wswz)) * 4 + kk_m] = lv;
    }
    *reinterpret_cast<float2*>(&wl.vf[2 * wm][2 * nbm]) = make_float2(mul_f16<0>(vcs, vss), mul_f16<0>(vcs, vzs));
    *reinterpret_cast<float2*>(&wl.vf[2 * wm + 1][2 * nbm]) = make_float2(mul_f16<1>(vcs, vss), mul_f16<1>(vcs, vzs));
    float bp[4];
#pragma unroll
    for (int qh = 0; qh < 4; ++qh) bp[qh] = fmaf(qr[qh][0], cz0, qr[qh][1] * cz1);
    const float bq = reduce4(bp, c) * qscale;
    wave_sync();

    // ---- scores: S = sum_j q_tj a_j for the lane's 8 (or 16) tokens and query head c/2 % 4
    h8v bk[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int unit = (s * 4 + g) * 8 + ((c & 7) ^ ((2 * s + (g >> 1)) & 7));
      bk[s] = __builtin_bit_cast(h8v, wl.bop[unit]);
    }
    const float K1 = qscale * invSB;
    // Columns 8..15 repeat 0..7, so from here lane c < 8 takes the even 16-token blocks
    // (mb % 2 = 0) and lane c + 8 the odd ones; partial sums meet through row_ror:8.
    float lsc[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f4v sc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t x0 = kc[2 * kb + h2].x, x1 = kc[2 * kb + h2].y;
        const uint32_t e0 = x0 & kNib, o0 = (x0 >> 2) & kNib, e1 = x1 & kNib, o1 = (x1 >> 2) & kNib;
        f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
        h8v av0 = as_h8(cvt2<0>(e0), cvt2<0>(o0), cvt2<1>(e0), cvt2<1>(o0));
        h8v av1 = as_h8(cvt2<2>(e0), cvt2<2>(o0), cvt2<3>(e0), cvt2<3>(o0));
        h8v av2 = as_h8(cvt2<0>(e1), cvt2<0>(o1), cvt2<1>(e1), cvt2<1>(o1));
        h8v av3 = as_h8(cvt2<2>(e1), cvt2<2>(o1), cvt2<3>(e1), cvt2<3>(o1));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, bk[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, bk[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av2, bk[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av3, bk[3], acc, 0, 0, 0);
        asm volatile("" : "+v"(acc) : "v"(av0), "v"(av1), "v"(av2), "v"(av3), "v"(bk[0]), "v"(bk[1]), "v"(bk[2]),
                     "v"(bk[3]));
        if constexpr (BITS > 2) {
          uint32_t eb0, ob0, eb1, ob1;  // nibble planes of plane B, as e0, o0, e1, o1 above
          if constexpr (BITS == 4) {
            const uint32_t y0 = kcb[2 * kb + h2].x, y1 = kcb[2 * kb + h2].y;
            eb0 = y0 & kNib, ob0 = (y0 >> 2) & kNib, eb1 = y1 & kNib, ob1 = (y1 >> 2) & kNib;
          } else {
            const uint32_t y = kcb[2 * kb + h2].x;
            eb0 = y & kBit, ob0 = (y >> 1) & kBit, eb1 = (y >> 2) & kBit, ob1 = (y >> 3) & kBit;
          }
          const h8v bv0 = as_h8(cvt2_hi<0>(eb0), cvt2_hi<0>(ob0), cvt2_hi<1>(eb0), cvt2_hi<1>(ob0));
          const h8v bv1 = as_h8(cvt2_hi<2>(eb0), cvt2_hi<2>(ob0), cvt2_hi<3>(eb0), cvt2_hi<3>(ob0));
          const h8v bv2 = as_h8(cvt2_hi<0>(eb1), cvt2_hi<0>(ob1), cvt2_hi<1>(eb1), cvt2_hi<1>(ob1));
          const h8v bv3 = as_h8(cvt2_hi<2>(eb1), cvt2_hi<2>(ob1), cvt2_hi<3>(eb1), cvt2_hi<3>(ob1));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv0, bk[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv1, bk[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv2, bk[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv3, bk[3], acc, 0, 0, 0);
          asm volatile("" : "+v"(acc) : "v"(bv0), "v"(bv1), "v"(bv2), "v"(bv3), "v"(bk[0]), "v"(bk[1]),
                       "v"(bk[2]), "v"(bk[3]));
        }
        sc[h2] = acc;
      }
      // r of this lane's tokens 32 kb + 8 g + tau(2 i + parity): dwords 2 (i/2) + parity
      const uint4 rr = kr[kb];
      const uint32_t rd[2] = {rows_lo ? rr.x : rr.y, rows_lo ? rr.z : rr.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = rows_lo ? sc[0][i] : sc[1][i];
        const float S = x + dppf<kQx1>(x);  // hi + lo columns
        const uint32_t rw = rd[i >> 1];
        const float r = (i & 1) ? f16hi(rw) : f16lo(rw);
        lsc[kb][i] = fmaf(S, K1, bq) * r;
      }
    }

    // ---- online softmax (query head c/2 % 4; all 4 rows hold the same head)
    float tmax = lsc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = vmax(tmax, lsc[kb][i]);
    tmax = vmax(tmax, dppf<kRor8>(tmax));
    tmax = rows_max(tmax);
    const float mnew = vmax(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
    float psum = 0.0f, wsum = 0.0f, wmx = 0.0f;
    float pr[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint4 rr = vr[kb];
      const uint32_t rd[2] = {rows_lo ? rr.x : rr.y, rows_lo ? rr.z : rr.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(lsc[kb][i] - mnew);
        const uint32_t rw = rd[i >> 1];
        const float r = (i & 1) ? f16hi(rw) : f16lo(rw);
        psum += p;
        pr[kb][i] = p * r;
        wsum += pr[kb][i];
        wmx = fmaxf(wmx, pr[kb][i]);
      }
    }
    l_run = fmaf(l_run, alpha, psum);  // this lane's blocks; the partner's half joins at the end
    m_run = mnew;
    wsum += dppf<kRor8>(wsum);
    wsum = rows_sum(wsum);
    float sV, invSV;
    pow2_scale(wave_max_pos(wmx), sV, invSV);

    // ---- V: weights (hi or lo part by column parity) against the codes. Each lane packs
    // its own tokens in pairs (i, i+1); the A operand wants (even block, odd block) of the
    // same i, so the pairs are merged with the partner's by byte permutes.
    h8v aw1[NKB], aw2[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      uint32_t d[4];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const float w0 = pr[kb][2 * pp] * sV, w1 = pr[kb][2 * pp + 1] * sV;
        const uint32_t hv = pack_f16(w0, w1);
        const uint32_t mine = pack_f16(sub_f16<0>(w0, hv, partf), sub_f16<1>(w1, hv, partf));
        const uint32_t theirs = (uint32_t)__builtin_amdgcn_mov_dpp((int)mine, kRor8, 0xF, 0xF, true);
        d[2 * pp] = __builtin_amdgcn_perm(theirs, mine, sel_lo);
        d[2 * pp + 1] = __builtin_amdgcn_perm(theirs, mine, sel_hi);
      }
      const h8v wv = as_h8(d[0], d[1], d[2], d[3]);
      const h8v zv = as_h8(0u, 0u, 0u, 0u);
      aw1[kb] = rows_lo ? wv : zv;
      aw2[kb] = rows_lo ? zv : wv;
    }
    f4v cv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t x = vq[i][kb];
        const uint32_t e = x & kNib, od = (x >> 2) & kNib;
        const h8v b1 = as_h8(cvt2<0>(e), cvt2<0>(od), cvt2<1>(e), cvt2<1>(od));
        const h8v b2 = as_h8(cvt2<2>(e), cvt2<2>(od), cvt2<3>(e), cvt2<3>(od));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw1[kb], b1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw2[kb], b2, acc, 0, 0, 0);
        asm volatile("" : "+v"(acc) : "v"(aw1[kb]), "v"(aw2[kb]), "v"(b1), "v"(b2));
        if constexpr (BITS > 2) {
          uint32_t eb, odb;
          if constexpr (BITS == 4) {
            const uint32_t y = vqb[i][kb];
            eb = y & kNib, odb = (y >> 2) & kNib;
          } else {
            const uint32_t y = vqb[i >> 1][kb] >> (2 * (i & 1));
            eb = y & kBit, odb = (y >> 1) & kBit;
          }
          const h8v c1 = as_h8(cvt2_hi<0>(eb), cvt2_hi<0>(odb), cvt2_hi<1>(eb), cvt2_hi<1>(odb));
          const h8v c2 = as_h8(cvt2_hi<2>(eb), cvt2_hi<2>(odb), cvt2_hi<3>(eb), cvt2_hi<3>(odb));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw1[kb], c1, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw2[kb], c2, acc, 0, 0, 0);
          asm volatile("" : "+v"(acc) : "v"(aw1[kb]), "v"(aw2[kb]), "v"(c1), "v"(c2));
        }
      }
      cv[i] = acc;
    }

    // ---- fold: o += (c s) acc + (c z) W for query heads 2 (g%2) + {0, 1}
    const float wb0 = dppf<kNewBcast + 0>(wsum), wb2 = dppf<kNewBcast + 2>(wsum);
    const float wb4 = dppf<kNewBcast + 4>(wsum), wb6 = dppf<kNewBcast + 6>(wsum);
    const float wf[2] = {sh_g1 ? wb4 : wb0, sh_g1 ? wb6 : wb2};
    if (__builtin_amdgcn_ballot_w64(alpha < 1.0f)) {
      const float ab0 = dppf<kNewBcast + 0>(alpha), ab2 = dppf<kNewBcast + 2>(alpha);
      const float ab4 = dppf<kNewBcast + 4>(alpha), ab6 = dppf<kNewBcast + 6>(alpha);
      const float af0 = sh_g1 ? ab4 : ab0, af1 = sh_g1 ? ab6 : ab2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[0][i] *= af0;
        o[1][i] *= af1;
      }
    }
    const float4* vfp = reinterpret_cast<const float4*>(&wl.vf[c][8 * (g >> 1)]);
    const float4 f01 = vfp[0], f23 = vfp[1];
    const float fcs[4] = {f01.x, f01.z, f23.x, f23.z}, fcz[4] = {f01.y, f01.w, f23.y, f23.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float csv = fcs[i] * invSV;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
        o[qq][i] = fmaf(csv, cv[i][2 * qq] + cv[i][2 * qq + 1], fmaf(fcz[i], wf[qq], o[qq][i]));
    }
  }

  // --- merge the 4 waves of the span (fixed order), one partial per query head
  l_run += dppf<kRor8>(l_run);
  l_run = rows_sum(l_run);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) sh.u.oo[wave][2 * (g & 1) + qq][16 * (i + 4 * (g >> 1)) + c] = o[qq][i];
  if (g == 0 && c < 8 && (c & 1) == 0) {
    sh.mm[wave][c >> 1] = m_run;
    sh.ll[wave][c >> 1] = l_run;
  }
  __syncthreads();
  const int qh = threadIdx.x >> 6, j = 2 * lane;
  if (q0 + qh < a.grp) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.mm[w][qh]);
    float Ls = 0.0f, O0 = 0.0f, O1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.mm[w][qh];
      if (mw == -INFINITY) continue;  // a wave without tiles
      const float f = __builtin_amdgcn_exp2f(mw - M);
      Ls = fmaf(f, sh.ll[w][qh], Ls);
      O0 = fmaf(f, sh.u.oo[w][qh][j], O0);
      O1 = fmaf(f, sh.u.oo[w][qh][j + 1], O1);
    }
    float* dst = a.ws + (((long long)b * a.Hq + h * a.grp + q0 + qh) * a.nspan + span) * kPart;
    if (lane == 0) {
      dst[0] = M;
      dst[1] = Ls;
    }
    *reinterpret_cast<float2*>(dst + 4 + j) = make_float2(O0, O1);
  }
}

// Merge: one work-group per (b, q head) row. Its 16 groups of 16 lanes (lane cg holds
// channels 8cg .. 8cg+7) take spans gi, gi+16, ... and tail tokens gi, gi+16, ...; each
// group issues all its loads at once and folds its items into one (m, l, o_rot, o_orig)
// state in log2 units. The 16 states meet in LDS in group order, one thread per output
// channel; group 0 then applies H_D^T to the rotated part and normalizes. Every result
// depends only on the data, not on timing.
struct MergeLds {
  float m[16], l[16];
  float o[16][2 * kD];  // per group: o_rot[D], o_orig[D]
  float fin[2 * kD];
  float lsum;
};

// A state folded with scores that may all be -inf: an empty state keeps weight 1
// (m == mn) and an empty item gets 0.
__device__ __forceinline__ float rescale(float m, float mn) { return m == mn ? 1.0f : __builtin_amdgcn_exp2f(m - mn); }
__device__ __forceinline__ float weight(float x, float mn) {
  return x > -INFINITY ? __builtin_amdgcn_exp2f(x - mn) : 0.0f;
}

// FUSED: work-groups past the rows' ones run the append jobs (one (b, h, s) each, on
// G/32 waves; the other waves exit).
template <bool FUSED, int NW, bool ABL>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const long long nrows = (long long)a.L.B * a.Hq;
  if constexpr (FUSED) {
    if ((long long)blockIdx.x >= nrows) {
      __shared__ TileLds<NW> sh;
      const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      if (wave >= NW) return;
      const AppendArgs ap{a.L, a.cache_rw, a.kn, a.vn};
      append_job<NW, ABL>(ap, (int)(blockIdx.x - nrows), wave, threadIdx.x & 63, sh);
      return;
    }
  }
  __shared__ MergeLds sm;
  const int tid = threadIdx.x, gi = tid >> 4, cg = tid & 15;
  const int rr = (int)blockIdx.x;  // b * Hq + q head
  const int b = rr / a.Hq, qhead = rr - b * a.Hq, h = qhead / a.grp;
  const int G = a.L.G;
  // independent of the length: q and sigma
  const uint4 qw = *reinterpret_cast<const uint4*>(a.q + (long long)rr * kD + 8 * cg);
  float sg[8];
  load_sigma(a.cache, cg, sg);
  // a fused call reads the length the tile pass saw; its append jobs move len meanwhile
  const int n = FUSED ? a.lens_ws[b * a.L.Hkv + h] : *reinterpret_cast<const int32_t*>(a.cache + a.L.len_off(b, h, 0));
  const int nfull = n / G, nt_old = n - nfull * G;
  // the call's own token (fused, unless the sequence is full) follows the tail
  const int nt = nt_old + ((FUSED && n < a.L.cap) ? 1 : 0);
  const int nsp = min(a.nspan, nfull);  // the tile pass's non-empty spans
  const float* w = a.ws + (long long)rr * a.nspan * kPart;

  // tail tokens gi + 16k (k < kt), loaded up front; slots past the tail read the last
  // stored one (finite values) and get -inf scores
  constexpr int KT = 4;  // G <= 64
  const int kt = (nt + 15) / 16;  // uniform over the work-group
  uint4 kw[KT], vw[KT];
  const uint8_t* tk = a.cache + a.L.tail_row(b, h, 0, 0);
  const uint8_t* tv = a.cache + a.L.tail_row(b, h, 1, 0);
  {
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (k >= kt) break;
      const int t = min(gi + 16 * k, nt - 1);
      if (FUSED && t == nt_old) {  // the new token, canonical as the append stores it
        const long long src = ((long long)b * a.L.Hkv + h) * kD + 8 * cg;
        uint32_t seen = 0;  // the append job of this launch raises the token's flags
        kw[k] = canon8(*reinterpret_cast<const uint4*>(a.kn + src), seen);
        vw[k] = canon8(*reinterpret_cast<const uint4*>(a.vn + src), seen);
      } else {
        kw[k] = *reinterpret_cast<const uint4*>(tk + t * 2 * kD + 16 * cg);
        vw[k] = *reinterpret_cast<const uint4*>(tv + t * 2 * kD + 16 * cg);
      }
    }
  }
  // the first span of the group, loaded with the tokens
  float m = -INFINITY, l = 0.0f, orot[8] = {0, 0, 0, 0, 0, 0, 0, 0}, oorig[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = gi; s < nsp; s += 16) {  // uniform over the group
    const float* p = w + s * kPart;
    const float pm = p[0], pl = p[1];
    const float4 x0 = *reinterpret_cast<const float4*>(p + 4 + 8 * cg);
    const float4 x1 = *reinterpret_cast<const float4*>(p + 8 + 8 * cg);
    const float mn = fmaxf(m, pm);
    const float al = rescale(m, mn), be = __builtin_amdgcn_exp2f(pm - mn);
    l = fmaf(l, al, pl * be);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) orot[e] = fmaf(orot[e], al, xs[e] * be);
    m = mn;
  }
  if (nt > 0) {
    float qv[8];
    const uint32_t qq[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qv[2 * k] = bf16lo(qq[k]);
      qv[2 * k + 1] = bf16hi(qq[k]);
    }
    if ((a.flags & KVARN_Q_PREROTATED) && !a.idr) {  // q = q_rot H_D^T
      fwht128(qv, cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] *= kInvSqrtD * sg[e];
    }
    const float qs = kLog2e * a.scale;
    float lt[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      lt[k] = -INFINITY;
      if (k >= kt) continue;
      const uint32_t kk[4] = {kw[k].x, kw[k].y, kw[k].z, kw[k].w};
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) d = fmaf(qv[2 * e], bf16lo(kk[e]), fmaf(qv[2 * e + 1], bf16hi(kk[e]), d));
      d = row16_sum(d);
      lt[k] = gi + 16 * k < nt ? d * qs : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int k = 0; k < KT; ++k) mn = fmaxf(mn, lt[k]);
    const float al = rescale(m, mn);
    l *= al;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      orot[e] *= al;
      oorig[e] *= al;
    }
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (k >= kt) break;
      const float pw = weight(lt[k], mn);
      l += pw;
      const uint32_t vv[4] = {vw[k].x, vw[k].y, vw[k].z, vw[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oorig[2 * e] = fmaf(pw, bf16lo(vv[e]), oorig[2 * e]);
        oorig[2 * e + 1] = fmaf(pw, bf16hi(vv[e]), oorig[2 * e + 1]);
      }
    }
    m = mn;
  }
  // the 16 group states, combined in group order by one thread per output channel
  if (cg == 0) {
    sm.m[gi] = m;
    sm.l[gi] = l;
  }
  store8f(&sm.o[gi][8 * cg], orot);
  store8f(&sm.o[gi][kD + 8 * cg], oorig);
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < 16; ++g) M = fmaxf(M, sm.m[g]);
  float acc = 0.0f, L = 0.0f;
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const float f = weight(sm.m[g], M);
    acc = fmaf(f, sm.o[g][tid], acc);
    L = fmaf(f, sm.l[g], L);
  }
  sm.fin[tid] = acc;
  if (tid == 0) sm.lsum = L;
  __syncthreads();
  if (tid >= 64) return;  // wave 0 finishes; its four groups do the same work, group 0 stores
  float fr[8], fo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fr[e] = sm.fin[8 * cg + e];
    fo[e] = sm.fin[kD + 8 * cg + e];
  }
  if (!a.idr) fwht128(fr, cg);
  const float Ls = sm.lsum;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (fr[e] * (a.idr ? 1.0f : kInvSqrtD * sg[e]) + fo[e]) * inv;
  if (gi == 0) store8f(a.out + (long long)rr * kD + 8 * cg, o);
}

// ----------------------------------------------------------------------------- static workspace
// The span partials of kvarn_attn_decode_noalloc live in a file-scope device array instead
// of a caller's workspace; every GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel (on the host it is only
// a stand-in): the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t attn_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);  // the same value from every caller
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  const long long blocks = (long long)a.L.B * a.L.Hkv * a.nqg * a.nspan;
  if (blocks > 0) {
    const dim3 grid((unsigned)blocks);
    const int which = (a.L.G == 32 ? 0 : 3) + (a.L.bits - 2);
    switch (which) {
      case 0: hipLaunchKernelGGL((attn_kernel<32, 2>), grid, dim3(256), 0, st, a); break;
      case 1: hipLaunchKernelGGL((attn_kernel<32, 3>), grid, dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL((attn_kernel<32, 4>), grid, dim3(256), 0, st, a); break;
      case 3: hipLaunchKernelGGL((attn_kernel<64, 2>), grid, dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((attn_kernel<64, 3>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((attn_kernel<64, 4>), grid, dim3(256), 0, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long row_blocks = (long long)a.L.B * a.Hq;  // one work-group per (b, q head)
  if (!a.kn) {
    hipLaunchKernelGGL((merge_kernel<false, 1, false>), dim3((unsigned)row_blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(row_blocks + 2LL * a.L.B * a.L.Hkv));
  const bool abl = a.L.variant != 0 || a.L.bits != 2;  // the extended build
  if (a.L.G == 32) {
    if (abl)
      hipLaunchKernelGGL((merge_kernel<true, 1, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((merge_kernel<true, 1, false>), grid, dim3(256), 0, st, a);
  } else {
    if (abl)
      hipLaunchKernelGGL((merge_kernel<true, 2, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((merge_kernel<true, 2, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace kvarn
