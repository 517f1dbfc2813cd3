// KVarN read path on gfx950: single-query decode attention over the 2-bit cache.
//
// The query takes the same randomized Hadamard rotation as the keys, so scores are
// computed in rotated space without rotating the cache back (ai-paper-analysis page,
// section 3.1: H H^T = I leaves Q K^T unchanged). Dequantization is folded into the
// dot products: for a K tile with scales r (token), c, s, z (channel),
//   score_t = scale * r_t * (sum_j a_j q_tj + b),  a_j = q_rot,j c_j s_j,  b = sum_j q_rot,j c_j z_j,
// and for a V tile with weights w_t = p_t r_t,
//   o_rot,j += c_j (s_j sum_t w_t q_tj + z_j sum_t w_t).
// Tail tokens (fp16, unrotated) are scored and accumulated in original space. Each
// work-group handles one (batch, kv head, split) with an online softmax; a merge
// kernel combines the splits in a fixed order (log-sum-exp), rotates the V
// accumulator back by H_D^T, adds the tail part and normalizes.
#include "kvarn_common.h"
#include "kvarn_launch.h"

namespace kvarn {

constexpr int kWs = 2 + 2 * kD;  // floats per (b, q head, split): m, l, o_rot[D], o_orig[D]

template <int GM>
struct AttnLds {
  float qrot[GM][kD];
  float qorig[GM][kD];
  float av[GM][kD];   // a_j of the current K tile
  float bpart[2][GM];
  float sc[GM][64];   // scores of the current tile
  float wts[GM][64];  // softmax weights times the V token scale
  float alpha[GM], sumw[GM];
};

template <int GM>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  __shared__ AttnLds<GM> sh;
  const Layout& L = a.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = L.G, grp = a.grp;
  const int split = blockIdx.x % a.n_split;
  const int bh = blockIdx.x / a.n_split;
  const int h = bh % L.Hkv, b = bh / L.Hkv;
  const int n = *reinterpret_cast<const int32_t*>(a.cache + L.len_off(b, h, 0));
  const int nfull = n / G, ntail = n % G;
  const int lo = split * a.tiles_per_split;
  const int hi = min(lo + a.tiles_per_split, nfull);
  const bool do_tail = ntail > 0 && nfull >= lo && nfull < lo + a.tiles_per_split;

  // --- query: rotate into the cache basis (or back, when it arrives rotated)
  if (wave < 2) {
    const int rg = lane >> 4, cg = lane & 15;
    const int gi = wave * 4 + rg;
    float sg[8];
    load_sigma(a.cache, cg, sg);
    float qv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (gi < grp) {
      const uint4 w = *reinterpret_cast<const uint4*>(a.q + ((long long)b * a.Hq + h * grp + gi) * kD + 8 * cg);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      for (int k = 0; k < 4; ++k) {
        qv[2 * k] = bf16lo(ws[k]);
        qv[2 * k + 1] = bf16hi(ws[k]);
      }
    }
    float t[8];
    const bool pre = a.flags & KVARN_Q_PREROTATED;
    for (int e = 0; e < 8; ++e) t[e] = pre ? qv[e] : qv[e] * sg[e];
    fwht128(t, cg);
    for (int e = 0; e < 8; ++e) t[e] *= kInvSqrtD;
    if (pre)
      for (int e = 0; e < 8; ++e) t[e] *= sg[e];  // q = q_rot H_D^T
    if (gi < GM) {
      for (int e = 0; e < 8; ++e) {
        sh.qrot[gi][8 * cg + e] = pre ? qv[e] : t[e];
        sh.qorig[gi][8 * cg + e] = pre ? t[e] : qv[e];
      }
    }
  }
  __syncthreads();

  float m[GM], l[GM], orot[GM], oorig[GM];  // o*: channel j = tid >> 1 (lanes with tid even)
  for (int gi = 0; gi < GM; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.0f;
    orot[gi] = oorig[gi] = 0.0f;
  }
  const float scale = a.scale;
  const int ro = G * kD / 4, co = ro + 2 * G, so = co + 2 * kD, zo = so + 2 * kD;

  for (int tile = lo; tile < hi; ++tile) {
    const uint8_t* rk = a.cache + L.record(b, h, tile, 0);
    const uint8_t* rvp = rk + L.tr;
    // A: per-channel query factors of this K tile
    if (tid < kD) {
      const int j = tid;
      const float c = (float)*reinterpret_cast<const _Float16*>(rk + co + 2 * j);
      const float s = (float)*reinterpret_cast<const _Float16*>(rk + so + 2 * j);
      const float z = (float)*reinterpret_cast<const _Float16*>(rk + zo + 2 * j);
      for (int gi = 0; gi < grp; ++gi) {
        const float qc = sh.qrot[gi][j] * c;
        sh.av[gi][j] = qc * s;
        float bz = qc * z;
        for (int o = 32; o >= 1; o >>= 1) bz += __shfl_xor(bz, o);
        if (lane == 0) sh.bpart[wave][gi] = bz;
      }
    }
    __syncthreads();
    // B: scores; thread = (token, code word `part`: channels 16m + 2 part + d in slot 8d + m)
    {
      const int part = tid & 7;
      for (int tok = tid >> 3; tok < G; tok += 32) {
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(rk + tok * 32 + 4 * part);
        float d[GM];
        for (int gi = 0; gi < GM; ++gi) d[gi] = 0.0f;
        for (int k = 0; k < 16; ++k) {
          const float qq = (float)((cw >> (2 * k)) & 3u);
          const int j = 16 * (k & 7) + 2 * part + (k >> 3);
          for (int gi = 0; gi < grp; ++gi) d[gi] = fmaf(sh.av[gi][j], qq, d[gi]);
        }
        const float rt = (float)*reinterpret_cast<const _Float16*>(rk + ro + 2 * tok);
        for (int gi = 0; gi < grp; ++gi) {
          float v = d[gi];
          v += xshfl<1>(v);
          v += xshfl<2>(v);
          v += xshfl<4>(v);
          if (part == 0) sh.sc[gi][tok] = scale * rt * (v + (sh.bpart[0][gi] + sh.bpart[1][gi]));
        }
      }
    }
    __syncthreads();
    // C: online softmax (wave 0); V token scales folded into the weights
    if (wave == 0) {
      float rvv = 0.0f;
      if (lane < G) rvv = (float)*reinterpret_cast<const _Float16*>(rvp + ro + 2 * lane);
      for (int gi = 0; gi < grp; ++gi) {
        const float x = lane < G ? sh.sc[gi][lane] : -INFINITY;
        float mt = x;
        for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
        const float mn = fmaxf(m[gi], mt);
        const float al = __expf(m[gi] - mn);
        const float p = lane < G ? __expf(x - mn) : 0.0f;
        const float w = p * rvv;
        float ps = p, ws = w;
        for (int o = 32; o >= 1; o >>= 1) {
          ps += __shfl_xor(ps, o);
          ws += __shfl_xor(ws, o);
        }
        sh.wts[gi][lane] = w;
        l[gi] = l[gi] * al + ps;
        m[gi] = mn;
        if (lane == 0) {
          sh.alpha[gi] = al;
          sh.sumw[gi] = ws;
        }
      }
    }
    __syncthreads();
    // D: V accumulation; thread = (channel j, half of the tokens)
    {
      const int j = tid >> 1, half = tid & 1;
      const int nb = G / 4;  // bytes per channel
      float acc[GM];
      for (int gi = 0; gi < GM; ++gi) acc[gi] = 0.0f;
      for (int wq = 0; wq < nb / 8; ++wq) {  // 16 tokens per dword
        const int dw = half * (nb / 8) + wq;
        const uint32_t cw = *reinterpret_cast<const uint32_t*>(rvp + j * nb + 4 * dw);
        for (int k = 0; k < 16; ++k) {
          const float qq = (float)((cw >> (2 * k)) & 3u);
          for (int gi = 0; gi < grp; ++gi) acc[gi] = fmaf(sh.wts[gi][16 * dw + k], qq, acc[gi]);
        }
      }
      for (int gi = 0; gi < grp; ++gi) acc[gi] += xshfl<1>(acc[gi]);
      if (half == 0) {
        const float c = (float)*reinterpret_cast<const _Float16*>(rvp + co + 2 * j);
        const float s = (float)*reinterpret_cast<const _Float16*>(rvp + so + 2 * j);
        const float z = (float)*reinterpret_cast<const _Float16*>(rvp + zo + 2 * j);
        for (int gi = 0; gi < grp; ++gi)
          orot[gi] = orot[gi] * sh.alpha[gi] + c * fmaf(s, acc[gi], z * sh.sumw[gi]);
      }
    }
    __syncthreads();
  }

  if (do_tail) {
    const uint8_t* tk = a.cache + L.tail_row(b, h, 0, 0);
    const uint8_t* tv = a.cache + L.tail_row(b, h, 1, 0);
    {
      const int part = tid & 7;
      for (int tok = tid >> 3; tok < G; tok += 32) {
        float d[GM];
        for (int gi = 0; gi < GM; ++gi) d[gi] = 0.0f;
        if (tok < ntail) {
          const uint4* kp = reinterpret_cast<const uint4*>(tk + tok * 2 * kD + 32 * part);
          float kv[16];
          const uint4 w0 = kp[0], w1 = kp[1];
          const uint32_t ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          for (int k = 0; k < 8; ++k) {
            kv[2 * k] = f16lo(ws[k]);
            kv[2 * k + 1] = f16hi(ws[k]);
          }
          for (int k = 0; k < 16; ++k)
            for (int gi = 0; gi < grp; ++gi) d[gi] = fmaf(sh.qorig[gi][16 * part + k], kv[k], d[gi]);
        }
        for (int gi = 0; gi < grp; ++gi) {
          float v = d[gi];
          v += xshfl<1>(v);
          v += xshfl<2>(v);
          v += xshfl<4>(v);
          if (part == 0) sh.sc[gi][tok] = scale * v;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      for (int gi = 0; gi < grp; ++gi) {
        const float x = lane < ntail ? sh.sc[gi][lane] : -INFINITY;
        float mt = x;
        for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
        const float mn = fmaxf(m[gi], mt);
        const float al = __expf(m[gi] - mn);
        const float p = lane < ntail ? __expf(x - mn) : 0.0f;
        float ps = p;
        for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
        sh.wts[gi][lane] = p;
        l[gi] = l[gi] * al + ps;
        m[gi] = mn;
        if (lane == 0) sh.alpha[gi] = al;
      }
    }
    __syncthreads();
    {
      const int j = tid >> 1, half = tid & 1;
      float acc[GM];
      for (int gi = 0; gi < GM; ++gi) acc[gi] = 0.0f;
      for (int tok = half; tok < ntail; tok += 2) {
        const float vv = (float)*reinterpret_cast<const _Float16*>(tv + tok * 2 * kD + 2 * j);
        for (int gi = 0; gi < grp; ++gi) acc[gi] = fmaf(sh.wts[gi][tok], vv, acc[gi]);
      }
      for (int gi = 0; gi < grp; ++gi) acc[gi] += xshfl<1>(acc[gi]);
      if (half == 0) {
        for (int gi = 0; gi < grp; ++gi) {
          orot[gi] *= sh.alpha[gi];
          oorig[gi] = oorig[gi] * sh.alpha[gi] + acc[gi];
        }
      }
    }
  }

  // partials: m and l live in wave 0, o_rot / o_orig in the even threads
  for (int gi = 0; gi < grp; ++gi) {
    float* w = a.ws + (((long long)b * a.Hq + h * grp + gi) * a.n_split + split) * kWs;
    if (tid == 0) {
      w[0] = m[gi];
      w[1] = l[gi];
    }
    if ((tid & 1) == 0) {
      w[2 + (tid >> 1)] = orot[gi];
      w[2 + kD + (tid >> 1)] = oorig[gi];
    }
  }
}

// One 16-lane row per (b, q head): combine splits in index order, un-rotate, normalize.
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63, rg = lane >> 4, cg = lane & 15;
  const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + rg;  // b * Hq + g
  const long long nrows = (long long)a.L.B * a.Hq;
  const bool live = row < nrows;
  const long long rr = live ? row : 0;
  const float* w = a.ws + rr * a.n_split * kWs;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, w[s * kWs]);
  float Lsum = 0.0f, orot[8] = {0, 0, 0, 0, 0, 0, 0, 0}, oorig[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = 0; s < a.n_split; ++s) {
    const float* p = w + s * kWs;
    if (!(p[1] > 0.0f)) continue;
    const float f = __expf(p[0] - M);
    Lsum += f * p[1];
    for (int e = 0; e < 8; ++e) {
      orot[e] = fmaf(f, p[2 + 8 * cg + e], orot[e]);
      oorig[e] = fmaf(f, p[2 + kD + 8 * cg + e], oorig[e]);
    }
  }
  float sg[8];
  load_sigma(a.cache, cg, sg);
  fwht128(orot, cg);  // all 16 lanes of the row take part, live or not
  if (!live) return;
  float o[8];
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  for (int e = 0; e < 8; ++e) o[e] = (orot[e] * kInvSqrtD * sg[e] + oorig[e]) * inv;
  store8f(a.out + rr * kD + 8 * cg, o);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((long long)a.L.B * a.L.Hkv * a.n_split));
  if (a.grp <= 1)
    hipLaunchKernelGGL(attn_kernel<1>, grid, dim3(256), 0, st, a);
  else if (a.grp <= 2)
    hipLaunchKernelGGL(attn_kernel<2>, grid, dim3(256), 0, st, a);
  else if (a.grp <= 4)
    hipLaunchKernelGGL(attn_kernel<4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_kernel<8>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.L.B * a.Hq;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
