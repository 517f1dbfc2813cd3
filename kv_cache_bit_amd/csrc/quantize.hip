// KVarN write path on gfx950: the prefill and decode-append kernels and their launchers.
// The device code they share (and its description) is in quantize_dev.h.
#include "quantize_dev.h"

namespace kvarn {

// ----------------------------------------------------------------------------- prefill
// Work-groups [0, tile_blocks) quantize full tiles, TPW tiles (NW waves each) per
// work-group; the remaining work-groups write the bf16 tail and len[], one (b, h, s)
// per wave.
// Work-group `blk` of one layer's prefill, whose cache and inputs are `cache`, `kin`, `vin`
// (the other fields of `a` are shared by every layer of a multi-layer launch).
template <int NW, bool DBG, bool ABL, int TPW>
__device__ __forceinline__ void prefill_block(const PrefillArgs& a, uint8_t* cache, const uint16_t* kin,
                                              const uint16_t* vin, uint32_t blk, TileLds<NW> (&sh_all)[TPW]) {
  constexpr int WPG = NW * TPW;  // waves per work-group
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: job math on the SALU
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = cache;
  uint32_t flags = 0;
  const uint32_t tile_blocks = ((uint32_t)a.jobs + TPW - 1) / TPW;

  if (blk >= tile_blocks) {
    const uint32_t sj = (blk - tile_blocks) * WPG + wave;  // (b, h, s)
    if (sj >= 2u * L.B * L.Hkv) return;
    const uint32_t q = fdiv(sj >> 1, a.dhkv);
    const int s = (int)(sj & 1u), h = (int)((sj >> 1) - q * (uint32_t)L.Hkv), b = (int)q;
    const uint16_t* src = s ? vin : kin;
    for (int t = a.nfull * L.G + g; t < a.T; t += 4) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + (((long long)b * a.T + t) * L.Hkv + h) * kD + 8 * c);
      *reinterpret_cast<uint4*>(cache + L.tail_row(b, h, s, t % L.G) + 16 * c) = canon8(w, flags);
    }
    if (lane == 0) *reinterpret_cast<int32_t*>(cache + L.len_off(b, h, s)) = a.T;
    raise_flags(hdr, flags);
    return;
  }

  const int tw = wave / NW, sub = wave % NW;
  TileLds<NW>& sh = sh_all[tw];
  uint32_t job = blk * TPW + tw;
  const bool valid = job < (uint32_t)a.jobs;
  if (!valid) job = 0;  // keep the barrier sequence uniform; results are discarded
  // job = ((b * nfull + tile) * 2 + s) * Hkv + h : neighbouring waves read neighbouring heads
  const uint32_t q1 = fdiv(job, a.dhkv), q2 = q1 >> 1, q3 = fdiv(q2, a.dnfull);
  const int h = (int)(job - q1 * (uint32_t)L.Hkv);
  const int s = (int)(q1 & 1u);
  const int tile = (int)(q2 - q3 * (uint32_t)a.nfull);
  const int b = (int)q3;
  const uint16_t* src = s ? vin : kin;
  const int t0 = tile * L.G + sub * 32;  // first token of this wave's block
  const bool idr = ABL && (L.variant & KVARN_VARIANT_NO_ROTATION);
  const Frags hf = frags_v<ABL>(idr, lane);

  // A rows are tokens t0 + 16mb + c; K chunk 4ks + g holds channels 8(4ks + g) .. +7
  const uint16_t* rows = src + (((long long)b * a.T + t0 + c) * L.Hkv + h) * kD + 8 * g;
  const long long row16 = 16LL * L.Hkv * kD;  // 16 tokens further
  float p[2][8][4];
  f4v w4[2][8];
  float st;
  b8v av[2][4];
  {
    // the sign masks (header, cached) first: loads complete in issue order
    SigMask m[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) m[ks] = masks_v<ABL>(idr, hdr, 4 * ks + g);
    __builtin_amdgcn_sched_barrier(0);
    uint4 raw[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) raw[mb][ks] = *reinterpret_cast<const uint4*>(rows + mb * row16 + 32 * ks);
    // every input load is issued before any of them is used (one memory round trip per
    // tile), and the first token block is converted and rotated while the second one's
    // loads are still in flight
    __builtin_amdgcn_sched_barrier(0);
    float d[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[mb][ks] = sign8(raw[mb][ks], m[ks]);
      d[mb] = rotate_squares_mb_v<ABL>(idr, av[mb], hf, w4[mb], p[mb], c, sh.xt[sub]);
      __builtin_amdgcn_sched_barrier(0);
    }
    st = gram_own_v<ABL>(idr, d[0], d[1], c);
  }
  // a value beyond 2^16, a NaN, or a token too small for fp32 squares: the checked rotation
  int sx_own = 0;
  if (__any(!rotation_stands(idr, st)))
    st = rotate_checked<ABL>(
        idr,
        [&](int mb, int ks) {
          // a fresh read each time: the compiler must not keep the first pass's registers for it
          const uint16_t* r = rows;
          asm volatile("" : "+v"(r));
          return *reinterpret_cast<const uint4*>(r + mb * row16 + 32 * ks);
        },
        hdr, hf, av, w4, p, g, c, flags, sx_own, sh.xt[sub]);

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
  tile_finish<NW, DBG, ABL>(av, hf, w4, p, st, sx_own, lane, sub, s, L.n_it, L.variant, L.bits, sh, flags, dw, dy,
                            dstride);
  if (valid) {
    const long long ro = record_at(cache, L, b, h, tile, s);
    if (ro >= 0)
      copy_record<NW>(sh, cache + ro, lane, sub, L.tr);
    else
      flags |= KVARN_FLAG_UNMAPPED;
    raise_flags(hdr, flags);
  }
}

template <int NW, bool DBG, bool ABL, int TPW>
__global__ __launch_bounds__(64 * NW * TPW) void prefill_kernel(PrefillArgs a) {
  __shared__ TileLds<NW> sh_all[TPW];
  prefill_block<NW, DBG, ABL, TPW>(a, a.cache, a.k, a.v, blockIdx.x, sh_all);
}

// Several layers of one geometry in one launch: work-groups [l * blocks, (l + 1) * blocks)
// run layer l's prefill. One launch pays the ramp (every wave of the first round waiting
// for its input) and the tail (the last partial round) once for all the layers.
template <int NW, bool ABL, int TPW>
__global__ __launch_bounds__(64 * NW * TPW) void prefill_layers_kernel(PrefillArgs a, PrefillLayers ly) {
  __shared__ TileLds<NW> sh_all[TPW];
  const uint32_t l = fdiv(blockIdx.x, ly.dblocks);
  prefill_block<NW, false, ABL, TPW>(a, ly.cache[l], ly.k[l], ly.v[l], blockIdx.x - l * ly.blocks, sh_all);
}

// ----------------------------------------------------------------------------- append
// One work-group (G/32 waves) per (b, h, s).
template <int NW, bool ABL>
__global__ __launch_bounds__(64 * NW) void append_kernel(AppendArgs a) {
  __shared__ TileLds<NW> sh;
  append_job<NW, ABL>(a, blockIdx.x, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63, sh);
}

// ----------------------------------------------------------------------------- multi-token append
// counts[b] tokens (T when counts is null) go after each sequence's stored ones, as that
// many single-token appends would place them. Tile pass: each group the new tokens
// complete is quantized from its stored tail tokens and the new input rows; job
// (b, j, s, h) takes the j-th such group, one job per work-group, and jobs past the
// sequence's last completed group run on clamped inputs and store nothing (the
// work-group's barriers stay uniform). Tail pass, a second launch so that the tail is read
// before it is overwritten: the new tokens after the last complete group go to the tail
// and len moves on.
__device__ __forceinline__ void tokens_range(const TokensArgs& a, int b, int h, int s, int& l0, int& l1,
                                             bool& dropped) {
  l0 = *reinterpret_cast<const int32_t*>(a.cache + a.L.len_off(b, h, s));
  const int cnt = min(max(a.counts ? a.counts[b] : a.T, 0), a.T);
  l1 = min(l0 + cnt, a.L.cap);
  dropped = l0 + cnt > a.L.cap;
}

template <int NW, bool ABL>
__global__ __launch_bounds__(64 * NW) void tokens_tile_kernel(TokensArgs a) {
  constexpr int G = 32 * NW;
  __shared__ TileLds<NW> sh;
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const Layout& L = a.L;
  uint8_t* hdr = a.cache;
  uint32_t job = blockIdx.x;
  const bool in_grid = job < (uint32_t)a.jobs;
  if (!in_grid) job = 0;  // keep the barrier sequence uniform; results are discarded
  // job = ((b * max_tiles + j) * 2 + s) * Hkv + h: neighbouring work-groups read neighbouring heads
  const uint32_t q1 = fdiv(job, a.dhkv), q2 = q1 >> 1, q3 = fdiv(q2, a.dmt);
  const int h = (int)(job - q1 * (uint32_t)L.Hkv), s = (int)(q1 & 1u);
  const int j = (int)(q2 - q3 * (uint32_t)a.max_tiles), b = (int)q3;
  int l0, l1;
  bool dropped;
  tokens_range(a, b, h, s, l0, l1, dropped);
  const int tile = l0 / G + j;
  const bool valid = in_grid && tile < l1 / G;
  const bool idr = ABL && (L.variant & KVARN_VARIANT_NO_ROTATION);
  const Frags hf = frags_v<ABL>(idr, lane);
  const uint16_t* src = (s ? a.v : a.k) + ((long long)b * a.T * L.Hkv + h) * kD;  // + row * Hkv * D
  uint32_t flags = 0;
  // token 16 mb + c of this wave's block, channels 8 (4 ks + g) .. +7, as given: stored in
  // the tail (canonical already), or a new input row (clamped in range for the rows of a
  // job that stores nothing). As in the prefill, the values go into the rotation as they
  // are, and a token whose sum of squares leaves the range takes the checked rotation,
  // which canonicalizes and raises the flags.
  auto row = [&](int mb, int ks, const uint16_t* sp, const uint8_t* cp) -> uint4 {
    const int tt = tile * G + sub * 32 + 16 * mb + c;  // token of this A row in the sequence
    if (tt < l0) return *reinterpret_cast<const uint4*>(cp + L.tail_row(b, h, s, tt % G) + 16 * (4 * ks + g));
    const int r = min(tt - l0, a.T - 1);
    return *reinterpret_cast<const uint4*>(sp + (long long)r * L.Hkv * kD + 8 * (4 * ks + g));
  };
  b8v av[2][4];
  {
    SigMask m[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) m[ks] = masks_v<ABL>(idr, hdr, 4 * ks + g);
    __builtin_amdgcn_sched_barrier(0);
    uint4 raw[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) raw[mb][ks] = row(mb, ks, src, a.cache);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[mb][ks] = sign8(raw[mb][ks], m[ks]);
  }
  float p[2][8][4];
  f4v w4[2][8];
  float st = rotate_squares_v<ABL>(idr, av, hf, w4, p, c, sh.xt[sub]);
  int sx_own = 0;
  if (__any(!rotation_stands(idr, st)))
    st = rotate_checked<ABL>(
        idr,
        [&](int mb, int ks) {
          // a fresh read each time: the compiler must not keep the first pass's registers for it
          const uint16_t* sp = src;
          const uint8_t* cp = a.cache;
          asm volatile("" : "+v"(sp), "+v"(cp));
          return row(mb, ks, sp, cp);
        },
        hdr, hf, av, w4, p, g, c, flags, sx_own, sh.xt[sub]);
  tile_finish<NW, false, ABL>(av, hf, w4, p, st, sx_own, lane, sub, s, L.n_it, L.variant, L.bits, sh, flags, nullptr,
                              nullptr, 0);
  if (valid) {
    const long long ro = record_at(a.cache, L, b, h, tile, s);
    if (ro >= 0)
      copy_record<NW>(sh, a.cache + ro, lane, sub, L.tr);
    else
      flags |= KVARN_FLAG_UNMAPPED;
    raise_flags(hdr, flags);
  }
}

// One wave per (b, h, s): 4 tokens per step, 16 lanes x 8 channels each.
__global__ __launch_bounds__(256) void tokens_tail_kernel(TokensArgs a) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const Layout& L = a.L;
  const long long sj = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sj >= 2LL * L.B * L.Hkv) return;
  const int s = (int)(sj % 2), h = (int)((sj / 2) % L.Hkv), b = (int)(sj / 2 / L.Hkv);
  int l0, l1;
  bool dropped;
  tokens_range(a, b, h, s, l0, l1, dropped);
  uint32_t flags = dropped ? (uint32_t)KVARN_FLAG_CAPACITY : 0u;
  const uint16_t* src = (s ? a.v : a.k) + ((long long)b * a.T * L.Hkv + h) * kD;
  for (int t = max(l0, l1 / L.G * L.G) + g; t < l1; t += 4)
    *reinterpret_cast<uint4*>(a.cache + L.tail_row(b, h, s, t % L.G) + 16 * c) =
        canon8(*reinterpret_cast<const uint4*>(src + (long long)(t - l0) * L.Hkv * kD + 8 * c), flags);
  raise_flags(a.cache, flags);
  if (lane == 0) *reinterpret_cast<int32_t*>(a.cache + L.len_off(b, h, s)) = l1;  // the wave read len first
}

// ----------------------------------------------------------------------------- launchers
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  // One tile per work-group: a tile's waves finish on their own schedule, and a slot freed
  // by one wave (G = 32) can take the next tile at once instead of waiting for three others.
  constexpr int TPW = 1;
  const int nw = a.L.G / 32;
  const long long tile_blocks = (a.jobs + TPW - 1) / TPW;
  const long long tail_blocks = (2LL * a.L.B * a.L.Hkv + nw * TPW - 1) / (nw * TPW);
  const dim3 grid((unsigned)(tile_blocks + tail_blocks)), block((unsigned)(64 * nw * TPW));
  const bool dbg = a.wk || a.wv || a.yk || a.yv;
  const bool abl = a.L.variant != 0 || a.L.bits != 2;  // the extended build
  const int which = (a.L.G == 32 ? 0 : 4) + (dbg ? 2 : 0) + (abl ? 1 : 0);
  switch (which) {
    case 0: hipLaunchKernelGGL((prefill_kernel<1, false, false, TPW>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((prefill_kernel<1, false, true, TPW>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<1, true, false, TPW>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<1, true, true, TPW>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<2, false, false, TPW>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((prefill_kernel<2, false, true, TPW>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((prefill_kernel<2, true, false, TPW>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((prefill_kernel<2, true, true, TPW>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

// ly.cache/k/v hold n_layers entries; blocks and dblocks are filled in here.
hipError_t launch_prefill_layers(const PrefillArgs& a, PrefillLayers& ly, int n_layers, hipStream_t st) {
  constexpr int TPW = 1;
  const int nw = a.L.G / 32;
  const long long tile_blocks = (a.jobs + TPW - 1) / TPW;
  const long long tail_blocks = (2LL * a.L.B * a.L.Hkv + nw * TPW - 1) / (nw * TPW);
  ly.blocks = (uint32_t)(tile_blocks + tail_blocks);
  ly.dblocks = make_fastdiv(ly.blocks);
  const dim3 grid((unsigned)((long long)n_layers * ly.blocks)), block((unsigned)(64 * nw * TPW));
  const bool abl = a.L.variant != 0 || a.L.bits != 2;  // the extended build
  const int which = (a.L.G == 32 ? 0 : 2) + (abl ? 1 : 0);
  switch (which) {
    case 0: hipLaunchKernelGGL((prefill_layers_kernel<1, false, TPW>), grid, block, 0, st, a, ly); break;
    case 1: hipLaunchKernelGGL((prefill_layers_kernel<1, true, TPW>), grid, block, 0, st, a, ly); break;
    case 2: hipLaunchKernelGGL((prefill_layers_kernel<2, false, TPW>), grid, block, 0, st, a, ly); break;
    default: hipLaunchKernelGGL((prefill_layers_kernel<2, true, TPW>), grid, block, 0, st, a, ly); break;
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(2LL * a.L.B * a.L.Hkv));
  const bool abl = a.L.variant != 0 || a.L.bits != 2;  // the extended build
  if (a.L.G == 32) {
    if (abl)
      hipLaunchKernelGGL((append_kernel<1, true>), grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((append_kernel<1, false>), grid, dim3(64), 0, st, a);
  } else {
    if (abl)
      hipLaunchKernelGGL((append_kernel<2, true>), grid, dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL((append_kernel<2, false>), grid, dim3(128), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_tokens(const TokensArgs& a, hipStream_t st) {
  if (a.jobs > 0) {
    // one tile job per work-group of G/32 waves, as in the prefill
    const dim3 grid((unsigned)a.jobs);
    const bool abl = a.L.variant != 0 || a.L.bits != 2;  // the extended build
    if (a.L.G == 32) {
      if (abl)
        hipLaunchKernelGGL((tokens_tile_kernel<1, true>), grid, dim3(64), 0, st, a);
      else
        hipLaunchKernelGGL((tokens_tile_kernel<1, false>), grid, dim3(64), 0, st, a);
    } else {
      if (abl)
        hipLaunchKernelGGL((tokens_tile_kernel<2, true>), grid, dim3(128), 0, st, a);
      else
        hipLaunchKernelGGL((tokens_tile_kernel<2, false>), grid, dim3(128), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long streams = 2LL * a.L.B * a.L.Hkv;
  hipLaunchKernelGGL(tokens_tail_kernel, dim3((unsigned)((streams + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
