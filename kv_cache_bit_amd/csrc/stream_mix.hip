// A measurement kernel for the benchmark, not part of the libkvarn boundary: it streams
// `in_bytes` of reads and `out_bytes` of writes through HBM in one launch, with no other
// work, so the benchmark can quote the practical ceiling of a kernel with the same mix of
// reads and writes as the prefill quantizer (about 81.5% read, 18.5% written) or the bf16
// dequantizer (about 15% read, 85% written).
//
// Reads at least the writes: output word o (16 B) is the XOR of input words o, o + n_out,
// o + 2 n_out, ... Fewer reads: output word o is input word o / k where k divides o (k the
// rounded-up ratio), and its own index elsewhere. Consecutive lanes read and write
// consecutive 16-byte words, and every input byte is read once. The stores are plain or,
// in the second variant, marked non-temporal (the library's dequantizer writes its
// output that way); the ceiling is the faster of the two.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void put(uint4* p, uint4 v) {
  if constexpr (NT) {
    const u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_mix_kernel(const uint4* __restrict__ in, long long n_in,
                                                           uint4* __restrict__ out, long long n_out) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  if (n_in < n_out) {
    const long long k = (n_out + n_in - 1) / n_in;
    for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < n_out; o += stride) {
      uint4 v = make_uint4((uint32_t)o, 0u, 0u, 0u);
      if (o % k == 0 && o / k < n_in) v = in[o / k];
      put<NT>(out + o, v);
    }
    return;
  }
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < n_out; o += stride) {
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (long long i = o; i < n_in; i += n_out) {
      const uint4 v = in[i];
      acc.x ^= v.x;
      acc.y ^= v.y;
      acc.z ^= v.z;
      acc.w ^= v.w;
    }
    put<NT>(out + o, acc);
  }
}

}  // namespace

static int launch_mix(bool nt, const void* in, size_t in_bytes, void* out, size_t out_bytes, int grid,
                      void* stream) {
  if (!in || !out || out_bytes < 16 || in_bytes < 16 || (in_bytes | out_bytes) & 15 || grid <= 0) return 1;
  if (((uintptr_t)in | (uintptr_t)out) & 15) return 2;
  auto kern = nt ? stream_mix_kernel<true> : stream_mix_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(in), (long long)(in_bytes / 16), static_cast<uint4*>(out),
                     (long long)(out_bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" __attribute__((visibility("default"))) int kvarn_bench_stream_mix(const void* in, size_t in_bytes,
                                                                           void* out, size_t out_bytes,
                                                                           int grid, void* stream) {
  return launch_mix(false, in, in_bytes, out, out_bytes, grid, stream);
}

// The same with non-temporal stores.
extern "C" __attribute__((visibility("default"))) int kvarn_bench_stream_mix_nt(const void* in, size_t in_bytes,
                                                                              void* out, size_t out_bytes,
                                                                              int grid, void* stream) {
  return launch_mix(true, in, in_bytes, out, out_bytes, grid, stream);
}
