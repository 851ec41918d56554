// Measurement kernels for the benchmark's second denominators: the rate the
// INT8 matrix cores reach in a loop of independent products, and the rate a
// plain streaming read reaches from HBM. Not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probes.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulators per wavefront

// Every wavefront issues `iters` rounds of kChains independent
// v_mfma_i32_32x32x32_i8 (32 x 32 x 32 MACs each) and stores its
// accumulators, so none of the products is dead code.
__global__ __launch_bounds__(256) void mfma_i8_loop(int iters, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const v4i a = v4i{lane, lane + 1, lane + 2, lane + 3};
  const v4i b = v4i{3 - lane, 1, lane ^ 5, 7};
  v16i acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = c + i;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  }
  int32_t* o = out + (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int32_t s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][i];
    o[i] = s;
  }
}

// Grid-stride read of n16 16-byte words (four loads in flight per lane),
// folded into one word per thread.
__global__ __launch_bounds__(256) void hbm_read(const v4u* src, int64_t n16, uint32_t* out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u w0 = __builtin_nontemporal_load(src + i);
    const v4u w1 = __builtin_nontemporal_load(src + i + stride);
    const v4u w2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u w3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= w0.x ^ w0.y ^ w0.z ^ w0.w ^ w1.x ^ w1.y ^ w1.z ^ w1.w;
    x ^= w2.x ^ w2.y ^ w2.z ^ w2.w ^ w3.x ^ w3.y ^ w3.z ^ w3.w;
  }
  for (; i < n16; i += stride) {
    const v4u w = __builtin_nontemporal_load(src + i);
    x ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = x;
}

}  // namespace

extern "C" {

int attn_probe_mfma_i8(int32_t n_blocks, int32_t iters, int32_t* out, void* stream) {
  if (n_blocks < 1 || iters < 1 || !out) return 1;
  hipLaunchKernelGGL(mfma_i8_loop, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int attn_probe_hbm_read(const void* src, int64_t n_bytes, int32_t n_blocks, uint32_t* out, void* stream) {
  if (!src || !out || n_blocks < 1 || n_bytes < 16 || (n_bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return 1;
  hipLaunchKernelGGL(hbm_read, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4u*>(src), n_bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
