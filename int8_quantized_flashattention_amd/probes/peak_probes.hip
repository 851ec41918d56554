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

// Each workgroup streams one contiguous slice of n16 16-byte words (a
// multiple of 1024 words per slice; the tail slice may be shorter): every lane
// keeps four 16-byte loads in flight, 16 KB per workgroup per round, and folds
// the words into one value per thread. NT: non-temporal loads.
template <bool NT>
__global__ __launch_bounds__(256) void hbm_read(const v4u* src, int64_t n16, int64_t per_block, uint32_t* out) {
  const int64_t beg = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t end = beg + per_block < n16 ? beg + per_block : n16;
  uint32_t x = 0;
  int64_t i = beg + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    v4u w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = NT ? __builtin_nontemporal_load(src + i + u * 256) : src[i + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < end; i += 256) {
    const v4u w = NT ? __builtin_nontemporal_load(src + i) : src[i];
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

int attn_probe_hbm_read(const void* src, int64_t n_bytes, int32_t n_blocks, int32_t nontemporal, uint32_t* out,
                        void* stream) {
  if (!src || !out || n_blocks < 1 || n_bytes < 16 || (n_bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return 1;
  const int64_t n16 = n_bytes / 16;
  const int64_t per_block = (n16 + n_blocks - 1) / n_blocks;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(hbm_read<true>, dim3(n_blocks), dim3(256), 0, st, static_cast<const v4u*>(src), n16, per_block,
                       out);
  else
    hipLaunchKernelGGL(hbm_read<false>, dim3(n_blocks), dim3(256), 0, st, static_cast<const v4u*>(src), n16, per_block,
                       out);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
