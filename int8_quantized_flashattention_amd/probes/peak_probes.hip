// Measurement kernels for the benchmark's second denominators: the rate the
// INT8 matrix cores reach in a loop of independent products, and the rate a
// plain streaming read reaches from HBM. Not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_probes.h"
#include "cdna4_ops.h"

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

// The LDS access patterns of one prefill tile (d = 128, 64 keys), issued in
// a loop over a resident K/V stage so that their LDS counters can be read
// apart: MODE 0 the K operand reads (16 bytes per lane from swizzled rows),
// 1 the transposing V operand reads (ds_read_b64_tr_b8), 2 the per-key scale
// reads (16 bytes, all lanes of a half-wave on one address), 3 the
// LDS-destination buffer loads that fill a stage. The addresses repeat the
// prefill kernel's formulas.
constexpr int kD = 128, kBN = 64;
__device__ __forceinline__ int probe_key_of_row(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

template <int MODE>
__global__ __launch_bounds__(256) void lds_patterns(const int8_t* src, int iters, uint32_t* out) {
  __shared__ alignas(16) int8_t stage[2 * kBN * kD + 2 * kBN * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < (2 * kBN * kD + 2 * kBN * 4) / 4; i += 256)
    reinterpret_cast<uint32_t*>(stage)[i] = static_cast<uint32_t>(i * 2654435761u);
  __syncthreads();
  const int lr = lane & 31, g = lane >> 5;
  const int kr = probe_key_of_row(lr);
  int koff[4], voff[4];
  const int q = lane >> 4, i16 = lane & 15;
  const int vr = 16 * (q >> 1) + (i16 >> 1);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    koff[c] = kr * kD + (((2 * c + g) ^ attn::swz<kD>(kr)) * 16);
    voff[c] = vr * kD + (((2 * c + (q & 1)) ^ attn::swz<kD>(vr)) * 16) + 8 * (i16 & 1);
  }
  const int8_t* kst = stage;
  const int8_t* vst = stage + kBN * kD;
  const float* sk = reinterpret_cast<const float*>(stage + 2 * kBN * kD);
  const __amdgpu_buffer_rsrc_t rs = attn::make_rsrc(src, kBN * kD);
  uint32_t x = 0;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4i v = *reinterpret_cast<const v4i*>(kst + kb * 32 * kD + koff[c]);
          x ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    } else if constexpr (MODE == 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const attn::v2i lo = attn::lds_read_tr8(vst + kb * 32 * kD + voff[c]);
          const attn::v2i hi = attn::lds_read_tr8(vst + kb * 32 * kD + voff[c] + 8 * kD);
          x ^= lo.x ^ lo.y ^ hi.x ^ hi.y;
        }
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const float4 f = *reinterpret_cast<const float4*>(sk + kb * 32 + g * 16 + j4 * 4);
          x ^= __float_as_uint(f.x) ^ __float_as_uint(f.y) ^ __float_as_uint(f.z) ^ __float_as_uint(f.w);
        }
    } else {
      // two 1 KB loads per wavefront into each of the K and V halves, as one
      // stage request of the prefill kernel
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = wave * 2 + i;
        attn::lds_load16(rs, stage + n * 1024, attn::tile_load_off<kD>(n, lane), 0);
        attn::lds_load16(rs, stage + kBN * kD + n * 1024, attn::tile_load_off<kD>(n, lane), 0);
      }
      attn::wait_vm_lds<0>();
      attn::bare_barrier();
      x ^= reinterpret_cast<const uint32_t*>(stage)[tid];
      attn::bare_barrier();
    }
    asm volatile("" : "+v"(x));
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + tid] = x;
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

int attn_probe_lds_patterns(int32_t mode, const void* src, int32_t n_blocks, int32_t iters, uint32_t* out,
                            void* stream) {
  if (mode < 0 || mode > 3 || !src || !out || n_blocks < 1 || iters < 1 ||
      (reinterpret_cast<uintptr_t>(src) & 15))
    return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int8_t* s8 = static_cast<const int8_t*>(src);
  switch (mode) {
    case 0: hipLaunchKernelGGL(lds_patterns<0>, dim3(n_blocks), dim3(256), 0, st, s8, iters, out); break;
    case 1: hipLaunchKernelGGL(lds_patterns<1>, dim3(n_blocks), dim3(256), 0, st, s8, iters, out); break;
    case 2: hipLaunchKernelGGL(lds_patterns<2>, dim3(n_blocks), dim3(256), 0, st, s8, iters, out); break;
    default: hipLaunchKernelGGL(lds_patterns<3>, dim3(n_blocks), dim3(256), 0, st, s8, iters, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
