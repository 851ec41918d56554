// Symmetric INT8 quantization of row groups for gfx950.
//
// Operation ("IntAttention: A Fully Integer Attention Pipeline for Efficient
// Edge Inference", §2.1 Eq. 3, zero point 0; one scale per token as in the
// "INT-FlashAttention" abstract, or one per larger group of rows):
//   a = max |x| over the group; a == 0 -> s = 0, q = 0;
//   else s = a / 127, r = 127 / a (correctly rounded fp32 divisions) and
//   q = clamp(rne(x * r), -127, 127) with x * r one rounded fp32 multiply.
//
// The pass is HBM-bound (2 or 4 bytes in, 1 byte out per element), so the
// design is about streaming: every lane moves one 16-byte (fp16) or 32-byte
// (fp32) chunk of 8 elements per load, a group small enough for one wavefront
// (per-token rows) is reduced with cross-lane max inside the wavefront and
// quantized from registers in the same pass, and large groups (per-tensor or
// per-head scales) take two passes: an order-free maximum through atomicMax on
// the bit pattern of |x| (non-negative floats order like their bits), then the
// quantizing pass, whose re-read mostly hits the 256 MB last-level cache.
#include "attn_internal.h"
#include "cdna4_ops.h"

#include <hip/hip_fp16.h>

#include <algorithm>

namespace attn {
namespace {

constexpr int kChunk = 8;          // elements per lane per load
constexpr int kThreads = 256;
constexpr int kUnroll = 4;         // loads in flight per lane in the large-group quantize pass
constexpr int kUnrollMax = 8;      // loads in flight per lane in the large-group absmax pass
// blocks per group of the absmax pass at most: each ends with one atomicMax
// on the group's slot, and same-address atomics serialize in L2
constexpr int kMaxAbsmaxBlocks = 256;    // measured: 128 and 512+ are slower

struct Chunk8 { float x[kChunk]; };

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// The input is read once per pass: non-temporal loads stream it past the
// caches (measured 3 % faster for the K and V passes than cached loads; in
// the attention step, cached loads made the per-tensor V maximum 29 % slower).
template <bool F16>
__device__ __forceinline__ Chunk8 load_chunk(const void* base, int64_t elem) {
  Chunk8 c;
  if constexpr (F16) {
    const v4u raw = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(static_cast<const __half*>(base) + elem));
    const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 f = __half22float2(h[i]);
      c.x[2 * i] = f.x;
      c.x[2 * i + 1] = f.y;
    }
  } else {
    const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(base) + elem);
    const v4f a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
    c.x[0] = a.x; c.x[1] = a.y; c.x[2] = a.z; c.x[3] = a.w;
    c.x[4] = b.x; c.x[5] = b.y; c.x[6] = b.z; c.x[7] = b.w;
  }
  return c;
}

__device__ __forceinline__ float chunk_absmax(const Chunk8& c) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) m = fmaxf(m, fabsf(c.x[i]));
  return m;
}

__device__ __forceinline__ void store_codes(int8_t* q, int64_t elem, const Chunk8& c, float r, bool zero) {
  uint32_t w0 = 0, w1 = 0;
  if (!zero) {
    w0 = quant_word(&c.x[0], r);
    w1 = quant_word(&c.x[4], r);
  }
  *reinterpret_cast<uint2*>(q + elem) = make_uint2(w0, w1);
}

// ---------------------------------------------------------------------------
// Small groups: a team of T lanes (a power of two <= 64) owns G consecutive
// groups; each lane holds up to CH chunks of each in registers. All loads of
// the G groups are issued before the first reduction, so a lane keeps
// G * CH chunks in flight.
// ---------------------------------------------------------------------------
// Where group g of the input goes (MAP): output group (g / seg_in) * seg_out +
// off + g % seg_in, e.g. new tokens into their rows of a cache.
struct RowMap {
  int64_t seg_in, seg_out, off;
};

template <bool F16, int T, int CH, int G, bool MAP>
__global__ __launch_bounds__(kThreads) void quantize_small_groups(
    const void* __restrict__ x, int64_t n_groups, int64_t group_elems, int8_t* __restrict__ q,
    float* __restrict__ scales, RowMap map) {
  constexpr int kTeams = kThreads / T;
  const int team = threadIdx.x / T;
  const int tl = threadIdx.x % T;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * kTeams + team) * G;
  const int n_chunks = static_cast<int>(group_elems / kChunk);

  Chunk8 c[G][CH];
  float a[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    a[j] = 0.0f;
    const int64_t base = (g0 + j) * group_elems;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ci = tl + i * T;
      if (g0 + j < n_groups && ci < n_chunks) c[j][i] = load_chunk<F16>(x, base + static_cast<int64_t>(ci) * kChunk);
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ci = tl + i * T;
      if (g0 + j < n_groups && ci < n_chunks) a[j] = fmaxf(a[j], chunk_absmax(c[j][i]));
    }
    // team-wide maximum (exact: max is order-free); teams of 8 or 16 lanes
    // by DPP moves inside the 16-lane rows, wider ones by lane shuffles
    if constexpr (T == 8 || T == 16) {
      a[j] = group_max_nonneg<T>(a[j]);
    } else {
#pragma unroll
      for (int off = T / 2; off > 0; off >>= 1) a[j] = fmaxf(a[j], __shfl_xor(a[j], off, T));
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int64_t g = g0 + j;
    if (g >= n_groups) break;
    const int64_t go = MAP ? (g / map.seg_in) * map.seg_out + map.off + g % map.seg_in : g;
    const bool zero = (a[j] == 0.0f);
    const float r = quant_recip(a[j]);
    if (tl == 0) scales[go] = quant_scale(a[j]);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ci = tl + i * T;
      if (ci < n_chunks) store_codes(q, go * group_elems + static_cast<int64_t>(ci) * kChunk, c[j][i], r, zero);
    }
  }
}

// ---------------------------------------------------------------------------
// Large groups: grid (n_groups, blocks_per_group); each block strides over its
// group's chunks.
// ---------------------------------------------------------------------------
__global__ void zero_bits(uint32_t* bits, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) bits[i] = 0u;
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void absmax_large_groups(const void* __restrict__ x,
                                                                int64_t group_elems,
                                                                uint32_t* __restrict__ bits) {
  const int64_t g = blockIdx.x;
  const int64_t base = g * group_elems;
  const int64_t n_chunks = group_elems / kChunk;
  // kUnrollMax independent loads per lane in flight per round
  const int64_t stride = static_cast<int64_t>(gridDim.y) * kThreads;
  float am[kUnrollMax];
#pragma unroll
  for (int u = 0; u < kUnrollMax; ++u) am[u] = 0.0f;
  int64_t ci = static_cast<int64_t>(blockIdx.y) * kThreads + threadIdx.x;
  for (; ci + (kUnrollMax - 1) * stride < n_chunks; ci += kUnrollMax * stride) {
    Chunk8 c[kUnrollMax];
#pragma unroll
    for (int u = 0; u < kUnrollMax; ++u) c[u] = load_chunk<F16>(x, base + (ci + u * stride) * kChunk);
#pragma unroll
    for (int u = 0; u < kUnrollMax; ++u) am[u] = fmaxf(am[u], chunk_absmax(c[u]));
  }
  for (; ci < n_chunks; ci += stride) am[0] = fmaxf(am[0], chunk_absmax(load_chunk<F16>(x, base + ci * kChunk)));
  float a = am[0];
#pragma unroll
  for (int u = 1; u < kUnrollMax; ++u) a = fmaxf(a, am[u]);
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wmax[0];
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, wmax[w]);
    atomicMax(bits + g, __float_as_uint(m));  // |x| >= 0: float order == bit order
  }
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void quantize_large_groups(const void* __restrict__ x,
                                                                  int64_t group_elems,
                                                                  const uint32_t* __restrict__ bits,
                                                                  int8_t* __restrict__ q) {
  const int64_t g = blockIdx.x;
  const int64_t base = g * group_elems;
  const int64_t n_chunks = group_elems / kChunk;
  const float a = __uint_as_float(bits[g]);
  const bool zero = (a == 0.0f);
  const float r = quant_recip(a);
  const int64_t stride = static_cast<int64_t>(gridDim.y) * kThreads;
  int64_t ci = static_cast<int64_t>(blockIdx.y) * kThreads + threadIdx.x;
  for (; ci + (kUnroll - 1) * stride < n_chunks; ci += kUnroll * stride) {
    Chunk8 c[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) c[u] = load_chunk<F16>(x, base + (ci + u * stride) * kChunk);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) store_codes(q, base + (ci + u * stride) * kChunk, c[u], r, zero);
  }
  for (; ci < n_chunks; ci += stride) store_codes(q, base + ci * kChunk, load_chunk<F16>(x, base + ci * kChunk), r, zero);
}

__global__ void finalize_scales(float* scales, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) {
    scales[i] = quant_scale(__uint_as_float(reinterpret_cast<const uint32_t*>(scales)[i]));
  }
}

// ---------------------------------------------------------------------------
// Column groups (one scale per column of each group of rows, e.g. per channel
// of each (batch, kv head) of V): grid (n_groups, blocks_per_group). A lane
// owns one 8-column chunk and strides over rows; the block's rows are cut in
// rpi slots of ncc lanes each (ncc = n_cols / 8 <= 256).
// ---------------------------------------------------------------------------
template <bool F16>
__global__ __launch_bounds__(kThreads) void absmax_cols(const void* __restrict__ x, int64_t rows, int n_cols,
                                                        uint32_t* __restrict__ bits) {
  __shared__ float red[kThreads * kChunk];
  const int ncc = n_cols / kChunk;
  const int rpi = kThreads / ncc;
  const int cc = threadIdx.x % ncc, rr = threadIdx.x / ncc;
  const int64_t g = blockIdx.x;
  float m[kChunk];
#pragma unroll
  for (int e = 0; e < kChunk; ++e) m[e] = 0.0f;
  if (rr < rpi) {
    const int64_t stride = static_cast<int64_t>(gridDim.y) * rpi;
    int64_t r = static_cast<int64_t>(blockIdx.y) * rpi + rr;
    for (; r + (kUnroll - 1) * stride < rows; r += kUnroll * stride) {
      Chunk8 c[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) c[u] = load_chunk<F16>(x, ((g * rows) + r + u * stride) * n_cols + cc * kChunk);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) m[e] = fmaxf(m[e], fabsf(c[u].x[e]));
    }
    for (; r < rows; r += stride) {
      const Chunk8 c = load_chunk<F16>(x, (g * rows + r) * n_cols + cc * kChunk);
#pragma unroll
      for (int e = 0; e < kChunk; ++e) m[e] = fmaxf(m[e], fabsf(c.x[e]));
    }
#pragma unroll
    for (int e = 0; e < kChunk; ++e) red[rr * n_cols + cc * kChunk + e] = m[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n_cols; c += kThreads) {
    float a = red[c];
    for (int i = 1; i < rpi; ++i) a = fmaxf(a, red[i * n_cols + c]);
    atomicMax(bits + g * n_cols + c, __float_as_uint(a));   // |x| >= 0: float order == bit order
  }
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void quantize_cols(const void* __restrict__ x, int64_t rows, int n_cols,
                                                          const uint32_t* __restrict__ bits, int8_t* __restrict__ q) {
  __shared__ float rc[kMaxQuantCols];
  const int64_t g = blockIdx.x;
  for (int c = threadIdx.x; c < n_cols; c += kThreads) rc[c] = quant_recip(__uint_as_float(bits[g * n_cols + c]));
  __syncthreads();
  const int ncc = n_cols / kChunk;
  const int rpi = kThreads / ncc;
  const int cc = threadIdx.x % ncc, rr = threadIdx.x / ncc;
  if (rr >= rpi) return;
  float r[kChunk];
#pragma unroll
  for (int e = 0; e < kChunk; ++e) r[e] = rc[cc * kChunk + e];
  const int64_t stride = static_cast<int64_t>(gridDim.y) * rpi;
  for (int64_t row = static_cast<int64_t>(blockIdx.y) * rpi + rr; row < rows; row += stride) {
    const int64_t elem = (g * rows + row) * n_cols + cc * kChunk;
    const Chunk8 c = load_chunk<F16>(x, elem);
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = quant_code(c.x[4 * h], r[4 * h]) | (quant_code(c.x[4 * h + 1], r[4 * h + 1]) << 8) |
             (quant_code(c.x[4 * h + 2], r[4 * h + 2]) << 16) | (quant_code(c.x[4 * h + 3], r[4 * h + 3]) << 24);
    *reinterpret_cast<uint2*>(q + elem) = make_uint2(w[0], w[1]);
  }
}

template <bool F16>
hipError_t run_cols(const void* x, int64_t n_groups, int64_t rows, int n_cols, int8_t* q, float* s, hipStream_t st) {
  const int64_t n = n_groups * n_cols;
  uint32_t* bits = reinterpret_cast<uint32_t*>(s);
  const unsigned zb = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(zero_bits, dim3(zb), dim3(256), 0, st, bits, n);
  // about 2048 workgroups in all, each row slot covering at least 16 rows
  const int rpi = kThreads / (n_cols / kChunk);
  int64_t bpg = (rows + int64_t{rpi} * 16 - 1) / (int64_t{rpi} * 16);
  const int64_t cap = std::max<int64_t>(1, 2048 / n_groups);
  if (bpg > cap) bpg = cap;
  const dim3 grid(static_cast<unsigned>(n_groups), static_cast<unsigned>(bpg));
  hipLaunchKernelGGL(absmax_cols<F16>, grid, dim3(kThreads), 0, st, x, rows, n_cols, bits);
  hipLaunchKernelGGL(quantize_cols<F16>, grid, dim3(kThreads), 0, st, x, rows, n_cols,
                     static_cast<const uint32_t*>(bits), q);
  hipLaunchKernelGGL(finalize_scales, dim3(zb), dim3(256), 0, st, s, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-token 4-bit codes (INT4 Q.K): s = a / 7, r = 7 / a, code = clamp(rne(x
// r), -7, 7); int8 codes and / or the packed form (per 8-channel group, byte
// j = (code[j] + 8) | (code[j + 4] + 8) << 4). A team of T lanes per row, CH
// chunks of 8 values per lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int code4(float x, float r) {
  const float t = fminf(7.0f, fmaxf(-7.0f, __builtin_rintf(__fmul_rn(x, r))));
  return static_cast<int>(t);
}

template <bool F16, int T, int CH, bool MAP>
__global__ __launch_bounds__(kThreads) void quantize_rows4(const void* __restrict__ x, int64_t n_rows, int n_cols,
                                                           int8_t* __restrict__ codes, uint8_t* __restrict__ packed,
                                                           float* __restrict__ scales, RowMap map) {
  constexpr int kTeams = kThreads / T;
  const int tl = threadIdx.x % T;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTeams + threadIdx.x / T;
  const int n_chunks = n_cols / kChunk;
  Chunk8 c[CH];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ci = tl + i * T;
    if (row < n_rows && ci < n_chunks) {
      c[i] = load_chunk<F16>(x, row * n_cols + static_cast<int64_t>(ci) * kChunk);
      a = fmaxf(a, chunk_absmax(c[i]));
    }
  }
  if constexpr (T == 8 || T == 16) {
    a = group_max_nonneg<T>(a);
  } else {
#pragma unroll
    for (int off = T / 2; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, T));
  }
  if (row >= n_rows) return;
  const int64_t go = MAP ? (row / map.seg_in) * map.seg_out + map.off + row % map.seg_in : row;
  const float r = a == 0.0f ? 0.0f : __fdiv_rn(7.0f, a);
  if (tl == 0) scales[go] = a == 0.0f ? 0.0f : __fdiv_rn(a, 7.0f);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ci = tl + i * T;
    if (ci >= n_chunks) continue;
    int k[kChunk];
#pragma unroll
    for (int e = 0; e < kChunk; ++e) k[e] = code4(c[i].x[e], r);
    if (codes) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        w[h] = (k[4 * h] & 0xff) | ((k[4 * h + 1] & 0xff) << 8) | ((k[4 * h + 2] & 0xff) << 16) |
               (static_cast<uint32_t>(k[4 * h + 3] & 0xff) << 24);
      *reinterpret_cast<uint2*>(codes + go * n_cols + static_cast<int64_t>(ci) * kChunk) = make_uint2(w[0], w[1]);
    }
    if (packed) {
      uint32_t p = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) p |= static_cast<uint32_t>((k[j] + 8) | ((k[j + 4] + 8) << 4)) << (8 * j);
      *reinterpret_cast<uint32_t*>(packed + go * (n_cols / 2) + static_cast<int64_t>(ci) * 4) = p;
    }
  }
}

template <bool F16, int T, int CH>
hipError_t run4(const void* x, int64_t n_rows, int n_cols, int8_t* codes, uint8_t* packed, float* s, hipStream_t st,
                const RowMap* map) {
  constexpr int kTeams = kThreads / T;
  const int64_t blocks = (n_rows + kTeams - 1) / kTeams;
  if (map)
    hipLaunchKernelGGL((quantize_rows4<F16, T, CH, true>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st,
                       x, n_rows, n_cols, codes, packed, s, *map);
  else
    hipLaunchKernelGGL((quantize_rows4<F16, T, CH, false>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       st, x, n_rows, n_cols, codes, packed, s, RowMap{1, 1, 0});
  return hipGetLastError();
}

template <bool F16>
hipError_t run_int4(const void* x, int64_t n_rows, int n_cols, int8_t* codes, uint8_t* packed, float* s,
                    hipStream_t st, const RowMap* map = nullptr) {
  const int n_chunks = n_cols / kChunk;
  if (n_chunks <= 8) return run4<F16, 8, 1>(x, n_rows, n_cols, codes, packed, s, st, map);
  if (n_chunks <= 16) return run4<F16, 16, 1>(x, n_rows, n_cols, codes, packed, s, st, map);
  if (n_chunks <= 32) return run4<F16, 32, 1>(x, n_rows, n_cols, codes, packed, s, st, map);
  if (n_chunks <= 64) return run4<F16, 64, 1>(x, n_rows, n_cols, codes, packed, s, st, map);
  return run4<F16, 64, 4>(x, n_rows, n_cols, codes, packed, s, st, map);
}

// ---------------------------------------------------------------------------
// Rows rotated by the normalized Hadamard matrix (n = 2^k columns), then
// per-token codes at BITS = 8 or 4. A team of T lanes per row, lane tl holding
// chunks tl + i T (i < CH) of 8 values. The fast transform runs its strides in
// increasing order, h = 1, 2, 4 inside a chunk, then chunk offsets 1 .. T / 2
// across lanes (shuffles) and T .. (CH / 2) T inside the lane; each pair
// becomes (a + b, a - b) with a the lower index, the upper side formed as
// fma(-1, own, partner) = partner - own, exactly the subtraction. Then every
// value times rn = fl32(1 / sqrt(n)).
// ---------------------------------------------------------------------------
template <bool F16, int T, int CH, int BITS>
__global__ __launch_bounds__(kThreads) void quantize_rows_rot(const void* __restrict__ x, int64_t n_rows, int n_cols,
                                                              float rn, int8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ packed, float* __restrict__ scales) {
  constexpr int kTeams = kThreads / T;
  const int tl = threadIdx.x % T;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kTeams + threadIdx.x / T;
  const bool valid = row < n_rows;
  Chunk8 c[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (valid) {
      c[i] = load_chunk<F16>(x, row * n_cols + static_cast<int64_t>(tl + i * T) * kChunk);
    } else {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) c[i].x[e] = 0.0f;
    }
  }
  // strides 1, 2, 4 inside each chunk
#pragma unroll
  for (int h = 1; h < kChunk; h <<= 1)
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int e = 0; e < kChunk; ++e)
        if (!(e & h)) {
          const float a = c[i].x[e], b = c[i].x[e + h];
          c[i].x[e] = a + b;
          c[i].x[e + h] = a - b;
        }
  // chunk offsets 1 .. T / 2: the partner lane tl ^ m
#pragma unroll
  for (int m = 1; m < T; m <<= 1) {
    const float sgn = (tl & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const float p = __shfl_xor(c[i].x[e], m, T);
        c[i].x[e] = __builtin_fmaf(sgn, c[i].x[e], p);
      }
  }
  // chunk offsets T .. (CH / 2) T: chunks i and i ^ (m / T) of the lane
#pragma unroll
  for (int m = 1; m < CH; m <<= 1)
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (!(i & m)) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const float a = c[i].x[e], b = c[i ^ m].x[e];
          c[i].x[e] = a + b;
          c[i ^ m].x[e] = a - b;
        }
      }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
#pragma unroll
    for (int e = 0; e < kChunk; ++e) c[i].x[e] = c[i].x[e] * rn;
    a = fmaxf(a, chunk_absmax(c[i]));
  }
#pragma unroll
  for (int off = T / 2; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, T));
  if (!valid) return;
  if constexpr (BITS == 8) {
    const float r = quant_recip(a);
    if (tl == 0) scales[row] = quant_scale(a);
#pragma unroll
    for (int i = 0; i < CH; ++i) store_codes(codes, row * n_cols + static_cast<int64_t>(tl + i * T) * kChunk, c[i], r,
                                             a == 0.0f);
  } else {
    const float r = a == 0.0f ? 0.0f : __fdiv_rn(7.0f, a);
    if (tl == 0) scales[row] = a == 0.0f ? 0.0f : __fdiv_rn(a, 7.0f);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t ci = tl + i * T;
      int k[kChunk];
#pragma unroll
      for (int e = 0; e < kChunk; ++e) k[e] = code4(c[i].x[e], r);
      if (codes) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          w[h] = (k[4 * h] & 0xff) | ((k[4 * h + 1] & 0xff) << 8) | ((k[4 * h + 2] & 0xff) << 16) |
                 (static_cast<uint32_t>(k[4 * h + 3] & 0xff) << 24);
        *reinterpret_cast<uint2*>(codes + row * n_cols + ci * kChunk) = make_uint2(w[0], w[1]);
      }
      if (packed) {
        uint32_t p = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) p |= static_cast<uint32_t>((k[j] + 8) | ((k[j + 4] + 8) << 4)) << (8 * j);
        *reinterpret_cast<uint32_t*>(packed + row * (n_cols / 2) + ci * 4) = p;
      }
    }
  }
}

template <bool F16, int T, int CH, int BITS>
hipError_t run_rot(const void* x, int64_t n_rows, int n_cols, float rn, int8_t* codes, uint8_t* packed, float* s,
                   hipStream_t st) {
  constexpr int kTeams = kThreads / T;
  const int64_t blocks = (n_rows + kTeams - 1) / kTeams;
  hipLaunchKernelGGL((quantize_rows_rot<F16, T, CH, BITS>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     st, x, n_rows, n_cols, rn, codes, packed, s);
  return hipGetLastError();
}

template <bool F16, int BITS>
hipError_t run_rot_n(const void* x, int64_t n_rows, int n_cols, float rn, int8_t* codes, uint8_t* packed, float* s,
                     hipStream_t st) {
  switch (n_cols / kChunk) {
    case 1: return run_rot<F16, 1, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 2: return run_rot<F16, 2, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 4: return run_rot<F16, 4, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 8: return run_rot<F16, 8, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 16: return run_rot<F16, 16, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 32: return run_rot<F16, 32, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 64: return run_rot<F16, 64, 1, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    case 128: return run_rot<F16, 64, 2, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
    default: return run_rot<F16, 64, 4, BITS>(x, n_rows, n_cols, rn, codes, packed, s, st);
  }
}

// packed 4-bit codes -> int8 codes, 8 per packed word: nibble n is code n - 8
// (per byte: set bit 7, subtract 8, clear bit 7 again: no borrow crosses bytes)
__global__ void unpack_int4(const uint32_t* __restrict__ packed, int64_t n_words, uint2* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += stride) {
    const uint32_t w = packed[i];
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    out[i] = make_uint2(((lo | 0x80808080u) - 0x08080808u) ^ 0x80808080u,
                        ((hi | 0x80808080u) - 0x08080808u) ^ 0x80808080u);
  }
}

template <bool F16, int T, int CH, int G>
hipError_t run_small(const void* x, int64_t n_groups, int64_t ge, int8_t* q, float* s, hipStream_t st,
                     const RowMap* map = nullptr) {
  constexpr int kTeams = kThreads / T;
  const int64_t per_block = int64_t{kTeams} * G;
  const int64_t blocks = (n_groups + per_block - 1) / per_block;
  if (map)
    hipLaunchKernelGGL((quantize_small_groups<F16, T, CH, G, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, st, x, n_groups, ge, q, s, *map);
  else
    hipLaunchKernelGGL((quantize_small_groups<F16, T, CH, G, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, st, x, n_groups, ge, q, s, RowMap{1, 1, 0});
  return hipGetLastError();
}

// Per-token groups of at most kMaxAppendCols columns, written through a row map.
template <bool F16>
hipError_t run_mapped(const void* x, int64_t n_rows, int n_cols, int8_t* q, float* s, const RowMap& map,
                      hipStream_t st) {
  const int64_t n_chunks = n_cols / kChunk;
  if (n_chunks <= 8) return run_small<F16, 8, 1, 1>(x, n_rows, n_cols, q, s, st, &map);
  if (n_chunks <= 16) return run_small<F16, 16, 1, 1>(x, n_rows, n_cols, q, s, st, &map);
  if (n_chunks <= 32) return run_small<F16, 32, 1, 1>(x, n_rows, n_cols, q, s, st, &map);
  if (n_chunks <= 64) return run_small<F16, 64, 1, 1>(x, n_rows, n_cols, q, s, st, &map);
  return run_small<F16, 64, 4, 1>(x, n_rows, n_cols, q, s, st, &map);
}

template <bool F16>
hipError_t run(const void* x, int64_t n_rows, int n_cols, int64_t rps, int8_t* q, float* s,
               hipStream_t st) {
  const int64_t ge = rps * static_cast<int64_t>(n_cols);
  const int64_t n_groups = n_rows / rps;
  const int64_t n_chunks = ge / kChunk;
  if (n_chunks <= 8) return run_small<F16, 8, 1, 1>(x, n_groups, ge, q, s, st);
  if (n_chunks <= 16) return run_small<F16, 16, 1, 2>(x, n_groups, ge, q, s, st);   // 2 rows per team: measured 6 % faster
  if (n_chunks <= 32) return run_small<F16, 32, 1, 1>(x, n_groups, ge, q, s, st);
  if (n_chunks <= 64) return run_small<F16, 64, 1, 1>(x, n_groups, ge, q, s, st);
  if (n_chunks <= 256) return run_small<F16, 64, 4, 1>(x, n_groups, ge, q, s, st);
  // large groups: zero the maxima, atomic max, quantize, turn maxima into scales
  uint32_t* bits = reinterpret_cast<uint32_t*>(s);
  const unsigned zb = static_cast<unsigned>((n_groups + 255) / 256);
  hipLaunchKernelGGL(zero_bits, dim3(zb), dim3(256), 0, st, bits, n_groups);
  const int64_t per_block = static_cast<int64_t>(kThreads) * 4 * kUnroll;   // chunks per block
  int64_t bpg = (n_chunks + per_block - 1) / per_block;
  if (bpg > 2048) bpg = 2048;
  const dim3 grid(static_cast<unsigned>(n_groups), static_cast<unsigned>(bpg));
  const dim3 grid_max(static_cast<unsigned>(n_groups), static_cast<unsigned>(bpg < kMaxAbsmaxBlocks ? bpg : kMaxAbsmaxBlocks));
  hipLaunchKernelGGL(absmax_large_groups<F16>, grid_max, dim3(kThreads), 0, st, x, ge, bits);
  hipLaunchKernelGGL(quantize_large_groups<F16>, grid, dim3(kThreads), 0, st, x, ge,
                     static_cast<const uint32_t*>(bits), q);
  hipLaunchKernelGGL(finalize_scales, dim3(zb), dim3(256), 0, st, s, n_groups);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, int x_f16, int64_t n_rows, int n_cols, int64_t rps,
                           int8_t* q, float* scales, hipStream_t st) {
  return x_f16 ? run<true>(x, n_rows, n_cols, rps, q, scales, st)
               : run<false>(x, n_rows, n_cols, rps, q, scales, st);
}

hipError_t launch_quantize_cols(const void* x, int x_f16, int64_t n_groups, int64_t rows_per_group, int n_cols,
                                int8_t* q, float* scales, hipStream_t st) {
  return x_f16 ? run_cols<true>(x, n_groups, rows_per_group, n_cols, q, scales, st)
               : run_cols<false>(x, n_groups, rows_per_group, n_cols, q, scales, st);
}

hipError_t launch_quantize_int4(const void* x, int x_f16, int64_t n_rows, int n_cols, int8_t* codes,
                                uint8_t* packed, float* scales, hipStream_t st) {
  return x_f16 ? run_int4<true>(x, n_rows, n_cols, codes, packed, scales, st)
               : run_int4<false>(x, n_rows, n_cols, codes, packed, scales, st);
}

hipError_t launch_append_int4(const void* x, int x_f16, int64_t segments, int t_new, int n_cols, int l_max, int pos,
                              uint8_t* cache4, float* scales, hipStream_t st) {
  const RowMap map{t_new, l_max, pos};
  const int64_t n_rows = segments * t_new;
  return x_f16 ? run_int4<true>(x, n_rows, n_cols, nullptr, cache4, scales, st, &map)
               : run_int4<false>(x, n_rows, n_cols, nullptr, cache4, scales, st, &map);
}

hipError_t launch_quantize_rotated(const void* x, int x_f16, int64_t n_rows, int n_cols, int bits, float rn,
                                   int8_t* codes, uint8_t* packed, float* scales, hipStream_t st) {
  if (bits == 8)
    return x_f16 ? run_rot_n<true, 8>(x, n_rows, n_cols, rn, codes, packed, scales, st)
                 : run_rot_n<false, 8>(x, n_rows, n_cols, rn, codes, packed, scales, st);
  return x_f16 ? run_rot_n<true, 4>(x, n_rows, n_cols, rn, codes, packed, scales, st)
               : run_rot_n<false, 4>(x, n_rows, n_cols, rn, codes, packed, scales, st);
}

hipError_t launch_unpack_int4(const uint8_t* packed, int64_t n_bytes, int8_t* out, hipStream_t st) {
  const int64_t n_words = n_bytes / 4;
  const int64_t blocks = std::min<int64_t>((n_words + 255) / 256, 8192);
  hipLaunchKernelGGL(unpack_int4, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(packed), n_words, reinterpret_cast<uint2*>(out));
  return hipGetLastError();
}

hipError_t launch_append(const void* x, int x_f16, int64_t segments, int t_new, int n_cols, int l_max,
                         int pos, int8_t* cache, float* scales, hipStream_t st) {
  const RowMap map{t_new, l_max, pos};
  const int64_t n_rows = segments * t_new;
  return x_f16 ? run_mapped<true>(x, n_rows, n_cols, cache, scales, map, st)
               : run_mapped<false>(x, n_rows, n_cols, cache, scales, map, st);
}

}  // namespace attn
