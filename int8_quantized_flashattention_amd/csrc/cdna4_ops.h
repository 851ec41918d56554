// gfx950 building blocks shared by the attention kernels of libattn_int8:
// the INT8 MFMA shapes, LDS-destination buffer loads, the transposing LDS
// read, explicit memory waits and a fence-free barrier, and the LDS row
// swizzle of K/V tiles. Internal header.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

// Lower bound on wavefronts per SIMD for a kernel (caps its registers); a
// host-side stand-in of the HIP headers may define it away.
#ifndef ATTN_WAVES_PER_EU
#define ATTN_WAVES_PER_EU(n) __attribute__((amdgpu_waves_per_eu(n)))
#endif

namespace attn {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kFltMin = 1.17549435e-38f;
constexpr int kBufWord3 = 0x00020000;        // raw buffer, 32-bit data format
// re-base an fp32 accumulator when the running max has grown by this much
// (base 2) since its frame was set
constexpr float kRebase = 60.0f;

__device__ __forceinline__ v16i zero16() { return v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ v4i zero4() { return v4i{0, 0, 0, 0}; }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest of the non-negative fp32 values of each aligned group of T lanes
// (T = 8 or 16), in every lane of the group: the bit patterns of non-negative
// floats order as the floats do, so unsigned maxima on them are exact. DPP
// moves inside the 16-lane rows (quad exchanges, then the half-row mirror, for
// T = 16 also the row mirror): VALU work only, no LDS round trip.
template <int T>
__device__ __forceinline__ float group_max_nonneg(float x) {
  static_assert(T == 8 || T == 16, "DPP groups of 8 or 16 lanes");
  uint32_t u = __float_as_uint(x);
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0xB1, 0xf, 0xf, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x4E, 0xf, 0xf, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x141, 0xf, 0xf, false)));
  if constexpr (T == 16)
    u = max(u, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x140, 0xf, 0xf, false)));
  return __uint_as_float(u);
}

// The same over all 64 lanes: each row's maximum, then one lane of each row.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  const uint32_t u = __float_as_uint(group_max_nonneg<16>(x));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 48));
  return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// log2(e) / sqrt(d) rounded to fp32 (d = 64, 128): a row's base-2 logit is
// (S_int (s_Q c)) s_K[j] with c this factor
template <int D>
constexpr float kLogitScale = D == 64 ? 0.18033687770366669f : 0.12751743197441101f;

// Exponent bias of a running max m (base 2): m - log2(127) in fp32, moved up
// one float when m minus it still exceeds log2(127) after rounding. Every
// logit x <= m then has x - b <= log2(127) in fp32, so 2^(x - b) stays within
// 127 (up to the exponential's own rounding) and its code fits a signed byte
// whatever the magnitude of m. The nudged value is never +-0.
__device__ __forceinline__ float exp_bias(float m) {
  const float b = m - kLog2_127;
  const uint32_t u = __float_as_uint(b);
  return (m - b > kLog2_127) ? __uint_as_float(b > 0.0f ? u + 1u : u - 1u) : b;
}

// 32x32x32 and 16x16x64 INT8 products with INT32 accumulation
__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most N vector-memory loads are outstanding and
// all LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier without a memory fence: the explicit waits above are
// the only ones a stage ring needs (a fenced barrier would also wait for the
// stages requested ahead). The empty asm statements keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS-destination buffer loads (16 or 4 bytes per lane, lane l's bytes at
// dst + size l) and the transposing LDS read, as plain functions: the
// gfx950-only forms are checked in the host compilation pass too, where a
// template would turn the check into a substitution failure.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, voff, soff, 0, 0);
}
// 8 or 16 bytes per lane from a raw buffer into registers (zero where the
// offset lies outside the buffer)
__device__ __forceinline__ v2i buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// The same loads with the non-temporal cache policy (the nt bit of the
// instruction's cache-policy field), for data read exactly once: a split-KV
// chunk streams its K and V rows past the caches instead of through them.
constexpr int kCpolNT = 2;
__device__ __forceinline__ void lds_load16_nt(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, kCpolNT);
}
__device__ __forceinline__ void lds_load4_nt(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, voff, soff, 0, kCpolNT);
}
__device__ __forceinline__ v2i buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCpolNT));
}
__device__ __forceinline__ v4i buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNT));
}
// ds_read_b64_tr_b8: in each group of 16 lanes, lane i receives byte i % 8 of
// the 8-byte rows addressed by lanes 2 b + i / 8 (b = 0..7 gives byte b)
__device__ __forceinline__ v2i lds_read_tr8(const int8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
}

// The per-group quantizer's arithmetic, shared by the quantization pass and
// the fused Q quantization (so both give identical codes): for absmax a,
// r = 127 / a and s = a / 127 (correctly rounded; 0 when a == 0), and
// q = clamp(rne(x * r), -127, 127) with x * r one rounded fp32 product.
__device__ __forceinline__ float quant_recip(float a) { return a == 0.0f ? 0.0f : __fdiv_rn(127.0f, a); }
__device__ __forceinline__ float quant_scale(float a) { return a == 0.0f ? 0.0f : __fdiv_rn(a, 127.0f); }
__device__ __forceinline__ uint32_t quant_code(float x, float r) {
  float t = __builtin_rintf(__fmul_rn(x, r));
  t = fminf(127.0f, fmaxf(-127.0f, t));
  return static_cast<uint32_t>(static_cast<int>(t)) & 0xffu;
}
// codes of 4 values, byte i from x[i], for r = 127 / absmax of a group that
// holds the x: then |x * r| <= 127 (1 + 2^-24) and rne(x * r) lies in
// [-127, 127], so the clamp never acts. Adding 1.5 * 2^23 to the rounded
// product rounds it to an integer (ties to even: the sum's ulp is 1) and
// leaves that integer's two's-complement low byte in the low byte of the
// sum's bits; three byte permutes pack the four low bytes. The product must
// be rounded on its own (a fused x * r + 1.5 * 2^23 would round the exact
// product instead, and differ at ties): both operations are written here,
// where contraction is off (the _rn helpers of the HIP headers carry the
// headers' own contraction setting).
__device__ __forceinline__ uint32_t quant_word(const float* x, float r) {
#pragma clang fp contract(off)
  uint32_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(x[i] * r + 12582912.0f);
  // v_perm_b32 (s0, s1, sel): byte k of the result is byte sel_k of s1:s0
  // (s1 = bytes 0-3, s0 = bytes 4-7), selector 12 gives 0
  const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// N runs of 16 consecutive Q values of one row, run c at element elem0 + c *
// stride. fp16 rows: q16_load issues every load of the row (raw halves in
// registers) and q16_f32 converts them once they are needed, so the row
// costs one memory latency and work placed between the two calls overlaps
// it. fp32 rows (q32_f32) are loaded and converted in one go.
template <int N>
__device__ __forceinline__ void q16_load(const void* base, int64_t elem0, int stride, v4i (&raw)[N][2]) {
  const uint16_t* p = static_cast<const uint16_t*>(base) + elem0;
#pragma unroll
  for (int c = 0; c < N; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) raw[c][h] = reinterpret_cast<const v4i*>(p + c * stride)[h];
}
template <int N>
__device__ __forceinline__ void q16_f32(const v4i (&raw)[N][2], float (&x)[N][16]) {
#pragma unroll
  for (int c = 0; c < N; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = static_cast<uint32_t>(raw[c][h][i]);
        x[c][h * 8 + 2 * i] = __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu)));
        x[c][h * 8 + 2 * i + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
      }
}
template <int N>
__device__ __forceinline__ void q32_f32(const void* base, int64_t elem0, int stride, float (&x)[N][16]) {
  const float* p = static_cast<const float*>(base) + elem0;
#pragma unroll
  for (int c = 0; c < N; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = reinterpret_cast<const float4*>(p + c * stride)[i];
      x[c][4 * i] = f.x; x[c][4 * i + 1] = f.y; x[c][4 * i + 2] = f.z; x[c][4 * i + 3] = f.w;
    }
}

// Raw buffer resource over nbytes bytes (loads at or past the end read 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, nbytes, kBufWord3);
}

// K/V tile rows of D bytes are stored with their 16-byte chunks permuted:
// chunk j of row r sits at chunk position j ^ swz(r). gfx950's LDS serves 64
// banks of 4 bytes per cycle, i.e. 16 lanes of a ds_read_b128 or 32 lanes of
// a ds_read_b64_tr_b8; the permutation spreads every such lane group over all
// 64 banks for the prefill's K operand reads (lanes 0-15 read rows 0-3,
// 16-19, 4-7, 20-23, one chunk each) and for the transposing V reads of the
// prefill and the decode kernels (32 lanes on 16 consecutive rows, two
// 8-byte halves of one chunk per row). Measured with the LDS counters: 4
// cycles per K read and 2 per V read, no bank-conflict cycles (the earlier
// form (r & 7) ^ ((r >> 2) & 4) took 8 cycles per K read).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
  else return (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
}

// Tile byte offset of the 16-byte chunk that a 1 KB LDS-destination load
// writes into LDS slot 64 n + lane of a swizzled tile.
template <int D>
__device__ __forceinline__ uint32_t tile_load_off(int n, int lane) {
  const int slot = n * 64 + lane;
  const int r = slot / (D / 16), pos = slot % (D / 16);
  return static_cast<uint32_t>(r * D + (pos ^ swz<D>(r)) * 16);
}

}  // namespace
}  // namespace attn
