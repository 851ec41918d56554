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
// relative guard on the softmax bias: exp2(u c2 - bias) with bias =
// m - log2(127) + |m| 2^-21 keeps the max key's 127 P_tilde below 127.5
// however large |m| is (the fp32 rounding of u c2 and of the bias grows with
// |m|); P_hat and the row sum scale together, so the guard cancels in O
constexpr float kBiasGuard = 4.76837158203125e-07f;   // 2^-21
// The guard is applied only from |m| = 2^15 on: below, the two fp32 roundings
// (of u c2 and of the bias, each at most |m| 2^-24) move the max key's
// exponent by less than 2^-8, short of the log2(127.5 / 127) = 0.0057 that a
// code of 128 needs, and an unneeded guard would shift every 127 P_tilde down
// by |m| 2^-21 and flip codes that sit near a rounding tie.
constexpr float kBiasGuardFrom = 32768.0f;

__device__ __forceinline__ v16i zero16() { return v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ v4i zero4() { return v4i{0, 0, 0, 0}; }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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
// codes of 4 values, byte i from x[i]
__device__ __forceinline__ uint32_t quant_word(const float* x, float r) {
  return quant_code(x[0], r) | (quant_code(x[1], r) << 8) | (quant_code(x[2], r) << 16) | (quant_code(x[3], r) << 24);
}

// 16 consecutive Q values of one row as fp32 (fp16 or fp32 storage)
__device__ __forceinline__ void load16_as_f32(const void* base, int64_t elem, bool f16, float (&x)[16]) {
  if (f16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 raw = p[h];
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __half2 hv = *reinterpret_cast<const __half2*>(&w[i]);
        const float2 f = __half22float2(hv);
        x[h * 8 + 2 * i] = f.x;
        x[h * 8 + 2 * i + 1] = f.y;
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
    }
  }
}

// Raw buffer resource over nbytes bytes (loads at or past the end read 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, nbytes, kBufWord3);
}

// K/V tile rows of D bytes are stored with their 16-byte chunks permuted:
// chunk j of row r sits at chunk position j ^ swz(r). The permutation makes
// the operand reads conflict-free: 8 lanes reading the same chunk of rows
// {0-3, 16-19} + 4 i, and 16 lanes reading 8 consecutive rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (r & 7) ^ ((r >> 2) & 4);
  else return ((r >> 1) & 3) ^ (((r >> 4) & 1) << 1);
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
