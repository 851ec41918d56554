// CPU stand-in for the subset of HIP that libattn_int8's sources use.
//
// TEST INFRASTRUCTURE: the unchanged kernel sources are compiled for the host
// against this header (it sits first on the include path) and run on small
// problems under AddressSanitizer/UBSan, so that an out-of-bounds or
// misaligned access shows up on the CPU, with a stack trace, instead of as a
// GPU memory fault. Every lane is a host thread; __syncthreads is a block-wide
// barrier; cross-lane operations (shuffles, MFMA) exchange operands through a
// per-wavefront buffer between two wavefront barriers. Blocks run one after
// another, so a function-local __shared__ variable (made static here) behaves
// as the block's LDS.
//
// The MFMA operand/result layouts encoded below are the documented CDNA ones
// (32x32: result element (i, j) in lane j + 32 * ((i / 4) % 2), register
// (i % 4) + 4 * (i / 8); 16x16: lane j + 16 * (i / 4), register i % 4;
// operand element (row r, k) in lane r + (lanes per block) * (k / kpl), byte
// k % kpl with kpl int8 values per lane). The GPU parity tests check them on
// the hardware.
#pragma once

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <thread>
#include <type_traits>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorNotSupported = 801 };
typedef struct ihipStream_t* hipStream_t;
inline hipError_t hipGetLastError() { return hipSuccess; }
// one emulated device; a __device__ variable is an ordinary host object whose
// address the symbol lookup returns
#define __align__(n) alignas(n)
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned x_ = 1, unsigned y_ = 1, unsigned z_ = 1) : x(x_), y(y_), z(z_) {}
};
struct emu_uint3 { unsigned x, y, z; };

struct alignas(8) float2 { float x, y; };
struct alignas(16) float4 { float x, y, z, w; };
struct alignas(8) uint2 { unsigned x, y; };
struct alignas(16) uint4 { unsigned x, y, z, w; };
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline float2 make_float2(float a, float b) { return {a, b}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return {a, b}; }

namespace emu {

// A reusable barrier with its own mutex and condition variable (generation
// count; arrive_and_drop leaves it for good). The C++ library's barrier parks
// its waiters in a process-wide pool of mutexes keyed by address, which
// ThreadSanitizer sees as ordering threads of unrelated barriers (other
// wavefronts) and so hides the races this emulation is also run to find.
class Barrier {
 public:
  explicit Barrier(int n) : expected_(n) {}
  void arrive_and_wait() {
    std::unique_lock<std::mutex> lk(mu_);
    const unsigned long gen = gen_;
    if (++arrived_ == expected_) {
      next_phase();
    } else {
      cv_.wait(lk, [&] { return gen_ != gen; });
    }
  }
  void arrive_and_drop() {
    std::lock_guard<std::mutex> lk(mu_);
    --expected_;
    if (arrived_ == expected_ && expected_ > 0) next_phase();
  }

 private:
  void next_phase() {
    arrived_ = 0;
    ++gen_;
    cv_.notify_all();
  }
  std::mutex mu_;
  std::condition_variable cv_;
  int expected_;
  int arrived_ = 0;
  unsigned long gen_ = 0;
};

struct Wave {
  explicit Wave(int n) : bar(n) {}
  Barrier bar;
  alignas(16) unsigned char slot[64][64];
};

struct Ctx {
  emu_uint3 tid, bid;
  Wave* wave;
  int lane;
};
inline thread_local Ctx ctx;
inline dim3 g_grid, g_block;
inline Barrier* g_block_bar = nullptr;

template <class F>
void launch(dim3 grid, dim3 block, F&& body) {
  g_grid = grid;
  g_block = block;
  const int nthreads = static_cast<int>(block.x * block.y * block.z);
  const int nwaves = (nthreads + 63) / 64;
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        Barrier bbar(nthreads);
        g_block_bar = &bbar;
        std::vector<std::unique_ptr<Wave>> waves;
        for (int w = 0; w < nwaves; ++w)
          waves.emplace_back(new Wave(std::min(64, nthreads - 64 * w)));
        std::vector<std::thread> th;
        th.reserve(nthreads);
        for (int t = 0; t < nthreads; ++t) {
          th.emplace_back([&, t]() {
            ctx.tid = {static_cast<unsigned>(t % block.x), static_cast<unsigned>((t / block.x) % block.y),
                       static_cast<unsigned>(t / (block.x * block.y))};
            ctx.bid = {bx, by, bz};
            ctx.wave = waves[t / 64].get();
            ctx.lane = t % 64;
            body();
            ctx.wave->bar.arrive_and_drop();
            g_block_bar->arrive_and_drop();
          });
        }
        for (auto& x : th) x.join();
        g_block_bar = nullptr;
      }
}

inline void syncthreads() { g_block_bar->arrive_and_wait(); }

template <class T>
T shfl_xor(T v, int mask, int width = 64) {
  static_assert(sizeof(T) <= 64, "exchange slot too small");
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  int src = self ^ mask;
  if (src >= ((self + width) & ~(width - 1))) src = self;
  std::memcpy(w.slot[self], &v, sizeof(T));
  w.bar.arrive_and_wait();
  T r;
  std::memcpy(&r, w.slot[src], sizeof(T));
  w.bar.arrive_and_wait();
  return r;
}

// result[i][j] += sum_k A[i][k] B[k][j] for int8 operands (kpl bytes per lane)
template <int M, class VA, class VC>
VC mfma_i8(VA a, VA b, VC c) {
  static_assert(sizeof(VA) == 16, "16 int8 per lane");
  constexpr int kpl = 16;
  constexpr int K = 64 / M * kpl;          // 32 for 32x32, 64 for 16x16
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &a, 16);
  std::memcpy(w.slot[self] + 16, &b, 16);
  w.bar.arrive_and_wait();
  VC d = c;
  constexpr int NREG = sizeof(VC) / 4;
  for (int v = 0; v < NREG; ++v) {
    int i, j;
    if constexpr (M == 32) {
      j = self % 32;
      i = (v / 4) * 8 + (self / 32) * 4 + v % 4;
    } else {
      j = self % 16;
      i = (self / 16) * 4 + v;
    }
    int32_t acc = d[v];
    for (int k = 0; k < K; ++k) {
      const int la = i + M * (k / kpl), lb = j + M * (k / kpl);
      acc += static_cast<int32_t>(static_cast<int8_t>(w.slot[la][k % kpl])) *
             static_cast<int32_t>(static_cast<int8_t>(w.slot[lb][16 + k % kpl]));
    }
    d[v] = acc;
  }
  w.bar.arrive_and_wait();
  return d;
}

// v_perm_b32: bytes 0-3 of the 64-bit source are src1, bytes 4-7 src0.
inline uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  const uint64_t src = (static_cast<uint64_t>(s0) << 32) | s1;
  uint32_t out = 0;
  for (int b = 0; b < 4; ++b) {
    const uint32_t s = (sel >> (8 * b)) & 0xffu;
    uint32_t byte;
    if (s < 8) byte = (src >> (8 * s)) & 0xffu;
    else if (s < 12) byte = ((src >> (8 * (2 * (s - 8) + 1))) & 0x80u) ? 0xffu : 0u;
    else if (s == 12) byte = 0u;
    else byte = 0xffu;
    out |= byte << (8 * b);
  }
  return out;
}

// v_permlane32_swap on (x, y) as measured on gfx950: lanes 0-31 get
// (x[l], x[l + 32]), lanes 32-63 get (y[l - 32], y[l]).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
inline u32x2 permlane32_swap(uint32_t x, uint32_t y) {
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &x, 4);
  std::memcpy(w.slot[self] + 4, &y, 4);
  w.bar.arrive_and_wait();
  u32x2 r;
  uint32_t a, b;
  if (self < 32) {
    std::memcpy(&a, w.slot[self], 4);
    std::memcpy(&b, w.slot[self + 32], 4);
  } else {
    std::memcpy(&a, w.slot[self - 32] + 4, 4);
    std::memcpy(&b, w.slot[self] + 4, 4);
  }
  w.bar.arrive_and_wait();
  r[0] = a;
  r[1] = b;
  return r;
}

// ds_swizzle_b32 in bit mode (offset bit 15 clear): within each group of 32
// lanes, lane l reads lane ((l & and_mask) | or_mask) ^ xor_mask, with the
// masks in offset bits 4:0, 9:5 and 14:10
inline int ds_swizzle(int x, int offset) {
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &x, 4);
  w.bar.arrive_and_wait();
  const int am = offset & 31, om = (offset >> 5) & 31, xm = (offset >> 10) & 31;
  const int src = (self & ~31) | ((((self & 31) & am) | om) ^ xm);
  int r;
  std::memcpy(&r, w.slot[src], 4);
  w.bar.arrive_and_wait();
  return r;
}

inline void wave_sync() { ctx.wave->bar.arrive_and_wait(); }

// DPP move inside rows of 16 lanes, for the controls the kernels use:
// quad_perm (0x00-0xff: lane 4q + i reads lane 4q + sel_i), row_mirror
// (0x140: lane i of a row reads lane 15 - i) and row_half_mirror (0x141:
// lane i of each half row reads lane 7 - i). All rows and banks enabled.
inline int update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
  (void)old; (void)bound_ctrl;
  if (row_mask != 0xf || bank_mask != 0xf) std::abort();
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &src, 4);
  w.bar.arrive_and_wait();
  const int row = self & ~15, i = self & 15;
  int from;
  if (ctrl >= 0 && ctrl < 0x100) from = row + (i & ~3) + ((ctrl >> (2 * (i & 3))) & 3);
  else if (ctrl == 0x140) from = row + 15 - i;
  else if (ctrl == 0x141) from = row + (i & 8) + 7 - (i & 7);
  else std::abort();
  int r;
  std::memcpy(&r, w.slot[from], 4);
  w.bar.arrive_and_wait();
  return r;
}

inline int readlane(int x, int lane) {
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &x, 4);
  w.bar.arrive_and_wait();
  int r;
  std::memcpy(&r, w.slot[lane & 63], 4);
  w.bar.arrive_and_wait();
  return r;
}

inline int wave_any(int p) {
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &p, 4);
  w.bar.arrive_and_wait();
  int any = 0;
  for (int l = 0; l < 64; ++l) {
    int v;
    std::memcpy(&v, w.slot[l], 4);
    any |= (v != 0);
  }
  w.bar.arrive_and_wait();
  return any;
}

// v_cvt_pk_u8_f32 as measured on gfx950: round to nearest even, saturate to [0, 255]
inline uint32_t cvt_pk_u8_f32(float f, int byte, uint32_t old) {
  float r = std::nearbyint(f);
  r = std::isnan(r) ? 0.0f : std::fmin(255.0f, std::fmax(0.0f, r));
  const uint32_t v = static_cast<uint32_t>(r);
  return (old & ~(0xffu << (8 * byte))) | (v << (8 * byte));
}

// raw buffer resource: base address and size in bytes; loads at or past the
// end return 0 per dword, as the hardware's range check does for raw buffers
struct BufRsrc {
  const unsigned char* base;
  uint32_t n;
};
inline BufRsrc make_buffer_rsrc(const void* base, int n) { return {static_cast<const unsigned char*>(base), static_cast<uint32_t>(n)}; }
template <int NDW>
inline void buffer_load(const BufRsrc& r, uint32_t voff, uint32_t soff, uint32_t* out) {
  for (int i = 0; i < NDW; ++i) {
    const uint64_t off = static_cast<uint64_t>(voff) + soff + 4u * i;
    if (off + 4 <= r.n) std::memcpy(&out[i], r.base + off, 4);
    else out[i] = 0u;
  }
}
typedef int emu_v4i __attribute__((ext_vector_type(4)));
typedef int emu_v2i __attribute__((ext_vector_type(2)));
inline uint32_t raw_buffer_load_b32(const BufRsrc& r, uint32_t voff, uint32_t soff) {
  uint32_t v; buffer_load<1>(r, voff, soff, &v); return v;
}
inline emu_v2i raw_buffer_load_b64(const BufRsrc& r, uint32_t voff, uint32_t soff) {
  uint32_t v[2]; buffer_load<2>(r, voff, soff, v); emu_v2i o; std::memcpy(&o, v, 8); return o;
}
inline emu_v4i raw_buffer_load_b128(const BufRsrc& r, uint32_t voff, uint32_t soff) {
  uint32_t v[4]; buffer_load<4>(r, voff, soff, v); emu_v4i o; std::memcpy(&o, v, 16); return o;
}

// buffer load with an LDS destination, as measured on gfx950: lane l's
// `size` bytes (fetched like a register load, 0 past the end) are written to
// LDS at dst + size * l
inline void buffer_load_lds(const BufRsrc& r, void* dst, int size, uint32_t voff, uint32_t soff) {
  uint32_t v[4];
  const int ndw = size / 4;
  for (int i = 0; i < ndw; ++i) buffer_load<1>(r, voff + 4u * i, soff, &v[i]);
  std::memcpy(static_cast<unsigned char*>(dst) + static_cast<size_t>(size) * ctx.lane, v, size);
}

// ds_read_b64_tr_b8 as measured on gfx950: in each group of 16 lanes, lane i
// receives byte i % 8 of the 8-byte rows addressed by lanes 2 b + i / 8 of
// its group, b = 0..7 giving result byte b
inline emu_v2i ds_read_tr8_b64(const void* p) {
  Wave& w = *ctx.wave;
  const int self = ctx.lane;
  std::memcpy(w.slot[self], &p, sizeof(p));
  w.bar.arrive_and_wait();
  unsigned char out[8];
  const int grp = self & ~15, i = self & 15;
  for (int b = 0; b < 8; ++b) {
    const unsigned char* src;
    std::memcpy(&src, w.slot[grp + 2 * b + i / 8], sizeof(src));
    out[b] = src[i % 8];
  }
  w.bar.arrive_and_wait();
  emu_v2i r;
  std::memcpy(&r, out, 8);
  return r;
}

// v_med3_f32 for b <= c: the middle value; a NaN first operand gives b
inline float fmed3(float a, float b, float c) { return std::fmin(std::fmax(a, b), c); }

// v_dot4_i32_i8: signed byte products of a and b, plus c
inline int sdot4(int a, int b, int c) {
  for (int i = 0; i < 4; ++i)
    c += static_cast<int>(static_cast<int8_t>(a >> (8 * i))) * static_cast<int>(static_cast<int8_t>(b >> (8 * i)));
  return c;
}

// v_dot4_u32_u8: sum of the four byte products of a and b, plus c
inline uint32_t udot4(uint32_t a, uint32_t b, uint32_t c) {
  for (int i = 0; i < 4; ++i) c += ((a >> (8 * i)) & 0xffu) * ((b >> (8 * i)) & 0xffu);
  return c;
}

inline float bits_to_float(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
inline uint32_t float_to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

}  // namespace emu

#define threadIdx (emu::ctx.tid)
#define blockIdx (emu::ctx.bid)
#define gridDim (emu::g_grid)
#define blockDim (emu::g_block)
#define __syncthreads() emu::syncthreads()
#define __shfl_xor(...) emu::shfl_xor(__VA_ARGS__)
#define __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, x, y, z) emu::mfma_i8<32>(a, b, c)
#define __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, x, y, z) emu::mfma_i8<16>(a, b, c)
#define __builtin_amdgcn_perm(a, b, s) emu::perm(a, b, s)
#define __builtin_amdgcn_exp2f(x) std::exp2(static_cast<float>(x))
#define __builtin_amdgcn_permlane32_swap(x, y, fi, bc) emu::permlane32_swap(x, y)
#define __builtin_amdgcn_cvt_pk_u8_f32(f, b, old) emu::cvt_pk_u8_f32(f, b, old)
#define __builtin_amdgcn_fmed3f(a, b, c) emu::fmed3(a, b, c)
#define __builtin_amdgcn_udot4(a, b, c, clamp) emu::udot4(a, b, c)
#define __builtin_amdgcn_sdot4(a, b, c, clamp) emu::sdot4(a, b, c)
#define __any(p) emu::wave_any(p)
#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) emu::update_dpp(old, src, ctrl, rm, bm, bc)
#define __builtin_amdgcn_readlane(x, l) emu::readlane(x, l)
typedef emu::BufRsrc __amdgpu_buffer_rsrc_t;
// no register-allocation hints on the host
#define ATTN_WAVES_PER_EU(n)
#define __builtin_amdgcn_make_buffer_rsrc(base, stride, n, flags) emu::make_buffer_rsrc(base, n)
#define __builtin_amdgcn_raw_buffer_load_b32(r, v, s, aux) emu::raw_buffer_load_b32(r, v, s)
#define __builtin_amdgcn_raw_buffer_load_b64(r, v, s, aux) emu::raw_buffer_load_b64(r, v, s)
#define __builtin_amdgcn_raw_buffer_load_b128(r, v, s, aux) emu::raw_buffer_load_b128(r, v, s)
#define __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, size, v, s, off, aux) \
  emu::buffer_load_lds(r, (void*)(dst), size, (v) + (off), s)
#define __builtin_amdgcn_ds_read_tr8_b64_v2i32(p) emu::ds_read_tr8_b64((const void*)(p))
// s_waitcnt: the wavefront's lanes run in lockstep on the hardware, so the
// loads every lane issued before the wait (LDS-destination loads included)
// are complete for all of them after it; the emulated lanes meet here
#define __builtin_amdgcn_s_waitcnt(x) emu::wave_sync()
#define __builtin_amdgcn_wave_barrier() emu::wave_sync()
#define __builtin_amdgcn_ds_swizzle(x, off) emu::ds_swizzle(x, off)
#define __builtin_amdgcn_s_barrier() emu::syncthreads()
#define __builtin_amdgcn_sched_group_barrier(m, n, id) ((void)0)
#define __builtin_amdgcn_sched_barrier(m) ((void)0)
#define __builtin_amdgcn_s_setprio(p) ((void)0)
#define hipLaunchKernelGGL(K, G, B, S, ST, ...) emu::launch(G, B, [&]() { K(__VA_ARGS__); })

using std::max;
using std::min;

inline float __fmul_rn(float a, float b) { return a * b; }   // built with -ffp-contract=off
inline float __fadd_rn(float a, float b) { return a + b; }   // built with -ffp-contract=off
inline float __fsub_rn(float a, float b) { return a - b; }   // built with -ffp-contract=off
inline float __fdiv_rn(float a, float b) { return a / b; }
inline float __uint_as_float(uint32_t u) { return emu::bits_to_float(u); }
inline float __int_as_float(int i) { return emu::bits_to_float(static_cast<uint32_t>(i)); }
inline int __float_as_int(float f) { return static_cast<int>(emu::float_to_bits(f)); }
inline uint32_t __float_as_uint(float f) { return emu::float_to_bits(f); }
inline uint32_t atomicMax(uint32_t* p, uint32_t v) { return __atomic_fetch_max(p, v, __ATOMIC_RELAXED); }

struct __half { _Float16 v; };
struct alignas(4) __half2 { _Float16 x, y; };
inline float2 __half22float2(__half2 h) { return {static_cast<float>(h.x), static_cast<float>(h.y)}; }
inline __half __float2half_rn(float a) { return {static_cast<_Float16>(a)}; }
inline __half __ushort_as_half(unsigned short u) { __half h; std::memcpy(&h.v, &u, 2); return h; }
inline float __half2float(__half h) { return static_cast<float>(h.v); }
inline __half2 __floats2half2_rn(float a, float b) {
  return {static_cast<_Float16>(a), static_cast<_Float16>(b)};
}
