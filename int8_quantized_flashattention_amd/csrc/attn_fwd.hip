// Fused INT8 attention forward (prefill) for gfx950 / CDNA4.
//
// Method: "INT-FlashAttention: Enabling Flash Attention for INT8 Quantization"
// (abstract: FlashAttention forward with fully INT8 Q, K, V and per-token
// scales); integer logits, dequantization by s_Q s_K / sqrt(d) and the
// s_V P V_hat output form from "IntAttention: A Fully Integer Attention
// Pipeline for Efficient Edge Inference" §2.1 and §3.1 (Eq. 4); probabilities
// quantized as signed INT8 with multiplier 127 (IntAttention §3.2, the
// prior-methods scheme); tile-wise fused online softmax as in
// "FlashAttention-3" (abstract).
//
// Mapping onto CDNA4
// ------------------
// One workgroup = 4 wavefronts = kPrefillBM (128) query rows of one (b, h);
// each wavefront owns 32 rows. K/V stream through LDS in tiles of kPrefillBN
// (64) keys shared by the 4 wavefronts.
//
// Both products use v_mfma_i32_32x32x32_i8. The logits are computed
// transposed, S^T = K_hat . Q_hat^T, so that in the 32x32 INT32 result every
// lane holds 16 keys of ONE query (lane l: query l % 32, keys
// (v/4)*8 + (l/32)*4 + v%4 for accumulator v): row max and row sum need one
// cross-half step (v_permlane32_swap). The quantized probabilities of a lane
// are exactly the 16 int8 B-operand values of O^T = V_hat^T . P_hat^T for the
// same 32 keys, so P never leaves registers. V tiles are transposed while
// staged (4x4 byte transposes with v_perm) and stored in the key order the P
// operand implies, so each operand fetch is one 16-byte LDS read. O^T keeps
// the query in the lane, so the per-row rescale is lane-local.
//
// Instruction budget. On gfx950 the issue time of the VALU work per
// (query, key) pair is the first-order cost next to the pair's MFMA work, so
// per pair the kernel spends only: one INT32->fp32 convert, one multiply by
// s_K[j], half a v_max3, one fma for the base-2 exponent (127 folded in), one
// v_exp_f32, one add for the row sum and one v_cvt_pk_u8_f32 (round to
// nearest even, saturating) that quantizes P and packs it into the MFMA
// operand. Everything else is per tile or per workgroup:
//  - loads use raw buffer resources built once per workgroup: the tile offset
//    is the scalar offset, per-lane offsets never change, and out-of-range
//    keys read as zero in hardware (no compares, no 64-bit address math);
//  - for per-tensor V the P_hat . V_hat products keep accumulating in the
//    INT32 MFMA accumulator while no row of the wavefront raises its max and
//    are folded into the fp32 accumulator (which keeps its own frame, and
//    lives in LDS since only folds touch it) only when one does; s_V is
//    applied once in the epilogue;
//  - masking code runs only on diagonal / ragged tiles.
// Software pipeline: iteration t issues the MFMAs of QK(t+1) and PV(t-1)
// next to the VALU work of softmax(t) and of dequantizing S(t+1), so the
// matrix core works while the VALU computes probabilities. K stages are
// triple-buffered and V stages double-buffered; each tile has one barrier.
#include "attn_internal.h"

#include <hip/hip_fp16.h>

namespace attn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr int NKB = BN / 32;                 // 32-key blocks per tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBufWord3 = 0x00020000;        // raw buffer, 32-bit data format
// the INT32 run of P_hat . V_hat is folded into fp32 at least every this many
// tiles, keeping |sum| <= 127 * 127 * keys below 2^31
constexpr int kMaxIntTiles = 32768 / BN;
// re-base the fp32 accumulator when the running max has grown by this much
// (base 2) since its frame was set
constexpr float kRebase = 60.0f;
// relative guard on the softmax bias (see the tile loop)
constexpr float kBiasGuard = 4.76837158203125e-07f;   // 2^-21

template <int D>
struct Geo {
  static constexpr int KSTR = D + 16;             // LDS bytes per K row (padding spreads banks)
  static constexpr int VSTR = BN + 16;            // LDS bytes per V^T row
  static constexpr int NC = D / 32;               // 32-channel chunks of the head dim
  static constexpr int KPT = BN * D / 16 / kThreads;            // 16-byte K chunks per thread
  static constexpr int VITEMS = (D / 4) * (BN / 8);             // (channel quad, key octet) items
  static constexpr int VPT_ITEMS = (VITEMS + kThreads - 1) / kThreads;
};

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16i zero16() { return v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Transpose a 4x4 byte block: r[i] holds bytes (row i, cols 0..3); returns
// c[j] holding bytes (rows 0..3, col j).
__device__ __forceinline__ void transpose4x4(const uint32_t* r, uint32_t* c) {
  const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  const uint32_t hi01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);  // r0b0 r1b0 r2b0 r3b0
  c[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// K stage: K rows (padded), per-key s_K, per-token V scales and the partial
// maxima of those scales (one per wavefront that loaded them).
struct KStage {
  alignas(16) int8_t k[BN * (128 + 16)];
  alignas(16) float sk[BN];
  alignas(16) float sv[BN];
  float stp[BN / 64];
};
// V stage: V^T rows (one per channel, padded), keys in P-operand order.
struct VStage {
  alignas(16) int8_t vt[128 * (BN + 16)];
};
// K and V stages are double-buffered: a stage is rewritten one barrier after
// its last read.
struct Smem {
  KStage ks[2];
  VStage vs[2];
};

struct Bufs {
  __amdgpu_buffer_rsrc_t k, v, sk, sv;
};

// Per-thread load/store offsets (fixed for the whole kernel).
template <int D>
struct Map {
  using G = Geo<D>;
  uint32_t k_src[G::KPT];        // byte offset of a 16-byte K chunk within a tile
  int k_dst[G::KPT];             // its LDS offset within the K stage
  uint32_t v_src[G::VPT_ITEMS];  // byte offset of key0's channel quad within a tile
  int v_dst[G::VPT_ITEMS];       // LDS offset of row 4*dq, 8-byte slot of the key octet
  bool v_live[G::VPT_ITEMS];

  __device__ __forceinline__ void init(int tid) {
#pragma unroll
    for (int i = 0; i < G::KPT; ++i) {
      const int id = tid + i * kThreads;
      const int row = id / (D / 16), cc = id % (D / 16);
      k_src[i] = static_cast<uint32_t>(row * D + cc * 16);
      k_dst[i] = row * G::KSTR + cc * 16;
    }
    // a wavefront takes 8 channel quads x 8 key octets, so its 8-byte LDS
    // writes spread over all banks
#pragma unroll
    for (int i = 0; i < G::VPT_ITEMS; ++i) {
      const int item = tid + i * kThreads;
      v_live[i] = item < G::VITEMS;
      const int wc = item / 64, l = item % 64;
      const int dq = (wc % (D / 32)) * 8 + (l % 8);
      const int ko = (wc / (D / 32)) * 8 + (l / 8);
      const int kb = ko / 4, gq = (ko % 4) / 2, hh = ko % 2;
      const int key0 = kb * 32 + 16 * hh + 4 * gq;     // keys key0..+3 and key0+8..+11
      v_src[i] = static_cast<uint32_t>(key0 * D + dq * 4);
      v_dst[i] = (dq * 4) * G::VSTR + kb * 32 + gq * 16 + 8 * hh;
    }
  }
};

// Next tiles' data between their global loads and their LDS stores.
template <int D>
struct KRegs {
  v4i k[Geo<D>::KPT];
  float sk, sv;
};
template <int D>
struct VRegs {
  uint32_t v[Geo<D>::VPT_ITEMS][8];
};

// SCALES: also load s_K (and, for per-token V, s_V); the logits-only kernel
// has no scale pointers and must not touch them.
template <int D, bool SCALES, bool VPT>
__device__ __forceinline__ void load_k(KRegs<D>& r, const Bufs& bf, const Map<D>& mp, int k0) {
  const int tid = threadIdx.x;
  const uint32_t soff = static_cast<uint32_t>(k0) * D;
#pragma unroll
  for (int i = 0; i < Geo<D>::KPT; ++i) r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(bf.k, mp.k_src[i], soff, 0);
  r.sk = 0.0f;
  r.sv = 0.0f;
  if constexpr (SCALES) {
    if (tid < BN) r.sk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bf.sk, tid * 4, k0 * 4, 0));
    if (VPT && tid >= kThreads - BN)
      r.sv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bf.sv, (tid - (kThreads - BN)) * 4, k0 * 4, 0));
  }
}

template <int D>
__device__ __forceinline__ void load_v(VRegs<D>& r, const Bufs& bf, const Map<D>& mp, int k0) {
  const uint32_t soff = static_cast<uint32_t>(k0) * D;
#pragma unroll
  for (int it = 0; it < Geo<D>::VPT_ITEMS; ++it) {
    if (!mp.v_live[it]) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[it][i] = __builtin_amdgcn_raw_buffer_load_b32(bf.v, mp.v_src[it] + i * D, soff, 0);
      r.v[it][4 + i] = __builtin_amdgcn_raw_buffer_load_b32(bf.v, mp.v_src[it] + (8 + i) * D, soff, 0);
    }
  }
}

template <int D, bool SCALES, bool VPT>
__device__ __forceinline__ void store_k(KStage& s, const KRegs<D>& r, const Map<D>& mp) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Geo<D>::KPT; ++i) *reinterpret_cast<v4i*>(s.k + mp.k_dst[i]) = r.k[i];
  if constexpr (SCALES) {
    if (tid < BN) s.sk[tid] = r.sk;
    if (VPT && tid >= kThreads - BN) {
      const int j = tid - (kThreads - BN);
      s.sv[j] = r.sv;
      float st = r.sv;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) st = fmaxf(st, __shfl_xor(st, off, 64));
      if ((j & 63) == 0) s.stp[j >> 6] = st;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_v(VStage& s, const VRegs<D>& r, const Map<D>& mp) {
  using G = Geo<D>;
#pragma unroll
  for (int it = 0; it < G::VPT_ITEMS; ++it) {
    if (!mp.v_live[it]) continue;
    uint32_t lo[4], hi[4];
    transpose4x4(&r.v[it][0], lo);
    transpose4x4(&r.v[it][4], hi);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint2*>(s.vt + mp.v_dst[it] + j * G::VSTR) = make_uint2(lo[j], hi[j]);
  }
}

// Scheduling hint for the straight-line block just emitted: alternate one
// MFMA with N_VALU VALU instructions, NM times, so the matrix core works
// while the VALU does the softmax arithmetic.
template <int NM, int N_VALU>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, N_VALU, 0);   // VALU
  }
}

// S^T for one tile: exact INT32 logits, 32 keys per block (shared with the
// logits-dump kernel).
template <int D>
__device__ __forceinline__ void qk_tile(v16i (&s)[NKB], const KStage& ks, const v4i (&qf)[D / 32], int lr, int g) {
  using G = Geo<D>;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
  for (int c = 0; c < G::NC; ++c)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const v4i ka = *reinterpret_cast<const v4i*>(ks.k + (kb * 32 + lr) * G::KSTR + c * 32 + g * 16);
      s[kb] = mfma_i8(ka, qf[c], s[kb]);
    }
}

// O^T contribution of one tile: acc[c] += V_hat^T . P_hat^T.
template <int D>
__device__ __forceinline__ void pv_tile(v16i (&acc)[D / 32], const VStage& vs, const v4i (&pv)[NKB], int lr, int g) {
  using G = Geo<D>;
#pragma unroll
  for (int c = 0; c < G::NC; ++c)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const v4i va = *reinterpret_cast<const v4i*>(vs.vt + (c * 32 + lr) * G::VSTR + kb * 32 + g * 16);
      acc[c] = mfma_i8(va, pv[kb], acc[c]);
    }
}

// u = S_int * s_K[j] for this lane's keys (the query's factor c2 comes
// later); masked keys get -inf. rel = (last visible key of the row) - k0 -
// 4 g, so key index j of the tile is visible iff (j - 4 g) <= rel, a compare
// of a compile-time constant with one per-lane value. Returns the max over
// the lane pair.
template <bool MASK>
__device__ __forceinline__ float dequant_tile(const v16i (&s)[NKB], const KStage& ks, float (&u)[NKB][16], int rel,
                                              int g) {
  // the maximum is taken as a tree (independent partial maxima), so a single
  // wavefront per SIMD is not held up by a long dependency chain
  float gm[NKB * 4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int jl = kb * 32 + j4 * 8 + g * 4;
      const float4 skv = *reinterpret_cast<const float4*>(ks.sk + jl);
      const float skk[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = static_cast<float>(s[kb][j4 * 4 + e]) * skk[e];
        if constexpr (MASK) x = (kb * 32 + j4 * 8 + e <= rel) ? x : kNegInf;
        u[kb][j4 * 4 + e] = x;
      }
      const float* x = &u[kb][j4 * 4];
      gm[kb * 4 + j4] = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    }
#pragma unroll
  for (int w = NKB * 4; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) gm[i] = fmaxf(gm[i], gm[i + w / 2]);
  const float mx = gm[0];
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// y = exp2(u c2 - bias) = 127 P_tilde; returns this lane's sum of y and packs
// P_hat = rne(y) (per-token V: rne(y s_V[j] / s_t)) into the PV operands.
template <bool VPT, bool MASK>
__device__ __forceinline__ float probs_tile(const float (&u)[NKB][16], float c2, float bias, const KStage& ks,
                                            float rst, v4i (&pv)[NKB], int g) {
  float gs[NKB * 4];                   // partial row sums, added as a tree
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    uint32_t pw[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float wr[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (VPT) {
        const float4 sv = *reinterpret_cast<const float4*>(ks.sv + kb * 32 + j4 * 8 + g * 4);
        wr[0] = sv.x * rst; wr[1] = sv.y * rst; wr[2] = sv.z * rst; wr[3] = sv.w * rst;
      }
      uint32_t word = 0;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float uu = u[kb][j4 * 4 + e];
        y[e] = exp2_hw(__builtin_fmaf(uu, c2, -bias));
        if constexpr (MASK) y[e] = (uu == kNegInf) ? 0.0f : y[e];
        word = __builtin_amdgcn_cvt_pk_u8_f32(VPT ? y[e] * wr[e] : y[e], e, word);
      }
      gs[kb * 4 + j4] = (y[0] + y[1]) + (y[2] + y[3]);
      pw[j4] = word;
    }
    pv[kb] = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]), static_cast<int>(pw[3])};
  }
#pragma unroll
  for (int w = NKB * 4; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) gs[i] += gs[i + w / 2];
  return gs[0];
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ Bufs make_bufs(const FwdArgs& a, int64_t kv_base, int D, bool scales, bool vpt) {
  Bufs bf;
  bf.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.k + kv_base * D), 0, a.Lkv * D, kBufWord3);
  bf.v = bf.k;
  bf.sk = bf.k;
  bf.sv = bf.k;
  if (scales) {
    bf.v = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.v + kv_base * D), 0, a.Lkv * D, kBufWord3);
    bf.sk = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.s_k + kv_base), 0, a.Lkv * 4, kBufWord3);
    if (vpt) bf.sv = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.s_v + kv_base), 0, a.Lkv * 4, kBufWord3);
  }
  return bf;
}

// Workgroup -> (b*h, row block). Workgroups are dealt to the 8 XCDs round
// robin, so consecutive ids land on different XCDs (each with its own L2);
// the id is re-numbered so that each XCD walks whole heads, row blocks of a
// head back to back (longest causal block first). The workgroups resident on
// one XCD then share the K/V of two or three heads.
__device__ __forceinline__ void tile_of_block(int n_rb, int& bh, int& rb) {
  const int n = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int w = xcd * (n >> 3) + min(xcd, n & 7) + slot;
  bh = w / n_rb;
  rb = n_rb - 1 - (w - bh * n_rb);
}

template <int D, bool CAUSAL, bool VPT, bool OUT_F16>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a) {
  using G = Geo<D>;
  __shared__ Smem sm;

  const int n_rb = (a.Lq + BM - 1) / BM;
  int bh, rb;
  tile_of_block(n_rb, bh, rb);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / (a.H / a.Hkv);
  const int64_t kv_base = (static_cast<int64_t>(b) * a.Hkv + hk) * a.Lkv;
  const int64_t q_base = static_cast<int64_t>(bh) * a.Lq;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets tile decisions be scalar
  const int lane = tid & 63;
  const int g = lane >> 5;          // which 16 keys / channels of a 32-block this lane holds
  const int lr = lane & 31;         // query row within the wavefront
  const int qw0 = rb * BM + wave * 32;
  const int qi = qw0 + lr;
  const bool qvalid = qi < a.Lq;
  const int shift = a.Lkv - a.Lq;   // bottom-right causal alignment

  const Bufs bf = make_bufs(a, kv_base, D, true, VPT);
  Map<D> mp;
  mp.init(tid);

  // Q fragment (B operand of S^T): 16 bytes per 32-channel chunk.
  v4i qf[G::NC];
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    qf[c] = v4i{0, 0, 0, 0};
    if (qvalid) qf[c] = *reinterpret_cast<const v4i*>(a.q + (q_base + qi) * D + c * 32 + g * 16);
  }
  const float sq = qvalid ? a.s_q[q_base + qi] : 0.0f;
  const float inv_sqrt_d = (D == 64) ? 0.125f : static_cast<float>(0.08838834764831845);
  const float c2 = sq * inv_sqrt_d * kLog2e;          // base-2 logit per unit of S_int * s_K
  const int lim = CAUSAL ? qi + shift : a.Lkv - 1;    // last visible key of this row
  const int lim_first = CAUSAL ? qw0 + shift : a.Lkv - 1;   // smallest in the wavefront

  const int last_q = min(rb * BM + BM - 1, a.Lq - 1);
  const int kv_end = CAUSAL ? min(a.Lkv, last_q + shift + 1) : a.Lkv;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // softmax state: running max (base 2), partial sum of 127 P_tilde over this lane's keys
  float m = kNegInf, l = 0.0f;
  float acc[G::NC][16];                // fp32 O^T accumulator
  v16i acc_i[G::NC];                   // INT32 accumulation of P_hat . V_hat
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    acc_i[c] = zero16();
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  }
  float m_f = kNegInf;                 // frame of acc (per-tensor V)
  int int_tiles = 0;                   // tiles in the current INT32 run

  // ---- prologue: K(0), V(0) staged ----
  KRegs<D> kx;
  VRegs<D> vx;
  load_k<D, true, VPT>(kx, bf, mp, 0);
  load_v<D>(vx, bf, mp, 0);
  store_k<D, true, VPT>(sm.ks[0], kx, mp);
  store_v<D>(sm.vs[0], vx, mp);
  __syncthreads();

  // One tile: QK(t) [MFMA] | dequant, softmax(t) [VALU] | fold | PV(t)
  // [MFMA] | stage K(t+1), V(t+1) | barrier. The wavefront of the other
  // workgroup on the same SIMD issues its VALU work while this one waits on
  // the matrix core, and the other way round.
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN;
    const KStage& ks_cur = sm.ks[t & 1];
    const bool more = t + 1 < n_tiles;
    // global loads of the next tile, in flight during this tile's math
    if (more) {
      load_k<D, true, VPT>(kx, bf, mp, k0 + BN);
      load_v<D>(vx, bf, mp, k0 + BN);
    }
    v16i s[NKB];
    qk_tile<D>(s, ks_cur, qf, lr, g);
    const bool mask = (k0 + BN > a.Lkv) || (CAUSAL && k0 + BN - 1 > lim_first);
    // key index j of the tile is visible iff j - 4 g <= rel
    const int rel = mask ? min(lim, a.Lkv - 1) - k0 - 4 * g : BN;
    float u[NKB][16];
    const float mx = dequant_tile<true>(s, ks_cur, u, rel, g);

    // ---- softmax(t): running max, 127 P_tilde, row sum, P_hat ----
    const float mx2 = (mx == kNegInf) ? kNegInf : mx * c2;   // c2 >= 0: max(u) c2 == max(u c2)
    const float m_new = fmaxf(m, mx2);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = exp2_hw(m - m_use);            // 1 if unchanged, 0 on the first tile
    // exp2(u c2 - bias) = 127 P_tilde. The guard term |m| 2^-21 keeps the
    // max key's value below 127.5 however large |m| is (the fp32 rounding of
    // u c2 and of the bias grows with |m|); P_hat and the row sum scale
    // together, so it cancels in O.
    const float bias = __builtin_fmaf(fabsf(m_use), kBiasGuard, m_use - kLog2_127);
    float rst = 0.0f, st_cur = 0.0f;
    if constexpr (VPT) {
      st_cur = ks_cur.stp[0];
#pragma unroll
      for (int i = 1; i < BN / 64; ++i) st_cur = fmaxf(st_cur, ks_cur.stp[i]);
      rst = st_cur > 0.0f ? 1.0f / st_cur : 0.0f;
    }
    v4i p[NKB];
    const float lsum = probs_tile<VPT, true>(u, c2, bias, ks_cur, rst, p, g);
    l = alpha * l + lsum;

    if constexpr (!VPT) {
      if (__any(m_new > m) || ++int_tiles > kMaxIntTiles) {
        // tile t raised some row's max: the INT32 run (tiles before t, frame
        // m) goes into acc (frame m_f) before PV(t) starts a new run
        if (m_f == kNegInf) m_f = m_use;
        float f = exp2_hw(m - m_f);                   // 0 before the first tile
        float r = 1.0f;
        if (__any(m_use - m_f > kRebase)) {           // keep acc far from overflow
          r = exp2_hw(m_f - m_use);
          f *= r;
          m_f = m_use;
        }
#pragma unroll
        for (int c = 0; c < G::NC; ++c) {
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[c][v] = __builtin_fmaf(f, static_cast<float>(acc_i[c][v]), acc[c][v] * r);
          acc_i[c] = zero16();
        }
        int_tiles = 1;
      }
    } else {
#pragma unroll
      for (int c = 0; c < G::NC; ++c) acc_i[c] = zero16();
    }
    m = m_new;

    pv_tile<D>(acc_i, sm.vs[t & 1], p, lr, g);
    if constexpr (VPT) {
      // per-token V: tile scales differ, so each tile's INT32 product is
      // converted on its own: acc = alpha acc + s_t PV(t)
#pragma unroll
      for (int c = 0; c < G::NC; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[c][v] = __builtin_fmaf(alpha, acc[c][v], st_cur * static_cast<float>(acc_i[c][v]));
    }

    // ---- stage K(t+1), V(t+1) ----
    if (more) {
      store_k<D, true, VPT>(sm.ks[(t + 1) & 1], kx, mp);
      store_v<D>(sm.vs[(t + 1) & 1], vx, mp);
    }
    __syncthreads();
  }

  if constexpr (!VPT) {
    // total in the frame of the final max m: 2^(m_f - m) acc + INT32 run
    const float back = exp2_hw(m_f - m);
#pragma unroll
    for (int c = 0; c < G::NC; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = __builtin_fmaf(back, acc[c][v], static_cast<float>(acc_i[c][v]));
  }

  const float ltot = pair_sum(l);                      // 127 * l
  if (!qvalid) return;
  const float scale = (VPT ? 1.0f : a.s_v[0]) / ltot;
  const int64_t orow = (q_base + qi) * D;
#pragma unroll
  for (int c = 0; c < G::NC; ++c)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = c * 32 + j4 * 8 + g * 4;
      const float o0 = acc[c][j4 * 4 + 0] * scale, o1 = acc[c][j4 * 4 + 1] * scale;
      const float o2 = acc[c][j4 * 4 + 2] * scale, o3 = acc[c][j4 * 4 + 3] * scale;
      if constexpr (OUT_F16) {
        const __half2 h01 = __floats2half2_rn(o0, o1);
        const __half2 h23 = __floats2half2_rn(o2, o3);
        uint2 pk;
        pk.x = *reinterpret_cast<const uint32_t*>(&h01);
        pk.y = *reinterpret_cast<const uint32_t*>(&h23);
        *reinterpret_cast<uint2*>(static_cast<__half*>(a.o) + orow + d0) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow + d0) = make_float4(o0, o1, o2, o3);
      }
    }
  if (a.lse && g == 0) a.lse[q_base + qi] = (m + __builtin_log2f(ltot) - kLog2_127) * kLn2;
}

// Logits dump: the same K staging and Q.K^T tile code as the forward, writing
// the exact INT32 logit of every visible pair.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_logits_kernel(FwdArgs a) {
  __shared__ KStage ks;
  const int bh = blockIdx.x;
  const int rb = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / (a.H / a.Hkv);
  const int64_t kv_base = (static_cast<int64_t>(b) * a.Hkv + hk) * a.Lkv;
  const int64_t q_base = static_cast<int64_t>(bh) * a.Lq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 5, lr = lane & 31;
  const int qi = rb * BM + (tid >> 6) * 32 + lr;
  const bool qvalid = qi < a.Lq;
  const int lim = CAUSAL ? qi + (a.Lkv - a.Lq) : a.Lkv - 1;
  const Bufs bf = make_bufs(a, kv_base, D, false, false);
  Map<D> mp;
  mp.init(tid);
  v4i qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    qf[c] = v4i{0, 0, 0, 0};
    if (qvalid) qf[c] = *reinterpret_cast<const v4i*>(a.q + (q_base + qi) * D + c * 32 + g * 16);
  }
  const int last_q = min(rb * BM + BM - 1, a.Lq - 1);
  const int kv_end = CAUSAL ? min(a.Lkv, last_q + (a.Lkv - a.Lq) + 1) : a.Lkv;
  for (int k0 = 0; k0 < kv_end; k0 += BN) {
    KRegs<D> kx;
    load_k<D, false, false>(kx, bf, mp, k0);
    __syncthreads();
    store_k<D, false, false>(ks, kx, mp);
    __syncthreads();
    v16i s[NKB];
    qk_tile<D>(s, ks, qf, lr, g);
    if (qvalid) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          if (key < a.Lkv && key <= lim) a.s_dump[(q_base + qi) * a.Lkv + key] = s[kb][v];
        }
    }
  }
}

template <int D, bool CAUSAL, bool VPT, bool OUT_F16>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * n_rb));
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VPT, OUT_F16>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_vo(const FwdArgs& a, hipStream_t st) {
  if (a.v_per_token)
    return a.o_f16 ? launch_t<D, CAUSAL, true, true>(a, st) : launch_t<D, CAUSAL, true, false>(a, st);
  return a.o_f16 ? launch_t<D, CAUSAL, false, true>(a, st) : launch_t<D, CAUSAL, false, false>(a, st);
}

template <int D, bool CAUSAL>
hipError_t launch_logits_t(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>(n_rb));
  hipLaunchKernelGGL((attn_logits_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, hipStream_t st) {
  if (a.d == 64) return a.causal ? launch_vo<64, true>(a, st) : launch_vo<64, false>(a, st);
  return a.causal ? launch_vo<128, true>(a, st) : launch_vo<128, false>(a, st);
}

hipError_t launch_debug_logits(const FwdArgs& a, hipStream_t st) {
  if (a.d == 64) return a.causal ? launch_logits_t<64, true>(a, st) : launch_logits_t<64, false>(a, st);
  return a.causal ? launch_logits_t<128, true>(a, st) : launch_logits_t<128, false>(a, st);
}

}  // namespace attn
