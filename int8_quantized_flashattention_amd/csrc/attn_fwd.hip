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
// each wavefront owns 32 rows. K/V are streamed in tiles of kPrefillBN (64)
// keys through LDS and shared by the 4 wavefronts.
//
// Both products use v_mfma_i32_32x32x32_i8 (32x32 output, K = 32 int8 per
// step, 16 int8 per lane per operand). The logits are computed transposed,
// S^T = K_hat . Q_hat^T, so that in the 32x32 INT32 result every lane holds
// 16 keys of ONE query (lane l: query l % 32, keys (v/4)*8 + (l/32)*4 + v%4
// for accumulator v). The softmax statistics of a query therefore live in one
// lane pair (l, l ^ 32): row max and row sum need a single cross-half step.
// The quantized probabilities P_hat of a lane are exactly the 16 int8 B-operand
// values of O^T = V_hat^T . P_hat^T for the same 32-key block, so P never
// leaves registers. The A operand V_hat^T needs, per lane, 16 keys of one
// head-dim channel: V tiles are transposed while they are staged into LDS
// (4x4 byte transposes with v_perm) and stored with the key order the P
// operand implies, so each operand fetch is one 16-byte LDS read.
// The output accumulator O^T keeps the query in the lane too, so the
// per-row rescale alpha is lane-local.
//
// Pipeline per KV tile: the next tile's global loads are issued before the
// current tile's math and written to the other of two LDS stages after it,
// so there is one barrier per tile. The softmax works in base 2 with 127
// folded into the exponent: y = exp2(u c2 - m + log2 127) = 127 P_tilde, the
// row sum accumulates y, and v_cvt_pk_u8_f32 (round to nearest even,
// saturating) turns y into P_hat and packs it into the operand in one step.
// For per-tensor V the P_hat . V_hat products keep accumulating in the INT32
// MFMA accumulator while no row of the wavefront raises its max (alpha = 1),
// and are converted to fp32 (and the older fp32 part rescaled) only when one
// does; s_V is applied once in the epilogue.
#include "attn_internal.h"

#include <hip/hip_fp16.h>

namespace attn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

template <int D>
struct Geo {
  static constexpr int KSTR = D + 16;     // LDS bytes per K row (padding breaks bank aliasing)
  static constexpr int VSTR = BN + 16;    // LDS bytes per V^T row
  static constexpr int NC = D / 32;       // 32-channel chunks of the head dim
};

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Transpose a 4x4 byte block: r[i] holds bytes (row i, cols 0..3); returns
// c[j] holding bytes (rows 0..3, col j).
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t c[4]) {
  // interleave rows 0/1 and 2/3 byte-wise
  const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
  const uint32_t hi01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
  const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);  // r0b0 r1b0 r2b0 r3b0
  c[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);  // r0b1 r1b1 r2b1 r3b1
  c[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Position of tile-local key j inside a V^T LDS row: the 16 keys that one lane
// half (g) contributes to a 32-key MFMA step are stored contiguously, in the
// order of that lane's logit accumulators.
__device__ __forceinline__ int vt_pos(int j) {
  const int kb = j >> 5, r = j & 31;
  return kb * 32 + ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// One LDS stage of a KV tile. Two of them alternate: while the wavefronts
// compute on one, the next tile (already loaded into registers) is written to
// the other.
struct Stage {
  alignas(16) int8_t k[BN * (128 + 16)];   // K rows, padded
  alignas(16) int8_t vt[128 * (BN + 16)];  // V^T rows (one per channel), padded
  alignas(16) float sk[BN];                // s_K of the tile's keys
  alignas(16) float wr[BN];                // per-token V: s_V[j] / s_t
  float st;                                // per-token V: s_t, the largest s_V of the tile
};
struct Smem {
  Stage stage[2];
};

// The next tile held in registers between its global loads and its LDS store.
template <int D>
struct TileRegs {
  static constexpr int kCPR = D / 16;                 // 16-byte chunks per K row
  static constexpr int kKIters = BN * kCPR / kThreads;
  static constexpr int kNDQ = D / 4;                  // channel quads
  static constexpr int kKQPerIter = kThreads / kNDQ;  // key quads per pass
  static constexpr int kVIters = (BN / 4) / kKQPerIter;
  v4i k[kKIters];
  uint32_t v[kVIters][4];
  float sk;
  float sv;
};

// Global loads of tile k0 (out-of-range keys read as zero). The logits-only
// variant is given no V or scale pointers and must not touch them.
template <int D, bool VPT, bool LOGITS_ONLY>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const FwdArgs& a, int64_t kv_base, int k0) {
  using R = TileRegs<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < R::kKIters; ++it) {
    const int id = tid + it * kThreads;
    const int row = id / R::kCPR, cc = id % R::kCPR;
    r.k[it] = v4i{0, 0, 0, 0};
    if (k0 + row < a.Lkv) r.k[it] = *reinterpret_cast<const v4i*>(a.k + (kv_base + k0 + row) * D + cc * 16);
  }
  if constexpr (LOGITS_ONLY) return;
  const int dq = tid % R::kNDQ;
#pragma unroll
  for (int it = 0; it < R::kVIters; ++it) {
    const int kq = tid / R::kNDQ + it * R::kKQPerIter;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + kq * 4 + i;
      r.v[it][i] = (key < a.Lkv) ? *reinterpret_cast<const uint32_t*>(a.v + (kv_base + key) * D + dq * 4) : 0u;
    }
  }
  r.sk = 0.0f;
  r.sv = 0.0f;
  if (tid < BN) {
    if (k0 + tid < a.Lkv) r.sk = a.s_k[kv_base + k0 + tid];
  } else if (VPT && tid < 2 * BN) {
    if (k0 + tid - BN < a.Lkv) r.sv = a.s_v[kv_base + k0 + tid - BN];
  }
}

// LDS store of a tile held in registers: K rows as they are, V transposed
// into V^T in the key order of the P operand, the per-key scales, and for
// per-token V the tile scale s_t and the ratios s_V[j] / s_t.
template <int D, bool VPT, bool LOGITS_ONLY>
__device__ __forceinline__ void store_tile(Stage& sg, const TileRegs<D>& r) {
  using R = TileRegs<D>;
  using G = Geo<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < R::kKIters; ++it) {
    const int id = tid + it * kThreads;
    const int row = id / R::kCPR, cc = id % R::kCPR;
    *reinterpret_cast<v4i*>(sg.k + row * G::KSTR + cc * 16) = r.k[it];
  }
  if constexpr (LOGITS_ONLY) return;
  const int dq = tid % R::kNDQ;
#pragma unroll
  for (int it = 0; it < R::kVIters; ++it) {
    const int kq = tid / R::kNDQ + it * R::kKQPerIter;
    uint32_t c[4];
    transpose4x4(r.v[it], c);
    const int pos = vt_pos(kq * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(sg.vt + (dq * 4 + j) * G::VSTR + pos) = c[j];
  }
  if (tid < BN) {
    sg.sk[tid] = r.sk;
  } else if (VPT && tid < 2 * BN) {
    // one wavefront (threads BN..2BN-1) reduces the tile's largest V scale
    float st = r.sv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) st = fmaxf(st, __shfl_xor(st, off, 64));
    sg.wr[tid - BN] = (st > 0.0f) ? __fdiv_rn(r.sv, st) : 0.0f;
    if (tid == BN) sg.st = st;
  }
}

// max / sum of a value over the lane pair (l, l ^ 32) that holds one query
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// INT8 P_hat . V_hat for one tile: acc[c] (+)= sum over the 32-key blocks.
template <int D, bool FROM_ZERO>
__device__ __forceinline__ void pv_tile(v16i (&acc)[D / 32], const Stage& sg, const v4i (&pv)[BN / 32], int lr, int g) {
  using G = Geo<D>;
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    v16i t = FROM_ZERO ? v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0} : acc[c];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      const v4i va = *reinterpret_cast<const v4i*>(sg.vt + (c * 32 + lr) * G::VSTR + kb * 32 + g * 16);
      t = mfma_i8(va, pv[kb], t);
    }
    acc[c] = t;
  }
}

// u = S_int * s_K[j] for this lane's keys of the tile (the query's factor c2
// is applied later); masked keys get -inf. Returns the lane's max of u.
template <int D, bool MASK>
__device__ __forceinline__ float dequant_tile(const v16i (&s)[BN / 32], const Stage& sg, float (&u)[BN / 32][16],
                                              int k0, int lim, int Lkv, int g) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int jl = kb * 32 + j4 * 8 + g * 4;
      const float4 skv = *reinterpret_cast<const float4*>(sg.sk + jl);
      const float skk[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = static_cast<float>(s[kb][j4 * 4 + e]) * skk[e];
        if constexpr (MASK) {
          const int key = k0 + jl + e;
          x = (key < Lkv && key <= lim) ? x : kNegInf;
        }
        u[kb][j4 * 4 + e] = x;
        mx = fmaxf(mx, x);
      }
    }
  return mx;
}

// y = exp2(u c2 - bias) = 127 P_tilde; returns the lane's sum of y and packs
// P_hat = rne(y) (per-token V: rne(y s_V[j] / s_t)) into the PV operands.
// CLAMP: when the running max is so large (|m| >= 2^15 in base-2 units) that
// the fp32 rounding of the exponent argument could push the max key's y past
// 127.5, y is clamped to 127 (the value the max key has exactly).
template <bool VPT, bool MASK, bool CLAMP>
__device__ __forceinline__ float probs_tile(const float (&u)[BN / 32][16], float c2, float bias, const Stage& sg,
                                            v4i (&pv)[BN / 32], int g) {
  float lsum = 0.0f;
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb) {
    uint32_t pw[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float wr[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (VPT) {
        const float4 wv = *reinterpret_cast<const float4*>(sg.wr + kb * 32 + j4 * 8 + g * 4);
        wr[0] = wv.x; wr[1] = wv.y; wr[2] = wv.z; wr[3] = wv.w;
      }
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float uu = u[kb][j4 * 4 + e];
        float y = exp2_hw(__builtin_fmaf(uu, c2, -bias));
        if constexpr (MASK) y = (uu == kNegInf) ? 0.0f : y;
        if constexpr (CLAMP) y = fminf(y, 127.0f);
        lsum += y;
        word = __builtin_amdgcn_cvt_pk_u8_f32(VPT ? y * wr[e] : y, e, word);
      }
      pw[j4] = word;
    }
    pv[kb] = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]), static_cast<int>(pw[3])};
  }
  return lsum;
}

constexpr float kLog2_127 = 6.988684686772166f;
// the INT32 run of P_hat . V_hat is converted to fp32 at least every this many
// tiles, keeping |sum| <= 127 * 127 * keys below 2^31
constexpr int kMaxIntTiles = 32768 / BN;
// re-base the fp32 accumulator when the running max has grown by this much
// (base 2) since its frame was set
constexpr float kRebase = 60.0f;

template <int D, bool CAUSAL, bool VPT, bool OUT_F16, bool DUMP>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdArgs a) {
  using G = Geo<D>;
  __shared__ Smem sm;

  const int bh = blockIdx.x;
  const int rb = gridDim.y - 1 - blockIdx.y;          // longest (causal) row blocks first
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / (a.H / a.Hkv);
  const int64_t kv_base = (static_cast<int64_t>(b) * a.Hkv + hk) * a.Lkv;
  const int64_t q_base = static_cast<int64_t>(bh) * a.Lq;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;          // which 16 keys / channels of a 32-block this lane holds
  const int lr = lane & 31;         // query row within the wavefront
  const int qw0 = rb * BM + wave * 32;
  const int qi = qw0 + lr;
  const bool qvalid = qi < a.Lq;
  const bool wave_live = qw0 < a.Lq;
  const int shift = a.Lkv - a.Lq;   // bottom-right causal alignment

  // Q fragment (B operand of S^T): 16 bytes per 32-channel chunk.
  v4i qf[G::NC];
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    qf[c] = v4i{0, 0, 0, 0};
    if (qvalid) qf[c] = *reinterpret_cast<const v4i*>(a.q + (q_base + qi) * D + c * 32 + g * 16);
  }
  const float sq = (qvalid && !DUMP) ? a.s_q[q_base + qi] : 0.0f;
  const float inv_sqrt_d = (D == 64) ? 0.125f : static_cast<float>(0.08838834764831845);
  const float c2 = sq * inv_sqrt_d * kLog2e;          // base-2 logit per unit of S_int * s_K
  const int lim = CAUSAL ? qi + shift : a.Lkv - 1;    // last visible key of this row
  const int lim_first = CAUSAL ? qw0 + shift : a.Lkv - 1;                        // smallest in the wave
  const int lim_last = CAUSAL ? min(qw0 + 31, a.Lq - 1) + shift : a.Lkv - 1;     // largest in the wave

  const int last_q = min(rb * BM + BM - 1, a.Lq - 1);
  const int kv_end = CAUSAL ? min(a.Lkv, last_q + shift + 1) : a.Lkv;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // running max (base 2), partial row sum of 127 * P_tilde over this lane's keys
  float m = kNegInf, l = 0.0f;
  float acc[G::NC][16];                // fp32 output accumulator (O^T, query in the lane)
  v16i acc_i[G::NC];                   // INT32 run of P_hat . V_hat since the last conversion
#pragma unroll
  for (int c = 0; c < G::NC; ++c) {
    acc_i[c] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  }
  int int_tiles = 0;
  float m_f = kNegInf;                 // frame of acc (per-tensor V)

  TileRegs<D> nx;
  load_tile<D, VPT, DUMP>(nx, a, kv_base, 0);
  store_tile<D, VPT, DUMP>(sm.stage[0], nx);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN;
    const Stage& sg = sm.stage[t & 1];
    const bool more = t + 1 < n_tiles;
    if (more) load_tile<D, VPT, DUMP>(nx, a, kv_base, k0 + BN);   // in flight during compute

    if (wave_live && k0 <= lim_last) {
      // ---- S^T = K_hat . Q_hat^T, exact INT32, 32 keys per block ----
      v16i s[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        s[kb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < G::NC; ++c) {
          const v4i ka = *reinterpret_cast<const v4i*>(sg.k + (kb * 32 + lr) * G::KSTR + c * 32 + g * 16);
          s[kb] = mfma_i8(ka, qf[c], s[kb]);
        }
      }

      if constexpr (DUMP) {
        if (qvalid) {
#pragma unroll
          for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = k0 + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
              if (key < a.Lkv && key <= lim) a.s_dump[(q_base + qi) * a.Lkv + key] = s[kb][v];
            }
        }
      } else {
        // ---- dequantize (u = S_int * s_K[j]; the row factor is c2), mask ----
        const bool need_mask = (k0 + BN > a.Lkv) || (CAUSAL && k0 + BN - 1 > lim_first);
        float u[BN / 32][16];
        float mx = need_mask ? dequant_tile<D, true>(s, sg, u, k0, lim, a.Lkv, g)
                             : dequant_tile<D, false>(s, sg, u, k0, lim, a.Lkv, g);
        mx = pair_max(mx);
        // c2 >= 0, so max(u) * c2 == max(u * c2) under monotone rounding
        const float mx2 = (mx == kNegInf) ? kNegInf : mx * c2;
        const float m_new = fmaxf(m, mx2);
        const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
        const float alpha = exp2_hw(m - m_use);        // 1 if unchanged, 0 on the first tile
        const float bias = m_use - kLog2_127;          // exp2(u c2 - bias) = 127 P_tilde

        // ---- 127 P_tilde, row sum, P_hat = rne(127 P_tilde) packed as MFMA operands ----
        v4i pv[BN / 32];
        const bool clamp = __any(fabsf(m_use) >= 32768.0f);
        float lsum;
        if (clamp)
          lsum = need_mask ? probs_tile<VPT, true, true>(u, c2, bias, sg, pv, g)
                           : probs_tile<VPT, false, true>(u, c2, bias, sg, pv, g);
        else
          lsum = need_mask ? probs_tile<VPT, true, false>(u, c2, bias, sg, pv, g)
                           : probs_tile<VPT, false, false>(u, c2, bias, sg, pv, g);
        l = alpha * l + lsum;

        if constexpr (VPT) {
          // per-token V: the tile scale s_t changes per tile, so convert every tile
          v16i tv[G::NC];
          pv_tile<D, true>(tv, sg, pv, lr, g);
          const float st = sg.st;
#pragma unroll
          for (int c = 0; c < G::NC; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] = alpha * acc[c][v] + st * static_cast<float>(tv[c][v]);
        } else {
          // per-tensor V: keep summing P_hat . V_hat in INT32 while no row of
          // the wavefront moves its max (alpha == 1 for all); convert to fp32
          // when one does (same sums, fp32 rounding only)
          // acc is kept in its own frame m_f (it holds 2^(m_f - m) times the
          // fp32 part of the total); the INT32 run is in the frame of m, the
          // max before this tile, and is folded in with one factor per lane.
          const bool flush = __any(m_new > m) || int_tiles >= kMaxIntTiles;
          if (flush) {
            if (m_f == kNegInf) m_f = m_use;
            float fold = exp2_hw(m - m_f);               // 0 before the first tile
            if (__any(m_use - m_f > kRebase)) {          // keep acc far from overflow
              const float r = exp2_hw(m_f - m_use);
#pragma unroll
              for (int c = 0; c < G::NC; ++c)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[c][v] *= r;
              fold *= r;
              m_f = m_use;
            }
#pragma unroll
            for (int c = 0; c < G::NC; ++c) {
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[c][v] = __builtin_fmaf(fold, static_cast<float>(acc_i[c][v]), acc[c][v]);
              acc_i[c] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            }
            int_tiles = 0;
          }
          pv_tile<D, false>(acc_i, sg, pv, lr, g);
          ++int_tiles;
        }
        m = m_new;
      }
    }

    if (more) store_tile<D, VPT, DUMP>(sm.stage[(t + 1) & 1], nx);
    __syncthreads();
  }

  if constexpr (DUMP) return;
  if (!wave_live) return;
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

template <int D, bool CAUSAL, bool VPT, bool OUT_F16, bool DUMP>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>(n_rb));
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VPT, OUT_F16, DUMP>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DUMP>
hipError_t launch_vo(const FwdArgs& a, hipStream_t st) {
  if (DUMP) return launch_t<D, CAUSAL, false, false, DUMP>(a, st);
  if (a.v_per_token)
    return a.o_f16 ? launch_t<D, CAUSAL, true, true, DUMP>(a, st) : launch_t<D, CAUSAL, true, false, DUMP>(a, st);
  return a.o_f16 ? launch_t<D, CAUSAL, false, true, DUMP>(a, st) : launch_t<D, CAUSAL, false, false, DUMP>(a, st);
}

template <bool DUMP>
hipError_t launch_any(const FwdArgs& a, hipStream_t st) {
  if (a.d == 64)
    return a.causal ? launch_vo<64, true, DUMP>(a, st) : launch_vo<64, false, DUMP>(a, st);
  return a.causal ? launch_vo<128, true, DUMP>(a, st) : launch_vo<128, false, DUMP>(a, st);
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, hipStream_t st) { return launch_any<false>(a, st); }
hipError_t launch_debug_logits(const FwdArgs& a, hipStream_t st) { return launch_any<true>(a, st); }

}  // namespace attn
