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
// fma(p, w, kMagic) = kMagic + rne(p * w) for 0 <= p * w < 2^22: the exact
// product is rounded once at unit spacing, ties to even (kMagic is even).
constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
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

// Byte 0 of a, b, c, d packed into one dword (a lowest).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Position of tile-local key j inside a V^T LDS row: the 16 keys that one lane
// half (g) contributes to a 32-key MFMA step are stored contiguously, in the
// order of that lane's logit accumulators.
__device__ __forceinline__ int vt_pos(int j) {
  const int kb = j >> 5, r = j & 31;
  return kb * 32 + ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

struct Smem {
  alignas(16) int8_t k[BN * (128 + 16)];
  alignas(16) int8_t vt[128 * (BN + 16)];
  alignas(16) float sk[BN];
  alignas(16) float w[BN];
  float st;
};

// Stages the K tile (and, unless LOGITS_ONLY, the V^T tile and the per-key
// scales). The logits-only variant is given no V or scale pointers and must
// not touch them.
template <int D, bool VPT, bool LOGITS_ONLY>
__device__ __forceinline__ void stage_tile(Smem& sm, const FwdArgs& a, int64_t kv_base, int k0) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
  // K rows: 16-byte chunks, coalesced along the row.
  constexpr int kCPR = D / 16;                       // chunks per row
  constexpr int kKIters = BN * kCPR / kThreads;
#pragma unroll
  for (int it = 0; it < kKIters; ++it) {
    const int id = tid + it * kThreads;
    const int row = id / kCPR, cc = id % kCPR;
    v4i val = {0, 0, 0, 0};
    if (k0 + row < a.Lkv)
      val = *reinterpret_cast<const v4i*>(a.k + (kv_base + k0 + row) * D + cc * 16);
    *reinterpret_cast<v4i*>(sm.k + row * G::KSTR + cc * 16) = val;
  }
  if constexpr (LOGITS_ONLY) return;
  // V: lanes run along the head dim (4 channels each), 4 keys per lane,
  // transposed in registers and written as V^T.
  constexpr int kNDQ = D / 4;                        // channel quads
  constexpr int kKQPerIter = kThreads / kNDQ;        // key quads per pass
  constexpr int kVIters = (BN / 4) / kKQPerIter;
  const int dq = tid % kNDQ;
#pragma unroll
  for (int it = 0; it < kVIters; ++it) {
    const int kq = tid / kNDQ + it * kKQPerIter;
    uint32_t r[4], c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + kq * 4 + i;
      r[i] = (key < a.Lkv)
                 ? *reinterpret_cast<const uint32_t*>(a.v + (kv_base + key) * D + dq * 4)
                 : 0u;
    }
    transpose4x4(r, c);
    const int pos = vt_pos(kq * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint32_t*>(sm.vt + (dq * 4 + j) * G::VSTR + pos) = c[j];
  }
  // per-key logit scales, and for per-token V the tile scale and multipliers
  if (tid < BN) {
    const int key = k0 + tid;
    sm.sk[tid] = (key < a.Lkv) ? a.s_k[kv_base + key] : 0.0f;
  } else if (VPT && tid < 2 * BN) {
    const int j = tid - BN;
    const int key = k0 + j;
    const float sv = (key < a.Lkv) ? a.s_v[kv_base + key] : 0.0f;
    float st = sv;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) st = fmaxf(st, __shfl_xor(st, off, 64));
    sm.w[j] = (st > 0.0f) ? __fdiv_rn(127.0f * sv, st) : 0.0f;
    if (j == 0) sm.st = st;
  }
}

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
  const int lim = CAUSAL ? qi + shift : a.Lkv - 1;  // last visible key of this row
  const int wave_lim = CAUSAL ? min(qw0 + 31, a.Lq - 1) + shift : a.Lkv - 1;

  const int last_q = min(rb * BM + BM - 1, a.Lq - 1);
  const int kv_end = CAUSAL ? min(a.Lkv, last_q + shift + 1) : a.Lkv;
  const int n_tiles = (kv_end + BN - 1) / BN;

  float m = kNegInf, l = 0.0f;
  float acc[G::NC][16];
#pragma unroll
  for (int c = 0; c < G::NC; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN;
    __syncthreads();                 // previous tile fully consumed
    stage_tile<D, VPT, DUMP>(sm, a, kv_base, k0);
    __syncthreads();
    if (!wave_live || k0 > wave_lim) continue;   // every key of the tile is masked for this wave

    // ---- S^T = K_hat . Q_hat^T for the two 32-key blocks (exact INT32) ----
    v16i s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < G::NC; ++c) {
        const v4i ka = *reinterpret_cast<const v4i*>(sm.k + (kb * 32 + lr) * G::KSTR + c * 32 + g * 16);
        s[kb] = mfma_i8(ka, qf[c], s[kb]);
      }
    }

    if constexpr (DUMP) {
      if (qvalid) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kb * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
            if (key < a.Lkv && key <= lim) a.s_dump[(q_base + qi) * a.Lkv + key] = s[kb][v];
          }
      }
      continue;
    }

    // ---- dequantize + mask: u = S_int * s_K[j] (the row factor is c2) ----
    float u[2][16];
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int jl = kb * 32 + j4 * 8 + g * 4;
        const float4 skv = *reinterpret_cast<const float4*>(sm.sk + jl);
        const float skk[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + jl + e;
          const float x = static_cast<float>(s[kb][j4 * 4 + e]) * skk[e];
          const bool vis = key < a.Lkv && key <= lim;
          u[kb][j4 * 4 + e] = vis ? x : kNegInf;
          mx = fmaxf(mx, u[kb][j4 * 4 + e]);
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // c2 >= 0, so max(u) * c2 == max(u * c2) under monotone rounding
    const float mx2 = (mx == kNegInf) ? kNegInf : mx * c2;
    const float m_new = fmaxf(m, mx2);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = exp2_hw(m - m_use);           // 0 on the first visible tile

    // ---- probabilities, row sum, INT8 quantization into MFMA operands ----
    float lsum = 0.0f;
    v4i pv[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t pw[4];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        float wk[4] = {127.0f, 127.0f, 127.0f, 127.0f};
        if constexpr (VPT) {
          const float4 wv = *reinterpret_cast<const float4*>(sm.w + kb * 32 + j4 * 8 + g * 4);
          wk[0] = wv.x; wk[1] = wv.y; wk[2] = wv.z; wk[3] = wv.w;
        }
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float uu = u[kb][j4 * 4 + e];
          const float p = (uu == kNegInf) ? 0.0f : exp2_hw(__builtin_fmaf(uu, c2, -m_use));
          lsum += p;
          bits[e] = __float_as_uint(__builtin_fmaf(p, wk[e], kMagic));
        }
        pw[j4] = pack_low_bytes(bits[0], bits[1], bits[2], bits[3]);
      }
      pv[kb] = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]),
                   static_cast<int>(pw[3])};
    }
    l = alpha * l + lsum;
    const float st = VPT ? sm.st : a.s_v[0];

    // ---- O^T += V_hat^T . P_hat^T (INT32 per tile), fp32 across tiles ----
#pragma unroll
    for (int c = 0; c < G::NC; ++c) {
      v16i tacc = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v4i va = *reinterpret_cast<const v4i*>(sm.vt + (c * 32 + lr) * G::VSTR + kb * 32 + g * 16);
        tacc = mfma_i8(va, pv[kb], tacc);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = alpha * acc[c][v] + st * static_cast<float>(tacc[v]);
    }
    m = m_new;
  }

  if constexpr (DUMP) return;
  if (!wave_live) return;
  const float ltot = l + __shfl_xor(l, 32, 64);
  if (!qvalid) return;
  const float rcp = 1.0f / (127.0f * ltot);
  const int64_t orow = (q_base + qi) * D;
#pragma unroll
  for (int c = 0; c < G::NC; ++c)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = c * 32 + j4 * 8 + g * 4;
      const float o0 = acc[c][j4 * 4 + 0] * rcp, o1 = acc[c][j4 * 4 + 1] * rcp;
      const float o2 = acc[c][j4 * 4 + 2] * rcp, o3 = acc[c][j4 * 4 + 3] * rcp;
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
  if (a.lse && g == 0) a.lse[q_base + qi] = (m + __builtin_log2f(ltot)) * kLn2;
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
