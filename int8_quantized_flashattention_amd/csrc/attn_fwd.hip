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
// (64) keys shared by the 4 wavefronts. Two workgroups share a CU (256 VGPRs
// per lane at d = 128): while one wavefront of a SIMD waits on the matrix
// core, the other issues its softmax arithmetic.
//
// Both products use v_mfma_i32_32x32x32_i8. The logits are computed
// transposed, S^T = K_hat . Q_hat^T, so that every lane holds keys of ONE
// query: row max and row sum need one cross-half step (v_permlane32_swap).
// The K operand rows are read in a permuted order chosen so that lane l holds
// the 16 CONSECUTIVE keys 16 (l / 32) .. +15 of each 32-key block; those 16
// values, quantized, are exactly the lane's B operand of O^T = V_hat^T .
// P_hat^T, so P never leaves registers. O^T keeps the query in the lane, so
// the per-row rescale is lane-local.
//
// Staging. K and V tiles go from HBM straight into LDS (buffer loads with
// the LDS destination: no registers, no LDS store instructions), in their
// natural [key][channel] layout with the 16-byte chunks of each row XOR-
// swizzled. The V^T operand is read with ds_read_b64_tr_b8, which hands each
// lane 8 consecutive keys of one channel. Four stages form a ring that
// holds the pair of tiles being computed and the pair in flight: before an
// even tile t the workgroup requests tiles t+2 and t+3, and after the odd
// tile t+1 one wait and one barrier make them visible, so the four
// wavefronts meet once per two tiles.
//
// Instruction budget. On gfx950 the issue time of the VALU work per
// (query, key) pair is the first-order cost next to the pair's MFMA work.
// The logit is taken in base 2 with the row's factor s_Q log2(e) / sqrt(d)
// formed once, and it and the exponent argument x - b (b: the exponent bias
// of the running max, 127 folded in) are formed exactly as the oracle rounds
// them (two fp32 products, one fp32 difference), so that only the last-ulp
// behaviour of the exponential can move a quantized probability; per pair the
// kernel spends one INT32->fp32 convert, two multiplies, half a v_max3, one
// subtract, one v_exp_f32, one add for the row sum and one v_cvt_pk_u8_f32
// (round to nearest even, saturating) that quantizes P and packs it into the
// MFMA operand. Everything else is per tile or per workgroup:
//  - for per-tensor V the P_hat . V_hat products keep accumulating in the
//    INT32 MFMA accumulator while no row of the wavefront raises its max and
//    are folded into the fp32 accumulator (which keeps its own frame) only
//    when one does; s_V is applied once in the epilogue;
//  - masking code runs only on diagonal / ragged tiles.
#include "attn_internal.h"
#include "cdna4_ops.h"

#include <hip/hip_fp16.h>

// Every fp32 product and sum below is rounded as written: the logits and the
// exponent argument (a logit minus the bias of the running max) must be the
// oracle's values bit for bit, so no multiply may be fused into a following
// add (fma only where written).
#pragma clang fp contract(off)

namespace attn {
namespace {

constexpr int BM = kPrefillBM;
constexpr int BN = kPrefillBN;
constexpr int NKB = BN / 32;                 // 32-key blocks per tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 4;
// the INT32 run of P_hat . V_hat is folded into fp32 at least every this many
// tiles, keeping |sum| <= 127 * 127 * keys below 2^31
constexpr int kMaxIntTiles = 32768 / BN;

// One pipeline stage: a K tile and a V tile ([key][channel], 16-byte chunks
// swizzled per row), s_K and s_V of the tile's keys.
template <int D>
struct Stage {
  alignas(16) int8_t k[BN * D];
  alignas(16) int8_t v[BN * D];
  alignas(16) float sk[BN];
  alignas(16) float sv[BN];
};

// Key held by MFMA row i of the S^T tile: row i = 8 (v / 4) + 4 g + v % 4 of
// lane group g, register v, carries key 16 g + v.
__device__ __forceinline__ int key_of_row(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

struct Bufs {
  __amdgpu_buffer_rsrc_t k, v, sk, sv;
};

// Per-lane LDS / global offsets, fixed for the whole kernel.
template <int D>
struct Lanes {
  static constexpr int NC = D / 32;                  // 32-channel chunks of the head dim
  static constexpr int LPW = BN * D / 1024 / kWaves; // 1 KB stage loads per wavefront per operand
  uint32_t ld[LPW];   // tile byte offset of the 16-byte chunk this lane moves in load i
  int koff[NC];       // LDS offset (block 0) of this lane's K operand, channel chunk c
  int voff[NC];       // LDS offset (block 0, first 8 keys) of this lane's transposed V read

  __device__ __forceinline__ void init(int wave, int lane) {
    // load i of this wavefront fills LDS slots 64 (LPW wave + i) + lane
#pragma unroll
    for (int i = 0; i < LPW; ++i) ld[i] = tile_load_off<D>(wave * LPW + i, lane);
    const int lr = lane & 31, g = lane >> 5;
    const int kr = key_of_row(lr);
#pragma unroll
    for (int c = 0; c < NC; ++c) koff[c] = kr * D + (((2 * c + g) ^ swz<D>(kr)) * 16);
    // ds_read_b64_tr_b8: in each group of 16 lanes, lane i receives byte
    // i % 8 of the rows addressed by lanes 2 b + i / 8 (b = 0..7). Lane
    // 16 q + i addresses key 16 (q / 2) + i / 2, channels 32 c + 16 (q % 2)
    // + 8 (i % 2) .. +7, so lane l ends with channel 32 c + l % 32, keys
    // 16 (l / 32) .. +7.
    const int q = lane >> 4, i16 = lane & 15;
    const int vr = 16 * (q >> 1) + (i16 >> 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) voff[c] = vr * D + (((2 * c + (q & 1)) ^ swz<D>(vr)) * 16) + 8 * (i16 & 1);
  }
};

// Request tile k0 into a stage: K (and V) rows plus the scales. Wavefront 0
// loads s_K (wavefront 1 s_V when it varies per key); every wavefront then
// moves LPW 1 KB pieces of each operand, so a tile is complete once every
// wavefront's loads have landed.
template <int D, bool KV, bool VPT>
__device__ __forceinline__ void request_tile(Stage<D>& st, const Bufs& bf, const Lanes<D>& ln, int wave, int lane,
                                             int k0) {
  constexpr int LPW = Lanes<D>::LPW;
  if (KV) {
    if (wave == 0) lds_load4(bf.sk, st.sk, lane * 4, k0 * 4);
    if (VPT && wave == 1) lds_load4(bf.sv, st.sv, lane * 4, k0 * 4);
  }
  const uint32_t soff = static_cast<uint32_t>(k0) * D;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int n = wave * LPW + i;
    lds_load16(bf.k, st.k + n * 1024, ln.ld[i], soff);
    if (KV) lds_load16(bf.v, st.v + n * 1024, ln.ld[i], soff);
  }
}

// S^T for one tile: exact INT32 logits, 32 keys per block (shared with the
// logits-dump kernel).
template <int D>
__device__ __forceinline__ void qk_tile(v16i (&s)[NKB], const int8_t* kst, const Lanes<D>& ln, const v4i (&qf)[D / 32]) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const v4i ka = *reinterpret_cast<const v4i*>(kst + kb * 32 * D + ln.koff[c]);
      s[kb] = mfma_i8(ka, qf[c], s[kb]);
    }
}

// One V^T operand (channel chunk c, key block kb) read from a stage.
template <int D>
__device__ __forceinline__ v4i v_operand(const int8_t* vst, const Lanes<D>& ln, int c, int kb) {
  const int8_t* p = vst + kb * 32 * D + ln.voff[c];
  const v2i lo = lds_read_tr8(p);
  const v2i hi = lds_read_tr8(p + 8 * D);
  return v4i{lo.x, lo.y, hi.x, hi.y};
}

// O^T contribution of one tile: acc[c] += V_hat^T . P_hat^T (FRESH: acc[c] =
// V_hat^T . P_hat^T, the first product taking the inline constant 0 as its
// accumulator, so a new INT32 run needs no zeroing instructions). The
// operands of the first PRE channel chunks were read earlier (vpre).
template <int D, bool FRESH, int PRE>
__device__ __forceinline__ void pv_tile(v16i (&acc)[D / 32], const int8_t* vst, const Lanes<D>& ln,
                                        const v4i (&pv)[NKB], const v4i (&vpre)[PRE > 0 ? PRE : 1][NKB]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const v4i vo = c < PRE ? vpre[c < PRE ? c : 0][kb] : v_operand<D>(vst, ln, c, kb);
      acc[c] = mfma_i8(vo, pv[kb], (FRESH && kb == 0) ? zero16() : acc[c]);
    }
}

// The dequantized logits of this lane's keys, masked keys -inf; returns the
// max over the lane pair. EXP (exp softmax): the base-2 logit x =
// (float(S_int) * aq) * s_K[j], two rounded fp32 products in that order with
// aq = s_Q log2(e) / sqrt(d) formed once per row, the oracle's logit bit for
// bit. !EXP (IndexSoftmax): x = float(S_int) * s_K[j] (aq unused), the table
// path's u. rel =
// (last visible key of the row) - k0 - 16 g, so entry v of block kb is
// visible iff 32 kb + v <= rel, a compare of a compile-time constant with one
// per-lane value.
template <int D, bool MASK, bool EXP>
__device__ __forceinline__ float dequant_tile(const v16i (&s)[NKB], const float* sk, float aq, float (&x)[NKB][16],
                                              int rel, int g) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const float4 skv = *reinterpret_cast<const float4*>(sk + kb * 32 + g * 16 + j4 * 4);
      const float skk[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = static_cast<float>(s[kb][j4 * 4 + e]);
        if constexpr (EXP) {
          t = (t * aq) * skk[e];
        } else {
          t = t * skk[e];
        }
        if constexpr (MASK) t = (kb * 32 + j4 * 4 + e <= rel) ? t : kNegInf;
        x[kb][j4 * 4 + e] = t;
      }
    }
  // the maximum: per 32-key block a chain of three-input maxima (v_max3),
  // the blocks' chains independent of each other
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    float pm = fmaxf(fmaxf(x[kb][0], x[kb][1]), x[kb][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) pm = fmaxf(fmaxf(pm, x[kb][e]), x[kb][e + 1]);
    mx = fmaxf(mx, fmaxf(pm, x[kb][15]));
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// y = 2^(x - eb) = 127 P_tilde, with eb the exponent bias of the running max
// (exp_bias) and x - eb the oracle's rounded fp32 difference; returns this
// lane's sum of y and packs P_hat = rne(y) (per-token V: rne(y w_j), the fp32
// product, with the key multipliers w_j = s_V[j] / s_t read from wr) into the
// PV operands. Masked keys have x = -inf, so their y is exactly 0.
template <bool VPT>
__device__ __forceinline__ float probs_tile(const float (&x)[NKB][16], float eb, const float* wr_s,
                                            v4i (&pv)[NKB], int g) {
  float gs[NKB * 4];                   // partial row sums, added as a tree
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    uint32_t pw[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float wr[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (VPT) {
        const float4 w4 = *reinterpret_cast<const float4*>(wr_s + kb * 32 + g * 16 + j4 * 4);
        wr[0] = w4.x; wr[1] = w4.y; wr[2] = w4.z; wr[3] = w4.w;
      }
      uint32_t word = 0;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = exp2_hw(x[kb][j4 * 4 + e] - eb);
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

// IndexSoftmax in place of exp2: x = m_u kappa - u kappa (one fma), the
// table index is floor(x) clamped to [0, n] (med3, then a truncating convert
// of a non-negative value), E = table[index] read from LDS; masked keys read
// the zero slot. Packs E into the PV operands and returns this lane's integer
// sum of E (four bytes per dot4 against ones).
template <bool MASK>
__device__ __forceinline__ float lut_tile(const float (&u)[NKB][16], float kap, float mu, float nf,
                                          const uint8_t* tab, int rel, v4i (&pv)[NKB]) {
  uint32_t sum = 0;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    uint32_t pw[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __builtin_amdgcn_fmed3f(__builtin_fmaf(u[kb][j4 * 4 + e], -kap, mu), 0.0f, nf);
        uint32_t idx = static_cast<uint32_t>(x);
        if constexpr (MASK) idx = (kb * 32 + j4 * 4 + e <= rel) ? idx : static_cast<uint32_t>(kLutZero);
        word |= static_cast<uint32_t>(tab[idx]) << (8 * e);
      }
      sum = __builtin_amdgcn_udot4(word, 0x01010101u, sum, false);
      pw[j4] = word;
    }
    pv[kb] = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]), static_cast<int>(pw[3])};
  }
  return static_cast<float>(sum);
}

// The same with a table of key pairs (tables of at most 32 entries): entry
// ia + 33 ib of the pair table holds E[ia] | E[ib] << 8, index 32 being the
// zero slot, so one 16-bit LDS read serves two keys and two reads fill a
// packed word of the PV operand.
template <bool MASK>
__device__ __forceinline__ float lut2_tile(const float (&u)[NKB][16], float kap, float mu, float nf,
                                           const uint16_t* tab2, int rel, v4i (&pv)[NKB]) {
  uint32_t sum = 0;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    uint32_t pw[4];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      uint32_t idx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __builtin_amdgcn_fmed3f(__builtin_fmaf(u[kb][j4 * 4 + e], -kap, mu), 0.0f, nf);
        idx[e] = static_cast<uint32_t>(x);
        if constexpr (MASK) idx[e] = (kb * 32 + j4 * 4 + e <= rel) ? idx[e] : 32u;
      }
      const uint32_t lo = tab2[idx[0] + idx[1] * kLutPairRows];
      const uint32_t hi = tab2[idx[2] + idx[3] * kLutPairRows];
      const uint32_t word = lo | (hi << 16);
      sum = __builtin_amdgcn_udot4(word, 0x01010101u, sum, false);
      pw[j4] = word;
    }
    pv[kb] = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]), static_cast<int>(pw[3])};
  }
  return static_cast<float>(sum);
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_t of a tile for per-token V: the largest s_V[j] over the tile's keys
// below Lkv (a stage may hold stale entries past the end).
__device__ __forceinline__ float tile_vscale(float svl) { return wave_max_nonneg(svl); }

__device__ __forceinline__ Bufs make_bufs(const FwdArgs& a, int64_t kv_base, int D, bool scales, bool vpt) {
  Bufs bf;
  bf.k = make_rsrc(a.k + kv_base * D, a.Lkv * D);
  bf.v = bf.k;
  bf.sk = bf.k;
  bf.sv = bf.k;
  if (scales) {
    bf.v = make_rsrc(a.v + kv_base * D, a.Lkv * D);
    bf.sk = make_rsrc(a.s_k + kv_base, a.Lkv * 4);
    if (vpt) bf.sv = make_rsrc(a.s_v + kv_base, a.Lkv * 4);
  }
  return bf;
}

// Workgroup -> (b*h, row block). Workgroups are dealt to the 8 XCDs round
// robin, so consecutive ids land on different XCDs (each with its own L2),
// and each XCD takes a contiguous range of heads. When every XCD holds whole
// heads, its heads are taken in groups of up to 4 and each group row block by
// row block, longest (causal) first: every head's longest blocks start early,
// so the launch does not end waiting on a long block that started late, while
// the workgroups in flight on an XCD share the K/V of at most 4 heads (4 MB at
// L = 4096, d = 128, the size of an XCD's L2). Measured at B4 H32 L4096 d128
// causal: groups of 1, 2, 4 and 8 heads take 0.556, 0.525, 0.507 and 0.507 ms
// and miss the L2 for 271, 273, 358 and 666 MB per launch.
// Otherwise heads are walked one after the other, longest block first.
__device__ __forceinline__ void tile_of_block(int n_rb, int& bh, int& rb) {
  const int n = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int per = n >> 3;
  if ((n & 7) == 0 && per % n_rb == 0) {
    const int nh = per / n_rb;                 // heads of this XCD
    int G = nh < 4 ? nh : 4;
    while (nh % G) --G;                        // groups of G heads
    const int grp = slot / (G * n_rb), s = slot - grp * G * n_rb;
    rb = n_rb - 1 - s / G;
    bh = xcd * nh + grp * G + s % G;
    return;
  }
  const int w = xcd * per + min(xcd, n & 7) + slot;
  bh = w / n_rb;
  rb = n_rb - 1 - (w - bh * n_rb);
}

// LUT: 0 exp2 softmax; 1 IndexSoftmax with the byte table; 2 IndexSoftmax
// with the pair table (tables of at most 32 entries). IndexSoftmax only with
// V scales constant along the keys (per tensor, head or channel) and INT8 Q.
// QF: 0 INT8 Q; 1 fp16/fp32 Q quantized here; 2 the same after the
// normalized Hadamard rotation of each Q row.
// DUMP: the logits-dump instance (test hook). It runs the same grid, the same
// K staging ring, barriers and Q.K^T tile code, and writes the INT32 logit
// of every visible pair instead of the softmax and P.V (INT8 Q, no scales).
template <int D, bool CAUSAL, bool VPT, bool OUT_F16, int QF, int LUT, bool DUMP = false>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a) {
  static_assert(!LUT || (!VPT && !QF), "IndexSoftmax takes INT8 Q and V scales constant along the keys");
  static_assert(!DUMP || (!VPT && !QF && !LUT), "the dump instance takes INT8 Q");
  constexpr int NC = D / 32;
  // PRE: V operands of this many channel chunks are read right after Q.K^T,
  // ahead of the softmax (the IndexSoftmax kernels have registers for one)
  constexpr int PRE = LUT ? 1 : 2;
  __shared__ Stage<D> sm[kStages];
  __shared__ uint32_t lut_s[LUT ? 65 : 1];
  __shared__ uint16_t lut2_s[LUT == 2 ? kLutPairRows * kLutPairRows : 1];
  // per-token V: each wavefront's key multipliers s_V[j] / s_t of the tile
  __shared__ float wr_s[VPT ? kWaves : 1][VPT ? BN : 1];

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

  // the dump instance has no V or scales: its V stages and scale slots are
  // filled from K (and never read)
  const Bufs bf = make_bufs(a, kv_base, D, !DUMP, VPT);
  Lanes<D> ln;
  ln.init(wave, lane);

  const int last_q = min(rb * BM + BM - 1, a.Lq - 1);
  const int kv_end = CAUSAL ? min(a.Lkv, last_q + shift + 1) : a.Lkv;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // scale slots start at zero: a load past Lkv may leave a slot untouched
  for (int i = tid; i < kStages * BN; i += kThreads) {
    sm[i / BN].sk[i % BN] = 0.0f;
    sm[i / BN].sv[i % BN] = 0.0f;
  }
  if constexpr (LUT) {
    if (tid < 65) lut_s[tid] = a.lut_w[tid];
  }
  if constexpr (LUT == 2) {
    __syncthreads();
    const uint8_t* tab = reinterpret_cast<const uint8_t*>(lut_s);   // zero from entry 32 on
    for (int e = tid; e < kLutPairRows * kLutPairRows; e += kThreads) {
      const int ia = e % kLutPairRows, ib = e / kLutPairRows;
      lut2_s[e] = static_cast<uint16_t>(tab[ia] | (tab[ib] << 8));
    }
  }

  // Q fragment (B operand of S^T): 16 bytes per 32-channel chunk. Requested
  // before the first stage requests, so that the prologue's wait covers it.
  // QF: the row arrives in fp16/fp32 and is quantized here, per token with
  // the quantizer's arithmetic; the lane pair (l, l ^ 32) holds the row. An
  // fp16 row is requested whole here and converted after the stage requests.
  v4i qf[NC];
  float sq = 0.0f;
  float xq[QF ? NC : 1][16];
  v4i q16[QF ? NC : 1][2];
  if constexpr (QF) {
    if (qvalid && a.q_float_f16) q16_load<NC>(a.q_float, (q_base + qi) * D + g * 16, 32, q16);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = v4i{0, 0, 0, 0};
      if (qvalid) qf[c] = *reinterpret_cast<const v4i*>(a.q + (q_base + qi) * D + c * 32 + g * 16);
    }
    sq = (qvalid && !DUMP) ? a.s_q[q_base + qi] : 0.0f;
  }
  __syncthreads();
  request_tile<D, true, VPT>(sm[0], bf, ln, wave, lane, 0);
  if (n_tiles > 1) request_tile<D, true, VPT>(sm[1], bf, ln, wave, lane, BN);
  if constexpr (QF) {
    // the Q row, converted once the first tiles are requested
    if (qvalid) {
      if (a.q_float_f16) q16_f32<NC>(q16, xq);
      else q32_f32<NC>(a.q_float, (q_base + qi) * D + g * 16, 32, xq);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) xq[c][e] = 0.0f;
    }
  }
  if constexpr (QF == 2) {
    // Hadamard rotation of the row (the rotated quantizer's butterflies, strides
    // in increasing order): 1 .. 8 inside the lane's 16 channels, 16 across the
    // lane pair, 32 and 64 across the lane's 32-channel chunks; then times rn
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!(e & h)) {
            const float x0 = xq[c][e], x1 = xq[c][e + h];
            xq[c][e] = x0 + x1;
            xq[c][e + h] = x0 - x1;
          }
    // stride 32 across the lane pair: v_permlane32_swap hands lanes 0-31
    // (own, partner) and lanes 32-63 (partner, own), so one fma gives own +
    // partner below and partner - own above (VALU only, no LDS round trip)
    const float sgn = g ? -1.0f : 1.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(xq[c][e]), __float_as_uint(xq[c][e]), false, false);
        xq[c][e] = __builtin_fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
      }
#pragma unroll
    for (int m = 1; m < NC; m <<= 1)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (!(c & m)) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float x0 = xq[c][e], x1 = xq[c ^ m][e];
            xq[c][e] = x0 + x1;
            xq[c ^ m][e] = x0 - x1;
          }
        }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) xq[c][e] = xq[c][e] * a.q_rot_scale;
  }
  if constexpr (QF) {
    float am = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(xq[c][e]));
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
    am = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    const float r = quant_recip(am);
    sq = quant_scale(am);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = v4i{static_cast<int>(quant_word(&xq[c][0], r)), static_cast<int>(quant_word(&xq[c][4], r)),
                  static_cast<int>(quant_word(&xq[c][8], r)), static_cast<int>(quant_word(&xq[c][12], r))};
    if (qvalid) {
      if (a.q_hat_out) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          *reinterpret_cast<v4i*>(a.q_hat_out + (q_base + qi) * D + c * 32 + g * 16) = qf[c];
      }
      if (a.s_q_out && g == 0) a.s_q_out[q_base + qi] = sq;
    }
  }
  const int lim = CAUSAL ? qi + shift : a.Lkv - 1;    // last visible key of this row
  const int lim_first = CAUSAL ? qw0 + shift : a.Lkv - 1;   // smallest in the wavefront

  // softmax state: running max (base 2), partial sum of 127 P_tilde over this lane's keys
  float m = kNegInf, l = 0.0f;
  float acc[NC][16];                   // fp32 O^T accumulator
  v16i acc_i[NC];                      // INT32 accumulation of P_hat . V_hat
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    acc_i[c] = zero16();
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  }
  float m_f = kNegInf;                 // frame of acc (per-tensor V)
  int int_tiles = 0;                   // tiles in the current INT32 run
  bool fresh = true;                   // the next PV starts a new INT32 run

  // tiles 0 and 1 must have landed
  wait_vm_lds<0>();
  bare_barrier();
  // The wait above also covered the Q loads (issued before it). Passing the
  // fragment and s_Q through empty asm statements tells the compiler so; otherwise
  // it waits for them again inside the tile loop, which would also wait for
  // the newest stage request.
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
  asm volatile("" : "+v"(sq));
  const float inv_sqrt_d = (D == 64) ? 0.125f : static_cast<float>(0.08838834764831845);
  // The running max m is in base-2 logits. Exp softmax: the oracle's fp32
  // running max of x = (S_int aq) s_K[j], aq = s_Q log2(e) / sqrt(d).
  // IndexSoftmax: the max of u times c2 = s_Q log2 e / sqrt(d), kept >=
  // FLT_MIN so that -inf * c2 stays -inf for masked keys.
  const float aq = sq * kLogitScale<D>;
  const float c2 = fmaxf(sq * inv_sqrt_d * kLog2e, kFltMin);
  // IndexSoftmax: table index per unit of u below the running max, and the
  // running max of u itself (kept beside m)
  const float kap = (sq * inv_sqrt_d) * a.lut_k;
  const float nf = static_cast<float>(a.lut_n);
  float m_u = kNegInf;

  // One tile: (even t) request t+2, t+3 | QK(t) [MFMA] | dequant, softmax(t)
  // [VALU] | fold | PV(t) [MFMA] | (odd t) wait for t+1, t+2 | barrier. The
  // stage being read and the stages being filled are distinct objects, passed
  // as restrict pointers: the compiler then knows that this tile's LDS reads
  // do not depend on the loads just issued and adds no wait for them.
  auto step = [&](int t, const Stage<D>* __restrict__ st, Stage<D>* __restrict__ nx,
                  Stage<D>* __restrict__ nx2) __attribute__((always_inline)) {
    const int k0 = t * BN;
    if (!(t & 1) && t + 2 < n_tiles) {
      request_tile<D, true, VPT>(*nx, bf, ln, wave, lane, k0 + 2 * BN);
      if (t + 3 < n_tiles) request_tile<D, true, VPT>(*nx2, bf, ln, wave, lane, k0 + 3 * BN);
    }

    // causal: a tile past the last row of this wavefront changes nothing (a
    // fully masked tile is a no-op), so its arithmetic is skipped; the
    // wavefront still issues its share of the stage loads and meets the
    // barrier. (The last tile of a row block lies past the first two
    // wavefronts' rows.)
    const bool dead = CAUSAL && k0 > min(qw0 + 31, a.Lq - 1) + shift;
    if (DUMP || !dead) {
    v16i s[NKB];
    qk_tile<D>(s, st->k, ln, qf);
    if constexpr (DUMP) {
      if (qvalid) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kb * 32 + g * 16 + v;
            if (key < a.Lkv && key <= lim) a.s_dump[(q_base + qi) * a.Lkv + key] = s[kb][v];
          }
      }
    } else {
    // Issue priority (s_setprio) rises through the tile's VALU work: 1 from
    // here, 2 for the probabilities (exp or table), 3 for the P.V issue, back
    // to 0 once it is issued. Of the two wavefronts that share a SIMD, the one further
    // along its softmax wins the VALU arbitration and reaches its products
    // first, so the pair drifts out of step instead of running both
    // softmaxes together and then both waiting on the matrix core (which
    // leaves the VALU idle). The arithmetic is unchanged.
    __builtin_amdgcn_s_setprio(1);
    v4i vpre[PRE > 0 ? PRE : 1][NKB];
#pragma unroll
    for (int c = 0; c < PRE; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) vpre[c][kb] = v_operand<D>(st->v, ln, c, kb);
    if constexpr (PRE > 0) __builtin_amdgcn_sched_barrier(0);
    const bool mask = (k0 + BN > a.Lkv) || (CAUSAL && k0 + BN - 1 > lim_first);
    float u[NKB][16];                  // logits x (exp softmax) or u (IndexSoftmax)
    float mx;
    if (!mask) {
      mx = dequant_tile<D, false, !LUT>(s, st->sk, aq, u, 0, g);
    } else {
      mx = dequant_tile<D, true, !LUT>(s, st->sk, aq, u, min(lim, a.Lkv - 1) - k0 - 16 * g, g);
    }

    // ---- softmax(t): running max, 127 P_tilde, row sum, P_hat ----
    // (IndexSoftmax: c2 > 0, so max(u) c2 == max(u c2))
    const float mx2 = !LUT ? mx : (mx == kNegInf) ? kNegInf : mx * c2;
    const float m_new = fmaxf(m, mx2);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    // alpha = 2^(m - m_use): 1 when no row of the wavefront raised its max
    // (then it is not computed), 0 on a row's first visible tile
    float alpha = 1.0f;
    const bool rose = __any(m_new > m);
    if (VPT && rose) alpha = exp2_hw(m - m_use);
    v4i p[NKB];
    float lsum;
    float st_cur = 0.0f;
    if constexpr (LUT) {
      m_u = fmaxf(m_u, mx);
      __builtin_amdgcn_s_setprio(2);
      const float mu = m_u * kap;
      const int rel = min(lim, a.Lkv - 1) - k0 - 16 * g;
      if constexpr (LUT == 2) {
        if (!mask) lsum = lut2_tile<false>(u, kap, mu, nf, lut2_s, 0, p);
        else lsum = lut2_tile<true>(u, kap, mu, nf, lut2_s, rel, p);
      } else {
        const uint8_t* tab = reinterpret_cast<const uint8_t*>(lut_s);
        if (!mask) lsum = lut_tile<false>(u, kap, mu, nf, tab, 0, p);
        else lsum = lut_tile<true>(u, kap, mu, nf, tab, rel, p);
      }
    } else {
      if constexpr (VPT) {
        // s_t and the multiplier of this lane's key (lane = key of the tile),
        // s_V[j] / s_t as the oracle's one rounded division, formed once per
        // key and shared through the wavefront's LDS row: the LDS executes a
        // wavefront's accesses in order, and the wave barrier keeps the
        // compiler from moving the reads above the write
        const float svl = (k0 + lane < a.Lkv) ? st->sv[lane] : 0.0f;
        st_cur = tile_vscale(svl);
        wr_s[wave][lane] = st_cur > 0.0f ? __fdiv_rn(svl, st_cur) : 0.0f;
        __builtin_amdgcn_wave_barrier();
      }
      __builtin_amdgcn_s_setprio(2);
      lsum = probs_tile<VPT>(u, exp_bias(m_use), wr_s[VPT ? wave : 0], p, g);
    }

    if constexpr (!VPT) {
      if (rose || ++int_tiles > kMaxIntTiles) {
        alpha = exp2_hw(m - m_use);
        // tile t raised some row's max: the INT32 run (tiles before t, frame
        // m) goes into acc (frame m_f) before PV(t) starts a new run
        if (m_f == kNegInf) m_f = m_use;
        float f = exp2_hw(m - m_f);                   // 0 before the first tile
        if (__any(m_use - m_f > kRebase)) {           // keep acc far from overflow
          const float r = exp2_hw(m_f - m_use);
          f *= r;
          m_f = m_use;
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] *= r;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[c][v] = __builtin_fmaf(f, static_cast<float>(acc_i[c][v]), acc[c][v]);
        }
        fresh = true;
        int_tiles = 1;
      }
    }
    l = __builtin_fmaf(alpha, l, lsum);
    m = m_new;

    __builtin_amdgcn_s_setprio(3);
    // per-token V converts every tile's product on its own: always a new run
    if (VPT || fresh) pv_tile<D, true, PRE>(acc_i, st->v, ln, p, vpre);
    else pv_tile<D, false, PRE>(acc_i, st->v, ln, p, vpre);
    __builtin_amdgcn_s_setprio(0);
    fresh = false;
    if constexpr (VPT) {
      // per-token V: tile scales differ, so each tile's INT32 product is
      // converted on its own: acc = alpha acc + s_t PV(t), the product by
      // alpha only on tiles that raised a max, both in place (written as one
      // fma, the compiler accumulates into the product's register and the
      // loop then copies all of acc back every tile)
      if (rose) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[c][v] *= alpha;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[c][v] = __builtin_fmaf(st_cur, static_cast<float>(acc_i[c][v]), acc[c][v]);
    }
    }  // !DUMP
    }  // live tile

    // after an odd tile: tiles t+1 and t+2 must have landed before anyone
    // reads them; after the barrier every wavefront is done with stages t-1
    // and t, which tiles t+3 and t+4 reuse
    if ((t & 1) && t + 1 < n_tiles) {
      wait_vm_lds<0>();
      bare_barrier();
    }
  };

  for (int t = 0; t < n_tiles; ++t) step(t, &sm[t & 3], &sm[(t + 2) & 3], &sm[(t + 3) & 3]);
  if constexpr (DUMP) return;

  if constexpr (!VPT) {
    // total in the frame of the final max m: 2^(m_f - m) acc + INT32 run
    const float back = exp2_hw(m_f - m);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = __builtin_fmaf(back, acc[c][v], static_cast<float>(acc_i[c][v]));
  }

  const float ltot = pair_sum(l);                      // 127 * l
  if (!qvalid) return;
  const float scale = (VPT ? 1.0f : a.s_v[a.v_per_head ? b * a.Hkv + hk : 0]) / ltot;
  // per-channel V: channel c of the output takes its own scale
  const float* sch = a.s_v + (static_cast<int64_t>(b) * a.Hkv + hk) * D;
  const float rl = 1.0f / ltot;
  const int64_t orow = (q_base + qi) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d0 = c * 32 + j4 * 8 + g * 4;
      float cs[4] = {scale, scale, scale, scale};
      if (!VPT && a.v_per_channel) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[e] = sch[d0 + e] * rl;
      }
      const float o0 = acc[c][j4 * 4 + 0] * cs[0], o1 = acc[c][j4 * 4 + 1] * cs[1];
      const float o2 = acc[c][j4 * 4 + 2] * cs[2], o3 = acc[c][j4 * 4 + 3] * cs[3];
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

template <int D, bool CAUSAL, bool VPT, bool OUT_F16>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * n_rb));
  if (a.q_float && a.q_rotate)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VPT, OUT_F16, 2, 0>), grid, dim3(kThreads), 0, st, a);
  else if (a.q_float)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VPT, OUT_F16, 1, 0>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VPT, OUT_F16, 0, 0>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool OUT_F16>
hipError_t launch_lut(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * n_rb));
  if (a.lut_n < kLutPairRows - 1)      // n <= 31: entries and the zero slot fit
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, false, OUT_F16, 0, 2>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, false, OUT_F16, 0, 1>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_vo(const FwdArgs& a, hipStream_t st) {
  if (a.lut_n) return a.o_f16 ? launch_lut<D, CAUSAL, true>(a, st) : launch_lut<D, CAUSAL, false>(a, st);
  if (a.v_per_token)
    return a.o_f16 ? launch_t<D, CAUSAL, true, true>(a, st) : launch_t<D, CAUSAL, true, false>(a, st);
  return a.o_f16 ? launch_t<D, CAUSAL, false, true>(a, st) : launch_t<D, CAUSAL, false, false>(a, st);
}

template <int D, bool CAUSAL>
hipError_t launch_logits_t(const FwdArgs& a, hipStream_t st) {
  const int n_rb = (a.Lq + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.B * a.H * n_rb));
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, false, false, 0, 0, true>), grid, dim3(kThreads), 0, st, a);
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
