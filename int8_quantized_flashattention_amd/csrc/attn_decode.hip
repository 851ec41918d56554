// Split-KV INT8 attention for decode-shaped problems on gfx950: few query
// rows per KV head (a GQA group of H / Hkv heads times Lq queries, at most
// 16 rows), long KV. The work is bound by streaming K_hat and V_hat from HBM
// once, so the KV length is split into chunks processed in parallel, each by
// one wavefront, and a second kernel merges the chunks.
//
// Method as in the prefill kernel: "INT-FlashAttention: Enabling Flash
// Attention for INT8 Quantization" (abstract); integer logits, the
// s_Q s_K / sqrt(d) dequantization and the s_V P V_hat form from "IntAttention:
// A Fully Integer Attention Pipeline for Efficient Edge Inference" §2.1, §3.1
// (Eq. 4); P quantized with multiplier 127 (IntAttention §3.2); each chunk is
// one online-softmax pass in tiles of kDecodeBN keys and the chunk results are
// merged by their row maxima (the same identity as the per-tile rescale of
// "FlashAttention-3", abstract).
//
// Per wavefront: the 16 rows of one v_mfma_i32_16x16x64_i8 tile hold the
// group's query rows (row r = (head - Hkv-group start) * Lq + query). K tiles
// go from HBM straight into registers, already in the MFMA operand layout
// (two register slots: tile t+2 is loaded into tile t's slot as soon as the
// QK of tile t has read it); V tiles and the scales go into a 3-stage LDS ring
// (buffer loads with LDS destination, rows swizzled), since the V^T operands
// need the transposing ds_read_b64_tr_b8. Keeping K out of LDS halves the ring,
// so twice as many wavefronts (and loads in flight) fit on a CU. Every K, V
// and scale byte is read exactly once, with the non-temporal cache policy.
// Lane l holds query row l % 16 and, in each of the 4 key blocks of 16, keys
// 4 b + 0..3 of its lane group, that is the 16 consecutive keys 16 (l / 16)
// .. +15 of the tile, which are exactly its P operand for O^T = V^T P^T.
#include "attn_internal.h"
#include "cdna4_ops.h"

#include <hip/hip_fp16.h>

#include <type_traits>

// fp32 products and sums are rounded as written (the logits and the exponent
// argument, a logit minus the bias of the running max, are the oracle's values
// bit for bit); fma only where written.
#pragma clang fp contract(off)

namespace attn {
namespace {

constexpr int BN = kDecodeBN;
static_assert(BN == kPrefillBN, "one KV tile size for every schedule");
constexpr int NB = BN / 16;                  // 16-key blocks per tile
constexpr int kStages = 3;
// the INT32 run of P_hat . V_hat is folded into fp32 at least every this many
// tiles, keeping |sum| <= 127 * 127 * keys below 2^31
constexpr int kMaxIntTiles = 32768 / BN;

template <int D>
struct DStage {
  alignas(16) int8_t v[BN * D];
  alignas(16) float sk[BN];
  alignas(16) float sv[BN];
};

// Key of the tile held by MFMA row r of key block b of S^T (16x16 C layout:
// lane l holds rows 4 (l / 16) + 0..3), chosen so that lane l ends up with
// keys 16 (l / 16) + 4 b + 0..3.
__device__ __forceinline__ int key_of_row16(int b, int r) { return 16 * (r >> 2) + 4 * b + (r & 3); }

template <int D>
struct DLanes {
  static constexpr int NC = D / 64;            // 64-channel chunks (K dim of QK)
  static constexpr int NCB = D / 16;           // 16-channel blocks of O
  static constexpr int NLD = BN * D / 1024;    // 1 KB LDS loads of V per tile
  uint32_t ld[NLD];
  // K operand of key block kb, channel chunk c: 16 bytes of key row
  // key_of_row16(kb & 1, r) + 8 (kb >> 1), channels 64 c + 16 grp; the byte
  // offset within the tile is kg[kb & 1] + (8 D (kb >> 1) + 64 c)
  uint32_t kg[2];
  int voff[NCB];       // transposed V read offset, channel block cb, keys +0..7 (+8 D: 8..15)

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) ld[n] = tile_load_off<D>(n, lane);
    const int r = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) kg[b] = static_cast<uint32_t>(key_of_row16(b, r) * D + 16 * grp);
    // lane 16 grp + i addresses key 16 grp + i / 2, channels 16 cb + 8 (i % 2)
    // .. +7, so after the transposing read lane l holds channel 16 cb + l % 16,
    // keys 16 (l / 16) .. +7
    const int vr = 16 * grp + (r >> 1);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) voff[cb] = vr * D + ((cb ^ swz<D>(vr)) * 16) + 8 * (r & 1);
  }
};

// K operand registers of one tile: key block kb, channel chunk c at kb NC + c
template <int D>
using KRegs = v4i[NB * (D / 64)];

// Packed 4-bit K (INT4 Q.K): the same operands at 8 bytes each. A key row is
// d / 2 bytes; in each group of 8 channels, byte j holds channel j in its low
// nibble and channel j + 4 in its high nibble, both stored as code + 8 (1..15).
template <int D>
using KRegs4 = v2i[NB * (D / 64)];

// After a wait that covered a slot's loads: passing the slot through an empty
// asm statement makes that point its definition for the compiler, which then
// adds no wait of its own before the MFMAs that read it.
template <int D>
__device__ __forceinline__ void landed(KRegs<D>& kr) {
#pragma unroll
  for (int i = 0; i < NB * (D / 64); ++i) asm volatile("" : "+v"(kr[i]));
}
template <int D>
__device__ __forceinline__ void landed(KRegs4<D>& kr) {
#pragma unroll
  for (int i = 0; i < NB * (D / 64); ++i) {
    double t = __builtin_bit_cast(double, kr[i]);    // a 64-bit register pair
    asm volatile("" : "+v"(t));
    kr[i] = __builtin_bit_cast(v2i, t);
  }
}

// 16 packed channels -> the 16 biased codes (1..15) of an INT8 operand: low
// nibbles are channels 0..3 of each 8-channel group, high nibbles 4..7.
__device__ __forceinline__ v4i unpack4(v2i p) {
  const int m = 0x0F0F0F0F;
  return v4i{p.x & m, (p.x >> 4) & m, p.y & m, (p.y >> 4) & m};
}

// Loads per tile issued by the (single) wavefront (all count in vmcnt).
template <int D, bool VPT>
constexpr int loads_per_tile() { return DLanes<D>::NLD + 1 + (VPT ? 1 : 0) + NB * (D / 64); }

// V tile and scales of the tile at key k0 into an LDS stage
template <int D, bool VPT>
__device__ __forceinline__ void request_vs(DStage<D>& st, __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t rsk,
                                           __amdgpu_buffer_rsrc_t rsv, const DLanes<D>& ln, int lane, int k0) {
  lds_load4_nt(rsk, st.sk, lane * 4, k0 * 4);
  if (VPT) lds_load4_nt(rsv, st.sv, lane * 4, k0 * 4);
  const uint32_t soff = static_cast<uint32_t>(k0) * D;
#pragma unroll
  for (int n = 0; n < DLanes<D>::NLD; ++n) lds_load16_nt(rv, st.v + n * 1024, ln.ld[n], soff);
}

// K operands of the tile at key k0 into a register slot
template <int D>
__device__ __forceinline__ void request_k(KRegs<D>& kr, __amdgpu_buffer_rsrc_t rk, const DLanes<D>& ln, int k0) {
  constexpr int NC = D / 64;
  const uint32_t soff = static_cast<uint32_t>(k0) * D;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[kb * NC + c] = buf_load16_nt(rk, ln.kg[kb & 1] + 8 * D * (kb >> 1) + 64 * c, soff);
}

// packed K operands of the tile at key k0 into a register slot (d / 2 bytes per key)
template <int D>
__device__ __forceinline__ void request_k(KRegs4<D>& kr, __amdgpu_buffer_rsrc_t rk, const DLanes<D>& ln, int k0) {
  constexpr int NC = D / 64;
  const uint32_t soff = static_cast<uint32_t>(k0) * (D / 2);
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kr[kb * NC + c] = buf_load8_nt(rk, ln.kg[kb & 1] / 2 + 4 * D * (kb >> 1) + 32 * c, soff);
}

// x of lane l ^ 16 (ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 within 32
// lanes); max / sum over a row's lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float row_max4(float x) {
  x = fmaxf(x, xor16(x));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  x = x + xor16(x);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Partial result of one (KV group, chunk): per row the running max m (base
// 2, -inf if the chunk had no visible key), 127 l, and acc[D] (fp32, frame m;
// per-tensor V without s_V).
struct Partials {
  float* acc;     // [groups][n_split][R][D]
  float* ml;      // [groups][n_split][R][2]
};

__device__ __forceinline__ Partials partials(void* ws, int groups, int n_split, int R, int D) {
  Partials p;
  p.acc = static_cast<float*>(ws);
  p.ml = p.acc + static_cast<int64_t>(groups) * n_split * R * D;
  return p;
}

// LUT: IndexSoftmax (table lookup) in place of the exp2 softmax; only with
// V scales constant along the keys (per tensor, head or channel) and INT8 Q.
// K4: K packed at 4 bits (INT4 Q.K); the biased codes k + 8 enter the MFMA
// and its accumulator starts at -8 sum_c q_c, so S_int is exact.
// QF: 0 INT8 Q; 1 fp16/fp32 Q quantized here; 2 the same after the
// normalized Hadamard rotation of each Q row.
template <int D, bool CAUSAL, bool VPT, int QF, bool LUT, bool K4>
// two wavefronts per SIMD (registers <= 256): the LDS ring allows six per CU
__global__ __launch_bounds__(64) ATTN_WAVES_PER_EU(2) void attn_decode_kernel(FwdArgs a, int split_len, int n_split) {
  static_assert(!LUT || (!VPT && !QF), "IndexSoftmax takes INT8 Q and V scales constant along the keys");
  static_assert(!K4 || (!LUT && !QF), "packed K with the exp softmax and INT8 Q");
  constexpr int NC = D / 64;
  constexpr int NCB = D / 16;
  constexpr int NL = loads_per_tile<D, VPT>();
  __shared__ DStage<D> sm[kStages];
  __shared__ uint32_t lut_s[LUT ? 65 : 1];
  // per-token V: the key multipliers s_V[j] / s_t of the current tile
  __shared__ float wr_s[VPT ? BN : 1];

  const int G = a.H / a.Hkv;                 // query heads per KV head
  const int R = G * a.Lq;                    // query rows of the group (<= 16)
  const int groups = a.B * a.Hkv;
  const int gi = blockIdx.x / n_split, split = blockIdx.x % n_split;
  const int b = gi / a.Hkv, hk = gi % a.Hkv;
  const int64_t kv_base = static_cast<int64_t>(gi) * a.Lkv;

  const int lane = threadIdx.x;
  const int grp = lane >> 4, r = lane & 15;
  const bool rvalid = r < R;
  const int head = hk * G + (rvalid ? r / a.Lq : 0);
  const int qi = rvalid ? r % a.Lq : 0;
  const int64_t qrow = (static_cast<int64_t>(b) * a.H + head) * a.Lq + qi;
  const int shift = a.Lkv - a.Lq;            // bottom-right causal alignment
  const int lim = CAUSAL ? qi + shift : a.Lkv - 1;   // last visible key of this row
  const int lim_first = CAUSAL ? shift : a.Lkv - 1;  // smallest over the rows

  // this chunk's keys [s0, s1), cut at the last key any row sees
  const int s0 = split * split_len;
  const int kv_end = CAUSAL ? min(a.Lkv, a.Lq - 1 + shift + 1) : a.Lkv;
  const int s1 = min(kv_end, s0 + split_len);
  const int n_tiles = s1 > s0 ? (s1 - s0 + BN - 1) / BN : 0;

  const __amdgpu_buffer_rsrc_t rk = K4 ? make_rsrc(a.k + kv_base * (D / 2), a.Lkv * (D / 2))
                                      : make_rsrc(a.k + kv_base * D, a.Lkv * D);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_base * D, a.Lkv * D);
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(a.s_k + kv_base, a.Lkv * 4);
  const __amdgpu_buffer_rsrc_t rsv = make_rsrc(VPT ? a.s_v + kv_base : a.s_k + kv_base, a.Lkv * 4);
  DLanes<D> ln;
  ln.init(lane);

  // Q fragment (B operand of S^T): 16 bytes per 64-channel chunk; s_Q. QF:
  // the row arrives in fp16/fp32 and is quantized here (the quantizer's
  // arithmetic; the row's 4 lanes share its absmax); an fp16 row is requested
  // whole here and converted after the first tile requests.
  v4i qf[NC];
  float sq = 0.0f;
  float xq[QF ? NC : 1][16];
  v4i q16[QF ? NC : 1][2];
  if constexpr (QF) {
    if (rvalid && a.q_float_f16) q16_load<NC>(a.q_float, qrow * D + grp * 16, 64, q16);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = zero4();
      if (rvalid) qf[c] = *reinterpret_cast<const v4i*>(a.q + qrow * D + c * 64 + grp * 16);
    }
    sq = rvalid ? a.s_q[qrow] : 0.0f;
  }

  // scale slots start at zero: a load past Lkv may leave a slot untouched
  for (int i = lane; i < kStages * BN; i += 64) {
    sm[i / BN].sk[i % BN] = 0.0f;
    sm[i / BN].sv[i % BN] = 0.0f;
  }
  if constexpr (LUT) {
    for (int i = lane; i < 65; i += 64) lut_s[i] = a.lut_w[i];
  }
  __syncthreads();
  // Every request is issued, also past the last tile: such a request starts at
  // key Lkv, where every lane's offset lies outside the buffers, so it fetches
  // nothing (the loads return 0). Unconditional loads keep the compiler's own
  // register waits exact.
  std::conditional_t<K4, KRegs4<D>, KRegs<D>> kr[2];   // K operands, slot t % 2 holds tile t
  const int k_first = n_tiles > 0 ? s0 : a.Lkv, k_second = n_tiles > 1 ? s0 + BN : a.Lkv;
  request_vs<D, VPT>(sm[0], rv, rsk, rsv, ln, lane, k_first);
  request_k<D>(kr[0], rk, ln, k_first);
  request_vs<D, VPT>(sm[1], rv, rsk, rsv, ln, lane, k_second);
  request_k<D>(kr[1], rk, ln, k_second);
  if constexpr (QF) {
    // the Q row, converted once the first tiles are requested
    if (rvalid) {
      if (a.q_float_f16) q16_f32<NC>(q16, xq);
      else q32_f32<NC>(a.q_float, qrow * D + grp * 16, 64, xq);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) xq[c][e] = 0.0f;
    }
  }
  if constexpr (QF == 2) {
    // Hadamard rotation of the row (the rotated quantizer's butterflies, strides
    // in increasing order): 1 .. 8 inside the lane's 16 channels, 16 and 32
    // across the row's lane groups (lanes l ^ 16, l ^ 32), 64 across the
    // lane's 64-channel chunks; then times rn
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
    {
      // stride 16 by a lane shuffle; stride 32 by v_permlane32_swap, which
      // hands lanes 0-31 (own, partner) and lanes 32-63 (partner, own), so one
      // fma gives own + partner below and partner - own above
      const float sgn16 = (lane & 16) ? -1.0f : 1.0f, sgn32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) xq[c][e] = __builtin_fmaf(sgn16, xq[c][e], __shfl_xor(xq[c][e], 16, 64));
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(xq[c][e]), __float_as_uint(xq[c][e]), false, false);
          xq[c][e] = __builtin_fmaf(sgn32, __uint_as_float(r[1]), __uint_as_float(r[0]));
        }
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
    am = row_max4(am);
    const float r = quant_recip(am);
    sq = quant_scale(am);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = v4i{static_cast<int>(quant_word(&xq[c][0], r)), static_cast<int>(quant_word(&xq[c][4], r)),
                  static_cast<int>(quant_word(&xq[c][8], r)), static_cast<int>(quant_word(&xq[c][12], r))};
    // each row of the group is written by exactly one chunk's wavefront
    if (rvalid && split == 0) {
      if (a.q_hat_out) {
#pragma unroll
        for (int c = 0; c < NC; ++c) *reinterpret_cast<v4i*>(a.q_hat_out + qrow * D + c * 64 + grp * 16) = qf[c];
      }
      if (a.s_q_out && grp == 0) a.s_q_out[qrow] = sq;
    }
  }
  wait_vm_lds<NL>();                   // tile 0 (and the Q loads, issued first) landed
  landed<D>(kr[0]);
  // the wait covered the Q loads too; tell the compiler
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
  asm volatile("" : "+v"(sq));

  const float inv_sqrt_d = (D == 64) ? 0.125f : static_cast<float>(0.08838834764831845);
  // The running max m is in base-2 logits, as in the prefill kernel: exp
  // softmax, the oracle's fp32 running max of u = (S_int aq) s_K[j] with aq =
  // s_Q log2(e) / sqrt(d); IndexSoftmax, the max of u times c2 = s_Q log2 e /
  // sqrt(d) (kept >= FLT_MIN: -inf * c2 stays -inf)
  const float aq = sq * kLogitScale<D>;
  const float c2 = fmaxf(sq * inv_sqrt_d * kLog2e, kFltMin);
  // packed K: the QK accumulator starts at -8 sum_c q_c (the codes' bias)
  int s_init = 0;
  if constexpr (K4) {
    int qs = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) qs = __builtin_amdgcn_sdot4(qf[c][i], 0x01010101, qs, false);
    s_init = -8 * static_cast<int>(row_sum4(static_cast<float>(qs)));
  }
  // IndexSoftmax: table index per unit of u below the running max of u
  const float kap = (sq * inv_sqrt_d) * a.lut_k;
  const float nf = static_cast<float>(a.lut_n);
  float m_u = kNegInf;

  float m = kNegInf, l = 0.0f;
  float acc[NCB][4];
  v4i acc_i[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    acc_i[cb] = zero4();
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[cb][v] = 0.0f;
  }
  float m_f = kNegInf;
  int int_tiles = 0;

  // One tile t with K in register slot S = t % 2 (a compile-time index, so the
  // slots stay in registers): request V and scales of t+2 | QK | request K of
  // t+2 into slot S | softmax | PV | wait for t+1. The LDS stage read and the
  // stage filled are passed as restrict pointers so the compiler adds no waits
  // for the loads just issued.
  auto step = [&](auto slot, int t, const DStage<D>* __restrict__ st, DStage<D>* __restrict__ nx)
                  __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    const int k0 = s0 + t * BN;
    const int kq = t + 2 < n_tiles ? k0 + 2 * BN : a.Lkv;
    request_vs<D, VPT>(*nx, rv, rsk, rsv, ln, lane, kq);

    // S^T = K_hat . Q_hat^T, exact INT32
    v4i s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) s[kb] = K4 ? v4i{s_init, s_init, s_init, s_init} : zero4();
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        if constexpr (K4) s[kb] = mfma16(unpack4(kr[S][kb * NC + c]), qf[c], s[kb]);
        else s[kb] = mfma16(kr[S][kb * NC + c], qf[c], s[kb]);
      }
    request_k<D>(kr[S], rk, ln, kq);

    // exp softmax: the base-2 logit u = (float(S_int) aq) s_K[j], the
    // oracle's two rounded fp32 products; IndexSoftmax: u = S_int s_K[j].
    // -inf past the chunk
    // end or the causal limit; key 16 grp + 4 kb + e of the tile is visible
    // iff 4 kb + e <= rel
    const bool mask = (k0 + BN > s1) || (CAUSAL && k0 + BN - 1 > lim_first);
    const int rel = min(lim, s1 - 1) - k0 - 16 * grp;
    float u[NB][4];
    float gm[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const float4 skv = *reinterpret_cast<const float4*>(st->sk + grp * 16 + kb * 4);
      const float skk[4] = {skv.x, skv.y, skv.z, skv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = static_cast<float>(s[kb][e]);
        if constexpr (!LUT) {
          x = (x * aq) * skk[e];
        } else {
          x = x * skk[e];
        }
        u[kb][e] = (!mask || kb * 4 + e <= rel) ? x : kNegInf;
      }
      gm[kb] = fmaxf(fmaxf(u[kb][0], u[kb][1]), fmaxf(u[kb][2], u[kb][3]));
    }
    const float mx = row_max4(fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3])));

    // online softmax (IndexSoftmax: c2 > 0, so max(u) c2 == max(u c2))
    const float mx2 = !LUT ? mx : (mx == kNegInf) ? kNegInf : mx * c2;
    const float m_new = fmaxf(m, mx2);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = exp2_hw(m - m_use);
    float st_cur = 0.0f;
    uint32_t pw[NB];
    float lsum;
    if constexpr (LUT) {
      // IndexSoftmax: E = table[min(floor(max(m_u kappa - u kappa, 0)), n)],
      // masked keys read the zero slot; integer row sum by dot4
      m_u = fmaxf(m_u, mx);
      const float mu = m_u * kap;
      const uint8_t* tab = reinterpret_cast<const uint8_t*>(lut_s);
      uint32_t isum = 0;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = __builtin_amdgcn_fmed3f(__builtin_fmaf(u[kb][e], -kap, mu), 0.0f, nf);
          uint32_t idx = static_cast<uint32_t>(x);
          idx = (!mask || kb * 4 + e <= rel) ? idx : static_cast<uint32_t>(kLutZero);
          word |= static_cast<uint32_t>(tab[idx]) << (8 * e);
        }
        isum = __builtin_amdgcn_udot4(word, 0x01010101u, isum, false);
        pw[kb] = word;
      }
      lsum = static_cast<float>(isum);
    } else {
      if constexpr (VPT) {
        // s_t: largest s_V[j] over the tile's keys inside the chunk; then the
        // multiplier of this lane's key, s_V[j] / s_t as the oracle's one
        // rounded division, shared through LDS (a wavefront's LDS accesses
        // execute in order; the wave barrier keeps the reads after the write)
        const float svl = (k0 + lane < s1) ? st->sv[lane] : 0.0f;
        st_cur = wave_max_nonneg(svl);
        wr_s[VPT ? lane : 0] = st_cur > 0.0f ? __fdiv_rn(svl, st_cur) : 0.0f;
        __builtin_amdgcn_wave_barrier();
      }
      const float eb = exp_bias(m_use);
      float gs[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        float wr[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (VPT) {
          const float4 w4 = *reinterpret_cast<const float4*>(wr_s + grp * 16 + kb * 4);
          wr[0] = w4.x; wr[1] = w4.y; wr[2] = w4.z; wr[3] = w4.w;
        }
        uint32_t word = 0;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // 127 P_tilde = 2^(u - eb), the oracle's rounded difference
          y[e] = exp2_hw(u[kb][e] - eb);
          word = __builtin_amdgcn_cvt_pk_u8_f32(VPT ? y[e] * wr[e] : y[e], e, word);
        }
        gs[kb] = (y[0] + y[1]) + (y[2] + y[3]);
        pw[kb] = word;
      }
      lsum = (gs[0] + gs[1]) + (gs[2] + gs[3]);
    }
    const v4i p = v4i{static_cast<int>(pw[0]), static_cast<int>(pw[1]), static_cast<int>(pw[2]),
                      static_cast<int>(pw[3])};
    l = __builtin_fmaf(alpha, l, lsum);

    if constexpr (!VPT) {
      if (__any(m_new > m) || ++int_tiles > kMaxIntTiles) {
        // fold the INT32 run (frame m) into acc (frame m_f)
        if (m_f == kNegInf) m_f = m_use;
        float f = exp2_hw(m - m_f);
        if (__any(m_use - m_f > kRebase)) {
          const float rb = exp2_hw(m_f - m_use);
          f *= rb;
          m_f = m_use;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[cb][v] *= rb;
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[cb][v] = __builtin_fmaf(f, static_cast<float>(acc_i[cb][v]), acc[cb][v]);
          acc_i[cb] = zero4();
        }
        int_tiles = 1;
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc_i[cb] = zero4();
    }
    m = m_new;

    // O^T += V_hat^T . P_hat^T
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const v2i lo = lds_read_tr8(st->v + ln.voff[cb]);
      const v2i hi = lds_read_tr8(st->v + ln.voff[cb] + 8 * D);
      acc_i[cb] = mfma16(v4i{lo.x, lo.y, hi.x, hi.y}, p, acc_i[cb]);
    }
    if constexpr (VPT) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[cb][v] = __builtin_fmaf(alpha, acc[cb][v], st_cur * static_cast<float>(acc_i[cb][v]));
    }

    // tile t+1 must have landed; this wavefront is the stage ring's only user
    wait_vm_lds<NL>();
    landed<D>(kr[1 - S]);
  };

  int s_cur = 0;                       // LDS stage of tile t; tile t+2 goes to the one before it
  auto next = [](int i) { return i == kStages - 1 ? 0 : i + 1; };
  auto prev = [](int i) { return i == 0 ? kStages - 1 : i - 1; };
  // pairs of tiles (slots 0, 1) with no branch between them, then an odd last
  // tile: the K slots then stay in fixed registers across the loop
  int t = 0;
  for (; t + 2 <= n_tiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t, &sm[s_cur], &sm[prev(s_cur)]);
    s_cur = next(s_cur);
    step(std::integral_constant<int, 1>{}, t + 1, &sm[s_cur], &sm[prev(s_cur)]);
    s_cur = next(s_cur);
  }
  if (t < n_tiles) step(std::integral_constant<int, 0>{}, t, &sm[s_cur], &sm[prev(s_cur)]);
  wait_vm_lds<0>();                    // the last (empty) requests, before the LDS is released

  if constexpr (!VPT) {
    const float back = (m == kNegInf) ? 0.0f : exp2_hw(m_f - m);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[cb][v] = __builtin_fmaf(back, acc[cb][v], static_cast<float>(acc_i[cb][v]));
  }
  const float ltot = row_sum4(l);
  if (!rvalid) return;
  const Partials pt = partials(a.workspace, groups, n_split, R, D);
  const int64_t prow = (static_cast<int64_t>(gi) * n_split + split) * R + r;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<float4*>(pt.acc + prow * D + cb * 16 + grp * 4) =
        make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
  // the partial's max (base 2, -inf stays -inf): the merge weighs chunks by 2^(m_s - M)
  if (grp == 0) *reinterpret_cast<float2*>(pt.ml + prow * 2) = make_float2(m, ltot);
}

// Merge of the chunk partials of one query row per wavefront:
// O = sum_s 2^(m_s - M) acc_s * scale / sum_s 2^(m_s - M) 127 l_s.
template <int D, bool OUT_F16>
__global__ __launch_bounds__(256) void attn_decode_combine(FwdArgs a, int n_split) {
  constexpr int CPL = D / 64;                // channels per lane
  const int G = a.H / a.Hkv;
  const int R = G * a.Lq;
  const int groups = a.B * a.Hkv;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(a.B) * a.H * a.Lq) return;
  const int lane = threadIdx.x & 63;
  const int qi = static_cast<int>(row % a.Lq);
  const int head = static_cast<int>((row / a.Lq) % a.H);
  const int b = static_cast<int>(row / (static_cast<int64_t>(a.Lq) * a.H));
  const int gi = b * a.Hkv + head / G;
  const int r = (head % G) * a.Lq + qi;
  const Partials pt = partials(a.workspace, groups, n_split, R, D);
  const int64_t p0 = static_cast<int64_t>(gi) * n_split * R + r;   // split s: p0 + s R

  float M = kNegInf;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, pt.ml[(p0 + static_cast<int64_t>(s) * R) * 2]);
  float L = 0.0f, o[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.0f;
  for (int s = 0; s < n_split; ++s) {
    const int64_t pr = p0 + static_cast<int64_t>(s) * R;
    const float ms = pt.ml[pr * 2];
    if (ms == kNegInf) continue;
    const float f = exp2_hw(ms - M);
    L = __builtin_fmaf(f, pt.ml[pr * 2 + 1], L);
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = __builtin_fmaf(f, pt.acc[pr * D + lane * CPL + c], o[c]);
  }
  const float scale = (a.v_per_token ? 1.0f : a.s_v[a.v_per_head ? gi : 0]) / L;
  const float rl = 1.0f / L;
  float cs[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c)   // per-channel V: each channel its own scale
    cs[c] = a.v_per_channel ? a.s_v[static_cast<int64_t>(gi) * D + lane * CPL + c] * rl : scale;
  if constexpr (OUT_F16) {
    __half* out = static_cast<__half*>(a.o) + row * D + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = __float2half_rn(o[c] * cs[c]);
  } else {
    float* out = static_cast<float*>(a.o) + row * D + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = o[c] * cs[c];
  }
  if (a.lse && lane == 0) a.lse[row] = (M + __builtin_log2f(L) - kLog2_127) * kLn2;
}

template <int D, bool CAUSAL, bool VPT>
hipError_t launch_dec(const FwdArgs& a, int split_len, int n_split, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.Hkv * n_split));
  if (a.q_float && a.q_rotate)
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, VPT, 2, false, false>), grid, dim3(64), 0, st, a, split_len, n_split);
  else if (a.q_float)
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, VPT, 1, false, false>), grid, dim3(64), 0, st, a, split_len, n_split);
  else if (a.k_int4)
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, VPT, 0, false, true>), grid, dim3(64), 0, st, a, split_len, n_split);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, VPT, 0, false, false>), grid, dim3(64), 0, st, a, split_len, n_split);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dec_lut(const FwdArgs& a, int split_len, int n_split, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.Hkv * n_split));
  hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, false, 0, true, false>), grid, dim3(64), 0, st, a, split_len, n_split);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int split_len, int n_split, hipStream_t st) {
  if (a.lut_n) return a.causal ? launch_dec_lut<D, true>(a, split_len, n_split, st)
                               : launch_dec_lut<D, false>(a, split_len, n_split, st);
  if (a.causal) return a.v_per_token ? launch_dec<D, true, true>(a, split_len, n_split, st)
                                     : launch_dec<D, true, false>(a, split_len, n_split, st);
  return a.v_per_token ? launch_dec<D, false, true>(a, split_len, n_split, st)
                       : launch_dec<D, false, false>(a, split_len, n_split, st);
}

template <int D>
hipError_t launch_combine(const FwdArgs& a, int n_split, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.H * a.Lq;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (a.o_f16) hipLaunchKernelGGL((attn_decode_combine<D, true>), grid, dim3(256), 0, st, a, n_split);
  else hipLaunchKernelGGL((attn_decode_combine<D, false>), grid, dim3(256), 0, st, a, n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, int split_len, hipStream_t st) {
  const int n_split = (a.Lkv + split_len - 1) / split_len;
  hipError_t e = a.d == 64 ? launch_d<64>(a, split_len, n_split, st) : launch_d<128>(a, split_len, n_split, st);
  if (e != hipSuccess) return e;
  return a.d == 64 ? launch_combine<64>(a, n_split, st) : launch_combine<128>(a, n_split, st);
}

}  // namespace attn
