// CPU oracle for the fully-INT8 FlashAttention-style attention forward.
//
// TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously-correct
// statement of what the GPU library computes. Only the tests, the smoke check
// and the CPU-baseline leg of the benchmark load it. It shares no code, header,
// table or helper with the HIP library, and the HIP library never calls it.
//
// Sources (the method is stated in the pages listed here; every step below
// names the passage it follows):
//  [IFA]  "INT-FlashAttention: Enabling Flash Attention for INT8 Quantization",
//         abstract: FlashAttention forward with fully INT8 Q/K/V input and
//         token-level (one scale per row) post-training quantization.
//  [IA]   "IntAttention: A Fully Integer Attention Pipeline for Efficient Edge
//         Inference", §2.1 (standard scaled-dot-product attention; symmetric
//         INT8 quantization with zero point 0 and scale absmax/127, Eq. 3;
//         integer logits with INT32 accumulation; output O ~ s_V * P * V_hat),
//         §2.2 (max-subtracted stable softmax), §3.1 (logit rescale factor
//         alpha = s_Q s_K / sqrt(d), Eq. 4; IndexSoftmax: clipping of the
//         distance to the row max at c, a 2^b-entry exponential table indexed
//         by floor(distance / c * (2^b - 1))), §3.2 (prior methods quantize
//         the probabilities as signed INT8 with a multiplier of 127; integer
//         row sum and normalisation of the table's values), §4 ablation
//         (recommended (b, c) = (5, 6.6)).
//  [FA3]  "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
//         Low-precision", abstract: tiled attention with the softmax fused
//         block by block (online softmax).
//  [FA3] also lists incoherent processing (a Hadamard rotation of Q and K
//         before low-precision quantization, to spread outliers).
//  [LLMI8] "LLM.int8(): 8-bit Matrix Multiplication for Transformers at Scale",
//         abstract: vector-wise quantization, i.e. one scale per row of the
//         left operand times one scale per column of the right operand.
//
// Readings of points the pages leave open (each is also listed in the design
// notes of the repository):
//  * quantizer: q = clamp(rne(x * r), -127, 127) with r = 127/a and s = a/127,
//    a = absmax of the group; x*r is one rounded fp32 multiply; an all-zero
//    group gets s = 0 and q = 0.
//  * logits in base 2: t = (S_int * (s_Q * c)) * s_K[j] in fp32, with
//    c = fl32(log2(e) / sqrt(d)); e^(S - m) is then 2^(t - m') (the
//    rescale factor alpha = s_Q s_K / sqrt(d) of IA §3.1, Eq. 4, times
//    log2(e), its row part formed once per row).
//  * 127 P_tilde = y = 2^(t - b(m')), b(m') = m' - log2(127) in fp32 (moved
//    up one float when m' - b still exceeds log2(127), see exp_bias), with
//    fp32 exp2 of the fp32 difference.
//  * per-token V inside the INT8 P.V product: the scale of tile t is
//    s_t = max of s_V over the tile's in-range keys; key j's probability is
//    quantized with multiplier w_j = s_V[j] / s_t (one rounded fp32
//    division) on y.
//  * P_hat = rne(fl32(y * w)): the product rounded to fp32 first, the
//    precision of the code decision; w = 1 for per-tensor V.
//  * per-head V (one scale per (batch, kv head), a block granularity that
//    IA §3.3 lists as compatible): the tile scale is that head's s_V and
//    w = 1, i.e. the per-tensor arithmetic with the head's own scale.
//  * per-channel V (one scale per (batch, kv head, channel), the per-channel
//    granularity of IA §3.3): the scale is constant along the keys, so the
//    tile sums carry no V scale (s_t = 1, w = 1) and channel c of the
//    output is multiplied by its scale at the end.
//  * the running max used to quantize a tile is the max after that tile (m').
//  * rowsum l accumulates the fp32 y = 127 P_tilde before quantization, and
//    O = acc / l.
//  * INT32 accumulation inside a tile, fp32 across tiles.
//  * causal mask is bottom-right aligned: query i sees key j iff
//    j <= i + (Lkv - Lq).
//  * GQA: query head h reads kv head h / (H / Hkv).
//  * 1/sqrt(d) (IndexSoftmax) and log2(e)/sqrt(d) (exp softmax) are the fp32
//    roundings of the double values.
//  * IndexSoftmax: see index_softmax_lut and attend_row_lut below (table
//    sampled at the left end of each index bucket with multiplier 127; the
//    distance taken on the dequantized logit; online rescale by exp; the
//    normalisation by the integer row sum at the output).
//
// Build: g++ -std=c++17 -O2 -fno-fast-math -ffp-contract=off -fPIC -shared
//        -pthread (see oracle/build.py). -ffp-contract=off keeps every fp32
//        multiply and add separately rounded, as the steps below state them.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

#ifdef ORACLE_PLANT
// A planted mistake (compiled only into throw-away test builds, never into the
// oracle the tests compare against) to show that the pins catch it.
#define PLANT(name) (std::strcmp(ORACLE_PLANT, name) == 0)
#else
#define PLANT(name) false
#endif

namespace {

// ---------------------------------------------------------------------------
// IEEE binary16 codec, written from the format's definition (1 sign bit,
// 5 exponent bits with bias 15, 10 fraction bits, subnormals at exponent 0).
// ---------------------------------------------------------------------------
float half_bits_to_float(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h >> 15) << 31;
  const uint32_t e = (h >> 10) & 0x1fu;
  const uint32_t f = h & 0x3ffu;
  uint32_t bits;
  if (e == 0) {
    // subnormal or zero: f * 2^-24, exact in fp32 (f < 2^10, power-of-two factor)
    const float mag = static_cast<float>(f) * 5.9604644775390625e-8f;
    std::memcpy(&bits, &mag, 4);
    bits |= sign;
  } else if (e == 31) {
    bits = sign | 0x7f800000u | (f << 13);     // infinity or NaN
  } else {
    // normal: same value with the exponent re-biased from 15 to 127
    bits = sign | ((e + 112u) << 23) | (f << 13);
  }
  float out;
  std::memcpy(&out, &bits, 4);
  return out;
}

// Round-to-nearest-even encoding of an fp32 value as binary16.
uint16_t float_to_half_bits(float x) {
  uint32_t bits;
  std::memcpy(&bits, &x, 4);
  const uint16_t sign = static_cast<uint16_t>((bits >> 16) & 0x8000u);
  const double a = std::fabs(static_cast<double>(x));
  if (std::isnan(x)) return sign | 0x7e00u;
  if (a >= 65520.0) return sign | 0x7c00u;  // rounds to infinity
  if (a < std::ldexp(1.0, -14)) {
    // subnormal grid: multiples of 2^-24
    const double n = std::nearbyint(a * std::ldexp(1.0, 24));  // exact scaling
    return sign | static_cast<uint16_t>(n);  // n == 1024 encodes 2^-14 exactly
  }
  int e2;
  std::frexp(a, &e2);     // a = m * 2^e2 with m in [0.5, 1)
  int E = e2 - 1;         // a in [2^E, 2^(E+1))
  double n = std::nearbyint(std::ldexp(a, 10 - E));  // in [1024, 2048]
  if (n >= 2048.0) { n = 1024.0; ++E; }
  if (E + 15 >= 31) return sign | 0x7c00u;
  return sign | static_cast<uint16_t>(((E + 15) << 10) | (static_cast<int>(n) - 1024));
}

// ---------------------------------------------------------------------------
// Symmetric INT8 quantization of one group (IA §2.1, Eq. 3; IFA abstract for
// the token-level granularity).
// ---------------------------------------------------------------------------
// qmax = 2^(bits - 1) - 1: 127 for INT8; 7 for the 4-bit codes of INT4 Q.K
// (the same symmetric form with 7 levels on each side; INT-FlashAttention's
// abstract names INT4 as a format the scheme carries over to).
void quantize_group(const float* x, int64_t n, int8_t* q, float* s_out, float qmax = 127.0f) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i) a = std::max(a, std::fabs(x[i]));
  if (a == 0.0f) {
    *s_out = 0.0f;
    for (int64_t i = 0; i < n; ++i) q[i] = 0;
    return;
  }
  const float s = a / qmax;     // stored scale: X ~ s * X_hat
  const float r = qmax / a;     // multiplier applied to every element
  *s_out = s;
  for (int64_t i = 0; i < n; ++i) {
    const float y = x[i] * r;                  // one rounded fp32 multiply
    float t = PLANT("quant_round_away") ? std::round(y) : std::nearbyint(y);
    t = std::min(qmax, std::max(-qmax, t));
    q[i] = static_cast<int8_t>(t);
  }
}

// Exact integer dot product of two int8 rows (IA §2.1: INT8 x INT8 products
// accumulated in 32-bit integers).
int32_t dot_i8(const int8_t* a, const int8_t* b, int d) {
  int32_t acc = 0;
  for (int c = 0; c < d; ++c) acc += static_cast<int32_t>(a[c]) * static_cast<int32_t>(b[c]);
  return acc;
}

struct Problem {
  const int8_t* q; const float* s_q;
  const int8_t* k; const float* s_k;
  const int8_t* v; const float* s_v;
  int v_mode;    // V scales: 0 one per tensor, 1 per token, 2 per (batch, kv head),
                 // 3 per (batch, kv head, channel)
  int B, H, Hkv, Lq, Lkv, d, causal;
  int kv_tile, kv_split_len;
  int lut_bits;  // 0: exp softmax; b >= 1: IndexSoftmax with a 2^b-entry table
  float clip;    // IndexSoftmax clipping threshold c (natural-log units)
};

// Per-key trace of one row, for the invariant tests.
struct RowTrace {
  float* t;        // [Lkv] dequantized logit in base 2, S log2(e) (-inf if masked)
  float* m_tile;   // [Lkv] running max m' of t used for the key's tile
  float* y;        // [Lkv] 127 P_tilde as computed: 2^(t - b(m'))
  int32_t* p_hat;  // [Lkv] quantized probability rne(y w)
  float* w;        // [Lkv] multiplier of y (1, or s_V[j] / s_t for per-token V)
  float* split_m;  // [Lkv] final running max of the key's split
};

// log2(127) as an fp32 value.
const float kLog2_127 = static_cast<float>(std::log2(127.0));

// The exponent bias of a running max m (base-2 units): b = m - log2(127) in
// fp32, moved up to the next float when m - b still exceeds log2(127) after
// rounding. Then every visible key has t - b <= log2(127) in fp32, so
// 2^(t - b) stays at or below 127 (plus the exponential's own rounding) and
// the probability code never exceeds 127, whatever the size of m.
float exp_bias(float m) {
  float b = m - kLog2_127;
  if (!PLANT("no_bias_nudge") && m - b > kLog2_127) b = std::nextafter(b, std::numeric_limits<float>::infinity());
  return b;
}

// One query row, step by step. Returns O[d] (fp32) and lse.
void attend_row(const Problem& P, int b, int h, int i, float* o, float* lse, RowTrace* tr) {
  const int d = P.d;
  const int group = P.H / P.Hkv;
  const int hk = PLANT("gqa_wrong_head") ? (h % P.Hkv) : (h / group);  // GQA mapping
  const int64_t qrow = (static_cast<int64_t>(b) * P.H + h) * P.Lq + i;
  const int8_t* qv = P.q + qrow * d;
  const float sq = P.s_q[qrow];
  const int64_t kv_base = (static_cast<int64_t>(b) * P.Hkv + hk) * P.Lkv;
  const int8_t* kmat = P.k + kv_base * d;
  const int8_t* vmat = P.v + kv_base * d;
  const float* sk = P.s_k + kv_base;
  const float* sv = P.v_mode == 1 ? (P.s_v + kv_base)
                  : P.v_mode == 2 ? (P.s_v + (PLANT("v_head_no_batch") ? hk : static_cast<int64_t>(b) * P.Hkv + hk))
                  : P.v_mode == 3 ? (P.s_v + (PLANT("v_channel_no_head") ? 0 : (static_cast<int64_t>(b) * P.Hkv + hk) * d))
                  : P.s_v;

  // Bottom-right aligned causal mask: last visible key of this row.
  int64_t last = P.Lkv - 1;
  if (P.causal) {
    last = static_cast<int64_t>(i) + (P.Lkv - P.Lq);
    if (PLANT("causal_off_by_one")) last -= 1;
  }
  // Base-2 logit factor of the row: the rescale factor alpha = s_Q s_K / sqrt(d)
  // (IA §3.1, Eq. 4) times log2(e), so that e^(S - m) = 2^(t - m') with
  // t = S log2(e). The row's part a = s_Q c is formed once, with c = log2(e) /
  // sqrt(d) rounded to fp32; each key's scale multiplies after it.
  const double c_d = PLANT("no_log2e") ? 1.0 / std::sqrt(static_cast<double>(d))
                                       : 1.0 / (std::log(2.0) * std::sqrt(static_cast<double>(d)));
  const float c = static_cast<float>(c_d);
  const float a = sq * c;
  const float NEG_INF = -std::numeric_limits<float>::infinity();

  const int Bc = P.kv_tile;
  const int split_len = P.kv_split_len > 0 ? P.kv_split_len : P.Lkv;
  const int n_splits = (P.Lkv + split_len - 1) / split_len;

  std::vector<float> acc(d), S(Bc), yv(Bc), w(Bc);
  std::vector<int32_t> ph(Bc), T(d);
  std::vector<float> sm(n_splits), sl(n_splits), sacc(static_cast<size_t>(n_splits) * d);

  for (int sp = 0; sp < n_splits; ++sp) {
    const int s0 = sp * split_len;
    const int s1 = std::min(P.Lkv, s0 + split_len);
    // Online softmax state of this split (FA3 abstract: softmax fused tile by
    // tile; IA §2.2: max-subtracted stable softmax), in base-2 logit units.
    float m = NEG_INF, l = 0.0f;
    std::fill(acc.begin(), acc.end(), 0.0f);
    for (int t0 = s0; t0 < s1; t0 += Bc) {         // ascending tile order
      const int t1 = std::min(s1, t0 + Bc);
      const int n = t1 - t0;
      // Dequantized logits in base 2: t = (S_int * a) * s_K[j], two rounded
      // fp32 products (IA §2.1 integer logits; the per-row x per-column scale
      // product is LLM.int8()'s vector-wise form).
      float mt = NEG_INF;
      for (int jj = 0; jj < n; ++jj) {
        const int j = t0 + jj;
        if (j > last) { S[jj] = NEG_INF; continue; }
        const int32_t s_int = dot_i8(qv, kmat + static_cast<int64_t>(j) * d, d);
        float x = static_cast<float>(s_int) * a;
        if (!PLANT("drop_sk")) x = x * sk[j];
        S[jj] = x;
        mt = std::max(mt, x);
      }
      const float m_new = std::max(m, mt);
      if (m_new == NEG_INF) continue;                // nothing visible yet
      float alpha = (m == NEG_INF) ? 0.0f : std::exp2(m - m_new);
      if (PLANT("alpha_sign")) alpha = (m == NEG_INF) ? 0.0f : std::exp2(m_new - m);
      if (PLANT("no_alpha")) alpha = (m == NEG_INF) ? 0.0f : 1.0f;
      const float eb = PLANT("bias_sign") ? m_new + kLog2_127 : exp_bias(m_new);
      // Scale of this tile's V contribution and per-key multipliers of y.
      float st;
      if (P.v_mode == 1) {
        st = 0.0f;
        for (int jj = 0; jj < n; ++jj) st = std::max(st, sv[t0 + jj]);
      } else if (P.v_mode == 3) {
        st = 1.0f;       // per-channel scales multiply the output channels
      } else {
        st = sv[0];
      }
      float lsum = 0.0f;
      for (int jj = 0; jj < n; ++jj) {
        // y = 127 P_tilde = 2^(t - b(m')): the C library's fp32 exp2 of the
        // fp32 difference
        const float y = (S[jj] == NEG_INF) ? 0.0f : std::exp2(S[jj] - eb);
        yv[jj] = y;
        lsum += y;
        float wj;
        if (P.v_mode == 1) wj = (st > 0.0f) ? sv[t0 + jj] / st : 0.0f;
        else wj = 1.0f;
        w[jj] = wj;
        // P_hat = rne(127 P_tilde w): signed INT8 probabilities with
        // multiplier 127 (IA §3.2 describes this as the prior methods'
        // choice); y w is one rounded fp32 product (exact when w = 1), the
        // precision in which the kernels take the same decision.
        const float yw = y * wj;
        ph[jj] = static_cast<int32_t>(std::nearbyint(yw));
      }
      l = PLANT("l_no_rescale") ? (l + lsum) : (alpha * l + lsum);
      // T = P_hat . V_hat over this tile, exact in INT32.
      for (int c2 = 0; c2 < d; ++c2) T[c2] = 0;
      for (int jj = 0; jj < n; ++jj) {
        if (ph[jj] == 0) continue;
        const int8_t* vr = vmat + static_cast<int64_t>(t0 + jj) * d;
        for (int c2 = 0; c2 < d; ++c2) {
          const int8_t vv = PLANT("transpose_v") ? vmat[static_cast<int64_t>(c2 % P.Lkv) * d + ((t0 + jj) % d)] : vr[c2];
          T[c2] += ph[jj] * static_cast<int32_t>(vv);
        }
      }
      // fp32 accumulation across tiles: acc = alpha * acc + s_t * T
      // (IA §2.1: O ~ s_V * P * V_hat).
      for (int c2 = 0; c2 < d; ++c2) acc[c2] = alpha * acc[c2] + st * static_cast<float>(T[c2]);
      m = m_new;
      if (tr) {
        for (int jj = 0; jj < n; ++jj) {
          const int j = t0 + jj;
          tr->t[j] = S[jj]; tr->m_tile[j] = m_new; tr->y[j] = yv[jj];
          tr->p_hat[j] = ph[jj]; tr->w[j] = w[jj];
        }
      }
    }
    sm[sp] = m; sl[sp] = l;
    std::copy(acc.begin(), acc.end(), sacc.begin() + static_cast<size_t>(sp) * d);
    if (tr) for (int j = s0; j < s1; ++j) tr->split_m[j] = m;
  }

  // Merge the splits by their maxima (same identity as the tile rescale).
  float M = NEG_INF;
  for (int sp = 0; sp < n_splits; ++sp) M = std::max(M, sm[sp]);
  float L = 0.0f;
  std::fill(acc.begin(), acc.end(), 0.0f);
  for (int sp = 0; sp < n_splits; ++sp) {
    if (sm[sp] == NEG_INF) continue;
    const float f = std::exp2(sm[sp] - M);
    L += f * sl[sp];
    for (int c2 = 0; c2 < d; ++c2) acc[c2] += f * sacc[static_cast<size_t>(sp) * d + c2];
  }
  // Output: O = acc / l, l = sum of 127 P_tilde; s_V is already inside acc,
  // except per-channel scales, which multiply their channel here.
  for (int c2 = 0; c2 < d; ++c2) {
    const float sc = P.v_mode == 3 ? sv[PLANT("v_channel_transposed") ? (c2 * 7) % d : c2] : 1.0f;
    o[c2] = (acc[c2] * sc) / L;
  }
  // natural log of sum_j e^(S_j) = ln 2 * (M - log2(127) + log2(l))
  if (lse) *lse = static_cast<float>((static_cast<double>(M) - std::log2(127.0) + std::log2(static_cast<double>(L))) *
                                     std::log(2.0));
}

// ---------------------------------------------------------------------------
// IndexSoftmax (IA §3.1 "IndexSoftmax": integer-domain clipping and the
// table-driven exponential; IA §3.2: integer row sum and normalisation),
// read for this path's per-token scales and online tiles.
//
// Table: 2^b entries over the clipped distance range [0, c]; entry i stands
// for the exponential at the left end of its index bucket, i.e. distance
// c * i / (2^b - 1), as a signed 7-bit probability (the INT8 products are
// signed, so the multiplier is 127 as for the exp path, not 255):
//   LUT[i] = rne(127 * exp(-x_i)),  x_i = (double)c * i / (2^b - 1)
// evaluated in double, left to right.
void index_softmax_lut(int bits, float c, int32_t* lut) {
  const int n = (1 << bits) - 1;
  for (int i = 0; i <= n; ++i) {
    double x = static_cast<double>(c) * static_cast<double>(i) / static_cast<double>(n);
    if (PLANT("lut_half_step")) x = x * 0.5;
    lut[i] = static_cast<int32_t>(std::nearbyint(127.0 * std::exp(-x)));
  }
}

// One query row with IndexSoftmax in place of exp.
//
// The pages define the distance on the integer logits of per-tensor scales
// (Delta = rowmax(A_hat) - A_hat, c_int = round(c sqrt(d) / (s_Q s_K)),
// idx = floor(min(Delta, c_int) / c_int * (2^b - 1))). With one scale per
// key, integer distances no longer measure logit differences, so the
// distance is taken on the dequantized logit instead, which is the pages'
// formula with c_int replaced by its exact value c / alpha:
//   u_j   = S_int[j] * s_K[j]                        (fp32)
//   m_u   = running max of u over the visible keys so far (this tile included)
//   kappa = (s_Q * (1/sqrt(d))) * ((2^b - 1) / c)     (fp32, in that order)
//   x_j   = fma(u_j, -kappa, m_u * kappa)             (fp32, one rounding)
//   idx_j = min(floor(max(x_j, 0)), 2^b - 1)
//   E_j   = LUT[idx_j] for visible keys, 0 for masked ones
// Online over tiles as in the exp path: when the max rises, acc and the row
// sum are rescaled by alpha = exp((m_u_old - m_u_new) * s_Q / sqrt(d)) (fp32);
// the row sum adds the integer sum of the tile's E (IA §3.2's wide integer
// accumulation), T = E . V_hat is exact INT32, and the normalisation by the
// row sum moves to the output, O = acc / l (the FlashAttention order: the
// pages normalise P before P.V, which needs the whole row first).
void attend_row_lut(const Problem& P, int b, int h, int i, float* o, float* lse, RowTrace* tr) {
  const int d = P.d;
  const int group = P.H / P.Hkv;
  const int hk = h / group;
  const int64_t qrow = (static_cast<int64_t>(b) * P.H + h) * P.Lq + i;
  const int8_t* qv = P.q + qrow * d;
  const float sq = P.s_q[qrow];
  const int64_t kv_base = (static_cast<int64_t>(b) * P.Hkv + hk) * P.Lkv;
  const int8_t* kmat = P.k + kv_base * d;
  const int8_t* vmat = P.v + kv_base * d;
  const float* sk = P.s_k + kv_base;
  // V scale of the tile sums (1 for per-channel scales, applied at the output)
  const float sv = P.v_mode == 2 ? P.s_v[static_cast<int64_t>(b) * P.Hkv + hk] : P.v_mode == 3 ? 1.0f : P.s_v[0];
  const float* sv_ch = P.s_v + (static_cast<int64_t>(b) * P.Hkv + hk) * d;

  int64_t last = P.Lkv - 1;                      // bottom-right aligned causal mask
  if (P.causal) last = static_cast<int64_t>(i) + (P.Lkv - P.Lq);
  const float inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  const float NEG_INF = -std::numeric_limits<float>::infinity();

  const int n_idx = (1 << P.lut_bits) - 1;
  std::vector<int32_t> lut(static_cast<size_t>(n_idx) + 1);
  index_softmax_lut(P.lut_bits, P.clip, lut.data());
  const float g = sq * inv_sqrt_d;               // natural-log logit per unit of u
  const float g2 = static_cast<float>(static_cast<double>(g) / std::log(2.0));   // base-2 (trace only)
  const float k_b = static_cast<float>(static_cast<double>(n_idx) / static_cast<double>(P.clip));
  const float kappa = PLANT("lut_no_query_scale") ? inv_sqrt_d * k_b : g * k_b;

  const int Bc = P.kv_tile;
  const int split_len = P.kv_split_len > 0 ? P.kv_split_len : P.Lkv;
  const int n_splits = (P.Lkv + split_len - 1) / split_len;

  std::vector<float> acc(d), u(Bc);
  std::vector<int32_t> e(Bc), T(d);
  std::vector<float> sm(n_splits), sl(n_splits), sacc(static_cast<size_t>(n_splits) * d);

  for (int sp = 0; sp < n_splits; ++sp) {
    const int s0 = sp * split_len;
    const int s1 = std::min(P.Lkv, s0 + split_len);
    float m = NEG_INF, l = 0.0f;                 // running max (u units), row sum (table units)
    std::fill(acc.begin(), acc.end(), 0.0f);
    for (int t0 = s0; t0 < s1; t0 += Bc) {
      const int n = std::min(s1, t0 + Bc) - t0;
      float mt = NEG_INF;
      for (int jj = 0; jj < n; ++jj) {
        const int j = t0 + jj;
        if (j > last) { u[jj] = NEG_INF; continue; }
        u[jj] = static_cast<float>(dot_i8(qv, kmat + static_cast<int64_t>(j) * d, d)) * sk[j];
        mt = std::max(mt, u[jj]);
      }
      const float m_new = std::max(m, mt);
      if (m_new == NEG_INF) continue;            // nothing visible yet
      const float alpha = (m == NEG_INF) ? 0.0f : std::exp((m - m_new) * g);
      const float mu = m_new * kappa;
      int64_t esum = 0;                          // integer row sum of the tile
      for (int jj = 0; jj < n; ++jj) {
        if (u[jj] == NEG_INF) { e[jj] = 0; continue; }
        const float x = std::fma(u[jj], -kappa, mu);
        int idx;
        if (PLANT("lut_round_index")) idx = x <= 0.0f ? 0 : (x >= n_idx ? n_idx : static_cast<int>(std::nearbyint(x)));
        else idx = x <= 0.0f ? 0 : (x >= n_idx ? n_idx : static_cast<int>(std::floor(x)));
        if (PLANT("lut_no_clip")) idx = x <= 0.0f ? 0 : static_cast<int>(std::floor(x)) % (n_idx + 1);
        e[jj] = lut[idx];
        esum += e[jj];
      }
      l = alpha * l + static_cast<float>(esum);
      for (int c = 0; c < d; ++c) T[c] = 0;      // T = E . V_hat, exact
      for (int jj = 0; jj < n; ++jj) {
        if (e[jj] == 0) continue;
        const int8_t* vr = vmat + static_cast<int64_t>(t0 + jj) * d;
        for (int c = 0; c < d; ++c) T[c] += e[jj] * static_cast<int32_t>(vr[c]);
      }
      for (int c = 0; c < d; ++c) acc[c] = alpha * acc[c] + sv * static_cast<float>(T[c]);
      m = m_new;
      if (tr) {
        for (int jj = 0; jj < n; ++jj) {
          const int j = t0 + jj;
          tr->t[j] = u[jj] == NEG_INF ? NEG_INF : u[jj] * g2;
          tr->m_tile[j] = m_new * g2;
          tr->y[j] = static_cast<float>(e[jj]);
          tr->p_hat[j] = e[jj];
          tr->w[j] = 1.0f;
        }
      }
    }
    sm[sp] = m; sl[sp] = l;
    std::copy(acc.begin(), acc.end(), sacc.begin() + static_cast<size_t>(sp) * d);
    if (tr) for (int j = s0; j < s1; ++j) tr->split_m[j] = m == NEG_INF ? NEG_INF : m * g2;
  }

  // merge the splits by their maxima
  float M = NEG_INF;
  for (int sp = 0; sp < n_splits; ++sp) M = std::max(M, sm[sp]);
  float L = 0.0f;
  std::fill(acc.begin(), acc.end(), 0.0f);
  for (int sp = 0; sp < n_splits; ++sp) {
    if (sm[sp] == NEG_INF) continue;
    const float f = std::exp((sm[sp] - M) * g);
    L += f * sl[sp];
    for (int c = 0; c < d; ++c) acc[c] += f * sacc[static_cast<size_t>(sp) * d + c];
  }
  // O = acc / l: the table's factor 127 is in both, so it cancels
  for (int c = 0; c < d; ++c) o[c] = (acc[c] * (P.v_mode == 3 ? sv_ch[c] : 1.0f)) / L;
  if (lse) *lse = M * g + std::log(L / 127.0f);
}

template <class F>
void parallel_for(int64_t n, int nthreads, F f) {
  if (nthreads <= 0) nthreads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  nthreads = static_cast<int>(std::min<int64_t>(nthreads, std::max<int64_t>(1, n)));
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    for (;;) {
      const int64_t i0 = next.fetch_add(16);
      if (i0 >= n) break;
      const int64_t i1 = std::min(n, i0 + 16);
      for (int64_t i = i0; i < i1; ++i) f(i);
    }
  };
  std::vector<std::thread> th;
  for (int t = 1; t < nthreads; ++t) th.emplace_back(worker);
  worker();
  for (auto& t : th) t.join();
}

bool problem_ok(const Problem& P) {
  if (P.B < 1 || P.H < 1 || P.Hkv < 1 || P.Lq < 1 || P.Lkv < 1 || P.d < 1) return false;
  if (P.H % P.Hkv) return false;
  if (P.kv_tile < 1) return false;
  if (P.kv_split_len < 0 || (P.kv_split_len > 0 && P.kv_split_len % P.kv_tile)) return false;
  if (P.causal && P.Lq > P.Lkv) return false;
  if (P.v_mode < 0 || P.v_mode > 3) return false;
  if (P.lut_bits < 0 || P.lut_bits > 8) return false;
  // IndexSoftmax: a finite positive clip, and no per-token V (whose per-key
  // weights would re-round the table's codes)
  if (P.lut_bits > 0 && (!(P.clip > 0.0f) || !std::isfinite(P.clip) || P.v_mode == 1)) return false;
  return true;
}

}  // namespace

extern "C" {

int oracle_half_to_float(const uint16_t* h, float* f, int64_t n) {
  for (int64_t i = 0; i < n; ++i) f[i] = half_bits_to_float(h[i]);
  return 0;
}

int oracle_float_to_half(const float* f, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = float_to_half_bits(f[i]);
  return 0;
}

// x: fp32 [n_rows, n_cols] (x_is_half = 0) or binary16 bits (x_is_half = 1).
// Groups of rows_per_scale consecutive rows share one scale.
int oracle_quantize_rows(const void* x, int x_is_half, int64_t n_rows, int32_t n_cols,
                         int64_t rows_per_scale, int8_t* q, float* scales) {
  if (n_rows < 1 || n_cols < 1 || rows_per_scale < 1 || n_rows % rows_per_scale) return 1;
  const int64_t n_groups = n_rows / rows_per_scale;
  const int64_t gsize = rows_per_scale * n_cols;
  std::vector<float> buf(static_cast<size_t>(gsize));
  for (int64_t g = 0; g < n_groups; ++g) {
    const int64_t off = g * gsize;
    if (x_is_half) {
      const uint16_t* hx = static_cast<const uint16_t*>(x) + off;
      for (int64_t i = 0; i < gsize; ++i) buf[i] = half_bits_to_float(hx[i]);
    } else {
      const float* fx = static_cast<const float*>(x) + off;
      std::copy(fx, fx + gsize, buf.begin());
    }
    quantize_group(buf.data(), gsize, q + off, scales + g);
  }
  return 0;
}

// The IndexSoftmax table for b = bits (1..8) and clip c: 2^b entries.
int oracle_index_softmax_lut(int32_t bits, float c, int32_t* lut) {
  if (bits < 1 || bits > 8 || !(c > 0.0f) || !std::isfinite(c)) return 1;
  index_softmax_lut(bits, c, lut);
  return 0;
}

// Normalized Walsh-Hadamard rotation of one row of n = 2^k values (the
// "incoherent processing" of the FlashAttention-3 page: an orthogonal
// rotation of Q and K before quantization spreads outlier channels over the
// whole row, and (Q H)(K H)^T = Q K^T). Sylvester ordering, H[i][j] =
// (-1)^popcount(i & j). Computed as the fast transform in fp32: strides
// h = 1, 2, 4, ..., n / 2; for each pair (a at index e with bit h clear, b at
// e + h): a <- a + b, b <- a - b; then every value times fl32(1 / sqrt(n)).
void hadamard_row(float* x, int n) {
  for (int h = 1; h < n; h <<= 1)
    for (int e = 0; e < n; ++e) {
      if (e & h) continue;
      const float a = x[e], b = x[e + h];
      x[e] = a + b;
      x[e + h] = PLANT("fwht_sign") ? b - a : a - b;
    }
  const float r = static_cast<float>(1.0 / std::sqrt(static_cast<double>(n)));
  if (!PLANT("fwht_no_norm"))
    for (int e = 0; e < n; ++e) x[e] = x[e] * r;
}

// Per-token 4-bit codes (values in [-7, 7], one int8 each) and scales a / 7.
int oracle_quantize_rows_int4(const void* x, int x_is_half, int64_t n_rows, int32_t n_cols, int8_t* q,
                              float* scales) {
  if (n_rows < 1 || n_cols < 1) return 1;
  std::vector<float> buf(static_cast<size_t>(n_cols));
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int32_t c = 0; c < n_cols; ++c) {
      const int64_t e = r * n_cols + c;
      buf[c] = x_is_half ? half_bits_to_float(static_cast<const uint16_t*>(x)[e]) : static_cast<const float*>(x)[e];
    }
    quantize_group(buf.data(), n_cols, q + r * n_cols, scales + r, PLANT("q4_qmax_8") ? 8.0f : 7.0f);
  }
  return 0;
}

// Rows rotated by the normalized Hadamard matrix, then quantized per token
// with qmax = 127 (bits 8) or 7 (bits 4). n_cols a power of two.
int oracle_quantize_rows_hadamard(const void* x, int x_is_half, int64_t n_rows, int32_t n_cols, int32_t bits,
                                  int8_t* q, float* scales) {
  if (n_rows < 1 || n_cols < 1 || (n_cols & (n_cols - 1)) || (bits != 8 && bits != 4)) return 1;
  std::vector<float> buf(static_cast<size_t>(n_cols));
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int32_t c = 0; c < n_cols; ++c) {
      const int64_t e = r * n_cols + c;
      buf[c] = x_is_half ? half_bits_to_float(static_cast<const uint16_t*>(x)[e]) : static_cast<const float*>(x)[e];
    }
    hadamard_row(buf.data(), n_cols);
    quantize_group(buf.data(), n_cols, q + r * n_cols, scales + r, bits == 8 ? 127.0f : 7.0f);
  }
  return 0;
}

// The rotation alone (fp32 rows in, fp32 rows out), for the pins.
int oracle_hadamard_rows(const float* x, int64_t n_rows, int32_t n_cols, float* y) {
  if (n_rows < 1 || n_cols < 1 || (n_cols & (n_cols - 1))) return 1;
  for (int64_t r = 0; r < n_rows; ++r) {
    std::copy(x + r * n_cols, x + (r + 1) * n_cols, y + r * n_cols);
    hadamard_row(y + r * n_cols, n_cols);
  }
  return 0;
}

// Column groups: x is [n_groups, rows_per_group, n_cols]; each column of each
// group is one quantization group (IA §3.3 lists per-channel scales as a
// granularity the method is compatible with): scales [n_groups, n_cols].
int oracle_quantize_cols(const void* x, int x_is_half, int64_t n_groups, int64_t rows_per_group,
                         int32_t n_cols, int8_t* q, float* scales) {
  if (n_groups < 1 || rows_per_group < 1 || n_cols < 1) return 1;
  std::vector<float> col(static_cast<size_t>(rows_per_group));
  std::vector<int8_t> qc(static_cast<size_t>(rows_per_group));
  for (int64_t g = 0; g < n_groups; ++g)
    for (int32_t c = 0; c < n_cols; ++c) {
      for (int64_t r = 0; r < rows_per_group; ++r) {
        const int64_t e = ((PLANT("cols_no_group") ? 0 : g * rows_per_group) + r) * n_cols + c;
        col[r] = x_is_half ? half_bits_to_float(static_cast<const uint16_t*>(x)[e]) : static_cast<const float*>(x)[e];
      }
      quantize_group(col.data(), rows_per_group, qc.data(), scales + g * n_cols + c);
      for (int64_t r = 0; r < rows_per_group; ++r) q[(g * rows_per_group + r) * n_cols + c] = qc[r];
    }
  return 0;
}

// S_int[b,h,i,j] = sum_c Q_hat[b,h,i,c] * K_hat[b,h/(H/Hkv),j,c] for every pair
// (mask not applied; the caller compares the visible pairs).
int oracle_logits_i32(const int8_t* q, const int8_t* k, int32_t B, int32_t H, int32_t Hkv,
                      int32_t Lq, int32_t Lkv, int32_t d, int32_t* s_out, int nthreads) {
  if (B < 1 || H < 1 || Hkv < 1 || Lq < 1 || Lkv < 1 || d < 1 || H % Hkv) return 1;
  const int group = H / Hkv;
  parallel_for(static_cast<int64_t>(B) * H * Lq, nthreads, [&](int64_t r) {
    const int64_t bh = r / Lq;
    const int b = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int64_t kv_base = (static_cast<int64_t>(b) * Hkv + h / group) * Lkv;
    for (int j = 0; j < Lkv; ++j)
      s_out[r * Lkv + j] = dot_i8(q + r * d, k + (kv_base + j) * d, d);
  });
  return 0;
}

// INT8 attention forward, step by step, with the KV schedule as parameters.
// rows == NULL: every (b,h,i) row; o is [B,H,Lq,d], lse is [B,H,Lq].
// rows != NULL: n_rows flat row ids (b*H + h)*Lq + i; o is [n_rows,d], lse [n_rows].
int oracle_attn_int8(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                     const int8_t* v, const float* s_v, int32_t v_mode,
                     int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                     int32_t causal, int32_t kv_tile, int32_t kv_split_len, int32_t lut_bits,
                     float clip, const int64_t* rows, int64_t n_rows, float* o, float* lse,
                     int nthreads) {
  Problem P{q, s_q, k, s_k, v, s_v, v_mode, B, H, Hkv, Lq, Lkv, d, causal, kv_tile, kv_split_len,
            lut_bits, clip};
  if (!problem_ok(P)) return 1;
  const int64_t total = static_cast<int64_t>(B) * H * Lq;
  const int64_t n = rows ? n_rows : total;
  for (int64_t r = 0; rows && r < n; ++r)
    if (rows[r] < 0 || rows[r] >= total) return 1;
  parallel_for(n, nthreads, [&](int64_t r) {
    const int64_t id = rows ? rows[r] : r;
    const int i = static_cast<int>(id % Lq);
    const int64_t bh = id / Lq;
    (P.lut_bits ? attend_row_lut : attend_row)(P, static_cast<int>(bh / H), static_cast<int>(bh % H), i,
                                               o + r * d, lse ? lse + r : nullptr, nullptr);
  });
  return 0;
}

// Same as oracle_attn_int8 for one row, also returning the per-key trace
// (each array has Lkv entries; masked keys keep t = -inf and y = 0).
int oracle_attn_int8_trace(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                           const int8_t* v, const float* s_v, int32_t v_mode,
                           int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                           int32_t causal, int32_t kv_tile, int32_t kv_split_len,
                           int32_t lut_bits, float clip,
                           int32_t b, int32_t h, int32_t i, float* o, float* lse,
                           float* t, float* m_tile, float* y, int32_t* p_hat, float* w,
                           float* split_m) {
  Problem P{q, s_q, k, s_k, v, s_v, v_mode, B, H, Hkv, Lq, Lkv, d, causal, kv_tile, kv_split_len,
            lut_bits, clip};
  if (!problem_ok(P) || b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Lq) return 1;
  const float NEG_INF = -std::numeric_limits<float>::infinity();
  for (int j = 0; j < Lkv; ++j) {
    t[j] = NEG_INF; m_tile[j] = NEG_INF; y[j] = 0.0f; p_hat[j] = 0; w[j] = 0.0f; split_m[j] = NEG_INF;
  }
  RowTrace tr{t, m_tile, y, p_hat, w, split_m};
  (P.lut_bits ? attend_row_lut : attend_row)(P, b, h, i, o, lse, &tr);
  return 0;
}

// Exact scaled-dot-product attention in fp64 on un-quantized fp32 inputs
// (IA §2.1: A = Q K^T, P = softmax(A / sqrt(d)), O = P V), same mask and GQA
// mapping. rows/n_rows as in oracle_attn_int8.
int oracle_attn_ref_f64(const float* q, const float* k, const float* v,
                        int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                        int32_t causal, const int64_t* rows, int64_t n_rows, double* o, int nthreads) {
  if (B < 1 || H < 1 || Hkv < 1 || Lq < 1 || Lkv < 1 || d < 1 || H % Hkv) return 1;
  if (causal && Lq > Lkv) return 1;
  const int group = H / Hkv;
  const int64_t total = static_cast<int64_t>(B) * H * Lq;
  const int64_t n = rows ? n_rows : total;
  for (int64_t r = 0; rows && r < n; ++r)
    if (rows[r] < 0 || rows[r] >= total) return 1;
  parallel_for(n, nthreads, [&](int64_t r) {
    const int64_t id = rows ? rows[r] : r;
    const int i = static_cast<int>(id % Lq);
    const int64_t bh = id / Lq;
    const int b = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int64_t kv_base = (static_cast<int64_t>(b) * Hkv + h / group) * Lkv;
    const float* qv = q + id * d;
    const int64_t last = causal ? static_cast<int64_t>(i) + (Lkv - Lq) : Lkv - 1;
    std::vector<double> a(static_cast<size_t>(last + 1));
    double mx = -std::numeric_limits<double>::infinity();
    const double scale = 1.0 / std::sqrt(static_cast<double>(d));
    for (int64_t j = 0; j <= last; ++j) {
      const float* kv = k + (kv_base + j) * d;
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += static_cast<double>(qv[c]) * static_cast<double>(kv[c]);
      a[j] = dot * scale;
      mx = std::max(mx, a[j]);
    }
    double den = 0.0;
    for (int64_t j = 0; j <= last; ++j) { a[j] = std::exp(a[j] - mx); den += a[j]; }
    double* orow = o + r * d;
    for (int c = 0; c < d; ++c) orow[c] = 0.0;
    for (int64_t j = 0; j <= last; ++j) {
      const float* vv = v + (kv_base + j) * d;
      const double p = a[j] / den;
      for (int c = 0; c < d; ++c) orow[c] += p * static_cast<double>(vv[c]);
    }
  });
  return 0;
}

}  // extern "C"
