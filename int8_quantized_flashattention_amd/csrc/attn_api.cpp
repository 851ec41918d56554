// Host side of the C ABI declared in include/attn_int8.h: argument checks,
// schedule selection and kernel dispatch. Nothing here allocates, copies or
// synchronizes; every check happens before the first launch.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "attn_internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

attn_status check_shape(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                        int32_t causal) {
  if (B < 1 || H < 1 || Hkv < 1 || Lq < 1 || Lkv < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (H % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (causal && Lq > Lkv) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int64_t nq = int64_t{B} * H * Lq * d;
  const int64_t nk = int64_t{B} * Hkv * Lkv * d;
  if (nq > kMaxElems || nk > kMaxElems) return ATTN_ERR_UNSUPPORTED;
  if (int64_t{B} * H > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// IndexSoftmax parameters: 1 <= b <= 8, clip c finite in [1e-3, 1e3]
bool lut_params_ok(int32_t bits, float clip) {
  return bits >= 1 && bits <= 8 && std::isfinite(clip) && clip >= 1e-3f && clip <= 1e3f;
}

}  // namespace

namespace attn {

// Entry i samples the exponential at the left end of index bucket i, the
// distance c i / (2^b - 1), as a signed 7-bit probability:
// rne(127 exp(-(double)c * i / (2^b - 1))), in double, left to right.
void index_softmax_table(int bits, float clip, uint8_t* out) {
  const int n = (1 << bits) - 1;
  for (int i = 0; i <= n; ++i) {
    const double x = static_cast<double>(clip) * static_cast<double>(i) / static_cast<double>(n);
    out[i] = static_cast<uint8_t>(std::nearbyint(127.0 * std::exp(-x)));
  }
}

// Decode-shaped problems (at most kDecodeRows query rows per KV head: the
// GQA group's heads times Lq) take the split-KV kernel, the KV length cut in
// chunks so that about kDecodeTargetChunks chunks stream in parallel;
// everything else takes the prefill kernel with one KV pass per row block.
void fwd_schedule(int B, int H, int Hkv, int Lq, int Lkv, int d, int causal, int* kv_tile,
                  int* kv_split_len, int* use_decode) {
  (void)d; (void)causal;
  *kv_tile = kPrefillBN;
  *kv_split_len = 0;
  *use_decode = 0;
  if (int64_t{H / Hkv} * Lq > kDecodeRows) return;
  const int64_t groups = int64_t{B} * Hkv;
  const int64_t want = (kDecodeTargetChunks + groups - 1) / groups;
  const int64_t most = std::max<int64_t>(1, (Lkv + kDecodeMinChunk - 1) / kDecodeMinChunk);
  const int64_t n = std::min(std::max<int64_t>(1, want), most);
  const int64_t len = (Lkv + n - 1) / n;
  *kv_split_len = static_cast<int>((len + kDecodeBN - 1) / kDecodeBN * kDecodeBN);
  *use_decode = 1;
}

size_t fwd_workspace_bytes(int B, int H, int Hkv, int Lq, int Lkv, int d, int causal) {
  int tile, split, dec;
  fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  if (!dec || split == 0) return 0;
  const int64_t n_splits = (Lkv + split - 1) / split;
  // per (query row, split): running max, row sum, d accumulators (fp32)
  const int64_t rows = int64_t{B} * H * Lq;
  const int64_t bytes = rows * n_splits * (2 + d) * 4;
  return static_cast<size_t>((bytes + 255) / 256 * 256);
}

}  // namespace attn

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

attn_status attn_quantize_rows(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols,
                               int64_t rows_per_scale, int8_t* q, float* scales, void* stream) {
  if (!x || !q || !scales) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (n_rows < 1 || n_cols < 1 || rows_per_scale < 1 || n_rows % rows_per_scale != 0)
    return ATTN_ERR_INVALID_ARG;
  if (n_rows > INT64_MAX / n_cols) return ATTN_ERR_INVALID_ARG;
  if (n_cols % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (n_rows / rows_per_scale > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scales, 4)) return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_quantize(x, x_dt == ATTN_F16, n_rows, n_cols, rows_per_scale, q,
                                             scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_quantize_cols(const void* x, attn_dtype x_dt, int64_t n_groups, int64_t rows_per_group,
                               int32_t n_cols, int8_t* q, float* scales, void* stream) {
  if (!x || !q || !scales) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (n_groups < 1 || rows_per_group < 1 || n_cols < 1) return ATTN_ERR_INVALID_ARG;
  if (n_cols % 8 != 0 || n_cols > attn::kMaxQuantCols) return ATTN_ERR_UNSUPPORTED;
  if (n_groups > INT64_MAX / rows_per_group || n_groups * rows_per_group > INT64_MAX / n_cols)
    return ATTN_ERR_INVALID_ARG;
  if (n_groups * n_cols > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scales, 4)) return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_quantize_cols(x, x_dt == ATTN_F16, n_groups, rows_per_group, n_cols, q,
                                                  scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_quantize_rows_int4(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols, int8_t* codes,
                                    uint8_t* packed, float* scales, void* stream) {
  if (!x || !scales || (!codes && !packed)) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (n_rows < 1 || n_cols < 1) return ATTN_ERR_INVALID_ARG;
  if (n_rows > INT64_MAX / n_cols) return ATTN_ERR_INVALID_ARG;
  if (n_cols % 8 != 0 || n_cols > attn::kMaxAppendCols) return ATTN_ERR_UNSUPPORTED;
  if ((n_rows + 3) / 4 > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || (codes && !aligned(codes, 8)) || (packed && !aligned(packed, 4)) || !aligned(scales, 4))
    return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_quantize_int4(x, x_dt == ATTN_F16, n_rows, n_cols, codes, packed, scales,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_quantize_rows_hadamard(const void* x, attn_dtype x_dt, int64_t n_rows, int32_t n_cols, int32_t bits,
                                        int8_t* codes, uint8_t* packed, float* scales, void* stream) {
  if (!x || !scales) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (bits == 8 ? (!codes || packed) : bits == 4 ? (!codes && !packed) : true) return ATTN_ERR_INVALID_ARG;
  if (n_rows < 1 || n_cols < 1) return ATTN_ERR_INVALID_ARG;
  if (n_rows > INT64_MAX / n_cols) return ATTN_ERR_INVALID_ARG;
  if ((n_cols & (n_cols - 1)) || n_cols < 8 || n_cols > attn::kMaxAppendCols) return ATTN_ERR_UNSUPPORTED;
  if ((n_rows + 3) / 4 > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || (codes && !aligned(codes, 8)) || (packed && !aligned(packed, 4)) || !aligned(scales, 4))
    return ATTN_ERR_INVALID_ARG;
  const float rn = static_cast<float>(1.0 / std::sqrt(static_cast<double>(n_cols)));
  const hipError_t e = attn::launch_quantize_rotated(x, x_dt == ATTN_F16, n_rows, n_cols, bits, rn, codes, packed,
                                                     scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_kv_append_int4(const void* x, attn_dtype x_dt, int32_t B, int32_t Hkv, int32_t T, int32_t d,
                                uint8_t* cache4, float* scales, int32_t L_max, int32_t pos, void* stream) {
  if (!x || !cache4 || !scales) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || T < 1 || d < 1 || L_max < 1 || pos < 0 || T > L_max - pos)
    return ATTN_ERR_INVALID_ARG;
  if (d % 8 != 0 || d > attn::kMaxAppendCols) return ATTN_ERR_UNSUPPORTED;
  if (int64_t{B} * Hkv * L_max * d > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(cache4, 4) || !aligned(scales, 4)) return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_append_int4(x, x_dt == ATTN_F16, int64_t{B} * Hkv, T, d, L_max, pos, cache4,
                                                scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_kv_append(const void* x, attn_dtype x_dt, int32_t B, int32_t Hkv, int32_t T, int32_t d,
                           int8_t* cache, float* scales, int32_t L_max, int32_t pos, void* stream) {
  if (!x || !cache || !scales) return ATTN_ERR_INVALID_ARG;
  if (x_dt != ATTN_F32 && x_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hkv < 1 || T < 1 || d < 1 || L_max < 1 || pos < 0 || T > L_max - pos)
    return ATTN_ERR_INVALID_ARG;
  if (d % 8 != 0 || d > attn::kMaxAppendCols) return ATTN_ERR_UNSUPPORTED;
  if (int64_t{B} * Hkv * L_max * d > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(cache, 8) || !aligned(scales, 4)) return ATTN_ERR_INVALID_ARG;
  const hipError_t e = attn::launch_append(x, x_dt == ATTN_F16, int64_t{B} * Hkv, T, d, L_max, pos, cache,
                                           scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_int4qk_fwd_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                      int32_t causal) {
  if (check_shape(B, H, Hkv, Lq, Lkv, d, causal) != ATTN_OK) return 0;
  int tile, split, dec;
  attn::fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  if (dec) return attn::fwd_workspace_bytes(B, H, Hkv, Lq, Lkv, d, causal);
  // prefill shapes: K unpacked to INT8 codes
  const int64_t bytes = int64_t{B} * Hkv * Lkv * d;
  return static_cast<size_t>((bytes + 255) / 256 * 256);
}

size_t attn_int8_fwd_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                    int32_t d, int32_t causal) {
  if (check_shape(B, H, Hkv, Lq, Lkv, d, causal) != ATTN_OK) return 0;
  return attn::fwd_workspace_bytes(B, H, Hkv, Lq, Lkv, d, causal);
}

attn_status attn_int8_fwd_schedule(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                   int32_t d, int32_t causal, int32_t* kv_tile,
                                   int32_t* kv_split_len) {
  if (!kv_tile || !kv_split_len) return ATTN_ERR_INVALID_ARG;
  const attn_status s = check_shape(B, H, Hkv, Lq, Lkv, d, causal);
  if (s != ATTN_OK) return s;
  int tile, split, dec;
  attn::fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  *kv_tile = tile;
  *kv_split_len = split;
  return ATTN_OK;
}

namespace {

// Shared body of attn_int8_fwd and attn_int8_fwd_qfloat (q_float != NULL:
// float Q, quantized in the kernels).
attn_status fwd_common(const int8_t* q, const float* s_q, const void* q_float, attn_dtype q_dt,
                       int8_t* q_hat, float* s_q_out, const int8_t* k, const float* s_k,
                       const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                       attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv, int32_t Lq,
                       int32_t Lkv, int32_t d, int32_t causal, int32_t lut_bits, float clip,
                       void* workspace, size_t workspace_bytes, void* stream, int q_rotate = 0) {
  if (!k || !s_k || !v || !s_v || !o) return ATTN_ERR_INVALID_ARG;
  if (lut_bits != 0 && !lut_params_ok(lut_bits, clip)) return ATTN_ERR_INVALID_ARG;
  if (q_float) {
    if (q_dt != ATTN_F32 && q_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q_float, 16) || (q_hat && !aligned(q_hat, 16)) || (s_q_out && !aligned(s_q_out, 4)))
      return ATTN_ERR_INVALID_ARG;
  } else {
    if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(s_q, 4)) return ATTN_ERR_INVALID_ARG;
  }
  if (v_mode != ATTN_VSCALE_PER_TENSOR && v_mode != ATTN_VSCALE_PER_TOKEN && v_mode != ATTN_VSCALE_PER_HEAD &&
      v_mode != ATTN_VSCALE_PER_CHANNEL)
    return ATTN_ERR_INVALID_ARG;
  if (o_dt != ATTN_F32 && o_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  const attn_status s = check_shape(B, H, Hkv, Lq, Lkv, d, causal);
  if (s != ATTN_OK) return s;
  // IndexSoftmax kernels take INT8 Q and V scales constant along the keys
  if (lut_bits != 0 && (q_float || v_mode == ATTN_VSCALE_PER_TOKEN)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(s_k, 4) || !aligned(s_v, 4) || (lse && !aligned(lse, 4))) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::fwd_workspace_bytes(B, H, Hkv, Lq, Lkv, d, causal);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return ATTN_ERR_INVALID_ARG;

  attn::FwdArgs a{};
  a.q = q; a.s_q = s_q; a.k = k; a.s_k = s_k; a.v = v; a.s_v = s_v;
  a.q_float = q_float; a.q_float_f16 = (q_dt == ATTN_F16); a.q_hat_out = q_hat; a.s_q_out = s_q_out;
  a.o = o; a.lse = lse; a.s_dump = nullptr;
  a.B = B; a.H = H; a.Hkv = Hkv; a.Lq = Lq; a.Lkv = Lkv; a.d = d;
  a.causal = causal; a.v_per_token = (v_mode == ATTN_VSCALE_PER_TOKEN);
  a.v_per_head = (v_mode == ATTN_VSCALE_PER_HEAD); a.v_per_channel = (v_mode == ATTN_VSCALE_PER_CHANNEL);
  a.o_f16 = (o_dt == ATTN_F16);
  a.workspace = workspace;
  a.q_rotate = q_rotate;
  a.q_rot_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  if (lut_bits != 0) {
    uint8_t tab[sizeof(a.lut_w)] = {};
    attn::index_softmax_table(lut_bits, clip, tab);
    std::memcpy(a.lut_w, tab, sizeof(tab));
    a.lut_n = (1 << lut_bits) - 1;
    a.lut_k = static_cast<float>(static_cast<double>(a.lut_n) / static_cast<double>(clip));
  }
  int tile, split, dec;
  attn::fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = dec ? attn::launch_decode(a, split, st) : attn::launch_prefill(a, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

attn_status attn_int8_fwd(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                          attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv,
                          int32_t Lq, int32_t Lkv, int32_t d, int32_t causal, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  return fwd_common(q, s_q, nullptr, ATTN_F32, nullptr, nullptr, k, s_k, v, s_v, v_mode, o, o_dt, lse,
                    B, H, Hkv, Lq, Lkv, d, causal, 0, 0.0f, workspace, workspace_bytes, stream);
}

attn_status attn_int8_fwd_qfloat_hadamard(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                          attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                          int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                          int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q) return ATTN_ERR_INVALID_ARG;
  return fwd_common(nullptr, nullptr, q, q_dt, q_hat, s_q, k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq,
                    Lkv, d, causal, 0, 0.0f, workspace, workspace_bytes, stream, 1);
}

attn_status attn_int8_fwd_index_softmax(const int8_t* q, const float* s_q, const int8_t* k,
                                        const float* s_k, const int8_t* v, const float* s_v,
                                        attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse,
                                        int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                        int32_t d, int32_t causal, int32_t lut_bits, float clip,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  if (!lut_params_ok(lut_bits, clip)) return ATTN_ERR_INVALID_ARG;
  return fwd_common(q, s_q, nullptr, ATTN_F32, nullptr, nullptr, k, s_k, v, s_v, v_mode, o, o_dt, lse,
                    B, H, Hkv, Lq, Lkv, d, causal, lut_bits, clip, workspace, workspace_bytes, stream);
}

attn_status attn_int4qk_fwd(const int8_t* q, const float* s_q, const uint8_t* k4, const float* s_k, const int8_t* v,
                            const float* s_v, attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse, int32_t B,
                            int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !s_q || !k4 || !s_k || !v || !s_v || !o) return ATTN_ERR_INVALID_ARG;
  if (v_mode != ATTN_VSCALE_PER_TENSOR && v_mode != ATTN_VSCALE_PER_TOKEN && v_mode != ATTN_VSCALE_PER_HEAD &&
      v_mode != ATTN_VSCALE_PER_CHANNEL)
    return ATTN_ERR_INVALID_ARG;
  if (o_dt != ATTN_F32 && o_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  const attn_status s = check_shape(B, H, Hkv, Lq, Lkv, d, causal);
  if (s != ATTN_OK) return s;
  if (!aligned(q, 16) || !aligned(k4, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(s_q, 4) || !aligned(s_k, 4) || !aligned(s_v, 4) || (lse && !aligned(lse, 4)))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = attn_int4qk_fwd_workspace_size(B, H, Hkv, Lq, Lkv, d, causal);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ATTN_ERR_INVALID_ARG;

  attn::FwdArgs a{};
  a.q = q; a.s_q = s_q; a.k = reinterpret_cast<const int8_t*>(k4); a.s_k = s_k; a.v = v; a.s_v = s_v;
  a.o = o; a.lse = lse; a.s_dump = nullptr;
  a.B = B; a.H = H; a.Hkv = Hkv; a.Lq = Lq; a.Lkv = Lkv; a.d = d;
  a.causal = causal; a.v_per_token = (v_mode == ATTN_VSCALE_PER_TOKEN);
  a.v_per_head = (v_mode == ATTN_VSCALE_PER_HEAD); a.v_per_channel = (v_mode == ATTN_VSCALE_PER_CHANNEL);
  a.o_f16 = (o_dt == ATTN_F16);
  a.workspace = workspace;
  int tile, split, dec;
  attn::fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dec) {
    a.k_int4 = 1;                      // the decode kernel reads the packed codes itself
    e = attn::launch_decode(a, split, st);
  } else {
    // prefill shapes: unpack K into the workspace, then the INT8 kernel
    e = attn::launch_unpack_int4(k4, int64_t{B} * Hkv * Lkv * d / 2, static_cast<int8_t*>(workspace), st);
    if (e == hipSuccess) {
      a.k = static_cast<const int8_t*>(workspace);
      a.workspace = nullptr;
      e = attn::launch_prefill(a, st);
    }
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_index_softmax_table(int32_t lut_bits, float clip, uint8_t* table) {
  if (!table || !lut_params_ok(lut_bits, clip)) return ATTN_ERR_INVALID_ARG;
  attn::index_softmax_table(lut_bits, clip, table);
  return ATTN_OK;
}

attn_status attn_int8_fwd_qfloat(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                 const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                 attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                 int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                 int32_t causal, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!q) return ATTN_ERR_INVALID_ARG;
  return fwd_common(nullptr, nullptr, q, q_dt, q_hat, s_q, k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H,
                    Hkv, Lq, Lkv, d, causal, 0, 0.0f, workspace, workspace_bytes, stream);
}

attn_status attn_int8_debug_logits(const int8_t* q, const int8_t* k, int32_t B, int32_t H,
                                   int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                                   int32_t* s_out, void* stream) {
  if (!q || !k || !s_out) return ATTN_ERR_INVALID_ARG;
  const attn_status s = check_shape(B, H, Hkv, Lq, Lkv, d, causal);
  if (s != ATTN_OK) return s;
  if (int64_t{B} * H * Lq * Lkv > kMaxElems) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(s_out, 16)) return ATTN_ERR_INVALID_ARG;
  attn::FwdArgs a{};
  a.q = q; a.k = k; a.s_dump = s_out;
  a.B = B; a.H = H; a.Hkv = Hkv; a.Lq = Lq; a.Lkv = Lkv; a.d = d; a.causal = causal;
  const hipError_t e = attn::launch_debug_logits(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
