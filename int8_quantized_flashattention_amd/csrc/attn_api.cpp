// Host side of the C ABI declared in include/attn_int8.h: argument checks,
// schedule selection and kernel dispatch. Nothing here allocates, copies or
// synchronizes; every check happens before the first launch.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

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

namespace {

// Workspace of the forward: the split-KV partials for decode shapes; for
// packed 4-bit K on other shapes, room for K widened to INT8 codes.
size_t workspace_need(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                      bool k_int4) {
  int tile, split, dec;
  attn::fwd_schedule(B, H, Hkv, Lq, Lkv, d, causal, &tile, &split, &dec);
  if (dec || !k_int4) return attn::fwd_workspace_bytes(B, H, Hkv, Lq, Lkv, d, causal);
  const int64_t bytes = int64_t{B} * Hkv * Lkv * d;
  return static_cast<size_t>((bytes + 255) / 256 * 256);
}

// One forward request, as the entry points fill it in.
struct FwdRequest {
  const int8_t* q = nullptr;           // INT8 Q codes and scales ...
  const float* s_q = nullptr;
  const void* q_float = nullptr;       // ... or fp16 / fp32 Q, quantized in the kernels
  attn_dtype q_dt = ATTN_F32;
  int8_t* q_hat = nullptr;             // optional outputs of the in-kernel quantization
  float* s_q_out = nullptr;
  int q_rotate = 0;                    // rotate the fp16 / fp32 Q rows first (Hadamard)
  const int8_t* k = nullptr;           // INT8 codes, or packed 4-bit codes when k_int4
  const float* s_k = nullptr;
  int k_int4 = 0;
  const int8_t* v = nullptr;
  const float* s_v = nullptr;
  attn_vscale v_mode = ATTN_VSCALE_PER_TENSOR;
  void* o = nullptr;
  attn_dtype o_dt = ATTN_F32;
  float* lse = nullptr;
  int32_t B = 0, H = 0, Hkv = 0, Lq = 0, Lkv = 0, d = 0, causal = 0;
  int32_t lut_bits = 0;                // IndexSoftmax table bits (0: exp softmax)
  float clip = 0.0f;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  void* stream = nullptr;
};

// Checks every argument (the workspace only when check_ws).
attn_status check_fwd(const FwdRequest& r, bool check_ws) {
  if (!r.k || !r.s_k || !r.v || !r.s_v || !r.o) return ATTN_ERR_INVALID_ARG;
  if (r.lut_bits != 0 && !lut_params_ok(r.lut_bits, r.clip)) return ATTN_ERR_INVALID_ARG;
  if (r.q_float) {
    if (r.q_dt != ATTN_F32 && r.q_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
    if (!aligned(r.q_float, 16) || (r.q_hat && !aligned(r.q_hat, 16)) || (r.s_q_out && !aligned(r.s_q_out, 4)))
      return ATTN_ERR_INVALID_ARG;
  } else {
    if (!r.q || !r.s_q) return ATTN_ERR_INVALID_ARG;
    if (!aligned(r.q, 16) || !aligned(r.s_q, 4)) return ATTN_ERR_INVALID_ARG;
  }
  if (r.v_mode != ATTN_VSCALE_PER_TENSOR && r.v_mode != ATTN_VSCALE_PER_TOKEN &&
      r.v_mode != ATTN_VSCALE_PER_HEAD && r.v_mode != ATTN_VSCALE_PER_CHANNEL)
    return ATTN_ERR_INVALID_ARG;
  if (r.o_dt != ATTN_F32 && r.o_dt != ATTN_F16) return ATTN_ERR_INVALID_ARG;
  const attn_status s = check_shape(r.B, r.H, r.Hkv, r.Lq, r.Lkv, r.d, r.causal);
  if (s != ATTN_OK) return s;
  // IndexSoftmax kernels take INT8 Q and V scales constant along the keys
  if (r.lut_bits != 0 && (r.q_float || r.v_mode == ATTN_VSCALE_PER_TOKEN)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(r.k, 16) || !aligned(r.v, 16) || !aligned(r.o, 16)) return ATTN_ERR_INVALID_ARG;
  if (!aligned(r.s_k, 4) || !aligned(r.s_v, 4) || (r.lse && !aligned(r.lse, 4))) return ATTN_ERR_INVALID_ARG;
  const size_t need = workspace_need(r.B, r.H, r.Hkv, r.Lq, r.Lkv, r.d, r.causal, r.k_int4);
  if (check_ws && need > 0 && (!r.workspace || r.workspace_bytes < need || !aligned(r.workspace, 256)))
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Checks every argument, then launches. Nothing is launched on any error.
attn_status run_fwd(const FwdRequest& r) {
  const attn_status chk = check_fwd(r, true);
  if (chk != ATTN_OK) return chk;

  attn::FwdArgs a{};
  a.q = r.q; a.s_q = r.s_q; a.k = r.k; a.s_k = r.s_k; a.v = r.v; a.s_v = r.s_v;
  a.q_float = r.q_float; a.q_float_f16 = (r.q_dt == ATTN_F16); a.q_hat_out = r.q_hat; a.s_q_out = r.s_q_out;
  a.o = r.o; a.lse = r.lse; a.s_dump = nullptr;
  a.B = r.B; a.H = r.H; a.Hkv = r.Hkv; a.Lq = r.Lq; a.Lkv = r.Lkv; a.d = r.d;
  a.causal = r.causal; a.v_per_token = (r.v_mode == ATTN_VSCALE_PER_TOKEN);
  a.v_per_head = (r.v_mode == ATTN_VSCALE_PER_HEAD); a.v_per_channel = (r.v_mode == ATTN_VSCALE_PER_CHANNEL);
  a.o_f16 = (r.o_dt == ATTN_F16);
  a.workspace = r.workspace;
  a.q_rotate = r.q_rotate;
  a.q_rot_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(r.d)));
  if (r.lut_bits != 0) {
    uint8_t tab[sizeof(a.lut_w)] = {};
    attn::index_softmax_table(r.lut_bits, r.clip, tab);
    std::memcpy(a.lut_w, tab, sizeof(tab));
    a.lut_n = (1 << r.lut_bits) - 1;
    a.lut_k = static_cast<float>(static_cast<double>(a.lut_n) / static_cast<double>(r.clip));
  }
  int tile, split, dec;
  attn::fwd_schedule(r.B, r.H, r.Hkv, r.Lq, r.Lkv, r.d, r.causal, &tile, &split, &dec);
  const hipStream_t st = static_cast<hipStream_t>(r.stream);
  hipError_t e;
  if (dec) {
    a.k_int4 = r.k_int4;               // the decode kernel reads packed codes itself
    e = attn::launch_decode(a, split, st);
  } else if (r.k_int4) {
    // prefill shapes with packed K: widen K into the workspace, then the INT8 kernel
    e = attn::launch_unpack_int4(reinterpret_cast<const uint8_t*>(r.k), int64_t{r.B} * r.Hkv * r.Lkv * r.d / 2,
                                 static_cast<int8_t*>(r.workspace), st);
    if (e == hipSuccess) {
      a.k = static_cast<const int8_t*>(r.workspace);
      a.workspace = nullptr;
      e = attn::launch_prefill(a, st);
    }
  } else {
    e = attn::launch_prefill(a, st);
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Scratch of attn_int8_fwd_noalloc: the split-KV partials live in a static
// device array (one copy per GPU, held until the process ends) instead of a
// caller-provided workspace. In host code `scratch` names a host-side stand-in,
// not a device address: the device address of each GPU's copy is looked up
// once per device, with that device current, and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;   // 32 MiB
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This thread's current device's copy of scratch (looked up on first use).
attn_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_HIP;
  if (dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// the arguments every forward shares
FwdRequest request(const int8_t* k, const float* s_k, const int8_t* v, const float* s_v, attn_vscale v_mode,
                   void* o, attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                   int32_t d, int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  FwdRequest r;
  r.k = k; r.s_k = s_k; r.v = v; r.s_v = s_v; r.v_mode = v_mode; r.o = o; r.o_dt = o_dt; r.lse = lse;
  r.B = B; r.H = H; r.Hkv = Hkv; r.Lq = Lq; r.Lkv = Lkv; r.d = d; r.causal = causal;
  r.workspace = workspace; r.workspace_bytes = workspace_bytes; r.stream = stream;
  return r;
}

}  // namespace

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
  return workspace_need(B, H, Hkv, Lq, Lkv, d, causal, true);
}

size_t attn_int8_fwd_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                    int32_t d, int32_t causal) {
  if (check_shape(B, H, Hkv, Lq, Lkv, d, causal) != ATTN_OK) return 0;
  return workspace_need(B, H, Hkv, Lq, Lkv, d, causal, false);
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

attn_status attn_int8_fwd(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                          attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv,
                          int32_t Lq, int32_t Lkv, int32_t d, int32_t causal, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq, Lkv, d, causal, workspace,
                         workspace_bytes, stream);
  r.q = q; r.s_q = s_q;
  return run_fwd(r);
}

size_t attn_int8_fwd_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

attn_status attn_int8_fwd_noalloc(const int8_t* q, const float* s_q, const int8_t* k, const float* s_k,
                                  const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                  attn_dtype o_dt, float* lse, int32_t B, int32_t H, int32_t Hkv,
                                  int32_t Lq, int32_t Lkv, int32_t d, int32_t causal, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq, Lkv, d, causal, nullptr, 0, stream);
  r.q = q; r.s_q = s_q;
  const attn_status chk = check_fwd(r, false);       // every argument but the workspace
  if (chk != ATTN_OK) return chk;
  const size_t need = attn::fwd_workspace_bytes(B, H, Hkv, Lq, Lkv, d, causal);
  if (need > kNoAllocScratchBytes) return ATTN_ERR_UNSUPPORTED;
  if (need > 0) {
    // every partial the merge reads is written by the split-KV kernel first,
    // so the scratch needs no clearing between calls
    void* ws = nullptr;
    const attn_status e = current_scratch(&ws);
    if (e != ATTN_OK) return e;
    r.workspace = ws;
    r.workspace_bytes = kNoAllocScratchBytes;
  }
  return run_fwd(r);
}

attn_status attn_int8_fwd_qfloat(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                 const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                 attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                 int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                 int32_t causal, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!q) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq, Lkv, d, causal, workspace,
                         workspace_bytes, stream);
  r.q_float = q; r.q_dt = q_dt; r.q_hat = q_hat; r.s_q_out = s_q;
  return run_fwd(r);
}

attn_status attn_int8_fwd_qfloat_hadamard(const void* q, attn_dtype q_dt, const int8_t* k, const float* s_k,
                                          const int8_t* v, const float* s_v, attn_vscale v_mode, void* o,
                                          attn_dtype o_dt, float* lse, int8_t* q_hat, float* s_q, int32_t B,
                                          int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d,
                                          int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq, Lkv, d, causal, workspace,
                         workspace_bytes, stream);
  r.q_float = q; r.q_dt = q_dt; r.q_hat = q_hat; r.s_q_out = s_q; r.q_rotate = 1;
  return run_fwd(r);
}

attn_status attn_int8_fwd_index_softmax(const int8_t* q, const float* s_q, const int8_t* k,
                                        const float* s_k, const int8_t* v, const float* s_v,
                                        attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse,
                                        int32_t B, int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv,
                                        int32_t d, int32_t causal, int32_t lut_bits, float clip,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  if (!lut_params_ok(lut_bits, clip)) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(k, s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq, Lkv, d, causal, workspace,
                         workspace_bytes, stream);
  r.q = q; r.s_q = s_q; r.lut_bits = lut_bits; r.clip = clip;
  return run_fwd(r);
}

attn_status attn_int4qk_fwd(const int8_t* q, const float* s_q, const uint8_t* k4, const float* s_k, const int8_t* v,
                            const float* s_v, attn_vscale v_mode, void* o, attn_dtype o_dt, float* lse, int32_t B,
                            int32_t H, int32_t Hkv, int32_t Lq, int32_t Lkv, int32_t d, int32_t causal,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !s_q) return ATTN_ERR_INVALID_ARG;
  FwdRequest r = request(reinterpret_cast<const int8_t*>(k4), s_k, v, s_v, v_mode, o, o_dt, lse, B, H, Hkv, Lq,
                         Lkv, d, causal, workspace, workspace_bytes, stream);
  r.q = q; r.s_q = s_q; r.k_int4 = 1;
  return run_fwd(r);
}

attn_status attn_index_softmax_table(int32_t lut_bits, float clip, uint8_t* table) {
  if (!table || !lut_params_ok(lut_bits, clip)) return ATTN_ERR_INVALID_ARG;
  attn::index_softmax_table(lut_bits, clip, table);
  return ATTN_OK;
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
