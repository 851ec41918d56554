// Internal declarations shared by the HIP sources of libattn_int8.
// Not part of the public ABI (include/attn_int8.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_int8.h"

namespace attn {

// Problem description after host-side validation.
struct FwdArgs {
  const int8_t* q; const float* s_q;
  // fused Q quantization: float Q in, optional code / scale outputs
  const void* q_float; int q_float_f16; int8_t* q_hat_out; float* s_q_out;
  const int8_t* k; const float* s_k;
  const int8_t* v; const float* s_v;
  void* o; float* lse;
  int32_t* s_dump;          // debug logits output (dump variant only)
  int B, H, Hkv, Lq, Lkv, d;
  int causal, v_per_token, o_f16;
  int v_per_head;      // s_v holds one scale per (batch, kv head)
  int v_per_channel;   // s_v holds one scale per (batch, kv head, channel)
  int k_int4;          // k holds packed 4-bit codes (d / 2 bytes per key)
  int q_rotate;        // fused Q: rotate each row by the normalized Hadamard matrix first
  float q_rot_scale;   // fl32(1 / sqrt(d)) for that rotation
  void* workspace;
  // IndexSoftmax: lut_n = 2^b - 1 (0: exp softmax), lut_k = (2^b - 1) / c in
  // fp32, lut_w = the table's bytes (entry i at byte i), zero from byte
  // lut_n + 1 on; byte kLutZero is the slot masked keys read
  int lut_n;
  float lut_k;
  uint32_t lut_w[65];
};
constexpr int kLutZero = 256;
// pair table: indices 0 .. 31 and the zero slot 32 for either key
constexpr int kLutPairRows = 33;

// The IndexSoftmax table for b = bits and clip c (entries 0 .. 2^b - 1).
void index_softmax_table(int bits, float clip, uint8_t* out);

// Prefill kernel geometry: BM query rows per workgroup, BN keys per KV tile.
constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 64;

// Decode (split-KV) geometry.
constexpr int kDecodeBN = 64;              // keys per tile (the same tile as prefill)
constexpr int kDecodeRows = 16;            // query rows per KV head (GQA group x Lq) at most
// KV chunks (one wavefront each) to aim for: about four per CU of the 256,
// all resident at once; measured faster than more, shorter chunks
constexpr int kDecodeTargetChunks = 1024;
constexpr int kDecodeMinChunk = 256;       // keys per chunk at least

// Schedule the fused forward uses for this problem (what changes the result).
void fwd_schedule(int B, int H, int Hkv, int Lq, int Lkv, int d, int causal, int* kv_tile,
                  int* kv_split_len, int* use_decode);
size_t fwd_workspace_bytes(int B, int H, int Hkv, int Lq, int Lkv, int d, int causal);

hipError_t launch_quantize(const void* x, int x_f16, int64_t n_rows, int n_cols,
                           int64_t rows_per_scale, int8_t* q, float* scales, hipStream_t st);
// per-token quantization of segments x t_new new rows into rows pos .. pos +
// t_new - 1 of each segment's l_max-row block of (cache, scales)
constexpr int kMaxAppendCols = 2048;
hipError_t launch_append(const void* x, int x_f16, int64_t segments, int t_new, int n_cols, int l_max,
                         int pos, int8_t* cache, float* scales, hipStream_t st);
// per-column quantization of n_groups groups of rows_per_group rows
constexpr int kMaxQuantCols = 2048;
hipError_t launch_quantize_cols(const void* x, int x_f16, int64_t n_groups, int64_t rows_per_group, int n_cols,
                                int8_t* q, float* scales, hipStream_t st);
// per-token 4-bit codes (int8 codes and / or packed nibbles) and scales
hipError_t launch_quantize_int4(const void* x, int x_f16, int64_t n_rows, int n_cols, int8_t* codes,
                                uint8_t* packed, float* scales, hipStream_t st);
// per-token packed 4-bit codes of new rows into their rows of a packed cache
hipError_t launch_append_int4(const void* x, int x_f16, int64_t segments, int t_new, int n_cols, int l_max, int pos,
                              uint8_t* cache4, float* scales, hipStream_t st);
// rows rotated by the normalized Hadamard matrix (n_cols = 2^k <= 2048,
// rn = fl32(1 / sqrt(n_cols))), then per-token codes at 8 or 4 bits
hipError_t launch_quantize_rotated(const void* x, int x_f16, int64_t n_rows, int n_cols, int bits, float rn,
                                   int8_t* codes, uint8_t* packed, float* scales, hipStream_t st);
// packed 4-bit codes (n_bytes, a multiple of 4) -> int8 codes (2 n_bytes)
hipError_t launch_unpack_int4(const uint8_t* packed, int64_t n_bytes, int8_t* out, hipStream_t st);
hipError_t launch_prefill(const FwdArgs& a, hipStream_t st);
hipError_t launch_debug_logits(const FwdArgs& a, hipStream_t st);
hipError_t launch_decode(const FwdArgs& a, int split_len, hipStream_t st);

}  // namespace attn
