/*
 * attn_probes.h — C ABI of libattn_probes, two measurement kernels that the
 * benchmark uses as second denominators next to MI355X's published peaks
 * (dense INT8 matrix rate, HBM bandwidth). They are not part of the attention
 * path. The rate of a fused kernel is judged against the peak of the unit
 * that bounds it (the "utilization" figures of "FlashAttention-3: Fast and
 * Accurate Attention with Asynchrony and Low-precision", abstract); these
 * probes measure what that unit delivers on the machine at hand.
 *
 * Both take device pointers owned by the caller, enqueue one launch on
 * `stream` (a hipStream_t as void*, NULL = default) and return at once: 0 on
 * success, 1 for an invalid argument (nothing launched), 3 when the HIP
 * runtime reports a launch error. Neither allocates or synchronizes.
 */
#ifndef ATTN_PROBES_H
#define ATTN_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* attn_probe_mfma_i8 — n_blocks workgroups of 4 wavefronts; every wavefront
 * issues iters x 4 independent v_mfma_i32_32x32x32_i8 (65536 INT8 ops each)
 * on register operands. out: int32 [n_blocks * 256 * 16], device, receives
 * the accumulators. INT8 ops per launch = n_blocks * 4 * iters * 4 * 65536. */
int attn_probe_mfma_i8(int32_t n_blocks, int32_t iters, int32_t* out, void* stream);

/* attn_probe_hbm_read — reads n_bytes (a multiple of 16, src 16-byte aligned)
 * once with 16-byte loads (non-temporal when `nontemporal` is nonzero):
 * n_blocks workgroups of 256 lanes, each streaming one contiguous slice with
 * four loads per lane in flight. out: uint32 [n_blocks * 256], device,
 * receives one XOR fold per lane. Bytes per launch = n_bytes. */
int attn_probe_hbm_read(const void* src, int64_t n_bytes, int32_t n_blocks, int32_t nontemporal, uint32_t* out,
                        void* stream);

/* attn_probe_lds_patterns — one LDS access pattern of the prefill kernel's
 * tile (d = 128, 64 keys) in a loop of `iters` rounds on a resident K/V
 * stage, n_blocks workgroups of 256 lanes, so that LDS counters (bank
 * conflicts per instruction) can be read for that pattern alone. mode: 0 the
 * K operand reads (8 ds_read_b128 per round), 1 the transposing V operand
 * reads (16 ds_read_b64_tr_b8), 2 the per-key scale reads (8 ds_read_b128,
 * each half-wave on one address), 3 the LDS-destination buffer loads of one
 * stage request from src (8 KB read, 16-byte aligned, device; four 1 KB loads
 * per wavefront) with a wait and two barriers per round. out: uint32
 * [n_blocks * 256], device. */
int attn_probe_lds_patterns(int32_t mode, const void* src, int32_t n_blocks, int32_t iters, uint32_t* out,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBES_H */
