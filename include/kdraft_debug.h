/*
 * Test and debugging entry points of libkdraft. They exercise the production
 * device code paths but are not part of a round.
 */
#ifndef KDRAFT_DEBUG_H
#define KDRAFT_DEBUG_H

#include "kdraft.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Decodes every e4m3 code (0..255) with the bf16 weight decoder (block-FP8
 * values as they meet bf16 activations on the matrix cores: the small-batch
 * path's tapped-state and embedding projections) and writes the bf16 bit
 * patterns to out_bf16[256] (device). Blocks until done. */
kd_status kd_probe_decode_e4m3(uint16_t* out_bf16);

/* Decodes every e4m3 code (0..255) with the f16 weight decoder (block-FP8
 * values as they meet f16 activations on the matrix cores: every other
 * projection) and writes the f16 bit patterns to out_f16[256] (device).
 * Blocks until done. */
kd_status kd_probe_decode_e4m3_f16(uint16_t* out_f16);

/* Decodes every (e4m3 scale code s, e2m1 code c) pair with the head kernels'
 * decoder, e2m1(c) * e4m3(s) as f16, into out_f16[s*16 + c] (device,
 * 4096 entries). Blocks until done. */
kd_status kd_probe_decode_nvfp4(uint16_t* out_f16);

/* Runs only the first n body layers in later rounds (n in [0, layers]);
 * n < 0 restores the full depth. For bisecting parity failures. */
kd_status kd_debug_set_layers(kd_ctx* ctx, int n);

/* Device pointer to the fp32 residual stream [4*streams][hidden] as the last
 * round left it (before the final RMSNorm), and to the fused tap states
 * [streams][hidden]. */
kd_status kd_debug_buffers(kd_ctx* ctx, const float** hidden, const float** fused);

/* Chooses how later rounds run: 0 automatic (the small-batch phases as
 * separate launches for up to 4 streams, the general multi-kernel path above
 * 4 streams), 1 the general path, 2 the small-batch phases as separate
 * launches, 3 the small-batch persistent kernel. Paths 2 and 3 apply only to
 * rounds of at most 4 streams; larger rounds use path 1. KD_ERR_ARG for a
 * path outside 0..3; KD_ERR_UNSUPPORTED if 3 is asked for without cooperative
 * launch. */
kd_status kd_debug_set_path(kd_ctx* ctx, int path);

/* General path with more than 32 block rows: on = 1 (the default) runs the
 * q|k|v and gate|up projections in one split each with RoPE and SwiGLU
 * applied in the projection kernel; on = 0 runs split projections followed by
 * the separate reduction and epilogue kernels. For comparing the two. */
kd_status kd_debug_set_fused(kd_ctx* ctx, int on);

/* The path the last round ran on (1, 2 or 3; 0 before any round). */
int kd_debug_last_path(const kd_ctx* ctx);

/* Stage tracing of the small-batch paths: later rounds write 100 MHz
 * wall-clock stamps into buf (device, [phases][workgroups][8] uint64, caller
 * owned; slots: 0 phase entry or barrier arrival, 1 barrier passed, 2 unit
 * inputs issued, 3 compute done, 4 epilogue done, 7 phase exit). buf = NULL
 * turns tracing off. *workgroups (if not NULL) receives the workgroup count. */
kd_status kd_debug_set_trace(kd_ctx* ctx, unsigned long long* buf, int phases, int* workgroups);

#ifdef __cplusplus
}
#endif
#endif /* KDRAFT_DEBUG_H */
