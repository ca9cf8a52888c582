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

/* Decodes every e4m3 code (0..255) with the body kernels' weight decoder
 * (block-FP8 values as they enter the matrix cores) and writes the bf16 bit
 * patterns to out_bf16[256] (device). Blocks until done. */
kd_status kd_probe_decode_e4m3(uint16_t* out_bf16);

/* Decodes every (e4m3 scale code s, e2m1 code c) pair with the head kernel's
 * decoder, e2m1(c) * e4m3(s) as bf16, into out_bf16[s*16 + c] (device,
 * 4096 entries). Blocks until done. */
kd_status kd_probe_decode_nvfp4(uint16_t* out_bf16);

/* Runs only the first n body layers in later rounds (n in [0, layers]);
 * n < 0 restores the full depth. For bisecting parity failures. */
kd_status kd_debug_set_layers(kd_ctx* ctx, int n);

/* Device pointer to the fp32 residual stream [4*streams][hidden] as the last
 * round left it (before the final RMSNorm), and to the fused tap states
 * [streams][hidden]. */
kd_status kd_debug_buffers(kd_ctx* ctx, const float** hidden, const float** fused);

#ifdef __cplusplus
}
#endif
#endif /* KDRAFT_DEBUG_H */
