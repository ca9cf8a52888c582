/*
 * libkdraft: one batched round of the Kolibri-1 block drafter on one MI355X
 * (gfx950), as a C ABI.
 *
 * What a round computes is fixed by the model card "Kolibri-1 block drafter",
 * section "Architecture":
 *   Input     - the target's normed outputs of layers 44, 47, 49 are
 *               concatenated and fused 3x2560 -> 2560; context rows are
 *               [fused state ; embedding of the next token] -> 5120 -> 2560.
 *   Position 1 - block row 0 is the anchor's own row in that context-row form.
 *   Positions 2-4 - rows 1..3 read the learned mask row plus the anchor's
 *               fused state, plus the rank-256 predecessor term
 *               U silu(A h + B embed(token before)).
 *   Spine     - before layers 2-4, row j reads row j-1 through
 *               RMSNorm -> A -> silu -> U (rank 256); row 0 is untouched.
 *   Body      - 4 layers: hidden 2560, 20 heads x 128, SwiGLU 6144, RoPE
 *               theta 10,000; each layer cross-attends to the last 2,048
 *               context rows and is causal inside the block.
 *   Output    - RMSNorm, then the LM head restricted to the draft vocabulary.
 * and the Serving paragraph: every stream is drafted in one batched pass; the
 * body is block-FP8 (e4m3, one fp32 scale per row and 64 inputs) and the
 * 60k-row head slice is NVFP4 (e2m1, one e4m3 scale per 16 inputs, one fp32
 * tensor scale). The draft for a row is the argmax of its restricted logits.
 *
 * Conventions (all entry points):
 *  - Device pointers are HIP device addresses the caller owns (for example
 *    torch tensors). Host pointers are only read during the call.
 *  - Calls enqueue work on the context's HIP stream and return without
 *    waiting for the device (argument blocks are staged through pinned
 *    buffers; graphs are cached per set of caller pointers, so a loop that
 *    rotates among a few buffer sets captures each once). Argument and state
 *    errors are reported synchronously and enqueue nothing. A fault on the
 *    device surfaces as KD_ERR_HIP on a later call, and so does a bounded
 *    device wait that timed out (the rounds that saw it wrote -2 ids).
 *  - A context is not thread-safe. kd_round / kd_ingest never allocate.
 *  - Token ids on the device are checked before they index the embedding
 *    table: an id outside [0, full_vocab) reads a zero row, and every block
 *    row whose anchor or earlier predecessor ids (rows 1..j for row j) are out
 *    of range gets out_ids -1. Lengths must be >= 0.
 */
#ifndef KDRAFT_H
#define KDRAFT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kd_ctx kd_ctx;

typedef enum {
  KD_OK = 0,
  KD_ERR_ARG = -1,         /* a NULL or out-of-range argument */
  KD_ERR_STATE = -2,       /* e.g. kd_round before kd_load_weights */
  KD_ERR_OOM = -3,         /* device allocation failed (create / load only) */
  KD_ERR_HIP = -4,         /* a HIP runtime call failed */
  KD_ERR_UNSUPPORTED = -5, /* a shape or format this build does not implement */
  KD_ERR_RANGE = -6        /* an earlier round (or ingest) stored an activation beyond the
                              f16 range (+-65504) or not finite; it was stored saturated
                              and that round's drafts are unreliable. Returned once by the
                              next kd_round / kd_round_depth / kd_ingest, which then does
                              nothing else. The flag is kept per device: with several
                              contexts on one device, the next round of any of them may
                              report it. */
} kd_status;

enum { KD_QUANT_FP8_BLOCK64 = 1, KD_QUANT_NVFP4 = 2, KD_QUANT_BF16 = 3 };
enum { KD_MAX_INGEST = 8 };  /* rows per stream per kd_ingest call */
enum { KD_MAX_DEPTH = 8 };   /* rounds per kd_round_depth call */
enum { KD_MAX_COPY = 48 };   /* tokens per copy-draft proposal */
enum { KD_GUARD_MAX_WINDOW = 64 };  /* proposals the pause guard can track */
/* Context K/V storage formats (kd_kv.format). */
enum { KD_KV_BF16 = 0, KD_KV_INT4_ROT = 1 };

/* Model shape and limits. The kernels are built for the model card's shape;
 * kd_create returns KD_ERR_UNSUPPORTED for any other hidden, heads, head_dim,
 * ffn, layers, block, rank or taps. draft_vocab, full_vocab and window are
 * free (window >= 1). */
typedef struct {
  int hidden;        /* 2560 */
  int heads;         /* 20 */
  int head_dim;      /* 128 */
  int ffn;           /* 6144 */
  int layers;        /* 4 */
  int block;         /* 4 rows drafted per stream per round */
  int rank;          /* 256: predecessor and spine adapters */
  int taps;          /* 3 tapped target layers (44, 47, 49) */
  int window;        /* 2048: context rows attended, the last min(len, window) */
  int draft_vocab;   /* 60614 */
  int full_vocab;    /* 131072: rows of the embedding/head table */
  int max_streams;   /* largest `streams` any call will pass */
  float rope_theta;  /* 10000 */
  float rms_eps;     /* 1e-6 */
  int body_quant;    /* KD_QUANT_FP8_BLOCK64 (default), or KD_QUANT_NVFP4 /
                        KD_QUANT_BF16 (every body format runs on both the
                        small-batch and the general path) */
  int head_quant;    /* KD_QUANT_NVFP4, or KD_QUANT_BF16 / KD_QUANT_FP8_BLOCK64
                        (the card's Use section offers bf16, FP8 and NVFP4
                        head slices; every head runs on both the small-batch
                        and the general path) */
} kd_config;

/* Fills *cfg with the model card's shape, max_streams = 256. */
void kd_default_config(kd_config* cfg);

/* A weight matrix W[rows][cols] on the host, row-major, in the format
 * kd_config.body_quant names (the block-FP8 head slice, head_fp8, is always
 * block-FP8); fields a format does not use are ignored (model card, section
 * Use: FP8, NVFP4 and bf16 bodies):
 *   KD_QUANT_FP8_BLOCK64: q = e4m3 codes [rows][cols]; s = fp32 scales
 *     [rows][cols/64]; W = e4m3(q) * s[r][c/64].
 *   KD_QUANT_NVFP4: q = e2m1 codes [rows][cols/2], column 2m in the low
 *     nibble of byte m; s4 = e4m3 scale codes [rows][cols/16]; g = fp32
 *     tensor scale; W = e2m1(q) * e4m3(s4[r][c/16]) * g.
 *   KD_QUANT_BF16: q = bf16 values [rows][cols], 2 bytes each (little-endian).
 * kd_load_weights rejects NaN e4m3 codes, non-finite scales and non-finite
 * bf16 values. */
typedef struct {
  const uint8_t* q;
  const float* s;
  const uint8_t* s4;
  float g;
} kd_matrix;

typedef struct {
  kd_matrix wq, wk, wv, wo;  /* [hidden][hidden] */
  kd_matrix w_gate, w_up;    /* [ffn][hidden] */
  kd_matrix w_down;          /* [hidden][ffn] */
  const float* attn_norm;        /* [hidden] RMSNorm gains */
  const float* ffn_norm;         /* [hidden] */
  /* Spine applied before this layer (layers 1..3); ignored for layer 0. */
  const float* spine_norm;       /* [hidden] */
  kd_matrix spine_a;         /* [rank][hidden] */
  kd_matrix spine_u;         /* [hidden][rank] */
} kd_layer_weights;

/* Host copies of the weights (copied and repacked by kd_load_weights), except
 * the embedding table, which is borrowed: it is the target's frozen bf16
 * table, a device pointer that must outlive the context. */
typedef struct {
  kd_matrix fuse;            /* [hidden][taps*hidden] */
  kd_matrix fc;              /* [hidden][2*hidden]: input [fused ; embedding] */
  kd_matrix pred_a;          /* [rank][hidden] applied to the fused state */
  kd_matrix pred_b;          /* [rank][hidden] applied to embed(predecessor) */
  kd_matrix pred_u;          /* [hidden][rank] */
  const float* mask_row;         /* [hidden] */
  kd_layer_weights layer[4];
  const float* final_norm;       /* [hidden] */
  const uint8_t* head_q4;        /* [draft_vocab][hidden/2] e2m1 codes, even column in the low nibble */
  const uint8_t* head_s4;        /* [draft_vocab][hidden/16] e4m3 block scales */
  float head_g;                  /* fp32 tensor scale */
  const int32_t* draft_vocab;    /* [draft_vocab] target-vocabulary id of each head row */
  const void* embed_table;       /* DEVICE, bf16 [full_vocab][hidden], borrowed */
  /* Sign vectors s of the rotated 4-bit cache, [layers][head_dim] int8, each
   * +1 or -1 (see kd_kv), or NULL when no cache in that format is used. */
  const int8_t* kv_rot_signs;
  /* head_quant = KD_QUANT_BF16: the head slice as bf16 [draft_vocab][hidden]
   * (host; finite values), used instead of head_q4 / head_s4 / head_g. */
  const void* head_bf16;
  /* head_quant = KD_QUANT_FP8_BLOCK64: the head slice in block-FP8,
   * [draft_vocab][hidden], as the body matrices. */
  kd_matrix head_fp8;
} kd_weights;

/* The context K/V cache (device), one K and one V tensor per layer. A
 * context of len tokens keeps position p at slot p % capacity; a round attends
 * positions [len - n, len) with n = min(len, window), so capacity >= window.
 * K is stored after RoPE.
 *
 * format KD_KV_BF16: element (stream b, head h, slot s, dim d) of layer l is
 *   the bf16 at k[l] + b*stride_stream + h*stride_head + s*stride_slot + d
 *   (strides in elements, multiples of 8; head_dim contiguous). k_so/v_so
 *   are ignored.
 * format KD_KV_INT4_ROT (the article "Serving Kolibri-1 with a 4-bit KV
 *   cache", section What we do): per layer a fixed R = H diag(s)/sqrt(128),
 *   H the 128x128 Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i&j)) and
 *   s the layer's kv_rot_signs; the cache holds R k for keys and v unrotated,
 *   each (stream, head, slot) row as 128 4-bit codes plus an fp16 scale and
 *   offset: value = scale * code + offset. Row index
 *   i = b*stride_stream + h*stride_head + s*stride_slot (strides count rows);
 *   its codes are the 64 bytes at k[l] + 64*i (dim 2m in the low nibble of
 *   byte m, dim 2m+1 in the high nibble; 16-byte aligned tensors) and its
 *   (scale, offset) pair the two fp16 at k_so[l] + 4*i (4-byte aligned); the
 *   same for v / v_so. kd_ingest writes codes with scale = fp16((max-min)/15),
 *   offset = fp16(min) over the row, code = clamp(round_half_even((x -
 *   offset)/scale), 0, 15) (0 when the scale is 0). Rounds on this format
 *   run the general (any batch) path and need kv_rot_signs loaded.
 */
typedef struct {
  void* k[4];
  void* v[4];
  int64_t stride_stream, stride_head, stride_slot;
  int capacity;
  int format;        /* KD_KV_BF16 or KD_KV_INT4_ROT */
  void* k_so[4];     /* KD_KV_INT4_ROT: (scale, offset) fp16 pairs of K, per row */
  void* v_so[4];     /* KD_KV_INT4_ROT: the same for V */
} kd_kv;

/* Creates a context whose work goes to hip_stream (a hipStream_t; NULL is the
 * null stream). Allocates the workspace for cfg->max_streams. */
kd_status kd_create(const kd_config* cfg, void* hip_stream, kd_ctx** out);

/* Copies, validates and repacks the weights into device memory (synchronous).
 * May be called again to replace them. The roles follow the model card
 * "Kolibri-1 block drafter", section Architecture (Input, Positions 2-4,
 * Predecessor head, Spine, Body, Output) and its Serving paragraph for the
 * formats: block-FP8 body matrices and the NVFP4 head slice are quantised
 * outside the library (the card's section Files: FP8 and NVFP4 are made at
 * load time), so the library decodes exactly the codes it is given.
 * Errors: KD_ERR_ARG for NULL or invalid data (NaN codes, non-finite scales,
 * vocabulary ids out of range), KD_ERR_OOM, KD_ERR_HIP. */
kd_status kd_load_weights(kd_ctx* ctx, const kd_weights* w);

/* One round for `streams` streams (1 <= streams <= max_streams): the model
 * card "Kolibri-1 block drafter", section Architecture (Input through
 * Output), with every stream in one batched pass (its Serving paragraph).
 *   tapped_states [streams][taps][hidden] bf16 (order: layers 44, 47, 49)
 *   anchor_ids    [streams]     int32, target-vocabulary ids (row 0's token)
 *   pred_ids      [streams][3]  int32, pred_ids[b][j-1] is the token before
 *                               the one block row j drafts (j = 1..3)
 *   ctx_kv        the K/V cache (struct on the host, tensors on the device)
 *   ctx_lens      [streams] int32, tokens seen; block row j is at position len + j
 *   out_ids       [streams][4] int32: target-vocabulary id of each row's
 *                 argmax (lowest draft index on ties); -1 if no logit is
 *                 finite or an id the row reads is out of range; -2 for
 *                 every row of a round whose bounded device wait timed out
 *                 (the next call then returns KD_ERR_HIP)
 *   out_logits    [streams][4][draft_vocab] fp32 in draft-vocabulary order, or NULL
 * All arrays are device pointers except ctx_kv itself. */
kd_status kd_round(kd_ctx* ctx, int streams, const void* tapped_states,
                   const int32_t* anchor_ids, const int32_t* pred_ids,
                   const kd_kv* ctx_kv, const int32_t* ctx_lens,
                   int32_t* out_ids, float* out_logits);

/* `depth` rounds in a row before the target verifies (model card,
 * Architecture: Serving runs several drafter rounds in a row, and at serving
 * the predecessor token a row reads is the drafter's own previous draft;
 * section Files: the serving default is depth 2). Round 1 is kd_round with
 * the caller's pred_ids; every later round is the same round with
 * pred_ids[b][j-1] = the previous round's out_ids[b][j-1], taken on the
 * device. out_ids and out_logits receive the last round's results (earlier
 * rounds write out_ids and no logits). depth = 1 is kd_round. Arguments as
 * for kd_round; KD_ERR_ARG for depth < 1 or depth > KD_MAX_DEPTH. */
kd_status kd_round_depth(kd_ctx* ctx, int depth, int streams, const void* tapped_states,
                         const int32_t* anchor_ids, const int32_t* pred_ids,
                         const kd_kv* ctx_kv, const int32_t* ctx_lens,
                         int32_t* out_ids, float* out_logits);

/* Appends n_new context rows per stream (1 <= n_new <= KD_MAX_INGEST), the
 * context-row form of the model card's Architecture section (Input: fused
 * state and next-token embedding, 5120 -> 2560; Body: each layer's K/V of a
 * context row, RoPE at its position): row i
 * of stream b is [fuse(taps[b][i]) ; embed(next_ids[b][i])] -> fc, projected
 * through each layer's attention RMSNorm and W_k / W_v, K rotated at position
 * len + i, both rounded to bf16 (or, for KD_KV_INT4_ROT, K turned by R and
 * both coded as described at kd_kv) and written at slot (len + i) % capacity;
 * then ctx_lens[b] += n_new on the device.
 *   taps     [streams][n_new][taps][hidden] bf16 (device)
 *   next_ids [streams][n_new] int32 (device) */
kd_status kd_ingest(kd_ctx* ctx, int streams, int n_new, const void* taps,
                    const int32_t* next_ids, const kd_kv* ctx_kv, int32_t* ctx_lens);

/* Copy drafts (model card, section Use: copy drafts from the context are
 * tried before the learned block; the frozen-corpus drafting article: the
 * continuation after the longest suffix of the context, suffix length 8 down
 * to 3, most recent occurrence, a span of up to K tokens that never crosses a
 * -1 separator). Per stream, the sources are its own history and an optional
 * corpus; at each suffix length the history is tried before the corpus. An
 * occurrence must be followed by a token (in the corpus, not a separator).
 *   tokens     [streams][stride] int32 (device): each stream's history, oldest
 *              first; token ids >= 0
 *   lens       [streams] int32 (device): tokens in each history; values
 *              outside [0, stride] are clamped into it
 *   corpus     [corpus_len] int32 (device) or NULL: frozen ids, -1 between spans
 *   K          proposal length limit, 1..KD_MAX_COPY
 *   out_ids    [streams][K] int32 (device): the proposed span, -1 past its end
 *   out_info   [streams][3] int32 (device): tokens proposed (0 = no match),
 *              matched suffix length (0 or 3..8), source (0 none, 1 history,
 *              2 corpus)
 * stride and corpus_len must be below 2^31. Asynchronous on the context's
 * stream; uses the context's workspace (calls on one context must not
 * overlap). */
kd_status kd_copy_draft(kd_ctx* ctx, int streams, const int32_t* tokens, long long stride,
                        const int32_t* lens, const int32_t* corpus, long long corpus_len, int K,
                        int32_t* out_ids, int32_t* out_info);

/* kd_copy_draft without a context, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid hipMalloc):
 * it allocates nothing. Arguments and results are kd_copy_draft's; `stream`
 * is a hipStream_t (NULL: the null stream) of the current device. The
 * per-stream match keys live in a fixed device array of
 * KD_COPY_NOALLOC_MAX_STREAMS entries, one array per GPU, held until the
 * process ends and shared by every call on that GPU: calls that overlap on one
 * GPU race (serialize them, e.g. on one stream). Each call clears the keys it
 * uses before its scans. Errors: KD_ERR_ARG for streams outside
 * 1..KD_COPY_NOALLOC_MAX_STREAMS and the argument errors of kd_copy_draft;
 * KD_ERR_HIP if the array's device address cannot be found or a launch fails;
 * KD_ERR_UNSUPPORTED on a device index of 64 or more. */
#define KD_COPY_NOALLOC_MAX_STREAMS 1024
kd_status kd_copy_draft_noalloc(void* stream, int streams, const int32_t* tokens, long long stride,
                                const int32_t* lens, const int32_t* corpus, long long corpus_len,
                                int K, int32_t* out_ids, int32_t* out_info);

/* The copy source's pause guard (frozen-corpus drafting article: when fewer
 * than min_accept of the tokens proposed over the last `window` proposals were
 * accepted, the source pauses for `pause` decoded tokens, then re-arms with an
 * empty window; its defaults are 24, 0.5 and 256). Host-only state, one per
 * stream; the caller records each proposal's outcome and the tokens decoded. */
typedef struct {
  int window, pause, paused_left, count, next;
  float min_accept;
  int proposed[KD_GUARD_MAX_WINDOW], accepted[KD_GUARD_MAX_WINDOW];
} kd_copy_guard;
/* window is clamped into [1, KD_GUARD_MAX_WINDOW], pause to >= 0. */
void kd_copy_guard_init(kd_copy_guard* g, int window, float min_accept, int pause);
/* 1 while the source may propose, 0 while paused. */
int kd_copy_guard_armed(const kd_copy_guard* g);
/* One proposal of `proposed` tokens of which `accepted` were kept. */
void kd_copy_guard_record(kd_copy_guard* g, int proposed, int accepted);
/* `tokens` tokens were decoded (with or without proposals). */
void kd_copy_guard_advance(kd_copy_guard* g, int tokens);

/* Moves the context to another HIP stream. */
kd_status kd_set_stream(kd_ctx* ctx, void* hip_stream);

void kd_destroy(kd_ctx* ctx);
const char* kd_status_string(kd_status s);
/* Last error message of this context ("" if none); valid until the next call. */
const char* kd_last_error(const kd_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* KDRAFT_H */
