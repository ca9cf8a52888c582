// Host-side view of libkdraft's device state and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kd_device.h"

namespace kd {

// Device code reads the structures below through global-address-space
// pointers (a load through a generic pointer compiles to a flat access, which
// also occupies the LDS wait counter); host code sees ordinary pointers. Both
// views share one layout.
#if defined(__HIP_DEVICE_COMPILE__)
#define KD_GLOBAL __attribute__((address_space(1)))
#else
#define KD_GLOBAL
#endif
template <class T> using HostPtr = T*;
template <class T> using GlobalPtr = KD_GLOBAL T*;

// A repacked weight matrix on the device.
template <template <class> class P>
struct WMatT {
  P<const uint8_t> w = nullptr;   // codes (FP8, NVFP4) or bf16 values
  P<const float> s = nullptr;     // FP8: block scales; NVFP4: tensor scales [2][N]
  P<const uint8_t> s4 = nullptr;  // NVFP4: block-scale codes
  int N = 0, K = 0;
  int fmt = WF_FP8;
  int ks = 0;                     // NVFP4: first 64-input block of the second tensor scale
};

template <template <class> class P>
struct DevLayerT {
  WMatT<P> qkv, wo, gu, down, sa, su;
  P<const float> attn_norm = nullptr;
  P<const float> ffn_norm = nullptr;
  P<const float> spine_norm = nullptr;
};

template <template <class> class P>
struct DevWeightsT {
  WMatT<P> fuse, fc, pred_ab, pred_u;   // pred_ab = [A_p | B_p] along K
  P<const float> mask = nullptr;
  DevLayerT<P> layer[4];
  P<const float> final_norm = nullptr;
  P<const uint8_t> hq = nullptr;          // repacked NVFP4 codes
  P<const uint8_t> hs = nullptr;          // repacked e4m3 block scales
  float hg = 1.f;
  int VD = 0, VT = 0;                     // draft vocab rows, 16-row tiles
  P<const int32_t> vocab = nullptr;
  P<const uint16_t> table = nullptr;      // borrowed bf16 [full_vocab][H]
  P<const uint16_t> zrow = nullptr;       // bf16 zeros [H]: read in place of an out-of-range id's row
  int V = 0;                              // rows of the table (full vocabulary)
  P<const float> kv_signs = nullptr;      // [NL][DH] +-1 of the rotated 4-bit cache, or null
  int head_fmt = 0;                       // 0 NVFP4 (hq, hs, hg), 1 bf16 (hb), 2 FP8 (hf8)
  P<const uint16_t> hb = nullptr;         // bf16 head [VT][H/32][64 lanes][8]
  WMatT<P> hf8;                           // block-FP8 head, VT * 16 rows (zero-padded)
};

// Context K/V description passed to kernels. fmt 0: bf16 elements, strides
// in elements. fmt 1: rotated 4-bit rows (64 code bytes at k + 64 i, an fp16
// (scale, offset) pair at kso + 2 i, i = b ss + h sh + slot sl).
template <template <class> class P>
struct KVT {
  P<const uint16_t> k[4];
  P<const uint16_t> v[4];
  int64_t ss, sh, sl;
  int cap;
  int fmt = 0;
  P<const uint16_t> kso[4] = {};
  P<const uint16_t> vso[4] = {};
};

using WMat = WMatT<HostPtr>;
using DevLayer = DevLayerT<HostPtr>;
using DevWeights = DevWeightsT<HostPtr>;
using KV = KVT<HostPtr>;

// Workspace (allocated once per context for max_streams).
struct Work {
  int Bmax = 0, Rmax = 0, Imax = 0;   // streams, block rows, ingest rows
  float* f = nullptr;                 // [max(Bmax, Imax)][H] fused taps
  float* x = nullptr;                 // [Rmax][H] residual stream
  float* c = nullptr;                 // [Imax][H] ingest rows after fc
  float* part = nullptr;              // split-K partial sums
  size_t part_elems = 0;
  uint16_t* af_in = nullptr;          // afrag (f16) [max(Bmax, Imax)][NTAP*H]
  uint16_t* af_fc = nullptr;          // afrag [max(Bmax, Imax)][2H]
  uint16_t* af_ab = nullptr;          // afrag [3 Bmax][2H]
  uint16_t* af_rank = nullptr;        // afrag [3 Bmax][RK]
  uint16_t* af_x = nullptr;           // afrag [max(Rmax, Imax)][H]
  uint16_t* af_sp = nullptr;          // afrag [3 Bmax][H]
  uint16_t* af_h = nullptr;           // afrag [Rmax][FF]
  uint16_t* af_o = nullptr;           // afrag [Rmax][H]
  float* q = nullptr;                 // [Rmax][H] post-RoPE queries
  float* kb = nullptr;                // [Rmax][H] block keys (post-RoPE)
  float* vb = nullptr;                // [Rmax][H] block values
  float* rope = nullptr;              // [Bmax][BLK][DH/2][2] cos, sin
  float* att_m = nullptr;             // [Bmax][NH][nch][BLK]
  float* att_l = nullptr;             // [Bmax][NH][nch][BLK]
  float* att_o = nullptr;             // [Bmax][NH][nch][BLK][DH]
  int att_nch = 0;                    // chunks per (stream, head) = ceil(window / ATT_CH)
  unsigned* att_cnt = nullptr;        // [Bmax][NH][32] segments stored per (stream, head);
                                      // zero between attention launches
  uint16_t* af_ing = nullptr;         // afrag [NL][Imax][H]: ingest rows, RMSNorm with each layer's
  size_t af_ing_layer = 0;            //   attention gain; elements per layer
  unsigned long long* keys = nullptr; // [Rmax] argmax keys
  unsigned long long* copy_keys = nullptr;  // [2 Bmax] copy-draft (match, position) keys
};

// Row tiles of 16 for R rows.
__host__ __device__ inline int mtiles(int R) { return (R + 15) / 16; }
// Elements of an afrag buffer for R rows and K inputs.
inline size_t afrag_elems(int R, int K) { return (size_t)mtiles(R) * (K / 32) * 512; }

// Split-K policy for a projection with K/64 blocks over R rows: fixed per
// matrix while R <= 16 (one row tile), so a stream's result does not depend on
// the batch around it; fewer splits as row tiles multiply.
int gemm_splits(int K, int N, int R);

// Epilogue of a fused projection (launch_proj).
enum ProjEpiKind {
  PE_QKV = 0,     // RoPE on q and k -> q, kb, vb
  PE_SWIGLU = 1,  // silu(gate) * up -> af (afrag [R][FF])
};
struct ProjEpi {
  int kind = PE_QKV;
  const float* rope = nullptr;
  float* q = nullptr;
  float* kb = nullptr;
  float* vb = nullptr;
  uint16_t* af = nullptr;
};

// Epilogue of the ingest's k|v projections of every layer in one launch
// (launch_ingest_proj): RoPE on k at each row's absolute position len + i,
// then the cache format's store at the row's ring slot.
struct IngestEpi {
  int n_new = 1;                  // rows per stream; row r is stream r / n_new, row r % n_new
  const int32_t* lens = nullptr;  // lengths before the ingest
  float theta = 0.f;
  KV kv;
  const float* signs = nullptr;   // rotated 4-bit cache: [NL][DH] signs of R
};

// ---- launchers (kd_kernels.hip) ----
void launch_gemm(hipStream_t st, const uint16_t* af, int R, const WMat& W, int n_off_tiles,
                 int N, float* part, int splits);
void launch_prep(hipStream_t st, const Work& w, const DevWeights& d, int B, const uint16_t* taps,
                 const int32_t* lens, float theta);
// pred_stride: ids per stream in pred (3, or 4 for a previous round's out_ids)
void launch_post_fuse(hipStream_t st, const Work& w, const DevWeights& d, int B, int splits,
                      const int32_t* anchor, const int32_t* pred, int pred_stride);
void launch_silu_rank(hipStream_t st, const float* part, int splits, int rows, uint16_t* af);
void launch_rowbuild(hipStream_t st, const Work& w, const DevWeights& d, int B, int splits_fc,
                     int splits_u, const float* gain, float eps);
void launch_spine_add_norm(hipStream_t st, const Work& w, int B, int splits, const float* gain,
                           float eps);
void launch_qkv_post(hipStream_t st, const Work& w, int B, int splits);
void launch_attention(hipStream_t st, const Work& w, const DevWeights& d, int B, const KV& kv, int layer,
                      const int32_t* lens, int window);
void launch_resid_norm(hipStream_t st, const Work& w, int R, int splits, const float* gain,
                       float eps, uint16_t* af_out, int spine_rows);
void launch_swiglu(hipStream_t st, const Work& w, int R, int splits);
void launch_head(hipStream_t st, const Work& w, const DevWeights& d, int R, float* logits);
// Writes out_ids; a row whose anchor or earlier predecessor ids lie outside
// the table (see id_row_valid) gets -1.
// range_word: host-visible word set to 1 when an f16 activation store of
// this round (or of an ingest since the last round) saturated.
void launch_finalize(hipStream_t st, const Work& w, const DevWeights& d, int R, int32_t* out_ids,
                     const int32_t* anchor, const int32_t* pred, int pred_stride, unsigned* range_word);
// ingest
void launch_ingest_prep(hipStream_t st, const Work& w, int rows, const uint16_t* taps);
void launch_ingest_post_fuse(hipStream_t st, const Work& w, const DevWeights& d, int rows,
                             int splits, const int32_t* next_ids);
void launch_ingest_c(hipStream_t st, const Work& w, int rows, int splits);
// RMSNorm of each row with every layer's attention gain: af + l * af_layer.
void launch_norm_rows_layers(hipStream_t st, const float* x, int rows, const DevWeights& d,
                             float eps, uint16_t* af, size_t af_layer);
void launch_norm_rows(hipStream_t st, const float* x, int rows, const float* gain, float eps,
                      uint16_t* af);
void launch_ingest_store(hipStream_t st, const Work& w, const DevWeights& d, int B, int n_new, int splits, const KV& kv,
                         int layer, const int32_t* lens, float theta);
void launch_bump_lens(hipStream_t st, int32_t* lens, int B, int n);
// many block rows (kd_mm.hip): matrix-core tiles of 64 rows x 256 columns
bool gemm_mm_fits(int R, int N);
int gemm_mm_splits(int K, int N, int R);
void launch_gemm_mm(hipStream_t st, const uint16_t* af, int R, const WMat& W, int n_off_tiles,
                    int N, float* part, int splits);
// Projection of R rows (more than 32) with its epilogue fused, in one split.
void launch_proj(hipStream_t st, const uint16_t* af, int R, const WMat& W, const ProjEpi& e);
// The ingest's k|v projections of R rows (more than 32) for every layer in one
// launch (layer l reads af + l * af_layer), stored into the cache.
void launch_ingest_proj(hipStream_t st, const uint16_t* af, size_t af_layer, int R,
                        const DevWeights& d, const IngestEpi& e);
bool head_mm_fits(int R);
void launch_head_mm(hipStream_t st, const uint16_t* af, int R, const DevWeights& d, float* logits,
                    unsigned long long* keys);
// copy drafts (kd_copy.hip); keys: [2 B] workspace
void launch_copy_draft(hipStream_t st, int B, const int32_t* tokens, long long stride,
                       const int32_t* lens, const int32_t* corpus, long long n, int K,
                       unsigned long long* keys, int32_t* out_ids, int32_t* out_info);
// probes
void launch_probe_e4m3(hipStream_t st, uint16_t* out);
void launch_probe_nvfp4(hipStream_t st, uint16_t* out);
void launch_probe_e4m3_f16(hipStream_t st, uint16_t* out);

}  // namespace kd
