// HIP kernels of one Kolibri-1 block-drafter round for gfx950.
//
// The round (model card "Kolibri-1 block drafter", section Architecture):
//   tap fuse -> row build (anchor row through fc; rows 1-3 = mask + fused
//   state + predecessor term) -> 4 layers [spine (layers 2-4) -> RMSNorm ->
//   QKV -> RoPE -> block-causal cross-attention over the last window rows ->
//   O + residual -> RMSNorm -> SwiGLU FFN + residual] -> RMSNorm -> NVFP4 head
//   restricted to the draft vocabulary -> argmax.
//
// Projections run on the matrix cores (v_mfma_f32_16x16x32_f16): weights are
// decoded exactly from e4m3 to f16 in registers, activations enter as f16,
// and the fp32 block scale of each 64 inputs is applied to the partial sum of
// that block. Split-K partial sums are reduced in a fixed order
// by the consumer kernel, so results are deterministic.
#include "kd_device.h"
#include "kd_runtime.h"

namespace kd {

// v[0..8) += the 8 floats at p + s * stride for s = 0 .. n-1, added in that
// order (so the sum is the same as a plain loop's), the loads of up to 8
// partials issued before the first of them is added: the reductions of
// split-K partial sums are bound by load latency, not by the adds.
template <int N>
__device__ __forceinline__ void add_splits8_n(const float* p, size_t stride, float (&v)[8]) {
  f32x4 a[N][2];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    a[k][0] = *reinterpret_cast<const f32x4*>(p + (size_t)k * stride);
    a[k][1] = *reinterpret_cast<const f32x4*>(p + (size_t)k * stride + 4);
  }
#pragma unroll
  for (int k = 0; k < N; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[k][0][i];
      v[4 + i] += a[k][1][i];
    }
}
__device__ __forceinline__ void add_splits8(const float* p, size_t stride, int n, float (&v)[8]) {
  int s0 = 0;
  for (; n - s0 >= 8; s0 += 8) add_splits8_n<8>(p + (size_t)s0 * stride, stride, v);
  const float* q = p + (size_t)s0 * stride;
  switch (n - s0) {
    case 1: add_splits8_n<1>(q, stride, v); break;
    case 2: add_splits8_n<2>(q, stride, v); break;
    case 3: add_splits8_n<3>(q, stride, v); break;
    case 4: add_splits8_n<4>(q, stride, v); break;
    case 5: add_splits8_n<5>(q, stride, v); break;
    case 6: add_splits8_n<6>(q, stride, v); break;
    case 7: add_splits8_n<7>(q, stride, v); break;
    default: break;
  }
}

// ---------------------------------------------------------------------------
// Projection: part[split][r][n] = sum over the split's inputs of
// X[r][k] * W[n_off*16 + n][k], W in one of the body formats (WF).
// ---------------------------------------------------------------------------
struct GemmK {
  const uint16_t* af;
  int R, KT;
  const uint8_t* w;
  const float* s;
  const uint8_t* s4;
  int KB;        // 64-input blocks per weight row
  int N;         // output columns of this launch (multiple of 64)
  int n_off;     // first 16-row weight tile
  int WN, ks;    // NVFP4: rows of the whole matrix, first block of its second tensor scale
  float* part;
  int splits, kbs;
};

template <int WF>
__global__ __launch_bounds__(256) void k_gemm(GemmK g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ngroups = g.N >> 6;
  int u = blockIdx.x;
  const int ng = u % ngroups;
  u /= ngroups;
  const int sp = u % g.splits;
  const int mt = u / g.splits;
  const int nt = ng * 4 + wave;
  const int ntw = nt + g.n_off;
  const int b0 = sp * g.kbs;
  const int row = mt * 16 + (lane & 15);
  const bool rv = row < g.R;
  // the block multiplier: FP8 its block scale; NVFP4 the column's tensor
  // scale of the block's side of the split; bf16 none
  const float* spp = g.s + ((size_t)ntw * g.KB + b0) * 16 + (lane & 15);
  float gt0 = 1.f, gt1 = 1.f;
  if constexpr (WF == WF_NVFP4) {
    gt0 = g.s[ntw * 16 + (lane & 15)];
    gt1 = g.s[g.WN + ntw * 16 + (lane & 15)];
  }
  const uint16_t* ap = g.af + ((size_t)mt * g.KT + 2 * b0) * 512 + lane * 8;
  const f16x8 zero = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int i = 0; i < g.kbs; ++i) {
    const WBlock<WF> wb = load_wblock<WF>(g.w, g.s4, g.KB, ntw, b0 + i, lane);
    float sc = 1.f;
    if constexpr (WF == WF_FP8) sc = spp[i * 16];
    if constexpr (WF == WF_NVFP4) sc = b0 + i < g.ks ? gt0 : gt1;
    f16x8 a0 = zero, a1 = zero;
    if (rv) {
      const uint16_t* a = ap + (size_t)i * 1024;
      a0 = *reinterpret_cast<const f16x8*>(a);
      a1 = *reinterpret_cast<const f16x8*>(a + 512);
    }
    const f32x4 t = wb.mul(a0, a1);
    if constexpr (WF == WF_BF16) acc += t;
    else acc += sc * t;
  }
  float* out = g.part + (size_t)sp * g.R * g.N + nt * 16 + (lane & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = mt * 16 + 4 * (lane >> 4) + e;
    if (r < g.R) out[(size_t)r * g.N] = acc[e];
  }
}

static int splits_for(int KB, int want) {
  int s = want < 1 ? 1 : (want > KB ? KB : want);
  while (KB % s) --s;
  return s;
}

int gemm_splits(int K, int N, int R) {
  if (gemm_mm_fits(R, N)) return gemm_mm_splits(K, N, R);
  const int KB = K / 64;
  int base;
  if (N <= 256) base = KB / 4;           // rank-256 adapters: thin matrices, split deep
  else if (KB <= 4) base = 1;            // K = 256 (adapter U)
  else if (KB >= 96) base = KB / 8;      // fuse (120), down (96)
  else if (KB >= 80) base = KB / 8;      // fc (80)
  else base = KB / 4;                    // K = 2560
  const int mt = mtiles(R);
  return splits_for(KB, mt == 1 ? base : base / mt);
}

void launch_gemm(hipStream_t st, const uint16_t* af, int R, const WMat& W, int n_off_tiles,
                 int N, float* part, int splits) {
  if (gemm_mm_fits(R, N)) return launch_gemm_mm(st, af, R, W, n_off_tiles, N, part, splits);
  GemmK g;
  g.af = af;
  g.R = R;
  g.KT = W.K / 32;
  g.w = W.w;
  g.s = W.s;
  g.s4 = W.s4;
  g.KB = W.K / 64;
  g.N = N;
  g.n_off = n_off_tiles;
  g.WN = W.N;
  g.ks = W.ks;
  g.part = part;
  g.splits = splits;
  g.kbs = g.KB / splits;
  const int blocks = mtiles(R) * splits * (N / 64);
  if (W.fmt == WF_NVFP4) k_gemm<WF_NVFP4><<<blocks, 256, 0, st>>>(g);
  else if (W.fmt == WF_BF16) k_gemm<WF_BF16><<<blocks, 256, 0, st>>>(g);
  else k_gemm<WF_FP8><<<blocks, 256, 0, st>>>(g);
}

// ---------------------------------------------------------------------------
// Round prologue: tapped states -> afrag, argmax keys cleared, RoPE table for
// block positions len + j (angles in double: positions reach the thousands).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prep(uint16_t* af_in, const uint16_t* taps,
                                              unsigned long long* keys, float* rope,
                                              const int32_t* lens, float theta) {
  const int b = blockIdx.x;
  constexpr int K = NTAP * H, KT = K / 32;
  for (int g = threadIdx.x; g < K / 8; g += blockDim.x) {
    u32x4 bits = *reinterpret_cast<const u32x4*>(taps + (size_t)b * K + g * 8);
    store_afrag8_bf16(af_in, KT, b, g * 8, bits);
  }
  if (threadIdx.x < BLK) keys[b * BLK + threadIdx.x] = 0ull;
  const int j = threadIdx.x >> 6, fi = threadIdx.x & 63;
  const double pos = (double)lens[b] + j;
  const double ang = pos * pow((double)theta, -(double)fi / (DH / 2));
  rope[((b * BLK + j) * (DH / 2) + fi) * 2 + 0] = (float)cos(ang);
  rope[((b * BLK + j) * (DH / 2) + fi) * 2 + 1] = (float)sin(ang);
}

void launch_prep(hipStream_t st, const Work& w, const DevWeights& d, int B, const uint16_t* taps,
                 const int32_t* lens, float theta) {
  (void)d;
  k_prep<<<B, 256, 0, st>>>(w.af_in, taps, w.keys, w.rope, lens, theta);
}

// f = sum of fuse partials; afrag of [f ; E[anchor]] (fc input) and of
// [f ; E[pred_j]] for j = 0..2 (input of [A_p | B_p]).
__global__ __launch_bounds__(320) void k_post_fuse(const float* part, int splits, int B, float* f,
                                                   uint16_t* af_fc, uint16_t* af_ab,
                                                   const uint16_t* table, const uint16_t* zrow,
                                                   int V, const int32_t* anchor,
                                                   const int32_t* pred, int pred_stride) {
  const int b = blockIdx.x, c0 = threadIdx.x * 8;
  constexpr int KT = 2 * H / 32;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  add_splits8(part + (size_t)b * H + c0, (size_t)B * H, splits, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[(size_t)b * H + c0 + i] = v[i];
  store_afrag8(af_fc, KT, b, c0, v);
  const u32x4 ea = *reinterpret_cast<const u32x4*>(table_row(table, zrow, anchor[b], V, H) + c0);
  store_afrag8_bf16(af_fc, KT, b, H + c0, ea);
  for (int j = 0; j < BLK - 1; ++j) {
    store_afrag8(af_ab, KT, b * 3 + j, c0, v);
    const u32x4 ep =
        *reinterpret_cast<const u32x4*>(table_row(table, zrow, pred[b * pred_stride + j], V, H) + c0);
    store_afrag8_bf16(af_ab, KT, b * 3 + j, H + c0, ep);
  }
}

void launch_post_fuse(hipStream_t st, const Work& w, const DevWeights& d, int B, int splits,
                      const int32_t* anchor, const int32_t* pred, int pred_stride) {
  k_post_fuse<<<B, 320, 0, st>>>(w.part, splits, B, w.f, w.af_fc, w.af_ab, d.table, d.zrow, d.V, anchor,
                                 pred, pred_stride);
}

// afrag of silu(sum of partials) for a rank-256 hidden vector.
__global__ __launch_bounds__(32) void k_silu_rank(const float* part, int splits, int rows,
                                                  uint16_t* af) {
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  add_splits8(part + (size_t)r * RK + c0, (size_t)rows * RK, splits, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = silu(v[i]);
  store_afrag8(af, RK / 32, r, c0, v);
}

void launch_silu_rank(hipStream_t st, const float* part, int splits, int rows, uint16_t* af) {
  k_silu_rank<<<rows, 32, 0, st>>>(part, splits, rows, af);
}

// RMSNorm of one row (8 values per thread, 320 threads) with the gain, into
// afrag row `row`.
__device__ __forceinline__ void norm_row_store(const float (&v)[8], int row, const float* gain, float eps,
                                               uint16_t* af, float* red) {
  const int c0 = threadIdx.x * 8;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  ss = block_sum<5>(ss, red);
  const float inv = 1.0f / sqrtf(ss / H + eps);
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = gain[c0 + i] * v[i] * inv;
  store_afrag8(af, H / 32, row, c0, o);
}

// Block rows: x0 = fc partials; x_j = mask + f + U_p partials (j = 1..3);
// then the first layer's attention RMSNorm into afrag. One workgroup per
// block row (stream b = row / 4, j = row % 4).
__global__ __launch_bounds__(320) void k_rowbuild(const float* __restrict__ part_fc, int splits_fc,
                                                  const float* __restrict__ part_u, int splits_u, int B,
                                                  const float* __restrict__ f, const float* __restrict__ mask,
                                                  float* __restrict__ x, const float* __restrict__ gain,
                                                  float eps, uint16_t* __restrict__ af) {
  __shared__ float red[8];
  const int row = blockIdx.x, b = row >> 2, j = row & 3, c0 = threadIdx.x * 8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (j == 0) {
    add_splits8(part_fc + (size_t)b * H + c0, (size_t)B * H, splits_fc, v);
  } else {
    add_splits8(part_u + (size_t)(b * 3 + j - 1) * H + c0, (size_t)3 * B * H, splits_u, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (mask[c0 + i] + f[(size_t)b * H + c0 + i]) + v[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[(size_t)row * H + c0 + i] = v[i];
  norm_row_store(v, row, gain, eps, af, red);
}

void launch_rowbuild(hipStream_t st, const Work& w, const DevWeights& d, int B, int splits_fc,
                     int splits_u, const float* gain, float eps) {
  const size_t half = w.part_elems / 2;
  k_rowbuild<<<BLK * B, 320, 0, st>>>(w.part, splits_fc, w.part + half, splits_u, B, w.f, d.mask, w.x,
                                      gain, eps, w.af_x);
}

// Spine add (rows 1..3 of each stream) and the layer's attention RMSNorm.
__global__ __launch_bounds__(320) void k_spine_add_norm(const float* __restrict__ part, int splits, int B,
                                                        float* __restrict__ x, const float* __restrict__ gain,
                                                        float eps, uint16_t* __restrict__ af) {
  __shared__ float red[8];
  const int row = blockIdx.x, b = row >> 2, j = row & 3, c0 = threadIdx.x * 8;
  float* xr = x + (size_t)row * H + c0;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = xr[i];
  if (j > 0) {
    float add[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) add[i] = 0.f;
    add_splits8(part + (size_t)(b * 3 + j - 1) * H + c0, (size_t)3 * B * H, splits, add);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] += add[i];
      xr[i] = v[i];
    }
  }
  norm_row_store(v, row, gain, eps, af, red);
}

void launch_spine_add_norm(hipStream_t st, const Work& w, int B, int splits, const float* gain,
                           float eps) {
  k_spine_add_norm<<<BLK * B, 320, 0, st>>>(w.part, splits, B, w.x, gain, eps, w.af_x);
}

// q|k|v partials -> q, k (RoPE, rotate-half) and v for every block row.
__global__ __launch_bounds__(256) void k_qkv_post(const float* part, int splits, int R,
                                                  const float* rope, float* q, float* kb,
                                                  float* vb) {
  const int r = blockIdx.x, b = r >> 2, j = r & 3;
  for (int p = threadIdx.x; p < NH * DH / 2; p += blockDim.x) {
    const int h = p >> 6, fi = p & 63;
    const int c0 = h * DH + fi, c1 = c0 + DH / 2;
    float qa = 0.f, qb = 0.f, ka = 0.f, kb2 = 0.f, va = 0.f, vb2 = 0.f;
    const int pq0 = qkv_position(c0), pq1 = qkv_position(c1);
    const int pk0 = qkv_position(H + c0), pk1 = qkv_position(H + c1);
    const int pv0 = qkv_position(2 * H + c0), pv1 = qkv_position(2 * H + c1);
    for (int s = 0; s < splits; ++s) {
      const float* pr = part + ((size_t)s * R + r) * QKV;
      qa += pr[pq0];
      qb += pr[pq1];
      ka += pr[pk0];
      kb2 += pr[pk1];
      va += pr[pv0];
      vb2 += pr[pv1];
    }
    const float cs = rope[((b * BLK + j) * (DH / 2) + fi) * 2];
    const float sn = rope[((b * BLK + j) * (DH / 2) + fi) * 2 + 1];
    float* qr = q + (size_t)r * H;
    float* kr = kb + (size_t)r * H;
    float* vr = vb + (size_t)r * H;
    qr[c0] = qa * cs - qb * sn;
    qr[c1] = qa * sn + qb * cs;
    kr[c0] = ka * cs - kb2 * sn;
    kr[c1] = ka * sn + kb2 * cs;
    vr[c0] = va;
    vr[c1] = vb2;
  }
}

void launch_qkv_post(hipStream_t st, const Work& w, int B, int splits) {
  k_qkv_post<<<B * BLK, 256, 0, st>>>(w.part, splits, B * BLK, w.rope, w.q, w.kb, w.vb);
}

// ---------------------------------------------------------------------------
// Cross-attention over the context window (model card, Architecture, Body:
// every block row attends to the last window rows of its stream's cached K/V
// and causally to the block). A workgroup takes one segment of one (stream,
// head): segments of equal length (segb 16-key blocks, chosen per launch so
// that a full window gives enough workgroups to fill the chip), as many as
// the stream's visible context needs. Wave w takes the
// segment's blocks w, w + 4, ..., with the next block's keys and values in
// flight while one is computed:
//   scores  S^T[key][j] = K Q^T on the matrix cores (16x16x32 bf16): keys as
//           the A operand (lane: key lane%16, dims 32kb + 8(lane/16)), the
//           queries (pre-scaled by log2(e)/sqrt(128)) split into bf16 hi + lo
//           as the B operand (column j < 4 of the 4 block rows);
//   softmax running max and sum per row j (log2 units), the output rescaled
//           when the max grows;
//   P V     on the vector units: lane (g, c) adds keys 4g..4g+3 of the block
//           for dims 8c..8c+7 of all 4 rows.
// The 4 waves' states are merged in LDS. With one segment the workgroup also
// adds the block's own keys (row j sees block rows 0..j), normalises, and
// writes the output rows; otherwise it stores the segment's max m, sum l and
// unnormalised output o, and the workgroup that stores the pair's last
// segment merges them with the block's own keys.
// ---------------------------------------------------------------------------
struct AttnK {
  const float* q;
  const float* kb;
  const float* vb;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kso;    // rotated 4-bit cache: (scale, offset) fp16 pairs
  const uint16_t* vso;
  const float* signs;     // rotated 4-bit cache: the layer's [DH] signs
  int64_t ss, sh, sl;
  int cap, window, nch;
  int segb;               // 16-key blocks per segment (a pair has ceil(blocks / segb) segments)
  const int32_t* lens;
  float* pm;
  float* pl;
  float* po;
  unsigned* cnt;          // [B][NH][32] segments stored per pair, zero between launches
  uint16_t* af_o;
};

// The block's own keys for rows j = 0..3 of one (stream, head), merged into
// (M, L, O) of thread item (j, d); returns the normalised output.
__device__ __forceinline__ float attn_block_merge(const float* sblk, const float* vb, size_t vrow0,
                                                  int j, int d, float M, float L, float O) {
  float Mn = M;
#pragma unroll
  for (int i = 0; i < BLK; ++i)
    if (i <= j) Mn = fmaxf(Mn, sblk[j * BLK + i]);
  const float f = M == -__builtin_inff() ? 0.f : exp2f(M - Mn);
  L *= f;
  O *= f;
#pragma unroll
  for (int i = 0; i < BLK; ++i)
    if (i <= j) {
      const float p = exp2f(sblk[j * BLK + i] - Mn);
      L += p;
      O += p * vb[vrow0 + (size_t)i * H + d];
    }
  return O / L;
}

// The end of a segment workgroup: the 4 key groups of each wave summed, the
// 4 waves merged in LDS, then either the block's own keys added and the
// output rows written (one segment) or the segment's (m, l, o) stored.
// Thread (lr, lg) of wave w holds o[j][e] = unnormalised output of row j,
// dims 8 lr + e, over its key group; m_run / l_run are row lr's (lr < 4).
struct AttnLds {
  float o[4][BLK][DH];           // per wave: unnormalised output of each row
  float m[4][BLK], l[4][BLK];    // per wave: running max and sum of each row
  float blk[BLK * BLK];          // the block's own scores
  int last;                      // this workgroup stored its pair's last segment
};

__device__ __forceinline__ void attn_merge(const AttnK& a, AttnLds& s, float m_run, float l_run,
                                           int seg, int nseg, int h, int b, size_t qrow0);

__device__ __forceinline__ void attn_finish(const AttnK& a, AttnLds& s, float (&o)[BLK][8],
                                            float m_run, float l_run, int seg, int nseg, int h,
                                            int b, size_t qrow0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // sum the 4 key groups of the wave: lanes lg = 0 end with o[j][8 lr + e]
#pragma unroll
  for (int j = 0; j < BLK; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[j][e] += __shfl_xor(o[j][e], 16, 64);
      o[j][e] += __shfl_xor(o[j][e], 32, 64);
    }
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < BLK; ++j) {
      *reinterpret_cast<f32x4*>(&s.o[wave][j][8 * lr]) = f32x4{o[j][0], o[j][1], o[j][2], o[j][3]};
      *reinterpret_cast<f32x4*>(&s.o[wave][j][8 * lr + 4]) = f32x4{o[j][4], o[j][5], o[j][6], o[j][7]};
    }
  }
  attn_merge(a, s, m_run, l_run, seg, nseg, h, b, qrow0);
}

// The block's own scores s.blk[j][i] (i <= j), scaled like the context's:
// wave j, lane l covers dims 2l, 2l+1.
__device__ __forceinline__ void attn_block_scores(const AttnK& a, AttnLds& s, size_t qrow0) {
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  const float q0 = a.q[qrow0 + (size_t)j * H + 2 * lane], q1 = a.q[qrow0 + (size_t)j * H + 2 * lane + 1];
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    if (i > j) break;
    const float* kp = a.kb + qrow0 + (size_t)i * H + 2 * lane;
    const float p = wave_sum(q0 * kp[0] + q1 * kp[1]);
    if (lane == 0) s.blk[j * BLK + i] = p * qs;
  }
}

// Wave w's s.o[w] must hold its rows' unnormalised outputs; m_run / l_run
// are row lr's (lanes lr < 4). Merges the 4 waves and finishes the segment:
// a pair with one segment adds the block's own keys and writes the output
// rows; otherwise the segment's (m, l, o) is stored (written through to the
// device-coherent level), the pair's counter counts it, and the workgroup
// that stores the pair's last segment merges all of them in segment order
// (so the result does not depend on which one that is) and resets the
// counter for the next launch.
__device__ __forceinline__ void attn_merge(const AttnK& a, AttnLds& s, float m_run, float l_run,
                                           int seg, int nseg, int h, int b, size_t qrow0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // row lr's max and sum live in every lane with lane % 16 == lr
  if (lane < BLK) {
    s.m[wave][lane] = m_run;
    s.l[wave][lane] = l_run;
  }
  if (nseg == 1) attn_block_scores(a, s, qrow0);
  __syncthreads();
  const size_t pair = (size_t)(b * NH + h);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (threadIdx.x >> 7) + 2 * it, d = threadIdx.x & 127;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s.m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (s.m[w][j] != -__builtin_inff()) {
        const float f = exp2f(s.m[w][j] - M);
        L += s.l[w][j] * f;
        O += s.o[w][j][d] * f;
      }
    }
    if (nseg == 1) {
      const float out = attn_block_merge(s.blk, a.vb, qrow0, j, d, M, L, O);
      a.af_o[afrag_off(b * BLK + j, h * DH + d, H / 32)] = __builtin_bit_cast(uint16_t, f16_checked(out));
    } else {
      const size_t pb = (pair * a.nch + seg) * BLK + j;
      __hip_atomic_store(&a.po[pb * DH + d], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(&a.pm[pb], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.pl[pb], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (nseg == 1) return;
  // count the segment once every store of the workgroup is acknowledged
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = a.cnt + pair * 32;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(nseg - 1);
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.last = last;
  }
  __syncthreads();
  if (!s.last) return;
  // thread (j, d) of rows j = tid / 128 and j + 2: every segment's partial
  // loaded at once (indices clamped to the last segment, the extra ones
  // masked; lane c < 16 loads segment c's max and sum of row j, lane 16 + c
  // those of row j + 2), with the block's own scores in flight, then merged
  // in segment order
  constexpr int MAXS = 16;
  const size_t pbl = pair * a.nch * BLK + (threadIdx.x >> 7) + 2 * ((lane >> 4) & 1) +
                     (size_t)min(lane & 15, nseg - 1) * BLK;
  const float m_lane = __hip_atomic_load(&a.pm[pbl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float l_lane = __hip_atomic_load(&a.pl[pbl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float po[2][MAXS];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (threadIdx.x >> 7) + 2 * it, d = threadIdx.x & 127;
    const size_t pb0 = pair * a.nch * BLK + j;
#pragma unroll
    for (int c = 0; c < MAXS; ++c) {
      const size_t pb = pb0 + (size_t)min(c, nseg - 1) * BLK;
      po[it][c] = __hip_atomic_load(&a.po[pb * DH + d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  attn_block_scores(a, s, qrow0);
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (threadIdx.x >> 7) + 2 * it, d = threadIdx.x & 127;
    float pm[MAXS], pl[MAXS];
#pragma unroll
    for (int c = 0; c < MAXS; ++c) {
      pm[c] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_lane), 16 * it + c));
      pl[c] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_lane), 16 * it + c));
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < MAXS; ++c)
      if (c < nseg) M = fmaxf(M, pm[c]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int c = 0; c < MAXS; ++c) {
      if (c < nseg && pm[c] != -__builtin_inff()) {
        const float f = exp2f(pm[c] - M);
        L += pl[c] * f;
        O += po[it][c] * f;
      }
    }
    const float out = attn_block_merge(s.blk, a.vb, qrow0, j, d, M, L, O);
    a.af_o[afrag_off(b * BLK + j, h * DH + d, H / 32)] = __builtin_bit_cast(uint16_t, f16_checked(out));
  }
}

__global__ __launch_bounds__(256) void k_attn_split(AttnK a) {
  __shared__ AttnLds lds;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int len = a.lens[b];
  const int n = min(len, a.window);
  const int nblk = (n + 15) >> 4;
  // segments of a.segb blocks; workgroups past the pair's last segment have
  // no work (an empty context still has one segment: the block's own keys)
  const int nseg = max(1, (nblk + a.segb - 1) / a.segb);
  if (seg >= nseg) return;
  const int blk0 = seg * a.segb, blk1 = min(nblk, blk0 + a.segb);
  const float qs = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  const size_t qrow0 = (size_t)(b * BLK) * H + h * DH;

  float m_run = -__builtin_inff(), l_run = 0.f;
  float o[BLK][8];
#pragma unroll
  for (int j = 0; j < BLK; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;

  if (blk0 < blk1) {
    // queries as the B operand: lane (lr, lg) holds q_lr[32kb + 8lg .. + 8] (rows >= 4 zero)
    bf16x8 qh[4], ql[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float qv[8];
      if (lr < BLK) {
        const float* qp = a.q + qrow0 + (size_t)lr * H + 32 * kb + 8 * lg;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(qp);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(qp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[e] = x0[e] * qs;
          qv[4 + e] = x1[e] * qs;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hh = (__bf16)qv[e];
        qh[kb][e] = hh;
        ql[kb][e] = (__bf16)(qv[e] - (float)hh);
      }
    }
    const uint16_t* kbase = a.k + b * a.ss + h * a.sh;
    const uint16_t* vbase = a.v + b * a.ss + h * a.sh;
    const int f0 = (len - n) % a.cap;
    auto slot_of = [&](int key) {
      const int s_ = f0 + min(key, n - 1);
      return s_ - (s_ >= a.cap ? a.cap : 0);
    };
    // keys past n are clamped to the last visible key and masked in the scores
    auto load_blk = [&](int bi, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
      const uint16_t* kp = kbase + (size_t)slot_of(16 * bi + lr) * a.sl + 8 * lg;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kr[kb] = *reinterpret_cast<const u32x4*>(kp + 32 * kb);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vr[t] = *reinterpret_cast<const u32x4*>(vbase + (size_t)slot_of(16 * bi + 4 * lg + t) * a.sl + 8 * lr);
    };
    auto process = [&](int bi, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) __attribute__((always_inline)) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kk = __builtin_bit_cast(bf16x8, kr[kb]);
        acc = mfma_bf16(kk, qh[kb], acc);
        acc = mfma_bf16(kk, ql[kb], acc);
      }
      // lane (lr, lg): acc[e] = S^T[key 4lg + e][row lr]
      float sc[4], mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = 16 * bi + 4 * lg + e < n ? acc[e] : -__builtin_inff();
        mx = fmaxf(mx, sc[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -__builtin_inff() ? 0.f : exp2f(m_run - m_new);
      float pe[4], ls = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = sc[e] == -__builtin_inff() ? 0.f : exp2f(sc[e] - m_new);
        ls += pe[e];
      }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l_run = l_run * alpha + ls;
      m_run = m_new;
      // the outputs are rescaled only when some row's maximum grew
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int j = 0; j < BLK; ++j) {
          const float aj = __shfl(alpha, j, 64);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[j][e] *= aj;
        }
      }
      // lane (g = lg, c = lr) gathers P[j][4g + t] from lane (j, g)
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        float pj[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) pj[t] = __shfl(pe[t], (lg << 4) | j, 64);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float vf[8];
          bf16x8_to_f32(vr[t], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[j][e] += pj[t] * vf[e];
        }
      }
    };
    // blocks of this wave: blk0 + wave + 4i; two register sets alternate so the
    // next block's loads are in flight while one is computed
    const int last = blk1 - 1;
    int bi = blk0 + wave;
    u32x4 kA[4], vA[4], kB[4], vB[4];
    load_blk(min(bi, last), kA, vA);
    for (; bi <= last; bi += 8) {
      load_blk(min(bi + 4, last), kB, vB);
      process(bi, kA, vA);
      if (bi + 4 > last) break;
      load_blk(min(bi + 8, last), kA, vA);
      process(bi + 4, kB, vB);
    }
  }
  attn_finish(a, lds, o, m_run, l_run, seg, nseg, h, b, qrow0);
}


// ---------------------------------------------------------------------------
// Rotated 4-bit context cache (the article "Serving Kolibri-1 with a 4-bit KV
// cache", section What we do): keys are cached as codes of R k with
// R = H diag(s)/sqrt(128), values as codes of v, one fp16 (scale, offset) per
// (stream, head, slot) row; the query is turned by the same R, so the scores
// are those of the unrotated keys.
// ---------------------------------------------------------------------------

// The segment workgroup of k_attn_split for the rotated 4-bit cache. Per
// 16-key block, lane (lr, lg):
//   scores  K codes of key lr, dims 32 lg .. 32 lg + 31 (one 16-byte load),
//           as the A operand of four 16x16x32 f16 MFMAs, MFMA kb pairing
//           operand column 8 lg + e with dim 32 lg + 8 kb + e; the rotated
//           queries (split into f16 hi + lo) use the same pairing. A key's
//           score is scale * (q_rot . codes) + offset * sum(q_rot);
//   P V     on the matrix cores too, as O^T = V^T P'^T with P' = p * scale
//           (16x16x16 f16, k = the block's 16 keys): the lane loads the V
//           codes of keys 4 lg + e, dims 8 lr .. 8 lr + 7, and MFMA t (t =
//           0..7) takes dim 8 i + t as its operand row i, so nibble t of the
//           lane's 4 dwords is its A operand; its B operand, P'[lr][4 lg + e],
//           is exactly what the lane's scores produced. MFMA t leaves
//           O[lr][32 lg + 8 e + t] in element e of accumulator t. The sum over
//           keys of p * offset is one number per row, carried beside the
//           output and added to every dim.
__global__ __launch_bounds__(256) void k_attn_split_q4(AttnK a) {
  __shared__ AttnLds lds;
  __shared__ float s_q[BLK][DH];
  __shared__ float s_qsum[BLK];
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int len = a.lens[b];
  const int n = min(len, a.window);
  const int nblk = (n + 15) >> 4;
  // segments of a.segb blocks; workgroups past the pair's last segment have
  // no work (an empty context still has one segment: the block's own keys)
  const int nseg = max(1, (nblk + a.segb - 1) / a.segb);
  if (seg >= nseg) return;
  const int blk0 = seg * a.segb, blk1 = min(nblk, blk0 + a.segb);
  const float qs = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  const size_t qrow0 = (size_t)(b * BLK) * H + h * DH;

  float m_run = -__builtin_inff(), l_run = 0.f, w_run = 0.f;
  f32x4 oa[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) oa[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (blk0 < blk1) {
    // wave j turns block row j's query: R q = H (s * q) / sqrt(128), scaled
    // like the scores (1/sqrt(128) * log2(e))
    {
      const float* qp = a.q + qrow0 + (size_t)wave * H;
      float y0 = qp[lane] * a.signs[lane], y1 = qp[lane + 64] * a.signs[lane + 64];
      fwht128(y0, y1, lane);
      const float f = 0.08838834764831845f * qs;
      y0 *= f;
      y1 *= f;
      s_q[wave][lane] = y0;
      s_q[wave][lane + 64] = y1;
      const float t = wave_sum(y0 + y1);
      if (lane == 0) s_qsum[wave] = t;
    }
    __syncthreads();
    f16x8 qh[4], ql[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = lr < BLK ? s_q[lr][32 * lg + 8 * kb + e] : 0.f;
        const _Float16 hh = (_Float16)v;
        qh[kb][e] = hh;
        ql[kb][e] = (_Float16)(v - (float)hh);
      }
    const float qsum = lr < BLK ? s_qsum[lr] : 0.f;

    // the rows of this (stream, head) through buffer resources: 32-bit
    // offsets from a base held in scalar registers, and the hardware returns
    // 0 for any offset past the span (the host checks the span fits 4 GiB)
    const size_t row0 = (size_t)(b * a.ss + h * a.sh);
    const uint32_t span = (uint32_t)((a.cap - 1) * a.sl + 1);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(a.k) + row0 * 64), (short)0, span * 64, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const uint8_t*>(a.v) + row0 * 64), (short)0, span * 64, 0x00020000);
    const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kso + row0 * 2), (short)0, span * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.vso + row0 * 2), (short)0, span * 4, 0x00020000);
    const uint32_t sl = (uint32_t)a.sl;
    const int f0 = (len - n) % a.cap;
    auto row_of = [&](int key) {
      const int s_ = f0 + min(key, n - 1);
      return (uint32_t)(s_ - (s_ >= a.cap ? a.cap : 0)) * sl;
    };
    // keys past n are clamped to the last visible key and masked in the scores
    // lane (lr, lg) reads key lr's K codes (dims 32 lg ..) and its scale
    // and offset pairs; the V codes of keys 4 lg + t (dims 8 lr ..)
    auto load_blk = [&](int bi, u32x4& kr, uint32_t (&vr)[4], uint32_t& ks, uint32_t& vs) {
      const uint32_t rk0 = row_of(16 * bi + lr);
      kr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, rk0 * 64 + 16 * lg, 0, 0));
      ks = __builtin_amdgcn_raw_buffer_load_b32(rks, rk0 * 4, 0, 0);
      vs = __builtin_amdgcn_raw_buffer_load_b32(rvs, rk0 * 4, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vr[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, row_of(16 * bi + 4 * lg + t) * 64 + 4 * lr, 0, 0);
    };
    auto process = [&](int bi, const u32x4& kr, const uint32_t (&vr)[4], uint32_t ks_l,
                       uint32_t vs_l) __attribute__((always_inline)) {
      // the scale and offset pairs of keys 4 lg + e come from lanes 4 lg + e
      uint32_t ks[4], vs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ks[e] = __shfl(ks_l, 4 * lg + e, 64);
        vs[e] = __shfl(vs_l, 4 * lg + e, 64);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f16x8 kk = nib8_f16(kr[kb]);
        acc = mfma_f16(kk, qh[kb], acc);
        acc = mfma_f16(kk, ql[kb], acc);
      }
      // lane (lr, lg): acc[e] = q_rot[lr] . codes[key 4lg + e] * 2^-24
      float sc[4], mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float ksc, kof;
        so_unpack(ks[e], ksc, kof);
        sc[e] = 16 * bi + 4 * lg + e < n ? (ksc * KD_2P24) * acc[e] + kof * qsum : -__builtin_inff();
        mx = fmaxf(mx, sc[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -__builtin_inff() ? 0.f : exp2f(m_run - m_new);
      f16x4 pb;
      float ls = 0.f, ws = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = sc[e] == -__builtin_inff() ? 0.f : exp2f(sc[e] - m_new);
        float vsc, vof;
        so_unpack(vs[e], vsc, vof);
        ls += p;
        ws += p * vof;
        pb[e] = (_Float16)(p * vsc);
      }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l_run = l_run * alpha + ls;
      w_run = w_run * alpha + ws;
      m_run = m_new;
      // even nibbles (dims 8 lr + 2m) and odd nibbles (8 lr + 2m + 1) per key
      uint32_t ev[4], od[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ev[e] = vr[e] & 0x0F0F0F0Fu;
        od[e] = (vr[e] >> 4) & 0x0F0F0F0Fu;
      }
      // the outputs are rescaled only when some row's maximum grew (after
      // the first blocks, most blocks leave every maximum as it was)
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) oa[t] *= alpha;
      }
#define KD_PV_TILE(T, X, M)                                                    \
  {                                                                            \
    const f16x2 lo = byte_pair_f16<M>(X[0], X[1]);                             \
    const f16x2 hi = byte_pair_f16<M>(X[2], X[3]);                             \
    oa[T] = mfma_16x16x16_f16(f16x4{lo.x, lo.y, hi.x, hi.y}, pb, oa[T]);       \
  }
      KD_PV_TILE(0, ev, 0)
      KD_PV_TILE(1, od, 0)
      KD_PV_TILE(2, ev, 1)
      KD_PV_TILE(3, od, 1)
      KD_PV_TILE(4, ev, 2)
      KD_PV_TILE(5, od, 2)
      KD_PV_TILE(6, ev, 3)
      KD_PV_TILE(7, od, 3)
#undef KD_PV_TILE
    };
    // blocks of this wave: blk0 + wave + 4i; two register sets alternate so
    // the next block's loads are in flight while one is computed
    const int last = blk1 - 1;
    int bi = blk0 + wave;
    u32x4 kA, kB;
    uint32_t vA[4], vB[4], ksA, ksB, vsA, vsB;
    load_blk(min(bi, last), kA, vA, ksA, vsA);
    for (; bi <= last; bi += 8) {
      load_blk(min(bi + 4, last), kB, vB, ksB, vsB);
      process(bi, kA, vA, ksA, vsA);
      if (bi + 4 > last) break;
      load_blk(min(bi + 8, last), kA, vA, ksA, vsA);
      process(bi + 4, kB, vB, ksB, vsB);
    }
  }
  // the offsets' share of row lr, summed over the 4 key groups
  w_run += __shfl_xor(w_run, 16, 64);
  w_run += __shfl_xor(w_run, 32, 64);
  // lane (lr < 4, lg) holds dims 32 lg + 8 e + t of row lr, times 2^-24
  if (lr < BLK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = oa[t][e] * KD_2P24 + w_run;
      float* dst = &lds.o[wave][lr][32 * lg + 8 * e];
      *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
  }
  attn_merge(a, lds, m_run, l_run, seg, nseg, h, b, qrow0);
}

// workgroups a full window of every pair is split into (about four per CU;
// B16 with ragged contexts measured 0.695 ms per step at 2048, six segments
// per pair, and 0.672 ms at 1024, three)
constexpr int ATT_WG = 1024;

void launch_attention(hipStream_t st, const Work& w, const DevWeights& dw, int B, const KV& kv,
                      int layer, const int32_t* lens, int window) {
  AttnK a;
  a.kso = kv.kso[layer];
  a.vso = kv.vso[layer];
  a.signs = dw.kv_signs ? dw.kv_signs + layer * DH : nullptr;
  a.q = w.q;
  a.kb = w.kb;
  a.vb = w.vb;
  a.k = kv.k[layer];
  a.v = kv.v[layer];
  a.ss = kv.ss;
  a.sh = kv.sh;
  a.sl = kv.sl;
  a.cap = kv.cap;
  a.window = window;
  a.nch = w.att_nch;
  // segments of equal length (segb blocks of 16 keys): a full window splits
  // into as many segments as keep the pairs' workgroups at or below ATT_WG
  // (one segment once the pairs alone reach it), at most the partial slots
  // per pair; shorter contexts take fewer segments
  // up to 4 streams (a comparison path there: the small-batch path serves
  // them) every pair takes the most segments, so that a stream's partials are
  // the same alone and among up to 4
  const int pairs = B * NH;
  const int wb = (window + 15) / 16;
  int S = B <= 4 ? w.att_nch : ATT_WG / pairs;
  S = std::max(1, std::min(S, w.att_nch));
  a.segb = (wb + S - 1) / S;
  S = (wb + a.segb - 1) / a.segb;
  a.lens = lens;
  a.pm = w.att_m;
  a.pl = w.att_l;
  a.po = w.att_o;
  a.cnt = w.att_cnt;
  a.af_o = w.af_o;
  if (kv.fmt == 1)
    k_attn_split_q4<<<dim3(S, NH, B), 256, 0, st>>>(a);
  else
    k_attn_split<<<dim3(S, NH, B), 256, 0, st>>>(a);
}

// x += sum of partials; afrag of RMSNorm(x; gain). spine_rows: write row
// 4b+j (j < 3) as row 3b+j (the spine's input rows), else every row.
__global__ __launch_bounds__(320) void k_resid_norm(float* x, const float* part, int splits, int R,
                                                    const float* gain, float eps, uint16_t* af,
                                                    int spine_rows) {
  __shared__ float red[8];
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  float* xr = x + (size_t)r * H + c0;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  add_splits8(part + (size_t)r * H + c0, (size_t)R * H, splits, v);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = xr[i] + v[i];
    xr[i] = v[i];
    ss += v[i] * v[i];
  }
  ss = block_sum<5>(ss, red);
  const float inv = 1.0f / sqrtf(ss / H + eps);
  int orow = r;
  if (spine_rows) {
    if ((r & 3) == 3) return;
    orow = (r >> 2) * 3 + (r & 3);
  }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = gain[c0 + i] * v[i] * inv;
  store_afrag8(af, H / 32, orow, c0, o);
}

void launch_resid_norm(hipStream_t st, const Work& w, int R, int splits, const float* gain,
                       float eps, uint16_t* af_out, int spine_rows) {
  k_resid_norm<<<R, 320, 0, st>>>(w.x, w.part, splits, R, gain, eps, af_out, spine_rows);
}

// h = silu(gate) * up from the gate|up partials -> afrag.
__global__ __launch_bounds__(256) void k_swiglu(const float* part, int splits, int R,
                                                uint16_t* af) {
  const int r = blockIdx.x;
  for (int gidx = threadIdx.x; gidx < FF / 8; gidx += blockDim.x) {
    const int c0 = gidx * 8;
    float gt[8], up[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gt[i] = up[i] = 0.f;
    // columns c0..c0+7 of gate and of up sit in one 16-row tile (gu_position)
    const float* p = part + (size_t)r * GU + gu_position(c0);
    add_splits8(p, (size_t)R * GU, splits, gt);
    add_splits8(p + 8, (size_t)R * GU, splits, up);
    float hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[i] = silu(gt[i]) * up[i];
    store_afrag8(af, FF / 32, r, c0, hv);
  }
}

void launch_swiglu(hipStream_t st, const Work& w, int R, int splits) {
  k_swiglu<<<R, 256, 0, st>>>(w.part, splits, R, w.af_h);
}

// ---------------------------------------------------------------------------
// NVFP4 head over the draft vocabulary with a fused per-row argmax.
// logits[r][v] = g * sum_k z[r][k] * e2m1(q) * e4m3(s); the argmax key
// (order-preserving logit bits, then the complement of the index) is reduced
// across lanes and merged with a 64-bit atomicMax, which is independent of
// scheduling: ties go to the lowest draft index.
// ---------------------------------------------------------------------------
constexpr int HEAD_NV = 4;  // vocab tiles per wave

struct HeadK {
  const uint16_t* af;
  int R;
  const uint8_t* hq;
  const uint8_t* hs;
  float g;
  int VD, VT;
  float* logits;
  unsigned long long* keys;
};

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

__global__ __launch_bounds__(256) void k_head(HeadK a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vt0 = (blockIdx.x * 4 + wave) * HEAD_NV;
  if (vt0 >= a.VT) return;
  constexpr int KT = H / 32, KG = H / 128;
  const f16x8 zero = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
  const int MT = mtiles(a.R);
  for (int mt = 0; mt < MT; ++mt) {
    f32x4 acc[HEAD_NV];
#pragma unroll
    for (int v = 0; v < HEAD_NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool rv = mt * 16 + (lane & 15) < a.R;
    for (int kg = 0; kg < KG; ++kg) {
      u32x4 qv[HEAD_NV];
      uint32_t sv[HEAD_NV];
#pragma unroll
      for (int v = 0; v < HEAD_NV; ++v) {
        const int vt = vt0 + v;
        if (vt < a.VT) {
          const size_t idx = ((size_t)vt * KG + kg) * 64 + lane;
          qv[v] = *reinterpret_cast<const u32x4*>(a.hq + idx * 16);
          sv[v] = *reinterpret_cast<const uint32_t*>(a.hs + idx * 4);
        } else {
          qv[v] = u32x4{0u, 0u, 0u, 0u};
          sv[v] = 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = kg * 4 + i;
        f16x8 av = zero;
        if (rv) av = *reinterpret_cast<const f16x8*>(a.af + (size_t)(mt * KT + t) * 512 + lane * 8);
#pragma unroll
        for (int v = 0; v < HEAD_NV; ++v)
          acc[v] = mfma_f16(av, nvfp4x8_f16(qv[v][i], (sv[v] >> (8 * i)) & 0xffu), acc[v]);
      }
    }
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int v = 0; v < HEAD_NV; ++v) {
      const int voc = (vt0 + v) * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = mt * 16 + 4 * (lane >> 4) + e;
        const float val = acc[v][e] * a.g;
        if (r < a.R && voc < a.VD) {
          if (a.logits) a.logits[(size_t)r * a.VD + voc] = val;
          const unsigned long long key = argmax_key(val, (uint32_t)voc);
          best[e] = key > best[e] ? key : best[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) {
        const unsigned long long o = shfl_xor_u64(best[e], m);
        best[e] = o > best[e] ? o : best[e];
      }
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = mt * 16 + 4 * (lane >> 4) + e;
        if (r < a.R && best[e]) atomicMax(&a.keys[r], best[e]);
      }
    }
  }
}

void launch_head(hipStream_t st, const Work& w, const DevWeights& d, int R, float* logits) {
  if (head_mm_fits(R) || d.head_fmt != 0) return launch_head_mm(st, w.af_x, R, d, logits, w.keys);
  HeadK a;
  a.af = w.af_x;
  a.R = R;
  a.hq = d.hq;
  a.hs = d.hs;
  a.g = d.hg;
  a.VD = d.VD;
  a.VT = d.VT;
  a.logits = logits;
  a.keys = w.keys;
  const int waves = (d.VT + HEAD_NV - 1) / HEAD_NV;
  k_head<<<(waves + 3) / 4, 256, 0, st>>>(a);
}

__global__ void k_finalize(const unsigned long long* keys, const int32_t* vocab, int R,
                           int32_t* out, const int32_t* anchor, const int32_t* pred,
                           int pred_stride, int V, unsigned* range_word) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r == 0) flush_f16_range(range_word);   // the round's (and earlier ingests') f16 stores are done
  if (r >= R) return;
  const unsigned long long k = keys[r];
  const bool ok = id_row_valid(anchor, pred, pred_stride, r / BLK, r % BLK, V);
  out[r] = k && ok ? vocab[0xffffffffu - (uint32_t)(k & 0xffffffffu)] : -1;
}

void launch_finalize(hipStream_t st, const Work& w, const DevWeights& d, int R, int32_t* out_ids,
                     const int32_t* anchor, const int32_t* pred, int pred_stride, unsigned* range_word) {
  k_finalize<<<(R + 255) / 256, 256, 0, st>>>(w.keys, d.vocab, R, out_ids, anchor, pred, pred_stride,
                                               d.V, range_word);
}

// ---------------------------------------------------------------------------
// Context ingest: new rows -> fuse -> fc -> per layer RMSNorm -> K, V -> RoPE(K)
// -> bf16 into the ring at slot (len + i) % capacity; then len += n.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ingest_prep(uint16_t* af_in, const uint16_t* taps) {
  const int r = blockIdx.x;
  constexpr int K = NTAP * H, KT = K / 32;
  for (int g = threadIdx.x; g < K / 8; g += blockDim.x) {
    u32x4 bits = *reinterpret_cast<const u32x4*>(taps + (size_t)r * K + g * 8);
    store_afrag8_bf16(af_in, KT, r, g * 8, bits);
  }
}

void launch_ingest_prep(hipStream_t st, const Work& w, int rows, const uint16_t* taps) {
  k_ingest_prep<<<rows, 256, 0, st>>>(w.af_in, taps);
}

__global__ __launch_bounds__(320) void k_ingest_post_fuse(const float* part, int splits, int rows,
                                                          uint16_t* af_fc, const uint16_t* table,
                                                          const uint16_t* zrow, int V,
                                                          const int32_t* next_ids) {
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  constexpr int KT = 2 * H / 32;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  add_splits8(part + (size_t)r * H + c0, (size_t)rows * H, splits, v);
  store_afrag8(af_fc, KT, r, c0, v);
  const u32x4 e = *reinterpret_cast<const u32x4*>(table_row(table, zrow, next_ids[r], V, H) + c0);
  store_afrag8_bf16(af_fc, KT, r, H + c0, e);
}

void launch_ingest_post_fuse(hipStream_t st, const Work& w, const DevWeights& d, int rows,
                             int splits, const int32_t* next_ids) {
  k_ingest_post_fuse<<<rows, 320, 0, st>>>(w.part, splits, rows, w.af_fc, d.table, d.zrow, d.V, next_ids);
}

__global__ __launch_bounds__(320) void k_ingest_c(const float* part, int splits, int rows,
                                                  float* c) {
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  add_splits8(part + (size_t)r * H + c0, (size_t)rows * H, splits, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) c[(size_t)r * H + c0 + i] = v[i];
}

void launch_ingest_c(hipStream_t st, const Work& w, int rows, int splits) {
  k_ingest_c<<<rows, 320, 0, st>>>(w.part, splits, rows, w.c);
}

__global__ __launch_bounds__(320) void k_norm_rows(const float* x, const float* gain, float eps,
                                                   uint16_t* af) {
  __shared__ float red[8];
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  float v[8], ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = x[(size_t)r * H + c0 + i];
    ss += v[i] * v[i];
  }
  ss = block_sum<5>(ss, red);
  const float inv = 1.0f / sqrtf(ss / H + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = gain[c0 + i] * v[i] * inv;
  store_afrag8(af, H / 32, r, c0, v);
}

void launch_norm_rows(hipStream_t st, const float* x, int rows, const float* gain, float eps,
                      uint16_t* af) {
  k_norm_rows<<<rows, 320, 0, st>>>(x, gain, eps, af);
}

// One row's RMS, then the row with every layer's attention gain (afrag).
__global__ __launch_bounds__(320) void k_norm_rows_layers(const float* x, DevWeights d, float eps,
                                                          uint16_t* af, size_t af_layer) {
  __shared__ float red[8];
  const int r = blockIdx.x, c0 = threadIdx.x * 8;
  float v[8], ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = x[(size_t)r * H + c0 + i];
    ss += v[i] * v[i];
  }
  ss = block_sum<5>(ss, red);
  const float inv = 1.0f / sqrtf(ss / H + eps);
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const float* gain = d.layer[l].attn_norm;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = gain[c0 + i] * v[i] * inv;
    store_afrag8(af + l * af_layer, H / 32, r, c0, y);
  }
}

void launch_norm_rows_layers(hipStream_t st, const float* x, int rows, const DevWeights& d,
                             float eps, uint16_t* af, size_t af_layer) {
  k_norm_rows_layers<<<rows, 320, 0, st>>>(x, d, eps, af, af_layer);
}

// k|v partials (N = 2H) -> RoPE(k) at position len + i -> bf16 (nearest even)
// into the ring.
__global__ __launch_bounds__(256) void k_ingest_store(const float* part, int splits, int rows,
                                                      int n_new, uint16_t* kc, uint16_t* vc,
                                                      int64_t ss, int64_t sh, int64_t sl, int cap,
                                                      const int32_t* lens, float theta) {
  const int r = blockIdx.x, b = r / n_new, i = r % n_new;
  const long pos = (long)lens[b] + i;
  if (pos < 0) return;   // a negative length stores nothing
  const int slot = (int)(pos % cap);
  for (int p = threadIdx.x; p < NH * DH / 2; p += blockDim.x) {
    const int h = p >> 6, fi = p & 63;
    const int c0 = h * DH + fi, c1 = c0 + DH / 2;
    float ka = 0.f, kb2 = 0.f, va = 0.f, vb2 = 0.f;
    // this launch covers q|k|v positions H..3H-1 (the k and v sections)
    const int pk0 = qkv_position(H + c0) - H, pk1 = qkv_position(H + c1) - H;
    const int pv0 = qkv_position(2 * H + c0) - H, pv1 = qkv_position(2 * H + c1) - H;
    for (int s = 0; s < splits; ++s) {
      const float* pr = part + ((size_t)s * rows + r) * (2 * H);
      ka += pr[pk0];
      kb2 += pr[pk1];
      va += pr[pv0];
      vb2 += pr[pv1];
    }
    const double ang = (double)pos * pow((double)theta, -(double)fi / (DH / 2));
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    const size_t base = (size_t)b * ss + (size_t)h * sh + (size_t)slot * sl;
    kc[base + fi] = (uint16_t)bf16_rne(ka * cs - kb2 * sn);
    kc[base + fi + DH / 2] = (uint16_t)bf16_rne(ka * sn + kb2 * cs);
    vc[base + fi] = (uint16_t)bf16_rne(va);
    vc[base + fi + DH / 2] = (uint16_t)bf16_rne(vb2);
  }
}


// The same rows for the rotated 4-bit cache (the article "Serving Kolibri-1
// with a 4-bit KV cache", section What we do): wave w takes heads w, w + 4,
// ...; lane l holds dims l and l + 64 (the RoPE pair). K after RoPE is turned
// by R = H diag(s)/sqrt(128); K and V rows then get scale = fp16((max -
// min)/15), offset = fp16(min) and codes clamp(rne((x - offset)/scale), 0,
// 15) (0 for a zero scale).
__global__ __launch_bounds__(256) void k_ingest_store_q4(const float* part, int splits, int rows,
                                                         int n_new, uint8_t* kc, uint8_t* vc,
                                                         uint32_t* kso, uint32_t* vso,
                                                         int64_t ss, int64_t sh, int64_t sl,
                                                         int cap, const int32_t* lens,
                                                         float theta, const float* signs) {
  const int r = blockIdx.x, b = r / n_new, i = r % n_new;
  const long pos = (long)lens[b] + i;
  if (pos < 0) return;   // a negative length stores nothing
  const int slot = (int)(pos % cap);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fi = lane;
  const double ang = (double)pos * pow((double)theta, -(double)fi / (DH / 2));
  const float cs = (float)cos(ang), sn = (float)sin(ang);
  const float s0 = signs[fi], s1 = signs[fi + DH / 2];
  for (int h = wave; h < NH; h += 4) {
    const int c0 = h * DH + fi, c1 = c0 + DH / 2;
    float ka = 0.f, kb2 = 0.f, va = 0.f, vb2 = 0.f;
    const int pk0 = qkv_position(H + c0) - H, pk1 = qkv_position(H + c1) - H;
    const int pv0 = qkv_position(2 * H + c0) - H, pv1 = qkv_position(2 * H + c1) - H;
    for (int s = 0; s < splits; ++s) {
      const float* pr = part + ((size_t)s * rows + r) * (2 * H);
      ka += pr[pk0];
      kb2 += pr[pk1];
      va += pr[pv0];
      vb2 += pr[pv1];
    }
    float y0 = (ka * cs - kb2 * sn) * s0, y1 = (ka * sn + kb2 * cs) * s1;
    fwht128(y0, y1, lane);
    y0 *= 0.08838834764831845f;
    y1 *= 0.08838834764831845f;
    const size_t row = (size_t)b * ss + (size_t)h * sh + (size_t)slot * sl;
    store_row_q4(y0, y1, lane, kc + row * 64, kso + row);
    store_row_q4(va, vb2, lane, vc + row * 64, vso + row);
  }
}

void launch_ingest_store(hipStream_t st, const Work& w, const DevWeights& d, int B, int n_new,
                         int splits, const KV& kv, int layer, const int32_t* lens, float theta) {
  if (kv.fmt == 1) {
    k_ingest_store_q4<<<B * n_new, 256, 0, st>>>(
        w.part, splits, B * n_new, n_new,
        reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(kv.k[layer])),
        reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(kv.v[layer])),
        reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(kv.kso[layer])),
        reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(kv.vso[layer])), kv.ss, kv.sh, kv.sl,
        kv.cap, lens, theta, d.kv_signs + layer * DH);
    return;
  }
  k_ingest_store<<<B * n_new, 256, 0, st>>>(w.part, splits, B * n_new, n_new,
                                            const_cast<uint16_t*>(kv.k[layer]),
                                            const_cast<uint16_t*>(kv.v[layer]), kv.ss, kv.sh,
                                            kv.sl, kv.cap, lens, theta);
}

__global__ void k_bump_lens(int32_t* lens, int B, int n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) lens[b] += n;
}

void launch_bump_lens(hipStream_t st, int32_t* lens, int B, int n) {
  k_bump_lens<<<(B + 255) / 256, 256, 0, st>>>(lens, B, n);
}

// ---------------------------------------------------------------------------
// Codec probes: the exact decoders the projection and head kernels use.
// ---------------------------------------------------------------------------
__global__ void k_probe_e4m3(uint16_t* out) {
  const uint32_t c = threadIdx.x;
  const bf16x8 v = e4m3x8_bf16(c, 0u);
  out[c] = (uint16_t)(__builtin_bit_cast(u32x4, v).x & 0xffffu);
}

__global__ void k_probe_e4m3_f16(uint16_t* out) {
  const uint32_t c = threadIdx.x;
  const f16x8 v = e4m3x8_f16(c, 0u);
  out[c] = (uint16_t)(__builtin_bit_cast(u32x4, v).x & 0xffffu);
}

__global__ void k_probe_nvfp4(uint16_t* out) {
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t s = idx >> 4, c = idx & 15u;
  const f16x8 v = nvfp4x8_f16(c, s);
  out[idx] = (uint16_t)(__builtin_bit_cast(u32x4, v).x & 0xffffu);
}

void launch_probe_e4m3(hipStream_t st, uint16_t* out) { k_probe_e4m3<<<1, 256, 0, st>>>(out); }
void launch_probe_e4m3_f16(hipStream_t st, uint16_t* out) { k_probe_e4m3_f16<<<1, 256, 0, st>>>(out); }
void launch_probe_nvfp4(hipStream_t st, uint16_t* out) { k_probe_nvfp4<<<16, 256, 0, st>>>(out); }

}  // namespace kd
