// Projections and the restricted head for many block rows (more than 32):
// matrix-core tiles in which a workgroup's four waves share one activation
// tile through LDS (model card "Kolibri-1 block drafter", section Architecture:
// the body's block-FP8 projections and the NVFP4 head over the draft
// vocabulary, served as one batched pass over every stream's block rows).
//
// A workgroup owns 64 rows (four 16-row tiles) and 256 output columns; wave w
// computes columns 64w .. 64w+63 for all 64 rows. Per step, the activation
// rows of the step's inputs (f16 fragments) are loaded once per workgroup
// (each wave stages one row tile) and written to LDS; the weights are read by
// the wave that uses them and decoded exactly to f16 in registers. Steps are double-buffered: the next step's
// loads are in flight while the current step runs on the matrix cores.
//
// Workgroups are laid out per XCD: workgroup i runs on XCD i % 8 (the
// dispatcher deals workgroups to the XCDs in turn), and all row blocks of one
// output-column block run on the same XCD, so that the column block's weights
// are fetched into that XCD's L2 once and reused by its row blocks.
#include <algorithm>

#include "kd_device.h"
#include "kd_runtime.h"

namespace kd {

constexpr int MM_RT = 4;                          // 16-row tiles per workgroup
constexpr int MM_WAVES = 4;
// 4 column tiles per wave (256 columns per workgroup) once the
// rows make the work matrix-core bound; 1 (64 columns) for fewer rows, where
// the weights stream from HBM and narrower tiles give more workgroups with
// fewer split-K partial sums.
constexpr int MM_SMALL_R = 256;
__host__ __device__ inline int mm_ct(int R) { return R > MM_SMALL_R ? 4 : 1; }

// Workgroup -> (row block, column block, split). Column unit c = (column
// block, split) runs on XCD c % 8; its row blocks are consecutive slots there.
struct MmMap {
  int rb, cb, sp;
  bool ok;
};
__device__ __forceinline__ MmMap mm_map(int RB, int CB, int S) {
  const int id = blockIdx.x, x = id & 7, slot = id >> 3;
  const int k = slot / RB, rb = slot - k * RB;
  const int c = x + 8 * k;
  MmMap m;
  m.ok = c < CB * S;
  m.rb = rb;
  m.sp = c / CB;
  m.cb = c - m.sp * CB;
  return m;
}
static int mm_grid(int R, int CB, int S) {
  const int RB = (R + 63) / 64, units = CB * S;
  return 8 * RB * ((units + 7) / 8);
}

// ---------------------------------------------------------------------------
// Projection: part[split][r][n] = sum over the split's inputs of
// X[r][k] * W[n_off*16 + n][k], W in one of the body formats (WF); one step
// is one 64-input block (a block-FP8 block's fp32 scale multiplies its
// partial sum, as the scale is defined per row and 64 inputs; an NVFP4
// block's partial sum is multiplied by its column's tensor scale).
// ---------------------------------------------------------------------------
struct GemmMM {
  const uint16_t* af;   // afrag of X: [mtiles(R)][KT][512] f16
  int R, KT;
  const uint8_t* w;     // repacked weights (layout per format in kd_device.h)
  const float* s;       // FP8 scales [N/16][KB][16]; NVFP4 tensor scales [2][WN]
  const uint8_t* s4;    // NVFP4 block-scale codes
  int KB;
  int N, n_off;         // output columns (a multiple of the workgroup's), first weight tile
  int WN, ks;           // NVFP4: rows of the matrix, first block of its second tensor scale
  float* part;
  int splits, kbs;
};

// The projection's main loop for one (row block rb, column block cb, split
// sp): acc[r][c] = sum over the split's 64-input steps of the row tile r x
// column tile c products (each block-FP8 or NVFP4 step's partial sum times
// its scale). sa: the workgroup's double-buffered activation tile in LDS.
// KS = 2: the workgroup has two groups of four waves, group q taking the
// q-th half of the split's steps with its own activation buffers (sa + 2q);
// each group's sums are its own (the caller adds them).
template <int CT, int D, int WF, int KS = 1>
__device__ __forceinline__ void mm_accumulate(const GemmMM& g, int rb, int cb, int sp,
                                              f32x4 (&acc)[MM_RT][CT], u32x4 (*sa_all)[MM_RT * 2][64]) {
  constexpr int COLS = 16 * CT * MM_WAVES;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & (MM_WAVES - 1);
  const int grp = KS == 1 ? 0 : (int)(threadIdx.x >> 8);
  u32x4 (*sa)[MM_RT * 2][64] = sa_all + 2 * grp;
  const int MT = mtiles(g.R);
  const int nb = g.kbs / KS, b0 = sp * g.kbs + grp * nb;
  // wave w stages row tile rb*4 + w (clamped: a tile past the last repeats it,
  // and its output rows are past R and discarded)
  const int mt_ld = min(rb * MM_RT + wave, MT - 1);
  const uint16_t* ap = g.af + ((size_t)mt_ld * g.KT + 2 * b0) * 512 + lane * 8;
  const int nt0 = g.n_off + cb * (COLS / 16) + wave * CT;
  const float* spp = g.s + ((size_t)nt0 * g.KB + b0) * 16 + (lane & 15);
  const size_t st_stride = (size_t)g.KB * 16;
  float gt[CT][2];   // NVFP4: the columns' tensor scales before / from the split block
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    gt[c][0] = gt[c][1] = 1.f;
    if constexpr (WF == WF_NVFP4) {
      gt[c][0] = g.s[(nt0 + c) * 16 + (lane & 15)];
      gt[c][1] = g.s[g.WN + (nt0 + c) * 16 + (lane & 15)];
    }
  }

#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A register ring of D steps: slot d holds the activation fragments (bound
  // for LDS) and the weights of the steps s with s % D == d. Step s's weights
  // are decoded, the slot is refilled with step s + D, and step s runs on the
  // matrix cores while D - 1 later steps are in flight. Loads past the last
  // step re-load it (unconditional loads keep the compiler from waiting for
  // them at a join).
  u32x4 ar[D][2];
  WBlock<WF> wr[D][CT];
  float sr[D][CT];
  auto load = [&](int st, int d) __attribute__((always_inline)) {
    const int sc = min(st, nb - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) ar[d][j] = *reinterpret_cast<const u32x4*>(ap + (size_t)sc * 1024 + j * 512);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      wr[d][c] = load_wblock<WF>(g.w, g.s4, g.KB, nt0 + c, b0 + sc, lane);
      if constexpr (WF == WF_FP8) sr[d][c] = spp[c * st_stride + (size_t)sc * 16];
      if constexpr (WF == WF_NVFP4) sr[d][c] = b0 + sc < g.ks ? gt[c][0] : gt[c][1];
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
#pragma unroll
  for (int j = 0; j < 2; ++j) sa[0][wave * 2 + j][lane] = ar[0][j];
  __syncthreads();

  for (int i0 = 0; i0 < nb; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      if (i < nb) {
        WBlock<WF> wv[CT];
        float sc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          wv[c] = wr[d][c];
          sc[c] = sr[d][c];
        }
        // the slot's activations went to LDS a step ago: refill it
        load(i + D, d);
        const int buf = i & 1;
#pragma unroll
        for (int r = 0; r < MM_RT; ++r) {
          const f16x8 a0 = __builtin_bit_cast(f16x8, sa[buf][r * 2 + 0][lane]);
          const f16x8 a1 = __builtin_bit_cast(f16x8, sa[buf][r * 2 + 1][lane]);
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            const f32x4 t = wv[c].mul(a0, a1);
            if constexpr (WF == WF_BF16) acc[r][c] += t;
            else acc[r][c] += sc[c] * t;
          }
        }
        // wide tiles store unconditionally (after the last step, an unused
        // re-loaded copy of it): with no branch in the step, the compiler
        // interleaves the scale multiply-adds with the matrix-core work
        if (CT == 4 || i + 1 < nb) {
          const int dn = d + 1 == D ? 0 : d + 1;
#pragma unroll
          for (int j = 0; j < 2; ++j) sa[buf ^ 1][wave * 2 + j][lane] = ar[dn][j];
        }
        __syncthreads();
      }
    }
  }
}

// KS = 2 (at most 64 rows): 8 waves, the split's inputs in two halves, the
// second group's sums added to the first's through LDS before the store.
template <int CT, int D, int WF, int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_mm(GemmMM g) {
  constexpr int COLS = 16 * CT * MM_WAVES;
  // [group][buffer][row tile][k tile t, t+1][lane]
  __shared__ __attribute__((aligned(16))) u32x4 sa[2 * KS][MM_RT * 2][64];
  const int RB = (g.R + 63) / 64, CB = g.N / COLS;
  const MmMap m = mm_map(RB, CB, g.splits);
  if (!m.ok) return;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & (MM_WAVES - 1);
  f32x4 acc[MM_RT][CT];
  mm_accumulate<CT, D, WF, KS>(g, m.rb, m.cb, m.sp, acc, sa);   // ends at a barrier: LDS is free
  if constexpr (KS == 2) {
    static_assert(sizeof(sa) >= MM_WAVES * MM_RT * CT * 64 * sizeof(f32x4), "staging area");
    f32x4* T = reinterpret_cast<f32x4*>(&sa[0][0][0]);
    auto tix = [&](int r, int c) { return ((wave * MM_RT + r) * CT + c) * 64 + lane; };
    if (threadIdx.x >= 256) {
#pragma unroll
      for (int r = 0; r < MM_RT; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) T[tix(r, c)] = acc[r][c];
    }
    __syncthreads();
    if (threadIdx.x >= 256) return;
#pragma unroll
    for (int r = 0; r < MM_RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[r][c] += T[tix(r, c)];
  }

  float* out = g.part + (size_t)m.sp * g.R * g.N;
#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int col = (m.cb * (COLS / 16) + wave * CT + c) * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = (m.rb * MM_RT + r) * 16 + 4 * (lane >> 4) + e;
        if (row < g.R) out[(size_t)row * g.N + col] = acc[r][c][e];
      }
    }
}

// Up to 64 rows the workgroups have 8 waves (the split's inputs in two
// halves), so half as many splits keep the same waves in flight with half the
// partial sums.
static bool mm_halves(int R) { return R <= 64; }

int gemm_mm_splits(int K, int N, int R) {
  const int KB = K / 64;
  const int wgs = ((R + 63) / 64) * (N / (64 * mm_ct(R)));
  const int per_cu = mm_halves(R) ? 256 : 512;   // about two workgroups (of 4 or 8 waves) per CU
  int want = (per_cu + wgs - 1) / wgs;
  want = std::min(want, std::max(KB / 4, 1));  // at least 4 blocks per split
  int s = std::max(want, 1);
  while (s > 1 && (KB % s || (mm_halves(R) && (KB / s) % 2))) --s;
  return s;
}

bool gemm_mm_fits(int R, int N) { return R > 32 && N % (64 * mm_ct(R)) == 0; }

void launch_gemm_mm(hipStream_t st, const uint16_t* af, int R, const WMat& W, int n_off_tiles,
                    int N, float* part, int splits) {
  GemmMM g;
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
  const bool wide = mm_ct(R) == 4;
  const bool halves = !wide && mm_halves(R) && g.kbs % 2 == 0;
  const dim3 grid(mm_grid(R, N / (wide ? 256 : 64), splits));
  switch (W.fmt) {
    case WF_NVFP4:
      if (wide) k_gemm_mm<4, 2, WF_NVFP4, 1><<<grid, 256, 0, st>>>(g);
      else if (halves) k_gemm_mm<1, 4, WF_NVFP4, 2><<<grid, 512, 0, st>>>(g);
      else k_gemm_mm<1, 4, WF_NVFP4, 1><<<grid, 256, 0, st>>>(g);
      break;
    case WF_BF16:
      if (wide) k_gemm_mm<4, 2, WF_BF16, 1><<<grid, 256, 0, st>>>(g);
      else if (halves) k_gemm_mm<1, 4, WF_BF16, 2><<<grid, 512, 0, st>>>(g);
      else k_gemm_mm<1, 4, WF_BF16, 1><<<grid, 256, 0, st>>>(g);
      break;
    default:
      if (wide) k_gemm_mm<4, 2, WF_FP8, 1><<<grid, 256, 0, st>>>(g);
      else if (halves) k_gemm_mm<1, 4, WF_FP8, 2><<<grid, 512, 0, st>>>(g);
      else k_gemm_mm<1, 4, WF_FP8, 1><<<grid, 256, 0, st>>>(g);
  }
}

// ---------------------------------------------------------------------------
// Projections with their epilogue fused (model card "Kolibri-1 block
// drafter", section Architecture: Body; every stream's block rows in one
// batched pass): q|k|v followed by RoPE on q and k, and gate|up followed by
// SwiGLU. The main loop is k_gemm_mm's over the whole input range (one split,
// so no partial sums leave the workgroup); the workgroup stages its output
// tile in LDS and applies the epilogue per 16-column tile, which holds the
// RoPE partners (d, d + 64) or a gate row block and its up rows.
// ---------------------------------------------------------------------------
// KS = 2 (used for at most 64 rows, where the 64-column tiles leave the
// grid small and each wave's chain of steps long): 8 waves, the input range
// split between two groups of four, the second group's sums added to the
// first's in LDS before the epilogue.
template <int CT, int D, int WF, int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2))) void k_proj(GemmMM g, ProjEpi e) {
  constexpr int COLS = 16 * CT * MM_WAVES;
  constexpr int TP = COLS + 4;                        // LDS row pitch of the staged tile (floats)
  constexpr int SA_BYTES = KS * 2 * MM_RT * 2 * 64 * 16;
  constexpr int T_BYTES = KS * 64 * TP * 4;           // one staged tile per group
  __shared__ __attribute__((aligned(16))) unsigned char lds[SA_BYTES > T_BYTES ? SA_BYTES : T_BYTES];
  auto sa = reinterpret_cast<u32x4(*)[MM_RT * 2][64]>(lds);
  float* T = reinterpret_cast<float*>(lds);
  const int RB = (g.R + 63) / 64, CB = g.N / COLS;
  const MmMap m = mm_map(RB, CB, 1);
  if (!m.ok) return;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & (MM_WAVES - 1);
  const int grp = threadIdx.x >> 8;
  f32x4 acc[MM_RT][CT];
  mm_accumulate<CT, D, WF, KS>(g, m.rb, m.cb, 0, acc, sa);   // ends at a barrier: LDS is free
  auto tix = [&](int r, int c, int q) { return (r * 16 + 4 * (lane >> 4) + q) * TP + (wave * CT + c) * 16 + (lane & 15); };
  // group q > 0 stages its sums at T + q * 64 * TP; group 0 adds them in group
  // order and stages the total at T
  if (KS == 1 || grp > 0) {
    float* Tg = T + (size_t)grp * 64 * TP;
#pragma unroll
    for (int r = 0; r < MM_RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) Tg[tix(r, c, q)] = acc[r][c][q];
  }
  __syncthreads();
  if (KS > 1 && grp == 0) {
#pragma unroll
    for (int r = 0; r < MM_RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = acc[r][c][q];
#pragma unroll
          for (int k = 1; k < KS; ++k) v += T[k * 64 * TP + tix(r, c, q)];
          T[tix(r, c, q)] = v;
        }
  }
  if (KS > 1) __syncthreads();
  // items: (row, 16-column tile)
  constexpr int NT = COLS / 16;
  for (int it = threadIdx.x; it < 64 * NT; it += 256 * KS) {
    const int rl = it / NT, ti = it - rl * NT, row = m.rb * 64 + rl;
    if (row >= g.R) continue;
    const float* tp = T + rl * TP + ti * 16;
    const int tg = m.cb * NT + ti;
    if (e.kind == PE_SWIGLU) {
      float h[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) h[n] = silu(tp[n]) * tp[8 + n];
      store_afrag8(e.af, FF / 32, row, 8 * tg, h);
    } else {
      const int nat = qkv_natural(tg * 16), sec = nat / H, c = nat - sec * H;
      float* dst = (sec == 0 ? e.q : sec == 1 ? e.kb : e.vb) + (size_t)row * H + c;
      const float* rp = e.rope + ((size_t)((row >> 2) * BLK + (row & 3)) * (DH / 2) + c % DH) * 2;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float a = tp[n], b = tp[8 + n];
        if (sec < 2) {
          const float cs = rp[2 * n], sn = rp[2 * n + 1];
          dst[n] = a * cs - b * sn;
          dst[n + DH / 2] = a * sn + b * cs;
        } else {
          dst[n] = a;
          dst[n + DH / 2] = b;
        }
      }
    }
  }
}

void launch_proj(hipStream_t st, const uint16_t* af, int R, const WMat& W, const ProjEpi& e) {
  GemmMM g;
  g.af = af;
  g.R = R;
  g.KT = W.K / 32;
  g.w = W.w;
  g.s = W.s;
  g.s4 = W.s4;
  g.KB = W.K / 64;
  g.N = W.N;
  g.n_off = 0;
  g.WN = W.N;
  g.ks = W.ks;
  g.part = nullptr;
  g.splits = 1;
  g.kbs = g.KB;
  const bool wide = mm_ct(R) == 4;
  // at most one row block: the input range in two halves inside the workgroup
  const bool halves = !wide && mm_halves(R) && g.KB % 2 == 0;
  const dim3 grid(mm_grid(R, W.N / (wide ? 256 : 64), 1));
  switch (W.fmt) {
    case WF_NVFP4:
      if (wide) k_proj<4, 2, WF_NVFP4, 1><<<grid, 256, 0, st>>>(g, e);
      else if (halves) k_proj<1, 4, WF_NVFP4, 2><<<grid, 512, 0, st>>>(g, e);
      else k_proj<1, 4, WF_NVFP4, 1><<<grid, 256, 0, st>>>(g, e);
      break;
    case WF_BF16:
      if (wide) k_proj<4, 2, WF_BF16, 1><<<grid, 256, 0, st>>>(g, e);
      else if (halves) k_proj<1, 4, WF_BF16, 2><<<grid, 512, 0, st>>>(g, e);
      else k_proj<1, 4, WF_BF16, 1><<<grid, 256, 0, st>>>(g, e);
      break;
    default:
      if (wide) k_proj<4, 2, WF_FP8, 1><<<grid, 256, 0, st>>>(g, e);
      else if (halves) k_proj<1, 4, WF_FP8, 2><<<grid, 512, 0, st>>>(g, e);
      else k_proj<1, 4, WF_FP8, 1><<<grid, 256, 0, st>>>(g, e);
  }
}

// ---------------------------------------------------------------------------
// The ingest's k|v projections of every layer in one launch (model card
// "Kolibri-1 block drafter", section Architecture: Body, the cached K/V each
// layer attends to; every layer projects the same context row through its
// attention RMSNorm and W_k, W_v). Workgroup (column block, row block) of
// layer blockIdx.y: the main loop of k_proj over the layer's k|v rows of
// q|k|v (256 output columns, one split), the output tile staged in LDS. A
// 256-column block is two whole heads of k or of v (a head's RoPE pairs
// (d, d + 64) are one 16-column tile, its 8 tiles consecutive), so the
// epilogue finishes the rows there: RoPE on k at the row's absolute position
// (angle pos * theta^(-f/64), the frequency in double precision, the angle
// reduced in double precision, its sine and cosine in single precision),
// then either bf16 (nearest even) at the row's ring slot, or, for the
// rotated 4-bit cache (the article "Serving Kolibri-1 with a 4-bit KV
// cache", section What we do), k turned by the layer's R and both rows coded
// to 4 bits with their fp16 scale and offset.
// ---------------------------------------------------------------------------
struct IngestProj {
  GemmMM g[NL];
  IngestEpi e;
};

// N rows at once (independent lane-exchange chains interleave): the in-wave
// Walsh-Hadamard transform of fwht128 and the 4-bit coding of store_row_q4
// (rows with ok[i] false take part in the exchanges and store nothing).
template <int N>
__device__ __forceinline__ void fwht128_n(float (&y0)[N], float (&y1)[N], int lane) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float a = y0[i], c = y1[i];
    y0[i] = a + c;
    y1[i] = a - c;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float p0[N], p1[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      p0[i] = __shfl_xor(y0[i], m, 64);
      p1[i] = __shfl_xor(y1[i], m, 64);
    }
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      y0[i] = up ? p0[i] - y0[i] : y0[i] + p0[i];
      y1[i] = up ? p1[i] - y1[i] : y1[i] + p1[i];
    }
  }
}

template <int N>
__device__ __forceinline__ void store_rows_q4_n(const float (&x0)[N], const float (&x1)[N], const bool (&ok)[N],
                                                int lane, uint8_t* const (&codes)[N], uint32_t* const (&so)[N]) {
  float mn[N], mx[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    mn[i] = fminf(x0[i], x1[i]);
    mx[i] = fmaxf(x0[i], x1[i]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float pn[N], px[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      pn[i] = __shfl_xor(mn[i], m, 64);
      px[i] = __shfl_xor(mx[i], m, 64);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      mn[i] = fminf(mn[i], pn[i]);
      mx[i] = fmaxf(mx[i], px[i]);
    }
  }
  uint32_t c0[N], c1[N];
  _Float16 sc_h[N], of_h[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    sc_h[i] = f16_checked((mx[i] - mn[i]) / 15.0f);
    of_h[i] = f16_checked(mn[i]);
    const float sc = (float)sc_h[i], of = (float)of_h[i];
    auto code = [&](float x) -> uint32_t {
      if (!(sc > 0.f)) return 0u;
      const float c = __builtin_rintf((x - of) / sc);
      return (uint32_t)fminf(fmaxf(c, 0.f), 15.f);
    };
    c0[i] = code(x0[i]);
    c1[i] = code(x1[i]);
  }
  // dims (2m, 2m + 1) meet in the even lane
  uint32_t n0[N], n1[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    n0[i] = __shfl_xor(c0[i], 1, 64);
    n1[i] = __shfl_xor(c1[i], 1, 64);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (!ok[i]) continue;
    if ((lane & 1) == 0) {
      codes[i][lane >> 1] = (uint8_t)(c0[i] | (n0[i] << 4));
      codes[i][32 + (lane >> 1)] = (uint8_t)(c1[i] | (n1[i] << 4));
    }
    if (lane == 0)
      *so[i] = (uint32_t)__builtin_bit_cast(uint16_t, sc_h[i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, of_h[i]) << 16);
  }
}

template <int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_ingest_proj(IngestProj p) {
  constexpr int CT = 4, COLS = 256, TP = COLS + 4;
  constexpr int SA_BYTES = 2 * MM_RT * 2 * 64 * 16;
  constexpr int T_BYTES = 64 * TP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[SA_BYTES > T_BYTES ? SA_BYTES : T_BYTES];
  __shared__ double s_invf[DH / 2];
  auto sa = reinterpret_cast<u32x4(*)[MM_RT * 2][64]>(lds);
  float* T = reinterpret_cast<float*>(lds);
  const int l = blockIdx.y;
  GemmMM g = p.g[0];
#pragma unroll
  for (int i = 1; i < NL; ++i)
    if (l == i) g = p.g[i];
  const IngestEpi& e = p.e;
  const int RB = (g.R + 63) / 64, CB = g.N / COLS;
  const MmMap m = mm_map(RB, CB, 1);
  if (!m.ok) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < DH / 2) s_invf[threadIdx.x] = pow((double)e.theta, -(double)threadIdx.x / (DH / 2));
  f32x4 acc[MM_RT][CT];
  mm_accumulate<CT, 2, WF>(g, m.rb, m.cb, 0, acc, sa);   // ends at a barrier: LDS is free
#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        T[(r * 16 + 4 * (lane >> 4) + q) * TP + (wave * CT + c) * 16 + (lane & 15)] = acc[r][c][q];
  __syncthreads();
  // the block's first column in q|k|v order: section (1 = k, 2 = v) and head
  const int nat0 = qkv_natural((g.n_off + m.cb * (COLS / 16)) * 16);
  const int sec = nat0 / H, h0 = (nat0 - sec * H) / DH;
  const bool is_k = sec == 1;
  constexpr double TWO_PI = 6.283185307179586;
  auto angle = [&](long pos, int fi, float& cs, float& sn) {
    const double a = (double)pos * s_invf[fi];
    const float red = (float)(a - rint(a * (1.0 / TWO_PI)) * TWO_PI);
    sn = sinf(red);
    cs = cosf(red);
  };
  if (e.kv.fmt == 0) {
    // items (row, 8-dim group pg): dims 8 pg .. 8 pg + 7 and their partners
    // + 64 of both heads (tiles pg and 8 + pg), one angle per dim
    for (int it = threadIdx.x; it < 64 * 8; it += 256) {
      const int rl = it >> 3, pg = it & 7, row = m.rb * 64 + rl;
      if (row >= g.R) continue;
      const int b = row / e.n_new, i = row - b * e.n_new;
      const long pos = (long)e.lens[b] + i;
      if (pos < 0) continue;   // a negative length stores nothing
      const int slot = (int)(pos % e.kv.cap);
      float cs[8], sn[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        cs[n] = 1.f;
        sn[n] = 0.f;
        if (is_k) angle(pos, 8 * pg + n, cs[n], sn[n]);
      }
      uint16_t* cache = const_cast<uint16_t*>(is_k ? e.kv.k[l] : e.kv.v[l]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float* tp = T + rl * TP + (8 * hh + pg) * 16;
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int n = 0; n < 8; n += 2) {
          const float a0 = tp[n], b0 = tp[8 + n], a1 = tp[n + 1], b1 = tp[9 + n];
          lo[n / 2] = bf16_rne(a0 * cs[n] - b0 * sn[n]) | (bf16_rne(a1 * cs[n + 1] - b1 * sn[n + 1]) << 16);
          hi[n / 2] = bf16_rne(a0 * sn[n] + b0 * cs[n]) | (bf16_rne(a1 * sn[n + 1] + b1 * cs[n + 1]) << 16);
        }
        uint16_t* dst = cache + (size_t)b * e.kv.ss + (size_t)(h0 + hh) * e.kv.sh + (size_t)slot * e.kv.sl + 8 * pg;
        *reinterpret_cast<u32x4*>(dst) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<u32x4*>(dst + DH / 2) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      }
    }
  } else {
    // items (row, head): wave w takes items w, w + 4, ..., NI at a time; lane
    // l holds dims l and l + 64 (tile l / 8 of the head, columns l % 8 and
    // 8 + l % 8)
    constexpr int NI = 4;
    const float s0 = is_k ? e.signs[l * DH + lane] : 1.f, s1 = is_k ? e.signs[l * DH + lane + DH / 2] : 1.f;
    uint8_t* codes = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(is_k ? e.kv.k[l] : e.kv.v[l]));
    uint32_t* so = reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(is_k ? e.kv.kso[l] : e.kv.vso[l]));
    for (int it0 = wave; it0 < 64 * 2; it0 += 4 * NI) {
      float y0[NI], y1[NI];
      bool ok[NI];
      uint8_t* cp[NI];
      uint32_t* sp[NI];
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int it = it0 + 4 * n, rl = it >> 1, hh = it & 1, row = m.rb * 64 + rl;
        const int b = min(row, g.R - 1) / e.n_new, i = min(row, g.R - 1) - b * e.n_new;
        const long pos = (long)e.lens[b] + i;
        ok[n] = row < g.R && pos >= 0;   // a negative length stores nothing
        const int slot = (int)((pos < 0 ? 0 : pos) % e.kv.cap);
        const float* tp = T + rl * TP + (8 * hh + (lane >> 3)) * 16 + (lane & 7);
        y0[n] = tp[0];
        y1[n] = tp[8];
        if (is_k) {
          float cs, sn;
          angle(pos, lane, cs, sn);
          const float k0 = y0[n] * cs - y1[n] * sn, k1 = y0[n] * sn + y1[n] * cs;
          y0[n] = k0 * s0;
          y1[n] = k1 * s1;
        }
        const size_t crow = (size_t)b * e.kv.ss + (size_t)(h0 + hh) * e.kv.sh + (size_t)slot * e.kv.sl;
        cp[n] = codes + crow * 64;
        sp[n] = so + crow;
      }
      if (is_k) {
        fwht128_n<NI>(y0, y1, lane);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          y0[n] *= 0.08838834764831845f;
          y1[n] *= 0.08838834764831845f;
        }
      }
      store_rows_q4_n<NI>(y0, y1, ok, lane, cp, sp);
    }
  }
}

void launch_ingest_proj(hipStream_t st, const uint16_t* af, size_t af_layer, int R,
                        const DevWeights& d, const IngestEpi& e) {
  IngestProj p;
  for (int l = 0; l < NL; ++l) {
    const WMat& W = d.layer[l].qkv;
    GemmMM& g = p.g[l];
    g.af = af + l * af_layer;
    g.R = R;
    g.KT = W.K / 32;
    g.w = W.w;
    g.s = W.s;
    g.s4 = W.s4;
    g.KB = W.K / 64;
    g.N = 2 * H;          // the k and v sections of q|k|v
    g.n_off = H / 16;
    g.WN = W.N;
    g.ks = W.ks;
    g.part = nullptr;
    g.splits = 1;
    g.kbs = g.KB;
  }
  p.e = e;
  const dim3 grid(mm_grid(R, 2 * H / 256, 1), NL);
  switch (d.layer[0].qkv.fmt) {
    case WF_NVFP4: k_ingest_proj<WF_NVFP4><<<grid, 256, 0, st>>>(p); break;
    case WF_BF16: k_ingest_proj<WF_BF16><<<grid, 256, 0, st>>>(p); break;
    default: k_ingest_proj<WF_FP8><<<grid, 256, 0, st>>>(p);
  }
}

// ---------------------------------------------------------------------------
// NVFP4 head over the draft vocabulary with a fused per-row argmax:
// logits[r][v] = g * sum_k z[r][k] * e2m1(q) * e4m3(s). One step is one
// 128-input group (the repacked code layout's unit). The f16 activations
// multiply the exactly decoded f16 head values on the f16 matrix cores. Each
// row's best (logit, index)
// key over the workgroup's 256 vocabulary rows is merged with a 64-bit
// atomicMax: the result does not depend on scheduling, and ties go to the
// lowest draft index.
// ---------------------------------------------------------------------------
struct HeadMM {
  const uint16_t* af;   // afrag of z = RMSNorm(x; g_final): [mtiles(R)][H/32][512] f16
  int R;
  const uint8_t* hq;    // [VT][H/128][64][16] e2m1 codes
  const uint8_t* hs;    // [VT][H/128][64][4] e4m3 scale codes
  const uint16_t* hb;   // bf16 head instead: [VT][H/32][64][8]
  const uint8_t* fw;    // or a block-FP8 head: codes [VT][H/64][64][16]
  const float* fs;      //   and scales [VT][H/64][16]
  float g;
  int VD, VT;
  float* logits;        // [R][VD] or null
  unsigned long long* keys;
};

// HQ = 0: NVFP4 head (e2m1 x e4m3 decoded exactly to f16, f16 matrix
// cores). HQ = 1: bf16 head; each f16 activation is split exactly into two
// bf16 terms (hi = its top 8 significant bits, lo = the rest, at most 3
// bits) for the bf16 matrix cores. HQ = 2: block-FP8 head, e4m3 decoded
// exactly to f16, each 64-input block's product scaled by its row's scale.
template <int CT, int D, int HQ, int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(2))) void k_head_mm(HeadMM a) {
  // [group][buffer][row tile][k tiles 0..3][lane] f16
  __shared__ __attribute__((aligned(16))) u32x4 sa_all[2 * KS][MM_RT * 4][64];
  __shared__ unsigned long long best_s[MM_RT * 16];
  constexpr int KT = H / 32, KG = H / 128;
  // KS = 2 (at most 64 rows): two groups of four waves take the two halves of
  // the input groups; the second group's sums are added to the first's in
  // LDS and the first group runs the argmax
  constexpr int NK = KG / KS;
  static_assert(KG % KS == 0, "input groups per half");
  const int grp = KS == 1 ? 0 : (int)(threadIdx.x >> 8), kb0 = grp * NK;
  u32x4 (*sa)[MM_RT * 4][64] = sa_all + 2 * grp;
  const int RB = (a.R + 63) / 64, CB = (a.VT + 4 * CT - 1) / (4 * CT);
  const MmMap m = mm_map(RB, CB, 1);
  if (!m.ok) return;
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & (MM_WAVES - 1);
  const int MT = mtiles(a.R);
  if (threadIdx.x < MM_RT * 16) best_s[threadIdx.x] = 0ull;
  const int mt_ld = min(m.rb * MM_RT + wave, MT - 1);
  const uint16_t* ap = a.af + (size_t)mt_ld * KT * 512 + lane * 8;
  // vocab tiles of this wave (tiles past the last repeat it and are masked)
  const int vt0 = (m.cb * MM_WAVES + wave) * CT;
  const uint8_t* qp[CT];
  const uint8_t* sp[CT];
  const uint16_t* bp[CT];
  const float* fsp[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int vt = min(vt0 + c, a.VT - 1);
    if constexpr (HQ == 0) {
      qp[c] = a.hq + (size_t)vt * KG * 1024 + lane * 16;
      sp[c] = a.hs + (size_t)vt * KG * 256 + lane * 4;
    } else if constexpr (HQ == 1) {
      bp[c] = a.hb + (size_t)vt * KT * 512 + lane * 8;
    } else {
      qp[c] = a.fw + (size_t)vt * (H / 64) * 1024 + lane * 16;
      fsp[c] = a.fs + (size_t)vt * (H / 64) * 16 + (lane & 15);
    }
  }

  f32x4 acc[MM_RT][CT];
#pragma unroll
  for (int r = 0; r < MM_RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // register ring of D steps (128-input groups), as in k_gemm_mm
  constexpr int NQ = HQ == 0 ? 1 : (HQ == 1 ? 4 : 2);
  u32x4 ar[D][4], qr[D][CT][NQ];
  uint32_t sr[D][CT];
  float fr[D][CT][2];
  auto load = [&](int st, int d) __attribute__((always_inline)) {
    const size_t kc = (size_t)(kb0 + min(st, NK - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) ar[d][j] = *reinterpret_cast<const u32x4*>(ap + kc * 2048 + j * 512);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if constexpr (HQ == 0) {
        qr[d][c][0] = *reinterpret_cast<const u32x4*>(qp[c] + kc * 1024);
        sr[d][c] = *reinterpret_cast<const uint32_t*>(sp[c] + kc * 256);
      } else if constexpr (HQ == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qr[d][c][i] = *reinterpret_cast<const u32x4*>(bp[c] + (kc * 4 + i) * 512);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          qr[d][c][j] = *reinterpret_cast<const u32x4*>(qp[c] + (kc * 2 + j) * 1024);
          fr[d][c][j] = fsp[c][(kc * 2 + j) * 16];
        }
      }
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
#pragma unroll
  for (int j = 0; j < 4; ++j) sa[0][wave * 4 + j][lane] = ar[0][j];
  __syncthreads();

  for (int k0 = 0; k0 < NK; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kg = k0 + d;
      if (kg < NK) {
        u32x4 q[CT][NQ];
        uint32_t sv[CT];
        float fv[CT][2];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
          for (int i = 0; i < NQ; ++i) q[c][i] = qr[d][c][i];
          sv[c] = sr[d][c];
          fv[c][0] = fr[d][c][0];
          fv[c][1] = fr[d][c][1];
        }
        load(kg + D, d);
        const int buf = kg & 1;
        if constexpr (HQ == 2) {
          // two 64-input blocks per step, each scaled by its row's scale
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f16x8 w0[CT], w1[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) {
              w0[c] = e4m3x8_f16(q[c][j].x, q[c][j].y);
              w1[c] = e4m3x8_f16(q[c][j].z, q[c][j].w);
            }
#pragma unroll
            for (int r = 0; r < MM_RT; ++r) {
              const f16x8 a0 = __builtin_bit_cast(f16x8, sa[buf][r * 4 + 2 * j][lane]);
              const f16x8 a1 = __builtin_bit_cast(f16x8, sa[buf][r * 4 + 2 * j + 1][lane]);
#pragma unroll
              for (int c = 0; c < CT; ++c) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
                t = mfma_f16(a0, w0[c], t);
                t = mfma_f16(a1, w1[c], t);
                acc[r][c] += fv[c][j] * t;
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < (HQ == 2 ? 0 : 4); ++i) {
          if constexpr (HQ == 0) {
            f16x8 w[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) w[c] = nvfp4x8_f16(q[c][0][i], (sv[c] >> (8 * i)) & 0xffu);
#pragma unroll
            for (int r = 0; r < MM_RT; ++r) {
              const f16x8 av = __builtin_bit_cast(f16x8, sa[buf][r * 4 + i][lane]);
#pragma unroll
              for (int c = 0; c < CT; ++c) acc[r][c] = mfma_f16(av, w[c], acc[r][c]);
            }
          } else if constexpr (HQ == 1) {
#pragma unroll
            for (int r = 0; r < MM_RT; ++r) {
              const f16x8 av = __builtin_bit_cast(f16x8, sa[buf][r * 4 + i][lane]);
              u32x4 hi, lo;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float v0 = (float)av[2 * e], v1 = (float)av[2 * e + 1];
                const float h0 = u2f(f2u(v0) & 0xffff0000u), h1 = u2f(f2u(v1) & 0xffff0000u);
                hi[e] = pack_hi16(h0, h1);
                // v - h is exact and has at most 3 significant bits
                lo[e] = pack_hi16(v0 - h0, v1 - h1);
              }
              const bf16x8 ah = __builtin_bit_cast(bf16x8, hi), al = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
              for (int c = 0; c < CT; ++c) {
                const bf16x8 w = __builtin_bit_cast(bf16x8, q[c][i]);
                acc[r][c] = mfma_bf16(ah, w, acc[r][c]);
                acc[r][c] = mfma_bf16(al, w, acc[r][c]);
              }
            }
          }
        }
        if (kg + 1 < NK) {
          const int dn = d + 1 == D ? 0 : d + 1;
#pragma unroll
          for (int j = 0; j < 4; ++j) sa[buf ^ 1][wave * 4 + j][lane] = ar[dn][j];
        }
        __syncthreads();
      }
    }
  }

  if constexpr (KS == 2) {
    static_assert(sizeof(sa_all) >= MM_WAVES * MM_RT * CT * 64 * sizeof(f32x4), "staging area");
    f32x4* T = reinterpret_cast<f32x4*>(&sa_all[0][0][0]);
    auto tix = [&](int r, int c) { return ((wave * MM_RT + r) * CT + c) * 64 + lane; };
    if (grp == 1) {
#pragma unroll
      for (int r = 0; r < MM_RT; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) T[tix(r, c)] = acc[r][c];
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < MM_RT; ++r)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[r][c] += T[tix(r, c)];
    }
  }
  // logits, per-row best over this wave's 64 vocabulary rows, then over the
  // workgroup's waves in LDS, then one atomicMax per row
#pragma unroll
  for (int r = 0; r < MM_RT; ++r) {
    if (grp != 0) break;
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int voc = (vt0 + c) * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = (m.rb * MM_RT + r) * 16 + 4 * (lane >> 4) + e;
        const float val = acc[r][c][e] * a.g;
        if (row < a.R && voc < a.VD) {
          if (a.logits) a.logits[(size_t)row * a.VD + voc] = val;
          const unsigned long long key = argmax_key(val, (uint32_t)voc);
          best[e] = key > best[e] ? key : best[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int msk = 8; msk >= 1; msk >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best[e], msk, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(best[e] >> 32), msk, 64);
        const unsigned long long o = ((unsigned long long)hi << 32) | lo;
        best[e] = o > best[e] ? o : best[e];
      }
      if ((lane & 15) == 0 && best[e])
        __hip_atomic_fetch_max(&best_s[r * 16 + 4 * (lane >> 4) + e], best[e], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  if (threadIdx.x < MM_RT * 16) {
    const int row = m.rb * MM_RT * 16 + threadIdx.x;
    const unsigned long long k = best_s[threadIdx.x];
    if (row < a.R && k) atomicMax(&a.keys[row], k);
  }
}

bool head_mm_fits(int R) { return R > 32; }

void launch_head_mm(hipStream_t st, const uint16_t* af, int R, const DevWeights& d, float* logits,
                    unsigned long long* keys) {
  HeadMM a;
  a.af = af;
  a.R = R;
  a.hq = d.hq;
  a.hs = d.hs;
  a.hb = d.hb;
  a.fw = d.hf8.w;
  a.fs = d.hf8.s;
  a.g = d.hg;
  a.VD = d.VD;
  a.VT = d.VT;
  a.logits = logits;
  a.keys = keys;
  if (d.head_fmt == 2) {
    // block-FP8 head (2 times the NVFP4 bytes): 128 vocabulary rows per
    // workgroup, two steps in flight, at every row count
    k_head_mm<2, 2, 2, 1><<<mm_grid(R, (d.VT + 7) / 8, 1), 256, 0, st>>>(a);
    return;
  }
  if (d.head_fmt == 1) {
    // bf16 head (4 times the NVFP4 bytes): 128 vocabulary rows per
    // workgroup, two steps in flight, at every row count
    k_head_mm<2, 2, 1, 1><<<mm_grid(R, (d.VT + 7) / 8, 1), 256, 0, st>>>(a);
    return;
  }
  // 256 vocabulary rows per workgroup at every row count (narrower tiles
  // measured slower at 64 rows); up to 64 rows the input groups in two
  // halves inside the workgroup (B16 0.615 -> 0.613 ms; the bf16 and FP8
  // heads measured 1.5-2.4 % slower that way)
  if (R <= 64) k_head_mm<4, 3, 0, 2><<<mm_grid(R, (d.VT + 15) / 16, 1), 512, 0, st>>>(a);
  else k_head_mm<4, 3, 0, 1><<<mm_grid(R, (d.VT + 15) / 16, 1), 256, 0, st>>>(a);
}

}  // namespace kd
