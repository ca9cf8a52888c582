// The block-drafter round for up to 4 streams (16 block rows) as a sequence of
// workgroup-level phases (model card "Kolibri-1 block drafter", section
// Architecture: Input, Positions 2-4, Predecessor head, Spine, Body, Output).
//
//   PRE0  fuse = W_fuse taps;  fce = W_fc[:, H:] E[anchor];  pb = B_p E[pred]
//   PRE1  row 0 = W_fc[:, :H] f + fce;  sp = silu(A_p f + pb)
//   PRE2  rows 1..3 = mask + f + U_p sp
//   per layer l:
//     SA   (l >= 1) ss = silu(A_s (g_s * x_{j-1}) / rms(x_{j-1}))
//     SU   (l >= 1) x_j += U_s ss   (rows 1..3; row 0 copied)
//     QKV  q,k,v = W_qkv (g_a * x) / rms(x), RoPE on q and k
//     ATTN partial softmax over 128 context keys per (stream, head, chunk)
//     MERGE chunks + the block's own keys (causal) -> o
//     O    x += W_o o
//     GU   h = silu(W_g (g_f * x) / rms(x)) * (W_u (g_f * x) / rms(x))
//     DOWN x += W_down h
//   HEAD  logits = Head (g_o * x) / rms(x) * g_tensor -> per-workgroup argmax
//   FINAL per-row argmax over workgroups -> target id
//
// A workgroup (8 waves) owns whole output tiles: its waves split the inputs,
// an LDS reduction sums them in a fixed order, and the epilogue applies the
// elementwise steps, so every phase writes final values once. RMSNorm is
// deferred: the projection runs on g * x and the epilogue scales by 1/rms(x),
// with rms from per-tile sums of squares written by the producer of x.
//
// In the persistent kernel, phases are separated by a two-level counter
// barrier without cache-wide fences. That is safe because every buffer a phase
// reads from another workgroup is written at most once per launch, with
// write-through stores, and is not read before the barrier that follows the
// write (L1/L2 are clean for these lines at kernel start). Each workgroup
// issues the weight loads of its first unit of a phase before waiting at the
// barrier, so weight streaming overlaps the synchronisation.
#include "kd_device.h"
#include "kd_small.h"

namespace kd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum Phase {
  PH_PRE0 = 0, PH_PRE1 = 1, PH_PRE2 = 2,
  PH_SA = 0, PH_SU = 1, PH_QKV = 2, PH_ATTN = 3, PH_MERGE = 4, PH_O = 5, PH_GU = 6, PH_DOWN = 7,
  PH_HEAD = 3 + 8 * NL, PH_FINAL = 4 + 8 * NL
};

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_rlx(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// e4m3 pairs -> bf16 pairs with unit scale (exact on gfx950).
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// 8 e2m1 codes (even element in the low nibble) times an e4m3 block scale,
// exactly in f16: e2m1 decoded with unit scale, then one packed f16 multiply
// per pair (<= 6 significant bits, within f16's normal range).
__device__ __forceinline__ f16x8 nvfp4x8_f16(uint32_t nib, uint32_t scode) {
  const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scode, 1.0f, false);
  const f16x2 sc = {s2.x, s2.x};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 3) * sc;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ void split_bf16(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)v[i];
    hi[i] = h;
    lo[i] = (__bf16)(v[i] - (float)h);
  }
}
__device__ __forceinline__ void split_f16(const float* v, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)v[i];
    hi[i] = h;
    lo[i] = (_Float16)(v[i] - (float)h);
  }
}

__device__ __forceinline__ unsigned long long u64_max(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long shfl_xor_u64s(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Grid barrier: two-level counters (groups of 16 workgroups), monotonic so
// nothing is ever reset, a generation word, and a wall-clock bound: after
// 0.2 s the workgroup sets the error word and goes on, so every wave still
// reaches the end of the kernel.
// ---------------------------------------------------------------------------
struct SyncState {
  unsigned epoch;  // barriers passed in this launch
  unsigned base;   // generation word at kernel start
};

__device__ void grid_sync(const SmallArgs& a, SyncState& sy) {
  ++sy.epoch;
  const unsigned target = sy.base + sy.epoch;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* bar = a.s.bar;
    const unsigned G = gridDim.x, grp = blockIdx.x >> 4, ngrp = (G + 15) >> 4;
    const unsigned gsize = min(16u, G - grp * 16);
    const unsigned v = __hip_atomic_fetch_add(&bar[grp * 32], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if ((v + 1) % gsize == 0) {
      const unsigned w = __hip_atomic_fetch_add(&bar[16 * 32], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      if ((w + 1) % ngrp == 0)
        __hip_atomic_store(&bar[17 * 32], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const unsigned long long t0 = wall_clock64();
    while ((int)(ld_rlx(&bar[17 * 32]) - target) < 0) {
      if (wall_clock64() - t0 > 20000000ull) {      // 0.2 s at the 100 MHz wall clock
        __hip_atomic_store(&bar[18 * 32], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Projection units: NT consecutive 16-row weight tiles; wave w (< AW) takes
// the 64-input blocks kb0 + w*KBS .. + KBS.
// ---------------------------------------------------------------------------
template <int NT, int KBS>
struct WRegs {
  u32x4 w[NT][KBS];
  float s[NT][KBS];
};

template <int NT, int KBS, int AW>
__device__ __forceinline__ void load_w(WRegs<NT, KBS>& r, const Fp8Mat& W, int tile0, int ntv,
                                       int kb0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KB = W.K >> 6;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < KBS; ++j) {
      r.w[i][j] = u32x4{0u, 0u, 0u, 0u};
      r.s[i][j] = 0.f;
      if (wave < AW && i < ntv) {
        const size_t blk = (size_t)(tile0 + i) * KB + kb0 + wave * KBS + j;
        r.w[i][j] = *reinterpret_cast<const u32x4*>(W.w + blk * 1024 + lane * 16);
        r.s[i][j] = W.s[blk * 16 + (lane & 15)];
      }
    }
}

// Activation rows for the A operand.
struct ASrc {
  const void* base;
  int ld;               // elements per row
  int mode;             // 0: row r; 1: row r/3; 2: row 4(r/3) + r%3; 3: row ids[r]
  const int32_t* ids;
  const float* gain;    // per-column gain, or null
  int kb_off;           // weight block of column 0
  int R;
  int bf16;             // 1: bf16 rows (exact, lo = 0); 0: fp32 rows
};

__device__ __forceinline__ size_t a_row(const ASrc& A, int r) {
  switch (A.mode) {
    case 1: return (size_t)(r / 3);
    case 2: return (size_t)(4 * (r / 3) + r % 3);
    case 3: return (size_t)A.ids[r];
    default: return (size_t)r;
  }
}

__device__ __forceinline__ void load_a(const ASrc& A, int kb, bf16x8& h0, bf16x8& l0, bf16x8& h1,
                                       bf16x8& l1) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  h0 = l0 = h1 = l1 = z;
  if (r >= A.R) return;
  const int c0 = (kb - A.kb_off) * 64 + 8 * (lane >> 4);
  const size_t row = a_row(A, r);
  if (A.bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(A.base) + row * A.ld + c0;
    h0 = *reinterpret_cast<const bf16x8*>(p);
    h1 = *reinterpret_cast<const bf16x8*>(p + 32);
    return;
  }
  const float* p = static_cast<const float*>(A.base) + row * A.ld + c0;
  float v0[8], v1[8];
  *reinterpret_cast<f32x4*>(v0) = *reinterpret_cast<const f32x4*>(p);
  *reinterpret_cast<f32x4*>(v0 + 4) = *reinterpret_cast<const f32x4*>(p + 4);
  *reinterpret_cast<f32x4*>(v1) = *reinterpret_cast<const f32x4*>(p + 32);
  *reinterpret_cast<f32x4*>(v1 + 4) = *reinterpret_cast<const f32x4*>(p + 36);
  if (A.gain) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v0[i] *= A.gain[c0 + i];
      v1[i] *= A.gain[c0 + 32 + i];
    }
  }
  split_bf16(v0, h0, l0);
  split_bf16(v1, h1, l1);
}

// Partial products of each wave into LDS: red[((wave*NT + i)*4 + e)*64 + lane].
template <int NT, int KBS, int AW>
__device__ __forceinline__ void gemm_compute(const WRegs<NT, KBS>& r, const ASrc& A, int kb0,
                                             float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < AW) {
#pragma unroll
    for (int j = 0; j < KBS; ++j) {
      bf16x8 h0, l0, h1, l1;
      load_a(A, kb0 + wave * KBS + j, h0, l0, h1, l1);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const bf16x8 w0 = e4m3x8_bf16(r.w[i][j].x, r.w[i][j].y);
        const bf16x8 w1 = e4m3x8_bf16(r.w[i][j].z, r.w[i][j].w);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        t = mfma_bf16(h0, w0, t);
        t = mfma_bf16(l0, w0, t);
        t = mfma_bf16(h1, w1, t);
        t = mfma_bf16(l1, w1, t);
        acc[i] += r.s[i][j] * t;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * NT + i) * 4 + e) * 64 + lane] = acc[i][e];
  __syncthreads();
}

// Sums the 8 waves' partials in a fixed order and calls f(i, m, n, v) for
// output row m and column n of tile i. Within a wave the 64 items cover 4 rows
// x 16 columns of one tile, so f may use shuffles across columns (xor 1..8).
template <int NT, class F>
__device__ __forceinline__ void gemm_epilogue(const float* red, F&& f) {
  for (int it = threadIdx.x; it < NT * 256; it += SMALL_WG) {
    const int i = it >> 8, m = (it >> 4) & 15, n = it & 15;
    const int L = 16 * (m >> 2) + n, e = m & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) v += red[((w * NT + i) * 4 + e) * 64 + L];
    f(i, m, n, v);
  }
  __syncthreads();
}

// 1/rms of up to 16 rows of a residual stage from its per-tile sums of
// squares, into LDS inv[16]; `map` gives the stage row of row r.
template <class Map>
__device__ __forceinline__ void inv_rms_rows(const float* ssq, int nrows, Map map, float eps,
                                             float* inv) {
  const int t = threadIdx.x, r = t >> 5, l32 = t & 31;
  float sum = 0.f;
  if (r < nrows) {
    const float* p = ssq + (size_t)map(r) * HT;
    for (int k = l32; k < HT; k += 32) sum += p[k];
  }
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if (r < nrows && l32 == 0) inv[r] = 1.0f / sqrtf(sum / H + eps);
  __syncthreads();
}

// Sum of squares of this tile's 16 columns for the item's row (all lanes).
__device__ __forceinline__ float tile_ssq(float x) {
  float s = x * x;
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1) s += __shfl_xor(s, m, 64);
  return s;
}

// One projection unit: prefetch weights, wait at the barrier if this is the
// workgroup's first unit of the phase, then compute, reduce and run `epi`.
template <int NT, int KBS, int AW, class Prep, class Epi>
__device__ __forceinline__ void gemm_unit(const SmallArgs& a, SyncState& epoch, bool sync,
                                          const Fp8Mat& W, int tile0, int ntv, int kb0,
                                          const ASrc& A, float* red, Prep&& prep, Epi&& epi) {
  WRegs<NT, KBS> r;
  load_w<NT, KBS, AW>(r, W, tile0, ntv, kb0);
  if (sync) grid_sync(a, epoch);
  prep();
  gemm_compute<NT, KBS, AW>(r, A, kb0, red);
  gemm_epilogue<NT>(red, epi);
}

struct NoPrep {
  __device__ void operator()() const {}
};

// ---------------------------------------------------------------------------
// Phases. `sync` is true when the phase must wait at a grid barrier first
// (persistent kernel); every workgroup then calls grid_sync exactly once.
// ---------------------------------------------------------------------------
__device__ __attribute__((noinline)) void ph_pre0(const SmallArgs& a, float* red, SyncState& epoch) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevWeights& d = a.d;
  const int B = a.B, R = a.R;
  // RoPE table for every block row: positions len + j, angles in fp64.
  if (wg == G - 1) {
    for (int t = threadIdx.x; t < R * (DH / 2); t += SMALL_WG) {
      const int r = t / (DH / 2), fi = t % (DH / 2);
      const double pos = (double)a.lens[r >> 2] + (r & 3);
      const double ang = pos * pow((double)a.theta, -(double)fi / (DH / 2));
      st_wt(&s.rope[t * 2], (float)cos(ang));
      st_wt(&s.rope[t * 2 + 1], (float)sin(ang));
    }
  }
  const int n_fuse = HT, n_fce = HT, n_pb = RK / 16;
  for (int u = wg; u < n_fuse + n_fce + n_pb; u += G) {
    if (u < n_fuse) {
      const ASrc A{a.taps, NTAP * H, 0, nullptr, nullptr, 0, B, 1};
      gemm_unit<1, 15, 8>(a, epoch, false, d.fuse, u, 1, 0, A, red, NoPrep{},
                          [&](int, int m, int n, float v) {
                            if (m < B) st_wt(&s.f[m * H + u * 16 + n], v);
                          });
    } else if (u < n_fuse + n_fce) {
      const int t = u - n_fuse;
      const ASrc A{d.table, H, 3, a.anchor, nullptr, 40, B, 1};
      gemm_unit<1, 5, 8>(a, epoch, false, d.fc, t, 1, 40, A, red, NoPrep{},
                         [&](int, int m, int n, float v) {
                           if (m < B) st_wt(&s.fce[m * H + t * 16 + n], v);
                         });
    } else {
      const int t = u - n_fuse - n_fce;
      const ASrc A{d.table, H, 3, a.pred, nullptr, 40, 3 * B, 1};
      gemm_unit<1, 5, 8>(a, epoch, false, d.pred_ab, t, 1, 40, A, red, NoPrep{},
                         [&](int, int m, int n, float v) {
                           if (m < 3 * B) st_wt(&s.pb[m * RK + t * 16 + n], v);
                         });
    }
  }
}

__device__ __attribute__((noinline)) void ph_pre1(const SmallArgs& a, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevWeights& d = a.d;
  const int B = a.B;
  bool first = sync;
  for (int u = wg; u < HT + RK / 16; u += G) {
    if (u < HT) {
      const ASrc A{s.f, H, 0, nullptr, nullptr, 0, B, 0};
      gemm_unit<1, 5, 8>(a, epoch, first, d.fc, u, 1, 0, A, red, NoPrep{},
                         [&](int, int m, int n, float v) {
                           const int col = u * 16 + n;
                           const float x = v + (m < B ? s.fce[m * H + col] : 0.f);
                           const float q = tile_ssq(x);
                           if (m < B) {
                             st_wt(&s.x[0][(4 * m) * H + col], x);
                             if (n == 0) st_wt(&s.ssq[0][(4 * m) * HT + u], q);
                           }
                         });
    } else {
      const int t = u - HT;
      const ASrc A{s.f, H, 1, nullptr, nullptr, 0, 3 * B, 0};
      gemm_unit<1, 5, 8>(a, epoch, first, d.pred_ab, t, 1, 0, A, red, NoPrep{},
                         [&](int, int m, int n, float v) {
                           if (m < 3 * B) {
                             const int c = t * 16 + n;
                             st_wt(&s.sp[m * RK + c], silu(v + s.pb[m * RK + c]));
                           }
                         });
    }
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

__device__ __attribute__((noinline)) void ph_pre2(const SmallArgs& a, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevWeights& d = a.d;
  const int B = a.B;
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{s.sp, RK, 0, nullptr, nullptr, 0, 3 * B, 0};
    gemm_unit<1, 1, 4>(a, epoch, first, d.pred_u, u, 1, 0, A, red, NoPrep{},
                       [&](int, int m, int n, float v) {
                         const int col = u * 16 + n;
                         const int row = 4 * (m / 3) + m % 3 + 1;
                         const float x =
                             m < 3 * B ? d.mask[col] + s.f[(m / 3) * H + col] + v : 0.f;
                         const float q = tile_ssq(x);
                         if (m < 3 * B) {
                           st_wt(&s.x[0][row * H + col], x);
                           if (n == 0) st_wt(&s.ssq[0][row * HT + u], q);
                         }
                       });
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// Spine A: ss = silu(A_s (g_s * x_{j-1}) / rms(x_{j-1})) for rows j = 1..3.
__device__ __attribute__((noinline)) void ph_sa(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevLayer& L = a.d.layer[l];
  const int B = a.B, src = xs_d(l - 1);
  float* inv = red + 8192;
  bool first = sync;
  for (int u = wg; u < RK / 16; u += G) {
    const ASrc A{s.x[src], H, 2, nullptr, L.spine_norm, 0, 3 * B, 0};
    gemm_unit<1, 5, 8>(
        a, epoch, first, L.sa, u, 1, 0, A, red,
        [&] { inv_rms_rows(s.ssq[src], 3 * B, [](int r) { return 4 * (r / 3) + r % 3; }, a.eps, inv); },
        [&](int, int m, int n, float v) {
          if (m < 3 * B) st_wt(&s.ss[l][m * RK + u * 16 + n], silu(v * inv[m]));
        });
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// Spine U: x_j (j = 1..3) = x_{j} + U_s ss; row 0 copied into the new stage.
__device__ __attribute__((noinline)) void ph_su(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevLayer& L = a.d.layer[l];
  const int B = a.B, src = xs_d(l - 1), dst = xs_in(l);
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{s.ss[l], RK, 0, nullptr, nullptr, 0, 3 * B, 0};
    gemm_unit<1, 1, 4>(a, epoch, first, L.su, u, 1, 0, A, red, NoPrep{},
                       [&](int, int m, int n, float v) {
                         const int col = u * 16 + n;
                         const int row = 4 * (m / 3) + m % 3 + 1;
                         const float x = m < 3 * B ? s.x[src][row * H + col] + v : 0.f;
                         const float q = tile_ssq(x);
                         if (m < 3 * B) {
                           st_wt(&s.x[dst][row * H + col], x);
                           if (n == 0) st_wt(&s.ssq[dst][row * HT + u], q);
                         }
                       });
    // row 0 of every stream is untouched by the spine
    for (int t = threadIdx.x; t < B * 17; t += SMALL_WG) {
      const int b = t / 17, c = t % 17, row = 4 * b;
      if (c < 16)
        st_wt(&s.x[dst][row * H + u * 16 + c], s.x[src][row * H + u * 16 + c]);
      else
        st_wt(&s.ssq[dst][row * HT + u], s.ssq[src][row * HT + u]);
    }
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// q|k|v = W (g_a * x) / rms(x); RoPE on q and k inside each paired tile.
__device__ __attribute__((noinline)) void ph_qkv(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevLayer& L = a.d.layer[l];
  const int R = a.R, src = xs_in(l);
  float* inv = red + 8192;
  constexpr int NT = 2, NTILE = QKV / 16, NU = NTILE / NT;
  bool first = sync;
  for (int u = wg; u < NU; u += G) {
    const ASrc A{s.x[src], H, 0, nullptr, L.attn_norm, 0, R, 0};
    gemm_unit<NT, 5, 8>(
        a, epoch, first, L.qkv, u * NT, NT, 0, A, red,
        [&] { inv_rms_rows(s.ssq[src], R, [](int r) { return r; }, a.eps, inv); },
        [&](int i, int m, int n, float v) {
          const int t = u * NT + i, sec = t / HT;
          const int nat = qkv_natural(t * 16 + n) - sec * H;      // column within q, k or v
          const float val = m < R ? v * inv[m] : 0.f;
          const float partner = __shfl_xor(val, 8, 64);
          float out = val;
          if (sec < 2) {
            const int fi = (nat % DH) & 63;
            const float cs = m < R ? s.rope[(m * (DH / 2) + fi) * 2] : 0.f;
            const float sn = m < R ? s.rope[(m * (DH / 2) + fi) * 2 + 1] : 0.f;
            out = n < 8 ? val * cs - partner * sn : partner * sn + val * cs;
          }
          if (m < R) {
            float* dstp = sec == 0 ? s.q[l] : (sec == 1 ? s.k[l] : s.v[l]);
            st_wt(&dstp[m * H + nat], out);
          }
        });
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// Attention over one chunk of 128 context keys for one (stream, head):
// wave w takes keys 16w..16w+15 (4 keys per step, 16 lanes x 8 dims per key).
__device__ __attribute__((noinline)) void ph_attn(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, d0 = (lane & 15) * 8;
  const int nch = a.nch, nunits = a.B * NH * nch;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  float* s_o = red;                   // [8][4][128]
  float* s_m = red + 8 * 4 * DH;      // [8][4]
  float* s_l = s_m + 32;              // [8][4]
  bool first = sync;
  for (int u = wg; u < nunits; u += G) {
    const int b = u / (NH * nch), h = (u / nch) % NH, c = u % nch;
    const int len = a.lens[b];
    const int n = min(len, a.window), first_pos = len - n;
    const bool active = c * ATT_CH < n;
    u32x4 kr[4], vr[4];
    const uint16_t* kbase = a.kv.k[l] + b * a.kv.ss + h * a.kv.sh + d0;
    const uint16_t* vbase = a.kv.v[l] + b * a.kv.ss + h * a.kv.sh + d0;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int idx = c * ATT_CH + wave * 16 + st * 4 + g;
      kr[st] = vr[st] = u32x4{0u, 0u, 0u, 0u};
      if (active && idx < n) {
        const int slot = (first_pos + idx) % a.kv.cap;
        kr[st] = *reinterpret_cast<const u32x4*>(kbase + (size_t)slot * a.kv.sl);
        vr[st] = *reinterpret_cast<const u32x4*>(vbase + (size_t)slot * a.kv.sl);
      }
    }
    if (first) grid_sync(a, epoch);
    first = false;
    if (!active) continue;
    float q[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) q[j][e] = s.q[l][(b * 4 + j) * H + h * DH + d0 + e] * qs;
    float sc[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int idx = c * ATT_CH + wave * 16 + st * 4 + g;
      float kf[8];
      bf16x8_to_f32(kr[st], kf);
      float dot[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dot[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot[j] += q[j][e] * kf[e];
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) dot[j] += __shfl_xor(dot[j], m, 64);
        sc[j][st] = idx < n ? dot[j] : -__builtin_inff();
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = fmaxf(fmaxf(sc[j][0], sc[j][1]), fmaxf(sc[j][2], sc[j][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float lsum = 0.f, o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float p = sc[j][st] == -__builtin_inff() ? 0.f : exp2f(sc[j][st] - mx);
        float vf[8];
        bf16x8_to_f32(vr[st], vf);
        lsum += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += p * vf[e];
      }
      lsum += __shfl_xor(lsum, 16, 64);
      lsum += __shfl_xor(lsum, 32, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 16, 64);
        o[e] += __shfl_xor(o[e], 32, 64);
      }
      if (g == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[(wave * 4 + j) * DH + d0 + e] = o[e];
      if (lane == 0) {
        s_m[wave * 4 + j] = mx;
        s_l[wave * 4 + j] = lsum;
      }
    }
    __syncthreads();
    {
      const int j = threadIdx.x >> 7, dd = threadIdx.x & 127;
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < 8; ++w) M = fmaxf(M, s_m[w * 4 + j]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float mw = s_m[w * 4 + j];
        if (mw != -__builtin_inff()) {
          const float f = exp2f(mw - M);
          Ls += s_l[w * 4 + j] * f;
          O += s_o[(w * 4 + j) * DH + dd] * f;
        }
      }
      const size_t pb = ((size_t)(b * NH + h) * nch + c) * 4 + j;
      st_wt(&s.ao[l][pb * DH + dd], O);
      if (dd == 0) {
        st_wt(&s.am[l][pb], M);
        st_wt(&s.al[l][pb], Ls);
      }
    }
    __syncthreads();
  }
  if (first) grid_sync(a, epoch);
}

// Merge of the chunk partials with the block's own keys (row j sees block
// rows 0..j) for one (stream, head); thread (j, d).
__device__ __attribute__((noinline)) void ph_merge(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = a.nch;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;
  bool first = sync;
  for (int u = wg; u < a.B * NH; u += G) {
    if (first) grid_sync(a, epoch);
    first = false;
    const int b = u / NH, h = u % NH;
    const int n = min(a.lens[b], a.window), nc = (n + ATT_CH - 1) / ATT_CH;
    // block scores s[j][i] = q_j . k_i: wave w covers row j = w/2, dims 64*(w%2)..
    {
      const int j = wave >> 1, dd = 64 * (wave & 1) + lane;
      const float qv = s.q[l][(b * 4 + j) * H + h * DH + dd];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = wave_sum(qv * s.k[l][(b * 4 + i) * H + h * DH + dd]);
        if (lane == 0) red[wave * 4 + i] = p;
      }
    }
    __syncthreads();
    const int j = threadIdx.x >> 7, dd = threadIdx.x & 127;
    float sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sb[i] = (red[(2 * j) * 4 + i] + red[(2 * j + 1) * 4 + i]) * qs;
    float M = -__builtin_inff();
    for (int c = 0; c < nc; ++c) M = fmaxf(M, s.am[l][((size_t)(b * NH + h) * nch + c) * 4 + j]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i <= j) M = fmaxf(M, sb[i]);
    float Ls = 0.f, O = 0.f;
    for (int c = 0; c < nc; ++c) {
      const size_t pb = ((size_t)(b * NH + h) * nch + c) * 4 + j;
      const float f = exp2f(s.am[l][pb] - M);
      Ls += s.al[l][pb] * f;
      O += s.ao[l][pb * DH + dd] * f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i <= j) {
        const float f = exp2f(sb[i] - M);
        Ls += f;
        O += f * s.v[l][(b * 4 + i) * H + h * DH + dd];
      }
    st_wt(&s.o[l][(b * 4 + j) * H + h * DH + dd], O / Ls);
    __syncthreads();
  }
  if (first) grid_sync(a, epoch);
}

// x_{out} = x_{in} + W v for a 2560-wide output, with per-tile sums of squares.
template <int KBS>
__device__ __attribute__((noinline)) void ph_resid(const SmallArgs& a, const Fp8Mat& W, const float* srcA, int ldA,
                         int xin, int xout, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const int R = a.R;
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{srcA, ldA, 0, nullptr, nullptr, 0, R, 0};
    gemm_unit<1, KBS, 8>(a, epoch, first, W, u, 1, 0, A, red, NoPrep{},
                         [&](int, int m, int n, float v) {
                           const int col = u * 16 + n;
                           const float x = m < R ? s.x[xin][m * H + col] + v : 0.f;
                           const float q = tile_ssq(x);
                           if (m < R) {
                             st_wt(&s.x[xout][m * H + col], x);
                             if (n == 0) st_wt(&s.ssq[xout][m * HT + u], q);
                           }
                         });
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// h = silu(gate / rms) * (up / rms) with gate, up = W (g_f * x).
__device__ __attribute__((noinline)) void ph_gu(const SmallArgs& a, int l, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevLayer& L = a.d.layer[l];
  const int R = a.R, src = xs_o(l);
  float* inv = red + 8192;
  constexpr int NT = 3, NU = GU / 16 / NT;
  bool first = sync;
  for (int u = wg; u < NU; u += G) {
    const ASrc A{s.x[src], H, 0, nullptr, L.ffn_norm, 0, R, 0};
    gemm_unit<NT, 5, 8>(
        a, epoch, first, L.gu, u * NT, NT, 0, A, red,
        [&] { inv_rms_rows(s.ssq[src], R, [](int r) { return r; }, a.eps, inv); },
        [&](int i, int m, int n, float v) {
          const int t = u * NT + i;
          const float val = m < R ? v * inv[m] : 0.f;
          const float up = __shfl_xor(val, 8, 64);
          if (m < R && n < 8) st_wt(&s.h[l][m * FF + 8 * t + n], silu(val) * up);
        });
    first = false;
  }
  if (first) grid_sync(a, epoch);
}

// NVFP4 head over 16-row vocab tiles (HEAD_NT per unit): wave w takes the
// 128-input groups kg0(w)..kg1(w); per-workgroup argmax candidates per row.
__device__ __attribute__((noinline)) void ph_head(const SmallArgs& a, float* red, SyncState& epoch, bool sync) {
  const int G = gridDim.x, wg = blockIdx.x;
  const SmallBufs& s = a.s;
  const DevWeights& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = a.R, VT = d.VT, VD = d.VD;
  constexpr int KG = H / 128;
  const int kg0 = (KG * wave) >> 3, kg1 = (KG * (wave + 1)) >> 3, ng = kg1 - kg0;  // 2 or 3
  const int src = a.nl == 0 ? 0 : xs_d(a.nl - 1);
  const int nunits = (VT + HEAD_NT - 1) / HEAD_NT;
  float* inv = red + 8192;
  unsigned long long* best = reinterpret_cast<unsigned long long*>(red + 8192 + 32);  // [16]
  if (threadIdx.x < SR_MAX) best[threadIdx.x] = 0ull;

  auto load_unit = [&](int u, u32x4 (&q)[HEAD_NT][3], uint32_t (&sv)[HEAD_NT][3]) {
#pragma unroll
    for (int i = 0; i < HEAD_NT; ++i)
#pragma unroll
      for (int gg = 0; gg < 3; ++gg) {
        q[i][gg] = u32x4{0u, 0u, 0u, 0u};
        sv[i][gg] = 0u;
        const int vt = u * HEAD_NT + i;
        if (vt < VT && gg < ng) {
          const size_t idx = ((size_t)vt * KG + kg0 + gg) * 64 + lane;
          q[i][gg] = *reinterpret_cast<const u32x4*>(d.hq + idx * 16);
          sv[i][gg] = *reinterpret_cast<const uint32_t*>(d.hs + idx * 4);
        }
      }
  };

  u32x4 q[HEAD_NT][3];
  uint32_t sv[HEAD_NT][3];
  if (wg < nunits) load_unit(wg, q, sv);
  if (sync) grid_sync(a, epoch);
  inv_rms_rows(s.ssq[src], R, [](int r) { return r; }, a.eps, inv);
  // A operand (g_o * x, hi/lo f16) for this wave's inputs, kept for all units
  f16x8 ah[3][4], al[3][4];
  {
    const int r = lane & 15;
#pragma unroll
    for (int gg = 0; gg < 3; ++gg)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
        const int c0 = (kg0 + gg) * 128 + t * 32 + 8 * (lane >> 4);
        if (r < R && gg < ng)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = s.x[src][r * H + c0 + e] * d.final_norm[c0 + e];
        split_f16(v, ah[gg][t], al[gg][t]);
      }
  }
  for (int u = wg; u < nunits; u += G) {
    if (u != wg) load_unit(u, q, sv);
    f32x4 acc[HEAD_NT];
#pragma unroll
    for (int i = 0; i < HEAD_NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < 3; ++gg) {
      if (gg < ng) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < HEAD_NT; ++i) {
            const f16x8 w = nvfp4x8_f16(q[i][gg][t], sv[i][gg] >> (8 * t));
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[gg][t], w, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[gg][t], w, acc[i], 0, 0, 0);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < HEAD_NT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * HEAD_NT + i) * 4 + e) * 64 + lane] = acc[i][e];
    __syncthreads();
    gemm_epilogue<HEAD_NT>(red, [&](int i, int m, int n, float v) {
      const int voc = (u * HEAD_NT + i) * 16 + n;
      const bool ok = m < R && voc < VD;
      const float logit = ok ? v * inv[m] * d.hg : 0.f;
      if (ok && a.out_logits) a.out_logits[(size_t)m * VD + voc] = logit;
      unsigned long long key = ok ? argmax_key(logit, (uint32_t)voc) : 0ull;
#pragma unroll
      for (int mm = 1; mm <= 8; mm <<= 1) key = u64_max(key, shfl_xor_u64s(key, mm));
      if (n == 0 && key) atomicMax(&best[m], key);
    });
  }
  __syncthreads();
  if (threadIdx.x < SR_MAX) st_wt64(&s.cand[wg * SR_MAX + threadIdx.x], best[threadIdx.x]);
}

__device__ __attribute__((noinline)) void ph_final(const SmallArgs& a, SyncState& epoch, bool sync) {
  if (sync) grid_sync(a, epoch);
  if (blockIdx.x != 0) return;
  const int G = gridDim.x, t = threadIdx.x, r = t >> 5, l32 = t & 31;
  unsigned long long k = 0ull;
  if (r < a.R)
    for (int g = l32; g < G; g += 32) k = u64_max(k, a.s.cand[g * SR_MAX + r]);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) k = u64_max(k, shfl_xor_u64s(k, m));
  const bool failed = ld_rlx(&a.s.bar[18 * 32]) != 0u;
  if (r < a.R && l32 == 0)
    a.out_ids[r] = failed ? -2 : (k ? a.d.vocab[0xffffffffu - (uint32_t)(k & 0xffffffffu)] : -1);
}

// ---------------------------------------------------------------------------
// Phase dispatch
// ---------------------------------------------------------------------------
__device__ void run_phase(const SmallArgs& a, int p, float* red, SyncState& epoch, bool sync) {
  if (p == PH_PRE0) return ph_pre0(a, red, epoch);
  if (p == PH_PRE1) return ph_pre1(a, red, epoch, sync);
  if (p == PH_PRE2) return ph_pre2(a, red, epoch, sync);
  if (p == PH_HEAD) return ph_head(a, red, epoch, sync);
  if (p == PH_FINAL) return ph_final(a, epoch, sync);
  const int l = (p - 3) >> 3, k = (p - 3) & 7;
  const SmallBufs& s = a.s;
  const DevLayer& L = a.d.layer[l];
  switch (k) {
    case PH_SA: return ph_sa(a, l, red, epoch, sync);
    case PH_SU: return ph_su(a, l, red, epoch, sync);
    case PH_QKV: return ph_qkv(a, l, red, epoch, sync);
    case PH_ATTN: return ph_attn(a, l, red, epoch, sync);
    case PH_MERGE: return ph_merge(a, l, red, epoch, sync);
    case PH_O: return ph_resid<5>(a, L.wo, s.o[l], H, xs_in(l), xs_o(l), red, epoch, sync);
    case PH_GU: return ph_gu(a, l, red, epoch, sync);
    case PH_DOWN: return ph_resid<12>(a, L.down, s.h[l], FF, xs_o(l), xs_d(l), red, epoch, sync);
  }
}

__host__ __device__ int small_phase_count(int nl) {
  int n = 3 + 2;
  for (int l = 0; l < nl; ++l) n += l == 0 ? 6 : 8;
  return n;
}

__host__ __device__ int small_phase_id(int nl, int i) {
  if (i < 3) return i;
  i -= 3;
  for (int l = 0; l < nl; ++l) {
    const int nk = l == 0 ? 6 : 8;
    if (i < nk) return 3 + 8 * l + (l == 0 ? i + 2 : i);
    i -= nk;
  }
  return i == 0 ? PH_HEAD : PH_FINAL;
}

constexpr int RED_FLOATS = 8192 + 32 + 32;   // partial sums, inv rms, argmax candidates

// The argument block lives in device memory (read through scalar loads), so
// no per-lane copy of it is made when it is passed down to the phases.
__global__ __launch_bounds__(SMALL_WG) void k_small_phase(const SmallArgs* __restrict__ ap, int p) {
  __shared__ __attribute__((aligned(16))) float red[RED_FLOATS];
  SyncState sy{0u, 0u};
  run_phase(*ap, p, red, sy, false);
}

__global__ __launch_bounds__(SMALL_WG) void k_small_mega(const SmallArgs* __restrict__ ap) {
  __shared__ __attribute__((aligned(16))) float red[RED_FLOATS];
  __shared__ unsigned base;
  const SmallArgs& a = *ap;
  // the previous launch has finished, so the generation word is stable here
  if (threadIdx.x == 0) base = ld_rlx(&a.s.bar[17 * 32]);
  __syncthreads();
  SyncState sy{0u, base};
  const int np = small_phase_count(a.nl);
  for (int i = 0; i < np; ++i) run_phase(a, small_phase_id(a.nl, i), red, sy, i > 0);
}

void launch_small_phase(hipStream_t st, const SmallArgs* dev_args, int G, int phase) {
  k_small_phase<<<G, SMALL_WG, 0, st>>>(dev_args, phase);
}

hipError_t launch_small_mega(hipStream_t st, const SmallArgs* dev_args, int G) {
  const SmallArgs* p = dev_args;
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_small_mega), dim3(G),
                                    dim3(SMALL_WG), args, 0, st);
}

int small_mega_occupancy() {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_small_mega, SMALL_WG, 0) != hipSuccess)
    return 0;
  return occ;
}

// ---------------------------------------------------------------------------
// Buffer layout
// ---------------------------------------------------------------------------
static size_t carve(char* base, size_t& off, size_t bytes, void** out) {
  off = (off + 255) & ~(size_t)255;
  if (out) *out = base ? base + off : nullptr;
  off += bytes;
  return off;
}

static size_t small_layout(char* base, int nch, SmallBufs* s) {
  SmallBufs tmp;
  SmallBufs* o = s ? s : &tmp;
  size_t off = 0;
  const size_t F = sizeof(float);
  carve(base, off, (size_t)SB_MAX * H * F, (void**)&o->f);
  carve(base, off, (size_t)SB_MAX * H * F, (void**)&o->fce);
  carve(base, off, (size_t)3 * SB_MAX * RK * F, (void**)&o->pb);
  carve(base, off, (size_t)3 * SB_MAX * RK * F, (void**)&o->sp);
  carve(base, off, (size_t)SR_MAX * (DH / 2) * 2 * F, (void**)&o->rope);
  for (int i = 0; i < NXS; ++i) {
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->x[i]);
    carve(base, off, (size_t)SR_MAX * HT * F, (void**)&o->ssq[i]);
  }
  for (int l = 0; l < NL; ++l) {
    carve(base, off, (size_t)3 * SB_MAX * RK * F, (void**)&o->ss[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->q[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->k[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->v[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * F, (void**)&o->am[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * F, (void**)&o->al[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * DH * F, (void**)&o->ao[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->o[l]);
    carve(base, off, (size_t)SR_MAX * FF * F, (void**)&o->h[l]);
  }
  carve(base, off, (size_t)MAX_G * SR_MAX * sizeof(unsigned long long), (void**)&o->cand);
  carve(base, off, (size_t)19 * 32 * sizeof(unsigned), (void**)&o->bar);
  return (off + 255) & ~(size_t)255;
}

size_t small_bytes(int nch) { return small_layout(nullptr, nch, nullptr); }
void small_carve(char* base, int nch, SmallBufs* s) { small_layout(base, nch, s); }

}  // namespace kd
