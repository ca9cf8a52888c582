// The block-drafter round for up to 4 streams as one persistent kernel whose
// weight and context streaming is decoupled from the round's dependency chain
// (model card "Kolibri-1 block drafter", section Architecture: Input,
// Positions 2-4, Predecessor head, Spine, Body, Output).
//
// The round is the phase sequence of the small-batch path (PRE0, PRE1, PRE2,
// per layer [SA, SU,] QKV, ATTN, O, GU, DOWN, then HEAD), but each workgroup
// (one per CU) splits its waves into three roles:
//
//   waves 0..5  compute: load the activations a unit needs (after the phase
//               opens), read the unit's weights from the LDS ring, run the
//               matrix-core products and leave per-wave partial sums in LDS;
//   wave  6     streamer: copies every weight block and context K/V block the
//               workgroup will consume, in consumption order, from HBM into a
//               ring of 1 KB LDS slots (direct global-to-LDS loads), with a
//               bounded number in flight. Weights and context rows do not
//               depend on the round's activations, so the streamer runs ahead
//               of the dependency chain, across phase boundaries, limited
//               only by ring space;
//   wave  7     IO: sums the compute waves' partials in a fixed order, runs the
//               phase epilogue (RMSNorm scaling, RoPE, SwiGLU, residual adds,
//               the attention merges, the argmax), stores the results with
//               write-through stores, and runs the grid barrier that opens the
//               next phase.
//
// Roles synchronise through LDS counters only (no s_barrier after start-up),
// so the streamer never stalls on a grid barrier and the waves that wait on
// activations or store results never have weight loads queued ahead of them.
//
// Every workgroup derives the same static schedule: the units (16-row output
// tiles, 96-key attention chunks, 16-row vocab tiles) of each phase are dealt
// round-robin with an offset that carries over from phase to phase, so the
// bytes each CU streams over the round are balanced.
//
// Cross-workgroup buffers are written at most once per launch with
// write-through stores and read only after the barrier (or completion
// counter) that follows the write, so no cache holds a stale copy.
#include "kd_device.h"
#include "kd_small.h"

namespace kd {

namespace {

#define KD_CONST __attribute__((address_space(4)))
#define KD_LDS __attribute__((address_space(3)))
typedef const SmallArgsT<GlobalPtr> KD_CONST Args;
typedef const SmallBufsT<GlobalPtr> KD_CONST Bufs;
typedef const Fp8MatT<GlobalPtr> KD_CONST Mat;
template <class T> using gptr = KD_GLOBAL T*;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int WG = 512;
constexpr int NCW = 6;            // compute waves
constexpr int STREAM_WAVE = 6;       // wave 7 is the IO wave
constexpr int RING = 112;         // 1 KB LDS slots
constexpr int PASS_KB = 42;       // 64-input blocks per pass: at most 7 per compute wave
constexpr int KBW = 7;            // blocks of a pass per compute wave
constexpr int ACH = 96;           // context keys per attention unit: 16 per compute wave
constexpr int SDEPTH = 24;        // streamer blocks in flight
constexpr int PART = 576;         // floats of one wave's partial (4 x 128 + m, l)
constexpr int HEAD_KG = H / 128;  // 128-input groups of a head tile
static_assert(SDEPTH + PASS_KB + 3 <= RING, "a pass must fit in the ring beside the loads in flight");

// Pause between polls of a word in global memory (units of 64 clocks): the
// pollers of 256 workgroups must not crowd the memory channel that holds it.
constexpr int POLL_SLEEP = 8;
constexpr unsigned long long SPIN_LIMIT = 20000000ull;  // 0.2 s at the 100 MHz wall clock

enum Kind { K_PRE0, K_PRE1, K_PRE2, K_SA, K_SU, K_QKV, K_ATTN, K_O, K_GU, K_DOWN, K_HEAD };
enum Epi { E_FUSE, E_FCE, E_PB, E_ROW0, E_SP, E_ROWS, E_SA, E_SU, E_QKV, E_O, E_GU, E_DOWN };

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ const T KD_CONST& uni(const T KD_CONST& a) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(&a);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  return *reinterpret_cast<const T KD_CONST*>(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void st_wt(gptr<float> p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt64(gptr<unsigned long long> p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_rlx(gptr<unsigned> p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_rlx(gptr<unsigned> p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS control words, read and written by single lanes with LDS atomics so that
// every access is one ds instruction and never cached in registers.
__device__ __forceinline__ unsigned lds_ld(KD_LDS unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(KD_LDS unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add(KD_LDS unsigned* p, unsigned v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The same for the streamer wave, as inline assembly: the compiler treats any
// LDS access issued behind a global-to-LDS copy as a possible alias of it and
// would wait for every copy in flight; these words are never copy targets.
__device__ __forceinline__ unsigned lds_ld_asm(KD_LDS unsigned* p) {
  unsigned v;
  const unsigned addr = (unsigned)(uintptr_t)p;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_st_asm(KD_LDS unsigned* p, unsigned v) {
  const unsigned addr = (unsigned)(uintptr_t)p;
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Waits for this wave's own LDS operations (not for its global loads).
__device__ __forceinline__ void lds_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Waits until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// 8 e2m1 codes (even element in the low nibble) times an e4m3 block scale,
// exactly in f16.
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
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}
// Sum over the 16 lanes of each row of 16 (xor 1, 2, 4, 8).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int m = 1; m <= 8; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ __forceinline__ float lane_read(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// ---------------------------------------------------------------------------
// Shared LDS state
// ---------------------------------------------------------------------------
struct Lds {
  float part[2][NCW][PART];        // per-unit partials of the compute waves
  float inv[16];                   // IO: 1/rms of the rows of the current phase
  unsigned landed;                 // blocks landed in the ring (streamer)
  unsigned cons[NCW];              // ring position each compute wave has finished with
  unsigned open;                   // phases whose inputs are ready (IO)
  unsigned done[NCW];              // unit partials each compute wave has written
  unsigned freed;                  // units whose partials the IO wave has read
  unsigned fail;                   // a bounded wait expired in this workgroup
};

typedef Lds KD_LDS LdsA;

// The workgroup's LDS state, at file scope so that every role function
// addresses it with constant offsets. The ring is an object of its own: the
// compiler then knows that the streamer's control-word accesses cannot alias
// its in-flight global-to-LDS copies and does not wait for them.
__shared__ Lds g_lds;
__shared__ u32x4 g_ring[RING][64];  // weight / context blocks, 1 KB each
__device__ __forceinline__ LdsA& lds() { return *(LdsA*)&g_lds; }
typedef u32x4 KD_LDS RingSlot[64];
__device__ __forceinline__ RingSlot& ring(unsigned i) { return ((RingSlot*)g_ring)[i % RING]; }

__device__ __forceinline__ gptr<unsigned> err_word(Args& a) { return a.s.bar + 18 * 32; }

// Bounded wait on an LDS counter; on expiry sets the error flags and returns.
__device__ __forceinline__ void wait_lds_ge(Args& a, LdsA& S, KD_LDS unsigned* p, unsigned target) {
  if ((int)(lds_ld(p) - target) >= 0) return;
  // The CU's one scalar unit is shared by all its waves: a waiting wave
  // polls sparingly and looks at the clock and the failure word only every
  // 256 polls, so that the streamer's scalar work is not starved.
  unsigned long long t0 = 0;
  for (unsigned it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(2);
    if ((int)(lds_ld(p) - target) >= 0) return;
    if ((it & 255) == 0) {
      if (lds_ld(&S.fail)) return;
      const unsigned long long now = wall_clock64();
      if (t0 == 0) {
        t0 = now;
      } else if (now - t0 > SPIN_LIMIT) {
        lds_st(&S.fail, 1u);
        if ((threadIdx.x & 63) == 0)
          __hip_atomic_store(err_word(a), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The static schedule
// ---------------------------------------------------------------------------
// Activation rows feeding a projection.
struct ASrc {
  gptr<const void> base;
  int ld;        // elements per row
  int mode;      // 0: row r; 1: row r/3; 2: row 4(r/3) + r%3; 3: table row ids[r]
  gptr<const int32_t> ids;
  int kb_off;    // weight block of activation column 0
  int R;         // valid rows
  bool bf;       // bf16 rows (else fp32)
};

struct Seg {
  const Fp8MatT<GlobalPtr> KD_CONST* W;
  int nt;        // 16-row tiles
  int kb0, nkb;  // 64-input blocks of the matrix this segment reads
  int epi;
  ASrc A;
};

// Context rows of each stream, read once; kept as separate scalars (an
// indexed array would live in scratch memory).
__device__ __forceinline__ int pick4(int b, int x0, int x1, int x2, int x3) {
  return b == 0 ? x0 : (b == 1 ? x1 : (b == 2 ? x2 : x3));
}
struct StreamLens {
  int n0, n1, n2, n3;          // visible context rows min(len, window)
  int f0, f1, f2, f3;          // position of the first visible row
  int c0, c1, c2, c3;          // 96-key chunks
  int o1, o2, o3, total;       // first attention unit of streams 1..3; all units
  __device__ __forceinline__ void load(Args& a) {
    const int B = a.B, W = a.window, lane = threadIdx.x & 63;
    const int mine = a.lens[min(lane, B - 1)];
    const int l0 = __builtin_amdgcn_readlane(mine, 0);
    const int l1 = B > 1 ? __builtin_amdgcn_readlane(mine, 1) : 0;
    const int l2 = B > 2 ? __builtin_amdgcn_readlane(mine, 2) : 0;
    const int l3 = B > 3 ? __builtin_amdgcn_readlane(mine, 3) : 0;
    n0 = min(l0, W); n1 = min(l1, W); n2 = min(l2, W); n3 = min(l3, W);
    f0 = l0 - n0; f1 = l1 - n1; f2 = l2 - n2; f3 = l3 - n3;
    c0 = (n0 + ACH - 1) / ACH; c1 = (n1 + ACH - 1) / ACH;
    c2 = (n2 + ACH - 1) / ACH; c3 = (n3 + ACH - 1) / ACH;
    o1 = NH * c0;
    o2 = o1 + NH * c1;
    o3 = o2 + NH * c2;
    total = o3 + NH * c3;
  }
  __device__ __forceinline__ int vis(int b) const { return pick4(b, n0, n1, n2, n3); }
  __device__ __forceinline__ int first(int b) const { return pick4(b, f0, f1, f2, f3); }
  __device__ __forceinline__ int nch(int b) const { return pick4(b, c0, c1, c2, c3); }
  // attention unit u -> stream b, head h, chunk c (the chunks of one
  // (stream, head) are consecutive units); a stream without units shares its
  // offset with the next one, which then wins
  __device__ __forceinline__ void unit(int u, int& b, int& h, int& c) const {
    b = u >= o3 ? 3 : (u >= o2 ? 2 : (u >= o1 ? 1 : 0));
    const int loc = u - pick4(b, 0, o1, o2, o3);
    const int nc = nch(b);
    h = loc / nc;
    c = loc - h * nc;
  }
};

// A phase as scalars; its segments are built on demand (no array of
// segments, which would live in scratch memory).
struct Phase {
  int kind, l;
  int nseg, nt0, nt1;  // segments and the tiles of the first two
  int U;               // units of the phase over the whole grid
};

__device__ __forceinline__ ASrc asrc(gptr<const void> base, int ld, int mode, gptr<const int32_t> ids,
                                     int kb_off, int R, bool bf) {
  ASrc s;
  s.base = base; s.ld = ld; s.mode = mode; s.ids = ids; s.kb_off = kb_off; s.R = R; s.bf = bf;
  return s;
}
__device__ __forceinline__ Seg seg(Mat& W, int kb0, int nkb, int epi, ASrc A) {
  Seg s;
  s.W = &W; s.nt = W.N / 16; s.kb0 = kb0; s.nkb = nkb; s.epi = epi; s.A = A;
  return s;
}

__device__ __forceinline__ int stream_phase_count(int nl) {
  int n = 3 + 1;
  for (int l = 0; l < nl; ++l) n += l == 0 ? 5 : 7;
  return n;
}

// Phase i of the round (same order as the small-batch path).
__device__ __forceinline__ Phase make_phase(Args& a, int i, const StreamLens& sl) {
  Phase p;
  p.nseg = 1;
  p.l = 0;
  p.nt1 = 0;
  if (i == 0) {
    p.kind = K_PRE0;
    p.nseg = 3;
    p.nt0 = H / 16;
    p.nt1 = H / 16;
    p.U = H / 16 + H / 16 + RK / 16;
  } else if (i == 1) {
    p.kind = K_PRE1;
    p.nseg = 2;
    p.nt0 = H / 16;
    p.U = H / 16 + RK / 16;
  } else if (i == 2) {
    p.kind = K_PRE2;
    p.nt0 = p.U = H / 16;
  } else {
    int j = i - 3, l = 0, k = -1;
    for (; l < a.nl; ++l) {
      const int nk = l == 0 ? 5 : 7;
      if (j < nk) { k = l == 0 ? j + 2 : j; break; }
      j -= nk;
    }
    p.l = l;
    switch (k) {
      case 0: p.kind = K_SA; p.nt0 = RK / 16; break;
      case 1: p.kind = K_SU; p.nt0 = H / 16; break;
      case 2: p.kind = K_QKV; p.nt0 = QKV / 16; break;
      case 3: p.kind = K_ATTN; p.nt0 = sl.total; break;
      case 4: p.kind = K_O; p.nt0 = H / 16; break;
      case 5: p.kind = K_GU; p.nt0 = GU / 16; break;
      case 6: p.kind = K_DOWN; p.nt0 = H / 16; break;
      default: p.kind = K_HEAD; p.nt0 = a.d.VT; break;
    }
    p.U = p.nt0;
  }
  return p;
}

// Segment sg of a projection phase.
__device__ __forceinline__ Seg phase_seg(Args& a, const Phase& p, int sg) {
  auto& d = a.d;
  auto& s = a.s;
  const int B = a.B, R = a.R, l = p.l;
  switch (p.kind) {
    case K_PRE0:
      if (sg == 0) return seg(d.fuse, 0, NTAP * H / 64, E_FUSE, asrc(a.taps, NTAP * H, 0, nullptr, 0, B, true));
      if (sg == 1) return seg(d.fc, H / 64, H / 64, E_FCE, asrc(d.table, H, 3, a.anchor, H / 64, B, true));
      return seg(d.pred_ab, H / 64, H / 64, E_PB, asrc(d.table, H, 3, a.pred, H / 64, 3 * B, true));
    case K_PRE1:
      if (sg == 0) return seg(d.fc, 0, H / 64, E_ROW0, asrc(s.f, H, 0, nullptr, 0, B, false));
      return seg(d.pred_ab, 0, H / 64, E_SP, asrc(s.f, H, 1, nullptr, 0, 3 * B, false));
    case K_PRE2:
      return seg(d.pred_u, 0, RK / 64, E_ROWS, asrc(s.sp, RK, 0, nullptr, 0, 3 * B, false));
    case K_SA:
      return seg(d.layer[l].sa, 0, H / 64, E_SA, asrc(s.xg[xs_d(l - 1)], H, 2, nullptr, 0, 3 * B, false));
    case K_SU:
      return seg(d.layer[l].su, 0, RK / 64, E_SU, asrc(s.ss[l], RK, 0, nullptr, 0, 3 * B, false));
    case K_QKV:
      return seg(d.layer[l].qkv, 0, H / 64, E_QKV, asrc(s.xg[xs_in(l)], H, 0, nullptr, 0, R, false));
    case K_O:
      return seg(d.layer[l].wo, 0, H / 64, E_O, asrc(s.o[l], H, 0, nullptr, 0, R, false));
    case K_GU:
      return seg(d.layer[l].gu, 0, H / 64, E_GU, asrc(s.xg[xs_o(l)], H, 0, nullptr, 0, R, false));
    default:
      return seg(d.layer[l].down, 0, FF / 64, E_DOWN, asrc(s.h[l], FF, 0, nullptr, 0, R, false));
  }
}

// Unit k of a projection phase -> segment and tile.
__device__ __forceinline__ void proj_unit(const Phase& p, int k, int& sg, int& t) {
  sg = 0;
  t = k;
  if (p.nseg > 1 && t >= p.nt0) {
    t -= p.nt0;
    sg = 1;
    if (p.nseg > 2 && t >= p.nt1) {
      t -= p.nt1;
      sg = 2;
    }
  }
}

// Passes of a unit with nkb blocks: each at most PASS_KB blocks.
__device__ __forceinline__ int npass(int nkb) { return (nkb + PASS_KB - 1) / PASS_KB; }
__device__ __forceinline__ void pass_range(int nkb, int q, int& j0, int& pk) {
  const int np = npass(nkb), full = (nkb + np - 1) / np;
  j0 = q * full;
  pk = min(nkb - j0, full);
}
__device__ __forceinline__ int pass_blocks(int pk) { return pk + (pk + 15) / 16; }

// This workgroup's first unit of a phase with U units dealt from offset rot.
__device__ __forceinline__ int first_unit(int rot) {
  const int G = gridDim.x;
  return ((int)blockIdx.x - rot + G) % G;
}

// Grid barrier: two-level counters (groups of 16 workgroups) and a generation
// word; counters only grow, so nothing is reset. Called by the IO wave.
__device__ __forceinline__ void grid_barrier(Args& a, LdsA& S, unsigned target) {
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    auto bar = a.s.bar;
    const unsigned G = gridDim.x, grp = blockIdx.x >> 4, ngrp = (G + 15) >> 4;
    const unsigned gsize = min(16u, G - grp * 16);
    const unsigned v = add_rlx(&bar[grp * 32], 1u);
    if ((v + 1) % gsize == 0) {
      const unsigned w = add_rlx(&bar[16 * 32], 1u);
      if ((w + 1) % ngrp == 0)
        __hip_atomic_store(&bar[17 * 32], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const unsigned long long t0 = wall_clock64();
    for (unsigned it = 1; (int)(ld_rlx(&bar[17 * 32]) - target) < 0; ++it) {
      if ((it & 63) == 0 && (wall_clock64() - t0 > SPIN_LIMIT || ld_rlx(err_word(a)) != 0u)) {
        __hip_atomic_store(err_word(a), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_st(&S.fail, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
    }
  }
}

__device__ __forceinline__ void trace_mark(Args& a, int ph, int k) {
  if (a.trace && (threadIdx.x & 63) == 0 && ph < a.trace_phases)
    a.trace[((size_t)ph * gridDim.x + blockIdx.x) * 8 + k] = wall_clock64();
}

// ---------------------------------------------------------------------------
// Streamer wave
// ---------------------------------------------------------------------------
// The streamer's state is wave-uniform and lives in scalar registers; the
// common path of issue() is one copy, a counter update and a vmcnt wait.
struct Streamer {
  Args& a;
  LdsA& S;
  unsigned pos;        // blocks issued
  unsigned slot;       // pos % RING
  unsigned limit;      // pos may grow to limit before the ring needs checking
  unsigned long long stall;  // wall-clock ticks spent waiting for ring space (tracing)

  // lane 0 writes the landed count
  __device__ __forceinline__ void publish(unsigned v) {
    const unsigned addr = (unsigned)(uintptr_t)&S.landed;
    unsigned long long saved;
    asm volatile(
        "s_mov_b64 %0, exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "ds_write_b32 %1, %2\n\t"
        "s_mov_b64 exec, %0"
        : "=&s"(saved)
        : "v"(addr), "v"(v)
        : "memory");
  }
  // Minimum consumer position: lanes 0..NCW-1 read one word each (one LDS
  // instruction), then a scalar minimum over those lanes.
  __device__ __forceinline__ unsigned cons_min() {
    const int lane = threadIdx.x & 63;
    const unsigned c = lds_ld_asm(&S.cons[min(lane, NCW - 1)]);
    unsigned m = (unsigned)__builtin_amdgcn_readlane((int)c, 0);
#pragma unroll
    for (int w = 1; w < NCW; ++w) {
      const unsigned cw = (unsigned)__builtin_amdgcn_readlane((int)c, w);
      if ((int)(cw - m) < 0) m = cw;
    }
    return m;
  }
  // pos reached limit: first look again at the consumers; only if the ring is
  // really full, let everything issued land, publish it and wait for space.
  __device__ __forceinline__ void wait_space() {
    limit = cons_min() + RING;
    if ((int)(limit - pos) > 0) return;
    wait_vm<0>();
    publish(pos);
    const unsigned long long t0 = wall_clock64();
    for (unsigned it = 1;; ++it) {
      __builtin_amdgcn_s_sleep(1);
      limit = cons_min() + RING;
      if ((int)(limit - pos) > 0) break;
      if ((it & 63) == 0 && (uni((int)lds_ld_asm(&S.fail)) || wall_clock64() - t0 > SPIN_LIMIT)) {
        lds_st_asm(&S.fail, 1u);
        __hip_atomic_store(err_word(a), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        limit = pos + RING;  // give up waiting; the round is already marked failed
        break;
      }
    }
    stall += wall_clock64() - t0;
  }
  // Issues one 1 KB block; lane l copies 16 bytes from src (per lane).
  __device__ __forceinline__ void issue(gptr<const void> src) {
    if (pos == limit) wait_space();
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                     (KD_LDS void*)&g_ring[slot][0], 16, 0, 0);
    ++pos;
    slot = slot + 1 == RING ? 0u : slot + 1;
    // at most SDEPTH copies in flight: every block before pos - SDEPTH has landed
    wait_vm<SDEPTH>();
    if ((pos & 7) == 0) {
      if (pos > SDEPTH) publish(pos - SDEPTH);
      // keep the ring limit fresh so that reaching it is rare
      if ((pos & 15) == 0) limit = cons_min() + RING;
    }
  }
  __device__ void flush() {
    wait_vm<0>();
    publish(pos);
  }
};

__device__ __forceinline__ void stream_proj_unit(Streamer& st, const Seg& sg, int t) {
  const int lane = threadIdx.x & 63;
  Mat& W = *sg.W;
  const int KB = W.K >> 6;
  const int np = npass(sg.nkb);
  for (int q = 0; q < np; ++q) {
    int j0, pk;
    pass_range(sg.nkb, q, j0, pk);
    const size_t blk0 = (size_t)t * KB + sg.kb0 + j0;
    gptr<const uint8_t> pw = W.w + blk0 * 1024 + lane * 16;
#pragma unroll 1
    for (int j = 0; j < pk; ++j, pw += 1024) st.issue(pw);
    // scales of the pass: pk x 16 floats, contiguous (the allocation is padded
    // so the last 1 KB chunk may run past the matrix)
    const int nsc = (pk + 15) / 16;
    gptr<const uint8_t> ps = reinterpret_cast<gptr<const uint8_t>>(W.s + blk0 * 16) + lane * 16;
#pragma unroll 1
    for (int c = 0; c < nsc; ++c, ps += 1024) st.issue(ps);
  }
}

// The K and V blocks of one 96-key chunk: for key group g (16 keys) four K
// blocks in matrix-core A-operand order (lane: key g*16 + l%16, dims
// 32 ks + 8 (l/16) .. +8) and four V blocks of 4 keys x 128 dims row-major.
// Keys past the visible rows repeat the last visible one (masked later).
__device__ __forceinline__ void stream_attn_unit(Streamer& st, int l, const StreamLens& sl, int u) {
  Args& a = st.a;
  const int lane = threadIdx.x & 63;
  int b, h, c;
  sl.unit(u, b, h, c);
  const int n = sl.vis(b), fp = sl.first(b), cap = a.kv.cap;
  auto kb = a.kv.k[l] + b * a.kv.ss + h * a.kv.sh;
  auto vb = a.kv.v[l] + b * a.kv.ss + h * a.kv.sh;
  const long long sls = a.kv.sl;
  for (int g = 0; g < NCW; ++g) {
    {
      const int key = min(c * ACH + g * 16 + (lane & 15), n - 1);
      const int slot = (fp + key) % cap;
      auto p = kb + (size_t)slot * sls + 8 * (lane >> 4);
#pragma unroll 1
      for (int ks = 0; ks < 4; ++ks) st.issue(p + 32 * ks);
    }
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
      const int key = min(c * ACH + g * 16 + 4 * j + (lane >> 4), n - 1);
      const int slot = (fp + key) % cap;
      st.issue(vb + (size_t)slot * sls + 8 * (lane & 15));
    }
  }
}

// One vocab tile: 20 code blocks then 5 scale blocks.
__device__ __forceinline__ void stream_head_unit(Streamer& st, int vt) {
  Args& a = st.a;
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)vt * HEAD_KG * 64;
  gptr<const uint8_t> pq = a.d.hq + base * 16 + lane * 16;
#pragma unroll 1
  for (int g = 0; g < HEAD_KG; ++g, pq += 1024) st.issue(pq);
  gptr<const uint8_t> ps = a.d.hs + base * 4 + lane * 16;
#pragma unroll 1
  for (int c = 0; c < HEAD_KG * 64 * 4 / 1024; ++c, ps += 1024) st.issue(ps);
}

__device__ __attribute__((noinline, not_tail_called)) void role_stream(Args& a_, int np_) {
  Args& a = uni(a_);
  LdsA& S = lds();
  const int np = uni(np_);
  StreamLens sl;
  sl.load(a);
  Streamer st{a, S, 0u, 0u, (unsigned)RING, 0ull};
  const int G = gridDim.x;
  int rot = 0;
  for (int i = 0; i < np; ++i) {
    const Phase p = make_phase(a, i, sl);
    // trace rows 32 + i: phase start, ring-full stall so far, blocks issued.
    // (A store counted among the copies in flight only makes the landed
    // count the streamer publishes more conservative.)
    if (a.trace && (threadIdx.x & 63) == 0 && 32 + i < a.trace_phases) {
      auto tr = a.trace + ((size_t)(32 + i) * gridDim.x + blockIdx.x) * 8;
      tr[0] = wall_clock64();
      tr[1] = st.stall;
      tr[2] = st.pos;
    }
    for (int k = first_unit(rot); k < p.U; k += G) {
      if (p.kind == K_ATTN) {
        stream_attn_unit(st, p.l, sl, k);
      } else if (p.kind == K_HEAD) {
        stream_head_unit(st, k);
      } else {
        int sg, t;
        proj_unit(p, k, sg, t);
        stream_proj_unit(st, phase_seg(a, p, sg), t);
      }
    }
    rot = (rot + p.U) % G;
  }
  st.flush();
}

// ---------------------------------------------------------------------------
// Compute waves
// ---------------------------------------------------------------------------
struct Compute {
  Args& a;
  LdsA& S;
  int w;               // compute wave index
  int phase;           // current phase (tracing)
  unsigned pos;        // ring position
  unsigned useq;       // units completed
};

// Activation fragments of one pass for this wave: per local block, hi and lo
// of k-tile 0, then hi and lo of k-tile 1.
typedef bf16x8 Frag[KBW][4];

__device__ __forceinline__ size_t a_row(const ASrc& A, int r) {
  switch (A.mode) {
    case 1: return (size_t)(r / 3);
    case 2: return (size_t)(4 * (r / 3) + r % 3);
    case 3: return (size_t)A.ids[r];
    default: return (size_t)r;
  }
}

// Loads this wave's activation fragments for a pass: local blocks
// j = w, w + NCW, ... < pk of the pass starting at block kb_start. Loads go out
// in two groups so that at most 4 blocks of raw fp32 values are live.
__device__ __forceinline__ void load_act(Frag& ah, int w, const ASrc& A, int kb_start, int pk) {
  const int lane = threadIdx.x & 63;
  const int r = min(lane & 15, A.R - 1);
  const size_t row = a_row(A, r);
#pragma unroll
  for (int i0 = 0; i0 < KBW; i0 += 4) {
    u32x4 raw[4][4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = i0 + ii;
      if (i >= KBW) break;
      const int j = min(w + NCW * i, pk - 1);
      const int c0 = (kb_start + j - A.kb_off) * 64 + 8 * (lane >> 4);
      if (A.bf) {
        auto pa = static_cast<gptr<const uint16_t>>(A.base) + row * A.ld + c0;
        raw[ii][0] = *reinterpret_cast<gptr<const u32x4>>(pa);
        raw[ii][1] = *reinterpret_cast<gptr<const u32x4>>(pa + 32);
      } else {
        auto pa = static_cast<gptr<const float>>(A.base) + row * A.ld + c0;
        raw[ii][0] = *reinterpret_cast<gptr<const u32x4>>(pa);
        raw[ii][1] = *reinterpret_cast<gptr<const u32x4>>(pa + 4);
        raw[ii][2] = *reinterpret_cast<gptr<const u32x4>>(pa + 32);
        raw[ii][3] = *reinterpret_cast<gptr<const u32x4>>(pa + 36);
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = i0 + ii;
      if (i >= KBW) break;
      if (A.bf) {
        const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        ah[i][0] = __builtin_bit_cast(bf16x8, raw[ii][0]);
        ah[i][2] = __builtin_bit_cast(bf16x8, raw[ii][1]);
        ah[i][1] = z;
        ah[i][3] = z;
      } else {
        float v0[8], v1[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = u2f(raw[ii][0][e]);
          v0[4 + e] = u2f(raw[ii][1][e]);
          v1[e] = u2f(raw[ii][2][e]);
          v1[4 + e] = u2f(raw[ii][3][e]);
        }
        split_bf16(v0, ah[i][0], ah[i][1]);
        split_bf16(v1, ah[i][2], ah[i][3]);
      }
    }
  }
}

// Waits for the unit's partial buffer, writes this wave's partial, counts it.
__device__ __forceinline__ KD_LDS float* part_begin(Compute& cw) {
  // the IO wave has read the partials of unit useq - 2 (same buffer)
  if (cw.useq >= 2) wait_lds_ge(cw.a, cw.S, &cw.S.freed, cw.useq - 1);
  return reinterpret_cast<KD_LDS float*>(&cw.S.part[cw.useq & 1][cw.w][0]);
}
__device__ __forceinline__ void part_end(Compute& cw) {
  lds_done();
  ++cw.useq;
  if ((threadIdx.x & 63) == 0) lds_st(&cw.S.done[cw.w], cw.useq);
}
__device__ __forceinline__ void release(Compute& cw, unsigned upto) {
  lds_done();
  if ((threadIdx.x & 63) == 0) lds_st(&cw.S.cons[cw.w], upto);
}

__device__ __forceinline__ void compute_proj_unit(Compute& cw, Frag& ah, int& cache_key, const Seg& sg,
                                                  int segkey, int t) {
  const int lane = threadIdx.x & 63;
  const int np = npass(sg.nkb);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < np; ++q) {
    int j0, pk;
    pass_range(sg.nkb, q, j0, pk);
    const int key = segkey * 8 + q;
    if (cache_key != key) {
      load_act(ah, cw.w, sg.A, sg.kb0 + j0, pk);
      cache_key = key;
    }
    const unsigned p0 = cw.pos;
    wait_lds_ge(cw.a, cw.S, &cw.S.landed, p0 + pass_blocks(pk));
    if (cw.w == 0 && q == 0) trace_mark(cw.a, cw.phase, 5);
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      const int j = cw.w + NCW * i;
      if (j < pk) {
        const u32x4 wv = ring(p0 + j)[lane];
        const unsigned sb = p0 + pk + (j >> 4);
        const float sc = reinterpret_cast<KD_LDS const float*>(&ring(sb)[0])
            [(j & 15) * 16 + (lane & 15)];
        const bf16x8 w0 = e4m3x8_bf16(wv.x, wv.y);
        const bf16x8 w1 = e4m3x8_bf16(wv.z, wv.w);
        f32x4 tt = {0.f, 0.f, 0.f, 0.f};
        tt = mfma_bf16(ah[i][0], w0, tt);
        tt = mfma_bf16(ah[i][1], w0, tt);
        tt = mfma_bf16(ah[i][2], w1, tt);
        tt = mfma_bf16(ah[i][3], w1, tt);
        acc += sc * tt;
      }
    }
    cw.pos = p0 + pass_blocks(pk);
    release(cw, cw.pos);
  }
  KD_LDS float* pp = part_begin(cw);
  *reinterpret_cast<KD_LDS f32x4*>(pp + lane * 4) = acc;
  part_end(cw);
}

// One 96-key chunk for one (stream, head): this wave takes key group g = w.
__device__ __forceinline__ void compute_attn_unit(Compute& cw, int l, const StreamLens& sl, int u, const float (&qf)[4][8],
                                  bool qvalid) {
  Args& a = cw.a;
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  int b, h, c;
  sl.unit(u, b, h, c);
  const int n = sl.vis(b);
  const unsigned p0 = cw.pos;
  const unsigned gb = p0 + 8 * cw.w;  // this wave's 8 blocks
  wait_lds_ge(a, cw.S, &cw.S.landed, gb + 8);
  // scores S^T[key][j] = K Q^T: K rows as A, queries (hi, lo) as B
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 qh, ql;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qvalid ? qf[ks][e] : 0.f;
    split_bf16(qv, qh, ql);
    const bf16x8 kk = __builtin_bit_cast(bf16x8, ring(gb + ks)[lane]);
    acc = mfma_bf16(kk, qh, acc);
    acc = mfma_bf16(kk, ql, acc);
  }
  // lane holds S^T[key 4 lg + e][j = lr]; softmax over the wave's 16 keys
  float sc[4], mx = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = c * ACH + cw.w * 16 + 4 * lg + e;
    sc[e] = key < n ? acc[e] : -__builtin_inff();
    mx = fmaxf(mx, sc[e]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float pe[4], ls = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pe[e] = sc[e] == -__builtin_inff() ? 0.f : exp2f(sc[e] - mx);
    ls += pe[e];
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  // P V on the vector units: lane owns dims 2 lane, 2 lane + 1 of 4 rows;
  // p[key][j] lives in lane 16 (key / 4) + j, element key % 4
  float o[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j][0] = o[j][1] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const uint32_t vv = reinterpret_cast<KD_LDS const uint32_t*>(&ring(gb + 4 + (kk >> 2))[0])
        [(kk & 3) * 64 + lane];
    const float v0 = u2f(vv << 16), v1 = u2f(vv & 0xffff0000u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = lane_read(pe[kk & 3], 16 * (kk >> 2) + j);
      o[j][0] += pj * v0;
      o[j][1] += pj * v1;
    }
  }
  cw.pos = p0 + 8 * NCW;
  release(cw, cw.pos);
  KD_LDS float* pp = part_begin(cw);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<KD_LDS f32x2*>(pp + j * DH + 2 * lane) = f32x2{o[j][0], o[j][1]};
  if (lane < 4) {
    pp[512 + lane] = mx;
    pp[516 + lane] = ls;
  }
  part_end(cw);
}

// Queries of (stream b, head h) as this lane's B-operand values (column j =
// lane % 16 < 4), pre-scaled by 1/sqrt(128) * log2(e).
__device__ __forceinline__ void load_q(Args& a, int l, int b, int h, float (&qf)[4][8]) {
  const int lane = threadIdx.x & 63;
  const int j = min(lane & 15, 3);
  const float qs = 0.08838834764831845f * 1.4426950408889634f;
  auto p = a.s.q[l] + (b * 4 + j) * H + h * DH + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f32x4 x0 = *reinterpret_cast<gptr<const f32x4>>(p + 32 * ks);
    const f32x4 x1 = *reinterpret_cast<gptr<const f32x4>>(p + 32 * ks + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[ks][e] = x0[e] * qs;
      qf[ks][4 + e] = x1[e] * qs;
    }
  }
}

// One 16-row vocab tile: this wave takes the 128-input groups g = w, w + 6, ...
__device__ __forceinline__ void compute_head_unit(Compute& cw, const f16x8 (&zh)[4][4], const f16x8 (&zl)[4][4]) {
  const int lane = threadIdx.x & 63;
  const unsigned p0 = cw.pos;
  wait_lds_ge(cw.a, cw.S, &cw.S.landed, p0 + HEAD_KG + 5);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = cw.w + NCW * i;
    if (g < HEAD_KG) {
      const u32x4 qv = ring(p0 + g)[lane];
      const uint32_t sv = reinterpret_cast<KD_LDS const uint32_t*>(
          &ring(p0 + HEAD_KG + (g >> 2))[0])[(g & 3) * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x8 wv = nvfp4x8_f16(qv[t], sv >> (8 * t));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zh[i][t], wv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(zl[i][t], wv, acc, 0, 0, 0);
      }
    }
  }
  cw.pos = p0 + HEAD_KG + 5;
  release(cw, cw.pos);
  KD_LDS float* pp = part_begin(cw);
  *reinterpret_cast<KD_LDS f32x4*>(pp + lane * 4) = acc;
  part_end(cw);
}

__device__ __attribute__((noinline, not_tail_called)) void role_compute(Args& a_, int np_, int w_) {
  Args& a = uni(a_);
  LdsA& S = lds();
  const int np = uni(np_), w = uni(w_);
  StreamLens sl;
  sl.load(a);
  Compute cw{a, S, w, 0, 0u, 0u};
  const int G = gridDim.x, lane = threadIdx.x & 63;
  int rot = 0;
  for (int i = 0; i < np; ++i) {
    const Phase p = make_phase(a, i, sl);
    if (i > 0) wait_lds_ge(a, S, &S.open, (unsigned)i + 1u);
    if (w == 0) trace_mark(a, i, 2);
    cw.phase = i;
    const int k0 = first_unit(rot);
    if (p.kind == K_ATTN) {
      float qf[4][8], qn[4][8];
      int bc = -1, hc = -1;
      if (k0 < p.U) {
        int b, h, c;
        sl.unit(k0, b, h, c);
        load_q(a, p.l, b, h, qf);
        bc = b; hc = h;
      }
      for (int k = k0; k < p.U; k += G) {
        // queries of the next unit, if it is another (stream, head)
        int bn = bc, hn = hc;
        if (k + G < p.U) {
          int c;
          sl.unit(k + G, bn, hn, c);
          if (bn != bc || hn != hc) load_q(a, p.l, bn, hn, qn);
        }
        compute_attn_unit(cw, p.l, sl, k, qf, (lane & 15) < 4);
        if (bn != bc || hn != hc) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = qn[ks][e];
          bc = bn; hc = hn;
        }
      }
    } else if (p.kind == K_HEAD) {
      // the final residual stage times the final gain, as f16 hi + lo, for
      // this wave's input groups; kept for every unit of the phase
      f16x8 zh[4][4], zl[4][4];
      const int src = a.nl == 0 ? 0 : xs_d(a.nl - 1);
      const int r = min(lane & 15, a.R - 1);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int g = min(w + NCW * ii, HEAD_KG - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          auto pz = a.s.xg[src] + r * H + g * 128 + t * 32 + 8 * (lane >> 4);
          const f32x4 x0 = *reinterpret_cast<gptr<const f32x4>>(pz);
          const f32x4 x1 = *reinterpret_cast<gptr<const f32x4>>(pz + 4);
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[e] = x0[e]; v[4 + e] = x1[e]; }
          split_f16(v, zh[ii][t], zl[ii][t]);
        }
      }
      for (int k = k0; k < p.U; k += G) compute_head_unit(cw, zh, zl);
    } else {
      Frag ah;
      int cache_key = -1;  // activations are new in every phase
      for (int k = k0; k < p.U; k += G) {
        int sg, t;
        proj_unit(p, k, sg, t);
        compute_proj_unit(cw, ah, cache_key, phase_seg(a, p, sg), sg, t);
      }
    }
    if (w == 0) trace_mark(a, i, 3);
    rot = (rot + p.U) % G;
  }
}

// ---------------------------------------------------------------------------
// IO wave
// ---------------------------------------------------------------------------
struct IO {
  Args& a;
  LdsA& S;
  unsigned useq;
  unsigned long long best[4];  // running argmax keys of this lane's rows (head)
};

// Waits until every compute wave has written its partial of unit useq.
__device__ __forceinline__ void io_wait_done(Args& a, LdsA& S, unsigned useq) {
  const int lane = threadIdx.x & 63;
  const unsigned target = useq + 1;
  auto ready = [&]() {
    const unsigned d = lds_ld(&S.done[min(lane, NCW - 1)]);
    return __all((int)(d - target) >= 0);
  };
  if (ready()) return;
  unsigned long long t0 = 0;
  for (unsigned it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(2);
    if (ready()) return;
    if ((it & 255) == 0) {
      if (lds_ld(&S.fail)) return;
      const unsigned long long now = wall_clock64();
      if (t0 == 0) {
        t0 = now;
      } else if (now - t0 > SPIN_LIMIT) {
        lds_st(&S.fail, 1u);
        if (lane == 0) __hip_atomic_store(err_word(a), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
  }
}

// Waits for all compute waves' partials of the next unit and returns them
// summed in wave order (a projection unit: the lane's 4 accumulator values).
__device__ __forceinline__ f32x4 io_take_proj(IO& io) {
  const int lane = threadIdx.x & 63;
  io_wait_done(io.a, io.S, io.useq);
  KD_LDS float* base = &io.S.part[io.useq & 1][0][0];
  f32x4 v = *reinterpret_cast<KD_LDS f32x4*>(base + lane * 4);
#pragma unroll
  for (int w = 1; w < NCW; ++w) v += *reinterpret_cast<KD_LDS f32x4*>(base + w * PART + lane * 4);
  lds_done();
  if ((threadIdx.x & 63) == 0) lds_st(&io.S.freed, io.useq + 1);
  ++io.useq;
  return v;
}

// 1/rms of R rows of a residual stage (per-tile sums of squares), into S.inv.
// mode 2 takes rows 4(r/3) + r%3 for r < nrows.
__device__ __forceinline__ void io_inv_rms(IO& io, gptr<const float> ssq, int nrows, int mode) {
  const int lane = threadIdx.x & 63;
  const int r = lane >> 2, qd = lane & 3;  // 16 rows x 4 quarters of 40 tiles
  const int rr = min(r, nrows - 1);
  const int row = mode == 2 ? 4 * (rr / 3) + rr % 3 : rr;
  auto p = ssq + (size_t)row * HT + qd * 40;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const f32x4 v = *reinterpret_cast<gptr<const f32x4>>(p + 4 * i);
    s += (v.x + v.y) + (v.z + v.w);
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  if (qd == 0) io.S.inv[r] = 1.0f / sqrtf(s / H + io.a.eps);
  lds_done();
}

// Residual-stage store of one lane's 4 rows at column col of tile `tile`:
// raw x, the copy times the consumer's gain and the tile's sum of squares.
__device__ __forceinline__ void put_x4(Bufs& s, int stage, gptr<const float> gain, const int (&row)[4],
                                       int col, int tile, const float (&x)[4], const bool (&ok)[4]) {
  const int n = threadIdx.x & 15;
  const float g = gain[col];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float q = row16_sum(x[e] * x[e]);
    if (ok[e]) {
      st_wt(&s.x[stage][row[e] * H + col], x[e]);
      st_wt(&s.xg[stage][row[e] * H + col], x[e] * g);
      if (n == 0) st_wt(&s.ssq[stage][row[e] * HT + tile], q);
    }
  }
}

__device__ __forceinline__ gptr<const float> gain_in(Args& a, int l) {
  return l < a.nl ? a.d.layer[l].attn_norm : a.d.final_norm;
}
__device__ __forceinline__ gptr<const float> gain_after_down(Args& a, int l) {
  return l + 1 < a.nl ? a.d.layer[l + 1].spine_norm : a.d.final_norm;
}

// Epilogue of one projection tile; v[e] is row 4 (lane / 16) + e, column
// 16 t + lane % 16 of the segment's matrix.
__device__ __forceinline__ void io_proj_epilogue(IO& io, const Phase& p, const Seg& sg, int t, const f32x4 v) {
  Args& a = io.a;
  auto& s = a.s;
  auto& d = a.d;
  const int lane = threadIdx.x & 63, n = lane & 15, m0 = 4 * (lane >> 4);
  const int B = a.B, R = a.R, l = p.l;
  const int col = t * 16 + n;
  switch (sg.epi) {
    case E_FUSE:
    case E_FCE: {
      gptr<float> dst = sg.epi == E_FUSE ? s.f : s.fce;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (m0 + e < B) st_wt(&dst[(m0 + e) * H + col], v[e]);
      break;
    }
    case E_PB:
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (m0 + e < 3 * B) st_wt(&s.pb[(m0 + e) * RK + col], v[e]);
      break;
    case E_SP:
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (m0 + e < 3 * B) {
          const int m = m0 + e;
          st_wt(&s.sp[m * RK + col], silu(v[e] + s.pb[m * RK + col]));
        }
      break;
    case E_ROW0: {
      int row[4];
      float x[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + e;
        ok[e] = m < B;
        row[e] = 4 * min(m, B - 1);
        x[e] = ok[e] ? v[e] + s.fce[m * H + col] : 0.f;
      }
      put_x4(s, 0, gain_in(a, 0), row, col, t, x, ok);
      break;
    }
    case E_ROWS: {
      int row[4];
      float x[4];
      bool ok[4];
      const float mk = d.mask[col];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = min(m0 + e, 3 * B - 1);
        ok[e] = m0 + e < 3 * B;
        row[e] = 4 * (m / 3) + m % 3 + 1;
        x[e] = ok[e] ? mk + s.f[(m / 3) * H + col] + v[e] : 0.f;
      }
      put_x4(s, 0, gain_in(a, 0), row, col, t, x, ok);
      break;
    }
    case E_SA:
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (m0 + e < 3 * B) {
          const int m = m0 + e;
          st_wt(&s.ss[l][m * RK + col], silu(v[e] * io.S.inv[m]));
        }
      break;
    case E_SU: {
      const int src = xs_d(l - 1), dst = xs_in(l);
      auto gain = gain_in(a, l);
      int row[4];
      float x[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = min(m0 + e, 3 * B - 1);
        ok[e] = m0 + e < 3 * B;
        row[e] = 4 * (m / 3) + m % 3 + 1;
        x[e] = ok[e] ? s.x[src][row[e] * H + col] + v[e] : 0.f;
      }
      put_x4(s, dst, gain, row, col, t, x, ok);
      // row 0 of every stream is untouched by the spine: copied, with its
      // sum of squares
      if (lane < 16 * B) {
        const int b = lane >> 4, r0 = 4 * b;
        const float x0 = s.x[src][r0 * H + col];
        st_wt(&s.x[dst][r0 * H + col], x0);
        st_wt(&s.xg[dst][r0 * H + col], x0 * gain[col]);
        if (n == 0) st_wt(&s.ssq[dst][r0 * HT + t], s.ssq[src][r0 * HT + t]);
      }
      break;
    }
    case E_QKV: {
      const int sec = t / HT;
      const int nat = qkv_natural(col) - sec * H;  // column within q, k or v
      gptr<float> dstp = sec == 0 ? s.q[l] : (sec == 1 ? s.k[l] : s.v[l]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + e;
        const float val = m < R ? v[e] * io.S.inv[m] : 0.f;
        const float partner = __shfl_xor(val, 8, 64);
        float out = val;
        if (sec < 2) {
          const int fi = (nat % DH) & 63;
          const int mm = min(m, R - 1);
          const float cs = s.rope[(mm * (DH / 2) + fi) * 2];
          const float sn = s.rope[(mm * (DH / 2) + fi) * 2 + 1];
          out = n < 8 ? val * cs - partner * sn : partner * sn + val * cs;
        }
        if (m < R) st_wt(&dstp[m * H + nat], out);
      }
      break;
    }
    case E_O:
    case E_DOWN: {
      const int xin = sg.epi == E_O ? xs_in(l) : xs_o(l);
      const int xout = sg.epi == E_O ? xs_o(l) : xs_d(l);
      auto gain = sg.epi == E_O ? d.layer[l].ffn_norm : gain_after_down(a, l);
      int row[4];
      float x[4];
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = min(m0 + e, R - 1);
        ok[e] = m0 + e < R;
        row[e] = m;
        x[e] = ok[e] ? s.x[xin][m * H + col] + v[e] : 0.f;
      }
      put_x4(s, xout, gain, row, col, t, x, ok);
      break;
    }
    case E_GU: {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + e;
        const float val = m < R ? v[e] * io.S.inv[m] : 0.f;
        const float up = __shfl_xor(val, 8, 64);
        if (m < R && n < 8) st_wt(&s.h[l][m * FF + 8 * t + n], silu(val) * up);
      }
      break;
    }
  }
}

// Attention: merge of the 6 waves' partials of one chunk into the chunk's
// partial (max, sum, unnormalised output) in global memory.
__device__ __forceinline__ void io_attn_unit(IO& io, int l, const StreamLens& sl, int u) {
  Args& a = io.a;
  const int lane = threadIdx.x & 63;
  int b, h, c;
  sl.unit(u, b, h, c);
  io_wait_done(a, io.S, io.useq);
  KD_LDS float* base = &io.S.part[io.useq & 1][0][0];
  float M[4], Ls[4], O[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NCW; ++w) m = fmaxf(m, base[w * PART + 512 + j]);
    M[j] = m;
    Ls[j] = 0.f;
    O[j][0] = O[j][1] = 0.f;
#pragma unroll
    for (int w = 0; w < NCW; ++w) {
      const float mw = base[w * PART + 512 + j];
      if (mw != -__builtin_inff()) {
        const float f = exp2f(mw - m);
        Ls[j] += base[w * PART + 516 + j] * f;
        const f32x2 ow = *reinterpret_cast<KD_LDS const f32x2*>(base + w * PART + j * DH + 2 * lane);
        O[j][0] += ow.x * f;
        O[j][1] += ow.y * f;
      }
    }
  }
  lds_done();
  if (lane == 0) lds_st(&io.S.freed, io.useq + 1);
  ++io.useq;
  const int nchm = a.nch;
  const size_t pb = ((size_t)(b * NH + h) * nchm + c) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st_wt(&a.s.ao[l][(pb + j) * DH + 2 * lane], O[j][0]);
    st_wt(&a.s.ao[l][(pb + j) * DH + 2 * lane + 1], O[j][1]);
  }
  if (lane < 4) {
    st_wt(&a.s.am[l][pb + lane], M[lane]);
    st_wt(&a.s.al[l][pb + lane], Ls[lane]);
  }
}

// Final merge of one (stream, head): every chunk partial plus the block's own
// keys (row j sees block rows 0..j), normalised, into s.o. Lane l owns dims
// 2l, 2l+1 of the 4 rows.
__device__ __forceinline__ void io_attn_merge(IO& io, int l, const StreamLens& sl, int b, int h) {
  Args& a = io.a;
  auto& s = a.s;
  const int lane = threadIdx.x & 63;
  const int nc = sl.nch(b), nchm = a.nch;
  const size_t base = (size_t)(b * NH + h) * nchm;
  // block queries, keys and values of this head
  float q[4][2], k[4][2], v[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t o = (size_t)(b * 4 + j) * H + h * DH + 2 * lane;
    const f32x2 qq = *reinterpret_cast<gptr<const f32x2>>(s.q[l] + o);
    const f32x2 kk = *reinterpret_cast<gptr<const f32x2>>(s.k[l] + o);
    const f32x2 vv = *reinterpret_cast<gptr<const f32x2>>(s.v[l] + o);
    q[j][0] = qq.x; q[j][1] = qq.y;
    k[j][0] = kk.x; k[j][1] = kk.y;
    v[j][0] = vv.x; v[j][1] = vv.y;
  }
  const float qs = 0.08838834764831845f * 1.4426950408889634f;
  float M[4], Ls[4], O[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    M[j] = -__builtin_inff();
    Ls[j] = 0.f;
    O[j][0] = O[j][1] = 0.f;
  }
  // chunk partials, 4 at a time with every load of a group issued together
  for (int c0 = 0; c0 < nc; c0 += 4) {
    float pm[4][4], pl[4][4];
    f32x2 po[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cc = min(c0 + i, nc - 1);
      const size_t pb = (base + cc) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pm[i][j] = s.am[l][pb + j];
        pl[i][j] = s.al[l][pb + j];
        po[i][j] = *reinterpret_cast<gptr<const f32x2>>(s.ao[l] + (pb + j) * DH + 2 * lane);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c0 + i < nc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float m1 = pm[i][j];
          if (m1 == -__builtin_inff()) continue;
          const float mn = fmaxf(M[j], m1);
          const float f0 = M[j] == -__builtin_inff() ? 0.f : exp2f(M[j] - mn);
          const float f1 = exp2f(m1 - mn);
          Ls[j] = Ls[j] * f0 + pl[i][j] * f1;
          O[j][0] = O[j][0] * f0 + po[i][j].x * f1;
          O[j][1] = O[j][1] * f0 + po[i][j].y * f1;
          M[j] = mn;
        }
      }
    }
  }
  // block keys: s[j][i] = q_j . k_i for i <= j
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i > j) continue;
      float d = q[j][0] * k[i][0] + q[j][1] * k[i][1];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) d += __shfl_xor(d, m, 64);
      const float sc = d * qs;
      const float mn = fmaxf(M[j], sc);
      const float f0 = M[j] == -__builtin_inff() ? 0.f : exp2f(M[j] - mn);
      const float f1 = exp2f(sc - mn);
      Ls[j] = Ls[j] * f0 + f1;
      O[j][0] = O[j][0] * f0 + v[i][0] * f1;
      O[j][1] = O[j][1] * f0 + v[i][1] * f1;
      M[j] = mn;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t o = (size_t)(b * 4 + j) * H + h * DH + 2 * lane;
    st_wt(&s.o[l][o], O[j][0] / Ls[j]);
    st_wt(&s.o[l][o + 1], O[j][1] / Ls[j]);
  }
}

// After every chunk partial of this workgroup is stored: completion counters,
// then the merges this workgroup is designated for (one (stream, head) per
// workgroup, spread over the grid), each after its counter is complete.
__device__ __forceinline__ void io_attn_finish(IO& io, int l, const StreamLens& sl, int k0, int U) {
  Args& a = io.a;
  const int G = gridDim.x, lane = threadIdx.x & 63;
  __builtin_amdgcn_s_waitcnt(0);  // the partial stores are acknowledged
  // one increment per unit this workgroup completed (lanes in parallel)
  for (int k = k0 + G * lane; k < U; k += 64 * G) {
    int b, h, c;
    sl.unit(k, b, h, c);
    add_rlx(&a.s.att_cnt[((l * SB_MAX + b) * NH + h) * 32], 1u);
  }
  const int nbh = a.B * NH;
  for (int i = 0; i < nbh; ++i) {
    if ((i * G) / nbh != (int)blockIdx.x) continue;
    const int b = i / NH, h = i % NH;
    auto cnt = &a.s.att_cnt[((l * SB_MAX + b) * NH + h) * 32];
    const unsigned need = (unsigned)sl.nch(b);
    if (need) {
      const unsigned long long t0 = wall_clock64();
      for (unsigned it = 1; ld_rlx(cnt) < need; ++it) {
        if ((it & 63) == 0 && (wall_clock64() - t0 > SPIN_LIMIT || ld_rlx(err_word(a)) != 0u)) {
          if (lane == 0)
            __hip_atomic_store(err_word(a), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(POLL_SLEEP);
      }
      if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    io_attn_merge(io, l, sl, b, h);
  }
}

// Head tile epilogue: logits, optional logit store, running argmax.
__device__ __forceinline__ void io_head_unit(IO& io, int vt, const f32x4 v) {
  Args& a = io.a;
  auto& d = a.d;
  const int lane = threadIdx.x & 63, n = lane & 15, m0 = 4 * (lane >> 4);
  const int R = a.R, VD = d.VD;
  const int voc = vt * 16 + n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = m0 + e;
    const bool ok = m < R && voc < VD;
    const float logit = ok ? v[e] * io.S.inv[m] * d.hg : 0.f;
    if (ok && a.out_logits) a.out_logits[(size_t)m * VD + voc] = logit;
    unsigned long long key = ok ? argmax_key(logit, (uint32_t)voc) : 0ull;
#pragma unroll
    for (int mm = 1; mm <= 8; mm <<= 1) key = u64_max(key, shfl_xor_u64(key, mm));
    io.best[e] = u64_max(io.best[e], key);
  }
}

// The last workgroup to finish the head reduces every workgroup's candidates.
__device__ __forceinline__ void io_head_finish(IO& io) {
  Args& a = io.a;
  auto& s = a.s;
  const int lane = threadIdx.x & 63, G = gridDim.x, R = a.R;
  if ((lane & 15) == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st_wt64(&s.cand[blockIdx.x * SR_MAX + 4 * (lane >> 4) + e], io.best[e]);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the candidate stores are acknowledged
  unsigned v = 0;
  if (lane == 0) v = add_rlx(&s.bar[19 * 32], 1u);
  v = __builtin_amdgcn_readfirstlane(v);
  if (v != (unsigned)(G - 1)) return;
  if (lane == 0) __hip_atomic_store(&s.bar[19 * 32], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // lane r < 16 reduces row r over all workgroups
  const int r = lane & 15;
  unsigned long long k = 0ull;
  for (int gi = lane >> 4; gi < G; gi += 4) k = u64_max(k, s.cand[gi * SR_MAX + r]);
  k = u64_max(k, shfl_xor_u64(k, 16));
  k = u64_max(k, shfl_xor_u64(k, 32));
  const bool failed = ld_rlx(err_word(a)) != 0u;
  if (lane < R)
    a.out_ids[lane] = failed ? -2 : (k ? a.d.vocab[0xffffffffu - (uint32_t)(k & 0xffffffffu)] : -1);
}

__device__ __attribute__((noinline, not_tail_called)) void role_io(Args& a_, int np_, unsigned epoch0_) {
  Args& a = uni(a_);
  LdsA& S = lds();
  const int np = uni(np_);
  const unsigned epoch0 = (unsigned)uni((int)epoch0_);
  StreamLens sl;
  sl.load(a);
  IO io{a, S, 0u, {0ull, 0ull, 0ull, 0ull}};
  const int G = gridDim.x, lane = threadIdx.x & 63;
  // RoPE table of the block rows (positions len + j, angles in fp64), spread
  // over the grid: entry t of R x 64
  for (int t = blockIdx.x + G * lane; t < a.R * (DH / 2); t += 64 * G) {
    const int r = t / (DH / 2), fi = t % (DH / 2);
    const double pos = (double)a.lens[r >> 2] + (r & 3);
    const double ang = pos * pow((double)a.theta, -(double)fi / (DH / 2));
    st_wt(&a.s.rope[t * 2], (float)cos(ang));
    st_wt(&a.s.rope[t * 2 + 1], (float)sin(ang));
  }
  int rot = 0;
  for (int i = 0; i < np; ++i) {
    const Phase p = make_phase(a, i, sl);
    trace_mark(a, i, 1);
    const int k0 = first_unit(rot);
    // row scales of the phase's input stage
    if (p.kind == K_QKV) io_inv_rms(io, a.s.ssq[xs_in(p.l)], a.R, 0);
    else if (p.kind == K_GU) io_inv_rms(io, a.s.ssq[xs_o(p.l)], a.R, 0);
    else if (p.kind == K_SA) io_inv_rms(io, a.s.ssq[xs_d(p.l - 1)], 3 * a.B, 2);
    else if (p.kind == K_HEAD) io_inv_rms(io, a.s.ssq[a.nl == 0 ? 0 : xs_d(a.nl - 1)], a.R, 0);
    if (p.kind == K_ATTN) {
      for (int k = k0; k < p.U; k += G) io_attn_unit(io, p.l, sl, k);
      io_attn_finish(io, p.l, sl, k0, p.U);
    } else if (p.kind == K_HEAD) {
      for (int k = k0; k < p.U; k += G) io_head_unit(io, k, io_take_proj(io));
    } else {
      for (int k = k0; k < p.U; k += G) {
        int sg, t;
        proj_unit(p, k, sg, t);
        const f32x4 v = io_take_proj(io);
        trace_mark(a, i, 6);
        io_proj_epilogue(io, p, phase_seg(a, p, sg), t, v);
        trace_mark(a, i, 7);
      }
    }
    trace_mark(a, i, 4);
    if (p.kind == K_HEAD) {
      io_head_finish(io);
    } else {
      __builtin_amdgcn_s_waitcnt(0);  // this workgroup's stores are acknowledged
      trace_mark(a, i + 1, 0);
      grid_barrier(a, S, epoch0 + (unsigned)i + 1u);
      if (lane == 0) lds_st(&S.open, (unsigned)i + 2u);
    }
    rot = (rot + p.U) % G;
  }
}

}  // namespace

__global__ __launch_bounds__(WG) void k_stream(const SmallArgs* __restrict__ ap, unsigned epoch0) {
  LdsA& S = lds();
  Args& a = *(Args*)ap;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    if (lane == 0) {
      S.landed = 0u; S.open = 1u; S.freed = 0u; S.fail = 0u;
    }
    if (lane < NCW) {
      S.cons[lane] = 0u;
      S.done[lane] = 0u;
    }
  }
  __syncthreads();
  const int np = stream_phase_count(a.nl);
  if (wave < NCW) role_compute(a, np, wave);
  else if (wave == STREAM_WAVE) role_stream(a, np);
  else role_io(a, np, epoch0);
}

size_t stream_lds_bytes() { return sizeof(Lds); }

hipError_t launch_stream(hipStream_t st, const SmallArgs* dev_args, int G, unsigned epoch0) {
  const SmallArgs* p = dev_args;
  void* args[] = {&p, &epoch0};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_stream), dim3(G), dim3(WG), args,
                                    0, st);
}

int stream_occupancy() {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_stream, WG, 0) != hipSuccess) return 0;
  return occ;
}

int stream_chunk_keys() { return ACH; }

}  // namespace kd
