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
//     ATTN online softmax over each workgroup's contiguous range of 128-key
//          chunks, one partial per (stream, head) segment of the range; a
//          designated workgroup per (stream, head) merges the segments with
//          the block's own keys (causal) -> o
//     O    x += W_o o
//     GU   h = silu(W_g (g_f * x) / rms(x)) * (W_u (g_f * x) / rms(x))
//     DOWN x += W_down h   (inputs split in thirds across workgroups)
//   HEAD  logits = Head (g_o * x) / rms(x) * g_tensor -> per-workgroup argmax;
//         the last workgroup to finish reduces the candidates -> target ids
//
// A workgroup (8 waves) owns whole output tiles: its waves split the inputs,
// an LDS reduction sums them in a fixed order, and the epilogue applies the
// elementwise steps, so every phase writes final values once. RMSNorm is
// deferred: the projection runs on g * x (each producer of x also writes the
// gained copy its matrix consumer needs) and the epilogue scales by 1/rms(x),
// with rms from per-tile sums of squares written by the producer of x.
//
// Per-phase launches (the default): phase p's unit u runs on workgroup u.
// Workgroups with no unit in a phase read ahead the weights of a later phase
// for the workgroups on their XCD (cache warming).
//
// In the persistent kernel, phases are separated by a two-level counter
// barrier without cache-wide fences. That is safe because every buffer a phase
// reads from another workgroup is written at most once per launch, with
// write-through stores, and is read only after the barrier (or counter) that
// follows the write; L1/L2 hold no copy of those lines at kernel start. A
// workgroup arrives at the barrier, issues the weight loads of its first unit
// of the next phase, and only then waits, so weight streaming overlaps the
// synchronisation.
#include "kd_device.h"
#include "kd_small.h"

namespace kd {

#define KD_CONST __attribute__((address_space(4)))
#define KD_LDS __attribute__((address_space(3)))
// The argument block as device code reads it: constant address space (scalar
// loads), global-address-space pointers inside.
typedef const SmallArgsT<GlobalPtr> KD_CONST Args;
typedef const SmallBufsT<GlobalPtr> KD_CONST Bufs;
typedef const WMatT<GlobalPtr> KD_CONST Mat;
typedef KD_LDS float* lds_f;
typedef const KD_LDS float* lds_cf;
template <class T> using gptr = KD_GLOBAL T*;
static_assert(sizeof(SmallArgsT<GlobalPtr>) == sizeof(SmallArgs), "one layout for both views");

enum Phase {
  PH_PRE0 = 0, PH_PRE1 = 1, PH_PRE2 = 2,
  PH_SA = 0, PH_SU = 1, PH_QKV = 2, PH_ATTN = 3, PH_O = 5, PH_GU = 6, PH_DOWN = 7,
  PH_HEAD = 3 + 8 * NL
};

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
// The argument block's address is uniform, but a called (not inlined) phase
// receives it in vector registers; re-establish it as a scalar so that the
// fields are fetched with scalar loads.
template <class T>
__device__ __forceinline__ const T KD_CONST& uni(const T KD_CONST& a) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(&a);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  return *reinterpret_cast<const T KD_CONST*>(((unsigned long long)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ KD_GLOBAL T* uni(KD_GLOBAL T* q) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(q);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  return reinterpret_cast<KD_GLOBAL T*>(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void st_wt(gptr<float> p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// f16 bits of v (round to nearest even), written through like st_wt.
__device__ __forceinline__ void st_wt_h(gptr<uint16_t> p, float v) {
  __hip_atomic_store(p, __builtin_bit_cast(uint16_t, f16_checked(v)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
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

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads or stores.
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void split_bf16(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)v[i];
    hi[i] = h;
    lo[i] = (__bf16)(v[i] - (float)h);
  }
}

__device__ __forceinline__ unsigned long long u64_max(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
// Exchanges between the wave's lane halves (pl32: lanes l and l ^ 32) or
// 16-lane rows (pl16: l and l ^ 16) in one instruction each, without the LDS
// crossbar: r0 = (a of the lower lane, b of the lower lane), r1 = (a of the
// upper lane, b of the upper lane) of each pair, as seen from both lanes of
// the pair (lower lane: r0 = its own a, r1 = the upper lane's a; upper lane:
// r0 = the lower lane's b, r1 = its own b).
// (the pair of results is bit-cast to floats as one vector: bit-casting the
// two elements one by one has been compiled to code that reads the first
// result twice)
__device__ __forceinline__ void pl32(float a, float b, float& r0, float& r1) {
  const f32x2 r = __builtin_bit_cast(
      f32x2, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                              false, false));
  r0 = r[0];
  r1 = r[1];
}
__device__ __forceinline__ void pl16(float a, float b, float& r0, float& r1) {
  const f32x2 r = __builtin_bit_cast(
      f32x2, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                              false, false));
  r0 = r[0];
  r1 = r[1];
}

// Lane moves within 16-lane rows by data-parallel primitives (no LDS):
// quad_perm xor 1 and xor 2, rotations by 8 and 4, and the row's half and
// full mirrors. A butterfly step v + move(v) equals v + v(l ^ m) when
// move(l) = l ^ m, or when the earlier steps left v equal on the lanes that
// move(l) and l ^ m name.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128,
              DPP_MIRROR = 0x140, DPP_HALF_MIRROR = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64s(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Grid barrier: two-level counters (groups of 16 workgroups), monotonic so
// nothing is ever reset, a generation word, and a wall-clock bound: after
// 0.2 s a workgroup sets the error word and goes on, so every wave still
// reaches the end of the kernel. Split into arrive and wait so a workgroup can
// issue loads of data it does not depend on in between.
// ---------------------------------------------------------------------------
struct SyncState {
  unsigned epoch0;  // barriers completed by earlier launches (from the host)
  int slot;         // phase index within the launch; phase i > 0 passes barrier i
};

// Stage timestamps for tracing: slot 0 barrier arrival, 1 barrier passed,
// 2 unit inputs issued, 3 compute done, 4 epilogue done, 7 phase exit.
__device__ __forceinline__ void trace_mark(Args& a, const SyncState sy, int k, int who = 0) {
  if (a.trace && threadIdx.x == who && sy.slot < a.trace_phases)
    a.trace[((size_t)sy.slot * gridDim.x + blockIdx.x) * 8 + k] = wall_clock64();
}

// Wave POLL_WAVE publishes the arrival and polls. A wave's vector loads
// complete in issue order, so a poll issued behind a weight prefetch would see
// the barrier only after the whole prefetch has landed; the polling wave
// therefore issues its own loads of the next phase only after the barrier,
// while the other waves prefetch before it.
constexpr int POLL_WAVE = SMALL_WG / 64 - 1;
constexpr int POLL_LANE0 = POLL_WAVE * 64;

__device__ __forceinline__ bool is_poll_wave() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == POLL_WAVE;
}

__device__ void grid_arrive(Args& a, SyncState sy) {
  // every wave's global stores of the previous phase are acknowledged before
  // the arrival is published: one atomic add on the group's counter whose
  // result is not waited for
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
  __syncthreads();
  if (threadIdx.x == POLL_LANE0) {
    trace_mark(a, sy, 0, POLL_LANE0);
    __hip_atomic_fetch_add(&a.s.bar[(blockIdx.x >> 4) * 32], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Called by the whole polling wave, before it issues any load of the phase:
// lane g < 16 watches group g's counter until it holds the group's size times
// the number of barriers completed so far (every counter starts at zero and
// grows by its group's size per barrier; 32-bit wrap-around is harmless).
__device__ void grid_poll(Args& a, SyncState sy) {
  const int lane = threadIdx.x & 63, G = gridDim.x, ngrp = (G + 15) >> 4;
  const int g = min(lane, ngrp - 1);
  const unsigned gsize = min(16, G - g * 16);
  const unsigned target = gsize * (sy.epoch0 + (unsigned)sy.slot);
  auto cnt = &a.s.bar[g * 32];
  const unsigned long long t0 = wall_clock64();
  while (true) {
    const bool ok = (int)(ld_rlx(cnt) - target) >= 0;
    if (__all(ok)) break;
    if (wall_clock64() - t0 > 20000000ull) {  // 0.2 s at the 100 MHz wall clock
      if (lane == 0) __hip_atomic_store(&a.s.bar[18 * 32], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  trace_mark(a, sy, 1, POLL_LANE0);
}

// Arrival and wait with no prefetch in between.
__device__ __forceinline__ void grid_wait(Args& a, SyncState sy) {
  if (is_poll_wave()) grid_poll(a, sy);
  lds_sync();
}

__device__ __forceinline__ void grid_sync(Args& a, SyncState sy) {
  grid_arrive(a, sy);
  grid_wait(a, sy);
}

// LDS of the attention phase: 16 ring slots of 8 KB, two per wave (slot s at
// half s / 8, blocks 8 (s % 8) ..), each holding one 16-key block as it
// arrives by global-to-LDS copies (4 key blocks, 4 value blocks of 1 KB; a
// copy puts lane l's 16 bytes at l * 16, and the same lane reads them back).
// The last 2 KB of each half are spare. The ring is also the reduction area
// of every other phase.
constexpr int ATT_WAVE_BLOCKS = 8;
constexpr int ATT_SLOT_BLOCKS = 8 * ATT_WAVE_BLOCKS + 2;
constexpr unsigned ATT_SLOT_BYTES = ATT_SLOT_BLOCKS * 1024u;
__shared__ __attribute__((aligned(16))) u32x4 g_att_ring[2][ATT_SLOT_BLOCKS][64];
// per-wave outputs [8][4][128], softmax max and sum [8][4] each, probabilities [8][4][16]
constexpr int ATT_SMALL = 8 * 4 * DH + 32 + 32 + 8 * 4 * 16;
__shared__ __attribute__((aligned(16))) float g_att_small[ATT_SMALL];

// Waits until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void att_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Waits until at most n blocks' copies (8 per 16-key block, n = 0..7,
// wave-uniform) of this wave are in flight.
__device__ __forceinline__ void att_wait_blocks(int n) {
  switch (n) {
    case 0: att_wait_vm<0>(); break;
    case 1: att_wait_vm<8>(); break;
    case 2: att_wait_vm<16>(); break;
    case 3: att_wait_vm<24>(); break;
    case 4: att_wait_vm<32>(); break;
    case 5: att_wait_vm<40>(); break;
    case 6: att_wait_vm<48>(); break;
    default: att_wait_vm<56>(); break;
  }
}
// (n is wave-uniform; values the attention loop uses: 0, 2, 5, 8, 10, 11, 13)
__device__ __forceinline__ void att_wait_vm(int n) {
  if (n >= 13) att_wait_vm<13>();
  else if (n >= 11) att_wait_vm<11>();
  else if (n >= 10) att_wait_vm<10>();
  else if (n >= 8) att_wait_vm<8>();
  else if (n >= 5) att_wait_vm<5>();
  else if (n >= 2) att_wait_vm<2>();
  else att_wait_vm<0>();
}

// ---------------------------------------------------------------------------
// Cache warming by idle workgroups
// ---------------------------------------------------------------------------
// Unit u of a phase with at most G units runs on workgroup u, which the
// dispatcher places on XCD u % 8 (workgroups are dealt to the 8 XCDs in turn).
// Workgroups idle in the current phase read the data of units of a later
// phase on the XCD that will run them, so that those loads find the lines in
// that XCD's L2 or the memory-side cache. The reads are global-to-LDS copies
// of one dword per 128-byte line into a scratch area of LDS: they hold no
// registers and nothing waits for them until the end.
__device__ __forceinline__ void touch(gptr<const uint8_t> p, size_t bytes) {
  KD_LDS void* dump = (KD_LDS void*)(KD_LDS float*)g_att_small;
  for (size_t off = (size_t)threadIdx.x * 128; off < bytes; off += (size_t)SMALL_WG * 128)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p + off), dump, 4, 0, 0);
}
// The weights and scales of tiles [t0, t0 + ntile), input blocks [kb0, kb0 + nkb).
__device__ __forceinline__ void touch_tiles(Mat& W, int t0, int ntile, int kb0, int nkb) {
  const int KB = W.K >> 6, fmt = uni(W.fmt);
  // code bytes per 16 outputs x 64 inputs: block-FP8 1024 (+ 64 of scales),
  // NVFP4 512 (+ 64 of scale codes), bf16 2048
  const size_t cb = fmt == WF_NVFP4 ? 512 : (fmt == WF_BF16 ? 2048 : 1024);
  for (int t = t0; t < t0 + ntile; ++t) {
    const size_t blk = (size_t)t * KB + kb0;
    touch(W.w + blk * cb, (size_t)nkb * cb);
    if (fmt == WF_FP8) touch(reinterpret_cast<gptr<const uint8_t>>(W.s + blk * 16), (size_t)nkb * 64);
    if (fmt == WF_NVFP4) touch(W.s4 + blk * 64, (size_t)nkb * 64);
  }
}
// Idle workgroups [i0, G): workgroup w on XCD x = w % 8 takes the units
// u = x (mod 8) of the later phase in turn with the other idle workgroups of
// that XCD; touch_unit(u) reads what unit u will load.
template <class F>
__device__ __forceinline__ void warm(int i0, int nunits, F&& touch_unit) {
  const int w = blockIdx.x, G = gridDim.x;
  if (w < i0) return;
  const int x = w & 7, f = i0 + ((x - i0) & 7);
  const int k = (w - f) >> 3, nk = (G - f + 7) >> 3;
  for (int u = x + 8 * k; u < nunits; u += 8 * nk) touch_unit(u);
}
// Every copy has landed (before the workgroup ends, while its LDS is still its own).
__device__ __forceinline__ void warm_done() { att_wait_vm<0>(); }
// q|k|v units [u0, u1) of layer l (two tiles each), by idle workgroups [i0, G).
__device__ __forceinline__ void warm_qkv(Args& a, int l, int i0, int u0, int u1) {
  Mat& W = a.d.layer[l].qkv;
  warm(i0, u1, [&](int u) {
    if (u >= u0) touch_tiles(W, 2 * u, 2, 0, H / 64);
  });
}

// ---------------------------------------------------------------------------
// Projection units: NT consecutive 16-row weight tiles; wave w (< AW) takes
// the 64-input blocks kb0 + w*KBS .. + KBS.
// ---------------------------------------------------------------------------
template <int WF, int NT, int KBS>
struct WRegs;
template <int NT, int KBS>
struct WRegs<WF_FP8, NT, KBS> {   // 16 e4m3 codes and the block's scale per lane
  u32x4 w[NT][KBS];
  float s[NT][KBS];
};
template <int NT, int KBS>
struct WRegs<WF_NVFP4, NT, KBS> {  // 16 e2m1 codes and two e4m3 scale codes per lane
  uint2 q[NT][KBS];
  uint32_t sc[NT][KBS];
  float g[NT][2];                  // the column's tensor scales (blocks before / from ks)
};
template <int NT, int KBS>
struct WRegs<WF_BF16, NT, KBS> {   // 16 bf16 values per lane
  u32x4 w0[NT][KBS], w1[NT][KBS];
};

// Loads are unconditional (indices clamped into range): a load inside a
// conditional block with a fallback value makes the compiler wait for it at the
// join, which would serialise the prefetch. Waves past AW load wave AW-1's
// blocks and ignore them; tiles past ntv repeat the last valid tile, whose
// results the epilogue discards. The lane's part of a block is laid out as in
// the general path's tiles (kd_device.h: load_wblock).
template <int WF, int NT, int KBS, int AW>
__device__ __forceinline__ void load_w(WRegs<WF, NT, KBS>& r, Mat& W, int tile0, int ntv,
                                       int kb0) {
  const int lane = threadIdx.x & 63, wave = min((int)(threadIdx.x >> 6), AW - 1);
  const int KB = W.K >> 6;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int nt = tile0 + min(i, ntv - 1);
    if constexpr (WF == WF_NVFP4) {
      r.g[i][0] = W.s[nt * 16 + (lane & 15)];
      r.g[i][1] = W.s[W.N + nt * 16 + (lane & 15)];
    }
#pragma unroll
    for (int j = 0; j < KBS; ++j) {
      const size_t blk = (size_t)nt * KB + kb0 + wave * KBS + j;
      if constexpr (WF == WF_FP8) {
        r.w[i][j] = *reinterpret_cast<gptr<const u32x4>>(W.w + blk * 1024 + lane * 16);
        r.s[i][j] = W.s[blk * 16 + (lane & 15)];
      } else if constexpr (WF == WF_NVFP4) {
        r.q[i][j] = *reinterpret_cast<gptr<const uint2>>(W.w + blk * 512 + lane * 8);
        const uint32_t sw = *reinterpret_cast<gptr<const uint32_t>>(W.s4 + blk * 64 + (lane & 15) * 4);
        const int sh = 8 * ((lane >> 4) >> 1);
        r.sc[i][j] = ((sw >> sh) & 0xffu) | (((sw >> (sh + 16)) & 0xffu) << 8);
      } else {
        r.w0[i][j] = *reinterpret_cast<gptr<const u32x4>>(W.w + blk * 2048 + lane * 16);
        r.w1[i][j] = *reinterpret_cast<gptr<const u32x4>>(W.w + blk * 2048 + 1024 + lane * 16);
      }
    }
  }
}

// The bf16 bits of 8 f16 values that need no more than 8 significant bits
// (NVFP4 values: at most 6).
__device__ __forceinline__ bf16x8 f16x8_to_bf16_exact(f16x8 v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float)v[i];
  return r;
}

// Activation rows of the A operand: bf16 (the tapped states and embedding
// rows, taken exactly on the bf16 matrix cores) or f16 (activations the round
// produces, on the f16 matrix cores).
struct ASrc {
  gptr<const void> base;
  int ld;               // elements per row
  int mode;             // 0: row r; 1: row r/3; 2: row 4(r/3) + r%3; 3: row ids[r];
                        // 4: row ids[4(r/3) + r%3]
  gptr<const int32_t> ids;
  int kb_off;           // weight block of column 0
  int R;
  gptr<const uint16_t> zrow = nullptr;  // modes 3, 4: read for an id outside [0, V)
  int V = 0;
};

// The lane's activation row: modes 3 and 4 take a table row by token id (the
// zero row for an out-of-range id), the others a row of A.base.
__device__ __forceinline__ gptr<const uint16_t> a_row_ptr(const ASrc& A, int r) {
  auto base = static_cast<gptr<const uint16_t>>(A.base);
  switch (A.mode) {
    case 1: return base + (size_t)(r / 3) * A.ld;
    case 2: return base + (size_t)(4 * (r / 3) + r % 3) * A.ld;
    case 3: return table_row(base, A.zrow, A.ids[r], A.V, A.ld);
    case 4: return table_row(base, A.zrow, A.ids[4 * (r / 3) + r % 3], A.V, A.ld);
    default: return base + (size_t)r * A.ld;
  }
}

// Issues the loads of one 64-input block of the lane's row: 8 values at
// inputs 8 (lane / 16) .. + 8 of each of the block's two 32-input halves.
__device__ __forceinline__ void a_issue(const ASrc& A, int kb, u32x4 (&raw)[2]) {
  // rows past R repeat row R-1; they only feed output rows that are discarded
  const int lane = threadIdx.x & 63, r = min(lane & 15, A.R - 1);
  const int c0 = (kb - A.kb_off) * 64 + 8 * (lane >> 4);
  auto p = a_row_ptr(A, r) + c0;
  raw[0] = *reinterpret_cast<gptr<const u32x4>>(p);
  raw[1] = *reinterpret_cast<gptr<const u32x4>>(p + 32);
}

// Partial products of each wave into LDS: red[((wave*NT + i)*4 + e)*64 + lane].
// The A loads of up to C blocks are in flight together. ABF: bf16 activations
// (weights decoded to bf16), else f16 (weights decoded to f16; bf16 weights
// take each f16 activation as two exact bf16 terms); every decode is exact.
// Each block's product is scaled by its block-FP8 scale or its column's
// NVFP4 tensor scale.
template <int WF, int NT, int KBS, int AW, bool ABF>
__device__ __forceinline__ void gemm_compute(const WRegs<WF, NT, KBS>& r, const ASrc& A, int kb0,
                                             lds_f red, int ks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int C = KBS < 8 ? KBS : 8;
  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave < AW) {
#pragma unroll
    for (int c0 = 0; c0 < KBS; c0 += C) {
      u32x4 raw[C][2];
#pragma unroll
      for (int j = 0; j < C; ++j)
        if (c0 + j < KBS) a_issue(A, kb0 + wave * KBS + c0 + j, raw[j]);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (c0 + j < KBS) {
#pragma unroll
          for (int i = 0; i < NT; ++i) {
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            if constexpr (WF == WF_FP8) {
              const u32x4 wv = r.w[i][c0 + j];
              if (ABF) {
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][0]), e4m3x8_bf16(wv.x, wv.y), t);
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][1]), e4m3x8_bf16(wv.z, wv.w), t);
              } else {
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, raw[j][0]),
                                                           e4m3x8_f16(wv.x, wv.y), t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, raw[j][1]),
                                                           e4m3x8_f16(wv.z, wv.w), t, 0, 0, 0);
              }
              acc[i] += r.s[i][c0 + j] * t;
            } else if constexpr (WF == WF_NVFP4) {
              const uint2 q = r.q[i][c0 + j];
              const uint32_t sc = r.sc[i][c0 + j];
              const f16x8 w0 = nvfp4x8_f16(q.x, sc & 0xffu), w1 = nvfp4x8_f16(q.y, sc >> 8);
              if (ABF) {
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][0]), f16x8_to_bf16_exact(w0), t);
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][1]), f16x8_to_bf16_exact(w1), t);
              } else {
                t = mfma_f16(__builtin_bit_cast(f16x8, raw[j][0]), w0, t);
                t = mfma_f16(__builtin_bit_cast(f16x8, raw[j][1]), w1, t);
              }
              acc[i] += (kb0 + wave * KBS + c0 + j < ks ? r.g[i][0] : r.g[i][1]) * t;
            } else {
              const bf16x8 w0 = __builtin_bit_cast(bf16x8, r.w0[i][c0 + j]);
              const bf16x8 w1 = __builtin_bit_cast(bf16x8, r.w1[i][c0 + j]);
              if (ABF) {
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][0]), w0, t);
                t = mfma_bf16(__builtin_bit_cast(bf16x8, raw[j][1]), w1, t);
              } else {
                bf16x8 h0, l0, h1, l1;
                split_f16_bf16(__builtin_bit_cast(f16x8, raw[j][0]), h0, l0);
                split_f16_bf16(__builtin_bit_cast(f16x8, raw[j][1]), h1, l1);
                t = mfma_bf16(h0, w0, t);
                t = mfma_bf16(l0, w0, t);
                t = mfma_bf16(h1, w1, t);
                t = mfma_bf16(l1, w1, t);
              }
              acc[i] += t;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * NT + i) * 4 + e) * 64 + lane] = acc[i][e];
  lds_sync();
}

// Sums the 8 waves' partials in a fixed order and calls f(i, m, n, v) for
// output row m and column n of tile i. Within a wave the 64 items cover 4 rows
// x 16 columns of one tile, so f may use shuffles across columns (xor 1..8).
template <int NT, class F>
__device__ __forceinline__ void gemm_epilogue(lds_cf red, F&& f) {
  for (int it = threadIdx.x; it < NT * 256; it += SMALL_WG) {
    const int i = it >> 8, m = (it >> 4) & 15, n = it & 15;
    const int L = 16 * (m >> 2) + n, e = m & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) v += red[((w * NT + i) * 4 + e) * 64 + L];
    f(i, m, n, v);
  }
  lds_sync();
}


// 1/rms of up to 16 rows of a residual stage from its per-tile sums of
// squares. issue() loads, finish() reduces into LDS inv[16].
struct RmsRows {
  gptr<const float> ssq;
  int nrows, mode;      // mode 0: row r; 2: row 4(r/3) + r%3
  float eps;
  lds_f inv;
  float v[5];
  __device__ __forceinline__ void issue() {
    if (!ssq) return;  // v stays unset and unused
    const int r = min((int)(threadIdx.x >> 5), nrows - 1), l32 = threadIdx.x & 31;
    const int row = mode == 2 ? 4 * (r / 3) + r % 3 : r;
    auto p = ssq + (size_t)row * HT + l32;
#pragma unroll
    for (int k = 0; k < 5; ++k) v[k] = p[32 * k];
  }
  __device__ __forceinline__ void finish() {
    if (!ssq) return;
    const int r = threadIdx.x >> 5, l32 = threadIdx.x & 31;
    float sum = v[0] + v[1] + v[2] + v[3] + v[4];
    // butterfly over the 32 lanes l32 (xor 16, 8, 4, 2, 1)
    {
      float r0, r1;
      pl16(sum, sum, r0, r1);
      sum = r0 + r1;
    }
    sum += dpp_f<DPP_ROR8>(sum);   // = lane ^ 8
    sum += dpp_f<DPP_ROR4>(sum);   // lanes 8 apart now agree: = lane ^ 4
    sum += dpp_f<DPP_XOR2>(sum);
    sum += dpp_f<DPP_XOR1>(sum);
    if (r < nrows && l32 == 0) inv[r] = 1.0f / sqrtf(sum / H + eps);
    lds_sync();
  }
};

// Sum of squares of this tile's 16 columns for the item's row (all lanes).
__device__ __forceinline__ float tile_ssq(float x) {
  float s = x * x;
  // butterfly over the 16-lane row (xor 1, 2, 4, 8)
  s += dpp_f<DPP_XOR1>(s);
  s += dpp_f<DPP_XOR2>(s);
  s += dpp_f<DPP_HALF_MIRROR>(s);   // quads now agree: = lane ^ 4
  s += dpp_f<DPP_MIRROR>(s);        // halves now agree: = lane ^ 8
  return s;
}

// One projection unit: if this is the workgroup's first unit of the phase,
// arrive at the barrier, issue the weight loads, then wait; compute; reduce;
// run `epi`.
template <int WF, int NT, int KBS, int AW, bool ABF>
__device__ __forceinline__ void gemm_body(Args& a, SyncState sy, bool sync, Mat& W, int tile0, int ntv,
                                          int kb0, const ASrc& A, lds_f red, RmsRows& rms) {
  WRegs<WF, NT, KBS> r;
  load_w<WF, NT, KBS, AW>(r, W, tile0, ntv, kb0);
  if (sync) lds_sync();
  trace_mark(a, sy, 2);
  rms.issue();
  gemm_compute<WF, NT, KBS, AW, ABF>(r, A, kb0, red, W.ks);
  rms.finish();
}

template <int WF, int NT, int KBS, int AW, bool ABF, class Epi>
__device__ __forceinline__ void gemm_unit(Args& a, SyncState sy, bool sync,
                                          Mat& W, int tile0, int ntv, int kb0,
                                          const ASrc& A, lds_f red, RmsRows rms, Epi&& epi) {
  if (sync) {
    grid_arrive(a, sy);
    if (is_poll_wave()) grid_poll(a, sy);
  }
  gemm_body<WF, NT, KBS, AW, ABF>(a, sy, sync, W, tile0, ntv, kb0, A, red, rms);
  trace_mark(a, sy, 3);
  gemm_epilogue<NT>(red, epi);
  trace_mark(a, sy, 4);
}

__device__ __forceinline__ RmsRows no_rms() { return RmsRows{nullptr, 0, 0, 0.f, nullptr, {}}; }

// Stores one element of a residual stage: raw x, gained copy and (once per
// tile row) the tile's sum of squares.
__device__ __forceinline__ void put_x(Bufs& s, int stage, gptr<const float> gain, int row,
                                      int col, int tile, int n, float x, bool ok) {
  const float q = tile_ssq(x);
  if (ok) {
    st_wt(&s.x[stage][row * H + col], x);
    st_wt_h(&s.xg[stage][row * H + col], x * gain[col]);
    if (n == 0) st_wt(&s.ssq[stage][row * HT + tile], q);
  }
}

// Gain of the matrix consumer of a residual stage.
__device__ __forceinline__ gptr<const float> gain_in(Args& a, int l) {
  return l < a.nl ? a.d.layer[l].attn_norm : a.d.final_norm;
}
__device__ __forceinline__ gptr<const float> gain_after_down(Args& a, int l) {
  return l + 1 < a.nl ? a.d.layer[l + 1].spine_norm : a.d.final_norm;
}

// ---------------------------------------------------------------------------
// Phases. `sync` is true when the phase must wait at a grid barrier first
// (persistent kernel); every workgroup then passes exactly one barrier.
// ---------------------------------------------------------------------------
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_pre0(Args& a_, lds_f red, SyncState sy) {
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int B = a.B, R = a.R;
  // a new round: no bounded wait of it has timed out yet
  if (wg == 0 && threadIdx.x == 0)
    __hip_atomic_store(&s.bar[18 * 32], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // units: the fuse tiles (120 input blocks each), then the fc and
  // predecessor tiles (40 each). With enough workgroups every fuse tile gets
  // its own and the other workgroups share the light tiles; otherwise they
  // are dealt in turn.
  const int n_fuse = HT, n_fce = HT, n_pb = RK / 16, n_all = n_fuse + n_fce + n_pb;
  const bool split = G > n_fuse;
  const int u_first = split ? (wg < n_fuse ? wg : n_fuse + (wg - n_fuse)) : wg;
  const int u_end = split && wg < n_fuse ? wg + 1 : n_all;
  const int u_step = split ? G - n_fuse : G;
  for (int u = u_first; u < u_end; u += u_step) {
    if (u < n_fuse) {
      const ASrc A{a.taps, NTAP * H, 0, nullptr, 0, B};
      gemm_unit<WF, 1, 15, 8, true>(a, sy, false, d.fuse, u, 1, 0, A, red, no_rms(),
                                [&](int, int m, int n, float v) {
                                  if (m < B) {
                                    st_wt(&s.f[m * H + u * 16 + n], v);
                                    st_wt_h(&s.fh[m * H + u * 16 + n], v);
                                  }
                                });
    } else if (u < n_fuse + n_fce) {
      const int t = u - n_fuse;
      const ASrc A{d.table, H, 3, a.anchor, 40, B, d.zrow, d.V};
      gemm_unit<WF, 1, 5, 8, true>(a, sy, false, d.fc, t, 1, 40, A, red, no_rms(),
                               [&](int, int m, int n, float v) {
                                 if (m < B) st_wt(&s.fce[m * H + t * 16 + n], v);
                               });
    } else {
      const int t = u - n_fuse - n_fce;
      const ASrc A{d.table, H, a.pred_stride == 4 ? 4 : 3, a.pred, 40, 3 * B, d.zrow, d.V};
      gemm_unit<WF, 1, 5, 8, true>(a, sy, false, d.pred_ab, t, 1, 40, A, red, no_rms(),
                               [&](int, int m, int n, float v) {
                                 if (m < 3 * B) st_wt(&s.pb[m * RK + t * 16 + n], v);
                               });
    }
  }
}

template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_pre1(Args& a_, lds_f red, SyncState sy,
                                                  bool sync) {
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int B = a.B;
  auto gain = gain_in(a, 0);
  bool first = sync;
  for (int u = wg; u < HT + RK / 16; u += G) {
    if (u < HT) {
      const ASrc A{s.fh, H, 0, nullptr, 0, B};
      gemm_unit<WF, 1, 5, 8, false>(a, sy, first, d.fc, u, 1, 0, A, red, no_rms(),
                                [&](int, int m, int n, float v) {
                                  const int col = u * 16 + n;
                                  const float x = v + (m < B ? s.fce[m * H + col] : 0.f);
                                  put_x(s, 0, gain, 4 * m, col, u, n, x, m < B);
                                });
    } else {
      const int t = u - HT;
      const ASrc A{s.fh, H, 1, nullptr, 0, 3 * B};
      gemm_unit<WF, 1, 5, 8, false>(a, sy, first, d.pred_ab, t, 1, 0, A, red, no_rms(),
                                [&](int, int m, int n, float v) {
                                  if (m < 3 * B) {
                                    const int c = t * 16 + n;
                                    st_wt_h(&s.sp[m * RK + c], silu(v + s.pb[m * RK + c]));
                                  }
                                });
    }
    first = false;
  }
  if (first) grid_sync(a, sy);
  // idle workgroups warm the first half of layer 0's q|k|v (per-phase path)
  if (!sync) {
    warm_qkv(a, 0, HT + RK / 16, 0, QKV / 32 / 2);
    warm_done();
  }
}

template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_pre2(Args& a_, lds_f red, SyncState sy,
                                                  bool sync) {
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int B = a.B;
  auto gain = gain_in(a, 0);
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{s.sp, RK, 0, nullptr, 0, 3 * B};
    gemm_unit<WF, 1, 1, 4, false>(a, sy, first, d.pred_u, u, 1, 0, A, red, no_rms(),
                              [&](int, int m, int n, float v) {
                                const int col = u * 16 + n;
                                const bool ok = m < 3 * B;
                                const float x = ok ? d.mask[col] + s.f[(m / 3) * H + col] + v : 0.f;
                                put_x(s, 0, gain, 4 * (m / 3) + m % 3 + 1, col, u, n, x, ok);
                              });
    first = false;
  }
  if (first) grid_sync(a, sy);
  // idle workgroups warm the second half of layer 0's q|k|v (per-phase path)
  if (!sync && a.nl > 0) {
    warm_qkv(a, 0, HT, QKV / 32 / 2, QKV / 32);
    warm_done();
  }
}

// Spine A: ss = silu(A_s (g_s * x_{j-1}) / rms(x_{j-1})) for rows j = 1..3.
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_sa(Args& a_, int l_, lds_f red,
                                                SyncState sy, bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int B = a.B, src = xs_d(l - 1);
  lds_f inv = red + 8192;
  bool first = sync;
  for (int u = wg; u < RK / 16; u += G) {
    const ASrc A{s.xg[src], H, 2, nullptr, 0, 3 * B};
    gemm_unit<WF, 1, 5, 8, false>(a, sy, first, L.sa, u, 1, 0, A, red,
                              RmsRows{s.ssq[src], 3 * B, 2, a.eps, inv, {}},
                              [&](int, int m, int n, float v) {
                                if (m < 3 * B) st_wt_h(&s.ss[l][m * RK + u * 16 + n], silu(v * inv[m]));
                              });
    first = false;
  }
  if (first) grid_sync(a, sy);
  // the workgroups without a tile warm the next phases' weights: the spine U
  // (one tile per unit) and the first half of q|k|v (two); not in the
  // persistent kernel
  if (!sync) {
    warm(RK / 16, HT, [&](int u) { touch_tiles(L.su, u, 1, 0, RK / 64); });
    warm_qkv(a, l, RK / 16, 0, QKV / 32 / 2);
    warm_done();
  }
}

// Spine U: x_j (j = 1..3) += U_s ss; row 0 copied into the new stage.
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_su(Args& a_, int l_, lds_f red,
                                                SyncState sy, bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int B = a.B, src = xs_d(l - 1), dst = xs_in(l);
  auto gain = gain_in(a, l);
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{s.ss[l], RK, 0, nullptr, 0, 3 * B};
    gemm_unit<WF, 1, 1, 4, false>(a, sy, first, L.su, u, 1, 0, A, red, no_rms(),
                              [&](int, int m, int n, float v) {
                                const int col = u * 16 + n;
                                const int row = 4 * (m / 3) + m % 3 + 1;
                                const bool ok = m < 3 * B;
                                const float x = ok ? s.x[src][row * H + col] + v : 0.f;
                                put_x(s, dst, gain, row, col, u, n, x, ok);
                              });
    // row 0 of every stream is untouched by the spine
    for (int t = threadIdx.x; t < B * 17; t += SMALL_WG) {
      const int b = t / 17, c = t % 17, row = 4 * b, col = u * 16 + c;
      if (c < 16) {
        const float x = s.x[src][row * H + col];
        st_wt(&s.x[dst][row * H + col], x);
        st_wt_h(&s.xg[dst][row * H + col], x * gain[col]);
      } else {
        st_wt(&s.ssq[dst][row * HT + u], s.ssq[src][row * HT + u]);
      }
    }
    first = false;
  }
  if (first) grid_sync(a, sy);
  // idle workgroups warm the second half of q|k|v (per-phase path)
  if (!sync) {
    warm_qkv(a, l, HT, QKV / 32 / 2, QKV / 32);
    warm_done();
  }
}

// q|k|v = W (g_a * x) / rms(x); RoPE on q and k inside each paired tile.
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_qkv(Args& a_, int l_, lds_f red,
                                                 SyncState sy, bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int R = a.R, src = xs_in(l);
  lds_f inv = red + 8192;
  constexpr int NT = 2, NTILE = QKV / 16, NU = NTILE / NT;
  bool first = sync;
  for (int u = wg; u < NU; u += G) {
    const ASrc A{s.xg[src], H, 0, nullptr, 0, R};
    gemm_unit<WF, NT, 5, 8, false>(
        a, sy, first, L.qkv, u * NT, NT, 0, A, red, RmsRows{s.ssq[src], R, 0, a.eps, inv, {}},
        [&](int i, int m, int n, float v) {
          const int t = u * NT + i, sec = t / HT;
          const int nat = qkv_natural(t * 16 + n) - sec * H;  // column within q, k or v
          const float val = m < R ? v * inv[m] : 0.f;
          const float partner = dpp_f<DPP_ROR8>(val);
          float out = val;
          if (sec < 2) {
            const int fi = (nat % DH) & 63;
            const float cs = m < R ? s.rope[(m * (DH / 2) + fi) * 2] : 0.f;
            const float sn = m < R ? s.rope[(m * (DH / 2) + fi) * 2 + 1] : 0.f;
            out = n < 8 ? val * cs - partner * sn : partner * sn + val * cs;
          }
          if (m < R) {
            gptr<float> dstp = sec == 0 ? s.q[l] : (sec == 1 ? s.k[l] : s.v[l]);
            st_wt(&dstp[m * H + nat], out);
          }
        });
    first = false;
  }
  if (first) grid_sync(a, sy);
}

// Cross-lane steps inside a wavefront without LDS traffic. row16_sum: sum
// over the 16 lanes of each row by DPP (quad swaps, then the half-row and row
// mirrors; every lane ends with the same bits). rows_sum_to_row3: per lane
// position, the sum over the 4 rows, valid in row 3 only; it uses the first
// result of the gfx950 row-swap permutes (which moves row 0 to row 1, row 2 to
// row 3, and then the lower half to the upper half). rows_max4 / rows_sum4:
// combine a value that is uniform within each row across the 4 rows, in every
// lane, through scalar lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float rows_sum_to_row3(float x) {
  const unsigned xb = __builtin_bit_cast(unsigned, x);
  const float s = x + __builtin_bit_cast(float, __builtin_amdgcn_permlane16_swap(xb, xb, false, false)[0]);
  const unsigned sb = __builtin_bit_cast(unsigned, s);
  return s + __builtin_bit_cast(float, __builtin_amdgcn_permlane32_swap(sb, sb, false, false)[0]);
}
__device__ __forceinline__ float lane_read(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float rows_max4(float x) {
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}
__device__ __forceinline__ float rows_sum4(float x) {
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}

// Context rows of each stream of the round, read once per phase; kept as
// separate scalars (an indexed array would live in scratch memory).
__device__ __forceinline__ int pick4(int b, int x0, int x1, int x2, int x3) {
  return b == 0 ? x0 : (b == 1 ? x1 : (b == 2 ? x2 : x3));
}
template <int CH>
struct StreamLensT {
  int n0, n1, n2, n3;      // visible context rows min(len, window)
  int f0, f1, f2, f3;      // position of the first visible row
  int c0, c1, c2, c3;      // chunks of CH rows per (stream, head)
  int o1, o2, o3, total;   // first attention unit of streams 1..3; all units
  __device__ __forceinline__ void load(Args& a) {
    const int B = a.B, W = a.window;
    // lane b < B reads stream b's length (one load), then every lane takes
    // the four values from lanes 0..3
    const int lane = threadIdx.x & 63;
    const int mine = a.lens[min(lane, B - 1)];
    const int l0 = __builtin_amdgcn_readlane(mine, 0);
    const int l1 = B > 1 ? __builtin_amdgcn_readlane(mine, 1) : 0;
    const int l2 = B > 2 ? __builtin_amdgcn_readlane(mine, 2) : 0;
    const int l3 = B > 3 ? __builtin_amdgcn_readlane(mine, 3) : 0;
    n0 = min(l0, W); n1 = min(l1, W); n2 = min(l2, W); n3 = min(l3, W);
    f0 = l0 - n0; f1 = l1 - n1; f2 = l2 - n2; f3 = l3 - n3;
    c0 = (n0 + CH - 1) / CH;
    c1 = (n1 + CH - 1) / CH;
    c2 = (n2 + CH - 1) / CH;
    c3 = (n3 + CH - 1) / CH;
    o1 = NH * c0;
    o2 = o1 + NH * c1;
    o3 = o2 + NH * c2;
    total = o3 + NH * c3;
  }
  __device__ __forceinline__ int vis(int b) const { return pick4(b, n0, n1, n2, n3); }
  __device__ __forceinline__ int first(int b) const { return pick4(b, f0, f1, f2, f3); }
  __device__ __forceinline__ int chunks(int b) const { return pick4(b, c0, c1, c2, c3); }
  // Unit u -> stream b, chunk c, head h (stream-major, then head, then chunk,
  // so the chunks of one (stream, head) are consecutive units). A stream with
  // no units shares its offset with the next one, which then wins.
  __device__ __forceinline__ void unit(int u, int& b, int& c, int& h) const {
    b = u >= o3 ? 3 : (u >= o2 ? 2 : (u >= o1 ? 1 : 0));
    const int loc = u - pick4(b, 0, o1, o2, o3), nc = chunks(b);
    h = loc / nc;
    c = loc - h * nc;
  }
  __device__ __forceinline__ int first_unit(int b, int h) const {
    return pick4(b, 0, o1, o2, o3) + h * chunks(b);
  }
};
// Attention units are chunks of ATT_CH = 128 keys.
using StreamLens = StreamLensT<ATT_CH>;

// Reads the lane's 4 key and 4 value blocks (at kva, 1 KB apart) and waits
// for the reads. The copies that filled them must have landed.
__device__ __forceinline__ void att_read_kv(unsigned kva, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(vr[0]), "=&v"(vr[1]),
        "=&v"(vr[2]), "=&v"(vr[3])
      : "v"(kva)
      : "memory");
}

// LDS reads of the attention phase that the compiler must not see: it would
// make every LDS read wait for all global-to-LDS copies in flight. Each reads
// and waits for its own results.
// Four 16-byte reads at addr + 64 i.
__device__ __forceinline__ void att_read_p(unsigned addr, f32x4 (&r)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:64\n\t"
      "ds_read_b128 %2, %4 offset:128\n\t"
      "ds_read_b128 %3, %4 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(addr)
      : "memory");
}
// A write-through store that is exactly one vector memory instruction, so the
// attention loop can count it in its waits.
__device__ __forceinline__ void att_store(gptr<float> p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
// Merge of one (stream, head) pair by a single wave: the chunk partials in
// chunk order (groups of 16, each group's maximum first), then the block's
// own keys (causal within the block). Lane (j, r) = (lane / 16, lane % 16)
// makes dims 8 r .. 8 r + 7 of block row j and stores them as f16.
__device__ __forceinline__ void attn_merge_wave(Args& a_, int l_, int b_, int h_,
                                                          int n_) {
  const auto l = uni(l_);
  const auto b = uni(b_);
  const auto h = uni(h_);
  const auto n = uni(n_);
  Args& a = uni(a_);
  auto& s = a.s;
  const int lane = threadIdx.x & 63, j = lane >> 4, r = lane & 15;
  const int nch = a.nch, nc = (n + ATT_CH - 1) / ATT_CH;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)
  // the block's own rows: query j, keys and values 0..3 (fp32, dims 8 r ..)
  const size_t hb = (size_t)b * BLK * H + h * DH + 8 * r;
  f32x4 qv[2], kv4[4][2], vv4[4][2];
  qv[0] = *reinterpret_cast<const f32x4*>(s.q[l] + hb + j * H);
  qv[1] = *reinterpret_cast<const f32x4*>(s.q[l] + hb + j * H + 4);
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    kv4[i][0] = *reinterpret_cast<const f32x4*>(s.k[l] + hb + i * H);
    kv4[i][1] = *reinterpret_cast<const f32x4*>(s.k[l] + hb + i * H + 4);
    vv4[i][0] = *reinterpret_cast<const f32x4*>(s.v[l] + hb + i * H);
    vv4[i][1] = *reinterpret_cast<const f32x4*>(s.v[l] + hb + i * H + 4);
  }
  // the block part: s_i = q_j . k_i for i <= j
  float sb[BLK];
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) d += qv[0][e] * kv4[i][0][e] + qv[1][e] * kv4[i][1][e];
    sb[i] = i <= j ? row16_sum(d) * qs : -__builtin_inff();
  }
  float M = -__builtin_inff(), Ls = 0.f, O[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) O[e] = 0.f;
  const size_t pb = (size_t)(b * NH + h) * nch * 4 + j;   // (pair, chunk c, row j) at pb + 4 c
  for (int c0 = 0; c0 < nc; c0 += 16) {
    const int cn = min(16, nc - c0);
    // lane (j, r) takes chunk c0 + r's max and sum of row j
    const int cr = c0 + min(r, cn - 1);
    float mc = s.am[l][pb + 4 * cr], lc = s.al[l][pb + 4 * cr];
    if (r >= cn) {
      mc = -__builtin_inff();
      lc = 0.f;
    }
    f32x4 oc[16][2];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const size_t po = (pb + 4 * (size_t)(c0 + min(k, cn - 1))) * DH + 8 * r;
      oc[k][0] = *reinterpret_cast<const f32x4*>(s.ao[l] + po);
      oc[k][1] = *reinterpret_cast<const f32x4*>(s.ao[l] + po + 4);
    }
    const float Mn = fmaxf(M, row16_max(mc));
    const float fs = M == -__builtin_inff() ? 0.f : exp2f(M - Mn);
    const float fc = mc == -__builtin_inff() ? 0.f : exp2f(mc - Mn);
    Ls = Ls * fs + row16_sum(lc * fc);
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] *= fs;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float fk = __shfl(fc, (lane & 48) | k, 64);   // 0 past the group's chunks
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        O[e] += fk * oc[k][0][e];
        O[4 + e] += fk * oc[k][1][e];
      }
    }
    M = Mn;
  }
  float Mb = M;
#pragma unroll
  for (int i = 0; i < BLK; ++i) Mb = fmaxf(Mb, sb[i]);
  const float fs = M == -__builtin_inff() ? 0.f : exp2f(M - Mb);
  Ls *= fs;
#pragma unroll
  for (int e = 0; e < 8; ++e) O[e] *= fs;
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    if (i <= j) {
      const float p = exp2f(sb[i] - Mb);
      Ls += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        O[e] += p * vv4[i][0][e];
        O[4 + e] += p * vv4[i][1][e];
      }
    }
  }
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, f16_checked(O[2 * e] / Ls));
    const uint32_t hi = __builtin_bit_cast(uint16_t, f16_checked(O[2 * e + 1] / Ls));
    packed[e] = lo | (hi << 16);
  }
  gptr<uint16_t> dst = s.o[l] + (size_t)(b * BLK + j) * H + h * DH + 8 * r;
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(dst), "v"(packed) : "memory");
  // the attention loop's waits count only its own copies
  __builtin_amdgcn_s_waitcnt(0);
}

// Waits until the LDS word *p equals want (set by another wave of the
// workgroup); after 0.2 s it sets the round's error word and goes on, so the
// wave still ends.
__device__ __forceinline__ void lds_wait_eq(Args& a, KD_LDS unsigned* p, unsigned want) {
  const unsigned long long t0 = wall_clock64();
  for (unsigned it = 1; __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != want; ++it) {
    if ((it & 63) == 0 && wall_clock64() - t0 > 20000000ull) {
      __hip_atomic_store(&a.s.bar[18 * 32], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The state of one half (64 keys) of a chunk after the 4 key groups are
// summed: lane (g, r) holds row g's unnormalised output at dims 8 r .. + 8
// and the row's max (log2 units) and sum. A chunk's partial is always
// half_merge(first half, second half), whichever waves computed the halves.
struct HalfState {
  f32x4 o0, o1;
  float m, l;
};
// o[j][e]: the wave's per-key-group sums (lane (g, c): keys 4g..4g+3, dims
// 8c..8c+7 of row j); m_run, l_run: row lr's max and sum in lane lr.
__device__ __forceinline__ HalfState half_reduce(const float (&o)[4][8], float m_run, float l_run, int lg) {
  // sum the 4 key groups: groups g and g^2 exchange, g < 2 keeping rows
  // 0, 1 and g >= 2 rows 2, 3; then g and g^1, odd groups keeping the
  // second of their rows -- group g ends with row g, dims 8 lr .. + 8
  float r1[2][8];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x0, x1;
      pl32(o[jj][e], o[2 + jj][e], x0, x1);
      r1[jj][e] = x0 + x1;
    }
  HalfState r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x0, x1;
    pl16(r1[0][e], r1[1][e], x0, x1);
    const float v = x0 + x1;
    if (e < 4) r.o0[e] = v; else r.o1[e - 4] = v;
  }
  // row lg's max and sum from lane lg
  const int mi = __builtin_bit_cast(int, m_run), li = __builtin_bit_cast(int, l_run);
  r.m = __builtin_bit_cast(float, pick4(lg, __builtin_amdgcn_readlane(mi, 0), __builtin_amdgcn_readlane(mi, 1),
                                        __builtin_amdgcn_readlane(mi, 2), __builtin_amdgcn_readlane(mi, 3)));
  r.l = __builtin_bit_cast(float, pick4(lg, __builtin_amdgcn_readlane(li, 0), __builtin_amdgcn_readlane(li, 1),
                                        __builtin_amdgcn_readlane(li, 2), __builtin_amdgcn_readlane(li, 3)));
  return r;
}
__device__ __forceinline__ HalfState half_merge(const HalfState& A, const HalfState& B) {
  const float M = fmaxf(A.m, B.m);
  const float fa = A.m == -__builtin_inff() ? 0.f : exp2f(A.m - M);
  const float fb = B.m == -__builtin_inff() ? 0.f : exp2f(B.m - M);
  HalfState r;
  r.m = M;
  r.l = A.l * fa + B.l * fb;
  r.o0 = A.o0 * fa + B.o0 * fb;
  r.o1 = A.o1 * fa + B.o1 * fb;
  return r;
}


// Read-ahead by single waves, after their own work: worker (workgroup w, wave
// v < nwk) on XCD w % 8 takes the units u = w % 8 (mod 8) of a later phase in
// turn with that XCD's other workers; touch_unit(u) reads what unit u will
// load, one dword per 128-byte line, into the wave's own LDS scratch, with at
// most 8 copies in flight so that the other waves' loads are not held up.
template <class F>
__device__ __forceinline__ void warm_waves(int nwk, int nunits, F&& touch_unit) {
  const int wave = threadIdx.x >> 6;
  const int w = blockIdx.x, G = gridDim.x, x = w & 7;
  const int k = (w >> 3) * nwk + wave, nk = ((G - 1 - x) / 8 + 1) * nwk;
  for (int u = x + 8 * k; u < nunits; u += 8 * nk) touch_unit(u);
}
__device__ __forceinline__ void touch_wave(gptr<const uint8_t> p, size_t bytes, KD_LDS void* dump) {
  for (size_t off = (size_t)(threadIdx.x & 63) * 128; off < bytes; off += 64 * 128) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p + off), dump, 4, 0, 0);
    att_wait_vm<8>();
  }
}
__device__ __forceinline__ void touch_tiles_wave(Mat& W, int t0, int ntile, KD_LDS void* dump) {
  const int KB = W.K >> 6, fmt = uni(W.fmt);
  const size_t cb = fmt == WF_NVFP4 ? 512 : (fmt == WF_BF16 ? 2048 : 1024);
  for (int t = t0; t < t0 + ntile; ++t) {
    const size_t blk = (size_t)t * KB;
    touch_wave(W.w + blk * cb, (size_t)KB * cb, dump);
    if (fmt == WF_FP8) touch_wave(reinterpret_cast<gptr<const uint8_t>>(W.s + blk * 16), (size_t)KB * 64, dump);
    if (fmt == WF_NVFP4) touch_wave(W.s4 + blk * 64, (size_t)KB * 64, dump);
  }
}

// Byte offset of wave w's first attention ring slot.
__device__ __forceinline__ unsigned slot0_bytes(int w) { return (unsigned)(((2 * w) >> 3) * ATT_SLOT_BYTES + ((2 * w) & 7) * ATT_WAVE_BLOCKS * 1024); }
// A four-float write-through store (one vector memory instruction).
__device__ __forceinline__ void att_store4(gptr<float> p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

// Attention of the block rows to the context. Unit u = (stream, head, chunk
// of ATT_CH = 128 keys), computed as two halves of 4 blocks of 16 keys: with
// at most 4 units per workgroup wave pair (2v, 2v + 1) of workgroup g takes
// the units g + G (v + 4 i), one half each; otherwise wave w takes the units
// g + G (w + 8 i), both halves in turn. Each half runs in key order through
// the wave's two LDS ring slots (global-to-LDS copies, the next block in
// flight while one is computed), per block
//   scores  S^T[key][j] = K Q^T on the matrix cores (16x16x32 bf16): keys as
//           the A operand (lane: key lane%16, dims 32kb + 8(lane/16)), the
//           queries (pre-scaled by log2(e)/sqrt(128)) split into bf16 hi + lo
//           as the B operand (column j < 4 of the 4 block rows), the hi and
//           lo products in two accumulators added at the end;
//   softmax running max and sum per row j (log2 units), the output rescaled
//           by the growth of the max;
//   P V     on the vector units: lane (g, c) adds keys 4g..4g+3 of the block
//           for dims 8c..8c+7 of all 4 rows (the probabilities pass through
//           the wave's own LDS area).
// The chunk's partial (max, sum, unnormalised output of each row) is the
// merge of its two half states, the same arithmetic whichever waves computed
// them; it is stored at its slot and the pair's counter counts it. The wave
// that counts the pair's last chunk merges the pair's partials in chunk order
// (so a stream's result does not depend on the batch around it) with the
// block's own keys.
__device__ __attribute__((noinline, not_tail_called)) void ph_attn(Args& a_, int l_, SyncState sy,
                                                  bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = uni(wave);
  const int lr = lane & 15, lg = lane >> 4;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;
  lds_f s_p = (lds_f)g_att_small + wave_s * 64;   // the wave's probabilities [4][16]

  StreamLens sl;
  sl.load(a);  // an input: read before the arrival
  const int U = sl.total;
  auto kb_l = a.kv.k[l], vb_l = a.kv.v[l];
  const long long kv_ss = a.kv.ss, kv_sh = a.kv.sh, kv_sl = a.kv.sl;
  const int kv_cap = a.kv.cap;
  const int nch = a.nch;
  auto q_l = s.q[l];
  const unsigned ring0 = (unsigned)(uintptr_t)&g_att_ring[0][0][0];

  // With at most 4 units per workgroup the two halves of a unit run on the
  // wave pair (2v, 2v + 1) and the second half's state reaches the first
  // wave through LDS (x_area: [64 lanes][8] outputs, [4] maxima, [4] sums,
  // then a ready flag and an acknowledgement); otherwise one wave computes
  // both halves, one after the other.
  const bool split = U <= 4 * G;
  const int pv = wave_s >> 1, half = wave_s & 1;
  lds_f x_area = (lds_f)g_att_small + 512 + pv * 528;
  KD_LDS unsigned* x_flag = reinterpret_cast<KD_LDS unsigned*>(x_area + 520);
  KD_LDS unsigned* x_ack = x_flag + 1;
  if (sync) {
    grid_arrive(a, sy);
    grid_wait(a, sy);
  }
  if (threadIdx.x < 4) {
    lds_f xa = (lds_f)g_att_small + 512 + threadIdx.x * 528;
    *reinterpret_cast<KD_LDS unsigned*>(xa + 520) = 0u;
    *reinterpret_cast<KD_LDS unsigned*>(xa + 521) = 0u;
  }
  lds_sync();
  trace_mark(a, sy, 2);
  // each wave owns two LDS ring slots of 8 KB (one 16-key block each): one
  // block is computed while the next is in flight
  constexpr int ns = 2;
  const int slot0 = wave_s * ns;
  const int k0 = split ? 4 * half : 0, k1 = split ? k0 + 4 : 8;
  unsigned iter = 0;
  bool merged = false, worked = false;
  for (int u = split ? wg + G * pv : wg + G * wave_s; u < U; u += split ? 4 * G : 8 * G, ++iter) {
    int b, c, h;
    worked = true;
    sl.unit(u, b, c, h);
    const int n = sl.vis(b), fp = sl.first(b);
    auto kbase = kb_l + b * kv_ss + h * kv_sh;
    auto vbase = vb_l + b * kv_ss + h * kv_sh;
    // slot of the chunk's first key; keys past the visible rows are clamped
    // to the last one and masked out of the scores
    const int s0 = (fp + c * ATT_CH) % kv_cap;
    const int last = n - 1 - c * ATT_CH;
    auto slot_of = [&](int off) {
      int sl_ = s0 + min(off, last);
      return sl_ - (sl_ >= kv_cap ? kv_cap : 0);
    };
    // block k (16 keys) of the chunk comes by global-to-LDS copies into the
    // wave's ring slot (k - k0) % ns: lane (key lr, group lg) brings key
    // dims 32 kb + 8 lg .. + 8 (kb = 0..3), lane (group g = lg, c = lr)
    // brings key 4 g + t, dims 8 c .. + 8 (t = 0..3); 8 copies per block
    auto slot_addr = [&](int k) {   // byte offset of block k's slot in the ring
      const int sl_ = slot0 + (k - k0) % ns;
      return (unsigned)((sl_ >> 3) * ATT_SLOT_BYTES + (sl_ & 7) * ATT_WAVE_BLOCKS * 1024);
    };
    auto copy_blk = [&](int k) __attribute__((always_inline)) {
      KD_LDS u32x4* dst = (KD_LDS u32x4*)((KD_LDS char*)&g_att_ring[0][0][0] + slot_addr(k));
      const size_t krow = (size_t)slot_of(16 * k + lr) * kv_sl;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kbase + krow + 32 * kb + 8 * lg),
                                         (KD_LDS void*)(dst + kb * 64), 16, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(vbase + (size_t)slot_of(16 * k + 4 * lg + t) * kv_sl + 8 * lr),
            (KD_LDS void*)(dst + (4 + t) * 64), 16, 0, 0);
    };
    // the pair's 4 query rows as the B operand: lane (lr < 4, lg) takes row
    // lr, dims 32 kb + 8 lg .. + 8 (loaded before the first two blocks'
    // copies, so the first block's wait covers them)
    bf16x8 qh[4], ql[4];
    {
      const float* qp = q_l + (size_t)(b * 4 + min(lr, 3)) * H + h * DH + 8 * lg;
      f32x4 qx[8];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        qx[2 * kb] = *reinterpret_cast<const f32x4*>(qp + 32 * kb);
        qx[2 * kb + 1] = *reinterpret_cast<const f32x4*>(qp + 32 * kb + 4);
      }
      for (int k = k0; k < k0 + ns; ++k) copy_blk(k);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 x0 = qx[2 * kb], x1 = qx[2 * kb + 1];
        float qv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qv[e] = lr < 4 ? x0[e] * qs : 0.f;
          qv[4 + e] = lr < 4 ? x1[e] * qs : 0.f;
        }
        split_bf16(qv, qh[kb], ql[kb]);
      }
    }
    float m_run = -__builtin_inff(), l_run = 0.f;
    float o[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    HalfState hA;   // the first half's state when one wave computes both
#pragma unroll 1
    for (int k = k0; k < k1; ++k) {
      if (k == 4 && !split) {
        hA = half_reduce(o, m_run, l_run, lg);
        m_run = -__builtin_inff();
        l_run = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
      }
      // block k has landed once at most the later blocks' copies (8 each)
      // are in flight; its slot is refilled with block k + ns after the read
      att_wait_blocks(min(ns - 1, k1 - 1 - k));
      u32x4 kk[4], vv[4];
      att_read_kv(ring0 + slot_addr(k) + lane * 16, kk, vv);
      if (k + ns < k1) copy_blk(k + ns);
      // two independent accumulation chains (the queries' bf16 high and low
      // parts), added at the end
      f32x4 acch = {0.f, 0.f, 0.f, 0.f}, accl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kx = __builtin_bit_cast(bf16x8, kk[kb]);
        acch = mfma_bf16(kx, qh[kb], acch);
        accl = mfma_bf16(kx, ql[kb], accl);
      }
      // lane holds S^T[key 4 lg + e][j = lr] of the block's 16 keys
      float sc[4], mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = 16 * k + 4 * lg + e <= last ? acch[e] + accl[e] : -__builtin_inff();
        mx = fmaxf(mx, sc[e]);
      }
      {
        float r0, r1;
        pl16(mx, mx, r0, r1);   // the max over lane rows (l, l ^ 16)
        mx = fmaxf(r0, r1);
        pl32(mx, mx, r0, r1);   // and over lane halves
        mx = fmaxf(r0, r1);
      }
      const float m_new = fmaxf(m_run, mx);
      // rescale of the state so far (0 while it is empty)
      const float alpha = m_run == -__builtin_inff() ? 0.f : exp2f(m_run - m_new);
      float pe[4], ls = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = sc[e] == -__builtin_inff() ? 0.f : exp2f(sc[e] - m_new);
        ls += pe[e];
      }
      {
        float r0, r1;
        pl16(ls, ls, r0, r1);
        ls = r0 + r1;
        pl32(ls, ls, r0, r1);
        ls = r0 + r1;
      }
      l_run = l_run * alpha + ls;
      m_run = m_new;
      if (lr < 4) *reinterpret_cast<KD_LDS f32x4*>(s_p + lr * 16 + 4 * lg) = f32x4{pe[0], pe[1], pe[2], pe[3]};
      // the rescale factor of row j lives in lane j
      float aj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        aj[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), j));
      // P V: pj[j] = probabilities of row j, keys 4g .. 4g+3 (the wave's own
      // LDS writes complete before its reads)
      f32x4 pj[4];
      att_read_p((unsigned)(uintptr_t)(s_p + 4 * lg), pj);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] *= aj[j];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float vf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vf[2 * i] = u2f(vv[t][i] << 16);
          vf[2 * i + 1] = u2f(vv[t][i] & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[j][e] += pj[j][t] * vf[e];
      }
    }
    HalfState hB = half_reduce(o, m_run, l_run, lg);
    if (split) {
      if (half == 1) {
        // the second half's state to the first wave of the pair, once it
        // has taken the previous one
        lds_wait_eq(a, x_ack, iter);
        *reinterpret_cast<KD_LDS f32x4*>(x_area + lane * 8) = hB.o0;
        *reinterpret_cast<KD_LDS f32x4*>(x_area + lane * 8 + 4) = hB.o1;
        if (lr == 0) {
          x_area[512 + lg] = hB.m;
          x_area[516 + lg] = hB.l;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the writes have landed
        if (lane == 0) __hip_atomic_store(x_flag, iter + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        continue;
      }
      hA = hB;
      lds_wait_eq(a, x_flag, iter + 1);
      hB.o0 = *reinterpret_cast<KD_LDS f32x4*>(x_area + lane * 8);
      hB.o1 = *reinterpret_cast<KD_LDS f32x4*>(x_area + lane * 8 + 4);
      hB.m = x_area[512 + lg];
      hB.l = x_area[516 + lg];
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if (lane == 0) __hip_atomic_store(x_ack, iter + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const HalfState hc = half_merge(hA, hB);
    // the chunk's partial at its slot: row lg, dims 8 lr .. + 8; the row's
    // max and sum from lane (lg, 0)
    const size_t pb = ((size_t)(b * NH + h) * nch + c) * 4;
    att_store4(s.ao[l] + (pb + lg) * DH + 8 * lr, hc.o0);
    att_store4(s.ao[l] + (pb + lg) * DH + 8 * lr + 4, hc.o1);
    if (lr == 0) {
      att_store(s.am[l] + pb + lg, hc.m);
      att_store(s.al[l] + pb + lg, hc.l);
    }
    // counted once the wave's stores are acknowledged; the wave that counts
    // the pair's last chunk merges the pair and resets its counter
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    auto cnt = &s.att_cnt[((l * SB_MAX + b) * NH + h) * 32];
    unsigned before = 0;
    if (lane == 0) before = add_rlx(cnt, 1u);
    before = (unsigned)__builtin_amdgcn_readlane((int)before, 0);
    if (before + 1 == (unsigned)sl.chunks(b)) {
      if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      attn_merge_wave(a, l, b, h, n);
      merged = true;
    }
  }
  trace_mark(a, sy, 3);
  // the waves that computed units and merged none read ahead the output
  // projection's weights (one tile per unit) on the XCDs that will load them
  // (not in the persistent kernel, where a late arrival holds up the barrier)
  if (!sync && worked && !merged) {
    const int nwk = min(8, split ? 2 * ((U + G - 1) / G) : (U + G - 1) / G);
    KD_LDS void* dump = (KD_LDS void*)((KD_LDS char*)&g_att_ring[0][0][0] + slot0_bytes(wave_s));
    auto& L = a.d.layer[l];
    warm_waves(nwk, HT, [&](int u) { touch_tiles_wave(L.wo, u, 1, dump); });
    warm_done();
  }
  // pairs of streams with no visible context attend to the block only:
  // (stream, head) i by wave 0 of workgroup i
  const int nbh = a.B * NH;
  if (wg < nbh && wave_s == 0 && sl.vis(wg / NH) == 0) attn_merge_wave(a, l, wg / NH, wg % NH, 0);
  trace_mark(a, sy, 4);
}

// Attention over the rotated 4-bit cache (the 4-bit KV article, "What we do"):
// the units, chunk partials, counters and last-arriving merges of ph_attn.
// Wave w of workgroup g takes the units g + G (w + 8 i), each whole: the
// chunk's 8 blocks of 16 keys in key order, straight into registers by buffer
// loads (K codes, V codes, each key's fp16 scale and offset), one block
// ahead of the one computed. Per unit the wave turns the block rows' queries
// by the layer's rotation (signs, then an in-wave Walsh-Hadamard transform)
// through its own LDS area and takes them as the B operand (f16 hi + lo). Per block: scores = scale * (q_rot . codes)
// + offset * sum(q_rot), with the codes as f16 subnormals on the matrix
// cores; an online softmax; P V on the matrix cores as well (16x16x16, V
// codes as the A operand, p * scale as the B operand), the offsets' share
// added per row. One wave makes each chunk's partial, so it does not depend
// on the batch.
__device__ __attribute__((noinline, not_tail_called)) void ph_attn_q4(Args& a_, int l_, SyncState sy,
                                                     bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = uni(wave);
  const int lr = lane & 15, lg = lane >> 4;
  const float qs = 0.08838834764831845f * 1.4426950408889634f;
  lds_f s_q = (lds_f)g_att_small + wave_s * 528;   // the wave's rotated queries [4][128], then [4] their sums

  StreamLens sl;
  sl.load(a);  // an input: read before the arrival
  const int U = sl.total;
  const uint8_t* k_l = reinterpret_cast<const uint8_t*>(a.kv.k[l]);
  const uint8_t* v_l = reinterpret_cast<const uint8_t*>(a.kv.v[l]);
  const uint16_t* ks_l = a.kv.kso[l];
  const uint16_t* vs_l = a.kv.vso[l];
  const long long kv_ss = a.kv.ss, kv_sh = a.kv.sh;
  const uint32_t kv_sl = (uint32_t)a.kv.sl;
  const int kv_cap = a.kv.cap;
  const uint32_t span = (uint32_t)((kv_cap - 1) * a.kv.sl + 1);   // rows of one (stream, head)
  auto q_l = s.q[l];
  const float* signs = a.d.kv_signs + l * DH;
  const int nch = a.nch;

  if (sync) {
    grid_arrive(a, sy);
    grid_wait(a, sy);
  }
  trace_mark(a, sy, 2);

  // One block's keys for this wave: key lr's K codes (dims 32 lg ..), keys
  // 4 lg + t's V codes (dims 8 lr ..), key lr's (scale, offset) pairs.
  struct KvRegs {
    u32x4 k;
    uint32_t v[4];
    uint32_t ks, vs;
  };
  constexpr int NB = ATT_CH / 16;
  for (int u = wg + G * wave_s; u < U; u += 8 * G) {
    int b, c, h;
    sl.unit(u, b, c, h);
    const int n = sl.vis(b), fp = sl.first(b);
    // the rows of one (stream, head) are read through buffer resources
    // (32-bit offsets; the hardware returns 0 past the span, which the host
    // checks fits 4 GiB); keys past the visible rows are clamped to the last
    // one and masked in the scores
    const size_t row0 = (size_t)(b * kv_ss + h * kv_sh);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k_l + row0 * 64), (short)0, span * 64, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v_l + row0 * 64), (short)0, span * 64, 0x00020000);
    const __amdgpu_buffer_rsrc_t rks =
        __builtin_amdgcn_make_buffer_rsrc((void*)(ks_l + row0 * 2), (short)0, span * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vs_l + row0 * 2), (short)0, span * 4, 0x00020000);
    const int s0 = (fp + c * ATT_CH) % kv_cap;
    const int last = n - 1 - c * ATT_CH;
    auto row_of = [&](int off) {
      const int r_ = s0 + min(off, last);
      return (uint32_t)(r_ - (r_ >= kv_cap ? kv_cap : 0)) * kv_sl;
    };
    auto load_blk = [&](int k, KvRegs& r) __attribute__((always_inline)) {
      const uint32_t rk0 = row_of(16 * k + lr);
      r.k = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, rk0 * 64 + 16 * lg, 0, 0));
      r.ks = __builtin_amdgcn_raw_buffer_load_b32(rks, rk0 * 4, 0, 0);
      r.vs = __builtin_amdgcn_raw_buffer_load_b32(rvs, rk0 * 4, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        r.v[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, row_of(16 * k + 4 * lg + t) * 64 + 4 * lr, 0, 0);
    };
    KvRegs cur, nxt;
    load_blk(0, cur);
    f16x8 qh[4], ql[4];
    float qsum;
    {
      // row j's query turned by R: R q = H (s * q) / sqrt(128), scaled like
      // the scores (1/sqrt(128) * log2(e)); made again for every unit, so
      // nothing of it stays live across a merge
      const float f = 0.08838834764831845f * qs;
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        const float* qp = q_l + (size_t)(b * BLK + j) * H + h * DH;
        float y0 = qp[lane] * signs[lane], y1 = qp[lane + 64] * signs[lane + 64];
        fwht128(y0, y1, lane);
        y0 *= f;
        y1 *= f;
        s_q[j * DH + lane] = y0;
        s_q[j * DH + lane + 64] = y1;
        const float t = wave_sum(y0 + y1);
        if (lane == 0) s_q[BLK * DH + j] = t;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = lr < BLK ? s_q[lr * DH + 32 * lg + 8 * kb + e] : 0.f;
          const _Float16 hh = (_Float16)v;
          qh[kb][e] = hh;
          ql[kb][e] = (_Float16)(v - (float)hh);
        }
      qsum = lr < BLK ? s_q[BLK * DH + lr] : 0.f;
    }
    float m_run = -__builtin_inff(), l_run = 0.f;
    float o[8][4];   // lane (lr < 4, lg): row lr, dims 32 lg + 8 e + t at o[t][e]
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[t][e] = 0.f;
#pragma unroll 1
    for (int k = 0; k < NB; ++k) {
      load_blk(min(k + 1, NB - 1), nxt);   // the next block's keys go out first
      // the scale and offset pairs of keys 4 lg + e come from lanes 4 lg + e
      uint32_t ks[4], vs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ks[e] = __shfl(cur.ks, 4 * lg + e, 64);
        vs[e] = __shfl(cur.vs, 4 * lg + e, 64);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f16x8 kk = nib8_f16(cur.k[kb]);
        acc = mfma_f16(kk, qh[kb], acc);
        acc = mfma_f16(kk, ql[kb], acc);
      }
      // lane (lr, lg): acc[e] = q_rot[lr] . codes[key 4 lg + e] * 2^-24
      float sc[4], mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float ksc, kof;
        so_unpack(ks[e], ksc, kof);
        const int key = c * ATT_CH + 16 * k + 4 * lg + e;
        sc[e] = key < n ? (ksc * KD_2P24) * acc[e] + kof * qsum : -__builtin_inff();
        mx = fmaxf(mx, sc[e]);
      }
      {
        float r0, r1;
        pl16(mx, mx, r0, r1);
        mx = fmaxf(r0, r1);
        pl32(mx, mx, r0, r1);
        mx = fmaxf(r0, r1);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -__builtin_inff() ? 0.f : exp2f(m_run - m_new);
      f16x4 pb;
      float ls = 0.f, ws = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = sc[e] == -__builtin_inff() ? 0.f : exp2f(sc[e] - m_new);
        float vsc, vof;
        so_unpack(vs[e], vsc, vof);
        ls += pe;
        ws += pe * vof;
        pb[e] = (_Float16)(pe * vsc);
      }
      {
        float r0, r1;
        pl16(ls, ls, r0, r1);
        ls = r0 + r1;
        pl32(ls, ls, r0, r1);
        ls = r0 + r1;
        pl16(ws, ws, r0, r1);
        ws = r0 + r1;
        pl32(ws, ws, r0, r1);
        ws = r0 + r1;
      }
      l_run = l_run * alpha + ls;
      m_run = m_new;
      // even nibbles (dims 8 lr + 2m) and odd nibbles (8 lr + 2m + 1) per key
      uint32_t ev[4], od[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ev[e] = cur.v[e] & 0x0F0F0F0Fu;
        od[e] = (cur.v[e] >> 4) & 0x0F0F0F0Fu;
      }
      f32x4 oa[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) oa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[t][e] = o[t][e] * alpha + (oa[t][e] * KD_2P24 + ws);
      cur = nxt;
    }
    // the chunk's partial at its slot: lanes (lr < 4, lg) store row lr's
    // dims 32 lg + 8 e .. + 8; lane (lr, 0) its max and sum
    const size_t pb = ((size_t)(b * NH + h) * nch + c) * 4;
    if (lr < BLK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gptr<float> dst = s.ao[l] + (pb + lr) * DH + 32 * lg + 8 * e;
        att_store4(dst, f32x4{o[0][e], o[1][e], o[2][e], o[3][e]});
        att_store4(dst + 4, f32x4{o[4][e], o[5][e], o[6][e], o[7][e]});
      }
      if (lg == 0) {
        att_store(s.am[l] + pb + lr, m_run);
        att_store(s.al[l] + pb + lr, l_run);
      }
    }
    // counted once the stores are acknowledged; the wave that counts the
    // pair's last chunk merges the pair and resets its counter
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    auto cnt = &s.att_cnt[((l * SB_MAX + b) * NH + h) * 32];
    unsigned before = 0;
    if (lane == 0) before = add_rlx(cnt, 1u);
    before = (unsigned)__builtin_amdgcn_readlane((int)before, 0);
    if (before + 1 == (unsigned)sl.chunks(b)) {
      if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      attn_merge_wave(a, l, b, h, n);
    }
  }
  trace_mark(a, sy, 3);
  // pairs of streams with no visible context attend to the block only
  const int nbh = a.B * NH;
  if (wg < nbh && wave_s == 0 && sl.vis(wg / NH) == 0) attn_merge_wave(a, l, wg / NH, wg % NH, 0);
  trace_mark(a, sy, 4);
}

// Output projection: x_{out} = x_{in} + W_o o, with the gained copy and
// per-tile sums of squares; one 16-column tile per unit. The workgroups
// without a tile warm the weights of the down projection two phases on.
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_o(Args& a_, int l_, lds_f red, SyncState sy,
                                               bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int R = a.R, xin = xs_in(l), xout = xs_o(l);
  const auto gain = L.ffn_norm;
  bool first = sync;
  for (int u = wg; u < HT; u += G) {
    const ASrc A{s.o[l], H, 0, nullptr, 0, R};
    gemm_unit<WF, 1, 5, 8, false>(a, sy, first, L.wo, u, 1, 0, A, red, no_rms(),
                              [&](int, int m, int n, float v) {
                                const int col = u * 16 + n;
                                const bool ok = m < R;
                                const float x = ok ? s.x[xin][m * H + col] + v : 0.f;
                                put_x(s, xout, gain, m, col, u, n, x, ok);
                              });
    first = false;
  }
  if (first) grid_sync(a, sy);
  // down units u: tile pair u / DOWN_KS, input third u % DOWN_KS (not in
  // the persistent kernel, where an idle workgroup's late arrival would hold
  // up the next barrier)
  if (!sync) {
    constexpr int DKB = FF / 64 / DOWN_KS;
    warm(HT, HT / 2 * DOWN_KS, [&](int u) {
      const int tp = u / DOWN_KS, p = u - tp * DOWN_KS;
      touch_tiles(L.down, 2 * tp, 2, p * DKB, DKB);
    });
    warm_done();
  }
}

// x_{out} = x_{in} + W_down h, with the 6144 inputs split in DOWN_KS thirds
// across workgroups: unit u covers the tile pair u / DOWN_KS (32 output
// columns) over third u % DOWN_KS, so that 240 units spread over the grid and
// each loads a third of the activations. Every unit stores its partial; the
// last of a pair's units to finish (counter) adds the thirds in a fixed order
// and runs the residual epilogue.
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_down(Args& a_, int l_, lds_f red, SyncState sy,
                                                  bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int R = a.R;
  const int xin = xs_o(l), xout = xs_d(l);
  const auto gain = gain_after_down(a, l);
  constexpr int NT = 2, KBS = FF / 64 / DOWN_KS / 8;
  static_assert(KBS * 8 * DOWN_KS * 64 == FF, "down split");
  constexpr int NU = HT / NT * DOWN_KS;
  auto part = s.dpart[l];
  KD_LDS unsigned* s_last = reinterpret_cast<KD_LDS unsigned*>(red + 8192 + 64);
  bool first = sync;
  for (int u = wg; u < NU; u += G) {
    const int tp = u / DOWN_KS, p = u - tp * DOWN_KS;
    const ASrc A{s.h[l], FF, 0, nullptr, 0, R};
    // thread (i, m, n) = (tid / 256, (tid / 16) % 16, tid % 16) holds one
    // output of the pair after the epilogue's reduction over the 8 waves
    float mine = 0.f;
    gemm_unit<WF, NT, KBS, 8, false>(a, sy, first, L.down, tp * NT, NT, p * KBS * 8, A, red, no_rms(),
                                 [&](int i, int m, int n, float v) {
                                   mine = v;
                                   if (m < R) st_wt(&part[((size_t)p * SR_MAX + m) * H + (tp * NT + i) * 16 + n], v);
                                 });
    first = false;
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
      auto cnt = &s.down_cnt[(l * (HT / 2) + tp) * 32];
      const bool last = add_rlx(cnt, 1u) == (unsigned)(DOWN_KS - 1);
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = last ? 1u : 0u;
    }
    lds_sync();
    if (*s_last) {
      const int it = threadIdx.x, i = it >> 8, m = (it >> 4) & 15, n = it & 15;
      const int tile = tp * NT + i, col = tile * 16 + n;
      const bool ok = m < R;
      float pv[DOWN_KS];
#pragma unroll
      for (int q = 0; q < DOWN_KS; ++q)
        pv[q] = q == p ? mine : (ok ? part[((size_t)q * SR_MAX + m) * H + col] : 0.f);
      float v = pv[0];
#pragma unroll
      for (int q = 1; q < DOWN_KS; ++q) v += pv[q];
      const float x = ok ? s.x[xin][m * H + col] + v : 0.f;
      put_x(s, xout, gain, m, col, tile, n, x, ok);
    }
    lds_sync();
  }
  if (first) grid_sync(a, sy);
}

// h = silu(gate / rms) * (up / rms) with gate, up = W (g_f * x).
template <int WF>
__device__ __attribute__((noinline, not_tail_called)) void ph_gu(Args& a_, int l_, lds_f red,
                                                SyncState sy, bool sync) {
  const auto l = uni(l_);
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& L = a.d.layer[l];
  const int R = a.R, src = xs_o(l);
  lds_f inv = red + 8192;
  constexpr int NT = 3, NU = GU / 16 / NT;
  bool first = sync;
  for (int u = wg; u < NU; u += G) {
    const ASrc A{s.xg[src], H, 0, nullptr, 0, R};
    gemm_unit<WF, NT, 5, 8, false>(
        a, sy, first, L.gu, u * NT, NT, 0, A, red, RmsRows{s.ssq[src], R, 0, a.eps, inv, {}},
        [&](int i, int m, int n, float v) {
          const int t = u * NT + i;
          const float val = m < R ? v * inv[m] : 0.f;
          const float up = dpp_f<DPP_ROR8>(val);
          if (m < R && n < 8) st_wt_h(&s.h[l][m * FF + 8 * t + n], silu(val) * up);
        });
    first = false;
  }
  if (first) grid_sync(a, sy);
}

// The end of every head phase: the workgroup's per-row argmax candidates go
// out; the last workgroup to finish reduces every workgroup's candidates to
// the target ids (and publishes a timed-out wait and the f16 range flag).
__device__ __forceinline__ void head_finish(Args& a, KD_LDS unsigned long long* best, KD_LDS unsigned* s_flag,
                                            SyncState sy) {
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int R = a.R;
  lds_sync();
  const int t = threadIdx.x;
  if (t < SR_MAX) st_wt64(&s.cand[wg * SR_MAX + t], best[t]);
  trace_mark(a, sy, 4);
  // what the last workgroup needs besides the candidates is final before
  // this phase (the timed-out-wait word, the f16 range flag, the caller's
  // ids): read now, off its path
  unsigned failed = 0u, ranged = 0u;
  if (t == 0) {
    failed = ld_rlx(&s.bar[18 * 32]);
    ranged = __hip_atomic_load(&g_f16_range, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int r = t >> 5, l32 = t & 31;
  const bool ok = r < R && l32 == 0 && id_row_valid(a.anchor, a.pred, a.pred_stride, r / BLK, r % BLK, d.V);
  // the last workgroup to finish reduces every workgroup's candidates
  __builtin_amdgcn_s_waitcnt(0);  // the candidate stores are acknowledged
  __syncthreads();
  if (t == 0) {
    auto cnt = &s.bar[19 * 32];
    const unsigned v = add_rlx(cnt, 1u);
    const bool last = v == (unsigned)(G - 1);
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[0] = last ? 1u : 0u;
    s_flag[1] = failed;
  }
  lds_sync();
  if (!s_flag[0]) return;
  // every candidate load is issued before the first is needed
  unsigned long long kc[MAX_G / 32];
#pragma unroll
  for (int i = 0; i < MAX_G / 32; ++i) {
    const int gi = l32 + 32 * i;
    kc[i] = r < R && gi < G ? s.cand[gi * SR_MAX + r] : 0ull;
  }
  unsigned long long k = 0ull;
#pragma unroll
  for (int i = 0; i < MAX_G / 32; ++i) k = u64_max(k, kc[i]);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) k = u64_max(k, shfl_xor_u64s(k, m));
  const bool fail = s_flag[1] != 0u;
  if (t == 0 && a.status) {
    if (fail) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    // every workgroup's f16 stores of the round are done: status[1] is the range word
    if (ranged) {
      __hip_atomic_store(&g_f16_range, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  } else if (t == 0 && ranged) {
    __hip_atomic_store(&g_f16_range, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (r < R && l32 == 0)
    a.out_ids[r] = fail ? -2 : (k && ok ? d.vocab[0xffffffffu - (uint32_t)(k & 0xffffffffu)] : -1);
}

// NVFP4 head over 16-row vocab tiles (HEAD_NT per unit): wave w takes the
// 128-input groups kg0(w)..kg1(w); the next unit's codes are loaded while one
// is computed. Argmax candidates per row are kept per workgroup; the last
// workgroup to finish reduces them to the output ids.
__device__ __attribute__((noinline, not_tail_called)) void ph_head(Args& a_, lds_f red, SyncState sy,
                                                  bool sync) {
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = a.R, VT = d.VT, VD = d.VD;
  constexpr int KG = H / 128;
  const int wave_s = uni(wave);
  const int kg0 = (KG * wave_s) >> 3, kg1 = (KG * (wave_s + 1)) >> 3, ng = kg1 - kg0;  // 2 or 3
  const int src = a.nl == 0 ? 0 : xs_d(a.nl - 1);
  const int nunits = (VT + HEAD_NT - 1) / HEAD_NT;
  lds_f inv = red + 8192;
  KD_LDS unsigned long long* best = reinterpret_cast<KD_LDS unsigned long long*>(red + 8192 + 32);  // [16]
  KD_LDS unsigned* s_flag = reinterpret_cast<KD_LDS unsigned*>(red + 8192 + 64);

  // unit u < nunits: tiles past the last repeat it (their columns are past
  // the vocabulary and masked); a wave with 2 input groups repeats its last
  // group in slot 2 and skips it
  // (block addresses are wave-uniform, so they stay in scalar registers and
  // only the lane offset is a vector one)
  auto load_unit = [&](int u, u32x4 (&q)[HEAD_NT][3], uint32_t (&sv)[HEAD_NT][3]) {
#pragma unroll
    for (int i = 0; i < HEAD_NT; ++i)
#pragma unroll
      for (int gg = 0; gg < 3; ++gg) {
        const int vt = min(u * HEAD_NT + i, VT - 1);
        const size_t blk = (size_t)vt * KG + kg0 + min(gg, ng - 1);
        q[i][gg] = *(uni(reinterpret_cast<gptr<const u32x4>>(d.hq + blk * 1024)) + lane);
        sv[i][gg] = *(uni(reinterpret_cast<gptr<const uint32_t>>(d.hs + blk * 256)) + lane);
      }
  };

  if (sync) {
    grid_arrive(a, sy);
    if (is_poll_wave()) grid_poll(a, sy);
    lds_sync();
  }
  trace_mark(a, sy, 2);
  if (threadIdx.x < SR_MAX) best[threadIdx.x] = 0ull;
  RmsRows rms{s.ssq[src], R, 0, a.eps, inv, {}};
  // the activations (written by the previous phase) are loaded before the
  // first unit's codes, so that they land first (a wave's loads complete in
  // issue order)
  rms.issue();
  const int ar = min(lane & 15, R - 1);
  // A operand (g_o * x in f16) for this wave's inputs, kept for all units
  f16x8 ah[3][4];
#pragma unroll
  for (int gg = 0; gg < 3; ++gg)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // rows past R repeat row R-1 (their logits are discarded); slot 2 of a
      // wave with 2 input groups repeats group 1 and is skipped
      const int c0 = (kg0 + min(gg, ng - 1)) * 128 + t * 32 + 8 * (lane >> 4);
      ah[gg][t] = *reinterpret_cast<gptr<const f16x8>>(s.xg[src] + ar * H + c0);
    }
  // two register sets of codes and scales alternate (an unrolled pair of
  // units, so that no copy between them makes the compiler wait for loads in
  // flight); units past the last repeat it and are skipped
  u32x4 qa[HEAD_NT][3], qb[HEAD_NT][3];
  uint32_t sa[HEAD_NT][3], sb[HEAD_NT][3];
  const int ulast = max(nunits - 1, 0);
  load_unit(min(wg, ulast), qa, sa);
  rms.finish();
  trace_mark(a, sy, 3);
  auto unit_body = [&](int u, const u32x4 (&q)[HEAD_NT][3], const uint32_t (&sv)[HEAD_NT][3])
                       __attribute__((always_inline)) {
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
          }
      }
    }
#pragma unroll
    for (int i = 0; i < HEAD_NT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * HEAD_NT + i) * 4 + e) * 64 + lane] = acc[i][e];
    lds_sync();
    gemm_epilogue<HEAD_NT>(red, [&](int i, int m, int n, float v) {
      const int voc = (u * HEAD_NT + i) * 16 + n;
      const bool ok = m < R && voc < VD;
      const float logit = ok ? v * inv[m] * d.hg : 0.f;
      if (ok && a.out_logits) a.out_logits[(size_t)m * VD + voc] = logit;
      unsigned long long key = ok ? argmax_key(logit, (uint32_t)voc) : 0ull;
      // max over the 16-lane row (xor 1, 2, then the mirrors of agreeing quads and halves)
      key = u64_max(key, dpp_u64<DPP_XOR1>(key));
      key = u64_max(key, dpp_u64<DPP_XOR2>(key));
      key = u64_max(key, dpp_u64<DPP_HALF_MIRROR>(key));
      key = u64_max(key, dpp_u64<DPP_MIRROR>(key));
      if (n == 0 && key)
        __hip_atomic_fetch_max(&best[m], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    });
    if (u == wg) trace_mark(a, sy, 5);
  };
  for (int u = wg; u < nunits; u += 2 * G) {
    load_unit(min(u + G, ulast), qb, sb);
    unit_body(u, qa, sa);
    if (u + G >= nunits) break;
    load_unit(min(u + 2 * G, ulast), qa, sa);
    unit_body(u + G, qb, sb);
  }
  head_finish(a, best, s_flag, sy);
}

// bf16 (HQ = 1) and block-FP8 (HQ = 2) head slices over the same 16-row
// vocabulary tiles, wave input groups, epilogue and argmax as the NVFP4 head.
// bf16: each f16 activation is split exactly into two bf16 terms (its top 8
// significant bits, and the rest) for the bf16 matrix cores; a unit is one
// tile, whose codes are 4 times the NVFP4 tile's. FP8: e4m3 decoded exactly to
// f16, each 64-input block's product scaled by its row's fp32 scale. Two
// register sets of codes alternate, as in the NVFP4 head.
template <int HQ>
__device__ __attribute__((noinline, not_tail_called)) void ph_head_q(Args& a_, lds_f red, SyncState sy,
                                                    bool sync) {
  Args& a = uni(a_);
  const int G = gridDim.x, wg = blockIdx.x;
  auto& s = a.s;
  auto& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = a.R, VT = d.VT, VD = d.VD;
  constexpr int KG = H / 128;
  constexpr int NTU = HQ == 1 ? 1 : HEAD_NT;   // vocabulary tiles per unit
  constexpr int NQ = HQ == 1 ? 4 : 2;          // 16-byte code loads per tile and input group
  const int wave_s = uni(wave);
  const int kg0 = (KG * wave_s) >> 3, kg1 = (KG * (wave_s + 1)) >> 3, ng = kg1 - kg0;  // 2 or 3
  const int src = a.nl == 0 ? 0 : xs_d(a.nl - 1);
  const int nunits = (VT + NTU - 1) / NTU;
  lds_f inv = red + 8192;
  KD_LDS unsigned long long* best = reinterpret_cast<KD_LDS unsigned long long*>(red + 8192 + 32);  // [16]
  KD_LDS unsigned* s_flag = reinterpret_cast<KD_LDS unsigned*>(red + 8192 + 64);

  // unit u < nunits (tiles past the last repeat it and are masked; a wave
  // with 2 input groups repeats its last group in slot 2 and skips it)
  auto load_unit = [&](int u, u32x4 (&q)[NTU][3][NQ], float (&sv)[NTU][3][2]) {
#pragma unroll
    for (int i = 0; i < NTU; ++i)
#pragma unroll
      for (int gg = 0; gg < 3; ++gg) {
        const int vt = min(u * NTU + i, VT - 1);
        const int kg = kg0 + min(gg, ng - 1);
        if constexpr (HQ == 1) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            q[i][gg][t] = *(uni(reinterpret_cast<gptr<const u32x4>>(d.hb + ((size_t)vt * (H / 32) + kg * 4 + t) * 512)) + lane);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const size_t blk = (size_t)vt * (H / 64) + kg * 2 + j;
            q[i][gg][j] = *(uni(reinterpret_cast<gptr<const u32x4>>(d.hf8.w + blk * 1024)) + lane);
            sv[i][gg][j] = d.hf8.s[blk * 16 + (lane & 15)];
          }
        }
      }
  };

  if (sync) {
    grid_arrive(a, sy);
    if (is_poll_wave()) grid_poll(a, sy);
    lds_sync();
  }
  trace_mark(a, sy, 2);
  if (threadIdx.x < SR_MAX) best[threadIdx.x] = 0ull;
  RmsRows rms{s.ssq[src], R, 0, a.eps, inv, {}};
  rms.issue();
  const int ar = min(lane & 15, R - 1);
  // A operand (g_o * x in f16) for this wave's inputs, kept for all units
  f16x8 ah[3][4];
#pragma unroll
  for (int gg = 0; gg < 3; ++gg)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c0 = (kg0 + min(gg, ng - 1)) * 128 + t * 32 + 8 * (lane >> 4);
      ah[gg][t] = *reinterpret_cast<gptr<const f16x8>>(s.xg[src] + ar * H + c0);
    }
  u32x4 qa[NTU][3][NQ], qb[NTU][3][NQ];
  float sa[NTU][3][2], sb[NTU][3][2];
  const int ulast = max(nunits - 1, 0);
  load_unit(min(wg, ulast), qa, sa);
  rms.finish();
  // bf16: the activations' exact two-term split, once for all units
  bf16x8 ahh[HQ == 1 ? 3 : 1][4], ahl[HQ == 1 ? 3 : 1][4];
  if constexpr (HQ == 1) {
#pragma unroll
    for (int gg = 0; gg < 3; ++gg)
#pragma unroll
      for (int t = 0; t < 4; ++t) split_f16_bf16(ah[gg][t], ahh[gg][t], ahl[gg][t]);
  }
  trace_mark(a, sy, 3);
  auto unit_body = [&](int u, const u32x4 (&q)[NTU][3][NQ], const float (&sv)[NTU][3][2])
                       __attribute__((always_inline)) {
    f32x4 acc[NTU];
#pragma unroll
    for (int i = 0; i < NTU; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < 3; ++gg) {
      if (gg < ng) {
        if constexpr (HQ == 1) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < NTU; ++i) {
              const bf16x8 w = __builtin_bit_cast(bf16x8, q[i][gg][t]);
              acc[i] = mfma_bf16(ahh[gg][t], w, acc[i]);
              acc[i] = mfma_bf16(ahl[gg][t], w, acc[i]);
            }
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < NTU; ++i) {
              const u32x4 c = q[i][gg][j];
              f32x4 t = {0.f, 0.f, 0.f, 0.f};
              t = mfma_f16(ah[gg][2 * j], e4m3x8_f16(c.x, c.y), t);
              t = mfma_f16(ah[gg][2 * j + 1], e4m3x8_f16(c.z, c.w), t);
              acc[i] += sv[i][gg][j] * t;
            }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NTU; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * NTU + i) * 4 + e) * 64 + lane] = acc[i][e];
    lds_sync();
    gemm_epilogue<NTU>(red, [&](int i, int m, int n, float v) {
      const int voc = (u * NTU + i) * 16 + n;
      const bool ok = m < R && voc < VD;
      const float logit = ok ? v * inv[m] * d.hg : 0.f;
      if (ok && a.out_logits) a.out_logits[(size_t)m * VD + voc] = logit;
      unsigned long long key = ok ? argmax_key(logit, (uint32_t)voc) : 0ull;
      // max over the 16-lane row (xor 1, 2, then the mirrors of agreeing quads and halves)
      key = u64_max(key, dpp_u64<DPP_XOR1>(key));
      key = u64_max(key, dpp_u64<DPP_XOR2>(key));
      key = u64_max(key, dpp_u64<DPP_HALF_MIRROR>(key));
      key = u64_max(key, dpp_u64<DPP_MIRROR>(key));
      if (n == 0 && key)
        __hip_atomic_fetch_max(&best[m], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    });
    if (u == wg) trace_mark(a, sy, 5);
  };
  for (int u = wg; u < nunits; u += 2 * G) {
    load_unit(min(u + G, ulast), qb, sb);
    unit_body(u, qa, sa);
    if (u + G >= nunits) break;
    load_unit(min(u + 2 * G, ulast), qa, sa);
    unit_body(u + G, qb, sb);
  }
  head_finish(a, best, s_flag, sy);
}

// ---------------------------------------------------------------------------
// Phase dispatch
// ---------------------------------------------------------------------------
template <int WF>
__device__ void run_phase(Args& a, int p, lds_f red, SyncState sy, bool sync) {
  if (p == PH_PRE0) return ph_pre0<WF>(a, red, sy);
  if (p == PH_PRE1) return ph_pre1<WF>(a, red, sy, sync);
  if (p == PH_PRE2) return ph_pre2<WF>(a, red, sy, sync);
  if (p == PH_HEAD) {
    const int hf = uni(a.d.head_fmt);
    if (hf == 1) return ph_head_q<1>(a, red, sy, sync);
    if (hf == 2) return ph_head_q<2>(a, red, sy, sync);
    return ph_head(a, red, sy, sync);
  }
  const int l = (p - 3) >> 3, k = (p - 3) & 7;
  switch (k) {
    case PH_SA: return ph_sa<WF>(a, l, red, sy, sync);
    case PH_SU: return ph_su<WF>(a, l, red, sy, sync);
    case PH_QKV: return ph_qkv<WF>(a, l, red, sy, sync);
    case PH_ATTN:
      if (uni(a.kv.fmt) == 1) return ph_attn_q4(a, l, sy, sync);
      return ph_attn(a, l, sy, sync);
    case PH_O: return ph_o<WF>(a, l, red, sy, sync);
    case PH_GU: return ph_gu<WF>(a, l, red, sy, sync);
    case PH_DOWN: return ph_down<WF>(a, l, red, sy, sync);
  }
}

__host__ __device__ int small_phase_count(int nl) {
  int n = 3 + 1;
  for (int l = 0; l < nl; ++l) n += l == 0 ? 5 : 7;
  return n;
}

__host__ __device__ int small_phase_id(int nl, int i) {
  if (i < 3) return i;
  i -= 3;
  for (int l = 0; l < nl; ++l) {
    // SA, SU (layers >= 1), QKV, ATTN, O, GU, DOWN
    const int nk = l == 0 ? 5 : 7;
    if (i < nk) {
      const int k = l == 0 ? i + 2 : i;
      return 3 + 8 * l + (k >= 4 ? k + 1 : k);
    }
    i -= nk;
  }
  return PH_HEAD;
}

constexpr int RED_FLOATS = 8192 + 32 + 32 + 32;   // partials, inv rms, argmax candidates, flag
static_assert(sizeof(g_att_ring) >= RED_FLOATS * sizeof(float), "reduction area");

// The reduction area of the phases other than attention (which has its own).
__device__ __forceinline__ lds_f red_area() { return (lds_f)&g_att_ring[0][0][0]; }

// The argument block lives in device memory (read through scalar loads), so
// no per-lane copy of it is made when it is passed down to the phases.
template <int WF>
__global__ __launch_bounds__(SMALL_WG) void k_small_phase(const SmallArgs* __restrict__ ap, int p,
                                                         int slot) {
  const unsigned long long t_entry = wall_clock64();
  const SyncState sy{0u, slot};
  Args& a = *(Args*)ap;
  run_phase<WF>(a, p, red_area(), sy, false);
  // stage 0 (the barrier arrival of the persistent kernel) holds the entry time
  if (a.trace && threadIdx.x == 0 && slot < a.trace_phases)
    a.trace[((size_t)slot * gridDim.x + blockIdx.x) * 8] = t_entry;
  trace_mark(a, sy, 7);
}

template <int WF>
__global__ __launch_bounds__(SMALL_WG) void k_small_mega(const SmallArgs* __restrict__ ap,
                                                        unsigned epoch0) {
  Args& a = *(Args*)ap;
  const int np = small_phase_count(a.nl);
  for (int i = 0; i < np; ++i) {
    const SyncState sy{epoch0, i};
    run_phase<WF>(a, small_phase_id(a.nl, i), red_area(), sy, i > 0);
    trace_mark(a, sy, 7);
  }
}

// One instance of the phase kernels per body format (the projections'
// loads and matrix-core loops differ; nothing else does).
void launch_small_phase(hipStream_t st, const SmallArgs* dev_args, int G, int phase, int slot, int body_fmt) {
  if (body_fmt == WF_NVFP4) k_small_phase<WF_NVFP4><<<G, SMALL_WG, 0, st>>>(dev_args, phase, slot);
  else if (body_fmt == WF_BF16) k_small_phase<WF_BF16><<<G, SMALL_WG, 0, st>>>(dev_args, phase, slot);
  else k_small_phase<WF_FP8><<<G, SMALL_WG, 0, st>>>(dev_args, phase, slot);
}

static const void* mega_kernel(int body_fmt) {
  if (body_fmt == WF_NVFP4) return reinterpret_cast<const void*>(k_small_mega<WF_NVFP4>);
  if (body_fmt == WF_BF16) return reinterpret_cast<const void*>(k_small_mega<WF_BF16>);
  return reinterpret_cast<const void*>(k_small_mega<WF_FP8>);
}

hipError_t launch_small_mega(hipStream_t st, const SmallArgs* dev_args, int G, unsigned epoch0, int body_fmt) {
  const SmallArgs* p = dev_args;
  void* args[] = {&p, &epoch0};
  return hipLaunchCooperativeKernel(mega_kernel(body_fmt), dim3(G), dim3(SMALL_WG), args, 0, st);
}

int small_mega_occupancy() {
  // the smallest over the three instances
  int best = 1 << 30;
  for (int f : {WF_FP8, WF_NVFP4, WF_BF16}) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, mega_kernel(f), SMALL_WG, 0) != hipSuccess) return 0;
    best = occ < best ? occ : best;
  }
  return best;
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
  const size_t F2 = sizeof(uint16_t);
  carve(base, off, (size_t)SB_MAX * H * F, (void**)&o->f);
  carve(base, off, (size_t)SB_MAX * H * F2, (void**)&o->fh);
  carve(base, off, (size_t)SB_MAX * H * F, (void**)&o->fce);
  carve(base, off, (size_t)3 * SB_MAX * RK * F, (void**)&o->pb);
  carve(base, off, (size_t)3 * SB_MAX * RK * F2, (void**)&o->sp);
  carve(base, off, (size_t)SR_MAX * (DH / 2) * 2 * F, (void**)&o->rope);
  for (int i = 0; i < NXS; ++i) {
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->x[i]);
    carve(base, off, (size_t)SR_MAX * H * F2, (void**)&o->xg[i]);
    carve(base, off, (size_t)SR_MAX * HT * F, (void**)&o->ssq[i]);
  }
  for (int l = 0; l < NL; ++l) {
    carve(base, off, (size_t)3 * SB_MAX * RK * F2, (void**)&o->ss[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->q[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->k[l]);
    carve(base, off, (size_t)SR_MAX * H * F, (void**)&o->v[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * F, (void**)&o->am[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * F, (void**)&o->al[l]);
    carve(base, off, (size_t)SB_MAX * NH * nch * 4 * DH * F, (void**)&o->ao[l]);
    carve(base, off, (size_t)SR_MAX * H * F2, (void**)&o->o[l]);
    carve(base, off, (size_t)SR_MAX * FF * F2, (void**)&o->h[l]);
  }
  carve(base, off, (size_t)MAX_G * SR_MAX * sizeof(unsigned long long), (void**)&o->cand);
  carve(base, off, (size_t)20 * 32 * sizeof(unsigned), (void**)&o->bar);
  carve(base, off, (size_t)NL * SB_MAX * NH * 32 * sizeof(unsigned), (void**)&o->att_cnt);
  for (int l = 0; l < NL; ++l) carve(base, off, (size_t)DOWN_KS * SR_MAX * H * F, (void**)&o->dpart[l]);
  carve(base, off, (size_t)NL * (HT / 2) * 32 * sizeof(unsigned), (void**)&o->down_cnt);
  return (off + 255) & ~(size_t)255;
}

size_t small_bytes(int nch) { return small_layout(nullptr, nch, nullptr); }
void small_carve(char* base, int nch, SmallBufs* s) { small_layout(base, nch, s); }

}  // namespace kd
