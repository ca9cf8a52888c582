// The small-batch round (up to 4 streams = 16 block rows): workgroup-level
// phases that run either one launch per phase or all inside one persistent
// cooperative kernel separated by grid barriers.
#pragma once

#include "kd_runtime.h"

namespace kd {

constexpr int SB_MAX = 4;      // streams
constexpr int SR_MAX = 16;     // block rows (one matrix-core row tile)
constexpr int NXS = 12;        // residual-stream stages written in one round
constexpr int HT = H / 16;     // 160 column tiles of a hidden vector
constexpr int SMALL_WG = 512;  // 8 waves per workgroup
constexpr int HEAD_NT = 2;     // vocab tiles per head unit
constexpr int MAX_G = 256;     // workgroups (one per CU); barrier tree is 16 x 16
constexpr int DOWN_KS = 3;     // the down projection's inputs split in thirds across workgroups

// Attention partial slots per (stream, head) for a window: one per 128-key
// chunk, padded to whole 128-byte lines of the per-chunk max and sum (8
// chunks), so different pairs never share a line.
__host__ __device__ inline int small_nch(int window) { return ((window + ATT_CH - 1) / ATT_CH + 7) / 8 * 8; }

// Stage index of the residual stream: the layer input, after O, after down.
__host__ __device__ inline int xs_in(int l) { return l == 0 ? 0 : 3 * l; }
__host__ __device__ inline int xs_o(int l) { return 3 * l + 1; }
__host__ __device__ inline int xs_d(int l) { return 3 * l + 2; }

// Buffers written at most once per round (so no cache ever holds a stale
// copy within a launch); every buffer starts on a 256-byte boundary and no two
// phases write into the same 128-byte line. Activations that only enter the
// matrix cores are stored as f16 bits (fh, sp, xg, ss, o, h); the residual
// stream, its sums of squares and the attention inputs stay fp32.
template <template <class> class P>
struct SmallBufsT {
  P<float> f;                  // [SB][H]   fused tap state
  P<uint16_t> fh;              // [SB][H]   the same, f16 (matrix input)
  P<float> fce;                // [SB][H]   fc (embedding half) . E[anchor]
  P<float> pb;                 // [3SB][RK] B_p . E[pred]
  P<uint16_t> sp;              // [3SB][RK] silu(A_p f + B_p E[pred]), f16
  P<float> rope;               // [SR][64][2] cos, sin at the block positions
  P<float> x[NXS];             // [SR][H]   residual stream stages
  P<uint16_t> xg[NXS];         // [SR][H]   the stage times the RMSNorm gain of its consumer, f16
  P<float> ssq[NXS];           // [SR][HT]  sum of squares of each 16-column tile
  P<uint16_t> ss[NL];          // [3SB][RK] spine hidden (layers 1..3), f16
  P<float> q[NL];              // [SR][H]   post-RoPE, natural head-major layout
  P<float> k[NL];
  P<float> v[NL];
  P<float> am[NL];             // [SB][NH][nch][4] chunk max (log2 units)
  P<float> al[NL];             // [SB][NH][nch][4] chunk sum of 2^(s - max)
  P<float> ao[NL];             // [SB][NH][nch][4][DH]
  P<uint16_t> o[NL];           // [SR][H]   merged attention output, f16
  P<uint16_t> h[NL];           // [SR][FF]  silu(gate) * up, f16
  P<unsigned long long> cand;  // [MAX_G][SR] per-workgroup argmax candidates
  P<unsigned> bar;             // control words, 32 u32 apart: [0..15] arrival counters of
                               // the 16-workgroup groups, [18] error, [19] head counter
  P<unsigned> att_cnt;         // [NL][SB][NH] chunk counters, one 128-byte line each
  P<float> dpart[NL];          // [DOWN_KS][SR][H] down projection partials over thirds of FF
  P<unsigned> down_cnt;        // [NL][HT / 2] counters of the partials, one 128-byte line each
};

template <template <class> class P>
struct SmallArgsT {
  int B, R, nl, window, nch;
  float eps, theta;
  P<const uint16_t> taps;
  P<const int32_t> anchor;
  P<const int32_t> pred;
  int pred_stride;              // ids per stream in pred: 3 (caller's), 4 (previous round's out_ids)
  P<const int32_t> lens;
  KVT<P> kv;
  P<int32_t> out_ids;
  P<float> out_logits;
  DevWeightsT<P> d;
  SmallBufsT<P> s;
  // Host-visible status words (mapped pinned memory): [0] set to 1 when a
  // bounded wait of the round timed out, [1] when an f16 activation store
  // saturated.
  P<unsigned> status;
  // Optional stage timestamps (100 MHz wall clock), [phase slot][G][8]; null = off.
  P<unsigned long long> trace;
  int trace_phases;
};

using SmallBufs = SmallBufsT<HostPtr>;
using SmallArgs = SmallArgsT<HostPtr>;

// Bytes of the small-path buffers for a window (nch = ceil(window / 128)).
size_t small_bytes(int nch);
void small_carve(char* base, int nch, SmallBufs* s);
__host__ __device__ int small_phase_count(int nl);
__host__ __device__ int small_phase_id(int nl, int i);
// dev_args: a device copy of the SmallArgs.
void launch_small_phase(hipStream_t st, const SmallArgs* dev_args, int G, int phase, int slot, int body_fmt);
// epoch0: grid barriers completed by earlier persistent launches on these
// buffers (each launch completes small_phase_count(nl) - 1).
hipError_t launch_small_mega(hipStream_t st, const SmallArgs* dev_args, int G, unsigned epoch0, int body_fmt);
int small_mega_occupancy();


}  // namespace kd
