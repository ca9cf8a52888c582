// Copy (suffix-match) drafts: the model card "Kolibri-1 block drafter",
// section Use, tries copy drafts from the context before the learned block;
// the frozen-corpus drafting article fixes the rule: the continuation after
// the longest suffix of the current context, suffix length 8 down to 3, most
// recent occurrence, a span of up to K tokens that never crosses a -1
// separator of the corpus.
//
// For every stream, m(p) is the length (at most 8) of the match between the
// stream's last tokens and the tokens just before candidate position p, and a
// candidate needs a token at p (in the context p < len; in the corpus
// corpus[p] is no separator). A source's winner is the largest (m, p) pair,
// kept as the 64-bit key m << 32 | p and merged with atomicMax, which does
// not depend on the order workgroups finish in. The proposal comes from the
// context when its best m is at least the corpus's (the context is tried
// first at equal length), from the corpus otherwise, and exists when that m is
// at least 3.
#include "kd_device.h"
#include "kd_runtime.h"

namespace kd {

constexpr int CP_SMAX = 8, CP_SMIN = 3;
constexpr int CP_WG = 256, CP_PER_THREAD = 4;

__global__ void k_copy_clear(unsigned long long* keys, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) keys[i] = 0ull;
}

// The last min(8, len) tokens of a history, latest first; absent ones are -2
// (tokens are >= 0 and corpus separators -1, so -2 matches nothing).
__device__ __forceinline__ void load_suffix(const int32_t* hist, int len, int (&suf)[CP_SMAX]) {
#pragma unroll
  for (int i = 0; i < CP_SMAX; ++i) suf[i] = i < len ? hist[len - 1 - i] : -2;
}

// Match length at p: the number of consecutive i = 0, 1, ... with
// before[i] == suf[i], where before[i] is the token at p - 1 - i.
__device__ __forceinline__ int match_len(const int (&before)[CP_SMAX], const int (&suf)[CP_SMAX]) {
  int m = 0;
  bool on = true;
#pragma unroll
  for (int i = 0; i < CP_SMAX; ++i) {
    on = on && before[i] == suf[i];
    m += on ? 1 : 0;
  }
  return m;
}

// A history's length, clamped into [0, stride] (the caller's lengths are
// trusted otherwise; the clamp keeps every read inside the histories).
__device__ __forceinline__ int hist_len(const int32_t* lens, int b, long long stride) {
  const long long l = lens[b];
  return (int)(l < 0 ? 0 : (l > stride ? stride : l));
}

__device__ __forceinline__ unsigned long long u64_max2(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    v = u64_max2(v, ((unsigned long long)hi << 32) | lo);
  }
  return v;
}

// Context source: workgroup (x, b) scans positions of stream b's history.
__global__ __launch_bounds__(CP_WG) void k_copy_context(const int32_t* tokens, long long stride,
                                                        const int32_t* lens,
                                                        unsigned long long* keys) {
  const int b = blockIdx.y;
  const int len = hist_len(lens, b, stride);
  const int32_t* hist = tokens + (size_t)b * stride;
  const long long p0 = (long long)blockIdx.x * CP_WG * CP_PER_THREAD;
  if (len < CP_SMIN || p0 >= len) return;
  int suf[CP_SMAX];
  load_suffix(hist, len, suf);
  unsigned long long best = 0ull;
#pragma unroll
  for (int k = 0; k < CP_PER_THREAD; ++k) {
    const long long p = p0 + k * CP_WG + threadIdx.x;
    if (p >= 1 && p <= len - 1) {          // a continuation token exists
      int before[CP_SMAX];
#pragma unroll
      for (int i = 0; i < CP_SMAX; ++i) before[i] = p - 1 - i >= 0 ? hist[p - 1 - i] : -3;
      const int m = match_len(before, suf);
      if (m >= CP_SMIN) best = u64_max2(best, ((unsigned long long)m << 32) | (unsigned long long)p);
    }
  }
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0 && best) atomicMax(&keys[2 * b], best);
}

// Corpus source: workgroup x scans a span of the corpus against every
// stream's suffix (the corpus is read once for all streams).
__global__ __launch_bounds__(CP_WG) void k_copy_corpus(const int32_t* tokens, long long stride,
                                                       const int32_t* lens, int B,
                                                       const int32_t* corpus, long long n,
                                                       unsigned long long* keys) {
  extern __shared__ int cp_smem[];
  int* s_suf = cp_smem;                                                      // [B][8]
  unsigned long long* s_best = reinterpret_cast<unsigned long long*>(cp_smem + 8 * B);  // [B]
  for (int i = threadIdx.x; i < B * CP_SMAX; i += CP_WG) {
    const int b = i / CP_SMAX, k = i % CP_SMAX;
    const int len = hist_len(lens, b, stride);
    s_suf[i] = k < len ? tokens[(size_t)b * stride + len - 1 - k] : -2;
  }
  for (int b = threadIdx.x; b < B; b += CP_WG) s_best[b] = 0ull;
  __syncthreads();
  const long long p0 = (long long)blockIdx.x * CP_WG * CP_PER_THREAD;
#pragma unroll 1
  for (int k = 0; k < CP_PER_THREAD; ++k) {
    const long long p = p0 + k * CP_WG + threadIdx.x;
    // a continuation token exists and is no separator
    if (p < 1 || p >= n || corpus[p] == -1) continue;
    int before[CP_SMAX];
#pragma unroll
    for (int i = 0; i < CP_SMAX; ++i) before[i] = p - 1 - i >= 0 ? corpus[p - 1 - i] : -3;
    for (int b = 0; b < B; ++b) {
      if (before[0] != s_suf[b * CP_SMAX]) continue;   // most positions stop here
      int suf[CP_SMAX];
#pragma unroll
      for (int i = 0; i < CP_SMAX; ++i) suf[i] = s_suf[b * CP_SMAX + i];
      const int m = match_len(before, suf);
      if (m >= CP_SMIN)
        __hip_atomic_fetch_max(&s_best[b], ((unsigned long long)m << 32) | (unsigned long long)p,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += CP_WG)
    if (s_best[b]) atomicMax(&keys[2 * b + 1], s_best[b]);
}

// One thread per stream: the winning source, its span, the report.
__global__ void k_copy_finalize(const int32_t* tokens, long long stride, const int32_t* lens,
                                const int32_t* corpus, long long n, int B, int K,
                                const unsigned long long* keys, int32_t* out_ids,
                                int32_t* out_info) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const unsigned long long kc = keys[2 * b], ko = keys[2 * b + 1];
  const int mc = (int)(kc >> 32), mo = (int)(ko >> 32);
  int cnt = 0, s = 0, src = 0;
  int32_t* out = out_ids + (size_t)b * K;
  if (mc >= CP_SMIN && mc >= mo) {
    const long long p = (long long)(kc & 0xffffffffull);
    const int len = hist_len(lens, b, stride);
    const int32_t* hist = tokens + (size_t)b * stride;
    for (long long q = p; q < len && cnt < K; ++q) out[cnt++] = hist[q];
    s = mc;
    src = 1;
  } else if (mo >= CP_SMIN) {
    const long long p = (long long)(ko & 0xffffffffull);
    for (long long q = p; q < n && cnt < K && corpus[q] != -1; ++q) out[cnt++] = corpus[q];
    s = mo;
    src = 2;
  }
  for (int i = cnt; i < K; ++i) out[i] = -1;
  out_info[3 * b + 0] = cnt;
  out_info[3 * b + 1] = s;
  out_info[3 * b + 2] = src;
}

void launch_copy_draft(hipStream_t st, int B, const int32_t* tokens, long long stride,
                       const int32_t* lens, const int32_t* corpus, long long n, int K,
                       unsigned long long* keys, int32_t* out_ids, int32_t* out_info) {
  k_copy_clear<<<(2 * B + 255) / 256, 256, 0, st>>>(keys, 2 * B);
  const long long span = (long long)CP_WG * CP_PER_THREAD;
  if (stride > 0)
    k_copy_context<<<dim3((unsigned)((stride + span - 1) / span), B), CP_WG, 0, st>>>(tokens, stride,
                                                                                    lens, keys);
  if (corpus && n > 1) {
    const size_t smem = (size_t)8 * B * sizeof(int) + (size_t)B * sizeof(unsigned long long);
    k_copy_corpus<<<(unsigned)((n + span - 1) / span), CP_WG, smem, st>>>(tokens, stride, lens, B,
                                                                          corpus, n, keys);
  }
  k_copy_finalize<<<(B + 63) / 64, 64, 0, st>>>(tokens, stride, lens, corpus, n, B, K, keys,
                                                out_ids, out_info);
}

}  // namespace kd
