// Device-side building blocks of libkdraft for gfx950 (CDNA4).
//
// Data layouts shared by the kernels:
//
//  * Activation fragments ("afrag"): an activation matrix X[R][K] (fp32 in
//    value) is stored in f16 (round to nearest even), arranged as the A
//    operand of v_mfma_f32_16x16x32_f16. For row tile mt (16 rows) and k tile
//    t (32 inputs) the fragment holds 64 lanes x 8 f16; lane l, element e is
//    X[16*mt + l%16][32*t + 8*(l/16) + e]. Element offset of (mt, t):
//    (mt*KT + t) * 512 with KT = K/32. f16 keeps 11 significant bits; the
//    weights it multiplies are decoded exactly into f16 and the products are
//    summed in fp32.
//
//  * Block-FP8 weights W[N][K] are repacked once at load to the B operand of
//    the same instruction: [N/16][K/64][64 lanes][16 bytes]. Lane l's 16 bytes
//    are W[16*nt + l%16][64*b + 8*(l/16) + e] for e = 0..7 (k tile 2b), then
//    the same for k tile 2b+1 (+32). Scales: [N/16][K/64][16] fp32.
//
//  * NVFP4 body weights W[N][K] (e2m1 codes, an e4m3 scale per 16 inputs of
//    a row, an fp32 tensor scale): codes [N/16][K/64][64 lanes][8 bytes],
//    lane l's bytes 0..3 holding W[16*nt + l%16][64*b + 8*(l/16) + e],
//    e = 0..7, even e in the low nibble (k tile 2b), bytes 4..7 the same at
//    +32 (k tile 2b+1); block-scale codes [N/16][K/64][16 rows][4 bytes],
//    byte i the scale of inputs 64*b + 16*i .. + 15; the tensor scale per
//    output row, twice ([2][N]: for blocks before the matrix's split block
//    and from it on, where two matrices are joined along K).
//
//  * bf16 body weights W[N][K]: [N/16][K/64][2 k tiles][64 lanes][8 bf16],
//    lane l holding W[16*nt + l%16][64*b + 32*j + 8*(l/16) + e].
//
//  * NVFP4 head rows are repacked to [V/16][K/128][64 lanes][16 bytes] of
//    e2m1 nibbles (lane l, k tile t = 4*g + i: bytes 4i..4i+3 hold
//    W[16*vt + l%16][32*t + 8*(l/16) + e], e = 0..7, even e in the low
//    nibble) and [V/16][K/128][64][4] e4m3 scale codes (byte i is the scale of
//    the 16-input block holding those 8 values).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

constexpr int H = 2560;      // hidden
constexpr int NH = 20;       // heads
constexpr int DH = 128;      // head dim
constexpr int FF = 6144;     // SwiGLU width
constexpr int NL = 4;        // layers
constexpr int BLK = 4;       // block rows per stream
constexpr int RK = 256;      // adapter rank
constexpr int NTAP = 3;      // tapped target layers
constexpr int QKV = 3 * H;   // fused q|k|v output width
constexpr int GU = 2 * FF;   // fused gate|up output width
constexpr int ATT_CH = 128;  // context keys per attention workgroup

// Body-matrix formats (layouts above).
enum { WF_FP8 = 0, WF_NVFP4 = 1, WF_BF16 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return u2f(b << 16); }

// Two fp32 values whose low 16 bits are zero -> packed bf16x2 (element 0 low).
__device__ __forceinline__ uint32_t pack_hi16(float e0, float e1) {
  return __builtin_amdgcn_perm(f2u(e1), f2u(e0), 0x07060302u);
}

// Embedding-table row of a token id, or the zero row when the id lies
// outside [0, V): ids are caller data (or a previous round's drafts, which
// may be the -1 / -2 sentinels) and are never used unchecked as an index.
template <class T>
__device__ __forceinline__ T* table_row(T* table, T* zrow, int id, int V, int H_) {
  return (id >= 0 && id < V) ? table + (size_t)id * H_ : zrow;
}
// Block row j of stream b reads the anchor (through row 0) and the
// predecessor ids of rows 1..j; its draft is valid only if all lie in [0, V).
template <class P>
__device__ __forceinline__ bool id_row_valid(P anchor, P pred, int pred_stride, int b, int j, int V) {
  bool ok = anchor[b] >= 0 && anchor[b] < V;
  for (int i = 0; i < j; ++i) {
    const int p = pred[b * pred_stride + i];
    ok = ok && p >= 0 && p < V;
  }
  return ok;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 e4m3 codes (little-endian in two dwords) -> 8 exact bf16 values
// (gfx950's scaled conversion with a unit scale).
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// 8 e4m3 codes -> 8 exact f16 values: every e4m3 value (at most 4
// significant bits, magnitudes 2^-9 .. 448) is an f16 normal or zero.
__device__ __forceinline__ f16x8 e4m3x8_f16(uint32_t lo, uint32_t hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// 8 e2m1 codes (even element in the low nibble) times their e4m3 block scale,
// exactly in f16: e2m1 decoded with a unit scale, then one packed f16
// multiply per pair (the product has at most 6 significant bits and lies
// within f16's normal range).
__device__ __forceinline__ f16x8 nvfp4x8_f16(uint32_t nib, uint32_t scode) {
  const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scode, 1.0f, false);
  const f16x2 sc = {s2.x, s2.x};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 0) * sc;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 1) * sc;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 2) * sc;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 3) * sc;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// 8 bf16 (packed in 4 dwords) -> 8 fp32.
__device__ __forceinline__ void bf16x8_to_f32(u32x4 w, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = u2f(w[i] << 16);
    o[2 * i + 1] = u2f(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// An f16 operand as two exact bf16 terms for the bf16 matrix cores: hi keeps
// the top 8 significant bits of each value, lo the rest (at most 3 bits), so
// W * hi + W * lo is W * a exactly in fp32.
__device__ __forceinline__ void split_f16_bf16(f16x8 a, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v0 = (float)a[2 * e], v1 = (float)a[2 * e + 1];
    const float h0 = u2f(f2u(v0) & 0xffff0000u), h1 = u2f(f2u(v1) & 0xffff0000u);
    h[e] = pack_hi16(h0, h1);
    l[e] = pack_hi16(v0 - h0, v1 - h1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// One 64-input block of a 16x16 output tile: the f16 activation fragments
// a0, a1 (k tiles 2b, 2b+1) times the block's weights, as an fp32 partial sum
// before any block or tensor scale.
template <int WF>
struct WBlock;
template <>
struct WBlock<WF_FP8> {   // 16 e4m3 codes
  u32x4 q;
  __device__ __forceinline__ f32x4 mul(f16x8 a0, f16x8 a1) const {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    t = mfma_f16(a0, e4m3x8_f16(q.x, q.y), t);
    return mfma_f16(a1, e4m3x8_f16(q.z, q.w), t);
  }
};
template <>
struct WBlock<WF_NVFP4> {   // 16 e2m1 codes and the lane's two e4m3 block scales
  uint32_t q0, q1, sc;
  __device__ __forceinline__ f32x4 mul(f16x8 a0, f16x8 a1) const {
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    t = mfma_f16(a0, nvfp4x8_f16(q0, sc & 0xffu), t);
    return mfma_f16(a1, nvfp4x8_f16(q1, sc >> 8), t);
  }
};
template <>
struct WBlock<WF_BF16> {   // 16 bf16 values
  u32x4 w0, w1;
  __device__ __forceinline__ f32x4 mul(f16x8 a0, f16x8 a1) const {
    bf16x8 h0, l0, h1, l1;
    split_f16_bf16(a0, h0, l0);
    split_f16_bf16(a1, h1, l1);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    t = mfma_bf16(h0, __builtin_bit_cast(bf16x8, w0), t);
    t = mfma_bf16(l0, __builtin_bit_cast(bf16x8, w0), t);
    t = mfma_bf16(h1, __builtin_bit_cast(bf16x8, w1), t);
    return mfma_bf16(l1, __builtin_bit_cast(bf16x8, w1), t);
  }
};

// Lane `lane`'s part of block (nt, b) of a repacked matrix. NVFP4: the lane's
// inputs 8 (lane/16) .. + 8 of k tile 2b lie in 16-input scale block
// (lane/16)/2, those of k tile 2b+1 in block 2 + (lane/16)/2.
template <int WF>
__device__ __forceinline__ WBlock<WF> load_wblock(const uint8_t* w, const uint8_t* s4, int KB, int nt, int b,
                                                  int lane) {
  const size_t blk = (size_t)nt * KB + b;
  WBlock<WF> r;
  if constexpr (WF == WF_FP8) {
    r.q = *reinterpret_cast<const u32x4*>(w + blk * 1024 + lane * 16);
  } else if constexpr (WF == WF_NVFP4) {
    const uint2 q = *reinterpret_cast<const uint2*>(w + blk * 512 + lane * 8);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(s4 + blk * 64 + (lane & 15) * 4);
    const int sh = 8 * ((lane >> 4) >> 1);
    r.q0 = q.x;
    r.q1 = q.y;
    r.sc = ((sw >> sh) & 0xffu) | (((sw >> (sh + 16)) & 0xffu) << 8);
  } else {
    r.w0 = *reinterpret_cast<const u32x4*>(w + blk * 2048 + lane * 16);
    r.w1 = *reinterpret_cast<const u32x4*>(w + blk * 2048 + 1024 + lane * 16);
  }
  return r;
}

// Element offset of afrag(row, k).
__device__ __forceinline__ size_t afrag_off(int row, int k, int KT) {
  int mt = row >> 4, t = k >> 5;
  int lane = (row & 15) + 16 * ((k & 31) >> 3);
  return (size_t)(mt * KT + t) * 512 + lane * 8 + (k & 7);
}

// f16 range of activation stores. A value beyond the largest finite f16
// (65504) or not finite is stored saturated (NaN as +65504) and sets this
// translation unit's flag; the round's last kernel moves the flag into the
// context's host-visible range word, which the next call reports.
static __device__ unsigned g_f16_range = 0u;
__device__ __forceinline__ _Float16 f16_checked(float v) {
  if (!(fabsf(v) <= 65504.0f)) {
    __hip_atomic_fetch_or(&g_f16_range, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = v < 0.0f ? -65504.0f : 65504.0f;
  }
  return (_Float16)v;
}
// Moves this translation unit's f16 range flag into *range_word (one thread;
// a plain store, no read-modify-write on host memory).
__device__ __forceinline__ void flush_f16_range(unsigned* range_word) {
  if (__hip_atomic_load(&g_f16_range, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(&g_f16_range, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (range_word) __hip_atomic_store(range_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Stores 8 consecutive fp32 values X[row][k0..k0+8) (k0 % 8 == 0) as f16.
__device__ __forceinline__ void store_afrag8(uint16_t* af, int KT, int row, int k0, const float* v) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = f16_checked(v[i]);
  *reinterpret_cast<f16x8*>(af + afrag_off(row, k0, KT)) = h;
}

// Stores 8 consecutive bf16 values (given as bits) as f16.
__device__ __forceinline__ void store_afrag8_bf16(uint16_t* af, int KT, int row, int k0, u32x4 bits) {
  float v[8];
  bf16x8_to_f32(bits, v);
  store_afrag8(af, KT, row, k0, v);
}

__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

// Order-preserving map of an fp32 to uint32 (NaN handled by the caller).
__device__ __forceinline__ uint32_t f32_order(float x) {
  uint32_t u = f2u(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Argmax key: larger logit wins, then the lower index. 0 = no finite logit.
__device__ __forceinline__ unsigned long long argmax_key(float x, uint32_t idx) {
  if (!(x == x) || x == __builtin_inff() || x == -__builtin_inff()) return 0ull;
  return ((unsigned long long)f32_order(x) << 32) | (0xffffffffu - idx);
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over a workgroup of `nwaves` waves; every thread gets the result.
template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) t += red[i];
  return t;
}

// ---------------------------------------------------------------------------
// Rotated 4-bit K/V (the 4-bit KV article, "What we do": keys turned by a
// signed Walsh-Hadamard rotation, every row coded to 4 bits with an fp16
// scale and offset per row and head).
// ---------------------------------------------------------------------------
// In-wave Walsh-Hadamard transform of 128 values: lane l holds x[l] (y0) and
// x[l + 64] (y1) and ends with (H x)[l], (H x)[l + 64], H[i][k] =
// (-1)^popcount(i & k). One butterfly per index bit: (a, c) -> (a + c, a - c)
// for the pair differing in that bit; bit 6 pairs the two registers, bits
// 5..0 pair lanes.
__device__ __forceinline__ void fwht128(float& y0, float& y1, int lane) {
  const float a = y0, c = y1;
  y0 = a + c;
  y1 = a - c;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float p0 = __shfl_xor(y0, m, 64), p1 = __shfl_xor(y1, m, 64);
    const bool up = (lane & m) != 0;
    y0 = up ? p0 - y0 : y0 + p0;
    y1 = up ? p1 - y1 : y1 + p1;
  }
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Codes one 128-value row held as (x0 at dim lane, x1 at dim lane + 64):
// scale = fp16((max - min)/15), offset = fp16(min), codes clamp(rne((x -
// offset)/scale), 0, 15) (0 for a zero scale), dims 2m and 2m + 1 in the low
// and high nibble of byte m; writes the 64 code bytes and the (scale,
// offset) pair.
__device__ __forceinline__ void store_row_q4(float x0, float x1, int lane, uint8_t* codes,
                                             uint32_t* so) {
  const float mn = wave_min(fminf(x0, x1)), mx = wave_max(fmaxf(x0, x1));
  const _Float16 sc_h = f16_checked((mx - mn) / 15.0f), of_h = f16_checked(mn);
  const float sc = (float)sc_h, of = (float)of_h;
  auto code = [&](float x) -> uint32_t {
    if (!(sc > 0.f)) return 0u;
    const float c = __builtin_rintf((x - of) / sc);
    return (uint32_t)fminf(fmaxf(c, 0.f), 15.f);
  };
  const uint32_t c0 = code(x0), c1 = code(x1);
  // dims (2m, 2m + 1) meet in the even lane
  const uint32_t n0 = __shfl_xor(c0, 1, 64), n1 = __shfl_xor(c1, 1, 64);
  if ((lane & 1) == 0) {
    codes[lane >> 1] = (uint8_t)(c0 | (n0 << 4));
    codes[32 + (lane >> 1)] = (uint8_t)(c1 | (n1 << 4));
  }
  if (lane == 0)
    *so = (uint32_t)__builtin_bit_cast(uint16_t, sc_h) | ((uint32_t)__builtin_bit_cast(uint16_t, of_h) << 16);
}

// 8 4-bit codes (one dword, dim 2i in the low nibble of byte i) -> 8 f16
// values code * 2^-24: each code becomes the mantissa of an f16 subnormal
// (exact; the matrix cores take f16 subnormals as they are). Users scale
// the products by 2^24.
__device__ __forceinline__ f16x8 nib8_f16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x0C040C00u));
  const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x0C050C01u));
  const f16x2 p2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x0C060C02u));
  const f16x2 p3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x0C070C03u));
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
constexpr float KD_2P24 = 16777216.0f;

// (scale, offset) fp16 pair in one dword -> two floats.
__device__ __forceinline__ void so_unpack(uint32_t w, float& sc, float& of) {
  sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  of = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_16x16x16_f16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Byte m of x0 and of x1 (each a code 0..15) -> f16x2 of the two codes
// times 2^-24 (f16 subnormals, as in nib8_f16).
template <int M>
__device__ __forceinline__ f16x2 byte_pair_f16(uint32_t x0, uint32_t x1) {
  constexpr uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + M) << 16) | (uint32_t)M;
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(x1, x0, sel));
}

// ---------------------------------------------------------------------------
// Output-row order of the repacked q|k|v and gate|up matrices.
//
// q|k|v: a 16-row tile holds 8 dims of one head and their rotate-half
// partners (d and d + 64), so a tile's epilogue can apply RoPE. Tile t of
// section s (0 q, 1 k, 2 v): head t/8 within the section, dims 8*(t%8) + i
// (rows 0..7) and 64 + 8*(t%8) + i (rows 8..15).
// gate|up: tile t holds gate rows 8t..8t+7 then up rows 8t..8t+7, so a tile's
// epilogue can form silu(gate) * up.
// ---------------------------------------------------------------------------
__host__ __device__ inline int qkv_natural(int pos) {
  const int t = pos >> 4, n = pos & 15;
  const int s = t / (H / 16), tt = t % (H / 16);
  const int hh = tt >> 3, pg = tt & 7;
  const int d = n < 8 ? 8 * pg + n : 64 + 8 * pg + (n - 8);
  return s * H + hh * DH + d;
}
__host__ __device__ inline int qkv_position(int nat) {
  const int s = nat / H, c = nat % H;
  const int hh = c / DH, d = c % DH;
  const int pg = (d & 63) >> 3, n = (d & 7) + (d >= 64 ? 8 : 0);
  return 16 * (s * (H / 16) + hh * 8 + pg) + n;
}
__host__ __device__ inline int gu_natural(int pos) {  // gate rows 0..FF-1, up rows FF..2FF-1
  const int t = pos >> 4, n = pos & 15;
  return n < 8 ? 8 * t + n : FF + 8 * t + (n - 8);
}
__host__ __device__ inline int gu_position(int nat) {
  const int up = nat >= FF, g = up ? nat - FF : nat;
  return 16 * (g >> 3) + (g & 7) + (up ? 8 : 0);
}

}  // namespace kd
