// C ABI of libkdraft: context, load-time weight repacking, workspace and the
// launch sequences of a round and of a context ingest.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/kdraft.h"
#include "../../include/kdraft_debug.h"
#include "kd_device.h"
#include "kd_runtime.h"
#include "kd_small.h"

// Uploads argument blocks to device memory without waiting on the stream:
// each upload copies from the next of NSTAGE pinned staging buffers, which is
// reused only after the copy recorded on it has completed (normally long
// before: NSTAGE uploads later).
struct ArgStager {
  static constexpr int NSTAGE = 8;
  void* buf[NSTAGE] = {};
  hipEvent_t ev[NSTAGE] = {};
  bool pending[NSTAGE] = {};
  int next = 0;
  size_t bytes = 0;

  bool init(size_t n) {
    bytes = n;
    for (int i = 0; i < NSTAGE; ++i) {
      if (hipHostMalloc(&buf[i], n, hipHostMallocDefault) != hipSuccess) return false;
      if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) return false;
    }
    return true;
  }
  hipError_t upload(void* dev, const void* src, size_t n, hipStream_t st) {
    if (n > bytes) return hipErrorInvalidValue;
    const int i = next;
    next = (next + 1) % NSTAGE;
    if (pending[i]) {
      const hipError_t e = hipEventSynchronize(ev[i]);
      if (e != hipSuccess) return e;
    }
    memcpy(buf[i], src, n);
    hipError_t e = hipMemcpyAsync(dev, buf[i], n, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipEventRecord(ev[i], st);
    pending[i] = e == hipSuccess;
    return e;
  }
  void destroy() {
    for (int i = 0; i < NSTAGE; ++i) {
      if (ev[i]) (void)hipEventDestroy(ev[i]);
      if (buf[i]) (void)hipHostFree(buf[i]);
      ev[i] = nullptr;
      buf[i] = nullptr;
    }
  }
};

struct kd_ctx {
  kd_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  kd::Work w;
  kd::DevWeights d;
  std::vector<void*> work_allocs;
  std::vector<void*> weight_allocs;
  bool loaded = false;
  int debug_layers = -1;
  int fused_proj = 1;        // general path above 32 rows: q|k|v and gate|up epilogues fused
  int last_streams = 0;
  int last_path = 0;
  std::string err;
  // small-batch path (<= 4 streams)
  char* small_mem = nullptr;
  kd::SmallBufs small{};
  int G = 0;                 // workgroups of the small path (one per CU, <= 256)
  bool small_ok = false;     // the window fits the small path's attention phase
  unsigned epoch = 0;        // grid barriers completed by persistent launches so far
  bool mega_ok = false;      // persistent cooperative kernel available
  int path = 0;              // 0 auto, 1 general, 2 small per-phase, 3 small persistent
  // Device copies of the small-path arguments, one per kind of round so that
  // a serving loop finds each block unchanged from call to call: slot 0 a
  // call's only round, 1 the first of several (no logits), 2 a middle round
  // and 3 the last round of kd_round_depth (predecessors from the previous
  // round's ids).
  static constexpr int NSLOT = 4;
  kd::SmallArgs* args_dev[NSLOT] = {};
  kd::SmallArgs args_cur[NSLOT];   // what each device slot holds once the queued uploads run
  bool args_valid[NSLOT] = {};
  ArgStager stager;
  // The per-phase launches of path 2 as one graph per slot: the kernels read
  // their arguments from args_dev[slot], so a graph depends only on the layer
  // count and the grid; it is captured on a private stream and launched on the
  // caller's.
  hipStream_t cap_stream = nullptr;
  hipGraphExec_t phase_graph[NSLOT] = {};
  int phase_graph_nl[NSLOT] = {-1, -1, -1, -1};
  // Host-mapped status word: a kernel sets it when one of its bounded waits
  // timed out; the next call reports KD_ERR_HIP and clears it.
  unsigned* status_host = nullptr;
  unsigned* status_dev = nullptr;
  unsigned long long* trace = nullptr;  // caller's device buffer for stage timestamps
  int trace_phases = 0;
  // The general path's launches of a round (and of an ingest) as graphs: their
  // kernel arguments hold the caller's pointers, so each graph is kept with the
  // arguments it was captured for. Up to GRAPH_CACHE graphs per kind are kept
  // (least recently used dropped first), so a serving loop that rotates among
  // a few buffer sets captures each set once.
  struct CachedGraph {
    hipGraphExec_t exec = nullptr;
    std::vector<unsigned char> key;
    unsigned long long used = 0;
  };
  static constexpr int GRAPH_CACHE = 8;
  CachedGraph round_graph[GRAPH_CACHE], ingest_graph[GRAPH_CACHE];
  unsigned long long graph_clock = 0;
};

namespace {

kd_status fail(kd_ctx* c, kd_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

kd_status hip_fail(kd_ctx* c, hipError_t e, const char* what) {
  return fail(c, KD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void drop_graph(kd_ctx::CachedGraph& g) {
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  g.exec = nullptr;
  g.key.clear();
}

// Appends the bytes of v (a scalar or pointer: no padding) to a graph key.
template <class T>
void key_add(std::vector<unsigned char>& key, const T& v) {
  static_assert(std::is_scalar<T>::value, "key fields are scalars");
  const unsigned char* p = reinterpret_cast<const unsigned char*>(&v);
  key.insert(key.end(), p, p + sizeof(T));
}
void key_add_kv(std::vector<unsigned char>& key, const kd::KV& k) {
  for (int l = 0; l < 4; ++l) {
    key_add(key, k.k[l]);
    key_add(key, k.v[l]);
  }
  key_add(key, k.ss);
  key_add(key, k.sh);
  key_add(key, k.sl);
  key_add(key, k.cap);
  key_add(key, k.fmt);
  for (int l = 0; l < 4; ++l) {
    key_add(key, k.kso[l]);
    key_add(key, k.vso[l]);
  }
}

void drop_graphs(kd_ctx::CachedGraph (&gs)[kd_ctx::GRAPH_CACHE]) {
  for (auto& g : gs) drop_graph(g);
}

// Launches `enqueue`'s kernels on st as a graph: replayed from the cache when
// a graph with this key is there, else captured on the private stream into the
// least recently used entry.
template <class F>
kd_status launch_cached(kd_ctx* c, kd_ctx::CachedGraph (&cache)[kd_ctx::GRAPH_CACHE],
                        std::vector<unsigned char>&& key, hipStream_t st, F&& enqueue, const char* what) {
  kd_ctx::CachedGraph* hit = nullptr;
  kd_ctx::CachedGraph* victim = &cache[0];
  for (auto& e : cache) {
    if (e.exec && e.key == key) hit = &e;
    if (!e.exec || (victim->exec && e.used < victim->used)) victim = &e;
  }
  kd_ctx::CachedGraph& g = hit ? *hit : *victim;
  g.used = ++c->graph_clock;
  if (!hit) {
    drop_graph(g);
    hipError_t e = hipSuccess;
    if (!c->cap_stream) e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking);
    hipGraph_t graph = nullptr;
    if (e == hipSuccess) e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      enqueue(c->cap_stream);
      e = hipStreamEndCapture(c->cap_stream, &graph);
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    if (e != hipSuccess) {
      g.exec = nullptr;
      return hip_fail(c, e, what);
    }
    g.key = std::move(key);
  }
  const hipError_t e = hipGraphLaunch(g.exec, st);
  if (e != hipSuccess) return hip_fail(c, e, what);
  return KD_OK;
}

template <typename T>
bool dev_alloc(std::vector<void*>& list, T** p, size_t elems) {
  void* q = nullptr;
  if (hipMalloc(&q, std::max<size_t>(elems * sizeof(T), 256)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  list.push_back(q);
  *p = static_cast<T*>(q);
  return true;
}

void free_all(std::vector<void*>& list) {
  for (void* p : list) (void)hipFree(p);
  list.clear();
}

bool shape_is_supported(const kd_config& c) {
  return c.hidden == kd::H && c.heads == kd::NH && c.head_dim == kd::DH && c.ffn == kd::FF &&
         c.layers == kd::NL && c.block == kd::BLK && c.rank == kd::RK && c.taps == kd::NTAP;
}

// The GEMM calls a round and an ingest make, as (K, N, rows per stream).
struct GemmUse {
  int K, N, rows_per_stream;
};
const GemmUse kRoundUses[] = {
    {kd::NTAP * kd::H, kd::H, 1}, {2 * kd::H, kd::H, 1},  {2 * kd::H, kd::RK, 3},
    {kd::RK, kd::H, 3},           {kd::H, kd::RK, 3},     {kd::H, kd::QKV, 4},
    {kd::H, kd::H, 4},            {kd::H, kd::GU, 4},     {kd::FF, kd::H, 4}};
const GemmUse kIngestUses[] = {
    {kd::NTAP * kd::H, kd::H, 1}, {2 * kd::H, kd::H, 1}, {kd::H, 2 * kd::H, 1}};

size_t part_region_elems(int Bmax) {
  size_t best = 0;
  for (int B = 1; B <= Bmax; ++B) {
    for (const GemmUse& u : kRoundUses) {
      const int R = B * u.rows_per_stream;
      best = std::max(best, (size_t)kd::gemm_splits(u.K, u.N, R) * R * u.N);
    }
    for (int n = 1; n <= KD_MAX_INGEST; ++n)
      for (const GemmUse& u : kIngestUses) {
        const int R = B * n;
        best = std::max(best, (size_t)kd::gemm_splits(u.K, u.N, R) * R * u.N);
      }
  }
  return best;
}

// Block-FP8 repack (layout documented in kd_device.h). q: [N][K], s: [N][K/64].
void repack_fp8(const uint8_t* q, const float* s, int N, int K, uint8_t* wo, float* so) {
  const int KB = K / 64;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int b = 0; b < KB; ++b) {
      uint8_t* dst = wo + ((size_t)nt * KB + b) * 1024;
      for (int lane = 0; lane < 64; ++lane) {
        const int n = nt * 16 + (lane & 15), g = lane >> 4;
        const uint8_t* src = q + (size_t)n * K + 64 * b + 8 * g;
        memcpy(dst + lane * 16, src, 8);
        memcpy(dst + lane * 16 + 8, src + 32, 8);
      }
      for (int j = 0; j < 16; ++j) so[((size_t)nt * KB + b) * 16 + j] = s[(size_t)(nt * 16 + j) * KB + b];
    }
}

bool fp8_codes_ok(const uint8_t* q, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if ((q[i] & 0x7f) == 0x7f) return false;
  return true;
}
bool floats_ok(const float* s, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(s[i])) return false;
  return true;
}
bool bf16_ok(const uint8_t* q, size_t n) {   // n values, 2 bytes each, little-endian
  for (size_t i = 0; i < n; ++i)
    if ((q[2 * i + 1] & 0x7f) == 0x7f && (q[2 * i] & 0x80)) return false;   // exponent all ones
  return true;
}

// Host staging of a (possibly joined) weight matrix before upload, row-major.
struct HostMat {
  int fmt = kd::WF_FP8;
  int N = 0, K = 0;
  int ks = 0;                  // NVFP4: first 64-input block of the second tensor scale
  std::vector<uint8_t> q;      // per row: K code bytes (FP8), K/2 (NVFP4), 2K value bytes (bf16)
  std::vector<float> s;        // FP8: [N][K/64] block scales
  std::vector<uint8_t> s4;     // NVFP4: [N][K/16] block-scale codes
  std::vector<float> g0, g1;   // NVFP4: per row, the tensor scale before / from block ks
  size_t row_bytes(int k) const { return fmt == kd::WF_FP8 ? (size_t)k : (fmt == kd::WF_NVFP4 ? (size_t)k / 2 : (size_t)k * 2); }
};

// A host matrix in format fmt, rows x cols: pointers present, values valid
// (no NaN codes, finite scales and bf16 values).
bool mat_ok(const kd_matrix& x, int fmt, int rows, int cols) {
  const size_t n = (size_t)rows * cols;
  if (!x.q) return false;
  if (fmt == kd::WF_FP8) return x.s && fp8_codes_ok(x.q, n) && floats_ok(x.s, n / 64);
  if (fmt == kd::WF_NVFP4) return x.s4 && fp8_codes_ok(x.s4, n / 16) && std::isfinite(x.g);
  return bf16_ok(x.q, n);
}

bool append_rows(HostMat& m, const kd_matrix& src, int rows, int cols) {
  if (m.K == 0) m.K = cols;
  if (m.K != cols || !mat_ok(src, m.fmt, rows, cols)) return false;
  const size_t rb = m.row_bytes(cols);
  m.q.insert(m.q.end(), src.q, src.q + (size_t)rows * rb);
  if (m.fmt == kd::WF_FP8) m.s.insert(m.s.end(), src.s, src.s + (size_t)rows * cols / 64);
  if (m.fmt == kd::WF_NVFP4) {
    m.s4.insert(m.s4.end(), src.s4, src.s4 + (size_t)rows * cols / 16);
    m.g0.insert(m.g0.end(), rows, src.g);
    m.g1.insert(m.g1.end(), rows, src.g);
    m.ks = cols / 64;
  }
  m.N += rows;
  return true;
}

// [a | b] along the input dimension (same row count).
bool concat_cols(HostMat& m, const kd_matrix& a, const kd_matrix& b, int rows, int ca, int cb) {
  if (!mat_ok(a, m.fmt, rows, ca) || !mat_ok(b, m.fmt, rows, cb)) return false;
  m.N = rows;
  m.K = ca + cb;
  const size_t ra = m.row_bytes(ca), rb = m.row_bytes(cb);
  m.q.resize((size_t)rows * (ra + rb));
  for (int r = 0; r < rows; ++r) {
    memcpy(&m.q[(size_t)r * (ra + rb)], a.q + (size_t)r * ra, ra);
    memcpy(&m.q[(size_t)r * (ra + rb) + ra], b.q + (size_t)r * rb, rb);
  }
  if (m.fmt == kd::WF_FP8) {
    m.s.resize((size_t)rows * m.K / 64);
    for (int r = 0; r < rows; ++r) {
      memcpy(&m.s[(size_t)r * m.K / 64], a.s + (size_t)r * ca / 64, ca / 64 * sizeof(float));
      memcpy(&m.s[(size_t)r * m.K / 64 + ca / 64], b.s + (size_t)r * cb / 64, cb / 64 * sizeof(float));
    }
  }
  if (m.fmt == kd::WF_NVFP4) {
    m.s4.resize((size_t)rows * m.K / 16);
    for (int r = 0; r < rows; ++r) {
      memcpy(&m.s4[(size_t)r * m.K / 16], a.s4 + (size_t)r * ca / 16, ca / 16);
      memcpy(&m.s4[(size_t)r * m.K / 16 + ca / 16], b.s4 + (size_t)r * cb / 16, cb / 16);
    }
    m.g0.assign(rows, a.g);   // a's tensor scale on its blocks, b's from block ca / 64 on
    m.g1.assign(rows, b.g);
    m.ks = ca / 64;
  }
  return true;
}

// Reorders rows: row p of the result is row nat(p) of m.
void permute_rows(HostMat& m, int (*nat)(int)) {
  HostMat o = m;
  const size_t rb = m.row_bytes(m.K);
  for (int p = 0; p < m.N; ++p) {
    const int r = nat(p);
    memcpy(&o.q[(size_t)p * rb], &m.q[(size_t)r * rb], rb);
    if (m.fmt == kd::WF_FP8)
      memcpy(&o.s[(size_t)p * m.K / 64], &m.s[(size_t)r * m.K / 64], m.K / 64 * sizeof(float));
    if (m.fmt == kd::WF_NVFP4) {
      memcpy(&o.s4[(size_t)p * m.K / 16], &m.s4[(size_t)r * m.K / 16], m.K / 16);
      o.g0[p] = m.g0[r];
      o.g1[p] = m.g1[r];
    }
  }
  m = std::move(o);
}

// NVFP4 repack (layout in kd_device.h): codes [N/16][K/64][64 lanes][8],
// block-scale codes [N/16][K/64][16][4].
void repack_nvfp4(const uint8_t* q, const uint8_t* s4, int N, int K, uint8_t* wo, uint8_t* so) {
  const int KB = K / 64;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int b = 0; b < KB; ++b) {
      const size_t blk = (size_t)nt * KB + b;
      for (int lane = 0; lane < 64; ++lane) {
        const int n = nt * 16 + (lane & 15), g = lane >> 4;
        const uint8_t* src = q + (size_t)n * (K / 2) + (64 * b + 8 * g) / 2;
        memcpy(wo + blk * 512 + lane * 8, src, 4);
        memcpy(wo + blk * 512 + lane * 8 + 4, src + 16, 4);
      }
      for (int j = 0; j < 16; ++j) memcpy(so + blk * 64 + j * 4, s4 + (size_t)(nt * 16 + j) * (K / 16) + 4 * b, 4);
    }
}

// bf16 repack: [N/16][K/64][2 k tiles][64 lanes][8 values].
void repack_bf16(const uint8_t* q, int N, int K, uint8_t* wo) {
  const int KB = K / 64;
  for (int nt = 0; nt < N / 16; ++nt)
    for (int b = 0; b < KB; ++b)
      for (int j = 0; j < 2; ++j)
        for (int lane = 0; lane < 64; ++lane) {
          const int n = nt * 16 + (lane & 15), g = lane >> 4;
          memcpy(wo + (((size_t)nt * KB + b) * 2 + j) * 1024 + lane * 16,
                 q + ((size_t)n * K + 64 * b + 32 * j + 8 * g) * 2, 16);
        }
}

// An empty staging matrix in the context's body format.
HostMat body_mat(const kd_ctx* c) {
  HostMat m;
  m.fmt = c->cfg.body_quant == KD_QUANT_NVFP4 ? kd::WF_NVFP4
                                             : (c->cfg.body_quant == KD_QUANT_BF16 ? kd::WF_BF16 : kd::WF_FP8);
  return m;
}

kd_status upload_mat(kd_ctx* c, const HostMat& m, kd::WMat* out) {
  std::vector<uint8_t> wq(m.row_bytes(m.K) * m.N);
  std::vector<float> ws;
  std::vector<uint8_t> ws4;
  if (m.fmt == kd::WF_FP8) {
    ws.resize((size_t)m.N * m.K / 64);
    repack_fp8(m.q.data(), m.s.data(), m.N, m.K, wq.data(), ws.data());
  } else if (m.fmt == kd::WF_NVFP4) {
    ws4.resize((size_t)m.N * m.K / 16);
    repack_nvfp4(m.q.data(), m.s4.data(), m.N, m.K, wq.data(), ws4.data());
    ws = m.g0;
    ws.insert(ws.end(), m.g1.begin(), m.g1.end());
  } else {
    repack_bf16(m.q.data(), m.N, m.K, wq.data());
  }
  uint8_t* dw = nullptr;
  float* ds = nullptr;
  uint8_t* ds4 = nullptr;
  // scales get 1 KB of slack: the streamed round copies them in whole 1 KB
  // chunks, the last of which may run past the matrix
  if (!dev_alloc(c->weight_allocs, &dw, wq.size()) ||
      (!ws.empty() && !dev_alloc(c->weight_allocs, &ds, ws.size() + 256)) ||
      (!ws4.empty() && !dev_alloc(c->weight_allocs, &ds4, ws4.size())))
    return fail(c, KD_ERR_OOM, "weight allocation failed");
  hipError_t e = hipMemcpy(dw, wq.data(), wq.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess && ds) e = hipMemcpy(ds, ws.data(), ws.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess && ds4) e = hipMemcpy(ds4, ws4.data(), ws4.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(c, e, "weight upload");
  out->w = dw;
  out->s = ds;
  out->s4 = ds4;
  out->N = m.N;
  out->K = m.K;
  out->fmt = m.fmt;
  out->ks = m.fmt == kd::WF_NVFP4 ? m.ks : m.K / 64;
  return KD_OK;
}

kd_status upload_vec(kd_ctx* c, const float* src, size_t n, const float** out) {
  if (!src) return fail(c, KD_ERR_ARG, "NULL vector in weights");
  if (!floats_ok(src, n)) return fail(c, KD_ERR_ARG, "non-finite vector in weights");
  float* d;
  if (!dev_alloc(c->weight_allocs, &d, n)) return fail(c, KD_ERR_OOM, "weight allocation failed");
  hipError_t e = hipMemcpy(d, src, n * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(c, e, "weight upload");
  *out = d;
  return KD_OK;
}

kd::KV make_kv(const kd_kv* kv) {
  kd::KV k;
  k.fmt = kv->format;
  for (int l = 0; l < 4; ++l) {
    k.k[l] = static_cast<const uint16_t*>(kv->k[l]);
    k.v[l] = static_cast<const uint16_t*>(kv->v[l]);
    k.kso[l] = kv->format == KD_KV_INT4_ROT ? static_cast<const uint16_t*>(kv->k_so[l]) : nullptr;
    k.vso[l] = kv->format == KD_KV_INT4_ROT ? static_cast<const uint16_t*>(kv->v_so[l]) : nullptr;
  }
  k.ss = kv->stride_stream;
  k.sh = kv->stride_head;
  k.sl = kv->stride_slot;
  k.cap = kv->capacity;
  return k;
}

kd_status check_kv(kd_ctx* c, const kd_kv* kv) {
  if (!kv) return fail(c, KD_ERR_ARG, "ctx_kv is NULL");
  for (int l = 0; l < 4; ++l)
    if (!kv->k[l] || !kv->v[l]) return fail(c, KD_ERR_ARG, "NULL K/V tensor");
  if (kv->capacity < c->cfg.window)
    return fail(c, KD_ERR_ARG, "K/V capacity is smaller than the window");
  if (kv->format == KD_KV_INT4_ROT) {
    if (!c->d.kv_signs)
      return fail(c, KD_ERR_ARG, "a 4-bit cache needs kv_rot_signs in the loaded weights");
    for (int l = 0; l < 4; ++l) {
      if (!kv->k_so[l] || !kv->v_so[l]) return fail(c, KD_ERR_ARG, "NULL K/V scale tensor");
      if ((reinterpret_cast<uintptr_t>(kv->k[l]) | reinterpret_cast<uintptr_t>(kv->v[l])) & 15)
        return fail(c, KD_ERR_ARG, "K/V code tensors must be 16-byte aligned");
      if ((reinterpret_cast<uintptr_t>(kv->k_so[l]) | reinterpret_cast<uintptr_t>(kv->v_so[l])) & 3)
        return fail(c, KD_ERR_ARG, "K/V scale tensors must be 4-byte aligned");
    }
    if (kv->stride_slot < 1 || kv->stride_head < 1 || kv->stride_stream < 1)
      return fail(c, KD_ERR_ARG, "bad K/V strides");
    // the attention addresses one (stream, head)'s slots with 32-bit offsets
    if ((int64_t)(kv->capacity - 1) * kv->stride_slot * 64 + 64 > (int64_t)0xffffffffLL)
      return fail(c, KD_ERR_ARG, "4-bit cache: one (stream, head) spans more than 4 GiB of codes");
    return KD_OK;
  }
  if (kv->format != KD_KV_BF16) return fail(c, KD_ERR_ARG, "unknown K/V format");
  if (kv->stride_slot < kd::DH || kv->stride_head < 1 || kv->stride_stream < 1)
    return fail(c, KD_ERR_ARG, "bad K/V strides");
  for (int l = 0; l < 4; ++l)
    if ((reinterpret_cast<uintptr_t>(kv->k[l]) | reinterpret_cast<uintptr_t>(kv->v[l])) & 15)
      return fail(c, KD_ERR_ARG, "K/V tensors must be 16-byte aligned");
  if ((kv->stride_slot | kv->stride_head | kv->stride_stream) & 7)
    return fail(c, KD_ERR_ARG, "K/V strides must be multiples of 8 elements");
  return KD_OK;
}

}  // namespace

extern "C" {

void kd_default_config(kd_config* cfg) {
  if (!cfg) return;
  cfg->hidden = kd::H;
  cfg->heads = kd::NH;
  cfg->head_dim = kd::DH;
  cfg->ffn = kd::FF;
  cfg->layers = kd::NL;
  cfg->block = kd::BLK;
  cfg->rank = kd::RK;
  cfg->taps = kd::NTAP;
  cfg->window = 2048;
  cfg->draft_vocab = 60614;
  cfg->full_vocab = 131072;
  cfg->max_streams = 256;
  cfg->rope_theta = 10000.0f;
  cfg->rms_eps = 1e-6f;
  cfg->body_quant = KD_QUANT_FP8_BLOCK64;
  cfg->head_quant = KD_QUANT_NVFP4;
}

const char* kd_status_string(kd_status s) {
  switch (s) {
    case KD_OK: return "ok";
    case KD_ERR_ARG: return "invalid argument";
    case KD_ERR_STATE: return "invalid state";
    case KD_ERR_OOM: return "out of device memory";
    case KD_ERR_HIP: return "HIP runtime error";
    case KD_ERR_UNSUPPORTED: return "unsupported configuration";
    case KD_ERR_RANGE: return "an activation left the f16 range";
  }
  return "unknown status";
}

const char* kd_last_error(const kd_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

kd_status kd_create(const kd_config* cfg, void* hip_stream, kd_ctx** out) {
  if (!out) return KD_ERR_ARG;
  *out = nullptr;
  if (!cfg) return KD_ERR_ARG;
  if (!shape_is_supported(*cfg)) return KD_ERR_UNSUPPORTED;
  if ((cfg->body_quant != KD_QUANT_FP8_BLOCK64 && cfg->body_quant != KD_QUANT_NVFP4 &&
       cfg->body_quant != KD_QUANT_BF16) ||
      (cfg->head_quant != KD_QUANT_NVFP4 && cfg->head_quant != KD_QUANT_BF16 &&
       cfg->head_quant != KD_QUANT_FP8_BLOCK64))
    return KD_ERR_UNSUPPORTED;
  if (cfg->window < 1 || cfg->draft_vocab < 1 || cfg->full_vocab < 1 || cfg->max_streams < 1 ||
      !(cfg->rms_eps >= 0.f) || !(cfg->rope_theta > 0.f))
    return KD_ERR_ARG;
  if (cfg->max_streams > (1 << 20) || cfg->draft_vocab > (1 << 28) || cfg->window > (1 << 24))
    return KD_ERR_OOM;
  kd_ctx* c = new kd_ctx;
  c->cfg = *cfg;
  c->stream = static_cast<hipStream_t>(hip_stream);
  (void)hipGetDevice(&c->device);
  kd::Work& w = c->w;
  w.Bmax = cfg->max_streams;
  w.Rmax = kd::BLK * w.Bmax;
  w.Imax = KD_MAX_INGEST * w.Bmax;
  w.af_ing_layer = kd::afrag_elems(w.Imax, kd::H);
  w.att_nch = (cfg->window + kd::ATT_CH - 1) / kd::ATT_CH;
  const int BI = std::max(w.Bmax, w.Imax), RI = std::max(w.Rmax, w.Imax);
  w.part_elems = 2 * part_region_elems(w.Bmax);
  bool ok = dev_alloc(c->work_allocs, &w.f, (size_t)BI * kd::H) &&
            dev_alloc(c->work_allocs, &w.x, (size_t)w.Rmax * kd::H) &&
            dev_alloc(c->work_allocs, &w.c, (size_t)w.Imax * kd::H) &&
            dev_alloc(c->work_allocs, &w.part, w.part_elems) &&
            dev_alloc(c->work_allocs, &w.af_in, kd::afrag_elems(BI, kd::NTAP * kd::H)) &&
            dev_alloc(c->work_allocs, &w.af_fc, kd::afrag_elems(BI, 2 * kd::H)) &&
            dev_alloc(c->work_allocs, &w.af_ab, kd::afrag_elems(3 * w.Bmax, 2 * kd::H)) &&
            dev_alloc(c->work_allocs, &w.af_rank, kd::afrag_elems(3 * w.Bmax, kd::RK)) &&
            dev_alloc(c->work_allocs, &w.af_x, kd::afrag_elems(RI, kd::H)) &&
            dev_alloc(c->work_allocs, &w.af_sp, kd::afrag_elems(3 * w.Bmax, kd::H)) &&
            dev_alloc(c->work_allocs, &w.af_h, kd::afrag_elems(w.Rmax, kd::FF)) &&
            dev_alloc(c->work_allocs, &w.af_o, kd::afrag_elems(w.Rmax, kd::H)) &&
            dev_alloc(c->work_allocs, &w.q, (size_t)w.Rmax * kd::H) &&
            dev_alloc(c->work_allocs, &w.kb, (size_t)w.Rmax * kd::H) &&
            dev_alloc(c->work_allocs, &w.vb, (size_t)w.Rmax * kd::H) &&
            dev_alloc(c->work_allocs, &w.rope, (size_t)w.Bmax * kd::BLK * kd::DH) &&
            dev_alloc(c->work_allocs, &w.att_m, (size_t)w.Bmax * kd::NH * w.att_nch * kd::BLK) &&
            dev_alloc(c->work_allocs, &w.att_l, (size_t)w.Bmax * kd::NH * w.att_nch * kd::BLK) &&
            dev_alloc(c->work_allocs, &w.att_o,
                      (size_t)w.Bmax * kd::NH * w.att_nch * kd::BLK * kd::DH) &&
            dev_alloc(c->work_allocs, &w.af_ing, kd::NL * kd::afrag_elems(w.Imax, kd::H)) &&
            dev_alloc(c->work_allocs, &w.att_cnt, (size_t)w.Bmax * kd::NH * 32) &&
            hipMemset(w.att_cnt, 0, (size_t)w.Bmax * kd::NH * 32 * sizeof(unsigned)) == hipSuccess &&
            hipDeviceSynchronize() == hipSuccess &&
            dev_alloc(c->work_allocs, &w.keys, (size_t)w.Rmax) &&
            dev_alloc(c->work_allocs, &w.copy_keys, (size_t)2 * w.Bmax);
  hipDeviceProp_t prop;
  const bool have_prop = hipGetDeviceProperties(&prop, c->device) == hipSuccess;
  c->G = have_prop ? std::min(prop.multiProcessorCount, kd::MAX_G) : 128;
  // the small-batch paths serve any window; their attention merges one
  // (stream, head) per workgroup, so the grid must cover every pair
  c->small_ok = c->G >= kd::SB_MAX * kd::NH;
  if (ok && c->small_ok) {
    ok = dev_alloc(c->work_allocs, &c->small_mem, kd::small_bytes(kd::small_nch(cfg->window)));
    for (int i = 0; i < kd_ctx::NSLOT; ++i) ok = ok && dev_alloc(c->work_allocs, &c->args_dev[i], 1);
    if (ok) {
      kd::small_carve(c->small_mem, kd::small_nch(cfg->window), &c->small);
      ok = hipMemset(c->small.bar, 0, 20 * 32 * sizeof(unsigned)) == hipSuccess &&
           hipMemset(c->small.att_cnt, 0, kd::NL * kd::SB_MAX * kd::NH * 32 * sizeof(unsigned)) ==
               hipSuccess &&
           hipMemset(c->small.down_cnt, 0, kd::NL * (kd::HT / 2) * 32 * sizeof(unsigned)) == hipSuccess &&
           hipDeviceSynchronize() == hipSuccess;
    }
  }
  ok = ok && c->stager.init(sizeof(kd::SmallArgs)) &&
       hipHostMalloc((void**)&c->status_host, 64, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
       hipHostGetDevicePointer((void**)&c->status_dev, c->status_host, 0) == hipSuccess;
  if (ok) c->status_host[0] = c->status_host[1] = 0u;
  if (!ok) {
    free_all(c->work_allocs);
    c->stager.destroy();
    if (c->status_host) (void)hipHostFree(c->status_host);
    delete c;
    return KD_ERR_OOM;
  }
  c->mega_ok = c->small_ok && have_prop && prop.cooperativeLaunch && kd::small_mega_occupancy() >= 1;
  (void)hipGetLastError();
  *out = c;
  return KD_OK;
}

kd_status kd_set_stream(kd_ctx* ctx, void* hip_stream) {
  if (!ctx) return KD_ERR_ARG;
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  return KD_OK;
}

void kd_destroy(kd_ctx* ctx) {
  if (!ctx) return;
  (void)hipStreamSynchronize(ctx->stream);
  for (int i = 0; i < kd_ctx::NSLOT; ++i)
    if (ctx->phase_graph[i]) (void)hipGraphExecDestroy(ctx->phase_graph[i]);
  drop_graphs(ctx->round_graph);
  drop_graphs(ctx->ingest_graph);
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  free_all(ctx->work_allocs);
  free_all(ctx->weight_allocs);
  ctx->stager.destroy();
  if (ctx->status_host) (void)hipHostFree(ctx->status_host);
  delete ctx;
}

kd_status kd_load_weights(kd_ctx* c, const kd_weights* wt) {
  if (!c) return KD_ERR_ARG;
  if (!wt) return fail(c, KD_ERR_ARG, "weights is NULL");
  const int H = kd::H, F = kd::FF, r = kd::RK;
  const int VD = c->cfg.draft_vocab;
  const bool head_bf16 = c->cfg.head_quant == KD_QUANT_BF16;
  const bool head_fp8 = c->cfg.head_quant == KD_QUANT_FP8_BLOCK64;
  if ((head_bf16 ? !wt->head_bf16
                 : head_fp8 ? (!wt->head_fp8.q || !wt->head_fp8.s) : (!wt->head_q4 || !wt->head_s4)) ||
      !wt->draft_vocab ||
      !wt->embed_table || !wt->mask_row || !wt->final_norm)
    return fail(c, KD_ERR_ARG, "NULL pointer in weights");
  if (!head_bf16 && !head_fp8 && !std::isfinite(wt->head_g))
    return fail(c, KD_ERR_ARG, "non-finite head scale");
  for (int i = 0; i < VD; ++i)
    if (wt->draft_vocab[i] < 0 || wt->draft_vocab[i] >= c->cfg.full_vocab)
      return fail(c, KD_ERR_ARG, "draft vocabulary id out of range");
  (void)hipStreamSynchronize(c->stream);
  free_all(c->weight_allocs);
  c->loaded = false;
  kd::DevWeights& d = c->d;
  d.zrow = nullptr;

  kd_status st;
  {
    HostMat m = body_mat(c);
    if (!append_rows(m, wt->fuse, H, kd::NTAP * H)) return fail(c, KD_ERR_ARG, "bad fuse matrix");
    if ((st = upload_mat(c, m, &d.fuse)) != KD_OK) return st;
  }
  {
    HostMat m = body_mat(c);
    if (!append_rows(m, wt->fc, H, 2 * H)) return fail(c, KD_ERR_ARG, "bad fc matrix");
    if ((st = upload_mat(c, m, &d.fc)) != KD_OK) return st;
  }
  {
    HostMat m = body_mat(c);
    if (!concat_cols(m, wt->pred_a, wt->pred_b, r, H, H))
      return fail(c, KD_ERR_ARG, "bad predecessor A/B matrix");
    if ((st = upload_mat(c, m, &d.pred_ab)) != KD_OK) return st;
  }
  {
    HostMat m = body_mat(c);
    if (!append_rows(m, wt->pred_u, H, r)) return fail(c, KD_ERR_ARG, "bad predecessor U matrix");
    if ((st = upload_mat(c, m, &d.pred_u)) != KD_OK) return st;
  }
  if ((st = upload_vec(c, wt->mask_row, H, &d.mask)) != KD_OK) return st;
  for (int l = 0; l < kd::NL; ++l) {
    const kd_layer_weights& L = wt->layer[l];
    kd::DevLayer& D = d.layer[l];
    HostMat qkv = body_mat(c), wo = qkv, gu = qkv, dn = qkv;
    if (!append_rows(qkv, L.wq, H, H) || !append_rows(qkv, L.wk, H, H) ||
        !append_rows(qkv, L.wv, H, H))
      return fail(c, KD_ERR_ARG, "bad q/k/v matrix");
    if (!append_rows(wo, L.wo, H, H)) return fail(c, KD_ERR_ARG, "bad o matrix");
    if (!append_rows(gu, L.w_gate, F, H) || !append_rows(gu, L.w_up, F, H))
      return fail(c, KD_ERR_ARG, "bad gate/up matrix");
    if (!append_rows(dn, L.w_down, H, F)) return fail(c, KD_ERR_ARG, "bad down matrix");
    permute_rows(qkv, kd::qkv_natural);
    permute_rows(gu, kd::gu_natural);
    if ((st = upload_mat(c, qkv, &D.qkv)) != KD_OK || (st = upload_mat(c, wo, &D.wo)) != KD_OK ||
        (st = upload_mat(c, gu, &D.gu)) != KD_OK || (st = upload_mat(c, dn, &D.down)) != KD_OK)
      return st;
    if ((st = upload_vec(c, L.attn_norm, H, &D.attn_norm)) != KD_OK ||
        (st = upload_vec(c, L.ffn_norm, H, &D.ffn_norm)) != KD_OK)
      return st;
    if (l >= 1) {
      HostMat sa = body_mat(c), su = sa;
      if (!append_rows(sa, L.spine_a, r, H) || !append_rows(su, L.spine_u, H, r))
        return fail(c, KD_ERR_ARG, "bad spine matrix");
      if ((st = upload_mat(c, sa, &D.sa)) != KD_OK || (st = upload_mat(c, su, &D.su)) != KD_OK)
        return st;
      if ((st = upload_vec(c, L.spine_norm, H, &D.spine_norm)) != KD_OK) return st;
    }
  }
  if ((st = upload_vec(c, wt->final_norm, H, &d.final_norm)) != KD_OK) return st;
  // signs of the rotated 4-bit cache, kept as +-1.0f
  d.kv_signs = nullptr;
  if (wt->kv_rot_signs) {
    std::vector<float> sg((size_t)kd::NL * kd::DH);
    for (size_t i = 0; i < sg.size(); ++i) {
      const int8_t v = wt->kv_rot_signs[i];
      if (v != 1 && v != -1) return fail(c, KD_ERR_ARG, "kv_rot_signs entries must be +1 or -1");
      sg[i] = (float)v;
    }
    if ((st = upload_vec(c, sg.data(), sg.size(), &d.kv_signs)) != KD_OK) return st;
  }

  const int VT = (VD + 15) / 16;
  d.hf8 = kd::WMat();
  if (head_fp8) {
    // block-FP8 head rows, zero rows (code 0, scale 1) up to whole 16-row
    // tiles, repacked as a body matrix
    HostMat m;
    if (!append_rows(m, wt->head_fp8, VD, H)) return fail(c, KD_ERR_ARG, "bad FP8 head");
    m.q.resize((size_t)VT * 16 * H, 0);
    m.s.resize((size_t)VT * 16 * H / 64, 1.0f);
    m.N = VT * 16;
    if ((st = upload_mat(c, m, &d.hf8)) != KD_OK) return st;
    int32_t* dv;
    if (!dev_alloc(c->weight_allocs, &dv, (size_t)VD)) return fail(c, KD_ERR_OOM, "head allocation failed");
    const hipError_t e = hipMemcpy(dv, wt->draft_vocab, (size_t)VD * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(c, e, "head upload");
    d.head_fmt = 2;
    d.hb = nullptr;
    d.hq = nullptr;
    d.hs = nullptr;
    d.hg = 1.f;
    d.VD = VD;
    d.VT = VT;
    d.vocab = dv;
  } else if (head_bf16) {
    // bf16 head rows repacked to the B operand of the 16x16x32 bf16 matrix
    // cores: [VT][H/32][64 lanes][8] (lane l: row 16 vt + l % 16, inputs
    // 32 t + 8 (l / 16) .. + 8), rows past the vocabulary zero
    const uint16_t* src = static_cast<const uint16_t*>(wt->head_bf16);
    for (size_t i = 0; i < (size_t)VD * H; ++i)
      if ((src[i] & 0x7f80) == 0x7f80) return fail(c, KD_ERR_ARG, "non-finite bf16 head value");
    const int KT = H / 32;
    std::vector<uint16_t> hb((size_t)VT * KT * 512, 0);
    for (int vt = 0; vt < VT; ++vt)
      for (int t = 0; t < KT; ++t)
        for (int lane = 0; lane < 64; ++lane) {
          const int row = 16 * vt + (lane & 15);
          if (row >= VD) continue;
          memcpy(&hb[((size_t)(vt * KT + t) * 64 + lane) * 8], src + (size_t)row * H + 32 * t + 8 * (lane >> 4),
                 16);
        }
    uint16_t* dh;
    int32_t* dv;
    if (!dev_alloc(c->weight_allocs, &dh, hb.size()) || !dev_alloc(c->weight_allocs, &dv, (size_t)VD))
      return fail(c, KD_ERR_OOM, "head allocation failed");
    hipError_t e = hipMemcpy(dh, hb.data(), hb.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(dv, wt->draft_vocab, (size_t)VD * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(c, e, "head upload");
    d.head_fmt = 1;
    d.hb = dh;
    d.hq = nullptr;
    d.hs = nullptr;
    d.hg = 1.f;
    d.VD = VD;
    d.VT = VT;
    d.vocab = dv;
  } else {
  // NVFP4 head, repacked to 16-row vocab tiles (layout in kd_device.h).
  const int KG = H / 128;
  for (size_t i = 0; i < (size_t)VD * H / 16; ++i)
    if ((wt->head_s4[i] & 0x7f) == 0x7f) return fail(c, KD_ERR_ARG, "NaN head block scale");
  std::vector<uint8_t> hq((size_t)VT * KG * 64 * 16, 0), hs((size_t)VT * KG * 64 * 4, 0);
  for (int vt = 0; vt < VT; ++vt)
    for (int kg = 0; kg < KG; ++kg)
      for (int lane = 0; lane < 64; ++lane) {
        const int row = vt * 16 + (lane & 15), g = lane >> 4;
        if (row >= VD) continue;
        const size_t o = ((size_t)vt * KG + kg) * 64 + lane;
        for (int i = 0; i < 4; ++i) {
          const int kbase = 32 * (4 * kg + i) + 8 * g;
          memcpy(&hq[o * 16 + 4 * i], wt->head_q4 + (size_t)row * (H / 2) + kbase / 2, 4);
          hs[o * 4 + i] = wt->head_s4[(size_t)row * (H / 16) + kbase / 16];
        }
      }
  uint8_t *dq, *ds;
  int32_t* dv;
  if (!dev_alloc(c->weight_allocs, &dq, hq.size()) || !dev_alloc(c->weight_allocs, &ds, hs.size()) ||
      !dev_alloc(c->weight_allocs, &dv, (size_t)VD))
    return fail(c, KD_ERR_OOM, "weight allocation failed");
  hipError_t e = hipMemcpy(dq, hq.data(), hq.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(ds, hs.data(), hs.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(dv, wt->draft_vocab, (size_t)VD * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(c, e, "head upload");
  d.hq = dq;
  d.hs = ds;
  d.hg = wt->head_g;
  d.VD = VD;
  d.VT = VT;
  d.vocab = dv;
  d.head_fmt = 0;
  d.hb = nullptr;
  }
  d.table = static_cast<const uint16_t*>(wt->embed_table);
  d.V = c->cfg.full_vocab;
  if (!d.zrow) {
    uint16_t* z;
    if (!dev_alloc(c->weight_allocs, &z, (size_t)kd::H)) return fail(c, KD_ERR_OOM, "weight allocation failed");
    const hipError_t e = hipMemset(z, 0, (size_t)kd::H * sizeof(uint16_t));
    if (e != hipSuccess) return hip_fail(c, e, "zero row");
    d.zrow = z;
  }
  for (int i = 0; i < kd_ctx::NSLOT; ++i) c->args_valid[i] = false;
  drop_graphs(c->round_graph);
  drop_graphs(c->ingest_graph);
  c->loaded = true;
  c->err.clear();
  return KD_OK;
}

// `depth` rounds; round r > 0 reads its predecessor ids from out_ids (the
// previous round's drafts, 4 per stream).
// A bounded device wait of an earlier call timed out (its rounds wrote -2 ids).
// The status words earlier rounds left in mapped host memory: [0] a bounded
// wait timed out, [1] an f16 activation store saturated. Each is read and
// cleared once.
static kd_status take_device_status(kd_ctx* c) {
  if (!c->status_host) return KD_OK;
  const unsigned timeout = __atomic_exchange_n(&c->status_host[0], 0u, __ATOMIC_ACQ_REL);
  const unsigned range = __atomic_exchange_n(&c->status_host[1], 0u, __ATOMIC_ACQ_REL);
  if (timeout) return fail(c, KD_ERR_HIP, "a device wait of an earlier round timed out; that round wrote -2 ids");
  if (range)
    return fail(c, KD_ERR_RANGE,
                "an earlier round stored an f16 activation beyond +-65504 or not finite (stored saturated); "
                "its drafts are unreliable");
  return KD_OK;
}

static kd_status round_impl(kd_ctx* c, int depth, int B, const void* taps, const int32_t* anchor,
                            const int32_t* pred, const kd_kv* kv, const int32_t* lens,
                            int32_t* out_ids, float* out_logits) {
  if (!c->loaded) return fail(c, KD_ERR_STATE, "kd_round before kd_load_weights");
  {
    const kd_status ds = take_device_status(c);
    if (ds != KD_OK) return ds;
  }
  if (B < 1 || B > c->cfg.max_streams) return fail(c, KD_ERR_ARG, "streams out of range");
  if (!taps || !anchor || !pred || !lens || !out_ids)
    return fail(c, KD_ERR_ARG, "NULL device pointer");
  if (reinterpret_cast<uintptr_t>(taps) & 15)
    return fail(c, KD_ERR_ARG, "tapped_states must be 16-byte aligned");
  kd_status s = check_kv(c, kv);
  if (s != KD_OK) return s;
  const kd::KV k = make_kv(kv);
  const kd::Work& w = c->w;
  const kd::DevWeights& d = c->d;
  const hipStream_t st = c->stream;
  const float eps = c->cfg.rms_eps;
  const int R = kd::BLK * B, B3 = 3 * B;
  int path = c->path;
  // automatic: the per-phase launches (path 2) are the fastest measured small-
  // batch form on MI355X; the persistent form (3) is kept selectable
  if (path == 0) path = B <= kd::SB_MAX && c->small_ok ? 2 : 1;
  if (!c->small_ok) path = 1;
  if (path == 3 && !c->mega_ok) path = 2;
  if (path != 1 && B > kd::SB_MAX) path = 1;
  c->last_path = path;
  if (path != 1) {
    (void)hipGetLastError();
    for (int r = 0; r < depth; ++r) {
      const bool first = r == 0, last = r + 1 == depth;
      const int slot = first && last ? 0 : first ? 1 : last ? 3 : 2;
      kd::SmallArgs a;
      memset(&a, 0, sizeof a);
      a.B = B;
      a.R = R;
      a.nl = c->debug_layers < 0 ? kd::NL : c->debug_layers;
      a.window = c->cfg.window;
      // partial slots per (stream, head), as the buffers were carved
      a.nch = kd::small_nch(c->cfg.window);
      a.eps = eps;
      a.theta = c->cfg.rope_theta;
      a.taps = static_cast<const uint16_t*>(taps);
      a.anchor = anchor;
      a.pred = r == 0 ? pred : out_ids;
      a.pred_stride = r == 0 ? kd::BLK - 1 : kd::BLK;
      a.lens = lens;
      a.kv = k;
      a.out_ids = out_ids;
      a.out_logits = r + 1 == depth ? out_logits : nullptr;
      a.d = d;
      a.s = c->small;
      a.status = c->status_dev;
      a.trace = c->trace;
      a.trace_phases = c->trace_phases;
      // upload the argument block only when it changed (a serving loop that
      // reuses its buffers uploads it once); the upload is queued on the
      // stream ahead of the launches that read it
      if (!c->args_valid[slot] || memcmp(&c->args_cur[slot], &a, sizeof a) != 0) {
        const hipError_t e = c->stager.upload(c->args_dev[slot], &a, sizeof a, st);
        if (e != hipSuccess) return hip_fail(c, e, "argument upload");
        c->args_cur[slot] = a;
        c->args_valid[slot] = true;
      }
      const int np = kd::small_phase_count(a.nl);
      if (path == 3) {
        const hipError_t e = kd::launch_small_mega(st, c->args_dev[slot], c->G, c->epoch, d.fuse.fmt);
        if (e != hipSuccess) return hip_fail(c, e, "persistent round launch");
        c->epoch += (unsigned)(np - 1);
      } else {
        if (!c->phase_graph[slot] || c->phase_graph_nl[slot] != a.nl) {
          hipError_t e = hipSuccess;
          if (c->phase_graph[slot]) {
            (void)hipGraphExecDestroy(c->phase_graph[slot]);
            c->phase_graph[slot] = nullptr;
          }
          if (!c->cap_stream) e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking);
          hipGraph_t g = nullptr;
          if (e == hipSuccess) e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
          if (e == hipSuccess) {
            for (int i = 0; i < np; ++i)
              kd::launch_small_phase(c->cap_stream, c->args_dev[slot], c->G, kd::small_phase_id(a.nl, i), i,
                                     d.fuse.fmt);
            e = hipStreamEndCapture(c->cap_stream, &g);
          }
          if (e == hipSuccess) e = hipGraphInstantiate(&c->phase_graph[slot], g, nullptr, nullptr, 0);
          if (g) (void)hipGraphDestroy(g);
          if (e != hipSuccess) return hip_fail(c, e, "phase graph capture");
          c->phase_graph_nl[slot] = a.nl;
        }
        const hipError_t e = hipGraphLaunch(c->phase_graph[slot], st);
        if (e != hipSuccess) return hip_fail(c, e, "phase graph launch");
      }
    }
    c->last_streams = B;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(c, e, "kd_round launch");
    return KD_OK;
  }
  float* partA = w.part;
  float* partB = w.part + w.part_elems / 2;
  const int nl = c->debug_layers < 0 ? kd::NL : c->debug_layers;
  // more than two row tiles: q|k|v and gate|up run with their epilogues fused
  const bool fused = R > 32 && c->fused_proj;
  (void)hipGetLastError();
  auto enqueue = [&](hipStream_t st) {
    for (int r = 0; r < depth; ++r) {
      const int32_t* pred_r = r == 0 ? pred : out_ids;
      const int pred_stride = r == 0 ? kd::BLK - 1 : kd::BLK;
      kd::launch_prep(st, w, d, B, static_cast<const uint16_t*>(taps), lens, c->cfg.rope_theta);
      const int s_fuse = kd::gemm_splits(d.fuse.K, d.fuse.N, B);
      kd::launch_gemm(st, w.af_in, B, d.fuse, 0, d.fuse.N, partA, s_fuse);
      kd::launch_post_fuse(st, w, d, B, s_fuse, anchor, pred_r, pred_stride);
      const int s_fc = kd::gemm_splits(d.fc.K, d.fc.N, B);
      kd::launch_gemm(st, w.af_fc, B, d.fc, 0, d.fc.N, partA, s_fc);
      const int s_ab = kd::gemm_splits(d.pred_ab.K, d.pred_ab.N, B3);
      kd::launch_gemm(st, w.af_ab, B3, d.pred_ab, 0, d.pred_ab.N, partB, s_ab);
      kd::launch_silu_rank(st, partB, s_ab, B3, w.af_rank);
      const int s_u = kd::gemm_splits(d.pred_u.K, d.pred_u.N, B3);
      kd::launch_gemm(st, w.af_rank, B3, d.pred_u, 0, d.pred_u.N, partB, s_u);
      kd::launch_rowbuild(st, w, d, B, s_fc, s_u, d.layer[0].attn_norm, eps);

      for (int l = 0; l < nl; ++l) {
        const kd::DevLayer& L = d.layer[l];
        if (l >= 1) {
          const int s_sa = kd::gemm_splits(L.sa.K, L.sa.N, B3);
          kd::launch_gemm(st, w.af_sp, B3, L.sa, 0, L.sa.N, partA, s_sa);
          kd::launch_silu_rank(st, partA, s_sa, B3, w.af_rank);
          const int s_su = kd::gemm_splits(L.su.K, L.su.N, B3);
          kd::launch_gemm(st, w.af_rank, B3, L.su, 0, L.su.N, partA, s_su);
          kd::launch_spine_add_norm(st, w, B, s_su, L.attn_norm, eps);
        }
        if (fused) {
          // one split, RoPE in the projection's epilogue
          kd::ProjEpi e;
          e.kind = kd::PE_QKV;
          e.rope = w.rope;
          e.q = w.q;
          e.kb = w.kb;
          e.vb = w.vb;
          kd::launch_proj(st, w.af_x, R, L.qkv, e);
        } else {
          const int s_qkv = kd::gemm_splits(L.qkv.K, L.qkv.N, R);
          kd::launch_gemm(st, w.af_x, R, L.qkv, 0, L.qkv.N, partA, s_qkv);
          kd::launch_qkv_post(st, w, B, s_qkv);
        }
        kd::launch_attention(st, w, d, B, k, l, lens, c->cfg.window);
        const int s_o = kd::gemm_splits(L.wo.K, L.wo.N, R);
        kd::launch_gemm(st, w.af_o, R, L.wo, 0, L.wo.N, partA, s_o);
        kd::launch_resid_norm(st, w, R, s_o, L.ffn_norm, eps, w.af_x, 0);
        if (fused) {
          // one split, SwiGLU in the projection's epilogue
          kd::ProjEpi e;
          e.kind = kd::PE_SWIGLU;
          e.af = w.af_h;
          kd::launch_proj(st, w.af_x, R, L.gu, e);
        } else {
          const int s_gu = kd::gemm_splits(L.gu.K, L.gu.N, R);
          kd::launch_gemm(st, w.af_x, R, L.gu, 0, L.gu.N, partA, s_gu);
          kd::launch_swiglu(st, w, R, s_gu);
        }
        const int s_d = kd::gemm_splits(L.down.K, L.down.N, R);
        kd::launch_gemm(st, w.af_h, R, L.down, 0, L.down.N, partA, s_d);
        if (l + 1 < nl)
          kd::launch_resid_norm(st, w, R, s_d, d.layer[l + 1].spine_norm, eps, w.af_sp, 1);
        else
          kd::launch_resid_norm(st, w, R, s_d, d.final_norm, eps, w.af_x, 0);
      }
      if (nl == 0) kd::launch_norm_rows(st, w.x, R, d.final_norm, eps, w.af_x);
      kd::launch_head(st, w, d, R, r + 1 == depth ? out_logits : nullptr);
      kd::launch_finalize(st, w, d, R, out_ids, anchor, pred_r, pred_stride, c->status_dev + 1);
    }
  };
  std::vector<unsigned char> key;
  key_add(key, depth);
  key_add(key, B);
  key_add(key, nl);
  key_add(key, taps);
  key_add(key, anchor);
  key_add(key, pred);
  key_add_kv(key, k);
  key_add(key, lens);
  key_add(key, out_ids);
  key_add(key, out_logits);
  s = launch_cached(c, c->round_graph, std::move(key), st, enqueue, "general round graph");
  if (s != KD_OK) return s;
  c->last_streams = B;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(c, e, "kd_round launch");
  return KD_OK;
}

kd_status kd_round(kd_ctx* c, int B, const void* taps, const int32_t* anchor, const int32_t* pred,
                   const kd_kv* kv, const int32_t* lens, int32_t* out_ids, float* out_logits) {
  if (!c) return KD_ERR_ARG;
  return round_impl(c, 1, B, taps, anchor, pred, kv, lens, out_ids, out_logits);
}

kd_status kd_round_depth(kd_ctx* c, int depth, int B, const void* taps, const int32_t* anchor,
                         const int32_t* pred, const kd_kv* kv, const int32_t* lens,
                         int32_t* out_ids, float* out_logits) {
  if (!c) return KD_ERR_ARG;
  if (depth < 1 || depth > KD_MAX_DEPTH) return fail(c, KD_ERR_ARG, "depth out of range");
  return round_impl(c, depth, B, taps, anchor, pred, kv, lens, out_ids, out_logits);
}

kd_status kd_ingest(kd_ctx* c, int B, int n_new, const void* taps, const int32_t* next_ids,
                    const kd_kv* kv, int32_t* lens) {
  if (!c) return KD_ERR_ARG;
  if (!c->loaded) return fail(c, KD_ERR_STATE, "kd_ingest before kd_load_weights");
  {
    const kd_status ds = take_device_status(c);
    if (ds != KD_OK) return ds;
  }
  if (B < 1 || B > c->cfg.max_streams) return fail(c, KD_ERR_ARG, "streams out of range");
  if (n_new < 1 || n_new > KD_MAX_INGEST) return fail(c, KD_ERR_ARG, "n_new out of range");
  if (!taps || !next_ids || !lens) return fail(c, KD_ERR_ARG, "NULL device pointer");
  if (reinterpret_cast<uintptr_t>(taps) & 15)
    return fail(c, KD_ERR_ARG, "taps must be 16-byte aligned");
  kd_status s = check_kv(c, kv);
  if (s != KD_OK) return s;
  const kd::KV k = make_kv(kv);
  const kd::Work& w = c->w;
  const kd::DevWeights& d = c->d;
  const hipStream_t st = c->stream;
  const int rows = B * n_new;
  (void)hipGetLastError();
  auto enqueue = [&](hipStream_t st) {
    kd::launch_ingest_prep(st, w, rows, static_cast<const uint16_t*>(taps));
    const int s_fuse = kd::gemm_splits(d.fuse.K, d.fuse.N, rows);
    kd::launch_gemm(st, w.af_in, rows, d.fuse, 0, d.fuse.N, w.part, s_fuse);
    kd::launch_ingest_post_fuse(st, w, d, rows, s_fuse, next_ids);
    const int s_fc = kd::gemm_splits(d.fc.K, d.fc.N, rows);
    kd::launch_gemm(st, w.af_fc, rows, d.fc, 0, d.fc.N, w.part, s_fc);
    kd::launch_ingest_c(st, w, rows, s_fc);
    if (rows > 32 && c->fused_proj) {
      // every layer's normed rows, then every layer's k|v projection with the
      // cache store in one launch
      kd::launch_norm_rows_layers(st, w.c, rows, d, c->cfg.rms_eps, w.af_ing, w.af_ing_layer);
      kd::IngestEpi e;
      e.n_new = n_new;
      e.lens = lens;
      e.theta = c->cfg.rope_theta;
      e.kv = k;
      e.signs = d.kv_signs;
      kd::launch_ingest_proj(st, w.af_ing, w.af_ing_layer, rows, d, e);
    } else {
      for (int l = 0; l < kd::NL; ++l) {
        const kd::DevLayer& L = d.layer[l];
        kd::launch_norm_rows(st, w.c, rows, L.attn_norm, c->cfg.rms_eps, w.af_x);
      const int s_kv = kd::gemm_splits(L.qkv.K, 2 * kd::H, rows);
      kd::launch_gemm(st, w.af_x, rows, L.qkv, kd::H / 16, 2 * kd::H, w.part, s_kv);
        kd::launch_ingest_store(st, w, d, B, n_new, s_kv, k, l, lens, c->cfg.rope_theta);
      }
    }
    kd::launch_bump_lens(st, lens, B, n_new);
  };
  std::vector<unsigned char> key;
  key_add(key, B);
  key_add(key, n_new);
  key_add(key, taps);
  key_add(key, next_ids);
  key_add_kv(key, k);
  key_add(key, lens);
  s = launch_cached(c, c->ingest_graph, std::move(key), st, enqueue, "ingest graph");
  if (s != KD_OK) return s;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(c, e, "kd_ingest launch");
  return KD_OK;
}

kd_status kd_copy_draft(kd_ctx* c, int B, const int32_t* tokens, long long stride,
                        const int32_t* lens, const int32_t* corpus, long long corpus_len, int K,
                        int32_t* out_ids, int32_t* out_info) {
  if (!c) return KD_ERR_ARG;
  if (B < 1 || B > c->cfg.max_streams) return fail(c, KD_ERR_ARG, "streams out of range");
  if (K < 1 || K > KD_MAX_COPY) return fail(c, KD_ERR_ARG, "K out of range");
  if (stride < 0 || stride >= (1ll << 31) || corpus_len < 0 || corpus_len >= (1ll << 31))
    return fail(c, KD_ERR_ARG, "history stride or corpus length out of range");
  if ((stride > 0 && !tokens) || !lens || !out_ids || !out_info || (corpus_len > 0 && !corpus))
    return fail(c, KD_ERR_ARG, "NULL device pointer");
  (void)hipGetLastError();
  kd::launch_copy_draft(c->stream, B, tokens, stride, lens, corpus_len > 0 ? corpus : nullptr,
                        corpus_len, K, c->w.copy_keys, out_ids, out_info);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(c, e, "kd_copy_draft launch");
  return KD_OK;
}

// The per-stream match keys of kd_copy_draft_noalloc (two per stream): one
// fixed array on every GPU the library runs on. Host code never uses this
// name as an address; it uses the device address looked up per device below.
static __device__ __align__(256) unsigned long long scratch[2 * KD_COPY_NOALLOC_MAX_STREAMS];

static constexpr int KD_SCRATCH_DEVICES = 64;
static std::mutex g_scratch_mu;
static unsigned long long* g_scratch_ptr[KD_SCRATCH_DEVICES] = {};   // address of `scratch` per device

// The device address of `scratch` on the current device, looked up on the
// first call there (with that device current).
static kd_status scratch_on_current_device(unsigned long long** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KD_ERR_HIP;
  if (dev < 0 || dev >= KD_SCRATCH_DEVICES) return KD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KD_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<unsigned long long*>(p);
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}

kd_status kd_copy_draft_noalloc(void* stream, int B, const int32_t* tokens, long long stride,
                                const int32_t* lens, const int32_t* corpus, long long corpus_len, int K,
                                int32_t* out_ids, int32_t* out_info) {
  if (B < 1 || B > KD_COPY_NOALLOC_MAX_STREAMS) return KD_ERR_ARG;
  if (K < 1 || K > KD_MAX_COPY) return KD_ERR_ARG;
  if (stride < 0 || stride >= (1ll << 31) || corpus_len < 0 || corpus_len >= (1ll << 31)) return KD_ERR_ARG;
  if ((stride > 0 && !tokens) || !lens || !out_ids || !out_info || (corpus_len > 0 && !corpus))
    return KD_ERR_ARG;
  unsigned long long* keys = nullptr;
  const kd_status s = scratch_on_current_device(&keys);
  if (s != KD_OK) return s;
  (void)hipGetLastError();
  kd::launch_copy_draft(static_cast<hipStream_t>(stream), B, tokens, stride, lens,
                        corpus_len > 0 ? corpus : nullptr, corpus_len, K, keys, out_ids, out_info);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

void kd_copy_guard_init(kd_copy_guard* g, int window, float min_accept, int pause) {
  if (!g) return;
  memset(g, 0, sizeof *g);
  g->window = window < 1 ? 1 : (window > KD_GUARD_MAX_WINDOW ? KD_GUARD_MAX_WINDOW : window);
  g->min_accept = min_accept;
  g->pause = pause < 0 ? 0 : pause;
}

int kd_copy_guard_armed(const kd_copy_guard* g) { return g && g->paused_left == 0 ? 1 : 0; }

void kd_copy_guard_record(kd_copy_guard* g, int proposed, int accepted) {
  if (!g) return;
  g->proposed[g->next] = proposed;
  g->accepted[g->next] = accepted;
  g->next = (g->next + 1) % g->window;
  if (g->count < g->window) ++g->count;
  if (g->count == g->window) {
    long long p = 0, a = 0;
    for (int i = 0; i < g->window; ++i) {
      p += g->proposed[i];
      a += g->accepted[i];
    }
    if (p > 0 && (double)a < (double)g->min_accept * (double)p) {
      g->paused_left = g->pause;
      g->count = 0;
      g->next = 0;
    }
  }
}

void kd_copy_guard_advance(kd_copy_guard* g, int tokens) {
  if (!g || tokens <= 0) return;
  g->paused_left = g->paused_left > tokens ? g->paused_left - tokens : 0;
}

// ---- debug / probes ----

kd_status kd_probe_decode_e4m3(uint16_t* out) {
  if (!out) return KD_ERR_ARG;
  kd::launch_probe_e4m3(nullptr, out);
  return hipDeviceSynchronize() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

kd_status kd_probe_decode_e4m3_f16(uint16_t* out) {
  if (!out) return KD_ERR_ARG;
  kd::launch_probe_e4m3_f16(nullptr, out);
  return hipDeviceSynchronize() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

kd_status kd_probe_decode_nvfp4(uint16_t* out) {
  if (!out) return KD_ERR_ARG;
  kd::launch_probe_nvfp4(nullptr, out);
  return hipDeviceSynchronize() == hipSuccess ? KD_OK : KD_ERR_HIP;
}

kd_status kd_debug_set_layers(kd_ctx* c, int n) {
  if (!c) return KD_ERR_ARG;
  if (n > kd::NL) return fail(c, KD_ERR_ARG, "more layers than the model has");
  c->debug_layers = n < 0 ? -1 : n;
  return KD_OK;
}

kd_status kd_debug_buffers(kd_ctx* c, const float** hidden, const float** fused) {
  if (!c || !hidden || !fused) return KD_ERR_ARG;
  if (c->last_path >= 2) {
    const int nl = c->debug_layers < 0 ? kd::NL : c->debug_layers;
    *hidden = c->small.x[nl == 0 ? 0 : kd::xs_d(nl - 1)];
    *fused = c->small.f;
  } else {
    *hidden = c->w.x;
    *fused = c->w.f;
  }
  return KD_OK;
}

kd_status kd_debug_set_path(kd_ctx* c, int path) {
  if (!c) return KD_ERR_ARG;
  if (path < 0 || path > 3) return fail(c, KD_ERR_ARG, "path must be 0..3");
  if (path >= 2 && !c->small_ok)
    return fail(c, KD_ERR_UNSUPPORTED, "the window is too long for the small-batch path");
  if (path == 3 && !c->mega_ok) return fail(c, KD_ERR_UNSUPPORTED, "no cooperative launch");
  c->path = path;
  return KD_OK;
}

kd_status kd_debug_set_fused(kd_ctx* c, int on) {
  if (!c) return KD_ERR_ARG;
  c->fused_proj = on ? 1 : 0;
  return KD_OK;
}

int kd_debug_last_path(const kd_ctx* c) { return c ? c->last_path : 0; }

kd_status kd_debug_set_trace(kd_ctx* c, unsigned long long* buf, int phases, int* workgroups) {
  if (!c) return KD_ERR_ARG;
  if (buf && phases < 1) return fail(c, KD_ERR_ARG, "trace needs at least one phase row");
  c->trace = buf;
  c->trace_phases = buf ? phases : 0;
  if (workgroups) *workgroups = c->G;
  return KD_OK;
}

}  // extern "C"
