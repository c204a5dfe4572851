// Host side of the Blockwise Parallel Transformer layer: descriptor
// validation, workspace planning and the launch sequence of the forward and
// the recompute-based backward on the caller's stream.
//
// Forward per sequence ("Blockwise Parallel Transformer for Long Context Large
// Models", §3.2 and Algorithm 1; head chunks from "Untied Ulysses", §3.2):
//   xn = Norm1(x)
//   for each head chunk: Q, K, V of the chunk's heads (bias, RoPE) -> blockwise
//                        attention -> O[:, chunk heads] and the per-row LSE
//   h1 = x + O W_o + b_o                    (whole sequence, fp32 workspace)
//   for each group of whole query blocks (at most min(8192, s/2) rows):
//       z  = Norm2(h1_g); u = act(z W_1 + b_1)  (group x ffn_dim scratch only)
//       y_g = h1_g + u W_2 + b_2
// Backward per sequence: recompute h1; per group of query blocks recompute z,
// the FFN pre-activation and u, then the FFN and Norm2 backward and the FFN
// weight gradients; the O-projection backward over the whole sequence; then
// per head chunk recompute Q, K, V and run the attention backward, the QKV
// weight gradient and dxn; finally Norm1's backward plus the residual.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/bpt.h"
#include "attention.hpp"
#include "attention_dma.hpp"
#include "gemm_dma.hpp"
#include "peak.hpp"
#include "gemm.hpp"
#include "lm_head.hpp"
#include "rowwise.hpp"

using namespace bpt;

namespace {

thread_local std::string g_last_error;

bpt_status fail(bpt_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

#define BPT_TRY(expr)                                  \
  do {                                                 \
    bpt_status _st = (expr);                           \
    if (_st != BPT_OK) return _st;                     \
  } while (0)

// ---- Optional instrumentation, switched by environment variables read once:
// BPT_ROCTX=1 brackets every phase (layer forward / backward, head chunk, FFN
// group, stack layer, LM-head chunk) with a roctx range, which `rocprofv3
// --marker-trace` records next to the kernels; BPT_LOG=1 prints each call's
// plan (shape, chunks, groups, buffer sizes) to stderr. Both are off by
// default and cost one branch per phase then.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}
bool markers_on() {
  static const bool on = env_on("BPT_ROCTX");
  return on;
}
bool log_on() {
  static const bool on = env_on("BPT_LOG");
  return on;
}

struct Range {
  bool on;
  explicit Range(const char* fmt, ...) : on(markers_on()) {
    if (!on) return;
    char buf[128];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    roctxRangePush(buf);
  }
  ~Range() {
    if (on) roctxRangePop();
  }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

void log_line(const char* fmt, ...) {
  if (!log_on()) return;
  va_list ap;
  va_start(ap, fmt);
  std::fputs("[bpt] ", stderr);
  std::vfprintf(stderr, fmt, ap);
  std::fputc('\n', stderr);
  va_end(ap);
}

bpt_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(BPT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return BPT_OK;
}

// ----------------------------------------------------------------- timing
// Optional event timing of kernel classes (see bpt_timing_enable).
struct TimingState {
  std::mutex mu;
  uint32_t mask = 0;
  struct Rec { int cls; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double ms[BPT_KERNEL_CLASSES] = {};
  int64_t n[BPT_KERNEL_CLASSES] = {};
};
TimingState& timing() {
  static TimingState t;
  return t;
}

struct TimedLaunch {
  int cls; hipStream_t st; hipEvent_t a = nullptr, b = nullptr;
  TimedLaunch(int c, hipStream_t s) : cls(c), st(s) {
    TimingState& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!(t.mask & (1u << c))) return;
    for (hipEvent_t* e : {&a, &b}) {
      if (!t.pool.empty()) { *e = t.pool.back(); t.pool.pop_back(); }
      else if (hipEventCreate(e) != hipSuccess) *e = nullptr;
    }
    if (a && b) hipEventRecord(a, st);
  }
  ~TimedLaunch() {
    if (!a || !b) return;
    hipEventRecord(b, st);
    TimingState& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    t.pending.push_back({cls, a, b});
  }
};

constexpr int kColsumParts = 64;   // row splits of the bias-gradient column sums
constexpr int kNormWaves = 2048;   // waves of the norm backward (partial rows)
// Norm2 and the FFN (forward, and in the backward their recompute and
// gradients) run over groups of whole consecutive query blocks of at most
// kFfnGroupRows rows and at most half the sequence (a single block of more
// rows runs alone): GEMMs taller than one block, fewer launches, and one
// read-modify-write of the fp32 dW_1 / dW_2 per group. The FFN scratch is one
// group's rows x ffn_dim, never s x ffn_dim.
constexpr int64_t kFfnGroupRows = 8192;
constexpr int64_t kMaxHidden = 16384;  // widest row the norm kernels take
constexpr int kDkvMaxParts = 4;  // query-head split of the dK/dV pass (see attn_bwd)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ----------------------------------------------------------------- plan
struct Plan {
  int dtype, norm, ffn, causal, rope, window;
  int drop_thr;        // attention dropout threshold (0: none)
  float drop_scale;
  uint64_t seed;
  int64_t b, s, h, H, Hkv, D, f, cq, ckv, U, G, nkvc, qkv_cols, chunk_cols;
  int64_t gq;  // query blocks per weight-gradient group (backward)
  double rope_base;
  float eps;
  size_t esz;  // storage element size
};

bpt_status make_plan(const bpt_layer_desc* d, Plan& p) {
  if (!d) return fail(BPT_EINVAL, "desc is NULL");
  if (d->abi_version != BPT_ABI_VERSION) return fail(BPT_EINVAL, "abi_version mismatch");
  if (d->dtype != BPT_F32 && d->dtype != BPT_BF16) return fail(BPT_EINVAL, "dtype");
  if (d->norm != BPT_LAYERNORM && d->norm != BPT_RMSNORM) return fail(BPT_EINVAL, "norm");
  if (d->ffn != BPT_RELU && d->ffn != BPT_GELU_ERF && d->ffn != BPT_SWIGLU)
    return fail(BPT_EINVAL, "ffn");
  if (d->causal != 0 && d->causal != 1) return fail(BPT_EINVAL, "causal must be 0 or 1");
  if (d->use_rope != 0 && d->use_rope != 1) return fail(BPT_EINVAL, "use_rope must be 0 or 1");
  if (d->batch < 1 || d->batch > (1 << 20)) return fail(BPT_EINVAL, "batch");
  if (d->seq_len < 16 || d->seq_len % 16 != 0 || d->seq_len > (1 << 24))
    return fail(BPT_EINVAL, "seq_len must be a positive multiple of 16 (<= 2^24)");
  if (d->n_heads < 1 || d->n_heads > kMaxHidden || d->n_kv_heads < 1 ||
      d->n_heads % d->n_kv_heads != 0)
    return fail(BPT_EINVAL, "n_kv_heads must divide n_heads (n_heads <= 16384)");
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
    return fail(BPT_EUNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (d->dtype == BPT_F32 && d->head_dim > 64)
    return fail(BPT_EUNSUPPORTED, "fp32 mode supports head_dim 32 or 64");
  if (d->hidden != d->n_heads * d->head_dim)
    return fail(BPT_EINVAL, "hidden must equal n_heads * head_dim");
  if (d->hidden % 64 != 0) return fail(BPT_EINVAL, "hidden must be a multiple of 64");
  if (d->hidden > kMaxHidden) return fail(BPT_EUNSUPPORTED, "hidden above 16384");
  if (d->ffn_dim < 64 || d->ffn_dim % 64 != 0 || d->ffn_dim > (1 << 20))
    return fail(BPT_EINVAL, "ffn_dim must be a positive multiple of 64");
  if (d->q_block < 8 || d->q_block % 8 != 0 || d->seq_len % d->q_block != 0)
    return fail(BPT_EINVAL, "q_block must be a multiple of 8 dividing seq_len");
  if (d->kv_block < 1 || d->seq_len % d->kv_block != 0)
    return fail(BPT_EINVAL, "kv_block must divide seq_len");
  const int64_t G = d->n_heads / d->n_kv_heads;
  if (d->head_chunk < 1 || d->n_heads % d->head_chunk != 0 || d->head_chunk % G != 0)
    return fail(BPT_EINVAL, "head_chunk must divide n_heads and be a multiple of the GQA group");
  if (d->use_rope && !(d->rope_base > 1.0 && std::isfinite(d->rope_base)))
    return fail(BPT_EINVAL, "rope_base");
  if (!(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps)) return fail(BPT_EINVAL, "norm_eps");
  if (d->window < 0) return fail(BPT_EINVAL, "window must be >= 0");
  if (!(d->dropout_p >= 0.f && d->dropout_p < 1.f))
    return fail(BPT_EINVAL, "dropout_p must be in [0, 1)");
  const int drop_thr = (int)std::lround(256.0 * (double)d->dropout_p);
  if (drop_thr > 255) return fail(BPT_EINVAL, "dropout_p rounds to a threshold of 256");
  if (d->window > 0 && !d->causal) return fail(BPT_EINVAL, "a sliding window requires causal = 1");
  const int64_t qkv_cols = (d->n_heads + 2 * d->n_kv_heads) * d->head_dim;
  if (d->seq_len * std::max<int64_t>(std::max(d->hidden, qkv_cols), d->ffn_dim) >= (int64_t(1) << 40))
    return fail(BPT_EUNSUPPORTED, "problem too large");
  p.dtype = d->dtype; p.norm = d->norm; p.ffn = d->ffn; p.causal = d->causal; p.rope = d->use_rope;
  p.window = d->window;
  p.drop_thr = drop_thr;
  p.drop_scale = drop_thr ? (float)(256.0 / (256.0 - drop_thr)) : 1.f;
  p.seed = d->seed;
  p.b = d->batch; p.s = d->seq_len; p.h = d->hidden; p.H = d->n_heads; p.Hkv = d->n_kv_heads;
  p.D = d->head_dim; p.f = d->ffn_dim; p.cq = d->q_block; p.ckv = d->kv_block;
  p.U = d->head_chunk; p.G = G; p.nkvc = p.U / G; p.qkv_cols = qkv_cols;
  p.chunk_cols = (p.U + 2 * p.nkvc) * p.D;
  p.gq = std::max<int64_t>(1, std::min<int64_t>(p.s / p.cq / 2, kFfnGroupRows / p.cq));
  p.rope_base = d->rope_base; p.eps = d->norm_eps;
  p.esz = d->dtype == BPT_BF16 ? 2 : 4;
  return BPT_OK;
}

// Largest query-head split of the dK/dV pass that the workspace provides for:
// a power of two dividing G, at most kDkvMaxParts, for bf16 with head_dim 64
// or 128 and fewer than 8 KV heads per chunk (more give enough workgroups).
void log_plan(const char* what, const Plan& p, size_t ws_bytes) {
  log_line("%s: b=%lld s=%lld h=%lld heads=%lld/%lld d=%lld ffn=%lld %s, head chunk %lld "
           "(%lld chunks), FFN groups of %lld rows, causal=%d window=%d dropout_thr=%d, "
           "workspace %zu bytes", what, (long long)p.b, (long long)p.s, (long long)p.h,
           (long long)p.H, (long long)p.Hkv, (long long)p.D, (long long)p.f,
           p.dtype == BPT_BF16 ? "bf16" : "fp32", (long long)p.U, (long long)(p.H / p.U),
           (long long)(p.gq * p.cq), p.causal, p.window, p.drop_thr, ws_bytes);
}

int dkv_parts_max(const Plan& p) {
  if (p.dtype != BPT_BF16 || (p.D != 64 && p.D != 128) || p.nkvc >= 8) return 1;
  int m = 1;
  while (m < kDkvMaxParts && p.G % (2 * m) == 0) m *= 2;
  return m;
}

// Workspace carve-up: a running offset over 256-byte aligned regions.
struct Carver {
  char* base; size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename X> X* take(size_t count) {
    X* r = base ? (X*)(base + off) : nullptr;
    off = align_up(off + count * sizeof(X), 256);
    return r;
  }
};

template <typename T>
struct FwdWs {
  T *xn, *q, *k, *v, *z, *u, *gate, *wc, *bc;
  float* h1;
  float2* rope;
};

template <typename T>
FwdWs<T> carve_fwd(Carver& c, const Plan& p) {
  FwdWs<T> w{};
  w.xn = c.take<T>(p.s * p.h);
  w.rope = p.rope ? c.take<float2>(p.s * (p.D / 2)) : nullptr;
  w.q = c.take<T>(p.U * p.s * p.D);
  w.k = c.take<T>(p.nkvc * p.s * p.D);
  w.v = c.take<T>(p.nkvc * p.s * p.D);
  if (p.U < p.H) {  // a head chunk's Q|K|V weight columns (and biases), gathered
    w.wc = c.take<T>(p.h * p.chunk_cols);
    w.bc = c.take<T>(p.chunk_cols);
  }
  // FFN scratch for a group of gq query blocks, with the group's
  // h1 = x + O W_o + b_o (fp32).
  const int64_t grp = p.gq * p.cq;
  w.h1 = c.take<float>(grp * p.h);
  w.z = c.take<T>(grp * p.h);
  w.u = c.take<T>(grp * p.f);
  w.gate = p.ffn == BPT_SWIGLU ? c.take<T>(grp * p.f) : nullptr;
  return w;
}

template <typename T>
struct BwdWs {
  T *xn, *q, *k, *v, *dO, *dqkv, *z, *a, *u, *up, *da, *dup, *dh_t, *wc, *bc;
  float *dvec, *dh, *dxn, *h1, *dz, *part, *npart_g, *npart_b, *kbuf, *dkv_part;
  int64_t kbuf_floats;
  float2* rope;
};

template <typename T>
BwdWs<T> carve_bwd(Carver& c, const Plan& p) {
  BwdWs<T> w{};
  const int64_t HD = p.H * p.D;
  w.xn = c.take<T>(p.s * p.h);
  w.rope = p.rope ? c.take<float2>(p.s * (p.D / 2)) : nullptr;
  w.dO = c.take<T>(p.s * HD);
  w.dvec = c.take<float>(p.H * p.s);
  w.dh = c.take<float>(p.s * p.h);
  w.dxn = c.take<float>(p.s * p.h);
  w.q = c.take<T>(p.U * p.s * p.D);
  w.k = c.take<T>(p.nkvc * p.s * p.D);
  w.v = c.take<T>(p.nkvc * p.s * p.D);
  w.dqkv = c.take<T>(p.s * p.chunk_cols);
  if (p.U < p.H) {
    w.wc = c.take<T>(p.h * p.chunk_cols);
    w.bc = c.take<T>(p.chunk_cols);
  }
  // FFN activations and gradients for a group of gq query blocks, with the
  // group's recomputed h1 = x + O W_o + b_o (fp32).
  const int64_t grp = p.gq * p.cq;
  w.h1 = c.take<float>(grp * p.h);
  w.z = c.take<T>(grp * p.h);
  w.a = c.take<T>(grp * p.f);
  w.u = c.take<T>(grp * p.f);
  w.up = p.ffn == BPT_SWIGLU ? c.take<T>(grp * p.f) : nullptr;
  w.da = c.take<T>(grp * p.f);
  w.dup = p.ffn == BPT_SWIGLU ? c.take<T>(grp * p.f) : nullptr;
  w.dz = c.take<float>(grp * p.h);
  w.dh_t = c.take<T>(p.s * p.h);  // dh in the storage type, whole sequence
  const int64_t maxn = std::max<int64_t>(std::max(p.h, p.f), std::max(p.chunk_cols, HD));
  w.part = c.take<float>(kColsumParts * maxn);
  w.npart_g = c.take<float>(kNormWaves * p.h);
  w.npart_b = c.take<float>(kNormWaves * p.h);
  // Split-K partial sums of the weight-gradient GEMMs whose outputs have few
  // tiles (bf16 path): s h / 4 floats, one byte per token and hidden unit.
  w.kbuf_floats = p.dtype == BPT_BF16 ? p.s * p.h / 4 : 0;
  w.kbuf = w.kbuf_floats ? c.take<float>(w.kbuf_floats) : nullptr;
  // Partial dK/dV sums of the query-head split (bf16, GQA with fewer than 8
  // KV heads per chunk): parts x 2 x (KV heads of a chunk) x s x d fp32.
  const int parts = dkv_parts_max(p);
  w.dkv_part = parts > 1 ? c.take<float>((int64_t)parts * 2 * p.nkvc * p.s * p.D) : nullptr;
  return w;
}

size_t fwd_ws_bytes(const Plan& p) {
  Carver c(nullptr);
  if (p.dtype == BPT_BF16) carve_fwd<bf16>(c, p); else carve_fwd<float>(c, p);
  return c.off;
}
size_t bwd_ws_bytes(const Plan& p) {
  Carver c(nullptr);
  if (p.dtype == BPT_BF16) carve_bwd<bf16>(c, p); else carve_bwd<float>(c, p);
  return c.off;
}
size_t saved_bytes(const Plan& p) {
  return align_up((size_t)(p.b * p.s * p.H * p.D) * p.esz, 256) + (size_t)(p.b * p.H * p.s) * 4;
}

// ----------------------------------------------------------------- launchers
template <typename T, bool AK, bool BK, int BM, int BN, int BKK, int WM, int WN, class Epi>
void launch_gemm(hipStream_t st, const T* A, int64_t lda, const T* B, int64_t ldb, int64_t M,
                 int64_t N, int64_t K, const Epi& epi, bool even) {
  const int64_t nt = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (even)
    hipLaunchKernelGGL((gemm_kernel<T, AK, BK, BM, BN, BKK, WM, WN, true, Epi>), dim3((unsigned)nt),
                       dim3(256), 0, st, A, lda, B, ldb, (int)M, (int)N, (int)K, epi);
  else
    hipLaunchKernelGGL((gemm_kernel<T, AK, BK, BM, BN, BKK, WM, WN, false, Epi>), dim3((unsigned)nt),
                       dim3(256), 0, st, A, lda, B, ldb, (int)M, (int)N, (int)K, epi);
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <bool AK, bool BK, int BM, int BN, int BKK, int ST, int WM, int WN, int NW, class Epi>
bpt_status launch_gemm_dma(hipStream_t st, const bf16* A, int64_t lda, const bf16* B, int64_t ldb,
                           int64_t M, int64_t N, int64_t K, const Epi& epi, int ksplit = 1) {
  constexpr int kLds = ST * (BM + BN) * BKK * 2;
  auto kern = gemm_dma_kernel<AK, BK, BM, BN, BKK, ST, WM, WN, NW, Epi>;
  // The dynamic-LDS limit is raised once per instantiation and device (a bit
  // per device in `raised`, set only once the call succeeded; setting it
  // twice from racing threads is harmless).
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  const uint64_t bit = known ? 1ull << dev : 0;
  if (!known || !(raised.load(std::memory_order_acquire) & bit)) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess)
      return fail(BPT_EHIP, std::string("raising the GEMM's dynamic LDS limit: ") +
                                hipGetErrorString(e));
    if (known) raised.fetch_or(bit, std::memory_order_release);
  }
  const int64_t nt = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)(nt * ksplit)), dim3(64 * NW), kLds, st, A, lda, B, ldb,
                     (int)M, (int)N, (int)K, ksplit, epi);
  return BPT_OK;
}

// kbuf (kbuf_floats fp32 elements of workspace), when given, lets a weight
// gradient with too few output tiles to fill the GPU run split-K: ksplit
// copies of the tile grid each sum a share of the reduction steps into kbuf,
// and a second kernel applies the epilogue to their sum (in a fixed order).
// Long reductions (K >= 16384, the sequence) use 256 x 256 tiles and shares
// of at least 2048; smaller outputs (fewer 256 x 256 tiles than CUs, e.g. the
// per-group FFN weight gradients of a narrow layer) 128 x 128 tiles and
// shares of at least two steps.
template <typename T, bool AK, bool BK, class Epi>
bpt_status gemm(hipStream_t st, const T* A, int64_t lda, const T* B, int64_t ldb, int64_t M,
                int64_t N, int64_t K, const Epi& epi, const char* what, float* kbuf = nullptr,
                int64_t kbuf_floats = 0, int cls = BPT_KERNEL_GEMM) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int BKK = sizeof(T) == 2 ? 64 : 32;
  // Layout invariants of the tile loaders (16-byte vectors along the
  // contiguous axis, every vector fully inside or outside the matrix).
  bool ok = M >= 0 && N >= 0 && K >= 0 && M < (1LL << 31) && N < (1LL << 31) && K < (1LL << 31);
  ok = ok && (AK ? (K % VEC == 0 && lda >= K) : (M % VEC == 0 && lda >= M));
  ok = ok && (BK ? (K % VEC == 0 && ldb >= K) : (N % VEC == 0 && ldb >= N));
  ok = ok && ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) && (lda % VEC == 0) &&
       (ldb % VEC == 0);
  if (!ok) return fail(BPT_EUNSUPPORTED, std::string("gemm layout invariant: ") + what);
  if (M == 0 || N == 0) return BPT_OK;
  TimedLaunch tl(cls, st);
  if constexpr (sizeof(T) == 2) {
    if (K % 64 == 0) {
      // Direct-to-LDS pipelines, 8 waves per workgroup. Shapes with at least
      // one 256 x 256 tile per CU use that tile (half the L2 -> LDS traffic
      // per flop of a 128 x 128 tile); smaller outputs use 128 x 128 tiles
      // (waves of 32 x 64) to keep every CU busy.
      const int64_t nt256 = ((M + 255) / 256) * ((N + 255) / 256);
      if constexpr (!AK && !BK && !Epi::kPair) {
        if (kbuf && K >= 16384) {
          int ks = 1;
          while (nt256 * ks < 2 * device_cus() && ks < 64) ks *= 2;
          while (ks > 1 && (ks * M * N > kbuf_floats || K % (ks * 64) != 0 || K / ks < 2048))
            ks /= 2;
          if (ks > 1) {
            EpiPart ep{kbuf, N, M * N};
            BPT_TRY((launch_gemm_dma<AK, BK, 256, 256, 64, 2, 128, 64, 8>(st, A, lda, B, ldb, M, N,
                                                                          K, ep, ks)));
            hipLaunchKernelGGL(splitk_reduce_kernel<Epi>, dim3((unsigned)((M * N + 255) / 256)),
                               dim3(256), 0, st, kbuf, ks, (int)M, (int)N, epi);
            return check_launch(what);
          }
        } else if (kbuf && K >= 1024 && nt256 < device_cus()) {
          const int64_t nt128 = ((M + 127) / 128) * ((N + 127) / 128), nkt = K / 64;
          int ks = 1;
          while (nt128 * ks < 2 * device_cus() && ks < 64 && nkt / (2 * ks) >= 2) ks *= 2;
          while (ks > 1 && ks * M * N > kbuf_floats) ks /= 2;
          if (ks > 1) {
            EpiPart ep{kbuf, N, M * N};
            BPT_TRY((launch_gemm_dma<AK, BK, 128, 128, 64, 2, 32, 64, 8>(st, A, lda, B, ldb, M, N,
                                                                        K, ep, ks)));
            hipLaunchKernelGGL(splitk_reduce_kernel<Epi>, dim3((unsigned)((M * N + 255) / 256)),
                               dim3(256), 0, st, kbuf, ks, (int)M, (int)N, epi);
            return check_launch(what);
          }
        }
      }
      if (nt256 >= device_cus()) {
        // Waves of 128 x 64 when B is N-major (half as many of its transpose
        // reads per MFMA as 64 x 128 waves; 3-20 % faster on such shapes),
        // 64 x 128 when both operands are K-major.
        if constexpr (BK)
          BPT_TRY((launch_gemm_dma<AK, BK, 256, 256, 64, 2, 64, 128, 8>(st, A, lda, B, ldb, M, N, K,
                                                                        epi)));
        else
          BPT_TRY((launch_gemm_dma<AK, BK, 256, 256, 64, 2, 128, 64, 8>(st, A, lda, B, ldb, M, N, K,
                                                                        epi)));
      } else if (K >= 32768) {
        // long reductions (weight gradients over the sequence): three stages
        BPT_TRY((launch_gemm_dma<AK, BK, 128, 128, 64, 3, 64, 32, 8>(st, A, lda, B, ldb, M, N, K,
                                                                     epi)));
      } else {
        BPT_TRY((launch_gemm_dma<AK, BK, 128, 128, 64, 2, 32, 64, 8>(st, A, lda, B, ldb, M, N, K,
                                                                     epi)));
      }
      return check_launch(what);
    }
  }
  // Register-staged path (fp32, and bf16 with K not a multiple of 64):
  // 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per CU.
  const bool even = M % 128 == 0 && N % 128 == 0 && K % BKK == 0;
  launch_gemm<T, AK, BK, 128, 128, BKK, 64, 64>(st, A, lda, B, ldb, M, N, K, epi, even);
  return check_launch(what);
}

template <typename T, typename Tin, typename Tout>
bpt_status norm_fwd(hipStream_t st, const Plan& p, const Tin* x, int64_t ldx, const T* g,
                    const T* bta, Tout* out, int64_t ldo, int64_t rows) {
  const int nch = (int)((p.h / 8 + 63) / 64);
  const dim3 grid((unsigned)((rows + 3) / 4)), blk(256);
  const int kind = p.norm == BPT_LAYERNORM ? NORM_LAYER : NORM_RMS;
  if (rows == 0) return BPT_OK;
  TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
#define NF(NC) hipLaunchKernelGGL((norm_fwd_kernel<T, Tin, Tout, NC>), grid, blk, 0, st, x, ldx, g, \
                                  bta, out, ldo, (int)rows, (int)p.h, kind, p.eps)
  if (nch <= 1) NF(1); else if (nch <= 2) NF(2); else if (nch <= 4) NF(4);
  else if (nch <= 8) NF(8); else if (nch <= 16) NF(16); else if (nch <= 32) NF(32);
  else return fail(BPT_EUNSUPPORTED, "hidden too large for norm kernel");
#undef NF
  return check_launch("norm_fwd");
}

// Norm backward over `rows` rows. The gain / shift gradients go to per-wave
// partial rows (part_g / part_b, kNormWaves x h): with `stage` == 0 they are
// written, 1 accumulated (several calls over row blocks), and with `finish`
// reduced into dg / db (+=).
template <typename T, typename Tin, typename Tres>
bpt_status norm_bwd(hipStream_t st, const Plan& p, const float* dz, int64_t lddz, const Tin* xin,
                    int64_t ldx, const T* g, const Tres* res, int64_t ldr, float* out_f, T* out_t,
                    int64_t ldo, int64_t rows, float* dg, float* db, float* part_g, float* part_b,
                    int stage, bool finish, int* nparts) {
  if (rows == 0) return BPT_OK;
  const int kind = p.norm == BPT_LAYERNORM ? NORM_LAYER : NORM_RMS;
  // Rows of up to 2048 elements: one wave per row; wider rows: the four waves
  // of a workgroup share a row (a lane then holds at most 32 elements of each
  // per-row array).
  const bool wide = p.h > 2048;
  const int nch = wide ? (int)((p.h / 8 + 255) / 256) : (int)((p.h / 8 + 63) / 64);
  const int nblk = wide ? (int)std::min<int64_t>(kNormWaves / 4, rows)
                        : (int)std::min<int64_t>(kNormWaves / 4, (rows + 3) / 4);
  float* pg = dg ? part_g : nullptr;
  float* pb = db ? part_b : nullptr;
  const dim3 grid(nblk), blk(256);
  TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
#define NB(NC, W) hipLaunchKernelGGL((norm_bwd_kernel<T, Tin, Tres, NC, W>), grid, blk, 0, st, dz, lddz, \
                                     xin, ldx, g, res, ldr, out_f, out_t, ldo, pg, pb, (int)rows,     \
                                     (int)p.h, kind, p.eps, stage)
  if (!wide) {
    if (nch <= 1) NB(1, 1); else if (nch <= 2) NB(2, 1); else NB(4, 1);
  } else {
    if (nch <= 2) NB(2, 4); else if (nch <= 4) NB(4, 4); else if (nch <= 8) NB(8, 4);
    else return fail(BPT_EUNSUPPORTED, "hidden too large for norm kernel");
  }
#undef NB
  BPT_TRY(check_launch("norm_bwd"));
  // The first call of a series writes the most partial rows (it has the most
  // rows); later calls accumulate into a prefix of them.
  if (stage == 0) *nparts = wide ? nblk : nblk * 4;
  if (!finish) return BPT_OK;
  const int P = *nparts;
  const dim3 g2((unsigned)((p.h + 63) / 64));
  const dim3 bf(64 * kColsumFinalLanes);
  if (dg) hipLaunchKernelGGL(colsum_final_kernel, g2, bf, 0, st, pg, P, (int)p.h, dg, 1);
  if (db) hipLaunchKernelGGL(colsum_final_kernel, g2, bf, 0, st, pb, P, (int)p.h, db, 1);
  return check_launch("norm_bwd reduce");
}

// out[col] += sum over rows of X[:, col]. A series of calls over row blocks
// can share the partial rows: `stage` 0 writes them, 1 accumulates; `finish`
// reduces them into out. The first call of a series must have the most rows.
template <typename Tin>
bpt_status colsum(hipStream_t st, const Tin* X, int64_t ldx, int64_t rows, int64_t N, float* part,
                  float* out, int stage = 0, bool finish = true, int* nparts = nullptr) {
  if (!out || N == 0) return BPT_OK;
  int P = (int)std::min<int64_t>(kColsumParts, rows);
  TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
  constexpr int V = 16 / (int)sizeof(Tin);
  const bool vec = (uintptr_t)X % 16 == 0 && N % V == 0 && ldx % V == 0;
  if (rows > 0 && vec)
    hipLaunchKernelGGL(colsum_partial_vec_kernel<Tin>, dim3((unsigned)((N + 64 * V - 1) / (64 * V)), P),
                       dim3(256), 0, st, X, ldx, (int)rows, (int)N, part, stage);
  else if (rows > 0)
    hipLaunchKernelGGL(colsum_partial_kernel<Tin>, dim3((unsigned)((N + 63) / 64), P), dim3(256), 0,
                       st, X, ldx, (int)rows, (int)N, part, stage);
  if (nparts) {
    if (stage == 0) *nparts = P;
    P = *nparts;
  }
  if (finish && P > 0)
    hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((N + 63) / 64)),
                       dim3(64 * kColsumFinalLanes), 0, st, part, P, (int)N, out, 1);
  return check_launch("colsum");
}

bpt_status fill(hipStream_t st, float* ptr, int64_t n, float v) {
  if (!ptr || n == 0) return BPT_OK;
  TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ptr, n, v);
  return check_launch("fill");
}

bpt_status rope_table(hipStream_t st, const Plan& p, float2* tab) {
  if (!p.rope) return BPT_OK;
  const int64_t n = p.s * (p.D / 2);
  TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab,
                     (int)p.s, (int)p.D, p.rope_base);
  return check_launch("rope_table");
}

// Calls f(window flag, dropout flag) with compile-time booleans matching the
// plan: the sliding-window and dropout code exists only in the variants that
// use it.
template <class F>
void with_variants(const Plan& p, F&& f) {
  if (p.window) {
    if (p.drop_thr) f(std::true_type(), std::true_type()); else f(std::true_type(), std::false_type());
  } else {
    if (p.drop_thr) f(std::false_type(), std::true_type()); else f(std::false_type(), std::false_type());
  }
}

DropArgs drop_args(const Plan& p, int64_t head0, int64_t batch) {
  DropArgs d;
  d.seed_lo = (uint32_t)(p.seed & 0xFFFFFFFFu);
  d.seed_hi = (uint32_t)(p.seed >> 32);
  d.thr = p.drop_thr;
  d.scale = p.drop_scale;
  d.head0 = (int)head0;
  d.batch = (int)batch;
  return d;
}

// The projection stores q multiplied by log2(e)/sqrt(D), the softmax's
// scale and its change to base 2 (BPT Section 3.4, Eq. 3, evaluated with
// exp2): every attention kernel then reads Q K^T directly as scores in base-2
// units, and its log-sum-exp is base 2.
inline float q_log2_scale(const Plan& p) {
  return (float)(1.4426950408889634 / std::sqrt((double)p.D));
}

template <typename T>
bpt_status attn_fwd(hipStream_t st, const Plan& p, const T* q, const T* k, const T* v, T* o,
                    float* lse, int64_t head0, int64_t batch) {
  AttnFwdArgs<T> a;
  a.drop = drop_args(p, head0, batch);
  a.q = q; a.k = k; a.v = v; a.o = o; a.ldo = p.H * p.D; a.lse = lse;
  a.s = (int)p.s; a.nh = (int)p.U; a.group = (int)p.G; a.causal = p.causal; a.window = p.window;
  const dim3 grid((unsigned)(p.U * ((p.s + 127) / 128))), blk(256);
  TimedLaunch tl(BPT_KERNEL_ATTN_FWD, st);
  // The sliding window is a compile-time variant (WIN), so the unwindowed
  // kernels carry none of its code.
  auto go = [&](auto winc, auto dropc) {
    constexpr bool W = decltype(winc)::value, R = decltype(dropc)::value;
    if constexpr (sizeof(T) == 2) {
      if (p.D == 128) { hipLaunchKernelGGL((attn_fwd_dma_kernel<128, W, R>), grid, blk, 0, st, a); return; }
      if (p.D == 64) { hipLaunchKernelGGL((attn_fwd_dma_kernel<64, W, R>), grid, blk, 0, st, a); return; }
    }
    if (p.D == 64) hipLaunchKernelGGL((attn_fwd_kernel<T, 64, W, R>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<T, 32, W, R>), grid, blk, 0, st, a);
  };
  with_variants(p, go);
  return check_launch("attn_fwd");
}

template <typename T>
bpt_status attn_bwd(hipStream_t st, const Plan& p, const T* q, const T* k, const T* v,
                    const T* dout, const float* lse, const float* dvec, T* dq, T* dk, T* dv,
                    const float2* rope, float* dkv_part, int64_t head0, int64_t batch) {
  AttnBwdArgs<T> a;
  a.drop = drop_args(p, head0, batch);
  a.part = nullptr;
  a.nparts = 1;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.lddo = p.H * p.D; a.lse = lse; a.dvec = dvec;
  a.dq = dq; a.lddq = p.chunk_cols; a.dk = dk; a.dv = dv; a.lddkv = p.chunk_cols; a.rope = rope;
  a.s = (int)p.s; a.nh = (int)p.U; a.nkv = (int)p.nkvc; a.group = (int)p.G; a.causal = p.causal;
  a.window = p.window;
  // q carries log2(e)/sqrt(D) (see q_log2_scale): dQ = dS K / sqrt(D) as
  // usual, and dK = dS^T q / sqrt(D) = ln(2) dS^T Q for the stored Q.
  a.scale = (float)(1.0 / std::sqrt((double)p.D));
  a.dk_scale = (float)0.6931471805599453;
  const dim3 gkv((unsigned)(p.nkvc * ((p.s + 127) / 128))), gq((unsigned)(p.U * ((p.s + 127) / 128)));
  const dim3 blk(256);
  if (p.D == 128 && sizeof(T) != 2)
    return fail(BPT_EUNSUPPORTED, "fp32 attention backward supports head_dim <= 64");
  // The sliding window is a compile-time variant (W) of every kernel below.
  auto dkdv_pass = [&](auto winc, auto dropc) {
    constexpr bool W = decltype(winc)::value, R = decltype(dropc)::value;
    TimedLaunch tl(BPT_KERNEL_ATTN_BWD_DKDV, st);
    bool done = false;
    if constexpr (sizeof(T) == 2) {
      // Few KV heads per chunk leave too few key-tile workgroups to balance
      // the causal work (the first key tile of a head carries the most):
      // split each KV head's query heads over up to kDkvMaxParts workgroups.
      const int64_t wgs = p.nkvc * ((p.s + 127) / 128);
      if (dkv_part)
        while (a.nparts < dkv_parts_max(p) && wgs * a.nparts < 8 * device_cus()) a.nparts *= 2;
      if (a.nparts > 1) a.part = dkv_part;
      const dim3 gsplit((unsigned)(wgs * a.nparts));
      if (a.nparts > 1) {
        if (p.D == 128) hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<128, true, W, R>), gsplit, blk, 0, st, a);
        if (p.D == 64) hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<64, true, W, R>), gsplit, blk, 0, st, a);
      } else {
        if (p.D == 128) hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<128, false, W, R>), gsplit, blk, 0, st, a);
        if (p.D == 64) hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<64, false, W, R>), gsplit, blk, 0, st, a);
      }
      done = p.D == 128 || p.D == 64;
      if (a.nparts > 1) {
        const dim3 gr((unsigned)((p.s * p.nkvc * (p.D / 2) + 255) / 256));
        if (p.D == 128) hipLaunchKernelGGL((dkdv_reduce_kernel<128>), gr, blk, 0, st, a);
        if (p.D == 64) hipLaunchKernelGGL((dkdv_reduce_kernel<64>), gr, blk, 0, st, a);
      }
    }
    if (!done) {
      if (p.D == 64) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, 64, W, R>), gkv, blk, 0, st, a);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, 32, W, R>), gkv, blk, 0, st, a);
    }
  };
  auto dq_pass = [&](auto winc, auto dropc) {
    constexpr bool W = decltype(winc)::value, R = decltype(dropc)::value;
    TimedLaunch tl(BPT_KERNEL_ATTN_BWD_DQ, st);
    bool done = false;
    if constexpr (sizeof(T) == 2) {
      if (p.D == 128) { hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<128, W, R>), gq, blk, 0, st, a); done = true; }
      if (p.D == 64) { hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<64, W, R>), gq, blk, 0, st, a); done = true; }
    }
    if (!done) {
      if (p.D == 64) hipLaunchKernelGGL((attn_bwd_dq_kernel<T, 64, W, R>), gq, blk, 0, st, a);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, 32, W, R>), gq, blk, 0, st, a);
    }
  };
  with_variants(p, dkdv_pass);
  BPT_TRY(check_launch("attn_bwd_dkdv"));
  with_variants(p, dq_pass);
  return check_launch("attn_bwd_dq");
}

// Column offsets in W_qkv of head chunk c's Q, K and V parts.
struct ChunkCols {
  int64_t off[3], width[3];
};
inline ChunkCols chunk_cols_of(const Plan& p, int64_t c) {
  const int64_t hq0 = c * p.U, hk0 = hq0 / p.G;
  return {{hq0 * p.D, (p.H + hk0) * p.D, (p.H + p.Hkv + hk0) * p.D},
          {p.U * p.D, p.nkvc * p.D, p.nkvc * p.D}};
}

// Q, K, V of head chunk c (query heads [c U, (c+1) U)) into head-major
// buffers. With several chunks, the chunk's weight columns (and biases) are
// first gathered into one contiguous [h, chunk_cols] block wc (bc), so the
// projection is a single GEMM; the backward reuses wc for dxn.
template <typename T>
bpt_status qkv_chunk(hipStream_t st, const Plan& p, const T* xn, const T* wqkv, const T* bqkv,
                     int64_t c, T* q, T* k, T* v, const float2* rope, T* wc, T* bc) {
  const int c1 = (int)(p.U * p.D), c2 = (int)((p.U + p.nkvc) * p.D);
  if (p.U == p.H) {  // all heads in one chunk: one GEMM over the packed Q|K|V columns
    EpiQKV3<T> e{q, k, v, p.s * p.D, (int)p.D, bqkv, rope, c1, c2, q_log2_scale(p)};
    BPT_TRY((gemm<T, true, false>(st, xn, p.h, wqkv, p.qkv_cols, p.s, p.qkv_cols, p.h, e,
                                  "qkv projection")));
    return BPT_OK;
  }
  const ChunkCols cc = chunk_cols_of(p, c);
  {
    constexpr int V = 16 / (int)sizeof(T);
    TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
    const int64_t nv = p.h * p.chunk_cols / V;
    // W_qkv is 16-byte aligned with rows and head columns of 16-byte
    // multiples; the bias is only element-aligned, so it is copied per element.
    hipLaunchKernelGGL((gather_cols3_kernel<T, V>), dim3((unsigned)((nv + 255) / 256)), dim3(256),
                       0, st, wqkv, p.qkv_cols, wc, (int)p.h, c1, c2, (int)p.chunk_cols,
                       cc.off[0], cc.off[1], cc.off[2]);
    if (bqkv)
      hipLaunchKernelGGL((gather_cols3_kernel<T, 1>), dim3((unsigned)((p.chunk_cols + 255) / 256)),
                         dim3(256), 0, st, bqkv, p.qkv_cols, bc, 1, c1, c2, (int)p.chunk_cols,
                         cc.off[0], cc.off[1], cc.off[2]);
    BPT_TRY(check_launch("gather qkv chunk"));
  }
  EpiQKV3<T> e{q, k, v, p.s * p.D, (int)p.D, bqkv ? bc : nullptr, rope, c1, c2,
               q_log2_scale(p)};
  BPT_TRY((gemm<T, true, false>(st, xn, p.h, wc, p.chunk_cols, p.s, p.chunk_cols, p.h, e,
                                "qkv projection (chunk)")));
  return BPT_OK;
}

// ----------------------------------------------------------------- forward
template <typename T>
bpt_status forward_impl(const Plan& p, const T* x, const bpt_layer_weights* wt, T* y, void* saved,
                        void* ws, hipStream_t st) {
  Carver c(ws);
  FwdWs<T> w = carve_fwd<T>(c, p);
  const T* wqkv = (const T*)wt->w_qkv; const T* bqkv = (const T*)wt->b_qkv;
  const T* wo = (const T*)wt->w_o; const T* bo = (const T*)wt->b_o;
  const T* w1 = (const T*)wt->w_1; const T* b1 = (const T*)wt->b_1;
  const T* w2 = (const T*)wt->w_2; const T* b2 = (const T*)wt->b_2;
  const T* w3 = (const T*)wt->w_3;
  const T* g1 = (const T*)wt->n1_g; const T* sh1 = (const T*)wt->n1_b;
  const T* g2 = (const T*)wt->n2_g; const T* sh2 = (const T*)wt->n2_b;
  const int64_t HD = p.H * p.D;
  T* O = (T*)saved;
  float* LSE = (float*)((char*)saved + align_up((size_t)(p.b * p.s * HD) * p.esz, 256));
  BPT_TRY(rope_table(st, p, w.rope));
  const int act = p.ffn == BPT_RELU ? ACT_RELU : ACT_GELU;
  Range r_all("bpt layer forward (s=%lld)", (long long)p.s);

  for (int64_t bi = 0; bi < p.b; ++bi) {
    const T* xb = x + bi * p.s * p.h;
    T* yb = y + bi * p.s * p.h;
    T* Ob = O + bi * p.s * HD;
    float* Lb = LSE + bi * p.H * p.s;
    BPT_TRY((norm_fwd<T, T, T>(st, p, xb, p.h, g1, sh1, w.xn, p.h, p.s)));
    for (int64_t ch = 0; ch < p.H / p.U; ++ch) {
      Range r_ch("forward: projection and attention, head chunk %lld", (long long)ch);
      BPT_TRY(qkv_chunk<T>(st, p, w.xn, wqkv, bqkv, ch, w.q, w.k, w.v, w.rope, w.wc, w.bc));
      BPT_TRY(attn_fwd<T>(st, p, w.q, w.k, w.v, Ob + ch * p.U * p.D, Lb + ch * p.U * p.s,
                          ch * p.U, bi));
    }
    // Output projection + residual, Norm2 and the FFN, a group of gq
    // consecutive query blocks at a time.
    const int64_t grp = p.gq * p.cq;
    for (int64_t g0 = 0; g0 < p.s; g0 += grp) {
      const int64_t rows = std::min(grp, p.s - g0);  // a multiple of c_q
      Range r_g("forward: O projection, Norm2, FFN, rows %lld-%lld", (long long)g0,
                (long long)(g0 + rows));
      const float* h1g = w.h1;
      {
        EpiResid<T, T, float> eo{w.h1, p.h, xb + g0 * p.h, p.h, bo};
        BPT_TRY((gemm<T, true, false>(st, Ob + g0 * HD, HD, wo, p.h, rows, p.h, HD, eo,
                                      "o projection")));
      }
      BPT_TRY((norm_fwd<T, float, T>(st, p, h1g, p.h, g2, sh2, w.z, p.h, rows)));
      if (p.ffn == BPT_SWIGLU) {
        EpiOut<T, T> eg{w.gate, p.f, b1, 1.f, 0};
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w1, p.f, rows, p.f, p.h, eg, "ffn gate")));
        EpiSwiUp<T> eu{w.u, nullptr, w.gate, p.f};
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w3, p.f, rows, p.f, p.h, eu, "ffn up")));
      } else {
        EpiAct<T> ea{w.u, nullptr, p.f, b1, act};
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w1, p.f, rows, p.f, p.h, ea, "ffn fc1")));
      }
      EpiResid<T, float, T> ey{yb + g0 * p.h, p.h, h1g, p.h, b2};
      BPT_TRY((gemm<T, true, false>(st, w.u, p.f, w2, p.h, rows, p.h, p.f, ey, "ffn fc2")));
    }
  }
  return BPT_OK;
}

// ----------------------------------------------------------------- backward
template <typename T>
bpt_status backward_impl(const Plan& p, const T* x, const bpt_layer_weights* wt, const void* saved,
                         const T* dy, T* dx, const bpt_layer_grads* gr, void* ws, hipStream_t st) {
  Carver c(ws);
  BwdWs<T> w = carve_bwd<T>(c, p);
  const T* wqkv = (const T*)wt->w_qkv; const T* bqkv = (const T*)wt->b_qkv;
  const T* wo = (const T*)wt->w_o; const T* bo = (const T*)wt->b_o;
  const T* w1 = (const T*)wt->w_1; const T* b1 = (const T*)wt->b_1;
  const T* w2 = (const T*)wt->w_2;
  const T* w3 = (const T*)wt->w_3;
  const T* g1 = (const T*)wt->n1_g; const T* sh1 = (const T*)wt->n1_b;
  const T* g2 = (const T*)wt->n2_g; const T* sh2 = (const T*)wt->n2_b;
  const int64_t HD = p.H * p.D;
  const T* O = (const T*)saved;
  const float* LSE =
      (const float*)((const char*)saved + align_up((size_t)(p.b * p.s * HD) * p.esz, 256));
  const bool swiglu = p.ffn == BPT_SWIGLU;
  const int act = p.ffn == BPT_RELU ? ACT_RELU : ACT_GELU;

  // Gradients that are computed, with their sizes; zeroed unless accumulating.
  float* dwqkv = gr->dw_qkv; float* dbqkv = bqkv ? gr->db_qkv : nullptr;
  float* dwo = gr->dw_o; float* dbo = bo ? gr->db_o : nullptr;
  float* dw1 = gr->dw_1; float* db1 = b1 ? gr->db_1 : nullptr;
  float* dw2 = gr->dw_2; float* db2 = wt->b_2 ? gr->db_2 : nullptr;
  float* dw3 = swiglu ? gr->dw_3 : nullptr;
  float* dg1 = gr->dn1_g; float* dsh1 = sh1 ? gr->dn1_b : nullptr;
  float* dg2 = gr->dn2_g; float* dsh2 = sh2 ? gr->dn2_b : nullptr;
  if (!gr->accumulate) {
    BPT_TRY(fill(st, dwqkv, p.h * p.qkv_cols, 0.f)); BPT_TRY(fill(st, dbqkv, p.qkv_cols, 0.f));
    BPT_TRY(fill(st, dwo, HD * p.h, 0.f)); BPT_TRY(fill(st, dbo, p.h, 0.f));
    BPT_TRY(fill(st, dw1, p.h * p.f, 0.f)); BPT_TRY(fill(st, db1, p.f, 0.f));
    BPT_TRY(fill(st, dw2, p.f * p.h, 0.f)); BPT_TRY(fill(st, db2, p.h, 0.f));
    BPT_TRY(fill(st, dw3, p.h * p.f, 0.f));
    BPT_TRY(fill(st, dg1, p.h, 0.f)); BPT_TRY(fill(st, dsh1, p.h, 0.f));
    BPT_TRY(fill(st, dg2, p.h, 0.f)); BPT_TRY(fill(st, dsh2, p.h, 0.f));
  }
  BPT_TRY(rope_table(st, p, w.rope));
  Range r_all("bpt layer backward (s=%lld)", (long long)p.s);

  for (int64_t bi = 0; bi < p.b; ++bi) {
    const T* xb = x + bi * p.s * p.h;
    const T* dyb = dy + bi * p.s * p.h;
    T* dxb = dx + bi * p.s * p.h;
    const T* Ob = O + bi * p.s * HD;
    const float* Lb = LSE + bi * p.H * p.s;
    BPT_TRY((norm_fwd<T, T, T>(st, p, xb, p.h, g1, sh1, w.xn, p.h, p.s)));

    // ---- FFN and Norm2 backward, a group of gq consecutive query blocks at
    // a time (h1 = x + O W_o + b_o recomputed for the group, the whole FFN
    // chain of the group, then its weight gradients).
    int np_db1 = 0, np_n2 = 0;
    const int64_t grp = p.gq * p.cq;
    for (int64_t g0 = 0; g0 < p.s; g0 += grp) {
      const int64_t rows = std::min(grp, p.s - g0);  // a multiple of c_q
      Range r_g("backward: FFN and Norm2 (recomputed), rows %lld-%lld", (long long)g0,
                (long long)(g0 + rows));
      const T* dyg = dyb + g0 * p.h;
      const float* h1g = w.h1;
      {
        EpiResid<T, T, float> eo{w.h1, p.h, xb + g0 * p.h, p.h, bo};
        BPT_TRY((gemm<T, true, false>(st, Ob + g0 * HD, HD, wo, p.h, rows, p.h, HD, eo,
                                      "o projection (re)")));
      }
      BPT_TRY((norm_fwd<T, float, T>(st, p, h1g, p.h, g2, sh2, w.z, p.h, rows)));
      if (swiglu) {
        EpiOut<T, T> eg{w.a, p.f, b1, 1.f, 0};   // w.a holds the gate pre-activation
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w1, p.f, rows, p.f, p.h, eg, "ffn gate (re)")));
        EpiSwiUp<T> eu{w.u, w.up, w.a, p.f};
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w3, p.f, rows, p.f, p.h, eu, "ffn up (re)")));
        EpiSwiGrad<T> e{w.da, w.dup, w.a, w.up, p.f};
        BPT_TRY((gemm<T, true, true>(st, dyg, p.h, w2, p.h, rows, p.f, p.h, e, "du (swiglu)")));
      } else {
        EpiAct<T> ea{w.u, w.a, p.f, b1, act};
        BPT_TRY((gemm<T, true, false>(st, w.z, p.h, w1, p.f, rows, p.f, p.h, ea, "ffn fc1 (re)")));
        EpiActGrad<T> e{w.da, w.a, p.f, act};
        BPT_TRY((gemm<T, true, true>(st, dyg, p.h, w2, p.h, rows, p.f, p.h, e, "du")));
      }
      // Bias and norm-parameter gradients: partial column sums accumulate over
      // the groups and are reduced after the last one.
      const int first = g0 == 0 ? 0 : 1;
      const bool last = g0 + rows >= p.s;
      BPT_TRY(colsum<T>(st, w.da, p.f, rows, p.f, w.part, db1, first, last, &np_db1));
      {
        EpiOut<T, float> e{w.dz, p.h, nullptr, 1.f, 0};
        BPT_TRY((gemm<T, true, true>(st, w.da, p.f, w1, p.f, rows, p.h, p.f, e, "dz")));
        if (swiglu) {
          EpiOut<T, float> e3{w.dz, p.h, nullptr, 1.f, 1};
          BPT_TRY((gemm<T, true, true>(st, w.dup, p.f, w3, p.f, rows, p.h, p.f, e3, "dz (up)")));
        }
      }
      BPT_TRY((norm_bwd<T, float, T>(st, p, w.dz, p.h, h1g, p.h, g2, dyg, p.h, w.dh + g0 * p.h,
                                     w.dh_t + g0 * p.h, p.h, rows, dg2, dsh2, w.npart_g,
                                     w.npart_b, first, last, &np_n2)));
      // Weight gradients of the group, reduced over all of its rows.
      if (dw2) {
        EpiOut<T, float> e{dw2, p.h, nullptr, 1.f, 1};
        BPT_TRY((gemm<T, false, false>(st, w.u, p.f, dyg, p.h, p.f, p.h, rows, e, "dW2", w.kbuf,
                                       w.kbuf_floats)));
      }
      if (dw1) {
        EpiOut<T, float> e{dw1, p.f, nullptr, 1.f, 1};
        BPT_TRY((gemm<T, false, false>(st, w.z, p.h, w.da, p.f, p.h, p.f, rows, e, "dW1", w.kbuf,
                                       w.kbuf_floats)));
      }
      if (dw3) {
        EpiOut<T, float> e{dw3, p.f, nullptr, 1.f, 1};
        BPT_TRY((gemm<T, false, false>(st, w.z, p.h, w.dup, p.f, p.h, p.f, rows, e, "dW3", w.kbuf,
                                       w.kbuf_floats)));
      }
    }
    // ---- O-projection backward over the whole sequence: dW_o += O^T dh,
    // dO = dh W_o^T.
    if (dwo) {
      EpiOut<T, float> e{dwo, p.h, nullptr, 1.f, 1};
      BPT_TRY((gemm<T, false, false>(st, Ob, HD, w.dh_t, p.h, HD, p.h, p.s, e, "dWo", w.kbuf,
                                     w.kbuf_floats)));
    }
    {
      EpiOut<T, T> e{w.dO, HD, nullptr, 1.f, 0};
      BPT_TRY((gemm<T, true, true>(st, w.dh_t, p.h, wo, p.h, p.s, HD, p.h, e, "dO")));
    }

    // Output-bias gradients over the whole sequence: db_2 = sum of dy rows,
    // db_o = sum of the rows of dh (the gradient at the attention residual).
    BPT_TRY(colsum<T>(st, dyb, p.h, p.s, p.h, w.part, db2));
    BPT_TRY(colsum<float>(st, w.dh, p.h, p.s, p.h, w.part, dbo));

    // ---- attention backward per head chunk
    {
    TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
    // D / 8 lanes per (row, head); D is 32, 64 or 128 (validated)
    const dim3 gd((unsigned)((p.s * p.H * (p.D / 8) + 255) / 256));
    if (p.D == 128)
      hipLaunchKernelGGL((attn_dvec_kernel<T, 16>), gd, dim3(256), 0, st, w.dO, Ob, HD, w.dvec,
                         (int)p.s, (int)p.H);
    else if (p.D == 64)
      hipLaunchKernelGGL((attn_dvec_kernel<T, 8>), gd, dim3(256), 0, st, w.dO, Ob, HD, w.dvec,
                         (int)p.s, (int)p.H);
    else
      hipLaunchKernelGGL((attn_dvec_kernel<T, 4>), gd, dim3(256), 0, st, w.dO, Ob, HD, w.dvec,
                         (int)p.s, (int)p.H);
    BPT_TRY(check_launch("attn_dvec"));
    }
    for (int64_t ch = 0; ch < p.H / p.U; ++ch) {
      Range r_ch("backward: projection (recomputed), attention and QKV, head chunk %lld",
                 (long long)ch);
      const int64_t hq0 = ch * p.U, hk0 = hq0 / p.G;
      BPT_TRY(qkv_chunk<T>(st, p, w.xn, wqkv, bqkv, ch, w.q, w.k, w.v, w.rope, w.wc, w.bc));
      T* dK = w.dqkv + p.U * p.D;
      T* dV = w.dqkv + (p.U + p.nkvc) * p.D;
      BPT_TRY(attn_bwd<T>(st, p, w.q, w.k, w.v, w.dO + hq0 * p.D, Lb + hq0 * p.s,
                          w.dvec + hq0 * p.s, w.dqkv, dK, dV, w.rope, w.dkv_part, hq0, bi));
      const int64_t segc[3] = {0, p.U * p.D, (p.U + p.nkvc) * p.D};
      const int64_t wcol[3] = {hq0 * p.D, (p.H + hk0) * p.D, (p.H + p.Hkv + hk0) * p.D};
      const int64_t wid[3] = {p.U * p.D, p.nkvc * p.D, p.nkvc * p.D};
      if (p.U == p.H) {
        // One chunk: dQ|dK|dV are the packed QKV columns in order, so the
        // weight gradient, bias gradient and dxn are single GEMMs / sums.
        if (dwqkv) {
          EpiOut<T, float> e{dwqkv, p.qkv_cols, nullptr, 1.f, 1};
          BPT_TRY((gemm<T, false, false>(st, w.xn, p.h, w.dqkv, p.chunk_cols, p.h, p.qkv_cols,
                                         p.s, e, "dWqkv", w.kbuf, w.kbuf_floats)));
        }
        BPT_TRY(colsum<T>(st, w.dqkv, p.chunk_cols, p.s, p.qkv_cols, w.part, dbqkv));
        EpiOut<T, float> e{w.dxn, p.h, nullptr, 1.f, 0};
        BPT_TRY((gemm<T, true, true>(st, w.dqkv, p.chunk_cols, wqkv, p.qkv_cols, p.s, p.h,
                                     p.qkv_cols, e, "dxn")));
        continue;
      }
      // Several chunks: dQ|dK|dV of the chunk are contiguous in dqkv, so the
      // weight gradient is one GEMM whose epilogue scatters the three column
      // segments to their places in dW_qkv, and dxn is one GEMM against the
      // gathered weight columns wc (from qkv_chunk above).
      const ChunkCols cc = chunk_cols_of(p, ch);
      if (dwqkv) {
        EpiOut3<T> e{dwqkv + cc.off[0], dwqkv + cc.off[1], dwqkv + cc.off[2], p.qkv_cols,
                     (int)segc[1], (int)segc[2], 1};
        BPT_TRY((gemm<T, false, false>(st, w.xn, p.h, w.dqkv, p.chunk_cols, p.h, p.chunk_cols,
                                       p.s, e, "dWqkv (chunk)", w.kbuf, w.kbuf_floats)));
      }
      for (int seg = 0; seg < 3; ++seg)
        BPT_TRY(colsum<T>(st, w.dqkv + segc[seg], p.chunk_cols, p.s, wid[seg], w.part,
                          dbqkv ? dbqkv + wcol[seg] : nullptr));
      EpiOut<T, float> e{w.dxn, p.h, nullptr, 1.f, ch == 0 ? 0 : 1};
      BPT_TRY((gemm<T, true, true>(st, w.dqkv, p.chunk_cols, w.wc, p.chunk_cols, p.s, p.h,
                                   p.chunk_cols, e, "dxn (chunk)")));
    }
    // ---- Norm1 backward + residual: dx = dh + Norm1'(dxn)
    int np_n1 = 0;
    BPT_TRY((norm_bwd<T, T, float>(st, p, w.dxn, p.h, xb, p.h, g1, w.dh, p.h, nullptr, dxb, p.h,
                                   p.s, dg1, dsh1, w.npart_g, w.npart_b, 0, true, &np_n1)));
  }
  return BPT_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// ----------------------------------------------------------------- static scratch
// Workspace of the allocation-free forward (bpt_layer_forward_noalloc): a
// device array in the library's code object, so every GPU the library runs on
// holds its own copy for the life of the process. Host code never passes the
// array's name to a kernel (in host code it is only a stand-in symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device and cached.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

bpt_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BPT_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BPT_EUNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(BPT_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BPT_OK;
}

bpt_status check_weights(const Plan& p, const bpt_layer_weights* w) {
  if (!w) return fail(BPT_EINVAL, "weights is NULL");
  const void* mats[4] = {w->w_qkv, w->w_o, w->w_1, w->w_2};
  for (const void* m : mats)
    if (!m || !aligned16(m)) return fail(BPT_EINVAL, "weight matrix NULL or not 16-byte aligned");
  if (p.ffn == BPT_SWIGLU && (!w->w_3 || !aligned16(w->w_3)))
    return fail(BPT_EINVAL, "SwiGLU needs w_3 (16-byte aligned)");
  if (!w->n1_g || !w->n2_g) return fail(BPT_EINVAL, "norm scales n1_g and n2_g are required");
  if (p.norm == BPT_RMSNORM && (w->n1_b || w->n2_b))
    return fail(BPT_EINVAL, "RMSNorm takes no shift (n1_b, n2_b must be NULL)");
  const void* vecs[8] = {w->b_qkv, w->b_o, w->b_1, w->b_2, w->n1_g, w->n1_b, w->n2_g, w->n2_b};
  for (const void* v : vecs)
    if (v && ((uintptr_t)v % p.esz) != 0) return fail(BPT_EINVAL, "vector parameter misaligned");
  return BPT_OK;
}

// ================================================================= layer stack
// L layers with checkpointing every k layers ("Training memory...", §3,
// checkpoint every k layers: the input of every k-th layer is kept; the
// backward rebuilds one segment of k layers at a time, keeping that segment's
// layer inputs and saved states, then runs its layers' backward in reverse).
// k = 0 keeps every layer's input and saved state (no recompute).
struct StackPlan {
  Plan lp;
  int64_t L, k, nck;  // nck: checkpoint slots (k >= 1) or stored inputs (k = 0)
  size_t act, sv;     // one activation [b, s, h] and one layer saved buffer, 256-aligned
};

bpt_status make_stack_plan(const bpt_stack_desc* d, StackPlan& sp) {
  if (!d) return fail(BPT_EINVAL, "desc is NULL");
  BPT_TRY(make_plan(&d->layer, sp.lp));
  if (d->n_layers < 1 || d->n_layers > 4096) return fail(BPT_EINVAL, "n_layers must be 1..4096");
  if (d->checkpoint_every < 0 || d->checkpoint_every > d->n_layers)
    return fail(BPT_EINVAL, "checkpoint_every must be 0..n_layers");
  sp.L = d->n_layers;
  sp.k = d->checkpoint_every;
  sp.nck = sp.k ? (sp.L + sp.k - 1) / sp.k - 1 : sp.L - 1;
  sp.act = align_up((size_t)(sp.lp.b * sp.lp.s * sp.lp.h) * sp.lp.esz, 256);
  sp.sv = align_up(saved_bytes(sp.lp), 256);
  return BPT_OK;
}

size_t stack_saved_bytes(const StackPlan& sp) {
  return (size_t)sp.nck * sp.act + (sp.k ? 0 : (size_t)sp.L * sp.sv);
}

// Forward workspace: two ping-pong activations, one transient saved buffer
// (k >= 1) and the layer's forward workspace.
size_t stack_fwd_ws_bytes(const StackPlan& sp) {
  return 2 * sp.act + (sp.k ? sp.sv : 0) + fwd_ws_bytes(sp.lp);
}

// Backward workspace: the rebuilt segment (k - 1 layer inputs, k saved
// buffers, one scratch output) for k >= 1, two gradient ping-pong buffers and
// the layer workspace.
size_t stack_bwd_ws_bytes(const StackPlan& sp) {
  const size_t lw = std::max(fwd_ws_bytes(sp.lp), bwd_ws_bytes(sp.lp));
  const size_t seg = sp.k ? (size_t)(sp.k - 1) * sp.act + (size_t)sp.k * sp.sv + sp.act : 0;
  return seg + 2 * sp.act + (sp.k ? lw : bwd_ws_bytes(sp.lp));
}

template <typename T>
bpt_status stack_forward_impl(const StackPlan& sp, const T* x, const bpt_layer_weights* w, T* y,
                              char* saved, char* ws, hipStream_t st) {
  char* pp[2] = {ws, ws + sp.act};
  char* tsaved = ws + 2 * sp.act;
  char* lws = tsaved + (sp.k ? sp.sv : 0);
  const T* cur = x;
  for (int64_t l = 0; l < sp.L; ++l) {
    T* out;
    if (l == sp.L - 1) out = y;
    else if (sp.k == 0) out = (T*)(saved + (size_t)l * sp.act);            // input of layer l + 1
    else if ((l + 1) % sp.k == 0) out = (T*)(saved + (size_t)((l + 1) / sp.k - 1) * sp.act);
    else out = (T*)pp[l & 1];
    void* lsaved = sp.k ? (void*)tsaved : (void*)(saved + (size_t)sp.nck * sp.act + l * sp.sv);
    Range r_l("stack forward: layer %lld", (long long)l);
    BPT_TRY(forward_impl<T>(sp.lp, cur, &w[l], out, lsaved, lws, st));
    cur = out;
  }
  return BPT_OK;
}

template <typename T>
bpt_status stack_backward_impl(const StackPlan& sp, const T* x, const bpt_layer_weights* w,
                               const char* saved, const T* dy, T* dx, const bpt_layer_grads* gr,
                               char* ws, hipStream_t st) {
  const int64_t kk = sp.k ? sp.k : sp.L;
  char* seg_in = ws;                                        // k - 1 layer inputs
  char* seg_sv = seg_in + (sp.k ? (size_t)(sp.k - 1) * sp.act : 0);
  char* scratch = seg_sv + (sp.k ? (size_t)sp.k * sp.sv : 0);
  char* gb[2] = {scratch + (sp.k ? sp.act : 0), scratch + (sp.k ? sp.act : 0) + sp.act};
  char* lws = gb[1] + sp.act;
  const T* g_cur = dy;
  const int64_t nseg = (sp.L + kk - 1) / kk;
  std::vector<const T*> in(kk + 1);
  std::vector<const void*> sv(kk);
  for (int64_t j = nseg - 1; j >= 0; --j) {
    const int64_t l0 = j * kk, cnt = std::min(kk, sp.L - l0);
    if (sp.k) {
      // Rebuild the segment from its checkpoint: each layer's input and saved state.
      in[0] = j == 0 ? x : (const T*)(saved + (size_t)(j - 1) * sp.act);
      for (int64_t i = 0; i < cnt; ++i) {
        T* out = i < cnt - 1 ? (T*)(seg_in + (size_t)i * sp.act) : (T*)scratch;
        void* lsv = seg_sv + (size_t)i * sp.sv;
        Range r_l("stack backward: layer %lld recomputed", (long long)(l0 + i));
        BPT_TRY(forward_impl<T>(sp.lp, in[i], &w[l0 + i], out, lsv, lws, st));
        in[i + 1] = out;
        sv[i] = lsv;
      }
    } else {
      for (int64_t i = 0; i < cnt; ++i) {
        const int64_t l = l0 + i;
        in[i] = l == 0 ? x : (const T*)(saved + (size_t)(l - 1) * sp.act);
        sv[i] = saved + (size_t)sp.nck * sp.act + (size_t)l * sp.sv;
      }
    }
    for (int64_t i = cnt - 1; i >= 0; --i) {
      const int64_t l = l0 + i;
      T* g_out = l == 0 ? dx : (T*)(g_cur == (const T*)gb[0] ? gb[1] : gb[0]);
      Range r_l("stack backward: layer %lld", (long long)l);
      BPT_TRY(backward_impl<T>(sp.lp, in[i], &w[l], sv[i], g_cur, g_out, &gr[l], lws, st));
      g_cur = g_out;
    }
  }
  return BPT_OK;
}

// ================================================================= LM head
// Blockwise LM head with cross-entropy: chunks of chunk_rows rows, whose
// logits (z W) exist only inside the GEMM's epilogue in the forward and as a
// chunk x V dlogit buffer in the backward.
struct LmPlan {
  int dtype;
  int64_t n, h, V, c, nb;
  size_t esz;
};

bpt_status make_lm_plan(const bpt_lm_head_desc* d, LmPlan& p) {
  if (!d) return fail(BPT_EINVAL, "desc is NULL");
  if (d->abi_version != BPT_ABI_VERSION) return fail(BPT_EINVAL, "abi_version mismatch");
  if (d->dtype != BPT_F32 && d->dtype != BPT_BF16) return fail(BPT_EINVAL, "dtype");
  if (d->rows < 1 || d->rows > (int64_t(1) << 30)) return fail(BPT_EINVAL, "rows");
  if (d->hidden < 64 || d->hidden % 64 != 0 || d->hidden > 65536)
    return fail(BPT_EINVAL, "hidden must be a positive multiple of 64 (<= 65536)");
  if (d->vocab < 64 || d->vocab % 64 != 0 || d->vocab > (int64_t(1) << 24))
    return fail(BPT_EINVAL, "vocab must be a positive multiple of 64 (<= 2^24)");
  if (d->chunk_rows < 64 || d->chunk_rows % 64 != 0)
    return fail(BPT_EINVAL, "chunk_rows must be a positive multiple of 64");
  p.dtype = d->dtype; p.n = d->rows; p.h = d->hidden; p.V = d->vocab;
  p.c = std::min<int64_t>(d->chunk_rows, (d->rows + 63) / 64 * 64);
  if (p.c * p.V >= (int64_t(1) << 31) || p.c * p.h >= (int64_t(1) << 31))
    return fail(BPT_EUNSUPPORTED, "chunk_rows x vocab (or x hidden) must stay below 2^31");
  p.nb = p.V / 32;
  p.esz = d->dtype == BPT_BF16 ? 2 : 4;
  return BPT_OK;
}

struct LmWs {
  float2* part; float* tlogit; void* dl; float* logits; float* lse2;
};

// mode 0: forward (partials, target logits); 1: backward (dlogits); 2: the
// fused call (both, plus the chunk's fp32 logits and log-sum-exps).
LmWs carve_lm(Carver& c, const LmPlan& p, int mode) {
  LmWs w{};
  if (mode != 1) {
    w.part = c.take<float2>(p.c * p.nb);
    w.tlogit = c.take<float>(p.c);
  }
  if (mode != 0) w.dl = c.take<char>(p.c * p.V * p.esz);
  if (mode == 2) {
    w.logits = c.take<float>(p.c * p.V);
    w.lse2 = c.take<float>(p.c);
  }
  return w;
}

size_t lm_ws_bytes(const LmPlan& p, int mode) {
  Carver c(nullptr);
  carve_lm(c, p, mode);
  return c.off;
}

template <typename T>
bpt_status lm_forward_impl(const LmPlan& p, const T* z, const T* w, const int* tg, float* loss,
                           float* lse2, void* ws, hipStream_t st) {
  Carver c(ws);
  LmWs wk = carve_lm(c, p, 0);
  for (int64_t r0 = 0; r0 < p.n; r0 += p.c) {
    const int64_t rows = std::min(p.c, p.n - r0);
    Range r_c("lm head forward: rows %lld-%lld", (long long)r0, (long long)(r0 + rows));
    EpiCEStats<> e{wk.part, p.nb, wk.tlogit, tg + r0, (int)p.V, nullptr};
    BPT_TRY((gemm<T, true, false>(st, z + r0 * p.h, p.h, w, p.V, rows, p.V, p.h, e, "lm logits",
                                  nullptr, 0, BPT_KERNEL_LM_HEAD)));
    TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
    hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       wk.part, p.nb, wk.tlogit, tg + r0, (int)rows, (int)p.V, lse2 + r0,
                       loss + r0);
    BPT_TRY(check_launch("ce combine"));
  }
  return BPT_OK;
}

template <typename T>
bpt_status lm_backward_impl(const LmPlan& p, const T* z, const T* w, const int* tg,
                            const float* lse2, const float* dloss, T* dz, float* dw,
                            int accumulate, void* ws, hipStream_t st) {
  Carver c(ws);
  LmWs wk = carve_lm(c, p, 1);
  T* dl = (T*)wk.dl;
  if (dw && !accumulate) BPT_TRY(fill(st, dw, p.h * p.V, 0.f));
  for (int64_t r0 = 0; r0 < p.n; r0 += p.c) {
    const int64_t rows = std::min(p.c, p.n - r0);
    Range r_c("lm head backward: rows %lld-%lld", (long long)r0, (long long)(r0 + rows));
    EpiCEGrad<T> eg{dl, p.V, lse2 + r0, tg + r0, dloss + r0, (int)p.V};
    BPT_TRY((gemm<T, true, false>(st, z + r0 * p.h, p.h, w, p.V, rows, p.V, p.h, eg,
                                  "lm logits (re) -> dlogits", nullptr, 0, BPT_KERNEL_LM_HEAD)));
    if (dz) {
      EpiOut<T, T> ez{dz + r0 * p.h, p.h, nullptr, 1.f, 0};
      BPT_TRY((gemm<T, true, true>(st, dl, p.V, w, p.V, rows, p.h, p.V, ez, "lm dz", nullptr, 0,
                                   BPT_KERNEL_LM_HEAD)));
    }
    if (dw) {
      EpiOut<T, float> ew{dw, p.V, nullptr, 1.f, 1};
      BPT_TRY((gemm<T, false, false>(st, z + r0 * p.h, p.h, dl, p.V, p.h, p.V, rows, ew, "lm dW",
                                     nullptr, 0, BPT_KERNEL_LM_HEAD)));
    }
  }
  return BPT_OK;
}

// Forward and backward in one pass over the chunks: the logits GEMM stores
// the chunk's fp32 logits beside its statistics, and the dlogits come from
// them (same arithmetic as the backward's recompute epilogue) instead of from
// a second logits GEMM. lse2 (the saved state) may be NULL.
template <typename T>
bpt_status lm_fused_impl(const LmPlan& p, const T* z, const T* w, const int* tg,
                         const float* dloss, float* loss, float* lse2, T* dz, float* dw,
                         int accumulate, void* ws, hipStream_t st) {
  Carver c(ws);
  LmWs wk = carve_lm(c, p, 2);
  T* dl = (T*)wk.dl;
  if (dw && !accumulate) BPT_TRY(fill(st, dw, p.h * p.V, 0.f));
  for (int64_t r0 = 0; r0 < p.n; r0 += p.c) {
    const int64_t rows = std::min(p.c, p.n - r0);
    Range r_c("lm head forward+backward: rows %lld-%lld", (long long)r0, (long long)(r0 + rows));
    float* l2 = lse2 ? lse2 + r0 : wk.lse2;
    EpiCEStats<true> e{wk.part, p.nb, wk.tlogit, tg + r0, (int)p.V, wk.logits};
    BPT_TRY((gemm<T, true, false>(st, z + r0 * p.h, p.h, w, p.V, rows, p.V, p.h, e,
                                  "lm logits (stored)", nullptr, 0, BPT_KERNEL_LM_HEAD)));
    {
      TimedLaunch tl(BPT_KERNEL_ROWWISE, st);
      hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                         wk.part, p.nb, wk.tlogit, tg + r0, (int)rows, (int)p.V, l2, loss + r0);
      const int64_t n4 = rows * (p.V / 4);
      hipLaunchKernelGGL((ce_dlogit_kernel<T>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                         st, wk.logits, l2, tg + r0, dloss + r0, (int)rows, (int)p.V, dl);
      BPT_TRY(check_launch("ce combine / dlogits"));
    }
    if (dz) {
      EpiOut<T, T> ez{dz + r0 * p.h, p.h, nullptr, 1.f, 0};
      BPT_TRY((gemm<T, true, true>(st, dl, p.V, w, p.V, rows, p.h, p.V, ez, "lm dz", nullptr, 0,
                                   BPT_KERNEL_LM_HEAD)));
    }
    if (dw) {
      EpiOut<T, float> ew{dw, p.V, nullptr, 1.f, 1};
      BPT_TRY((gemm<T, false, false>(st, z + r0 * p.h, p.h, dl, p.V, p.h, p.V, rows, ew, "lm dW",
                                     nullptr, 0, BPT_KERNEL_LM_HEAD)));
    }
  }
  return BPT_OK;
}

}  // namespace

// ================================================================= C ABI
extern "C" {

bpt_status bpt_layer_validate(const bpt_layer_desc* desc) {
  Plan p;
  return make_plan(desc, p);
}

size_t bpt_layer_saved_size(const bpt_layer_desc* desc) {
  Plan p;
  if (make_plan(desc, p) != BPT_OK) return 0;
  return saved_bytes(p);
}

size_t bpt_layer_workspace_size(const bpt_layer_desc* desc, int32_t backward) {
  Plan p;
  if (make_plan(desc, p) != BPT_OK) return 0;
  return backward ? bwd_ws_bytes(p) : fwd_ws_bytes(p);
}

bpt_status bpt_layer_forward(const bpt_layer_desc* desc, const void* x, const bpt_layer_weights* w,
                             void* y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  Plan p;
  BPT_TRY(make_plan(desc, p));
  BPT_TRY(check_weights(p, w));
  if (!x || !y || !saved || !ws) return fail(BPT_EINVAL, "x, y, saved and ws must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved) || ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "x, y, saved must be 16-byte and ws 256-byte aligned");
  if (ws_bytes < fwd_ws_bytes(p)) return fail(BPT_EWORKSPACE, "workspace too small");
  log_plan("bpt_layer_forward", p, fwd_ws_bytes(p));
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return forward_impl<bf16>(p, (const bf16*)x, w, (bf16*)y, saved, ws, st);
  return forward_impl<float>(p, (const float*)x, w, (float*)y, saved, ws, st);
}

bpt_status bpt_layer_forward_noalloc(const bpt_layer_desc* desc, const void* x,
                                     const bpt_layer_weights* w, void* y, void* saved,
                                     void* stream) {
  g_last_error.clear();
  Plan p;
  BPT_TRY(make_plan(desc, p));
  BPT_TRY(check_weights(p, w));
  if (!x || !y || !saved) return fail(BPT_EINVAL, "x, y and saved must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved))
    return fail(BPT_EINVAL, "x, y and saved must be 16-byte aligned");
  const size_t need = fwd_ws_bytes(p);
  if (need > kScratchBytes)
    return fail(BPT_EWORKSPACE, "this layer's forward needs " + std::to_string(need) +
                                    " bytes of scratch; the static scratch holds " +
                                    std::to_string(kScratchBytes) +
                                    " (use bpt_layer_forward with a workspace)");
  void* ws = nullptr;
  BPT_TRY(scratch_address(&ws));
  log_plan("bpt_layer_forward_noalloc", p, need);
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return forward_impl<bf16>(p, (const bf16*)x, w, (bf16*)y, saved, ws, st);
  return forward_impl<float>(p, (const float*)x, w, (float*)y, saved, ws, st);
}

size_t bpt_layer_noalloc_scratch_bytes(void) { return kScratchBytes; }

bpt_status bpt_layer_backward(const bpt_layer_desc* desc, const void* x, const bpt_layer_weights* w,
                              const void* saved, const void* dy, void* dx,
                              const bpt_layer_grads* grads, void* ws, size_t ws_bytes,
                              void* stream) {
  g_last_error.clear();
  Plan p;
  BPT_TRY(make_plan(desc, p));
  BPT_TRY(check_weights(p, w));
  if (!grads) return fail(BPT_EINVAL, "grads is NULL");
  if (grads->accumulate != 0 && grads->accumulate != 1)
    return fail(BPT_EINVAL, "grads->accumulate must be 0 or 1");
  if (!x || !saved || !dy || !dx || !ws)
    return fail(BPT_EINVAL, "x, saved, dy, dx and ws must be non-NULL");
  if (!aligned16(x) || !aligned16(saved) || !aligned16(dy) || !aligned16(dx) || ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "x, saved, dy, dx must be 16-byte and ws 256-byte aligned");
  const float* gp[13] = {grads->dw_qkv, grads->db_qkv, grads->dw_o, grads->db_o, grads->dw_1,
                         grads->db_1, grads->dw_2, grads->db_2, grads->dw_3, grads->dn1_g,
                         grads->dn1_b, grads->dn2_g, grads->dn2_b};
  for (const float* g : gp)
    if (g && ((uintptr_t)g & 3)) return fail(BPT_EINVAL, "gradient buffer misaligned");
  if (ws_bytes < bwd_ws_bytes(p)) return fail(BPT_EWORKSPACE, "workspace too small");
  log_plan("bpt_layer_backward", p, bwd_ws_bytes(p));
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return backward_impl<bf16>(p, (const bf16*)x, w, saved, (const bf16*)dy, (bf16*)dx, grads, ws,
                               st);
  return backward_impl<float>(p, (const float*)x, w, saved, (const float*)dy, (float*)dx, grads, ws,
                              st);
}

bpt_status bpt_stack_validate(const bpt_stack_desc* desc) {
  StackPlan sp;
  return make_stack_plan(desc, sp);
}

size_t bpt_stack_saved_size(const bpt_stack_desc* desc) {
  StackPlan sp;
  if (make_stack_plan(desc, sp) != BPT_OK) return 0;
  return stack_saved_bytes(sp);
}

size_t bpt_stack_workspace_size(const bpt_stack_desc* desc, int32_t backward) {
  StackPlan sp;
  if (make_stack_plan(desc, sp) != BPT_OK) return 0;
  return backward ? stack_bwd_ws_bytes(sp) : stack_fwd_ws_bytes(sp);
}

bpt_status bpt_stack_forward(const bpt_stack_desc* desc, const void* x,
                             const bpt_layer_weights* w, void* y, void* saved, void* ws,
                             size_t ws_bytes, void* stream) {
  g_last_error.clear();
  StackPlan sp;
  BPT_TRY(make_stack_plan(desc, sp));
  if (!w) return fail(BPT_EINVAL, "weights is NULL");
  for (int64_t l = 0; l < sp.L; ++l) BPT_TRY(check_weights(sp.lp, &w[l]));
  if (!x || !y || !ws || (stack_saved_bytes(sp) && !saved))
    return fail(BPT_EINVAL, "x, y, ws (and saved unless empty) must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)saved & 255) || ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "x, y 16-byte and saved, ws 256-byte aligned");
  if (ws_bytes < stack_fwd_ws_bytes(sp)) return fail(BPT_EWORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (sp.lp.dtype == BPT_BF16)
    return stack_forward_impl<bf16>(sp, (const bf16*)x, w, (bf16*)y, (char*)saved, (char*)ws, st);
  return stack_forward_impl<float>(sp, (const float*)x, w, (float*)y, (char*)saved, (char*)ws, st);
}

bpt_status bpt_stack_backward(const bpt_stack_desc* desc, const void* x,
                              const bpt_layer_weights* w, const void* saved, const void* dy,
                              void* dx, const bpt_layer_grads* grads, void* ws, size_t ws_bytes,
                              void* stream) {
  g_last_error.clear();
  StackPlan sp;
  BPT_TRY(make_stack_plan(desc, sp));
  if (!w || !grads) return fail(BPT_EINVAL, "weights and grads must be non-NULL");
  for (int64_t l = 0; l < sp.L; ++l) {
    BPT_TRY(check_weights(sp.lp, &w[l]));
    const bpt_layer_grads& g = grads[l];
    if (g.accumulate != 0 && g.accumulate != 1)
      return fail(BPT_EINVAL, "grads[l].accumulate must be 0 or 1");
    const float* gp[13] = {g.dw_qkv, g.db_qkv, g.dw_o, g.db_o, g.dw_1, g.db_1, g.dw_2,
                           g.db_2, g.dw_3, g.dn1_g, g.dn1_b, g.dn2_g, g.dn2_b};
    for (const float* q : gp)
      if (q && ((uintptr_t)q & 3)) return fail(BPT_EINVAL, "gradient buffer misaligned");
  }
  if (!x || !dy || !dx || !ws || (stack_saved_bytes(sp) && !saved))
    return fail(BPT_EINVAL, "x, dy, dx, ws (and saved unless empty) must be non-NULL");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || ((uintptr_t)saved & 255) ||
      ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "x, dy, dx 16-byte and saved, ws 256-byte aligned");
  if (ws_bytes < stack_bwd_ws_bytes(sp)) return fail(BPT_EWORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (sp.lp.dtype == BPT_BF16)
    return stack_backward_impl<bf16>(sp, (const bf16*)x, w, (const char*)saved, (const bf16*)dy,
                                     (bf16*)dx, grads, (char*)ws, st);
  return stack_backward_impl<float>(sp, (const float*)x, w, (const char*)saved, (const float*)dy,
                                    (float*)dx, grads, (char*)ws, st);
}

bpt_status bpt_lm_head_validate(const bpt_lm_head_desc* desc) {
  LmPlan p;
  return make_lm_plan(desc, p);
}

size_t bpt_lm_head_saved_size(const bpt_lm_head_desc* desc) {
  LmPlan p;
  if (make_lm_plan(desc, p) != BPT_OK) return 0;
  return (size_t)p.n * 4;
}

size_t bpt_lm_head_workspace_size(const bpt_lm_head_desc* desc, int32_t backward) {
  LmPlan p;
  if (make_lm_plan(desc, p) != BPT_OK || backward < 0 || backward > 2) return 0;
  return lm_ws_bytes(p, backward);
}

bpt_status bpt_lm_head_forward(const bpt_lm_head_desc* desc, const void* z, const void* w_head,
                               const int32_t* targets, float* loss, void* saved, void* ws,
                               size_t ws_bytes, void* stream) {
  g_last_error.clear();
  LmPlan p;
  BPT_TRY(make_lm_plan(desc, p));
  if (!z || !w_head || !targets || !loss || !saved || !ws)
    return fail(BPT_EINVAL, "z, w_head, targets, loss, saved and ws must be non-NULL");
  if (!aligned16(z) || !aligned16(w_head) || ((uintptr_t)targets & 3) || ((uintptr_t)loss & 3) ||
      ((uintptr_t)saved & 3) || ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "z, w_head 16-byte, targets/loss/saved 4-byte, ws 256-byte aligned");
  if (ws_bytes < lm_ws_bytes(p, 0)) return fail(BPT_EWORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return lm_forward_impl<bf16>(p, (const bf16*)z, (const bf16*)w_head, targets, loss,
                                 (float*)saved, ws, st);
  return lm_forward_impl<float>(p, (const float*)z, (const float*)w_head, targets, loss,
                                (float*)saved, ws, st);
}

bpt_status bpt_lm_head_backward(const bpt_lm_head_desc* desc, const void* z, const void* w_head,
                                const int32_t* targets, const void* saved, const float* dloss,
                                void* dz, float* dw_head, int32_t accumulate, void* ws,
                                size_t ws_bytes, void* stream) {
  g_last_error.clear();
  LmPlan p;
  BPT_TRY(make_lm_plan(desc, p));
  if (!z || !w_head || !targets || !saved || !dloss || !ws)
    return fail(BPT_EINVAL, "z, w_head, targets, saved, dloss and ws must be non-NULL");
  if (!dz && !dw_head) return fail(BPT_EINVAL, "dz and dw_head are both NULL");
  if (accumulate != 0 && accumulate != 1) return fail(BPT_EINVAL, "accumulate must be 0 or 1");
  if (!aligned16(z) || !aligned16(w_head) || (dz && !aligned16(dz)) || ((uintptr_t)targets & 3) ||
      ((uintptr_t)saved & 3) || ((uintptr_t)dloss & 3) || ((uintptr_t)dw_head & 3) ||
      ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL, "z, w_head, dz 16-byte, targets/saved/dloss/dw_head 4-byte, ws 256-byte aligned");
  if (ws_bytes < lm_ws_bytes(p, 1)) return fail(BPT_EWORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return lm_backward_impl<bf16>(p, (const bf16*)z, (const bf16*)w_head, targets,
                                  (const float*)saved, dloss, (bf16*)dz, dw_head, accumulate, ws,
                                  st);
  return lm_backward_impl<float>(p, (const float*)z, (const float*)w_head, targets,
                                 (const float*)saved, dloss, (float*)dz, dw_head, accumulate, ws,
                                 st);
}

bpt_status bpt_lm_head_forward_backward(const bpt_lm_head_desc* desc, const void* z,
                                        const void* w_head, const int32_t* targets,
                                        const float* dloss, float* loss, void* saved, void* dz,
                                        float* dw_head, int32_t accumulate, void* ws,
                                        size_t ws_bytes, void* stream) {
  g_last_error.clear();
  LmPlan p;
  BPT_TRY(make_lm_plan(desc, p));
  if (!z || !w_head || !targets || !dloss || !loss || !ws)
    return fail(BPT_EINVAL, "z, w_head, targets, dloss, loss and ws must be non-NULL");
  if (!dz && !dw_head) return fail(BPT_EINVAL, "dz and dw_head are both NULL");
  if (accumulate != 0 && accumulate != 1) return fail(BPT_EINVAL, "accumulate must be 0 or 1");
  if (!aligned16(z) || !aligned16(w_head) || (dz && !aligned16(dz)) || ((uintptr_t)targets & 3) ||
      ((uintptr_t)dloss & 3) || ((uintptr_t)loss & 3) || ((uintptr_t)saved & 3) ||
      ((uintptr_t)dw_head & 3) || ((uintptr_t)ws & 255))
    return fail(BPT_EINVAL,
                "z, w_head, dz 16-byte, targets/dloss/loss/saved/dw_head 4-byte, ws 256-byte aligned");
  if (ws_bytes < lm_ws_bytes(p, 2)) return fail(BPT_EWORKSPACE, "workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (p.dtype == BPT_BF16)
    return lm_fused_impl<bf16>(p, (const bf16*)z, (const bf16*)w_head, targets, dloss, loss,
                               (float*)saved, (bf16*)dz, dw_head, accumulate, ws, st);
  return lm_fused_impl<float>(p, (const float*)z, (const float*)w_head, targets, dloss, loss,
                              (float*)saved, (float*)dz, dw_head, accumulate, ws, st);
}

const char* bpt_status_string(bpt_status s) {
  int code;  // a C caller may pass any int; read it without assuming a valid enumerator
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case BPT_OK: return "ok";
    case BPT_EINVAL: return "invalid argument";
    case BPT_EWORKSPACE: return "workspace too small";
    case BPT_EUNSUPPORTED: return "unsupported configuration";
    case BPT_EHIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* bpt_last_error(void) { return g_last_error.c_str(); }

bpt_status bpt_timing_enable(uint32_t class_mask) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.mask = class_mask & ((1u << BPT_KERNEL_CLASSES) - 1);
  return BPT_OK;
}

bpt_status bpt_mfma_peak_probe(double* tflops, void* stream) {
  if (!tflops) return fail(BPT_EINVAL, "tflops is NULL");
  hipStream_t st = (hipStream_t)stream;
  const int cus = device_cus();
  const int iters = 2048;
  const dim3 grid((unsigned)(2 * cus)), blk(256);  // two waves per SIMD
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return fail(BPT_EHIP, "hipEventCreate");
  if (hipEventCreate(&e1) != hipSuccess) { hipEventDestroy(e0); return fail(BPT_EHIP, "hipEventCreate"); }
  hipLaunchKernelGGL(mfma_peak_kernel, grid, blk, 0, st, iters, 1e-3f);  // warm-up
  hipEventRecord(e0, st);
  hipLaunchKernelGGL(mfma_peak_kernel, grid, blk, 0, st, iters, 1e-3f);
  hipEventRecord(e1, st);
  bpt_status res = BPT_OK;
  float ms = 0.f;
  if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess ||
      hipGetLastError() != hipSuccess || ms <= 0.f)
    res = fail(BPT_EHIP, "mfma peak probe failed");
  else
    *tflops = (double)grid.x * 4.0 * iters * 8.0 * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return res;
}

bpt_status bpt_timing_read(double* total_ms, int64_t* launches, int32_t reset) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  bpt_status st = BPT_OK;
  for (auto& r : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = fail(BPT_EHIP, "timing event query failed");
    t.ms[r.cls] += ms;
    t.n[r.cls] += 1;
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  for (int c = 0; c < BPT_KERNEL_CLASSES; ++c) {
    if (total_ms) total_ms[c] = t.ms[c];
    if (launches) launches[c] = t.n[c];
    if (reset) { t.ms[c] = 0.0; t.n[c] = 0; }
  }
  return st;
}

}  // extern "C"
