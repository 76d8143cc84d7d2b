// C ABI of the low-rank block library: argument validation, workspace
// carving and the launch sequences of the forward and backward passes.
//
// Every check runs before anything is enqueued; a failed check returns a
// negative status with a message for lr_last_error() and no HIP call is
// made, so argument errors are reported identically on hosts without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lr_block.h"
#include "lr_internal.hpp"
#include "lr_attn.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define LR_HIP(call, what)                        \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// ---------------------------------------------------------------------------
// Measurement hook: HIP events around each launch while enabled.
// ---------------------------------------------------------------------------
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
  int reps;      // launches between the two events
  double bytes;  // algorithmic HBM bytes of those launches (memory-bound kernels)
};
std::atomic<bool> g_prof_on{false};
std::atomic<int> g_prof_repeat{1};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start event on construction and a stop event on destruction.
// A memory-bound launch site passes its algorithmic bytes and marks itself
// repeatable: while recording with a repeat count n, it enqueues its kernel
// reps() = n times back to back between the events (such kernels only read
// buffers they do not write, so the result is unchanged).
struct ProfScope {
  hipStream_t s;
  size_t idx = SIZE_MAX;
  int n = 1;
  ProfScope(const char* name, hipStream_t st, double bytes = 0.0, bool repeatable = false)
      : s(st) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    ProfRec r{name, prof_event(), prof_event(), 1, 0.0};
    if (!r.a || !r.b) return;
    if (repeatable) n = g_prof_repeat.load(std::memory_order_relaxed);
    r.reps = n;
    r.bytes = bytes * n;
    (void)hipEventRecord(r.a, s);
    idx = g_prof.size();
    g_prof.push_back(r);
  }
  int reps() const { return n; }
  ~ProfScope() {
    if (idx == SIZE_MAX) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    (void)hipEventRecord(g_prof[idx].b, s);
  }
};

// Enqueues a memory-bound launch reps() times (once unless the measurement
// hook asks for repetitions).
template <class F>
hipError_t launch_rep(const ProfScope& ps, F launch) {
  hipError_t e = hipSuccess;
  for (int i = 0; i < ps.reps() && e == hipSuccess; ++i) e = launch();
  return e;
}

size_t elem_size(int dtype) { return dtype == LR_F32 ? 4 : 2; }
int vec_elems(int dtype) { return dtype == LR_F32 ? 4 : 8; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Workspace carving: each region starts on a 256-byte boundary.
struct Carver {
  unsigned char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<unsigned char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

int check_shape(const lr_block_shape* s) {
  if (!s) return fail(LR_ERR_INVALID_ARG, "shape is NULL");
  if (s->dtype != LR_F32 && s->dtype != LR_BF16)
    return fail(LR_ERR_INVALID_ARG, "dtype %d is neither LR_F32 nor LR_BF16", s->dtype);
  const int64_t dims[5] = {s->T, s->d, s->r, s->d_ff, s->d_norm};
  const char* names[5] = {"T", "d", "r", "d_ff", "d_norm"};
  for (int i = 0; i < 5; ++i)
    if (dims[i] < 1 || dims[i] > kMaxDim)
      return fail(LR_ERR_INVALID_ARG, "%s = %lld is out of range [1, 2^30]", names[i],
                  (long long)dims[i]);
  const int v = vec_elems(s->dtype);
  if (s->d % v || s->r % v || s->d_ff % v)
    return fail(LR_ERR_INVALID_ARG, "d, r and d_ff must be multiples of %d for this dtype", v);
  if (s->n_panels < 1 || s->n_panels > 8)
    return fail(LR_ERR_INVALID_ARG, "n_panels = %d is out of range [1, 8]", s->n_panels);
  if (s->n_panels > 1) {
    if (s->d % s->n_panels)
      return fail(LR_ERR_INVALID_ARG, "d = %lld does not split into %d panels", (long long)s->d,
                  s->n_panels);
    if ((s->d / s->n_panels) % 64)
      return fail(LR_ERR_UNSUPPORTED, "panel width %lld is not a multiple of 64",
                  (long long)(s->d / s->n_panels));
  }
  if (!(s->eps >= 0.0f) || !std::isfinite(s->eps))
    return fail(LR_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (s->emit_partials != 0 && s->emit_partials != 1)
    return fail(LR_ERR_INVALID_ARG, "emit_partials must be 0 or 1");
  if ((int64_t)s->T * s->d_ff > ((int64_t)1 << 40))
    return fail(LR_ERR_UNSUPPORTED, "T * d_ff too large");
  return LR_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(LR_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(LR_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return LR_OK;
}

#define CHECK_PTR(p)                                  \
  do {                                                \
    int rc_ = check_ptr((const void*)(p), #p);        \
    if (rc_) return rc_;                              \
  } while (0)

int check_weights(const lr_block_weights* w) {
  if (!w) return fail(LR_ERR_INVALID_ARG, "weights is NULL");
  CHECK_PTR(w->gamma1);
  CHECK_PTR(w->gamma2);
  CHECK_PTR(w->A_qkv);
  CHECK_PTR(w->B_q);
  CHECK_PTR(w->B_k);
  CHECK_PTR(w->B_v);
  CHECK_PTR(w->A_o);
  CHECK_PTR(w->B_o);
  CHECK_PTR(w->A_gu);
  CHECK_PTR(w->B_g);
  CHECK_PTR(w->B_u);
  CHECK_PTR(w->A_dn);
  CHECK_PTR(w->B_dn);
  return LR_OK;
}

int check_saved(const lr_block_saved* sv) {
  if (!sv) return fail(LR_ERR_INVALID_ARG, "saved is NULL");
  CHECK_PTR(sv->qkv_r);
  CHECK_PTR(sv->o_r);
  CHECK_PTR(sv->gu_r);
  CHECK_PTR(sv->d_r);
  CHECK_PTR(sv->rms1);
  CHECK_PTR(sv->rms2);
  return LR_OK;
}

// ---------------------------------------------------------------------------
// Workspace layouts
// ---------------------------------------------------------------------------
struct FwdWs {
  void *Ag_qkv, *Ag_gu, *h, *m;
};

struct BwdWs {
  void *h, *dh, *m, *dg, *du, *dd_r, *dgus, *do_r, *dqs;
  float *coef1, *coef2, *colpart;
  void* wpart;         // split-K partials of the weight gradients
  size_t wpart_bytes;
  // Transposed copies of the weights the data gradients multiply by (null
  // when the shape does not allow them): B_dn^T [r, d], A_dn^T [F, r],
  // B_g^T, B_u^T [r, F], A_gu^T [d, 2r], B_o^T [r, d], A_o^T [d, r],
  // B_q^T, B_k^T, B_v^T [r, d], A_qkv^T [d, 3r].
  void *tB_dn, *tA_dn, *tB_g, *tB_u, *tA_gu, *tB_o, *tA_o, *tB_q, *tB_k, *tB_v, *tA_qkv;
};

// The backward's data-gradient products multiply an activation gradient by a
// weight whose rows run along the output (NN). On the pipelined engine they
// run as NT products against transposed copies of their weights, made once
// per call in one launch per stage: the NN tiles' transposing LDS reads cost
// 3-10% at these shapes (measured against NT with the transposed weight).
// The copies need bf16 and every side a multiple of 64 (whole tiles of the
// transpose kernel and whole k-tiles of the products).
bool transposed_weights(const lr_block_shape* s) {
  return s->dtype == LR_BF16 && s->d % 64 == 0 && s->r % 64 == 0 && s->d_ff % 64 == 0;
}

// A weight-gradient (TN) descriptor: out [M, N] = a^T b over K rows.
lr::GemmDesc tn_desc(int M, int N, int K, const void* a, int64_t lda, const void* b, int64_t ldb,
                     float* c, const void* colscale) {
  lr::GemmDesc g;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a[0] = a;
  g.lda[0] = lda;
  g.b[0] = b;
  g.ldb[0] = ldb;
  g.c[0] = c;
  g.ldc[0] = N;
  g.colscale = colscale;
  return g;
}

// Partial-sum workspace of the largest split-K weight gradient of the block:
// (M, N, lda, ldb, groups) of every TN GEMM lr_block_bwd runs, K = T.
size_t wgrad_part_max(const lr_block_shape* s) {
  const int64_t T = s->T, d = s->d, r = s->r, F = s->d_ff;
  const int64_t shapes[8][5] = {
      {d, r, d, r, 1},          // dB_dn
      {r, F, r, F, 1},          // dA_dn
      {F, r, F, 2 * r, 2},      // dB_g, dB_u
      {2 * r, d, 2 * r, d, 1},  // dA_gu
      {d, r, d, r, 1},          // dB_o
      {r, d, r, d, 1},          // dA_o
      {d, r, d, 3 * r, 3},      // dB_q, dB_k, dB_v
      {3 * r, d, 3 * r, d, 1},  // dA_qkv
  };
  size_t mx = 0;
  for (const auto& sh : shapes) {
    lr::GemmDesc g;
    g.M = (int)sh[0];
    g.N = (int)sh[1];
    g.K = (int)T;
    for (int i = 0; i < (int)sh[4]; ++i) {
      g.lda[i] = sh[2];
      g.ldb[i] = sh[3];
    }
    const size_t b = lr::wgrad_part_bytes(s->dtype, g, (int)sh[4]);
    mx = b > mx ? b : mx;
  }
  // The weight gradients that run together in one launch.
  const int Ti = (int)T, di = (int)d, ri = (int)r;
  const lr::GemmDesc g3[3] = {tn_desc(2 * ri, di, Ti, nullptr, 2 * r, nullptr, d, nullptr, nullptr),
                              tn_desc(di, ri, Ti, nullptr, d, nullptr, r, nullptr, nullptr),
                              tn_desc(ri, di, Ti, nullptr, r, nullptr, d, nullptr, nullptr)};
  const lr::GemmDesc g2[2] = {tn_desc(3 * ri, di, Ti, nullptr, 3 * r, nullptr, d, nullptr, nullptr),
                              tn_desc(di, ri, Ti, nullptr, d, nullptr, r, nullptr, nullptr)};
  if (lr::wgrad_multi_ok(s->dtype, g3, 3)) {
    const size_t b = lr::wgrad_multi_part_bytes(g3, 3, lr::wgrad_multi_split(g3, 3));
    mx = b > mx ? b : mx;
  }
  if (lr::wgrad_multi_ok(s->dtype, g2, 2)) {
    const size_t b = lr::wgrad_multi_part_bytes(g2, 2, lr::wgrad_multi_split(g2, 2));
    mx = b > mx ? b : mx;
  }
  return mx;
}

size_t carve_fwd(const lr_block_shape* s, void* base, FwdWs* out) {
  const size_t e = elem_size(s->dtype);
  Carver c(base);
  FwdWs w;
  w.Ag_qkv = c.take(e * 3 * s->r * s->d);
  w.Ag_gu = c.take(e * 2 * s->r * s->d);
  w.h = c.take(e * s->T * s->d);
  w.m = c.take(e * s->T * s->d_ff);
  if (out) *out = w;
  return c.off + 256;
}

size_t carve_bwd(const lr_block_shape* s, void* base, BwdWs* out) {
  const size_t e = elem_size(s->dtype);
  Carver c(base);
  BwdWs w;
  w.h = c.take(e * s->T * s->d);
  w.dh = c.take(e * s->T * s->d);
  w.m = c.take(e * s->T * s->d_ff);
  w.dg = c.take(e * s->T * s->d_ff);
  w.du = c.take(e * s->T * s->d_ff);
  w.dd_r = c.take(e * s->T * s->r);
  w.dgus = c.take(e * s->T * 2 * s->r);
  w.do_r = c.take(e * s->T * s->r);
  w.dqs = c.take(e * s->T * 3 * s->r);
  w.coef1 = static_cast<float*>(c.take(4 * s->T));
  w.coef2 = static_cast<float*>(c.take(4 * s->T));
  const int64_t tiles = (s->T + lr::kMinTileM - 1) / lr::kMinTileM;
  w.colpart = static_cast<float*>(c.take(4 * tiles * s->d));
  w.wpart_bytes = wgrad_part_max(s);
  w.wpart = c.take(w.wpart_bytes);
  const bool tw = transposed_weights(s);
  const int64_t d = s->d, r = s->r, F = s->d_ff;
  auto tk = [&](int64_t n) { return tw ? c.take(e * n) : nullptr; };
  w.tB_dn = tk(r * d);
  w.tA_dn = tk(F * r);
  w.tB_g = tk(r * F);
  w.tB_u = tk(r * F);
  w.tA_gu = tk(d * 2 * r);
  w.tB_o = tk(r * d);
  w.tA_o = tk(d * r);
  w.tB_q = tk(r * d);
  w.tB_k = tk(r * d);
  w.tB_v = tk(r * d);
  w.tA_qkv = tk(d * 3 * r);
  if (out) *out = w;
  return c.off + 256;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(LR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  if (!ws) return fail(LR_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(LR_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return LR_OK;
}

// One GEMM launch with error reporting.
int gemm(int op, int dtype, const lr::GemmDesc& d, int groups, hipStream_t st,
         const char* what) {
  ProfScope ps(what, st);
  hipError_t e = lr::run_gemm(op, dtype, d, groups, st);
  if (e != hipSuccess) return hip_fail(e, what);
  return LR_OK;
}

// A data-gradient product X W (NN, `nn`), or, with the transposed weights
// `wt` (one per group, [N, K] rows), the same product as X wt^T (NT) when
// the pipelined engine takes it. The operation and descriptor it ran go to
// *op_run and *used.
int nn_or_nt(int op_nn, int op_nt, int dtype, const lr::GemmDesc& nn, const void* const* wt,
             int groups, hipStream_t st, const char* what, int* op_run = nullptr,
             lr::GemmDesc* used = nullptr) {
  if (wt != nullptr && wt[0] != nullptr) {
    lr::GemmDesc g = nn;
    for (int i = 0; i < groups; ++i) {
      g.b[i] = wt[i];
      g.ldb[i] = nn.K;
    }
    if (lr::uses_engine2(op_nt, dtype, g, groups)) {
      if (op_run) *op_run = op_nt;
      if (used) *used = g;
      return gemm(op_nt, dtype, g, groups, st, what);
    }
  }
  if (op_run) *op_run = op_nn;
  if (used) *used = nn;
  return gemm(op_nn, dtype, nn, groups, st, what);
}

// One weight-gradient GEMM (split-K through the workspace when it pays):
// the GEMM, then, with more than one K-slice, the fixed-order sum of the
// slices (recorded by the measurement hook as `sum_name`).
int wgrad(int dtype, const lr::GemmDesc& d, int groups, void* part, size_t part_bytes,
          hipStream_t st, const char* what, const char* sum_name) {
  const int splits = lr::wgrad_splits(dtype, d, groups, part, part_bytes);
  {
    ProfScope ps(what, st);
    hipError_t e = lr::run_wgrad_gemm(dtype, d, groups, splits, part, st);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  if (splits > 1) {
    const double mn = (double)d.M * d.N;
    const double bytes = groups * mn * 4.0 * (splits + 1) + (d.colscale ? 2.0 * d.N : 0.0);
    ProfScope ps(sum_name, st, bytes, true);
    hipError_t e = launch_rep(ps, [&] { return lr::run_wgrad_sum(d, groups, splits, part, st); });
    if (e != hipSuccess) return hip_fail(e, sum_name);
  }
  return LR_OK;
}

int wgrad(int dtype, const lr::GemmDesc& d, int groups, const BwdWs& W, hipStream_t st,
          const char* what, const char* sum_name) {
  return wgrad(dtype, d, groups, W.wpart, W.wpart_bytes, st, what, sum_name);
}

// Weight gradients of n problems of different shapes in one launch (each
// with its own output and column scale), K split over the workspace when
// their tiles together are too few; then each problem's split-K sum.
int wgrad_multi(int dtype, const lr::GemmDesc* p, int n, const BwdWs& W, hipStream_t st,
                const char* what, const char* const* sum_names) {
  const int splits = lr::wgrad_multi_split(p, n);
  if (lr::wgrad_multi_part_bytes(p, n, splits) > W.wpart_bytes)
    return fail(LR_ERR_WORKSPACE, "%s: split-K partials exceed the workspace", what);
  {
    ProfScope ps(what, st);
    hipError_t e = lr::run_wgrad_multi_gemm(p, n, splits, W.wpart, st);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  for (int i = 0; splits > 1 && i < n; ++i) {
    const float* part = static_cast<const float*>(W.wpart) + lr::wgrad_multi_part_offset(p, i, splits);
    const double mn = (double)p[i].M * p[i].N;
    ProfScope ps(sum_names[i], st, mn * 4.0 * (splits + 1) + (p[i].colscale ? 2.0 * p[i].N : 0.0),
                 true);
    hipError_t e = launch_rep(ps, [&] { return lr::run_wgrad_sum(p[i], 1, splits, part, st); });
    if (e != hipSuccess) return hip_fail(e, sum_names[i]);
  }
  return LR_OK;
}


#define RUN(x)            \
  do {                    \
    int rc_ = (x);        \
    if (rc_) return rc_;  \
  } while (0)

const char* B(const void* p, int64_t off_elems, size_t e) {
  return static_cast<const char*>(p) + off_elems * e;
}
char* Bm(void* p, int64_t off_elems, size_t e) { return static_cast<char*>(p) + off_elems * e; }

}  // namespace

extern "C" {

const char* lr_last_error(void) { return g_err.c_str(); }

const char* lr_version(void) { return "lrblock 0.1 gfx950"; }

// ---------------------------------------------------------------------------
// Causal RoPE attention.
// ---------------------------------------------------------------------------
namespace {

constexpr int kAttnHeadDim = 128;

int check_attn(const lr_attn_shape* s) {
  if (!s) return fail(LR_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 1 || s->seq_len < 1 || s->T > kMaxDim || s->seq_len > kMaxDim)
    return fail(LR_ERR_INVALID_ARG, "T and seq_len must be in [1, 2^30]");
  if (s->T % s->seq_len)
    return fail(LR_ERR_INVALID_ARG, "T = %lld is not a multiple of seq_len = %lld",
                (long long)s->T, (long long)s->seq_len);
  if (s->n_heads < 1 || s->n_kv_heads < 1 || s->n_heads % s->n_kv_heads)
    return fail(LR_ERR_INVALID_ARG, "n_heads = %d must be a positive multiple of n_kv_heads = %d",
                s->n_heads, s->n_kv_heads);
  if (s->dtype != LR_F32 && s->dtype != LR_BF16)
    return fail(LR_ERR_INVALID_ARG, "dtype %d is neither LR_F32 nor LR_BF16", s->dtype);
  if (s->dtype != LR_BF16)
    return fail(LR_ERR_UNSUPPORTED, "attention runs in bf16 only");
  if (s->head_dim < 1) return fail(LR_ERR_INVALID_ARG, "head_dim must be positive");
  if (s->head_dim != kAttnHeadDim)
    return fail(LR_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", s->head_dim);
  if (!(s->rope_base > 1.0) || !std::isfinite(s->rope_base))
    return fail(LR_ERR_INVALID_ARG, "rope_base must be finite and > 1");
  // Byte offsets inside one sequence's head slice are 32-bit.
  if ((int64_t)s->seq_len * s->n_heads * kAttnHeadDim * 2 >= ((int64_t)1 << 31))
    return fail(LR_ERR_UNSUPPORTED, "seq_len * n_heads * 256 bytes must stay below 2^31");
  if (s->T * (int64_t)s->n_heads * kAttnHeadDim >= ((int64_t)1 << 40))
    return fail(LR_ERR_INVALID_ARG, "tensor too large");
  return LR_OK;
}

struct AttnWs {
  void* qr;
  void* kr;
  float* dsum;
  float* lse2;
  size_t bytes;
};

AttnWs attn_carve(const lr_attn_shape* s, void* base, bool bwd) {
  Carver c(base);
  AttnWs w;
  w.qr = c.take((size_t)s->T * s->n_heads * kAttnHeadDim * 2);
  w.kr = c.take((size_t)s->T * s->n_kv_heads * kAttnHeadDim * 2);
  w.dsum = bwd ? static_cast<float*>(c.take((size_t)s->T * s->n_heads * 4)) : nullptr;
  w.lse2 = bwd ? static_cast<float*>(c.take((size_t)s->T * s->n_heads * 4)) : nullptr;
  w.bytes = c.off;
  return w;
}

lr::AttnDesc attn_desc(const lr_attn_shape* s) {
  lr::AttnDesc d;
  d.T = (int)s->T;
  d.seq_len = (int)s->seq_len;
  d.H = s->n_heads;
  d.Hkv = s->n_kv_heads;
  d.rope_base = s->rope_base;
  return d;
}

int check_attn_ws(const lr_attn_shape* s, void* ws, size_t ws_bytes, bool bwd) {
  const size_t need = attn_carve(s, nullptr, bwd).bytes;
  if (!ws || ws_bytes < need)
    return fail(LR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  if (!aligned16(ws)) return fail(LR_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  return LR_OK;
}

// Rotated copies of Q and K into the workspace.
int attn_rotate(const lr_attn_shape* s, const void* Q, const void* K, const AttnWs& w,
                hipStream_t st) {
  {
    ProfScope ps("RoPE Q", st);
    LR_HIP(lr::run_rope(Q, w.qr, (int)s->T, s->n_heads, (int)s->seq_len, s->rope_base, false, st),
           "RoPE Q");
  }
  {
    ProfScope ps("RoPE K", st);
    LR_HIP(lr::run_rope(K, w.kr, (int)s->T, s->n_kv_heads, (int)s->seq_len, s->rope_base, false,
                        st),
           "RoPE K");
  }
  return LR_OK;
}

}  // namespace

size_t lr_attention_workspace_bytes(const lr_attn_shape* shape, int32_t is_bwd) {
  if (check_attn(shape) != LR_OK) return 0;
  return attn_carve(shape, nullptr, is_bwd != 0).bytes;
}

int lr_attention_fwd(const lr_attn_shape* shape, const void* Q, const void* K, const void* V,
                     void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn(shape);
  if (rc != LR_OK) return rc;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(O);
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(LR_ERR_INVALID_ARG, "lse is NULL or not 4-byte aligned");
  rc = check_attn_ws(shape, ws, ws_bytes, false);
  if (rc != LR_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AttnWs w = attn_carve(shape, ws, false);
  rc = attn_rotate(shape, Q, K, w, st);
  if (rc != LR_OK) return rc;
  lr::AttnDesc d = attn_desc(shape);
  d.q = w.qr;
  d.k = w.kr;
  d.v = V;
  d.o = O;
  d.lse = lse;
  ProfScope ps("attention fwd", st);
  LR_HIP(lr::run_attn_fwd(d, st), "attention fwd");
  return LR_OK;
}

int lr_attention_bwd(const lr_attn_shape* shape, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* lse, void* dQ, void* dK,
                     void* dV, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn(shape);
  if (rc != LR_OK) return rc;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(O);
  CHECK_PTR(dO);
  CHECK_PTR(dQ);
  CHECK_PTR(dK);
  CHECK_PTR(dV);
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(LR_ERR_INVALID_ARG, "lse is NULL or not 4-byte aligned");
  rc = check_attn_ws(shape, ws, ws_bytes, true);
  if (rc != LR_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AttnWs w = attn_carve(shape, ws, true);
  rc = attn_rotate(shape, Q, K, w, st);
  if (rc != LR_OK) return rc;
  lr::AttnDesc d = attn_desc(shape);
  d.q = w.qr;
  d.k = w.kr;
  d.v = V;
  d.o = const_cast<void*>(O);
  d.dout = dO;
  d.lse = const_cast<float*>(lse);
  d.dsum = w.dsum;
  d.lse2 = w.lse2;
  d.dq = dQ;
  d.dk = dK;
  d.dv = dV;
  {
    ProfScope ps("attention bwd dQ", st);
    LR_HIP(lr::run_attn_dq(d, st), "attention bwd dQ");
  }
  {
    ProfScope ps("attention bwd dK dV", st);
    LR_HIP(lr::run_attn_dkdv(d, st), "attention bwd dK dV");
  }
  return LR_OK;
}

int lr_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    for (auto& r : g_prof) {
      g_prof_pool.push_back(r.a);
      g_prof_pool.push_back(r.b);
    }
    g_prof.clear();
  }
  g_prof_on.store(on != 0);
  return LR_OK;
}

int lr_profile_repeat(int32_t n) {
  if (n < 1 || n > 1000) return fail(LR_ERR_INVALID_ARG, "repeat count %d is out of range [1, 1000]", n);
  g_prof_repeat.store(n);
  return LR_OK;
}

int lr_profile_collect(lr_kernel_time* out, int32_t max) {
  if (max < 0 || (max > 0 && !out)) return fail(LR_ERR_INVALID_ARG, "bad output array");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  struct Agg {
    const char* name;
    int count;
    double ms;
    double bytes;
  };
  std::vector<Agg> agg;
  for (auto& r : g_prof) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "profile event");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "profile elapsed time");
    size_t i = 0;
    while (i < agg.size() && std::strcmp(agg[i].name, r.name) != 0) ++i;
    if (i == agg.size()) agg.push_back({r.name, 0, 0.0, 0.0});
    agg[i].count += r.reps;
    agg[i].ms += ms;
    agg[i].bytes += r.bytes;
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof.clear();
  for (size_t i = 0; i < agg.size() && (int)i < max; ++i) {
    std::snprintf(out[i].name, sizeof(out[i].name), "%s", agg[i].name);
    out[i].count = agg[i].count;
    out[i].total_ms = (float)agg[i].ms;
    out[i].bytes = agg[i].bytes;
  }
  return (int)agg.size();
}

size_t lr_block_workspace_bytes(const lr_block_shape* shape, int is_bwd) {
  if (check_shape(shape)) return 0;
  return is_bwd ? carve_bwd(shape, nullptr, nullptr) : carve_fwd(shape, nullptr, nullptr);
}

int lr_block_workspace_tensor(const lr_block_shape* shape, int32_t is_bwd, int32_t which,
                              size_t* offset, size_t* bytes) {
  RUN(check_shape(shape));
  if (which != LR_WS_H && which != LR_WS_M)
    return fail(LR_ERR_INVALID_ARG, "which = %d is not an lr_ws_tensor", which);
  if (!offset || !bytes) return fail(LR_ERR_INVALID_ARG, "offset or bytes is NULL");
  // Carved from a base of 256 (a null base carves sizes only), so that a
  // region at offset 0 is told apart from a missing one.
  void* const base = reinterpret_cast<void*>(uintptr_t(256));
  const size_t e = elem_size(shape->dtype);
  void* p;
  if (is_bwd) {
    BwdWs W;
    carve_bwd(shape, base, &W);
    p = which == LR_WS_H ? W.h : W.m;
  } else {
    FwdWs W;
    carve_fwd(shape, base, &W);
    p = which == LR_WS_H ? W.h : W.m;
  }
  *offset = reinterpret_cast<uintptr_t>(p) - 256;
  *bytes = e * (size_t)shape->T * (size_t)(which == LR_WS_H ? shape->d : shape->d_ff);
  return LR_OK;
}

int lr_block_fwd(const lr_block_shape* s, const lr_block_weights* w, const void* X,
                 const void* O_attn, void* Q, void* K, void* V, void* Y,
                 const lr_block_saved* sv, const lr_block_partials* pt, int32_t stage, void* ws,
                 size_t ws_bytes, void* stream) {
  RUN(check_shape(s));
  RUN(check_weights(w));
  RUN(check_saved(sv));
  if (stage < LR_STAGE_ALL || stage > LR_STAGE_POST_ATTN)
    return fail(LR_ERR_INVALID_ARG, "stage %d is not an lr_stage", stage);
  const bool pre = stage != LR_STAGE_POST_ATTN, post = stage != LR_STAGE_PRE_ATTN;
  CHECK_PTR(X);
  if (pre) {
    CHECK_PTR(Q);
    CHECK_PTR(K);
    CHECK_PTR(V);
  }
  if (post) {
    CHECK_PTR(O_attn);
    CHECK_PTR(Y);
  }
  const bool part = s->emit_partials != 0;
  if (part) {
    if (!pt) return fail(LR_ERR_INVALID_ARG, "partials is NULL with emit_partials = 1");
    if (pre) {
      CHECK_PTR(pt->P_qkv);
      CHECK_PTR(pt->ss1);
    }
    if (post) {
      CHECK_PTR(pt->P_gu);
      CHECK_PTR(pt->ss2);
    }
  }
  const size_t need = carve_fwd(s, nullptr, nullptr);
  RUN(check_ws(ws, ws_bytes, need));
  FwdWs W;
  carve_fwd(s, ws, &W);

  const int dt = s->dtype;
  const size_t e = elem_size(dt);
  const int T = (int)s->T, d = (int)s->d, r = (int)s->r, F = (int)s->d_ff;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float inv_D = 1.0f / (float)s->d_norm;
  // Per-panel sums of squares are written in normal mode when asked for.
  float* ssp1 = (!part && pt && s->n_panels > 1) ? pt->ss1 : nullptr;
  float* ssp2 = (!part && pt && s->n_panels > 1) ? pt->ss2 : nullptr;

  // gamma1 and gamma2 folded into copies of the grouped down-projection
  // weights (one launch when both stages run).
  if (pre && post) {
    ProfScope ps("fold gamma1, gamma2", st, (double)e * (2.0 * 5 * r * d + 2 * d), true);
    hipError_t he = launch_rep(ps, [&] {
      return lr::run_fold_gamma2(dt, w->A_qkv, d, w->gamma1, W.Ag_qkv, 3 * r, w->A_gu, d,
                                 w->gamma2, W.Ag_gu, 2 * r, d, st);
    });
    if (he != hipSuccess) return hip_fail(he, "fold gamma");
  }
  if (pre) {
    // Online RMSNorm + grouped [A_q; A_k; A_v] down-projection.
    hipError_t he = hipSuccess;
    if (!post) {
      ProfScope ps("fold gamma1", st, (double)e * (2.0 * 3 * r * d + d), true);
      he = launch_rep(ps, [&] {
        return lr::run_fold_gamma(dt, w->A_qkv, d, w->gamma1, W.Ag_qkv, 3 * r, d, st);
      });
    }
    if (he != hipSuccess) return hip_fail(he, "fold gamma1");
    lr::GemmDesc g;
    g.M = T;
    g.N = 3 * r;
    g.K = d;
    g.a[0] = X;
    g.lda[0] = d;
    g.b[0] = W.Ag_qkv;
    g.ldb[0] = d;
    g.c[0] = part ? pt->P_qkv : sv->qkv_r;
    g.ldc[0] = 3 * r;
    g.rms_out = part ? nullptr : sv->rms1;
    g.ss_out = part ? pt->ss1 : ssp1;
    g.n_panels = s->n_panels;
    g.panel_width = d / s->n_panels;
    g.inv_D = inv_D;
    g.eps = s->eps;
    g.emit_partial = part;
    RUN(gemm(lr::OP_NT_ORMS, dt, g, 1, st, "QKV Online RMSNorm GEMM"));
    if (part) {
      ProfScope ps("QKV finalize", st, (double)e * 2.0 * T * 3 * r + 8.0 * T, true);
      he = launch_rep(ps, [&] {
        return lr::run_finalize(dt, pt->P_qkv, 3 * r, pt->ss1, T, 3 * r, inv_D, s->eps,
                                sv->qkv_r, 3 * r, sv->rms1, st);
      });
      if (he != hipSuccess) return hip_fail(he, "QKV finalize");
    }
    // Grouped Q, K, V up-projections: three (input, weight) pairs.
    lr::GemmDesc u;
    u.M = T;
    u.N = d;
    u.K = r;
    const void* Bs[3] = {w->B_q, w->B_k, w->B_v};
    void* Outs[3] = {Q, K, V};
    for (int i = 0; i < 3; ++i) {
      u.a[i] = B(sv->qkv_r, (int64_t)i * r, e);
      u.lda[i] = 3 * r;
      u.b[i] = Bs[i];
      u.ldb[i] = r;
      u.c[i] = Outs[i];
      u.ldc[i] = d;
    }
    RUN(gemm(lr::OP_NT_STORE, dt, u, 3, st, "QKV grouped up-projection"));
  }

  if (post) {
    // o_r = O A_o^T
    lr::GemmDesc g;
    g.M = T;
    g.N = r;
    g.K = d;
    g.a[0] = O_attn;
    g.lda[0] = d;
    g.b[0] = w->A_o;
    g.ldb[0] = d;
    g.c[0] = sv->o_r;
    g.ldc[0] = r;
    RUN(gemm(lr::OP_NT_STORE, dt, g, 1, st, "O down-projection"));
    // h = X + o_r B_o^T
    lr::GemmDesc hgm;
    hgm.M = T;
    hgm.N = d;
    hgm.K = r;
    hgm.a[0] = sv->o_r;
    hgm.lda[0] = r;
    hgm.b[0] = w->B_o;
    hgm.ldb[0] = r;
    hgm.c[0] = W.h;
    hgm.ldc[0] = d;
    hgm.res = X;
    hgm.ldres = d;
    RUN(gemm(lr::OP_NT_STORE, dt, hgm, 1, st, "O up-projection + residual"));
    // Online RMSNorm + grouped [A_g; A_u] down-projection.
    hipError_t he = hipSuccess;
    if (!pre) {
      ProfScope ps("fold gamma2", st, (double)e * (2.0 * 2 * r * d + d), true);
      he = launch_rep(ps, [&] {
        return lr::run_fold_gamma(dt, w->A_gu, d, w->gamma2, W.Ag_gu, 2 * r, d, st);
      });
    }
    if (he != hipSuccess) return hip_fail(he, "fold gamma2");
    lr::GemmDesc n2;
    n2.M = T;
    n2.N = 2 * r;
    n2.K = d;
    n2.a[0] = W.h;
    n2.lda[0] = d;
    n2.b[0] = W.Ag_gu;
    n2.ldb[0] = d;
    n2.c[0] = part ? pt->P_gu : sv->gu_r;
    n2.ldc[0] = 2 * r;
    n2.rms_out = part ? nullptr : sv->rms2;
    n2.ss_out = part ? pt->ss2 : ssp2;
    n2.n_panels = s->n_panels;
    n2.panel_width = d / s->n_panels;
    n2.inv_D = inv_D;
    n2.eps = s->eps;
    n2.emit_partial = part;
    RUN(gemm(lr::OP_NT_ORMS, dt, n2, 1, st, "gate/up Online RMSNorm GEMM"));
    if (part) {
      ProfScope ps("gate/up finalize", st, (double)e * 2.0 * T * 2 * r + 8.0 * T, true);
      he = launch_rep(ps, [&] {
        return lr::run_finalize(dt, pt->P_gu, 2 * r, pt->ss2, T, 2 * r, inv_D, s->eps,
                                sv->gu_r, 2 * r, sv->rms2, st);
      });
      if (he != hipSuccess) return hip_fail(he, "gate/up finalize");
    }
    // m = SiLU(g_r B_g^T) * (u_r B_u^T), both pairs in one tile.
    lr::GemmDesc sw;
    sw.M = T;
    sw.N = F;
    sw.K = r;
    sw.a[0] = sv->gu_r;
    sw.lda[0] = 2 * r;
    sw.b[0] = w->B_g;
    sw.ldb[0] = r;
    sw.a[1] = B(sv->gu_r, r, e);
    sw.lda[1] = 2 * r;
    sw.b[1] = w->B_u;
    sw.ldb[1] = r;
    sw.c[0] = W.m;
    sw.ldc[0] = F;
    RUN(gemm(lr::OP_NT_SWIGLU, dt, sw, 1, st, "gate/up up-projection + SwiGLU"));
    // d_r = m A_dn^T
    lr::GemmDesc dn;
    dn.M = T;
    dn.N = r;
    dn.K = F;
    dn.a[0] = W.m;
    dn.lda[0] = F;
    dn.b[0] = w->A_dn;
    dn.ldb[0] = F;
    dn.c[0] = sv->d_r;
    dn.ldc[0] = r;
    RUN(gemm(lr::OP_NT_STORE, dt, dn, 1, st, "down-projection"));
    // Y = h + d_r B_dn^T
    lr::GemmDesc yo;
    yo.M = T;
    yo.N = d;
    yo.K = r;
    yo.a[0] = sv->d_r;
    yo.lda[0] = r;
    yo.b[0] = w->B_dn;
    yo.ldb[0] = r;
    yo.c[0] = Y;
    yo.ldc[0] = d;
    yo.res = W.h;
    yo.ldres = d;
    RUN(gemm(lr::OP_NT_STORE, dt, yo, 1, st, "down up-projection + residual"));
  }
  return LR_OK;
}

int lr_block_bwd(const lr_block_shape* s, const lr_block_weights* w, const void* X,
                 const void* O_attn, const lr_block_saved* sv, const void* dY, const void* dQ,
                 const void* dK, const void* dV, void* dX, void* dO_attn,
                 const lr_block_grads* gr, int32_t stage, void* ws, size_t ws_bytes,
                 void* stream) {
  RUN(check_shape(s));
  RUN(check_weights(w));
  RUN(check_saved(sv));
  if (!gr) return fail(LR_ERR_INVALID_ARG, "grads is NULL");
  if (stage < LR_STAGE_ALL || stage > LR_STAGE_POST_ATTN)
    return fail(LR_ERR_INVALID_ARG, "stage %d is not an lr_stage", stage);
  const bool pre = stage != LR_STAGE_POST_ATTN, post = stage != LR_STAGE_PRE_ATTN;
  CHECK_PTR(X);
  if (post) {
    CHECK_PTR(O_attn);
    CHECK_PTR(dY);
    CHECK_PTR(dO_attn);
    CHECK_PTR(gr->gamma2);
    CHECK_PTR(gr->A_o);
    CHECK_PTR(gr->B_o);
    CHECK_PTR(gr->A_gu);
    CHECK_PTR(gr->B_g);
    CHECK_PTR(gr->B_u);
    CHECK_PTR(gr->A_dn);
    CHECK_PTR(gr->B_dn);
  }
  if (pre) {
    CHECK_PTR(dQ);
    CHECK_PTR(dK);
    CHECK_PTR(dV);
    CHECK_PTR(dX);
    CHECK_PTR(gr->gamma1);
    CHECK_PTR(gr->A_qkv);
    CHECK_PTR(gr->B_q);
    CHECK_PTR(gr->B_k);
    CHECK_PTR(gr->B_v);
  }
  const size_t need = carve_bwd(s, nullptr, nullptr);
  RUN(check_ws(ws, ws_bytes, need));
  BwdWs W;
  carve_bwd(s, ws, &W);

  const int dt = s->dtype;
  const size_t e = elem_size(dt);
  const int T = (int)s->T, d = (int)s->d, r = (int)s->r, F = (int)s->d_ff;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float inv_D = 1.0f / (float)s->d_norm;

  int cs_tiles = 0;  // M-tiles of the RMSNorm backward (rows of its column partials)
  // Weight gradients that run together, one launch per group, when their
  // tiles fit the pipelined engine: dA_gu, dB_o, dA_o once do_r exists, and
  // (whole backward in one call) dB_dn, held back to run beside dA_qkv.
  const lr::GemmDesc dB_dn = tn_desc(d, r, T, dY, d, sv->d_r, r, gr->B_dn, nullptr);
  lr::GemmDesc last2[2] = {tn_desc(3 * r, d, T, W.dqs, 3 * r, X, d, gr->A_qkv, w->gamma1), dB_dn};
  const bool late_dbdn = stage == LR_STAGE_ALL && lr::wgrad_multi_ok(dt, last2, 2);
  if (post) {
    if (W.tB_dn) {
      const lr::TransposeJob jobs[7] = {
          {w->B_dn, r, d, r, W.tB_dn, d},        {w->A_dn, F, r, F, W.tA_dn, r},
          {w->B_g, r, F, r, W.tB_g, F},          {w->B_u, r, F, r, W.tB_u, F},
          {w->A_gu, d, 2 * r, d, W.tA_gu, 2 * r}, {w->B_o, r, d, r, W.tB_o, d},
          {w->A_o, d, r, d, W.tA_o, r}};
      ProfScope ps("transpose B_dn, A_dn, B_g, B_u, A_gu, B_o, A_o", st,
                   2.0 * e * r * (5.0 * d + 3.0 * F), true);
      hipError_t he = launch_rep(ps, [&] { return lr::run_transpose_bf16(jobs, 7, st); });
      if (he != hipSuccess) return hip_fail(he, "weight transposes");
    }
    // dB_dn = dY^T d_r
    if (!late_dbdn) RUN(wgrad(dt, dB_dn, 1, W, st, "dB_dn", "dB_dn split-K sum"));
    // dd_r = dY B_dn
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = r;
      g.K = d;
      g.a[0] = dY;
      g.lda[0] = d;
      g.b[0] = w->B_dn;
      g.ldb[0] = r;
      g.c[0] = W.dd_r;
      g.ldc[0] = r;
      const void* wt[1] = {W.tB_dn};
      RUN(nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, g, wt, 1, st, "dd_r"));
    }
    // Recompute g, u and dm = dd_r A_dn in one tile; m, dg, du out.
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = F;
      g.K = r;
      g.a[0] = sv->gu_r;
      g.lda[0] = 2 * r;
      g.b[0] = w->B_g;
      g.ldb[0] = r;
      g.a[1] = B(sv->gu_r, r, e);
      g.lda[1] = 2 * r;
      g.b[1] = w->B_u;
      g.ldb[1] = r;
      g.a[2] = W.dd_r;
      g.lda[2] = r;
      g.b[2] = w->A_dn;
      g.ldb[2] = F;
      g.c[0] = W.m;
      g.ldc[0] = F;
      g.c[1] = W.dg;
      g.ldc[1] = F;
      g.c[2] = W.du;
      g.ldc[2] = F;
      // On the pipelined engine dm = dd_r A_dn is its own GEMM (written into
      // du's buffer, on whichever engine takes its shape), then one two-pair
      // tile recomputes g and u and reads dm in its epilogue, which
      // overwrites dm with du element by element. The two-pair tile takes
      // exactly the shapes the forward's gate/up tile takes, so the gate is
      // rounded alike in both (bitwise equal m); other shapes run both on the
      // general engine.
      lr::GemmDesc dmg;
      dmg.M = T;
      dmg.N = F;
      dmg.K = r;
      dmg.a[0] = W.dd_r;
      dmg.lda[0] = r;
      dmg.b[0] = w->A_dn;
      dmg.ldb[0] = F;
      dmg.c[0] = W.du;
      dmg.ldc[0] = F;
      lr::GemmDesc two = g;
      two.a[2] = nullptr;
      two.b[2] = nullptr;
      two.res = W.du;
      two.ldres = F;
      if (lr::uses_engine2(lr::OP_SWIGLU_BWD2, dt, two, 1)) {
        const void* wt[1] = {W.tA_dn};
        RUN(nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, dmg, wt, 1, st, "dm = dd_r A_dn"));
        RUN(gemm(lr::OP_SWIGLU_BWD2, dt, two, 1, st, "SwiGLU recompute + backward"));
      } else {
        RUN(gemm(lr::OP_SWIGLU_BWD, dt, g, 1, st, "SwiGLU recompute + backward"));
      }
    }
    // dA_dn = dd_r^T m
    {
      lr::GemmDesc g;
      g.M = r;
      g.N = F;
      g.K = T;
      g.a[0] = W.dd_r;
      g.lda[0] = r;
      g.b[0] = W.m;
      g.ldb[0] = F;
      g.c[0] = gr->A_dn;
      g.ldc[0] = F;
      RUN(wgrad(dt, g, 1, W, st, "dA_dn", "dA_dn split-K sum"));
    }
    // dB_g = dg^T g_r, dB_u = du^T u_r (grouped)
    {
      lr::GemmDesc g;
      g.M = F;
      g.N = r;
      g.K = T;
      g.a[0] = W.dg;
      g.lda[0] = F;
      g.b[0] = sv->gu_r;
      g.ldb[0] = 2 * r;
      g.c[0] = gr->B_g;
      g.ldc[0] = r;
      g.a[1] = W.du;
      g.lda[1] = F;
      g.b[1] = B(sv->gu_r, r, e);
      g.ldb[1] = 2 * r;
      g.c[1] = gr->B_u;
      g.ldc[1] = r;
      RUN(wgrad(dt, g, 2, W, st, "dB_g, dB_u", "dB_g, dB_u split-K sum"));
    }
    // dgus = [dg B_g | du B_u] / rms2 (grouped, row-scaled)
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = r;
      g.K = F;
      g.a[0] = W.dg;
      g.lda[0] = F;
      g.b[0] = w->B_g;
      g.ldb[0] = r;
      g.c[0] = W.dgus;
      g.ldc[0] = 2 * r;
      g.a[1] = W.du;
      g.lda[1] = F;
      g.b[1] = w->B_u;
      g.ldb[1] = r;
      g.c[1] = Bm(W.dgus, r, e);
      g.ldc[1] = 2 * r;
      g.rowdiv = sv->rms2;
      const void* wt[2] = {W.tB_g, W.tB_u};
      RUN(nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, g, wt, 2, st, "dgu_r"));
    }
    // coef2 = (dgus . gu_r) / (rms2 D)
    {
      ProfScope ps("row dot 2", st, (double)e * 2.0 * T * 2 * r + 8.0 * T, true);
      hipError_t he = launch_rep(ps, [&] {
        return lr::run_rowdot_coef(dt, W.dgus, 2 * r, sv->gu_r, 2 * r, 2 * r, sv->rms2, inv_D,
                                   W.coef2, T, st);
      });
      if (he != hipSuccess) return hip_fail(he, "row dot 2");
    }
    // Recompute h = X + o_r B_o^T.
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = d;
      g.K = r;
      g.a[0] = sv->o_r;
      g.lda[0] = r;
      g.b[0] = w->B_o;
      g.ldb[0] = r;
      g.c[0] = W.h;
      g.ldc[0] = d;
      g.res = X;
      g.ldres = d;
      RUN(gemm(lr::OP_NT_STORE, dt, g, 1, st, "recompute h"));
    }
    // dh = dY + gamma2 * (dgus A_gu) - coef2 * h; dgamma2 partials.
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = d;
      g.K = 2 * r;
      g.a[0] = W.dgus;
      g.lda[0] = 2 * r;
      g.b[0] = w->A_gu;
      g.ldb[0] = d;
      g.c[0] = W.dh;
      g.ldc[0] = d;
      g.res = dY;
      g.ldres = d;
      g.hsrc = W.h;
      g.ldh = d;
      g.colscale = w->gamma2;
      g.rowcoef = W.coef2;
      g.colsum = W.colpart;
      const void* wt[1] = {W.tA_gu};
      int op_run = lr::OP_NN_RMSBWD;
      lr::GemmDesc used;
      RUN(nn_or_nt(lr::OP_NN_RMSBWD, lr::OP_NT_RMSBWD, dt, g, wt, 1, st, "RMSNorm-2 backward",
                   &op_run, &used));
      const int bm = lr::gemm_tile_m_used(op_run, dt, used, 1);
      cs_tiles = (T + bm - 1) / bm;
    }
    // do_r = dh B_o
    auto do_r_gemm = [&]() {
      lr::GemmDesc g;
      g.M = T;
      g.N = r;
      g.K = d;
      g.a[0] = W.dh;
      g.lda[0] = d;
      g.b[0] = w->B_o;
      g.ldb[0] = r;
      g.c[0] = W.do_r;
      g.ldc[0] = r;
      const void* wt[1] = {W.tB_o};
      return nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, g, wt, 1, st, "do_r");
    };
    // dA_gu = gamma2 * (dgus^T h), dB_o = dh^T o_r, dA_o = do_r^T O. On the
    // pipelined engine the (first) launch also sums the RMSNorm backward's
    // per-tile column partials into dgamma2 as a side job after its own
    // outputs; otherwise a kernel of its own does.
    lr::GemmDesc mid3[3] = {tn_desc(2 * r, d, T, W.dgus, 2 * r, W.h, d, gr->A_gu, w->gamma2),
                            tn_desc(d, r, T, W.dh, d, sv->o_r, r, gr->B_o, nullptr),
                            tn_desc(r, d, T, W.do_r, r, O_attn, d, gr->A_o, nullptr)};
    const bool side2 = lr::uses_engine2(lr::OP_TN_WGRAD, dt, mid3[0], 1);
    if (side2) {
      mid3[0].cs_part = W.colpart;
      mid3[0].cs_rows = cs_tiles;
      mid3[0].cs_n = d;
      mid3[0].cs_out = gr->gamma2;
    }
    if (lr::wgrad_multi_ok(dt, mid3, 3)) {
      RUN(do_r_gemm());
      static const char* const sums[3] = {"dA_gu split-K sum", "dB_o split-K sum",
                                          "dA_o split-K sum"};
      RUN(wgrad_multi(dt, mid3, 3, W, st, "dA_gu, dB_o, dA_o", sums));
    } else {
      RUN(wgrad(dt, mid3[0], 1, W, st, "dA_gu", "dA_gu split-K sum"));
      RUN(wgrad(dt, mid3[1], 1, W, st, "dB_o", "dB_o split-K sum"));
      RUN(do_r_gemm());
      RUN(wgrad(dt, mid3[2], 1, W, st, "dA_o", "dA_o split-K sum"));
    }
    if (!side2) {
      ProfScope ps("dgamma2 column sum", st, 4.0 * cs_tiles * d + 4.0 * d, true);
      hipError_t he = launch_rep(
          ps, [&] { return lr::run_colsum(W.colpart, cs_tiles, d, gr->gamma2, st); });
      if (he != hipSuccess) return hip_fail(he, "dgamma2");
    }
    // dO = do_r A_o
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = d;
      g.K = r;
      g.a[0] = W.do_r;
      g.lda[0] = r;
      g.b[0] = w->A_o;
      g.ldb[0] = d;
      g.c[0] = dO_attn;
      g.ldc[0] = d;
      const void* wt[1] = {W.tA_o};
      RUN(nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, g, wt, 1, st, "dO"));
    }
  }

  if (pre) {
    if (W.tB_q) {
      const lr::TransposeJob jobs[4] = {{w->B_q, r, d, r, W.tB_q, d},
                                        {w->B_k, r, d, r, W.tB_k, d},
                                        {w->B_v, r, d, r, W.tB_v, d},
                                        {w->A_qkv, d, 3 * r, d, W.tA_qkv, 3 * r}};
      ProfScope ps("transpose B_q, B_k, B_v, A_qkv", st, 2.0 * e * 6.0 * r * d, true);
      hipError_t he = launch_rep(ps, [&] { return lr::run_transpose_bf16(jobs, 4, st); });
      if (he != hipSuccess) return hip_fail(he, "weight transposes");
    }
    const void* dQKV[3] = {dQ, dK, dV};
    const void* Bs[3] = {w->B_q, w->B_k, w->B_v};
    float* dBs[3] = {gr->B_q, gr->B_k, gr->B_v};
    // dB_{q,k,v} = d{Q,K,V}^T {q,k,v}_r (grouped)
    {
      lr::GemmDesc g;
      g.M = d;
      g.N = r;
      g.K = T;
      for (int i = 0; i < 3; ++i) {
        g.a[i] = dQKV[i];
        g.lda[i] = d;
        g.b[i] = B(sv->qkv_r, (int64_t)i * r, e);
        g.ldb[i] = 3 * r;
        g.c[i] = dBs[i];
        g.ldc[i] = r;
      }
      RUN(wgrad(dt, g, 3, W, st, "dB_q, dB_k, dB_v", "dB_q, dB_k, dB_v split-K sum"));
    }
    // dqs = [dQ B_q | dK B_k | dV B_v] / rms1 (grouped, row-scaled)
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = r;
      g.K = d;
      for (int i = 0; i < 3; ++i) {
        g.a[i] = dQKV[i];
        g.lda[i] = d;
        g.b[i] = Bs[i];
        g.ldb[i] = r;
        g.c[i] = Bm(W.dqs, (int64_t)i * r, e);
        g.ldc[i] = 3 * r;
      }
      g.rowdiv = sv->rms1;
      const void* wt[3] = {W.tB_q, W.tB_k, W.tB_v};
      RUN(nn_or_nt(lr::OP_NN_STORE, lr::OP_NT_STORE, dt, g, wt, 3, st, "dqkv_r"));
    }
    // coef1 = (dqs . qkv_r) / (rms1 D)
    {
      ProfScope ps("row dot 1", st, (double)e * 2.0 * T * 3 * r + 8.0 * T, true);
      hipError_t he = launch_rep(ps, [&] {
        return lr::run_rowdot_coef(dt, W.dqs, 3 * r, sv->qkv_r, 3 * r, 3 * r, sv->rms1, inv_D,
                                   W.coef1, T, st);
      });
      if (he != hipSuccess) return hip_fail(he, "row dot 1");
    }
    // dX = dh + gamma1 * (dqs A_qkv) - coef1 * X; dgamma1 partials.
    {
      lr::GemmDesc g;
      g.M = T;
      g.N = d;
      g.K = 3 * r;
      g.a[0] = W.dqs;
      g.lda[0] = 3 * r;
      g.b[0] = w->A_qkv;
      g.ldb[0] = d;
      g.c[0] = dX;
      g.ldc[0] = d;
      g.res = W.dh;
      g.ldres = d;
      g.hsrc = X;
      g.ldh = d;
      g.colscale = w->gamma1;
      g.rowcoef = W.coef1;
      g.colsum = W.colpart;
      const void* wt[1] = {W.tA_qkv};
      int op_run = lr::OP_NN_RMSBWD;
      lr::GemmDesc used;
      RUN(nn_or_nt(lr::OP_NN_RMSBWD, lr::OP_NT_RMSBWD, dt, g, wt, 1, st, "RMSNorm-1 backward",
                   &op_run, &used));
      const int bm = lr::gemm_tile_m_used(op_run, dt, used, 1);
      cs_tiles = (T + bm - 1) / bm;
    }
    // dA_qkv = gamma1 * (dqs^T X) (with dB_dn beside it when held back); on
    // the pipelined engine the launch also sums the RMSNorm backward's
    // per-tile column partials into dgamma1, else a kernel of its own does.
    const bool side1 = lr::uses_engine2(lr::OP_TN_WGRAD, dt, last2[0], 1);
    if (side1) {
      last2[0].cs_part = W.colpart;
      last2[0].cs_rows = cs_tiles;
      last2[0].cs_n = d;
      last2[0].cs_out = gr->gamma1;
    }
    if (late_dbdn) {
      static const char* const sums[2] = {"dA_qkv split-K sum", "dB_dn split-K sum"};
      RUN(wgrad_multi(dt, last2, 2, W, st, "dA_qkv, dB_dn", sums));
    } else {
      RUN(wgrad(dt, last2[0], 1, W, st, "dA_qkv", "dA_qkv split-K sum"));
    }
    if (!side1) {
      ProfScope ps("dgamma1 column sum", st, 4.0 * cs_tiles * d + 4.0 * d, true);
      hipError_t he = launch_rep(
          ps, [&] { return lr::run_colsum(W.colpart, cs_tiles, d, gr->gamma1, st); });
      if (he != hipSuccess) return hip_fail(he, "dgamma1");
    }
  }
  return LR_OK;
}

namespace {
// Validates a grouped call and builds its descriptor and operation.
int grouped_desc(int32_t G, const lr_gemm_pair* pairs, int32_t dtype, int32_t layout,
                 int32_t epilogue, lr::GemmDesc& g, int& op, int& groups);
}  // namespace

int lr_grouped_lowrank_gemm(int32_t G, const lr_gemm_pair* pairs, int32_t dtype, int32_t layout,
                            int32_t epilogue, void* stream) {
  lr::GemmDesc g;
  int op = 0, groups = 0;
  RUN(grouped_desc(G, pairs, dtype, layout, epilogue, g, op, groups));
  return gemm(op, dtype, g, groups, static_cast<hipStream_t>(stream), "grouped low-rank GEMM");
}

size_t lr_grouped_lowrank_gemm_workspace_bytes(int32_t G, const lr_gemm_pair* pairs,
                                               int32_t dtype, int32_t layout) {
  lr::GemmDesc g;
  int op = 0, groups = 0;
  if (grouped_desc(G, pairs, dtype, layout, LR_EPI_NONE, g, op, groups)) return 0;
  if (op != lr::OP_TN_WGRAD) return 0;
  return lr::wgrad_part_bytes(dtype, g, groups);
}

int lr_grouped_lowrank_gemm_ws(int32_t G, const lr_gemm_pair* pairs, int32_t dtype,
                               int32_t layout, int32_t epilogue, void* ws, size_t ws_bytes,
                               void* stream) {
  lr::GemmDesc g;
  int op = 0, groups = 0;
  RUN(grouped_desc(G, pairs, dtype, layout, epilogue, g, op, groups));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t need = op == lr::OP_TN_WGRAD ? lr::wgrad_part_bytes(dtype, g, groups) : 0;
  if (need == 0) return gemm(op, dtype, g, groups, st, "grouped low-rank GEMM");
  RUN(check_ws(ws, ws_bytes, need));
  return wgrad(dtype, g, groups, ws, ws_bytes, st, "grouped low-rank GEMM",
               "grouped low-rank GEMM split-K sum");
}

namespace {
int grouped_desc(int32_t G, const lr_gemm_pair* pairs, int32_t dtype, int32_t layout,
                 int32_t epilogue, lr::GemmDesc& g, int& op, int& groups) {
  if (dtype != LR_F32 && dtype != LR_BF16)
    return fail(LR_ERR_INVALID_ARG, "dtype %d is neither LR_F32 nor LR_BF16", dtype);
  if (G < 1 || G > 3) return fail(LR_ERR_INVALID_ARG, "G = %d is out of range [1, 3]", G);
  if (!pairs) return fail(LR_ERR_INVALID_ARG, "pairs is NULL");
  if (layout < LR_LAYOUT_NT || layout > LR_LAYOUT_TN)
    return fail(LR_ERR_INVALID_ARG, "layout %d is not an lr_layout", layout);
  if (epilogue < LR_EPI_NONE || epilogue > LR_EPI_ROW_SCALE)
    return fail(LR_ERR_INVALID_ARG, "epilogue %d is not an lr_epilogue", epilogue);
  const int v = vec_elems(dtype);
  const lr_gemm_pair& p0 = pairs[0];
  for (int i = 0; i < G; ++i) {
    const lr_gemm_pair& p = pairs[i];
    if (p.M < 1 || p.N < 1 || p.K < 1 || p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim)
      return fail(LR_ERR_INVALID_ARG, "pair %d: M, N, K must be in [1, 2^30]", i);
    if (p.M != p0.M || p.N != p0.N || p.K != p0.K)
      return fail(LR_ERR_UNSUPPORTED, "pair %d: all pairs of a call must have equal M, N, K", i);
    if (check_ptr(p.X, "X") || check_ptr(p.W, "W") || check_ptr(p.Y, "Y"))
      return fail(LR_ERR_INVALID_ARG, "pair %d: %s", i, g_err.c_str());
    const int64_t minx = layout == LR_LAYOUT_TN ? p.M : p.K;
    const int64_t minw = layout == LR_LAYOUT_NT ? p.K : p.N;
    if (p.ldx < minx || p.ldw < minw || p.ldy < p.N)
      return fail(LR_ERR_INVALID_ARG, "pair %d: leading dimension smaller than the row", i);
    if (p.ldx % v || p.ldw % v || p.ldy % v)
      return fail(LR_ERR_INVALID_ARG, "pair %d: leading dimensions must be multiples of %d", i,
                  v);
    if (epilogue == LR_EPI_ADD_RESIDUAL) {
      if (check_ptr(p.aux, "aux")) return fail(LR_ERR_INVALID_ARG, "pair %d: %s", i, g_err.c_str());
      if (p.ldaux < p.N || p.ldaux % v)
        return fail(LR_ERR_INVALID_ARG, "pair %d: bad residual leading dimension", i);
    }
    if (epilogue == LR_EPI_ROW_SCALE && !p.aux)
      return fail(LR_ERR_INVALID_ARG, "pair %d: row scale aux is NULL", i);
  }
  if (layout == LR_LAYOUT_TN && epilogue != LR_EPI_NONE)
    return fail(LR_ERR_UNSUPPORTED, "the TN layout takes no epilogue");
  if (epilogue == LR_EPI_SWIGLU_PAIR && (G != 2 || layout != LR_LAYOUT_NT))
    return fail(LR_ERR_UNSUPPORTED, "LR_EPI_SWIGLU_PAIR needs G = 2 and the NT layout");
  if ((epilogue == LR_EPI_ADD_RESIDUAL || epilogue == LR_EPI_ROW_SCALE) && G > 1) {
    for (int i = 1; i < G; ++i)
      if (pairs[i].aux != p0.aux || pairs[i].ldaux != p0.ldaux)
        return fail(LR_ERR_UNSUPPORTED, "grouped epilogue inputs must be shared by all pairs");
    if (epilogue == LR_EPI_ADD_RESIDUAL)
      return fail(LR_ERR_UNSUPPORTED, "the residual epilogue takes G = 1");
  }
  g = lr::GemmDesc();
  g.M = (int)p0.M;
  g.N = (int)p0.N;
  g.K = (int)p0.K;
  for (int i = 0; i < G; ++i) {
    g.a[i] = pairs[i].X;
    g.lda[i] = pairs[i].ldx;
    g.b[i] = pairs[i].W;
    g.ldb[i] = pairs[i].ldw;
    g.c[i] = pairs[i].Y;
    g.ldc[i] = pairs[i].ldy;
  }
  if (epilogue == LR_EPI_ADD_RESIDUAL) {
    g.res = p0.aux;
    g.ldres = p0.ldaux;
  } else if (epilogue == LR_EPI_ROW_SCALE) {
    g.rowdiv = static_cast<const float*>(p0.aux);
  }
  groups = G;
  if (epilogue == LR_EPI_SWIGLU_PAIR) {
    op = lr::OP_NT_SWIGLU;
    groups = 1;
  } else if (layout == LR_LAYOUT_NT) {
    op = lr::OP_NT_STORE;
  } else if (layout == LR_LAYOUT_NN) {
    op = lr::OP_NN_STORE;
  } else {
    op = lr::OP_TN_WGRAD;
  }
  return LR_OK;
}
}  // namespace

size_t lr_online_rmsnorm_gemm_workspace_bytes(int64_t N, int64_t d, int32_t dtype) {
  if ((dtype != LR_F32 && dtype != LR_BF16) || N < 1 || d < 1) return 0;
  return (size_t)N * (size_t)d * elem_size(dtype);
}

namespace {
// Argument checks of the Online RMSNorm GEMM (no HIP call).
int check_orms(int64_t T, int64_t d, int64_t N, int32_t n_panels, int64_t d_norm, float eps,
               const void* X, int64_t ldx, const void* gamma, const void* A, int64_t lda,
               void* out, int64_t ldo, float* rms_out, float* ss_out, int32_t emit_partial,
               int32_t dtype) {
  if (dtype != LR_F32 && dtype != LR_BF16)
    return fail(LR_ERR_INVALID_ARG, "dtype %d is neither LR_F32 nor LR_BF16", dtype);
  if (T < 1 || d < 1 || N < 1 || d_norm < 1 || T > kMaxDim || d > kMaxDim || N > kMaxDim ||
      d_norm > kMaxDim)
    return fail(LR_ERR_INVALID_ARG, "T, d, N, d_norm must be in [1, 2^30]");
  const int v = vec_elems(dtype);
  if (d % v) return fail(LR_ERR_INVALID_ARG, "d must be a multiple of %d for this dtype", v);
  if (ldx < d || lda < d || ldo < N || ldx % v || lda % v || ldo % v)
    return fail(LR_ERR_INVALID_ARG, "leading dimensions must cover the row and be multiples of %d",
                v);
  if (n_panels < 1 || n_panels > 8)
    return fail(LR_ERR_INVALID_ARG, "n_panels = %d is out of range [1, 8]", n_panels);
  if (n_panels > 1 && (d % n_panels || (d / n_panels) % 64))
    return fail(d % n_panels ? LR_ERR_INVALID_ARG : LR_ERR_UNSUPPORTED,
                "d = %lld does not split into %d panels of a multiple of 64 columns",
                (long long)d, n_panels);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(LR_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (emit_partial != 0 && emit_partial != 1)
    return fail(LR_ERR_INVALID_ARG, "emit_partial must be 0 or 1");
  CHECK_PTR(X);
  CHECK_PTR(A);
  CHECK_PTR(out);
  if (gamma) CHECK_PTR(gamma);
  if (rms_out && (reinterpret_cast<uintptr_t>(rms_out) & 3u))
    return fail(LR_ERR_INVALID_ARG, "rms_out is not 4-byte aligned");
  if (ss_out && (reinterpret_cast<uintptr_t>(ss_out) & 3u))
    return fail(LR_ERR_INVALID_ARG, "ss_out is not 4-byte aligned");
  return LR_OK;
}

// The launches of the Online RMSNorm GEMM once its arguments are checked:
// with gamma, the gamma-folded copy of A goes to `fold` (N x d elements).
int run_orms(int64_t T, int64_t d, int64_t N, int32_t n_panels, int64_t d_norm, float eps,
             const void* X, int64_t ldx, const void* gamma, const void* A, int64_t lda, void* out,
             int64_t ldo, float* rms_out, float* ss_out, int32_t emit_partial, int32_t dtype,
             void* fold, hipStream_t st) {
  const void* Aeff = A;
  int64_t ldaeff = lda;
  if (gamma) {
    ProfScope ps("fold gamma", st, (double)elem_size(dtype) * (2.0 * N * d + d), true);
    hipError_t he = launch_rep(
        ps, [&] { return lr::run_fold_gamma(dtype, A, lda, gamma, fold, (int)N, (int)d, st); });
    if (he != hipSuccess) return hip_fail(he, "fold gamma");
    Aeff = fold;
    ldaeff = d;
  }
  lr::GemmDesc g;
  g.M = (int)T;
  g.N = (int)N;
  g.K = (int)d;
  g.a[0] = X;
  g.lda[0] = ldx;
  g.b[0] = Aeff;
  g.ldb[0] = ldaeff;
  g.c[0] = out;
  g.ldc[0] = ldo;
  g.rms_out = emit_partial ? nullptr : rms_out;
  g.ss_out = ss_out;
  g.n_panels = n_panels;
  g.panel_width = (int)(d / n_panels);
  g.inv_D = 1.0f / (float)d_norm;
  g.eps = eps;
  g.emit_partial = emit_partial;
  return gemm(lr::OP_NT_ORMS, dtype, g, 1, st, "Online RMSNorm GEMM");
}

// Scratch of the no-allocation variant: the gamma-folded copy of A. Each
// GPU the library runs on holds its own copy of this array until the
// process ends. In host code `scratch` names a host-side stand-in, never
// the device memory: the device address comes from hipGetSymbolAddress,
// once per device, and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the
// first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LR_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LR_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LR_OK;
}
}  // namespace

int lr_online_rmsnorm_gemm(int64_t T, int64_t d, int64_t N, int32_t n_panels, int64_t d_norm,
                           float eps, const void* X, int64_t ldx, const void* gamma,
                           const void* A, int64_t lda, void* out, int64_t ldo, float* rms_out,
                           float* ss_out, int32_t emit_partial, int32_t dtype, void* ws,
                           size_t ws_bytes, void* stream) {
  RUN(check_orms(T, d, N, n_panels, d_norm, eps, X, ldx, gamma, A, lda, out, ldo, rms_out, ss_out,
                 emit_partial, dtype));
  if (gamma) {
    const size_t need = (size_t)N * (size_t)d * elem_size(dtype);
    if (ws_bytes < need || !ws)
      return fail(LR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  ws_bytes, need);
    if (!aligned16(ws)) return fail(LR_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  }
  return run_orms(T, d, N, n_panels, d_norm, eps, X, ldx, gamma, A, lda, out, ldo, rms_out, ss_out,
                  emit_partial, dtype, ws, static_cast<hipStream_t>(stream));
}

size_t lr_online_rmsnorm_gemm_noalloc_max_bytes(void) { return kScratchBytes; }

int lr_online_rmsnorm_gemm_noalloc(int64_t T, int64_t d, int64_t N, int32_t n_panels,
                                   int64_t d_norm, float eps, const void* X, int64_t ldx,
                                   const void* gamma, const void* A, int64_t lda, void* out,
                                   int64_t ldo, float* rms_out, float* ss_out,
                                   int32_t emit_partial, int32_t dtype, void* stream) {
  RUN(check_orms(T, d, N, n_panels, d_norm, eps, X, ldx, gamma, A, lda, out, ldo, rms_out, ss_out,
                 emit_partial, dtype));
  void* fold = nullptr;
  if (gamma) {
    const size_t need = (size_t)N * (size_t)d * elem_size(dtype);
    if (need > kScratchBytes)
      return fail(LR_ERR_WORKSPACE,
                  "the gamma-folded A (N x d = %lld x %lld) needs %zu bytes, more than the %zu "
                  "bytes of built-in scratch of the no-allocation variant",
                  (long long)N, (long long)d, need, kScratchBytes);
    RUN(scratch_address(&fold));
  }
  return run_orms(T, d, N, n_panels, d_norm, eps, X, ldx, gamma, A, lda, out, ldo, rms_out, ss_out,
                  emit_partial, dtype, fold, static_cast<hipStream_t>(stream));
}

}  // extern "C"
