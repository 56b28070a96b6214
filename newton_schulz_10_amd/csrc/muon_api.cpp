// C ABI of libmuon (include/muon.h): argument validation, planning and the
// launch sequence of the batched Muon step on the caller's HIP stream.
//
// Paper: arXiv:2609.21594 section 6.2 (one step: momentum update, batched
// NS, local update), section 6.6 (shape groups fused into one batched NS
// with one workspace per batched invocation, 2^29-element batch cap) and
// section 6.7 (largest matrices first).
//
// Launch sequence per batch, all asynchronous on `stream`:
//   momentum   (per chunk of <= 128 matrices)  -> X0 = u (wide, padded), partials
//   finalize                                   -> s_i = 1/(||u_i||_F + eps)
//   ns_steps x { gram, poly, update }          -> X_k (s_i folded into step 1)
//   apply      (per chunk)                     -> p' (or out)
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "muon.h"
#include "plan.h"

namespace muon {
namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  std::string m = std::string(where) + ": " + hipGetErrorString(e);
  g_err = m;
  return e == hipErrorOutOfMemory ? MUON_ERR_OUT_OF_MEMORY : MUON_ERR_HIP;
}

// ---- stream-ordered workspace from a library-owned pool per device ------

std::mutex g_pool_mu;
std::map<int, hipMemPool_t> g_pools;

hipError_t get_pool(int dev, hipMemPool_t* out) {
  std::lock_guard<std::mutex> lk(g_pool_mu);
  auto it = g_pools.find(dev);
  if (it != g_pools.end()) { *out = it->second; return hipSuccess; }
  hipMemPoolProps props;
  std::memset(&props, 0, sizeof(props));
  props.allocType = hipMemAllocationTypePinned;
  props.handleTypes = hipMemHandleTypeNone;
  props.location.type = hipMemLocationTypeDevice;
  props.location.id = dev;
  hipMemPool_t pool;
  hipError_t e = hipMemPoolCreate(&pool, &props);
  if (e != hipSuccess) return e;
  // Keep freed workspace reserved in the pool between steps.
  uint64_t thr = ~0ull;
  e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
  if (e != hipSuccess) return e;
  g_pools[dev] = pool;
  *out = pool;
  return hipSuccess;
}

// ---- optional per-launch event timing -----------------------------------

struct Pending {
  std::string kind;
  hipEvent_t e0, e1;
  double flops, bytes;
};
struct ProfTotal { int launches = 0; double ms = 0, flops = 0, bytes = 0; };

std::mutex g_prof_mu;
bool g_prof_on = false;
// MUON_PROFILE=1 in the environment turns the per-launch timing on from the
// start (as muon_profile_enable(1) would).
const bool g_prof_env = [] {
  const char* v = std::getenv("MUON_PROFILE");
  if (v && v[0] == '1') g_prof_on = true;
  return true;
}();
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free_events;
std::map<std::string, ProfTotal> g_totals;
std::vector<std::string> g_kind_order;

// Events for the timing come from a free list (g_prof_mu held). A failed
// event call clears HIP's last-error state, which the kernel launchers
// read after each launch: profiling must never fail a step.
hipEvent_t take_event() {
  if (!g_free_events.empty()) { hipEvent_t e = g_free_events.back(); g_free_events.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}
void give_event(hipEvent_t e) {
  if (e) g_free_events.push_back(e);
}

struct ProfScope {
  bool on = false;
  Pending p;
  hipStream_t s;
  ProfScope(const char* kind, double flops, double bytes, hipStream_t st) : s(st) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    p.kind = kind; p.flops = flops; p.bytes = bytes;
    p.e0 = take_event(); p.e1 = take_event();
    on = p.e0 && p.e1 && hipEventRecord(p.e0, s) == hipSuccess;
    if (!on) {
      (void)hipGetLastError();
      give_event(p.e0);
      give_event(p.e1);
    }
  }
  ~ProfScope() {
    if (!on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (hipEventRecord(p.e1, s) == hipSuccess) {
      g_pending.push_back(p);
    } else {
      (void)hipGetLastError();
      give_event(p.e0);
      give_event(p.e1);
    }
  }
};

// ---- named host ranges ------------------------------------------------------

// A roctx range around a phase of the call (shown by `rocprofv3
// --marker-trace`; a no-op when no tool is attached). Popped on every exit.
struct PhaseRange {
  explicit PhaseRange(const std::string& name) { roctxRangePushA(name.c_str()); }
  ~PhaseRange() { roctxRangePop(); }
  PhaseRange(const PhaseRange&) = delete;
  PhaseRange& operator=(const PhaseRange&) = delete;
};

// ---- the launch sequence --------------------------------------------------

struct MatRef {
  void* param;        // param (step) or output (orthogonalize)
  const void* src;    // grad (step) or input (orthogonalize)
  float* mom;         // momentum (step) or nullptr
  int rows, cols;
  int ld;             // row stride in elements of param, src and mom (>= cols)
};

// Element type the NS iteration runs in: options.ns_dtype, or the tensors'.
muon_dtype ns_type(const muon_options& o, muon_dtype dtype) {
  return o.ns_dtype < 0 ? dtype : static_cast<muon_dtype>(o.ns_dtype);
}

double update_scale(const muon_options& o, int rows, int cols) {
  switch (o.scale_rule) {
    case 0: return (double)o.rms_target * std::sqrt((double)std::max(rows, cols));
    case 1: return std::sqrt(std::max(1.0, (double)rows / (double)cols));
    default: return 1.0;
  }
}

// Compute units the batch split is fitted to: options.compute_units, or
// for -1 the current device's count (0, i.e. no fitting, when no device is
// visible).
int fit_units(const muon_options& o) {
  if (o.compute_units >= 0) return o.compute_units;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

// The launch sequence of one call. With use_static, the workspace is the
// current device's static array (muon_step_noalloc: batches sized to fit
// it, nothing allocated or freed); otherwise one stream-ordered allocation
// from the library's pool, freed stream-ordered at the end.
int run(const std::vector<MatRef>& mats, float lr, float beta, int ns_steps, muon_dtype dtype,
        const muon_options& o, bool orthogonalize_only, hipStream_t stream, bool use_static = false) {
  if (mats.empty()) return MUON_OK;
  PhaseRange call_range(std::string(orthogonalize_only ? "muon_orthogonalize" : "muon_step") + " (" +
                   std::to_string(mats.size()) + " matrices)");
  const int num = (int)mats.size();
  std::vector<int> rows(num), cols(num);
  for (int i = 0; i < num; ++i) { rows[i] = mats[i].rows; cols[i] = mats[i].cols; }
  // Tensors (params, grads, in/out) are `dtype`; the NS iterate and its
  // workspace are `ns`, which also sets the plan's padding and layout.
  const muon_dtype ns = ns_type(o, dtype);
  Plan plan;
  std::string err;
  const int* set_of = o.num_coeff_sets > 0 ? o.coeff_set_of : nullptr;
  hipError_t e = hipSuccess;
  void* ws = nullptr;
  size_t static_bytes = 0;
  if (use_static) {
    e = static_workspace(&ws, &static_bytes);
    if (e != hipSuccess) return hip_fail(e, "static workspace (hipGetSymbolAddress)");
  }
  int rc = build_plan(rows.data(), cols.data(), num, ns, o.batch_cap_elems, use_static ? 0 : fit_units(o), plan,
                      err, set_of, o.num_coeff_sets, static_bytes);
  if (rc) return fail(rc, use_static ? err + " (the static workspace of muon_step_noalloc)" : err);

  if (!use_static) {
    if (const char* f = std::getenv("MUON_TEST_FAIL_ALLOC"))
      if (f[0] == '1') return fail(MUON_ERR_OUT_OF_MEMORY, "workspace allocation failed (MUON_TEST_FAIL_ALLOC=1)");
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipMemPool_t pool;
    e = get_pool(dev, &pool);
    if (e != hipSuccess) return hip_fail(e, "hipMemPoolCreate");
    e = hipMallocFromPoolAsync(&ws, plan.workspace_bytes, pool, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MUON_ERR_OUT_OF_MEMORY, std::string("workspace allocation of ") +
                  std::to_string(plan.workspace_bytes) + " bytes failed: " + hipGetErrorString(e));
    }
  }

  const bool bf16 = ns == MUON_BF16;           // NS kernels: bf16 MFMA, else fp32
  const bool t_bf16 = dtype == MUON_BF16;      // params / grads / in / out
  const size_t es = dtype_size(dtype), wes = dtype_size(ns);
  char* W = static_cast<char*>(ws);
  const float kg = o.momentum_form == 0 ? 1.0f - beta : 1.0f;
  int status = MUON_OK;

  for (const Batch& B : plan.batches) {
    PhaseRange batch_range("batch: " + std::to_string(B.count) + " x " + std::to_string(B.m) + "x" +
                      std::to_string(B.n) + " (group " + std::to_string(B.group) + ")");
    const Layout L = batch_layout(B.count, B.m_pad, B.n_pad, ns);
    void* x0 = W + L.x0;
    void* x1 = W + L.x1;
    void* Am = W + L.a;
    void* Bm = W + L.b;
    float* partials = reinterpret_cast<float*>(W + L.partials);
    int* nonzero = reinterpret_cast<int*>(W + L.nonzero);
    int* live = reinterpret_cast<int*>(W + L.live);
    int* live_list = reinterpret_cast<int*>(W + L.live_list);
    int* nlive = reinterpret_cast<int*>(W + L.nlive);
    int* sched = reinterpret_cast<int*>(W + L.sched);
    // bf16 with NS steps: matrices whose input is exactly zero (idle experts)
    // get no GEMM work; their O is exactly 0.
    const bool skip_zero = bf16 && ns_steps > 0;
    float* scales = reinterpret_cast<float*>(W + L.scales);
    ApplyEntry* ptab = reinterpret_cast<ApplyEntry*>(W + L.ptab);
    const double elems = (double)B.m * B.n;
    // bf16 tensors and NS with at least one NS step: the apply runs inside
    // the last Update GEMM (it needs whole, aligned 16 B runs along rows of
    // both orientations, so every row stride is a multiple of 8).
    bool fused_apply = bf16 && t_bf16 && ns_steps > 0 && B.m % 8 == 0 && B.n % 8 == 0;
    for (int k = 0; k < B.count && fused_apply; ++k) fused_apply = mats[plan.order[B.first + k]].ld % 8 == 0;
    const float apply_alpha = (float)(1.0 - (double)lr * (double)o.weight_decay);
    const float apply_gamma[2] = {(float)((double)lr * update_scale(o, B.m, B.n)),
                                  (float)((double)lr * update_scale(o, B.n, B.m))};

    // 1. momentum (+ transpose, cast, partial sums)
    for (int c0 = 0; c0 < B.count && status == MUON_OK; c0 += kEwChunk) {
      const int cn = std::min(kEwChunk, B.count - c0);
      EwMats em;
      std::memset(&em, 0, sizeof(em));
      for (int k = 0; k < cn; ++k) {
        const MatRef& r = mats[plan.order[B.first + c0 + k]];
        em.src[k] = r.src;
        em.buf[k] = r.mom;
        em.dst[k] = r.param;
        em.ld[k] = r.ld;
        em.tr[k] = r.rows > r.cols ? 1 : 0;
      }
      MomentumArgs a;
      a.count = cn; a.m = B.m; a.n = B.n; a.m_pad = B.m_pad; a.n_pad = B.n_pad;
      a.ew_blocks = L.ew_blocks; a.first = c0; a.x0 = x0; a.mat_x = L.mat_x;
      a.partials = partials; a.nonzero = nonzero; a.has_buf = orthogonalize_only ? 0 : 1;
      a.beta = beta; a.kg = kg; a.nesterov = o.nesterov;
      a.ptab = fused_apply ? ptab : nullptr;
      const double bytes = cn * elems * ((orthogonalize_only ? es : es + 4 + 4) + wes);
      ProfScope ps("momentum", 0.0, bytes, stream);
      e = launch_momentum(em, a, t_bf16, bf16, stream);
      if (e != hipSuccess) status = hip_fail(e, "momentum kernel launch");
    }
    if (status) break;

    // 2. per-matrix Frobenius scale
    {
      FinalizeArgs f{B.count, L.ew_blocks, partials, scales, o.eps, nonzero, live};
      ProfScope ps("norm_finalize", 0.0, (double)B.count * L.ew_blocks * 4, stream);
      e = launch_finalize(f, stream);
      if (e != hipSuccess) { status = hip_fail(e, "finalize kernel launch"); break; }
      if (skip_zero) {
        e = launch_compact(live, B.count, live_list, nlive, sched, stream);
        if (e != hipSuccess) { status = hip_fail(e, "compact kernel launch"); break; }
      }
    }

    // 3. NS iterations; the Frobenius scale is folded into the first step.
    // The batch's coefficient table: its set's (per-parameter sets), the
    // call's, or the standard quintic at every step.
    const float* tab = o.num_coeff_sets > 0 ? o.coeff_sets + (size_t)B.set * (size_t)ns_steps * 3 : o.coeffs;
    void* X = x0;
    void* Xn = x1;
    for (int k = 0; k < ns_steps && status == MUON_OK; ++k) {
      PhaseRange step_range("ns step " + std::to_string(k + 1));
      GemmArgs g{};
      g.mat_x = L.mat_x; g.mat_a = L.mat_a; g.count = B.count;
      g.m = B.m; g.n = B.n; g.m_pad = B.m_pad; g.n_pad = B.n_pad;
      g.ca = tab ? tab[3 * k + 0] : 3.4445f;
      g.cb = tab ? tab[3 * k + 1] : -4.7750f;
      g.cc = tab ? tab[3 * k + 2] : 2.0315f;
      // bf16, MUON_POLY_DIRECT: Gram writes A, Poly b A + c A A (A tile in
      // its epilogue), Update a X + B X (X tile in its epilogue).
      // MUON_POLY_SQUARE with c != 0: the polynomial is completed to a square,
      //   a I + b A + c A^2 = c (A + beta I)^2 + (a - b^2/(4c)) I,
      //   beta = b / (2c),
      // so Gram writes A' = A + beta I, Poly c A'A' + (a - b^2/(4c)) I and
      // Update B' X, with no operand tile; with c = 0 Poly forms a I + b A
      // + c A A with the A tile. The step's arithmetic is in double,
      // rounded once to float.
      // MUON_POLY_FOLDED (and the square form with c = 0): Gram writes A,
      // Poly a I + b A + c A A from the A tile, Update B' X.
      const bool square = bf16 && o.poly_form == MUON_POLY_SQUARE;
      const bool folded = bf16 && (o.poly_form == MUON_POLY_FOLDED || (square && g.cc == 0.0f));
      const bool shifted = square && g.cc != 0.0f;
      const double beta_sq = shifted ? (double)g.cb / (2.0 * (double)g.cc) : 0.0;
      const float gram_diag = (float)beta_sq;
      const float poly_diag = shifted ? (float)((double)g.ca - (double)g.cb * (double)g.cb / (4.0 * (double)g.cc))
                                      : (folded ? g.ca : 0.0f);
      const GemmRole roles[3] = {kGram, kPoly, kUpdate};
      const char* names[3] = {"ns_gram", "ns_poly", "ns_update"};
      for (int r = 0; r < 3; ++r) {
        g.x = X; g.a = Am; g.b = Bm;
        g.out = r == 0 ? Am : (r == 1 ? Bm : Xn);
        g.scales = (k == 0 && r != 1) ? scales : nullptr;
        g.diag_add = r == 0 ? gram_diag : (r == 1 ? poly_diag : 0.0f);
        g.live_list = skip_zero ? live_list : nullptr;
        g.nlive = nlive;
        // Dynamic tile schedule for Gram (its diagonal tiles multiply 36 of
        // 64 blocks, and K = n makes its tiles long); measured on the MoE
        // bank it is 2.8% faster there, neutral for Poly and 6% slower for
        // Update (all its tiles alike) at the default batch cap. The
        // counters are zeroed by the compact kernel.
        g.sched = (skip_zero && r == 0) ? sched : nullptr;
        g.poly_operand = shifted ? 0 : 1;
        g.update_operand = (bf16 && !square && !folded) ? 1 : 0;
        const bool apply_here = fused_apply && r == 2 && k + 1 == ns_steps;
        g.ptab = apply_here ? ptab : nullptr;
        g.alpha = apply_alpha;
        g.gamma[0] = apply_gamma[0];
        g.gamma[1] = apply_gamma[1];
        g.apply_mode = orthogonalize_only ? 1 : 0;
        ProfScope ps(names[r], gemm_flops(roles[r], g), 0.0, stream);
        e = bf16 ? launch_gemm_bf16(roles[r], g, stream) : launch_gemm_f32(roles[r], g, stream);
        if (e != hipSuccess) { status = hip_fail(e, names[r]); break; }
      }
      std::swap(X, Xn);
    }
    if (status) break;

    // 4. apply (+ transpose back). With the apply fused into the last
    // Update, only the skipped (zero-input) matrices remain, and only when
    // their update p' = alpha*p (or out = 0) is not a no-op.
    const bool dead_pass = fused_apply && (orthogonalize_only || apply_alpha != 1.0f);
    for (int c0 = 0; c0 < B.count && status == MUON_OK && (!fused_apply || dead_pass); c0 += kEwChunk) {
      const int cn = std::min(kEwChunk, B.count - c0);
      EwMats em;
      std::memset(&em, 0, sizeof(em));
      for (int k = 0; k < cn; ++k) {
        const MatRef& r = mats[plan.order[B.first + c0 + k]];
        em.src[k] = r.param;
        em.dst[k] = r.param;
        em.ld[k] = r.ld;
        em.tr[k] = r.rows > r.cols ? 1 : 0;
      }
      ApplyArgs a;
      a.live = skip_zero ? live : nullptr;
      a.dead_only = fused_apply ? 1 : 0;
      a.count = cn; a.m = B.m; a.n = B.n; a.n_pad = B.n_pad; a.first = c0;
      a.x = X; a.mat_x = L.mat_x; a.scales = scales; a.use_scale = ns_steps == 0 ? 1 : 0;
      a.mode = orthogonalize_only ? 1 : 0;
      a.alpha = apply_alpha;
      a.gamma[0] = apply_gamma[0];
      a.gamma[1] = apply_gamma[1];
      const double bytes = cn * elems * (orthogonalize_only ? wes + es : wes + es + es);
      ProfScope ps("apply", 0.0, bytes, stream);
      e = launch_apply(em, a, t_bf16, bf16, stream);
      if (e != hipSuccess) status = hip_fail(e, "apply kernel launch");
    }
    if (status) break;
  }

  if (!use_static) {
    hipError_t ef = hipFreeAsync(ws, stream);
    if (status == MUON_OK && ef != hipSuccess) status = hip_fail(ef, "hipFreeAsync");
  }
  return status;
}

// Batch cap used when the caller leaves it at 0 (or passes no options):
// MUON_BATCH_CAP from the environment if it is a positive integer, else 2^29.
size_t default_batch_cap() {
  if (const char* v = std::getenv("MUON_BATCH_CAP")) {
    char* end = nullptr;
    const unsigned long long c = std::strtoull(v, &end, 10);
    if (end != v && *end == '\0' && c > 0) return (size_t)c;
  }
  return MUON_DEFAULT_BATCH_CAP;
}

int validate_common(float lr, float beta, int ns_steps, muon_dtype dtype, const muon_options* opts,
                    muon_options& o) {
  std::string err;
  int rc = check_scalars(lr, beta, ns_steps, dtype, err);
  if (rc) return fail(rc, err);
  default_options(o);
  if (opts) o = *opts;
  if (!opts || o.batch_cap_elems == 0) o.batch_cap_elems = default_batch_cap();
  rc = check_options(o, ns_steps, err);
  if (rc) return fail(rc, err);
  return MUON_OK;
}

int validate_mats(const std::vector<MatRef>& mats, muon_dtype dtype, bool orthogonalize_only) {
  std::string err;
  const size_t es = dtype_size(dtype);
  std::vector<Range> ranges;
  for (int i = 0; i < (int)mats.size(); ++i) {
    const MatRef& r = mats[i];
    int rc = check_shape(r.rows, r.cols, err, i);
    if (rc) return fail(rc, err);
    const char* pn = orthogonalize_only ? "out" : "params";
    const char* sn = orthogonalize_only ? "in" : "grads";
    if ((rc = check_ptr(r.param, pn, i, err))) return fail(rc, err);
    if ((rc = check_ptr(r.src, sn, i, err))) return fail(rc, err);
    if (!orthogonalize_only && (rc = check_ptr(r.mom, "momentum", i, err))) return fail(rc, err);
    const unsigned long long rows = (unsigned long long)r.rows, cols = (unsigned long long)r.cols,
                             ld = (unsigned long long)r.ld;
    if (orthogonalize_only) {
      // out may be exactly in (in place); any other overlap is an error.
      if (r.param != r.src) ranges.push_back(strided_range(r.src, rows, cols * es, ld * es, sn, i));
      ranges.push_back(strided_range(r.param, rows, cols * es, ld * es, pn, i));
    } else {
      ranges.push_back(strided_range(r.param, rows, cols * es, ld * es, pn, i));
      ranges.push_back(strided_range(r.src, rows, cols * es, ld * es, sn, i));
      ranges.push_back(strided_range(r.mom, rows, cols * 4, ld * 4, "momentum", i));
    }
  }
  int rc = check_no_overlap(ranges, err);
  if (rc) return fail(rc, err);
  return MUON_OK;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

void muon_default_options(muon_options* opts) {
  if (opts) default_options(*opts);
}

int muon_step(const muon_matrix* mats, int num, float lr, float beta, int ns_steps, muon_dtype dtype,
              const muon_options* opts, void* stream) {
  try {
    g_err.clear();
    if (num < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "num < 0");
    if (num > 0 && !mats) return fail(MUON_ERR_INVALID_ARGUMENT, "mats is NULL");
    muon_options o;
    int rc = validate_common(lr, beta, ns_steps, dtype, opts, o);
    if (rc) return rc;
    std::vector<MatRef> v(num);
    for (int i = 0; i < num; ++i)
      v[i] = MatRef{mats[i].param, mats[i].grad, mats[i].momentum, mats[i].rows, mats[i].cols, mats[i].cols};
    rc = validate_mats(v, dtype, false);
    if (rc) return rc;
    return run(v, lr, beta, ns_steps, dtype, o, false, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MUON_ERR_HIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

int muon_step_noalloc(const muon_matrix* mats, int num, float lr, float beta, int ns_steps, muon_dtype dtype,
                      const muon_options* opts, void* stream) {
  try {
    g_err.clear();
    if (num < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "num < 0");
    if (num > 0 && !mats) return fail(MUON_ERR_INVALID_ARGUMENT, "mats is NULL");
    muon_options o;
    int rc = validate_common(lr, beta, ns_steps, dtype, opts, o);
    if (rc) return rc;
    std::vector<MatRef> v(num);
    for (int i = 0; i < num; ++i)
      v[i] = MatRef{mats[i].param, mats[i].grad, mats[i].momentum, mats[i].rows, mats[i].cols, mats[i].cols};
    rc = validate_mats(v, dtype, false);
    if (rc) return rc;
    return run(v, lr, beta, ns_steps, dtype, o, false, static_cast<hipStream_t>(stream), true);
  } catch (const std::exception& ex) {
    return fail(MUON_ERR_HIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

int muon_step_views(const muon_matrix_view* views, int num, float lr, float beta, int ns_steps,
                    muon_dtype dtype, const muon_options* opts, void* stream) {
  try {
    g_err.clear();
    if (num < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "num < 0");
    if (num > 0 && !views) return fail(MUON_ERR_INVALID_ARGUMENT, "views is NULL");
    muon_options o;
    int rc = validate_common(lr, beta, ns_steps, dtype, opts, o);
    if (rc) return rc;
    std::vector<MatRef> v(num);
    for (int i = 0; i < num; ++i) {
      const muon_matrix_view& w = views[i];
      std::string err;
      if ((rc = check_shape(w.rows, w.cols, err, i))) return fail(rc, err);
      const long long ld = w.ld == 0 ? (long long)w.cols : w.ld;
      if (ld < w.cols || ld > 0x7fffffffLL)
        return fail(MUON_ERR_INVALID_ARGUMENT, "views[" + std::to_string(i) + "].ld = " + std::to_string(w.ld) +
                                                   " outside [cols, 2^31 - 1]");
      v[i] = MatRef{w.param, w.grad, w.momentum, w.rows, w.cols, (int)ld};
    }
    rc = validate_mats(v, dtype, false);
    if (rc) return rc;
    return run(v, lr, beta, ns_steps, dtype, o, false, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MUON_ERR_HIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

int muon_group_step(void* const* params, const void* const* grads, float* const* momentum, int count,
                    int m, int n, float lr, float beta, int ns_steps, muon_dtype dtype, void* stream) {
  try {
    g_err.clear();
    if (count < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "count < 0");
    if (count > 0 && (!params || !grads || !momentum))
      return fail(MUON_ERR_INVALID_ARGUMENT, "params, grads or momentum array is NULL");
    muon_options o;
    int rc = validate_common(lr, beta, ns_steps, dtype, nullptr, o);
    if (rc) return rc;
    if (count > 0) {
      std::string err;
      if ((rc = check_shape(m, n, err))) return fail(rc, err);
    }
    std::vector<MatRef> v(count);
    for (int i = 0; i < count; ++i) v[i] = MatRef{params[i], grads[i], momentum[i], m, n, n};
    rc = validate_mats(v, dtype, false);
    if (rc) return rc;
    return run(v, lr, beta, ns_steps, dtype, o, false, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MUON_ERR_HIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

int muon_orthogonalize(const void* const* in, void* const* out, int count, int m, int n, int ns_steps,
                       muon_dtype dtype, const muon_options* opts, void* stream) {
  try {
    g_err.clear();
    if (count < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "count < 0");
    if (count > 0 && (!in || !out)) return fail(MUON_ERR_INVALID_ARGUMENT, "in or out array is NULL");
    muon_options o;
    int rc = validate_common(0.0f, 0.0f, ns_steps, dtype, opts, o);
    if (rc) return rc;
    if (count > 0) {
      std::string err;
      if ((rc = check_shape(m, n, err))) return fail(rc, err);
    }
    std::vector<MatRef> v(count);
    for (int i = 0; i < count; ++i) v[i] = MatRef{out[i], in[i], nullptr, m, n, n};
    rc = validate_mats(v, dtype, true);
    if (rc) return rc;
    return run(v, 0.0f, 0.0f, ns_steps, dtype, o, true, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MUON_ERR_HIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

int muon_plan_query(const int* rows, const int* cols, int num, muon_dtype dtype, const muon_options* opts,
                    muon_plan_batch* batches, int cap, int* num_batches, int* order, size_t* workspace_bytes) {
  try {
    g_err.clear();
    muon_options o;
    default_options(o);
    if (opts) o = *opts;
    if (!opts || o.batch_cap_elems == 0) o.batch_cap_elems = default_batch_cap();
    Plan plan;
    std::string err;
    if (o.compute_units < -1) return fail(MUON_ERR_INVALID_ARGUMENT, "options.compute_units must be >= -1");
    if (o.ns_dtype != -1 && o.ns_dtype != MUON_F32 && o.ns_dtype != MUON_BF16)
      return fail(MUON_ERR_INVALID_ARGUMENT, "options.ns_dtype must be -1, MUON_F32 or MUON_BF16");
    if (o.num_coeff_sets < 0) return fail(MUON_ERR_INVALID_ARGUMENT, "options.num_coeff_sets must be >= 0");
    if (o.num_coeff_sets > 0 && !o.coeff_set_of)
      return fail(MUON_ERR_INVALID_ARGUMENT, "options.coeff_set_of is required when num_coeff_sets > 0");
    const int* set_of = o.num_coeff_sets > 0 ? o.coeff_set_of : nullptr;
    int rc = build_plan(rows, cols, num, ns_type(o, dtype), o.batch_cap_elems, fit_units(o), plan, err, set_of,
                        o.num_coeff_sets);
    if (rc) return fail(rc, err);
    if (cap > 0 && !batches) return fail(MUON_ERR_INVALID_ARGUMENT, "batches is NULL with cap > 0");
    for (int i = 0; i < cap && i < (int)plan.batches.size(); ++i) {
      const Batch& b = plan.batches[i];
      batches[i] = muon_plan_batch{b.group, b.m, b.n, b.m_pad, b.n_pad, b.first, b.count, b.set};
    }
    if (num_batches) *num_batches = (int)plan.batches.size();
    if (order) std::copy(plan.order.begin(), plan.order.end(), order);
    if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
    return MUON_OK;
  } catch (...) {
    return fail(MUON_ERR_HIP, "internal error");
  }
}

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported";
    case MUON_ERR_MISALIGNED: return "misaligned pointer";
    case MUON_ERR_OUT_OF_MEMORY: return "out of memory";
    case MUON_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* muon_last_error(void) { return g_err.c_str(); }

int muon_version(void) { return 200; }

int muon_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int prev = g_prof_on ? 1 : 0;
  g_prof_on = on != 0;
  return prev;
}

int muon_profile_read(muon_profile_entry* out, int cap, int reset) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int status = 0;
  for (Pending& p : g_pending) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(p.e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.e0, p.e1);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      status = -MUON_ERR_HIP;
      g_err = hipGetErrorString(e);
    }
    if (!g_totals.count(p.kind)) g_kind_order.push_back(p.kind);
    ProfTotal& t = g_totals[p.kind];
    t.launches += 1; t.ms += ms; t.flops += p.flops; t.bytes += p.bytes;
    g_free_events.push_back(p.e0);
    g_free_events.push_back(p.e1);
  }
  g_pending.clear();
  if (status) return status;
  int n = 0;
  for (const std::string& k : g_kind_order) {
    if (n < cap && out) {
      const ProfTotal& t = g_totals[k];
      std::memset(&out[n], 0, sizeof(out[n]));
      std::strncpy(out[n].name, k.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = t.launches; out[n].total_ms = t.ms; out[n].flops = t.flops; out[n].bytes = t.bytes;
    }
    ++n;
  }
  if (reset) { g_totals.clear(); g_kind_order.clear(); }
  return n;
}

}  // extern "C"
