// forge_host.cpp -- the C ABI declared in include/forge.h: argument validation, per-step
// scalars (fp64 on the host, handed to the kernels as fp32), device check and dispatch.
//
// Validation runs before any HIP call, so a bad call returns its error code without a GPU
// being touched (and without one being present).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "forge.h"
#include "forge_internal.h"

namespace {

thread_local std::string g_last_error;

forge_status fail(forge_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

int64_t dtype_size(int32_t dt) {
  switch (dt) {
    case FORGE_F32: return 4;
    case FORGE_BF16: return 2;
    case FORGE_FP8_E4M3:
    case FORGE_I8_B64:
    case FORGE_U8_B64:
    case FORGE_I8DYN_B64:
    case FORGE_U8DYN_B64: return 1;
  }
  return 0;
}

bool rule_has_m(int32_t opt) {
  return opt == FORGE_ADAMW || opt == FORGE_NADAM || opt == FORGE_RADAM || opt == FORGE_LION ||
         opt == FORGE_SGD_MOMENTUM;
}
bool rule_has_v(int32_t opt) {
  return opt == FORGE_ADAMW || opt == FORGE_NADAM || opt == FORGE_RADAM || opt == FORGE_RMSPROP ||
         opt == FORGE_ADAGRAD;
}

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  const char* name = "";
};

Range range_of(const void* p, int64_t bytes, const char* name) {
  Range r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (uintptr_t)(bytes > 0 ? bytes : 0);
  r.name = name;
  return r;
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Every tensor stays below 2^48 bytes, so the size products below (and the kernels' own
// bounds, which are tighter) cannot overflow 64-bit arithmetic.
constexpr int64_t kMaxBytes = int64_t(1) << 48;

forge_status check_tensor(const forge_tensor* t, const char* name) {
  if (!t) return fail(FORGE_ERR_ARG, "%s is NULL", name);
  if (t->rows < 0 || t->cols < 0) return fail(FORGE_ERR_SHAPE, "%s has a negative dimension", name);
  if (dtype_size(t->dtype) == 0) return fail(FORGE_ERR_DTYPE, "%s has unknown dtype %d", name, (int)t->dtype);
  int64_t elems = 0, bytes = 0;
  if (__builtin_mul_overflow(t->rows, t->cols, &elems) || __builtin_mul_overflow(elems, dtype_size(t->dtype), &bytes) ||
      bytes >= kMaxBytes)
    return fail(FORGE_ERR_SHAPE, "%s [%lld, %lld] is too large", name, (long long)t->rows, (long long)t->cols);
  if (elems > 0 && !t->data) return fail(FORGE_ERR_ARG, "%s->data is NULL", name);
  if (!aligned16(t->data)) return fail(FORGE_ERR_LAYOUT, "%s->data is not 16-byte aligned", name);
  if (t->rows > 0 && t->ld != t->cols)
    return fail(FORGE_ERR_LAYOUT, "%s has row stride %lld, expected %lld (contiguous rows)", name, (long long)t->ld,
                (long long)t->cols);
  return FORGE_OK;
}

int64_t bytes_of(const forge_tensor* t) { return t->rows * t->cols * dtype_size(t->dtype); }

// device check, cached per device
std::atomic<int> g_dev_ok[64];

forge_status device_ok() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FORGE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64 && g_dev_ok[dev].load(std::memory_order_relaxed) == 1) return FORGE_OK;
  return forge_device_check(dev);
}

forge_status to_status(int herr) {
  if (herr == (int)hipSuccess) return FORGE_OK;
  return fail(FORGE_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString((hipError_t)herr));
}

}  // namespace

// ------------------------------------------------------------------ per-step scalars
// fp64 -> fp32 for a per-step scalar; false if it is not finite in fp32.
static bool to_f32(double x, float* out) {
  if (!(std::fabs(x) <= 3.4028234663852886e38)) return false;
  *out = (float)x;
  return std::isfinite(*out);
}

static forge_status compute_scalars(int32_t opt, const forge_hyper* h, int64_t step, forge::OptScalars* out) {
  if (!h) return fail(FORGE_ERR_ARG, "hyper is NULL");
  if (opt < FORGE_ADAMW || opt > FORGE_SGD_MOMENTUM) return fail(FORGE_ERR_ARG, "unknown optimizer %d", (int)opt);
  if (step < 1) return fail(FORGE_ERR_ARG, "step must be >= 1 (got %lld)", (long long)step);
  if (h->wd_mode < FORGE_WD_DEFAULT || h->wd_mode > FORGE_WD_L2)
    return fail(FORGE_ERR_ARG, "unknown wd_mode %d", (int)h->wd_mode);
  const bool adam_family = opt == FORGE_ADAMW || opt == FORGE_NADAM || opt == FORGE_RADAM;
  if (adam_family && !(h->beta1 >= 0.0f && h->beta1 < 1.0f && h->beta2 >= 0.0f && h->beta2 < 1.0f))
    return fail(FORGE_ERR_ARG, "beta1 and beta2 must lie in [0, 1) (got %g, %g)", (double)h->beta1, (double)h->beta2);
  if (opt == FORGE_NADAM && !(h->momentum_decay >= 0.0f && std::isfinite(h->momentum_decay)))
    return fail(FORGE_ERR_ARG, "NAdam needs a finite momentum_decay >= 0");
  // fields a rule does not use are not read (they may hold anything)
  const bool uses_betas = opt == FORGE_ADAMW || opt == FORGE_NADAM || opt == FORGE_RADAM || opt == FORGE_LION;
  const bool uses_eps = uses_betas ? opt != FORGE_LION : (opt == FORGE_RMSPROP || opt == FORGE_ADAGRAD);
  const double lr = h->lr, wd = h->weight_decay;
  const double b1 = uses_betas ? h->beta1 : 0.0, b2 = uses_betas ? h->beta2 : 0.0, eps = uses_eps ? h->eps : 0.0;
  const double t = (double)step;
  const bool dec = h->wd_mode == FORGE_WD_DECOUPLED ||
                   (h->wd_mode == FORGE_WD_DEFAULT && (opt == FORGE_ADAMW || opt == FORGE_LION));
  double d[12] = {dec ? 1.0 - lr * wd : 1.0, dec ? 0.0 : wd, 0.0, 0.0, 0.0, b1, 1.0 - b1, b2, 1.0 - b2, eps, lr, 0.0};
  double &c1 = d[2], &c2 = d[3], &c3 = d[4];
  int32_t rect = 0;
  const double bc1 = 1.0 - std::pow(b1, t), bc2 = 1.0 - std::pow(b2, t);
  switch (opt) {
    case FORGE_ADAMW:
      c1 = lr / bc1;
      c2 = 1.0 / bc2;
      break;
    case FORGE_NADAM: {
      // momentum schedule mu_i = beta1 (1 - 0.5 * 0.96^(i psi)); prod_t = mu_1 ... mu_t
      // Every factor lies in [0, 1], so once prod < 2^-60 both 1 - prod and 1 - prod * mu_next
      // round to exactly 1 for this and any later factor: the loop stops there with the same
      // scalars (and its length no longer grows with the step count).
      const double psi = h->momentum_decay;
      double prod = 1.0;
      for (int64_t i = 1; i <= step && prod >= 0x1p-60; ++i) prod *= b1 * (1.0 - 0.5 * std::pow(0.96, (double)i * psi));
      const double mu = b1 * (1.0 - 0.5 * std::pow(0.96, t * psi));
      const double mu_next = b1 * (1.0 - 0.5 * std::pow(0.96, (t + 1.0) * psi));
      c1 = lr * (1.0 - mu) / (1.0 - prod);
      c2 = 1.0 / bc2;
      c3 = lr * mu_next / (1.0 - prod * mu_next);
      break;
    }
    case FORGE_RADAM: {
      const double rho_inf = 2.0 / (1.0 - b2) - 1.0;
      const double rho_t = rho_inf - 2.0 * t * std::pow(b2, t) / bc2;
      if (rho_t > 5.0) {
        const double r = std::sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t));
        rect = 1;
        c1 = lr * r * std::sqrt(bc2) / bc1;
      } else {
        c1 = lr / bc1;
      }
      break;
    }
    case FORGE_RMSPROP:
      d[7] = h->alpha;
      d[8] = 1.0 - (double)h->alpha;
      break;
    case FORGE_SGD_MOMENTUM:
      c1 = h->momentum;
      break;
    default:
      break;
  }
  static const char* const names[12] = {"decay", "l2", "c1", "c2", "c3", "b1", "1 - b1", "b2", "1 - b2", "eps", "lr", ""};
  float f[12];
  for (int i = 0; i < 11; ++i)
    if (!to_f32(d[i], &f[i]))
      return fail(FORGE_ERR_ARG, "the hyper-parameters give a non-finite step scalar %s (%g) at step %lld", names[i],
                  d[i], (long long)step);
  forge::OptScalars s{};
  s.decay = f[0];
  s.l2 = f[1];
  s.c1 = f[2];
  s.c2 = f[3];
  s.c3 = f[4];
  s.b1 = f[5];
  s.omb1 = f[6];
  s.b2 = f[7];
  s.omb2 = f[8];
  s.eps = f[9];
  s.lr = f[10];
  s.rect = rect;
  *out = s;
  return FORGE_OK;
}

// ------------------------------------------------------------------ shared validation of the step
struct StepPlan {
  int w_type = 0, s_type = 0;
  forge::EpiArgs e{};
};

static forge_status validate_step_outputs(int64_t N, int64_t K, forge_tensor* W, forge_tensor* m, forge_tensor* v,
                                          const forge_hyper* hyper, int32_t opt, int64_t step, uint64_t seed,
                                          const forge_step_opts* opts, StepPlan* plan, Range* outs, int* n_outs) {
  forge_status st;
  if ((st = check_tensor(W, "W")) != FORGE_OK) return st;
  if (W->rows != N || W->cols != K)
    return fail(FORGE_ERR_SHAPE, "W is [%lld, %lld], expected [%lld, %lld]", (long long)W->rows, (long long)W->cols,
                (long long)N, (long long)K);
  if (N % 128 || K % 128)
    return fail(FORGE_ERR_SHAPE, "N = %lld and K = %lld must be multiples of 128", (long long)N, (long long)K);
  if (N * K >= (int64_t(1) << 32)) return fail(FORGE_ERR_SHAPE, "N * K must be below 2^32");
  if (W->dtype != FORGE_F32 && W->dtype != FORGE_BF16) return fail(FORGE_ERR_DTYPE, "W must be F32 or BF16");

  forge::OptScalars s;
  if ((st = compute_scalars(opt, hyper, step, &s)) != FORGE_OK) return st;

  const bool need_m = rule_has_m(opt), need_v = rule_has_v(opt);
  if (need_m != (m != nullptr))
    return fail(FORGE_ERR_ARG, need_m ? "this rule keeps a first moment m: pass it" : "this rule keeps no m: pass NULL");
  if (need_v != (v != nullptr))
    return fail(FORGE_ERR_ARG, need_v ? "this rule keeps a second moment v: pass it" : "this rule keeps no v: pass NULL");
  int s_type = -1;
  int n = 0;
  outs[n++] = range_of(W->data, bytes_of(W), "W");
  for (int which = 0; which < 2; ++which) {
    forge_tensor* t = which ? v : m;
    const char* name = which ? "v" : "m";
    if (!t) continue;
    if ((st = check_tensor(t, name)) != FORGE_OK) return st;
    if (t->rows != N || t->cols != K) return fail(FORGE_ERR_SHAPE, "%s must have the shape of W", name);
    int ty;
    if (t->dtype == FORGE_F32) ty = forge::FORGE_S_F32;
    else if (t->dtype == (which ? FORGE_U8_B64 : FORGE_I8_B64)) ty = forge::FORGE_S_Q8;
    else if (t->dtype == (which ? FORGE_U8DYN_B64 : FORGE_I8DYN_B64)) ty = forge::FORGE_S_Q8D;
    else
      return fail(FORGE_ERR_DTYPE, "%s must be F32, %s or %s", name, which ? "U8_B64" : "I8_B64",
                  which ? "U8DYN_B64" : "I8DYN_B64");
    if (s_type >= 0 && ty != s_type)
      return fail(FORGE_ERR_DTYPE, (s_type == forge::FORGE_S_F32) != (ty == forge::FORGE_S_F32)
                                       ? "m and v must both be fp32 or both be 8-bit"
                                       : "m and v must use the same 8-bit map");
    s_type = ty;
    outs[n++] = range_of(t->data, bytes_of(t), name);
    if (ty != forge::FORGE_S_F32) {
      if (!t->scale) return fail(FORGE_ERR_ARG, "%s->scale (block scales) is NULL", name);
      if (!aligned4(t->scale)) return fail(FORGE_ERR_LAYOUT, "%s->scale is not 4-byte aligned", name);
      outs[n++] = range_of(t->scale, N * K / 64 * 4, which ? "v scales" : "m scales");
    }
  }
  if (s_type < 0) s_type = forge::FORGE_S_F32;
  float* w_pre = opts ? opts->w_preround_out : nullptr;
  if (w_pre) {
    if (!aligned16(w_pre)) return fail(FORGE_ERR_LAYOUT, "w_preround_out is not 16-byte aligned");
    outs[n++] = range_of(w_pre, N * K * 4, "w_preround_out");
  }
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (overlap(outs[i], outs[j])) return fail(FORGE_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
  *n_outs = n;

  plan->w_type = W->dtype == FORGE_BF16 ? forge::FORGE_W_BF16 : forge::FORGE_W_F32;
  plan->s_type = s_type;
  forge::EpiArgs& e = plan->e;
  e.W = W->data;
  e.m = m ? m->data : nullptr;
  e.v = v ? v->data : nullptr;
  e.m_scale = m ? static_cast<float*>(m->scale) : nullptr;
  e.v_scale = v ? static_cast<float*>(v->scale) : nullptr;
  e.w_pre = w_pre;
  e.seed = seed;
  e.step = (uint64_t)step;
  e.sr = opts ? (opts->sr_enable != 0) : 1;
  e.s = s;
  return FORGE_OK;
}

static forge_status validate_inputs(const forge_tensor* X, const forge_tensor* dY, int* in_type, forge::GemmArgs* g,
                                    Range* ins, int* n_ins) {
  forge_status st;
  if ((st = check_tensor(X, "X")) != FORGE_OK) return st;
  if ((st = check_tensor(dY, "dY")) != FORGE_OK) return st;
  if (X->dtype != dY->dtype) return fail(FORGE_ERR_DTYPE, "X and dY must have the same dtype");
  if (X->dtype == FORGE_F32) *in_type = forge::FORGE_IN_F32;
  else if (X->dtype == FORGE_BF16) *in_type = forge::FORGE_IN_BF16;
  else if (X->dtype == FORGE_FP8_E4M3) *in_type = forge::FORGE_IN_FP8;
  else return fail(FORGE_ERR_DTYPE, "X and dY must be F32, BF16 or FP8_E4M3");
  if (X->rows != dY->rows)
    return fail(FORGE_ERR_SHAPE, "X has %lld tokens, dY has %lld", (long long)X->rows, (long long)dY->rows);
  int n = 0;
  ins[n++] = range_of(X->data, bytes_of(X), "X");
  ins[n++] = range_of(dY->data, bytes_of(dY), "dY");
  g->x_scale = g->dy_scale = nullptr;
  if (*in_type == forge::FORGE_IN_FP8) {
    if (!X->scale || !dY->scale) return fail(FORGE_ERR_ARG, "fp8 inputs need their per-tensor scale pointers");
    if (!aligned4(X->scale) || !aligned4(dY->scale)) return fail(FORGE_ERR_LAYOUT, "fp8 scale not 4-byte aligned");
    g->x_scale = static_cast<const float*>(X->scale);
    g->dy_scale = static_cast<const float*>(dY->scale);
    ins[n++] = range_of(X->scale, 4, "X scale");
    ins[n++] = range_of(dY->scale, 4, "dY scale");
  }
  // the kernels address X and dY with 32-bit byte offsets (one spare slab of tokens included)
  const int64_t esz = dtype_size(X->dtype);
  if ((X->rows + 128) * X->cols * esz >= (int64_t(1) << 32) || (dY->rows + 128) * dY->cols * esz >= (int64_t(1) << 32))
    return fail(FORGE_ERR_SHAPE, "X and dY must each stay below 4 GiB");
  g->X = X->data;
  g->dY = dY->data;
  g->T = X->rows;
  g->K = X->cols;
  g->N = dY->cols;
  *n_ins = n;
  return FORGE_OK;
}

extern "C" {

forge_status forge_wgrad_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W, forge_tensor* m,
                              forge_tensor* v, const forge_hyper* hyper, int32_t opt, int64_t step, uint64_t seed,
                              const forge_step_opts* opts, void* stream) {
  g_last_error.clear();
  Range ins[4], outs[6];
  int n_in = 0, n_out = 0, in_type = 0;
  forge::GemmArgs g{};
  forge_status st;
  if ((st = validate_inputs(X, dY, &in_type, &g, ins, &n_in)) != FORGE_OK) return st;
  StepPlan plan;
  if ((st = validate_step_outputs(g.N, g.K, W, m, v, hyper, opt, step, seed, opts, &plan, outs, &n_out)) != FORGE_OK)
    return st;
  for (int i = 0; i < n_out; ++i)
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return fail(FORGE_ERR_ALIAS, "%s overlaps %s", outs[i].name, ins[j].name);
  if (g.N == 0 || g.K == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  return to_status(forge::launch_fused_step(in_type, plan.w_type, plan.s_type, opt, g, plan.e, stream));
}

forge_status forge_wgrad_gemm(const forge_tensor* X, const forge_tensor* dY, forge_tensor* dW, void* stream) {
  g_last_error.clear();
  Range ins[4];
  int n_in = 0, in_type = 0;
  forge::GemmArgs g{};
  forge_status st;
  if ((st = validate_inputs(X, dY, &in_type, &g, ins, &n_in)) != FORGE_OK) return st;
  if ((st = check_tensor(dW, "dW")) != FORGE_OK) return st;
  if (dW->dtype != FORGE_F32) return fail(FORGE_ERR_DTYPE, "dW must be F32");
  if (dW->rows != g.N || dW->cols != g.K) return fail(FORGE_ERR_SHAPE, "dW must be [N, K]");
  if (g.N % 128 || g.K % 128) return fail(FORGE_ERR_SHAPE, "N and K must be multiples of 128");
  if (g.N * g.K >= (int64_t(1) << 32)) return fail(FORGE_ERR_SHAPE, "N * K must be below 2^32");
  const Range o = range_of(dW->data, bytes_of(dW), "dW");
  for (int j = 0; j < n_in; ++j)
    if (overlap(o, ins[j])) return fail(FORGE_ERR_ALIAS, "dW overlaps %s", ins[j].name);
  if (g.N == 0 || g.K == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  return to_status(forge::launch_wgrad_gemm(in_type, g, static_cast<float*>(dW->data), stream));
}

forge_status forge_optimizer_step(const forge_tensor* dW, forge_tensor* W, forge_tensor* m, forge_tensor* v,
                                  const forge_hyper* hyper, int32_t opt, int64_t step, uint64_t seed,
                                  const forge_step_opts* opts, void* stream) {
  g_last_error.clear();
  forge_status st;
  if ((st = check_tensor(dW, "dW")) != FORGE_OK) return st;
  if (dW->dtype != FORGE_F32) return fail(FORGE_ERR_DTYPE, "dW must be F32");
  Range outs[6];
  int n_out = 0;
  StepPlan plan;
  if ((st = validate_step_outputs(dW->rows, dW->cols, W, m, v, hyper, opt, step, seed, opts, &plan, outs, &n_out)) !=
      FORGE_OK)
    return st;
  const Range in = range_of(dW->data, bytes_of(dW), "dW");
  for (int i = 0; i < n_out; ++i)
    if (overlap(outs[i], in)) return fail(FORGE_ERR_ALIAS, "%s overlaps dW", outs[i].name);
  const int64_t n = dW->rows * dW->cols;
  if (n == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  return to_status(forge::launch_optimizer(plan.w_type, plan.s_type, opt, static_cast<const float*>(dW->data), n,
                                           plan.e, stream));
}

forge_status forge_dgrad(const forge_tensor* dY, const forge_tensor* W, forge_tensor* dX, void* stream) {
  g_last_error.clear();
  forge_status st;
  if ((st = check_tensor(dY, "dY")) != FORGE_OK) return st;
  if ((st = check_tensor(W, "W")) != FORGE_OK) return st;
  if ((st = check_tensor(dX, "dX")) != FORGE_OK) return st;
  if (dY->dtype != FORGE_BF16 || W->dtype != FORGE_BF16 || dX->dtype != FORGE_BF16)
    return fail(FORGE_ERR_DTYPE, "dgrad takes BF16 dY and W and writes BF16 dX");
  const int64_t T = dY->rows, N = dY->cols, K = W->cols;
  if (W->rows != N) return fail(FORGE_ERR_SHAPE, "W has %lld rows, dY has %lld columns", (long long)W->rows, (long long)N);
  if (dX->rows != T || dX->cols != K) return fail(FORGE_ERR_SHAPE, "dX must be [T, K]");
  if (N % 128 || K % 128) return fail(FORGE_ERR_SHAPE, "N and K must be multiples of 128");
  // the kernel addresses dY (padded to whole 256-token tiles) and W with 32-bit byte offsets
  if ((T + 256) * N * 2 >= (int64_t(1) << 32) || N * K * 2 >= (int64_t(1) << 32))
    return fail(FORGE_ERR_SHAPE, "dY (plus one tile of tokens) and W must each stay below 4 GiB");
  const Range o = range_of(dX->data, bytes_of(dX), "dX");
  if (overlap(o, range_of(dY->data, bytes_of(dY), "dY")) || overlap(o, range_of(W->data, bytes_of(W), "W")))
    return fail(FORGE_ERR_ALIAS, "dX overlaps an input");
  if (T == 0 || K == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  return to_status(forge::launch_dgrad(dY->data, W->data, dX->data, T, N, K, stream));
}

// Validation shared by the two backward-step entry points: both calls' arguments, before either
// is enqueued, so that an error leaves every buffer untouched.
static forge_status validate_backward(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W, forge_tensor* dX,
                                      forge_tensor* m, forge_tensor* v, const forge_hyper* hyper, int32_t opt,
                                      int64_t step, uint64_t seed, const forge_step_opts* opts, forge::GemmArgs* g,
                                      StepPlan* plan, Range* ranges, int* n_ranges) {
  Range ins[4], outs[6];
  int n_in = 0, n_out = 0, in_type = 0;
  forge_status st;
  if ((st = validate_inputs(X, dY, &in_type, g, ins, &n_in)) != FORGE_OK) return st;
  if ((st = validate_step_outputs(g->N, g->K, W, m, v, hyper, opt, step, seed, opts, plan, outs, &n_out)) != FORGE_OK)
    return st;
  if ((st = check_tensor(dX, "dX")) != FORGE_OK) return st;
  if (in_type != forge::FORGE_IN_BF16 || W->dtype != FORGE_BF16 || dX->dtype != FORGE_BF16)
    return fail(FORGE_ERR_DTYPE, "the backward step takes BF16 X, dY, W and dX");
  if (dX->rows != g->T || dX->cols != g->K) return fail(FORGE_ERR_SHAPE, "dX must be [T, K]");
  const Range rdx = range_of(dX->data, bytes_of(dX), "dX");
  for (int i = 0; i < n_out; ++i) {
    if (overlap(outs[i], rdx)) return fail(FORGE_ERR_ALIAS, "%s overlaps dX", outs[i].name);
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return fail(FORGE_ERR_ALIAS, "%s overlaps %s", outs[i].name, ins[j].name);
  }
  for (int j = 0; j < n_in; ++j)
    if (overlap(rdx, ins[j])) return fail(FORGE_ERR_ALIAS, "dX overlaps %s", ins[j].name);
  int n = 0;
  for (int j = 0; j < n_in; ++j) ranges[n++] = ins[j];
  for (int i = 0; i < n_out; ++i) ranges[n++] = outs[i];
  ranges[n++] = rdx;
  *n_ranges = n;
  return FORGE_OK;
}

forge_status forge_linear_backward_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                                        forge_tensor* dX, forge_tensor* m, forge_tensor* v, const forge_hyper* hyper,
                                        int32_t opt, int64_t step, uint64_t seed, const forge_step_opts* opts,
                                        void* stream) {
  g_last_error.clear();
  forge::GemmArgs g{};
  StepPlan plan;
  Range ranges[11];
  int n_ranges = 0;
  forge_status st;
  if ((st = validate_backward(X, dY, W, dX, m, v, hyper, opt, step, seed, opts, &g, &plan, ranges, &n_ranges)) !=
      FORGE_OK)
    return st;
  if ((st = forge_dgrad(dY, W, dX, stream)) != FORGE_OK) return st;
  return forge_wgrad_step(X, dY, W, m, v, hyper, opt, step, seed, opts, stream);
}

int64_t forge_backward_workspace_bytes(int64_t K) {
  if (K < 0 || K > (int64_t(1) << 40)) return -1;
  return 4 * forge::backward_workspace_words(K);
}

// Checks of the one-launch backward step beyond the backward step's own.
static forge_status validate_one_launch(const forge::GemmArgs& g) {
  if (g.N % 256 || g.K % 128)
    return fail(FORGE_ERR_SHAPE, "the one-launch backward step needs N %% 256 == 0 and K %% 128 == 0");
  // the dX tiles address dY (padded to whole 256-token tiles) and W with 32-bit byte offsets
  if ((g.T + 256) * g.N * 2 >= (int64_t(1) << 32) || g.N * g.K * 2 >= (int64_t(1) << 32))
    return fail(FORGE_ERR_SHAPE, "dY (plus one tile of tokens) and W must each stay below 4 GiB");
  if (g.N * g.K >= (int64_t(1) << 32)) return fail(FORGE_ERR_SHAPE, "N * K must be below 2^32");
  return FORGE_OK;
}

forge_status forge_linear_backward_step_fused(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                                              forge_tensor* dX, forge_tensor* m, forge_tensor* v,
                                              const forge_hyper* hyper, int32_t opt, int64_t step, uint64_t seed,
                                              const forge_step_opts* opts, void* workspace, int64_t workspace_bytes,
                                              void* stream) {
  g_last_error.clear();
  forge::GemmArgs g{};
  StepPlan plan;
  Range ranges[11];
  int n_ranges = 0;
  forge_status st;
  if ((st = validate_backward(X, dY, W, dX, m, v, hyper, opt, step, seed, opts, &g, &plan, ranges, &n_ranges)) !=
      FORGE_OK)
    return st;
  if ((st = validate_one_launch(g)) != FORGE_OK) return st;
  const int64_t need = forge_backward_workspace_bytes(g.K);
  if (!workspace) return fail(FORGE_ERR_ARG, "workspace is NULL");
  if (!aligned4(workspace)) return fail(FORGE_ERR_LAYOUT, "workspace is not 4-byte aligned");
  if (workspace_bytes < need)
    return fail(FORGE_ERR_ARG, "workspace has %lld bytes, the call needs %lld", (long long)workspace_bytes,
                (long long)need);
  const Range rw = range_of(workspace, need, "workspace");
  for (int i = 0; i < n_ranges; ++i)
    if (overlap(rw, ranges[i])) return fail(FORGE_ERR_ALIAS, "workspace overlaps %s", ranges[i].name);
  if (g.N == 0 || g.K == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  return to_status(forge::launch_backward_step(plan.s_type, opt, g, plan.e, W->data, dX->data,
                                               static_cast<int*>(workspace), stream));
}

forge_status forge_linear_backward_step_fused_noalloc(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                                                      forge_tensor* dX, forge_tensor* m, forge_tensor* v,
                                                      const forge_hyper* hyper, int32_t opt, int64_t step,
                                                      uint64_t seed, const forge_step_opts* opts, void* stream) {
  g_last_error.clear();
  forge::GemmArgs g{};
  StepPlan plan;
  Range ranges[11];
  int n_ranges = 0;
  forge_status st;
  if ((st = validate_backward(X, dY, W, dX, m, v, hyper, opt, step, seed, opts, &g, &plan, ranges, &n_ranges)) !=
      FORGE_OK)
    return st;
  if ((st = validate_one_launch(g)) != FORGE_OK) return st;
  if (forge::backward_workspace_words(g.K) > forge::kBackwardScratchWords)
    return fail(FORGE_ERR_SHAPE, "K = %lld is beyond the allocation-free variant's limit of %lld columns",
                (long long)g.K, (long long)(forge::kBackwardScratchWords - forge::backward_workspace_words(0)) * 128);
  if (g.N == 0 || g.K == 0) return FORGE_OK;
  if ((st = device_ok()) != FORGE_OK) return st;
  int* counters = nullptr;
  const int herr = forge::backward_scratch(&counters);
  if (herr != (int)hipSuccess)
    return fail(FORGE_ERR_LAUNCH, "the device address of the library's counters: %s", hipGetErrorString((hipError_t)herr));
  return to_status(forge::launch_backward_step(plan.s_type, opt, g, plan.e, W->data, dX->data, counters, stream));
}

forge_status forge_step_scalars(int32_t opt, const forge_hyper* hyper, int64_t step, float* out, int32_t n_out) {
  g_last_error.clear();
  forge::OptScalars s;
  forge_status st = compute_scalars(opt, hyper, step, &s);
  if (st != FORGE_OK) return st;
  if (!out && n_out > 0) return fail(FORGE_ERR_ARG, "out is NULL");
  const float v[12] = {s.decay, s.l2, s.c1, s.c2, s.c3, s.b1, s.omb1, s.b2, s.omb2, s.eps, s.lr, (float)s.rect};
  for (int i = 0; i < n_out && i < 12; ++i) out[i] = v[i];
  return FORGE_OK;
}

const char* forge_status_string(forge_status s) {
  switch (s) {
    case FORGE_OK: return "ok";
    case FORGE_ERR_ARG: return "invalid argument";
    case FORGE_ERR_SHAPE: return "invalid shape";
    case FORGE_ERR_DTYPE: return "unsupported dtype";
    case FORGE_ERR_LAYOUT: return "invalid layout or alignment";
    case FORGE_ERR_ALIAS: return "overlapping buffers";
    case FORGE_ERR_DEVICE: return "unsupported device";
    case FORGE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* forge_last_error(void) { return g_last_error.c_str(); }

int32_t forge_version(void) { return FORGE_VERSION; }

#ifndef FORGE_BUILD_ID
#define FORGE_BUILD_ID "unknown"
#endif
const char* forge_build_id(void) { return FORGE_BUILD_ID; }

forge_status forge_device_check(int32_t device) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count == 0) return fail(FORGE_ERR_DEVICE, "no HIP device");
  if (device < 0 || device >= count) return fail(FORGE_ERR_DEVICE, "device %d does not exist", (int)device);
  hipDeviceProp_t p;
  e = hipGetDeviceProperties(&p, device);
  if (e != hipSuccess) return fail(FORGE_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(FORGE_ERR_DEVICE, "device %d is %s; this library is built for gfx950", (int)device, p.gcnArchName);
  if (device < 64) g_dev_ok[device].store(1, std::memory_order_relaxed);
  return FORGE_OK;
}

}  // extern "C"
