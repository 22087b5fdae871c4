// C ABI of the forge library: host-side validation, per-step scalars and
// dispatch to the gfx950 kernels. Nothing here allocates device memory or
// synchronises the host; every error is detected before anything is enqueued.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "forge_internal.h"

using namespace forge;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

int elem_size(int dt) { return dt == FORGE_F32 ? 4 : dt == FORGE_BF16 ? 2 : 1; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte range a row-major tensor may touch.
struct Range {
  uintptr_t lo, hi;
};
Range range_of(const forge_tensor* t) {
  const uintptr_t lo = (uintptr_t)t->data;
  const int64_t n = t->rows == 0 ? 0 : ((t->rows - 1) * t->ld + t->cols) * elem_size(t->dtype);
  return Range{lo, lo + (uintptr_t)n};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

int check_shape(const forge_tensor* t) {
  if (t->rows < 0 || t->cols < 0 || t->rows >= kMaxDim || t->cols >= kMaxDim) return FORGE_ERR_SHAPE;
  if (t->ld < t->cols) return FORGE_ERR_SHAPE;
  return FORGE_OK;
}

// Dense io tensor (X, dY, W, dX): fp32 or bf16, 16-byte vectors along rows.
int check_io(const forge_tensor* t, int dtype) {
  if (!t) return FORGE_ERR_NULL;
  if (!t->data && t->rows != 0 && t->cols != 0) return FORGE_ERR_NULL;  // empty tensors may be NULL
  if (t->dtype != dtype) return FORGE_ERR_DTYPE;
  int r = check_shape(t);
  if (r) return r;
  const int ve = dtype == FORGE_BF16 ? 8 : 4;
  if (!aligned16(t->data) || t->cols % ve || t->ld % ve) return FORGE_ERR_ALIGN;
  return FORGE_OK;
}

bool is_fp8(int dt) { return dt == FORGE_E4M3 || dt == FORGE_E5M2; }

// FP8 input tensor (X, dY): one byte per element, 16-byte chunks along rows, and a
// device pointer to its float32 dequantisation scale.
int check_fp8(const forge_tensor* t, bool allow_e5m2) {
  if (!t) return FORGE_ERR_NULL;
  if (!t->data && t->rows != 0 && t->cols != 0) return FORGE_ERR_NULL;
  if (!(t->dtype == FORGE_E4M3 || (allow_e5m2 && t->dtype == FORGE_E5M2))) return FORGE_ERR_DTYPE;
  if (!t->scale) return FORGE_ERR_NULL;
  int r = check_shape(t);
  if (r) return r;
  if (!aligned16(t->data) || ((uintptr_t)t->scale & 3u) || t->cols % 16 || t->ld % 16) return FORGE_ERR_ALIGN;
  return FORGE_OK;
}

bool finite(double x) { return isfinite(x) != 0; }

// The kernels address each tensor through 32-bit byte offsets below 2^31.
bool fits_31(const forge_tensor* t) {
  return !t || !t->data || t->rows * t->ld * (int64_t)elem_size(t->dtype) < ((int64_t)1 << 31);
}

int check_hyper(int opt, const forge_hyper* h, int64_t step) {
  if (!h) return FORGE_ERR_NULL;
  if (opt < FORGE_ADAMW || opt > FORGE_RADAM) return FORGE_ERR_HYPER;
  if (step < 1 || step >= ((int64_t)1 << 31)) return FORGE_ERR_HYPER;
  const double f[] = {h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->momentum, h->dampening, h->alpha,
                      h->lr_decay, h->momentum_decay};
  for (double x : f)
    if (!finite(x)) return FORGE_ERR_HYPER;
  if (h->lr < 0.0 || h->eps < 0.0 || h->lr_decay < 0.0) return FORGE_ERR_HYPER;
  switch (opt) {
    case FORGE_ADAMW:
    case FORGE_NADAM:
    case FORGE_RADAM:
    case FORGE_LION:
      if (h->beta1 < 0.0 || h->beta1 >= 1.0 || h->beta2 < 0.0 || h->beta2 >= 1.0) return FORGE_ERR_HYPER;
      if (opt == FORGE_NADAM && h->momentum_decay < 0.0) return FORGE_ERR_HYPER;
      break;
    case FORGE_SGD_MOMENTUM:
      if (h->momentum < 0.0 || h->momentum >= 1.0 || h->dampening < 0.0 || h->dampening > 1.0) return FORGE_ERR_HYPER;
      break;
    case FORGE_RMSPROP:
      if (h->alpha < 0.0 || h->alpha >= 1.0) return FORGE_ERR_HYPER;
      break;
    default:
      break;
  }
  if (opt == FORGE_RADAM && h->beta2 <= 0.0) return FORGE_ERR_HYPER;
  return FORGE_OK;
}

// Moment slots: returns the state format (ST_F32 / ST_Q8 / ST_Q8D / ST_BF16) or a negative status.
int check_states(int opt, int io_dtype, const forge_tensor* W, const forge_tensor* m, const forge_tensor* v) {
  const int sl = opt_slots(opt);
  const forge_tensor* slot[2] = {m, v};
  int fmt = -1;
  for (int k = 0; k < 2; ++k) {
    if (!(sl & (1 << k))) continue;
    const forge_tensor* t = slot[k];
    if (!t || (!t->data && t->rows != 0 && t->cols != 0)) return FORGE_ERR_NULL;  // empty states may be NULL
    int r = check_shape(t);
    if (r) return r;
    if (t->rows != W->rows || t->cols != W->cols) return FORGE_ERR_SHAPE;
    int f;
    if (t->dtype == FORGE_F32) {
      f = ST_F32;
      if (!aligned16(t->data) || t->ld % 4) return FORGE_ERR_ALIGN;
    } else if (t->dtype == FORGE_BF16) {
      f = ST_BF16;
      if (io_dtype != FORGE_BF16) return FORGE_ERR_DTYPE;
      if (!aligned16(t->data) || t->ld % 8) return FORGE_ERR_ALIGN;
    } else if ((k == 0 && (t->dtype == FORGE_I8 || t->dtype == FORGE_I8_DYN)) ||
               (k == 1 && (t->dtype == FORGE_U8 || t->dtype == FORGE_U8_DYN))) {
      f = (t->dtype == FORGE_I8 || t->dtype == FORGE_U8) ? ST_Q8 : ST_Q8D;
      if (io_dtype != FORGE_BF16) return FORGE_ERR_DTYPE;
      if (!t->scale) return FORGE_ERR_NULL;
      if (!aligned16(t->data) || t->ld % 16 || ((uintptr_t)t->scale & 3u)) return FORGE_ERR_ALIGN;
      if (t->cols % 64) return FORGE_ERR_UNSUPPORTED;
    } else {
      return FORGE_ERR_DTYPE;
    }
    if (fmt >= 0 && f != fmt) return FORGE_ERR_DTYPE;
    fmt = f;
  }
  return fmt < 0 ? ST_F32 : fmt;
}

// Byte range of a tensor's scale: the [rows, cols / 64] float32 block scales of an INT8
// state, the one float32 dequantisation scale of an FP8 input; empty otherwise.
Range scale_range_of(const forge_tensor* t) {
  const uintptr_t lo = (uintptr_t)t->scale;
  if (!t->scale) return Range{0, 0};
  if (is_fp8(t->dtype)) return Range{lo, lo + 4};
  if (t->dtype == FORGE_I8 || t->dtype == FORGE_U8 || t->dtype == FORGE_I8_DYN || t->dtype == FORGE_U8_DYN)
    return Range{lo, lo + (uintptr_t)(t->rows * (t->cols / 64) * 4)};
  return Range{0, 0};
}

// Everything an output writes (its data and block scales) must overlap nothing else the
// call reads or writes: other outputs' data and scales, inputs' data and scales.
int check_alias(const forge_tensor* const* outs, int n_out, const forge_tensor* const* ins, int n_in) {
  for (int a = 0; a < n_out; ++a) {
    if (!outs[a]) continue;
    const Range wa[2] = {range_of(outs[a]), scale_range_of(outs[a])};
    for (const Range& ra : wa) {
      for (int b = 0; b < n_out; ++b) {
        if (!outs[b]) continue;
        if (b != a && overlap(ra, range_of(outs[b]))) return FORGE_ERR_ALIAS;
        if (overlap(ra, scale_range_of(outs[b])) && !(b == a && &ra == &wa[1])) return FORGE_ERR_ALIAS;
      }
      for (int b = 0; b < n_in; ++b)
        if (ins[b] && (overlap(ra, range_of(ins[b])) || overlap(ra, scale_range_of(ins[b])))) return FORGE_ERR_ALIAS;
    }
  }
  return FORGE_OK;
}

OptArgs make_args(forge_tensor* W, forge_tensor* m, forge_tensor* v, int opt, const forge_scalars& s,
                  uint64_t seed, int64_t step) {
  const int sl = opt_slots(opt);
  OptArgs a{};
  a.W = W->data;
  a.ldw = W->ld;
  if (sl & 1) {
    a.m = m->data;
    a.ldm = m->ld;
    a.m_scale = m->scale;
  }
  if (sl & 2) {
    a.v = v->data;
    a.ldv = v->ld;
    a.v_scale = v->scale;
  }
  a.out = (int32_t)W->rows;
  a.in = (int32_t)W->cols;
  a.rng_base = rng_base(seed, (uint64_t)step);
  a.s = s;
  return a;
}

// Scratch of the no-allocation unfused baseline: the float32 dW of a layer of at most
// kScratchElems weights (64 MiB) in a file-scope device array. Every GPU the library runs
// on holds its own copy until the process ends; host code addresses it only through the
// device pointer hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address), fetched once per device and kept.
constexpr int64_t kScratchElems = (int64_t)1 << 24;
static __device__ __align__(256) float scratch[kScratchElems];
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FORGE_ERR_HIP;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return FORGE_ERR_HIP;
      p = static_cast<float*>(q);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FORGE_OK;
}

// A validated step: what the launches need.
struct StepPlan {
  int io, fmt, sr;
  bool f8, empty;
  OptArgs a;
  GemmDims d;
};

// Validates the arguments of a weight-gradient step (fused, or unfused through the float32
// workspace ws [out, ld_ws] when ws is not NULL) and fills *p. Nothing is enqueued.
int plan_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W, forge_tensor* m, forge_tensor* v,
              int32_t opt, const forge_hyper* hyper, int64_t step, uint64_t seed, float* ws, int64_t ld_ws,
              StepPlan* p) {
  if (!X || !dY || !W) return FORGE_ERR_NULL;
  int r = check_hyper(opt, hyper, step);
  if (r) return r;
  const int io = W->dtype;
  if (io != FORGE_F32 && io != FORGE_BF16) return FORGE_ERR_DTYPE;
  const bool f8 = is_fp8(X->dtype) || is_fp8(dY->dtype);
  if (f8) {
    if (io != FORGE_BF16) return FORGE_ERR_DTYPE;
    if ((r = check_fp8(X, false)) || (r = check_fp8(dY, true)) || (r = check_io(W, io))) return r;
  } else if ((r = check_io(X, io)) || (r = check_io(dY, io)) || (r = check_io(W, io))) {
    return r;
  }
  if (X->rows != dY->rows || X->cols != W->cols || dY->cols != W->rows) return FORGE_ERR_SHAPE;
  const int fmt = check_states(opt, io, W, m, v);
  if (fmt < 0) return fmt;
  if (W->rows * W->cols >= ((int64_t)1 << 32)) return FORGE_ERR_UNSUPPORTED;
  const int sl = opt_slots(opt);
  if (!fits_31(X) || !fits_31(dY) || !fits_31(W) || ((sl & 1) && !fits_31(m)) || ((sl & 2) && !fits_31(v)))
    return FORGE_ERR_UNSUPPORTED;
  const forge_tensor* ins[2] = {X, dY};
  if (ws) {
    // the workspace is written by the GEMM and read by the optimizer pass: it may overlap
    // nothing else
    if (ld_ws < W->cols) return FORGE_ERR_SHAPE;
    if (((uintptr_t)ws & 15u) || ld_ws % 4) return FORGE_ERR_ALIGN;
    const forge_tensor wst{ws, FORGE_F32, 0, W->rows, W->cols, ld_ws, nullptr};
    if (!fits_31(&wst)) return FORGE_ERR_UNSUPPORTED;
    const forge_tensor* outs4[4] = {W, (sl & 1) ? m : nullptr, (sl & 2) ? v : nullptr, &wst};
    if ((r = check_alias(outs4, 4, ins, 2))) return r;
  } else {
    const forge_tensor* outs[3] = {W, (sl & 1) ? m : nullptr, (sl & 2) ? v : nullptr};
    if ((r = check_alias(outs, 3, ins, 2))) return r;
  }
  forge_scalars sc;
  if ((r = forge_step_scalars(opt, hyper, step, &sc))) return r;
  p->io = io;
  p->fmt = fmt;
  p->f8 = f8;
  p->sr = (io == FORGE_BF16 && hyper->stochastic_round) ? 1 : 0;
  p->empty = W->rows == 0 || W->cols == 0;
  p->a = make_args(W, m, v, opt, sc, seed, step);
  p->d = GemmDims{(int32_t)X->rows, (int32_t)W->rows, (int32_t)W->cols, X->ld, dY->ld};
  return FORGE_OK;
}

// The two-phase baseline on a validated plan: float32 dW into ws, then the optimizer pass.
int enqueue_unfused(const forge_tensor* X, const forge_tensor* dY, const StepPlan& p, int32_t opt, float* ws,
                    int64_t ld_ws, hipStream_t st) {
  hipError_t e = p.f8 ? launch_wgrad_store_f8(dY->dtype == FORGE_E5M2, X->data, X->scale, dY->data, dY->scale, p.d,
                                              ws, ld_ws, st)
                      : launch_wgrad_store(p.io == FORGE_BF16, X->data, dY->data, p.d, ws, ld_ws, st);
  if (e != hipSuccess) return FORGE_ERR_HIP;
  e = launch_optimizer(p.io == FORGE_BF16, p.fmt, opt, p.sr, ws, ld_ws, p.a, st);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

}  // namespace

extern "C" {

int forge_version(void) { return 100; }

const char* forge_status_str(int status) {
  switch (status) {
    case FORGE_OK: return "ok";
    case FORGE_ERR_NULL: return "a required pointer is NULL";
    case FORGE_ERR_SHAPE: return "tensor dimensions are inconsistent";
    case FORGE_ERR_DTYPE: return "unsupported dtype combination";
    case FORGE_ERR_ALIGN: return "pointer not 16-byte aligned or cols/ld not a multiple of the vector width";
    case FORGE_ERR_UNSUPPORTED: return "size not supported by the kernels";
    case FORGE_ERR_HYPER: return "invalid optimizer, step or hyper-parameter";
    case FORGE_ERR_HIP: return "HIP kernel launch failed";
    case FORGE_ERR_ALIAS: return "output tensors overlap each other or an input";
    case FORGE_ERR_SCRATCH: return "the layer's float32 dW exceeds the no-allocation scratch (2^24 elements)";
    default: return "unknown status";
  }
}

int forge_default_hyper(int32_t opt, forge_hyper* h) {
  if (!h) return FORGE_ERR_NULL;
  if (opt < FORGE_ADAMW || opt > FORGE_RADAM) return FORGE_ERR_HYPER;
  *h = forge_hyper{};
  h->lr = 1e-3;
  h->beta1 = 0.9;
  h->beta2 = 0.999;
  h->eps = 1e-8;
  h->alpha = 0.99;
  h->momentum_decay = 4e-3;
  h->stochastic_round = 1;
  switch (opt) {
    case FORGE_ADAMW: h->weight_decay = 0.01; break;
    case FORGE_SGD_MOMENTUM: h->momentum = 0.9; break;
    case FORGE_LION:
      h->lr = 1e-4;
      h->beta2 = 0.99;
      h->weight_decay = 0.1;
      break;
    case FORGE_ADAGRAD: h->eps = 1e-10; break;
    default: break;
  }
  return FORGE_OK;
}

int forge_step_scalars(int32_t opt, const forge_hyper* h, int64_t step, forge_scalars* out) {
  if (!out) return FORGE_ERR_NULL;
  int r = check_hyper(opt, h, step);
  if (r) return r;
  const double t = (double)step;
  const double lr = h->lr, b1 = h->beta1, b2 = h->beta2, wd = h->weight_decay;
  forge_scalars s{};
  s.opt = opt;
  s.lr = (float)lr;
  s.wd = (float)wd;
  s.eps = (float)h->eps;
  s.decay = (float)(1.0 - lr * wd);
  s.b1 = (float)b1;
  s.omb1 = (float)(1.0 - b1);
  s.b2 = (float)b2;
  s.omb2 = (float)(1.0 - b2);
  const double bc1 = 1.0 - pow(b1, t), bc2 = 1.0 - pow(b2, t);
  switch (opt) {
    case FORGE_ADAMW:
      s.step_size = (float)(lr / bc1);
      s.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
      break;
    case FORGE_SGD_MOMENTUM: {
      const double mu = h->momentum;
      // The momentum buffer starts as the first (decayed) gradient itself.
      s.b1 = step == 1 ? 0.f : (float)mu;
      s.omb1 = step == 1 ? 1.f : (float)(1.0 - h->dampening);
      s.c_m = (float)mu;
      s.flag = h->nesterov ? 1 : 0;
      break;
    }
    case FORGE_RMSPROP:
      s.b2 = (float)h->alpha;
      s.omb2 = (float)(1.0 - h->alpha);
      break;
    case FORGE_ADAGRAD:
      s.lr = (float)(lr / (1.0 + (t - 1.0) * h->lr_decay));
      break;
    case FORGE_NADAM: {
      // mu_k = beta1 (1 - q^k / 2) with q = 0.96^psi. The product over k <= t has an
      // exact series of constant cost in t (psi >= 0, so q^k / 2 <= 1/2):
      //   log prod_{k<=t} (1 - q^k / 2) = -sum_{n>=1} (2^-n / n) q^n (1 - q^(n t)) / (1 - q^n),
      // both differences through expm1; 64 terms reach double precision (terms ~ 2^-n).
      const double L = h->momentum_decay * log(0.96);  // log q
      auto mu = [&](double k) { return b1 * (1.0 - 0.5 * exp(k * L)); };
      double S = 0.0, half_n = 1.0;
      for (int n = 1; n <= 64; ++n) {
        half_n *= 0.5;
        const double ratio = (L == 0.0) ? t : expm1((double)n * t * L) / expm1((double)n * L);
        S += half_n / n * exp((double)n * L) * ratio;
      }
      const double prod = b1 > 0.0 ? exp(t * log(b1) - S) : 0.0;
      const double mu_t = mu(t), mu_n = mu(t + 1.0);
      s.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
      s.c_g = (float)(lr * (1.0 - mu_t) / (1.0 - prod));
      s.c_m = (float)(lr * mu_n / (1.0 - prod * mu_n));
      break;
    }
    case FORGE_RADAM: {
      const double rho_inf = 2.0 / (1.0 - b2) - 1.0;
      const double rho_t = rho_inf - 2.0 * t * pow(b2, t) / bc2;
      if (rho_t > 5.0) {
        const double rect = sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t));
        s.flag = 1;
        s.step_size = (float)(lr * rect * sqrt(bc2) / bc1);
      } else {
        s.flag = 0;
        s.step_size = (float)(lr / bc1);
      }
      break;
    }
    default:
      break;
  }
  *out = s;
  return FORGE_OK;
}

uint32_t forge_rand16(uint64_t seed, int64_t step, uint32_t idx) {
  return rand16_from_base(rng_base(seed, (uint64_t)step), idx);
}

uint16_t forge_sr_bf16(float x, uint32_t r16) { return (uint16_t)sr_bf16_bits(x, r16 & 0xFFFFu); }

// Host copy of the dynamic-code tables (the same constexpr construction as the
// kernels' constant-memory copy).
static constexpr DynTables kDynHost = make_dyn_tables();

float forge_dyn_value(int32_t is_signed, int32_t code) {
  if (code < 0 || code > 255) return __builtin_nanf("");
  return is_signed ? dyn_decode_s((uint32_t)code, kDynHost.vs) : kDynHost.vu[code];
}

int32_t forge_dyn_encode(int32_t is_signed, float y) {
  return (int32_t)(is_signed ? dyn_encode_s(y, kDynHost.ms) : dyn_encode_u(y, kDynHost.mu));
}

int forge_linear_wgrad_step(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W, forge_tensor* m,
                            forge_tensor* v, int32_t opt, const forge_hyper* hyper, int64_t step, uint64_t seed,
                            forge_stream_t stream) {
  StepPlan p;
  int r = plan_step(X, dY, W, m, v, opt, hyper, step, seed, nullptr, 0, &p);
  if (r || p.empty) return r;
  hipError_t e = p.f8 ? launch_wgrad_fused_f8(dY->dtype == FORGE_E5M2, p.fmt, opt, p.sr, X->data, X->scale, dY->data,
                                              dY->scale, p.d, p.a, (hipStream_t)stream)
                      : launch_wgrad_fused(p.io == FORGE_BF16, p.fmt, opt, p.sr, X->data, dY->data, p.d, p.a,
                                           (hipStream_t)stream);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

int forge_linear_wgrad_step_group(const forge_tensor* X, int32_t n_layers, const forge_tensor* dY, forge_tensor* W,
                                  forge_tensor* m, forge_tensor* v, int32_t opt, const forge_hyper* hyper,
                                  int64_t step, const uint64_t* seeds, forge_stream_t stream) {
  if (!X || !dY || !W || !seeds) return FORGE_ERR_NULL;
  if (n_layers < 1 || n_layers > FORGE_MAX_GROUP) return FORGE_ERR_SHAPE;
  StepPlan p[FORGE_MAX_GROUP];
  for (int l = 0; l < n_layers; ++l) {
    int r = plan_step(X, &dY[l], &W[l], m ? &m[l] : nullptr, v ? &v[l] : nullptr, opt, hyper, step, seeds[l],
                      nullptr, 0, &p[l]);
    if (r) return r;
    if (p[l].io != FORGE_BF16) return FORGE_ERR_UNSUPPORTED;
    // one operand format and one moment format for the whole group
    if (p[l].f8 != p[0].f8 || (p[l].f8 && dY[l].dtype != dY[0].dtype) || p[l].fmt != p[0].fmt) return FORGE_ERR_DTYPE;
  }
  // a layer's outputs overlap no other layer's tensors (each plan checked its own)
  const int sl = opt_slots(opt);
  const forge_tensor* outs[3 * FORGE_MAX_GROUP];
  const forge_tensor* ins[FORGE_MAX_GROUP + 1];
  int n_out = 0;
  ins[0] = X;
  for (int l = 0; l < n_layers; ++l) {
    outs[n_out++] = &W[l];
    outs[n_out++] = (sl & 1) ? &m[l] : nullptr;
    outs[n_out++] = (sl & 2) ? &v[l] : nullptr;
    ins[l + 1] = &dY[l];
  }
  int r = check_alias(outs, n_out, ins, n_layers + 1);
  if (r) return r;
  GroupLayer layers[FORGE_MAX_GROUP];
  int n = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (p[l].empty) continue;  // no weights: nothing to update
    layers[n++] = GroupLayer{dY[l].data, dY[l].ld, dY[l].scale, p[l].a};
  }
  if (n == 0) return FORGE_OK;
  const StepPlan& p0 = p[0];
  hipError_t e = p0.f8 ? launch_wgrad_fused_f8_group(dY[0].dtype == FORGE_E5M2, p0.fmt, opt, p0.sr, X->data, X->scale,
                                                     p0.d, layers, n, (hipStream_t)stream)
                       : launch_wgrad_fused_bf16_group(p0.fmt, opt, p0.sr, X->data, p0.d, layers, n, (hipStream_t)stream);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

int forge_linear_wgrad_unfused(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W, forge_tensor* m,
                               forge_tensor* v, int32_t opt, const forge_hyper* hyper, int64_t step, uint64_t seed,
                               float* dW_workspace, int64_t ld_ws, forge_stream_t stream) {
  // a layer with no elements needs no workspace
  if (!dW_workspace && !(W && (W->rows == 0 || W->cols == 0))) return FORGE_ERR_NULL;
  StepPlan p;
  int r = plan_step(X, dY, W, m, v, opt, hyper, step, seed, dW_workspace, ld_ws, &p);
  if (r || p.empty) return r;
  return enqueue_unfused(X, dY, p, opt, dW_workspace, ld_ws, (hipStream_t)stream);
}

int forge_linear_wgrad_unfused_noalloc(const forge_tensor* X, const forge_tensor* dY, forge_tensor* W,
                                       forge_tensor* m, forge_tensor* v, int32_t opt, const forge_hyper* hyper,
                                       int64_t step, uint64_t seed, forge_stream_t stream) {
  StepPlan p;
  int r = plan_step(X, dY, W, m, v, opt, hyper, step, seed, nullptr, 0, &p);
  if (r || p.empty) return r;
  if (W->rows * W->cols > kScratchElems) return FORGE_ERR_SCRATCH;
  float* ws = nullptr;
  if ((r = scratch_of_current_device(&ws))) return r;
  return enqueue_unfused(X, dY, p, opt, ws, W->cols, (hipStream_t)stream);
}

int forge_linear_dgrad(const forge_tensor* dY, const forge_tensor* W, forge_tensor* dX, forge_stream_t stream) {
  if (!dY || !W || !dX) return FORGE_ERR_NULL;
  if (is_fp8(dY->dtype)) return FORGE_ERR_UNSUPPORTED;
  const int io = W->dtype;
  if (io != FORGE_F32 && io != FORGE_BF16) return FORGE_ERR_DTYPE;
  int r;
  if ((r = check_io(dY, io)) || (r = check_io(W, io)) || (r = check_io(dX, io))) return r;
  if (dY->cols != W->rows || dX->rows != dY->rows || dX->cols != W->cols) return FORGE_ERR_SHAPE;
  if (!fits_31(dY) || !fits_31(W) || !fits_31(dX)) return FORGE_ERR_UNSUPPORTED;
  const forge_tensor* outs[1] = {dX};
  const forge_tensor* ins[2] = {dY, W};
  if ((r = check_alias(outs, 1, ins, 2))) return r;
  if (dX->rows == 0 || dX->cols == 0) return FORGE_OK;
  hipError_t e = launch_dgrad(io == FORGE_BF16, dY->data, dY->ld, W->data, W->ld, dX->data, dX->ld,
                              (int32_t)dY->rows, (int32_t)W->rows, (int32_t)W->cols, (hipStream_t)stream);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

int forge_linear_wgrad(const forge_tensor* X, const forge_tensor* dY, float* dW, int64_t ld_dw,
                       forge_stream_t stream) {
  if (!X || !dY || !dW) return FORGE_ERR_NULL;
  const int io = X->dtype;
  const bool f8 = is_fp8(X->dtype) || is_fp8(dY->dtype);
  if (!f8 && io != FORGE_F32 && io != FORGE_BF16) return FORGE_ERR_DTYPE;
  int r;
  if (f8) {
    if ((r = check_fp8(X, false)) || (r = check_fp8(dY, true))) return r;
  } else if ((r = check_io(X, io)) || (r = check_io(dY, io))) {
    return r;
  }
  if (X->rows != dY->rows) return FORGE_ERR_SHAPE;
  if (ld_dw < X->cols) return FORGE_ERR_SHAPE;
  if (!aligned16(dW) || ld_dw % 4) return FORGE_ERR_ALIGN;
  const forge_tensor dWt{dW, FORGE_F32, 0, dY->cols, X->cols, ld_dw, nullptr};
  if (!fits_31(X) || !fits_31(dY) || !fits_31(&dWt)) return FORGE_ERR_UNSUPPORTED;
  const forge_tensor* outs[1] = {&dWt};
  const forge_tensor* ins[2] = {X, dY};
  if ((r = check_alias(outs, 1, ins, 2))) return r;
  if (dY->cols == 0 || X->cols == 0) return FORGE_OK;
  const GemmDims d{(int32_t)X->rows, (int32_t)dY->cols, (int32_t)X->cols, X->ld, dY->ld};
  hipError_t e = f8 ? launch_wgrad_store_f8(dY->dtype == FORGE_E5M2, X->data, X->scale, dY->data, dY->scale, d, dW,
                                            ld_dw, (hipStream_t)stream)
                    : launch_wgrad_store(io == FORGE_BF16, X->data, dY->data, d, dW, ld_dw, (hipStream_t)stream);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

int forge_optimizer_step(const float* dW, int64_t ld_dw, forge_tensor* W, forge_tensor* m, forge_tensor* v,
                         int32_t opt, const forge_hyper* hyper, int64_t step, uint64_t seed, forge_stream_t stream) {
  if (!dW || !W) return FORGE_ERR_NULL;
  int r = check_hyper(opt, hyper, step);
  if (r) return r;
  const int io = W->dtype;
  if (io != FORGE_F32 && io != FORGE_BF16) return FORGE_ERR_DTYPE;
  if ((r = check_io(W, io))) return r;
  if (ld_dw < W->cols) return FORGE_ERR_SHAPE;
  if (!aligned16(dW) || ld_dw % 4) return FORGE_ERR_ALIGN;
  const int fmt = check_states(opt, io, W, m, v);
  if (fmt < 0) return fmt;
  if (W->rows * W->cols >= ((int64_t)1 << 32)) return FORGE_ERR_UNSUPPORTED;
  const int sl = opt_slots(opt);
  const forge_tensor dWt{const_cast<float*>(dW), FORGE_F32, 0, W->rows, W->cols, ld_dw, nullptr};
  const forge_tensor* outs[3] = {W, (sl & 1) ? m : nullptr, (sl & 2) ? v : nullptr};
  const forge_tensor* ins[1] = {&dWt};
  if ((r = check_alias(outs, 3, ins, 1))) return r;
  forge_scalars s;
  if ((r = forge_step_scalars(opt, hyper, step, &s))) return r;
  if (W->rows == 0 || W->cols == 0) return FORGE_OK;
  const OptArgs a = make_args(W, m, v, opt, s, seed, step);
  const int sr = (io == FORGE_BF16 && hyper->stochastic_round) ? 1 : 0;
  hipError_t e = launch_optimizer(io == FORGE_BF16, fmt, opt, sr, dW, ld_dw, a, (hipStream_t)stream);
  return e == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

}  // extern "C"
