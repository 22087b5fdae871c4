// Launch entry points of the GEMM core (kernel and configurations in
// forge_gemm_kernel.h): the fused weight-gradient + optimizer step on bf16 / fp32
// or FP8 operands, the float32 dW store of the two-phase baseline, and dgrad.
#include "forge_gemm_kernel.h"

namespace forge {

FORGE_EXTERN_BF16(FORGE_ADAMW)
FORGE_EXTERN_BF16(FORGE_SGD)
FORGE_EXTERN_BF16(FORGE_SGD_MOMENTUM)
FORGE_EXTERN_BF16(FORGE_LION)
FORGE_EXTERN_BF16(FORGE_RMSPROP)
FORGE_EXTERN_BF16(FORGE_ADAGRAD)
FORGE_EXTERN_BF16(FORGE_NADAM)
FORGE_EXTERN_BF16(FORGE_RADAM)
#define FORGE_EXTERN_F8_ALL(FB)             \
  FORGE_EXTERN_F8(FORGE_ADAMW, FB)          \
  FORGE_EXTERN_F8(FORGE_SGD, FB)            \
  FORGE_EXTERN_F8(FORGE_SGD_MOMENTUM, FB)   \
  FORGE_EXTERN_F8(FORGE_LION, FB)           \
  FORGE_EXTERN_F8(FORGE_RMSPROP, FB)        \
  FORGE_EXTERN_F8(FORGE_ADAGRAD, FB)        \
  FORGE_EXTERN_F8(FORGE_NADAM, FB)          \
  FORGE_EXTERN_F8(FORGE_RADAM, FB)          \
  extern template hipError_t wgrad_store_f8<FB>(const GArgs&, hipStream_t);
FORGE_EXTERN_F8_ALL(0)
FORGE_EXTERN_F8_ALL(1)

hipError_t launch_wgrad_fused_bf16(int state_fmt, int opt, int sr, const void* X, const void* dY, const GemmDims& d,
                                   const OptArgs& a, hipStream_t st) {
  GArgs g{X, dY, d.ldx, d.lddy,
          d.in, d.out, d.T, nullptr, 0, extent(d.T, d.in, d.ldx, 2), extent(d.T, d.out, d.lddy, 2), 0};
  switch (opt) {
    case FORGE_ADAMW: return wgrad_fused_bf16_opt<FORGE_ADAMW>(state_fmt, sr, g, a, st);
    case FORGE_SGD: return wgrad_fused_bf16_opt<FORGE_SGD>(state_fmt, sr, g, a, st);
    case FORGE_SGD_MOMENTUM: return wgrad_fused_bf16_opt<FORGE_SGD_MOMENTUM>(state_fmt, sr, g, a, st);
    case FORGE_LION: return wgrad_fused_bf16_opt<FORGE_LION>(state_fmt, sr, g, a, st);
    case FORGE_RMSPROP: return wgrad_fused_bf16_opt<FORGE_RMSPROP>(state_fmt, sr, g, a, st);
    case FORGE_ADAGRAD: return wgrad_fused_bf16_opt<FORGE_ADAGRAD>(state_fmt, sr, g, a, st);
    case FORGE_NADAM: return wgrad_fused_bf16_opt<FORGE_NADAM>(state_fmt, sr, g, a, st);
    case FORGE_RADAM: return wgrad_fused_bf16_opt<FORGE_RADAM>(state_fmt, sr, g, a, st);
    default: return hipErrorInvalidValue;
  }
}

// The member table of a grouped launch (eb: bytes per operand element) and the launch's
// common arguments: the A operand and the sizes the members share; B and N come from each
// member.
static GroupArgs group_args(const GroupLayer* layers, int n, const GemmDims& d, int eb) {
  GroupArgs gr{};
  gr.count = n;
  for (int j = 0; j < n; ++j) {
    const OptArgs& a = layers[j].a;
    GroupMember& M = gr.mb[j];
    M.B = layers[j].dY;
    M.b_scale = layers[j].dy_scale;
    M.ldb = layers[j].lddy;
    M.b_bytes = extent(d.T, a.out, layers[j].lddy, eb);
    M.N = a.out;
    M.W = a.W;
    M.m = a.m;
    M.v = a.v;
    M.m_scale = a.m_scale;
    M.v_scale = a.v_scale;
    M.ldw = a.ldw;
    M.ldm = a.ldm;
    M.ldv = a.ldv;
    M.rng_base = a.rng_base;
  }
  return gr;
}

hipError_t launch_wgrad_fused_bf16_group(int state_fmt, int opt, int sr, const void* X, const GemmDims& d,
                                         const GroupLayer* layers, int n, hipStream_t st) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  const GroupArgs gr = group_args(layers, n, d, 2);
  GArgs g{X, layers[0].dY, d.ldx, layers[0].lddy, d.in, layers[0].a.out, d.T, nullptr, 0,
          extent(d.T, d.in, d.ldx, 2), gr.mb[0].b_bytes, 0};
  const OptArgs& a = layers[0].a;
  switch (opt) {
    case FORGE_ADAMW: return wgrad_fused_bf16_group_opt<FORGE_ADAMW>(state_fmt, sr, g, a, gr, st);
    case FORGE_SGD: return wgrad_fused_bf16_group_opt<FORGE_SGD>(state_fmt, sr, g, a, gr, st);
    case FORGE_SGD_MOMENTUM: return wgrad_fused_bf16_group_opt<FORGE_SGD_MOMENTUM>(state_fmt, sr, g, a, gr, st);
    case FORGE_LION: return wgrad_fused_bf16_group_opt<FORGE_LION>(state_fmt, sr, g, a, gr, st);
    case FORGE_RMSPROP: return wgrad_fused_bf16_group_opt<FORGE_RMSPROP>(state_fmt, sr, g, a, gr, st);
    case FORGE_ADAGRAD: return wgrad_fused_bf16_group_opt<FORGE_ADAGRAD>(state_fmt, sr, g, a, gr, st);
    case FORGE_NADAM: return wgrad_fused_bf16_group_opt<FORGE_NADAM>(state_fmt, sr, g, a, gr, st);
    case FORGE_RADAM: return wgrad_fused_bf16_group_opt<FORGE_RADAM>(state_fmt, sr, g, a, gr, st);
    default: return hipErrorInvalidValue;
  }
}

template <int FB>
static hipError_t wgrad_fused_f8_group(int sf, int opt, int sr, const GArgs& g, const OptArgs& a, const GroupArgs& gr,
                                       hipStream_t st) {
  switch (opt) {
    case FORGE_ADAMW: return wgrad_fused_f8_group_opt<FORGE_ADAMW, FB>(sf, sr, g, a, gr, st);
    case FORGE_SGD: return wgrad_fused_f8_group_opt<FORGE_SGD, FB>(sf, sr, g, a, gr, st);
    case FORGE_SGD_MOMENTUM: return wgrad_fused_f8_group_opt<FORGE_SGD_MOMENTUM, FB>(sf, sr, g, a, gr, st);
    case FORGE_LION: return wgrad_fused_f8_group_opt<FORGE_LION, FB>(sf, sr, g, a, gr, st);
    case FORGE_RMSPROP: return wgrad_fused_f8_group_opt<FORGE_RMSPROP, FB>(sf, sr, g, a, gr, st);
    case FORGE_ADAGRAD: return wgrad_fused_f8_group_opt<FORGE_ADAGRAD, FB>(sf, sr, g, a, gr, st);
    case FORGE_NADAM: return wgrad_fused_f8_group_opt<FORGE_NADAM, FB>(sf, sr, g, a, gr, st);
    case FORGE_RADAM: return wgrad_fused_f8_group_opt<FORGE_RADAM, FB>(sf, sr, g, a, gr, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad_fused_f8_group(int dy_e5m2, int state_fmt, int opt, int sr, const void* X,
                                       const float* x_scale, const GemmDims& d, const GroupLayer* layers, int n,
                                       hipStream_t st) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  const GroupArgs gr = group_args(layers, n, d, 1);
  GArgs g{X, layers[0].dY, d.ldx, layers[0].lddy, d.in, layers[0].a.out, d.T, nullptr, 0,
          extent(d.T, d.in, d.ldx, 1), gr.mb[0].b_bytes, 0, x_scale, layers[0].dy_scale};
  const OptArgs& a = layers[0].a;
  return dy_e5m2 ? wgrad_fused_f8_group<1>(state_fmt, opt, sr, g, a, gr, st)
                 : wgrad_fused_f8_group<0>(state_fmt, opt, sr, g, a, gr, st);
}

hipError_t launch_wgrad_store_bf16(const void* X, const void* dY, const GemmDims& d, float* dW, int64_t ld_dw,
                                   hipStream_t st) {
  GArgs g{X, dY, d.ldx, d.lddy,
          d.in, d.out, d.T, dW, ld_dw, extent(d.T, d.in, d.ldx, 2), extent(d.T, d.out, d.lddy, 2), extent(d.out, d.in, ld_dw, 4)};
  OptArgs a{};
  return g_pick<WgradBig, WgradSmall, WgradSplit, WgradBand, WgradTiny>(
      g, [&](auto c, const GArgs& gc) { return g_launch<decltype(c), G_EPI_STORE, FORGE_SGD, ST_F32, false>(gc, a, st); });
}

template <int FB>
static hipError_t wgrad_fused_f8(int sf, int opt, int sr, const GArgs& g, const OptArgs& a, hipStream_t st) {
  switch (opt) {
    case FORGE_ADAMW: return wgrad_fused_f8_opt<FORGE_ADAMW, FB>(sf, sr, g, a, st);
    case FORGE_SGD: return wgrad_fused_f8_opt<FORGE_SGD, FB>(sf, sr, g, a, st);
    case FORGE_SGD_MOMENTUM: return wgrad_fused_f8_opt<FORGE_SGD_MOMENTUM, FB>(sf, sr, g, a, st);
    case FORGE_LION: return wgrad_fused_f8_opt<FORGE_LION, FB>(sf, sr, g, a, st);
    case FORGE_RMSPROP: return wgrad_fused_f8_opt<FORGE_RMSPROP, FB>(sf, sr, g, a, st);
    case FORGE_ADAGRAD: return wgrad_fused_f8_opt<FORGE_ADAGRAD, FB>(sf, sr, g, a, st);
    case FORGE_NADAM: return wgrad_fused_f8_opt<FORGE_NADAM, FB>(sf, sr, g, a, st);
    case FORGE_RADAM: return wgrad_fused_f8_opt<FORGE_RADAM, FB>(sf, sr, g, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad_fused_f8(int dy_e5m2, int state_fmt, int opt, int sr, const void* X, const float* x_scale, const void* dY,
                                 const float* dy_scale, const GemmDims& d, const OptArgs& a, hipStream_t st) {
  GArgs g{X, dY, d.ldx, d.lddy, d.in, d.out, d.T, nullptr, 0, extent(d.T, d.in, d.ldx, 1), extent(d.T, d.out, d.lddy, 1), 0,
          x_scale, dy_scale};
  return dy_e5m2 ? wgrad_fused_f8<1>(state_fmt, opt, sr, g, a, st) : wgrad_fused_f8<0>(state_fmt, opt, sr, g, a, st);
}

hipError_t launch_wgrad_store_f8(int dy_e5m2, const void* X, const float* x_scale, const void* dY,
                                 const float* dy_scale, const GemmDims& d, float* dW, int64_t ld_dw, hipStream_t st) {
  GArgs g{X, dY, d.ldx, d.lddy, d.in, d.out, d.T, dW, ld_dw, extent(d.T, d.in, d.ldx, 1), extent(d.T, d.out, d.lddy, 1),
          extent(d.out, d.in, ld_dw, 4), x_scale, dy_scale};
  return dy_e5m2 ? wgrad_store_f8<1>(g, st) : wgrad_store_f8<0>(g, st);
}

hipError_t launch_dgrad_bf16(const void* dY, int64_t lddy, const void* W, int64_t ldw, void* dX, int64_t lddx,
                             int32_t T, int32_t n_out, int32_t n_in, hipStream_t st) {
  GArgs g{W, dY, ldw, lddy,
          n_in, T, n_out, dX, lddx, extent(n_out, n_in, ldw, 2), extent(T, n_out, lddy, 2), extent(T, n_in, lddx, 2)};
  OptArgs a{};
  return g_pick<DgradBig, DgradSmall, DgradSplit, DgradBand, DgradTiny>(
      g, [&](auto c, const GArgs& gc) { return g_launch<decltype(c), G_EPI_DX, FORGE_SGD, ST_F32, false>(gc, a, st); });
}

}  // namespace forge
