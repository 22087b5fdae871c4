// float32 input gradient dX = dY W of a linear layer (FORGE explainer, §5
// limitations: the input gradient is read from the old weights, before the
// update; the bfloat16 kernel lives in forge_gemm_kernel.h), and the stand-alone
// element-wise optimizer pass of the two-phase baseline (§1).
//
// dgrad mapping: the MFMA (v_mfma_f32_16x16x4_f32) computes
// C[m = i][n = t] = sum_o W[o][i] dY[t][o], i.e. dX^T tiles, so a lane's four
// accumulator rows are four consecutive columns of one dX row. W rows and dY
// rows are staged in LDS as they sit in memory (padded rows) and read directly.
#include "forge_internal.h"

namespace forge {

// BM (in) x BN (tokens) output tile, BK (out) per stage, WM x WN waves.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
};

template <class C>
__global__ __launch_bounds__(C::NT) void dgrad_f32_kernel(const void* __restrict__ dYp, int64_t lddy,
                                                      const void* __restrict__ Wp, int64_t ldw,
                                                      void* __restrict__ dXp, int64_t lddx, int T, int n_out,
                                                      int n_in) {
  constexpr int ES = 4;                          // element size
  constexpr int VE = 16 / ES;                    // elements per 16-byte chunk
  constexpr int LA = C::BM + 16;                 // W stage row pitch (elements)
  constexpr int LB = C::BK + 4;                  // dY stage row pitch (elements), padded
  constexpr int STAGE = (C::BK * LA + C::BN * LB) * ES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int wave_m0 = wm * C::TM, wave_n0 = wn * C::TN;
  const int g16 = lane >> 4, l16 = lane & 15;

  const int tiles_i = (n_in + C::BM - 1) / C::BM;
  const int bi = blockIdx.x % tiles_i, bt = blockIdx.x / tiles_i;
  const int i0 = bi * C::BM, t0 = bt * C::BN;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int CA = C::BK * C::BM / VE;  // chunks of W per stage
  constexpr int CB = C::BN * C::BK / VE;  // chunks of dY per stage
  constexpr int PA = (CA + C::NT - 1) / C::NT, PB = (CB + C::NT - 1) / C::NT;
  u32x4 ra[PA], rb[PB];
  const char* Wb = reinterpret_cast<const char*>(Wp);
  const char* dYb = reinterpret_cast<const char*>(dYp);
  auto As = [&](int buf) { return smem + buf * STAGE; };
  auto Bs = [&](int buf) { return smem + buf * STAGE + C::BK * LA * ES; };

  auto gload = [&](int s) {
    const int k0 = s * C::BK;
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      const int c = tid + j * C::NT;
      const int row = c / (C::BM / VE), col = (c % (C::BM / VE)) * VE;
      const int o = k0 + row, i = i0 + col;
      ra[j] = u32x4{0u, 0u, 0u, 0u};
      if ((CA % C::NT == 0 || c < CA) && o < n_out && i < n_in)
        ra[j] = *reinterpret_cast<const u32x4*>(Wb + ((int64_t)o * ldw + i) * ES);
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int c = tid + j * C::NT;
      const int row = c / (C::BK / VE), col = (c % (C::BK / VE)) * VE;
      const int t = t0 + row, o = k0 + col;
      rb[j] = u32x4{0u, 0u, 0u, 0u};
      if ((CB % C::NT == 0 || c < CB) && t < T && o < n_out)
        rb[j] = *reinterpret_cast<const u32x4*>(dYb + ((int64_t)t * lddy + o) * ES);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PA; ++j) {
      const int c = tid + j * C::NT;
      if (CA % C::NT == 0 || c < CA) {
        const int row = c / (C::BM / VE), cc = c % (C::BM / VE);
        const int off = row * LA + cc * 4;
        *reinterpret_cast<u32x4*>(As(buf) + off * ES) = ra[j];
      }
    }
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int c = tid + j * C::NT;
      if (CB % C::NT == 0 || c < CB) {
        const int row = c / (C::BK / VE), cc = c % (C::BK / VE);
        *reinterpret_cast<u32x4*>(Bs(buf) + (row * LB + cc * VE) * ES) = rb[j];
      }
    }
  };

  const int nstages = (n_out + C::BK - 1) / C::BK;
  if (nstages > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  const int r4 = l16 >> 2, c4 = l16 & 3;
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) gload(s + 1);
    {
      const float* A = reinterpret_cast<const float*>(As(buf));
      const float* B = reinterpret_cast<const float*>(Bs(buf));
#pragma unroll
      for (int kk = 0; kk < C::BK / 4; ++kk) {
        const int k = kk * 4 + g16;
        float af[C::FM], bfr[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) af[fm] = A[k * LA + wave_m0 + 16 * fm + l16];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) bfr[fn] = B[(wave_n0 + 16 * fn + l16) * LB + k];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
    }
    if (s + 1 < nstages) sstore(buf ^ 1);
    __syncthreads();
  }

  // C[m = i][n = t]: lane holds dX[t][i..i+3].
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int t = t0 + wave_n0 + 16 * fn + l16;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int i = i0 + wave_m0 + 16 * fm + 4 * g16;
      if (t < T && i < n_in) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dXp) + (int64_t)t * lddx + i) = acc[fm][fn];
      }
    }
  }
}

using DCfgF32 = DCfg<64, 64, 16, 2, 2>;

hipError_t launch_dgrad(int io_bf16, const void* dY, int64_t lddy, const void* W, int64_t ldw, void* dX,
                        int64_t lddx, int32_t T, int32_t n_out, int32_t n_in, hipStream_t stream) {
  if (io_bf16) return launch_dgrad_bf16(dY, lddy, W, ldw, dX, lddx, T, n_out, n_in, stream);
  using C = DCfgF32;
  const int tiles = ((n_in + C::BM - 1) / C::BM) * ((T + C::BN - 1) / C::BN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((dgrad_f32_kernel<C>), dim3(tiles), dim3(C::NT), 0, stream, dY, lddy, W, ldw, dX, lddx, T,
                     n_out, n_in);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Element-wise optimizer pass of the unfused baseline: each thread owns four
// consecutive elements of one row; 16 consecutive threads cover one INT8 block
// of 64 (rows are multiples of 64 long in that mode).
// ---------------------------------------------------------------------------
template <bool W_BF16, int OPT, int SF, bool SR>
__global__ __launch_bounds__(256) void optimizer_kernel(const float* __restrict__ dW, int64_t ld_dw, OptArgs a) {
  constexpr bool Q8D = SF == ST_Q8D, Q8 = SF == ST_Q8 || Q8D, B16S = SF == ST_BF16;
  constexpr int SL = opt_slots(OPT);
  constexpr bool HAS_M = SL & 1, HAS_V = SL & 2;
  // dynamic-code tables staged in LDS, as in the fused epilogue
  const DynTables* dyn = &g_dyn;
  if constexpr (Q8D) {
    __shared__ DynTables dyn_lds;
    float* dst = reinterpret_cast<float*>(&dyn_lds);
    const float* src = reinterpret_cast<const float*>(&g_dyn);
    for (int j = threadIdx.x; j < (int)(sizeof(DynTables) / 4); j += 256) dst[j] = src[j];
    __syncthreads();
    dyn = &dyn_lds;
  }
  const int64_t vec_per_row = a.in >> 2;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.out * vec_per_row;
  const bool valid = gid < total;
  const int o = valid ? (int)(gid / vec_per_row) : 0;
  const int i = valid ? (int)(gid % vec_per_row) * 4 : 0;
  float w[4] = {0.f, 0.f, 0.f, 0.f}, m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f}, g[4];
  uint64_t zz[4] = {0ull, 0ull, 0ull, 0ull};  // random words of the four elements (W, m, v fields)
  if (valid) {
    load_f4(dW, ld_dw, o, i, g);
    load_w4<W_BF16>(a, o, i, w);
    if constexpr (Q8D) {
      const int64_t si = (int64_t)o * (a.in >> 6) + (i >> 6);
      if constexpr (HAS_M) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.m) + (int64_t)o * a.ldm + i);
        const float sc = a.m_scale[si];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = dyn_decode_s((q >> (8 * j)) & 0xFFu, dyn->vs) * sc;
      }
      if constexpr (HAS_V) {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.v) + (int64_t)o * a.ldv + i);
        const float sc = a.v_scale[si];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = dyn->vu[(q >> (8 * j)) & 0xFFu] * sc;
      }
    } else if constexpr (Q8) {
      if constexpr (HAS_M) dequant_m4(a, o, i, m);
      if constexpr (HAS_V) dequant_v4(a, o, i, v);
    } else if constexpr (B16S) {
      if constexpr (HAS_M) bf16x4_to_f32(*reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.m) + (int64_t)o * a.ldm + i), m);
      if constexpr (HAS_V) bf16x4_to_f32(*reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.v) + (int64_t)o * a.ldv + i), v);
    } else {
      if constexpr (HAS_M) load_f4(a.m, a.ldm, o, i, m);
      if constexpr (HAS_V) load_f4(a.v, a.ldv, o, i, v);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) opt_apply<OPT>(g[j], w[j], m[j], v[j], a.s);
    rand64x4<SR>(a.rng_base, (uint32_t)o * (uint32_t)a.in + (uint32_t)i, zz);
    store_w4<W_BF16, SR>(a, o, i, w, zz);
  }
  if constexpr (Q8) {
    // linear codes: absmax of m and sqrt(v); dynamic codes: of m and v
    float r[4], mmax = 0.f, vmax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = Q8D ? v[j] : sqrtf(v[j]);
      mmax = fmaxf(mmax, fabsf(m[j]));
      vmax = fmaxf(vmax, r[j]);
    }
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) {
      mmax = fmaxf(mmax, __shfl_xor(mmax, sh));
      vmax = fmaxf(vmax, __shfl_xor(vmax, sh));
    }
    const float sm = Q8D ? mmax : mmax * (1.f / 127.f), sv = Q8D ? vmax : vmax * (1.f / 255.f);
    const float im = block_inv(mmax, Q8D ? 1.f : 127.f), iv = block_inv(vmax, Q8D ? 1.f : 255.f);
    if (valid) {
      if constexpr (HAS_M)
        *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(a.m) + (int64_t)o * a.ldm + i) =
            Q8D ? quant_dyn_m4(m, im, dyn->ms) : quant_m4(m, im);
      if constexpr (HAS_V)
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.v) + (int64_t)o * a.ldv + i) =
            Q8D ? quant_dyn_v4(r, iv, dyn->mu) : quant_v4(r, iv);
      if ((i & 63) == 0) {
        const int64_t si = (int64_t)o * (a.in >> 6) + (i >> 6);
        if constexpr (HAS_M) a.m_scale[si] = sm;
        if constexpr (HAS_V) a.v_scale[si] = sv;
      }
    }
  } else if constexpr (B16S) {
    if (valid) {
      if constexpr (HAS_M)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.m) + (int64_t)o * a.ldm + i) =
            pack_bf16x4<SR>(m, zz, RF_M);
      if constexpr (HAS_V)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.v) + (int64_t)o * a.ldv + i) =
            pack_bf16x4<SR>(v, zz, RF_V);
    }
  } else {
    if (valid) {
      if constexpr (HAS_M) store_f4(a.m, a.ldm, o, i, m);
      if constexpr (HAS_V) store_f4(a.v, a.ldv, o, i, v);
    }
  }
}

template <int OPT, int SF>
static void launch_opt_sf(int sr, dim3 grid, const float* dW, int64_t ld_dw, const OptArgs& a, hipStream_t st) {
  if (sr) hipLaunchKernelGGL((optimizer_kernel<true, OPT, SF, true>), grid, dim3(256), 0, st, dW, ld_dw, a);
  else hipLaunchKernelGGL((optimizer_kernel<true, OPT, SF, false>), grid, dim3(256), 0, st, dW, ld_dw, a);
}

template <int OPT>
static hipError_t launch_opt_t(int w_bf16, int sf, int sr, const float* dW, int64_t ld_dw, const OptArgs& a,
                               hipStream_t st) {
  const int64_t total = (int64_t)a.out * (a.in >> 2);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (!w_bf16)
    hipLaunchKernelGGL((optimizer_kernel<false, OPT, ST_F32, false>), grid, dim3(256), 0, st, dW, ld_dw, a);
  else if (sf == ST_Q8)
    launch_opt_sf<OPT, ST_Q8>(sr, grid, dW, ld_dw, a, st);
  else if (sf == ST_Q8D)
    launch_opt_sf<OPT, ST_Q8D>(sr, grid, dW, ld_dw, a, st);
  else if (sf == ST_BF16)
    launch_opt_sf<OPT, ST_BF16>(sr, grid, dW, ld_dw, a, st);
  else
    launch_opt_sf<OPT, ST_F32>(sr, grid, dW, ld_dw, a, st);
  return hipGetLastError();
}

hipError_t launch_optimizer(int w_bf16, int state_fmt, int opt, int sr, const float* dW, int64_t ld_dw,
                            const OptArgs& a, hipStream_t stream) {
  switch (opt) {
    case FORGE_ADAMW: return launch_opt_t<FORGE_ADAMW>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_SGD: return launch_opt_t<FORGE_SGD>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_SGD_MOMENTUM: return launch_opt_t<FORGE_SGD_MOMENTUM>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_LION: return launch_opt_t<FORGE_LION>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_RMSPROP: return launch_opt_t<FORGE_RMSPROP>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_ADAGRAD: return launch_opt_t<FORGE_ADAGRAD>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_NADAM: return launch_opt_t<FORGE_NADAM>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    case FORGE_RADAM: return launch_opt_t<FORGE_RADAM>(w_bf16, state_fmt, sr, dW, ld_dw, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace forge
