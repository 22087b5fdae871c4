// float32 weight-gradient GEMM dW = dY^T X over tokens, tile by tile, with the
// fused optimizer epilogue (FORGE, §2 Method, "Core mechanism": accumulate the
// tile in FP32 registers, update it in registers, write back only W and the
// moments) or a plain float32 dW store (the two-phase baseline of §1). The
// bfloat16 path lives in forge_gemm_kernel.h; this kernel serves float32 layers.
//
// Mapping: a workgroup owns a BM x BN tile of dW^T (BM along `in`, BN along
// `out`) with WM x WN wave tiles, replicated KS times to split the token range
// inside the workgroup (partial tiles are summed through LDS, never through
// device memory). v_mfma_f32_16x16x4_f32 reads one float per lane per operand,
// so X and dY token rows are staged in LDS as they sit in memory (padded rows)
// and read directly; the accumulator layout gives each lane four consecutive
// `in` elements of one W row.
#include "forge_internal.h"

namespace forge {

// ---------------------------------------------------------------------------
// Tile geometry.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int BKG_, int WM_, int WN_, int KS_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BKG = BKG_, WM = WM_, WN = WN_, KS = KS_;
  static constexpr int NW = WM * WN * KS;
  static constexpr int NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int BK = BKG * KS;  // tokens per LDS stage
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(KS == 1 || (KS == 2 && FN % 2 == 0), "split-K of 1 or 2 wave groups");
};

// XCD-aware tile order: consecutive workgroup ids are dealt round-robin to the
// 8 XCDs, so remap them so each XCD walks a contiguous range of tiles, and walk
// that range in column groups so concurrently resident tiles share X/dY panels
// in the XCD's own L2.
__device__ __forceinline__ void tile_coords(int tiles_o, int tiles_i, int& bo, int& bi) {
  const int n = tiles_o * tiles_i;
  int w = blockIdx.x;
  int L = w;
  if ((n & 7) == 0) L = (w & 7) * (n >> 3) + (w >> 3);
  const int GROUP = 8;
  const int per_group = GROUP * tiles_i;
  const int g = L / per_group;
  const int first = g * GROUP;
  const int gs = min(tiles_o - first, GROUP);
  const int r = L - g * per_group;
  bo = first + r % gs;
  bi = r / gs;
}

// Epilogue kinds.
enum { EPI_STORE = 0, EPI_OPT = 1 };

template <class C>
struct Smem {
  static constexpr int PADF = 16;  // staging row pad (floats)
  static constexpr int STAGE_BYTES = C::BK * (C::BM + C::BN + 2 * PADF) * 4;
  static constexpr int RED_BYTES = (C::KS - 1) * C::BM * C::BN * 4;
  static constexpr int BYTES = (2 * STAGE_BYTES > RED_BYTES) ? 2 * STAGE_BYTES : RED_BYTES;
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <class C, int EPI, int OPT>
__global__ __launch_bounds__(C::NT) void wgrad_f32_kernel(const void* __restrict__ Xp, const void* __restrict__ dYp,
                                                          GemmDims d, OptArgs a, float* __restrict__ dW,
                                                          int64_t ld_dw) {
  using S = Smem<C>;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = wave / (C::WM * C::WN);  // split-K group
  const int wg = wave % (C::WM * C::WN);
  const int wm = wg % C::WM, wn = wg / C::WM;
  const int wave_m0 = wm * C::TM, wave_n0 = wn * C::TN;
  const int g16 = lane >> 4, l16 = lane & 15;

  const int tiles_o = (d.out + C::BN - 1) / C::BN;
  const int tiles_i = (d.in + C::BM - 1) / C::BM;
  int bo, bi;
  tile_coords(tiles_o, tiles_i, bo, bi);
  const int o0 = bo * C::BN, i0 = bi * C::BM;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nstages = (d.T + C::BK - 1) / C::BK;

  {
    // ---------------- fp32 mainloop ----------------
    constexpr int PADF = S::PADF;
    constexpr int LA = C::BM + PADF, LB = C::BN + PADF;
    constexpr int CA = C::BK * C::BM / 4;
    constexpr int CB = C::BK * C::BN / 4;
    constexpr int PA = (CA + C::NT - 1) / C::NT;
    constexpr int PB = (CB + C::NT - 1) / C::NT;
    const float* X = reinterpret_cast<const float*>(Xp);
    const float* dY = reinterpret_cast<const float*>(dYp);
    auto As = [&](int buf) { return reinterpret_cast<float*>(smem) + buf * (C::BK * (LA + LB)); };
    auto Bs = [&](int buf) { return As(buf) + C::BK * LA; };
    f32x4 ra[PA], rb[PB];
    auto gload = [&](int s) {
      const int t0 = s * C::BK;
#pragma unroll
      for (int j = 0; j < PA; ++j) {
        const int c = tid + j * C::NT;
        const int row = c / (C::BM / 4), col = (c % (C::BM / 4)) * 4;
        const int t = t0 + row, i = i0 + col;
        ra[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((CA % C::NT == 0 || c < CA) && t < d.T && i < d.in)
          ra[j] = *reinterpret_cast<const f32x4*>(X + (int64_t)t * d.ldx + i);
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int c = tid + j * C::NT;
        const int row = c / (C::BN / 4), col = (c % (C::BN / 4)) * 4;
        const int t = t0 + row, o = o0 + col;
        rb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((CB % C::NT == 0 || c < CB) && t < d.T && o < d.out)
          rb[j] = *reinterpret_cast<const f32x4*>(dY + (int64_t)t * d.lddy + o);
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < PA; ++j) {
        const int c = tid + j * C::NT;
        if (CA % C::NT == 0 || c < CA)
          *reinterpret_cast<f32x4*>(As(buf) + (c / (C::BM / 4)) * LA + (c % (C::BM / 4)) * 4) = ra[j];
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int c = tid + j * C::NT;
        if (CB % C::NT == 0 || c < CB)
          *reinterpret_cast<f32x4*>(Bs(buf) + (c / (C::BN / 4)) * LB + (c % (C::BN / 4)) * 4) = rb[j];
      }
    };
    if (nstages > 0) {
      gload(0);
      sstore(0);
    }
    __syncthreads();
    for (int s = 0; s < nstages; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstages) gload(s + 1);
      const float* A = As(buf);
      const float* B = Bs(buf);
#pragma unroll
      for (int kk = 0; kk < C::BKG / 4; ++kk) {
        const int k = kg * C::BKG + kk * 4 + g16;
        float af[C::FM], bfr[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) af[fm] = A[k * LA + wave_m0 + 16 * fm + l16];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) bfr[fn] = B[k * LB + wave_n0 + 16 * fn + l16];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
      if (s + 1 < nstages) sstore(buf ^ 1);
      __syncthreads();
    }

  }

  // ---------------- in-workgroup split-K reduction through LDS ----------------
  // Group kg owns output column blocks fn in [kg*FN/KS, (kg+1)*FN/KS); it hands
  // the other blocks to their owner through LDS and adds the ones it receives.
  constexpr int FNO = C::FN / C::KS;
  const int fn_begin = kg * FNO;
  if constexpr (C::KS == 2) {
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    // region of group kg: [wg][fm][fn % FNO][lane]
    const int other = kg ^ 1;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if (fn / FNO == other)
          red[(((kg * (C::WM * C::WN) + wg) * C::FM + fm) * FNO + (fn % FNO)) * 64 + lane] = acc[fm][fn];
      }
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if (fn / FNO == kg)
          acc[fm][fn] += red[(((other * (C::WM * C::WN) + wg) * C::FM + fm) * FNO + (fn % FNO)) * 64 + lane];
      }
  }

  // ---------------- epilogue ----------------
  const int o_base = o0 + wave_n0 + l16;
  const int i_base = i0 + wave_m0 + 4 * g16;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if (fn / FNO != kg) continue;
      const int o = o_base + 16 * fn;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int i = i_base + 16 * fm;
        if (o < d.out && i < d.in) *reinterpret_cast<f32x4*>(dW + (int64_t)o * ld_dw + i) = acc[fm][fn];
      }
    }
  } else {
    constexpr int SL = opt_slots(OPT);
    constexpr bool HAS_M = SL & 1, HAS_V = SL & 2;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if (fn / FNO != kg) continue;
      const int o = o_base + 16 * fn;
      const bool ov = o < d.out;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int i = i_base + 16 * fm;
        if (!(ov && i < d.in)) continue;
        float w[4], m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
        load_w4<false>(a, o, i, w);
        if constexpr (HAS_M) load_f4(a.m, a.ldm, o, i, m);
        if constexpr (HAS_V) load_f4(a.v, a.ldv, o, i, v);
        const float g[4] = {acc[fm][fn].x, acc[fm][fn].y, acc[fm][fn].z, acc[fm][fn].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) opt_apply<OPT>(g[j], w[j], m[j], v[j], a.s);
        store_w4<false, false>(a, o, i, w, nullptr);
        if constexpr (HAS_M) store_f4(a.m, a.ldm, o, i, m);
        if constexpr (HAS_V) store_f4(a.v, a.ldv, o, i, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers (float32; bfloat16 goes to forge_gemm.hip and forge_gemm_kernel.h).
// ---------------------------------------------------------------------------
using CfgF32 = TileCfg<64, 64, 16, 2, 2, 2>;  // 8 waves: 2x2 wave tiles of 32x32, 2-way token split

template <int EPI, int OPT>
static hipError_t launch_f32(const void* X, const void* dY, const GemmDims& d, const OptArgs& a, float* dW,
                             int64_t ld_dw, hipStream_t stream) {
  using C = CfgF32;
  const int tiles = ((d.out + C::BN - 1) / C::BN) * ((d.in + C::BM - 1) / C::BM);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((wgrad_f32_kernel<C, EPI, OPT>), dim3(tiles), dim3(C::NT), 0, stream, X, dY, d, a, dW, ld_dw);
  return hipGetLastError();
}

hipError_t launch_wgrad_fused(int io_bf16, int state_fmt, int opt, int sr, const void* X, const void* dY,
                              const GemmDims& d, const OptArgs& a, hipStream_t stream) {
  if (io_bf16) return launch_wgrad_fused_bf16(state_fmt, opt, sr, X, dY, d, a, stream);
  switch (opt) {
    case FORGE_ADAMW: return launch_f32<EPI_OPT, FORGE_ADAMW>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_SGD: return launch_f32<EPI_OPT, FORGE_SGD>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_SGD_MOMENTUM: return launch_f32<EPI_OPT, FORGE_SGD_MOMENTUM>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_LION: return launch_f32<EPI_OPT, FORGE_LION>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_RMSPROP: return launch_f32<EPI_OPT, FORGE_RMSPROP>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_ADAGRAD: return launch_f32<EPI_OPT, FORGE_ADAGRAD>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_NADAM: return launch_f32<EPI_OPT, FORGE_NADAM>(X, dY, d, a, nullptr, 0, stream);
    case FORGE_RADAM: return launch_f32<EPI_OPT, FORGE_RADAM>(X, dY, d, a, nullptr, 0, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad_store(int io_bf16, const void* X, const void* dY, const GemmDims& d, float* dW,
                              int64_t ld_dw, hipStream_t stream) {
  if (io_bf16) return launch_wgrad_store_bf16(X, dY, d, dW, ld_dw, stream);
  OptArgs a{};
  return launch_f32<EPI_STORE, FORGE_SGD>(X, dY, d, a, dW, ld_dw, stream);
}

}  // namespace forge
