// Weight-gradient GEMM dW = dY^T X over tokens, tile by tile, with either the
// fused optimizer epilogue (FORGE, §2 Method, "Core mechanism": accumulate the
// tile in FP32 registers, update it in registers, discard it, write back only
// W and the moments) or a plain float32 dW store (the two-phase baseline of §1).
//
// gfx950 mapping. A workgroup owns a BM x BN tile of dW^T (BM along `in`, BN
// along `out`); its waves form a WM x WN grid of wave tiles, replicated KS times
// for an in-workgroup split of the token range (reduced through LDS at the end,
// never through device memory). Tokens are the contraction index and are the
// slow index of both X [T, in] and dY [T, out], so both operands are staged in
// LDS exactly as they sit in memory (rows of tokens, coalesced 16-byte loads)
// and turned K-major on the way to the matrix cores by the LDS transpose read
// ds_read_b64_tr_b16. The MFMA computes C[m = i][n = o], so each lane's four
// accumulator rows are four consecutive `in` columns of one W row, which makes
// the epilogue's W/m/v accesses 8- and 16-byte vectors.
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

// XOR swizzle of 32-byte column groups within an LDS row of a bf16 stage, so the
// rows one transpose read touches (k, k+1, k+2, k+3 and k+8..k+11) fall in
// different banks.
__device__ __forceinline__ int swz(int row) { return (row & 3) | ((row >> 1) & 4); }

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  typedef __bf16 v4bf_t __attribute__((__vector_size__(8)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  auto lp = (__attribute__((address_space(3))) v4bf_t*)(const_cast<uint16_t*>(p));
#pragma clang diagnostic pop
  v4bf_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp);
  return __builtin_bit_cast(bf16x4, r);
}

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

template <class C, bool BF16>
struct Smem {
  static constexpr int PADF = 16;  // fp32 staging row pad (floats)
  static constexpr int STAGE_BYTES = BF16 ? C::BK * (C::BM + C::BN) * 2 : C::BK * (C::BM + C::BN + 2 * PADF) * 4;
  static constexpr int RED_BYTES = (C::KS - 1) * C::BM * C::BN * 4;
  static constexpr int BYTES = (2 * STAGE_BYTES > RED_BYTES) ? 2 * STAGE_BYTES : RED_BYTES;
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <class C, bool BF16, int EPI, int OPT, bool Q8, bool SR>
__global__ __launch_bounds__(C::NT) void wgrad_kernel(const void* __restrict__ Xp, const void* __restrict__ dYp,
                                                      GemmDims d, OptArgs a, float* __restrict__ dW,
                                                      int64_t ld_dw) {
  using S = Smem<C, BF16>;
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

  if constexpr (BF16) {
    // ---------------- bf16 mainloop ----------------
    constexpr int CA = C::BK * C::BM / 8;  // 16-byte chunks per stage of X
    constexpr int CB = C::BK * C::BN / 8;
    constexpr int PA = (CA + C::NT - 1) / C::NT;
    constexpr int PB = (CB + C::NT - 1) / C::NT;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(Xp);
    const uint16_t* dY = reinterpret_cast<const uint16_t*>(dYp);
    auto As = [&](int buf) { return reinterpret_cast<uint16_t*>(smem) + buf * (C::BK * (C::BM + C::BN)); };
    auto Bs = [&](int buf) { return As(buf) + C::BK * C::BM; };

    u32x4 ra[PA], rb[PB];
    auto gload = [&](int s) {
      const int t0 = s * C::BK;
#pragma unroll
      for (int j = 0; j < PA; ++j) {
        const int c = tid + j * C::NT;
        const int row = c / (C::BM / 8), col = (c % (C::BM / 8)) * 8;
        const int t = t0 + row, i = i0 + col;
        ra[j] = u32x4{0u, 0u, 0u, 0u};
        if ((CA % C::NT == 0 || c < CA) && t < d.T && i < d.in)
          ra[j] = *reinterpret_cast<const u32x4*>(X + (int64_t)t * d.ldx + i);
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int c = tid + j * C::NT;
        const int row = c / (C::BN / 8), col = (c % (C::BN / 8)) * 8;
        const int t = t0 + row, o = o0 + col;
        rb[j] = u32x4{0u, 0u, 0u, 0u};
        if ((CB % C::NT == 0 || c < CB) && t < d.T && o < d.out)
          rb[j] = *reinterpret_cast<const u32x4*>(dY + (int64_t)t * d.lddy + o);
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < PA; ++j) {
        const int c = tid + j * C::NT;
        if (CA % C::NT == 0 || c < CA) {
          const int row = c / (C::BM / 8), c8 = c % (C::BM / 8);
          const int grp = (c8 >> 1) ^ (swz(row) & (C::BM / 16 - 1));
          *reinterpret_cast<u32x4*>(As(buf) + row * C::BM + grp * 16 + (c8 & 1) * 8) = ra[j];
        }
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int c = tid + j * C::NT;
        if (CB % C::NT == 0 || c < CB) {
          const int row = c / (C::BN / 8), c8 = c % (C::BN / 8);
          const int grp = (c8 >> 1) ^ (swz(row) & (C::BN / 16 - 1));
          *reinterpret_cast<u32x4*>(Bs(buf) + row * C::BN + grp * 16 + (c8 & 1) * 8) = rb[j];
        }
      }
    };

    if (nstages > 0) {
      gload(0);
      sstore(0);
    }
    __syncthreads();
    const int r4 = l16 >> 2, c4 = l16 & 3;
    for (int s = 0; s < nstages; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstages) gload(s + 1);
      const uint16_t* A = As(buf);
      const uint16_t* B = Bs(buf);
#pragma unroll
      for (int kk = 0; kk < C::BKG / 32; ++kk) {
        const int k0 = kg * C::BKG + kk * 32 + 8 * g16 + r4;
        const int k1 = k0 + 4;
        bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          const int grp = (wave_m0 >> 4) + fm;
          bf16x4 lo = lds_read_tr(A + k0 * C::BM + ((grp ^ (swz(k0) & (C::BM / 16 - 1))) << 4) + 4 * c4);
          bf16x4 hi = lds_read_tr(A + k1 * C::BM + ((grp ^ (swz(k1) & (C::BM / 16 - 1))) << 4) + 4 * c4);
          af[fm] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int grp = (wave_n0 >> 4) + fn;
          bf16x4 lo = lds_read_tr(B + k0 * C::BN + ((grp ^ (swz(k0) & (C::BN / 16 - 1))) << 4) + 4 * c4);
          bf16x4 hi = lds_read_tr(B + k1 * C::BN + ((grp ^ (swz(k1) & (C::BN / 16 - 1))) << 4) + 4 * c4);
          bfr[fn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
      if (s + 1 < nstages) sstore(buf ^ 1);
      __syncthreads();
    }
  } else {
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
      if constexpr (!Q8) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          const int i = i_base + 16 * fm;
          if (!(ov && i < d.in)) continue;
          float w[4], m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
          load_w4<BF16>(a, o, i, w);
          if constexpr (HAS_M) load_f4(a.m, a.ldm, o, i, m);
          if constexpr (HAS_V) load_f4(a.v, a.ldv, o, i, v);
          const float g[4] = {acc[fm][fn].x, acc[fm][fn].y, acc[fm][fn].z, acc[fm][fn].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) opt_apply<OPT>(g[j], w[j], m[j], v[j], a.s);
          store_w4<BF16, SR>(a, o, i, w);
          if constexpr (HAS_M) store_f4(a.m, a.ldm, o, i, m);
          if constexpr (HAS_V) store_f4(a.v, a.ldv, o, i, v);
        }
      } else {
        // INT8 block-64 states: a wave tile is 64 wide along `in`, so the 16 values
        // of this lane and those of lanes ^16, ^32, ^48 form one block of row o.
        static_assert(C::TM == 64, "INT8 states need 64-wide wave tiles");
        float mq[C::FM][4], vq[C::FM][4];
        float mmax = 0.f, vmax = 0.f;
        const bool blk_ok = ov && (i0 + wave_m0) < d.in;
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
          const int i = i_base + 16 * fm;
          float w[4], m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
          if (blk_ok) {
            load_w4<BF16>(a, o, i, w);
            if constexpr (HAS_M) dequant_m4(a, o, i, m);
            if constexpr (HAS_V) dequant_v4(a, o, i, v);
            const float g[4] = {acc[fm][fn].x, acc[fm][fn].y, acc[fm][fn].z, acc[fm][fn].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) opt_apply<OPT>(g[j], w[j], m[j], v[j], a.s);
            store_w4<BF16, SR>(a, o, i, w);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            mq[fm][j] = m[j];
            vq[fm][j] = sqrtf(v[j]);
            mmax = fmaxf(mmax, fabsf(m[j]));
            vmax = fmaxf(vmax, vq[fm][j]);
          }
        }
        mmax = fmaxf(mmax, __shfl_xor(mmax, 16));
        mmax = fmaxf(mmax, __shfl_xor(mmax, 32));
        vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
        vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
        const float sm = mmax / 127.f, sv = vmax / 255.f;
        if (blk_ok) {
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm) {
            const int i = i_base + 16 * fm;
            if constexpr (HAS_M)
              *reinterpret_cast<uint32_t*>(reinterpret_cast<int8_t*>(a.m) + (int64_t)o * a.ldm + i) = quant_m4(mq[fm], sm);
            if constexpr (HAS_V)
              *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.v) + (int64_t)o * a.ldv + i) = quant_v4(vq[fm], sv);
          }
          if (g16 == 0) {
            const int64_t si = (int64_t)o * (a.in >> 6) + ((i0 + wave_m0) >> 6);
            if constexpr (HAS_M) a.m_scale[si] = sm;
            if constexpr (HAS_V) a.v_scale[si] = sv;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
using CfgBF16 = TileCfg<128, 128, 32, 2, 2, 2>;  // 8 waves: 2x2 wave tiles of 64x64, 2-way token split
using CfgF32 = TileCfg<64, 64, 16, 2, 2, 2>;     // 8 waves: 2x2 wave tiles of 32x32, 2-way token split

template <class C, bool BF16, int EPI, int OPT, bool Q8, bool SR>
static hipError_t launch_one(const void* X, const void* dY, const GemmDims& d, const OptArgs& a, float* dW,
                             int64_t ld_dw, hipStream_t stream) {
  const int tiles = ((d.out + C::BN - 1) / C::BN) * ((d.in + C::BM - 1) / C::BM);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((wgrad_kernel<C, BF16, EPI, OPT, Q8, SR>), dim3(tiles), dim3(C::NT), 0, stream, X, dY, d, a,
                     dW, ld_dw);
  return hipGetLastError();
}

template <int OPT>
static hipError_t launch_fused_opt(int io_bf16, int q8, int sr, const void* X, const void* dY, const GemmDims& d,
                                   const OptArgs& a, hipStream_t st) {
  if (!io_bf16) return launch_one<CfgF32, false, EPI_OPT, OPT, false, false>(X, dY, d, a, nullptr, 0, st);
  if (q8) {
    if (sr) return launch_one<CfgBF16, true, EPI_OPT, OPT, true, true>(X, dY, d, a, nullptr, 0, st);
    return launch_one<CfgBF16, true, EPI_OPT, OPT, true, false>(X, dY, d, a, nullptr, 0, st);
  }
  if (sr) return launch_one<CfgBF16, true, EPI_OPT, OPT, false, true>(X, dY, d, a, nullptr, 0, st);
  return launch_one<CfgBF16, true, EPI_OPT, OPT, false, false>(X, dY, d, a, nullptr, 0, st);
}

hipError_t launch_wgrad_fused(int io_bf16, int state_q8, int opt, int sr, const void* X, const void* dY,
                              const GemmDims& d, const OptArgs& a, hipStream_t stream) {
  switch (opt) {
    case FORGE_ADAMW: return launch_fused_opt<FORGE_ADAMW>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_SGD: return launch_fused_opt<FORGE_SGD>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_SGD_MOMENTUM: return launch_fused_opt<FORGE_SGD_MOMENTUM>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_LION: return launch_fused_opt<FORGE_LION>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_RMSPROP: return launch_fused_opt<FORGE_RMSPROP>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_ADAGRAD: return launch_fused_opt<FORGE_ADAGRAD>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_NADAM: return launch_fused_opt<FORGE_NADAM>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    case FORGE_RADAM: return launch_fused_opt<FORGE_RADAM>(io_bf16, state_q8, sr, X, dY, d, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad_store(int io_bf16, const void* X, const void* dY, const GemmDims& d, float* dW,
                              int64_t ld_dw, hipStream_t stream) {
  OptArgs a{};
  if (io_bf16) return launch_one<CfgBF16, true, EPI_STORE, FORGE_SGD, false, false>(X, dY, d, a, dW, ld_dw, stream);
  return launch_one<CfgF32, false, EPI_STORE, FORGE_SGD, false, false>(X, dY, d, a, dW, ld_dw, stream);
}

}  // namespace forge
