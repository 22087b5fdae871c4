// bfloat16 GEMM core of the library on gfx950, with three epilogues:
//   * fused weight-gradient + optimizer step (FORGE, §2 Method, "Core mechanism":
//     each weight tile is accumulated over all tokens in FP32 accumulators, the
//     optimizer update runs on those registers, only W and the moments are
//     written back; the gradient tile never reaches device memory),
//   * float32 dW store (the two-phase baseline of §1),
//   * input gradient dX = dY W in bfloat16 (§5: computed from the old W).
//
// Mapping. C[m][n] = sum_k A[m][k] B[k][n] with
//   wgrad: m = in (i), n = out (o), k = tokens; A[i][t] = X[t][i], B[t][o] = dY[t][o]
//   dgrad: m = in (i), n = tokens (t), k = out;  A[i][o] = W[o][i], B[o][t] = dY[t][o]
// so each lane's accumulator rows are consecutive `in` elements of one W (or dX)
// row: the epilogue moves W/m/v/dX as 8- and 16-byte vectors.
// A is always stored with k as the slow index (rows of X or W), B either the same
// way (wgrad: rows of dY) or with k fast (dgrad: rows of dY). Rows are staged in
// LDS as they sit in memory and turned K-major for the matrix cores by the LDS
// transpose read ds_read_b64_tr_b16; k-fast B rows are read with 16-byte LDS reads.
// Matrix instruction: v_mfma_f32_32x32x16_bf16 (the 16x16x32 form issues at half
// the rate on this part). Each workgroup has WM x WN waves; a wave owns a
// (BM/WM) x (BN/WN) block of C. Operand stages of BK tokens are prefetched
// two stages ahead into registers and double-buffered in LDS. Tiles are walked by
// a persistent grid in an XCD-aware order so the workgroups that run at the same
// time on one XCD share the X/dY panels in that XCD's L2.
#include <type_traits>

#include "forge_internal.h"

namespace forge {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>), always unrolled,
// so small per-lane arrays indexed by it stay in registers.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

enum { G_EPI_STORE = 0, G_EPI_OPT = 1, G_EPI_DX = 2 };

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool B_TR_, int OCC_>
struct GCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int OCC = OCC_;  // waves per SIMD
  static constexpr bool B_TR = B_TR_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int KSTEPS = BK / 16;
  // LDS stage rows. Rows read with the transpose read are padded by 64 bytes so the
  // four rows one read touches fall into four different bank windows; k-fast B rows
  // are padded by 16 bytes for the 16-byte reads.
  static constexpr int LDA = BM + 32;
  static constexpr int LDB = B_TR ? BN + 32 : BK + 8;
  static constexpr int A_ELEMS = BK * LDA;
  static constexpr int B_ELEMS = B_TR ? BK * LDB : BN * LDB;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  // LDS: a ring of three operand stages, reused after the mainloop for one TN-row
  // chunk of the finished tile as float rows of BM + 4.
  static constexpr int NSTAGE = 3;
  static constexpr int EPI_ELEMS = TN * (BM + 4) * 2;
  static constexpr int SMEM_ELEMS = NSTAGE * STAGE_ELEMS > EPI_ELEMS ? NSTAGE * STAGE_ELEMS : EPI_ELEMS;
  static constexpr int A_CPR = BM / 8;                     // 16-byte chunks per A row
  static constexpr int B_CPR = B_TR ? BN / 8 : BK / 8;     // chunks per B row
  static constexpr int CA = BK * A_CPR;
  static constexpr int CB = B_TR ? BK * B_CPR : BN * B_CPR;
  static constexpr int PA = CA / NT, PB = CB / NT;         // chunks per thread per stage
  static_assert(CA % NT == 0 && CB % NT == 0, "stage must split evenly over threads");
  static_assert(NT % A_CPR == 0 && NT % B_CPR == 0, "a thread's chunks share a column");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "tile shape");
};

struct GArgs {
  const uint16_t* A;  // wgrad: X; dgrad: W
  const uint16_t* B;  // dY
  int64_t lda, ldb;
  int32_t M, N, K;
  void* out;          // dW (float) or dX (bf16)
  int64_t ldo;
  uint32_t a_bytes, b_bytes, out_bytes;  // extents addressed through buffer resources
};

// A byte offset that no buffer resource here covers: loads through it return 0,
// stores through it are dropped.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x4 lds_tr(const uint16_t* p) {
  typedef __bf16 v4bf_t __attribute__((__vector_size__(8)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  auto lp = (__attribute__((address_space(3))) v4bf_t*)(const_cast<uint16_t*>(p));
#pragma clang diagnostic pop
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// Persistent tile order: tile ids a workgroup takes are blockIdx.x + r*gridDim.x.
// Workgroups are dealt to the 8 XCDs round-robin, so within a full round the ids of
// one XCD are made contiguous, and contiguous ids walk GROUP tile-rows at a time.
__device__ __forceinline__ void g_tile(int tile, int ntm, int ntn, int& tm, int& tn) {
  const int G = gridDim.x;
  const int ntiles = ntm * ntn;
  int L = tile;
  const int round0 = (tile / G) * G;
  if ((G & 7) == 0 && round0 + G <= ntiles) {
    const int w = tile - round0;
    L = round0 + (w & 7) * (G >> 3) + (w >> 3);
  }
  constexpr int GROUP = 4;
  const int per = GROUP * ntn;
  const int g = L / per;
  const int first = g * GROUP;
  const int gs = min(ntm - first, GROUP);
  const int r = L - g * per;
  tm = first + r % gs;
  tn = r / gs;
}

// Epilogue memory access through buffer resources (32-bit offsets; an out-of-range
// offset turns loads into zeros and drops stores).
struct EpiRes {
  __amdgpu_buffer_rsrc_t W, m, v, ms, vs;
};

template <int OPT, bool Q8>
__device__ __forceinline__ EpiRes epi_res(const OptArgs& a) {
  EpiRes r;
  const uint32_t n = (uint32_t)a.out;
  r.W = make_rsrc(a.W, n * (uint32_t)a.ldw * 2u);
  constexpr int SL = opt_slots(OPT);
  const uint32_t es = Q8 ? 1u : 4u;
  r.m = make_rsrc((SL & 1) ? a.m : a.W, (SL & 1) ? n * (uint32_t)a.ldm * es : 0u);
  r.v = make_rsrc((SL & 2) ? a.v : a.W, (SL & 2) ? n * (uint32_t)a.ldv * es : 0u);
  const uint32_t sb = Q8 ? n * (uint32_t)(a.in >> 6) * 4u : 0u;
  r.ms = make_rsrc(((SL & 1) && Q8) ? (const void*)a.m_scale : a.W, ((SL & 1) && Q8) ? sb : 0u);
  r.vs = make_rsrc(((SL & 2) && Q8) ? (const void*)a.v_scale : a.W, ((SL & 2) && Q8) ? sb : 0u);
  return r;
}

template <class C, int EPI, int OPT, bool Q8, bool SR>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void gemm_kernel(GArgs g, OptArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::SMEM_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int wave_m0 = wm * C::TM, wave_n0 = wn * C::TN;
  const int l32 = lane & 31, hi = lane >> 5;
  const int r4 = (lane & 15) >> 2, c4 = lane & 3, half = (lane >> 4) & 1;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B, g.b_bytes);

  const int ntm = (g.M + C::BM - 1) / C::BM, ntn = (g.N + C::BN - 1) / C::BN;
  const int ntiles = ntm * ntn;
  const int nst = (g.K + C::BK - 1) / C::BK;

  // This thread's staging chunks: chunk j of a stage is tid + j*NT, i.e. the same
  // column and rows spaced NT / chunks-per-row apart.
  const int a_row0 = tid / C::A_CPR, a_col = (tid % C::A_CPR) * 8;
  const int b_row0 = tid / C::B_CPR, b_col = (tid % C::B_CPR) * 8;
  constexpr int A_RSTEP = C::NT / C::A_CPR, B_RSTEP = C::NT / C::B_CPR;
  // LDS element offsets of the staging chunks and of this lane's fragment reads
  const int a_st = a_row0 * C::LDA + a_col;
  const int b_st = C::A_ELEMS + b_row0 * C::LDB + b_col;
  const int a_fr = (8 * hi + r4) * C::LDA + wave_m0 + 16 * half + 4 * c4;
  const int b_fr = C::B_TR ? C::A_ELEMS + (8 * hi + r4) * C::LDB + wave_n0 + 16 * half + 4 * c4
                           : C::A_ELEMS + (wave_n0 + l32) * C::LDB + 8 * hi;

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tm, tn;
    g_tile(tile, ntm, ntn, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[fm][fn][e] = 0.f;

    // Byte offsets of this thread's chunks in stage 0 (kOOB where the column is out
    // of range); stage s adds s * BK rows (A, B_TR) or s * BK columns (!B_TR).
    const bool a_cok = m0 + a_col < g.M;
    const uint32_t a_off0 = a_cok ? (uint32_t)((a_row0 * g.lda + m0 + a_col) * 2) : kOOB;
    const uint32_t a_rowb = (uint32_t)(A_RSTEP * g.lda * 2), a_stageb = (uint32_t)(C::BK * g.lda * 2);
    uint32_t b_off0, b_rowb, b_stageb;
    if constexpr (C::B_TR) {
      b_off0 = (n0 + b_col < g.N) ? (uint32_t)((b_row0 * g.ldb + n0 + b_col) * 2) : kOOB;
      b_rowb = (uint32_t)(B_RSTEP * g.ldb * 2);
      b_stageb = (uint32_t)(C::BK * g.ldb * 2);
    } else {
      b_off0 = (uint32_t)(((int64_t)(n0 + b_row0) * g.ldb + b_col) * 2);
      b_rowb = (uint32_t)(B_RSTEP * g.ldb * 2);
      b_stageb = (uint32_t)(C::BK * 2);
    }

    // ---- staging: global -> registers -> LDS ----
    auto gload = [&](int s, u32x4 (&ra)[C::PA], u32x4 (&rb)[C::PB]) {
      const int k0 = s * C::BK;
#pragma unroll
      for (int j = 0; j < C::PA; ++j) {
        const bool ok = a_cok && (k0 + a_row0 + j * A_RSTEP < g.K);
        const uint32_t off = ok ? a_off0 + (uint32_t)s * a_stageb + (uint32_t)j * a_rowb : kOOB;
        ra[j] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < C::PB; ++j) {
        bool ok;
        if constexpr (C::B_TR)
          ok = (b_off0 != kOOB) && (k0 + b_row0 + j * B_RSTEP < g.K);
        else
          ok = (n0 + b_row0 + j * B_RSTEP < g.N) && (k0 + b_col < g.K);
        const uint32_t off = ok ? b_off0 + (uint32_t)s * b_stageb + (uint32_t)j * b_rowb : kOOB;
        rb[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
      }
    };
    auto sstore = [&](int buf, const u32x4 (&ra)[C::PA], const u32x4 (&rb)[C::PB]) {
      uint16_t* S = smem + buf * C::STAGE_ELEMS;
#pragma unroll
      for (int j = 0; j < C::PA; ++j) *reinterpret_cast<u32x4*>(S + a_st + j * A_RSTEP * C::LDA) = ra[j];
#pragma unroll
      for (int j = 0; j < C::PB; ++j) *reinterpret_cast<u32x4*>(S + b_st + j * B_RSTEP * C::LDB) = rb[j];
    };
    // Operand fragments of one 16-deep k-step.
    struct Frag {
      bf16x8 a[C::FM], b[C::FN];
    };
    auto load_frag = [&](Frag& F, int buf, int kk) {
      const uint16_t* S = smem + buf * C::STAGE_ELEMS;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const uint16_t* p = S + a_fr + kk * 16 * C::LDA + 32 * fm;
        bf16x4 x0 = lds_tr(p), x1 = lds_tr(p + 4 * C::LDA);
        F.a[fm] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if constexpr (C::B_TR) {
          const uint16_t* p = S + b_fr + kk * 16 * C::LDB + 32 * fn;
          bf16x4 y0 = lds_tr(p), y1 = lds_tr(p + 4 * C::LDB);
          F.b[fn] = __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          F.b[fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(S + b_fr + 32 * fn * C::LDB + kk * 16));
        }
      }
    };
    auto mma = [&](const Frag& F) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[fm], F.b[fn], acc[fm][fn], 0, 0, 0);
    };

    // ---- mainloop ----
    // LDS ring of three stages and two register staging sets: while stage s is
    // multiplied, stage s+1 is already in LDS, stage s+2 moves from registers to
    // LDS, and stage s+4 is being fetched. Fragments of the next k-step (the next
    // stage's first one at the end of a stage) are read while the current k-step's
    // MFMAs run, so the matrix pipe keeps working across the stage barrier.
    static_assert(C::KSTEPS % 2 == 0, "fragment double-buffering pairs k-steps");
    {
      u32x4 ra0[C::PA], rb0[C::PB], ra1[C::PA], rb1[C::PB];
      Frag F0, F1;
      gload(0, ra0, rb0);
      gload(1, ra1, rb1);
      __syncthreads();  // the previous tile's epilogue is done with LDS
      sstore(0, ra0, rb0);
      gload(2, ra0, rb0);
      sstore(1, ra1, rb1);
      gload(3, ra1, rb1);
      __syncthreads();
      load_frag(F0, 0, 0);
      // Stage st of the ring: R = st % 6 fixes every LDS buffer index at compile time.
      auto stage = [&](auto R_c, int st, u32x4 (&ra)[C::PA], u32x4 (&rb)[C::PB]) {
        constexpr int R = decltype(R_c)::value;
        constexpr int cur = R % 3, nxt = (R + 1) % 3, fill = (R + 2) % 3;
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; kk += 2) {
          load_frag(F1, cur, kk + 1);
          mma(F0);
          if (kk == 0) {
            sstore(fill, ra, rb);     // stage st+2
            gload(st + 4, ra, rb);
          }
          if (kk + 2 < C::KSTEPS) load_frag(F0, cur, kk + 2);
          else load_frag(F0, nxt, 0);  // first k-step of stage st+1
          mma(F1);
        }
        __syncthreads();
      };
      // stages past the last one read zeros; the count is rounded up to a multiple of 6
      const int nst6 = ((nst + 5) / 6) * 6;
      for (int st = 0; st < nst6; st += 6) {
        stage(std::integral_constant<int, 0>{}, st + 0, ra0, rb0);
        stage(std::integral_constant<int, 1>{}, st + 1, ra1, rb1);
        stage(std::integral_constant<int, 2>{}, st + 2, ra0, rb0);
        stage(std::integral_constant<int, 3>{}, st + 3, ra1, rb1);
        stage(std::integral_constant<int, 4>{}, st + 4, ra0, rb0);
        stage(std::integral_constant<int, 5>{}, st + 5, ra1, rb1);
      }
    }

    // ---- epilogue ----
    // The finished tile is handed through LDS one wave-column (TN rows of n) at a
    // time: the waves that own those rows write their accumulators (lane holds
    // C[m = 8q + 4*hi + j][n = l32] of each 32x32 block) as float rows, then every
    // thread takes 4 consecutive m of a row, so each wave reads and writes whole
    // contiguous row segments of W / m / v / dW / dX.
    float* E = reinterpret_cast<float*>(smem);
    constexpr int LDE = C::BM + 4;
    constexpr int VPR = C::BM / 4;                   // 4-element vectors per row
    constexpr int NV = C::TN * VPR / C::NT;          // vectors per thread per chunk
    static_assert((C::TN * VPR) % C::NT == 0, "chunk must split evenly over threads");
    static_assert(VPR % 16 == 0, "an INT8 block of 64 must be 16 adjacent lanes");
    __syncthreads();  // every wave is done reading the operand stages
#pragma unroll 1
    for (int c = 0; c < C::WN; ++c) {
      if (wn == c) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<f32x4*>(E + (32 * fn + l32) * LDE + wave_m0 + 32 * fm + 8 * q + 4 * hi) =
                  f32x4{acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
      }
      __syncthreads();
      const int nrow0 = n0 + c * C::TN;
      if constexpr (EPI == G_EPI_STORE || EPI == G_EPI_DX) {
        const __amdgpu_buffer_rsrc_t rO = make_rsrc(g.out, g.out_bytes);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int vi = tid + k * C::NT, row = vi / VPR, col = (vi % VPR) * 4;
          const int n = nrow0 + row, m = m0 + col;
          const f32x4 x = *reinterpret_cast<const f32x4*>(E + row * LDE + col);
          const bool ok = n < g.N && m < g.M;
          if constexpr (EPI == G_EPI_STORE) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rO,
                                                   ok ? (uint32_t)((n * g.ldo + m) * 4) : kOOB, 0, 0);
          } else {
            const u32x2 r{rne_bf16_bits(x.x) | (rne_bf16_bits(x.y) << 16), rne_bf16_bits(x.z) | (rne_bf16_bits(x.w) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(r, rO, ok ? (uint32_t)((n * g.ldo + m) * 2) : kOOB, 0, 0);
          }
        }
      } else {
        constexpr int SL = opt_slots(OPT);
        constexpr bool HAS_M = SL & 1, HAS_V = SL & 2;
        const EpiRes R = epi_res<OPT, Q8>(a);
        // loads of KB vectors are issued before any of them is consumed; KB bounds the
        // registers a batch holds next to the accumulators still to be written out
        constexpr int KB_MAX = C::OCC >= 2 ? 2 : (Q8 ? 4 : 8);
        constexpr int KB = NV > KB_MAX ? KB_MAX : NV;
#pragma unroll
        for (int kb = 0; kb < NV; kb += KB) {
        uint32_t ow[KB], om[KB], ov_[KB], osc[KB];
        u32x2 wb[KB];
        f32x4 mv[KB], vv[KB];
        uint32_t qm[KB], qv[KB];
        float msc[KB], vsc[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int vi = tid + (kb + k) * C::NT, row = vi / VPR, col = (vi % VPR) * 4;
          const int o = nrow0 + row, i = m0 + col;
          const bool ok = o < g.N && i < g.M;
          ow[k] = ok ? (uint32_t)(o * a.ldw + i) * 2u : kOOB;
          wb[k] = __builtin_amdgcn_raw_buffer_load_b64(R.W, ow[k], 0, 0);
          if constexpr (!Q8) {
            om[k] = ok ? (uint32_t)(o * a.ldm + i) * 4u : kOOB;
            ov_[k] = ok ? (uint32_t)(o * a.ldv + i) * 4u : kOOB;
            if constexpr (HAS_M) mv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(R.m, om[k], 0, 0));
            if constexpr (HAS_V) vv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(R.v, ov_[k], 0, 0));
          } else {
            om[k] = ok ? (uint32_t)(o * a.ldm + i) : kOOB;
            ov_[k] = ok ? (uint32_t)(o * a.ldv + i) : kOOB;
            osc[k] = ok ? (uint32_t)(o * (a.in >> 6) + (i >> 6)) * 4u : kOOB;
            if constexpr (HAS_M) {
              qm[k] = __builtin_amdgcn_raw_buffer_load_b32(R.m, om[k], 0, 0);
              msc[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.ms, osc[k], 0, 0));
            }
            if constexpr (HAS_V) {
              qv[k] = __builtin_amdgcn_raw_buffer_load_b32(R.v, ov_[k], 0, 0);
              vsc[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.vs, osc[k], 0, 0));
            }
          }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int vi = tid + (kb + k) * C::NT, row = vi / VPR, col = (vi % VPR) * 4;
          const int o = nrow0 + row, i = m0 + col;
          const f32x4 gx = *reinterpret_cast<const f32x4*>(E + row * LDE + col);
          const float gg[4] = {gx.x, gx.y, gx.z, gx.w};
          float w[4] = {bits_f32(wb[k].x << 16), bits_f32(wb[k].x & 0xFFFF0000u), bits_f32(wb[k].y << 16),
                        bits_f32(wb[k].y & 0xFFFF0000u)};
          float m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (!Q8) {
            if constexpr (HAS_M) { m[0] = mv[k].x; m[1] = mv[k].y; m[2] = mv[k].z; m[3] = mv[k].w; }
            if constexpr (HAS_V) { v[0] = vv[k].x; v[1] = vv[k].y; v[2] = vv[k].z; v[3] = vv[k].w; }
          } else {
            if constexpr (HAS_M) {
#pragma unroll
              for (int j = 0; j < 4; ++j) m[j] = (float)(int8_t)((qm[k] >> (8 * j)) & 0xFF) * msc[k];
            }
            if constexpr (HAS_V) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float r = (float)((qv[k] >> (8 * j)) & 0xFF) * vsc[k];
                v[j] = r * r;
              }
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) opt_apply<OPT>(gg[j], w[j], m[j], v[j], a.s);
          const uint32_t idx0 = (uint32_t)o * (uint32_t)a.in + (uint32_t)i;
          uint32_t bb[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bb[j] = SR ? sr_bf16_bits(w[j], rand16_from_base(a.rng_base, idx0 + j)) : rne_bf16_bits(w[j]);
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16)}, R.W, ow[k], 0, 0);
          if constexpr (!Q8) {
            if constexpr (HAS_M)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{m[0], m[1], m[2], m[3]}), R.m, om[k], 0, 0);
            if constexpr (HAS_V)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), R.v, ov_[k], 0, 0);
          } else {
            // block-64 absmax over the 16 adjacent lanes holding this row's block
            float r[4], mmax = 0.f, vmax = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              r[j] = sqrtf(v[j]);
              mmax = fmaxf(mmax, fabsf(m[j]));
              vmax = fmaxf(vmax, r[j]);
            }
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) {
              mmax = fmaxf(mmax, __shfl_xor(mmax, sh));
              vmax = fmaxf(vmax, __shfl_xor(vmax, sh));
            }
            const float sm = mmax / 127.f, sv = vmax / 255.f;
            if constexpr (HAS_M) __builtin_amdgcn_raw_buffer_store_b32(quant_m4(m, sm), R.m, om[k], 0, 0);
            if constexpr (HAS_V) __builtin_amdgcn_raw_buffer_store_b32(quant_v4(r, sv), R.v, ov_[k], 0, 0);
            if ((col & 63) == 0) {
              if constexpr (HAS_M) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sm), R.ms, osc[k], 0, 0);
              if constexpr (HAS_V) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sv), R.vs, osc[k], 0, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();  // the chunk's LDS rows are consumed before the next chunk overwrites them
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers. Large problems use 256x256 workgroup tiles (8 waves of 128x64, two
// per SIMD); problems with fewer such tiles than compute units use 128x128 tiles
// (4 waves of 64x64, two workgroups per compute unit).
// ---------------------------------------------------------------------------
// Tile configurations (BM, BN, BK, WM, WN, B_TR, OCC); FORGE_*_CFG override them
// at build time for tuning sweeps.
#ifndef FORGE_WGRAD_BIG_CFG
#define FORGE_WGRAD_BIG_CFG 256, 256, 32, 2, 4, true, 2
#endif
#ifndef FORGE_WGRAD_SMALL_CFG
#define FORGE_WGRAD_SMALL_CFG 128, 128, 32, 2, 2, true, 2
#endif
#ifndef FORGE_DGRAD_BIG_CFG
#define FORGE_DGRAD_BIG_CFG 256, 256, 32, 2, 4, false, 2
#endif
#ifndef FORGE_DGRAD_SMALL_CFG
#define FORGE_DGRAD_SMALL_CFG 128, 128, 32, 2, 2, false, 2
#endif
using WgradBig = GCfg<FORGE_WGRAD_BIG_CFG>;
using WgradSmall = GCfg<FORGE_WGRAD_SMALL_CFG>;
using DgradBig = GCfg<FORGE_DGRAD_BIG_CFG>;
using DgradSmall = GCfg<FORGE_DGRAD_SMALL_CFG>;

static int g_num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <class C, int EPI, int OPT, bool Q8, bool SR>
static hipError_t g_launch(const GArgs& g, const OptArgs& a, hipStream_t st) {
  const int ntiles = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN);
  if (ntiles == 0) return hipSuccess;
  const int resident = C::OCC * 4 / C::NW * g_num_cus();  // OCC waves on each of 4 SIMDs
  const int grid = ntiles < resident ? ntiles : resident;
  hipLaunchKernelGGL((gemm_kernel<C, EPI, OPT, Q8, SR>), dim3(grid), dim3(C::NT), 0, st, g, a);
  return hipGetLastError();
}

template <class Big>
static bool use_big(const GArgs& g) {
  const int big = ((g.M + Big::BM - 1) / Big::BM) * ((g.N + Big::BN - 1) / Big::BN);
  return big >= g_num_cus();
}

template <int OPT>
static hipError_t wgrad_opt_v2(int q8, int sr, const GArgs& g, const OptArgs& a, hipStream_t st) {
  const bool big = use_big<WgradBig>(g);
  if (q8) {
    if (sr) return big ? g_launch<WgradBig, G_EPI_OPT, OPT, true, true>(g, a, st)
                       : g_launch<WgradSmall, G_EPI_OPT, OPT, true, true>(g, a, st);
    return big ? g_launch<WgradBig, G_EPI_OPT, OPT, true, false>(g, a, st)
               : g_launch<WgradSmall, G_EPI_OPT, OPT, true, false>(g, a, st);
  }
  if (sr) return big ? g_launch<WgradBig, G_EPI_OPT, OPT, false, true>(g, a, st)
                     : g_launch<WgradSmall, G_EPI_OPT, OPT, false, true>(g, a, st);
  return big ? g_launch<WgradBig, G_EPI_OPT, OPT, false, false>(g, a, st)
             : g_launch<WgradSmall, G_EPI_OPT, OPT, false, false>(g, a, st);
}

static uint32_t extent(int64_t rows, int64_t ld, int64_t es) { return (uint32_t)(rows * ld * es); }

hipError_t launch_wgrad_fused_bf16(int state_q8, int opt, int sr, const void* X, const void* dY, const GemmDims& d,
                                   const OptArgs& a, hipStream_t st) {
  GArgs g{reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(dY), d.ldx, d.lddy,
          d.in, d.out, d.T, nullptr, 0, extent(d.T, d.ldx, 2), extent(d.T, d.lddy, 2), 0};
  switch (opt) {
    case FORGE_ADAMW: return wgrad_opt_v2<FORGE_ADAMW>(state_q8, sr, g, a, st);
    case FORGE_SGD: return wgrad_opt_v2<FORGE_SGD>(state_q8, sr, g, a, st);
    case FORGE_SGD_MOMENTUM: return wgrad_opt_v2<FORGE_SGD_MOMENTUM>(state_q8, sr, g, a, st);
    case FORGE_LION: return wgrad_opt_v2<FORGE_LION>(state_q8, sr, g, a, st);
    case FORGE_RMSPROP: return wgrad_opt_v2<FORGE_RMSPROP>(state_q8, sr, g, a, st);
    case FORGE_ADAGRAD: return wgrad_opt_v2<FORGE_ADAGRAD>(state_q8, sr, g, a, st);
    case FORGE_NADAM: return wgrad_opt_v2<FORGE_NADAM>(state_q8, sr, g, a, st);
    case FORGE_RADAM: return wgrad_opt_v2<FORGE_RADAM>(state_q8, sr, g, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad_store_bf16(const void* X, const void* dY, const GemmDims& d, float* dW, int64_t ld_dw,
                                   hipStream_t st) {
  GArgs g{reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(dY), d.ldx, d.lddy,
          d.in, d.out, d.T, dW, ld_dw, extent(d.T, d.ldx, 2), extent(d.T, d.lddy, 2), extent(d.out, ld_dw, 4)};
  OptArgs a{};
  return use_big<WgradBig>(g) ? g_launch<WgradBig, G_EPI_STORE, FORGE_SGD, false, false>(g, a, st)
                          : g_launch<WgradSmall, G_EPI_STORE, FORGE_SGD, false, false>(g, a, st);
}

hipError_t launch_dgrad_bf16(const void* dY, int64_t lddy, const void* W, int64_t ldw, void* dX, int64_t lddx,
                             int32_t T, int32_t n_out, int32_t n_in, hipStream_t st) {
  GArgs g{reinterpret_cast<const uint16_t*>(W), reinterpret_cast<const uint16_t*>(dY), ldw, lddy,
          n_in, T, n_out, dX, lddx, extent(n_out, ldw, 2), extent(T, lddy, 2), extent(T, lddx, 2)};
  OptArgs a{};
  return use_big<DgradBig>(g) ? g_launch<DgradBig, G_EPI_DX, FORGE_SGD, false, false>(g, a, st)
                           : g_launch<DgradSmall, G_EPI_DX, FORGE_SGD, false, false>(g, a, st);
}

}  // namespace forge
