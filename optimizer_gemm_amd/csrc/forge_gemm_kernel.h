// Internal: the gfx950 GEMM kernel template of the library, its tile
// configurations and launch helpers. Included by the launcher sources; the
// fused-step instantiations are spread over several translation units so the
// library builds in parallel.
#pragma once
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
// way (wgrad: rows of dY) or with k fast (dgrad: rows of dY).
//
// Mainloop. Operand stages of BK tokens go from global memory straight into LDS:
// buffer loads with the LDS bit write one wave's 64 x 16 bytes to 1 KiB of
// consecutive LDS, and out-of-range offsets write zeros (ragged k needs no other
// masking). Four stages are in flight in a ring, so a stage's loads are issued three
// stages before it is multiplied. Rows are kept as they sit in memory; the matrix
// cores get them K-major through the LDS transpose read ds_read_b64_tr_b16 (k-fast B
// rows through 16-byte reads), and XOR swizzles of the 16-byte chunks keep those
// reads free of bank conflicts. Matrix instruction: v_mfma_f32_32x32x16_bf16 (the
// 16x16x32 form issues at half the rate on this part). Each workgroup has WM x WN
// waves; a wave owns a (BM/WM) x (BN/WN) block of C. The fragments of the next
// k-step are read between the MFMAs of the current one. Tiles are walked by a
// persistent grid in an XCD-aware order so the workgroups that run at the same time
// on one XCD share the X/dY panels in that XCD's L2.
#include <type_traits>

#include "forge_internal.h"

namespace forge {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// Cache policy of the optimizer epilogue's W / m / v (and block-scale) loads and
// stores: non-temporal (the nt bit of the buffer instructions), since each state
// element is read once and written once per step; the X / dY operand stages keep
// the default policy so their panels stay in L2 for the neighbouring tiles.
#ifndef FORGE_EPI_LD_CPOL
#define FORGE_EPI_LD_CPOL 2
#endif
#ifndef FORGE_EPI_ST_CPOL
#define FORGE_EPI_ST_CPOL 2
#endif


// 4-element vectors whose W / m / v loads the optimizer epilogue issues before consuming
// any of them (KB1: configurations with one wave per SIMD, none of the default ones, whose
// accumulators sit in AGPRs and leave room for a deeper batch; with half the waves of the
// others they need more loads in flight per wave), and whether the compiler may move work
// across batches
#ifndef FORGE_EPI_KB
#define FORGE_EPI_KB 2
#endif
#ifndef FORGE_EPI_KB1
#define FORGE_EPI_KB1 4
#endif
#ifndef FORGE_EPI_SCHED_BARRIER
#define FORGE_EPI_SCHED_BARRIER 1
#endif
// tiles without a k-split: each wave writes out its own accumulators (no workgroup
// barriers in the epilogue)
#ifndef FORGE_EPI_WAVE
#define FORGE_EPI_WAVE 1
#endif

// issue priority of a ping-pong wave over its compute phase
// ping-pong mainloop: read the next stage's first k-step during the compute phase
#ifndef FORGE_PP_SPLIT
#define FORGE_PP_SPLIT 1
#endif
#ifndef FORGE_PP_PRIO
#define FORGE_PP_PRIO 1
#endif

// Operand formats of the GEMM core: bfloat16, or OCP FP8 (E4M3 / E5M2 per operand).
enum { G_BF16 = 0, G_FP8 = 1 };

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool B_TR_, int OCC_, int NSTAGE_ = 4, int KS_ = 1,
          int IN_ = G_BF16, int FA_ = 0, int FB_ = 0, int PP_ = 0>
struct GCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  // PP: ping-pong mainloop. The waves form two groups with one wave of each on every
  // SIMD; while one group multiplies a stage held in its registers, the other reads
  // the next stage's fragments from LDS and issues operand loads, and a workgroup
  // barrier swaps the roles, so each SIMD's matrix pipe is fed by one group at a time.
  static constexpr bool PP = PP_ != 0;
  static constexpr int OCC = OCC_;  // waves per SIMD
  static constexpr bool B_TR = B_TR_;
  // IN = G_FP8: both operands are OCP 8-bit codes, A in format FA and B in format FB
  // (0 = E4M3, 1 = E5M2), multiplied by v_mfma_f32_32x32x64_f8f6f4 (64 tokens per
  // instruction) instead of v_mfma_f32_32x32x16_bf16 (16 tokens).
  static constexpr bool F8 = IN_ == G_FP8;
  static constexpr int FA = FA_, FB = FB_;
  static constexpr int EB = F8 ? 1 : 2;        // bytes per operand element
  static constexpr int KSTEP = F8 ? 64 : 16;   // tokens per MFMA
  static_assert(!F8 || B_TR, "FP8 operands are token-major on both sides");
  // KS > 1: in-workgroup split-K. KS groups of WM x WN waves each take their own
  // k-steps of every stage; the partial tiles are summed through LDS in the epilogue.
  static constexpr int KS = KS_;
  static constexpr int NW = WM * WN * KS, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int KSTEPS = BK / KSTEP;
  static constexpr int KPW = KSTEPS / KS;  // k-steps of a stage per wave
  // One LDS stage (bytes): A as BK rows of BM; B as BK rows of BN (B_TR) or BN rows of BK.
  static constexpr int ROWA = BM * EB, ROWB = (B_TR ? BN : BK) * EB;
  static constexpr int A_BYTES = BK * ROWA, B_BYTES = BK * BN * EB;
  // LDS: a ring of NSTAGE stages (the A parts of all stages first, then the B parts,
  // so every fragment read reaches its stage through an immediate offset below 64 KiB),
  // reused after the mainloop for one TN-row chunk of the finished tile as float rows
  // of BM + 4.
  static constexpr int NSTAGE = NSTAGE_;
  static_assert(NSTAGE >= 2, "ring");
  static constexpr int a_base(int buf) { return buf * A_BYTES; }
  static constexpr int b_base(int buf) { return NSTAGE * A_BYTES + buf * B_BYTES; }
  // (KS = 1: each wave stages 32 rows of its TM columns at a time; else one TN-row chunk)
  static constexpr int EPI_BYTES = KS == 1 ? NW * 32 * (TM + 4) * 4 : TN * (BM + 4) * 4;
  static constexpr int RING_BYTES = NSTAGE * (A_BYTES + B_BYTES);
  static constexpr int SMEM_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
  static constexpr int A_CPR = ROWA / 16, B_CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int PA = A_BYTES / 16 / NT, PB = B_BYTES / 16 / NT;  // chunks per thread per stage
  static_assert((A_BYTES / 16) % NT == 0 && (B_BYTES / 16) % NT == 0, "stage must split evenly over threads");
  static_assert(NT % A_CPR == 0 && NT % B_CPR == 0, "a thread's chunks share a column");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % KSTEP == 0 && KSTEPS % KS == 0 && KPW >= 1, "tile shape");
  static_assert(F8 || PP || KPW % 2 == 0, "bf16 stages hold an even number of k-steps per wave");
  static_assert(!PP || (KS == 1 && WM * WN == 8 && OCC == 2 && NSTAGE >= 3),
                "ping-pong: 8 waves (two per SIMD), no k-split, a ring of three or more stages");
  // Chunk swizzles (XOR of the 16-byte chunk index of a row):
  //  * rows read with the 16-bit transpose read: 4 * (row % 4), so the four rows one read
  //    touches land in four different 64-byte bank groups (16 or more chunks per row);
  //    rows of 8 chunks (128 bytes, two rows per 256-byte bank period): 4 * ((row / 2) % 2),
  //    so rows r and r + 2 of those four take the other 64-byte half of their row;
  //  * rows read with the 8-bit transpose read (8 rows x 32 bytes per half-wave): with
  //    16 or more chunks per row 2 * (row % 8), with 8 chunks 2 * ((row / 2) % 4), so the
  //    eight 32-byte pieces fall in eight different 32-byte bank groups;
  //  * k-fast bf16 B rows of 4 or 8 chunks (KW = 4 or 2 rows per 256 bytes):
  //    (row / KW) % chunks, so 16 consecutive rows cover all 16 bank groups.
  // A thread's chunks are NT / chunks-per-row rows apart, a multiple of the swizzle
  // period, so they all share one swizzled column.
  static constexpr int KW = B_TR ? 1 : 16 / B_CPR;
  static constexpr int TR_PERIOD = F8 ? 8 : 4;
  __host__ __device__ static constexpr int swz_tr(int row, int cpr) {
    return F8 ? (cpr >= 16 ? 2 * (row & 7) : 2 * ((row >> 1) & 3)) : (cpr >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1));
  }
  __host__ __device__ static constexpr int swz_b(int row) { return B_TR ? swz_tr(row, B_CPR) : (row / KW) % B_CPR; }
  static_assert(A_CPR >= 8 && (NT / A_CPR) % TR_PERIOD == 0, "A swizzle");
  static_assert(B_TR ? (B_CPR >= 8 && (NT / B_CPR) % TR_PERIOD == 0)
                     : ((B_CPR == 4 || B_CPR == 8) && (NT / B_CPR) % 16 == 0), "B swizzle");
  // transpose reads per operand fragment and the k rows one read covers
  static constexpr int RA = F8 ? 4 : 2, RSTEP = F8 ? 8 : 4;
  // the 16-bit offset field of the LDS reads
  static_assert((NSTAGE - 1) * A_BYTES + ((KPW - 1) * KSTEP + (RA - 1) * RSTEP) * ROWA < 65536, "A read offsets");
  static_assert((NSTAGE - 1) * B_BYTES +
                (B_TR ? ((KPW - 1) * KSTEP + (RA - 1) * RSTEP) * ROWB : 32 * (FN - 1) * ROWB) < 65536,
                "B read offsets");
};

struct GArgs {
  const void* A;      // wgrad: X; dgrad: W
  const void* B;      // dY
  int64_t lda, ldb;   // row pitches in elements
  int32_t M, N, K;
  void* out;          // dW (float) or dX (bf16)
  int64_t ldo;
  uint32_t a_bytes, b_bytes, out_bytes;  // extents addressed through buffer resources
  const float* a_scale;  // FP8 operands: dequantisation scale of A and of B (one float each)
  const float* b_scale;
  // Origin of this launch's tiles in C: the launch covers rows [m_off, M) and columns
  // [n_off, N); all addressing (and the weight element index of the RNG) stays absolute.
  int32_t m_off, n_off;
};

// A grouped fused step: up to kMaxGroup layers that share the A operand (X) and the
// optimizer, each with its own dY, W, moments and seed, in one launch. Member j owns the
// tile columns [tn1 of member j-1, tn1 of member j) of the launch; inside them everything
// (rows, element indices, random streams) is the member's own, as in a launch of its own.
constexpr int kMaxGroup = FORGE_MAX_GROUP;
struct GroupMember {
  const void* B;
  const float* b_scale;  // FP8 B: its dequantisation scale
  int64_t ldb;
  uint32_t b_bytes;
  int32_t N;    // the member's rows of C (its out)
  int32_t tn1;  // one past its last tile column in the launch
  void* W;
  void* m;
  void* v;
  float* m_scale;
  float* v_scale;
  int64_t ldw, ldm, ldv;
  uint64_t rng_base;
};
struct GroupArgs {
  int32_t count;  // 0: not a grouped launch
  GroupMember mb[kMaxGroup];
};

template <class C>
__host__ __device__ inline int g_ntm(const GArgs& g) { return (g.M - g.m_off + C::BM - 1) / C::BM; }
template <class C>
__host__ __device__ inline int g_ntn(const GArgs& g) { return (g.N - g.n_off + C::BN - 1) / C::BN; }

// A byte offset that no buffer resource here covers: loads through it return 0,
// stores through it are dropped.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Fragment reads, written as inline assembly with explicit lgkmcnt waits: an LDS read
// the compiler can see makes it wait for every outstanding global->LDS load first
// (vmcnt(0)), which would drain the ring at every k-step. Target builtins and LDS
// address casts stay in these __device__ helpers: in a kernel body the host pass
// rejects them and silently drops the kernel's launch stub.
template <int OFF>
__device__ __forceinline__ u32x2 ds_tr_asm(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_tr8_asm(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 ds_b128_asm(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// 32-bit LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
#pragma clang diagnostic pop
}
// 16 bytes per lane from buffer offset off into LDS at dst + 16 * lane (zeros where
// off is out of range).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t off) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
#pragma clang diagnostic pop
}
// The first or second of two objects, chosen at compile time (keeps two register sets
// as separate variables, which the compiler keeps in registers, unlike an array).
template <int I, class T>
__device__ __forceinline__ T& pick2(T& a, T& b) {
  if constexpr (I == 0)
    return a;
  else
    return b;
}
// An empty asm that claims to rewrite v: any use of v after it is ordered after the
// wait that precedes it.
__device__ __forceinline__ void pin_reg(u32x2& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_reg(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_reg(i32x8& v) { asm volatile("" : "+v"(v)); }
// Waits until at most N LDS reads of this wave are outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}
// Waits until at most N global loads of this wave are outstanding and no LDS read is,
// then joins the workgroup barrier.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

// Workgroup barrier alone (the waits it needs are explicit at each use).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Issue priority of this wave relative to the other waves of its SIMD.
template <int P>
__device__ __forceinline__ void issue_prio() {
  __builtin_amdgcn_s_setprio(P);
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

template <int OPT, int SF>
__device__ __forceinline__ EpiRes epi_res(const OptArgs& a) {
  EpiRes r;
  constexpr bool Q8 = SF == ST_Q8 || SF == ST_Q8D;
  const uint32_t n = (uint32_t)a.out;
  // each resource spans its view exactly: (rows - 1) * ld + cols elements
  const uint32_t in = (uint32_t)a.in;
  r.W = make_rsrc(a.W, ((n - 1u) * (uint32_t)a.ldw + in) * 2u);
  constexpr int SL = opt_slots(OPT);
  const uint32_t es = Q8 ? 1u : (SF == ST_BF16 ? 2u : 4u);
  r.m = make_rsrc((SL & 1) ? a.m : a.W, (SL & 1) ? ((n - 1u) * (uint32_t)a.ldm + in) * es : 0u);
  r.v = make_rsrc((SL & 2) ? a.v : a.W, (SL & 2) ? ((n - 1u) * (uint32_t)a.ldv + in) * es : 0u);
  const uint32_t sb = Q8 ? n * (uint32_t)(a.in >> 6) * 4u : 0u;
  r.ms = make_rsrc(((SL & 1) && Q8) ? (const void*)a.m_scale : a.W, ((SL & 1) && Q8) ? sb : 0u);
  r.vs = make_rsrc(((SL & 2) && Q8) ? (const void*)a.v_scale : a.W, ((SL & 2) && Q8) ? sb : 0u);
  return r;
}

// SF: moment storage format (StateFmt: float32, INT8 block-64, or bfloat16).
template <class C, int EPI, int OPT, int SF, bool SR>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void gemm_kernel(GArgs g, OptArgs a, GroupArgs gr) {
  // Q8: INT8 codes with block scales, linear (ST_Q8) or the dynamic code (ST_Q8D)
  constexpr bool Q8D = SF == ST_Q8D, Q8 = SF == ST_Q8 || Q8D, B16S = SF == ST_BF16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::SMEM_BYTES];
  // dynamic-code tables, copied to LDS once (the first tile's barrier publishes them)
  const DynTables* dyn = nullptr;
  if constexpr (Q8D) {
    __shared__ DynTables dyn_lds;
    float* dst = reinterpret_cast<float*>(&dyn_lds);
    const float* src = reinterpret_cast<const float*>(&g_dyn);
    for (int j = threadIdx.x; j < (int)(sizeof(DynTables) / 4); j += C::NT) dst[j] = src[j];
    dyn = &dyn_lds;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ks = wave / (C::WM * C::WN), wsp = wave % (C::WM * C::WN);
  const int wm = wsp % C::WM, wn = wsp / C::WM;
  const int wave_m0 = wm * C::TM, wave_n0 = wn * C::TN;
  const int l32 = lane & 31, hi = lane >> 5;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A, g.a_bytes);
  // FP8 operands: the gradient is the product of the two dequantisation scales times
  // the sum of code products (B's scale is the tile's layer's, in a grouped launch)
  const float a_sc = C::F8 ? g.a_scale[0] : 1.f;

  const int ntm = g_ntm<C>(g), ntn = g_ntn<C>(g);
  const int ntiles = ntm * ntn;
  const int nst = (g.K + C::BK - 1) / C::BK;
  // Stages are issued in groups of the ring size; stages past the last one, like rows
  // past the last token, load through out-of-range offsets and so hold zeros.
  const int nstr = ((nst + C::NSTAGE - 1) / C::NSTAGE) * C::NSTAGE;
  constexpr int LPS = C::PA + C::PB;                                     // loads per stage and wave
  constexpr int NRA = C::RA * C::FM, NRB = C::B_TR ? C::RA * C::FN : C::FN;
  constexpr int NR = NRA + NRB;                                           // LDS reads per k-step and wave
  static_assert((C::NSTAGE - 1) * LPS <= 63, "vmcnt range");

  constexpr int A_RSTEP = C::NT / C::A_CPR, B_RSTEP = C::NT / C::B_CPR;
  const uint32_t a_rowb = (uint32_t)(A_RSTEP * g.lda * C::EB), a_stageb = (uint32_t)(C::BK * g.lda * C::EB);
  const uint32_t lds0 = lds_addr(smem);
  // A wave of k-split group ks reads k-steps ks*KPW .. ks*KPW + KPW-1 of each stage.
  const int kr0 = ks * C::KPW * C::KSTEP;  // first k row of this wave in a stage

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tm, tn;
    g_tile(tile, ntm, ntn, tm, tn);
    // the tile's layer (a grouped launch): its B operand, rows and pitch, and the
    // epilogue's tensors and random stream; chosen with uniform selects
    const void* t_B = g.B;
    const float* t_bsc = g.b_scale;
    uint32_t t_b_bytes = g.b_bytes;
    int64_t gt_ldb = g.ldb;
    int gt_N = g.N;
    OptArgs at = a;
    if (gr.count > 0) {
      int tn0 = 0;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) {
        const int start = j == 0 ? 0 : gr.mb[j - 1].tn1;
        if (j < gr.count && tn >= start && tn < gr.mb[j].tn1) {
          const GroupMember& M = gr.mb[j];
          tn0 = start;
          t_B = M.B;
          t_bsc = M.b_scale;
          t_b_bytes = M.b_bytes;
          gt_ldb = M.ldb;
          gt_N = M.N;
          at.W = M.W;
          at.m = M.m;
          at.v = M.v;
          at.m_scale = M.m_scale;
          at.v_scale = M.v_scale;
          at.ldw = M.ldw;
          at.ldm = M.ldm;
          at.ldv = M.ldv;
          at.out = M.N;
          at.rng_base = M.rng_base;
        }
      }
      tn -= tn0;
    }
    const float gscale = C::F8 ? a_sc * t_bsc[0] : 1.f;
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(t_B, t_b_bytes);
    const uint32_t b_rowb = (uint32_t)(B_RSTEP * gt_ldb * C::EB);
    const uint32_t b_stageb = C::B_TR ? (uint32_t)(C::BK * gt_ldb * C::EB) : (uint32_t)(C::BK * C::EB);
    const int m0 = g.m_off + tm * C::BM, n0 = g.n_off + tn * C::BN;
    // Per-thread staging offsets and fragment addresses, from an opaque copy of the thread
    // index: recomputed at every tile, so none of them is held (or spilled) through the
    // epilogue, where the registers are full.
    int ttid = tid;
    asm volatile("" : "+v"(ttid));
    const int t_lane = ttid & 63, t_hi = t_lane >> 5, t_l32 = t_lane & 31;
    // Staging: the LDS slot of this thread's chunk j in a stage is tid + j*NT (a wave's
    // load fills 64 consecutive 16-byte slots); the swizzle picks the global chunk that
    // lands there. Chunk j is A_RSTEP (B_RSTEP) rows below chunk 0.
    const int a_row0 = ttid / C::A_CPR, b_row0 = ttid / C::B_CPR;
    const int a_colb = ((ttid % C::A_CPR) ^ C::swz_tr(a_row0, C::A_CPR)) * 16;  // byte column in the row
    const int b_colb = ((ttid % C::B_CPR) ^ C::swz_b(b_row0)) * 16;

    // Byte addresses of this lane's fragment reads in stage buffer 0, k-step 0, with the
    // chunk index swizzled as the loads placed it; buffers, k-steps and the reads of one
    // fragment are immediates.
    //  * 16-bit transpose read: lane (r4, c4, half, hi) reads row 8 hi + r4, elements
    //    16 half + 4 c4 .. +3 of the 32-wide fragment; the lane receives 4 k of column l32.
    //  * 8-bit transpose read: lane pair p = (lane % 16) / 2 reads row 32 hi + p, bytes
    //    16 mh + 8 (lane % 2) .. +7 (mh = (lane / 16) % 2); the lane receives 8 k of
    //    column l32. Operand byte b of lane l then holds k = 32 (l / 32) + b in both A and B.
    auto tr_addr = [&](int base, int rowbytes, int cpr, int col0) -> uint32_t {
      int row, chunk, byte;
      if constexpr (C::F8) {
        row = kr0 + 32 * t_hi + ((t_lane & 15) >> 1);
        chunk = col0 / 16 + ((t_lane >> 4) & 1);
        byte = 8 * (t_lane & 1);
      } else {
        const int r4 = (t_lane & 15) >> 2, c4 = t_lane & 3;
        row = kr0 + 8 * t_hi + r4;
        chunk = col0 * 2 / 16 + 2 * ((t_lane >> 4) & 1) + (c4 >> 1);
        byte = 8 * (c4 & 1);
      }
      return lds0 + (uint32_t)(base + row * rowbytes + 16 * (chunk ^ C::swz_tr(row, cpr)) + byte);
    };
    uint32_t a_ad[C::FM], b_ad[C::B_TR ? C::FN : C::KPW];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) a_ad[fm] = tr_addr(C::a_base(0), C::ROWA, C::A_CPR, wave_m0 + 32 * fm);
    if constexpr (C::B_TR) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b_ad[fn] = tr_addr(C::b_base(0), C::ROWB, C::B_CPR, wave_n0 + 32 * fn);
    } else {
#pragma unroll
      for (int kk = 0; kk < C::KPW; ++kk)
        b_ad[kk] = lds0 + (uint32_t)(C::b_base(0) + (wave_n0 + t_l32) * C::ROWB +
                                     16 * ((2 * (ks * C::KPW + kk) + t_hi) ^ C::swz_b(t_l32)));
    }

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[fm][fn][e] = 0.f;

    // Only the k range is checked per load: a chunk past the M or N edge feeds
    // accumulator rows or columns that are never stored (the buffer resource still
    // bounds every access), while a k past the end must read as zero.
    const uint32_t a_base0 = (uint32_t)((a_row0 * g.lda + m0) * C::EB + a_colb);
    uint32_t b_base0;
    if constexpr (C::B_TR)
      b_base0 = (uint32_t)((b_row0 * gt_ldb + n0) * C::EB + b_colb);
    else
      b_base0 = (uint32_t)((int64_t)(n0 + b_row0) * gt_ldb * C::EB + b_colb);
    auto dma = [&](auto buf_c, int s) {
      constexpr int buf = decltype(buf_c)::value;
      const int k0 = s * C::BK;
#pragma unroll
      for (int j = 0; j < C::PA; ++j) {
        const uint32_t off = (k0 + a_row0 + j * A_RSTEP < g.K) ? a_base0 + (uint32_t)s * a_stageb + (uint32_t)j * a_rowb : kOOB;
        dma16(rA, smem + C::a_base(buf) + (j * C::NT + wave_u * 64) * 16, off);
      }
#pragma unroll
      for (int j = 0; j < C::PB; ++j) {
        const int kb = C::B_TR ? k0 + b_row0 + j * B_RSTEP : k0 + b_colb / C::EB;
        const uint32_t off = (kb < g.K) ? b_base0 + (uint32_t)s * b_stageb + (uint32_t)j * b_rowb : kOOB;
        dma16(rB, smem + C::b_base(buf) + (j * C::NT + wave_u * 64) * 16, off);
      }
    };
    // Operand fragments of one k-step as the LDS reads return them: RA pieces of 8 bytes
    // per transposed operand, one 16-byte read per k-fast B operand.
    struct FragBf16 {
      u32x2 a[C::FM][C::RA];
      u32x2 bt[C::B_TR ? C::FN : 1][C::RA];
      u32x4 bk[C::B_TR ? 1 : C::FN];
    };
    // FP8: one 8-register operand vector per fragment, filled read by read
    struct FragF8 {
      i32x8 a[C::FM];
      i32x8 bt[C::FN];
    };
    using Frag = std::conditional_t<C::F8, FragF8, FragBf16>;
    // The r-th of the NR reads of a k-step's fragments.
    auto read_one = [&](Frag& F, auto buf_c, auto kk_c, auto r_c) {
      constexpr int buf = decltype(buf_c)::value, kk = decltype(kk_c)::value, r = decltype(r_c)::value;
      if constexpr (r < NRA) {
        constexpr int fm = r / C::RA, h = r % C::RA;
        constexpr int off = C::a_base(buf) + (kk * C::KSTEP + h * C::RSTEP) * C::ROWA;
        if constexpr (C::F8) {
          const u32x2 x = ds_tr8_asm<off>(a_ad[fm]);
          F.a[fm][2 * h] = (int)x.x;
          F.a[fm][2 * h + 1] = (int)x.y;
        } else {
          F.a[fm][h] = ds_tr_asm<off>(a_ad[fm]);
        }
      } else if constexpr (C::B_TR) {
        constexpr int fn = (r - NRA) / C::RA, h = (r - NRA) % C::RA;
        constexpr int off = buf * C::B_BYTES + (kk * C::KSTEP + h * C::RSTEP) * C::ROWB;
        if constexpr (C::F8) {
          const u32x2 x = ds_tr8_asm<off>(b_ad[fn]);
          F.bt[fn][2 * h] = (int)x.x;
          F.bt[fn][2 * h + 1] = (int)x.y;
        } else {
          F.bt[fn][h] = ds_tr_asm<off>(b_ad[fn]);
        }
      } else {
        constexpr int fn = r - NRA;
        F.bk[fn] = ds_b128_asm<buf * C::B_BYTES + 32 * fn * C::ROWB>(b_ad[kk]);
      }
    };
    // Orders every later use of F's registers after the wait that precedes this.
    auto settle = [&](Frag& F) {
      if constexpr (C::F8) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) pin_reg(F.a[fm]);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) pin_reg(F.bt[fn]);
        return;
      } else {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int h = 0; h < C::RA; ++h) pin_reg(F.a[fm][h]);
      }
      if constexpr (C::B_TR && !C::F8) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int h = 0; h < C::RA; ++h) pin_reg(F.bt[fn][h]);
      } else if constexpr (!C::F8) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) pin_reg(F.bk[fn]);
      }
    };
    auto mfma_one = [&](const Frag& F, auto i_c) {
      constexpr int fm = decltype(i_c)::value / C::FN, fn = decltype(i_c)::value % C::FN;
      if constexpr (C::F8) {
        // block scales of 2^0 (E8M0 code 127): the tensor scales are applied to the sum
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[fm], F.bt[fn], acc[fm][fn], C::FA, C::FB, 0, 127,
                                                                      0, 127);
      } else {
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{F.a[fm][0].x, F.a[fm][0].y, F.a[fm][1].x, F.a[fm][1].y});
        bf16x8 bv;
        if constexpr (C::B_TR)
          bv = __builtin_bit_cast(bf16x8, u32x4{F.bt[fn][0].x, F.bt[fn][0].y, F.bt[fn][1].x, F.bt[fn][1].y});
        else
          bv = __builtin_bit_cast(bf16x8, F.bk[fn]);
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[fm][fn], 0, 0, 0);
      }
    };
    // The MFMAs of fragment set F, with the reads of the next set G spread over the
    // first half of them and `after_first` run after the first; sched_barrier keeps
    // this order.
    constexpr int NM = C::FM * C::FN;
    constexpr int RPM = (NR + NM / 2 - 1) / (NM / 2);
    auto mma_reading = [&](const Frag& F, Frag& G, auto buf_c, auto kk_c, auto&& after_first) {
      static_for<0, NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        mfma_one(F, i_c);
        if constexpr (i == 0) after_first();
        static_for<i * RPM, (i + 1) * RPM < NR ? (i + 1) * RPM : NR>([&](auto r_c) { read_one(G, buf_c, kk_c, r_c); });
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    if constexpr (C::PP) {
    // ---- ping-pong mainloop ----
    // Waves 0..3 (group A) and 4..7 (group B) hold one wave of each group on every
    // SIMD. Each group alternates a memory phase M_i (issue its share of the operand
    // loads of stage i - 1 + NSTAGE, read all fragments of stage i from LDS, wait for
    // them and for its own loads of stage i + 1) with a compute phase C_i (the MFMAs of
    // stage i from registers). Group B runs one phase behind group A, and every phase
    // ends at a workgroup barrier, so while one group multiplies, the other reads:
    //   phase 2i:   A in M_i,  B in C_{i-1}
    //   phase 2i+1: A in C_i,  B in M_i
    // Stage i's buffer is read in phases 2i and 2i+1 and refilled (stage i + NSTAGE)
    // by A in phase 2i+2 and by B in phase 2i+3, each wave loading its own share as in
    // the prologue. A wave's loads of stage s are issued in M_{s+1-NSTAGE} and waited
    // for in M_{s-1}; the barrier that ends that phase publishes them before either
    // group reads stage s.
    const bool grp_b = wave_u >= C::NW / 2;
    // Split reads: a group reads k-step 0 of stage i + 1 during C_i, between its MFMAs,
    // so M_i reads only k-step 1 of stage i and the memory phase fits under the other
    // group's MFMAs. Each wave then waits for its own loads of stage i + 2 at the end of
    // C_i, so both groups' shares of stage i + 1 have landed by the barrier before either
    // C_i (group A's C_i runs beside group B's M_i). A stage's buffer is refilled two
    // phases after its last read. Not for the dynamic 8-bit code, whose epilogue leaves no
    // registers for the third fragment set.
    constexpr bool SPLIT = FORGE_PP_SPLIT && C::KPW == 2 && C::NSTAGE % 2 == 0 && C::NSTAGE >= 4 && !Q8D;
    __syncthreads();  // the previous tile's epilogue is done with LDS
    static_for<0, C::NSTAGE>([&](auto b_c) { dma(b_c, decltype(b_c)::value); });
    if constexpr (SPLIT) {
    Frag F0[2], F1;  // k-step 0 of this stage and of the next (alternating), k-step 1
    vm_wait_barrier<(C::NSTAGE - 2) * LPS>();  // stages 0 and 1 published
    static_for<0, NR>([&](auto r_c) {
      read_one(F0[0], std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, r_c);
    });
    if (grp_b) wg_barrier();  // group B starts one phase later
    auto pp_stage = [&](auto R_c, int i) {
      constexpr int R = decltype(R_c)::value;  // i % NSTAGE
      constexpr int cur = R % 2, nxt = 1 - cur;
      // memory phase M_i: this wave's loads of stage i - 1 + NSTAGE (past the last stage
      // too: the vmcnt waits count a fixed number of loads per phase), k-step 1 of stage i
      if (i >= 1) dma(std::integral_constant<int, (R + C::NSTAGE - 1) % C::NSTAGE>{}, i - 1 + C::NSTAGE);
      static_for<0, NR>([&](auto r_c) { read_one(F1, R_c, std::integral_constant<int, 1>{}, r_c); });
      vm_wait_barrier<(C::NSTAGE - 2) * LPS>();  // fragments landed (the loads are waited in C)
      // compute phase C_i, reading k-step 0 of stage i + 1 over the first MFMAs
      settle(F0[cur]);
      settle(F1);
      __builtin_amdgcn_sched_barrier(0);
      issue_prio<FORGE_PP_PRIO>();
      mma_reading(F0[cur], F0[nxt], std::integral_constant<int, (R + 1) % C::NSTAGE>{},
                  std::integral_constant<int, 0>{}, [] {});
      static_for<0, C::FM * C::FN>([&](auto i_c) { mfma_one(F1, i_c); });
      issue_prio<0>();
      __builtin_amdgcn_sched_barrier(0);
      // own loads of stage i + 2 landed (stage i + 3's may still be in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"((C::NSTAGE - 3) * LPS) : "memory");
      wg_barrier();
    };
    for (int i0 = 0; i0 < nst; i0 += C::NSTAGE)
      static_for<0, C::NSTAGE>([&](auto r_c) {
        const int i = i0 + decltype(r_c)::value;
        if (i < nst) pp_stage(r_c, i);
      });
    // the last compute phase read k-step 0 of a stage past the end: those registers stay
    // pinned until the reads have landed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    settle(F0[0]);
    settle(F0[1]);
    } else {
    Frag F[C::KPW];
    vm_wait_barrier<(C::NSTAGE - 1) * LPS>();  // stage 0 published
    if (grp_b) wg_barrier();                     // group B starts one phase later
    auto pp_stage = [&](auto R_c, int i) {
      constexpr int R = decltype(R_c)::value;  // i % NSTAGE
      // memory phase M_i. Stages past the last one are issued too (their offsets are out of
      // range and load zeros): the vmcnt waits count a fixed number of loads per phase, and a
      // skipped load would let the wait for stage i + 1 pass before that stage has landed.
      if (i >= 1) dma(std::integral_constant<int, (R + C::NSTAGE - 1) % C::NSTAGE>{}, i - 1 + C::NSTAGE);
      static_for<0, C::KPW>([&](auto kk_c) {
        static_for<0, NR>([&](auto r_c) { read_one(F[decltype(kk_c)::value], R_c, kk_c, r_c); });
      });
      // own loads of stage i + 1 landed (later stages may still be in flight), fragments landed
      vm_wait_barrier<(C::NSTAGE - 2) * LPS>();
      // compute phase C_i
#pragma unroll
      for (int kk = 0; kk < C::KPW; ++kk) settle(F[kk]);
      __builtin_amdgcn_sched_barrier(0);
      issue_prio<FORGE_PP_PRIO>();
      static_for<0, C::KPW>([&](auto kk_c) {
        static_for<0, C::FM * C::FN>([&](auto i_c) { mfma_one(F[decltype(kk_c)::value], i_c); });
      });
      issue_prio<0>();
      __builtin_amdgcn_sched_barrier(0);
      wg_barrier();
    };
    for (int i0 = 0; i0 < nst; i0 += C::NSTAGE)
      static_for<0, C::NSTAGE>([&](auto r_c) {
        const int i = i0 + decltype(r_c)::value;
        if (i < nst) pp_stage(r_c, i);
      });
    }
    if (!grp_b) wg_barrier();  // both groups pass the same number of barriers
    // the loads of the stages past the last one still write LDS: let them land
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    } else {
    // ---- mainloop ----
    // Stage st sits in ring buffer st % NSTAGE. The k-steps' MFMAs run back to back,
    // each set reading the next set's fragments (two register sets alternate). Before
    // the last k-step of a stage every wave waits for its own loads of stage st+1 and
    // for its LDS reads, the barrier then makes stage st+1 visible and frees buffer
    // st % NSTAGE (all its reads are done), and the loads of stage st + NSTAGE into
    // that buffer are issued.
    Frag F0, F1;
    __syncthreads();  // the previous tile's epilogue is done with LDS
    static_for<0, C::NSTAGE>([&](auto b_c) { dma(b_c, decltype(b_c)::value); });
    vm_wait_barrier<(C::NSTAGE - 1) * LPS>();
    static_for<0, NR>([&](auto r_c) {
      read_one(F0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, r_c);
    });
    static_assert((C::NSTAGE * C::KPW) % 2 == 0, "register sets alternate evenly over a round of the ring");
    auto stage = [&](auto R_c, int st) {
      constexpr int R = decltype(R_c)::value;
      static_for<0, C::KPW>([&](auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
        constexpr int cur = (R * C::KPW + kk) % 2;
        Frag& Fc = pick2<cur>(F0, F1);
        Frag& Fn = pick2<1 - cur>(F0, F1);
        if constexpr (kk + 1 < C::KPW) {
          lgkm_wait<0>();
          settle(Fc);
          mma_reading(Fc, Fn, R_c, std::integral_constant<int, kk + 1>{}, [] {});
        } else {
          vm_wait_barrier<(C::NSTAGE - 2) * LPS>();
          settle(Fc);
          mma_reading(Fc, Fn, std::integral_constant<int, (R + 1) % C::NSTAGE>{}, std::integral_constant<int, 0>{},
                      [&] { dma(R_c, st + C::NSTAGE); });
        }
      });
    };
    for (int st = 0; st < nstr; st += C::NSTAGE)
      static_for<0, C::NSTAGE>([&](auto r_c) { stage(r_c, st + decltype(r_c)::value); });
    // the loads issued past the end still write LDS: let them land before it is reused.
    // The last k-step also read fragments that nothing consumes: the compiler takes
    // their registers as free once the reads are issued, so both sets stay pinned
    // until those reads have landed, else a later value placed there is overwritten.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    settle(F0);
    settle(F1);
    }

    // ---- epilogue ----
    {
    // Thread coordinates again, from an opaque copy of the thread index: nothing the epilogue
    // derives from them stays live through the mainloop, where the registers are full.
    int etid = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(etid));
    const int tid = etid, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int ks = wave / (C::WM * C::WN), wsp = wave % (C::WM * C::WN);
    const int wm = wsp % C::WM, wn = wsp / C::WM;
    const int wave_m0 = wm * C::TM;
    const int l32 = lane & 31, hi = lane >> 5;
    // The finished tile is handed through LDS one wave-column (TN rows of n) at a
    // time: the waves that own those rows write their accumulators (lane holds
    // C[m = 8q + 4*hi + j][n = l32] of each 32x32 block) as float rows, then every
    // thread takes 4 consecutive m of a row, so each wave reads and writes whole
    // contiguous row segments of W / m / v / dW / dX.
    // One 4-element vector of a weight row (elements i .. i+3 of row o): the stored moments
    // are decoded, the optimizer updates W and the moments from the FP32 gradient gx, and W and
    // the moments are rounded and stored. Raw values as stored: wb = 4 bfloat16 weights; mr / vr
    // the moments (float32: 4 words; bfloat16: .xy; INT8 codes: .x) with block scales msc / vsc.
    constexpr int ST_CPOL = FORGE_EPI_ST_CPOL;
    auto apply_vec = [&](const EpiRes& R, f32x4 gx, u32x2 wb, u32x4 mr, u32x4 vr, float msc, float vsc, int o,
                         int i, bool ok) {
      constexpr int SL = opt_slots(OPT);
      constexpr bool HAS_M = SL & 1, HAS_V = SL & 2;
      constexpr uint32_t es = Q8 ? 1u : (B16S ? 2u : 4u);
      const uint32_t ow = ok ? (uint32_t)(o * at.ldw + i) * 2u : kOOB;
      const uint32_t om = ok ? (uint32_t)(o * at.ldm + i) * es : kOOB;
      const uint32_t ov = ok ? (uint32_t)(o * at.ldv + i) * es : kOOB;
      const uint32_t osc = ok ? (uint32_t)(o * (at.in >> 6) + (i >> 6)) * 4u : kOOB;
      if constexpr (C::F8) gx = gx * gscale;
      const u32x2 mb{mr.x, mr.y}, vb{vr.x, vr.y};
      const f32x4 mv = __builtin_bit_cast(f32x4, mr), vv = __builtin_bit_cast(f32x4, vr);
      const uint32_t qm = mr.x, qv = vr.x;
      const float gg[4] = {gx.x, gx.y, gx.z, gx.w};
      float w[4] = {bits_f32(wb.x << 16), bits_f32(wb.x & 0xFFFF0000u), bits_f32(wb.y << 16),
                    bits_f32(wb.y & 0xFFFF0000u)};
      float m[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (B16S) {
        if constexpr (HAS_M) bf16x4_to_f32(mb, m);
        if constexpr (HAS_V) bf16x4_to_f32(vb, v);
      } else if constexpr (!Q8) {
        if constexpr (HAS_M) { m[0] = mv.x; m[1] = mv.y; m[2] = mv.z; m[3] = mv.w; }
        if constexpr (HAS_V) { v[0] = vv.x; v[1] = vv.y; v[2] = vv.z; v[3] = vv.w; }
      } else {
        if constexpr (Q8D) {
          if constexpr (HAS_M) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = dyn_decode_s((qm >> (8 * j)) & 0xFFu, dyn->vs) * msc;
          }
          if constexpr (HAS_V) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = dyn->vu[(qv >> (8 * j)) & 0xFFu] * vsc;
          }
        } else {
          if constexpr (HAS_M) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = (float)(int8_t)((qm >> (8 * j)) & 0xFF) * msc;
          }
          if constexpr (HAS_V) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float r = (float)((qv >> (8 * j)) & 0xFF) * vsc;
              v[j] = r * r;
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) opt_apply<OPT>(gg[j], w[j], m[j], v[j], at.s);
      const uint32_t idx0 = (uint32_t)o * (uint32_t)at.in + (uint32_t)i;
      uint64_t zz[4];  // one random word per element serves W, m and v
      rand64x4<SR>(at.rng_base, idx0, zz);
      uint32_t bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = SR ? sr_bf16_bits(w[j], rand_field(zz[j], RF_W)) : rne_bf16_bits(w[j]);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16)}, R.W, ow, 0,
                                            ST_CPOL);
      if constexpr (B16S) {
        if constexpr (HAS_M)
          __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4<SR>(m, zz, RF_M), R.m, om, 0, ST_CPOL);
        if constexpr (HAS_V)
          __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4<SR>(v, zz, RF_V), R.v, ov, 0, ST_CPOL);
      } else if constexpr (!Q8) {
        if constexpr (HAS_M)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{m[0], m[1], m[2], m[3]}), R.m, om, 0,
                                                 ST_CPOL);
        if constexpr (HAS_V)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), R.v, ov, 0,
                                                 ST_CPOL);
      } else {
        // block-64 absmax over the 16 adjacent lanes holding this row's block
        // (linear codes: of m and sqrt(v); dynamic codes: of m and v)
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
        if constexpr (Q8D) {
          if constexpr (HAS_M) __builtin_amdgcn_raw_buffer_store_b32(quant_dyn_m4(m, im, dyn->ms), R.m, om, 0, ST_CPOL);
          if constexpr (HAS_V) __builtin_amdgcn_raw_buffer_store_b32(quant_dyn_v4(r, iv, dyn->mu), R.v, ov, 0, ST_CPOL);
        } else {
          if constexpr (HAS_M) __builtin_amdgcn_raw_buffer_store_b32(quant_m4(m, im), R.m, om, 0, ST_CPOL);
          if constexpr (HAS_V) __builtin_amdgcn_raw_buffer_store_b32(quant_v4(r, iv), R.v, ov, 0, ST_CPOL);
        }
        if ((i & 63) == 0) {
          if constexpr (HAS_M) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sm), R.ms, osc, 0, ST_CPOL);
          if constexpr (HAS_V) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sv), R.vs, osc, 0, ST_CPOL);
        }
      }
    };
    // One staged block of the finished tile, as float rows of pitch LD holding VPRc 4-element
    // vectors each: NTHR threads (this one is t) take NVc vectors each; row r, column c of the
    // block is output row obase + r, column ibase + c.
    auto proc = [&](const float* Es, auto ld_c, auto vpr_c, auto nv_c, auto nthr_c, int t, int obase, int ibase) {
      constexpr int LD = decltype(ld_c)::value, VPRc = decltype(vpr_c)::value, NVc = decltype(nv_c)::value;
      constexpr int NTHR = decltype(nthr_c)::value;
      static_assert(VPRc % 16 == 0, "an INT8 block of 64 must be 16 adjacent lanes");
      if constexpr (EPI == G_EPI_STORE || EPI == G_EPI_DX) {
        const __amdgpu_buffer_rsrc_t rO = make_rsrc(g.out, g.out_bytes);
#pragma unroll
        for (int k = 0; k < NVc; ++k) {
          const int vi = t + k * NTHR, row = vi / VPRc, col = (vi % VPRc) * 4;
          const int n = obase + row, m = ibase + col;
          f32x4 x = *reinterpret_cast<const f32x4*>(Es + row * LD + col);
          if constexpr (C::F8) x = x * gscale;
          const bool ok = n < gt_N && m < g.M;
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
        const EpiRes R = epi_res<OPT, SF>(at);
        // loads of KB vectors are issued before any of them is consumed; KB bounds the
        // registers a batch holds next to the accumulators still to be written out
        constexpr int KB_MAX = Q8 && C::OCC >= 2 ? 1 : (C::OCC == 1 ? FORGE_EPI_KB1 : FORGE_EPI_KB);
        constexpr int KB = NVc > KB_MAX ? KB_MAX : NVc;
        // at most 8 batches unrolled (the one-wave FP8 tiles have 32 vectors per thread and
        // chunk: unrolling all of them exhausts the scalar registers)
#pragma unroll 8
        for (int kb = 0; kb < NVc; kb += KB) {
        uint32_t ow[KB], om[KB], ov_[KB], osc[KB];
        u32x2 wb[KB], mb[KB], vb[KB];
        f32x4 mv[KB], vv[KB];
        uint32_t qm[KB], qv[KB];
        float msc[KB], vsc[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int vi = t + (kb + k) * NTHR, row = vi / VPRc, col = (vi % VPRc) * 4;
          const int o = obase + row, i = ibase + col;
          const bool ok = o < gt_N && i < g.M;
          ow[k] = ok ? (uint32_t)(o * at.ldw + i) * 2u : kOOB;
          wb[k] = __builtin_amdgcn_raw_buffer_load_b64(R.W, ow[k], 0, FORGE_EPI_LD_CPOL);
          if constexpr (B16S) {
            om[k] = ok ? (uint32_t)(o * at.ldm + i) * 2u : kOOB;
            ov_[k] = ok ? (uint32_t)(o * at.ldv + i) * 2u : kOOB;
            if constexpr (HAS_M) mb[k] = __builtin_amdgcn_raw_buffer_load_b64(R.m, om[k], 0, FORGE_EPI_LD_CPOL);
            if constexpr (HAS_V) vb[k] = __builtin_amdgcn_raw_buffer_load_b64(R.v, ov_[k], 0, FORGE_EPI_LD_CPOL);
          } else if constexpr (!Q8) {
            om[k] = ok ? (uint32_t)(o * at.ldm + i) * 4u : kOOB;
            ov_[k] = ok ? (uint32_t)(o * at.ldv + i) * 4u : kOOB;
            if constexpr (HAS_M)
              mv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(R.m, om[k], 0, FORGE_EPI_LD_CPOL));
            if constexpr (HAS_V)
              vv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(R.v, ov_[k], 0, FORGE_EPI_LD_CPOL));
          } else {
            om[k] = ok ? (uint32_t)(o * at.ldm + i) : kOOB;
            ov_[k] = ok ? (uint32_t)(o * at.ldv + i) : kOOB;
            osc[k] = ok ? (uint32_t)(o * (at.in >> 6) + (i >> 6)) * 4u : kOOB;
            if constexpr (HAS_M) {
              qm[k] = __builtin_amdgcn_raw_buffer_load_b32(R.m, om[k], 0, FORGE_EPI_LD_CPOL);
              msc[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.ms, osc[k], 0, FORGE_EPI_LD_CPOL));
            }
            if constexpr (HAS_V) {
              qv[k] = __builtin_amdgcn_raw_buffer_load_b32(R.v, ov_[k], 0, FORGE_EPI_LD_CPOL);
              vsc[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.vs, osc[k], 0, FORGE_EPI_LD_CPOL));
            }
          }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int vi = t + (kb + k) * NTHR, row = vi / VPRc, col = (vi % VPRc) * 4;
          const int o = obase + row, i = ibase + col;
          const f32x4 gx = *reinterpret_cast<const f32x4*>(Es + row * LD + col);
          u32x4 mr{0u, 0u, 0u, 0u}, vr{0u, 0u, 0u, 0u};
          float ms_k = 0.f, vs_k = 0.f;
          if constexpr (B16S) {
            if constexpr (HAS_M) mr = u32x4{mb[k].x, mb[k].y, 0u, 0u};
            if constexpr (HAS_V) vr = u32x4{vb[k].x, vb[k].y, 0u, 0u};
          } else if constexpr (!Q8) {
            if constexpr (HAS_M) mr = __builtin_bit_cast(u32x4, mv[k]);
            if constexpr (HAS_V) vr = __builtin_bit_cast(u32x4, vv[k]);
          } else {
            if constexpr (HAS_M) { mr = u32x4{qm[k], 0u, 0u, 0u}; ms_k = msc[k]; }
            if constexpr (HAS_V) { vr = u32x4{qv[k], 0u, 0u, 0u}; vs_k = vsc[k]; }
          }
          apply_vec(R, gx, wb[k], mr, vr, ms_k, vs_k, o, i, o < gt_N && i < g.M);
        }
#if FORGE_EPI_SCHED_BARRIER
        __builtin_amdgcn_sched_barrier(0);
#endif
        }
      }
    };
    __syncthreads();  // every wave is done reading the operand stages
    // Linear INT8 codes keep the workgroup-wide staging where it fits the LDS: its rows are
    // twice as long, so the one-byte code rows move as 256-byte segments rather than 128-byte
    // ones (measured 3-4% faster on the INT8 down_proj); the other formats are as fast or
    // faster per wave.
    constexpr bool WG_FITS = C::TN * (C::BM + 4) * 4 <= C::SMEM_BYTES;
    if constexpr (C::KS == 1 && FORGE_EPI_WAVE && (SF != ST_Q8 || !WG_FITS)) {
      // Each wave stages its own accumulators, one 32-row block (fn) at a time, in a private
      // LDS region and writes them out itself: no workgroup barrier between blocks, so the
      // waves' load, arithmetic and store phases drift apart instead of running in step.
      constexpr int LDW = C::TM + 4;
      static_assert(C::NW * 32 * LDW * 4 <= C::SMEM_BYTES, "wave staging fits the workgroup's LDS");
      float* Ew = reinterpret_cast<float*>(smem) + wave_u * (32 * LDW);
      // fn is a run-time loop (one copy of the block's processing); the accumulators are
      // selected with compile-time indices under a uniform branch, so they stay in registers
#pragma unroll 1
      for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
        for (int f = 0; f < C::FN; ++f) {
          if (f == fn) {
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(Ew + l32 * LDW + 32 * fm + 8 * q + 4 * hi) =
                    f32x4{acc[fm][f][4 * q], acc[fm][f][4 * q + 1], acc[fm][f][4 * q + 2], acc[fm][f][4 * q + 3]};
          }
        }
        // the other lanes' rows are written (and, after the block, read) before going on
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        proc(Ew, std::integral_constant<int, LDW>{}, std::integral_constant<int, C::TM / 4>{},
             std::integral_constant<int, C::TM / 8>{}, std::integral_constant<int, 64>{}, lane,
             n0 + wave_n0 + 32 * fn, m0 + wave_m0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    } else {
    float* E = reinterpret_cast<float*>(smem);
    constexpr int LDE = C::BM + 4;
    constexpr int VPR = C::BM / 4;                   // 4-element vectors per row
    constexpr int NV = C::TN * VPR / C::NT;          // vectors per thread per chunk
    static_assert((C::TN * VPR) % C::NT == 0, "chunk must split evenly over threads");
    static_assert(C::TN * LDE * 4 <= C::SMEM_BYTES, "workgroup staging fits the workgroup's LDS");
#pragma unroll 1
    for (int c = 0; c < C::WN; ++c) {
      // k-split group 0 writes its partial tile, groups 1.. add theirs in order
#pragma unroll 1
      for (int kg = 0; kg < C::KS; ++kg) {
        if (wn == c && ks == kg) {
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                f32x4* e = reinterpret_cast<f32x4*>(E + (32 * fn + l32) * LDE + wave_m0 + 32 * fm + 8 * q + 4 * hi);
                f32x4 x{acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
                if (kg > 0) x = *e + x;
                *e = x;
              }
        }
        __syncthreads();
      }
      proc(E, std::integral_constant<int, LDE>{}, std::integral_constant<int, VPR>{}, std::integral_constant<int, NV>{},
           std::integral_constant<int, C::NT>{}, tid, n0 + c * C::TN, m0);
      __syncthreads();  // the chunk's LDS rows are consumed before the next chunk overwrites them
    }
    }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers. Large problems use 256x256 workgroup tiles (8 waves of 128x64, two
// per SIMD), also when they fill only part of one round (more than half of the
// compute units); smaller problems use 128x128 tiles (4 waves of 64x64, two
// workgroups per compute unit) when those fill a round, else 128x128 tiles with a
// 2-way in-workgroup split-K (8 waves of 64x64, one workgroup per compute unit), so
// a compute unit that holds a single tile still runs two waves per SIMD. A last round of 256x256
// tiles that would be at most half full is replaced by a second launch of 256x128
// tiles (8 waves of 128x64, 2-way in-workgroup split-K) over the rest of C. Split-K
// tiles that would fill at most half of the compute units become 64x128 tiles.
// ---------------------------------------------------------------------------
// Tile configurations (BM, BN, BK, WM, WN, B_TR, OCC[, NSTAGE, KS]); FORGE_*_CFG
// override them at build time for tuning sweeps.
#ifndef FORGE_BIG_PP
#define FORGE_BIG_PP 1
#endif
#ifndef FORGE_WGRAD_BIG_CFG
#define FORGE_WGRAD_BIG_CFG 256, 256, 32, 2, 4, true, 2, 4, 1, G_BF16, 0, 0, FORGE_BIG_PP
#endif
#ifndef FORGE_WGRAD_SMALL_CFG
#define FORGE_WGRAD_SMALL_CFG 128, 128, 32, 2, 2, true, 2
#endif
#ifndef FORGE_WGRAD_SPLIT_CFG
#define FORGE_WGRAD_SPLIT_CFG 128, 128, 64, 2, 2, true, 2, 4, 2
#endif
// the rest of a problem whose last round of 256x256 tiles would be at most half full:
// 256x128 tiles (half a large tile each), 8 waves of 128x64 in two k-split groups,
// a 2-deep ring of 64-token stages
#ifndef FORGE_WGRAD_BAND_CFG
#define FORGE_WGRAD_BAND_CFG 256, 128, 64, 2, 2, true, 2, 2, 2
#endif
#ifndef FORGE_DGRAD_BAND_CFG
#define FORGE_DGRAD_BAND_CFG 256, 128, 64, 2, 2, false, 2, 2, 2
#endif
// scarce 128x128 tiles (fewer than half the compute units): 64x128 tiles, 64 columns of the
// A side (in) by 128 of the B side, 8 waves of 32x64 in two k-split groups, so a problem
// with 128 or 512 output rows covers twice as many compute units
#ifndef FORGE_WGRAD_TINY_CFG
#define FORGE_WGRAD_TINY_CFG 64, 128, 64, 2, 2, true, 2, 4, 2
#endif
#ifndef FORGE_DGRAD_TINY_CFG
#define FORGE_DGRAD_TINY_CFG 64, 128, 64, 2, 2, false, 2, 4, 2
#endif
#ifndef FORGE_DGRAD_BIG_CFG
#define FORGE_DGRAD_BIG_CFG 256, 256, 32, 2, 4, false, 2, 4, 1, G_BF16, 0, 0, FORGE_BIG_PP
#endif
#ifndef FORGE_DGRAD_SMALL_CFG
#define FORGE_DGRAD_SMALL_CFG 128, 128, 32, 2, 2, false, 2
#endif
#ifndef FORGE_DGRAD_SPLIT_CFG
#define FORGE_DGRAD_SPLIT_CFG 128, 128, 64, 2, 2, false, 2, 4, 2
#endif
// FP8 operands (X in E4M3, dY in format FB): 64-token stages, one MFMA k-step each. The
// large tile runs 8 waves of 128x64 (two per SIMD) with the ping-pong mainloop: one
// fragment set of a k-step per group fits next to the 128 accumulators, and the
// epilogue has twice the waves of a one-wave-per-SIMD layout.
#ifndef FORGE_WGRAD_F8_BIG_CFG
#define FORGE_WGRAD_F8_BIG_CFG 256, 256, 64, 2, 4, true, 2, 4, 1
#endif
#ifndef FORGE_WGRAD_F8_SMALL_CFG
#define FORGE_WGRAD_F8_SMALL_CFG 128, 128, 64, 2, 2, true, 2, 4, 1
#endif
template <int FB>
#ifndef FORGE_F8_BIG_PP
#define FORGE_F8_BIG_PP 1
#endif
using WgradF8Big = GCfg<FORGE_WGRAD_F8_BIG_CFG, G_FP8, 0, FB, FORGE_F8_BIG_PP>;
template <int FB>
using WgradF8Small = GCfg<FORGE_WGRAD_F8_SMALL_CFG, G_FP8, 0, FB>;
using WgradBig = GCfg<FORGE_WGRAD_BIG_CFG>;
using WgradSmall = GCfg<FORGE_WGRAD_SMALL_CFG>;
using WgradSplit = GCfg<FORGE_WGRAD_SPLIT_CFG>;
using WgradBand = GCfg<FORGE_WGRAD_BAND_CFG>;
using WgradTiny = GCfg<FORGE_WGRAD_TINY_CFG>;
using DgradTiny = GCfg<FORGE_DGRAD_TINY_CFG>;
using DgradBand = GCfg<FORGE_DGRAD_BAND_CFG>;
using DgradBig = GCfg<FORGE_DGRAD_BIG_CFG>;
using DgradSmall = GCfg<FORGE_DGRAD_SMALL_CFG>;
using DgradSplit = GCfg<FORGE_DGRAD_SPLIT_CFG>;

// Compute units of the device current at the first launch (the library targets one
// part, gfx950); the function-local static is initialised once, thread-safely.
static int g_num_cus() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return n;
}

template <class C, int EPI, int OPT, int SF, bool SR>
static hipError_t g_launch(const GArgs& g0, const OptArgs& a, hipStream_t st, const GroupArgs* grp = nullptr) {
  GArgs g = g0;
  GroupArgs gr{};
  if (grp != nullptr) {
    // the members' tile columns one after another (C::BN rows each, a member's last one partial)
    gr = *grp;
    int tn = 0;
    for (int j = 0; j < gr.count; ++j) {
      tn += (gr.mb[j].N + C::BN - 1) / C::BN;
      gr.mb[j].tn1 = tn;
    }
    g.n_off = 0;
    g.N = tn * C::BN;
  }
  const int ntiles = g_ntm<C>(g) * g_ntn<C>(g);
  if (ntiles == 0) return hipSuccess;
  const int resident = C::OCC * 4 / C::NW * g_num_cus();  // OCC waves on each of 4 SIMDs
  const int grid = ntiles < resident ? ntiles : resident;
  hipLaunchKernelGGL((gemm_kernel<C, EPI, OPT, SF, SR>), dim3(grid), dim3(C::NT), 0, st, g, a, gr);
  return hipGetLastError();
}

template <class C>
static int g_tiles(const GArgs& g) {
  return g_ntm<C>(g) * g_ntn<C>(g);
}

// Calls f(C{}, g') for each launch of the tile configuration C over the part g' of
// the problem. Large tiles are used when there are more than half as many as compute
// units.
// When their last round would leave more than half of the compute units idle, the
// whole rounds run as large tiles over a band of tile columns (or rows, whichever
// band holds more of them), and the rest of C runs as a second launch on the same
// stream: Band tiles (half a large tile) when they fit in one round, else 128x128
// tiles. Each tile still owns its output elements outright.
template <class Big, class Small, class Split, class Band, class Tiny = Split, class F>
static hipError_t g_pick(const GArgs& g, F&& f) {
  const int cus = g_num_cus();
  const int tiles = g_tiles<Big>(g);
  if (tiles >= cus) {
    const int full = (tiles / cus) * cus, rem = tiles - full;
    const int ntm = g_ntm<Big>(g), ntn = g_ntn<Big>(g);
    const int nb = full / ntm, mb = full / ntn;  // whole tile columns / rows the rounds hold
    if (rem > 0 && 2 * rem <= cus && (nb > 0 || mb > 0)) {
      GArgs g1 = g, g2 = g;
      if (nb * ntm >= mb * ntn) {
        g1.N = g.n_off + nb * Big::BN;
        g2.n_off = g1.N;
      } else {
        g1.M = g.m_off + mb * Big::BM;
        g2.m_off = g1.M;
      }
      hipError_t e = f(Big{}, g1);
      if (e != hipSuccess) return e;
      if (g_tiles<Band>(g2) <= cus) return f(Band{}, g2);
      return g_tiles<Small>(g2) > cus ? f(Small{}, g2) : f(Split{}, g2);
    }
    return f(Big{}, g);
  }
  // more than half a round of large tiles: one partial round of them beats the 128x128
  // tiles' two rounds (their per-CU rate is lower: twice the operand bytes per flop)
  if (2 * tiles > cus) return f(Big{}, g);
  if (g_tiles<Small>(g) >= 2 * cus) return f(Small{}, g);
  // split-K tiles that would leave compute units idle: the narrower tiles when they still
  // fit in one round
  if (g_tiles<Tiny>(g) > g_tiles<Split>(g) && g_tiles<Tiny>(g) <= cus) return f(Tiny{}, g);
  return f(Split{}, g);
}

// Bytes a row-major view of rows x cols with row pitch ld spans: the last row ends at its
// last column, so a view that ends at the end of its allocation is never read past.
static uint32_t extent(int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  return rows <= 0 ? 0u : (uint32_t)(((rows - 1) * ld + cols) * es);
}

// Fused step for one optimizer on bf16 / fp32 operands (instantiated per optimizer
// in the forge_gemm_bf16_*.hip sources).
template <class C, int OPT>
static hipError_t g_launch_opt(int sf, int sr, const GArgs& g, const OptArgs& a, hipStream_t st,
                               const GroupArgs* gr = nullptr) {
  switch (sf) {
    case ST_Q8:
      return sr ? g_launch<C, G_EPI_OPT, OPT, ST_Q8, true>(g, a, st, gr)
                : g_launch<C, G_EPI_OPT, OPT, ST_Q8, false>(g, a, st, gr);
    case ST_Q8D:
      return sr ? g_launch<C, G_EPI_OPT, OPT, ST_Q8D, true>(g, a, st, gr)
                : g_launch<C, G_EPI_OPT, OPT, ST_Q8D, false>(g, a, st, gr);
    case ST_BF16:
      return sr ? g_launch<C, G_EPI_OPT, OPT, ST_BF16, true>(g, a, st, gr)
                : g_launch<C, G_EPI_OPT, OPT, ST_BF16, false>(g, a, st, gr);
    default:
      return sr ? g_launch<C, G_EPI_OPT, OPT, ST_F32, true>(g, a, st, gr)
                : g_launch<C, G_EPI_OPT, OPT, ST_F32, false>(g, a, st, gr);
  }
}

// Tile configuration of a grouped launch (the members' tiles counted together), by the same
// rules as g_pick without the band of a last round: large tiles for more than half a round,
// 128x128 tiles for at least two per compute unit, else the split-K tiles that fill more of
// the compute units in one round.
// Tile configuration(s) of a grouped launch, chosen as g_pick chooses for one layer from
// the members' total tile count. The last-round band works at member boundaries: when the
// large tiles' last round would be at most half full and a subset of the members fills
// whole rounds of large tiles while the others fit in one round of band tiles, the two
// subsets run as two launches on the stream (a band round counted as half a large one).
// f(C{}, members) launches configuration C over a group of members.
template <class Big, class Small, class Split, class Band, class Tiny, class F>
static hipError_t g_pick_group(const GArgs& g, const GroupArgs& gr, F&& f) {
  const int cus = g_num_cus();
  const unsigned all = (1u << gr.count) - 1u;
  auto tiles = [&](auto c, unsigned mask) {
    using C = decltype(c);
    int tn = 0;
    for (int j = 0; j < gr.count; ++j)
      if (mask >> j & 1u) tn += (gr.mb[j].N + C::BN - 1) / C::BN;
    return tn * ((g.M - g.m_off + C::BM - 1) / C::BM);
  };
  auto subset = [&](unsigned mask) {
    GroupArgs s{};
    for (int j = 0; j < gr.count; ++j)
      if (mask >> j & 1u) s.mb[s.count++] = gr.mb[j];
    return s;
  };
  const int tb = tiles(Big{}, all);
  if (tb >= cus) {
    const int rounds = (tb + cus - 1) / cus, rem = tb % cus;
    if (rem > 0 && 2 * rem <= cus) {
      for (unsigned s = 1; s < all; ++s) {
        const int ts = tiles(Big{}, s);
        if (ts % cus == 0 && 2 * (ts / cus) + 1 < 2 * rounds && tiles(Band{}, all & ~s) <= cus) {
          hipError_t e = f(Big{}, subset(s));
          return e != hipSuccess ? e : f(Band{}, subset(all & ~s));
        }
      }
    }
    return f(Big{}, gr);
  }
  if (2 * tb > cus) return f(Big{}, gr);
  if (tiles(Small{}, all) >= 2 * cus) return f(Small{}, gr);
  if (tiles(Tiny{}, all) > tiles(Split{}, all) && tiles(Tiny{}, all) <= cus) return f(Tiny{}, gr);
  return f(Split{}, gr);
}

// The fused step of the layers of a group (bf16 operands): one launch over all their
// tiles (two when the last round is filled with band tiles).
template <int OPT>
hipError_t wgrad_fused_bf16_group_opt(int sf, int sr, const GArgs& g, const OptArgs& a, const GroupArgs& gr,
                                      hipStream_t st) {
  return g_pick_group<WgradBig, WgradSmall, WgradSplit, WgradBand, WgradTiny>(
      g, gr, [&](auto c, const GroupArgs& sub) { return g_launch_opt<decltype(c), OPT>(sf, sr, g, a, st, &sub); });
}

template <int OPT>
hipError_t wgrad_fused_bf16_opt(int sf, int sr, const GArgs& g, const OptArgs& a, hipStream_t st) {
  return g_pick<WgradBig, WgradSmall, WgradSplit, WgradBand, WgradTiny>(
      g, [&](auto c, const GArgs& gc) { return g_launch_opt<decltype(c), OPT>(sf, sr, gc, a, st); });
}

// FP8 operands, dY in format FB (0 = E4M3, 1 = E5M2): the fused step of one
// optimizer, and the float32 dW store (instantiated in forge_gemm_f8_*.hip).
template <class C, int OPT>
static hipError_t g_launch_opt_f8(int sf, int sr, const GArgs& g, const OptArgs& a, hipStream_t st) {
  return g_launch_opt<C, OPT>(sf, sr, g, a, st);
}

// sf: any moment format (float32, bfloat16, INT8 linear or dynamic codes)
template <int OPT, int FB>
hipError_t wgrad_fused_f8_opt(int sf, int sr, const GArgs& g, const OptArgs& a, hipStream_t st) {
  return g_pick<WgradF8Big<FB>, WgradF8Small<FB>, WgradF8Small<FB>, WgradF8Small<FB>>(
      g, [&](auto c, const GArgs& gc) { return g_launch_opt_f8<decltype(c), OPT>(sf, sr, gc, a, st); });
}

// The fused step of the layers of a group, FP8 operands (dY of every layer in format FB).
template <int OPT, int FB>
hipError_t wgrad_fused_f8_group_opt(int sf, int sr, const GArgs& g, const OptArgs& a, const GroupArgs& gr,
                                    hipStream_t st) {
  return g_pick_group<WgradF8Big<FB>, WgradF8Small<FB>, WgradF8Small<FB>, WgradF8Small<FB>, WgradF8Small<FB>>(
      g, gr, [&](auto c, const GroupArgs& sub) { return g_launch_opt<decltype(c), OPT>(sf, sr, g, a, st, &sub); });
}

template <int FB>
hipError_t wgrad_store_f8(const GArgs& g, hipStream_t st) {
  OptArgs a{};
  return g_pick<WgradF8Big<FB>, WgradF8Small<FB>, WgradF8Small<FB>, WgradF8Small<FB>>(
      g, [&](auto c, const GArgs& gc) { return g_launch<decltype(c), G_EPI_STORE, FORGE_SGD, ST_F32, false>(gc, a, st); });
}

#define FORGE_EXTERN_BF16(OPT)                                                                          \
  extern template hipError_t wgrad_fused_bf16_opt<OPT>(int, int, const GArgs&, const OptArgs&, hipStream_t); \
  extern template hipError_t wgrad_fused_bf16_group_opt<OPT>(int, int, const GArgs&, const OptArgs&,         \
                                                             const GroupArgs&, hipStream_t);
#define FORGE_INST_BF16(OPT)                                                                     \
  template hipError_t wgrad_fused_bf16_opt<OPT>(int, int, const GArgs&, const OptArgs&, hipStream_t); \
  template hipError_t wgrad_fused_bf16_group_opt<OPT>(int, int, const GArgs&, const OptArgs&, const GroupArgs&, hipStream_t);
#define FORGE_EXTERN_F8(OPT, FB)                                                                          \
  extern template hipError_t wgrad_fused_f8_opt<OPT, FB>(int, int, const GArgs&, const OptArgs&, hipStream_t); \
  extern template hipError_t wgrad_fused_f8_group_opt<OPT, FB>(int, int, const GArgs&, const OptArgs&,         \
                                                               const GroupArgs&, hipStream_t);
#define FORGE_INST_F8(OPT, FB)                                                                       \
  template hipError_t wgrad_fused_f8_opt<OPT, FB>(int, int, const GArgs&, const OptArgs&, hipStream_t); \
  template hipError_t wgrad_fused_f8_group_opt<OPT, FB>(int, int, const GArgs&, const OptArgs&, const GroupArgs&, hipStream_t);

}  // namespace forge
