// Internal device/host helpers of the forge library (not part of the C ABI).
//
// Everything here serves the fused weight-gradient + optimizer step of the
// FORGE explainer pages (technical summary, §2 Method): the counter-hash RNG
// and stochastic rounding for the bfloat16 weight write-back, the per-element
// optimizer arithmetic that runs on the FP32 accumulator registers, and the
// INT8 block-64 moment codec.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/forge.h"

namespace forge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// State formats of the moment slots.
enum StateFmt { ST_F32 = 0, ST_Q8 = 1, ST_BF16 = 2, ST_Q8D = 3 };
// Which slots an optimizer keeps (bit 0: m, bit 1: v).
__host__ __device__ constexpr int opt_slots(int opt) {
  return opt == FORGE_ADAMW ? 3 : opt == FORGE_SGD ? 0 : opt == FORGE_SGD_MOMENTUM ? 1
       : opt == FORGE_LION ? 1 : opt == FORGE_RMSPROP ? 2 : opt == FORGE_ADAGRAD ? 2
       : opt == FORGE_NADAM ? 3 : 3;
}

// ---------------------------------------------------------------------------
// Counter-based random bits and stochastic rounding (§2 "Precision and
// fidelity": stochastic rounding of the bfloat16 weight write-back so sub-ULP
// updates accumulate without bias). The counter of element idx at step t is
// (t << 32) | idx; its random word is SplitMix64 output number counter+1 from
// state `seed` (Steele, Lea & Flood, OOPSLA 2014); the top 16 bits are used.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// seed + gamma*(counter+1) for counter = (step<<32)|idx, split so the step part
// is computed once per launch: base = seed + gamma*(step<<32).
__host__ __device__ __forceinline__ uint64_t rng_base(uint64_t seed, uint64_t step) {
  return seed + 0x9E3779B97F4A7C15ull * (step << 32);
}
// The random word of element idx; its 16-bit fields round the element's bfloat16
// write-backs: bits 48..63 the weight, bits 32..47 the first moment m, bits 16..31
// the second moment v (one SplitMix64 evaluation serves all three).
__host__ __device__ __forceinline__ uint64_t rand64_from_base(uint64_t base, uint32_t idx) {
  return splitmix64_mix(base + 0x9E3779B97F4A7C15ull * ((uint64_t)idx + 1ull));
}
enum RandField { RF_W = 0, RF_M = 1, RF_V = 2 };
__host__ __device__ __forceinline__ uint32_t rand_field(uint64_t z, int field) {
  return (uint32_t)(z >> (48 - 16 * field)) & 0xFFFFu;
}
__host__ __device__ __forceinline__ uint32_t rand16_from_base(uint64_t base, uint32_t idx) {
  return rand_field(rand64_from_base(base, idx), RF_W);
}

__host__ __device__ __forceinline__ uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}
__host__ __device__ __forceinline__ float bits_f32(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}

// bfloat16 bits of x rounded stochastically with random bits r16 < 2^16.
__host__ __device__ __forceinline__ uint32_t sr_bf16_bits(float x, uint32_t r16) {
  const uint32_t u = f32_bits(x);
  const uint32_t rounded = (u + r16) >> 16, qnan = ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rounded;  // a select, not a branch
}
// bfloat16 bits of x rounded to nearest, ties to even.
__host__ __device__ __forceinline__ uint32_t rne_bf16_bits(float x) {
  const uint32_t u = f32_bits(x);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16, qnan = ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rounded;
}
__host__ __device__ __forceinline__ float bf16_bits_f32(uint32_t b) { return bits_f32(b << 16); }

// ---------------------------------------------------------------------------
// Per-element optimizer updates on FP32 registers (§2 "Core mechanism", step 2:
// the update runs on the completed gradient tile inside the registers). g is
// the gradient element, w the weight, m/v the moment slots. Scalars come from
// the host (forge_step_scalars), so the same code serves every step.
// ---------------------------------------------------------------------------
template <int OPT>
__device__ __forceinline__ void opt_apply(float g, float& w, float& m, float& v, const forge_scalars& s) {
  if constexpr (OPT == FORGE_ADAMW) {
    w = w * s.decay;
    m = fmaf(s.b1, m, s.omb1 * g);
    v = fmaf(s.b2, v, s.omb2 * (g * g));
    float denom = fmaf(sqrtf(v), s.inv_sqrt_bc2, s.eps);
    w = w - s.step_size * (m / denom);
  } else if constexpr (OPT == FORGE_SGD) {
    float d = fmaf(s.wd, w, g);
    w = w - s.lr * d;
  } else if constexpr (OPT == FORGE_SGD_MOMENTUM) {
    float d = fmaf(s.wd, w, g);
    m = fmaf(s.b1, m, s.omb1 * d);  // b1 = 0, omb1 = 1 on step 1 (buffer starts as d)
    float dir = s.flag ? fmaf(s.c_m, m, d) : m;
    w = w - s.lr * dir;
  } else if constexpr (OPT == FORGE_LION) {
    float c = fmaf(s.b1, m, s.omb1 * g);
    float sg = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
    w = w * s.decay - s.lr * sg;
    m = fmaf(s.b2, m, s.omb2 * g);
  } else if constexpr (OPT == FORGE_RMSPROP) {
    float d = fmaf(s.wd, w, g);
    v = fmaf(s.b2, v, s.omb2 * (d * d));
    w = w - s.lr * (d / (sqrtf(v) + s.eps));
  } else if constexpr (OPT == FORGE_ADAGRAD) {
    float d = fmaf(s.wd, w, g);
    v = fmaf(d, d, v);
    w = w - s.lr * (d / (sqrtf(v) + s.eps));
  } else if constexpr (OPT == FORGE_NADAM) {
    float d = fmaf(s.wd, w, g);
    m = fmaf(s.b1, m, s.omb1 * d);
    v = fmaf(s.b2, v, s.omb2 * (d * d));
    float denom = fmaf(sqrtf(v), s.inv_sqrt_bc2, s.eps);
    w = w - fmaf(s.c_g, d, s.c_m * m) / denom;
  } else {  // FORGE_RADAM
    float d = fmaf(s.wd, w, g);
    m = fmaf(s.b1, m, s.omb1 * d);
    v = fmaf(s.b2, v, s.omb2 * (d * d));
    if (s.flag)
      w = w - s.step_size * (m / (sqrtf(v) + s.eps));
    else
      w = w - s.step_size * m;
  }
}

// Arguments of the optimizer part, shared by the fused epilogue and the
// stand-alone element-wise kernel of the unfused baseline.
struct OptArgs {
  void* W;            // [out, ldw] bf16 or f32
  void* m;            // [out, ldm] f32, bf16 or int8
  void* v;            // [out, ldv] f32, bf16 or uint8
  float* m_scale;     // [out, in/64]  (INT8 codes only)
  float* v_scale;     // [out, in/64]  (INT8 codes only)
  int64_t ldw, ldm, ldv;
  int32_t out, in;
  uint64_t rng_base;  // rng_base(seed, step)
  forge_scalars s;
};

// Loads 4 consecutive weights W[o][i..i+3] as float.
template <bool W_BF16>
__device__ __forceinline__ void load_w4(const OptArgs& a, int o, int i, float w[4]) {
  if constexpr (W_BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(a.W) + (int64_t)o * a.ldw + i;
    u32x2 r = *reinterpret_cast<const u32x2*>(p);
    w[0] = bits_f32(r.x << 16);
    w[1] = bits_f32(r.x & 0xFFFF0000u);
    w[2] = bits_f32(r.y << 16);
    w[3] = bits_f32(r.y & 0xFFFF0000u);
  } else {
    const float* p = reinterpret_cast<const float*>(a.W) + (int64_t)o * a.ldw + i;
    f32x4 r = *reinterpret_cast<const f32x4*>(p);
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  }
}

// Stores 4 consecutive weights; bfloat16 with stochastic rounding or nearest-even.
// Four consecutive bfloat16 values (8 bytes) <-> float.
__device__ __forceinline__ void bf16x4_to_f32(u32x2 r, float x[4]) {
  x[0] = bits_f32(r.x << 16);
  x[1] = bits_f32(r.x & 0xFFFF0000u);
  x[2] = bits_f32(r.y << 16);
  x[3] = bits_f32(r.y & 0xFFFF0000u);
}
// Rounds four consecutive elements to bfloat16: stochastically with field `field`
// of their random words z[0..3], or to nearest-even.
template <bool SR>
__device__ __forceinline__ u32x2 pack_bf16x4(const float x[4], const uint64_t z[4], int field) {
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = SR ? sr_bf16_bits(x[j], rand_field(z[j], field)) : rne_bf16_bits(x[j]);
  return u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
}
// The random words of four consecutive elements idx0..idx0+3 (only with stochastic rounding).
// Consecutive counters differ by one, so their SplitMix64 states differ by the golden gamma:
// one 64-bit product for the first, additions for the rest (element indices stay below 2^32).
template <bool SR>
__device__ __forceinline__ void rand64x4(uint64_t base, uint32_t idx0, uint64_t z[4]) {
  if constexpr (SR) {
    uint64_t c = base + 0x9E3779B97F4A7C15ull * ((uint64_t)idx0 + 1ull);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = splitmix64_mix(c);
      c += 0x9E3779B97F4A7C15ull;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = 0ull;
  }
}

// Stores four consecutive weights; bf16 weights round with field RF_W of z[0..3].
template <bool W_BF16, bool SR>
__device__ __forceinline__ void store_w4(const OptArgs& a, int o, int i, const float w[4], const uint64_t z[4]) {
  if constexpr (W_BF16) {
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (SR)
        b[j] = sr_bf16_bits(w[j], rand_field(z[j], RF_W));
      else
        b[j] = rne_bf16_bits(w[j]);
    }
    u32x2 r;
    r.x = b[0] | (b[1] << 16);
    r.y = b[2] | (b[3] << 16);
    uint16_t* p = reinterpret_cast<uint16_t*>(a.W) + (int64_t)o * a.ldw + i;
    *reinterpret_cast<u32x2*>(p) = r;
  } else {
    float* p = reinterpret_cast<float*>(a.W) + (int64_t)o * a.ldw + i;
    *reinterpret_cast<f32x4*>(p) = f32x4{w[0], w[1], w[2], w[3]};
  }
}

__device__ __forceinline__ void load_f4(const void* base, int64_t ld, int o, int i, float x[4]) {
  f32x4 r = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + (int64_t)o * ld + i);
  x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
}
__device__ __forceinline__ void store_f4(void* base, int64_t ld, int o, int i, const float x[4]) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + (int64_t)o * ld + i) = f32x4{x[0], x[1], x[2], x[3]};
}

// INT8 block-64 codec (§2 "Precision and fidelity": INT8 optimizer states with
// blocks of 64). m: signed codes, value q*s, s = absmax/127. v: unsigned codes
// of sqrt(v), value (q*s)^2, s = max sqrt(v)/255. All-zero block: s = 0, q = 0.
__device__ __forceinline__ void dequant_m4(const OptArgs& a, int o, int i, float x[4]) {
  const int8_t* p = reinterpret_cast<const int8_t*>(a.m) + (int64_t)o * a.ldm + i;
  uint32_t q = *reinterpret_cast<const uint32_t*>(p);
  float s = a.m_scale[(int64_t)o * (a.in >> 6) + (i >> 6)];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = (float)(int8_t)((q >> (8 * j)) & 0xFF) * s;
}
__device__ __forceinline__ void dequant_v4(const OptArgs& a, int o, int i, float x[4]) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(a.v) + (int64_t)o * a.ldv + i;
  uint32_t q = *reinterpret_cast<const uint32_t*>(p);
  float s = a.v_scale[(int64_t)o * (a.in >> 6) + (i >> 6)];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r = (float)((q >> (8 * j)) & 0xFF) * s;
    x[j] = r * r;
  }
}
// Quantises 4 values with the reciprocal of the block scale, inv = 127 / absmax (m) or
// 255 / absmax (sqrt v), 0 for an all-zero block (already reduced over the block): the
// code is RNE(x * inv), clamped. Multiplying by the reciprocal instead of dividing by the
// stored scale moves x * inv by at most about one float32 ulp, which changes a code only
// where the quotient lies that close to a rounding midpoint, and then by one step.
__device__ __forceinline__ uint32_t quant_m4(const float x[4], float inv) {
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = fminf(fmaxf(rintf(x[j] * inv), -127.f), 127.f);
    q |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * j);
  }
  return q;
}
__device__ __forceinline__ uint32_t quant_v4(const float r[4], float inv) {  // r = sqrt(v)
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = fminf(fmaxf(rintf(r[j] * inv), 0.f), 255.f);
    q |= ((uint32_t)c & 0xFFu) << (8 * j);
  }
  return q;
}
// inv of a block from its absmax: levels / absmax through the hardware reciprocal (within
// one ulp; it only feeds the code decision above), or 0 for an all-zero block
__device__ __forceinline__ float block_inv(float absmax, float levels) {
  return absmax > 0.f ? levels * __builtin_amdgcn_rcpf(absmax) : 0.f;
}

// ---------------------------------------------------------------------------
// Dynamic 8-bit moment code on blocks of 64 (normalised by the block absmax):
// the code family of the standard 8-bit optimizers (dynamic tree quantization,
// Dettmers et al., "8-bit Optimizers via Block-wise Quantization"), with values
// of this library's own construction. A code's n magnitude bits hold, from the
// top, E zeros (the decade), an indicator 1, then F = n - 1 - E fraction bits f;
// its magnitude is 10^-E (0.1 + 0.9 (f + 1) / 2^F), i.e. the exact rational
// (2^F + 9 (f + 1)) / (2^F 10^(E+1)), taken as float of its double quotient;
// the all-zero magnitude is 0, the all-ones one exactly 1. Signed codes (m):
// sign << 7 | 7-bit magnitude index; unsigned codes (v): 8-bit index. Encoding
// takes the nearest magnitude: the index is the number of float midpoints of
// neighbouring magnitudes that are <= |y|, ties going to the larger.
// ---------------------------------------------------------------------------
struct DynTables {
  float vs[128];  // signed-code magnitudes
  float ms[128];  // their 127 midpoints, then +inf
  float vu[256];  // unsigned-code magnitudes
  float mu[256];  // their 255 midpoints, then +inf
};
constexpr float dyn_magnitude(int k, int nbits) {
  if (k == 0) return 0.f;
  int F = 0;
  while ((k >> (F + 1)) != 0) ++F;
  const int E = nbits - 1 - F, f = k - (1 << F);
  double den = (double)(1 << F);
  for (int j = 0; j <= E; ++j) den *= 10.0;
  return (float)((double)((1 << F) + 9 * (f + 1)) / den);
}
constexpr DynTables make_dyn_tables() {
  DynTables t{};
  for (int k = 0; k < 128; ++k) t.vs[k] = dyn_magnitude(k, 7);
  for (int k = 0; k < 256; ++k) t.vu[k] = dyn_magnitude(k, 8);
  for (int k = 0; k < 127; ++k) t.ms[k] = (float)(((double)t.vs[k] + (double)t.vs[k + 1]) * 0.5);
  for (int k = 0; k < 255; ++k) t.mu[k] = (float)(((double)t.vu[k] + (double)t.vu[k + 1]) * 0.5);
  t.ms[127] = __builtin_huge_valf();
  t.mu[255] = __builtin_huge_valf();
  return t;
}
// Device copy (one per translation unit that uses it; read-only).
static __constant__ DynTables g_dyn = make_dyn_tables();

// Number of the N sorted midpoints mid[0..N-1] (padded with +inf) that are <= a:
// plain binary search (the reference form of the encoder).
template <int N>
__host__ __device__ __forceinline__ uint32_t dyn_search(const float* mid, float a) {
  uint32_t k = 0;
#pragma unroll
  for (int step = N / 2; step >= 1; step >>= 1) k += (mid[k + step - 1] <= a) ? (uint32_t)step : 0u;
  return k;
}
// The same count for a code of NB magnitude bits, from a guess and one check: the
// decade of a is found by comparing with the float powers 10^-1 .. 10^-(NB-1), the
// index inside it by inverting the linear fraction (k = 2^F (t + 0.8) / 0.9 - 1 for
// t = a 10^E); the guess is within one step of the count for every float a in
// [0, 1] (checked exhaustively on the host), so the midpoints on either side of it
// settle the answer. All operations are IEEE float with no contraction, so the
// guess is the same on host and device.
// a <= 0 (and NaN) give 0.
template <int NB>
__host__ __device__ __forceinline__ uint32_t dyn_search_fast(const float* mid, float a) {
#pragma clang fp contract(off)
  if (!(a > 0.f)) return 0u;
  constexpr float kPow10Neg[8] = {1.f, 1e-1f, 1e-2f, 1e-3f, 1e-4f, 1e-5f, 1e-6f, 1e-7f};
  float p = 1.f;
  int F = NB - 1;
#pragma unroll
  for (int j = 1; j < NB; ++j) {
    const bool below = a <= kPow10Neg[j];
    p = below ? p * 10.f : p;
    F -= below ? 1 : 0;
  }
  const float kr = ldexpf((a * p + 0.8f) * (1.f / 0.9f), F) - 1.f;
  int k = (int)rintf(kr);
  k = k < 0 ? 0 : (k > (1 << NB) - 1 ? (1 << NB) - 1 : k);
  const float hi = mid[k];
  const float lo = k > 0 ? mid[k - 1] : -__builtin_huge_valf();
  return (uint32_t)(k + (hi <= a ? 1 : 0) - (lo > a ? 1 : 0));
}
__host__ __device__ __forceinline__ uint32_t dyn_encode_s(float y, const float* mid) {
  const uint32_t k = dyn_search_fast<7>(mid, fabsf(y));
  return (y < 0.f && k != 0u) ? (k | 0x80u) : k;
}
__host__ __device__ __forceinline__ uint32_t dyn_encode_u(float y, const float* mid) { return dyn_search_fast<8>(mid, y); }
__host__ __device__ __forceinline__ float dyn_decode_s(uint32_t b, const float* vs) {
  const float x = vs[b & 0x7Fu];
  return (b & 0x80u) ? -x : x;
}
// 4 values with the reciprocal inv = 1 / absmax of their block (0 for an all-zero block,
// already reduced over the block) -> 4 codes; as for the linear codes, the product stands
// in for the quotient.
__host__ __device__ __forceinline__ uint32_t quant_dyn_m4(const float x[4], float inv, const float* mid) {
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) q |= dyn_encode_s(x[j] * inv, mid) << (8 * j);
  return q;
}
__host__ __device__ __forceinline__ uint32_t quant_dyn_v4(const float x[4], float inv, const float* mid) {
  uint32_t q = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) q |= dyn_encode_u(x[j] * inv, mid) << (8 * j);
  return q;
}

// Host-side launchers (defined in the .hip files).
struct GemmDims {
  int32_t T, out, in;
  int64_t ldx, lddy;
};

hipError_t launch_wgrad_fused(int io_bf16, int state_fmt, int opt, int sr, const void* X, const void* dY,
                              const GemmDims& d, const OptArgs& a, hipStream_t stream);
hipError_t launch_wgrad_store(int io_bf16, const void* X, const void* dY, const GemmDims& d, float* dW,
                              int64_t ld_dw, hipStream_t stream);
hipError_t launch_optimizer(int w_bf16, int state_fmt, int opt, int sr, const float* dW, int64_t ld_dw,
                            const OptArgs& a, hipStream_t stream);
hipError_t launch_dgrad(int io_bf16, const void* dY, int64_t lddy, const void* W, int64_t ldw, void* dX,
                        int64_t lddx, int32_t T, int32_t out, int32_t in, hipStream_t stream);
// bfloat16 / FP8 kernels (forge_gemm.hip, forge_gemm_kernel.h)
hipError_t launch_wgrad_fused_bf16(int state_fmt, int opt, int sr, const void* X, const void* dY, const GemmDims& d,
                                   const OptArgs& a, hipStream_t stream);
hipError_t launch_wgrad_store_bf16(const void* X, const void* dY, const GemmDims& d, float* dW, int64_t ld_dw,
                                   hipStream_t stream);
hipError_t launch_wgrad_fused_f8(int dy_e5m2, int state_fmt, int opt, int sr, const void* X, const float* x_scale, const void* dY,
                                 const float* dy_scale, const GemmDims& d, const OptArgs& a, hipStream_t st);
hipError_t launch_wgrad_store_f8(int dy_e5m2, const void* X, const float* x_scale, const void* dY,
                                 const float* dy_scale, const GemmDims& d, float* dW, int64_t ld_dw, hipStream_t st);
hipError_t launch_dgrad_bf16(const void* dY, int64_t lddy, const void* W, int64_t ldw, void* dX, int64_t lddx,
                             int32_t T, int32_t out, int32_t in, hipStream_t stream);
// One member of a grouped fused step (layers sharing X): its dY and epilogue arguments.
struct GroupLayer {
  const void* dY;
  int64_t lddy;
  const float* dy_scale;  // FP8 dY: its dequantisation scale (else unused)
  OptArgs a;
};
// The fused step of n (1..FORGE_MAX_GROUP) layers that share X, one launch; d holds T, in
// and X's pitch; a's scalars are common to the layers. bf16 operands, or FP8 codes (X in
// E4M3 with scale x_scale, every dY in E4M3 or, dy_e5m2, E5M2, each with its own scale).
hipError_t launch_wgrad_fused_bf16_group(int state_fmt, int opt, int sr, const void* X, const GemmDims& d,
                                         const GroupLayer* layers, int n, hipStream_t stream);
hipError_t launch_wgrad_fused_f8_group(int dy_e5m2, int state_fmt, int opt, int sr, const void* X,
                                       const float* x_scale, const GemmDims& d, const GroupLayer* layers, int n,
                                       hipStream_t stream);

}  // namespace forge
