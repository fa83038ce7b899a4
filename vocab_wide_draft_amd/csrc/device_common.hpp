// Device building blocks shared by the row kernels: block geometry, wave and
// block reductions/scans, order-preserving keys, the correctly rounded
// binary32 exponential and the exact weight-sum accumulator.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int BS = 1024;            // threads per row workgroup (16 wave64s)
constexpr int NW = BS / 64;         // waves per workgroup
constexpr uint32_t kMass = 1u << 24;
constexpr int kHistBins = 4096;     // histogram bins of one select pass
constexpr int kCandCap = 2048;      // candidates a select may collect in LDS
constexpr int kMaxIter = 256;       // (V_MAX / 4) / BS vector iterations per row

// Phase hooks: with DSPARK_PHASE_TIMING defined, DSPARK_PHASE(k) adds the
// cycles since the previous hook of the workgroup to counter k (read with
// dspark_debug_phases); otherwise they compile to nothing.
#ifdef DSPARK_PHASE_TIMING
extern __device__ unsigned long long g_phase[128];  // [k] cycles, [64 + k] calls; [110 + ...] workgroups
#define DSPARK_PHASE_BEGIN long long dspark_pt0_ = clock64();
#define DSPARK_PHASE(k)                                                                   \
  do {                                                                                    \
    __syncthreads();                                                                      \
    if (threadIdx.x == 0) {                                                               \
      const long long t_ = clock64();                                                     \
      atomicAdd(&g_phase[k], (unsigned long long)(t_ - dspark_pt0_));                     \
      atomicAdd(&g_phase[64 + (k)], 1ull);                                                \
      dspark_pt0_ = t_;                                                                   \
    }                                                                                     \
  } while (0)
#define DSPARK_PHASE_ARG , dspark_pt0_
#define DSPARK_PHASE_PARAM , long long& dspark_pt0_
// the same, once every outstanding vector memory access has completed
#define DSPARK_PHASE_LOADED(k)                        \
  do {                                                \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); \
    DSPARK_PHASE(k);                                  \
  } while (0)
// per-kind workgroup wall time (100 MHz counter) and shader cycles
#define DSPARK_WG_BEGIN                                     \
  const long long dspark_w0_ = wall_clock64(), dspark_c0_ = clock64();
#define DSPARK_WG_END(kind)                                                                 \
  do {                                                                                      \
    __syncthreads();                                                                        \
    if (threadIdx.x == 0) {                                                                 \
      const long long w1_ = wall_clock64();                                                 \
      atomicAdd(&g_phase[110 + (kind)], (unsigned long long)(w1_ - dspark_w0_));           \
      atomicAdd(&g_phase[113 + (kind)], (unsigned long long)(clock64() - dspark_c0_));     \
      atomicAdd(&g_phase[116 + (kind)], 1ull);                                              \
      if (blockIdx.x < kTraceMax) {                                                         \
        uint32_t hw_, xcc_;                                                                 \
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw_));                  \
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc_));                \
        g_trace[3 * blockIdx.x] = (unsigned long long)dspark_w0_;                           \
        g_trace[3 * blockIdx.x + 1] = (unsigned long long)w1_;                              \
        g_trace[3 * blockIdx.x + 2] = ((unsigned long long)xcc_ << 32) | hw_ | ((unsigned long long)(kind) << 48); \
      }                                                                                     \
    }                                                                                       \
  } while (0)
#else
#define DSPARK_PHASE_LOADED(k) \
  do {                         \
  } while (0)
#define DSPARK_WG_BEGIN
#define DSPARK_WG_END(kind) \
  do {                      \
  } while (0)
#define DSPARK_PHASE_ARG
#define DSPARK_PHASE_PARAM
#define DSPARK_PHASE_BEGIN
#define DSPARK_PHASE(k) \
  do {                  \
  } while (0)
#endif

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------- wave ops
// 32-bit sum over the 64 lanes with DPP moves (quad swaps, half-row and row
// mirrors, then the row broadcasts of lanes 15 and 31); lane 63 ends with the
// total, which is read back as a scalar.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xb1, 0xf, 0xf, false);   // quad_perm 1,0,3,2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4e, 0xf, 0xf, false);   // quad_perm 2,3,0,1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, false);  // row_half_mirror
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xf, 0xf, false);  // row_mirror
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
// DPP lane moves (all lanes of the wave active): lanes whose source is out
// of range, or whose row / bank is masked off, keep `old`.
template <int CTRL, int RM, int BM>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, RM, BM, false);
}
template <int CTRL, int RM, int BM, class T>
__device__ __forceinline__ T dpp_t(T old, T x) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit lane values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_u32<CTRL, RM, BM>(__builtin_bit_cast(uint32_t, old), __builtin_bit_cast(uint32_t, x)));
  } else {
    const uint64_t o = __builtin_bit_cast(uint64_t, old), v = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = dpp_u32<CTRL, RM, BM>((uint32_t)o, (uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, RM, BM>((uint32_t)(o >> 32), (uint32_t)(v >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
template <class T>
__device__ __forceinline__ T readlane63(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, (uint32_t)__builtin_amdgcn_readlane((int)__builtin_bit_cast(uint32_t, v), 63));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
// Reduction over the 64 lanes: quad swaps, half-row and row mirrors give
// every lane its row's result; the row broadcasts of lanes 15 and 31 then
// fold the four rows into lane 63, which is read back as a scalar.
template <class T, class OP>
__device__ __forceinline__ T wave_reduce(T v, T id, OP op) {
  v = op(v, dpp_t<0xb1, 0xf, 0xf>(id, v));   // quad_perm 1,0,3,2
  v = op(v, dpp_t<0x4e, 0xf, 0xf>(id, v));   // quad_perm 2,3,0,1
  v = op(v, dpp_t<0x141, 0xf, 0xf>(id, v));  // row_half_mirror
  v = op(v, dpp_t<0x140, 0xf, 0xf>(id, v));  // row_mirror
  v = op(v, dpp_t<0x142, 0xa, 0xf>(id, v));  // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_t<0x143, 0xc, 0xf>(id, v));  // row_bcast:31 into rows 2 and 3
  return readlane63(v);
}
template <class T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, T(0), [](T a, T b) { return a + b; });
}
template <>
__device__ __forceinline__ uint32_t wave_sum<uint32_t>(uint32_t v) {
  return wave_sum_u32(v);
}
// identities of max and min for the lane types used
__device__ __forceinline__ int lowest_of(int) { return -2147483647 - 1; }
__device__ __forceinline__ uint32_t lowest_of(uint32_t) { return 0u; }
__device__ __forceinline__ float lowest_of(float) { return -__builtin_inff(); }
__device__ __forceinline__ int highest_of(int) { return 2147483647; }
__device__ __forceinline__ uint32_t highest_of(uint32_t) { return 0xffffffffu; }
__device__ __forceinline__ float highest_of(float) { return __builtin_inff(); }
__device__ __forceinline__ uint64_t lowest_of(uint64_t) { return 0ull; }
__device__ __forceinline__ uint64_t highest_of(uint64_t) { return ~0ull; }
// inclusive prefix sum over the 64 lanes: row shifts by 1, 2, 4, 8 (scan
// inside each row of 16), then the row broadcasts of lanes 15 and 31
template <class T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  v += dpp_t<0x111, 0xf, 0xf>(T(0), v);  // row_shr:1
  v += dpp_t<0x112, 0xf, 0xf>(T(0), v);  // row_shr:2
  v += dpp_t<0x114, 0xf, 0xf>(T(0), v);  // row_shr:4
  v += dpp_t<0x118, 0xf, 0xf>(T(0), v);  // row_shr:8
  v += dpp_t<0x142, 0xa, 0xf>(T(0), v);  // row_bcast:15
  v += dpp_t<0x143, 0xc, 0xf>(T(0), v);  // row_bcast:31
  return v;
}

// Wave 0 (all 64 lanes): the first i < n (n <= 64) with tab[0] + ... + tab[i] > u.
// Returns it (-1 if the total is <= u) and *before = tab[0] + ... + tab[i-1];
// the other waves get nothing.  One scan instead of a serial walk.
__device__ __forceinline__ int wave_first_above(const uint64_t* tab, int n, uint64_t u, uint64_t* before) {
  const int l = threadIdx.x & 63;
  const uint64_t v = l < n ? tab[l] : 0ull;
  const uint64_t inc = wave_incl_scan(v);
  const uint64_t hit = __ballot(l < n && inc > u);
  if (!hit) return -1;
  const int i = __builtin_ctzll(hit);
  const uint64_t exc = inc - v;
  *before = (uint64_t)__builtin_amdgcn_readlane((int)(uint32_t)exc, i) |
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(exc >> 32), i) << 32);
  return i;
}

// Scratch for block-wide collectives (must be __shared__).
struct BlockScratch {
  uint64_t w[NW + 1];
};

// Block reductions: every thread calls, every thread gets the result.  The
// per-wave slots of the scratch are written only before a collective's first
// barrier and the result slot only after it, so one collective may follow
// another without a barrier in between (nothing else writes the scratch).
template <class T, class OP>
__device__ __forceinline__ T block_reduce(T v, T id, OP op, BlockScratch& s) {
  v = wave_reduce(v, id, op);
  if (lane_id() == 0) reinterpret_cast<T*>(s.w)[wave_id()] = v;
  __syncthreads();
  if (threadIdx.x < 64) {
    T t = threadIdx.x < NW ? reinterpret_cast<T*>(s.w)[threadIdx.x] : id;
    t = wave_reduce(t, id, op);
    if (threadIdx.x == 0) reinterpret_cast<T*>(s.w)[NW] = t;
  }
  __syncthreads();
  return reinterpret_cast<T*>(s.w)[NW];
}
template <class T>
__device__ __forceinline__ T block_sum(T v, BlockScratch& s) {
  return block_reduce(v, T(0), [](T a, T b) { return a + b; }, s);
}
template <class T>
__device__ __forceinline__ T block_max(T v, BlockScratch& s) {
  return block_reduce(v, lowest_of(T()), [](T a, T b) { return b > a ? b : a; }, s);
}
template <class T>
__device__ __forceinline__ T block_min(T v, BlockScratch& s) {
  return block_reduce(v, highest_of(T()), [](T a, T b) { return b < a ? b : a; }, s);
}
// maxima of the two unsigned 16-bit halves, independently
__device__ __forceinline__ uint32_t block_max_u16x2(uint32_t v, BlockScratch& s) {
  typedef unsigned short h2 __attribute__((ext_vector_type(2)));
  return block_reduce(v, 0u, [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b)));
  }, s);
}
// Exclusive prefix sum over threads in threadIdx order; *total gets the sum.
template <class T>
__device__ __forceinline__ T block_excl_scan(T v, BlockScratch& s, T* total) {
  T inc = wave_incl_scan(v);
  if (lane_id() == 63) reinterpret_cast<T*>(s.w)[wave_id()] = inc;
  __syncthreads();
  if (threadIdx.x < 64) {
    T t = threadIdx.x < NW ? reinterpret_cast<T*>(s.w)[threadIdx.x] : T(0);
    T ti = wave_incl_scan(t);
    if (threadIdx.x < NW) reinterpret_cast<T*>(s.w)[threadIdx.x] = ti - t;
    if (threadIdx.x == NW - 1) reinterpret_cast<T*>(s.w)[NW] = ti;
  }
  __syncthreads();
  T r = reinterpret_cast<T*>(s.w)[wave_id()] + inc - v;
  if (total) *total = reinterpret_cast<T*>(s.w)[NW];
  return r;
}

// Streaming loads: marked non-temporal, for data read once (or read again
// only after a pass over far more bytes than the caches hold).  On this chip
// they also stream faster: a pass over 364 MB of logits reads at 4.4 TB/s
// with ordinary loads and at 6.5 TB/s with these.  Data that the next pass
// reads again (the weights between the floor and cand passes of the split
// rows) keeps ordinary loads: there the cached copy is worth more.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const nt_u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return uint4{t.x, t.y, t.z, t.w};
}
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint16_t ld_nt(const uint16_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ld_nt(const float* p) { return __builtin_nontemporal_load(p); }

// a value that is the same in every lane, moved to scalar registers
__device__ __forceinline__ double uniform_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return __longlong_as_double((long long)((hi << 32) | lo));
}

// ------------------------------------------------------------------- keys
// Order-preserving map of a non-NaN binary32 to uint32; -0 and +0 map to the
// same key (IEEE equality).  NaN never reaches it.
__device__ __forceinline__ uint32_t key32(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// Order-preserving, exact map of a remainder r in [0, 1) to uint64.  For
// r >= 2^-11 the key is 2^63 + r * 2^63 (an integer: such an r is a multiple
// of 2^-63), which spreads the usual remainders evenly over the top bits; a
// smaller r keeps its binary64 bit pattern, which is below 2^63.
__device__ __forceinline__ uint64_t rem_key(double r) {
  uint64_t b = (uint64_t)__double_as_longlong(r);
  uint32_t e = (uint32_t)(b >> 52);
  if (e >= 1012u) return (1ull << 63) | (((b & ((1ull << 52) - 1)) | (1ull << 52)) << (e - 1012u));
  return b;
}

// ------------------------------------------- correctly rounded exp, binary32
#include "exp_table.inc"

// RN32(exp(d)) for binary32 d <= 0 (or -inf), Tang's table method in
// binary64: d = (64 e + j) ln2/64 + r with |r| <= ln2/128, exp(d) =
// 2^e 2^(j/64) exp(r).  This is the accurate evaluation: a double-double
// table entry, a degree-7 polynomial (truncation < 2^-74), and the product
// kept as an unevaluated pair H + L (relative error about 2^-70), rounded to
// binary32 once, with the side of a midpoint within 2^-48 decided from H and
// L exactly.
__device__ __forceinline__ float cr_expf_accurate(float d) {
  if (!(d > -104.0f)) return 0.0f;  // exp(-104) < 2^-150 rounds to 0; also -inf
  if (d == 0.0f) return 1.0f;
  const double dd = (double)d;
  const double kf = __builtin_rint(dd * kExpInvL);
  const int k = (int)kf;
  const int j = k & 63;
  const int e = k >> 6;  // floor(k / 64)
  const double rhi = __builtin_fma(-kf, kExpCHi, dd);  // exact: k*C_HI is exact and close to d
  const double t = kf * kExpCLo;
  const double r1 = rhi - t;
  const double r2 = (rhi - r1) - t;  // r1 + r2 = rhi - t to ~2^-100
  double P = __builtin_fma(r1, kExpP7, kExpP6);
  P = __builtin_fma(r1, P, kExpP5);
  P = __builtin_fma(r1, P, kExpP4);
  P = __builtin_fma(r1, P, kExpP3);
  P = __builtin_fma(r1, P, kExpP2);
  const double s = __builtin_fma(r1 * r1, P, r2);  // exp(r) = 1 + r1 + s
  const double Th = kExpTabHi[j], Tl = kExpTabLo[j];
  const double ph = Th * r1;
  const double pl = __builtin_fma(Th, r1, -ph);
  const double H = Th + ph;
  const double e1 = ph - (H - Th);
  const double L = e1 + (pl + __builtin_fma(Th, s, Tl * ((1.0 + r1) + s)));
  const double tv = __builtin_ldexp(H + L, e);
  const float f = (float)tv;
  const double g = (double)f;
  if (g == tv) return f;
  // neighbour of f (>= 0) on tv's side: one unit in the last place up or down
  const uint32_t fb = __float_as_uint(f);
  const float nb = __uint_as_float(tv > g ? fb + 1u : (fb ? fb - 1u : 0u));
  const double mid = 0.5 * (g + (double)nb);
  if (__builtin_fabs(tv - mid) > 0x1p-48 * tv) return f;
  const double delta = (__builtin_ldexp(H, e) - mid) + __builtin_ldexp(L, e);
  const float up = f > nb ? f : nb, dn = f > nb ? nb : f;
  if (delta > 0.0) return up;
  if (delta < 0.0) return dn;
  return (__float_as_uint(up) & 1u) ? dn : up;  // exact tie: even significand
}

// Half-width, in units in the last place of a binary64 value, of the band
// around a binary32 rounding midpoint in which cr_expf's first evaluation
// does not decide the rounding (its error is below 400 such units).
constexpr uint32_t kExpBandUlps = 4096u;

// RN32(exp(d)) for binary32 d <= 0 (or -inf; never NaN).  A first
// evaluation, branch-free, of exp(max(d, -110)): k = RN(d 64/ln2) from the
// low word of d 64/ln2 + 1.5 2^52, the reduced argument r in two fused
// multiply-adds, a degree-4 Taylor polynomial for exp(r) - 1 (truncation
// below 2^-44.5 for |r| <= ln2/128), and tv = 2^e 2^(j/64) (1 + (exp(r) - 1))
// with a binary64 table entry: relative error below 2^-44.4, under 400 units
// in the last place of tv.  For a normal binary32 result the 29 low bits of
// tv's significand are those that binary32 rounding drops, and the rounding
// midpoint sits at 2^28 of them; unless tv lies within kExpBandUlps of it,
// the binary32 rounding of tv is that of exp(d).  Below d = -104.08 (k <
// -9610) exp(d) and tv are both below 2^-150.03, and tv rounds to 0 as
// exp(d) does.  The band (a few values in a million) and k in [-9610,
// -8001] (d in [-104.08, -86.64]: results near or below the binary32
// subnormal threshold 2^-126, or near 2^-150) take the accurate evaluation;
// a wave with no such lane skips it.  Checked against an independent
// evaluation for every binary32 d in [-104, 0].
// tab: the 64 entries kExpTabHi, from global memory or from an LDS copy
// (exp_table_to_lds): in LDS the per-lane lookup stays off the vector
// memory counter, so a loop's streamed loads need not drain to serve it.
__device__ __forceinline__ float cr_expf(float d, const double* tab = kExpTabHi) {
  const double dd = (double)__builtin_fmaxf(d, -110.0f);
  const double kb = __builtin_fma(dd, kExpInvL, 0x1.8p52);  // 1.5 2^52 + k
  const int k = (int)(uint32_t)__double_as_longlong(kb);
  const double kf = kb - 0x1.8p52;
  double r = __builtin_fma(-kf, kExpCHi, dd);
  r = __builtin_fma(-kf, kExpCLo, r);
  double Q = __builtin_fma(r, kExpP4, kExpP3);
  Q = __builtin_fma(r, Q, kExpP2);
  const double q = __builtin_fma(r * r, Q, r);  // exp(r) - 1
  const double T = tab[k & 63];
  const double tv = __builtin_ldexp(__builtin_fma(T, q, T), k >> 6);
  const float f = (float)tv;
  const uint32_t low = (uint32_t)__double_as_longlong(tv) & 0x1fffffffu;
  const bool band = low - (0x10000000u - kExpBandUlps) <= 2u * kExpBandUlps;
  const bool tiny = (uint32_t)(k + 9610) < 1610u;  // k in [-9610, -8001]
  if (__builtin_expect(band || tiny, 0)) return cr_expf_accurate(d);
  return f;
}

// copies cr_expf's table into s[64] (the caller's barrier publishes it)
__device__ __forceinline__ void exp_table_to_lds(double* s) {
  for (int i = (int)threadIdx.x; i < 64; i += (int)blockDim.x) s[i] = kExpTabHi[i];
}

// ------------------------------------------------- exact weight accumulator
// Sum of binary32 weights w in [0, 1], exactly.  Weights >= 2^-47 go to a
// 128-bit fixed-point word with LSB 2^-70 (each is an integer there; 2^20 of
// them stay below 2^90), smaller ones to a 128-bit word with LSB 2^-149
// (each below 2^102, 2^20 of them below 2^122).
struct Acc {
  uint64_t mlo, mhi, tlo, thi;
};
__device__ __forceinline__ void acc_zero(Acc& a) { a.mlo = a.mhi = a.tlo = a.thi = 0; }
__device__ __forceinline__ void add128(uint64_t& lo, uint64_t& hi, uint64_t alo, uint64_t ahi) {
  lo += alo;
  hi += ahi + (lo < alo ? 1u : 0u);
}
// adds n * w (n < 2^21) where wb are the bits of w in [0, 1]
__device__ __forceinline__ void acc_add(Acc& a, uint32_t wb, uint32_t n = 1) {
  wb &= 0x7fffffffu;  // -0.0 is 0
  if (wb == 0u || n == 0u) return;
  const uint32_t E = wb >> 23;
  const uint64_t mant = (uint64_t)((wb & 0x7fffffu) | (E ? 0x800000u : 0u)) * n;  // < 2^45
  if (E >= 80u) {
    const uint32_t sh = E - 80u;  // 0..47: mant * 2^(E-150) in units of 2^-70
    const uint64_t lo = mant << sh;
    const uint64_t hi = sh ? (mant >> (64 - sh)) : 0ull;
    add128(a.mlo, a.mhi, lo, hi);
  } else {
    const uint32_t sh = E ? E - 1u : 0u;  // 0..78: in units of 2^-149
    const uint64_t lo = sh < 64 ? (mant << sh) : 0ull;
    const uint64_t hi = sh == 0 ? 0ull : (sh < 64 ? (mant >> (64 - sh)) : (mant << (sh - 64)));
    add128(a.tlo, a.thi, lo, hi);
  }
}
// A faster tier for many weights, without branches for the usual ones:
// weights of at least 2^-24 (exponent field E >= 103) are integers in units
// of 2^-47 below 2^48, added in the 64-bit word hi; weights in [2^-47,
// 2^-24) (80 <= E < 103) are integers in units of 2^-70 below 2^47, added
// in the 64-bit word lo.  Each word takes 2^16 additions.  Smaller weights
// go to the accumulator.  acc_fold adds both words to the accumulator's
// main word (units 2^-70: hi 2^23 + lo).
struct AccQ {
  uint64_t hi, lo;
};
__device__ __forceinline__ void accq_zero(AccQ& q) { q.hi = q.lo = 0; }
__device__ __forceinline__ void acc_add_q(Acc& a, AccQ& q, uint32_t wb) {
  wb &= 0x7fffffffu;
  const uint32_t E = wb >> 23;
  const uint64_t mant = (wb & 0x7fffffu) | 0x800000u;
  const bool big = E >= 103u;
  const uint64_t v = mant << ((big ? E - 103u : E - 80u) & 63u);
  q.hi += big ? v : 0ull;
  q.lo += !big && E >= 80u ? v : 0ull;
  if (E < 80u && wb) acc_add(a, wb);
}
// The cheapest tier, for streams of weights: binary64 words that stay exact
// for a bounded number of additions.  Weights of at least 2^-24 are
// multiples of 2^-47: their sum is exact in binary64 below 2^6, so for up to
// 63 weights (each at most 1).  Weights in [2^-47, 2^-24) are multiples of
// 2^-70: exact below 2^-17, so for up to 127 of them.  Each weight goes to
// its word by a fused multiply-add with 1 or 0 (no branch); accd_flush moves
// both words, as integers in units of 2^-47 and 2^-70, into the AccQ words,
// and must follow every kAccDRun additions.  Smaller weights go to the
// accumulator.
constexpr int kAccDRun = 32;
struct AccD {
  double big, mid;
};
__device__ __forceinline__ void accd_zero(AccD& d) { d.big = d.mid = 0.0; }
__device__ __forceinline__ void accd_add(Acc& a, AccD& d, uint32_t wb) {  // wb: the bits of a weight in [0, 1]
  if (wb - 1u < (80u << 23) - 1u) {  // 0 < w < 2^-47: rare
    acc_add(a, wb);
    return;
  }
  const double w = (double)__uint_as_float(wb);
  const bool big = wb >= (103u << 23);
  d.big = __builtin_fma(w, big ? 1.0 : 0.0, d.big);
  d.mid = __builtin_fma(w, big ? 0.0 : 1.0, d.mid);
}
__device__ __forceinline__ void accd_flush(AccQ& q, AccD& d) {
  q.hi += (uint64_t)(d.big * 0x1p47);  // integers below 2^53
  q.lo += (uint64_t)(d.mid * 0x1p70);
  accd_zero(d);
}
__device__ __forceinline__ void acc_fold(Acc& a, const AccQ& q) {
  add128(a.mlo, a.mhi, q.hi << 23, q.hi >> 41);
  add128(a.mlo, a.mhi, q.lo, 0ull);
}
struct AccScratch {
  Acc w[NW];
  double s64;
};
// RN64 of the accumulated sum (round to nearest, ties to even).
__device__ inline double acc_rn64(const Acc& a) {
  // S in units of 2^-149 as a 192-bit integer L2:L1:L0 (the main word is in
  // units of 2^-70 = 2^79 * 2^-149)
  uint64_t L0 = a.tlo, L1 = a.thi, L2 = 0;
  const uint64_t add1 = a.mlo << 15;
  L1 += add1;
  L2 += (L1 < add1 ? 1u : 0u) + (a.mlo >> 49) + (a.mhi << 15);
  int p;  // index of the highest set bit
  if (L2) p = 128 + 63 - __builtin_clzll(L2);
  else if (L1) p = 64 + 63 - __builtin_clzll(L1);
  else if (L0) p = 63 - __builtin_clzll(L0);
  else return 0.0;
  auto limb = [&](int q) -> uint64_t { return q == 0 ? L0 : q == 1 ? L1 : q == 2 ? L2 : 0ull; };
  auto bit_range = [&](int lo) -> uint64_t {  // 64 bits starting at bit lo (lo >= 0)
    const int q = lo >> 6, r = lo & 63;
    uint64_t v = limb(q) >> r;
    if (r) v |= limb(q + 1) << (64 - r);
    return v;
  };
  if (p <= 52) return __builtin_ldexp((double)L0, -149);  // exact
  const int sh = p - 52;
  uint64_t mant = bit_range(sh) & ((1ull << 53) - 1);
  const uint64_t rb = (bit_range(sh - 1) & 1ull);
  bool sticky = false;
  if (sh - 1 > 0) {
    const int nb = sh - 1;  // bits [0, nb) below the round bit
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int take = nb - q * 64;
      if (take > 0) {
        const uint64_t m = take >= 64 ? ~0ull : ((1ull << take) - 1);
        if (limb(q) & m) sticky = true;
      }
    }
  }
  if (rb && (sticky || (mant & 1ull))) mant += 1;
  return __builtin_ldexp((double)mant, sh - 149);  // mant may be 2^53: still exact
}
// One step of a wave-wide sum of 128-bit integers held as four 32-bit limbs
// (lowest first): every enabled lane adds the limbs of the lane that the DPP
// control names, the carry running through VCC; rows outside the row mask
// keep their value.  The leading s_nop covers the two wait states a DPP read
// needs after a VALU write of the same register.
#define DSPARK_ADD128_DPP(L0, L1, L2, L3, DPP)                              \
  asm volatile("s_nop 1\n\t"                                               \
               "v_add_co_u32_dpp %0, vcc, %0, %0 " DPP "\n\t"              \
               "v_addc_co_u32_dpp %1, vcc, %1, %1, vcc " DPP "\n\t"        \
               "v_addc_co_u32_dpp %2, vcc, %2, %2, vcc " DPP "\n\t"        \
               "v_addc_co_u32_dpp %3, vcc, %3, %3, vcc " DPP                \
               : "+v"(L0), "+v"(L1), "+v"(L2), "+v"(L3)                     \
               :                                                            \
               : "vcc")
struct Limbs4 {
  uint32_t l0, l1, l2, l3;
};
__device__ __forceinline__ Limbs4 limbs_of(uint64_t lo, uint64_t hi) {
  return Limbs4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
__device__ __forceinline__ uint64_t limbs_lo(const Limbs4& x) { return ((uint64_t)x.l1 << 32) | x.l0; }
__device__ __forceinline__ uint64_t limbs_hi(const Limbs4& x) { return ((uint64_t)x.l3 << 32) | x.l2; }
// the sum of the word over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ void add128_rows(Limbs4& x) {
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf");
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf");
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "row_half_mirror row_mask:0xf bank_mask:0xf");
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "row_mirror row_mask:0xf bank_mask:0xf");
}
// the sum of the word over the wave, in lane 63
__device__ __forceinline__ void add128_wave(Limbs4& x) {
  add128_rows(x);
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "row_bcast:15 row_mask:0xa bank_mask:0xf");
  DSPARK_ADD128_DPP(x.l0, x.l1, x.l2, x.l3, "row_bcast:31 row_mask:0xc bank_mask:0xf");
}
#undef DSPARK_ADD128_DPP

// Block-wide exact sum; every thread gets RN64(S).  The small-weight word is
// summed only where some lane holds a part of it.
__device__ inline double block_acc_rn64(Acc a, AccScratch& s) {
  Limbs4 mw = limbs_of(a.mlo, a.mhi);
  add128_wave(mw);
  Limbs4 tw = limbs_of(a.tlo, a.thi);
  const bool tiny = __ballot((a.tlo | a.thi) != 0ull) != 0ull;  // uniform over the wave
  if (tiny) add128_wave(tw);
  if (lane_id() == 63) {
    Acc w;
    w.mlo = limbs_lo(mw);
    w.mhi = limbs_hi(mw);
    w.tlo = tiny ? limbs_lo(tw) : 0ull;
    w.thi = tiny ? limbs_hi(tw) : 0ull;
    s.w[wave_id()] = w;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0 merges the NW wave sums within its first row
    Acc t;
    if (threadIdx.x < NW) t = s.w[threadIdx.x];
    else acc_zero(t);
    Limbs4 m = limbs_of(t.mlo, t.mhi);
    add128_rows(m);
    const bool ttiny = __ballot((t.tlo | t.thi) != 0ull) != 0ull;
    Limbs4 tt = limbs_of(t.tlo, t.thi);
    if (ttiny) add128_rows(tt);
    if (threadIdx.x == 0) {
      const uint64_t mlo = limbs_lo(m), mhi = limbs_hi(m);
      double r;
      if (!ttiny && mhi < (1ull << 26)) {
        // S = M 2^-70 with M < 2^90: M = H 2^38 + L with H < 2^52 and
        // L < 2^38, both exact in binary64, so one addition rounds S once
        const uint64_t H = (mhi << 26) | (mlo >> 38), L = mlo & ((1ull << 38) - 1);
        r = __builtin_ldexp((double)H, -32) + __builtin_ldexp((double)L, -70);
      } else {
        Acc u;
        u.mlo = mlo;
        u.mhi = mhi;
        u.tlo = ttiny ? limbs_lo(tt) : 0ull;
        u.thi = ttiny ? limbs_hi(tt) : 0ull;
        r = acc_rn64(u);
      }
      s.s64 = r;
    }
  }
  __syncthreads();
  return s.s64;  // (written again only after the next call's first barrier)
}

}  // namespace dspark
