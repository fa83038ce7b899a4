// Exact draws from the target distribution p of a logit row, and from the
// residual max(p - q, 0) against a draft row's dyadic q.
//
// "PP1 q transport and scheduling design", section "Distribution contract
// and precision": the full target p is the distribution at T = 1, rounding
// to dyadic counts changes the proposal only, and ratio tests and
// full-vocabulary residual sampling use that p and the defined q; section
// "Sparse support and vocabulary-sharded TP2 follow-up": max(p - q, 0) is
// formed for every token, including tokens outside a sparse q's support.
//
// p_v = A_v / A with the exact integers A_v = w_v 2^149 of the row's weights
// w_v = RN32(exp(RN32(x_v - m))) (the weights of the draft's q), and
// A = sum_v A_v.  A draw u (uniform 64-bit) picks the first token v, in
// ascending id order, whose inclusive cumulative weight C_v satisfies
// C_v > T = floor(u W / 2^64), W the total weight.  Residual weights are
// max(2^24 A_v - c_v A, 0) for q counts c_v.  Everything is integer: the
// per-element weights are summed exactly (a 64-bit word for weights of at
// least 2^-24, the 128-bit accumulator below), wave and row totals are
// 256-bit integers.
//
// Layout: wave w owns a contiguous id range, cut into chunks of 64 lanes x E
// consecutive ids; lane l of chunk c holds ids base + c * 64E + l E + e.  A
// pass accumulates per lane over the wave's chunks and reduces once per
// wave; the draw finds the wave from the 16 wave totals, then that wave alone
// walks its chunks (one wave reduction each) to the crossing chunk, scans its
// lanes and walks the crossing lane's E elements.
//
// Two sources: bf16 rows of up to 131072 ids held in registers (16 chunks of
// 512 ids per wave, one HBM read of the row), and rows streamed from memory
// (float32 rows, or longer bf16 rows), reloaded by each pass.
#pragma once
#include "fast_q.hpp"

namespace dspark {

// ------------------------------------------------------------ 256-bit ints
struct U256 {
  uint64_t w[4];
};
__device__ __forceinline__ U256 u256_zero() { return U256{{0ull, 0ull, 0ull, 0ull}}; }
__device__ __forceinline__ bool u256_is_zero(const U256& a) { return (a.w[0] | a.w[1] | a.w[2] | a.w[3]) == 0ull; }
__device__ __forceinline__ U256 u256_add(const U256& a, const U256& b) {
  U256 r;
  uint64_t c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t s = a.w[i] + b.w[i];
    const uint64_t c1 = s < a.w[i] ? 1ull : 0ull;
    r.w[i] = s + c;
    c = c1 | (r.w[i] < s ? 1ull : 0ull);
  }
  return r;
}
// a - b for a >= b
__device__ __forceinline__ U256 u256_sub(const U256& a, const U256& b) {
  U256 r;
  uint64_t br = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t d = a.w[i] - b.w[i];
    const uint64_t b1 = a.w[i] < b.w[i] ? 1ull : 0ull;
    r.w[i] = d - br;
    br = b1 | (d < br ? 1ull : 0ull);
  }
  return r;
}
__device__ __forceinline__ bool u256_lt(const U256& a, const U256& b) {
#pragma unroll
  for (int i = 3; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i];
  return false;
}
// a * 2^s, 0 < s < 64, for a < 2^(256 - s)
__device__ __forceinline__ U256 u256_shl(const U256& a, int s) {
  return U256{{a.w[0] << s, (a.w[1] << s) | (a.w[0] >> (64 - s)), (a.w[2] << s) | (a.w[1] >> (64 - s)),
               (a.w[3] << s) | (a.w[2] >> (64 - s))}};
}
// the five 64-bit limbs of a * b
__device__ __forceinline__ void u256_mul64_full(const U256& a, uint64_t b, uint64_t (&p)[5]) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t lo = a.w[i] * b, hi = __umul64hi(a.w[i], b);
    const uint64_t s = lo + carry;
    p[i] = s;
    carry = hi + (s < lo ? 1ull : 0ull);
  }
  p[4] = carry;
}
// a * b, for a product below 2^256
__device__ __forceinline__ U256 u256_mul64(const U256& a, uint64_t b) {
  uint64_t p[5];
  u256_mul64_full(a, b, p);
  return U256{{p[0], p[1], p[2], p[3]}};
}
// floor(a * b / 2^64)
__device__ __forceinline__ U256 u256_mulhi64(const U256& a, uint64_t b) {
  uint64_t p[5];
  u256_mul64_full(a, b, p);
  return U256{{p[1], p[2], p[3], p[4]}};
}
// m * 2^s for m < 2^25 and 0 <= s < 200
__device__ __forceinline__ U256 u256_shifted(uint64_t m, int s) {
  U256 r = u256_zero();
  const int q = s >> 6, o = s & 63;
  const uint64_t lo = m << o, hi = o ? (m >> (64 - o)) : 0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i == q) r.w[i] = lo;
    if (i == q + 1) r.w[i] = hi;
  }
  return r;
}
// A_v = w * 2^149 for the bits of a binary32 weight w in [0, 1]
__device__ __forceinline__ U256 u256_of_weight(uint32_t wb) {
  wb &= 0x7fffffffu;
  const uint32_t E = wb >> 23;
  const uint64_t mant = (wb & 0x7fffffu) | (E ? 0x800000u : 0u);
  return u256_shifted(mant, E ? (int)E - 1 : 0);
}
// the accumulated sum, in units of 2^-149 (the main word is in units of
// 2^-70 = 2^79 units of 2^-149)
__device__ __forceinline__ U256 u256_of_acc(const Acc& a) {
  U256 m = U256{{0ull, a.mlo << 15, (a.mlo >> 49) | (a.mhi << 15), a.mhi >> 49}};  // main << 79
  return u256_add(m, U256{{a.tlo, a.thi, 0ull, 0ull}});
}
// Exact sums of the draws' weights.  Weights of at least 2^-24 (binary32
// exponent field E >= 103; nearly every weight of a row) are integers in
// units of 2^-47 below 2^48, added in one 64-bit word: a lane adds at most
// 2^10 of them and a wave 2^16 (V <= 2^20), so neither a lane's nor a wave's
// word overflows.  Smaller weights go to the 128-bit accumulator.
struct DAcc {
  uint64_t q;
  Acc a;
};
__device__ __forceinline__ void dacc_zero(DAcc& s) {
  s.q = 0ull;
  acc_zero(s.a);
}
__device__ __forceinline__ void dacc_add(DAcc& s, uint32_t wb) {
  wb &= 0x7fffffffu;
  const uint32_t E = wb >> 23;
  if (E >= 103u) s.q += (uint64_t)((wb & 0x7fffffu) | 0x800000u) << (E - 103u);
  else if (wb) acc_add(s.a, wb);
}
// the sum in units of 2^-149
__device__ __forceinline__ U256 u256_of_dacc(const DAcc& s) {
  const U256 q = U256{{0ull, s.q << 38, s.q >> 26, 0ull}};  // q * 2^102
  return u256_add(q, u256_of_acc(s.a));
}
// a * 2^-149 to about 2^-60 relative (only used to pre-sort comparisons)
__device__ __forceinline__ double u256_approx_scaled(const U256& a) {
  double r = 0.0;
#pragma unroll
  for (int i = 3; i >= 0; --i) r = r * 0x1p64 + (double)a.w[i];
  return __builtin_ldexp(r, -149);
}

// inclusive prefix sum over the 64 lanes (all lanes active)
template <int CTRL, int RM, int BM>
__device__ __forceinline__ void u256_scan_step(U256& v) {
  U256 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.w[i] = dpp_t<CTRL, RM, BM>((uint64_t)0, v.w[i]);
  v = u256_add(v, t);
}
__device__ __forceinline__ U256 u256_wave_incl_scan(U256 v) {
  u256_scan_step<0x111, 0xf, 0xf>(v);  // row_shr:1
  u256_scan_step<0x112, 0xf, 0xf>(v);  // row_shr:2
  u256_scan_step<0x114, 0xf, 0xf>(v);  // row_shr:4
  u256_scan_step<0x118, 0xf, 0xf>(v);  // row_shr:8
  u256_scan_step<0x142, 0xa, 0xf>(v);  // row_bcast:15
  u256_scan_step<0x143, 0xc, 0xf>(v);  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32);
}
__device__ __forceinline__ U256 u256_readlane(const U256& v, int l) {
  return U256{{readlane_u64(v.w[0], l), readlane_u64(v.w[1], l), readlane_u64(v.w[2], l), readlane_u64(v.w[3], l)}};
}
// wave-uniform copy of a value every lane holds (scalar registers)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32);
}
__device__ __forceinline__ U256 uniform_u256(const U256& v) {
  return U256{{uniform_u64(v.w[0]), uniform_u64(v.w[1]), uniform_u64(v.w[2]), uniform_u64(v.w[3])}};
}
// wave totals of an exact draw sum and a 64-bit count, in every lane (the
// 128-bit words only when some lane holds a small weight)
__device__ __forceinline__ void wave_total(const DAcc& s, uint64_t s2, DAcc* ts, uint64_t* ts2) {
  ts->q = wave_sum<uint64_t>(s.q);
  const Acc& a = s.a;
  const bool main = __ballot((a.mlo | a.mhi) != 0ull) != 0ull;
  const bool tiny = __ballot((a.tlo | a.thi) != 0ull) != 0ull;
  acc_zero(ts->a);
  if (main) {
    Limbs4 mw = limbs_of(a.mlo, a.mhi);
    add128_wave(mw);
    ts->a.mlo = readlane_u64(limbs_lo(mw), 63);
    ts->a.mhi = readlane_u64(limbs_hi(mw), 63);
  }
  if (tiny) {
    Limbs4 tw = limbs_of(a.tlo, a.thi);
    add128_wave(tw);
    ts->a.tlo = readlane_u64(limbs_lo(tw), 63);
    ts->a.thi = readlane_u64(limbs_hi(tw), 63);
  }
  *ts2 = __ballot(s2 != 0ull) ? wave_sum<uint64_t>(s2) : 0ull;
}

// ---------------------------------------------------------------- context
enum DrawMode { kDrawPlain = 0, kDrawResidual = 1 };

// What the weight of an element depends on.  For a bf16 row whose maximum
// admits the value table of fast_q.hpp, the weights of every table entry are
// computed once (wtab) and looked up per element; otherwise each element
// takes the correctly rounded exponential itself.
struct DrawCtx {
  float m;
  FMap f;
  bool table;
  // residual mode: the plain total A, its rough binary64 value, the q row
  U256 A;
  double s64;
  const uint32_t* dense;  // counts row (dense q) or nullptr
  int sp_len;             // sparse q: entries held in the shared ids / counts
  int V;
};

struct DrawShared : SmemBase {
  float wtab[kNBFD];                  // weight of each table entry; 0 past NB
  int32_t sid[DSPARK_K_MAX];          // sparse q ids (ascending) and counts
  uint32_t scnt[DSPARK_K_MAX];
  uint32_t gbits[DSPARK_V_MAX / 256];  // one bit per 8 ids: some sparse id in the group
  U256 wtot[NW];
  U256 total;
  U256 rest;     // the draw's threshold, less everything before the crossing wave (then chunk)
  int wstar;
  int token;
  int ichunk;                            // the crossing chunk of a streamed row
  U256 ctot[DSPARK_V_MAX / (64 * NW * 4)];  // chunk totals of the crossing wave's range (streamed rows)
};

// Builds the weight table of a bf16 row (all threads; ends with a barrier).
__device__ __forceinline__ void draw_table(DrawCtx& c, DrawShared& sh) {
  for (int b = (int)threadIdx.x; b < kNBFD; b += BS)
    sh.wtab[b] = b < c.f.NB ? cr_expf(bf16_to_f32(fmap_raw(b, c.f)) - c.m) : 0.0f;
  __syncthreads();
}

// Loads a sparse q row into the shared arrays and marks its id groups (all
// threads; ends with a barrier).
__device__ __forceinline__ void draw_sparse_q(const int32_t* ids, const uint32_t* cnt, int len, DrawShared& sh) {
  for (int g = (int)threadIdx.x; g < DSPARK_V_MAX / 256; g += BS) sh.gbits[g] = 0u;
  __syncthreads();
  for (int j = (int)threadIdx.x; j < len; j += BS) {
    const int id = ids[j];
    sh.sid[j] = id;
    sh.scnt[j] = cnt[j];
    if (id >= 0 && id < DSPARK_V_MAX) atomicOr(&sh.gbits[id >> 8], 1u << ((id >> 3) & 31));
  }
  __syncthreads();
}

// q's count at id v (v < V)
__device__ __forceinline__ uint32_t draw_count(const DrawCtx& c, const DrawShared& sh, int v) {
  if (c.dense) return c.dense[v];
  if (c.sp_len <= 0 || !((sh.gbits[v >> 8] >> ((v >> 3) & 31)) & 1u)) return 0u;
  int lo = 0, hi = c.sp_len;  // first entry with id >= v
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sh.sid[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo < c.sp_len && sh.sid[lo] == v ? sh.scnt[lo] : 0u;
}

// Residual sign of one element, 2^24 A_v > c A (w > 0): decided in binary64
// unless the two sides are within 2^-40 of each other (relative), then in
// 256-bit integers.
__device__ __forceinline__ bool resid_positive(uint32_t wb, uint32_t cnt, const DrawCtx& c) {
  if ((wb & 0x7fffffffu) == 0u) return false;
  if (cnt == 0u) return true;
  const double lhs = (double)__uint_as_float(wb) * 16777216.0;
  const double rhs = (double)cnt * c.s64;
  const double d = lhs - rhs;
  if (__builtin_fabs(d) > 0x1p-40 * rhs) return d > 0.0;
  return u256_lt(u256_mul64(c.A, cnt), u256_shl(u256_of_weight(wb), 24));
}
// exact weight of one element in the mode's units
template <int mode>
__device__ __forceinline__ U256 elem_weight(uint32_t wb, uint32_t cnt, const DrawCtx& c) {
  if (mode == kDrawPlain) return u256_of_weight(wb);
  if (!resid_positive(wb, cnt, c)) return u256_zero();
  return u256_sub(u256_shl(u256_of_weight(wb), 24), u256_mul64(c.A, cnt));
}
// the exact total of a group from its accumulated weights and counts
template <int mode>
__device__ __forceinline__ U256 group_weight(const DAcc& s1, uint64_t s2, const DrawCtx& c) {
  const U256 a = u256_of_dacc(s1);
  if (mode == kDrawPlain) return a;
  return u256_sub(u256_shl(a, 24), u256_mul64(c.A, s2));
}
// adds one element (weight bits wb, id v) to a lane's sums
template <int mode>
__device__ __forceinline__ void draw_add(uint32_t wb, int v, const DrawCtx& c, const DrawShared& sh, DAcc& s1,
                                         uint64_t& s2) {
  if (mode == kDrawPlain) {
    dacc_add(s1, wb);
    return;
  }
  if ((wb & 0x7fffffffu) == 0u) return;
  const uint32_t cnt = draw_count(c, sh, v);
  if (resid_positive(wb, cnt, c)) {
    dacc_add(s1, wb);
    s2 += cnt;
  }
}

// weight bits of a bf16 element (raw bits b) from the value table
__device__ __forceinline__ uint32_t bf16_weight_table(uint32_t b, const DrawCtx& c, const DrawShared& sh) {
  const int bin = fmap_bin(b, c.f);
  return bin >= 0 && bin < c.f.NB ? __float_as_uint(sh.wtab[bin]) : 0u;
}
// ... from the table when it applies, else from the exponential
__device__ __forceinline__ uint32_t bf16_weight_bits(uint32_t b, const DrawCtx& c, const DrawShared& sh) {
  if (c.table) return bf16_weight_table(b, c, sh);
  return __float_as_uint(cr_expf(bf16_to_f32(b) - c.m));
}

// ------------------------------------------------------------- sources
// bf16 rows in registers: wave w holds ids [8192 w, 8192 (w + 1)); chunk i
// (0..15) of lane l holds the 8 ids 8192 w + 512 i + 8 l + e.
__device__ __forceinline__ int wres_base(int i) { return wave_id() * 8192 + i * 512 + lane_id() * 8; }

__device__ __forceinline__ void wres_load(Res& R, const uint16_t* p, int V) {
  const int nfull = V >> 3;
  const u32x4 pad = {kNegInf2, kNegInf2, kNegInf2, kNegInf2};
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, V * 2, 0x00020000);
  const int toff = wave_id() * 16384 + lane_id() * 16;
#pragma unroll
  for (int i = 0; i < NI; ++i) store_vec(R, i, __builtin_amdgcn_raw_buffer_load_b128(rs, toff, i * 1024, 2));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wres_base(i) >> 3;  // this lane's vector, in units of 8 ids
    if (q >= nfull) store_vec(R, i, pad);
  }
  if (V & 7) {
    // the one partial vector: its owner patches it from 2-byte loads (picked
    // by selects, so that the row stays in registers)
    const int it = (nfull >> 6) & 15;
    const bool owner = wave_id() == (nfull >> 10) && lane_id() == (nfull & 63);
    u32x4 part = pad;
    if (owner) {
      uint32_t h[8];
#pragma unroll
      for (int l = 0; l < 8; ++l) h[l] = nfull * 8 + l < V ? (uint32_t)p[nfull * 8 + l] : 0xff80u;
      part = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool sel = owner && i == it;
      R.w[i][0] = sel ? part.x : R.w[i][0];
      R.w[i][1] = sel ? part.y : R.w[i][1];
      R.w[i][2] = sel ? part.z : R.w[i][2];
      R.w[i][3] = sel ? part.w : R.w[i][3];
    }
  }
}

// this lane's plain sum over chunk v of a resident row, weights from the
// value table
__device__ __forceinline__ void wres_chunk(u32x4 v, const DrawCtx& c, const DrawShared& sh, DAcc& s1) {
#pragma unroll
  for (int e = 0; e < 8; ++e) dacc_add(s1, bf16_weight_table(elem(v, e), c, sh));
}

// streamed rows: wave w holds chunks [cpw w, cpw (w + 1)) of 64 vectors
template <int DT>
struct StreamSrc {
  Row<DT> row;
  int cpw;
  static constexpr int E = Row<DT>::EPV;
  __device__ int vec(int ch) const { return (wave_id() * cpw + ch) * 64 + lane_id(); }
};
// One chunk of a lane: its E logits (bf16: the raw patterns, two per word;
// past V: -inf) and, for residual sums over a dense q, their E counts, all
// loaded before any is used (counts past V read 0).
template <int DT>
struct ChunkData {
  static constexpr int E = StreamSrc<DT>::E;
  static constexpr int NW_ = DT == DSPARK_BF16 ? E / 2 : E;
  uint32_t w[NW_];
  uint32_t cnt[E];
  // weight-relevant bits of element e: the bf16 pattern, or the binary32 bits
  __device__ __forceinline__ uint32_t bits(int e) const {
    if constexpr (DT == DSPARK_BF16) return (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
    else return w[e];
  }
};
template <int DT>
__device__ __forceinline__ void chunk_load_values(const Row<DT>& row, int q, ChunkData<DT>& d) {
  constexpr int E = StreamSrc<DT>::E;
  const int base = q * E;
  const int nv = row.V - base < E ? row.V - base : E;
  if (nv == E) {
    const uint4 u = ld_nt(reinterpret_cast<const uint4*>(row.p) + q);
    const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < ChunkData<DT>::NW_; ++i) d.w[i] = v[i];
  } else if constexpr (DT == DSPARK_BF16) {
    const uint16_t* s = static_cast<const uint16_t*>(row.p);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const uint32_t lo = 2 * i < nv ? (uint32_t)s[base + 2 * i] : 0xff80u;
      const uint32_t hi = 2 * i + 1 < nv ? (uint32_t)s[base + 2 * i + 1] : 0xff80u;
      d.w[i] = lo | (hi << 16);
    }
  } else {
    const uint32_t* s = static_cast<const uint32_t*>(row.p);
#pragma unroll
    for (int i = 0; i < E; ++i) d.w[i] = i < nv ? s[base + i] : 0xff800000u;
  }
}
template <int mode, int DT>
__device__ __forceinline__ void stream_load_vec(const StreamSrc<DT>& s, int q, const DrawCtx& c,
                                                __amdgpu_buffer_rsrc_t crs, bool c16, ChunkData<DT>& d) {
  constexpr int E = StreamSrc<DT>::E;
  chunk_load_values<DT>(s.row, q, d);
  if (mode != kDrawPlain && c.dense) {
    if (c16) {  // a 16-byte aligned count row: E / 4 vector loads
#pragma unroll
      for (int h = 0; h < E / 4; ++h) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(crs, (q * E + 4 * h) * 4, 0, 0);
        d.cnt[4 * h] = v.x;
        d.cnt[4 * h + 1] = v.y;
        d.cnt[4 * h + 2] = v.z;
        d.cnt[4 * h + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) d.cnt[e] = __builtin_amdgcn_raw_buffer_load_b32(crs, (q * E + e) * 4, 0, 0);
    }
  }
}
template <int mode, int DT>
__device__ __forceinline__ void stream_load(const StreamSrc<DT>& s, int ch, const DrawCtx& c,
                                            __amdgpu_buffer_rsrc_t crs, bool c16, ChunkData<DT>& d) {
  stream_load_vec<mode, DT>(s, s.vec(ch), c, crs, c16, d);
}
// buffer over a dense q row (reads past V give 0)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t count_rsrc(const DrawCtx& c) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(c.dense), (short)0, c.dense ? c.V * 4 : 0,
                                           0x00020000);
}
template <int DT>
__device__ __forceinline__ uint32_t chunk_weight_bits(uint32_t b, const DrawCtx& c, const DrawShared& sh) {
  return DT == DSPARK_BF16 ? bf16_weight_bits(b, c, sh)
                            : __float_as_uint(cr_expf(__uint_as_float(b) - c.m, sh.etab));
}
template <int mode, int DT>
__device__ __forceinline__ void stream_add(const ChunkData<DT>& d, int q, const DrawCtx& c, const DrawShared& sh,
                                           DAcc& s1, uint64_t& s2) {
  constexpr int E = StreamSrc<DT>::E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t wb = chunk_weight_bits<DT>(d.bits(e), c, sh);
    if (mode == kDrawPlain) {
      dacc_add(s1, wb);
    } else if ((wb & 0x7fffffffu) != 0u) {
      const uint32_t cnt = c.dense ? d.cnt[e] : draw_count(c, sh, q * E + e);
      if (resid_positive(wb, cnt, c)) {
        dacc_add(s1, wb);
        s2 += cnt;
      }
    }
  }
}
// this lane's sums over every chunk of its wave, DrawPF<mode>::n chunks' loads in
// flight together (fewer for residual sums, whose chunks carry counts)
template <int mode>
struct DrawPF {
  static constexpr int n = mode == kDrawPlain ? 4 : 2;
};
template <int mode, int DT>
__device__ __forceinline__ void stream_sums(const StreamSrc<DT>& s, const DrawCtx& c, const DrawShared& sh, DAcc& s1,
                                            uint64_t& s2) {
  const __amdgpu_buffer_rsrc_t crs = count_rsrc(c);
  const bool c16 = (reinterpret_cast<uintptr_t>(c.dense) & 15u) == 0u;
  constexpr int PF = DrawPF<mode>::n;
  for (int ch0 = 0; ch0 < s.cpw; ch0 += PF) {
    ChunkData<DT> d[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (ch0 + k < s.cpw) stream_load<mode, DT>(s, ch0 + k, c, crs, c16, d[k]);
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (ch0 + k < s.cpw) stream_add<mode, DT>(d[k], s.vec(ch0 + k), c, sh, s1, s2);
  }
}

// ----------------------------------------------------------------- passes
// Wave totals of the mode's weights from each lane's sums (all threads; ends
// with a barrier): sh.wtot[w] (each wave's own, from its lane 0) and
// sh.total (a 256-bit scan of the NW wave totals by wave 0).
template <int mode>
__device__ __forceinline__ void draw_totals(const DAcc& s1, uint64_t s2, const DrawCtx& c,
                                            DrawShared& sh) {
  DAcc ta;
  uint64_t ts2;
  wave_total(s1, s2, &ta, &ts2);
  if (lane_id() == 0) sh.wtot[wave_id()] = group_weight<mode>(ta, ts2, c);
  __syncthreads();
  if (wave_id() == 0) {
    const U256 inc = u256_wave_incl_scan(lane_id() < NW ? sh.wtot[lane_id()] : u256_zero());
    if (lane_id() == 63) sh.total = inc;
  }
  __syncthreads();
}

// Wave 0: the wave holding the draw's crossing and the threshold left
// inside it, from one 256-bit scan of the wave totals (after draw_totals;
// ends with a barrier).  A zero total gives wstar = -1.
__device__ __forceinline__ void draw_find_wave(uint64_t u, DrawShared& sh) {
  if (wave_id() == 0) {
    const U256 total = uniform_u256(sh.total);
    const int l = lane_id();
    const U256 v = l < NW ? sh.wtot[l] : u256_zero();
    const U256 inc = u256_wave_incl_scan(v);
    int ws = -1;
    U256 rest = u256_zero();
    if (!u256_is_zero(total)) {
      const U256 t = u256_mulhi64(total, u);  // < total
      const uint64_t hit = __ballot(l < NW && u256_lt(t, inc));
      ws = hit ? __builtin_ctzll(hit) : -1;
      if (ws >= 0) rest = u256_sub(t, u256_readlane(u256_sub(inc, v), ws));
    }
    if (l == 0) {
      sh.token = -1;
      sh.wstar = ws;
      sh.rest = rest;
    }
  }
  __syncthreads();
}

// In the crossing chunk (this lane's sums s1, s2 of it; t = the threshold
// left at the chunk's start): the lane holding the crossing and the
// threshold left inside that lane.  Wave-uniform results.
template <int mode>
__device__ __forceinline__ int draw_find_lane(const DAcc& s1, uint64_t s2, const DrawCtx& c,
                                              const U256& t, U256* lane_rest) {
  const U256 wl = group_weight<mode>(s1, s2, c);
  const U256 inc = u256_wave_incl_scan(wl);
  const uint64_t hit = __ballot(u256_lt(t, inc));
  const int l = hit ? __builtin_ctzll(hit) : 63;
  const U256 exc = u256_sub(inc, wl);
  *lane_rest = u256_sub(t, u256_readlane(exc, l));
  return l;
}

// The draw itself, from the totals of draw_totals: every wave totals its
// share of the crossing wave's chunks (one load round each), wave 0 finds the
// crossing chunk with 256-bit scans of the chunk totals, the wave that
// totalled that chunk reloads it and scans its lanes, and the crossing lane
// walks its elements.  Returns the token (-1 for a zero total).
template <int mode, int DT>
__device__ __forceinline__ int stream_walk(const StreamSrc<DT>& s, const DrawCtx& c, uint64_t u, DrawShared& sh) {
  draw_find_wave(u, sh);
  const int ws = sh.wstar;
  if (ws < 0) return -1;
  constexpr int E = StreamSrc<DT>::E;
  const __amdgpu_buffer_rsrc_t crs = count_rsrc(c);
  const bool c16 = (reinterpret_cast<uintptr_t>(c.dense) & 15u) == 0u;
  StreamSrc<DT> sw = s;  // the crossing wave's chunks, addressed from any wave
  auto vec_of = [&](int ch) { return (ws * s.cpw + ch) * 64 + lane_id(); };
  for (int ch = wave_id(); ch < s.cpw; ch += NW) {
    ChunkData<DT> d;
    stream_load_vec<mode, DT>(sw, vec_of(ch), c, crs, c16, d);
    DAcc a;
    dacc_zero(a);
    uint64_t b = 0;
    stream_add<mode, DT>(d, vec_of(ch), c, sh, a, b);
    DAcc ta;
    uint64_t tb;
    wave_total(a, b, &ta, &tb);
    if (lane_id() == 0) sh.ctot[ch] = group_weight<mode>(ta, tb, c);
  }
  __syncthreads();
  if (wave_id() == 0) {
    U256 t = uniform_u256(sh.rest);
    int ich = -1;
    for (int base = 0; base < s.cpw && ich < 0; base += 64) {  // (wave-uniform)
      const int ch = base + lane_id();
      const U256 v = ch < s.cpw ? sh.ctot[ch] : u256_zero();
      const U256 inc = u256_wave_incl_scan(v);
      const uint64_t hit = __ballot(ch < s.cpw && u256_lt(t, inc));
      if (hit) {
        const int l = __builtin_ctzll(hit);
        ich = base + l;
        t = u256_sub(t, u256_readlane(u256_sub(inc, v), l));
      } else {
        t = u256_sub(t, u256_readlane(inc, 63));
      }
    }
    if (lane_id() == 0) {
      sh.ichunk = ich;
      sh.rest = t;
    }
  }
  __syncthreads();
  const int ich = sh.ichunk;
  if (ich >= 0 && wave_id() == ich % NW) {
    ChunkData<DT> d;
    const int q = vec_of(ich);
    stream_load_vec<mode, DT>(sw, q, c, crs, c16, d);
    DAcc a;
    dacc_zero(a);
    uint64_t b = 0;
    stream_add<mode, DT>(d, q, c, sh, a, b);
    U256 lr;
    const int l = draw_find_lane<mode>(a, b, c, uniform_u256(sh.rest), &lr);
    if (lane_id() == l) {
      int tok = -1;
      U256 run = u256_zero();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (tok < 0) {
          const uint32_t wb = chunk_weight_bits<DT>(d.bits(e), c, sh);
          // ids past V carry weight 0 and have no count
          uint32_t cnt = 0u;
          if (mode != kDrawPlain && (wb & 0x7fffffffu) != 0u)
            cnt = c.dense ? d.cnt[e] : draw_count(c, sh, q * E + e);
          run = u256_add(run, elem_weight<mode>(wb, cnt, c));
          if (u256_lt(lr, run)) tok = q * E + e;
        }
      }
      sh.token = tok;
    }
  }
  __syncthreads();
  return sh.token;
}

// The same draw for a resident bf16 row whose weights come from the value
// table: the crossing wave parks its 16 chunks in LDS (the histogram area,
// unused by the draws), every wave totals one of them, wave 0 finds the
// crossing chunk by a 256-bit scan, and one wave scans that chunk's lanes.
__device__ __forceinline__ int wres_walk(Res& R, const DrawCtx& c, uint64_t u, DrawShared& sh) {
  static_assert(sizeof(sh.hist) >= NI * 64 * sizeof(u32x4), "chunk area");
  static_assert(NI == NW, "one chunk per wave");
  draw_find_wave(u, sh);
  const int ws = sh.wstar;
  if (ws < 0) return -1;
  u32x4* park = reinterpret_cast<u32x4*>(sh.hist);
  if (wave_id() == ws) {
    touch(R);
#pragma unroll
    for (int i = 0; i < NI; ++i) park[i * 64 + lane_id()] = fetch(R, i);
  }
  __syncthreads();
  {
    const int i = wave_id();  // chunk i of the crossing wave
    DAcc a;
    dacc_zero(a);
    wres_chunk(park[i * 64 + lane_id()], c, sh, a);
    DAcc ta;
    uint64_t tb;
    wave_total(a, 0ull, &ta, &tb);
    if (lane_id() == 0) sh.ctot[i] = u256_of_dacc(ta);
  }
  __syncthreads();
  if (wave_id() == 0) {
    const U256 t = uniform_u256(sh.rest);
    const int l = lane_id();
    const U256 v = l < NI ? sh.ctot[l] : u256_zero();
    const U256 inc = u256_wave_incl_scan(v);
    const uint64_t hit = __ballot(l < NI && u256_lt(t, inc));
    const int ich = hit ? __builtin_ctzll(hit) : 0;
    const U256 rest = u256_sub(t, u256_readlane(u256_sub(inc, v), ich));
    if (l == 0) {
      sh.ichunk = ich;
      sh.rest = rest;
    }
  }
  __syncthreads();
  const int ich = sh.ichunk;
  if (wave_id() == ich) {
    const u32x4 v = park[ich * 64 + lane_id()];
    DAcc a;
    dacc_zero(a);
    wres_chunk(v, c, sh, a);
    U256 lr;
    const int l = draw_find_lane<kDrawPlain>(a, 0ull, c, uniform_u256(sh.rest), &lr);
    if (lane_id() == l) {
      const int base = ws * 8192 + ich * 512 + lane_id() * 8;  // ids of the crossing wave's chunk ich
      int tok = -1;
      U256 run = u256_zero();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (tok < 0) {
          run = u256_add(run, u256_of_weight(bf16_weight_table(elem(v, e), c, sh)));
          if (u256_lt(lr, run)) tok = base + e;
        }
      }
      sh.token = tok;
    }
  }
  __syncthreads();
  return sh.token;
}

// Streamed row: per-lane sums over the wave's chunks, totals, and (with
// u_valid) the draw.  Returns the token (-1 if the total weight is zero or
// no draw was asked; sh.total holds the total either way).
template <int mode, int DT>
__device__ __forceinline__ int stream_draw(const StreamSrc<DT>& s, const DrawCtx& c, bool u_valid, uint64_t u,
                                           DrawShared& sh) {
  DAcc s1;
  dacc_zero(s1);
  uint64_t s2 = 0;
  stream_sums<mode, DT>(s, c, sh, s1, s2);
  draw_totals<mode>(s1, s2, c, sh);
  if (!u_valid) return -1;
  return stream_walk<mode, DT>(s, c, u, sh);
}

// Resident bf16 row (loaded by wres_load from p): the plain sums come from
// the registers when the value table applies; otherwise, for residual sums
// (one row per request, whose per-element count lookups would not fit beside
// the row's registers) and for the walk, the row is reloaded.
// Resident bf16 row (loaded by wres_load) whose weights come from the value
// table (c.table): plain sums and the draw from its registers.
__device__ __forceinline__ int wres_draw(Res& R, const DrawCtx& c, bool u_valid, uint64_t u, DrawShared& sh) {
  DAcc s1;
  dacc_zero(s1);
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) wres_chunk(fetch(R, i), c, sh, s1);
  draw_totals<kDrawPlain>(s1, 0ull, c, sh);
  if (!u_valid) return -1;
  return wres_walk(R, c, u, sh);
}

}  // namespace dspark
