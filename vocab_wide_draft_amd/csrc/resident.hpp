// bf16 rows held in registers: each of the 1024 threads keeps NI 16-byte
// vectors (8 bf16 each), so a row of up to NI*1024*8 = 131072 tokens is read
// from HBM exactly once and every later pass runs on chip.
//
// Keys: for bf16 bits b, K16(b) = 0x8000 + (b sign ? -(b & 0x7fff) : b), an
// order-preserving 16-bit key in which -0 and +0 coincide (IEEE equality).
#pragma once
#include "row_alloc.hpp"

namespace dspark {

constexpr int NI = 16;
constexpr uint32_t kNegInf2 = 0xff80ff80u;  // two bf16 -inf (padding lanes)
constexpr int kKeyNegInf = 0x8000 - 0x7f80;  // K16(-inf)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int k16(uint32_t b) {
  const int mag = (int)(b & 0x7fffu);
  return 0x8000 + ((b & 0x8000u) ? -mag : mag);
}
__device__ __forceinline__ uint32_t bf16_of_k16(int k) {
  const int s = k - 0x8000;
  return s >= 0 ? (uint32_t)s : (0x8000u | (uint32_t)(-s));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
// element l (0..7) of a vector, as bf16 bits
__device__ __forceinline__ uint32_t elem(u32x4 v, int l) {
  const uint32_t w = (l >> 1) == 0 ? v.x : (l >> 1) == 1 ? v.y : (l >> 1) == 2 ? v.z : v.w;
  return (l & 1) ? (w >> 16) : (w & 0xffffu);
}

struct Res {
  uint32_t w[NI][4];  // 64 scalar words, all indices static: the array lives in registers
};

// An empty asm that claims to rewrite every row register in place.  Called at
// the start of each pass, it keeps the compiler from hoisting values derived
// from the row (keys, masks) out of one pass into an earlier one, which would
// need far more registers than the row itself; it creates no copies.
__device__ __forceinline__ void touch(Res& R) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
    asm volatile("" : "+v"(R.w[i][0]), "+v"(R.w[i][1]), "+v"(R.w[i][2]), "+v"(R.w[i][3]));
}
// Reads vector i through an in-place empty asm on its four words: work on
// vector i cannot be hoisted above this read, so a pass does not compute keys
// or lookups for all sixteen vectors at once.
__device__ __forceinline__ u32x4 fetch(Res& R, int i) {
  asm volatile("" : "+v"(R.w[i][0]), "+v"(R.w[i][1]), "+v"(R.w[i][2]), "+v"(R.w[i][3]));
  return u32x4{R.w[i][0], R.w[i][1], R.w[i][2], R.w[i][3]};
}
// vector i (block-uniform, 0 <= i < NI) picked by a select chain over
// barrier-read vectors (so that it never becomes an indexed memory access)
__device__ __forceinline__ u32x4 select_vec(Res& R, int i) {
  u32x4 v = fetch(R, 0);
#pragma unroll
  for (int j = 1; j < NI; ++j) {
    const u32x4 w = fetch(R, j);
    v = (i == j) ? w : v;
  }
  return v;
}
__device__ __forceinline__ void store_vec(Res& R, int i, u32x4 v) {
  R.w[i][0] = v.x;
  R.w[i][1] = v.y;
  R.w[i][2] = v.z;
  R.w[i][3] = v.w;
}

// All NI loads are issued back to back with no branch between them (a
// branch per load makes the compiler wait for each load before the next);
// lanes past the last full vector read vector 0 and become -inf padding.
// Only one vector of a row can be partial (V % 8 != 0); its single owner
// thread patches it from 2-byte loads.
__device__ __forceinline__ void res_load(Res& R, const uint16_t* p, int V) {
  const int nfull = V >> 3;
  const u32x4 pad = {kNegInf2, kNegInf2, kNegInf2, kNegInf2};
  // A buffer resource that covers exactly the row: every load is the
  // thread's offset plus a constant, all sixteen go out back to back, and
  // lanes past the row end read zeros from the hardware bounds check
  // (replaced by -inf below) instead of touching memory beyond the row.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, V * 2, 0x00020000);
  const int toff = (int)threadIdx.x * 16;
#pragma unroll
  for (int i = 0; i < NI; ++i)
    store_vec(R, i, __builtin_amdgcn_raw_buffer_load_b128(rs, toff, i * BS * 16, 2));  // nt: read once
  // only vectors that reach past the last full one can hold padding lanes
  // (a uniform test), so the others need not wait for their loads here
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if ((i + 1) * BS > nfull) {
      const int q = i * BS + (int)threadIdx.x;
      if (q >= nfull) store_vec(R, i, pad);
    }
  }
  if ((V & 7) && (int)threadIdx.x == nfull % BS) {
    const int it = nfull / BS;
    uint32_t h[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) h[l] = nfull * 8 + l < V ? (uint32_t)p[nfull * 8 + l] : 0xff80u;
    const u32x4 part = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (i == it) store_vec(R, i, part);
  }
}

// ------------------------------------------------------------- statistics
struct RStats {
  int status;
  uint32_t m_raw;   // bf16 bits of the row maximum
  int smax_t;       // this thread's largest raw int16 (one of its elements)
};

// Row maximum and validity from packed int16 maxima of the raw bits: the
// signed maximum is the true maximum whenever some value is >= +0; a
// positive NaN shows as a signed maximum above +inf, a negative NaN as an
// unsigned maximum above -inf.  Rows with only negative values take one more
// pass (their maximum has the smallest unsigned pattern).
__device__ __forceinline__ RStats res_stats(Res& R, SmemBase& sh) {
  // no touch of the whole row first: each vector is taken as soon as its own
  // load has returned, so this pass overlaps the tail of the row load
  s16x2 sm[4] = {{(short)-32768, (short)-32768}, {(short)-32768, (short)-32768},
                 {(short)-32768, (short)-32768}, {(short)-32768, (short)-32768}};
  u16x2 umax = {0, 0};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 vi = fetch(R, i);
    const uint32_t w[4] = {vi.x, vi.y, vi.z, vi.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sm[c] = __builtin_elementwise_max(sm[c], __builtin_bit_cast(s16x2, w[c]));
      umax = __builtin_elementwise_max(umax, __builtin_bit_cast(u16x2, w[c]));
    }
  }
  RStats s;
  const s16x2 smax = __builtin_elementwise_max(__builtin_elementwise_max(sm[0], sm[1]),
                                               __builtin_elementwise_max(sm[2], sm[3]));
  s.smax_t = smax.x > smax.y ? smax.x : smax.y;
  const int um_t = umax.x > umax.y ? umax.x : umax.y;
  if (threadIdx.x == 0) sh.amin = 0x7fffffff;  // for res_argmax (ordered by the barriers below)
  // one reduction for both: the signed maximum biased into the high half
  const uint32_t SU = block_max_u16x2(((uint32_t)(s.smax_t + 0x8000) << 16) | (uint32_t)um_t, sh.bs);
  const int S = (int)(SU >> 16) - 0x8000;
  const int U = (int)(SU & 0xffffu);
  if (S > 0x7f80 || U > 0xff80) {
    s.status = DSPARK_ST_ROW_NAN;
    s.m_raw = 0;
    return s;
  }
  if (S == 0x7f80) {
    s.status = DSPARK_ST_ROW_POSINF;
    s.m_raw = 0;
    return s;
  }
  if (S >= 0) {
    s.m_raw = (uint32_t)S;
  } else {  // every value negative (or -0): the maximum has the smallest pattern
    touch(R);
    u16x2 umin = {0xffff, 0xffff};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u32x4 vi = fetch(R, i);
    const uint32_t w[4] = {vi.x, vi.y, vi.z, vi.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) umin = __builtin_elementwise_min(umin, __builtin_bit_cast(u16x2, w[c]));
    }
    const int mn_t = umin.x < umin.y ? umin.x : umin.y;
    s.m_raw = (uint32_t)block_min<int>(mn_t, sh.bs);
  }
  s.status = s.m_raw == 0xff80u ? DSPARK_ST_ROW_ZERO_MASS : DSPARK_ST_OK;
  return s;
}

// Lowest index holding the maximum (value compare, so -0 == +0).  For a
// positive maximum only threads whose own signed maximum equals it can hold
// it, so the other threads skip the scan.
// 8-bit mask (bit l = element l) of the halves of vector v equal to T
// (T2 = T twice) in the bits of M2 (both halves all ones: the whole pattern;
// 0x7fff7fff: +0 and -0 alike): a half h is zero exactly when bit 15 of
// ((h & 0x7fff) + 0x7fff) | h is clear.
__device__ __forceinline__ uint32_t eq16_mask8(u32x4 v, uint32_t T2, uint32_t M2 = 0xffffffffu) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = (w[c] ^ T2) & M2;
    const uint32_t z = ~(((x & 0x7fff7fffu) + 0x7fff7fffu) | x) & 0x80008000u;
    m |= ((z >> 15) & 1u) << (2 * c);
    m |= (z >> 31) << (2 * c + 1);
  }
  return m;
}

__device__ __forceinline__ int res_argmax(Res& R, const RStats& st, SmemBase& sh) {
  touch(R);
  const bool pos = st.m_raw > 0u && st.m_raw < 0x8000u;
  int first = 0x7fffffff;
  if (!pos || (uint32_t)st.smax_t == st.m_raw) {  // threads that can hold the maximum
    const float m = bf16_to_f32(st.m_raw);
    const uint32_t T2 = st.m_raw * 0x10001u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u32x4 v = fetch(R, i);
      if (pos) {  // a positive maximum has one bit pattern: a zero half of v ^ T2
        const u16x2 x0 = __builtin_bit_cast(u16x2, v.x ^ T2), x1 = __builtin_bit_cast(u16x2, v.y ^ T2);
        const u16x2 x2 = __builtin_bit_cast(u16x2, v.z ^ T2), x3 = __builtin_bit_cast(u16x2, v.w ^ T2);
        const u16x2 p = __builtin_elementwise_min(__builtin_elementwise_min(x0, x1), __builtin_elementwise_min(x2, x3));
        if ((p.x == 0 || p.y == 0) && first == 0x7fffffff)
          first = (i * BS + (int)threadIdx.x) * 8 + __builtin_ctz(eq16_mask8(v, T2));
      } else {
        uint32_t msk = 0;
#pragma unroll
        for (int l = 0; l < 8; ++l) msk |= (bf16_to_f32(elem(v, l)) == m ? 1u : 0u) << l;
        if (msk && first == 0x7fffffff) first = (i * BS + (int)threadIdx.x) * 8 + __builtin_ctz(msk);
      }
    }
  }
  // the threads that hold the maximum (usually one) meet in one LDS minimum
  if (first != 0x7fffffff) atomicMin(&sh.amin, first);
  __syncthreads();
  return sh.amin;
}

// 1 / sum_v exp(x_v - m); x_v - m is exact in binary32 for bf16 operands of
// close magnitude, the exponential is the hardware base-2 one.
__device__ __forceinline__ float res_conf(Res& R, float m, SmemBase& sh) {
  touch(R);
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 vi = fetch(R, i);
    const uint32_t w[4] = {vi.x, vi.y, vi.z, vi.w};
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = __uint_as_float(w[c] << 16), hi = __uint_as_float(w[c] & 0xffff0000u);
      part += __builtin_amdgcn_exp2f((lo - m) * 1.4426950408889634f);
      part += __builtin_amdgcn_exp2f((hi - m) * 1.4426950408889634f);
    }
    sum += (double)part;
  }
  const double s = block_sum<double>(sum, sh.bs);
  return (float)(1.0 / s);
}

// ------------------------------------------------ locate and compaction
// First element (ID order) whose running 0/1 weight exceeds u; mf(i, v)
// gives the 8-bit mask of the lanes of vector i*BS + thread that weigh 1.
template <class MF>
__device__ __forceinline__ int res_locate(Res& R, MF mf, uint32_t u, SmemBase& sh) {
  touch(R);
  if (threadIdx.x < NI) sh.tab[threadIdx.x] = 0;
  __syncthreads();
  uint32_t m4[NI / 4] = {0, 0, 0, 0};  // the 16 lane masks, 8 bits each
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t msk = mf(i, fetch(R, i)) & 0xffu;
    m4[i >> 2] |= msk << ((i & 3) * 8);
    const uint32_t c = (uint32_t)__builtin_popcount(msk);
    if (__ballot(c != 0u)) {
      const uint32_t s = wave_sum(c);
      if (lane_id() == 0 && s) atomicAdd((unsigned long long*)&sh.tab[i], (unsigned long long)s);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint64_t before = 0;
    const int i = wave_first_above(sh.tab, NI, u, &before);
    if (threadIdx.x == 0) {
      sh.bi[1] = i;
      sh.bu[1] = before;
    }
  }
  __syncthreads();
  const int istar = sh.bi[1];
  int result = -1;
  if (istar >= 0) {
    const uint32_t u2 = u - (uint32_t)sh.bu[1];
    const int g = istar >> 2;
    const uint32_t word = g == 0 ? m4[0] : g == 1 ? m4[1] : g == 2 ? m4[2] : m4[3];
    const uint32_t msk = (word >> ((istar & 3) * 8)) & 0xffu;
    const uint32_t c = (uint32_t)__builtin_popcount(msk);
    uint32_t tot;
    const uint32_t pre = block_excl_scan<uint32_t>(c, sh.bs, &tot);
    if (pre <= u2 && u2 < pre + c) {
      uint32_t run = pre;
      int hit = -1;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        if (msk & (1u << l)) {
          if (run == u2 && hit < 0) hit = l;
          ++run;
        }
      }
      sh.bi[2] = (istar * BS + (int)threadIdx.x) * 8 + hit;
    }
    __syncthreads();
    result = sh.bi[2];
  }
  __syncthreads();
  return result;
}

// res_locate for the members of one table entry, from registers that hold
// two 16-bit table offsets per word (T: the entry's offset): the id of the
// (u+1)-th member in id order, or -1 when there are at most u members.  The
// count of each (vector, wave) cell comes from wave ballots of the 16-bit
// compares (scalar population counts); wave 0 finds the cell, and that
// cell's wave alone finds the lane.
__device__ __forceinline__ int tie_locate(Res& R, uint32_t T, uint32_t u, SmemBase& sh) {
  touch(R);
  const uint16_t T16 = (uint16_t)T;
  uint32_t* cells = sh.hist;  // [NI][NW] member counts, in id order: vector, then wave
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = fetch(R, i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    // a zero half of w ^ T2 marks a member: a packed minimum tells whether
    // this lane has one, and most cells hold none
    const uint32_t T2 = T * 0x10001u;
    const u16x2 p = __builtin_elementwise_min(
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, w[0] ^ T2), __builtin_bit_cast(u16x2, w[1] ^ T2)),
        __builtin_elementwise_min(__builtin_bit_cast(u16x2, w[2] ^ T2), __builtin_bit_cast(u16x2, w[3] ^ T2)));
    uint32_t cnt = 0;
    if (__ballot(p.x == 0 || p.y == 0) != 0ull) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cnt += (uint32_t)__builtin_popcountll(__ballot((uint16_t)w[c] == T16));
        cnt += (uint32_t)__builtin_popcountll(__ballot((uint16_t)(w[c] >> 16) == T16));
      }
    }
    if (lane_id() == 0) cells[i * NW + wave_id()] = cnt;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // lane l takes cells 4l .. 4l + 3
    const int l = lane_id();
    uint64_t c4[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c4[j] = cells[4 * l + j];
      s += c4[j];
    }
    const uint64_t inc = wave_incl_scan(s);
    const uint64_t hit = __ballot(inc > (uint64_t)u);
    if (l == 0) sh.bi[2] = -1;
    if (hit == 0ull) {
      if (l == 0) sh.bi[1] = -1;
    } else if (l == __builtin_ctzll(hit)) {
      uint64_t run = inc - s;
      int cell = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cell < 0 && run + c4[j] > (uint64_t)u) cell = 4 * l + j;
        if (cell < 0) run += c4[j];
      }
      sh.bi[1] = cell;
      sh.bu[1] = run;  // members before the cell
    }
  }
  __syncthreads();
  const int cell = sh.bi[1];
  int result = -1;
  if (cell >= 0) {
    if (wave_id() == (cell % NW)) {
      const int i = cell / NW;
      const u32x4 v = select_vec(R, i);
      const uint32_t m = eq16_mask8(v, T * 0x10001u);
      const uint64_t pc = (uint64_t)__builtin_popcount(m);
      const uint64_t exc = wave_incl_scan(pc) - pc;
      const uint64_t u2 = (uint64_t)u - sh.bu[1];
      if (exc <= u2 && u2 < exc + pc) {
        uint32_t mm = m;
        for (uint64_t k = exc; k < u2; ++k) mm &= mm - 1u;  // drop the members before
        sh.bi[2] = (i * BS + (int)threadIdx.x) * 8 + __builtin_ctz(mm);
      }
    }
    __syncthreads();
    result = sh.bi[2];
  }
  return result;  // (bi[1], bi[2], bu[1] are written again only after later barriers)
}

// Writes the selected elements (mf mask) to (sh.cid, sh.sx) in ascending ID
// order.  Returns the count (at most cap are stored).
template <class MF>
__device__ __forceinline__ int res_compact(Res& R, MF mf, int cap, RowShared& sh) {
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t c = (uint32_t)__builtin_popcount(mf(i, fetch(R, i)));
    uint32_t wc = 0;
    if (__ballot(c != 0u)) wc = wave_sum(c);
    if (lane_id() == 0) sh.ctab[i * NW + wave_id()] = wc;
  }
  __syncthreads();
  {
    const uint32_t v = threadIdx.x < NI * NW ? sh.ctab[threadIdx.x] : 0u;
    uint32_t tot;
    const uint32_t pre = block_excl_scan<uint32_t>(v, sh.bs, &tot);
    if (threadIdx.x < NI * NW) sh.ctab[threadIdx.x] = pre;
    if (threadIdx.x == 0) sh.bi[3] = (int)tot;
  }
  __syncthreads();
  const int total = sh.bi[3];
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t msk = mf(i, fetch(R, i));
    const uint32_t c = (uint32_t)__builtin_popcount(msk);
    if (__ballot(c != 0u)) {
      const uint32_t inc = wave_incl_scan(c);
      int pos = (int)(sh.ctab[i * NW + wave_id()] + inc - c);
      const int q = i * BS + (int)threadIdx.x;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        if (msk & (1u << l)) {
          if (pos < cap) {
            sh.cid[pos] = (uint32_t)(q * 8 + l);
            sh.sx[pos] = bf16_to_f32(elem(fetch(R, i), l));
          }
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  return total < cap ? total : cap;
}

// -------------------------------------------------------- sparse top-k
// k-th largest of one key (< 2^16) per thread: two byte passes.
__device__ __forceinline__ int block_kth_largest16(int v, int k, SmemBase& sh) {
  uint32_t prefix = 0, pmask = 0;
  uint64_t need = (uint64_t)k;
  for (int shift = 8; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0;
    __syncthreads();
    if (((uint32_t)v & pmask) == prefix) atomicAdd(&sh.hist[((uint32_t)v >> shift) & 255u], 1u);
    __syncthreads();
    uint64_t before;
    const int d = block_find_crossing(sh.hist, 256, need, false, sh, &before);
    need -= before;
    prefix |= (uint32_t)d << shift;
    pmask |= 0xffu << shift;
  }
  return (int)prefix;
}

// mask of lanes with K16 >= lo (lo > K16(-inf)); positive lo values compare
// raw patterns with a saturating packed subtraction.
__device__ __forceinline__ uint32_t ge_mask(u32x4 v, int lo) {
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (lo > 0x8000) {
    const short rl = (short)(lo - 0x8000);
    const s16x2 L = {rl, rl};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const s16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(s16x2, w[c]), L);
      m |= (d.x >= 0 ? 1u : 0u) << (2 * c);
      m |= (d.y >= 0 ? 1u : 0u) << (2 * c + 1);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      m |= (k16(w[c] & 0xffffu) >= lo ? 1u : 0u) << (2 * c);
      m |= (k16(w[c] >> 16) >= lo ? 1u : 0u) << (2 * c + 1);
    }
  }
  return m;
}

// Top-k support of a resident bf16 row by (logit desc, id asc), without -inf
// entries (they would carry weight 0 and be dropped), into sh.cid / sh.sx.
// Returns the support size.
__device__ __forceinline__ int res_topk_support(Res& R, const RStats& st, int k, RowShared& sh) {
  const int Km = k16(st.m_raw);
  int lo = block_kth_largest16(k16((uint32_t)st.smax_t & 0xffffu), k, sh);
  if (lo <= kKeyNegInf) lo = kKeyNegInf + 1;
  int hi = Km;
  uint64_t need = (uint64_t)k;
  bool first = true;
  int T = 0, cut = 0x7fffffff;
  bool all_ge = false;
  for (;;) {
    const int range = hi - lo;
    const int shift = range < kHistBins ? 0 : (32 - __builtin_clz((uint32_t)range)) - 12;
    const int nb = (range >> shift) + 1;
    for (int b = threadIdx.x; b < nb; b += BS) sh.hist[b] = 0;
    __syncthreads();
    touch(R);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t msk = ge_mask(fetch(R, i), lo);
      if (msk) {
#pragma unroll
        for (int l = 0; l < 8; ++l) {
          const int K = k16(elem(fetch(R, i), l));
          if ((msk & (1u << l)) && K <= hi) atomicAdd(&sh.hist[(hi - K) >> shift], 1u);
        }
      }
    }
    __syncthreads();
    uint64_t total = 0;
    for (int b = threadIdx.x; b < nb; b += BS) total += sh.hist[b];
    total = block_sum<uint64_t>(total, sh.bs);
    if (first) {  // fewer finite entries than k: the support is every finite entry
      if (total < need) need = total;
      first = false;
    }
    if (need == 0) return 0;
    uint64_t before;
    const int b = block_find_crossing(sh.hist, nb, need, true, sh, &before);
    need -= before;
    const uint32_t cnt = sh.hist[b];
    __syncthreads();
    const int bhi = hi - (b << shift);
    const int blo = (bhi - lo) > ((1 << shift) - 1) ? bhi - ((1 << shift) - 1) : lo;
    if (cnt == need) {
      T = blo;
      all_ge = true;
      break;
    }
    if (shift == 0) {
      T = bhi;
      cut = res_locate(R, [&](int, u32x4 v) -> uint32_t {
        uint32_t m = 0;
#pragma unroll
        for (int l = 0; l < 8; ++l) m |= (k16(elem(v, l)) == T ? 1u : 0u) << l;
        return m;
      }, (uint32_t)(need - 1), sh);
      break;
    }
    hi = bhi;
    lo = blo;
  }
  // the support: K > T, or K == T and (all_ge or id <= cut)
  return res_compact(R, [&](int i, u32x4 v) -> uint32_t {
    const uint32_t m = ge_mask(v, T);
    if (all_ge || m == 0u) return m;
    const int base = (i * BS + (int)threadIdx.x) * 8;
    uint32_t out = 0;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const int K = k16(elem(v, l));
      out |= ((m & (1u << l)) && (K > T || base + l <= cut) ? 1u : 0u) << l;
    }
    return out;
  }, DSPARK_K_MAX, sh);
}

}  // namespace dspark
