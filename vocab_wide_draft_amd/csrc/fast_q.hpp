// dyadic24 q of a register-resident bf16 draft row from a compressed value
// table ("PP1 q transport and scheduling design", "Distribution contract and
// precision" for the allocation; "Sparse support and vocabulary-sharded TP2
// follow-up" for the top-k support).
//
// Every quantity of the allocation before the id tie-break is a function of
// d = RN32(x - m), the binary32 difference of a logit and the row maximum.
// Logits whose magnitude is below tau = 2^(e_m - 26) (an eighth of a binary32
// ulp of m, m > 0) all give d = -m exactly, so they share one table entry
// (the "collapsed" entry); every other bf16 value in the weight window
// [m - 105, m] has an entry of its own.  Entries are ordered by value, largest
// first, so the table is both a histogram for the allocation and an order
// statistic for the top-k threshold.  For a row maximum of ordinary size the
// table has about 7k entries (instead of the ~34k bf16 values of the window),
// which leaves room in LDS to keep each entry's weight and remainder key
// between passes.  Rows whose table would exceed kNBF entries (a maximum
// below about 0.04, or not positive) take the general per-value path of
// dense_vd.hpp.
//
// The confidence 1 / sum_v exp(x_v - m) is also taken from the table.  A
// dense row has the exact sum S of its weights and uses 1 / RN64(S) (error
// bound at pass A of fast_dense_q).  A sparse row sums n * exp(x - m) per entry with
// x - m exact in binary64; there the collapsed entry uses exp(-m), which is
// within a relative 2^(e_m - 26) of each of its terms and holds at most a
// fraction V e^-m / (1 + V e^-m) of the sum (below 1.2e-7 of the confidence
// for any m).
#pragma once
#include "dense_vd.hpp"
#include "resident.hpp"

namespace dspark {

constexpr int kNBF = 8192;         // largest compressed table
// internal row status: several table entries share the threshold remainder
// key exactly, and the general per-value path decides the row
constexpr int kStGeneral = -1;
constexpr int kNBFD = kNBF + 64;   // plus one overflow slot per lane

// Table layout of one row.  bin(x) = B0 - c(|x|) for x with the sign bit
// clear, B0 + c(|x|) with it set, where c(a) = max(a, tb1) - tb1 on the
// magnitude bits; magnitudes <= tb1 give c = 0, the collapsed entry B0.
struct FMap {
  int B0, tb1, NB;
  int NBc;  // entries of the values >= m - 28 (the confidence range)
  uint32_t Cp2, Tp2, Cn2, Tn2;  // the formula's constants, twice per word
};

__device__ __forceinline__ int fmap_c(uint32_t mag, int tb1) {
  const int a = (int)mag;
  return (a > tb1 ? a : tb1) - tb1;
}
__device__ __forceinline__ int fmap_bin(uint32_t raw, const FMap& f) {
  const int c = fmap_c(raw & 0x7fffu, f.tb1);
  return (raw & 0x8000u) ? f.B0 + c : f.B0 - c;
}
// bf16 pattern of the values in entry b (for the collapsed entry: +0, whose d
// is -m like every member's)
__device__ __forceinline__ uint32_t fmap_raw(int b, const FMap& f) {
  if (b <= f.B0) {
    const int c = f.B0 - b;
    return c == 0 ? 0u : (uint32_t)(c + f.tb1);
  }
  return 0x8000u | (uint32_t)(b - f.B0 + f.tb1);
}

// Layout for the row maximum m_raw (valid row).  NB > kNBF means "not
// applicable".
__device__ __forceinline__ FMap fmap_make(uint32_t m_raw) {
  FMap f;
  const uint32_t mag_m = m_raw & 0x7fffu;
  const bool mneg = (m_raw & 0x8000u) != 0;
  f.tb1 = 0;
  if (!mneg && mag_m != 0u) {
    const int Em = (int)(mag_m >> 7);  // bf16 exponent field of m
    if (Em - 26 >= 1) f.tb1 = ((Em - 26) << 7) - 1;
  }
  const int cm = fmap_c(mag_m, f.tb1);
  f.B0 = mneg ? -cm : cm;
  // smallest bf16 >= m - t (binary32), never below the most negative finite value
  const float m = bf16_to_f32(m_raw);
  auto lowest_at_or_above = [&](float t) -> uint32_t {
    const uint32_t b = __float_as_uint(m - t);
    uint32_t hb = b >> 16;
    if ((b & 0xffffu) && !(b & 0x80000000u)) hb += 1u;
    hb &= 0xffffu;
    return hb > 0xff7fu ? 0xff7fu : hb;
  };
  f.NB = fmap_bin(lowest_at_or_above(105.0f), f) + 1;
  f.NBc = fmap_bin(lowest_at_or_above(28.0f), f) + 1;
  const uint32_t Cp = (uint32_t)(f.B0 + f.tb1) & 0xffffu, Tp = (uint32_t)f.tb1;
  const uint32_t Cn = (uint32_t)(f.B0 - f.tb1 - 0x8000) & 0xffffu, Tn = 0x8000u + (uint32_t)f.tb1;
  f.Cp2 = Cp * 0x10001u;
  f.Tp2 = Tp * 0x10001u;
  f.Cn2 = Cn * 0x10001u;
  f.Tn2 = Tn * 0x10001u;
  return f;
}

// Byte offsets (bin * 4) of the two bf16 values of word w, in the low and
// high halves; out-of-window values and -inf land in [NB, kNBFD) (the
// overflow slots spread by lane).  Packed 16-bit arithmetic: no entry
// exceeds 0xffff before the clamp, and kNBFD * 4 < 2^16.
__device__ __forceinline__ uint32_t fmap_off2(uint32_t w, const FMap& f, uint32_t D2) {
  const u16x2 v = __builtin_bit_cast(u16x2, w);
  const u16x2 pos = __builtin_bit_cast(u16x2, f.Cp2) - __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, f.Tp2));
  const u16x2 neg = __builtin_bit_cast(u16x2, f.Cn2) + __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, f.Tn2));
  const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (short)15);
  const uint32_t bin = (__builtin_bit_cast(uint32_t, neg) & s) | (__builtin_bit_cast(uint32_t, pos) & ~s);
  const u16x2 bc = __builtin_elementwise_min(__builtin_bit_cast(u16x2, bin), __builtin_bit_cast(u16x2, D2));
  const u16x2 two = {2, 2};
  return __builtin_bit_cast(uint32_t, bc << two);
}
__device__ __forceinline__ uint32_t fmap_dummy2() {
  const uint32_t d = (uint32_t)(kNBF + lane_id());
  return d * 0x10001u;
}

// exp(x) for binary64 x in [-106, 0] to about 1e-16 relative (Tang's table
// reduction with the library's constants, degree-5 Taylor polynomial).
__device__ __forceinline__ double exp64(double x) {
  const double kf = __builtin_rint(x * kExpInvL);
  const int k = (int)kf;
  const double r = __builtin_fma(-kf, kExpCHi, x) - kf * kExpCLo;
  double P = __builtin_fma(r, kExpP5, kExpP4);
  P = __builtin_fma(r, P, kExpP3);
  P = __builtin_fma(r, P, kExpP2);
  const double p = __builtin_fma(r * r, P, r);
  return __builtin_ldexp(__builtin_fma(kExpTabHi[k & 63], p, kExpTabHi[k & 63]), k >> 6);
}

// --------------------------------------------------------------- shared
struct FastDenseShared : SmemBase {
  uint32_t nb[kNBFD];   // counts, then final counts (a tie entry holds its floor)
  float wb[kNBF];       // binary32 weight of each occupied entry
  uint32_t kb[kNBF];    // top 32 bits of each entry's remainder key (0: r = 0)
  uint16_t occ[kNBF];   // the occupied entries, in no particular order
  uint64_t ckey[kVdCand];
  uint32_t cbin[kVdCand];
};
// The sparse layout keeps the table first (below 64 KB of LDS, so that its
// base folds into the offset field of the LDS atomics).
struct FastSparseShared : SmemBase {
  uint32_t nb[kNBFD];
  uint32_t bmA[NI * NW * 16];  // bitmap over ids: selected elements
  uint32_t bmB[NI * NW * 16];  // bitmap over ids: members of the threshold entry
  uint64_t ckey[kCandCap];     // candidates (K16 << 32 | id); later remainder keys
  uint32_t cid[kCandCap];      // support ids, ascending
  float sx[DSPARK_K_MAX];      // support logits
  uint32_t ctab[kMaxIter * NW];  // remainder bucket members
};

// Clears the whole table (entries and overflow slots); the callers do this
// while the row is still loading.
__device__ __forceinline__ void fast_clear(uint32_t* nb) {
  for (int b = (int)threadIdx.x; b < kNBFD; b += BS) nb[b] = 0u;
}
// Histogram of the row into nb[0, NB) (overflow slots take the rest), on a
// table cleared by fast_clear before some earlier barrier.  With KEEP, every
// register word is replaced by its two table byte offsets, which is all the
// later passes of the dense path need.
template <bool KEEP>
__device__ __forceinline__ void fast_hist(Res& R, const FMap& f, uint32_t* nb) {
  touch(R);
  const uint32_t D2 = fmap_dummy2();
  char* base = reinterpret_cast<char*>(nb);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = fetch(R, i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t o = fmap_off2(w[c], f, D2);
      atomicAdd(reinterpret_cast<uint32_t*>(base + (o & 0xffffu)), 1u);
      atomicAdd(reinterpret_cast<uint32_t*>(base + (o >> 16)), 1u);
      if (KEEP) R.w[i][c] = o;
    }
  }
  __syncthreads();
}

// The confidence sum over the table, n exp(x - m) per entry in binary64.
// Entries more than 28 below the maximum are left out: together they add at
// most V e^-28 < 9e-8 to a sum that is at least 1.
__device__ __forceinline__ double fast_conf_sum(const FMap& f, float m, const uint32_t* nb) {
  const double md = (double)m;
  double cs = 0.0;
  for (int b = (int)threadIdx.x; b < f.NBc; b += BS) {
    const uint32_t n = nb[b];
    if (n) {
      const double dx = (double)bf16_to_f32(fmap_raw(b, f)) - md;
      if (dx >= -28.0) cs += (double)n * exp64(dx);
    }
  }
  return cs;
}

// binary64 floor and exact remainder key of entry b
__device__ __forceinline__ void fast_floor_key(float w, const SumR& S, uint32_t& c, uint64_t& key) {
  double r;
  floor_rem(w, S, c, r);
  key = r > 0.0 ? rem_key(r) : 0ull;
}

// --------------------------------------------------------------- dense
__device__ __forceinline__ QOut fast_dense_q(Res& R, const RStats& st, const FMap& f, uint32_t* drow, int V,
                                             bool want_s, uint32_t u, bool want_conf, float* conf,
                                             FastDenseShared& sh DSPARK_PHASE_PARAM) {
  QOut res{DSPARK_ST_OK, 0};
  const float m = bf16_to_f32(st.m_raw);
  const int NB = f.NB;
  if (threadIdx.x == 0) sh.bi[3] = 0;  // (ordered by the histogram's barriers)
  fast_hist<true>(R, f, sh.nb);  // the registers now hold table offsets
  // overflow slots read 0 from here on (the final pass looks up
  // out-of-window elements there)
  for (int b = NB + (int)threadIdx.x; b < kNBFD; b += BS) sh.nb[b] = 0u;
  // The per-entry passes below run over the occupied entries only (about 40 %
  // of the table, in runs): listed once, every pass then keeps all lanes
  // busy and every wave equally loaded.  No pass depends on the order.
  for (int b = (int)threadIdx.x; b < NB; b += BS)
    if (sh.nb[b]) sh.occ[atomicAdd(&sh.bi[3], 1)] = (uint16_t)b;
  __syncthreads();
  const int nocc = sh.bi[3];
  DSPARK_PHASE(11);
  // A. weights and their exact sum; the confidence is 1 / RN64 of the sum:
  // each weight RN32(exp(RN32(x - m))) is within 2^-24 (1 + |x - m|) of
  // exp(x - m) relatively, and the e^(x-m)-weighted mean of |x - m| over at
  // most 2^17 terms, one of them 0, stays below 9, so the sum is within 6e-7
  // of sum exp(x - m) relatively
  // the first digit histogram and the candidate counter start empty (the
  // barriers of the reductions below order this first)
  uint64_t* rh = reinterpret_cast<uint64_t*>(sh.hist);  // 2048 digits
  for (int d = (int)threadIdx.x; d < 2048; d += BS) rh[d] = 0ull;
  if ((int)threadIdx.x == 0) sh.bi[4] = 0;
  Acc acc;
  acc_zero(acc);
  for (int j = (int)threadIdx.x; j < nocc; j += BS) {
    const int b = sh.occ[j];
    const uint32_t n = sh.nb[b];
    const float w = cr_expf(bf16_to_f32(fmap_raw(b, f)) - m);
    sh.wb[b] = w;
    acc_add(acc, __float_as_uint(w), n);
  }
  DSPARK_PHASE(36);
  const SumR S = sum_r(block_acc_rn64(acc, sh.acc));
  if (want_conf) *conf = (float)S.y;
  if (!(S.s > 0.0)) {
    res.status = DSPARK_ST_ROW_ZERO_MASS;
    return res;
  }
  DSPARK_PHASE(12);
  // B. floors, remaining, keys, first 11-bit digit
  uint64_t csum = 0, npos = 0;
  for (int j = (int)threadIdx.x; j < nocc; j += BS) {
    const int b = sh.occ[j];
    const uint32_t n = sh.nb[b];
    uint32_t c;
    uint64_t key;
    fast_floor_key(sh.wb[b], S, c, key);
    csum += (uint64_t)n * c;
    sh.kb[b] = (uint32_t)(key >> 32);
    if (key) {
      npos += n;
      atomicAdd((unsigned long long*)&rh[key >> 53], (unsigned long long)n | (1ull << 32));
    }
  }
  {  // one reduction for both: the floor sum is at most M, npos at most 2^20
    const uint64_t both = block_sum<uint64_t>(csum | (npos << 32), sh.bs);
    csum = both & 0xffffffffull;
    npos = both >> 32;
  }
  const int64_t remaining = (int64_t)kMass - (int64_t)csum;
  if (remaining < 0 || remaining >= (int64_t)kMass || remaining > (int64_t)npos) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  DSPARK_PHASE(13);
  // C. threshold over entries weighted by their counts: 11-bit digits, the
  // first 32 key bits from kb, lower ones recomputed
  enum { NONE = 0, ALL = 1, CAND = 2, EXACT = 3 };
  int mode = NONE;
  uint64_t prefix = 0, pmask = 0, need = (uint64_t)remaining;
  if (remaining > 0) {
    int shift = 53, nd = 2048;
    for (;;) {
      uint64_t before;
      const int d = vd_find_digit(rh, nd, need, sh, &before);
      need -= before;
      const uint64_t e = rh[d];
      prefix |= (uint64_t)d << shift;
      pmask |= (uint64_t)(nd - 1) << shift;
      if ((e & 0xffffffffull) == need) { mode = ALL; break; }
      if ((e >> 32) <= (uint64_t)kVdCand) { mode = CAND; break; }
      if (shift == 0) { mode = EXACT; break; }  // entries with equal keys: the general path decides
      __syncthreads();  // every thread has read rh[d] before it is cleared for the next digit
      const int nsh = shift > 11 ? shift - 11 : 0;
      nd = 1 << (shift - nsh);
      shift = nsh;
      for (int dd = (int)threadIdx.x; dd < nd; dd += BS) rh[dd] = 0ull;
      __syncthreads();
      for (int j = (int)threadIdx.x; j < nocc; j += BS) {
        const int b = sh.occ[j];
        const uint32_t n = sh.nb[b];
        if (sh.kb[b]) {
          uint64_t key = (uint64_t)sh.kb[b] << 32;
          if (shift < 32) {
            uint32_t c;
            fast_floor_key(sh.wb[b], S, c, key);
          }
          if ((key & pmask) == prefix)
            atomicAdd((unsigned long long*)&rh[(key >> shift) & (uint64_t)(nd - 1)],
                      (unsigned long long)n | (1ull << 32));
        }
      }
      __syncthreads();
    }
  }
  if (mode == EXACT) {
    res.status = kStGeneral;
    return res;
  }
  DSPARK_PHASE(14);
  // D. final count of every entry; the threshold bucket's entries wait (CAND)
  for (int j = (int)threadIdx.x; j < nocc; j += BS) {
    const int b = sh.occ[j];
    uint32_t c;
    uint64_t key;
    fast_floor_key(sh.wb[b], S, c, key);
    const bool pos = key != 0ull && mode != NONE;
    const uint64_t kp = key & pmask;
    const bool above = pos && kp > prefix, inb = pos && kp == prefix;
    if (inb && mode == CAND) {
      const int slot = atomicAdd(&sh.bi[4], 1);
      sh.ckey[slot] = key;
      sh.cbin[slot] = (uint32_t)b;
    } else {
      sh.nb[b] = c + ((above || (inb && mode == ALL)) ? 1u : 0u);
    }
  }
  __syncthreads();
  DSPARK_PHASE(15);
  // E. the threshold bucket's entries (CAND): exact weighted threshold
  uint64_t need_t = need;
  int ntie = 0;
  int tie_bin = -1;
  if (mode == CAND) {
    const int nc = sh.bi[4];
    const int j = (int)threadIdx.x;
    uint64_t kj = 0, above = 0, eq = 0;
    uint32_t bj = 0;
    if (j < nc) {
      kj = sh.ckey[j];
      bj = sh.cbin[j];
      for (int i = 0; i < nc; ++i) {
        const uint64_t ki = sh.ckey[i];
        const uint32_t ni = sh.nb[sh.cbin[i]];
        if (ki > kj) above += ni;
        if (ki == kj) eq += ni;
      }
    }
    if ((int)threadIdx.x == 0) sh.bi[5] = 0;
    __syncthreads();
    const bool is_t = j < nc && above < need && need <= above + eq;
    if (is_t) {  // every entry of the threshold key writes the same values
      sh.bu[2] = kj;
      sh.bu[3] = need - above;
      if (need - above < eq) atomicAdd(&sh.bi[5], 1);
    }
    __syncthreads();
    const uint64_t T = sh.bu[2];
    need_t = sh.bu[3];
    ntie = sh.bi[5];
    uint32_t c = 0;
    uint64_t key;
    if (j < nc) fast_floor_key(sh.wb[bj], S, c, key);
    __syncthreads();
    if (j < nc) {
      const bool partial = kj == T && ntie > 0;
      sh.nb[bj] = c + (!partial && kj >= T ? 1u : 0u);
      if (partial) sh.bi[6] = (int)bj;
    }
    __syncthreads();
    if (ntie == 1) tie_bin = sh.bi[6];
    __syncthreads();
  }
  if (ntie > 1) {  // several entries with the threshold key: the general path decides
    res.status = kStGeneral;
    return res;
  }
  DSPARK_PHASE(16);
  // F. a split tie: the need_t lowest ids among the members of the tie
  // entry (the registers hold table offsets)
  const char* nbb = reinterpret_cast<const char*>(sh.nb);
  const uint32_t T4 = (uint32_t)(tie_bin < 0 ? 0 : tie_bin * 4);
  int cut = -1;
  if (tie_bin >= 0) cut = tie_locate(R, T4, (uint32_t)(need_t - 1), sh);
  DSPARK_PHASE(17);
  // G. counts of every element: the entry's count, plus one for the members of
  // a tie entry at or below the cut.  Each 16-lane row of a wave sums its
  // counts of every vector into a cell; the cells, in id order (vector, wave,
  // row), give the total and locate the draw.
  uint32_t* cells = sh.hist;  // NI * NW * 4 cells
  touch(R);
  const int nvec = (V + 7) >> 3;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
  const bool row_lead = (lane_id() & 15) == 0;
  const int cell0 = wave_id() * 4 + (lane_id() >> 4);
  auto counts8 = [&](u32x4 v, int q, uint32_t (&c)[8]) {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[2 * k] = *reinterpret_cast<const uint32_t*>(nbb + (wv[k] & 0xffffu));
      c[2 * k + 1] = *reinterpret_cast<const uint32_t*>(nbb + (wv[k] >> 16));
    }
    const int lim = cut - q * 8;  // lanes l <= lim are at or below the cut
    if (lim >= 7) {  // the whole vector: every member of the tie entry
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[2 * k] += (uint16_t)wv[k] == (uint16_t)T4 ? 1u : 0u;
        c[2 * k + 1] += (uint16_t)(wv[k] >> 16) == (uint16_t)T4 ? 1u : 0u;
      }
    } else if (lim >= 0) {  // the vector of the cut
      const uint32_t m = eq16_mask8(v, T4 * 0x10001u) & ((2u << lim) - 1u);
#pragma unroll
      for (int l = 0; l < 8; ++l) c[l] += (m >> l) & 1u;
    }
  };
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = i * BS + (int)threadIdx.x;
    uint32_t c[8];
    counts8(fetch(R, i), q, c);
    {
      // The four lanes of a quad hold four consecutive vectors (128 bytes of
      // counts).  They trade halves with DPP so that each store instruction
      // writes whole 64-byte pieces: the first one vectors 4j and 4j + 1, the
      // second 4j + 2 and 4j + 3; lane l of the quad takes half (l & 1) of
      // lane (l & 3) >> 1 (then of 2 + ((l & 3) >> 1)).  Whole pieces go out
      // as streaming stores with no partial writes (storing each lane's own
      // 32 bytes instead fills half of every piece per instruction).
      const uint32_t l4 = threadIdx.x & 3u;
      const bool hi = (l4 & 1u) != 0u;
      uint32_t f[4], g[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a0 = dpp_t<0x50, 0xf, 0xf>(0u, c[k]), a1 = dpp_t<0x50, 0xf, 0xf>(0u, c[k + 4]);  // quad_perm 0,0,1,1
        const uint32_t b0 = dpp_t<0xfa, 0xf, 0xf>(0u, c[k]), b1 = dpp_t<0xfa, 0xf, 0xf>(0u, c[k + 4]);  // quad_perm 2,2,3,3
        f[k] = hi ? a1 : a0;
        g[k] = hi ? b1 : b0;
      }
      const int q4 = q & ~3;
      if (!drow) {
        // no count row wanted: the counts only feed the cells of the draw
      } else if (q4 * 8 + 32 <= V && vec_ok) {  // the quad's four vectors are whole
        char* dst = reinterpret_cast<char*>(drow + (size_t)q4 * 8) + l4 * 16;
        __builtin_nontemporal_store(u32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(u32x4{g[0], g[1], g[2], g[3]}, reinterpret_cast<u32x4*>(dst + 64));
      } else if (q < nvec) {  // the ragged end of the row: element by element
#pragma unroll
        for (int l = 0; l < 8; ++l)
          if (q * 8 + l < V) drow[(size_t)q * 8 + l] = c[l];
      }
    }
    uint32_t vs = 0;  // at most 2^31 in a row of 16 lanes (every count <= M)
#pragma unroll
    for (int l = 0; l < 8; ++l) vs += c[l];
    vs += dpp_t<0xb1, 0xf, 0xf>(0u, vs);   // quad_perm 1,0,3,2
    vs += dpp_t<0x4e, 0xf, 0xf>(0u, vs);   // quad_perm 2,3,0,1
    vs += dpp_t<0x141, 0xf, 0xf>(0u, vs);  // row_half_mirror
    vs += dpp_t<0x140, 0xf, 0xf>(0u, vs);  // row_mirror: the row's sum in every lane
    if (row_lead) cells[i * (NW * 4) + cell0] = vs;
  }
  __syncthreads();
  // H. wave 0: the total, and the cell whose running count passes u (lane l
  // takes cells 16 l .. 16 l + 15)
  if (threadIdx.x < 64) {
    const int l = lane_id();
    uint64_t s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += cells[16 * l + j];
    const uint64_t inc = wave_incl_scan(s);
    if (l == 63) sh.bu[0] = inc;
    if (l == 0) sh.bi[2] = -1;  // the sample's element (written by one lane below)
    if (want_s) {
      const uint64_t hit = __ballot(inc > (uint64_t)u);
      if (l == 0) sh.bi[1] = -1;
      if (hit != 0ull && l == __builtin_ctzll(hit)) {
        uint64_t run = inc - s;
        int cell = -1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t cj = cells[16 * l + j];
          if (cell < 0 && run + cj > (uint64_t)u) cell = 16 * l + j;
          if (cell < 0) run += cj;
        }
        sh.bi[1] = cell;
        sh.bu[1] = run;  // counts before the cell
      }
    }
  }
  __syncthreads();
  if (sh.bu[0] != kMass) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  DSPARK_PHASE(18);
  // the sample: the 16 lanes of the draw's cell recompute their counts of its
  // vector and scan them
  if (want_s) {
    const int cell = sh.bi[1];
    if (cell >= 0 && wave_id() == ((cell >> 2) & (NW - 1)) && (lane_id() >> 4) == (cell & 3)) {
      const int i = cell / (NW * 4);
      const int q = i * BS + (int)threadIdx.x;
      uint32_t c[8];
      counts8(select_vec(R, i), q, c);
      uint32_t vs = 0;
#pragma unroll
      for (int l = 0; l < 8; ++l) vs += c[l];
      uint32_t inc = vs;  // inclusive scan over the 16 lanes of the row
      inc += dpp_t<0x111, 0xf, 0xf>(0u, inc);  // row_shr:1
      inc += dpp_t<0x112, 0xf, 0xf>(0u, inc);  // row_shr:2
      inc += dpp_t<0x114, 0xf, 0xf>(0u, inc);  // row_shr:4
      inc += dpp_t<0x118, 0xf, 0xf>(0u, inc);  // row_shr:8
      const uint32_t u2 = (uint32_t)((uint64_t)u - sh.bu[1]);
      const uint32_t pre = inc - vs;
      if (pre <= u2 && u2 < inc) {
        uint32_t run = pre;
        int hit = -1;
#pragma unroll
        for (int l = 0; l < 8; ++l) {
          run += c[l];
          if (run > u2 && hit < 0) hit = l;
        }
        sh.bi[2] = q * 8 + hit;
      }
    }
    __syncthreads();
    res.token = sh.bi[2];
    if (res.token < 0) res.status = DSPARK_ST_ALLOC_INCONSISTENT;
  }
  return res;
}

// --------------------------------------------------------------- sparse
// Candidates of vector v above a positive threshold: raw bf16 patterns
// compare like signed 16-bit integers for positive values, and negative
// values (sign bit set) are below.  Returns the four sign words: bit 15 / 31
// of word c set for the low / high element of word c when it is a candidate.
__device__ __forceinline__ void cand_words(u32x4 v, uint32_t rl2, uint32_t (&s)[4]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const s16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(s16x2, w[c]), __builtin_bit_cast(s16x2, rl2));
    s[c] = ~__builtin_bit_cast(uint32_t, d) & 0x80008000u;
  }
}

// The same test as an 8-bit mask in a fixed permuted order: bits 3..0 are
// the low halves of words 0..3 (elements 0, 2, 4, 6) and bits 7..4 the high
// halves of words 0..3 (elements 1, 3, 5, 7); cand_elem maps a bit back.
__device__ __forceinline__ uint32_t cand_mask8(u32x4 v, uint32_t rl2) {
  uint32_t s[4];
  cand_words(v, rl2, s);
  const uint32_t t = s[0] | (s[1] >> 1) | (s[2] >> 2) | (s[3] >> 3);
  return ((t >> 12) & 0xfu) | ((t >> 24) & 0xf0u);
}
__device__ __forceinline__ int cand_elem(int b) { return b < 4 ? 6 - 2 * b : 15 - 2 * b; }

// Support of the top-k by (logit desc, id asc) into (sh.cid, sh.sx) in
// ascending id order, from the table (already filled by fast_hist).
// Returns the support size, or -1 when the exact multi-pass selection must
// decide: the threshold falls inside the collapsed entry (whose members are
// distinct values) and takes only part of it, or takes all of a collapsed
// entry too large for the candidate list.  Entries below the weight window
// would all get count 0 and be dropped, so the support is taken inside the
// window.
// Wave 0 (all 64 lanes): walks the table from its largest entry in chunks
// of 256 (four consecutive entries per lane) until the running count reaches
// `target`.  Returns the entry where it does (-1 if the whole table holds
// fewer) with *before = the count of the entries above it; *seen = the count
// walked (the table total when -1).  The top-k threshold of a row sits in the
// first few chunks.
__device__ __forceinline__ int wave0_top_crossing(const uint32_t* nb, int NB, uint32_t target, uint32_t* before,
                                                  uint32_t* seen) {
  const int l = threadIdx.x & 63;
  uint32_t run = 0;
  for (int base = 0; base < NB; base += 256) {
    const int e = base + 4 * l;
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = e + i < NB ? nb[e + i] : 0u;
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    const uint32_t inc = wave_incl_scan(s);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    if (run + total >= target) {  // the crossing is in this chunk, in the first lane that reaches it
      const uint64_t hit = __ballot(run + inc >= target);
      const int lc = __builtin_ctzll(hit);
      uint32_t r = run + (uint32_t)__builtin_amdgcn_readlane((int)(inc - s), lc);
      int ent = -1;
      uint32_t bef = 0;
      if (l == lc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (ent < 0 && r + c[i] >= target) {
            ent = e + i;
            bef = r;
          }
          r += c[i];
        }
      }
      *before = (uint32_t)__builtin_amdgcn_readlane((int)bef, lc);
      *seen = run + total;
      return __builtin_amdgcn_readlane(ent, lc);
    }
    run += total;
  }
  *before = run;
  *seen = run;
  return -1;
}

__device__ __forceinline__ int fast_topk(Res& R, const FMap& f, int k, FastSparseShared& sh DSPARK_PHASE_PARAM) {
  // the threshold entry: where the count from the top reaches k, or, when the
  // window holds fewer than k elements, the last occupied entry
  if (threadIdx.x < 64) {
    uint32_t before, seen;
    int ent = wave0_top_crossing(sh.nb, f.NB, (uint32_t)k, &before, &seen);
    uint32_t need = (uint32_t)k;
    if (ent < 0) {
      need = seen;
      ent = need > 0 ? wave0_top_crossing(sh.nb, f.NB, need, &before, &seen) : -1;
    }
    if (threadIdx.x == 0) {
      sh.bu[0] = need;
      sh.bi[0] = ent;
      sh.bu[1] = before;
    }
  }
  __syncthreads();
  const uint64_t need = sh.bu[0];
  if (need == 0) return 0;
  const int bT = sh.bi[0];
  const uint64_t before = sh.bu[1];
  const uint32_t nT = sh.nb[bT];
  const uint32_t need_t = (uint32_t)(need - before);
  if (bT == f.B0 && f.tb1 > 0 && nT != need_t) return -1;
  // keys (K16) of the smallest and largest values of the threshold entry
  const bool coll = bT == f.B0 && f.tb1 > 0;
  const int Klo = coll ? k16(0x8000u | (uint32_t)f.tb1) : k16(fmap_raw(bT, f));
  const int Khi = coll ? k16((uint32_t)f.tb1) : Klo;
  // a threshold entry too large for the candidate list: its members go
  // straight from the registers into bitmap B, the list takes only the
  // elements above it (fewer than k).  The collapsed entry holds distinct
  // values, so there the exact multi-pass selection decides.
  const bool big = before + nT > (uint64_t)kCandCap;
  if (big && coll) return -1;
  const int Kc = big ? Khi + 1 : Klo;  // candidates: every element with key >= Kc
  DSPARK_PHASE(1);
  // candidates: per-thread masks of the sixteen vectors (kept in four
  // registers), one block scan for each thread's base, then the writes
  for (int w = threadIdx.x; w < NI * NW * 16; w += BS) {
    sh.bmA[w] = 0u;
    if (!big) sh.bmB[w] = 0u;
  }
  const bool posT = Kc > 0x8000;
  const uint32_t rl2 = posT ? (uint32_t)(Kc - 0x8000) * 0x10001u : 0u;
  const uint32_t T2 = fmap_raw(bT, f) * 0x10001u;
  const bool tz = Klo == 0x8000;
  uint8_t* bmb = reinterpret_cast<uint8_t*>(sh.bmB);  // byte q: elements 8q..8q+7
  uint32_t M[4] = {0u, 0u, 0u, 0u};
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = fetch(R, i);
    const uint32_t m8 = posT ? cand_mask8(v, rl2) : ge_mask(v, Kc);
    M[i >> 2] |= m8 << (8 * (i & 3));
    if (big) bmb[i * BS + (int)threadIdx.x] = (uint8_t)eq16_mask8(v, T2, tz ? 0x7fff7fffu : 0xffffffffu);
  }
  const uint32_t tot = (uint32_t)(__builtin_popcount(M[0]) + __builtin_popcount(M[1]) + __builtin_popcount(M[2]) +
                                  __builtin_popcount(M[3]));
  uint32_t nc;
  uint32_t pos = block_excl_scan<uint32_t>(tot, sh.bs, &nc);
  DSPARK_PHASE(27);
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    uint32_t m8 = (M[i >> 2] >> (8 * (i & 3))) & 0xffu;
    if (m8) {  // candidates stored as (raw bf16 << 32 | id)
      const u32x4 v = fetch(R, i);
      const uint32_t base = (uint32_t)((i * BS + (int)threadIdx.x) * 8);
      do {
        const int bt = __builtin_ctz(m8);
        m8 &= m8 - 1u;
        const int e = posT ? cand_elem(bt) : bt;
        const uint32_t wd = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
        const uint32_t raw = (e & 1) ? wd >> 16 : wd & 0xffffu;
        if (pos < (uint32_t)kCandCap) sh.ckey[pos] = ((uint64_t)raw << 32) | (uint64_t)(base + (uint32_t)e);
        ++pos;
      } while (m8);
    }
  }
  __syncthreads();
  DSPARK_PHASE(26);
  if (nc > (uint32_t)kCandCap) nc = kCandCap;
  // bitmaps over ids: A = above the threshold entry, B = its members
  for (int e = threadIdx.x; e < (int)nc; e += BS) {
    const uint64_t ck = sh.ckey[e];
    const int K = k16((uint32_t)(ck >> 32));
    const uint32_t id = (uint32_t)ck;
    atomicOr(K > Khi ? &sh.bmA[id >> 5] : &sh.bmB[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  DSPARK_PHASE(2);
  // the need_t lowest ids of B join A, and the per-word prefix of the joined
  // A in sh.hist, from one scan of both counts: A and B are disjoint, so
  // before word j the joined A holds preA + min(preB, need_t) ids
  {
    const int w0 = threadIdx.x * 4;
    uint32_t aw[4], bw[4];
    uint64_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      aw[j] = sh.bmA[w0 + j];
      bw[j] = sh.bmB[w0 + j];
      s += (uint64_t)__builtin_popcount(aw[j]) | ((uint64_t)__builtin_popcount(bw[j]) << 32);
    }
    uint64_t t;
    const uint64_t pre = block_excl_scan<uint64_t>(s, sh.bs, &t);
    uint32_t preA = (uint32_t)pre, preB = (uint32_t)(pre >> 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t keep = bw[j];
      const uint32_t pb = (uint32_t)__builtin_popcount(bw[j]);
      if (preB >= need_t) {
        keep = 0u;
      } else if (preB + pb > need_t) {  // keep the first need_t - preB members of this word
        uint32_t rem = need_t - preB, m = bw[j];
        keep = 0u;
        while (rem) {
          const uint32_t low = m & (0u - m);
          keep |= low;
          m ^= low;
          --rem;
        }
      }
      sh.hist[w0 + j] = preA + (preB < need_t ? preB : need_t);
      sh.bmA[w0 + j] = aw[j] | keep;
      preA += (uint32_t)__builtin_popcount(aw[j]);
      preB += pb;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < (int)nc; e += BS) {
    const uint64_t ck = sh.ckey[e];
    const uint32_t id = (uint32_t)ck;
    const uint32_t wd = sh.bmA[id >> 5];
    if (wd & (1u << (id & 31))) {
      const uint32_t r = sh.hist[id >> 5] + (uint32_t)__builtin_popcount(wd & ((1u << (id & 31)) - 1u));
      if (r >= (uint32_t)DSPARK_K_MAX) continue;  // cannot happen: |A| = need <= k
      sh.cid[r] = id;
      sh.sx[r] = bf16_to_f32((uint32_t)(ck >> 32));
    }
  }
  if (big) {  // the chosen members of the threshold entry: in A and in B, not in the list
    const float xT = bf16_to_f32(fmap_raw(bT, f));
    const int w0 = threadIdx.x * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = sh.bmA[w0 + j], h = sh.hist[w0 + j];
      uint32_t sel = a & sh.bmB[w0 + j];
      while (sel) {
        const int bt = __builtin_ctz(sel);
        sel &= sel - 1u;
        const uint32_t r = h + (uint32_t)__builtin_popcount(a & ((1u << bt) - 1u));
        if (r < (uint32_t)DSPARK_K_MAX) {
          sh.cid[r] = (uint32_t)((w0 + j) * 32 + bt);
          sh.sx[r] = xT;
        }
      }
    }
  }
  __syncthreads();
  DSPARK_PHASE(3);
  return (int)need;
}

}  // namespace dspark
