// Dense dyadic24 counts of a register-resident bf16 row, computed per
// distinct logit value ("PP1 q transport and scheduling design",
// "Distribution contract and precision").
//
// Every quantity of the allocation before the tie-break -- d = RN32(x - m),
// w = RN32(exp(d)), p = RN64(w / S64), the floor and the remainder -- is a
// function of the logit value alone.  A bf16 row has at most 33,957 distinct
// values in the window [m - 105, m] (values below it have weight 0), so the
// row is histogrammed by value into an LDS table indexed by key distance from
// the maximum, the binary64 work runs once per occupied bin, the
// largest-remainder threshold is found over bins weighted by their counts,
// and a split tie at the threshold is cut by element index.  A last pass over
// the registers writes every count.  The result is the same function of the
// row as the per-element definition.
#pragma once
#include "resident.hpp"

namespace dspark {

constexpr int kBinsMax = 34048;  // >= 33,957 distinct bf16 values in any [m - 105, m]
constexpr int kVdCand = 256;     // bins a threshold bucket may hold to be resolved in LDS
constexpr uint32_t kTieFlag = 1u << 30;

struct DenseShared : SmemBase {
  uint64_t ckey[kVdCand];
  uint32_t cbin[kVdCand];
  uint32_t bins[kBinsMax];
};

// weight of bin b: the logit with key Km - b
__device__ __forceinline__ float vd_weight(int Km, int b, float m) {
  return cr_expf(bf16_to_f32(bf16_of_k16(Km - b)) - m);
}

// Per-element bin lookup of one vector: counts for its 8 lanes.
__device__ __forceinline__ void vd_counts(u32x4 v, int Km, int NB, int base, int cut, const DenseShared& sh,
                                          uint32_t (&c)[8]) {
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    const int bin = Km - k16(elem(v, l));
    uint32_t x = 0;
    if ((unsigned)bin < (unsigned)NB) {
      const uint32_t t = sh.bins[bin];
      x = (t & (kTieFlag - 1u)) + (((t & kTieFlag) && base + l <= cut) ? 1u : 0u);
    }
    c[l] = x;
  }
}

// Crossing over a uint64 digit histogram (low 32 bits: element count, high 32
// bits: bin count), from the highest digit down.  Returns the digit; *before
// is the element count above it.
__device__ __forceinline__ int vd_find_digit(const uint64_t* rh, int nd, uint64_t need, SmemBase& sh,
                                             uint64_t* before) {
  const int per = (nd + BS - 1) / BS;
  uint64_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int pos = threadIdx.x * per + i;
    if (pos < nd) s += rh[nd - 1 - pos] & 0xffffffffull;
  }
  uint64_t tot;
  const uint64_t pre = block_excl_scan<uint64_t>(s, sh.bs, &tot);
  if (pre < need && need <= pre + s) {
    uint64_t run = pre;
    for (int i = 0; i < per; ++i) {
      const int d = nd - 1 - (threadIdx.x * per + i);
      const uint64_t c = rh[d] & 0xffffffffull;
      if (run + c >= need) {
        sh.bi[0] = d;
        sh.bu[0] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  const int d = sh.bi[0];
  *before = sh.bu[0];
  return d;  // (bi[0] and bu[0] are written again only after later barriers)
}

__device__ __forceinline__ QOut res_dense_q(Res& R, const RStats& st, uint32_t* drow, int V, bool want_s,
                                            uint32_t u, DenseShared& sh DSPARK_PHASE_PARAM) {
  QOut res{DSPARK_ST_OK, 0};
  const int Km = k16(st.m_raw);
  const float m = bf16_to_f32(st.m_raw);
  int Klo;
  {  // key of the smallest bf16 >= m - 105 (binary32), never below the smallest finite value
    const uint32_t b = __float_as_uint(m - 105.0f);
    uint32_t hb = b >> 16;
    if ((b & 0xffffu) && !(b & 0x80000000u)) hb += 1u;
    Klo = k16(hb & 0xffffu);
    if (Klo < kKeyNegInf + 1) Klo = kKeyNegInf + 1;
    if (Km - Klo + 1 > kBinsMax) Klo = Km - kBinsMax + 1;
  }
  const int NB = Km - Klo + 1;
  for (int b = threadIdx.x; b < NB; b += BS) sh.bins[b] = 0u;
  __syncthreads();
  // 1. histogram of the row by value
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = fetch(R, i);
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const int bin = Km - k16(elem(v, l));
      if ((unsigned)bin < (unsigned)NB) atomicAdd(&sh.bins[bin], 1u);
    }
  }
  __syncthreads();
  DSPARK_PHASE(11);
  // 2. weights and their exact sum, per occupied bin
  Acc acc;
  acc_zero(acc);
  for (int b = threadIdx.x; b < NB; b += BS) {
    const uint32_t n = sh.bins[b];
    if (n) acc_add(acc, __float_as_uint(vd_weight(Km, b, m)), n);
  }
  const double s64 = block_acc_rn64(acc, sh.acc);
  const SumR S = sum_r(s64);
  if (!(s64 > 0.0)) {
    res.status = DSPARK_ST_ROW_ZERO_MASS;
    return res;
  }
  DSPARK_PHASE(12);
  // 3. floors, remaining, and the first 11-bit digit of the remainder keys
  uint64_t* rh = reinterpret_cast<uint64_t*>(sh.hist);  // 2048 x uint64 in the 16 KB histogram
  for (int d = threadIdx.x; d < 2048; d += BS) rh[d] = 0ull;
  __syncthreads();
  uint64_t csum = 0, npos = 0;
  for (int b = threadIdx.x; b < NB; b += BS) {
    const uint32_t n = sh.bins[b];
    if (n) {
      uint32_t c;
      double r;
      floor_rem(vd_weight(Km, b, m), S, c, r);
      csum += (uint64_t)n * c;
      if (r > 0.0) {
        npos += n;
        atomicAdd((unsigned long long*)&rh[rem_key(r) >> 53], (unsigned long long)n | (1ull << 32));
      }
    }
  }
  csum = block_sum<uint64_t>(csum, sh.bs);
  npos = block_sum<uint64_t>(npos, sh.bs);
  const int64_t remaining = (int64_t)kMass - (int64_t)csum;
  if (remaining < 0 || remaining >= (int64_t)kMass || remaining > (int64_t)npos) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  DSPARK_PHASE(13);
  // 4. threshold over bins weighted by their counts: digits of 11 bits
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
      __syncthreads();
      prefix |= (uint64_t)d << shift;
      pmask |= (uint64_t)(nd - 1) << shift;
      if ((e & 0xffffffffull) == need) { mode = ALL; break; }
      if ((e >> 32) <= (uint64_t)kVdCand) { mode = CAND; break; }
      if (shift == 0) { mode = EXACT; break; }
      const int nsh = shift > 11 ? shift - 11 : 0;
      nd = 1 << (shift - nsh);
      shift = nsh;
      for (int dd = threadIdx.x; dd < nd; dd += BS) rh[dd] = 0ull;
      __syncthreads();
      for (int b = threadIdx.x; b < NB; b += BS) {
        const uint32_t n = sh.bins[b];
        if (n) {
          uint32_t c;
          double r;
          floor_rem(vd_weight(Km, b, m), S, c, r);
          const uint64_t key = rem_key(r);
          if (r > 0.0 && (key & pmask) == prefix)
            atomicAdd((unsigned long long*)&rh[(key >> shift) & (uint64_t)(nd - 1)],
                      (unsigned long long)n | (1ull << 32));
        }
      }
      __syncthreads();
    }
  }
  DSPARK_PHASE(14);
  // 5. mark every occupied bin with its final count (candidates wait)
  if (threadIdx.x == 0) sh.bi[4] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += BS) {
    const uint32_t n = sh.bins[b];
    if (n) {
      uint32_t c;
      double r;
      floor_rem(vd_weight(Km, b, m), S, c, r);
      const uint64_t kp = r > 0.0 ? (rem_key(r) & pmask) : 0ull;
      const bool pos = r > 0.0 && mode != NONE;
      const bool above = pos && kp > prefix, inb = pos && kp == prefix;
      if (inb && mode == CAND) {
        const int slot = atomicAdd(&sh.bi[4], 1);
        sh.ckey[slot] = rem_key(r);
        sh.cbin[slot] = (uint32_t)b;
      } else if (inb && mode == EXACT) {
        sh.bins[b] = kTieFlag | c;
      } else {
        sh.bins[b] = c + ((above || (inb && mode == ALL)) ? 1u : 0u);
      }
    }
  }
  __syncthreads();
  DSPARK_PHASE(15);
  // 6. candidates of the threshold bucket: exact weighted threshold in LDS
  uint64_t need_t = need;
  int ntie_bins = mode == EXACT ? 2 : 0;  // EXACT: tie bins found through the table
  int tie_bin = -1;
  if (mode == CAND) {
    const int nc = sh.bi[4];
    const int j = threadIdx.x;
    uint64_t kj = 0, above = 0, eq = 0;
    uint32_t nj = 0, bj = 0;
    if (j < nc) {
      kj = sh.ckey[j];
      bj = sh.cbin[j];
      nj = sh.bins[bj];
      for (int i = 0; i < nc; ++i) {
        const uint64_t ki = sh.ckey[i];
        const uint32_t ni = sh.bins[sh.cbin[i]];
        if (ki > kj) above += ni;
        if (ki == kj) eq += ni;
      }
    }
    if (threadIdx.x == 0) sh.bi[5] = 0;
    __syncthreads();
    const bool is_t = j < nc && above < need && need <= above + eq;
    if (is_t) {  // every candidate of the threshold key writes the same values
      sh.bu[2] = kj;
      sh.bu[3] = need - above;
      if (need - above < eq) atomicAdd(&sh.bi[5], 1);
    }
    __syncthreads();
    const uint64_t T = sh.bu[2];
    need_t = sh.bu[3];
    ntie_bins = sh.bi[5];
    uint32_t c = 0;
    double r = 0.0;
    if (j < nc) floor_rem(vd_weight(Km, (int)bj, m), S, c, r);
    __syncthreads();
    if (j < nc) {
      const bool partial = kj == T && ntie_bins > 0;
      sh.bins[bj] = partial ? (kTieFlag | c) : c + ((kj > T || kj == T) ? 1u : 0u);
      if (partial) sh.bi[6] = (int)bj;
    }
    __syncthreads();
    if (ntie_bins == 1) tie_bin = sh.bi[6];
    __syncthreads();
  }
  DSPARK_PHASE(16);
  // 7. a split tie: the need_t lowest ids among the elements of the tie bins
  int cut = -1;
  if (ntie_bins > 0) {
    const bool one = tie_bin >= 0;
    const int Kt = Km - tie_bin;
    cut = res_locate(R, [&](int, u32x4 v) -> uint32_t {
      uint32_t msk = 0;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        const int K = k16(elem(v, l));
        const int bin = Km - K;
        const bool t = one ? K == Kt : ((unsigned)bin < (unsigned)NB && (sh.bins[bin] & kTieFlag));
        msk |= (t ? 1u : 0u) << l;
      }
      return msk;
    }, (uint32_t)(need_t - 1), sh);
  }
  DSPARK_PHASE(17);
  // 8. counts of every element, written in place of the row
  if (threadIdx.x < NI) sh.tab[threadIdx.x] = 0ull;
  __syncthreads();
  touch(R);
  const int nvec = (V + 7) >> 3;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
  uint64_t total = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = i * BS + (int)threadIdx.x;
    uint32_t c[8];
    vd_counts(fetch(R, i), Km, NB, q * 8, cut, sh, c);
    uint32_t vs = 0;
#pragma unroll
    for (int l = 0; l < 8; ++l) vs += c[l];
    if (drow && q < nvec) {  // no count row wanted: the counts only feed the draw
      if (q * 8 + 8 <= V && vec_ok) {
        u32x4* dst = reinterpret_cast<u32x4*>(drow + (size_t)q * 8);
        // plain (write-back) stores: each instruction fills half of every
        // 32-byte piece it touches, and L2 merges the two halves before the
        // line goes out; streaming stores left part of them as separate
        // partial writes (about a quarter more HBM write traffic)
        dst[0] = u32x4{c[0], c[1], c[2], c[3]};
        dst[1] = u32x4{c[4], c[5], c[6], c[7]};
      } else {
#pragma unroll
        for (int l = 0; l < 8; ++l)
          if (q * 8 + l < V) drow[(size_t)q * 8 + l] = c[l];
      }
    }
    total += vs;
    if (want_s && __ballot(vs != 0u)) {
      const uint32_t w = wave_sum(vs);
      if (lane_id() == 0 && w) atomicAdd((unsigned long long*)&sh.tab[i], (unsigned long long)w);
    }
  }
  total = block_sum<uint64_t>(total, sh.bs);
  if (total != kMass) {
    res.status = DSPARK_ST_ALLOC_INCONSISTENT;
    return res;
  }
  DSPARK_PHASE(18);
  // 9. the sample: first element whose running count exceeds u; the counts
  // of the vector holding it are recomputed from the registers
  if (want_s) {
    if (threadIdx.x == 0) {
      uint64_t run = 0;
      sh.bi[1] = -1;
      for (int i = 0; i < NI; ++i) {
        if (run + sh.tab[i] > u) {
          sh.bi[1] = i;
          sh.bu[1] = run;
          break;
        }
        run += sh.tab[i];
      }
    }
    __syncthreads();
    const int istar = sh.bi[1];
    const uint64_t u2 = (uint64_t)u - sh.bu[1];
    const int q = istar * BS + (int)threadIdx.x;
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (istar >= 0) vd_counts(select_vec(R, istar), Km, NB, q * 8, cut, sh, c);
    uint32_t vs = 0;
#pragma unroll
    for (int l = 0; l < 8; ++l) vs += c[l];
    uint64_t tot;
    const uint64_t pre = block_excl_scan<uint64_t>(vs, sh.bs, &tot);
    if (istar >= 0 && vs && pre <= u2 && u2 < pre + vs) {
      uint64_t run = pre;
      int hit = -1;
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        run += c[l];
        if (run > u2 && hit < 0) hit = l;
      }
      sh.bi[2] = q * 8 + hit;
    }
    __syncthreads();
    res.token = istar >= 0 ? sh.bi[2] : -1;
    __syncthreads();
    if (res.token < 0) res.status = DSPARK_ST_ALLOC_INCONSISTENT;
  }
  return res;
}

}  // namespace dspark
