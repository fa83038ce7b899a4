// Sparse top-k support of a register-resident bf16 row ("Sparse support and
// vocabulary-sharded TP2 follow-up": global support first, deterministic
// ties -- here logit descending, then token id ascending).
//
// 1. Each thread's eight packed per-position maxima are eight of its
//    elements; the k-th largest of these 8192 values is a lower bound `lo`
//    for the k-th largest logit (k of them are at least lo).
// 2. One pass over the registers appends every element >= lo to an LDS
//    candidate list (about 1 % of a row for the configurations here).
// 3. The k-th largest candidate (and, inside a tie at that value, the
//    lowest ids) is found in LDS.
// 4. A bitmap over token ids turns the selected candidates into ascending id
//    order without sorting.
// Rows whose candidates overflow the list (long runs of equal values) take
// the exact multi-pass selection res_topk_support instead.
#pragma once
#include "resident.hpp"

namespace dspark {

// first bin b (ascending) at which the running count reaches need; one wave
// scans `nbins` bins, 64 lanes x (nbins / 64) consecutive bins each
__device__ __forceinline__ void wave0_crossing_asc(const uint32_t* hist, int nbins, uint32_t need, SmemBase& sh) {
  if (threadIdx.x < 64) {
    const int per = nbins / 64;
    const int l = lane_id();
    uint32_t s = 0;
    for (int j = 0; j < per; ++j) s += hist[l * per + j];
    const uint32_t inc = wave_incl_scan(s);
    const uint32_t pre = inc - s;
    if (threadIdx.x == 0) sh.bi[0] = nbins - 1;
    if (pre < need && need <= inc) {
      uint32_t run = pre;
      for (int j = 0; j < per; ++j) {
        const uint32_t c = hist[l * per + j];
        if (run + c >= need) {
          sh.bi[0] = l * per + j;
          sh.bu[0] = run;
          break;
        }
        run += c;
      }
    }
  }
}

// Returns the support size n (entries in sh.cid / sh.sx, ascending id), or
// -1 when the candidates overflow the list.
__device__ __forceinline__ int res_topk_fast(Res& R, const RStats& st, int k, RowShared& sh DSPARK_PHASE_PARAM) {
  const int Km = k16(st.m_raw);
  // 1. lower bound from 8 representatives per thread (distance from the max)
  for (int b = threadIdx.x; b < kHistBins; b += BS) sh.hist[b] = 0;
  if (threadIdx.x == 0) sh.bi[4] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = Km - k16((st.rep[c] >> (16 * h)) & 0xffffu);
      atomicAdd(&sh.hist[d < kHistBins ? d : kHistBins - 1], 1u);
    }
  }
  __syncthreads();
  wave0_crossing_asc(sh.hist, kHistBins, (uint32_t)k, sh);
  __syncthreads();
  // a crossing in the last (clamped) bin bounds nothing: take every finite entry
  int lo = sh.bi[0] == kHistBins - 1 ? kKeyNegInf + 1 : Km - sh.bi[0];
  if (lo <= kKeyNegInf) lo = kKeyNegInf + 1;  // -inf entries never enter the support
  DSPARK_PHASE(1);
  // 2. candidates: every element with key >= lo, as (key << 32 | ~id)
  touch(R);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = fetch(R, i);
    const uint32_t msk = ge_mask(v, lo);
    // one LDS atomic per wave and vector: a wave-level exclusive scan of the
    // lanes' hit counts gives each lane its slot after the wave's base
    const uint32_t n = (uint32_t)__builtin_popcount(msk);
    if (__ballot(n != 0u)) {
      const uint32_t inc = wave_incl_scan(n);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      uint32_t wbase = 0;
      if (lane_id() == 63) wbase = (uint32_t)atomicAdd(&sh.bi[4], (int)wtot);
      wbase = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 63);
      int pos = (int)(wbase + inc - n);
      const uint32_t base = (uint32_t)((i * BS + (int)threadIdx.x) * 8);
#pragma unroll
      for (int l = 0; l < 8; ++l) {
        if (msk & (1u << l)) {
          if (pos < kCandCap)
            sh.ckey[pos] = ((uint64_t)k16(elem(v, l)) << 32) | (uint64_t)(0xffffffffu - (base + (uint32_t)l));
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  const int nc = sh.bi[4];
  if (nc > kCandCap) return -1;
  const uint32_t need = (uint32_t)(k < nc ? k : nc);  // fewer finite entries than k: all of them
  if (need == 0) return 0;
  DSPARK_PHASE(2);
  // 3. threshold key among the candidates: histogram of the distance from the max
  for (int b = threadIdx.x; b < kHistBins; b += BS) sh.hist[b] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < nc; e += BS) {
    const int d = Km - (int)(sh.ckey[e] >> 32);
    atomicAdd(&sh.hist[d < kHistBins ? d : kHistBins - 1], 1u);
  }
  __syncthreads();
  wave0_crossing_asc(sh.hist, kHistBins, need, sh);
  __syncthreads();
  const int bT = sh.bi[0];
  const uint32_t need_t = need - (uint32_t)sh.bu[0];
  const uint32_t cntT = sh.hist[bT];
  __syncthreads();
  if (bT == kHistBins - 1 && cntT != need_t) return -1;  // threshold beyond the histogram range
  const int T = Km - bT;  // one key unless bT is the clamped last bin (then every candidate there is taken)
  // tie at T: the need_t lowest ids among candidates with key T
  uint32_t cut = 0xffffffffu;  // ids <= cut selected among the tie
  if (cntT != need_t) {
    if (threadIdx.x == 0) sh.bi[5] = 0;
    __syncthreads();
    uint32_t* tie = sh.ctab;  // reused: at most kCandCap ids
    for (int e = threadIdx.x; e < nc; e += BS)
      if ((int)(sh.ckey[e] >> 32) == T) tie[atomicAdd(&sh.bi[5], 1)] = 0xffffffffu - (uint32_t)sh.ckey[e];
    __syncthreads();
    const int nt = sh.bi[5];
    for (int e = threadIdx.x; e < nt; e += BS) {
      const uint32_t id = tie[e];
      uint32_t rank = 0;
      for (int f = 0; f < nt; ++f) rank += tie[f] < id ? 1u : 0u;
      if (rank == need_t - 1) sh.bi[6] = (int)id;
    }
    __syncthreads();
    cut = (uint32_t)sh.bi[6];
    __syncthreads();
  }
  DSPARK_PHASE(3);
  // 4. ascending id order through a bitmap over the row (ctab: 4096 words)
  uint32_t* bm = sh.ctab;
  for (int w = threadIdx.x; w < NI * NW * 16; w += BS) bm[w] = 0u;
  __syncthreads();
  auto selected = [&](uint64_t ck) -> bool {  // clamped distance below bT, or the tie up to the cut
    const int d = Km - (int)(ck >> 32);
    const int dc = d < kHistBins ? d : kHistBins - 1;
    const uint32_t id = 0xffffffffu - (uint32_t)ck;
    return dc < bT || (dc == bT && id <= cut);
  };
  for (int e = threadIdx.x; e < nc; e += BS) {
    const uint64_t ck = sh.ckey[e];
    const uint32_t id = 0xffffffffu - (uint32_t)ck;
    if (selected(ck)) atomicOr(&bm[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  uint32_t wcnt[4];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wcnt[j] = (uint32_t)__builtin_popcount(bm[threadIdx.x * 4 + j]);
    s += wcnt[j];
  }
  uint32_t tot;
  uint32_t pre = block_excl_scan<uint32_t>(s, sh.bs, &tot);
  __syncthreads();
  // per-word prefix, kept in the histogram array (4096 words)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sh.hist[threadIdx.x * 4 + j] = pre;
    pre += wcnt[j];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nc; e += BS) {
    const uint64_t ck = sh.ckey[e];
    const int K = (int)(ck >> 32);
    const uint32_t id = 0xffffffffu - (uint32_t)ck;
    if (selected(ck)) {
      const uint32_t r = sh.hist[id >> 5] + (uint32_t)__builtin_popcount(bm[id >> 5] & ((1u << (id & 31)) - 1u));
      sh.cid[r] = id;
      sh.sx[r] = bf16_to_f32(bf16_of_k16(K));
    }
  }
  __syncthreads();
  return (int)tot;
}

}  // namespace dspark
