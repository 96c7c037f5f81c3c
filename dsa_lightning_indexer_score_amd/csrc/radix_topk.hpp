// Exact per-row top-k by digit refinement of order keys (internal to libidxc;
// shared by the top-k kernels).
//
// I_l = TopK(s_l, k) ("IndexCache：跨层复用稀疏注意力的索引", section
// "从 DSA 的成本分解开始"), under the library's fixed order: higher score
// first, then lower position.
//
// A workgroup of NT threads selects one row. Keys are 32-bit order-preserving
// images of the scores (larger key = larger score). The k-th best key is found
// digit by digit: the top 11 bits, the next 11, the last 10. Each level counts
// the digits of the keys that share the digits found so far in a 2048-bin LDS
// histogram, and one block scan (bins in descending order) finds the bin that
// holds the remaining rank. A level ends the search early when every key of
// its bin is needed. The outcome is a threshold: keep every key >= T, or keep
// every key > T and, of the keys equal to T, the `rem` lowest positions.
//
// The winners then leave in position order: each thread's elements sit in
// groups of G consecutive elements (group v of thread t holds elements
// G*(t + NT*v) + j, so a group is one 16- or 32-byte load and a wave's groups
// are contiguous), and one block scan of packed (above, equal) counts over
// every group at once gives each winner its output slot.
#pragma once

#include "common.hpp"
#include "select.hpp"

namespace idxc {

// Resolved digits of the k-th best key. Keys are taken relative to lo (the
// least key of the row, or 0): rel = key - lo < 2^B, B = the bit length of
// the row's key span. Level L's digit is bits [sh[L], sh[L-1]) of rel (level
// 0: [sh[0], B)); every level has at most 11 bits, sh[2] = 0, and a level
// whose shift is 0 resolves the key fully.
//   prefix: the resolved digits of rel in place, lower bits zero
//   rem: rank of the k-th best key among the keys sharing those digits
//   level: next level to resolve (3 = fully resolved)
//   done: the last resolved bin is kept whole (keep rel >= prefix);
//         otherwise, fully resolved, keep rel > prefix and the rem lowest
//         positions of rel == prefix
//   all: the row has at most k keys (keep all of them)
struct RdxState {
  uint32_t lo;
  uint32_t prefix;
  int sh0, sh1;
  int rem;
  int level;
  bool done;
  bool all;
};

__device__ __forceinline__ RdxState rdx_start(int n, int k, uint32_t lo, uint32_t hi) {
  RdxState s;
  const int B = hi > lo ? 32 - __clz((int)(hi - lo)) : 0;
  s.lo = lo;
  s.prefix = 0u;
  s.sh0 = max(0, B - kSelBinsLog2);
  s.sh1 = max(0, s.sh0 - kSelBinsLog2);
  s.rem = k;
  s.level = 0;
  s.done = false;
  s.all = n <= k;
  return s;
}

__device__ __forceinline__ int rdx_shift(const RdxState& s, int L) {
  return L == 0 ? s.sh0 : (L == 1 ? s.sh1 : 0);
}

// The functions below take rel = key - lo. Callers convert their keys once
// and give the elements past the row (a register block is rarely full) rel =
// 0, the row's least key, at positions after every real element. While the
// row has more than k keys this cannot change the selection: such an element
// ranks below every real one under (key desc, position asc), so the top-k
// contains none of them, and the searches below only count ranks. With at
// most k keys (`all`), the emit takes the real elements alone.

// Digit of level L.
__device__ __forceinline__ uint32_t rdx_digit(const RdxState& s, int L, uint32_t rel) {
  if (L == 0) return rel >> s.sh0;
  const int hi = L == 1 ? s.sh0 : s.sh1;
  const int lo = rdx_shift(s, L);
  return (rel >> lo) & ((1u << (hi - lo)) - 1u);
}

// rel shares the digits above level L with the prefix.
__device__ __forceinline__ bool rdx_match(const RdxState& s, int L, uint32_t rel) {
  if (L == 0) return true;
  const int hi = L == 1 ? s.sh0 : s.sh1;
  return (rel >> hi) == (s.prefix >> hi);
}

// Keep decision under a final state (not `all`): 1 = kept, 2 = equal to the
// threshold (kept in position order while fewer than rem were), 0 = dropped.
__device__ __forceinline__ int rdx_class(uint32_t rel, const RdxState& s) {
  if (s.done) return rel >= s.prefix ? 1 : 0;
  return rel > s.prefix ? 1 : (rel == s.prefix ? 2 : 0);
}

// Histogram add into packed 16-bit counts (bin b in half b % 2 of word b / 2).
__device__ __forceinline__ void hist16_add(uint32_t* hist, uint32_t b) {
  atomicAdd(&hist[b >> 1], 1u << ((b & 1u) << 4));
}

// Scratch of one selection by NT threads with up to NGRP element groups per
// thread in the emit scan. Scan totals and the broadcast alternate between
// two slots by level, so consecutive levels need no barrier between a read
// and the next write.
template <int NT, int NGRP>
struct RdxSmem {
  alignas(16) uint32_t hist[kSelBins];  // packed 16-bit (first half) or 32-bit counts
  int wtot[2][NGRP * (NT / kWave)];
  int scan[2][NT / kWave];
  int bc[2][4];
  uint32_t red[2 * (NT / kWave)];
  int par;
};

template <int NT, int NGRP>
__device__ __forceinline__ void rdx_clear(RdxSmem<NT, NGRP>& sm, int words) {
  for (int w = threadIdx.x; w < words; w += NT) sm.hist[w] = 0u;
}

// Block min / max of the valid keys (each thread passes its own); contains
// one barrier.
template <int NT, int NGRP>
__device__ __forceinline__ void rdx_key_range(uint32_t kmin, uint32_t kmax,
                                              RdxSmem<NT, NGRP>& sm, uint32_t& lo,
                                              uint32_t& hi) {
  constexpr int NW = NT / kWave;
  wave_minmax(kmin, kmax);
  if (lane_id() == 0) {
    sm.red[threadIdx.x / kWave] = kmin;
    sm.red[NW + threadIdx.x / kWave] = kmax;
  }
  __syncthreads();
  lo = sm.red[0];
  hi = sm.red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = min(lo, sm.red[w]);
    hi = max(hi, sm.red[NW + w]);
  }
}

// Finds the bin (descending order) holding rank st.rem of the complete
// histogram (a barrier after the last count is needed on entry) and resolves
// level st.level with it. PACKED: 16-bit counts in kSelBins / 2 words, else
// 32-bit counts in kSelBins words. Clears the histogram; a barrier is still
// needed before counting into it again. par: the slot parity of this level
// (alternate between consecutive levels). Returns the bin's count.
template <int NT, int NGRP, bool PACKED>
__device__ __forceinline__ int rdx_resolve(RdxSmem<NT, NGRP>& sm, RdxState& st, int par) {
  constexpr int BPT = kSelBins / NT;  // bins per thread, >= 2
  constexpr int NW = NT / kWave;
  static_assert(BPT >= 2 && BPT % 2 == 0, "whole histogram words per thread");
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int top = kSelBins - 1 - BPT * tid;  // odd
  int c[BPT];
  int local = 0;
#pragma unroll
  for (int q = 0; q < BPT; q += 2) {
    if constexpr (PACKED) {
      const uint32_t w = sm.hist[(top - q) >> 1];
      c[q] = (int)(w >> 16);
      c[q + 1] = (int)(w & 0xFFFFu);
    } else {
      c[q] = (int)sm.hist[top - q];
      c[q + 1] = (int)sm.hist[top - q - 1];
    }
    local += c[q] + c[q + 1];
  }
  const int incl = wave_incl_scan(local);
  if (lane_id() == kWave - 1) sm.scan[par][wave] = incl;
  __syncthreads();  // every histogram read is done
  int excl = incl - local;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) excl += sm.scan[par][w];
  if (excl < st.rem && excl + local >= st.rem) {
    int acc = excl;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (acc < st.rem && acc + c[q] >= st.rem) {
        sm.bc[par][0] = top - q;
        sm.bc[par][1] = acc;
        sm.bc[par][2] = c[q];
      }
      acc += c[q];
    }
  }
  rdx_clear(sm, PACKED ? kSelBins / 2 : kSelBins);
  __syncthreads();
  const int L = st.level;
  const uint32_t bin = (uint32_t)sm.bc[par][0];
  const int cnt = sm.bc[par][2];
  st.rem -= sm.bc[par][1];
  st.prefix |= bin << rdx_shift(st, L);
  st.level = rdx_shift(st, L) == 0 ? 3 : L + 1;
  st.done = cnt == st.rem;
  return cnt;
}

// Levels of the search over rel values held in registers (padded as above),
// in groups of four elements: group v of this thread is element group
// tid + NT*v, and the row has n elements, so only the first
// nvg = ceil(n / (4 NT)) groups of every thread hold any (the others are
// skipped: a workgroup-uniform branch). Level 0 counts the groups that hold
// row elements (the padding would pile onto one bin); later levels count
// every element whose higher digits match, which a padding element only does
// when the threshold lies in the row's lowest bin. The packed histogram must
// be zero on entry; it is zero again on return.
template <int NT>
__device__ __forceinline__ int rdx_live_groups(int n) {
  return (n + 4 * NT - 1) / (4 * NT);
}

template <int NT, int NGRP, int R>
__device__ __forceinline__ void rdx_search_regs(const uint32_t (&rel)[R], int n, RdxSmem<NT, NGRP>& sm,
                                RdxState& st) {
  static_assert(R == 4 * NGRP, "groups of four");
  if (st.all) return;  // block-uniform
  const int nvg = rdx_live_groups<NT>(n);
  // level 0: the groups holding row elements
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v < nvg && 4 * ((int)threadIdx.x + NT * v) < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) hist16_add(sm.hist, rel[4 * v + j] >> st.sh0);
    }
  }
  __syncthreads();
  rdx_resolve<NT, NGRP, true>(sm, st, 0);
  // levels 1 and 2: the elements sharing the digits found
  int par = 1;
  while (!st.done && st.level < 3) {
    const int hi = st.level == 1 ? st.sh0 : st.sh1;
    const int lo = st.level == 1 ? st.sh1 : 0;
    const uint32_t want = st.prefix >> hi;
    const uint32_t mask = (1u << (hi - lo)) - 1u;
#pragma unroll
    for (int v = 0; v < NGRP; ++v) {
      if (v < nvg) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = rel[4 * v + j];
          if ((x >> hi) == want) hist16_add(sm.hist, (x >> lo) & mask);
        }
      }
    }
    __syncthreads();
    rdx_resolve<NT, NGRP, true>(sm, st, par);
    par ^= 1;
  }
}

// Position-ordered emit of the winners held in registers, by class: cls(r)
// is 1 for a winner, 2 for an element tied with the threshold (the first
// rem_eq of them in position order win), 0 otherwise; emit(slot, r) is called
// for every winner, slot = its rank in position order. One block scan over
// all NGRP groups (one barrier; wtot slot `buf`). Returns the number of
// winners.
template <int NT, int NGRP, int G, typename Cls, typename Emit>
__device__ __forceinline__ int rdx_emit_by(int n, Cls cls, int rem_eq, RdxSmem<NT, NGRP>& sm, int buf, Emit emit) {
  static_assert(G == 4, "groups of four");
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nvg = rdx_live_groups<NT>(n);
  uint32_t kept[NGRP], eqm[NGRP];
  int cnt[NGRP], inc[NGRP];
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    kept[v] = 0u;
    eqm[v] = 0u;
    cnt[v] = 0;
    inc[v] = 0;
    if (v >= nvg) continue;  // workgroup-uniform
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int c = cls(v * G + j);
      if (c == 1) kept[v] |= 1u << j;
      else if (c == 2) eqm[v] |= 1u << j;
    }
    cnt[v] = __popc(kept[v]) | (__popc(eqm[v]) << 16);
    inc[v] = wave_incl_scan(cnt[v]);
    if (lane == kWave - 1) sm.wtot[buf][v * NW + wave] = inc[v];
  }
  __syncthreads();
  int base = 0;  // packed (above, equal) counts of all earlier groups
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    int before = base, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int x = sm.wtot[buf][v * NW + w];
      if (w < wave) before += x;
      tot += x;
    }
    base += tot;
    const int excl = before + inc[v] - cnt[v];
    int eq_before = excl >> 16;
    int slot = (excl & 0xFFFF) + min(eq_before, rem_eq);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = v * G + j;
      if ((kept[v] >> j) & 1u) {
        emit(slot++, r);
      } else if ((eqm[v] >> j) & 1u) {
        if (eq_before < rem_eq) emit(slot++, r);
        ++eq_before;
      }
    }
  }
  return (base & 0xFFFF) + min(base >> 16, rem_eq);
}

// The same under a digit-search outcome (rel values, final state st; valid(r)
// marks the row's elements and is only consulted when every element is
// kept): emit(slot, rel, r). Returns the number of winners, min(k, n).
template <int NT, int NGRP, int G, int R, typename Valid, typename Emit>
__device__ __forceinline__ int rdx_emit_regs(const uint32_t (&key)[R], int n, Valid valid, const RdxState& st,
                             RdxSmem<NT, NGRP>& sm, int buf, Emit emit) {
  static_assert(R == NGRP * G, "groups of four");
  const bool all = st.all;
  auto cls = [&](int r) { return all ? (valid(r) ? 1 : 0) : rdx_class(key[r], st); };
  return rdx_emit_by<NT, NGRP, G>(n, cls, all || st.done ? 0 : st.rem, sm, buf,
                                  [&](int slot, int r) { emit(slot, key[r], r); });
}

// ---------------------------------------------------------------------------
// Score order: the kk winners' 64-bit words (key << 32 | ~position, all
// distinct) in words[0..kk) (the array holds kk + 3 words: the ranks read
// three words of padding past the winners) are ranked into descending order through 2048
// buckets linear in the score value between the least and greatest winner:
// bucket(x) = clamp(floor((x - lo) * 2048 / (hi - lo))), a non-decreasing
// function of the key, so rank = winners in higher buckets + larger words in
// the own bucket. The words are scattered into bucket order over the same
// array (buckets descending); then each bucket-ordered slot's rank is its
// bucket's start plus the bucket's members with larger words, read four at
// a time (a wave's slots are consecutive, and so are their buckets'
// members, which keeps the LDS reads free of most bank conflicts; ranking
// each thread's own winners instead read scattered addresses and took 155
// vs 140 us on 8192 causal rows of 8192). The positions go to
// out[0..kk) in rank order through LDS (coalesced stores), then -1 up to k.
// Returns false, having written no output and left the words in place, when
// a bucket holds more than kMaxRankBucket winners (the caller then sorts).
// The histogram is zero on return either way (for the caller's sort, which
// does not use it).
// ---------------------------------------------------------------------------
constexpr int kMaxRankBucket = 48;

template <int NT, int NGRP>
__device__ __forceinline__ bool rdx_rank_output(uint64_t* words, int kk, int k, uint32_t wlo, uint32_t whi,
                                RdxSmem<NT, NGRP>& sm, int32_t* orow) {
  constexpr int BPT = kSelBins / NT;
  constexpr int EPT = (kMaxK + NT - 1) / NT;
  const int tid = threadIdx.x;
  uint32_t* cur = sm.hist;  // packed 16-bit bucket counts, then cursors
  const float vlo = key_to_float(wlo), vhi = key_to_float(whi);
  const float span = vhi - vlo;  // may round to +inf: then every winner lands in bucket 0
  const float sc = (span > 0.0f && span <= 3.4028234663852886e38f) ? (float)kSelBins / span : 0.0f;
  auto bucket_of = [&](uint64_t w) {
    const float x = (key_to_float((uint32_t)(w >> 32)) - vlo) * sc;  // NaN only for 0 * inf
    return (uint32_t)fminf(fmaxf(x, 0.0f), (float)(kSelBins - 1));
  };
  // this thread's winners (slots tid + i * NT): words, counted into their
  // buckets; the histogram is zero here (rdx_resolve cleared it, or it was
  // never used)
  uint64_t wv[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int sl = tid + i * NT;
    wv[i] = sl < kk ? words[sl] : 0ull;
    if (sl < kk) hist16_add(cur, bucket_of(wv[i]));
  }
  __syncthreads();
  const int top = kSelBins - 1 - BPT * tid;
  int cnts[BPT];
  int local = 0;
  uint32_t most = 0u, unused = 0xFFFFFFFFu;
#pragma unroll
  for (int q = 0; q < BPT; q += 2) {
    const uint32_t w = cur[(top - q) >> 1];
    cnts[q] = (int)(w >> 16);
    cnts[q + 1] = (int)(w & 0xFFFFu);
    local += cnts[q] + cnts[q + 1];
    most = max(most, max(w >> 16, w & 0xFFFFu));
  }
  int total;
  const int excl = sel_excl_scan<NT>(local, sm.scan[0], &total);
  wave_minmax(unused, most);
  if (lane_id() == 0) sm.red[tid / kWave] = most;
  __syncthreads();
  uint32_t bmax = 0u;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) bmax = max(bmax, sm.red[w]);
  if (bmax > (uint32_t)kMaxRankBucket) {  // block-uniform
    rdx_clear(sm, kSelBins / 2);
    __syncthreads();
    return false;
  }
  // cursors: each bucket's start, in descending bucket order
  int acc = excl;
#pragma unroll
  for (int q = 0; q < BPT; q += 2) {
    const uint32_t start_hi = (uint32_t)acc;
    acc += cnts[q];
    cur[(top - q) >> 1] = (start_hi << 16) | (uint32_t)acc;
    acc += cnts[q + 1];
  }
  __syncthreads();  // also: every thread holds its words, so the array can be rewritten
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (tid + i * NT < kk) {
      const uint32_t b = bucket_of(wv[i]);
      const uint32_t sh = (b & 1u) << 4;
      const uint32_t old = atomicAdd(&cur[b >> 1], 1u << sh);
      words[(old >> sh) & 0xFFFFu] = wv[i];
    }
  }
  if (tid < 3) words[kk + tid] = 0ull;  // padding read by the ranks below
  __syncthreads();
  // each cursor now holds its bucket's end; bucket b starts where bucket b+1 ends
  auto end_of = [&](uint32_t b) { return (cur[b >> 1] >> ((b & 1u) << 4)) & 0xFFFFu; };
  // ranks by bucket-ordered slot (slots tid + i * NT: a wave reads
  // consecutive words, and each compares with its bucket's neighbours)
  uint32_t rk[EPT], pv[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    rk[i] = 0u;
    pv[i] = 0u;
    if (tid + i * NT < kk) {
      const uint64_t w = words[tid + i * NT];
      const uint32_t b = bucket_of(w);
      const uint32_t e = end_of(b);
      const uint32_t st = b + 1 < (uint32_t)kSelBins ? end_of(b + 1) : 0u;
      // the slots past the bucket's end hold smaller words (lower buckets,
      // then the zero padding past the winners): read without bounds checks
      uint32_t rank = st;
      for (uint32_t j = st; j < e; j += 4) {
        uint64_t m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) m[u] = words[j + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += m[u] > w ? 1u : 0u;
      }
      rk[i] = rank;
      pv[i] = ~(uint32_t)(w & 0xFFFFFFFFull);
    }
  }
  __syncthreads();  // every word read: reuse the words' LDS for the output
  uint32_t* obuf = reinterpret_cast<uint32_t*>(words);
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (tid + i * NT < kk) obuf[rk[i]] = pv[i];
  rdx_clear(sm, kSelBins / 2);
  __syncthreads();
  for (int j = tid; j < k; j += NT) orow[j] = j < kk ? (int32_t)obuf[j] : -1;
  return true;
}

}  // namespace idxc
