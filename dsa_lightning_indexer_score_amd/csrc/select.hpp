// Block-wide exact top-k selection over keys staged in LDS (shared by the
// selection kernels and the decode indexer). Internal to libidxc.
//
// Input: n <= kSelMaxKeys order-preserving 32-bit keys skey[0..n) (16-byte
// aligned) in increasing position order; pos_group(e0, bits, pv) fills pv[j]
// with the position of entry e0 + j for every set bit j of `bits` (entries
// that may be kept; e0 is a multiple of kSelPerThread and e0 + j < n for
// those). Output: the min(k, n) best entries under (key desc, position asc),
// emitted in position order through emit(slot, key, position),
// slot = 0..min(k,n)-1.
//
// Method: the keys lie in [lo, hi]; each pass histograms them into at most
// kSelBins bins of one power-of-two width (the smallest that covers the range,
// so a bin index is a shift of key - lo), finds the bin holding the rem-th
// largest key and narrows the range to it. It ends when the range is one key
// (ties: keep the `rem` lowest positions of it) or when every key of the bin
// is needed. An ordered pass (block prefix sums) then emits the winners.
#pragma once

#include "common.hpp"

namespace idxc {

constexpr int kSelThreads = 256;  // default workgroup size
constexpr int kSelBinsLog2 = 11;
constexpr int kSelBins = 1 << kSelBinsLog2;
constexpr int kSelPerThread = 8;  // ordered pass: consecutive entries per thread

// Scratch of a selection by an NT-thread workgroup. The histogram packs two
// 16-bit counts per word (bin b in half b % 2 of word b / 2): a selection
// covers fewer than 65536 keys, so no count carries into its neighbour. It
// comes last, so a caller can overlay a larger buffer on it once the
// selection is done.
template <int NT = kSelThreads>
struct SelectSmemT {
  int scan[NT / kWave];
  int bcast[4];
  uint32_t kred[2 * (NT / kWave)];
  alignas(16) uint32_t hist[kSelBins / 2];
};
constexpr int kSelMaxKeys = 65535;
using SelectSmem = SelectSmemT<>;

// Block-wide exclusive prefix sum (NT threads); *total = block sum.
template <int NT>
__device__ __forceinline__ int sel_excl_scan(int v, int* scan, int* total) {
  constexpr int kSelWaves = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scan[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = scan[w];
    if (w < wave) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// The key range of a selection gathered while the keys are staged: each
// thread passes the least and greatest key it stored (UINT32_MAX and 0 if
// none), each wave's reduction lands in the scratch, and a barrier must come
// before block_topk_collect(..., range_ready = true) reads it.
template <int NT>
__device__ __forceinline__ void sel_store_key_range(uint32_t kmin, uint32_t kmax,
                                                    SelectSmemT<NT>& sm) {
  wave_minmax(kmin, kmax);
  if (lane_id() == 0) {
    const int wave = threadIdx.x / kWave;
    sm.kred[wave] = kmin;
    sm.kred[NT / kWave + wave] = kmax;
  }
}

template <int NT = kSelThreads, typename PosGroup, typename Emit>
__device__ int block_topk_collect(const uint32_t* skey, int n, int k, SelectSmemT<NT>& sm,
                                  PosGroup pos_group, Emit emit, bool range_ready = false) {
  constexpr int kSelThreads = NT;
  constexpr int kSelWaves = NT / kWave;
  constexpr int kSelChunk = NT * kSelPerThread;
  static_assert(kSelBins % (2 * NT) == 0, "whole histogram words per thread");
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  // ---- select the k-th best key (only needed when n > k). The keys lie in
  // [lo, hi]; each pass histograms them into bins of width 2^shift, the
  // smallest power of two with (hi - lo) >> shift < kSelBins, finds the bin
  // holding the rem-th largest key and narrows the range to it (by a factor
  // of at least kSelBins / 2, so at most three passes). It ends when the
  // range is one key (ties: keep the `rem` lowest positions of it) or when
  // every key of the bin is needed.
  uint32_t lo = 0u, hi = 0u;  // final key range; keys above hi are all kept
  int rem = 0;
  bool take_range = true;  // keep every key of [lo, hi]
  const bool select_all = n <= k;
  if (!select_all) {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    if (!range_ready) {  // block-uniform
      for (int e = tid; e < n; e += kSelThreads) {
        const uint32_t key = skey[e];
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
      sel_store_key_range<NT>(kmin, kmax, sm);
      __syncthreads();
    }
    kmin = sm.kred[0];
    kmax = sm.kred[kSelWaves];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) {
      kmin = min(kmin, sm.kred[w]);
      kmax = max(kmax, sm.kred[kSelWaves + w]);
    }
    lo = kmin;
    hi = kmax;
    rem = k;
    take_range = false;
    constexpr int BPT = kSelBins / kSelThreads;  // bins per thread
    while (hi > lo) {
      const uint32_t span = hi - lo;
      const int shift = max(0, (32 - __clz((int)span)) - kSelBinsLog2);
      for (int b = tid; b < kSelBins / 2; b += kSelThreads) sm.hist[b] = 0u;
      __syncthreads();
      auto count = [&](uint32_t key) {
        if (key >= lo && key <= hi) {
          const uint32_t bin = (key - lo) >> shift;
          atomicAdd(&sm.hist[bin >> 1], 1u << ((bin & 1u) << 4));
        }
      };
      // keys four at a time (16-byte LDS reads), then the tail
      const int n4 = n >> 2;
      for (int e = tid; e < n4; e += kSelThreads) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(skey + 4 * e);
        count(kv[0]);
        count(kv[1]);
        count(kv[2]);
        count(kv[3]);
      }
      for (int e = 4 * n4 + tid; e < n; e += kSelThreads) count(skey[e]);
      __syncthreads();
      // thread tid owns bins top - q, q = 0..BPT-1 (highest first; top is
      // odd, so bins top - q and top - q - 1 share a word for even q)
      const int top = kSelBins - 1 - BPT * tid;
      int cnts[BPT];
      int local = 0;
#pragma unroll
      for (int q = 0; q < BPT; q += 2) {
        const uint32_t w = sm.hist[(top - q) >> 1];
        cnts[q] = (int)(w >> 16);
        cnts[q + 1] = (int)(w & 0xFFFFu);
        local += cnts[q] + cnts[q + 1];
      }
      int total;
      const int excl = sel_excl_scan<NT>(local, sm.scan, &total);
      if (excl < rem && excl + local >= rem) {
        int acc = excl;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
          if (acc < rem && acc + cnts[q] >= rem) {
            sm.bcast[0] = top - q;
            sm.bcast[1] = acc;
            sm.bcast[2] = cnts[q];
          }
          acc += cnts[q];
        }
      }
      __syncthreads();
      const uint32_t bstar = (uint32_t)sm.bcast[0];
      rem -= sm.bcast[1];
      const int cnt_b = sm.bcast[2];
      __syncthreads();
      // keys of bin b*: key - lo in [b* 2^shift, (b*+1) 2^shift - 1], within [lo, hi]
      const uint32_t nlo = lo + (bstar << shift);
      hi = nlo + min(hi - nlo, (1u << shift) - 1u);
      lo = nlo;
      if (cnt_b == rem) {
        take_range = true;
        break;
      }
    }
  }

  // ---- ordered collection (position order; equal-to-T entries limited to
  // the `rem` lowest positions)
  int out_count = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kSelChunk) {
    uint32_t keys[kSelPerThread];
    unsigned gt_bits = 0u, eq_bits = 0u;
    const int e0 = base + tid * kSelPerThread;
    if (e0 + kSelPerThread <= n) {
      // whole group in range: two 16-byte LDS reads (lanes 32 bytes apart)
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(skey + e0);
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(skey + e0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        keys[j] = k0[j];
        keys[4 + j] = k1[j];
      }
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j) {
        if (select_all || keys[j] > hi || (take_range && keys[j] >= lo)) gt_bits |= 1u << j;
        else if (keys[j] >= lo) eq_bits |= 1u << j;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j) {
        const int e = e0 + j;
        keys[j] = 0u;
        if (e < n) {
          keys[j] = skey[e];
          if (select_all || keys[j] > hi || (take_range && keys[j] >= lo)) gt_bits |= 1u << j;
          else if (keys[j] >= lo) eq_bits |= 1u << j;
        }
      }
    }
    // positions of the entries that may be kept, fetched before the prefix
    // sums so that a pos_group that reads memory overlaps them
    uint32_t pv[kSelPerThread];
    pos_group(e0, gt_bits | eq_bits, pv);
    // entries equal to the threshold key exist only after a selection that
    // ended on a single key (a block-uniform condition)
    int eq_total = 0, eq_excl = eq_seen;
    if (!select_all && !take_range)
      eq_excl += sel_excl_scan<NT>(__popc(eq_bits), sm.scan, &eq_total);
    unsigned keep_bits = gt_bits;
    int r = eq_excl;
#pragma unroll
    for (int j = 0; j < kSelPerThread; ++j) {
      if (eq_bits & (1u << j)) {
        if (r < rem) keep_bits |= 1u << j;
        ++r;
      }
    }
    int keep_total;
    int pos = out_count + sel_excl_scan<NT>(__popc(keep_bits), sm.scan, &keep_total);
#pragma unroll
    for (int j = 0; j < kSelPerThread; ++j) {
      if (keep_bits & (1u << j)) {
        emit(pos, keys[j], pv[j]);
        ++pos;
      }
    }
    out_count += keep_total;
    eq_seen += eq_total;
  }
  return out_count;  // == min(k, n)
}

}  // namespace idxc
