// Per-query top-k for gfx950.
//
// I_l = TopK(s_l, k) ("IndexCache：跨层复用稀疏注意力的索引", section
// "从 DSA 的成本分解开始"); the order is fixed as higher score first, then
// lower position, with -0.0 == +0.0, and rows shorter than k return all of
// their t+1 positions followed by -1.
//
// A materialised row of up to 8192 scores is held in registers (32 per
// thread, one 256-thread workgroup per row). Its threshold comes from 2048
// buckets linear in the score over a sample of the row's range: the bucket
// holding the k-th best score (typically a few dozen scores) is gathered and
// ranked by one wave. Rows whose threshold bucket holds more than 64 scores
// (ties, outliers) take the digit search below instead. Candidate lists
// become order-preserving 32-bit keys held in registers (16 per thread in
// 1024-thread workgroups for up to 16384 pairs), and radix_topk.hpp finds
// the k-th best key digit by digit. Either way the winners leave in position
// order; score order then ranks them by value buckets (a bitonic sort when
// scores bunch on few values).
//
// Rows of up to 65536 scores are held in registers by one 1024-thread
// workgroup each (64 per thread), threshold again by value buckets; the
// winners gather in an LDS bitmap and leave by one scan over it. Rows the
// buckets do not settle take the digit search of the longer rows, its top
// digit counted over the row.
//
// Longer rows take three launches: one workgroup per (row, 8192-score
// chunk) counts the top 11 bits of its keys into a global histogram slice;
// one workgroup per (row, chunk) then resolves the row's top digit from the
// slices and writes its chunk's keys at or above it into the row's
// candidate list (position order, slots from the earlier chunks' counts);
// last, one 1024-thread workgroup per row selects from that list or, when the
// list would not fit, refines the digit in passes over the row and gathers
// the survivors into LDS itself.
//
// Candidate lists of (order key, position) pairs, in increasing position
// order, come from the fused indexer (one list per row) or from the per-chunk
// top-k of the decode indexer (several segments per row, whose concatenation
// is position-ordered).
#include "common.hpp"
#include "kernels.hpp"
#include "radix_topk.hpp"

#include <type_traits>

namespace idxc {

namespace {

constexpr int kRowThreads = 256;  // one row of up to kTopkChunk scores
constexpr int kRowR = kTopkChunk / kRowThreads;
constexpr int kWideThreads = 1024;  // long rows and multi-segment lists
constexpr int kWideR = kMaxStagePairs / kWideThreads;
constexpr int kLongCap = kMaxStagePairs;  // keys a long row gathers into LDS
constexpr int kHistWords = kSelBins / 2;  // packed 16-bit level-0 histogram
static_assert(kRowR % 4 == 0 && kWideR % 4 == 0, "groups of four elements");
static_assert(kTopkChunk <= kSelMaxKeys && kMaxStagePairs <= kSelMaxKeys,
              "16-bit histogram counts");

enum OutKind { kOutPos = 0, kOutScore = 1, kOutPart = 2 };
enum SrcKind { kSrcCand1 = 0, kSrcCandSeg = 1 };

// 64-bit word of lane (l ^ m) for m = 1 .. 32 (constant once unrolled).
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t plo, phi;
  switch (m) {
    case 1: plo = lane_xor<1>(lo); phi = lane_xor<1>(hi); break;
    case 2: plo = lane_xor<2>(lo); phi = lane_xor<2>(hi); break;
    case 4: plo = lane_xor<4>(lo); phi = lane_xor<4>(hi); break;
    case 8: plo = lane_xor<8>(lo); phi = lane_xor<8>(hi); break;
    case 16: plo = lane_xor<16>(lo); phi = lane_xor<16>(hi); break;
    default: plo = lane_xor<32>(lo); phi = lane_xor<32>(hi); break;
  }
  return ((uint64_t)phi << 32) | plo;
}

// Descending bitonic sort of 2048 64-bit words held 8 per thread by the
// first 256 threads of the workgroup (thread t holds slots 8t..8t+7; `act`
// marks them, whole waves: the others only take part in the barriers).
// Strides 1-4 stay in the thread, 8-256 cross lanes of the wave (DPP and
// permlane exchanges), 512 and 1024 go through LDS (2048 words). Fully
// unrolled.
__device__ __forceinline__ void sort2048_regs(uint64_t (&v)[8], uint64_t* lds, int tid,
                                              bool act) {
#pragma unroll
  for (int size = 2; size <= 2048; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 8) {
        uint64_t p[8];
        if (stride >= 8 * kWave) {
          __syncthreads();
          if (act) {
#pragma unroll
            for (int j = 0; j < 8; ++j) lds[tid * 8 + j] = v[j];
          }
          __syncthreads();
          if (act) {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = lds[(tid * 8 + j) ^ stride];
          }
        } else if (act) {
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] = lane_xor64(v[j], stride >> 3);
        }
        if (!act) continue;
        // the lane keeps the larger word when it is the lower slot of a
        // descending pair or the upper slot of an ascending one (the same
        // for all 8 words of the thread)
        const int i = tid * 8;
        const bool take_max = ((i & stride) == 0) == ((i & size) == 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool gt = v[j] > p[j];
          v[j] = (gt == take_max) ? v[j] : p[j];
        }
      } else if (act) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if ((j & stride) == 0) {
            const bool desc = ((tid * 8 + j) & size) == 0;
            const uint64_t x = v[j], y = v[j + stride];
            if ((x < y) == desc) {
              v[j] = y;
              v[j + stride] = x;
            }
          }
        }
      }
    }
  }
}


// Score rows are read through a buffer resource whose size is the row's
// valid part: reads past it return 0 instead of faulting, so every load is
// issued unconditionally. A 16-byte-aligned row is read 16 bytes (one group
// of four scores) at a time; its last group, when partly valid, is read again
// one score at a time. Rows that are not 16-byte aligned are read one score
// at a time.
struct RowSrc {
  __amdgpu_buffer_rsrc_t rs;
  int n;
  bool vec;
};

__device__ __forceinline__ RowSrc row_src(const float* src, int n) {
  RowSrc r;
  r.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), (short)0, n * 4, 0x00020000);
  r.n = n;
  r.vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  return r;
}

__device__ __forceinline__ uint32_t row_load1(const RowSrc& s, int e) {
  return __builtin_amdgcn_raw_buffer_load_b32(s.rs, e * 4, 0, 0);
}

// Raw bits of group g (scores 4g .. 4g+3; 0 past n).
__device__ __forceinline__ u32x4 row_load4(const RowSrc& s, int g) {
  if (s.vec) return __builtin_amdgcn_raw_buffer_load_b128(s.rs, g * 16, 0, 0);
  return u32x4{row_load1(s, 4 * g), row_load1(s, 4 * g + 1), row_load1(s, 4 * g + 2),
               row_load1(s, 4 * g + 3)};
}

// The partly valid last group of an aligned row, one score at a time.
__device__ __forceinline__ void row_fix_tail(const RowSrc& s, int g, u32x4& raw) {
  if (s.vec && (s.n & 3) != 0 && g == (s.n >> 2)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = row_load1(s, 4 * g + j);
  }
}

// Keys of one score row (n scores) into registers, group v of this thread
// being row group tid + NT*v; elements past the row get key 0.
template <int NT, int R>
__device__ __forceinline__ void load_row_keys(const float* src, int n, uint32_t (&key)[R]) {
  const RowSrc rs = row_src(src, n);
  const int tid = threadIdx.x;
  const int nvg = rdx_live_groups<NT>(n);
  u32x4 raw[R / 4];
#pragma unroll
  for (int v = 0; v < R / 4; ++v)
    raw[v] = v < nvg ? row_load4(rs, tid + NT * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int v = 0; v < R / 4; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    const int g = tid + NT * v;
    row_fix_tail(rs, g, raw[v]);
#pragma unroll
    for (int j = 0; j < 4; ++j) key[4 * v + j] = order_key(__uint_as_float(raw[v][j]));
    if (4 * g + 3 >= n) {  // the row's last group (or past the row)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j >= n) key[4 * v + j] = 0u;
    }
  }
}

// The same, with the least / greatest valid key of the thread (UINT32_MAX / 0
// if none).
template <int NT, int R>
__device__ __forceinline__ void load_row_keys(const float* src, int n, uint32_t (&key)[R],
                                              uint32_t& kmin, uint32_t& kmax) {
  const RowSrc rs = row_src(src, n);
  const int tid = threadIdx.x;
  const int nvg = rdx_live_groups<NT>(n);
  u32x4 raw[R / 4];
#pragma unroll
  for (int v = 0; v < R / 4; ++v)
    raw[v] = v < nvg ? row_load4(rs, tid + NT * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int v = 0; v < R / 4; ++v)
    if (v < nvg) row_fix_tail(rs, tid + NT * v, raw[v]);
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int v = 0; v < R / 4; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * (tid + NT * v) + j;
      const uint32_t kv = order_key(__uint_as_float(raw[v][j]));
      key[4 * v + j] = kv;
      if (e < n) {
        kmin = min(kmin, kv);
        kmax = max(kmax, kv);
      }
    }
  }
}


// One score row (n scores) as floats in registers, group v of this thread
// being row group tid + NT*v; elements past the row become -inf.
template <int NT, int R>
__device__ __forceinline__ void load_row_floats(const float* src, int n, float (&x)[R]) {
  const RowSrc rs = row_src(src, n);
  const int tid = threadIdx.x;
  const int nvg = rdx_live_groups<NT>(n);
  u32x4 raw[R / 4];
#pragma unroll
  for (int v = 0; v < R / 4; ++v)
    raw[v] = v < nvg ? row_load4(rs, tid + NT * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int v = 0; v < R / 4; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    const int g = tid + NT * v;
    row_fix_tail(rs, g, raw[v]);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * v + j] = __uint_as_float(raw[v][j]);
    if (4 * g + 3 >= n) {  // the row's last group (or past the row)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j >= n) x[4 * v + j] = -INFINITY;
    }
  }
}

// Least and greatest of this thread's row elements in its first and last
// live groups (+inf / -inf if none): a sample of the row's range that takes
// in both of its ends.
template <int NT, int R>
__device__ __forceinline__ void sample_range(const float (&x)[R], int n, float& mn, float& mx) {
  const int tid = threadIdx.x;
  const int nvg = rdx_live_groups<NT>(n);
  mn = INFINITY;
  mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < R / 4; ++v) {
    if (v != 0 && v != nvg - 1) continue;  // workgroup-uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * (tid + NT * v) + j < n) {
        mn = fminf(mn, x[4 * v + j]);
        mx = fmaxf(mx, x[4 * v + j]);
      }
    }
  }
}

template <int NT>
__device__ __forceinline__ int elem_of(int r) {
  return 4 * ((int)threadIdx.x + NT * (r >> 2)) + (r & 3);
}

// orow[0..k) = obuf[0..kk), then -1: 16-byte stores when the row allows.
template <int NT>
__device__ __forceinline__ void store_row_positions(const int* obuf, int kk, int k, int32_t* orow) {
  const int tid = threadIdx.x;
  if ((k & 3) == 0 && (reinterpret_cast<uintptr_t>(orow) & 15) == 0) {
    for (int j = 4 * tid; j < k; j += 4 * NT) {
      int4 v = *reinterpret_cast<const int4*>(obuf + j);
      if (j + 3 >= kk) {
        v.x = j < kk ? v.x : -1;
        v.y = j + 1 < kk ? v.y : -1;
        v.z = j + 2 < kk ? v.z : -1;
        v.w = -1;
      }
      *reinterpret_cast<int4*>(orow + j) = v;
    }
  } else {
    for (int j = tid; j < k; j += NT) orow[j] = j < kk ? obuf[j] : -1;
  }
}

// ---------------------------------------------------------------------------
// Threshold of a materialised score row by value buckets. The row's scores
// (floats in registers, n > k of them, spanning [lo, hi], lo < hi finite) are
// counted into kSelBins buckets linear in the value,
//   bucket(x) = trunc(clamp(fma(x, sc, c), 0, kSelBins - 1)),
//   sc = kSelBins / (hi - lo), c = -lo * sc,
// a non-decreasing function of x (each step rounds monotonically), so the
// k-th best score lies in the bucket b* where the count from the top first
// reaches k, and every score in a higher bucket is a winner. Linear buckets
// spread a row's scores evenly where the digits of their bit patterns would
// pile them onto the few bins of a handful of exponents, so b* typically
// holds a few dozen scores. Those are gathered into LDS and one wave ranks
// them by value: the threshold T is the score of rank rem = k - (scores in
// higher buckets) among them, and the winners are the scores above T and the
// first rem_eq of the scores equal to T in position order. Returns false
// (block-uniform; nothing written but LDS) when b* holds more than kVbCap
// scores. The histogram is left as counted.
// ---------------------------------------------------------------------------
constexpr int kVbCap = 64;

// threadIdx.x as a value the compiler cannot tie to earlier uses: the group
// indices derived from it are recomputed (one add) in each phase instead of
// being kept live, or spilled, across the phases.
__device__ __forceinline__ int fresh_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// LDS of the selection of a row held by NT threads, NGRP element groups each.
template <int NT, int NGRP>
struct VbSmemT {
  float cv[kVbCap];  // b*'s scores and positions
  int cp[kVbCap];
  int cnt;
  float thr;
  int rem_eq;
  int ok;
  // the scores equal to T that win, as a bitmap over the row's positions,
  // and per (element group, wave) whether it holds any of them
  uint32_t eqbits[NT * NGRP * 4 / 32];
  int eqflag[NGRP * (NT / kWave)];
  int bstar;         // the bucket of the k-th best score
  int trash[kWave];  // targets of the stores of elements that lose
  uint64_t trash64[kWave];
};

using VbSmem = VbSmemT<kRowThreads, kRowR / 4>;

// Clears the tie bitmap and flags (needs a barrier before vb_threshold).
template <int NT, int NGRP>
__device__ __forceinline__ void vb_clear(VbSmemT<NT, NGRP>& vs) {
  constexpr int kBits = NT * NGRP / 8, kFlags = NGRP * (NT / kWave);
  static_assert(kBits % NT == 0 && kFlags <= NT, "whole bitmap words per thread");
#pragma unroll
  for (int w = 0; w < kBits / NT; ++w) vs.eqbits[(int)threadIdx.x + w * NT] = 0u;
  if (threadIdx.x < kFlags) vs.eqflag[threadIdx.x] = 0;
}

__device__ __forceinline__ float vb_y(float x, float sc, float c) { return fmaf(x, sc, c); }

__device__ __forceinline__ uint32_t vb_bucket(float x, float sc, float c) {
  return (uint32_t)__builtin_amdgcn_fmed3f(vb_y(x, sc, c), 0.0f, (float)(kSelBins - 1));
}

// sc and c for the row range [lo, hi], or false when value buckets do not
// apply (block-uniform inputs).
__device__ __forceinline__ bool vb_scale(float lo, float hi, float& sc, float& c) {
  const float span = hi - lo;
  if (!(span > 0.0f) || !(span <= 3.4028234663852886e38f)) return false;  // also NaN
  sc = (float)kSelBins / span;
  c = -lo * sc;
  return sc <= 3.4028234663852886e38f && fabsf(c) <= 3.4028234663852886e38f;
}

// Bins p[0 .. BPT) of a 32-bit histogram, in 16- or 8-byte LDS reads
// (p aligned to them), and their store.
template <int BPT>
__device__ __forceinline__ void vb_bins(const uint32_t* p, uint32_t (&cb)[BPT]) {
  static_assert(BPT % 4 == 0 || BPT == 2, "whole 16- or 8-byte reads");
  if constexpr (BPT == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    cb[0] = v[0];
    cb[1] = v[1];
  } else {
#pragma unroll
    for (int q = 0; q < BPT; q += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + q);
      cb[q] = v.x;
      cb[q + 1] = v.y;
      cb[q + 2] = v.z;
      cb[q + 3] = v.w;
    }
  }
}
template <int BPT>
__device__ __forceinline__ void vb_store_bins(uint32_t* p, const uint32_t (&cb)[BPT]) {
  if constexpr (BPT == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{cb[0], cb[1]};
  } else {
#pragma unroll
    for (int q = 0; q < BPT; q += 4)
      *reinterpret_cast<u32x4*>(p + q) = u32x4{cb[q], cb[q + 1], cb[q + 2], cb[q + 3]};
  }
}

// Counts the row's scores into the 32-bit bucket bins (clear on entry), then
// a barrier. Only groups holding row elements are counted; the padding in
// the row's last group, -inf, lands in bucket 0 and never takes a slot.
template <int NT, int NGRP, int R>
__device__ __forceinline__ void vb_histogram(const float (&x)[R], int n, float sc, float c,
                                             RdxSmem<NT, NGRP>& sm) {
  const int tid = threadIdx.x;
  const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v < nvg && 4 * (tid + NT * v) < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) atomicAdd(&sm.hist[vb_bucket(x[4 * v + j], sc, c)], 1u);
    }
  }
  __syncthreads();
}

template <int NT, int NGRP, int R>
__device__ __forceinline__ bool vb_threshold(const float (&x)[R], int n, int k, float sc, float c,
                             RdxSmem<NT, NGRP>& sm, VbSmemT<NT, NGRP>& vs, float& thr, int& rem_eq) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int nvg = rdx_live_groups<NT>(n);
  if (tid == 0) vs.cnt = 0;  // read after the barriers of the resolve below
  vb_histogram<NT, NGRP, R>(x, n, sc, c, sm);
  // b*: the bucket where the count from the top first reaches k (a block
  // scan of the 32-bit counts, bins in descending order; the thread whose
  // range holds it reads its bins again)
  {
    constexpr int BPT = kSelBins / NT;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int top = kSelBins - 1 - BPT * tid;
    uint32_t cb[BPT];
    vb_bins<BPT>(sm.hist + top - (BPT - 1), cb);
    int local = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) local += (int)cb[q];
    const int incl = wave_incl_scan(local);
    if (lane == kWave - 1) sm.scan[0][wave] = incl;
    __syncthreads();
    int excl = incl - local;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w)
      if (w < wave) excl += sm.scan[0][w];
    if (excl < k && excl + local >= k) {
      int acc = excl;
      for (int q = 0; q < BPT; ++q) {
        const int c = (int)sm.hist[top - q];
        if (acc < k && acc + c >= k) {
          sm.bc[0][0] = top - q;
          sm.bc[0][1] = acc;
          sm.bc[0][2] = c;
        }
        acc += c;
      }
    }
    __syncthreads();
  }
  const int cnt = sm.bc[0][2];
  if (cnt > kVbCap) return false;  // block-uniform
  const uint32_t bs = (uint32_t)sm.bc[0][0];  // b*
  if (tid == 0) vs.bstar = (int)bs;           // read after the barriers below
  const int rem = k - sm.bc[0][1];
  // bucket(x) == b*  <=>  ylo <= fma(x, sc, c) < yhi
  // (the top bucket has no upper bound: there y may overflow to +inf)
  const float ylo = bs == 0u ? -INFINITY : (float)bs;
  const bool top = bs == (uint32_t)(kSelBins - 1);
  const float yhi = (float)(bs + 1u);
  const int ftid = fresh_tid();
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v < nvg && 4 * (ftid + NT * v) < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = vb_y(x[4 * v + j], sc, c);
        if (y >= ylo && (top || y < yhi)) {
          const int s = atomicAdd(&vs.cnt, 1);
          if (s < kVbCap) {
            vs.cv[s] = x[4 * v + j];
            vs.cp[s] = 4 * (ftid + NT * v) + j;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int m = min(vs.cnt, kVbCap);
    const float mine = lane < m ? vs.cv[lane] : -INFINITY;
    int gt = 0, ge = 0;
    for (int j = 0; j < m; ++j) {
      const float u = vs.cv[j];
      gt += u > mine ? 1 : 0;
      ge += u >= mine ? 1 : 0;
    }
    const uint64_t hit = ballot(lane < m && gt < rem && rem <= ge);
    const int src = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    if (lane == 0) vs.ok = (hit && vs.cnt == cnt) ? 1 : 0;  // the gathered scores are b*'s
    const float t = __shfl(mine, src, kWave);
    const int req = rem - __shfl(gt, src, kWave);
    if (lane == 0) {
      vs.thr = t;
      vs.rem_eq = req;
    }
    // the scores equal to T rank by position: the first req of them win (a
    // lone T wins without the ranking)
    const int mp = lane < m ? vs.cp[lane] : 0x7FFFFFFF;
    const bool is_t = lane < m && mine == t;
    int rp = 0;
    if (popc64(ballot(is_t)) > 1) {
      for (int j = 0; j < m; ++j) rp += (vs.cv[j] == t && vs.cp[j] < mp) ? 1 : 0;
    }
    if (hit && is_t && rp < req) {
      const int g = mp >> 2;  // element group tid + NT*v of the row
      atomicOr(&vs.eqbits[mp >> 5], 1u << (mp & 31));
      vs.eqflag[(g / NT) * (NT / kWave) + (g % NT) / kWave] = 1;
    }
  }
  __syncthreads();
  thr = vs.thr;
  rem_eq = vs.rem_eq;
  return vs.ok != 0;
}

// Position-ordered winners after vb_threshold: the scores above T, and the
// scores equal to T marked in the tie bitmap. Each thread keeps a 4-bit mask
// of winners per element group; one block scan of the group counts gives the
// groups' first slots, then emit(win, slot, r, pos) runs for every element r
// (row position pos) of the thread, slot being its rank among the winners in
// position order when win (the callback stores without a branch per element: a loser's store
// goes to a trash word). Returns the number of winners (k).
template <int NT, int NGRP, int R, typename Emit>
__device__ __forceinline__ int vb_emit(const float (&x)[R], int n, float thr, RdxSmem<NT, NGRP>& sm,
                                       VbSmemT<NT, NGRP>& vs,
                       Emit emit) {
  constexpr int NW = NT / kWave;
  const int tid = fresh_tid();
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nvg = rdx_live_groups<NT>(n);
  uint32_t msk[NGRP];
  int inc[NGRP];
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    msk[v] = 0u;
    inc[v] = 0;
    if (v >= nvg) continue;  // workgroup-uniform
    const int g = tid + NT * v;
    uint32_t m = (x[4 * v] > thr ? 1u : 0u) | (x[4 * v + 1] > thr ? 2u : 0u) |
                 (x[4 * v + 2] > thr ? 4u : 0u) | (x[4 * v + 3] > thr ? 8u : 0u);
    if (vs.eqflag[v * NW + wave])  // wave-uniform: this group holds winning ties
      m |= (vs.eqbits[g >> 3] >> (4 * (g & 7))) & 15u;
    msk[v] = m;
    inc[v] = wave_incl_scan(__popc(m));
    if (lane == kWave - 1) sm.wtot[0][v * NW + wave] = inc[v];
  }
  __syncthreads();
  int base = 0;  // winners of all earlier groups
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    int before = base, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int y = sm.wtot[0][v * NW + w];
      if (w < wave) before += y;
      tot += y;
    }
    base += tot;
    const uint32_t m = msk[v];
    const int slot0 = before + inc[v] - __popc(m);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      emit(((m >> j) & 1u) != 0u, slot0 + __popc(m & ((1u << j) - 1u)), 4 * v + j,
           4 * (tid + NT * v) + j);
  }
  return base;
}

// Position-ordered winners after vb_threshold through the tie bitmap: each
// thread ORs in the bits of its scores above T (group g's four bits at bits
// 4 (g % 8) .. of word g / 8, the eight lanes of a word combined by lane
// exchanges), then one block scan over the bitmap's words (one or two per
// thread) gives every winner its slot: pbuf[slot] = its position. Returns
// the number of winners; a barrier must come before pbuf is read.
template <int NT, int NGRP, int R>
__device__ __forceinline__ int vb_bitmap_emit(const float (&x)[R], int n, float thr,
                                              RdxSmem<NT, NGRP>& sm, VbSmemT<NT, NGRP>& vs,
                                              int* pbuf) {
  constexpr int NW = NT / kWave;
  constexpr int kWords = NT * NGRP / 8;
  constexpr int WPT = kWords / NT;
  static_assert(WPT * NT == kWords && (WPT == 1 || WPT == 2), "whole bitmap words per thread");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    const uint32_t m = (x[4 * v] > thr ? 1u : 0u) | (x[4 * v + 1] > thr ? 2u : 0u) |
                       (x[4 * v + 2] > thr ? 4u : 0u) | (x[4 * v + 3] > thr ? 8u : 0u);
    uint32_t w = m << (4 * (lane & 7));
    w |= lane_xor<1>(w);
    w |= lane_xor<2>(w);
    w |= lane_xor<4>(w);
    if ((lane & 7) == 0 && w != 0u) atomicOr(&vs.eqbits[(tid + NT * v) >> 3], w);
  }
  __syncthreads();
  uint32_t bw[WPT];
  if constexpr (WPT == 2) {
    const u32x2 b2 = *reinterpret_cast<const u32x2*>(vs.eqbits + 2 * tid);
    bw[0] = b2[0];
    bw[1] = b2[1];
  } else {
    bw[0] = vs.eqbits[tid];
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) cnt += __popc(bw[j]);
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) sm.scan[0][wave] = incl;
  __syncthreads();
  int slot = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int y = sm.scan[0][w];
    if (w < wave) slot += y;
    total += y;
  }
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    uint32_t bits = bw[j];
    while (bits != 0u) {
      pbuf[slot++] = 32 * (WPT * tid + j) + __ffs((int)bits) - 1;
      bits &= bits - 1u;
    }
  }
  return total;
}

// Score order after vb_threshold, from the row's own bucket counts (still in
// the histogram): buckets above b* hold winners only, so a winner's rank is
// the number of scores in higher buckets plus the larger (key, ~position)
// words in its own bucket. The counts become per-bucket cursors starting at
// the scores above each bucket (a block scan), every winner takes a slot of
// its bucket's range with an LDS atomic and stores its word there, and each
// slot then ranks its word within its bucket (its members lie between the
// next bucket's cursor and its own). The positions leave in rank order
// through LDS. kk = the number of winners (k, or n for a row of at most k
// scores, which takes every score: thr = -inf, vs.bstar = -1). Returns false
// (block-uniform, nothing written but LDS) when a bucket above b* holds more
// than kMaxRankBucket scores: the caller then takes another path.
template <int NT, int NGRP, int R>
__device__ __forceinline__ bool vb_score_order(const float (&x)[R], int n, int k, int kk, float thr,
                                               float sc, float c, RdxSmem<NT, NGRP>& sm,
                                               VbSmemT<NT, NGRP>& vs, uint64_t* words, int32_t* orow) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kSelBins / NT;
  const int tid = fresh_tid();
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int bs = vs.bstar;
  // ---- cursors: bin b <- scores in bins above b (thread t holds bins
  // top-7 .. top, top = kSelBins-1-8t, in descending order by thread)
  {
    const int top = kSelBins - 1 - BPT * tid;
    uint32_t* hb = sm.hist + top - (BPT - 1);
    uint32_t cb[BPT];  // bins top-BPT+1 .. top
    vb_bins<BPT>(hb, cb);
    int local = 0;
    uint32_t most = 0u;  // greatest count of a bin above b*
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      local += (int)cb[q];
      if (top - (BPT - 1) + q > bs) most = max(most, cb[q]);
    }
    const int incl = wave_incl_scan(local);
    uint32_t unused = 0xFFFFFFFFu;
    wave_minmax(unused, most);
    if (lane == kWave - 1) sm.scan[1][wave] = incl;
    if (lane == 0) sm.red[wave] = most;
    __syncthreads();  // every bin is read
    int excl = incl - local;
    uint32_t bmax = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) excl += sm.scan[1][w];
      bmax = max(bmax, sm.red[w]);
    }
    uint32_t cur[BPT];  // bin top starts at excl, each lower one after the bins above it
    uint32_t run = (uint32_t)excl;
#pragma unroll
    for (int q = BPT - 1; q >= 0; --q) {
      cur[q] = run;
      run += cb[q];
    }
    if (bmax > (uint32_t)kMaxRankBucket) return false;  // block-uniform; the counts stay
    vb_store_bins<BPT>(hb, cur);
  }
  if (tid < 3) words[kk + tid] = 0ull;  // padding read by the ranks below
  __syncthreads();  // cursors written
  // ---- every winner takes a slot of its bucket's range
  const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    const int g = tid + NT * v;
    uint32_t m = (x[4 * v] > thr ? 1u : 0u) | (x[4 * v + 1] > thr ? 2u : 0u) |
                 (x[4 * v + 2] > thr ? 4u : 0u) | (x[4 * v + 3] > thr ? 8u : 0u);
    if (vs.eqflag[v * NW + wave])  // wave-uniform: this group holds winning ties
      m |= (vs.eqbits[g >> 3] >> (4 * (g & 7))) & 15u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((m >> j) & 1u) {
        const uint32_t bk = vb_bucket(x[4 * v + j], sc, c);
        const uint32_t slot = atomicAdd(&sm.hist[bk], 1u);
        words[slot] = ((uint64_t)order_key(x[4 * v + j]) << 32) | (uint64_t)(~(uint32_t)(4 * g + j));
      }
    }
  }
  __syncthreads();
  // ---- rank of each bucket-ordered slot; bucket b spans [cursor(b+1), cursor(b))
  constexpr int EPT = kMaxK / NT;
  uint32_t rk[EPT], pv[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int sl = tid + i * NT;
    rk[i] = 0u;
    pv[i] = 0u;
    if (sl < kk) {
      const uint64_t w = words[sl];
      const uint32_t bk = vb_bucket(key_to_float((uint32_t)(w >> 32)), sc, c);
      const uint32_t e = sm.hist[bk];
      const uint32_t st = bk + 1 < (uint32_t)kSelBins ? sm.hist[bk + 1] : 0u;
      // the slots past the bucket's end hold smaller words (lower buckets,
      // then the zero padding past the winners), so reading them counts
      // nothing: no bounds check per member
      uint32_t rank = st;
      for (uint32_t j = st; j < e; j += 4) {
        uint64_t mm[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) mm[u] = words[j + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += mm[u] > w ? 1u : 0u;
      }
      rk[i] = rank;
      pv[i] = ~(uint32_t)(w & 0xFFFFFFFFull);
    }
  }
  __syncthreads();  // every word read: the positions go over them
  uint32_t* obuf = reinterpret_cast<uint32_t*>(words);
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (tid + i * NT < kk) obuf[rk[i]] = pv[i];
  __syncthreads();
  store_row_positions<NT>(reinterpret_cast<const int*>(obuf), kk, k, orow);
  return true;
}

// A position-ordered list of n (key, position) pairs into registers (element
// r of this thread at elem_of<NT>(r); zeros past the list), through a buffer
// resource of its n pairs (reads past them return 0): two 16-byte loads per
// group of four pairs, issued unconditionally; a partly valid last group is
// read again pair by pair.
template <int NT, int R>
__device__ __forceinline__ void load_pair_list(const u32x2* src, int n, uint32_t (&key)[R],
                                               uint32_t (&pos)[R]) {
  constexpr int NGRP = R / 4;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x2*>(src), (short)0, n * 8, 0x00020000);
  u32x4 p0[NGRP], p1[NGRP];
  const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    const int g = tid + NT * v;
    p0[v] = p1[v] = u32x4{0u, 0u, 0u, 0u};
    if (v < nvg) {  // workgroup-uniform
      p0[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, g * 32, 0, 0);
      p1[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, g * 32 + 16, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    const int g = tid + NT * v;
    if ((n & 3) != 0 && g == (n >> 2)) {
      const u32x2 q0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, g * 32, 0, 0));
      const u32x2 q1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, g * 32 + 8, 0, 0));
      const u32x2 q2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, g * 32 + 16, 0, 0));
      p0[v] = u32x4{q0[0], q0[1], q1[0], q1[1]};
      p1[v] = u32x4{q2[0], q2[1], 0u, 0u};
    }
    key[4 * v + 0] = p0[v][0];
    pos[4 * v + 0] = p0[v][1];
    key[4 * v + 1] = p0[v][2];
    pos[4 * v + 1] = p0[v][3];
    key[4 * v + 2] = p1[v][0];
    pos[4 * v + 2] = p1[v][1];
    key[4 * v + 3] = p1[v][2];
    pos[4 * v + 3] = p1[v][3];
  }
}

// Score-order finish: the kk winners' words are in `words`, their key range
// in [wmin, wmax] per thread. Ranks them (or sorts them) into orow.
template <int NT, int NGRP>
__device__ __forceinline__ void score_order_output(uint64_t* words, int kk, int k,
                                   uint32_t wmin, uint32_t wmax, RdxSmem<NT, NGRP>& sm,
                                   int32_t* orow) {
  const int tid = threadIdx.x;
  wave_minmax(wmin, wmax);
  if (lane_id() == 0) {
    sm.red[tid / kWave] = wmin;
    sm.red[NT / kWave + tid / kWave] = wmax;
  }
  __syncthreads();  // also: every word is written
  uint32_t wlo = sm.red[0], whi = sm.red[NT / kWave];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) {
    wlo = min(wlo, sm.red[w]);
    whi = max(whi, sm.red[NT / kWave + w]);
  }
  __syncthreads();  // red is reused below
  if (rdx_rank_output<NT, NGRP>(words, kk, k, wlo, whi, sm, orow)) return;
  // bitonic sort of the kk winners padded with zero words (every winner's word
  // is nonzero, so they sort last); the first 256 threads hold the words
  static_assert(kMaxK == 8 * 256 && NT % 256 == 0, "register sort layout");
  const bool act = tid < 256;
  uint64_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = tid * 8 + j;
    v[j] = (act && idx < kk) ? words[idx] : 0ull;
  }
  sort2048_regs(v, words, tid, act);
  if (act) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid * 8 + j;
      if (idx < k) orow[idx] = (idx < kk) ? (int32_t)(~(uint32_t)(v[j] & 0xFFFFFFFFull)) : -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of up to kTopkChunk materialised scores, one 256-thread workgroup per
// row, longest rows first. Row r = b*Lq + i holds candidates 0..t, t =
// q_pos0 + i (never more than Lk).
// ---------------------------------------------------------------------------
// (position order runs eight waves per SIMD in 64 registers: 41 us, against
// 43 us at seven, its few spills outside the value-bucket path; score order
// runs at five: six measured 119 vs 89 us)
template <int OUT>
__global__ __launch_bounds__(kRowThreads, OUT == kOutPos ? 8 : 5)
void topk_rows_kernel(const float* __restrict__ scores, int B, int Lq, int Lk, int q_pos0, int k,
                      int32_t* __restrict__ out) {
  constexpr int NT = kRowThreads, R = kRowR, NGRP = R / 4;
  __shared__ RdxSmem<NT, NGRP> sm;
  __shared__ uint64_t words[OUT == kOutScore ? kMaxK + 3 : 2];  // + padding of the bucket ranks
  const int tid = threadIdx.x;
  const int i = Lq - 1 - (int)(blockIdx.x / (unsigned)B);
  const int b = (int)(blockIdx.x % (unsigned)B);
  const size_t row = (size_t)b * Lq + i;
  const int n = min(q_pos0 + i + 1, Lk);
  int32_t* orow = out + row * k;
  if (OUT == kOutPos && n <= k) {  // every candidate, in position order
    for (int j = tid; j < k; j += NT) orow[j] = j < n ? j : -1;
    return;
  }
  rdx_clear(sm, kSelBins);  // 32-bit bucket counts (the digit search uses the first half)
  __shared__ VbSmem vs;
  vb_clear(vs);
  float x[R];
  load_row_floats<NT, R>(scores + row * Lk, n, x);
  // A sample of the row's range sets the buckets (scores outside it fall
  // into the end buckets, which keeps the bucket function monotonic): one
  // barrier, which also orders the histogram clear.
  {
    float fmn, fmx;
    sample_range<NT, R>(x, n, fmn, fmx);
    uint32_t kmn = fmn <= fmx ? order_key(fmn) : 0xFFFFFFFFu;
    uint32_t kmx = fmn <= fmx ? order_key(fmx) : 0u;
    wave_minmax(kmn, kmx);
    if (lane_id() == 0) {
      sm.red[tid / kWave] = kmn;
      sm.red[NT / kWave + tid / kWave] = kmx;
    }
  }
  __syncthreads();
  uint32_t klo = sm.red[0], khi = sm.red[NT / kWave];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) {
    klo = min(klo, sm.red[w]);
    khi = max(khi, sm.red[NT / kWave + w]);
  }
  float sc = 0.0f, c = 0.0f, thr = 0.0f;
  int rem_eq = 0;
  if (n > k && vb_scale(key_to_float(klo), key_to_float(khi), sc, c) &&
      vb_threshold<NT, NGRP, R>(x, n, k, sc, c, sm, vs, thr, rem_eq)) {  // block-uniform
    const int lane = lane_id();
    if (OUT == kOutPos) {
      // the winners' positions gather in LDS by slot (over the histogram, not
      // read after vb_emit's barrier), then leave in 16-byte stores
      static_assert(kSelBins >= kMaxK, "positions staged over the histogram");
      int* obuf = reinterpret_cast<int*>(sm.hist);
      const int kk = vb_bitmap_emit<NT, NGRP, R>(x, n, thr, sm, vs, obuf);
      __syncthreads();
      store_row_positions<NT>(obuf, kk, k, orow);
    } else {
      if (vb_score_order<NT, NGRP, R>(x, n, k, k, thr, sc, c, sm, vs, words, orow)) return;
      // the least winner is T; the greatest is the row's greatest score.
      // The bucket ranks need a clear histogram (ordered by vb_emit's barrier).
      rdx_clear(sm, kSelBins / 2);
      const uint32_t wmin = order_key(thr);
      uint32_t wmax = 0u;
      const int kk = vb_emit<NT, NGRP, R>(x, n, thr, sm, vs, [&](bool win, int slot, int r, int p) {
        const uint32_t kv = order_key(x[r]);
        *(win ? words + slot : vs.trash64 + lane) = ((uint64_t)kv << 32) | (uint64_t)(~(uint32_t)p);
        wmax = max(wmax, win ? kv : 0u);
      });
      score_order_output<NT, NGRP>(words, kk, k, wmin, wmax, sm, orow);
    }
    return;
  }
  // Score order of a row of at most k scores: every score wins, ranked from
  // the row's bucket counts (the histogram is clear: vb_threshold never ran).
  if (OUT == kOutScore && n <= k && vb_scale(key_to_float(klo), key_to_float(khi), sc, c)) {
    if (tid == 0) vs.bstar = -1;  // every bucket's size is bounded; read after vb_histogram's barrier
    vb_histogram<NT, NGRP, R>(x, n, sc, c, sm);
    if (vb_score_order<NT, NGRP, R>(x, n, k, n, -INFINITY, sc, c, sm, vs, words, orow)) return;
    rdx_clear(sm, kSelBins);  // the counts stay on that return
    __syncthreads();
  }
  // Digit search over the keys (rows of at most k scores, or whose scores
  // bunch in one value bucket). A full score row spans most of the key
  // space, so the digits are taken of the keys themselves (base 0): no key
  // range to find. Elements past the row get key 0, below the key of every
  // finite score. The histogram may hold the value-bucket counts.
  rdx_clear(sm, kHistWords);
  __syncthreads();
  uint32_t key[R];
  {
    const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
    for (int v = 0; v < NGRP; ++v) {
      if (v >= nvg) continue;  // workgroup-uniform
      const int g = tid + NT * v;
#pragma unroll
      for (int j = 0; j < 4; ++j) key[4 * v + j] = 4 * g + j < n ? order_key(x[4 * v + j]) : 0u;
    }
  }
  auto valid = [&](int r) { return elem_of<NT>(r) < n; };
  constexpr uint32_t lo = 0u;
  RdxState st = rdx_start(n, k, 0u, 0xFFFFFFFFu);
  rdx_search_regs<NT, NGRP, R>(key, n, sm, st);
  if (OUT == kOutPos) {
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, n, valid, st, sm, 0, [&](int slot, uint32_t, int r) { orow[slot] = elem_of<NT>(r); });
    for (int j = kk + tid; j < k; j += NT) orow[j] = -1;
  } else {
    uint32_t wmin = 0xFFFFFFFFu, wmax = 0u;
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(key, n, valid, st, sm, 0,
                                                 [&](int slot, uint32_t rv, int r) {
                                                   const uint32_t kv = rv + lo;
                                                   words[slot] = ((uint64_t)kv << 32) |
                                                                 (uint64_t)(~(uint32_t)elem_of<NT>(r));
                                                   wmin = min(wmin, kv);
                                                   wmax = max(wmax, kv);
                                                 });
    score_order_output<NT, NGRP>(words, kk, k, wmin, wmax, sm, orow);
  }
}

// ---------------------------------------------------------------------------
// Long rows, first launch: one workgroup per (row, kTopkChunk-score chunk)
// writes the packed 16-bit histogram of its keys' top 11 bits to
// ghist[(row * nch + chunk) * kHistWords ..]. Chunks past the row's end write
// nothing (the second launch reads only the row's own chunks).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads)
void topk_chunk_hist_kernel(const float* __restrict__ scores, int Lq, int Lk, int q_pos0,
                            int nch, uint32_t* __restrict__ ghist) {
  constexpr int NT = kRowThreads, R = kRowR;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x / (unsigned)nch;
  const int c = (int)(blockIdx.x % (unsigned)nch);
  const int i = (int)(row % (size_t)Lq);
  const int n = min(q_pos0 + i + 1, Lk);
  const int c0 = c * kTopkChunk;
  if (c0 >= n) return;
  const int m = min(kTopkChunk, n - c0);
  for (int w = tid; w < kHistWords; w += NT) hist[w] = 0u;
  uint32_t key[R], kmin, kmax;
  load_row_keys<NT, R>(scores + row * Lk + c0, m, key, kmin, kmax);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (elem_of<NT>(r) < m) hist16_add(hist, key[r] >> 21);  // the top 11 bits
  __syncthreads();
  u32x4* dst = reinterpret_cast<u32x4*>(ghist + (row * nch + c) * kHistWords);
  const u32x4* srch = reinterpret_cast<const u32x4*>(hist);
  for (int w = tid; w < kHistWords / 4; w += NT) dst[w] = srch[w];
}

// ---------------------------------------------------------------------------
// Rows of more than kLongCap scores, second launch: one workgroup per (row,
// chunk). Every workgroup of a row sums the row's chunk histograms and
// resolves the top digit of the row's k-th best key (all of them reach the
// same digit). The row's keys at or above that digit (at least k of them)
// form its candidate list when they number at most kLongCap: each workgroup
// writes its chunk's share in position order, at the slot where the earlier
// chunks' shares end (their counts read off their histograms). lcnt[row]
// receives the list's length, or -1 when it would not fit (the last launch
// then refines the digit over the row itself).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads)
void topk_chunk_gather_kernel(const float* __restrict__ scores, int Lq, int Lk, int q_pos0, int k,
                              int nch, const uint32_t* __restrict__ ghist,
                              u32x2* __restrict__ lcand, int* __restrict__ lcnt) {
  constexpr int NT = kRowThreads, R = kRowR, NGRP = R / 4, NW = NT / kWave;
  constexpr int BPT = kSelBins / NT;  // bins summed per thread: BPT / 2 histogram words
  static_assert(BPT == 8, "two 16-byte histogram loads per chunk and thread");
  __shared__ RdxSmem<NT, NGRP> sm;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x / (unsigned)nch;
  const int c = (int)(blockIdx.x % (unsigned)nch);
  const int i = (int)(row % (size_t)Lq);
  const int n = min(q_pos0 + i + 1, Lk);
  const int c0 = c * kTopkChunk;
  if (n <= kLongCap || c0 >= n) return;  // rows the last launch loads whole; chunks past the row
  const int nc = (n + kTopkChunk - 1) / kTopkChunk;
  // the row's counts of bins 8 tid .. 8 tid + 7 (and those of the chunks
  // before this one), the chunks' words in batches of loads
  uint32_t tot[BPT], bef[BPT];
#pragma unroll
  for (int q = 0; q < BPT; ++q) tot[q] = bef[q] = 0u;
  const u32x4* gw = reinterpret_cast<const u32x4*>(ghist + row * nch * kHistWords) + tid;
  constexpr int kBatch = 8;
  for (int cc0 = 0; cc0 < nc; cc0 += kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      v[q] = cc0 + q < nc ? gw[(size_t)(cc0 + q) * (kHistWords / 4)] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const bool before = cc0 + q < c;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo16 = v[q][w] & 0xFFFFu, hi16 = v[q][w] >> 16;  // bins 2w, 2w + 1
        tot[2 * w] += lo16;
        tot[2 * w + 1] += hi16;
        if (before) {
          bef[2 * w] += lo16;
          bef[2 * w + 1] += hi16;
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < BPT; ++q) sm.hist[BPT * tid + q] = tot[q];  // 32-bit counts
  __syncthreads();
  RdxState st = rdx_start(n, k, 0u, 0xFFFFFFFFu);
  const int cnt = rdx_resolve<NT, NGRP, false>(sm, st, 0);
  const uint32_t bin = st.prefix >> st.sh0;  // the top digit (21-bit shift)
  const int m = (k - st.rem) + cnt;          // keys at or above it
  if (m > kLongCap) {  // block-uniform
    if (c == 0 && tid == 0) lcnt[row] = -1;
    return;
  }
  if (c == 0 && tid == 0) lcnt[row] = m;
  // this chunk's first slot: such keys in the earlier chunks
  int mine = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q)
    if ((uint32_t)(BPT * tid + q) >= bin) mine += (int)bef[q];
  const int wsum = wave_sum(mine);
  if (lane_id() == 0) sm.scan[1][tid / kWave] = wsum;
  // the chunk's keys; a key is kept when its top digit is at least `bin`
  // (bin > 0 here, as m < n: elements past the chunk, key 0, are never kept)
  const int mc = min(kTopkChunk, n - c0);
  uint32_t key[R];
  load_row_keys<NT, R>(scores + row * Lk + c0, mc, key);
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) off += sm.scan[1][w];
  RdxState keep = st;
  keep.prefix = bin << st.sh0;
  keep.done = true;
  keep.all = false;
  auto valid = [&](int r) { return elem_of<NT>(r) < mc; };
  u32x2* dst = lcand + row * kLongCap + off;
  rdx_emit_regs<NT, NGRP, 4, R>(key, mc, valid, keep, sm, 0, [&](int slot, uint32_t kv, int r) {
    dst[slot] = u32x2{kv, (uint32_t)(c0 + elem_of<NT>(r))};
  });
}

// Streaming count of level st.level over a whole score row into the 32-bit
// histogram, then its resolution (par: the level's slot parity).
template <int NT, int NGRP>
__device__ void stream_level(const float* src, int n, RdxSmem<NT, NGRP>& sm, RdxState& st,
                             int par) {
  const RowSrc rs = row_src(src, n);
  const int ng = (n + 3) / 4;
  const int L = st.level;
  constexpr int BATCH = 4;
  for (int g0 = 0; g0 < ng; g0 += NT * BATCH) {
    u32x4 raw[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) raw[q] = row_load4(rs, g0 + q * NT + (int)threadIdx.x);
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int g = g0 + q * NT + (int)threadIdx.x;
      row_fix_tail(rs, g, raw[q]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kv = order_key(__uint_as_float(raw[q][j]));
        if (4 * g + j < n && rdx_match(st, L, kv)) atomicAdd(&sm.hist[rdx_digit(st, L, kv)], 1u);
      }
    }
  }
  __syncthreads();
  rdx_resolve<NT, NGRP, false>(sm, st, par);
}

// ---------------------------------------------------------------------------
// Long rows, last launch: one 1024-thread workgroup per row (longest rows
// first). VB (rows of at most kWideRowCap scores, the only launch): the row
// is selected by value buckets as a whole, 64 scores per thread in registers;
// rows the buckets do not settle continue below, the top digit then counted
// over the row itself. Rows of at most kLongCap scores are loaded straight
// into registers; longer ones take the candidate list of the chunk-gather
// launch when it fit. Otherwise: the row's chunk histograms give the top digit; while the keys
// at or above the digits found so far exceed kLongCap, one more digit is
// resolved by a pass over the row; then a pass gathers those keys (for a
// fully resolved key: the keys above it and the first `rem` equal to it) into
// LDS in position order, and the selection finishes on them in registers.
// Dynamic LDS: RdxSmem, then kLongCap keys and kLongCap positions (the
// score-order words reuse the keys' area); the value buckets' scratch
// overlays them.
// ---------------------------------------------------------------------------
constexpr int kWideRowCap = 65536;  // scores a 1024-thread workgroup holds in registers
constexpr int kWideRowR = kWideRowCap / kWideThreads;
using WideVbSmem = RdxSmem<kWideThreads, kWideRowR / 4>;
using WideVbTies = VbSmemT<kWideThreads, kWideRowR / 4>;
constexpr size_t kWideOffTies = (sizeof(WideVbSmem) + 15) / 16 * 16;
constexpr size_t kWideOffWords = (kWideOffTies + sizeof(WideVbTies) + 15) / 16 * 16;
constexpr size_t kWideOffPos = kWideOffWords + (size_t)(kMaxK + 3 + 1) / 2 * 16;
constexpr size_t kWideVbBytes = kWideOffPos + (size_t)kMaxK * 4;

// Value-bucket selection of a row of n scores (at most kWideRowCap) by a
// 1024-thread workgroup, its LDS at dyn: true when done, false
// (block-uniform, LDS left dirty) when the buckets do not settle the row. The
// threshold is found as for the shorter rows; the winners then gather in the
// tie bitmap (each thread ORs in the bits of its scores above T, eight lanes'
// groups to a word), and leave by one block scan over its words in position
// order. Score order then reads the winners' scores back from the row (two
// per thread, both loads in flight) and ranks them.
template <int OUT>
__device__ __forceinline__ bool wide_vb_select(const float* src, int n, int k, uint8_t* dyn,
                                               int32_t* orow) {
  constexpr int NT = kWideThreads, R = kWideRowR, NGRP = R / 4, NW = NT / kWave;
  constexpr int kWords = NT * NGRP / 8;  // bitmap words: 32 positions each
  static_assert(kWords == 2 * NT, "two bitmap words per thread");
  WideVbSmem& sm = *reinterpret_cast<WideVbSmem*>(dyn);
  WideVbTies& vs = *reinterpret_cast<WideVbTies*>(dyn + kWideOffTies);
  uint64_t* words = reinterpret_cast<uint64_t*>(dyn + kWideOffWords);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  if (OUT == kOutScore && n <= k) {  // every score wins (the packed histogram is cleared)
    rdx_clear(sm, kSelBins / 2);
    uint32_t wmin = 0xFFFFFFFFu, wmax = 0u;
    for (int p = tid; p < n; p += NT) {
      const uint32_t kv = order_key(src[p]);
      words[p] = ((uint64_t)kv << 32) | (uint64_t)(~(uint32_t)p);
      wmin = min(wmin, kv);
      wmax = max(wmax, kv);
    }
    score_order_output<NT, NGRP>(words, n, k, wmin, wmax, sm, orow);
    return true;
  }
  rdx_clear(sm, kSelBins);
  vb_clear(vs);
  float x[R];
  load_row_floats<NT, R>(src, n, x);
  {
    float fmn, fmx;
    sample_range<NT, R>(x, n, fmn, fmx);
    uint32_t kmn = fmn <= fmx ? order_key(fmn) : 0xFFFFFFFFu;
    uint32_t kmx = fmn <= fmx ? order_key(fmx) : 0u;
    wave_minmax(kmn, kmx);
    if (lane == 0) {
      sm.red[wave] = kmn;
      sm.red[NW + wave] = kmx;
    }
  }
  __syncthreads();  // also orders the clears
  uint32_t klo = sm.red[0], khi = sm.red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    klo = min(klo, sm.red[w]);
    khi = max(khi, sm.red[NW + w]);
  }
  float sc = 0.0f, c = 0.0f, thr = 0.0f;
  int rem_eq = 0;
  if (!(vb_scale(key_to_float(klo), key_to_float(khi), sc, c) &&
        vb_threshold<NT, NGRP, R>(x, n, k, sc, c, sm, vs, thr, rem_eq)))
    return false;  // block-uniform
  // the scores above T join the winning ties in the bitmap: group g's four
  // bits go to bits 4 (g % 8) .. of word g / 8, the eight lanes of a word
  // combined by lane exchanges
  const int nvg = rdx_live_groups<NT>(n);
#pragma unroll
  for (int v = 0; v < NGRP; ++v) {
    if (v >= nvg) continue;  // workgroup-uniform
    const uint32_t m = (x[4 * v] > thr ? 1u : 0u) | (x[4 * v + 1] > thr ? 2u : 0u) |
                       (x[4 * v + 2] > thr ? 4u : 0u) | (x[4 * v + 3] > thr ? 8u : 0u);
    uint32_t w = m << (4 * (lane & 7));
    w |= lane_xor<1>(w);
    w |= lane_xor<2>(w);
    w |= lane_xor<4>(w);
    if ((lane & 7) == 0 && w != 0u) atomicOr(&vs.eqbits[(tid + NT * v) >> 3], w);
  }
  if (OUT == kOutScore) rdx_clear(sm, kSelBins / 2);  // for the ranks (the histogram is free)
  __syncthreads();
  // winners in position order: words 2 tid, 2 tid + 1, slots from a block scan
  const u32x2 bw = *reinterpret_cast<const u32x2*>(vs.eqbits + 2 * tid);
  const int cnt = __popc(bw[0]) + __popc(bw[1]);
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) sm.scan[0][wave] = incl;
  __syncthreads();
  int slot = incl - cnt;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) slot += sm.scan[0][w];
  // positions by slot: over the histogram (position order) or in an area of
  // their own (score order, whose ranks need the histogram clear)
  int* pbuf = OUT == kOutPos ? reinterpret_cast<int*>(sm.hist)
                             : reinterpret_cast<int*>(dyn + kWideOffPos);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t bits = bw[j];
    while (bits != 0u) {
      pbuf[slot++] = 32 * (2 * tid + j) + __ffs((int)bits) - 1;
      bits &= bits - 1u;
    }
  }
  __syncthreads();
  if (OUT == kOutPos) {
    store_row_positions<NT>(pbuf, k, k, orow);
  } else {
    constexpr int EPT = (kMaxK + NT - 1) / NT;
    int pv[EPT];
    float sv[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * NT;
      pv[e] = i < k ? pbuf[i] : 0;
      sv[e] = i < k ? src[pv[e]] : 0.0f;
    }
    uint32_t wmax = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid + e * NT;
      if (i < k) {
        const uint32_t kv = order_key(sv[e]);
        words[i] = ((uint64_t)kv << 32) | (uint64_t)(~(uint32_t)pv[e]);
        wmax = max(wmax, kv);
      }
    }
    // the least winner is T
    score_order_output<NT, NGRP>(words, k, k, order_key(thr), wmax, sm, orow);
  }
  return true;
}

template <int OUT, bool VB>
__global__ __launch_bounds__(kWideThreads)
void topk_long_kernel(const float* __restrict__ scores, int B, int Lq, int Lk, int q_pos0, int k,
                      int nch, const uint32_t* __restrict__ ghist,
                      const u32x2* __restrict__ lcand, const int* __restrict__ lcnt,
                      int32_t* __restrict__ out) {
  constexpr int NT = kWideThreads, R = kWideR, NGRP = R / 4, NW = NT / kWave;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  RdxSmem<NT, NGRP>& sm = *reinterpret_cast<RdxSmem<NT, NGRP>*>(dyn);
  constexpr size_t kOffKeys = (sizeof(RdxSmem<NT, NGRP>) + 15) / 16 * 16;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(dyn + kOffKeys);
  uint32_t* cpos = ckey + kLongCap;
  uint64_t* words = reinterpret_cast<uint64_t*>(ckey);  // score order, after the keys are read
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int i = Lq - 1 - (int)(blockIdx.x / (unsigned)B);
  const int b = (int)(blockIdx.x % (unsigned)B);
  const size_t row = (size_t)b * Lq + i;
  const int n = min(q_pos0 + i + 1, Lk);
  const float* src = scores + row * Lk;
  int32_t* orow = out + row * k;
  if (OUT == kOutPos && n <= k) {
    for (int j = tid; j < k; j += NT) orow[j] = j < n ? j : -1;
    return;
  }
  if constexpr (VB) {
    if (wide_vb_select<OUT>(src, n, k, dyn, orow)) return;  // block-uniform
    __syncthreads();  // the buckets' scratch is free
  }
  uint32_t key[R], pos[R], kmin, kmax;
  int m;  // elements held in registers
  if (n <= kLongCap) {
    rdx_clear(sm, kHistWords);
    load_row_keys<NT, R>(src, n, key, kmin, kmax);
#pragma unroll
    for (int r = 0; r < R; ++r) pos[r] = (uint32_t)elem_of<NT>(r);
    m = n;
  } else if (!VB && lcnt[row] >= 0) {
    // the row's candidate list from the previous launch (position-ordered,
    // a superset of the top-k holding every key equal to its least member)
    m = lcnt[row];
    rdx_clear(sm, kHistWords);  // the key-range barrier below ends the clear
    load_pair_list<NT, R>(lcand + row * kLongCap, m, key, pos);
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (elem_of<NT>(r) < m) {
        kmin = min(kmin, key[r]);
        kmax = max(kmax, key[r]);
      }
    }
  } else {
    // level 0 (the top 11 bits) from the chunk histograms, as 32-bit sums
    // (VB: counted over the row)
    RdxState st = rdx_start(n, k, 0u, 0xFFFFFFFFu);
    static_assert(kHistWords == NT, "one histogram word per thread");
    int par = 0, cnt;
    if constexpr (VB) {
      rdx_clear(sm, kSelBins);
      __syncthreads();
      stream_level<NT, NGRP>(src, n, sm, st, par);
      cnt = sm.bc[par][2];
    } else {
      // the chunks' words, kSumBatch loads in flight per thread
      const int nc = (n + kTopkChunk - 1) / kTopkChunk;
      constexpr int kSumBatch = 8;
      const uint32_t* gw = ghist + row * nch * kHistWords + tid;
      uint32_t lo = 0u, hi = 0u;
      for (int c0 = 0; c0 < nc; c0 += kSumBatch) {
        uint32_t v[kSumBatch];
#pragma unroll
        for (int q = 0; q < kSumBatch; ++q)
          v[q] = c0 + q < nc ? gw[(size_t)(c0 + q) * kHistWords] : 0u;
#pragma unroll
        for (int q = 0; q < kSumBatch; ++q) {
          lo += v[q] & 0xFFFFu;
          hi += v[q] >> 16;
        }
      }
      sm.hist[2 * tid] = lo;
      sm.hist[2 * tid + 1] = hi;
      __syncthreads();
      cnt = rdx_resolve<NT, NGRP, false>(sm, st, par);
    }
    // refine over the row while the keys at or above the digits found do
    // not fit in LDS
    while (!st.done && st.level < 3 && (k - st.rem) + cnt > kLongCap) {
      par ^= 1;
      stream_level<NT, NGRP>(src, n, sm, st, par);
      cnt = sm.bc[par][2];
    }
    // gather the keys at or above the digits found (a fully resolved key
    // with ties: those above it and the first `rem` equal to it), in
    // position order, four groups per thread between barriers
    const bool exact = st.level == 3 && !st.done;
    const uint32_t t = st.prefix;  // lo = 0: the threshold key itself
    const RowSrc rs = row_src(src, n);
    const int ng = (n + 3) / 4;
    int above_tot = 0, eq_tot = 0, buf = 0;
    constexpr int BATCH = NGRP;
    u32x4 raw[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) raw[q] = row_load4(rs, q * NT + tid);
    for (int g0 = 0; g0 < ng; g0 += NT * BATCH) {
      uint32_t kv[BATCH][4], keep[BATCH], eqm[BATCH];
      int cntq[BATCH], inc[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        row_fix_tail(rs, g0 + q * NT + tid, raw[q]);
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[q][j] = order_key(__uint_as_float(raw[q][j]));
      }
      // the next batch's loads, in flight while this one is gathered
#pragma unroll
      for (int q = 0; q < BATCH; ++q) raw[q] = row_load4(rs, g0 + NT * BATCH + q * NT + tid);
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int g = g0 + q * NT + tid;
        keep[q] = 0u;
        eqm[q] = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (4 * g + j < n) {
            const uint32_t kj = kv[q][j];
            if (exact ? kj > t : kj >= t) keep[q] |= 1u << j;
            else if (exact && kj == t) eqm[q] |= 1u << j;
          }
        }
        cntq[q] = __popc(keep[q]) | (__popc(eqm[q]) << 16);
        inc[q] = wave_incl_scan(cntq[q]);
        if (lane == kWave - 1) sm.wtot[buf][q * NW + wave] = inc[q];
      }
      __syncthreads();
      int base = 0;
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        int before = base, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int x = sm.wtot[buf][q * NW + w];
          if (w < wave) before += x;
          tot += x;
        }
        base += tot;
        const int excl = before + inc[q] - cntq[q];
        int eq_before = eq_tot + (excl >> 16);
        int slot = above_tot + (excl & 0xFFFF) + min(eq_before, st.rem);
        const int g = g0 + q * NT + tid;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((keep[q] >> j) & 1u) {
            ckey[slot] = kv[q][j];
            cpos[slot] = (uint32_t)(4 * g + j);
            ++slot;
          } else if ((eqm[q] >> j) & 1u) {
            if (eq_before < st.rem) {
              ckey[slot] = kv[q][j];
              cpos[slot] = (uint32_t)(4 * g + j);
              ++slot;
            }
            ++eq_before;
          }
        }
      }
      above_tot += base & 0xFFFF;
      eq_tot += base >> 16;
      buf ^= 1;
    }
    m = above_tot + (exact ? min(eq_tot, st.rem) : 0);
    __syncthreads();  // the gathered keys are in LDS
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = elem_of<NT>(r);
      key[r] = e < m ? ckey[e] : 0u;
      pos[r] = e < m ? cpos[e] : 0u;
      if (e < m) {
        kmin = min(kmin, key[r]);
        kmax = max(kmax, key[r]);
      }
    }
    // the selection restarts on the gathered keys (a superset of the row's
    // top-k holding every key equal to its least member) with digits over
    // their own range; rdx_resolve left the histogram zero
  }
  uint32_t lo, hi;
  rdx_key_range(kmin, kmax, sm, lo, hi);  // also: every gathered key is read
  auto valid = [&](int r) { return elem_of<NT>(r) < m; };
#pragma unroll
  for (int r = 0; r < R; ++r) key[r] = valid(r) ? key[r] - lo : 0u;  // rel, padded
  RdxState st = rdx_start(m, k, lo, hi);
  rdx_search_regs<NT, NGRP, R>(key, m, sm, st);
  if (OUT == kOutPos) {
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, m, valid, st, sm, 0, [&](int slot, uint32_t, int r) { orow[slot] = (int32_t)pos[r]; });
    for (int j = kk + tid; j < k; j += NT) orow[j] = -1;
  } else {
    uint32_t wmin = 0xFFFFFFFFu, wmax = 0u;
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, m, valid, st, sm, 0, [&](int slot, uint32_t rv, int r) {
          const uint32_t kv = rv + lo;
          words[slot] = ((uint64_t)kv << 32) | (uint64_t)(~pos[r]);
          wmin = min(wmin, kv);
          wmax = max(wmax, kv);
        });
    score_order_output<NT, NGRP>(words, kk, k, wmin, wmax, sm, orow);
  }
}

// ---------------------------------------------------------------------------
// Candidate lists. SRC kSrcCand1: row r's list at cand + r*seg_cap, count
// cand_count[r] (<= NT*R). SRC kSrcCandSeg: segments s0..s0+ns-1 of the row
// (all of them, or group `grp` of nseg / ngroups consecutive ones), whose
// concatenation is position-ordered. OUT: final indices (position or score
// order, a.pos_order) or, kOutPart, the group's winners as (key, position)
// pairs into a.part (count in a.part_count).
// ---------------------------------------------------------------------------
// (position-order prefill lists of up to 5120 pairs run six waves per SIMD:
// 218 vs 233 us per 32768-row layer, two registers spilled once)
template <int SRC, int OUT, int NT, int R>
__global__ __launch_bounds__(NT, (OUT == kOutPos && NT == kRowThreads && R <= 20) ? 6 : 1)
void topk_pairs_kernel(TopkArgs a, int ngroups) {
  constexpr int NGRP = R / 4;
  __shared__ RdxSmem<NT, NGRP> sm;
  __shared__ uint64_t words[OUT == kOutScore ? kMaxK + 3 : 2];  // + padding of the bucket ranks
  __shared__ int seg_off[kMaxSegments + 1];
  const int tid = threadIdx.x;
  const int row = (int)(blockIdx.x / (unsigned)ngroups);
  const int grp = (int)(blockIdx.x % (unsigned)ngroups);
  const int k = a.k;
  rdx_clear(sm, kHistWords);
  uint32_t key[R], pos[R];
  int n;
  if (SRC == kSrcCand1) {
    n = a.cand_count[row];
    load_pair_list<NT, R>(a.cand + (size_t)row * a.seg_cap, n, key, pos);
  } else {
    const int per_group = (a.nseg + ngroups - 1) / ngroups;
    const int s0 = min(a.nseg, grp * per_group);
    const int ns = min(a.nseg, s0 + per_group) - s0;
    if (tid == 0) {
      int off = 0;
      for (int s = 0; s < ns; ++s) {
        seg_off[s] = off;
        off += a.cand_count[(size_t)row * a.nseg + s0 + s];
      }
      seg_off[ns] = off;
    }
    __syncthreads();
    n = seg_off[ns];
    const u32x2* base = a.cand + ((size_t)row * a.nseg + s0) * a.seg_cap;
    int s = 0;  // elements grow with r: the segment search resumes
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = elem_of<NT>(r);
      u32x2 p = u32x2{0u, 0u};
      if (e < n) {
        while (s + 1 < ns && seg_off[s + 1] <= e) ++s;
        p = base[(size_t)s * a.seg_cap + (e - seg_off[s])];
      }
      key[r] = p[0];
      pos[r] = p[1];
    }
  }
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, lo, hi;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (elem_of<NT>(r) < n) {
      kmin = min(kmin, key[r]);
      kmax = max(kmax, key[r]);
    }
  }
  rdx_key_range(kmin, kmax, sm, lo, hi);  // its barrier also ends the clear
  auto valid = [&](int r) { return elem_of<NT>(r) < n; };
#pragma unroll
  for (int r = 0; r < R; ++r) key[r] = valid(r) ? key[r] - lo : 0u;  // rel, padded
  RdxState st = rdx_start(n, k, lo, hi);
  rdx_search_regs<NT, NGRP, R>(key, n, sm, st);
  if (OUT == kOutPart) {
    u32x2* part = a.part + ((size_t)row * ngroups + grp) * k;
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, n, valid, st, sm, 0,
        [&](int slot, uint32_t rv, int r) { part[slot] = u32x2{rv + lo, pos[r]}; });
    if (tid == 0) a.part_count[(size_t)row * ngroups + grp] = kk;
    return;
  }
  int32_t* orow = a.out + (size_t)row * k;
  if (OUT == kOutPos) {
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, n, valid, st, sm, 0, [&](int slot, uint32_t, int r) { orow[slot] = (int32_t)pos[r]; });
    for (int j = kk + tid; j < k; j += NT) orow[j] = -1;
  } else {
    uint32_t wmin = 0xFFFFFFFFu, wmax = 0u;
    const int kk = rdx_emit_regs<NT, NGRP, 4, R>(
        key, n, valid, st, sm, 0, [&](int slot, uint32_t rv, int r) {
          const uint32_t kv = rv + lo;
          words[slot] = ((uint64_t)kv << 32) | (uint64_t)(~pos[r]);
          wmin = min(wmin, kv);
          wmax = max(wmax, kv);
        });
    score_order_output<NT, NGRP>(words, kk, k, wmin, wmax, sm, orow);
  }
}

template <int SRC, int OUT, int NT, int R>
hipError_t launch_pairs(const TopkArgs& a, int ngroups, hipStream_t st) {
  hipLaunchKernelGGL((topk_pairs_kernel<SRC, OUT, NT, R>), dim3((unsigned)(a.rows * ngroups)),
                     dim3(NT), 0, st, a, ngroups);
  return hipGetLastError();
}

template <int SRC, int NT, int R>
hipError_t launch_pairs_final(const TopkArgs& a, int ngroups, hipStream_t st) {
  return a.pos_order ? launch_pairs<SRC, kOutPos, NT, R>(a, ngroups, st)
                     : launch_pairs<SRC, kOutScore, NT, R>(a, ngroups, st);
}

// Scratch of long materialised rows, in a.ghist: the chunk histograms, then
// (rows longer than kLongCap) kLongCap candidate pairs and a count per row.
size_t hist_bytes(int rows, int nch) { return (size_t)rows * nch * kHistWords * 4; }
u32x2* topk_lcand(const TopkArgs& a, int nch) {
  return reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.ghist) + hist_bytes(a.rows, nch));
}
int* topk_lcnt(const TopkArgs& a, int nch) {
  return reinterpret_cast<int*>(topk_lcand(a, nch) + (size_t)a.rows * kLongCap);
}

constexpr size_t kLongLdsBytes =
    (sizeof(RdxSmem<kWideThreads, kWideR / 4>) + 15) / 16 * 16 + (size_t)kLongCap * 8;
static_assert(kWideVbBytes <= kLongLdsBytes, "the value buckets' scratch overlays the long rows'");

// VB: rows of at most kWideRowCap scores in this launch alone (no scratch).
template <int OUT, bool VB>
hipError_t launch_long(const TopkArgs& a, int nch, hipStream_t st) {
  const size_t shmem = kLongLdsBytes;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_long_kernel<OUT, VB>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  if (e != hipSuccess) return e;
  const int B = a.rows / a.Lq;
  hipLaunchKernelGGL((topk_long_kernel<OUT, VB>), dim3((unsigned)a.rows), dim3(kWideThreads),
                     shmem, st, a.scores, B, a.Lq, a.Lk, a.q_pos0, a.k, nch,
                     VB ? nullptr : reinterpret_cast<const uint32_t*>(a.ghist),
                     VB ? nullptr : topk_lcand(a, nch), VB ? nullptr : topk_lcnt(a, nch), a.out);
  return hipGetLastError();
}

}  // namespace

int topk_row_chunks(int Lk) { return (Lk + kTopkChunk - 1) / kTopkChunk; }

size_t topk_part_bytes(int rows, int Lk, int k) {
  (void)k;
  const int nch = topk_row_chunks(Lk);
  if (nch <= 1 || Lk <= kWideRowCap) return 0;  // one launch, no scratch
  size_t b = hist_bytes(rows, nch);
  if (Lk > kLongCap) b += (size_t)rows * kLongCap * 8 + (size_t)rows * 4;
  return b;
}

int topk_segment_groups(int nseg, int k) {
  if ((long long)nseg * k <= kMaxStagePairs) return 1;
  const int per_group = kMaxStagePairs / k;  // segments one workgroup stages
  const int groups = (nseg + per_group - 1) / per_group;
  return (long long)groups * k <= kMaxStagePairs ? groups : 0;
}

size_t topk_group_bytes(int rows, int nseg, int k) {
  const int g = topk_segment_groups(nseg, k);
  if (g <= 1) return 0;
  return (size_t)rows * g * k * 8 + (size_t)rows * g * 4 + 256;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.cand) {
    if (a.nseg == 1) {
      // one position-ordered list per row (the fused indexer's candidates)
      // the fewest registers that hold the list: fewer registers, more waves
      // per SIMD (20 pairs per thread: 82 VGPRs, five waves; 32: 110, four;
      // 239 vs 315 us on the 32768-row prefill layer's lists of up to 5120)
      if (a.stage_cap <= kRowThreads * 20) return launch_pairs_final<kSrcCand1, kRowThreads, 20>(a, 1, st);
      if (a.stage_cap <= kRowThreads * 28) return launch_pairs_final<kSrcCand1, kRowThreads, 28>(a, 1, st);
      if (a.stage_cap <= kTopkChunk) return launch_pairs_final<kSrcCand1, kRowThreads, kRowR>(a, 1, st);
      return launch_pairs_final<kSrcCand1, kWideThreads, kWideR>(a, 1, st);
    }
    const int groups = topk_segment_groups(a.nseg, a.k);
    // (up to four 2048-entry segments, a 65536-key decode row: 8 pairs per
    // thread, half the per-thread work of 16; 13.2 vs 14.2 us)
    if (groups <= 1 && a.stage_cap <= kWideThreads * 8) return launch_pairs_final<kSrcCandSeg, kWideThreads, 8>(a, 1, st);
    if (groups <= 1) return launch_pairs_final<kSrcCandSeg, kWideThreads, kWideR>(a, 1, st);
    // too many segments for one workgroup: the exact top-k of each group of
    // consecutive segments (into a.part), then of the groups' winners (every
    // key of the row's top-k is in its group's top-k)
    hipError_t e = launch_pairs<kSrcCandSeg, kOutPart, kWideThreads, kWideR>(a, groups, st);
    if (e != hipSuccess) return e;
    TopkArgs f = a;
    f.cand = a.part;
    f.cand_count = a.part_count;
    f.nseg = groups;
    f.seg_cap = a.k;
    return launch_pairs_final<kSrcCandSeg, kWideThreads, kWideR>(f, 1, st);
  }
  const int B = a.rows / a.Lq;
  const int nch = topk_row_chunks(a.Lk);
  if (nch <= 1) {
    if (a.pos_order)
      hipLaunchKernelGGL((topk_rows_kernel<kOutPos>), dim3((unsigned)a.rows), dim3(kRowThreads), 0,
                         st, a.scores, B, a.Lq, a.Lk, a.q_pos0, a.k, a.out);
    else
      hipLaunchKernelGGL((topk_rows_kernel<kOutScore>), dim3((unsigned)a.rows),
                         dim3(kRowThreads), 0, st, a.scores, B, a.Lq, a.Lk, a.q_pos0, a.k, a.out);
    return hipGetLastError();
  }
  // rows of up to kWideRowCap scores: one 1024-thread workgroup per row
  if (a.Lk <= kWideRowCap)
    return a.pos_order ? launch_long<kOutPos, true>(a, nch, st)
                       : launch_long<kOutScore, true>(a, nch, st);
  // longer rows: per-chunk histograms of the top digit, then one workgroup per row
  hipLaunchKernelGGL(topk_chunk_hist_kernel, dim3((unsigned)((size_t)a.rows * nch)),
                     dim3(kRowThreads), 0, st, a.scores, a.Lq, a.Lk, a.q_pos0, nch,
                     reinterpret_cast<uint32_t*>(a.ghist));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.Lk > kLongCap) {
    // rows longer than kLongCap: each chunk adds its share of the row's
    // candidate list
    hipLaunchKernelGGL(topk_chunk_gather_kernel, dim3((unsigned)((size_t)a.rows * nch)),
                       dim3(kRowThreads), 0, st, a.scores, a.Lq, a.Lk, a.q_pos0, a.k, nch,
                       reinterpret_cast<const uint32_t*>(a.ghist), topk_lcand(a, nch),
                       topk_lcnt(a, nch));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return a.pos_order ? launch_long<kOutPos, false>(a, nch, st)
                     : launch_long<kOutScore, false>(a, nch, st);
}

}  // namespace idxc
