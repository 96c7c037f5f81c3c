// Per-query top-k for gfx950: one workgroup per query row.
//
// I_l = TopK(s_l, k) ("IndexCache：跨层复用稀疏注意力的索引", section
// "从 DSA 的成本分解开始"); the order is fixed as higher score first, then
// lower position, with -0.0 == +0.0, and rows shorter than k return all of
// their t+1 positions followed by -1.
//
// Scores become order-preserving 32-bit keys. A radix select (8 bits per
// pass, per-wave LDS histograms) finds the key T of the k-th best entry and
// how many entries equal to T are still needed; an ordered pass then keeps
// every key above T and the lowest-position entries equal to T; a bitonic sort
// in LDS of 64-bit (key, ~position) words puts the k winners in order. The
// input is either a materialised score row (positions implicit) or a candidate
// list of (score, position) pairs in increasing position order. Rows that fit
// are staged in LDS once; longer rows are re-read from global memory (L2).
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStageBytes = 40 * 1024;
constexpr int kStageKeys = kStageBytes / 4;      // materialised rows
constexpr int kStagePairs = kStageBytes / 8;     // candidate lists
constexpr int kPerThread = 8;                    // ordered pass: consecutive entries
constexpr int kChunk = kThreads * kPerThread;

struct Smem {
  uint64_t sortbuf[kMaxK];
  uint32_t hist[kWaves * 256];
  int scan[kWaves];
  int bcast[4];
};

// Block-wide exclusive prefix sum; *total gets the block total.
__device__ __forceinline__ int block_excl_scan(int v, int* scan, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scan[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = scan[w];
    if (w < wave) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

template <bool CAND>
struct RowSource {
  // materialised
  const float* srow;
  // candidates
  const u32x2* crow;
  // staging
  const uint32_t* skeys;
  const u32x2* spairs;
  bool staged;

  __device__ __forceinline__ void fetch(int e, uint32_t& key, uint32_t& pos) const {
    if (CAND) {
      u32x2 v = staged ? spairs[e] : crow[e];
      key = staged ? v.x : order_key(__uint_as_float(v.x));
      pos = v.y;
    } else {
      key = staged ? skeys[e] : order_key(srow[e]);
      pos = (uint32_t)e;
    }
  }
};

template <bool CAND>
__global__ __launch_bounds__(kThreads)
void topk_rows_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  Smem& sm = *reinterpret_cast<Smem*>(dyn);
  uint8_t* stage = dyn + sizeof(Smem);

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int k = a.k;

  int n;
  RowSource<CAND> src;
  src.srow = nullptr;
  src.crow = nullptr;
  if (CAND) {
    n = a.cand_count[row];
    src.crow = a.cand + (size_t)row * a.cap;
  } else {
    const int i = row % a.Lq;
    n = min(a.q_pos0 + i + 1, a.Lk);
    src.srow = a.scores + (size_t)row * a.Lk;
  }
  src.skeys = reinterpret_cast<const uint32_t*>(stage);
  src.spairs = reinterpret_cast<const u32x2*>(stage);
  src.staged = CAND ? (n <= kStagePairs) : (n <= kStageKeys);

  if (src.staged) {
    if (CAND) {
      u32x2* sp = reinterpret_cast<u32x2*>(stage);
      for (int e = tid; e < n; e += kThreads) {
        u32x2 v = src.crow[e];
        sp[e] = u32x2{order_key(__uint_as_float(v.x)), v.y};
      }
    } else {
      uint32_t* sk = reinterpret_cast<uint32_t*>(stage);
      for (int e = tid; e < n; e += kThreads) sk[e] = order_key(src.srow[e]);
    }
    __syncthreads();
  }

  // ---- radix select of the k-th best key (only needed when n > k)
  uint32_t prefix = 0u;
  int rem = 0;
  const bool select_all = n <= k;
  if (!select_all) {
    uint32_t pmask = 0u;
    rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < kWaves * 256; b += kThreads) sm.hist[b] = 0u;
      __syncthreads();
      uint32_t* wh = sm.hist + wave * 256;
      for (int e = tid; e < n; e += kThreads) {
        uint32_t key, pos;
        src.fetch(e, key, pos);
        if ((key & pmask) == prefix) atomicAdd(&wh[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      const int bin = 255 - tid;  // descending bins across threads
      int cnt = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) cnt += (int)sm.hist[w * 256 + bin];
      int total;
      const int excl = block_excl_scan(cnt, sm.scan, &total);
      if (excl < rem && excl + cnt >= rem) {
        sm.bcast[0] = bin;
        sm.bcast[1] = excl;
      }
      __syncthreads();
      prefix |= ((uint32_t)sm.bcast[0]) << shift;
      pmask |= 255u << shift;
      rem -= sm.bcast[1];
      __syncthreads();
    }
  }

  // ---- ordered collection into the sort buffer (entries kept in position
  // order; equal-to-T entries limited to the `rem` lowest positions)
  int out_count = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kChunk) {
    uint32_t keys[kPerThread], poss[kPerThread];
    unsigned gt_bits = 0u, eq_bits = 0u;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int e = base + tid * kPerThread + j;
      keys[j] = 0u;
      poss[j] = 0u;
      if (e < n) {
        src.fetch(e, keys[j], poss[j]);
        if (select_all || keys[j] > prefix) gt_bits |= 1u << j;
        else if (keys[j] == prefix) eq_bits |= 1u << j;
      }
    }
    int eq_total;
    const int eq_excl = eq_seen + block_excl_scan(__popc(eq_bits), sm.scan, &eq_total);
    unsigned keep_bits = gt_bits;
    int r = eq_excl;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (eq_bits & (1u << j)) {
        if (r < rem) keep_bits |= 1u << j;
        ++r;
      }
    }
    int keep_total;
    int pos = out_count + block_excl_scan(__popc(keep_bits), sm.scan, &keep_total);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if (keep_bits & (1u << j)) {
        sm.sortbuf[pos++] = (((uint64_t)keys[j]) << 32) | (uint64_t)(~poss[j]);
      }
    }
    out_count += keep_total;
    eq_seen += eq_total;
  }
  const int kk = out_count;  // == min(k, n)

  // ---- bitonic sort, descending, of the kk winners padded to a power of two
  int P = 1;
  while (P < kk) P <<= 1;
  for (int e = kk + tid; e < P; e += kThreads) sm.sortbuf[e] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P >> 1); i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = sm.sortbuf[lo], y = sm.sortbuf[hi];
        const bool desc = (lo & size) == 0;
        if ((x < y) == desc) {
          sm.sortbuf[lo] = y;
          sm.sortbuf[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  int32_t* orow = a.out + (size_t)row * k;
  for (int j = tid; j < k; j += kThreads) {
    orow[j] = (j < kk) ? (int32_t)(~(uint32_t)(sm.sortbuf[j] & 0xFFFFFFFFull)) : -1;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const size_t shmem = sizeof(Smem) + kStageBytes;
  dim3 grid((unsigned)a.rows), block(kThreads);
  if (a.cand) {
    hipLaunchKernelGGL(topk_rows_kernel<true>, grid, block, shmem, st, a);
  } else {
    hipLaunchKernelGGL(topk_rows_kernel<false>, grid, block, shmem, st, a);
  }
  return hipGetLastError();
}

}  // namespace idxc
