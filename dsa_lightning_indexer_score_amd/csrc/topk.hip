// Per-query top-k for gfx950.
//
// I_l = TopK(s_l, k) ("IndexCache：跨层复用稀疏注意力的索引", section
// "从 DSA 的成本分解开始"); the order is fixed as higher score first, then
// lower position, with -0.0 == +0.0, and rows shorter than k return all of
// their t+1 positions followed by -1.
//
// Scores become order-preserving 32-bit keys. A workgroup stages its input in
// LDS once (loads batched so many are in flight), selects the exact top-k in
// position order (select.hpp: range-narrowing radix select plus an ordered
// pass), and a bitonic sort of 64-bit (key, ~position) words puts the k
// winners in score order (in the wide final stage of long rows, ranks from key
// buckets when the scores are spread out); the index cache of a layer stack
// keeps them in position order instead (gathers then sweep the keys in
// order), which needs no sort.
//
// Inputs: a materialised score row (positions implicit), or candidate lists of
// (order key, position) pairs in increasing position order, possibly split in
// segments whose concatenation is position-ordered. Rows longer than one
// workgroup's stage are cut into chunks; each chunk's exact top-k is written
// as a position-ordered candidate segment (stage 1) and a second launch
// selects from the concatenated segments (stage 2). Every entry of the final
// top-k is in its chunk's top-k, so the result is the same.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace idxc {

namespace {

constexpr int kThreads = kSelThreads;
// multi-segment selections (few rows, up to 16384 candidates each) use wider
// workgroups: there are few of them, so latency per row is what counts
constexpr int kThreadsWide = 1024;
constexpr int kBatch = 8;  // staged loads in flight per thread
static_assert(kTopkChunk <= kSelMaxKeys && kMaxStagePairs <= kSelMaxKeys,
              "selection histogram counts fit 16 bits");

// LDS: segment offsets and selection scratch, then the staged keys, then
// (multi-segment candidate lists only) the staged positions. Score-order
// output sorts its winners in a buffer laid over the selection histogram
// (which the winners' collection no longer reads), extended past the end of
// the scratch, so the staged keys start after it. Position-order output needs
// no sort buffer, and single-segment lists read their winners' positions
// back from memory, so the common candidate case stages keys alone.
template <int NT>
struct Smem {
  int seg_off[kMaxSegments + 1];
  SelectSmemT<NT> sel;  // histogram last
};
template <int NT>
constexpr size_t smem_bytes() {
  return (sizeof(Smem<NT>) + 15) / 16 * 16;
}
template <int NT>
constexpr size_t sort_off() {
  return offsetof(Smem<NT>, sel) + offsetof(SelectSmemT<NT>, hist);
}
constexpr size_t kSortBytes = (size_t)kMaxK * 8;

enum SrcKind { kSrcRow = 0, kSrcCand = 1, kSrcCand1 = 2 };
enum OutKind { kOutFinal = 0, kOutPart = 1 };

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

// Score order by bucket ranks. The kk winners' 64-bit words (key, ~position)
// sit in sortbuf in position order, and their keys span [wlo, whi]; split
// that range into kSelBins buckets of one power-of-two width. A winner's rank
// is the number of winners in higher buckets plus the number of larger words
// in its own bucket (words are distinct: positions are). `scratch` (8 KB of
// LDS) takes the packed 16-bit bucket cursors, then the buckets' members as
// 16-bit slots. Returns false, having written no output, when a bucket holds
// more than kMaxBucket winners (scores bunched on few values, or spread over
// many binades): the caller then sorts.
constexpr int kMaxBucket = 64;
constexpr int kBucketScratchBytes = kSelBins / 2 * 4 + kMaxK * 2;

template <int NT>
__device__ bool bucket_rank_output(uint64_t* sortbuf, int kk, int k, uint32_t wlo,
                                   uint32_t whi, uint32_t* scratch, SelectSmemT<NT>& sm,
                                   int32_t* orow) {
  constexpr int BPT = kSelBins / NT;  // buckets per thread
  const int tid = threadIdx.x;
  uint32_t* cur = scratch;  // kSelBins / 2 words, bucket b in half b % 2 of word b / 2
  uint16_t* mem = reinterpret_cast<uint16_t*>(scratch + kSelBins / 2);
  const int shift = max(0, (32 - __clz((int)(whi - wlo))) - kSelBinsLog2);
  auto bucket_of = [&](uint64_t w) { return ((uint32_t)(w >> 32) - wlo) >> shift; };
  for (int b = tid; b < kSelBins / 2; b += NT) cur[b] = 0u;
  __syncthreads();
  for (int sl = tid; sl < kk; sl += NT) {
    const uint32_t b = bucket_of(sortbuf[sl]);
    atomicAdd(&cur[b >> 1], 1u << ((b & 1u) << 4));
  }
  __syncthreads();
  // bucket starts in descending bucket order: thread tid owns buckets
  // top - q, q = 0..BPT-1 (top is odd: buckets top - q and top - q - 1 share
  // a word for even q)
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
  const int excl = sel_excl_scan<NT>(local, sm.scan, &total);
  wave_minmax(unused, most);
  if (lane_id() == 0) sm.kred[tid / kWave] = most;
  __syncthreads();
  uint32_t bmax = 0u;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) bmax = max(bmax, sm.kred[w]);
  if (bmax > (uint32_t)kMaxBucket) return false;  // block-uniform
  int acc = excl;
#pragma unroll
  for (int q = 0; q < BPT; q += 2) {
    const uint32_t start_hi = (uint32_t)acc;
    acc += cnts[q];
    cur[(top - q) >> 1] = (start_hi << 16) | (uint32_t)acc;
    acc += cnts[q + 1];
  }
  __syncthreads();
  for (int sl = tid; sl < kk; sl += NT) {
    const uint32_t b = bucket_of(sortbuf[sl]);
    const uint32_t sh = (b & 1u) << 4;
    const uint32_t old = atomicAdd(&cur[b >> 1], 1u << sh);
    mem[(old >> sh) & 0xFFFFu] = (uint16_t)sl;
  }
  __syncthreads();
  // each cursor now holds its bucket's end; bucket b starts where bucket b+1
  // (the next higher one) ends
  auto end_of = [&](uint32_t b) { return (cur[b >> 1] >> ((b & 1u) << 4)) & 0xFFFFu; };
  constexpr int EPT = kMaxK / NT;  // winners per thread at most
  uint32_t rk[EPT], pv[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int sl = tid + i * NT;
    rk[i] = 0u;
    pv[i] = 0u;
    if (sl < kk) {
      const uint64_t w = sortbuf[sl];
      const uint32_t b = bucket_of(w);
      const uint32_t e = end_of(b);
      const uint32_t st = b + 1 < (uint32_t)kSelBins ? end_of(b + 1) : 0u;
      uint32_t rank = st;
      for (uint32_t j = st; j < e; ++j) rank += sortbuf[mem[j]] > w ? 1u : 0u;
      rk[i] = rank;
      pv[i] = ~(uint32_t)(w & 0xFFFFFFFFull);
    }
  }
  // the row in rank order through LDS (over the words, all read by now), so
  // that it is written with coalesced stores
  __syncthreads();
  uint32_t* obuf = reinterpret_cast<uint32_t*>(sortbuf);
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (tid + i * NT < kk) obuf[rk[i]] = pv[i];
  __syncthreads();
  for (int j = tid; j < k; j += NT) orow[j] = j < kk ? (int32_t)obuf[j] : -1;
  return true;
}

// One workgroup = one (row, chunk). SRC kSrcRow: positions [c0, c1) of a score
// row. SRC kSrcCand: the concatenation of nseg segments of a row (positions
// staged too). SRC kSrcCand1: one segment (positions read back for winners).
// The staged input starts at byte stage_off of the dynamic LDS.
template <int SRC, int OUT, int NT>
__global__ __launch_bounds__(NT)
void topk_kernel(TopkArgs a, int chunk_len, int nchunks, int stage_off, int stage_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  Smem<NT>& sm = *reinterpret_cast<Smem<NT>*>(dyn);
  uint32_t* skey = reinterpret_cast<uint32_t*>(dyn + stage_off);
  uint32_t* spos = nullptr;  // SRC kSrcCand: positions after the keys
  uint64_t* sortbuf = reinterpret_cast<uint64_t*>(dyn + sort_off<NT>());

  const int tid = threadIdx.x;
  const int k = a.k;
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;

  // ---- stage the input in LDS (keys, and positions for candidate lists),
  // noting the range of the keys this thread stores
  int n;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  int pos0 = 0;  // kSrcRow: position of entry 0
  if (SRC == kSrcRow) {
    const int i = row % a.Lq;
    const int len = min(a.q_pos0 + i + 1, a.Lk);
    pos0 = chunk * chunk_len;
    n = max(0, min(len, pos0 + chunk_len) - pos0);
    const float* src = a.scores + (size_t)row * a.Lk + pos0;
    int done = 0;
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      // 16-byte loads (4 keys each), kBatch of them in flight per thread
      const int n4 = n >> 2;
      const f32x4* src4 = reinterpret_cast<const f32x4*>(src);
      for (int base = 0; base < n4; base += NT * kBatch) {
        f32x4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          v[j] = e < n4 ? src4[e] : f32x4{};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          if (e < n4) {
            const u32x4 kv = u32x4{order_key(v[j][0]), order_key(v[j][1]),
                                   order_key(v[j][2]), order_key(v[j][3])};
            *reinterpret_cast<u32x4*>(skey + 4 * e) = kv;
            kmin = min(min(kmin, min(kv[0], kv[1])), min(kv[2], kv[3]));
            kmax = max(max(kmax, max(kv[0], kv[1])), max(kv[2], kv[3]));
          }
        }
      }
      done = n4 * 4;
    }
    // the rest: a tail of up to 3 keys, or a row that is not 16-byte aligned
    for (int base = done; base < n; base += NT * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int e = base + j * NT + tid;
        v[j] = e < n ? src[e] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int e = base + j * NT + tid;
        if (e < n) {
          const uint32_t key = order_key(v[j]);
          skey[e] = key;
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
      }
    }
  } else if (SRC == kSrcCand1) {
    n = a.cand_count[row];
    const u32x2* src = a.cand + (size_t)row * a.seg_cap;
    int done = 0;
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      // 16-byte loads (2 pairs each), kBatch of them in flight per thread
      const int n2 = n >> 1;
      const u32x4* src2 = reinterpret_cast<const u32x4*>(src);
      for (int base = 0; base < n2; base += NT * kBatch) {
        u32x4 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          v[j] = e < n2 ? src2[e] : u32x4{};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          if (e < n2) {
            *reinterpret_cast<u32x2*>(skey + 2 * e) = u32x2{v[j][0], v[j][2]};
            kmin = min(kmin, min(v[j][0], v[j][2]));
            kmax = max(kmax, max(v[j][0], v[j][2]));
          }
        }
      }
      done = n2 * 2;
    }
    for (int base = done; base < n; base += NT * kBatch) {
      uint32_t v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int e = base + j * NT + tid;
        v[j] = e < n ? src[e].x : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int e = base + j * NT + tid;
        if (e < n) {
          skey[e] = v[j];
          kmin = min(kmin, v[j]);
          kmax = max(kmax, v[j]);
        }
      }
    }
  } else {
    // segments [s0, s1) of the row: all of them (nchunks = 1), or group
    // `chunk` of ceil(nseg / nchunks) consecutive segments (a stage of a
    // two-level selection); consecutive segments keep position order
    const int per_group = (a.nseg + nchunks - 1) / nchunks;
    const int s0 = min(a.nseg, chunk * per_group);
    const int ns = min(a.nseg, s0 + per_group) - s0;
    if (tid == 0) {
      int off = 0;
      for (int s = 0; s < ns; ++s) {
        sm.seg_off[s] = off;
        off += a.cand_count[row * a.nseg + s0 + s];
      }
      sm.seg_off[ns] = off;
    }
    __syncthreads();
    n = sm.seg_off[ns];
    spos = skey + a.stage_cap;
    for (int s = 0; s < ns; ++s) {
      const int off = sm.seg_off[s];
      const int cnt = sm.seg_off[s + 1] - off;
      const u32x2* src = a.cand + ((size_t)row * a.nseg + s0 + s) * a.seg_cap;
      for (int base = 0; base < cnt; base += NT * kBatch) {
        u32x2 v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          v[j] = e < cnt ? src[e] : u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * NT + tid;
          if (e < cnt) {
            skey[off + e] = v[j].x;
            kmin = min(kmin, v[j].x);
            kmax = max(kmax, v[j].x);
            spos[off + e] = v[j].y;
          }
        }
      }
    }
  }
  sel_store_key_range<NT>(kmin, kmax, sm.sel);
  __syncthreads();

  u32x2* part = nullptr;
  if (OUT == kOutPart) part = a.part + ((size_t)row * nchunks + chunk) * a.k;
  int32_t* orow = a.out + (size_t)row * k;
  const bool pos_order = OUT == kOutFinal && a.pos_order;
  const u32x2* cand1 = (SRC == kSrcCand1) ? a.cand + (size_t)row * a.seg_cap : nullptr;
  // positions of a group of kSelPerThread consecutive entries (those of `bits`)
  const bool cand1_aligned =
      SRC == kSrcCand1 && (reinterpret_cast<uintptr_t>(cand1) & 15) == 0;
  auto pos_group = [&](int e0, unsigned bits, uint32_t (&pv)[kSelPerThread]) {
    if (SRC == kSrcRow) {
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j) pv[j] = (uint32_t)(pos0 + e0 + j);
    } else if (SRC == kSrcCand) {
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j) pv[j] = ((bits >> j) & 1u) ? spos[e0 + j] : 0u;
    } else if (cand1_aligned && bits != 0u && e0 + kSelPerThread <= n) {
      // the group's pairs in four 16-byte loads (positions are the odd words)
      const u32x4* g = reinterpret_cast<const u32x4*>(cand1 + e0);
#pragma unroll
      for (int q = 0; q < kSelPerThread / 2; ++q) {
        const u32x4 w = g[q];
        pv[2 * q] = w[1];
        pv[2 * q + 1] = w[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j) pv[j] = ((bits >> j) & 1u) ? cand1[e0 + j].y : 0u;
    }
  };
  uint32_t wmin = 0xFFFFFFFFu, wmax = 0u;  // score order: this thread's winners' key range
  const int kk = block_topk_collect<NT>(
      skey, n, k, sm.sel, pos_group, [&](int slot, uint32_t key, uint32_t pos) {
        if (OUT == kOutPart) {
          part[slot] = u32x2{key, pos};
        } else if (pos_order) {
          orow[slot] = (int32_t)pos;
        } else {
          sortbuf[slot] = (((uint64_t)key) << 32) | (uint64_t)(~pos);
          wmin = min(wmin, key);
          wmax = max(wmax, key);
        }
      },
      /*range_ready=*/true);
  if (OUT == kOutPart) {
    if (tid == 0) a.part_count[row * nchunks + chunk] = kk;
    return;
  }
  if (pos_order) {  // winners are emitted in position order: no sort
    for (int j = kk + tid; j < k; j += NT) orow[j] = -1;
    return;
  }

  // ---- score order. Wide workgroups (the final stage of long rows) rank by
  // buckets when the scores are spread out, with every wave busy (the staged
  // keys are no longer read, so their LDS is the scratch); otherwise, and in
  // 256-thread workgroups, where it measured faster, a bitonic sort,
  // descending, of the kk winners padded to a power of two.
  if (NT > kThreads && kk >= 512 && stage_bytes >= kBucketScratchBytes) {
    sel_store_key_range<NT>(wmin, wmax, sm.sel);
    __syncthreads();
    uint32_t wlo = sm.sel.kred[0], whi = sm.sel.kred[NT / kWave];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) {
      wlo = min(wlo, sm.sel.kred[w]);
      whi = max(whi, sm.sel.kred[NT / kWave + w]);
    }
    if (bucket_rank_output<NT>(sortbuf, kk, k, wlo, whi, skey, sm.sel, orow)) return;
  }
  int P = 1;
  while (P < kk) P <<= 1;
  static_assert(kMaxK == 8 * kThreads && NT % kThreads == 0, "register sort layout");
  if (P >= 512) {
    // the register sort of all 2048 slots, the ones past kk zero (every
    // winner's word is nonzero, so they sort last)
    const bool act = NT == kThreads || tid < kThreads;
    __syncthreads();
    uint64_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid * 8 + j;
      v[j] = (act && idx < kk) ? sortbuf[idx] : 0ull;
    }
    sort2048_regs(v, sortbuf, tid, act);
    if (act) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = tid * 8 + j;
        if (idx < k) orow[idx] = (idx < kk) ? (int32_t)(~(uint32_t)(v[j] & 0xFFFFFFFFull)) : -1;
      }
    }
    return;
  }
  for (int e = kk + tid; e < P; e += NT) sortbuf[e] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P >> 1); i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = sortbuf[lo], y = sortbuf[hi];
        const bool desc = (lo & size) == 0;
        if ((x < y) == desc) {
          sortbuf[lo] = y;
          sortbuf[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  for (int j = tid; j < k; j += NT) {
    orow[j] = (j < kk) ? (int32_t)(~(uint32_t)(sortbuf[j] & 0xFFFFFFFFull)) : -1;
  }
}

// stage_bytes: the staged input, after the scratch or, for score-order
// output, after the sort buffer laid over the histogram
template <int SRC, int OUT, int NT = kThreads>
hipError_t launch_one(const TopkArgs& a, int chunk_len, int nchunks, size_t stage_bytes,
                      hipStream_t st) {
  static_assert(sort_off<NT>() % 16 == 0, "aligned sort buffer");
  const bool need_sort = OUT == kOutFinal && !a.pos_order;
  size_t stage_off = smem_bytes<NT>();
  if (need_sort && sort_off<NT>() + kSortBytes > stage_off) stage_off = sort_off<NT>() + kSortBytes;
  const size_t shmem = stage_off + (stage_bytes + 15) / 16 * 16;
  auto fn = topk_kernel<SRC, OUT, NT>;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)(a.rows * nchunks)), dim3(NT), shmem, st, a,
                     chunk_len, nchunks, (int)stage_off, (int)stage_bytes);
  return hipGetLastError();
}

}  // namespace

int topk_row_chunks(int Lk) { return (Lk + kTopkChunk - 1) / kTopkChunk; }

size_t topk_part_bytes(int rows, int Lk, int k) {
  const int nch = topk_row_chunks(Lk);
  if (nch <= 1) return 0;
  return (size_t)rows * nch * k * 8 + (size_t)rows * nch * 4 + 256;
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

hipError_t launch_topk(const TopkArgs& a0, hipStream_t st) {
  TopkArgs a = a0;
  if (a.cand) {
    // candidate lists (one or more position-ordered segments per row); keys,
    // then positions when there are several segments, each area a multiple
    // of 16 bytes
    if (a.nseg == 1) {
      a.stage_cap = (a.stage_cap + 3) / 4 * 4;
      return launch_one<kSrcCand1, kOutFinal>(a, 0, 1, (size_t)a.stage_cap * 4, st);
    }
    const int groups = topk_segment_groups(a.nseg, a.k);
    if (groups <= 1) {
      a.stage_cap = (a.stage_cap + 3) / 4 * 4;
      return launch_one<kSrcCand, kOutFinal, kThreadsWide>(a, 0, 1, (size_t)a.stage_cap * 8,
                                                           st);
    }
    // too many segments for one workgroup: the exact top-k of each group of
    // consecutive segments (into a.part), then of the groups' winners (every
    // key of the row's top-k is in its group's top-k)
    TopkArgs g = a;
    const int per_group = (a.nseg + groups - 1) / groups;
    g.stage_cap = (per_group * a.k + 3) / 4 * 4;
    hipError_t e = launch_one<kSrcCand, kOutPart, kThreadsWide>(g, 0, groups,
                                                                (size_t)g.stage_cap * 8, st);
    if (e != hipSuccess) return e;
    TopkArgs f = a;
    f.cand = a.part;
    f.cand_count = a.part_count;
    f.nseg = groups;
    f.seg_cap = a.k;
    f.stage_cap = (groups * a.k + 3) / 4 * 4;
    return launch_one<kSrcCand, kOutFinal, kThreadsWide>(f, 0, 1, (size_t)f.stage_cap * 8, st);
  }
  const int nch = topk_row_chunks(a.Lk);
  if (nch <= 1) {
    return launch_one<kSrcRow, kOutFinal>(a, kTopkChunk, 1, (size_t)kTopkChunk * 4, st);
  }
  // long rows: exact top-k per chunk, then top-k of the chunks' winners
  hipError_t e = launch_one<kSrcRow, kOutPart>(a, kTopkChunk, nch, (size_t)kTopkChunk * 4, st);
  if (e != hipSuccess) return e;
  TopkArgs b = a;
  b.cand = a.part;
  b.cand_count = a.part_count;
  b.nseg = nch;
  b.seg_cap = a.k;
  b.stage_cap = (nch * a.k + 3) / 4 * 4;
  return launch_one<kSrcCand, kOutFinal, kThreadsWide>(b, 0, 1, (size_t)b.stage_cap * 8, st);
}

}  // namespace idxc
