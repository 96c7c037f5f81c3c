// Lightning-indexer score kernels for gfx950 (bf16 MFMA, fp32 epilogue).
//
// Score of query position t against key position s <= t:
//     score[t, s] = sum_h w[t, h] * max(0, q_I[t, h, :] . k_I[s, :])
// ("NLP——IndexCache" notes, section "背景 & 问题提出": a lightweight indexer
// scores every query against all earlier tokens and keeps the top-k; the
// per-head ReLU, per-query head weight and head sum are this library's reading
// of the indexer, which the pages name without writing out.)
//
// The contraction over d_I runs on 32x32x16 bf16 MFMAs with the indexer heads
// on the M dimension and keys on N, so one lane ends up holding 16 heads of one
// key: ReLU, the head weight and most of the head sum stay in registers, and a
// single lane-half swap finishes the sum. The L x L score matrix is either
// written out (materialising mode, for tests and small problems) or filtered on
// chip against a running per-query threshold (candidate mode, see below).
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace idxc {

namespace {

constexpr int kRowWaves = 8;          // queries per workgroup (one per wave)
constexpr int kKeyTile = 128;         // keys per LDS tile (four 32-key N-blocks)

// Wave-level synchronisation point for LDS/global data written by other lanes
// of the same wave (waits for outstanding memory operations).
__device__ __forceinline__ void wave_mem_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Candidate buffer compaction (one wave, one query).
//
// buf[0..n) holds (order key, position) pairs in increasing position order.
// Keeps exactly the k best under (key desc, position asc), stably, and
// returns the order key of the k-th best in *tkey: every later key position
// is larger than all buffered ones, so it can only enter the top-k with a
// strictly larger order key. Radix select over the key bits below the
// highest bit in which the keys differ, 11 bits per pass, with a 2048-bin
// histogram in `hist` (this wave's 8 KB of LDS). Global loads are batched.
// ---------------------------------------------------------------------------
constexpr int kCompactBins = 2048;

__device__ void wave_compact(u32x2* __restrict__ buf, int& n, int k, uint32_t& tkey,
                             uint32_t* hist) {
  constexpr int kBatch = 8;  // loads in flight per lane
  const int lane = lane_id();
  wave_mem_sync();
  // bits shared by every key
  const uint32_t first = buf[0].x;
  uint32_t diff = 0u;
  for (int base = 0; base < n; base += kWave * kBatch) {
    uint32_t keys[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = base + j * kWave + lane;
      keys[j] = e < n ? buf[e].x : first;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) diff |= keys[j] ^ first;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) diff |= __shfl_xor(diff, off, kWave);

  uint32_t prefix = first, pmask = 0xFFFFFFFFu;
  int rem = k;
  if (diff != 0u) {
    const int top = 31 - __builtin_clz(diff);  // highest differing bit
    pmask = (top == 31) ? 0u : (0xFFFFFFFFu << (top + 1));
    prefix = first & pmask;
    int shift = top + 1;
    while (shift > 0) {
      const int nbits = min(11, shift);
      shift -= nbits;
      const int nbins = 1 << nbits;
      const uint32_t dmask = (uint32_t)nbins - 1u;
      for (int b = lane; b < nbins; b += kWave) hist[b] = 0u;
      wave_mem_sync();
      for (int base = 0; base < n; base += kWave * kBatch) {
        uint32_t keys[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * kWave + lane;
          keys[j] = e < n ? buf[e].x : 0u;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int e = base + j * kWave + lane;
          if (e < n && (keys[j] & pmask) == prefix)
            atomicAdd(&hist[(keys[j] >> shift) & dmask], 1u);
        }
      }
      wave_mem_sync();
      // lane owns bins [hi - bpl + 1, hi], hi = nbins - 1 - lane * bpl (descending)
      const int bpl = nbins >= kWave ? nbins / kWave : 1;
      const int hi = nbins - 1 - lane * bpl;
      int local = 0;
      if (hi >= 0)
        for (int q = 0; q < bpl; ++q) local += (int)hist[hi - q];
      const int incl = wave_incl_scan(local);
      const int excl = incl - local;
      const int src = __builtin_ctzll(ballot(incl >= rem));
      int bin = 0, above = 0;
      if (lane == src) {
        int acc = excl;
        for (int q = 0; q < bpl; ++q) {
          const int c = (int)hist[hi - q];
          if (acc + c >= rem) {
            bin = hi - q;
            above = acc;
            break;
          }
          acc += c;
        }
      }
      bin = __shfl(bin, src, kWave);
      above = __shfl(above, src, kWave);
      prefix |= ((uint32_t)bin) << shift;
      pmask |= dmask << shift;
      rem -= above;
      wave_mem_sync();
    }
  }
  // prefix = order key of the k-th best; keep all larger keys and the first
  // `rem` entries equal to it (lowest positions: the buffer is position-sorted).
  // Windows are read a batch ahead of the in-place writes, which never pass
  // the read position.
  int out = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kWave * kBatch) {
    u32x2 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = base + j * kWave + lane;
      v[j] = e < n ? buf[e] : u32x2{0u, 0u};
    }
    wave_mem_sync();
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = base + j * kWave + lane;
      const bool gt = (e < n) && v[j].x > prefix;
      const bool eq = (e < n) && v[j].x == prefix;
      const uint64_t me = ballot(eq);
      const int eqr = eq_seen + lanes_below(me);
      const bool keep = gt || (eq && eqr < rem);
      const uint64_t mk = ballot(keep);
      if (keep) buf[out + lanes_below(mk)] = v[j];
      out += popc64(mk);
      eq_seen += popc64(me);
    }
  }
  wave_mem_sync();
  n = out;
  tkey = prefix;
}

// ---------------------------------------------------------------------------
// Row-stationary kernel: a workgroup owns 8 consecutive query rows (one per
// wave) and streams all their causal keys through LDS in 128-key tiles, one
// tile ahead.
//   MODE 0: write scores[b, i, 0..Lk) (score for s <= t, -inf beyond).
//   MODE 1: append (order key, s) for keys at or above the row's threshold to
//           cand[row*cap ..] (position order); the final count goes to
//           cand_count[row].
//
// MODE 1 threshold. Rows longer than the candidate capacity first score a
// stratified sample of their keys: up to 16 tiles of 128 consecutive keys
// spread evenly over [0, t_first] (t_first = the workgroup's least position), run
// through the same pipeline before the key sweep; the tile count grows with
// the row length so that about kSampleHits sampled keys land above the
// threshold. A row's threshold is the m-th largest sampled order key, m
// chosen so that about slack * k keys of the row are expected at or
// above it. The threshold is only a filter:
//  * if the buffer still overflows, it is compacted to the exact k best seen
//    so far (wave_compact) and the threshold rises to the k-th of them;
//  * if a row ends with fewer than k candidates and never compacted, keys of
//    its top-k may have been filtered out, so the workgroup sweeps the keys
//    again for that row without a threshold.
// Otherwise the buffer holds every key at or above the threshold, at least k
// of them, hence the whole top-k; the selection kernel picks the exact k.
// ---------------------------------------------------------------------------
constexpr int kSampleTiles = 16;  // at most
constexpr int kSampleKeys = kSampleTiles * kKeyTile;
// a wave's sample area doubles as the histogram of its compactions
static_assert(kSampleKeys >= kCompactBins, "compaction histogram fits the sample area");
// The survivor count of a threshold set at about kSampleHits sampled hits has
// a relative spread of about 1/sqrt(kSampleHits) = 10%: a row falls short of k
// (and its workgroup sweeps again) beyond (1 - 1/slack) / 0.1 standard
// deviations. A sweep again delays a launch by up to one workgroup's time, so
// launches of many workgroups take slack 1.5 (3.3 sigma, cheaper selection)
// and smaller ones 1.75 (4.3 sigma); the host passes it in.
constexpr float kSampleSlackMany = 1.5f;
constexpr float kSampleSlackFew = 1.75f;
constexpr int kSlackManyRows = 16384;  // query rows per launch for the smaller slack
// Rows so long that the sample reaches kSampleTiles first get fewer sampled
// hits (about 48 at 196K keys with this slack: 3.9 sigma).
constexpr float kSampleSlackCapped = 2.25f;
// expected sampled keys at or above the threshold; the threshold's rank in the
// row then has a relative spread of about 1/sqrt(kSampleHits)
constexpr float kSampleHits = 100.0f;

template <int DI, int HB, int MODE>
__global__ __launch_bounds__(kRowWaves * kWave, 1)
void indexer_rows_kernel(const uint16_t* __restrict__ q_idx,
                         const uint16_t* __restrict__ k_idx,
                         const uint16_t* __restrict__ w, int B, int Lq, int Lk,
                         int q_pos0, int H_I, float* __restrict__ scores,
                         u32x2* __restrict__ cand, int* __restrict__ cand_count,
                         int cap, int k, const int32_t* __restrict__ q_pos,
                         float slack_rows) {
  constexpr int NCH = DI / 8;            // 16-byte chunks per key row
  constexpr int KS = DI / 16;            // MFMA k-steps over d_I
  constexpr int TILE_CHUNKS = kKeyTile * NCH;
  constexpr int ROW_BYTES = DI * 2;
  constexpr int THREADS = kRowWaves * kWave;
  constexpr int CPT = (TILE_CHUNKS + THREADS - 1) / THREADS;  // chunks per thread

  __shared__ __attribute__((aligned(16))) uint8_t tile_lds[2][kKeyTile * ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t samp_lds[MODE == 1 ? kRowWaves * kSampleKeys : 4];
  __shared__ int rescan_lds;
  __shared__ int trange_lds[2];

  const int nqb = (Lq + kRowWaves - 1) / kRowWaves;
  // longest rows first: block 0 takes the last query block of every batch
  const int b = blockIdx.x % B;
  const int qb = nqb - 1 - blockIdx.x / B;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i_row = qb * kRowWaves + wave;
  const bool active = i_row < Lq;
  const size_t row = (size_t)b * Lq + (active ? i_row : 0);
  // Query positions: q_pos0 + i, or per row from q_pos (ragged batches;
  // negative = no candidates, past the keys = the last key). t_first / t_last
  // are the least / greatest position of the workgroup's rows that have
  // candidates.
  int t = q_pos0 + i_row;
  int t_first = q_pos0 + qb * kRowWaves;
  int t_last = q_pos0 + min(qb * kRowWaves + kRowWaves - 1, Lq - 1);
  if (q_pos != nullptr) {
    t = active ? q_pos[row] : -1;
    t = t < 0 ? -1 : min(t, Lk - 1);
    if (threadIdx.x == 0) {
      trange_lds[0] = 0x7FFFFFFF;
      trange_lds[1] = -1;
    }
    __syncthreads();
    if (lane == 0 && t >= 0) {
      atomicMin(&trange_lds[0], t);
      atomicMax(&trange_lds[1], t);
    }
    __syncthreads();
    t_last = trange_lds[1];
    t_first = t_last < 0 ? -1 : trange_lds[0];
  }
  const int ntiles = t_last < 0 ? 0 : t_last / kKeyTile + 1;

  // --- query operands (A: heads x d) and head weights, held in registers
  bf16x8 a_op[HB][KS];
  // head weights as bf16 pairs (even head in the low half): bf16 -> fp32 is
  // a shift or a mask, and the pairs halve the registers held
  uint32_t wp[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      if (active && h < H_I) {
        a_op[hb][ks] = *reinterpret_cast<const bf16x8*>(
            q_idx + (row * H_I + h) * DI + c * 8);
      } else {
        a_op[hb][ks] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = hb * 32 + acc_row(i, lane);
      const uint32_t wb = (active && hh < H_I) ? (uint32_t)w[row * H_I + hh] : 0u;
      if (i & 1) wp[hb][i >> 1] |= wb << 16;
      else wp[hb][i >> 1] = wb;
    }
  }

  const uint16_t* kbase = k_idx + (size_t)b * Lk * DI;

  // --- cooperative tile load, global -> LDS directly (16 bytes per lane),
  // one tile ahead of the tile being scored. LDS chunk position p of key row
  // r holds the row's 16-byte chunk p ^ (r % NCH) (XOR swizzle: the MFMA
  // operand reads of 16 rows at one chunk hit 16 different bank groups); a
  // lane picks the chunk that belongs at its position. Keys past Lk load row
  // Lk - 1: they are never kept (every kept key is <= t < Lk).
  static_assert(TILE_CHUNKS % THREADS == 0, "tile chunks must fill the workgroup");
  auto load_tile = [&](int s_begin, int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = threadIdx.x + c * THREADS;
      const int r = chunk / NCH;
      const int p = chunk % NCH;
      const int s = min(s_begin + r, Lk - 1);
      const uint16_t* src = kbase + (size_t)s * DI + (p ^ (r % NCH)) * 8;
      uint8_t* dst = &tile_lds[buf][(wave * kWave + c * THREADS) * 16];  // wave-uniform
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16,
                                       0, 0);
    }
  };
  // the tile's loads have landed in LDS for every wave
  auto tile_ready = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Scores of this wave's row against the keys of LDS tile `buf`: vals[h]
  // gets key h*64 + lane for h = 0 and, if `both`, h = 1. The tile's 32-key
  // blocks are software-pipelined: the MFMAs of block j+1 are issued before
  // the ReLU / head-weight reduction of block j, so this wave's vector work
  // overlaps its own matrix work (the waves of a workgroup run in step
  // between the per-tile barriers and cannot cover each other).
  auto tile_vals = [&](int buf, bool both, float (&vals)[2], auto after_reads) {
    const uint8_t* tl = tile_lds[buf];
    f32x16 acc[2][HB];
    float sc[4];
    auto issue = [&](int j) {
      const int r = j * 32 + (lane & 31);
      bf16x8 b_op[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 2 + (lane >> 5);
        b_op[ks] = *reinterpret_cast<const bf16x8*>(&tl[r * ROW_BYTES + ((c ^ (r % NCH)) * 16)]);
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[j & 1][hb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[j & 1][hb] = mfma32(a_op[hb][ks], b_op[ks], acc[j & 1][hb]);
      }
    };
    auto reduce = [&](int j) {
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const uint32_t pw = wp[hb][i >> 1];
          part0 = fmaf(__uint_as_float(pw << 16), relu_bits(acc[j & 1][hb][i]), part0);
          part1 = fmaf(__uint_as_float(pw & 0xFFFF0000u), relu_bits(acc[j & 1][hb][i + 1]),
                       part1);
        }
      }
      sc[j] = pair_sum(part0 + part1);
    };
    issue(0);
    issue(1);
    reduce(0);
    if (both) {
      issue(2);
      reduce(1);
      issue(3);
      after_reads();  // the tile's last operand reads are issued
      reduce(2);
      reduce(3);
      vals[1] = ((lane < 32) ? sc[2] : sc[3]) + 0.0f;
    } else {
      after_reads();
      reduce(1);
    }
    vals[0] = ((lane < 32) ? sc[0] : sc[1]) + 0.0f;
  };

  // --- candidate state (MODE 1)
  int n_cand = 0;
  uint32_t tkey = 0u;  // keep keys > tkey
  bool compacted = false;
  u32x2* my_cand = (MODE == 1) ? cand + row * (size_t)cap : nullptr;
  uint32_t* my_samp = (MODE == 1) ? samp_lds + wave * kSampleKeys : nullptr;
  float* my_scores = (MODE == 0) ? scores + row * (size_t)Lk : nullptr;

  // pass 0: sample tiles (if any) then the causal key sweep; pass 1 (rare):
  // the sweep again, without threshold, for rows whose sampled threshold
  // turned out too high
  bool compute_row = active && t >= 0;
  for (int pass = 0; pass < (MODE == 1 ? 2 : 1); ++pass) {
    int nsamp = 0;
    float slack = slack_rows;
    if (MODE == 1 && pass == 0 && t_first + 1 > cap) {
      const float tiles = kSampleHits * (float)(t_first + 1) / (slack_rows * (float)k * kKeyTile);
      if (tiles > (float)kSampleTiles) slack = kSampleSlackCapped;
      nsamp = max(2, min(kSampleTiles, (int)ceilf(tiles)));
    }
    const int nv = nsamp + ntiles;
    const int span = t_first + 1 - kKeyTile;
    auto tile_start = [&](int v) {
      return v < nsamp ? (int)(((long long)v * span) / (nsamp - 1)) : (v - nsamp) * kKeyTile;
    };

    load_tile(tile_start(0), 0);
    tile_ready();

    for (int v = 0; v < nv; ++v) {
      // Tile v is in LDS buffer v&1; tile v+1 streams into the other buffer
      // (last read in tile v-1, before the barrier that ended it). Its loads
      // are issued after this wave's last operand read of tile v: the
      // compiler cannot tell the two buffers apart and waits for every
      // outstanding global-to-LDS load before an LDS read, so loads issued
      // before the reads would be waited for before the tile is scored.
      bool next_issued = false;
      auto next_tile = [&]() {
        if (v + 1 < nv) load_tile(tile_start(v + 1), (v + 1) & 1);
        next_issued = true;
      };
      if (MODE == 1 && v == nsamp && nsamp > 0 && compute_row) {
        // threshold = m-th largest sampled order key (binary search on bits)
        const int nkeys = nsamp * kKeyTile;
        const float want = slack * (float)k * (float)nkeys / (float)(t + 1);
        const int m = max(1, min(nkeys, (int)ceilf(want)));
        uint32_t T = 0u;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t candT = T | (1u << bit);
          int c = 0;
          for (int e = lane * 4; e < nkeys; e += kWave * 4) {
            const u32x4 kv = *reinterpret_cast<const u32x4*>(my_samp + e);
            c += (kv[0] >= candT) + (kv[1] >= candT) + (kv[2] >= candT) + (kv[3] >= candT);
          }
          if (wave_sum(c) >= m) T = candT;
        }
        tkey = T - 1u;  // keep keys >= T (finite scores have keys > 0)
      }
      const int tile_s0 = tile_start(v);
      if (v < nsamp) {
        // sampled keys are all <= t_first <= t
        if (compute_row) {
          float vals[2];
          tile_vals(v & 1, true, vals, next_tile);
#pragma unroll
          for (int half = 0; half < 2; ++half)
            my_samp[v * kKeyTile + half * 64 + lane] = order_key(vals[half]);
        }
      } else if (compute_row && tile_s0 <= t) {
        // the second half is skipped when it lies wholly above this row
        const bool both = tile_s0 + 64 <= t;
        float vals[2];
        tile_vals(v & 1, both, vals, next_tile);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int s = tile_s0 + half * 64 + lane;
          if (half == 1 && !both) {
            if (MODE == 0 && s < Lk) my_scores[s] = -INFINITY;
            continue;
          }
          const float val = vals[half];
          if (MODE == 0) {
            if (s < Lk) my_scores[s] = (s <= t) ? val : -INFINITY;
          } else {
            const uint32_t key = order_key(val);
            bool pass_key = (s <= t) && key > tkey;
            uint64_t m = ballot(pass_key);
            int cnt = popc64(m);
            if (cnt > 0) {
              if (n_cand + cnt > cap) {
                wave_compact(my_cand, n_cand, k, tkey, my_samp);
                compacted = true;
                pass_key = (s <= t) && key > tkey;
                m = ballot(pass_key);
                cnt = popc64(m);
              }
              if (pass_key) my_cand[n_cand + lanes_below(m)] = u32x2{key, (uint32_t)s};
              n_cand += cnt;
            }
          }
        }
      } else if (MODE == 0 && active) {
        // a tile wholly above this row's position (the block straddles a tile)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int s = tile_s0 + half * 64 + lane;
          if (s < Lk) my_scores[s] = -INFINITY;
        }
      }
      if (!next_issued) next_tile();  // this wave scored no key of tile v
      tile_ready();
    }

    if (MODE == 0 || nsamp == 0) break;
    // rows whose filtered buffer may miss part of the top-k sweep again
    const bool redo = compute_row && !compacted && n_cand < k;
    if (threadIdx.x == 0) rescan_lds = 0;
    __syncthreads();
    if (redo && lane == 0) atomicOr(&rescan_lds, 1);
    __syncthreads();
    if (rescan_lds == 0) break;
    compute_row = redo;
    if (redo) {
      n_cand = 0;
      tkey = 0u;
    }
  }

  if (!active) return;
  if (MODE == 0) {
    for (int s = ntiles * kKeyTile + lane; s < Lk; s += kWave) my_scores[s] = -INFINITY;
  } else {
    if (lane == 0) cand_count[row] = n_cand;
  }
}

// ---------------------------------------------------------------------------
// Split-key kernel for few query rows (decode): a workgroup owns one query row
// and a 2048-key chunk; each wave streams 512 keys straight from global memory
// into MFMA B operands (no reuse across waves, so no LDS staging), writing the
// materialised scores.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 4;
constexpr int kSplitKeysPerWave = 512;
constexpr int kSplitChunk = kSplitWaves * kSplitKeysPerWave;

template <int DI, int HB>
__global__ __launch_bounds__(kSplitWaves * kWave, 2)
void indexer_split_kernel(const uint16_t* __restrict__ q_idx,
                          const uint16_t* __restrict__ k_idx,
                          const uint16_t* __restrict__ w, int B, int Lq, int Lk,
                          int q_pos0, int H_I, float* __restrict__ scores) {
  constexpr int KS = DI / 16;
  const int nchunks = (Lk + kSplitChunk - 1) / kSplitChunk;
  const int chunk = blockIdx.x % nchunks;
  const size_t row = blockIdx.x / nchunks;  // b * Lq + i
  const int b = (int)(row / Lq);
  const int i_row = (int)(row % Lq);
  const int t = q_pos0 + i_row;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();

  bf16x8 a_op[HB][KS];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      a_op[hb][ks] = (h < H_I) ? *reinterpret_cast<const bf16x8*>(
                                     q_idx + (row * H_I + h) * DI + c * 8)
                               : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = hb * 32 + acc_row(i, lane);
      wv[hb][i] = (hh < H_I) ? bf16_to_f32(w[row * H_I + hh]) : 0.0f;
    }
  }

  const uint16_t* kbase = k_idx + (size_t)b * Lk * DI;
  float* srow = scores + row * (size_t)Lk;
  const int s_begin = chunk * kSplitChunk + wave * kSplitKeysPerWave;
  const int s_end = min(s_begin + kSplitKeysPerWave, Lk);
  if (s_begin >= Lk) return;

  auto load_b = [&](int s0, bf16x8* dst) {
    const int s = s0 + (lane & 31);
    const bool ok = s < Lk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      dst[ks] = ok ? *reinterpret_cast<const bf16x8*>(kbase + (size_t)s * DI + c * 8) : bf16x8{};
    }
  };

  bf16x8 cur[KS], nxt[KS];
  load_b(s_begin, cur);
  for (int s0 = s_begin; s0 < s_end; s0 += 32) {
    if (s0 + 32 < s_end) load_b(s0 + 32, nxt);
    float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(a_op[hb][ks], cur[ks], acc);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        part0 = fmaf(wv[hb][i], relu_bits(acc[i]), part0);
        part1 = fmaf(wv[hb][i + 1], relu_bits(acc[i + 1]), part1);
      }
    }
    const float part = pair_sum(part0 + part1);
    const int s = s0 + lane;
    if (lane < 32 && s < s_end) srow[s] = (s <= t) ? part + 0.0f : -INFINITY;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cur[ks] = nxt[ks];
  }
}

// ---------------------------------------------------------------------------
// Split-key kernel with chunk-local top-k (few query rows, e.g. decode): a
// workgroup of 8 waves owns one query row and a 16384-key chunk (every eighth
// 32-key block per wave, three blocks in flight per wave), keeps the chunk's order
// keys in LDS and writes the chunk's exact top-k, in position order, as one
// candidate segment; a selection launch over the row's segments finishes the
// row. Every key of the row's top-k is in its chunk's top-k. (16384-key
// chunks halve the segments the final selection stages, against 8192.)
// ---------------------------------------------------------------------------
constexpr int kDecChunk = 16384;
static_assert(kDecChunk <= kSelMaxKeys, "selection histogram counts fit 16 bits");
constexpr int kDecWaves = 8;

template <int DI, int HB>
__global__ __launch_bounds__(kDecWaves * kWave, 2)
void indexer_split_topk_kernel(const uint16_t* __restrict__ q_idx,
                               const uint16_t* __restrict__ k_idx,
                               const uint16_t* __restrict__ w, int B, int Lq, int Lk,
                               int q_pos0, int H_I, int k, int nchunks,
                               u32x2* __restrict__ part, int* __restrict__ part_count,
                               const int32_t* __restrict__ q_pos) {
  constexpr int KS = DI / 16;
  constexpr int NCH = DI / 8;         // 16-byte chunks per key row
  constexpr int RPI = kWave / NCH;    // key rows per load instruction
  constexpr int ROW_BYTES = DI * 2;
  static_assert(32 / RPI == KS, "one load instruction per MFMA k-step");
  __shared__ __attribute__((aligned(16))) uint32_t skey[kDecChunk];
  __shared__ SelectSmemT<kDecWaves * kWave> sel;
  // per wave: one 32-key block of k_I rows, XOR-swizzled like the row
  // kernel's tiles (position p of row r holds chunk p ^ (r % NCH))
  __shared__ __attribute__((aligned(16))) uint8_t blk_lds[kDecWaves][32 * ROW_BYTES];
  const int chunk = blockIdx.x % nchunks;
  const size_t row = blockIdx.x / nchunks;  // b * Lq + i
  const int b = (int)(row / Lq);
  const int i_row = (int)(row % Lq);
  // per-row positions (ragged batches): negative = no candidates, past the
  // keys = the last key
  const int t = q_pos ? (q_pos[row] < 0 ? -1 : min(q_pos[row], Lk - 1)) : q_pos0 + i_row;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int c0 = chunk * kDecChunk;
  const int n = max(0, min(t + 1, c0 + kDecChunk) - c0);  // causal keys of this chunk

  bf16x8 a_op[HB][KS];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      a_op[hb][ks] = (h < H_I) ? *reinterpret_cast<const bf16x8*>(
                                     q_idx + (row * H_I + h) * DI + c * 8)
                               : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = hb * 32 + acc_row(i, lane);
      wv[hb][i] = (hh < H_I) ? bf16_to_f32(w[row * H_I + hh]) : 0.0f;
    }
  }

  const uint16_t* kbase = k_idx + (size_t)b * Lk * DI;
  // The waves take the chunk's 32-key blocks in turn (block j of wave w is
  // block j * kDecWaves + w), so that a workgroup streams one contiguous
  // range at a time rather than eight.
  const int nblk = (n + 31) / 32;
  const int nb = nblk > wave ? (nblk - wave + kDecWaves - 1) / kDecWaves : 0;
  auto blk_key = [&](int j) { return (j * kDecWaves + wave) * 32; };  // chunk-local

  // A block's k_I rows are read in row layout (NCH lanes cover one row, so
  // each load instruction covers whole 128-byte lines) with non-temporal
  // loads (the stream has no reuse), then pass through the wave's LDS block
  // into the MFMA operand layout. (Loads straight into the operand layout
  // read each line in four instructions: the line must then stay cached,
  // and marked non-temporal it is fetched again.)
  // Loads are issued unconditionally, at the last key for rows past the
  // keys (blocks past the wave's range included): their scores are never
  // stored, and loads under a branch would make the compiler wait for every
  // outstanding load at the top of the loop instead of for the oldest block.
  auto load_b = [&](int j, bf16x8* dst) {
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int s = min(c0 + blk_key(j) + q * RPI + lane / NCH, Lk - 1);
      dst[q] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(kbase + (size_t)s * DI + (lane % NCH) * 8));
    }
  };
  uint8_t* my_blk = blk_lds[wave];
  auto to_operand = [&](bf16x8* b) {
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int r = q * RPI + lane / NCH, c = lane % NCH;
      *reinterpret_cast<bf16x8*>(my_blk + r * ROW_BYTES + ((c ^ (r % NCH)) * 16)) = b[q];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = lane & 31, c = ks * 2 + (lane >> 5);
      b[ks] = *reinterpret_cast<const bf16x8*>(my_blk + r * ROW_BYTES + ((c ^ (r % NCH)) * 16));
    }
  };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;  // range of the keys this lane stores
  auto score_block = [&](int j, bf16x8* bop) {
    to_operand(bop);
    float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(a_op[hb][ks], bop[ks], acc);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        part0 = fmaf(wv[hb][i], relu_bits(acc[i]), part0);
        part1 = fmaf(wv[hb][i + 1], relu_bits(acc[i + 1]), part1);
      }
    }
    const float val = pair_sum(part0 + part1) + 0.0f;
    const int e = blk_key(j) + lane;
    if (lane < 32 && e < n) {
      const uint32_t key = order_key(val);
      skey[e] = key;
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  };

  if (nb > 0) {  // wave-uniform; inside, every block's loads and MFMAs run
    bf16x8 b0[KS], b1[KS], b2[KS];
    load_b(0, b0);
    load_b(1, b1);
    load_b(2, b2);
    for (int j = 0; j < nb; j += 3) {
      score_block(j, b0);
      load_b(j + 3, b0);
      score_block(j + 1, b1);
      load_b(j + 4, b1);
      score_block(j + 2, b2);
      load_b(j + 5, b2);
    }
  }
  sel_store_key_range<kDecWaves * kWave>(kmin, kmax, sel);
  __syncthreads();

  u32x2* seg = part + row * (size_t)nchunks * k + (size_t)chunk * k;
  const int kk = block_topk_collect<kDecWaves * kWave>(
      skey, n, k, sel,
      [&](int e0, unsigned, uint32_t (&pv)[kSelPerThread]) {
#pragma unroll
        for (int j = 0; j < kSelPerThread; ++j) pv[j] = (uint32_t)(c0 + e0 + j);
      },
      [&](int slot, uint32_t key, uint32_t pos) { seg[slot] = u32x2{key, pos}; },
      /*range_ready=*/true);
  if (threadIdx.x == 0) part_count[row * nchunks + chunk] = kk;
}

template <int DI, int HB>
hipError_t launch_split_topk(const IndexerArgs& a, hipStream_t st) {
  const int nchunks = (a.Lk + kDecChunk - 1) / kDecChunk;
  dim3 grid((unsigned)(nchunks * a.B * a.Lq)), block(kDecWaves * kWave);
  hipLaunchKernelGGL((indexer_split_topk_kernel<DI, HB>), grid, block, 0, st, a.q_idx, a.k_idx,
                     a.w, a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, a.k, nchunks, a.cand, a.cand_count,
                     a.q_pos);
  return hipGetLastError();
}

template <int DI, int HB>
hipError_t launch_rows(const IndexerArgs& a, int mode, hipStream_t st) {
  const int nqb = (a.Lq + kRowWaves - 1) / kRowWaves;
  dim3 grid((unsigned)(nqb * a.B)), block(kRowWaves * kWave);
  if (mode == 0) {
    hipLaunchKernelGGL((indexer_rows_kernel<DI, HB, 0>), grid, block, 0, st, a.q_idx, a.k_idx,
                       a.w, a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, a.scores, nullptr, nullptr, 0,
                       a.k, nullptr, kSampleSlackMany);
  } else {
    hipLaunchKernelGGL((indexer_rows_kernel<DI, HB, 1>), grid, block, 0, st, a.q_idx, a.k_idx,
                       a.w, a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, nullptr, a.cand, a.cand_count,
                       a.cap, a.k, a.q_pos,
                       a.B * a.Lq >= kSlackManyRows ? kSampleSlackMany : kSampleSlackFew);
  }
  return hipGetLastError();
}

template <int DI, int HB>
hipError_t launch_split(const IndexerArgs& a, hipStream_t st) {
  const int nchunks = (a.Lk + kSplitChunk - 1) / kSplitChunk;
  dim3 grid((unsigned)(nchunks * a.B * a.Lq)), block(kSplitWaves * kWave);
  hipLaunchKernelGGL((indexer_split_kernel<DI, HB>), grid, block, 0, st, a.q_idx, a.k_idx, a.w,
                     a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, a.scores);
  return hipGetLastError();
}

// kind: 0 materialised rows, 1 candidate rows, 2 materialised split, 3 split
// with chunk-local top-k
template <int DI>
hipError_t dispatch_hb(const IndexerArgs& a, int kind, hipStream_t st) {
  const int hb = (a.H_I + 31) / 32;
  if (hb == 1) {
    if (kind == 2) return launch_split<DI, 1>(a, st);
    if (kind == 3) return launch_split_topk<DI, 1>(a, st);
    return launch_rows<DI, 1>(a, kind, st);
  }
  if (kind == 2) return launch_split<DI, 2>(a, st);
  if (kind == 3) return launch_split_topk<DI, 2>(a, st);
  return launch_rows<DI, 2>(a, kind, st);
}

hipError_t dispatch(const IndexerArgs& a, int kind, hipStream_t st) {
  switch (a.d_I) {
    case 32: return dispatch_hb<32>(a, kind, st);
    case 64: return dispatch_hb<64>(a, kind, st);
    default: return dispatch_hb<128>(a, kind, st);
  }
}

}  // namespace

bool indexer_prefers_split(int B, int Lq, int Lk) {
  // Few query rows against a long key range: the row-stationary kernel would
  // run too few workgroups, so split the keys instead.
  const long long rows = (long long)B * Lq;
  const long long row_blocks = (long long)B * ((Lq + kRowWaves - 1) / kRowWaves);
  return row_blocks < 256 && (long long)Lk >= 4LL * kSplitChunk && rows <= 4096;
}

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t st) {
  return dispatch(a, indexer_prefers_split(a.B, a.Lq, a.Lk) ? 2 : 0, st);
}

hipError_t launch_indexer_candidates(const IndexerArgs& a, hipStream_t st) {
  return dispatch(a, 1, st);
}

int indexer_split_chunks(int Lk) { return (Lk + kDecChunk - 1) / kDecChunk; }

hipError_t launch_indexer_split_topk(const IndexerArgs& a, hipStream_t st) {
  return dispatch(a, 3, st);
}

}  // namespace idxc
