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

namespace idxc {

namespace {

constexpr int kRowWaves = 8;          // queries per workgroup (one per wave)
constexpr int kKeyTile = 64;          // keys per LDS tile (two 32-key N-blocks)

// Wave-level synchronisation point for LDS/global data written by other lanes
// of the same wave (waits for outstanding memory operations).
__device__ __forceinline__ void wave_mem_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Candidate buffer compaction (one wave, one query).
//
// buf[0..n) holds (score bits, position) pairs in increasing position order.
// Keeps exactly the k best under (score desc, position asc), stably, and
// returns the order key of the k-th best in *tkey: every later key position
// is larger than all buffered ones, so it can only enter the top-k with a
// strictly larger order key. Radix select over the 32-bit order keys, 8 bits
// per pass, with a 256-bin histogram in this wave's LDS slice.
// ---------------------------------------------------------------------------
__device__ void wave_compact(u32x2* __restrict__ buf, int& n, int k, uint32_t& tkey,
                             uint32_t* hist) {
  const int lane = lane_id();
  wave_mem_sync();
  uint32_t prefix = 0, pmask = 0;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += kWave) hist[b] = 0u;
    wave_mem_sync();
    for (int e = lane; e < n; e += kWave) {
      uint32_t key = order_key(__uint_as_float(buf[e].x));
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    wave_mem_sync();
    // lane owns bins 255-4l .. 252-4l (descending)
    const int b0 = 255 - 4 * lane;
    const int c0 = (int)hist[b0], c1 = (int)hist[b0 - 1], c2 = (int)hist[b0 - 2],
              c3 = (int)hist[b0 - 3];
    const int local = c0 + c1 + c2 + c3;
    const int incl = wave_incl_scan(local);
    const int excl = incl - local;
    const uint64_t hit = ballot(incl >= rem);
    const int src = __builtin_ctzll(hit);
    int bin = 0, above = 0;
    if (lane == src) {
      int acc = excl;
      if (acc + c0 >= rem) { bin = b0; above = acc; }
      else if (acc + c0 + c1 >= rem) { bin = b0 - 1; above = acc + c0; }
      else if (acc + c0 + c1 + c2 >= rem) { bin = b0 - 2; above = acc + c0 + c1; }
      else { bin = b0 - 3; above = acc + c0 + c1 + c2; }
    }
    bin = __shfl(bin, src, kWave);
    above = __shfl(above, src, kWave);
    prefix |= ((uint32_t)bin) << shift;
    pmask |= 255u << shift;
    rem -= above;
    wave_mem_sync();
  }
  // prefix = order key of the k-th best; keep all larger keys and the first
  // `rem` entries equal to it (lowest positions: the buffer is position-sorted).
  int out = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kWave) {
    const int e = base + lane;
    u32x2 v = {0u, 0u};
    uint32_t key = 0u;
    if (e < n) {
      v = buf[e];
      key = order_key(__uint_as_float(v.x));
    }
    const bool gt = (e < n) && key > prefix;
    const bool eq = (e < n) && key == prefix;
    const uint64_t me = ballot(eq);
    const int eqr = eq_seen + lanes_below(me);
    const bool keep = gt || (eq && eqr < rem);
    const uint64_t mk = ballot(keep);
    wave_mem_sync();  // all lanes have read this window before any write
    if (keep) buf[out + lanes_below(mk)] = v;
    out += popc64(mk);
    eq_seen += popc64(me);
  }
  wave_mem_sync();
  n = out;
  tkey = prefix;
}

// ---------------------------------------------------------------------------
// Row-stationary kernel: a workgroup owns 8 consecutive query rows (one per
// wave) and streams all their causal keys through LDS in 64-key tiles.
//   MODE 0: write scores[b, i, 0..Lk) (score for s <= t, -inf beyond).
//   MODE 1: append (score, s) with order key above the query's threshold to
//           cand[row*cap ..], compacting to the k best when full; the final
//           count goes to cand_count[row].
// ---------------------------------------------------------------------------
template <int DI, int HB, int MODE>
__global__ __launch_bounds__(kRowWaves * kWave, 1)
void indexer_rows_kernel(const uint16_t* __restrict__ q_idx,
                         const uint16_t* __restrict__ k_idx,
                         const uint16_t* __restrict__ w, int B, int Lq, int Lk,
                         int q_pos0, int H_I, float* __restrict__ scores,
                         u32x2* __restrict__ cand, int* __restrict__ cand_count,
                         int cap, int k) {
  constexpr int NCH = DI / 8;            // 16-byte chunks per key row
  constexpr int KS = DI / 16;            // MFMA k-steps over d_I
  constexpr int TILE_CHUNKS = kKeyTile * NCH;
  constexpr int ROW_BYTES = DI * 2;
  constexpr int THREADS = kRowWaves * kWave;
  constexpr int CPT = (TILE_CHUNKS + THREADS - 1) / THREADS;  // chunks per thread

  __shared__ __attribute__((aligned(16))) uint8_t tile_lds[2][kKeyTile * ROW_BYTES];
  __shared__ uint32_t hist_lds[MODE == 1 ? kRowWaves * 256 : 1];

  const int nqb = (Lq + kRowWaves - 1) / kRowWaves;
  // longest rows first: block 0 takes the last query block of every batch
  const int b = blockIdx.x % B;
  const int qb = nqb - 1 - blockIdx.x / B;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i_row = qb * kRowWaves + wave;
  const bool active = i_row < Lq;
  const int t = q_pos0 + i_row;
  const int last_row = min(qb * kRowWaves + kRowWaves - 1, Lq - 1);
  const int t_last = q_pos0 + last_row;
  const int ntiles = t_last / kKeyTile + 1;
  const size_t row = (size_t)b * Lq + (active ? i_row : 0);

  // --- query operands (A: heads x d) and head weights, held in registers
  bf16x8 a_op[HB][KS];
  float wv[HB][16];
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
      wv[hb][i] = (active && hh < H_I) ? bf16_to_f32(w[row * H_I + hh]) : 0.0f;
    }
  }

  const uint16_t* kbase = k_idx + (size_t)b * Lk * DI;

  // --- cooperative tile load: global -> registers -> swizzled LDS
  u32x4 pref[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = threadIdx.x + c * THREADS;
      const int r = chunk / NCH;
      const int s = j * kKeyTile + r;
      if (chunk < TILE_CHUNKS && s < Lk) {
        pref[c] = *reinterpret_cast<const u32x4*>(kbase + (size_t)s * DI + (chunk % NCH) * 8);
      } else {
        pref[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = threadIdx.x + c * THREADS;
      if (chunk < TILE_CHUNKS) {
        const int r = chunk / NCH;
        const int cc = chunk % NCH;
        *reinterpret_cast<u32x4*>(&tile_lds[buf][r * ROW_BYTES + ((cc ^ (r % NCH)) * 16)]) =
            pref[c];
      }
    }
  };

  // --- candidate state (MODE 1)
  int n_cand = 0;
  uint32_t tkey = 0u;
  u32x2* my_cand = (MODE == 1) ? cand + row * (size_t)cap : nullptr;
  uint32_t* my_hist = (MODE == 1) ? hist_lds + wave * 256 : nullptr;
  float* my_scores = (MODE == 0) ? scores + row * (size_t)Lk : nullptr;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);
    const int tile_s0 = j * kKeyTile;
    if (active && tile_s0 <= t) {
      const uint8_t* tl = tile_lds[j & 1];
      float sc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int r = nb * 32 + (lane & 31);
        bf16x8 b_op[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = ks * 2 + (lane >> 5);
          b_op[ks] = *reinterpret_cast<const bf16x8*>(&tl[r * ROW_BYTES + ((c ^ (r % NCH)) * 16)]);
        }
        float part = 0.0f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma32(a_op[hb][ks], b_op[ks], acc);
#pragma unroll
          for (int i = 0; i < 16; ++i) part = fmaf(wv[hb][i], fmaxf(acc[i], 0.0f), part);
        }
        part = pair_sum(part);
        sc[nb] = part;
      }
      // lane l now scores key tile_s0 + l
      const float val = ((lane < 32) ? sc[0] : sc[1]) + 0.0f;
      const int s = tile_s0 + lane;
      if (MODE == 0) {
        if (s < Lk) my_scores[s] = (s <= t) ? val : -INFINITY;
      } else {
        bool pass = (s <= t) && order_key(val) > tkey;
        uint64_t m = ballot(pass);
        int cnt = popc64(m);
        if (cnt > 0) {
          if (n_cand + cnt > cap) {
            wave_compact(my_cand, n_cand, k, tkey, my_hist);
            pass = (s <= t) && order_key(val) > tkey;
            m = ballot(pass);
            cnt = popc64(m);
          }
          if (pass) {
            my_cand[n_cand + lanes_below(m)] = u32x2{__float_as_uint(val), (uint32_t)s};
          }
          n_cand += cnt;
        }
      }
    } else if (MODE == 0 && active) {
      // a tile wholly above this row's position (the block straddles a tile)
      const int s = tile_s0 + lane;
      if (s < Lk) my_scores[s] = -INFINITY;
    }
    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
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
    float part = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma32(a_op[hb][ks], cur[ks], acc);
#pragma unroll
      for (int i = 0; i < 16; ++i) part = fmaf(wv[hb][i], fmaxf(acc[i], 0.0f), part);
    }
    part = pair_sum(part);
    const int s = s0 + lane;
    if (lane < 32 && s < s_end) srow[s] = (s <= t) ? part + 0.0f : -INFINITY;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cur[ks] = nxt[ks];
  }
}

template <int DI, int HB>
hipError_t launch_rows(const IndexerArgs& a, int mode, hipStream_t st) {
  const int nqb = (a.Lq + kRowWaves - 1) / kRowWaves;
  dim3 grid((unsigned)(nqb * a.B)), block(kRowWaves * kWave);
  if (mode == 0) {
    hipLaunchKernelGGL((indexer_rows_kernel<DI, HB, 0>), grid, block, 0, st, a.q_idx, a.k_idx,
                       a.w, a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, a.scores, nullptr, nullptr, 0,
                       a.k);
  } else {
    hipLaunchKernelGGL((indexer_rows_kernel<DI, HB, 1>), grid, block, 0, st, a.q_idx, a.k_idx,
                       a.w, a.B, a.Lq, a.Lk, a.q_pos0, a.H_I, nullptr, a.cand, a.cand_count,
                       a.cap, a.k);
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

template <int DI>
hipError_t dispatch_hb(const IndexerArgs& a, int kind, hipStream_t st) {
  const int hb = (a.H_I + 31) / 32;
  if (hb == 1) return kind == 2 ? launch_split<DI, 1>(a, st) : launch_rows<DI, 1>(a, kind, st);
  return kind == 2 ? launch_split<DI, 2>(a, st) : launch_rows<DI, 2>(a, kind, st);
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

}  // namespace idxc
