// Host-side launchers of the gfx950 kernels (internal to libidxc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idxc {

struct IndexerArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const uint16_t* w;
  int B, Lq, Lk, q_pos0, H_I, d_I, k;
  float* scores;                       // materialising mode
  uint32_t __attribute__((ext_vector_type(2)))* cand;  // candidate mode
  int* cand_count;
  int cap;
};

// Materialised scores [B, Lq, Lk].
hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t st);
// Candidate mode: per row, a superset of its top-k in cand[row*cap ..] with
// the count in cand_count[row].
hipError_t launch_indexer_candidates(const IndexerArgs& a, hipStream_t st);
bool indexer_prefers_split(int B, int Lq, int Lk);

struct TopkArgs {
  // source A: materialised scores rows (row r = b*Lq + i, candidates 0..t)
  const float* scores;
  int Lq, Lk, q_pos0;
  // source B: candidate lists (cand != nullptr)
  const uint32_t __attribute__((ext_vector_type(2)))* cand;
  const int* cand_count;
  int cap;
  int rows, k;
  int32_t* out;  // [rows, k]
};

hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* key;
  const uint16_t* val;
  const int32_t* indices;
  int B, Lq, Lk, H, D, topk;
  float scale;
  uint16_t* out;
};

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);

}  // namespace idxc
