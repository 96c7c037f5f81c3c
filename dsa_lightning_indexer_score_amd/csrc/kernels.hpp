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
  uint32_t __attribute__((ext_vector_type(2)))* cand;  // candidate mode: (order key, s)
  int* cand_count;
  int cap;
  // per-row query positions [B*Lq] (device; NULL = q_pos0 + i); candidate
  // and few-row top-k modes only
  const int32_t* q_pos;
};

// Materialised scores [B, Lq, Lk].
hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t st);
// Candidate mode: per row, a superset of its top-k in cand[row*cap ..] with
// the count in cand_count[row].
hipError_t launch_indexer_candidates(const IndexerArgs& a, hipStream_t st);
bool indexer_prefers_split(int B, int Lq, int Lk);
// Few-row path: per (row, 8192-key chunk) exact top-k segments written to
// cand (segments of k entries, counts in cand_count[row * chunks + chunk]).
int indexer_split_chunks(int Lk);
hipError_t launch_indexer_split_topk(const IndexerArgs& a, hipStream_t st);

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTopkChunk = 8192;       // keys per workgroup for materialised rows
constexpr int kMaxSegments = 64;       // candidate segments per row
constexpr int kMaxStagePairs = 16384;  // candidate pairs one workgroup can stage

struct TopkArgs {
  // source A: materialised score rows (row r = b*Lq + i, candidates 0..t)
  const float* scores;
  int Lq, Lk, q_pos0;
  // source B: candidate lists of (order key, position), position-ordered:
  // nseg segments of seg_cap entries per row, counts in cand_count[row*nseg+s]
  const u32x2_t* cand;
  const int* cand_count;
  int nseg, seg_cap, stage_cap;
  // scratch of the per-group stage of many-segment candidate lists
  u32x2_t* part;
  int* part_count;
  // scratch of long materialised rows: per (row, chunk) top-digit histograms
  void* ghist;
  int rows, k;
  int32_t* out;  // [rows, k]
  // 0: score order (higher score, then lower position); 1: increasing
  // position order (the selected set is the same)
  int pos_order;
};

// Number of kTopkChunk-score chunks of materialised rows of length Lk (1 =
// one pass per row, no scratch).
int topk_row_chunks(int Lk);
// Scratch bytes launch_topk needs for materialised rows of length Lk (4 KB
// per chunk of every row).
size_t topk_part_bytes(int rows, int Lk, int k);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// Candidate rows of nseg segments of k: groups of segments selected first when
// one workgroup cannot stage them all (1 = single stage, 0 = unsupported),
// and the scratch (TopkArgs::part / part_count) that first stage writes.
int topk_segment_groups(int nseg, int k);
size_t topk_group_bytes(int rows, int nseg, int k);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* key;
  const uint16_t* val;
  const int32_t* indices;
  int B, Lq, Lk, H, D, topk;
  float scale;
  uint16_t* out;
  void* workspace;  // NULL: one pass per row; else partials of split rows
  // Nonzero when the lists are the library's own top-k output: row r's valid
  // entries are then its first min(k, t_r + 1), t_r = q_pos0 + (r % Lq) (or
  // q_pos[r], negative = none, past the keys = the last key), and the rest
  // are -1, so blocks past them hold only padding and are skipped (the
  // result is the same: padding adds exact zeros). 0: any list.
  int prefix_lists;
  int q_pos0;
  const int32_t* q_pos;
};

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);
// Index-list slices per row (1 = no split) and the workspace they need.
int attn_splits(int B, int Lq, int k);
size_t attn_part_o_bytes(int B, int Lq, int H, int D, int nsplit);
size_t attn_workspace_bytes(int B, int Lq, int H, int D, int k);

// Cross-layer agreement of two [rows, k] index tensors (per-row |A ∩ B|,
// overlap, Jaccard; any output may be null).
size_t overlap_lds_bytes(int Lk);
hipError_t launch_overlap(const int32_t* a, const int32_t* b, int rows, int k, int Lk,
                          int32_t* inter, float* overlap, float* jaccard, hipStream_t st);
// Multi-teacher distillation loss: per row (b, i), keys 0..q_pos0+i of
// logits [B,Lq,Lk] and of n_teachers distributions [n][B,Lq,Lk]; row_loss
// [B*Lq] and grad [B,Lq,Lk] (q - mean teacher, 0 past the row's keys) may be
// null.
hipError_t launch_distill(const float* logits, const float* teachers, int n_teachers, int B,
                          int Lq, int Lk, int q_pos0, float* row_loss, float* grad,
                          hipStream_t st);

// Overlap matrix of n index tensors sel[n][rows][k] (matrix[a*n+b] = mean over
// rows of overlap(sel[a], sel[b])); acc is a device workspace of n*n uint64.
size_t overlap_matrix_lds_bytes(int n, int Lk);
hipError_t launch_overlap_matrix(const int32_t* sel, int n, int rows, int k, int Lk,
                                 unsigned long long* acc, float* matrix, hipStream_t st);

}  // namespace idxc
