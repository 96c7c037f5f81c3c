// C ABI of libidxc: argument checks, workspace sizing and the F/S layer loop.
//
// Every check runs on the host before any launch: a call that returns an
// error has launched nothing and has not touched device memory or initialised
// a HIP device.
//
// The F/S scheduler follows the state machine of "IndexCache：跨层复用稀疏注意力
// 的索引" (wineandchord.com), section "从 DSA 的成本分解开始" (an F layer
// recomputes the top-k and overwrites the single cached index tensor, an S
// layer reuses it, the first layer must be F, roles outside {F, S} are errors)
// and the loop of the "NLP——IndexCache" notes, section "IndexCache 方法"
// (compute and cache on F, read the cache on S; f(l) = max{j < l : c_j = F}).
#include <stdarg.h>
#include <mutex>
#include <stdio.h>
#include <string.h>

#include "../../include/idxc.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace idxc;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return IDXC_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(IDXC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The attention kernels take the softmax maximum over unscaled scores and
// scale it afterwards, and mask padding with -inf before scaling: both need
// a finite scale > 0.
bool scale_ok(float scale) { return scale > 0.0f && scale <= 3.4028234663852886e38f; }

#define REQUIRE_PTR(p, name)                                                          \
  do {                                                                                \
    if ((p) == nullptr) return fail(IDXC_ERR_INVALID_ARG, "%s is NULL", name);         \
    if (!aligned16(p)) return fail(IDXC_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

constexpr int kMaxRows = 1 << 24;
constexpr int kMaxLk = 1 << 24;

// Common size checks. need: bit 0 = indexer fields, bit 1 = attention fields,
// bit 2 = k.
constexpr int kMaxOverlapLk = 262144;  // two LDS bitmaps of Lk bits (64 KB)
constexpr int kMaxMatrixLayers = 64;   // n*n 64-bit LDS accumulators (32 KB)
constexpr int kMaxTeachers = 64;       // layers one indexer serves

int check_dims(const idxc_dims* d, int need) {
  if (d == nullptr) return fail(IDXC_ERR_INVALID_ARG, "dims is NULL");
  if (d->B < 1 || d->Lq < 1 || d->Lk < 1)
    return fail(IDXC_ERR_INVALID_ARG, "B, Lq and Lk must be >= 1 (got %d, %d, %d)", d->B, d->Lq,
                d->Lk);
  if (d->q_pos0 < 0) return fail(IDXC_ERR_INVALID_ARG, "q_pos0 must be >= 0");
  if ((long long)d->q_pos0 + d->Lq > d->Lk)
    return fail(IDXC_ERR_INVALID_ARG, "q_pos0 + Lq (%lld) exceeds Lk (%d)",
                (long long)d->q_pos0 + d->Lq, d->Lk);
  if ((long long)d->B * d->Lq > kMaxRows || d->Lk > kMaxLk)
    return fail(IDXC_ERR_UNSUPPORTED, "B*Lq or Lk too large");
  if (need & 1) {
    if (d->H_I < 1 || d->d_I < 1) return fail(IDXC_ERR_INVALID_ARG, "H_I and d_I must be >= 1");
    if (d->H_I > 64) return fail(IDXC_ERR_UNSUPPORTED, "H_I = %d > 64", d->H_I);
    if (d->d_I != 32 && d->d_I != 64 && d->d_I != 128)
      return fail(IDXC_ERR_UNSUPPORTED, "d_I = %d not in {32, 64, 128}", d->d_I);
  }
  if (need & 2) {
    if (d->H < 1 || d->D < 1) return fail(IDXC_ERR_INVALID_ARG, "H and D must be >= 1");
    if (d->H > 64) return fail(IDXC_ERR_UNSUPPORTED, "H = %d > 64", d->H);
    if (d->D != 64 && d->D != 128) return fail(IDXC_ERR_UNSUPPORTED, "D = %d not in {64, 128}", d->D);
  }
  if (need & 4) {
    if (d->k < 1) return fail(IDXC_ERR_INVALID_ARG, "k must be >= 1");
    if (d->k > kMaxK) return fail(IDXC_ERR_UNSUPPORTED, "k = %d > %d", d->k, kMaxK);
  }
  return IDXC_OK;
}

int check_pattern(const char* pattern, int32_t n_layers, int32_t* n_full) {
  if (pattern == nullptr) return fail(IDXC_ERR_INVALID_ARG, "pattern is NULL");
  if (n_layers < 1) return fail(IDXC_ERR_INVALID_ARG, "n_layers must be >= 1");
  const size_t len = strnlen(pattern, (size_t)n_layers + 1);
  if (len != (size_t)n_layers)
    return fail(IDXC_ERR_PATTERN, "pattern length %zu != n_layers %d", len, n_layers);
  int nf = 0;
  for (int l = 0; l < n_layers; ++l) {
    const char c = pattern[l];
    if (c == 'F') ++nf;
    else if (c != 'S') return fail(IDXC_ERR_PATTERN, "unknown role '%c' at layer %d (only F and S)", c, l);
  }
  if (pattern[0] != 'F') return fail(IDXC_ERR_PATTERN, "layer 0 has no earlier F layer to share from: it must be F");
  if (n_full) *n_full = nf;
  return IDXC_OK;
}

// ---- workspace plan -------------------------------------------------------
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Smallest candidate capacity: after a compaction a row holds k entries and
// must still take one more 64-key tile.
int min_cap(int k) { return (k + 64 + 63) / 64 * 64; }

// Default candidate capacity: room for the 1.5k-1.75k keys a sampled
// threshold lets through (2.25k on rows long enough to use the larger slack,
// which only key ranges beyond 60000 have), with a margin of several standard
// deviations; also the number of candidates the selection kernel stages per
// row.
int default_cap(int k, int Lk) {
  int cap = Lk > 60000 ? 7 * k / 2 : 5 * k / 2;
  if (cap < k + 64) cap = k + 64;
  if (cap < 1024) cap = 1024;
  if (cap > kMaxStagePairs) cap = kMaxStagePairs;
  return (cap + 63) / 64 * 64;
}

struct Plan {
  bool split;      // per-chunk indexer top-k, then selection (few rows)
  size_t bytes;    // workspace needed at full speed
  size_t min_bytes;
};

// The few-row path writes per-chunk top-k segments; one workgroup per row
// selects from them, after a per-group stage when there are too many to
// stage at once.
bool split_topk_fits(const idxc_dims* d) {
  const int nch = indexer_split_chunks(d->Lk);
  return nch <= kMaxSegments && topk_segment_groups(nch, d->k) >= 1;
}

size_t split_part_bytes(const idxc_dims* d) {
  const size_t rows = (size_t)d->B * d->Lq;
  const size_t nch = (size_t)indexer_split_chunks(d->Lk);
  return align_up(rows * nch * d->k * 8) + align_up(rows * nch * 4) +
         align_up(topk_group_bytes((int)rows, (int)nch, d->k));
}

Plan plan_for(const idxc_dims* d, bool with_attn = false) {
  Plan p;
  const size_t rows = (size_t)d->B * d->Lq;
  p.split = indexer_prefers_split(d->B, d->Lq, d->Lk) && split_topk_fits(d);
  if (p.split) {
    p.bytes = split_part_bytes(d);
    p.min_bytes = p.bytes;
  } else {
    p.bytes = align_up(rows * 4) + rows * (size_t)default_cap(d->k, d->Lk) * 8;
    p.min_bytes = align_up(rows * 4) + rows * (size_t)min_cap(d->k) * 8;
  }
  if (with_attn) {
    // the layer loop reuses the same workspace for attention partials
    const size_t att = attn_workspace_bytes(d->B, d->Lq, d->H, d->D, d->k);
    if (att > p.bytes) p.bytes = att;
    if (att > p.min_bytes) p.min_bytes = att;
  }
  return p;
}

// Largest candidate capacity (multiple of 64, <= default) that fits.
int cap_for(const idxc_dims* d, size_t ws_bytes) {
  const size_t rows = (size_t)d->B * d->Lq;
  const size_t head = align_up(rows * 4);
  if (ws_bytes < head) return 0;
  size_t cap = (ws_bytes - head) / (rows * 8);
  cap = cap / 64 * 64;
  const size_t dc = (size_t)default_cap(d->k, d->Lk);
  if (cap > dc) cap = dc;
  return (int)cap;
}

// Scratch of the top-k of long materialised rows (chunk histograms), at `base`.
void set_parts(TopkArgs& ta, uint8_t* base, const idxc_dims* d) {
  if (topk_row_chunks(d->Lk) > 1) ta.ghist = base;
}

// Indexer + top-k for one layer into `indices`, using the workspace.
hipError_t run_indexer_topk(const void* q_idx, const void* k_idx, const void* w,
                            const idxc_dims* d, void* ws, size_t ws_bytes, int32_t* indices,
                            bool pos_order, const int32_t* q_pos, hipStream_t st) {
  IndexerArgs ia{};
  ia.q_pos = q_pos;
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.k_idx = static_cast<const uint16_t*>(k_idx);
  ia.w = static_cast<const uint16_t*>(w);
  ia.B = d->B;
  ia.Lq = d->Lq;
  ia.Lk = d->Lk;
  ia.q_pos0 = d->q_pos0;
  ia.H_I = d->H_I;
  ia.d_I = d->d_I;
  ia.k = d->k;
  const int rows = d->B * d->Lq;
  TopkArgs ta{};
  ta.Lq = d->Lq;
  ta.Lk = d->Lk;
  ta.q_pos0 = d->q_pos0;
  ta.rows = rows;
  ta.k = d->k;
  ta.out = indices;
  ta.pos_order = pos_order ? 1 : 0;
  if (plan_for(d).split) {
    const int nch = indexer_split_chunks(d->Lk);
    uint8_t* base = static_cast<uint8_t*>(ws);
    ia.cand = reinterpret_cast<decltype(ia.cand)>(base);
    ia.cand_count = reinterpret_cast<int*>(base + align_up((size_t)rows * nch * d->k * 8));
    hipError_t e = launch_indexer_split_topk(ia, st);
    if (e != hipSuccess) return e;
    ta.cand = ia.cand;
    ta.cand_count = ia.cand_count;
    const int groups = topk_segment_groups(nch, d->k);
    if (groups > 1) {  // scratch of the per-group stage, after the segments
      uint8_t* gb = base + align_up((size_t)rows * nch * d->k * 8) + align_up((size_t)rows * nch * 4);
      ta.part = reinterpret_cast<u32x2_t*>(gb);
      ta.part_count = reinterpret_cast<int*>(gb + (size_t)rows * groups * d->k * 8);
    }
    ta.nseg = nch;
    ta.seg_cap = d->k;
    ta.stage_cap = nch * d->k;
    return launch_topk(ta, st);
  }
  const int cap = cap_for(d, ws_bytes);
  ia.cand_count = static_cast<int*>(ws);
  ia.cand = reinterpret_cast<decltype(ia.cand)>(static_cast<uint8_t*>(ws) + align_up((size_t)rows * 4));
  ia.cap = cap;
  hipError_t e = launch_indexer_candidates(ia, st);
  if (e != hipSuccess) return e;
  ta.cand = ia.cand;
  ta.cand_count = ia.cand_count;
  ta.nseg = 1;
  ta.seg_cap = cap;
  ta.stage_cap = cap;
  return launch_topk(ta, st);
}

// prefix: the lists are the stack's own top-k output (valid entries first,
// min(k, t + 1) of them; t from q_pos0 or q_pos).
AttnArgs attn_args(const void* q, const void* k, const void* v, const int32_t* indices,
                   const idxc_dims* d, float scale, void* out, void* workspace,
                   bool prefix = false, const int32_t* q_pos = nullptr) {
  AttnArgs a{};
  a.workspace = workspace;
  a.prefix_lists = prefix ? 1 : 0;
  a.q_pos0 = d->q_pos0;
  a.q_pos = q_pos;
  a.q = static_cast<const uint16_t*>(q);
  a.key = static_cast<const uint16_t*>(k);
  a.val = static_cast<const uint16_t*>(v);
  a.indices = indices;
  a.B = d->B;
  a.Lq = d->Lq;
  a.Lk = d->Lk;
  a.H = d->H;
  a.D = d->D;
  a.topk = d->k;
  a.scale = scale;
  a.out = static_cast<uint16_t*>(out);
  return a;
}

// ---- device-resident scratch of idxc_layer_stack_forward_noalloc ----------
// One copy per GPU, alive until the process ends. In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress (per device, with that device current) and is the only
// form ever handed to a kernel or a copy.
static_assert(IDXC_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[IDXC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up once per device).
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(IDXC_ERR_UNSUPPORTED, "device ordinal %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(IDXC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return IDXC_OK;
}

}  // namespace

extern "C" {

const char* idxc_last_error(void) { return g_err; }

const char* idxc_version(void) { return "idxc 0.1.0 gfx950"; }

int idxc_validate_pattern(const char* pattern, int32_t n_layers, int32_t* n_full) {
  const int r = check_pattern(pattern, n_layers, n_full);
  return r == IDXC_OK ? ok() : r;
}

int idxc_schedule(const char* pattern, int32_t n_layers, int32_t* source) {
  const int r = check_pattern(pattern, n_layers, nullptr);
  if (r != IDXC_OK) return r;
  if (source == nullptr) return fail(IDXC_ERR_INVALID_ARG, "source is NULL");
  int last_f = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (pattern[l] == 'F') last_f = l;
    source[l] = last_f;
  }
  return ok();
}

int idxc_workspace_bytes(const idxc_dims* dims, size_t* bytes) {
  int r = check_dims(dims, 1 | 4);
  if (r != IDXC_OK) return r;
  if (bytes == nullptr) return fail(IDXC_ERR_INVALID_ARG, "bytes is NULL");
  const bool with_attn = dims->H > 0 && dims->D > 0;
  if (with_attn) {
    r = check_dims(dims, 2);
    if (r != IDXC_OK) return r;
  }
  *bytes = plan_for(dims, with_attn).bytes;
  return ok();
}

int idxc_indexer_scores(const void* q_idx, const void* k_idx, const void* w,
                        const idxc_dims* dims, float* scores, void* hip_stream) {
  int r = check_dims(dims, 1);
  if (r != IDXC_OK) return r;
  REQUIRE_PTR(q_idx, "q_idx");
  REQUIRE_PTR(k_idx, "k_idx");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(scores, "scores");
  IndexerArgs ia{};
  ia.q_idx = static_cast<const uint16_t*>(q_idx);
  ia.k_idx = static_cast<const uint16_t*>(k_idx);
  ia.w = static_cast<const uint16_t*>(w);
  ia.B = dims->B;
  ia.Lq = dims->Lq;
  ia.Lk = dims->Lk;
  ia.q_pos0 = dims->q_pos0;
  ia.H_I = dims->H_I;
  ia.d_I = dims->d_I;
  ia.k = dims->k;
  ia.scores = scores;
  return hip_status(launch_indexer_scores(ia, static_cast<hipStream_t>(hip_stream)),
                    "indexer_scores launch");
}

int idxc_topk_workspace_bytes(const idxc_dims* dims, size_t* bytes) {
  int r = check_dims(dims, 4);
  if (r != IDXC_OK) return r;
  if (bytes == nullptr) return fail(IDXC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = topk_part_bytes(dims->B * dims->Lq, dims->Lk, dims->k);
  return ok();
}

int idxc_topk(const float* scores, const idxc_dims* dims, int32_t order, void* workspace,
              size_t workspace_bytes, int32_t* indices, void* hip_stream) {
  int r = check_dims(dims, 4);
  if (r != IDXC_OK) return r;
  if (order != IDXC_ORDER_SCORE && order != IDXC_ORDER_POSITION)
    return fail(IDXC_ERR_INVALID_ARG, "order = %d is not an IDXC_ORDER_* value", order);
  REQUIRE_PTR(scores, "scores");
  REQUIRE_PTR(indices, "indices");
  const size_t need = topk_part_bytes(dims->B * dims->Lq, dims->Lk, dims->k);
  if (need > 0) {
    REQUIRE_PTR(workspace, "workspace");
    if (workspace_bytes < need)
      return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the minimum %zu",
                  workspace_bytes, need);
  }
  TopkArgs ta{};
  ta.scores = scores;
  ta.Lq = dims->Lq;
  ta.Lk = dims->Lk;
  ta.q_pos0 = dims->q_pos0;
  ta.rows = dims->B * dims->Lq;
  ta.k = dims->k;
  ta.out = indices;
  ta.pos_order = order == IDXC_ORDER_POSITION ? 1 : 0;
  set_parts(ta, static_cast<uint8_t*>(workspace), dims);
  return hip_status(launch_topk(ta, static_cast<hipStream_t>(hip_stream)), "topk launch");
}

int idxc_indexer_topk(const void* q_idx, const void* k_idx, const void* w,
                      const idxc_dims* dims, int32_t order, void* workspace,
                      size_t workspace_bytes, int32_t* indices, void* hip_stream) {
  int r = check_dims(dims, 1 | 4);
  if (r != IDXC_OK) return r;
  if (order != IDXC_ORDER_SCORE && order != IDXC_ORDER_POSITION)
    return fail(IDXC_ERR_INVALID_ARG, "order = %d is not an IDXC_ORDER_* value", order);
  REQUIRE_PTR(q_idx, "q_idx");
  REQUIRE_PTR(k_idx, "k_idx");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(workspace, "workspace");
  REQUIRE_PTR(indices, "indices");
  const Plan p = plan_for(dims);
  if (workspace_bytes < p.min_bytes)
    return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, p.min_bytes);
  return hip_status(run_indexer_topk(q_idx, k_idx, w, dims, workspace, workspace_bytes, indices,
                                     order == IDXC_ORDER_POSITION, nullptr,
                                     static_cast<hipStream_t>(hip_stream)),
                    "indexer_topk launch");
}

int idxc_indexer_topk_ragged(const void* q_idx, const void* k_idx, const void* w,
                             const idxc_dims* dims, const int32_t* q_pos, int32_t order,
                             void* workspace, size_t workspace_bytes, int32_t* indices,
                             void* hip_stream) {
  REQUIRE_PTR(q_pos, "q_pos");
  int r = check_dims(dims, 1 | 4);
  if (r != IDXC_OK) return r;
  if (order != IDXC_ORDER_SCORE && order != IDXC_ORDER_POSITION)
    return fail(IDXC_ERR_INVALID_ARG, "order = %d is not an IDXC_ORDER_* value", order);
  REQUIRE_PTR(q_idx, "q_idx");
  REQUIRE_PTR(k_idx, "k_idx");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(workspace, "workspace");
  REQUIRE_PTR(indices, "indices");
  const Plan p = plan_for(dims);
  if (workspace_bytes < p.min_bytes)
    return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, p.min_bytes);
  return hip_status(run_indexer_topk(q_idx, k_idx, w, dims, workspace, workspace_bytes, indices,
                                     order == IDXC_ORDER_POSITION, q_pos,
                                     static_cast<hipStream_t>(hip_stream)),
                    "indexer_topk launch");
}

int idxc_sparse_attn_workspace_bytes(const idxc_dims* dims, size_t* bytes) {
  int r = check_dims(dims, 2 | 4);
  if (r != IDXC_OK) return r;
  if (bytes == nullptr) return fail(IDXC_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = attn_workspace_bytes(dims->B, dims->Lq, dims->H, dims->D, dims->k);
  return ok();
}

int idxc_sparse_attn(const void* q, const void* k, const void* v, const int32_t* indices,
                     const idxc_dims* dims, float scale, void* workspace, size_t workspace_bytes,
                     void* out, void* hip_stream) {
  int r = check_dims(dims, 2 | 4);
  if (r != IDXC_OK) return r;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(indices, "indices");
  REQUIRE_PTR(out, "out");
  if (!scale_ok(scale)) return fail(IDXC_ERR_INVALID_ARG, "scale = %g: must be finite and > 0", (double)scale);
  void* ws = nullptr;
  if (workspace != nullptr) {
    if (!aligned16(workspace)) return fail(IDXC_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const size_t need = attn_workspace_bytes(dims->B, dims->Lq, dims->H, dims->D, dims->k);
    if (need > 0) {
      if (workspace_bytes < need)
        return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the %zu needed",
                    workspace_bytes, need);
      ws = workspace;
    }
  }
  return hip_status(launch_sparse_attn(attn_args(q, k, v, indices, dims, scale, out, ws),
                                       static_cast<hipStream_t>(hip_stream)),
                    "sparse_attn launch");
}

int idxc_overlap(const int32_t* a, const int32_t* b, const idxc_dims* dims, int32_t* inter,
                 float* overlap, float* jaccard, void* hip_stream) {
  int r = check_dims(dims, 4);
  if (r != IDXC_OK) return r;
  auto aligned4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (a == nullptr || b == nullptr) return fail(IDXC_ERR_INVALID_ARG, "a and b must not be NULL");
  const void* ptrs[5] = {a, b, inter, overlap, jaccard};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned4(p)) return fail(IDXC_ERR_INVALID_ARG, "pointer not 4-byte aligned");
  if (overlap_lds_bytes(dims->Lk) > overlap_lds_bytes(kMaxOverlapLk))
    return fail(IDXC_ERR_UNSUPPORTED, "Lk = %d above %d for idxc_overlap", dims->Lk, kMaxOverlapLk);
  if (inter == nullptr && overlap == nullptr && jaccard == nullptr) return ok();
  return hip_status(launch_overlap(a, b, dims->B * dims->Lq, dims->k, dims->Lk, inter, overlap,
                                   jaccard, static_cast<hipStream_t>(hip_stream)),
                    "overlap launch");
}

size_t idxc_overlap_matrix_workspace_bytes(int32_t n_layers) {
  if (n_layers < 1 || n_layers > kMaxMatrixLayers) return 0;
  return align_up((size_t)n_layers * n_layers * 8);
}

int idxc_overlap_matrix(const int32_t* sel, int32_t n_layers, const idxc_dims* dims,
                        void* workspace, size_t workspace_bytes, float* matrix,
                        void* hip_stream) {
  int r = check_dims(dims, 4);
  if (r != IDXC_OK) return r;
  if (n_layers < 1) return fail(IDXC_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (n_layers > kMaxMatrixLayers)
    return fail(IDXC_ERR_UNSUPPORTED, "n_layers = %d above %d", n_layers, kMaxMatrixLayers);
  if (dims->Lk > kMaxOverlapLk)
    return fail(IDXC_ERR_UNSUPPORTED, "Lk = %d above %d for idxc_overlap_matrix", dims->Lk,
                kMaxOverlapLk);
  if (sel == nullptr || matrix == nullptr || workspace == nullptr)
    return fail(IDXC_ERR_INVALID_ARG, "sel, matrix and workspace must not be NULL");
  if ((reinterpret_cast<uintptr_t>(sel) & 3u) || (reinterpret_cast<uintptr_t>(matrix) & 3u))
    return fail(IDXC_ERR_INVALID_ARG, "sel and matrix must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u)
    return fail(IDXC_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const size_t need = idxc_overlap_matrix_workspace_bytes(n_layers);
  if (workspace_bytes < need)
    return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the %zu needed",
                workspace_bytes, need);
  return hip_status(launch_overlap_matrix(sel, n_layers, dims->B * dims->Lq, dims->k, dims->Lk,
                                          static_cast<unsigned long long*>(workspace), matrix,
                                          static_cast<hipStream_t>(hip_stream)),
                    "overlap matrix launch");
}

int idxc_distill_loss(const float* logits, const float* teachers, int32_t n_teachers,
                      const idxc_dims* dims, float* row_loss, float* grad, void* hip_stream) {
  int r = check_dims(dims, 0);
  if (r != IDXC_OK) return r;
  if (n_teachers < 1) return fail(IDXC_ERR_INVALID_ARG, "n_teachers must be >= 1");
  if (n_teachers > kMaxTeachers)
    return fail(IDXC_ERR_UNSUPPORTED, "n_teachers = %d above %d", n_teachers, kMaxTeachers);
  REQUIRE_PTR(logits, "logits");
  REQUIRE_PTR(teachers, "teachers");
  if (row_loss != nullptr && !aligned16(row_loss))
    return fail(IDXC_ERR_INVALID_ARG, "row_loss is not 16-byte aligned");
  if (grad != nullptr && !aligned16(grad))
    return fail(IDXC_ERR_INVALID_ARG, "grad is not 16-byte aligned");
  if (row_loss == nullptr && grad == nullptr) return ok();
  return hip_status(launch_distill(logits, teachers, n_teachers, dims->B, dims->Lq, dims->Lk,
                                   dims->q_pos0, row_loss, grad,
                                   static_cast<hipStream_t>(hip_stream)),
                    "distill launch");
}

int idxc_overlap_proxy_loss(const char* pattern, int32_t n_layers, const float* matrix,
                            double* loss) {
  const int r = check_pattern(pattern, n_layers, nullptr);
  if (r != IDXC_OK) return r;
  if (matrix == nullptr || loss == nullptr)
    return fail(IDXC_ERR_INVALID_ARG, "matrix and loss must not be NULL");
  double sum = 0.0;
  int last_f = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (pattern[l] == 'F') {
      last_f = l;
      continue;
    }
    sum += 1.0 - (double)matrix[(size_t)l * n_layers + last_f];
  }
  *loss = sum / (double)n_layers;
  return ok();
}

int idxc_greedy_pattern(int32_t n_layers, int32_t removals, idxc_loss_fn loss, void* user,
                        char* pattern, int64_t* evals) {
  if (n_layers < 1) return fail(IDXC_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (removals < 0 || removals > n_layers - 1)
    return fail(IDXC_ERR_INVALID_ARG, "removals = %d outside [0, %d]", removals, n_layers - 1);
  if (loss == nullptr || pattern == nullptr)
    return fail(IDXC_ERR_INVALID_ARG, "loss and pattern must not be NULL");
  // the working pattern lives in the caller's buffer (n_layers + 1 chars)
  memset(pattern, 'F', (size_t)n_layers);
  pattern[n_layers] = '\0';
  int64_t count = 0;
  for (int step = 0; step < removals; ++step) {
    int best = -1;
    double best_v = 0.0;
    for (int l = 1; l < n_layers; ++l) {
      if (pattern[l] != 'F') continue;
      pattern[l] = 'S';
      const double v = loss(pattern, user);
      pattern[l] = 'F';
      ++count;
      if (!(v == v)) {
        if (evals) *evals = count;
        return fail(IDXC_ERR_INVALID_ARG, "loss returned NaN for layer %d at step %d", l, step);
      }
      if (best < 0 || v < best_v) {  // ties keep the lower layer
        best = l;
        best_v = v;
      }
    }
    pattern[best] = 'S';
  }
  if (evals) *evals = count;
  return ok();
}

// Every argument check of the stack entry points except the workspace's.
static int stack_checks(const char* pattern, int32_t n_layers, const idxc_layer* layers,
                        const idxc_dims* dims, float scale, int32_t* index_cache,
                        int32_t* indexer_calls, int32_t* debug_indices) {
  int r = check_pattern(pattern, n_layers, nullptr);
  if (r != IDXC_OK) return r;
  r = check_dims(dims, 1 | 2 | 4);
  if (r != IDXC_OK) return r;
  if (layers == nullptr) return fail(IDXC_ERR_INVALID_ARG, "layers is NULL");
  if (indexer_calls == nullptr) return fail(IDXC_ERR_INVALID_ARG, "indexer_calls is NULL");
  REQUIRE_PTR(index_cache, "index_cache");
  if (debug_indices != nullptr && !aligned16(debug_indices))
    return fail(IDXC_ERR_INVALID_ARG, "debug_indices is not 16-byte aligned");
  if (!scale_ok(scale)) return fail(IDXC_ERR_INVALID_ARG, "scale = %g: must be finite and > 0", (double)scale);
  for (int l = 0; l < n_layers; ++l) {
    const idxc_layer& L = layers[l];
    char name[64];
    if (pattern[l] == 'F') {
      snprintf(name, sizeof(name), "layers[%d].q_idx", l);
      REQUIRE_PTR(L.q_idx, name);
      snprintf(name, sizeof(name), "layers[%d].k_idx", l);
      REQUIRE_PTR(L.k_idx, name);
      snprintf(name, sizeof(name), "layers[%d].w", l);
      REQUIRE_PTR(L.w, name);
    }
    snprintf(name, sizeof(name), "layers[%d].q", l);
    REQUIRE_PTR(L.q, name);
    snprintf(name, sizeof(name), "layers[%d].k", l);
    REQUIRE_PTR(L.k, name);
    snprintf(name, sizeof(name), "layers[%d].v", l);
    REQUIRE_PTR(L.v, name);
    snprintf(name, sizeof(name), "layers[%d].out", l);
    REQUIRE_PTR(L.out, name);
  }
  return IDXC_OK;
}

// The layer loop, after every check has passed.
static int stack_run(const char* pattern, int32_t n_layers, const idxc_layer* layers,
                     const idxc_dims* dims, const int32_t* q_pos, float scale,
                     int32_t* index_cache, void* workspace, size_t workspace_bytes,
                     int32_t* indexer_calls, int32_t* debug_indices, hipStream_t st) {
  const size_t cache_elems = (size_t)dims->B * dims->Lq * dims->k;
  int calls = 0;
  for (int l = 0; l < n_layers; ++l) {
    const idxc_layer& L = layers[l];
    if (pattern[l] == 'F') {
      // the cache keeps each row's top-k set in position order: attention
      // does not depend on the order, and its gathers then sweep the keys
      hipError_t e = run_indexer_topk(L.q_idx, L.k_idx, L.w, dims, workspace, workspace_bytes,
                                      index_cache, true, q_pos, st);
      if (e != hipSuccess) {
        *indexer_calls = calls;
        return hip_status(e, "stack indexer launch");
      }
      ++calls;
    }
    // the cache is the stack's own top-k output: its padding blocks are skipped
    hipError_t e = launch_sparse_attn(
        attn_args(L.q, L.k, L.v, index_cache, dims, scale, L.out, workspace, true, q_pos), st);
    if (e != hipSuccess) {
      *indexer_calls = calls;
      return hip_status(e, "stack attention launch");
    }
    if (debug_indices != nullptr) {
      e = hipMemcpyAsync(debug_indices + (size_t)l * cache_elems, index_cache,
                         cache_elems * sizeof(int32_t), hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) {
        *indexer_calls = calls;
        return hip_status(e, "debug index copy");
      }
    }
  }
  *indexer_calls = calls;
  return ok();
}

static int stack_forward(const char* pattern, int32_t n_layers, const idxc_layer* layers,
                         const idxc_dims* dims, const int32_t* q_pos, float scale,
                         int32_t* index_cache, void* workspace, size_t workspace_bytes,
                         int32_t* indexer_calls, int32_t* debug_indices, void* hip_stream) {
  int r = stack_checks(pattern, n_layers, layers, dims, scale, index_cache, indexer_calls,
                       debug_indices);
  if (r != IDXC_OK) return r;
  REQUIRE_PTR(workspace, "workspace");
  const Plan p = plan_for(dims, true);
  if (workspace_bytes < p.min_bytes)
    return fail(IDXC_ERR_INVALID_ARG, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, p.min_bytes);
  return stack_run(pattern, n_layers, layers, dims, q_pos, scale, index_cache, workspace,
                   workspace_bytes, indexer_calls, debug_indices,
                   static_cast<hipStream_t>(hip_stream));
}

int idxc_layer_stack_forward(const char* pattern, int32_t n_layers, const idxc_layer* layers,
                             const idxc_dims* dims, float scale, int32_t* index_cache,
                             void* workspace, size_t workspace_bytes, int32_t* indexer_calls,
                             int32_t* debug_indices, void* hip_stream) {
  return stack_forward(pattern, n_layers, layers, dims, nullptr, scale, index_cache, workspace,
                       workspace_bytes, indexer_calls, debug_indices, hip_stream);
}

int idxc_layer_stack_forward_noalloc(const char* pattern, int32_t n_layers,
                                     const idxc_layer* layers, const idxc_dims* dims,
                                     float scale, int32_t* index_cache, int32_t* indexer_calls,
                                     int32_t* debug_indices, void* hip_stream) {
  int r = stack_checks(pattern, n_layers, layers, dims, scale, index_cache, indexer_calls,
                       debug_indices);
  if (r != IDXC_OK) return r;
  const Plan p = plan_for(dims, true);
  if (p.min_bytes > (size_t)IDXC_NOALLOC_SCRATCH_BYTES)
    return fail(IDXC_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of scratch, above the static %zu bytes",
                p.min_bytes, (size_t)IDXC_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  r = current_scratch(&ws);
  if (r != IDXC_OK) return r;
  const size_t ws_bytes =
      p.bytes < (size_t)IDXC_NOALLOC_SCRATCH_BYTES ? p.bytes : (size_t)IDXC_NOALLOC_SCRATCH_BYTES;
  return stack_run(pattern, n_layers, layers, dims, nullptr, scale, index_cache, ws, ws_bytes,
                   indexer_calls, debug_indices, static_cast<hipStream_t>(hip_stream));
}

int idxc_layer_stack_forward_ragged(const char* pattern, int32_t n_layers,
                                    const idxc_layer* layers, const idxc_dims* dims,
                                    const int32_t* q_pos, float scale, int32_t* index_cache,
                                    void* workspace, size_t workspace_bytes,
                                    int32_t* indexer_calls, int32_t* debug_indices,
                                    void* hip_stream) {
  REQUIRE_PTR(q_pos, "q_pos");
  return stack_forward(pattern, n_layers, layers, dims, q_pos, scale, index_cache, workspace,
                       workspace_bytes, indexer_calls, debug_indices, hip_stream);
}

}  // extern "C"
