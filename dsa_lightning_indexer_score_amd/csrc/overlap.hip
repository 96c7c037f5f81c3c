// Cross-layer index-set agreement for gfx950.
//
// For two index tensors A, B [rows, k] (entries are positions in [0, Lk) or
// -1 padding, in any order), per row:
//   inter   = |A ∩ B|,
//   overlap = |A ∩ B| / |A|        (1 when A and B are both empty, 0 when
//                                   only A is),
//   jaccard = |A ∩ B| / |A ∪ B|    (1 when both are empty),
// over the valid entries taken as sets. These are the agreement measures of
// "IndexCache：跨层复用稀疏注意力的索引" (section on the cross-layer overlap of
// indexer top-k selections), and of the Jaccard similarity the "NLP——IndexCache"
// notes use for adjacent layers; with |A| = k the overlap equals the pages'
// |A ∩ B| / k.
//
// One workgroup per row. Each list is turned into a bitmap over [0, Lk) in
// LDS with atomic ORs (the returned old word tells whether a position is new,
// so duplicates count once), then the second list's new positions are tested
// against the first bitmap. The lists are read once, coalesced, with each
// thread's entries loaded before its bitmap updates: the kernel is bound by
// HBM reads of the two index tensors.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kOvThreads = 256;
constexpr int kOvBatch = 8;  // list entries per thread in flight

__global__ __launch_bounds__(kOvThreads)
void overlap_kernel(const int32_t* __restrict__ a, const int32_t* __restrict__ b, int k, int Lk,
                    int words, int32_t* __restrict__ inter_out, float* __restrict__ overlap_out,
                    float* __restrict__ jaccard_out) {
  extern __shared__ uint32_t bits[];  // [2][words]
  __shared__ int red[3][kOvThreads / kWave];
  uint32_t* bits_a = bits;
  uint32_t* bits_b = bits + words;
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const int32_t* ar = a + row * k;
  const int32_t* br = b + row * k;
  // Entries are loaded kOvBatch per thread at a time, all issued before the
  // bitmap updates use them; lists of up to kOvThreads * kOvBatch entries
  // (k <= 2048) also have B's entries loaded before A's bitmap is built.
  auto load_batch = [&](const int32_t* r, int base, int (&p)[kOvBatch]) {
#pragma unroll
    for (int u = 0; u < kOvBatch; ++u) {
      const int e = base + u * kOvThreads + tid;
      p[u] = e < k ? __builtin_nontemporal_load(r + e) : -1;
    }
  };
  const bool one_batch = k <= kOvThreads * kOvBatch;
  int pa[kOvBatch], pb[kOvBatch];
  load_batch(ar, 0, pa);
  if (one_batch) load_batch(br, 0, pb);
  // the bitmaps are cleared while the first loads are in flight
  for (int w = tid; w < 2 * words; w += kOvThreads) bits[w] = 0u;
  __syncthreads();
  int na = 0;
  for (int base = 0; base < k; base += kOvThreads * kOvBatch) {
    if (base > 0) load_batch(ar, base, pa);
#pragma unroll
    for (int u = 0; u < kOvBatch; ++u) {
      const int p = pa[u];
      if (p >= 0 && p < Lk) {
        const uint32_t m = 1u << (p & 31);
        na += (atomicOr(&bits_a[p >> 5], m) & m) ? 0 : 1;
      }
    }
  }
  __syncthreads();
  int nb = 0, ni = 0;
  for (int base = 0; base < k; base += kOvThreads * kOvBatch) {
    if (!one_batch) load_batch(br, base, pb);
#pragma unroll
    for (int u = 0; u < kOvBatch; ++u) {
      const int p = pb[u];
      if (p >= 0 && p < Lk) {
        const uint32_t m = 1u << (p & 31);
        if (!(atomicOr(&bits_b[p >> 5], m) & m)) {
          ++nb;
          ni += (bits_a[p >> 5] & m) ? 1 : 0;
        }
      }
    }
  }
  na = wave_sum(na);
  nb = wave_sum(nb);
  ni = wave_sum(ni);
  const int wave = tid / kWave;
  if (lane_id() == 0) {
    red[0][wave] = na;
    red[1][wave] = nb;
    red[2][wave] = ni;
  }
  __syncthreads();
  if (tid == 0) {
    int sa = 0, sb = 0, si = 0;
#pragma unroll
    for (int w = 0; w < kOvThreads / kWave; ++w) {
      sa += red[0][w];
      sb += red[1][w];
      si += red[2][w];
    }
    const int su = sa + sb - si;
    if (inter_out) inter_out[row] = si;
    if (overlap_out) overlap_out[row] = sa > 0 ? (float)si / (float)sa : (sb > 0 ? 0.0f : 1.0f);
    if (jaccard_out) jaccard_out[row] = su > 0 ? (float)si / (float)su : 1.0f;
  }
}

// ---------------------------------------------------------------------------
// Overlap matrix of n index tensors sel[n][rows][k]: M[a][b] = mean over rows
// of overlap(sel[a], sel[b]) (same per-row definition as above, so M[a][a] =
// 1). One wave per workgroup walks rows blockIdx.x, blockIdx.x + gridDim.x,
// ...; per row it builds layer a's bitmap, then for every b > a a bitmap of
// b's new positions, counting |B| and |A ∩ B| in one pass. Each per-row
// ratio is added as a 32.32 fixed-point integer (floor(inter * 2^32 / |A|),
// error below 2^-32), first into the workgroup's LDS accumulators, then with
// one 64-bit atomic add per pair into acc[n*n]: integer sums do not depend
// on the order of the additions, so the result is deterministic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void ov_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// overlap(X -> Y) as 32.32 fixed point: inter / |X|, 1 if both are empty, 0
// if only X is
__device__ __forceinline__ unsigned long long ov_fix(int inter, int nx, int ny) {
  if (nx > 0) return ((unsigned long long)inter << 32) / (unsigned long long)nx;
  return ny > 0 ? 0ull : (1ull << 32);
}

__global__ __launch_bounds__(kWave)
void overlap_matrix_kernel(const int32_t* __restrict__ sel, int n, int rows, int k, int Lk,
                           int words, unsigned long long* __restrict__ acc_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(smem);  // [n*n]
  uint32_t* bits_a = reinterpret_cast<uint32_t*>(smem + (size_t)n * n * 8);
  uint32_t* bits_b = bits_a + words;
  const int lane = lane_id();
  for (int p = lane; p < n * n; p += kWave) acc[p] = 0ull;
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    for (int a = 0; a < n; ++a) {
      const int32_t* A = sel + ((size_t)a * rows + row) * k;
      for (int w = lane; w < words; w += kWave) bits_a[w] = 0u;
      ov_wave_sync();
      int na = 0;
      for (int e = lane; e < k; e += kWave) {
        const int p = A[e];
        if (p >= 0 && p < Lk) {
          const uint32_t m = 1u << (p & 31);
          na += (atomicOr(&bits_a[p >> 5], m) & m) ? 0 : 1;
        }
      }
      na = wave_sum(na);
      ov_wave_sync();
      for (int b = a + 1; b < n; ++b) {
        const int32_t* Bl = sel + ((size_t)b * rows + row) * k;
        for (int w = lane; w < words; w += kWave) bits_b[w] = 0u;
        ov_wave_sync();
        int nb = 0, ni = 0;
        for (int e = lane; e < k; e += kWave) {
          const int p = Bl[e];
          if (p >= 0 && p < Lk) {
            const uint32_t m = 1u << (p & 31);
            if (!(atomicOr(&bits_b[p >> 5], m) & m)) {
              ++nb;
              ni += (bits_a[p >> 5] & m) ? 1 : 0;
            }
          }
        }
        nb = wave_sum(nb);
        ni = wave_sum(ni);
        if (lane == 0) {
          acc[a * n + b] += ov_fix(ni, na, nb);
          acc[b * n + a] += ov_fix(ni, nb, na);
        }
        ov_wave_sync();
      }
    }
  }
  ov_wave_sync();
  for (int p = lane; p < n * n; p += kWave)
    if (acc[p] != 0ull) atomicAdd(&acc_out[p], acc[p]);
}

__global__ void overlap_matrix_zero(unsigned long long* __restrict__ acc, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) acc[i] = 0ull;
}

__global__ void overlap_matrix_finish(const unsigned long long* __restrict__ acc, int n, int rows,
                                      float* __restrict__ matrix) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * n) return;
  const int a = i / n, b = i % n;
  matrix[i] = (a == b) ? 1.0f : (float)((double)acc[i] * 0x1p-32 / (double)rows);
}

}  // namespace

size_t overlap_matrix_lds_bytes(int n, int Lk) {
  return (size_t)n * n * 8 + (size_t)2 * ((Lk + 31) / 32) * 4;
}

hipError_t launch_overlap_matrix(const int32_t* sel, int n, int rows, int k, int Lk,
                                 unsigned long long* acc, float* matrix, hipStream_t st) {
  const int words = (Lk + 31) / 32;
  const size_t shmem = overlap_matrix_lds_bytes(n, Lk);
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(overlap_matrix_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const int nn = n * n;
  hipLaunchKernelGGL(overlap_matrix_zero, dim3((unsigned)((nn + 255) / 256)), dim3(256), 0, st,
                     acc, nn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // enough single-wave workgroups to fill the chip; each walks several rows
  const int grid = rows < 4096 ? rows : 4096;
  hipLaunchKernelGGL(overlap_matrix_kernel, dim3((unsigned)grid), dim3(kWave), shmem, st, sel, n,
                     rows, k, Lk, words, acc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(overlap_matrix_finish, dim3((unsigned)((nn + 255) / 256)), dim3(256), 0, st,
                     acc, n, rows, matrix);
  return hipGetLastError();
}

size_t overlap_lds_bytes(int Lk) { return (size_t)2 * ((Lk + 31) / 32) * 4; }

hipError_t launch_overlap(const int32_t* a, const int32_t* b, int rows, int k, int Lk,
                          int32_t* inter, float* overlap, float* jaccard, hipStream_t st) {
  const int words = (Lk + 31) / 32;
  const size_t shmem = overlap_lds_bytes(Lk);
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(overlap_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)rows), dim3(kOvThreads), shmem, st, a, b, k,
                     Lk, words, inter, overlap, jaccard);
  return hipGetLastError();
}

}  // namespace idxc
