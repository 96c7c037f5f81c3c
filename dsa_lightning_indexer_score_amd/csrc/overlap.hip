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
// against the first bitmap. The lists are read once, coalesced: the kernel is
// bound by HBM reads of the two index tensors.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kOvThreads = 256;

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
  for (int w = tid; w < 2 * words; w += kOvThreads) bits[w] = 0u;
  __syncthreads();

  const int32_t* ar = a + row * k;
  const int32_t* br = b + row * k;
  int na = 0;
  for (int e = tid; e < k; e += kOvThreads) {
    const int p = ar[e];
    if (p >= 0 && p < Lk) {
      const uint32_t m = 1u << (p & 31);
      na += (atomicOr(&bits_a[p >> 5], m) & m) ? 0 : 1;
    }
  }
  __syncthreads();
  int nb = 0, ni = 0;
  for (int e = tid; e < k; e += kOvThreads) {
    const int p = br[e];
    if (p >= 0 && p < Lk) {
      const uint32_t m = 1u << (p & 31);
      if (!(atomicOr(&bits_b[p >> 5], m) & m)) {
        ++nb;
        ni += (bits_a[p >> 5] & m) ? 1 : 0;
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

}  // namespace

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
