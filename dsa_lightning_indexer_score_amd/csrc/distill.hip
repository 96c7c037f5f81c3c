// Multi-layer distillation loss of an index-sharing layer group, for gfx950.
//
// "NLP——IndexCache" notes, section "方法二：Training-Aware IndexCache": an F
// layer l whose indexer also serves the S layers l+1 .. l+m is trained with
//     L_multi = sum_{j=0..m} 1/(m+1) sum_t KL(p_t^(l+j) || q_t),
//     q_t = Softmax(I_t) over the keys of query t,
// where p_t^(l+j) are the served layers' attention distributions (the
// teachers) and I_t the indexer scores. By Proposition 1 there (also the
// "Training-aware" section of "IndexCache：跨层复用稀疏注意力的索引") its
// gradient with respect to the logits is that of one KL against the mean
// teacher p_bar: dL/dI_t = q_t - p_bar_t.
//
// One workgroup per query row. Pass 1 runs an online max / sum of
// exponentials over the row's logits (keys 0..t); pass 2 reads each key's
// logit and the n teachers' probabilities once and writes the gradient, and
// the row's loss sum_s [ (1/n) sum_j p_j log p_j - p_bar log q ] is reduced
// in a fixed order (per thread, then per wave, then over the waves). The kernel is bound by HBM traffic: the logits are read
// twice, each teacher once, the gradient written once.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kDistThreads = 256;
constexpr int kDistWaves = kDistThreads / kWave;

// (m, z) with z = sum exp(x - m); merging two partial states
__device__ __forceinline__ void lse_merge(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  z = z * __expf(m - M) + z2 * __expf(m2 - M);
  m = M;
}

// Per-thread work on 4 consecutive keys at a time (16-byte loads) when rows
// start 16-byte aligned (VEC: Lk % 4 == 0), single keys otherwise.
template <bool VEC>
__global__ __launch_bounds__(kDistThreads)
void distill_kernel(const float* __restrict__ logits, const float* __restrict__ teachers,
                    int n_teachers, int Lq, int Lk, int q_pos0, size_t teacher_stride,
                    float* __restrict__ row_loss, float* __restrict__ grad) {
  __shared__ float red_m[kDistWaves], red_z[kDistWaves], red_l[kDistWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const size_t row = blockIdx.x;
  const int t = q_pos0 + (int)(row % Lq);
  const int n = min(t + 1, Lk);
  const int nv = VEC ? (n & ~3) : 0;  // keys handled 4 at a time
  const float* x = logits + row * Lk;

  // ---- pass 1: log-sum-exp of the row's logits
  float m = -INFINITY, z = 0.0f;
  auto add = [&](float v) {
    if (v > m) {
      z = z * __expf(m - v) + 1.0f;
      m = v;
    } else {
      z += __expf(v - m);
    }
  };
  for (int s = tid * 4; s < nv; s += kDistThreads * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + s);
    add(v[0]);
    add(v[1]);
    add(v[2]);
    add(v[3]);
  }
  for (int s = nv + tid; s < n; s += kDistThreads) add(x[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float z2 = __shfl_xor(z, off, kWave);
    lse_merge(m, z, m2, z2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_z[wave] = z;
  }
  __syncthreads();
  m = red_m[0];
  z = red_z[0];
#pragma unroll
  for (int w = 1; w < kDistWaves; ++w) lse_merge(m, z, red_m[w], red_z[w]);
  const float lse = m + __logf(z);

  // ---- pass 2: gradient and loss terms
  const float inv_n = 1.0f / (float)n_teachers;
  float acc = 0.0f;
  const float* prow = teachers + row * Lk;
  float* grow = grad ? grad + row * Lk : nullptr;
  for (int s = tid * 4; s < nv; s += kDistThreads * 4) {
    const f32x4 lv = *reinterpret_cast<const f32x4*>(x + s);
    f32x4 pbar = {0.0f, 0.0f, 0.0f, 0.0f};
    float plogp = 0.0f;
    for (int j = 0; j < n_teachers; ++j) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(prow + (size_t)j * teacher_stride + s);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pbar[c] += p[c];
        if (p[c] > 0.0f) plogp += p[c] * __logf(p[c]);
      }
    }
    f32x4 gv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lq = lv[c] - lse;
      const float pb = pbar[c] * inv_n;
      acc -= pb * lq;
      gv[c] = __expf(lq) - pb;
    }
    acc += plogp * inv_n;
    if (grow) *reinterpret_cast<f32x4*>(grow + s) = gv;
  }
  for (int s = nv + tid; s < n; s += kDistThreads) {
    const float lq = x[s] - lse;
    float pbar = 0.0f, plogp = 0.0f;
    for (int j = 0; j < n_teachers; ++j) {
      const float p = prow[(size_t)j * teacher_stride + s];
      pbar += p;
      if (p > 0.0f) plogp += p * __logf(p);
    }
    pbar *= inv_n;
    acc += plogp * inv_n - pbar * lq;
    if (grow) grow[s] = __expf(lq) - pbar;
  }
  if (grow)
    for (int s = n + tid; s < Lk; s += kDistThreads) grow[s] = 0.0f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) red_l[wave] = acc;
  __syncthreads();
  if (tid == 0 && row_loss) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kDistWaves; ++w) l += red_l[w];
    row_loss[row] = l;
  }
}

}  // namespace

hipError_t launch_distill(const float* logits, const float* teachers, int n_teachers, int B,
                          int Lq, int Lk, int q_pos0, float* row_loss, float* grad,
                          hipStream_t st) {
  const size_t stride = (size_t)B * Lq * Lk;
  if (Lk % 4 == 0)
    hipLaunchKernelGGL(distill_kernel<true>, dim3((unsigned)(B * Lq)), dim3(kDistThreads), 0, st,
                       logits, teachers, n_teachers, Lq, Lk, q_pos0, stride, row_loss, grad);
  else
    hipLaunchKernelGGL(distill_kernel<false>, dim3((unsigned)(B * Lq)), dim3(kDistThreads), 0, st,
                       logits, teachers, n_teachers, Lq, Lk, q_pos0, stride, row_loss, grad);
  return hipGetLastError();
}

}  // namespace idxc
