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
// One workgroup per query row; the kernel is bound by HBM traffic. Rows of up
// to 32768 keys with at most four teachers (an F layer and the S layers it
// serves under the usual patterns) keep the row's logits in registers: each
// logit is read once, each teacher entry once, each gradient entry written
// once. Pass 1 takes the log-sum-exp of the held logits (keys 0..t); pass 2
// streams the teachers and writes the gradient. Other aligned rows (longer,
// or more teachers) run the same two passes streamed, reading the logits
// twice; rows that are not 16-byte aligned, one key per thread at a time.
// The row's loss
// sum_s [ (1/n) sum_j p_j log p_j - p_bar log q ] (terms with p = 0 are 0) is
// reduced in a fixed order (per thread, then per wave, then over the waves).
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

// Rows that do not start 16-byte aligned (Lk % 4 != 0): the two passes one
// key per thread at a time, the logits read twice.
__global__ __launch_bounds__(kDistThreads)
void distill_scalar_kernel(const float* __restrict__ logits, const float* __restrict__ teachers,
                           int n_teachers, int Lq, int Lk, int q_pos0, size_t teacher_stride,
                           float* __restrict__ row_loss, float* __restrict__ grad) {
  __shared__ float red_m[kDistWaves], red_z[kDistWaves], red_l[kDistWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const size_t row = blockIdx.x;
  const int t = q_pos0 + (int)(row % Lq);
  const int n = min(t + 1, Lk);
  const float* x = logits + row * Lk;

  // ---- pass 1: log-sum-exp of the row's logits
  float m = -INFINITY, z = 0.0f;
  for (int s = tid; s < n; s += kDistThreads) {
    const float v = x[s];
    if (v > m) {
      z = z * __expf(m - v) + 1.0f;
      m = v;
    } else {
      z += __expf(v - m);
    }
  }
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
  for (int s = tid; s < n; s += kDistThreads) {
    const float lq = x[s] - lse;
    float pbar = 0.0f, plogp = 0.0f;
    for (int j = 0; j < n_teachers; ++j) {
      const float p = __builtin_nontemporal_load(prow + (size_t)j * teacher_stride + s);
      pbar += p;
      if (p > 0.0f) plogp += p * __logf(p);
    }
    pbar *= inv_n;
    acc += plogp * inv_n - (pbar > 0.0f ? pbar * lq : 0.0f);
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

// ---- register-resident rows
constexpr int kRegThreads = 512;
constexpr int kRegWaves = kRegThreads / kWave;
constexpr int kRegMaxGroups = 16;  // 4-key groups per thread: rows up to 32768 keys
constexpr int kRegMaxTeachers = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMinNormal = 1.17549435e-38f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const float* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, bytes, 0x00020000);
}

// e^v as the hardware's base-2 exponential of v log2(e)
__device__ __forceinline__ float exp_hw(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// (m, z) with z = sum exp(x - m)
__device__ __forceinline__ void lse_merge_hw(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  z = z * exp_hw(m - M) + z2 * exp_hw(m2 - M);
  m = M;
}

// p log2 p, with p below the smallest normal float taken as 0 (its term is
// under 1e-36; the hardware log is only used on normal inputs)
__device__ __forceinline__ float plog2p(float p) {
  const float v = p * __builtin_amdgcn_logf(p);
  return p >= kMinNormal ? v : 0.0f;
}

// Key group g = c * kRegThreads + tid (keys 4g .. 4g+3) is held by thread tid
// as xv[c]. Exponentials and logarithms use the hardware's base-2
// instructions (single instructions, about 1 ulp): exponents are scaled by
// log2(e) only after the max or the log-sum-exp is subtracted, so the large
// probabilities see the rounding of a small number, and the teachers'
// entropy terms are summed in base 2 and scaled by ln 2 once per thread.
// Rows start 16-byte aligned (Lk % 4 == 0) and Lk <= 4 * CH * kRegThreads.
// The row's full groups (nvec = n / 4 of them) are read through buffer
// resources sized to them, so every load is issued unconditionally and
// groups past them read 0; the partly valid last group (n % 4 keys) is read
// key by key by the one thread that owns it. Gradient stores go through a
// resource sized to the row (size 0 without a gradient output), so groups
// past Lk are dropped and groups in [n/4, Lk/4) receive zeros. Logit and
// teacher loads carry the non-temporal hint (aux 2): every byte is read once,
// and measured it streams faster; the gradient stores stay ordinary (the
// hint on them measured slower).
template <int CH, int NT>
__global__ __launch_bounds__(kRegThreads, 4)  // 4 waves per SIMD: two rows per CU
void distill_reg_kernel(const float* __restrict__ logits, const float* __restrict__ teachers,
                        int Lq, int Lk, int q_pos0, size_t teacher_stride,
                        float* __restrict__ row_loss, float* __restrict__ grad) {
  __shared__ float red_m[kRegWaves], red_z[kRegWaves], red_l[kRegWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const size_t row = blockIdx.x;
  const int t = q_pos0 + (int)(row % Lq);
  const int n = min(t + 1, Lk);
  const int nvec = n >> 2;
  const int tail = n & 3;
  const bool tail_owner = tail != 0 && tid == nvec % kRegThreads;
  const float* x = logits + row * Lk;
  const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};

  // ---- pass 1: hold the row, log-sum-exp
  const __amdgpu_buffer_rsrc_t xr = span_rsrc(x, nvec * 16);
  f32x4 xv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
    xv[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          xr, (c * kRegThreads + tid) * 16, 0, 2));
  // the partly valid last group, key by key, through a resource sized to the
  // row's keys (every other thread reads past it and gets 0)
  const __amdgpu_buffer_rsrc_t xr1 = span_rsrc(x, n * 4);
  f32x4 xt;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    xt[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          xr1, tail_owner ? (4 * nvec + e) * 4 : n * 4, 0, 0));
  // the first teacher group's loads go out now and land during the reduction
  const float* prow = teachers + row * Lk;
  __amdgpu_buffer_rsrc_t pr[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) pr[j] = span_rsrc(prow + (size_t)j * teacher_stride, nvec * 16);
  f32x4 pn[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    pn[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr[j], tid * 16, 0, 2));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CH; ++c) xv[c] = c * kRegThreads + tid < nvec ? xv[c] : ninf;
#pragma unroll
  for (int e = 0; e < 4; ++e) xt[e] = tail_owner && e < tail ? xt[e] : -INFINITY;
  float m = fmaxf(fmaxf(xt[0], xt[1]), fmaxf(xt[2], xt[3]));
#pragma unroll
  for (int c = 0; c < CH; ++c)
    m = fmaxf(m, fmaxf(fmaxf(xv[c][0], xv[c][1]), fmaxf(xv[c][2], xv[c][3])));
  const float ms = m == -INFINITY ? 0.0f : m;  // a thread with no keys: z = 0
  float z = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) z += exp_hw(xv[c][e] - ms);
#pragma unroll
  for (int e = 0; e < 4; ++e) z += exp_hw(xt[e] - ms);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float z2 = __shfl_xor(z, off, kWave);
    lse_merge_hw(m, z, m2, z2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_z[wave] = z;
  }
  __syncthreads();
  m = red_m[0];
  z = red_z[0];
#pragma unroll
  for (int w = 1; w < kRegWaves; ++w) lse_merge_hw(m, z, red_m[w], red_z[w]);
  // z >= 1 when the row has a finite logit
  const float lse = m + __builtin_amdgcn_logf(z) * kLn2;

  // ---- pass 2: stream the teachers, write the gradient
  const float inv_n = 1.0f / (float)NT;
  float* grow = grad ? grad + row * Lk : nullptr;
  const __amdgpu_buffer_rsrc_t gr = span_rsrc(grow, grow ? Lk * 4 : 0);
  float acc = 0.0f;    // - sum p_bar log q
  float acc_h2 = 0.0f;  // (1/n) sum_j p_j log2 p_j
  // one group's teacher loads in flight ahead of the group being reduced; the
  // scheduling barriers keep the compiler from hoisting every load (which
  // would need all CH * NT groups in registers at once)
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int g = c * kRegThreads + tid;
    f32x4 p[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) p[j] = pn[j];
    if (c + 1 < CH) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
        pn[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              pr[j], (g + kRegThreads) * 16, 0, 2));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 pb = p[0];
#pragma unroll
    for (int j = 1; j < NT; ++j) pb += p[j];
    float plogp = 0.0f;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) plogp += plog2p(p[j][e]);
    f32x4 gv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lq = xv[c][e] - lse;
      const float pbe = pb[e] * inv_n;
      acc -= pbe > 0.0f ? pbe * lq : 0.0f;
      gv[e] = exp_hw(lq) - pbe;
    }
    acc_h2 += plogp * inv_n;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, gv), gr,
                                           (tail != 0 && g == nvec) ? Lk * 4 : g * 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (tail_owner) {
    f32x4 pb = {0.0f, 0.0f, 0.0f, 0.0f};
    float plogp = 0.0f;
    for (int j = 0; j < NT; ++j)
      for (int e = 0; e < tail; ++e) {
        const float p = prow[(size_t)j * teacher_stride + 4 * nvec + e];
        pb[e] += p;
        plogp += plog2p(p);
      }
    f32x4 gv = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int e = 0; e < tail; ++e) {
      const float lq = xt[e] - lse;
      const float pbe = pb[e] * inv_n;
      acc -= pbe > 0.0f ? pbe * lq : 0.0f;
      gv[e] = exp_hw(lq) - pbe;
    }
    acc_h2 += plogp * inv_n;
    if (grow) *reinterpret_cast<f32x4*>(grow + 4 * nvec) = gv;
  }
  acc += acc_h2 * kLn2;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) red_l[wave] = acc;
  __syncthreads();
  if (tid == 0 && row_loss) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kRegWaves; ++w) l += red_l[w];
    row_loss[row] = l;
  }
}

// ---- streamed rows: aligned rows the register-held kernel does not take
// (longer than 32768 keys, or more than four teachers). The same two passes
// with the logits read twice (the second read, their last, mostly from the
// last-level cache) and the teachers once; the teacher loads and the second
// logit read carry the non-temporal hint. Loads go
// through buffer resources sized to the row's full 4-key groups and are
// issued unconditionally, four groups deep in pass 1 and two groups (and two
// teachers) deep in pass 2; the partly valid last group is the owning
// thread's, as in the register-held kernel.
constexpr int kStreamThreads = 1024;  // measured faster than 512 with eight teachers

template <int NTHR>
__global__ __launch_bounds__(NTHR)
void distill_stream_kernel(const float* __restrict__ logits, const float* __restrict__ teachers,
                           int n_teachers, int Lq, int Lk, int q_pos0, size_t teacher_stride,
                           float* __restrict__ row_loss, float* __restrict__ grad) {
  constexpr int NW = NTHR / kWave;
  __shared__ float red_m[NW], red_z[NW], red_l[NW];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const size_t row = blockIdx.x;
  const int t = q_pos0 + (int)(row % Lq);
  const int n = min(t + 1, Lk);
  const int nvec = n >> 2;
  const int tail = n & 3;
  const bool tail_owner = tail != 0 && tid == nvec % NTHR;
  const float* x = logits + row * Lk;
  const __amdgpu_buffer_rsrc_t xr = span_rsrc(x, nvec * 16);

  // ---- pass 1: online log-sum-exp over the row's logits
  float m = -INFINITY, z = 0.0f;
  auto add4 = [&](const f32x4& v) {
    const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    if (mx > m) {
      z *= exp_hw(m - mx);  // 0 while m is -inf
      m = mx;
    }
    if (m != -INFINITY) z += exp_hw(v[0] - m) + exp_hw(v[1] - m) + exp_hw(v[2] - m) + exp_hw(v[3] - m);
  };
  for (int g0 = tid; g0 < nvec; g0 += 4 * NTHR) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           xr, (g0 + u * NTHR) * 16, 0, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (g0 + u * NTHR < nvec) add4(v[u]);
  }
  f32x4 xt = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (tail_owner) {
    for (int e = 0; e < tail; ++e) xt[e] = x[4 * nvec + e];
    add4(xt);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float z2 = __shfl_xor(z, off, kWave);
    lse_merge_hw(m, z, m2, z2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_z[wave] = z;
  }
  __syncthreads();
  m = red_m[0];
  z = red_z[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) lse_merge_hw(m, z, red_m[w], red_z[w]);
  const float lse = m + __builtin_amdgcn_logf(z) * kLn2;

  // ---- pass 2: teachers, gradient and loss terms over every group of the
  // row (groups past the row's keys get zero gradients)
  const float inv_n = 1.0f / (float)n_teachers;
  const float* prow = teachers + row * Lk;
  float* grow = grad ? grad + row * Lk : nullptr;
  const __amdgpu_buffer_rsrc_t gr = span_rsrc(grow, grow ? Lk * 4 : 0);
  const int ngrp = Lk >> 2;
  float acc = 0.0f, acc_h2 = 0.0f;
  for (int g0 = tid; g0 < ngrp; g0 += 2 * NTHR) {
    f32x4 xv[2], pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      xv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xr, (g0 + u * NTHR) * 16, 0, 2));
      pb[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float plogp = 0.0f;
#pragma unroll 2
    for (int j = 0; j < n_teachers; ++j) {
      const __amdgpu_buffer_rsrc_t pr = span_rsrc(prow + (size_t)j * teacher_stride, nvec * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x4 p = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      pr, (g0 + u * NTHR) * 16, 0, 2));
        pb[u] += p;
#pragma unroll
        for (int e = 0; e < 4; ++e) plogp += plog2p(p[e]);
      }
    }
    acc_h2 += plogp * inv_n;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int g = g0 + u * NTHR;
      f32x4 gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lq = g < nvec ? xv[u][e] - lse : -INFINITY;
        const float pbe = pb[u][e] * inv_n;
        acc -= pbe > 0.0f ? pbe * lq : 0.0f;
        gv[e] = exp_hw(lq) - pbe;
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, gv), gr,
                                             (tail != 0 && g == nvec) ? Lk * 4 : g * 16, 0, 0);
    }
  }
  if (tail_owner) {
    f32x4 pb = {0.0f, 0.0f, 0.0f, 0.0f};
    float plogp = 0.0f;
    for (int j = 0; j < n_teachers; ++j)
      for (int e = 0; e < tail; ++e) {
        const float p = prow[(size_t)j * teacher_stride + 4 * nvec + e];
        pb[e] += p;
        plogp += plog2p(p);
      }
    f32x4 gv = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int e = 0; e < tail; ++e) {
      const float lq = xt[e] - lse;
      const float pbe = pb[e] * inv_n;
      acc -= pbe > 0.0f ? pbe * lq : 0.0f;
      gv[e] = exp_hw(lq) - pbe;
    }
    acc_h2 += plogp * inv_n;
    if (grow) *reinterpret_cast<f32x4*>(grow + 4 * nvec) = gv;
  }
  acc += acc_h2 * kLn2;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) red_l[wave] = acc;
  __syncthreads();
  if (tid == 0 && row_loss) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) l += red_l[w];
    row_loss[row] = l;
  }
}

template <int CH>
hipError_t launch_reg(const float* logits, const float* teachers, int n_teachers, int rows,
                      int Lq, int Lk, int q_pos0, size_t stride, float* row_loss, float* grad,
                      hipStream_t st) {
  switch (n_teachers) {
#define IDXC_DISTILL_NT(NT)                                                                  \
  case NT:                                                                                   \
    hipLaunchKernelGGL((distill_reg_kernel<CH, NT>), dim3((unsigned)rows), dim3(kRegThreads), \
                       0, st, logits, teachers, Lq, Lk, q_pos0, stride, row_loss, grad);     \
    break;
    IDXC_DISTILL_NT(1)
    IDXC_DISTILL_NT(2)
    IDXC_DISTILL_NT(3)
    IDXC_DISTILL_NT(4)
#undef IDXC_DISTILL_NT
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_distill(const float* logits, const float* teachers, int n_teachers, int B,
                          int Lq, int Lk, int q_pos0, float* row_loss, float* grad,
                          hipStream_t st) {
  const size_t stride = (size_t)B * Lq * Lk;
  const int rows = B * Lq;
  if (Lk % 4 == 0 && n_teachers <= kRegMaxTeachers) {
    if (Lk <= 4 * kRegThreads * 4)
      return launch_reg<4>(logits, teachers, n_teachers, rows, Lq, Lk, q_pos0, stride, row_loss,
                           grad, st);
    if (Lk <= 4 * kRegThreads * 8)
      return launch_reg<8>(logits, teachers, n_teachers, rows, Lq, Lk, q_pos0, stride, row_loss,
                           grad, st);
    if (Lk <= 4 * kRegThreads * kRegMaxGroups)
      return launch_reg<kRegMaxGroups>(logits, teachers, n_teachers, rows, Lq, Lk, q_pos0, stride,
                                       row_loss, grad, st);
  }
  if (Lk % 4 == 0)
    hipLaunchKernelGGL(distill_stream_kernel<kStreamThreads>, dim3((unsigned)rows),
                       dim3(kStreamThreads), 0, st, logits, teachers, n_teachers, Lq, Lk, q_pos0,
                       stride, row_loss, grad);
  else
    hipLaunchKernelGGL(distill_scalar_kernel, dim3((unsigned)rows), dim3(kDistThreads), 0, st,
                       logits, teachers, n_teachers, Lq, Lk, q_pos0, stride, row_loss, grad);
  return hipGetLastError();
}

}  // namespace idxc
