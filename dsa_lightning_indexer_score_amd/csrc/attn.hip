// Gathered sparse core attention for gfx950 (one shared K/V head, MQA).
//
// Core attention runs only on the k positions the indexer selected
// ("NLP——IndexCache" notes, section "背景 & 问题提出"; the fugumt.com summary
// of arXiv 2603.12201, abstract): for every query row t and head h,
//     O[t,h] = sum_{s in I_t} softmax_s(scale * Q[t,h] . K[s]) V[s],
// skipping -1 entries of I_t.
//
// One wave owns all heads of a query (or a slice of its index list), so each
// gathered K/V row (2 x D bf16) feeds every head. Scores are computed
// transposed, S^T = K_sel . Q^T, on 32x32x16 MFMAs: a lane then holds 16 keys
// of one head, so the online-softmax max/sum stays in registers apart from one
// lane-half swap, and the rescale of the output accumulators (O^T, heads on
// the N dimension) is a per-lane multiply. P stays in registers as the B
// operand of O^T += V^T P^T; V rows are transposed through a per-wave LDS
// slice whose key order matches the accumulator layout of S^T.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kAttnWaves = 4;
constexpr int kVtRow = 40;  // bf16 per transposed-V row: 32 keys + 8 pad (80 B)

__device__ __forceinline__ void lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Position of key-quad qd (keys 4qd..4qd+3 of a 32-key block) inside a
// transposed-V row, so that the 8 keys one lane needs for a P.V k-step are
// contiguous (they follow the row order of the S^T accumulator layout).
__device__ __forceinline__ int vt_quad_pos(int qd) {
  return (qd & 4) | ((qd & 1) << 1) | ((qd >> 1) & 1);
}

template <int D>
struct BlockRegs {
  static constexpr int KS = D / 16;
  static constexpr int VPL = D / 64;  // (quad, chunk) pairs per lane
  bf16x8 ka[KS];
  u32x4 vr[VPL][4];
  uint32_t vmask;
};

template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D>& br, const uint16_t* __restrict__ kb,
                                           const uint16_t* __restrict__ vb,
                                           const int32_t* __restrict__ irow, int e0, int kend,
                                           int Lk) {
  constexpr int KS = D / 16;
  constexpr int NCHV = D / 8;
  const int lane = lane_id();
  const int e = e0 + (lane & 31);
  int idx = (e < kend) ? irow[e] : -1;
  const bool valid = idx >= 0 && idx < Lk;
  const int srow = valid ? idx : 0;
  br.vmask = (uint32_t)(ballot(valid) & 0xFFFFFFFFull);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    br.ka[ks] = *reinterpret_cast<const bf16x8*>(kb + (size_t)srow * D + (ks * 2 + (lane >> 5)) * 8);
  }
#pragma unroll
  for (int vp = 0; vp < BlockRegs<D>::VPL; ++vp) {
    const int pi = lane + kWave * vp;
    const int qd = pi / NCHV;
    const int c = pi % NCHV;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = __shfl(srow, 4 * qd + r, kWave);
      br.vr[vp][r] = *reinterpret_cast<const u32x4*>(vb + (size_t)rr * D + c * 8);
    }
  }
}

template <int D, int HB>
__global__ __launch_bounds__(kAttnWaves * kWave, 1)
void sparse_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kmat,
                        const uint16_t* __restrict__ vmat, const int32_t* __restrict__ indices,
                        int B, int Lq, int Lk, int H, int k, float sl2,
                        uint16_t* __restrict__ out, int wpq) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NCHV = D / 8;
  constexpr int VPL = D / 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int rows = B * Lq;
  int rowq, kbeg, kend;
  if (wpq == 1) {
    rowq = blockIdx.x * kAttnWaves + wave;
    kbeg = 0;
    kend = k;
    if (rowq >= rows) return;
  } else {
    rowq = blockIdx.x;
    const int per = ((k + kAttnWaves * 32 - 1) / (kAttnWaves * 32)) * 32;
    kbeg = min(k, wave * per);
    kend = min(k, kbeg + per);
  }
  const int b = rowq / Lq;
  const uint16_t* kb = kmat + (size_t)b * Lk * D;
  const uint16_t* vb = vmat + (size_t)b * Lk * D;
  const int32_t* irow = indices + (size_t)rowq * k;
  uint16_t* vt = reinterpret_cast<uint16_t*>(dyn) + wave * D * kVtRow;

  // Q^T as the B operand of S^T = K . Q^T (heads on N)
  bf16x8 qb[HB][KS];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qb[hb][ks] = (h < H) ? *reinterpret_cast<const bf16x8*>(
                                 q + ((size_t)rowq * H + h) * D + (ks * 2 + (lane >> 5)) * 8)
                           : bf16x8{};
    }
  }

  float m[HB], lsum[HB];
  f32x16 o[DB][HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m[hb] = -INFINITY;
    lsum[hb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][hb] = f32x16{};
  }

  BlockRegs<D> cur, nxt;
  if (kbeg < kend) load_block<D>(cur, kb, vb, irow, kbeg, kend, Lk);
  for (int e0 = kbeg; e0 < kend; e0 += 32) {
    if (e0 + 32 < kend) load_block<D>(nxt, kb, vb, irow, e0 + 32, kend, Lk);

    // ---- V^T of this block into the wave's LDS slice (4 keys x 8 d per pair)
#pragma unroll
    for (int vp = 0; vp < VPL; ++vp) {
      const int pi = lane + kWave * vp;
      const int qd = pi / NCHV;
      const int c = pi % NCHV;
      const int col = vt_quad_pos(qd) * 4;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int wd = jj >> 1;
        const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pk;
        pk.x = __builtin_amdgcn_perm(cur.vr[vp][1][wd], cur.vr[vp][0][wd], sel);
        pk.y = __builtin_amdgcn_perm(cur.vr[vp][3][wd], cur.vr[vp][2][wd], sel);
        *reinterpret_cast<u32x2*>(&vt[(c * 8 + jj) * kVtRow + col]) = pk;
      }
    }

    // ---- S^T = K . Q^T, online softmax (log2 domain), P^T as bf16 B operands
    bf16x8 pb[HB][2];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = mfma32(cur.ka[ks], qb[hb][ks], s);
      float x[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = acc_row(i, lane);
        const bool ok = (cur.vmask >> slot) & 1u;
        x[i] = ok ? s[i] * sl2 : -INFINITY;
        mloc = fmaxf(mloc, x[i]);
      }
      const float mblk = pair_max(mloc);
      const float mnew = fmaxf(m[hb], mblk);
      const bool none = mnew == -INFINITY;
      const float alpha = none ? 1.0f : exp2f(m[hb] - mnew);
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = none ? 0.0f : exp2f(x[i] - mnew);
        psum += p;
        pb[hb][i >> 3][i & 7] = (__bf16)p;
      }
      lsum[hb] = lsum[hb] * alpha + psum;
      m[hb] = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][hb] *= alpha;
    }

    lds_fence();
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(
            &vt[(db * 32 + (lane & 31)) * kVtRow + 16 * kk + 8 * (lane >> 5)]);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[db][hb] = mfma32(va, pb[hb][kk], o[db][hb]);
      }
    }
    lds_fence();
    cur = nxt;
  }

  float lt[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) lt[hb] = pair_sum(lsum[hb]);

  if (wpq != 1) {
    // ---- merge the 4 waves' partial softmax states through LDS into wave 0
    constexpr int NF = DB * HB * 16 + 2 * HB;  // floats per lane
    float* slot = reinterpret_cast<float*>(dyn);
    for (int ws = 1; ws < kAttnWaves; ++ws) {
      __syncthreads();
      if (wave == ws) {
        int f = 0;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) slot[(f++) * kWave + lane] = o[db][hb][i];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          slot[(f++) * kWave + lane] = m[hb];
          slot[(f++) * kWave + lane] = lt[hb];
        }
      }
      __syncthreads();
      if (wave == 0) {
        float a0[HB], a1[HB];
        int f = DB * HB * 16;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const float m1 = slot[(f++) * kWave + lane];
          const float l1 = slot[(f++) * kWave + lane];
          const float mn = fmaxf(m[hb], m1);
          a0[hb] = (m[hb] == -INFINITY) ? 0.0f : exp2f(m[hb] - mn);
          a1[hb] = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mn);
          lt[hb] = lt[hb] * a0[hb] + l1 * a1[hb];
          m[hb] = mn;
        }
        f = 0;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              o[db][hb][i] = o[db][hb][i] * a0[hb] + slot[(f++) * kWave + lane] * a1[hb];
            }
      }
    }
    if (wave != 0) return;
  }

  // ---- normalise and store bf16 (acc rows = d, cols = heads)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 32 + (lane & 31);
    if (h >= H) continue;
    const float inv = lt[hb] > 0.0f ? 1.0f / lt[hb] : 0.0f;
    uint16_t* orow = out + ((size_t)rowq * H + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * (lane >> 5);
        u32x2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[db][hb][4 * g + 0] * inv) |
               ((uint32_t)f32_to_bf16(o[db][hb][4 * g + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[db][hb][4 * g + 2] * inv) |
               ((uint32_t)f32_to_bf16(o[db][hb][4 * g + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
    }
  }
}

template <int D, int HB>
hipError_t launch(const AttnArgs& a, hipStream_t st) {
  const int rows = a.B * a.Lq;
  const int wpq = rows >= 1024 ? 1 : kAttnWaves;
  const unsigned grid = wpq == 1 ? (unsigned)((rows + kAttnWaves - 1) / kAttnWaves) : (unsigned)rows;
  constexpr int DB = D / 32;
  const size_t vt_bytes = (size_t)kAttnWaves * D * kVtRow * 2;
  const size_t merge_bytes = (size_t)(DB * HB * 16 + 2 * HB) * kWave * 4;
  const size_t shmem = vt_bytes > merge_bytes ? vt_bytes : merge_bytes;
  const float sl2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((sparse_attn_kernel<D, HB>), dim3(grid), dim3(kAttnWaves * kWave), shmem, st,
                     a.q, a.key, a.val, a.indices, a.B, a.Lq, a.Lk, a.H, a.topk, sl2, a.out, wpq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  const int hb = (a.H + 31) / 32;
  if (a.D == 64) return hb == 1 ? launch<64, 1>(a, st) : launch<64, 2>(a, st);
  return hb == 1 ? launch<128, 1>(a, st) : launch<128, 2>(a, st);
}

}  // namespace idxc
