// Gathered sparse core attention for gfx950 (one shared K/V head, MQA).
//
// Core attention runs only on the k positions the indexer selected
// ("NLP——IndexCache" notes, section "背景 & 问题提出"; the fugumt.com summary
// of arXiv 2603.12201, abstract): for every query row t and head h,
//     O[t,h] = sum_{s in I_t} softmax_s(scale * Q[t,h] . K[s]) V[s],
// skipping -1 entries of I_t.
//
// Work unit = (query row, slice of its index list). A unit's 32-key blocks of
// K and V rows are gathered once into LDS and shared by the waves that own
// the unit's head blocks (32 heads each), so every gathered row feeds all
// heads of the query. With two head blocks, one wave gathers K and the other
// V, two blocks ahead in registers. Scores are computed transposed,
// S^T = K_sel . Q^T, on 32x32x16 MFMAs: a lane holds 16 keys of one head, so
// the online-softmax max/sum stays in registers apart from one lane-half
// swap, and rescaling the output accumulators (O^T, heads on N) is a per-lane
// multiply. The running maximum is only moved (and the accumulators rescaled)
// when a block raises it by more than 2^8 in the exp2 domain, which keeps
// every P below 256. V rows are transposed on the way into LDS so that the
// P.V MFMA reads contiguous keys.
//
// A unit covering only a slice of the list writes a partial result (bf16
// output normalised by its own sum, plus that sum and the max); a second
// kernel combines the slices of each row.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kAttnWaves = 4;
constexpr int kVtRow = 40;          // bf16 per transposed-V row: 32 keys + 8 pad (80 B)
constexpr float kLazyLog2 = 8.0f;   // rescale threshold (exp2 domain)
constexpr int kMaxAttnSplits = 32;

// Position of key-quad qd (keys 4qd..4qd+3 of a 32-key block) inside a
// transposed-V row, so that the 8 keys one lane needs for a P.V k-step are
// contiguous (they follow the row order of the S^T accumulator layout).
__device__ __forceinline__ int vt_quad_pos(int qd) {
  return (qd & 4) | ((qd & 1) << 1) | ((qd >> 1) & 1);
}

// Byte offset of 16-byte chunk ch (0..3) of transposed-V row d. Rows are
// 80 bytes apart, so 16 consecutive rows hit 16 different bank groups (the
// P.V operand reads); the chunk is XOR-ed with (d / 16) % 4 so that the rows
// 8 apart written by one instruction of the transpose spread over 8 bank
// groups instead of 2.
__device__ __forceinline__ int vt_off(int d, int ch) {
  return d * (kVtRow * 2) + ((ch ^ ((d >> 4) & 3)) << 4);
}

// Gathered rows of one 32-key block in registers. A K-gathering wave holds
// r[ks] = (slot l%32, 16 B chunk 2ks + l/32); a V-gathering wave holds, for
// each of its D/64 (key quad, chunk) pairs, 4 rows x 16 B. Both need D/16
// registers of 16 B; a wave that gathers both uses 2*D/16.
template <int D, int NR>
struct Gather {
  u32x4 r[NR];
};

template <int D, int NR>
__device__ __forceinline__ void gather_k(Gather<D, NR>& g, const uint16_t* __restrict__ kb,
                                         int srow) {
  const int lane = lane_id();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    g.r[ks] = *reinterpret_cast<const u32x4*>(kb + (size_t)srow * D + (ks * 2 + (lane >> 5)) * 8);
}

template <int D, int NR, int OFF>
__device__ __forceinline__ void gather_v(Gather<D, NR>& g, const uint16_t* __restrict__ vb,
                                         int srow) {
  constexpr int NCHV = D / 8;
  const int lane = lane_id();
#pragma unroll
  for (int vp = 0; vp < D / 64; ++vp) {
    const int pi = lane + kWave * vp;
    const int qd = pi / NCHV;
    const int c = pi % NCHV;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = __shfl(srow, 4 * qd + r, kWave);
      g.r[OFF + vp * 4 + r] = *reinterpret_cast<const u32x4*>(vb + (size_t)rr * D + c * 8);
    }
  }
}

template <int D, int NR>
__device__ __forceinline__ void stage_k(const Gather<D, NR>& g, uint8_t* kl) {
  const int lane = lane_id();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    *reinterpret_cast<u32x4*>(kl + ks * 1024 + lane * 16) = g.r[ks];
}

template <int D, int NR, int OFF>
__device__ __forceinline__ void stage_v(const Gather<D, NR>& g, uint16_t* vt) {
  constexpr int NCHV = D / 8;
  const int lane = lane_id();
#pragma unroll
  for (int vp = 0; vp < D / 64; ++vp) {
    const int pi = lane + kWave * vp;
    const int qd = pi / NCHV;
    const int c = pi % NCHV;
    const int pq = vt_quad_pos(qd);  // 8-byte slot within the 64 data bytes
    const u32x4* rows = &g.r[OFF + vp * 4];
    uint8_t* vtb = reinterpret_cast<uint8_t*>(vt);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int wd = jj >> 1;
      const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
      u32x2 pk;
      pk.x = __builtin_amdgcn_perm(rows[1][wd], rows[0][wd], sel);
      pk.y = __builtin_amdgcn_perm(rows[3][wd], rows[2][wd], sel);
      *reinterpret_cast<u32x2*>(vtb + vt_off(c * 8 + jj, pq >> 1) + (pq & 1) * 8) = pk;
    }
  }
}

// LDS bytes of one unit's buffer: K operand slabs + transposed V.
template <int D>
constexpr int unit_lds_bytes() {
  return (D / 16) * 1024 + D * kVtRow * 2;
}

template <int D, int HB>
__global__ __launch_bounds__(kAttnWaves * kWave, (D == 128 && HB == 1) ? 1 : 2)
void sparse_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kmat,
                        const uint16_t* __restrict__ vmat, const int32_t* __restrict__ indices,
                        int B, int Lq, int Lk, int H, int k, int nsplit, float sl2,
                        uint16_t* __restrict__ out, uint16_t* __restrict__ part_o,
                        float* __restrict__ part_ml) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int UPW = kAttnWaves / HB;  // units per workgroup
  constexpr int UB = unit_lds_bytes<D>();
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int ul = wave / HB;  // unit slot in this workgroup
  const int hb = wave % HB;
  const int rows = B * Lq;
  const int unit = blockIdx.x * UPW + ul;
  const int rowq = unit / nsplit;
  const int split = unit % nsplit;
  const bool active = rowq < rows;
  const int per = ((k + nsplit * 32 - 1) / (nsplit * 32)) * 32;  // keys per split
  const int kbeg = min(k, split * per);
  const int kend = min(k, kbeg + per);
  const int nblk = per / 32;  // same for every unit: keeps the barriers aligned
  const int b = active ? rowq / Lq : 0;
  const uint16_t* kb = kmat + (size_t)b * Lk * D;
  const uint16_t* vb = vmat + (size_t)b * Lk * D;
  const int32_t* irow = indices + (size_t)(active ? rowq : 0) * k;

  // Q^T (this wave's 32 heads) as the B operand of S^T = K . Q^T
  const int h = hb * 32 + (lane & 31);
  bf16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qb[ks] = (active && h < H) ? *reinterpret_cast<const bf16x8*>(
                                     q + ((size_t)rowq * H + h) * D + (ks * 2 + (lane >> 5)) * 8)
                               : bf16x8{};
  }

  float m_used = -INFINITY, lsum = 0.0f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  // gather row of this lane's slot (l % 32) of block j; *vmask = valid slots
  auto slot_index = [&](int j, uint32_t* vmask) {
    const int e = kbeg + j * 32 + (lane & 31);
    const int idx = (active && e < kend) ? irow[e] : -1;
    const bool valid = idx >= 0 && idx < Lk;
    *vmask = (uint32_t)(ballot(valid) & 0xFFFFFFFFull);
    return valid ? idx : 0;
  };

  // with two head blocks, wave hb=0 gathers K and wave hb=1 gathers V
  constexpr int NR = (HB == 1) ? 2 * KS : KS;
  constexpr int VOFF = (HB == 1) ? KS : 0;
  Gather<D, NR> ga, gb;  // ga: block j+2 (in flight), gb: block j+1
  uint32_t vm_a = 0, vm_b = 0, vm_c = 0;
  uint8_t* base = dyn + ul * 2 * UB;

  auto gather = [&](Gather<D, NR>& g, int srow) {
    if (HB == 1 || hb == 0) gather_k<D, NR>(g, kb, srow);
    if (HB == 1 || hb == 1) gather_v<D, NR, VOFF>(g, vb, srow);
  };
  auto stage = [&](const Gather<D, NR>& g, int buf) {
    uint8_t* kl = base + buf * UB;
    uint16_t* vt = reinterpret_cast<uint16_t*>(kl + KS * 1024);
    if (HB == 1 || hb == 0) stage_k<D, NR>(g, kl);
    if (HB == 1 || hb == 1) stage_v<D, NR, VOFF>(g, vt);
  };

  // raw index-list entries, loaded two blocks before their gather is issued
  auto raw_index = [&](int j) {
    const int e = kbeg + j * 32 + (lane & 31);
    return (active && j < nblk && e < kend) ? irow[e] : -1;
  };
  auto resolve = [&](int idx, uint32_t* vmask) {
    const bool valid = idx >= 0 && idx < Lk;
    *vmask = (uint32_t)(ballot(valid) & 0xFFFFFFFFull);
    return valid ? idx : 0;
  };
  int ix2 = raw_index(2), ix3 = raw_index(3);
  {
    const int r0 = slot_index(0, &vm_c);
    gather(ga, r0);
    if (nblk > 1) {
      const int r1 = slot_index(1, &vm_b);
      gather(gb, r1);
    }
    stage(ga, 0);
  }
  __syncthreads();

  // One 32-key block. g_far receives block j+2, g_next (block j+1) is staged
  // at the end; the loop alternates the two register sets.
  auto block = [&](int j, Gather<D, NR>& g_far, Gather<D, NR>& g_next) {
    if (j + 2 < nblk) {
      const int r2 = resolve(ix2, &vm_a);
      gather(g_far, r2);
    }
    ix2 = ix3;
    ix3 = raw_index(j + 4);
    const uint8_t* kl = base + (j & 1) * UB;
    const uint16_t* vt = reinterpret_cast<const uint16_t*>(kl + KS * 1024);

    // ---- S^T = K . Q^T for this wave's 32 heads
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + ks * 1024 + lane * 16);
      s = mfma32(ka, qb[ks], s);
    }
    // ---- online softmax in the exp2 domain with a lazily moved maximum
    float x[16];
    float mloc = -INFINITY;
    if (vm_c == 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = s[i] * sl2;
        mloc = fmaxf(mloc, x[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = (vm_c >> acc_row(i, lane)) & 1u;
        x[i] = ok ? s[i] * sl2 : -INFINITY;
        mloc = fmaxf(mloc, x[i]);
      }
    }
    const float mblk = pair_max(mloc);
    const bool move = mblk > m_used + kLazyLog2;
    if (ballot(move)) {
      const float mnew = move ? mblk : m_used;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_used - mnew) : 1.0f;  // 2^-inf = 0
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_used = mnew;
    }
    // x - m_used <= 8 keeps P <= 256; -inf maps to 0
    const float mu = (m_used == -INFINITY) ? 0.0f : m_used;
    u32x4 pw[2];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[i] - mu);
      const float p1 = __builtin_amdgcn_exp2f(x[i + 1] - mu);
      psum += p0 + p1;
      pw[i >> 3][(i & 7) >> 1] = pack_bf16x2(p0, p1);
    }
    lsum += psum;
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[kk]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(
            reinterpret_cast<const uint8_t*>(vt) + vt_off(db * 32 + (lane & 31), 2 * kk + (lane >> 5)));
        o[db] = mfma32(va, pb, o[db]);
      }
    }
    // ---- stage block j+1 into the other buffer (nobody has read it since
    // the barrier that ended block j-1)
    if (j + 1 < nblk) stage(g_next, (j + 1) & 1);
    vm_c = vm_b;
    vm_b = vm_a;
    __syncthreads();
  };
  for (int j = 0; j < nblk; j += 2) {
    block(j, ga, gb);
    if (j + 1 < nblk) block(j + 1, gb, ga);
  }

  if (!active || h >= H) return;
  const float lt = pair_sum(lsum);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* orow;
  if (nsplit == 1) {
    orow = out + ((size_t)rowq * H + h) * D;
  } else {
    orow = part_o + ((size_t)unit * H + h) * D;
    if (lane < 32) {
      part_ml[((size_t)unit * H + h) * 2 + 0] = m_used;
      part_ml[((size_t)unit * H + h) * 2 + 1] = lt;
    }
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * (lane >> 5);
      u32x2 pk;
      pk.x = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      pk.y = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d0) = pk;
    }
  }
}

// Combine the nsplit partial results of each (row, head): weights
// l_s * 2^(m_s - max m) over the slices, applied to the normalised partials.
// One workgroup per row: the weights go through LDS, the partial outputs are
// read 8 bf16 at a time.
__global__ __launch_bounds__(256)
void attn_merge_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
                       int H, int D, int nsplit, uint16_t* __restrict__ out) {
  __shared__ float wgt[kMaxAttnSplits * 64];
  __shared__ float inv[64];
  const int row = blockIdx.x;
  const size_t u0 = (size_t)row * nsplit;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float mmax = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mmax = fmaxf(mmax, part_ml[((u0 + s) * H + h) * 2]);
    float wsum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = part_ml[((u0 + s) * H + h) * 2];
      const float ls = part_ml[((u0 + s) * H + h) * 2 + 1];
      const float wv = (ms == -INFINITY || ls <= 0.0f) ? 0.0f : ls * exp2f(ms - mmax);
      wgt[s * 64 + h] = wv;
      wsum += wv;
    }
    inv[h] = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  }
  __syncthreads();
  const int nvec = H * D / 8;
  for (int e8 = threadIdx.x; e8 < nvec; e8 += blockDim.x) {
    const int h = (e8 * 8) / D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float wv = wgt[s * 64 + h];
      const u32x4 v = *reinterpret_cast<const u32x4*>(part_o + (u0 + s) * H * D + (size_t)e8 * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += wv * __uint_as_float(v[j] << 16);
        acc[2 * j + 1] += wv * __uint_as_float(v[j] & 0xFFFF0000u);
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = (uint32_t)f32_to_bf16(acc[2 * j] * inv[h]) |
             ((uint32_t)f32_to_bf16(acc[2 * j + 1] * inv[h]) << 16);
    }
    *reinterpret_cast<u32x4*>(out + (size_t)row * H * D + (size_t)e8 * 8) = o;
  }
}

template <int D, int HB>
hipError_t launch(const AttnArgs& a, int nsplit, hipStream_t st) {
  constexpr int UPW = kAttnWaves / HB;
  const long long units = (long long)a.B * a.Lq * nsplit;
  const unsigned grid = (unsigned)((units + UPW - 1) / UPW);
  const size_t shmem = (size_t)UPW * 2 * unit_lds_bytes<D>();
  const float sl2 = a.scale * 1.4426950408889634f;
  uint16_t* po = nsplit > 1 ? reinterpret_cast<uint16_t*>(a.workspace) : nullptr;
  float* pml = nsplit > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) +
                                                    attn_part_o_bytes(a.B, a.Lq, a.H, a.D, nsplit))
                          : nullptr;
  hipLaunchKernelGGL((sparse_attn_kernel<D, HB>), dim3(grid), dim3(kAttnWaves * kWave), shmem, st,
                     a.q, a.key, a.val, a.indices, a.B, a.Lq, a.Lk, a.H, a.topk, nsplit, sl2,
                     a.out, po, pml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(a.B * a.Lq)), dim3(256), 0, st, po, pml,
                     a.H, a.D, nsplit, a.out);
  return hipGetLastError();
}

}  // namespace

size_t attn_part_o_bytes(int B, int Lq, int H, int D, int nsplit) {
  const size_t units = (size_t)B * Lq * nsplit;
  return (units * H * D * 2 + 255) / 256 * 256;
}

int attn_splits(int B, int Lq, int k) {
  // Enough units to fill the chip (about 1024), at least 128 keys each.
  const long long rows = (long long)B * Lq;
  int ns = 1;
  while (rows * ns < 1024 && ns * 2 * 128 <= k && ns < kMaxAttnSplits) ns *= 2;
  return ns;
}

size_t attn_workspace_bytes(int B, int Lq, int H, int D, int k) {
  const int ns = attn_splits(B, Lq, k);
  if (ns == 1) return 0;
  const size_t units = (size_t)B * Lq * ns;
  return attn_part_o_bytes(B, Lq, H, D, ns) + units * H * 2 * 4;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  const int ns = a.workspace ? attn_splits(a.B, a.Lq, a.topk) : 1;
  const int hb = (a.H + 31) / 32;
  if (a.D == 64) return hb == 1 ? launch<64, 1>(a, ns, st) : launch<64, 2>(a, ns, st);
  return hb == 1 ? launch<128, 1>(a, ns, st) : launch<128, 2>(a, ns, st);
}

}  // namespace idxc
