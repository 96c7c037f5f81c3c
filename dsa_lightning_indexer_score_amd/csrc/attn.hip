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
// heads of the query. The waves split each block's gather (whole rows, 16
// bytes per lane), two blocks ahead in registers. Scores are computed
// transposed, S^T = K_sel . Q^T, on 32x32x16 MFMAs: a lane holds 16 keys of
// one head, so the online-softmax max/sum stays in registers apart from one
// lane-half swap, and rescaling the output accumulators (O^T, heads on N) is
// a per-lane multiply. The running maximum is only moved (and the
// accumulators rescaled) when a block raises it by more than 2^8 in the exp2
// domain, which keeps every P below 256. V rows stay row-major in LDS; the
// P.V MFMA takes its V^T operand through transposing LDS reads.
//
// A unit covering only a slice of the list writes a partial result (bf16
// output normalised by its own sum, plus that sum and the max); a second
// kernel combines the slices of each row.
//
// For the stack's own caches (valid entries first, min(k, t+1) of them) the
// blocks past a row's valid entries are skipped. Workgroups are dealt to the
// XCDs in chunks of consecutive rows, every XCD taking chunks from the whole
// range.
#include "common.hpp"
#include "kernels.hpp"

namespace idxc {

namespace {

constexpr int kAttnWaves = 4;
constexpr float kLazyLog2 = 8.0f;   // rescale threshold (exp2 domain)
constexpr int kMaxAttnSplits = 32;
constexpr int kXcdChunk = 64;  // consecutive workgroups an XCD takes at a time

// One gathered 32-key block in LDS: whole K rows SK bytes apart, then whole V
// rows SV bytes apart. The padding spreads the MFMA operand reads over the
// banks: the K reads take 16 rows at one column (rows 16 bytes apart modulo
// 256), the transposed V reads take 4 consecutive rows at one 64-byte column
// range (rows 64 bytes apart modulo 256).
// A gather instruction moves KPI whole rows (16 bytes per lane, NCH lanes per
// row); lane l gathers rows (l / NCH) * NI + r of the block. The block's 32
// indices are loaded once (one per lane) and spread with lane shuffles.
template <int D>
struct Blk {
  static constexpr int NCH = D / 8;
  static constexpr int KPI = kWave / NCH;
  static constexpr int NI = 32 / KPI;
  static constexpr int SK = 2 * D + 16;
  static constexpr int SV = 2 * D + 64;
  static constexpr int KB = 32 * SK;
  static constexpr int BYTES = 32 * SK + 32 * SV;
};

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 4 bf16 addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  auto lp = (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

// Online softmax of one 32-key block in the exp2 domain with a lazily moved
// maximum, then O^T += V^T . P^T with V^T read through transposing LDS reads
// of the block's V rows at vl. s holds this lane's 16 raw scores (keys
// acc_row(i, lane) of the block, one head), vmask the block's valid keys. The
// scale (> 0) commutes with the maximum, so the raw scores' maximum is scaled
// once and each exponent is one fma, s * sl2 - m.
template <int D>
__device__ __forceinline__ void attend_block(const f32x16& s, uint32_t vmask, const uint8_t* vl,
                                             int vt_lane, float sl2, float& m_used, float& lsum,
                                             f32x16 (&o)[D / 32]) {
  using BL = Blk<D>;
  constexpr int DB = D / 32;
  const int lane = lane_id();
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = s[i];
  if (__builtin_expect(vmask != 0xFFFFFFFFu, 0)) {  // wave-uniform: padded entries
    // key of x[i] = acc_row(i, lane) = 4(l/32) + 8(i/4) + i%4
    const uint32_t vml = vmask >> (4 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!((vml >> (8 * (i >> 2) + (i & 3))) & 1u)) x[i] = -INFINITY;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
  const float mblk = pair_max(mloc) * sl2;
  const bool move = mblk > m_used + kLazyLog2;
  if (ballot(move)) {
    const float mnew = move ? mblk : m_used;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_used - mnew) : 1.0f;  // 2^-inf = 0
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    m_used = mnew;
  }
  // x * sl2 - m_used <= 8 keeps P <= 256; -inf maps to 0. The row sum
  // accumulates the bf16-rounded weights that the P.V product uses
  // (two-way dot products with 1), in two chains.
  const float mu = (m_used == -INFINITY) ? 0.0f : m_used;
  u32x4 pw[2];
  float psum0 = 0.0f, psum1 = 0.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(x[i], sl2, -mu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(x[i + 1], sl2, -mu));
    const uint32_t pk = pack_bf16x2(p0, p1);
    pw[i >> 3][(i & 7) >> 1] = pk;
    const bf16x2 pb2 = __builtin_bit_cast(bf16x2, pk);
    if (i & 2) psum1 = __builtin_amdgcn_fdot2_f32_bf16(pb2, ones, psum1, false);
    else psum0 = __builtin_amdgcn_fdot2_f32_bf16(pb2, ones, psum0, false);
  }
  lsum += psum0 + psum1;
  // ---- O^T += V^T . P^T; P^T's k index 8(l/32) + jj is key
  // 16kk + 8(jj/4) + 4(l/32) + jj%4, which the transposed reads match
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[kk]);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint8_t* p0 = vl + vt_lane + 16 * kk * BL::SV + 64 * db;
      const u32x2 lo = lds_read_tr16(p0);
      const u32x2 hi = lds_read_tr16(p0 + 8 * BL::SV);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      o[db] = mfma32(va, pb, o[db]);
    }
  }
}

template <int D, int HB>
__global__ __launch_bounds__(kAttnWaves * kWave, (D == 128 && HB == 1) ? 1 : 2)
void sparse_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kmat,
                        const uint16_t* __restrict__ vmat, const int32_t* __restrict__ indices,
                        int B, int Lq, int Lk, int H, int k, int nsplit, float sl2,
                        uint16_t* __restrict__ out, uint16_t* __restrict__ part_o,
                        float* __restrict__ part_ml, int prefix_lists, int q_pos0,
                        const int32_t* __restrict__ q_pos) {
  using BL = Blk<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int UPW = kAttnWaves / HB;  // units per workgroup
  constexpr int NRW = BL::NI / HB;      // gather instructions per wave and matrix
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  const int ul = wave / HB;  // unit slot in this workgroup
  const int hb = wave % HB;
  const int rows = B * Lq;
  // Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
  // b % 8). Renumber them so that each XCD takes chunks of kXcdChunk
  // consecutive workgroups (neighbouring rows: its L2 sees their index lists
  // and gathers together), the chunks dealt to the XCDs in turn, so that
  // every XCD gets an equal share of short rows (padding blocks skipped).
  // A bijection: the first nwg rounded down to 8 chunks go chunk-wise, the
  // rest keep their number; grids of fewer than 8 chunks give each XCD one
  // contiguous range (XCD x holds nwg/8, +1 for x < nwg % 8).
  const int nwg = (int)gridDim.x;
  const int xcd = (int)(blockIdx.x % 8);
  const int pos = (int)(blockIdx.x / 8);  // order within the XCD
  int wg;
  if (nwg < 8 * kXcdChunk) {
    wg = xcd * (nwg / 8) + min(xcd, nwg % 8) + pos;
  } else if ((int)blockIdx.x < nwg / (8 * kXcdChunk) * (8 * kXcdChunk)) {
    wg = ((pos / kXcdChunk) * 8 + xcd) * kXcdChunk + pos % kXcdChunk;
  } else {
    wg = (int)blockIdx.x;
  }
  const int unit = wg * UPW + ul;
  const int rowq = unit / nsplit;
  const int split = unit % nsplit;
  const bool active = rowq < rows;
  const int per = ((k + nsplit * 32 - 1) / (nsplit * 32)) * 32;  // keys per split
  const int kbeg = min(k, split * per);
  const int kend = min(k, kbeg + per);
  const int nblk = per / 32;  // same for every unit: keeps the barriers aligned
  // Blocks the workgroup runs: all nblk, or, for prefix-valid lists, up to
  // the last block holding a valid entry of any of its units (every wave
  // computes the same count, so the barriers stay aligned).
  int nrun = nblk;
  if (prefix_lists) {
    nrun = 0;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int uu = wg * UPW + u;
      const int rq = uu / nsplit;
      if (rq >= rows) continue;
      int t = q_pos0 + rq % Lq;
      if (q_pos != nullptr) {
        const int p = q_pos[rq];
        t = p < 0 ? -1 : min(p, Lk - 1);
      }
      const int b0 = min(k, (uu % nsplit) * per);
      const int e = min(min(k, b0 + per), min(k, t + 1));
      nrun = max(nrun, e > b0 ? (e - b0 + 31) / 32 : 0);
    }
  }
  const int b = active ? rowq / Lq : 0;
  const uint16_t* kb = kmat + (size_t)b * Lk * D;
  const uint16_t* vb = vmat + (size_t)b * Lk * D;
  const int32_t* irow = indices + (size_t)(active ? rowq : 0) * k;

  // the row's index list through a buffer resource (a 32-bit offset, no
  // 64-bit address registers): every load is issued unconditionally, at
  // entry 0 when it lies outside the unit's slice
  const __amdgpu_buffer_rsrc_t irsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(irow), (short)0, k * 4, 0x00020000);
  auto raw_index = [&](int j) {
    const int e = kbeg + j * 32 + (lane & 31);
    const bool in = active && j < nblk && e < kend;
    const int v = __builtin_amdgcn_raw_buffer_load_b32(irsrc, (in ? e : 0) * 4, 0, 0);
    return in ? v : -1;
  };
  // the first blocks' index loads go out before the Q loads: loads complete
  // in issue order, so the gathers that wait on the indices do not also wait
  // for Q
  const int rx0 = raw_index(0), rx1 = raw_index(1), rx2 = raw_index(2), rx3 = raw_index(3),
            rx4 = raw_index(4);
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

  // The waves of a unit split the gather: wave hb moves rows r0 .. r0+NRW-1
  // of every row group, K and V alike.
  const int gkey0 = (lane / BL::NCH) * BL::NI + (HB == 1 ? 0 : hb * NRW);
  const int gch = lane % BL::NCH;
  // rows to gather, from the resolved index of key (lane % 32) (lanes l and
  // l + 32 hold the same key)
  // (32-bit byte offsets from the batch's K and V bases: Lk <= 2^24 keeps
  // them below 2^32)
  const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(kb);
  const uint8_t* vb8 = reinterpret_cast<const uint8_t*>(vb);
  struct Off {
    uint32_t o[NRW];
  };
  struct Rows {
    u32x4 r[NRW];
  };
  auto offsets = [&](int row_of_lane) {
    Off f;
#pragma unroll
    for (int r = 0; r < NRW; ++r)
      f.o[r] = (uint32_t)__shfl(row_of_lane, gkey0 + r, kWave) * (uint32_t)(2 * D) +
               (uint32_t)gch * 16u;
    return f;
  };
  auto gather = [&](const uint8_t* src, const Off& f, Rows& g) {
#pragma unroll
    for (int r = 0; r < NRW; ++r) g.r[r] = *reinterpret_cast<const u32x4*>(src + f.o[r]);
  };
  uint8_t* base = dyn + ul * 2 * BL::BYTES;
  auto kbuf = [&](int b) { return base + (b & 1) * BL::BYTES; };
  auto vbuf = [&](int b) { return base + (b & 1) * BL::BYTES + BL::KB; };
  auto stage_k = [&](const Rows& g, int b) {
#pragma unroll
    for (int r = 0; r < NRW; ++r)
      *reinterpret_cast<u32x4*>(kbuf(b) + (gkey0 + r) * BL::SK + gch * 16) = g.r[r];
  };
  auto stage_v = [&](const Rows& g, int b) {
#pragma unroll
    for (int r = 0; r < NRW; ++r)
      *reinterpret_cast<u32x4*>(vbuf(b) + (gkey0 + r) * BL::SV + gch * 16) = g.r[r];
  };
  // index of key (lane % 32) of block j; invalid entries gather row 0 and are
  // masked out of the softmax
  auto resolve = [&](int idx, uint32_t* vmask) {
    const bool valid = idx >= 0 && idx < Lk;
    *vmask = (uint32_t)(ballot(valid) & 0xFFFFFFFFull);
    return valid ? idx : 0;
  };
  // S^T = K . Q^T for this wave's 32 heads, K rows of LDS buffer b
  auto qk = [&](int b) {
    const uint8_t* kl = kbuf(b);
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + (lane & 31) * BL::SK +
                                                         (ks * 2 + (lane >> 5)) * 16);
      s = mfma32(ka, qb[ks], s);
    }
    // keep four K reads in flight ahead of the MFMA chain (the default
    // schedule waits on each pair of reads): four reads, then MFMA and read
    // alternating, then the last four MFMAs (1-2% faster per prefill layer)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 0x100: LDS reads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    return s;
  };

  // V^T operand rows for this lane: key 16kk + 8t + 4(l/32) + (l%16)/4 at
  // column 64db + 32((l/16)%2) + 8(l%4) bytes (t selects operand half)
  const int vt_lane = (4 * (lane >> 5) + ((lane & 15) >> 2)) * BL::SV + 32 * ((lane >> 4) & 1) +
                      8 * (lane & 3);

  // Pipeline. K runs one block ahead of V: at the start of iteration j the K
  // rows of block j+1 and the V rows of block j are in LDS, and S(j) is
  // already computed. Iteration j issues the gathers of K(j+3) and V(j+2),
  // computes S(j+1) (MFMAs independent of block j's softmax), finishes block
  // j (softmax, O^T += V^T . P^T), then stages K(j+2) over K(j) and V(j+1)
  // over V(j-1), both last read before the previous barrier. In flight in
  // registers: K(j+2), K(j+3), V(j+1), V(j+2).
  uint32_t vm0 = 0, vm1 = 0, vm2 = 0, vm3 = 0;  // masks of blocks j .. j+3
  Rows ka_, kb_, va_, vb_;  // alternate register sets: (kb_, vb_) near, (ka_, va_) far
  Off off_prev;             // row offsets of the block whose K was issued last
  {
    const Off o0 = offsets(resolve(rx0, &vm0));
    const Off o1 = offsets(resolve(rx1, &vm1));
    off_prev = offsets(resolve(rx2, &vm2));
    gather(kb8, o0, ka_);
    gather(vb8, o0, va_);
    gather(kb8, o1, kb_);
    gather(vb8, o1, vb_);
    stage_k(ka_, 0);
    stage_v(va_, 0);
    stage_k(kb_, 1);
    gather(kb8, off_prev, kb_);  // K(2) in flight; vb_ holds V(1)
  }
  int ix3 = rx3, ix4 = rx4;
  __syncthreads();
  f32x16 s_cur = qk(0);
  // iteration 0 stages K(2) over K(0): every wave of the unit must have read
  // K(0) first
  __syncthreads();

  auto iteration = [&](int j, Rows& k_far, Rows& v_far, Rows& k_near, Rows& v_near) {
    // issued unconditionally (blocks past the end gather row 0, masked out):
    // a conditional load here would make the compiler drain every
    // outstanding load before the staging below
    const Off on = offsets(resolve(ix3, &vm3));
    ix3 = ix4;
    ix4 = raw_index(j + 5);
    gather(kb8, on, k_far);        // K(j+3)
    gather(vb8, off_prev, v_far);  // V(j+2)
    off_prev = on;
    // the two waves of a SIMD alternate between this MFMA run and softmax
    // work; raising the wave's priority for the run keeps the matrix pipe fed
    // (1.6-1.8% faster per prefill layer)
    __builtin_amdgcn_s_setprio(1);
    const f32x16 s_nxt = qk(j + 1);  // past the last block: masked rows
    __builtin_amdgcn_s_setprio(0);

    attend_block<D>(s_cur, vm0, vbuf(j), vt_lane, sl2, m_used, lsum, o);
    // ---- stage K(j+2) over K(j) and V(j+1) over V(j-1) (past the last
    // block: buffers nobody reads)
    stage_k(k_near, j);
    stage_v(v_near, j + 1);
    vm0 = vm1;
    vm1 = vm2;
    vm2 = vm3;
    s_cur = s_nxt;
    __syncthreads();
  };
  // Pairs of iterations, then a last single one: the loop's back edge
  // follows only the second of a pair, so the loads the first one issues are
  // never pending at the top of the loop (a path from the first straight
  // back to the top made the compiler wait there for them, a whole iteration
  // before they are staged).
  int j = 0;
  for (; j + 1 < nrun; j += 2) {
    iteration(j, ka_, va_, kb_, vb_);
    iteration(j + 1, kb_, vb_, ka_, va_);
  }
  if (j < nrun) iteration(j, ka_, va_, kb_, vb_);

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
// l_s * 2^(m_s - max m) over the slices, normalised, applied to the
// normalised partials. One workgroup per (row, group of kMergeHeads heads):
// 32 lanes per head compute its slice weights together (shuffle reductions),
// then each thread combines 4 consecutive outputs over the slices.
constexpr int kMergeHeads = 8;

__global__ __launch_bounds__(256)
void attn_merge_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
                       int H, int D, int nsplit, int hgroups, uint16_t* __restrict__ out) {
  __shared__ float wgt[kMergeHeads][kMaxAttnSplits];
  const int row = blockIdx.x / hgroups;
  const int hg = blockIdx.x % hgroups;
  const int tid = threadIdx.x;
  const size_t u0 = (size_t)row * nsplit;
  {
    const int hl = tid >> 5, sl = tid & 31;
    const int h = hg * kMergeHeads + hl;
    float m = -INFINITY, l = 0.0f;
    if (h < H && sl < nsplit) {
      m = part_ml[((u0 + sl) * H + h) * 2];
      l = part_ml[((u0 + sl) * H + h) * 2 + 1];
    }
    float mmax = m;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off, 32));
    const float wv = (m == -INFINITY || l <= 0.0f) ? 0.0f : l * exp2f(m - mmax);
    float wsum = wv;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off, 32);
    wgt[hl][sl] = wsum > 0.0f ? wv / wsum : 0.0f;
  }
  __syncthreads();
  const int e = tid * 4;  // 4 consecutive outputs of head hl
  const int hl = e / D;
  const int d = e % D;
  const int h = hg * kMergeHeads + hl;
  if (hl >= kMergeHeads || h >= H) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* src = part_o + (u0 * H + h) * D + d;
  const size_t stride = (size_t)H * D;  // next slice
#pragma unroll 4
  for (int s = 0; s < nsplit; ++s) {
    const float wv = wgt[hl][s];
    const u32x2 v = *reinterpret_cast<const u32x2*>(src + s * stride);
    acc[0] += wv * __uint_as_float(v[0] << 16);
    acc[1] += wv * __uint_as_float(v[0] & 0xFFFF0000u);
    acc[2] += wv * __uint_as_float(v[1] << 16);
    acc[3] += wv * __uint_as_float(v[1] & 0xFFFF0000u);
  }
  u32x2 o;
  o[0] = pack_bf16x2(acc[0], acc[1]);
  o[1] = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<u32x2*>(out + ((size_t)row * H + h) * D + d) = o;
}

template <int D, int HB>
hipError_t launch(const AttnArgs& a, int nsplit, hipStream_t st) {
  constexpr int UPW = kAttnWaves / HB;
  const long long units = (long long)a.B * a.Lq * nsplit;
  const unsigned grid = (unsigned)((units + UPW - 1) / UPW);
  const size_t shmem = (size_t)UPW * 2 * Blk<D>::BYTES;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_kernel<D, HB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  uint16_t* po = nsplit > 1 ? reinterpret_cast<uint16_t*>(a.workspace) : nullptr;
  float* pml = nsplit > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) +
                                                    attn_part_o_bytes(a.B, a.Lq, a.H, a.D, nsplit))
                          : nullptr;
  hipLaunchKernelGGL((sparse_attn_kernel<D, HB>), dim3(grid), dim3(kAttnWaves * kWave), shmem, st,
                     a.q, a.key, a.val, a.indices, a.B, a.Lq, a.Lk, a.H, a.topk, nsplit, sl2,
                     a.out, po, pml, a.prefix_lists, a.q_pos0, a.q_pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const int hgroups = (a.H + kMergeHeads - 1) / kMergeHeads;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(a.B * a.Lq * hgroups)), dim3(256), 0, st,
                     po, pml, a.H, a.D, nsplit, hgroups, a.out);
  return hipGetLastError();
}

}  // namespace

size_t attn_part_o_bytes(int B, int Lq, int H, int D, int nsplit) {
  const size_t units = (size_t)B * Lq * nsplit;
  return (units * H * D * 2 + 255) / 256 * 256;
}

int attn_splits(int B, int Lq, int k) {
  // About 512 units (two per CU: each runs a few key blocks, so fewer, longer
  // units pipeline better than filling every slot), at least 128 keys each.
  const long long rows = (long long)B * Lq;
  int ns = 1;
  while (rows * ns < 512 && ns * 2 * 128 <= k && ns < kMaxAttnSplits) ns *= 2;
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
