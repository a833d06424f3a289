// Exact attention forward on one rank's head group, full sequence.
//
// O = softmax(Q K^T / sqrt(d_h)) V per (batch, head), causal or not
// (papers.chlience.com reading note, section 5.1; paper-graph summary of
// arXiv 2309.14509, sections 3.2 and 3.4.5). The N x N score matrix is never
// formed in memory (paper-graph summary, section 3.4.5, on FlashAttention):
// each workgroup walks the key blocks of its query block with a running row
// maximum and row sum, and writes the log-sum-exp of every row for the
// backward pass.
//
// bf16 path (gfx950 MFMA, 32x32x16), key tiles of 64 rows:
//   each wave owns 32 query rows and computes S^T = K Q^T for them (keys down
//   the accumulator rows, queries across lanes), so a query's scores sit in
//   one lane pair and the row max / sum need one cross-lane exchange.
//   O^T = V^T P^T reuses the score registers as the B operand; V is read
//   transposed from its row-major LDS tile with ds_read_b64_tr_b16. Q stays
//   in registers for the whole key walk; the next K/V tile is loaded into
//   registers while the current one is used from LDS. Causal query blocks are
//   dispatched longest first and never visit key blocks above the diagonal.
//   Dense attention: 8 waves x 32 rows = 256 rows per workgroup in two groups
//   whose MFMA and softmax phases alternate (attn_fwd_bf16_kernel); launches
//   of only a few hundred query blocks instead split each 128-row block's key
//   walk between two wave groups and merge the halves through LDS, and the
//   smallest launches each 64-row block's walk between four
//   (attn_fwd_split_bf16_kernel). Block layouts: 4 waves x 32 rows = 128
//   rows, the layout's block, walking the active key blocks
//   (attn_fwd_sparse_bf16_kernel). The single-walk kernels compute every row
//   with the same sequence of operations, so a full layout gives their result
//   bit for bit.
// Grouped-query attention (pinyu.ai, section "Head-count constraints"): the
//   key/value buffers may hold fewer heads than the query buffer; query head h
//   reads key head h / G. Queries and keys may have different lengths
//   (cross-attention, papers.chlience.com note, section 5.4; bidirectional only).
// Block layouts (paper-graph summary, section 3.4 and Figs 6-7, "blocked
//   sparse attention"): the workgroup of a query block visits only the key
//   blocks its layout row marks, found with a 64-lane ballot over the row.
// fp32 path: the same shape on the fp32 MFMA (v_mfma_f32_32x32x2_f32), 4 waves
//   x 32 query rows, key tiles of 32 (attn_fwd_f32_kernel).
#include <math.h>

#include <type_traits>

#include "block_sparse.h"
#include "common.h"
#include "kernels.h"
#include "mfma_frag.h"

namespace ulysses {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kFwdXcdRun = 16;   // consecutive dense forward jobs per XCD (half of the 32 it holds at once)
constexpr float kLog2e = 1.44269504088896340736f;

// Block layouts: workgroup = 4 waves x 32 query rows, one 128-row query block;
// it walks the active key blocks of the block's layout row.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_sparse_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb,
    float sl2, const uint8_t* __restrict__ layout, int nb) {
  constexpr int BM = 128, BN = 64, KS = D / 16, DT = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;         // chunks per thread per tile
  constexpr int RSTEP = 256 / CPR;           // rows between a thread's chunks
  constexpr int KST = Stride<D>::row;        // K is read along rows (S^T = K Q^T)
  constexpr int VST = Stride<D>::col;        // V is read transposed (O^T += V^T P^T)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KST];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * VST];

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / nhb;  // longest rows first
  const int hb = bid % nhb;            // (batch, query head) pair
  const int b = hb / Hq, h = hb - b * Hq;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;   // row strides
  const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
  const size_t koff = ((size_t)b * Lk * Hk + h / G) * D;
  const __bf16* qh = q + qoff;
  const __bf16* kh = k + koff;
  const __bf16* vh = v + koff;
  const int q0 = qb * BM;
  const int qw0 = q0 + 32 * wave;      // first query row of this wave
  const int qrow = qw0 + l32;

  // Q^T as the B operand: lane holds Q[qrow][16 ks + 8 hl .. +7]
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < Lq)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * rsq + 16 * ks + 8 * hl);
    else
      qf[ks] = bf16x8{};
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  // running maximum in log2 units and this lane's share of the running sum
  float m_run = -INFINITY, l_run = 0.f;

  // staging: thread tid moves chunks of rows srow + j * RSTEP, columns scol .. scol+7,
  // through buffer loads (constant per-lane offset, scalar tile offset)
  const int srow = tid / CPR, scol = (tid % CPR) * 8;
  const uint32_t head_bytes = (uint32_t)((size_t)Lk * rsk * 2);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kh, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vh, head_bytes);
  uint32_t voff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) voff[j] = (uint32_t)(((srow + j * RSTEP) * rsk + scol) * 2);
  const uint32_t tile_bytes = (uint32_t)(BN * rsk * 2);
  u32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int kb) {
    const uint32_t soff = (uint32_t)kb * tile_bytes;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      kreg[j] = buf_load16(krs, voff[j] + soff, 0);
      vreg[j] = buf_load16(vrs, voff[j] + soff, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      *reinterpret_cast<u32x4*>(&Ks[buf][(srow + j * RSTEP) * KST + scol]) = kreg[j];
      *reinterpret_cast<u32x4*>(&Vs[buf][(srow + j * RSTEP) * VST + scol]) = vreg[j];
    }
  };

  // One key tile kb, held in LDS buffer cur; afterwards the tile in the
  // staging registers goes to the other buffer (if store) and key tile `next2`
  // is loaded into the registers (if >= 0). The mask applies only where the
  // tile crosses the diagonal or the end of the keys.
  auto tile = [&](int cur, int kb, bool store, int next2) {
    const __bf16* Kc = Ks[cur];
    const __bf16* Vc = Vs[cur];
    const int k0 = kb * BN;

    // S^T = K Q^T for the tile's two 32-key halves (independent MFMA chains)
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32(frag_row<KST>(Kc, 0, 16 * ks, lane), qf[ks], s0);
      s1 = mfma32(frag_row<KST>(Kc, 32, 16 * ks, lane), qf[ks], s1);
    }

    if (CAUSAL ? (k0 + BN - 1 > qw0) : (k0 + BN > Lk)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (CAUSAL ? (key > qrow) : (key >= Lk)) s0[e] = -INFINITY;
        if (CAUSAL ? (key + 32 > qrow) : (key + 32 >= Lk)) s1[e] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(fmaxf(mx, s0[e]), s1[e]);   // v_max3_f32
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * sl2;
    // The running maximum is raised only when some row's maximum grew by more
    // than 8 (log2 units): in between, probabilities stay below 2^8 and the
    // O accumulators need no rescaling. Normalisation at the end is exact.
    if (__ballot(mcand > m_run + 8.f)) {
      const float m2 = fmaxf(m_run, mcand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m2;
    }
    // (a block-sparse row may meet a fully masked tile before any visible key)
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
    float rsum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (c < 2) ? s0[8 * (c & 1) + i] : s1[8 * (c & 1) + i];
        const float p = __builtin_amdgcn_exp2f(fmaf(x, sl2, nm));
        rsum += p;
        pf[c][i] = (__bf16)p;
      }
    }
    l_run += rsum;

    // O^T += V^T P^T over four 16-key chunks
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32(frag_col<VST>(Vc, 16 * c, 32 * dt, lane), pf[c], oacc[dt]);
    }

    if (store) store_tile(cur ^ 1);
    if (next2 >= 0) load_tile(next2);
    __syncthreads();
  };
  {
    // The active key blocks j of this query block (ascending; causal: j <= qb),
    // two key tiles each: tile (j, half) sits in LDS buffer `half`. A second
    // tile past the end of the keys is fully masked (its loads read zeros).
    // Every tile takes the masked path, which masks only where a tile crosses
    // the diagonal or the end of the keys.
    LayoutScan scan;
    scan.reset(layout + ((size_t)h * nb + qb) * nb, 1, 0, CAUSAL ? qb + 1 : nb);
    int j = scan.next(lane);
    if (j >= 0) {
      int jn = scan.next(lane);
      load_tile(2 * j);
      store_tile(0);
      __syncthreads();
      load_tile(2 * j + 1);
      int half = 0;
      while (j >= 0) {
        // next tile: (j, 1) or (jn, 0); the one after: (jn, half)
        tile(half, 2 * j + half, half == 0 || jn >= 0, jn >= 0 ? 2 * jn + half : -1);
        if (half == 1) {
          j = jn;
          if (j >= 0) jn = scan.next(lane);
        }
        half ^= 1;
      }
    }
  }

  // a row that sees no key (possible only under a block layout) has zero output and LSE -inf
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Lq) {
    __bf16* orow = o + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * hl) = acc_quad_bf16(oacc[dt], a, inv);
    }
    if (hl == 0) lse[(size_t)hb * Lq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Dense bf16 forward for grids too small to fill the chip: a workgroup of 8
// waves owns 128 query rows and splits their key walk in two. Waves w and
// w + 4 own the same 32 rows; group 0 (waves 0-3) takes the first half of the
// key tiles, group 1 (waves 4-7) the second half, each through its own
// double-buffered K/V tiles in LDS, and at the end group 0 folds group 1's
// running maximum, sum and O accumulators into its own through LDS. The
// longest query block's chain of key tiles is half as long as in the
// single-walk kernels, which is what bounds a causal launch of a few hundred
// query blocks. NGRP = 4 (launches of very few blocks): four groups
// of two waves share a 64-row block, each over a quarter of its key tiles of
// 32 keys, in the same LDS (their double-buffered tiles are half as long);
// group 0 folds in groups 1-3 in order.
template <int D, bool CAUSAL, int NGRP = 2>
__global__ __launch_bounds__(512, 1) void attn_fwd_split_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb,
    float sl2) {
  static_assert(NGRP == 2 || NGRP == 4, "two or four wave groups");
  constexpr int WPG = 8 / NGRP, GT = 64 * WPG;   // waves and threads per group
  constexpr int BM = 32 * WPG, BN = NGRP == 2 ? 64 : 32, KS = D / 16, DT = D / 32, NC = BN / 16;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CH = BN * CPR / GT;          // chunks per thread of its group's tile
  constexpr int RSTEP = GT / CPR;            // rows between a thread's chunks
  constexpr int KST = Stride<D>::row;
  constexpr int VST = Stride<D>::col;
  constexpr int KBYTES = NGRP * 2 * BN * KST * 2, VBYTES = NGRP * 2 * BN * VST * 2;
  // [group][buffer] K and V tiles; reused for the merge once the walks are done
  __shared__ __attribute__((aligned(16))) char smem[KBYTES + VBYTES];
  typedef __bf16 KTile[BN * KST];
  typedef __bf16 VTile[BN * VST];
  KTile* Ks = reinterpret_cast<KTile*>(smem);
  VTile* Vs = reinterpret_cast<VTile*>(smem + KBYTES);
  // merge record of one wave of group 1: DT * 16 O values, the running
  // maximum and the partial sum, each as [value][lane]
  constexpr int MREC = (DT * 16 + 2) * 64;
  static_assert((NGRP - 1) * WPG * MREC * 4 <= KBYTES + VBYTES, "merge records exceed the tile buffers");
  float* mbuf = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / WPG, wq = wave % WPG;
  const int gtid = tid % GT;                 // thread index within the group
  // jobs (query block, head pair), longest rows first, in runs of 16 per
  // XCD as in the ping-pong kernel
  int rank, hb;
  if (!xcd_run_block((int)blockIdx.x, kFwdXcdRun, nhb, nqb, &rank, &hb)) return;   // grid rounded up
  const int qb = nqb - 1 - rank;
  const int b = hb / Hq, h = hb - b * Hq;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;
  const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
  const size_t koff = ((size_t)b * Lk * Hk + h / G) * D;
  const __bf16* qh = q + qoff;
  const int q0 = qb * BM;
  const int qw0 = q0 + 32 * wq;
  const int qrow = qw0 + l32;

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < Lq)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * rsq + 16 * ks + 8 * hl);
    else
      qf[ks] = bf16x8{};
  }
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // key tiles [0, n): group 0 walks [0, n / 2), group 1 [n / 2, n) -- the
  // diagonal tiles under the causal mask, and one tile more when n is odd
  const int kend = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int n = (kend + BN - 1) / BN;
  const int t0 = grp * n / NGRP;
  const int cnt = (grp + 1) * n / NGRP - t0;
  const int steps = (n + NGRP - 1) / NGRP;   // every group passes this many barriers

  const int srow = gtid / CPR, scol = (gtid % CPR) * 8;
  const uint32_t head_bytes = (uint32_t)((size_t)Lk * rsk * 2);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(k + koff, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(v + koff, head_bytes);
  uint32_t voff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) voff[j] = (uint32_t)(((srow + j * RSTEP) * rsk + scol) * 2);
  const uint32_t tile_bytes = (uint32_t)(BN * rsk * 2);
  u32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int kb) {
    const uint32_t soff = (uint32_t)kb * tile_bytes;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      kreg[j] = buf_load16(krs, voff[j] + soff, 0);
      vreg[j] = buf_load16(vrs, voff[j] + soff, 0);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* kt = Ks[2 * grp + buf];
    __bf16* vt = Vs[2 * grp + buf];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      *reinterpret_cast<u32x4*>(&kt[(srow + j * RSTEP) * KST + scol]) = kreg[j];
      *reinterpret_cast<u32x4*>(&vt[(srow + j * RSTEP) * VST + scol]) = vreg[j];
    }
  };

  // one key tile of this group, as in the four-wave kernel
  auto tile = [&](int cur, int kb, bool store, int next2) {
    const __bf16* Kc = Ks[2 * grp + cur];
    const __bf16* Vc = Vs[2 * grp + cur];
    const int k0 = kb * BN;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32(frag_row<KST>(Kc, 0, 16 * ks, lane), qf[ks], s0);
      if constexpr (BN == 64) s1 = mfma32(frag_row<KST>(Kc, 32, 16 * ks, lane), qf[ks], s1);
    }
    if (CAUSAL ? (k0 + BN - 1 > qw0) : (k0 + BN > Lk)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (CAUSAL ? (key > qrow) : (key >= Lk)) s0[e] = -INFINITY;
        if (BN == 64 && (CAUSAL ? (key + 32 > qrow) : (key + 32 >= Lk))) s1[e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; e += 2)   // three-operand maxima (v_max3_f32)
      mx = BN == 64 ? fmaxf(fmaxf(fmaxf(mx, s0[e]), s1[e]), fmaxf(s0[e + 1], s1[e + 1]))
                    : fmaxf(fmaxf(mx, s0[e]), s0[e + 1]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * sl2;
    if (__ballot(mcand > m_run + 8.f)) {
      const float m2 = fmaxf(m_run, mcand);
      // (a lane whose rows have seen only masked keys keeps its empty state)
      const float alpha = m2 == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m2;
    }
    // group 1's rows of the first query tiles meet only masked keys in a
    // diagonal tile before any visible one
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
    float rsum = 0.f;
    bf16x8 pf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (c < 2) ? s0[8 * (c & 1) + i] : s1[8 * (c & 1) + i];
        const float p = __builtin_amdgcn_exp2f(fmaf(x, sl2, nm));
        rsum += p;
        pf[c][i] = (__bf16)p;
      }
    }
    l_run += rsum;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32(frag_col<VST>(Vc, 16 * c, 32 * dt, lane), pf[c], oacc[dt]);
    }
    if (store) store_tile(cur ^ 1);
    if (next2 >= 0) load_tile(next2);
    __syncthreads();
  };

  if (cnt > 0) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();
  if (cnt > 1) load_tile(t0 + 1);
  for (int st = 0; st < steps; ++st) {
    if (st < cnt)
      tile(st & 1, t0 + st, st + 1 < cnt, st + 2 < cnt ? t0 + st + 2 : -1);
    else
      __syncthreads();   // group 0's idle step when n is odd
  }

  // every tile read ended at the last barrier: group 1 leaves its state in
  // the tile buffers, group 0 folds it into its own
  if (grp > 0) {
    float* rec = mbuf + ((grp - 1) * WPG + wq) * MREC;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) rec[(dt * 16 + e) * 64 + lane] = oacc[dt][e];
    }
    rec[DT * 16 * 64 + lane] = m_run;
    rec[(DT * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp > 0) return;
  // group 0 folds in groups 1 .. NGRP-1 in order
  for (int g = 1; g < NGRP; ++g) {
    const float* rec = mbuf + ((g - 1) * WPG + wq) * MREC;
    const float m1 = rec[DT * 16 * 64 + lane];
    const float l1 = rec[(DT * 16 + 1) * 64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] = oacc[dt][e] * a0 + rec[(dt * 16 + e) * 64 + lane] * a1;
    }
    l_run = l_run * a0 + l1 * a1;
    m_run = m;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Lq) {
    __bf16* orow = o + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * hl) = acc_quad_bf16(oacc[dt], a, inv);
    }
    if (hl == 0) lse[(size_t)hb * Lq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Dense bf16 forward as a ping-pong of two wave groups. A workgroup has 8
// waves and 256 query rows: group A = waves 0-3, group B = waves 4-7; wave
// (group g, index w) owns rows q0 + 64 w + 32 g .. +31, so both groups span
// the block alike. With the usual in-order placement each SIMD hosts one wave
// of each group. The groups alternate phases separated by barriers: while one
// runs its MFMA phase for key tile k (O^T += V^T P^T of tile k, then the
// scores of tile k+1), the other runs its softmax phase (mask, row max,
// exponentials, row sums, P to bf16) and stages the next tile, so every SIMD
// has MFMA work from one wave and VALU work from the other at all times.
// Group A stages K tiles (K(k+1) during its softmax of tile k), group B stages
// V tiles (V(k+1) during its softmax of tile k); each LDS buffer is free by
// the time it is written (K(k+1) replaces K(k-1), last read by B's scores of
// tile k-1 one phase earlier; likewise for V).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb,
    float sl2) {
  constexpr int BM = 256, BN = 64, KS = D / 16, DT = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CH = BN * CPR / 256;         // chunks per thread of its group's tile
  constexpr int RSTEP = 256 / CPR;           // rows between a thread's chunks
  constexpr int KST = Stride<D>::row;
  constexpr int VST = Stride<D>::col;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KST];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * VST];

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool groupA = wave < 4;
  const int gtid = tid & 255;                // thread index within the group
  // jobs (query block, head pair), longest rows first, in runs of 16 per XCD
  // (an XCD holds 32 workgroups, one per CU, so two runs at once): the blocks
  // of a run walk the same key tiles a few steps apart and share them
  // through the XCD's L2; runs of 16 measured 0.3-0.9 % faster than 32
  int rank, hb;
  if (!xcd_run_block((int)blockIdx.x, kFwdXcdRun, nhb, nqb, &rank, &hb)) return;   // grid rounded up
  const int qb = nqb - 1 - rank;             // longest rows first
  const int b = hb / Hq, h = hb - b * Hq;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;
  const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
  const size_t koff = ((size_t)b * Lk * Hk + h / G) * D;
  const __bf16* qh = q + qoff;
  const int q0 = qb * BM;
  const int qw0 = q0 + 64 * (wave & 3) + 32 * (wave >> 2);
  const int qrow = qw0 + l32;

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (qrow < Lq)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qrow * rsq + 16 * ks + 8 * hl);
    else
      qf[ks] = bf16x8{};
  }
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int n = (kend + BN - 1) / BN;
  // causal: the last BM / BN key tiles reach above some row of the block;
  // otherwise only a ragged last tile holds keys past the end
  const int nsteady = CAUSAL ? max(0, n - BM / BN) : (Lk % BN ? n - 1 : n);

  // staging: group A moves K tiles, group B V tiles; thread gtid handles
  // chunks of rows srow + j * RSTEP, columns scol .. scol + 7
  const int srow = gtid / CPR, scol = (gtid % CPR) * 8;
  const uint32_t head_bytes = (uint32_t)((size_t)Lk * rsk * 2);
  const __amdgpu_buffer_rsrc_t rsrc = head_rsrc((groupA ? k : v) + koff, head_bytes);
  uint32_t voff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) voff[j] = (uint32_t)(((srow + j * RSTEP) * rsk + scol) * 2);
  const uint32_t tile_bytes = (uint32_t)(BN * rsk * 2);
  u32x4 sreg[CH];
  auto load = [&](int kb) {
    const uint32_t soff = (uint32_t)kb * tile_bytes;
#pragma unroll
    for (int j = 0; j < CH; ++j) sreg[j] = buf_load16(rsrc, voff[j] + soff, 0);
  };
  auto store = [&](int buf) {
    __bf16* t = groupA ? Ks[buf] : Vs[buf];
    const int st = groupA ? KST : VST;
#pragma unroll
    for (int j = 0; j < CH; ++j) *reinterpret_cast<u32x4*>(&t[(srow + j * RSTEP) * st + scol]) = sreg[j];
  };

  f32x16 s0, s1;        // scores of the current tile
  bf16x8 pf[4];         // its probabilities as MFMA operands
  auto scores = [&](int kb) {
    const __bf16* Kc = Ks[kb & 1];
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32(frag_row<KST>(Kc, 0, 16 * ks, lane), qf[ks], s0);
      s1 = mfma32(frag_row<KST>(Kc, 32, 16 * ks, lane), qf[ks], s1);
    }
  };
  auto pv = [&](int kb) {
    const __bf16* Vc = Vs[kb & 1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32(frag_col<VST>(Vc, 16 * c, 32 * dt, lane), pf[c], oacc[dt]);
    }
  };
  auto softmax = [&](int kb) {
    const int k0 = kb * BN;
    if (kb >= nsteady && (CAUSAL ? (k0 + BN - 1 > qw0) : (k0 + BN > Lk))) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (CAUSAL ? (key > qrow) : (key >= Lk)) s0[e] = -INFINITY;
        if (CAUSAL ? (key + 32 > qrow) : (key + 32 >= Lk)) s1[e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(fmaxf(mx, s0[e]), s1[e]);   // v_max3_f32
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mcand = mx * sl2;
    // lazy rescale, as in the four-wave kernel
    if (__ballot(mcand > m_run + 8.f)) {
      const float m2 = fmaxf(m_run, mcand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m2;
    }
    const float nm = -m_run;
    float rsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (c < 2) ? s0[8 * (c & 1) + i] : s1[8 * (c & 1) + i];
        const float p = __builtin_amdgcn_exp2f(fmaf(x, sl2, nm));
        rsum += p;
        pf[c][i] = (__bf16)p;
      }
    }
    l_run += rsum;
  };

  // prologue: K(0) and V(0) into LDS, K(1) / V(1) in flight; group A forms
  // the scores of tile 0 while group B waits
  load(0);
  store(0);
  if (n > 1) load(1);
  __syncthreads();
  if (groupA) scores(0);
  __syncthreads();

  if (groupA) {
    for (int kb = 0; kb < n; ++kb) {
      softmax(kb);
      if (kb + 1 < n) store((kb + 1) & 1);   // K(kb+1)
      if (kb + 2 < n) load(kb + 2);
      __syncthreads();
      pv(kb);
      if (kb + 1 < n) scores(kb + 1);
      __syncthreads();
    }
  } else {
    for (int kb = 0; kb < n; ++kb) {
      if (kb >= 1) pv(kb - 1);
      scores(kb);
      __syncthreads();
      softmax(kb);
      if (kb + 1 < n) store((kb + 1) & 1);   // V(kb+1)
      if (kb + 2 < n) load(kb + 2);
      __syncthreads();
    }
    pv(n - 1);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < Lq) {
    __bf16* orow = o + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * hl) = acc_quad_bf16(oacc[dt], a, inv);
    }
    if (hl == 0) lse[(size_t)hb * Lq + qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp32 on the fp32 MFMA: workgroup = 4 waves x 32 query rows, key tiles of
// 32 in LDS. Each wave forms S^T = K Q^T (keys down the accumulator rows,
// queries across lanes; Q^T in registers) and O^T += V^T P^T with the score
// registers as the B operand, as the bf16 kernels do, with a running row
// maximum and sum.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb,
    float sl2) {
  constexpr int BN = 32, ST = StrideF32<D>::row, KS = D / 2, DT = D / 32, C4 = D / 4;
  __shared__ __attribute__((aligned(16))) float Ks[BN * ST];
  __shared__ __attribute__((aligned(16))) float Vs[BN * ST];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = nqb - 1 - (int)blockIdx.x / nhb;   // longest rows first
  const int hb = blockIdx.x % nhb;
  const int b = hb / Hq, h = hb - b * Hq;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;
  const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
  const size_t koff = ((size_t)b * Lk * Hk + h / G) * D;
  const int q0 = qb * 128, qw0 = q0 + 32 * wave, qrow = qw0 + l32;

  // Q^T as the B operand: step t holds Q[qrow][2t + hl]
  float qf[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) qf[t] = qrow < Lq ? q[qoff + (size_t)qrow * rsq + 2 * t + hl] : 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  // running maximum in log2 units and this lane's share of the running sum
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(Lk, q0 + 128) : Lk;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * C4; c += 256) {
      const int r = c / C4, e = (c - r * C4) * 4, key = k0 + r;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (key < Lk) {
        kv = *reinterpret_cast<const f32x4*>(k + koff + (size_t)key * rsk + e);
        vv = *reinterpret_cast<const f32x4*>(v + koff + (size_t)key * rsk + e);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Ks[r * ST + e + i] = kv[i];
        Vs[r * ST + e + i] = vv[i];
      }
    }
    __syncthreads();
    if (CAUSAL && k0 > qw0 + 31) continue;   // every key of the tile above this wave's rows
    f32x16 sc = f32x16{};
#pragma unroll
    for (int t = 0; t < KS; ++t) sc = mfma32_f32(Ks[l32 * ST + 2 * t + hl], qf[t], sc);
    if (CAUSAL ? (k0 + BN - 1 > qw0) : (k0 + BN > Lk)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kslot_row(e, lane);
        if ((CAUSAL && key > qrow) || key >= Lk) sc[e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // finite from the first tile on: key 0 is visible to every row
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, -m_run));
      sc[e] = p;
      rs += p;
    }
    l_run += rs;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kr = kslot_row(j, lane);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32_f32(Vs[kr * ST + 32 * dt + l32], sc[j], oacc[dt]);
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < Lq) {
    const float inv = 1.f / l_tot;
    float* orow = o + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = oacc[dt][4 * a + i] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * a + 4 * hl) = w;
      }
    }
    if (hl == 0) lse[(size_t)hb * Lq + qrow] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// Dense launches with few 256-row query blocks W (over all batch entries and
// heads) split each block's key walk between two wave groups. Causal: below
// ~512 blocks the longest walk, not the total work, sets the kernel time
// (measured at W = 256: +20-33 %; at W = 512 the single walk is 15 % faster).
// Bidirectional walks are all equally long: splitting pays when the doubled
// workgroup count still fits the 256 CUs at once (W = 128: +50 %).
constexpr int64_t kSplitCausalBelow = 384;
constexpr int64_t kSplitFullUpTo = 128;
// Causal launches of fewer than 192 such blocks (the longest walk then twice
// the average or more even when split in two) give each 64-row block to four
// groups of two waves over 32-key tiles instead: twice the workgroups, half
// the longest walk, at half the MFMA work per barrier (measured: 64 blocks
// -18 to -25 %, 128 blocks -15 %; at 256 blocks two groups are 25 % faster).
// Bidirectional launches of at most 64 blocks, which two groups leave on half
// the CUs, likewise (-20 to -23 %; at 128 blocks two groups fill the chip and
// are 25 % faster).
constexpr int64_t kSplit4CausalBelow = 192;
constexpr int64_t kSplit4FullUpTo = 64;

template <int D, bool CAUSAL>
hipError_t fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const AttnShape& s,
                    hipStream_t stream) {
  const int nqb = (s.Lq + 127) / 128;
  const int nhb = s.B * s.Hq;
  const float sl2 = kLog2e / sqrtf((float)D);
  const int nb = (s.Lk + kSparseBlock - 1) / kSparseBlock;
  if (s.layout)
    hipLaunchKernelGGL((attn_fwd_sparse_bf16_kernel<D, CAUSAL>), dim3((unsigned)nqb * nhb), dim3(256), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, s.Lq, s.Lk, s.Hq,
                       s.Hk, s.Hq / s.Hk, nqb, nhb, sl2, s.layout, nb);
  else {
    const int nqb2 = (s.Lq + 255) / 256;
    const int64_t W = (int64_t)nqb2 * nhb;
    if (CAUSAL ? W < kSplit4CausalBelow : W <= kSplit4FullUpTo) {
      const int nqb64 = (s.Lq + 63) / 64;
      hipLaunchKernelGGL((attn_fwd_split_bf16_kernel<D, CAUSAL, 4>), dim3(xcd_run_grid((long long)nqb64 * nhb, kFwdXcdRun)),
                         dim3(512), 0, stream,
                         (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, s.Lq, s.Lk, s.Hq,
                         s.Hk, s.Hq / s.Hk, nqb64, nhb, sl2);
    } else if (CAUSAL ? W < kSplitCausalBelow : W <= kSplitFullUpTo)
      hipLaunchKernelGGL((attn_fwd_split_bf16_kernel<D, CAUSAL>), dim3(xcd_run_grid((long long)nqb * nhb, kFwdXcdRun)),
                         dim3(512), 0, stream,
                         (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, s.Lq, s.Lk, s.Hq,
                         s.Hk, s.Hq / s.Hk, nqb, nhb, sl2);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(xcd_run_grid((long long)nqb2 * nhb, kFwdXcdRun)),
                         dim3(512), 0, stream,
                         (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, s.Lq, s.Lk, s.Hq,
                         s.Hk, s.Hq / s.Hk, nqb2, nhb, sl2);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, const AttnShape& s,
                   hipStream_t stream) {
  const int nqb = (s.Lq + 127) / 128;
  const int nhb = s.B * s.Hq;
  const float sl2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nqb * nhb), dim3(256), 0, stream, q, k, v,
                     o, lse, s.Lq, s.Lk, s.Hq, s.Hk, s.Hq / s.Hk, nqb, nhb, sl2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const AttnShape& s, hipStream_t stream) {
  if (s.D == 128) return s.causal ? fwd_bf16<128, true>(q, k, v, o, lse, s, stream)
                                  : fwd_bf16<128, false>(q, k, v, o, lse, s, stream);
  return s.causal ? fwd_bf16<64, true>(q, k, v, o, lse, s, stream) : fwd_bf16<64, false>(q, k, v, o, lse, s, stream);
}

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               const AttnShape& s, hipStream_t stream) {
  if (s.D == 128) return s.causal ? fwd_f32<128, true>(q, k, v, o, lse, s, stream)
                                  : fwd_f32<128, false>(q, k, v, o, lse, s, stream);
  return s.causal ? fwd_f32<64, true>(q, k, v, o, lse, s, stream) : fwd_f32<64, false>(q, k, v, o, lse, s, stream);
}

}  // namespace ulysses
