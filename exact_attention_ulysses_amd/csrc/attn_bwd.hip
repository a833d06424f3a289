// Exact attention backward on one rank's head group.
//
// The pages train with the method but leave its backward implicit; this is
// the exact gradient of softmax(Q K^T / sqrt(d_h)) V. The probabilities are
// not stored by the forward pass (the N x N matrix is never materialised,
// paper-graph summary of arXiv 2309.14509, section 3.4.5 on FlashAttention);
// they are recomputed from the saved log-sum-exp: P_ij = exp(S_ij - lse_i).
//   delta_i = sum_e dO_ie O_ie                  (preprocess kernel)
//   dV = P^T dO, dS = P o (dO V^T - delta)        (dK/dV kernel)
//   dK = dS^T Q / sqrt(d_h)                       (dK/dV kernel)
//   dQ = dS K / sqrt(d_h)                         (dQ kernel)
// dK/dV and dQ are produced by two kernels that each own their output rows,
// so every output element is written once, without atomics, and results are
// bitwise reproducible; the price is that S and dP are formed twice.
//
// bf16 dK/dV kernel: workgroup = 4 producer waves x 32 key rows and 4
//   consumer waves (dV or dK of 64 keys each); K and V of a producer's keys
//   stay in its registers; query tiles of 64 rows (Q, dO, lse, delta) are
//   staged through LDS. S = Q K^T and dP = dO V^T put keys across lanes, so
//   the accumulators become the B operands of dV^T += dO^T P and
//   dK^T += Q^T dS directly; dO^T and Q^T are read transposed from LDS.
// bf16 dQ kernel: workgroup = 8 waves x 32 query rows, one per CU, sharing
//   the staging of every K/V tile (block layouts, split and chunked walks:
//   4 waves x 32 rows, two per CU); the forward kernel's orientation, with
//   dP^T = V dO^T added and dQ^T += K^T dS^T in place of O^T.
//   Launches of a few hundred query blocks use 8 waves per 128-row block
//   instead, two groups that each walk half of its key tiles and add their dQ
//   accumulators at the end (the longest block's walk sets their time), or
//   cut every block's walk into chunks run by separate workgroups whose fp32
//   partial sums a reduce kernel adds in chunk order, whichever a cost model
//   of the launch ranks faster;
//   dK/dV launches of a few hundred key blocks likewise give each key
//   block's walk to two workgroups (causal launches of at most 128 key
//   blocks: to near-equal parts, more for the longer walks), whose fp32
//   partial sums the block-layout reduce kernel adds.
// Grouped-query attention (pinyu.ai, section "Head-count constraints"): a key
//   head shared by G query heads gets the sum of their gradients; the dK/dV
//   workgroup walks the query tiles of all G heads in turn and accumulates
//   into the same registers. Keys may be fewer or more than queries
//   (cross-attention, bidirectional only).
// Block layouts: the same kernels visit only the active (query block, key
//   block) pairs; heavily attended key blocks are split across workgroups
//   whose fp32 partial sums a last kernel adds in a fixed order.
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "block_sparse.h"
#include "common.h"
#include "kernels.h"
#include "mfma_frag.h"

namespace ulysses {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kDqXcdRun = 32;   // one-walk dQ workgroups an XCD holds at once (one per CU)

// Chunked causal walks (common.h): 128-row block x - 1 has 2x key tiles of
// 64 under the causal mask, cut into ceil(x / t) parts of at most 2t tiles.

// delta[b][h][i] = sum_e dO[b][i][h][e] * O[b][i][h][e]; D/8 lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ d_o,
                                                        float* __restrict__ delta, int Lq, int Hq, int rows) {
  constexpr int G = D / 8;
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int r = gt / G, part = gt % G;
  float acc = 0.f;
  if (r < rows) {
    const T* po = o + (size_t)r * D + part * 8;
    const T* pd = d_o + (size_t)r * D + part * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)po[i], (float)pd[i], acc);
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (r < rows && part == 0) {
    const int h = r % Hq;
    const int bl = r / Hq;
    const int b = bl / Lq, i = bl - b * Lq;
    delta[((size_t)b * Hq + h) * Lq + i] = acc;
  }
}

// ---------------------------------------------------------------------------
// Block layouts: the dK/dV work plan. The column kernel lists the active
// (query head, query block) pairs of every layout column once, in the order
// the dK/dV kernel visits them, so that its workgroups copy a contiguous list
// instead of scanning a layout column (one byte every nb bytes). A column that
// many query blocks attend (a global block) would make one dK/dV workgroup
// walk all of them: a single workgroup plans the work (plan kernel), cutting
// columns with more than kSparseChunk pairs into equal chunks, each chunk a
// work item of its own, as long as the partial-sum slots of the workspace
// last (later heavy columns stay whole); the dK/dV kernel writes a split
// column's chunks as fp32 partial sums and the reduce kernel adds them in
// chunk order. No atomics: the result does not depend on timing.
// ---------------------------------------------------------------------------

// Grid: one workgroup (one wave) per layout column hk * nb + kb.
template <bool CAUSAL>
__global__ __launch_bounds__(64) void bwd_sparse_columns_kernel(const uint8_t* __restrict__ layout, int nb, int G,
                                                                int nlcol, SparsePlan plan) {
  const int col = blockIdx.x;
  if (col >= nlcol) return;
  const int lane = threadIdx.x;
  const int hk = col / nb, kb = col - hk * nb;
  uint16_t* out = plan.colpairs + (size_t)col * G * nb;
  int c = 0;
  for (int g = 0; g < G; ++g) {
    const uint8_t* cp = layout + (size_t)(hk * G + g) * nb * nb + kb;
    for (int base = CAUSAL ? kb : 0; base < nb; base += 64) {
      const int i = base + lane;
      const bool act = i < nb && cp[(size_t)i * nb] != 0;
      const uint64_t m = __ballot(act);
      if (act) out[c + __builtin_popcountll(m & ((uint64_t(1) << lane) - 1))] = (uint16_t)(g * 8192 + i);
      c += __builtin_popcountll(m);
    }
  }
  if (lane == 0) plan.cnt[col] = c;
}

// One workgroup of 256 threads; thread t plans the work columns of a
// contiguous range (work column c has the pairs of layout column c mod nlcol).
__global__ __launch_bounds__(256) void bwd_sparse_plan_kernel(int ncol, int nlcol, SparsePlan plan) {
  __shared__ int s_slots[256], s_items[256], s_splits[256];
  const int t = threadIdx.x;
  const int per = (ncol + 255) / 256;
  const int c0 = min(ncol, t * per), c1 = min(ncol, c0 + per);
  // slots each column would need if split (0 when it stays whole)
  auto demand = [&](int c) {
    const int n = plan.cnt[c % nlcol];
    return n > kSparseChunk ? (n + kSparseChunk - 1) / kSparseChunk : 0;
  };
  auto exclusive_prefix = [&](int* a) {   // serial over 256 values
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = a[i];
      a[i] = acc;
      acc += x;
    }
    return acc;
  };
  int my_slots = 0;
  for (int c = c0; c < c1; ++c) my_slots += demand(c);
  s_slots[t] = my_slots;
  __syncthreads();
  if (t == 0) exclusive_prefix(s_slots);
  __syncthreads();
  // a column is split when its whole demand fits the slots in column order
  int slot = s_slots[t], my_items = 0, my_splits = 0;
  for (int c = c0; c < c1; ++c) {
    const int dmd = demand(c);
    const bool split = dmd > 0 && slot + dmd <= kSparseSlots;
    my_items += split ? dmd : 1;
    my_splits += split;
    slot += dmd;
  }
  s_items[t] = my_items;
  s_splits[t] = my_splits;
  __syncthreads();
  if (t == 0) {
    plan.header[0] = exclusive_prefix(s_items);
    plan.header[1] = exclusive_prefix(s_splits);
  }
  __syncthreads();
  slot = s_slots[t];
  int item = s_items[t], sp = s_splits[t];
  for (int c = c0; c < c1; ++c) {
    const int dmd = demand(c);
    const bool split = dmd > 0 && slot + dmd <= kSparseSlots;
    const int nch = split ? dmd : 1;
    for (int j = 0; j < nch; ++j) plan.items[item + j] = make_int4(c, j, nch, split ? slot : 0);
    if (split) {
      plan.split_col[sp] = c;
      plan.split_slot[sp] = slot;
      plan.split_nch[sp] = nch;
      ++sp;
    }
    item += nch;
    slot += dmd;
  }
}

// dK, dV of the split columns: the chunks' partial sums added in chunk order.
// Work unit u: split column u / (D/4), and 1024/D of its 256 [dK | dV] rows
// from row (1024/D) * (u mod (D/4)) on; each thread sums one 4-float group.
// DENSE: every one of the ndense dense work columns (kb * nb + hb, nb = head
// pairs) has two chunks in slots 2c, 2c + 1.
template <int D, bool DENSE = false>
__global__ __launch_bounds__(256) void bwd_sparse_reduce_kernel(SparsePlan plan, int nb, int Lk, int Hk,
                                                                __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                                                                float scale, int ndense, int nkb, int ck) {
  constexpr int UNITS = D / 4, ROWS = 1024 / D;   // units per split column, rows per unit
  const int nunits = (DENSE ? ndense : plan.header[1]) * UNITS;
  const size_t rsk = (size_t)Hk * D;
  for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
    const int sp = u / UNITS;
    const int col = DENSE ? sp : plan.split_col[sp];
    int slot = DENSE ? 2 * sp : plan.split_slot[sp];
    int nch = DENSE ? 2 : plan.split_nch[sp];
    if (DENSE && ck > 0) {
      // causal key block kb = nkb - x in ceil(x / ck) parts, numbered as the
      // dK/dV kernel numbers its work items (nb = batch x K/V heads here)
      const int x = nkb - col / nb;
      nch = (x + ck - 1) / ck;
      slot = causal_chunk_first(x, col % nb, nkb, nb, ck);
    }
    const int kb = DENSE ? col / nb : col % nb, hb = DENSE ? col % nb : col / nb;
    const int b = hb / Hk, hk = hb - b * Hk;
    const int row = (u - sp * UNITS) * ROWS + (int)threadIdx.x / (D / 4);   // of [dK | dV][128]
    const int c4 = ((int)threadIdx.x % (D / 4)) * 4;
    const int which = row >> 7, r = row & 127;
    f32x4 acc = f32x4{};
    for (int j = 0; j < nch; ++j)
      acc += *reinterpret_cast<const f32x4*>(plan.partials + ((size_t)(slot + j) * 256 + row) * D + c4);
    const int key = kb * 128 + r;
    if (key < Lk) {
      __bf16* dst = (which ? dv : dk) + ((size_t)b * Lk * Hk + hk) * D + (size_t)key * rsk + c4;
      const float sc = which ? 1.f : scale;
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[i] * sc);
      *reinterpret_cast<bf16x4*>(dst) = o;
    }
  }
}

// dK/dV as producer and consumer waves. A workgroup owns 128 keys and has 8
// waves: producer wave w (0..3) owns keys 32w..32w+31; consumer wave 4 + c
// accumulates one product, dV (c even) or dK (c odd), for the 64 keys of
// producers 2 (c / 2) and 2 (c / 2) + 1. For each 64-row query tile a
// producer forms S = Q K^T and dP = dO V^T (K and V of its keys stay in its
// registers), the probabilities P and dS = P o (dP - delta), and writes both
// as bf16 MFMA operands to LDS; one tile later the consumers read them and
// accumulate dV^T += dO^T P or dK^T += Q^T dS, each transposed dO^T or Q^T
// fragment they read from LDS feeding the MFMAs of both 32-key halves.
// Neither role needs more than 256 registers, so a producer and a consumer
// share each SIMD (in-order placement of a workgroup's waves) and the
// producer's exponentials and products run while the consumer's MFMAs do.
// Tiles are double buffered; each step ends with two barriers (hand-over,
// then the staging of the next tile, which producers (dO) and consumers (Q)
// share).
// SPLIT (dense launches of few key blocks): workgroup 2c + h walks half h of
// key-block column c's query tiles and leaves unscaled fp32 partial sums in
// slot 2c + h, which the reduce kernel adds in order; with ck > 0 (causal)
// key block kb is cut into ceil((nkb_all - kb) / ck) parts instead, work
// item i writing slot i.
template <int D, bool CAUSAL, bool SPARSE, bool SPLIT = false>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Lq, int Lk, int Hq, int Hk, int G, int nhb, float sl2,
    float scale, const uint8_t* __restrict__ layout, int nb, const SparsePlan plan, int nkb_all, int ck) {
  constexpr int BQ = 64, KS = D / 16, DT = D / 32, CPR = D / 8, CH = BQ * CPR / 256, RSTEP = 256 / CPR;
  constexpr int ST = Stride<D>::both;  // Q and dO tiles are read along rows and transposed
  __shared__ __attribute__((aligned(16))) __bf16 Qs[2][BQ * ST];
  __shared__ __attribute__((aligned(16))) __bf16 Ds[2][BQ * ST];   // dO tiles
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dls[2][BQ];
  // hand-over: [buffer][producer][P or dS][half u * 2 + chunk c][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 hand[2][4][2][4][64];
  // block layouts: this work item's (query head g, query block i) pairs,
  // g * 8192 + i, in visiting order
  __shared__ uint16_t pairs[SPARSE ? kMaxSparsePairs : 1];

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < 4;
  const int pw = wave & 3;                 // key group of this wave (shared by the pair)
  // dense: job (key block, head pair), key block 0 having the most query
  // tiles under the causal mask; block layouts: the planned work item (key
  // block column, chunk of its pairs)
  int col = blockIdx.x, chunk = 0, nchunk = 1, slot = 0;
  if constexpr (SPARSE) {
    if ((int)blockIdx.x >= plan.header[0]) return;   // no work item (uniform for the workgroup)
    const int4 it = plan.items[blockIdx.x];
    col = it.x;
    chunk = it.y;
    nchunk = it.z;
    slot = it.w;
  }
  if constexpr (SPLIT) {
    if (CAUSAL && ck > 0) {
      // key block kb = nkb_all - x (its column has x query blocks) cut into
      // ceil(x / ck) parts, columns longest first
      const int i = blockIdx.x;
      int x, hbi;
      causal_chunk_item(i, nkb_all, nhb, ck, &x, &hbi, &chunk, &nchunk);
      col = (nkb_all - x) * nhb + hbi;
      slot = i - chunk;
    } else {
      col = (int)blockIdx.x >> 1;
      chunk = (int)blockIdx.x & 1;
      nchunk = 2;
      slot = 2 * col;
    }
  } else if constexpr (!SPARSE) {
    // jobs (key block kb, head pair hb), longest first. Workgroup i runs on
    // XCD i mod 8 (round-robin dispatch); each XCD takes runs of 32 jobs,
    // neighbouring key blocks of one head pair where the head pairs divide a
    // round, so that the workgroups sharing its L2 read the same query tiles
    // a few steps apart. Runs go to XCDs 0..7 and 7..0 in alternate rounds of
    // 256 jobs, which keeps the causal work of the XCDs even.
    int rank, hbr;
    if (!xcd_run_block((int)blockIdx.x, 32, nhb, nkb_all, &rank, &hbr)) return;   // grid rounded up
    col = rank * nhb + hbr;
  }
  const int kb = SPARSE ? col % (nb) : col / nhb;
  const int hb = SPARSE ? col / (nb) : col % nhb;   // (batch, key head) pair
  const int b = hb / Hk, hk = hb - b * Hk;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;   // row strides
  // query heads hk*G .. hk*G + G-1 share this key head; g selects one of them
  const size_t qoff = ((size_t)b * Lq * Hq + (size_t)hk * G) * D;
  const size_t koff = ((size_t)b * Lk * Hk + hk) * D;
  const __bf16* qh = q + qoff;
  const __bf16* doh = d_o + qoff;
  const float* lseh = lse + ((size_t)b * Hq + (size_t)hk * G) * Lq;   // head g at + g * Lq
  const float* dlh = delta + ((size_t)b * Hq + (size_t)hk * G) * Lq;
  const int key = kb * 128 + 32 * pw + l32;

  const int qstart = CAUSAL ? kb * 128 : 0;
  const int nqt = (Lq - qstart + BQ - 1) / BQ;   // query tiles per query head
  int nsteps = G * nqt;
  int tbase = 0;   // first step of this workgroup's share of the walk (SPLIT)
  if constexpr (SPLIT) {
    tbase = chunk * nsteps / nchunk;
    nsteps = (chunk + 1) * nsteps / nchunk - tbase;
  }
  // under the causal mask only the first two query tiles reach above a key of this block
  const int nmask = CAUSAL ? min(nqt, 2) : 0;
  if constexpr (SPARSE) {
    // this work item's share of the layout column's listed pairs (query head,
    // query block; causal: from the diagonal block on): chunk `chunk` of
    // `nchunk` equal parts, copied to LDS; each query block is two 64-row
    // query tiles
    const int lcol = hk * nb + kb;
    const int npairs = plan.cnt[lcol];
    const int per = (npairs + nchunk - 1) / nchunk;
    const int pair0 = chunk * per;
    const int n = max(0, min(npairs, pair0 + per) - pair0);
    const uint16_t* src = plan.colpairs + (size_t)lcol * G * nb + pair0;
    for (int i = tid; i < n; i += 512) pairs[i] = src[i];
    nsteps = 2 * n;
    __syncthreads();
  }

  // staging of the query tiles through buffer loads, split between the roles
  // so that each wave moves half as much while the workgroup waits between
  // its two barriers: the producers stage dO (and the LSE / delta rows), the
  // consumers Q; each role's 256 threads cover one 64 x D tile. Rows past the
  // end of the sequence read as zero (the range covers Lq rows from the
  // group's first head, and every head of the group lies inside a row).
  const int stid = tid & 255;
  const int srow = stid / CPR, scol = (stid % CPR) * 8;
  const uint32_t head_bytes = (uint32_t)((size_t)Lq * rsq * 2);
  const __amdgpu_buffer_rsrc_t srs = head_rsrc(producer ? doh : qh, head_bytes);
  uint32_t voff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) voff[j] = (uint32_t)(((srow + j * RSTEP) * rsq + scol) * 2);
  u32x4 sreg[CH];
  float lse_r = 0.f, dl_r = 0.f;
  bool row_ok = false;
  // Step t handles the query tile starting at row q0 of the group's query head
  // g: dense, tile t mod nqt of head t div nqt; with a block layout, half t & 1
  // of the listed pair t / 2. `diag` marks the tiles that reach above a key of
  // this block under the causal mask.
  const FastDiv fq = make_fastdiv((uint32_t)nqt);
  auto tile_of = [&](int t, int& g, int& q0, bool& diag) {
    if constexpr (SPARSE) {
      const int e = pairs[t >> 1];
      g = e >> 13;
      const int i = e & 8191;
      q0 = (2 * i + (t & 1)) * BQ;
      diag = CAUSAL && i == kb;
    } else {
      g = (int)fdiv((uint32_t)(t + tbase), fq);
      const int qt = t + tbase - g * nqt;
      q0 = qstart + qt * BQ;
      diag = CAUSAL && qt < nmask;
    }
  };
  auto load_tile = [&](int t) {
    int g, q0;
    bool diag;
    tile_of(t, g, q0, diag);
    const uint32_t soff = (uint32_t)q0 * (uint32_t)(rsq * 2) + (uint32_t)(g * D * 2);
#pragma unroll
    for (int j = 0; j < CH; ++j) sreg[j] = buf_load16(srs, voff[j] + soff, 0);
    if (tid < BQ) {
      // raw values only: they are first used when the tile is stored, a step
      // later, so this wave does not wait here for the loads (rows past the
      // end read the last row and are fixed up at the store)
      const int qi = q0 + tid;
      row_ok = qi < Lq;
      const size_t qc = (size_t)g * Lq + (row_ok ? qi : Lq - 1);
      lse_r = lseh[qc];
      dl_r = dlh[qc];
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* dst = producer ? Ds[buf] : Qs[buf];
#pragma unroll
    for (int j = 0; j < CH; ++j) *reinterpret_cast<u32x4*>(&dst[(srow + j * RSTEP) * ST + scol]) = sreg[j];
    if (tid < BQ) {
      // rows past the end, and rows that see no key (LSE -inf, block layouts
      // only), get lse = +inf, so their probabilities are exactly 0
      lse2s[buf][tid] = (!row_ok || lse_r == -INFINITY) ? INFINITY : lse_r * kLog2e;
      dls[buf][tid] = row_ok ? -dl_r : 0.f;   // -delta: the dP accumulator starts from it
    }
  };

  // both roles stage their half of tile 0 and load their half of tile 1
  if (nsteps > 0) load_tile(0);
  store_tile(0);
  __syncthreads();
  if (nsteps > 1) load_tile(1);

  if (producer) {
    // ---------------- producer: S, dP, P, dS ----------------
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (key < Lk) {
        kf[ks] = *reinterpret_cast<const bf16x8*>(k + koff + (size_t)key * rsk + 16 * ks + 8 * hl);
        vf[ks] = *reinterpret_cast<const bf16x8*>(v + koff + (size_t)key * rsk + 16 * ks + 8 * hl);
      } else {
        kf[ks] = bf16x8{};
        vf[ks] = bf16x8{};
      }
    }
    // step s (LDS buffer s & 1) handles query tile qt of one query head
    auto produce = [&](int s, int q0, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int cur = s & 1;
      const __bf16* Qc = Qs[cur];
      const __bf16* Dc = Ds[cur];
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sc[u] = f32x16{};
        // dP - delta: the accumulator starts from -delta of its rows (element
        // 4a + i holds row 32u + 8a + 4 * (lane / 32) + i), so the MFMAs leave
        // dP - delta and the softmax step needs no subtraction
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 nd4 = *reinterpret_cast<const f32x4*>(&dls[cur][32 * u + 8 * a + 4 * hl]);
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[u][4 * a + i] = nd4[i];
        }
        // all of the half's Q and dO fragments are read before its MFMAs
        // start, so that the MFMAs do not each wait on a fresh LDS read
        bf16x8 qa[KS], da[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qa[ks] = frag_row<ST>(Qc, 32 * u, 16 * ks, lane);
          da[ks] = frag_row<ST>(Dc, 32 * u, 16 * ks, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sc[u] = mfma32(qa[ks], kf[ks], sc[u]);
          dp[u] = mfma32(da[ks], vf[ks], dp[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int r0 = 32 * u + 8 * a + 4 * hl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[cur][r0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * a + i;
            float p = __builtin_amdgcn_exp2f(fmaf(sc[u][e], sl2, -l4[i]));
            float ds = p * dp[u][e];
            if (MASK && key > q0 + r0 + i) {  // keys above the query row
              p = 0.f;
              ds = 0.f;
            }
            sc[u][e] = p;
            dp[u][e] = ds;
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          hand[cur][pw][0][2 * u + c][lane] = acc_chunk_bf16(sc[u], c);
          hand[cur][pw][1][2 * u + c][lane] = acc_chunk_bf16(dp[u], c);
        }
      }
    };
    for (int s = 0; s <= nsteps; ++s) {
      if (s < nsteps) {
        int g, q0;
        bool diag;
        tile_of(s, g, q0, diag);
        if (diag)
          produce(s, q0, std::integral_constant<bool, true>{});
        else
          produce(s, q0, std::integral_constant<bool, false>{});
      }
      __syncthreads();  // hand-over of tile s; consumers are done with tile s-1's buffers
      if (s + 1 < nsteps) store_tile((s + 1) & 1);
      if (s + 2 < nsteps) load_tile(s + 2);
      __syncthreads();  // tile s+1 staged
    }
  } else {
    // ---------------- consumer: dV or dK of 64 keys ----------------
    // consumer wave c (c = wave - 4) takes the keys of producers 2 (c / 2) and
    // 2 (c / 2) + 1 and one product: dV^T += dO^T P (c even) or dK^T += Q^T dS
    // (c odd), so every transposed dO^T or Q^T fragment it reads from LDS
    // feeds two MFMAs, one per 32-key half.
    const int cw = wave - 4, kp = cw >> 1, role = cw & 1;
    f32x16 acc[2][DT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[h][dt] = f32x16{};
    }
    for (int s = 0; s <= nsteps; ++s) {
      if (s >= 1) {
        const int prev = (s - 1) & 1;
        const __bf16* Tc = role ? Qs[prev] : Ds[prev];
#pragma unroll
        for (int uc = 0; uc < 4; ++uc) {
          const bf16x8 b0 = hand[prev][2 * kp][role][uc][lane];
          const bf16x8 b1 = hand[prev][2 * kp + 1][role][uc][lane];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 a = frag_col<ST>(Tc, 16 * uc, 32 * dt, lane);
            acc[0][dt] = mfma32(a, b0, acc[0][dt]);
            acc[1][dt] = mfma32(a, b1, acc[1][dt]);
          }
        }
      }
      __syncthreads();  // consumers are done with tile s-1's buffers
      if (s + 1 < nsteps) store_tile((s + 1) & 1);
      if (s + 2 < nsteps) load_tile(s + 2);
      __syncthreads();
    }
    if ((SPARSE && nchunk > 1) || SPLIT) {
      // one chunk of a split column: unscaled fp32 partial sums, [dK | dV][128 keys][D],
      // summed in chunk order by the reduce kernel
      float* part = plan.partials + ((size_t)(slot + chunk) * 2 * 128 + (role ? 0 : 128)) * D;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = 64 * kp + 32 * h + l32;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4 x4;
#pragma unroll
            for (int i = 0; i < 4; ++i) x4[i] = acc[h][dt][4 * a + i];
            *reinterpret_cast<f32x4*>(part + (size_t)kr * D + 32 * dt + 8 * a + 4 * hl) = x4;
          }
        }
      }
    } else {
      __bf16* out = role ? dk : dv;
      const float sc = role ? scale : 1.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = kb * 128 + 64 * kp + 32 * h + l32;
        if (kk < Lk) {
          __bf16* row = out + koff + (size_t)kk * rsk;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<bf16x4*>(row + 32 * dt + 8 * a + 4 * hl) = acc_quad_bf16(acc[h][dt], a, sc);
          }
        }
      }
    }
  }
}

// NG = 2 (dense launches too small to fill the chip): 8 waves, two groups
// over the same 128 rows; group 0 walks the first half of the key tiles and
// group 1 the second, each through its own K/V buffers, and group 0 adds
// group 1's dQ accumulators to its own through LDS at the end.
template <int D, bool CAUSAL, bool SPARSE, int NG = 1, bool CHUNK = false, int RW = 4>
__global__ __launch_bounds__(64 * RW * NG, RW * NG == 4 ? 2 : 1) void bwd_dq_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    __bf16* __restrict__ dq, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb, float sl2, float scale,
    const uint8_t* __restrict__ layout, int nb, int ck, float* __restrict__ part) {
  static_assert(NG == 1 || (NG == 2 && !SPARSE), "split key walks are for dense attention");
  static_assert(!CHUNK || (NG == 1 && !SPARSE), "chunked key walks are for dense attention");
  static_assert((RW == 8) == (NG == 1 && !CHUNK && !SPARSE), "256-row blocks exactly for dense one-walk launches");
  constexpr int TPG = 64 * RW;             // threads of one key-walk group, which stage its tiles
  constexpr int BM = 32 * RW, BN = 64, KS = D / 16, DT = D / 32, CPR = D / 8, CH = BN * CPR / TPG,
                RSTEP = TPG / CPR;
  constexpr int KST = Stride<D>::both;  // K: rows for S^T = K Q^T, transposed for dQ^T += K^T dS^T
  constexpr int VST = Stride<D>::row;   // V: rows for dP^T = V dO^T
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2 * NG][BN * KST];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2 * NG][BN * VST];

  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (RW - 1);   // row group of this wave
  const int grp = NG == 2 ? __builtin_amdgcn_readfirstlane(tid >> 8) : 0;   // key half (NG = 2)
  // jobs (query block, head pair), longest rows first; the dense one-walk
  // launch takes them in runs of 32 per XCD (one workgroup per CU), so that
  // the blocks on one XCD walk the same key tiles a few steps apart and
  // share them through its L2
  int rank = (int)blockIdx.x / nhb;
  int hb = (int)blockIdx.x % nhb;          // (batch, query head) pair
  if constexpr (!SPARSE && NG == 1 && !CHUNK) {
    if (!xcd_run_block((int)blockIdx.x, kDqXcdRun, nhb, nqb, &rank, &hb)) return;   // grid rounded up
  }
  int qb = nqb - 1 - rank;
  int chunk = 0, nchunk = 1;               // this workgroup's part of the block's key walk (CHUNK)
  if constexpr (CHUNK) {
    const int i = blockIdx.x;
    if constexpr (CAUSAL) {
      // block qb = x - 1 has ceil(x / ck) chunks, blocks longest first
      int x;
      causal_chunk_item(i, nqb, nhb, ck, &x, &hb, &chunk, &nchunk);
      qb = x - 1;
    } else {
      nchunk = ck;   // every block: ck chunks
      const int bi = i / nchunk;
      chunk = i - bi * nchunk;
      qb = nqb - 1 - bi / nhb;
      hb = bi % nhb;
    }
  }
  const int b = hb / Hq, h = hb - b * Hq;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;
  const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
  const size_t koff = ((size_t)b * Lk * Hk + h / G) * D;
  const __bf16* kh = k + koff;
  const __bf16* vh = v + koff;
  const int q0 = qb * BM;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + l32;
  const bool valid = qrow < Lq;

  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (valid) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(q + qoff + (size_t)qrow * rsq + 16 * ks + 8 * hl);
      df[ks] = *reinterpret_cast<const bf16x8*>(d_o + qoff + (size_t)qrow * rsq + 16 * ks + 8 * hl);
    } else {
      qf[ks] = bf16x8{};
      df[ks] = bf16x8{};
    }
  }
  // a row that sees no key (LSE -inf, block layouts only) has probabilities 0
  const float lse_i = valid ? lse[(size_t)hb * Lq + qrow] : 0.f;
  const float nlse2 = lse_i == -INFINITY ? -INFINITY : -lse_i * kLog2e;
  const float dl = valid ? delta[(size_t)hb * Lq + qrow] : 0.f;

  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

  const int kend = CAUSAL ? min(Lk, q0 + BM) : Lk;
  const int nkb = (kend + BN - 1) / BN;
  const int srow = (tid & (TPG - 1)) / CPR, scol = (tid % CPR) * 8;
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
      *reinterpret_cast<u32x4*>(&Ks[2 * grp + buf][(srow + j * RSTEP) * KST + scol]) = kreg[j];
      *reinterpret_cast<u32x4*>(&Vs[2 * grp + buf][(srow + j * RSTEP) * VST + scol]) = vreg[j];
    }
  };

  // key tile kb in LDS buffer cur; then the staged tile goes to the other
  // buffer (if store) and key tile next2 into the staging registers (if >= 0)
  auto tile = [&](int cur, int kb, bool store, int next2, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const __bf16* Kc = Ks[2 * grp + cur];
    const __bf16* Vc = Vs[2 * grp + cur];
    const int k0 = kb * BN;
    const bool edge = EDGE && (CAUSAL ? (k0 + BN - 1 > qw0) : (k0 + BN > Lk));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        bf16x8 ka[KS], va[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ka[ks] = frag_row<KST>(Kc, 32 * mt, 16 * ks, lane);
          va[ks] = frag_row<VST>(Vc, 32 * mt, 16 * ks, lane);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = mfma32(ka[ks], qf[ks], s);
          dp = mfma32(va[ks], df[ks], dp);
        }
        // LDS reads run LOOK fragments ahead of the MFMAs that use them (the
        // registers of this kernel leave room for 8 in 256-row workgroups,
        // whose staging holds half as much per thread, and for 4 in 128-row
        // ones, where a few values live across the two tile loops go to
        // scratch once per workgroup, outside the loops)
        constexpr int LOOK = RW == 8 ? 8 : 4;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK, 0);
#pragma unroll
        for (int i = 0; i < 2 * KS - LOOK; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, LOOK, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, nlse2));
        s[e] = p * (dp[e] - dl);  // dS^T of this 32-key half
      }
      if (edge) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = k0 + 32 * mt + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (CAUSAL ? (kk > qrow) : (kk >= Lk)) s[e] = 0.f;
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 dsf = acc_chunk_bf16(s, c);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dqacc[dt] = mfma32(frag_col<KST>(Kc, 32 * mt + 16 * c, 32 * dt, lane), dsf, dqacc[dt]);
      }
    }
    if (store) store_tile(cur ^ 1);
    if (next2 >= 0) load_tile(next2);
    __syncthreads();
  };
  const auto steady = std::integral_constant<bool, false>{};
  const auto edge = std::integral_constant<bool, true>{};

  if constexpr (CHUNK) {
    // key tiles [t0, t1): part `chunk` of `nchunk` near-equal parts of the walk
    const int t0 = chunk * nkb / nchunk, cnt = (chunk + 1) * nkb / nchunk - t0;
    const int nsteady = CAUSAL ? max(0, nkb - 2) : (Lk % BN ? nkb - 1 : nkb);
    load_tile(t0);
    store_tile(0);
    __syncthreads();
    if (cnt > 1) load_tile(t0 + 1);
    int i = 0;
    for (; i < cnt && t0 + i < nsteady; ++i)
      tile(i & 1, t0 + i, i + 1 < cnt, i + 2 < cnt ? t0 + i + 2 : -1, steady);
    for (; i < cnt; ++i) tile(i & 1, t0 + i, i + 1 < cnt, i + 2 < cnt ? t0 + i + 2 : -1, edge);
  } else if constexpr (!SPARSE && NG == 1) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    if (nkb > 1) load_tile(1);
    // as in the forward pass: only the last BM / BN key tiles (causal) or a ragged last tile need a mask
    const int nsteady = CAUSAL ? max(0, nkb - BM / BN) : (Lk % BN ? nkb - 1 : nkb);
    int kb = 0;
    for (; kb < nsteady; ++kb) tile(kb & 1, kb, kb + 1 < nkb, kb + 2 < nkb ? kb + 2 : -1, steady);
    for (; kb < nkb; ++kb) tile(kb & 1, kb, kb + 1 < nkb, kb + 2 < nkb ? kb + 2 : -1, edge);
  } else if constexpr (!SPARSE) {
    // this group's key tiles [t0, t0 + cnt); both groups pass `steps` barriers
    const int nsteady = CAUSAL ? max(0, nkb - 2) : (Lk % BN ? nkb - 1 : nkb);
    const int t0 = grp ? nkb / 2 : 0;
    const int cnt = grp ? nkb - nkb / 2 : nkb / 2;
    const int steps = nkb - nkb / 2;
    if (cnt > 0) {
      load_tile(t0);
      store_tile(0);
    }
    __syncthreads();
    if (cnt > 1) load_tile(t0 + 1);
    int i = 0;
    for (; i < cnt && t0 + i < nsteady; ++i)
      tile(i & 1, t0 + i, i + 1 < cnt, i + 2 < cnt ? t0 + i + 2 : -1, steady);
    for (; i < cnt; ++i) tile(i & 1, t0 + i, i + 1 < cnt, i + 2 < cnt ? t0 + i + 2 : -1, edge);
    for (; i < steps; ++i) __syncthreads();   // group 0's idle step when nkb is odd
    // every tile read ended at the last barrier: group 1's accumulators go
    // through the K/V buffers to group 0
    static_assert(4 * DT * 16 * 64 * 4 <= (int)(sizeof(Ks) + sizeof(Vs)), "merge exceeds the tile buffers");
    float* rec = reinterpret_cast<float*>(&Ks[0][0]) + wave * (DT * 16 * 64);
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) rec[(dt * 16 + e) * 64 + lane] = dqacc[dt][e];
      }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) dqacc[dt][e] += rec[(dt * 16 + e) * 64 + lane];
    }
  } else {
    // active key blocks of this query block, two key tiles each, as in the forward kernel
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
        tile(half, 2 * j + half, half == 0 || jn >= 0, jn >= 0 ? 2 * jn + half : -1, edge);
        if (half == 1) {
          j = jn;
          if (j >= 0) jn = scan.next(lane);
        }
        half ^= 1;
      }
    }
  }

  if constexpr (CHUNK) {
    // unscaled fp32 partial sums of the block's 128 rows in slot blockIdx.x,
    // [128][D]; the reduce kernel adds a block's slots in chunk order
    float* prow = part + ((size_t)blockIdx.x * 128 + 32 * wave + l32) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = dqacc[dt][4 * a + i];
        *reinterpret_cast<f32x4*>(prow + 32 * dt + 8 * a + 4 * hl) = v4;
      }
    }
  } else if (valid) {
    __bf16* row = dq + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<bf16x4*>(row + 32 * dt + 8 * a + 4 * hl) = acc_quad_bf16(dqacc[dt], a, scale);
    }
  }
}

// Chunked dQ: block (x = query block + 1, head pair hb) owns ceil(x / ck)
// consecutive slots (causal; ck per block when bidirectional), in the order
// the dQ kernel numbers its work items; their sum, scaled and rounded once,
// is the block's dQ.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const float* __restrict__ part, __bf16* __restrict__ dq,
                                                            int Lq, int Hq, int nqb, int nhb, int ck, float scale) {
  constexpr int UNITS = 128 * D / 1024, ROWS = 1024 / D;   // units per block, rows per unit
  const int nunits = nqb * nhb * UNITS;
  for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
    const int bi = u / UNITS;                    // blocks longest first, head pairs inner
    const int x = nqb - bi / nhb, hb = bi % nhb;
    const int nch = CAUSAL ? (x + ck - 1) / ck : ck;
    const int base = CAUSAL ? causal_chunk_first(x, hb, nqb, nhb, ck) : bi * nch;
    const int row = (u - bi * UNITS) * ROWS + (int)threadIdx.x / (D / 4);
    const int c4 = ((int)threadIdx.x % (D / 4)) * 4;
    f32x4 acc = f32x4{};
    for (int j = 0; j < nch; ++j)
      acc += *reinterpret_cast<const f32x4*>(part + ((size_t)(base + j) * 128 + row) * D + c4);
    const int qrow = (x - 1) * 128 + row;
    if (qrow < Lq) {
      const int b = hb / Hq, h = hb - b * Hq;
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[i] * scale);
      *reinterpret_cast<bf16x4*>(dq + (((size_t)b * Lq + qrow) * Hq + h) * D + c4) = o;
    }
  }
}

// fp32 dK/dV on the fp32 MFMA: workgroup = 4 waves x 32 key rows (128 keys),
// query tiles of 32 rows (Q, dO, LSE, delta) in LDS. Each wave forms
// S = Q K^T (and for dK dP = dO V^T) with keys across lanes, K and V of its
// keys in registers, so that P and dS = P o (dP - delta) are the B operands
// of dV^T += dO^T P and dK^T += Q^T dS directly; dO^T and Q^T are read from
// the row-major tiles in the accumulator's row order. Grouped-query heads:
// the walk covers the query tiles of the G query heads in turn. dK and dV
// sum over every query, which with few keys means long sums of sizeable
// terms: each tile's 16 MFMA steps accumulate in fp32 from zero and the tile
// is added to fp64 running sums, so the result carries the rounding of the
// small tile sums and one final rounding. The fp64 sums of both outputs do
// not fit the registers at once: the kernel runs once for dV (WHICH = 0,
// no dP) and once for dK (WHICH = 1).
template <int D, bool CAUSAL, int WHICH>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ out, int Lq, int Lk, int Hq, int Hk, int G, int nhb, float sl2, float scale) {
  constexpr int BQ = 32, ST = StrideF32<D>::row, KS = D / 2, DT = D / 32, C4 = D / 4;
  constexpr bool DK = WHICH == 1;
  __shared__ __attribute__((aligned(16))) float Qs[BQ * ST];
  __shared__ __attribute__((aligned(16))) float Ds[BQ * ST];   // dO rows
  __shared__ float ls[BQ], dls[BQ];   // LSE (log2 units; +inf past the end) and delta per row
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = blockIdx.x / nhb;
  const int hb = blockIdx.x % nhb;         // (batch, key head) pair
  const int b = hb / Hk, hk = hb - b * Hk;
  const size_t rsq = (size_t)Hq * D, rsk = (size_t)Hk * D;
  const size_t koff = ((size_t)b * Lk * Hk + hk) * D;
  const int kw0 = kb * 128 + 32 * wave, key = kw0 + l32;

  // K^T (and V^T) as B operands: step t holds K[key][2t + hl]
  float kf[KS], vf[DK ? KS : 1];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    kf[t] = key < Lk ? k[koff + (size_t)key * rsk + 2 * t + hl] : 0.f;
    if constexpr (DK) vf[t] = key < Lk ? v[koff + (size_t)key * rsk + 2 * t + hl] : 0.f;
  }
  double sum[DT][16];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[dt][e] = 0.0;
  }
  const int qstart = CAUSAL ? kb * 128 : 0;   // causal: no earlier query sees a key of this block
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const size_t qoff = ((size_t)b * Lq * Hq + h) * D;
    const size_t loff = ((size_t)b * Hq + h) * Lq;
    for (int q0 = qstart; q0 < Lq; q0 += BQ) {
      __syncthreads();
      for (int c = tid; c < BQ * C4; c += 256) {
        const int r = c / C4, e = (c - r * C4) * 4, qi = q0 + r;
        f32x4 qv = f32x4{}, dv4 = f32x4{};
        if (qi < Lq) {
          qv = *reinterpret_cast<const f32x4*>(q + qoff + (size_t)qi * rsq + e);
          dv4 = *reinterpret_cast<const f32x4*>(d_o + qoff + (size_t)qi * rsq + e);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Qs[r * ST + e + i] = qv[i];
          Ds[r * ST + e + i] = dv4[i];
        }
      }
      if (tid < BQ) {
        const int qi = q0 + tid;
        ls[tid] = qi < Lq ? lse[loff + qi] * kLog2e : INFINITY;
        dls[tid] = qi < Lq ? delta[loff + qi] : 0.f;
      }
      __syncthreads();
      if (CAUSAL && q0 + BQ - 1 < kw0) continue;   // every query of the tile before this wave's keys
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        sc = mfma32_f32(Qs[l32 * ST + 2 * t + hl], kf[t], sc);
        if constexpr (DK) dp = mfma32_f32(Ds[l32 * ST + 2 * t + hl], vf[t], dp);
      }
      // element e: query row q0 + kslot_row(e), this lane's key
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = kslot_row(e, lane);
        float p = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, -ls[r]));   // 0 past the end (LSE +inf)
        if (CAUSAL && key > q0 + r) p = 0.f;
        sc[e] = DK ? p * (dp[e] - dls[r]) : p;   // dS or P
      }
      f32x16 acc[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = kslot_row(j, lane);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = mfma32_f32(DK ? Qs[r * ST + 32 * dt + l32] : Ds[r * ST + 32 * dt + l32], sc[j], acc[dt]);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[dt][e] += (double)acc[dt][e];
      }
    }
  }
  if (key < Lk) {
    float* row = out + koff + (size_t)key * rsk;
    const double sc = DK ? (double)scale : 1.0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (float)(sum[dt][4 * a + i] * sc);
        *reinterpret_cast<f32x4*>(row + 32 * dt + 8 * a + 4 * hl) = w;
      }
    }
  }
}

// fp32 dQ on the fp32 MFMA: workgroup = 4 waves x 32 query rows, key tiles of
// 32 in LDS; S^T = K Q^T and dP^T = V dO^T (queries across lanes, Q and dO in
// registers), then dQ^T += K^T dS^T with dS^T as the B operand.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, int Lq, int Lk, int Hq, int Hk, int G, int nqb, int nhb, float sl2, float scale) {
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
  const bool rv = qrow < Lq;

  float qf[KS], df[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    qf[t] = rv ? q[qoff + (size_t)qrow * rsq + 2 * t + hl] : 0.f;
    df[t] = rv ? d_o[qoff + (size_t)qrow * rsq + 2 * t + hl] : 0.f;
  }
  const float l2 = rv ? lse[(size_t)hb * Lq + qrow] * kLog2e : INFINITY;   // rows past the end: P = 0
  const float dl = rv ? delta[(size_t)hb * Lq + qrow] : 0.f;
  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

  const int kend = CAUSAL ? min(Lk, q0 + 128) : Lk;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * C4; c += 256) {
      const int r = c / C4, e = (c - r * C4) * 4, kk = k0 + r;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (kk < Lk) {
        kv = *reinterpret_cast<const f32x4*>(k + koff + (size_t)kk * rsk + e);
        vv = *reinterpret_cast<const f32x4*>(v + koff + (size_t)kk * rsk + e);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Ks[r * ST + e + i] = kv[i];
        Vs[r * ST + e + i] = vv[i];
      }
    }
    __syncthreads();
    if (CAUSAL && k0 > qw0 + 31) continue;   // every key of the tile above this wave's rows
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      sc = mfma32_f32(Ks[l32 * ST + 2 * t + hl], qf[t], sc);
      dp = mfma32_f32(Vs[l32 * ST + 2 * t + hl], df[t], dp);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kk = k0 + kslot_row(e, lane);
      float p = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, -l2));
      if ((CAUSAL && kk > qrow) || kk >= Lk) p = 0.f;
      sc[e] = p * (dp[e] - dl);   // dS^T
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kr = kslot_row(j, lane);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dqacc[dt] = mfma32_f32(Ks[kr * ST + 32 * dt + l32], sc[j], dqacc[dt]);
    }
  }
  if (rv) {
    float* row = dq + qoff + (size_t)qrow * rsq;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = dqacc[dt][4 * a + i] * scale;
        *reinterpret_cast<f32x4*>(row + 32 * dt + 8 * a + 4 * hl) = w;
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_delta(const T* o, const T* d_o, float* delta, const AttnShape& s, hipStream_t stream) {
  const int rows = s.B * s.Lq * s.Hq;
  const long long threads = (long long)rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3(blocks), dim3(256), 0, stream, o, d_o, delta, s.Lq, s.Hq, rows);
  return hipGetLastError();
}

// Dense bf16 dK/dV launches of few key-block columns C (over batch entries
// and K/V heads) split every column's walk over the query tiles in two. One
// workgroup per CU: under the causal mask the longest column is twice the
// average, so a launch runs at about C / 512 of the chip without the split
// and min(1, C / 256) with it (split below 512 columns); bidirectional
// columns are equally long and pay once the halves still fit the CUs at once
// (at most 128 columns).
inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

inline size_t delta_bytes(const AttnShape& s) { return round256((size_t)s.B * s.Hq * s.Lq * sizeof(float)); }

// fp32 partial sums of the split dK/dV walks: two [dK | dV][128][d_h] slots per column
inline size_t dkdv_split_bytes(const AttnShape& s) {
  const size_t ncol = (size_t)s.B * s.Hk * ((s.Lk + 127) / 128);
  return round256(2 * ncol * 2 * 128 * (size_t)s.D * sizeof(float));
}

inline bool dkdv_split(const AttnShape& s) {
  if (!s.bf16 || s.layout) return false;
  const int64_t ncol = (int64_t)s.B * s.Hk * ((s.Lk + 127) / 128);
  if (!(s.causal ? ncol < 512 : ncol <= 128)) return false;
  return s.ws_cap == 0 || delta_bytes(s) + dkdv_split_bytes(s) <= s.ws_cap;
}

// Causal splits of at most 128 columns run all their halves at once, so the
// half of key block 0 (about G * nkb query tiles) sets the time, twice the
// average. Such launches cut key block kb instead into ceil((nkb - kb) / t)
// near-equal parts (at most 2t G tiles each): the smallest t whose parts
// still fit one round (256 workgroups) and the halves' two slots per column,
// taken when it shortens the longest item by a fifth or more. 0: halves.
inline int dkdv_chunk_t(const AttnShape& s) {
  if (!dkdv_split(s) || !s.causal) return 0;
  const int64_t nkb = (s.Lk + 127) / 128, nkhb = (int64_t)s.B * s.Hk, ncol = nkb * nkhb;
  if (2 * ncol > 256) return 0;   // several rounds of halves: longest first already pairs them evenly
  for (int64_t t = 1; t < nkb; ++t)
    if (nkhb * chunk_prefix((int)nkb, (int)t) <= 2 * ncol) return 10 * t <= 4 * nkb ? (int)t : 0;
  return 0;
}

// Dense dQ launches with few 128-row query blocks W split each block's key
// walk between two wave groups of one workgroup (as the forward does for
// small launches), or cut it into chunks (below).
constexpr int64_t kDqSplitCausalBelow = 512;
constexpr int64_t kDqSplitFullUpTo = 256;

// Dense bf16 dQ launches of few 128-row query blocks can instead cut every
// block's walk over its key tiles into chunks that separate workgroups run
// (two per CU, 512 at once), each leaving unscaled fp32 partial sums in a
// slot of the workspace that a reduce kernel adds in chunk order. Under the
// causal mask block qb has 2(qb + 1) tiles of 64 keys: whole walks leave the
// longest block setting the time of a launch of up to ~1000 blocks (twice
// the balanced time or more), while ceil((qb + 1) / t) near-equal parts of
// block qb make every work item at most 2t tiles long. The host takes the
// t (bidirectional: parts per block) that a cost model in tile steps ranks
// best -- critical path (the longest item when all fit in one round of 512
// workgroups, else the average load of a slot plus half an item), start-up
// per round, partial-sum traffic and the extra launch -- and cuts only where
// that beats the whole walks by 10 %.
struct DqChunks {
  int ck = 0;      // t (causal) or parts per block (bidirectional); 0: whole walks
  int items = 0;   // work items, one partial-sum slot each
};
constexpr int kDqSlots = 512;
constexpr int kDqMaxItems = 4 * kDqSlots;

inline DqChunks dq_chunks(const AttnShape& s) {
  DqChunks best;
  if (!s.bf16 || s.layout) return best;
  const int64_t nqb = (s.Lq + 127) / 128, nhb = (int64_t)s.B * s.Hq, W = nqb * nhb;
  const int64_t nkt = (s.Lk + 63) / 64;   // key tiles of the longest block
  if (W >= kDqMaxItems) return best;
  const double total = s.causal ? (double)nhb * (nqb * (nqb - 1) + nkt) : (double)W * nkt;
  const double avg = total / kDqSlots;
  auto rounds = [](int64_t n, int64_t per) { return (double)((n + per - 1) / per); };
  // whole walks: two wave groups per block below the thresholds above, else one
  const bool ng2 = s.causal ? W < kDqSplitCausalBelow : W <= kDqSplitFullUpTo;
  const double whole = ng2 ? std::max((double)((nkt + 1) / 2), avg) + 2 * rounds(W, 256)
                           : std::max((double)nkt, avg) + 2 * rounds(W, kDqSlots);
  double best_cost = 0.9 * whole;
  // a capped workspace holds as many dQ slots as remain after delta and the dK/dV split
  int64_t max_items = kDqMaxItems;
  if (s.ws_cap) {
    const size_t used = delta_bytes(s) + (dkdv_split(s) ? dkdv_split_bytes(s) : 0);
    max_items = used >= s.ws_cap ? 0 : (int64_t)((s.ws_cap - used) / (128 * (size_t)s.D * sizeof(float)));
  }
  auto consider = [&](int64_t ck, int64_t items, int64_t longest) {
    if (items > kDqMaxItems || items > max_items) return;
    // one round: every item has a slot of its own
    const double path = items <= kDqSlots ? (double)longest : std::max((double)longest, avg + 0.5 * longest);
    const double cost = path + 2 * rounds(items, kDqSlots) + items / 64.0 + 3;
    if (cost < best_cost) {
      best_cost = cost;
      best.ck = (int)ck;
      best.items = (int)items;
    }
  };
  if (s.causal) {
    for (int64_t t = 1; t < nqb; ++t)
      consider(t, nhb * chunk_prefix((int)nqb, (int)t), std::min(2 * t, nkt));
  } else {
    for (int64_t c = 2; c <= nkt && W * c <= kDqMaxItems; ++c) consider(c, W * c, (nkt + c - 1) / c);
  }
  return best;
}

// Workspace: delta [B][Hq][Lq] fp32, then (dense) the dK/dV and the dQ
// partial-sum slots of launches that split their walks, or (block layouts)
// the layout columns' pair counts and lists, the plan and the partial-sum
// slots, each 256-byte aligned.
size_t workspace_layout(const AttnShape& s, bool sparse, SparsePlan* plan, char* base, float** dq_part = nullptr) {
  const size_t ncol = (size_t)s.B * s.Hk * ((s.Lk + kSparseBlock - 1) / kSparseBlock);
  size_t off = delta_bytes(s);
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += round256(bytes);
    return p;
  };
  if (!sparse) {
    if (dkdv_split(s)) {
      SparsePlan pl{};
      pl.partials = (float*)take(dkdv_split_bytes(s));
      if (plan) *plan = pl;
    }
    const DqChunks dc = dq_chunks(s);
    if (dc.items) {
      float* p = (float*)take((size_t)dc.items * 128 * s.D * sizeof(float));
      if (dq_part) *dq_part = p;
    }
    return off;
  }
  const size_t nb = (s.Lk + kSparseBlock - 1) / kSparseBlock, nlcol = (size_t)s.Hk * nb;
  SparsePlan pl;
  pl.cnt = (int*)take(nlcol * sizeof(int));
  pl.colpairs = (uint16_t*)take(nlcol * (s.Hq / s.Hk) * nb * sizeof(uint16_t));
  pl.header = (int*)take(4 * sizeof(int));
  pl.items = (int4*)take((ncol + kSparseSlots) * sizeof(int4));
  pl.split_col = (int*)take(kMaxSplitColumns * sizeof(int));
  pl.split_slot = (int*)take(kMaxSplitColumns * sizeof(int));
  pl.split_nch = (int*)take(kMaxSplitColumns * sizeof(int));
  pl.partials = (float*)take((size_t)kSparseSlots * 2 * 128 * s.D * sizeof(float));
  if (plan) *plan = pl;
  return off;
}

template <int D, bool CAUSAL>
hipError_t bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                    void* dq, void* dk, void* dv, float* delta, const AttnShape& s, hipStream_t stream) {
  hipError_t e = launch_delta<__bf16, D>((const __bf16*)o, (const __bf16*)d_o, delta, s, stream);
  if (e != hipSuccess) return e;
  const int G = s.Hq / s.Hk;
  const float scale = 1.f / sqrtf((float)D);
  const float sl2 = scale * kLog2e;
  const int nkhb = s.B * s.Hk;
  const int nkb = (s.Lk + 127) / 128;
  const int nb = (s.Lk + kSparseBlock - 1) / kSparseBlock;
  if (s.layout) {
    SparsePlan plan;
    workspace_layout(s, true, &plan, reinterpret_cast<char*>(delta));
    const int ncol = nkb * nkhb, nlcol = s.Hk * nb;
    hipLaunchKernelGGL((bwd_sparse_columns_kernel<CAUSAL>), dim3((unsigned)nlcol), dim3(64), 0, stream, s.layout, nb,
                       G, nlcol, plan);
    hipLaunchKernelGGL(bwd_sparse_plan_kernel, dim3(1), dim3(256), 0, stream, ncol, nlcol, plan);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, true>), dim3((unsigned)(ncol + kSparseSlots)), dim3(512), 0,
                       stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dk, (__bf16*)dv, s.Lq, s.Lk, s.Hq, s.Hk, G, nkhb, sl2, scale, s.layout, nb, plan,
                       nkb, 0);
    hipLaunchKernelGGL((bwd_sparse_reduce_kernel<D>), dim3(1024), dim3(256), 0, stream, plan, nb, s.Lk, s.Hk,
                       (__bf16*)dk, (__bf16*)dv, scale, 0, 0, 0);
  } else if (dkdv_split(s)) {
    SparsePlan plan;
    workspace_layout(s, false, &plan, reinterpret_cast<char*>(delta));
    const int ncol = nkb * nkhb;
    const int ck = dkdv_chunk_t(s);
    const int items = ck ? nkhb * chunk_prefix(nkb, ck) : 2 * ncol;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, false, true>), dim3((unsigned)items), dim3(512), 0,
                       stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dk, (__bf16*)dv, s.Lq, s.Lk, s.Hq, s.Hk, G, nkhb, sl2, scale, nullptr, 0, plan,
                       nkb, ck);
    hipLaunchKernelGGL((bwd_sparse_reduce_kernel<D, true>), dim3(1024), dim3(256), 0, stream, plan, nkhb, s.Lk,
                       s.Hk, (__bf16*)dk, (__bf16*)dv, scale, ncol, nkb, ck);
  } else {
    const unsigned grid = xcd_run_grid((long long)nkb * nkhb, 32);   // whole rounds of 256 jobs
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, false>), dim3(grid), dim3(512), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dk, (__bf16*)dv, s.Lq, s.Lk, s.Hq, s.Hk, G, nkhb, sl2, scale, nullptr, 0,
                       SparsePlan{}, nkb, 0);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nhb = s.B * s.Hq;
  const int nqb = (s.Lq + 127) / 128;
  const DqChunks dc = dq_chunks(s);
  if (s.layout)
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, true>), dim3((unsigned)nqb * nhb), dim3(256), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dq, s.Lq, s.Lk, s.Hq, s.Hk, G, nqb, nhb, sl2, scale, s.layout, nb, 0, nullptr);
  else if (dc.items) {
    float* part = nullptr;
    workspace_layout(s, false, nullptr, reinterpret_cast<char*>(delta), &part);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, false, 1, true>), dim3((unsigned)dc.items), dim3(256), 0,
                       stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dq, s.Lq, s.Lk, s.Hq, s.Hk, G, nqb, nhb, sl2, scale, nullptr, 0, dc.ck, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned units = (unsigned)nqb * nhb * (128 * D / 1024);
    hipLaunchKernelGGL((bwd_dq_reduce_kernel<D, CAUSAL>), dim3(std::min(units, 2048u)), dim3(256), 0, stream, part,
                       (__bf16*)dq, s.Lq, s.Hq, nqb, nhb, dc.ck, scale);
  } else if ((int64_t)nqb * nhb < (CAUSAL ? kDqSplitCausalBelow : kDqSplitFullUpTo + 1))
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, false, 2>), dim3((unsigned)nqb * nhb), dim3(512), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dq, s.Lq, s.Lk, s.Hq, s.Hk, G, nqb, nhb, sl2, scale, nullptr, 0, 0, nullptr);
  else {
    const int nqb2 = (s.Lq + 255) / 256;
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, false, 1, false, 8>),
                       dim3(xcd_run_grid((long long)nqb2 * nhb, kDqXcdRun)), dim3(512), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)d_o, lse, delta,
                       (__bf16*)dq, s.Lq, s.Lk, s.Hq, s.Hk, G, nqb2, nhb, sl2, scale, nullptr, 0, 0, nullptr);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* d_o,
                   const float* lse, float* dq, float* dk, float* dv, float* delta, const AttnShape& s,
                   hipStream_t stream) {
  hipError_t e = launch_delta<float, D>(o, d_o, delta, s, stream);
  if (e != hipSuccess) return e;
  const int G = s.Hq / s.Hk;
  const float scale = 1.f / sqrtf((float)D);
  const float sl2 = kLog2e * scale;
  const int nkhb = s.B * s.Hk;
  const int nkb = (s.Lk + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, 0>), dim3((unsigned)nkb * nkhb), dim3(256), 0, stream, q, k,
                     v, d_o, lse, delta, dv, s.Lq, s.Lk, s.Hq, s.Hk, G, nkhb, sl2, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, 1>), dim3((unsigned)nkb * nkhb), dim3(256), 0, stream, q, k,
                     v, d_o, lse, delta, dk, s.Lq, s.Lk, s.Hq, s.Hk, G, nkhb, sl2, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nhb = s.B * s.Hq;
  const int nqb = (s.Lq + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)nqb * nhb), dim3(256), 0, stream, q, k, v,
                     d_o, lse, delta, dq, s.Lq, s.Lk, s.Hq, s.Hk, G, nqb, nhb, sl2, scale);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape& s, bool sparse) {
  return workspace_layout(s, sparse, nullptr, nullptr);
}

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                const AttnShape& s, hipStream_t stream) {
  float* delta = static_cast<float*>(workspace);
  if (s.D == 128)
    return s.causal ? bwd_bf16<128, true>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream)
                    : bwd_bf16<128, false>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream);
  return s.causal ? bwd_bf16<64, true>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream)
                  : bwd_bf16<64, false>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream);
}

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* d_o,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace,
                               const AttnShape& s, hipStream_t stream) {
  float* delta = static_cast<float*>(workspace);
  if (s.D == 128)
    return s.causal ? bwd_f32<128, true>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream)
                    : bwd_f32<128, false>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream);
  return s.causal ? bwd_f32<64, true>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream)
                  : bwd_f32<64, false>(q, k, v, o, d_o, lse, dq, dk, dv, delta, s, stream);
}

}  // namespace ulysses
