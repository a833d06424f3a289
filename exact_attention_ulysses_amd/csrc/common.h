// Internal helpers of the HIP library (gfx950 only). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulysses {

// ---------------------------------------------------------------------------
// vector types for MFMA operands and wide memory access
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// division by a runtime constant without a hardware divide: q = n / d for
// n < 2^32, with m = ceil(2^(32+s) / d) - 2^32 (Granlund & Montgomery 1994,
// "Division by invariant integers using multiplication", round-up variant).
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t s;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  f.s = s;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = uint32_t((uint64_t(n) * f.m) >> 32);   // high half of the product (v_mul_hi_u32)
  return uint32_t((uint64_t(t) + n) >> f.s);
}

// ---------------------------------------------------------------------------
// XCD-aware job order. The eight XCDs of the chip each have their own L2, and
// workgroup i of a launch runs on XCD i mod 8. Attention workgroups that walk
// the same tiles at the same time share them through the L2 only when they
// sit on one XCD, so this map gives each XCD runs of `run` consecutive jobs
// (run = the workgroups an XCD holds at once), the XCDs taking the runs of a
// round of 8 * run jobs in alternating directions to keep their work even
// when jobs shrink (longest first). Launches round their grid up to whole
// rounds; workgroups past the last job exit at once.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int xcd_run_job(int bid, int run) {
  const int x = bid & 7, j = bid >> 3;
  const int round = j / run;
  return 8 * run * round + run * ((round & 1) ? 7 - x : x) + (j - round * run);
}

__host__ __device__ inline unsigned xcd_run_grid(long long jobs, int run) {
  return (unsigned)((jobs + 8LL * run - 1) / (8LL * run) * (8LL * run));
}

// Jobs (block rank, head pair hb), the ranks longest first: job j is rank
// j / nhb of head pair j % nhb. With xcd_run_job's runs, a round of
// 8 * run consecutive jobs holds (8 * run) / nhb ranks of every head pair;
// when nhb divides the round they are taken head by head, so that a run is
// consecutive ranks of one head pair (each XCD then streams the tiles of
// one head) rather than every head's at once. Returns false past the last
// job.
__host__ __device__ __forceinline__ bool xcd_run_block(int bid, int run, int nhb, int nranks, int* rank, int* hb) {
  const int j = xcd_run_job(bid, run);
  const int span = 8 * run;
  if (span % nhb == 0) {
    const int round = j / span, i = j - round * span, per = span / nhb;
    *hb = i / per;
    *rank = round * per + (i - *hb * per);
  } else {
    *rank = j / nhb;
    *hb = j - *rank * nhb;
  }
  return *rank < nranks;
}

// ---------------------------------------------------------------------------
// Chunked causal walks. Under the causal mask query block x - 1 (x = 1 ..
// nblk) walks a number of key tiles proportional to x; cutting it into
// ceil(x / t) near-equal parts bounds every part by the length of t blocks'
// worth of diagonal. Work items are numbered blocks longest first, head pairs
// inner, a block's parts consecutive.
// S(m) = sum over x = 1..m of ceil(x / t): the parts of blocks 0..m-1.
// ---------------------------------------------------------------------------
__host__ __device__ inline int chunk_prefix(int m, int t) {
  const int a = m / t, r = m - a * t;
  return t * a * (a + 1) / 2 + r * (a + 1);
}

// First work item of block x - 1, head pair hb: the items of the longer
// blocks x + 1 .. nblk come first (nhb (S(nblk) - S(x)) of them), then the
// ceil(x / t) parts of each head pair before hb. Reduce kernels read a
// block's parts from here on.
__host__ __device__ inline int causal_chunk_first(int x, int hb, int nblk, int nhb, int t) {
  return nhb * (chunk_prefix(nblk, t) - chunk_prefix(x, t)) + hb * ((x + t - 1) / t);
}

// Work item i of nhb * S(nblk): block x - 1 (returned as x), head pair hb,
// part `chunk` of nchunk = ceil(x / t). The items before block x number
// nhb (S(nblk) - S(x)); x is the smallest block whose predecessors number at
// most i.
__host__ __device__ inline void causal_chunk_item(int i, int nblk, int nhb, int t, int* x, int* hb, int* chunk,
                                                  int* nchunk) {
  const int sn = chunk_prefix(nblk, t);
  int lo = 1, hi = nblk;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (nhb * (sn - chunk_prefix(mid, t)) <= i)
      hi = mid;
    else
      lo = mid + 1;
  }
  *x = lo;
  *nchunk = (lo + t - 1) / t;
  const int loc = i - nhb * (sn - chunk_prefix(lo, t));
  *hb = loc / *nchunk;
  *chunk = loc - *hb * *nchunk;
}

// ---------------------------------------------------------------------------
// launch-side error reporting (thread-local last error text)
// ---------------------------------------------------------------------------
void set_last_hip_error(hipError_t e);

}  // namespace ulysses
