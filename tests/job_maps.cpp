// Host-side check of the kernels' work decomposition (compiled for the host
// only, no GPU): the index helpers the kernels use to turn a workgroup index
// into its job are exercised over whole launches and checked against plain
// arithmetic.
//   fdiv                  n / d without a divide (layout changes, tile walks)
//   xcd_run_block         dense attention jobs (block rank, head pair) in XCD runs
//   causal_chunk_item     chunked causal walks: work item -> (block, head pair, part)
//   causal_chunk_first    where a reduce kernel finds a block's parts
// Prints one line per family and "ok" at the end; exits non-zero at the first
// mismatch, naming it.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "common.h"

using namespace ulysses;

static int fail(const char* what, long long a, long long b, long long c, long long d) {
  std::printf("FAIL %s: %lld %lld %lld %lld\n", what, a, b, c, d);
  std::exit(1);
}

static void check_fdiv() {
  std::mt19937_64 rng(12345);
  long long n_checked = 0;
  auto one = [&](uint32_t n, uint32_t d, const FastDiv& f) {
    if (fdiv(n, f) != n / d) fail("fdiv", n, d, fdiv(n, f), n / d);
    ++n_checked;
  };
  std::vector<uint32_t> divisors;
  for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
  for (int i = 0; i < 2000; ++i) divisors.push_back(uint32_t(rng() % 0xFFFFFFFFull) + 1);
  for (int s = 12; s < 32; ++s) {   // powers of two and their neighbours
    divisors.push_back(1u << s);
    divisors.push_back((1u << s) - 1);
    divisors.push_back((1u << s) + 1);
  }
  divisors.push_back(0xFFFFFFFFu);
  for (const uint32_t d : divisors) {
    const FastDiv f = make_fastdiv(d);
    for (const uint32_t n : {0u, 1u, d - 1, d, d + 1, 0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFEu, 0xFFFFFFFFu}) one(n, d, f);
    // the multiples of d and their neighbours, where a rounding error would show
    for (int i = 0; i < 64; ++i) {
      const uint64_t k = rng() % (0xFFFFFFFFull / d + 1);
      const uint64_t m = k * d;
      for (const int64_t delta : {-1, 0, 1}) {
        const int64_t n = int64_t(m) + delta;
        if (n >= 0 && n <= 0xFFFFFFFFll) one(uint32_t(n), d, f);
      }
      one(uint32_t(rng()), d, f);
    }
  }
  std::printf("fdiv: %lld quotients over %zu divisors\n", n_checked, divisors.size());
}

static void check_xcd_runs() {
  long long launches = 0;
  std::vector<int> seen;
  auto launch = [&](int run, int nhb, int nranks) {
    const long long jobs = (long long)nhb * nranks;
    const unsigned grid = xcd_run_grid(jobs, run);
    if (grid % (8 * run) != 0 || grid < jobs || grid >= jobs + 8 * run) fail("xcd_run_grid", run, nhb, nranks, grid);
    seen.assign((size_t)jobs, 0);
    long long taken = 0;
    for (unsigned bid = 0; bid < grid; ++bid) {
      int rank = -1, hb = -1;
      if (!xcd_run_block((int)bid, run, nhb, nranks, &rank, &hb)) continue;
      if (rank < 0 || rank >= nranks || hb < 0 || hb >= nhb) fail("xcd_run_block range", run, nhb, nranks, bid);
      if (seen[(size_t)rank * nhb + hb]++) fail("xcd_run_block twice", run, nhb, rank, hb);
      ++taken;
    }
    if (taken != jobs) fail("xcd_run_block coverage", run, nhb, nranks, taken);
    ++launches;
  };
  for (const int run : {16, 32, 64}) {   // the runs the kernels take, and one more
    for (int nhb = 1; nhb <= 40; ++nhb)
      for (int nranks = 1; nranks <= 160; ++nranks) launch(run, nhb, nranks);
    for (const int nhb : {48, 64, 96, 128, 256, 512, 1024})
      for (const int nranks : {1, 2, 3, 31, 64, 127})
        launch(run, nhb, nranks);
    for (const int nhb : {1, 2, 4, 8})
      for (const int nranks : {1000, 4096, 8191})
        launch(run, nhb, nranks);
  }
  std::printf("xcd_run_block: %lld launches, every job once\n", launches);
}

static void check_causal_chunks() {
  long long launches = 0;
  for (int nblk = 1; nblk <= 96; ++nblk) {
    for (int t = 1; t <= nblk; ++t) {
      // S(m) against its definition
      int s = 0;
      for (int x = 1; x <= nblk; ++x) {
        s += (x + t - 1) / t;
        if (chunk_prefix(x, t) != s) fail("chunk_prefix", x, t, chunk_prefix(x, t), s);
      }
      for (const int nhb : {1, 2, 3, 4, 7, 8}) {
        const int items = nhb * chunk_prefix(nblk, t);
        int prev_x = nblk + 1;
        std::vector<int> seen((size_t)(nblk + 1) * nhb * nblk, 0);
        for (int i = 0; i < items; ++i) {
          int x, hb, chunk, nchunk;
          causal_chunk_item(i, nblk, nhb, t, &x, &hb, &chunk, &nchunk);
          if (x < 1 || x > nblk || hb < 0 || hb >= nhb) fail("causal_chunk_item range", nblk, t, nhb, i);
          if (nchunk != (x + t - 1) / t || chunk < 0 || chunk >= nchunk) fail("causal_chunk_item parts", nblk, t, i, chunk);
          if (x > prev_x) fail("causal_chunk_item order (longest first)", nblk, t, nhb, i);
          prev_x = x;
          // the reduce kernels find this part at causal_chunk_first + chunk
          if (causal_chunk_first(x, hb, nblk, nhb, t) + chunk != i) fail("causal_chunk_first", nblk, t, nhb, i);
          if (seen[((size_t)x * nhb + hb) * nblk + chunk]++) fail("causal_chunk_item twice", nblk, t, nhb, i);
        }
        // every block's every part exactly once
        long long want = 0;
        for (int x = 1; x <= nblk; ++x) want += (long long)nhb * ((x + t - 1) / t);
        if (want != items) fail("causal_chunk_item count", nblk, t, nhb, items);
        ++launches;
      }
    }
  }
  std::printf("causal_chunk_item / causal_chunk_first: %lld launches, every part once\n", launches);
}

int main() {
  check_fdiv();
  check_xcd_runs();
  check_causal_chunks();
  std::printf("ok\n");
  return 0;
}
