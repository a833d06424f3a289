// seq <-> head layout change over P virtual ranks (the two all-to-alls of one
// attention block, done as on-device permutations).
//
// "Ulysses Sequence Parallelism: A Temporary Change of Layout" (pinyu.ai),
// section "Use the other independent axis": each sender cuts its heads into P
// groups and each receiver concatenates the token blocks it gets in sender
// order; paper-graph summary of arXiv 2309.14509, section 3.4.1: contiguous
// token chunks before, contiguous head groups after.
//
// Both directions are one 5-D axis permutation whose innermost run is one
// (token, head-group) slab of H/P * d_h elements: 128 B .. 1 KiB for the
// supported d_h and dtypes, always a whole number of 128-byte lines. The
// kernel therefore copies 16-byte words straight from HBM to HBM: a wave's
// 64 lanes move 1 KiB of consecutive words of the tensor it walks, which on
// the other side form runs of at least 128 contiguous bytes, so every line
// read and written is a full line. Staging through LDS adds a round trip
// without making any access wider (measured: LDS-staged tiles were no
// faster). Values are never converted; bits are copied as they are. The
// kernel walks the seq-layout tensor in order (seq_to_head reads it,
// head_to_seq writes it) except for seq_to_head with runs of 256 bytes or
// less, which walks the head layout (gathering its runs and writing in
// order): with 32 destination groups of 256-byte runs that measured 2 %
// faster than scattering them.
//
// K/V heads of grouped-query attention (pinyu.ai, section "Head-count
// constraints"): with fewer K/V heads than ranks, every rank receives the one
// K/V head its query heads share, so each head group goes to rep = P / H_kv
// consecutive ranks. The same kernel writes each word it reads rep times.
// The gradient of that gather sums the rep replicas back into their token
// shards (kv_grad_reduce_kernel): the only arithmetic in this file.
#include "common.h"
#include "kernels.h"

namespace ulysses {

namespace {

// One wave per workgroup and one 16-byte word per lane: 1 KiB per workgroup.
// Many small workgroups keep more independent streams in flight than a few
// large ones (measured on the 1 GiB tensor of the 131K-token GPT-7B shape:
// 83 % of HBM peak against 70-78 % for 256 threads x 1-4 words).
constexpr int kThreads = 64;
constexpr int kUnroll = 1;
// seq_to_head walking the head layout (runs of 256 bytes or less) in
// workgroups of 4 waves instead: at 1M tokens (32 head groups of 256-byte
// runs) 6.31-6.34 TB/s against 6.04-6.10 with one wave, while 128, 192,
// 320, 384, 512 and 1024 threads all measured 5.4-6.0 TB/s, and the other
// forms lose with larger workgroups.
constexpr int kWalkThreads = 256;

// The kernel walks one tensor's words in order ("own" index) and computes
// where each word sits in the other tensor:
//   scatter: read src[own], write dst[other] (rep copies, srep apart);
//   gather:  read src[other], write dst[own].
struct PermArgs {
  const u32x4* __restrict__ src;
  u32x4* __restrict__ dst;
  uint32_t total;            // 16-byte words walked
  FastDiv fU, f3, f2, f1;    // extents of the walked tensor: [n0][n1][n2][n3][U]
  uint32_t s0, s1, s2, s3;   // strides (words) in the other tensor of coords i0..i3
  uint32_t rep, srep;        // copies of each word and the distance between them (scatter)
};

template <bool GATHER, int THREADS>
__global__ __launch_bounds__(THREADS) void perm_kernel(PermArgs a) {
  const uint32_t base = blockIdx.x * (THREADS * kUnroll) + threadIdx.x;
  u32x4 val[kUnroll];
  uint32_t dsto[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t idx = base + u * THREADS;
    if (!GATHER && idx < a.total) val[u] = __builtin_nontemporal_load(a.src + idx);
    const uint32_t run = fdiv(idx, a.fU);
    const uint32_t w = idx - run * a.fU.d;
    const uint32_t t3 = fdiv(run, a.f3);
    const uint32_t i3 = run - t3 * a.f3.d;
    const uint32_t t2 = fdiv(t3, a.f2);
    const uint32_t i2 = t3 - t2 * a.f2.d;
    const uint32_t i0 = fdiv(t2, a.f1);
    const uint32_t i1 = t2 - i0 * a.f1.d;
    dsto[u] = i0 * a.s0 + i1 * a.s1 + i2 * a.s2 + i3 * a.s3 + w;
    if (GATHER && idx < a.total) val[u] = __builtin_nontemporal_load(a.src + dsto[u]);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t idx = base + u * THREADS;
    if (idx < a.total) {
      if (GATHER)
        __builtin_nontemporal_store(val[u], a.dst + idx);
      else
        for (uint32_t j = 0; j < a.rep; ++j) __builtin_nontemporal_store(val[u], a.dst + dsto[u] + j * a.srep);
    }
  }
}

// dst [r][b][t][g][w] = sum over j < rep of src [g*rep + j][b][r*Lp + t][w]
// (one head per rank in src, G = P / rep heads in dst); one thread per
// destination word, replicas summed in order in fp32.
struct ReduceArgs {
  const u32x4* __restrict__ src;
  u32x4* __restrict__ dst;
  uint32_t total;            // destination words
  FastDiv fU, fG, fLp, fB;   // destination extents [P][B][Lp][G][U]
  uint32_t rep;
  uint32_t sp, sb, sn;       // source strides (words) of rank, batch, token
};

template <bool BF16>
__global__ __launch_bounds__(kThreads) void kv_grad_reduce_kernel(ReduceArgs a) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= a.total) return;
  const uint32_t run = fdiv(idx, a.fU);
  const uint32_t w = idx - run * a.fU.d;
  const uint32_t t2 = fdiv(run, a.fG);
  const uint32_t g = run - t2 * a.fG.d;
  const uint32_t t3 = fdiv(t2, a.fLp);
  const uint32_t t = t2 - t3 * a.fLp.d;
  const uint32_t r = fdiv(t3, a.fB);
  const uint32_t b = t3 - r * a.fB.d;
  const u32x4* s = a.src + (g * a.rep) * a.sp + b * a.sb + (r * a.fLp.d + t) * a.sn + w;
  constexpr int N = BF16 ? 8 : 4;
  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.f;
  for (uint32_t j = 0; j < a.rep; ++j) {
    const u32x4 x = s[j * a.sp];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t bits = BF16 ? ((x[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16 : x[i];
      acc[i] += __uint_as_float(bits);
    }
  }
  u32x4 out;
  if (BF16) {
    bf16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (__bf16)acc[i];  // round to nearest even
    out = __builtin_bit_cast(u32x4, h);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __float_as_uint(acc[i]);
  }
  a.dst[idx] = out;
}

}  // namespace

hipError_t launch_seq_head_perm(const void* src, void* dst, const PermShape& s, bool seq_to_head,
                                hipStream_t stream) {
  const uint32_t U = s.run_bytes / 16;  // words per (token, head-group) slab
  const uint32_t P = s.P, B = s.B, Lp = s.Lp;
  PermArgs a;
  a.src = static_cast<const u32x4*>(src);
  a.dst = static_cast<u32x4*>(dst);
  a.total = s.total_words;
  a.fU = make_fastdiv(U);
  a.rep = 1;
  a.srep = 0;
  // By default both directions walk the seq-layout tensor [r][b][t][g][w] (g: head group,
  // P / rep of them) and find the word in the head-layout tensor
  // [g*rep + j][b][r][t][w]: seq_to_head scatters (rep copies), head_to_seq
  // gathers. Either way the seq-layout side is read or written in order and
  // the head-layout side in runs of U words.
  const uint32_t rank_words = B * P * Lp * U;
  a.f1 = make_fastdiv(B);
  a.f2 = make_fastdiv(Lp);
  a.f3 = make_fastdiv(P / s.rep);
  a.s0 = Lp * U;             // r
  a.s1 = P * Lp * U;         // b
  a.s2 = U;                  // t
  a.s3 = s.rep * rank_words; // g
  a.rep = s.rep;
  a.srep = rank_words;
  // seq_to_head with short runs walks the head layout [g][b][r][t][w] in
  // order instead, gathering from the seq layout (strides below)
  const bool head_walk = seq_to_head && s.rep == 1 && U <= 16;
  if (head_walk) {
    const uint32_t G = P;
    a.f1 = make_fastdiv(B);    // extents [g][b][r][t][w]
    a.f2 = make_fastdiv(P);
    a.f3 = make_fastdiv(Lp);
    a.s0 = U;                  // g
    a.s1 = Lp * G * U;         // b
    a.s2 = B * Lp * G * U;     // r
    a.s3 = G * U;              // t
  }
  // the walked tensor is the source (scatter) or the destination (gather)
  if (head_walk) {
    const uint32_t blocks = (a.total + kWalkThreads * kUnroll - 1) / (kWalkThreads * kUnroll);
    hipLaunchKernelGGL((perm_kernel<true, kWalkThreads>), dim3(blocks), dim3(kWalkThreads), 0, stream, a);
    return hipGetLastError();
  }
  const uint32_t blocks = (a.total + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (seq_to_head)
    hipLaunchKernelGGL((perm_kernel<false, kThreads>), dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((perm_kernel<true, kThreads>), dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_grad_reduce(const void* src, void* dst, const PermShape& s, bool bf16, hipStream_t stream) {
  const uint32_t U = s.run_bytes / 16;  // words per (token, head)
  const uint32_t P = s.P, B = s.B, Lp = s.Lp, G = s.P / s.rep;
  ReduceArgs a;
  a.src = static_cast<const u32x4*>(src);
  a.dst = static_cast<u32x4*>(dst);
  a.total = s.total_words;
  a.fU = make_fastdiv(U);
  a.fG = make_fastdiv(G);
  a.fLp = make_fastdiv(Lp);
  a.fB = make_fastdiv(B);
  a.rep = s.rep;
  a.sn = U;
  a.sb = P * Lp * U;
  a.sp = B * P * Lp * U;
  const uint32_t blocks = (a.total + kThreads - 1) / kThreads;
  if (bf16)
    hipLaunchKernelGGL(kv_grad_reduce_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_grad_reduce_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ulysses
