// C ABI of the library: argument validation (before any HIP call) and
// dispatch to the kernels. See include/ulysses.h for the contract.
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/ulysses.h"
#include "block_sparse.h"
#include "common.h"
#include "kernels.h"

namespace ulysses {

namespace {
thread_local char g_last_hip_error[256] = "";

constexpr int64_t kMaxWords = int64_t(1) << 31;  // 16-byte words per tensor (32 GiB)

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

inline bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

inline int64_t elem_size(int dtype) { return dtype == ULYSSES_FP32 ? 4 : 2; }

inline bool valid_dtype(int dtype) { return dtype == ULYSSES_BF16 || dtype == ULYSSES_FP32; }

inline bool valid_head_dim(int64_t d) { return d == 64 || d == 128; }

// The product of positive factors is at most cap (checked factor by factor,
// so that no partial product can overflow).
inline bool product_at_most(std::initializer_list<int64_t> factors, int64_t cap) {
  int64_t p = 1;
  for (const int64_t f : factors) {
    if (p > cap / f) return false;
    p *= f;
  }
  return true;
}

// common size checks; returns OK or the status to report
int check_dims(int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int dtype) {
  if (B <= 0 || L <= 0 || H <= 0 || d_h <= 0 || P <= 0) return ULYSSES_INVALID_ARGUMENT;
  if (!valid_dtype(dtype)) return ULYSSES_UNSUPPORTED;
  if (H % P != 0) return ULYSSES_NOT_DIVISIBLE;
  if (!valid_head_dim(d_h)) return ULYSSES_UNSUPPORTED;
  if (B > (int64_t(1) << 30) || L > (int64_t(1) << 30) || H > (int64_t(1) << 20)) return ULYSSES_UNSUPPORTED;
  // each tensor below 32 GiB (kMaxWords 16-byte words)
  if (!product_at_most({B, L, H, d_h, elem_size(dtype)}, kMaxWords * 16 - 1)) return ULYSSES_UNSUPPORTED;
  return ULYSSES_OK;
}

int report(hipError_t e) {
  if (e == hipSuccess) return ULYSSES_OK;
  set_last_hip_error(e);
  return ULYSSES_HIP_ERROR;
}

int perm_entry(const void* src, void* dst, int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int dtype,
               void* stream, bool seq_to_head) {
  if (!src || !dst) return ULYSSES_INVALID_ARGUMENT;
  int st = check_dims(B, L, H, d_h, P, dtype);
  if (st != ULYSSES_OK) return st;
  if (L % P != 0) return ULYSSES_NOT_DIVISIBLE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return ULYSSES_MISALIGNED;
  const int64_t bytes = B * L * H * d_h * elem_size(dtype);
  if (overlap(range_of(src, bytes), range_of(dst, bytes))) return ULYSSES_ALIASING;
  PermShape s;
  s.P = (uint32_t)P;
  s.B = (uint32_t)B;
  s.Lp = (uint32_t)(L / P);
  s.run_bytes = (uint32_t)(H / P * d_h * elem_size(dtype));
  s.total_words = (uint32_t)(bytes / 16);
  s.rep = 1;
  return report(launch_seq_head_perm(src, dst, s, seq_to_head, static_cast<hipStream_t>(stream)));
}

// K/V heads per rank after the layout change: H_kv / P when the heads split
// evenly, else 1 (replicated over P / H_kv ranks); 0 when neither divides.
int64_t kv_local_heads(int64_t Hkv, int64_t P) {
  if (Hkv % P == 0) return Hkv / P;
  if (P % Hkv == 0) return 1;
  return 0;
}

// K/V layout change (replicating) and its gradient (summing replicas)
int kv_perm_entry(const void* src, void* dst, int64_t B, int64_t L, int64_t Hkv, int64_t d_h, int64_t P, int dtype,
                  void* stream, bool seq_to_head) {
  if (!src || !dst) return ULYSSES_INVALID_ARGUMENT;
  if (B <= 0 || L <= 0 || Hkv <= 0 || d_h <= 0 || P <= 0) return ULYSSES_INVALID_ARGUMENT;
  if (!valid_dtype(dtype)) return ULYSSES_UNSUPPORTED;
  const int64_t Hl = kv_local_heads(Hkv, P);
  if (Hl == 0 || L % P != 0) return ULYSSES_NOT_DIVISIBLE;
  if (!valid_head_dim(d_h)) return ULYSSES_UNSUPPORTED;
  if (B > (int64_t(1) << 30) || L > (int64_t(1) << 30) || Hkv > (int64_t(1) << 20) || P > (int64_t(1) << 20))
    return ULYSSES_UNSUPPORTED;
  const int64_t es = elem_size(dtype);
  // the head-side tensor (rep times the seq side) below 32 GiB
  if (!product_at_most({P, B, L, Hl, d_h, es}, kMaxWords * 16 - 1)) return ULYSSES_UNSUPPORTED;
  const int64_t seq_bytes = B * L * Hkv * d_h * es;
  const int64_t head_bytes = P * B * L * Hl * d_h * es;   // = seq_bytes * rep
  if (!aligned(src, 16) || !aligned(dst, 16)) return ULYSSES_MISALIGNED;
  const int64_t src_bytes = seq_to_head ? seq_bytes : head_bytes;
  const int64_t dst_bytes = seq_to_head ? head_bytes : seq_bytes;
  if (overlap(range_of(src, src_bytes), range_of(dst, dst_bytes))) return ULYSSES_ALIASING;
  PermShape s;
  s.P = (uint32_t)P;
  s.B = (uint32_t)B;
  s.Lp = (uint32_t)(L / P);
  s.run_bytes = (uint32_t)(Hl * d_h * es);
  s.total_words = (uint32_t)(seq_bytes / 16);
  s.rep = (uint32_t)(P * Hl / Hkv);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (seq_to_head || s.rep == 1) return report(launch_seq_head_perm(src, dst, s, seq_to_head, hs));
  return report(launch_kv_grad_reduce(src, dst, s, dtype == ULYSSES_BF16, hs));
}

// Attention sizes: B batch, Lq query rows, Lk key rows, Hq / Hkv global query /
// key-value heads, P ranks; the buffers hold one rank's Hq / P query heads and
// its K/V heads (kv_local_heads).
int attn_dims(int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t d_h, int64_t P, int causal,
              int dtype, AttnShape* s) {
  if (B <= 0 || Lq <= 0 || Lk <= 0 || Hq <= 0 || Hkv <= 0 || d_h <= 0 || P <= 0) return ULYSSES_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return ULYSSES_INVALID_ARGUMENT;
  if (!valid_dtype(dtype)) return ULYSSES_UNSUPPORTED;
  if (Hq % P != 0 || Hq % Hkv != 0 || kv_local_heads(Hkv, P) == 0) return ULYSSES_NOT_DIVISIBLE;
  if (!valid_head_dim(d_h)) return ULYSSES_UNSUPPORTED;
  // the causal mask is defined on a shared token axis (self-attention)
  if (causal == 1 && Lq != Lk) return ULYSSES_UNSUPPORTED;
  if (B > (int64_t(1) << 30) || Lq > (int64_t(1) << 30) || Lk > (int64_t(1) << 30) || Hq > (int64_t(1) << 20))
    return ULYSSES_UNSUPPORTED;
  const int64_t Hql = Hq / P, Hkl = kv_local_heads(Hkv, P), es = elem_size(dtype);
  if (B * Hql > (int64_t(1) << 24) || B * Lq * Hql >= (int64_t(1) << 31) || B * Lk * Hkl >= (int64_t(1) << 31))
    return ULYSSES_UNSUPPORTED;
  // each tensor below 32 GiB (this also keeps every grid below 2^32 work-items)
  if (B * Lq * Hql * d_h * es / 16 >= kMaxWords || B * Lk * Hkl * d_h * es / 16 >= kMaxWords)
    return ULYSSES_UNSUPPORTED;
  // the kernels address one batch's rows (plus a padded last tile) with 32-bit byte offsets
  if ((Lq + 256) * Hql * d_h * es >= (int64_t(1) << 32) || (Lk + 256) * Hkl * d_h * es >= (int64_t(1) << 32))
    return ULYSSES_UNSUPPORTED;
  s->B = (int)B;
  s->Lq = (int)Lq;
  s->Lk = (int)Lk;
  s->Hq = (int)Hql;
  s->Hk = (int)Hkl;
  s->D = (int)d_h;
  s->causal = causal == 1;
  s->bf16 = dtype == ULYSSES_BF16;
  return ULYSSES_OK;
}

int64_t q_bytes(const AttnShape& s, int dtype) { return (int64_t)s.B * s.Lq * s.Hq * s.D * elem_size(dtype); }
int64_t k_bytes(const AttnShape& s, int dtype) { return (int64_t)s.B * s.Lk * s.Hk * s.D * elem_size(dtype); }
int64_t lse_bytes(const AttnShape& s) { return (int64_t)s.B * s.Hq * s.Lq * 4; }

// Block layouts: 128-token blocks, bf16, self-attention; the dK/dV kernel's
// pair list bounds the query heads per K/V head and the blocks per column.
int sparse_supported(int64_t block, int64_t Lq, int64_t Lk, int dtype, const AttnShape& s, bool backward) {
  if (block != kSparseBlock || dtype != ULYSSES_BF16 || Lq != Lk) return ULYSSES_UNSUPPORTED;
  const int64_t nb = (Lk + kSparseBlock - 1) / kSparseBlock, G = s.Hq / s.Hk;
  if (backward && (G > kMaxSparseGroup || G * nb > kMaxSparsePairs)) return ULYSSES_UNSUPPORTED;
  return ULYSSES_OK;
}

int sparse_dims(const uint8_t* layout, int64_t block, int64_t Lq, int64_t Lk, int dtype, AttnShape* s,
                bool backward) {
  if (!layout) return ULYSSES_INVALID_ARGUMENT;
  const int st = sparse_supported(block, Lq, Lk, dtype, *s, backward);
  if (st != ULYSSES_OK) return st;
  s->layout = layout;
  return ULYSSES_OK;
}

int64_t layout_bytes(const AttnShape& s) {
  const int64_t nb = (s.Lk + kSparseBlock - 1) / kSparseBlock;
  return (int64_t)s.Hq * nb * nb;
}

int attn_fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Lq,
                   int64_t Lk, int64_t Hq, int64_t Hkv, int64_t d_h, int64_t P, int causal, int dtype,
                   void* stream, const uint8_t* layout = nullptr, int64_t block = 0) {
  if (!q || !k || !v || !o || !lse) return ULYSSES_INVALID_ARGUMENT;
  AttnShape s;
  int st = attn_dims(B, Lq, Lk, Hq, Hkv, d_h, P, causal, dtype, &s);
  if (st != ULYSSES_OK) return st;
  if (block != 0 || layout) {
    st = sparse_dims(layout, block, Lq, Lk, dtype, &s, false);
    if (st != ULYSSES_OK) return st;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ULYSSES_MISALIGNED;
  const int64_t tq = q_bytes(s, dtype), tk = k_bytes(s, dtype);
  const Range ro = range_of(o, tq), rl = range_of(lse, lse_bytes(s));
  const Range rin[4] = {range_of(q, tq), range_of(k, tk), range_of(v, tk),
                        range_of(layout, layout ? layout_bytes(s) : 0)};
  for (const Range& r : rin)
    if (overlap(ro, r) || overlap(rl, r)) return ULYSSES_ALIASING;
  if (overlap(ro, rl)) return ULYSSES_ALIASING;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ULYSSES_BF16) return report(launch_attn_fwd_bf16(q, k, v, o, lse, s, hs));
  return report(launch_attn_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, s, hs));
}

size_t attn_ws_entry(int64_t B, int64_t Lq, int64_t Lk, int64_t Hq, int64_t Hkv, int64_t d_h, int64_t P,
                     int causal, int dtype) {
  AttnShape s;
  if (attn_dims(B, Lq, Lk, Hq, Hkv, d_h, P, causal, dtype, &s) != ULYSSES_OK) return 0;
  return attn_bwd_workspace_bytes(s, false);
}

// Validation of a backward call (no HIP call): fills the shape; the
// workspace is checked against the planner's need unless it is the library's
// own scratch (workspace == nullptr, capped at ws_cap).
int attn_bwd_check(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t Lq,
                   int64_t Lk, int64_t Hq, int64_t Hkv, int64_t d_h, int64_t P, int causal, int dtype,
                   const uint8_t* layout, int64_t block, size_t ws_cap, AttnShape* sp) {
  AttnShape& s = *sp;
  int st = attn_dims(B, Lq, Lk, Hq, Hkv, d_h, P, causal, dtype, &s);
  if (st != ULYSSES_OK) return st;
  s.ws_cap = ws_cap;
  if (block != 0 || layout) {
    st = sparse_dims(layout, block, Lq, Lk, dtype, &s, true);
    if (st != ULYSSES_OK) return st;
  }
  const void* al16[] = {q, k, v, o, d_o, dq, dk, dv, workspace};
  for (const void* p : al16)
    if (!aligned(p, 16)) return ULYSSES_MISALIGNED;
  if (!aligned(lse, 4)) return ULYSSES_MISALIGNED;
  const size_t need = attn_bwd_workspace_bytes(s, layout != nullptr);
  if (workspace ? workspace_bytes < need : need > ws_cap) return ULYSSES_WORKSPACE_TOO_SMALL;
  const int64_t tq = q_bytes(s, dtype), tk = k_bytes(s, dtype);
  const Range outs[4] = {range_of(dq, tq), range_of(dk, tk), range_of(dv, tk),
                         range_of(workspace, workspace ? (int64_t)need : 0)};
  const Range ins[7] = {range_of(q, tq), range_of(k, tk), range_of(v, tk), range_of(o, tq), range_of(d_o, tq),
                        range_of(lse, lse_bytes(s)), range_of(layout, layout ? layout_bytes(s) : 0)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ULYSSES_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return ULYSSES_ALIASING;
  }
  return ULYSSES_OK;
}

int attn_bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                    void* dq, void* dk, void* dv, void* workspace, const AttnShape& s, int dtype, void* stream) {
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ULYSSES_BF16)
    return report(launch_attn_bwd_bf16(q, k, v, o, d_o, lse, dq, dk, dv, workspace, s, hs));
  return report(launch_attn_bwd_f32((const float*)q, (const float*)k, (const float*)v, (const float*)o,
                                    (const float*)d_o, lse, (float*)dq, (float*)dk, (float*)dv, workspace, s, hs));
}

int attn_bwd_entry(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t Lq,
                   int64_t Lk, int64_t Hq, int64_t Hkv, int64_t d_h, int64_t P, int causal, int dtype,
                   void* stream, const uint8_t* layout = nullptr, int64_t block = 0) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv || !workspace) return ULYSSES_INVALID_ARGUMENT;
  AttnShape s;
  const int st = attn_bwd_check(q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, Lq, Lk, Hq, Hkv,
                                d_h, P, causal, dtype, layout, block, 0, &s);
  if (st != ULYSSES_OK) return st;
  return attn_bwd_launch(q, k, v, o, d_o, lse, dq, dk, dv, workspace, s, dtype, stream);
}

// Scratch of the backward entry point that allocates nothing: delta and the
// partial sums of split walks live here instead of in a caller's workspace.
// The array's name is a host-side stand-in in host code; kernels get the
// device address that hipGetSymbolAddress returns for the device at hand.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.
int scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return report(e);
  if (dev < 0 || dev >= kMaxDevices) return ULYSSES_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return report(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return report(e);
    void* p = nullptr;
    const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return report(e);
    if (eg != hipSuccess) return report(eg);
    if (!p) return ULYSSES_HIP_ERROR;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ULYSSES_OK;
}

// ulysses_attn_bwd with the library's scratch as the workspace: the planner
// is capped at the scratch size, so only delta has to fit. Every argument is
// validated before the first HIP call (the device lookup).
int attn_bwd_noalloc_entry(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                           const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t L, int64_t H,
                           int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return ULYSSES_INVALID_ARGUMENT;
  AttnShape s;
  int st = attn_bwd_check(q, k, v, o, d_o, lse, dq, dk, dv, nullptr, 0, B, L, L, H, H, d_h, P, causal, dtype,
                          nullptr, 0, kScratchBytes, &s);
  if (st != ULYSSES_OK) return st;
  void* ws = nullptr;
  st = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (st != ULYSSES_OK) return st;
  return attn_bwd_launch(q, k, v, o, d_o, lse, dq, dk, dv, ws, s, dtype, stream);
}

}  // namespace

void set_last_hip_error(hipError_t e) {
  strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
}

}  // namespace ulysses

using namespace ulysses;

extern "C" {

int ulysses_seq_to_head(const void* x_seq, void* x_head, int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                        int dtype, void* stream) {
  return perm_entry(x_seq, x_head, B, L, H, d_h, P, dtype, stream, true);
}

int ulysses_head_to_seq(const void* x_head, void* x_seq, int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                        int dtype, void* stream) {
  return perm_entry(x_head, x_seq, B, L, H, d_h, P, dtype, stream, false);
}

int ulysses_seq_to_head_kv(const void* x_seq, void* x_head, int64_t B, int64_t L, int64_t H_kv, int64_t d_h,
                           int64_t P, int dtype, void* stream) {
  return kv_perm_entry(x_seq, x_head, B, L, H_kv, d_h, P, dtype, stream, true);
}

int ulysses_head_to_seq_kv_grad(const void* dx_head, void* dx_seq, int64_t B, int64_t L, int64_t H_kv, int64_t d_h,
                                int64_t P, int dtype, void* stream) {
  return kv_perm_entry(dx_head, dx_seq, B, L, H_kv, d_h, P, dtype, stream, false);
}

int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t L,
                     int64_t H, int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  return attn_fwd_entry(q, k, v, o, lse, B, L, L, H, H, d_h, P, causal, dtype, stream);
}

int ulysses_attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t L_q,
                         int64_t L_kv, int64_t H_q, int64_t H_kv, int64_t d_h, int64_t P, int causal, int dtype,
                         void* stream) {
  return attn_fwd_entry(q, k, v, o, lse, B, L_q, L_kv, H_q, H_kv, d_h, P, causal, dtype, stream);
}

size_t ulysses_attn_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int causal,
                                        int dtype) {
  return attn_ws_entry(B, L, L, H, H, d_h, P, causal, dtype);
}

size_t ulysses_attn_bwd_gqa_workspace_bytes(int64_t B, int64_t L_q, int64_t L_kv, int64_t H_q, int64_t H_kv,
                                            int64_t d_h, int64_t P, int causal, int dtype) {
  return attn_ws_entry(B, L_q, L_kv, H_q, H_kv, d_h, P, causal, dtype);
}

size_t ulysses_attn_bwd_block_sparse_workspace_bytes(int64_t B, int64_t L, int64_t H_q, int64_t H_kv, int64_t d_h,
                                                     int64_t P, int64_t block, int causal, int dtype) {
  AttnShape s;
  if (attn_dims(B, L, L, H_q, H_kv, d_h, P, causal, dtype, &s) != ULYSSES_OK) return 0;
  if (sparse_supported(block, L, L, dtype, s, true) != ULYSSES_OK) return 0;
  return attn_bwd_workspace_bytes(s, true);
}

int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t L,
                     int64_t H, int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  return attn_bwd_entry(q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, L, L, H, H, d_h, P, causal,
                        dtype, stream);
}

int ulysses_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t L_q, int64_t L_kv, int64_t H_q, int64_t H_kv, int64_t d_h, int64_t P,
                         int causal, int dtype, void* stream) {
  return attn_bwd_entry(q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, L_q, L_kv, H_q, H_kv, d_h,
                        P, causal, dtype, stream);
}

int ulysses_attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const uint8_t* layout, int64_t block, int64_t B, int64_t L, int64_t H_q,
                                  int64_t H_kv, int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  if (!layout) return ULYSSES_INVALID_ARGUMENT;
  return attn_fwd_entry(q, k, v, o, lse, B, L, L, H_q, H_kv, d_h, P, causal, dtype, stream, layout, block);
}

int ulysses_attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                                  const float* lse, void* dq, void* dk, void* dv, const uint8_t* layout,
                                  int64_t block, void* workspace, size_t workspace_bytes, int64_t B, int64_t L,
                                  int64_t H_q, int64_t H_kv, int64_t d_h, int64_t P, int causal, int dtype,
                                  void* stream) {
  if (!layout) return ULYSSES_INVALID_ARGUMENT;
  return attn_bwd_entry(q, k, v, o, d_o, lse, dq, dk, dv, workspace, workspace_bytes, B, L, L, H_q, H_kv, d_h, P,
                        causal, dtype, stream, layout, block);
}

int ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                             const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t L, int64_t H,
                             int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  return attn_bwd_noalloc_entry(q, k, v, o, d_o, lse, dq, dk, dv, B, L, H, d_h, P, causal, dtype, stream);
}

const char* ulysses_status_string(int status) {
  switch (status) {
    case ULYSSES_OK: return "ULYSSES_OK";
    case ULYSSES_INVALID_ARGUMENT: return "ULYSSES_INVALID_ARGUMENT";
    case ULYSSES_NOT_DIVISIBLE: return "ULYSSES_NOT_DIVISIBLE";
    case ULYSSES_UNSUPPORTED: return "ULYSSES_UNSUPPORTED";
    case ULYSSES_MISALIGNED: return "ULYSSES_MISALIGNED";
    case ULYSSES_ALIASING: return "ULYSSES_ALIASING";
    case ULYSSES_WORKSPACE_TOO_SMALL: return "ULYSSES_WORKSPACE_TOO_SMALL";
    case ULYSSES_HIP_ERROR: return "ULYSSES_HIP_ERROR";
    default: return "ULYSSES_UNKNOWN_STATUS";
  }
}

const char* ulysses_last_hip_error(void) { return ulysses::g_last_hip_error; }

}  // extern "C"
