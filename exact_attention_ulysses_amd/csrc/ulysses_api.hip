// C ABI of the library: argument validation (before any HIP call) and
// dispatch to the kernels. See include/ulysses.h for the contract.
#include <string.h>


#include "../../include/ulysses.h"
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

// common size checks; returns OK or the status to report
int check_dims(int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int dtype) {
  if (B <= 0 || L <= 0 || H <= 0 || d_h <= 0 || P <= 0) return ULYSSES_INVALID_ARGUMENT;
  if (!valid_dtype(dtype)) return ULYSSES_UNSUPPORTED;
  if (H % P != 0) return ULYSSES_NOT_DIVISIBLE;
  if (!valid_head_dim(d_h)) return ULYSSES_UNSUPPORTED;
  // every product below stays far from int64 overflow once each factor is capped
  if (B > (int64_t(1) << 30) || L > (int64_t(1) << 30) || H > (int64_t(1) << 20)) return ULYSSES_UNSUPPORTED;
  const int64_t words = B * L * H * d_h * elem_size(dtype) / 16;
  if (words >= kMaxWords) return ULYSSES_UNSUPPORTED;
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
  return report(launch_seq_head_perm(src, dst, s, seq_to_head, static_cast<hipStream_t>(stream)));
}

int attn_dims(int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int causal, int dtype, AttnShape* s) {
  int st = check_dims(B, L, H, d_h, P, dtype);
  if (st != ULYSSES_OK) return st;
  if (causal != 0 && causal != 1) return ULYSSES_INVALID_ARGUMENT;
  const int64_t Hh = H / P;
  if (B * Hh > (int64_t(1) << 24) || B * L * Hh >= (int64_t(1) << 31)) return ULYSSES_UNSUPPORTED;
  // the kernels address one head's rows (plus a padded last tile) with 32-bit byte offsets
  if ((L + 256) * Hh * d_h * elem_size(dtype) >= (int64_t(1) << 32)) return ULYSSES_UNSUPPORTED;
  s->B = (int)B;
  s->L = (int)L;
  s->Hh = (int)Hh;
  s->D = (int)d_h;
  s->causal = causal == 1;
  return ULYSSES_OK;
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

int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t L,
                     int64_t H, int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return ULYSSES_INVALID_ARGUMENT;
  AttnShape s;
  int st = attn_dims(B, L, H, d_h, P, causal, dtype, &s);
  if (st != ULYSSES_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ULYSSES_MISALIGNED;
  const int64_t tb = B * L * (H / P) * d_h * elem_size(dtype);
  const int64_t lb = B * (H / P) * L * 4;
  const Range ro = range_of(o, tb), rl = range_of(lse, lb);
  const Range rin[3] = {range_of(q, tb), range_of(k, tb), range_of(v, tb)};
  for (const Range& r : rin)
    if (overlap(ro, r) || overlap(rl, r)) return ULYSSES_ALIASING;
  if (overlap(ro, rl)) return ULYSSES_ALIASING;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ULYSSES_BF16) return report(launch_attn_fwd_bf16(q, k, v, o, lse, s, hs));
  return report(launch_attn_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lse, s, hs));
}

size_t ulysses_attn_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P, int causal,
                                        int dtype) {
  AttnShape s;
  if (attn_dims(B, L, H, d_h, P, causal, dtype, &s) != ULYSSES_OK) return 0;
  return attn_bwd_workspace_bytes(s);
}

int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t L,
                     int64_t H, int64_t d_h, int64_t P, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv || !workspace) return ULYSSES_INVALID_ARGUMENT;
  AttnShape s;
  int st = attn_dims(B, L, H, d_h, P, causal, dtype, &s);
  if (st != ULYSSES_OK) return st;
  const void* al16[] = {q, k, v, o, d_o, dq, dk, dv, workspace};
  for (const void* p : al16)
    if (!aligned(p, 16)) return ULYSSES_MISALIGNED;
  if (!aligned(lse, 4)) return ULYSSES_MISALIGNED;
  const size_t need = attn_bwd_workspace_bytes(s);
  if (workspace_bytes < need) return ULYSSES_WORKSPACE_TOO_SMALL;
  const int64_t tb = B * L * (H / P) * d_h * elem_size(dtype);
  const int64_t lb = B * (H / P) * L * 4;
  const Range outs[4] = {range_of(dq, tb), range_of(dk, tb), range_of(dv, tb), range_of(workspace, (int64_t)need)};
  const Range ins[6] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(o, tb), range_of(d_o, tb),
                        range_of(lse, lb)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ULYSSES_ALIASING;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return ULYSSES_ALIASING;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dtype == ULYSSES_BF16)
    return report(launch_attn_bwd_bf16(q, k, v, o, d_o, lse, dq, dk, dv, workspace, s, hs));
  return report(launch_attn_bwd_f32((const float*)q, (const float*)k, (const float*)v, (const float*)o,
                                    (const float*)d_o, lse, (float*)dq, (float*)dk, (float*)dv, workspace, s, hs));
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
