// Internal launcher declarations (validated arguments only). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ulysses {

struct PermShape {
  uint32_t P, B, Lp;       // ranks, batch, tokens per rank
  uint32_t run_bytes;      // local heads * d_h * element size (multiple of 128)
  uint32_t total_words;    // seq-layout tensor size in 16-byte words (< 2^31)
  uint32_t rep;            // ranks that receive each head group (1, or P / H_kv for
                           // replicated K/V heads); the head tensor is rep times larger
};

// seq_to_head (rep copies of every head group) or head_to_seq (rep must be 1)
hipError_t launch_seq_head_perm(const void* src, void* dst, const PermShape& s, bool seq_to_head,
                                hipStream_t stream);
// head_to_seq for gradients of replicated K/V heads: the rep replicas are summed
// (fp32 accumulation, one rounding to the element type)
hipError_t launch_kv_grad_reduce(const void* src, void* dst, const PermShape& s, bool bf16, hipStream_t stream);

struct AttnShape {
  int B;        // batch (times ranks when several head groups run at once)
  int Lq, Lk;   // query rows and key rows (equal for self-attention; causal needs equal)
  int Hq;       // heads in the query-side buffers q, o, d_o, dq (and lse, delta)
  int Hk;       // heads in the key-side buffers k, v, dk, dv; query head h uses
                // key head h / (Hq / Hk)
  int D;        // head dim (64 or 128)
  bool causal;
  bool bf16 = true;   // element type bf16 (else fp32)
  // block-sparse attention (bf16 only): per local query head uint8 layout
  // [Hq][nb][nb] over 128-token blocks, nb = ceil(L / 128); nullptr = dense
  const uint8_t* layout = nullptr;
  // backward only: upper bound on the workspace (0 = none). A dense bf16
  // launch then leaves out the split walks whose partial sums would not fit
  // and takes the whole-walk kernels instead; delta always has to fit.
  size_t ws_cap = 0;
};

// bf16 operands, fp32 lse
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                const AttnShape& s, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               const AttnShape& s, hipStream_t stream);

// workspace layout: delta [B][Hq][Lq] fp32; with a block layout also the
// backward's work plan and partial-sum slots; for dense bf16 launches of few
// key blocks the partial sums of their split key-block walks (all 256-byte
// aligned)
size_t attn_bwd_workspace_bytes(const AttnShape& s, bool sparse);
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const void* d_o, const float* lse, void* dq, void* dk, void* dv,
                                void* workspace, const AttnShape& s, hipStream_t stream);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                               const float* d_o, const float* lse, float* dq, float* dk, float* dv,
                               void* workspace, const AttnShape& s, hipStream_t stream);

}  // namespace ulysses
