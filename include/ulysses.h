/*
 * ulysses.h -- C ABI of the Ulysses per-rank hot path on one AMD Instinct
 * MI355X (gfx950): the sequence<->head layout change over P virtual ranks and
 * exact full-sequence attention (forward and backward) on one rank's heads.
 *
 * Sources of the operations (web pages on DeepSpeed-Ulysses, arXiv 2309.14509):
 *  - "Ulysses Sequence Parallelism: A Temporary Change of Layout" (pinyu.ai):
 *    sections "Use the other independent axis" and "One attention block, end
 *    to end" give the layout change [B, L/P, H, d_h] -> [B, L, H/P, d_h] and
 *    back, and section "Head-count constraints" the rule H % P == 0.
 *  - paper-graph summary of arXiv 2309.14509, section 3.4.1: contiguous token
 *    chunks before the change, contiguous head groups after it; section 3.2
 *    item 3 and 3.4.5: per-head scaled dot-product attention, causal or not,
 *    on the full sequence with no communication.
 *  - papers.chlience.com reading note, section 5.1: O'_p = softmax(Q'_p K'_p^T /
 *    sqrt(d_h)) V'_p on rank p's head group; section 5.4: cross-attention
 *    among the attention kinds the method carries.
 *  - pinyu.ai, "Head-count constraints", and the aifetchly blog, "Practical
 *    Deployment Checklist for Long-Context Training": grouped-query /
 *    multi-query attention has fewer K/V heads than query heads; they split
 *    over P ranks when H_kv % P == 0, and otherwise each rank holds a replica
 *    of the K/V head its query heads use.
 *
 * Conventions shared by every entry point
 *  - Element types: ULYSSES_BF16 (bfloat16) or ULYSSES_FP32. The layout
 *    changes move raw bits and accept either. bf16 attention accumulates in
 *    fp32 and rounds its outputs to nearest-even bf16.
 *  - Dense row-major layouts, all pointers are device pointers:
 *      seq buffer  [P][B][L/P][H][d_h]   (rank-major token shards; for B = 1
 *                                         byte-identical to a global [1][L][H][d_h])
 *      head buffer [P][B][L][H/P][d_h]   (rank p holds heads p*H/P .. (p+1)*H/P-1)
 *      attention operands: ONE rank's head block [B][L][H/P][d_h]; pass B*P as B
 *      with the whole head buffer to run every rank's head group at once.
 *      lse         [B][H/P][L] float32, natural-log log-sum-exp of each query
 *                  row's scaled scores.
 *  - Causal: key j is visible to query i iff j <= i, on global token positions.
 *    Scale: exactly 1/sqrt(d_h).
 *  - Ownership: the caller allocates and owns every buffer, the workspace
 *    included. The library never allocates, frees or synchronises; all work is
 *    enqueued on `stream` (a hipStream_t passed as void*, NULL = null stream)
 *    in stream order, so outputs are ready when the stream reaches that point.
 *    Inputs are read only. Outputs must not overlap inputs or each other.
 *  - Errors: every function returns a ulysses_status. Arguments are validated
 *    before any HIP call, so a rejected call touches no device state. After
 *    validation a launch failure reported by the runtime returns
 *    ULYSSES_HIP_ERROR; faults inside a kernel surface at the caller's next
 *    synchronisation, as usual for asynchronous work.
 *  - Limits: d_h in {64, 128}; any L >= 1 (partial tiles are masked); each
 *    tensor below 32 GiB; for attention, one batch entry of each tensor (L *
 *    heads * d_h elements, plus 256 rows of slack) below 4 GiB, and B * L *
 *    heads < 2^31.
 *    Calls outside these limits return ULYSSES_UNSUPPORTED.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ulysses_status {
  ULYSSES_OK = 0,
  ULYSSES_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad flag */
  ULYSSES_NOT_DIVISIBLE = 2,      /* H % P != 0 or L % P != 0 (or a head-count rule of GQA) */
  ULYSSES_UNSUPPORTED = 3,        /* d_h or dtype or size outside what the kernels implement */
  ULYSSES_MISALIGNED = 4,         /* a pointer not 16-byte aligned */
  ULYSSES_ALIASING = 5,           /* an output overlaps an input or another output */
  ULYSSES_WORKSPACE_TOO_SMALL = 6,
  ULYSSES_HIP_ERROR = 7           /* the HIP runtime rejected a launch */
} ulysses_status;

typedef enum ulysses_dtype {
  ULYSSES_BF16 = 0,
  ULYSSES_FP32 = 1
} ulysses_dtype;

/*
 * First all-to-all of one attention block, as an on-device permutation over P
 * virtual ranks: x_seq [P][B][L/P][H][d_h] -> x_head [P][B][L][H/P][d_h], with
 *   x_head[p][b][r*L/P + t][j][:] = x_seq[r][b][t][p*H/P + j][:].
 * Every sender r cuts its local heads into P groups; receiver p concatenates
 * the token blocks it gets, in sender order (pinyu.ai, "Use the other
 * independent axis"; paper-graph summary, section 3.4.1). Bits are copied
 * unchanged (NaN payloads included). Not in place: x_head must not overlap x_seq.
 */
int ulysses_seq_to_head(const void* x_seq, void* x_head,
                        int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                        int dtype, void* stream);

/*
 * Second all-to-all, the inverse permutation: x_head [P][B][L][H/P][d_h] ->
 * x_seq [P][B][L/P][H][d_h], with
 *   x_seq[r][b][t][p*H/P + j][:] = x_head[p][b][r*L/P + t][j][:]
 * (pinyu.ai, "One attention block, end to end", step 4; paper-graph summary,
 * section 3.4.1, "After attention: the reverse transformation").
 */
int ulysses_head_to_seq(const void* x_head, void* x_seq,
                        int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                        int dtype, void* stream);

/*
 * First all-to-all for the K or V tensor of grouped-query attention with H_kv
 * key/value heads (pinyu.ai, "Head-count constraints"). Let Hl = H_kv / P if
 * H_kv % P == 0, else Hl = 1 (then P % H_kv must be 0, and R = P / H_kv
 * consecutive ranks receive the same head). x_seq [P][B][L/P][H_kv][d_h] ->
 * x_head [P][B][L][Hl][d_h]:
 *   H_kv % P == 0:  exactly ulysses_seq_to_head with H = H_kv;
 *   otherwise:      x_head[p][b][r*L/P + t][0][:] = x_seq[r][b][t][p / R][:].
 * With these K/V heads, rank p's query heads p*H_q/P .. (p+1)*H_q/P - 1 find
 * their shared K/V head (h / (H_q/H_kv)) locally. x_head is R times the size
 * of x_seq. Bits are copied unchanged. Not in place. ULYSSES_NOT_DIVISIBLE if
 * L % P != 0 or neither of H_kv, P divides the other.
 */
int ulysses_seq_to_head_kv(const void* x_seq, void* x_head,
                           int64_t B, int64_t L, int64_t H_kv, int64_t d_h, int64_t P,
                           int dtype, void* stream);

/*
 * Gradient of ulysses_seq_to_head_kv (its adjoint): dx_head [P][B][L][Hl][d_h]
 * -> dx_seq [P][B][L/P][H_kv][d_h]. Without replication this is exactly
 * ulysses_head_to_seq with H = H_kv (bits copied). With replication the R
 * replicas of a head are summed:
 *   dx_seq[r][b][t][g][:] = sum_{j<R} dx_head[g*R + j][b][r*L/P + t][0][:],
 * accumulated in fp32 in the order j = 0..R-1 and rounded once to `dtype`
 * (round to nearest even for bf16).
 */
int ulysses_head_to_seq_kv_grad(const void* dx_head, void* dx_seq,
                                int64_t B, int64_t L, int64_t H_kv, int64_t d_h, int64_t P,
                                int dtype, void* stream);

/*
 * Exact attention on one rank's head group (papers.chlience.com note,
 * section 5.1; paper-graph summary, sections 3.2 and 3.4.5):
 *   O = softmax(Q K^T / sqrt(d_h)) V  per (batch, local head), full length L,
 * causal (causal = 1) or bidirectional (causal = 0). q, k, v, o are
 * [B][L][H/P][d_h] of `dtype`; lse [B][H/P][L] float32 receives
 * m_i + ln(sum_j exp(S_ij - m_i)) over the visible keys of row i, which the
 * backward pass uses to recompute the probabilities.
 * Results are bitwise reproducible for identical calls. The kernels pick
 * their schedule from the launch size: launches of a few hundred query
 * blocks or fewer split each row's key walk in two or four (forward), and
 * the backward cuts the walks of small launches into halves or chunks whose
 * partial sums are added in a fixed order (dQ, dK/dV). Calls that differ in
 * B, heads or L may therefore round an element differently in the last
 * bits; the attention entry points below behave the same way.
 */
int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                     int causal, int dtype, void* stream);

/*
 * Gradient of the attention above w.r.t. q, k, v given dO = d_o (the pages
 * train with the method but leave its backward implicit; this is the exact
 * gradient). With P_ij = exp(S_ij - lse_i) recomputed from the saved lse:
 *   D_i = sum_e dO_ie O_ie, dV = P^T dO, dS = P o (dO V^T - D),
 *   dQ = dS K / sqrt(d_h), dK = dS^T Q / sqrt(d_h).
 * All tensors [B][L][H/P][d_h] of `dtype` except lse (as written by
 * ulysses_attn_fwd for the same q, k, v). `workspace` is device scratch of at
 * least ulysses_attn_bwd_workspace_bytes(...) bytes, 256-byte aligned,
 * owned by the caller; its contents on entry do not matter.
 */
int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                     int causal, int dtype, void* stream);

/*
 * Workspace ulysses_attn_bwd needs for these sizes (0 if the sizes are
 * invalid): delta [B][H/P][L] fp32; for bf16 launches of few key-block
 * columns (B x local heads x ceil(L / 128): causal below 512, bidirectional
 * up to 128) two fp32 partial sums [dK | dV][128][d_h] per column, so that
 * two workgroups can share each column's walk; and for bf16 launches of few
 * 128-row query blocks (fewer than 2048 over B x local heads, where cutting
 * the blocks' key walks into chunks pays) one fp32 [128][d_h] partial sum per
 * chunk, at most 2048 chunks (128 MiB at d_h = 128).
 */
size_t ulysses_attn_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t d_h,
                                        int64_t P, int causal, int dtype);

/*
 * ulysses_attn_bwd for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it): the
 * same arguments without the workspace. Delta and the partial sums of split
 * walks live in a fixed scratch array of the library, 64 MiB per device,
 * held from the first call on a device until the process ends. Launches
 * whose split walks would not fit beside delta take the whole-walk kernels
 * instead, so results may differ from ulysses_attn_bwd in the last bits
 * (same tolerance). Delta must fit: B * (H/P) * L <= 16,777,216 rows, else
 * ULYSSES_WORKSPACE_TOO_SMALL (before any HIP call). The call allocates and
 * frees nothing. Every call on one device shares that device's scratch:
 * calls that overlap on one device (two streams, two threads) race and must
 * be serialised by the caller. Nothing in the scratch needs clearing between
 * calls; every byte a call reads was written earlier in the same call.
 */
int ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const void* d_o, const float* lse,
                             void* dq, void* dk, void* dv,
                             int64_t B, int64_t L, int64_t H, int64_t d_h, int64_t P,
                             int causal, int dtype, void* stream);

/*
 * ulysses_attn_fwd generalised to grouped-query attention and to queries and
 * keys of different lengths (cross-attention). H_q query heads, H_kv K/V heads
 * (global counts; H_q % P == 0, H_q % H_kv == 0, and H_kv % P == 0 or
 * P % H_kv == 0, else ULYSSES_NOT_DIVISIBLE). One rank's buffers:
 *   q, o   [B][L_q][H_q/P][d_h]       lse [B][H_q/P][L_q] float32
 *   k, v   [B][L_kv][Hl][d_h]         Hl as in ulysses_seq_to_head_kv
 * Local query head j uses local K/V head j / (H_q/P / Hl), i.e. global query
 * head h uses K/V head h / (H_q/H_kv). causal = 1 requires L_q == L_kv
 * (ULYSSES_UNSUPPORTED otherwise). With H_q == H_kv and L_q == L_kv this is
 * ulysses_attn_fwd.
 */
int ulysses_attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t L_q, int64_t L_kv, int64_t H_q, int64_t H_kv,
                         int64_t d_h, int64_t P, int causal, int dtype, void* stream);

/*
 * Gradient of ulysses_attn_fwd_gqa. dq has q's layout; dk, dv have k's, and a
 * K/V head shared by several query heads receives the sum of their
 * contributions (accumulated in fp32, rounded once). Workspace as for
 * ulysses_attn_bwd, sized by ulysses_attn_bwd_gqa_workspace_bytes.
 */
int ulysses_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                         const void* d_o, const float* lse,
                         void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t L_q, int64_t L_kv, int64_t H_q, int64_t H_kv,
                         int64_t d_h, int64_t P, int causal, int dtype, void* stream);

/* Workspace ulysses_attn_bwd_gqa needs for these sizes (0 if the sizes are invalid). */
size_t ulysses_attn_bwd_gqa_workspace_bytes(int64_t B, int64_t L_q, int64_t L_kv, int64_t H_q,
                                            int64_t H_kv, int64_t d_h, int64_t P, int causal,
                                            int dtype);

/*
 * Block-sparse attention: ulysses_attn_fwd_gqa / ulysses_attn_bwd_gqa (self-
 * attention, L_q = L_kv = L) restricted to the (query block, key block) pairs a
 * block layout marks. The pages run "blocked sparse attention" after the same
 * all-to-all and note that each rank, holding the full sequence of its heads,
 * applies the sparsity pattern locally (paper-graph summary, section 3.4 and
 * Figs 6-7); they do not fix the pattern, so the layout is an argument.
 *   layout  device uint8 [H_q/P][nb][nb], nb = ceil(L / block), row-major, one
 *           per local query head and shared by the batch: entry (h, i, j) != 0
 *           lets the queries of block i attend the keys of block j. Read only.
 *   block   tokens per layout block; 128 is the only supported value.
 * Key j is visible to query i iff layout[h][i / block][j / block] != 0 and,
 * with causal = 1, j <= i (entries above the block diagonal are then ignored).
 * A query row that sees no key gets O = 0 and lse = -inf, and passes no
 * gradient. bf16 only (ULYSSES_UNSUPPORTED otherwise). The backward pass also
 * needs (H_q/H_kv) <= 8 and (H_q/H_kv) * nb <= 8192 (UNSUPPORTED otherwise)
 * and a workspace of at least ulysses_attn_bwd_block_sparse_workspace_bytes
 * bytes (ULYSSES_WORKSPACE_TOO_SMALL otherwise): besides the per-row delta it
 * holds each layout column's list of active (query head, query block) pairs
 * (2 bytes per layout entry), a work plan that cuts key blocks attended by
 * many query blocks into chunks handled by separate workgroups, and at most
 * 512 fp32 partial-sum slots of 2 x 128 x d_h that a last pass adds in a
 * fixed order, so results do not depend on scheduling. Only the active blocks
 * are computed.
 */
int ulysses_attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const uint8_t* layout, int64_t block,
                                  int64_t B, int64_t L, int64_t H_q, int64_t H_kv, int64_t d_h, int64_t P,
                                  int causal, int dtype, void* stream);

int ulysses_attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                                  const void* d_o, const float* lse,
                                  void* dq, void* dk, void* dv,
                                  const uint8_t* layout, int64_t block,
                                  void* workspace, size_t workspace_bytes,
                                  int64_t B, int64_t L, int64_t H_q, int64_t H_kv, int64_t d_h, int64_t P,
                                  int causal, int dtype, void* stream);

/* Workspace bytes for ulysses_attn_bwd_block_sparse with these sizes; 0 if
 * they are invalid or unsupported. */
size_t ulysses_attn_bwd_block_sparse_workspace_bytes(int64_t B, int64_t L, int64_t H_q, int64_t H_kv,
                                                     int64_t d_h, int64_t P, int64_t block, int causal,
                                                     int dtype);

/* Static, NUL-terminated name of a status code ("ULYSSES_OK", ...). */
const char* ulysses_status_string(int status);

/* Text of the last HIP error this thread saw inside the library, or "". */
const char* ulysses_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
