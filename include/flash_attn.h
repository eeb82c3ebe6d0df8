/*
 * flash_attn.h -- C ABI of libflashattn.so: exact softmax attention on one
 * AMD MI355X (gfx950), computed tile by tile with the online softmax so that
 * the N x N score matrix never exists in device memory.
 *
 * What is computed (per batch b and query head hq, with K/V head
 * g = hq / (Hq / Hkv)):
 *   S   = scale * Q K^T                 score equation of mentria.ai "Exact
 *                                       attention, sped up by never writing the
 *                                       giant grid down", card "So don't load it
 *                                       all. Work one block at a time."
 *   S_ij = -inf for j > i when causal   the mask step of fanfani.net
 *                                       "FlashAttention", section "The
 *                                       bottleneck was never the arithmetic"
 *   P   = row-wise softmax(S)           mentria.ai, card "But softmax needs the
 *                                       whole row at once."
 *   O   = P V                           (same fanfani.net section)
 *   lse = ln(sum_j exp(S_ij))           the per-query statistics kept for the
 *                                       backward, fanfani.net section "The
 *                                       backward pass, and where the memory
 *                                       saving comes from"; P_ij = exp(S_ij - lse_i)
 * O is reached by the running max / running normaliser / rescaled running
 * output recurrence of fanfani.net section "A pinch of math: making the
 * softmax work in pieces", dividing by the normaliser once at the end. The
 * backward recomputes each score block from Q, K and lse (same "backward
 * pass" section; synthetic.wiki "FlashAttention: attention's bottleneck is
 * the wire, not the maths", section "The backward pass buys memory with
 * recompute") and returns the chain-rule gradients of sum(dO * O).
 *
 * Layout: every tensor is dense row-major.
 *   q, o, dout, dq : [B, Hq,  N, d]
 *   k, v, dk, dv   : [B, Hkv, N, d]
 *   lse            : [B, Hq,  N]      float32, natural-log units of the scaled scores
 * Grouped K/V heads (GQA, MQA when Hkv == 1; synthetic.wiki page, section
 * "Versions, and what the numbers say"): query head hq reads K/V head
 * hq / (Hq / Hkv); Hq must be a multiple of Hkv.
 * Head dims: d in {64, 128, 256} (the same section: head dims up to 256).
 * Causal mask: key j is visible to query i iff j <= i (0-based, queries and
 * keys both of length N).
 *
 * Element types: the plain entry points take bf16 tensors as raw 16-bit
 * patterns (uint16 storage; torch.bfloat16 storage is exactly this) and
 * accumulate in fp32; P is rounded to bf16 (round to nearest even) before the
 * P V product and O, dq, dk, dv are rounded to bf16 on store. The _f32 entry
 * points are an fp32 check mode: the same kernels with fp32 storage and fp32
 * matrix-core products, for tight comparison against a reference.
 *
 * Ownership: every pointer is a device pointer owned by the caller (the
 * backward workspace included). The library never allocates, frees or keeps
 * device memory and keeps no state between calls: it is reentrant. Outputs
 * must not alias inputs. All pointers must be 16-byte aligned.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising. The caller orders and
 * synchronises; the next use of the outputs must be on `stream` or after it.
 *
 * Errors: every argument is checked on the host before any HIP call; a
 * non-zero fa_status is returned and nothing is enqueued. After the launches,
 * a failing hipGetLastError gives FA_ERR_HIP. Nothing is printed, thrown or
 * aborted across this boundary. flash_attn_status_str names a status.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, Hq, Hkv or N <= 0, Hq % Hkv != 0, or a size overflows int32 indexing */
  FA_ERR_UNSUPPORTED = 3, /* d not in {64, 128, 256}, or causal not 0/1 */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  FA_ERR_SCALE = 5,       /* scale is not finite or is negative */
  FA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  FA_ERR_WORKSPACE = 7,   /* a required workspace is NULL or smaller than its *_workspace_bytes */
  FA_ERR_SCRATCH = 8      /* flash_attn_fwd_kv_noalloc: the split partials exceed FLASH_ATTN_SCRATCH_BYTES */
} fa_status;

/*
 * Forward, bf16 storage, fp32 accumulation.
 *   q [B,Hq,N,d], k, v [B,Hkv,N,d]: inputs (bf16 bits).
 *   o [B,Hq,N,d]: output (bf16 bits).
 *   lse [B,Hq,N]: output (fp32), ln of the softmax denominator of each row of
 *     scale*QK^T (masked), i.e. lse_i = max_j S_ij + ln(sum_j exp(S_ij - max_j S_ij)).
 *   scale: finite, >= 0 (1/sqrt(d) for standard attention; 0 gives uniform weights).
 *   causal: 0 or 1.
 * Returns FA_OK or an fa_status (see above).
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream);

/* Forward, fp32 check mode: as flash_attn_fwd with fp32 q, k, v, o. */
int flash_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * General forward, bf16 storage: rectangular problems, split keys, and
 * variable-length batches. Same operation as flash_attn_fwd per (sequence,
 * query head), with these differences:
 *   - Nq queries and Nk keys per sequence; the causal mask is aligned to the
 *     bottom right: query i sees key j iff j <= i + Nk - Nq, so the last query
 *     sees every key (with Nq == Nk this is flash_attn_fwd's mask). A query
 *     that sees no key (causal with Nq > Nk) gets O = 0 and lse = -inf.
 *   - Split keys (decoding: few queries, a long key/value cache): the keys of
 *     each sequence are cut into num_splits ranges, each range gives a
 *     partial result (o/l in fp32 and its lse) in the workspace, and a second
 *     kernel merges them with the online softmax's rescale step (fanfani.net
 *     "FlashAttention", section "A pinch of math: making the softmax work in
 *     pieces": a partial enters like one block whose maximum is its lse and
 *     whose exponential sum is 1). The result equals the unsplit one up to
 *     fp32 rounding order.
 *   - The G = Hq/Hkv query heads of a K/V head share each staged K/V block.
 *
 * flash_attn_fwd_kv: uniform lengths.
 *   q, o [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] (bf16 bits), lse [B,Hq,Nq] fp32.
 * flash_attn_fwd_varlen: B sequences packed along the token axis.
 *   q, o [Hq,Tq,d], k, v [Hkv,Tk,d] (bf16 bits), lse [Hq,Tq] fp32;
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B+1], non-decreasing, from 0 to
 *   Tq (resp. Tk): sequence b owns query tokens cu_seqlens_q[b] ..
 *   cu_seqlens_q[b+1]-1 and key tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.
 *   max_seqlen_q / max_seqlen_k: upper bounds of the per-sequence lengths (they
 *   size the launch). Offsets are clamped into [0, T] on the device, so any
 *   contents keep every access in bounds; results are defined for offsets
 *   that rise from 0 to T with sequences of at most max_seqlen tokens, and
 *   tokens outside every sequence are left unspecified.
 * num_splits: 1 = no split; 0 = the library's choice
 *   (flash_attn_fwd_kv_num_splits); at most 256.
 * workspace: caller-owned device buffer of flash_attn_fwd_kv_workspace_bytes(
 *   rows, d, splits) bytes, rows = B*Hq*Nq (uniform) or Hq*Tq (varlen), with
 *   the split count actually used; NULL is allowed when that is 1. Contents on
 *   entry ignored, on return unspecified.
 * Errors as flash_attn_fwd; FA_ERR_SHAPE also for num_splits outside
 * [0, 256] or a launch beyond 65536 x 65535 workgroups, FA_ERR_WORKSPACE
 * for a missing or short workspace.
 */
int flash_attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                          int Tq, int Tk, int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * flash_attn_fwd_kv without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it. Same
 * arguments, result and errors as flash_attn_fwd_kv (the caller still passes
 * q, k, v, o and lse); the split partials go to a static device array of
 * FLASH_ATTN_SCRATCH_BYTES inside the library, one per device, held until the
 * process ends.
 *   num_splits: as flash_attn_fwd_kv, except that 0 takes the library's count
 *     lowered until the partials (flash_attn_fwd_kv_workspace_bytes) fit the
 *     scratch; an explicit count whose partials do not fit gives
 *     FA_ERR_SCRATCH before any device work.
 * Every call on one device shares that device's scratch and leaves its own
 * partials there: calls that overlap in time on one device (two streams, two
 * host threads) race and must be ordered by the caller. Nothing in the
 * scratch needs to start at zero. The first call on a device is its set-up:
 * it looks up the scratch's address on that device (hipGetSymbolAddress;
 * FA_ERR_HIP if that fails), which makes the HIP runtime map the scratch onto
 * the device once; make that first call before capturing a graph or entering
 * a loop that must not see device memory change. Later calls allocate nothing.
 */
#define FLASH_ATTN_SCRATCH_BYTES (32u << 20)
int flash_attn_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                              int num_splits, void* stream);

/* Split count the library picks for num_splits = 0 (Nq, Nk: the largest
 * sequence lengths); 0 for invalid sizes. */
int flash_attn_fwd_kv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/* Workspace bytes of the general forward for `rows` query rows and
 * `num_splits` splits (0 when num_splits == 1; 0 for invalid sizes). */
size_t flash_attn_fwd_kv_workspace_bytes(long long rows, int d, int num_splits);

/*
 * Standard (materialising) attention in three passes, bf16 storage: the
 * baseline the method removes (fanfani.net "FlashAttention", section "The
 * bottleneck was never the arithmetic": scores written to slow memory, read
 * back for the mask and the softmax, the weights written and read back for
 * the product with V). Same inputs, outputs and conventions as
 * flash_attn_fwd (square, top-left causal mask), same O and lse up to
 * rounding; it exists to measure on the same chip the traffic and time the
 * fused forward saves.
 *   workspace: caller-owned device buffer of flash_attn_naive_workspace_bytes
 *     (B*Hq*N*N fp32 scores then B*Hq*N*N bf16 weights, each rounded up to 256
 *     bytes): quadratic in N by design.
 * Errors as flash_attn_fwd; FA_ERR_SHAPE also when B*Hq*N exceeds 2^31-1,
 * FA_ERR_WORKSPACE for a missing or short workspace.
 */
int flash_attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t flash_attn_naive_workspace_bytes(int B, int Hq, int N);

/*
 * Bytes of device workspace flash_attn_bwd / flash_attn_bwd_f32 need for these
 * sizes: two fp32 per query row (D_i = sum_c dO_ic O_ic, and lse_i * log2(e)),
 * 2*A(4R) bytes with R = B*Hq*N and A() rounding up to a multiple of 256.
 * Linear in N: no N x N buffer. Returns 0 for invalid sizes.
 */
size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Backward, bf16 storage, fp32 accumulation. Recomputes every score block from
 * q, k and the forward's lse; returns the gradients of sum(dout * O). dK and
 * dV come from a pass over the query blocks of each key block, dQ from a pass
 * over the key blocks of each query block, which recomputes the scores once
 * more; no atomics, so every run gives the same bits.
 *   q, o, dout [B,Hq,N,d], k, v [B,Hkv,N,d] (bf16 bits), lse [B,Hq,N] fp32:
 *     the forward's inputs and outputs (o and lse exactly as flash_attn_fwd
 *     returned them for the same q, k, v, scale, causal).
 *   dq [B,Hq,N,d], dk, dv [B,Hkv,N,d]: outputs (bf16 bits); with GQA dk and dv
 *     of a K/V head sum over its Hq/Hkv query heads.
 *   workspace, workspace_bytes: caller-owned device buffer and its size in
 *     bytes, at least flash_attn_bwd_workspace_bytes(B,Hq,Hkv,N,d); its
 *     contents on entry are ignored and on return are unspecified. A NULL or
 *     shorter workspace gives FA_ERR_WORKSPACE before any device work.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * General backward, bf16 storage: the gradients of the general forward's
 * problems (flash_attn_fwd_kv / flash_attn_fwd_varlen without split keys),
 * computed as flash_attn_bwd computes them:
 *   - Nq queries and Nk keys per sequence, the causal mask aligned to the
 *     bottom right (query i sees key j iff j <= i + Nk - Nq). A query that
 *     sees no key (O = 0, lse = -inf) has dq = 0 and adds nothing to dk, dv.
 *   - o and lse exactly as the forward returned them.
 * flash_attn_bwd_kv: q, o, dout, dq [B,Hq,Nq,d]; k, v, dk, dv [B,Hkv,Nk,d]
 *   (bf16 bits); lse [B,Hq,Nq] fp32.
 * flash_attn_bwd_varlen: B sequences packed along the token axis, the layout
 *   and cu_seqlens conventions of flash_attn_fwd_varlen: q, o, dout, dq
 *   [Hq,Tq,d]; k, v, dk, dv [Hkv,Tk,d]; lse [Hq,Tq]. A sequence without keys
 *   gets dq = 0, one without queries dk = dv = 0; rows outside every
 *   sequence, and rows beyond max_seqlen_q / max_seqlen_k in a sequence, are
 *   left unspecified.
 * workspace, workspace_bytes: caller-owned device buffer of at least
 *   flash_attn_bwd_kv_workspace_bytes(rows, d) bytes, rows = B*Hq*Nq
 *   (uniform) or Hq*Tq (varlen); contents on entry ignored, on return
 *   unspecified.
 * Errors as flash_attn_fwd_kv; FA_ERR_WORKSPACE for a missing or short
 * workspace.
 */
size_t flash_attn_bwd_kv_workspace_bytes(long long rows, int d);
int flash_attn_bwd_kv(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream);
int flash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                          const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                          int Tq, int Tk, int max_seqlen_q, int max_seqlen_k, int d, float scale, int causal,
                          void* stream);

/* Backward, fp32 check mode: as flash_attn_bwd with fp32 tensors. */
int flash_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                       const float* dout, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal, void* stream);

/* Static, NUL-terminated name of a status code ("FA_OK", ...); "FA_UNKNOWN" otherwise. */
const char* flash_attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
