/*
 * ringattn.h — C ABI of one context-parallel rank's share of ring attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources: the pages' own wording is restated, not quoted):
 *  - Context parallelism splits every sequence into equal contiguous chunks, one
 *    per rank (axolotl docs "Sequence Parallelism", section Implementation
 *    Details); K/V chunks rotate around a ring of ranks so that no device ever
 *    holds the whole sequence, while each query still sees every key it is
 *    allowed to (aicassindra "Transformer math: SP math", section "Context
 *    parallelism is the axis that is independent").
 *  - Each rank's partial results per chunk are combined as they arrive
 *    (axolotl docs, introduction: results aggregated through a ring pattern);
 *    the combination is the log-sum-exp merge of partial softmax results.
 *  - No S x S score matrix is ever stored; the backward pass recomputes the
 *    probabilities from the saved log-sum-exp (archcrux, "sequence-parallel
 *    long-context attention OOM": FlashAttention-style kernels avoid the full
 *    score matrix but still compute and backpropagate over the whole context).
 *  - Packed rows: sample membership comes from position ids by a cumulative sum
 *    over the global row (axolotl docs, section Mamba/SSM Hybrid Models, item on
 *    seq_idx; section Sample Packing with Sequence Parallelism).
 *  - There is no silent fallback: an unsupported shape is an error (archcrux:
 *    check that the intended attention kernel really runs for the shape/mask).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers, owned by the caller, contiguous
 *    row-major in the stated layout and 16-byte aligned.  The library allocates
 *    no memory and keeps no state apart from a thread-local error message.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously.  Faults inside kernels surface at the caller's
 *    next synchronisation.  Arguments are validated on the host before any
 *    launch; on any non-OK status nothing has been enqueued by that call
 *    (except RA_ERR_HIP, where the failing launch is reported).
 *  - No C++ exception crosses this boundary.
 *
 * Layouts (B batch rows, Sq local query rows, Sk keys of one chunk):
 *    Q, O, dO   [B, Sq, Hq, d]     K, V   [B, Sk, Hkv, d]
 *    LSE, delta [B, Hq, Sq] fp32   segment ids [B, seg_len] int32 (global row)
 *  Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARGUMENT = 1, /* a pointer, size or flag is invalid */
  RA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head_dim 96) */
  RA_ERR_HIP = 3               /* a HIP launch failed; see ra_last_error() */
} ra_status;

typedef enum { RA_DTYPE_F32 = 0, RA_DTYPE_BF16 = 1 } ra_dtype;

/* Shape and mask of one ring step: the local query shard against one KV chunk. */
typedef struct {
  int32_t batch;     /* B >= 1 */
  int32_t q_len;     /* 1 <= Sq <= 2^30: rows of the local query shard */
  int32_t kv_len;    /* 1 <= Sk <= 2^30: keys of this chunk */
  int32_t heads_q;   /* 1 <= Hq <= 4096, a multiple of heads_kv */
  int32_t heads_kv;  /* Hkv >= 1 */
  int32_t head_dim;  /* d: 64 or 128 */
  int64_t q_offset;  /* global token index of query row 0 (rank * chunk length) */
  int64_t kv_offset; /* global token index of key 0 of this chunk */
  int32_t causal;    /* 1: key j visible to query i iff kv_offset+j <= q_offset+i */
  float softmax_scale; /* multiplies q.k; callers pass 1/sqrt(head_dim) */
  int32_t dtype;     /* ra_dtype of Q, K, V (and of O/dO in the backward) */
} ra_shape;

/*
 * ring_attn_fwd_step — partial attention of the local queries against one KV
 * chunk (one ring step).
 * Defining passages: every query must see every key, and under context
 * parallelism K/V chunks rotate around a ring so that a rank sees one chunk per
 * step (aicassindra "Transformer math: SP math", section "Context parallelism is
 * the axis that is independent"); the step never stores the score matrix of the
 * chunk (archcrux, "sequence-parallel long-context attention OOM").  The
 * softmax(scale q.k) form is the standard definition, which the pages name but do
 * not print.
 *
 * Computes, per (b, h, i), over the visible keys j of this chunk:
 *   s_ij = softmax_scale * q_i . k_j,  LSE_i = ln sum_j exp(s_ij),
 *   O_i  = sum_j exp(s_ij - LSE_i) v_j.
 * A row with no visible key gets O = 0 and LSE = -inf (the merge identity).
 * Visibility: causal rule above (if causal) AND, if seg_ids != NULL,
 * seg_ids[b, kv_offset + j] == seg_ids[b, q_offset + i].
 *
 *  q        [B, Sq, Hq, d]  dtype          k, v [B, Sk, Hkv, d] dtype
 *  seg_ids  [B, seg_len] int32 or NULL: segment id of every token of the global
 *           row; must be nondecreasing along each row (segment_mask_from_pos
 *           produces such ids); q_offset+Sq and kv_offset+Sk must be <= seg_len.
 *           Ids that decrease along a row give unspecified values (never an
 *           out-of-bounds access).
 *  o_step   [B, Sq, Hq, d] fp32 out;  lse_step [B, Hq, Sq] fp32 out (natural log).
 * Errors: RA_ERR_INVALID_ARGUMENT for NULL q/k/v/o_step/lse_step, sizes < 1
 * or above the ra_shape limits, Hq % Hkv != 0, negative offsets, seg ranges past seg_len, misaligned pointers;
 * RA_ERR_UNSUPPORTED for head_dim not in {64, 128} or an unknown dtype.
 */
ra_status ring_attn_fwd_step(const ra_shape* shape, const void* q, const void* k, const void* v,
                             const int32_t* seg_ids, int64_t seg_len, float* o_step,
                             float* lse_step, void* stream);

/*
 * lse_merge — fold one step's partial result into the running result, in place.
 * Defining passage: the ranks' partial results are combined as they pass around
 * the ring (axolotl docs "Sequence Parallelism", introduction).  The pages do not
 * print the rule; the log-sum-exp merge below is the exact combination of two
 * softmax partials over disjoint key sets:
 *   M = max(L, L_s);  L' = M + ln(e^(L-M) + e^(L_s-M));
 *   O' = e^(L-L') O + e^(L_s-L') O_s;   rows where both L and L_s are -inf are
 *   left unchanged.
 * o_acc, o_step [B, Sq, Hq, d] fp32;  lse_acc, lse_step [B, Hq, Sq] fp32.
 * If o_out != NULL the merged O is also written there converted to out_dtype
 * (bf16: round to nearest even; f32: copy).  If o_step and lse_step are both
 * NULL no merge happens and o_acc is only converted into o_out (the final
 * conversion of a single-chunk ring).
 * Errors: RA_ERR_INVALID_ARGUMENT for NULL o_acc/lse_acc, exactly one of
 * o_step/lse_step NULL, nothing to do (both NULL and o_out NULL), sizes < 1,
 * misalignment; RA_ERR_UNSUPPORTED for d not a multiple of 4 or unknown out_dtype.
 */
ra_status lse_merge(int32_t batch, int32_t q_len, int32_t heads_q, int32_t head_dim, float* o_acc,
                    float* lse_acc, const float* o_step, const float* lse_step, void* o_out,
                    int32_t out_dtype, void* stream);

/*
 * ring_attn_fwd_step_merge — ring_attn_fwd_step and lse_merge of its result in one
 * launch (axolotl docs "Sequence Parallelism": the per-chunk results are
 * aggregated as they travel around the ring).  The step's partial (O_s, LSE_s) of
 * the local queries against this KV chunk, defined as for ring_attn_fwd_step, is
 * folded into the running (o_acc, lse_acc) in place with the lse_merge rule and is
 * never written out.  Equal, bit for bit, to ring_attn_fwd_step into scratch
 * followed by lse_merge(o_acc, lse_acc, scratch, ..., o_out, out_dtype).
 *  shape, q, k, v, seg_ids, seg_len: as ring_attn_fwd_step.
 *  o_acc    [B, Sq, Hq, d] fp32, read and written;  lse_acc [B, Hq, Sq] fp32, read
 *           and written (natural log; -inf for rows that have seen no key yet).
 *  o_out    NULL, or [B, Sq, Hq, d] in out_dtype (RA_DTYPE_F32 or RA_DTYPE_BF16,
 *           round to nearest even): the merged O (the last ring step's output).
 * o_acc/lse_acc must not overlap q, k, v or o_out; one call per running result at
 * a time (the call reads and writes it).
 * Errors: as ring_attn_fwd_step (with o_acc/lse_acc in place of o_step/lse_step);
 * RA_ERR_UNSUPPORTED for an unknown out_dtype; RA_ERR_INVALID_ARGUMENT for o_out
 * not 8-byte aligned.
 */
ra_status ring_attn_fwd_step_merge(const ra_shape* shape, const void* q, const void* k, const void* v,
                                   const int32_t* seg_ids, int64_t seg_len, float* o_acc, float* lse_acc,
                                   void* o_out, int32_t out_dtype, void* stream);

/*
 * segment_mask_from_pos — sample (segment) id of every token of packed rows.
 * Defining passages: axolotl docs "Sequence Parallelism", section Mamba/SSM Hybrid
 * Models (sample ids derived from position_ids by a cumulative sum that stays
 * correct across chunk boundaries) and section Sample Packing with Sequence
 * Parallelism (samples are packed before the row is split):
 *   seg_ids[b, t] = #{t' <= t : position_ids[b, t'] == 0} - 1,
 * computed over the GLOBAL row so that a context-parallel chunk that starts in
 * the middle of a sample keeps that sample's id.  Tokens before the first zero
 * get -1.  position_ids, seg_ids: [B, S] int32.
 * Errors: RA_ERR_INVALID_ARGUMENT for NULL pointers, B < 1, S < 1, or
 * S > 2^31 - 1.
 */
ra_status segment_mask_from_pos(int32_t batch, int64_t seq_len, const int32_t* position_ids,
                                int32_t* seg_ids, void* stream);

/*
 * ring_attn_bwd_preprocess — delta[b, h, i] = sum_d dO[b, i, h, :] * O[b, i, h, :]
 * (fp32 accumulation), the per-row term of the softmax gradient.
 * The pages do not describe this step; it belongs to the closed-form gradient of
 * softmax attention that the backward recomputes (archcrux, "sequence-parallel
 * long-context attention OOM": the backward still runs over the whole context),
 * and is computed once per backward from the forward's returned O, before the
 * ring steps.
 * o, d_o [B, Sq, Hq, d] in dtype;  delta [B, Hq, Sq] fp32 out.
 * Errors: as lse_merge; RA_ERR_UNSUPPORTED for d not in {64, 128}.
 */
ra_status ring_attn_bwd_preprocess(int32_t batch, int32_t q_len, int32_t heads_q, int32_t head_dim,
                                   int32_t dtype, const void* o, const void* d_o, float* delta,
                                   void* stream);

/*
 * ring_attn_bwd_step — one ring step of the backward pass for one KV chunk.
 * Defining passages: archcrux, "sequence-parallel long-context attention OOM"
 * (FlashAttention-style kernels avoid the score matrix but still backpropagate
 * over the whole context; recomputing it trades compute for memory), with the
 * ring order of aicassindra "Transformer math: SP math", section "Context
 * parallelism is the axis that is independent".  The gradient formulas are the
 * closed form of softmax attention (not printed on the pages).
 * With the FINAL merged lse of the forward and delta from the preprocess:
 *   P_ij = exp(s_ij - LSE_i) on visible pairs (0 elsewhere), s as in the forward;
 *   dV_j += sum_i P_ij dO_i;  dP_ij = dO_i . v_j;  dS_ij = P_ij (dP_ij - delta_i);
 *   dQ_i += scale sum_j dS_ij k_j;  dK_j += scale sum_i dS_ij q_i;
 * dK/dV of KV head g sum the contributions of all its query heads.
 *  q, d_o [B, Sq, Hq, d] dtype;  k, v [B, Sk, Hkv, d] dtype;  lse, delta [B, Hq, Sq].
 *  dq_acc [B, Sq, Hq, d] fp32, dk_acc / dv_acc [B, Sk, Hkv, d] fp32: accumulated
 *  with +=; the caller zeroes them before the first step.
 * Masks and seg_ids exactly as in ring_attn_fwd_step.
 * Resources (bf16, head_dim 128): the dQ kernel runs on a side stream of the device
 * (created on first use, default priority) that joins `stream` before the call's
 * work is complete in `stream` order; a step whose dK/dV key blocks are split
 * (causal diagonal chunk or packed rows on small grids) uses 64 MiB + 256 KiB of
 * device scratch, allocated on the device by the first such step and kept until the
 * process ends.  Steps that overlap on one device (concurrent streams) must not
 * both split.  Results are deterministic: split partial sums are added in a fixed
 * order.
 * Errors: as ring_attn_fwd_step; RA_ERR_HIP if the side stream or the scratch cannot
 * be created.
 */
ra_status ring_attn_bwd_step(const ra_shape* shape, const void* q, const void* k, const void* v,
                             const void* d_o, const float* lse, const float* delta,
                             const int32_t* seg_ids, int64_t seg_len, float* dq_acc,
                             float* dk_acc, float* dv_acc, void* stream);

/*
 * ring_attn_bwd_step_noalloc — ring_attn_bwd_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, same kernels, bit-identical results; it calls
 * no allocating routine.
 * Scratch: the split dK/dV kernel's arrival counters and partial sums live in a
 * static device array of the library (64 MiB + 256 KiB on each GPU it runs on, held
 * until the process ends; its address is looked up once per device).  The split is
 * sized to that array, so no step needs more; the array is shared by every call on
 * the GPU, so calls that overlap on one GPU (concurrent streams) race and must not
 * be issued.  Both kernels of the step run on `stream` (no side stream).
 * Errors: as ring_attn_bwd_step; RA_ERR_HIP if the scratch address lookup fails.
 */
ra_status ring_attn_bwd_step_noalloc(const ra_shape* shape, const void* q, const void* k,
                                     const void* v, const void* d_o, const float* lse,
                                     const float* delta, const int32_t* seg_ids, int64_t seg_len,
                                     float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/*
 * ring_recv_copy — the transfer of one ring step, on one GPU: copies `bytes` bytes
 * from `src` (the buffer that stands for the peer's K/V chunk, or for a travelling
 * dK/dV partial) to `dst` (a receive slot) on `stream`, with the DMA engines
 * (hipMemcpyDeviceToDeviceNoCU), so the copy takes no compute units from the step
 * kernels running on another stream.  K/V rotate around the ring while each rank
 * attends to the chunk it holds (aicassindra, "Transformer math: SP math",
 * section on context parallelism; axolotl docs "Sequence Parallelism",
 * introduction).
 *
 *  dst, src  device pointers of the same device, regions of `bytes` bytes that do
 *            not overlap; bytes == 0 is a no-op.
 * Asynchronous: ordering against other streams is the caller's (events).
 * Errors: RA_ERR_INVALID_ARGUMENT for NULL pointers (with bytes > 0);
 * RA_ERR_HIP if the runtime rejects the copy.
 */
ra_status ring_recv_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* ra_status_string(ra_status status);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* ra_last_error(void);

/* Library ABI version: 3 (2 added ring_recv_copy, 3 ring_attn_fwd_step_merge). */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
