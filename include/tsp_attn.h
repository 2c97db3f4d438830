/*
 * tsp_attn.h -- C ABI of the per-rank zigzag / GQA causal attention forward for MI355X
 * (gfx950).
 *
 * The operation: one sequence-parallel rank holds a zigzag share of the queries and
 * attends causally to the all-gathered full-sequence keys and values
 * ("Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
 * Inference", section 2 Methodology, attention layers: all-gather of K/V along the
 * sequence, attention of the local queries, zigzag partitioning for causal balance).
 * Causal visibility is decided by global token position, recomputed for the sharded
 * layout ("AutoSP: Unlocking Long-Context LLM Training Via Compiler-Based Sequence
 * Parallelism", section 2.A, item 4). Query heads are grouped over KV heads
 * ("Tensor, pipeline e sequence parallelism", section 01, GQA paragraph); D = 1 is the
 * Ulysses case of full attention over a head subset (same page, sequence-parallel
 * paragraph).
 *
 * Conventions shared by every entry point:
 *  - Zigzag map: the sequence of S_total tokens is cut into 2*D chunks of
 *    C = S_total / (2*D); rank r holds chunk r in local rows [0, C) and chunk 2*D-1-r in
 *    local rows [C, 2C). Local row i has global position
 *        g(i) = r*C + i                 for i <  C
 *        g(i) = (2*D-1-r)*C + (i - C)   for i >= C.
 *    With D = 1 the map is the identity.
 *  - Key j is visible to local row i iff j <= g(i) (inclusive diagonal).
 *  - Query head h reads KV head h / (Hq / Hkv) (contiguous grouping).
 *  - Scores are scaled by 1/sqrt(dh); lse is the natural-log log-sum-exp of the scaled
 *    scores over the visible keys.
 *
 * Status codes: every int-returning function returns TSP_OK (0) or a negative code.
 * Arguments are validated before anything is enqueued, so on error nothing is launched
 * and no output byte is written. No C++ exception crosses this boundary. A message for
 * the calling thread's last failure is available from tsp_attn_last_error().
 *
 * Ownership: all buffers belong to the caller. The library allocates no device memory,
 * frees nothing and keeps no pointer after a call returns. Work is enqueued
 * asynchronously on the caller's stream on the current HIP device; the library never
 * synchronizes the stream.
 */
#ifndef TSP_ATTN_H
#define TSP_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TSP_OK 0
#define TSP_EINVAL (-1)       /* bad pointer, size, rank or divisibility */
#define TSP_EUNSUPPORTED (-2) /* head dim or element type without a kernel */
#define TSP_ELAUNCH (-3)      /* the HIP runtime rejected the launch */
#define TSP_EINTERNAL (-4)    /* a HIP runtime query failed */

/* element types of q_local / k_full / v_full / out */
#define TSP_BF16 0 /* bfloat16, MFMA bf16 products, fp32 accumulation */
#define TSP_F32 1  /* float32, MFMA fp32 products, fp32 accumulation */

/*
 * tsp_attn_fwd -- causal attention of one rank's zigzag queries against the full K/V.
 *
 *   q_local  device, [B, 2C, Hq, dh] contiguous (BSHD), element type `dtype`
 *   k_full   device, [B, S_total, Hkv, dh] contiguous, row j = global token j
 *   v_full   device, [B, S_total, Hkv, dh] contiguous, row j = global token j
 *   out      device, [B, 2C, Hq, dh] contiguous, element type `dtype` (written)
 *   lse      device, [B, Hq, 2C] float32 (written)
 *   B, S_total, D, rank, Hq, Hkv, dh   sizes as above; C = S_total / (2*D)
 *   dtype    TSP_BF16 or TSP_F32
 *   stream   a hipStream_t (NULL = the default stream)
 *
 * Requirements: B >= 1, D >= 1, 0 <= rank < D, S_total > 0 and divisible by 2*D,
 * Hq >= 1, Hkv >= 1, Hq divisible by Hkv, dh in {64, 128, 256}, all pointers non-NULL
 * and 16-byte aligned, out/lse not overlapping the inputs. Keys past the largest global
 * position of the rank's queries are never read, so they may hold anything.
 * Rounding: out is the fp32 result rounded to nearest-even in `dtype`.
 * Returns TSP_OK, TSP_EINVAL, TSP_EUNSUPPORTED or TSP_ELAUNCH.
 */
int tsp_attn_fwd(const void* q_local, const void* k_full, const void* v_full, void* out,
                 float* lse, int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                 int64_t Hkv, int64_t dh, int dtype, void* stream);

/*
 * tsp_attn_fwd_range -- tsp_attn_fwd restricted to the keys j in [kv_begin, kv_end)
 * (0 <= kv_begin <= kv_end <= S_total), still causal by global position, so that a rank
 * can attend to each gathered chunk of K/V as it arrives ("Folding Tensor and Sequence
 * Parallelism ...", section 2, attention layers: the all-gather along the sequence;
 * section 3 item 3: communication overlapped with compute).
 *   accumulate = 0: out / lse receive the partial result over the range; a local row with
 *                   no visible key in the range gets out = 0 and lse = -inf.
 *   accumulate = 1: out / lse already hold a result over keys disjoint from the range
 *                   (lse = -inf where that result has no key); the partial is merged into
 *                   them with the tsp_attn_merge rule in the kernel's epilogue, and rows
 *                   with no visible key in the range are left untouched.
 * Only keys in [kv_begin rounded down to 64, kv_end) and below the rank's last position
 * are read. Same arguments, layouts, ownership and errors as tsp_attn_fwd, plus
 * TSP_EINVAL for a range outside [0, S_total] or accumulate not in {0, 1}.
 */
int tsp_attn_fwd_range(const void* q_local, const void* k_full, const void* v_full, void* out,
                       float* lse, int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                       int64_t Hkv, int64_t dh, int64_t kv_begin, int64_t kv_end, int accumulate,
                       int dtype, void* stream);

/*
 * tsp_attn_fwd_range2 -- tsp_attn_fwd_range over the union of two key ranges
 * [kv_begin, kv_end) and [kv_begin2, kv_end2), kv_end <= kv_begin2 <= kv_end2 <= S_total
 * (an empty second range reduces to tsp_attn_fwd_range): the two chunks a rank receives
 * from one peer in a step of the zigzag all-gather (chunks r' and 2D-1-r') are taken in
 * one launch, with one merge into the running result when accumulate = 1. bf16 sweeps
 * both ranges in one kernel (the running max, sum and output carry from the first range
 * to the second); fp32 runs one launch per range. Same arguments, layouts, ownership and
 * errors as tsp_attn_fwd_range, plus TSP_EINVAL for a second range that is not ordered
 * after the first or not inside [0, S_total].
 */
int tsp_attn_fwd_range2(const void* q_local, const void* k_full, const void* v_full, void* out,
                        float* lse, int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                        int64_t Hkv, int64_t dh, int64_t kv_begin, int64_t kv_end,
                        int64_t kv_begin2, int64_t kv_end2, int accumulate, int dtype, void* stream);

/*
 * tsp_attn_fwd_ring -- tsp_attn_fwd computed chunk by chunk in the order a ring all-gather
 * of the zigzag chunks delivers them ("Folding Tensor and Sequence Parallelism ...",
 * section 2 Methodology: K/V gathered along the sequence, zigzag partitioning), so that the
 * attention can start before the gather has finished.
 *
 * Two launches on `stream`: the rank's own chunks r and 2D-1-r (as tsp_attn_fwd_range2,
 * written fresh), then one sweep over the peers' chunks in arrival order -- for ring steps
 * s = 1 .. D-1, chunks p and 2D-1-p of peer p = (rank - s) mod D -- each taken whole by
 * the query rows that see it and merged into the first launch's result in the epilogue.
 * Before reading chunk c (its keys [c*C, (c+1)*C) of k_full / v_full), the second launch
 * waits until chunk_ready[c] == ready_value (device int32 [2D], read with system-scope
 * acquire loads, so a writer on another stream, device or a DMA engine may set it while
 * the kernel runs). With chunk_ready = NULL every chunk is taken as present. A wait polls
 * at most spin_limit times; a wait that gives up sets bit 0 of *wait_status (device int32)
 * and the sweep goes on with whatever the chunk holds, so the kernel always completes and
 * the caller must treat out / lse as invalid whenever that bit is set (the caller clears
 * *wait_status beforehand). The result equals tsp_attn_fwd's up to the rounding order of
 * the sums.
 *
 * Arguments, layouts, ownership and the other errors as tsp_attn_fwd. bf16 only
 * (TSP_EUNSUPPORTED for fp32). TSP_EUNSUPPORTED also when C is not a multiple of 64 or of
 * the kernel's query tile (tsp_attn_schedule's rows per tile, 256 at dh 128), since every
 * tile must lie in one chunk. TSP_EINVAL when chunk_ready is given without wait_status or
 * with spin_limit < 1. With D = 1 only the first launch runs.
 */
int tsp_attn_fwd_ring(const void* q_local, const void* k_full, const void* v_full, void* out,
                      float* lse, int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                      int64_t Hkv, int64_t dh, const int32_t* chunk_ready, int32_t ready_value,
                      int32_t spin_limit, int32_t* wait_status, int dtype, void* stream);

/*
 * tsp_attn_merge -- combine two partial results over disjoint key sets:
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   out = exp(lse_a - lse) * out_a + exp(lse_b - lse) * out_b,
 * a partial with lse = -inf contributing nothing (both -inf: out = 0, lse = -inf).
 *   out_a, out_b, out   device, [B, S_local, Hq, dh] contiguous, element type `dtype`
 *   lse_a, lse_b, lse   device, [B, Hq, S_local] float32
 * out / lse may be the same buffers as out_a / lse_a (in-place accumulation); no other
 * overlap is allowed. Pointers 16-byte aligned, dh in {64, 128, 256}. Enqueued on
 * `stream`. Returns TSP_OK, TSP_EINVAL, TSP_EUNSUPPORTED or TSP_ELAUNCH.
 */
int tsp_attn_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
                   void* out, float* lse, int64_t B, int64_t S_local, int64_t Hq, int64_t dh,
                   int dtype, void* stream);

/*
 * tsp_attn_bwd -- backward of tsp_attn_fwd: the gradients of the rank's attention for an
 * upstream gradient dout of out. The systems on the pages train models ("Folding Tensor
 * and Sequence Parallelism for Memory-Efficient Transformer Training & Inference";
 * "AutoSP ...", section 2.B: attention recomputed in the backward pass); with
 * P_ij = exp(s_ij - lse_i) on visible pairs and delta_i = dout_i . out_i:
 *   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i . v_j - delta_i),
 *   dq_i = sum_j dS_ij k_j / sqrt(dh),  dk_j = sum_i dS_ij q_i / sqrt(dh).
 *   q_local, k_full, v_full   the forward's inputs (layouts as in tsp_attn_fwd)
 *   out, lse                  the forward's outputs for them
 *   dout      device, [B, 2C, Hq, dh] contiguous, element type `dtype`
 *   dq_local  device, [B, 2C, Hq, dh] (written)
 *   dk_full   device, [B, S_total, Hkv, dh] (written), likewise dv_full: this rank's
 *             partial gradients of the gathered K/V, summed over the query heads of each
 *             KV head; the gradient of the full K/V is the sum of all ranks' partials (the
 *             adjoint of the all-gather, a reduce-scatter). Keys that no local row sees
 *             get 0.
 *   delta     device, [B, Hq, 2C] float32 (written): dout_i . out_i per row and head
 * dtype TSP_BF16 or TSP_F32 (fp32 throughout; meant for small shards); bf16 outputs are
 * the fp32 results rounded to nearest even. Same size rules as tsp_attn_fwd plus
 * Hq * dh <= 2^22; all
 * pointers non-NULL and 16-byte aligned, outputs not overlapping the inputs or each
 * other. Enqueued on `stream`; returns TSP_OK, TSP_EINVAL, TSP_EUNSUPPORTED or
 * TSP_ELAUNCH.
 */
int tsp_attn_bwd(const void* q_local, const void* k_full, const void* v_full, const void* out,
                 const float* lse, const void* dout, void* dq_local, void* dk_full, void* dv_full,
                 float* delta, int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                 int64_t Hkv, int64_t dh, int dtype, void* stream);

/*
 * tsp_attn_bwd_noalloc -- tsp_attn_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc): the same kernels and results, but delta (dout_i . out_i per row and head)
 * lives in a static device array of TSP_BWD_NOALLOC_MAX_ROWS floats (16 MiB) that the
 * library holds on every GPU it runs on until the process ends, so the call takes no
 * delta argument and calls no allocator. Arguments, layouts, dtypes and size rules are
 * those of tsp_attn_bwd, plus B * Hq * 2C <= TSP_BWD_NOALLOC_MAX_ROWS (else TSP_EINVAL,
 * nothing enqueued). The first call on a device looks the array's address up for that
 * device (TSP_EINTERNAL if that fails). The array is fully rewritten by every call before
 * it is read, so nothing carries over from the previous call; but all calls on one GPU
 * share it: calls that overlap in time on one GPU (other streams, other threads) race and
 * must be ordered by the caller.
 */
#define TSP_BWD_NOALLOC_MAX_ROWS (4 * 1024 * 1024)
int tsp_attn_bwd_noalloc(const void* q_local, const void* k_full, const void* v_full,
                         const void* out, const float* lse, const void* dout, void* dq_local,
                         void* dk_full, void* dv_full, int64_t B, int64_t S_total, int64_t D,
                         int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
                         void* stream);

/*
 * Ulysses layout changes around the one-rank (D = 1) attention. DeepSpeed-Ulysses
 * transposes between sequence partitions and head partitions with an all-to-all, so each
 * of P ranks attends over the whole sequence for H/P heads, then transposes back
 * ("Tensor, pipeline e sequence parallelism", section 01, sequence-parallel paragraph;
 * "AutoSP ...", section 2.A items 2-3). Rank p holds the contiguous sequence chunk p of
 * S_local tokens; heads are split contiguously (rank r: heads r*H/P .. (r+1)*H/P - 1).
 * These are the local permutes on either side of the collective; the collective itself
 * moves block r of a rank's send buffer to rank r, which stores it as block p (p = the
 * sender), so the receive buffer is in sequence order.
 *
 *   tsp_ulysses_pack_heads      x [B, S_local, H, dh] -> send [P, B, S_local, H/P, dh]
 *                               (send[r] = this rank's tokens, heads of rank r)
 *   tsp_ulysses_unpack_heads    send [P, B, S_local, H/P, dh] -> x [B, S_local, H, dh]
 *   tsp_ulysses_gather_sequence recv [P, B, S_local, Hl, dh] -> full [B, P*S_local, Hl, dh]
 *                               (block p = sequence chunk p; the attention input)
 *   tsp_ulysses_scatter_sequence full [B, P*S_local, Hl, dh] -> send [P, B, S_local, Hl, dh]
 *
 * Device buffers, contiguous, element type `dtype` (TSP_BF16 or TSP_F32; the data is only
 * moved), 16-byte aligned, input and output not overlapping; dh * element size a multiple
 * of 16; H divisible by P; at most 64 GiB per tensor. Enqueued on `stream`. Returns
 * TSP_OK, TSP_EINVAL, TSP_EUNSUPPORTED or TSP_ELAUNCH. Results are bit-exact copies.
 */
int tsp_ulysses_pack_heads(const void* x, void* send, int64_t B, int64_t S_local, int64_t H,
                           int64_t dh, int64_t P, int dtype, void* stream);
int tsp_ulysses_unpack_heads(const void* send, void* x, int64_t B, int64_t S_local, int64_t H,
                             int64_t dh, int64_t P, int dtype, void* stream);
int tsp_ulysses_gather_sequence(const void* recv, void* full, int64_t B, int64_t S_local,
                                int64_t Hl, int64_t dh, int64_t P, int dtype, void* stream);
int tsp_ulysses_scatter_sequence(const void* full, void* send, int64_t B, int64_t S_local,
                                 int64_t Hl, int64_t dh, int64_t P, int dtype, void* stream);

/*
 * tsp_gemm_bf16_nt -- C = A B^T for bf16 A [M, K] (row stride lda) and B [N, K] (row stride
 * ldb), fp32 accumulation; the projection products of the attention layer below.
 *   mode 0: C is bf16 [M, N] (row stride ldc), the result rounded to nearest even;
 *   mode 1: C is float32, the result stored; mode 2: C is float32, the result added to it.
 * Device buffers, 16-byte aligned; K a multiple of 64; N, ldc multiples of 4; lda, ldb
 * multiples of 8 and at most 2^22. Enqueued on `stream`; returns TSP_OK or TSP_EINVAL /
 * TSP_ELAUNCH.
 */
int tsp_gemm_bf16_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, int mode, void* stream);

/*
 * tsp_attn_layer_fwd -- one rank's TSP attention layer forward ("Folding Tensor and
 * Sequence Parallelism ...", section 2, attention layers): the ranks iterate over D weight
 * shards (packed W_Q, W_K, W_V, W_O of H/D heads each, broadcast by their owner); for each
 * shard every rank projects its own tokens, the K/V of all ranks are gathered along the
 * sequence, the rank's queries attend causally (zigzag positions) to them, and the output
 * projection of the shard's heads is accumulated. On one GPU the shards are resident and
 * the gather's other rows are given: this call runs one rank's share of every step.
 *   x_local     device bf16 [B, 2C, d_model], the rank's tokens in local row order
 *   w_qkv       device bf16 [(Hq + 2*Hkv) * dh, d_model]: the rows of W_Q (query heads in
 *               order), then W_K, then W_V (out_features x in_features); shard i holds
 *               query heads i*Hq/D .. and KV heads i*Hkv/D ..
 *   w_o         device bf16 [d_model, Hq * dh]
 *   k_gathered, v_gathered  device bf16 [B, S_total, Hkv, dh]: the gathered K/V; rows at the
 *               rank's global positions are overwritten with its own projections, the
 *               others are read as given (the other ranks' rows)
 *   y_local     device bf16 [B, 2C, d_model] (written): softmax(Q K^T / sqrt(dh)) V W_O^T
 *               over all heads for the rank's tokens
 *   workspace   device, at least tsp_attn_layer_workspace_bytes(...) bytes for the same
 *               shards_per_group (caller-owned; holds a group's Q and attention output, its
 *               lse and the fp32 sum of the output projection)
 *   shards_per_group  G, a divisor of D: the shards are taken in order G at a time, one
 *               projection GEMM (Q, K and V of the group's heads), one attention launch and
 *               one output-projection GEMM per group. G = 1 is the shard-by-shard schedule;
 *               a larger G lets one launch cover the CUs when a shard has few heads, at the
 *               cost of a G times larger workspace. 0: the fewest shards whose attention
 *               launch has a workgroup per CU of the current device (the workspace size for
 *               0 covers any G).
 * The result does not depend on G beyond fp32 summation order of the output projection.
 * Hq and Hkv divisible by D (whole heads per shard), d_model a multiple of 64, dh in
 * {64, 128, 256}, other size rules as tsp_attn_fwd. Enqueued on `stream`; returns TSP_OK,
 * TSP_EINVAL, TSP_EUNSUPPORTED or TSP_ELAUNCH.
 */
int tsp_attn_layer_workspace_bytes(int64_t B, int64_t S_total, int64_t D, int64_t Hq,
                                   int64_t Hkv, int64_t dh, int64_t d_model,
                                   int64_t shards_per_group, int64_t* bytes);
int tsp_attn_layer_fwd(const void* x_local, const void* w_qkv, const void* w_o, void* k_gathered,
                       void* v_gathered, void* y_local, void* workspace, int64_t workspace_bytes,
                       int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                       int64_t Hkv, int64_t dh, int64_t d_model, int64_t shards_per_group,
                       void* stream);

/*
 * tsp_attn_zigzag_positions -- the zigzag map on the host: writes g(i) for the 2C local
 * rows of `rank` into out_host (caller-owned host memory of 2C int64).
 * ("Folding Tensor and Sequence Parallelism ...", section 2, zigzag partitioning.)
 * Returns TSP_OK or TSP_EINVAL.
 */
int tsp_attn_zigzag_positions(int64_t S_total, int64_t D, int64_t rank, int64_t* out_host);

/*
 * tsp_attn_zigzag_positions_device -- the same map as evaluated by the attention
 * kernel's own device code: writes g(i) for the 2C local rows into out_dev
 * (caller-owned device memory of 2C int32), enqueued on `stream`. Positions are below
 * 2^31 by the S_total limit checked here. Returns TSP_OK, TSP_EINVAL or TSP_ELAUNCH.
 */
int tsp_attn_zigzag_positions_device(int32_t* out_dev, int64_t S_total, int64_t D,
                                     int64_t rank, void* stream);

/*
 * tsp_attn_unmasked_pairs -- visible (query, key) pairs of `rank` per (batch, query head):
 * the sum over local rows of g(i) + 1. Equal for every rank: C * (S_total + 1).
 * Returns the count, or TSP_EINVAL for invalid arguments.
 */
int64_t tsp_attn_unmasked_pairs(int64_t S_total, int64_t D, int64_t rank);

/*
 * tsp_attn_schedule -- the work decomposition tsp_attn_fwd launches for these sizes:
 * writes the number of workgroups to *n_workgroups and, if kv_tiles_per_workgroup is
 * non-NULL, the number of key/value tiles each workgroup processes (caller-owned host
 * memory of at least *n_workgroups int64; call once with NULL to size it), and the key
 * tile length to *kv_tile (may be NULL). Pure host computation.
 * Returns TSP_OK, TSP_EINVAL or TSP_EUNSUPPORTED.
 */
int tsp_attn_schedule(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq,
                      int64_t Hkv, int64_t dh, int dtype, int64_t* n_workgroups,
                      int64_t* kv_tiles_per_workgroup, int64_t* kv_tile);

/* tsp_attn_strerror -- static description of a status code. */
const char* tsp_attn_strerror(int status);

/* tsp_attn_last_error -- message of the calling thread's last failed call ("" if none). */
const char* tsp_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TSP_ATTN_H */
