/*
 * rdg.h -- C ABI of librdg.so: one GPU's share of a DeepSeek-V3-style
 * mixture-of-experts layer on AMD MI355X (gfx950).
 *
 *   rdg_route        group-limited top-k gating
 *   rdg_eplb_place   EPLB placement of experts and redundant copies (host)
 *   rdg_eplb_remap   logical -> physical expert remap (redundant experts)
 *   rdg_tbo_split    two-batch-overlap cut of a batch into micro-batches (host)
 *   rdg_dispatch     token -> expert permutation into a contiguous or masked layout
 *   rdg_grouped_ffn  grouped gate/up GEMM + SiLU-gated product + down GEMM
 *                    (rdg_grouped_ffn_gather: reading the token rows through
 *                    the layout instead of a permuted copy)
 *   rdg_combine      routing-weighted unpermute-and-sum (optionally polling
 *                    the down GEMM's per-row-tile completion signals;
 *                    rdg_combine_finish: the rest once the GEMM is done)
 *
 * Page names used in the citations below:
 *   [LEP]  "Large-scale EP: DeepEP, EPLB and two-batch overlap" (SGLang handbook)
 *   [SBO]  "Single Batch Overlap (SBO): Overlaping of Down GEMM with Combine Send"
 *          (DeepGEMM pull request)
 *   [H100] SGLang's DeepSeek-V3/R1 deployment on 96 H100s (Chinese article)
 *   [DEEP] "DeepEP, fully taken apart" (Chinese deep-dive on DeepEP)
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  They must be 16-byte
 *     aligned.  The caller owns (allocates and frees) every buffer, including
 *     workspaces sized by the *_bytes queries; the library allocates nothing.
 *   - Every compute call only enqueues work on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns without waiting.  Argument errors are
 *     returned synchronously (RDG_EINVAL / RDG_EUNSUPPORTED) and then nothing
 *     is enqueued.  A failed launch returns RDG_EHIP.
 *   - Errors found on the device (capacity overflow, signal timeout) are
 *     written to the layout's status word [code, detail], first error wins;
 *     rdg_check_status is the one call that waits for the stream.
 *   - No C++ exception crosses this boundary.
 */
#ifndef RDG_H
#define RDG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* rdg_stream_t; /* the same type as hipStream_t */

enum {
    RDG_OK = 0,
    RDG_EINVAL = -1,       /* bad argument: nothing was enqueued */
    RDG_ECAPACITY = -2,    /* rows did not fit the preallocated layout (device status) */
    RDG_ETIMEOUT = -3,     /* a polled signal never reached its threshold (device status) */
    RDG_EHIP = -4,         /* the HIP runtime refused a launch or a query */
    RDG_EUNSUPPORTED = -5  /* a valid but unimplemented combination of sizes / types */
};

/* element types.  RDG_FP8_E4M3_UE8M0: e4m3 codes whose block scales are
 * powers of two (still stored as fp32 values 2^k; an 8-bit exponent-only
 * scale, the form gfx950's scaled MFMA applies in hardware). */
enum { RDG_F32 = 0, RDG_BF16 = 1, RDG_FP8_E4M3 = 2, RDG_FP8_E4M3_UE8M0 = 3 };
enum { RDG_CONTIGUOUS = 0, RDG_MASKED = 1 };            /* layout kinds */

/* A dispatch layout ([LEP] DeepEP modes paragraph: the contiguous layout
 * orders tokens by expert for dynamic shapes, the masked layout keeps fixed
 * shapes and marks the valid rows; [H100] "DeepGEMM integration").
 * Filled by the caller: the scalar fields and the buffer pointers.  Written
 * by rdg_dispatch / rdg_layout_dense: the buffers' contents.
 *
 *   kind      RDG_CONTIGUOUS: expert e's rows are [offsets[e], offsets[e] +
 *             masked_m[e]), segments padded to block_m rows.
 *             RDG_MASKED: expert e owns rows [e*m_max, (e+1)*m_max); the first
 *             masked_m[e] are valid.
 *   n_local   experts held by this GPU (1..1024)
 *   block_m   contiguous: padding granularity in rows, a multiple of 16 (128
 *             lets the GEMMs use their largest row tile)
 *   m_max     masked: rows per expert
 *   m_cap     rows of x_perm / y / row_src.  Masked: n_local*m_max.
 *             Contiguous: at least n_rows + n_local*(block_m-1) never overflows.
 *   n_rows    the number of (token, slot) entries dispatched, T*K (sizes grids)
 *   counts    [n_local]   rows routed to each expert
 *   offsets   [n_local+1] first row of each expert's segment
 *   masked_m  [n_local]   rows kept for each expert (counts clipped to capacity)
 *   pos       [T*K]       layout row of entry t*K+k, or -1 (not local / dropped)
 *   row_src   [m_cap]     entry t*K+k stored in each row, or -1 (padding)
 *   status    [2]         {code, detail}; cleared by rdg_dispatch
 *   work      rdg_dispatch_workspace_bytes(T, K, n_local) bytes
 *   expert_load  NULL, or [n_local] int64 kept by the caller across calls:
 *             rdg_dispatch adds each expert's routed-row count (before any
 *             capacity drop) to it -- the expert-load statistics that
 *             rebalancing works from ([LEP] "EPLB": replicas and placement
 *             follow the recorded load; [H100] "Case study: expert
 *             distribution statistics").  The caller zeroes it; concurrent
 *             dispatches may share it (device-scope atomic adds).
 */
typedef struct rdg_layout {
    int32_t kind, n_local, block_m, m_max, m_cap, n_rows;
    int32_t* counts;
    int32_t* offsets;
    int32_t* masked_m;
    int32_t* pos;
    int32_t* row_src;
    int32_t* status;
    void* work;
    int64_t* expert_load;
} rdg_layout;

/* Group-limited top-k gating ([DEEP] "group-limited gating": pick the best
 * groups first, then the top-K experts inside them; [DEEP] "EP": the token's
 * output is the routing-weighted sum over its K experts).
 *   logits    [B, N] fp32, row-major
 *   n_group   groups of N/n_group consecutive experts; topk_group of them kept
 *   K         experts per token (K <= topk_group*N/n_group, K <= 32)
 *   scale     the renormalised weights sum to this
 *   topk_ids  [B, K] int32 out: experts in (score desc, id asc) order
 *   topk_w    [B, K] fp32 out
 * Score: sigmoid evaluated in fp64 and rounded once to fp32 (a fixed
 * evaluation, bit-identical wherever it is implemented); group score: fp32
 * sum of the group's two largest scores; ties go to the lower index.
 * Limits: N <= 1024.  B = 0 is a no-op. */
int rdg_route(const float* logits, int B, int N, int n_group, int topk_group, int K, float scale,
              int32_t* topk_ids, float* topk_w, rdg_stream_t stream);

/* The same with a selection-only bias (a variant not on the pages, as
 * DeepSeek-style routers use: a per-expert correction that steers the choice
 * without entering the weights).
 *   bias  [N] fp32, finite: groups and experts are chosen by the fp32 sums
 *         score + bias (same rules and ties); the weights renormalise the
 *         plain scores of the chosen experts; slots are in (score + bias
 *         desc, id asc) order. */
int rdg_route_biased(const float* logits, const float* bias, int B, int N, int n_group, int topk_group, int K,
                     float scale, int32_t* topk_ids, float* topk_w, rdg_stream_t stream);

/* EPLB logical -> physical remap ([LEP] self-test answer 3 and the EPLB
 * paragraph: 256 logical experts in 288 physical slots, popular experts
 * replicated, each copy taking a share; [H100] "EPLB").
 *   ids        [T, K] logical expert ids (-1: entry not sent to this GPU)
 *   token_gidx [T] int64 global token index; replica = gidx mod n_replica[e]
 *   log2phy    [n_logical, r_max] physical id of each replica
 *   n_replica  [n_logical] replicas per logical expert (1..r_max)
 *   local_ids  [T, K] out: physical id - phys_begin when it lies in
 *              [phys_begin, phys_begin + n_local), else -1
 * May run in place (local_ids == ids). */
int rdg_eplb_remap(const int32_t* ids, const int64_t* token_gidx, int T, int K, const int32_t* log2phy,
                   const int32_t* n_replica, int r_max, int n_logical, int phys_begin, int n_local,
                   int32_t* local_ids, rdg_stream_t stream);

/* EPLB placement: where the logical experts and their redundant copies go
 * ([LEP] "EPLB": the measured per-expert load becomes a new expert-to-GPU
 * map, hierarchically -- groups spread over nodes, then each node's experts
 * placed inside it -- with extra copies of the popular experts; [H100]
 * "Expert-parallel load balancer": the busiest experts get the most copies,
 * rare ones share a GPU with busier ones, any GPU count).  Host code, all
 * pointers host pointers; no GPU work, no global state (thread-safe).
 *   load        [n_logical] host, finite and >= 0: e.g. token counts summed by
 *               the dispatch recorder (rdg_layout.expert_load), as doubles
 *   n_groups    groups of n_logical/n_groups consecutive experts
 *   n_nodes     nodes of n_gpus/n_nodes GPUs; the hierarchical placement is
 *               used when n_groups is a multiple of n_nodes (> 1), else the
 *               machine is placed as one node
 *   n_physical  slots, n_physical/n_gpus per GPU (>= n_logical)
 *   r_max       columns of log2phy
 *   phy2log     [n_physical] host out: logical expert in each slot
 *   log2phy     [n_logical, r_max] host out: physical id of each copy, -1 pad
 *   n_replica   [n_logical] host out: copies per expert (>= 1)
 *   gpu_load    [n_gpus] host out (may be NULL): the load each GPU receives
 * Rules: (1) groups by decreasing summed load, each to the least-loaded node
 * that still takes groups (each takes n_groups/n_nodes); (2) in each node,
 * one copy per expert, then every spare slot to the expert with the largest
 * load per copy; (3) copies (load / copies each) by decreasing load, each to
 * the node's least-loaded GPU with a free slot, which gives it its next slot:
 * physical id = GPU * (n_physical/n_gpus) + slot.  Ties go to the lower
 * group, node, expert, copy or GPU index.  Returns RDG_EINVAL for shapes that
 * do not divide as stated or loads that are negative or not finite, and
 * RDG_ECAPACITY when an expert would need more than r_max copies (outputs
 * then undefined). */
int rdg_eplb_place(const double* load, int n_logical, int n_groups, int n_nodes, int n_gpus, int n_physical,
                   int r_max, int32_t* phy2log, int32_t* log2phy, int32_t* n_replica, double* gpu_load);

/* Two-batch overlap split ([LEP] "TBO": a batch is cut into two micro-batches
 * whose stages interleave; a prefill batch at the sequence boundary whose
 * cumulative token count is closest to half, never inside a sequence; a
 * decode batch in half by request count).  Host code.
 *   seq_lens  [n_seqs] host: tokens of each sequence (>= 0), in batch order
 *   decode    nonzero: one token per request, cut at n_seqs / 2
 * Returns i: micro-batch A is sequences [0, i), B the rest; 0 when n_seqs < 2
 * (no cut); for prefill i minimises |2 * tokens(A) - total| over 1..n_seqs-1,
 * ties to the lower i.  RDG_EINVAL for a negative length or count. */
int rdg_tbo_split(const int32_t* seq_lens, int n_seqs, int decode);

/* Bytes of rdg_layout.work for a dispatch of T tokens x K slots over n_local experts. */
size_t rdg_dispatch_workspace_bytes(int T, int K, int n_local);

/* Dispatch ([LEP] self-test answer 1: the contiguous layout needs a permute
 * that orders tokens by expert; [H100] "DeepEP-based EP": exceeding a
 * preallocated fixed buffer is a runtime error; [DEEP] "How large is the
 * traffic": each token's H-vector goes to each of its K experts).
 *   x         [T, H] tokens: fp32, bf16 or fp8 e4m3 (dtype)
 *   x_scales  [T, H/128] fp32 block scales (fp8 only, else NULL)
 *   ids       [T, K] local expert ids in [0, n_local), -1 = skip
 *   x_perm    [m_cap, H] out (dtype); x_perm_scales [m_cap, H/128] (fp8)
 * Rows of one expert keep their (t, k) order (a stable counting sort), so the
 * layout is deterministic.  Overflow drops the extra rows and sets status
 * RDG_ECAPACITY (masked: detail = the largest count; contiguous: detail =
 * the rows needed).  Padding rows of x_perm are left untouched.
 * x_perm = NULL (and x_perm_scales = NULL): the layout only -- counts,
 * offsets, pos, row_src, tile tables -- and no rows are copied; x and
 * x_scales are then not read (may be NULL).  The grouped GEMMs read the rows
 * through row_src instead (rdg_grouped_ffn_gather).
 * H must be a multiple of 16 (fp8: of 128).  T = 0 is allowed (the layout
 * is cleared; x, ids, x_perm and the scale pointers may then be NULL). */
int rdg_dispatch(const void* x, const float* x_scales, int dtype, int T, int H, const int32_t* ids, int K,
                 const rdg_layout* L, void* x_perm, float* x_perm_scales, rdg_stream_t stream);

/* Allocation-free dispatch, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Computes exactly what rdg_dispatch computes; its scratch
 * (per-chunk expert counts and one rank per dispatched entry) lives in a
 * static device array inside the library, 4.25 MiB per GPU, held until the
 * process ends, instead of in a caller workspace.  L->work then needs only
 * the layout's row-tile tables, rdg_layout_tables_bytes(L->n_local) bytes,
 * which the grouped GEMMs read later.  At most 2^20 dispatched entries
 * (T * K); more returns RDG_EUNSUPPORTED and enqueues nothing.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or on one stream under concurrent graph replays) race,
 * so serialise them.  Nothing in the array needs clearing between calls.
 * No allocating call is made (the array's device address is looked up once
 * per device on the first call). */
size_t rdg_layout_tables_bytes(int n_local);
int rdg_dispatch_noalloc(const void* x, const float* x_scales, int dtype, int T, int H, const int32_t* ids, int K,
                         const rdg_layout* L, void* x_perm, float* x_perm_scales, rdg_stream_t stream);

/* Describe T rows as one expert's segment (rows [0, T)), for running a dense
 * FFN -- the shared expert -- through rdg_grouped_ffn with n_local = 1.
 * Writes counts, offsets, masked_m and the work area; L->kind must be
 * RDG_CONTIGUOUS, L->n_local 1, L->m_cap >= T, L->n_rows = T. */
int rdg_layout_dense(int T, const rdg_layout* L, rdg_stream_t stream);

/* Grouped expert FFN over a layout (the expert FFN of [DEEP] "EP"; the
 * contiguous and masked grouped GEMMs of [H100] "DeepGEMM integration"; the
 * fp8 "1d2d" block-scaled masked GEMM and the signalled down GEMM of [SBO]
 * sections 2-3).  For every valid row r of expert e:
 *   h[r] = silu(x[r] W1_e^T) * (x[r] W3_e^T)      (stored in h_ws)
 *   y[r] = h[r] W2_e^T                             (stored in y)
 * Weights: W1, W3 hold [n_local, I, H] and W2 [n_local, H, I], each packed
 * by rdg_pack_weights (n_mat = n_local).
 * dtype RDG_F32: everything fp32.  RDG_BF16: bf16 operands, fp32
 * accumulation, h and y bf16.  RDG_FP8_E4M3: e4m3 operands, x_perm_scales
 * [m_cap, H/128], weight scales W1_s, W3_s [n_local, I/128, H/128] and
 * W2_s [n_local, H/128, I/128]; every 128-long partial product is scaled by
 * its activation and weight block scales in fp32; h is re-quantised to e4m3
 * with 1x128 scales (h_scales_ws [m_cap, I/128]); y is bf16.
 * RDG_FP8_E4M3_UE8M0: the same with power-of-two scales everywhere (inputs
 * from rdg_quantize_fp8_ue8m0, h re-quantised with power-of-two scales); the
 * 128-row kernels hand the scales to the MFMA as 8-bit exponents, so the
 * block products are accumulated in fp32 by the matrix core with no
 * per-block promotion.
 *   h_ws      [m_cap, I] (dtype's storage: fp32 / bf16 / e4m3)
 *   y         [m_cap, H] fp32 (RDG_F32) or bf16
 *   signals   NULL, or [ceil(m_cap / rdg_signal_rows(L, dtype, H, I)) + 2] int32, zeroed by
 *             the caller (rdg_fill_i32) before this call (the last two words
 *             are the polling combine's, see rdg_combine): after the down GEMM
 *             has stored a row tile's outputs for a block of columns it adds
 *             the block's column count to that tile's counter at device
 *             scope, once those outputs are visible at device scope (they are
 *             written through to memory and waited for: release ordering for
 *             a reader that loads them at device scope, as rdg_combine does);
 *             a tile is complete when its counter reaches
 *             rdg_signal_threshold(H, dtype) = H.
 * Rows outside [offsets[e], offsets[e] + masked_m[e]) are neither read nor
 * written.  H and I must be multiples of 128.  A layout with L->n_rows = 0
 * is a no-op (nothing is launched; the buffer pointers may be NULL). */
int rdg_grouped_ffn(const rdg_layout* L, int dtype, int H, int I, const void* x_perm, const float* x_perm_scales,
                    const void* W1, const void* W3, const void* W2, const float* W1_s, const float* W3_s,
                    const float* W2_s, void* h_ws, float* h_scales_ws, void* y, int32_t* signals,
                    rdg_stream_t stream);

/* Weight packing, done once when weights are loaded.  The grouped GEMMs
 * read every weight matrix in a tiled order in which each 16-row x KS tile
 * (KS = 4 fp32, 32 bf16, 128 fp8 elements of the reduction dimension) is
 * stored contiguously in the order the 64 lanes of a wavefront consume it
 * as an MFMA operand, so that each load instruction fetches one contiguous
 * KiB (fp8: the tile is two such KiB halves).  Tiles are ordered by matrix,
 * then by 16-row group, then along the reduction dimension.
 *   W         [n_mat, rows, cols] row-major (cols = the reduction dimension)
 *   W_packed  the same number of bytes, packed
 * rows must be a multiple of 16 and cols of 128.  The block scales of fp8
 * weights are not packed. */
size_t rdg_packed_weight_bytes(int dtype, int n_mat, int rows, int cols);
int rdg_pack_weights(const void* W, int dtype, int n_mat, int rows, int cols, void* W_packed, rdg_stream_t stream);

/* The two stages of rdg_grouped_ffn as separate launches (same arguments
 * and rules): the gate/up GEMM with the SiLU-gated product writing h (and
 * its fp8 scales), and the down GEMM reading h and writing y (optionally
 * signalling).  rdg_grouped_ffn = rdg_grouped_gate_up then rdg_grouped_down
 * on the same stream. */
int rdg_grouped_gate_up(const rdg_layout* L, int dtype, int H, int I, const void* x_perm, const float* x_perm_scales,
                        const void* W1, const void* W3, const float* W1_s, const float* W3_s, void* h_ws,
                        float* h_scales_ws, rdg_stream_t stream);
int rdg_grouped_down(const rdg_layout* L, int dtype, int H, int I, const void* h_ws, const float* h_scales_ws,
                     const void* W2, const float* W2_s, void* y, int32_t* signals, rdg_stream_t stream);

/* The grouped FFN reading its token rows straight from the dispatched
 * tokens instead of a permuted copy: the dispatch's row permutation ([H100]
 * "DeepGEMM integration": rows ordered by expert for the contiguous grouped
 * GEMM; [DEEP] "EP": each token's vector goes to each of its K experts)
 * folded into the gate/up GEMM's loads.  Same arguments, rules and results
 * as rdg_grouped_ffn / rdg_grouped_gate_up, bit for bit, except:
 *   x         [n_rows / K, H] the tokens given to rdg_dispatch (dtype)
 *   x_scales  [n_rows / K, H/128] fp32 (fp8 only, else NULL)
 *   K         the slots per token of that dispatch
 * Layout row r of expert e reads token row_src[r] / K.  L must be the
 * layout of an rdg_dispatch (or rdg_dispatch_noalloc) of those tokens --
 * with x_perm = NULL, which skips the copy -- whose row_src this reads;
 * not a layout from rdg_layout_dense.  RDG_EINVAL when K is outside
 * [1, 32], L has no row_src, or L->n_rows is not a multiple of K. */
int rdg_grouped_ffn_gather(const rdg_layout* L, int dtype, int H, int I, const void* x, const float* x_scales, int K,
                           const void* W1, const void* W3, const void* W2, const float* W1_s, const float* W3_s,
                           const float* W2_s, void* h_ws, float* h_scales_ws, void* y, int32_t* signals,
                           rdg_stream_t stream);
int rdg_grouped_gate_up_gather(const rdg_layout* L, int dtype, int H, int I, const void* x, const float* x_scales,
                               int K, const void* W1, const void* W3, const float* W1_s, const float* W3_s,
                               void* h_ws, float* h_scales_ws, rdg_stream_t stream);

/* Rows per signal counter (the grouped GEMMs' row tile for this layout,
 * type and size: 16, 32, 64 or 128) and the counter value that means "row
 * tile done" (H), for the down GEMM of rdg_grouped_ffn.  With signals, the
 * down GEMM takes the row tiles in layout order (one at a time, or in groups
 * of a few for the 128-row tiles), so they complete in about that order; at
 * most 65535 row tiles (RDG_EUNSUPPORTED beyond). */
int rdg_signal_rows(const rdg_layout* L, int dtype, int H, int I);
int rdg_signal_threshold(int H, int dtype);


/* Combine ([DEEP] "EP": weighted sum back to the token; [DEEP] "why is
 * combine slower": transfer plus weighted reduction; [DEEP] "limitations":
 * bf16 pre-reduction is imprecise and non-deterministic, so the sum here is
 * fp32, in k order, rounded once; [SBO] section 2: poll each row tile's
 * counter until it reaches the threshold before using its rows).
 *   out[t] = shared_out[t] + sum_{k: pos[t,k] >= 0} topk_w[t,k] * y[pos[t,k]]
 *   y          [m_cap, H] (y_dtype: RDG_F32 or RDG_BF16)
 *   topk_w     [T, K] fp32
 *   shared_out [T, H] in out_dtype, or NULL
 *   out        [T, H] out_dtype (RDG_F32 or RDG_BF16)
 *   signals    NULL, or the counters given to rdg_grouped_ffn, with
 *              signal_rows = rdg_signal_rows(L, dtype, H, I) of that call,
 *              threshold and a timeout in microseconds (a tile still
 *              incomplete then is skipped and status = RDG_ETIMEOUT with
 *              detail = the tile index).  Word ceil(m_cap / signal_rows) of
 *              the array (zeroed with the counters) counts the work units
 *              the polling waves have claimed
 *   max_blocks 0 = one wavefront per token and 512-feature slice; else at
 *              most this many 256-thread workgroups loop over the work.  The
 *              polling form never uses more than a quarter of the GPU's CUs'
 *              worth of workgroups (fewer if max_blocks says so): waiting
 *              workgroups hold their CU, and the down GEMM's workgroups must
 *              always find CUs to run on.
 * The polling form may run on another stream concurrently with the down
 * GEMM, which must have been enqueued first.  Each token is combined at its
 * last layout row (L->row_src must be set), once every row tile it reads is
 * complete, and the tokens with no local row after them; the waves claim
 * these units in layout order, one at a time, until none are left or
 * rdg_combine_finish has taken the rest.  The output does not depend on the
 * visiting order: it equals the plain form bit for bit.  RDG_EUNSUPPORTED
 * when m_cap + ceil(T / 64) reaches 2^30. */
int rdg_combine(const void* y, int y_dtype, const rdg_layout* L, const float* topk_w, int T, int K, int H,
                const void* shared_out, void* out, int out_dtype, int32_t* signals, int signal_rows,
                int threshold, int64_t timeout_us, int max_blocks, rdg_stream_t stream);

/* The rest of a polling combine ([SBO] section 2: the consumer takes each
 * row block as its counter completes; once the producer has finished there
 * is nothing left to wait for).  Enqueue it on the down GEMM's stream after
 * rdg_grouped_ffn / rdg_grouped_down, while the polling rdg_combine with the
 * same signals runs on another stream.  It closes the polling form's unit
 * counter (polling waves stop claiming) and combines every token whose unit
 * no polling wave had claimed, one wavefront per token and 512-feature slice
 * as the plain form does; the polling waves finish the units they hold.
 * Each token is combined exactly once, and out equals the plain form bit for
 * bit.  The output is complete once both this call and the polling combine
 * have finished.  Arguments as for rdg_combine (signals and signal_rows
 * required). */
int rdg_combine_finish(const void* y, int y_dtype, const rdg_layout* L, const float* topk_w, int T, int K, int H,
                       const void* shared_out, void* out, int out_dtype, int32_t* signals, int signal_rows,
                       rdg_stream_t stream);

/* fp8 e4m3 block quantiser (the "1d2d" scales of [SBO] section 3): blocks of
 * block_rows x 128 (1 for activations, 128 for weights); scale = amax/448 in
 * fp32 (1 for an all-zero block), code = round-to-nearest-even of
 * clamp(v / scale, -448, 448).
 *   src     [rows, cols] fp32 or bf16 (src_dtype)
 *   q       [rows, cols] e4m3 codes out
 *   scales  [ceil(rows/block_rows), cols/128] fp32 out
 * cols must be a multiple of 128; block_rows is 1 or 128. */
int rdg_quantize_fp8(const void* src, int src_dtype, int rows, int cols, int block_rows, uint8_t* q,
                     float* scales, rdg_stream_t stream);

/* The same quantiser with power-of-two scales: scale = the smallest 2^k with
 * amax / 2^k <= 448 (k in [-126, 127]; 1 for an all-zero block), stored as
 * the fp32 value 2^k.  For RDG_FP8_E4M3_UE8M0 layers.  (A variant of the
 * [SBO] section 3 block format: its scales as 8-bit exponents, the form that
 * scaled matrix instructions take.) */
int rdg_quantize_fp8_ue8m0(const void* src, int src_dtype, int rows, int cols, int block_rows, uint8_t* q,
                           float* scales, rdg_stream_t stream);

/* Fill n int32 words with value (a kernel, so it is safe inside captured graphs). */
int rdg_fill_i32(int32_t* p, int32_t value, int64_t n, rdg_stream_t stream);

/* Wait for the stream, then copy the status word {code, detail} to the host
 * array host_status[2].  Returns the code (RDG_OK when no error was found). */
int rdg_check_status(const int32_t* status, int32_t* host_status, rdg_stream_t stream);

/* A static string for a return or status code. */
const char* rdg_strerror(int code);

/* Library version, major*10000 + minor*100 + patch. */
int rdg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RDG_H */
