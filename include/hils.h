/*
 * hils.h -- C ABI of the HiLS-Attention forward path on AMD Instinct MI355X (gfx950).
 *
 * HiLS-Attention ("Hierarchical Sparse Attention Done Right: Toward Infinite
 * Context Modeling") factorises causal attention hierarchically: every query
 * attends, independently, to each retrieved chunk and to a chunk-aligned
 * sliding window, and the per-group results are fused with weights given by
 * learned chunk retrieval scores.  This library computes the forward pass in
 * four calls:
 *
 *   hils_summarize    landmark chunk summaries (k', b')
 *   hils_select       retrieval scores and top-k chunk selection
 *   hils_attend_fuse  per-group attention and the fusion
 *   hils_decode_step  all of the above for one new token per sequence
 *   hils_decode_multi the same for several adjacent new tokens per sequence
 *
 * and the gradients of the prefill path in two more:
 *
 *   hils_attend_fuse_backward  attention and fusion, given the selection
 *   hils_summarize_backward    the landmark summaries
 *
 * plus a selection diagnostic (naive Block Sparse Attention's exact chunk-mass
 * top-k, and the overlap of two selections):
 *
 *   hils_bsa_select, hils_selection_overlap
 *
 * and the two variants of the steps before scoring: the calibrated retrieval
 * query and summaries from one shared query per head:
 *
 *   hils_qcal, hils_select_qcal, hils_summarize_shared
 *
 * Notation: B batch, Hq query heads, Hkv key/value heads, G = Hq/Hkv heads per
 * group, d head dimension, S chunk size, W window, k top-k, T tokens,
 * NC = floor(T/S) complete chunks, scale = 1/sqrt(d) unless given.  Token i
 * lies in chunk floor(i/S).  The window of position i is [l_i, i] with
 * l_i = max(0, S*floor((i-W+1)/S)) (its left edge rounded down to a chunk
 * boundary); the candidate chunks of i are C_i = {c : (c+1)*S <= l_i}, the
 * complete chunks left of the window (paper-body page, Block Sparse Attention
 * preliminaries).
 *
 * Conventions for every call:
 *  - Tensors are caller-owned device memory, contiguous and row-major,
 *    head-major ([B, H, T, d]), 16-byte aligned.  The compute calls allocate no
 *    memory and keep no pointer after returning; their scratch memory is the
 *    caller's workspace, sized by hils_workspace_bytes().  Calls on different
 *    streams may run concurrently as long as their buffers are disjoint.  The
 *    only process-wide state is the optional kernel timing below (off unless
 *    hils_timing_enable() switched it on), which keeps a pool of HIP events.
 *  - Every check runs on the host before anything is enqueued.  A nonzero
 *    status means nothing was enqueued and nothing was written.  Work is
 *    asynchronous on `stream` (NULL = the default stream); a fault inside a
 *    kernel surfaces at the caller's next synchronisation with that stream.
 *  - Outputs are overwritten completely (index pads -1, score pads -inf).
 *  - Supported: d in {64, 128}; S = 64; Hq % Hkv == 0 with G in {1, 2, 4, 8};
 *    0 <= k <= 64; W >= 1; io_dtype in {F32, BF16} and
 *    summary_dtype == io_dtype.  Anything else returns HILS_E_UNSUPPORTED.
 *  - Results are deterministic: the same inputs give bitwise identical
 *    outputs on every run.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HILS_ABI_VERSION 3

typedef enum {
    HILS_OK = 0,
    HILS_E_NULL = -1,          /* a required pointer is NULL */
    HILS_E_SHAPE = -2,         /* inconsistent or out-of-range sizes */
    HILS_E_DTYPE = -3,         /* unknown dtype code */
    HILS_E_ALIGN = -4,         /* a tensor pointer is not 16-byte aligned */
    HILS_E_WORKSPACE = -5,     /* workspace missing or smaller than required */
    HILS_E_POS = -6,           /* decode position outside the cache */
    HILS_E_NEED_QLAND = -7,    /* a chunk completes but no landmark query was given */
    HILS_E_UNSUPPORTED = -8,   /* valid, but outside what this build implements */
    HILS_E_LAUNCH = -9,        /* the HIP runtime refused a launch */
    HILS_E_SCRATCH = -10       /* the shape needs more than the built-in scratch
                                  of hils_decode_step_noalloc */
} hils_status;

typedef enum { HILS_F32 = 0, HILS_BF16 = 1 } hils_dtype;

typedef enum {
    HILS_OP_SUMMARIZE = 0,
    HILS_OP_SELECT = 1,
    HILS_OP_ATTEND_FUSE = 2,
    HILS_OP_DECODE = 3,
    HILS_OP_ATTEND_BACKWARD = 4
} hils_op;

typedef struct {
    int32_t batch;          /* B */
    int32_t heads_q;        /* Hq */
    int32_t heads_kv;       /* Hkv */
    int32_t head_dim;       /* d */
    int32_t chunk;          /* S */
    int32_t window;         /* W */
    int32_t top_k;          /* k */
    int64_t seq_len;        /* prefill: T; decode: cache capacity Lcap (a multiple of S) */
    float scale;            /* logit scale; 0 selects 1/sqrt(d) */
    hils_dtype io_dtype;    /* q, q_hat, q_land, k, v, out */
    hils_dtype summary_dtype; /* k' (b' is always fp32) */
} hils_shape;

/*
 * Landmark chunk summaries (summary page, Methodology 1, Eq. 8; paper-body
 * page, RQ1: the landmark token appended to a chunk supplies q'_c, and the
 * pair (k', b') is the chunk's entropy-calibrated compressed key).
 * For every b, query head h (KV head g = h/G) and chunk c in
 * [chunk_begin, chunk_begin + n_chunks):
 *     s_j = scale * q'_{h,c} . k_{g, cS+j},  j = 0..S-1,   p = softmax(s)
 *     k'_{h,c} = sum_j p_j k_{g,cS+j}      (rounded once to summary_dtype)
 *     b'_{h,c} = -sum_j p_j log p_j        (fp32)
 *
 * k       [B, Hkv, seq_len, d]      io_dtype (rows of chunks in range are read)
 * q_land  [B, Hq,  seq_len/S, d]    io_dtype
 * k_sum   [B, Hq,  seq_len/S, d]    summary_dtype; only the chunks in range are written
 * b_sum   [B, Hq,  seq_len/S]       fp32; likewise
 * Requires 0 <= chunk_begin, chunk_begin + n_chunks <= seq_len/S.  n_chunks == 0
 * is a no-op.  Needs no workspace.
 */
hils_status hils_summarize(const hils_shape* shape, const void* k, const void* q_land,
                           int64_t chunk_begin, int64_t n_chunks,
                           void* k_sum, float* b_sum, hipStream_t stream);

/*
 * Landmark summaries with one shared query per head (paper-body page,
 * implementation: a learnable query shared by every chunk of a layer, in place
 * of the landmark tokens): hils_summarize with q'_{h,c} = q_shared[h] for every
 * sequence b and chunk c.
 * q_shared [Hq, d] io_dtype; the other arguments, limits and errors as
 * hils_summarize.
 */
hils_status hils_summarize_shared(const hils_shape* shape, const void* k, const void* q_shared,
                                  int64_t chunk_begin, int64_t n_chunks,
                                  void* k_sum, float* b_sum, hipStream_t stream);

/*
 * Low-rank query calibration of the retrieval query (paper-body page,
 * implementation: Q-Cal; summary page, practical enhancements): the query that
 * scores the chunk summaries is the token query plus a rank-r correction of
 * the token's hidden state,
 *     q_hat[b,h,t,:] = q[b,h,t,:] + W_up[h] (W_down hs[b,t,:])
 * computed in fp32 (both products and the add) and rounded once to io_dtype:
 * the q_hat that hils_select and hils_decode_step read.
 * q [B,Hq,T,d], hs [B,T,d_model], w_down [rank,d_model], w_up [Hq,d,rank]: io_dtype
 * q_hat [B,Hq,T,d] io_dtype out (must not be q: HILS_E_SHAPE).
 * Requires d_model a multiple of 32 (at most 65536) and rank in {16, 32, 64, 128},
 * else HILS_E_UNSUPPORTED.  Needs no workspace.
 */
hils_status hils_qcal(const hils_shape* shape, const void* q, const void* hs, const void* w_down,
                      const void* w_up, int32_t d_model, int32_t rank, void* q_hat,
                      hipStream_t stream);

/*
 * Retrieval scores and top-k selection (paper-body page, RQ1: every complete
 * chunk's summary is scored with the linear estimate of Eq. 7 and the k highest
 * are chosen; summary page, Eq. 10: s_hat = q_hat . k' / sqrt(d) + b';
 * paper-body page, GQA-aware chunk selection).  For every b, position i < T and group g:
 *     s_hat_{h,i,c} = scale * q_hat_{h,i} . k'_{h,c} + b'_{h,c},   c in C_i
 *     rank key r_c  = s_hat_{h,i,c}                              (G == 1)
 *                   = max_{h in g} (s_hat_{h,i,c} - LSE_{c' in C_i} s_hat_{h,i,c'})   (G > 1)
 *     Sel = the k candidates with the largest r (equal r: lower c first);
 *           all of C_i when |C_i| <= k.
 * The max over heads of log-normalised scores ranks chunks exactly as the max
 * over heads of each head's softmax weights over C_i.
 *
 * q_hat     [B, Hq, T, d]        io_dtype (the calibrated query; pass q when none)
 * k_sum     [B, Hq, T/S, d]      summary_dtype
 * b_sum     [B, Hq, T/S]         fp32
 * sel_idx   [B, Hkv, T, k]       int32 out: chunk ids ascending, -1 padded
 * sel_score [B, Hq, T, k]        fp32 out: each head's s_hat at sel_idx, -inf padded
 * Requires T <= 64 * 8192 (at most 8192 chunks: the 512K context) for this build.
 * The workspace holds each head's LSE and the rank keys of every (b, group); a
 * workspace smaller than hils_workspace_bytes() but holding at least one
 * (b, group)'s keys runs the same computation a few (b, group) pairs at a time.
 * On return, for G > 1, the workspace starts (at its first 256-byte aligned
 * address) with L [B, Hq, T] fp32: each head's L_{h,i} = LSE_{c in C_i} s_hat_{h,i,c}
 * as used in the rank keys (-inf where C_i is empty), so that a caller can
 * rebuild the rank key of every chosen chunk from sel_score.
 */
hils_status hils_select(const hils_shape* shape, const void* q_hat, const void* k_sum,
                        const float* b_sum, int32_t* sel_idx, float* sel_score,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * hils_select with the query calibration fused into scoring (paper-body page,
 * implementation: Q-Cal, applied to the retrieval query only; summary page,
 * practical enhancements).  The down-projection z = W_down hs (fp32, shared by
 * every head) runs once per token; the first scoring pass then forms each
 * query's q_hat = q + W_up[h] z, rounds it once and scores with it, and stores
 * it for the later passes (it is also the caller's q_hat).  The results are bit
 * for bit those of hils_qcal followed by hils_select.
 * q, hs, w_down, w_up, d_model, rank: as hils_qcal; k_sum, b_sum, sel_idx,
 * sel_score: as hils_select; q_hat [B,Hq,T,d] io_dtype out (must not be q).
 * Workspace: hils_select_qcal_workspace_bytes(shape, rank) (z first, then the
 * selection's workspace with the same rules as hils_select's; its L table
 * starts at the first 256-byte boundary after z).  With k = 0 only q_hat is
 * computed.  Same limits and errors as hils_qcal and hils_select.
 */
hils_status hils_select_qcal(const hils_shape* shape, const void* q, const void* hs, const void* w_down,
                             const void* w_up, int32_t d_model, int32_t rank, const void* k_sum,
                             const float* b_sum, void* q_hat, int32_t* sel_idx, float* sel_score,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of hils_select_qcal for `shape` and `rank` (0 when unsupported). */
size_t hils_select_qcal_workspace_bytes(const hils_shape* shape, int32_t rank);

/*
 * Per-group attention and fusion (summary page, Methodology 2, Eq. 10, the
 * hierarchical softmax; paper-body page, implementation: the normaliser adds
 * the window's exact token-level mass to the selected chunks' surrogate
 * masses).  For every b, query head h (group g), position i:
 *     for each selected chunk c and for the window Win_i = [l_i, i]:
 *         s_ij = scale * q_{h,i} . k_{g,j}
 *         log Z_gamma = LSE_j s_ij,   o_gamma = sum_j exp(s_ij - log Z_gamma) v_{g,j}
 *     log Zhat_i = LSE({s_hat_c : c in Sel} + {log Z_win})   (the window enters
 *                  at its true token-level log-mass)
 *     out_i = sum_c exp(s_hat_c - log Zhat_i) o_c + exp(log Z_win - log Zhat_i) o_win
 *     lse_i = log Zhat_i
 * Token logits use q (not q_hat).
 *
 * q [B,Hq,T,d], k and v [B,Hkv,T,d]: io_dtype
 * sel_idx [B,Hkv,T,k] and sel_score [B,Hq,T,k]: as written by hils_select
 * (each row's valid ids ascending and < |C_i|, pads -1 at the end)
 * out [B,Hq,T,d] io_dtype; lse [B,Hq,T] fp32 or NULL.
 * The workspace holds per-(query, head, selected chunk) partial outputs; a
 * workspace smaller than hils_workspace_bytes() but at least the size for one
 * KV head runs the same computation in several passes.
 */
hils_status hils_attend_fuse(const hils_shape* shape, const void* q, const void* k, const void* v,
                             const int32_t* sel_idx, const float* sel_score,
                             void* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step for every sequence of the batch (summary page, Summary:
 * constant per-token decoding; the step is the prefill row i = pos[b] of the
 * definitions above).  For each b with position i = pos[b]:
 *   1. write k_new, v_new into row i of the caches;
 *   2. select over C_i using the cached summaries and q_hat (as hils_select);
 *   3. attend and fuse for query q over the selection and the window [l_i, i]
 *      (which includes the new token) (as hils_attend_fuse);
 *   4. if (i+1) % S == 0, summarise the chunk that token i completes with
 *      q_land_new[b] into row i/S of k_sum, b_sum (as hils_summarize).  That chunk
 *      is never a candidate of its own completing step, since W >= 1.
 * The caller owns and advances pos.
 *
 * pos        host array [B]: 0 <= pos[b] < seq_len (seq_len = cache capacity)
 * q, q_hat   [B, Hq, d]      io_dtype
 * k_new, v_new [B, Hkv, d]   io_dtype
 * q_land_new [B, Hq, d] io_dtype, or NULL when no sequence completes a chunk
 *            (HILS_E_NEED_QLAND otherwise)
 * k_cache, v_cache [B, Hkv, seq_len, d] io_dtype (rows <= pos[b] valid after step 1)
 * k_sum [B, Hq, seq_len/S, d] summary_dtype, b_sum [B, Hq, seq_len/S] fp32:
 *            rows of every complete chunk before pos[b] must be valid
 * out [B, Hq, d] io_dtype; lse [B, Hq] fp32 or NULL; sel_idx [B, Hkv, k] int32 or NULL
 */
hils_status hils_decode_step(const hils_shape* shape, const int64_t* pos,
                             const void* q, const void* q_hat,
                             const void* k_new, const void* v_new, const void* q_land_new,
                             void* k_cache, void* v_cache, void* k_sum, float* b_sum,
                             void* out, float* lse, int32_t* sel_idx,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The decode step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments and results are those of
 * hils_decode_step; the scratch memory is the library's own, a static device
 * array of HILS_NOALLOC_SCRATCH_BYTES bytes that each GPU holds until the
 * process ends (its address is looked up once per device, on the first call
 * with that device current).  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.  A shape whose decode workspace
 * (hils_workspace_bytes(shape, HILS_OP_DECODE)) exceeds the scratch returns
 * HILS_E_SCRATCH with nothing enqueued (512K tokens x 4 sequences, 32/8 heads,
 * needs about 8 MiB; 4M tokens x 1 sequence about 9 MiB).  Every call on one
 * GPU shares that GPU's scratch: calls that may overlap on one GPU (different
 * streams, different host threads) race and must be serialised by the caller.
 * Each call writes every scratch element it reads, so no clearing is needed
 * between calls.
 */
#define HILS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hils_status hils_decode_step_noalloc(const hils_shape* shape, const int64_t* pos,
                                     const void* q, const void* q_hat,
                                     const void* k_new, const void* v_new, const void* q_land_new,
                                     void* k_cache, void* v_cache, void* k_sum, float* b_sum,
                                     void* out, float* lse, int32_t* sel_idx, hipStream_t stream);

/*
 * Backward of hils_attend_fuse and of the retrieval scores that weight it
 * (paper-body page, RQ2: the chunk scores enter the fused token weights, so the
 * loss gradient reaches the summaries and the calibrated query; summary page,
 * Methodology 2, Eq. 10).  The selection is held fixed: top-k is piecewise
 * constant in the inputs and has no gradient.  With upstream gradients
 * g = dout and gl = dlse of a row (b, h, i), its forward output out and lse = L:
 *     D = g . out;  window token j: a_j = exp(s_ij - L),
 *         ds_ij = a_j (g . v_j - D + gl),  dv_j += a_j g
 *     selected chunk c, w_c = exp(s_hat_c - L), p = the chunk's softmax of s_ij,
 *         D_c = sum_j p_j g . v_j,  ds_ij = w_c p_j (g . v_j - D_c),
 *         dv_j += w_c p_j g,  d s_hat_c = w_c (D_c - D + gl)
 *     dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_(h,i) ds_ij q_i
 *     dq_hat_i = scale sum_c d s_hat_c k'_c,  dk'_c = scale sum_i d s_hat_c q_hat_i,
 *     db'_c = sum_i d s_hat_c
 * (sums over the G heads of a group for dk and dv).
 *
 * q, k, v, q_hat, k_sum, sel_idx, sel_score: the inputs of the forward calls
 *   (k_sum [B,Hq,T/S,d] summary_dtype; sel_idx and sel_score as from hils_select)
 * out [B,Hq,T,d] io_dtype and lse [B,Hq,T] fp32: as written by hils_attend_fuse
 * dout [B,Hq,T,d] io_dtype; dlse [B,Hq,T] fp32, or NULL for a zero gradient
 * dq, dq_hat [B,Hq,T,d], dk, dv [B,Hkv,T,d], dk_sum [B,Hq,T/S,d], db_sum [B,Hq,T/S]:
 *   fp32 outputs, overwritten (zero where nothing reaches them)
 * The workspace (hils_workspace_bytes(shape, HILS_OP_ATTEND_BACKWARD)) holds
 * per-(query, head, selected chunk) dq parts; one smaller than that but with
 * room for one KV head's parts runs several passes.  Same limits as
 * hils_attend_fuse.
 */
hils_status hils_attend_fuse_backward(const hils_shape* shape, const void* q, const void* k,
                                      const void* v, const void* q_hat, const void* k_sum,
                                      const int32_t* sel_idx, const float* sel_score,
                                      const void* out, const float* lse, const void* dout,
                                      const float* dlse, float* dq, float* dk, float* dv,
                                      float* dq_hat, float* dk_sum, float* db_sum,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of hils_summarize (summary page, Methodology 1, Eq. 8: the gradients
 * of k'_c and b'_c flow through the chunk's softmax to the landmark query and
 * the chunk's keys).  For each b, h, chunk c in range, with s_j, p as in
 * hils_summarize:
 *     e_j = dk'_c . k_j - db'_c s_j,   ds_j = p_j (e_j - sum_l p_l e_l)
 *     dq_land_c = scale sum_j ds_j k_j
 *     dk_j += p_j dk'_c + scale ds_j q_land_c      (summed over the group's heads)
 * k [B,Hkv,seq_len,d] and q_land [B,Hq,seq_len/S,d] io_dtype: the forward inputs
 * dk_sum [B,Hq,seq_len/S,d] and db_sum [B,Hq,seq_len/S] fp32: the gradients of k_sum, b_sum
 * dk [B,Hkv,seq_len,d] fp32: added to (rows of chunks in range only)
 * dq_land [B,Hq,seq_len/S,d] fp32: written for the chunks in range
 * Requires 0 <= chunk_begin, chunk_begin + n_chunks <= seq_len/S; n_chunks == 0
 * is a no-op.  Needs no workspace.  The summary's forward rounding of k' to
 * summary_dtype is passed through unchanged.
 */
hils_status hils_summarize_backward(const hils_shape* shape, const void* k, const void* q_land,
                                    const float* dk_sum, const float* db_sum, int64_t chunk_begin,
                                    int64_t n_chunks, float* dk, float* dq_land, hipStream_t stream);

/*
 * Naive Block Sparse Attention selection, a diagnostic of the retrieval
 * (paper-body page, Block Sparse Attention preliminaries: a chunk's mass is the
 * sum of the query's exponentiated token logits over the chunk, and naive BSA
 * keeps the k candidates of largest mass; it needs every token logit, so its
 * cost grows as T^2 d, and it is not part of the HiLS path).  For every b,
 * position i < T and group g:
 *     log Z_{h,i,c} = LSE_{j in chunk c} scale * q_{h,i} . k_{g,j},   c in C_i
 *     rank key and Sel exactly as hils_select, with log Z in place of s_hat.
 * q [B,Hq,T,d] and k [B,Hkv,T,d]: io_dtype (the token query, not q_hat)
 * sel_idx [B,Hkv,T,k] int32 out: chunk ids ascending, -1 padded
 * Workspace: hils_workspace_bytes(shape, HILS_OP_SELECT), with the same rule for
 * a smaller one (at least one (b, group)'s keys: several passes).
 */
hils_status hils_bsa_select(const hils_shape* shape, const void* q, const void* k, int32_t* sel_idx,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Overlap of two selections of the same shape (for the recall of HiLS's
 * selection against naive BSA's): count[b,g,i] = the number of chunk ids that
 * rows (b, g, i) of idx_a and idx_b [B,Hkv,T,k] (ascending, -1 padded) share.
 * count [B,Hkv,T] int32 out.  Needs no workspace.
 */
hils_status hils_selection_overlap(const hils_shape* shape, const int32_t* idx_a, const int32_t* idx_b,
                                   int32_t* count, hipStream_t stream);

/*
 * Several adjacent queries per sequence in one step: speculative or multi-token
 * decoding (paper-body page, implementation, kernel design: adjacent queries
 * attend the union of their selected chunks, which fills the matrix tiles with
 * M x G rows and loads each chunk once; the summary page's practical
 * enhancements).  For each b the n_queries = M new tokens sit at positions
 * pos[b] + m (m < M); token m is exactly the prefill row i = pos[b] + m of the
 * definitions above, so it sees the earlier new tokens of its sequence:
 *   1. write k_new, v_new row m into cache row pos[b] + m;
 *   2. for each m: select over C_i (as hils_select), attend and fuse (as
 *      hils_attend_fuse) over the cache rows <= i;
 *   3. summarise the chunk completed by these tokens, if any (at most one per
 *      sequence), with q_land_new[b] (as hils_decode_step).
 * Every k' row is read once for up to four queries of a sequence, and each chunk
 * of the union of a (b, group)'s M selections is attended once for all M G
 * (query, head) pairs.
 * q, q_hat [B, M, Hq, d]; k_new, v_new [B, M, Hkv, d]; q_land_new [B, Hq, d] or NULL
 * (io_dtype); caches, k_sum, b_sum as hils_decode_step;
 * out [B, M, Hq, d] io_dtype; lse [B, M, Hq] fp32 or NULL; sel_idx [B, M, Hkv, k] or NULL.
 * Requires 1 <= M <= min(16, W) (else HILS_E_SHAPE), M G <= 16, B M <= 64 and, for
 * M > 1, k + W / S + 3 <= 256 (else HILS_E_UNSUPPORTED), pos[b] + M <= cache
 * capacity (else HILS_E_POS), the same
 * shape limits as hils_decode_step; workspace hils_decode_multi_workspace_bytes().
 * M = 1 runs hils_decode_step.
 */
hils_status hils_decode_multi(const hils_shape* shape, int32_t n_queries, const int64_t* pos,
                              const void* q, const void* q_hat, const void* k_new, const void* v_new,
                              const void* q_land_new, void* k_cache, void* v_cache, void* k_sum,
                              float* b_sum, void* out, float* lse, int32_t* sel_idx,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of hils_decode_multi for `shape` and n_queries (0 when either
 * is outside its limits). */
size_t hils_decode_multi_workspace_bytes(const hils_shape* shape, int32_t n_queries);

/* Workspace bytes `op` needs for `shape` (0 for HILS_OP_SUMMARIZE); 0 as well
 * for an invalid shape. */
size_t hils_workspace_bytes(const hils_shape* shape, hils_op op);

/* Static, human-readable name of a status code. */
const char* hils_status_string(hils_status status);

/* HILS_ABI_VERSION of the built library. */
int hils_abi_version(void);

/* ---- Diagnostics: per-kernel timing ------------------------------------
 * Not part of the computation.  While enabled, each launch of a selected
 * kernel is bracketed by two HIP events recorded on the stream it is launched
 * on, so the measured time is that kernel's own duration on the device.
 *
 * hils_timing_enable(kernels): kernels is a comma-separated list of kernel
 *   names, "*" for all, or NULL to switch timing off.  Enabling clears every
 *   earlier record (after waiting for its events).  Names: summarize,
 *   score_lse, idx_count, idx_scan_tiles, idx_scan_buckets,
 *   idx_fill, lsel, window (window attention and the fusion), chunk_attend,
 *   dec_score, dec_select,
 *   dec_attend, dec_fuse, dec_summarize (the summaries of chunks
 *   completed by a decode step), v_transpose, rank_keys,
 *   topk_scores, for the backward calls bwd_rowstat, bwd_kv, bwd_dq,
 *   bwd_qhat and summarize_bwd (the entry lists of the
 *   backward count under the idx_* names), bsa_keys, bsa_topk, qcal,
 *   qcal_zdown (the down-projection of hils_select_qcal, whose fused scoring
 *   pass counts as score_lse), and for hils_decode_multi dec_append and
 *   dec_gsel (its other kernels count under the dec_* names above).  HILS_E_UNSUPPORTED for an unknown name
 *   (timing is then left off).
 * hils_timing_get(kernel, total_ms, launches): waits for the recorded events
 *   of that kernel and returns the summed duration and the number of timed
 *   launches since the last enable.  HILS_E_NULL for NULL outputs or name,
 *   HILS_E_UNSUPPORTED for an unknown name.
 * The timing state is process-wide and not thread-safe; calls that launch
 * while timing is enabled must come from one host thread. */
hils_status hils_timing_enable(const char* kernels);
hils_status hils_timing_get(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H_ */
