/*
 * bllm.h -- C ABI of the dynamic-chunking layer of tokenizer-free hierarchical
 * byte models, built for AMD Instinct MI355X (gfx950).
 *
 * Two downsamplers and two upsamplers sit between a byte-level local encoder
 * and a global model:
 *   H-Net style:   bllm_route -> bllm_compact -> ... -> bllm_dechunk_ema
 *   ByteFlow:      bllm_coding_rate -> bllm_topk_select -> bllm_compact (gather)
 *                  -> ... -> bllm_upsample_bins
 *
 * Sources of the operations (page titles; sections as on the page):
 *   [BG]  "ByteGen: A Tokenizer-Free Generative Model for Orderbook Events in
 *         Byte Space" analyst report, section 2.3 Methodology.
 *   [BF2] "ByteFlow: Language Modeling through Adaptive Byte Compression
 *         without a Tokenizer" paper notes, key designs 2 and 4.
 *   [BF4] ByteFlow paper page (arXiv 2603.03583), "lossy coding rate"
 *         prerequisite and "method step details" stages 2 and 4.
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to caller-owned memory.  The
 *     library never allocates device memory, frees or synchronises; every
 *     call only enqueues kernels on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream) and returns.  The library keeps no state
 *     between calls (no streams, events or memory of its own), so calls from
 *     several host threads on different streams are independent.
 *   - Scratch memory comes in through (ws, ws_bytes); its size is given by the
 *     matching bllm_*_workspace() function.  Contents need not be initialised
 *     and are clobbered.  Workspaces must not be shared by calls that may
 *     run concurrently.
 *   - Row-major, densely packed rows.  A ragged batch is packed rows of all
 *     sequences back to back plus `offsets` (int64 [nseq+1], device,
 *     offsets[0] = 0, non-decreasing, offsets[nseq] = total).
 *   - dtype is BLLM_F32 or BLLM_BF16 (bf16 bit patterns, fp32 accumulation,
 *     round-to-nearest-even on output).  Row pointers must be 16-byte aligned
 *     and d * element size a multiple of 16 bytes.
 *   - An empty batch (total = 0) is valid: data pointers of the empty arrays
 *     may then be NULL (offsets and chunk offsets are still required).
 *   - Return value: BLLM_OK or a negative BLLM_E_* code.  Argument errors are
 *     detected on the host before anything is enqueued.  Data-dependent
 *     conditions (capacity overflow, non-finite values) are reported through
 *     an optional device int32 `status` word that the call ORs flags into
 *     (BLLM_S_* bits); the caller zeroes it beforehand and reads it after its
 *     own synchronisation.
 */
#ifndef BLLM_H
#define BLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define BLLM_OK 0
#define BLLM_E_INVAL (-1)  /* bad argument (null pointer, size out of range) */
#define BLLM_E_NOTSUP (-2) /* valid but unsupported shape/dtype/alignment     */
#define BLLM_E_WS (-3)     /* workspace too small                            */
#define BLLM_E_HIP (-4)    /* the HIP runtime reported an error at launch    */

/* device status flags (ORed into *status) */
#define BLLM_S_CAPACITY 1  /* compaction produced more rows than `capacity`   */
#define BLLM_S_NONFINITE 2 /* a NaN/Inf input or a non-positive pivot was met */
#define BLLM_S_INCOMPLETE 4 /* a bounded device-side wait gave up: the stage
                               quantile's workgroups were not all resident
                               within about a second; tau and b are invalid   */

/* dtypes */
#define BLLM_F32 0
#define BLLM_BF16 1

int bllm_version(void);
const char* bllm_status_string(int code);

/*
 * bllm_route -- H-Net boundary scoring ([BG] 2.3: boundary probability from
 * the cosine similarity of adjacent byte representations).
 *
 *   p_t = (1 - cos(q_t, k_{t-1})) / 2, clamped to [0, 1];  p = 1 at every
 *   sequence start (no pair crosses offsets).  cos = <q,k> / max(|q||k|, 1e-12).
 *   b_t = [p_t >= tau] decided in fp32; NaN p gives b = 0.
 *   tau = threshold when quantile < 0; otherwise tau is the order statistic
 *   of rank floor(quantile * (total - 1)) (0-based, ascending, NaN last) of all
 *   `total` scores of the batch (one threshold per call = per hierarchy stage).
 *
 * q, k     : [total x d] rows of dtype (the routing projections of h).
 * offsets  : int64 [nseq+1] device.
 * p_out    : fp32 [total]; b_out : uint8 [total] (0/1); tau_out : fp32 [1]
 *            device, may be NULL.
 * status   : optional device word (may be NULL).  With a quantile, the
 *            threshold is found by one launch whose workgroups meet at
 *            grid-wide barriers with a bounded wait; if a wait gives up,
 *            BLLM_S_INCOMPLETE is ORed in and tau (NaN) and b must not be used.
 * ws       : bllm_route_workspace(total) bytes (needed when quantile >= 0).
 * Errors   : BLLM_E_INVAL for null q/k/offsets/p_out/b_out, d < 1, nseq < 1,
 *            total < 0, quantile > 1; BLLM_E_NOTSUP for bad dtype/alignment.
 */
size_t bllm_route_workspace(int64_t total);
int bllm_route(const void* q, const void* k, int dtype, int64_t d, const int64_t* offsets,
               int64_t nseq, int64_t total, float threshold, double quantile, float* p_out,
               uint8_t* b_out, float* tau_out, int32_t* status, void* ws, size_t ws_bytes,
               void* stream);

/*
 * bllm_route_fused -- bllm_route computed straight from the encoder output:
 * q = h Wq and k = h Wk (row-vector convention, fp32 accumulation of the bf16
 * products) are formed on the fly and never stored; p, b and tau follow
 * exactly as in bllm_route.
 *
 * h        : [total x d] bf16 rows; Wq, Wk : [d x d] bf16, row-major.
 * d        : a multiple of 128, at most 4096 (else BLLM_E_NOTSUP); bf16 only.
 * Other arguments, outputs, workspace (bllm_route_workspace) and errors as
 * for bllm_route.
 */
int bllm_route_fused(const void* h, const void* Wq, const void* Wk, int dtype, int64_t d,
                     const int64_t* offsets, int64_t nseq, int64_t total, float threshold,
                     double quantile, float* p_out, uint8_t* b_out, float* tau_out,
                     int32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * bllm_compact -- keep the boundary positions of a ragged batch ([BG] 2.3
 * chunking into a shorter sequence; also the gather z = [h_{s_1} .. h_{s_K}]
 * of [BF4] stage 2 when `mask` is the Top-K mask).
 *
 *   idx_out[r]          = global position of the r-th set mask byte (ascending)
 *   chunk_offsets_out[s]= number of set bytes before offsets[s]  (int64 [nseq+1];
 *                         chunk_offsets_out[nseq] = M, the total count)
 *   rows_out[r]         = rows[idx_out[r]]   (if rows != NULL)
 *   P_out[r]            = p[idx_out[r]]      (if p != NULL)
 * At most `capacity` entries are written; if M > capacity the
 * BLLM_S_CAPACITY flag is set in *status (chunk_offsets still hold the true
 * counts).  idx_out is int32 (total must be < 2^31).
 * ws: bllm_compact_workspace(total) bytes.
 */
size_t bllm_compact_workspace(int64_t total);
int bllm_compact(const uint8_t* mask, const float* p, const void* rows, int dtype, int64_t d,
                 const int64_t* offsets, int64_t nseq, int64_t total, int64_t capacity,
                 int32_t* idx_out, int64_t* chunk_offsets_out, void* rows_out, float* P_out,
                 int32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * bllm_compact_noalloc -- bllm_compact for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid hipMalloc): the same operation, arguments, outputs and status, with
 * no workspace argument.  The scratch the kernels need lives in a static
 * device array of the library (262,656 bytes, one copy per GPU, held until the
 * process ends); its address is looked up once per device at the first call.
 * The call allocates nothing and calls no allocating routine.
 * Limit  : total <= 2^27 (134,217,728 positions), else BLLM_E_WS and nothing
 *          is enqueued.
 * Sharing: every call on one GPU uses that GPU's one array, so calls that
 *          may overlap on the same GPU (other streams, other threads) race;
 *          calls queued in order on one stream are safe.  The kernels write
 *          every scratch word before reading it, so no clearing is needed.
 * Errors : as bllm_compact; BLLM_E_HIP if the array's address cannot be found.
 */
int bllm_compact_noalloc(const uint8_t* mask, const float* p, const void* rows, int dtype, int64_t d,
                         const int64_t* offsets, int64_t nseq, int64_t total, int64_t capacity,
                         int32_t* idx_out, int64_t* chunk_offsets_out, void* rows_out, float* P_out,
                         int32_t* status, void* stream);

/*
 * bllm_dechunk_ema -- EMA smoothing back to byte length ([BG] 2.3).
 *
 *   per sequence s, over its chunks c = chunk_offsets[s] .. chunk_offsets[s+1]-1:
 *     zbar_c = P_c * z_c + (1 - P_c) * zbar_{c-1},  zbar before the first chunk = 0
 *   out_t = zbar_{c(t)} for every position t of the sequence, c(t) the last chunk
 *   with idx[c] <= t; positions before a sequence's first chunk get 0.
 *
 * z        : [max_chunks x d] dtype, P : fp32 [max_chunks], idx : int32
 *            [max_chunks] (global positions, ascending, inside their
 *            sequence), chunk_offsets : int64 [nseq+1] device (read on the
 *            device).
 * max_chunks: the number of chunk rows the caller provides (typically the
 *            compaction capacity).  Every chunk offset is clamped to it on the
 *            device, so M = min(chunk_offsets[nseq], max_chunks) chunks are
 *            used and nothing past row max_chunks - 1 of z, P or idx is read:
 *            after a compaction that overflowed its capacity (BLLM_S_CAPACITY;
 *            chunk_offsets then hold the true counts), the chunks it could not
 *            store are absent -- a sequence cut short keeps its last stored
 *            chunk to its end, a sequence left without chunks gets zero rows.
 *            z, P and idx may be NULL when max_chunks = 0.
 * out      : [total x d] dtype.
 * ws       : bllm_dechunk_workspace(d) bytes.
 */
size_t bllm_dechunk_workspace(int64_t d);
int bllm_dechunk_ema(const void* z, const float* P, int dtype, int64_t d, const int32_t* idx,
                     const int64_t* chunk_offsets, const int64_t* offsets, int64_t nseq,
                     int64_t total, int64_t max_chunks, void* out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * bllm_dechunk_ema_backward -- gradients of the EMA dechunk ([BG] 2.3: the
 * EMA over chunks keeps the boundary choice differentiable end to end).
 *
 * With L = sum over positions t and features of dout[t] * out[t] for the
 * out of bllm_dechunk_ema(z, P, idx, chunk_offsets, offsets), per chunk c:
 *   gbar_c = sum of dout over the positions chunk c covers
 *   lam_c  = gbar_c + (1 - P_{c+1}) lam_{c+1}   (lam_c = gbar_c for a
 *            sequence's last chunk)
 *   dz_out[c] = dL/dz_c = P_c lam_c
 *   dP_out[c] = dL/dP_c = lam_c . (z_c - zbar_{c-1}), zbar_{c-1} = 0 at a
 *            sequence's first chunk (zbar: the forward EMA, recomputed here
 *            in fp32 from z and P)
 * Arguments as for bllm_dechunk_ema, plus dout : [total x d] dtype (the
 * gradient of out), dz_out : [M x d] dtype (RNE for bf16), dP_out : fp32 [M].
 * max_chunks: the number of chunk rows provided, clamping the chunk offsets
 *            exactly as in bllm_dechunk_ema (dz_out and dP_out are written for
 *            the M used); it also sizes the workspace.
 * ws       : bllm_dechunk_ema_backward_workspace(d, max_chunks) bytes.
 * Errors   : as bllm_dechunk_ema; dout/dz_out must be 16-byte aligned.
 */
size_t bllm_dechunk_ema_backward_workspace(int64_t d, int64_t max_chunks);
int bllm_dechunk_ema_backward(const void* z, const float* P, const void* dout, int dtype, int64_t d,
                              const int32_t* idx, const int64_t* chunk_offsets,
                              const int64_t* offsets, int64_t nseq, int64_t total,
                              int64_t max_chunks, void* dz_out, float* dP_out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * bllm_coding_rate -- marginal lossy coding rate ([BF4] prerequisite "lossy
 * coding rate" and stage 2):
 *   R(H) = 1/2 logdet(I + alpha H H^T) = 1/2 logdet(I_d + alpha H^T H),
 *   alpha = d / eps2,  dR_t = R(h_1..t) - R(h_1..t-1)  for t = 0..T-1 (0-based;
 *   dR_0 = R(h_1)).
 * Computed exactly (up to fp32 rounding) as the logs of the Cholesky pivots of
 * I_T + alpha H H^T, obtained block by block from the d x d prefix matrices
 * (the incremental Sherman-Morrison-Woodbury route the [BF4] weakness
 * analysis suggests).
 *
 * h : [nseq x T x d] dtype, dense.  dR_out : fp32 [nseq x T].
 * status : optional device word (BLLM_S_NONFINITE on NaN/Inf or lost
 *          positive definiteness).
 * Limits : 1 <= d <= 640 (BLLM_E_NOTSUP beyond), T >= 1, eps2 > 0.
 * ws     : bllm_coding_rate_workspace(nseq, T, d) bytes.
 */
size_t bllm_coding_rate_workspace(int64_t nseq, int64_t T, int64_t d);
int bllm_coding_rate(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d, double eps2,
                     float* dR_out, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * bllm_coding_rate_split -- bllm_coding_rate with the batch split over two
 * streams of the caller: the first half of the sequences on `stream`, the
 * second on `stream2`, forked from `stream` by recording `fork_event` there
 * and joined back by recording `join_event` on `stream2` and making `stream`
 * wait for it.  Work queued on `stream` after the call sees every result; the
 * halves' launch sequences overlap, so one half's latency-bound launches run
 * beside the other half's work.  Each sequence's values are bit-identical to
 * the one-stream call's.  The streams (on the same device) and the events are
 * caller-owned (created beforehand, e.g. outside a graph capture; the call
 * records and waits on them and creates nothing).  A call on a one-sequence
 * batch runs on `stream` alone.
 * Errors : as bllm_coding_rate; BLLM_E_INVAL for a NULL stream2, fork or join
 *          event, or stream2 == stream; BLLM_E_HIP if recording or waiting fails.
 */
int bllm_coding_rate_split(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d, double eps2,
                           float* dR_out, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                           void* stream2, void* fork_event, void* join_event);

/*
 * bllm_coding_rate_stream -- the coding rate of one window of a byte stream
 * (the streaming chunker that the [BF4] weakness analysis suggests for
 * autoregressive inference: a sliding window with a local Top-K).  The
 * chunker carries the prefix matrix A = I_d + alpha sum h h^T over every byte
 * already seen; Delta R is causal, so each window's values equal the
 * whole-sequence values of bllm_coding_rate (up to fp32 rounding).
 *
 * h         : [nseq x W x d] dtype, dense (the window's rows).
 * state_in  : fp32 [nseq x d x d] row major, symmetric (entries on both
 *             sides of the diagonal are read), or NULL at the stream's start
 *             (A = I).  Device memory, caller-owned.
 * state_out : fp32 [nseq x d x d] or NULL; receives state_in + alpha H^T H
 *             over the window (full symmetric matrix).  May equal state_in
 *             (updated in place); any other overlap is an error of the caller.
 * dR_out, status, eps2, limits, errors : as bllm_coding_rate, with T = W.
 * ws        : bllm_coding_rate_workspace(nseq, W, d) bytes.
 */
int bllm_coding_rate_stream(const void* h, int dtype, int64_t nseq, int64_t W, int64_t d, double eps2,
                            const float* state_in, float* state_out, float* dR_out, int32_t* status,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * bllm_topk_select -- ByteFlow boundary set ([BF4] stage 2, [BF2] key design 2):
 *   S = {0} U {the K-1 largest score_t, t = 1..T-1}, in increasing time order.
 *   Ties go to the earlier position; NaN ranks below every number (and sets
 *   BLLM_S_NONFINITE); -0.0 equals +0.0.
 * score : fp32 [nseq x T].  idx_out : int32 [nseq x K] (positions inside the
 * sequence, idx_out[s*K] = 0).  mask_out : uint8 [nseq x T] or NULL.
 * Limits: 1 <= K <= T <= 65536 (BLLM_E_NOTSUP above).  Up to T = 16384 the
 * keys of a sequence live in LDS; longer sequences re-read their scores from
 * memory in every radix pass.
 */
int bllm_topk_select(const float* score, int64_t nseq, int64_t T, int64_t K, int32_t* idx_out,
                     uint8_t* mask_out, int32_t* status, void* stream);

/*
 * bllm_topk_select_window -- the local Top-K of one window of a stream (the
 * [BF4] weakness analysis: sliding window plus local Top-K at inference).
 * first != 0 (the stream's first window): exactly bllm_topk_select.
 * first == 0: the K largest scores of the window, no forced position.
 * Ties, NaN, layouts, limits and errors as bllm_topk_select with T = W;
 * idx_out holds positions inside the window.
 */
int bllm_topk_select_window(const float* score, int64_t nseq, int64_t W, int64_t K, int first,
                            int32_t* idx_out, uint8_t* mask_out, int32_t* status, void* stream);

/*
 * bllm_gather_topk -- the chunk inputs z = [h_{s_1}, ..., h_{s_K}] of every
 * sequence ([BF4] stage 2: the hidden states at the selected positions, in
 * time order, before the global model), straight from the Top-K positions.
 * h     : [nseq x T x d] rows of dtype (device).
 * idx   : int32 [nseq x K] positions inside each sequence (device), e.g. the
 *         idx_out of bllm_topk_select; an index outside [0, T) is clamped
 *         into it (the library never reads outside h).
 * z_out : [nseq x K x d] of dtype (device, caller-owned); row s*K + i is
 *         h[s, idx[s*K + i]].
 * The same rows as bllm_compact on the Top-K mask gives, without the mask's
 * count and prefix passes.
 * Errors : BLLM_E_INVAL for null pointers, nseq < 1, T < 1, d < 1, K < 1 or
 *          K > T; BLLM_E_NOTSUP for a bad dtype, rows not a multiple of 16
 *          bytes (or over 1 MB), unaligned h/z_out or nseq * T >= 2^31.
 */
int bllm_gather_topk(const void* h, int dtype, int64_t nseq, int64_t T, int64_t d, int64_t K,
                     const int32_t* idx, void* z_out, void* stream);

/*
 * bllm_upsample_bins -- multi-linear reconstruction with the large residual
 * ([BF4] stage 4, [BF2] key design 4):
 *   c(t)   = last i with idx[i] <= t,  L_c = idx[c+1] - idx[c] (idx[K] = T)
 *   bin(t) = floor(nbins * (t - idx[c]) / L_c)          (relative position in chunk)
 *   s_t    = h_t + g_{c(t)} W_{bin(t)}                  (row vectors)
 * g : [nseq x K x d_global], W : [nbins x d_global x d_local],
 * idx : int32 [nseq x K] (ascending, idx[s*K] = 0, as bllm_topk_select gives
 *       them), h, s_out : [nseq x T x d_local].  Other idx are clamped into
 *       [0, T); then positions no chunk covers keep their contents and
 *       overlapping chunks give unspecified rows, but no access leaves the
 *       arguments or the workspace.
 * dtype must be BLLM_BF16 (bf16 MFMA, fp32 accumulate).
 * Limits: nbins <= 64, d_global % 8 == 0, d_local % 8 == 0, nseq * T < 2^31,
 *         T <= 2^20 (else BLLM_E_NOTSUP).
 * ws : bllm_upsample_workspace(nseq, T, K, d_global, d_local, nbins) bytes
 *      (per-block counts, bin offsets and the bin-bucketed work items; W is
 *      read as stored).
 */
size_t bllm_upsample_workspace(int64_t nseq, int64_t T, int64_t K, int64_t d_global,
                               int64_t d_local, int64_t nbins);
int bllm_upsample_bins(const void* g, const void* W, const int32_t* idx, const void* h, int dtype,
                       int64_t nseq, int64_t T, int64_t K, int64_t d_global, int64_t d_local,
                       int64_t nbins, void* s_out, void* ws, size_t ws_bytes, void* stream);

/*
 * bllm_upsample_plan / bllm_upsample_apply -- bllm_upsample_bins in its two
 * parts ([BF4] stage 4).  The plan needs only the chunk starts: it buckets
 * every (chunk, bin) run of positions into the workspace (its kernels read
 * idx, nothing else), so it can run as soon as Top-K is done, beside the
 * gather and the global model; the apply is the binned GEMM with the
 * residual, from that plan.  plan followed by apply (same nseq, T, K, nbins
 * and ws; the apply queued after the plan on one stream, or ordered after it
 * by the caller's events) gives bit for bit the result of bllm_upsample_bins.
 * Arguments, layouts, limits and errors as bllm_upsample_bins (the plan's
 * ws as bllm_upsample_workspace sizes it: it does not depend on d_global or
 * d_local).  The workspace holds the plan until the next plan into it; an
 * apply from a workspace that holds no plan for these shapes gives
 * unspecified rows, but no access leaves the arguments or the workspace.
 */
int bllm_upsample_plan(const int32_t* idx, int64_t nseq, int64_t T, int64_t K, int64_t nbins, void* ws,
                       size_t ws_bytes, void* stream);
int bllm_upsample_apply(const void* g, const void* W, const void* h, int dtype, int64_t nseq, int64_t T,
                        int64_t K, int64_t d_global, int64_t d_local, int64_t nbins, void* s_out,
                        const void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BLLM_H */
