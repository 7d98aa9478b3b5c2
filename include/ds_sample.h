/*
 * ds_sample.h -- C ABI of the MI355X (gfx950) per-position full-vocabulary sampler.
 *
 * The library reduces packed logits [rows, positions, vocab] to one
 * (token, logprob) pair per position, and reduces plain logit rows to the greedy
 * draft triple (token, log-sum-exp, logprob).  Every step runs in HIP kernels on
 * the caller's stream; the host side only validates arguments and launches.
 *
 * Sources, cited by page title and section:
 *   [ISSUE] mstar issue "Sampler support for discrete diffusion" -- opening
 *           request, the comment on the API shape, and the comment measuring
 *           graphs at batch 1 and batch 8.
 *   [PR]    mstar PR "Add a sampler resource for discrete diffusion" -- section
 *           "What does this PR do?" (the sample(request_ids, c_logits, u_logits,
 *           seq_lens, iterations) contract).
 *   [DRAFT] LightLLM PR "perf: avoid full-vocab all-gather for draft greedy
 *           sampling" -- section "Design and invariants".
 *
 * Conventions shared by every entry point
 *   - Pointers named "device" are HIP device pointers (for example a torch
 *     tensor's data_ptr()); pointers named "host" are ordinary host memory.
 *   - The caller owns every buffer it passes.  Outputs are written, never
 *     allocated.  Inputs must stay alive and unchanged until the stream reaches
 *     the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *     Calls are asynchronous; results are valid once the stream has reached them.
 *   - Calls return a status code (DS_OK on success).  Arguments are validated
 *     before anything is enqueued, so a rejected call touches no output.  The
 *     text of the last failure on the calling thread is ds_last_error().
 *   - A sampler handle is not thread-safe and owns device scratch memory: calls
 *     on one handle must be ordered (same stream, or externally synchronised).
 */
#ifndef DS_SAMPLE_H
#define DS_SAMPLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ds_sampler ds_sampler;

/* Element type of the logit tensors. */
enum { DS_DTYPE_F32 = 0, DS_DTYPE_BF16 = 1 };

/* Status codes. */
enum {
    DS_OK = 0,
    DS_ERR_INVALID_ARG = 1, /* a pointer, size or value is outside its contract  */
    DS_ERR_UNSUPPORTED = 2, /* valid request the library does not implement      */
    DS_ERR_CAPACITY = 3,    /* sizes exceed what the handle was created for      */
    DS_ERR_NO_MEMORY = 4,   /* device or host allocation failed at create time   */
    DS_ERR_HIP = 5          /* a HIP runtime call failed; see ds_last_error()    */
};

/* Creation flags. */
enum {
    DS_FLAG_NONE = 0,
    /* Route every cell through the plain multi-pass kernels (exact threshold by
     * radix select over re-reads, Gumbel over every kept id) instead of the
     * single-pass fast paths.  Results are identical; this exists so tests can
     * compare the two paths. */
    DS_FLAG_FORCE_FALLBACK = 1,
    /* ds_sample reads u_logits in the compacted layout [C, P_u, V], holding only
     * the positions of requests whose guidance scale is not 0, in request order:
     * request r with guidance != 0 owns u positions [uoff_r, uoff_r + seq_lens[r])
     * with uoff_r = the sum of seq_lens over the earlier guided requests, and P_u
     * = the sum over all of them ([PR] "What does this PR do?": a request with
     * guidance 0 builds no unconditional document).  The streaming kernels (V
     * beyond the wave-per-cell kernel, or DS_FLAG_FORCE_FALLBACK) need V * b to
     * be a multiple of 16 bytes for this (b = 2 for bf16, 4 for f32); otherwise
     * ds_sample returns DS_ERR_UNSUPPORTED.  ds_sample_device_params does not
     * take this layout (DS_ERR_UNSUPPORTED). */
    DS_FLAG_COMPACT_U = 2
};

/*
 * ds_sample_create -- allocate a sampler for one vocabulary size and dtype.
 *
 *   out           host; receives the handle.
 *   device        HIP device ordinal the handle's scratch lives on; every later
 *                 call must pass pointers and a stream of that device.
 *   vocab         V >= 1 (ids 0 .. V-1).
 *   dtype         DS_DTYPE_F32 or DS_DTYPE_BF16.
 *   max_rows      largest `num_rows` (C) a ds_sample call may pass (>= 1).
 *   max_positions largest total positions P = sum(seq_lens) (>= 1); also bounds
 *                 ds_greedy_lse's n_rows by max_rows * max_positions.
 *   max_requests  largest `num_requests` (>= 1).
 *   top_k         ids kept by the top-ratio filter; 0 selects ceil(V / 10) =
 *                 (V + 9) / 10 ([ISSUE], comment on the API shape).  1 .. V.
 *   vocab_chunks  contiguous vocabulary chunks of ceil(V / vocab_chunks) ids each
 *                 reduced to a (max, lse, argmax) triple and merged ([DRAFT]);
 *                 1 .. min(V, 1024).  Results do not depend on it.
 *   flags         DS_FLAG_*.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_NO_MEMORY or DS_ERR_HIP.
 */
int ds_sample_create(ds_sampler **out, int device, int32_t vocab, int32_t dtype,
                     int32_t max_rows, int64_t max_positions, int32_t max_requests,
                     int32_t top_k, int32_t vocab_chunks, uint32_t flags);

/*
 * ds_sample -- one diffusion sampling step over every position handed in
 * ([PR] "What does this PR do?", [ISSUE] comment on the API shape).
 *
 * Logits are packed as [C, P, V] row-major (vocab fastest), requests
 * concatenated along positions in argument order: request r owns positions
 * [off_r, off_r + seq_lens[r]) with off_r = seq_lens[0] + ... + seq_lens[r-1].
 * For cell (row, p) of request r at offset t = p - off_r:
 *   h[v]     = c[v] when guidance_scale[r] == 0 (u is not read), otherwise
 *              fmaf(s, c[v] - u[v], c[v]) in fp32; a c of -inf stays -inf.
 *   logprob  = log-probability, over the full vocabulary, before temperature and
 *              filtering, of the guided distribution lc + s*(lc - lu) on
 *              log-softmaxed c and u, renormalised; equal to h[token] - LSE(h).
 *   temperature[r] == 0: token = smallest id with the largest h.
 *   temperature[r]  > 0: keep the ids whose h is >= the top_k-th largest h (ties
 *              kept); token = argmax over kept ids of h/tau + G, smallest id on
 *              exact ties, with Gumbel noise G = -log(-log U) from Philox4x32-10:
 *              key (seed low, seed high), counter (v >> 2, t,
 *              (row & 0xFFFF) | (iterations[r] << 16), (uint32)request_ids[r]),
 *              word v & 3, U = ((word >> 9) * 2 + 1) * 2^-24.
 *
 *   request_ids    host [R]; the low 32 bits key the noise.
 *   c_logits       device [C, P, V] of the handle's dtype; 4-byte aligned (f32)
 *                  or 2-byte aligned (bf16).  Values finite or -inf.
 *   u_logits       device, same layout; may be NULL iff every guidance scale is
 *                  0.  Rows of requests with guidance 0 are never read (they may
 *                  hold anything).  Elsewhere finite, or -inf where c is -inf.
 *   seq_lens       host [R], each >= 0; P = sum <= max_positions.
 *   iterations     host [R]; diffusion step index, keys the noise (16 bits used).
 *   guidance_scale host [R]; finite.
 *   temperature    host [R]; >= 0 and finite; 0 means greedy.
 *   num_requests   R, 1 .. max_requests.
 *   num_rows       C, 1 .. max_rows.
 *   seed           64-bit noise key.
 *   tokens_out     device int32 [C, P].
 *   logprobs_out   device float [C, P].
 *   threshold_out  device float [C, P] or NULL; the top_k-th largest h of each
 *                  sampled cell, NaN for greedy cells.
 *   stream         hipStream_t.
 */
int ds_sample(ds_sampler *s, const int64_t *request_ids, const void *c_logits,
              const void *u_logits, const int32_t *seq_lens, const int32_t *iterations,
              const float *guidance_scale, const float *temperature, int32_t num_requests,
              int32_t num_rows, uint64_t seed, int32_t *tokens_out, float *logprobs_out,
              float *threshold_out, void *stream);

/*
 * ds_sample_device_params -- ds_sample with a fixed launch shape and the
 * per-request parameters in device memory, for a call captured once in a HIP
 * graph and replayed while the batch changes: the GPU reads the parameters when
 * the call runs, so updating the arrays between replays (a new iteration, other
 * lengths, guidance or temperature) changes what the next replay computes.  The
 * pages capture their sampler in graphs and pad the batch to the captured shape
 * ([DRAFT] "Design and invariants": graph pad/unpad keeps the per-row results),
 * and graphs pay off where launch overhead dominates, at batch 1 ([ISSUE],
 * comment measuring graphs at batch 1 and batch 8).
 *
 * Same computation and outputs as ds_sample, cell for cell, for valid values.
 * The packed layout is [C, positions, V] with `positions` fixed at capture:
 * request r owns positions [off_r, off_r + seq_lens[r]) as in ds_sample, the
 * positions from sum(seq_lens) to `positions` are padding, and their outputs are
 * not written.
 *
 *   request_ids, seq_lens, iterations, guidance_scale, temperature
 *                  device arrays [num_requests], aligned to their element size,
 *                  read on the GPU when the call runs.  A negative length counts
 *                  as 0; lengths past `positions` are cut there.  A guidance scale
 *                  that is not finite, or any scale when u_logits is NULL, counts
 *                  as 0.  A temperature that is not a positive finite number
 *                  samples greedily.  (ds_sample rejects such values instead.)
 *   c_logits       device [C, positions, V]; alignment as in ds_sample.
 *   u_logits       device, same layout, or NULL (then every request is unguided).
 *   num_requests   1 .. min(64, max_requests); pad with zero-length requests.
 *   num_rows       C, 1 .. max_rows.
 *   positions      1 .. min(max_positions, 2^24): the row stride of the layout and
 *                  the extent of the launch.
 *   seed, tokens_out [C, positions], logprobs_out [C, positions],
 *   threshold_out [C, positions] or NULL, stream: as in ds_sample.
 * Every vocabulary size is supported, through the same kernels as ds_sample
 * (the streaming kernels run over every cell of the fixed layout, and padding
 * cells leave at once); DS_FLAG_FORCE_FALLBACK applies as it does to ds_sample.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY, DS_ERR_UNSUPPORTED or
 * DS_ERR_HIP; the host-side checks run before anything is enqueued.
 */
int ds_sample_device_params(ds_sampler *s, const int64_t *request_ids, const void *c_logits,
                            const void *u_logits, const int32_t *seq_lens, const int32_t *iterations,
                            const float *guidance_scale, const float *temperature,
                            int32_t num_requests, int32_t num_rows, int64_t positions, uint64_t seed,
                            int32_t *tokens_out, float *logprobs_out, float *threshold_out,
                            void *stream);

/*
 * ds_greedy_lse -- draft greedy reduction of plain logit rows ([DRAFT]).
 *
 *   logits       device [n_rows, V] of the handle's dtype (alignment as above),
 *                values finite or -inf, no row entirely -inf.
 *   n_rows       0 .. max_rows * max_positions (0 is a no-op).
 *   token_out    device int32 [n_rows]: smallest id attaining the row maximum.
 *   lse_out      device float [n_rows]: log-sum-exp over the full row.
 *   logprob_out  device float [n_rows]: logits[token] - lse, the log of the
 *                exact selected-token probability.
 *   triples_out  device float [vocab_chunks][n_rows][3] or NULL: per chunk
 *                (max, lse, id) with the int32 id stored bit-for-bit in the third
 *                float word (reinterpret, never convert); an empty chunk is
 *                (-inf, -inf, INT32_MAX).
 *   stream       hipStream_t.
 * Launch shape (results do not depend on it): when the rows fill every compute
 * unit in whole rounds, V and ceil(V / vocab_chunks) are multiples of the ids
 * in 16 bytes and logits is 16-byte aligned, one workgroup reduces each row in a
 * single kernel; otherwise parts of rows are reduced into the handle's
 * workspace and merged by a second kernel.
 */
int ds_greedy_lse(ds_sampler *s, const void *logits, int64_t n_rows, int32_t *token_out,
                  float *lse_out, float *logprob_out, float *triples_out, void *stream);

/*
 * ds_reveal_topk -- the confidence reveal that follows a sampling step
 * ([ISSUE], comment on the API shape: the step scores every position, ranks
 * them by confidence and commits the best, a top-k over the request's [C, T]
 * scores flattened row-major).  For every request r, returns its reveal_counts[r]
 * best cells, best first; equal scores keep the smaller flattened index first
 * (the smallest-id rule of [DRAFT] "Design and invariants").
 *
 *   scores         device float [C, P], requests packed along positions as in
 *                  ds_sample (for example ds_sample's logprobs_out, or the
 *                  caller's confidence with committed positions set to -inf);
 *                  4-byte aligned; values finite or -inf (NaN unsupported).
 *   num_rows       C, 1 .. max_rows.
 *   seq_lens       host [R], each >= 0; P = sum <= max_positions.
 *   reveal_counts  host [R]; 0 <= reveal_counts[r] <= C * seq_lens[r], and at
 *                  most 16384 per request (DS_ERR_UNSUPPORTED above).
 *   num_requests   R, 1 .. max_requests.
 *   index_out      device int32 [sum(reveal_counts)]: request by request in
 *                  argument order, the flattened index c * seq_lens[r] + t of each
 *                  revealed cell (row c, position t of the request).
 *   score_out      device float [sum(reveal_counts)] or NULL: their scores.
 *   stream         hipStream_t.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY, DS_ERR_UNSUPPORTED or
 * DS_ERR_HIP.  Nothing is written when every reveal count is 0.
 */
int ds_reveal_topk(ds_sampler *s, const float *scores, int32_t num_rows, const int32_t *seq_lens,
                   const int32_t *reveal_counts, int32_t num_requests, int32_t *index_out,
                   float *score_out, void *stream);

/*
 * ds_repetition_penalty -- the repetition penalty of the autoregressive mode
 * ([ISSUE]: the existing sampler draws one token per request and applies a
 * repetition penalty over seen-token masks; the pages give no formula).  Reading:
 * every seen id's logit x becomes x / theta when x > 0 and x * theta otherwise,
 * computed in binary32 and written back in place in the handle's dtype (bf16
 * rounded to nearest even).  An autoregressive step is this call followed by
 * sampling the same rows as one position per request (guidance 0, no u),
 * with the top-ratio filter given by the handle's top_k (V keeps every id);
 * ds_sample_ar runs both in one call.
 *
 *   logits       device [n_rows, V] of the handle's dtype, modified in place at
 *                the seen ids only; values finite or -inf (NaN unsupported).
 *   n_rows       0 .. max_rows * max_positions (0 is a no-op).
 *   seen_mask    device uint32 [n_rows, ceil(V / 32)], 4-byte aligned: id v of
 *                row i is seen when bit (v & 31) of word i * ceil(V / 32) + (v >> 5)
 *                is set; bits past V are ignored.
 *   penalty      device float [n_rows], 4-byte aligned: theta of each row; a row
 *                whose theta is not finite and > 0 is left unchanged (theta = 1
 *                changes nothing either).
 *   stream       hipStream_t.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY or DS_ERR_HIP.  Rows whose
 * mask words overlap in memory with another row's logits race.
 */
int ds_repetition_penalty(ds_sampler *s, void *logits, int64_t n_rows, const uint32_t *seen_mask,
                          const float *penalty, void *stream);

/*
 * ds_sample_ar -- one autoregressive step: one token per request ([ISSUE]: the
 * existing sampler draws one token per request and applies a repetition penalty
 * over seen-token masks).  The repetition penalty (as ds_repetition_penalty, in
 * place) and then every row sampled as the only position of its request.  On
 * the streaming path (V above the wave-per-cell kernel's limit, or the forced
 * fallback) each part of a row penalises its own ids just before it reads them,
 * so the row is read once; otherwise the penalty kernel runs first.  Either
 * way the penalised logits and the results are the same.  Each row is sampled
 * with guidance 0, the request's temperature (0 = greedy), the handle's top_k,
 * Gumbel noise keyed by (seed, request id, iteration, row 0, position 0, id)
 * exactly as ds_sample keys a request with one position, and the
 * full-vocabulary log-probability of the penalised row.
 *
 *   request_ids   device int64 [R], 8-byte aligned.
 *   logits        device [R, V] of the handle's dtype; penalised in place.
 *   seen_mask     device uint32 [R, ceil(V / 32)] as in ds_repetition_penalty,
 *                 or NULL together with penalty for no penalty.
 *   penalty       device float [R] as in ds_repetition_penalty, or NULL.
 *   iterations    device int32 [R]; keys the noise.
 *   temperature   device float [R]; a value that is not finite and > 0 samples
 *                 greedily.
 *   num_requests  R, 1 .. min(max_requests, max_positions).
 *   seed          keys the noise.
 *   tokens_out    device int32 [R]; logprobs_out device float [R].
 *   stream        hipStream_t.
 * Returns DS_OK, DS_ERR_INVALID_ARG, DS_ERR_CAPACITY or DS_ERR_HIP.  The
 * parameters are read when the call runs, so a captured call follows updates to
 * the device arrays between replays.
 */
int ds_sample_ar(ds_sampler *s, const int64_t *request_ids, void *logits, const uint32_t *seen_mask,
                 const float *penalty, const int32_t *iterations, const float *temperature,
                 int32_t num_requests, uint64_t seed, int32_t *tokens_out, float *logprobs_out,
                 void *stream);

/*
 * ds_sample_static -- ds_sample without a handle, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, and harnesses that forbid hipMalloc.  It allocates nothing: the
 * streaming kernels' per-(row, part) records live in a fixed 512 KB array of the
 * library's own device memory (one copy per device, present from load to process
 * exit), and the handle's settings come as arguments.
 *
 * Same computation, checks and outputs as ds_sample on a handle created with the
 * same vocab, dtype, top_k, vocab_chunks and flags (see ds_sample_create), cell
 * for cell, on the calling thread's current HIP device.  The handle's capacity
 * limits are replaced by one: num_rows * sum(seq_lens) must stay below 2^31.
 * Every vocabulary size runs: rows that need more records than the array holds
 * are processed in several launches on `stream`, as ds_sample does with its
 * workspace.
 *
 * The array is shared by every call on a device and keeps the last call's
 * records: calls that may run at the same time on one device (different streams
 * without ordering between them) race and give wrong results; order them on one
 * stream.  The first call on each device looks up the array's address there
 * (hipGetSymbolAddress, no allocation).  Returns what ds_sample returns, and
 * DS_ERR_UNSUPPORTED on a device ordinal of 64 or more.
 */
int ds_sample_static(int32_t vocab, int32_t dtype, int32_t top_k, int32_t vocab_chunks, uint32_t flags,
                     const int64_t *request_ids, const void *c_logits, const void *u_logits,
                     const int32_t *seq_lens, const int32_t *iterations, const float *guidance_scale,
                     const float *temperature, int32_t num_requests, int32_t num_rows, uint64_t seed,
                     int32_t *tokens_out, float *logprobs_out, float *threshold_out, void *stream);

/*
 * ds_read_probe -- measurement aid, not part of the sampling path: the HBM read
 * ceiling at a launch shape.  n_rows workgroups of `threads` threads each read
 * one row of row_bytes once, with the 16-byte nontemporal loads of the streaming
 * sampler kernels, and write the xor of the row's words to sink[row] (so that no
 * load can be dropped).  Timing this call next to a sampler call of the same
 * bytes and shape shows how close the sampler comes to what the memory system
 * delivers on the running device.  No handle is needed.
 *
 *   x          device, 16-byte aligned, n_rows * row_bytes bytes.
 *   n_rows     1 .. 2^31 - 1 (one workgroup each).
 *   row_bytes  a positive multiple of 16.
 *   threads    256, 512 or 1024 threads per workgroup.
 *   sink       device uint32 [n_rows], 4-byte aligned.
 *   stream     hipStream_t.
 * Returns DS_OK, DS_ERR_INVALID_ARG or DS_ERR_HIP.
 */
int ds_read_probe(const void *x, int64_t n_rows, int64_t row_bytes, int32_t threads, uint32_t *sink,
                  void *stream);

/* Release a handle and its device scratch.  NULL is a no-op.  The caller must
 * make sure no call on the handle is still pending on a stream. */
void ds_sample_destroy(ds_sampler *s);

/* Text of the last failure on the calling thread ("" if none).  The pointer
 * stays valid until the next call on the same thread. */
const char *ds_last_error(void);

/* Library version, as MAJOR * 10000 + MINOR * 100 + PATCH. */
int ds_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS_SAMPLE_H */
