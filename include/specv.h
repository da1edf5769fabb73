/*
 * specv — batched speculative-sampling verification for AMD Instinct MI355X (gfx950).
 *
 * For each of B sequences the library takes the draft model's logits at N
 * positions and the verifier's logits at N+1 positions over one shared
 * vocabulary of V tokens (the draft and verifier must share a tokenizer: blog
 * post "LLM 추론 지연을 2배 이상 단축하는 투기적 디코딩(Speculative Decoding)과
 * 검증 샘플링 아키텍처", tech.blogsailing.com, section 3, first design decision),
 * and decides how many drafts to keep and which token to emit after them.
 *
 * The rule (lesson "추측 디코딩 — 초안 작성, 검증, 반복", factory.pai-world.com,
 * section "핵심 알고리즘(Core algorithm)", steps 4-6, and its Steps 1-3):
 *   p_i = softmax(draft_i / T), q_i = softmax(target_i / T) with the
 *   sequence's temperature T; draft token d_i is accepted, left to right, iff
 *   u_i < q_i(d_i) / p_i(d_i) (probability min(1, q/p)); a draft token with
 *   p_i(d_i) = 0 is accepted. At the first rejection j the emitted token is
 *   drawn from (q_j - p_j)_+ normalised; if all N are accepted it is drawn
 *   from q_N (the bonus token). T = 0 is greedy: d_i is accepted iff it is the
 *   first (lowest-index) argmax of target row i, and the emitted token is the
 *   first argmax of target row j.
 * Every draw uses an inverse CDF in ascending token order: the smallest k with
 *   C_k > u * S, C_k = sum_{x<=k} w_x, S = sum_x w_x (the pages call a
 *   categorical sampler without defining one; this is the library's choice).
 * All randomness is passed in as uniforms, so outputs are a deterministic
 * function of the inputs (bitwise reproducible across calls).
 *
 * Threading and streams: a handle owns scratch device memory and is not
 * thread-safe. Calls on one handle must be ordered (one stream, or explicit
 * synchronisation); use one handle per concurrent stream.
 *
 * Device pointers are plain HIP device addresses on the handle's device; the
 * caller owns every buffer passed in and the library never frees them.
 * `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 */
#ifndef SPECV_H
#define SPECV_H

#include <stdint.h>

#if defined(__GNUC__)
#define SPECV_API __attribute__((visibility("default")))
#else
#define SPECV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque handle; created by specv_create, released by specv_destroy. */
typedef struct specv_ctx* specv_handle;

/* Storage type of the logits (passed as an int-sized enum). */
typedef enum specv_dtype {
  SPECV_F32 = 0,  /* IEEE float32 */
  SPECV_BF16 = 1, /* bfloat16 (upper half of a float32) */
} specv_dtype;

/* Return codes. Host-detectable errors return before anything is enqueued. */
enum specv_status {
  SPECV_OK = 0,
  SPECV_EINVAL = -1, /* bad argument: null pointer, size out of range, bad dtype */
  SPECV_ENOMEM = -2, /* device allocation failed in specv_create */
  SPECV_EHIP = -3,   /* a HIP runtime call or kernel launch failed */
  SPECV_EALIGN = -4, /* a device pointer is not aligned as required */
  SPECV_ESTATE = -5, /* specv_row_stats before any successful specv_verify */
  SPECV_ERANGE = -6, /* specv_verify_static: a size beyond its static workspace */
};

/* Largest n_draft a handle accepts (one 64-lane wavefront holds a sequence's decisions). */
#define SPECV_MAX_DRAFT 64

/* Largest vocabulary a handle accepts (2^18 tokens). */
#define SPECV_MAX_VOCAB 262144

/*
 * Create a handle for calls with batch <= max_batch, 1 <= n_draft <= max_draft,
 * vocabulary size `vocab` (V >= 1) and logits stored as `dtype`, on HIP device
 * `device`. Allocates the scratch workspace on that device (size grows with
 * max_batch * (2*max_draft+1) * ceil(V*dtype_bytes/65536) row partials plus
 * max_batch * ceil(V/4096) draw records). On success *out is set and
 * SPECV_OK returned; on failure *out is NULL.
 * If the environment variable SPECV_DEBUG is set (and not "0") when the handle
 * is created, its calls also check on the device that every uniform lies in
 * [0, 1): a sequence with one outside gets the invalid-input sentinel (-1).
 * Errors: SPECV_EINVAL (out NULL, max_batch < 1, max_draft outside
 * [1, SPECV_MAX_DRAFT], vocab < 1 or > SPECV_MAX_VOCAB, unknown dtype, bad device),
 * SPECV_ENOMEM, SPECV_EHIP.
 */
SPECV_API int specv_create(specv_handle* out, int max_batch, int max_draft, int vocab, specv_dtype dtype,
                           int device);

/*
 * Verify one batch. All pointers are device pointers; layouts are row-major
 * and contiguous:
 *   draft_logits    [batch][n_draft][V]    dtype; 16-byte aligned
 *   target_logits   [batch][n_draft+1][V]  dtype; 16-byte aligned
 *   draft_tokens    [batch][n_draft]       int32 in [0, V)
 *   accept_uniforms [batch][n_draft]       float32 in [0, 1): u_i of decision i
 *   sample_uniforms [batch]                float32 in [0, 1): the one draw per sequence
 *   temperature     [batch]                float32; 0 = greedy, > 0 finite = sampled
 *   out_tokens      [batch][n_draft+1]     int32, written: d_0..d_{j-1}, the drawn
 *                                          token at index j, then -1
 *   out_n_accepted  [batch]                int32, written: j in [0, n_draft]
 * Logits must be finite or -inf (a masked token), with at least one finite
 * logit per row, and |logit| <= 2^64. Temperatures are 0 (greedy) or finite
 * and >= 2^-60. Work is enqueued on `stream` and the call returns without
 * waiting; outputs are valid once the stream reaches this point.
 * Per-sequence input faults that only the device can see — a draft token
 * outside [0, V), a temperature that is negative, NaN, infinite or positive
 * below 2^-60 (and, with SPECV_DEBUG, a uniform outside [0, 1)) — make that
 * sequence's out_n_accepted = -1 and all its out_tokens = -1; other sequences
 * are unaffected.
 * The workgroups of one call hand work to each other; every wait for another
 * workgroup is bounded by the handle's wait limit (specv_set_wait_limit).
 * A sequence whose wait gave up — not expected: it means the device did not
 * run a workgroup of the call within the limit — gets out_n_accepted = -2,
 * and its out_tokens are then unspecified (each is -2 or a value the call
 * was writing). Nothing is left behind that a later call could take for its
 * own (every hand-off word carries the number of the call that wrote it).
 * batch == 0 is a no-op returning SPECV_OK.
 * Errors (nothing enqueued): SPECV_EINVAL (null handle or pointer, batch < 0
 * or > max_batch, n_draft < 1 or > max_draft), SPECV_EALIGN (logits not
 * 16-byte aligned, other arrays not 4-byte aligned), SPECV_EHIP (launch failure).
 */
SPECV_API int specv_verify(specv_handle h, int batch, int n_draft,
                 const void* draft_logits, const void* target_logits,
                 const int32_t* draft_tokens, const float* accept_uniforms,
                 const float* sample_uniforms, const float* temperature,
                 int32_t* out_tokens, int32_t* out_n_accepted, void* stream);

/*
 * specv_verify with the same arguments and results, reading each sequence's
 * rows only as far as its first rejection (guide "친구가 먼저 쓰고 선생님이
 * 채점합니다", section "몇 글자를 미리 쓰게 할까요": position k is reached with
 * probability alpha^k, so most rows past an early rejection need never be
 * read). The positions go in stages [0,2), [2,8), [8,32), ... up to
 * n_draft ([0,2), [2,4), [4,8), ... when one position of the batch, its
 * draft and target rows, is 96 MB or more), one after the other in one
 * kernel launch on `stream`: a stage
 * reads the rows of the sequences still going on at its first position,
 * which its workgroups learn from the previous stage's decisions. The row
 * statistics, the accept tests and the draw are those of specv_verify, so
 * tokens and n_accepted are identical to its. Bytes read fall from 2N+1
 * rows per sequence toward the rows up to the first rejection (plus the
 * draw's re-read). A sequence whose wait gave up (-2) may keep the row
 * diagnostics of its earlier stages. Afterwards
 * specv_row_stats reports NaN / -1 for the rows not read, and
 * specv_acceptance_rates NaN for the positions not reached.
 * Errors: as specv_verify.
 */
SPECV_API int specv_verify_lazy(specv_handle h, int batch, int n_draft, const void* draft_logits,
                                const void* target_logits, const int32_t* draft_tokens,
                                const float* accept_uniforms, const float* sample_uniforms,
                                const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted,
                                void* stream);

/*
 * Draw one token from each of n_rows rows of logits (the draft model's step
 * before verification: lesson "추측 디코딩 — 초안 작성, 검증, 반복",
 * section "핵심 알고리즘(Core algorithm)" step 2, and the draft loop of its
 * "Step 3"): token r ~ softmax(logits[r] / temperature[r]) by the same inverse
 * CDF as every other draw (the smallest k with C_k > uniforms[r] * S, fp64
 * weights), or the first argmax where temperature[r] = 0.
 *   logits       [n_rows][V]  the handle's dtype; 16-byte aligned (device)
 *   temperature  [n_rows]     float32, as for specv_verify (device)
 *   uniforms     [n_rows]     float32 in [0, 1) (device)
 *   out_tokens   [n_rows]     int32, written: the drawn token, or -1 where the
 *                             temperature is invalid (-2 as for specv_verify)
 * 0 <= n_rows <= the handle's max_batch; V is the handle's vocabulary.
 * Asynchronous on `stream` like specv_verify; specv_row_stats afterwards
 * gives each row's log-normaliser and argmax ([n_rows][1]).
 * Errors (nothing enqueued): SPECV_EINVAL, SPECV_EALIGN, SPECV_EHIP.
 */
SPECV_API int specv_sample(specv_handle h, int n_rows, const void* logits, const float* temperature,
                           const float* uniforms, int32_t* out_tokens, void* stream);

/*
 * Diagnostics of the most recent specv_verify (or specv_sample, with
 * n_draft = 0) on this handle: for every
 * sequence b and row r (draft rows 0..n_draft-1, then target rows 0..n_draft),
 *   out_lse    [batch][2*n_draft+1] float32: log sum_x exp(z_x / T), the row's
 *              tempered log-normaliser (lesson, "Core algorithm" step 2-3
 *              probabilities p_i, q_i are exp(z/T - lse)); NaN for T = 0 rows,
 *              for rows a greedy sequence never reads, and for invalid sequences;
 *   out_argmax [batch][2*n_draft+1] int32: first index of the row's largest
 *              logit; -1 where the row was not read.
 * Both device pointers, 4-byte aligned. Enqueued on `stream`, which must be
 * ordered after that verify call. Errors: SPECV_EINVAL, SPECV_ESTATE (no
 * verify yet), SPECV_EHIP.
 */
SPECV_API int specv_row_stats(specv_handle h, float* out_lse, int32_t* out_argmax, void* stream);

/*
 * Acceptance telemetry of the most recent specv_verify on this handle, which
 * must have been called with this batch and n_draft and with these same
 * buffers (their contents unchanged since): for every sequence b and position
 * i < n_draft,
 *   out_alpha [batch][n_draft] float32: alpha_i = sum_x min(p_i(x), q_i(x)),
 *     the probability that draft i is accepted once position i is reached
 *     (lesson "추측 디코딩 — 초안 작성, 검증, 반복", section "속도 향상을
 *     결정하는 것"); at T = 0, 1 if d_i is the verifier's first argmax, else 0;
 *   out_tau [batch] float32: tau = sum_{k=0..n_draft} prod_{i<k} alpha_i, the
 *     expected number of tokens one verifier pass emits (with alpha held
 *     fixed, (1 - alpha^(N+1)) / (1 - alpha)).
 * NaN for sequences the verification found invalid. p and q come from the
 * fp64 row log-normalisers the verification left in the handle; one more
 * pass reads the 2*n_draft draft and target rows (about 1e-6 absolute error
 * on alpha: fp64 arguments, fp32 exps). Asynchronous on `stream`.
 * Errors (nothing enqueued): SPECV_EINVAL, SPECV_EALIGN, SPECV_ESTATE (the
 * last call on the handle had another batch or n_draft, or was specv_sample),
 * SPECV_EHIP.
 */
SPECV_API int specv_acceptance_rates(specv_handle h, int batch, int n_draft, const void* draft_logits,
                                     const void* target_logits, const int32_t* draft_tokens, const float* temperature,
                                     float* out_alpha, float* out_tau, void* stream);

/*
 * Bound of every wait between the workgroups of one call, in microseconds
 * (0 <= microseconds <= 3.6e9; default 100000). Applies to later calls on the
 * handle. A wait normally lasts microseconds. 0 makes every wait give up at
 * once, whether or not what it waits for is there, so every sequence of the
 * call reports -2 (or -1 if its inputs are invalid): a way to exercise that
 * path. Errors: SPECV_EINVAL (null handle, value out of range).
 */
SPECV_API int specv_set_wait_limit(specv_handle h, int64_t microseconds);

/*
 * Kernel timing (diagnostic). With enable != 0, every later specv_verify on
 * this handle records a HIP event on its stream before each kernel stage and
 * after the last one; specv_last_timings then waits for the most recent call's
 * final event and writes the duration of each stage in milliseconds to
 * ms[0..*count-1] (at most `capacity` entries; *count is the number of stages
 * the call launched). specv_stage_name(i) names stage i. Recording events
 * adds a few microseconds per call, so leave it off when timing whole calls.
 * Errors: SPECV_EINVAL (null handle/pointers, capacity < 1), SPECV_ESTATE (no
 * timed call yet), SPECV_EHIP.
 */
SPECV_API int specv_set_timing(specv_handle h, int enable);
SPECV_API int specv_last_timings(specv_handle h, float* ms, int capacity, int* count);
SPECV_API const char* specv_stage_name(int stage);

/*
 * specv_verify without a handle and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Arguments, layouts and results are
 * those of specv_verify, on the current HIP device; `vocab` and `dtype` are
 * passed per call.
 * Its workspace is a fixed device array inside the library (about 8 MB on
 * each GPU it runs on, held until the process ends), cleared by a kernel on
 * `stream` before the first call on each device; the first call also looks up
 * that array's device address. Limits: batch <= 256, n_draft <= 16,
 * vocab <= SPECV_MAX_VOCAB; beyond them it returns SPECV_ERANGE. Every call on
 * one GPU shares that array: calls that overlap on one GPU (on different
 * streams, or from several host threads) race and must not be issued;
 * successive calls on one stream are fine. Waits use the default bound
 * (specv_set_wait_limit has no effect here); SPECV_DEBUG is read at the first
 * call on each device.
 * Errors (nothing enqueued): SPECV_EINVAL (batch < 0, n_draft < 1, vocab < 1,
 * bad dtype, null pointer), SPECV_ERANGE, SPECV_EALIGN, SPECV_EHIP.
 */
SPECV_API int specv_verify_static(int batch, int n_draft, int vocab, specv_dtype dtype, const void* draft_logits,
                                  const void* target_logits, const int32_t* draft_tokens,
                                  const float* accept_uniforms, const float* sample_uniforms,
                                  const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted,
                                  void* stream);

/*
 * Commit the accepted drafts' KV entries after a verification (lesson
 * "추측 디코딩 — 초안 작성, 검증, 반복", section "KV 캐시 처리(KV cache dance)"
 * and exercise 4): the verifier's pass wrote one entry per draft into a
 * scratch area; for each sequence b with n = n_accepted[b] in [0, n_draft] and
 * cache_len[b] + n <= max_len, scratch entries 0..n-1 of every plane are copied
 * to cache entries cache_len[b] .. cache_len[b]+n-1 and out_cache_len[b] =
 * cache_len[b] + n; any other sequence (n_accepted -1 or -2 from an invalid or
 * failed verification, or entries that would not fit) is left as it is and
 * gets out_cache_len[b] = -1. Cache entries past the new length are not
 * touched. Needs no handle and allocates nothing.
 *   cache    device bytes: entry (p, b, t) at cache + p*cache_plane_stride
 *            + b*cache_seq_stride + t*entry_bytes, for t < max_len
 *   scratch  device bytes: entry (p, b, t) at scratch + p*scratch_plane_stride
 *            + b*scratch_seq_stride + t*entry_bytes, for t < n_draft
 *   n_accepted, cache_len, out_cache_len: device int32 [batch]
 * A plane is one contiguous [len][entry] array, e.g. the keys or the values
 * of one layer; an entry is entry_bytes bytes (heads * head_dim * element
 * size). n_planes = 0 only computes the new lengths (caches the verifier
 * wrote in place need nothing else). entry_bytes, the strides and the cache
 * and scratch bases must be multiples of 16 bytes; the two areas must not
 * overlap, and out_cache_len must not alias cache_len. Asynchronous on
 * `stream`. Errors (nothing enqueued): SPECV_EINVAL (negative sizes,
 * n_draft < 1, entry_bytes < 16, null pointers), SPECV_EALIGN, SPECV_EHIP.
 */
SPECV_API int specv_kv_commit(int n_planes, int batch, int n_draft, int max_len, int64_t entry_bytes, void* cache,
                              int64_t cache_plane_stride, int64_t cache_seq_stride, const void* scratch,
                              int64_t scratch_plane_stride, int64_t scratch_seq_stride, const int32_t* n_accepted,
                              const int32_t* cache_len, int32_t* out_cache_len, void* stream);

/* Release the handle and its workspace (synchronises the handle's device first). NULL is ignored. */
SPECV_API void specv_destroy(specv_handle h);

/* Static description of a return code. */
SPECV_API const char* specv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPECV_H */
