/*
 * specverify.h - C ABI of the MI355X (gfx950) speculative-sampling
 * verification library (libspecverify.so).
 *
 * The operation: given the target model's logits over K+1 positions and the
 * draft model's logits over K positions, each drafted token x_i is accepted
 * with probability min(1, p_i(x_i) / q_i(x_i)); verification stops at the
 * first rejection and replaces that token with a draw from
 * norm(max(0, p_i - q_i)); if all K drafts are accepted one more token is
 * drawn from p_K.  Sources: page www.cf-1.com/news/5155685 section 2.2 and
 * page www.2kiu.com/news/5895634 section 2.2 (the accept/reject rule and its
 * lossless output law), page www.gsyq.cn/news/428210 section 3.1 (one target
 * forward scores every drafted position; positions are judged in order and
 * the first wrong one is replaced), page www.gsyq.cn/news/428210 section 3.2
 * and page www.2kiu.com/news/5895634 section 3.1 (1 + a + ... + a^K tokens per
 * target forward: the last term is the all-accepted draw), and page
 * www.gsyq.cn/news/428210 section 3.3 (temperature, top-k and top-p applied
 * identically to the target and the draft).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *_logits, draft_tokens, uniforms and out_* are DEVICE
 *   pointers on the current HIP device, owned by the caller; the library never
 *   frees or retains them.  Logit tensors are row-major with the vocabulary
 *   contiguous.  Any alignment is accepted; 16-byte aligned bases with
 *   V * sizeof(dtype) a multiple of 16 take the vectorised path.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and returns without synchronising.
 * - Scratch: the library keeps device scratch per (device, stream): calls on
 *   different streams never share it, so they may run concurrently, from any
 *   host threads.  A stream's scratch is allocated on its first call and grown
 *   when a call needs more; a growth synchronises that stream only (the one
 *   stream whose queued work can still use the old buffer) before freeing
 *   it.  sv_init() sizes a stream's scratch up front, after which calls
 *   within its bounds never allocate or synchronise.  Calls on one stream
 *   from several host threads are serialised by the library (each holds the
 *   stream's scratch from its look-up to its last launch).  No call depends
 *   on what an earlier call left in the scratch.  sv_stream_release() and
 *   sv_release() free it.
 * - Temperature T: 0 selects greedy decoding (p and q one-hot at their
 *   arg-max, ties to the lowest index); otherwise T must be a finite normal
 *   float >= FLT_MIN.  top_k: 0 or >= V disables it.  top_p in (0, 1]; 1
 *   disables it.  top-k is applied before top-p, both after temperature; both
 *   keep every token tied with their last kept token.
 * - Logits may be -inf (token masked out).  NaN and +inf logits are outside
 *   the defined input range.  uniforms must lie in [0, 1).
 * - Return value: SV_OK or a negative sv_status.  Argument errors are
 *   detected on the host before anything is enqueued; SV_ERR_HIP reports a
 *   failed HIP runtime call (allocation or launch).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = -1,      /* a required pointer is NULL                          */
  SV_ERR_SHAPE = -2,     /* B < 0, K < 0, K > SV_MAX_K, V < 1, V > SV_MAX_V, or a
                            launch grid that would exceed 2^32 threads           */
  SV_ERR_DTYPE = -3,     /* dtype is not one of sv_dtype                          */
  SV_ERR_PARAM = -4,     /* temperature, top_k or top_p out of range              */
  SV_ERR_HIP = -5,       /* a HIP runtime call failed                             */
  SV_ERR_WORKSPACE = -6  /* scratch could not be provided                         */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

#define SV_MAX_K 64
#define SV_MAX_V 2097152 /* 256 chunks of 8192 logits per row */
/* Size of the device array that sv_spec_verify_noalloc works in (one per
 * device the library runs on, held until the process ends).  It holds every
 * call with B <= 64, K <= 6 and V <= 128256, in any mode and dtype; a call
 * whose scratch would not fit returns SV_ERR_WORKSPACE. */
#define SV_NOALLOC_SCRATCH_BYTES (32 << 20)
/* sv_init flag: also size the stream's buffer of projection logits for
 * sv_spec_verify_lmhead. */
#define SV_INIT_LMHEAD 1

/*
 * sv_spec_verify - verify one round of K drafted tokens for B sequences.
 *
 * target_logits    [B, K+1, V] dtype   target logits for positions 0..K
 * draft_logits     [B, K,   V] dtype   draft logits for positions 0..K-1
 *                                      (not read when temperature == 0)
 * draft_tokens     [B, K] int32        drafted tokens x_i, drawn from q_i
 * uniforms         [B, K+1] float32    U[0,1): column i < K drives the accept
 *                                      test at draft i (accept iff
 *                                      u_i * q_i(x_i) < p_i(x_i)); column K is
 *                                      the one uniform of the inverse-CDF draw
 *                                      (residual or bonus), taken in ascending
 *                                      vocabulary order: token = min{j :
 *                                      u*Z < C_j}
 * out_tokens       [B, K+1] int32      written: x_0..x_{n-1}, then the drawn
 *                                      token at index n, then -1 padding
 * out_num_accepted [B] int32           written: n in [0, K], the number of
 *                                      accepted drafts (n + 1 tokens are
 *                                      emitted).  A sequence with a row whose
 *                                      logits are all -inf, or a drafted token
 *                                      outside [0, V), gets n = -1 and tokens
 *                                      all -1.
 * B, K, V, dtype   shapes and logit type (sv_dtype)
 * stream           hipStream_t
 *
 * B == 0 returns SV_OK without touching any pointer.
 */
int sv_spec_verify(const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const float* uniforms,
                   float temperature, int32_t top_k, float top_p,
                   int32_t* out_tokens, int32_t* out_num_accepted,
                   int32_t B, int32_t K, int32_t V, int32_t dtype,
                   void* stream);

/*
 * sv_spec_verify_noalloc - sv_spec_verify for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, results and errors as
 * sv_spec_verify, but the call never allocates or frees memory and never
 * synchronises: its scratch is one file-scope device array per device of
 * SV_NOALLOC_SCRATCH_BYTES bytes, loaded with the library's code.  A call
 * whose scratch would exceed it returns SV_ERR_WORKSPACE before anything is
 * enqueued.  Every call on a device works in that device's one array: calls
 * that may overlap on one device (different streams, or different host
 * threads without ordering) race on it and must be serialised by the
 * caller.  No call depends on what an earlier call left in the array (the
 * call's first kernel clears what must start at zero).  Not timed by
 * sv_profile_start.  sv_init() resolves the array's address on a device
 * (otherwise the first call on the device does).
 */
int sv_spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms,
                           float temperature, int32_t top_k, float top_p,
                           int32_t* out_tokens, int32_t* out_num_accepted,
                           int32_t B, int32_t K, int32_t V, int32_t dtype,
                           void* stream);

/*
 * sv_spec_verify_debug - sv_spec_verify plus the intermediate values the
 * decisions were taken on (for tests and diagnostics).
 *
 * out_p   [B, K] double   p_i(x_i): the filtered target probability of each
 *                         drafted token (NaN for a sentinel sequence)
 * out_q   [B, K] double   q_i(x_i): the same for the draft
 * out_z   [B]    double   Z: total weight of the row the last token was drawn
 *                         from (residual or bonus), as used by the draw
 * Any of out_p, out_q, out_z may be NULL.  Same return values as
 * sv_spec_verify.
 */
int sv_spec_verify_debug(const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const float* uniforms,
                         float temperature, int32_t top_k, float top_p,
                         int32_t* out_tokens, int32_t* out_num_accepted,
                         double* out_p, double* out_q, double* out_z,
                         int32_t B, int32_t K, int32_t V, int32_t dtype,
                         void* stream);

/*
 * sv_spec_verify_dt - sv_spec_verify (with the outputs of
 * sv_spec_verify_debug) for drafts that were sampled at their own
 * temperature draft_temperature (page www.2kiu.com/news/5895634 section 7:
 * a lower draft temperature such as 0.5 makes the drafts more certain).  The
 * draft rows' q is then the filtered distribution at draft_temperature, with
 * the shared top_k and top_p: each draft is tested against the q it was drawn
 * from, so the output still follows p.  In greedy mode (temperature == 0)
 * draft_temperature is not used; otherwise it must be a valid temperature
 * above 0 (SV_ERR_PARAM).  With draft_temperature == temperature the results
 * equal sv_spec_verify's.
 */
int sv_spec_verify_dt(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms,
                      float temperature, float draft_temperature,
                      int32_t top_k, float top_p,
                      int32_t* out_tokens, int32_t* out_num_accepted,
                      double* out_p, double* out_q, double* out_z,
                      int32_t B, int32_t K, int32_t V, int32_t dtype,
                      void* stream);

/*
 * sv_spec_verify_ragged - verification of a batch whose sequences carry
 * different numbers of drafts, as when the draft length is tuned per
 * sequence from its acceptance history (page www.cf-1.com/news/5155685
 * section 2.4, page www.2kiu.com/news/5895634 section 4.4; see
 * sv_dynk_observe).  Each sequence follows the rule of sv_spec_verify with its
 * own K_b = cu_num_draft[b+1] - cu_num_draft[b] drafts (0 allowed: the
 * sequence only draws its bonus token from its one target row).
 *
 * Packed layout (device pointers), with N = total_draft = cu_num_draft[B]:
 * target_logits  [N + B, V] dtype   sequence b's K_b + 1 rows from row
 *                                   cu_num_draft[b] + b
 * draft_logits   [N, V] dtype       its K_b rows from row cu_num_draft[b]
 *                                   (not read when temperature == 0)
 * draft_tokens   [N] int32          its drafts from cu_num_draft[b]
 * uniforms       [N + B] float32    its K_b accept uniforms, then its one
 *                                   sampling uniform, from cu_num_draft[b] + b
 * cu_num_draft   [B + 1] int32      device offsets: cu[0] = 0, nondecreasing,
 *                                   every K_b <= max_k, cu[B] = total_draft
 * out_tokens     [B, max_k + 1] int32   as for sv_spec_verify; every entry
 *                                   after the drawn token is -1
 * out_num_accepted [B] int32        n in [0, K_b], or -1 for a sentinel
 * out_p, out_q   [N] double or NULL p_i(x_i), q_i(x_i) at each draft's packed
 *                                   index (as sv_spec_verify_debug)
 * out_z          [B] double or NULL as sv_spec_verify_debug
 * draft_temperature                 as sv_spec_verify_dt (pass temperature
 *                                   for drafts sampled at the target's)
 * B, total_draft, max_k, V, dtype   host values; max_k <= SV_MAX_K and
 *                                   total_draft <= B * max_k (else
 *                                   SV_ERR_SHAPE)
 *
 * The offsets are only read on the device.  When they describe no packing
 * of the rows (cu[0] != 0, a K_b < 0 or > max_k, or cu[B] != total_draft),
 * every sequence is written as a sentinel (n = -1, tokens -1; out_p and
 * out_q are left untouched) and the call still returns SV_OK.  With every
 * K_b equal to K the results equal sv_spec_verify_dt's on the same rows.
 */
int sv_spec_verify_ragged(const void* target_logits, const void* draft_logits,
                          const int32_t* draft_tokens, const float* uniforms,
                          const int32_t* cu_num_draft,
                          float temperature, float draft_temperature,
                          int32_t top_k, float top_p,
                          int32_t* out_tokens, int32_t* out_num_accepted,
                          double* out_p, double* out_q, double* out_z,
                          int32_t B, int32_t total_draft, int32_t max_k,
                          int32_t V, int32_t dtype, void* stream);

/*
 * sv_spec_verify_probs - sv_spec_verify (with the outputs of
 * sv_spec_verify_debug) where each draft distribution q_i is supplied as
 * probabilities instead of logits: the distribution the draft actually drew
 * x_i from, whatever sampling pipeline produced it (page www.2kiu.com/news/
 * 5895634 section 7: the drafts are verified against the q they were drawn
 * from, which keeps the output law p).  The target rows are filtered by
 * temperature, top_k and top_p as usual; q_i is used exactly as given.
 *
 * draft_probs  [B, K, V] float32, device   q_i(j) >= 0, each row summing to 1
 *                                          (not checked; entries above 1,
 *                                          negative or non-finite values are
 *                                          outside the defined range)
 * Other arguments as sv_spec_verify_debug (out_q returns the given q_i(x_i)).
 *
 * Only the target rows are streamed: q enters through q_i(x_i) and, after a
 * rejection at position n, through q_n at the tokens the residual
 * max(0, p_n - q_n) can be positive on (the target's kept set; every token
 * of an unfiltered row).  draft_probs may be NULL when temperature == 0
 * (greedy verification does not use q) or K == 0.
 */
int sv_spec_verify_probs(const void* target_logits, const float* draft_probs,
                         const int32_t* draft_tokens, const float* uniforms,
                         float temperature, int32_t top_k, float top_p,
                         int32_t* out_tokens, int32_t* out_num_accepted,
                         double* out_p, double* out_q, double* out_z,
                         int32_t B, int32_t K, int32_t V, int32_t dtype,
                         void* stream);

/*
 * Draft-length controller (host only; no device work).  The rule of page
 * www.2kiu.com/news/5895634 section 4.4 (the policy of page
 * www.cf-1.com/news/5155685 section 2.4): keep the acceptance statistics of
 * the last `window` batches (100 on the page); once the window is full, a
 * window acceptance rate above raise_above (0.8) lengthens the draft by one
 * and one below lower_below (0.6) shortens it by one, within [k_min, k_max]
 * ([2, 10]).  The window rate is its accepted drafts over its drafted tokens
 * (exact integer totals, one division).  The window starts empty after every
 * change of K, so each decision rests on batches drafted at the current K.
 * A batch that drafted nothing is not observed.
 *
 * One handle holds `lanes` independent controllers: 1 for a batch-wide draft
 * length (observe the batch's totals), B for one draft length per sequence
 * (observe each sequence's n and K_b; feed the result to
 * sv_spec_verify_ragged).  Handles are not thread-safe; distinct handles
 * are independent.
 *
 * sv_dynk_create   returns a handle, or NULL if lanes < 1, window < 1,
 *                  not 0 <= k_min <= k_init <= k_max, not 0 <= lower_below
 *                  <= raise_above <= 1, or memory is short.
 * sv_dynk_observe  accepted[l], drafted[l]: host arrays [lanes] for one
 *                  batch; k_next[l] (host [lanes], may be NULL) receives the
 *                  draft length to use next.  SV_ERR_NULL for a NULL handle or
 *                  input; SV_ERR_PARAM (nothing recorded) unless
 *                  0 <= accepted[l] <= drafted[l] for every lane.
 * sv_dynk_k        current draft length of a lane (-1 for a bad handle/lane).
 * sv_dynk_destroy  frees the handle (NULL allowed).
 */
typedef struct sv_dynk sv_dynk;
sv_dynk* sv_dynk_create(int32_t lanes, int32_t window, double raise_above, double lower_below,
                        int32_t k_min, int32_t k_max, int32_t k_init);
int sv_dynk_observe(sv_dynk* ctrl, const int64_t* accepted, const int64_t* drafted, int32_t* k_next);
int32_t sv_dynk_k(const sv_dynk* ctrl, int32_t lane);
void sv_dynk_destroy(sv_dynk* ctrl);

/*
 * sv_filtered_probs - the filtered distribution of every row: temperature,
 * then top-k, then top-p, then the softmax over the kept tokens (page
 * www.gsyq.cn/news/428210 section 3.3 for the parameters; the distribution
 * is the p or q of the accept test).
 *
 * logits     [rows, V] dtype   device
 * out_probs  [rows, V] float   device; written with the probabilities
 *                              (0 for tokens outside the kept set).  A row
 *                              with every logit -inf is written as all NaN.
 * temperature must be > 0 here (greedy rows are one-hot by definition).
 */
int sv_filtered_probs(const void* logits, int32_t rows, int32_t V, int32_t dtype,
                      float temperature, int32_t top_k, float top_p,
                      float* out_probs, void* stream);

/*
 * sv_sample - draw one token per row from the row's filtered distribution:
 * the drafting step that comes before verification (x ~ q, and q(x) for the
 * accept test).  Page www.gsyq.cn/news/428210 section 3.1 (the small model
 * samples the drafted tokens) and section 3.3 (the same sampling parameters
 * as the target).  The draw is the one sv_spec_verify makes for its last
 * token: inverse CDF in ascending vocabulary order, token = min{j : u*Z < C_j}
 * over the filtered probabilities (in greedy mode the arg-max, lowest index on
 * ties).
 *
 * logits      [rows, V] dtype   device
 * uniforms    [rows] float32    device; U[0, 1), one per row
 * out_tokens  [rows] int32      device; written with the drawn token, or -1
 *                               for a row whose logits are all -inf
 * out_prob    [rows] double     device, may be NULL; written with the
 *                               filtered probability of the drawn token (1 in
 *                               greedy mode; NaN for an all -inf row)
 * temperature, top_k, top_p as for sv_spec_verify.  Errors as for
 * sv_spec_verify with B = rows and K = 0 (rows < 0, V < 1 or V > SV_MAX_V:
 * SV_ERR_SHAPE); rows == 0 returns SV_OK without touching any pointer.
 */
int sv_sample(const void* logits, const float* uniforms, float temperature,
              int32_t top_k, float top_p, int32_t* out_tokens, double* out_prob,
              int32_t rows, int32_t V, int32_t dtype, void* stream);

/*
 * sv_lm_logits - the output projection of a language model: logits[m, j] =
 * sum_i hidden[m, i] * weight[j, i], every position's hidden state mapped to
 * one logit per vocabulary entry (the step whose weight reads dominate a
 * decoding step: page www.2kiu.com/news/5895634 section 1, page
 * www.cf-1.com/news/5155685 section 2.1).  Products of two bfloat16 values
 * are exact in float32; the sums are accumulated in float32 by the matrix
 * cores (v_mfma_f32_32x32x16_bf16), in an order the library fixes.
 *
 * hidden      [M, d] bfloat16, device, 16-byte aligned
 * weight      [V, d] bfloat16, device, 16-byte aligned (d contiguous in both)
 * out_logits  [M, V] float32, device (any alignment), written entirely
 * M >= 0, 1 <= V <= SV_MAX_V, d a multiple of 64 in [64, 65536] (else
 * SV_ERR_SHAPE; misaligned operands are SV_ERR_SHAPE too).  M == 0 does
 * nothing.  The library allocates nothing for this call.
 */
int sv_lm_logits(const void* hidden, const void* weight, float* out_logits,
                 int32_t M, int32_t V, int32_t d, void* stream);

/*
 * sv_spec_verify_lmhead - verification fed directly by the two models'
 * output projections: the target's logits for all K+1 positions come from
 * its hidden states and its projection in one pass (page www.gsyq.cn/news/
 * 428210 section 3.1), the draft's K rows from its own (a smaller model of
 * the same family: its width d_draft may differ, the vocabulary is shared;
 * page www.2kiu.com/news/5895634 section 4.1), and the verification of
 * sv_spec_verify_debug runs on them.  Decides as sv_lm_logits on both
 * followed by sv_spec_verify_debug with dtype SV_F32 (the same logits; the
 * normalisers may differ in float rounding, well within the verification's
 * 1e-6 bound on p(x) and q(x)).
 *
 * When V % 4 == 0 the verification does not stream the logits again: the
 * projections' epilogues reduce each row's 64-column tiles to a record (the
 * tile max and its exp2 sum, or its arg-max at temperature 0), the chunk
 * statistics are formed from those records, and only the tiles that can
 * hold a filter candidate are read back.  The logits are still written once
 * (the kept lists and the full-row draws read them).  Other V stream them.
 *
 * hidden_target  [B, K+1, d_target] bfloat16, device, 16-byte aligned
 * weight_target  [V, d_target] bfloat16, device, 16-byte aligned
 * hidden_draft   [B, K, d_draft] bfloat16, device, 16-byte aligned
 * weight_draft   [V, d_draft] bfloat16, device, 16-byte aligned
 *                (both draft arguments unused, and may be NULL, when
 *                temperature == 0 or K == 0)
 * draft_tokens, uniforms, temperature, top_k, top_p, out_tokens,
 * out_num_accepted, out_p, out_q, out_z, B, K, V: as sv_spec_verify_debug.
 * d_target, d_draft: as d of sv_lm_logits.
 *
 * The logits live in a second buffer of the stream's scratch set, of
 * (B(K+1) + BK) * V float32 and 8 bytes per row and 64 columns of tile
 * records, grown on demand like the scratch (a growth
 * synchronises the stream) or sized by sv_init with SV_INIT_LMHEAD, and freed
 * by sv_stream_release and sv_release.  Under launch timing the first two
 * events of the call bracket the two projections (its stream_kernel_ms) and
 * the third follows the verification.
 */
int sv_spec_verify_lmhead(const void* hidden_target, const void* weight_target,
                          const void* hidden_draft, const void* weight_draft,
                          const int32_t* draft_tokens, const float* uniforms,
                          float temperature, int32_t top_k, float top_p,
                          int32_t* out_tokens, int32_t* out_num_accepted,
                          double* out_p, double* out_q, double* out_z,
                          int32_t B, int32_t K, int32_t V,
                          int32_t d_target, int32_t d_draft, void* stream);

/*
 * sv_read_floor - measurement aid, not part of the verification: reads the
 * nbytes at `data` (device memory) once, 16 KiB per workgroup with the
 * loads of the streaming pass (16-byte buffer loads, four per thread), and
 * does nothing else with them.  Its duration over a batch's logit bytes is
 * the plain-read floor that the streaming pass of sv_spec_verify is compared
 * against (that pass reads every logit once, as the pages' decode-step cost
 * model has it: page www.gsyq.cn/news/428210 section 1.2).  out (device,
 * ceil(nbytes / 16384) words, caller-owned) receives at out[i] the xor of
 * block i's 32-bit words only when that xor equals key; other words are left
 * as they were.  Asynchronous on `stream`.  Errors: SV_ERR_SHAPE (nbytes < 0,
 * not a multiple of 16, or too many blocks for one launch; data must be
 * 16-byte aligned), SV_ERR_NULL (data or out NULL with
 * nbytes > 0), SV_ERR_HIP (launch failure).  nbytes == 0 does nothing.
 */
int sv_read_floor(const void* data, int64_t nbytes, uint32_t key, uint32_t* out, void* stream);

/*
 * Launch timing for benchmarks.  Between sv_profile_start() and
 * sv_profile_stop(), every sv_spec_verify / sv_spec_verify_debug /
 * sv_spec_verify_dt / sv_spec_verify_ragged / sv_spec_verify_probs /
 * sv_sample call records three HIP events on its own stream: the start and
 * the end of its streaming kernel (the pass that reads every logit once),
 * taken by that kernel's launch (hipExtLaunchKernel), and one after the
 * call's last kernel.  sv_profile_stop() waits for the recorded events and
 * returns the summed durations in milliseconds of the streaming kernel and
 * of what follows it up to the call's end (row merge, sequence
 * finalisation, full-row draw), and the number of calls timed.  Any output
 * pointer may be NULL.  An sv_spec_verify_lmhead call is timed too, with
 * its two projections in place of the streaming kernel.  Timing is
 * host-global (not per device).  Returns SV_ERR_HIP if an event could not be
 * created, recorded or read.
 */
int sv_profile_start(void);
int sv_profile_stop(double* stream_kernel_ms, double* other_kernels_ms, int64_t* calls);

/*
 * sv_init - size the scratch of calls on `stream` (on `device`) up front, so
 * that every later call on that stream within the bounds runs without
 * allocating or synchronising: verification of B <= max_B sequences of
 * K <= max_K drafts with V <= max_V (any mode, dtype and variant; ragged
 * batches of total_draft <= max_B * max_K; sv_sample and sv_filtered_probs
 * of rows <= max_B * (2 * max_K + 1)).  flags: 0, or SV_INIT_LMHEAD to also
 * size the logits buffer of sv_spec_verify_lmhead for those bounds.  Also
 * resolves the address of sv_spec_verify_noalloc's array on `device`.  The
 * current device is restored before returning.  Errors: SV_ERR_PARAM (device
 * outside [0, 64) or unknown flags), SV_ERR_SHAPE (max_B < 0, max_K outside
 * [0, SV_MAX_K], max_V outside [1, SV_MAX_V]), SV_ERR_WORKSPACE (allocation
 * failed), SV_ERR_HIP.  Calling it again with larger bounds grows the
 * buffers (synchronising the stream); with smaller ones it does nothing.
 */
int sv_init(int device, void* stream, int32_t max_B, int32_t max_K, int32_t max_V, int32_t flags);

/* Frees the scratch (and logits buffer) bound to `stream` on the current
 * device, after synchronising the stream.  The next call on the stream
 * allocates again.  Call it before destroying a stream whose handle may be
 * reused. */
int sv_stream_release(void* stream);

/* Frees the scratch (and logits buffers) of every stream on every device the
 * library has used, after synchronising those devices. */
int sv_release(void);

/* Bytes of device scratch and logits buffers currently held on `device`,
 * summed over its streams (0 if none; the array of sv_spec_verify_noalloc is
 * not counted). */
int64_t sv_scratch_bytes(int device);

/* Human-readable name of a status code. */
const char* sv_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
