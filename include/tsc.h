/*
 * tsc.h -- batched top-k / top-p / min-p sampler with exact support capture, for AMD MI355X
 * (gfx950). C ABI: plain pointers and sizes only.
 *
 * What one call computes, per row r of a [B, V] logits matrix x (definitions from the pages):
 *   - weights w_i = exp((x_i - max x) / T) over the finite logits (a temperature softmax without
 *     its normalizer); a -inf logit is an excluded token (vLLM "Sampling Mask / Distribution
 *     Replay" article, "How it works", steps 1-2);
 *   - joint top-k and top-p on that one distribution, as thresholds that keep every token tied
 *     with a cutoff, so the support may hold more than k tokens; top-p keeps a token when the mass
 *     of the tokens with strictly larger logit is at most top_p times the total mass; then min-p
 *     keeps w_i >= min_p (sglang PR #36630 summary, "Implementation breakdown" items 2-3 and the
 *     "Key code" tie test);
 *   - the token, drawn by the exponential race argmax_i w_i / E_i over the support (Gaudi
 *     cookbook "topk-subset-sampler", "The fix"), with E_i = -ln u_i and u_i a Philox4x32-10
 *     uniform keyed by the row's seed and counter (token id / 4, 0, position lo, position hi),
 *     word id % 4, u = (2 * (word >> 9) + 1) / 2^24 (Salmon et al., SC'11); equal scores go to
 *     the lowest id;
 *   - for opt-in rows only: the support S = {i | w_i > 0 after filtering} packed as token ids in
 *     (logit descending, id ascending) order, its length clamped to the packed width W, the
 *     logprobs log(w_i / sum_S w) and the sampled token's logprob (sglang PR #40986, "Contract",
 *     "Design" and "Checks removed": no opt-in costs nothing, lengths are clamped to the packed
 *     width, a wider support has OVERFLOW status, a greedy row has width 1 and length 1; its
 *     "Correctness" section: the selected logprob equals the token's support logprob).
 *
 * Conventions: all array arguments are DEVICE pointers on the current HIP device unless noted.
 * The call is asynchronous on `stream` (a hipStream_t passed as void*; NULL = default stream);
 * outputs are valid once the stream has synchronized. The caller owns every buffer; the library
 * keeps no per-call state and never allocates device memory on this path. The return code
 * covers host-checkable errors only; per-row data problems go to row_status without a host sync.
 */
#ifndef TSC_H_
#define TSC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the host entry points. */
enum {
  TSC_OK = 0,
  TSC_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad dtype, misaligned logits        */
  TSC_ERR_UNSUPPORTED = 2,      /* a valid request the library does not serve (W too large)    */
  TSC_ERR_WORKSPACE = 3,        /* workspace smaller than tsc_workspace_size()                 */
  TSC_ERR_HIP = 4               /* the HIP runtime reported an error at launch                  */
};

/* Logits element types. */
enum { TSC_DTYPE_F32 = 0, TSC_DTYPE_BF16 = 1 };

/* Per-row status codes written to row_status. */
enum {
  TSC_ROW_OK = 0,
  TSC_ROW_OVERFLOW = 1,      /* opt-in row whose support is wider than W: the first W entries of
                                the ordered support are written, logprobs still use the full S */
  TSC_ROW_NO_SUPPORT = 2,    /* every logit is -inf                                            */
  TSC_ROW_NONFINITE = 3,     /* some logit is NaN or +inf                                       */
  TSC_ROW_INVALID_PARAM = 4, /* temperature negative / non-finite / subnormal, or top_p or min_p
                                NaN or outside [0, 1]                                          */
  TSC_ROW_ABORTED = 5        /* a wait between the waves of the row's workgroup reached its limit
                                (tsc_set_wait_limit): token -1, length 0, selected logprob NaN;
                                the slot's packed entries and bitmask row may be written in part.
                                Never produced by a correct run with the default limit.        */
};

/* Largest packed width W the library accepts. */
#define TSC_MAX_PACKED_WIDTH 16384

/*
 * tsc_sample_with_mask -- sample one token per row and capture the support of opt-in rows.
 *
 * logits       [B, V] row-major with row stride ld >= V elements; float32 or bfloat16 (raw bits)
 *              per dtype; naturally aligned for its element type. Read only.
 * dtype        TSC_DTYPE_F32 or TSC_DTYPE_BF16.
 * B, V, ld     batch rows (>= 0), vocabulary size (1 <= V < 2^31), row stride in elements.
 * temperature  [B] float32: 0 = greedy (first index of the maximum, width-1 support, logprob 0);
 *              otherwise a normal positive finite value.
 * top_k        [B] int32: <= 0 or >= the number of finite logits disables the filter.
 * top_p        [B] float32 in [0, 1]; 1 disables it; 0 keeps only the top tie group.
 * min_p        [B] float32 in [0, 1]; 0 disables it.
 * optin_rows   [R] int32 capture rows; slot j is valid iff 0 <= optin_rows[j] < B and it exceeds
 *              every earlier entry (a strictly ascending list in range makes every slot valid).
 *              An invalid slot gets lengths[j] = 0 and selected_logprob[j] = NaN. May be NULL
 *              when R = 0.
 * R            number of capture slots, 0 <= R <= B. With R = 0 no capture work runs and
 *              packed_ids, logprobs, lengths and selected_logprob may be NULL.
 * seeds        [B] uint64 per-row Philox key.
 * positions    [B] uint64 per-row Philox counter words (e.g. the decode position).
 * W            packed width, 1 <= W <= TSC_MAX_PACKED_WIDTH (ignored when R = 0).
 * tokens       [B] int32 out: sampled token id; -1 when row_status >= TSC_ROW_NO_SUPPORT.
 * row_status   [B] int8 out: one of TSC_ROW_*. OVERFLOW is reported for captured rows only.
 * packed_ids   [R, W] int32 out: slot j's first lengths[j] entries hold the support ids in
 *              (logit descending, id ascending) order; entries past the length are unspecified.
 * logprobs     [R, W] float32 out, aligned with packed_ids; NULL selects "selected mode" (ids and
 *              the selected logprob only).
 * lengths      [R] int32 out: min(|S|, W); 0 for invalid slots and rows with status >= 2.
 * selected_logprob [R] float32 out: the sampled token's logprob (bit-identical to its packed
 *              logprob entry); NaN for invalid slots and rows with status >= 2.
 * workspace, workspace_bytes  device scratch of at least tsc_workspace_size() bytes (may be
 *              NULL when that is 0).
 * stream       hipStream_t as void*.
 * Returns TSC_OK or a TSC_ERR_* code; on an error nothing is launched.
 */
int32_t tsc_sample_with_mask(const void* logits, int32_t dtype, int64_t B, int64_t V, int64_t ld,
                             const float* temperature, const int32_t* top_k, const float* top_p,
                             const float* min_p, const int32_t* optin_rows, int64_t R,
                             const uint64_t* seeds, const uint64_t* positions, int32_t W,
                             int32_t* tokens, int8_t* row_status, int32_t* packed_ids,
                             float* logprobs, int32_t* lengths, float* selected_logprob,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * tsc_sample_with_mask_bits -- tsc_sample_with_mask, plus the exact support of every OVERFLOW
 * slot as a bitmask (vLLM "Sampling Mask / Distribution Replay" article, "How it works" step 2:
 * beside the compact id buffer of bounded width, a bit-packed mask of ceil(V / 8) bytes per row
 * encodes a wider support exactly).
 *
 * All other arguments and outputs are those of tsc_sample_with_mask.
 * support_bits [R, bits_ld] uint8 out, or NULL (then this is tsc_sample_with_mask). Written only
 *              for slots whose row status is TSC_ROW_OVERFLOW: bit i % 8 of byte i / 8 is set iff
 *              token i is in the support S, for 0 <= i < V. The first tsc_support_bits_ld(V)
 *              bytes of the row are written (bits past V are zero); the rest of the row and the
 *              rows of other slots are left untouched. The number of set bits equals |S|.
 * bits_ld      row stride in bytes: a multiple of 16 and >= tsc_support_bits_ld(V); the buffer
 *              must be 16-byte aligned. Both are checked only when support_bits is not NULL and
 *              R > 0 (TSC_ERR_INVALID_ARGUMENT otherwise).
 * Costs nothing extra for rows that do not overflow; an overflowing row adds one write of its
 * bitmask row and one atomic OR per support token.
 */
int32_t tsc_sample_with_mask_bits(const void* logits, int32_t dtype, int64_t B, int64_t V,
                                  int64_t ld, const float* temperature, const int32_t* top_k,
                                  const float* top_p, const float* min_p,
                                  const int32_t* optin_rows, int64_t R, const uint64_t* seeds,
                                  const uint64_t* positions, int32_t W, int32_t* tokens,
                                  int8_t* row_status, int32_t* packed_ids, float* logprobs,
                                  int32_t* lengths, float* selected_logprob,
                                  uint8_t* support_bits, int64_t bits_ld, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of a support bitmask row that tsc_sample_with_mask_bits writes: ceil(V / 8) rounded up
 * to a multiple of 16 (the smallest valid bits_ld); 0 for V < 1. */
int64_t tsc_support_bits_ld(int64_t V);

/*
 * tsc_replay_logprob -- the log-probability of each row's sampled token under new logits,
 * normalized over the support captured for that row (vLLM "Sampling Mask / Distribution Replay"
 * article, section "RL training side: computing pi_theta with the mask": the training logits
 * are masked to the returned support, every other token at -inf, and the log-softmax is taken
 * at the sampled token). With z_i = x_i / T:
 *     selected_logprob[j] = z_a - ln sum_{i in S_j} exp(z_i)      (a = tokens[j])
 * T = 1 is the article's recipe; passing the sampling temperature puts the result on the scale of
 * the sampler's own logprobs. A token outside S_j gets -inf.
 *
 * logits       [N, V] row-major, row stride ld >= V elements, float32 or bfloat16 (dtype): row j
 *              holds the new logits of the position captured in slot j. Read only.
 * temperature  [N] float32: a normal positive finite value (else INVALID_PARAM).
 * packed_ids, lengths  [N, W] int32 and [N] int32, as tsc_sample_with_mask writes them: the
 *              support of row j is its first lengths[j] ids (1 <= lengths[j] <= W, ids in
 *              [0, V), distinct), unless its capture overflowed.
 * capture_status [N] int8 or NULL (all TSC_ROW_OK): the capture's row status. For
 *              TSC_ROW_OVERFLOW the support is read from support_bits; for a status >= 2 the row
 *              gets that status and a NaN logprob.
 * support_bits [N, bits_ld] uint8 or NULL: bitmasks as tsc_sample_with_mask_bits writes them
 *              (bit i % 8 of byte i / 8; bits past V ignored); bits_ld >= ceil(V / 8) bytes.
 * tokens       [N] int32: the sampled token of each row, in [0, V).
 * selected_logprob [N] float32 out; NaN unless row_status is TSC_ROW_OK.
 * logprobs     [N, W] float32 out or NULL: the logprob of each of the first lengths[j] packed ids
 *              (for an overflowing row, of its packed prefix), normalized over the full support.
 * row_status   [N] int8 out: TSC_ROW_OK; TSC_ROW_INVALID_PARAM (temperature, token, length, an
 *              id out of range, an empty support, OVERFLOW without support_bits);
 *              TSC_ROW_NONFINITE (a support logit is NaN or +inf); TSC_ROW_NO_SUPPORT (every
 *              support logit is -inf); or the capture status >= 2 it was given.
 * Asynchronous on `stream`; allocates nothing. Returns TSC_OK or TSC_ERR_* (host checks: sizes,
 * dtype, null pointers, alignment of logits, bits_ld).
 */
int32_t tsc_replay_logprob(const void* logits, int32_t dtype, int64_t N, int64_t V, int64_t ld,
                           const float* temperature, const int32_t* packed_ids,
                           const int32_t* lengths, int32_t W, const int8_t* capture_status,
                           const uint8_t* support_bits, int64_t bits_ld, const int32_t* tokens,
                           float* selected_logprob, float* logprobs, int8_t* row_status,
                           void* stream);

/*
 * tsc_support_csr -- the captured supports back to back (CSR), so that a copy to the host can be
 * sized by the realized support rather than by the packed capacity R * W (sglang PR #40986,
 * "Limitations": the packed [B, max tokens] buffer crosses every step whole).
 *
 * lengths, packed_ids, logprobs  [R], [R, W], [R, W] as tsc_sample_with_mask writes them;
 *              logprobs may be NULL (then csr_logprobs is not written). A length outside
 *              [0, W] counts as clamped into it. Read only.
 * offsets      [R + 1] int64 out: offsets[0] = 0, offsets[j + 1] = offsets[j] + lengths[j].
 * csr_ids      [cap] int32 out: slot j's ids at offsets[j] .. offsets[j + 1] - 1.
 * csr_logprobs [cap] float32 out or NULL, aligned with csr_ids.
 * cap          capacity of the payload buffers in entries: entries at positions >= cap are not
 *              written (offsets[R] is always the full total; R * W never overflows).
 * One kernel (R <= 2048) or two on `stream`, asynchronous, no allocation: the caller reads
 * offsets[R] and copies that many entries. Returns TSC_OK or TSC_ERR_INVALID_ARGUMENT / UNSUPPORTED / HIP.
 */
int32_t tsc_support_csr(const int32_t* lengths, const int32_t* packed_ids, const float* logprobs,
                        int64_t R, int32_t W, int64_t* offsets, int32_t* csr_ids,
                        float* csr_logprobs, int64_t cap, void* stream);

/* Device scratch bytes tsc_sample_with_mask needs for these sizes (currently always 0). */
size_t tsc_workspace_size(int64_t B, int64_t V, int64_t R, int32_t W, int32_t dtype);

/* Static, human-readable name of a TSC_* return code. */
const char* tsc_status_string(int32_t status);

/*
 * tsc_set_wait_limit -- the limit of the bounded waits inside the single-read sampler kernel.
 *
 * The waves of a row's workgroup hand work to each other through flags in shared memory; each
 * wait for such a flag sleeps at most `sleeps` times (one sleep is 64 clocks) before the row
 * gives up with TSC_ROW_ABORTED, so that a row whose flag is never published still ends and the
 * kernel exits normally. 0 restores the default (2^20 sleeps, tens of milliseconds, far beyond
 * any wait of a correct row: microseconds). A small value makes rows give up on purpose, for
 * tests of that path. Process-wide; takes effect at the next launch; returns the previous limit.
 * Not a sampling parameter: results are unchanged for every row that does not report ABORTED.
 */
uint32_t tsc_set_wait_limit(uint32_t sleeps);

/*
 * tsc_set_debug_poison -- a debugging aid for code that reads the capture buffers.
 *
 * While on (nonzero), every tsc_sample_with_mask / tsc_sample_with_mask_bits call that captures
 * rows (R > 0) also fills each slot's packed entries past its length with id -1 and (when
 * `logprobs` is passed) logprob NaN, in one more kernel on the same stream, so that a reader
 * that looks past `lengths[r]` sees values no valid capture holds. Off by default (0) unless the
 * library was built with TSC_DEBUG_POISON defined. Process-wide; takes effect at the next call;
 * returns the previous setting. The entries up to each length, the tokens and every other
 * output are unchanged.
 */
int32_t tsc_set_debug_poison(int32_t on);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t tsc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TSC_H_ */
