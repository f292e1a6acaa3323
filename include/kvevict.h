/*
 * kvevict.h -- C ABI of libkvevict: heavy-hitter KV-cache eviction fused into
 * decode attention, for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Each unit u = (layer, sequence, head) keeps a cache of at
 * most `capacity` key/value slots.  A prefill call scores the prompt and builds
 * the cache; each decode call attends one new query over the kept slots, adds
 * every slot's softmax weight to that slot's running score, and evicts the
 * lowest-scoring slot outside the recent window, writing the new token's key
 * and value into it in place.  Sources:
 *   - H2O review page ("H2O: Heavy-Hitter Oracle for Efficient Generative
 *     Inference of Large Language Models"), sections on motivation and on the
 *     proposed method: heavy hitters hold most of the attention; eviction is a
 *     cheap dynamic greedy rule on each decode step's attention statistics,
 *     balancing recency and relevance.
 *   - Scissorhands summary page (Abstract): the cache is held at a fixed budget
 *     and keeps the tokens that were pivotal (persistence of importance).
 *   - FastGen review page ("Model Tells You What to Discard"), Abstract and
 *     proposed-method list, Figure 2 caption: per-head policies -- full cache,
 *     local window, special (+ punctuation) tokens only, frequency (H2O scores)
 *     plus local window.
 *   - HashEvict summary page (original abstract): pre-attention replacement of
 *     the key whose binarised Gaussian projection is farthest in Hamming
 *     distance from the query's, using a small binary structure in GPU memory.
 *
 * Conventions for every call.
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never allocates device memory and never frees what it is given.  All
 *     state lives in one caller-owned workspace (see kvevict_workspace_size).
 *   - Calls are stream-ordered on `stream` (a hipStream_t; NULL is the default
 *     stream) and return once the work is enqueued.  The return code reports
 *     argument and state validation done on the host before anything is
 *     enqueued; on any error nothing is enqueued and no state changes.  A
 *     launch failure reports KVE_EDEVICE.  With the environment variable
 *     KVEVICT_SYNC_CHECK=1 every call also synchronises the stream and reports
 *     device faults as KVE_EDEVICE (debugging only).
 *   - Layouts are dense and row-major; `d` = head_dim, U = batch * heads units
 *     per layer, unit index u = b * heads + h.  Storage dtype of q/k/v is
 *     kve_config.dtype (fp32, fp16 or bf16, little-endian).
 *   - A handle is not thread-safe and its calls must be ordered on one stream
 *     at a time.  No exceptions cross the ABI.
 */
#ifndef KVEVICT_H
#define KVEVICT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kve_ctx* kve_handle;

typedef enum {
  KVE_OK = 0,
  KVE_EINVAL = 1,        /* bad argument: null pointer, out-of-range size, bad table entry */
  KVE_ESTATE = 2,        /* call out of order: decode before prefill, context full */
  KVE_ENOMEM = 3,        /* workspace smaller than kvevict_workspace_size */
  KVE_EDEVICE = 4,       /* a HIP call or kernel launch failed */
  KVE_EUNSUPPORTED = 5   /* valid but not built: dtype/head_dim/policy combination */
} kve_status;

typedef enum { KVE_F32 = 0, KVE_F16 = 1, KVE_BF16 = 2 } kve_dtype;

/* Per-head cache policy (FastGen page, proposed method; H2O page; HashEvict page).
 *   KVE_FULL    keep every token (capacity = max_context); nothing is evicted.
 *   KVE_H2O     heavy + recent slots: a decode step evicts, among the kept
 *               tokens not in the recent window (t - recent, t] (token t
 *               included as a candidate), the one with the lowest accumulated
 *               score, oldest first on equal scores.  The prompt keeps
 *               [P - recent, P) plus the `heavy` best-scoring earlier tokens
 *               (the newer first on equal scores).  FastGen's frequency+local
 *               heads are H2O heads with recent = the local window.
 *   KVE_LOCAL   keep the last `recent` tokens (ring of `recent` slots).
 *   KVE_SPECIAL keep the tokens whose id is set in keep_token_bitmap; the
 *               step-t query also attends token t, which stays only if kept.
 *   KVE_HASH    HashEvict: `heavy` is the budget B.  Before attention, when
 *               the cache is full, the token whose sketch is farthest in
 *               Hamming distance from the query's sketch (oldest first on
 *               equal distance) is replaced by token t; the query then attends
 *               the cache with t in it.  The prompt is replayed through the
 *               same rule from the cache [0, B).
 *   KVE_PERSIST persistence of importance (Scissorhands page, Abstract; the
 *               rule is a reading of its hypothesis): a token is pivotal at a
 *               step if that step's query gives it a weight >= 1/|A|, |A| the
 *               number of keys the query attends (prompt row i: i + 1; decode
 *               step: kept tokens + 1).  Each kept token carries its pivotal
 *               bits of the last `history` steps (1..64); its count is their
 *               number.  Otherwise as KVE_H2O with the count in place of the
 *               accumulated score: heavy + recent slots, the lowest count
 *               outside the recent window is evicted (oldest first on equal
 *               counts), and the prompt keeps [P - recent, P) plus the
 *               `heavy` earlier tokens with the highest counts over the last
 *               `history` prompt rows (the newer first on equal counts).
 *   KVE_ADAPTIVE FastGen profiling (FastGen page, proposed method; the
 *               profile and composites are a reading): at prefill each unit
 *               (sequence, head) tries the composites C1 = special tokens,
 *               C2 = C1 + punctuation, C3 = C2 + `heavy` frequent tokens,
 *               C4 = C3 + a local window of `recent` tokens, in that order,
 *               and takes the first whose end-of-prompt kept set receives at
 *               least `profile_threshold` of the softmax mass of the last
 *               `profile_rows` prompt rows (averaged over the rows); else
 *               C5 = the full cache.  Tokens whose id is in the composite's
 *               id set are kept for good; the others form an H2O cache of
 *               heavy + recent tokens (C1, C2: none; C3: no window).
 *               Capacity max_context.  kvevict_unit_policies reports the
 *               choice. */
typedef enum { KVE_FULL = 0, KVE_H2O = 1, KVE_LOCAL = 2, KVE_SPECIAL = 3, KVE_HASH = 4,
               KVE_PERSIST = 5, KVE_ADAPTIVE = 6 } kve_policy;

typedef struct {
  int32_t layers;              /* >= 1; each layer has its own caches and position counter */
  int32_t batch;               /* >= 1 */
  int32_t heads;               /* >= 1 */
  int32_t head_dim;            /* 64 or 128 */
  int32_t max_context;         /* N >= 1: upper bound on P + T; positions are int32 */
  int32_t dtype;               /* kve_dtype of q/k/v inputs and of the cached K/V */
  float softmax_scale;         /* > 0, or 0 for 1/sqrt(head_dim) */
  /* Host tables, [layers * heads], copied at create; row = layer, column = head.
   * The policy of a head is shared by every sequence of the batch. */
  const int32_t* policy;       /* kve_policy */
  const int32_t* heavy;        /* H2O, PERSIST: heavy slots >= 0; HASH: budget B >= 1;
                                  ADAPTIVE: frequent slots >= 0; others: 0 */
  const int32_t* recent;       /* H2O, PERSIST: recent window >= 0 with heavy + recent >= 1;
                                  LOCAL: window W >= 1; ADAPTIVE: local window >= 0 (the
                                  ADAPTIVE heads of a layer share heavy and recent); others: 0 */
  /* SPECIAL and ADAPTIVE heads only (else may be NULL/0): host bitmaps over
   * token ids, bit (id & 31) of word id >> 5; ids outside [0, vocab) are in
   * no set.  keep_token_bitmap: the SPECIAL heads' kept ids. */
  int32_t vocab;
  const uint32_t* keep_token_bitmap;   /* [(vocab + 31) / 32] */
  /* HASH heads only (else may be NULL/0): sketch width and the Gaussian
   * projection, host, one [head_dim][sketch_bits] row-major matrix per layer
   * of bfloat16 bit patterns.  Bit b of a sketch (b-th least significant) is
   * set iff the exact value of sum_i W[i][b] x[i] is > 0.  The HASH budget is
   * at most 16384 slots (12288 with 64-bit sketches). */
  int32_t sketch_bits;                 /* 16, 32 or 64 */
  const uint16_t* lsh_proj_bf16;       /* [layers][head_dim][sketch_bits] */
  /* PERSIST heads only (else may be NULL): host [layers * heads] history
   * window in steps, 1..64; entries of other heads are ignored. */
  const int32_t* history;
  /* ADAPTIVE heads only (else may be NULL/0): the special and punctuation id
   * sets ([(vocab + 31) / 32] words each), the profiled prompt rows (>= 1;
   * min(profile_rows, P) are used) and the recovered share (finite; above 1
   * always selects the full cache). */
  const uint32_t* special_token_bitmap;
  const uint32_t* punct_token_bitmap;
  int32_t profile_rows;
  float profile_threshold;
  /* Cached K/V format (Scissorhands page, Abstract: the budgeted cache
   * combines with 4-bit quantisation; the format is a reading).
   *   0  rows in the storage dtype.
   *   4  4-bit slots: each row of head_dim elements is head_dim / 32 groups
   *      of 32; a group stores a float32 scale = (its largest magnitude) *
   *      fl32(1/7) and codes c = rint(x / scale) clamped to [-7, 7], the
   *      quotient a correctly rounded float32 division and rint half to even
   *      (a zero scale gives codes 0); the row reads back as c * scale.
   *      Every head of every layer must be KVE_H2O, KVE_PERSIST or KVE_HASH
   *      (KVE_EUNSUPPORTED otherwise).  Prompt scores, sketches and the
   *      prompt output use the inputs at full precision; rows are quantised
   *      when they enter the cache.  H2O and PERSIST steps use token t's own
   *      key and value unquantised at step t; a HASH step attends the cache
   *      after the replacement, so token t is read from its 4-bit slot like
   *      every kept token. */
  int32_t cache_bits;
} kve_config;

/* Bytes of device workspace the configuration needs (including 256-byte
 * alignment of every array).  EINVAL on a bad config. */
kve_status kvevict_workspace_size(const kve_config* cfg, size_t* bytes);

/* Validates cfg, carves `d_workspace` (device memory, >= the size above,
 * 256-byte aligned) and copies the tables to it (synchronous host-to-device
 * copies on the null stream).  The workspace must stay valid until destroy;
 * the handle owns no device memory.  ENOMEM if bytes is too small. */
kve_status kvevict_create(const kve_config* cfg, void* d_workspace, size_t bytes, kve_handle* out);

/* Frees the host-side handle.  Does not touch the workspace. */
kve_status kvevict_destroy(kve_handle h);

/* Prefill of one layer with a prompt of P = prompt_len tokens (1 <= P <=
 * max_context), resetting that layer's caches and setting its position to P.
 * q, k, v: [batch][heads][P][d] in the storage dtype.  token_ids: [batch][P]
 * int32, required if the layer has a SPECIAL or ADAPTIVE head, else may be NULL.
 * out: [batch][heads][P][d] fp32 causal attention of the prompt over itself
 * (uncompressed), or NULL to skip it.
 * H2O heads score every prompt token by the column sums of the causal softmax
 * (the weight each later prompt query gives it, its own row included) and keep
 * the recent window plus the best-scoring earlier tokens (H2O page, proposed
 * method).  PERSIST heads count the pivotal prompt rows among the last
 * `history` ones instead.  HASH heads replay the prompt (HashEvict page).  Positional
 * policies keep what their rule names (FastGen page). */
kve_status kvevict_prefill(kve_handle h, int32_t layer, int32_t prompt_len,
                           const void* q, const void* k, const void* v,
                           const int32_t* token_ids, float* out, void* stream);

/* One decode step of one layer at its current position t (then t + 1): per
 * unit, attention of the step's query over the kept slots and token t, each
 * kept slot's score raised by its softmax weight, then the head's policy
 * frees a slot for token t (H2O review page, proposed method: each decode
 * step's attention statistics drive a greedy eviction of the token expected
 * to matter least, with the recent tokens kept; Scissorhands summary page,
 * Abstract: the cache stays at a fixed budget; FastGen review page, proposed
 * method: the per-head positional and id-based policies; HashEvict summary
 * page, original abstract: HASH heads replace the farthest key by sketch
 * before attention).
 * q, k, v: [batch][heads][d] storage dtype, the new token's projections.
 * token_ids: [batch] int32 (required if the layer has a SPECIAL or ADAPTIVE head).
 * out: [batch][heads][d] fp32 attention output of the step.
 * evicted_pos: [batch][heads] int32, the position that left each unit's cache
 * at this step (for SPECIAL: t itself if not kept), -1 if none; or NULL.
 * ESTATE before the layer's prefill or once t == max_context. */
kve_status kvevict_decode_step(kve_handle h, int32_t layer,
                               const void* q, const void* k, const void* v,
                               const int32_t* token_ids, float* out, int32_t* evicted_pos,
                               void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as kvevict_decode_step, with the same arguments, results and errors,
 * except that layers using the split decode (slot stride above 1,024) keep
 * its per-chunk partials and logits in a static device array of the library
 * (32 MiB per GPU, held from the library's load on that GPU until the process
 * ends) instead of the workspace.  Nothing is allocated and no scratch needs
 * clearing: every partial and logit a step reads is written earlier in the
 * same step.  KVE_EUNSUPPORTED if the layer needs more than the array holds
 * (batch * heads * (chunks * (head_dim + 2) + capacity) * 4 bytes, each part
 * rounded up to 256), KVE_EDEVICE if the array's address could not be looked
 * up when the handle was created.  Every call on one GPU, from any handle,
 * shares the array: calls that overlap on one GPU (different streams or host
 * threads) race and must be serialised by the caller. */
kve_status kvevict_decode_step_noalloc(kve_handle h, int32_t layer,
                                       const void* q, const void* k, const void* v,
                                       const int32_t* token_ids, float* out, int32_t* evicted_pos,
                                       void* stream);

/* Exports one layer's cache in slot order: which prompt and generated
 * tokens each unit still keeps, and their accumulated scores (the kept set
 * the eviction policies maintain -- H2O review page, proposed method:
 * heavy hitters plus recent tokens; Scissorhands summary page, Abstract: the
 * pivotal tokens kept under a fixed budget).
 * pos_out: [batch][heads][capacity] int32 position held by each slot, -1 for
 * an empty slot.  count_out: [batch][heads] int32 number of occupied slots.
 * scores_out: [batch][heads][capacity] float64 accumulated score per slot
 * (H2O heads; PERSIST heads store the 64-bit pivotal history in the same 8
 * bytes, bit k = pivotal k steps before the latest one; ADAPTIVE units that
 * chose C3 or C4 export the score of unprotected tokens and +inf for
 * protected ones; other heads export 0), or NULL.  `capacity` is kvevict_capacity(h, layer). */
kve_status kvevict_kept_indices(kve_handle h, int32_t layer, int32_t* pos_out,
                                int32_t* count_out, double* scores_out, void* stream);

/* Copies one layer's slot contents in slot order (device pointers,
 * stream-ordered; ESTATE before the layer's prefill).  `capacity` is
 * kvevict_capacity(h, layer), U = batch * heads, d = head_dim.
 * cache_bits 0: k_out, v_out [U][capacity][d] storage dtype; the scale
 *   arguments are ignored (may be NULL).
 * cache_bits 4: k_out, v_out [U][capacity][d / 2] bytes, byte b of a row
 *   holding element 2b in its low nibble and 2b + 1 in its high nibble, each
 *   as c + 8; k_scale_out, v_scale_out [U][capacity][d / 32] float32.
 * Slots beyond a unit's count hold stale bytes. */
kve_status kvevict_cache_rows(kve_handle h, int32_t layer, void* k_out, void* v_out, float* k_scale_out,
                              float* v_scale_out, void* stream);

/* The composite each unit of the layer chose at its last prefill (FastGen
 * profiling, KVE_ADAPTIVE heads): choice_out [batch][heads] int32 receives
 * 1 = special, 2 = + punctuation, 3 = + frequent, 4 = + local, 5 = full, and
 * 0 for units of other policies.  Device pointer, stream-ordered; ESTATE
 * before the layer's prefill. */
kve_status kvevict_unit_policies(kve_handle h, int32_t layer, int32_t* choice_out, void* stream);

/* Slots per unit in the layer's layout (the largest per-head capacity of the
 * layer), or -1 for a bad handle/layer. */
int32_t kvevict_capacity(kve_handle h, int32_t layer);

/* The layer's next decode position (P after prefill), -1 before prefill or
 * for a bad handle/layer. */
int32_t kvevict_position(kve_handle h, int32_t layer);

/* Measurement aid, not part of the method: reads `bytes` bytes of device
 * memory at `src` (16-byte aligned, a positive multiple of 16) with the same
 * 16-byte non-temporal loads the decode kernels use for cached rows, and does
 * nothing with them.  Timing it gives the streaming-read ceiling of the GPU
 * for a given byte count, the reference a decode step's achieved bandwidth is
 * compared with (a step's cost is the read of its kept rows: H2O review page,
 * main findings).  `sink` is a device word that is written only in the
 * (practically impossible) case that the bytes a workgroup read XOR to a fixed
 * constant.  Stream-ordered; EINVAL on bad arguments. */
kve_status kvevict_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* kvevict_status_string(kve_status s);

/* Detail of the calling thread's last error ("" if none). */
const char* kvevict_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVEVICT_H */
