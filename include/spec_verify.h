/*
 * spec_verify.h -- C ABI of the batched draft-verification sampler (gfx950).
 *
 * One call verifies a batch of B speculative-decoding requests.  For each
 * request the target model has scored the K drafted positions plus one bonus
 * position in a single verify pass, giving K+1 logit rows over a vocabulary
 * of V tokens (mini-sglang PR #134, "Modifications": verify_drafts takes the
 * draft tokens and the target's K+1 verify-pass logits; spec-decode README,
 * "How it works": the target scores all k+1 positions in one forward pass).
 * The call turns them into an accepted prefix, one bonus or residual token,
 * and per-token target and behaviour log-probs (nanospec README, acceptance
 * rules: every emitted token carries log pi and log mu).
 *
 * Memory and layout
 *   Every pointer is a DEVICE pointer unless stated otherwise.  Logits are
 *   row-major and contiguous: request b, row r starts at element
 *   (b * rows + r) * V.  dtype is SPEC_BF16 (16-bit brain float, read as the
 *   top half of an fp32) or SPEC_F32.  Every array is aligned to its element
 *   size (2 bytes for bf16, 4 for fp32 and int32), as any tensor or array of
 *   that type is.  No output, record, sums or workspace buffer may overlap
 *   an input of the same call (inputs are read through caches that a call's
 *   own writes do not update).  Rows whose start is 16-byte aligned
 *   (pointer % 16 == 0 and V * element size % 16 == 0) take the vector fast
 *   path; any other V is handled element by element.  Logit rows must hold
 *   at least one finite value; -inf entries are allowed and have probability
 *   zero; NaN and +inf give unspecified tokens (never out-of-bounds access).
 *   Softmax is taken at temperature 1; callers pre-scale for other
 *   temperatures.
 *
 * Outputs (caller-owned, device)
 *   out_tokens[b][i]            emitted tokens, i <= out_accept_len[b];
 *                               later entries are set to -1
 *   out_accept_len[b]           number of accepted drafts (0..K); the
 *                               request emits out_accept_len[b] + 1 tokens
 *   out_target_logprob[b][i]    log p_i(token i) under the target softmax
 *   out_behavior_logprob[b][i]  log mu(token i), the probability that this
 *                               sampler emitted it given the drafted token
 *                               (nanospec README, acceptance rules); both
 *                               log-prob arrays may be NULL (then not
 *                               written); later entries are set to 0
 *   out_status[b]               0, or 1 when the request's device data was
 *                               malformed (a consulted draft token outside
 *                               [0,V), or a tree parent outside [-1, i)):
 *                               the offending draft counts as rejected and
 *                               the offending tree node as unmatched.  2
 *                               (every rule) when a wait for data from another
 *                               workgroup of the same launch ran out (about
 *                               a second); the request's other outputs are
 *                               then undefined.
 *                               It does not occur on a working device.
 *
 * Randomness is supplied by the caller (spec-decode README, "Use it": the
 * generator takes an rng), as uniforms[b][K+1] in [0,1): uniforms[b][j]
 * drives the acceptance test of draft j, uniforms[b][K] drives the terminal
 * sample.  Identical inputs give bitwise-identical outputs.
 *
 * Workspace
 *   Each call needs a device workspace of at least
 *   spec_verify_workspace_bytes(B, rows_per_request, V) bytes, 256-byte
 *   aligned, for the per-tile, per-row and per-chunk records passed between
 *   the call's workgroups.  It must be zero-filled before its first call (for
 *   example allocated zeroed); every call leaves every byte of it zero
 *   again, so one workspace serves calls of any rule and shape in turn on
 *   the same stream with no further initialization.  (Every rule's call and
 *   the draft sampler run as one launch whose workgroups pass data through
 *   the workspace while the launch runs, and read a zero word as "not
 *   written yet".)  Calls that run concurrently (different streams) need
 *   different workspaces.  A call that reports status 2 for a request (see
 *   out_status) may leave its workspace dirty: zero-fill it before reusing
 *   it.  The library allocates nothing and keeps no state besides the
 *   one-shot, per-thread profiling hook (spec_verify_profile_next_call) and
 *   the static array of spec_verify_exact_noalloc.
 *
 * Streams and errors
 *   stream is a hipStream_t (NULL = the default stream).  Calls enqueue
 *   their kernels and return without synchronising.  Argument errors are
 *   detected on the host before anything is enqueued and return SPEC_EINVAL,
 *   SPEC_EDTYPE or SPEC_EWORKSPACE; a failed launch returns SPEC_EHIP.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = 1,     /* bad size, null required pointer, bad tau/top_k */
    SPEC_EDTYPE = 2,     /* dtype is neither SPEC_F32 nor SPEC_BF16 */
    SPEC_EWORKSPACE = 3, /* workspace null, misaligned or too small */
    SPEC_EHIP = 4,       /* the HIP runtime refused a launch */
    SPEC_ESCRATCH = 5    /* the call needs more than the static scratch array holds */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Largest K (drafts per request), N (tree nodes per request), V (vocabulary)
 * and B (requests per call).  A call's logits must also span fewer than 2^24
 * tiles of 16 KiB, counted per row (B * rows_per_request * ceil(V * element
 * size / 16 KiB)), since the streaming launch runs one 256-thread workgroup
 * per tile and a launch holds fewer than 2^32 threads; larger calls return
 * SPEC_EINVAL. */
#define SPEC_MAX_K 63
#define SPEC_MAX_NODES 64
#define SPEC_MAX_V 262144
#define SPEC_MAX_B 65536

/*
 * Host-only query.  rows_per_request is the number of logit rows one request
 * streams: K+1 for greedy and relaxed, 2K+1 for exact (target K+1 plus
 * draft K), N for tree.  Returns 0 for invalid sizes.
 */
size_t spec_verify_workspace_bytes(int B, int rows_per_request, int V);

/* Host-only: static description of a status code. */
const char *spec_status_string(int status);

/*
 * Host-only profiling hook (for benchmarks).  The arguments are hipEvent_t
 * handles created by the caller (with timing enabled), or NULL.  The next
 * spec_verify_* or spec_sample_drafts call made from the calling thread
 * launches its streaming kernel (the one that reads every logit once: for
 * the calls made as one launch, that launch) with before_stream and
 * after_stream as the dispatch's own start and stop events, so that
 * hipEventElapsedTime(before_stream, after_stream) is that kernel's
 * duration, and records after_call on its stream after the call's last
 * kernel.  The hook applies to one call and is then cleared; passing NULLs
 * clears it.
 */
void spec_verify_profile_next_call(void *before_stream, void *after_stream, void *after_call);

/*
 * Host-only testing aid for callers that check the timeout path: the bound,
 * in polling rounds, of every wait a single-launch call (greedy, exact,
 * relaxed, power, tree, draft sampler) makes for data from another
 * workgroup of the same launch.  Calls launched afterwards, from any thread, carry it.
 * With 0, a wait that does not find its data on the first poll gives up at
 * once: the request reports status 2 (its other outputs undefined, the
 * workspace possibly left dirty), and every kernel still ends.  A negative
 * limit restores the default (2^20 rounds, about a second).
 */
void spec_set_spin_limit(int limit);

/*
 * Host-only benchmarking aid: the practical read ceiling.  spec_read_ceiling
 * reads `bytes` bytes (a multiple of 16, from a 16-byte aligned device
 * pointer) with the streaming kernel's access pattern and no arithmetic: one
 * workgroup per 16 KiB, non-temporal 16-byte loads; it writes one word per
 * 16 KiB to out (spec_read_ceiling_out_words(bytes) words, device memory;
 * their values carry no meaning).  The profiling hook above applies to it
 * (its only kernel).  SPEC_EINVAL for a null pointer, a misaligned pointer
 * or a size that is zero or not a multiple of 16.
 */
size_t spec_read_ceiling_out_words(size_t bytes);
spec_status spec_read_ceiling(const void *data, size_t bytes, uint32_t *out, void *stream);

/*
 * Greedy chain verification (mini-sglang PR #134, "Modifications",
 * verify_drafts): draft j is accepted while it equals the argmax of target
 * row j (lowest index among equal maxima); the first unmatched row (row K if
 * all match) contributes its argmax as the bonus token.  Behaviour log-probs
 * are 0 (the rule is deterministic).
 *
 *   target_logits  [B][K+1][V]   dtype
 *   draft_tokens   [B][K]        int32
 *   outputs        tokens/log-probs [B][K+1], accept_len/status [B]
 * Log-probs cost one exp per logit; pass NULL for both to skip them.
 */
spec_status spec_verify_greedy(const void *target_logits, spec_dtype dtype,
                               const int32_t *draft_tokens, int B, int K, int V,
                               int32_t *out_tokens, int32_t *out_accept_len,
                               float *out_target_logprob, float *out_behavior_logprob,
                               int32_t *out_status, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Exact (lossless) speculative sampling (spec-decode README, "How it works"
 * and "Provably exact"): with p = softmax(target row j), q = softmax(draft
 * row j), draft x_j is accepted iff uniforms[b][j] < p(x_j)/q(x_j), in order;
 * at the first rejection n the sampler emits y ~ normalize(relu(p_n - q_n))
 * and stops; if all K are accepted it emits y ~ p_K.  y is the inverse CDF of
 * that distribution in ascending token order at uniforms[b][K].  Behaviour
 * log-probs: min(0, log p - log q) for accepted drafts, log(1 - r_n) +
 * log w(y) - log Z for a residual sample, log p_K(y) for the bonus.
 *
 *   target_logits  [B][K+1][V], draft_logits [B][K][V], same dtype
 *   draft_tokens   [B][K] int32, uniforms [B][K+1] float
 */
spec_status spec_verify_exact(const void *target_logits, const void *draft_logits,
                              spec_dtype dtype, const int32_t *draft_tokens, const float *uniforms,
                              int B, int K, int V, int32_t *out_tokens, int32_t *out_accept_len,
                              float *out_target_logprob, float *out_behavior_logprob,
                              int32_t *out_status, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Relaxed acceptance (nanospec README, acceptance rules): draft x_j is
 * accepted iff p_j(x_j) >= tau or x_j is in the target's top-k, where top-k
 * membership is rank based: #{t : l_t > l_{x_j}} < top_k (tied tokens share
 * a rank).  The rule is deterministic, so accepted drafts carry behaviour
 * log-prob 0.  After the first rejection n (or n = K) the sampler emits
 * y ~ p_n by inverse CDF at uniforms[b][K], with behaviour log-prob log p_n(y).
 * Only uniforms[b][K] is read.  tau must not be NaN; top_k >= 0.
 */
spec_status spec_verify_relaxed(const void *target_logits, spec_dtype dtype,
                                const int32_t *draft_tokens, const float *uniforms, int B, int K,
                                int V, float tau, int top_k, int32_t *out_tokens,
                                int32_t *out_accept_len, float *out_target_logprob,
                                float *out_behavior_logprob, int32_t *out_status, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Greedy tree verification (nanospec README: EAGLE-style chain/tree
 * speculation whose output is identical to plain greedy decoding).  Node 0
 * is the root (the last committed token; its token is not verified); node
 * i >= 1 carries node_tokens[b][i] and has parent parents[b][i] < i.  Row i
 * of the logits scores the token that follows node i.  A node is accepted
 * when its token equals the argmax of its parent's row and its parent is
 * accepted.  The deepest accepted node e (lowest index among equal depths)
 * defines the emitted path; the argmax of row e is the bonus token.
 *
 *   target_logits   [B][N][V]
 *   node_tokens     [B][N] int32, parents [B][N] int32 (parents[b][0] ignored)
 *   num_nodes       [B] int32 valid nodes per request (1..N), or NULL for N
 *   out_path_nodes  [B][N] accepted node ids root-first (root excluded), -1 pad
 *   out_tokens, out_target_logprob, out_behavior_logprob [B][N]
 */
spec_status spec_verify_tree(const void *target_logits, spec_dtype dtype,
                             const int32_t *node_tokens, const int32_t *parents,
                             const int32_t *num_nodes, int B, int N, int V,
                             int32_t *out_path_nodes, int32_t *out_tokens, int32_t *out_accept_len,
                             float *out_target_logprob, float *out_behavior_logprob,
                             int32_t *out_status, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Power acceptance (nanospec README, acceptance rules: accept with
 * probability min(1, p/rest)^alpha; stochastic, full support, exact
 * weights).  Reading of "rest": the draft probability q, so draft x_j is
 * accepted iff uniforms[b][j] < a_j = min(1, p_j(x_j)/q_j(x_j))^alpha, in
 * order.  At the first rejection n the sampler emits y ~ p_n (the target row:
 * full support); if all K are accepted it emits y ~ p_K; both by inverse CDF
 * at uniforms[b][K].  Behaviour log-probs: log a_j for accepted drafts,
 * log(1 - a_n) + log p_n(y) after a rejection, log p_K(y) for the bonus.
 * alpha = 1 accepts exactly as spec_verify_exact (only the draw after a
 * rejection differs); alpha = 0 accepts every draft.  alpha must be finite
 * and >= 0.  Shapes, outputs and workspace (rows_per_request 2K+1) as for
 * spec_verify_exact.
 */
spec_status spec_verify_power(const void *target_logits, const void *draft_logits,
                              spec_dtype dtype, const int32_t *draft_tokens, const float *uniforms,
                              int B, int K, int V, float alpha, int32_t *out_tokens,
                              int32_t *out_accept_len, float *out_target_logprob,
                              float *out_behavior_logprob, int32_t *out_status, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Draft-token sampler: the proposal step that feeds the verifier (spec-decode
 * README, "How it works": the draft model samples its k tokens from its own
 * distribution q).  One independent draw per logit row r: the token is the
 * smallest t whose inclusive prefix of softmax(row r) exceeds uniforms[r]
 * (ascending token order, fp64 sums), and out_logprob[r] = log q_r(token),
 * the log-prob the exact rule later reads as log q.  Rows need at least one
 * finite logit.
 *
 *   logits       [rows][V] dtype, e.g. a draft's [B][K][V] logits as B*K rows
 *   uniforms     [rows] float in [0,1)
 *   out_tokens   [rows] int32
 *   out_logprob  [rows] float, or NULL (not written)
 *   out_status   [rows] int32: 0, or 2 when the row's drawing workgroup's
 *                wait for the chunk sums of the same launch ran out (about a
 *                second; the row's other outputs are then undefined, and the
 *                workspace may be left dirty).  It does not occur on a
 *                working device.
 * rows <= SPEC_MAX_B; the workspace (256-byte aligned, zero-filled as above) must
 * hold spec_sample_workspace_bytes(rows, V) bytes.
 */
size_t spec_sample_workspace_bytes(int rows, int V);

spec_status spec_sample_drafts(const void *logits, spec_dtype dtype, const float *uniforms,
                               int rows, int V, int32_t *out_tokens, float *out_logprob,
                               int32_t *out_status, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * ------------------------------------------------------------------------
 * Vocabulary-sharded verification.  When the target's (and draft's) output
 * layer is split over G devices by vocabulary columns, shard s holds columns
 * [s*Vs, (s+1)*Vs) of every logit row, Vs = V / G (V must be a multiple of
 * G).  The rules are the same as above (greedy: mini-sglang PR #134,
 * "Modifications"; exact: spec-decode README, "How it works"; tree: nanospec
 * README); only the data each device holds changes.  Each shard streams its
 * own columns once and exchanges small per-row records instead of logits:
 *
 *   1. stats    every shard: its columns -> one "record slot" (tile maxima,
 *               argmaxes, exp sums; for the exact rule also the logits of
 *               drafted tokens that fall in its columns).
 *   -- exchange 1: all-gather of the G record slots, in shard order, into one
 *               buffer of G * spec_shard_record_bytes(...) bytes.
 *   2. combine  greedy/tree: every shard folds the gathered records, decides
 *               and writes the complete outputs (identical on every shard).
 *      sweep    exact: every shard folds, decides, writes the accepted prefix,
 *               and sums its columns of the row(s) the terminal token is drawn
 *               from into one "sums slot".
 *   -- exchange 2 (exact): all-gather of the G sums slots, in shard order.
 *   3. sample   exact: every shard finds which shard's columns hold the
 *               terminal draw; that shard alone writes the terminal token and
 *               its log-probs; all write that shard's index.
 *   -- exchange 3 (exact): broadcast of the terminal token and its two
 *               log-probs from the owning shard.
 *
 * The exchanges are the caller's (e.g. collectives over the devices); on one
 * device the G shards may share the gathered buffers and the outputs, each
 * call writing its own slot.  Results equal the unsharded entry points' up
 * to floating-point summation order (identical decisions away from near
 * ties); with G = 1 they are bitwise identical.
 *
 * Shapes: the shard's logits are [B][rows][Vs] (rows as above: K+1 target,
 * K draft, N tree), row-major, the shard's own columns only.  Token ids,
 * parents, uniforms and outputs are global (0..V-1) and identical on every
 * shard.  Limits: 1 <= G, V % G == 0, G * ceil(Vs / (16384 / element size))
 * <= 64 and G * ceil(Vs / 4096) <= 64, besides the unsharded limits for V.
 * Record and sums buffers are 256-byte aligned; they need no initialization.
 * Every buffer comes with its size in bytes, gathered inputs included, and
 * is checked before anything is enqueued.  Errors as above (SPEC_EINVAL also
 * for a shard index outside [0, G) and for G or V outside the limits;
 * SPEC_EWORKSPACE for a record, sums, values or workspace buffer that is
 * null, misaligned or too small).
 */

/* Host-only sizes; 0 for invalid arguments.  rows_per_request as for
 * spec_verify_workspace_bytes (K+1 greedy, 2K+1 exact, N tree). */
size_t spec_shard_record_bytes(spec_dtype dtype, int B, int rows_per_request, int V, int G);
size_t spec_shard_sums_bytes(int B, int V, int G);
size_t spec_shard_workspace_bytes(int B);

/* Step 1.  out_record: this shard's slot (record_bytes >= the query).
 * logprobs != 0 adds the exp sums the combine needs for log-probs; the
 * combine may ask for log-probs only if every shard's stats call did. */
spec_status spec_shard_stats_greedy(const void *target_shard, spec_dtype dtype, int B, int K,
                                    int V, int G, int shard, int logprobs, void *out_record,
                                    size_t record_bytes, void *stream);
spec_status spec_shard_stats_tree(const void *target_shard, spec_dtype dtype,
                                  const int32_t *num_nodes, int B, int N, int V, int G, int shard,
                                  int logprobs, void *out_record, size_t record_bytes,
                                  void *stream);
spec_status spec_shard_stats_exact(const void *target_shard, const void *draft_shard,
                                   spec_dtype dtype, const int32_t *draft_tokens, int B, int K,
                                   int V, int G, int shard, void *out_record, size_t record_bytes,
                                   void *stream);

/* Step 2, greedy and tree: records = the G gathered slots (records_bytes >=
 * G * spec_shard_record_bytes(...), else SPEC_EWORKSPACE before any launch).
 * Outputs as for spec_verify_greedy / spec_verify_tree. */
spec_status spec_shard_combine_greedy(const void *records, size_t records_bytes, spec_dtype dtype,
                                      const int32_t *draft_tokens, int B, int K, int V, int G,
                                      int32_t *out_tokens, int32_t *out_accept_len,
                                      float *out_target_logprob, float *out_behavior_logprob,
                                      int32_t *out_status, void *stream);
spec_status spec_shard_combine_tree(const void *records, size_t records_bytes, spec_dtype dtype,
                                    const int32_t *node_tokens, const int32_t *parents,
                                    const int32_t *num_nodes, int B, int N, int V, int G,
                                    int32_t *out_path_nodes, int32_t *out_tokens,
                                    int32_t *out_accept_len, float *out_target_logprob,
                                    float *out_behavior_logprob, int32_t *out_status,
                                    void *stream);

/* Step 2, exact: records = the G gathered record slots (records_bytes >= G *
 * the record query).  Writes outputs 0..accept_len-1 (and the padding after the
 * terminal position), accept_len and status, this shard's sums slot
 * (out_sums, sums_bytes >= spec_shard_sums_bytes) and the decision into the
 * workspace (spec_shard_workspace_bytes(B) bytes, one per shard: step 3 of
 * the same shard reads it). */
spec_status spec_shard_sweep_exact(const void *target_shard, const void *draft_shard,
                                   spec_dtype dtype, const void *records, size_t records_bytes,
                                   const int32_t *draft_tokens, const float *uniforms, int B,
                                   int K, int V, int G,
                                   int shard, int32_t *out_tokens, int32_t *out_accept_len,
                                   float *out_target_logprob, float *out_behavior_logprob,
                                   int32_t *out_status, void *out_sums, size_t sums_bytes,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Steps 2 and 3 of the power rule (spec_verify_power's rule and outputs; alpha
 * finite and >= 0).  Its statistics are the exact rule's: step 1 is
 * spec_shard_stats_exact, with record and sums slots sized alike. */
spec_status spec_shard_sweep_power(const void *target_shard, const void *draft_shard,
                                   spec_dtype dtype, const void *records, size_t records_bytes,
                                   const int32_t *draft_tokens, const float *uniforms, int B,
                                   int K, int V, int G, int shard, float alpha,
                                   int32_t *out_tokens, int32_t *out_accept_len,
                                   float *out_target_logprob, float *out_behavior_logprob,
                                   int32_t *out_status, void *out_sums, size_t sums_bytes,
                                   void *workspace, size_t workspace_bytes, void *stream);
spec_status spec_shard_sample_power(const void *target_shard, const void *draft_shard,
                                    spec_dtype dtype, const void *sums, size_t sums_bytes,
                                    const float *uniforms,
                                    int B, int K, int V, int G, int shard, int32_t *out_tokens,
                                    float *out_target_logprob, float *out_behavior_logprob,
                                    int32_t *out_sample_shard, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* The relaxed rule over shards (spec_verify_relaxed's rule and outputs; tau
 * not NaN, top_k >= 0).  Its rank count #{t : l_t > l_x} needs the drafted
 * token's logit on every shard, so it takes one more exchange first:
 *   0. spec_shard_values_relaxed: the shard whose columns hold a drafted token
 *      writes that token's target logit into its values slot ([B][K] floats,
 *      spec_shard_values_bytes(B, K) bytes; entries of other shards' tokens
 *      are left as they are and never read).
 *   -- exchange 0: all-gather of the G values slots, in shard order.
 *   1. spec_shard_stats_relaxed (values = the gathered slots, values_bytes >=
 *      G * spec_shard_values_bytes(B, K); record slot as above with
 *      rows_per_request K+1).
 *   2, 3. spec_shard_sweep_relaxed and spec_shard_sample_relaxed, as for the
 *      exact rule (no draft logits). */
size_t spec_shard_values_bytes(int B, int K);
spec_status spec_shard_values_relaxed(const void *target_shard, spec_dtype dtype,
                                      const int32_t *draft_tokens, int B, int K, int V, int G,
                                      int shard, void *out_values, size_t values_bytes,
                                      void *stream);
spec_status spec_shard_stats_relaxed(const void *target_shard, spec_dtype dtype,
                                     const int32_t *draft_tokens, const void *values,
                                     size_t values_bytes, int B, int K,
                                     int V, int G, int shard, void *out_record, size_t record_bytes,
                                     void *stream);
spec_status spec_shard_sweep_relaxed(const void *target_shard, spec_dtype dtype, const void *records,
                                     size_t records_bytes, const int32_t *draft_tokens, const float *uniforms, int B,
                                     int K, int V, int G, int shard, float tau, int top_k,
                                     int32_t *out_tokens, int32_t *out_accept_len,
                                     float *out_target_logprob, float *out_behavior_logprob,
                                     int32_t *out_status, void *out_sums, size_t sums_bytes,
                                     void *workspace, size_t workspace_bytes, void *stream);
spec_status spec_shard_sample_relaxed(const void *target_shard, spec_dtype dtype, const void *sums,
                                      size_t sums_bytes, const float *uniforms, int B, int K, int V, int G, int shard,
                                      int32_t *out_tokens, float *out_target_logprob,
                                      float *out_behavior_logprob, int32_t *out_sample_shard,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Step 3, exact: sums = the G gathered sums slots (sums_bytes >= G *
 * spec_shard_sums_bytes(...), else SPEC_EWORKSPACE).  The owning shard writes
 * out_tokens[b][accept_len[b]] and the two log-probs there (NULL log-prob
 * arrays are skipped); every shard writes out_sample_shard[b] = the owning
 * shard (NULL: not written). */
spec_status spec_shard_sample_exact(const void *target_shard, const void *draft_shard,
                                    spec_dtype dtype, const void *sums, size_t sums_bytes,
                                    const float *uniforms,
                                    int B, int K, int V, int G, int shard, int32_t *out_tokens,
                                    float *out_target_logprob, float *out_behavior_logprob,
                                    int32_t *out_sample_shard, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * ------------------------------------------------------------------------
 * Exact verification that allocates nothing, for callers that cannot call
 * hipMalloc: code under HIP graph capture, serving loops and harnesses that
 * forbid device allocation.  Same rule, arguments and outputs as
 * spec_verify_exact, without the workspace: the records the call's
 * workgroups publish to each other (tile, row and chunk records) go to a
 * static device array of SPEC_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.  A call whose workspace
 * size (spec_verify_workspace_bytes(B, 2K+1, V)) exceeds it returns
 * SPEC_ESCRATCH before anything is enqueued; 4 MiB covers, for example,
 * B = 128, K = 8 at V = 262144 in fp32.  The library makes no allocating
 * call on this path.
 *
 * The array is per device and shared by every call on that device.  Each
 * call first zeroes the part it uses, with a fill kernel on the same stream
 * (not hipMemsetAsync, so the call may be captured into a HIP graph): the
 * previous call's contents never matter, even when that call timed out
 * (status 2).  Calls that overlap on one device -- on different streams, or
 * from several threads without ordering -- race on it and corrupt each
 * other's results; calls ordered on one stream are fine.  The device is the
 * calling thread's current HIP device, which must be the one the stream
 * belongs to.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
spec_status spec_verify_exact_noalloc(const void *target_logits, const void *draft_logits,
                                      spec_dtype dtype, const int32_t *draft_tokens,
                                      const float *uniforms, int B, int K, int V,
                                      int32_t *out_tokens, int32_t *out_accept_len,
                                      float *out_target_logprob, float *out_behavior_logprob,
                                      int32_t *out_status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
