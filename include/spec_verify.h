/*
 * spec_verify.h -- C ABI of libspecverify, batched speculative-decoding
 * verification on AMD MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *   - "推测解码：先猜几个 token，为什么答案仍然没变" (speculative-decoding tutorial),
 *     section "一轮推测解码究竟发生什么": the target scores gamma+1 positions in one
 *     pass; drafts are examined left to right, draft x_i is accepted with
 *     probability min(1, p_i(x_i)/q_i(x_i)); at the first rejection every later
 *     draft is discarded and one token is drawn from the corrected residual
 *     distribution; if all are accepted one extra token is drawn from the
 *     target's next-position distribution.  A round emits 1..gamma+1 tokens.
 *   - same page, section "为什么“猜错再改”不会偏离目标分布": residual
 *     p'(x) = norm(max(0, p(x) - q(x))); greedy decoding accepts a draft while
 *     it equals the target argmax and emits the target token at the first
 *     mismatch.
 *   - "AdaPLD" page, section 3.3 and Algorithm 1: a draft token tree (main copy
 *     path, branches, successors) verified in one target pass; the accepted
 *     tokens end with the bonus token, and an empty acceptance is one
 *     autoregressive step.
 *
 * Conventions shared by all entry points:
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library keeps no reference after the call returns.
 *   - Calls are asynchronous on `stream` (NULL = the null stream).
 *     They return after enqueueing; results are valid once the stream reaches
 *     that point.
 *   - Scalar and pointer arguments are checked on the host before anything is
 *     launched; on failure the call returns SV_ERR_INVALID_ARG (or
 *     SV_ERR_UNSUPPORTED / SV_ERR_WORKSPACE) and launches nothing.
 *   - Logit tensors are row-major, contiguous in V; dtype SV_F32 (IEEE binary32)
 *     or SV_BF16 (bfloat16).  Logits must not be NaN or +inf; -inf entries are
 *     allowed and mean probability 0, but every row needs a finite entry.
 *     Logit pointers aligned to 16 bytes with V*sizeof(dtype) a multiple of 16
 *     take the vectorised path; other layouts are supported at lower speed.
 *   - Token ids outside [0, V) are never used as addresses: a chain draft id
 *     outside [0, V) is rejected at its position (stochastic: its ratio is 0;
 *     greedy: it never matches) and reported in req_status.
 *   - Argmax ties are broken to the lowest vocabulary index.
 *   - The same inputs give bit-identical outputs (no floating-point atomics).
 *   - The workspace is scratch device memory supplied by the caller, of at
 *     least the size returned by the matching *_workspace_bytes query, aligned
 *     to 256 bytes.  It holds no state between calls; concurrent calls must
 *     not share one workspace.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

/* The HIP stream handle, declared here as the HIP runtime declares it so that
 * this header needs no HIP header; a C99 translation unit that also includes
 * the HIP runtime header includes that one first. */
#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t *hipStream_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1, /* bad scalar, NULL required pointer, misaligned workspace */
    SV_ERR_UNSUPPORTED = 2, /* dtype other than SV_F32/SV_BF16, or a size above a limit */
    SV_ERR_WORKSPACE = 3,   /* workspace_bytes below the required size */
    SV_ERR_HIP = 4,         /* the HIP runtime reported an error while enqueueing */
    SV_ERR_SCRATCH = 5,     /* spec_verify_sample_noalloc: the sizes need more than
                               SV_NOALLOC_SCRATCH_BYTES of scratch */
    /* not statuses: they make the type span every int, so that any int a caller
       passes is a value of the type (the library rejects those it does not know) */
    SV_STATUS_MIN_ENUM = -0x7fffffff - 1,
    SV_STATUS_MAX_ENUM = 0x7fffffff
} sv_status;

typedef enum {
    SV_F32 = 0,
    SV_BF16 = 1,
    SV_DTYPE_MIN_ENUM = -0x7fffffff - 1, /* not dtypes: the type spans every int */
    SV_DTYPE_MAX_ENUM = 0x7fffffff
} sv_dtype;

/* Largest tree (nodes per request) spec_verify_tree accepts. */
#define SV_MAX_TREE_NODES 2048
/* Longest draft chain (K) spec_verify_sample and spec_verify_greedy accept. */
#define SV_MAX_DRAFT_LEN 1024

/* Workspace bytes needed by spec_verify_sample for these sizes (0 if the sizes
 * are invalid). */
size_t sv_sample_workspace_bytes(int B, int K, int V, sv_dtype dt);

/* Workspace bytes needed by spec_verify_greedy (rows_per_req = K+1) or
 * spec_verify_tree (rows_per_req = N). */
size_t sv_greedy_workspace_bytes(int B, int rows_per_req, int V, sv_dtype dt);

/*
 * Stochastic chain verification (speculative sampling).
 *
 *   target_logits [B][K+1][V]  row i (i < K) is the target distribution that
 *                              scores draft i+1; row K is the bonus row.
 *   draft_logits  [B][K][V]    row i is the draft distribution that proposed
 *                              draft i+1 (may be NULL when K = 0).
 *   draft_tokens  [B][K]       int32 draft ids.
 *   u_accept      [B][K]       float32 uniforms in [0,1): draft i is accepted
 *                              iff u_accept[b][i] < p_i(x)/q_i(x).
 *   u_sample      [B][K+1]     float32 uniforms in [0,1); entry n is used for
 *                              the token drawn at row n (residual if n < K,
 *                              bonus if n = K); other entries are ignored.
 *   temperature   T > 0, finite; p = softmax(target/T), q = softmax(draft/T).
 *                 T so small that log2(e)/T overflows float32 (below about
 *                 1e-38) returns SV_ERR_UNSUPPORTED.  Scaled logits are
 *                 formed in float32, so every finite logit needs
 *                 |L| * log2(e) / T < 2^128.
 *   0 <= K <= SV_MAX_DRAFT_LEN.
 *
 * Outputs:
 *   accept_len [B]       n_b in [0, K], accepted drafts.
 *   out_tokens [B][K+1]  the n_b accepted drafts, then the drawn token, then -1.
 *   lse_target [B][K+1]  optional (NULL = not written): log sum_v exp(L[v]/T).
 *   lse_draft  [B][K]    optional: the same for the draft rows.
 *   req_status [B]       optional: 0, or 1 if a draft id of the request is
 *                        outside [0, V).
 *
 * Rows read: when lse_target and lse_draft are both NULL (and K <= 31), the
 * rows of positions after each request's first rejection are skipped, except
 * by segments already in flight when that rejection is decided; otherwise
 * every row is read once for its log-sum-exp.  The outputs are the same.
 *
 * The drawn token is the smallest id v with positive mass m(v) whose running
 * mass sum_{w <= v} m(w) exceeds u * Z, Z the total mass (if none, the largest
 * id with positive mass), where m = max(0, p_n - q_n) after a rejection and
 * m = p_K for the bonus.  If rounding leaves a zero residual after a rejection
 * the token is drawn from p_n with the same uniform.
 */
sv_status spec_verify_sample(const void *target_logits, const void *draft_logits,
                             const int32_t *draft_tokens, const float *u_accept,
                             const float *u_sample, int B, int K, int V, sv_dtype dt,
                             float temperature, int32_t *accept_len, int32_t *out_tokens,
                             float *lse_target, float *lse_draft, int32_t *req_status,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spec_verify_sample without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid allocation.  The call itself allocates nothing.
 *
 * Arguments, outputs, rows read and results are those of spec_verify_sample
 * (the same kernels run), with the workspace taken from a scratch array of
 * SV_NOALLOC_SCRATCH_BYTES (8 MiB) that the library holds in the device memory
 * of every GPU it runs on, from the library's load until the process ends.
 * The array of the current device is used, so `stream` must belong to the
 * current device.  Sizes whose workspace (sv_sample_workspace_bytes) exceeds
 * SV_NOALLOC_SCRATCH_BYTES return SV_ERR_SCRATCH and launch nothing; at
 * V = 151936 bf16 and K = 7 that admits B up to 1186.
 *
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (the kernels clear what must start at zero themselves):
 * calls that overlap on one device - on two streams, or from two host threads
 * without ordering between their streams - race on it and give wrong results.
 * The first call on each device looks up the array's address there
 * (hipGetSymbolAddress) and may return SV_ERR_HIP if that fails.
 */
#define SV_NOALLOC_SCRATCH_BYTES 8388608
sv_status spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits,
                                     const int32_t *draft_tokens, const float *u_accept,
                                     const float *u_sample, int B, int K, int V, sv_dtype dt,
                                     float temperature, int32_t *accept_len, int32_t *out_tokens,
                                     float *lse_target, float *lse_draft, int32_t *req_status,
                                     hipStream_t stream);

/*
 * Greedy chain verification.
 *
 *   target_logits [B][K+1][V], draft_tokens [B][K] (0 <= K <= SV_MAX_DRAFT_LEN).
 *   accept_len [B]      n_b = first i with draft_tokens[b][i] != argmax(row i),
 *                       else K.
 *   out_tokens [B][K+1] drafts 0..n_b-1, argmax(row n_b), then -1.
 *   req_status [B]      optional: 0, or 1 if a draft id is outside [0, V).
 *
 * Rows read: for K <= 31 the rows of positions after each request's first
 * mismatch are skipped, except by segments already in flight when that
 * mismatch is decided; for larger K every row is read.
 */
sv_status spec_verify_greedy(const void *target_logits, const int32_t *draft_tokens, int B, int K,
                             int V, sv_dtype dt, int32_t *accept_len, int32_t *out_tokens,
                             int32_t *req_status, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Greedy tree verification (AdaPLD-style draft trees).
 *
 *   target_logits [B][N][V]  row j is the target prediction after the path
 *                            that ends at node j.
 *   node_tokens   [B][N]     node 0 is the root (its token is not verified).
 *   parents       [B][N]     parents[b][0] = -1 and 0 <= parents[b][j] < j.
 *   1 <= N <= SV_MAX_TREE_NODES.
 *
 * Node j >= 1 is accepted iff its parent is accepted and node_tokens[b][j] ==
 * argmax(row parents[b][j]); the root is accepted.  The chosen node is the
 * deepest accepted node (lowest index among equals).
 *   accept_len [B]      depth of the chosen node, or -1 if the parent array is
 *                       malformed (then path_nodes and out_tokens are all -1).
 *   path_nodes [B][N]   node ids on the path from depth 1 to the chosen node,
 *                       then -1 (for compacting the target's cache).
 *   out_tokens [B][N]   tokens of those nodes, then argmax(row of the chosen
 *                       node) as the bonus, then -1.
 *   req_status [B]      optional: 0, 1 if a node id (j >= 1) is outside
 *                       [0, V), 2 if the parent array is malformed.
 *
 * Rows read: for N <= 64 the rows of nodes known to be rejected (a node whose
 * token differs from its parent row's argmax, and its descendants) are
 * skipped, except by segments already in flight when that is decided; for
 * larger N every row is read.
 */
sv_status spec_verify_tree(const void *target_logits, const int32_t *node_tokens,
                           const int32_t *parents, int B, int N, int V, sv_dtype dt,
                           int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                           int32_t *req_status, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Greedy verification fused with the target's LM-head projection: the logits
 * of every verified position, H W^T, are formed on the matrix cores and reduced
 * to their row argmax at once; they are never written.  (The speculative-
 * decoding tutorial page, section "一轮推测解码究竟发生什么": the target scores
 * every draft position in one parallel pass; the DLite notes, section 2: the
 * D x V vocabulary projection is the per-position cost.)
 *
 *   hidden   [rows][D] bf16: the target's final hidden state of every
 *            verified position, rows = B*(K+1) for a chain (request-major,
 *            position-minor) or B*N for a tree (node-minor).
 *   lm_head  [V][D] bf16: the projection, one row per vocabulary id.
 *   D a positive multiple of 128 (else SV_ERR_UNSUPPORTED); both pointers
 *   16-byte aligned.
 * The logit of id v at a row is the fp32 sum over k of hidden[k] * lm_head[v][k]
 * (products exact, fp32 accumulation in an unspecified order).  Everything
 * else is exactly spec_verify_greedy / spec_verify_tree on those logits.
 * Workspace: sv_lmhead_workspace_bytes(rows, V).
 */
size_t sv_lmhead_workspace_bytes(int rows, int V);

sv_status spec_verify_greedy_lmhead(const void *hidden, const void *lm_head,
                                    const int32_t *draft_tokens, int B, int K, int D, int V,
                                    int32_t *accept_len, int32_t *out_tokens, int32_t *req_status,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

sv_status spec_verify_tree_lmhead(const void *hidden, const void *lm_head,
                                  const int32_t *node_tokens, const int32_t *parents, int B, int N,
                                  int D, int V, int32_t *accept_len, int32_t *path_nodes,
                                  int32_t *out_tokens, int32_t *req_status, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Stochastic chain verification (speculative sampling) fused with the target's
 * LM-head projection: the target rows are the logits H W^T, formed on the
 * matrix cores and reduced at once to the row statistics the acceptance test
 * and the lse outputs need (and to the logit at each draft), so the B*(K+1)
 * target rows are never written.  The one row per request that a token is
 * drawn from is formed again afterwards (B rows of V fp32 logits, in the
 * workspace).  Same pages and sections as spec_verify_sample and
 * spec_verify_greedy_lmhead.
 *
 *   hidden        [B][K+1][D] bf16, lm_head [V][D] bf16, D a positive multiple
 *                 of 128, both 16-byte aligned (as for spec_verify_greedy_lmhead).
 *   draft_logits  [B][K][V] of dtype dt (the draft model's own logits).
 *   draft_tokens, u_accept, u_sample, temperature, and every output: as for
 *                 spec_verify_sample.
 * The target logit of id v at a row is the fp32 sum over k of
 * hidden[k] * lm_head[v][k] (products exact, fp32 accumulation in an
 * unspecified order; both passes over a row walk D in the same order, with the
 * row at a different place in the tile, and were measured on MI355X to agree
 * bit for bit); everything else is spec_verify_sample on those logits.  Every target row is formed whether or
 * not lse outputs are requested.
 * Workspace: sv_sample_lmhead_workspace_bytes(B, K, D, V, dt) (0 for invalid
 * or unsupported sizes).
 */
size_t sv_sample_lmhead_workspace_bytes(int B, int K, int D, int V, sv_dtype dt);

sv_status spec_verify_sample_lmhead(const void *hidden, const void *lm_head, const void *draft_logits,
                                    const int32_t *draft_tokens, const float *u_accept,
                                    const float *u_sample, int B, int K, int D, int V, sv_dtype dt,
                                    float temperature, int32_t *accept_len, int32_t *out_tokens,
                                    float *lse_target, float *lse_draft, int32_t *req_status,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Commit of a verified draft tree's accepted path in the target's KV cache
 * (AdaPLD page, Algorithm 1: the accepted tokens are appended and the context
 * updated; section 3.3: the whole tree is verified in one target pass, which
 * leaves one KV row per tree node).  Moves the rows of the accepted nodes,
 * depth 1 first, into consecutive slots.
 *
 *   src_kv, dst_kv  [G][B][S][row_bytes] bytes on the device, 16-byte
 *                   aligned, row_bytes a positive multiple of 16.  G counts
 *                   independent row groups (e.g. layers x {K, V}).  dst_kv
 *                   may be src_kv (in place); otherwise the two must not
 *                   overlap.
 *   tree_base [B]   slot of tree node 0 of each request.
 *   commit_base [B] slot that receives the first accepted node.
 *   accept_len [B], path_nodes [B][N]  as written by spec_verify_tree.
 *   req_status [B]  optional: 0 committed (accept_len 0 commits nothing);
 *                   1 a slot outside [0, S); 2 accept_len outside [0, N-1],
 *                   or a path node outside [1, N) or not strictly increasing;
 *                   3 in place with commit_base in [tree_base + 2,
 *                   tree_base + N), where a write could land on a source row
 *                   still to be read.  A request with a non-zero status is
 *                   left untouched.
 *
 * For every group g, request b and k < accept_len[b]:
 *   dst[g][b][commit_base[b] + k] = src[g][b][tree_base[b] + path_nodes[b][k]]
 * with every source row read as it was on entry.  The usual in-place call has
 * commit_base = tree_base + 1 (the root's row stays where it is).
 */
sv_status spec_commit_tree_kv(const void *src_kv, void *dst_kv, int G, int B, int S, int row_bytes,
                              const int32_t *tree_base, const int32_t *commit_base,
                              const int32_t *accept_len, const int32_t *path_nodes, int N,
                              int32_t *req_status, hipStream_t stream);

/*
 * AdaPLD lexical retrieval (AdaPLD page, section 3.2 and Algorithm 1,
 * LexicalRetrieval): the positions of each request's reuse context where the
 * last n tokens of its current prefix occur, each with at least one token
 * after it to copy as a draft.
 *
 *   context   [B][L] int32 token ids; request b uses its first lengths[b].
 *   lengths   [B] int32 (device).
 *   queries   [B][n] int32: the last n tokens of each prefix (query[n-1] is
 *             the newest token), 1 <= n <= 64.
 *   count     [B] int32: number of candidates p, n-1 <= p <= lengths[b]-2,
 *             with context[b][p-k] == queries[b][n-1-k] for every k < n.
 *   positions [B][cap] int32: the first min(count, cap) candidates in
 *             ascending order, then -1 (may be NULL when cap == 0).
 *   req_status [B] optional: 0, or 1 if lengths[b] is outside [0, L] (then
 *             count 0).
 * Workspace: sv_ngram_workspace_bytes(B, L).
 */
size_t sv_ngram_workspace_bytes(int B, int L);

sv_status spec_ngram_candidates(const int32_t *context, int B, int L, const int32_t *lengths,
                                const int32_t *queries, int n, int cap, int32_t *count,
                                int32_t *positions, int32_t *req_status, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Measurement aid, not a step of the method: reads the `bytes` bytes at `buf`
 * (device memory, 16-byte aligned, bytes a multiple of 16) once, with the
 * same non-temporal coalesced 16-byte loads as the row passes.  folds[i]
 * (device uint32, sv_read_probe_folds(bytes) entries) receives the XOR of the
 * 32-bit words in bytes [16384 i, 16384 (i + 1)) of the buffer, so every load
 * is used and the writes are 1/4096 of the bytes read.  Timed with the tracer
 * (kernel SV_K_READ_PROBE) it gives the read rate this device reaches.
 */
size_t sv_read_probe_folds(size_t bytes);
sv_status sv_read_probe(const void *buf, size_t bytes, unsigned *folds, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *sv_status_string(sv_status s);

/* Library version string (static storage). */
const char *sv_version(void);

/*
 * Per-kernel timing.  Between sv_trace_begin(capacity, kernel_mask) and
 * sv_trace_end(), every kernel the library launches whose id bit is set in
 * kernel_mask (0 = all kernels) is bracketed by a pair of HIP events recorded
 * on the stream it runs on (up to `capacity` launches; later ones are not
 * timed).  An event pair measures from the start event to the stop event, so
 * it includes the launch latency of that kernel.  sv_trace_end waits for the
 * recorded events, writes up to `max_records` records (kernel id, elapsed
 * milliseconds) and returns how many launches were recorded.  Launches from
 * several host threads are each recorded under their own kernel id, but
 * sv_trace_begin and sv_trace_end must not overlap launches.  Meant for
 * benchmarking.
 */
typedef struct {
    int kernel; /* an sv_kernel_id */
    float ms;   /* elapsed time between the two events */
} sv_kernel_time;

typedef enum {
    SV_K_ROWSTATS = 0,     /* per-row max / sum-exp partials of target and draft rows */
    SV_K_ACCEPT = 1,       /* merge partials, acceptance scan, lse outputs */
    SV_K_RESID_MASS = 2,   /* residual / bonus mass per tile of the chosen row */
    SV_K_RESID_SELECT = 3, /* inverse-CDF selection of the drawn token */
    SV_K_ARGMAX = 4,       /* per-row argmax partials */
    SV_K_MATCH = 5,        /* greedy chain acceptance */
    SV_K_TREE = 6,         /* greedy tree walk */
    SV_K_SKIP_STATS = 7,   /* row statistics + acceptance, skipping rows after a rejection */
    SV_K_SKIP_ARGMAX = 8,  /* row argmax + greedy chain acceptance, skipping rows after a mismatch */
    SV_K_COMMIT = 9,       /* KV rows of accepted tree paths moved to consecutive slots */
    SV_K_LMHEAD = 10,      /* LM-head projection on the matrix cores + row argmax partials */
    SV_K_NGRAM_COUNT = 11, /* lexical retrieval: candidates per chunk */
    SV_K_NGRAM_EMIT = 12,  /* lexical retrieval: candidate positions in order */
    SV_K_SKIP_TREE = 13,   /* node-row argmax + tree walk, skipping rows of rejected nodes */
    SV_K_READ_PROBE = 14,  /* read-only stream (measurement aid) */
    SV_K_LMHEAD_STATS = 15, /* LM-head projection + row statistics partials and draft logits */
    SV_K_LMHEAD_ROWS = 16,  /* LM-head projection of the rows tokens are drawn from, written */
    SV_K_MERGE_PARTS = 17,  /* row partials merged to one per row (fused projection) */
    SV_K_COUNT = 18
} sv_kernel_id;

sv_status sv_trace_begin(int capacity, unsigned kernel_mask);
int sv_trace_end(sv_kernel_time *records, int max_records);
const char *sv_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
