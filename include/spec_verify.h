/*
 * spec_verify.h -- C ABI of libspecverify.so, the verify-and-resample step of speculative
 * sampling on AMD Instinct MI355X (gfx950).
 *
 * What is computed (notation of the page "Accelerating Large Language Model Decoding with
 * Speculative Sampling", Chen et al. notes: q = TARGET distribution, p = DRAFT distribution,
 * x~ = draft token, K = draft tokens per call):
 *
 *   1. Every logit row is turned into a distribution by temperature, then top-k, then top-p
 *      (section A2, compatibility with standard sampling methods; the Leviathan blog's
 *      section on the standardised sampling framework says the same).  Temperature 0 means
 *      argmax.  Top-k keeps every logit >= the k-th largest (ties kept); top-p keeps the
 *      smallest decreasing-probability prefix whose mass reaches P plus every token tied with
 *      its last member, and renormalises; top-p acts after top-k.
 *   2. Draft token k is accepted with probability a_k = min(1, q_k(x~_k) / (l * p_k(x~_k)))
 *      (section A2, modified rejection sampling; lenience l from the Leviathan blog, App. F),
 *      decided as u[b,k] < a_k.  p = 0 < q gives a = 1; p = q = 0 gives a = 0.
 *   3. n = the first rejected position (K if none).
 *   4. n < K: the token at position n is drawn from (q_n - p_n)_+ (Theorem 1); if that has
 *      zero mass, from q_n.  n = K: a bonus token is drawn from q_K (section A2, the remark
 *      that a call yields up to K+1 tokens).  The draw is the inverse CDF in vocabulary index
 *      order with u[b,K]: the smallest i whose cumulative weight exceeds u * (total weight).
 *
 * Mentored decoding (sv_sampling.mentor_kl = D > 0) replaces steps 2 and 4 per position: over
 * the target's kept tokens, r_i = min(1, q_i / (alpha p_i)) and replacement weights
 * w_i = max(0, q_i / beta - p_i), where beta makes sum_i (p_i r_i + w_i) = 1 and alpha is the
 * upper end of 50 bisection steps on [0, 1] for KL(q || p r + w) <= D; if KL(q || p) <= D
 * every draft token with p > 0 is accepted.  a_k = r at the draft token; the token at n < K is
 * drawn from w (from q if w has no mass).  A position whose target or draft row has more than
 * 1024 kept tokens (ties at the top-k boundary) uses the lossless rule.
 *
 * spec_verify_tree is the greedy exact-match rule for a token tree laid out in BFS order (the
 * REST article, section on retrieval-based speculative decoding): a node is accepted iff its
 * parent is accepted and its token equals the argmax of the parent's target row.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are caller-owned DEVICE memory, row-major and contiguous along V.
 *     Scalars and sv_sampling are host values.  Logit pointers must be aligned to their
 *     element size (else SV_ERR_INVALID_ARG); rows may start at any such offset and V may be
 *     any size (on rows whose start or length is not a multiple of 16 bytes, the final draw of
 *     dense rows and the dense acceptance rates use element-wise loads).
 *   - The library allocates nothing and never synchronises.  All work is enqueued on
 *     `stream`; outputs are valid once the caller synchronises with that stream.
 *   - Arguments are checked on the host before anything is enqueued; on an error status
 *     nothing is enqueued and the outputs are untouched.  A failed kernel launch returns
 *     SV_ERR_LAUNCH.  Device data (tokens, parents) is not checked on the host; the rules for
 *     out-of-range device values are stated per argument.
 *   - Logits must be finite or -inf, and every row needs at least one finite logit.
 *   - `workspace` is caller-owned device memory of at least *_workspace_size() bytes.  It
 *     needs no initialisation; calls that share a workspace must be ordered on one stream.
 *   - The library keeps no global state (apart from spec_verify_noalloc's scratch buffer, one
 *     per GPU) and is deterministic: equal inputs give bitwise equal outputs (fixed-order
 *     reductions, no floating-point atomics).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = 1,          /* a size, pointer or sampling parameter is out of range */
  SV_ERR_UNSUPPORTED_DTYPE = 2,    /* dtype is not SV_DTYPE_F32 / SV_DTYPE_BF16 */
  SV_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < the matching *_workspace_size() */
  SV_ERR_LAUNCH = 4,               /* a kernel launch failed (hipGetLastError) */
  SV_ERR_SCRATCH_TOO_SMALL = 5     /* spec_verify_noalloc: the problem's workspace exceeds the
                                      library's built-in scratch buffer */
} sv_status;

/* Element type of the logit tensors.  An int32_t rather than an enum, so that whatever value a
   caller passes is a valid argument for the library to check (SV_ERR_UNSUPPORTED_DTYPE). */
typedef int32_t sv_dtype;
enum { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1 };

/* Sampling parameters, applied identically to q and p (Chen et al. notes, A2). */
typedef struct {
  float temperature; /* >= 0.  0 = argmax (lowest index on ties) */
  int32_t top_k;     /* >= 0.  0, or >= V, = off */
  float top_p;       /* in (0, 1].  1 = off */
  float lenience;    /* in (0, 1].  1 = the lossless rule; < 1 = App. F of the Leviathan blog */
  float mentor_kl;   /* >= 0, finite.  0 = off; D > 0 = mentored decoding with KL bound D (the
                        community blog on an optimal lossy variant of speculative decoding, its
                        sections on mentored decoding and on solving the optimisation problem).
                        D > 0 with K > 0 requires lenience 1 and, unless temperature is 0, a
                        top-k of 1..256 (top-p may be combined with it); otherwise
                        SV_ERR_INVALID_ARG.  At temperature 0 the rule equals the lossless one. */
} sv_sampling;

/* Bytes of workspace spec_verify needs for these sizes and parameters (0 on invalid input). */
size_t spec_verify_workspace_size(int B, int K, int V, sv_dtype dtype, const sv_sampling* params);

/*
 * One verify-and-resample step for B sequences.
 *
 *   target_logits  [B, K+1, V]          target rows; row K feeds the bonus draw
 *   draft_logits   [B, draft_rows, V]   draft rows; rows 0..K-1 are read; draft_rows in {K, K+1}
 *                                       (may be NULL when K == 0)
 *   dtype          element type of both logit tensors
 *   B >= 1, K >= 0, V >= 1; B*(2K+1) rows must fit in int32 and V*(K+1) elements per sequence
 *   draft_tokens   [B, K] int32; a token outside [0, V) has p = q = 0 and is rejected
 *   uniforms       [B, K+1] float in [0, 1): u[b,k] for accept test k, u[b,K] for the final draw
 *   params         host pointer, see sv_sampling
 *   out_tokens     [B, K+1] int32: x~_0..x~_{n-1}, the drawn token at n, then -1
 *   out_num_accepted [B] int32: n in 0..K (n+1 tokens are emitted)
 *   out_accept_prob  [B, K] float or NULL: a_k for EVERY k, also past the first rejection
 *   out_q_draft      [B, K] float or NULL: q_k(x~_k)
 *   out_p_draft      [B, K] float or NULL: p_k(x~_k)
 */
int spec_verify(const void* target_logits, const void* draft_logits, sv_dtype dtype, int B, int K,
                int V, int draft_rows, const int32_t* draft_tokens, const float* uniforms,
                const sv_sampling* params, int32_t* out_tokens, int32_t* out_num_accepted,
                float* out_accept_prob, float* out_q_draft, float* out_p_draft, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * spec_verify without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * library's own scratch buffer stands in for the workspace.  That buffer is one static device
 * array of SPEC_VERIFY_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's load
 * until the process ends; its device address is looked up once per GPU, on the first call
 * whose stream is on that GPU.  The call allocates nothing (no hipMalloc, no library
 * allocator).
 *   - Arguments and results are those of spec_verify; the results are identical.
 *   - A problem whose spec_verify_workspace_size() exceeds the buffer returns
 *     SV_ERR_SCRATCH_TOO_SMALL before anything is enqueued (64 MiB covers, e.g., B=256 K=7
 *     V=128256 bf16 with top-k 50, which needs about 30 MiB).
 *   - Every call on one GPU uses that GPU's buffer and leaves its contents behind; the kernels
 *     need no initialisation of it.  Calls that may overlap on one GPU (different streams,
 *     host threads, or graph replays in flight) race on the buffer and must be serialised
 *     by the caller, e.g. by issuing them all on one stream.
 *   - SV_ERR_LAUNCH if the buffer's address cannot be obtained from the HIP runtime.
 */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int spec_verify_noalloc(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                        int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                        const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                        int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                        float* out_p_draft, hipStream_t stream);

/*
 * spec_verify with per-phase timing, for profiling.  `events` holds n_events >= 2 events
 * created by the caller with hipEventCreate; the library records events[0] before its first
 * kernel, events[1] after the row-streaming kernel (the one that reads every logit), and, if
 * n_events >= 3, events[2] after its last kernel.  Results are identical to spec_verify.
 */
int spec_verify_profiled(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                         int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                         const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                         int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                         float* out_p_draft, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipEvent_t* events, int n_events);

/*
 * spec_verify for draft rows that spec_sample has already processed.  The draft model draws
 * each draft token from its processed row (spec_sample); that call leaves in its workspace the
 * row's summary (maximum, kept-set threshold and normaliser, the kept tokens), which is exactly
 * what verification needs of the draft row.  With `sample_workspace` holding the workspace of
 * one spec_sample call on the B*K draft rows, row b*K + k = draft_logits[b, k] (so
 * draft_rows == K), made with the same dtype, V and sampling parameters and not used by
 * another call since, only the B*(K+1) target rows are streamed; the draft logits are still
 * read at single tokens.  Results are identical to spec_verify's.  Needs K >= 1, temperature
 * > 0 and top_k in 1..256 (mentored decoding included), else SV_ERR_INVALID_ARG;
 * sample_workspace_bytes >= spec_sample_workspace_size(B*K, V, dtype, params), else
 * SV_ERR_WORKSPACE_TOO_SMALL.  Other arguments as spec_verify.
 */
int spec_verify_presampled(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                           int B, int K, int V, const int32_t* draft_tokens,
                           const float* uniforms, const sv_sampling* params,
                           int32_t* out_tokens, int32_t* out_num_accepted,
                           float* out_accept_prob, float* out_q_draft, float* out_p_draft,
                           const void* sample_workspace, size_t sample_workspace_bytes,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Draw one token per row from its processed distribution: the draft model's own sampling
 * step (Chen et al. notes, A1: the draft samples its K tokens one at a time).  Identical to
 * spec_verify with K = 0 on each row (the "bonus" draw).
 *   logits [R, V], uniforms [R] in [0, 1), out_tokens [R] int32.
 */
size_t spec_sample_workspace_size(int R, int V, sv_dtype dtype, const sv_sampling* params);
int spec_sample(const void* logits, sv_dtype dtype, int R, int V, const float* uniforms,
                const sv_sampling* params, int32_t* out_tokens, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace spec_verify_tree needs (0 on invalid input). */
size_t spec_verify_tree_workspace_size(int B, int N, int V, sv_dtype dtype);

/*
 * Greedy verification of a draft token tree (REST article, retrieval-based speculative
 * decoding: BFS pseudo-sequence, tree attention, exact-match acceptance).
 *
 *   target_logits [B, N, V]: row n = the target's next-token logits after the path root..n
 *   B >= 1, N >= 1, V >= 1, 0 <= max_depth
 *   parent      [B, N] int32: parent[., 0] is ignored (node 0 is the root, the last committed
 *               token); for n >= 1 a valid parent satisfies 0 <= parent < n.  A node with an
 *               invalid parent, or deeper than max_depth, is not accepted.
 *   node_tokens [B, N] int32: token of each node (node 0's is ignored)
 *   out_tokens  [B, max_depth+1] int32: tokens of the accepted path root->d (root excluded),
 *               then the argmax of node d's row (the bonus token), then -1
 *   out_num_accepted [B] int32: depth of d.  d is the deepest accepted node, lowest index on ties.
 *   out_last_node    [B] int32 or NULL: d
 *   Argmax ties go to the lowest vocabulary index.
 */
int spec_verify_tree(const void* target_logits, sv_dtype dtype, int B, int N, int V,
                     const int32_t* parent, const int32_t* node_tokens, int max_depth,
                     int32_t* out_tokens, int32_t* out_num_accepted, int32_t* out_last_node,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * spec_verify_tree with per-phase timing, for profiling.  `events` holds n_events >= 2 events
 * created by the caller with hipEventCreate; the library records events[0] before its first
 * kernel, events[1] after the row-streaming kernel (the per-row argmax, which reads every
 * logit), and, if n_events >= 3, events[2] after its last kernel.  Results are identical to
 * spec_verify_tree.
 */
int spec_verify_tree_profiled(const void* target_logits, sv_dtype dtype, int B, int N, int V,
                              const int32_t* parent, const int32_t* node_tokens, int max_depth,
                              int32_t* out_tokens, int32_t* out_num_accepted,
                              int32_t* out_last_node, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t* events, int n_events);

/*
 * Acceptance rate of every draft position (Leviathan blog, section on the method's theory:
 * beta = 1 - D_LK(p, q) = sum_x min(p(x), q(x)) is the probability that a draft token x ~ p is
 * accepted, alpha = E(beta); with lenience l the test compares against q/l and
 * beta = sum_x min(p(x), q(x)/l)).  Same logits, sizes and sampling parameters as spec_verify
 * (mentor_kl must be 0), no draft tokens or uniforms; K >= 1.
 *   out_beta [B, K] float, device.
 * Workspace: spec_verify_workspace_size(B, K, V, dtype, params) bytes.
 */
int spec_acceptance_rate(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                         int B, int K, int V, int draft_rows, const sv_sampling* params,
                         float* out_beta, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * spec_verify and spec_acceptance_rate in one call: the verify step's results, identical to
 * spec_verify's, plus out_beta [B, K] float (device), identical to spec_acceptance_rate's on
 * the same logits and parameters.  The rates come from the row summaries the verify step makes
 * anyway, so the logits are streamed once; a serving loop can track alpha = mean beta (and the
 * draft length that maximises the wall-clock factor below) at no second pass.
 * K >= 1, out_beta non-NULL and mentor_kl == 0, else SV_ERR_INVALID_ARG.  Workspace:
 * spec_verify_workspace_size(B, K, V, dtype, params) bytes.
 */
int spec_verify_rates(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                      int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                      const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                      int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                      float* out_p_draft, float* out_beta, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Host-side analytics of the same blog (section on the method's theory; FAQ on choosing
 * gamma), for an i.i.d. acceptance rate alpha in [0, 1] and gamma draft tokens per call:
 *   expected tokens per target call  (1 - alpha^(gamma+1)) / (1 - alpha)  (gamma + 1 at 1)
 *   wall-clock factor                 expected tokens / (gamma * c + 1), c = draft/target cost
 *   operations factor                 (gamma * c_hat + gamma + 1) / expected tokens
 *   optimal gamma                     the gamma in 1..max_gamma with the largest wall-clock
 *                                     factor (the smallest on ties)
 * Out-of-range arguments give NaN (-1 for the optimal gamma).  No GPU work.
 */
double spec_expected_tokens(double alpha, int gamma);
double spec_walltime_speedup(double alpha, int gamma, double c);
double spec_ops_factor(double alpha, int gamma, double c_hat);
int spec_optimal_gamma(double alpha, double c, int max_gamma);

/*
 * Draft tree of a REST step (REST article, section on retrieval-based speculative decoding):
 * the candidate continuations retrieved for each sequence are put in a trie whose node weight
 * is the number of candidates starting with that node's prefix; the N-1 nodes first in the
 * order (weight descending, depth ascending, lowest candidate index carrying the prefix
 * ascending) form a subtree (a parent always precedes its children in that order), which is
 * laid out breadth-first -- children of earlier nodes first, siblings in the same order -- as
 * the pseudo-sequence that spec_verify_tree takes.
 *
 *   candidates [B, M, L] int32, device: token ids; a candidate ends at its first negative
 *               entry; duplicates count once each.  1 <= M <= 128, 1 <= L <= 32.
 *   N          nodes per tree, root included, 1 <= N <= 256.
 *   out_parent [B, N] int32: parent's index (-1 for node 0, the root = the context's last
 *               token, carried by the caller; -1 in unused slots)
 *   out_tokens [B, N] int32: token of each node (-1 for the root and unused slots)
 *   out_num_nodes [B] int32: nodes used, 1 + min(N - 1, distinct non-empty prefixes)
 *   out_depth  [B, N] int32 or NULL: prefix length (0 for the root, -1 unused)
 *   out_weight [B, N] int32 or NULL: candidates carrying the prefix (root: non-empty
 *               candidates; -1 unused)
 *   out_mask   [B, N, N] uint8 or NULL: tree attention, 1 iff node j is node i or one of its
 *               ancestors (0 in unused rows and columns)
 * No workspace; deterministic.  Argument errors return SV_ERR_INVALID_ARG before any launch.
 */
int spec_build_tree(const int32_t* candidates, int B, int M, int L, int N, int32_t* out_parent,
                    int32_t* out_tokens, int32_t* out_num_nodes, int32_t* out_depth,
                    int32_t* out_weight, uint8_t* out_mask, hipStream_t stream);

/*
 * Uniforms for the accept tests and draws, generated on the device (the draft -> verify
 * hand-off then needs no host data): Philox4x64-10 (Salmon et al., "Parallel random numbers:
 * as easy as 1, 2, 3", SC 2011) with key (key0, key1).  out[i] = (w_i >> 40) * 2^-24 in
 * [0, 1 - 2^-24], where w_i is word i mod 4 of the Philox block at the 256-bit counter
 * counter + floor(i / 4).  Disjoint counter ranges give independent streams, e.g. counter =
 * step * ceil(n / 4).
 *   n >= 0 (n <= 2^40); out: device float[n] (may be NULL when n == 0).
 * Argument errors return SV_ERR_INVALID_ARG before any launch.
 */
int spec_philox_uniform(uint64_t key0, uint64_t key1, uint64_t counter, int64_t n, float* out,
                        hipStream_t stream);

/* Static string for a status code. */
const char* spec_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
