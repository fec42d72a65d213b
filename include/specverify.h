/* specverify.h - C ABI of the MI355X (gfx950) speculative-sampling verification library.
 *
 * The library computes, on one GPU, the data-parallel hot path of lossless speculative sampling
 * and of Saguaro's outcome cache:
 *
 *   spec_verify          - per request: temperature / top-k / nucleus processing of draft and
 *                          target rows, optional Saguaro downweight sigma_{F,C} of the draft, the
 *                          min(1, q/p) acceptance scan with first-rejection cutoff, and the
 *                          correction token from the normalised residual (q - p)+ (or the bonus
 *                          token from the target's extra position when every draft token is
 *                          accepted).  Outputs the verification outcome (k, t*).
 *   saguaro_downweight   - sigma_{F,C} of the processed draft rows (the downweighted set, its
 *                          normaliser and, optionally, the full distribution).
 *   saguaro_cache_build  - the geometric fan-out F_k (Theorem 12) and, per verify depth k, the
 *                          F_k guessed outcome tokens.
 *   saguaro_cache_lookup - hit / miss of the verified outcome (k, t*) against the cache, or the
 *                          branch-reuse test of a branch-complete tree.
 *   saguaro_verify_cache - spec_verify and saguaro_cache_build fused: one pass over the draft
 *                          rows serves both (the cache's token sets are the leading tokens of
 *                          the same rows the verification reads).
 *   saguaro_backup_plan  - the batch-aware fallback on a cache miss: which requests take the
 *                          random-token backup speculator this round (verified by spec_verify
 *                          with SPEC_UNIFORM_DRAFT).
 *   mirror_signposts     - Mirror-SD early-exit signposts: the kappa most likely tokens of a
 *                          logit row with their log-probabilities (the draft's token-channel
 *                          message).
 *   mirror_tree_lookup   - reuse of the committed prefix against a draft tree that may branch
 *                          below its roots.
 *   pyramid_verify       - PyramidSD fuzzy acceptance (lossy, behind its own entry point):
 *                          spec_verify where a position whose distributions are within a
 *                          divergence threshold keeps its drafted token outright.
 *
 * Sources (notation p = draft, q = target, as on the DeepMind page):
 *   [SpS]   "Accelerating LLM Decoding with Speculative Sampling" (DeepMind, arXiv 2302.01318),
 *           knowledge-base reading, sections 1, 3 and 6.
 *   [SSD]   "Speculative Speculative Decoding" reading notes, sections 1.3, 2.2, 4.3, 4.4, 5.1, 7.1.
 *   [SSD-H] hyper.ai summary of arXiv 2603.03251, "Method" (fan-out closed form, sigma_{F,C}).
 *   [MSD]   "Mirror Speculative Decoding" reading notes, sections 2, 3.1, 3.2 and 3.3.
 *   [PSD]   "3-Model Speculative Decoding (PyramidSD)" notes, method, key designs 1 and 2.
 *
 * Conventions for every entry point:
 *   - Array pointers are HIP device memory owned by the caller (unless marked "host"); the
 *     library never allocates, frees or retains them, and keeps no state between calls.
 *   - Every call is asynchronous on `stream` (0 = the default stream); outputs are valid once
 *     the stream has reached them.  Calls on different streams with disjoint outputs and
 *     workspaces may run concurrently.
 *   - Host-detectable argument errors return a negative SPEC_E* code and launch nothing.
 *     Data-dependent conditions are reported per request in status bits (a kernel cannot
 *     return an error code).
 *   - Logits are row-major and contiguous with the vocabulary fastest: draft [B][Kd][V],
 *     target [B][K+1][V]; element type SPEC_FP32 (float) or SPEC_BF16 (bfloat16 bits).
 *   - Token order used by every selection (top-k, nucleus, the downweighted set, cache ranks,
 *     greedy argmax): logit descending, then token id ascending on equal logits.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
enum {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,      /* null pointer, size < 1, F outside [0, SPEC_MAX_F], C outside [0, 1], ... */
    SPEC_EDTYPE = -2,      /* dtype is neither SPEC_FP32 nor SPEC_BF16 */
    SPEC_EWORKSPACE = -3,  /* workspace null or smaller than spec_workspace_bytes() */
    SPEC_EHIP = -4         /* a kernel launch failed (hipGetLastError after the launch) */
};

enum { SPEC_FP32 = 0, SPEC_BF16 = 1 };

#define SPEC_MAX_F 64          /* largest downweighted set */
#define SPEC_MAX_FANOUT 1024   /* largest cache width for one depth */
#define SPEC_MAX_KAPPA 16      /* most signposts per request */
#define SPEC_NOALLOC_SCRATCH_BYTES (32u << 20)  /* static scratch of saguaro_verify_cache_noalloc, per GPU */

/* Per-request processing, applied to the draft AND the target rows of that request ([SpS]
 * section 6: temperature, top-k and nucleus act on both distributions before the correction).
 * Order: temperature, then top-k, then softmax, then nucleus.
 *   temperature  > 0, or 0 for greedy verification (argmax match, [MSD] section 2)
 *   top_k        <= 0 or >= V: off; else keep exactly top_k tokens (ties by lower id)
 *   top_p        in (0, 1): keep the smallest prefix of the token order whose mass reaches
 *                top_p; >= 1: off.  temperature < 0, NaN or top_p <= 0 sets SPEC_ST_BAD_PARAM. */
typedef struct {
    float temperature;
    int32_t top_k;
    float top_p;
} spec_params;

/* flags for spec_verify (and pyramid_verify) */
enum {
    SPEC_SAMPLE_DRAFT = 1, /* draft_tokens is an output: s_j is drawn from the processed (and
                              downweighted) draft row j by inverse CDF in token-id order with
                              Philox lane 2, or is the draft argmax when temperature is 0 */
    SPEC_UNIFORM_DRAFT = 2,/* the draft distribution of every position is uniform on [0, V):
                              the random-token backup speculator ([SSD] section 7.1).  No draft
                              row is read (draft_logits may be NULL), F and C do not apply, and
                              temperature, top-k and top-p act on the target rows only; with
                              SPEC_SAMPLE_DRAFT, s_j = floor(u V) for the Philox lane-2 uniform u
                              (the inverse CDF of the uniform law, taken exactly) */
    SPEC_ASSISTED = 4      /* pyramid_verify only: a rejected position draws its correction from
                              the verifier's processed distribution q_j itself, not from the
                              residual ([PSD] key design 2, the assisted variant) */
};

/* per-request status bits (out_status) */
enum {
    SPEC_ST_EMPTY_RESIDUAL = 8,            /* rejection with no residual mass: t* drawn from q_k */
    SPEC_ST_OUTSIDE_DRAFT_SUPPORT = 16,    /* an evaluated draft token has p'(s) = 0; it is
                                              accepted iff q(s) > 0 */
    SPEC_ST_BAD_LOGIT = 32,                /* NaN / +inf logit, or a row with no finite logit:
                                              k = 0, t* = -1 */
    SPEC_ST_BAD_TOKEN = 64,                /* a draft token outside [0, V): k = 0, t* = -1 */
    SPEC_ST_DEGENERATE_DOWNWEIGHT = 128,   /* C = 0 and the set holds all the draft mass: the
                                              row is left undownweighted */
    SPEC_ST_BAD_PARAM = 256,               /* invalid spec_params: k = 0, t* = -1 */
    SPEC_ST_PLACEMENT = 512                /* the exact-count path found the workgroups of one
                                              position on different XCDs (its slices meet in one
                                              XCD's L2): the request was redone by the general
                                              path.  Never expected; a guard on the launch map */
};

/* Uniforms.  Counter-based Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and counter
 * (round, b, j, 0) gives the block of request b and position j = 0..K; word w of the block
 * becomes the uniform ((w >> 12) + 0.5) * 2^-52 in (0, 1).  Word 0: acceptance u_j; word 1:
 * residual / bonus v_j; word 2: draft sampling (SPEC_SAMPLE_DRAFT). */

/* Bytes of scratch spec_verify needs for B requests of K draft positions over V tokens (pure
 * host function).  The workspace must be zero-filled before its first use; every call that
 * completes leaves its arrival counters at zero again, so it can be reused without clearing
 * for the same (B, K, V); the counters' places depend on the shape, so a workspace taken over
 * for another shape is zero-filled again first.  It carries no results between calls.  One
 * workspace serves one call at a time. */
size_t spec_workspace_bytes(int B, int K, int V);

/* spec_verify - batched speculative-sampling verification ([SpS] sections 1 and 3; [SSD]
 * section 2.2; outcome (k, t*) as in [SSD] section 1.3).
 *
 * For each request b, with p_j the processed draft row j after sigma_{F,C} (F > 0 and C < 1;
 * [SSD-H] Method, [SSD] section 4.4) and q_j the processed target row j:
 *   for j = 0..K-1: accept s_j iff u_j * p_j(s_j) < q_j(s_j); stop at the first rejection.
 *   k = number of accepted tokens.  k < K: t* ~ (q_k - p_k)+ / sum (q_k - p_k)+ with v_k;
 *   k = K: t* ~ q_K with v_K.  Sampling is the inverse CDF in token-id order: the first token
 *   whose running mass exceeds v times the total.  Greedy requests (temperature 0) accept s_j
 *   iff it is the argmax of q_j and take t* = argmax q_k.
 *
 *   draft_logits    [B][draft_rows][V]; draft_rows = K or K+1 (row K, used by the cache, is
 *                   ignored here); not read with SPEC_UNIFORM_DRAFT
 *   target_logits   [B][K+1][V]
 *   params          [B] spec_params (device)
 *   F, C            downweighted set size (0 = off) and factor in [0, 1] (1 = off)
 *   draft_tokens    [B][K] int32: read, or written when flags has SPEC_SAMPLE_DRAFT
 *   seed, round     Philox key and first counter word
 *   out_k           [B] int32 in [0, K]
 *   out_tstar       [B] int32 correction / bonus token, -1 for bad requests
 *   out_resid_mass  [B] float: sum (q_k - p_k)+ when k < K, else 0 (nullable)
 *   out_status      [B] uint32 status bits (nullable)
 *   workspace       >= spec_workspace_bytes(B, K, V) bytes of device memory
 * Paths: bf16 logits with V % 8 == 0, 2048 <= V <= 262144, 16-byte aligned rows and K <= 63
 * take the exact-count path (two launches); every other shape takes the general path (one
 * workgroup per position).  Both give the same outputs.
 * Returns SPEC_OK or a negative SPEC_E* code. */
int spec_verify(const void* draft_logits, int draft_rows, const void* target_logits, int dtype, int B, int K,
                int V, const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                uint64_t round, uint32_t flags, int32_t* out_k, int32_t* out_tstar, float* out_resid_mass,
                uint32_t* out_status, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* saguaro_downweight - Saguaro sampling sigma_{F,C} ([SSD-H] Method; [SSD] section 4.4 with the
 * Theorem 19 example): on each processed draft row j < K the first F tokens of the token order
 * that carry mass form the set S; with P_S their mass, Z = 1 - (1 - C) P_S and
 * p'_i = p_i C / Z on S, p_i / Z elsewhere.
 *   out_ids    [B][K][F] int32, S in rank order, -1 past its end
 *   out_Z      [B][K] float (nullable)
 *   out_probs  [B][K][V] float, the full p' (nullable; for tests)
 *   out_status [B][K] uint32 (nullable): SPEC_ST_BAD_LOGIT / _BAD_PARAM / _DEGENERATE_DOWNWEIGHT */
int saguaro_downweight(const void* draft_logits, int draft_rows, int dtype, int B, int K, int V,
                       const spec_params* params, int F, float C, int32_t* out_ids, float* out_Z, float* out_probs,
                       uint32_t* out_status, hipStream_t stream);

/* Host helper: the Theorem 12 fan-out ([SSD] section 4.3; [SSD-H] Method).  Real values
 * F_k = F0 a^{k/(1+r)} (k < K) and F_K = F0 a^{K/(1+r)} (1 - a)^{-1/(1+r)} with F0 such that
 * they sum to `budget`; integers by largest remainder (ties to the smaller k) so that they
 * sum to the budget exactly.  a in (0, 1), r > -1.  out_fanout [K+1] host. */
int saguaro_fanout(int K, int budget, double a, double r, int32_t* out_fanout);

/* saguaro_cache_build - the outcome cache's token sets ([SSD] section 5.1; [SSD-H] Method).
 * For depth k < K: the first F_k tokens of draft row k in token order other than the drafted
 * token s_k; for depth K: the first F_K tokens of draft row K.  NaN logits rank last.
 *   draft_logits     [B][K+1][V]
 *   draft_tokens     [B][K]
 *   out_fanout_host  [K+1] host, the fan-out used (nullable)
 *   out_cache        [B][budget] int32, depth-major, rank order, -1 past a row's end */
int saguaro_cache_build(const void* draft_logits, int dtype, int B, int K, int V, const int32_t* draft_tokens,
                        int budget, double a, double r, int32_t* out_fanout_host, int32_t* out_cache,
                        hipStream_t stream);

/* saguaro_verify_cache - spec_verify followed by saguaro_cache_build on the same inputs, in
 * one pass over the logits ([SSD] sections 4.3 and 5.1: the cache is built from the draft
 * distributions the verification reads).  Outputs are exactly those of
 *   spec_verify(draft_logits, K + 1, target_logits, dtype, B, K, V, params, F, C, draft_tokens,
 *               seed, round, flags, out_k, out_tstar, out_resid_mass, out_status, workspace, ...)
 *   saguaro_cache_build(draft_logits, dtype, B, K, V, draft_tokens, budget, a, r,
 *                       out_fanout_host, out_cache, stream)
 * (with SPEC_SAMPLE_DRAFT the cache leaves out the drafted tokens this call samples).
 *   draft_logits  [B][K+1][V] (draft row K feeds the cache only)
 *   workspace     spec_workspace_bytes(B, K, V) bytes, same contract as spec_verify
 * Return codes: as spec_verify and saguaro_cache_build (SPEC_EINVAL also for a null out_cache
 * or an invalid fan-out). */
int saguaro_verify_cache(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                         const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                         uint64_t round, uint32_t flags, int budget, double a, double r, int32_t* out_fanout_host,
                         int32_t* out_k, int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status,
                         int32_t* out_cache, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* saguaro_backup_plan - the batch-aware fallback on a cache miss ([SSD] section 7.1; [SSD-H]
 * Method, fallback).  Any miss makes the whole batch wait for the fallback, so from a critical
 * batch size b_star on, the missed requests switch to the fast random-token backup speculator
 * (verified with SPEC_UNIFORM_DRAFT) while requests that hit keep their cached speculation;
 * below b_star the primary drafter serves the misses.  The text does not give b_star's formula,
 * so it is an argument.
 *   hit             [B] uint8, the lookup's per-request hit flags
 *   batch           [2] int32, the lookup's {hit count, all-hit flag}
 *   out_use_backup  [B] int32: 1 where request b takes random tokens this round
 *   out_switch      [1] int32: 1 when the backup serves this round (a miss and B >= b_star)
 * Returns SPEC_EINVAL for a null pointer or B < 1. */
int saguaro_backup_plan(int B, const uint8_t* hit, const int32_t* batch, int b_star, int32_t* out_use_backup,
                        int32_t* out_switch, hipStream_t stream);

/* saguaro_cache_lookup - hit / miss of the verified outcome.
 * mode 0 ([SSD-H] Method: cache lookup; [SSD] section 7.1): cache [B][sum F] from
 *   saguaro_cache_build, fanout_or_shape = the [K+1] fan-out (host), k / tstar [B];
 *   out_slot[b] = offset(k_b) + rank of t*_b in C_{k_b}, or -1 on a miss.
 * mode 1 ([MSD] sections 3.2-3.3, branch-complete tree): cache = branch tokens [B][kappa][gamma],
 *   fanout_or_shape = {kappa, gamma} (host), k / tstar [B][kappa] per chain, chain 0 of each
 *   request being the verified path; out_slot[b] = lowest branch whose first k+1 tokens equal
 *   (accepted tokens, t*), -1 if none, -2 when all gamma tokens were accepted.
 *   out_hit [B] uint8 (slot >= 0); out_batch [2] int32 = {hits, 1 if every request hit}. */
int saguaro_cache_lookup(int mode, const int32_t* cache, const int32_t* fanout_or_shape, int K, int B,
                         const int32_t* k, const int32_t* tstar, int32_t* out_slot, uint8_t* out_hit,
                         int32_t* out_batch, hipStream_t stream);

/* mirror_signpost_workspace_bytes - device workspace mirror_signposts needs for (B, V, kappa);
 * 0 for sizes it rejects.  Same contract as the verification workspace: zero-filled before its
 * first use; every completed call leaves its arrival counters at zero again (the rest is
 * scratch each call writes before reading), so it is reused without clearing; one call at a
 * time per workspace. */
size_t mirror_signpost_workspace_bytes(int B, int V, int kappa);

/* mirror_signposts - early-exit signposts ([MSD] sections 3.1 and 3.3: the LM head at the
 * early-exit layer gives a distribution p~; its top kappa tokens with log p~ form the message to
 * the draft).  p~ is read as the softmax of the given logits at temperature 1; tokens are
 * ranked by logit descending, ties to the lower id (-0 ties +0), and
 * log p~(v) = z_v - m - log sum_i exp(z_i - m), m the row maximum.
 *   logits         [B][V] device, dtype SPEC_FP32 or SPEC_BF16 (V <= 2^19)
 *   kappa          1..SPEC_MAX_KAPPA signposts per request
 *   out_ids        [B][kappa] int32, rank order; -1 past the vocabulary
 *   out_logp       [B][kappa] float32 log p~ (-inf past the vocabulary or for a -inf logit)
 *   out_logp_bf16  [B][kappa] bf16 bits, round-to-nearest-even of out_logp (nullable): the
 *                  message's compact form
 *   out_status     [B] (nullable): SPEC_ST_BAD_LOGIT for a row with a NaN or +inf logit or no
 *                  finite one (its ids are -1 and its log-probabilities NaN), else 0
 *   workspace      mirror_signpost_workspace_bytes(B, V, kappa) bytes
 * Return codes: SPEC_EINVAL (null pointer, sizes out of range), SPEC_EDTYPE, SPEC_EWORKSPACE,
 * SPEC_EHIP. */
int mirror_signposts(const void* logits, int dtype, int B, int V, int kappa, int32_t* out_ids, float* out_logp,
                     uint16_t* out_logp_bf16, uint32_t* out_status, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* mirror_tree_lookup - reuse against a draft tree ([MSD] sections 3.2-3.3: the committed
 * prefix, accepted tokens then the correction, is reused when it is one of the paths the draft
 * precomputed; the worked example forks below a root).  Per request the tree is N nodes listed
 * parents first: tree_tokens[b][n] and tree_parents[b][n] (-1 for a root, i.e. a signpost the
 * draft expanded).  A node with a negative token or a parent outside [-1, n) is not part of the
 * tree, nor is anything below it.
 *   path_tokens  [B][gamma] the verified chain's draft tokens (gamma <= 1024)
 *   k, tstar     [B] accepted count and correction token (spec_verify's outputs for the chain)
 *   out_node     [B] the lowest node whose root path equals (path[0..k-1], t*), so at depth
 *                k + 1; -1 when there is none (or k, t* out of range), -2 when k == gamma
 *   out_hit      [B] uint8 (out_node >= 0)
 *   out_batch    [2] int32 {hits, 1 if every request hit} (nullable)
 * Returns SPEC_EINVAL for a null pointer or sizes out of range. */
int mirror_tree_lookup(const int32_t* tree_tokens, const int32_t* tree_parents, int B, int N, int gamma,
                       const int32_t* path_tokens, const int32_t* k, const int32_t* tstar, int32_t* out_node,
                       uint8_t* out_hit, int32_t* out_batch, hipStream_t stream);

/* pyramid_verify - fuzzy acceptance ([PSD] key design 1: a drafted token passes when
 * Div(P_verifier, P_drafter) <= tau; one call per stage, drafter -> qualifier with tau_Q and
 * qualifier -> target with tau_T).  Div is read as the Jensen-Shannon divergence in bits
 * (in [0, 1]) of the processed verifier row q_j and the processed, downweighted drafter row
 * p'_j.  Where Div_j <= tau[b], s_j is kept outright; elsewhere the lossless test of
 * spec_verify decides and a rejection draws the correction from the residual, or from q_j with
 * SPEC_ASSISTED.  A threshold below every divergence (e.g. a negative one) is exactly
 * spec_verify.  The output distribution is NOT the verifier's: this is a lossy variant.
 * Arguments as spec_verify (verifier_logits in the place of target_logits), plus
 *   tau        [B] float32 device, per-request thresholds
 *   flags      SPEC_SAMPLE_DRAFT | SPEC_UNIFORM_DRAFT | SPEC_ASSISTED
 *   out_div    [B][K] float32 device (nullable): Div_j of every position whose drafted token
 *              is valid, whether or not the scan reached it
 * bf16 rows with V a multiple of 8, 2048 <= V <= 262144 and 16-byte aligned logits, given (or
 * uniform) drafted tokens, no SPEC_ASSISTED and K < 64 take the register-resident path: a
 * divergence pass runs between its count and resolve kernels.  Everything else runs on the
 * general path (one workgroup per position).  Both sum the divergence in fp64; the decision
 * Div_j <= tau[b] is taken on that sum.  Return codes as spec_verify (SPEC_EINVAL also for a
 * null tau). */
int pyramid_verify(const void* draft_logits, int draft_rows, const void* verifier_logits, int dtype, int B, int K,
                   int V, const spec_params* params, int F, float C, const float* tau, int32_t* draft_tokens,
                   uint64_t seed, uint64_t round, uint32_t flags, int32_t* out_k, int32_t* out_tstar,
                   float* out_resid_mass, uint32_t* out_status, float* out_div, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* saguaro_verify_cache_lookup - one round of Saguaro's verification and outcome cache in one
 * call: saguaro_verify_cache followed by the lookup of the verified outcomes in the cache just
 * built ([SSD] sections 5.1 and 7.1).  Outputs are exactly those of
 *   saguaro_verify_cache(..., out_cache, workspace, workspace_bytes, stream)
 *   saguaro_cache_lookup(0, out_cache, fanout, K, B, out_k, out_tstar, out_slot, out_hit, out_batch, stream)
 * where fanout is the call's fan-out (returned in out_fanout_host).  On the bf16 path the lookup
 * runs inside the verification's last kernel, as each request's outcome is settled (one kernel
 * launch fewer); elsewhere the two calls run one after the other.
 *   out_slot [B] int32, out_hit [B] uint8, out_batch [2] int32 (nullable): as saguaro_cache_lookup
 *   workspace  spec_workspace_bytes(B, K, V) bytes, same contract as spec_verify
 * Return codes: as saguaro_verify_cache (SPEC_EINVAL also for a null out_slot or out_hit). */
int saguaro_verify_cache_lookup(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                                const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                                uint64_t round, uint32_t flags, int budget, double a, double r, int32_t* out_fanout_host,
                                int32_t* out_k, int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status,
                                int32_t* out_cache, int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* saguaro_verify_cache_noalloc - saguaro_verify_cache for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and outputs without the workspace: a static device array of
 * SPEC_NOALLOC_SCRATCH_BYTES inside the library takes its place (each GPU the library runs on
 * holds one until the process ends; the call allocates nothing).  Calls on one GPU share that
 * scratch: the call clears what must start at zero with a fill kernel on `stream` (so shapes
 * may change between calls), and calls that overlap on one GPU (e.g. on two streams) race.
 * Returns SPEC_EWORKSPACE when spec_workspace_bytes(B, K, V) exceeds the scratch (e.g. B = 16,
 * K = 5, V = 128256 needs 18.5 MiB and fits; B = 32 at that K and V does not), SPEC_EHIP when
 * the scratch's device address cannot be had, otherwise the codes of saguaro_verify_cache. */
int saguaro_verify_cache_noalloc(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                                 const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                                 uint64_t round, uint32_t flags, int budget, double a, double r,
                                 int32_t* out_fanout_host, int32_t* out_k, int32_t* out_tstar, float* out_resid_mass,
                                 uint32_t* out_status, int32_t* out_cache, hipStream_t stream);

/* saguaro_verify_cache_lookup_timed - measurement helper, not part of the method:
 * saguaro_verify_cache_lookup with the same arguments and outputs, plus two HIP events
 * (created by the caller, with timing enabled) that bound the execution of the kernel that reads
 * every logit: the start and stop events of the bf16 path's count kernel launch (elsewhere,
 * events recorded on `stream` before and after the verification, ahead of the lookup).
 * hipEventElapsedTime of the pair gives that kernel's duration; the call's outputs and the work
 * done are unchanged.
 * Return codes as saguaro_verify_cache_lookup, SPEC_EINVAL also for a null event, SPEC_EHIP
 * when an event cannot be recorded. */
int saguaro_verify_cache_lookup_timed(const void* draft_logits, const void* target_logits, int dtype, int B, int K,
                                      int V, const spec_params* params, int F, float C, int32_t* draft_tokens,
                                      uint64_t seed, uint64_t round, uint32_t flags, int budget, double a, double r,
                                      int32_t* out_fanout_host, int32_t* out_k, int32_t* out_tstar,
                                      float* out_resid_mass, uint32_t* out_status, int32_t* out_cache,
                                      int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, hipEvent_t count_before,
                                      hipEvent_t count_after);

/* spec_read_ceiling - measurement helper, not part of the method: one plain streaming read of
 * `bytes` bytes of device memory at `data` (16-byte aligned, bytes a multiple of 16), the
 * bandwidth ceiling a verification call that reads the same number of logit bytes is compared
 * against.  sink: [1] uint32 device word, written only if the xor of the data equals a fixed
 * value (never in practice).  Returns SPEC_EINVAL for a null pointer, zero or unaligned sizes. */
int spec_read_ceiling(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
