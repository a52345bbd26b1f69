/*
 * spec_tree.h - C ABI of libspectree, the MI355X (gfx950) verification hot path
 * of EAGLE-2-style dynamic-tree speculative decoding.
 *
 * Pipeline per decoding step and layer:
 *   spec_tree_build_step (x depth) -> spec_tree_build_finish      draft tree
 *     (or spec_tree_build_step_finish x depth, the same in fewer launches)
 *   spec_tree_attention                                            tree attention
 *     (or spec_tree_attention_fp8 over an E4M3 KV cache)
 *   spec_tree_verify                                               accepted path + bonus
 *   spec_kv_compact                                                keep accepted KV
 *   spec_kv_prune                                 release rejected branches' pages
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *     row-major memory (shapes in brackets, outermost first). The library never
 *     allocates, frees or synchronizes, and keeps no global state besides a
 *     thread-local error string.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     on it and the call returns immediately.
 *   - Return value: SPEC_OK or a negative SPEC_E_* code. Every code is decided
 *     on the host before any launch (shape, range and workspace checks), so a
 *     failing call enqueues nothing; spec_last_error() describes the failure.
 *   - Problems in the DATA (which the host cannot see) never abort: they are
 *     reported in per-sequence `status` words (SPEC_STATUS_* bits) and have
 *     the defined fallbacks documented below.
 *   - Workspaces: caller-allocated device memory (ws, ws_bytes), 16-byte
 *     aligned (else SPEC_E_INVAL), of at least the size the matching
 *     *_workspace_size() returns for the same arguments. A workspace must be zero-filled before its FIRST use; every
 *     call leaves the parts that must start at zero at zero again. Those
 *     parts and the rest sit at opposite ends of ws_bytes (tree build: the
 *     pool at the start, tickets at the end; verification: keys, flags and
 *     tickets at the start, the rest at the end; attention: fixed offsets),
 *     so one zero-filled workspace serves calls of several shapes without
 *     clearing when ws_bytes is at least the *_workspace_size() of each
 *     call's V (verification) taken with the largest B, max_T, max_topk and
 *     max_depth of the calls. The steps and finish of one tree build pass
 *     the same ws and ws_bytes. Calls that share one workspace must not
 *     overlap in time.
 *
 * Notation: B sequences; node 0 of a tree is the root (the last emitted token,
 * whose KV the target writes in the same forward pass) and nodes 1..N are
 * drafts; T_b = N_b + 1 <= max_T <= 65; parents[i] < i; Hq query heads,
 * Hkv KV heads, G = Hq / Hkv (query head h reads KV head h / G); d = head dim.
 */
#ifndef SPEC_TREE_H
#define SPEC_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 1

/* return codes */
#define SPEC_OK 0
#define SPEC_E_INVAL (-1)       /* null pointer, bad shape or range */
#define SPEC_E_UNSUPPORTED (-2) /* valid but not implemented (e.g. head dim 96) */
#define SPEC_E_WORKSPACE (-3)   /* workspace too small */
#define SPEC_E_DEVICE (-4)      /* HIP runtime error at launch */

/* per-sequence status bits (data problems; OR-ed together) */
#define SPEC_STATUS_INVALID_PARENT 1u  /* parents[i] outside [0, i): node treated as a child of the root */
#define SPEC_STATUS_INVALID_TOKEN 2u   /* draft token outside [0, V): never accepted, never tested */
#define SPEC_STATUS_NAN_INPUT 4u       /* NaN in a target row, or in the q row of a sampling node with children */
#define SPEC_STATUS_ZERO_Q 8u          /* sampling node on the path with children but a missing / all-zero q row */
#define SPEC_STATUS_ZERO_RESIDUAL 16u  /* sampling node on the path whose residual max(0, p - q) became zero */
#define SPEC_STATUS_INVALID_PAGE 32u   /* page-table entry outside [0, num_pages): its keys are skipped */
#define SPEC_STATUS_INVALID_LENGTH 64u /* prefix_lens[b] < 0 or prefix + T_b beyond the page table: clamped */
#define SPEC_STATUS_INVALID_PATH 128u  /* accept_len / accept_nodes not a path of the tree: page table left as is */

/* verification modes (per sequence, int8) */
#define SPEC_MODE_GREEDY 0
#define SPEC_MODE_SAMPLE 1

/* Library ABI version (SPEC_ABI_VERSION of the build). Pure host call. */
int32_t spec_abi_version(void);

/* Message of the last failing call on this thread ("" if none). Pure host call. */
const char* spec_last_error(void);

/* ----------------------------------------------------------------------------
 * Draft-tree construction - EAGLE-2 expansion and reranking.
 * Follows the SGLang "Speculative Decoding" page, sections "EAGLE Decoding"
 * (speculative_num_steps = depth D, speculative_eagle_topk = k,
 * speculative_num_draft_tokens = N) and "References" (tree-style expansion
 * with topk branches per step, unlikely branches stop, final rerank to the
 * top N), and lesty.tech "EAGLE-2 & Lookahead Decoding", section 4 "Dynamic
 * Tree Construction Mechanics" (path confidence = product of conditional
 * probabilities = sum of log-probs).
 *
 * Step 1 expands the root's row: its top-k tokens (by log-prob desc, token
 * asc; NaN -> -inf, log-probs >= 0 clamp to 0) become pool entries with score
 * = log-prob (fp64). Step d >= 2 expands each of the k frontier entries f
 * (rank order) with row f of this step: its top-k tokens join the pool with
 * score = parent score + log-prob, and the k best of these k*k candidates (by
 * score desc, pool index asc) are the next frontier. Finish keeps the N best
 * pool entries (same order), numbers them 1..N in pool order, and derives
 * parents, depth, the ancestor bitmask and q_row.
 *
 * Draft rows: the caller's draft model produces, for step d, one log-prob row
 * per frontier slot; rows for sequence b, slot f start at
 * draft_logprobs + b * seq_stride + f * V (fp32). Step 1 reads slot 0 only;
 * step d >= 2 reads slots f < max_topk of EVERY sequence (rows past k_b and
 * rows of sequences with D_b < d are read and ignored), so the buffer holds
 * (B - 1) * seq_stride + max_topk * V floats.
 * Per-sequence k, D, N are device int32 [B] arrays; values outside
 * [1, max_topk], [1, max_depth], [1, min(pool, max_T - 1)] are clamped.
 * ------------------------------------------------------------------------- */
size_t spec_tree_build_workspace_size(int32_t B, int32_t max_topk, int32_t max_depth);

/* step: 1..max_depth (sequences with depth[b] < step are left alone).
 * frontier_tokens: int32 [B, max_topk] out - the new frontier's tokens in rank
 * order (-1 past k_b), i.e. the tokens the draft model extends next.
 * Requires 1 <= max_topk <= 8, 1 <= max_depth <= 16, max_topk <= V. */
int32_t spec_tree_build_step(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                             int64_t seq_stride, const int32_t* topk, const int32_t* depth, int32_t B,
                             int32_t max_topk, int32_t max_depth, int32_t V, int32_t* frontier_tokens,
                             void* stream);

/* Outputs, all [B, max_T]: tokens (node 0 = root_tokens[b]), parents (-1 for
 * the root), depth_out, anc_mask (uint64, bit j-1 set iff draft j is an
 * ancestor of node i or i itself; 0 for the root), q_row (row of the per-
 * sequence draft-row array holding node i's children distribution: 0 for the
 * root, 1 + (d - 1) * max_topk + f for a node that was frontier slot f at
 * depth d < D_b, -1 otherwise). Entries i >= N_b + 1 are -1 / 0. */
int32_t spec_tree_build_finish(void* ws, size_t ws_bytes, const int32_t* root_tokens, const int32_t* topk,
                               const int32_t* depth, const int32_t* num_draft, int32_t B, int32_t max_topk,
                               int32_t max_depth, int32_t max_T, int32_t* tokens, int32_t* parents,
                               int32_t* depth_out, uint64_t* anc_mask, int32_t* q_row, void* stream);

/* Step `step` and, in the same launch, the finish of every sequence whose depth
 * D_b equals `step` (its pool is complete once its last step has run): the
 * outputs are exactly those of spec_tree_build_step followed, after the last
 * step, by spec_tree_build_finish with the same arguments. Calling it for steps
 * 1..max_depth replaces the step calls plus the finish call and saves a launch
 * (the rerank follows the last expansion directly, as on the SGLang page,
 * section "References": the top num_draft_tokens are kept after the last
 * step). Requirements and errors: those of both calls. */
int32_t spec_tree_build_step_finish(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                    int64_t seq_stride, const int32_t* topk, const int32_t* depth, int32_t B,
                                    int32_t max_topk, int32_t max_depth, int32_t V, int32_t* frontier_tokens,
                                    const int32_t* root_tokens, const int32_t* num_draft, int32_t max_T,
                                    int32_t* tokens, int32_t* parents, int32_t* depth_out, uint64_t* anc_mask,
                                    int32_t* q_row, void* stream);

/* Truncated draft vocabulary - SGLang "Speculative Decoding" page, section
 * "EAGLE-2 Decoding via Frequency-Ranked Speculative Sampling" (the draft's
 * LM head covers only a high-frequency token subset, passed as a token map).
 * The same calls with the draft rows over that subset: V is the subset size
 * (the row length) and token_map (device int32 [V]) gives the token that row
 * entry i stands for. Ranking runs on the entry index exactly as above (ties
 * to the smaller index, i.e. the higher-ranked token of the subset); every
 * token the build writes (frontier_tokens, tokens) is token_map[i]. Map
 * values are copied as given (verification checks tokens against its own
 * vocabulary). token_map NULL: identical to the calls without _map. The
 * draft probabilities that spec_tree_verify reads stay over the target's
 * vocabulary (zero outside the subset). Errors: those of the plain calls. */
int32_t spec_tree_build_step_map(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                 const int32_t* token_map, int64_t seq_stride, const int32_t* topk,
                                 const int32_t* depth, int32_t B, int32_t max_topk, int32_t max_depth, int32_t V,
                                 int32_t* frontier_tokens, void* stream);
int32_t spec_tree_build_step_finish_map(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                        const int32_t* token_map, int64_t seq_stride, const int32_t* topk,
                                        const int32_t* depth, int32_t B, int32_t max_topk, int32_t max_depth,
                                        int32_t V, int32_t* frontier_tokens, const int32_t* root_tokens,
                                        const int32_t* num_draft, int32_t max_T, int32_t* tokens, int32_t* parents,
                                        int32_t* depth_out, uint64_t* anc_mask, int32_t* q_row, void* stream);

/* ----------------------------------------------------------------------------
 * Tree mask - tanhdev "Tech Radar: SGLang EAGLE-2", section 2 "Dynamic
 * Tree-Attention Verification" (node i attends exactly to its ancestors and
 * itself) and section 5 "FlashAttention-3 Tree Kernel Design" (one 64-bit
 * word per node; ancestry is one AND).
 * anc_mask[b, i] = anc_mask[b, parents[i]] | (1 << (i - 1)), anc_mask[b, 0] = 0;
 * depth[b, i] = depth of node i. parents int32 [B, max_T]; T_b int32 [B] or
 * NULL (= max_T); anc_mask uint64 [B, max_T]; depth int32 [B, max_T] or NULL;
 * status uint32 [B] or NULL (INVALID_PARENT; such a node hangs off the root).
 * ------------------------------------------------------------------------- */
int32_t spec_tree_mask(const int32_t* parents, const int32_t* T_b, int32_t B, int32_t max_T,
                       uint64_t* anc_mask, int32_t* depth, uint32_t* status, void* stream);

/* ----------------------------------------------------------------------------
 * Tree attention - every tree node attends to the whole paged prefix plus the
 * root, its ancestors and itself (mask as above; the tree is flattened into
 * the sequence as in n1n.ai "Speculative Decoding in Production: EAGLE-3
 * Dynamic Trees", section "From Linear Sequences to Dynamic Draft Trees", and
 * evaluated in one fused pass as in tanhdev section 5).
 *
 * q        bf16 [B, max_T, Hq, d]        query of node i, head h
 * k_pages  bf16 [num_pages, page, Hkv, d] paged KV pool; token slot s of
 * v_pages  bf16 [num_pages, page, Hkv, d] sequence b is in page
 *                                         page_table[b, s / page], row s % page
 * page_table int32 [B, max_pages]
 * prefix_lens int32 [B]: L_b prefix tokens; tree node j's K/V is at slot L_b + j
 * parents  int32 [B, max_T]; T_b int32 [B] or NULL (= max_T)
 * out      bf16 [B, max_T, Hq, d]  (rows of nodes i >= T_b are not written)
 * lse      fp32 [B, max_T, Hq] natural-log log-sum-exp of the scaled scores, or NULL
 * status   uint32 [B] or NULL: INVALID_PARENT / INVALID_PAGE / INVALID_LENGTH (OR-ed in)
 * sm_scale softmax scale (typically 1/sqrt(d)).
 * Supported: d in {64, 128}; page a power of two in [1, 1024]; 1 <= max_T <= 65;
 * Hq % Hkv == 0 and G <= 16; a page (page x Hkv x d x 2 bytes) under 2^31 bytes.
 * q, k_pages, v_pages and out 16-byte aligned (else SPEC_E_INVAL). bf16 inputs,
 * fp32 accumulation and softmax.
 * ------------------------------------------------------------------------- */
size_t spec_tree_attention_workspace_size(int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d,
                                          int32_t page, int32_t max_pages);
int32_t spec_tree_attention(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                            const int32_t* prefix_lens, const int32_t* parents, const int32_t* T_b, int32_t B,
                            int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                            int32_t num_pages, float sm_scale, void* out, float* lse, uint32_t* status, void* ws,
                            size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * FP8-KV variant of tree attention - tanhdev section 3 "Quantitative Hardware
 * Benchmarks on NVIDIA H100" (FP8 targets); n1n.ai page, FAQ "Can speculative
 * decoding be combined with FP8 or AWQ quantization?". The pages fix no
 * format; this variant's is:
 *   k_pages, v_pages  uint8 [num_pages, page, Hkv, d]: OCP E4M3 ("fn") codes;
 *                     slot s's value is code value * k_scale[g] (v_scale[g])
 *   k_scale, v_scale  fp32 [Hkv] device arrays
 *   q                 bf16 as in spec_tree_attention; each (node, head) row is
 *                     rounded to E4M3 (nearest, ties to even) after scaling by
 *                     2^-e, e the smallest integer with max|q| <= 448 * 2^e,
 *                     and stands for code value * 2^e.
 * The attention is spec_tree_attention's over those values. Both products run
 * on E4M3 MFMAs: the softmax weights p (each at most 256 times the row's
 * largest, never above 448) are rounded to E4M3 before the P V product and
 * the row sums add the rounded weights. Codes 0x7f / 0xff (NaN) must not occur.
 * Supported: d = 128 only (SPEC_E_UNSUPPORTED otherwise); all other shapes,
 * arguments, outputs, status bits and the workspace (same size as
 * spec_tree_attention_workspace_size) as spec_tree_attention.
 * ------------------------------------------------------------------------- */
int32_t spec_tree_attention_fp8(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                                const float* v_scale, const int32_t* page_table, const int32_t* prefix_lens,
                                const int32_t* parents, const int32_t* T_b, int32_t B, int32_t max_T, int32_t Hq,
                                int32_t Hkv, int32_t d, int32_t page, int32_t max_pages, int32_t num_pages,
                                float sm_scale, void* out, float* lse, uint32_t* status, void* ws, size_t ws_bytes,
                                void* stream);

/* spec_tree_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * split-K workspace is a library-held device array of 64 MiB per GPU (reserved
 * when the library is loaded, held until the process ends); the call allocates
 * nothing and takes no ws argument. A call whose workspace would exceed 64 MiB
 * (spec_tree_attention_workspace_size) fails with SPEC_E_WORKSPACE and enqueues
 * nothing. All calls on one GPU share that GPU's array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must not be made.
 * Arguments, outputs and other errors: those of spec_tree_attention. */
int32_t spec_tree_attention_noalloc(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                                    const int32_t* prefix_lens, const int32_t* parents, const int32_t* T_b, int32_t B,
                                    int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                                    int32_t num_pages, float sm_scale, void* out, float* lse, uint32_t* status,
                                    void* stream);

/* ----------------------------------------------------------------------------
 * Tree verification - greedy, or rejection sampling with residual resampling
 * (n1n.ai page, section "Mathematical Proof of Lossless Speedup", steps 1-3;
 * tanhdev section 5 "Speculative Rejection Sampling: Mathematical Invariance";
 * lesty.tech "Tree Attention Masking and Target Verification": the longest
 * valid path is accepted and one more token is emitted).
 *
 * target      fp32 [B, max_T, V]: node u's target row - logits for greedy
 *             sequences, probabilities (temperature already applied) for
 *             sampling sequences.
 * draft_probs fp32 [B, R, V] draft probabilities, or NULL if no sequence samples;
 *             q_row int32 [B, max_T] selects node u's children distribution.
 * tokens, parents int32 [B, max_T]; T_b int32 [B] or NULL; mode int8 [B].
 * Philox4x64-10 key (philox_key0, philox_key1); node i of sequence b uses
 * counter (philox_offset, b, i, 0): m = (word0 >> 40) + 1 is its acceptance
 * uniform r = m / 2^24, K = word1 >> 32 its resampling uniform K / 2^32.
 *
 * Greedy: a_u = argmax of row u (ties -> smallest index, NaN = -inf); node i
 * is valid iff its parent is valid and tokens[i] == a_parent; the end node is
 * the deepest valid node (ties -> smallest index); bonus = a_end.
 * Sampling at node u, exact integer arithmetic on 2^-32 fixed point
 * (fx(x) = 0 if NaN or x <= 0, 2^32-1 if x >= 1, else floor(x * 2^32)):
 * P = fx(target row), Q = fx(q row), S_P = sum P, S_Q = sum Q; residual after
 * j rejections N_j[v] = max(0, P[v] S_Q - G_j Q[v]), W_j = sum N_j, G_0 = 0,
 * G_{j+1} = G_j + floor(W_j / S_Q). Children in index order: child c with
 * token t is accepted iff N_j[t] > 0 and m_c Q[t] W_j <= 2^24 N_j[t] S_Q.
 * If none is accepted: bonus = smallest v with 2^32 sum_{w<=v} N[w] > K_u W
 * (argmax of P if W = 0); a leaf, or a node whose q row is missing or sums
 * to 0, resamples from P.
 *
 * Outputs: accept_len int32 [B] (accepted drafts, root and bonus excluded);
 * accept_nodes int32 [B, max_T] (root first, then the accepted nodes);
 * out_tokens int32 [B, max_T] (the accepted drafts' tokens then the bonus:
 * accept_len + 1 entries); status uint32 [B] (overwritten).
 * Requires 1 <= max_T <= 65, 1 <= V < 2^24.
 * ------------------------------------------------------------------------- */
size_t spec_tree_verify_workspace_size(int32_t B, int32_t max_T, int32_t V);
int32_t spec_tree_verify(const float* target, const float* draft_probs, const int32_t* q_row,
                         const int32_t* tokens, const int32_t* parents, const int32_t* T_b, const int8_t* mode,
                         uint64_t philox_key0, uint64_t philox_key1, uint64_t philox_offset, int32_t B,
                         int32_t max_T, int32_t R, int32_t V, int32_t* accept_len, int32_t* accept_nodes,
                         int32_t* out_tokens, uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Tree verification from target logits - the same rule as spec_tree_verify,
 * with the sampling sequences' target distributions formed inside the library
 * from the target's logits and a per-sequence temperature (n1n.ai page,
 * "Mathematical Proof of Lossless Speedup": p is the target model's
 * distribution; SGLang "Speculative Decoding": temperature is a sampling
 * parameter of the request).
 *
 * logits      fp32 [B, max_T, V]: node u's target logits (every sequence).
 * temperature fp32 [B] or NULL (= 1 for every sequence); read for sampling
 *             sequences only.
 * Greedy sequences: exactly spec_tree_verify on the logits (argmax).
 * Sampling sequences: p = softmax(logits / temperature[b]) per row, computed
 * in fp32 (x = l * (1 / T), the row's max, sum of exp(x - max) over slices of
 * the row merged in a fixed order, p = exp(x - max) * (1 / sum), exp of the
 * non-positive x - max through the hardware base-2 exponential; every
 * reduction in a fixed order, so repeated calls agree bit for bit), then
 * exactly the sampling rule of spec_tree_verify on p. p is never stored: one
 * pass over the logits keeps each slice's max and sum, and the sampling
 * passes form p from the logits as they read them. Because p is formed in
 * fp32 rather than supplied, its values can differ from an exact softmax by a
 * few units in the last place, and a decision whose margin is below that can
 * differ from one taken on exact probabilities (a draft row q equal to the
 * exact p is such a case: the exact residual max(0, p - q) is zero, the one
 * left by fp32 p is not). A non-finite logit gives a
 * NaN probability (zero in the rule, SPEC_STATUS_NAN_INPUT); a temperature
 * that is not a finite positive number makes all of that sequence's
 * probabilities NaN.
 * Other arguments, outputs and errors as spec_tree_verify. The workspace
 * (spec_tree_verify_logits_workspace_size) also holds the slices' partials:
 * 8 bytes per 8192 logits beyond the verify workspace, at its end. Requires
 * B * max_T <= 65535.
 * ------------------------------------------------------------------------- */
size_t spec_tree_verify_logits_workspace_size(int32_t B, int32_t max_T, int32_t V);
int32_t spec_tree_verify_logits(const float* logits, const float* temperature, const float* draft_probs,
                                const int32_t* q_row, const int32_t* tokens, const int32_t* parents,
                                const int32_t* T_b, const int8_t* mode, uint64_t philox_key0, uint64_t philox_key1,
                                uint64_t philox_offset, int32_t B, int32_t max_T, int32_t R, int32_t V,
                                int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, uint32_t* status,
                                void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Accepted-path KV compaction - tanhdev section 2 sequence diagram ("Retain
 * Accepted Path KV & Discard Rejected Branches"); lesty.tech section 6
 * ("Paged Tree KV-Cache Allocation").
 * For every layer l (pools at k_pages + l * layer_stride_elems, same for v)
 * and KV head, the k-th accepted node n_k (accept_nodes[b, k], k = 1..
 * accept_len[b]) moves from slot L_b + n_k to slot L_b + k; the root stays
 * at L_b. All sources are read before any destination is written.
 * new_prefix_lens int32 [B] = L_b + 1 + accept_len[b]; it must not overlap
 * prefix_lens (SPEC_E_INVAL), since other blocks still read L_b while it is
 * written. k_pages / v_pages are modified in place; other inputs are read only.
 * Invalid accept_len or accept_nodes (not increasing, >= max_T) leave that
 * sequence's cache untouched.
 * ------------------------------------------------------------------------- */
int32_t spec_kv_compact(void* k_pages, void* v_pages, const int32_t* page_table, const int32_t* prefix_lens,
                        const int32_t* accept_nodes, const int32_t* accept_len, int32_t B, int32_t max_T,
                        int32_t Hkv, int32_t d, int32_t page, int32_t max_pages, int32_t num_pages,
                        int32_t num_layers, int64_t layer_stride_elems, int32_t* new_prefix_lens, void* stream);

/* ----------------------------------------------------------------------------
 * Page-table pruning of rejected branches - tanhdev section 4 "Production
 * Failure Modes", Failure Mode 2 "KV Cache Memory Fragmentation" (the tree
 * cache prunes discarded branches without copying KV); lesty.tech section 6
 * "Paged Tree KV-Cache Allocation" (rejected candidates' physical blocks go
 * straight back to the free pool). No KV moves; only page_table changes.
 *
 * Sequence b's tree used logical slots L_b .. L_b + T_b - 1 (node i at L_b + i)
 * and verification accepted the path n_0 = 0 < n_1 < ... < n_a (accept_nodes,
 * accept_len). Afterwards the path reads, in order, at logical slots
 * L_b .. L_b + a, and new_prefix_lens[b] = L_b + 1 + a.
 *   mode SPEC_PRUNE_REMAP (page must be 1, a table of token slots): zero-copy.
 *     Entry L_b + k takes the old entry of slot L_b + n_k (k = 1..a), entries
 *     L_b + a + 1 .. L_b + T_b - 1 become -1, and the old entries of the
 *     T_b - 1 - a rejected nodes are returned in node order. Call it INSTEAD
 *     of spec_kv_compact.
 *   mode SPEC_PRUNE_TAIL (any page size): call it AFTER spec_kv_compact with
 *     the same accept_nodes / accept_len. The pages the tree touched whose
 *     slots all lie at or past L_b + 1 + a (logical pages ceil((L_b + 1 + a) /
 *     page) .. floor((L_b + T_b - 1) / page)) are returned in logical order and
 *     their entries become -1.
 * page_table      int32 [B, max_pages], rewritten in place
 * prefix_lens, T_b, accept_len int32 [B]; accept_nodes int32 [B, max_T]
 * freed           int32 [B, max_T] out: released entries (physical page ids,
 *                 token slots for REMAP), then -1 up to max_T
 * freed_count     int32 [B] out
 * new_prefix_lens int32 [B] out; it may be prefix_lens itself (in place)
 * status          uint32 [B] out or NULL: SPEC_STATUS_INVALID_PAGE when a
 *                 touched entry lies outside [0, num_pages) (cleared, never
 *                 returned); SPEC_STATUS_INVALID_LENGTH (T_b outside
 *                 [1, max_T], L_b < 0, or the tree past the table) or
 *                 SPEC_STATUS_INVALID_PATH: that sequence's table is left as
 *                 is, nothing is returned and new_prefix_lens[b] = max(L_b, 0).
 * Outputs must not overlap each other or the inputs (apart from the in-place
 * new_prefix_lens). Host checks: sizes, max_T <= 65, page, mode
 * (SPEC_E_INVAL / SPEC_E_UNSUPPORTED), null pointers.
 * ------------------------------------------------------------------------- */
#define SPEC_PRUNE_TAIL 0
#define SPEC_PRUNE_REMAP 1
int32_t spec_kv_prune(int32_t* page_table, const int32_t* prefix_lens, const int32_t* T_b, const int32_t* accept_nodes,
                      const int32_t* accept_len, int32_t B, int32_t max_T, int32_t page, int32_t max_pages,
                      int32_t num_pages, int32_t mode, int32_t* freed, int32_t* freed_count, int32_t* new_prefix_lens,
                      uint32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_TREE_H */
