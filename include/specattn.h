/*
 * specattn.h -- C ABI of the block draft/verify attention + speculative accept
 * library for MI355X (gfx950).
 *
 * One decode round of block-diffusion self-speculative decoding runs, on one
 * HIP stream and without any host/device synchronisation:
 *
 *   spec_prepare_block  (draft pass)  -> block ids / positions / KV slots
 *                        (spec_prepare_tree for a tree or quadratic block)
 *   [caller writes the block's K/V at the slots]
 *   block_attn(SPEC_BIDIR)            -> draft-pass attention
 *   spec_draft_argmax                 -> greedy draft tokens
 *   spec_prepare_block  (verify pass, with the draft tokens)
 *   block_attn(SPEC_CAUSAL | SPEC_MIXED), or block_attn_tree for a token tree
 *   [caller produces target rows p]
 *   spec_accept (or spec_accept_tree) -> accepted prefix, bonus, new lengths
 *                        (spec_accept_prepare also prepares the next block)
 *   spec_commit_kv / spec_quadratic_handoff -> committed K/V, next drafts
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array argument is a DEVICE pointer to memory owned by the caller
 *   (the library never keeps a pointer past the call). Arrays are dense and
 *   row-major with the shapes given below.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *   only enqueue work on it: no allocation, no free, no host<->device copy, no
 *   synchronisation. Outputs are valid once the stream reaches that point.
 * - Return value: SPEC_OK when the work was queued; a negative status when a
 *   host-detectable argument error was found, in which case nothing was
 *   launched and no output was touched.
 * - `err_flags` (nullable, one int32 on the device): data errors found by the
 *   kernels are OR-ed into it (SPEC_ERR_* bits). The caller clears it and
 *   reads it whenever convenient; the library never reads it back.
 * - Token ids, positions, lengths and slots are int32.
 *
 * KV cache format (the pages leave it open; chosen for 16-byte MFMA operand
 * loads on both contractions):
 *   k_pool [num_pages][Hkv][P][D]   K rows token-major inside a page
 *   v_pool [num_pages][Hkv][D][P]   V columns dim-major inside a page
 *   page_table [bs][max_pages]      physical page of logical page n of request b
 *   The token at logical position n of request b lives in physical page
 *   page_table[b][n / P] at offset n % P; its slot id is page * P + n % P.
 */
#ifndef SPECATTN_H
#define SPECATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SPEC_OK 0
#define SPEC_EINVAL (-1)  /* null pointer, bad shape or count              */
#define SPEC_ENOTSUP (-2) /* dtype, head_dim or page size not supported    */
#define SPEC_ENOSPC (-3)  /* workspace smaller than the *_workspace_bytes  */
#define SPEC_EHIP (-4)    /* the HIP runtime refused the launch            */
#define SPEC_ESCRATCH (-5) /* sizes exceed an allocation-free call's fixed scratch */

/* err_flags bits, set by kernels */
#define SPEC_ERR_SLOT 1           /* a page-table entry the call needed is outside [0, num_pages) */
#define SPEC_ERR_CAPACITY 2       /* seq_len < 0 or seq_len + B > max_pages * P                 */
#define SPEC_ERR_TOKEN 4          /* a draft token id is outside [0, V)                          */
#define SPEC_ERR_ZERO_RESIDUAL 8  /* residual mass was zero; the draw used the target row        */
#define SPEC_ERR_TREE 16          /* a tree node's parent is not an earlier node (node ignored)  */

typedef enum { SPEC_BIDIR = 0, SPEC_CAUSAL = 1, SPEC_MIXED = 2, SPEC_TREE = 3 } spec_mode;
typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Library version (major * 10000 + minor * 100 + patch). */
int spec_version(void);

/* Text for a status code. Static string, never NULL. */
const char* spec_status_string(int status);

/*
 * spec_prepare_block -- the block of one round, for every request.
 *
 * Follows "From DFlash to dLLM Self-Spec (2): SGLang Spec V2", section 2.2.2
 * (block token 0 = the previous round's verified id, tokens 1..B-1 = the mask
 * token; positions and KV locations built in the same step) and section 2.2.4
 * (the verify pass feeds the draft tokens instead of the mask token). Slots
 * follow the request -> token map of section 2.3.5, whose over-allocation
 * rule (committed + 2 * block reserved) is what makes seq_len + B fit.
 *
 *   bs, B           requests and block length (B >= 1)
 *   page_size       P, tokens per page (> 0)
 *   max_pages       columns of page_table
 *   num_pages       pages in the pool (page ids must be < num_pages)
 *   mask_token_id   id written at block positions 1..B-1 on the draft pass
 *   verified_id     [bs]      token 0 of each block
 *   seq_lens        [bs]      committed length L_b (the block starts there)
 *   page_table      [bs, max_pages]
 *   draft_tokens    [bs, B-1] verify pass tokens, or NULL for the draft pass
 * Outputs:
 *   block_ids [bs, B], positions [bs, B] (= L_b + i),
 *   cache_loc [bs, B] (= page_table[b][pos / P] * P + pos % P, or -1 with
 *   SPEC_ERR_SLOT / SPEC_ERR_CAPACITY set when it cannot be formed).
 * Errors: SPEC_EINVAL for bs <= 0, B <= 0, P <= 0, max_pages <= 0,
 *   num_pages <= 0 or a NULL required pointer.
 */
int spec_prepare_block(int bs, int B, int page_size, int max_pages, int num_pages,
                       int32_t mask_token_id, const int32_t* verified_id,
                       const int32_t* seq_lens, const int32_t* page_table,
                       const int32_t* draft_tokens, int32_t* block_ids, int32_t* positions,
                       int32_t* cache_loc, int32_t* err_flags, void* stream);

/*
 * spec_prepare_tree -- the block of one round when its tokens form a tree
 * (or any layout given as parents in position order), for every request.
 *
 * Follows the block preparation of "From DFlash to dLLM Self-Spec (2): SGLang
 * Spec V2", section 2.2.2 (ids, positions and KV locations of the block in one
 * step), for a block laid out as the Tree sampler of "Unlocking Lossless
 * Speedups in LLMs via Discrete Diffusion" verifies it (method steps: top
 * candidates kept as a tree of prefixes) or as the quadratic layout of "From
 * DFlash to dLLM Self-Spec (4)", section 4.4.1 (MASK groups after every
 * speculative token). Node n sits at block row n (node 0, the root, is the
 * previous round's verified token):
 *   block_ids[b,0] = verified_id[b]; block_ids[b,n] = node_tokens[b,n] (or
 *   mask_token_id when node_tokens is NULL);
 *   positions[b,n] = L_b + depth(n), depth(0) = 0, depth(n) = depth(parent) + 1
 *   (a node continues its parent's sequence: siblings share a position);
 *   cache_loc[b,n] = the slot of position L_b + n (node n's K/V go to the
 *   n-th slot after the committed prefix, as block_attn_tree reads them).
 *
 *   bs, N           requests and block nodes (1..512)
 *   page_size, max_pages, num_pages, mask_token_id, verified_id, seq_lens,
 *   page_table      as spec_prepare_block
 *   parent          [N] (parent_per_request == 0) or [bs, N]; parent[0] is not
 *                   read; node n >= 1 needs 0 <= parent < n
 *   node_tokens     [bs, N] or NULL (node_tokens[b,0] is not read)
 * Outputs: block_ids, positions, cache_loc [bs, N]. A node whose parent is
 *   not an earlier node, or that descends from one, gets position -1 and sets
 *   SPEC_ERR_TREE; missing slots give -1 with SPEC_ERR_SLOT, and L_b + N past
 *   the page-table row sets SPEC_ERR_CAPACITY.
 * Errors: SPEC_EINVAL for bs <= 0, N outside 1..512, page_size, max_pages or
 *   num_pages <= 0, or a NULL required pointer.
 */
int spec_prepare_tree(int bs, int N, int page_size, int max_pages, int num_pages,
                      int32_t mask_token_id, const int32_t* verified_id, const int32_t* seq_lens,
                      const int32_t* page_table, const int32_t* parent, int parent_per_request,
                      const int32_t* node_tokens, int32_t* block_ids, int32_t* positions,
                      int32_t* cache_loc, int32_t* err_flags, void* stream);

/*
 * block_attn -- block-query attention over the paged KV cache.
 *
 * Follows "SGLang strengthens diffusion LLMs: LLaDA 2.0", section "Attention
 * Mask": the block's queries attend to the whole cached context (as chunked
 * prefill) and to the block's own K/V with a rectangular mask (block
 * diffusion, SPEC_BIDIR) or a triangular one (AR chunked prefill,
 * SPEC_CAUSAL); "From DFlash to dLLM Self-Spec (4)", sections 4.4-4.4.1
 * (bidirectional draft pass, causal verify pass of one model) and 4.3.1
 * (I-DLM layout: clean positions, then MASK positions) for SPEC_MIXED: block
 * rows i < n_c are causal, rows i >= n_c see the context and the whole block.
 *
 * For request b with L = seq_lens[b], block row i (query token at position
 * L + i) and query head h (KV head h / (Hq / Hkv)):
 *   o[b,i,h,:] = sum_j softmax_j(s_j) v_j over visible keys j in [0, L + B),
 *   s_j = sm_scale * <q[b,i,h,:], k_j>; key j < L is always visible; block key
 *   j = L + j' is visible iff BIDIR, or j' <= i (CAUSAL), or i >= n_c or
 *   j' <= i (MIXED). lse[b,i,h] = natural log of sum_j exp(s_j).
 * The block's own K/V must already be in the cache at positions L..L+B-1.
 *
 *   mode              SPEC_BIDIR / SPEC_CAUSAL / SPEC_MIXED
 *   n_causal          MIXED: clean rows per request (0..B) when
 *   n_causal_per_req  is NULL, else per-request counts [bs] (device)
 *   dtype             SPEC_BF16 (q, pools, o in bf16) or SPEC_F32
 *   bs, B, Hq, Hkv    Hq % Hkv == 0; g = Hq / Hkv; g * B <= 2048 (a KV
 *                     head's g * B query rows beyond 128 run as row groups
 *                     of at most 128 rows, each streaming the head's keys)
 *   D                 head dim: 64 or 128
 *   page_size         16 or 32
 *   max_pages, num_pages   page-table columns, pages in the pool
 *   max_kv_len        host upper bound of L_b + B over the batch; sizes the
 *                     split-KV plan only (a request longer than it is still
 *                     computed correctly, more slowly)
 *   q [bs, B, Hq, D]; k_pool, v_pool as in the file header; page_table;
 *   seq_lens [bs]; sm_scale (0 -> 1/sqrt(D))
 * Outputs: o [bs, B, Hq, D] (dtype), lse [bs, B, Hq] float (nullable).
 * Workspace: at least block_attn_workspace_bytes(...) bytes of device memory
 *   (0 when the plan needs no split-KV partials; then workspace may be NULL),
 *   16-byte aligned, contents irrelevant. It holds per-split partial outputs
 *   between the attention kernel and the merge kernel of the same call, so
 *   calls that share a workspace must be ordered (same stream, or synchronised).
 *   The plan (and so the size) depends on the compute-unit count of the
 *   current HIP device: size the workspace with the device current that the
 *   call will run on.
 * Errors: SPEC_EINVAL (bad counts, Hq % Hkv != 0, g * B > 2048, mode, n_causal
 *   outside [0, B], NULL pointers), SPEC_ENOTSUP (D, P, dtype), SPEC_ENOSPC.
 *   Kernels set SPEC_ERR_SLOT for a page id outside [0, num_pages) (physical
 *   page 0 is read in its place) and SPEC_ERR_CAPACITY for L_b < 0 or L_b + B
 *   > max_pages * P (the request is clamped to the table).
 */
size_t block_attn_workspace_bytes(int bs, int B, int Hq, int Hkv, int D, int max_kv_len);

int block_attn(int mode, int n_causal, const int32_t* n_causal_per_req, int dtype, int bs,
               int B, int Hq, int Hkv, int D, int page_size, int max_pages, int num_pages,
               int max_kv_len, const void* q, const void* k_pool, const void* v_pool,
               const int32_t* page_table, const int32_t* seq_lens, float sm_scale, void* o,
               float* lse, void* workspace, size_t ws_bytes, int32_t* err_flags, void* stream);

/*
 * block_attn_tree -- block_attn for a block that is a token tree.
 *
 * Follows the Tree sampler of "Unlocking Lossless Speedups in LLMs via
 * Discrete Diffusion" (method steps: candidate prefixes verified in parallel
 * with tree attention): the B block tokens are tree nodes, and a node must see
 * the context and its own root path only. Row i's visibility over the block
 * is a bitmask of W = ceil(B / 64) uint64 words: block key j' (0 <= j' < B)
 * is visible to block row i iff bit j' % 64 of word j' / 64 of row i is set,
 * the row being tree_mask[i * W ..] (shared tree) or tree_mask[(b * B + i) *
 * W ..] (one tree per request); context keys are always visible. Callers
 * set, for node i, the bits of node i and of its ancestors; a row whose mask
 * and context are both empty has no defined output.
 *
 *   tree_mask         uint64 row masks (device): [B, W] when tree_per_request
 *                     is 0, else [bs, B, W]; B <= 512 (W = 1 for B <= 64)
 *   other arguments, outputs, workspace (block_attn_workspace_bytes) and
 *   errors as for block_attn; SPEC_EINVAL also for tree_mask == NULL or
 *   B > 512.
 */
int block_attn_tree(const uint64_t* tree_mask, int tree_per_request, int dtype, int bs, int B,
                    int Hq, int Hkv, int D, int page_size, int max_pages, int num_pages,
                    int max_kv_len, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* page_table, const int32_t* seq_lens, float sm_scale, void* o,
                    float* lse, void* workspace, size_t ws_bytes, int32_t* err_flags,
                    void* stream);

/*
 * spec_draft_argmax -- greedy draft tokens from the draft pass's logits.
 *
 * Follows "From DFlash to dLLM Self-Spec (2)", section 2.2.3: the draft
 * tokens are the greedy choice of the target lm_head over the draft hidden
 * states at block positions 1..B-1 (the vocab projection itself is outside
 * this library). tokens[r] = smallest index among the maxima of logits[r, :].
 *
 *   rows, V   logits is [rows, V] (for a draft pass, rows = bs * (B - 1))
 *   dtype     SPEC_BF16 or SPEC_F32
 * Output: tokens [rows]. NaN entries never win; a row without a non-NaN
 * entry gives 0.
 * Errors: SPEC_EINVAL (rows <= 0, V <= 0, NULL), SPEC_ENOTSUP (dtype).
 */
int spec_draft_argmax(int rows, int V, int dtype, const void* logits, int32_t* tokens,
                      void* stream);

/*
 * spec_quadratic_handoff -- the next round's drafts from a quadratic block.
 *
 * Follows "From DFlash to dLLM Self-Spec (4)", section 4.4.1 (the paragraph
 * comparing recursive compaction with Quadratic Decoding: MASK tokens among
 * the speculative tokens keep supplying speculative tokens for the next step
 * after a speculative position fails) and "Unlocking Lossless Speedups in LLMs
 * via Discrete Diffusion", future work (2) (draft and verify in one forward).
 * The block of k drafts has n = (k + 1)^2 rows: the spine (root, s_1 .. s_k)
 * at rows i * (k + 1), and after spine token j the group G_j of k MASK rows
 * j * (k + 1) + 1 + m. When the accept keeps a = accept_len[b] drafts, the
 * correction takes the position after s_a and G_a's members propose the k
 * tokens after it:
 *   next_draft[b,m] = smallest index among the maxima of
 *   logits[b, a * (k + 1) + 1 + m, :] (NaN never wins), m = 0 .. k-1;
 *   next_block[b] (nullable) = the next round's quadratic block tokens:
 *   row 0 = bonus[b], row (m + 1) * (k + 1) = next_draft[b,m], every group
 *   row = mask_token_id.
 * Only the k rows of G_a are read per request.
 *
 *   bs, k, V        requests, drafts per block (1..21), vocabulary
 *   dtype           SPEC_BF16 or SPEC_F32 logits [bs, (k + 1)^2, V]
 *   accept_len [bs] as spec_accept returns it (0..k); bonus [bs] (needed only
 *   with next_block)
 * Outputs: next_draft [bs, k], next_block [bs, (k + 1)^2] or NULL. An
 *   accept_len outside 0..k gives drafts of -1 and sets SPEC_ERR_TREE.
 * Workspace: spec_quadratic_handoff_workspace_bytes(bs, k, V) bytes of device
 *   memory, contents irrelevant (per-segment maxima passed between the call's
 *   two kernels); calls sharing it must be ordered.
 * The accepted spine becomes contiguous with spec_commit_kv(B = (k + 1)^2,
 *   path_nodes[b, i] = (i + 1) * (k + 1)).
 * Errors: SPEC_EINVAL (sizes, NULL), SPEC_ENOTSUP (dtype), SPEC_ENOSPC.
 */
size_t spec_quadratic_handoff_workspace_bytes(int bs, int k, int V);

int spec_quadratic_handoff(int bs, int k, int V, int dtype, const void* logits,
                           const int32_t* accept_len, const int32_t* bonus,
                           int32_t mask_token_id, int32_t* next_draft, int32_t* next_block,
                           void* workspace, size_t ws_bytes, int32_t* err_flags, void* stream);

/*
 * spec_accept -- speculative accept / bonus epilogue.
 *
 * Follows "Unlocking Lossless Speedups in LLMs via Discrete Diffusion"
 * (prerequisite on speculative decoding and rejection sampling; the Psi-Spec
 * linear sampler keeps the longest accepted prefix and re-draws the rejected
 * slot from the residual, leaving the target distribution unchanged), "From
 * DFlash to dLLM Self-Spec (4)", section 4.3.1 (accept with probability
 * min(1, p/q); a reject emits a correction from the anchor side), and "From
 * DFlash to dLLM Self-Spec (2)", section 2.2.5 (outputs accept_len,
 * commit_len = accept_len + 1, bonus, out_tokens, new_seq_lens; the greedy rule).
 *
 * Per request b with K draft tokens d_0..d_{K-1} (block tokens 1..K):
 *   target row i of p scores block token i + 1; row K is the bonus row.
 *   test i: accept iff u[b,i] * q[b,i,d_i] < p[b,i,d_i] (exact, in double);
 *   accept_len = number of leading accepted tests (a token id outside [0, V)
 *   ends the prefix and sets SPEC_ERR_TOKEN);
 *   j = accept_len; r = max(p[b,j,:] - q[b,j,:], 0) if j < K else p[b,K,:]
 *   (double); bonus = smallest t with sum_{v<=t} r_v > u[b,K] * sum_v r_v;
 *   if sum r is zero the draw uses p[b,j,:] and sets SPEC_ERR_ZERO_RESIDUAL.
 *   commit_len = accept_len + 1; new_seq_lens = seq_lens + commit_len;
 *   out_tokens[b] = d_0..d_{j-1}, bonus, then -1 up to K + 1 entries.
 * greedy != 0: test i is d_i == argmax p[b,i,:] and bonus = argmax p[b,j,:]
 *   (lowest index on ties; p may hold logits); q and u are not read.
 *
 *   bs, K, V      requests, draft tokens per request (1..63), vocabulary
 *   p [bs, K+1, V] float, q [bs, K, V] float, draft [bs, K], u [bs, K+1] float
 *   in [0, 1), seq_lens [bs]
 * Outputs: accept_len, commit_len, bonus, new_seq_lens [bs]; out_tokens [bs, K+1].
 * Workspace: spec_accept_workspace_bytes(bs, K, V, greedy) bytes of device
 *   memory, 16-byte aligned, contents irrelevant (per-chunk residual masses
 *   and accept lengths passed between the call's two kernels). Calls that
 *   share a workspace must be ordered (same stream, or synchronised).
 * Errors: SPEC_EINVAL (bs <= 0, K outside 1..63, V <= 0, NULL), SPEC_ENOSPC,
 *   SPEC_ENOTSUP (greedy == 0 with V > 524288).
 */
size_t spec_accept_workspace_bytes(int bs, int K, int V, int greedy);

int spec_accept(int bs, int K, int V, int greedy, const float* p, const float* q,
                const int32_t* draft, const float* u, const int32_t* seq_lens,
                int32_t* accept_len, int32_t* commit_len, int32_t* bonus, int32_t* out_tokens,
                int32_t* new_seq_lens, void* workspace, size_t ws_bytes, int32_t* err_flags,
                void* stream);

/*
 * spec_accept_quadratic -- one quadratic round's tail in one call: the accept
 * of the k spine drafts, the hand-off of the next round's drafts and the
 * spine's commit.
 *
 * Every output, both pools and freed_loc equal those of the three calls in
 * order: spec_accept(bs, k, V, greedy = 0, p, q, draft, u, seq_lens, ...),
 * spec_quadratic_handoff(bs, k, V, logits_dtype, logits, accept_len, bonus,
 * mask_token_id, next_draft, next_block), and spec_commit_kv(kv_dtype, bs,
 * B = (k + 1)^2, Hkv, D, page_size, max_pages, num_pages, seq_lens,
 * accept_len, path_nodes[b, i] = (i + 1) * (k + 1), page_table, k_pool,
 * v_pool, freed_loc) ("From DFlash to dLLM Self-Spec (4)", section 4.4.1,
 * Quadratic Decoding and recursive compaction; section 4.6 for the released
 * slots). With next_positions / next_cache_loc, the call also prepares the
 * next round's block: they equal spec_prepare_tree's positions and cache_loc
 * for verified_id = bonus, seq_lens = new_seq_lens and the layout's position
 * order (row j' (k + 1) + m' at depth j' + m'), the same page table (so the
 * next round needs no preparation launch; next_block holds its tokens). Two
 * launches instead of five (six with the preparation): the hand-off's and the
 * commit's workgroups ride in the accept's two kernels (each finds the accept
 * length from the same gathered tests).
 *
 *   bs, k (1..21), V, p [bs, k+1, V], q [bs, k, V], draft [bs, k], u [bs, k+1],
 *   seq_lens: as spec_accept with K = k (stochastic form only)
 *   logits_dtype, logits [bs, (k + 1)^2, V], mask_token_id: as
 *   spec_quadratic_handoff
 *   kv_dtype, Hkv, D, page_size, max_pages, num_pages, page_table, k_pool,
 *   v_pool: as spec_commit_kv (pools updated in place)
 * Outputs: accept_len, commit_len, bonus, new_seq_lens [bs], out_tokens
 *   [bs, k+1], next_draft [bs, k], next_block [bs, (k + 1)^2] (nullable),
 *   next_positions, next_cache_loc [bs, (k + 1)^2] (both or neither; missing
 *   slots give -1 with SPEC_ERR_SLOT, a block past the table row
 *   SPEC_ERR_CAPACITY), freed_loc [bs, (k + 1)^2].
 * Workspace: spec_accept_quadratic_workspace_bytes(bs, k, V) bytes, contents
 *   irrelevant; calls sharing it must be ordered.
 * Errors: those of the three calls.
 */
size_t spec_accept_quadratic_workspace_bytes(int bs, int k, int V);

int spec_accept_quadratic(int bs, int k, int V, const float* p, const float* q,
                          const int32_t* draft, const float* u, const int32_t* seq_lens,
                          int logits_dtype, const void* logits, int32_t mask_token_id,
                          int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                          int32_t* out_tokens, int32_t* new_seq_lens, int32_t* next_draft,
                          int32_t* next_block, int32_t* next_positions, int32_t* next_cache_loc,
                          int kv_dtype, int Hkv, int D, int page_size,
                          int max_pages, int num_pages, const int32_t* page_table, void* k_pool,
                          void* v_pool, int32_t* freed_loc, void* workspace, size_t ws_bytes,
                          int32_t* err_flags, void* stream);

/*
 * spec_accept_prepare -- spec_accept, then the next round's block in the same
 * call.
 *
 * The accept outputs are the next round's inputs ("From DFlash to dLLM
 * Self-Spec (2)", section 2.2.5: the bonus becomes the next verified id and
 * the new lengths the next committed lengths; section 2.2.2: the next round
 * starts by preparing its block from them). Every output equals that of
 * spec_accept followed by spec_prepare_block(bs, B_next, page_size,
 * max_pages, num_pages, mask_token_id, verified_id = bonus, seq_lens =
 * new_seq_lens, page_table, draft_tokens = NULL): the next draft pass's block
 * (token 0 = the bonus, the rest the mask token), its positions and slots.
 * One launch fewer: the accept's last kernel writes the block.
 *
 *   the accept's arguments and outputs: as spec_accept (same workspace)
 *   B_next, page_size, max_pages, num_pages, mask_token_id, page_table: as
 *   spec_prepare_block
 * Outputs also: block_ids, positions, cache_loc [bs, B_next], with the data
 *   errors spec_prepare_block reports.
 * Errors: those of both calls.
 */
int spec_accept_prepare(int bs, int K, int V, int greedy, const float* p, const float* q,
                        const int32_t* draft, const float* u, const int32_t* seq_lens,
                        int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                        int32_t* out_tokens, int32_t* new_seq_lens, int B_next, int page_size,
                        int max_pages, int num_pages, int32_t mask_token_id,
                        const int32_t* page_table, int32_t* block_ids, int32_t* positions,
                        int32_t* cache_loc, void* workspace, size_t ws_bytes, int32_t* err_flags,
                        void* stream);

/*
 * spec_accept_static -- spec_accept without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and outputs as spec_accept, bit for bit, with the workspace
 * taken from a fixed device array the library owns, one copy per GPU, kept
 * until the process ends. The call allocates nothing and frees nothing.
 *
 *   arguments and outputs: as spec_accept, without workspace / ws_bytes
 * Limit: spec_accept_workspace_bytes(bs, K, V, greedy) must not exceed
 *   SPEC_ACCEPT_STATIC_SCRATCH_BYTES (4 MiB: for V = 151936 about 880
 *   requests of the stochastic accept); larger calls return SPEC_ESCRATCH and
 *   launch nothing.
 * Concurrency: every call on one GPU uses that GPU's one array, so calls that
 *   may run at the same time on one GPU (unordered streams) race on it and
 *   must be ordered by the caller. Its contents persist between calls; no
 *   call depends on them.
 * Errors: those of spec_accept (SPEC_ENOSPC excepted), SPEC_ESCRATCH, and
 *   SPEC_EHIP when the array's device address cannot be obtained.
 */
#define SPEC_ACCEPT_STATIC_SCRATCH_BYTES (4u << 20)

int spec_accept_static(int bs, int K, int V, int greedy, const float* p, const float* q,
                       const int32_t* draft, const float* u, const int32_t* seq_lens,
                       int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                       int32_t* out_tokens, int32_t* new_seq_lens, int32_t* err_flags,
                       void* stream);

/*
 * spec_accept_tree -- speculative accept for a token tree (tree verify).
 *
 * Follows the Tree sampler of "Unlocking Lossless Speedups in LLMs via
 * Discrete Diffusion" (method steps: top candidates per position kept as a
 * tree, verified in parallel, lossless through rejection sampling). Its
 * candidates are deterministic, so every child is a draft whose draft
 * distribution is one-hot; the rejection rule for such drafts, applied from
 * the root down, is:
 *   at node x (start: the root, node 0), try the children c of x in
 *   increasing node order; with T the target mass p[b,x,.] of the distinct
 *   tokens already tried at x, child c is accepted iff
 *   u[b,c] * (1 - T) < p[b,x,token[c]] (double); the first accepted child
 *   becomes the next node. A child repeating a tried token is never accepted;
 *   a token id outside [0, V) is a reject and sets SPEC_ERR_TOKEN.
 *   When no child of x is accepted (or x is a leaf), the bonus is the smallest
 *   t with C_t > u[b,0] * S, where C is the running sum (double, vocabulary
 *   order) of r = p[b,x,.] with the tried tokens set to 0 and S = sum r (S <= 0:
 *   drawn from p[b,x,.] itself, SPEC_ERR_ZERO_RESIDUAL).
 * Every emitted token is then distributed as the target's next-token
 * distribution at its position, as for the linear rule.
 *
 *   bs, N, V          requests, tree nodes per request (1..512), vocabulary
 *                     (<= 524288)
 *   parent [bs, N]    parent node; parent[b,0] = -1 (the root is the last
 *                     committed token); a node n >= 1 needs 0 <= parent < n
 *                     (else it is ignored and SPEC_ERR_TREE is set)
 *   token [bs, N]     candidate token of node n (token[b,0] is not read)
 *   p [bs, N, V]      float target rows: row n is the distribution of the
 *                     token that follows node n's root path
 *   u [bs, N]         float uniforms in [0, 1): u[b,c] drives child c's test,
 *                     u[b,0] the bonus draw
 *   seq_lens [bs]
 * Outputs: accept_len [bs] (accepted nodes), path_nodes [bs, N] (their ids in
 *   order, then -1), out_tokens [bs, N] (their tokens, the bonus, then -1),
 *   bonus, commit_len = accept_len + 1, new_seq_lens = seq_lens + commit_len.
 * Workspace: spec_accept_tree_workspace_bytes(bs, N, V) bytes, 16-byte
 *   aligned, contents irrelevant; calls sharing it must be ordered.
 * Errors: SPEC_EINVAL (bs <= 0, N outside 1..512, V <= 0, NULL), SPEC_ENOSPC,
 *   SPEC_ENOTSUP (V > 524288).
 */
size_t spec_accept_tree_workspace_bytes(int bs, int N, int V);

int spec_accept_tree(int bs, int N, int V, const int32_t* parent, const int32_t* token,
                     const float* p, const float* u, const int32_t* seq_lens,
                     int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                     int32_t* out_tokens, int32_t* path_nodes, int32_t* new_seq_lens,
                     void* workspace, size_t ws_bytes, int32_t* err_flags, void* stream);

/*
 * spec_sampling_filter -- temperature / top-k / top-p processing of logits rows.
 *
 * Follows the evaluation protocol of "Unlocking Lossless Speedups in LLMs via
 * Discrete Diffusion" (reproduction section: sampling with temperature, top-p
 * and top-k) and the I-DLM verify of "From DFlash to dLLM Self-Spec (4)",
 * section 4.3.1 (the verify consumes logits through softmax / top-k). The
 * pages do not fix the order or the boundary rules; this library takes:
 *   1. rank the tokens of a row by logit, largest first; equal logits (-0 and
 *      +0 are equal) rank the lower index first; NaN logits are never kept;
 *   2. keep the first top_k ranks;
 *   3. e_r = exp((l_r - l_max) / temperature) in double over the kept ranks;
 *   4. top_p < 1: keep rank r iff (sum_{s<r} e_s) / (sum_s e_s) < top_p, the
 *      shortest rank prefix whose mass reaches top_p; top_p >= 1 keeps all;
 *   5. prob_r = e_r / sum_{kept} e.
 *
 *   rows, V        logits is [rows, V] (V <= 524288), dtype SPEC_F32 / SPEC_BF16
 *   temperature    > 0 and finite; top_k 1..64; top_p > 0 (>= 1: no top-p);
 *                  both are used at their float32 values, widened to double
 * Outputs: kept_ids [rows, top_k] int32 in rank order then -1, kept_probs
 *   [rows, top_k] double (0 past the kept ones), n_kept [rows]. A row without a
 *   finite logit among its top ranks gives n_kept = 0.
 * Workspace: spec_sampling_filter_workspace_bytes(rows, V) bytes (one float
 *   per 64 logits), contents irrelevant; calls sharing it must be ordered.
 * Errors: SPEC_EINVAL (rows <= 0, V <= 0, NULL, parameters out of range),
 *   SPEC_ENOTSUP (dtype, V > 524288), SPEC_ENOSPC.
 */
size_t spec_sampling_filter_workspace_bytes(int rows, int V);

int spec_sampling_filter(int rows, int V, int dtype, const void* logits, float temperature,
                         int top_k, float top_p, int32_t* kept_ids, double* kept_probs,
                         int32_t* n_kept, void* workspace, size_t ws_bytes, void* stream);

/*
 * spec_accept_logits -- speculative accept on logits under sampling parameters.
 *
 * The lossless rule (as spec_accept, from "Unlocking Lossless Speedups in
 * LLMs via Discrete Diffusion" and section 4.3.1 of "From DFlash to dLLM
 * Self-Spec (4)") applied to processed distributions: every target row and
 * every draft row is processed as spec_sampling_filter describes, with the
 * same parameters, and then
 *   test i: accept iff u[b,i] * q_i(d_i) < p_i(d_i) (double; a token outside
 *   the kept set has probability 0; an id outside [0, V) is a reject and sets
 *   SPEC_ERR_TOKEN); j = accept_len; r = max(p_j - q_j, 0) over p_j's kept
 *   set (p_K's kept set when j = K); bonus = smallest kept t (vocabulary
 *   order) whose running sum of r exceeds u[b,K] * sum r; a zero residual
 *   draws from p_j and sets SPEC_ERR_ZERO_RESIDUAL. The outputs are those of
 *   spec_accept. The emitted tokens are distributed as the processed target.
 *
 *   bs, K, V            requests, draft tokens (1..63), vocabulary (<= 524288)
 *   dtype               SPEC_F32 or SPEC_BF16 for both logits tensors
 *   temperature, top_k, top_p   as spec_sampling_filter
 *   target_logits [bs, K+1, V]  row i scores block token i + 1 (row K: bonus)
 *   draft_logits  [bs, K, V]    the drafter's logits of draft token i
 *   draft [bs, K], u [bs, K+1] float in [0, 1), seq_lens [bs]
 * Outputs: accept_len, commit_len, bonus, new_seq_lens [bs]; out_tokens [bs, K+1].
 * Workspace: spec_accept_logits_workspace_bytes(bs, K, V, top_k) bytes,
 *   16-byte aligned, contents irrelevant; calls sharing it must be ordered.
 * Errors: SPEC_EINVAL (sizes, NULL, parameters), SPEC_ENOTSUP (dtype,
 *   V > 524288), SPEC_ENOSPC.
 */
size_t spec_accept_logits_workspace_bytes(int bs, int K, int V, int top_k);

int spec_accept_logits(int bs, int K, int V, int dtype, float temperature, int top_k, float top_p,
                       const void* target_logits, const void* draft_logits, const int32_t* draft,
                       const float* u, const int32_t* seq_lens, int32_t* accept_len,
                       int32_t* commit_len, int32_t* bonus, int32_t* out_tokens,
                       int32_t* new_seq_lens, void* workspace, size_t ws_bytes,
                       int32_t* err_flags, void* stream);

/*
 * spec_commit_kv -- the committed prefix's K/V after an accept, and the
 * released slots of the rejected suffix.
 *
 * Follows "From DFlash to dLLM Self-Spec (4)", section 4.6 (after a round the
 * runtime releases the KV of the speculative suffix that was not accepted and
 * advances the request by its commit length) and the recursive dynamic
 * compaction note of section 4.4.1 (the committable path is fixed inside the
 * candidate block, then the rejected suffix is released); for trees, the
 * Tree sampler of "Unlocking Lossless Speedups in LLMs via Discrete
 * Diffusion". The block of request b occupies positions L .. L + B - 1
 * (L = seq_lens[b]) with node / block row n at L + n (node 0: the root, the
 * last committed token). With d = accept_len[b] and path p_1 .. p_d
 * (path_nodes[b, 0 .. d-1], as spec_accept_tree returns them):
 *   position L + k receives the K and V of position L + p_k (k = 1 .. d,
 *   every KV head; all sources are read before any destination is written);
 *   path_nodes == NULL is the chain p_k = k (a linear verify: nothing moves);
 *   freed_loc[b] = slots of positions L + d + 1 .. L + B - 1, then -1.
 * The bonus token is not written: it becomes the next round's first block
 * token at position L + d + 1 = new_seq_lens[b].
 *
 *   dtype SPEC_F32 / SPEC_BF16; D 64 or 128; page_size 16 or 32; B 1..512
 *   k_pool, v_pool, page_table as block_attn (updated in place)
 * Data errors (flagged, the request is left unchanged): L + B past the page
 *   table (SPEC_ERR_CAPACITY), d outside 0..B-1 or a path that is not
 *   increasing with k + 1 <= p_k < B (SPEC_ERR_TREE), a page id out of range
 *   (SPEC_ERR_SLOT: that row is skipped).
 * Errors: SPEC_EINVAL (sizes, NULL), SPEC_ENOTSUP (dtype, D, page_size).
 */
int spec_commit_kv(int dtype, int bs, int B, int Hkv, int D, int page_size, int max_pages,
                   int num_pages, const int32_t* seq_lens, const int32_t* accept_len,
                   const int32_t* path_nodes, const int32_t* page_table, void* k_pool,
                   void* v_pool, int32_t* freed_loc, int32_t* err_flags, void* stream);

/*
 * spec_accept_tree_commit -- spec_accept_tree and spec_commit_kv in one call.
 *
 * The tree accept (spec_accept_tree) followed by the commit of its accepted
 * path (spec_commit_kv with B = N, accept_len and path_nodes as the accept
 * returns them): every output, both pools and freed_loc are exactly those of
 * the two calls in order. One launch fewer: the path is fixed by the walk of
 * the accept's first kernel (the bonus draw of the second does not change
 * it), so the first kernel also moves the rows and lists the released slots.
 *
 *   bs, N, V, parent, token, p, u, seq_lens and the outputs: as
 *   spec_accept_tree (same workspace: spec_accept_tree_workspace_bytes)
 *   dtype, Hkv, D, page_size, max_pages, num_pages, page_table, k_pool,
 *   v_pool, freed_loc [bs, N]: as spec_commit_kv with B = N
 * Data errors: those of both calls (a request whose block lies past its page
 *   table keeps its rows in place and releases nothing).
 * Errors: those of both calls.
 */
int spec_accept_tree_commit(int bs, int N, int V, const int32_t* parent, const int32_t* token,
                            const float* p, const float* u, const int32_t* seq_lens,
                            int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                            int32_t* out_tokens, int32_t* path_nodes, int32_t* new_seq_lens,
                            int dtype, int Hkv, int D, int page_size, int max_pages,
                            int num_pages, const int32_t* page_table, void* k_pool, void* v_pool,
                            int32_t* freed_loc, void* workspace, size_t ws_bytes,
                            int32_t* err_flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECATTN_H */
