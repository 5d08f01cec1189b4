// Internal interface between the C-ABI host layer (capi.hip) and the kernels.
#pragma once

#include "common.h"

namespace specattn {

// Token-tree blocks hold at most 512 nodes (8 uint64 mask words per row).
constexpr int kMaxTreeNodes = 512;
// Quadratic layouts of k drafts take (k + 1)^2 block rows.
constexpr int kMaxQuadK = 21;
static_assert((kMaxQuadK + 1) * (kMaxQuadK + 1) <= kMaxTreeNodes, "a quadratic block is a tree block");

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* nc_per_req;
  const uint64_t* tree;  // TREE mode: row masks over the block keys, [B][W] or [bs][B][W]
  int tree_words;        // W = ceil(B / 64) (1 for the other modes)
  void* o;
  float* lse;
  float* part_o;      // [slots][M][D] partial outputs (unnormalised): split or cut-unit pieces
  float* part_ml;     // [slots][M][2] partial (max, sum), log2 domain
  int32_t* err;
  // The Mt = g * B query rows of a KV head are cut into RG row groups of M
  // rows (the last may be short); a unit is (request, KV head, row group),
  // Hv = Hkv * RG units per request, unit = b * Hv + kvh * RG + rg.
  int bs, B, Hq, Hkv, g, M, Mt, RG, Hv;
  int P, p_shift, max_pages, num_pages;
  int mode, n_causal;
  int tree_per_req;
  int splits, steps_per_split;
  int balanced, G;   // balanced schedule: G persistent workgroups
  int piece_cost;    // balanced schedule: a unit's weight is its stage pairs + piece_cost
  float scale_log2;  // sm_scale * log2(e)
};

// Largest batch the balanced schedule handles (its prefix sums live in LDS).
constexpr int kMaxBalancedBatch = 2048;

hipError_t launch_block_attn(const AttnArgs& a, bool bf16, int D, int total_blocks,
                             hipStream_t stream);

struct PrepareArgs {
  const int32_t* verified_id;
  const int32_t* seq_lens;
  const int32_t* page_table;
  const int32_t* draft;
  int32_t* block_ids;
  int32_t* positions;
  int32_t* cache_loc;
  int32_t* err;
  int bs, B, P, max_pages, num_pages;
  int32_t mask_token_id;
};

hipError_t launch_prepare_block(const PrepareArgs& a, hipStream_t stream);

// A block given as parents in position order (a token tree, or the quadratic
// layout's position order): ids, positions L + depth(n), slots of L + n.
struct PrepareTreeArgs {
  const int32_t* verified_id;
  const int32_t* seq_lens;
  const int32_t* page_table;
  const int32_t* parent;       // [N] or [bs][N]
  const int32_t* node_tokens;  // [bs][N] or null (mask fill)
  int32_t* block_ids;
  int32_t* positions;
  int32_t* cache_loc;
  int32_t* err;
  int bs, N, P, max_pages, num_pages, parent_per_req;
  int32_t mask_token_id;
};

hipError_t launch_prepare_tree(const PrepareTreeArgs& a, hipStream_t stream);

// The quadratic layout's hand-off: the greedy tokens of the group after the
// last accepted spine token become the next round's drafts.
struct HandoffArgs {
  const void* logits;          // [bs][n][V], n = (k + 1)^2
  const int32_t* accept_len;   // [bs]
  const int32_t* bonus;        // [bs] (next block's root), may be null without next_block
  int32_t* next_draft;         // [bs][k]
  int32_t* next_block;         // [bs][n] or null
  int32_t* err;
  float* part_v;               // [bs][k][S] segment maxima (workspace)
  int32_t* part_i;             // [bs][k][S] their lowest indices
  int bs, k, n, V;
  int S, seg_len;              // segments per row and their length (a multiple of 8)
  int32_t mask_token_id;
};

hipError_t launch_quadratic_handoff(const HandoffArgs& a, bool bf16, hipStream_t stream);

hipError_t launch_argmax_rows(const void* x, bool bf16, int rows, int V, int32_t* out,
                              hipStream_t stream);

struct AcceptArgs {
  const float* p;
  const float* q;
  const int32_t* draft;
  const float* u;
  const int32_t* seq_lens;
  int32_t* accept_len;
  int32_t* commit_len;
  int32_t* bonus;
  int32_t* out_tokens;
  int32_t* new_seq_lens;
  int32_t* err;
  double* partial;     // [bs][ceil(V / 256)] residual mass per 256-entry sub-block
  int32_t* jbuf;       // [bs] accept length (| token-error flag) from the first kernel
  int32_t* greedy_ids; // [bs][K+1] row argmax (greedy mode)
  // tree verify (K = N nodes): parent, token [bs][N]; accepted node ids out
  const int32_t* parent;
  const int32_t* token;
  int32_t* path_nodes;  // [bs][N] output
  int32_t* pathbuf;     // [bs][N] accepted nodes passed between the two kernels
  // tree verify with the commit in the same call (commit_k null: no commit):
  // the accepted path's K/V rows moved, the rest of the block released
  void* commit_k;                 // k_pool [num_pages][Hkv][P][D]
  void* commit_v;                 // v_pool [num_pages][Hkv][D][P]
  const int32_t* commit_tab;      // page_table [bs][commit_max_pages]
  int32_t* commit_freed;          // [bs][N] released slots
  int commit_bf16, commit_Hkv, commit_D, commit_P, commit_max_pages, commit_num_pages;
  // linear accept with the next round's block (spec_accept_prepare; next_ids
  // null: none): the draft-pass block of B_next tokens at the new lengths
  int32_t* next_ids;              // [bs][next_B]
  int32_t* next_pos;              // [bs][next_B]
  int32_t* next_loc;              // [bs][next_B]
  const int32_t* next_tab;        // page_table [bs][next_max_pages]
  int next_B, next_P, next_max_pages, next_num_pages;
  int32_t next_mask;
  // quadratic round in one call (spec_accept_quadratic): the hand-off of the
  // next drafts from the layout's logits [bs][quad_n][V] and the spine commit
  // (the commit_* fields above, with quad_n rows per block)
  const void* quad_logits;
  int32_t* quad_next_draft;       // [bs][K]
  int32_t* quad_next_block;       // [bs][quad_n] or null
  float* quad_part_v;             // [bs][K][quad_S] segment maxima (workspace)
  int32_t* quad_part_i;           // [bs][K][quad_S] their lowest indices
  int quad_n, quad_S, quad_seg;
  int32_t quad_mask;
  int bs, K, V, nchunk, chunk;
};

// Largest vocabulary of the stochastic accept: its select pass holds each
// request's sub-block masses (256 entries each) in registers, 8 per thread.
constexpr int kMaxAcceptVocab = 8 * 256 * 256;

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);
hipError_t launch_accept_quadratic(const AcceptArgs& a, bool logits_bf16, hipStream_t stream);

// Sampling parameters (temperature, top-k, top-p) in front of the accept.
constexpr int kMaxSampVocab = 524288;  // tile maxima of a row: 32 per thread of 256
constexpr int kMaxTopK = 64;           // one wave holds a row's top list

struct SampArgs {
  const void* x0;       // rows [0, R1): [R1][V] logits (the target rows for the accept)
  const void* x1;       // rows [R1, R1 + R2): [R2][V] (the draft rows), may be null
  int R1, R2, V, ntiles, top_k;
  int stride;           // kept row stride: top_k (filter outputs) or kMaxTopK (accept workspace)
  float temperature, top_p;
  float* tmax;          // [R1 + R2][ntiles] tile maxima (workspace)
  int32_t* kept_ids;    // [R1 + R2][stride] kept ids in rank order, -1 padded
  double* kept_probs;   // [R1 + R2][stride] their probabilities, 0 padded
  int32_t* n_kept;      // [R1 + R2]
  // accept (bs requests, K drafts each)
  int bs, K;
  const int32_t* draft;
  const float* u;
  const int32_t* seq_lens;
  int32_t* accept_len;
  int32_t* commit_len;
  int32_t* bonus;
  int32_t* out_tokens;
  int32_t* new_seq_lens;
  int32_t* err;
};

// Committed-prefix K/V after an accept.
struct CommitArgs {
  void* k;                   // k_pool [num_pages][Hkv][P][D]
  void* v;                   // v_pool [num_pages][Hkv][D][P]
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* accept_len;
  const int32_t* path;       // [bs][B] accepted node ids, or null (the chain)
  int32_t* freed;            // [bs][B] released slots, -1 padded
  int32_t* err;
  int bs, B, Hkv, D, P, max_pages, num_pages;
};

hipError_t launch_commit_kv(const CommitArgs& a, bool bf16, hipStream_t stream);

// Device address and size of the current GPU's copy of the library's fixed
// scratch array (scratch.hip), for the allocation-free entry points.
hipError_t scratch_on_current_device(void** ptr, size_t* bytes);

hipError_t launch_sampling_filter(const SampArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_accept_logits(const SampArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_accept_tree(const AcceptArgs& a, hipStream_t stream);
hipError_t launch_greedy_accept(const AcceptArgs& a, hipStream_t stream);

}  // namespace specattn
