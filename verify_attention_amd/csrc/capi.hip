// Host side of the C ABI declared in include/specattn.h: argument checks,
// split-KV / vocabulary-chunk planning, workspace layout and kernel launches.
// Every entry point only enqueues work on the caller's stream.
#include <climits>
#include <cmath>

#include "specattn.h"
#include "kernels.h"

#define SPEC_API extern "C" __attribute__((visibility("default")))

using namespace specattn;

namespace {

constexpr int kStepKeys = 32;
constexpr int kMaxSplits = 64;  // splits per unit (each keeps at least 8 stages when planned)
constexpr int kMaxChunks = 256;
constexpr int kMaxUnitRows = 128;   // query rows one workgroup holds (8 MFMA row tiles)
constexpr int kMaxQueryRows = 2048; // g * B: at most 16 row groups
constexpr int kMaxDevices = 64;
constexpr int kDefaultCUs = 256;    // MI355X; used only if the device cannot be queried

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ilog2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

// Compute units of the current device, queried once per device: the
// attention plan sizes its grids (one workgroup per CU for the balanced
// schedule, enough splits to cover the CUs otherwise) from it, so the
// workspace size and the call must be planned on the same device.
int device_cus() {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = kDefaultCUs;
  __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  return n;
}

struct AttnPlan {
  int M = 0, Mt = 0, RG = 1, units = 0, splits = 1, steps_per_split = 1;
  bool balanced = false;
  int grid = 0;
  size_t off_ml = 0, off_o = 0, ws_bytes = 0;
};

// Two schedules. Large batches (units x stages of the longest request at
// least kBalancedMinStages) use the balanced schedule: one workgroup per CU,
// each taking an equal share of all units' weight (stage pairs plus a fixed
// per-piece cost), so that lengths that differ widely do not leave CUs idle;
// units cut by a share boundary leave
// partial states in the workspace (two slots per workgroup). Smaller batches
// use one workgroup per (request, KV head, split): enough splits for one
// workgroup per CU when the batch has few units, every split keeping at least
// 8 stages of 32 keys.
constexpr long long kBalancedMinStages = 32768;
// A workgroup pays a fixed cost per piece it streams (the Q and page-table
// loads, the first DMA round trip, the merge of the two sets and the output
// stores: about 4 stage pairs of streaming). The balanced schedule weighs
// each unit as its stage pairs plus this many, so ranges that hold many
// short units get fewer pairs.
constexpr int kPieceCostPairs = 4;

// Query rows per KV head beyond kMaxUnitRows are cut into row groups of at
// most kMaxUnitRows (equal sizes, rounded up to the 16-row MFMA tile); each
// group streams the head's keys on its own. The balanced schedule keeps the
// RG workgroups of a group team on one XCD so that they share the keys in L2.
AttnPlan plan_attn(int bs, int B, int Hq, int Hkv, int D, int max_kv_len,
                   bool allow_balanced = true) {
  AttnPlan p;
  p.Mt = (Hq / Hkv) * B;
  p.RG = (p.Mt + kMaxUnitRows - 1) / kMaxUnitRows;
  p.M = p.RG == 1 ? p.Mt : (int)align_up((size_t)((p.Mt + p.RG - 1) / p.RG), 16);
  p.RG = (p.Mt + p.M - 1) / p.M;  // no empty group after the rounding
  p.units = bs * Hkv * p.RG;
  const int max_steps = std::max(1, (max_kv_len + kStepKeys - 1) / kStepKeys);
  const int cus = device_cus();
  p.balanced = allow_balanced && bs <= kMaxBalancedBatch &&
               (long long)p.units * max_steps >= kBalancedMinStages;
  if (p.balanced) {
    // G = teams x RG workgroups, a multiple of 8 * RG (one team per XCD slot)
    p.grid = p.RG == 1 ? cus : std::max(1, cus / (8 * p.RG)) * 8 * p.RG;
    const size_t slots = 2 * (size_t)p.grid;
    p.off_ml = 0;
    p.off_o = align_up(slots * p.M * 2 * sizeof(float), 256);
    p.ws_bytes = p.off_o + slots * p.M * D * sizeof(float);
    return p;
  }
  int splits = (cus + p.units - 1) / p.units;
  splits = std::min(splits, std::max(1, max_steps / 8));
  splits = std::max(1, std::min(splits, std::min(kMaxSplits, max_steps)));
  p.steps_per_split = (max_steps + splits - 1) / splits;
  p.splits = (max_steps + p.steps_per_split - 1) / p.steps_per_split;
  p.grid = p.units * p.splits;
  if (p.splits > 1) {
    p.off_ml = 0;
    p.off_o = align_up((size_t)p.units * p.splits * p.M * 2 * sizeof(float), 256);
    p.ws_bytes = p.off_o + (size_t)p.units * p.splits * p.M * D * sizeof(float);
  }
  return p;
}

struct AccPlan {
  int nchunk = 1, chunk = 0;
  size_t off_jbuf = 0, off_partial = 0, off_ids = 0, off_path = 0, ws_bytes = 0;
};

// Vocabulary chunks per request: about 2048 workgroups over the batch, chunks a
// multiple of 1024 entries (256 threads x one float4), at most 256 chunks.
AccPlan plan_accept(int bs, int K, int V, int greedy) {
  AccPlan p;
  if (greedy) {
    p.off_ids = 0;
    p.ws_bytes = (size_t)bs * (K + 1) * sizeof(int32_t);
    return p;
  }
  int want = std::max(1, std::min(kMaxChunks, (2048 + bs - 1) / bs));
  int chunk = (V + want - 1) / want;
  chunk = (int)align_up((size_t)chunk, 1024);
  p.chunk = chunk;
  p.nchunk = (V + chunk - 1) / chunk;
  p.off_jbuf = 0;
  p.off_partial = align_up((size_t)bs * sizeof(int32_t), 256);
  p.ws_bytes = p.off_partial + (size_t)bs * ((V + 255) / 256) * sizeof(double);
  return p;
}

// Tree verify: the same chunking, plus the accepted node ids [bs][N].
AccPlan plan_accept_tree(int bs, int N, int V) {
  AccPlan p = plan_accept(bs, N, V, 0);
  p.off_path = align_up(p.ws_bytes, 256);
  p.ws_bytes = p.off_path + (size_t)bs * N * sizeof(int32_t);
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_EHIP; }

}  // namespace

SPEC_API int spec_version(void) { return 100; }

SPEC_API const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument (null pointer, count or shape)";
    case SPEC_ENOTSUP: return "unsupported dtype, head dim or page size";
    case SPEC_ENOSPC: return "workspace too small";
    case SPEC_EHIP: return "HIP launch failed";
    case SPEC_ESCRATCH: return "sizes exceed the fixed scratch of the allocation-free call";
    default: return "unknown status";
  }
}

SPEC_API int spec_prepare_block(int bs, int B, int page_size, int max_pages, int num_pages,
                                int32_t mask_token_id, const int32_t* verified_id,
                                const int32_t* seq_lens, const int32_t* page_table,
                                const int32_t* draft_tokens, int32_t* block_ids,
                                int32_t* positions, int32_t* cache_loc, int32_t* err_flags,
                                void* stream) {
  if (bs <= 0 || B <= 0 || page_size <= 0 || max_pages <= 0 || num_pages <= 0) return SPEC_EINVAL;
  if ((long long)bs * B > INT_MAX) return SPEC_EINVAL;
  if (!verified_id || !seq_lens || !page_table || !block_ids || !positions || !cache_loc)
    return SPEC_EINVAL;
  PrepareArgs a;
  a.verified_id = verified_id;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.draft = B > 1 ? draft_tokens : nullptr;
  a.block_ids = block_ids;
  a.positions = positions;
  a.cache_loc = cache_loc;
  a.err = err_flags;
  a.bs = bs;
  a.B = B;
  a.P = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.mask_token_id = mask_token_id;
  return hip_status(launch_prepare_block(a, static_cast<hipStream_t>(stream)));
}

SPEC_API int spec_prepare_tree(int bs, int N, int page_size, int max_pages, int num_pages,
                               int32_t mask_token_id, const int32_t* verified_id,
                               const int32_t* seq_lens, const int32_t* page_table,
                               const int32_t* parent, int parent_per_request,
                               const int32_t* node_tokens, int32_t* block_ids,
                               int32_t* positions, int32_t* cache_loc, int32_t* err_flags,
                               void* stream) {
  if (bs <= 0 || N < 1 || N > kMaxTreeNodes || page_size <= 0 || max_pages <= 0 ||
      num_pages <= 0)
    return SPEC_EINVAL;
  if ((long long)bs * N > INT_MAX) return SPEC_EINVAL;
  if (!verified_id || !seq_lens || !page_table || !parent || !block_ids || !positions ||
      !cache_loc)
    return SPEC_EINVAL;
  PrepareTreeArgs a{};
  a.verified_id = verified_id;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.parent = parent;
  a.parent_per_req = parent_per_request ? 1 : 0;
  a.node_tokens = node_tokens;
  a.block_ids = block_ids;
  a.positions = positions;
  a.cache_loc = cache_loc;
  a.err = err_flags;
  a.bs = bs;
  a.N = N;
  a.P = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.mask_token_id = mask_token_id;
  return hip_status(launch_prepare_tree(a, static_cast<hipStream_t>(stream)));
}

SPEC_API size_t block_attn_workspace_bytes(int bs, int B, int Hq, int Hkv, int D, int max_kv_len) {
  if (bs <= 0 || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || max_kv_len <= 0) return 0;
  const size_t ws = plan_attn(bs, B, Hq, Hkv, D, max_kv_len).ws_bytes;
  // fp32 trees of more than 64 nodes at D = 128 take the split schedule (the
  // balanced kernel's LDS has no room for their mask words): cover both
  if (B <= 64 || D != 128) return ws;
  return std::max(ws, plan_attn(bs, B, Hq, Hkv, D, max_kv_len, false).ws_bytes);
}

namespace {

int attn_common(int mode, int n_causal, const int32_t* n_causal_per_req, const uint64_t* tree,
                int tree_per_request, int dtype, int bs, int B, int Hq, int Hkv, int D,
                int page_size, int max_pages, int num_pages, int max_kv_len, const void* q,
                const void* k_pool, const void* v_pool, const int32_t* page_table,
                const int32_t* seq_lens, float sm_scale, void* o, float* lse, void* workspace,
                size_t ws_bytes, int32_t* err_flags, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (D != 64 && D != 128) return SPEC_ENOTSUP;
  if (page_size != 16 && page_size != 32) return SPEC_ENOTSUP;
  if (bs <= 0 || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return SPEC_EINVAL;
  if ((long long)(Hq / Hkv) * B > kMaxQueryRows) return SPEC_EINVAL;
  if (max_pages <= 0 || num_pages <= 0 || max_kv_len <= 0) return SPEC_EINVAL;
  if ((long long)max_pages * page_size < B) return SPEC_EINVAL;
  if ((long long)max_pages * page_size > INT_MAX / 2) return SPEC_EINVAL;
  if (mode == SPEC_MIXED && !n_causal_per_req && (n_causal < 0 || n_causal > B)) return SPEC_EINVAL;
  if (mode == SPEC_TREE && (!tree || B > kMaxTreeNodes)) return SPEC_EINVAL;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !o) return SPEC_EINVAL;
  if (!(std::isfinite(sm_scale))) return SPEC_EINVAL;
  const int tree_words = mode == SPEC_TREE ? (B + 63) / 64 : 1;
  const bool split_only = tree_words > 1 && dtype == SPEC_F32 && D == 128;
  const AttnPlan plan = plan_attn(bs, B, Hq, Hkv, D, max_kv_len, !split_only);
  if (plan.ws_bytes > 0 && (!workspace || ws_bytes < plan.ws_bytes)) return SPEC_ENOSPC;

  AttnArgs a;
  a.q = q;
  a.k = k_pool;
  a.v = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.nc_per_req = mode == SPEC_MIXED ? n_causal_per_req : nullptr;
  a.tree = mode == SPEC_TREE ? tree : nullptr;
  a.tree_per_req = tree_per_request ? 1 : 0;
  a.tree_words = tree_words;
  a.o = o;
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  a.part_ml = plan.ws_bytes > 0 ? reinterpret_cast<float*>(ws + plan.off_ml) : nullptr;
  a.part_o = plan.ws_bytes > 0 ? reinterpret_cast<float*>(ws + plan.off_o) : nullptr;
  a.err = err_flags;
  a.bs = bs;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = Hq / Hkv;
  a.M = plan.M;
  a.Mt = plan.Mt;
  a.RG = plan.RG;
  a.Hv = Hkv * plan.RG;
  a.P = page_size;
  a.p_shift = ilog2_exact(page_size);
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.mode = mode;
  a.n_causal = mode == SPEC_MIXED ? n_causal : (mode == SPEC_CAUSAL ? B : 0);
  a.splits = plan.splits;
  a.steps_per_split = plan.steps_per_split;
  a.balanced = plan.balanced ? 1 : 0;
  a.G = plan.grid;
  a.piece_cost = kPieceCostPairs;
  const float scale = sm_scale == 0.0f ? 1.0f / std::sqrt((float)D) : sm_scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(launch_block_attn(a, dtype == SPEC_BF16, D, plan.grid,
                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

SPEC_API int block_attn(int mode, int n_causal, const int32_t* n_causal_per_req, int dtype, int bs,
                        int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                        int num_pages, int max_kv_len, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                        float sm_scale, void* o, float* lse, void* workspace, size_t ws_bytes,
                        int32_t* err_flags, void* stream) {
  if (mode < SPEC_BIDIR || mode > SPEC_MIXED) return SPEC_EINVAL;
  return attn_common(mode, n_causal, n_causal_per_req, nullptr, 0, dtype, bs, B, Hq, Hkv, D,
                     page_size, max_pages, num_pages, max_kv_len, q, k_pool, v_pool, page_table,
                     seq_lens, sm_scale, o, lse, workspace, ws_bytes, err_flags, stream);
}

SPEC_API int block_attn_tree(const uint64_t* tree_mask, int tree_per_request, int dtype, int bs,
                             int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                             int num_pages, int max_kv_len, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* page_table,
                             const int32_t* seq_lens, float sm_scale, void* o, float* lse,
                             void* workspace, size_t ws_bytes, int32_t* err_flags, void* stream) {
  return attn_common(SPEC_TREE, 0, nullptr, tree_mask, tree_per_request, dtype, bs, B, Hq, Hkv,
                     D, page_size, max_pages, num_pages, max_kv_len, q, k_pool, v_pool,
                     page_table, seq_lens, sm_scale, o, lse, workspace, ws_bytes, err_flags,
                     stream);
}

SPEC_API int spec_draft_argmax(int rows, int V, int dtype, const void* logits, int32_t* tokens,
                               void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (rows <= 0 || V <= 0 || !logits || !tokens) return SPEC_EINVAL;
  return hip_status(launch_argmax_rows(logits, dtype == SPEC_BF16, rows, V, tokens,
                                       static_cast<hipStream_t>(stream)));
}

namespace {

// The hand-off's segments: enough workgroups (about 1024) to keep every CU
// streaming, each segment a multiple of 8 entries (16-byte vectors stay
// aligned), at most 16 segments per row.
struct HandoffPlan {
  int S = 1, seg_len = 0;
  size_t off_i = 0, ws_bytes = 0;
};

HandoffPlan plan_handoff(int bs, int k, int V) {
  HandoffPlan p;
  const long long rows = (long long)bs * k;
  p.S = (int)std::max(1LL, std::min(16LL, (1024 + rows - 1) / rows));
  p.seg_len = (int)align_up((size_t)((V + p.S - 1) / p.S), 8);
  p.S = (V + p.seg_len - 1) / p.seg_len;
  const size_t parts = (size_t)rows * p.S;
  p.off_i = align_up(parts * sizeof(float), 256);
  p.ws_bytes = p.off_i + parts * sizeof(int32_t);
  return p;
}

}  // namespace

SPEC_API size_t spec_quadratic_handoff_workspace_bytes(int bs, int k, int V) {
  if (bs <= 0 || k < 1 || k > kMaxQuadK || V <= 0) return 0;
  return plan_handoff(bs, k, V).ws_bytes;
}

SPEC_API int spec_quadratic_handoff(int bs, int k, int V, int dtype, const void* logits,
                                    const int32_t* accept_len, const int32_t* bonus,
                                    int32_t mask_token_id, int32_t* next_draft,
                                    int32_t* next_block, void* workspace, size_t ws_bytes,
                                    int32_t* err_flags, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (bs <= 0 || k < 1 || k > kMaxQuadK || V <= 0) return SPEC_EINVAL;
  const int n = (k + 1) * (k + 1);
  if ((long long)bs * n > INT_MAX / 16) return SPEC_EINVAL;
  if (!logits || !accept_len || !next_draft || (next_block && !bonus)) return SPEC_EINVAL;
  const HandoffPlan plan = plan_handoff(bs, k, V);
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  char* ws = static_cast<char*>(workspace);
  HandoffArgs h{};
  h.logits = logits;
  h.accept_len = accept_len;
  h.bonus = bonus;
  h.next_draft = next_draft;
  h.next_block = next_block;
  h.err = err_flags;
  h.part_v = reinterpret_cast<float*>(ws);
  h.part_i = reinterpret_cast<int32_t*>(ws + plan.off_i);
  h.bs = bs;
  h.k = k;
  h.n = n;
  h.V = V;
  h.S = plan.S;
  h.seg_len = plan.seg_len;
  h.mask_token_id = mask_token_id;
  return hip_status(launch_quadratic_handoff(h, dtype == SPEC_BF16,
                                             static_cast<hipStream_t>(stream)));
}

SPEC_API size_t spec_accept_workspace_bytes(int bs, int K, int V, int greedy) {
  if (bs <= 0 || K < 1 || K > 63 || V <= 0) return 0;
  return plan_accept(bs, K, V, greedy).ws_bytes;
}

namespace {

// Checks shared by the linear accept entry points; fills the kernels'
// arguments (workspace pointers excepted) and the plan.
int accept_check_args(int bs, int K, int V, int greedy, const float* p, const float* q,
                        const int32_t* draft, const float* u, const int32_t* seq_lens,
                        int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                        int32_t* out_tokens, int32_t* new_seq_lens, int32_t* err_flags,
                        AcceptArgs* a, AccPlan* plan) {
  if (bs <= 0 || K < 1 || K > 63 || V <= 0) return SPEC_EINVAL;
  if ((long long)bs * (K + 1) > INT_MAX) return SPEC_EINVAL;
  if (!p || !draft || !seq_lens || !accept_len || !commit_len || !bonus || !out_tokens ||
      !new_seq_lens)
    return SPEC_EINVAL;
  if (!greedy && (!q || !u)) return SPEC_EINVAL;
  if (!greedy && V > kMaxAcceptVocab) return SPEC_ENOTSUP;
  *plan = plan_accept(bs, K, V, greedy);
  *a = AcceptArgs{};
  a->p = p;
  a->q = q;
  a->draft = draft;
  a->u = u;
  a->seq_lens = seq_lens;
  a->accept_len = accept_len;
  a->commit_len = commit_len;
  a->bonus = bonus;
  a->out_tokens = out_tokens;
  a->new_seq_lens = new_seq_lens;
  a->err = err_flags;
  a->bs = bs;
  a->K = K;
  a->V = V;
  a->nchunk = plan->nchunk;
  a->chunk = plan->chunk;
  return SPEC_OK;
}

// Launches the linear accept with its workspace at ws (plan.ws_bytes bytes).
int accept_launch(AcceptArgs a, const AccPlan& plan, char* ws, int greedy, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (greedy) {
    a.partial = nullptr;
    a.jbuf = nullptr;
    a.greedy_ids = reinterpret_cast<int32_t*>(ws + plan.off_ids);
    return hip_status(launch_greedy_accept(a, s));
  }
  a.jbuf = reinterpret_cast<int32_t*>(ws + plan.off_jbuf);
  a.partial = reinterpret_cast<double*>(ws + plan.off_partial);
  a.greedy_ids = nullptr;
  return hip_status(launch_accept(a, s));
}

}  // namespace

SPEC_API int spec_accept(int bs, int K, int V, int greedy, const float* p, const float* q,
                         const int32_t* draft, const float* u, const int32_t* seq_lens,
                         int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                         int32_t* out_tokens, int32_t* new_seq_lens, void* workspace,
                         size_t ws_bytes, int32_t* err_flags, void* stream) {
  AcceptArgs a;
  AccPlan plan;
  const int st = accept_check_args(bs, K, V, greedy, p, q, draft, u, seq_lens, accept_len,
                                     commit_len, bonus, out_tokens, new_seq_lens, err_flags, &a,
                                     &plan);
  if (st != SPEC_OK) return st;
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  return accept_launch(a, plan, static_cast<char*>(workspace), greedy, stream);
}

SPEC_API int spec_accept_prepare(int bs, int K, int V, int greedy, const float* p,
                                 const float* q, const int32_t* draft, const float* u,
                                 const int32_t* seq_lens, int32_t* accept_len,
                                 int32_t* commit_len, int32_t* bonus, int32_t* out_tokens,
                                 int32_t* new_seq_lens, int B_next, int page_size, int max_pages,
                                 int num_pages, int32_t mask_token_id, const int32_t* page_table,
                                 int32_t* block_ids, int32_t* positions, int32_t* cache_loc,
                                 void* workspace, size_t ws_bytes, int32_t* err_flags,
                                 void* stream) {
  AcceptArgs a;
  AccPlan plan;
  const int st = accept_check_args(bs, K, V, greedy, p, q, draft, u, seq_lens, accept_len,
                                     commit_len, bonus, out_tokens, new_seq_lens, err_flags, &a,
                                     &plan);
  if (st != SPEC_OK) return st;
  if (B_next <= 0 || page_size <= 0 || max_pages <= 0 || num_pages <= 0) return SPEC_EINVAL;
  if ((long long)bs * B_next > INT_MAX) return SPEC_EINVAL;
  if (!page_table || !block_ids || !positions || !cache_loc) return SPEC_EINVAL;
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  a.next_ids = block_ids;
  a.next_pos = positions;
  a.next_loc = cache_loc;
  a.next_tab = page_table;
  a.next_B = B_next;
  a.next_P = page_size;
  a.next_max_pages = max_pages;
  a.next_num_pages = num_pages;
  a.next_mask = mask_token_id;
  return accept_launch(a, plan, static_cast<char*>(workspace), greedy, stream);
}

namespace {

// spec_accept_quadratic's workspace: the accept's (accept lengths, sub-block
// masses) followed by the hand-off's segment maxima.
struct QuadPlan {
  AccPlan acc;
  HandoffPlan ho;
  size_t off_ho = 0, ws_bytes = 0;
};

QuadPlan plan_quadratic(int bs, int k, int V) {
  QuadPlan p;
  p.acc = plan_accept(bs, k, V, 0);
  p.ho = plan_handoff(bs, k, V);
  p.off_ho = align_up(p.acc.ws_bytes, 256);
  p.ws_bytes = p.off_ho + p.ho.ws_bytes;
  return p;
}

}  // namespace

SPEC_API size_t spec_accept_quadratic_workspace_bytes(int bs, int k, int V) {
  if (bs <= 0 || k < 1 || k > kMaxQuadK || V <= 0) return 0;
  return plan_quadratic(bs, k, V).ws_bytes;
}

SPEC_API int spec_accept_quadratic(int bs, int k, int V, const float* p, const float* q,
                                   const int32_t* draft, const float* u, const int32_t* seq_lens,
                                   int logits_dtype, const void* logits, int32_t mask_token_id,
                                   int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                                   int32_t* out_tokens, int32_t* new_seq_lens,
                                   int32_t* next_draft, int32_t* next_block,
                                   int32_t* next_positions, int32_t* next_cache_loc, int kv_dtype,
                                   int Hkv, int D, int page_size, int max_pages, int num_pages,
                                   const int32_t* page_table, void* k_pool, void* v_pool,
                                   int32_t* freed_loc, void* workspace, size_t ws_bytes,
                                   int32_t* err_flags, void* stream) {
  if (logits_dtype != SPEC_F32 && logits_dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (kv_dtype != SPEC_F32 && kv_dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (D != 64 && D != 128) return SPEC_ENOTSUP;
  if (page_size != 16 && page_size != 32) return SPEC_ENOTSUP;
  if (k < 1 || k > kMaxQuadK) return SPEC_EINVAL;
  AcceptArgs a;
  AccPlan acc_plan;
  const int st = accept_check_args(bs, k, V, 0, p, q, draft, u, seq_lens, accept_len, commit_len,
                                   bonus, out_tokens, new_seq_lens, err_flags, &a, &acc_plan);
  if (st != SPEC_OK) return st;
  const int n = (k + 1) * (k + 1);
  if ((long long)bs * n > INT_MAX / 16) return SPEC_EINVAL;
  if (Hkv <= 0 || max_pages <= 0 || num_pages <= 0) return SPEC_EINVAL;
  if ((long long)max_pages * page_size > INT_MAX / 2) return SPEC_EINVAL;
  if (!logits || !next_draft || !page_table || !k_pool || !v_pool || !freed_loc)
    return SPEC_EINVAL;
  if (!next_positions != !next_cache_loc) return SPEC_EINVAL;
  const QuadPlan plan = plan_quadratic(bs, k, V);
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  char* ws = static_cast<char*>(workspace);
  a.jbuf = reinterpret_cast<int32_t*>(ws + plan.acc.off_jbuf);
  a.partial = reinterpret_cast<double*>(ws + plan.acc.off_partial);
  a.quad_logits = logits;
  a.quad_next_draft = next_draft;
  a.quad_next_block = next_block;
  a.quad_part_v = reinterpret_cast<float*>(ws + plan.off_ho);
  a.quad_part_i = reinterpret_cast<int32_t*>(ws + plan.off_ho + plan.ho.off_i);
  a.quad_n = n;
  a.quad_S = plan.ho.S;
  a.quad_seg = plan.ho.seg_len;
  a.quad_mask = mask_token_id;
  a.next_pos = next_positions;
  a.next_loc = next_cache_loc;
  a.commit_k = k_pool;
  a.commit_v = v_pool;
  a.commit_tab = page_table;
  a.commit_freed = freed_loc;
  a.commit_bf16 = kv_dtype == SPEC_BF16 ? 1 : 0;
  a.commit_Hkv = Hkv;
  a.commit_D = D;
  a.commit_P = page_size;
  a.commit_max_pages = max_pages;
  a.commit_num_pages = num_pages;
  return hip_status(launch_accept_quadratic(a, logits_dtype == SPEC_BF16,
                                            static_cast<hipStream_t>(stream)));
}

SPEC_API size_t spec_accept_tree_workspace_bytes(int bs, int N, int V) {
  if (bs <= 0 || N < 1 || N > kMaxTreeNodes || V <= 0) return 0;
  return plan_accept_tree(bs, N, V).ws_bytes;
}

namespace {

int accept_tree_common(int bs, int N, int V, const int32_t* parent, const int32_t* token,
                       const float* p, const float* u, const int32_t* seq_lens,
                       int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                       int32_t* out_tokens, int32_t* path_nodes, int32_t* new_seq_lens,
                       void* workspace, size_t ws_bytes, int32_t* err_flags, void* stream,
                       const AcceptArgs* commit) {
  if (bs <= 0 || N < 1 || N > kMaxTreeNodes || V <= 0) return SPEC_EINVAL;
  if ((long long)bs * N > INT_MAX) return SPEC_EINVAL;
  if (!parent || !token || !p || !u || !seq_lens || !accept_len || !commit_len || !bonus ||
      !out_tokens || !path_nodes || !new_seq_lens)
    return SPEC_EINVAL;
  if (V > kMaxAcceptVocab) return SPEC_ENOTSUP;
  const AccPlan plan = plan_accept_tree(bs, N, V);
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  char* ws = static_cast<char*>(workspace);
  AcceptArgs a = commit ? *commit : AcceptArgs{};
  a.p = p;
  a.q = nullptr;
  a.draft = nullptr;
  a.u = u;
  a.seq_lens = seq_lens;
  a.accept_len = accept_len;
  a.commit_len = commit_len;
  a.bonus = bonus;
  a.out_tokens = out_tokens;
  a.new_seq_lens = new_seq_lens;
  a.err = err_flags;
  a.jbuf = reinterpret_cast<int32_t*>(ws + plan.off_jbuf);
  a.partial = reinterpret_cast<double*>(ws + plan.off_partial);
  a.greedy_ids = nullptr;
  a.parent = parent;
  a.token = token;
  a.path_nodes = path_nodes;
  a.pathbuf = reinterpret_cast<int32_t*>(ws + plan.off_path);
  a.bs = bs;
  a.K = N;
  a.V = V;
  a.nchunk = plan.nchunk;
  a.chunk = plan.chunk;
  return hip_status(launch_accept_tree(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

SPEC_API int spec_accept_tree(int bs, int N, int V, const int32_t* parent, const int32_t* token,
                              const float* p, const float* u, const int32_t* seq_lens,
                              int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                              int32_t* out_tokens, int32_t* path_nodes, int32_t* new_seq_lens,
                              void* workspace, size_t ws_bytes, int32_t* err_flags,
                              void* stream) {
  return accept_tree_common(bs, N, V, parent, token, p, u, seq_lens, accept_len, commit_len,
                            bonus, out_tokens, path_nodes, new_seq_lens, workspace, ws_bytes,
                            err_flags, stream, nullptr);
}

SPEC_API int spec_accept_tree_commit(int bs, int N, int V, const int32_t* parent,
                                     const int32_t* token, const float* p, const float* u,
                                     const int32_t* seq_lens, int32_t* accept_len,
                                     int32_t* commit_len, int32_t* bonus, int32_t* out_tokens,
                                     int32_t* path_nodes, int32_t* new_seq_lens, int dtype,
                                     int Hkv, int D, int page_size, int max_pages, int num_pages,
                                     const int32_t* page_table, void* k_pool, void* v_pool,
                                     int32_t* freed_loc, void* workspace, size_t ws_bytes,
                                     int32_t* err_flags, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (D != 64 && D != 128) return SPEC_ENOTSUP;
  if (page_size != 16 && page_size != 32) return SPEC_ENOTSUP;
  if (Hkv <= 0 || max_pages <= 0 || num_pages <= 0) return SPEC_EINVAL;
  if ((long long)max_pages * page_size > INT_MAX / 2) return SPEC_EINVAL;
  if (!page_table || !k_pool || !v_pool || !freed_loc) return SPEC_EINVAL;
  AcceptArgs c{};
  c.commit_k = k_pool;
  c.commit_v = v_pool;
  c.commit_tab = page_table;
  c.commit_freed = freed_loc;
  c.commit_bf16 = dtype == SPEC_BF16 ? 1 : 0;
  c.commit_Hkv = Hkv;
  c.commit_D = D;
  c.commit_P = page_size;
  c.commit_max_pages = max_pages;
  c.commit_num_pages = num_pages;
  return accept_tree_common(bs, N, V, parent, token, p, u, seq_lens, accept_len, commit_len,
                            bonus, out_tokens, path_nodes, new_seq_lens, workspace, ws_bytes,
                            err_flags, stream, &c);
}

// ------------------------------------------------ sampling parameters
namespace {

struct SampPlan {
  int ntiles = 0;
  size_t off_tmax = 0, off_ids = 0, off_probs = 0, off_n = 0, ws_bytes = 0;
};

// Workspace of rows processed rows: tile maxima, and (for the accept) the
// kept ids / probabilities / counts.
SampPlan plan_sampling(long long rows, int V, int top_k, bool kept_in_ws) {
  SampPlan p;
  p.ntiles = (V + 63) / 64;
  p.off_tmax = 0;
  p.ws_bytes = align_up((size_t)rows * p.ntiles * sizeof(float), 256);
  if (kept_in_ws) {  // rows padded to kMaxTopK entries
    (void)top_k;
    p.off_probs = p.ws_bytes;
    p.off_ids = align_up(p.off_probs + (size_t)rows * kMaxTopK * sizeof(double), 256);
    p.off_n = align_up(p.off_ids + (size_t)rows * kMaxTopK * sizeof(int32_t), 256);
    p.ws_bytes = align_up(p.off_n + (size_t)rows * sizeof(int32_t), 256);
  }
  return p;
}

bool sampling_params_ok(float temperature, int top_k, float top_p) {
  return std::isfinite(temperature) && temperature > 0.0f && top_k >= 1 && top_k <= kMaxTopK &&
         top_p > 0.0f && !std::isnan(top_p);
}

}  // namespace

SPEC_API size_t spec_sampling_filter_workspace_bytes(int rows, int V) {
  if (rows <= 0 || V <= 0) return 0;
  return plan_sampling(rows, V, 1, false).ws_bytes;
}

SPEC_API int spec_sampling_filter(int rows, int V, int dtype, const void* logits,
                                  float temperature, int top_k, float top_p, int32_t* kept_ids,
                                  double* kept_probs, int32_t* n_kept, void* workspace,
                                  size_t ws_bytes, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (rows <= 0 || V <= 0 || !logits || !kept_ids || !kept_probs || !n_kept) return SPEC_EINVAL;
  if (!sampling_params_ok(temperature, top_k, top_p)) return SPEC_EINVAL;
  if (V > kMaxSampVocab) return SPEC_ENOTSUP;
  const SampPlan plan = plan_sampling(rows, V, top_k, false);
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  SampArgs a{};
  a.x0 = logits;
  a.R1 = rows;
  a.V = V;
  a.ntiles = plan.ntiles;
  a.top_k = top_k;
  a.temperature = temperature;
  a.top_p = top_p;
  a.tmax = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.off_tmax);
  a.kept_ids = kept_ids;
  a.kept_probs = kept_probs;
  a.n_kept = n_kept;
  a.stride = top_k;
  return hip_status(launch_sampling_filter(a, dtype == SPEC_BF16, static_cast<hipStream_t>(stream)));
}

SPEC_API size_t spec_accept_logits_workspace_bytes(int bs, int K, int V, int top_k) {
  if (bs <= 0 || K < 1 || K > 63 || V <= 0 || top_k < 1 || top_k > kMaxTopK) return 0;
  return plan_sampling((long long)bs * (2 * K + 1), V, top_k, true).ws_bytes;
}

SPEC_API int spec_accept_logits(int bs, int K, int V, int dtype, float temperature, int top_k,
                                float top_p, const void* target_logits,
                                const void* draft_logits, const int32_t* draft, const float* u,
                                const int32_t* seq_lens, int32_t* accept_len,
                                int32_t* commit_len, int32_t* bonus, int32_t* out_tokens,
                                int32_t* new_seq_lens, void* workspace, size_t ws_bytes,
                                int32_t* err_flags, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (bs <= 0 || K < 1 || K > 63 || V <= 0) return SPEC_EINVAL;
  if ((long long)bs * (2 * K + 1) > INT_MAX / 64) return SPEC_EINVAL;
  if (!target_logits || !draft_logits || !draft || !u || !seq_lens || !accept_len ||
      !commit_len || !bonus || !out_tokens || !new_seq_lens)
    return SPEC_EINVAL;
  if (!sampling_params_ok(temperature, top_k, top_p)) return SPEC_EINVAL;
  if (V > kMaxSampVocab) return SPEC_ENOTSUP;
  const SampPlan plan = plan_sampling((long long)bs * (2 * K + 1), V, top_k, true);
  if (!workspace || ws_bytes < plan.ws_bytes) return SPEC_ENOSPC;
  char* ws = static_cast<char*>(workspace);
  SampArgs a{};
  a.x0 = target_logits;
  a.x1 = draft_logits;
  a.R1 = bs * (K + 1);
  a.R2 = bs * K;
  a.V = V;
  a.ntiles = plan.ntiles;
  a.top_k = top_k;
  a.temperature = temperature;
  a.top_p = top_p;
  a.tmax = reinterpret_cast<float*>(ws + plan.off_tmax);
  a.kept_ids = reinterpret_cast<int32_t*>(ws + plan.off_ids);
  a.kept_probs = reinterpret_cast<double*>(ws + plan.off_probs);
  a.n_kept = reinterpret_cast<int32_t*>(ws + plan.off_n);
  a.stride = kMaxTopK;
  a.bs = bs;
  a.K = K;
  a.draft = draft;
  a.u = u;
  a.seq_lens = seq_lens;
  a.accept_len = accept_len;
  a.commit_len = commit_len;
  a.bonus = bonus;
  a.out_tokens = out_tokens;
  a.new_seq_lens = new_seq_lens;
  a.err = err_flags;
  return hip_status(launch_accept_logits(a, dtype == SPEC_BF16, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ committed prefix
SPEC_API int spec_commit_kv(int dtype, int bs, int B, int Hkv, int D, int page_size,
                            int max_pages, int num_pages, const int32_t* seq_lens,
                            const int32_t* accept_len, const int32_t* path_nodes,
                            const int32_t* page_table, void* k_pool, void* v_pool,
                            int32_t* freed_loc, int32_t* err_flags, void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ENOTSUP;
  if (D != 64 && D != 128) return SPEC_ENOTSUP;
  if (page_size != 16 && page_size != 32) return SPEC_ENOTSUP;
  if (bs <= 0 || B < 1 || B > kMaxTreeNodes || Hkv <= 0 || max_pages <= 0 || num_pages <= 0)
    return SPEC_EINVAL;
  if ((long long)max_pages * page_size > INT_MAX / 2) return SPEC_EINVAL;
  if (!seq_lens || !accept_len || !page_table || !k_pool || !v_pool || !freed_loc)
    return SPEC_EINVAL;
  CommitArgs a{};
  a.k = k_pool;
  a.v = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.accept_len = accept_len;
  a.path = path_nodes;
  a.freed = freed_loc;
  a.err = err_flags;
  a.bs = bs;
  a.B = B;
  a.Hkv = Hkv;
  a.D = D;
  a.P = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  return hip_status(launch_commit_kv(a, dtype == SPEC_BF16, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ accept without a workspace
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the linear accept with its workspace in the library's fixed per-GPU
// scratch array (scratch.hip) instead of a caller's buffer.
SPEC_API int spec_accept_static(int bs, int K, int V, int greedy, const float* p, const float* q,
                                const int32_t* draft, const float* u, const int32_t* seq_lens,
                                int32_t* accept_len, int32_t* commit_len, int32_t* bonus,
                                int32_t* out_tokens, int32_t* new_seq_lens, int32_t* err_flags,
                                void* stream) {
  AcceptArgs a;
  AccPlan plan;
  const int st = accept_check_args(bs, K, V, greedy, p, q, draft, u, seq_lens, accept_len,
                                     commit_len, bonus, out_tokens, new_seq_lens, err_flags, &a,
                                     &plan);
  if (st != SPEC_OK) return st;
  if (plan.ws_bytes > SPEC_ACCEPT_STATIC_SCRATCH_BYTES) return SPEC_ESCRATCH;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (scratch_on_current_device(&ws, &ws_bytes) != hipSuccess) return SPEC_EHIP;
  if (ws_bytes < plan.ws_bytes) return SPEC_ESCRATCH;
  return accept_launch(a, plan, static_cast<char*>(ws), greedy, stream);
}
