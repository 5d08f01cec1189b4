// spec_prepare_block kernel: one thread per (request, block position).
//
// Block token 0 is the previous round's verified id and tokens 1..B-1 are the
// mask token (draft pass) or the draft tokens (verify pass); positions run
// from the committed length; KV slots come from the page table ("From DFlash
// to dLLM Self-Spec (2)", sections 2.2.2, 2.2.4 and 2.3.5).
#include "kernels.h"

namespace specattn {

__global__ __launch_bounds__(256) void prepare_block_kernel(PrepareArgs a) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.bs * a.B) return;
  const int b = e / a.B;
  const int i = e - b * a.B;
  const int L = a.seq_lens[b];
  int32_t id;
  if (i == 0) id = a.verified_id[b];
  else if (a.draft) id = a.draft[(size_t)b * (a.B - 1) + (i - 1)];
  else id = a.mask_token_id;
  const long long pos = (long long)L + i;
  if (i == 0 && (L < 0 || (long long)L + a.B > (long long)a.max_pages * a.P))
    flag_error(a.err, kErrCapacity);
  int32_t slot = -1;
  if (pos >= 0) {
    const long long n = pos / a.P;
    if (n < a.max_pages) {
      const int32_t page = a.page_table[(size_t)b * a.max_pages + n];
      if (page >= 0 && page < a.num_pages) slot = page * a.P + (int32_t)(pos % a.P);
    }
  }
  if (slot < 0) flag_error(a.err, kErrSlot);
  a.block_ids[e] = id;
  a.positions[e] = (int32_t)pos;
  a.cache_loc[e] = slot;
}

hipError_t launch_prepare_block(const PrepareArgs& a, hipStream_t stream) {
  const int n = a.bs * a.B;
  hipLaunchKernelGGL(prepare_block_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace specattn

namespace specattn {

// spec_prepare_tree: one wave per request, lane n = node n (N <= 64). A
// node's depth is the length of its parent chain, found by pointer jumping
// over the parent links (six rounds reach 63 ancestors): each round a node
// adds the depth gathered so far by the node it points to and jumps to that
// node's pointer. A node whose parent is not an earlier node, or that
// descends from one, has no depth (position -1, SPEC_ERR_TREE).
__global__ __launch_bounds__(256) void prepare_tree_kernel(PrepareTreeArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.bs) return;  // whole waves leave together
  const int N = a.N;
  const bool live = lane < N;
  const int32_t* par = a.parent + (a.parent_per_req ? (size_t)b * N : 0);
  const int p = live && lane > 0 ? par[lane] : -1;
  const bool edge_ok = lane == 0 || (p >= 0 && p < lane);
  int depth = live && lane > 0 ? 1 : 0;
  int up = live && lane > 0 && edge_ok ? p : -1;
  int bad = live && !edge_ok ? 1 : 0;
#pragma unroll
  for (int it = 0; it < 6; ++it) {
    const int src = up >= 0 ? up : lane;
    const int d2 = __shfl(depth, src, 64);
    const int u2 = __shfl(up, src, 64);
    const int b2 = __shfl(bad, src, 64);
    if (up >= 0) {
      depth += d2;
      bad |= b2;
      up = u2;
    }
  }
  const int L = a.seq_lens[b];
  if (lane == 0 && (L < 0 || (long long)L + N > (long long)a.max_pages * a.P))
    flag_error(a.err, kErrCapacity);
  if (!live) return;
  int32_t id;
  if (lane == 0) id = a.verified_id[b];
  else if (a.node_tokens) id = a.node_tokens[(size_t)b * N + lane];
  else id = a.mask_token_id;
  const long long pos = (long long)L + lane;
  int32_t slot = -1;
  if (pos >= 0) {
    const long long n = pos / a.P;
    if (n < a.max_pages) {
      const int32_t page = a.page_table[(size_t)b * a.max_pages + n];
      if (page >= 0 && page < a.num_pages) slot = page * a.P + (int32_t)(pos % a.P);
    }
  }
  int err = slot < 0 ? kErrSlot : 0;
  if (bad) err |= kErrTree;
  if (err) flag_error(a.err, err);
  const size_t e = (size_t)b * N + lane;
  a.block_ids[e] = id;
  a.positions[e] = bad ? -1 : (int32_t)(L + depth);
  a.cache_loc[e] = slot;
}

// Blocks of more than 64 nodes: one workgroup of kMaxTreeNodes threads per
// request, thread n = node n, the same pointer jumping through LDS (nine
// rounds reach 511 ancestors).
__global__ __launch_bounds__(kMaxTreeNodes) void prepare_tree_wide_kernel(PrepareTreeArgs a) {
  __shared__ int s_depth[kMaxTreeNodes], s_up[kMaxTreeNodes], s_bad[kMaxTreeNodes];
  const int n = threadIdx.x, b = blockIdx.x, N = a.N;
  const bool live = n < N;
  const int32_t* par = a.parent + (a.parent_per_req ? (size_t)b * N : 0);
  const int p = live && n > 0 ? par[n] : -1;
  const bool edge_ok = n == 0 || (p >= 0 && p < n);
  int depth = live && n > 0 ? 1 : 0;
  int up = live && n > 0 && edge_ok ? p : -1;
  int bad = live && !edge_ok ? 1 : 0;
  for (int it = 0; it < 9; ++it) {
    s_depth[n] = depth;
    s_up[n] = up;
    s_bad[n] = bad;
    __syncthreads();
    if (up >= 0) {
      depth += s_depth[up];
      bad |= s_bad[up];
      up = s_up[up];
    }
    __syncthreads();
  }
  const int L = a.seq_lens[b];
  if (n == 0 && (L < 0 || (long long)L + N > (long long)a.max_pages * a.P))
    flag_error(a.err, kErrCapacity);
  if (!live) return;
  int32_t id;
  if (n == 0) id = a.verified_id[b];
  else if (a.node_tokens) id = a.node_tokens[(size_t)b * N + n];
  else id = a.mask_token_id;
  const long long pos = (long long)L + n;
  int32_t slot = -1;
  if (pos >= 0) {
    const long long pg = pos / a.P;
    if (pg < a.max_pages) {
      const int32_t page = a.page_table[(size_t)b * a.max_pages + pg];
      if (page >= 0 && page < a.num_pages) slot = page * a.P + (int32_t)(pos % a.P);
    }
  }
  int err = slot < 0 ? kErrSlot : 0;
  if (bad) err |= kErrTree;
  if (err) flag_error(a.err, err);
  const size_t e = (size_t)b * N + n;
  a.block_ids[e] = id;
  a.positions[e] = bad ? -1 : (int32_t)(L + depth);
  a.cache_loc[e] = slot;
}

hipError_t launch_prepare_tree(const PrepareTreeArgs& a, hipStream_t stream) {
  if (a.N > 64)
    hipLaunchKernelGGL(prepare_tree_wide_kernel, dim3(a.bs), dim3(kMaxTreeNodes), 0, stream, a);
  else
    hipLaunchKernelGGL(prepare_tree_kernel, dim3((a.bs + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace specattn
