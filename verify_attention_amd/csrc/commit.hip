// spec_commit_kv kernel for gfx950: the committed prefix's K/V after an
// accept, and the slots of the rejected suffix.
//
// The operation (see include/specattn.h): after a round the runtime releases
// the speculative suffix that was not accepted and advances each request by
// its commit length ("From DFlash to dLLM Self-Spec (4)", section 4.6, and
// the recursive dynamic compaction note of section 4.4.1). For a tree verify
// (the Tree sampler of "Unlocking Lossless Speedups in LLMs via Discrete
// Diffusion") the accepted nodes sit at scattered block positions L + p_k;
// they are moved to L + 1 + k so that the next round sees a contiguous
// causal prefix.
//
// One workgroup per (request, KV head): the accepted rows' K and V elements
// (D <= 128) move in rounds of 64 rows (128 at D 64): a round reads its rows
// into registers, a barrier separates the reads from the writes (a
// destination may be another row's source), then they are stored. The
// request's first workgroup lists the released slots.
#include "commit_rows.h"

namespace specattn {

template <typename T>
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(CommitArgs a) {
  const int b = blockIdx.x / a.Hkv, h = blockIdx.x - (blockIdx.x / a.Hkv) * a.Hkv;
  const int tid = threadIdx.x;
  const int P = a.P, B = a.B;
  const int32_t* tab = a.page_table + (size_t)b * a.max_pages;
  SPEC_COMMIT_ROWS(rows);
  __shared__ int s_path[kMaxCommitRows];
  __shared__ int s_err, s_bad;
  // the length and depth (every thread), the path entries into LDS, then
  // the path check: node p_k has depth k + 1, so k + 1 <= p_k < B, increasing
  const int L = a.seq_lens[b];
  int d = a.accept_len[b];
  int err = 0;
  if (L < 0 || (long long)L + B > (long long)a.max_pages * P) {
    err = kErrCapacity;
    d = -1;
  } else if (d < 0 || d > B - 1) {
    err = kErrTree;
    d = -1;
  }
  for (int k = tid; k < d; k += kCommitThreads)
    s_path[k] = a.path ? a.path[(size_t)b * B + k] : k + 1;
  if (tid == 0) s_err = s_bad = 0;
  __syncthreads();
  bool bad = false;
  if (a.path)
    for (int k = tid; k < d; k += kCommitThreads) {
      const int p = s_path[k];
      bad |= p < k + 1 || p >= B || (k > 0 && p <= s_path[k - 1]);
    }
  if (block_any(bad, &s_bad)) {
    err = kErrTree;
    d = -1;
  }
  bool bad_slot = commit_row_bases(rows, [&](int k) { return s_path[k]; }, tab, P, a.D, a.Hkv,
                                   a.num_pages, h, L, d);
  commit_move_rows<T>(rows, reinterpret_cast<T*>(a.k), reinterpret_cast<T*>(a.v), P, a.D, d);
  if (h == 0) bad_slot |= commit_freed(a.freed + (size_t)b * B, tab, P, B, a.num_pages, L, d);
  if (bad_slot) atomicOr(&s_err, kErrSlot);
  __syncthreads();
  if (tid == 0 && (err | s_err)) flag_error(a.err, err | s_err);
}

hipError_t launch_commit_kv(const CommitArgs& a, bool bf16, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(commit_kv_kernel<__bf16>, dim3(a.bs * a.Hkv), dim3(kCommitThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(commit_kv_kernel<float>, dim3(a.bs * a.Hkv), dim3(kCommitThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace specattn
