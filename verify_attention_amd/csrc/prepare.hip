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
