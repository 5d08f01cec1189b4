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
// One workgroup per (request, KV head): every accepted row's K and V
// elements (at most 63 rows of D <= 128) are read into registers, a barrier
// separates the reads from the writes (a destination may be another row's
// source), then they are stored. The request's first workgroup lists the
// released slots.
#include "kernels.h"

namespace specattn {

constexpr int kCommitThreads = 256;
constexpr int kCommitPer = 32;  // elements per thread: 63 rows x 128 dims fit
static_assert(kCommitThreads * kCommitPer >= 63 * 128, "one round of loads");

template <typename T>
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(CommitArgs a) {
  const int b = blockIdx.x / a.Hkv, h = blockIdx.x - (blockIdx.x / a.Hkv) * a.Hkv;
  const int tid = threadIdx.x;
  const int P = a.P, D = a.D, B = a.B, Hkv = a.Hkv;
  const int32_t* tab = a.page_table + (size_t)b * a.max_pages;
  __shared__ long long s_src[64], s_dst[64];  // element offsets of K rows (-1: skipped)
  __shared__ long long s_vsrc[64], s_vdst[64];
  __shared__ int s_d, s_err;
  // wave 0, lane k = accepted row k: the length, the depth and every path
  // entry are loaded at once, the path is checked by a ballot, then each lane
  // looks up its row's pages (two dependent loads in all)
  if (tid < 64) {
    const int L = a.seq_lens[b];
    int d = a.accept_len[b];
    const int p = a.path ? (tid < B ? a.path[(size_t)b * B + tid] : 0) : tid + 1;
    int err = 0;
    if (L < 0 || (long long)L + B > (long long)a.max_pages * P) {
      err = kErrCapacity;
      d = -1;
    } else if (d < 0 || d > B - 1) {
      err = kErrTree;
      d = -1;
    } else if (a.path) {
      // node p_k has depth k + 1: k + 1 <= p_k < B, increasing
      const int prev = __shfl_up(p, 1, 64);
      const bool bad = tid < d && (p < tid + 1 || p >= B || (tid > 0 && p <= prev));
      if (__builtin_amdgcn_ballot_w64(bad)) {
        err = kErrTree;
        d = -1;
      }
    }
    // row bases: K element (page, h, off, i) at ((page * Hkv + h) * P + off) * D + i,
    // V element (page, h, i, off) at ((page * Hkv + h) * D + i) * P + off
    long long ks = -1, kd = -1, vs = -1, vd = -1;
    bool bad_slot = false;
    if (tid < d) {
      const int src = L + p;
      const int dst = L + 1 + tid;
      const int ps = tab[src / P], pd = tab[dst / P];
      const bool ok = (unsigned)ps < (unsigned)a.num_pages && (unsigned)pd < (unsigned)a.num_pages;
      bad_slot = !ok;
      if (ok && src != dst) {
        ks = (((long long)ps * Hkv + h) * P + src % P) * D;
        kd = (((long long)pd * Hkv + h) * P + dst % P) * D;
        vs = ((long long)ps * Hkv + h) * D * P + src % P;
        vd = ((long long)pd * Hkv + h) * D * P + dst % P;
      }
    }
    if (__builtin_amdgcn_ballot_w64(bad_slot)) err |= kErrSlot;
    s_src[tid] = ks;
    s_dst[tid] = kd;
    s_vsrc[tid] = vs;
    s_vdst[tid] = vd;
    if (tid == 0) {
      s_d = d;
      s_err = err;
    }
  }
  __syncthreads();
  const int d = s_d;
  const int L = a.seq_lens[b];
  __syncthreads();
  T* K = reinterpret_cast<T*>(a.k);
  T* V = reinterpret_cast<T*>(a.v);
  T kr[kCommitPer], vr[kCommitPer];
#pragma unroll
  for (int i = 0; i < kCommitPer; ++i) {
    const int e = tid + i * kCommitThreads;
    const int k = e / D, dd = e - (e / D) * D;
    if (k < d && s_src[k] >= 0) {
      kr[i] = K[s_src[k] + dd];
      vr[i] = V[s_vsrc[k] + (long long)dd * P];
    }
  }
  __syncthreads();  // every source element is read before any is overwritten
#pragma unroll
  for (int i = 0; i < kCommitPer; ++i) {
    const int e = tid + i * kCommitThreads;
    const int k = e / D, dd = e - (e / D) * D;
    if (k < d && s_src[k] >= 0) {
      K[s_dst[k] + dd] = kr[i];
      V[s_vdst[k] + (long long)dd * P] = vr[i];
    }
  }
  if (h == 0) {
    // released slots: positions L + d + 1 .. L + B - 1 in order, then -1
    if (tid < B) {
      const int pos = L + d + 1 + tid;
      int slot = -1;
      if (d >= 0 && pos < L + B) {
        const int pg = tab[pos / P];
        if ((unsigned)pg < (unsigned)a.num_pages) slot = pg * P + pos % P;
        else atomicOr(&s_err, kErrSlot);
      }
      a.freed[(size_t)b * B + tid] = slot;
    }
    __syncthreads();
    if (tid == 0 && s_err) flag_error(a.err, s_err);
  } else if (tid == 0 && s_err) {
    flag_error(a.err, s_err);
  }
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
