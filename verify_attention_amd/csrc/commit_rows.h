// The row moves of the committed-prefix K/V (used by spec_commit_kv and by
// the tree accept that commits in the same call).
//
// After an accept of depth d along the path p_1 .. p_d (node ids, k + 1 <=
// p_{k+1} < B, increasing), position L + 1 + k of the request receives the K
// and V of position L + p_{k+1} ("From DFlash to dLLM Self-Spec (4)", section
// 4.6 and the recursive dynamic compaction note of section 4.4.1; the Tree
// sampler of "Unlocking Lossless Speedups in LLMs via Discrete Diffusion"),
// and the slots of positions L + d + 1 .. L + B - 1 are released.
#pragma once

#include "kernels.h"

namespace specattn {

constexpr int kCommitThreads = 256;
constexpr int kCommitPer = 32;  // elements per thread: 63 rows x 128 dims fit
static_assert(kCommitThreads * kCommitPer >= 63 * 128, "one round of loads");

// Element offsets of the moved rows of KV head h (LDS, 64 entries each; -1:
// the row stays in place).
struct CommitRows {
  long long* ksrc;
  long long* kdst;
  long long* vsrc;
  long long* vdst;
};

// Wave 0 (every lane calls it): lane k < d looks up the pages of row k's
// source L + p and destination L + 1 + k. Returns true on every lane when a
// page id lies outside [0, num_pages) (those rows stay in place).
__device__ __forceinline__ bool commit_row_bases(const CommitRows& s, const int32_t* tab, int P,
                                                 int D, int Hkv, int num_pages, int h, int L,
                                                 int d, int p) {
  const int lane = threadIdx.x & 63;
  // row bases: K element (page, h, off, i) at ((page * Hkv + h) * P + off) * D + i,
  // V element (page, h, i, off) at ((page * Hkv + h) * D + i) * P + off
  long long ks = -1, kd = -1, vs = -1, vd = -1;
  bool bad = false;
  if (lane < d) {
    const int src = L + p;
    const int dst = L + 1 + lane;
    const int ps = tab[src / P], pd = tab[dst / P];
    const bool ok = (unsigned)ps < (unsigned)num_pages && (unsigned)pd < (unsigned)num_pages;
    bad = !ok;
    if (ok && src != dst) {
      ks = (((long long)ps * Hkv + h) * P + src % P) * D;
      kd = (((long long)pd * Hkv + h) * P + dst % P) * D;
      vs = ((long long)ps * Hkv + h) * D * P + src % P;
      vd = ((long long)pd * Hkv + h) * D * P + dst % P;
    }
  }
  s.ksrc[lane] = ks;
  s.kdst[lane] = kd;
  s.vsrc[lane] = vs;
  s.vdst[lane] = vd;
  return __builtin_amdgcn_ballot_w64(bad) != 0;
}

// Every thread of the workgroup: reads every moved row's K and V elements
// into registers, a barrier (a destination may be another row's source), then
// writes them. The row bases must be in LDS (a barrier after
// commit_row_bases).
template <typename T>
__device__ __forceinline__ void commit_move_rows(const CommitRows& s, T* K, T* V, int P, int D,
                                                 int d) {
  const int tid = threadIdx.x;
  T kr[kCommitPer], vr[kCommitPer];
#pragma unroll
  for (int i = 0; i < kCommitPer; ++i) {
    const int e = tid + i * kCommitThreads;
    const int k = e / D, dd = e - (e / D) * D;
    if (k < d && s.ksrc[k] >= 0) {
      kr[i] = K[s.ksrc[k] + dd];
      vr[i] = V[s.vsrc[k] + (long long)dd * P];
    }
  }
  __syncthreads();  // every source element is read before any is overwritten
#pragma unroll
  for (int i = 0; i < kCommitPer; ++i) {
    const int e = tid + i * kCommitThreads;
    const int k = e / D, dd = e - (e / D) * D;
    if (k < d && s.ksrc[k] >= 0) {
      K[s.kdst[k] + dd] = kr[i];
      V[s.vdst[k] + (long long)dd * P] = vr[i];
    }
  }
}

// Threads tid < B: the released slots of positions L + d + 1 .. L + B - 1 in
// order, then -1 (all -1 when d < 0). Returns true on a thread that met a page
// id outside [0, num_pages).
__device__ __forceinline__ bool commit_freed(int32_t* freed_row, const int32_t* tab, int P, int B,
                                             int num_pages, int L, int d) {
  const int tid = threadIdx.x;
  bool bad = false;
  if (tid < B) {
    const int pos = L + d + 1 + tid;
    int slot = -1;
    if (d >= 0 && pos < L + B) {
      const int pg = tab[pos / P];
      if ((unsigned)pg < (unsigned)num_pages) slot = pg * P + pos % P;
      else bad = true;
    }
    freed_row[tid] = slot;
  }
  return bad;
}

}  // namespace specattn
