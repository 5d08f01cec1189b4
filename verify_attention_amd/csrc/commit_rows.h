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
constexpr int kCommitPer = 32;       // elements per thread and round
constexpr int kMaxCommitRows = 512;  // moved rows: depth <= B - 1 < 512
static_assert(kCommitThreads * kCommitPer >= 64 * 128, "64 rows of D 128 per round");

// Element offsets of the moved rows of KV head h (LDS, kMaxCommitRows entries
// each; -1: the row stays in place).
struct CommitRows {
  long long* ksrc;
  long long* kdst;
  long long* vsrc;
  long long* vdst;
};

#define SPEC_COMMIT_ROWS(name)                                                 \
  __shared__ long long name##_ks[kMaxCommitRows], name##_kd[kMaxCommitRows],   \
      name##_vs[kMaxCommitRows], name##_vd[kMaxCommitRows];                    \
  const CommitRows name{name##_ks, name##_kd, name##_vs, name##_vd}

// Whether p holds on any thread of the workgroup (every thread calls it):
// one LDS atomic per wave whose ballot is not empty. flag is an LDS int
// cleared before a barrier that precedes the call; ends with a barrier.
__device__ __forceinline__ bool block_any(bool p, int* flag) {
  if (__builtin_amdgcn_ballot_w64(p) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
  __syncthreads();
  return *flag != 0;
}

// Every thread of the workgroup: rows k = tid, tid + kCommitThreads, ... below
// d look up the pages of row k's source L + path(k) and destination L + 1 + k.
// Ends with a barrier (which publishes the row bases) and returns whether a
// page id of this thread's rows lay outside [0, num_pages) (those rows stay
// in place).
template <typename PathFn>
__device__ __forceinline__ bool commit_row_bases(const CommitRows& s, PathFn path,
                                                 const int32_t* tab, int P, int D, int Hkv,
                                                 int num_pages, int h, int L, int d) {
  // row bases: K element (page, h, off, i) at ((page * Hkv + h) * P + off) * D + i,
  // V element (page, h, i, off) at ((page * Hkv + h) * D + i) * P + off
  bool bad = false;
  for (int k = threadIdx.x; k < d; k += kCommitThreads) {
    long long ks = -1, kd = -1, vs = -1, vd = -1;
    const int src = L + path(k);
    const int dst = L + 1 + k;
    const int ps = tab[src / P], pd = tab[dst / P];
    const bool ok = (unsigned)ps < (unsigned)num_pages && (unsigned)pd < (unsigned)num_pages;
    bad |= !ok;
    if (ok && src != dst) {
      ks = (((long long)ps * Hkv + h) * P + src % P) * D;
      kd = (((long long)pd * Hkv + h) * P + dst % P) * D;
      vs = ((long long)ps * Hkv + h) * D * P + src % P;
      vd = ((long long)pd * Hkv + h) * D * P + dst % P;
    }
    s.ksrc[k] = ks;
    s.kdst[k] = kd;
    s.vsrc[k] = vs;
    s.vdst[k] = vd;
  }
  __syncthreads();
  return bad;
}

// Every thread of the workgroup, in rounds of kCommitThreads * kCommitPer / D
// rows in increasing row order: each round reads its rows' K and V elements
// into registers, a barrier, then writes them. Row k's destination L + 1 + k
// is at or before its source L + p_{k+1} (p_{k+1} >= k + 1, increasing), so
// a destination is only ever the source of an earlier row: the barrier of the
// round orders those reads before the write, and no row reads what an earlier
// round wrote. The row bases must be in LDS (commit_row_bases).
template <typename T>
__device__ __forceinline__ void commit_move_rows(const CommitRows& s, T* K, T* V, int P, int D,
                                                 int d) {
  const int tid = threadIdx.x;
  const int R = kCommitThreads * kCommitPer / D;
  for (int r0 = 0; r0 < d; r0 += R) {
    T kr[kCommitPer], vr[kCommitPer];
#pragma unroll
    for (int i = 0; i < kCommitPer; ++i) {
      const int e = tid + i * kCommitThreads;
      const int k = r0 + e / D, dd = e - (e / D) * D;
      if (k < d && s.ksrc[k] >= 0) {
        kr[i] = K[s.ksrc[k] + dd];
        vr[i] = V[s.vsrc[k] + (long long)dd * P];
      }
    }
    __syncthreads();  // every source element is read before any is overwritten
#pragma unroll
    for (int i = 0; i < kCommitPer; ++i) {
      const int e = tid + i * kCommitThreads;
      const int k = r0 + e / D, dd = e - (e / D) * D;
      if (k < d && s.ksrc[k] >= 0) {
        K[s.kdst[k] + dd] = kr[i];
        V[s.vdst[k] + (long long)dd * P] = vr[i];
      }
    }
  }
}

// Every thread: entries t = tid, tid + kCommitThreads, ... below B of the
// released slots of positions L + d + 1 .. L + B - 1 in order, then -1 (all
// -1 when d < 0). Returns true on a thread that met a page id outside
// [0, num_pages).
__device__ __forceinline__ bool commit_freed(int32_t* freed_row, const int32_t* tab, int P, int B,
                                             int num_pages, int L, int d) {
  bool bad = false;
  for (int t = threadIdx.x; t < B; t += kCommitThreads) {
    const int pos = L + d + 1 + t;
    int slot = -1;
    if (d >= 0 && pos < L + B) {
      const int pg = tab[pos / P];
      if ((unsigned)pg < (unsigned)num_pages) slot = pg * P + pos % P;
      else bad = true;
    }
    freed_row[t] = slot;
  }
  return bad;
}

}  // namespace specattn
