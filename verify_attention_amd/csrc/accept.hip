// spec_accept and spec_draft_argmax kernels for gfx950.
//
// Accept (the lossless rejection rule of speculative decoding as the Uno /
// Psi-Spec summary states it, the p/q acceptance of section 4.3.1 of "From
// DFlash to dLLM Self-Spec (4)" and the accept/bonus outputs of section 2.2.5
// of "From DFlash to dLLM Self-Spec (2)"):
//   * every workgroup of request b first recomputes the accept length with one
//     wave: lane i gathers p[i, d_i], q[i, d_i], u_i and tests u*q < p in
//     double; a ballot of the failures gives the first reject;
//   * the residual row r = max(p_j - q_j, 0) (or the bonus row p_K) is split
//     into vocabulary chunks, one workgroup per (request, chunk); each wave
//     sums 256-entry sub-blocks in double and stores one mass per sub-block;
//   * a second kernel, one workgroup per request, scans the sub-block masses,
//     finds the sub-block where the running mass passes u_K * S, re-reads only
//     that sub-block to locate the token, and writes every output (a kernel
//     boundary orders the two phases; no device-scope fences or counters).
// Only the residual (or bonus) row pair is streamed from HBM; the other target
// rows are touched at one gathered element each. The tree accept has the same
// two kernels (the walk in the first); when it also commits the accepted path
// (spec_accept_tree_commit), its second kernel adds one workgroup per KV head
// that moves that head's rows beside the one drawing the bonus.
#include "commit_rows.h"
#include "kernels.h"

namespace specattn {

constexpr int kAccThreads = 256;
static_assert(kAccThreads == kCommitThreads, "the accept kernels run the commit helpers");
constexpr int kJTokenErr = 1 << 16;  // jbuf flag: the first reject was an invalid token id

constexpr int kSub = 256;  // vocabulary entries per sub-block (one wave, 4 per lane)
constexpr int kSubInFlight = 4;  // sub-blocks whose loads a wave keeps in flight
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ reductions
__device__ __forceinline__ double wave_sum(double x) { return wave_sum_f64(x); }

__device__ __forceinline__ double wave_inclusive_scan(double x) { return wave_scan_f64(x); }

// Inclusive prefix sum of one double per thread over a 256-thread block, in a
// fixed order (wave scans, then the wave totals through LDS).
__device__ __forceinline__ double block_inclusive_scan(double x, double* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_inclusive_scan(x);
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  __syncthreads();
  return base + x;
}

// The 4 residual entries r_v (v = e .. e+3) of one lane, in double:
// max(p - q, 0), or p alone when q is absent; entries past V are 0.
__device__ __forceinline__ void resid4(const float* p, const float* q, int e, int V, bool vec,
                                       double (&r)[4]) {
  float pv[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
  if (vec && e + 4 <= V) {
    const float4 a = *reinterpret_cast<const float4*>(p + e);
    pv[0] = a.x; pv[1] = a.y; pv[2] = a.z; pv[3] = a.w;
    if (q) {
      const float4 b = *reinterpret_cast<const float4*>(q + e);
      qv[0] = b.x; qv[1] = b.y; qv[2] = b.z; qv[3] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = e + i < V ? p[e + i] : 0.f;
      if (q) qv[i] = e + i < V ? q[e + i] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!q) {
      r[i] = (double)pv[i];
    } else {
      const double d = (double)pv[i] - (double)qv[i];
      r[i] = d > 0.0 ? d : 0.0;
    }
  }
}

__device__ __forceinline__ bool rows_aligned(const float* p, const float* q) {
  return ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(q ? q : p)) & 15) == 0;
}

// Residual rows as functors: r(e .. e+3) for one lane.
// Linear verify: max(p - q, 0), or p alone (bonus row / fallback).
struct ResidPQ {
  const float* p;
  const float* q;
  int V;
  bool vec;
  __device__ __forceinline__ void operator()(int e, double (&r)[4]) const { resid4(p, q, e, V, vec, r); }
};

// Tree verify: p with the listed tokens (the tried children, in LDS) at 0.
struct ResidExcl {
  const float* p;
  int V;
  bool vec;
  const int* excl;
  int n;
  __device__ __forceinline__ void operator()(int e, double (&r)[4]) const {
    resid4(p, nullptr, e, V, vec, r);
    for (int k = 0; k < n; ++k) {
      const int t = excl[k];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t == e + i) r[i] = 0.0;
    }
  }
};

// The accept length of request b, computed by wave 0 and returned to every
// thread of the workgroup: lane i runs test i; a ballot of the failures gives
// the first reject (an invalid token id counts as a reject and is flagged in
// jbuf when write_jbuf).
__device__ int accept_len_of(const AcceptArgs& a, int b, bool write_jbuf) {
  const int K = a.K, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_j;
  if (wave == 0) {
    bool fail = false, bad = false;
    if (lane < K) {
      const double ui = a.u[(size_t)b * (K + 1) + lane];
      const int d = a.draft[(size_t)b * K + lane];
      bad = d < 0 || d >= V;
      if (bad) {
        fail = true;
      } else {
        const double pd = a.p[((size_t)b * (K + 1) + lane) * V + d];
        const double qd = a.q[((size_t)b * K + lane) * V + d];
        fail = !(ui * qd < pd);
      }
    }
    const uint64_t fails = __builtin_amdgcn_ballot_w64(fail);
    const int j = fails ? __builtin_ctzll(fails) : K;
    const uint64_t bads = __builtin_amdgcn_ballot_w64(bad);
    if (lane == 0) {
      s_j = j;
      if (write_jbuf) a.jbuf[b] = j | ((((bads >> j) & 1) && j < K) ? kJTokenErr : 0);
    }
  }
  __syncthreads();
  return s_j;
}

// Kernel 1's work for (request b, vocabulary chunk c): the accept length,
// then the residual (or bonus) mass of every 256-entry sub-block of the chunk
// (one wave per sub-block, 4 entries per lane).
__device__ void accept_partial_body(const AcceptArgs& a, int b, int c) {
  const int K = a.K, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = accept_len_of(a, b, c == 0);
  const float* prow = a.p + ((size_t)b * (K + 1) + j) * V;
  const float* qrow = j < K ? a.q + ((size_t)b * K + j) * V : nullptr;
  const bool vec = rows_aligned(prow, qrow);
  const int nsb = (V + kSub - 1) / kSub;
  const int sb0 = c * (a.chunk / kSub);
  const int sb1 = min(nsb, sb0 + a.chunk / kSub);
  double* out = a.partial + (size_t)b * nsb;
  // each wave streams its sub-blocks (every 4th of the chunk) in batches of
  // kSubInFlight: all of a batch's 16-byte loads of p and q are issued (non-
  // temporal: the rows are read once) before the first is used
  constexpr int kWaves = kAccThreads / 64;
  for (int base = sb0 + wave; base < sb1; base += kSubInFlight * kWaves) {
    f32x4 pv[kSubInFlight], qv[kSubInFlight];
#pragma unroll
    for (int t = 0; t < kSubInFlight; ++t) {
      const int sb = base + t * kWaves;
      const int e = sb * kSub + 4 * lane;
      pv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      qv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (sb < sb1 && vec && e + 4 <= V) {
        pv[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(prow + e));
        if (qrow) qv[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(qrow + e));
      } else if (sb < sb1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[t][i] = e + i < V ? prow[e + i] : 0.f;
          if (qrow) qv[t][i] = e + i < V ? qrow[e + i] : 0.f;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kSubInFlight; ++t) {
      const int sb = base + t * kWaves;
      if (sb >= sb1) break;
      double r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!qrow) {
          r[i] = (double)pv[t][i];
        } else {
          const double d = (double)pv[t][i] - (double)qv[t][i];
          r[i] = d > 0.0 ? d : 0.0;
        }
      }
      const double sum = wave_sum((r[0] + r[1]) + (r[2] + r[3]));
      if (lane == 0) out[sb] = sum;
    }
  }
}

// Kernel 1, one workgroup per (request, vocabulary chunk).
__global__ __launch_bounds__(kAccThreads) void accept_partial_kernel(AcceptArgs a) {
  accept_partial_body(a, blockIdx.x / a.nchunk, blockIdx.x % a.nchunk);
}

// Smallest index t of sub-block sb with base + sum_{v<=t} r_v > thr, found by
// wave 0 (4 entries per lane, then a wave scan); -1 when none passes, with
// *lastp the last index holding mass. Every thread gets the result.
template <typename R>
__device__ int sub_block_search(const R& res, int sb, double base, double thr, int* s_int,
                                int* lastp) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    const int e = sb * kSub + 4 * lane;
    double r[4];
    res(e, r);
    const double mine = (r[0] + r[1]) + (r[2] + r[3]);
    double run = base + (wave_inclusive_scan(mine) - mine);
    int found = -1, lp = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      run += r[i];
      if (found < 0 && run > thr) found = e + i;
      if (r[i] > 0.0) lp = e + i;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(found >= 0);
    const uint64_t pos = __builtin_amdgcn_ballot_w64(lp >= 0);
    const int first = hit ? __shfl(found, __builtin_ctzll(hit), 64) : -1;
    const int last = pos ? __shfl(lp, 63 - __builtin_clzll(pos), 64) : -1;
    if (lane == 0) {
      s_int[0] = first;
      s_int[1] = last;
    }
  }
  __syncthreads();
  const int found = s_int[0];
  *lastp = s_int[1];
  __syncthreads();
  return found;
}

// Draws the token from sub-block masses: thread tid holds the masses of
// sub-blocks [i0, i1) in mv (one pass over them, one sub-block re-read).
// Returns -1 if the total mass is not > 0.
constexpr int kMaxPer = kMaxAcceptVocab / (kSub * kAccThreads);  // sub-blocks per thread

template <typename R>
__device__ int draw_from_masses(const double (&mv)[kMaxPer], int i0, int i1, const R& res,
                                double u, double* s_wave, int* s_int, double* s_dbl) {
  const int tid = threadIdx.x;
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) mine += i0 + k < i1 ? mv[k] : 0.0;
  const double incl = block_inclusive_scan(mine, s_wave);
  if (tid == kAccThreads - 1) s_dbl[0] = incl;
  if (tid == 0) {
    s_int[0] = 0x7fffffff;
    s_int[1] = -1;
  }
  __syncthreads();
  const double S = s_dbl[0];
  if (!(S > 0.0)) return -1;
  const double thr = u * S;
  // first sub-block whose running mass passes thr, and the last one with mass
  double run = incl - mine;
  int hit = -1, lastm = -1;
  double hit_base = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    if (i0 + k >= i1) break;
    const double x = mv[k];
    if (hit < 0 && run + x > thr) {
      hit = i0 + k;
      hit_base = run;
    }
    run += x;
    if (x > 0.0) lastm = i0 + k;
  }
  // one LDS atomic per wave (same-address atomics serialise lane by lane):
  // sub-blocks ascend with the thread index, so the lowest lane with a hit
  // holds the wave's first hit and the highest lane with mass its last one
  const int lane = tid & 63;
  const uint64_t hm = __builtin_amdgcn_ballot_w64(hit >= 0);
  const uint64_t lm = __builtin_amdgcn_ballot_w64(lastm >= 0);
  if (hm && lane == __builtin_ctzll(hm)) atomicMin(&s_int[0], hit);
  if (lm && lane == 63 - __builtin_clzll(lm)) atomicMax(&s_int[1], lastm);
  __syncthreads();
  const int first_hit = s_int[0];
  const int sstar = first_hit != 0x7fffffff ? first_hit : s_int[1];
  // base: running mass before sub-block sstar, from the thread that holds it
  if (sstar >= i0 && sstar < i1) {
    double b0 = incl - mine;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k)
      if (i0 + k < sstar) b0 += mv[k];
    s_dbl[1] = first_hit != 0x7fffffff ? hit_base : b0;
  }
  __syncthreads();
  const double base = s_dbl[1];
  int lastp;
  int tok = sub_block_search(res, sstar, base, thr, s_int, &lastp);
  if (tok < 0) tok = lastp;
  return tok;
}

// The next round's draft-pass block of request b (spec_accept_prepare): token
// 0 is the bonus and the others the mask token; positions continue the new
// committed length; slots come through the page table, as spec_prepare_block
// forms them (-1 with SPEC_ERR_SLOT when the page is missing, SPEC_ERR_CAPACITY
// when the block does not fit the table row).
__device__ void write_next_block(const AcceptArgs& a, int b, int tok, int newL, int tid,
                                 int nthreads) {
  const int B = a.next_B, P = a.next_P;
  if (tid == 0 && (newL < 0 || (long long)newL + B > (long long)a.next_max_pages * P))
    flag_error(a.err, kErrCapacity);
  int errs = 0;
  for (int i = tid; i < B; i += nthreads) {
    const long long pos = (long long)newL + i;
    int32_t slot = -1;
    if (pos >= 0) {
      const long long n = pos / P;
      if (n < a.next_max_pages) {
        const int32_t page = a.next_tab[(size_t)b * a.next_max_pages + n];
        if (page >= 0 && page < a.next_num_pages) slot = page * P + (int32_t)(pos % P);
      }
    }
    if (slot < 0) errs |= kErrSlot;
    const size_t e = (size_t)b * B + i;
    a.next_ids[e] = i == 0 ? tok : a.next_mask;
    a.next_pos[e] = (int32_t)pos;
    a.next_loc[e] = slot;
  }
  if (errs) flag_error(a.err, errs);
}

// Kernel 2's work for request b: scan the sub-block masses, find the
// sub-block where the running mass passes u_K * S, locate the token inside it,
// write every output. Every load that does not depend on the accept length
// goes out first. Returns the drawn token to every thread.
__device__ int accept_select_body(const AcceptArgs& a, int b) {
  const int K = a.K, V = a.V;
  const int tid = threadIdx.x;
  __shared__ double s_wave[4];
  __shared__ double s_dbl[2];
  __shared__ int s_int[2];
  const int nsb = (V + kSub - 1) / kSub;
  const int per = (nsb + kAccThreads - 1) / kAccThreads;
  const int i0 = min(nsb, tid * per), i1 = min(nsb, i0 + per);
  const double* m = a.partial + (size_t)b * nsb;
  double mv[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) mv[k] = i0 + k < i1 ? m[i0 + k] : 0.0;
  const int dtok = tid < K ? a.draft[(size_t)b * K + tid] : -1;
  const int L = a.seq_lens[b];
  const double ub = (double)a.u[(size_t)b * (K + 1) + K];
  const int jw = a.jbuf[b];
  const int j = jw & 0xffff;
  const float* prow = a.p + ((size_t)b * (K + 1) + j) * V;
  const float* qrow = j < K ? a.q + ((size_t)b * K + j) * V : nullptr;
  const bool vec = rows_aligned(prow, qrow);
  int errs = (jw & kJTokenErr) ? kErrToken : 0;
  int tok = draw_from_masses(mv, i0, i1, ResidPQ{prow, qrow, V, vec}, ub, s_wave, s_int, s_dbl);
  if (tok < 0) {
    // zero residual mass: draw from the target row itself (its sub-block
    // masses recomputed into registers, thread by thread)
    errs |= kErrZeroResidual;
    const bool pvec = rows_aligned(prow, nullptr);
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      double t = 0.0;
      if (i0 + k < i1) {
        for (int e = (i0 + k) * kSub; e < min(V, (i0 + k + 1) * kSub); e += 4) {
          double r[4];
          resid4(prow, nullptr, e, V, pvec, r);
          t += (r[0] + r[1]) + (r[2] + r[3]);
        }
      }
      mv[k] = t;
    }
    tok = draw_from_masses(mv, i0, i1, ResidPQ{prow, nullptr, V, pvec}, ub, s_wave, s_int, s_dbl);
  }
  if (tok < 0) tok = 0;
  if (tid == 0) {
    a.accept_len[b] = j;
    a.commit_len[b] = j + 1;
    a.bonus[b] = tok;
    a.new_seq_lens[b] = L + j + 1;
  }
  if (tid <= K)
    a.out_tokens[(size_t)b * (K + 1) + tid] = tid < j ? dtok : (tid == j ? tok : -1);
  if (tid == 0 && errs) flag_error(a.err, errs);
  if (a.next_ids) write_next_block(a, b, tok, L + j + 1, tid, kAccThreads);
  return tok;
}

// Kernel 2, one workgroup per request.
__global__ __launch_bounds__(kAccThreads) void accept_select_kernel(AcceptArgs a) {
  accept_select_body(a, blockIdx.x);
}

// ------------------------------------------------------------- tree verify
// The walk of the Tree sampler's verification (recursive rejection over
// deterministic candidates): at node x, children c in increasing node order
// are accepted iff u[c] * (1 - T) < p_x(token[c]), T the target mass of the
// distinct tokens already tried at x; the first accepted child becomes the
// next node; with none (or at a leaf) the bonus is drawn from p_x with the
// tried tokens set to 0.
//
// One wave; lane l holds nodes l, l + 64, ... (chunks of 64 nodes, N <= 512).
// Every value a test may need, p[parent(n)][token(n)], is gathered in one
// round before the walk, so the walk itself is register work: per chunk the
// children of x are a ballot, T the mass of earlier chunks plus an exclusive
// wave scan, the accepted child the lowest set bit of a second ballot; the
// tokens of children in earlier chunks sit in LDS for the repeat test.
constexpr int kTreeChunks = kMaxTreeNodes / 64;

struct TreeWalk {
  int x;          // final node
  int depth;      // accepted nodes
  int errs;       // kErrToken / kErrTree
};

// jbuf of a tree request: final node | depth << 10 | error bits
constexpr int kJTreeDepthShift = 10;
constexpr int kJTreeMask = (1 << kJTreeDepthShift) - 1;
constexpr int kJTreeTokErr = 1 << 20;
constexpr int kJTreeErr = 1 << 21;
static_assert(kMaxTreeNodes <= kJTreeMask + 1, "node ids fit the jbuf fields");
static_assert(kMaxAcceptVocab <= (1 << (31 - kJTreeDepthShift)), "node | token << 10 fits an int");

__device__ __forceinline__ double wave_exclusive_scan(double x) {
  return wave_inclusive_scan(x) - x;
}

// Lane l's nodes l + 64 c, c < NC: parent and token (loaded once, shared by
// the walk and the excluded set). NC = 1 for trees of at most 64 nodes.
template <int NC>
struct TreeNodes {
  int par[NC], tok[NC];
};

template <int NC>
__device__ __forceinline__ TreeNodes<NC> tree_nodes(const AcceptArgs& a, int b) {
  const int N = a.K, lane = threadIdx.x & 63;
  TreeNodes<NC> t;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = c * 64 + lane;
    const bool in = n < N;
    t.par[c] = in ? a.parent[(size_t)b * N + n] : -2;
    t.tok[c] = in ? a.token[(size_t)b * N + n] : -1;
  }
  return t;
}

// Wave 0 only. path[] (LDS) receives the accepted nodes as node | token << 10
// (accepted tokens are valid ids, V <= 2^19); sib[] (LDS, N entries) is
// scratch for the tokens of the children already tried.
template <int NC>
__device__ TreeWalk tree_walk(const AcceptArgs& a, int b, const TreeNodes<NC>& nd, int* path,
                              int* sib) {
  const int N = a.K, V = a.V;
  const int lane = threadIdx.x & 63, nch = (N + 63) >> 6;
  const uint64_t below = (1ull << lane) - 1;
  // one chunk: every p[parent(n)][token(n)] gathered at once; more chunks:
  // gathered per level, only for the children of the current node (one row,
  // where the up-front gather of every node would touch N rows per
  // workgroup)
  double un[NC], pv[NC];
  bool vpar[NC], vtok[NC];
  TreeWalk w{0, 0, 0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = c * 64 + lane;
    const bool in = n < N;
    const int par = nd.par[c], tok = nd.tok[c];
    un[c] = in ? (double)a.u[(size_t)b * N + n] : 0.0;
    vpar[c] = in && n >= 1 && par >= 0 && par < n;
    vtok[c] = tok >= 0 && tok < V;
    if constexpr (NC == 1)
      pv[c] = (vpar[c] && vtok[c]) ? (double)a.p[((size_t)b * N + par) * V + tok] : 0.0;
    if (__builtin_amdgcn_ballot_w64(in && n >= 1 && !vpar[c])) w.errs |= kErrTree;
  }
  for (int level = 0; level < N; ++level) {
    double T0 = 0.0;  // mass of the distinct tokens tried in earlier chunks
    int nsib = 0, next = -1, ntok = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // children come after their parent: chunks before x's hold none
      if (c >= nch || c < (w.x + 1) >> 6) continue;
      const bool kid = vpar[c] && nd.par[c] == w.x;
      const uint64_t kids = __builtin_amdgcn_ballot_w64(kid);
      if (!kids) continue;
      const int tok = nd.tok[c];
      // a child repeating an earlier sibling's token has residual 0
      bool dup = false;
      for (uint64_t rest = kids; rest; rest &= rest - 1) {
        const int k = __builtin_ctzll(rest);
        const int tk = __builtin_amdgcn_readlane(tok, k);  // k is wave-uniform
        dup |= kid && lane > k && tk == tok;
      }
      if constexpr (NC > 1) {
        for (int i = 0; i < nsib; ++i) dup |= kid && sib[i] == tok;
        pv[c] = (kid && vtok[c]) ? (double)a.p[((size_t)b * N + w.x) * V + tok] : 0.0;
      }
      const double pres = (kid && vtok[c] && !dup) ? pv[c] : 0.0;
      const double incl = wave_inclusive_scan(pres);
      const double T = T0 + (incl - pres);
      const bool acc = kid && vtok[c] && !dup && un[c] * (1.0 - T) < pres;
      const uint64_t accm = __builtin_amdgcn_ballot_w64(acc);
      const int limit = accm ? __builtin_ctzll(accm) : 64;
      if (__builtin_amdgcn_ballot_w64(kid && !vtok[c] && lane < limit)) w.errs |= kErrToken;
      if (accm) {
        next = c * 64 + limit;
        ntok = __builtin_amdgcn_readlane(tok, limit);  // limit is wave-uniform
        break;
      }
      if constexpr (NC > 1) {
        T0 += __shfl(incl, 63, 64);
        if (kid) sib[nsib + __builtin_popcountll(kids & below)] = tok;
        nsib += __builtin_popcountll(kids);
      }
    }
    if (next < 0) break;
    w.x = next;
    if (lane == 0) path[w.depth] = next | (ntok << kJTreeDepthShift);
    ++w.depth;
  }
  return w;
}

// The final node's children tokens (valid ids) into excl[] in node order;
// returns the count. Wave 0 only.
template <int NC>
__device__ int tree_excluded(const AcceptArgs& a, const TreeNodes<NC>& nd, int x, int* excl) {
  const int N = a.K, V = a.V;
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = c * 64 + lane;
    const int par = nd.par[c], tok = nd.tok[c];
    const bool ex = n < N && n >= 1 && par == x && par < n && tok >= 0 && tok < V;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ex);
    if (ex) excl[cnt + __builtin_popcountll(m & below)] = tok;
    cnt += __builtin_popcountll(m);
  }
  return cnt;
}

// Kernel 1, one workgroup per (request, vocabulary chunk): the walk, then
// the residual mass of every 256-entry sub-block of the chunk.
template <int NC>
__global__ __launch_bounds__(kAccThreads) void accept_tree_partial_kernel(AcceptArgs a) {
  const int b = blockIdx.x / a.nchunk;
  const int c = blockIdx.x - b * a.nchunk;
  const int N = a.K, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_path[kMaxTreeNodes], s_excl[kMaxTreeNodes], s_fexcl[kMaxTreeNodes];
  __shared__ int s_sib[kMaxTreeNodes];
  __shared__ int s_x, s_nex, s_nf;
  if (wave == 0) {
    const TreeNodes<NC> nd = tree_nodes<NC>(a, b);
    const TreeWalk w = tree_walk<NC>(a, b, nd, s_path, s_sib);
    const int nex = tree_excluded(a, nd, w.x, s_excl);
    if (lane == 0) {
      s_x = w.x;
      s_nex = nex;
      if (c == 0)
        a.jbuf[b] = w.x | (w.depth << kJTreeDepthShift) |
                    ((w.errs & kErrToken) ? kJTreeTokErr : 0) |
                    ((w.errs & kErrTree) ? kJTreeErr : 0);
    }
    // the accepted nodes (node | token << 10) for the select and the commit
    if (c == 0)
      for (int k = lane; k < w.depth; k += 64) a.pathbuf[(size_t)b * N + k] = s_path[k];
  }
  __syncthreads();
  const int nsb = (V + kSub - 1) / kSub;
  const int sb0 = c * (a.chunk / kSub);
  const int sb1 = min(nsb, sb0 + a.chunk / kSub);
  // the excluded tokens inside this chunk
  if (tid == 0) {
    int nf = 0;
    for (int k = 0; k < s_nex; ++k)
      if (s_excl[k] >= sb0 * kSub && s_excl[k] < sb1 * kSub) s_fexcl[nf++] = s_excl[k];
    s_nf = nf;
  }
  __syncthreads();
  const float* prow = a.p + ((size_t)b * N + s_x) * V;
  const ResidExcl res{prow, V, rows_aligned(prow, nullptr), s_fexcl, s_nf};
  double* out = a.partial + (size_t)b * nsb;
#pragma unroll 2
  for (int sb = sb0 + wave; sb < sb1; sb += kAccThreads / 64) {
    double r[4];
    res(sb * kSub + 4 * lane, r);
    const double t = wave_sum((r[0] + r[1]) + (r[2] + r[3]));
    if (lane == 0) out[sb] = t;
  }
}

// Kernel 2, request b: the bonus from the sub-block masses, then every
// output (all threads of the workgroup).
template <int NC>
__device__ void tree_select(const AcceptArgs& a, int b) {
  const int N = a.K, V = a.V;
  const int tid = threadIdx.x;
  __shared__ double s_wave[4];
  __shared__ double s_dbl[2];
  __shared__ int s_int[2];
  __shared__ int s_excl[kMaxTreeNodes];
  __shared__ int s_nex;
  const int nsb = (V + kSub - 1) / kSub;
  const int per = (nsb + kAccThreads - 1) / kAccThreads;
  const int i0 = min(nsb, tid * per), i1 = min(nsb, i0 + per);
  const double* m = a.partial + (size_t)b * nsb;
  double mv[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) mv[k] = i0 + k < i1 ? m[i0 + k] : 0.0;
  const int L = a.seq_lens[b];
  const double ub = (double)a.u[(size_t)b * N];
  const int jw = a.jbuf[b];
  const int x = jw & kJTreeMask, depth = (jw >> kJTreeDepthShift) & kJTreeMask;
  if (tid < 64) {
    const int nex = tree_excluded<NC>(a, tree_nodes<NC>(a, b), x, s_excl);
    if (tid == 0) s_nex = nex;
  }
  __syncthreads();
  const float* prow = a.p + ((size_t)b * N + x) * V;
  const bool vec = rows_aligned(prow, nullptr);
  int errs = ((jw & kJTreeTokErr) ? kErrToken : 0) | ((jw & kJTreeErr) ? kErrTree : 0);
  int tok = draw_from_masses(mv, i0, i1, ResidExcl{prow, V, vec, s_excl, s_nex}, ub, s_wave,
                             s_int, s_dbl);
  if (tok < 0) {
    // zero residual mass: draw from the node's target row itself
    errs |= kErrZeroResidual;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      double t = 0.0;
      if (i0 + k < i1) {
        for (int e = (i0 + k) * kSub; e < min(V, (i0 + k + 1) * kSub); e += 4) {
          double r[4];
          resid4(prow, nullptr, e, V, vec, r);
          t += (r[0] + r[1]) + (r[2] + r[3]);
        }
      }
      mv[k] = t;
    }
    tok = draw_from_masses(mv, i0, i1, ResidPQ{prow, nullptr, V, vec}, ub, s_wave, s_int, s_dbl);
  }
  if (tok < 0) tok = 0;
  if (tid == 0) {
    a.accept_len[b] = depth;
    a.commit_len[b] = depth + 1;
    a.bonus[b] = tok;
    a.new_seq_lens[b] = L + depth + 1;
  }
  for (int t = tid; t < N; t += kAccThreads) {
    const int pw = t < depth ? a.pathbuf[(size_t)b * N + t] : -1;
    a.path_nodes[(size_t)b * N + t] = pw < 0 ? -1 : pw & kJTreeMask;
    a.out_tokens[(size_t)b * N + t] = pw >= 0 ? pw >> kJTreeDepthShift : (t == depth ? tok : -1);
  }
  if (tid == 0 && errs) flag_error(a.err, errs);
}

// The commit of KV head h of request b in the same call: the accepted path
// (fixed by the walk of kernel 1, which the draw does not change) from the
// workspace; head 0 also lists the released slots. A block past the page
// table keeps its rows and releases nothing.
template <typename KVT>
__device__ void tree_commit_head(const AcceptArgs& a, int b, int h) {
  SPEC_COMMIT_ROWS(rows);
  __shared__ int s_cerr;
  const int tid = threadIdx.x, N = a.K, P = a.commit_P;
  const int32_t* tab = a.commit_tab + (size_t)b * a.commit_max_pages;
  const int L = a.seq_lens[b];
  const bool cap_ok = L >= 0 && (long long)L + N <= (long long)a.commit_max_pages * P;
  const int d = cap_ok ? (a.jbuf[b] >> kJTreeDepthShift) & kJTreeMask : -1;
  if (tid == 0) s_cerr = cap_ok ? 0 : kErrCapacity;  // published by the barrier below
  const int32_t* path = a.pathbuf + (size_t)b * N;
  bool bad = commit_row_bases(rows, [&](int k) { return path[k] & kJTreeMask; }, tab, P,
                              a.commit_D,
                              a.commit_Hkv, a.commit_num_pages, h, L, d);
  commit_move_rows<KVT>(rows, reinterpret_cast<KVT*>(a.commit_k),
                        reinterpret_cast<KVT*>(a.commit_v), P, a.commit_D, d);
  if (h == 0) bad |= commit_freed(a.commit_freed + (size_t)b * N, tab, P, N, a.commit_num_pages,
                                  L, d);
  if (bad) atomicOr(&s_cerr, kErrSlot);
  __syncthreads();
  if (tid == 0 && s_cerr) flag_error(a.err, s_cerr);
}

// Kernel 2, one workgroup per request; with the commit, Hkv + 1 per request:
// workgroup h < Hkv commits KV head h while the last one draws the bonus and
// writes the accept's outputs, side by side.
template <bool COMMIT, typename KVT, int NC>
__global__ __launch_bounds__(kAccThreads) void accept_tree_select_kernel(AcceptArgs a) {
  const int H1 = COMMIT ? a.commit_Hkv + 1 : 1;
  const int b = blockIdx.x / H1, h = blockIdx.x - b * H1;
  if (h == H1 - 1) tree_select<NC>(a, b);
  else if constexpr (COMMIT) tree_commit_head<KVT>(a, b, h);
}

template <int NC>
static hipError_t launch_accept_tree_nc(const AcceptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(accept_tree_partial_kernel<NC>, dim3(a.bs * a.nchunk), dim3(kAccThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 block(kAccThreads);
  if (!a.commit_k)
    hipLaunchKernelGGL((accept_tree_select_kernel<false, float, NC>), dim3(a.bs), block, 0, stream,
                       a);
  else if (a.commit_bf16)
    hipLaunchKernelGGL((accept_tree_select_kernel<true, __bf16, NC>),
                       dim3(a.bs * (a.commit_Hkv + 1)), block, 0, stream, a);
  else
    hipLaunchKernelGGL((accept_tree_select_kernel<true, float, NC>),
                       dim3(a.bs * (a.commit_Hkv + 1)), block, 0, stream, a);
  return hipGetLastError();
}

// Trees of at most 64 nodes take the one-chunk walk (one node per lane).
hipError_t launch_accept_tree(const AcceptArgs& a, hipStream_t stream) {
  return a.K <= 64 ? launch_accept_tree_nc<1>(a, stream)
                   : launch_accept_tree_nc<kTreeChunks>(a, stream);
}

// ----------------------------------------------------------------- argmax
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// One workgroup per row; lowest index wins among equal maxima, NaN never
// wins. Aligned rows: every thread streams its 16-byte vectors (16 of them in
// flight, non-temporal: the logits are read once) keeping only the running
// maximum and the vector that first reached it; the winning vector is read
// again to locate the lowest index holding the value. Then (value, index)
// reductions over the wave and the workgroup.
// The whole workgroup scans `row`: the largest non-NaN value and the lowest
// index holding it (index 0x7fffffff when the row holds only NaN), valid in
// thread 0.
template <typename T>
__device__ __forceinline__ void argmax_row_pair(const T* row, int V, float& out_v, int& out_i) {
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kIn = 16;
  typedef T vecT __attribute__((ext_vector_type(kVec)));
  int t = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const int nv = V / kVec;
    const vecT* rv = reinterpret_cast<const vecT*>(row);
    // the last batch is partial: its loads past the row end are skipped, so
    // the tail keeps kIn loads in flight per lane like the rest
    for (int e = threadIdx.x; e < nv; e += kIn * kAccThreads) {
      vecT v[kIn];
#pragma unroll
      for (int k = 0; k < kIn; ++k)
        if (e + k * kAccThreads < nv) v[k] = __builtin_nontemporal_load(rv + e + k * kAccThreads);
#pragma unroll
      for (int k = 0; k < kIn; ++k) {
        if (e + k * kAccThreads >= nv) break;
        float m = to_f32(v[k][0]);
#pragma unroll
        for (int j = 1; j < kVec; ++j) m = fmaxf(m, to_f32(v[k][j]));
        // later vectors hold larger indices: only a larger value wins (the
        // first vector whose maximum is -inf counts when nothing was seen);
        // the winner's lowest index holding the value is found from the
        // registers, so the (non-temporal, evicted) vector is never re-read
        if (m > bv || (bi == 0x7fffffff && m == bv)) {
          int jf = kVec - 1;
#pragma unroll
          for (int j = kVec - 2; j >= 0; --j) jf = to_f32(v[k][j]) == m ? j : jf;
          bv = m;
          bi = (e + k * kAccThreads) * kVec + jf;
        }
      }
    }
    t = nv * kVec;
  }
  for (int e = t + threadIdx.x; e < V; e += kAccThreads) better(bv, bi, to_f32(row[e]), e);
  // wave then block reduction, comparing (value, -index)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    better(bv, bi, ov, oi);
  }
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < 4; ++w) better(bv, bi, s_v[w], s_i[w]);
  out_v = bv;
  out_i = bi;
}

// Lowest index among the maxima of `row` (0 for a row without a non-NaN
// entry), valid in thread 0.
template <typename T>
__device__ __forceinline__ int argmax_row(const T* row, int V) {
  float bv;
  int bi;
  argmax_row_pair(row, V, bv, bi);
  return bi == 0x7fffffff ? 0 : bi;
}

template <typename T>
__global__ __launch_bounds__(kAccThreads) void argmax_rows_kernel(const T* x, int V, int32_t* out) {
  const int bi = argmax_row(x + (size_t)blockIdx.x * V, V);
  if (threadIdx.x == 0) out[blockIdx.x] = bi;
}

// The quadratic layout's hand-off. With a = accept_len[b] drafts accepted,
// member m of the group after spine token a (block row a * (k + 1) + 1 + m)
// proposes the next round's draft m, its greedy token. The k rows of a request
// are cut into S segments so that the scan keeps the whole GPU busy
// (bs * k rows alone would leave CUs idle at serving batch sizes): kernel 1,
// one workgroup per (request, member, segment), stores the segment's largest
// value and lowest index holding it; kernel 2, one wave per request, merges
// the S segments of each member in index order (largest value, then lowest
// index: the whole-row rule) and writes the drafts and the next block's
// tokens. An accept length outside 0 .. k gives -1 drafts and SPEC_ERR_TREE.
template <typename T>
__global__ __launch_bounds__(kAccThreads) void handoff_partial_kernel(HandoffArgs h) {
  const int seg = blockIdx.x % h.S;
  const int r = blockIdx.x / h.S;  // b * k + m
  const int b = r / h.k, m = r - b * h.k;
  const int k = h.k;
  const int acc = h.accept_len[b];
  const bool ok = acc >= 0 && acc <= k;  // uniform over the workgroup
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  const int e0 = seg * h.seg_len;
  const int n = min(h.V - e0, h.seg_len);
  if (ok && n > 0) {
    const T* row = reinterpret_cast<const T*>(h.logits) +
                   ((size_t)b * h.n + (size_t)acc * (k + 1) + 1 + m) * h.V + e0;
    argmax_row_pair(row, n, bv, bi);
  }
  if (threadIdx.x == 0) {
    h.part_v[blockIdx.x] = bv;
    h.part_i[blockIdx.x] = bi == 0x7fffffff ? bi : bi + e0;
  }
}

__global__ __launch_bounds__(64) void handoff_select_kernel(HandoffArgs h) {
  const int b = blockIdx.x, lane = threadIdx.x, k = h.k;
  const int acc = h.accept_len[b];
  const bool ok = acc >= 0 && acc <= k;
  int tok = -1;
  if (lane < k && ok) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    const size_t base = ((size_t)b * k + lane) * h.S;
    for (int s = 0; s < h.S; ++s) better(bv, bi, h.part_v[base + s], h.part_i[base + s]);
    tok = bi == 0x7fffffff ? 0 : bi;
  }
  if (lane < k) h.next_draft[(size_t)b * k + lane] = tok;
  if (lane == 0 && !ok) flag_error(h.err, kErrTree);
  // row 0: the bonus (the next root); spine rows (m + 1) * (k + 1): the
  // drafts; every group row: the mask token (row e = e0 + lane)
  if (!h.next_block) return;
  for (int e0 = 0; e0 < h.n; e0 += 64) {
    const int e = e0 + lane, j = e / (k + 1), rem = e - j * (k + 1);
    const int draft = __shfl(tok, j > 0 && j <= k ? j - 1 : 0, 64);  // every lane takes part
    if (e < h.n) {
      int32_t v = h.mask_token_id;
      if (e == 0) v = h.bonus[b];
      else if (rem == 0) v = draft;
      h.next_block[(size_t)b * h.n + e] = v;
    }
  }
}

// ------------------------------------------------- quadratic round in one call
// spec_accept_quadratic: the accept of a quadratic block's k spine drafts, the
// hand-off of the next round's drafts and the spine's commit, as two kernels.
// Kernel 1 holds the accept's chunk workgroups and the hand-off's segment
// workgroups (each of which finds the accept length itself, from the same
// gathered tests, before scanning its segment of the chosen group's row).
// Kernel 2 holds, per request, the accept's draw (which then merges the
// hand-off's segments and writes the drafts and the next block) and one
// workgroup per KV head moving that head's accepted spine rows.
template <typename T>
__global__ __launch_bounds__(kAccThreads) void accept_quad_partial_kernel(AcceptArgs a) {
  const int nacc = a.bs * a.nchunk;
  if ((int)blockIdx.x < nacc) {
    accept_partial_body(a, blockIdx.x / a.nchunk, blockIdx.x % a.nchunk);
    return;
  }
  const int idx = blockIdx.x - nacc;
  const int k = a.K, S = a.quad_S;
  const int seg = idx % S, r = idx / S;
  const int b = r / k, m = r - b * k;
  const int j = accept_len_of(a, b, false);
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  const int e0 = seg * a.quad_seg;
  const int n = min(a.V - e0, a.quad_seg);
  if (n > 0) {
    const T* row = reinterpret_cast<const T*>(a.quad_logits) +
                   ((size_t)b * a.quad_n + (size_t)j * (k + 1) + 1 + m) * a.V + e0;
    argmax_row_pair(row, n, bv, bi);
  }
  if (threadIdx.x == 0) {
    a.quad_part_v[idx] = bv;
    a.quad_part_i[idx] = bi == 0x7fffffff ? bi : bi + e0;
  }
}

// Wave 0 of the drawing workgroup: the drafts from the segments of group
// G_j, and the next block (bonus, drafts on the spine rows, mask elsewhere);
// with next_pos, also the next block's positions and slots (the quadratic
// layout's position order: row r = j' (k + 1) + m' sits at depth j' + m'
// after the new committed length, and its K/V at slot L' + r), as
// spec_prepare_tree writes them.
__device__ void quad_handoff_merge(const AcceptArgs& a, int b, int j, int bonus) {
  const int lane = threadIdx.x, k = a.K, n = a.quad_n, S = a.quad_S;
  int tok = -1;
  if (lane < k) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    const size_t base = ((size_t)b * k + lane) * S;
    for (int s = 0; s < S; ++s) better(bv, bi, a.quad_part_v[base + s], a.quad_part_i[base + s]);
    tok = bi == 0x7fffffff ? 0 : bi;
    a.quad_next_draft[(size_t)b * k + lane] = tok;
  }
  // the next round's block, row e = e0 + lane (row e of the layout is
  // member rem of group jj, or spine token jj when rem = 0)
  const int L2 = a.seq_lens[b] + j + 1;  // the next block starts at the new committed length
  const int P = a.commit_P;
  if (a.next_pos && lane == 0 &&
      (L2 < 0 || (long long)L2 + n > (long long)a.commit_max_pages * P))
    flag_error(a.err, kErrCapacity);
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane, jj = e / (k + 1), rem = e - jj * (k + 1);
    const int draft = __shfl(tok, jj > 0 && jj <= k ? jj - 1 : 0, 64);  // every lane takes part
    if (e >= n) continue;
    if (a.quad_next_block) {
      int32_t v = a.quad_mask;
      if (e == 0) v = bonus;
      else if (rem == 0) v = draft;
      a.quad_next_block[(size_t)b * n + e] = v;
    }
    if (a.next_pos) {
      const long long pos = (long long)L2 + e;
      int32_t slot = -1;
      if (pos >= 0 && pos / P < a.commit_max_pages) {
        const int32_t page = a.commit_tab[(size_t)b * a.commit_max_pages + pos / P];
        if (page >= 0 && page < a.commit_num_pages) slot = page * P + (int32_t)(pos % P);
      }
      if (slot < 0) flag_error(a.err, kErrSlot);
      a.next_pos[(size_t)b * n + e] = L2 + jj + rem;
      a.next_loc[(size_t)b * n + e] = slot;
    }
  }
}

// One KV head's share of the spine commit: the accepted spine drafts (rows
// i * (k + 1), i = 1 .. d) move to positions L + 1 .. L + d; KV head 0 also
// lists the released slots of the n-row block.
template <typename KVT>
__device__ void quad_commit_head(const AcceptArgs& a, int b, int h) {
  SPEC_COMMIT_ROWS(rows);
  __shared__ int s_cerr;
  const int tid = threadIdx.x, n = a.quad_n, k = a.K, P = a.commit_P;
  const int32_t* tab = a.commit_tab + (size_t)b * a.commit_max_pages;
  const int L = a.seq_lens[b];
  const bool cap_ok = L >= 0 && (long long)L + n <= (long long)a.commit_max_pages * P;
  const int d = cap_ok ? a.jbuf[b] & 0xffff : -1;
  if (tid == 0) s_cerr = cap_ok ? 0 : kErrCapacity;  // published by the barrier below
  bool bad = commit_row_bases(rows, [&](int r) { return (r + 1) * (k + 1); }, tab, P, a.commit_D,
                              a.commit_Hkv, a.commit_num_pages, h, L, d);
  commit_move_rows<KVT>(rows, reinterpret_cast<KVT*>(a.commit_k),
                        reinterpret_cast<KVT*>(a.commit_v), P, a.commit_D, d);
  if (h == 0) bad |= commit_freed(a.commit_freed + (size_t)b * n, tab, P, n, a.commit_num_pages,
                                  L, d);
  if (bad) atomicOr(&s_cerr, kErrSlot);
  __syncthreads();
  if (tid == 0 && s_cerr) flag_error(a.err, s_cerr);
}

template <typename KVT>
__global__ __launch_bounds__(kAccThreads) void accept_quad_select_kernel(AcceptArgs a) {
  const int H1 = a.commit_Hkv + 1;
  const int b = blockIdx.x / H1, h = blockIdx.x - b * H1;
  if (h == H1 - 1) {
    const int tok = accept_select_body(a, b);
    if (threadIdx.x < 64) quad_handoff_merge(a, b, a.jbuf[b] & 0xffff, tok);
  } else {
    quad_commit_head<KVT>(a, b, h);
  }
}

hipError_t launch_accept_quadratic(const AcceptArgs& a, bool logits_bf16, hipStream_t stream) {
  const dim3 block(kAccThreads);
  const dim3 g1(a.bs * a.nchunk + a.bs * a.K * a.quad_S);
  if (logits_bf16)
    hipLaunchKernelGGL(accept_quad_partial_kernel<__bf16>, g1, block, 0, stream, a);
  else
    hipLaunchKernelGGL(accept_quad_partial_kernel<float>, g1, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(a.bs * (a.commit_Hkv + 1));
  if (a.commit_bf16)
    hipLaunchKernelGGL(accept_quad_select_kernel<__bf16>, g2, block, 0, stream, a);
  else
    hipLaunchKernelGGL(accept_quad_select_kernel<float>, g2, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quadratic_handoff(const HandoffArgs& h, bool bf16, hipStream_t stream) {
  const dim3 grid(h.bs * h.k * h.S);
  if (bf16)
    hipLaunchKernelGGL(handoff_partial_kernel<__bf16>, grid, dim3(kAccThreads), 0, stream, h);
  else
    hipLaunchKernelGGL(handoff_partial_kernel<float>, grid, dim3(kAccThreads), 0, stream, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(handoff_select_kernel, dim3(h.bs), dim3(64), 0, stream, h);
  return hipGetLastError();
}

hipError_t launch_argmax_rows(const void* x, bool bf16, int rows, int V, int32_t* out,
                              hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(argmax_rows_kernel<__bf16>, dim3(rows), dim3(kAccThreads), 0, stream,
                       reinterpret_cast<const __bf16*>(x), V, out);
  else
    hipLaunchKernelGGL(argmax_rows_kernel<float>, dim3(rows), dim3(kAccThreads), 0, stream,
                       reinterpret_cast<const float*>(x), V, out);
  return hipGetLastError();
}

// --------------------------------------------------------- greedy accept
// After the row argmaxes: accept while draft[i] == argmax p[i]; bonus =
// argmax p[accept_len] (the DFlash greedy rule of section 2.2.5).
__global__ __launch_bounds__(64) void greedy_commit_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int K = a.K;
  const int lane = threadIdx.x;
  const int32_t* ids = a.greedy_ids + (size_t)b * (K + 1);
  const bool fail = lane < K && a.draft[(size_t)b * K + lane] != ids[lane];
  const uint64_t fails = __builtin_amdgcn_ballot_w64(fail);
  const int j = fails ? __builtin_ctzll(fails) : K;
  const int tok = ids[j];
  if (lane == 0) {
    a.accept_len[b] = j;
    a.commit_len[b] = j + 1;
    a.bonus[b] = tok;
    a.new_seq_lens[b] = a.seq_lens[b] + j + 1;
  }
  for (int i = lane; i <= K; i += 64)
    a.out_tokens[(size_t)b * (K + 1) + i] = i < j ? a.draft[(size_t)b * K + i] : (i == j ? tok : -1);
  if (a.next_ids) write_next_block(a, b, tok, a.seq_lens[b] + j + 1, lane, 64);
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(accept_partial_kernel, dim3(a.bs * a.nchunk), dim3(kAccThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_select_kernel, dim3(a.bs), dim3(kAccThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_greedy_accept(const AcceptArgs& a, hipStream_t stream) {
  hipError_t e = launch_argmax_rows(a.p, false, a.bs * (a.K + 1), a.V, a.greedy_ids, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(greedy_commit_kernel, dim3(a.bs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace specattn
