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
//     into vocabulary chunks, one workgroup per (request, chunk), each
//     summing its chunk in double;
//   * a second kernel, one workgroup per request, scans the chunk sums, finds
//     the chunk where the running mass passes u_K * S, re-reads only that
//     chunk to locate the token, and writes every output (a kernel boundary
//     orders the two phases; no device-scope fences or counters).
// Only the residual (or bonus) row pair is streamed from HBM; the other target
// rows are touched at one gathered element each.
#include "kernels.h"

namespace specattn {

constexpr int kAccThreads = 256;
constexpr int kJTokenErr = 1 << 16;  // jbuf flag: the first reject was an invalid token id

// ------------------------------------------------------------ block scans
// Inclusive prefix sum of one double per thread over a 256-thread block, in a
// fixed order (wave shuffles, then the wave totals through LDS).
__device__ __forceinline__ double block_inclusive_scan(double x, double* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  __syncthreads();
  return base + x;
}

__device__ __forceinline__ double block_sum(double x, double* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  if (lane == 0) s_wave[wave] = x;
  __syncthreads();
  const double t = (s_wave[0] + s_wave[1]) + (s_wave[2] + s_wave[3]);
  __syncthreads();
  return t;
}

// residual entry in double: max(p - q, 0), or p alone when q is absent
__device__ __forceinline__ double resid(float p, const float* q, size_t i) {
  if (!q) return (double)p;
  const double r = (double)p - (double)q[i];
  return r > 0.0 ? r : 0.0;
}

// Sum of r over [lo, hi) of a row, one double per thread, vectorised when the
// row pointers are 16-byte aligned.
__device__ double range_mass(const float* p, const float* q, int lo, int hi) {
  double s = 0.0;
  const bool vec = ((reinterpret_cast<uintptr_t>(p + lo) | reinterpret_cast<uintptr_t>(q ? q + lo : p)) & 15) == 0;
  int t = lo;
  if (vec) {
    const int n4 = (hi - lo) / 4;
    const float4* p4 = reinterpret_cast<const float4*>(p + lo);
    const float4* q4 = q ? reinterpret_cast<const float4*>(q + lo) : nullptr;
#pragma unroll 4
    for (int e = threadIdx.x; e < n4; e += kAccThreads) {
      const float4 pv = p4[e];
      if (q4) {
        const float4 qv = q4[e];
        const double r0 = (double)pv.x - (double)qv.x, r1 = (double)pv.y - (double)qv.y;
        const double r2 = (double)pv.z - (double)qv.z, r3 = (double)pv.w - (double)qv.w;
        s += (r0 > 0.0 ? r0 : 0.0) + (r1 > 0.0 ? r1 : 0.0) + ((r2 > 0.0 ? r2 : 0.0) + (r3 > 0.0 ? r3 : 0.0));
      } else {
        s += ((double)pv.x + (double)pv.y) + ((double)pv.z + (double)pv.w);
      }
    }
    t = lo + 4 * n4;
  }
  for (int e = t + threadIdx.x; e < hi; e += kAccThreads) s += resid(p[e], q, e);
  return s;
}

// Smallest index t in [lo, hi) with base + sum_{lo<=v<=t} r_v > thr, found by
// giving each thread a contiguous sub-range. Returns -1 when no entry passes;
// *last_pos receives the last index with r > 0 (or -1).
__device__ int range_search(const float* p, const float* q, int lo, int hi, double base,
                            double thr, double* s_wave, int* s_int, int* last_pos) {
  const int n = hi - lo;
  const int per = (n + kAccThreads - 1) / kAccThreads;
  const int a0 = lo + min(n, (int)threadIdx.x * per);
  const int a1 = lo + min(n, ((int)threadIdx.x + 1) * per);
  double mine = 0.0;
  for (int e = a0; e < a1; ++e) mine += resid(p[e], q, e);
  const double incl = block_inclusive_scan(mine, s_wave);
  double run = base + (incl - mine);
  if (threadIdx.x == 0) {
    s_int[0] = 0x7fffffff;
    s_int[1] = -1;
  }
  __syncthreads();
  int found = -1, lastp = -1;
  for (int e = a0; e < a1; ++e) {
    const double r = resid(p[e], q, e);
    if (r > 0.0) lastp = e;
    run += r;
    if (found < 0 && run > thr) found = e;
  }
  if (found >= 0) atomicMin(&s_int[0], found);
  if (lastp >= 0) atomicMax(&s_int[1], lastp);
  __syncthreads();
  const int res = s_int[0] == 0x7fffffff ? -1 : s_int[0];
  *last_pos = s_int[1];
  __syncthreads();
  return res;
}

__device__ void write_outputs(const AcceptArgs& a, int b, int j, int tok) {
  const int K = a.K;
  if (threadIdx.x == 0) {
    a.accept_len[b] = j;
    a.commit_len[b] = j + 1;
    a.bonus[b] = tok;
    a.new_seq_lens[b] = a.seq_lens[b] + j + 1;
  }
  for (int i = threadIdx.x; i <= K; i += kAccThreads)
    a.out_tokens[(size_t)b * (K + 1) + i] = i < j ? a.draft[(size_t)b * K + i] : (i == j ? tok : -1);
}

// Kernel 1, one workgroup per (request, vocabulary chunk): accept length,
// then the residual (or bonus) mass of the chunk.
__global__ __launch_bounds__(kAccThreads) void accept_partial_kernel(AcceptArgs a) {
  const int b = blockIdx.x / a.nchunk;
  const int c = blockIdx.x - b * a.nchunk;
  const int K = a.K, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ int s_j;
  __shared__ double s_wave[4];

  // accept length: lane i runs test i; a ballot of the failures gives the
  // first reject (an invalid token id counts as a reject and is flagged)
  if (tid < 64) {
    bool fail = false, bad = false;
    if (lane < K) {
      const int d = a.draft[(size_t)b * K + lane];
      bad = d < 0 || d >= V;
      if (bad) {
        fail = true;
      } else {
        const double pd = a.p[((size_t)b * (K + 1) + lane) * V + d];
        const double qd = a.q[((size_t)b * K + lane) * V + d];
        const double ui = a.u[(size_t)b * (K + 1) + lane];
        fail = !(ui * qd < pd);
      }
    }
    const uint64_t fails = __builtin_amdgcn_ballot_w64(fail);
    const int j = fails ? __builtin_ctzll(fails) : K;
    const uint64_t bads = __builtin_amdgcn_ballot_w64(bad);
    if (lane == 0) {
      s_j = j;
      if (c == 0) a.jbuf[b] = j | (((bads >> j) & 1) && j < K ? kJTokenErr : 0);
    }
  }
  __syncthreads();
  const int j = s_j;
  const float* prow = a.p + ((size_t)b * (K + 1) + j) * V;
  const float* qrow = j < K ? a.q + ((size_t)b * K + j) * V : nullptr;
  const int lo = c * a.chunk, hi = min(V, lo + a.chunk);
  const double part = block_sum(range_mass(prow, qrow, lo, hi), s_wave);
  if (tid == 0) a.partial[(size_t)b * a.nchunk + c] = part;
}

// Kernel 2, one workgroup per request: scan the chunk masses, find the chunk
// where the running mass passes u_K * S, locate the token inside it, write
// every output.
__global__ __launch_bounds__(kAccThreads) void accept_select_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int K = a.K, V = a.V;
  const int tid = threadIdx.x;
  __shared__ double s_wave[4];
  __shared__ int s_int[2];
  __shared__ double s_tot, s_base;
  const int jw = a.jbuf[b];
  const int j = jw & 0xffff;
  const float* prow = a.p + ((size_t)b * (K + 1) + j) * V;
  const float* qrow = j < K ? a.q + ((size_t)b * K + j) * V : nullptr;
  const double ub = (double)a.u[(size_t)b * (K + 1) + K];
  // chunk masses scanned in chunk order (nchunk <= 256: one per thread)
  const double mine = tid < a.nchunk ? a.partial[(size_t)b * a.nchunk + tid] : 0.0;
  const double incl = block_inclusive_scan(mine, s_wave);
  if (tid == kAccThreads - 1) s_tot = incl;
  __syncthreads();
  const double S = s_tot;
  int tok = -1;
  int errs = (jw & kJTokenErr) ? kErrToken : 0;
  if (S > 0.0) {
    const double thr = ub * S;
    if (tid == 0) {
      s_int[0] = 0x7fffffff;
      s_int[1] = -1;
    }
    __syncthreads();
    if (tid < a.nchunk && incl > thr) atomicMin(&s_int[0], tid);
    if (tid < a.nchunk && mine > 0.0) atomicMax(&s_int[1], tid);
    __syncthreads();
    const int cstar = s_int[0] != 0x7fffffff ? s_int[0] : s_int[1];
    if (tid == cstar) s_base = incl - mine;
    __syncthreads();
    const double base = s_base;
    int lastp;
    const int clo = cstar * a.chunk, chi = min(V, clo + a.chunk);
    tok = range_search(prow, qrow, clo, chi, base, thr, s_wave, s_int, &lastp);
    if (tok < 0) tok = lastp;
  } else {
    // zero residual mass: draw from the target row itself
    errs |= kErrZeroResidual;
    const double S2 = block_sum(range_mass(prow, nullptr, 0, V), s_wave);
    int lastp;
    tok = range_search(prow, nullptr, 0, V, 0.0, ub * S2, s_wave, s_int, &lastp);
    if (tok < 0) tok = lastp;
  }
  if (tok < 0) tok = 0;
  write_outputs(a, b, j, tok);
  if (tid == 0 && errs) flag_error(a.err, errs);
}

// ----------------------------------------------------------------- argmax
// One workgroup per row; lowest index wins among equal maxima.
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T>
__global__ __launch_bounds__(kAccThreads) void argmax_rows_kernel(const T* x, int V, int32_t* out) {
  const T* row = x + (size_t)blockIdx.x * V;
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  constexpr int kVec = 16 / sizeof(T);
  typedef T vecT __attribute__((ext_vector_type(kVec)));
  int t = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const int nv = V / kVec;
    const vecT* rv = reinterpret_cast<const vecT*>(row);
    int e = threadIdx.x;
    // four independent 16-byte loads in flight per thread
    for (; e + 3 * kAccThreads < nv; e += 4 * kAccThreads) {
      vecT v0 = rv[e], v1 = rv[e + kAccThreads], v2 = rv[e + 2 * kAccThreads], v3 = rv[e + 3 * kAccThreads];
#pragma unroll
      for (int k = 0; k < kVec; ++k) better(bv, bi, to_f32(v0[k]), e * kVec + k);
#pragma unroll
      for (int k = 0; k < kVec; ++k) better(bv, bi, to_f32(v1[k]), (e + kAccThreads) * kVec + k);
#pragma unroll
      for (int k = 0; k < kVec; ++k) better(bv, bi, to_f32(v2[k]), (e + 2 * kAccThreads) * kVec + k);
#pragma unroll
      for (int k = 0; k < kVec; ++k) better(bv, bi, to_f32(v3[k]), (e + 3 * kAccThreads) * kVec + k);
    }
    for (; e < nv; e += kAccThreads) {
      vecT v0 = rv[e];
#pragma unroll
      for (int k = 0; k < kVec; ++k) better(bv, bi, to_f32(v0[k]), e * kVec + k);
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
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) better(bv, bi, s_v[w], s_i[w]);
    out[blockIdx.x] = bi == 0x7fffffff ? 0 : bi;
  }
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
