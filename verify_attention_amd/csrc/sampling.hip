// Sampling parameters in front of the accept, for gfx950: temperature,
// top-k and top-p processing of logits rows, and the speculative accept on
// the processed target and draft rows.
//
// The operation (see include/specattn.h, spec_sampling_filter and
// spec_accept_logits): the evaluation protocol of "Unlocking Lossless
// Speedups in LLMs via Discrete Diffusion" samples with temperature, top-p and
// top-k, and the I-DLM verify of "From DFlash to dLLM Self-Spec (4)", section
// 4.3.1, consumes logits (gather, softmax / top-k, correction). A row of
// logits becomes a distribution by ranking the tokens (largest logit first,
// lower index first on ties), keeping the first top_k, weighting them by
// exp((l - l_max) / T) and keeping the shortest rank prefix whose mass reaches
// top_p; the linear accept rule then runs on the processed rows.
//
// Three kernels:
//   * tile_max_kernel streams every row once (the HBM-bound pass) and stores
//     the maximum of each 64-entry tile;
//   * row_topk_kernel, one workgroup per row: tau = the top_k-th largest of
//     256 per-thread maxima of tile maxima is a logit that at least top_k
//     entries reach, so every top-k entry lies in a tile whose maximum is at
//     least tau. Only those tiles are read again; their entries >= tau are
//     ranked exactly by counting, and one wave applies temperature and top-p
//     and writes the kept ids and probabilities. Rows whose candidates do not
//     fit in LDS (massive ties) take an exact slow path;
//   * accept_logits_kernel, one wave per request: the tests u_i q_i(d_i) <
//     p_i(d_i) on the kept sets, the first reject, the residual max(p_j -
//     q_j, 0) (or the bonus row) over p_j's kept set drawn in vocabulary
//     order, and every output.
#include "kernels.h"

namespace specattn {

constexpr int kTile = 64;                       // entries per tile maximum
constexpr int kSampThreads = 256;
constexpr int kTilesPerThread = kMaxSampVocab / kTile / kSampThreads;
constexpr int kMaxCandTiles = 1024;             // candidate tiles held in LDS
constexpr int kMaxSurvivors = 2048;             // candidate entries held in LDS
constexpr int kTileIters = 8;                   // tile-max loop iterations per workgroup

static_assert(kTilesPerThread * kTile * kSampThreads == kMaxSampVocab, "vocabulary cap");

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const __bf16* p) { return (float)*p; }

// Row r of the two row sets: rows [0, R1) of x0, then rows of x1.
template <typename T>
__device__ __forceinline__ const T* row_ptr(const SampArgs& a, int r) {
  return r < a.R1 ? reinterpret_cast<const T*>(a.x0) + (size_t)r * a.V
                  : reinterpret_cast<const T*>(a.x1) + (size_t)(r - a.R1) * a.V;
}

// Order-preserving key of a non-NaN float (-0 and +0 share a key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Rank order: (v, i) comes before (w, j) iff v > w, or v == w and i < j.
__device__ __forceinline__ bool ranks_before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// ------------------------------------------------------------ tile maxima
// Grid (rows, blocks per row). Each lane loads 16 bytes; the lanes of one
// tile (16 for float, 8 for bf16) reduce with xor shuffles; NaN entries and
// entries past V count as -inf. kTileIters loads per lane are in flight.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void tile_max_kernel(SampArgs a) {
  constexpr int E = 16 / sizeof(T);
  constexpr int LPT = kTile / E;
  constexpr int TPI = kSampThreads / LPT;
  typedef T vecT __attribute__((ext_vector_type(E)));
  const int row = blockIdx.x;
  const T* x = row_ptr<T>(a, row);
  const int V = a.V;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (V % E == 0);
  const int tid = threadIdx.x;
  const int tile0 = blockIdx.y * (TPI * kTileIters) + tid / LPT;
  const int sub = (tid % LPT) * E;
  float m[kTileIters];
#pragma unroll
  for (int it = 0; it < kTileIters; ++it) {
    const int e0 = (tile0 + it * TPI) * kTile + sub;
    float mx = -__builtin_inff();
    if (vec) {
      if (e0 < V) {
        const vecT v = *reinterpret_cast<const vecT*>(x + e0);
#pragma unroll
        for (int k = 0; k < E; ++k) mx = fmaxf(mx, (float)v[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < E; ++k)
        if (e0 + k < V) mx = fmaxf(mx, load_f32(x + e0 + k));
    }
    m[it] = mx;
  }
#pragma unroll
  for (int it = 0; it < kTileIters; ++it) {
    float mx = m[it];
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const int tile = tile0 + it * TPI;
    if (tid % LPT == 0 && tile < a.ntiles) a.tmax[(size_t)row * a.ntiles + tile] = mx;
  }
}

// ------------------------------------------------------------ exact top-k
// The k-th largest of 256 keys held 4 per lane by one wave, by deciding one
// key bit at a time with ballots (wave-uniform result).
__device__ __forceinline__ uint32_t kth_largest_key(const uint32_t (&key)[4], int k) {
  uint32_t prefix = 0;
  int krem = k;
  for (int b = 31; b >= 0; --b) {
    const uint32_t hi = b == 31 ? 0u : (0xffffffffu << (b + 1));
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool c = ((key[i] & hi) == prefix) && ((key[i] >> b) & 1u);
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c));
    }
    if (cnt >= krem) prefix |= 1u << b;
    else krem -= cnt;
  }
  return prefix;
}

// Exact slow path for one row (candidates overflow LDS): top_k rounds, each
// a workgroup-wide search for the entry ranked right after the previous one.
template <typename T>
__device__ int topk_by_rounds(const T* x, int V, int k, float* s_v, int* s_i, float* s_rv,
                              int* s_ri) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float pv = __builtin_inff();
  int pi = -1;
  int n = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    for (int e = tid; e < V; e += kSampThreads) {
      const float v = load_f32(x + e);
      if (v != v) continue;
      const bool after = ranks_before(pv, pi, v, e);
      if (after && ranks_before(v, e, bv, bi)) {
        bv = v;
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_rv[wave] = bv;
      s_ri[wave] = bi;
    }
    __syncthreads();
    bv = s_rv[0];
    bi = s_ri[0];
    for (int w = 1; w < kSampThreads / 64; ++w)
      if (ranks_before(s_rv[w], s_ri[w], bv, bi)) {
        bv = s_rv[w];
        bi = s_ri[w];
      }
    __syncthreads();
    if (bi == 0x7fffffff) break;  // fewer than k non-NaN entries
    if (tid == 0) {
      s_v[r] = bv;
      s_i[r] = bi;
    }
    pv = bv;
    pi = bi;
    ++n;
  }
  __syncthreads();
  return n;
}

// One workgroup per row: exact top-k, then temperature and top-p (wave 0),
// written as kept ids / probabilities in rank order and the kept count.
template <typename T>
__global__ __launch_bounds__(kSampThreads) void row_topk_kernel(SampArgs a) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.top_k, V = a.V, ntiles = a.ntiles;
  const T* x = row_ptr<T>(a, row);
  __shared__ uint32_t s_key[kSampThreads];
  __shared__ int s_cand[kMaxCandTiles];
  __shared__ float s_sv[kMaxSurvivors];
  __shared__ int s_si[kMaxSurvivors];
  __shared__ float s_topv[kMaxTopK];
  __shared__ int s_topi[kMaxTopK];
  __shared__ float s_rv[4];
  __shared__ int s_ri[4];
  __shared__ int s_ncand, s_nsurv;
  __shared__ float s_tau;

  // per-thread maximum of its tile maxima (tiles tid, tid + 256, ...)
  const float* tm = a.tmax + (size_t)row * ntiles;
  float tv[kTilesPerThread];
  float lmax = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {
    const int t = tid + j * kSampThreads;
    tv[j] = t < ntiles ? tm[t] : -__builtin_inff();
    lmax = fmaxf(lmax, tv[j]);
  }
  s_key[tid] = fkey(lmax);
  if (tid == 0) {
    s_ncand = 0;
    s_nsurv = 0;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t key[4] = {s_key[4 * lane], s_key[4 * lane + 1], s_key[4 * lane + 2],
                             s_key[4 * lane + 3]};
    const uint32_t kk = kth_largest_key(key, k);
    if (lane == 0) s_tau = key_f(kk);
  }
  __syncthreads();
  const float tau = s_tau;
  // candidate tiles: maximum >= tau
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {
    const int t = tid + j * kSampThreads;
    if (t < ntiles && tv[j] >= tau) {
      const int slot = atomicAdd(&s_ncand, 1);
      if (slot < kMaxCandTiles) s_cand[slot] = t;
    }
  }
  __syncthreads();
  const int ncand = s_ncand;
  int ntop;
  if (ncand <= kMaxCandTiles) {
    // entries >= tau of the candidate tiles (one wave per tile, lane = entry)
    for (int c = wave; c < ncand; c += kSampThreads / 64) {
      const int e = s_cand[c] * kTile + lane;
      const float v = e < V ? load_f32(x + e) : -__builtin_inff();
      if (e < V && v >= tau) {
        const int slot = atomicAdd(&s_nsurv, 1);
        if (slot < kMaxSurvivors) {
          s_sv[slot] = v;
          s_si[slot] = e;
        }
      }
    }
    __syncthreads();
  }
  const int nsurv = s_nsurv;
  if (ncand <= kMaxCandTiles && nsurv <= kMaxSurvivors) {
    // exact ranks by counting; the first k go to the top list
    for (int s = tid; s < nsurv; s += kSampThreads) {
      const float v = s_sv[s];
      const int i = s_si[s];
      int rank = 0;
      for (int t = 0; t < nsurv; ++t) rank += ranks_before(s_sv[t], s_si[t], v, i) ? 1 : 0;
      if (rank < k) {
        s_topv[rank] = v;
        s_topi[rank] = i;
      }
    }
    ntop = min(k, nsurv);
    __syncthreads();
  } else {
    ntop = topk_by_rounds(x, V, k, s_topv, s_topi, s_rv, s_ri);
  }
  if (wave != 0) return;
  // temperature and top-p over the ranked top list, one lane per rank
  const bool in = lane < ntop;
  const double v0 = (double)s_topv[0];
  const double e = in ? exp(((double)s_topv[lane] - v0) / (double)a.temperature) : 0.0;
  bool keep = in;
  if (a.top_p < 1.0f) {
    double incl = e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const double zk = __shfl(incl, 63, 64);
    const double up1 = __shfl_up(incl, 1, 64);
    const double before = lane == 0 ? 0.0 : up1;  // mass of the ranks before this one
    keep = in && before / zk < (double)a.top_p;
  }
  double ek = keep ? e : 0.0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ek += __shfl_xor(ek, off, 64);
  const int nkept = __builtin_popcountll(__builtin_amdgcn_ballot_w64(keep));
  if (lane < k) {
    a.kept_ids[(size_t)row * k + lane] = keep ? s_topi[lane] : -1;
    a.kept_probs[(size_t)row * k + lane] = keep ? e / ek : 0.0;
  }
  if (lane == 0) a.n_kept[row] = nkept;
}

// ------------------------------------------------------------ accept
// Probability of token d in kept row r (0 when d is not kept): the row's ids
// (padded with -1) are loaded together, then one probability.
__device__ __forceinline__ double kept_prob(const SampArgs& a, int r, int d) {
  const int k = a.top_k;
  const int32_t* ids = a.kept_ids + (size_t)r * k;
  int at = -1;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s)
    if (s < k && ids[s] == d) at = s;
  return at >= 0 ? a.kept_probs[(size_t)r * k + at] : 0.0;
}

// One wave per request. Rows: target row i of request b is b * (K + 1) + i,
// draft row i is R1 + b * K + i.
__global__ __launch_bounds__(64) void accept_logits_kernel(SampArgs a) {
  const int b = blockIdx.x;
  const int K = a.K, V = a.V, k = a.top_k;
  const int lane = threadIdx.x;
  __shared__ double s_r[kMaxTopK];
  __shared__ int s_v[kMaxTopK];
  // tests: lane i looks up p_i(d_i) and q_i(d_i) in the kept sets
  bool fail = false, bad = false;
  int d = -1;
  if (lane < K) {
    d = a.draft[(size_t)b * K + lane];
    bad = d < 0 || d >= V;
    if (bad) {
      fail = true;
    } else {
      const double pd = kept_prob(a, b * (K + 1) + lane, d);
      const double qd = kept_prob(a, a.R1 + b * K + lane, d);
      const double ui = a.u[(size_t)b * (K + 1) + lane];
      fail = !(ui * qd < pd);
    }
  }
  const uint64_t fails = __builtin_amdgcn_ballot_w64(fail);
  const int j = fails ? __builtin_ctzll(fails) : K;
  int errs = (j < K && ((__builtin_amdgcn_ballot_w64(bad) >> j) & 1)) ? kErrToken : 0;
  // residual over p_j's kept set (lane = rank): max(p - q_j, 0), or p_K
  const int prow = b * (K + 1) + j;
  const int np = a.n_kept[prow];
  const bool in = lane < np;
  const int v = in ? a.kept_ids[(size_t)prow * k + lane] : 0x7fffffff;
  const double pv = in ? a.kept_probs[(size_t)prow * k + lane] : 0.0;
  double r = pv;
  if (j < K && in) {
    const double qv = kept_prob(a, a.R1 + b * K + j, v);
    r = pv - qv > 0.0 ? pv - qv : 0.0;
  }
  double tot = r;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  if (!(tot > 0.0)) {
    errs |= kErrZeroResidual;
    r = pv;
  }
  // vocabulary order: position of this lane's token among the kept ids
  int pos = 0;
  for (int s = 0; s < np; ++s) pos += __shfl(v, s, 64) < v ? 1 : 0;
  if (in) {
    s_r[pos] = r;
    s_v[pos] = v;
  }
  __syncthreads();
  const double rr = in ? s_r[lane] : 0.0;
  const int vv = in ? s_v[lane] : 0;
  double c = rr;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(c, off, 64);
    if (lane >= off) c += y;
  }
  const double S = __shfl(c, max(np, 1) - 1, 64);
  const double thr = (double)a.u[(size_t)b * (K + 1) + K] * S;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(in && c > thr);
  const uint64_t mass = __builtin_amdgcn_ballot_w64(in && rr > 0.0);
  int tok;
  if (hit) tok = __shfl(vv, __builtin_ctzll(hit), 64);
  else if (mass) tok = __shfl(vv, 63 - __builtin_clzll(mass), 64);
  else tok = 0;
  if (lane == 0) {
    a.accept_len[b] = j;
    a.commit_len[b] = j + 1;
    a.bonus[b] = tok;
    a.new_seq_lens[b] = a.seq_lens[b] + j + 1;
    if (errs) flag_error(a.err, errs);
  }
  if (lane <= K)
    a.out_tokens[(size_t)b * (K + 1) + lane] = lane < j ? d : (lane == j ? tok : -1);
}

// ------------------------------------------------------------ launch
template <typename T>
static hipError_t launch_filter_t(const SampArgs& a, hipStream_t stream) {
  constexpr int TPB = kSampThreads / (kTile / (16 / sizeof(T))) * kTileIters;  // tiles per block
  const int rows = a.R1 + a.R2;
  hipLaunchKernelGGL(tile_max_kernel<T>, dim3(rows, (a.ntiles + TPB - 1) / TPB),
                     dim3(kSampThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_topk_kernel<T>, dim3(rows), dim3(kSampThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sampling_filter(const SampArgs& a, bool bf16, hipStream_t stream) {
  return bf16 ? launch_filter_t<__bf16>(a, stream) : launch_filter_t<float>(a, stream);
}

hipError_t launch_accept_logits(const SampArgs& a, bool bf16, hipStream_t stream) {
  hipError_t e = launch_sampling_filter(a, bf16, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_logits_kernel, dim3(a.bs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace specattn
