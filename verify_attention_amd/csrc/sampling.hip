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
// Three passes, launched over the rows in two halves (the second half's
// tile maxima computed in the launch that ranks the first half, so that the
// latency-bound ranking runs beside the HBM-bound stream):
//   * tile maxima stream every row once (the HBM-bound pass) and store the
//     maximum of each 64-entry tile;
//   * the ranking, one workgroup per row: tau, the top_k-th largest of
//     256 per-thread maxima of tile maxima rounded down to 16 key bits, is a
//     logit that at least top_k entries reach, so every top-k entry lies in a
//     tile whose maximum is at least tau. Only those tiles are read again;
//     their entries >= tau are ranked exactly by counting, and one wave
//     applies temperature and top-p and writes the kept ids and
//     probabilities. Rows whose candidates do not fit in LDS (massive ties)
//     take an exact slow path;
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
constexpr int kTileIters = 16;                  // 16-byte loads in flight per lane (tile-max pass)

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

// Value of lane l (wave-uniform l) without an LDS round trip.
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
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
__device__ __forceinline__ void tile_max_block(const SampArgs& a, int row, int part) {
  constexpr int E = 16 / sizeof(T);
  constexpr int LPT = kTile / E;
  constexpr int TPI = kSampThreads / LPT;
  typedef T vecT __attribute__((ext_vector_type(E)));
  const T* x = row_ptr<T>(a, row);
  const int V = a.V;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (V % E == 0);
  const int tid = threadIdx.x;
  const int tile0 = part * (TPI * kTileIters) + tid / LPT;
  const int sub = (tid % LPT) * E;
  float m[kTileIters];
  if (vec) {
    // every load is issued before the first is used; the logits are read
    // once, so the loads carry the non-temporal hint
    vecT v[kTileIters];
#pragma unroll
    for (int it = 0; it < kTileIters; ++it) {
      const int e0 = (tile0 + it * TPI) * kTile + sub;
      if (e0 < V) v[it] = __builtin_nontemporal_load(reinterpret_cast<const vecT*>(x + e0));
      else
#pragma unroll
        for (int k = 0; k < E; ++k) v[it][k] = (T)(-__builtin_inff());
    }
#pragma unroll
    for (int it = 0; it < kTileIters; ++it) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < E; ++k) mx = fmaxf(mx, (float)v[it][k]);
      m[it] = mx;
    }
  } else {
#pragma unroll
    for (int it = 0; it < kTileIters; ++it) {
      const int e0 = (tile0 + it * TPI) * kTile + sub;
      float mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < E; ++k)
        if (e0 + k < V) mx = fmaxf(mx, load_f32(x + e0 + k));
      m[it] = mx;
    }
  }
#pragma unroll
  for (int it = 0; it < kTileIters; ++it) {
    float mx = m[it];
    mx = LPT == 16 ? row_max(mx) : half_row_max(mx);  // the tile's lanes
    const int tile = tile0 + it * TPI;
    if (tid % LPT == 0 && tile < a.ntiles) a.tmax[(size_t)row * a.ntiles + tile] = mx;
  }
}

// ------------------------------------------------------------ exact top-k
// Offset of this wave's items in a workgroup-wide list, from each wave's
// (wave-uniform) count; *total = the workgroup's count.
__device__ __forceinline__ int wave_offset(int wcnt, int* s_w, int* total) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_w[wave] = wcnt;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSampThreads / 64; ++w) {
    const int v = s_w[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base;
}

// A threshold for the top-k search: the key of the k-th largest of the 256
// per-thread keys with its low 16 bits cleared, i.e. the largest multiple P of
// 2^16 with at least k keys >= P. Wave 0 holds all 256 keys (4 per lane) and
// decides the 16 high bits from the top down, each by a count of the keys
// reaching the candidate (ballots; no LDS atomics, one barrier each way).
__device__ __forceinline__ uint32_t threshold_key(uint32_t key, int k, int* s_hist, int* s_sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  s_hist[tid] = (int)key;
  __syncthreads();
  if (wave == 0) {
    const uint32_t k0 = (uint32_t)s_hist[lane], k1 = (uint32_t)s_hist[64 + lane],
                   k2 = (uint32_t)s_hist[128 + lane], k3 = (uint32_t)s_hist[192 + lane];
    uint32_t prefix = 0;  // every key reaches 0
#pragma unroll
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(k0 >= cand)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(k1 >= cand)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(k2 >= cand)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(k3 >= cand));
      if (cnt >= k) prefix = cand;
    }
    if (lane == 0) s_sel[0] = (int)prefix;
  }
  __syncthreads();
  return (uint32_t)s_sel[0];
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
__device__ __forceinline__ void row_topk_block(const SampArgs& a, int row) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.top_k, V = a.V, ntiles = a.ntiles;
  const T* x = row_ptr<T>(a, row);
  constexpr int kBatch = 24;  // candidate tiles loaded together per wave
  __shared__ int s_hist[kSampThreads];
  __shared__ int s_rank2[kSampThreads];
  __shared__ int s_cand[kMaxCandTiles];
  __shared__ float s_sv[kMaxSurvivors];
  __shared__ int s_si[kMaxSurvivors];
  __shared__ float s_topv[kMaxTopK];
  __shared__ int s_topi[kMaxTopK];
  __shared__ float s_rv[4];
  __shared__ int s_ri[4], s_w[4], s_sel[2];

  // per-thread maximum of its tile maxima (tiles tid, tid + 256, ...); the
  // register loops are unrolled for the largest vocabulary and leave at the
  // row's own tile count (a uniform branch)
  const float* tm = a.tmax + (size_t)row * ntiles;
  const int jn = (ntiles + kSampThreads - 1) / kSampThreads;
  float tv[kTilesPerThread];
  float lmax = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {  // every load goes out before any use
    if (j >= jn) break;
    const int t = tid + j * kSampThreads;
    tv[j] = t < ntiles ? tm[t] : -__builtin_inff();
  }
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {
    if (j >= jn) break;
    lmax = fmaxf(lmax, tv[j]);
  }
  float tau = key_f(threshold_key(fkey(lmax), k, s_hist, s_sel));
  if (tau != tau) tau = -__builtin_inff();  // a prefix of the -inf key decodes to NaN

  // candidate tiles (maximum >= tau), compacted with ballots: per wave a
  // running count, the wave offsets through LDS
  int wcnt = 0;
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {
    if (j >= jn) break;
    wcnt += __builtin_popcountll(
        __builtin_amdgcn_ballot_w64(tid + j * kSampThreads < ntiles && tv[j] >= tau));
  }
  int ncand;
  int at = wave_offset(wcnt, s_w, &ncand);
#pragma unroll
  for (int j = 0; j < kTilesPerThread; ++j) {
    if (j >= jn) break;
    const int t = tid + j * kSampThreads;
    const bool take = t < ntiles && tv[j] >= tau;
    const uint64_t m = __builtin_amdgcn_ballot_w64(take);
    const int slot = at + lanes_below(m);
    if (take && slot < kMaxCandTiles) s_cand[slot] = t;
    at += __builtin_popcountll(m);
  }
  __syncthreads();
  int nsurv = 0;
  if (ncand <= kMaxCandTiles) {
    // entries >= tau of the candidate tiles (lane = entry of a tile); every
    // wave loads up to kBatch tiles at once (tiles dealt to the waves in
    // turn, so that a short list keeps all four busy), the survivors are
    // compacted by a scan
    for (int c0 = 0; c0 < ncand; c0 += kBatch * (kSampThreads / 64)) {
      float v[kBatch];
      int e[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const int c = c0 + t * (kSampThreads / 64) + wave;
        e[t] = c < ncand ? s_cand[c] * kTile + lane : V;
        v[t] = e[t] < V ? load_f32(x + e[t]) : -__builtin_inff();
      }
      int wc = 0;
#pragma unroll
      for (int t = 0; t < kBatch; ++t)
        wc += __builtin_popcountll(__builtin_amdgcn_ballot_w64(e[t] < V && v[t] >= tau));
      int tot;
      int o = nsurv + wave_offset(wc, s_w, &tot);
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const bool take = e[t] < V && v[t] >= tau;
        const uint64_t m = __builtin_amdgcn_ballot_w64(take);
        const int slot = o + lanes_below(m);
        if (take && slot < kMaxSurvivors) {
          s_sv[slot] = v[t];
          s_si[slot] = e[t];
        }
        o += __builtin_popcountll(m);
      }
      nsurv += tot;
    }
    __syncthreads();
  }
  int ntop;
  if (ncand <= kMaxCandTiles && nsurv <= 128) {
    // exact ranks by counting: every wave holds survivors lane and 64 + lane
    // in registers and counts, for both, the survivors t of its quarter of
    // the list that rank before them (t read by readlane); wave 0 adds
    const bool ina = lane < nsurv, inb = 64 + lane < nsurv;
    const float va = ina ? s_sv[lane] : -__builtin_inff();
    const int ia = ina ? s_si[lane] : 0x7fffffff;
    const float vb = inb ? s_sv[64 + lane] : -__builtin_inff();
    const int ib = inb ? s_si[64 + lane] : 0x7fffffff;
    const int q = (nsurv + 3) >> 2, t0 = wave * q, t1 = min(nsurv, t0 + q);
    int ra = 0, rb = 0;
    for (int t = t0; t < t1; ++t) {
      const float vt = lane_f(t < 64 ? va : vb, t & 63);
      const int it = lane_i(t < 64 ? ia : ib, t & 63);
      ra += ranks_before(vt, it, va, ia) ? 1 : 0;
      rb += ranks_before(vt, it, vb, ib) ? 1 : 0;
    }
    s_hist[tid] = ra;
    s_rank2[tid] = rb;
    __syncthreads();
    if (wave == 0) {
      ra += s_hist[64 + lane] + s_hist[128 + lane] + s_hist[192 + lane];
      rb += s_rank2[64 + lane] + s_rank2[128 + lane] + s_rank2[192 + lane];
      if (ina && ra < k) {
        s_topv[ra] = va;
        s_topi[ra] = ia;
      }
      if (inb && rb < k) {
        s_topv[rb] = vb;
        s_topi[rb] = ib;
      }
    }
    ntop = min(k, nsurv);
    __syncthreads();
  } else if (ncand <= kMaxCandTiles && nsurv <= kMaxSurvivors) {
    // exact ranks by counting over LDS
    for (int s2 = tid; s2 < nsurv; s2 += kSampThreads) {
      const float v = s_sv[s2];
      const int i = s_si[s2];
      int rank = 0;
#pragma unroll 8
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
    const double incl = wave_scan_f64(e);
    const double zk = __shfl(incl, 63, 64);
    const double up1 = __shfl_up(incl, 1, 64);
    const double before = lane == 0 ? 0.0 : up1;  // mass of the ranks before this one
    keep = in && before / zk < (double)a.top_p;
  }
  double ek = keep ? e : 0.0;
  ek = wave_sum_f64(ek);
  const int nkept = __builtin_popcountll(__builtin_amdgcn_ballot_w64(keep));
  if (lane < a.stride) {
    a.kept_ids[(size_t)row * a.stride + lane] = keep ? s_topi[lane] : -1;
    a.kept_probs[(size_t)row * a.stride + lane] = keep ? e / ek : 0.0;
  }
  if (lane == 0) a.n_kept[row] = nkept;
}

// ------------------------------------------------------------ accept
// Kept rows in the accept's workspace are padded to kMaxTopK entries (ids -1,
// probabilities 0), so a row is read whole with unguarded 16-byte loads.
// Position of token d in kept row r, or -1.
__device__ __forceinline__ int kept_slot(const SampArgs& a, int r, int d) {
  const int4* ids = reinterpret_cast<const int4*>(a.kept_ids + (size_t)r * kMaxTopK);
  int4 w[kMaxTopK / 4];
#pragma unroll
  for (int s = 0; s < kMaxTopK / 4; ++s) w[s] = ids[s];
  int at = -1;
#pragma unroll
  for (int s = kMaxTopK / 4 - 1; s >= 0; --s) {
    at = w[s].w == d ? 4 * s + 3 : at;
    at = w[s].z == d ? 4 * s + 2 : at;
    at = w[s].y == d ? 4 * s + 1 : at;
    at = w[s].x == d ? 4 * s : at;
  }
  return at;
}

// One wave per request. Rows: target row i of request b is b * (K + 1) + i,
// draft row i is R1 + b * K + i.
__global__ __launch_bounds__(64) void accept_logits_kernel(SampArgs a) {
  const int b = blockIdx.x;
  const int K = a.K, V = a.V;
  const int lane = threadIdx.x;
  __shared__ double s_r[kMaxTopK], s_qp[kMaxTopK];
  __shared__ int s_v[kMaxTopK], s_qid[kMaxTopK];
  // tests: lane i looks up p_i(d_i) and q_i(d_i) in the kept sets
  bool fail = false, bad = false;
  int d = -1;
  if (lane < K) {
    d = a.draft[(size_t)b * K + lane];
    const double ui = a.u[(size_t)b * (K + 1) + lane];
    bad = d < 0 || d >= V;
    const int rp = b * (K + 1) + lane, rq = a.R1 + b * K + lane;
    const int ap = kept_slot(a, rp, d), aq = kept_slot(a, rq, d);
    const double pd = ap >= 0 ? a.kept_probs[(size_t)rp * kMaxTopK + ap] : 0.0;
    const double qd = aq >= 0 ? a.kept_probs[(size_t)rq * kMaxTopK + aq] : 0.0;
    fail = bad || !(ui * qd < pd);
  }
  const uint64_t fails = __builtin_amdgcn_ballot_w64(fail);
  const int j = fails ? __builtin_ctzll(fails) : K;
  int errs = (j < K && ((__builtin_amdgcn_ballot_w64(bad) >> j) & 1)) ? kErrToken : 0;
  // residual over p_j's kept set (lane = rank): max(p - q_j, 0), or p_K
  const int prow = b * (K + 1) + j;
  const int v = a.kept_ids[(size_t)prow * kMaxTopK + lane];
  const double pv = a.kept_probs[(size_t)prow * kMaxTopK + lane];
  const bool in = v >= 0;
  const int np = __builtin_popcountll(__builtin_amdgcn_ballot_w64(in));
  double r = pv;
  if (j < K) {
    const size_t qrow = (size_t)(a.R1 + b * K + j) * kMaxTopK;
    s_qid[lane] = a.kept_ids[qrow + lane];
    s_qp[lane] = a.kept_probs[qrow + lane];
    __syncthreads();
    double qv = 0.0;
    for (int s = 0; s < kMaxTopK; ++s) qv = (in && s_qid[s] == v) ? s_qp[s] : qv;
    r = pv - qv > 0.0 ? pv - qv : 0.0;
  }
  double tot = r;
  tot = wave_sum_f64(tot);
  if (!(tot > 0.0)) {
    errs |= kErrZeroResidual;
    r = pv;
  }
  // vocabulary order: position of this lane's token among the kept ids
  int pos = 0;
  for (int s = 0; s < np; ++s) pos += lane_i(v, s) < v ? 1 : 0;
  if (in) {
    s_r[pos] = r;
    s_v[pos] = v;
  }
  __syncthreads();
  const bool inv = lane < np;
  const double rr = inv ? s_r[lane] : 0.0;
  const int vv = inv ? s_v[lane] : 0;
  const double c = wave_scan_f64(rr);
  const double S = __shfl(c, max(np, 1) - 1, 64);
  const double thr = (double)a.u[(size_t)b * (K + 1) + K] * S;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(inv && c > thr);
  const uint64_t mass = __builtin_amdgcn_ballot_w64(inv && rr > 0.0);
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

// Grid (rows, blocks per row): tile maxima of rows t0 ...
template <typename T>
__global__ __launch_bounds__(kSampThreads) void tile_max_kernel(SampArgs a, int t0) {
  tile_max_block<T>(a, t0 + blockIdx.x, blockIdx.y);
}

// One block per row: the ranks of rows k0 ...
template <typename T>
__global__ __launch_bounds__(kSampThreads) void row_topk_kernel(SampArgs a, int k0) {
  row_topk_block<T>(a, k0 + blockIdx.x);
}

// Blocks [0, nk) rank rows k0 .., one per block, whose tile maxima an earlier
// launch stored; the blocks after them compute tile maxima of rows t0 ..,
// bpr blocks per row. One launch thus ranks one part of the rows while
// streaming another (the ranking blocks, dispatched first, start at once).
template <typename T>
__global__ __launch_bounds__(kSampThreads) void tile_max_topk_kernel(SampArgs a, int k0, int nk,
                                                                     int t0, int bpr) {
  const int x = blockIdx.x;
  if (x < nk) row_topk_block<T>(a, k0 + x);
  else tile_max_block<T>(a, t0 + (x - nk) / bpr, (x - nk) % bpr);
}

// ------------------------------------------------------------ launch
// The rows are streamed in two halves: the second half's tile maxima are
// computed in the same launch that ranks the first half, so the ranking's
// latency-bound blocks run beside the HBM-bound stream.
template <typename T>
static hipError_t launch_filter_t(const SampArgs& a, hipStream_t stream) {
  constexpr int TPB = kSampThreads / (kTile / (16 / sizeof(T))) * kTileIters;  // tiles per block
  const int rows = a.R1 + a.R2, h = (rows + 1) / 2;
  const int bpr = (a.ntiles + TPB - 1) / TPB;
  // tile maxima of rows [0, h)
  hipLaunchKernelGGL(tile_max_kernel<T>, dim3(h, bpr), dim3(kSampThreads), 0, stream, a, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the ranks of rows [0, h) beside the tile maxima of rows [h, rows)
  hipLaunchKernelGGL(tile_max_topk_kernel<T>, dim3(h + (rows - h) * bpr), dim3(kSampThreads), 0,
                     stream, a, 0, h, h, bpr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // ranks of rows [h, rows)
  if (rows > h)
    hipLaunchKernelGGL(row_topk_kernel<T>, dim3(rows - h), dim3(kSampThreads), 0, stream, a, h);
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
