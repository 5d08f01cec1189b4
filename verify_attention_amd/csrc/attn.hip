// block_attn: block-query attention over a paged KV cache for gfx950.
//
// The operation (see include/specattn.h): every query row of a decode-round
// block attends to the request's cached context and to the block's own K/V
// under a per-launch intra-block mask -- a rectangle for the block-diffusion
// draft pass, a triangle for the AR verify pass, and the I-DLM mixed layout
// (causal clean rows, bidirectional MASK rows) -- as drawn in the "Attention
// Mask" section of "SGLang strengthens diffusion LLMs: LLaDA 2.0" and in
// sections 4.3.1 / 4.4.1 of "From DFlash to dLLM Self-Spec (4)".
//
// Work decomposition (one workgroup per (request, KV head, split)):
//   * All g * B query rows that share one KV head (the g query heads of the
//     GQA group times the B block tokens) form the MFMA N dimension, so each
//     K/V page is read from HBM once per KV head.
//   * A row group is 64 rows (4 MFMA tiles of 16); a 4-wave workgroup holds
//     one row group served by 4 key waves, or two row groups of 2 key waves
//     each. The key waves of a row group take interleaved 32-key steps of the
//     split's key range (a flash-decoding style key split inside the
//     workgroup), so no KV tile is staged or shared through LDS: every wave
//     loads its own MFMA operands straight from HBM with 16-byte loads and
//     prefetches the next step into registers. Only the last steps of a
//     sequence (the block and the ragged end) carry masks and bounds checks.
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16
//     (8 x v_mfma_f32_16x16x4f32 for fp32 inputs). Keys are permuted inside a
//     32-key step so that the accumulator layout of S^T is directly the B
//     operand of the PV product and the dim-major V page gives the A operand
//     as one contiguous 16-byte run: no shuffles between the two products.
//   * Online softmax in fp32 (exp2 domain), row max across the 4 lane groups
//     via permlane swaps, lazy rescaling (the reference max only moves when a
//     new max exceeds it by 2^8), masks applied only on steps that reach the
//     block.
//   * The 4 waves' partial states are merged through LDS in a fixed order;
//     with several splits per (request, KV head) the workgroup stores its
//     partial state and the last workgroup to finish (device-scope counter)
//     merges all splits: one kernel launch per call.
#include "kernels.h"

namespace specattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite start value for running maxima
constexpr float kRescale = 8.0f;      // lazy rescale threshold, log2 units
constexpr int kStep = 32;             // keys per step
constexpr int kRowsPerGroup = 64;

// ---------------------------------------------------------------- fragments
// A fragment is the 8 consecutive reduction-dimension elements one lane feeds
// to one 16x16x32 MFMA (bf16), or to eight 16x16x4 fp32 MFMAs.
template <typename T> struct Frag;

template <> struct Frag<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ vec load(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ vec zero() { return vec{}; }
  static __device__ __forceinline__ floatx4 mma(const vec& a, const vec& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec pack(const floatx8& x) {
    return __builtin_convertvector(x, bf16x8);  // v_cvt_pk_bf16_f32, round to nearest even
  }
  static __device__ __forceinline__ void clear(vec& v, int j) { v[j] = (__bf16)0.0f; }
  static __device__ __forceinline__ void store4(__bf16* p, floatx4 x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    *reinterpret_cast<bf16x4*>(p) = r;
  }
};

template <> struct Frag<float> {
  typedef floatx8 vec;
  static __device__ __forceinline__ vec load(const float* p) {
    return *reinterpret_cast<const floatx8*>(p);
  }
  static __device__ __forceinline__ vec zero() { return vec{}; }
  static __device__ __forceinline__ floatx4 mma(const vec& a, const vec& b, floatx4 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ vec pack(const floatx8& x) { return x; }
  static __device__ __forceinline__ void clear(vec& v, int j) { v[j] = 0.0f; }
  static __device__ __forceinline__ void store4(float* p, floatx4 x) {
    *reinterpret_cast<floatx4*>(p) = x;
  }
};

__device__ __forceinline__ bool block_visible(int mode, int i, int jb, int nc) {
  // mode 0 BIDIR (rectangle), 1 CAUSAL (triangle), 2 MIXED (causal clean rows,
  // all-visible MASK rows)
  return mode == 0 || jb <= i || (mode == 2 && i >= nc);
}

// Operand registers of one 32-key step.
template <typename T, int D>
struct StepFrags {
  typename Frag<T>::vec k[2][D / 32];  // A operands of S^T = K Q^T, two 16-key tiles
  typename Frag<T>::vec v[D / 16];     // A operands of O^T += V^T P^T, one per 16-dim tile
};

// Per-wave geometry of the current (request, KV head).
template <typename T>
struct KvView {
  const T* kbase;        // k_pool + kvh * P * D
  const T* vbase;        // v_pool + kvh * P * D
  const int32_t* ptab;   // page_table row of the request
  size_t page_stride;    // elements per physical page (all KV heads)
};

// Physical pages of the (at most two) pages of the step at key0; ids outside
// the pool are flagged and replaced by page 0.
template <typename T>
__device__ __forceinline__ void step_pages(const KvView<T>& kv, const AttnArgs& a, int key0,
                                           bool hi_valid, int& lo, int& hi) {
  lo = kv.ptab[key0 >> a.p_shift];
  hi = lo;
  if (a.P == 16 && hi_valid) hi = kv.ptab[(key0 >> a.p_shift) + 1];
  if ((unsigned)lo >= (unsigned)a.num_pages || (unsigned)hi >= (unsigned)a.num_pages) {
    if ((threadIdx.x & 63) == 0) flag_error(a.err, kErrSlot);
    if ((unsigned)lo >= (unsigned)a.num_pages) lo = 0;
    if ((unsigned)hi >= (unsigned)a.num_pages) hi = 0;
  }
}

// Loads the K and V operands of the step starting at key0. Lane (n, grp):
//   K tile T row n  <- key key0 + 8*(n/4) + 4*T + n%4, dims 32c + 8*grp .. +7
//   V tile dt row n <- dim 16*dt + n, keys key0 + 8*grp .. +7
// TAIL: keys at or past n_keys are read from a valid slot of the step and
// zeroed (their own slots may hold anything, or not exist).
template <typename T, int D, bool TAIL>
__device__ __forceinline__ void load_step(StepFrags<T, D>& f, const KvView<T>& kv,
                                          const AttnArgs& a, int key0, int n_keys, int lane) {
  const int n = lane & 15, grp = lane >> 4;
  const int P = a.P;
  int page_lo, page_hi;
  step_pages(kv, a, key0, !TAIL || key0 + 16 < n_keys, page_lo, page_hi);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kk = 8 * (n >> 2) + 4 * t + (n & 3);  // key inside the step
    const bool ok = !TAIL || key0 + kk < n_keys;
    const int kq = ok ? kk : 0;
    const int page = (P == 16 && kq >= 16) ? page_hi : page_lo;
    const T* src = kv.kbase + page * kv.page_stride + (size_t)((key0 + kq) & (P - 1)) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      f.k[t][c] = Frag<T>::load(src + 32 * c);
      if (TAIL && !ok) f.k[t][c] = Frag<T>::zero();
    }
  }
  {
    const int kk = 8 * grp;
    const bool ok = !TAIL || key0 + kk < n_keys;
    const int kq = ok ? kk : 0;
    const int page = (P == 16 && kq >= 16) ? page_hi : page_lo;
    const T* src = kv.vbase + page * kv.page_stride + (size_t)n * P + ((key0 + kq) & (P - 1));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = Frag<T>::load(src + (size_t)16 * dt * P);
    if (TAIL) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (key0 + kk + j >= n_keys) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) Frag<T>::clear(f.v[dt], j);
        }
    }
  }
}

// One 32-key step: S^T = K Q^T, (mask), online softmax update, O^T += V^T P^T.
// s[T][t][j] is key key0 + 8*grp + 4*T + j against row 16t + n of the wave;
// softmax runs in the exp2 domain with the scale folded into the exponent.
template <typename T, int D, int MT, bool MASKED>
__device__ __forceinline__ void compute_step(const StepFrags<T, D>& f,
                                             const typename Frag<T>::vec (&qf)[MT][D / 32],
                                             floatx4 (&acc)[D / 16][MT], float (&m_run)[MT],
                                             float (&l_run)[MT], const int (&blk_row)[MT],
                                             const AttnArgs& a, int key0, int L, int n_keys,
                                             int nc, int grp) {
  floatx4 s[2][MT];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) c = Frag<T>::mma(f.k[t2][cc], qf[t][cc], c);
      s[t2][t] = c;
    }

  if (MASKED) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + 8 * grp + 4 * t2 + j;
          const bool vis = key < L ||
                           (key < n_keys && block_visible(a.mode, blk_row[t], key - L, nc));
          if (!vis) s[t2][t][j] = -__builtin_inff();
        }
  }

  const float c2 = a.scale_log2;
  float m_new[MT];
  bool need_any = false;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float mx = fmaxf(fmaxf(fmaxf(s[0][t][0], s[0][t][1]), fmaxf(s[0][t][2], s[0][t][3])),
                     fmaxf(fmaxf(s[1][t][0], s[1][t][1]), fmaxf(s[1][t][2], s[1][t][3])));
    mx = group_max4(mx) * c2;
    m_new[t] = fmaxf(m_run[t], mx);
    need_any |= m_new[t] > m_run[t] + kRescale;
  }
  if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const bool need = m_new[t] > m_run[t] + kRescale;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run[t] - m_new[t]) : 1.0f;
      m_run[t] = need ? m_new[t] : m_run[t];
      l_run[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt][t] *= alpha;
    }
  }
  typename Frag<T>::vec pf[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    floatx8 pv;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pv[4 * t2 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t2][t][j], c2, -m_run[t]));
    l_run[t] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    pf[t] = Frag<T>::pack(pv);
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[dt][t] = Frag<T>::mma(f.v[dt], pf[t], acc[dt][t]);
}

// RG row groups of 64 rows, each served by 4 / RG key waves: the workgroup is
// always 4 waves, so a wave may use the whole 512-entry register file.
template <typename T, int D, int MT, int RG>
__global__ __launch_bounds__(kWave * 4, 1) void block_attn_kernel(AttnArgs a) {
  typedef typename Frag<T>::vec vec;
  constexpr int KW = 4 / RG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = wave / KW;   // row group
  const int kw = wave % KW;   // key wave inside the row group
  const int n = lane & 15, grp = lane >> 4;

  const int unit = blockIdx.x / a.splits;
  const int split = blockIdx.x - unit * a.splits;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;

  int L = a.seq_lens[b];
  const int cap = a.max_pages * a.P - a.B;
  if (L < 0 || L > cap) {
    if (tid == 0 && split == 0) flag_error(a.err, kErrCapacity);
    L = L < 0 ? 0 : cap;
  }
  const int n_keys = L + a.B;
  const int nc = a.nc_per_req ? a.nc_per_req[b] : a.n_causal;
  const int n_steps = (n_keys + kStep - 1) / kStep;
  const int s_lo = split * a.steps_per_split;
  const int s_hi = (split == a.splits - 1) ? n_steps : min(n_steps, s_lo + a.steps_per_split);
  const int s_full = min(s_hi, L / kStep);  // steps [s_lo, s_full) hold context keys only

  KvView<T> kv;
  kv.kbase = reinterpret_cast<const T*>(a.k) + (size_t)kvh * a.P * D;
  kv.vbase = reinterpret_cast<const T*>(a.v) + (size_t)kvh * a.P * D;
  kv.ptab = a.page_table + (size_t)b * a.max_pages;
  kv.page_stride = (size_t)a.P * D * a.Hkv;

  // ---- Q^T operands for this wave's 16*MT rows: lane (n, grp) holds row
  // 16t + n, dims 32c + 8*grp .. +7. Row r of the group is block token r / g,
  // query head kvh * g + r % g.
  const T* qg = reinterpret_cast<const T*>(a.q);
  vec qf[MT][D / 32];
  int blk_row[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = rg * kRowsPerGroup + 16 * t + n;
    const int i = r / a.g, hl = r - i * a.g;
    blk_row[t] = i;
    const int rr = r < a.M ? r : 0;
    const int ii = rr / a.g, hh = rr - ii * a.g;
    const T* src = qg + ((size_t)(b * a.B + ii) * a.Hq + kvh * a.g + hh) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      qf[t][c] = Frag<T>::load(src + 32 * c);
      if (r >= a.M) qf[t][c] = Frag<T>::zero();
    }
    (void)hl;
  }

  floatx4 acc[D / 16][MT];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[dt][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[MT], l_run[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    m_run[t] = kNegBig;
    l_run[t] = 0.f;
  }

  // ---- context steps: no mask, no bounds; two per trip so the prefetch
  // buffers alternate without register copies
  StepFrags<T, D> fa, fb;
  int st = s_lo + kw;
  if (st < s_full) load_step<T, D, false>(fa, kv, a, st * kStep, n_keys, lane);
  for (; st < s_full; st += 2 * KW) {
    if (st + KW < s_full) load_step<T, D, false>(fb, kv, a, (st + KW) * kStep, n_keys, lane);
    compute_step<T, D, MT, false>(fa, qf, acc, m_run, l_run, blk_row, a, st * kStep, L, n_keys,
                                  nc, grp);
    if (st + KW >= s_full) {
      st += KW;
      break;
    }
    if (st + 2 * KW < s_full) load_step<T, D, false>(fa, kv, a, (st + 2 * KW) * kStep, n_keys, lane);
    compute_step<T, D, MT, false>(fb, qf, acc, m_run, l_run, blk_row, a, (st + KW) * kStep, L,
                                  n_keys, nc, grp);
  }
  // ---- steps that reach the block or the end of the sequence
  for (; st < s_hi; st += KW) {
    load_step<T, D, true>(fa, kv, a, st * kStep, n_keys, lane);
    compute_step<T, D, MT, true>(fa, qf, acc, m_run, l_run, blk_row, a, st * kStep, L, n_keys,
                                 nc, grp);
  }

  // ---- merge the key waves of each row group through LDS (fixed order)
  constexpr int kOStride = D + 4;  // padded row stride (floats)
  __shared__ float s_ml[RG][KW][kRowsPerGroup][2];
  __shared__ float s_o[RG][kRowsPerGroup * kOStride];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    l_run[t] = group_sum4(l_run[t]);
    if (grp == 0) {
      s_ml[rg][kw][16 * t + n][0] = m_run[t];
      s_ml[rg][kw][16 * t + n][1] = l_run[t];
    }
  }
  __syncthreads();
  float m_tot[MT], l_tot[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < KW; ++w) mm = fmaxf(mm, s_ml[rg][w][16 * t + n][0]);
    float ll = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w)
      ll += s_ml[rg][w][16 * t + n][1] * __builtin_amdgcn_exp2f(s_ml[rg][w][16 * t + n][0] - mm);
    m_tot[t] = mm;
    l_tot[t] = ll;
    const float f = __builtin_amdgcn_exp2f(m_run[t] - mm);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt][t] *= f;
  }
  float* so = s_o[rg];
#pragma unroll
  for (int w = KW - 1; w >= 1; --w) {
    if (kw == w) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          floatx4* p = reinterpret_cast<floatx4*>(so + (16 * t + n) * kOStride + 16 * dt + 4 * grp);
          if (w < KW - 1) acc[dt][t] += *p;
          *p = acc[dt][t];
        }
    }
    __syncthreads();
  }

  const bool single = a.splits == 1;
  if (kw == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = rg * kRowsPerGroup + 16 * t + n;
      if (r >= a.M) continue;
      if (KW > 1) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          acc[dt][t] += *reinterpret_cast<floatx4*>(so + (16 * t + n) * kOStride + 16 * dt + 4 * grp);
      }
      const int i = r / a.g, hl = r - i * a.g;
      const size_t orow = (size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl;
      if (single) {
        const float inv = 1.0f / l_tot[t];
        T* dst = reinterpret_cast<T*>(a.o) + orow * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) Frag<T>::store4(dst + 16 * dt, acc[dt][t] * inv);
        if (a.lse && grp == 0) a.lse[orow] = (m_tot[t] + __log2f(l_tot[t])) * kLn2;
      } else {
        const size_t prow = ((size_t)blockIdx.x * a.M + r);
        float* dst = a.part_o + prow * D + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(dst + 16 * dt) = acc[dt][t];
        if (grp == 0) {
          a.part_ml[prow * 2 + 0] = m_tot[t];
          a.part_ml[prow * 2 + 1] = l_tot[t];
        }
      }
    }
  }
  if (single) return;

  // ---- split-KV merge by the last workgroup of this (request, KV head)
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&a.counters[unit], 1);
    s_last = prev == a.splits - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // per-row merge weights in LDS (reuses s_o): w[r][s], then 1/L per row
  float* wts = &s_o[0][0];
  const int S = a.splits;
  const size_t part0 = (size_t)unit * S;
  for (int r = tid; r < a.M; r += blockDim.x) {
    float mm = kNegBig;
    for (int s2 = 0; s2 < S; ++s2) mm = fmaxf(mm, a.part_ml[((part0 + s2) * a.M + r) * 2]);
    float ll = 0.f;
    for (int s2 = 0; s2 < S; ++s2) {
      const size_t pr = (part0 + s2) * a.M + r;
      const float w = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - mm);
      wts[r * (S + 1) + s2] = w;
      ll += w * a.part_ml[pr * 2 + 1];
    }
    wts[r * (S + 1) + S] = 1.0f / ll;
    if (a.lse) {
      const int i = r / a.g, hl = r - i * a.g;
      a.lse[(size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl] = (mm + __log2f(ll)) * kLn2;
    }
  }
  __syncthreads();
  const int n4 = a.M * (D / 4);
  for (int e = tid; e < n4; e += blockDim.x) {
    const int r = e / (D / 4), d4 = e - r * (D / 4);
    floatx4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2)
      sum += wts[r * (S + 1) + s2] *
             *reinterpret_cast<const floatx4*>(a.part_o + ((part0 + s2) * a.M + r) * D + 4 * d4);
    sum *= wts[r * (S + 1) + S];
    const int i = r / a.g, hl = r - i * a.g;
    T* dst = reinterpret_cast<T*>(a.o) + ((size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl) * D + 4 * d4;
    Frag<T>::store4(dst, sum);
  }
  if (tid == 0) a.counters[unit] = 0;
}

// ------------------------------------------------------------------ launch
template <typename T, int D>
static hipError_t launch_dt(const AttnArgs& a, int total_blocks, hipStream_t stream) {
  const int rows_wave = a.M > kRowsPerGroup ? kRowsPerGroup : a.M;
  const int mt = (rows_wave + 15) / 16;
  const int rg = (a.M + kRowsPerGroup - 1) / kRowsPerGroup;
  dim3 grid(total_blocks);
  if (rg == 2) {
    hipLaunchKernelGGL((block_attn_kernel<T, D, 4, 2>), grid, dim3(kWave * 4), 0, stream, a);
  } else {
    dim3 block(kWave * 4);
    switch (mt) {
      case 1: hipLaunchKernelGGL((block_attn_kernel<T, D, 1, 1>), grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL((block_attn_kernel<T, D, 2, 1>), grid, block, 0, stream, a); break;
      case 3: hipLaunchKernelGGL((block_attn_kernel<T, D, 3, 1>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((block_attn_kernel<T, D, 4, 1>), grid, block, 0, stream, a); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_block_attn(const AttnArgs& a, bool bf16, int D, int total_blocks,
                             hipStream_t stream) {
  if (bf16) {
    return D == 64 ? launch_dt<__bf16, 64>(a, total_blocks, stream)
                   : launch_dt<__bf16, 128>(a, total_blocks, stream);
  }
  return D == 64 ? launch_dt<float, 64>(a, total_blocks, stream)
                 : launch_dt<float, 128>(a, total_blocks, stream);
}

}  // namespace specattn
