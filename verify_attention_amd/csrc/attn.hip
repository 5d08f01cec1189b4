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
// Work decomposition: one 4-wave workgroup per (request, KV head, split).
//   * All g * B query rows that share a KV head (the GQA group's query heads
//     times the block tokens) are the MFMA N dimension, so each K/V page is
//     read from HBM once per KV head. Wave w owns 16 (or 32) of those rows.
//   * The split's keys stream through in 32-key stages. For each stage the 4
//     waves together issue the 16-byte loads of every MFMA operand fragment
//     (each wave a quarter), keep three stages in flight in registers, and
//     write each fragment to LDS in the lane order its MFMA consumes it, so
//     every wave then reads whole fragments with conflict-free ds_read_b128.
//     Three LDS stage buffers, one barrier per stage.
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16
//     (eight v_mfma_f32_16x16x4f32 for fp32 inputs). Keys are permuted inside
//     a stage so that the accumulator layout of S^T is directly the B operand
//     of the PV product and the dim-major V page gives the A operand as one
//     contiguous 16-byte run: no shuffles between the two products.
//   * Online softmax in fp32 (exp2 domain), row max across the 4 lane groups
//     via permlane swaps, lazy rescaling (the reference max only moves when a
//     new max exceeds it by 2^8), masks applied only on stages that reach the
//     block; keys past the sequence end are zeroed by the loading wave.
//   * With several splits per (request, KV head) each workgroup stores its
//     partial state and a second, small kernel merges the splits (a kernel
//     boundary instead of device-scope fences, which on gfx950 write back and
//     invalidate the L2 of the issuing XCD).
#include "kernels.h"

namespace specattn {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite start value for running maxima
constexpr float kRescale = 8.0f;      // lazy rescale threshold, log2 units
constexpr int kStep = 32;             // keys per stage
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kPageWin = 1024;        // page ids staged in LDS per window

typedef int intx4 __attribute__((ext_vector_type(4)));

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

// Fragments of one stage as the MFMAs consume them.
template <typename T, int D>
struct StepFrags {
  typename Frag<T>::vec k[2][D / 32];  // A operands of S^T = K Q^T, two 16-key tiles
  typename Frag<T>::vec v[D / 16];     // A operands of O^T += V^T P^T, one per 16-dim tile
};

// A stage is NP pieces of 1 KB (64 lanes x 16 bytes): the K fragments first,
// then the V fragments; a fragment is H = sizeof(T)/2 pieces. Wave w loads
// K pieces w, w+4, ... and V pieces w, w+4, ... of every stage.
template <typename T, int D>
struct StageShape {
  static constexpr int H = sizeof(T) / 2;
  static constexpr int KC = D / 32;           // K chunks along D per key tile
  static constexpr int NKP = 2 * KC * H;      // K pieces
  static constexpr int NVP = (D / 16) * H;    // V pieces
  static constexpr int KPW = NKP / kWaves;    // K pieces per wave
  static constexpr int VPW = NVP / kWaves;    // V pieces per wave
  static constexpr int PW = KPW + VPW;
  static constexpr int BYTES = (NKP + NVP) * 1024;
  typedef intx4 Regs[PW];  // one stage's pieces held by one wave
  static_assert(NKP % kWaves == 0 && NVP % kWaves == 0, "pieces must split over 4 waves");
};

struct KvView {
  const char* kbase;    // k_pool + kvh * P * D elements
  const char* vbase;    // v_pool + kvh * P * D elements
  size_t page_bytes;    // bytes per physical page (all KV heads)
};

// Loads this wave's pieces of the stage at key0 (pages page_lo for keys 0..15
// or all keys when P = 32, page_hi for keys 16..31). Lane (n, grp):
//   K piece (tile T, chunk c, half h): key key0 + 8*(n/4) + 4*T + n%4,
//     dims 32c + 8*grp + 4h (bf16: h = 0, 8 dims; fp32: 4 dims per half)
//   V piece (dim tile dt, half h): dim 16*dt + n, keys key0 + 8*grp + 4h ...
// Keys at or past n_keys are read from the stage's first slot instead (their
// own slots may hold anything, or not exist); store_stage zeroes them. One
// branch-free path, so the loads stay in flight until the data is stored.
template <typename T, int D>
__device__ __forceinline__ void load_stage(typename StageShape<T, D>::Regs& r, const KvView& kv,
                                           int P, int key0, int page_lo, int page_hi,
                                           int n_keys, int wave, int lane) {
  using SS = StageShape<T, D>;
  const int n = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < SS::KPW; ++j) {
    const int piece = wave + kWaves * j;
    const int f = piece / SS::H, h = piece % SS::H;
    const int t2 = f / SS::KC, c = f % SS::KC;
    const int kk = 8 * (n >> 2) + 4 * t2 + (n & 3);
    const int kq = key0 + kk < n_keys ? kk : 0;
    const int page = (P == 16 && kq >= 16) ? page_hi : page_lo;
    const size_t off = (size_t)page * kv.page_bytes +
                       (size_t)(((key0 + kq) & (P - 1)) * D + 32 * c + 8 * grp + 4 * h) * sizeof(T);
    r[j] = *reinterpret_cast<const intx4*>(kv.kbase + off);
  }
#pragma unroll
  for (int j = 0; j < SS::VPW; ++j) {
    const int piece = wave + kWaves * j;
    const int dt = piece / SS::H, h = piece % SS::H;
    const int kk = 8 * grp + 4 * h;
    const int kq = key0 + kk < n_keys ? kk : 0;
    const int page = (P == 16 && kq >= 16) ? page_hi : page_lo;
    const size_t off = (size_t)page * kv.page_bytes +
                       (size_t)((16 * dt + n) * P + ((key0 + kq) & (P - 1))) * sizeof(T);
    r[SS::KPW + j] = *reinterpret_cast<const intx4*>(kv.vbase + off);
  }
}

// Writes this wave's pieces to an LDS stage buffer at the positions the MFMA
// lanes read them from; on the stage that crosses n_keys the pieces (or
// elements) of keys past the end are zeroed first.
template <typename T, int D>
__device__ __forceinline__ void store_stage(typename StageShape<T, D>::Regs& r, char* buf, int key0,
                                            int n_keys, int wave, int lane) {
  using SS = StageShape<T, D>;
  constexpr int E = 16 / sizeof(T);  // elements per piece
  const int n = lane & 15, grp = lane >> 4;
  if (key0 + kStep > n_keys) {
#pragma unroll
    for (int j = 0; j < SS::KPW; ++j) {
      const int piece = wave + kWaves * j;
      const int t2 = (piece / SS::H) / SS::KC;
      if (key0 + 8 * (n >> 2) + 4 * t2 + (n & 3) >= n_keys) r[j] = intx4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < SS::VPW; ++j) {
      const int h = (wave + kWaves * j) % SS::H;
      const int k0 = key0 + 8 * grp + 4 * h;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (k0 + e >= n_keys) {
          if (sizeof(T) == 4) r[SS::KPW + j][e] = 0;
          else r[SS::KPW + j][e / 2] &= (e & 1) ? 0x0000ffff : (int)0xffff0000;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < SS::KPW; ++j)
    *reinterpret_cast<intx4*>(buf + (wave + kWaves * j) * 1024 + lane * 16) = r[j];
#pragma unroll
  for (int j = 0; j < SS::VPW; ++j)
    *reinterpret_cast<intx4*>(buf + (SS::NKP + wave + kWaves * j) * 1024 + lane * 16) = r[SS::KPW + j];
}

// Fragment starting at piece p0: one 16-byte piece (bf16) or two (fp32).
template <typename T>
__device__ __forceinline__ typename Frag<T>::vec read_frag(const char* buf, int p0, int lane);

template <>
__device__ __forceinline__ bf16x8 read_frag<__bf16>(const char* buf, int p0, int lane) {
  return *reinterpret_cast<const bf16x8*>(buf + p0 * 1024 + lane * 16);
}

template <>
__device__ __forceinline__ floatx8 read_frag<float>(const char* buf, int p0, int lane) {
  const floatx4 lo = *reinterpret_cast<const floatx4*>(buf + p0 * 1024 + lane * 16);
  const floatx4 hi = *reinterpret_cast<const floatx4*>(buf + (p0 + 1) * 1024 + lane * 16);
  return floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename T, int D>
__device__ __forceinline__ void read_stage(StepFrags<T, D>& f, const char* buf, int lane) {
  using SS = StageShape<T, D>;
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int c = 0; c < SS::KC; ++c) f.k[t2][c] = read_frag<T>(buf, (t2 * SS::KC + c) * SS::H, lane);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = read_frag<T>(buf, SS::NKP + dt * SS::H, lane);
}

// One stage: S^T = K Q^T, (mask), online softmax update, O^T += V^T P^T.
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

template <typename T, int D, int MT>
struct WaveState {
  typename Frag<T>::vec qf[MT][D / 32];
  floatx4 acc[D / 16][MT];
  float m_run[MT], l_run[MT];
  int blk_row[MT];
};

// Consumes stage key0 from LDS buffer buf.
template <typename T, int D, int MT>
__device__ __forceinline__ void consume(WaveState<T, D, MT>& ws, const char* buf, const AttnArgs& a,
                                        int key0, int L, int n_keys, int nc, int lane,
                                        bool has_rows) {
  if (!has_rows) return;
  StepFrags<T, D> f;
  read_stage<T, D>(f, buf, lane);
  if (key0 + kStep > L)
    compute_step<T, D, MT, true>(f, ws.qf, ws.acc, ws.m_run, ws.l_run, ws.blk_row, a, key0, L,
                                 n_keys, nc, lane >> 4);
  else
    compute_step<T, D, MT, false>(f, ws.qf, ws.acc, ws.m_run, ws.l_run, ws.blk_row, a, key0, L,
                                  n_keys, nc, lane >> 4);
}

template <typename T, int D>
__device__ __forceinline__ void issue(typename StageShape<T, D>::Regs& r, const KvView& kv,
                                      const AttnArgs& a, const int* s_pages, int pg0, int key0,
                                      int n_keys, int wave, int lane) {
  const int idx = (key0 >> a.p_shift) - pg0;
  const int page_lo = s_pages[idx];
  const int page_hi = (a.P == 16 && key0 + 16 < n_keys) ? s_pages[idx + 1] : page_lo;
  load_stage<T, D>(r, kv, a.P, key0, page_lo, page_hi, n_keys, wave, lane);
}

template <typename T, int D, int MT>
__global__ __launch_bounds__(kWave * kWaves, (MT == 1 ? 2 : 1)) void block_attn_kernel(AttnArgs a) {
  using SS = StageShape<T, D>;
  __shared__ __attribute__((aligned(16))) char s_buf[3][SS::BYTES];
  __shared__ int s_pages[kPageWin];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  KvView kv;
  kv.kbase = reinterpret_cast<const char*>(a.k) + (size_t)kvh * a.P * D * sizeof(T);
  kv.vbase = reinterpret_cast<const char*>(a.v) + (size_t)kvh * a.P * D * sizeof(T);
  kv.page_bytes = (size_t)a.P * D * a.Hkv * sizeof(T);
  const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;

  // ---- Q^T operands of this wave's rows: lane (n, grp) holds row 16t + n,
  // dims 32c + 8*grp .. +7. Row r of the group is block token r / g, query
  // head kvh * g + r % g.
  WaveState<T, D, MT> ws;
  const int row0 = wave * 16 * MT;
  const bool has_rows = row0 < a.M;
  const T* qg = reinterpret_cast<const T*>(a.q);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = row0 + 16 * t + n;
    ws.blk_row[t] = r / a.g;
    const int rr = r < a.M ? r : 0;
    const int ii = rr / a.g, hh = rr - ii * a.g;
    const T* src = qg + ((size_t)(b * a.B + ii) * a.Hq + kvh * a.g + hh) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      ws.qf[t][c] = Frag<T>::load(src + 32 * c);
      if (r >= a.M) ws.qf[t][c] = Frag<T>::zero();
    }
    ws.m_run[t] = kNegBig;
    ws.l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) ws.acc[dt][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- stream the split's stages, one window of staged page ids at a time
  const int win_steps = kPageWin * a.P / kStep;
  for (int w0 = s_lo; w0 < s_hi; w0 += win_steps) {
    const int w1 = min(s_hi, w0 + win_steps);
    const int pg0 = (w0 * kStep) >> a.p_shift;
    const int npg = ((min(w1 * kStep, n_keys) - 1) >> a.p_shift) - pg0 + 1;
    __syncthreads();  // the previous window is fully consumed
    for (int x = tid; x < npg; x += kWave * kWaves) {
      const int p = ptab[pg0 + x];
      const bool bad = (unsigned)p >= (unsigned)a.num_pages;
      if (bad) flag_error(a.err, kErrSlot);
      s_pages[x] = bad ? 0 : p;
    }
    __syncthreads();

    const int ns = w1 - w0;
    typename SS::Regs r0, r1, r2;
    // one pipeline step: load stage t + 3, consume stage t, stage t + 1 to LDS
    auto step = [&](typename SS::Regs& r_issue, char* b_cons, typename SS::Regs& r_store,
                    char* b_store, int t, bool do_issue, bool do_store) {
      if (do_issue) issue<T, D>(r_issue, kv, a, s_pages, pg0, (w0 + t + 3) * kStep, n_keys, wave, lane);
      consume<T, D, MT>(ws, b_cons, a, (w0 + t) * kStep, L, n_keys, nc, lane, has_rows);
      if (do_store) store_stage<T, D>(r_store, b_store, (w0 + t + 1) * kStep, n_keys, wave, lane);
      __syncthreads();
    };
    issue<T, D>(r0, kv, a, s_pages, pg0, w0 * kStep, n_keys, wave, lane);
    if (ns > 1) issue<T, D>(r1, kv, a, s_pages, pg0, (w0 + 1) * kStep, n_keys, wave, lane);
    if (ns > 2) issue<T, D>(r2, kv, a, s_pages, pg0, (w0 + 2) * kStep, n_keys, wave, lane);
    store_stage<T, D>(r0, s_buf[0], w0 * kStep, n_keys, wave, lane);
    __syncthreads();
    // steady state: three stages per trip with static register-set / buffer
    // indices and no conditions, so every load stays in flight until its
    // data is written to LDS two steps later
    int t = 0;
    for (; t + 6 <= ns; t += 3) {
      step(r0, s_buf[0], r1, s_buf[1], t, true, true);
      step(r1, s_buf[1], r2, s_buf[2], t + 1, true, true);
      step(r2, s_buf[2], r0, s_buf[0], t + 2, true, true);
    }
    // the last (at most five) stages
    if (t < ns) step(r0, s_buf[0], r1, s_buf[1], t, t + 3 < ns, t + 1 < ns);
    if (t + 1 < ns) step(r1, s_buf[1], r2, s_buf[2], t + 1, t + 4 < ns, t + 2 < ns);
    if (t + 2 < ns) step(r2, s_buf[2], r0, s_buf[0], t + 2, false, t + 3 < ns);
    if (t + 3 < ns) step(r0, s_buf[0], r1, s_buf[1], t + 3, false, t + 4 < ns);
    if (t + 4 < ns) step(r1, s_buf[1], r2, s_buf[2], t + 4, false, false);
  }

  // ---- this wave's rows: normalise and write, or store the split's partial state
  if (!has_rows) return;
  const bool single = a.splits == 1;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float l_tot = group_sum4(ws.l_run[t]);
    const int r = row0 + 16 * t + n;
    if (r >= a.M) continue;
    const int i = r / a.g, hl = r - i * a.g;
    const size_t orow = (size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl;
    if (single) {
      const float inv = 1.0f / l_tot;
      T* dst = reinterpret_cast<T*>(a.o) + orow * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) Frag<T>::store4(dst + 16 * dt, ws.acc[dt][t] * inv);
      if (a.lse && grp == 0) a.lse[orow] = (ws.m_run[t] + __log2f(l_tot)) * kLn2;
    } else {
      const size_t prow = ((size_t)blockIdx.x * a.M + r);
      float* dst = a.part_o + prow * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(dst + 16 * dt) = ws.acc[dt][t];
      if (grp == 0) {
        a.part_ml[prow * 2 + 0] = ws.m_run[t];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// Split-KV merge: O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^(m_s - max m),
// one workgroup per (request, KV head), a separate launch after the splits.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_attn_combine_kernel(AttnArgs a) {
  const int unit = blockIdx.x;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int S = a.splits;
  const size_t part0 = (size_t)unit * S;
  __shared__ float wts[128 * 65];  // M <= 128 rows x (splits <= 64, + 1/L)
  for (int r = threadIdx.x; r < a.M; r += blockDim.x) {
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
  for (int e = threadIdx.x; e < n4; e += blockDim.x) {
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
}

// ------------------------------------------------------------------ launch
template <typename T, int D>
static hipError_t launch_dt(const AttnArgs& a, int total_blocks, hipStream_t stream) {
  const dim3 grid(total_blocks), block(kWave * kWaves);
  if (a.M > 64)
    hipLaunchKernelGGL((block_attn_kernel<T, D, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((block_attn_kernel<T, D, 1>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((block_attn_combine_kernel<T, D>), dim3(a.bs * a.Hkv), dim3(256), 0, stream, a);
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
