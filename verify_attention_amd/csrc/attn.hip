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
//     waves together issue the 16-byte global->LDS DMA loads
//     (global_load_lds_dwordx4) of every MFMA operand fragment, each wave a
//     quarter, placing each fragment in the lane order its MFMA consumes it;
//     every wave then reads whole fragments with conflict-free ds_read_b128.
//     An LDS ring of 64 KB (two workgroups per CU, 3 stages in flight each)
//     or 128 KB (one workgroup, 7 stages) keeps stages in flight without
//     holding them in registers; hand-counted vmcnt waits and one barrier per
//     stage.
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

// 16 zero bytes: the DMA source for lanes whose key lies past the sequence end.
__device__ __attribute__((aligned(64))) int g_zero16[16];

constexpr int wait_vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// s_waitcnt vmcnt(per * m) for a small runtime m (the immediate must be static).
template <int PER>
__device__ __forceinline__ void wait_stages(int m) {
  switch (m) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm_imm(PER)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm_imm(2 * PER)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm_imm(3 * PER)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vm_imm(4 * PER)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vm_imm(5 * PER)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm_imm(6 * PER)); break;
  }
}

// Per-lane constants of this wave's DMA pieces. A stage starts on a page
// boundary (32 keys, P in {16, 32}), so the slot of a lane's key inside its
// page, and whether that page is the stage's first or second, never change.
template <typename T, int D>
struct DmaLanes {
  using SS = StageShape<T, D>;
  uint32_t off[SS::PW];  // byte offset inside the (page, KV head) tile
  int key[SS::PW];       // first key of the piece inside the stage
  bool hi[SS::PW];       // the key lies in the stage's second page (P = 16)
  uint32_t lds[SS::PW];  // piece offset inside a ring slot
};

template <typename T, int D>
__device__ __forceinline__ DmaLanes<T, D> dma_lanes(int P, int wave, int lane) {
  using SS = StageShape<T, D>;
  DmaLanes<T, D> d;
  const int n = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < SS::KPW; ++j) {
    const int piece = wave + kWaves * j;
    const int f = piece / SS::H, h = piece % SS::H;
    const int t2 = f / SS::KC, c = f % SS::KC;
    const int kk = 8 * (n >> 2) + 4 * t2 + (n & 3);
    d.key[j] = kk;
    d.hi[j] = P == 16 && kk >= 16;
    d.off[j] = (uint32_t)(((kk & (P - 1)) * D + 32 * c + 8 * grp + 4 * h) * sizeof(T));
    d.lds[j] = piece * 1024;
  }
#pragma unroll
  for (int j = 0; j < SS::VPW; ++j) {
    const int piece = wave + kWaves * j;
    const int dt = piece / SS::H, h = piece % SS::H;
    const int kk = 8 * grp + 4 * h;
    d.key[SS::KPW + j] = kk;
    d.hi[SS::KPW + j] = P == 16 && kk >= 16;
    d.off[SS::KPW + j] = (uint32_t)(((16 * dt + n) * P + (kk & (P - 1))) * sizeof(T));
    d.lds[SS::KPW + j] = (SS::NKP + piece) * 1024;
  }
  return d;
}

// Issues this wave's pieces of one stage as LDS DMA loads into a ring slot:
// the K/V tiles of the stage's two pages (one when P = 32) start at k_lo/k_hi
// and v_lo/v_hi. Each piece lands at slot + piece * 1024 + lane * 16, the
// position from which the MFMA lane that consumes it reads. TAIL: lanes whose
// first key lies at or past n_keys load zeros instead; a V piece that
// straddles n_keys is masked by its reader.
template <typename T, int D, bool TAIL>
__device__ __forceinline__ void issue_dma(char* slot, const DmaLanes<T, D>& dl, const char* k_lo,
                                          const char* k_hi, const char* v_lo, const char* v_hi,
                                          int key0, int n_keys) {
  using SS = StageShape<T, D>;
#pragma unroll
  for (int j = 0; j < SS::PW; ++j) {
    const bool is_k = j < SS::KPW;
    const char* base = is_k ? (dl.hi[j] ? k_hi : k_lo) : (dl.hi[j] ? v_hi : v_lo);
    const char* src = base + dl.off[j];
    if (TAIL && key0 + dl.key[j] >= n_keys) src = reinterpret_cast<const char*>(g_zero16);
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(slot + dl.lds[j]), 16, 0, 0);
  }
}

// Sixteen 16-byte pieces P0 .. P0+15 of a ring slot (lane-relative address
// `addr`) behind one s_waitcnt. Inline asm keeps the compiler's LDS-DMA
// tracking from inserting a wait for every DMA still in flight.
template <int P0>
__device__ __forceinline__ void read16(intx4* o, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:%17\n\t"
      "ds_read_b128 %1, %16 offset:%18\n\t"
      "ds_read_b128 %2, %16 offset:%19\n\t"
      "ds_read_b128 %3, %16 offset:%20\n\t"
      "ds_read_b128 %4, %16 offset:%21\n\t"
      "ds_read_b128 %5, %16 offset:%22\n\t"
      "ds_read_b128 %6, %16 offset:%23\n\t"
      "ds_read_b128 %7, %16 offset:%24\n\t"
      "ds_read_b128 %8, %16 offset:%25\n\t"
      "ds_read_b128 %9, %16 offset:%26\n\t"
      "ds_read_b128 %10, %16 offset:%27\n\t"
      "ds_read_b128 %11, %16 offset:%28\n\t"
      "ds_read_b128 %12, %16 offset:%29\n\t"
      "ds_read_b128 %13, %16 offset:%30\n\t"
      "ds_read_b128 %14, %16 offset:%31\n\t"
      "ds_read_b128 %15, %16 offset:%32\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]),
        "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(addr), "i"(P0 * 1024), "i"((P0 + 1) * 1024), "i"((P0 + 2) * 1024),
        "i"((P0 + 3) * 1024), "i"((P0 + 4) * 1024), "i"((P0 + 5) * 1024), "i"((P0 + 6) * 1024),
        "i"((P0 + 7) * 1024), "i"((P0 + 8) * 1024), "i"((P0 + 9) * 1024),
        "i"((P0 + 10) * 1024), "i"((P0 + 11) * 1024), "i"((P0 + 12) * 1024),
        "i"((P0 + 13) * 1024), "i"((P0 + 14) * 1024), "i"((P0 + 15) * 1024)
      : "memory");
}

// Eight pieces, for stages of eight pieces (bf16, 64 dims).
template <int P0>
__device__ __forceinline__ void read8(intx4* o, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(addr), "i"(P0 * 1024), "i"((P0 + 1) * 1024), "i"((P0 + 2) * 1024),
        "i"((P0 + 3) * 1024), "i"((P0 + 4) * 1024), "i"((P0 + 5) * 1024), "i"((P0 + 6) * 1024),
        "i"((P0 + 7) * 1024)
      : "memory");
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::vec frag_of(const intx4* pc);

template <>
__device__ __forceinline__ bf16x8 frag_of<__bf16>(const intx4* pc) {
  return __builtin_bit_cast(bf16x8, pc[0]);
}

template <>
__device__ __forceinline__ floatx8 frag_of<float>(const intx4* pc) {
  const floatx4 lo = __builtin_bit_cast(floatx4, pc[0]);
  const floatx4 hi = __builtin_bit_cast(floatx4, pc[1]);
  return floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// All fragments of a ring slot; on the stage that crosses n_keys the V
// elements of keys past the end are zeroed (their slots may hold anything).
template <typename T, int D>
__device__ __forceinline__ void read_stage(StepFrags<T, D>& f, unsigned addr, int key0,
                                           int n_keys, int lane) {
  using SS = StageShape<T, D>;
  constexpr int NP = SS::NKP + SS::NVP;
  static_assert(NP == 8 || NP == 16 || NP == 32, "stage piece counts");
  intx4 pc[NP];
  if constexpr (NP == 8) {
    read8<0>(pc, addr);
  } else {
    read16<0>(pc, addr);
    if constexpr (NP == 32) read16<16>(pc + 16, addr);
  }
  if (key0 + kStep > n_keys) {
    const int grp = lane >> 4;
    constexpr int E = 16 / sizeof(T);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int h = 0; h < SS::H; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (key0 + 8 * grp + 4 * h + e >= n_keys) {
            intx4& x = pc[SS::NKP + dt * SS::H + h];
            if (sizeof(T) == 4) x[e] = 0;
            else x[e / 2] &= (e & 1) ? 0x0000ffff : (int)0xffff0000;
          }
        }
  }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int c = 0; c < SS::KC; ++c) f.k[t2][c] = frag_of<T>(pc + (t2 * SS::KC + c) * SS::H);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = frag_of<T>(pc + SS::NKP + dt * SS::H);
}

// One stage: S^T = K Q^T, (mask), online softmax update, O^T += V^T P^T.
// s[T][t][j] is key key0 + 8*grp + 4*T + j against row 16t + n of the wave;
// softmax runs in the exp2 domain with the scale folded into the exponent.
template <typename T, int D, int MT>
__device__ __forceinline__ void compute_step(const StepFrags<T, D>& f,
                                             const typename Frag<T>::vec (&qf)[MT][D / 32],
                                             floatx4 (&acc)[D / 16][MT], float (&m_run)[MT],
                                             float (&l_run)[MT], const int (&blk_row)[MT],
                                             const AttnArgs& a, int key0, int L, int n_keys,
                                             int nc, int grp, bool masked) {
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

  if (masked) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + 8 * grp + 4 * t2 + j;
          const int jb = key - L, i = blk_row[t];
          const bool vis = (key < L) | ((key < n_keys) & ((a.mode == 0) | (jb <= i) | ((a.mode == 2) & (i >= nc))));
          s[t2][t][j] = vis ? s[t2][t][j] : -__builtin_inff();
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

// Consumes the stage at key0 from the ring slot at lane-relative LDS address addr.
template <typename T, int D, int MT>
__device__ __forceinline__ void consume(WaveState<T, D, MT>& ws, unsigned addr, const AttnArgs& a,
                                        int key0, int L, int n_keys, int nc, int lane,
                                        bool has_rows) {
  if (!has_rows) return;
  StepFrags<T, D> f;
  read_stage<T, D>(f, addr, key0, n_keys, lane);
  compute_step<T, D, MT>(f, ws.qf, ws.acc, ws.m_run, ws.l_run, ws.blk_row, a, key0, L, n_keys,
                         nc, lane >> 4, key0 + kStep > L);
}

// RING_KB: LDS for the stage ring; its depth NS = RING_KB KB / stage bytes
// (at most 8) sets how many stages are in flight (NS - 1).
template <typename T, int D, int MT, int RING_KB>
__global__ __launch_bounds__(kWave * kWaves, (MT == 1 ? 2 : 1)) void block_attn_kernel(AttnArgs a) {
  using SS = StageShape<T, D>;
  constexpr int NS = RING_KB * 1024 / SS::BYTES < 8 ? RING_KB * 1024 / SS::BYTES : 8;
  static_assert(NS >= 3, "the ring needs at least three stages");
  __shared__ __attribute__((aligned(16))) char s_ring[NS * SS::BYTES];
  __shared__ __attribute__((aligned(8))) int s_pages[kPageWin];

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
  const int win_steps = kPageWin / 2;  // (lo, hi) page pairs per window
  const DmaLanes<T, D> dl = dma_lanes<T, D>(a.P, wave, lane);
  for (int w0 = s_lo; w0 < s_hi; w0 += win_steps) {
    const int w1 = min(s_hi, w0 + win_steps);
    __syncthreads();  // the previous window is fully consumed
    // (lo, hi) physical pages of every stage of the window; hi = lo when the
    // stage has one page (P = 32) or its second page lies past the sequence
    for (int x = tid; x < 2 * (w1 - w0); x += kWave * kWaves) {
      const int key = (w0 + (x >> 1)) * kStep + (x & 1) * 16;
      const bool second = (x & 1) && a.P == 16 && key < n_keys;
      const int p = ptab[(second ? key : (key & ~31)) >> a.p_shift];
      const bool bad = (unsigned)p >= (unsigned)a.num_pages;
      if (bad) flag_error(a.err, kErrSlot);
      s_pages[x] = bad ? 0 : p;
    }
    // Q and the page ids are in: from here on the only vector-memory loads in
    // flight are the ring's DMAs, which the waits below count by hand
    __builtin_amdgcn_s_waitcnt(wait_vm_imm(0));
    __syncthreads();

    const int ns = w1 - w0;
    const unsigned ring_lane = (unsigned)(size_t)s_ring + (unsigned)lane * 16;
    // pages of stage t: s_pages[2t'] / [2t'+1] hold (lo, hi) of window stage t'
    auto issue = [&](int t, int2 pg) {
      const int key0 = (w0 + t) * kStep;
      const char* k_lo = kv.kbase + (size_t)pg.x * kv.page_bytes;
      const char* k_hi = kv.kbase + (size_t)pg.y * kv.page_bytes;
      const char* v_lo = kv.vbase + (size_t)pg.x * kv.page_bytes;
      const char* v_hi = kv.vbase + (size_t)pg.y * kv.page_bytes;
      char* slot = s_ring + (t % NS) * SS::BYTES;
      if (key0 + kStep <= n_keys)
        issue_dma<T, D, false>(slot, dl, k_lo, k_hi, v_lo, v_hi, key0, n_keys);
      else
        issue_dma<T, D, true>(slot, dl, k_lo, k_hi, v_lo, v_hi, key0, n_keys);
    };
    auto stage_pages = [&](int t) {
      const int2 pg = reinterpret_cast<const int2*>(s_pages)[t];
      return int2{__builtin_amdgcn_readfirstlane(pg.x), __builtin_amdgcn_readfirstlane(pg.y)};
    };
    // NS - 1 stages in flight; stage t lands in ring slot t % NS. Each wave
    // waits for its own DMA share of stage t (vmcnt counts this wave's
    // loads in issue order), the barrier publishes all shares, and the slot
    // consumed one step earlier is refilled with stage t + NS - 1.
    for (int t = 0; t < NS - 1 && t < ns; ++t) issue(t, stage_pages(t));
    int2 next_pg = stage_pages(min(NS - 1, ns - 1));
    for (int t = 0; t < ns; ++t) {
      wait_stages<SS::PW>(min(NS - 2, ns - 1 - t));
      asm volatile("s_barrier" ::: "memory");
      if (t + NS - 1 < ns) issue(t + NS - 1, next_pg);
      next_pg = stage_pages(min(t + NS, ns - 1));
      consume<T, D, MT>(ws, ring_lane + (t % NS) * SS::BYTES, a, (w0 + t) * kStep, L, n_keys, nc,
                        lane, has_rows);
    }
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
template <typename T, int D, int MT>
static void launch_mt(const AttnArgs& a, dim3 grid, dim3 block, int ring_kb, hipStream_t stream) {
  // fp32 stages of 128 dims are 32 KB: only the large ring holds 3 of them
  if constexpr (sizeof(T) == 4 && D == 128) {
    hipLaunchKernelGGL((block_attn_kernel<T, D, MT, 128>), grid, block, 0, stream, a);
  } else {
    if (ring_kb >= 128)
      hipLaunchKernelGGL((block_attn_kernel<T, D, MT, 128>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((block_attn_kernel<T, D, MT, 64>), grid, block, 0, stream, a);
  }
}

template <typename T, int D>
static hipError_t launch_dt(const AttnArgs& a, int total_blocks, int ring_kb, hipStream_t stream) {
  const dim3 grid(total_blocks), block(kWave * kWaves);
  if (a.M > 64)
    launch_mt<T, D, 2>(a, grid, block, ring_kb, stream);
  else
    launch_mt<T, D, 1>(a, grid, block, ring_kb, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((block_attn_combine_kernel<T, D>), dim3(a.bs * a.Hkv), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_attn(const AttnArgs& a, bool bf16, int D, int total_blocks, int ring_kb,
                             hipStream_t stream) {
  if (bf16) {
    return D == 64 ? launch_dt<__bf16, 64>(a, total_blocks, ring_kb, stream)
                   : launch_dt<__bf16, 128>(a, total_blocks, ring_kb, stream);
  }
  return D == 64 ? launch_dt<float, 64>(a, total_blocks, ring_kb, stream)
                 : launch_dt<float, 128>(a, total_blocks, ring_kb, stream);
}

}  // namespace specattn
