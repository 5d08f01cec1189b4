// block_attn: block-query attention over a paged KV cache for gfx950.
//
// The operation (see include/specattn.h): every query row of a decode-round
// block attends to the request's cached context and to the block's own K/V
// under a per-launch intra-block mask -- a rectangle for the block-diffusion
// draft pass, a triangle for the AR verify pass, and the I-DLM mixed layout
// (causal clean rows, bidirectional MASK rows) -- as drawn in the "Attention
// Mask" section of "SGLang strengthens diffusion LLMs: LLaDA 2.0" and in
// sections 4.3.1 / 4.4.1 of "From DFlash to dLLM Self-Spec (4)" -- or a
// per-row bitmask over the block keys for tree verification (the Tree
// sampler of "Unlocking Lossless Speedups in LLMs via Discrete Diffusion").
//
// Work decomposition: one 8-wave workgroup per (request, KV head, row group,
// split).
//   * All g * B query rows that share a KV head (the GQA group's query heads
//     times the block tokens) are the MFMA N dimension, so each K/V page is
//     read from HBM once per KV head; beyond 128 rows they are cut into row
//     groups (each streaming the head's keys; the groups of a head run on one
//     XCD and share them in its L2). A group's rows are cut into 4 row slots
//     of 16 (or 32 when the group has more than 64) rows; each row slot has
//     two waves, one per key half: the split's keys stream through in 32-key
//     stages taken in pairs,
//     wave set 0 consuming the even stage of a pair and set 1 the odd one.
//     The two sets' softmax states are merged through LDS at the end, so two
//     waves share every SIMD and one wave's MFMAs overlap the other's VALU.
//   * For each stage the 4 waves of its set issue the 16-byte global->LDS DMA
//     loads (global_load_lds_dwordx4) of every MFMA operand fragment, each a
//     quarter. A DMA instruction's 64 lanes all read from one page (the key
//     order inside a stage is chosen so that this holds for P = 16), so its
//     address is an SGPR page base plus a per-lane offset fixed for the whole
//     kernel. Each fragment lands where the MFMA lane that consumes it reads
//     it with one conflict-free ds_read_b128. A ring of three stage pairs
//     keeps two pairs (64 KB for bf16, 128 dims) in flight per CU; the loads
//     carry the non-temporal cache policy (the KV stream is read once), which
//     measurably raises the HBM read rate, except where a head's row groups
//     re-read its keys from L2. vmcnt waits are counted by hand and one
//     barrier per pair publishes a pair to both sets.
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16
//     (eight v_mfma_f32_16x16x4f32 for fp32 inputs). Keys are permuted inside
//     a stage so that the accumulator layout of S^T is directly the B operand
//     of the PV product and the dim-major V page gives the A operand as one
//     contiguous 16-byte run: no shuffles between the two products.
//   * Online softmax in fp32 (exp2 domain), row max (IEEE maximum) across
//     the 4 lane groups via permlane swaps, lazy rescaling (the reference max
//     only moves when a
//     new max exceeds it by 2^8), masks applied only on stages that reach the
//     block; keys past the sequence end load zeros (K) or are zeroed by the
//     reader (V).
//   * With several splits per unit (or units cut by the balanced schedule's
//     ranges) each workgroup stores its partial state and a second, small
//     kernel merges them (a kernel boundary instead of device-scope fences,
//     which on gfx950 write back and invalidate the L2 of the issuing XCD).
//   * The balanced schedule hands each workgroup a run of unit pieces. At a
//     piece boundary the next piece's page ids and Q fragments are requested
//     before the finished piece's rows are merged and stored, and the next
//     piece's first page offsets are staged during the merge; the barriers
//     there wait for LDS traffic only, so the next piece's DMAs go out while
//     the stores are still in flight.
#include "kernels.h"

namespace specattn {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite start value for running maxima
constexpr float kRescale = 8.0f;      // lazy rescale threshold, log2 units
constexpr int kStep = 32;             // keys per stage
constexpr int kRowSlots = 4;          // row slots per workgroup
constexpr int kSets = 2;              // key halves (stage parity) per row slot
constexpr int kWaves = kRowSlots * kSets;
constexpr int kRingBytes = 128 * 1024;  // ring capacity; at most 3 stage pairs are used
constexpr int kNonTemporal = 2;       // cache policy of KV loads read once (streamed)
constexpr int kTemporal = 0;          // ... and of KV loads the row-group team re-reads from L2
constexpr int kPageWin = 512;         // stages whose page offsets are staged at once

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
  static __device__ __forceinline__ void store4(float* p, floatx4 x) {
    *reinterpret_cast<floatx4*>(p) = x;
  }
};

// One stage of 32 keys as LDS pieces of 1 KB (64 lanes x 16 bytes).
//
// Key order. Inside a stage, S^T tile T (T = 0, 1) row n is key
// 8 * (n / 4) + 4 * T + n % 4, so the S^T accumulator lane (n, grp) holds keys
// 8 * grp .. 8 * grp + 7: exactly the B operand of the PV MFMA, whose A
// operand is then 8 consecutive keys of one dim-major V row. Keys 0..15 of a
// stage form half 0 and keys 16..31 half 1 (with P = 16 the two pages).
//
// K pieces. A K fragment (tile T, 32-dim chunk c, 16-byte part h2) has 64
// lanes; the 32 lanes with n < 8 read half 0 and the 32 with n >= 8 half 1.
// Fragment q = (T * KC + c) * H + h2 puts its half-h lanes into K piece
// h * NKP / 2 + q / 2, lanes 32 * (q % 2) + 8 * (grp ^ h) + n % 8, so every
// piece reads a single half. V pieces likewise: V fragment q = dt * H + h2
// (16 dims 16 dt .., 16-byte part h2) puts lane (n, grp) into V piece
// (grp / 2) * NVP / 2 + q / 2, lane 32 * (q % 2) + 16 * (grp % 2) + n. In both
// cases fragment q of a lane sits 512 * q bytes after that lane's first one.
template <typename T, int D>
struct StageShape {
  static constexpr int H = sizeof(T) / 2;        // 16-byte parts per fragment
  static constexpr int E = 16 / sizeof(T);       // elements per part
  static constexpr int KC = D / 32;              // 32-dim chunks per key
  static constexpr int NKP = 2 * KC * H;         // K pieces (= K fragments)
  static constexpr int NVP = (D / 16) * H;       // V pieces (= V fragments)
  static constexpr int KPW = NKP / kRowSlots;    // K pieces issued per wave
  static constexpr int VPW = NVP / kRowSlots;    // V pieces issued per wave
  static constexpr int PW = KPW + VPW;
  static constexpr int BYTES = (NKP + NVP) * 1024;
  static constexpr int PAIR = 2 * BYTES;
  static constexpr int NSP = kRingBytes / PAIR < 3 ? kRingBytes / PAIR : 3;  // ring depth (pairs)
  static_assert(NKP % kRowSlots == 0 && NVP % kRowSlots == 0 && KPW > 0 && VPW > 0,
                "pieces must split over the 4 waves of a set");
  static_assert(NSP >= 2, "the ring holds at least two stage pairs");
};

// 16 zero bytes: the DMA source for K lanes whose key lies past the sequence end.
__device__ __attribute__((aligned(64))) int g_zero16[16];

constexpr int wait_vm_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0) alone

// s_waitcnt vmcnt(per * m) for a small runtime m (the immediate must be
// static), then lgkmcnt(0). The lgkm wait, taken before the barrier that
// licenses a ring slot's refill, (1) completes this wave's V fragment reads
// of that slot, which set 1 leaves in flight across the barrier, and (2)
// retires the compiler-visible LDS read of the next page offsets on every
// path; left pending on any path, that read makes the compiler wait for all
// LDS reads (the in-flight V fragments included) where its registers are
// next written.
template <int PER>
__device__ __forceinline__ void wait_stages(int m) {
  switch (m) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm_imm(PER)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm_imm(2 * PER)); break;
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
}

// Per-lane constants of one wave's DMA pieces: the byte offset of the lane's
// 16 bytes inside the (page, KV head) tile and, for K pieces, the lane's key
// inside the stage. Stages start on page boundaries, so both are fixed.
template <typename T, int D>
struct DmaLanes {
  using SS = StageShape<T, D>;
  uint32_t off[SS::PW];
  int key[SS::KPW];
};

template <typename T, int D>
__device__ __forceinline__ DmaLanes<T, D> dma_lanes(int P, int r, int lane) {
  using SS = StageShape<T, D>;
  DmaLanes<T, D> d;
  const int wh = lane >> 5;
#pragma unroll
  for (int j = 0; j < SS::KPW; ++j) {
    const int p = r + kRowSlots * j;
    const int h = p / (SS::NKP / 2), q = 2 * (p % (SS::NKP / 2)) + wh;
    const int grp = ((lane >> 3) & 3) ^ h, n8 = lane & 7;
    const int h2 = q % SS::H, f = q / SS::H, t2 = f / SS::KC, c = f % SS::KC;
    const int ks = 16 * h + 8 * (n8 >> 2) + 4 * t2 + (n8 & 3);
    d.key[j] = ks;
    d.off[j] = (uint32_t)(((ks & (P - 1)) * D + 32 * c + 8 * grp + SS::E * h2) * sizeof(T));
  }
#pragma unroll
  for (int j = 0; j < SS::VPW; ++j) {
    const int p = r + kRowSlots * j;
    const int h = p / (SS::NVP / 2), q = 2 * (p % (SS::NVP / 2)) + wh;
    const int g1 = (lane >> 4) & 1, n = lane & 15;
    const int dt = q / SS::H, h2 = q % SS::H;
    const int ks = 16 * h + 8 * g1;
    d.off[SS::KPW + j] = (uint32_t)(((16 * dt + n) * P + (ks & (P - 1)) + SS::E * h2) * sizeof(T));
  }
  return d;
}

// Global base addresses of a stage's two halves for this KV head.
struct HalfBases {
  const char* k0;
  const char* k1;
  const char* v0;
  const char* v1;
};

// Bases from the staged (lo, hi) page byte offsets, made wave-uniform.
__device__ __forceinline__ HalfBases half_bases(const char* kbase, const char* vbase, uint4 po) {
  const uint64_t lo = ((uint64_t)__builtin_amdgcn_readfirstlane(po.y) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane(po.x);
  const uint64_t hi = ((uint64_t)__builtin_amdgcn_readfirstlane(po.w) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane(po.z);
  return HalfBases{kbase + lo, kbase + hi, vbase + lo, vbase + hi};
}

// Issues this wave's pieces of one stage into the ring slot `slot`. Piece p of
// wave r is r + 4 j; its half, hence its page base, is wave-uniform. TAIL:
// K lanes whose key lies at or past n_keys read zeros instead; V elements past
// n_keys are zeroed by their reader.
template <typename T, int D, bool TAIL, int CPOL>
__device__ __forceinline__ void issue_dma(char* slot, int r, const DmaLanes<T, D>& dl,
                                          const HalfBases& hb, int key0, int n_keys) {
  using SS = StageShape<T, D>;
#pragma unroll
  for (int j = 0; j < SS::KPW; ++j) {
    const int p = r + kRowSlots * j;
    const char* base = p >= SS::NKP / 2 ? hb.k1 : hb.k0;
    const char* src = base + dl.off[j];
    if (TAIL && key0 + dl.key[j] >= n_keys) src = reinterpret_cast<const char*>(g_zero16);
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(slot + p * 1024),
                                     16, 0, CPOL);
  }
#pragma unroll
  for (int j = 0; j < SS::VPW; ++j) {
    const int p = r + kRowSlots * j;
    const char* base = p >= SS::NVP / 2 ? hb.v1 : hb.v0;
    __builtin_amdgcn_global_load_lds(base + dl.off[SS::KPW + j],
                                     (__attribute__((address_space(3))) void*)(slot + (SS::NKP + p) * 1024),
                                     16, 0, CPOL);
  }
}

// Issues one stage (when it exists) whose first key is key0; the stage that
// crosses n_keys takes the zero-filling path. A head's keys are streamed once
// (non-temporal loads) unless its query rows are cut into row groups, whose
// workgroups run side by side on one XCD and read the same keys: then the
// loads keep the lines in that XCD's L2 for the other groups (at the
// draft-pass shape with 128-position blocks, four groups per head, HBM reads
// 764 -> 712 MB per launch for 701 MB of K, V and Q, same time).
template <typename T, int D>
__device__ __forceinline__ void issue_stage(char* slot, int r, const DmaLanes<T, D>& dl,
                                            const HalfBases& hb, int key0, int n_keys,
                                            bool exists, bool shared) {
  if (!exists) return;
  if (key0 + kStep <= n_keys) {
    if (shared) issue_dma<T, D, false, kTemporal>(slot, r, dl, hb, key0, n_keys);
    else issue_dma<T, D, false, kNonTemporal>(slot, r, dl, hb, key0, n_keys);
  } else {
    if (shared) issue_dma<T, D, true, kTemporal>(slot, r, dl, hb, key0, n_keys);
    else issue_dma<T, D, true, kNonTemporal>(slot, r, dl, hb, key0, n_keys);
  }
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only, so its vector-memory loads and stores stay in flight across it
// (__syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------- LDS reads
// N 16-byte fragment parts at lane-relative LDS address addr + 512 * i, then
// one s_waitcnt. Inline asm keeps the compiler's LDS-DMA tracking from
// inserting a wait for every DMA still in flight.
__device__ __forceinline__ void lds_read4(intx4* o, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n\t"
      "ds_read_b128 %1, %4 offset:512\n\t"
      "ds_read_b128 %2, %4 offset:1024\n\t"
      "ds_read_b128 %3, %4 offset:1536\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(addr)
      : "memory");
}

__device__ __forceinline__ void lds_read8(intx4* o, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:512\n\t"
      "ds_read_b128 %2, %8 offset:1024\n\t"
      "ds_read_b128 %3, %8 offset:1536\n\t"
      "ds_read_b128 %4, %8 offset:2048\n\t"
      "ds_read_b128 %5, %8 offset:2560\n\t"
      "ds_read_b128 %6, %8 offset:3072\n\t"
      "ds_read_b128 %7, %8 offset:3584\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(addr)
      : "memory");
}

__device__ __forceinline__ void lds_read16(intx4* o, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\t"
      "ds_read_b128 %1, %16 offset:512\n\t"
      "ds_read_b128 %2, %16 offset:1024\n\t"
      "ds_read_b128 %3, %16 offset:1536\n\t"
      "ds_read_b128 %4, %16 offset:2048\n\t"
      "ds_read_b128 %5, %16 offset:2560\n\t"
      "ds_read_b128 %6, %16 offset:3072\n\t"
      "ds_read_b128 %7, %16 offset:3584\n\t"
      "ds_read_b128 %8, %16 offset:4096\n\t"
      "ds_read_b128 %9, %16 offset:4608\n\t"
      "ds_read_b128 %10, %16 offset:5120\n\t"
      "ds_read_b128 %11, %16 offset:5632\n\t"
      "ds_read_b128 %12, %16 offset:6144\n\t"
      "ds_read_b128 %13, %16 offset:6656\n\t"
      "ds_read_b128 %14, %16 offset:7168\n\t"
      "ds_read_b128 %15, %16 offset:7680\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]),
        "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(addr)
      : "memory");
}

// K and V parts of a whole stage from two lane addresses behind one wait.
__device__ __forceinline__ void lds_read4_4(intx4* k, intx4* v, unsigned ka, unsigned va) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:512\n\t"
      "ds_read_b128 %2, %8 offset:1024\n\t"
      "ds_read_b128 %3, %8 offset:1536\n\t"
      "ds_read_b128 %4, %9 offset:0\n\t"
      "ds_read_b128 %5, %9 offset:512\n\t"
      "ds_read_b128 %6, %9 offset:1024\n\t"
      "ds_read_b128 %7, %9 offset:1536\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3])
      : "v"(ka), "v"(va)
      : "memory");
}

__device__ __forceinline__ void lds_read8_8(intx4* k, intx4* v, unsigned ka, unsigned va) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\t"
      "ds_read_b128 %1, %16 offset:512\n\t"
      "ds_read_b128 %2, %16 offset:1024\n\t"
      "ds_read_b128 %3, %16 offset:1536\n\t"
      "ds_read_b128 %4, %16 offset:2048\n\t"
      "ds_read_b128 %5, %16 offset:2560\n\t"
      "ds_read_b128 %6, %16 offset:3072\n\t"
      "ds_read_b128 %7, %16 offset:3584\n\t"
      "ds_read_b128 %8, %17 offset:0\n\t"
      "ds_read_b128 %9, %17 offset:512\n\t"
      "ds_read_b128 %10, %17 offset:1024\n\t"
      "ds_read_b128 %11, %17 offset:1536\n\t"
      "ds_read_b128 %12, %17 offset:2048\n\t"
      "ds_read_b128 %13, %17 offset:2560\n\t"
      "ds_read_b128 %14, %17 offset:3072\n\t"
      "ds_read_b128 %15, %17 offset:3584\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
        "=&v"(k[6]), "=&v"(k[7]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
        "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(ka), "v"(va)
      : "memory");
}

template <int N>
__device__ __forceinline__ void lds_read(intx4* o, unsigned addr) {
  static_assert(N == 4 || N == 8 || N == 16, "part counts");
  if constexpr (N == 4) lds_read4(o, addr);
  else if constexpr (N == 8) lds_read8(o, addr);
  else lds_read16(o, addr);
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

// Zeroes the V elements of keys at or past n_keys (their slots may hold
// anything, NaN included) on the stage that crosses the sequence end.
template <typename T, int D>
__device__ __forceinline__ void zero_v_tail(intx4* vp, int key0, int n_keys, int grp) {
  using SS = StageShape<T, D>;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < SS::H; ++h2)
#pragma unroll
      for (int e = 0; e < SS::E; ++e) {
        if (key0 + 8 * grp + SS::E * h2 + e >= n_keys) {
          intx4& x = vp[dt * SS::H + h2];
          if (sizeof(T) == 4) x[e] = 0;
          else x[e / 2] &= (e & 1) ? 0x0000ffff : (int)0xffff0000;
        }
      }
}

template <typename T, int D, int MT>
struct WaveState {
  typename Frag<T>::vec qf[MT][D / 32];
  floatx4 acc[D / 16][MT];
  float m_run[MT], l_run[MT];
  int blk_row[MT];
  uint64_t tmask[MT];  // TREE mode: the row's visibility bits over the block keys
};

// TREE blocks of more than 64 nodes: each row's visibility over the block is
// W = ceil(B / 64) words, staged in LDS for the block rows of the workgroup's
// row group (block rows ibase .. ilast), word w of row i at rows[(i - ibase)
// * W + w].
constexpr int kMaxTreeWords = kMaxTreeNodes / 64;
constexpr int kWideMaskWords = (128 + 1) * kMaxTreeWords;   // row group rows + 1
struct WideMask {
  const uint64_t* rows;
  int ibase, ilast, W;
};

// The block rows of the row group starting at query row row0, for LDS words s.
__device__ __forceinline__ WideMask wide_mask(const AttnArgs& a, uint64_t* s, int row0) {
  return WideMask{s, row0 / a.g, min(a.B - 1, (row0 + a.M - 1) / a.g), a.tree_words};
}

// Every thread: request b's mask words of the group's rows into LDS (the
// caller publishes them with a barrier).
__device__ __forceinline__ void stage_wide_mask(const AttnArgs& a, uint64_t* s,
                                                const WideMask& wm, int b, int tid) {
  const int n = (wm.ilast - wm.ibase + 1) * wm.W;
  const uint64_t* src = a.tree + ((a.tree_per_req ? (size_t)b * a.B : 0) + wm.ibase) * (size_t)wm.W;
  for (int e = tid; e < n; e += kWave * kWaves) s[e] = src[e];
}

// A stage is consumed in two halves so that the two waves sharing a SIMD can
// run them out of phase:
//   front: read the stage's K and V fragments from the ring, S^T = K Q^T;
//   back:  mask, online softmax update, O^T += V^T P^T (registers only).
// s[T][t][j] is key key0 + 8*grp + 4*T + j against row 16t + n of the wave;
// softmax runs in the exp2 domain with the scale folded into the exponent.
template <typename T, int D, int MT>
struct StageRegs {
  floatx4 s[2][MT];
  intx4 vp[StageShape<T, D>::NVP];
  int key0;
};

template <typename T, int D, int MT>
__device__ __forceinline__ void stage_front(StageRegs<T, D, MT>& st, const WaveState<T, D, MT>& ws,
                                            unsigned kaddr, unsigned vaddr, int key0) {
  using SS = StageShape<T, D>;
  intx4 kp[SS::NKP];
  constexpr bool together = MT == 1 && SS::NKP == SS::NVP && SS::NKP <= 8;
  if constexpr (together) {
    if constexpr (SS::NKP == 4) lds_read4_4(kp, st.vp, kaddr, vaddr);
    else lds_read8_8(kp, st.vp, kaddr, vaddr);
  } else {
    lds_read<SS::NKP>(kp, kaddr);
  }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < SS::KC; ++cc)
        c = Frag<T>::mma(frag_of<T>(kp + (t2 * SS::KC + cc) * SS::H), ws.qf[t][cc], c);
      st.s[t2][t] = c;
    }
  if constexpr (!together) lds_read<SS::NVP>(st.vp, vaddr);
  st.key0 = key0;
}

template <typename T, int D, int MT, bool WIDE = false>
__device__ __forceinline__ void stage_back(StageRegs<T, D, MT>& st, WaveState<T, D, MT>& ws,
                                           const AttnArgs& a, int L, int n_keys, int nc, int grp,
                                           const WideMask& wm) {
  using SS = StageShape<T, D>;
  const int key0 = st.key0;
  if (key0 + kStep > n_keys) zero_v_tail<T, D>(st.vp, key0, n_keys, grp);

  if (key0 + kStep > L) {
    // WIDE: bits key0 - L .. key0 - L + 31 of each row's mask, from at most
    // two LDS words (rows past the group's end read a neighbour: their
    // outputs are never written; bits outside the block read as 0, and the
    // keys there are context, always visible, or past the end, never)
    uint32_t win[MT];
    if constexpr (WIDE) {
      const int jb0 = key0 - L, wi = jb0 >> 6, sh = jb0 & 63;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int ic = min(max(ws.blk_row[t], wm.ibase), wm.ilast) - wm.ibase;
        const uint64_t* row = wm.rows + ic * wm.W;
        const uint64_t lo = wi >= 0 && wi < wm.W ? row[wi] : 0;
        const uint64_t hi = wi + 1 >= 0 && wi + 1 < wm.W ? row[wi + 1] : 0;
        win[t] = (uint32_t)(sh ? (lo >> sh) | (hi << (64 - sh)) : lo);
      }
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + 8 * grp + 4 * t2 + j;
          const int jb = key - L, i = ws.blk_row[t];
          bool intra;
          if constexpr (WIDE) {
            intra = (win[t] >> (8 * grp + 4 * t2 + j)) & 1;
          } else {
            intra = a.mode == 3 ? ((ws.tmask[t] >> (jb & 63)) & 1) != 0
                                : (a.mode == 0) | (jb <= i) | ((a.mode == 2) & (i >= nc));
          }
          const bool vis = (key < L) | ((key < n_keys) & intra);
          st.s[t2][t][j] = vis ? st.s[t2][t][j] : -__builtin_inff();
        }
  }

  const float c2 = a.scale_log2;
  float m_new[MT];
  bool need_any = false;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const floatx4 s0 = st.s[0][t], s1 = st.s[1][t];
    // scores are finite or -inf (masked) here: the NaN-propagating maximum
    // is exact and needs no operand quieting
    float mx = vmax(vmax(vmax(s0[0], s0[1]), vmax(s0[2], s0[3])),
                    vmax(vmax(s1[0], s1[1]), vmax(s1[2], s1[3])));
    mx = group_max4(mx) * c2;
    m_new[t] = vmax(ws.m_run[t], mx);
    need_any |= m_new[t] > ws.m_run[t] + kRescale;
  }
  if (__builtin_amdgcn_ballot_w64(need_any)) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const bool need = m_new[t] > ws.m_run[t] + kRescale;
      const float alpha = need ? __builtin_amdgcn_exp2f(ws.m_run[t] - m_new[t]) : 1.0f;
      ws.m_run[t] = need ? m_new[t] : ws.m_run[t];
      ws.l_run[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) ws.acc[dt][t] *= alpha;
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
        pv[4 * t2 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[t2][t][j], c2, -ws.m_run[t]));
    ws.l_run[t] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    pf[t] = Frag<T>::pack(pv);
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int t = 0; t < MT; ++t)
      ws.acc[dt][t] = Frag<T>::mma(frag_of<T>(st.vp + dt * SS::H), pf[t], ws.acc[dt][t]);
}

// WIDE: whether none of the wave's rows sees a key of the stage starting at
// key0, which lies wholly inside the block (the window test of stage_back,
// over the wave's rows; padding rows read a neighbour's words, so the answer
// errs on the side of computing). Such a stage changes no running state
// (every score is -inf: the maximum, the row sum and the output stay as they
// are), so the wave skips its products.
template <typename T, int D, int MT>
__device__ __forceinline__ bool wide_stage_masked(const WaveState<T, D, MT>& ws,
                                                  const WideMask& wm, int key0, int L) {
  if (key0 < L) return false;
  const int jb0 = key0 - L, wi = jb0 >> 6, sh = jb0 & 63;
  uint32_t any = 0;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int ic = min(max(ws.blk_row[t], wm.ibase), wm.ilast) - wm.ibase;
    const uint64_t* row = wm.rows + ic * wm.W;
    const uint64_t lo = wi < wm.W ? row[wi] : 0;
    const uint64_t hi = wi + 1 < wm.W ? row[wi + 1] : 0;
    any |= (uint32_t)(sh ? (lo >> sh) | (hi << (64 - sh)) : lo);
  }
  return __builtin_amdgcn_ballot_w64(any != 0) == 0;
}

// Per-wave constants of the stage pipeline.
template <typename T, int D>
struct WaveCtx {
  int tid, lane, set, rs, n, grp;
  DmaLanes<T, D> dl;
  unsigned k_lane, v_lane;  // lane-relative LDS addresses of the first K / V fragment parts
};

template <typename T, int D>
__device__ __forceinline__ WaveCtx<T, D> wave_ctx(const AttnArgs& a, const char* s_ring) {
  using SS = StageShape<T, D>;
  WaveCtx<T, D> c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((unsigned)c.tid >> 6);
  c.set = wave / kRowSlots;
  c.rs = wave % kRowSlots;
  c.n = c.lane & 15;
  c.grp = c.lane >> 4;
  c.dl = dma_lanes<T, D>(a.P, c.rs, c.lane);
  const int hk = c.n >> 3, hv = c.grp >> 1;
  const unsigned ring = (unsigned)(size_t)s_ring + (unsigned)c.set * SS::BYTES;
  c.k_lane = ring + hk * (SS::NKP / 2) * 1024 + (8 * (c.grp ^ hk) + (c.n & 7)) * 16;
  c.v_lane = ring + SS::NKP * 1024 + hv * (SS::NVP / 2) * 1024 + (16 * (c.grp & 1) + c.n) * 16;
  return c;
}

// A unit: request b, KV head kvh, and the row group whose first query row
// (of the head's Mt = g * B) is row0; its rows are row0 .. row0 + M - 1,
// clipped to Mt.
struct UnitRef {
  int b, kvh, row0;
};

__device__ __forceinline__ UnitRef unit_ref(const AttnArgs& a, int unit) {
  const int b = unit / a.Hv;
  const int vh = unit - b * a.Hv;
  const int kvh = vh / a.RG;
  return UnitRef{b, kvh, (vh - kvh * a.RG) * a.M};
}

// Whether local row r (0 .. M - 1) of a unit whose group starts at row0 exists.
__device__ __forceinline__ bool row_exists(const AttnArgs& a, int row0, int r) {
  return r < a.M && row0 + r < a.Mt;
}

// Q^T operands of this wave's rows of unit (b, kvh, row0): lane (n, grp)
// holds local row 16t + n, dims 32c + 8*grp .. +7. Row r of the head is block
// token r / g, query head kvh * g + r % g. Both waves of a row slot hold the
// same rows.
// Empty softmax state: running max, sum and output of every row tile.
template <typename T, int D, int MT>
__device__ __forceinline__ void reset_state(WaveState<T, D, MT>& ws) {
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    ws.m_run[t] = kNegBig;
    ws.l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) ws.acc[dt][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
}

// Q fragments of the wave's row tiles (and each row's block row and tree
// mask); with reset, an empty softmax state as well.
template <typename T, int D, int MT>
__device__ __forceinline__ void load_q(WaveState<T, D, MT>& ws, const AttnArgs& a, int b, int kvh,
                                       int row0, int rs, int n, int grp, bool reset = true) {
  const int rl0 = rs * 16 * MT;
  const T* qg = reinterpret_cast<const T*>(a.q);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int rl = rl0 + 16 * t + n;
    const bool in = row_exists(a, row0, rl);
    const int r = row0 + rl;
    ws.blk_row[t] = r / a.g;
    const int rr = in ? r : 0;
    const int ii = rr / a.g, hh = rr - ii * a.g;
    ws.tmask[t] = a.mode == 3 ? a.tree[((a.tree_per_req ? (size_t)b * a.B : 0) + ii) * a.tree_words]
                              : 0;
    // a row past the group's end reads the head's first row: its scores stay
    // finite, its softmax state is its own and its output is never written
    const T* src = qg + ((size_t)(b * a.B + ii) * a.Hq + kvh * a.g + hh) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) ws.qf[t][c] = Frag<T>::load(src + 32 * c);
  }
  if (reset) reset_state(ws);
}

// Page-table entries of stage t of a request: the pages of keys 32 t and
// 32 t + 16, read whenever they lie inside the table row (validated later,
// once the length says which stages exist).
__device__ __forceinline__ int2 table_pair(const AttnArgs& a, const int32_t* ptab, int t) {
  const int i_lo = (t * kStep) >> a.p_shift, i_hi = (t * kStep + 16) >> a.p_shift;
  return int2{i_lo < a.max_pages ? ptab[i_lo] : 0, i_hi < a.max_pages ? ptab[i_hi] : 0};
}

// Sequence length of request b clamped to the page-table capacity.
// Clean (causal) rows of request b's block in MIXED mode. b is wave-uniform:
// the per-request count is read with a scalar load, whose wait (lgkmcnt)
// does not drain the vector-memory queue.
__device__ __forceinline__ int causal_rows(const AttnArgs& a, int b) {
  if (!a.nc_per_req) return a.n_causal;
  const auto* p = (const __attribute__((address_space(4))) int32_t*)a.nc_per_req;
  return p[__builtin_amdgcn_readfirstlane(b)];
}

// Byte offsets of the (lo, hi) pages of stage t into window entry `slot`;
// hi = lo when the stage has one page (P = 32) or its second page lies past
// the sequence end. A page id outside the pool flags kErrSlot and reads page 0.
template <typename T, int D>
__device__ __forceinline__ void put_offsets(const AttnArgs& a, uint64_t* s_pgoff, int slot, int t,
                                            int2 pg, int n_keys) {
  const uint64_t page_bytes = (uint64_t)a.P * D * a.Hkv * sizeof(T);
  const bool second = a.P == 16 && t * kStep + 16 < n_keys;
  const bool bad_lo = (unsigned)pg.x >= (unsigned)a.num_pages;
  const bool bad_hi = second && (unsigned)pg.y >= (unsigned)a.num_pages;
  if (bad_lo || bad_hi) flag_error(a.err, kErrSlot);
  const uint64_t lo = (uint64_t)(bad_lo ? 0 : pg.x) * page_bytes;
  const uint64_t hi = second ? (uint64_t)(bad_hi ? 0 : pg.y) * page_bytes : lo;
  reinterpret_cast<uint4*>(s_pgoff)[slot] =
      uint4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

__device__ __forceinline__ int clamped_len(const AttnArgs& a, int b, bool flag) {
  int L = a.seq_lens[b];
  const int cap = a.max_pages * a.P - a.B;
  if (L < 0 || L > cap) {
    if (flag) flag_error(a.err, kErrCapacity);
    L = L < 0 ? 0 : cap;
  }
  return L;
}

// Streams stages [s_lo, s_hi) of unit (b, kvh), length L, through the ring
// into this wave's softmax state. Thread tid stages the page offsets of
// stage tid of each window (first window: the prefetched `first` entries).
template <typename T, int D, int MT, bool STAGED = false, bool WIDE = false>
__device__ __forceinline__ void stream_stages(WaveState<T, D, MT>& ws, const AttnArgs& a,
                                              const WaveCtx<T, D>& c, char* s_ring,
                                              uint64_t* s_pgoff, int b, int kvh, int row0, int L,
                                              int nc, int s_lo, int s_hi, int2 first,
                                              const WideMask& wm = WideMask{}) {
  using SS = StageShape<T, D>;
  constexpr int NSP = SS::NSP;
  static_assert(kPageWin == kWave * kWaves, "one thread per staged stage");
  const char* kbase = reinterpret_cast<const char*>(a.k) + (size_t)kvh * a.P * D * sizeof(T);
  const char* vbase = reinterpret_cast<const char*>(a.v) + (size_t)kvh * a.P * D * sizeof(T);
  const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
  const int n_keys = L + a.B;
  const bool has_rows = row_exists(a, row0, c.rs * 16 * MT);
  const int set = c.set;

  for (int w0 = s_lo; w0 < s_hi; w0 += kPageWin) {
    const int w1 = min(s_hi, w0 + kPageWin);
    const int ns = w1 - w0;
    lds_barrier();  // the previous window (or unit) is fully consumed
    // the page offsets of every stage of the window (STAGED: the caller has
    // already written the first window's)
    if (c.tid < ns && !(STAGED && w0 == s_lo))
      put_offsets<T, D>(a, s_pgoff, c.tid, w0 + c.tid,
                        w0 == s_lo ? first : table_pair(a, ptab, w0 + c.tid), n_keys);
    // The waits below count this wave's ring DMAs by hand. Older vector-memory
    // operations may still be in flight here (the Q loads, the previous
    // piece's output stores); they only make those waits longer: loads
    // complete in issue order and every older operation counts against a
    // wait, so none can pass before the DMAs it waits for have landed.
    lds_barrier();

    // pair u holds window stages 2u (set 0) and 2u + 1 (set 1) in ring slot u % NSP
    const int npairs = (ns + 1) >> 1;
    const int mine = (ns - set + 1) >> 1;  // pairs with a stage for this wave's set
    auto offsets = [&](int u) {
      const int t = min(2 * u + set, ns - 1);
      return reinterpret_cast<const uint4*>(s_pgoff)[t];
    };
    auto issue = [&](int u, uint4 po) {
      issue_stage<T, D>(s_ring + (u % NSP) * SS::PAIR + set * SS::BYTES, c.rs, c.dl,
                        half_bases(kbase, vbase, po), (w0 + 2 * u + set) * kStep, n_keys,
                        2 * u + set < ns, a.RG > 1);
    };
    // NSP - 1 pairs in flight. Each wave waits for its own DMA share of pair
    // u (vmcnt counts this wave's loads in issue order), the barrier
    // publishes every share, and the slot consumed one pair earlier is
    // refilled with pair u + NSP - 1.
    for (int u = 0; u < NSP - 1 && u < npairs; ++u) issue(u, offsets(u));
    uint4 po_next = offsets(NSP - 1);
    // Between two barriers set 0 runs the front then the back half of its
    // stage; set 1 first finishes the back half of its previous stage (held
    // in registers across the barrier), then runs the front half of its new
    // one. The two waves of a SIMD thus work on different halves at once:
    // one reads LDS and issues S MFMAs while the other runs the softmax.
    // Set 0 issues its share of the refill right after the barrier, set 1
    // only after its back half: the per-CU queue of vector-memory requests
    // then never holds both waves of a SIMD at once, so one of them always
    // has compute to issue while the other's loads wait for queue space.
    StageRegs<T, D, MT> st;
    bool pending = false;
    for (int u = 0; u < npairs; ++u) {
      wait_stages<SS::PW>(max(0, min(NSP - 2, mine - 1 - u)));
      asm volatile("s_barrier" ::: "memory");
      const bool more = u + NSP - 1 < npairs;
      if (more && (set == 0 || !has_rows)) issue(u + NSP - 1, po_next);
      if (has_rows) {
        if (pending) stage_back<T, D, MT, WIDE>(st, ws, a, L, n_keys, nc, c.grp, wm);
        pending = false;
        if (more && set == 1) issue(u + NSP - 1, po_next);
        const int t = 2 * u + set;
        bool skip = false;
        if constexpr (WIDE) skip = t < ns && wide_stage_masked(ws, wm, (w0 + t) * kStep, L);
        if (t < ns && !skip) {
          const unsigned so = (u % NSP) * SS::PAIR;
          stage_front<T, D, MT>(st, ws, c.k_lane + so, c.v_lane + so, (w0 + t) * kStep);
          if (set == 0) stage_back<T, D, MT, WIDE>(st, ws, a, L, n_keys, nc, c.grp, wm);
          else pending = true;
        }
      }
      po_next = offsets(u + NSP);
    }
    if (pending) stage_back<T, D, MT, WIDE>(st, ws, a, L, n_keys, nc, c.grp, wm);
  }
}

// Merges the two key halves of every row slot through LDS, then writes the
// unit's rows: normalised output (part < 0) or the unnormalised partial
// state into partial slot `part`.
template <typename T, int D, int MT, typename F>
__device__ __forceinline__ void finish_unit(WaveState<T, D, MT>& ws, const AttnArgs& a,
                                            const WaveCtx<T, D>& c, char* s_ring, int b, int kvh,
                                            int row0, int part, F&& between) {
  using SS = StageShape<T, D>;
  static_assert(kRowSlots * (D / 16) * MT * 1024 + kRowSlots * MT * 512 <= SS::NSP * SS::PAIR,
                "merge buffers fit the ring");
  const int rl0 = c.rs * 16 * MT;
  const bool has_rows = row_exists(a, row0, rl0);
  const int lane = c.lane;
  lds_barrier();  // every stage consumed: the ring and the page offsets are free
  between();
  floatx4* x_acc = reinterpret_cast<floatx4*>(s_ring) + (size_t)c.rs * (D / 16) * MT * 64;
  float2* x_ml = reinterpret_cast<float2*>(s_ring + kRowSlots * (D / 16) * MT * 1024) +
                 (size_t)c.rs * MT * 64;
  if (c.set == 1 && has_rows) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) x_acc[(dt * MT + t) * 64 + lane] = ws.acc[dt][t];
      x_ml[t * 64 + lane] = float2{ws.m_run[t], ws.l_run[t]};
    }
  }
  lds_barrier();
  if (c.set == 1 || !has_rows) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float2 ml = x_ml[t * 64 + lane];
    const float m = fmaxf(ws.m_run[t], ml.x);
    const float a0 = __builtin_amdgcn_exp2f(ws.m_run[t] - m);
    const float a1 = __builtin_amdgcn_exp2f(ml.x - m);
    ws.m_run[t] = m;
    ws.l_run[t] = a0 * ws.l_run[t] + a1 * ml.y;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      ws.acc[dt][t] = a0 * ws.acc[dt][t] + a1 * x_acc[(dt * MT + t) * 64 + lane];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float l_tot = group_sum4(ws.l_run[t]);
    const int rl = rl0 + 16 * t + c.n;
    if (!row_exists(a, row0, rl)) continue;
    const int r = row0 + rl;
    const int i = r / a.g, hl = r - i * a.g;
    const size_t orow = (size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl;
    if (part < 0) {
      const float inv = 1.0f / l_tot;
      T* dst = reinterpret_cast<T*>(a.o) + orow * D + 4 * c.grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) Frag<T>::store4(dst + 16 * dt, ws.acc[dt][t] * inv);
      if (a.lse && c.grp == 0) a.lse[orow] = (ws.m_run[t] + __log2f(l_tot)) * kLn2;
    } else {
      const size_t prow = (size_t)part * a.M + rl;
      float* dst = a.part_o + prow * D + 4 * c.grp;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(dst + 16 * dt) = ws.acc[dt][t];
      if (c.grp == 0) {
        a.part_ml[prow * 2 + 0] = ws.m_run[t];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// One workgroup per (request, KV head, split): the split is stages
// [split * steps_per_split, ...) of the unit. With one split the rows are
// written normalised, otherwise as partial state for the split merge.
//
// Workgroups are dealt to the 8 XCDs round robin. With row groups, hardware
// block x runs logical block (x % 8) * (n / 8) + x / 8 (n blocks, n % 8 == 0),
// so that each XCD takes a contiguous run of logical blocks: the row groups
// of one KV head then run side by side on one XCD and share its keys in L2.
__device__ __forceinline__ int logical_block(const AttnArgs& a, int x, int n) {
  return (a.RG > 1 && n % 8 == 0) ? (x % 8) * (n / 8) + x / 8 : x;
}

template <typename T, int D, int MT, bool WIDE = false>
__global__ __launch_bounds__(kWave * kWaves, 1) void block_attn_kernel(AttnArgs a) {
  using SS = StageShape<T, D>;
  __shared__ __attribute__((aligned(1024))) char s_ring[SS::NSP * SS::PAIR];
  __shared__ __attribute__((aligned(16))) uint64_t s_pgoff[2 * kPageWin];  // (lo, hi) per stage
  __shared__ uint64_t s_tm[WIDE ? kWideMaskWords : 1];

  const WaveCtx<T, D> c = wave_ctx<T, D>(a, s_ring);
  const int lb = logical_block(a, blockIdx.x, gridDim.x);
  const int unit = lb / a.splits;
  const int split = lb - unit * a.splits;
  const UnitRef u = unit_ref(a, unit);
  const int b = u.b, kvh = u.kvh;
  const int s_lo = split * a.steps_per_split;

  // loads that do not depend on the sequence length go out first, so that
  // their latency overlaps the length's
  WaveState<T, D, MT> ws;
  load_q<T, D, MT>(ws, a, b, kvh, u.row0, c.rs, c.n, c.grp);
  const int2 first = table_pair(a, a.page_table + (size_t)b * a.max_pages, s_lo + c.tid);
  const int L = clamped_len(a, b, c.tid == 0 && split == 0);
  const int n_steps = (L + a.B + kStep - 1) / kStep;
  const int s_hi = (split == a.splits - 1) ? n_steps : min(n_steps, s_lo + a.steps_per_split);
  const int nc = causal_rows(a, b);
  WideMask wm{s_tm, 0, 0, 1};
  if constexpr (WIDE) {
    // the row group's mask words into LDS (the streaming loop starts with a
    // barrier, which publishes them)
    wm = wide_mask(a, s_tm, u.row0);
    stage_wide_mask(a, s_tm, wm, b, c.tid);
  }
  stream_stages<T, D, MT, false, WIDE>(ws, a, c, s_ring, s_pgoff, b, kvh, u.row0, L, nc, s_lo,
                                       s_hi, first, wm);
  finish_unit<T, D, MT>(ws, a, c, s_ring, b, kvh, u.row0, a.splits == 1 ? -1 : lb, [] {});
}

// ------------------------------------------------------- balanced schedule
// For batches whose lengths may differ widely, a fixed grid of G workgroups
// shares the work evenly: the weighted pairs of all units, taken in unit
// order (unit = b * Hkv + kvh; each unit ceil(ceil((L_b + B) / 32) / 2) stage
// pairs behind piece_cost leading pairs that stand for a piece's fixed cost),
// are cut into G equal contiguous ranges, workgroup w taking weighted pairs
// [floor(TP * w / G), floor(TP * (w + 1) / G)). A unit whose stage pairs a
// range boundary cuts is written as partial states by the workgroups that
// share it -- into slot 2w when it is workgroup w's first unit, else 2w + 1 --
// and merged by the boundary-combine kernel; every other unit is written
// normalised.
//
// With row groups the G workgroups form T = G / RG teams of RG: the ranges
// are cut over the teams (a unit here is a (request, KV head) pair), and each
// member streams its team's range for its own row group. A team's members sit
// on one XCD, dealt out one after the other, so they share the keys in L2.
// Partial slots are (2 team + {0, 1}) * RG + rg.
__device__ __forceinline__ int2 team_of(const AttnArgs& a, int x, int G) {
  if (a.RG == 1) return int2{x, 0};
  const int per_xcd = G / 8, j = x / 8;
  return int2{(x % 8) * (per_xcd / a.RG) + j / a.RG, j % a.RG};
}

__device__ __forceinline__ int unit_pairs(const AttnArgs& a, int L) {
  const int n_steps = (L + a.B + kStep - 1) / kStep;
  return (n_steps + 1) >> 1;
}

__device__ __forceinline__ int block_exclusive_scan_int(int x, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int v = s_tmp[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// The balanced schedule deals out weighted pairs: unit (b, kvh) weighs its
// stage pairs np plus a.piece_cost leading pairs that stand for the fixed
// cost of a piece and hold no stages. A range that covers only some of a
// unit's leading pairs takes none of its stages.
__device__ __forceinline__ int unit_weight(const AttnArgs& a, int L) {
  return unit_pairs(a, L) + a.piece_cost;
}

// s_pre[b] = weight of all units of requests before b (b = 0 .. bs); returns
// the total. Thread tid covers a contiguous run of requests. With s_len, the
// clamped lengths are kept there too.
__device__ int balanced_prefix(const AttnArgs& a, int* s_pre, int* s_tmp, bool flag,
                               int* s_len = nullptr) {
  const int nthr = blockDim.x, tid = threadIdx.x;
  const int per = (a.bs + nthr - 1) / nthr;
  const int b0 = min(a.bs, tid * per), b1 = min(a.bs, b0 + per);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += a.Hkv * unit_weight(a, clamped_len(a, b, flag));
  int total;
  int run = block_exclusive_scan_int(sum, s_tmp, &total);
  for (int b = b0; b < b1; ++b) {
    s_pre[b] = run;
    const int L = clamped_len(a, b, false);
    if (s_len) s_len[b] = L;
    run += a.Hkv * unit_weight(a, L);
  }
  if (tid == 0) s_pre[a.bs] = total;
  __syncthreads();
  return total;
}

// Request holding weighted pair x: the largest b with s_pre[b] <= x.
__device__ __forceinline__ int request_of(const int* s_pre, int bs, int x) {
  int lo = 0, hi = bs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int range_start(int total, int w, int G) {
  return (int)((long long)total * w / G);
}

template <typename T, int D, int MT, bool WIDE = false>
__global__ __launch_bounds__(kWave * kWaves, 1) void block_attn_balanced_kernel(AttnArgs a) {
  using SS = StageShape<T, D>;
  __shared__ __attribute__((aligned(1024))) char s_ring[SS::NSP * SS::PAIR];
  __shared__ __attribute__((aligned(16))) uint64_t s_pgoff[2 * kPageWin];
  __shared__ uint64_t s_tm[WIDE ? kWideMaskWords : 1];
  __shared__ int s_pre[kMaxBalancedBatch + 1];
  __shared__ int s_len[kMaxBalancedBatch];
  __shared__ int s_tmp[kWaves];

  const WaveCtx<T, D> c = wave_ctx<T, D>(a, s_ring);
  const int2 tr = team_of(a, blockIdx.x, gridDim.x);
  const int T_ = gridDim.x / a.RG, w = tr.x, rg = tr.y, row0 = rg * a.M;
  const int total = balanced_prefix(a, s_pre, s_tmp, blockIdx.x == 0, s_len);
  const int start = range_start(total, w, T_), end = range_start(total, w + 1, T_);
  if (start >= end) return;
  const int X = a.piece_cost;
  int b = request_of(s_pre, a.bs, start);
  int L = s_len[b];
  int np = unit_pairs(a, L);
  int kvh = (start - s_pre[b]) / (np + X);
  int ustart = s_pre[b] + kvh * (np + X);  // weighted start of unit (b, kvh)
  // the unit's stage pairs [off, lim) inside this workgroup's range
  int off = max(0, start - ustart - X);
  int lim = max(0, min(np + X, end - ustart) - X);
  if (lim <= off) return;  // the range holds only leading pairs of one unit
  // stages [x, y) of the piece
  auto stage_range = [&]() {
    return int2{2 * off, min((L + a.B + kStep - 1) / kStep, 2 * lim)};
  };
  // the page offsets of the first window of a piece (stages r.x ..) from
  // its page ids pg (thread tid: stage r.x + tid)
  auto stage_first = [&](int2 r, int2 pg) {
    if (c.tid < min(r.y, r.x + kPageWin) - r.x)
      put_offsets<T, D>(a, s_pgoff, c.tid, r.x + c.tid, pg, L + a.B);
  };
  WaveState<T, D, MT> ws;
  load_q<T, D, MT>(ws, a, b, kvh, row0, c.rs, c.n, c.grp);
  int nc = causal_rows(a, b);
  int2 range = stage_range();
  stage_first(range, table_pair(a, a.page_table + (size_t)b * a.max_pages, range.x + c.tid));
  // TREE blocks of more than 64 nodes: the workgroup's row group is fixed,
  // so its mask words change only with the request (restaged with the next
  // piece's page offsets, after the barrier that ends their last reads)
  const WideMask wm = WIDE ? wide_mask(a, s_tm, row0) : WideMask{s_tm, 0, 0, 1};
  if constexpr (WIDE) stage_wide_mask(a, s_tm, wm, b, c.tid);
  for (bool first = true, next = true; next; first = false) {
    const bool whole = off == 0 && lim == np;
    const int part = whole ? -1 : (first ? 2 * w : 2 * w + 1) * a.RG + rg;
    stream_stages<T, D, MT, true, WIDE>(ws, a, c, s_ring, s_pgoff, b, kvh, row0, L, nc, range.x,
                                        range.y, int2{0, 0}, wm);
    const int fb = b, fkvh = kvh;
    // the next unit, if the range reaches past its leading pairs (the range
    // ends at or before the total, so the next unit exists when it starts
    // inside the range)
    next = false;
    if (lim == np && ustart + np + X < end) {
      ustart += np + X;
      if (++kvh == a.Hkv) {
        kvh = 0;
        ++b;
        L = s_len[b];
        np = unit_pairs(a, L);
      }
      off = 0;
      lim = max(0, min(np + X, end - ustart) - X);
      next = lim > 0;
    }
    // The next piece's page ids, Q fragments and causal-row count are
    // requested before this piece's rows are merged and stored, and its
    // first window's page offsets are written during the merge, before any
    // store is issued: the next piece then starts its DMAs at once, their
    // latency overlapping that of the stores (the Q registers are free once
    // the stages are streamed).
    int2 pg{0, 0};
    if (next) {
      range = stage_range();
      pg = table_pair(a, a.page_table + (size_t)b * a.max_pages, range.x + c.tid);
      load_q<T, D, MT>(ws, a, b, kvh, row0, c.rs, c.n, c.grp, false);
      nc = causal_rows(a, b);
    }
    finish_unit<T, D, MT>(ws, a, c, s_ring, fb, fkvh, row0, part, [&] {
      if (next) stage_first(range, pg);
      if constexpr (WIDE)
        if (next && b != fb && a.tree_per_req) stage_wide_mask(a, s_tm, wm, b, c.tid);
    });
    reset_state(ws);
  }
}

constexpr int kCombineFastPieces = 8;  // partial states loaded together per merge step

// Merge of n partial states (unnormalised output, max m and sum l in the
// log2 domain) for the 4 output dims 4 d4 .. 4 d4 + 3 of one row: piece i's
// state sits at partial row prow(i). Pieces are taken kCombineFastPieces at
// a time, every load of a chunk issued before any is used; the running
// (max, sum, output) is rescaled when a chunk raises the maximum. Returns the
// unnormalised output acc, its max mm and sum ll.
template <int D, typename F>
__device__ __forceinline__ void merge_pieces(const AttnArgs& a, int n, F prow, int d4, float& mm,
                                             float& ll, floatx4& acc) {
  mm = kNegBig;
  ll = 0.f;
  acc = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n; c0 += kCombineFastPieces) {
    float2 ml[kCombineFastPieces];
    floatx4 po[kCombineFastPieces];
#pragma unroll
    for (int i = 0; i < kCombineFastPieces; ++i) {
      if (c0 + i >= n) break;
      const size_t pr = prow(c0 + i);
      ml[i] = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
      po[i] = *reinterpret_cast<const floatx4*>(a.part_o + pr * D + 4 * d4);
    }
    float mc = mm;
#pragma unroll
    for (int i = 0; i < kCombineFastPieces; ++i)
      if (c0 + i < n) mc = fmaxf(mc, ml[i].x);
    const float sc = __builtin_amdgcn_exp2f(mm - mc);
    ll *= sc;
    acc *= sc;
    mm = mc;
#pragma unroll
    for (int i = 0; i < kCombineFastPieces; ++i) {
      if (c0 + i >= n) break;
      const float w = __builtin_amdgcn_exp2f(ml[i].x - mm);
      ll += w * ml[i].y;
      acc += w * po[i];
    }
  }
}

// Merge of the units cut by range boundaries. Boundary k (k = 1 .. T - 1,
// between teams) merges the unit containing weighted pair start(k) if the
// boundary splits the unit's stage pairs and no earlier boundary does (so
// each cut unit is merged once); each boundary's rows are spread over RG x
// kCombineRowGroups blocks.
constexpr int kCombineRowGroups = 4;
constexpr int kCombineMaxPieces = 256;  // a unit is shared by at most G workgroups

template <typename T, int D>
__global__ __launch_bounds__(256) void block_attn_boundary_combine_kernel(AttnArgs a) {
  __shared__ int s_pre[kMaxBalancedBatch + 1];
  __shared__ int s_tmp[4];
  __shared__ int s_slot[kCombineMaxPieces];
  const int G = a.G / a.RG, per_k = a.RG * kCombineRowGroups;
  const int k = blockIdx.x / per_k + 1, grp = (blockIdx.x % per_k) / kCombineRowGroups;
  const int rg = blockIdx.x % kCombineRowGroups, row0 = grp * a.M;
  const int total = balanced_prefix(a, s_pre, s_tmp, false);
  const int sk = range_start(total, k, G), sk1 = range_start(total, k - 1, G);
  if (sk >= total || sk1 >= sk) return;
  const int b = request_of(s_pre, a.bs, sk);
  const int nw = unit_weight(a, clamped_len(a, b, false));
  const int kvh = (sk - s_pre[b]) / nw;
  const int u0 = s_pre[b] + kvh * nw, u1 = u0 + nw;  // the unit's weighted pairs [u0, u1)
  const int s0 = u0 + a.piece_cost;                   // its first stage pair
  if (sk <= s0 || sk1 > s0) return;  // no stage pair before the cut, or cut at an earlier boundary
  // pieces: workgroups k - 1 .. wb with a non-empty range; the first one's
  // piece sits in its second slot unless the unit is that workgroup's first
  if (threadIdx.x == 0) {
    int n = 0;
    for (int wg = k - 1; wg < G && range_start(total, wg, G) < u1; ++wg) {
      if (range_start(total, wg, G) >= range_start(total, wg + 1, G)) continue;
      if (n < kCombineMaxPieces)
        s_slot[n] = (wg == k - 1 && u0 > sk1 ? 2 * wg + 1 : 2 * wg) * a.RG + grp;
      ++n;
    }
    s_tmp[0] = min(n, kCombineMaxPieces);
  }
  __syncthreads();
  const int npc = s_tmp[0];
  // local rows [r0, r1) of the unit's row group (rows past Mt do not exist)
  const int rows = min(a.M, a.Mt - row0);
  const int rpb = (rows + kCombineRowGroups - 1) / kCombineRowGroups;
  const int r0 = rg * rpb, r1 = min(rows, r0 + rpb);
  if (r0 >= r1) return;
  const int n4 = (r1 - r0) * (D / 4);
  for (int e = threadIdx.x; e < n4; e += blockDim.x) {
    const int rl = e / (D / 4), d4 = e - rl * (D / 4), r = r0 + rl;
    float mm, ll;
    floatx4 acc;
    merge_pieces<D>(a, npc, [&](int i) { return (size_t)s_slot[i] * a.M + r; }, d4, mm, ll, acc);
    const int rr = row0 + r, ii = rr / a.g, hl = rr - ii * a.g;
    const size_t orow = (size_t)(b * a.B + ii) * a.Hq + kvh * a.g + hl;
    if (d4 == 0 && a.lse) a.lse[orow] = (mm + __log2f(ll)) * kLn2;
    Frag<T>::store4(reinterpret_cast<T*>(a.o) + orow * D + 4 * d4, acc * (1.0f / ll));
  }
}

// Split-KV merge: O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^(m_s - max m),
// one workgroup per (request, KV head), a separate launch after the splits.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_attn_combine_kernel(AttnArgs a) {
  const int unit = blockIdx.x;
  const UnitRef u = unit_ref(a, unit);
  const int b = u.b, kvh = u.kvh;
  const int S = a.splits;
  const int rows = min(a.M, a.Mt - u.row0);  // local rows of the unit's row group
  const size_t part0 = (size_t)unit * S;
  const int n4 = rows * (D / 4);
  for (int e = threadIdx.x; e < n4; e += blockDim.x) {
    const int r = e / (D / 4), d4 = e - r * (D / 4);
    float mm, ll;
    floatx4 acc;
    merge_pieces<D>(a, S, [&](int s2) { return (part0 + s2) * a.M + r; }, d4, mm, ll, acc);
    const int rr = u.row0 + r, i = rr / a.g, hl = rr - i * a.g;
    const size_t orow = (size_t)(b * a.B + i) * a.Hq + kvh * a.g + hl;
    if (d4 == 0 && a.lse) a.lse[orow] = (mm + __log2f(ll)) * kLn2;
    Frag<T>::store4(reinterpret_cast<T*>(a.o) + orow * D + 4 * d4, acc * (1.0f / ll));
  }
}

// ------------------------------------------------------------------ launch
template <typename T, int D>
static hipError_t launch_dt(const AttnArgs& a, int total_blocks, hipStream_t stream) {
  const dim3 block(kWave * kWaves);
  if (a.balanced) {
    const dim3 grid(a.G);
    if (a.tree_words > 1) {  // TREE blocks of more than 64 nodes
      if constexpr (sizeof(T) == 4 && D == 128) {
        return hipErrorInvalidValue;  // no LDS room for the mask words: the planner never asks
      } else if (a.M > 64) {
        hipLaunchKernelGGL((block_attn_balanced_kernel<T, D, 2, true>), grid, block, 0, stream, a);
      } else {
        hipLaunchKernelGGL((block_attn_balanced_kernel<T, D, 1, true>), grid, block, 0, stream, a);
      }
    } else if (a.M > 64) {
      hipLaunchKernelGGL((block_attn_balanced_kernel<T, D, 2>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((block_attn_balanced_kernel<T, D, 1>), grid, block, 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    const int teams = a.G / a.RG;
    if (e != hipSuccess || teams < 2) return e;
    hipLaunchKernelGGL((block_attn_boundary_combine_kernel<T, D>),
                       dim3((teams - 1) * a.RG * kCombineRowGroups), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(total_blocks);
  if (a.tree_words > 1) {  // TREE blocks of more than 64 nodes
    if (a.M > 64)
      hipLaunchKernelGGL((block_attn_kernel<T, D, 2, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((block_attn_kernel<T, D, 1, true>), grid, block, 0, stream, a);
  } else if (a.M > 64) {
    hipLaunchKernelGGL((block_attn_kernel<T, D, 2>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((block_attn_kernel<T, D, 1>), grid, block, 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((block_attn_combine_kernel<T, D>), dim3(a.bs * a.Hv), dim3(256), 0, stream, a);
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
