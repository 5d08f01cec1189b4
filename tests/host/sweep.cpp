// Host-path sweep of the C ABI under AddressSanitizer / UBSan (built with the
// launch stubs of stubs.hip; no GPU): the workspace planners over a grid of
// sizes, every entry point with valid arguments (reaching the stub, which
// checks the plan and returns a launch error) and with invalid ones.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "specattn.h"

static int fails = 0;
#define EXPECT(call, want)                                                                 \
  do {                                                                                     \
    const int got_ = (call);                                                               \
    if (got_ != (want)) {                                                                  \
      std::printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
      ++fails;                                                                             \
    }                                                                                      \
  } while (0)

int main() {
  // never dereferenced: the kernels are stubbed
  void* F = reinterpret_cast<void*>(uintptr_t{4096});
  int32_t* I = static_cast<int32_t*>(F);
  const float* FL = static_cast<const float*>(F);
  const uint64_t* M = static_cast<const uint64_t*>(F);

  // block attention: planner and host path over a grid of shapes
  const int bss[] = {1, 2, 7, 32, 64, 256, 1000, 2048, 3000};
  const int Bs[] = {1, 8, 16, 25, 32, 64, 128, 256, 481, 512};
  const int heads[][2] = {{32, 8}, {16, 4}, {64, 8}, {8, 8}, {24, 8}, {2, 1}};
  const int kvs[] = {1, 100, 1040, 9232, 65536, 1 << 20};
  for (int bs : bss)
    for (int B : Bs)
      for (auto& hh : heads)
        for (int D : {64, 128})
          for (int kv : kvs) {
            const int g = hh[0] / hh[1];
            const size_t ws = block_attn_workspace_bytes(bs, B, hh[0], hh[1], D, kv);
            const int max_pages = (kv + 2 * B) / 16 + 2;
            const int want = g * B > 2048 ? SPEC_EINVAL : SPEC_EHIP;
            EXPECT(block_attn(SPEC_CAUSAL, 0, nullptr, SPEC_BF16, bs, B, hh[0], hh[1], D, 16,
                              max_pages, 1 << 20, kv, F, F, F, I, I, 0.0f, F, nullptr, F, ws,
                              nullptr, nullptr),
                   want);
            EXPECT(block_attn_tree(M, 1, SPEC_F32, bs, B, hh[0], hh[1], D, 32, max_pages,
                                   1 << 20, kv, F, F, F, I, I, 0.5f, F, nullptr,
                                   F, ws, I, nullptr),
                   want);
            if (ws > 0)
              EXPECT(block_attn(SPEC_BIDIR, 0, nullptr, SPEC_BF16, bs, B, hh[0], hh[1], D, 16,
                                max_pages, 1 << 20, kv, F, F, F, I, I, 0.0f, F, nullptr, F,
                                ws - 1, nullptr, nullptr),
                     g * B > 2048 ? SPEC_EINVAL : SPEC_ENOSPC);
          }
  EXPECT(block_attn(SPEC_MIXED, 17, nullptr, SPEC_BF16, 2, 16, 32, 8, 128, 16, 80, 200, 1040, F,
                    F, F, I, I, 0.0f, F, nullptr, F, 1 << 30, nullptr, nullptr),
         SPEC_EINVAL);
  EXPECT(block_attn(SPEC_CAUSAL, 0, nullptr, SPEC_BF16, 2, 16, 30, 8, 128, 16, 80, 200, 1040, F,
                    F, F, I, I, 0.0f, F, nullptr, F, 1 << 30, nullptr, nullptr),
         SPEC_EINVAL);

  // prepare, argmax
  EXPECT(spec_prepare_block(32, 16, 16, 80, 300, 7, I, I, I, I, I, I, I, I, nullptr), SPEC_EHIP);
  EXPECT(spec_prepare_block(0, 16, 16, 80, 300, 7, I, I, I, I, I, I, I, I, nullptr), SPEC_EINVAL);
  for (int N : {1, 5, 25, 64, 65, 481, 512})
    for (int per : {0, 1}) {
      EXPECT(spec_prepare_tree(32, N, 16, 80, 300, 7, I, I, I, I, per, I, I, I, I, I, nullptr),
             SPEC_EHIP);
      EXPECT(spec_prepare_tree(32, N, 16, 80, 300, 7, I, I, I, I, per, nullptr, I, I, I, nullptr,
                               nullptr),
             SPEC_EHIP);
    }
  EXPECT(spec_prepare_tree(32, 513, 16, 80, 300, 7, I, I, I, I, 0, I, I, I, I, I, nullptr),
         SPEC_EINVAL);
  EXPECT(spec_prepare_tree(32, 8, 16, 80, 300, 7, I, I, I, nullptr, 0, I, I, I, I, I, nullptr),
         SPEC_EINVAL);
  for (int bs : {1, 5, 32, 1000})
    for (int k : {1, 2, 4, 7, 8, 15, 21})
      for (int V : {1, 7, 1000, 151936}) {
        const size_t wh = spec_quadratic_handoff_workspace_bytes(bs, k, V);
        EXPECT(spec_quadratic_handoff(bs, k, V, SPEC_BF16, F, I, I, 9, I, I, F, wh, I, nullptr),
               SPEC_EHIP);
        EXPECT(spec_quadratic_handoff(bs, k, V, SPEC_F32, F, I, nullptr, 9, I, nullptr, F, wh, I,
                                      nullptr),
               SPEC_EHIP);
        EXPECT(spec_quadratic_handoff(bs, k, V, SPEC_F32, F, I, nullptr, 9, I, nullptr, F, wh - 1,
                                      I, nullptr),
               SPEC_ENOSPC);
      }
  EXPECT(spec_quadratic_handoff(32, 22, 151936, SPEC_BF16, F, I, I, 9, I, I, F, 1 << 30, I,
                                nullptr),
         SPEC_EINVAL);
  EXPECT(spec_quadratic_handoff(32, 4, 151936, SPEC_BF16, F, I, nullptr, 9, I, I, F, 1 << 30, I,
                                nullptr),
         SPEC_EINVAL);  // a next block needs the bonus
  for (int bs : {1, 32, 600})
    for (int k : {1, 2, 4, 7, 8, 15, 21})
      for (int V : {9, 4099, 151936}) {
        const size_t wq = spec_accept_quadratic_workspace_bytes(bs, k, V);
        EXPECT(spec_accept_quadratic(bs, k, V, FL, FL, I, FL, I, SPEC_BF16, F, 7, I, I, I, I, I, I,
                                     I, I, I, SPEC_BF16, 8, 128, 16, 80, 300, I, F, F, I, F, wq, I,
                                     nullptr),
               SPEC_EHIP);
        EXPECT(spec_accept_quadratic(bs, k, V, FL, FL, I, FL, I, SPEC_F32, F, 7, I, I, I, I, I, I,
                                     nullptr, nullptr, nullptr, SPEC_F32, 2, 64, 32, 80, 300, I, F,
                                     F, I, F, wq - 1, I, nullptr),
               SPEC_ENOSPC);
        EXPECT(spec_accept_quadratic(bs, k, V, FL, FL, I, FL, I, SPEC_F32, F, 7, I, I, I, I, I, I,
                                     nullptr, I, nullptr, SPEC_F32, 2, 64, 32, 80, 300, I, F, F, I,
                                     F, wq, I, nullptr),
               SPEC_EINVAL);  // positions without slots
      }
  EXPECT(spec_accept_quadratic(4, 22, 512, FL, FL, I, FL, I, SPEC_BF16, F, 7, I, I, I, I, I, I, I,
                               I, I, SPEC_BF16, 8, 128, 16, 80, 300, I, F, F, I, F, 1 << 30, I,
                               nullptr),
         SPEC_EINVAL);
  EXPECT(spec_accept_quadratic(4, 4, 512, FL, FL, I, FL, I, SPEC_BF16, F, 7, I, I, I, I, I, I, I,
                               I, I, SPEC_BF16, 8, 96, 16, 80, 300, I, F, F, I, F, 1 << 30, I,
                               nullptr),
         SPEC_ENOTSUP);
  EXPECT(spec_draft_argmax(1984, 157184, SPEC_BF16, F, I, nullptr), SPEC_EHIP);
  EXPECT(spec_draft_argmax(0, 157184, SPEC_BF16, F, I, nullptr), SPEC_EINVAL);

  // accept (stochastic and greedy), tree accept (with and without the commit)
  for (int bs : {1, 32, 256})
    for (int K : {1, 4, 15, 31, 63})
      for (int V : {5, 512, 151936, 524288}) {
        for (int greedy : {0, 1}) {
          const size_t ws = spec_accept_workspace_bytes(bs, K, V, greedy);
          EXPECT(spec_accept(bs, K, V, greedy, FL, FL, I, FL, I, I, I, I, I, I, F, ws, I, nullptr),
                 SPEC_EHIP);
        }
        for (int Bn : {1, 16, 300}) {
          const size_t ws = spec_accept_workspace_bytes(bs, K, V, 0);
          EXPECT(spec_accept_prepare(bs, K, V, 0, FL, FL, I, FL, I, I, I, I, I, I, Bn, 16, 80,
                                     300, 7, I, I, I, I, F, ws, I, nullptr),
                 V > 524288 ? SPEC_ENOTSUP : SPEC_EHIP);
          EXPECT(spec_accept_prepare(bs, K, V, 0, FL, FL, I, FL, I, I, I, I, I, I, Bn, 16, 80,
                                     300, 7, nullptr, I, I, I, F, ws, I, nullptr),
                 SPEC_EINVAL);
          if (ws > 0)
            EXPECT(spec_accept_prepare(bs, K, V, 0, FL, FL, I, FL, I, I, I, I, I, I, Bn, 16, 80,
                                       300, 7, I, I, I, I, F, ws - 1, I, nullptr),
                   SPEC_ENOSPC);
        }
        {
          const size_t ws = spec_accept_workspace_bytes(bs, K, V, 0);
          EXPECT(spec_accept_static(bs, K, V, 0, FL, FL, I, FL, I, I, I, I, I, I, I, nullptr),
                 ws > SPEC_ACCEPT_STATIC_SCRATCH_BYTES ? SPEC_ESCRATCH : SPEC_EHIP);
        }
        const int N = K + 1;
        const size_t wt = spec_accept_tree_workspace_bytes(bs, N, V);
        EXPECT(spec_accept_tree(bs, N, V, I, I, FL, FL, I, I, I, I, I, I, I, F, wt, I, nullptr),
               SPEC_EHIP);
        EXPECT(spec_accept_tree_commit(bs, N, V, I, I, FL, FL, I, I, I, I, I, I, I, SPEC_BF16, 8,
                                       128, 16, 80, 300, I, F, F, I, F, wt, I, nullptr),
               SPEC_EHIP);
        EXPECT(spec_accept_tree(bs, N, V, I, I, FL, FL, I, I, I, I, I, I, I, F, wt - 1, I, nullptr),
               SPEC_ENOSPC);
      }
  for (int bs : {1, 32})
    for (int N : {65, 481, 512})
      for (int V : {5, 151936}) {
        const size_t wt = spec_accept_tree_workspace_bytes(bs, N, V);
        EXPECT(spec_accept_tree(bs, N, V, I, I, FL, FL, I, I, I, I, I, I, I, F, wt, I, nullptr),
               SPEC_EHIP);
        EXPECT(spec_accept_tree(bs, N, V, I, I, FL, FL, I, I, I, I, I, I, I, F, wt - 1, I, nullptr),
               SPEC_ENOSPC);
      }
  EXPECT(spec_accept_tree(4, 513, 512, I, I, FL, FL, I, I, I, I, I, I, I, F, 1 << 30, I, nullptr),
         SPEC_EINVAL);
  EXPECT(spec_accept(4, 64, 512, 0, FL, FL, I, FL, I, I, I, I, I, I, F, 1 << 30, I, nullptr),
         SPEC_EINVAL);

  // sampling parameters and the logits accept
  for (int V : {30, 64, 5003, 151936, 524288})
    for (int k : {1, 50, 64}) {
      const size_t wf = spec_sampling_filter_workspace_bytes(8, V);
      EXPECT(spec_sampling_filter(8, V, SPEC_F32, F, 0.7f, k, 0.95f, I,
                                  static_cast<double*>(F), I, F, wf, nullptr),
             SPEC_EHIP);
      const size_t wl = spec_accept_logits_workspace_bytes(4, 15, V, k);
      EXPECT(spec_accept_logits(4, 15, V, SPEC_BF16, 1.0f, k, 0.95f, F, F, I, FL, I, I, I, I, I,
                                I, F, wl, I, nullptr),
             SPEC_EHIP);
    }
  EXPECT(spec_sampling_filter(8, 151936, SPEC_F32, F, 0.0f, 50, 0.95f, I,
                              static_cast<double*>(F), I, F, 1 << 30, nullptr),
         SPEC_EINVAL);

  // commit
  for (int B : {1, 8, 32, 64, 65, 481, 512})
    EXPECT(spec_commit_kv(SPEC_BF16, 32, B, 8, 128, 16, 80, 300, I, I, I, I, F, F, I, I, nullptr),
           SPEC_EHIP);
  EXPECT(spec_commit_kv(SPEC_BF16, 32, 513, 8, 128, 16, 80, 300, I, I, I, I, F, F, I, I, nullptr),
         SPEC_EINVAL);

  for (int st : {0, -1, -2, -3, -4, -5, -99}) (void)spec_status_string(st);
  std::printf(fails ? "sweep: %d failures\n" : "sweep ok (%d failures)\n", fails);
  return fails ? 1 : 0;
}
