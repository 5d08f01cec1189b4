// Launch stubs for the host-side sanitizer test: every entry point's host
// path (argument checks, planning, argument packing) runs, and the stub checks
// the plan it is handed instead of launching anything. No GPU is touched.
#include <cstdio>
#include <cstdlib>

#include "kernels.h"

namespace specattn {

static void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "plan check failed: %s\n", what);
    std::abort();
  }
}

hipError_t launch_block_attn(const AttnArgs& a, bool bf16, int D, int total_blocks, hipStream_t) {
  const bool f32 = !bf16;
  require(a.g * a.B == a.Mt, "Mt = g * B");
  require(a.M >= 1 && a.M <= 128 && a.RG >= 1 && (long long)a.RG * a.M >= a.Mt, "row groups cover Mt");
  require((a.RG - 1) * a.M < a.Mt, "no empty row group");
  require(a.Hv == a.Hkv * a.RG, "Hv");
  require(D == 64 || D == 128, "D");
  if (a.mode == 3) {
    require(a.tree && a.tree_words == (a.B + 63) / 64 && a.tree_words <= 8, "tree mask words");
    require(a.tree_words == 1 || !a.balanced || !(f32 && D == 128),
            "fp32 D 128 wide trees take the split schedule");
  } else {
    require(a.tree_words == 1, "one mask word outside TREE mode");
  }
  if (a.balanced) {
    require(a.G >= 1 && (a.RG == 1 || a.G % (8 * a.RG) == 0), "balanced grid of teams");
    require(a.part_o && a.part_ml, "balanced workspace");
  } else {
    require(total_blocks == a.bs * a.Hv * a.splits, "grid = units x splits");
    require(a.splits == 1 || (a.part_o && a.part_ml), "split workspace");
    require(a.splits >= 1 && a.steps_per_split >= 1, "split plan");
  }
  return hipErrorInvalidValue;
}
hipError_t launch_prepare_block(const PrepareArgs& a, hipStream_t) {
  require(a.bs > 0 && a.B > 0, "prepare sizes");
  return hipErrorInvalidValue;
}
hipError_t launch_prepare_tree(const PrepareTreeArgs& a, hipStream_t) {
  require(a.bs > 0 && a.N >= 1 && a.N <= kMaxTreeNodes && a.parent, "prepare_tree sizes");
  return hipErrorInvalidValue;
}
hipError_t launch_quadratic_handoff(const HandoffArgs& h, bool, hipStream_t) {
  require(h.k >= 1 && h.k <= kMaxQuadK && h.n == (h.k + 1) * (h.k + 1), "handoff layout");
  require(!h.next_block || h.bonus, "handoff block needs the bonus");
  require(h.part_v && h.part_i && h.S >= 1 && h.S <= 16 && h.seg_len % 8 == 0 &&
              (long long)h.S * h.seg_len >= h.V && (long long)(h.S - 1) * h.seg_len < h.V,
          "handoff segments cover the row");
  return hipErrorInvalidValue;
}
hipError_t launch_argmax_rows(const void*, bool, int rows, int V, int32_t*, hipStream_t) {
  require(rows > 0 && V > 0, "argmax sizes");
  return hipErrorInvalidValue;
}
hipError_t launch_accept(const AcceptArgs& a, hipStream_t) {
  require(a.nchunk >= 1 && (long long)a.nchunk * a.chunk >= a.V, "chunks cover V");
  require(a.partial && a.jbuf, "accept workspace");
  require(!a.next_ids || (a.next_pos && a.next_loc && a.next_tab && a.next_B > 0), "next block");
  return hipErrorInvalidValue;
}
hipError_t launch_accept_quadratic(const AcceptArgs& a, bool, hipStream_t) {
  require(a.nchunk >= 1 && (long long)a.nchunk * a.chunk >= a.V, "chunks cover V");
  require(a.partial && a.jbuf && a.quad_part_v && a.quad_part_i, "quadratic workspace");
  require(a.quad_n == (a.K + 1) * (a.K + 1) && a.K <= kMaxQuadK, "quadratic layout");
  require(a.quad_S >= 1 && a.quad_seg % 8 == 0 && (long long)a.quad_S * a.quad_seg >= a.V,
          "hand-off segments cover the row");
  require(a.commit_k && a.commit_v && a.commit_tab && a.commit_freed && a.commit_Hkv > 0,
          "commit arguments");
  return hipErrorInvalidValue;
}
hipError_t launch_greedy_accept(const AcceptArgs& a, hipStream_t) {
  require(a.greedy_ids != nullptr, "greedy workspace");
  return hipErrorInvalidValue;
}
hipError_t launch_accept_tree(const AcceptArgs& a, hipStream_t) {
  require(a.nchunk >= 1 && (long long)a.nchunk * a.chunk >= a.V, "chunks cover V");
  require(a.partial && a.jbuf && a.pathbuf, "tree workspace");
  require(!a.commit_k || (a.commit_v && a.commit_tab && a.commit_freed && a.commit_Hkv > 0),
          "commit arguments");
  return hipErrorInvalidValue;
}
hipError_t launch_sampling_filter(const SampArgs& a, bool, hipStream_t) {
  require(a.tmax && a.ntiles * 64 >= a.V, "tile maxima");
  return hipErrorInvalidValue;
}
hipError_t launch_accept_logits(const SampArgs& a, bool, hipStream_t) {
  require(a.tmax && a.kept_ids && a.kept_probs && a.n_kept, "logits accept workspace");
  return hipErrorInvalidValue;
}
hipError_t scratch_on_current_device(void**, size_t*) { return hipErrorNoDevice; }
hipError_t launch_commit_kv(const CommitArgs& a, bool, hipStream_t) {
  require(a.B >= 1 && a.B <= kMaxTreeNodes, "commit block");
  return hipErrorInvalidValue;
}

}  // namespace specattn
