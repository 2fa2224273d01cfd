// Split-KV work planner (host only, no HIP dependency).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

namespace mla {

constexpr int kLkv = 512;
constexpr int kRope = 64;
constexpr int kHead = kLkv + kRope;
constexpr int kGranule = 64;    // keys per planning granule
constexpr int kSegCost = 3;     // cost of a segment (query load + epilogue), in granules
constexpr int kMinChunk = 4;    // smallest chunk taken to top up a part that already has work
constexpr int kGroupRows = 128;  // query rows per head group (one workgroup)
// Largest seq_len a plan accepts: key indices, granule ends (rounded up to 64) and the
// kernels' key arithmetic (a key plus a 32-key tile) all stay far inside int32.
constexpr int32_t kMaxSeqLen = 1 << 30;

struct Segment {
  int32_t req, kv_start, kv_end, partial;  // partial == -1: writes the final output
};

struct Plan {
  int32_t B = 0, Sq = 0, N = 0, head_groups = 0;
  int32_t num_parts = 0, num_partials = 0;
  std::vector<int32_t> part_begin;  // [num_parts + 1] offsets into segs
  std::vector<Segment> segs;
  std::vector<int32_t> reduce;      // [n_reduce * 3]: req, first partial slot, count
};

inline int32_t head_groups(int32_t Sq, int32_t N) { return (Sq * N + kGroupRows - 1) / kGroupRows; }
// Rows of one partial output in the workspace: Sq*N rounded up to whole 32-row blocks
// (a block is stored in the order of the MFMA accumulators, see the decode kernels).
constexpr int64_t partial_rows(int32_t Sq, int32_t N) { return ((int64_t)Sq * N + 31) / 32 * 32; }
// Workspace of a plan: the fp16 partial outputs [num_partials][partial_rows][512], then the
// partial LSEs and the partial row sums, each fp32 [num_partials][Sq*N].
constexpr int64_t partial_o_bytes(int32_t Sq, int32_t N) { return partial_rows(Sq, N) * kLkv * 2; }
constexpr int64_t workspace_bytes(int32_t num_partials, int32_t Sq, int32_t N) {
  return (int64_t)num_partials * (partial_o_bytes(Sq, N) + (int64_t)Sq * N * 8);
}

// Builds the plan; returns false (with a message) only on invalid input.
bool build_plan(const int32_t* seq_lens, int32_t B, int32_t Sq, int32_t N, int32_t num_cus,
                Plan* out, std::string* err);

}  // namespace mla
