// Internal interface between the host-side entry points (tig_api.cpp) and the
// kernel launchers (tig_kernels.hip).  Not installed, not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace tig {

// Workgroup tile and k staging: fixed for every (K, leaves) this library
// accepts, never chosen from M or N.
constexpr int kBlockM = 128;   // MoE expert tiles; the dense kernels' smaller tile
// Tallest tile of the dense kernels: the leaf tree keeps log2(leaves) + 1
// accumulators per output element in registers, so up to 8 leaves leave room
// for 192 rows, 16 leaves for 128.
constexpr int block_m_for_log2(int leaves_log2) { return leaves_log2 <= 3 ? 192 : 128; }
// Rows per tile used for M rows: the tall tile where it needs fewer tiles
// (fewer passes over W), else 128.  Only the schedule depends on it, never a
// value: every output element is computed the same way in either tile.
inline int block_m_for(int64_t M, int leaves_log2) {
  if (block_m_for_log2(leaves_log2) == 192 && (M + 191) / 192 < (M + 127) / 128) return 192;
  return 128;
}
constexpr int kBlockN = 128;   // also the vocabulary tile of the log-softmax
constexpr int kBlockK = 64;
constexpr int kMfmaM = 32, kMfmaN = 32, kMfmaK = 16;
constexpr int kMaxLeavesLog2 = 4;  // leaves <= 16 implemented
constexpr int kMaxVocabTiles = 65536;
constexpr int kMaxTopk = 16;
constexpr int kPolicyVersion = 1;

enum Epilogue { kEpiF32 = 0, kEpiBF16 = 1 };

struct TreeGemmLaunch {
  const void* A; int64_t lda;
  const void* W; int64_t ldw;
  void* C; int64_t ldc;
  int epi;
  int64_t M, N, K;
  int leaves_log2;
};

struct LogprobLaunch {
  const void* H; const void* W; const int64_t* ids;
  float* logprob; float* lse;
  int64_t M, K, V;
  int leaves_log2;
  void* partials;   // float2 [M][n_vtiles]
  float* xleaf;     // float [M][leaves]
};

struct MoeLaunch {
  const void* H; const void* W;
  const int32_t* topk_ids; const float* topk_w;
  float* out;
  int64_t T, N, K;
  int n_experts, topk, leaves_log2;
  int32_t* counts;  // [n_experts]
  int32_t* rows;    // [n_experts][T*topk] pair indices, stable order
  float* Y;         // [T*topk][N] expert outputs (FP32 tree result)
};

// Workspace layout helpers (bytes, 256-aligned sections).
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t logprob_partials_bytes(int64_t M, int64_t V) {
  return align256(size_t(M) * size_t(cdiv(V, kBlockN)) * 8);
}
// partials float2 [M][vocabulary tiles], then the picked logit's leaf values float [M][leaves]
inline size_t logprob_ws_bytes(int64_t M, int64_t V, int leaves) {
  return logprob_partials_bytes(M, V) + align256(size_t(M) * size_t(leaves) * 4);
}
inline size_t moe_counts_bytes(int n_experts) { return align256(size_t(n_experts) * 4); }
inline size_t moe_rows_bytes(int64_t T, int topk, int n_experts) {
  return align256(size_t(n_experts) * size_t(T) * size_t(topk) * 4);
}
inline size_t moe_ws_bytes(int64_t T, int64_t N, int n_experts, int topk) {
  return moe_counts_bytes(n_experts) + moe_rows_bytes(T, topk, n_experts) +
         align256(size_t(T) * size_t(topk) * size_t(N) * 4);
}

// Launchers: enqueue on `stream`, return the first HIP error (hipSuccess if none).
hipError_t launch_tree_gemm(const TreeGemmLaunch& p, hipStream_t stream);
hipError_t launch_logprob(const LogprobLaunch& p, hipStream_t stream);
hipError_t launch_moe(const MoeLaunch& p, hipStream_t stream);

}  // namespace tig
