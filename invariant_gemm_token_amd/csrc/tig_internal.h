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
// The logprob path also takes 192-row tiles at 16 leaves: it keeps the left
// half of the leaf tree (the root of leaves 0..7) in global scratch instead
// of registers while the right half streams (see kSpillGrid).
// tig_tree_gemm's tile height: 64, 128 or (up to 8 leaves) 192 rows, whichever
// lets the busiest workgroup of the persistent grid finish first: the number
// of tiles it runs under the schedule's deal over this device's CUs, times the
// measured time of one tile of that height relative to a 128-row tile.
int tree_gemm_block_m(int64_t M, int64_t N, int leaves_log2);
constexpr int kLogprobMaxBlockM = 192;   // tallest tile of the logprob path, at every leaf count
inline int logprob_block_m_for(int64_t M, int leaves_log2) {
  (void)leaves_log2;
  return (M + 191) / 192 < (M + 127) / 128 ? 192 : 128;
}
// Scratch for that left half: one 192 x 128 FP32 tile per workgroup of a
// grid of at most kSpillGrid workgroups.
constexpr int kSpillGrid = 256;
constexpr size_t kSpillBytesPerGroup = 256 * 96 * 4;
constexpr int kBlockN = 128;   // also the vocabulary tile of the log-softmax
// Device array behind tig_logprob_gather_noalloc (callers that cannot allocate):
// one copy on every GPU the library runs on, held until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// Its address on the current device, looked up once per device.
hipError_t noalloc_scratch(void** ptr);
constexpr int kBlockK = 64;
constexpr int kMfmaM = 32, kMfmaN = 32, kMfmaK = 16;
constexpr int kMaxLeavesLog2 = 4;  // leaves <= 16 implemented
constexpr int kMaxVocabTiles = 65536;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 4096;   // per-chunk expert histogram in LDS
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
  float* spill;     // leaves == 16 with 192-row tiles: kSpillGrid * kSpillBytesPerGroup bytes
};

struct MoeLaunch {
  const void* H; const void* W;
  const int32_t* topk_ids; const float* topk_w;
  float* out;
  int64_t T, N, K;
  int n_experts, topk, leaves_log2;
  int32_t* hist;     // [pair chunks of 256][n_experts] pairs of the chunk routed to each expert
  int32_t* first;    // [pair chunks of 256][n_experts] first row of the chunk in the expert's list
  int32_t* counts;   // [n_experts] rows routed to each expert
  int32_t* prefix;   // [n_experts + 1] first row of each expert in Y, then the total
  int32_t* n_items;  // [1] number of (expert, m-tile) work items
  int32_t* items;    // [max items][4]: expert, m-tile, rows of the expert, its first row in Y
  int32_t* tok;      // [n_experts][T*topk] (+ one tile of padding): token of each of the
                     // expert's rows, in ascending (token, slot) order
  int32_t* pos;      // [T*topk] row of (token, slot) inside its expert's list
  float* Y;          // [T*topk][N] expert outputs (FP32 tree result), rows sorted by expert
};

// Workspace layout helpers (bytes, 256-aligned sections).
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t logprob_partials_bytes(int64_t M, int64_t V) {
  return align256(size_t(M) * size_t(cdiv(V, kBlockN)) * 8);
}
inline size_t logprob_xleaf_bytes(int64_t M, int leaves) { return align256(size_t(M) * size_t(leaves) * 4); }
inline size_t logprob_spill_bytes(int64_t M, int leaves) {
  return leaves == 16 && logprob_block_m_for(M, 4) == 192 ? size_t(kSpillGrid) * kSpillBytesPerGroup : 0;
}
// partials float2 [M][vocabulary tiles], then the picked logit's leaf values float [M][leaves],
// then the spill scratch of 16-leaf launches with 192-row tiles
inline size_t logprob_ws_bytes(int64_t M, int64_t V, int leaves) {
  return logprob_partials_bytes(M, V) + logprob_xleaf_bytes(M, leaves) + logprob_spill_bytes(M, leaves);
}
// MoE workspace, in this order (each part 256-byte aligned).
inline int64_t moe_max_items(int64_t T, int topk, int n_experts) {
  return cdiv(T * topk, kBlockM) + n_experts;   // m-tiles of 128 or more rows, one partial per expert
}
struct MoeWorkspace {
  size_t hist, first, counts, prefix, n_items, items, tok, pos, Y, total;
};
inline MoeWorkspace moe_ws_layout(int64_t T, int64_t N, int n_experts, int topk) {
  MoeWorkspace w;
  const size_t pairs = size_t(T) * size_t(topk);
  const size_t chunk_table = align256(size_t(cdiv(int64_t(pairs), 256)) * size_t(n_experts) * 4);
  w.hist = 0;
  w.first = w.hist + chunk_table;
  w.counts = w.first + chunk_table;
  w.prefix = w.counts + align256(size_t(n_experts) * 4);
  w.n_items = w.prefix + align256(size_t(n_experts + 1) * 4);
  w.items = w.n_items + 256;
  w.tok = w.items + align256(size_t(moe_max_items(T, topk, n_experts)) * 16);
  w.pos = w.tok + align256((size_t(n_experts) * pairs + 256) * 4);
  w.Y = w.pos + align256(pairs * 4);
  w.total = w.Y + align256(pairs * size_t(N) * 4);
  return w;
}
inline size_t moe_ws_bytes(int64_t T, int64_t N, int n_experts, int topk) {
  return moe_ws_layout(T, N, n_experts, topk).total;
}

// Expert GEMM on the masked or contiguous layout: per expert, its rows of X
// times its W slice, output rows at the input rows' indices.
constexpr int kMaxGroupExperts = 1024;
struct GroupLaunch {
  const void* X; const int32_t* counts; const void* W; void* Y;
  int epi;                 // kEpiF32 or kEpiBF16
  bool masked;
  int64_t rows;            // rows of X and Y (masked: n_experts * cap)
  int64_t cap, align;      // masked: rows per expert block; contiguous: segment alignment
  int64_t N, K;
  int n_experts, leaves_log2;
  int32_t* n_items;        // workspace: [1] number of work items
  int32_t* items;          // workspace: [max items][4]: expert, first row, rows, 0
};
inline int64_t group_max_items(int64_t rows, int n_experts) {
  return cdiv(rows, kBlockM) + n_experts;   // m-tiles of 128 or more rows, one partial per expert
}
inline size_t group_ws_bytes(int64_t rows, int n_experts) {
  return 256 + align256(size_t(group_max_items(rows, n_experts)) * 16);
}

// Launchers: enqueue on `stream`, return the first HIP error (hipSuccess if none).
hipError_t launch_tree_gemm(const TreeGemmLaunch& p, hipStream_t stream);
hipError_t launch_logprob(const LogprobLaunch& p, hipStream_t stream);
hipError_t launch_moe(const MoeLaunch& p, hipStream_t stream);
hipError_t launch_group_gemm(const GroupLaunch& p, hipStream_t stream);
// Block FP8: quantise bf16 X [R, C] (row stride ldx) into E4M3 bytes Q (row
// stride ldq) and E8M0 scale bytes S [ceil(R/block_rows)][ceil(C/128)];
// block_rows = 1 (activations) or 128 (weights).  Dequantise (Q with row
// stride C) to bf16 [R, C], exact.
hipError_t launch_fp8_quantize(const uint16_t* X, int64_t ldx, uint8_t* Q, int64_t ldq, uint8_t* S, int64_t R,
                               int64_t C, int block_rows, hipStream_t stream);
hipError_t launch_fp8_dequant(const uint8_t* Q, const uint8_t* S, int64_t R, int64_t C, int block_rows,
                              uint16_t* out, hipStream_t stream);
// SiLU(g) * u rounded to bf16 once, then quantised to block FP8 (1 x 128).
hipError_t launch_silu_mul_fp8(const float* GU, int64_t ldgu, uint8_t* Q, int64_t ldq, uint8_t* S, int64_t R,
                               int64_t I, hipStream_t stream);
// W8A8 block-FP8 leaf-tree GEMM on the FP8 matrix cores.  table: workspace
// for the per-call scale table [K/128][scw], scw = fp8_table_width(M, N).
struct Fp8GemmLaunch {
  const uint8_t* QA; const uint8_t* SA; const uint8_t* QW; const uint8_t* SW;
  void* C; int64_t ldc;
  int epi;
  int64_t M, N, K;
  int leaves_log2;
  uint8_t* table; int64_t mrows, scw;
};
inline int64_t fp8_table_rows(int64_t M) { return cdiv(M, 128) * 128; }
inline int64_t fp8_table_width(int64_t M, int64_t N) { return (fp8_table_rows(M) + cdiv(N, 128) + 3) / 4 * 4; }
inline size_t fp8_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return align256(size_t(K / 128) * size_t(fp8_table_width(M, N)));
}
hipError_t launch_fp8_gemm(const Fp8GemmLaunch& p, hipStream_t stream);
// The expert GEMM of the two layouts (as GroupLaunch) on the FP8 matrix cores:
// QX [rows, K] E4M3 with SX [rows, K/128], QW [E, N, K] with SW [E, nb, K/128].
struct Fp8GroupLaunch {
  const uint8_t* QX; const uint8_t* SX; const int32_t* counts; const uint8_t* QW; const uint8_t* SW; void* Y;
  int epi;
  bool masked;
  int64_t rows, cap, align, N, K;
  int n_experts, leaves_log2;
  int32_t* n_items; int32_t* items; uint8_t* table;   // workspace parts
};
inline int64_t fp8_group_table_width(int64_t rows, int n_experts, int64_t N) {
  return (group_max_items(rows, n_experts) * 128 + int64_t(n_experts) * cdiv(N, 128) + 3) / 4 * 4;
}
struct Fp8GroupWs { size_t items, table, total; };
inline Fp8GroupWs fp8_group_ws(int64_t rows, int n_experts, int64_t N, int64_t K) {
  Fp8GroupWs w;
  w.items = 256;
  w.table = w.items + align256(size_t(group_max_items(rows, n_experts)) * 16);
  w.total = w.table + align256(size_t(K / 128) * size_t(fp8_group_table_width(rows, n_experts, N)));
  return w;
}
hipError_t launch_fp8_group_gemm(const Fp8GroupLaunch& p, hipStream_t stream);
// out[r, i] = bf16(SiLU(g) * u) in FP32, g = GU[r, i], u = GU[r, I + i], one rounding.
hipError_t launch_silu_mul(const float* GU, int64_t ldgu, uint16_t* out, int64_t ldo, int64_t rows, int64_t I,
                           hipStream_t stream);
// Deterministic Top-K of positions: one workgroup of kTopkThreads per row,
// kTopkPerThread scores per thread in registers.
constexpr int kTopkThreads = 1024, kTopkPerThread = 64;
constexpr int64_t kTopkMaxLen = int64_t(kTopkThreads) * kTopkPerThread;
hipError_t launch_topk_positions(const float* scores, int64_t ld, const int32_t* lengths, int64_t R, int k,
                                 int32_t* out, hipStream_t stream);
// Router, after its logits are computed: per token the topk largest logits
// and their softmax gates.
constexpr int kMaxRouteExperts = 1024;
// The router's logits (FP32 leaf-tree contraction of H [T, K] and Wr [n_experts, K],
// the same bits as the tree GEMM), on 32-token x 64-expert blocks.
hipError_t launch_router_logits(const void* H, const void* Wr, float* logits, int64_t T, int64_t K,
                                int n_experts, int leaves_log2, hipStream_t s);
hipError_t launch_moe_route(const float* logits, int64_t T, int n_experts, int topk, int32_t* topk_ids,
                            float* topk_w, hipStream_t stream);

}  // namespace tig
