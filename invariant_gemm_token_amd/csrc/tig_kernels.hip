// Leaf-tree contraction, fused LM-head logprob and MoE combine for gfx950.
//
// Method: [IsoExec] "IsoExec: Unified Execution to Eliminate Trainer-Inference
// Mismatch in SkyRL", section "Parallelism-invariant kernels" (K cut into
// contiguous leaves, deterministic matrix-core product with FP32 accumulation
// per leaf, fixed binary combine, figure of the fixed reduction tree).
// [BitRL] "Termina el entrenamiento RL mas rapido: Consistente a nivel de bits,
// ...", sections 2 and 4.1 (one accumulation order for every M, per-token
// logprob identical across batch and phase), 4.4-4.5 (expert outputs combined
// in FP32 in a fixed order).
//
// What decides the bits, and nothing else does:
//   * v_mfma_f32_32x32x16_bf16, k-steps of 16 in ascending order inside a leaf,
//     each leaf accumulator starting at +0;
//   * the balanced adjacent-pair tree over leaves (FP32 adds);
//   * for the softmax: 128-column vocabulary tiles, adjacent-pair trees for the
//     in-tile sum and for the sum over tiles (zero-padded to a power of two).
// The workgroup tile, the k staging depth and the grid order only move data;
// no value in a row ever meets a value from another row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tig_internal.h"

#pragma clang fp contract(off)

namespace tig {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = kBlockM, BN = kBlockN, BK = kBlockK;
constexpr int NTHREADS = 256;                 // 4 waves of 64, 2 x 2 over the tile
constexpr int OPER_BYTES = BM * BK * 2;       // one operand's k-tile: 16 KiB
constexpr int STAGE_BYTES = 2 * OPER_BYTES;   // A and W
constexpr int EPI_LD = BN + 4;                // padded row of the epilogue tile (floats)
constexpr int MAIN_LDS = 2 * STAGE_BYTES;
constexpr int EPI_LDS = BM * EPI_LD * 4;
constexpr int LDS_BYTES = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
constexpr int GROUP_M = 8;                    // m-tiles that share each W tile in L2
constexpr uint32_t OOB = 0xFFFFFFF0u;         // offset past every buffer's range
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;

struct Acc { f32x16 c[2][2]; };   // one wave's 64 x 64 FP32 tile

__device__ __forceinline__ void acc_zero(Acc& a) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) a.c[i][j][v] = 0.0f;
}

// right <- left + right, elementwise FP32 (one node of the leaf tree).
__device__ __forceinline__ void acc_add_left(const Acc& left, Acc& right) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) right.c[i][j][v] = left.c[i][j][v] + right.c[i][j][v];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)RSRC_WORD3);
}

// 16-byte load; offsets at or past the resource's size read as zero.
__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Leaf `leaf` has finished with partial `cur`.  The pending stack `pend`
// holds, at level j, the finished left subtree of 2^j leaves still waiting for
// its right sibling.  Walking up while `leaf` has a 1 bit combines
// left + right; the first 0 bit parks the subtree.  After the last leaf (all
// bits 1) `cur` is the root: ((P0+P1)+(P2+P3))+... for every leaf count.
template <int LEV, int LG>
__device__ __forceinline__ void tree_fold(Acc (&pend)[LG > 0 ? LG : 1], Acc& cur, int leaf) {
  if constexpr (LEV < LG) {
    if (((leaf >> LEV) & 1) == 0) {
      pend[LEV] = cur;
    } else {
      acc_add_left(pend[LEV], cur);
      tree_fold<LEV + 1, LG>(pend, cur, leaf);
    }
  }
}

// Workgroup -> output tile.  Workgroups are dealt to the 8 XCDs round-robin,
// so the blocks of one XCD get one contiguous run of the logical order; that
// order walks GROUP_M m-tiles down each n-tile, so the ~32 workgroups live on
// one XCD share W tiles and A tiles in its L2.  Returns false for padding blocks.
__device__ __forceinline__ bool tile_of(int n_mt, int n_nt, int& mt, int& nt) {
  const int total = n_mt * n_nt;
  const int per_xcd = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int lam = (b & 7) * per_xcd + (b >> 3);
  if (lam >= total) return false;
  const int per_group = GROUP_M * n_nt;
  const int group = lam / per_group;
  const int first = group * GROUP_M;
  const int gm = min(n_mt - first, GROUP_M);
  const int local = lam - group * per_group;
  mt = first + local % gm;
  nt = local / gm;
  return true;
}

inline int grid_blocks(int64_t n_tiles) { return int(((n_tiles + 7) >> 3) << 3); }

// The leaf-tree main loop for one 128 x 128 tile.
//   aoff[i], woff[i]: byte offset of this thread's i-th staged row (rows
//   (tid>>3) + 32 i of the tile) plus its 16-byte column chunk, relative to the
//   resources ra / rw; OOB for a row that does not exist (reads zeros).
// On return `root` holds this wave's 64 x 64 part of the tree result; every
// wave has passed the last barrier, so the LDS may be reused.
template <int LG>
__device__ __forceinline__ void leaf_tree_mainloop(Acc& root, __amdgpu_buffer_rsrc_t ra,
                                                   const uint32_t (&aoff)[4],
                                                   __amdgpu_buffer_rsrc_t rw,
                                                   const uint32_t (&woff)[4],
                                                   int ktiles_per_leaf, char* smem) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Staging: row r = tid>>3 (+32 i), 16-byte chunk c = tid&7 stored at chunk
  // c ^ (r & 7) of the 128-byte LDS row, so the 32 rows one fragment read
  // touches fall in distinct banks.
  const int srow = tid >> 3;
  const uint32_t st_off = uint32_t(srow * 128 + (((tid & 7) ^ (srow & 7)) << 4));
  // Fragments: lane reads row (lane & 31) of a 32-row block at k-chunk
  // 2 s + (lane >> 5) of k-step s.
  const int fr = lane & 31, fk = lane >> 5;
  const uint32_t a_rd0 = uint32_t((wm * 64 + fr) * 128), a_rd1 = a_rd0 + 32 * 128;
  const uint32_t w_rd0 = uint32_t(OPER_BYTES + (wn * 64 + fr) * 128), w_rd1 = w_rd0 + 32 * 128;

  constexpr int L = 1 << LG;
  const int T = L * ktiles_per_leaf;

  i32x4 ga[4], gw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ga[i] = load16(ra, aoff[i]);
    gw[i] = load16(rw, woff[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<i32x4*>(smem + st_off + i * 4096) = ga[i];
    *reinterpret_cast<i32x4*>(smem + OPER_BYTES + st_off + i * 4096) = gw[i];
  }
  __syncthreads();

  Acc pend[LG > 0 ? LG : 1];
  Acc cur;
  int g = 0;
  for (int leaf = 0; leaf < L; ++leaf) {
    acc_zero(cur);
    for (int j = 0; j < ktiles_per_leaf; ++j, ++g) {
      const bool more = (g + 1) < T;
      if (more) {
        const uint32_t kb = uint32_t(g + 1) * (BK * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ga[i] = load16(ra, aoff[i] == OOB ? OOB : aoff[i] + kb);
          gw[i] = load16(rw, woff[i] == OOB ? OOB : woff[i] + kb);
        }
      }
      const char* base = smem + (g & 1) * STAGE_BYTES;
#pragma unroll
      for (int s = 0; s < BK / kMfmaK; ++s) {
        const uint32_t ch = uint32_t(((2 * s + fk) ^ (fr & 7)) << 4);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(base + a_rd0 + ch);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(base + a_rd1 + ch);
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(base + w_rd0 + ch);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(base + w_rd1 + ch);
        cur.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, cur.c[0][0], 0, 0, 0);
        cur.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, cur.c[0][1], 0, 0, 0);
        cur.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, cur.c[1][0], 0, 0, 0);
        cur.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, cur.c[1][1], 0, 0, 0);
      }
      if (more) {
        char* nb = smem + ((g + 1) & 1) * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<i32x4*>(nb + st_off + i * 4096) = ga[i];
          *reinterpret_cast<i32x4*>(nb + OPER_BYTES + st_off + i * 4096) = gw[i];
        }
      }
      __syncthreads();
    }
    tree_fold<0, LG>(pend, cur, leaf);
  }
  root = cur;
}

// Output position of accumulator element (block i, j; register v) of a lane:
// the 32 x 32 result puts column (lane & 31) in the lane and rows
// 8 (v / 4) + 4 (lane / 32) + (v % 4) in the registers.
__device__ __forceinline__ int acc_row(int wm, int i, int v, int lane) {
  return wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------------------
// tree_gemm: C = leaf-tree(A W^T), FP32 or bf16 out.
// ---------------------------------------------------------------------------
template <int LG, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tree_gemm_kernel(const uint16_t* __restrict__ A, int64_t lda,
                      const uint16_t* __restrict__ W, int64_t ldw,
                      void* __restrict__ C, int64_t ldc,
                      int64_t M, int64_t N, int ktiles_per_leaf, int n_mt, int n_nt) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  int mt, nt;
  if (!tile_of(n_mt, n_nt, mt, nt)) return;
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_w = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + m0 * lda, uint32_t(rows_a * lda * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + n0 * ldw, uint32_t(rows_w * ldw * 2));
  const int tid = threadIdx.x;
  uint32_t aoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    aoff[i] = r < rows_a ? uint32_t(r * lda * 2 + (tid & 7) * 16) : OOB;
    woff[i] = r < rows_w ? uint32_t(r * ldw * 2 + (tid & 7) * 16) : OOB;
  }
  Acc acc;
  leaf_tree_mainloop<LG>(acc, ra, aoff, rw, woff, ktiles_per_leaf, smem);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + acc_col(wn, j, lane);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + acc_row(wm, i, v, lane);
        if (row >= M) continue;
        if (EPI == kEpiF32)
          static_cast<float*>(C)[row * ldc + col] = acc.c[i][j][v];
        else
          static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16_rne(acc.c[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// logprob, pass 1: per (row, 128-column vocabulary tile) the max m_t and
// s_t = sum exp2((x - m_t) log2 e), plus the sampled token's logit.
// ---------------------------------------------------------------------------

// Balanced adjacent-pair tree over 64 values: (v0+v1), (v2+v3), ... level by level.
__device__ __forceinline__ float pair_tree_64(float (&e)[64]) {
#pragma unroll
  for (int w = 1; w < 64; w *= 2)
#pragma unroll
    for (int j = 0; j < 64; j += 2 * w) e[j] = e[j] + e[j + w];
  return e[0];
}

template <int LG>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void logprob_tile_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ W,
                         const int64_t* __restrict__ ids, float2* __restrict__ part,
                         float* __restrict__ xid, int64_t M, int64_t K, int64_t V,
                         int ktiles_per_leaf, int n_mt, int n_nt) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  int mt, nt;
  if (!tile_of(n_mt, n_nt, mt, nt)) return;
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
  const int64_t rows_w = V - n0 < BN ? V - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(H + m0 * K, uint32_t(rows_a * K * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + n0 * K, uint32_t(rows_w * K * 2));
  const int tid = threadIdx.x;
  uint32_t aoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    aoff[i] = r < rows_a ? uint32_t(r * K * 2 + (tid & 7) * 16) : OOB;
    woff[i] = r < rows_w ? uint32_t(r * K * 2 + (tid & 7) * 16) : OOB;
  }
  Acc acc;
  leaf_tree_mainloop<LG>(acc, ra, aoff, rw, woff, ktiles_per_leaf, smem);

  // Transpose the 128 x 128 FP32 tile through LDS so that each thread owns
  // half a row: thread t takes row t / 2, columns 64 (t % 2) .. + 63.
  float* E = reinterpret_cast<float*>(smem);
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        E[acc_row(wm, i, v, lane) * EPI_LD + acc_col(wn, j, lane)] = acc.c[i][j][v];
  __syncthreads();

  const int r = tid >> 1, h = tid & 1;
  const int64_t row = m0 + r;
  const int valid = int(rows_w) - 64 * h;   // valid columns in this half (may be <= 0)
  const float* src = E + r * EPI_LD + 64 * h;
  float x[64];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float4 t4 = *reinterpret_cast<const float4*>(src + 4 * q);
    x[4 * q + 0] = t4.x; x[4 * q + 1] = t4.y; x[4 * q + 2] = t4.z; x[4 * q + 3] = t4.w;
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < 64; ++c)
    if (c < valid) mx = fmaxf(mx, x[c]);
  mx = fmaxf(mx, __shfl_xor(mx, 1));   // tile max over both halves (exact)
#pragma unroll
  for (int c = 0; c < 64; ++c)
    x[c] = c < valid ? __builtin_amdgcn_exp2f((x[c] - mx) * LOG2E) : 0.0f;
  const float s_half = pair_tree_64(x);
  const float s_other = __shfl_xor(s_half, 1);
  const float s_tile = h == 0 ? s_half + s_other : s_other + s_half;   // top node: half 0 + half 1
  if (row < M) {
    const int n_vt = n_nt;
    if (h == 0) part[row * n_vt + nt] = make_float2(mx, s_tile);
    const int64_t id = ids[row];
    const int64_t c = id - n0 - 64 * h;
    if (id >= 0 && id < V && c >= 0 && c < 64) xid[row] = src[c];
  }
}

// ---------------------------------------------------------------------------
// logprob, pass 2: one wave per row combines the vocabulary tiles.
//   g = max_t m_t (exact); S = sum_t s_t exp2((m_t - g) log2 e) by the
//   balanced adjacent-pair tree over the tiles zero-padded to P = 64 * 2^q:
//   lane l owns tiles [l 2^q, (l+1) 2^q) and folds them with a pending stack;
//   the xor butterfly over lanes (masks 1, 2, ..., 32) forms the upper levels.
// ---------------------------------------------------------------------------
constexpr int MAX_Q = 10;   // 2^10 tiles per lane: up to 65536 tiles

// Same pending-stack fold as tree_fold, on one float per lane, for a chunk of
// 2^q terms (q <= MAX_Q): term i parks at its lowest 0 bit below q; the last
// term (all q bits 1) leaves the chunk's root in `cur`.
template <int LEV>
__device__ __forceinline__ void scalar_fold(float (&pend)[MAX_Q], float& cur, int i, int q) {
  if constexpr (LEV < MAX_Q) {
    if (LEV == q) return;
    if (((i >> LEV) & 1) == 0) {
      pend[LEV] = cur;
    } else {
      cur = pend[LEV] + cur;
      scalar_fold<LEV + 1>(pend, cur, i, q);
    }
  }
}

__global__ __launch_bounds__(256) void logprob_combine_kernel(
    const float2* __restrict__ part, const float* __restrict__ xid,
    const int64_t* __restrict__ ids, float* __restrict__ logprob, float* __restrict__ lse,
    int64_t M, int n_vt, int q, int64_t V) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float2* pr = part + row * n_vt;
  float g = -__builtin_inff();
  for (int t = lane; t < n_vt; t += 64) g = fmaxf(g, pr[t].x);
#pragma unroll
  for (int m = 1; m < 64; m *= 2) g = fmaxf(g, __shfl_xor(g, m));

  const int c = 1 << q;
  float pend[MAX_Q];
  float cur = 0.0f;
  for (int i = 0; i < c; ++i) {
    const int t = lane * c + i;
    float term = 0.0f;
    if (t < n_vt) {
      const float2 p = pr[t];
      term = p.y * __builtin_amdgcn_exp2f((p.x - g) * LOG2E);
    }
    cur = term;
    scalar_fold<0>(pend, cur, i, q);
  }
  float S = cur;
#pragma unroll
  for (int m = 1; m < 64; m *= 2) {
    const float o = __shfl_xor(S, m);
    S = (lane & m) ? o + S : S + o;   // lower lane's subtree on the left
  }
  if (lane == 0) {
    const float l = g + __builtin_amdgcn_logf(S) * LN2;
    const int64_t id = ids[row];
    const bool ok = id >= 0 && id < V;
    logprob[row] = ok ? xid[row] - l : __builtin_nanf("");
    if (lse) lse[row] = l;
  }
}

// ---------------------------------------------------------------------------
// MoE: route (stable per-expert row lists), per-expert leaf-tree GEMM with
// indirect rows, fixed-order FP32 combine.
// ---------------------------------------------------------------------------

// One workgroup per expert: scan the (token, slot) pairs in index order and
// list the ones routed to this expert, keeping that order.
__global__ __launch_bounds__(256) void moe_route_kernel(const int32_t* __restrict__ topk_ids,
                                                        int64_t n_pairs, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ rows) {
  __shared__ int wave_tot[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* out = rows + int64_t(e) * n_pairs;
  int base = 0;
  for (int64_t p0 = 0; p0 < n_pairs; p0 += 256) {
    const int64_t p = p0 + tid;
    const bool hit = p < n_pairs && topk_ids[p] == e;
    const uint64_t mask = __ballot(hit);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(mask);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_tot[w];
    if (hit) out[off + before] = int32_t(p);
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  if (tid == 0) counts[e] = base;
}

// Work item -> (expert, m-tile of that expert's rows).  Every workgroup reads
// the expert counts and walks their m-tile counts; items past the end exit.
__device__ __forceinline__ bool moe_item(const int32_t* counts, int n_experts, int item, int& e,
                                         int& mt) {
  int acc = 0;
  for (int x = 0; x < n_experts; ++x) {
    const int tiles = (counts[x] + BM - 1) / BM;
    if (item < acc + tiles) {
      e = x;
      mt = item - acc;
      return true;
    }
    acc += tiles;
  }
  return false;
}

template <int LG>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void moe_gemm_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wx,
                     const int32_t* __restrict__ counts, const int32_t* __restrict__ rows,
                     float* __restrict__ Y, int64_t T, int64_t N, int64_t K, int topk,
                     int n_experts, int64_t n_pairs, int ktiles_per_leaf, int n_items, int n_nt) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  __shared__ int32_t rowmap[BM];
  int item, nt;
  if (!tile_of(n_items, n_nt, item, nt)) return;
  int e, mt;
  if (!moe_item(counts, n_experts, item, e, mt)) return;
  const int cnt = counts[e];
  const int64_t r0 = int64_t(mt) * BM;
  const int64_t n0 = int64_t(nt) * BN;
  const int tid = threadIdx.x;
  if (tid < BM) rowmap[tid] = r0 + tid < cnt ? rows[int64_t(e) * n_pairs + r0 + tid] : -1;
  __syncthreads();
  const int64_t rows_w = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(H, uint32_t(T * K * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(Wx + (int64_t(e) * N + n0) * K, uint32_t(rows_w * K * 2));
  uint32_t aoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int pr = rowmap[r];
    aoff[i] = pr >= 0 ? uint32_t((pr / topk) * K * 2 + (tid & 7) * 16) : OOB;
    woff[i] = r < rows_w ? uint32_t(r * K * 2 + (tid & 7) * 16) : OOB;
  }
  Acc acc;
  leaf_tree_mainloop<LG>(acc, ra, aoff, rw, woff, ktiles_per_leaf, smem);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + acc_col(wn, j, lane);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int pr = rowmap[acc_row(wm, i, v, lane)];
        if (pr < 0) continue;
        Y[int64_t(pr) * N + col] = acc.c[i][j][v];
      }
    }
}

// out[t, n] = sum over the token's experts in ascending id (ties: slot order)
// of w * y, an FP32 multiply then an FP32 add, from +0.
__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* __restrict__ topk_ids,
                                                          const float* __restrict__ topk_w,
                                                          const float* __restrict__ Y,
                                                          float* __restrict__ out, int64_t N,
                                                          int topk, int n_experts) {
  const int64_t t = blockIdx.y;
  const int64_t n = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (n >= N) return;
  int order[kMaxTopk];
  bool bad = false;
  for (int s = 0; s < topk; ++s) {
    const int e = topk_ids[t * topk + s];
    bad |= e < 0 || e >= n_experts;
    int j = s;
    while (j > 0 && topk_ids[t * topk + order[j - 1]] > e) {   // stable insertion
      order[j] = order[j - 1];
      --j;
    }
    order[j] = s;
  }
  float acc = 0.0f;
  for (int k = 0; k < topk; ++k) {
    const int s = order[k];
    const float term = topk_w[t * topk + s] * Y[(t * topk + s) * N + n];
    acc = acc + term;
  }
  out[t * N + n] = bad ? __builtin_nanf("") : acc;
}

template <int LG>
hipError_t launch_tree_gemm_lg(const TreeGemmLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, BM)), n_nt = int(cdiv(p.N, BN));
  const int kpl = int((p.K >> LG) / BK);
  const dim3 grid(grid_blocks(int64_t(n_mt) * n_nt)), block(NTHREADS);
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((tree_gemm_kernel<LG, kEpiF32>), grid, block, 0, s,
                       static_cast<const uint16_t*>(p.A), p.lda, static_cast<const uint16_t*>(p.W),
                       p.ldw, p.C, p.ldc, p.M, p.N, kpl, n_mt, n_nt);
  else
    hipLaunchKernelGGL((tree_gemm_kernel<LG, kEpiBF16>), grid, block, 0, s,
                       static_cast<const uint16_t*>(p.A), p.lda, static_cast<const uint16_t*>(p.W),
                       p.ldw, p.C, p.ldc, p.M, p.N, kpl, n_mt, n_nt);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_logprob_lg(const LogprobLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, BM)), n_vt = int(cdiv(p.V, BN));
  const int kpl = int((p.K >> LG) / BK);
  float2* part = static_cast<float2*>(p.partials);
  hipLaunchKernelGGL((logprob_tile_kernel<LG>), dim3(grid_blocks(int64_t(n_mt) * n_vt)),
                     dim3(NTHREADS), 0, s, static_cast<const uint16_t*>(p.H),
                     static_cast<const uint16_t*>(p.W), p.ids, part, p.xid, p.M, p.K, p.V, kpl,
                     n_mt, n_vt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int q = 0;
  while ((64 << q) < n_vt) ++q;
  hipLaunchKernelGGL(logprob_combine_kernel, dim3(unsigned(cdiv(p.M, 4))), dim3(256), 0, s,
                     part, p.xid, p.ids, p.logprob, p.lse, p.M, n_vt, q, p.V);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_moe_lg(const MoeLaunch& p, hipStream_t s) {
  const int64_t n_pairs = p.T * p.topk;
  hipLaunchKernelGGL(moe_route_kernel, dim3(p.n_experts), dim3(256), 0, s, p.topk_ids, n_pairs,
                     p.counts, p.rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Static bound on the m-tiles of all experts together.
  const int n_items = int(cdiv(n_pairs, BM) + p.n_experts);
  const int n_nt = int(cdiv(p.N, BN));
  const int kpl = int((p.K >> LG) / BK);
  hipLaunchKernelGGL((moe_gemm_kernel<LG>), dim3(grid_blocks(int64_t(n_items) * n_nt)),
                     dim3(NTHREADS), 0, s, static_cast<const uint16_t*>(p.H),
                     static_cast<const uint16_t*>(p.W), p.counts, p.rows, p.Y, p.T, p.N, p.K,
                     p.topk, p.n_experts, n_pairs, kpl, n_items, n_nt);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(unsigned(cdiv(p.N, 256)), unsigned(p.T)), dim3(256),
                     0, s, p.topk_ids, p.topk_w, p.Y, p.out, p.N, p.topk, p.n_experts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_gemm(const TreeGemmLaunch& p, hipStream_t s) {
  switch (p.leaves_log2) {
    case 0: return launch_tree_gemm_lg<0>(p, s);
    case 1: return launch_tree_gemm_lg<1>(p, s);
    case 2: return launch_tree_gemm_lg<2>(p, s);
    case 3: return launch_tree_gemm_lg<3>(p, s);
    case 4: return launch_tree_gemm_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_logprob(const LogprobLaunch& p, hipStream_t s) {
  switch (p.leaves_log2) {
    case 0: return launch_logprob_lg<0>(p, s);
    case 1: return launch_logprob_lg<1>(p, s);
    case 2: return launch_logprob_lg<2>(p, s);
    case 3: return launch_logprob_lg<3>(p, s);
    case 4: return launch_logprob_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe(const MoeLaunch& p, hipStream_t s) {
  switch (p.leaves_log2) {
    case 0: return launch_moe_lg<0>(p, s);
    case 1: return launch_moe_lg<1>(p, s);
    case 2: return launch_moe_lg<2>(p, s);
    case 3: return launch_moe_lg<3>(p, s);
    case 4: return launch_moe_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tig
