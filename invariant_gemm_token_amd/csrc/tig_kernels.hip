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

#include <type_traits>

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
constexpr int STAGES = 4;                     // LDS ring of k-tiles: 3 in flight, 1 in use
constexpr int RING_BYTES = STAGES * STAGE_BYTES;   // 128 KiB
constexpr int EPI_ROWS = 64;                  // epilogue transposes 64 rows per pass
constexpr int EPI_REGION = EPI_ROWS * BN * 4; // 32 KiB
constexpr int P_LDS = RING_BYTES + EPI_REGION;     // 160 KiB: the whole LDS of a CU
constexpr uint32_t OOB_DMA = 0x80000000u;     // row offset past any tile (stays past it + K*2)
#define LDS_AS __attribute__((address_space(3)))
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
// Persistent leaf-tree pipeline.
//
// One workgroup per CU walks its tiles; the k-tiles of all its tiles form one
// stream that a 4-deep LDS ring keeps 3 k-tiles ahead of the matrix cores.
// Loads go straight from global memory to LDS (buffer_load ... lds), so no
// VGPRs hold staged data, and the waits are explicit vmcnt counts plus a bare
// s_barrier (no fence, which would drain the ring).
// ---------------------------------------------------------------------------

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Barrier without a memory fence; the asm memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
// LDS writes of this wave complete, then barrier.
__device__ __forceinline__ void lds_sync() {
  wait_lgkm0();
  bar();
}

// The tiles of one workgroup.  Blocks are dealt to the 8 XCDs round-robin;
// the blocks of XCD x own the logical tiles [x P, (x+1) P) and take them
// round-robin, so the ~32 workgroups running on one XCD always work on 32
// consecutive logical tiles; the logical order walks GROUP_M m-tiles down each
// n-tile so those 32 share A and W tiles in the XCD's L2.
struct TileSched {
  int n_mt, n_nt, slots, first, end;
  __device__ __forceinline__ void init(int n_mt_, int n_nt_) {
    n_mt = n_mt_;
    n_nt = n_nt_;
    const int total = n_mt * n_nt;
    const int per_xcd = (total + 7) >> 3;
    slots = int(gridDim.x) >> 3;
    const int x = blockIdx.x & 7;
    first = x * per_xcd + int(blockIdx.x >> 3);
    end = min((x + 1) * per_xcd, total);
  }
  __device__ __forceinline__ int count() const {
    return first < end ? (end - first + slots - 1) / slots : 0;
  }
  __device__ __forceinline__ void coords(int i, int& mt, int& nt) const {
    const int lam = first + i * slots;
    const int per_group = GROUP_M * n_nt;
    const int group = lam / per_group;
    const int f = group * GROUP_M;
    const int gm = min(n_mt - f, GROUP_M);
    const int local = lam - group * per_group;
    mt = f + local % gm;
    nt = local / gm;
  }
};

// Dense operands of one launch: A [M, K] (row stride lda), W [N, K] (ldw).
struct DenseOperands {
  const uint16_t* A; int64_t lda; int64_t M;
  const uint16_t* W; int64_t ldw; int64_t N;
};

// Where this lane's 8 DMA loads of a k-tile come from.  Wave w fills the
// 1 KiB segments 4w..4w+3 of the A half and of the W half of a stage; lane i
// of a segment writes LDS bytes 16 i.. of it, i.e. row r = 8 g + i/8 of the
// operand, physical chunk i%8.  Logical chunk c of row r lives at physical
// chunk c ^ ((r >> 1) & 7): with 64 four-byte banks a 256-byte bank line holds
// two rows, and the 16 lanes a 128-bit read serves at once (16 consecutive
// rows, one logical chunk) then hit 16 different 16-byte slots.
struct Loader {
  __amdgpu_buffer_rsrc_t ra, rw;
  uint32_t va[4], vw[4];
};

__device__ __forceinline__ void loader_setup(Loader& L, const DenseOperands& op, int mt, int nt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  const int64_t rows_a = op.M - m0 < BM ? op.M - m0 : BM;
  const int64_t rows_w = op.N - n0 < BN ? op.N - n0 : BN;
  L.ra = make_rsrc(op.A + m0 * op.lda, uint32_t(rows_a * op.lda * 2));
  L.rw = make_rsrc(op.W + n0 * op.ldw, uint32_t(rows_w * op.ldw * 2));
  const int rs = lane >> 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 8 + rs;
    const uint32_t chunk = uint32_t(((lane & 7) ^ ((row >> 1) & 7)) << 4);
    L.va[j] = row < rows_a ? uint32_t(row * op.lda * 2) + chunk : OOB_DMA;
    L.vw[j] = row < rows_w ? uint32_t(row * op.ldw * 2) + chunk : OOB_DMA;
  }
}

// The wave index as a scalar, so LDS destinations are SGPR arithmetic (M0).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ void loader_issue(const Loader& L, char* stage, int kt) {
  const int wave = wave_id();
  const int so = kt * (BK * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.ra, (LDS_AS void*)(stage + (wave * 4 + j) * 1024), 16,
                                             L.va[j], so, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        L.rw, (LDS_AS void*)(stage + OPER_BYTES + (wave * 4 + j) * 1024), 16, L.vw[j], so, 0, 0);
}

// Fragment registers of one k-step: A rows (2 blocks of 32) and W rows (2 blocks).
struct Frags { bf16x8 a0, a1, b0, b1; };

struct FragAddr {
  uint32_t a0, a1, w0, w1;
  int fr, fk;
  __device__ __forceinline__ void read(Frags& f, const char* st, int s) const {
    const uint32_t ch = uint32_t(((2 * s + fk) ^ ((fr >> 1) & 7)) << 4);
    f.a0 = *reinterpret_cast<const bf16x8*>(st + a0 + ch);
    f.a1 = *reinterpret_cast<const bf16x8*>(st + a1 + ch);
    f.b0 = *reinterpret_cast<const bf16x8*>(st + w0 + ch);
    f.b1 = *reinterpret_cast<const bf16x8*>(st + w1 + ch);
  }
};

// First k-step of a leaf: the accumulator input is the constant +0.
__device__ __forceinline__ void mfma4_first(Acc& c, const Frags& f) {
  const f32x16 z = {};
  c.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a0, f.b0, z, 0, 0, 0);
  c.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a0, f.b1, z, 0, 0, 0);
  c.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a1, f.b0, z, 0, 0, 0);
  c.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a1, f.b1, z, 0, 0, 0);
}

__device__ __forceinline__ void mfma4(Acc& c, const Frags& f) {
  c.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a0, f.b0, c.c[0][0], 0, 0, 0);
  c.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a0, f.b1, c.c[0][1], 0, 0, 0);
  c.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a1, f.b0, c.c[1][0], 0, 0, 0);
  c.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a1, f.b1, c.c[1][1], 0, 0, 0);
}

// Scheduling hint for one step: the 4 reads of the next step interleaved with
// the 4 MFMAs of this one.
__device__ __forceinline__ void sched_step() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// Wait until the DMA loads of stage `q` have landed, given how many later
// stages (at most STAGES - 2) have been issued after it.
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= STAGES - 2) wait_vmcnt<8 * (STAGES - 2)>();
  else if (later == 1) wait_vmcnt<8>();
  else wait_vmcnt<0>();
}

// Runs every tile of this workgroup: leaf-tree main loop, then epi(acc, mt, nt).
//
// The k-tiles of all tiles form one stream q = 0 .. total-1, computed as a
// software pipeline: while the last 4 MFMAs of stage q run, the wave has
// already waited for stage q+1, passed the barrier, issued the DMA of stage
// q+STAGES into the buffer stage q-1 just freed, and read the step-0 fragments
// of stage q+1.  At leaf ends the accumulator folds into the pending tree; at
// tile ends the epilogue runs.
template <int LG, class Epi>
__device__ __forceinline__ void leaf_tree_persistent(const DenseOperands& op, int ktiles,
                                                     const TileSched& ts, Epi& epi, char* smem) {
  const int n_my = ts.count();
  if (n_my == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  FragAddr fa;
  fa.fr = lane & 31;
  fa.fk = lane >> 5;
  fa.a0 = uint32_t((wm * 64 + fa.fr) * 128);
  fa.a1 = fa.a0 + 32 * 128;
  fa.w0 = uint32_t(OPER_BYTES + (wn * 64 + fa.fr) * 128);
  fa.w1 = fa.w0 + 32 * 128;
  constexpr int L = 1 << LG;
  const int kpl = ktiles >> LG;
  const int total = n_my * ktiles;

  Loader ld;
  int l_tile = 0, l_kt = 0;
  {
    int mt, nt;
    ts.coords(0, mt, nt);
    loader_setup(ld, op, mt, nt);
  }
  auto issue_next = [&](int stage) {
    loader_issue(ld, smem + (stage % STAGES) * STAGE_BYTES, l_kt);
    if (++l_kt == ktiles) {
      l_kt = 0;
      if (++l_tile < n_my) {
        int mt, nt;
        ts.coords(l_tile, mt, nt);
        loader_setup(ld, op, mt, nt);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < total) issue_next(p);

  Frags f0, f1;
  wait_stage(min(STAGES - 2, total - 1));
  bar();
  if (STAGES - 1 < total) issue_next(STAGES - 1);
  fa.read(f0, smem, 0);

  // One k-tile of the stream: steps 0..2 with the next step's fragments read
  // under the MFMAs; then the hand-over to stage q+1 (wait, barrier, DMA of
  // stage q+STAGES, step-0 fragments of q+1) before the last 4 MFMAs.
  auto stage = [&](Acc& cur, int q, auto first) {
    const char* st = smem + (q % STAGES) * STAGE_BYTES;
    fa.read(f1, st, 1);
    if constexpr (decltype(first)::value) mfma4_first(cur, f0);
    else mfma4(cur, f0);
    sched_step();
    fa.read(f0, st, 2);
    mfma4(cur, f1);
    sched_step();
    fa.read(f1, st, 3);
    mfma4(cur, f0);
    sched_step();
    if (q + 1 < total) {
      wait_stage(min(STAGES - 2, total - 2 - q));
      bar();
      if (q + STAGES < total) issue_next(q + STAGES);
      fa.read(f0, smem + ((q + 1) % STAGES) * STAGE_BYTES, 0);
    }
    mfma4(cur, f1);
  };

  int q = 0;
  for (int ti = 0; ti < n_my; ++ti) {
    Acc pend[LG > 0 ? LG : 1];
    Acc cur;
#pragma unroll 1
    for (int leaf = 0; leaf < L; ++leaf) {
      stage(cur, q++, std::true_type{});
      for (int j = 1; j < kpl; ++j) stage(cur, q++, std::false_type{});
      tree_fold<0, LG>(pend, cur, leaf);
    }
    int mt, nt;
    ts.coords(ti, mt, nt);
    epi(cur, mt, nt, smem + RING_BYTES);
  }
}

// Epilogue: store the tile (FP32, or bf16 by RNE).
template <int EPI>
struct StoreEpi {
  void* C; int64_t ldc; int64_t M, N;
  __device__ __forceinline__ void operator()(const Acc& acc, int mt, int nt, char*) const;
};

// Epilogue: per (row, 128-column vocabulary tile) max and sum of exp2, plus
// the sampled token's logit.  The 128 x 128 tile is transposed through LDS in
// two passes of 64 rows; in a pass, thread t owns row t/4, columns 32 (t%4)..+31.
struct LogprobEpi {
  float2* part; float* xid; const int64_t* ids; int64_t M, V; int n_vt;
  __device__ __forceinline__ void operator()(const Acc& acc, int mt, int nt, char* region) const;
};

// ---------------------------------------------------------------------------
// tree_gemm: C = leaf-tree(A W^T), FP32 or bf16 out.
// ---------------------------------------------------------------------------
template <int EPI>
__device__ __forceinline__ void StoreEpi<EPI>::operator()(const Acc& acc, int mt, int nt, char*) const {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
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

template <int LG, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tree_gemm_kernel(DenseOperands op, void* __restrict__ C, int64_t ldc, int ktiles, int n_mt,
                      int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[P_LDS];
  TileSched ts;
  ts.init(n_mt, n_nt);
  StoreEpi<EPI> epi{C, ldc, op.M, op.N};
  leaf_tree_persistent<LG>(op, ktiles, ts, epi, smem);
}

// ---------------------------------------------------------------------------
// logprob, pass 1: per (row, 128-column vocabulary tile) the max m_t and
// s_t = sum exp2((x - m_t) log2 e) by the balanced adjacent-pair tree over the
// 128 columns (padded columns add +0), plus the sampled token's logit.
// ---------------------------------------------------------------------------

// Balanced adjacent-pair tree over 32 values: (v0+v1), (v2+v3), ... level by level.
__device__ __forceinline__ float pair_tree_32(float (&e)[32]) {
#pragma unroll
  for (int w = 1; w < 32; w *= 2)
#pragma unroll
    for (int j = 0; j < 32; j += 2 * w) e[j] = e[j] + e[j + w];
  return e[0];
}

// [64][128] floats, 16-byte chunk index XOR (row % 32): a row's quarter read by
// 16 rows at once spreads over all banks.
__device__ __forceinline__ int epi_index(int r, int c) {
  return r * BN + (((c >> 2) ^ (r & 31)) << 2) + (c & 3);
}

__device__ __forceinline__ void LogprobEpi::operator()(const Acc& acc, int mt, int nt,
                                                       char* region) const {
  float* E = reinterpret_cast<float*>(region);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  const int valid = int(V - n0 < BN ? V - n0 : BN) - 32 * (tid & 3);  // columns of this quarter
  const int r = tid >> 2, h = tid & 3;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t row = m0 + pass * EPI_ROWS + r;
    // Loaded and consumed on every path, so no load is left pending past the tile.
    const int64_t id = ids[row < M ? row : M - 1];
    const int64_t c = id - n0 - 32 * h;
    const bool mine = row < M && id >= 0 && id < V && c >= 0 && c < 32;
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            E[epi_index(i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3), acc_col(wn, j, lane))] =
                acc.c[i][j][v];
    }
    lds_sync();
    float x[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 t4 = *reinterpret_cast<const float4*>(E + r * BN + (((8 * h + k) ^ (r & 31)) << 2));
      x[4 * k + 0] = t4.x; x[4 * k + 1] = t4.y; x[4 * k + 2] = t4.z; x[4 * k + 3] = t4.w;
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < 32; ++c)
      if (c < valid) mx = fmaxf(mx, x[c]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));     // tile max (exact, any order)
#pragma unroll
    for (int c = 0; c < 32; ++c)
      x[c] = c < valid ? __builtin_amdgcn_exp2f((x[c] - mx) * LOG2E) : 0.0f;
    float sq = pair_tree_32(x);
    float o = __shfl_xor(sq, 1);
    sq = (h & 1) ? o + sq : sq + o;          // (q0 + q1), (q2 + q3)
    o = __shfl_xor(sq, 2);
    sq = (h & 2) ? o + sq : sq + o;          // (q0 + q1) + (q2 + q3)
    if (row < M && h == 0) part[row * n_vt + nt] = make_float2(mx, sq);
    if (mine) xid[row] = E[epi_index(r, int(32 * h + c))];
    lds_sync();
  }
}

template <int LG>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void logprob_tile_kernel(DenseOperands op, int ktiles, int n_mt, int n_nt, float2* __restrict__ part,
                         float* __restrict__ xid, const int64_t* __restrict__ ids) {
  __shared__ __attribute__((aligned(1024))) char smem[P_LDS];
  TileSched ts;
  ts.init(n_mt, n_nt);
  LogprobEpi epi{part, xid, ids, op.M, op.N, n_nt};
  leaf_tree_persistent<LG>(op, ktiles, ts, epi, smem);
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

// Persistent grid: one workgroup per CU (multiple of 8 for the XCD deal), or
// one per tile when there are fewer tiles.  Only the schedule depends on it.
int persistent_grid(int64_t n_tiles) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  const int64_t full = int64_t(cus[dev] / 8) * 8 > 0 ? int64_t(cus[dev] / 8) * 8 : 8;
  const int64_t want = ((n_tiles + 7) / 8) * 8;
  return int(want < full ? want : full);
}

template <int LG>
hipError_t launch_tree_gemm_lg(const TreeGemmLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, BM)), n_nt = int(cdiv(p.N, BN));
  const DenseOperands op{static_cast<const uint16_t*>(p.A), p.lda, p.M,
                         static_cast<const uint16_t*>(p.W), p.ldw, p.N};
  const int ktiles = int(p.K / BK);
  const dim3 grid(persistent_grid(int64_t(n_mt) * n_nt)), block(NTHREADS);
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((tree_gemm_kernel<LG, kEpiF32>), grid, block, 0, s, op, p.C, p.ldc, ktiles,
                       n_mt, n_nt);
  else
    hipLaunchKernelGGL((tree_gemm_kernel<LG, kEpiBF16>), grid, block, 0, s, op, p.C, p.ldc, ktiles,
                       n_mt, n_nt);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_logprob_lg(const LogprobLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, BM)), n_vt = int(cdiv(p.V, BN));
  const DenseOperands op{static_cast<const uint16_t*>(p.H), p.K, p.M,
                         static_cast<const uint16_t*>(p.W), p.K, p.V};
  float2* part = static_cast<float2*>(p.partials);
  hipLaunchKernelGGL((logprob_tile_kernel<LG>), dim3(persistent_grid(int64_t(n_mt) * n_vt)),
                     dim3(NTHREADS), 0, s, op, int(p.K / BK), n_mt, n_vt, part, p.xid, p.ids);
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
