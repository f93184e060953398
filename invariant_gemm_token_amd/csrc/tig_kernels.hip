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

#include <mutex>
#include <type_traits>
#include <utility>

#include "tig_internal.h"

#pragma clang fp contract(off)

// Intermediate data of tig_logprob_gather_noalloc, for callers that cannot
// allocate device memory: kNoAllocScratchBytes on every GPU the library runs
// on, for the life of the process, shared by every such call on that GPU.
static __device__ __align__(256) char scratch[tig::kNoAllocScratchBytes];

namespace tig {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4v;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = kBlockM, BN = kBlockN, BK = kBlockK;   // BM: the MoE kernel's tile
constexpr int NTHREADS = 256;                 // 4 waves of 64, 2 x 2 over the tile
constexpr int GROUP_M = 8;                    // m-tiles that share each W tile in L2
constexpr int kLdsBytes = 160 * 1024;         // LDS of one CU: the persistent kernels' ring
#define LDS_AS __attribute__((address_space(3)))
// Read-only for the whole launch: uniform loads through it become scalar loads.
#define CONST_AS __attribute__((address_space(4)))
constexpr uint32_t OOB = 0xFFFFFFF0u;         // offset past every buffer's range
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;

// One wave's (32 MI) x 64 FP32 tile: MI x 2 blocks of 32 x 32.
template <int MI>
struct AccT { f32x16 c[MI][2]; };
using Acc = AccT<2>;

template <int MI>
__device__ __forceinline__ void acc_zero(AccT<MI>& a) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) a.c[i][j][v] = 0.0f;
}

// right <- left + right, elementwise FP32 (one node of the leaf tree).
template <int MI>
__device__ __forceinline__ void acc_add_left(const AccT<MI>& left, AccT<MI>& right) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
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
template <int LEV, int LG, class A>
__device__ __forceinline__ void tree_fold(A (&pend)[LG > 0 ? LG : 1], A& cur, int leaf) {
  if constexpr (LEV < LG) {
    if (((leaf >> LEV) & 1) == 0) {
      pend[LEV] = cur;
    } else {
      acc_add_left(pend[LEV], cur);
      tree_fold<LEV + 1, LG>(pend, cur, leaf);
    }
  }
}

// Output position of accumulator element (block i, j; register v) of a lane:
// the 32 x 32 result puts column (lane & 31) in the lane and rows
// 8 (v / 4) + 4 (lane / 32) + (v % 4) in the registers.
// A wave's rows start at 32 MI wm.
template <int MI = 2>
__device__ __forceinline__ int acc_row(int wm, int i, int v, int lane) {
  return wm * (32 * MI) + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------------------
// Persistent leaf-tree pipeline [IsoExec, Parallelism-invariant kernels].
//
// One workgroup per CU walks its tiles; the k-tiles of all its tiles form one
// stream that an LDS ring (the whole 160 KiB) keeps several k-tiles ahead of
// the matrix cores.  Loads go straight from global memory to LDS
// (buffer_load ... lds), so no VGPRs hold staged data, and the waits are
// explicit vmcnt counts plus a bare s_barrier (no fence, which would drain
// the ring).
//
// The tile is (64 MI) x 128 with 4 waves in 2 x 2, each (32 MI) x 64.  The
// leaf tree keeps log2(L) + 1 accumulators of the wave tile live, which is
// what bounds the tile: MI = 3 (192 x 128, 4 x 96 accumulator registers per
// lane at 8 leaves) up to 8 leaves, MI = 2 (128 x 128) at 16 leaves.  Every
// byte staged through L2 then feeds 77 instead of 64 flops.
// ---------------------------------------------------------------------------

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// vmcnt <= N and lgkmcnt == 0 (this wave's LDS reads have returned).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Barrier without a memory fence; the asm memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
// LDS writes of this wave complete, then barrier.
__device__ __forceinline__ void lds_sync() {
  wait_lgkm0();
  bar();
}

// threadIdx.x through an opaque move: address arithmetic derived from it is
// redone where it is used instead of being hoisted out of the tile loop, where
// it would hold registers through the whole main loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Geometry of the persistent kernels for MI 32-row blocks per wave.
template <int MI>
struct Geo {
  static constexpr int BM = 64 * MI;                    // tile rows
  static constexpr int A_BYTES = BM * BK * 2;           // A k-tile
  static constexpr int STAGE = A_BYTES + BN * BK * 2;   // A and W k-tiles
  static constexpr int STAGES = kLdsBytes / STAGE;      // 5 (MI = 2) or 4 (MI = 3)
  static constexpr int A_SEG = 2 * MI;                  // 1 KiB DMA segments of A per wave
  static constexpr int VM_PER_STAGE = A_SEG + 4;        // DMA instructions per wave per k-tile
  static_assert(STAGES >= 3, "ring too shallow");
  static_assert(VM_PER_STAGE * (STAGES - 2) < 64, "vmcnt range");
};


// The tiles of one workgroup.  Blocks are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8).  When there are enough n-tiles, XCD x owns the
// n-tiles [x N/8, (x+1) N/8) for every m: each W tile then comes from HBM
// once and its re-reads, like all of A, from the memory-side cache.  Inside
// an XCD the logical order walks GROUP_N n-tiles across each m-tile, so the
// ~32 workgroups running there at once (consecutive logical tiles, dealt
// round-robin) share 4 A tiles and 8 W tiles in its L2.  With few n-tiles
// the XCDs split the logical order of the whole grid instead.
constexpr int GROUP_N = 8;

struct TileSched {
  int n_mt, n_nt, slots, first, end, nb, nn, lmask;
  __device__ __forceinline__ void init(int n_mt_, int n_nt_) {
    n_mt = n_mt_;
    n_nt = n_nt_;
    slots = int(gridDim.x) >> 3;
    const int x = blockIdx.x & 7;
    // With a single row of tiles no two workgroups share an operand tile,
    // and the ~32 workgroups of an XCD would otherwise read the same k-slice
    // of their W tiles at the same moment (rows one leading dimension apart,
    // which the L2 serves through few of its channels).  Staggering their
    // leaf order by up to 4 positions spreads them.  With several m-tiles
    // the workgroups of an XCD share operands and run in step.
    lmask = n_mt == 1 ? int(blockIdx.x >> 3) & 3 : 0;
    if (n_nt >= 4 * GROUP_N) {
      nb = int(int64_t(n_nt) * x / 8);
      nn = int(int64_t(n_nt) * (x + 1) / 8) - nb;
      first = int(blockIdx.x >> 3);
      end = nn * n_mt;
    } else {
      const int total = n_mt * n_nt;
      const int per_xcd = (total + 7) >> 3;
      nb = 0;
      nn = n_nt;
      first = x * per_xcd + int(blockIdx.x >> 3);
      end = min((x + 1) * per_xcd, total);
    }
  }
  __device__ __forceinline__ int count() const {
    return first < end ? (end - first + slots - 1) / slots : 0;
  }
  __device__ __forceinline__ void coords(int i, int& mt, int& nt) const {
    const int lam = first + i * slots;
    const int per_group = GROUP_N * n_mt;
    const int group = lam / per_group;
    const int f = group * GROUP_N;
    const int gn = min(nn - f, GROUP_N);
    const int local = lam - group * per_group;
    nt = nb + f + local % gn;
    mt = local / gn;
  }
};

// Dense operands of one launch: A [M, K] (row stride lda), W [N, K] (ldw).
struct DenseOperands {
  const uint16_t* A; int64_t lda; int64_t M;
  const uint16_t* W; int64_t ldw; int64_t N;
};

// Where this lane's DMA loads of a k-tile come from.  Wave w fills the 1 KiB
// segments g = A_SEG w .. A_SEG (w+1) - 1 of the A part and 4w .. 4w+3 of the
// W part of a stage; lane i of segment g writes LDS bytes 16 i.. of it, i.e.
// row r = 8 g + i/8 of the operand, physical chunk i%8.  Logical chunk c of
// row r lives at physical chunk c ^ ((r >> 1) & 7): with 64 four-byte banks a
// 256-byte bank line holds two rows, and the 16 lanes a 128-bit read serves at
// once (16 consecutive rows, one logical chunk) then hit 16 different
// 16-byte slots.  Since (r >> 1) & 7 = 4 (g & 1) + (i / 16), the lane's byte
// offset is off[g & 1] + 16 g ld: two VGPRs per operand and a scalar stride.
// Rows past the tile's last row have offsets past the resource's size and
// read as zero.
// WAUX: cache policy of the W loads (0, or 2 = non-temporal when every W
// tile is read by one workgroup only).
template <int MI, int WAUX = 0>
struct Loader {
  using G = Geo<MI>;
  DenseOperands op;
  __amdgpu_buffer_rsrc_t ra, rw;
  uint32_t oa[2], ow[2];      // lane offsets for even / odd segments
  uint32_t sa, sw;            // 16 * leading dimension in bytes / 2 (one segment of rows)

  __device__ __forceinline__ void setup(int mt, int nt) {
    const int lane = threadIdx.x & 63;
    const int64_t m0 = int64_t(mt) * G::BM, n0 = int64_t(nt) * BN;
    const int64_t rows_a = op.M - m0 < G::BM ? op.M - m0 : G::BM;
    const int64_t rows_w = op.N - n0 < BN ? op.N - n0 : BN;
    ra = make_rsrc(op.A + m0 * op.lda, uint32_t(rows_a * op.lda * 2));
    rw = make_rsrc(op.W + n0 * op.ldw, uint32_t(rows_w * op.ldw * 2));
    const int rs = lane >> 3;
    const uint32_t c0 = uint32_t(((lane & 7) ^ (rs >> 1)) << 4), c1 = c0 ^ 64u;
    oa[0] = uint32_t(rs * op.lda * 2) + c0;
    oa[1] = uint32_t(rs * op.lda * 2) + c1;
    ow[0] = uint32_t(rs * op.ldw * 2) + c0;
    ow[1] = uint32_t(rs * op.ldw * 2) + c1;
    sa = uint32_t(op.lda * 16);
    sw = uint32_t(op.ldw * 16);
  }

  // DMA instruction J (0 <= J < VM_PER_STAGE) of k-tile kt of the current
  // tile into the ring buffer `stage`: J < A_SEG = this wave's A segment J,
  // else its W segment J - A_SEG.  One instruction at a time, so that the
  // issue can be spread evenly between the MFMAs of a stage.
  template <int J>
  __device__ __forceinline__ void seg(char* stage, int kt) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar: M0 arithmetic
    const int so = kt * (BK * 2);
    if constexpr (J < G::A_SEG) {
      const int g = wave * G::A_SEG + J;   // A_SEG is even: g & 1 == J & 1
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LDS_AS void*)(stage + g * 1024), 16,
                                               oa[J & 1] + uint32_t(g) * sa, so, 0, 0);
    } else {
      const int g = wave * 4 + (J - G::A_SEG);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LDS_AS void*)(stage + G::A_BYTES + g * 1024), 16,
                                               ow[J & 1] + uint32_t(g) * sw, so, 0, WAUX);
    }
  }
  template <int J0, int D>
  __device__ __forceinline__ void segs(char* stage, int kt) const {
    if constexpr (D > 0) {
      seg<J0>(stage, kt);
      segs<J0 + 1, D - 1>(stage, kt);
    }
  }
  __device__ __forceinline__ void issue_all(char* stage, int kt) const {
    segs<0, G::VM_PER_STAGE>(stage, kt);
  }
};

// Fragment registers of one k-step: A rows (MI blocks of 32) and W rows (2 blocks).
template <int MI>
struct Frags { bf16x8 a[MI], b0, b1; };

template <int MI>
struct FragAddr {
  uint32_t a0, w0, w1;
  int fr, fk;
  __device__ __forceinline__ void read(Frags<MI>& f, const char* st, int s) const {
    const uint32_t ch = uint32_t(((2 * s + fk) ^ ((fr >> 1) & 7)) << 4);
#pragma unroll
    for (int i = 0; i < MI; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(st + a0 + i * 32 * 128 + ch);
    f.b0 = *reinterpret_cast<const bf16x8*>(st + w0 + ch);
    f.b1 = *reinterpret_cast<const bf16x8*>(st + w1 + ch);
  }
  // Fragment IDX of k-step s alone: A block IDX (IDX < MI), else W block IDX - MI.
  template <int IDX>
  __device__ __forceinline__ void read_one(Frags<MI>& f, const char* st, int s) const {
    const uint32_t ch = uint32_t(((2 * s + fk) ^ ((fr >> 1) & 7)) << 4);
    if constexpr (IDX < MI)
      f.a[IDX] = *reinterpret_cast<const bf16x8*>(st + a0 + IDX * 32 * 128 + ch);
    else if constexpr (IDX == MI)
      f.b0 = *reinterpret_cast<const bf16x8*>(st + w0 + ch);
    else
      f.b1 = *reinterpret_cast<const bf16x8*>(st + w1 + ch);
  }
};

// f(integral_constant<int, K>) for K = 0 .. N-1, in order.
template <class F, int... K>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}

// The k-step's fragment set by index (compile time).
template <int S, class T>
__device__ __forceinline__ T& pick4(T& f0, T& f1, T& f2, T& f3) {
  if constexpr (S == 0) return f0;
  else if constexpr (S == 1) return f1;
  else if constexpr (S == 2) return f2;
  else return f3;
}

// One k-step of 16 on the wave tile.  The first k-step of a leaf takes the
// constant +0 as accumulator input.
template <bool FIRST, int MI>
__device__ __forceinline__ void mfma_step(AccT<MI>& c, const Frags<MI>& f) {
  const f32x16 z = {};
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    c.c[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b0, FIRST ? z : c.c[i][0], 0, 0, 0);
    c.c[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b1, FIRST ? z : c.c[i][1], 0, 0, 0);
  }
}

// Scheduling hint for one step: the 2 MI MFMAs of this step, with the MI + 2
// fragment reads of a later step and D DMA instructions spread between them.
template <int MI, int D>
__device__ __forceinline__ void sched_step() {
#pragma unroll
  for (int t = 0; t < 2 * MI; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (t < MI + 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (((t + 1) * D) / (2 * MI) > (t * D) / (2 * MI)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}

// Runs every tile of this workgroup: leaf-tree main loop, then epi(acc, mt, nt, region).
//
// The k-tiles of all tiles form one stream q = 0 .. total-1 through a ring of
// STAGES buffers.  Fragments are read two k-steps ahead of their MFMAs.  In
// the middle of stage q (after the MFMAs of steps 0 and 1) each wave waits
// for its DMA of stage q+1 and for its own reads of stage q, then passes the
// barrier: stage q+1 has landed everywhere and stage q's buffer is no longer
// read.  Stage q+STAGES-1 is loaded into the buffer of stage q-1 (free since
// the barrier of stage q-1), its DMA spread between the MFMA steps of stage
// q.  Past the end of the stream every stage
// still issues one k-tile (the last one again, into a buffer already
// consumed), so each stage carries the same number of loads, the wait count
// is a constant and the stage has no branch.  At leaf ends the accumulator
// folds into the pending tree; at tile ends the epilogue borrows the buffer of
// the tile's last stage, which no DMA targets until the next stage.
template <int LG, int MI, class Ld, class Epi>
__device__ __forceinline__ void leaf_tree_persistent(Ld& ld, int ktiles, const TileSched& ts, Epi& epi,
                                                     char* smem) {
  using G = Geo<MI>;
  constexpr int STAGES = G::STAGES;
  constexpr uint32_t RING = uint32_t(STAGES * G::STAGE);
  const int n_my = ts.count();
  if (n_my == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  FragAddr<MI> fa;
  fa.fr = lane & 31;
  fa.fk = lane >> 5;
  fa.a0 = uint32_t((wm * 32 * MI + fa.fr) * 128);
  fa.w0 = uint32_t(G::A_BYTES + (wn * 64 + fa.fr) * 128);
  fa.w1 = fa.w0 + 32 * 128;
  constexpr int L = 1 << LG;
  const int kpl = ktiles >> LG;
  const int total = n_my * ktiles;

  // DMA cursor: tile l_tile, leaf position l_pos, k-tile kt.  Position p of
  // a tile visits leaf p ^ m with m = m0 (the schedule's stagger) on even
  // tiles and m0 ^ (L - 1) on odd ones, so that a new round of tiles starts
  // on the k-slice the previous round used last (still in L2).  XOR with a
  // constant maps every aligned block of 2^k positions onto an aligned block
  // of 2^k leaves, so the pending-stack fold, which combines positions, still
  // combines exactly the sibling subtrees of the balanced adjacent-pair tree;
  // it meets some pairs in swapped operand order, which FP32 addition does
  // not see (a + b == b + a bit for bit), so the tree value is the same.
  const int m0 = __builtin_amdgcn_readfirstlane(ts.lmask & (L - 1));
  int l_tile = 0, l_pos = 0, l_j = 0, kt = m0 * kpl, issued = 0;
  {
    int mt, nt;
    ts.coords(0, mt, nt);
    ld.setup(mt, nt);
  }
  auto advance = [&]() {
    if (++issued >= total) return;   // past the end: keep re-issuing the last k-tile
    ++kt;
    if (++l_j == kpl) {
      l_j = 0;
      if (++l_pos == L) {
        l_pos = 0;
        ++l_tile;
        int mt, nt;
        ts.coords(l_tile, mt, nt);
        ld.setup(mt, nt);
      }
      kt = (l_pos ^ m0 ^ ((l_tile & 1) ? (L - 1) : 0)) * kpl;
    }
  };
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) {
    ld.issue_all(smem + p * G::STAGE, kt);
    advance();
  }

  // Ring offsets of stage q and of the buffer being refilled (stage q-1).
  uint32_t off_q = 0, off_pf = RING - uint32_t(G::STAGE);
  // Fragment registers of the four k-steps of a stage, read two steps ahead.
  Frags<MI> F0, F1, F2, F3;
  wait_vmcnt_lgkm0<G::VM_PER_STAGE * (STAGES - 2)>();
  bar();
  fa.read(F0, smem, 0);
  fa.read(F1, smem, 1);

  // One stage is 8 MI MFMAs (4 k-steps of 2 MI), issued one per section in a
  // fixed order; hard scheduling fences between sections pin the other
  // instructions of the stage beside them, so the matrix core gets a new
  // instruction every section instead of waiting behind clumps of LDS reads
  // and DMA issues:
  //   first half  (k-steps 0, 1): the reads of this stage's k-steps 2 and 3,
  //               spread over its first sections, and half of the stage's DMA;
  //   mid-stage:  wait for the DMA of stage q+1 and for this wave's reads of
  //               stage q, then the barrier: stage q+1 has landed everywhere
  //               and stage q's buffer is no longer read;
  //   second half (k-steps 2, 3): the reads of the next stage's k-steps 0 and
  //               1 and the rest of the DMA.
  // The reads of a half stop four MFMAs before its end, so that they have
  // returned when the mid-stage wait or the next stage's first MFMA needs them.
  constexpr int VM = G::VM_PER_STAGE;
  constexpr int NM = 8 * MI, HALF = NM / 2, NR = MI + 2;
  constexpr int RSPAN = HALF - 4 > HALF / 2 ? HALF - 4 : HALF / 2;
  constexpr int DH1 = VM / 2, DH2 = VM - VM / 2;
  // vmcnt once stage q+1 has landed, at the mid-stage wait of stage q: the
  // later stages q+2 .. q+STAGES-2 and this stage's first DH1 instructions.
  constexpr int MID_WAIT = VM * (STAGES - 3) + DH1;
  auto stage = [&](AccT<MI>& cur, auto first) {
    const char* st = smem + off_q;
    char* pb = smem + off_pf;
    const uint32_t off_n = off_q + G::STAGE == RING ? 0u : off_q + uint32_t(G::STAGE);
    const char* sn = smem + off_n;
    for_each_index(std::make_integer_sequence<int, NM>{}, [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ks = k / (2 * MI), t = k % (2 * MI), i = t >> 1, j = t & 1;
      constexpr bool second = k >= HALF;
      constexpr int hk = second ? k - HALF : k;
      {
        const Frags<MI>& F = pick4<ks>(F0, F1, F2, F3);
        const f32x16 z = {};
        cur.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[i], j ? F.b1 : F.b0,
                                                              (decltype(first)::value && ks == 0) ? z : cur.c[i][j],
                                                              0, 0, 0);
      }
      // LDS reads of this section: read r of the half goes to section r RSPAN / (2 NR).
      for_each_index(std::make_integer_sequence<int, 2 * NR>{}, [&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr ((r * RSPAN) / (2 * NR) == hk) {
          constexpr int step = second ? r / NR : 2 + r / NR;   // this stage's 2, 3 / the next one's 0, 1
          Frags<MI>& D = pick4<step>(F0, F1, F2, F3);
          fa.template read_one<r % NR>(D, second ? sn : st, step);
        }
      });
      // DMA of this section: instruction d of a half goes to section (2 d + 1) HALF / (2 D).
      for_each_index(std::make_integer_sequence<int, (DH1 > DH2 ? DH1 : DH2)>{}, [&](auto dc) {
        constexpr int d = decltype(dc)::value;
        if constexpr (!second && d < DH1 && ((2 * d + 1) * HALF) / (2 * DH1) == hk)
          ld.template seg<d>(pb, kt);
        if constexpr (second && d < DH2 && ((2 * d + 1) * HALF) / (2 * DH2) == hk)
          ld.template seg<DH1 + d>(pb, kt);
      });
      if constexpr (k == HALF - 1) {
        wait_vmcnt_lgkm0<MID_WAIT>();   // stage q+1 landed; this wave's reads of stage q returned
        bar();                          // every wave is done with stage q's buffer
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    advance();
    off_pf = off_q;
    off_q = off_n;
  };

  // With Epi::kSplitTop the top level of the tree is not held in registers:
  // each half of the positions is folded on its own, the first half's root
  // goes to the epilogue's spill area (epi.spill) and the epilogue adds it to
  // the second half's root, the same last addition of the same tree.
  constexpr bool SPLIT = Epi::kSplitTop && LG > 0;
  constexpr int PLG = SPLIT ? LG - 1 : LG;   // tree levels held in registers
  for (int ti = 0; ti < n_my; ++ti) {
    AccT<MI> pend[PLG > 0 ? PLG : 1];
    AccT<MI> cur;
#pragma unroll 1
    for (int pos = 0; pos < L; ++pos) {   // sequence position; leaf pos ^ m
      stage(cur, std::true_type{});
      for (int j = 1; j < kpl; ++j) stage(cur, std::false_type{});
      if constexpr (SPLIT) {
        tree_fold<0, PLG>(pend, cur, pos & ((1 << PLG) - 1));
        if (pos == (L >> 1) - 1) epi.spill(cur);
      } else {
        tree_fold<0, LG>(pend, cur, pos);
      }
    }
    int mt, nt;
    ts.coords(ti, mt, nt);
    epi(cur, mt, nt, smem + off_pf);   // the tile's last stage: read by all waves before the barrier
  }
  wait_vmcnt<0>();   // no LDS DMA may still be landing when the workgroup ends
}

// Epilogue: store the tile (FP32, or bf16 by RNE), with non-temporal stores.
template <int EPI, int MI>
struct StoreEpi {
  static constexpr bool kSplitTop = false;
  void* C; int64_t ldc; int64_t M, N;
  __device__ __forceinline__ void spill(const AccT<MI>&) const {}
  __device__ __forceinline__ void operator()(const AccT<MI>& acc, int mt, int nt, char*) const;
};

// Epilogue: per (row, 128-column vocabulary tile) max and sum of exp2.  The
// tile is transposed through LDS in passes of 64 rows; in a pass, thread t
// owns row t/4, columns 32 (t%4)..+31.  (The sampled token's logit is picked
// by its own kernel: a global load here would have to wait for the whole DMA
// ring, which returns in order.)
template <int MI, bool SPLIT = false>
struct LogprobEpi {
  static_assert(64 * BN * 4 <= Geo<MI>::STAGE, "the transpose pass must fit one ring buffer");
  static constexpr bool kSplitTop = SPLIT;
  float2* part; int64_t M, V; int n_vt;
  float* spill_base;   // SPLIT: this launch's spill area, kSpillBytesPerGroup bytes per workgroup
  __device__ __forceinline__ void operator()(AccT<MI>& acc, int mt, int nt, char* region) const;
  // The left half's root waits in the workgroup's area in the accumulator
  // layout: 16-byte chunk q of block (i, j) of thread t at byte
  // (((i 2 + j) 4 + q) 256 + t) 16.
  __device__ __forceinline__ float* area() const {
    return spill_base + size_t(blockIdx.x) * (kSpillBytesPerGroup / 4);
  }
  // One VGPR of lane offset for all 24 stores, the chunk offset in soffset
  // (always inside the area).
  __device__ __forceinline__ void spill(const AccT<MI>& c) const {
    if constexpr (SPLIT) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(area(), uint32_t(kSpillBytesPerGroup));
      const int voff = opaque_tid() * 16;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // Each element through a scalar first: __builtin_bit_cast applied to a
            // vector-element expression directly reads element 0 with this compiler.
            i32x4 d;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float f = c.c[i][j][4 * q + u];
              d[u] = __builtin_bit_cast(int, f);
            }
            __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, ((i * 2 + j) * 4 + q) * NTHREADS * 16, 0);
          }
    }
  }
  // Block (i, j) of the right half's root becomes left + right, the tree's
  // last addition.  The loads are asm blocks of two, each ending in its own
  // wait (device scope: read from L2), so that the compiler neither hoists
  // them nor keeps more than 8 extra registers live.  Their addresses are
  // per-lane 64-bit VGPR pointers: the blocks read no SGPR, so no scalar base
  // reloaded by a vector instruction (a spilled SGPR brought back with
  // v_readlane) can reach them without its wait states.
  __device__ __forceinline__ void join(int i, int j, f32x16& c) const {
    const float* b = area() + (size_t((i * 2 + j) * 4) * NTHREADS + size_t(opaque_tid())) * 4;
#pragma unroll
    for (int q = 0; q < 4; q += 2) {
      const float* p0 = b + size_t(q) * NTHREADS * 4;
      const float* p1 = p0 + NTHREADS * 4;
      float4 l0, l1;
      asm volatile(
          "global_load_dwordx4 %0, %2, off sc1\n global_load_dwordx4 %1, %3, off sc1\n"
          "s_waitcnt vmcnt(0)"
          : "=&v"(l0), "=&v"(l1)
          : "v"(p0), "v"(p1)
          : "memory");
      c[4 * q + 0] = l0.x + c[4 * q + 0];
      c[4 * q + 1] = l0.y + c[4 * q + 1];
      c[4 * q + 2] = l0.z + c[4 * q + 2];
      c[4 * q + 3] = l0.w + c[4 * q + 3];
      c[4 * q + 4] = l1.x + c[4 * q + 4];
      c[4 * q + 5] = l1.y + c[4 * q + 5];
      c[4 * q + 6] = l1.z + c[4 * q + 6];
      c[4 * q + 7] = l1.w + c[4 * q + 7];
    }
  }

};

// ---------------------------------------------------------------------------
// tree_gemm: C = leaf-tree(A W^T), FP32 or bf16 out [IsoExec, Parallelism-invariant
// kernels]; the same bits for every M [BitRL, 4.1].
// ---------------------------------------------------------------------------
template <int EPI, int MI>
__device__ __forceinline__ void StoreEpi<EPI, MI>::operator()(const AccT<MI>& acc, int mt, int nt,
                                                              char*) const {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(mt) * Geo<MI>::BM, n0 = int64_t(nt) * BN;
  // N and ldc multiples of 4, C aligned to four values: the lanes of a quad
  // hold columns c .. c + 3 of the same four rows (registers 4u .. 4u+3), and
  // two lane-swap levels (lanes 1 apart, then 2 apart) transpose that 4 x 4
  // block, so that lane q writes row q's four columns in one store (16 bytes
  // of FP32, 8 of bf16).
  if (((N | ldc) & 3) == 0 && (reinterpret_cast<uintptr_t>(C) & (EPI == kEpiF32 ? 15 : 7)) == 0) {
    const int q = lane & 3;
    auto swp = [](float x, auto ctrl) {
      return __builtin_bit_cast(
          float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value, 0xf, 0xf, false));
    };
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t qc = (n0 + acc_col(wn, j, lane)) & ~int64_t(3);   // the quad's first column
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a0 = acc.c[i][j][4 * u], a1 = acc.c[i][j][4 * u + 1];
          const float a2 = acc.c[i][j][4 * u + 2], a3 = acc.c[i][j][4 * u + 3];
          // Lanes 1 apart: the even lane keeps rows 0 and 2 (its columns c, c + 1),
          // the odd lane rows 1 and 3.
          const bool o1 = (q & 1) != 0;
          const float g0 = swp(o1 ? a0 : a1, std::integral_constant<int, 0xB1>{});
          const float g1 = swp(o1 ? a2 : a3, std::integral_constant<int, 0xB1>{});
          // pair (row r, columns 2p, 2p + 1) held: lo/hi of two rows
          const float p0l = o1 ? g0 : a0, p0h = o1 ? a1 : g0;   // row o1 (0 or 1)
          const float p1l = o1 ? g1 : a2, p1h = o1 ? a3 : g1;   // row 2 + o1
          // Lanes 2 apart: lanes 0, 1 keep their first row's pair and take the
          // partner's; lanes 2, 3 keep the second row's pair.
          const bool o2 = (q & 2) != 0;
          const float s0 = swp(o2 ? p0l : p1l, std::integral_constant<int, 0x4E>{});
          const float s1 = swp(o2 ? p0h : p1h, std::integral_constant<int, 0x4E>{});
          f32x4v out;
          out[0] = o2 ? s0 : p0l;
          out[1] = o2 ? s1 : p0h;
          out[2] = o2 ? p1l : s0;
          out[3] = o2 ? p1h : s1;
          const int64_t row = m0 + acc_row<MI>(wm, i, 4 * u + q, lane & ~3);
          if (qc < N && row < M) {
            if constexpr (EPI == kEpiF32) {
              __builtin_nontemporal_store(out, reinterpret_cast<f32x4v*>(&static_cast<float*>(C)[row * ldc + qc]));
            } else {
              u32x2 pk;
              pk[0] = uint32_t(f32_to_bf16_rne(out[0])) | (uint32_t(f32_to_bf16_rne(out[1])) << 16);
              pk[1] = uint32_t(f32_to_bf16_rne(out[2])) | (uint32_t(f32_to_bf16_rne(out[3])) << 16);
              __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(&static_cast<uint16_t*>(C)[row * ldc + qc]));
            }
          }
        }
      }
    return;
  }
  // Column pairs in one store (4 bytes of bf16, 8 of FP32): the lanes of an
  // even / odd pair hold columns c, c + 1 of the same rows, so a lane swap
  // gives the even lane row r's pair and the odd lane row r + 1's (half the
  // store instructions).  Needs N and ldc even and C aligned to the pair
  // (the same for every lane).
  if (((N | ldc) & 1) == 0 && (reinterpret_cast<uintptr_t>(C) & (EPI == kEpiF32 ? 7 : 3)) == 0) {
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t pc = (n0 + acc_col(wn, j, lane)) & ~int64_t(1);   // the pair's first column
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float a = acc.c[i][j][v], b = acc.c[i][j][v + 1];
          const float got = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, odd ? a : b), 0xB1, 0xf, 0xf, false));
          const float lo = odd ? got : a, hi = odd ? b : got;
          const int64_t row = m0 + acc_row<MI>(wm, i, v + (odd ? 1 : 0), lane);
          if (pc < N && row < M) {
            if constexpr (EPI == kEpiF32) {
              f32x2 pr;
              pr[0] = lo;
              pr[1] = hi;
              __builtin_nontemporal_store(pr, reinterpret_cast<f32x2*>(&static_cast<float*>(C)[row * ldc + pc]));
            } else {
              __builtin_nontemporal_store(uint32_t(f32_to_bf16_rne(lo)) | (uint32_t(f32_to_bf16_rne(hi)) << 16),
                                          reinterpret_cast<uint32_t*>(&static_cast<uint16_t*>(C)[row * ldc + pc]));
            }
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + acc_col(wn, j, lane);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + acc_row<MI>(wm, i, v, lane);
        if (row >= M) continue;
        // Non-temporal: the output streams past the L2, where the operand
        // tiles the workgroups of an XCD share stay resident.
        if (EPI == kEpiF32)
          __builtin_nontemporal_store(acc.c[i][j][v], &static_cast<float*>(C)[row * ldc + col]);
        else
          __builtin_nontemporal_store(f32_to_bf16_rne(acc.c[i][j][v]), &static_cast<uint16_t*>(C)[row * ldc + col]);
      }
    }
}

template <int LG, int MI, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tree_gemm_kernel(DenseOperands op, void* __restrict__ C, int64_t ldc, int ktiles, int n_mt,
                      int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(n_mt, n_nt);
  StoreEpi<EPI, MI> epi{C, ldc, op.M, op.N};
  Loader<MI> ld{op};
  leaf_tree_persistent<LG, MI>(ld, ktiles, ts, epi, smem);
}

// ---------------------------------------------------------------------------
// Block-FP8 W8A8 leaf-tree GEMM on the FP8 matrix cores [BitRL, 4.1]:
// v_mfma_scale_f32_32x32x64_f8f6f4 takes E4M3 operands and multiplies each
// product by the E8M0 scales of its A row and W column (exact for these
// power-of-two scales), accumulating in FP32.  The operand bytes ride the
// bf16 DMA path unchanged: a row of K E4M3 bytes is K/2 16-bit words, and a
// k-tile of 64 words is 128 values, one scale block.  Each stage adds one DMA
// per wave: the k-tile's 128 A-row scales and the tile's W scale, from a table
// SC [K/128][scw] built per call (the A rows' scales, then the n-blocks'),
// into a 256-byte area of the wave's own; every wave issues the same number of
// DMAs, so the constant wait count of the ring holds.  Two k-steps of 64 per
// k-tile; the leaves and their tree are those of the bf16 kernel.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) int i32x8;

struct GeoF8 {
  static constexpr int MI = 2;
  static constexpr int BM = 128;
  static constexpr int A_BYTES = BM * 128;
  static constexpr int W_BYTES = BN * 128;
  static constexpr int SC_OFF = A_BYTES + W_BYTES;     // the four waves' scale areas
  static constexpr int STAGE = SC_OFF + 4 * 256;
  static constexpr int STAGES = kLdsBytes / STAGE;     // 4
  static constexpr int A_SEG = 4;                      // 1 KiB A segments per wave, as the bf16 tile of 128 rows
  static constexpr int VM_PER_STAGE = A_SEG + 4 + 1;   // A, W, scales
  static_assert(STAGES >= 3, "ring too shallow");
  static_assert(VM_PER_STAGE * (STAGES - 2) < 64, "vmcnt range");
  static_assert(64 * BN * 4 <= STAGE, "epilogue pass must fit one ring buffer");
};

struct F8Operands {
  DenseOperands op;            // the E4M3 bytes as 16-bit words: lda = ldw = K / 2
  const uint8_t* sc;           // scale table [K/128][scw]
  int64_t scw, mrows, ksc;     // its row length, the A part of a row (M rounded up to 128), K/128
};

struct LoaderF8 : Loader<2> {
  F8Operands f;
  __amdgpu_buffer_rsrc_t rsc;
  uint32_t osc;                // this lane's byte offset in a row of the table (or past its end)

  __device__ __forceinline__ void setup(int mt, int nt) {
    Loader<2>::setup(mt, nt);
    const int lane = threadIdx.x & 63;
    rsc = make_rsrc(f.sc, uint32_t(f.ksc * f.scw));
    osc = lane < 32 ? uint32_t(int64_t(mt) * GeoF8::BM + 4 * lane)
                    : (lane == 32 ? uint32_t(f.mrows + (nt & ~3)) : OOB);
  }
  template <int J>
  __device__ __forceinline__ void seg(char* stage, int kt) const {
    if constexpr (J < GeoF8::A_SEG + 4) {
      Loader<2>::template seg<J>(stage, kt);
    } else {
      const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (LDS_AS void*)(stage + GeoF8::SC_OFF + wave * 256), 4, osc,
                                               uint32_t(kt) * uint32_t(f.scw), 0, 0);
    }
  }
  template <int J0, int D>
  __device__ __forceinline__ void segs(char* stage, int kt) const {
    if constexpr (D > 0) {
      seg<J0>(stage, kt);
      segs<J0 + 1, D - 1>(stage, kt);
    }
  }
  __device__ __forceinline__ void issue_all(char* stage, int kt) const {
    segs<0, GeoF8::VM_PER_STAGE>(stage, kt);
  }
  // Byte of the tile's W scale in the dword the scale DMA brought.
  __device__ __forceinline__ int wsel(int, int nt) const { return nt & 3; }
};

// The FP8 loader for expert work items (expert, first row, rows): A rows of
// the item, W the expert's slice; the table's A part holds 128 entries per
// item (item i's row scales from byte 128 i, dword-aligned), then E x nb W
// scales (expert e, n-block nt at e nb + nt).
struct F8GroupOperands {
  const uint16_t* X; const uint16_t* W; const int4* items;   // E4M3 bytes as 16-bit words
  const uint8_t* sc;
  int64_t N, K, scw, apart, ksc, nb;
};

struct LoaderF8G : Loader<2> {
  F8GroupOperands g;
  __amdgpu_buffer_rsrc_t rsc;
  uint32_t osc;
  __device__ __forceinline__ int expert_of(int item) const {
    return ((const CONST_AS int32_t*)g.items)[4 * item];
  }
  __device__ __forceinline__ void setup(int item, int nt) {
    const CONST_AS int32_t* it = (const CONST_AS int32_t*)g.items + 4 * item;
    const int e = it[0], row0 = it[1], rows = it[2];
    this->op = DenseOperands{g.X + int64_t(row0) * (g.K / 2), g.K / 2, rows, g.W + int64_t(e) * g.N * (g.K / 2),
                             g.K / 2, g.N};
    Loader<2>::setup(0, nt);
    const int lane = threadIdx.x & 63;
    rsc = make_rsrc(g.sc, uint32_t(g.ksc * g.scw));
    const int64_t w = int64_t(e) * g.nb + nt;
    osc = lane < 32 ? uint32_t(int64_t(item) * 128 + 4 * lane)
                    : (lane == 32 ? uint32_t(g.apart + (w & ~int64_t(3))) : OOB);
  }
  template <int J>
  __device__ __forceinline__ void seg(char* stage, int kt) const {
    if constexpr (J < GeoF8::A_SEG + 4) {
      Loader<2>::template seg<J>(stage, kt);
    } else {
      const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (LDS_AS void*)(stage + GeoF8::SC_OFF + wave * 256), 4, osc,
                                               uint32_t(kt) * uint32_t(g.scw), 0, 0);
    }
  }
  template <int J0, int D>
  __device__ __forceinline__ void segs(char* stage, int kt) const {
    if constexpr (D > 0) {
      seg<J0>(stage, kt);
      segs<J0 + 1, D - 1>(stage, kt);
    }
  }
  __device__ __forceinline__ void issue_all(char* stage, int kt) const {
    segs<0, GeoF8::VM_PER_STAGE>(stage, kt);
  }
  __device__ __forceinline__ int wsel(int item, int nt) const { return int((expert_of(item) * g.nb + nt) & 3); }
};

// Fragments of one k-step of 64: 32 bytes of a row per lane (two 16-byte
// chunks, logical chunks 4 s + 2 (lane / 32) and the next).
struct FragF8 { i32x8 a[2], b0, b1; };

struct FragAddrF8 {
  uint32_t a0, w0, w1;
  int fr, fk;
  __device__ __forceinline__ i32x8 pair(const char* st, uint32_t row_off, int s) const {
    const int sw = (fr >> 1) & 7;
    const int c0 = 4 * s + 2 * fk;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(st + row_off + uint32_t((c0 ^ sw) << 4));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(st + row_off + uint32_t(((c0 + 1) ^ sw) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ void read(FragF8& f, const char* st, int s) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = pair(st, a0 + i * 32 * 128, s);
    f.b0 = pair(st, w0, s);
    f.b1 = pair(st, w1, s);
  }
};

template <bool FIRST>
__device__ __forceinline__ void mfma_step_f8(AccT<2>& c, const FragF8& f, const int (&sa)[2], int sw) {
  const f32x16 z = {};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    c.c[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b0, FIRST ? z : c.c[i][0], 0, 0, 0, sa[i],
                                                                0, sw);
    c.c[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b1, FIRST ? z : c.c[i][1], 0, 0, 0, sa[i],
                                                                0, sw);
  }
}

// Scheduling hint for one FP8 step: 4 MFMAs with the 8 fragment reads of the
// next step and D DMA instructions between them.
template <int D>
__device__ __forceinline__ void sched_step_f8() {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (((t + 1) * D) / 4 > (t * D) / 4) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}

// The persistent leaf-tree loop of leaf_tree_persistent with FP8 stages: the
// same ring discipline (constant DMA count per stage, the mid-stage wait and
// barrier, the last k-tile re-issued past the end), two k-steps per stage,
// fragments read one step ahead, the stage's scales read at its start.
template <int LG, class Ld, class Epi>
__device__ __forceinline__ void leaf_tree_persistent_f8(Ld& ld, int ktiles, const TileSched& ts, Epi& epi,
                                                        char* smem) {
  using G = GeoF8;
  constexpr int STAGES = G::STAGES;
  constexpr uint32_t RING = uint32_t(STAGES * G::STAGE);
  const int n_my = ts.count();
  if (n_my == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  FragAddrF8 fa;
  fa.fr = lane & 31;
  fa.fk = lane >> 5;
  fa.a0 = uint32_t((wm * 64 + fa.fr) * 128);
  fa.w0 = uint32_t(G::A_BYTES + (wn * 64 + fa.fr) * 128);
  fa.w1 = fa.w0 + 32 * 128;
  const uint32_t sc_off = uint32_t(G::SC_OFF + wave * 256);
  constexpr int L = 1 << LG;
  const int kpl = ktiles >> LG;
  const int total = n_my * ktiles;
  const int m0 = __builtin_amdgcn_readfirstlane(ts.lmask & (L - 1));
  int l_tile = 0, l_pos = 0, l_j = 0, kt = m0 * kpl, issued = 0;
  {
    int mt, nt;
    ts.coords(0, mt, nt);
    ld.setup(mt, nt);
  }
  auto advance = [&]() {
    if (++issued >= total) return;
    ++kt;
    if (++l_j == kpl) {
      l_j = 0;
      if (++l_pos == L) {
        l_pos = 0;
        ++l_tile;
        int mt, nt;
        ts.coords(l_tile, mt, nt);
        ld.setup(mt, nt);
      }
      kt = (l_pos ^ m0 ^ ((l_tile & 1) ? (L - 1) : 0)) * kpl;
    }
  };
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) {
    ld.issue_all(smem + p * G::STAGE, kt);
    advance();
  }
  uint32_t off_q = 0, off_pf = RING - uint32_t(G::STAGE);
  FragF8 F0, F1;
  wait_vmcnt_lgkm0<G::VM_PER_STAGE * (STAGES - 2)>();
  bar();
  fa.read(F0, smem, 0);

  constexpr int VM = G::VM_PER_STAGE;
  constexpr int D0 = VM / 2, D1 = VM - VM / 2;
  constexpr int MID_WAIT = VM * (STAGES - 3) + D0;
  int wsel = 0;                 // byte of the W scale in its dword: the tile's n-block % 4
  auto stage = [&](AccT<2>& cur, auto first) {
    const char* st = smem + off_q;
    char* pb = smem + off_pf;
    const uint32_t off_n = off_q + G::STAGE == RING ? 0u : off_q + uint32_t(G::STAGE);
    int sa[2];
    sa[0] = *reinterpret_cast<const uint8_t*>(st + sc_off + wm * 64 + fa.fr);
    sa[1] = *reinterpret_cast<const uint8_t*>(st + sc_off + wm * 64 + 32 + fa.fr);
    const int sw = *reinterpret_cast<const uint8_t*>(st + sc_off + 128 + wsel);
    fa.read(F1, st, 1);
    mfma_step_f8<decltype(first)::value>(cur, F0, sa, sw);
    ld.template segs<0, D0>(pb, kt);
    sched_step_f8<D0>();
    wait_vmcnt_lgkm0<MID_WAIT>();   // stage q+1 landed; this wave's reads of stage q returned
    bar();                          // every wave is done with stage q's buffer
    fa.read(F0, smem + off_n, 0);
    mfma_step_f8<false>(cur, F1, sa, sw);
    ld.template segs<D0, D1>(pb, kt);
    sched_step_f8<D1>();
    advance();
    off_pf = off_q;
    off_q = off_n;
  };

  for (int ti = 0; ti < n_my; ++ti) {
    int mt, nt;
    ts.coords(ti, mt, nt);
    wsel = ld.wsel(mt, nt);
    AccT<2> pend[LG > 0 ? LG : 1];
    AccT<2> cur;
#pragma unroll 1
    for (int pos = 0; pos < L; ++pos) {
      stage(cur, std::true_type{});
      for (int j = 1; j < kpl; ++j) stage(cur, std::false_type{});
      tree_fold<0, LG>(pend, cur, pos);
    }
    epi(cur, mt, nt, smem + off_pf);
  }
  wait_vmcnt<0>();
}

template <int LG, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fp8_tree_gemm_kernel(F8Operands f, void* __restrict__ C, int64_t ldc, int ktiles, int n_mt, int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(n_mt, n_nt);
  StoreEpi<EPI, 2> epi{C, ldc, f.op.M, f.op.N};
  LoaderF8 ld;
  ld.op = f.op;
  ld.f = f;
  leaf_tree_persistent_f8<LG>(ld, ktiles, ts, epi, smem);
}

// The scale table of an expert call: row kb = [128 entries per work item
// (its rows' scales, 127 = 1 past them)][expert e's W scales at e nb + nt][127
// up to scw].
__global__ __launch_bounds__(256) void fp8_group_table_kernel(const int4* __restrict__ items,
                                                              const int32_t* __restrict__ n_items,
                                                              const uint8_t* __restrict__ SX,
                                                              const uint8_t* __restrict__ SW, int64_t n_experts,
                                                              int64_t nb, int64_t ksc, int64_t apart, int64_t scw,
                                                              uint8_t* __restrict__ sc) {
  const int64_t ni = *n_items;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < ksc * scw; i += int64_t(gridDim.x) * 256) {
    const int64_t kb = i / scw, c = i % scw;
    uint8_t v = 127;
    if (c < apart) {
      const int64_t item = c / 128, r = c % 128;
      if (item < ni) {
        const int4 it = items[item];
        if (r < it.z) v = SX[(int64_t(it.y) + r) * ksc + kb];
      }
    } else if (c < apart + n_experts * nb) {
      v = SW[(c - apart) * ksc + kb];
    }
    sc[i] = v;
  }
}

// The scale table of one call: row kb = [the A rows' scales (127 = 1 past M)
// up to mrows][the n-blocks' W scales][127 up to scw].
__global__ __launch_bounds__(256) void fp8_scale_table_kernel(const uint8_t* __restrict__ SA,
                                                              const uint8_t* __restrict__ SW, int64_t M, int64_t nb,
                                                              int64_t ksc, int64_t mrows, int64_t scw,
                                                              uint8_t* __restrict__ sc) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < ksc * scw; i += int64_t(gridDim.x) * 256) {
    const int64_t kb = i / scw, c = i % scw;
    uint8_t v = 127;
    if (c < M) v = SA[c * ksc + kb];
    else if (c >= mrows && c < mrows + nb) v = SW[(c - mrows) * ksc + kb];
    sc[i] = v;
  }
}

// ---------------------------------------------------------------------------
// logprob, pass 1 [BitRL, 2]: per (row, 128-column vocabulary tile) the max m_t and
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

// The two 32-lane halves of a wave exchange one float: lo = the value of lane
// l & 31, hi = that of lane (l & 31) + 32, on every lane.  One lane swap
// (the upper half of the first copy with the lower half of the second): no
// lane index and no LDS permute.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, unsigned(sw[0]));
  hi = __builtin_bit_cast(float, unsigned(sw[1]));
}

// Wave-private transpose area: 32 rows x 64 floats, 16-byte chunk index XOR
// (row % 16), so the 16 rows a 128-bit read serves at once hit all 64 banks.
__device__ __forceinline__ int tr_index(int r, int c) {
  return r * 64 + (((c >> 2) ^ (r & 15)) << 2) + (c & 3);
}

// Wave (wm, wn) owns rows 32 MI wm .. +32 MI and columns 64 wn .. +63 of the
// tile.  It transposes its blocks of 32 rows through its own 8 KiB of the
// borrowed buffer (no barrier: a wave's LDS operations execute in order), so
// lane l then holds row l % 32 of the block, columns 32 (l / 32) .. +31: the
// pair tree over those 32, then the two lane halves (one exchange) give
// the wave's 64-column max and sum; the two waves of a row pair meet through
// LDS.  Tree over the 128 columns: ((q0 + q1) + (q2 + q3)), q = 32-column
// quarters, the same as every other placement of this epilogue.
template <int MI, bool SPLIT>
__device__ __forceinline__ void LogprobEpi<MI, SPLIT>::operator()(AccT<MI>& acc, int mt, int nt,
                                                                  char* region) const {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  float* P = reinterpret_cast<float*>(region + wave * 8192);
  const float* Q = reinterpret_cast<const float*>(region + (wave ^ 1) * 8192);
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = int64_t(mt) * Geo<MI>::BM + wm * 32 * MI, n0 = int64_t(nt) * BN;
  const bool full = n0 + BN <= V;
  const int valid = int(V - n0) - 64 * wn - 32 * h;   // columns of this lane's 32 (when !full)
  float x[MI][32];
  float mw[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    if constexpr (SPLIT) {
      join(i, 0, acc.c[i][0]);
      join(i, 1, acc.c[i][1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        P[tr_index((v >> 2) * 8 + h * 4 + (v & 3), j * 32 + r)] = acc.c[i][j][v];
    {
      uint32_t ad[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        ad[k] = uint32_t(reinterpret_cast<uintptr_t>(P + r * 64 + (((8 * h + k) ^ (r & 15)) << 2)));
      float4 t0, t1, t2, t3, t4, t5, t6, t7;
      asm volatile(
          "ds_read_b128 %0, %8\n ds_read_b128 %1, %9\n ds_read_b128 %2, %10\n ds_read_b128 %3, %11\n"
          "ds_read_b128 %4, %12\n ds_read_b128 %5, %13\n ds_read_b128 %6, %14\n ds_read_b128 %7, %15\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
          : "memory");
      const float4 tt[8] = {t0, t1, t2, t3, t4, t5, t6, t7};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[i][4 * k + 0] = tt[k].x; x[i][4 * k + 1] = tt[k].y; x[i][4 * k + 2] = tt[k].z; x[i][4 * k + 3] = tt[k].w;
      }
    }
    float mx = -__builtin_inff();
    if (full) {
#pragma unroll
      for (int c = 0; c < 32; ++c) mx = fmaxf(mx, x[i][c]);
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (c < valid) mx = fmaxf(mx, x[i][c]);
    }
    float lo, hi;
    halves(mx, lo, hi);
    mw[i] = fmaxf(lo, hi);
  }
  // Publish this wave's 64-column maxes in its own area (the block data there
  // has been read: the writes queue behind those reads).
  if (h == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i) P[i * 32 + r] = mw[i];
  }
  lds_sync();
  float sw[MI], mtile[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    mtile[i] = fmaxf(mw[i], Q[i * 32 + r]);   // tile max (exact, any order)
    float e[32];
    if (full) {
#pragma unroll
      for (int c = 0; c < 32; ++c) e[c] = __builtin_amdgcn_exp2f((x[i][c] - mtile[i]) * LOG2E);
    } else {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        e[c] = c < valid ? __builtin_amdgcn_exp2f((x[i][c] - mtile[i]) * LOG2E) : 0.0f;
    }
    const float sq = pair_tree_32(e);
    float lo, hi;
    halves(sq, lo, hi);
    sw[i] = lo + hi;   // (q0 + q1) or (q2 + q3)
  }
  if (h == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i) P[128 + i * 32 + r] = sw[i];
  }
  lds_sync();
  if (wn == 0 && h == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const float st = sw[i] + Q[128 + i * 32 + r];   // (q0 + q1) + (q2 + q3)
      const int64_t row = m0 + i * 32 + r;
      if (row < M) part[row * n_vt + nt] = make_float2(mtile[i], st);
    }
  }
  lds_sync();   // the partner's slots are read before the buffer is refilled
}

__device__ __forceinline__ void pick_item(const uint16_t* __restrict__ H, const uint16_t* __restrict__ W,
                                          const int64_t* __restrict__ ids, float* __restrict__ xleaf,
                                          int64_t M, int64_t K, int64_t V, int group, int leaf, int leaves);

// SPLIT (16 leaves with 192-row tiles): the left half of the tree waits in
// `spill_base` instead of registers.
template <int LG, int MI, int WAUX, bool SPLIT>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void logprob_tile_kernel(DenseOperands op, int ktiles, int n_mt, int n_nt, float2* __restrict__ part,
                         float* __restrict__ spill_base, const int64_t* __restrict__ ids, float* __restrict__ xleaf,
                         int n_pick) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(n_mt, n_nt);
  LogprobEpi<MI, SPLIT> epi{part, op.M, op.N, n_nt, spill_base};
  Loader<MI, WAUX> ld{op};
  leaf_tree_persistent<LG, MI>(ld, ktiles, ts, epi, smem);
  // With one row of tiles the last round of tiles leaves workgroups idle: the
  // highest-numbered ones, which run the fewest tiles, also run the n_pick
  // items of the sampled-logit pass (one per wave; none when n_pick is 0).
  // (Compiled into the single-row instances only: WAUX == 2.)
  if constexpr (WAUX == 2) {
    const int j = (int(gridDim.x) - 1 - int(blockIdx.x)) * (NTHREADS / 64) + int(threadIdx.x >> 6);
    if (j < n_pick)
      pick_item(op.A, op.W, ids, xleaf, op.M, int64_t(ktiles) * BK, op.N, j >> LG, j & ((1 << LG) - 1), 1 << LG);
  } else {
    (void)ids;
    (void)xleaf;
    (void)n_pick;
  }
}

// ---------------------------------------------------------------------------
// logprob [BitRL, 2]: the sampled token's logit x[row, id[row]], computed exactly as the
// tile kernels compute that element.  One wave per (32 rows, leaf): it forms
// the 32 x 32 block H[rows] W[ids]^T of its leaf with the same
// v_mfma_f32_32x32x16_bf16 k-steps (ascending, from +0) and keeps the
// diagonal; the combine pass folds the leaves in the same balanced
// adjacent-pair tree.  An MFMA result element depends only on its own A row,
// B column and C input, so the diagonal holds the very bits the tile kernel
// produced for (row, id[row]).  Rows whose id is out of range read W row 0;
// their logprob becomes NaN in the combine.
// ---------------------------------------------------------------------------
constexpr int PICK_U = 32;   // k-steps loaded at once (a whole leaf of 512)

// One work item of the sampled-logit pass, run by one wave: rows
// 32 group .. 32 group + 31 and one leaf.
__device__ __forceinline__ void pick_item(const uint16_t* __restrict__ H, const uint16_t* __restrict__ W,
                                          const int64_t* __restrict__ ids, float* __restrict__ xleaf,
                                          int64_t M, int64_t K, int64_t V, int group, int leaf, int leaves) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 31, half = lane >> 5;
  const int64_t row0 = int64_t(group) * 32;
  const int64_t row = row0 + i < M ? row0 + i : M - 1;
  int64_t id = ids[row];
  if (id < 0 || id >= V) id = 0;
  const int64_t len = K / leaves;
  const bf16x8* pa = reinterpret_cast<const bf16x8*>(H + row * K + leaf * len + 8 * half);
  const bf16x8* pb = reinterpret_cast<const bf16x8*>(W + id * K + leaf * len + 8 * half);
  const int steps = int(len / kMfmaK);
  f32x16 c = {};
  for (int s0 = 0; s0 < steps; s0 += PICK_U) {
    bf16x8 a[PICK_U], b[PICK_U];
#pragma unroll
    for (int u = 0; u < PICK_U; ++u)
      if (s0 + u < steps) {
        a[u] = pa[(s0 + u) * 2];
        b[u] = pb[(s0 + u) * 2];
      }
#pragma unroll
    for (int u = 0; u < PICK_U; ++u)
      if (s0 + u < steps) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], c, 0, 0, 0);
  }
  // Element (i, i) sits in lane i + 32 ((i >> 2) & 1), register 4 (i >> 3) + (i & 3).
  if (((i >> 2) & 1) == half && row0 + i < M) {
    const int vsel = 4 * (i >> 3) + (i & 3);
    float d = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (v == vsel) d = c[v];
    xleaf[(row0 + i) * leaves + leaf] = d;
  }
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void logprob_pick_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ W,
                         const int64_t* __restrict__ ids, float* __restrict__ xleaf, int64_t M,
                         int64_t K, int64_t V) {
  pick_item(H, W, ids, xleaf, M, K, V, int(blockIdx.x), int(blockIdx.y), int(gridDim.y));
}

// ---------------------------------------------------------------------------
// logprob, pass 2 [BitRL, 2]: one workgroup of 256 per row combines the vocabulary tiles.
//   g = max_t m_t (exact); S = sum_t s_t exp2((m_t - g) log2 e) by the
//   balanced adjacent-pair tree over the tiles zero-padded to P = 256 2^q
//   (padding beyond the next power of two only adds +0 subtrees): thread t
//   owns tiles [t 2^q, (t+1) 2^q) and folds them with a pending stack; the
//   xor butterfly over lanes and then the pair tree over the 4 waves form the
//   upper levels.  x = the picked logit's leaves folded by the leaf tree.
// ---------------------------------------------------------------------------
constexpr int MAX_Q = 8;   // 2^8 tiles per thread: up to 65536 tiles

// Same pending-stack fold as tree_fold, on one float, for a chunk of 2^q
// terms (q <= MAX_Q): term i parks at its lowest 0 bit below q; the last
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
    const float2* __restrict__ part, const float* __restrict__ xleaf,
    const int64_t* __restrict__ ids, float* __restrict__ logprob, float* __restrict__ lse,
    int n_vt, int q, int64_t V, int leaves) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float2* pr = part + row * n_vt;
  const int c = 1 << q;
  const int t0 = tid * c;

  // Thread 0's operands of the final step, loaded while the tiles are reduced.
  float x[16];
  int64_t id = 0;
  if (tid == 0) {
    id = ids[row];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = j < leaves ? xleaf[row * leaves + j] : 0.0f;
  }
  // Up to 8 tiles per thread (vocabularies up to 262144) stay in registers
  // between the max and the sum; more are read again.
  constexpr int CACHE = 8;
  float2 v[CACHE];
#pragma unroll
  for (int i = 0; i < CACHE; ++i) v[i] = make_float2(-__builtin_inff(), 0.0f);
  if (c <= CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i)
      if (i < c && t0 + i < n_vt) v[i] = pr[t0 + i];
  }

  float g = -__builtin_inff();
  if (c <= CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i)
      if (i < c && t0 + i < n_vt) g = fmaxf(g, v[i].x);
  } else {
    for (int i = 0; i < c; ++i)
      if (t0 + i < n_vt) g = fmaxf(g, pr[t0 + i].x);
  }
#pragma unroll
  for (int m = 1; m < 64; m *= 2) g = fmaxf(g, __shfl_xor(g, m));
  if (lane == 0) red[wave] = g;
  __syncthreads();
  g = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));   // exact, any order
  __syncthreads();

  float pend[MAX_Q];
  float cur = 0.0f;
  if (c <= CACHE) {
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
      if (i < c) {
        float term = 0.0f;
        if (t0 + i < n_vt) term = v[i].y * __builtin_amdgcn_exp2f((v[i].x - g) * LOG2E);
        cur = term;
        scalar_fold<0>(pend, cur, i, q);
      }
    }
  } else {
    for (int i = 0; i < c; ++i) {
      float term = 0.0f;
      if (t0 + i < n_vt) {
        const float2 p = pr[t0 + i];
        term = p.y * __builtin_amdgcn_exp2f((p.x - g) * LOG2E);
      }
      cur = term;
      scalar_fold<0>(pend, cur, i, q);
    }
  }
  float S = cur;
#pragma unroll
  for (int m = 1; m < 64; m *= 2) {
    const float o = __shfl_xor(S, m);
    S = (lane & m) ? o + S : S + o;   // lower lane's subtree on the left
  }
  if (lane == 0) red[wave] = S;
  __syncthreads();
  if (tid == 0) {
    S = (red[0] + red[1]) + (red[2] + red[3]);
    const float l = g + __builtin_amdgcn_logf(S) * LN2;
#pragma unroll
    for (int w = 1; w < 16; w *= 2)
#pragma unroll
      for (int j = 0; j + w < 16; j += 2 * w)
        if (j + w < leaves) x[j] = x[j] + x[j + w];
    const bool ok = id >= 0 && id < V;
    logprob[row] = ok ? x[0] - l : __builtin_nanf("");
    if (lse) lse[row] = l;
  }
}

// ---------------------------------------------------------------------------
// MoE [BitRL, 4.4-4.5]: route (stable per-expert token lists), plan (work items), per-expert
// leaf-tree GEMM on the persistent pipeline with gathered A rows, and the
// fixed-order FP32 combine.
// ---------------------------------------------------------------------------

// Routing is a stable partition of the (token, slot) pairs p = t * topk + s
// by expert, in three steps: per-chunk expert histograms, a scan that gives
// every (chunk, expert) its first row and plans the work items, and a scatter
// that keeps pair order inside each expert.  The order of an expert's rows
// does not reach any value (a row's result depends on that row alone); it
// only keeps the workspace reproducible.
constexpr int ROUTE_CHUNK = 256;

// Chunk c of 256 pairs: hist[c][e] = pairs of the chunk routed to expert e.
__global__ __launch_bounds__(256) void moe_hist_kernel(const int32_t* __restrict__ topk_ids,
                                                       int64_t n_pairs, int n_experts,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  for (int e = threadIdx.x; e < n_experts; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t p = int64_t(blockIdx.x) * ROUTE_CHUNK + threadIdx.x;
  if (p < n_pairs) {
    const int e = topk_ids[p];
    if (e >= 0 && e < n_experts) atomicAdd(&h[e], 1);   // a count: the order of adds does not matter
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_experts; e += 256) hist[int64_t(blockIdx.x) * n_experts + e] = h[e];
}

// One workgroup of 1024: first[c][e] = first row of chunk c inside expert
// e's list (exclusive scan of hist over chunks), counts, the first row of
// each expert in Y (exclusive scan over experts) and the work items (expert,
// m-tile of bm rows, rows of the expert, first row), numbered in ascending
// expert order.  G = PLAN_THREADS / 64 threads share an expert (fewer when
// there are more than 64 experts), each owning a contiguous run of chunks
// whose counts it keeps in registers (the first PLAN_U; the rest of a longer
// run is read twice).
constexpr int PLAN_THREADS = 1024, PLAN_U = 8;

// Exclusive prefix sum over the workgroup's threads in thread order: a scan
// inside each wave, then over the wave totals.  buf holds >= 16 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int o = __shfl_up(x, d);
    if (lane >= d) x += o;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += buf[w];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(PLAN_THREADS) void moe_plan_kernel(const int32_t* __restrict__ hist,
                                                                int32_t* __restrict__ first, int n_chunks,
                                                                int n_experts, int bm,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ prefix,
                                                                int4* __restrict__ items,
                                                                int32_t* __restrict__ n_items) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int buf[PLAN_THREADS];
  int G = PLAN_THREADS / 64;
  while (G > 1 && G * n_experts > PLAN_THREADS) G >>= 1;
  const int per_pass = PLAN_THREADS / G;   // experts per pass
  // Thread t: expert e0 + t % per_pass (consecutive lanes, consecutive
  // experts: coalesced), chunk run q = t / per_pass.
  const int q = int(threadIdx.x) / per_pass, el = int(threadIdx.x) % per_pass;
  const int per = (n_chunks + G - 1) / G;
  const int c0 = q * per, c1 = min(n_chunks, c0 + per);
  for (int e0 = 0; e0 < n_experts; e0 += per_pass) {
    const int e = e0 + el;
    int v[PLAN_U];
    int sum = 0;
    if (e < n_experts) {
#pragma unroll
      for (int k = 0; k < PLAN_U; ++k) v[k] = c0 + k < c1 ? hist[int64_t(c0 + k) * n_experts + e] : 0;
#pragma unroll
      for (int k = 0; k < PLAN_U; ++k) sum += v[k];
      for (int c = c0 + PLAN_U; c < c1; ++c) sum += hist[int64_t(c) * n_experts + e];
    }
    buf[threadIdx.x] = sum;
    __syncthreads();
    if (e < n_experts) {
      int acc = 0;
      for (int k = 0; k < q; ++k) acc += buf[k * per_pass + el];
#pragma unroll
      for (int k = 0; k < PLAN_U; ++k)
        if (c0 + k < c1) {
          first[int64_t(c0 + k) * n_experts + e] = acc;
          acc += v[k];
        }
      for (int c = c0 + PLAN_U; c < c1; ++c) {
        first[int64_t(c) * n_experts + e] = acc;
        acc += hist[int64_t(c) * n_experts + e];
      }
      if (q == G - 1) {
        cnt[e] = acc;
        counts[e] = acc;
      }
    }
    __syncthreads();
  }
  // Exclusive scans over experts of rows and of work items; thread t owns
  // experts [t k, (t + 1) k).
  const int k = (n_experts + PLAN_THREADS - 1) / PLAN_THREADS;
  const int ea = min(n_experts, int(threadIdx.x) * k), eb = min(n_experts, ea + k);
  int rows = 0, nit = 0;
  for (int e = ea; e < eb; ++e) {
    rows += cnt[e];
    nit += (cnt[e] + bm - 1) / bm;
  }
  int row0 = block_exclusive_scan(rows, buf);
  int it0 = block_exclusive_scan(nit, buf);
  for (int e = ea; e < eb; ++e) {
    const int c = cnt[e];
    prefix[e] = row0;
    for (int mt = 0; mt * bm < c; ++mt) items[it0++] = make_int4(e, mt, c, row0);
    row0 += c;
  }
  if (threadIdx.x == PLAN_THREADS - 1) {
    prefix[n_experts] = row0;
    *n_items = it0;
  }
}

// Chunk c: each pair's row = first row of (c, e) + pairs of the chunk before
// it with the same expert; tok[e][row] = its token, pos[p] = row.
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ topk_ids,
                                                          int64_t n_pairs, int n_experts, int topk,
                                                          const int32_t* __restrict__ first,
                                                          int32_t* __restrict__ tok,
                                                          int32_t* __restrict__ pos) {
  __shared__ int ids[ROUTE_CHUNK];
  const int64_t p = int64_t(blockIdx.x) * ROUTE_CHUNK + threadIdx.x;
  const int e = p < n_pairs ? topk_ids[p] : -1;
  ids[threadIdx.x] = e;
  __syncthreads();
  if (e < 0 || e >= n_experts) return;
  int before = 0;
  for (int i = 0; i < int(threadIdx.x); ++i) before += ids[i] == e;
  const int row = first[int64_t(blockIdx.x) * n_experts + e] + before;
  tok[int64_t(e) * n_pairs + row] = int32_t(p / topk);
  pos[p] = row;
}

// Operands of the MoE GEMM: A rows are gathered tokens of H, W is the expert's slice.
struct MoeOperands {
  const uint16_t* H; const uint16_t* W;
  const int32_t* tok; const int4* items;
  float* Y;
  int64_t T, N, K, n_pairs;
};

// DMA loader for a work item (expert e, m-tile mt) and n-tile nt: the lane's
// A rows come from the expert's token list (the eight consecutive rows of a
// segment read by scalar loads), W rows as in the dense loader.  Rows past the
// expert's count read as zero.
template <int MI>
struct MoeLoader {
  using G = Geo<MI>;
  MoeOperands op;
  __amdgpu_buffer_rsrc_t ra, rw;
  uint32_t oa[G::A_SEG], ow[2];
  uint32_t sw;

  __device__ __forceinline__ void setup(int item, int nt) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const CONST_AS int32_t* it = (const CONST_AS int32_t*)op.items + 4 * item;
    const int e = it[0], mt = it[1], count = it[2];
    const int64_t n0 = int64_t(nt) * BN;
    const int64_t rows_w = op.N - n0 < BN ? op.N - n0 : BN;
    ra = make_rsrc(op.H, uint32_t(op.T * op.K * 2));
    rw = make_rsrc(op.W + (int64_t(e) * op.N + n0) * op.K, uint32_t(rows_w * op.K * 2));
    const int rs = lane >> 3;
    const uint32_t c0 = uint32_t(((lane & 7) ^ (rs >> 1)) << 4), c1 = c0 ^ 64u;
    ow[0] = uint32_t(rs * op.K * 2) + c0;
    ow[1] = uint32_t(rs * op.K * 2) + c1;
    sw = uint32_t(op.K * 16);
    const CONST_AS int32_t* tl =
        (const CONST_AS int32_t*)op.tok + int64_t(e) * op.n_pairs + int64_t(mt) * G::BM;
#pragma unroll
    for (int j = 0; j < G::A_SEG; ++j) {
      const int g = wave * G::A_SEG + j;
      int t8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t8[k] = tl[g * 8 + k];
      int t = t8[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) t = rs == k ? t8[k] : t;
      const int slot = mt * G::BM + g * 8 + rs;
      oa[j] = slot < count ? uint32_t(t) * uint32_t(op.K * 2) + ((j & 1) ? c1 : c0) : OOB;
    }
  }

  template <int J>
  __device__ __forceinline__ void seg(char* stage, int kt) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int so = kt * (BK * 2);
    if constexpr (J < G::A_SEG) {
      const int g = wave * G::A_SEG + J;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LDS_AS void*)(stage + g * 1024), 16,
                                               uint32_t(oa[J]), so, 0, 0);
    } else {
      const int g = wave * 4 + (J - G::A_SEG);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LDS_AS void*)(stage + G::A_BYTES + g * 1024), 16,
                                               ow[J & 1] + uint32_t(g) * sw, so, 0, 0);
    }
  }
  template <int J0, int D>
  __device__ __forceinline__ void segs(char* stage, int kt) const {
    if constexpr (D > 0) {
      seg<J0>(stage, kt);
      segs<J0 + 1, D - 1>(stage, kt);
    }
  }
  __device__ __forceinline__ void issue_all(char* stage, int kt) const {
    segs<0, G::VM_PER_STAGE>(stage, kt);
  }
};

// Epilogue: the item's rows go to Y rows prefix[e] + mt * BM + r (FP32).
template <int MI>
struct MoeStoreEpi {
  static constexpr bool kSplitTop = false;
  MoeOperands op;
  __device__ __forceinline__ void spill(const AccT<MI>&) const {}
  __device__ __forceinline__ void operator()(const AccT<MI>& acc, int item, int nt, char* region) const {
    const CONST_AS int32_t* it = (const CONST_AS int32_t*)op.items + 4 * item;
    const int rows = it[2] - it[1] * Geo<MI>::BM;
    float* C = op.Y + (int64_t(it[3]) + int64_t(it[1]) * Geo<MI>::BM) * op.N;
    const StoreEpi<kEpiF32, MI> st{C, op.N, rows, op.N};
    st(acc, 0, nt, region);
  }
};

template <int LG, int MI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void moe_tile_kernel(MoeOperands op, const int32_t* __restrict__ n_items, int ktiles, int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(*(const CONST_AS int32_t*)n_items, n_nt);
  MoeLoader<MI> ld{op};
  MoeStoreEpi<MI> epi{op};
  leaf_tree_persistent<LG, MI>(ld, ktiles, ts, epi, smem);
}

// out[t, n] = sum over the token's experts in ascending id (ties: slot order)
// of w * y, an FP32 multiply then an FP32 add, from +0.  One workgroup per
// token: the order and the Y rows are found once, then every thread walks
// its columns.
__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* __restrict__ topk_ids,
                                                          const float* __restrict__ topk_w,
                                                          const float* __restrict__ Y,
                                                          const int32_t* __restrict__ prefix,
                                                          const int32_t* __restrict__ pos,
                                                          float* __restrict__ out, int64_t N,
                                                          int topk, int n_experts) {
  __shared__ int64_t rows[kMaxTopk];
  __shared__ float wts[kMaxTopk];
  __shared__ int ex[kMaxTopk];
  __shared__ int bad;
  const int64_t t = blockIdx.x;
  const int s = threadIdx.x;
  // Thread s < topk owns slot s: its expert, weight and Y row are loaded in
  // parallel; its rank in (expert id, slot) order places it.
  int e = 0;
  float w = 0.0f;
  if (s < topk) {
    e = topk_ids[t * topk + s];
    w = topk_w[t * topk + s];
    ex[s] = e;
  }
  if (s == 0) bad = 0;
  __syncthreads();
  if (s < topk) {
    const bool ok = e >= 0 && e < n_experts;
    if (!ok) bad = 1;
    int rank = 0;
    for (int k = 0; k < topk; ++k) {
      const int ek = ex[k];
      rank += ek < e || (ek == e && k < s);
    }
    rows[rank] = ok ? (int64_t(prefix[e]) + pos[t * topk + s]) * N : 0;
    wts[rank] = w;
  }
  __syncthreads();
  const float nan = __builtin_nanf("");
  // Rows of Y (the workspace) and of out 16-byte aligned: four columns per thread.
  if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    const int64_t N4 = N >> 2;
    for (int64_t n = s; n < N4; n += 256) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      for (int k = 0; k < topk; ++k) {
        const float wk = wts[k];
        const float4 y = reinterpret_cast<const float4*>(Y + rows[k])[n];
        acc.x = acc.x + wk * y.x;
        acc.y = acc.y + wk * y.y;
        acc.z = acc.z + wk * y.z;
        acc.w = acc.w + wk * y.w;
      }
      reinterpret_cast<float4*>(out + t * N)[n] = bad ? make_float4(nan, nan, nan, nan) : acc;
    }
  } else {
    for (int64_t n = s; n < N; n += 256) {
      float acc = 0.0f;
      for (int k = 0; k < topk; ++k) {
        const float term = wts[k] * Y[rows[k] + n];
        acc = acc + term;
      }
      out[t * N + n] = bad ? nan : acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Expert GEMM on two layouts [BitRL, 4.4]: the rows of expert e are a block
// of `cap` rows at e * cap (masked) or a segment in expert order whose start
// is a multiple of `align` (contiguous).  Each expert's rows are cut into
// m-tiles (work items); every tile runs the dense leaf-tree pipeline on its
// rows with the expert's W slice, so a row's result depends on its own values
// and the expert only, never on the layout or on the other rows.
// ---------------------------------------------------------------------------
constexpr int GROUP_PLAN_THREADS = 1024;

// Exclusive prefix sum over the workgroup's threads in thread order, and the total.
__device__ __forceinline__ int64_t block_excl_i64(int64_t v, int64_t* red, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int64_t o = __shfl_up(x, d);
    if (lane >= d) x += o;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) {
    before += w < wave ? red[w] : 0;
    all += red[w];
  }
  total = all;
  return before + x - v;
}

// One workgroup: thread e places expert e's rows and writes its work items
// (expert, first row, rows, 0), the experts' items in expert order.  Rows that
// would lie past the buffer's `rows` rows are not computed.
__global__ __launch_bounds__(GROUP_PLAN_THREADS) void group_plan_kernel(const int32_t* __restrict__ counts,
                                                                        int n_experts, bool masked, int64_t cap,
                                                                        int64_t align, int64_t rows, int bm,
                                                                        int4* __restrict__ items,
                                                                        int32_t* __restrict__ n_items) {
  __shared__ int64_t red[GROUP_PLAN_THREADS / 64];
  const int e = threadIdx.x;
  int64_t c = e < n_experts ? counts[e] : 0;
  c = c < 0 ? 0 : c;
  int64_t start;
  if (masked) {
    c = c < cap ? c : cap;
    start = int64_t(e) * cap;
  } else {
    int64_t total;
    start = block_excl_i64((c + align - 1) / align * align, red, total);
    __syncthreads();
  }
  const int64_t fit = rows - start;
  c = c < fit ? c : (fit > 0 ? fit : 0);
  const int64_t tiles = (c + bm - 1) / bm;
  int64_t n_all;
  const int64_t first = block_excl_i64(tiles, red, n_all);
  for (int64_t t = 0; t < tiles; ++t) {
    const int64_t r0 = t * bm;
    items[first + t] = make_int4(e, int(start + r0), int(c - r0 < bm ? c - r0 : bm), 0);
  }
  if (threadIdx.x == 0) *n_items = int32_t(n_all);
}

// Work item i: rows X[row0 .. row0+rows) of expert e against W[e].
struct GroupOperands {
  const uint16_t* X; const uint16_t* W; void* Y; const int4* items;
  int64_t N, K;
};

template <int MI>
struct GroupLoader : Loader<MI> {
  GroupOperands g;
  __device__ __forceinline__ void setup(int item, int nt) {
    const CONST_AS int32_t* it = (const CONST_AS int32_t*)g.items + 4 * item;
    const int e = it[0], row0 = it[1], rows = it[2];
    this->op = DenseOperands{g.X + int64_t(row0) * g.K, g.K, rows, g.W + int64_t(e) * g.N * g.K, g.K, g.N};
    Loader<MI>::setup(0, nt);
  }
};

template <int EPI, int MI>
struct GroupStoreEpi {
  static constexpr bool kSplitTop = false;
  GroupOperands g;
  __device__ __forceinline__ void spill(const AccT<MI>&) const {}
  __device__ __forceinline__ void operator()(const AccT<MI>& acc, int item, int nt, char* region) const {
    const CONST_AS int32_t* it = (const CONST_AS int32_t*)g.items + 4 * item;
    const int row0 = it[1], rows = it[2];
    char* const base = static_cast<char*>(g.Y) + int64_t(row0) * g.N * (EPI == kEpiF32 ? 4 : 2);
    const StoreEpi<EPI, MI> st{base, g.N, rows, g.N};
    st(acc, 0, nt, region);
  }
};

template <int LG, int MI, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void group_tile_kernel(GroupOperands g, const int32_t* __restrict__ n_items, int ktiles, int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(*(const CONST_AS int32_t*)n_items, n_nt);
  GroupLoader<MI> ld;
  ld.g = g;
  GroupStoreEpi<EPI, MI> epi{g};
  leaf_tree_persistent<LG, MI>(ld, ktiles, ts, epi, smem);
}

template <int LG, int EPI>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fp8_group_tile_kernel(F8GroupOperands f, void* __restrict__ Y, const int32_t* __restrict__ n_items, int n_nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  TileSched ts;
  ts.init(*(const CONST_AS int32_t*)n_items, n_nt);
  LoaderF8G ld;
  ld.g = f;
  const GroupOperands go{nullptr, nullptr, Y, f.items, f.N, f.K};
  GroupStoreEpi<EPI, 2> epi{go};
  leaf_tree_persistent_f8<LG>(ld, int(f.ksc), ts, epi, smem);
}

// SiLU(g) * u between the expert GEMMs [BitRL, 4.4, condition 3]: in FP32,
// sigmoid(g) = 1 / (1 + t) for g >= 0 and t / (1 + t) below, t = e^-|g| by
// the hardware exp2 (so that very negative g keep their tiny values), times g,
// times u, then one rounding to bf16.  Thread: four consecutive columns.
__device__ __forceinline__ float silu_f32(float g) {
  const float t = __builtin_amdgcn_exp2f(-__builtin_fabsf(g) * LOG2E);
  const float d = 1.0f + t;
  const float s = g >= 0.0f ? 1.0f / d : t / d;
  return g * s;
}

// Vectorised path: the (row, 4-column chunk) pairs of the call in one flat
// range, four per thread per round (loads of all four first), so that a
// workgroup streams 32 KiB instead of one row's few KiB.
__global__ __launch_bounds__(256) void silu_mul_vec_kernel(const float* __restrict__ GU, int64_t ldgu,
                                                           uint16_t* __restrict__ out, int64_t ldo, uint32_t rows,
                                                           uint32_t q) {
  constexpr int U = 4;
  const uint32_t total = rows * q;                     // < 2^31, checked by the launcher
  const uint32_t step = gridDim.x * 256u * U;
  for (uint32_t base = blockIdx.x * 256u * U + threadIdx.x; base < total; base += step) {
    float4 gv[U], uv[U];
    uint32_t rr[U], cc[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t idx = base + 256u * k;
      rr[k] = idx / q;
      cc[k] = (idx - rr[k] * q) * 4u;
      if (idx < total) {
        const float* g = GU + int64_t(rr[k]) * ldgu + cc[k];
        gv[k] = *reinterpret_cast<const float4*>(g);
        uv[k] = *reinterpret_cast<const float4*>(g + int64_t(q) * 4);
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (base + 256u * k < total) {
        const uint32_t lo = uint32_t(f32_to_bf16_rne(silu_f32(gv[k].x) * uv[k].x)) |
                            (uint32_t(f32_to_bf16_rne(silu_f32(gv[k].y) * uv[k].y)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(silu_f32(gv[k].z) * uv[k].z)) |
                            (uint32_t(f32_to_bf16_rne(silu_f32(gv[k].w) * uv[k].w)) << 16);
        *reinterpret_cast<uint2*>(out + int64_t(rr[k]) * ldo + cc[k]) = make_uint2(lo, hi);
      }
    }
  }
}

// Any widths and alignments: one element at a time, rows across the grid.
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ GU, int64_t ldgu,
                                                       uint16_t* __restrict__ out, int64_t ldo, int64_t rows,
                                                       int64_t I) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float* g = GU + r * ldgu;
    const float* u = g + I;
    uint16_t* o = out + r * ldo;
    for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < I; c += int64_t(gridDim.x) * 256)
      o[c] = f32_to_bf16_rne(silu_f32(g[c]) * u[c]);
  }
}

// ---------------------------------------------------------------------------
// Block FP8 (W8A8) [BitRL, 4.1 and 4.4]: OCP E4M3 values with one power-of-two
// scale 2^e per block (128 x 128 for weights, 1 x 128 for activations), e the
// smallest integer >= -127 with amax <= 448 * 2^e, every element x * 2^-e
// rounded to E4M3 once, to nearest even.  Scales are stored as E8M0 bytes
// (e + 127).  Everything here is exact integer / power-of-two arithmetic.
// ---------------------------------------------------------------------------

// Smallest e >= -127 with a <= 448 * 2^e, for a finite a > 0 (448 = 1.75 * 2^8):
// with a = 1.f * 2^E, e = E - 8 when 1.f <= 1.75, else E - 7.
__device__ __forceinline__ int fp8_block_exponent(float a) {
  if (!(a > 0.0f)) return 0;
  uint32_t b = __builtin_bit_cast(uint32_t, a);
  int E = int(b >> 23) - 127;
  if ((b >> 23) == 0) {                                // subnormal: normalise exactly
    b = __builtin_bit_cast(uint32_t, a * 18446744073709551616.0f);   // * 2^64
    E = int(b >> 23) - 127 - 64;
  }
  const int e = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// E4M3 byte nearest to v (|v| <= 448, finite), halves to the even mantissa.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (b >> 24) & 0x80u, a = b & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {                              // |v| >= 2^-6: keep 3 mantissa bits
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // (exponent, mantissa) rounded
    code = r - (120u << 3);                           // rebias 127 -> 7
  } else {                                             // subnormal step 2^-9: an integer 0..8
    code = uint32_t(__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f));
  }
  return sign | code;
}

// Value of an E4M3 byte times 2^e, as a float (exact).
__device__ __forceinline__ float e4m3_scaled(uint32_t q, int e) {
  const uint32_t ex = (q >> 3) & 0xFu, man = q & 7u;
  const float mag = ex == 0 ? float(man) * 0.001953125f : float(8u + man) * __builtin_ldexpf(1.0f, int(ex) - 10);
  const float v = __builtin_ldexpf(mag, e);
  return (q & 0x80u) ? -v : v;
}

// One wave per 128-column group of one row (activations, blocks of 1 x 128):
// lane l holds columns 2l, 2l+1 of the group.
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                             uint8_t* __restrict__ Q, int64_t ldq,
                                                             uint8_t* __restrict__ S, int64_t R, int64_t C) {
  const int64_t ngroups = (C + 127) / 128;
  const int lane = threadIdx.x & 63;
  for (int64_t w = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); w < R * ngroups; w += int64_t(gridDim.x) * 4) {
    const int64_t r = w / ngroups, g = w % ngroups;
    const int64_t c0 = g * 128 + 2 * lane;
    const uint16_t* x = X + r * ldx;
    const float v0 = c0 < C ? __builtin_bit_cast(float, uint32_t(x[c0]) << 16) : 0.0f;
    const float v1 = c0 + 1 < C ? __builtin_bit_cast(float, uint32_t(x[c0 + 1]) << 16) : 0.0f;
    float m = __builtin_fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
#pragma unroll
    for (int d = 1; d < 64; d *= 2) m = __builtin_fmaxf(m, __shfl_xor(m, d));
    const int e = fp8_block_exponent(m);
    uint8_t* q = Q + r * ldq;
    if (c0 < C) q[c0] = uint8_t(f32_to_e4m3_rne(__builtin_ldexpf(v0, -e)));
    if (c0 + 1 < C) q[c0 + 1] = uint8_t(f32_to_e4m3_rne(__builtin_ldexpf(v1, -e)));
    if (lane == 0) S[r * ngroups + g] = uint8_t(e + 127);
  }
}

// Largest of x over each 32-lane half of the wave, on every lane: within
// 16-lane rows by DPP (lane swaps within pairs, within quads, mirrored halves
// of 8, mirrored rows; every lane has a source), then rows 0 / 1 and 2 / 3
// swapped.  The largest value does not depend on the order of the pairs.
__device__ __forceinline__ float half_wave_max(float x) {
  auto step = [](float v, auto ctrl) {
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf, 0xf, false);
    return __builtin_fmaxf(v, __builtin_bit_cast(float, o));
  };
  x = step(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  x = step(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  x = step(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  x = step(x, std::integral_constant<int, 0x140>{});   // row_mirror
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, unsigned(sw[0])), __builtin_bit_cast(float, unsigned(sw[1])));
}

// The same for C % 4 == 0 with 8-byte aligned rows: one wave per two groups
// (256 columns) of a row, lane l holding columns 4l .. 4l+3 (one 8-byte load,
// one 4-byte store); each half-wave reduces its group's amax by DPP and a
// row swap (an LDS butterfly took 3-7 % longer per call).
__global__ __launch_bounds__(256) void fp8_quant_rows4_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                              uint8_t* __restrict__ Q, int64_t ldq,
                                                              uint8_t* __restrict__ S, int64_t R, int64_t C) {
  const int64_t ngroups = (C + 127) / 128, npairs = (ngroups + 1) / 2;
  const int lane = threadIdx.x & 63;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y)
  for (int64_t gp = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); gp < npairs; gp += int64_t(gridDim.x) * 4) {
    const int64_t c0 = gp * 256 + 4 * lane;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 < C) {
      const uint2 d = *reinterpret_cast<const uint2*>(X + r * ldx + c0);
      v[0] = __builtin_bit_cast(float, d.x << 16);
      v[1] = __builtin_bit_cast(float, d.x & 0xFFFF0000u);
      v[2] = __builtin_bit_cast(float, d.y << 16);
      v[3] = __builtin_bit_cast(float, d.y & 0xFFFF0000u);
    }
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                              __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
    m = half_wave_max(m);
    const int e = fp8_block_exponent(m);
    if (c0 < C) {
      uint32_t q = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) q |= f32_to_e4m3_rne(__builtin_ldexpf(v[i], -e)) << (8 * i);
      *reinterpret_cast<uint32_t*>(Q + r * ldq + c0) = q;
    }
    const int64_t g = 2 * gp + (lane >> 5);
    if ((lane & 31) == 0 && g < ngroups) S[r * ngroups + g] = uint8_t(e + 127);
  }
}

// The same for C % 4 == 0 with 8-byte aligned rows: lane l of wave w takes
// columns 4 (l % 32) .. +3 of rows 8 i + 2 w + l / 32 (i = 0 .. 15), all 16
// loads in flight at once and the 64 values kept in registers between the
// block's amax and its rounding.
__global__ __launch_bounds__(256) void fp8_quant_blocks4_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                uint8_t* __restrict__ Q, int64_t ldq,
                                                                uint8_t* __restrict__ S, int64_t R, int64_t C) {
  __shared__ float red[4];
  const int64_t ngroups = (C + 127) / 128;
  const int64_t br = blockIdx.y, g = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t c0 = g * 128 + 4 * (lane & 31);
  const bool col_ok = c0 < C;
  uint2 d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = br * 128 + 8 * i + 2 * wave + (lane >> 5);
    d[i] = r < R && col_ok ? *reinterpret_cast<const uint2*>(X + r * ldx + c0) : make_uint2(0u, 0u);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, d[i].x << 16)));
    m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, d[i].x & 0xFFFF0000u)));
    m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, d[i].y << 16)));
    m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, d[i].y & 0xFFFF0000u)));
  }
#pragma unroll
  for (int k = 1; k < 64; k *= 2) m = __builtin_fmaxf(m, __shfl_xor(m, k));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const int e = fp8_block_exponent(m);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = br * 128 + 8 * i + 2 * wave + (lane >> 5);
    if (r < R && col_ok) {
      const uint32_t q = f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, d[i].x << 16), -e)) |
                         (f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, d[i].x & 0xFFFF0000u), -e)) << 8) |
                         (f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, d[i].y << 16), -e)) << 16) |
                         (f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, d[i].y & 0xFFFF0000u), -e)) << 24);
      *reinterpret_cast<uint32_t*>(Q + r * ldq + c0) = q;
    }
  }
  if (t == 0) S[br * ngroups + g] = uint8_t(e + 127);
}

// One workgroup per 128 x 128 block (weights): thread t takes columns
// 2 (t % 64), +1 of rows t / 64, t / 64 + 4, ...
__global__ __launch_bounds__(256) void fp8_quant_blocks_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                               uint8_t* __restrict__ Q, int64_t ldq,
                                                               uint8_t* __restrict__ S, int64_t R, int64_t C) {
  __shared__ float red[4];
  const int64_t ngroups = (C + 127) / 128;
  const int64_t br = blockIdx.y, g = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63;
  const int64_t c0 = g * 128 + 2 * lane;
  float m = 0.0f;
  for (int i = t >> 6; i < 128; i += 4) {
    const int64_t r = br * 128 + i;
    if (r >= R) break;
    const uint16_t* x = X + r * ldx;
    if (c0 < C) m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, uint32_t(x[c0]) << 16)));
    if (c0 + 1 < C) m = __builtin_fmaxf(m, __builtin_fabsf(__builtin_bit_cast(float, uint32_t(x[c0 + 1]) << 16)));
  }
#pragma unroll
  for (int d = 1; d < 64; d *= 2) m = __builtin_fmaxf(m, __shfl_xor(m, d));
  if (lane == 0) red[t >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const int e = fp8_block_exponent(m);
  for (int i = t >> 6; i < 128; i += 4) {
    const int64_t r = br * 128 + i;
    if (r >= R) break;
    const uint16_t* x = X + r * ldx;
    uint8_t* q = Q + r * ldq;
    if (c0 < C) q[c0] = uint8_t(f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, uint32_t(x[c0]) << 16), -e)));
    if (c0 + 1 < C)
      q[c0 + 1] = uint8_t(f32_to_e4m3_rne(__builtin_ldexpf(__builtin_bit_cast(float, uint32_t(x[c0 + 1]) << 16), -e)));
  }
  if (t == 0) S[br * ngroups + g] = uint8_t(e + 127);
}

// The activation between the expert GEMMs, then its FP8 input to the second
// [BitRL, 4.4, condition 3]: p = bf16(SiLU(g) u) (FP32, one rounding, as
// silu_mul_kernel), then p quantised in 1 x 128 blocks (as
// fp8_quant_rows4_kernel).  One workgroup per row; lane l of a wave holds
// columns 4l .. 4l+3 of a pair of 128-column groups (I % 4 == 0).
__global__ __launch_bounds__(256) void silu_mul_fp8_kernel(const float* __restrict__ GU, int64_t ldgu,
                                                           uint8_t* __restrict__ Q, int64_t ldq,
                                                           uint8_t* __restrict__ S, int64_t R, int64_t I) {
  const int64_t ngroups = (I + 127) / 128, npairs = (ngroups + 1) / 2;
  const int lane = threadIdx.x & 63;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y)
  for (int64_t gp = threadIdx.x >> 6; gp < npairs; gp += 4) {
    const int64_t c0 = gp * 256 + 4 * lane;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 < I) {
      const float4 g = *reinterpret_cast<const float4*>(GU + r * ldgu + c0);
      const float4 u = *reinterpret_cast<const float4*>(GU + r * ldgu + I + c0);
      v[0] = __builtin_bit_cast(float, uint32_t(f32_to_bf16_rne(silu_f32(g.x) * u.x)) << 16);
      v[1] = __builtin_bit_cast(float, uint32_t(f32_to_bf16_rne(silu_f32(g.y) * u.y)) << 16);
      v[2] = __builtin_bit_cast(float, uint32_t(f32_to_bf16_rne(silu_f32(g.z) * u.z)) << 16);
      v[3] = __builtin_bit_cast(float, uint32_t(f32_to_bf16_rne(silu_f32(g.w) * u.w)) << 16);
    }
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                              __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
#pragma unroll
    for (int d = 1; d < 32; d *= 2) m = __builtin_fmaxf(m, __shfl_xor(m, d));
    const int e = fp8_block_exponent(m);
    if (c0 < I) {
      uint32_t q = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) q |= f32_to_e4m3_rne(__builtin_ldexpf(v[i], -e)) << (8 * i);
      *reinterpret_cast<uint32_t*>(Q + r * ldq + c0) = q;
    }
    const int64_t g = 2 * gp + (lane >> 5);
    if ((lane & 31) == 0 && g < ngroups) S[r * ngroups + g] = uint8_t(e + 127);
  }
}

// Dequantise to bf16 (exact): out[r, c] = value(Q[r, c]) * 2^e of its block
// (block_rows rows x 128 columns).  Thread: 8 consecutive columns.
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ S,
                                                          int64_t R, int64_t C, int block_rows,
                                                          uint16_t* __restrict__ out) {
  const int64_t ngroups = (C + 127) / 128;
  const int64_t n8 = (C + 7) / 8;
  for (int64_t w = int64_t(blockIdx.x) * 256 + threadIdx.x; w < R * n8; w += int64_t(gridDim.x) * 256) {
    const int64_t r = w / n8, c0 = (w % n8) * 8;
    const int e = int(S[(r / block_rows) * ngroups + c0 / 128]) - 127;
    const uint8_t* q = Q + r * C;
    uint16_t* o = out + r * C;
    for (int j = 0; j < 8 && c0 + j < C; ++j) o[c0 + j] = f32_to_bf16_rne(e4m3_scaled(q[c0 + j], e));
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Persistent grid: one workgroup per CU (multiple of 8 for the XCD deal), or
// one per tile when there are fewer tiles.  Only the schedule depends on it.
int persistent_grid(int64_t n_tiles) {
  const int cus = device_cus();
  const int64_t full = int64_t(cus / 8) * 8 > 0 ? int64_t(cus / 8) * 8 : 8;
  const int64_t want = ((n_tiles + 7) / 8) * 8;
  return int(want < full ? want : full);
}

// Tiles the busiest workgroup runs: TileSched's deal of n_mt x n_nt tiles over
// a persistent grid (n-slices per XCD with at least 4 groups of n-tiles, else
// an even split of the logical order), slots workgroups per XCD.
int64_t busiest_tiles(int64_t n_mt, int64_t n_nt) {
  const int64_t slots = persistent_grid(n_mt * n_nt) / 8;
  const int64_t per_xcd = n_nt >= 4 * GROUP_N ? cdiv(n_nt, 8) * n_mt : cdiv(n_mt * n_nt, 8);
  return cdiv(per_xcd, slots);
}

int choose_tree_gemm_block_m(int64_t M, int64_t N, int leaves_log2) {
  // Time of one tile relative to a 128-row tile (x100), from event timings of
  // 4096-deep contractions at 8 leaves: rows 64 / 128 / 192 -> 70 / 100 / 138.
  const int heights[3] = {64, 128, 192}, cost[3] = {70, 100, 138};
  const int n_h = block_m_for_log2(leaves_log2) == 192 ? 3 : 2;
  const int64_t n_nt = cdiv(N, BN);
  int best = 64;
  int64_t best_t = -1;
  for (int i = 0; i < n_h; ++i) {
    const int64_t t = busiest_tiles(cdiv(M, heights[i]), n_nt) * cost[i];
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = heights[i];
    }
  }
  return best;
}

template <int LG, int MI>
hipError_t launch_tree_gemm_mi(const TreeGemmLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, 64 * MI)), n_nt = int(cdiv(p.N, BN));
  const DenseOperands op{static_cast<const uint16_t*>(p.A), p.lda, p.M,
                         static_cast<const uint16_t*>(p.W), p.ldw, p.N};
  const int ktiles = int(p.K / BK);
  const dim3 grid(persistent_grid(int64_t(n_mt) * n_nt)), block(NTHREADS);
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((tree_gemm_kernel<LG, MI, kEpiF32>), grid, block, 0, s, op, p.C, p.ldc,
                       ktiles, n_mt, n_nt);
  else
    hipLaunchKernelGGL((tree_gemm_kernel<LG, MI, kEpiBF16>), grid, block, 0, s, op, p.C, p.ldc,
                       ktiles, n_mt, n_nt);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_tree_gemm_lg(const TreeGemmLaunch& p, hipStream_t s) {
  const int bm = tree_gemm_block_m(p.M, p.N, LG);
  if (bm == 64) return launch_tree_gemm_mi<LG, 1>(p, s);
  if constexpr (block_m_for_log2(LG) == 192) {
    if (bm == 192) return launch_tree_gemm_mi<LG, 3>(p, s);
  }
  return launch_tree_gemm_mi<LG, 2>(p, s);
}

template <int LG, int MI>
hipError_t launch_logprob_mi(const LogprobLaunch& p, hipStream_t s) {
  const int n_mt = int(cdiv(p.M, 64 * MI)), n_vt = int(cdiv(p.V, BN));
  const DenseOperands op{static_cast<const uint16_t*>(p.H), p.K, p.M,
                         static_cast<const uint16_t*>(p.W), p.K, p.V};
  float2* part = static_cast<float2*>(p.partials);
  // One row of tiles (decode-sized batches): each W tile is read once, so its
  // loads bypass the caches' retention (non-temporal).  The split tree's
  // scratch holds kSpillGrid workgroups.
  constexpr bool SPLIT = LG == 4 && MI == 3;
  int grid = persistent_grid(int64_t(n_mt) * n_vt);
  if (SPLIT && grid > kSpillGrid) grid = kSpillGrid;
  if (SPLIT && !p.spill) return hipErrorInvalidValue;
  // The sampled-logit pass: inside the tile kernel's last round when there is
  // one row of tiles and a wave of the grid for each item, else its own kernel.
  const int64_t items = cdiv(p.M, 32) << LG;
  const int n_pick = n_mt == 1 && items <= int64_t(grid) * (NTHREADS / 64) ? int(items) : 0;
  if (n_pick == 0) {
    hipLaunchKernelGGL(logprob_pick_kernel, dim3(unsigned(cdiv(p.M, 32)), 1u << LG), dim3(64), 0, s,
                       static_cast<const uint16_t*>(p.H), static_cast<const uint16_t*>(p.W), p.ids,
                       p.xleaf, p.M, p.K, p.V);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_mt == 1)
    hipLaunchKernelGGL((logprob_tile_kernel<LG, MI, 2, SPLIT>), dim3(grid), dim3(NTHREADS), 0, s, op,
                       int(p.K / BK), n_mt, n_vt, part, p.spill, p.ids, p.xleaf, n_pick);
  else
    hipLaunchKernelGGL((logprob_tile_kernel<LG, MI, 0, SPLIT>), dim3(grid), dim3(NTHREADS), 0, s, op,
                       int(p.K / BK), n_mt, n_vt, part, p.spill, p.ids, p.xleaf, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int q = 0;
  while ((256 << q) < n_vt) ++q;
  hipLaunchKernelGGL(logprob_combine_kernel, dim3(unsigned(p.M)), dim3(256), 0, s, part, p.xleaf,
                     p.ids, p.logprob, p.lse, n_vt, q, p.V, 1 << LG);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_logprob_lg(const LogprobLaunch& p, hipStream_t s) {
  if (logprob_block_m_for(p.M, LG) == 192) return launch_logprob_mi<LG, 3>(p, s);
  return launch_logprob_mi<LG, 2>(p, s);
}

template <int LG, int MI>
hipError_t launch_moe_mi(const MoeLaunch& p, hipStream_t s) {
  const int64_t n_pairs = p.T * p.topk;
  const int n_chunks = int(cdiv(n_pairs, ROUTE_CHUNK));
  hipLaunchKernelGGL(moe_hist_kernel, dim3(n_chunks), dim3(256), size_t(p.n_experts) * 4, s, p.topk_ids,
                     n_pairs, p.n_experts, p.hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, p.hist, p.first, n_chunks, p.n_experts,
                     64 * MI, p.counts, p.prefix, reinterpret_cast<int4*>(p.items), p.n_items);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(n_chunks), dim3(256), 0, s, p.topk_ids, n_pairs,
                     p.n_experts, p.topk, p.first, p.tok, p.pos);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_nt = int(cdiv(p.N, BN));
  const MoeOperands op{static_cast<const uint16_t*>(p.H), static_cast<const uint16_t*>(p.W), p.tok,
                       reinterpret_cast<const int4*>(p.items), p.Y, p.T, p.N, p.K, n_pairs};
  // The grid is sized from the static bound on work items; workgroups without
  // a tile exit at once.
  const int64_t max_tiles = moe_max_items(p.T, p.topk, p.n_experts) * n_nt;
  hipLaunchKernelGGL((moe_tile_kernel<LG, MI>), dim3(persistent_grid(max_tiles)), dim3(NTHREADS), 0, s,
                     op, p.n_items, int(p.K / BK), n_nt);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(unsigned(p.T)), dim3(256), 0, s, p.topk_ids, p.topk_w, p.Y,
                     p.prefix, p.pos, p.out, p.N, p.topk, p.n_experts);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_moe_lg(const MoeLaunch& p, hipStream_t s) {
  if constexpr (block_m_for_log2(LG) == 192) return launch_moe_mi<LG, 3>(p, s);
  else return launch_moe_mi<LG, 2>(p, s);
}

template <int LG, int MI>
hipError_t launch_group_mi(const GroupLaunch& p, hipStream_t s) {
  constexpr int BMm = 64 * MI;
  hipLaunchKernelGGL(group_plan_kernel, dim3(1), dim3(GROUP_PLAN_THREADS), 0, s, p.counts, p.n_experts, p.masked,
                     p.cap, p.align, p.rows, BMm, reinterpret_cast<int4*>(p.items), p.n_items);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_nt = int(cdiv(p.N, BN));
  const GroupOperands g{static_cast<const uint16_t*>(p.X), static_cast<const uint16_t*>(p.W), p.Y,
                        reinterpret_cast<const int4*>(p.items), p.N, p.K};
  // The grid is sized from the static bound on work items; workgroups without
  // a tile exit at once.
  const dim3 grid(persistent_grid(group_max_items(p.rows, p.n_experts) * n_nt));
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((group_tile_kernel<LG, MI, kEpiF32>), grid, dim3(NTHREADS), 0, s, g, p.n_items,
                       int(p.K / BK), n_nt);
  else
    hipLaunchKernelGGL((group_tile_kernel<LG, MI, kEpiBF16>), grid, dim3(NTHREADS), 0, s, g, p.n_items,
                       int(p.K / BK), n_nt);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_group_lg(const GroupLaunch& p, hipStream_t s) {
  if constexpr (block_m_for_log2(LG) == 192) return launch_group_mi<LG, 3>(p, s);
  else return launch_group_mi<LG, 2>(p, s);
}

template <int LG>
hipError_t launch_fp8_group_lg(const Fp8GroupLaunch& p, hipStream_t s) {
  hipLaunchKernelGGL(group_plan_kernel, dim3(1), dim3(GROUP_PLAN_THREADS), 0, s, p.counts, p.n_experts, p.masked,
                     p.cap, p.align, p.rows, GeoF8::BM, reinterpret_cast<int4*>(p.items), p.n_items);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t ksc = p.K / 128, nb = cdiv(p.N, 128);
  const int64_t max_items = group_max_items(p.rows, p.n_experts);
  const int64_t apart = max_items * 128, scw = fp8_group_table_width(p.rows, p.n_experts, p.N);
  const int64_t cells = ksc * scw;
  hipLaunchKernelGGL(fp8_group_table_kernel, dim3(unsigned(cdiv(cells, 256) < 4096 ? cdiv(cells, 256) : 4096)),
                     dim3(256), 0, s, reinterpret_cast<const int4*>(p.items), p.n_items, p.SX, p.SW,
                     int64_t(p.n_experts), nb, ksc, apart, scw, p.table);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_nt = int(nb);
  const F8GroupOperands f{reinterpret_cast<const uint16_t*>(p.QX), reinterpret_cast<const uint16_t*>(p.QW),
                          reinterpret_cast<const int4*>(p.items), p.table, p.N, p.K, scw, apart, ksc, nb};
  const dim3 grid(persistent_grid(max_items * n_nt));
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((fp8_group_tile_kernel<LG, kEpiF32>), grid, dim3(NTHREADS), 0, s, f, p.Y, p.n_items, n_nt);
  else
    hipLaunchKernelGGL((fp8_group_tile_kernel<LG, kEpiBF16>), grid, dim3(NTHREADS), 0, s, f, p.Y, p.n_items, n_nt);
  return hipGetLastError();
}

template <int LG>
hipError_t launch_fp8_lg(const Fp8GemmLaunch& p, hipStream_t s) {
  const int64_t ksc = p.K / 128, nb = cdiv(p.N, 128);
  hipLaunchKernelGGL(fp8_scale_table_kernel, dim3(unsigned(cdiv(ksc * p.scw, 256) < 4096 ? cdiv(ksc * p.scw, 256) : 4096)),
                     dim3(256), 0, s, p.SA, p.SW, p.M, nb, ksc, p.mrows, p.scw, p.table);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_mt = int(cdiv(p.M, GeoF8::BM)), n_nt = int(cdiv(p.N, BN));
  const F8Operands f{DenseOperands{reinterpret_cast<const uint16_t*>(p.QA), p.K / 2, p.M,
                                   reinterpret_cast<const uint16_t*>(p.QW), p.K / 2, p.N},
                     p.table, p.scw, p.mrows, ksc};
  const dim3 grid(persistent_grid(int64_t(n_mt) * n_nt));
  if (p.epi == kEpiF32)
    hipLaunchKernelGGL((fp8_tree_gemm_kernel<LG, kEpiF32>), grid, dim3(NTHREADS), 0, s, f, p.C, p.ldc, int(ksc), n_mt,
                       n_nt);
  else
    hipLaunchKernelGGL((fp8_tree_gemm_kernel<LG, kEpiBF16>), grid, dim3(NTHREADS), 0, s, f, p.C, p.ldc, int(ksc), n_mt,
                       n_nt);
  return hipGetLastError();
}

}  // namespace

int tree_gemm_block_m(int64_t M, int64_t N, int leaves_log2) {
  return choose_tree_gemm_block_m(M, N, leaves_log2);
}

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

// The no-allocation entry point's intermediate data (tile partials, picked
// logit leaves and, at 16 leaves on 192-row tiles, the parked half trees) lives
// in the file-scope array `scratch`.  Host code never passes the array's name
// to a kernel (in host code it is only a stand-in for the symbol): the first
// call on a device looks up that device's copy with hipGetSymbolAddress, with
// the device current, and every later call on it reuses that address.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    status[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch));
    if (status[dev] == hipSuccess && addr[dev] == nullptr) status[dev] = hipErrorInvalidSymbol;
  });
  if (status[dev] != hipSuccess) return status[dev];
  *ptr = addr[dev];
  return hipSuccess;
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

// ---------------------------------------------------------------------------
// MoE router, after the logits (a tree_gemm with FP32 output, the same at
// every batch size): per token the topk largest logits, largest first, equal
// logits in ascending expert id, +0 equal to -0, NaN after every number; then
// the softmax over them: m = the largest, e_s = exp2((l_s - m) log2 e), the
// sum by the balanced adjacent-pair tree over the slots zero-padded to a power
// of two, gate_s = e_s / sum (FP32 division).  One wave per token.
// ---------------------------------------------------------------------------
namespace {

// Order key of a logit: larger key = ahead.  -0 becomes +0 (v + 0 under
// round to nearest even); negative floats are mirrored so that the integer
// order is the float order; NaN sorts below every number.
__device__ __forceinline__ int route_key(float v) {
  if (__builtin_isnan(v)) return INT_MIN;
  const int b = __builtin_bit_cast(int, v + 0.0f);
  return b >= 0 ? b : (b ^ 0x7FFFFFFF);
}

// PER = candidates per lane: ceil(E / 64) rounded up to a power of two (<= 16).
// Max of a 64-bit value over the wave, on every lane: rotations inside the
// 16-lane rows (DPP), then rows 0 / 1 and 2 / 3 swapped (v_permlane16_swap)
// and the wave halves swapped (v_permlane32_swap); the two 32-bit halves move
// together.  No LDS.
__device__ __forceinline__ int64_t wave_max_i64(int64_t x) {
  auto halves_of = [](int64_t v, int& lo, int& hi) {
    lo = int(uint32_t(uint64_t(v)));
    hi = int(uint32_t(uint64_t(v) >> 32));
  };
  auto join = [](int lo, int hi) { return int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)); };
  auto rot = [&](auto ctrl) {
    int lo, hi;
    halves_of(x, lo, hi);
    constexpr int C = decltype(ctrl)::value;
    const int64_t o = join(__builtin_amdgcn_mov_dpp(lo, C, 0xf, 0xf, true), __builtin_amdgcn_mov_dpp(hi, C, 0xf, 0xf, true));
    x = o > x ? o : x;
  };
  rot(std::integral_constant<int, 0x121>{});   // row_ror:1
  rot(std::integral_constant<int, 0x122>{});   // row_ror:2
  rot(std::integral_constant<int, 0x124>{});   // row_ror:4
  rot(std::integral_constant<int, 0x128>{});   // row_ror:8
  auto swap = [&](auto wide) {
    int lo, hi;
    halves_of(x, lo, hi);
    unsigned lo2 = unsigned(lo), hi2 = unsigned(hi);
    // Second operands the compiler cannot equate with the first: with two equal
    // operands it folds the swap away, although it exchanges rows.
    asm volatile("" : "+v"(lo2), "+v"(hi2));
    unsigned l0, l1, h0, h1;
    if constexpr (decltype(wide)::value) {
      const auto sl = __builtin_amdgcn_permlane32_swap(unsigned(lo), lo2, false, false);
      const auto sh = __builtin_amdgcn_permlane32_swap(unsigned(hi), hi2, false, false);
      l0 = sl[0]; l1 = sl[1]; h0 = sh[0]; h1 = sh[1];   // elements through scalars (see halves())
    } else {
      const auto sl = __builtin_amdgcn_permlane16_swap(unsigned(lo), lo2, false, false);
      const auto sh = __builtin_amdgcn_permlane16_swap(unsigned(hi), hi2, false, false);
      l0 = sl[0]; l1 = sl[1]; h0 = sh[0]; h1 = sh[1];
    }
    const int64_t a = join(int(l0), int(h0)), b = join(int(l1), int(h1));
    x = a > b ? a : b;
  };
  swap(std::false_type{});
  swap(std::true_type{});
  return x;
}

template <int PER>
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                        int topk, int32_t* __restrict__ ids,
                                                        float* __restrict__ gates) {
  constexpr int ROUTE_PER_LANE = PER;
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // the whole wave
  const float* row = logits + t * E;
  // Lane l holds experts l + 64 c; a candidate is (key << 32) | ~expert, so
  // the largest candidate is the largest logit, then the lowest expert id.
  float v[ROUTE_PER_LANE];
  int64_t cand[ROUTE_PER_LANE];
#pragma unroll
  for (int c = 0; c < ROUTE_PER_LANE; ++c) {
    const int e = c * 64 + lane;
    v[c] = e < E ? row[e] : 0.0f;
    cand[c] = e < E ? int64_t((uint64_t(uint32_t(route_key(v[c]))) << 32) | uint32_t(~e)) : INT64_MIN;
  }
  float my_v = 0.0f, vmax = 0.0f;
  int my_e = 0;
  for (int r = 0; r < topk; ++r) {
    int64_t best = INT64_MIN;
#pragma unroll
    for (int c = 0; c < ROUTE_PER_LANE; ++c) best = cand[c] > best ? cand[c] : best;
    best = wave_max_i64(best);
    // Every lane: the winner (uniform, so its lane is read with readlane).
    const int e = __builtin_amdgcn_readfirstlane(int(~uint32_t(uint64_t(best))));
    float mine = 0.0f;
#pragma unroll
    for (int c = 0; c < ROUTE_PER_LANE; ++c)
      if (c == (e >> 6)) mine = v[c];
    const float ve = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine), e & 63));
    if (lane == (e & 63)) {
#pragma unroll
      for (int c = 0; c < ROUTE_PER_LANE; ++c)
        if (c == (e >> 6)) cand[c] = INT64_MIN;
    }
    if (r == 0) vmax = ve;
    if (lane == r) {
      my_e = e;
      my_v = ve;
    }
  }
  float x = lane < topk ? __builtin_amdgcn_exp2f((my_v - vmax) * LOG2E) : 0.0f;
  float S = x;
  for (int d = 1; d < topk; d *= 2) {   // pair tree over lanes 0 .. 2^ceil(log2 topk) - 1
    const float o = __shfl_xor(S, d);
    S = (lane & d) ? o + S : S + o;
  }
  if (lane < topk) {
    ids[t * topk + lane] = my_e;
    gates[t * topk + lane] = x / S;
  }
}

// Router logits [BitRL, 4.1], the leaf-tree contraction with FP32 output for the router's
// shape (few experts): one workgroup per 32 tokens x 64 experts, so that
// T / 32 workgroups share the work instead of T / 64 tiles of the persistent
// kernel.  Wave w accumulates leaves w, w + 4, ...: the same
// v_mfma_f32_32x32x16_bf16 k-steps, ascending from +0, with the same operand
// layout (lane l: row l % 32, columns 8 (l / 32) .. +7 of the k-step) as the
// tile kernels, so each leaf is the same FP32 block.  Each wave streams its
// leaf through two 12 KiB stages of its own in LDS (64 columns of the 32
// token rows and 64 expert rows; direct-to-LDS DMA of 8 rows x 128 bytes per
// instruction, chunk c of row r at chunk c ^ ((r >> 1) & 7) as in the tile
// kernels; rows past T or the expert count read as zero).  The leaves' blocks
// stay in registers until every wave is done, then meet in LDS and fold by the
// balanced adjacent-pair tree, left + right, as in the tile kernels.
constexpr int kRouterStage = (32 + 64) * 128;   // bytes of one stage of one wave

template <int LG>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ H,
                                                            const uint16_t* __restrict__ Wr,
                                                            float* __restrict__ logits, int64_t T, int64_t K,
                                                            int E) {
  constexpr int L = 1 << LG;
  constexpr int NL = L < 4 ? 1 : L / 4;   // leaves per wave (waves past L have none)
  constexpr int STAGE_BYTES = 4 * 2 * kRouterStage;
  constexpr int PART_BYTES = L * 32 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) char smem[STAGE_BYTES > PART_BYTES ? STAGE_BYTES : PART_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = int64_t(blockIdx.x) * 32;
  const int e0 = int(blockIdx.y) * 64;
  const int64_t trows = T - t0 < 32 ? T - t0 : 32;
  const int erows = E - e0 < 64 ? E - e0 : 64;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(H + t0 * K, uint32_t(trows * K * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Wr + int64_t(e0) * K, uint32_t(int64_t(erows) * K * 2));
  // DMA lane offsets: instruction g loads rows 8 g .. 8 g + 7; lane i fills LDS
  // chunk i % 8 of row 8 g + i / 8 with logical chunk (i % 8) ^ ((row >> 1) & 7).
  // (row >> 1) & 7 = 4 (g & 1) + i / 16, so two offsets per operand cover every g.
  const int rs = lane >> 3;
  const uint32_t c0 = uint32_t(((lane & 7) ^ (rs >> 1)) << 4), c1 = c0 ^ 64u;
  const uint32_t lo0 = uint32_t(int64_t(rs) * K * 2) + c0, lo1 = uint32_t(int64_t(rs) * K * 2) + c1;
  const uint32_t gstride = uint32_t(8 * K * 2);   // 8 rows
  // Fragment reads: row fr = lane % 32 of the operand, logical chunk 2 s + fk.
  const int fr = lane & 31, fk = lane >> 5;
  char* const mine = smem + wave * 2 * kRouterStage;
  const int64_t kl = K >> LG;            // columns per leaf, a multiple of 64
  const int nst = int(kl / 64);          // stages per leaf
  const f32x16 z = {};
  f32x16 acc[NL][2];
  auto issue = [&](int buf, uint32_t kb) {   // one stage: 4 DMA of token rows, 8 of expert rows
    char* const st = mine + buf * kRouterStage;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LDS_AS void*)(st + g * 1024), 16,
                                               ((g & 1) ? lo1 : lo0) + uint32_t(g) * gstride, kb, 0, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LDS_AS void*)(st + 4096 + g * 1024), 16,
                                               ((g & 1) ? lo1 : lo0) + uint32_t(g) * gstride, kb, 0, 0);
  };
#pragma unroll
  for (int li = 0; li < NL; ++li) {
    const int l = wave + 4 * li;
    acc[li][0] = z;
    acc[li][1] = z;
    if (l < L) {
      const uint32_t kb0 = uint32_t(int64_t(l) * kl * 2);
      issue(0, kb0);
      for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) {
          issue(buf ^ 1, kb0 + uint32_t(st + 1) * 128);
          wait_vmcnt<12>();   // stage st has landed (the 12 loads of stage st + 1 may be in flight)
        } else {
          wait_vmcnt<0>();
        }
        asm volatile("" ::: "memory");
        const char* const sp = mine + buf * kRouterStage;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t ch = uint32_t(((2 * s + fk) ^ ((fr >> 1) & 7)) << 4);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(sp + fr * 128 + ch);
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sp + 4096 + fr * 128 + ch);
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sp + 4096 + (32 + fr) * 128 + ch);
          acc[li][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc[li][0], 0, 0, 0);
          acc[li][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc[li][1], 0, 0, 0);
        }
        // Every fragment read of this buffer has returned before its next DMA is issued.
        wait_lgkm0();
        asm volatile("" ::: "memory");
      }
    }
  }
  __syncthreads();   // every wave is done with its stages: the area takes the leaf blocks
  float* const part = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int li = 0; li < NL; ++li) {
    const int l = wave + 4 * li;
    if (l < L) {
      float* const pl = part + l * 32 * 64;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = (v >> 2) * 8 + fk * 4 + (v & 3);
        const float x0 = acc[li][0][v], x1 = acc[li][1][v];
        pl[row * 64 + fr] = x0;
        pl[row * 64 + 32 + fr] = x1;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int o = tid + 256 * q, row = o >> 6, col = o & 63;
    float p[L];
#pragma unroll
    for (int l = 0; l < L; ++l) p[l] = part[l * 32 * 64 + o];
#pragma unroll
    for (int w = 1; w < L; w *= 2)
#pragma unroll
      for (int j = 0; j + w < L; j += 2 * w) p[j] = p[j] + p[j + w];
    if (t0 + row < T && e0 + col < E) logits[(t0 + row) * int64_t(E) + e0 + col] = p[0];
  }
}

}  // namespace

hipError_t launch_router_logits(const void* H, const void* Wr, float* logits, int64_t T, int64_t K,
                                int n_experts, int leaves_log2, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (n_experts < 1 || K < 64 || leaves_log2 < 0 || leaves_log2 > 4 || (K >> leaves_log2) % 64 != 0 ||
      cdiv(T, 32) > 0x7FFFFFFF || 64 * K * 2 >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  const dim3 grid(unsigned(cdiv(T, 32)), unsigned(cdiv(n_experts, 64))), block(256);
  const uint16_t* h = static_cast<const uint16_t*>(H);
  const uint16_t* w = static_cast<const uint16_t*>(Wr);
  switch (leaves_log2) {
    case 0: hipLaunchKernelGGL(router_logits_kernel<0>, grid, block, 0, s, h, w, logits, T, K, n_experts); break;
    case 1: hipLaunchKernelGGL(router_logits_kernel<1>, grid, block, 0, s, h, w, logits, T, K, n_experts); break;
    case 2: hipLaunchKernelGGL(router_logits_kernel<2>, grid, block, 0, s, h, w, logits, T, K, n_experts); break;
    case 3: hipLaunchKernelGGL(router_logits_kernel<3>, grid, block, 0, s, h, w, logits, T, K, n_experts); break;
    default: hipLaunchKernelGGL(router_logits_kernel<4>, grid, block, 0, s, h, w, logits, T, K, n_experts); break;
  }
  return hipGetLastError();
}

hipError_t launch_moe_route(const float* logits, int64_t T, int n_experts, int topk, int32_t* topk_ids,
                            float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (n_experts < 1 || n_experts > kMaxRouteExperts || topk < 1 || topk > n_experts || topk > 64)
    return hipErrorInvalidValue;
  const dim3 grid(unsigned((T + 3) / 4)), block(256);
  const int per = (n_experts + 63) / 64;
  if (per <= 1)
    hipLaunchKernelGGL(moe_route_kernel<1>, grid, block, 0, s, logits, T, n_experts, topk, topk_ids, topk_w);
  else if (per <= 2)
    hipLaunchKernelGGL(moe_route_kernel<2>, grid, block, 0, s, logits, T, n_experts, topk, topk_ids, topk_w);
  else if (per <= 4)
    hipLaunchKernelGGL(moe_route_kernel<4>, grid, block, 0, s, logits, T, n_experts, topk, topk_ids, topk_w);
  else if (per <= 8)
    hipLaunchKernelGGL(moe_route_kernel<8>, grid, block, 0, s, logits, T, n_experts, topk, topk_ids, topk_w);
  else
    hipLaunchKernelGGL(moe_route_kernel<16>, grid, block, 0, s, logits, T, n_experts, topk, topk_ids, topk_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Deterministic Top-K of positions [BitRL, 4.3]: per row, the k positions of largest key,
// key = (order key of the score, position) as one 64-bit value, so equal
// scores go to the larger position; +0 equals -0, NaN below every number.
// The selected positions are written by descending position, then -1.
//
// One workgroup of 1024 threads per row (four waves per SIMD: the per-key
// phases are chains of dependent vector instructions, which more waves
// overlap).  Slot j of thread t holds position n-1-(1024j+t): each load
// instruction of a wave reads 64 consecutive scores,
// and (slot, wave, lane) order is descending position order.  The threshold
// T, the take-th largest 32-bit score key, is found by a radix select over
// LDS histograms of 11, 11 and 10 bits: each pass counts the keys that share
// the digits found so far and picks the digit at which the count from the
// top reaches the number still wanted.  Keys above T are selected, and of the
// keys equal to T the `need` at the largest positions.
//
// On long rows a sample of 1024 keys first bounds T from below.  When few
// enough keys reach the bound, they are listed in LDS with their positions, in
// descending position order (per-block counts from wave ballots, one scan,
// then each lane's rank in its wave's ballot): the passes count the list (the
// last one only when the keys of T's first bin have low bits set), and the
// output is read off it, each thread taking a run of entries.  Otherwise
// the passes count every key, and the wave ballots of "key > T" and
// "key == T" per slot give a bitmap of the row by descending position; one
// scan over their popcounts gives each 64-position block its output offset
// and tie rank, and the blocks' 16-position quarters, dealt round-robin to
// the threads, write the selected positions.
// ---------------------------------------------------------------------------
namespace {

constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkGroup = 16;                       // slots loaded and tested together
constexpr int kTopkCopies = 8;                       // histogram copies, by lane % 8
constexpr int kTopkHistStride = 2048 + 4;            // words from one copy to the next (4 banks on)
constexpr int kTopkBlocks = kTopkPerThread * kTopkWaves;   // 64-position blocks of the longest row
static_assert(kTopkThreads * 4 >= 2048, "every bin of an 11-bit histogram has an owner in the scan");
static_assert(2 * kTopkThreads * 8 <= kTopkCopies * kTopkHistStride * 4, "the blocks' offsets fit the histograms");
// Keys of the first pass's threshold bin that the last two passes can take
// from a list in LDS (the histogram copies past the first): more fall back to
// scanning every key again.
constexpr int kTopkListCap = (kTopkCopies - 1) * kTopkHistStride;
// The sample that bounds T from below: slot kTopkSampleStride * w of every
// thread of wave w, i.e. 16 runs of 64 consecutive positions spread over the
// longest row.  A row whose sample holds fewer than kTopkMinSample positions
// skips it.
constexpr int kTopkSampleStride = kTopkPerThread / kTopkWaves;
constexpr int kTopkMinSample = 256;
// Keys at or above the sample's bound that the three passes can take from a
// list in LDS.
constexpr int kTopkCandCap = 8192;
static_assert(kTopkBlocks == kTopkThreads, "thread t scans the count of block t");

// f(integral_constant<I>), f(integral_constant<I+1>), ..., below N.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The eight words w0..w7 (uniform) into lanes L..L+7 of `acc`.  The
// compiler does not insert the wait states between a vector instruction that
// writes an SGPR (as a ballot's compare does) and a lane write that reads it
// when the read is in inline asm, so the s_nop gives them.
template <int L>
__device__ __forceinline__ uint32_t write_lanes8(uint32_t acc, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                 uint32_t w4, uint32_t w5, uint32_t w6, uint32_t w7) {
  asm("s_nop 4\n\t"
      "v_writelane_b32 %0, %1, %9\n\t"
      "v_writelane_b32 %0, %2, %9+1\n\t"
      "v_writelane_b32 %0, %3, %9+2\n\t"
      "v_writelane_b32 %0, %4, %9+3\n\t"
      "v_writelane_b32 %0, %5, %9+4\n\t"
      "v_writelane_b32 %0, %6, %9+5\n\t"
      "v_writelane_b32 %0, %7, %9+6\n\t"
      "v_writelane_b32 %0, %8, %9+7"
      : "=v"(acc)
      : "s"(w0), "s"(w1), "s"(w2), "s"(w3), "s"(w4), "s"(w5), "s"(w6), "s"(w7), "n"(L), "0"(acc));
  return acc;
}

// Unsigned order key of a score, larger = ahead: -0 becomes +0; numbers map
// to keys >= 0x007FFFFF, NaN to 1, below every number.  Key 0 marks a slot
// past the row's end, below everything and never selected.
__device__ __forceinline__ uint32_t topk_key(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);
  const uint32_t kk = b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u);
  return __builtin_isnan(v) ? 1u : kk;
}

// Inclusive prefix sum over the wave's lanes: within each row of 16 lanes by
// row shifts, then across rows by the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// Inclusive prefix sums of a and b over the workgroup's threads in thread
// order (ia, ib) and their totals (ta, tb, the same for every thread).  One
// barrier; `red` (2 * waves ints) must not be written again before the
// workgroup has passed another barrier.
__device__ __forceinline__ void block_scan2_topk(int a, int b, int* red, int& ia, int& ib, int& ta, int& tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    red[wave] = xa;
    red[kTopkWaves + wave] = xb;
  }
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int ca = red[w], cb = red[kTopkWaves + w];
    ba += w < wave ? ca : 0;
    bb += w < wave ? cb : 0;
    sa += ca;
    sb += cb;
  }
  ia = ba + xa;
  ib = bb + xb;
  ta = sa;
  tb = sb;
}

// The same for one value.
__device__ __forceinline__ int block_scan1_topk(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = red[w];
    before += w < wave ? c : 0;
    all += c;
  }
  total = all;
  return before + x;
}

__global__ __launch_bounds__(kTopkThreads) void topk_positions_kernel(const float* __restrict__ scores, int64_t ld,
                                                                     const int32_t* __restrict__ lengths, int k,
                                                                     int32_t* __restrict__ out) {
  // The histograms, later the blocks' output offsets and tie ranks.
  __shared__ __attribute__((aligned(16))) uint32_t hist[kTopkCopies * kTopkHistStride];
  __shared__ __attribute__((aligned(16))) uint32_t masks[kTopkBlocks * 4];   // per block: gt lo, hi, eq lo, hi
  __shared__ __attribute__((aligned(16))) int red[4 * kTopkWaves];   // two halves, alternated by pass; scans
  __shared__ int found[2][3];   // per pass parity: digit, keys still wanted, keys in the digit's bin
  // The scores at or above the sample's bound with their positions, then one
  // entry per lane that takes the other slots' writes.
  __shared__ uint2 cand[kTopkCandCap + 64];
  __shared__ uint32_t low_bits;   // list path: OR of the low 10 key bits in the threshold's first bin
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = lengths[r];
  n = n < 0 ? 0 : (int64_t(n) > ld ? int(ld) : n);
  const int take = n < k ? n : k;
  int32_t* o = out + r * int64_t(k);
  const int groups = (n + kTopkThreads * kTopkGroup - 1) / (kTopkThreads * kTopkGroup);
  // The scores' bits, later (on the passes over every key) their keys.
  uint32_t key[kTopkPerThread];
  if (take > 0) {
    // Every load of the groups that reach into the row is issued at once.  A
    // slot before position 0 (only in the last group) has a byte offset that
    // wraps to 2^32 - 4|p| in 32 bits, past the buffer's range of
    // 4n <= 2^18 bytes: it returns 0 with no branch, and the slot then gets a
    // NaN, which no float comparison below selects.
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(scores + r * ld, uint32_t(n) * 4u);
    const uint32_t off0 = uint32_t(n - 1 - tid) * 4u;
    // This wave's sampled slot (see below) has a load of its own, issued
    // first, so that the sample can be counted while the rest lands.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t sv =
        __builtin_amdgcn_raw_buffer_load_b32(rs, off0 - uint32_t(kTopkThreads * 4 * kTopkSampleStride * wv), 0, 0);
#pragma unroll
    for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
      if (g < groups) {
#pragma unroll
        for (int i = 0; i < kTopkGroup; ++i) {
          const uint32_t off = off0 - uint32_t(kTopkThreads * 4 * (kTopkGroup * g + i));
          key[kTopkGroup * g + i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
      if (g == groups - 1) {
#pragma unroll
        for (int i = 0; i < kTopkGroup; ++i) {
          const int j = kTopkGroup * g + i;
          key[j] = n - 1 - (kTopkThreads * j + tid) >= 0 ? key[j] : 0x7FC00000u;
        }
      }
    }
    // Radix select of T.  `rem` = how many of the keys sharing the digits
    // found so far are still wanted.  Lane l counts into histogram copy l % 8
    // (equal digits in one wave then mostly land in different banks).
    uint32_t* const hcopy = hist + (lane & (kTopkCopies - 1)) * kTopkHistStride;
    // The histograms start at zero; each pass's scan clears the words it
    // reads, ready for the next pass.
    for (int i = tid; i < kTopkCopies * kTopkHistStride / 4; i += kTopkThreads)
      reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    // One pass's histogram (NCOP copies) to the digit at which the count from
    // the top reaches `want`: thread t owns bins 4t..4t+3 and clears them as it
    // reads them; `above` counts the bins of the threads after it, i.e. the
    // larger digits.  Ends with a barrier; `par` alternates the scan's area.
    // Bins below first_bin are known to be empty (and clear): their owners
    // skip them.
    auto scan_find = [&](auto ncop, int par, int want, int& digit, int& left, int& bin_n, int first_bin = 0) {
      constexpr int NCOP = decltype(ncop)::value;
      int h[4] = {0, 0, 0, 0};
      if (tid < 2048 / 4 && 4 * tid + 3 >= first_bin) {   // the 2048 bins' owners; the others add 0
#pragma unroll
        for (int c = 0; c < NCOP; ++c) {
          uint4* const w = reinterpret_cast<uint4*>(&hist[c * kTopkHistStride + 4 * tid]);
          const uint4 q = *w;
          *w = make_uint4(0u, 0u, 0u, 0u);
          h[0] += int(q.x);
          h[1] += int(q.y);
          h[2] += int(q.z);
          h[3] += int(q.w);
        }
      }
      const int mine = h[0] + h[1] + h[2] + h[3];
      int total;
      const int incl = block_scan1_topk(mine, red + par * kTopkWaves, total);
      int above = total - incl;
      if (above < want && above + mine >= want) {
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          if (above < want && above + h[b] >= want) {
            found[par][0] = 4 * tid + b;
            found[par][1] = want - above;
            found[par][2] = h[b];
          }
          above += h[b];
        }
      }
      __syncthreads();
      digit = found[par][0];
      left = found[par][1];
      bin_n = found[par][2];
    };
    // Candidates.  The sampled keys give a lower bound P on T: the low edge of
    // the first-digit bin that holds the sample's rs-th largest key, with rs
    // about 1.5 times the sample's share of `take` (plus 8).  If at least
    // `take` and at most kTopkCandCap keys are >= P, those keys are the row's
    // largest and hold every key >= T, so the take-th largest of them is T and
    // the number above T is the same: the three passes count them alone, from
    // a list in LDS, and the output is read off the list.  Otherwise (a
    // sample unlike the row, many equal keys) the passes run over every key.
    // P decides only how much is counted, never T or `need`.
    float Pf = 0.0f;                                 // the score whose key is P
    int ds = 0;                                      // P's first digit
    int total = 0;                                   // keys >= P
    bool use_list = false;
    // Per 64-position block e = slot * waves + wave: its keys >= P, then
    // (after a scan) the list index of its first one.
    uint32_t* const blk = masks;
    {
      int m = 0;                                     // sampled slots inside the row
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) {
        const int v = n - (kTopkThreads * kTopkSampleStride + 64) * w;
        m += v < 0 ? 0 : (v > 64 ? 64 : v);
      }
      const int rs = int(3 * int64_t(take) * m / (2 * int64_t(n))) + 8;
      if (m >= kTopkMinSample && 4 * rs <= m) {
        // This wave's sampled slot, sv; sampled slots past the row are not
        // counted.
        if (n - 1 - (kTopkThreads * kTopkSampleStride * wv + tid) >= 0)
          atomicAdd(&hist[topk_key(__builtin_bit_cast(float, sv)) >> 21], 1u);
        __syncthreads();
        int unused_left, unused_n;
        scan_find(std::integral_constant<int, 1>{}, 0, rs, ds, unused_left, unused_n);
        // Digit 0 holds NaN and the slots past the row: no bound below it.
        if (ds > 0) {
          // key >= P as a float comparison against the score whose key is P;
          // below the keys of numbers (P <= key(-inf)) every number passes.
          // A bound above key(+inf) reads as a NaN and passes nothing.
          const uint32_t P = uint32_t(ds) << 21;
          Pf = P <= 0x007FFFFFu ? -__builtin_inff()
                                : __builtin_bit_cast(float, P >= 0x80000000u ? P ^ 0x80000000u : ~P);
          // Lane j of the wave gathers slot j's count, eight slots at a time.
          uint32_t bc = 0u;
          static_for<0, kTopkPerThread / 8>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if (h / 2 < groups) {
              uint32_t c[8];
#pragma unroll
              for (int q = 0; q < 8; ++q)
                c[q] = uint32_t(__builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_bit_cast(float, key[8 * h + q]) >= Pf)));
              bc = write_lanes8<8 * h>(bc, c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]);
            }
          });
          blk[lane * kTopkWaves + wave] = bc;
          __syncthreads();
          const int c = int(blk[tid]);               // block tid (kTopkBlocks == kTopkThreads)
          const int first = block_scan1_topk(c, red, total) - c;
          blk[tid] = uint32_t(first);
          use_list = total >= take && total <= kTopkCandCap;
          __syncthreads();
        }
      }
    }
    if (use_list) {
      // Every score at or above the bound, with its position, into the list,
      // in block order and by lane within a block, i.e. by descending
      // position.  Other slots write to an entry of their lane past the list
      // (no branches).
      if (tid == 0) low_bits = 0u;
      const int firsts = int(blk[lane * kTopkWaves + wave]);   // lane j: block (slot j, this wave)
      int top_pos = n - 1 - tid;                               // slot 0's position
      float Pw = Pf;
      // Opaque copies (no instruction): the comparisons are made afresh here,
      // straight into the mask the lane counts read, rather than carried over
      // from the counting loop, and a slot's position stays one subtraction.
      asm volatile("" : "+v"(top_pos), "+v"(Pw));
#pragma unroll
      for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g)
        if (g < groups)
#pragma unroll
          for (int i = 0; i < kTopkGroup; ++i) {
            const int j = kTopkGroup * g + i;
            const bool c = __builtin_bit_cast(float, key[j]) >= Pw;
            const uint64_t b = __builtin_amdgcn_ballot_w64(c);
            // the block's first index plus the candidates in lanes below
            const uint32_t at = __builtin_amdgcn_mbcnt_hi(
                uint32_t(b >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(b), uint32_t(__builtin_amdgcn_readlane(firsts, j))));
            cand[c ? at : uint32_t(kTopkCandCap + lane)] = make_uint2(key[j], uint32_t(top_pos - kTopkThreads * j));
          }
      __syncthreads();
      int d0, d1, d2, rem, c0, n1, n2;
      for (int i = tid; i < total; i += kTopkThreads) {   // the listed scores become keys here
        const uint32_t kv = topk_key(__builtin_bit_cast(float, cand[i].x));
        cand[i].x = kv;
        atomicAdd(&hcopy[kv >> 21], 1u);
      }
      __syncthreads();
      // every listed key's first digit is >= P's
      scan_find(std::integral_constant<int, kTopkCopies>{}, 1, take, d0, rem, c0, ds);
      uint32_t prefix = uint32_t(d0);
      uint32_t low = 0u;
      for (int i = tid; i < total; i += kTopkThreads) {
        const uint32_t kv = cand[i].x;
        if ((kv >> 21) == prefix) {
          atomicAdd(&hist[(kv >> 10) & 2047u], 1u);
          low |= kv;
        }
      }
      if (low & 1023u) atomicOr(&low_bits, 1u);
      __syncthreads();
      scan_find(std::integral_constant<int, 1>{}, 0, rem, d1, rem, n1);
      prefix = (prefix << 11) | uint32_t(d1);
      // When every key of the first bin ends in ten zero bits (scores of bf16
      // or fp16 values, say), the keys with T's 22-bit prefix all equal
      // prefix << 10: that is T, and `rem` of them are wanted.  Otherwise the
      // last pass finds the low bits.
      if (low_bits != 0u) {
        for (int i = tid; i < total; i += kTopkThreads) {
          const uint32_t kv = cand[i].x;
          if ((kv >> 10) == prefix) atomicAdd(&hist[kv & 1023u], 1u);
        }
        __syncthreads();
        scan_find(std::integral_constant<int, 1>{}, 1, rem, d2, rem, n2);
      } else {
        d2 = 0;
      }
      const uint32_t T = (prefix << 10) | uint32_t(d2);
      const int need = rem;                          // keys equal to T to take, largest positions first
      // Output off the list: thread t reads a run of consecutive entries;
      // one scan of the runs' counts of keys > T and == T gives each run how
      // many of either come before it.  An entry's offset is the number of
      // selected entries before it: (keys > T before it) + min(need, ties
      // before it); of the ties, the first `need` are taken.
      const int per = (total + kTopkThreads - 1) / kTopkThreads;
      const int i0 = tid * per, i1 = i0 + per < total ? i0 + per : total;
      int ng = 0, nq = 0;
      for (int i = i0; i < i1; ++i) {
        const uint32_t kv = cand[i].x;
        ng += kv > T ? 1 : 0;
        nq += kv == T ? 1 : 0;
      }
      int ig, iq, tg, tq;
      block_scan2_topk(ng, nq, red + 2 * kTopkWaves, ig, iq, tg, tq);
      int gb = ig - ng, qb = iq - nq;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(o, uint32_t(k) * 4u);
      for (int i = i0; i < i1; ++i) {
        const uint2 e = cand[i];
        if (e.x > T) {
          __builtin_amdgcn_raw_buffer_store_b32(e.y, ro, uint32_t(gb + (qb < need ? qb : need)) * 4u, 0, 0);
          ++gb;
        } else if (e.x == T) {
          if (qb < need) __builtin_amdgcn_raw_buffer_store_b32(e.y, ro, uint32_t(gb + qb) * 4u, 0, 0);
          ++qb;
        }
      }
    } else {
      // Every score to its key; slots past the row get key 0.
#pragma unroll
      for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
        if (g < groups) {
#pragma unroll
          for (int i = 0; i < kTopkGroup; ++i) {
            const int j = kTopkGroup * g + i;
            key[j] = topk_key(__builtin_bit_cast(float, key[j]));
          }
          if (g == groups - 1) {
#pragma unroll
            for (int i = 0; i < kTopkGroup; ++i) {
              const int j = kTopkGroup * g + i;
              key[j] = n - 1 - (kTopkThreads * j + tid) >= 0 ? key[j] : 0u;
            }
          }
        }
      }
      int d0, rem, c0;
      // Pass 0 over every key: top 11 bits.
#pragma unroll
      for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
        if (g < groups) {
          if (g != groups - 1) {                       // full groups: every slot counts
#pragma unroll
            for (int i = 0; i < kTopkGroup; ++i) atomicAdd(&hcopy[key[kTopkGroup * g + i] >> 21], 1u);
          } else {                                     // the last group: slots past the row have key 0
#pragma unroll
            for (int i = 0; i < kTopkGroup; ++i) {
              const uint32_t kv = key[kTopkGroup * g + i];
              if (kv != 0u) atomicAdd(&hcopy[kv >> 21], 1u);
            }
          }
        }
      }
      __syncthreads();
      scan_find(std::integral_constant<int, kTopkCopies>{}, 0, take, d0, rem, c0);
      uint32_t prefix = uint32_t(d0);
      if (c0 <= kTopkListCap) {
        // The keys of bin d0 (c0 of them, slots past the row excluded) into a
        // list in the histogram copies past the first, at offsets from a scan of
        // the per-thread counts; passes 1 and 2 then read the list and count into
        // copy 0 alone.  The order of the list does not reach T or `need`.
        uint32_t* const list = hist + kTopkHistStride;
        int cnt = 0;
#pragma unroll
        for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g)
          if (g < groups)
#pragma unroll
            for (int i = 0; i < kTopkGroup; ++i) {
              const uint32_t kv = key[kTopkGroup * g + i];
              cnt += (kv != 0u && (kv >> 21) == prefix) ? 1 : 0;
            }
        int c_all;
        int at = block_scan1_topk(cnt, red + kTopkWaves, c_all) - cnt;
#pragma unroll
        for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g)
          if (g < groups)
#pragma unroll
            for (int i = 0; i < kTopkGroup; ++i) {
              const uint32_t kv = key[kTopkGroup * g + i];
              if (kv != 0u && (kv >> 21) == prefix) list[at++] = kv;
            }
        __syncthreads();
        int d1, d2, n1, n2;
        for (int i = tid; i < c0; i += kTopkThreads) atomicAdd(&hist[(list[i] >> 10) & 2047u], 1u);
        __syncthreads();
        scan_find(std::integral_constant<int, 1>{}, 0, rem, d1, rem, n1);
        prefix = (prefix << 11) | uint32_t(d1);
        for (int i = tid; i < c0; i += kTopkThreads)
          if ((list[i] >> 10) == prefix) atomicAdd(&hist[list[i] & 1023u], 1u);
        __syncthreads();
        scan_find(std::integral_constant<int, 1>{}, 1, rem, d2, rem, n2);
        prefix = (prefix << 10) | uint32_t(d2);
      } else {
        // Passes 1 and 2 over every key again.
#pragma unroll
        for (int pass = 1; pass < 3; ++pass) {
          const int shift = pass == 1 ? 10 : 0;
          const uint32_t dmask = pass == 2 ? 1023u : 2047u;
          const int pshift = pass == 1 ? 21 : 10;      // bits below the digits already found
#pragma unroll
          for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
            if (g < groups) {
              // Four slots per test: a wave with no match in any of them skips
              // the four (the common case in the last pass).
#pragma unroll
              for (int i0 = 0; i0 < kTopkGroup; i0 += 4) {
                bool m[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) m[q] = (key[kTopkGroup * g + i0 + q] >> pshift) == prefix;
                if (m[0] || m[1] || m[2] || m[3]) {
#pragma unroll
                  for (int q = 0; q < 4; ++q)
                    if (m[q]) atomicAdd(&hcopy[(key[kTopkGroup * g + i0 + q] >> shift) & dmask], 1u);
                }
              }
            }
          }
          __syncthreads();
          int d, nb;
          scan_find(std::integral_constant<int, kTopkCopies>{}, pass & 1, rem, d, rem, nb);
          prefix = (prefix << (pass == 2 ? 10 : 11)) | uint32_t(d);
        }
      }
      const uint32_t T = prefix;
      const int need = rem;                            // keys equal to T to take, largest positions first
      // Ballots per slot, gathered 16 slots to a register (lane 4s+q holds word
      // q of slot s of the group) and stored with one write per group.
#pragma unroll
      for (int g = 0; g < kTopkPerThread / kTopkGroup; ++g) {
        if (g < groups) {
          uint32_t acc = 0;
          static_for<0, kTopkGroup / 2>([&](auto ic) {
            constexpr int i = 2 * decltype(ic)::value;
            const uint32_t ka = key[kTopkGroup * g + i], kb = key[kTopkGroup * g + i + 1];
            const uint64_t ga = __builtin_amdgcn_ballot_w64(ka > T), ea = __builtin_amdgcn_ballot_w64(ka == T);
            const uint64_t gb = __builtin_amdgcn_ballot_w64(kb > T), eb = __builtin_amdgcn_ballot_w64(kb == T);
            acc = write_lanes8<4 * i>(acc, uint32_t(ga), uint32_t(ga >> 32), uint32_t(ea), uint32_t(ea >> 32),
                                      uint32_t(gb), uint32_t(gb >> 32), uint32_t(eb), uint32_t(eb >> 32));
          });
          masks[((kTopkGroup * g + (lane >> 2)) * kTopkWaves + wave) * 4 + (lane & 3)] = acc;
        }
      }
      __syncthreads();
      // Blocks e = slot * waves + wave (64 positions each, descending) in order;
      // thread t scans blocks 2t and 2t+1.  Blocks past the row's groups count 0.
      const int used = groups * kTopkGroup * kTopkWaves;
      int pg[2], pq[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * tid + u;
        pg[u] = pq[u] = 0;
        if (e < used) {
          const uint4 m = *reinterpret_cast<const uint4*>(&masks[4 * e]);
          pg[u] = __builtin_popcount(m.x) + __builtin_popcount(m.y);
          pq[u] = __builtin_popcount(m.z) + __builtin_popcount(m.w);
        }
      }
      int ig, iq, tg, tq;
      block_scan2_topk(pg[0] + pg[1], pq[0] + pq[1], red + 2 * kTopkWaves, ig, iq, tg, tq);
      const int gb = ig - pg[0] - pg[1], qb = iq - pq[0] - pq[1];
      // Per block: keys > T and keys == T in the blocks before it.
      int2* const before = reinterpret_cast<int2*>(hist);
      before[2 * tid] = make_int2(gb, qb);
      before[2 * tid + 1] = make_int2(gb + pg[0], qb + pq[0]);
      __syncthreads();
      // Output: a selected position's offset is the number of selected positions
      // above it, = (keys > T above it) + min(need, ties above it).  Quarter
      // u = 4e + c holds positions 16c .. 16c+15 of block e; thread t writes the
      // quarters t, t + 1024, ...  The stores go through a buffer over the row's
      // k outputs, so even an offset out of range could not write outside them.
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(o, uint32_t(k) * 4u);
      uint4 mu[kTopkPerThread / 16];
      int2 bu[kTopkPerThread / 16];
#pragma unroll
      for (int i = 0; i < kTopkPerThread / 16; ++i) {   // every read first, then the writes
        const int e = (tid + kTopkThreads * i) >> 2;
        mu[i] = *reinterpret_cast<const uint4*>(&masks[4 * e]);
        bu[i] = before[e];
      }
#pragma unroll
      for (int i = 0; i < kTopkPerThread / 16; ++i) {
        const int u = tid + kTopkThreads * i;
        if (u >= 4 * used) break;
        const int e = u >> 2, c = u & 3;
        const uint4 m = mu[i];
        const uint64_t gm = uint64_t(m.x) | (uint64_t(m.y) << 32), em = uint64_t(m.z) | (uint64_t(m.w) << 32);
        const uint64_t below = (uint64_t(1) << (16 * c)) - 1;
        uint32_t gq = uint32_t(gm >> (16 * c)) & 0xFFFFu, eq = uint32_t(em >> (16 * c)) & 0xFFFFu;
        if ((gq | eq) == 0u) continue;
        const int2 b = bu[i];
        const int at_g = b.x + __popcll(gm & below), at_q = b.y + __popcll(em & below);
        // The quarter's selected positions go to consecutive offsets from the
        // number selected above it; of its ties, the first need - at_q.
        const int allow = need - at_q;
        uint32_t keep = 0u;
        if (allow > 0) {                               // then keep has more than `drop` bits set
          keep = eq;
          for (int drop = __builtin_popcount(eq) - allow; drop > 0; --drop)
            keep &= ~(0x80000000u >> __builtin_clz(keep));
        }
        uint32_t sel = gq | keep;
        int at = at_g + (at_q < need ? at_q : need);
        const int top = n - 1 - ((e / kTopkWaves) * kTopkThreads + (e % kTopkWaves) * 64 + 16 * c);
        while (sel) {
          const int bit = __builtin_ctz(sel);
          sel &= sel - 1;
          __builtin_amdgcn_raw_buffer_store_b32(top - bit, ro, uint32_t(at) * 4u, 0, 0);
          ++at;
        }
      }
    }
  }
  for (int i = take + tid; i < k; i += kTopkThreads) o[i] = -1;
}

}  // namespace

hipError_t launch_topk_positions(const float* scores, int64_t ld, const int32_t* lengths, int64_t R, int k,
                                 int32_t* out, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (ld < 0 || ld > kTopkMaxLen || k < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_positions_kernel, dim3(unsigned(R)), dim3(kTopkThreads), 0, s, scores, ld, lengths, k,
                     out);
  return hipGetLastError();
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

hipError_t launch_group_gemm(const GroupLaunch& p, hipStream_t s) {
  if (p.n_experts < 1 || p.n_experts > kMaxGroupExperts) return hipErrorInvalidValue;
  switch (p.leaves_log2) {
    case 0: return launch_group_lg<0>(p, s);
    case 1: return launch_group_lg<1>(p, s);
    case 2: return launch_group_lg<2>(p, s);
    case 3: return launch_group_lg<3>(p, s);
    case 4: return launch_group_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp8_quantize(const uint16_t* X, int64_t ldx, uint8_t* Q, int64_t ldq, uint8_t* S, int64_t R,
                               int64_t C, int block_rows, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const int64_t ngroups = cdiv(C, 128);
  if (block_rows == 1 && C % 4 == 0 && ldx % 4 == 0 && ldq % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(Q) & 3) == 0) {
    // One workgroup per row (its four waves walk the row's group pairs):
    // short waves would leave the launch dominated by dispatch.
    hipLaunchKernelGGL(fp8_quant_rows4_kernel, dim3(1u, unsigned(R < 65535 ? R : 65535)), dim3(256), 0, s, X, ldx, Q,
                       ldq, S, R, C);
  } else if (block_rows == 1) {
    const int64_t waves = R * ngroups;
    const int64_t wgs = cdiv(waves, 4);
    hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3(unsigned(wgs < 65536 ? wgs : 65536)), dim3(256), 0, s, X, ldx,
                       Q, ldq, S, R, C);
  } else if (block_rows == 128) {
    if (cdiv(R, 128) > 65535) return hipErrorInvalidValue;
    if (C % 4 == 0 && ldx % 4 == 0 && ldq % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 7) == 0 &&
        (reinterpret_cast<uintptr_t>(Q) & 3) == 0)
      hipLaunchKernelGGL(fp8_quant_blocks4_kernel, dim3(unsigned(ngroups), unsigned(cdiv(R, 128))), dim3(256), 0, s,
                         X, ldx, Q, ldq, S, R, C);
    else
      hipLaunchKernelGGL(fp8_quant_blocks_kernel, dim3(unsigned(ngroups), unsigned(cdiv(R, 128))), dim3(256), 0, s,
                         X, ldx, Q, ldq, S, R, C);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fp8_group_gemm(const Fp8GroupLaunch& p, hipStream_t s) {
  if (p.n_experts < 1 || p.n_experts > kMaxGroupExperts) return hipErrorInvalidValue;
  switch (p.leaves_log2) {
    case 0: return launch_fp8_group_lg<0>(p, s);
    case 1: return launch_fp8_group_lg<1>(p, s);
    case 2: return launch_fp8_group_lg<2>(p, s);
    case 3: return launch_fp8_group_lg<3>(p, s);
    case 4: return launch_fp8_group_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp8_gemm(const Fp8GemmLaunch& p, hipStream_t s) {
  switch (p.leaves_log2) {
    case 0: return launch_fp8_lg<0>(p, s);
    case 1: return launch_fp8_lg<1>(p, s);
    case 2: return launch_fp8_lg<2>(p, s);
    case 3: return launch_fp8_lg<3>(p, s);
    case 4: return launch_fp8_lg<4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_silu_mul_fp8(const float* GU, int64_t ldgu, uint8_t* Q, int64_t ldq, uint8_t* S, int64_t R,
                               int64_t I, hipStream_t s) {
  if (R <= 0 || I <= 0) return hipSuccess;
  if (I % 4 || ldgu % 4 || ldq % 4 || (reinterpret_cast<uintptr_t>(GU) & 15) || (reinterpret_cast<uintptr_t>(Q) & 3))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(silu_mul_fp8_kernel, dim3(1u, unsigned(R < 65535 ? R : 65535)), dim3(256), 0, s, GU, ldgu, Q,
                     ldq, S, R, I);
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* Q, const uint8_t* S, int64_t R, int64_t C, int block_rows,
                              uint16_t* out, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const int64_t th = R * cdiv(C, 8);
  const int64_t wgs = cdiv(th, 256);
  hipLaunchKernelGGL(fp8_dequant_kernel, dim3(unsigned(wgs < 65536 ? wgs : 65536)), dim3(256), 0, s, Q, S, R, C,
                     block_rows, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* GU, int64_t ldgu, uint16_t* out, int64_t ldo, int64_t rows, int64_t I,
                           hipStream_t s) {
  if (rows <= 0 || I <= 0) return hipSuccess;
  const bool vec = I % 4 == 0 && ldgu % 4 == 0 && ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(GU) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & 7) == 0 && rows * (I / 4) < (int64_t(1) << 31);
  if (vec) {
    const int64_t total = rows * (I / 4);
    const int64_t wgs = cdiv(total, 256 * 4);
    hipLaunchKernelGGL(silu_mul_vec_kernel, dim3(unsigned(wgs < 65536 ? wgs : 65536)), dim3(256), 0, s, GU, ldgu,
                       out, ldo, uint32_t(rows), uint32_t(I / 4));
  } else {
    const int64_t cx = cdiv(I, 256);
    hipLaunchKernelGGL(silu_mul_kernel, dim3(unsigned(cx < 64 ? cx : 64), unsigned(rows < 65535 ? rows : 65535)),
                       dim3(256), 0, s, GU, ldgu, out, ldo, rows, I);
  }
  return hipGetLastError();
}

}  // namespace tig
