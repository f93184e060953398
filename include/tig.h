/*
 * tig.h -- batch-invariant token logprobs on AMD MI355X (gfx950), C ABI.
 *
 * The method (from three web pages; titles are given once here and shortened
 * afterwards):
 *   [IsoExec]  "IsoExec: Unified Execution to Eliminate Trainer-Inference
 *              Mismatch in SkyRL", section "Parallelism-invariant kernels" and
 *              its figure of the fixed binary reduction tree; the contract
 *              example in "Unified execution contract" (leaves = 8, FP32
 *              leaves).
 *   [BitRL]    "Termina el entrenamiento RL mas rapido: Consistente a nivel de
 *              bits, de alto rendimiento y dirigido por agentes", section 2
 *              (diff = 0 per sampled token; batch independence; prefill/decode
 *              consistency), 4.1 (one accumulation order for every M; block
 *              FP8 W8A8), 4.3
 *              (deterministic Top-K of positions: key, ties, order), 4.4 and
 *              4.5 (expert outputs combined in FP32 in a fixed order), 4.6
 *              (no host sync, workspaces sized from static bounds).
 *   [RZero]    "REINFORCE Zero: ..." section 6 (MI355X): libraries that pick
 *              kernels by shape (e.g. a different tile at 4096 vs 4097 rows)
 *              break batch invariance.
 *
 * Numerical contract, fixed per (K, leaves) and never chosen from M or N:
 *   - K is cut into `leaves` contiguous leaves of K/leaves columns;
 *   - inside a leaf, one matrix-core instruction (v_mfma_f32_32x32x16_bf16)
 *     accumulates 16-column k-steps in ascending order into an FP32 tile that
 *     starts at +0;
 *   - the leaves are combined by a balanced tree of adjacent pairs, level by
 *     level, in FP32 (round to nearest even);
 *   - for the log-softmax: per row and per 128-column vocabulary tile,
 *     m_t = max and s_t = sum of exp2((x - m_t) * log2(e)) over the tile by a
 *     balanced adjacent-pair tree (padded columns add exactly +0); then
 *     g = max_t m_t and S = sum_t s_t * exp2((m_t - g) * log2(e)) by a balanced
 *     adjacent-pair tree over the tiles zero-padded to a power of two, and
 *     lse = g + log2(S) * ln(2); logprob = x[id] - lse.
 * A row's bits therefore depend only on that row, the weights, K and leaves:
 * not on M, on the row's position, or on how rows are split into calls.
 *
 * Conventions for every entry point:
 *   - all matrices are row-major; bf16 operands are K-contiguous;
 *   - every pointer argument is a device pointer the caller owns (for example
 *     torch.empty(..., device="cuda")); the library allocates nothing and keeps
 *     no pointer after the call returns;
 *   - work is enqueued on `stream` (NULL = the default stream); no call waits
 *     on the device or reads device memory back;
 *   - arguments are validated on the host before any launch; a failing call
 *     launches nothing and returns a status; tig_last_error() gives a message
 *     for the calling thread's last failure;
 *   - bf16 pointers must be 16-byte aligned and their row strides multiples of
 *     8 elements (16 bytes), else TIG_ERR_UNSUPPORTED;
 *   - a workspace holds one call's intermediate data from its launch to its
 *     last kernel: calls that may run at the same time (other streams) need
 *     workspaces of their own; outputs must not overlap inputs.
 */
#ifndef TIG_H
#define TIG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TIG_OK = 0,
  TIG_ERR_INVALID_ARG = 1, /* null pointer, negative size, leaves not a power of two, ... */
  TIG_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  TIG_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query says */
  TIG_ERR_HIP = 4          /* a HIP runtime call or a launch failed */
} tig_status;

typedef enum { TIG_OUT_F32 = 0, TIG_OUT_BF16 = 1 } tig_out_dtype;

/*
 * Leaf-tree contraction  C[m, n] = tree_l( sum_{k in leaf l} A[m, k] * W[n, k] ).
 * [IsoExec, Parallelism-invariant kernels]; [BitRL, 4.1].
 *   A     bf16 [M, K], row stride lda (elements, >= K)
 *   W     bf16 [N, K], row stride ldw (elements, >= K)   (a Linear weight)
 *   C     [M, N], row stride ldc (elements, >= N); FP32 tree output, or that
 *         value rounded once to bf16 (nearest even) when out_dtype is BF16
 *   leaves  power of two in [1, 64]; K % leaves == 0
 * Implemented: leaves <= 16 and K/leaves a multiple of 64; A and W 16-byte
 * aligned with row strides a multiple of 8; 192 rows of A (128 at 16 leaves)
 * and 128 rows of W each spanning less than 2 GiB (else UNSUPPORTED).
 * M == 0 or N == 0 is TIG_OK and launches nothing.  C must not overlap A or W.
 */
tig_status tig_tree_gemm(const void* A, int64_t lda, const void* W, int64_t ldw,
                         void* C, int64_t ldc, tig_out_dtype out_dtype,
                         int64_t M, int64_t N, int64_t K, int32_t leaves,
                         hipStream_t stream);

/*
 * Fused LM-head logprob of the sampled tokens, the M x V logits never stored.
 * [BitRL, section 2]: the logprob of each sampled token, identical bit for bit
 * whatever the batch, position or prefill/decode split.
 *   H            bf16 [M, K] contiguous (hidden states)
 *   W            bf16 [n_vocab, K] contiguous (LM-head weight)
 *   ids          int64 [M], sampled token per row; an id outside
 *                [0, n_vocab) gives logprob NaN for that row only (checked
 *                on the device, no error code: nothing is read back)
 *   logprob_out  float [M]
 *   lse_out      float [M] log-sum-exp of the row's logits, or NULL to skip
 *   workspace    device scratch of at least tig_logprob_workspace_bytes()
 *                bytes, 256-byte aligned; contents on entry are ignored
 * Implemented: leaves <= 16, K/leaves a multiple of 64, n_vocab <= 2^23, and
 * 192 rows of H spanning less than 2 GiB (K < 5592406), at every M (else
 * UNSUPPORTED, whatever the batch size).
 * M == 0 is TIG_OK and launches nothing.
 */
tig_status tig_logprob_gather(const void* H, const void* W, const int64_t* ids,
                              float* logprob_out, float* lse_out,
                              int64_t M, int64_t K, int64_t n_vocab, int32_t leaves,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Workspace bytes tig_logprob_gather needs for these sizes (written to *bytes):
 * 8 bytes per row per 128-column vocabulary tile, 4 per row per leaf, and at
 * 16 leaves with 192-row tiles (M above 128 where that needs fewer tiles) a
 * further 24 MiB where each tile parks the root of its first 8 leaves.
 */
tig_status tig_logprob_workspace_bytes(int64_t M, int64_t K, int64_t n_vocab,
                                       int32_t leaves, size_t* bytes);

/*
 * tig_logprob_gather with no workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  The same kernels, so the same bits, as
 * tig_logprob_gather on the same arguments.  The intermediate data lives in a
 * fixed device array of TIG_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; its address is looked up once
 * per device, on the first call there.  No call allocates or frees memory.
 *   Limit: calls whose tig_logprob_workspace_bytes() exceeds
 *   TIG_NOALLOC_SCRATCH_BYTES return TIG_ERR_UNSUPPORTED (for a 151936-token
 *   vocabulary at 8 leaves: more than about 3500 rows).
 *   Every call on one GPU uses that GPU's one array: calls that may overlap on
 *   a GPU (other streams, other host threads) race, and the caller must order
 *   them.  Nothing in the array has to start at zero; it keeps the last call's
 *   contents.
 * Other arguments, limits and errors: as tig_logprob_gather.
 */
#define TIG_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
tig_status tig_logprob_gather_noalloc(const void* H, const void* W, const int64_t* ids,
                                      float* logprob_out, float* lse_out,
                                      int64_t M, int64_t K, int64_t n_vocab, int32_t leaves,
                                      hipStream_t stream);

/*
 * MoE-shaped contraction with a fixed-order FP32 combine.
 * [BitRL, 4.4] per-row expert result independent of layout; [BitRL, 4.5] and
 * [IsoExec, Parallelism-invariant kernels] expert outputs combined in a fixed
 * routing order.  Order used here: ascending expert id (equal ids keep slot
 * order); acc = acc + w * y, an FP32 multiply then an FP32 add, from +0.
 *   H          bf16 [T, K] contiguous (tokens)
 *   W_experts  bf16 [n_experts, N, K] contiguous
 *   topk_ids   int32 [T, topk], each in [0, n_experts); an id out of range
 *              makes that token's output NaN (device-side check)
 *   topk_w     float [T, topk] gate weights
 *   out        float [T, N]
 *   workspace  >= tig_moe_workspace_bytes() bytes, 256-byte aligned
 * Each expert's rows are gathered on the device (stable by token index) and
 * multiplied by the same leaf-tree kernel as tig_tree_gemm with FP32 output,
 * so a token's expert output equals tig_tree_gemm on that token's row alone.
 * The grid is sized from the static bound T*topk; nothing is read back.
 * Implemented: leaves <= 16, K/leaves a multiple of 64, topk <= 16, n_experts <= 4096.
 */
tig_status tig_moe_tree_gemm_combine(const void* H, const void* W_experts, int32_t n_experts,
                                     const int32_t* topk_ids, const float* topk_w, int32_t topk,
                                     float* out, int64_t T, int64_t N, int64_t K, int32_t leaves,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Workspace bytes tig_moe_tree_gemm_combine needs (written to *bytes). */
tig_status tig_moe_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t n_experts,
                                   int32_t topk, size_t* bytes);

/*
 * MoE router on the GPU, batch-invariant: [BitRL, 4.1] the router gate is one
 * GEMM with FP32 output at every batch size; [BitRL, 1] once the logits match,
 * the top-k tie-breaking and output order must be fixed too.
 *   logits = leaf-tree(H Wr^T) in FP32 (exactly tig_tree_gemm with FP32 out);
 *   topk_ids[t] = the topk largest logits of token t, largest first; equal
 *     logits in ascending expert id; +0 equals -0; NaN after every number;
 *   topk_w[t] = softmax over those logits: m = the largest,
 *     e_s = exp2((l_s - m) * log2 e) (hardware exp2), the sum of the e_s by
 *     the balanced adjacent-pair tree over the slots zero-padded to a power
 *     of two, topk_w = e_s / sum (IEEE FP32 division).
 * The outputs are the routing inputs of tig_moe_tree_gemm_combine.
 *   H         bf16 [T, K] contiguous (tokens)
 *   Wr        bf16 [n_experts, K] contiguous (router weight)
 *   logits    float [T, n_experts] out (caller-owned; also the kernel's scratch)
 *   topk_ids  int32 [T, topk] out
 *   topk_w    float [T, topk] out
 * Implemented: n_experts <= 1024, topk <= 16, leaves <= 16, K/leaves a
 * multiple of 64.  T == 0 is TIG_OK and launches nothing.
 */
tig_status tig_moe_route(const void* H, const void* Wr, float* logits, int32_t* topk_ids,
                         float* topk_w, int64_t T, int64_t K, int32_t n_experts, int32_t topk,
                         int32_t leaves, hipStream_t stream);

/*
 * Expert GEMM on two layouts with the same per-row result, [BitRL, 4.4]: the
 * rollout side feeds the experts a masked layout (a fixed-capacity block per
 * expert), the training side a contiguous one (experts packed in order, with
 * alignment padding); a row's result must not depend on which, nor on the
 * other rows.  Here every expert's rows are cut into m-tiles that run the
 * leaf-tree contraction of tig_tree_gemm against that expert's W slice:
 *   Y[r] = leaf-tree(X[r] W[e]^T) for every row r the layout gives to expert e,
 * bit for bit the row tig_tree_gemm gives for X[r] alone against W[e].
 *   X       bf16 [rows, K] contiguous; W bf16 [n_experts, N, K] contiguous
 *   counts  int32 [n_experts] on the device: rows of each expert (below 0
 *           counts as 0)
 *   Y       [rows, N] contiguous, FP32 or bf16 (RNE of the FP32 value); rows
 *           no expert owns are not written
 *   workspace >= tig_expert_workspace_bytes(rows, n_experts), 256-byte
 *           aligned (the work items, built on the device: nothing is read back)
 * Masked: rows = n_experts * cap; expert e owns rows e*cap .. e*cap +
 * min(count, cap) - 1.  Contiguous: expert e owns count_e rows from the sum
 * over e' < e of count_e' rounded up to a multiple of `align`; rows that would
 * lie at or past M are not computed.  Implemented: n_experts <= 1024,
 * leaves <= 16, K/leaves a multiple of 64, K a multiple of 8.
 */
tig_status tig_expert_gemm_masked(const void* X, const int32_t* counts, const void* W, void* Y,
                                  tig_out_dtype out_dtype, int32_t n_experts, int64_t cap, int64_t N,
                                  int64_t K, int32_t leaves, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
tig_status tig_expert_gemm_contiguous(const void* X, const int32_t* counts, int64_t align, const void* W,
                                      void* Y, tig_out_dtype out_dtype, int32_t n_experts, int64_t M,
                                      int64_t N, int64_t K, int32_t leaves, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of the expert GEMMs over `rows` rows (written to *bytes). */
tig_status tig_expert_workspace_bytes(int64_t rows, int32_t n_experts, size_t* bytes);

/*
 * The activation between the two expert GEMMs, [BitRL, 4.4] condition 3:
 * SiLU(gate) * up computed in FP32 and rounded to bf16 once (rounding SiLU
 * first can move the product by one bf16 step).
 *   GU   float [rows, ldgu]: gate in columns 0 .. I-1, up in I .. 2I-1
 *   out  bf16 [rows, ldo]: out[r, i] = RNE_bf16(SiLU(g) * u), SiLU(g) =
 *        g * sigmoid(g), sigmoid(g) = 1/(1+t) for g >= 0 and t/(1+t) below,
 *        t = 2^(-|g| log2 e) (hardware exp2), each step an FP32 operation
 * Needs ldgu >= 2I, ldo >= I.  rows == 0 or I == 0 is TIG_OK.
 */
tig_status tig_silu_mul(const float* GU, int64_t ldgu, void* out, int64_t ldo, int64_t rows, int64_t I,
                        hipStream_t stream);

/*
 * The expert GEMM of the two layouts in block FP8 on the FP8 matrix cores,
 * [BitRL, 4.4] (the experts' FP8 grouped GEMM; condition 1: the same FP8
 * input in both layouts, rounded per element to nearest; condition 2: a
 * layout-independent per-row result): the rows and layouts of
 * tig_expert_gemm_masked / _contiguous, the contraction of tig_fp8_tree_gemm
 * (so a row's result equals tig_fp8_tree_gemm on that row alone against its
 * expert's W).
 *   QX [rows, K] E4M3 and SX [rows, K/128] E8M0 (per row and 128 columns, as
 *   tig_fp8_quantize with block_rows = 1 writes them); QW [n_experts, N, K]
 *   and SW [n_experts, ceil(N/128), K/128] (each expert's W quantised in
 *   128 x 128 blocks); Y [rows, N] FP32 or bf16, rows no expert owns not
 *   written; workspace >= tig_expert_fp8_workspace_bytes(rows, n_experts, N,
 *   K), 256-byte aligned (work items and the call's scale table).
 * Implemented: n_experts <= 1024, K/leaves a multiple of 128, leaves <= 16.
 */
tig_status tig_expert_fp8_gemm_masked(const uint8_t* QX, const uint8_t* SX, const int32_t* counts, const uint8_t* QW,
                                      const uint8_t* SW, void* Y, tig_out_dtype out_dtype, int32_t n_experts,
                                      int64_t cap, int64_t N, int64_t K, int32_t leaves, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
tig_status tig_expert_fp8_gemm_contiguous(const uint8_t* QX, const uint8_t* SX, const int32_t* counts, int64_t align,
                                          const uint8_t* QW, const uint8_t* SW, void* Y, tig_out_dtype out_dtype,
                                          int32_t n_experts, int64_t M, int64_t N, int64_t K, int32_t leaves,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream);
tig_status tig_expert_fp8_workspace_bytes(int64_t rows, int32_t n_experts, int64_t N, int64_t K, size_t* bytes);

/*
 * The activation between the expert GEMMs and the FP8 input of the second,
 * [BitRL, 4.4] condition 3: SiLU(gate) * up in FP32, rounded to bf16 once
 * (exactly tig_silu_mul), then quantised to block FP8 in 1 x 128 blocks per
 * row (exactly tig_fp8_quantize with block_rows = 1 on that bf16 result).
 *   GU      float [rows, ldgu]: gate in columns 0 .. I-1, up in I .. 2I-1
 *   Q       uint8 [rows, ldq] out: E4M3 bytes; scales uint8 [rows, ceil(I/128)]
 *           out: E8M0 bytes
 * Needs I, ldgu and ldq multiples of 4, GU 16-byte and Q 4-byte aligned
 * (TIG_ERR_UNSUPPORTED otherwise).
 */
tig_status tig_silu_mul_fp8(const float* GU, int64_t ldgu, uint8_t* Q, int64_t ldq, uint8_t* scales, int64_t rows,
                            int64_t I, hipStream_t stream);

/*
 * Block FP8 quantisation, [BitRL, 4.1] (BF16 master weights quantised to block
 * FP8 by the deployment rule, W8A8) and [BitRL, 4.4] (per-element round to
 * nearest): OCP E4M3 values (largest 448) with one power-of-two scale 2^e per
 * block, e the smallest integer >= -127 with amax <= 448 * 2^e (0 for an
 * all-zero block); each element x * 2^-e (exact) is rounded to E4M3 once, to
 * nearest even.  Blocks are block_rows x 128: 1 x 128 for activations (one per
 * token and 128 columns), 128 x 128 for weights; a block cut by the matrix
 * edge takes the elements it has.
 *   X       bf16 [R, ldx] (row r at X + r*ldx)
 *   Q       uint8 [R, ldq] out: E4M3 bytes
 *   scales  uint8 [ceil(R/block_rows), ceil(C/128)] out, row-major: E8M0 bytes
 *           e + 127
 * A row's quantisation depends only on its own block(s).
 */
tig_status tig_fp8_quantize(const void* X, int64_t ldx, uint8_t* Q, int64_t ldq, uint8_t* scales, int64_t R,
                            int64_t C, int32_t block_rows, hipStream_t stream);

/* Dequantise (exact): out bf16 [R, C] = E4M3 value of Q [R, C] (contiguous)
 * times 2^e of its block; scales as written by tig_fp8_quantize. */
tig_status tig_fp8_dequantize(const uint8_t* Q, const uint8_t* scales, void* out, int64_t R, int64_t C,
                              int32_t block_rows, hipStream_t stream);

/*
 * W8A8 block-FP8 leaf-tree GEMM on the FP8 matrix cores, [BitRL, 4.1] (one
 * accumulation order for every M) with [IsoExec, Parallelism-invariant kernels]
 * (K cut into `leaves` contiguous leaves, FP32 per leaf, fixed binary tree):
 * A is quantised in 1 x 128 blocks, W in 128 x 128 blocks (tig_fp8_quantize).
 * Inside a leaf, one instruction (v_mfma_scale_f32_32x32x64_f8f6f4) takes
 * 64-wide k-steps in ascending order from +0: each E4M3 product times the
 * E8M0 scales of its row and column (exact: powers of two), accumulated in
 * FP32; the leaves combine by the balanced adjacent-pair tree in FP32.  A
 * row's result depends only on that row (its quantisation is per token).
 *   QA [M, K] and SA [M, K/128]; QW [N, K] and SW [ceil(N/128), K/128], all
 *   contiguous; C [M, ldc] FP32 or bf16 (RNE).
 *   workspace >= tig_fp8_gemm_workspace_bytes(M, N, K), 256-byte aligned (the
 *   call's scale table, built on the device).
 * Implemented: K/leaves a multiple of 128, leaves <= 16, QA/QW 16-byte aligned.
 */
tig_status tig_fp8_tree_gemm(const uint8_t* QA, const uint8_t* SA, const uint8_t* QW, const uint8_t* SW, void* C,
                             int64_t ldc, tig_out_dtype out_dtype, int64_t M, int64_t N, int64_t K, int32_t leaves,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);
tig_status tig_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);

/*
 * Deterministic Top-K of positions, [BitRL, 4.3] (the sparse-attention
 * indexer's selection and the figure of its 64-bit key): row r's candidates
 * are its positions 0 .. lengths[r]-1; a position is ahead of another when
 * its score is larger, or the scores are equal and its position is larger
 * (the key is score, then in-request position, so a request's result does not
 * depend on where it sits in the batch).  +0 equals -0; NaN scores come after
 * every number.  The min(k, lengths[r]) selected positions are written by
 * descending position, then -1 up to k.
 *   scores   float [R, ld] (row r at scores + r*ld; only the first
 *            lengths[r] entries are read)
 *   lengths  int32 [R] on the device; values below 0 count as 0, above ld
 *            as ld
 *   out      int32 [R, k] out
 * One workgroup per row.  Implemented: ld <= 65536 (TIG_ERR_UNSUPPORTED
 * above), k >= 1 (any k; entries past the row's length are -1).  R == 0 is
 * TIG_OK and launches nothing.
 */
tig_status tig_topk_positions(const float* scores, int64_t ld, const int32_t* lengths, int64_t R,
                              int32_t k, int32_t* out, hipStream_t stream);

/*
 * The pinned numerical policy for (K, leaves): the constants that decide the
 * bits, in the spirit of [IsoExec, Unified execution contract] (implementation
 * and constants pinned per region; identities are SHA-256 digests).
 * `policy` is a canonical NUL-terminated text; `digest` is SHA-256 of its bytes
 * (without the NUL).  N and M never enter it.
 */
typedef struct {
  int32_t version;     /* policy version */
  int32_t leaves;      /* L */
  int32_t leaf_len;    /* K / L */
  int32_t block_m;     /* rows of the dense kernels' tallest tile (192; 128 at 16 leaves); shorter tiles (128, and 64 in tig_tree_gemm) are a per-call schedule choice that never changes a bit */
  int32_t block_n;     /* columns per workgroup tile = vocabulary tile width */
  int32_t block_k;     /* k columns staged per LDS step (does not change bits) */
  int32_t mfma_m, mfma_n, mfma_k; /* 32, 32, 16 */
  int32_t tree_id;     /* 1 = balanced tree of adjacent pairs */
  uint8_t digest[32];
  char policy[512];
} tig_plan;

tig_status tig_plan_describe(int64_t K, int32_t leaves, tig_plan* out);

/* Static text for a status code ("unknown status" for other values). */
const char* tig_status_string(tig_status s);

/* Message for the calling thread's most recent failing call ("" if none). */
const char* tig_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TIG_H */
