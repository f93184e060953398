// Host side of the C ABI declared in include/tig.h: argument validation, the
// pinned policy descriptor, workspace queries and the calls into the kernel
// launchers.  Everything here runs on the host before any launch, so every
// error path can be exercised without a GPU.
#include "tig.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "tig_internal.h"

namespace {

thread_local std::string g_last_error;

tig_status fail(tig_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tig_status fail(tig_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tig_status ok() {
  g_last_error.clear();
  return TIG_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared checks on (K, leaves): the part of the contract that fixes the bits.
tig_status check_k_leaves(int64_t K, int32_t leaves) {
  if (K <= 0) return fail(TIG_ERR_INVALID_ARG, "K must be positive (got %lld)", (long long)K);
  if (!is_pow2(leaves) || leaves > 64)
    return fail(TIG_ERR_INVALID_ARG, "leaves must be a power of two in [1, 64] (got %d)", leaves);
  if (leaves > (1 << tig::kMaxLeavesLog2))
    return fail(TIG_ERR_UNSUPPORTED, "leaves > %d not implemented (got %d)",
                1 << tig::kMaxLeavesLog2, leaves);
  if (K % leaves != 0)
    return fail(TIG_ERR_UNSUPPORTED, "K (%lld) is not a multiple of leaves (%d)", (long long)K,
                leaves);
  if ((K / leaves) % tig::kBlockK != 0)
    return fail(TIG_ERR_UNSUPPORTED, "leaf length K/leaves = %lld is not a multiple of %d",
                (long long)(K / leaves), tig::kBlockK);
  return TIG_OK;
}

// Byte offsets inside one operand are 32-bit: bound the per-tile span.
tig_status check_span(const char* what, int64_t rows, int64_t ld) {
  if (rows * ld * 2 >= (int64_t(1) << 31))
    return fail(TIG_ERR_UNSUPPORTED, "%s spans too many bytes for 32-bit offsets", what);
  return TIG_OK;
}

// ---------------------------------------------------------------------------
// SHA-256 (FIPS 180-4), used for the policy digest.
// ---------------------------------------------------------------------------
struct Sha256 {
  uint32_t h[8] = {0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au,
                   0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u};
  uint8_t buf[64];
  uint64_t bits = 0;
  size_t used = 0;

  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

  void block(const uint8_t* p) {
    static const uint32_t k[64] = {
        0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u,
        0xab1c5ed5u, 0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu,
        0x9bdc06a7u, 0xc19bf174u, 0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu,
        0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau, 0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u,
        0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u, 0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu,
        0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u, 0xa2bfe8a1u, 0xa81a664bu,
        0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u, 0x19a4c116u,
        0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
        0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u,
        0xc67178f2u};
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = (uint32_t(p[4 * i]) << 24) | (uint32_t(p[4 * i + 1]) << 16) |
             (uint32_t(p[4 * i + 2]) << 8) | uint32_t(p[4 * i + 3]);
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = hh + S1 + ch + k[i] + w[i];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + mj;
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }

  void update(const uint8_t* p, size_t n) {
    bits += uint64_t(n) * 8;
    while (n--) {
      buf[used++] = *p++;
      if (used == 64) {
        block(buf);
        used = 0;
      }
    }
  }

  void finish(uint8_t out[32]) {
    const uint64_t total = bits;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (used != 56) update(&zero, 1);
    uint8_t len[8];
    for (int i = 0; i < 8; ++i) len[i] = uint8_t(total >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = uint8_t(h[i] >> (24 - 8 * j));
  }
};

}  // namespace

extern "C" {

const char* tig_status_string(tig_status s) {
  switch (s) {
    case TIG_OK: return "ok";
    case TIG_ERR_INVALID_ARG: return "invalid argument";
    case TIG_ERR_UNSUPPORTED: return "unsupported";
    case TIG_ERR_WORKSPACE: return "workspace too small";
    case TIG_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* tig_last_error(void) { return g_last_error.c_str(); }

tig_status tig_plan_describe(int64_t K, int32_t leaves, tig_plan* out) {
  if (!out) return fail(TIG_ERR_INVALID_ARG, "out is NULL");
  tig_status s = check_k_leaves(K, leaves);
  if (s != TIG_OK) return s;
  memset(out, 0, sizeof *out);
  out->version = tig::kPolicyVersion;
  out->leaves = leaves;
  out->leaf_len = int32_t(K / leaves);
  out->block_m = tig::block_m_for_log2(log2i(leaves));
  out->block_n = tig::kBlockN;
  out->block_k = tig::kBlockK;
  out->mfma_m = tig::kMfmaM;
  out->mfma_n = tig::kMfmaN;
  out->mfma_k = tig::kMfmaK;
  out->tree_id = 1;
  snprintf(out->policy, sizeof out->policy,
           "tig-policy v%d;K=%lld;leaves=%d;leaf_len=%d;leaf_split=contiguous-equal;"
           "leaf_acc=fp32;leaf_op=v_mfma_f32_32x32x16_bf16;kstep=16-ascending;leaf_init=+0;"
           "tree=balanced-adjacent-pairs-fp32-rne;vocab_tile=%d;"
           "tile_max=exact;tile_sum=balanced-adjacent-pairs(exp2((x-m)*log2e));"
           "tile_combine=balanced-adjacent-pairs-pow2-zero-pad(s*exp2((m-g)*log2e));"
           "lse=g+log2(S)*ln2;logprob=x[id]-lse;"
           "moe_combine=ascending-expert-id,acc+fl(w*y),fp32-rne,init+0;bf16_out=rne",
           tig::kPolicyVersion, (long long)K, leaves, int(K / leaves), tig::kBlockN);
  Sha256 h;
  h.update(reinterpret_cast<const uint8_t*>(out->policy), strlen(out->policy));
  h.finish(out->digest);
  return ok();
}

tig_status tig_tree_gemm(const void* A, int64_t lda, const void* W, int64_t ldw, void* C,
                         int64_t ldc, tig_out_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                         int32_t leaves, hipStream_t stream) {
  if (M < 0 || N < 0) return fail(TIG_ERR_INVALID_ARG, "M and N must be >= 0");
  tig_status s = check_k_leaves(K, leaves);
  if (s != TIG_OK) return s;
  if (out_dtype != TIG_OUT_F32 && out_dtype != TIG_OUT_BF16)
    return fail(TIG_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (lda < K || ldw < K || ldc < N)
    return fail(TIG_ERR_INVALID_ARG, "leading dimensions must cover the rows (lda, ldw >= K; ldc >= N)");
  if (M == 0 || N == 0) return ok();
  if (!A || !W || !C) return fail(TIG_ERR_INVALID_ARG, "A, W and C must not be NULL");
  if (!aligned(A, 16) || !aligned(W, 16) || lda % 8 || ldw % 8)
    return fail(TIG_ERR_UNSUPPORTED, "A and W must be 16-byte aligned with row strides a multiple of 8");
  if (!aligned(C, out_dtype == TIG_OUT_F32 ? 4 : 2))
    return fail(TIG_ERR_INVALID_ARG, "C is misaligned for its dtype");
  // The tallest tile bounds the span, whatever height this call runs on.
  const int bm = tig::block_m_for_log2(log2i(leaves));
  if ((s = check_span("A tile", bm, lda)) != TIG_OK) return s;
  if ((s = check_span("W tile", tig::kBlockN, ldw)) != TIG_OK) return s;
  if (tig::cdiv(M, bm) * tig::cdiv(N, tig::kBlockN) >= (int64_t(1) << 31) - 8)
    return fail(TIG_ERR_UNSUPPORTED, "too many output tiles");
  tig::TreeGemmLaunch p{A, lda, W, ldw, C, ldc,
                        out_dtype == TIG_OUT_F32 ? tig::kEpiF32 : tig::kEpiBF16,
                        M, N, K, log2i(leaves)};
  const hipError_t e = tig::launch_tree_gemm(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_logprob_workspace_bytes(int64_t M, int64_t K, int64_t n_vocab, int32_t leaves,
                                       size_t* bytes) {
  if (!bytes) return fail(TIG_ERR_INVALID_ARG, "bytes is NULL");
  if (M < 0) return fail(TIG_ERR_INVALID_ARG, "M must be >= 0");
  if (n_vocab < 1) return fail(TIG_ERR_INVALID_ARG, "n_vocab must be >= 1");
  tig_status s = check_k_leaves(K, leaves);
  if (s != TIG_OK) return s;
  if (tig::cdiv(n_vocab, tig::kBlockN) > tig::kMaxVocabTiles)
    return fail(TIG_ERR_UNSUPPORTED, "n_vocab > %d not implemented",
                tig::kMaxVocabTiles * tig::kBlockN);
  *bytes = tig::logprob_ws_bytes(M, n_vocab, leaves);
  return ok();
}

tig_status tig_logprob_gather(const void* H, const void* W, const int64_t* ids, float* logprob_out,
                              float* lse_out, int64_t M, int64_t K, int64_t n_vocab,
                              int32_t leaves, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  size_t need = 0;
  tig_status s = tig_logprob_workspace_bytes(M, K, n_vocab, leaves, &need);
  if (s != TIG_OK) return s;
  if (M == 0) return ok();
  if (!H || !W || !ids || !logprob_out)
    return fail(TIG_ERR_INVALID_ARG, "H, W, ids and logprob_out must not be NULL");
  if (!aligned(H, 16) || !aligned(W, 16) || K % 8)
    return fail(TIG_ERR_UNSUPPORTED, "H and W must be 16-byte aligned with K a multiple of 8");
  if (!aligned(ids, 8) || !aligned(logprob_out, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(TIG_ERR_INVALID_ARG, "ids, logprob_out or lse_out misaligned");
  if (!workspace || workspace_bytes < need)
    return fail(TIG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(TIG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  // The tallest tile bounds the span at every M, so that whether a row is
  // accepted never depends on the batch it arrives in.
  const int bm = tig::logprob_block_m_for(M, log2i(leaves));
  if ((s = check_span("H tile", tig::kLogprobMaxBlockM, K)) != TIG_OK) return s;
  if (tig::cdiv(M, bm) * tig::cdiv(n_vocab, tig::kBlockN) >= (int64_t(1) << 31) - 8)
    return fail(TIG_ERR_UNSUPPORTED, "too many output tiles");
  char* ws = static_cast<char*>(workspace);
  const size_t xoff = tig::logprob_partials_bytes(M, n_vocab);
  const size_t soff = xoff + tig::logprob_xleaf_bytes(M, leaves);
  tig::LogprobLaunch p{H, W, ids, logprob_out, lse_out, M, K, n_vocab, log2i(leaves), ws,
                       reinterpret_cast<float*>(ws + xoff),
                       tig::logprob_spill_bytes(M, leaves) ? reinterpret_cast<float*>(ws + soff) : nullptr};
  const hipError_t e = tig::launch_logprob(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static_assert(tig::kNoAllocScratchBytes == TIG_NOALLOC_SCRATCH_BYTES, "tig.h and the device array disagree");

tig_status tig_logprob_gather_noalloc(const void* H, const void* W, const int64_t* ids,
                                      float* logprob_out, float* lse_out, int64_t M, int64_t K,
                                      int64_t n_vocab, int32_t leaves, hipStream_t stream) {
  size_t need = 0;
  tig_status s = tig_logprob_workspace_bytes(M, K, n_vocab, leaves, &need);
  if (s != TIG_OK) return s;
  if (M == 0) return ok();
  if (need > tig::kNoAllocScratchBytes)
    return fail(TIG_ERR_UNSUPPORTED,
                "tig_logprob_gather_noalloc: %lld rows need %zu bytes of intermediate data, above its fixed "
                "%zu-byte device array; call tig_logprob_gather with a workspace",
                (long long)M, need, tig::kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = tig::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(TIG_ERR_HIP, "tig_logprob_gather_noalloc: device array lookup failed: %s", hipGetErrorString(e));
  return tig_logprob_gather(H, W, ids, logprob_out, lse_out, M, K, n_vocab, leaves, ws,
                            tig::kNoAllocScratchBytes, stream);
}

tig_status tig_moe_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t n_experts,
                                   int32_t topk, size_t* bytes) {
  if (!bytes) return fail(TIG_ERR_INVALID_ARG, "bytes is NULL");
  if (T < 0 || N < 0 || K <= 0) return fail(TIG_ERR_INVALID_ARG, "T, N >= 0 and K > 0 required");
  if (n_experts < 1 || topk < 1)
    return fail(TIG_ERR_INVALID_ARG, "n_experts and topk must be >= 1");
  if (topk > tig::kMaxTopk)
    return fail(TIG_ERR_UNSUPPORTED, "topk > %d not implemented", tig::kMaxTopk);
  if (n_experts > tig::kMaxExperts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts > %d not implemented", tig::kMaxExperts);
  if (int64_t(n_experts) * T * topk >= (int64_t(1) << 31))
    return fail(TIG_ERR_UNSUPPORTED, "n_experts * T * topk too large for 32-bit row lists");
  *bytes = tig::moe_ws_bytes(T, N, n_experts, topk);
  return ok();
}

tig_status tig_moe_route(const void* H, const void* Wr, float* logits, int32_t* topk_ids,
                         float* topk_w, int64_t T, int64_t K, int32_t n_experts, int32_t topk,
                         int32_t leaves, hipStream_t stream) {
  if (T < 0) return fail(TIG_ERR_INVALID_ARG, "T must be >= 0");
  if (n_experts < 1 || topk < 1 || topk > n_experts)
    return fail(TIG_ERR_INVALID_ARG, "need 1 <= topk <= n_experts");
  if (n_experts > tig::kMaxRouteExperts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts > %d not implemented", tig::kMaxRouteExperts);
  if (topk > tig::kMaxTopk) return fail(TIG_ERR_UNSUPPORTED, "topk > %d not implemented", tig::kMaxTopk);
  tig_status s = check_k_leaves(K, leaves);
  if (s != TIG_OK) return s;
  if (T == 0) return ok();
  if (!H || !Wr || !logits || !topk_ids || !topk_w)
    return fail(TIG_ERR_INVALID_ARG, "H, Wr, logits, topk_ids and topk_w must not be NULL");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(TIG_ERR_INVALID_ARG, "logits, topk_ids or topk_w misaligned");
  if (T * int64_t(n_experts) >= (int64_t(1) << 40))
    return fail(TIG_ERR_UNSUPPORTED, "T * n_experts too large");
  // Byte offsets inside the 64 router rows of a block are 32-bit.
  if (64 * K * 2 >= (int64_t(1) << 32)) return fail(TIG_ERR_UNSUPPORTED, "K (%lld) too large", (long long)K);
  // The logits: the leaf-tree contraction with FP32 output (the bits of tig_tree_gemm),
  // on 32-token blocks.
  int lg = 0;
  while ((1 << lg) < leaves) ++lg;
  hipError_t e = tig::launch_router_logits(H, Wr, logits, T, K, n_experts, lg, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  e = tig::launch_moe_route(logits, T, n_experts, topk, topk_ids, topk_w, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_expert_workspace_bytes(int64_t rows, int32_t n_experts, size_t* bytes) {
  if (!bytes) return fail(TIG_ERR_INVALID_ARG, "bytes is NULL");
  if (rows < 0) return fail(TIG_ERR_INVALID_ARG, "rows must be >= 0");
  if (n_experts < 1) return fail(TIG_ERR_INVALID_ARG, "n_experts must be >= 1");
  if (n_experts > tig::kMaxGroupExperts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts > %d not implemented", tig::kMaxGroupExperts);
  *bytes = tig::group_ws_bytes(rows, n_experts);
  return ok();
}

// Shared checks and launch of the two expert-GEMM layouts.
static tig_status expert_gemm(bool masked, const void* X, const int32_t* counts, const void* W, void* Y,
                              tig_out_dtype out_dtype, int32_t n_experts, int64_t rows, int64_t cap,
                              int64_t align, int64_t N, int64_t K, int32_t leaves, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  tig_status s = tig_expert_workspace_bytes(rows < 0 ? 0 : rows, n_experts, &need);
  if (s != TIG_OK) return s;
  if (rows < 0 || N < 0) return fail(TIG_ERR_INVALID_ARG, "row count and N must be >= 0");
  if ((s = check_k_leaves(K, leaves)) != TIG_OK) return s;
  if (out_dtype != TIG_OUT_F32 && out_dtype != TIG_OUT_BF16)
    return fail(TIG_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (rows >= (int64_t(1) << 31) - 256) return fail(TIG_ERR_UNSUPPORTED, "too many rows");
  if (rows == 0 || N == 0) return ok();
  if (!X || !counts || !W || !Y) return fail(TIG_ERR_INVALID_ARG, "X, counts, W and Y must not be NULL");
  if (!aligned(X, 16) || !aligned(W, 16) || K % 8)
    return fail(TIG_ERR_UNSUPPORTED, "X and W must be 16-byte aligned with K a multiple of 8");
  if (!aligned(counts, 4) || !aligned(Y, out_dtype == TIG_OUT_F32 ? 4 : 2))
    return fail(TIG_ERR_INVALID_ARG, "counts or Y misaligned");
  if ((s = check_span("X tile", 192, K)) != TIG_OK) return s;
  if ((s = check_span("W tile", tig::kBlockN, K)) != TIG_OK) return s;
  if (tig::group_max_items(rows, n_experts) * tig::cdiv(N, tig::kBlockN) >= (int64_t(1) << 31) - 8)
    return fail(TIG_ERR_UNSUPPORTED, "too many output tiles");
  if (!workspace || workspace_bytes < need)
    return fail(TIG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(TIG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  tig::GroupLaunch p{X, counts, W, Y, out_dtype == TIG_OUT_F32 ? tig::kEpiF32 : tig::kEpiBF16, masked, rows, cap,
                     align, N, K, n_experts, log2i(leaves), reinterpret_cast<int32_t*>(ws),
                     reinterpret_cast<int32_t*>(ws + 256)};
  const hipError_t e = tig::launch_group_gemm(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_expert_gemm_masked(const void* X, const int32_t* counts, const void* W, void* Y,
                                  tig_out_dtype out_dtype, int32_t n_experts, int64_t cap, int64_t N, int64_t K,
                                  int32_t leaves, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (cap < 0) return fail(TIG_ERR_INVALID_ARG, "cap must be >= 0");
  if (n_experts >= 1 && cap > ((int64_t(1) << 31) - 256) / n_experts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts * cap too large");
  return expert_gemm(true, X, counts, W, Y, out_dtype, n_experts, int64_t(n_experts < 0 ? 0 : n_experts) * cap,
                     cap, 1, N, K, leaves, workspace, workspace_bytes, stream);
}

tig_status tig_expert_gemm_contiguous(const void* X, const int32_t* counts, int64_t align, const void* W, void* Y,
                                      tig_out_dtype out_dtype, int32_t n_experts, int64_t M, int64_t N, int64_t K,
                                      int32_t leaves, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (align < 1 || align > (int64_t(1) << 20)) return fail(TIG_ERR_INVALID_ARG, "align must be in [1, 2^20]");
  return expert_gemm(false, X, counts, W, Y, out_dtype, n_experts, M, 0, align, N, K, leaves, workspace,
                     workspace_bytes, stream);
}

tig_status tig_silu_mul(const float* GU, int64_t ldgu, void* out, int64_t ldo, int64_t rows, int64_t I,
                        hipStream_t stream) {
  if (rows < 0 || I < 0) return fail(TIG_ERR_INVALID_ARG, "rows and I must be >= 0");
  if (ldgu < 2 * I || ldo < I) return fail(TIG_ERR_INVALID_ARG, "ldgu must be >= 2 I and ldo >= I");
  if (rows == 0 || I == 0) return ok();
  if (!GU || !out) return fail(TIG_ERR_INVALID_ARG, "GU and out must not be NULL");
  if (!aligned(GU, 4) || !aligned(out, 2)) return fail(TIG_ERR_INVALID_ARG, "GU or out misaligned");
  const hipError_t e = tig::launch_silu_mul(GU, ldgu, static_cast<uint16_t*>(out), ldo, rows, I, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_fp8_quantize(const void* X, int64_t ldx, uint8_t* Q, int64_t ldq, uint8_t* scales, int64_t R,
                            int64_t C, int32_t block_rows, hipStream_t stream) {
  if (R < 0 || C < 0) return fail(TIG_ERR_INVALID_ARG, "R and C must be >= 0");
  if (block_rows != 1 && block_rows != 128) return fail(TIG_ERR_INVALID_ARG, "block_rows must be 1 or 128");
  if (ldx < C || ldq < C) return fail(TIG_ERR_INVALID_ARG, "ldx and ldq must be >= C");
  if (R == 0 || C == 0) return ok();
  if (!X || !Q || !scales) return fail(TIG_ERR_INVALID_ARG, "X, Q and scales must not be NULL");
  if (!aligned(X, 2)) return fail(TIG_ERR_INVALID_ARG, "X misaligned");
  if (block_rows == 128 && tig::cdiv(R, 128) > 65535) return fail(TIG_ERR_UNSUPPORTED, "too many row blocks");
  const hipError_t e = tig::launch_fp8_quantize(static_cast<const uint16_t*>(X), ldx, Q, ldq, scales, R, C,
                                                block_rows, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_fp8_dequantize(const uint8_t* Q, const uint8_t* scales, void* out, int64_t R, int64_t C,
                              int32_t block_rows, hipStream_t stream) {
  if (R < 0 || C < 0) return fail(TIG_ERR_INVALID_ARG, "R and C must be >= 0");
  if (block_rows != 1 && block_rows != 128) return fail(TIG_ERR_INVALID_ARG, "block_rows must be 1 or 128");
  if (R == 0 || C == 0) return ok();
  if (!Q || !scales || !out) return fail(TIG_ERR_INVALID_ARG, "Q, scales and out must not be NULL");
  if (!aligned(out, 2)) return fail(TIG_ERR_INVALID_ARG, "out misaligned");
  const hipError_t e = tig::launch_fp8_dequant(Q, scales, R, C, block_rows, static_cast<uint16_t*>(out), stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(TIG_ERR_INVALID_ARG, "bytes is NULL");
  if (M < 0 || N < 0 || K < 0) return fail(TIG_ERR_INVALID_ARG, "M, N and K must be >= 0");
  *bytes = tig::fp8_ws_bytes(M, N, K);
  return ok();
}

tig_status tig_fp8_tree_gemm(const uint8_t* QA, const uint8_t* SA, const uint8_t* QW, const uint8_t* SW, void* C,
                             int64_t ldc, tig_out_dtype out_dtype, int64_t M, int64_t N, int64_t K, int32_t leaves,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || N < 0) return fail(TIG_ERR_INVALID_ARG, "M and N must be >= 0");
  tig_status s = check_k_leaves(K, leaves);
  if (s != TIG_OK) return s;
  if (K % (128 * int64_t(leaves)))
    return fail(TIG_ERR_UNSUPPORTED, "K/leaves must be a multiple of 128 (one scale block per k-tile)");
  if (out_dtype != TIG_OUT_F32 && out_dtype != TIG_OUT_BF16)
    return fail(TIG_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (ldc < N) return fail(TIG_ERR_INVALID_ARG, "ldc must be >= N");
  if (M == 0 || N == 0) return ok();
  if (!QA || !SA || !QW || !SW || !C) return fail(TIG_ERR_INVALID_ARG, "QA, SA, QW, SW and C must not be NULL");
  if (!aligned(QA, 16) || !aligned(QW, 16)) return fail(TIG_ERR_UNSUPPORTED, "QA and QW must be 16-byte aligned");
  if (!aligned(C, out_dtype == TIG_OUT_F32 ? 4 : 2)) return fail(TIG_ERR_INVALID_ARG, "C is misaligned");
  if ((s = check_span("A tile", 128, K / 2)) != TIG_OK) return s;
  if ((s = check_span("W tile", tig::kBlockN, K / 2)) != TIG_OK) return s;
  if (tig::cdiv(M, 128) * tig::cdiv(N, tig::kBlockN) >= (int64_t(1) << 31) - 8)
    return fail(TIG_ERR_UNSUPPORTED, "too many output tiles");
  if ((K / 128) * tig::fp8_table_width(M, N) >= (int64_t(1) << 32))
    return fail(TIG_ERR_UNSUPPORTED, "scale table too large");
  const size_t need = tig::fp8_ws_bytes(M, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(TIG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(TIG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  tig::Fp8GemmLaunch p{QA, SA, QW, SW, C, ldc, out_dtype == TIG_OUT_F32 ? tig::kEpiF32 : tig::kEpiBF16, M, N, K,
                       log2i(leaves), static_cast<uint8_t*>(workspace), tig::fp8_table_rows(M),
                       tig::fp8_table_width(M, N)};
  const hipError_t e = tig::launch_fp8_gemm(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_expert_fp8_workspace_bytes(int64_t rows, int32_t n_experts, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(TIG_ERR_INVALID_ARG, "bytes is NULL");
  if (rows < 0 || N < 0 || K < 0) return fail(TIG_ERR_INVALID_ARG, "rows, N and K must be >= 0");
  if (n_experts < 1) return fail(TIG_ERR_INVALID_ARG, "n_experts must be >= 1");
  if (n_experts > tig::kMaxGroupExperts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts > %d not implemented", tig::kMaxGroupExperts);
  *bytes = tig::fp8_group_ws(rows, n_experts, N, K).total;
  return ok();
}

static tig_status expert_fp8_gemm(bool masked, const uint8_t* QX, const uint8_t* SX, const int32_t* counts,
                                  const uint8_t* QW, const uint8_t* SW, void* Y, tig_out_dtype out_dtype,
                                  int32_t n_experts, int64_t rows, int64_t cap, int64_t align, int64_t N, int64_t K,
                                  int32_t leaves, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (rows < 0 || N < 0) return fail(TIG_ERR_INVALID_ARG, "row count and N must be >= 0");
  size_t need = 0;
  tig_status s = tig_expert_fp8_workspace_bytes(rows, n_experts, N, K, &need);
  if (s != TIG_OK) return s;
  if ((s = check_k_leaves(K, leaves)) != TIG_OK) return s;
  if (K % (128 * int64_t(leaves)))
    return fail(TIG_ERR_UNSUPPORTED, "K/leaves must be a multiple of 128 (one scale block per k-tile)");
  if (out_dtype != TIG_OUT_F32 && out_dtype != TIG_OUT_BF16)
    return fail(TIG_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (rows >= (int64_t(1) << 31) - 256) return fail(TIG_ERR_UNSUPPORTED, "too many rows");
  if (rows == 0 || N == 0) return ok();
  if (!QX || !SX || !counts || !QW || !SW || !Y)
    return fail(TIG_ERR_INVALID_ARG, "QX, SX, counts, QW, SW and Y must not be NULL");
  if (!aligned(QX, 16) || !aligned(QW, 16)) return fail(TIG_ERR_UNSUPPORTED, "QX and QW must be 16-byte aligned");
  if (!aligned(counts, 4) || !aligned(Y, out_dtype == TIG_OUT_F32 ? 4 : 2))
    return fail(TIG_ERR_INVALID_ARG, "counts or Y misaligned");
  if ((s = check_span("X tile", 128, K / 2)) != TIG_OK) return s;
  if ((s = check_span("W tile", tig::kBlockN, K / 2)) != TIG_OK) return s;
  if (tig::group_max_items(rows, n_experts) * tig::cdiv(N, tig::kBlockN) >= (int64_t(1) << 31) - 8)
    return fail(TIG_ERR_UNSUPPORTED, "too many output tiles");
  if ((K / 128) * tig::fp8_group_table_width(rows, n_experts, N) >= (int64_t(1) << 32))
    return fail(TIG_ERR_UNSUPPORTED, "scale table too large");
  if (!workspace || workspace_bytes < need)
    return fail(TIG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(TIG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const tig::Fp8GroupWs w = tig::fp8_group_ws(rows, n_experts, N, K);
  tig::Fp8GroupLaunch p{QX, SX, counts, QW, SW, Y, out_dtype == TIG_OUT_F32 ? tig::kEpiF32 : tig::kEpiBF16, masked,
                        rows, cap, align, N, K, n_experts, log2i(leaves), reinterpret_cast<int32_t*>(ws),
                        reinterpret_cast<int32_t*>(ws + w.items), reinterpret_cast<uint8_t*>(ws + w.table)};
  const hipError_t e = tig::launch_fp8_group_gemm(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_expert_fp8_gemm_masked(const uint8_t* QX, const uint8_t* SX, const int32_t* counts, const uint8_t* QW,
                                      const uint8_t* SW, void* Y, tig_out_dtype out_dtype, int32_t n_experts,
                                      int64_t cap, int64_t N, int64_t K, int32_t leaves, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (cap < 0) return fail(TIG_ERR_INVALID_ARG, "cap must be >= 0");
  if (n_experts >= 1 && cap > ((int64_t(1) << 31) - 256) / n_experts)
    return fail(TIG_ERR_UNSUPPORTED, "n_experts * cap too large");
  return expert_fp8_gemm(true, QX, SX, counts, QW, SW, Y, out_dtype, n_experts,
                         int64_t(n_experts < 0 ? 0 : n_experts) * cap, cap, 1, N, K, leaves, workspace,
                         workspace_bytes, stream);
}

tig_status tig_expert_fp8_gemm_contiguous(const uint8_t* QX, const uint8_t* SX, const int32_t* counts, int64_t align,
                                          const uint8_t* QW, const uint8_t* SW, void* Y, tig_out_dtype out_dtype,
                                          int32_t n_experts, int64_t M, int64_t N, int64_t K, int32_t leaves,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (align < 1 || align > (int64_t(1) << 20)) return fail(TIG_ERR_INVALID_ARG, "align must be in [1, 2^20]");
  return expert_fp8_gemm(false, QX, SX, counts, QW, SW, Y, out_dtype, n_experts, M, 0, align, N, K, leaves,
                         workspace, workspace_bytes, stream);
}

tig_status tig_silu_mul_fp8(const float* GU, int64_t ldgu, uint8_t* Q, int64_t ldq, uint8_t* scales, int64_t rows,
                            int64_t I, hipStream_t stream) {
  if (rows < 0 || I < 0) return fail(TIG_ERR_INVALID_ARG, "rows and I must be >= 0");
  if (ldgu < 2 * I || ldq < I) return fail(TIG_ERR_INVALID_ARG, "ldgu must be >= 2 I and ldq >= I");
  if (rows == 0 || I == 0) return ok();
  if (!GU || !Q || !scales) return fail(TIG_ERR_INVALID_ARG, "GU, Q and scales must not be NULL");
  if (I % 4 || ldgu % 4 || ldq % 4 || !aligned(GU, 16) || !aligned(Q, 4))
    return fail(TIG_ERR_UNSUPPORTED, "needs I, ldgu, ldq multiples of 4, GU 16-byte and Q 4-byte aligned");
  const hipError_t e = tig::launch_silu_mul_fp8(GU, ldgu, Q, ldq, scales, rows, I, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_topk_positions(const float* scores, int64_t ld, const int32_t* lengths, int64_t R,
                              int32_t k, int32_t* out, hipStream_t stream) {
  if (R < 0 || ld < 0) return fail(TIG_ERR_INVALID_ARG, "R and ld must be >= 0");
  if (k < 1) return fail(TIG_ERR_INVALID_ARG, "k must be >= 1");
  if (ld > tig::kTopkMaxLen)
    return fail(TIG_ERR_UNSUPPORTED, "rows longer than %lld not implemented", (long long)tig::kTopkMaxLen);
  if (R == 0) return ok();
  if (R > 0x7FFFFFFF) return fail(TIG_ERR_UNSUPPORTED, "R too large");
  if (!scores || !lengths || !out) return fail(TIG_ERR_INVALID_ARG, "scores, lengths and out must not be NULL");
  if (!aligned(scores, 4) || !aligned(lengths, 4) || !aligned(out, 4))
    return fail(TIG_ERR_INVALID_ARG, "scores, lengths or out misaligned");
  const hipError_t e = tig::launch_topk_positions(scores, ld, lengths, R, k, out, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

tig_status tig_moe_tree_gemm_combine(const void* H, const void* W_experts, int32_t n_experts,
                                     const int32_t* topk_ids, const float* topk_w, int32_t topk,
                                     float* out, int64_t T, int64_t N, int64_t K, int32_t leaves,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  size_t need = 0;
  tig_status s = tig_moe_workspace_bytes(T, N, K, n_experts, topk, &need);
  if (s != TIG_OK) return s;
  if ((s = check_k_leaves(K, leaves)) != TIG_OK) return s;
  if (T == 0 || N == 0) return ok();
  if (!H || !W_experts || !topk_ids || !topk_w || !out)
    return fail(TIG_ERR_INVALID_ARG, "H, W_experts, topk_ids, topk_w and out must not be NULL");
  if (!aligned(H, 16) || !aligned(W_experts, 16) || K % 8)
    return fail(TIG_ERR_UNSUPPORTED, "H and W_experts must be 16-byte aligned with K a multiple of 8");
  if (!aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(out, 4))
    return fail(TIG_ERR_INVALID_ARG, "topk_ids, topk_w or out misaligned");
  if (!workspace || workspace_bytes < need)
    return fail(TIG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(TIG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (T * K * 2 >= (int64_t(1) << 31))
    return fail(TIG_ERR_UNSUPPORTED, "H spans too many bytes for 32-bit offsets");
  if ((s = check_span("W tile", tig::kBlockN, K)) != TIG_OK) return s;
  if (T * topk >= (int64_t(1) << 30) || T >= 65536)
    return fail(TIG_ERR_UNSUPPORTED, "T or T*topk too large");
  char* ws = static_cast<char*>(workspace);
  const tig::MoeWorkspace w = tig::moe_ws_layout(T, N, n_experts, topk);
  tig::MoeLaunch p{H, W_experts, topk_ids, topk_w, out, T, N, K, n_experts, topk, log2i(leaves),
                   reinterpret_cast<int32_t*>(ws + w.hist), reinterpret_cast<int32_t*>(ws + w.first),
                   reinterpret_cast<int32_t*>(ws + w.counts), reinterpret_cast<int32_t*>(ws + w.prefix),
                   reinterpret_cast<int32_t*>(ws + w.n_items), reinterpret_cast<int32_t*>(ws + w.items),
                   reinterpret_cast<int32_t*>(ws + w.tok), reinterpret_cast<int32_t*>(ws + w.pos),
                   reinterpret_cast<float*>(ws + w.Y)};
  const hipError_t e = tig::launch_moe(p, stream);
  if (e != hipSuccess) return fail(TIG_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
