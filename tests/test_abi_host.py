"""Host-side tests of the C ABI (no GPU): symbols, plan digest, error paths.

Every call here fails validation on the host before any launch, or takes the
M == 0 no-op path; nothing reaches a kernel.  Calls that pass fake (non-NULL)
device pointers run only when no GPU is visible, so that a validation bug can
never turn into a launch on a real device.
"""

import ctypes
import hashlib
import os
import re

import pytest

import invariant_gemm_token_amd as tig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tig.h")
FAKE = 0x10000  # aligned, never dereferenced


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


fake_ptrs = pytest.mark.skipif(not _no_gpu(), reason="fake pointers only where no GPU is visible")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tig_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert {"tig_tree_gemm", "tig_logprob_gather", "tig_moe_tree_gemm_combine",
            "tig_plan_describe"} <= set(names)
    lib = ctypes.CDLL(tig.lib_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tig.h but not exported"
    tig.load()


def test_status_strings():
    assert tig.tig_status_string(tig.TIG_OK) == "ok"
    assert tig.tig_status_string(tig.TIG_ERR_WORKSPACE) == "workspace too small"
    assert tig.tig_status_string(99) == "unknown status"


@pytest.mark.parametrize("K,leaves", [(512, 8), (4096, 8), (7168, 16), (2048, 8), (1024, 1), (1024, 16)])
def test_plan_digest_is_sha256_of_policy(K, leaves):
    p = tig.tig_plan_describe(K, leaves)
    assert p["leaves"] == leaves and p["leaf_len"] == K // leaves
    # the dense kernels' tile: 192 rows while log2(leaves) + 1 accumulators fit, else 128
    assert (p["block_m"], p["block_n"], p["block_k"]) == (192 if leaves <= 8 else 128, 128, 64)
    assert (p["mfma_m"], p["mfma_n"], p["mfma_k"]) == (32, 32, 16)
    assert p["digest"] == hashlib.sha256(p["policy"].encode()).hexdigest()
    assert f"K={K};leaves={leaves};" in p["policy"]


def test_plan_digest_separates_policies():
    d = {tig.tig_plan_describe(K, L)["digest"] for K, L in [(4096, 8), (4096, 4), (8192, 8), (512, 8)]}
    assert len(d) == 4


@pytest.mark.parametrize("K,leaves,status", [
    (4096, 3, tig.TIG_ERR_INVALID_ARG),     # not a power of two
    (4096, 0, tig.TIG_ERR_INVALID_ARG),
    (4096, 128, tig.TIG_ERR_INVALID_ARG),   # above 64
    (4096, 32, tig.TIG_ERR_UNSUPPORTED),    # valid, not implemented
    (0, 8, tig.TIG_ERR_INVALID_ARG),
    (4100, 4, tig.TIG_ERR_UNSUPPORTED),     # leaf length 1025 not a multiple of 64
    (1000, 8, tig.TIG_ERR_UNSUPPORTED),     # 1000 / 8 = 125
    (256, 8, tig.TIG_ERR_UNSUPPORTED),      # leaf of 32 columns
])
def test_plan_rejects(K, leaves, status):
    with pytest.raises(tig.TigError) as e:
        tig.tig_plan_describe(K, leaves)
    assert e.value.status == status
    assert tig.tig_last_error()


def test_workspace_queries():
    # per-row partials of every 128-column vocabulary tile, then the picked logit's leaf values
    b = tig.tig_logprob_workspace_bytes(8192, 4096, 151936, 8)
    assert b == 8192 * 1187 * 8 + 8192 * 8 * 4
    # 16 leaves on 192-row tiles also keep the left half of each tile's leaf tree in
    # scratch: one 192 x 128 FP32 tile for each of up to 256 workgroups
    assert tig.tig_logprob_workspace_bytes(8192, 4096, 151936, 16) == (
        8192 * 1187 * 8 + 8192 * 16 * 4 + 256 * 192 * 128 * 4)
    # 128 rows fit one 128-row tile: no scratch
    assert tig.tig_logprob_workspace_bytes(128, 7168, 129280, 16) == 128 * 1010 * 8 + 128 * 16 * 4
    assert tig.tig_logprob_workspace_bytes(0, 4096, 151936, 8) == 0
    assert tig.tig_logprob_workspace_bytes(3, 512, 1, 8) == 256 + 256
    m = tig.tig_moe_workspace_bytes(4096, 1408, 2048, 64, 8)
    assert m >= 4096 * 8 * 1408 * 4
    with pytest.raises(tig.TigError) as e:
        tig.tig_logprob_workspace_bytes(8, 4096, 0, 8)
    assert e.value.status == tig.TIG_ERR_INVALID_ARG
    with pytest.raises(tig.TigError) as e:
        tig.tig_logprob_workspace_bytes(8, 4096, 128 * 65536 + 1, 8)
    assert e.value.status == tig.TIG_ERR_UNSUPPORTED
    with pytest.raises(tig.TigError) as e:
        tig.tig_moe_workspace_bytes(8, 8, 64, 4, 17)
    assert e.value.status == tig.TIG_ERR_UNSUPPORTED


def _raw():
    return tig.load()


def test_zero_rows_is_a_noop_even_with_null_pointers():
    lib = _raw()
    assert lib.tig_tree_gemm(None, 4096, None, 4096, None, 4096, 0, 0, 4096, 4096, 8, None) == tig.TIG_OK
    assert lib.tig_tree_gemm(None, 4096, None, 4096, None, 0, 0, 5, 0, 4096, 8, None) == tig.TIG_OK
    assert lib.tig_logprob_gather(None, None, None, None, None, 0, 4096, 151936, 8, None, 0, None) == tig.TIG_OK
    assert lib.tig_moe_tree_gemm_combine(None, None, 64, None, None, 8, None, 0, 1408, 2048, 8,
                                         None, 0, None) == tig.TIG_OK
    assert lib.tig_moe_route(None, None, None, None, None, 0, 2048, 64, 8, 8, None) == tig.TIG_OK
    assert lib.tig_topk_positions(None, 65536, None, 0, 2048, None, None) == tig.TIG_OK


def test_noalloc_logprob_limits_checked_before_any_device_call():
    lib = _raw()
    # M == 0: no-op even with NULL pointers; the device array is not looked up
    assert lib.tig_logprob_gather_noalloc(None, None, None, None, None, 0, 4096, 151936, 8, None) == tig.TIG_OK
    # argument errors as tig_logprob_gather
    assert lib.tig_logprob_gather_noalloc(None, None, None, None, None, -1, 4096, 151936, 8, None) == \
        tig.TIG_ERR_INVALID_ARG
    assert lib.tig_logprob_gather_noalloc(None, None, None, None, None, 4, 4096, 151936, 3, None) == \
        tig.TIG_ERR_INVALID_ARG
    # above the fixed array: rejected with a message naming the limit
    need = tig.tig_logprob_workspace_bytes(4000, 4096, 151936, 8)
    assert need > 32 << 20
    assert lib.tig_logprob_gather_noalloc(None, None, None, None, None, 4000, 4096, 151936, 8, None) == \
        tig.TIG_ERR_UNSUPPORTED
    assert "device array" in tig.tig_last_error()
    assert tig.tig_logprob_workspace_bytes(3000, 4096, 151936, 8) <= 32 << 20


def test_route_arguments_rejected_before_any_launch():
    lib = _raw()
    # topk outside [1, n_experts]
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 8, 9, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 8, 0, 8, None) == tig.TIG_ERR_INVALID_ARG
    # limits of this implementation
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 1025, 8, 8, None) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 64, 17, 8, None) == tig.TIG_ERR_UNSUPPORTED
    # leaves that do not split K into 64-multiples; negative T; NULL outputs
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 64, 8, 16, None) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_moe_route(None, None, None, None, None, -1, 512, 64, 8, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_moe_route(None, None, None, None, None, 4, 512, 64, 8, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert "NULL" in tig.tig_last_error()


def test_topk_arguments_rejected_before_any_launch():
    lib = _raw()
    # k < 1; negative R or ld; rows longer than one workgroup holds; NULL pointers
    assert lib.tig_topk_positions(None, 1024, None, 4, 0, None, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_topk_positions(None, 1024, None, -1, 8, None, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_topk_positions(None, -1, None, 4, 8, None, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_topk_positions(None, 65537, None, 4, 8, None, None) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_topk_positions(None, 65536, None, 4, 2048, None, None) == tig.TIG_ERR_INVALID_ARG
    assert "NULL" in tig.tig_last_error()


def test_expert_gemm_arguments_rejected_before_any_launch():
    lib = _raw()
    ws = None
    # n_experts out of range; negative cap / align below 1; NULL pointers; too small a workspace
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 0, 4, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 1025, 4, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 4, -1, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    assert lib.tig_expert_gemm_contiguous(None, None, 0, None, None, 0, 4, 64, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 4, 16, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    assert "NULL" in tig.tig_last_error()
    # leaves that do not split K into 64-multiples; an unknown output dtype
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 4, 16, 128, 512, 16, ws, 0, None) == \
        tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_expert_gemm_masked(None, None, None, None, 7, 4, 16, 128, 512, 8, ws, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    # nothing to do: no rows, or no columns
    assert lib.tig_expert_gemm_masked(None, None, None, None, 0, 4, 0, 128, 512, 8, ws, 0, None) == tig.TIG_OK
    assert lib.tig_expert_gemm_contiguous(None, None, 128, None, None, 0, 4, 64, 0, 512, 8, ws, 0, None) == \
        tig.TIG_OK
    assert tig.tig_expert_workspace_bytes(1000, 64) == 256 + 72 * 16 + 128   # 72 items, 256-byte aligned
    with pytest.raises(tig.TigError):
        tig.tig_expert_workspace_bytes(10, 0)


def test_silu_mul_arguments_rejected():
    lib = _raw()
    assert lib.tig_silu_mul(None, 10, None, 8, 4, 8, None) == tig.TIG_ERR_INVALID_ARG      # ldgu < 2 I
    assert lib.tig_silu_mul(None, 16, None, 7, 4, 8, None) == tig.TIG_ERR_INVALID_ARG      # ldo < I
    assert lib.tig_silu_mul(None, 16, None, 8, 4, 8, None) == tig.TIG_ERR_INVALID_ARG      # NULL
    assert lib.tig_silu_mul(None, 16, None, 8, 0, 8, None) == tig.TIG_OK


def test_fp8_arguments_rejected():
    lib = _raw()
    assert lib.tig_fp8_quantize(None, 256, None, 256, None, 4, 256, 64, None) == tig.TIG_ERR_INVALID_ARG   # block
    assert lib.tig_fp8_quantize(None, 100, None, 256, None, 4, 256, 1, None) == tig.TIG_ERR_INVALID_ARG    # ldx < C
    assert lib.tig_fp8_quantize(None, 256, None, 256, None, 4, 256, 1, None) == tig.TIG_ERR_INVALID_ARG    # NULL
    assert lib.tig_fp8_quantize(None, 256, None, 256, None, 0, 256, 128, None) == tig.TIG_OK
    assert lib.tig_fp8_tree_gemm(None, None, None, None, None, 64, 0, 8, 64, 1024, 8, None, 0, None) == \
        tig.TIG_ERR_INVALID_ARG
    # K/leaves must hold whole 128-wide scale blocks
    assert lib.tig_fp8_tree_gemm(None, None, None, None, None, 64, 0, 8, 64, 512, 8, None, 0, None) == \
        tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_fp8_tree_gemm(None, None, None, None, None, 64, 0, 0, 64, 1024, 8, None, 0, None) == tig.TIG_OK
    # the scale table: K/128 rows of (M rounded up to 128) + ceil(N/128) bytes, rounded up to 4
    assert tig.tig_fp8_gemm_workspace_bytes(10, 20, 512) == 768          # 4 * 132 = 528 -> 768
    assert lib.tig_fp8_dequantize(None, None, None, 4, 128, 2, None) == tig.TIG_ERR_INVALID_ARG


def test_expert_fp8_and_silu_fp8_arguments_rejected():
    lib = _raw()
    n = None
    # K/leaves not a whole number of 128-wide scale blocks; NULL pointers; nothing to do
    assert lib.tig_expert_fp8_gemm_masked(n, n, n, n, n, n, 0, 4, 16, 128, 512, 8, n, 0, n) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_expert_fp8_gemm_masked(n, n, n, n, n, n, 0, 4, 16, 128, 1024, 8, n, 0, n) == \
        tig.TIG_ERR_INVALID_ARG
    assert lib.tig_expert_fp8_gemm_masked(n, n, n, n, n, n, 0, 4, 0, 128, 1024, 8, n, 0, n) == tig.TIG_OK
    assert lib.tig_expert_fp8_gemm_contiguous(n, n, n, 0, n, n, n, 0, 4, 64, 128, 1024, 8, n, 0, n) == \
        tig.TIG_ERR_INVALID_ARG                                                           # align 0
    assert lib.tig_expert_fp8_gemm_masked(n, n, n, n, n, n, 0, 1025, 4, 128, 1024, 8, n, 0, n) == \
        tig.TIG_ERR_UNSUPPORTED
    # 1000 rows, 4 experts, N = 300, K = 1024: 12 items -> 256 + 256 + 8 rows of 1548 bytes (-> 12544)
    assert tig.tig_expert_fp8_workspace_bytes(1000, 4, 300, 1024) == 256 + 256 + 12544
    assert lib.tig_silu_mul_fp8(n, 16, n, 8, n, 4, 8, n) == tig.TIG_ERR_INVALID_ARG        # NULL
    assert lib.tig_silu_mul_fp8(n, 12, n, 6, n, 4, 6, n) == tig.TIG_ERR_INVALID_ARG        # NULL before the
    assert lib.tig_silu_mul_fp8(n, 16, n, 8, n, 0, 8, n) == tig.TIG_OK


def test_null_pointers_rejected():
    lib = _raw()
    assert lib.tig_tree_gemm(None, 512, None, 512, None, 64, 0, 4, 64, 512, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_logprob_gather(None, None, None, None, None, 4, 512, 64, 8, None, 0, None) == tig.TIG_ERR_INVALID_ARG
    assert "NULL" in tig.tig_last_error()


def test_negative_sizes_and_bad_strides_rejected():
    lib = _raw()
    assert lib.tig_tree_gemm(None, 512, None, 512, None, 64, 0, -1, 64, 512, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_tree_gemm(None, 256, None, 512, None, 64, 0, 4, 64, 512, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_tree_gemm(None, 512, None, 512, None, 32, 0, 4, 64, 512, 8, None) == tig.TIG_ERR_INVALID_ARG
    assert lib.tig_tree_gemm(None, 512, None, 512, None, 64, 7, 4, 64, 512, 8, None) == tig.TIG_ERR_INVALID_ARG


@fake_ptrs
def test_alignment_and_workspace_errors_with_fake_pointers():
    lib = _raw()
    F = FAKE
    # misaligned A, odd row stride
    assert lib.tig_tree_gemm(F + 2, 512, F, 512, F, 64, 0, 4, 64, 512, 8, None) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_tree_gemm(F, 516, F, 512, F, 64, 0, 4, 64, 512, 8, None) == tig.TIG_ERR_UNSUPPORTED
    # 192 rows of A spanning 2 GiB: rejected at every M, whatever tile height the call would run on
    big = (1 << 31) // (192 * 2) // 8 * 8 + 8
    for M in (1, 100, 5000):
        assert lib.tig_tree_gemm(F, big, F, 512, F, 64, 0, M, 64, 512, 8, None) == tig.TIG_ERR_UNSUPPORTED
    assert lib.tig_tree_gemm(F, 512, F, (1 << 31) // 256 // 8 * 8 + 8, F, 64, 0, 4, 64, 512, 8,
                             None) == tig.TIG_ERR_UNSUPPORTED
    # logprob: 192 rows of H spanning 2 GiB are rejected at every M, including the
    # batch sizes that would run on 128-row tiles (K = 5592576 = 10923 x 512)
    Kbig = 10923 * 512
    assert 128 * Kbig * 2 < (1 << 31) <= 192 * Kbig * 2
    for M in (1, 128, 300):
        wsb = tig.tig_logprob_workspace_bytes(M, Kbig, 64, 8)
        assert lib.tig_logprob_gather(F, F, F, F, None, M, Kbig, 64, 8, F, wsb, None) == tig.TIG_ERR_UNSUPPORTED
        assert "spans" in tig.tig_last_error()
    # workspace missing / too small / misaligned
    need = tig.tig_logprob_workspace_bytes(4, 512, 64, 8)
    assert lib.tig_logprob_gather(F, F, F, F, None, 4, 512, 64, 8, None, 0, None) == tig.TIG_ERR_WORKSPACE
    assert lib.tig_logprob_gather(F, F, F, F, None, 4, 512, 64, 8, F, need - 1, None) == tig.TIG_ERR_WORKSPACE
    assert lib.tig_logprob_gather(F, F, F, F, None, 4, 512, 64, 8, F + 16, need, None) == tig.TIG_ERR_INVALID_ARG
    needm = tig.tig_moe_workspace_bytes(16, 128, 512, 4, 2)
    assert lib.tig_moe_tree_gemm_combine(F, F, 4, F, F, 2, F, 16, 128, 512, 8, F, needm - 1,
                                         None) == tig.TIG_ERR_WORKSPACE
    assert lib.tig_moe_tree_gemm_combine(F, F, 4, F, F, 2, F, 16, 128, 512, 3, F, needm,
                                         None) == tig.TIG_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros((4, 512), dtype=torch.bfloat16)
    W = torch.zeros((64, 512), dtype=torch.bfloat16)
    C = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        tig.tig_tree_gemm(A, W, C, 8)
    with pytest.raises((TypeError, ValueError)):
        tig.tig_tree_gemm(A.float(), W, C, 8)
