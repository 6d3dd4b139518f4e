"""The C ABI library loads and exports every entry point include/moe.h declares; host-side
argument checks (no GPU calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ("moe_init_pool", "moe_cache_resolve", "moe_layer_forward", "moe_stats"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import moe_expert_offload_amd as M
    for n in declared():
        assert hasattr(M.lib(), n), n
        assert n in M.EXPORTED


def _cfg(**kw):
    import moe_expert_offload_amd as M
    base = dict(n_layers=2, n_experts=16, top_k=2, hidden=256, inter=512, n_shared=0, cache_slots=8,
                max_tokens=1)
    base.update(kw)
    return M.make_config(**base)


def test_query_sizes_and_blob_size():
    import moe_expert_offload_amd as M
    b, a, w = M.query_sizes(_cfg())
    assert b == 3 * 256 * 512 * 17 // 32
    assert a == 8 * b and w > 0
    b, _, _ = M.query_sizes(_cfg(hidden=2880, inter=2880, n_experts=128, top_k=4, cache_slots=1862))
    assert b == 13_219_200


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=100), -1), (dict(inter=48), -1), (dict(top_k=17), -1), (dict(top_k=20, n_experts=16), -1),
    (dict(n_experts=2000), -1), (dict(n_shared=2), -1), (dict(max_tokens=0), -1),
    (dict(cache_slots=3), -4), (dict(max_tokens=4, cache_slots=15), -4), (dict(cache_slots=32769), -1),
    (dict(pinned_mb=-1), -1),
])
def test_config_rejected(kw, status):
    import moe_expert_offload_amd as M
    with pytest.raises(M.MoeError) as ei:
        M.query_sizes(_cfg(**kw))
    assert ei.value.status == status


def test_null_context_calls_fail_cleanly():
    import moe_expert_offload_amd as M
    L = M.lib()
    assert L.moe_layer_forward(None, 0, 0, None, 1, None, None, None) == M.MOE_EINVAL
    assert L.moe_stack_forward(None, 0, None, 0, 1, None, 0, None, None) == M.MOE_EINVAL
    assert L.moe_cache_resolve(None, 0, 0, None, 1, None, None) == M.MOE_EINVAL
    assert L.moe_stats(None, None, None, 0, None) == M.MOE_EINVAL
    out = ctypes.c_void_p(1)
    assert L.moe_init_pool(ctypes.byref(_cfg()), None, None, None, None, 0, None, 0, None, None,
                           ctypes.byref(out)) == M.MOE_EINVAL
    assert out.value is None
    L.moe_destroy(None)


def test_hbm_read_rejects_bad_ranges_before_any_launch():
    import moe_expert_offload_amd as M
    L = M.lib()
    assert L.moe_hbm_read(None, 16, None) == M.MOE_EINVAL
    # fake device addresses: rejected on alignment or size alone, never dereferenced
    assert L.moe_hbm_read(ctypes.c_void_p(0x1000), 0, None) == M.MOE_EINVAL
    assert L.moe_hbm_read(ctypes.c_void_p(0x1000), 24, None) == M.MOE_EINVAL
    assert L.moe_hbm_read(ctypes.c_void_p(0x1008), 16, None) == M.MOE_EINVAL


def test_lookahead_up_to_seven_layers_is_accepted():
    import moe_expert_offload_amd as M
    for la in range(8):
        M.query_sizes(_cfg(lookahead=la))
    for la in (-1, 8):
        with pytest.raises(M.MoeError) as e:
            M.query_sizes(_cfg(lookahead=la))
        assert e.value.status == M.MOE_EINVAL


def test_grouped_workspace_grows_with_max_tokens():
    """Batches of tokens need the grouped plan and the per-row expert outputs in the workspace."""
    import moe_expert_offload_amd as M
    _, _, w1 = M.query_sizes(_cfg(cache_slots=64))
    _, _, w16 = M.query_sizes(_cfg(max_tokens=16, cache_slots=64))
    _, _, w100 = M.query_sizes(_cfg(max_tokens=100, cache_slots=64))
    rows16 = 16 * 2
    assert w16 - w1 >= rows16 * 256 * 2   # bf16 expert outputs, one row per (token, expert)
    assert w100 > w16


# --- cache auto-sizing (host arithmetic only: free bytes are given, so no device query) ---

GPTOSS = dict(n_layers=36, n_experts=128, top_k=4, hidden=2880, inter=2880, n_shared=0, cache_slots=0,
              max_tokens=1)


def test_query_sizes_accepts_auto_cache_slots():
    import moe_expert_offload_amd as M
    b, a, w = M.query_sizes(_cfg(cache_slots=0))
    b8, a8, w8 = M.query_sizes(_cfg(cache_slots=8))
    assert (b, a, w) == (b8, 0, w8)  # the workspace does not depend on C


def test_auto_cache_slots_caps_at_the_pool_and_kernel_limit():
    import moe_expert_offload_amd as M
    assert M.auto_cache_slots(_cfg(cache_slots=0), free_bytes=1 << 40) == 2 * 16
    # gpt-oss-120b shape: the 60.9 GB pool fits in 288 GB of HBM whole
    assert M.auto_cache_slots(_cfg(**GPTOSS), free_bytes=288 * 10**9) == 36 * 128
    # Qwen3.8 shape: the 48 x 512 keys (92 GB) fit whole, under the 32768 slots the resolve kernels
    # address
    q38 = dict(n_layers=48, n_experts=512, top_k=10, hidden=3072, inter=768, n_shared=1, cache_slots=0,
               max_tokens=2048)
    assert M.auto_cache_slots(_cfg(**q38), free_bytes=288 * 10**9) == 48 * 512
    # 80 x 512 small experts: the kernel limit
    many = dict(q38, n_layers=80, hidden=256, inter=256)
    assert M.auto_cache_slots(_cfg(**many), free_bytes=288 * 10**9) == 32768


def test_auto_cache_slots_is_the_largest_that_fits():
    import moe_expert_offload_amd as M
    cfg = _cfg(**GPTOSS)
    blob = M.query_sizes(cfg)[0]
    router = 36 * 128 * 2880 * 2
    reserve = 3 * 10**9
    prev = 0
    for free in range(25 * 10**9, 40 * 10**9, 997_000_001):
        C = M.auto_cache_slots(cfg, free_bytes=free, reserve_bytes=reserve)
        assert C * blob + router + reserve <= free            # what it returns fits
        assert (C + 1) * blob + router + reserve > free - (8 << 20)  # one more would not (state < 8 MiB)
        assert C >= prev
        prev = C
    # the pages' card: 24.6 GB of a 32 GB RTX 5090 held 40.4 % of the 4608 experts (1862 slots);
    # with that arena budget plus the library's own bytes, the same count comes out
    C = M.auto_cache_slots(cfg, free_bytes=1862 * blob + router + (6 << 20))
    assert C == 1862


def test_auto_cache_slots_reports_capacity_shortfall():
    import moe_expert_offload_amd as M
    cfg = _cfg(**dict(GPTOSS, max_tokens=16))  # needs 2 * min(16 * 4, 128) = 128 slots
    blob = M.query_sizes(cfg)[0]
    with pytest.raises(M.MoeError) as ei:
        M.auto_cache_slots(cfg, free_bytes=100 * blob)
    assert ei.value.status == -4 and "fits" in str(ei.value)
    assert M.auto_cache_slots(cfg, free_bytes=140 * blob) >= 128
    with pytest.raises(M.MoeError) as ei:
        M.auto_cache_slots(cfg, free_bytes=1000)
    assert ei.value.status == -4


def test_noalloc_entry_rejects_bad_arguments_before_any_gpu_call():
    """moe_expert_forward_noalloc checks its arguments on the host first: null buffers, token counts
    outside [1, 16] and intermediate vectors larger than the static scratch array fail with
    MOE_EINVAL and a message, with no GPU call."""
    import ctypes
    import moe_expert_offload_amd as M
    lib = M.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails before a launch
    cfg = M.make_config(1, 16, 2, 256, 512, 0, 8, 16)

    def call(cfg, n_tok, arena=fake, x=fake):
        return lib.moe_expert_forward_noalloc(ctypes.byref(cfg), arena, None, x, n_tok, fake, fake, fake, None)

    assert call(cfg, 0) == M.MOE_EINVAL
    assert b"n_tokens" in lib.moe_last_error(None)
    assert call(cfg, M.NOALLOC_MAX_TOKENS + 1) == M.MOE_EINVAL
    assert call(cfg, 1, arena=None) == M.MOE_EINVAL
    assert call(cfg, 1, x=None) == M.MOE_EINVAL
    shared = M.make_config(1, 16, 2, 256, 512, 1, 8, 16)
    assert call(shared, 1) == M.MOE_EINVAL  # n_shared = 1 needs the shared blob
    # the largest shape the kernels take ((k + n_shared) * I/32 * 80 B of LDS <= 60 KiB) at 16
    # tokens fits the scratch array; one expert more is rejected as a shape
    assert 16 * 12 * 2048 * 2 <= M.NOALLOC_SCRATCH_BYTES  # k = 11 + shared, I = 2048: the largest shape
    over = M.make_config(1, 16, 12, 256, 2048, 1, 32, 16)
    assert call(over, 1) == M.MOE_EINVAL and b"shape" in lib.moe_last_error(None)
    zero_slots = M.make_config(1, 16, 2, 256, 512, 0, 0, 16)
    assert call(zero_slots, 1) == M.MOE_EINVAL
