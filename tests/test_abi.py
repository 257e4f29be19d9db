"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/dms.h declares, and rejects bad arguments on the host before any HIP
call is made (no GPU needed)."""

import ctypes
import os
import re

import pytest

from decode_attention_learned_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dms.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dms_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libdms.so is not built: run __graft_entry__.build()")
    return lib.load()


def test_every_declared_symbol_is_exported(L):
    declared = _declared()
    assert declared == sorted(lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_test_build_exports_the_same_symbols(L):
    """libdms_generic.so (the test build) is the same ABI."""
    with lib.variant("generic"):
        G = lib.load()
        assert G is not L
        for name in _declared():
            assert hasattr(G, name), name
        assert lib.version() == 5


def test_version_and_strerror(L):
    assert lib.version() == 5
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.strerror(code), str)


def _shape(**kw):
    base = dict(batch=2, kv_heads=2, group=2, head_dim=64, page_size=64, window=16,
                max_pages_per_unit=8, num_pages=32, kv_dtype=lib.DMS_KV_F32)
    base.update(kw)
    return lib.DmsShape(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, lib.DMS_OK),
    ({"kv_dtype": lib.DMS_KV_BF16, "head_dim": 128, "group": 16}, lib.DMS_OK),
    ({"batch": 0}, lib.DMS_EINVAL),
    ({"window": 0}, lib.DMS_EINVAL),
    ({"num_pages": 0}, lib.DMS_EINVAL),
    ({"head_dim": 96}, lib.DMS_EUNSUPPORTED),
    ({"page_size": 32}, lib.DMS_EUNSUPPORTED),
    ({"group": 17}, lib.DMS_EUNSUPPORTED),
    ({"kv_dtype": 5}, lib.DMS_EUNSUPPORTED),
])
def test_check_shape(L, kw, code):
    assert lib.check_shape(_shape(**kw)) == code


def test_workspace_bytes(L):
    # header, first chunk per unit (+1), owning unit per chunk (at most 3 * 512
    # chunks up to 1536 units, else one per unit), merge count and last
    # compaction position per unit
    assert lib.plan_words(_shape()) == 16 + (4 + 1) + 1536 + 4 + 4
    assert lib.plan_words(_shape(batch=100, kv_heads=8)) == 16 + 801 + 1536 + 800 + 800
    assert lib.plan_words(_shape(batch=256, kv_heads=8)) == 16 + 2049 + 2048 + 2048 + 2048
    assert lib.plan_words(_shape(window=0)) == 0
    assert lib.decode_workspace_bytes(_shape()) > 0
    assert lib.decode_workspace_bytes(_shape(window=0)) == 0
    big = lib.decode_workspace_bytes(_shape(batch=64, kv_heads=8, group=4, head_dim=128))
    # partial outputs of (3 * 512 chunks, or one per unit past 512 units) x G x D floats dominate
    assert big >= 1536 * 4 * 128 * 4
    more = lib.decode_workspace_bytes(_shape(batch=256, kv_heads=8, group=4, head_dim=128))
    assert more >= 2048 * 4 * 128 * 4 > big


def test_chunk_split_workspace_bytes(L):
    """Workspace that lets a long bf16 chunk split its tiles: 512 queries of one
    sequence with 32/8 heads make 16 x 8 = 128 tiled workgroups, at most half
    a round of 768, so 4 splits of 512 x 32 rows of (m, l) and 128 floats."""
    one = _shape(batch=1, kv_heads=8, group=4, head_dim=128, kv_dtype=lib.DMS_KV_BF16)
    rows = 512 * 32
    want = -(-4 * rows * 8 // 256) * 256 + -(-4 * rows * 128 * 4 // 256) * 256
    assert lib.decode_multi_split_workspace_bytes(one, 512) == max(lib.decode_multi_workspace_bytes(one), want)
    # 3 splits from 193 to 256 workgroups (768 // 256 = 3)
    b3 = _shape(batch=4, kv_heads=4, group=4, head_dim=64, kv_dtype=lib.DMS_KV_BF16)   # 16 x 16 = 256
    r3 = 4 * 512 * 16
    want3 = -(-3 * r3 * 8 // 256) * 256 + -(-3 * r3 * 64 * 4 // 256) * 256
    assert lib.decode_multi_split_workspace_bytes(b3, 512) == max(lib.decode_multi_workspace_bytes(b3), want3)
    # no split: more than half a round (4 sequences: 512 workgroups), short
    # chunks (the decode kernel serves them), float32 caches
    sb = _shape(batch=4, kv_heads=8, group=4, head_dim=128, kv_dtype=lib.DMS_KV_BF16)
    base = lib.decode_multi_workspace_bytes(sb)
    assert lib.decode_multi_split_workspace_bytes(sb, 512) == base
    assert lib.decode_multi_split_workspace_bytes(one, 31) == lib.decode_multi_workspace_bytes(one)
    assert lib.decode_multi_split_workspace_bytes(_shape(kv_dtype=lib.DMS_KV_F32), 512) \
        == lib.decode_multi_workspace_bytes(_shape(kv_dtype=lib.DMS_KV_F32))
    assert lib.decode_multi_split_workspace_bytes(one, 0) == 0
    assert lib.decode_multi_split_workspace_bytes(_shape(window=0), 64) == 0


def test_host_side_errors_need_no_gpu(L):
    s = _shape()
    null_cache = lib.DmsCacheStruct()
    fake = ctypes.c_void_p(0x1000)
    full = lib.DmsCacheStruct(*([0x1000] * 14))
    assert L.dms_reset(None, None, None) == lib.DMS_EINVAL
    assert L.dms_reset(ctypes.byref(s), ctypes.byref(null_cache), None) == lib.DMS_EINVAL
    assert L.dms_append(ctypes.byref(s), ctypes.byref(full), fake, fake, fake, -1, None) == lib.DMS_EINVAL
    # n_new = 0 is a no-op that touches nothing
    assert L.dms_append(ctypes.byref(s), ctypes.byref(full), None, None, None, 0, None) == lib.DMS_OK
    assert L.dms_append(ctypes.byref(s), ctypes.byref(full), None, fake, fake, 4, None) == lib.DMS_EINVAL
    assert L.dms_decode_attn(ctypes.byref(s), ctypes.byref(full), fake, fake, 0.125, fake, 0, None) \
        == lib.DMS_EWORKSPACE
    assert L.dms_decode_attn(ctypes.byref(s), ctypes.byref(full), fake, fake, -1.0, fake, 1 << 30, None) \
        == lib.DMS_EINVAL
    assert L.dms_decode_attn(ctypes.byref(s), ctypes.byref(full), None, fake, 0.125, fake, 1 << 30, None) \
        == lib.DMS_EINVAL
    misaligned = ctypes.c_void_p(0x1008)
    assert L.dms_decode_attn(ctypes.byref(s), ctypes.byref(full), misaligned, fake, 0.125, fake,
                             1 << 30, None) == lib.DMS_EINVAL
    no_ref = lib.DmsCacheStruct(*([0x1000] * 13), None)
    assert L.dms_share_prefix(ctypes.byref(s), ctypes.byref(no_ref), 0, 1, 1, None) == lib.DMS_EINVAL
    assert L.dms_release(ctypes.byref(s), ctypes.byref(no_ref), 0, 1, None) == lib.DMS_EINVAL
    assert L.dms_share_prefix(ctypes.byref(s), ctypes.byref(full), 0, 0, 2, None) == lib.DMS_EINVAL  # src in range
    assert L.dms_share_prefix(ctypes.byref(s), ctypes.byref(full), 0, 1, 2, None) == lib.DMS_EINVAL  # past B
    assert L.dms_share_prefix(ctypes.byref(s), ctypes.byref(full), 2, 0, 1, None) == lib.DMS_EINVAL  # src past B
    assert L.dms_share_prefix(ctypes.byref(s), ctypes.byref(full), 1, 0, 0, None) == lib.DMS_EINVAL  # no receiver
    assert L.dms_release(ctypes.byref(s), ctypes.byref(full), 1, 2, None) == lib.DMS_EINVAL
    assert L.dms_release(ctypes.byref(s), ctypes.byref(full), 0, 0, None) == lib.DMS_OK
    # the decode step with the token in the decode launch
    assert L.dms_append_reserve(None, ctypes.byref(full), None) == lib.DMS_EINVAL
    assert L.dms_append_reserve(ctypes.byref(s), ctypes.byref(null_cache), None) == lib.DMS_EINVAL
    F = L.dms_decode_attn_fill
    args = [fake, fake, fake, fake, fake, 0.125, fake, 1 << 30, None]
    for i in (0, 1, 2, 3, 4, 6):  # k_new, v_new, logit, q, out, workspace
        bad_args = list(args)
        bad_args[i] = None
        assert F(ctypes.byref(s), ctypes.byref(full), *bad_args) == lib.DMS_EINVAL, i
    for i in (0, 1, 3, 4, 6):  # 16-byte alignment of k_new, v_new, q, out, workspace
        bad_args = list(args)
        bad_args[i] = misaligned
        assert F(ctypes.byref(s), ctypes.byref(full), *bad_args) == lib.DMS_EINVAL, i
    assert F(ctypes.byref(s), ctypes.byref(full), *args[:5], 0.0, *args[6:]) == lib.DMS_EINVAL
    assert F(ctypes.byref(s), ctypes.byref(full), *args[:7], 10, None) == lib.DMS_EWORKSPACE
    M = L.dms_decode_attn_multi
    sb = _shape(kv_dtype=lib.DMS_KV_BF16)
    assert M(ctypes.byref(sb), ctypes.byref(full), fake, 0, fake, 0.125, fake, 1 << 30, None) == lib.DMS_EINVAL
    assert M(ctypes.byref(sb), ctypes.byref(full), fake, 4, fake, 0.125, fake, 10, None) == lib.DMS_EWORKSPACE
    assert M(ctypes.byref(sb), ctypes.byref(full), fake, 4, fake, 0.0, fake, 1 << 30, None) == lib.DMS_EINVAL
    # float32 caches are served (by the float32 kernels); a short workspace is refused on the host
    assert M(ctypes.byref(_shape(kv_dtype=lib.DMS_KV_F32)), ctypes.byref(full), fake, 4, fake, 0.125, fake,
             10, None) == lib.DMS_EWORKSPACE
    # partials for 16 columns, whatever the group
    assert lib.decode_multi_workspace_bytes(sb) >= lib.decode_workspace_bytes(sb)
    bad = _shape(head_dim=80)
    assert L.dms_compact(ctypes.byref(bad), ctypes.byref(full), None) == lib.DMS_EUNSUPPORTED
    # export: count_out required, max_per_unit >= 0, all_slots 0 or 1
    E = L.dms_export_retained
    assert E(ctypes.byref(s), ctypes.byref(full), 0, 4, None, fake, None, None, None, None) == lib.DMS_EINVAL
    assert E(ctypes.byref(s), ctypes.byref(full), 0, -1, fake, fake, None, None, None, None) == lib.DMS_EINVAL
    assert E(ctypes.byref(s), ctypes.byref(full), 2, 4, fake, fake, None, None, None, None) == lib.DMS_EINVAL
    assert E(ctypes.byref(s), ctypes.byref(null_cache), 0, 4, fake, fake, None, None, None, None) \
        == lib.DMS_EINVAL
    assert E(ctypes.byref(bad), ctypes.byref(full), 0, 4, fake, fake, None, None, None, None) \
        == lib.DMS_EUNSUPPORTED


def test_prefill_host_errors(L):
    fake = ctypes.c_void_p(0x1000)
    f32 = _shape()
    bf = _shape(kv_dtype=lib.DMS_KV_BF16, head_dim=128)
    big = 1 << 40
    # float32 inputs are served (their own kernel, no workspace used, 256 bytes asked
    # for); a head dimension other than 64 or 128 is not
    f32_d96 = _shape(head_dim=96)
    assert L.dms_prefill_attn(ctypes.byref(f32_d96), fake, fake, fake, fake, 16, 0.1, fake, fake, big,
                              None) == lib.DMS_EUNSUPPORTED
    assert L.dms_prefill_attn(ctypes.byref(f32), fake, fake, fake, fake, 16, 0.1, fake, fake, 10, None) \
        == lib.DMS_EWORKSPACE
    assert L.dms_prefill_attn(ctypes.byref(f32), None, fake, fake, fake, 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EINVAL
    assert L.dms_prefill_attn(ctypes.byref(bf), fake, fake, fake, fake, -2, 0.1, fake, fake, big, None) \
        == lib.DMS_EINVAL
    assert L.dms_prefill_attn(ctypes.byref(bf), None, None, None, None, 0, 0.1, None, None, 0, None) \
        == lib.DMS_OK
    assert L.dms_prefill_attn(ctypes.byref(bf), None, fake, fake, fake, 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EINVAL
    assert L.dms_prefill_attn(ctypes.byref(bf), fake, fake, fake, fake, 16, 0.1, fake, fake, 10, None) \
        == lib.DMS_EWORKSPACE
    # 2 sequences x 2 KV heads x ceil(100/32) tiles x 16 KB, plus 32 floats per tile,
    # plus the far-tile copy (16 KB per tile)
    assert lib.prefill_workspace_bytes(bf, 100) == 2 * (2 * 2 * 4 * 16384) + 2 * 2 * 4 * 32 * 4
    assert lib.prefill_workspace_bytes(f32, 100) == 256
    assert lib.prefill_workspace_bytes(_shape(group=40), 100) == 256    # any group for float32
    assert lib.prefill_workspace_bytes(_shape(kv_dtype=lib.DMS_KV_BF16, group=17), 100) == 0
    # gathered: dense part, gathered copy of it, kept positions (S per unit),
    # counts (ntiles + 1 per unit) and kept bits (ntiles per unit), each 256-aligned
    dense = 2 * 2 * 4 * 16384 + 2 * 2 * 4 * 32 * 4
    assert lib.prefill_gathered_workspace_bytes(bf, 100) == 2 * dense + 1792 + 256 + 256
    R = L.dms_prefill_attn_relaxed
    assert R(ctypes.byref(bf), fake, fake, fake, fake, None, 0.0, 16, 0.1, fake, fake, big, None) == lib.DMS_EINVAL
    assert R(ctypes.byref(bf), fake, fake, fake, fake, None, float("inf"), 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EINVAL
    assert R(ctypes.byref(bf), fake, fake, fake, fake, None, 1.0, 16, 0.1, fake, fake, 10, None) \
        == lib.DMS_EWORKSPACE
    assert R(ctypes.byref(f32_d96), fake, fake, fake, fake, None, 1.0, 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EUNSUPPORTED
    assert R(ctypes.byref(f32), fake, fake, fake, fake, None, 0.0, 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EINVAL
    G = L.dms_prefill_attn_gathered
    assert G(ctypes.byref(f32_d96), fake, fake, fake, fake, 16, 0.1, fake, fake, big, None) \
        == lib.DMS_EUNSUPPORTED
    assert G(ctypes.byref(f32), fake, fake, fake, fake, 16, 0.1, fake, fake, 10, None) == lib.DMS_EWORKSPACE
    assert G(ctypes.byref(bf), fake, fake, fake, fake, -2, 0.1, fake, fake, big, None) == lib.DMS_EINVAL
    assert G(ctypes.byref(bf), None, None, None, None, 0, 0.1, None, None, 0, None) == lib.DMS_OK
    assert G(ctypes.byref(bf), None, fake, fake, fake, 16, 0.1, fake, fake, big, None) == lib.DMS_EINVAL
    assert G(ctypes.byref(bf), fake, fake, fake, fake, 16, -1.0, fake, fake, big, None) == lib.DMS_EINVAL
    assert G(ctypes.byref(bf), fake, fake, fake, fake, 16, 0.1, fake, fake, 10, None) == lib.DMS_EWORKSPACE
    assert lib.prefill_gathered_workspace_bytes(f32, 100) == 256
    # head_dim 64 is built (tiles of 8 KB), other dims are not
    d64 = _shape(kv_dtype=lib.DMS_KV_BF16, head_dim=64)
    d128 = _shape(kv_dtype=lib.DMS_KV_BF16, head_dim=128)
    assert 0 < lib.prefill_workspace_bytes(d64, 1000) < lib.prefill_workspace_bytes(d128, 1000)
    assert 0 < lib.prefill_gathered_workspace_bytes(d64, 1000) < lib.prefill_gathered_workspace_bytes(d128, 1000)


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "decode_attention_learned_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f
