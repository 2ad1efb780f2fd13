"""Host-side checks of libgqa's C ABI: it loads, exports every symbol the
header declares, plans shapes, and rejects bad arguments before touching a
GPU.  No kernel is launched.  CPU only."""
import ctypes
import os
import re

import pytest

import grouped_query_attention_decode_amd as gqa
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "gqa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gqa.library_path()):
        from grouped_query_attention_decode_amd import build
        build.build()
    return gqa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(gqa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version(lib):
    assert "gfx950" in gqa.version()
    assert lib.gqa_last_error() is not None


def _shape(**kw):
    base = dict(B=2, H=32, G=8, sq=1, T=4096, D=128, q_dtype=gqa.GQA_BF16,
                kv_dtype=gqa.GQA_BF16, out_dtype=gqa.GQA_F32)
    base.update(kw)
    return gqa.Shape(**base)


def _round256(x):
    return (x + 255) // 256 * 256


def test_plan_of_batched_gqa8(lib):
    p = gqa.plan(_shape(B=32))
    assert p["path"] == gqa.PATH_MFMA
    assert p["rows_per_group"] == 4
    # the matrix-core path works on 16-row query blocks (4 rows live)
    assert p["row_blocks"] == 1 and p["row_block"] == 16
    P = p["workgroups"]
    assert 1 <= P <= 4096
    # a fixed 1 MiB counter region, then two partial slots per workgroup, a
    # slot holding the 4 live query rows x 128 values + 16 lse floats -- far
    # below a repeated K/V copy (n_rep = 4 times the cache)
    assert p["workspace_bytes"] == (1 << 20) + _round256(P * 2 * (4 * 128 + 16) * 4)
    kv_bytes = 2 * 32 * 8 * 4096 * 128 * 2
    assert p["workspace_bytes"] < kv_bytes // 20
    assert gqa.workspace_bytes(_shape(B=32)) == p["workspace_bytes"]
    q = gqa.plan(_shape(B=32), path=gqa.PATH_MFMA_QK)
    assert q["path"] == gqa.PATH_MFMA_QK and q["row_block"] == 4
    assert q["workspace_bytes"] == (1 << 20) + _round256(q["workgroups"] * 2 * (4 * 128 + 16) * 4)


def test_plan_grid_per_compute_unit(lib):
    """One persistent workgroup grid per plan, sized per compute unit (256
    on MI355X, and the planner's count when no device is visible): two
    one-wave workgroups per CU when a wave carries one 16-row block of a bf16
    cache, four for an fp8 cache; one workgroup per CU for more than 16 rows
    per KV head (the 32 x 32 kernel: four or eight waves); a one-block bf16
    cache of at most 128 MB: workgroups of 4 waves (D = 64 or up to 32 MB) or
    2 that split each piece's rows, one per 128 KB of K/V between half the
    CUs and all of them; small caches otherwise: at least 256 cache rows per
    one-block wave, and at most 32 pieces per segment."""
    cu = 256
    hl = gqa.plan(_shape(B=32))                                                # batched GQA-8, 338 MB
    assert hl["workgroups"] == 2 * cu and hl["waves_per_group"] == 1
    assert gqa.plan(_shape(B=16, G=32, sq=2, T=16384))["workgroups"] == 2 * cu  # MHA, 2 rows
    assert gqa.plan(_shape(B=64, G=1, T=8192))["workgroups"] == cu             # MQA, 32 rows: 4 splits
    fp8 = _shape(B=32, kv_dtype=gqa.GQA_FP8_E4M3)
    assert gqa.plan(fp8)["workgroups"] == 4 * cu
    assert gqa.plan(_shape(B=16, G=1, sq=2, T=16384))["workgroups"] == cu      # 64 rows: 4-wave groups
    assert gqa.plan(_shape(B=8, G=8, sq=64))["workgroups"] == cu               # 256 rows: 8-wave groups
    # one-block bf16 caches up to 128 MB: row-split workgroups
    def rs(**kw):
        p = gqa.plan(_shape(**kw))
        return p["workgroups"], p["waves_per_group"], p["combine"]
    assert rs(B=1, G=8, D=64) == (cu // 2, 4, 0)              # Exaone layer, 8 MB
    assert rs(B=2, G=8, D=64) == (cu // 2, 4, 0)              # 16 MB
    assert rs(B=4, G=8, D=64) == (cu, 4, 0)                   # 32 MB
    assert rs(B=16, G=8, D=64) == (cu, 4, 0)                  # 128 MB
    assert rs(B=1, G=8, D=128) == (cu // 2, 4, 0)             # 16 MB
    assert rs(B=4, G=8, D=128) == (cu, 2, 0)                  # 64 MB: two waves
    assert rs(B=8, G=8, D=128) == (cu, 2, 0)                  # 128 MB
    assert rs(B=9, G=8, D=128)[1] == 1                        # above 128 MB: one-wave groups
    assert rs(B=1, G=8, D=64, T=64)[0] == 8 * 64 // (32 * 4)  # at least a tile per wave
    # a one-wave grid on small caches otherwise: at least 256 cache rows per
    # one-block wave, then at most 32 pieces per segment (forced here)
    import os
    os.environ["GQA_RSPLIT"] = "0"
    try:
        ex = gqa.plan(_shape(B=1, G=8, D=64))                                   # 8 x 4096 rows
        assert ex["workgroups"] == 8 * 4096 // 256 and ex["combine"] == 0 and ex["waves_per_group"] == 1
        assert gqa.plan(_shape(B=2, G=8, D=64))["workgroups"] == 2 * 8 * 4096 // 256
        d128 = gqa.plan(_shape(B=1, G=8, D=128))
        assert d128["workgroups"] == 8 * 4096 // 256 and d128["combine"] == 0   # 18 pieces x 2 KB merged in-kernel
        assert gqa.plan(_shape(B=1, G=8, D=64, T=16384))["workgroups"] == 8 * 32  # pieces-per-segment bound
    finally:
        del os.environ["GQA_RSPLIT"]
    # an fp8 cache too; the 32 x 32 kernel (MQA) at least 256 rows per workgroup
    assert gqa.plan(_shape(B=1, G=8, D=64, kv_dtype=gqa.GQA_FP8_E4M3))["workgroups"] == 8 * 4096 // 256
    assert gqa.plan(_shape(B=1, G=8, D=128, kv_dtype=gqa.GQA_FP8_E4M3))["workgroups"] == 8 * 4096 // 256
    assert gqa.plan(_shape(B=1, G=1, T=8192))["workgroups"] == 8192 // 256


def test_plan_workgroup_option(lib):
    p = gqa.plan(_shape(), workgroups=100)
    assert p["workgroups"] == 100
    small = gqa.plan(_shape(B=1, T=100))
    # a tiny cache gets no more row-split workgroups than it has 32-row tiles
    # per wave: 8 KV heads x 100 rows / (4 waves x 32)
    assert small["workgroups"] == 7 and small["waves_per_group"] == 4
    small = gqa.plan(_shape(B=1, T=100, q_dtype=gqa.GQA_F32, kv_dtype=gqa.GQA_F32))
    # ... and the vector-ALU path no more one-wave workgroups than it has
    # shares of two tiles (8 rows of 128 fp32 values each): 8 x 100 / 16
    assert small["workgroups"] == 50 and small["waves_per_group"] == 1


def test_plan_row_blocks_for_large_groups(lib):
    p = gqa.plan(_shape(G=1, sq=2, q_dtype=gqa.GQA_F32, kv_dtype=gqa.GQA_F32), path=gqa.PATH_VALU)
    assert p["rows_per_group"] == 64
    assert p["row_blocks"] == 4 and p["row_block"] == 16
    p = gqa.plan(_shape(H=6, G=1, sq=3), path=gqa.PATH_VALU)
    assert p["rows_per_group"] == 18 and p["row_blocks"] == 2
    p = gqa.plan(_shape(H=12, G=4, sq=1), path=gqa.PATH_VALU)
    assert p["rows_per_group"] == 3 and p["row_block"] == 4


def test_plan_matrix_path_row_blocks(lib):
    """The matrix-core path packs 16, 32, 64 or (a plain bf16 cache) 128 or
    256 query rows per segment, so the K/V of a group is read once for up to
    256 rows."""
    cases = [  # (H, G, sq) -> rows, row block, row blocks
        ((32, 8, 1), 4, 16, 1),
        ((32, 4, 2), 16, 16, 1),
        ((32, 1, 1), 32, 32, 1),
        ((6, 1, 3), 18, 32, 1),
        ((32, 1, 2), 64, 64, 1),
        ((32, 1, 3), 96, 128, 1),
        ((32, 8, 64), 256, 256, 1),
        ((32, 1, 5), 160, 256, 1),
        ((32, 1, 9), 288, 256, 2),
    ]
    for (H, G, sq), rows, rb, nrb in cases:
        p = gqa.plan(_shape(H=H, G=G, sq=sq))
        assert p["path"] == gqa.PATH_MFMA
        assert (p["rows_per_group"], p["row_block"], p["row_blocks"]) == (rows, rb, nrb), (H, G, sq)
        # slots (two per workgroup): min(rb, rows) rows of 128 values, then
        # their log-sum-exp floats padded to a multiple of 16 (at least 16)
        sr = min(rb, rows)
        lse = (max(sr, 16) + 15) // 16 * 16
        assert p["workspace_bytes"] == (1 << 20) + _round256(p["workgroups"] * 2 * (sr * 128 + lse) * 4)


def test_plan_merge_mode(lib):
    """Small merges stay in the decode kernel; a segment split into many
    pieces of many live rows goes to the combine kernel; both can be forced."""
    assert gqa.plan(_shape(B=32))["combine"] == 0                      # 4 live rows
    mqa = _shape(B=64, H=32, G=1, T=8192)                                # 32 live rows
    assert gqa.plan(mqa)["combine"] == 1
    assert gqa.plan(mqa, merge=gqa.MERGE_IN_KERNEL)["combine"] == 0
    assert gqa.plan(_shape(B=32), merge=gqa.MERGE_COMBINE)["combine"] == 1
    f32 = _shape(q_dtype=gqa.GQA_F32, kv_dtype=gqa.GQA_F32)
    with pytest.raises(gqa.GqaError) as ei:
        gqa.plan(f32, merge=gqa.MERGE_COMBINE)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    with pytest.raises(gqa.GqaError) as ei:
        gqa.plan(_shape(), merge=3)
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG

    # the combine flag does not change the workspace
    assert gqa.plan(mqa)["workspace_bytes"] == gqa.plan(mqa, merge=gqa.MERGE_IN_KERNEL)["workspace_bytes"]


@pytest.mark.parametrize("kw,status", [
    (dict(H=30, G=8), gqa.GQA_ERR_INVALID_ARG),
    (dict(G=0), gqa.GQA_ERR_INVALID_ARG),
    (dict(sq=0), gqa.GQA_ERR_INVALID_ARG),
    (dict(T=0), gqa.GQA_ERR_INVALID_ARG),
    (dict(B=-1), gqa.GQA_ERR_INVALID_ARG),
    (dict(D=96), gqa.GQA_ERR_UNSUPPORTED),
    (dict(q_dtype=gqa.GQA_F32), gqa.GQA_ERR_UNSUPPORTED),
    (dict(out_dtype=gqa.GQA_BF16), gqa.GQA_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), gqa.GQA_ERR_UNSUPPORTED),
    (dict(T=1 << 25, D=128), gqa.GQA_ERR_INVALID_ARG),
    (dict(B=1 << 16, G=8, H=32), gqa.GQA_ERR_INVALID_ARG),     # > 2^18 segments
])
def test_bad_shapes_rejected(lib, kw, status):
    s = _shape(**kw)
    with pytest.raises(gqa.GqaError) as ei:
        gqa.plan(s)
    assert ei.value.status == status
    assert gqa.workspace_bytes(s) == 0
    # the decode entry point refuses the same shape before any GPU work
    st = lib.gqa_decode(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, None)
    assert st == status
    assert lib.gqa_last_error().decode()


def test_null_and_misaligned_pointers_rejected(lib):
    s = _shape()
    st = lib.gqa_decode(ctypes.byref(s), None, 16, 16, None, ctypes.c_float(0.1), 16, None)
    assert st == gqa.GQA_ERR_INVALID_ARG
    st = lib.gqa_decode(ctypes.byref(s), 18, 16, 16, None, ctypes.c_float(0.1), 16, None)
    assert st == gqa.GQA_ERR_INVALID_ARG
    assert "aligned" in lib.gqa_last_error().decode()
    st = lib.gqa_decode(None, 16, 16, 16, None, ctypes.c_float(0.1), 16, None)
    assert st == gqa.GQA_ERR_INVALID_ARG


def test_workspace_clear_argument_checks(lib):
    """gqa_workspace_clear refuses a NULL workspace and one smaller than the
    1 MiB counter region, before any device call."""
    st = lib.gqa_workspace_clear(None, ctypes.c_size_t(1 << 20), None)
    assert st == gqa.GQA_ERR_INVALID_ARG and "NULL" in lib.gqa_last_error().decode()
    st = lib.gqa_workspace_clear(256, ctypes.c_size_t((1 << 20) - 4), None)
    assert st == gqa.GQA_ERR_INVALID_ARG and "counter region" in lib.gqa_last_error().decode()


def test_non_finite_scale_rejected(lib):
    s = _shape()
    for bad in (float("nan"), float("inf")):
        st = lib.gqa_decode(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(bad), 16, None)
        assert st == gqa.GQA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(lib):
    s = _shape(B=0)
    assert lib.gqa_decode(ctypes.byref(s), None, None, None, None, ctypes.c_float(0.1),
                          None, None) == gqa.GQA_OK
    assert lib.gqa_last_error().decode() == ""


def test_explicit_workspace_too_small_rejected(lib):
    s = _shape(B=32)
    need = gqa.workspace_bytes(s)
    assert need > 0
    st = lib.gqa_decode_ws(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16,
                           16, ctypes.c_size_t(need - 1), None)
    assert st == gqa.GQA_ERR_ALLOC


def test_bad_options_rejected(lib):
    s = _shape()
    with pytest.raises(gqa.GqaError) as ei:
        gqa.plan(s, path=9)
    assert ei.value.status == gqa.GQA_ERR_INVALID_ARG
    with pytest.raises(gqa.GqaError):
        gqa.plan(s, workgroups=-1)
    o = gqa.Options()
    o.reserved[2] = 1
    info = gqa.PlanInfo()
    assert lib.gqa_plan(ctypes.byref(s), ctypes.byref(o), ctypes.byref(info)) == \
        gqa.GQA_ERR_INVALID_ARG


def test_grid_capped_so_partial_offsets_fit_32_bits(lib):
    """The kernels address the partial slots with 32-bit byte offsets through
    a 2 GiB buffer resource.  A caller-set grid large enough to push the slot
    area past 2^31 bytes is capped (any grid gives the same result to
    rounding), never planned into offsets that wrap."""
    for H, G, sq, D in ((32, 8, 64, 128), (32, 1, 4, 128), (32, 1, 2, 128), (32, 1, 1, 128),
                        (32, 8, 64, 64)):
        s = _shape(B=64, H=H, G=G, sq=sq, D=D, T=4096)
        p = gqa.plan(s, workgroups=65536)
        rows = min(p["row_block"], p["rows_per_group"])
        lse = (max(rows, 16) + 15) // 16 * 16
        slot_bytes = 2 * (rows * D + lse) * 4
        part = p["workspace_bytes"] - (1 << 20)
        assert p["workgroups"] * slot_bytes < 1 << 31, (H, G, sq, D)
        assert part < 1 << 31
        if 65536 * slot_bytes >= 1 << 31:
            assert p["workgroups"] == ((1 << 31) - 256) // slot_bytes
        else:
            assert p["workgroups"] == 65536
    # the 256-row segments of 64 new tokens at D = 128: 33,024 floats a slot
    assert gqa.plan(_shape(B=64, G=8, sq=64), workgroups=65536)["workgroups"] == 8128
    # the combine kernel sizes its grid from the capped plan as well
    p = gqa.plan(_shape(B=64, G=8, sq=64), workgroups=65536, merge=gqa.MERGE_COMBINE)
    assert p["workgroups"] == 8128 and p["combine"] == 1


def test_injected_workspace_allocation_failure(lib, monkeypatch):
    """GQA_TEST_FAIL_ALLOC=1 makes the library-owned workspace report an
    allocation failure (before any device call), which every entry point with
    a library workspace returns as GQA_ERR_ALLOC with a message; a caller
    workspace is not affected by the hook."""
    s = _shape(B=32)
    monkeypatch.setenv("GQA_TEST_FAIL_ALLOC", "1")
    st = lib.gqa_decode(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, None)
    assert st == gqa.GQA_ERR_ALLOC
    assert "GQA_TEST_FAIL_ALLOC" in lib.gqa_last_error().decode()
    st = lib.gqa_decode_ex(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, None,
                           ctypes.c_size_t(0), None, None)
    assert st == gqa.GQA_ERR_ALLOC
    # a caller workspace that is too small is still the caller's error
    st = lib.gqa_decode_ws(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, 16,
                           ctypes.c_size_t(64), None)
    assert st == gqa.GQA_ERR_ALLOC and "needed" in lib.gqa_last_error().decode()
    monkeypatch.setenv("GQA_TEST_FAIL_ALLOC", "0")
    # without the hook the same call gets past the workspace step; with no
    # GPU it then fails at the device (GQA_ERR_HIP), never with ALLOC
    import torch
    if not torch.cuda.is_available():
        st = lib.gqa_decode(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, None)
        assert st == gqa.GQA_ERR_HIP


def test_plan_fp16(lib):
    """fp16 q/k/v plan exactly as bf16 does (the same grids, kernels and
    workspaces: the matrix-core kernels take either 2-byte type); above 16
    query rows per KV head the 32 x 32 kernel runs even when GQA_MFX=0 asks
    bf16 for the 16 x 16 one; appended tokens and paged caches plan as
    bf16 too.  fp16 has no scores-only matrix path and mixes with no other
    type."""
    f16 = dict(q_dtype=gqa.GQA_F16, kv_dtype=gqa.GQA_F16)
    for kw in (dict(B=32), dict(B=1, D=64), dict(B=4, D=128), dict(B=64, G=1, T=8192),
               dict(B=16, G=1, sq=2, T=16384), dict(B=8, sq=64), dict(B=1, T=100)):
        assert gqa.plan(_shape(**kw, **f16)) == gqa.plan(_shape(**kw)), kw
        assert gqa.workspace_bytes(_shape(**kw, **f16)) == gqa.workspace_bytes(_shape(**kw))
    v = gqa.plan(_shape(**f16), path=gqa.PATH_VALU)
    assert v == gqa.plan(_shape(), path=gqa.PATH_VALU) and v["path"] == gqa.PATH_VALU
    import os
    mqa = dict(B=64, G=1, T=8192)
    mfx = gqa.plan(_shape(**mqa))
    assert mfx["waves_per_group"] == 4
    os.environ["GQA_MFX"] = "0"
    try:
        assert gqa.plan(_shape(**mqa))["waves_per_group"] == 1
        assert gqa.plan(_shape(**mqa, **f16)) == mfx
    finally:
        del os.environ["GQA_MFX"]
    with pytest.raises(gqa.GqaError) as ei:
        gqa.plan(_shape(**f16), path=gqa.PATH_MFMA_QK)
    assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
    for q_dt, kv_dt, out_dt in ((gqa.GQA_F16, gqa.GQA_BF16, gqa.GQA_F32), (gqa.GQA_BF16, gqa.GQA_F16, gqa.GQA_F32),
                                (gqa.GQA_F16, gqa.GQA_FP8_E4M3, gqa.GQA_F32), (gqa.GQA_F16, gqa.GQA_F16, gqa.GQA_F16),
                                (gqa.GQA_F32, gqa.GQA_F16, gqa.GQA_F32)):
        s = _shape(q_dtype=q_dt, kv_dtype=kv_dt, out_dtype=out_dt)
        with pytest.raises(gqa.GqaError) as ei:
            gqa.plan(s)
        assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
        assert "F16,F16,F32" in lib.gqa_last_error().decode()
    for kw in (dict(B=32), dict(B=16, G=1, sq=2), dict(B=8, sq=64)):
        a = gqa.append_workspace_bytes(_shape(**kw, **f16))
        assert a > 0 and a == gqa.append_workspace_bytes(_shape(**kw))
    ps = dict(B=32, H=32, G=8, sq=1, D=128, page_size=16, num_pages=8192, max_pages=256, out_dtype=gqa.GQA_F32)
    a = gqa.paged_workspace_bytes(gqa.PagedShape(q_dtype=gqa.GQA_F16, kv_dtype=gqa.GQA_F16, **ps))
    assert a > 0 and a == gqa.paged_workspace_bytes(gqa.PagedShape(q_dtype=gqa.GQA_BF16, kv_dtype=gqa.GQA_BF16, **ps))


def test_plan_int8(lib):
    """An int8 cache plans exactly as an fp8 one (one byte per element, the
    one-block matrix-core kernel, four one-wave workgroups per CU); it runs
    on GQA_PATH_MFMA only, with bf16 queries and fp32 out."""
    for kw in (dict(B=32), dict(B=1, D=64), dict(B=64, G=1, T=8192), dict(B=8, sq=64)):
        a = gqa.plan(_shape(kv_dtype=gqa.GQA_INT8, **kw))
        assert a == gqa.plan(_shape(kv_dtype=gqa.GQA_FP8_E4M3, **kw)), kw
    for kw, status in ((dict(path=gqa.PATH_VALU), gqa.GQA_ERR_UNSUPPORTED),
                       (dict(path=gqa.PATH_MFMA_QK), gqa.GQA_ERR_UNSUPPORTED)):
        with pytest.raises(gqa.GqaError) as ei:
            gqa.plan(_shape(kv_dtype=gqa.GQA_INT8), **kw)
        assert ei.value.status == status
    for q_dt, out_dt in ((gqa.GQA_F16, gqa.GQA_F32), (gqa.GQA_F32, gqa.GQA_F32), (gqa.GQA_BF16, gqa.GQA_BF16)):
        with pytest.raises(gqa.GqaError) as ei:
            gqa.plan(_shape(q_dtype=q_dt, kv_dtype=gqa.GQA_INT8, out_dtype=out_dt))
        assert ei.value.status == gqa.GQA_ERR_UNSUPPORTED
        assert "BF16,INT8,F32" in lib.gqa_last_error().decode()
    # the entry points check the cache type before any device call
    s = _shape(kv_dtype=gqa.GQA_FP8_E4M3)
    st = lib.gqa_decode_int8(ctypes.byref(s), 16, 16, 16, None, None, None, ctypes.c_float(0.1), 16, None,
                             ctypes.c_size_t(0), None, None)
    assert st == gqa.GQA_ERR_INVALID_ARG and "GQA_INT8" in lib.gqa_last_error().decode()
    s = _shape(kv_dtype=gqa.GQA_INT8)
    st = lib.gqa_decode_fp8(ctypes.byref(s), 16, 16, 16, None, None, None, ctypes.c_float(0.1), 16, None,
                            ctypes.c_size_t(0), None, None)
    assert st == gqa.GQA_ERR_INVALID_ARG and "GQA_FP8_E4M3" in lib.gqa_last_error().decode()
    assert gqa.workspace_bytes(_shape(kv_dtype=gqa.GQA_INT8)) == gqa.workspace_bytes(_shape(kv_dtype=gqa.GQA_FP8_E4M3))


def test_append_workspace_bytes(lib):
    """Appended tokens above 16 query rows per KV head run one-wave
    workgroups of up to 64 rows, not the plain decode's 32 x 32 kernel:
    gqa_append_workspace_bytes reports the workspace that plan needs (equal
    to the plain decode's where the plans agree)."""
    for kw in (dict(B=32), dict(B=64, G=1, T=8192), dict(B=16, G=1, sq=2), dict(B=8, G=8, sq=64)):
        s = _shape(**kw)
        a = gqa.append_workspace_bytes(s)
        assert a > 0
        rows = s.H // s.G * s.sq
        if rows <= 16:
            assert a == gqa.workspace_bytes(s)
    s = _shape(B=16, G=1, sq=2)
    assert gqa.append_workspace_bytes(s) != gqa.workspace_bytes(s)
    assert gqa.append_workspace_bytes(_shape(H=30)) == 0


def test_noalloc_refuses_oversized_workspace_before_any_gpu_work(lib):
    """gqa_decode_noalloc's workspace is a fixed 64 MiB array: a plan that
    needs more (here 64 new tokens of 32 heads on 8 KV heads over 65536
    workgroups) is refused with GQA_ERR_ALLOC and a message, before any
    device call."""
    s = _shape(B=64, G=8, sq=64)
    o = gqa.Options()
    o.workgroups = 65536
    info = gqa.PlanInfo()
    assert lib.gqa_plan(ctypes.byref(s), ctypes.byref(o), ctypes.byref(info)) == gqa.GQA_OK
    assert info.workspace_bytes > 64 << 20
    st = lib.gqa_decode_noalloc(ctypes.byref(s), 16, 16, 16, None, ctypes.c_float(0.1), 16, ctypes.byref(o), None)
    assert st == gqa.GQA_ERR_ALLOC
    assert "scratch" in lib.gqa_last_error().decode()


def test_plan_paged_codes(lib):
    """A page pool of 8-bit codes (fp8 E4M3 or int8) plans as the contiguous
    8-bit cache of T = page_size * max_pages rows (the same kernel and grid:
    paging moves rows only); appended tokens into an 8-bit cache are refused
    before any device call."""
    ps = dict(B=32, H=32, G=8, sq=1, D=128, page_size=16, num_pages=8192, max_pages=256, out_dtype=gqa.GQA_F32)
    for kv in (gqa.GQA_FP8_E4M3, gqa.GQA_INT8):
        a = gqa.paged_workspace_bytes(gqa.PagedShape(q_dtype=gqa.GQA_BF16, kv_dtype=kv, **ps))
        assert a > 0 and a == gqa.plan(_shape(B=32, T=16 * 256, kv_dtype=kv))["workspace_bytes"]
        assert gqa.paged_workspace_bytes(gqa.PagedShape(q_dtype=gqa.GQA_F16, kv_dtype=kv, **ps)) == 0
        s = _shape(kv_dtype=kv)
        st = lib.gqa_decode_append(ctypes.byref(s), 16, 16, 16, 16, 16, None, ctypes.c_float(0.1), 16, None,
                                   ctypes.c_size_t(0), None, None)
        assert st == gqa.GQA_ERR_UNSUPPORTED and "bf16 / fp16 cache" in lib.gqa_last_error().decode()
