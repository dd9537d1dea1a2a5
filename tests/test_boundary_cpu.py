"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/gemm.h declares, and its host-side logic (plan creation,
validation, error reporting, kernel/schedule selection) behaves as documented.
No call here enqueues device work."""
import ctypes
import os
import re

import pytest

import dense_gemm_epilogue_02_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "gemm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gemm|grouped)_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "gemm_plan_create" in names and "grouped_gemm_run" in names
    for n in names:
        assert hasattr(g.lib, n), n           # ctypes resolves the symbol
        assert n in g.EXPORTED, n             # and the binding wraps it


def test_version_and_supported_tuples():
    assert "gfx950" in g.gemm_version()
    tuples = [g.gemm_supported_get(i) for i in range(g.gemm_supported_count())]
    D = g.Dtype
    assert (D.F32, D.F32, D.F32, D.F32, D.F32) in tuples
    assert (D.F16, D.F16, D.F16, D.F16, D.F32) in tuples
    assert (D.BF16, D.BF16, D.BF16, D.BF16, D.F32) in tuples
    assert (D.F8_E4M3, D.F8_E4M3, D.BF16, D.BF16, D.F32) in tuples
    with pytest.raises(g.GemmError) as e:
        g.gemm_supported_get(99)
    assert e.value.status == g.Status.INVALID_ARG


def test_status_strings():
    for s in g.Status:
        assert g.gemm_status_string(s) == "GEMM_" + s.name


def test_unsupported_tuple_is_named():
    D, L = g.Dtype, g.Layout
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create(D.F16, D.BF16, D.F16, D.F16, D.F32, L.ROW_MAJOR, L.ROW_MAJOR,
                           L.ROW_MAJOR, g.Epilogue.LINEAR)
    assert e.value.status == g.Status.UNSUPPORTED
    assert "A=F16, B=BF16" in str(e.value)
    with pytest.raises(g.GemmError) as e:   # fp16 accumulator is not offered
        g.gemm_plan_create(D.F16, D.F16, D.F16, D.F16, D.F16, L.ROW_MAJOR, L.ROW_MAJOR,
                           L.ROW_MAJOR, g.Epilogue.LINEAR)
    assert e.value.status == g.Status.UNSUPPORTED
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create_simple(D.F8_E4M3, L.ROW_MAJOR, g.Epilogue.LINEAR)
    assert e.value.status == g.Status.UNSUPPORTED


def test_bad_enums_and_handles():
    D, L = g.Dtype, g.Layout
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create(D.F16, D.F16, D.F16, D.F16, D.F32, 7, L.ROW_MAJOR, L.ROW_MAJOR, 0)
    assert e.value.status == g.Status.INVALID_ARG
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create(D.F16, D.F16, D.F16, D.F16, D.F32, 0, 0, 0, 5)
    assert e.value.status == g.Status.INVALID_ARG
    assert g.lib.gemm_plan_create(None, 0, 0, 0, 0, 0, 0, 0, 0, 0) == g.Status.INVALID_ARG
    assert g.lib.gemm_plan_run(None, None, None, None, None, 1, 1, 1, 1.0, 0.0, None) == \
        g.Status.NOT_INITIALIZED
    assert "invalid plan" in g.gemm_last_error()
    assert g.lib.gemm_plan_destroy(None) == g.Status.OK


def test_create_simple_and_destroy_without_device():
    for dt in (g.Dtype.F32, g.Dtype.F16, g.Dtype.BF16):
        h = g.gemm_plan_create_simple(dt, g.Layout.ROW_MAJOR, g.Epilogue.RELU)
        assert h
        g.gemm_plan_destroy(h)


def test_run_argument_validation_before_any_device_call():
    h = g.gemm_plan_create_simple(g.Dtype.F16, g.Layout.ROW_MAJOR, g.Epilogue.LINEAR)
    try:
        run = g.lib.gemm_plan_run
        assert run(h, 16, 16, 16, 16, -1, 4, 4, 1.0, 0.0, None) == g.Status.INVALID_ARG
        assert "negative size" in g.gemm_last_error()
        assert run(h, 16, 16, None, None, 4, 4, 4, 1.0, 0.0, None) == g.Status.INVALID_ARG
        assert "D is NULL" in g.gemm_last_error()
        assert run(h, None, 16, None, 16, 4, 4, 4, 1.0, 0.0, None) == g.Status.INVALID_ARG
        assert run(h, 16, 16, None, 16, 4, 4, 4, 1.0, 0.5, None) == g.Status.INVALID_ARG
        assert "C is NULL" in g.gemm_last_error()
        # empty output: a no-op that succeeds without touching the device
        assert run(h, None, None, None, None, 0, 8, 8, 1.0, 1.0, None) == g.Status.OK
        assert run(h, None, None, None, None, 8, 0, 8, 1.0, 1.0, None) == g.Status.OK
        assert g.gemm_last_error() == ""
        # grouped: count < 0, NULL array, empty problems
        assert g.lib.grouped_gemm_run(h, None, -1, 1.0, 0.0, None) == g.Status.INVALID_ARG
        assert g.lib.grouped_gemm_run(h, None, 2, 1.0, 0.0, None) == g.Status.INVALID_ARG
        assert g.lib.grouped_gemm_run(h, None, 0, 1.0, 0.0, None) == g.Status.OK
        g.grouped_gemm_run(h, [(0, 8, 8, None, None, None, None)], 1.0, 0.0, stream=0)
        with pytest.raises(g.GemmError) as e:
            g.grouped_gemm_run(h, [(4, 4, 4, 16, 16, None, None)], 1.0, 0.0, stream=0)
        assert "problem 0" in str(e.value)
    finally:
        g.gemm_plan_destroy(h)


def test_set_config_validation():
    h = g.gemm_plan_create_simple(g.Dtype.BF16, g.Layout.ROW_MAJOR, g.Epilogue.LINEAR)
    try:
        g.gemm_plan_set_config(h, g.Schedule.STREAM_K, g.Tile.T128x128, 64)
        for bad in ((9, 0, 0), (0, 9, 0), (0, 0, -1)):
            assert g.lib.gemm_plan_set_config(h, *bad) == g.Status.INVALID_ARG
    finally:
        g.gemm_plan_destroy(h)


def _plan(dtype_ab, la="row", lb="col", lc="row"):
    return g.Plan(dtype_ab, la=la, lb=lb, lc=lc)


def test_describe_transformer_layer_schedules():
    p = _plan("bf16")
    # hidden 8192 / FFN 28672 layer GEMMs at 4096 tokens on 256 CUs
    down = p.describe(4096, 8192, 28672)
    assert down["tile"] == "256x256" and down["schedule"] == "data_parallel"
    assert down["tiles"] == 512 and down["ipt"] == 448
    qkv = p.describe(4096, 10240, 8192)
    assert qkv["schedule"] == "hybrid" and qkv["tiles"] == 640 and qkv["sk_tiles"] == 128
    gate = p.describe(4096, 57344, 8192)
    assert gate["schedule"] == "data_parallel" and gate["tiles"] == 3584
    p.close()


def test_describe_small_and_skinny_use_stream_k():
    p = g.Plan("f16", la="row", lb="row", lc="row", relu=True)
    # 64 tiles of 128x128 for 256 CUs and K = 1024: the whole-K kernel, one
    # workgroup per 32x32 block, 16 MFMA steps per wave (4 x 256 of K)
    d = p.describe(1024, 1024, 1024)
    assert d["kernel"] == "wholek" and d["tile"] == "wholek32x32" and d["grid"] == 1024, d
    assert d["bk"] == 1024 and d["schedule"] == "data_parallel", d
    # K = 2048 is past its reach: 128x128 tiles under stream-K
    d = p.describe(1024, 1024, 2048)
    assert d["tile"] == "128x128" and d["schedule"] == "stream_k" and d["ipt"] == 32, d
    # the 128x128 tile on the 1024^3 problem, when pinned
    p.set_config(g.Schedule.AUTO, g.Tile.T128x128, 0)
    d = p.describe(1024, 1024, 1024)
    assert d["tile"] == "128x128" and d["schedule"] == "stream_k" and d["ipt"] == 16, d
    p.close()
    f = g.Plan("f32", la="row", lb="row", lc="row")
    d = f.describe(128, 64, 256)
    assert d["kernel"] == "wholek" and d["grid"] == 8 and d["bk"] == 256, d
    d = f.describe(1024, 1024, 1024)   # eight waves of 128 K each
    assert d["kernel"] == "wholek" and d["bk"] == 1024 and d["waves"] == 8, d
    d = f.describe(128, 64, 1040)   # fp32 whole-K reaches K = 1024
    assert d["kernel"] == "tile", d
    f.close()
    q = _plan("f8e4m3")
    # decode GEMMs on the four-stage fp8 tiles (one workgroup per CU): 32-64
    # tiles for 256 slots, so stream-K over every CU
    for M, N, K, tile in ((16, 8192, 28672, "64x256"), (64, 8192, 28672, "64x256"),
                          (128, 8192, 28672, "128x128")):
        d = q.describe(M, N, K)
        assert d["tile"] == tile and d["schedule"] == "stream_k", d
        assert d["grid"] == 256 and d["split"] == 0 and d["bk"] == 128, d
    # 224 tiles fill 87.5% of the slots: data-parallel
    for M in (16, 64):
        d = q.describe(M, 57344, 8192)
        assert d["tile"] == "64x256" and d["schedule"] == "data_parallel" and d["grid"] == 224, d
    # 448 tiles of 128x128 over 256 slots: one wave plus a stream-K remainder
    d = q.describe(128, 57344, 8192)
    assert d["tile"] == "128x128" and d["schedule"] == "hybrid" and d["grid"] == 256, d
    q.close()


def test_describe_generic_for_unaligned_extent():
    p = _plan("bf16")
    d = p.describe(100, 100, 13)        # K * 2 bytes not a multiple of 16
    assert d["kernel"] == "generic" and "multiple of 16" in d["generic_reason"]
    d = p.describe(100, 100, 0)         # K = 0: nothing to load, tile kernel
    assert d["kernel"] == "tile" and d["ipt"] == 0 and d["schedule"] == "data_parallel"
    p.close()


def test_describe_forced_configs():
    p = _plan("bf16")
    p.set_config(g.Schedule.STREAM_K, g.Tile.T256x256, 0)
    d = p.describe(4096, 8192, 8192)
    assert d["schedule"] == "stream_k" and d["tile"] == "256x256"
    p.set_config(g.Schedule.SPLIT_K, g.Tile.T128x128, 0)
    d = p.describe(256, 256, 8192)      # 4 tiles, 128 k-tiles: 16 units of 8
    assert d["schedule"] == "split_k" and d["split"] == 16 and d["grid"] == 64, d
    d = p.describe(4096, 8192, 8192)    # more tiles than slots: no split
    assert d["schedule"] == "data_parallel" and d["split"] == 0, d
    p.set_config(g.Schedule.DATA_PARALLEL, g.Tile.GENERIC, 0)
    assert p.describe(64, 64, 64)["kernel"] == "generic"
    p.close()


def test_activation_epilogues_and_run_ex_validation():
    D, L, E = g.Dtype, g.Layout, g.Epilogue
    for epi in (E.LINEAR, E.RELU, E.SIGMOID, E.TANH):
        h = g.gemm_plan_create(D.BF16, D.BF16, D.BF16, D.BF16, D.F32, L.ROW_MAJOR,
                               L.COL_MAJOR, L.ROW_MAJOR, epi)
        g.gemm_plan_destroy(h)
    with pytest.raises(g.GemmError) as e:
        g.gemm_plan_create(D.BF16, D.BF16, D.BF16, D.BF16, D.F32, 0, 0, 0, 4)
    assert e.value.status == g.Status.INVALID_ARG and "SIGMOID" in str(e.value)
    run_ex = g.lib.gemm_plan_run_ex
    assert run_ex(None, None, None, None, None, None, 1, 1, 1, 1.0, 0.0, None, None, None) == \
        g.Status.NOT_INITIALIZED
    h = g.gemm_plan_create_simple(D.F16, L.ROW_MAJOR, E.TANH)
    try:
        # negative sizes and a missing D fail before any device call
        assert run_ex(h, 16, 16, None, 16, 16, -1, 4, 4, 1.0, 0.0, None, None, None) == \
            g.Status.INVALID_ARG
        assert run_ex(h, 16, 16, None, None, 16, 4, 4, 4, 1.0, 0.0, None, None, None) == \
            g.Status.INVALID_ARG
        # an empty output is a no-op, bias or not
        assert run_ex(h, None, None, None, None, None, 0, 4, 4, 1.0, 0.0, None, None, None) == \
            g.Status.OK
    finally:
        g.gemm_plan_destroy(h)


def test_batched_validation_before_any_device_call():
    run_b = g.lib.gemm_plan_run_batched
    args = lambda h, cnt, sa, sb, sc, sd, M=8, N=8: (h, 16, 16, None, 16, None, M, N, 8, cnt, sa,
                                                      sb, sc, sd, 1.0, 0.0, None, None, None)
    assert run_b(*args(None, 2, 64, 64, 64, 64)) == g.Status.NOT_INITIALIZED
    h = g.gemm_plan_create_simple(g.Dtype.BF16, g.Layout.ROW_MAJOR, g.Epilogue.LINEAR)
    try:
        assert run_b(*args(h, -1, 64, 64, 64, 64)) == g.Status.INVALID_ARG
        assert run_b(*args(h, 2, -64, 64, 64, 64)) == g.Status.INVALID_ARG
        assert "negative" in g.gemm_last_error()
        # outputs of entries 0 and 1 would overlap
        assert run_b(*args(h, 2, 64, 64, 64, 63)) == g.Status.INVALID_ARG
        assert "overlap" in g.gemm_last_error()
        assert run_b(*args(h, 1 << 32, 64, 64, 64, 64)) == g.Status.UNSUPPORTED
        # empty batch or empty output: no-ops that touch no device
        assert run_b(*args(h, 0, 64, 64, 64, 64)) == g.Status.OK
        assert run_b(h, None, None, None, None, None, 8, 8, 8, 0, 0, 0, 0, 0, 1.0, 0.0, None,
                     None, None) == g.Status.OK
        assert run_b(*args(h, 3, 64, 64, 64, 0, M=0)) == g.Status.OK
        with pytest.raises(ValueError):   # the binding checks buffer extents too
            g.Plan("bf16").run_batched(None, None, None, None, 8, 8, 8, 2, (64, 64, 64, 64))
    finally:
        g.gemm_plan_destroy(h)


def test_mx_validation_before_any_device_call():
    D, L, E = g.Dtype, g.Layout, g.Epilogue
    run_mx = g.lib.gemm_plan_run_mx
    args = lambda h, K, xa=16, xb=16: (h, 16, 16, None, 16, None, 8, 8, K, 1.0, 0.0, xa, xb,
                                       None)
    assert run_mx(*args(None, 64)) == g.Status.NOT_INITIALIZED
    h = g.gemm_plan_create_simple(D.BF16, L.ROW_MAJOR, E.LINEAR)
    try:
        assert run_mx(*args(h, 64)) == g.Status.UNSUPPORTED
        assert "F8_E4M3" in g.gemm_last_error()
    finally:
        g.gemm_plan_destroy(h)
    h = g.gemm_plan_create(D.F8_E4M3, D.F8_E4M3, D.BF16, D.BF16, D.F32, L.ROW_MAJOR,
                           L.COL_MAJOR, L.ROW_MAJOR, E.LINEAR)
    try:
        assert run_mx(*args(h, 48)) == g.Status.INVALID_ARG
        assert "multiple of the 32-element" in g.gemm_last_error()
        assert run_mx(*args(h, 64, xa=None)) == g.Status.INVALID_ARG
        assert "NULL" in g.gemm_last_error()
        # an empty output is a no-op
        assert run_mx(h, None, None, None, None, None, 0, 8, 64, 1.0, 0.0, None, None,
                      None) == g.Status.OK
    finally:
        g.gemm_plan_destroy(h)


def test_aux_validation_before_any_device_call():
    run_aux = g.lib.gemm_plan_run_aux
    args = lambda h, op=0, pos=0, aux=32, out=48, D=16, M=8: (
        h, 16, 16, None, D, None, aux, op, pos, out, M, 8, 8, 1.0, 0.0, None, None, None)
    assert run_aux(*args(None)) == g.Status.NOT_INITIALIZED
    h = g.gemm_plan_create_simple(g.Dtype.F16, g.Layout.ROW_MAJOR, g.Epilogue.RELU)
    try:
        assert run_aux(*args(h, op=4)) == g.Status.INVALID_ARG
        assert "elementwise op" in g.gemm_last_error()
        assert run_aux(*args(h, op=-1)) == g.Status.INVALID_ARG
        assert run_aux(*args(h, pos=2)) == g.Status.INVALID_ARG
        assert "side of the activation" in g.gemm_last_error()
        assert run_aux(*args(h, out=16)) == g.Status.INVALID_ARG   # Z over D
        assert "same buffer" in g.gemm_last_error()
        # negative sizes fail; an empty output is a no-op
        assert run_aux(*args(h, M=-1)) == g.Status.INVALID_ARG
        assert run_aux(*args(h, D=None, aux=None, out=None, M=0)) == g.Status.OK
        with pytest.raises(ValueError):   # the binding checks buffer extents too
            g.Plan("f16").run_aux(None, None, None, None, 8, 8, 8, aux_op="mul")
    finally:
        g.gemm_plan_destroy(h)


def _cache_doc(entries, a="BF16", layout_b="col"):
    import json
    return json.dumps({"format": "mi355-gemm-config-cache", "version": 1, "arch": "gfx950",
                       "plan": {"a": a, "b": a, "c": a, "d": a, "acc": "F32", "layout_a": "row",
                                "layout_b": layout_b, "layout_c": "row"},
                       "entries": entries})


def test_config_cache_import_export_round_trip_without_device():
    import json
    D, L, E = g.Dtype, g.Layout, g.Epilogue
    mk = lambda: g.gemm_plan_create(D.BF16, D.BF16, D.BF16, D.BF16, D.F32, L.ROW_MAJOR,
                                    L.COL_MAJOR, L.ROW_MAJOR, E.LINEAR)
    h, h2 = mk(), mk()
    try:
        assert g.gemm_plan_cache_size(h) == 0
        empty = json.loads(g.gemm_plan_cache_export(h))
        assert empty["format"] == "mi355-gemm-config-cache" and empty["entries"] == []
        assert empty["plan"]["layout_b"] == "col" and empty["plan"]["a"] == "BF16"
        before = g.gemm_plan_describe(h, 4096, 8192, 8192)
        assert before["tile"] == "256x256" and before["schedule"] == "data_parallel"
        doc = _cache_doc([{"m": 4096, "n": 8192, "k": 8192, "mx": 0, "schedule": "stream_k",
                           "tile": "128x128", "sk_grid": 0, "us": 500.0},
                          {"m": 64, "n": 64, "k": 64, "schedule": "data_parallel",
                           "tile": "generic"}])
        g.gemm_plan_cache_import(h, doc)
        assert g.gemm_plan_cache_size(h) == 2
        # a cached shape changes what a run launches; other shapes do not change
        after = g.gemm_plan_describe(h, 4096, 8192, 8192)
        assert after["tile"] == "128x128" and after["schedule"] == "stream_k"
        assert g.gemm_plan_describe(h, 64, 64, 64)["kernel"] == "generic"
        assert g.gemm_plan_describe(h, 4096, 8192, 4096)["tile"] == "256x256"
        # an explicit override wins over the cache
        g.gemm_plan_set_config(h, g.Schedule.DATA_PARALLEL, g.Tile.T256x256, 0)
        assert g.gemm_plan_describe(h, 4096, 8192, 8192)["schedule"] == "data_parallel"
        g.gemm_plan_set_config(h, g.Schedule.AUTO, g.Tile.AUTO, 0)
        # export -> import into a fresh plan reproduces the cache
        text = g.gemm_plan_cache_export(h)
        g.gemm_plan_cache_import(h2, text)
        assert g.gemm_plan_cache_export(h2) == text
        ents = json.loads(text)["entries"]
        assert [(e["m"], e["tile"], e["schedule"]) for e in ents] == \
            [(64, "generic", "data_parallel"), (4096, "128x128", "stream_k")]
        g.gemm_plan_cache_clear(h2)
        assert g.gemm_plan_cache_size(h2) == 0
    finally:
        g.gemm_plan_destroy(h)
        g.gemm_plan_destroy(h2)


def test_config_cache_import_rejects_bad_text_and_keeps_cache():
    D, L, E = g.Dtype, g.Layout, g.Epilogue
    h = g.gemm_plan_create(D.BF16, D.BF16, D.BF16, D.BF16, D.F32, L.ROW_MAJOR, L.COL_MAJOR,
                           L.ROW_MAJOR, E.LINEAR)
    imp = lambda t: g.lib.gemm_plan_cache_import(h, t.encode())
    try:
        good = {"m": 1, "n": 2, "k": 3, "schedule": "hybrid", "tile": "64x256"}
        assert imp(_cache_doc([good])) == g.Status.OK
        assert g.gemm_plan_cache_size(h) == 1
        bad = [
            "", "{", "[1, 2]", "{\"format\": \"x\", \"version\": 1}",
            _cache_doc([good]) + " trailing",
            _cache_doc([dict(good, m=-1)]),
            _cache_doc([dict(good, m=1.5)]),
            _cache_doc([dict(good, tile="512x512")]),
            _cache_doc([dict(good, schedule="fastest")]),
            _cache_doc([good, {"m": 5}]),              # a bad entry rejects the whole text
            _cache_doc([good]).replace("\"version\": 1", "\"version\": 2"),
        ]
        for t in bad:
            assert imp(t) == g.Status.INVALID_ARG, t
            assert "gemm_plan_cache_import" in g.gemm_last_error()
        # written for another plan's types or layouts
        assert imp(_cache_doc([good], a="F16")) == g.Status.UNSUPPORTED
        assert imp(_cache_doc([good], layout_b="row")) == g.Status.UNSUPPORTED
        assert "layout_b" in g.gemm_last_error()
        assert g.gemm_plan_cache_size(h) == 1          # unchanged by every failure
        # a short export buffer is an error and writes nothing
        need = ctypes.c_int32(0)
        assert g.lib.gemm_plan_cache_export(h, None, 0, ctypes.byref(need)) == g.Status.OK
        buf = ctypes.create_string_buffer(need.value - 1)
        assert g.lib.gemm_plan_cache_export(h, buf, len(buf), ctypes.byref(need)) == \
            g.Status.INVALID_ARG
        assert buf.value == b""
        assert g.lib.gemm_plan_cache_size(None) == -1
        assert g.lib.gemm_plan_cache_import(None, b"{}") == g.Status.NOT_INITIALIZED
    finally:
        g.gemm_plan_destroy(h)


def test_profile_validation_before_any_device_call():
    prof = g.lib.gemm_plan_profile
    n = ctypes.c_int32(0)
    arr = (g.gemm_config * 4)()
    args = lambda h, iters=5, C=None, D=16, beta=0.0, res=arr, M=8: (
        h, 16, 16, C, D, M, 8, 8, 1.0, beta, iters, res, 4 if res is not None else 0,
        ctypes.byref(n), None)
    assert prof(*args(None)) == g.Status.NOT_INITIALIZED
    h = g.gemm_plan_create_simple(g.Dtype.F16, g.Layout.ROW_MAJOR, g.Epilogue.LINEAR)
    try:
        assert prof(*args(h, iters=0)) == g.Status.INVALID_ARG
        assert "iters" in g.gemm_last_error()
        assert prof(*args(h, C=16, D=16, beta=1.0)) == g.Status.INVALID_ARG
        assert "previous run" in g.gemm_last_error()
        assert prof(*args(h, M=-1)) == g.Status.INVALID_ARG
        assert prof(*args(h, D=None, M=0)) == g.Status.OK and n.value == 0
    finally:
        g.gemm_plan_destroy(h)


def test_describe_batched_tile_choice():
    """A batch that supplies a full wave of 256x256 tiles gets them when K is
    long (K >= 2048); with K = 1024 it keeps 128x128 tiles, and the tile count
    covers the batch. (A single 1024^3 problem goes to the whole-K kernel,
    which takes no batches.)"""
    h = g.gemm_plan_create_simple(g.Dtype.F16, g.Layout.ROW_MAJOR, g.Epilogue.LINEAR)
    try:
        one = g.gemm_plan_describe_batched(h, 1024, 1024, 1024, 1)
        assert one == g.gemm_plan_describe(h, 1024, 1024, 1024)
        assert one["tile"] == "wholek32x32"
        b16 = g.gemm_plan_describe_batched(h, 1024, 1024, 1024, 16)
        assert b16["tile"] == "128x128" and b16["tiles"] == 1024
        assert b16["schedule"] == "data_parallel"
        b16k = g.gemm_plan_describe_batched(h, 1024, 1024, 2048, 16)
        assert b16k["tile"] == "256x256" and b16k["tiles"] == 256
        assert g.gemm_plan_describe_batched(h, 64, 1024, 1024, 64)["tile"] == "64x256"
        assert g.lib.gemm_plan_describe_batched(h, 8, 8, 8, 0, 0, ctypes.create_string_buffer(64),
                                                64) == g.Status.INVALID_ARG
    finally:
        g.gemm_plan_destroy(h)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; --gpus N > 1 exits with a message
    (before touching any device)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_config_cache_import_survives_random_mutations():
    """Random byte edits, truncations and duplications of a valid cache text:
    the importer returns OK, INVALID_ARG or UNSUPPORTED and never crashes; a
    failed import leaves the cache as it was."""
    import random
    D, L, E = g.Dtype, g.Layout, g.Epilogue
    h = g.gemm_plan_create(D.BF16, D.BF16, D.BF16, D.BF16, D.F32, L.ROW_MAJOR, L.COL_MAJOR,
                           L.ROW_MAJOR, E.LINEAR)
    try:
        base = _cache_doc([{"m": 4096, "n": 8192, "k": 8192, "mx": 0, "schedule": "stream_k",
                            "tile": "128x128", "sk_grid": 0, "us": 500.0},
                           {"m": 1, "n": 2, "k": 3, "schedule": "hybrid", "tile": "64x256"}])
        rng = random.Random(9)
        alphabet = '{}[]:,"\\0123456789.eE+-truefalsn x\t\n'
        ok = bad = 0
        for trial in range(3000):
            s = list(base)
            for _ in range(rng.randint(1, 4)):
                kind = rng.randrange(4)
                pos = rng.randrange(len(s) + 1)
                if kind == 0 and s:
                    s[min(pos, len(s) - 1)] = rng.choice(alphabet)
                elif kind == 1:
                    s.insert(pos, rng.choice(alphabet))
                elif kind == 2 and s:
                    del s[min(pos, len(s) - 1)]
                else:
                    s = s[:pos]
            text = "".join(s)
            before = g.gemm_plan_cache_export(h)
            st = g.lib.gemm_plan_cache_import(h, text.encode())
            assert st in (g.Status.OK, g.Status.INVALID_ARG, g.Status.UNSUPPORTED), (st, text)
            if st == g.Status.OK:
                ok += 1
                g.gemm_plan_cache_clear(h)
            else:
                bad += 1
                assert g.gemm_plan_cache_export(h) == before
        assert bad > 0
        # deeply nested input is rejected, not recursed into without bound
        assert g.lib.gemm_plan_cache_import(h, ("[" * 100000).encode()) == g.Status.INVALID_ARG
    finally:
        g.gemm_plan_destroy(h)


def test_describe_wholek_eligibility():
    """Host-only: when the whole-K kernel is chosen (AUTO) or taken when
    pinned, and when a request for it falls back to the tile kernels."""
    def d(plan, M, N, K):
        return plan.describe(M, N, K)
    f16 = g.Plan("f16", la="row", lb="row", lc="row")
    # AUTO: few 128x128 tiles and K <= 1024 -> whole-K, one block per 32x32
    x = d(f16, 200, 136, 1000)
    assert x["kernel"] == "wholek" and x["grid"] == 7 * 5, x
    # K-contiguous A with rows that are not whole 16-byte chunks: not whole-K
    assert d(f16, 200, 136, 1001)["kernel"] != "wholek"
    # long K, or enough tiles to fill the GPU: the tile kernels
    assert d(f16, 200, 136, 1088)["kernel"] == "tile"
    assert d(f16, 4096, 4096, 512)["kernel"] == "tile"
    # a pinned schedule asks for the tile kernels even when whole-K could run
    f16.set_config(g.Schedule.STREAM_K, g.Tile.AUTO, 0)
    assert d(f16, 200, 136, 1000)["kernel"] == "tile"
    # pinned whole-K on a problem it cannot take: the heuristic tile
    f16.set_config(g.Schedule.AUTO, g.Tile.WHOLEK, 0)
    assert d(f16, 4096, 4096, 512)["kernel"] == "wholek"     # K fits: taken even when large
    assert d(f16, 64, 64, 2048)["kernel"] == "tile"
    # batched calls never take it
    assert f16.describe_batched(200, 136, 1000, 4)["kernel"] == "tile"
    f16.close()
    # M/N-contiguous operands load element by element: any K up to the limit
    cc = g.Plan("bf16", la="col", lb="row", lc="row")
    assert d(cc, 40, 31, 13)["kernel"] == "wholek"
    cc.close()
    # fp8 has no whole-K form
    f8 = g.Plan("f8e4m3", la="row", lb="col", lc="row")
    assert d(f8, 64, 64, 256)["kernel"] == "tile"
    f8.close()
    # fp32: four waves up to K = 512, eight up to 1024
    f32 = g.Plan("f32", la="row", lb="row", lc="row")
    assert d(f32, 128, 64, 512)["waves"] == 4 and d(f32, 128, 64, 1024)["waves"] == 8
    f32.close()
