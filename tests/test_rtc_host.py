"""Run-time specialisation without a GPU: hipRTC compiles the FP8 head GEMV for gfx950 from the
source built into the library, the code object lands in the disk cache under its key, a second
request is served from the cache, and bad arguments are refused before any compilation."""
import os

import pytest

import quantized_weight_streaming_amd as qws
from quantized_weight_streaming_amd import _lib


def test_compile_then_cache_hit(tmp_path):
    d = str(tmp_path / "cache")
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(1, 999, 96, "gfx950", d)
    files = os.listdir(d)
    assert len(files) == 1 and files[0].startswith("head_fp8_m1_r999_c96_gfx950_") and files[0].endswith(".co")
    with open(os.path.join(d, files[0]), "rb") as f:
        blob = f.read()
    assert blob[:8] == b"QWSRTC1\0" and b"\x7fELF" in blob
    s = qws.rtc_stats()
    assert s["compiles"] == 1 and s["disk_hits"] == 0 and s["compile_ms"] > 0
    qws.rtc_compile_head_fp8(1, 999, 96, "gfx950", d)          # same key: from the disk cache
    s = qws.rtc_stats()
    assert s["compiles"] == 1 and s["disk_hits"] == 1
    qws.rtc_compile_head_fp8(4, 999, 96, "gfx950", d)          # another M: another key
    assert len(os.listdir(d)) == 2 and qws.rtc_stats()["compiles"] == 2


def test_truncated_cache_file_is_recompiled(tmp_path):
    d = str(tmp_path / "cache")
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(2, 64, 2560, "gfx950", d)
    f = os.path.join(d, os.listdir(d)[0])
    with open(f, "r+b") as fh:
        fh.truncate(100)
    qws.rtc_compile_head_fp8(2, 64, 2560, "gfx950", d)
    s = qws.rtc_stats()
    assert s["compiles"] == 2 and s["disk_hits"] == 0
    assert os.path.getsize(f) > 100


@pytest.mark.parametrize("M,rows,cols,arch,status", [
    (0, 100, 64, "gfx950", _lib.QWS_ERR_SHAPE), (5, 100, 64, "gfx950", _lib.QWS_ERR_SHAPE),
    (1, 0, 64, "gfx950", _lib.QWS_ERR_SHAPE), (1, 100, 48, "gfx950", _lib.QWS_ERR_SHAPE),
    (1, 100, 2592, "gfx950", _lib.QWS_ERR_SHAPE), (1, 100, 64, "", _lib.QWS_ERR_ARG),
    (1, 100, 64, "gfx_no_such_arch", _lib.QWS_ERR_ARG), (1, 100, 64, "gfx950:xnack", _lib.QWS_ERR_ARG),
    (1, 100, 64, "gfx950;rm", _lib.QWS_ERR_ARG),
])
def test_compile_validation(tmp_path, M, rows, cols, arch, status):
    st = qws.lib().qws_rtc_compile_head_fp8(M, rows, cols, arch.encode(), str(tmp_path).encode())
    assert st == status
    assert os.listdir(tmp_path) == []


def test_architecture_without_the_conversions_reports_the_compiler_log(tmp_path):
    # gfx942 has no scaled FP8 -> bf16 conversion: the compiler refuses, and says why
    st = qws.lib().qws_rtc_compile_head_fp8(1, 100, 64, b"gfx942", str(tmp_path).encode())
    assert st == _lib.QWS_ERR_COMPILE
    msg = qws.lib().qws_strerror(st).decode()
    assert "compilation failed" in msg and "cvt_scalef32_pk_bf16_fp8" in msg
    assert os.listdir(tmp_path) == []


def test_full_architecture_name_is_its_own_key(tmp_path):
    qws.rtc_compile_head_fp8(1, 100, 64, "gfx950:sramecc+:xnack-", str(tmp_path))
    assert os.listdir(tmp_path)[0].startswith("head_fp8_m1_r100_c64_gfx950_sramecc__xnack-_")
