"""Run-time specialisation without a GPU: hipRTC compiles the FP8 head GEMV and the fused MoE
layers for gfx950 from the sources built into the library, the code object lands in the disk cache
under its key, a second request is served from the cache, bad arguments are refused before any
compilation, and the cache is used only as the header states (owner-only directory, regular files
of the user, not through links, code hash checked; no shared default directory)."""
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
    assert blob[:8] == b"QWSRTC2\0" and b"\x7fELF" in blob
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


def test_moe_compile_then_cache_hit(tmp_path):
    d = str(tmp_path / "cache")
    qws.rtc_reset()
    qws.rtc_compile_moe(1, 8, 512, 2560, 768, True, False, "gfx950", d)
    qws.rtc_compile_moe(4, 8, 512, 2560, 768, True, True, "gfx950", d)
    files = sorted(os.listdir(d))
    # one kernel for separate layers and one for chained sequences, per shape
    assert len(files) == 4
    assert files[0].startswith("moe_layers_m1_bf16_e512_h2560_i768_k8_s1_chain_gfx950_")
    assert files[1].startswith("moe_layers_m1_bf16_e512_h2560_i768_k8_s1_gfx950_")
    assert files[2].startswith("moe_layers_m4_w4a8_e512_h2560_i768_k8_s1_chain_gfx950_")
    assert files[3].startswith("moe_layers_m4_w4a8_e512_h2560_i768_k8_s1_gfx950_")
    assert oct(os.stat(d).st_mode & 0o777) == "0o700"
    assert all(os.stat(os.path.join(d, f)).st_mode & 0o077 == 0 for f in files)
    qws.rtc_compile_moe(1, 8, 512, 2560, 768, True, False, "gfx950", d)
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"]) == (4, 2)


@pytest.mark.parametrize("args,status", [
    ((0, 8, 512, 2560, 768, 1, 0), _lib.QWS_ERR_SHAPE), ((5, 8, 512, 2560, 768, 1, 0), _lib.QWS_ERR_SHAPE),
    ((1, 9, 512, 2560, 768, 1, 0), _lib.QWS_ERR_SHAPE), ((1, 8, 4, 2560, 768, 1, 0), _lib.QWS_ERR_SHAPE),
    ((1, 8, 512, 2592, 768, 1, 0), _lib.QWS_ERR_SHAPE), ((1, 8, 512, 2560, 1056, 1, 0), _lib.QWS_ERR_SHAPE),
    ((1, 8, 512, 2560, 770, 1, 0), _lib.QWS_ERR_SHAPE), ((1, 8, 512, 2560, 768, 2, 0), _lib.QWS_ERR_SHAPE),
    ((1, 8, 512, 2560, 768, 1, 2), _lib.QWS_ERR_ARG),
])
def test_moe_compile_validation(tmp_path, args, status):
    assert qws.lib().qws_rtc_compile_moe(*args, b"gfx950", str(tmp_path).encode()) == status
    assert os.listdir(tmp_path) == []


def _one_file(d):
    files = [f for f in os.listdir(d) if f.endswith(".co")]
    assert len(files) == 1
    return os.path.join(d, files[0])


def test_corrupted_code_object_is_recompiled(tmp_path):
    d = str(tmp_path / "cache")
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", d)
    f = _one_file(d)
    blob = bytearray(open(f, "rb").read())
    blob[-100] ^= 0x40                      # one bit of the code object, size unchanged
    open(f, "wb").write(bytes(blob))
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", d)
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"]) == (2, 0)
    assert open(f, "rb").read() != bytes(blob)   # rewritten whole


def test_cache_file_reached_through_a_link_is_not_read(tmp_path):
    d = str(tmp_path / "cache")
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", d)
    f = _one_file(d)
    elsewhere = str(tmp_path / "elsewhere.co")
    os.rename(f, elsewhere)
    os.symlink(elsewhere, f)
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", d)
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"]) == (2, 0)
    assert not os.path.islink(f)             # replaced by a regular file, the link's target untouched


def test_directory_others_may_write_is_not_used(tmp_path):
    d = tmp_path / "shared"
    d.mkdir()
    os.chmod(d, 0o777)
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", str(d))
    qws.rtc_compile_head_fp8(1, 640, 128, "gfx950", str(d))
    s = qws.rtc_stats()
    assert (s["compiles"], s["disk_hits"]) == (2, 0)
    assert os.listdir(d) == []


def test_no_shared_default_directory(tmp_path, monkeypatch):
    """With no cache directory given and none in the environment, nothing is written anywhere
    (there is no fallback under /tmp); with $XDG_CACHE_HOME set, the cache goes there."""
    for v in ("QWS_RTC_CACHE", "XDG_CACHE_HOME", "HOME"):
        monkeypatch.delenv(v, raising=False)
    before = os.path.exists("/tmp/.cache/qws_rtc")
    qws.rtc_reset()
    qws.rtc_compile_head_fp8(1, 640, 96, "gfx950", None)
    qws.rtc_compile_head_fp8(1, 640, 96, "gfx950", None)
    assert qws.rtc_stats()["compiles"] == 2
    assert os.path.exists("/tmp/.cache/qws_rtc") == before
    monkeypatch.setenv("XDG_CACHE_HOME", str(tmp_path / "xdg"))
    qws.rtc_compile_head_fp8(1, 640, 96, "gfx950", None)
    assert len(os.listdir(tmp_path / "xdg" / "qws_rtc")) == 1
