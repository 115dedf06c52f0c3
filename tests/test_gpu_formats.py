"""GPU parity of the format routines: the startup self-check, MXFP4 dequantisation through both
device paths (bit-exact), and the online FP8 quantiser (codes and scales bit-exact) on every
finite bf16 value, on tiny and zero rows, and on rows drawn like the LM head."""
import numpy as np
import pytest
import torch

import quantized_weight_streaming_amd as qws
import synth
from oracle import formats as OF
from oracle import lmhead as OL

from .helpers import bf16, say, u8

pytestmark = pytest.mark.gpu


def test_selfcheck():
    say("selfcheck")
    qws.selfcheck()


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("rows,cols", [(7, 32), (33, 96), (300, 2560), (1536, 768)])
def test_mxfp4_dequant_bit_exact(path, rows, cols):
    say("mxfp4 dequant", path, rows, cols)
    rng = np.random.default_rng(rows * 7 + cols + path)
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    s = rng.integers(2, 253, (rows, cols // 32), dtype=np.uint8)  # the exact range 2..252
    got = qws.debug_dequant_mxfp4(u8(q), u8(s), path).cpu().numpy()
    want = OF.mxfp4_dequant(q, s).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))  # includes -0.0


def test_mxfp4_dequant_config_scales_both_paths_agree():
    say("mxfp4 dequant config scales")
    q = synth.uniform_bytes_np(synth.hash_key(0, 0, synth.GU_Q, 3), 1536 * 1280).reshape(1536, 1280)
    s = synth.scale_bytes_np(synth.hash_key(0, 0, synth.GU_S, 3), 1536 * 80).reshape(1536, 80)
    a = qws.debug_dequant_mxfp4(u8(q), u8(s), 0).cpu().numpy()
    b = qws.debug_dequant_mxfp4(u8(q), u8(s), 1).cpu().numpy()
    want = OF.mxfp4_dequant(q, s).astype(np.float32)
    assert np.array_equal(a.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(b.view(np.uint32), want.view(np.uint32))


def _all_finite_bf16_rows(cols: int) -> np.ndarray:
    u = np.arange(65536, dtype=np.uint32)
    v = (u << np.uint32(16)).view(np.float32)
    bits = u[np.isfinite(v)].astype(np.uint16)
    rng = np.random.default_rng(0)
    bits = rng.permutation(bits)
    n = (bits.size + cols - 1) // cols * cols
    bits = np.concatenate([bits, bits[: n - bits.size]])
    return bits.reshape(-1, cols)


def _quant_case(w_bits: np.ndarray, what: str):
    say("fp8 quantize", what, w_bits.shape)
    head = qws.lmhead_quantize_fp8(bf16(w_bits))
    torch.cuda.synchronize()
    codes = qws.fp8_codes_rowmajor(head).cpu().numpy()
    scales = head.row_scale.cpu().numpy()
    rc, rs = OL.fp8_rowquant(w_bits)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32)), f"{what}: scales differ"
    bad = np.nonzero(codes != rc)
    assert bad[0].size == 0, f"{what}: {bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}: gpu {codes[bad][0]:#x} oracle {rc[bad][0]:#x}"
    deq = qws.debug_dequant_fp8(head).cpu().numpy()
    assert np.array_equal(deq.view(np.uint32), OL.fp8_dequant(rc, rs).view(np.uint32)), f"{what}: dequant differs"


def test_quantize_every_finite_bf16():
    _quant_case(_all_finite_bf16_rows(2560), "every finite bf16")


def test_quantize_narrow_rows_exercise_subnormal_codes():
    # rows spanning a few binades put many values into the E4M3 subnormal range
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((512, 256)) * np.exp2(rng.integers(-12, 3, (512, 1)) + rng.uniform(-9, 0, (512, 256))))
    _quant_case(synth.f32_to_bf16_bits(v.astype(np.float32)), "subnormal-heavy")


def test_quantize_zero_and_tiny_rows():
    w = np.zeros((6, 64), dtype=np.uint16)
    w[1, 3] = 0x0001                                            # smallest bf16 subnormal
    w[2, :] = 0x8000                                            # all -0.0
    w[3, 7] = 0x0080                                            # smallest bf16 normal
    w[4] = synth.f32_to_bf16_bits(np.linspace(-3e-38, 3e-38, 64).astype(np.float32))
    w[5] = synth.f32_to_bf16_bits(np.linspace(-1e30, 1e30, 64).astype(np.float32))
    _quant_case(w, "zero/tiny rows")


@pytest.mark.parametrize("rows,cols", [(1, 32), (1001, 96), (4097, 2560)])
def test_quantize_head_like_rows(rows, cols):
    _quant_case(synth.bf16_normal(5, 0, synth.HEAD, rows, (rows, cols), 0.02), f"head-like {rows}x{cols}")


def test_probe_read_checksum():
    say("probe read")
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2**32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(a.view(np.int32)).cuda()
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    qws.probe_read(buf, sink, 64)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(a)


@pytest.mark.parametrize("n_words,blocks", [(1 << 20, 64), (4 * 1000 + 12, 7), (8, 5)])
def test_probe_read_nt_checksum_per_share(n_words, blocks):
    """Workgroup b's word is the XOR of its contiguous share of 16-byte words (empty shares: 0)."""
    say(f"probe read nt words={n_words} blocks={blocks}")
    rng = np.random.default_rng(4)
    a = rng.integers(0, 2**32, n_words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(a.view(np.int32)).cuda()
    sink = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    qws.probe_read_nt(buf, sink, blocks)
    torch.cuda.synchronize()
    n16 = n_words // 4
    per = -(-n16 // blocks)
    want = [np.bitwise_xor.reduce(a[4 * min(b * per, n16):4 * min((b + 1) * per, n16)]) if b * per < n16 else 0
            for b in range(blocks)]
    assert [int(v) for v in sink.cpu().numpy().view(np.uint32)] == [int(w) for w in want]
