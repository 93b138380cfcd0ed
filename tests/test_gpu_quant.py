"""GPU parity of quantize / pack / dequantize: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import announce, bf16_dev, bits16, device, f16_dev, u8_dev
from oracle import gq_oracle as O
from w4a16_dequant_gemm_group_amd import binding as B
import synth

pytestmark = pytest.mark.gpu


def _to_dev(w_f64: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return bf16_dev(synth.f32_to_bf16_bits(w_f64.astype(np.float32)))
    if dtype == "f16":
        return f16_dev(w_f64.astype(np.float16).view(np.uint16))
    return torch.from_numpy(w_f64.astype(np.float32)).to(device())


def _input_values(w_dev: torch.Tensor) -> np.ndarray:
    """The exact input values the oracle sees (as float64)."""
    return w_dev.float().cpu().numpy().astype(np.float64)


def _check_quant(w_dev, bits, G, sym, what):
    announce(what)
    codes, scales, zeros = B.gq_quantize_groups(w_dev, bits, G, sym)
    torch.cuda.synchronize()
    c_ref, s_ref, z_ref = O.quantize_groups(_input_values(w_dev), bits, G, sym)
    got_c = codes.cpu().numpy().astype(np.int64)
    assert np.array_equal(got_c, c_ref), f"{what}: codes differ at {np.argwhere(got_c != c_ref)[:5]}"
    assert np.array_equal(bits16(scales), O.f64_to_f16_bits(s_ref)), f"{what}: scales differ"
    if not sym:
        assert np.array_equal(bits16(zeros), O.f64_to_f16_bits(z_ref)), f"{what}: zeros differ"
    else:
        assert zeros is None
    return codes, scales, zeros


def test_tiny_reference_case():
    w, _ = synth.tiny_reference()
    wd = bf16_dev(w)
    for G in (128, 512):
        _check_quant(wd, 4, G, False, f"tiny [256,512] asym G={G}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("sym", [False, True])
def test_bits_and_dtypes(dtype, sym):
    rng = np.random.default_rng(40 + sym)
    for bits in range(2, 9):
        for G in (32, 64):
            w = rng.normal(0, 0.05, size=(33, 256))
            w[:, 5] *= 20
            _check_quant(_to_dev(w, dtype), bits, G, sym, f"{dtype} sym={sym} bits={bits} G={G}")


def test_edge_groups():
    rng = np.random.default_rng(9)
    w = rng.normal(0, 1.0, size=(8, 256))
    w[0, :32] = 0.0                      # all-zero group -> scale 1
    w[1, :32] = np.abs(w[1, :32])        # all-positive -> zero point 0
    w[2, :32] = -np.abs(w[2, :32])       # all-negative -> zero point 15
    w[3, :32] = 0.37                     # constant
    w[4, :32] *= 1e-9                    # scale below fp16 range -> 2^-24
    w[5, :32] *= 1e-5                    # fp16 subnormal scales
    w[6, :32] *= 3e6                     # beyond fp16 range -> 65504
    w[7, ::2] = 0.0
    for sym in (False, True):
        _check_quant(_to_dev(w, "f32"), 4, 32, sym, f"edge groups f32 sym={sym}")
        _check_quant(_to_dev(np.clip(w, -6e4, 6e4), "bf16"), 4, 32, sym, f"edge groups bf16 sym={sym}")


def test_pack_and_dequant_bit_exact():
    w, _ = synth.weights(96, 512, seed=77)
    for sym, G in ((False, 128), (True, 32), (False, 64), (False, 512)):
        announce(f"pack/dequant sym={sym} G={G}")
        codes_ref, s_bits, z_bits = O.quantize_to_storage(w, 4, G, sym)
        qw_ref = O.pack_int4(codes_ref, sym)
        codes_dev = torch.from_numpy(codes_ref.astype(np.int8 if sym else np.uint8)).to(device())
        qw = B.gq_pack_int4(codes_dev, sym)
        assert np.array_equal(qw.cpu().numpy(), qw_ref)
        wh_ref = O.dequantize_packed(qw_ref, s_bits, z_bits, G, sym)
        sd, zd = f16_dev(s_bits), (None if sym else f16_dev(z_bits))
        out32 = B.gq_dequantize(u8_dev(qw_ref), sd, zd, G, sym, torch.float32)
        assert np.array_equal(out32.cpu().numpy().astype(np.float64), wh_ref)
        outb = B.gq_dequantize(u8_dev(qw_ref), sd, zd, G, sym, torch.bfloat16)
        assert np.array_equal(bits16(outb), O.f32_exact_to_bf16_bits(wh_ref))
        outh = B.gq_dequantize(u8_dev(qw_ref), sd, zd, G, sym, torch.float16)
        assert np.array_equal(bits16(outh), O.f64_to_f16_bits(wh_ref))
        # an output 2 bytes off a 16-byte boundary takes the per-byte kernel
        n, k = wh_ref.shape
        buf = torch.empty(n * k + 8, dtype=torch.bfloat16, device=device())
        outm = buf[1:1 + n * k].view(n, k)
        B.gq_dequantize(u8_dev(qw_ref), sd, zd, G, sym, torch.bfloat16, out=outm)
        assert np.array_equal(bits16(outm), O.f32_exact_to_bf16_bits(wh_ref))


def test_full_size_o_projection():
    w, _ = synth.decode_case("o")
    _check_quant(bf16_dev(w), 4, 128, False, "o [4096,4096] asym g128 full")


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_full_size_sampled_rows(name):
    w, _ = synth.decode_case(name)
    wd = bf16_dev(w)
    for sym, G in ((False, 128), (True, 32)):
        announce(f"{name} {w.shape} sym={sym} G={G} sampled rows")
        codes, scales, zeros = B.gq_quantize_groups(wd, 4, G, sym)
        qw = B.gq_pack_int4(codes, sym)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(1).choice(w.shape[0], 256, replace=False))
        c_ref, s_ref, z_ref = O.quantize_to_storage(w[rows], 4, G, sym)
        assert np.array_equal(qw.cpu().numpy()[rows], O.pack_int4(c_ref, sym))
        assert np.array_equal(bits16(scales)[rows], s_ref)
        if not sym:
            assert np.array_equal(bits16(zeros)[rows], z_ref)
