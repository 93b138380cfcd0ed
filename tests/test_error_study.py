"""CPU checks of the oracle-side error study (no GPU).

Pins: the SNR of uniform quantization of uniform data has a closed form
(signal power 1/3 against step^2/12, i.e. 20 log10(2 qmax) for the symmetric
and 20 log10(2^b - 1) for the asymmetric quantizer over [-1, 1]); the "量化"
chapter's statements in its "动手观察" panel (an fp16 scale per group of 8 costs
2 bits per weight; "4-bit" at groups of 32 is 4.5 bits and 3.56x smaller than
fp16; with a whole-tensor scale and outlier channels the SNR collapses and
smaller groups recover it) and its "亲手实现" paragraph (dequantizing into a
separate fp16 buffer moves more bytes than not quantizing at all).
"""
import numpy as np
import pytest

from oracle import error_study as E
from oracle import gq_oracle as O


@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("bits", [4, 6, 8])
def test_uniform_data_matches_closed_form(sym, bits):
    w = np.random.default_rng(3).uniform(-1.0, 1.0, size=(64, 4096))
    qmax = 2 ** (bits - 1) - 1 if sym else 2 ** bits - 1
    theory = 20 * np.log10(2 * qmax) if sym else 20 * np.log10(qmax)
    snr = O.snr_db(w, E.quant_dequant(w, bits, "tensor", sym))
    assert abs(snr - theory) < 0.1, (snr, theory)


@pytest.fixture(scope="module")
def study():
    w, cols = E.study_matrix()
    return w, cols


@pytest.mark.parametrize("sym", [True, False])
def test_snr_grows_with_bits_and_finer_groups(study, sym):
    w, _ = study
    t = E.snr_table(w, sym)
    for G in E.GROUPS:
        s = [t[(b, G)] for b in E.BITS]
        assert all(a < b for a, b in zip(s, s[1:])), (G, s)
    for b in E.BITS:
        s = [t[(b, G)] for G in E.GROUPS]  # groups of 8, 32, 128, a row, the tensor
        assert all(a > b for a, b in zip(s, s[1:])), (b, s)
    # roughly 6 dB per bit between 4 and 8 bits at groups of 32
    assert 4.5 < (t[(8, 32)] - t[(4, 32)]) / 4 < 6.5


def test_outliers_collapse_a_tensor_scale_and_groups_recover(study):
    w, cols = study
    e = E.outlier_experiment(w, cols, bits=4, symmetric=True)
    # with one scale for the tensor the regular weights fall onto level 0
    assert e["coarse"]["regular"] < 1.0
    # groups of 32 bring them back by more than the chapter's ~13 dB
    assert e["fine"]["regular"] - e["coarse"]["regular"] > 13.0
    assert e["fine"]["all"] - e["coarse"]["all"] > 13.0


def test_metadata_tax_and_compression():
    # fp16 scale per group of 8: 2 extra bits per 4-bit weight (a 50 % tax)
    assert E.effective_bits(4, 8, True) - 4 == 2.0
    # groups of 32: 4.5 bits per weight, 16 / 4.5 = 3.56x smaller than fp16
    assert E.effective_bits(4, 32, True) == 4.5
    assert round(16 / E.effective_bits(4, 32, True), 2) == 3.56
    # a zero point doubles the metadata
    assert E.effective_bits(4, 128, False) == 4.25


def test_per_group_beats_per_channel_at_equal_budget(study):
    w, _ = study
    rows = {label: (eb, snr) for label, eb, snr in E.budget_comparison(w)}
    ch5, g16 = rows["per-channel 5-bit"], rows["per-group 4-bit G=16"]
    assert abs(ch5[0] - g16[0]) < 0.01        # the same bits per weight
    assert g16[1] > ch5[1] + 6.0              # outlier input channels sit in every row


def test_unfused_moves_more_bytes_than_fp16():
    for n, k in ((6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)):
        b = E.traffic(n, k, 128)
        assert b["fused"] < b["fp16"] < b["unfused"]
        assert round(b["fp16"] / b["fused"], 2) in (3.76,)
        assert 2.2 < b["unfused"] / b["fp16"] < 2.3
    # the decode byte counts of the qkv projection at asym g128
    b = E.traffic(6144, 4096, 128)
    assert b["fused"] == 13_389_824 and b["fp16"] == 50_352_128
