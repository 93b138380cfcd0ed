"""Oracle-side quantization error study.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: it calls nothing but the
oracle's own quantizer and the seeded input generator, and the product path
never imports it.  ``python -m oracle.error_study`` prints the tables.

It recreates the experiments the "量化" chapter (S08) describes in its
"动手观察" panel and its "在本地运行" / exercise paragraphs:

* signal-to-noise ratio of group-wise quantization over bit width x group size
  (2, 3, 4, 8 bits; groups of 8, 32, 128, one per output row, one per tensor);
* the outlier experiment: with a whole-tensor scale two outlier channels
  stretch the range and the other weights collapse onto a few levels; with
  groups of 32 only the outliers' groups suffer;
* the metadata tax: an fp16 scale per group of G weights adds 16/G bits per
  weight (2 bits at G = 8, so "4-bit" at G = 32 is 4.5 bits, 3.56x smaller
  than fp16); an fp16 zero point doubles it;
* per-channel (one scale per output row) against per-group scales at the same
  bits per weight;
* the bytes a decode-time matmul moves when the weight is dequantized into a
  separate fp16 buffer first, against the fused kernel and against fp16.

SNR is 10 log10(sum w^2 / sum (w^ - w)^2) over the weights considered.
"""
from __future__ import annotations

import numpy as np

from oracle import gq_oracle as O

GROUPS = (8, 32, 128, "row", "tensor")
BITS = (2, 3, 4, 8)


def group_elems(G, n: int, k: int) -> int:
    """Weights per scale: an integer group, a whole output row, or the tensor."""
    if G == "row":
        return k
    if G == "tensor":
        return n * k
    return int(G)


def quant_dequant(w: np.ndarray, bits: int, G, symmetric: bool) -> np.ndarray:
    """Quantize and dequantize ``w`` [N, K] with the oracle's quantizer.  Groups
    run along K; "row" is one group per output row (per-channel), "tensor" one
    group for the whole matrix (the row-major flattening)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if G == "tensor":
        flat = w.reshape(1, n * k)
        c, s, z = O.quantize_groups(flat, bits, n * k, symmetric)
        return O.dequantize_codes(c, s, z, n * k).reshape(n, k)
    g = group_elems(G, n, k)
    c, s, z = O.quantize_groups(w, bits, g, symmetric)
    return O.dequantize_codes(c, s, z, g)


def effective_bits(bits: int, G, symmetric: bool, n: int = 1, k: int = 1) -> float:
    """Code bits plus the per-weight share of the fp16 scale (and zero)."""
    meta = 16 if symmetric else 32
    return bits + meta / group_elems(G, n, k)


def snr_table(w: np.ndarray, symmetric: bool, bits=BITS, groups=GROUPS):
    """{(bits, G): SNR dB} over the whole matrix."""
    return {(b, G): O.snr_db(w, quant_dequant(w, b, G, symmetric)) for b in bits for G in groups}


def outlier_experiment(w: np.ndarray, outlier_cols, bits: int = 4, symmetric: bool = True,
                       coarse="tensor", fine=32):
    """SNR over all weights, over the non-outlier weights and over the outlier
    weights, for a coarse (whole-tensor) and a fine (group) scale."""
    w = np.asarray(w, dtype=np.float64)
    mask = np.zeros(w.shape, dtype=bool)
    mask[:, np.asarray(outlier_cols, dtype=np.int64)] = True
    out = {}
    for name, G in (("coarse", coarse), ("fine", fine)):
        wh = quant_dequant(w, bits, G, symmetric)
        out[name] = {
            "all": O.snr_db(w, wh),
            "regular": O.snr_db(w[~mask], wh[~mask]),
            "outliers": O.snr_db(w[mask], wh[mask]) if mask.any() else float("nan"),
        }
    return out


def budget_comparison(w: np.ndarray, symmetric: bool = True):
    """Per-channel against per-group scales at (nearly) equal bits per weight:
    (scheme, bits/weight, SNR).  At ~5 bits: 5-bit per-channel against 4-bit
    groups of 16 (16/16 = 1 bit of scale); at ~4.5: 4-bit per-channel plus
    nothing to spend against 4-bit groups of 32."""
    n, k = w.shape
    rows = []
    for label, b, G in (("per-channel 4-bit", 4, "row"), ("per-group 4-bit G=32", 4, 32),
                        ("per-channel 5-bit", 5, "row"), ("per-group 4-bit G=16", 4, 16)):
        rows.append((label, effective_bits(b, G, symmetric, n, k),
                     O.snr_db(w, quant_dequant(w, b, G, symmetric))))
    return rows


def traffic(n: int, k: int, G: int, m: int = 1, symmetric: bool = False):
    """Bytes one M-row matmul moves: fused W4A16 (packed codes + metadata read
    once), unfused (that read, plus writing and re-reading an fp16 weight), and
    an fp16 weight; activations and outputs are 2-byte in all three."""
    q, s, z = O.packed_sizes(n, k, G, symmetric)
    io = 2 * m * k + 2 * m * n
    fused = q + s + z + io
    fp16 = 2 * n * k + io
    unfused = q + s + z + 2 * n * k + 2 * n * k + io
    return {"fused": fused, "unfused": unfused, "fp16": fp16}


def study_matrix(seed: int = 5, n: int = 256, k: int = 2048):
    """The synthetic weight matrix of the study: N(0, 0.02) with 0.1 % of the
    input channels (two) scaled by 20, as the bench's decode weights."""
    import synth
    bits, cols = synth.weights(n, k, seed=seed, outlier_frac=2.0 / k)
    return O.bf16_to_f64(bits), cols


def main() -> None:
    w, cols = study_matrix()
    n, k = w.shape
    for sym in (True, False):
        t = snr_table(w, sym)
        print(f"\nSNR dB, {'symmetric (scale)' if sym else 'asymmetric (scale + zero)'}, "
              f"[{n}, {k}] N(0, 0.02) with 2 input channels x20")
        print("| bits | " + " | ".join(f"G={g}" for g in GROUPS) + " |")
        print("|---" * (len(GROUPS) + 1) + "|")
        for b in BITS:
            print(f"| {b} | " + " | ".join(f"{t[(b, g)]:.1f}" for g in GROUPS) + " |")
        print("bits/weight at 4-bit: " + ", ".join(
            f"G={g}: {effective_bits(4, g, sym, n, k):.3f}" for g in GROUPS))
    e = outlier_experiment(w, cols)
    print("\noutlier experiment, 4-bit symmetric: whole-tensor scale -> groups of 32")
    for part in ("all", "regular", "outliers"):
        print(f"  {part:9s} {e['coarse'][part]:6.1f} dB -> {e['fine'][part]:6.1f} dB "
              f"({e['fine'][part] - e['coarse'][part]:+.1f})")
    print("\nper-channel vs per-group at equal bits per weight (symmetric)")
    for label, eb, snr in budget_comparison(w):
        print(f"  {label:22s} {eb:6.3f} bits/weight  {snr:6.1f} dB")
    print("\nbytes of one M=1 product, asym g128 (Llama-3-8B projections)")
    for name, (nn, kk) in (("qkv", (6144, 4096)), ("o", (4096, 4096)),
                           ("gate_up", (28672, 4096)), ("down", (4096, 14336))):
        b = traffic(nn, kk, 128)
        print(f"  {name:8s} fused {b['fused']:>11,}  unfused {b['unfused']:>11,}  fp16 {b['fp16']:>11,}  "
              f"unfused/fp16 {b['unfused'] / b['fp16']:.2f}  fp16/fused {b['fp16'] / b['fused']:.2f}")


if __name__ == "__main__":
    main()
