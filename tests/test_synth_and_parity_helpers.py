"""Generators are deterministic; the tolerance helper behaves as documented."""
import os
import sys

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_synth_hashes  # noqa: E402
import parity  # noqa: E402


def test_generator_hashes_stable():
    want = {}
    with open(os.path.join(HERE, "golden", "synth_sha256.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            i, k, v = line.split()
            want[(int(i), k)] = v
    for i in (0, 1):
        for k, v in make_synth_hashes.digests(i).items():
            assert want[(i, k)] == v, (i, k)


def test_generator_distributions():
    w = synth.workload(0)
    L = w.layers[0]
    assert w.x.dtype == np.uint16 and w.x.shape == (128, 512)
    assert L.gate.codes.shape == (32, 512, 256) and L.gate.scales.shape == (32, 512, 16)
    assert L.down.codes.shape == (32, 512, 256)
    assert L.gate.scales.min() == 121 and L.gate.scales.max() == 124
    nib = np.concatenate([(L.up.codes & 15).ravel(), (L.up.codes >> 4).ravel()])
    assert np.all(np.bincount(nib, minlength=16) > 0.9 * nib.size / 16)
    assert abs(float(np.std(L.w_router)) - 0.02) < 1e-3


def test_bf16_cast_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert synth.bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert synth.bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    assert synth.bf16_bits(np.array([-2.0]))[0] == 0xC000


def test_zipf_bias_is_log_rank():
    w = synth.workload(3, with_layers=False)
    assert w.E == 128 and w.T == 4096


def test_excess_error_rule():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(10000) * 500
    rounded = parity.bf16_out_to_f64(synth.bf16_bits(ref))
    m = parity.error_metrics(rounded, ref)
    assert m["excess"] == 0.0 and m["mean_rel"] < 2e-3
    bad = rounded.copy()
    bad[17] += 0.03 * m["rms"]
    m2 = parity.error_metrics(bad, ref)
    assert m2["excess"] > parity.EXCESS_TOL
