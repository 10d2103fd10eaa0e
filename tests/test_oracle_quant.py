"""Pins of the MXFP4 oracle to what the format's definition fixes: the E2M1
value set from a generic minifloat decoder, round-to-nearest-even and
saturation by brute force over the value set, the shared-scale rule's
invariants, exactness on representable blocks, the error bound, torch's E8M0
encoding of powers of two, and the block layout along K."""
import math

import numpy as np
import pytest

from oracle import quant as q


def _minifloat(code, ebits=2, mbits=1, bias=1):
    """A generic sign/exponent/mantissa decoder with subnormals, no inf/NaN."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = m / 2 ** mbits * 2.0 ** (1 - bias)
    else:
        v = (1 + m / 2 ** mbits) * 2.0 ** (e - bias)
    return -v if s else v


def test_e2m1_value_set():
    assert [q.e2m1_value(c) for c in range(16)] == [_minifloat(c) for c in range(16)]
    assert sorted(set(abs(v) for v in q.E2M1)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_rounding_against_brute_force():
    # every multiple of 1/64 in [-8, 8] and random values: the nearest value
    # of the set, the even mantissa (even code) on a midpoint, 6 beyond 6
    rng = np.random.default_rng(0)
    ys = np.concatenate([np.arange(-8 * 64, 8 * 64 + 1) / 64.0, rng.uniform(-10, 10, 5000)])
    codes = q.round_e2m1(ys)
    for y, c in zip(ys, codes):
        target = min(abs(y), 6.0)
        dists = [abs(target - abs(q.E2M1[k])) for k in range(8)]
        best = min(dists)
        ties = [k for k in range(8) if dists[k] == best]
        k = ties[0] if len(ties) == 1 else [t for t in ties if t % 2 == 0][0]
        assert int(c) & 7 == k, (y, c)
        assert (int(c) >> 3) == int(np.signbit(y)), (y, c)


def test_midpoints_go_to_the_even_mantissa():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    assert np.array_equal(q.E2M1[q.round_e2m1(mids)], want)
    assert np.array_equal(q.E2M1[q.round_e2m1(-mids)], -want)
    assert np.array_equal(q.E2M1[q.round_e2m1(np.array([6.0, 7.9, 100.0]))], [6.0, 6.0, 6.0])


def test_shared_scale_rule():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 0.02, size=(2000, 32)) * rng.uniform(0.01, 100, size=(2000, 1))
    codes, sc = q.quantize_blocks(x)
    s = sc.astype(np.int64) - 127
    amax = np.abs(x).max(axis=1)
    # the largest magnitude lands in [4, 8) after scaling: floor(log2 amax) - 2
    r = amax / 2.0 ** s
    assert np.all((r >= 4) & (r < 8))
    assert np.array_equal(s, np.floor(np.log2(amax)).astype(np.int64) - 2)
    # the error bound: half a step of the E2M1 grid at that magnitude, except
    # in the saturated band (6, 8)
    y = x / 2.0 ** s[:, None]
    err = np.abs(q.dequantize_blocks(codes, sc) - x) / 2.0 ** s[:, None]
    step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    sat = np.abs(y) > 6
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.allclose(err[sat], np.abs(y[sat]) - 6, atol=1e-12)


def test_representable_blocks_are_exact_and_zero_blocks():
    rng = np.random.default_rng(2)
    for s in (-20, -7, 0, 5):
        codes = rng.integers(0, 16, size=32).astype(np.uint8)
        codes[0] = 7  # a 6 (or -6) fixes the block's scale at s
        x = q.E2M1[codes] * 2.0 ** s
        c2, sc = q.quantize_blocks(x)
        assert int(sc) - 127 == s
        assert np.array_equal(q.dequantize_blocks(c2, sc), x)
    c, sc = q.quantize_blocks(np.zeros(32))
    assert int(sc) == 1 and np.all(q.E2M1[c] == 0)
    c, sc = q.quantize_blocks(np.full(32, 2.0 ** -140))
    assert int(sc) == 1  # clamped to 2^-126


def test_scale_bytes_match_torch_e8m0_on_powers_of_two():
    torch = pytest.importorskip("torch")
    for s in (-126, -30, -7, 0, 1, 60, 127):
        x = np.zeros(32)
        x[3] = 6.0 * 2.0 ** s if s + 2 <= 127 else 2.0 ** 127
        _, sc = q.quantize_blocks(x)
        ref = torch.tensor([2.0 ** (int(sc) - 127)], dtype=torch.float64).to(torch.float8_e8m0fnu)
        assert int(ref.view(torch.uint8)[0]) == int(sc)


def test_weight_blocks_run_along_k_per_column():
    rng = np.random.default_rng(3)
    K, N = 96, 5
    w = rng.normal(0, 0.02, size=(K, N))
    codes, sc = q.quantize_weight(w)
    assert codes.shape == (K, N) and sc.shape == (K // 32, N)
    for kb in range(K // 32):
        for n in range(N):
            c2, s2 = q.quantize_blocks(w[kb * 32:(kb + 1) * 32, n])
            assert np.array_equal(codes[kb * 32:(kb + 1) * 32, n], c2) and s2 == sc[kb, n]
    # changing one weight moves only its own block
    w2 = w.copy()
    w2[40, 2] *= 50
    c3, s3 = q.quantize_weight(w2)
    diff = np.argwhere((c3 != codes))
    assert set(map(tuple, diff)) <= {(k, 2) for k in range(32, 64)}
    assert np.array_equal(np.argwhere(s3 != sc), [[1, 2]])
    deq = q.mxfp4_weight(w)
    assert np.max(np.abs(deq - w)) <= np.max(np.abs(w)) / 4  # coarse sanity of the 4-bit grid


def test_oracle_weights_use_the_dequantised_experts():
    import dataclasses

    from oracle.inputs import weights_for
    from synth import C1, configs, gen

    m = dataclasses.replace(C1.model, dtype="bf16", expert_format="mxfp4", n_layers=1, global_layer_mask=1)
    w = dataclasses.replace(C1, model=m, seed=5)
    lw = weights_for(w).layer(0)
    raw = gen.layer_weights(w, 0)
    from oracle.model import bf16_bits_to_f64
    for e in (0, 7, 15):
        for k in ("w_gate", "w_up", "w_down"):
            assert np.array_equal(lw[k][e], q.mxfp4_weight(bf16_bits_to_f64(raw[k][e])))
    for k in ("sh_gate", "sh_up", "sh_down"):
        assert np.array_equal(lw[k], q.mxfp4_weight(bf16_bits_to_f64(raw[k])))
    # dense projections are not quantised
    assert np.array_equal(lw["wq"], bf16_bits_to_f64(raw["wq"]))
    native = weights_for(dataclasses.replace(w, model=dataclasses.replace(m, expert_format="native"))).layer(0)
    assert not np.array_equal(native["w_gate"][0], lw["w_gate"][0])
