"""Pins for the synthetic weight generator and the bf16 emulation (CPU only)."""
import math

import numpy as np
import torch

from oracle.weights import splitmix64, generate, weight_table, Dims, OracleWeights, tensor_key
from oracle.bf16 import round_bf16, f64_to_bf16_bits, bf16_bits_to_f64


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567: the first five outputs are the widely
    # published reference values of the generator.
    golden = 0x9E3779B97F4A7C15
    states = np.array([(1234567 + golden * i) % 2 ** 64 for i in range(5)], dtype=np.uint64)
    # splitmix64(x) is the output for state x before the increment, so the
    # i-th output of a generator seeded with s is splitmix64(s + i * golden)
    out = splitmix64(states).tolist()
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_bf16_round_to_nearest_even_by_hand():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0 - 2 ** -7, 0.6, 0.8, 1 / 3])
    expect = [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.0, 0.6015625, 0.80078125, 0.333984375]
    assert round_bf16(vals).tolist() == expect


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ours = f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_generator_is_counter_based_and_in_range():
    n = 5000
    full = generate(7, 0.125, "f32", 42, np.arange(n, dtype=np.uint64))
    picks = np.array([0, 17, 4999, 1234], dtype=np.uint64)
    assert np.array_equal(generate(7, 0.125, "f32", 42, picks), full[picks.astype(int)])
    assert np.all(np.abs(full) <= 0.125) and abs(full.mean()) < 0.01
    # uniform on [-scale, scale): variance scale^2 / 3
    assert abs(full.var() - 0.125 ** 2 / 3) < 0.0005
    # different tensor ids and seeds give different streams
    assert not np.array_equal(full, generate(8, 0.125, "f32", 42, np.arange(n, dtype=np.uint64)))
    assert not np.array_equal(full, generate(7, 0.125, "f32", 43, np.arange(n, dtype=np.uint64)))


def test_generator_first_element_by_hand():
    # One element written out from the definition with Python integers.
    M = 2 ** 64 - 1

    def sm(x):
        z = (x + 0x9E3779B97F4A7C15) & M
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    seed, t, e = 42, 21, 12345
    key = sm(seed ^ (t << 40))
    r = sm((key + e) & M)
    u = (r >> 40) / 2 ** 24
    w = float(np.float32((2 * u - 1) * float(np.float32(1 / math.sqrt(1024)))))
    assert int(tensor_key(t, seed)) == key
    assert generate(t, float(np.float32(1 / math.sqrt(1024))), "f32", seed, np.array([e], dtype=np.uint64))[0] == w


def test_gamma_and_bf16_kinds():
    g = generate(16, 0.0, "gamma", 42, np.arange(4096, dtype=np.uint64))
    assert np.all((g >= 0.75) & (g < 1.25))
    w = generate(17, 1 / 32, "bf16", 42, np.arange(4096, dtype=np.uint64))
    assert np.array_equal(round_bf16(w), w)


def test_weight_table_shapes_and_ids():
    d = Dims(64, 2, 256, 32)
    tab = weight_table(d, 1024)
    ids = [t for t, *_ in tab]
    assert len(ids) == len(set(ids))
    shapes = {name: shape for _, name, shape, _, _ in tab}
    assert shapes["l1.wqkv"] == (192, 64) and shapes["l0.w2"] == (64, 256) and shapes["l0.dist"] == (2, 127)
    w = OracleWeights(d, 1024)
    rows = w.embedding_rows(np.array([3, 1000]))
    t, _, shape, scale, kind = tab[0]
    full_row = generate(t, scale, kind, 42, np.arange(3 * 64, 4 * 64, dtype=np.uint64))
    assert np.array_equal(rows[0], full_row)
