"""The seeded input generator: Philox4x64-10 from its published definition
(checked against NumPy's own Philox) and the Irwin-Hall(12) transform."""
import numpy as np

import tmoe_inputs as ti

M64 = (1 << 64) - 1
# Philox4x64 constants (Salmon et al., SC'11, "Parallel random numbers: as easy as 1, 2, 3")
PM0, PM1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
PW0, PW1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def _philox4x64_10(ctr, key):
    c = list(ctr)
    k0, k1 = key
    for _ in range(10):
        p0, p1 = PM0 * c[0], PM1 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & M64, (p0 >> 64) ^ c[3] ^ k1, p0 & M64]
        k0, k1 = (k0 + PW0) & M64, (k1 + PW1) & M64
    return c


def test_philox_counter_layout():
    for stream, first in [(1, 0), (77, 5), (ti.stream_id(5, 23, 255, 2), 1 << 20)]:
        words = ti.philox_words(stream, first, 3)
        for i in range(3):
            assert [int(v) for v in words[i]] == _philox4x64_10([first + i, stream, 0, 0], [ti.KEY, 0])


def test_ih12_definition_and_moments():
    stream = ti.stream_id(2, 0, 3, 1)
    w = ti.ih12_normal(stream, 4096, first=100)
    words = ti.philox_words(stream, 100, 4096)
    for i in (0, 1, 4095):
        u = []
        for j in range(3):
            u += [(int(words[i, j]) >> (16 * m)) & 0xFFFF for m in range(4)]
        assert w[i] == np.float32((sum(u) - 393210) * 2.0 ** -16)
    big = ti.ih12_normal(1, 1 << 20)
    assert abs(big.mean()) < 5e-3 and abs(big.std() - 1) < 5e-3
    assert np.all(np.abs(big) < 6)
    # every draw is an integer multiple of 2^-16, hence exact in fp32 and in any fp64 sum
    assert np.all((big.astype(np.float64) * 65536) % 1 == 0)


def test_streams_distinct():
    ids = {ti.stream_id(c, l, e, m) for c in (1, 5) for l in (0, 23) for e in (0, 255, 1023) for m in range(4)}
    assert len(ids) == 2 * 2 * 3 * 4


def test_bias_recipes():
    z = ti.router_bias(3, "zipf")
    assert sorted(np.round(np.exp(-z / 1.1)).astype(int).tolist()) == list(range(1, 257))
    u = ti.router_bias(4, "uniform")
    assert u.shape == (256,) and np.all(np.abs(u) <= 0.1)
    assert ti.router_bias(2, None) is None


def test_activation_bits():
    x = ti.activations(2, 3)
    assert x.dtype == np.uint16 and x.shape == (3, 2048)
    f = ti.bf16_bits_to_f32(x)
    assert abs(float(f.std()) - 1) < 0.05
