"""Seeded input generators: determinism, formats and distributions."""
import numpy as np

import oracle
from lut_sketched_matmul_amd import synthetic as syn
from lut_sketched_matmul_amd import workloads as wl


def test_deterministic_by_name():
    a = syn.random_packed_indices("x/y/idx", 8, 64, 3)
    b = syn.random_packed_indices("x/y/idx", 8, 64, 3)
    c = syn.random_packed_indices("x/y/idx2", 8, 64, 3)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (8, 64 * 3 // 8) and a.dtype == np.uint8


def test_random_bytes_give_uniform_indices():
    # uniform bytes read as little-endian b-bit fields are uniform in [0, 2^b)
    for b in (2, 3, 4):
        p = syn.random_packed_indices(f"u/{b}", 64, 4096, b)
        idx = oracle.unpack_indices(p, 4096, b)
        counts = np.bincount(idx.ravel(), minlength=1 << b)
        expect = idx.size / (1 << b)
        assert np.all(np.abs(counts - expect) < 6 * np.sqrt(expect))


def test_lut_sorted_and_scaled():
    for dt in ("f32", "f16", "bf16"):
        lut = syn.random_lut(f"l/{dt}", 512, 4, 4, 0.02, dt)
        v = syn.to_float64(lut, dt)
        assert v.shape == (512, 4, 16)
        assert np.all(np.diff(v, axis=-1) >= 0)
        assert abs(v.std() - 0.02) < 0.002


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-3, 3.0e38], dtype=np.float32)
    back = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2**-6)
    assert back[3] == -2.5
    assert abs(back[4] - 1e-3) <= 1e-3 * 2**-8


def test_shape_pins_from_the_pages():
    # SpaLLM, section 3.1 (commonsense results): LLaMA-7B at one group per row
    # trains about 22 million parameters. 32 layers x (q,k,v,o: 4 x 4096 rows,
    # gate/up: 2 x 11008 rows, down: 4096 rows) x k=16 entries per table.
    rows = 32 * (4 * 4096 + 2 * 11008 + 4096)
    assert rows * 1 * 16 == 21_757_952
    assert abs(rows * 16 - 22e6) / 22e6 < 0.02
    # Sketch to Adapt, reply W2: compression factor c/(g k) >= 32 for LLaMA-2-7B
    w = wl.LLAMA2_7B_ATTN
    assert w.shapes[0].d / (w.gpr * 16) == 32


def test_workloads_well_formed():
    for w in wl.ALL:
        for s in w.shapes:
            assert s.d % w.gpr == 0 and (s.d // w.gpr) % 32 == 0, (w.name, s)
            for b in w.bits:
                assert (s.d * b) % 8 == 0


def test_workload_make_small():
    w = wl.TINY
    t = w.make(w.shapes[0], 4, 4)
    assert t["idx_packed"].shape == (256, 256)
    assert t["lut"].shape == (256, 1, 16) and t["lut"].dtype == np.float32
    assert t["X"].shape == (4, 512) and t["dY"].shape == (4, 256)
