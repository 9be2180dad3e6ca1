"""The FP64 oracle against the pins in oracle_pins.py (CPU only)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_k_layout_offsets_match_the_header():
    """include/pakv.h puts K element (page p, KV head g, slot t, dim i) at
    (p * Hkv + g) * 16 * d + (i / 32) * 512 + t * 32 + i % 32. Both the pins'
    own scatter and the oracle's reader must agree with that flat offset."""
    import numpy as np
    rng = np.random.default_rng(3)
    for d in (32, 64, 128):
        P, H = 3, 2
        by_slot = rng.integers(0, 1 << 16, (P, H, 16, d)).astype(np.uint16)
        flat = oracle_pins.to_k_slabs(by_slot).reshape(-1)
        p, g, t, i = np.meshgrid(np.arange(P), np.arange(H), np.arange(16), np.arange(d), indexing="ij")
        off = (p * H + g) * 16 * d + (i // 32) * 512 + t * 32 + i % 32
        assert np.array_equal(flat[off], by_slot), f"pins' K scatter, d={d}"
        k5 = flat.reshape(P, H, d // 32, 16, 32)
        for pp in range(P):
            for tt in range(16):
                row = oracle.k_slot_row(k5, pp, tt)
                assert np.array_equal(row, flat[off[pp, :, tt, :]]), f"oracle K reader, d={d}"
