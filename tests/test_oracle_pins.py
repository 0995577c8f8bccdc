"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins


def test_oracle_battery(oracle):
    results = oracle_pins.battery(oracle)
    failed = [(n, d) for n, ok, d in results if not ok]
    assert not failed, failed
    assert len(results) >= 15


def test_page_block_sizes():
    """Q8_0 is 32 codes + one binary16 scale = 34 bytes; NVFP4 keeps one scale per
    16 weights in 64-weight blocks (page facts fixture)."""
    f = oracle_pins.page_facts()
    assert f["q8_0_block"]["values_per_block"] * 1 + 2 == f["q8_0_block"]["bytes_per_block"]
    nv = f["nvfp4_block"]
    assert nv["weights_per_block"] // nv["weights_per_scale"] == 4
    # a 64-weight block: 32 bytes of 4-bit codes + 4 one-byte scales = 36 bytes = 4.5 bits/weight
    assert (nv["weights_per_block"] // 2 + nv["weights_per_block"] // nv["weights_per_scale"]) * 8 / 64 == 4.5
