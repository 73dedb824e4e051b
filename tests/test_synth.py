"""Seeded input generator: Philox4x32-10 known-answer vectors, bf16 rounding, moments."""
import numpy as np
import pytest

import synth

# Known-answer vectors of Philox4x32-10 published with the Random123 library
# (Salmon et al., SC'11): (counter, key) -> output.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert tuple(synth.philox4x32_10(ctr, key)) == want


def test_bf16_round_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0], dtype=np.float32)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0 (0x3F80)
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6 (0x3F82)
    # 1+2^-9 rounds down to 1.0; -2.5 = 0xC020 exactly; 0 -> 0
    assert synth.f32_to_bf16(vals).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x0000]


def test_normal_moments_and_determinism():
    z = synth.normal_f32(7, 1, 0, 0, (1 << 20,))
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert abs((z ** 4).mean() - 3.0) < 0.05
    z2 = synth.normal_f32(7, 1, 0, 0, (1 << 20,))
    assert np.array_equal(z, z2)
    # prefix property: a shorter request is a prefix of a longer one
    z3 = synth.normal_f32(7, 1, 0, 0, (1001,))
    assert np.array_equal(z3, z[:1001])
    # a different stream or counter word gives different numbers
    assert not np.array_equal(synth.normal_f32(7, 2, 0, 0, (64,)), z[:64])
    assert not np.array_equal(synth.normal_f32(7, 1, 1, 0, (64,)), z[:64])


def test_block_params_recipe():
    params = synth.block_params(0, 0, 256)
    names = [n for n, _, _ in params]
    assert names[0] == "adaln.weight" and names[-1] == "mlp.fc2.bias" and len(names) == 16
    bf = sum(a.size for _, dt, a in params if dt == "bf16")
    f32 = sum(a.size for _, dt, a in params if dt == "f32")
    assert bf == 18 * 256 * 256 and f32 == 19 * 256 + 2
    d = dict((n, a) for n, _, a in params)
    assert d["norm1.eps"][0] == np.float32(1e-6)
    assert abs(d["norm1.weight"].mean() - 1.0) < 0.01
    w = (d["attn.qkv.weight"].astype(np.uint32) << 16).view(np.float32)
    assert abs(w.std() - 0.02) < 1e-3
