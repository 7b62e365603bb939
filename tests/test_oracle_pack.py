"""Pins for the oracle's packing (CPU only).

Low-nibble-first packing of two 4-bit codes per byte follows the airllm
article §4.2: of each pair of neighbouring codes the even-indexed one takes the
low nibble; negative codes are stored as their 4-bit two's complement."""
import numpy as np
import pytest

from oracle import pack, unpack

pytestmark = pytest.mark.cpu


def test_every_byte_round_trips_unsigned_and_signed():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    for signed in (False, True):
        q = unpack(b, 4, signed)
        assert q.shape == (1, 512)
        assert np.array_equal(pack(q, 4), b)


def test_every_code_pair_lands_in_the_right_nibbles():
    for lo in range(16):
        for hi in range(16):
            q = np.array([[lo, hi]], dtype=np.int16)
            byte = int(pack(q, 4)[0, 0])
            assert byte == lo | (hi << 4)
            # signed view of the same nibbles
            sl = lo - 16 if lo >= 8 else lo
            sh = hi - 16 if hi >= 8 else hi
            assert list(unpack(np.array([[byte]], np.uint8), 4, True)[0]) == [sl, sh]
            assert int(pack(np.array([[sl, sh]], np.int16), 4)[0, 0]) == byte


@pytest.mark.parametrize("k", [0, 1, 2, 7, 8, 9, 31, 62, 63])
def test_element_k_sits_in_nibble_k_mod_8_of_little_endian_word_k_div_8(k):
    q = np.zeros((1, 64), dtype=np.int16)
    q[0, k] = 0xA
    words = pack(q, 4).view("<u4")[0]
    expect = np.zeros(8, dtype=np.uint32)
    expect[k // 8] = np.uint32(0xA) << np.uint32(4 * (k % 8))
    assert np.array_equal(words, expect)


def test_negative_codes_are_twos_complement_nibbles():
    q = np.array([[-7, 7, -1, 0]], dtype=np.int16)
    assert list(pack(q, 4)[0]) == [0x9 | (0x7 << 4), 0xF | (0x0 << 4)]


def test_eight_bit_codes_are_one_per_byte():
    q = np.arange(256, dtype=np.int16).reshape(2, 128)
    p = pack(q, 8)
    assert p.dtype == np.uint8 and np.array_equal(p.astype(np.int16), q)
    assert np.array_equal(unpack(p, 8, False), q)
