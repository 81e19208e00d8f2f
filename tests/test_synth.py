"""The seeded input generator: published Philox vectors, addressability, distribution."""
import math

import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library (Salmon et al., SC'11).
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, out in kat:
        assert synth.philox4x32_10(ctr, key) == out


def test_ranges_are_addressable_and_deterministic():
    w = synth.LLAMA3_8B
    whole = synth.contributions(w, 1, 3, 1000, 5000, 65536.0)
    part = synth.contributions(w, 1, 3, 1003, 777, 65536.0)
    assert np.array_equal(whole[3:780], part)
    mw = synth.masters(w, 17, 4000)
    assert np.array_equal(mw[100:200], synth.masters(w, 117, 100))
    # different rank, step or purpose -> different stream
    assert not np.array_equal(whole, synth.contributions(w, 1, 4, 1000, 5000, 65536.0))
    assert not np.array_equal(whole, synth.contributions(w, 2, 3, 1000, 5000, 65536.0))


def test_padding_is_zero():
    w = synth.TINY
    c = synth.contributions(w, 1, 0, w.psi - 5, 10, 1024.0)
    assert c[5:].tolist() == [0] * 5 and np.count_nonzero(c[:5]) > 0
    mm = synth.masters(w, w.psi - 2, 4)
    assert mm[2:].tolist() == [0.0, 0.0]


def test_fp16_table_is_the_discretised_normal():
    std = 65.536
    thr, val, guide = synth.fp16_normal_table(std)
    assert thr[-1] == 2**32 and (np.diff(thr.astype(np.int64)) >= 0).all()
    h = val.view(np.float16).astype(np.float64)
    # values ascend (with -0 just before +0)
    assert (np.diff(h) >= 0).all()
    # the mass of [-std, std) is about 68.27 %
    lo = np.searchsorted(h, -std)
    hi = np.searchsorted(h, std)
    mass = (int(thr[hi - 1]) - int(thr[lo - 1])) / 2**32
    assert abs(mass - math.erf(1 / math.sqrt(2))) < 1e-3


def test_sample_moments():
    w = synth.GPT2
    x = synth.contributions(w, 1, 0, 0, 1 << 21, 65536.0).view(np.float16).astype(np.float64)
    s = w.sigma * 65536.0
    assert abs(x.mean()) < 4 * s / math.sqrt(x.size)
    assert abs(x.std() / s - 1) < 0.005
    mm = synth.masters(w, 0, 1 << 21).astype(np.float64)
    assert abs(mm.std() / w.master_sigma - 1) < 0.005 and abs(mm.mean()) < 1e-4


def test_injection_site():
    w = synth.LLAMA3_8B
    assert synth.inject_site(w, 1) is None
    q, e = synth.inject_site(w, 2)
    assert 0 <= q < w.world_size and 0 <= e < w.psi // w.world_size
    c = synth.contributions(w, 2, q, e - 2, 5, 32768.0)
    assert c[2] == 0x7C00
