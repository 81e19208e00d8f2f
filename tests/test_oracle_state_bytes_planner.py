"""Oracle pins: the pages' printed model-state bytes, and the planner by brute force."""
import os
import shlex

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "state_bytes_printed.txt")


def _printed_rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = shlex.split(line)
            stage, psi, n, k, gb, hw = (float(x) for x in parts[:6])
            rows.append((int(stage), psi, n, k, gb, hw, parts[6]))
    return rows


@pytest.mark.parametrize("row", _printed_rows(), ids=lambda r: f"s{r[0]}-psi{r[1]:g}-n{r[2]:g}")
def test_state_bytes_matches_printed(row):
    stage, psi, n, k, gb, hw, cite = row
    got = oracle.state_bytes(stage, psi, n, k) / 1e9
    assert abs(got - gb) <= hw, (got, gb, cite)


def test_state_bytes_stage_structure():
    # With N = 1 every stage holds the full 16 bytes per parameter.
    for s in range(4):
        assert oracle.state_bytes(s, 1e9, 1) == 16e9
    # Large N tends to 4 psi, 2 psi and 0 (the ~4x, ~8x, ~Nx savings of table 10-2).
    big = 1e12
    assert abs(oracle.state_bytes(1, 1.0, big) - 4.0) < 1e-9
    assert abs(oracle.state_bytes(2, 1.0, big) - 2.0) < 1e-9
    assert oracle.state_bytes(3, 1.0, big) < 1e-9
    with pytest.raises(ValueError):
        oracle.state_bytes(4, 1.0, 1.0)


def _owners(p, numels):
    """Brute force: which rank owns each real flat element, by walking the shards."""
    owner = [None] * p.psi
    for r in range(p.world_size):
        for j in range(p.shard):
            e = r * p.shard + j
            if e < p.psi:
                assert owner[e] is None
                owner[e] = r
    return owner


def test_planner_brute_force():
    import random

    rnd = random.Random(7)
    for _ in range(300):
        t = rnd.randint(0, 6)
        numels = [rnd.randint(0, 40) for _ in range(t)]
        psi = sum(numels)
        n = rnd.randint(1, 17)
        align = rnd.choice([1, 2, 8])
        p = oracle.plan(numels, n, align)
        assert p.psi == psi and p.psi_padded == p.shard * n
        # offsets: tensor i starts after all earlier tensors
        run = 0
        for i, k in enumerate(numels):
            assert p.offsets[i] == run
            run += k
        # every real element owned exactly once; the shard is the smallest
        # multiple of align that covers psi with n ranks
        owner = _owners(p, numels)
        assert all(o is not None for o in owner)
        assert p.shard % align == 0 and p.shard * n >= psi
        assert (p.shard - align) * n < psi or p.shard == 0
        # segments of all ranks tile each tensor exactly, in order
        covered = [[False] * k for k in numels]
        for r in range(n):
            pos = 0
            for s in oracle.segments(p, numels, r):
                assert s.shard_begin >= pos
                pos = s.shard_begin + s.length
                for x in range(s.length):
                    e = p.offsets[s.tensor] + s.tensor_begin + x
                    assert owner[e] == r and e == r * p.shard + s.shard_begin + x
                    assert not covered[s.tensor][s.tensor_begin + x]
                    covered[s.tensor][s.tensor_begin + x] = True
            assert pos <= p.shard
        assert all(all(c) for c in covered)
        assert sum(p.real(r) for r in range(n)) == psi


def test_planner_whole_padding_shards():
    # psi = 5, N = 4: shard 2, the last shard is all padding.
    p = oracle.plan([5], 4)
    assert p.shard == 2 and [p.real(r) for r in range(4)] == [2, 2, 1, 0]
    assert oracle.segments(p, [5], 3) == []


def test_planner_workload_geometry():
    import synth

    expect = {  # psi, N, shard
        "tiny": (1_001_003, 4, 250_251),
        "gpt2_1p5b": (1_557_611_200, 64, 24_337_675),
        "flat_7p5b": (7_500_000_000, 64, 117_187_500),
        "llama3_8b": (8_030_261_248, 8, 1_003_782_656),
        "llama2_70b": (68_976_648_192, 64, 1_077_760_128),
    }
    for w in synth.ALL:
        p = oracle.plan(w.numels, w.world_size)
        assert (p.psi, p.world_size, p.shard) == expect[w.name]
    assert len(synth.GPT2.tensors) == 580 and len(synth.LLAMA3_8B.tensors) == 291
    assert len(synth.FLAT75.tensors) == 448 and len(synth.LLAMA2_70B.tensors) == 723
