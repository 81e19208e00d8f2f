"""The oracle's pins catch plausible mistakes.

Each mutant below plants one mistake in a copy of the oracle (its numpy
definitions or its C twin), on the CPU, in a scratch copy of the repository's
Python side; the oracle pin tests then run against that copy in a child
process and must fail.  The unmodified copy must pass the same tests, so a
caught mutant means the pins, not the copy, failed.  The numpy mutants run
every oracle pin except the C twin's own test (the twin is checked against the
numpy definitions, so it would not count as an independent pin); the C
mutants run the C twin's test, whose reference is the pinned numpy oracle.

Every mutant names the exact source text it replaces, which must occur once,
so a later edit of the oracle breaks this test loudly instead of leaving a
mutant that no longer applies.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PY = "oracle/zero_oracle.py"
C = "oracle/oracle_c.c"

# (name, file, old text, new text)
MUTANTS = [
    # model-state bytes ("第13篇 · ZeRO" §3.2)
    ("stage-1 optimizer term not divided by N", PY,
     "return 4.0 * psi + k * psi / n", "return 4.0 * psi + k * psi"),
    ("stage-2 gradient term dropped", PY,
     "return 2.0 * psi + (2.0 + k) * psi / n", "return 2.0 * psi + k * psi / n"),
    ("stage-3 parameter term dropped", PY,
     "return (4.0 + k) * psi / n", "return (2.0 + k) * psi / n"),
    # planner
    ("shard = floor(psi / N)", PY,
     "per_rank = -(-psi // world_size)", "per_rank = psi // world_size"),
    ("inclusive segment end", PY,
     "lo, hi = max(a, off), min(b, off + n)", "lo, hi = max(a, off), min(b, off + n + 1)"),
    ("unit rank offsets by unit length, not by shard", PY,
     "        roff += s\n", "        roff += p\n"),
    ("unit shard not rounded up to the alignment", PY,
     "s = -(-(-(-p // world_size)) // align) * align", "s = -(-p // world_size)"),
    ("plan shard not rounded up to the alignment", PY,
     "shard = -(-per_rank // align) * align", "shard = per_rank"),
    ("unit element map one rank off", PY,
     "local = np.arange(s, dtype=np.int64) + rank * s", "local = np.arange(s, dtype=np.int64) + (rank + 1) * s"),
    ("unit lookup takes the unit before a boundary", PY,
     'u = np.searchsorted(offs, pos, side="right") - 1', 'u = np.searchsorted(offs, pos, side="left") - 1'),
    ("padding of a rank's shard counted as real", PY,
     "return max(0, min(self.shard, self.psi - rank * self.shard))", "return self.shard"),
    # host scalars
    ("1 - beta1 rounded as 1f - 0.9f", PY,
     "omb1=F32(1.0 - beta1)", "omb1=F32(F32(1.0) - F32(beta1))"),
    ("no first-moment bias correction", PY,
     "step_size=F32(lr / (1.0 - p1))", "step_size=F32(lr)"),
    ("beta^t off by one", PY,
     "    for _ in range(t - 1):\n", "    for _ in range(t):\n"),
    ("no average over ranks", PY,
     "inv64 = 1.0 / (world_size * loss_scale)", "inv64 = 1.0 / loss_scale"),
    ("weight decay scaled without lr", PY,
     "decay=F32(1.0 - lr * weight_decay)", "decay=F32(1.0 - weight_decay)"),
    # reduce, overflow and exact norm
    ("reversed rank order", PY,
     "    for r in range(c.shape[0]):\n        acc = acc + c[r].astype(F32)",
     "    for r in reversed(range(c.shape[0])):\n        acc = acc + c[r].astype(F32)"),
    ("fp16 contributions summed in fp16", PY,
     "        acc = acc + c[r].astype(F32)", "        acc = (acc.astype(np.float16) + c[r]).astype(F32)"),
    ("overflow check misses inf", PY,
     "return bool(acc.size) and not bool(np.isfinite(acc).all())",
     "return bool(acc.size) and bool(np.isnan(acc).any())"),
    ("cross limb of the exact norm dropped", PY,
     " + (int((2 * h * l).sum()) << 24)", ""),
    # finalize (fp16 path)
    ("clip without the +1e-6", PY,
     "    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)",
     "    coef = min(1.0, max_norm / norm) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)"),
    ("clip coefficient not clamped at 1", PY,
     "    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)",
     "    coef = max_norm / (norm + 1e-6) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)"),
    ("other ranks' overflow ignored", PY,
     "skip = bool(own_overflow or other_overflow or too_big)", "skip = bool(own_overflow or too_big)"),
    ("norm without the square root", PY,
     "    norm = math.sqrt(total_sq)\n    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)",
     "    norm = total_sq\n    coef = min(1.0, max_norm / (norm + 1e-6)) if max_norm > 0 else 1.0\n"
     "    skip = bool(own_overflow or other_overflow or too_big)"),
    ("unscale applied once to the squared norm", PY,
     "total_sq = ((float(q_tot) * 2.0**-48) * inv64) * inv64 + other_sq",
     "total_sq = (float(q_tot) * 2.0**-48) * inv64 + other_sq"),
    ("other ranks' exact share left out", PY,
     "    q_tot = own_q + other_q\n", "    q_tot = own_q\n"),
    # Adam / AdamW
    ("unapplied clip", PY, "    gc = g * F32(coef)\n", "    gc = g\n"),
    ("swapped beta1 terms", PY,
     "m = sc.b1 * m + sc.omb1 * gc", "m = sc.omb1 * m + sc.b1 * gc"),
    ("second moment without the square", PY,
     "v = sc.b2 * v + sc.omb2 * (gc * gc)", "v = sc.b2 * v + sc.omb2 * gc"),
    ("eps inside the square root", PY,
     "den = np.sqrt(v) / sc.sqrt_bc2 + sc.eps", "den = np.sqrt(v + sc.eps) / sc.sqrt_bc2"),
    ("no second-moment bias correction", PY,
     "den = np.sqrt(v) / sc.sqrt_bc2 + sc.eps", "den = np.sqrt(v) + sc.eps"),
    ("weight decay after the update", PY,
     "    p = p * sc.decay - u\n", "    p = (p - u) * sc.decay\n"),
    ("update with the wrong sign", PY,
     "    p = p * sc.decay - u\n", "    p = p * sc.decay + u\n"),
    ("second-moment bias correction inside the root", PY,
     "den = np.sqrt(v) / sc.sqrt_bc2 + sc.eps", "den = np.sqrt(v / sc.sqrt_bc2) + sc.eps"),
    # loss scaling
    ("growth one step late", PY,
     "if good_steps >= growth_interval:", "if good_steps > growth_interval:"),
    ("clean-step counter kept on a skip", PY,
     "return max(scale * backoff, min_scale), 0", "return max(scale * backoff, min_scale), good_steps"),
    ("no floor on the scale", PY,
     "return max(scale * backoff, min_scale), 0", "return scale * backoff, 0"),
    # bf16 variant
    ("bf16 ties rounded away from zero", PY,
     "rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "rounded = (u + 0x8000) >> 16"),
    ("bf16 sum in sequential order", PY,
     "    while y.size > 1:\n        y = y[0::2] + y[1::2]\n    return float(y[0])",
     "    return float(sum(x.tolist()))"),
    ("bf16 squares as absolute values", PY,
     "sq = np.where(np.isfinite(a), a * a, 0.0)", "sq = np.where(np.isfinite(a), np.abs(a), 0.0)"),
    ("bf16 other ranks' overflow ignored", PY,
     "    skip = bool(own_overflow or other_overflow)\n    return FinalizeResult(0,",
     "    skip = bool(own_overflow)\n    return FinalizeResult(0,"),
    # the C twin
    ("C: fp16 ties rounded away from zero", C,
     "if (rest > half || (rest == half && (h & 1u))) h += 1u;", "if (rest >= half) h += 1u;"),
    ("C: reduce statistics in reversed rank order", C,
     "for (int r = 0; r < n; ++r) acc = acc + half_to_float(rows[r][j]);",
     "for (int r = n - 1; r >= 0; --r) acc = acc + half_to_float(rows[r][j]);"),
    ("C: eps inside the square root", C,
     "const float den = sqrtf(vt) / sqrt_bc2 + eps;", "const float den = sqrtf(vt + eps) / sqrt_bc2;"),
    ("C: bf16 ties rounded up", C,
     "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
     "if (lower >= 0x8000u) upper += 1u;"),
    ("C: bf16 tree summed left to right", C,
     "  for (int64_t half = width / 2; half >= 1; half /= 2)\n"
     "    for (int64_t i = 0; i < half; ++i) y[i] = y[2 * i] + y[2 * i + 1];",
     "  for (int64_t i = 1; i < width; ++i) y[0] = y[0] + y[i];"),
]

NUMPY_PINS = ["tests/test_oracle_reduce_norm.py", "tests/test_oracle_state_bytes_planner.py",
              "tests/test_oracle_units.py", "tests/test_oracle_adam.py",
              "tests/test_oracle_equivalence.py", "tests/test_oracle_bf16.py",
              "tests/test_oracle_clip_torch.py", "tests/test_oracle_scaler_torch.py"]
C_PINS = ["tests/test_oracle_c.py"]


def _copy_tree(dst):
    """The Python side the oracle pins need: oracle/, synth/, tests/ and the
    package (whose planner test_oracle_units compares with)."""
    ign = shutil.ignore_patterns("__pycache__", "*.pyc", "csrc", "*.tmp")
    for d in ("oracle", "synth", "tests", "zero_sharded_optimizer_rank_amd"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=ign)


def _run_pins(root, files):
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], cwd=root, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _mutate(root, path, old, new):
    f = os.path.join(root, path)
    with open(f) as fh:
        src = fh.read()
    assert src.count(old) == 1, f"mutant text occurs {src.count(old)} times in {path}"
    with open(f, "w") as fh:
        fh.write(src.replace(old, new, 1))
    so = os.path.join(root, "oracle", "liboracle.so")
    if path == C and os.path.exists(so):  # the C twin rebuilds from the mutated source
        os.remove(so)


def test_mutant_texts_apply_to_the_current_oracle():
    for name, path, old, _ in MUTANTS:
        with open(os.path.join(ROOT, path)) as fh:
            assert fh.read().count(old) == 1, name


@pytest.mark.timeout(1200)
def test_every_planted_mistake_fails_the_pins(tmp_path):
    def clean():
        d = str(tmp_path / "clean")
        _copy_tree(d)
        return _run_pins(d, NUMPY_PINS + C_PINS)

    def one(i):
        name, path, old, new = MUTANTS[i]
        d = str(tmp_path / f"m{i}")
        _copy_tree(d)
        _mutate(d, path, old, new)
        rc, out = _run_pins(d, C_PINS if path == C else NUMPY_PINS)
        shutil.rmtree(d, ignore_errors=True)
        return name, rc, out

    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        base = ex.submit(clean)
        results = list(ex.map(one, range(len(MUTANTS))))
        rc, out = base.result()
    assert rc == 0, "the unmodified copy fails its pins:\n" + out
    missed = [(name, out) for name, rc, out in results if rc == 0]
    assert not missed, "mutants the pins did not catch:\n" + "\n".join(
        f"- {name}\n{out}" for name, out in missed)
    # caught by a failing assertion, not by a mutant that no longer imports or builds
    broken = [(name, out) for name, rc, out in results
              if rc != 1 or " failed" not in out.strip().splitlines()[-1]]
    assert not broken, "mutants that failed for another reason:\n" + "\n".join(
        f"- {name}\n{out}" for name, out in broken)
