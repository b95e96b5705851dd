"""The layout, whole-tensor assignment and pack/gather pins catch plausible
mistakes in the Python oracle.

Each case plants one mistake in a copy of oracle/layout.py or
oracle/pack.py, inside a temporary tree whose other entries link to this
repository's, and runs the pins (tests/test_oracle_layout.py,
tests/test_oracle_tensor_layout.py, tests/test_oracle_gather.py) there;
at least one must fail.  The unmodified copy must pass them all."""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_layout.py", "tests/test_oracle_tensor_layout.py",
        "tests/test_oracle_gather.py"]

# (name, file, text, replacement, occurrence)
MUTATIONS = [
    ("bucket size rounded up past the cap", "layout.py",
     "full = ((bucket_cap_bytes // 2) // unit) * unit",
     "full = _roundup(bucket_cap_bytes // 2, unit)", 0),
    ("tensor starts not aligned", "layout.py",
     "        pos = _roundup(pos, align)\n", "        pos = pos\n", 0),
    ("alignment counted in bytes", "layout.py",
     "align = align_bytes // 2               # bf16 elements per alignment unit",
     "align = align_bytes", 0),
    ("last bucket not padded to W slices", "layout.py",
     "numel = min(full, _roundup(content_end - off, unit))",
     "numel = min(full, content_end - off)", 0),
    ("rank slices in reverse order", "layout.py",
     "        lo = b.flat_off + rank * b.slice_numel\n",
     "        lo = b.flat_off + (world - 1 - rank) * b.slice_numel\n", 0),
    ("chunk shard offset from the bucket start", "layout.py",
     "b.shard_off + (s - lo)))", "b.shard_off + (s - b.flat_off)))", 0),
    ("chunk tensor offset from the slice start", "layout.py",
     "chunks.append(Chunk(t_id, b_id, s - t0, e - s,",
     "chunks.append(Chunk(t_id, b_id, s - lo, e - s,", 0),
    ("whole tensors: shortest first", "layout.py",
     "key=lambda t: (-padded[t], t)", "key=lambda t: (padded[t], t)", 0),
    ("whole tensors: ties to the highest rank", "layout.py",
     "key=lambda q: (load[q], q)", "key=lambda q: (load[q], -q)", 0),
    ("whole tensors: shard in assignment order", "layout.py",
     "    for t in range(len(tensor_numel)):\n        owner_off[t] = fill[owner[t]]",
     "    for t in order:\n        owner_off[t] = fill[owner[t]]", 0),
    ("whole tensors: load counts unpadded sizes", "layout.py",
     "load[r] += padded[t]", "load[r] += tensor_numel[t]", 0),
    ("pack: slice placed at the rank's bucket offset", "pack.py",
     "else lay.rank * b.slice_numel)", "else lay.rank * lay.align_elems)", 0),
    ("pack to tensors: shard offset of the bucket", "pack.py",
     "shard[c.shard_off:c.shard_off + c.numel]",
     "shard[c.tensor_off:c.tensor_off + c.numel]", 0),
]


def plant(text, old, new, which):
    assert old in text, old
    parts = text.split(old)
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


def make_tree(d, mutation):
    """A tree with the entries the pins need linked to the repository's,
    oracle/ copied and, for a mutation, one file of the copy changed."""
    os.makedirs(d)
    for name in ("tests", "synth", "zero_sharded_optimizer_shard_amd",
                 "include", "pytest.ini"):
        os.symlink(os.path.join(ROOT, name), os.path.join(d, name))
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    if mutation is not None:
        _, fname, old, new, which = mutation
        p = os.path.join(d, "oracle", fname)
        text = open(p).read()
        with open(p, "w") as f:
            f.write(plant(text, old, new, which))
    return d


def run_pins(d):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                          cwd=d, env=env, capture_output=True, text=True)


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    base = str(tmp_path_factory.mktemp("lmut"))
    trees = {"control": make_tree(os.path.join(base, "control"), None)}
    for i, m in enumerate(MUTATIONS):
        trees[m[0]] = make_tree(os.path.join(base, f"m{i}"), m)
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        return dict(zip(trees, ex.map(run_pins, trees.values())))


def test_unmodified_oracle_passes_the_pins(results):
    p = results["control"]
    assert p.returncode == 0, p.stdout[-3000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_pins_catch_the_mutation(results, name):
    p = results[name]
    assert p.returncode == 1, (name, p.returncode, p.stdout[-2000:])
    assert " failed" in p.stdout, p.stdout[-2000:]
