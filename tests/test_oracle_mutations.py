"""The pins catch plausible mistakes in the C oracle.

Each case plants one mistake in a copy of oracle/zs_oracle.c (on the CPU,
in a temporary directory), builds it with the oracle's own flags, and runs
the step and accumulation pins (tests/test_oracle_step.py,
tests/test_oracle_accumulate.py and the exact-rational emulation in
tests/test_oracle_ieee_emulation.py) against that build through
ZS_ORACLE_LIB; at least one pin must fail with an assertion.  The
unmodified source, built the same way, must pass them all, so a failure is
the mutation's doing.  Two more cases build the unmodified source with
flags that change its arithmetic: contracted multiply-adds, and fast math
(reassociation, reciprocals, flushed denormals)."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zs_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_step.py"),
        os.path.join(ROOT, "tests", "test_oracle_accumulate.py"),
        os.path.join(ROOT, "tests", "test_oracle_ieee_emulation.py")]
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
         "-shared", "-w"]

# (name, text in zs_oracle.c, replacement, occurrence: 0-based or "all")
MUTATIONS = [
    ("eps inside the root",
     "float den = (root / c[5]) + c[7];",
     "float den = sqrtf(vi + c[7]) / c[5];", 0),
    ("decay applied to the updated weight",
     "float th = (*master * c[6]) - (c[4] * upd);",
     "float th = (*master - (c[4] * upd)) * c[6];", 0),
    ("first-moment bias correction dropped",
     "out[4] = (float)(lr / bc1);", "out[4] = (float)lr;", 0),
    ("second-moment bias correction dropped",
     "out[5] = (float)sqrt(bc2);", "out[5] = 1.0f;", 0),
    ("step counter off by one",
     "double bc1 = 1.0 - pow(b1, (double)t);\n    double bc2 = 1.0 - pow(b2, (double)t);",
     "double bc1 = 1.0 - pow(b1, (double)(t + 1));\n    double bc2 = 1.0 - pow(b2, (double)(t + 1));", 0),
    ("weight decay without lr",
     "out[6] = (float)(1.0 - lr * wd);", "out[6] = (float)(1.0 - wd);", 0),
    ("sum not divided by W",
     "return acc / (float)W;", "return acc;", 0),
    ("wrong slice index",
     "acc = acc + bf16_bits_to_float(grads[(int64_t)s * grad_stride + i]);",
     "acc = acc + bf16_bits_to_float(grads[(int64_t)(s - 1) * grad_stride + i]);", 0),
    ("sum in reverse rank order",
     "    float acc = bf16_bits_to_float(grads[i]);\n    for (int32_t s = 1; s < W; ++s)\n        acc = acc + bf16_bits_to_float(grads[(int64_t)s * grad_stride + i]);",
     "    float acc = bf16_bits_to_float(grads[(int64_t)(W - 1) * grad_stride + i]);\n    for (int32_t s = W - 2; s >= 0; --s)\n        acc = acc + bf16_bits_to_float(grads[(int64_t)s * grad_stride + i]);", 0),
    ("update sign flipped",
     "float th = (*master * c[6]) - (c[4] * upd);",
     "float th = (*master * c[6]) + (c[4] * upd);", 0),
    ("beta1 used for the second moment",
     "float vi = (c[1] * *v) + (c[3] * g2);",
     "float vi = (c[0] * *v) + (c[2] * g2);", 0),
    ("bf16 by truncation",
     "return (uint16_t)((u + 0x7fffu + lsb) >> 16);",
     "return (uint16_t)(u >> 16);", 0),
    ("pure bf16: decay on the updated parameter",
     "float th = (bf16_bits_to_float(param[i]) * c[6]) - (c[4] * upd);",
     "float th = (bf16_bits_to_float(param[i]) - (c[4] * upd)) * c[6];", 0),
    ("pure bf16: second moment without the square",
     "        float vi = (c[1] * v[i]) + (c[3] * g2);",
     "        float vi = (c[1] * v[i]) + (c[3] * g);", 0),
    ("accumulation not divided by k",
     "out[i] = float_to_bf16_rne(acc / (float)k);",
     "out[i] = float_to_bf16_rne(acc);", 0),
    ("accumulation drops the last micro-batch",
     "        for (int32_t j = 1; j < k; ++j)",
     "        for (int32_t j = 1; j < k - 1; ++j)", 0),
]



def _host_has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return any(l.startswith("flags") and " fma " in l + " "
                       for l in f)
    except OSError:
        return False


# (name, flags appended after the oracle's own, which they override)
FLAG_MUTATIONS = [
    ("multiply-adds contracted", ["-ffp-contract=fast", "-mfma"]),
    ("fast math", ["-ffast-math"]),
]
if not _host_has_fma():
    FLAG_MUTATIONS = FLAG_MUTATIONS[1:]


def build(src_text, d, name, extra=()):
    c = os.path.join(d, f"{name}.c")
    so = os.path.join(d, f"{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *FLAGS, *extra, c, "-o", so, "-lm"], check=True,
                   capture_output=True, text=True)
    return so


def run_pins(so):
    env = dict(os.environ, ZS_ORACLE_LIB=so)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True)


def plant(text, old, new, which):
    assert old in text, old
    if which == "all":
        return text.replace(old, new)
    parts = text.split(old)
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    """Build the control and every mutant, then run their pins in parallel
    subprocesses (independent builds, independent processes)."""
    d = str(tmp_path_factory.mktemp("mut"))
    src = open(SRC).read()
    libs = {"control": build(src, d, "control")}
    for i, (name, old, new, which) in enumerate(MUTATIONS):
        libs[name] = build(plant(src, old, new, which), d, f"m{i}")
    for i, (name, extra) in enumerate(FLAG_MUTATIONS):
        libs[name] = build(src, d, f"f{i}", extra)
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        done = dict(zip(libs, ex.map(run_pins, libs.values())))
    return done


def test_unmodified_oracle_passes_the_pins(results):
    p = results["control"]
    assert p.returncode == 0, p.stdout[-3000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS] +
                         [m[0] for m in FLAG_MUTATIONS])
def test_pins_catch_the_mutation(results, name):
    p = results[name]
    # 1: a test failed (an assertion, not a crash or a collection error)
    assert p.returncode == 1, (name, p.returncode, p.stdout[-2000:])
    assert " failed" in p.stdout, p.stdout[-2000:]
