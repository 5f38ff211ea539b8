"""The pins catch plausible mistakes in the oracle.

Each mutant is the oracle's C source with one planted mistake (a swapped
coefficient, a dropped term, a wrong sign, order or index, a rounding rule
changed), built on the CPU; the pin tests run against it in a subprocess
(oracle.lib() loads the build that ORACLE_LIB names) and must fail.  The
unmutated source, built the same way, must pass them: that shows the harness
itself is sound.  The two slow pins (the 2^32-pattern rounding sweep and the
64-replica rational re-evaluation) are left out to keep this quick; every
mutant here is caught by the others.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zero1_oracle.c")
PINS = "tests/test_oracle_pins.py"
SLOW_PINS = ["test_rne_against_torch_bfloat16_all_patterns", "test_oracle_matches_exact_rational[64]"]

MUTANTS = {
    "beta2 in the first moment": (
        "float mn = s->b1 * *m + s->a1 * g;", "float mn = s->b2 * *m + s->a1 * g;"),
    "1-beta1 in the second moment": (
        "float vn = s->b2 * *v + s->a2 * (g * g);", "float vn = s->b2 * *v + s->a1 * (g * g);"),
    "no bias correction": (
        "s->sigma = (float)(lr * sqrt(bc2) / bc1);", "s->sigma = (float)lr;"),
    "bias corrections swapped": (
        "s->sigma = (float)(lr * sqrt(bc2) / bc1);", "s->sigma = (float)(lr * sqrt(bc1) / bc2);"),
    "eps inside the square root": (
        "float d = sqrtf(vn) + s->eps;", "float d = sqrtf(vn + s->eps);"),
    "update sign flipped": (
        "        pn = *p - s->sigma * q;\n        pn = pn * s->delta;",
        "        pn = *p + s->sigma * q;\n        pn = pn * s->delta;"),
    "decay before the update": (
        "        pn = *p - s->sigma * q;\n        pn = pn * s->delta;",
        "        pn = *p * s->delta;\n        pn = pn - s->sigma * q;"),
    "decay factor without lr": (
        "s->delta = (float)(1.0 - lr * weight_decay);", "s->delta = (float)(1.0 - weight_decay);"),
    "sum not averaged": (
        "g[i] = average ? s / fw : s;", "g[i] = s;"),
    "average over W-1": (
        "const float fw = (float)W;", "const float fw = (float)(W > 1 ? W - 1 : 1);"),
    "replicas added in reverse order": (
        "        float s = bf16_to_f32(grads[0][i]);\n        for (int w = 1; w < W; ++w)",
        "        float s = bf16_to_f32(grads[W - 1][i]);\n        for (int w = W - 2; w >= 0; --w)"),
    "last replica dropped": (
        "        for (int w = 1; w < W; ++w)\n            s = s + bf16_to_f32(grads[w][i]);",
        "        for (int w = 1; w < W - 1; ++w)\n            s = s + bf16_to_f32(grads[w][i]);"),
    "norm without the square root": (
        "    return sqrt(q);", "    return q;"),
    "first rank's partial dropped": (
        "    for (int r = 0; r < n_ranks; ++r)\n        q = q + rank_sumsq[r];",
        "    for (int r = 1; r < n_ranks; ++r)\n        q = q + rank_sumsq[r];"),
    "sum of squares in fp32": (
        "            double s = 0.0;\n            for (int64_t i = lo; i < hi; ++i) {\n"
        "                double x = (double)g[i];",
        "            float s = 0.0f;\n            for (int64_t i = lo; i < hi; ++i) {\n"
        "                float x = g[i];"),
    "clip at norm == max_norm": (
        "    if (norm > max_norm) {", "    if (norm >= max_norm) {"),
    "clip coefficient inverted": (
        "        *coef = (float)(max_norm / norm);", "        *coef = (float)(norm / max_norm);"),
    "bf16 rounding by truncation": (
        "    if (d_lo < d_hi)\n        pick = lo_bits;", "    if (1)\n        pick = lo_bits;"),
    "bf16 ties away from zero": (
        "        pick = ((lo_bits >> 16) & 1u) ? hi_bits : lo_bits;", "        pick = hi_bits;"),
    "clip coefficient never applied": (
        "        float gi = clip ? g[i] * coef : g[i];", "        float gi = g[i];"),
    "|g| instead of g*g": (
        "float vn = s->b2 * *v + s->a2 * (g * g);", "float vn = s->b2 * *v + s->a2 * fabsf(g);"),
    "step count off by one": (
        "    double bc1 = 1.0 - pow(beta1, (double)t);", "    double bc1 = 1.0 - pow(beta1, (double)(t + 1));"),
    "bf16 moments stored unrounded (truncated)": (
        "            mb[i] = oracle_f32_to_bf16(mi);", "            mb[i] = (uint16_t)(f32_bits(mi) >> 16);"),
}


def _build(src_text: str, out: str):
    c = out + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *oracle.GCC_FLAGS, c, "-o", out, "-lm"], check=True, capture_output=True)


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    args = [sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"]
    for name in SLOW_PINS:
        args += ["--deselect", f"{PINS}::{name}"]
    return subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.slow
def test_pins_catch_every_planted_mistake(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = open(SRC).read()
    libs = {"control": str(tmp_path / "control.so")}
    _build(src, libs["control"])
    for k, (name, (old, new)) in enumerate(MUTANTS.items()):
        assert src.count(old) == 1, f"mutant {name!r}: its target is not unique in the source"
        libs[name] = str(tmp_path / f"mutant{k}.so")
        _build(src.replace(old, new), libs[name])
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(libs, ex.map(_run_pins, libs.values())))
    control = results.pop("control")
    assert control.returncode == 0, "the unmutated oracle fails its pins:\n" + control.stdout[-3000:]
    survivors = [name for name, r in results.items() if r.returncode == 0]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
