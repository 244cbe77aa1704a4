"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle.c with one plausible mistake planted: a dropped
term, a wrong sign or direction, a wrong index, an off-by-one, a different
tie-break or bin convention.  The mutant is compiled into a temporary
directory and the whole pin suite (tests/test_oracle_pins.py) is run against
it in a subprocess; at least one pin must fail.  A control build of the
unmodified source must pass, so a failure is the mistake's and not the
harness's.  The in-tree oracle is never modified.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("full KL weighted by q instead of p",
     "    kl += exp(lp) * (lp - lq);", "    kl += exp(lq) * (lq - lp);"),
    ("full KL log ratio sign",
     "    kl += exp(lp) * (lp - lq);", "    kl += exp(lp) * (lq - lp);"),
    ("other bucket dropped from top-k KL",
     "\n      klk += exp(lpo) * (lpo - lqo);", "\n      klk += 0.0 * (lpo - lqo);"),
    ("other bucket on the candidate side uses baseline mass",
     "        sy += exp(y[i] - mo_y);", "        sy += exp(x[i] - mo_y);"),
    ("other bucket misses its first token",
     "      for (int64_t j = keff; j < v; j++) {\n        const int64_t i = order[j].i;\n        sx",
     "      for (int64_t j = keff + 1; j < v; j++) {\n        const int64_t i = order[j].i;\n        sx"),
    ("normaliser without the log-sum",
     "  return m + log(s);", "  return m;"),
    ("top-k ties broken by the higher index",
     "  return (a->i < b->i) ? -1 : (a->i > b->i);", "  return (a->i > b->i) ? -1 : (a->i < b->i);"),
    ("top-k ranked by the candidate",
     "\n    order[i].x = x[i];", "\n    order[i].x = y[i];"),
    ("candidate argmax ties broken by the higher index",
     "\n    if (y[i] > y[best]) best = i;", "\n    if (y[i] >= y[best]) best = i;"),
    ("record compare argmax ties broken by the higher index",
     "\n        if (y[i] > y[best]) best = i;", "\n        if (y[i] >= y[best]) best = i;"),
    ("margin sign",
     "  o->margin = order[0].x - order[1].x;", "  o->margin = order[1].x - order[0].x;"),
    ("+inf not flagged",
     "x[i] == INFINITY || y[i] == INFINITY) bad = 1;", "0) bad = 1;"),
    ("ULP order folds -0 onto +0",
     "  return (u & sign) ? (~u & all) : (u | sign);",
     "  return (u & sign) ? (sign - (u & ~sign)) : (u | sign);"),
    ("bf16 pairs measured in fp32 units",
     "  const int width = (ta == ORC_BF16 && tb == ORC_BF16) ? 16 : 32;",
     "  const int width = 32;"),
    ("last differing column instead of the first",
     "        if (o.first_diff < 0) o.first_diff = i;", "        o.first_diff = i;"),
    ("relative L2 against the candidate",
     "        o.sum_sq_base += x * x;", "        o.sum_sq_base += y * y;"),
    ("mean abs over differing elements only",
     "    o.mean_abs = o.sum_abs / (double)cols;",
     "    o.mean_abs = o.sum_abs / (double)(o.ndiff > 0 ? o.ndiff : 1);"),
    ("non-finite pairs kept in the norms",
     "      if (fx && fy) {", "      if (1) {"),
    ("bins closed on the right",
     "    while (j < n_edges && !(m < edges[j])) j++;", "    while (j < n_edges && m > edges[j]) j++;"),
    ("big margin taken as >= 1",
     "    if (flip[r] && m > big_margin) summary[g].big_margin_flips++;",
     "    if (flip[r] && m >= big_margin) summary[g].big_margin_flips++;"),
    ("candidate log-probability normalised by the baseline",
     "      logp_cand[r] = y[t] - log_normaliser(y, v);", "      logp_cand[r] = y[t] - log_normaliser(x, v);"),
    ("target log-probability without the normaliser",
     "      logp_base[r] = x[t] - log_normaliser(x, v);", "      logp_base[r] = x[t];"),
    ("perturbation ties rounded away from zero",
     "  return rint(x / q) * q;", "  return round(x / q) * q;"),
    ("perturbation without the subnormal floor of the exponent",
     "  if (E < emin) E = emin;", "  (void)emin;"),
    ("e4m3 without saturation",
     "  if (r > 448.0) r = 448.0;", "  if (r > 480.0) r = 480.0;"),
    ("record rest mass includes the head",
     "        for (int64_t j = keff; j < v; j++) s += exp(order[j].x - m);",
     "        for (int64_t j = 0; j < v; j++) s += exp(order[j].x - m);"),
    ("record entries past k left out of the bucket",
     "        if (ri[j] >= 0) R = log_add(R, (double)rv[j]);", "        (void)rv;"),
    ("record baseline normalised without the bucket",
     "      double L = R;", "      double L = -INFINITY;"),
    ("candidate bucket includes the head",
     "          if (!in_head[i]) s += exp(y[i] - mo);", "          s += exp(y[i] - mo);"),
    ("record compare ignores a non-finite candidate",
     "(sr == ORC_ROW_NONFINITE || sc == ORC_ROW_NONFINITE)", "(sr == ORC_ROW_NONFINITE)"),
    ("flagged rows binned instead of excluded",
     "    if (status && status[r] != 0) {\n      summary[g].excluded++;\n      continue;\n    }",
     "    if (status && status[r] != 0) {\n      summary[g].excluded++;\n    }"),
]


def _build(tmp, name, text):
    src = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-w", "-o", so, src, "-lm"],
                   check=True)
    return so


def _pins_pass(so):
    env = dict(os.environ, ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode == 0, r.stdout[-400:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    source = open(SRC).read()
    builds = {"control": _build(str(tmp_path), "control", source)}
    for j, (name, old, new) in enumerate(MUTANTS):
        assert source.count(old) == 1, f"mutation site not unique or missing: {name}"
        builds[name] = _build(str(tmp_path), f"m{j}", source.replace(old, new))
    with cf.ThreadPoolExecutor(max_workers=4) as pool:
        res = dict(zip(builds, pool.map(_pins_pass, builds.values())))
    ok, tail = res.pop("control")
    assert ok, f"the unmodified oracle must pass its pins:\n{tail}"
    survivors = [name for name, (passed, _) in res.items() if passed]
    assert not survivors, f"mistakes no pin catches: {survivors}"
