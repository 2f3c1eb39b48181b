"""Planted mistakes: plausible errors written into copies of oracle/oracle.c,
each of which must fail at least one of the oracle's pins.

A mutant is a copy of the source with one pattern replaced, built with the
oracle's own compiler flags into a temporary directory and loaded through
SPEC_ORACLE_LIB by a child pytest over the pin files of that part of the
oracle.  Nothing here touches the GPU path; the mutants live only on the CPU.

  * the model forward ("the pages give no model equations", so it is held to
    the mathematics): pins in test_oracle_model.py and
    test_oracle_forward_pins.py;
  * the rule, the sampler and Philox: pins in test_oracle_philox.py,
    test_oracle_sampler.py and test_oracle_verify.py (the worked examples of
    the pages, exact rational comparisons, brute force over the 2^24 uniform
    grid, numpy's Philox)."""
import concurrent.futures
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (pattern, replacement, occurrence)
_ROPE_Q = ("for (int32_t hh = 0; hh < H; hh++) rope_head(q + (size_t)r * qd + (size_t)hh * hd, hd, "
           "pos, m->rope_theta);")
_ROPE_K = ("for (int32_t hh = 0; hh < Hkv; hh++) rope_head(k + (size_t)r * kvd + (size_t)hh * hd, "
           "hd, pos, m->rope_theta);")
_RESID = "for (size_t i = 0; i < (size_t)n * d; i++) x[i] += y[i];"
FORWARD_MUTANTS = {
    "attention scale 1/hd": ("const double scale = 1.0 / sqrt((double)hd);",
                             "const double scale = 1.0 / (double)hd;", 0),
    "attention weights unnormalised": ("const double p = sc[t] / den;", "const double p = sc[t];", 0),
    "values read from the keys": ("const double* vt = vbase", "const double* vt = kbase", 0),
    "no RoPE on keys": (_ROPE_K, "", 0),
    "RoPE on values too": (_ROPE_K, _ROPE_K + _ROPE_K.replace("rope_head(k", "rope_head(v"), 0),
    "queries rotated one position late": (_ROPE_Q, _ROPE_Q.replace("hd, pos,", "hd, pos + 1,"), 0),
    "RoPE exponent -j/hd": ("pow(theta, -2.0 * (double)j / (double)hd)",
                            "pow(theta, -(double)j / (double)hd)", 0),
    "non-causal window": ("(size_t)Hkv * hd, pos + 1, hd,", "(size_t)Hkv * hd, pos0 + n, hd,", 0),
    "GQA head mapping hh % Hkv": ("const int32_t kh = (int32_t)(((int64_t)hh * Hkv) / H);",
                                  "const int32_t kh = hh % Hkv;", 0),
    "attention residual dropped": (_RESID, _RESID.replace("x[i] += y[i]", "x[i] = y[i]"), 0),
    "feed-forward residual dropped": (_RESID, _RESID.replace("x[i] += y[i]", "x[i] = y[i]"), 1),
    "SiLU on the up projection": ("g[i] = silu(g[i]) * u[i];", "g[i] = g[i] * silu(u[i]);", 0),
    "RMSNorm epsilon outside the root": ("double inv = 1.0 / sqrt(ss / (double)d + eps);",
                                         "double inv = 1.0 / (sqrt(ss / (double)d) + eps);", 0),
    "RMSNorm gain dropped": ("h[k] = x[k] * inv * bf16_to_f64(g[k]);", "h[k] = x[k] * inv;", 0),
    "final norm with the attention gains": ("rmsnorm_row(x + (size_t)r * d, d, m->final_norm,",
                                            "rmsnorm_row(x + (size_t)r * d, d, m->attn_norm,", 0),
    "LM head on the un-normed state": ("if (logits) matmul_rows(h, n, d, m->lm_head, V, logits);",
                                       "if (logits) matmul_rows(x, n, d, m->lm_head, V, logits);", 0),
}
FORWARD_PINS = ("test_oracle_model.py", "test_oracle_forward_pins.py")

_RESIDUAL = "for (int32_t v = 0; v < V; v++) q[v] = q[v] > qd[v] ? q[v] - qd[v] : 0;"
RULE_MUTANTS = {
    "accept with <=": ("return (double)r * (double)D < (double)T;",
                       "return (double)r * (double)D <= (double)T;", 0),
    "accept ratio inverted": ("return (double)r * (double)D < (double)T;",
                              "return (double)r * (double)T < (double)D;", 0),
    "residual D - T": (_RESIDUAL,
                       "for (int32_t v = 0; v < V; v++) q[v] = qd[v] > q[v] ? qd[v] - q[v] : 0;", 0),
    "residual without the draft": (_RESIDUAL, "", 0),
    "needle off by one": ("if (acc > t) return v;", "if (acc >= t) return v;", 0),
    "needle without its low part": (
        "(uint64_t)u24 * (Z >> 24) + (((uint64_t)u24 * (Z & 0xFFFFFFULL)) >> 24);",
        "(uint64_t)u24 * (Z >> 24);", 0),
    "fix rounds to nearest": ("*out = (uint64_t)floor(y);", "*out = (uint64_t)floor(y + 0.5);", 0),
    "bonus from the last draft's row": ("sample_target_row(T + (size_t)K * V,",
                                        "sample_target_row(T + (size_t)(K - 1) * V,", 0),
    "accept uniform on a 2^-23 grid": ("float r = (float)u_acc[i] * 0x1p-24f;",
                                       "float r = (float)u_acc[i] * 0x1p-23f;", 0),
    "argmax ties to the highest index": ("if (x[v] > x[best]) best = v;",
                                         "if (x[v] >= x[best]) best = v;", 0),
    "first reject counted as accepted": ("    out[i] = tok;\n    *n_acc = i;",
                                         "    out[i] = tok;\n    *n_acc = i + 1;", 0),
    "Philox key bump swapped": ("k1 += PHILOX_W1;", "k1 += PHILOX_W0;", 0),
    "Philox output word": ("uint64_t n1 = lo1;", "uint64_t n1 = lo0;", 0),
    "u24 from the low bits": ("uint32_t orc_u24(uint64_t w) { return (uint32_t)(w >> 40); }",
                              "uint32_t orc_u24(uint64_t w) { return (uint32_t)(w & 0xFFFFFF); }", 0),
    "uniform counter shifted": ("const uint64_t ctr[4] = {p, s, c, 0};",
                                "const uint64_t ctr[4] = {p + 1, s, c, 0};", 0),
}
RULE_PINS = ("test_oracle_philox.py", "test_oracle_sampler.py", "test_oracle_verify.py")


def _mutate(src, pattern, repl, occurrence):
    parts = src.split(pattern)
    assert len(parts) > occurrence + 1, f"pattern not found (occurrence {occurrence}): {pattern}"
    return pattern.join(parts[:occurrence + 1]) + repl + pattern.join(parts[occurrence + 1:])


def _build_and_run(name, src, tmp, pins):
    path = os.path.join(tmp, "".join(ch if ch.isalnum() else "_" for ch in name))
    os.makedirs(path, exist_ok=True)
    c_file, so = os.path.join(path, "oracle.c"), os.path.join(path, "liboracle.so")
    with open(c_file, "w") as fh:
        fh.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-I", os.path.join(ROOT, "oracle"), c_file, "-o", so, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, SPEC_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *[os.path.join(ROOT, "tests", p) for p in pins]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode


def _check(mutants, pins, tmp):
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as fh:
        src = fh.read()
    sources = {name: _mutate(src, *spec) for name, spec in mutants.items()}
    assert all(m != src for m in sources.values())
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_build_and_run, name, m, tmp, pins) for name, m in sources.items()}
        rcs = {name: f.result() for name, f in futs.items()}
    survivors = [name for name, rc in rcs.items() if rc == 0]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    assert all(rc == 1 for rc in rcs.values()), rcs  # failed tests, not a crash or usage error


def test_forward_mistakes_fail_a_pin(tmp_path):
    _check(FORWARD_MUTANTS, FORWARD_PINS, str(tmp_path))


def test_rule_mistakes_fail_a_pin(tmp_path):
    _check(RULE_MUTANTS, RULE_PINS, str(tmp_path))
