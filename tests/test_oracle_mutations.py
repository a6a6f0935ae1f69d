"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a copy of the oracle's C source (on the
CPU, in a temporary directory), builds it, and runs the pin suite against
the broken copy in a subprocess; the suite must fail.  The real oracle is
never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attnres_oracle.c")

MUTATIONS = {
    "eps_dropped": ("return sqrt(s / (double)d + eps);", "return sqrt(s / (double)d);"),
    "eps_outside_mean": ("return sqrt(s / (double)d + eps);", "return sqrt((s + eps) / (double)d);"),
    "norm_not_rms": ("return sqrt(s / (double)d + eps);", "return sqrt(s + eps);"),
    "score_sign": ("zz[i] = s;                                         /* z_i = w^T key */",
                   "zz[i] = -s;"),
    "temperature_sqrt_d": ("zz[i] = s;                                         /* z_i = w^T key */",
                           "zz[i] = s / sqrt((double)d);"),
    "normalised_values": ("for (int64_t i = 0; i < n; ++i) acc += aa[i] * src[i][k];",
                          "for (int64_t i = 0; i < n; ++i) acc += aa[i] * src[i][k] / oracle_rms(d, src[i], eps);"),
    "gain_ignored": ("oracle_rmsnorm(d, src[i], g, eps, key);", "oracle_rmsnorm(d, src[i], NULL, eps, key);"),
    "empty_partial_is_source": ("if (j > 0) srcs[ns++] = partial;",
                                "if (j == 0) for (int64_t k = 0; k < d; ++k) partial[k] = 0.0;\n                    srcs[ns++] = partial;"),
    "partial_missing": ("if (j > 0) srcs[ns++] = partial;", ""),
    "next_sites_query": ("widen(d, w + l * d, wq);\n                    if (g) widen(d, g + l * d, gk);",
                         "widen(d, w + (l + 1) * d, wq);\n                    if (g) widen(d, g + (l + 1) * d, gk);"),
    "full_next_query": ("/* sublayer l+1 attends over v_0..v_l */\n                widen(d, w + l * d, wq);",
                        "widen(d, w + (l + 1 < L ? l + 1 : l) * d, wq);"),
    "prenorm_gain_ignored": ("oracle_rmsnorm(d, h, gamma ? gam : NULL, eps, x);\n                    const int64_t row = (l * n_tok + t) * d;\n                    if (x_out)",
                             "oracle_rmsnorm(d, h, NULL, eps, x);\n                    const int64_t row = (l * n_tok + t) * d;\n                    if (x_out)"),
    "lse_without_max": ("if (lse) *lse = mx + log(sum);", "if (lse) *lse = log(sum);"),
    "merge_unweighted": ("double den = a * lA + b * lB;", "double den = lA + lB;"),
}

# mistakes in the site backward, caught by its own pins
BACKWARD_MUTATIONS = {
    "bwd_logit_without_h": ("s += Gh[k] * (src[i][k] - h[k]);", "s += Gh[k] * src[i][k];"),
    "bwd_rms_radial_term_dropped": ("dx_out[k] = (G[k] - (x[k] / r) * yg / (double)d) / r;",
                                    "dx_out[k] = G[k] / r;"),
    "bwd_prenorm_gain_ignored": ("G[k] = (gamma ? gamma[k] : 1.0) * dx[k];", "G[k] = dx[k];"),
    "bwd_value_path_dropped": ("du[i][k] = alpha[i] * Gh[k] + t[k];", "du[i][k] = t[k];"),
    "bwd_key_gain_missing_in_dw": ("dw[k] += dz * gk * y;", "dw[k] += dz * y;"),
}
# mistakes in the backward through the block structure
BLOCK_BACKWARD_MUTATIONS = {
    "bbwd_partial_grad_dropped": ("for (int64_t k = 0; k < d; ++k) acc[k] += du[n * d + k];", ";"),
    "bbwd_block_sum_grad_dropped": ("memcpy(acc, db + n * d, sizeof(double) * (size_t)d);",
                                    "for (int64_t k = 0; k < d; ++k) acc[k] = 0.0;"),
    "bbwd_final_site_missing": ("if (final_site && dhf) {", "if (0) {"),
    "bbwd_partial_includes_own_output": (
        "memcpy(parts + l * d, bs, sizeof(double) * (size_t)d);\n"
        "                        const float* vl = v + (l * n_tok + t) * d;\n"
        "                        for (int64_t k = 0; k < d; ++k) bs[k] += (double)vl[k];",
        "const float* vl = v + (l * n_tok + t) * d;\n"
        "                        for (int64_t k = 0; k < d; ++k) bs[k] += (double)vl[k];\n"
        "                        memcpy(parts + l * d, bs, sizeof(double) * (size_t)d);"),
    "bbwd_prenorm_skipped": ("if (oracle_site_backward(ns, d, srcs, wq, g ? gk : NULL, gamma ? gm : NULL, 1, eps, dxt,",
                             "if (oracle_site_backward(ns, d, srcs, wq, g ? gk : NULL, gamma ? gm : NULL, 0, eps, dxt,"),
}
PINS = {name: "test_oracle_pins.py" for name in MUTATIONS}
PINS.update({name: "test_oracle_backward.py" for name in BACKWARD_MUTATIONS})
PINS.update({name: "test_oracle_block_backward.py" for name in BLOCK_BACKWARD_MUTATIONS})
MUTATIONS.update(BACKWARD_MUTATIONS)
MUTATIONS.update(BLOCK_BACKWARD_MUTATIONS)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not unique: " + name
    mutated = tmp_path / "attnres_oracle.c"
    mutated.write_text(src.replace(old, new))
    hdr = os.path.join(ROOT, "oracle", "attnres_oracle.h")
    (tmp_path / "attnres_oracle.h").write_text(open(hdr).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(mutated), "-lm"], check=True)
    env = dict(os.environ, ATTNRES_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", PINS[name])],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutation %s:\n%s" % (name, r.stdout[-2000:])
