"""The oracle's pins must catch plausible mistakes in the oracle.

Each case copies oracle/nm_oracle.c, plants one mistake in the copy (a dropped term, a flipped
sign, a wrong index, an off-by-one), builds it, and runs the oracle pin tests against it in a
subprocess.  The pins pass on the real oracle; every planted mistake must make them fail.
Mistakes are planted on the CPU only, in a temporary copy.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_noise.py", "tests/test_oracle_layer.py", "tests/test_oracle_pack.py",
        "tests/test_oracle_monitor.py", "tests/test_oracle_matmul.py", "tests/test_oracle_properties.py",
        "tests/test_oracle_wreg.py"]

MUTANTS = {
    "philox_swaps_hi_and_lo": ("uint32_t n0 = hi1 ^ x1 ^ k0;", "uint32_t n0 = lo1 ^ x1 ^ k0;"),
    "philox_bumps_key_before_first_round": ("if (r > 0) {", "if (r >= 0) {"),
    "philox_wrong_multiplier_word": ("(uint64_t)PHILOX_M1 * x2;", "(uint64_t)PHILOX_M1 * x1;"),
    "noise_wrong_word_of_block": ("return out[i & 3];", "return out[(i + 1) & 3];"),
    "noise_offset_not_in_counter": ("(uint32_t)offset, (uint32_t)(offset >> 32)}", "0u, 0u}"),
    "uniform_not_at_midpoint": ("+ 0.5) * 0x1p-23", "+ 1.0) * 0x1p-23"),
    "uniform_uses_24_bits": ("(double)(x >> 9)", "(double)(x >> 8)"),
    "gumbel_sign": ("return -log(-log(u));", "return log(-log(u));"),
    "gumbel_uses_log2": ("return -log(-log(u));", "return -log2(-log2(u));"),
    "noise_subtracted": ("(c->kappa * (double)l[k] + gk) / c->tau", "(c->kappa * (double)l[k] - gk) / c->tau"),
    "tau_multiplies": ("(c->kappa * (double)l[k] + gk) / c->tau", "(c->kappa * (double)l[k] + gk) * c->tau"),
    "kappa_dropped": ("(c->kappa * (double)l[k] + gk) / c->tau", "((double)l[k] + gk) / c->tau"),
    "softmax_without_max_shift": ("y[k] = exp(z[k] - mu);", "y[k] = exp(z[k]);"),
    "softmax_not_normalised": ("for (int32_t k = 0; k < c->K; ++k) y[k] /= sum;", ""),
    "soft_mask_wrong_candidate_bit": ("if (c->cand[k] >> j & 1u) mask[j] += y[k];",
                                      "if (c->cand[k] >> (c->m - 1 - j) & 1u) mask[j] += y[k];"),
    "backward_sign": ("y[k] * (d[k] - sdot)", "y[k] * (sdot - d[k])"),
    "backward_missing_weight": ("a[j] = load_w(jb->grad, s->wtype, base + j) * load_w(jb->w, s->wtype, base + j);",
                                "a[j] = load_w(jb->grad, s->wtype, base + j);"),
    "backward_inverse_scale": ("(c->kappa / c->tau) * y[k]", "(c->tau / c->kappa) * y[k]"),
    "backward_drops_softmax_centre": ("sdot += y[k] * d[k];", ""),
    "wreg_drops_factor_two": ("double up = gj + 2.0 * jb->lambda * wj * mask[j];",
                              "double up = gj + jb->lambda * wj * mask[j];"),
    "wreg_unmasked_weight": ("double up = gj + 2.0 * jb->lambda * wj * mask[j];",
                             "double up = gj + 2.0 * jb->lambda * wj;"),
    "wreg_sign": ("double up = gj + 2.0 * jb->lambda", "double up = gj - 2.0 * jb->lambda"),
    "wreg_missing_outer_weight": ("a[j] = up * wj;", "a[j] = up;"),
    "harden_last_max": ("if (l[k] > l[best]) best = k;", "if (l[k] >= l[best]) best = k;"),
    "pack_field_stride": ("put_bits(idx, (q * s->n + t) * nb, (uint32_t)j, nb);",
                          "put_bits(idx, (q * s->m + t) * nb, (uint32_t)j, nb);"),
    "pack_bits_for_m8": ("while ((1 << b) < m) ++b;", "while ((1 << b) < m) ++b;\n    if (m == 8) b = 4;"),
    "unpack_no_zero_fill": ("for (int64_t c = 0; c < s->cols; ++c) zero_w(jb->out, lr * s->cols + c, s->wtype);", ""),
    "prior_takes_last_of_ties": ("if (best < 0 || mag[j] > mag[best]) best = j;",
                                 "if (best < 0 || mag[j] >= mag[best]) best = j;"),
    "prior_signed_magnitude": ("mag[j] = fabs(load_w(", "mag[j] = (load_w("),
    "monitor_max_prob_drops_kappa": ("sum += exp(c->kappa * ((double)l[k] - lmax));",
                                     "sum += exp(((double)l[k] - lmax));"),
    "monitor_sample_last_max": ("if (k == 0 || z > zbest) {", "if (k == 0 || z >= zbest) {"),
    "monitor_sample_noise_subtracted": ("double z = (c->kappa * (double)l[k] + ref_gumbel(x)) / c->tau;",
                                        "double z = (c->kappa * (double)l[k] - ref_gumbel(x)) / c->tau;"),
    "monitor_sample_wrong_slot": ("(uint64_t)g * (uint64_t)c->K + (uint64_t)k);\n        double z =",
                                  "(uint64_t)g * (uint64_t)c->K + (uint64_t)(k + 1));\n        double z ="),
    "monitor_l1_counts_agreement": ("(int32_t)((a >> j & 1u) != (b >> j & 1u));",
                                    "(int32_t)((a >> j & 1u) == (b >> j & 1u));"),
    "monitor_prev_out_of_range_wraps": ("(prev >= 0 && prev < c->K) ? c->cand[prev] : 0u",
                                        "c->cand[prev % c->K]"),
    "matmul_position_ignored": ("load_w(jb->out2, jb->xtype, t * s->cols + q * s->m + p)",
                                "load_w(jb->out2, jb->xtype, t * s->cols + q * s->m + u)"),
    "matmul_skips_last_kept": ("for (int32_t u = 0; u < s->n; ++u) {\n                uint32_t p",
                               "for (int32_t u = 0; u + 1 < s->n; ++u) {\n                uint32_t p"),
    "matmul_subtracts": ("acc += v * load_w(", "acc -= v * load_w("),
    "candidates_skip_last": ("for (int32_t p = start; p <= m - (n - depth); ++p)",
                             "for (int32_t p = start; p < m - (n - depth); ++p)"),
}


def _run_mutant(name, old, new, workdir, probe):
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, f"{name}: snippet not found exactly once"
    d = os.path.join(workdir, name)
    os.makedirs(d)
    csrc = os.path.join(d, "nm_oracle.c")
    with open(csrc, "w") as f:
        f.write(src.replace(old, new))
    # the header sits next to the original source
    lib = oracle_build.build(out=os.path.join(d, "lib.so"), src=csrc,
                             extra=["-I", os.path.dirname(oracle_build.SRC), "-w"], quiet=True)
    env = dict(os.environ, NM_ORACLE_LIB=lib, NM_ROCRAND_PROBE=probe or "")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    return name, res.returncode, res.stdout[-600:]


@pytest.mark.slow
def test_every_planted_mistake_is_caught(rocrand_probe):
    with tempfile.TemporaryDirectory(prefix="nm_mutants_") as work:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, n, o, w, work, rocrand_probe)
                    for n, (o, w) in MUTANTS.items()]
            results = [f.result() for f in futs]
    # a mutant is caught when the pin run fails; a mistake that writes out of bounds may also
    # crash the pin process, which counts as caught (the pins cannot pass)
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mistakes not caught by any pin:\n" + "\n".join(
        f"{n}:\n{out}" for n, out in survivors)
