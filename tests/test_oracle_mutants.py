"""Planted mistakes in the oracle must fail its pins (CPU only).

Each mutant is a textual edit of a *copy* of ``oracle/kda_oracle.c`` (a dropped
term, a wrong sign, a wrong index or axis, a transposed operand, a missing
reset, a wrong step order), compiled to a temporary library and run against
``test_oracle_pins.py`` (forward mutants), ``test_oracle_bwd_pins.py``
(reverse-mode mutants), ``test_oracle_conv_pins.py`` (convolution mutants) or
``test_oracle_norm_pins.py`` (norm mutants) or ``test_oracle_l2_pins.py``
(q / k normalisation mutants) in a subprocess (a mutant may read out of bounds, so it
never runs in this process).  The committed oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

DECAY = ("const double a = exp(gt[i]);\n"
         "      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;")

MUTANTS = {
    "decay_on_value_axis": (DECAY, "for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= exp(gt[j % dk]);"),
    "no_decay": (DECAY, "(void)gt;"),
    "decay_by_log_not_exp": ("const double a = exp(gt[i]);", "const double a = 1.0 + gt[i];"),
    "decay_exp2": ("const double a = exp(gt[i]);", "const double a = exp2(gt[i]);"),
    "readback_uses_q": ("kv[j] += S[i * dv + j] * kt[i];", "kv[j] += S[i * dv + j] * qt[i];"),
    "error_sign": ("delta[j] = bt * (vt[j] - kv[j]);", "delta[j] = bt * (vt[j] + kv[j]);"),
    "beta_dropped": ("delta[j] = bt * (vt[j] - kv[j]);", "delta[j] = (vt[j] - kv[j]); (void)bt;"),
    "update_uses_q": ("S[i * dv + j] += kt[i] * delta[j];", "S[i * dv + j] += qt[i] * delta[j];"),
    "update_dropped": ("S[i * dv + j] += kt[i] * delta[j];", "(void)delta;"),
    "output_reads_k": ("acc += S[i * dv + j] * qt[i];", "acc += S[i * dv + j] * kt[i];"),
    "scale_dropped": ("ot[j] = scale * acc;", "ot[j] = acc; (void)scale;"),
    "transposed_readback": ("kv[j] += S[i * dv + j] * kt[i];",
                            "kv[j] += S[(j % dk) * dv + (i % dv)] * kt[i];"),
    "no_reset_between_units": ("memset(S, 0, sizeof(double) * dk * dv);", "(void)0;"),
    "init_state_ignored": ("if (init_state)\n    memcpy(S,", "if (0)\n    memcpy(S,"),
    "last_token_skipped": ("t < u->start + u->len; ++t", "t + 1 < u->start + u->len; ++t"),
    "head_stride_wrong": ("const double* kt = k + (t * H + h) * dk;",
                          "const double* kt = k + (t * H + (h + 1) % H) * dk;"),
}


# planted mistakes in the reverse mode, each a plausible slip in one chain-rule line
BWD_MUTANTS = {
    "bwd_dq_from_pre_update_state": ("acc += S[i * dv + j] * dot[j];", "acc += P[i * dv + j] * dot[j];"),
    "bwd_output_term_dropped": ("dS[i * dv + j] += scale * qt[i] * dot[j];", "(void)0;"),
    "bwd_dq_scale_dropped": ("dqt[i] = scale * acc;", "dqt[i] = acc;"),
    "bwd_dbeta_sign": ("acc += ddelta[j] * (vt[j] - kv[j]);", "acc += ddelta[j] * (vt[j] + kv[j]);"),
    "bwd_dkv_sign": ("dkv[j] = -bt * ddelta[j];", "dkv[j] = bt * ddelta[j];"),
    "bwd_dv_beta_dropped": ("dvt[j] = bt * ddelta[j];", "dvt[j] = ddelta[j];"),
    "bwd_ddelta_uses_q": ("ddelta[j] += dS[i * dv + j] * kt[i];", "ddelta[j] += dS[i * dv + j] * qt[i];"),
    "bwd_readback_dk_dropped": ("dkt[i] += acc;", "(void)acc;"),
    "bwd_readback_dP_dropped": ("dP[i * dv + j] = dS[i * dv + j] + kt[i] * dkv[j];",
                                "dP[i * dv + j] = dS[i * dv + j];"),
    "bwd_dlog_g_missing_exp": ("dgt[i] = a[i] * acc;", "dgt[i] = acc;"),
    "bwd_dS_not_decayed": ("dS[i * dv + j] = a[i] * dP[i * dv + j];", "dS[i * dv + j] = dP[i * dv + j];"),
    "bwd_dlog_g_uses_post_state": ("acc += dP[i * dv + j] * Sprev[i * dv + j];",
                                   "acc += dP[i * dv + j] * S[i * dv + j];"),
    "bwd_d_final_ignored": ("if (d_final)\n    memcpy(dS,", "if (0)\n    memcpy(dS,"),
    "bwd_history_after_decay": ("    memcpy(hist + s * sz, S, sizeof(double) * sz);\n"
                                "    for (int64_t i = 0; i < dk; ++i) {\n"
                                "      const double ai = exp(gt[i]);\n"
                                "      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= ai;\n"
                                "    }\n",
                                "    for (int64_t i = 0; i < dk; ++i) {\n"
                                "      const double ai = exp(gt[i]);\n"
                                "      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= ai;\n"
                                "    }\n"
                                "    memcpy(hist + s * sz, S, sizeof(double) * sz);\n"),
}


# planted mistakes in the short convolution
CONV_MUTANTS = {
    "conv_taps_reversed": ("acc += w[c * K + j] * xe[t + j];", "acc += w[c * K + (K - 1 - j)] * xe[t + j];"),
    "conv_window_one_late": ("acc += w[c * K + j] * xe[t + j];",
                             "acc += w[c * K + j] * (t + j + 1 < M + len ? xe[t + j + 1] : 0.0);"),
    "conv_cache_ignored": ("xe[m] = init_cache ? init_cache[(n * channels + c) * M + m] : 0.0;", "xe[m] = 0.0;"),
    "conv_no_reset_between_documents": ("xe[m] = init_cache ? init_cache[(n * channels + c) * M + m] : 0.0;",
                                        "xe[m] = start - M + m >= 0 ? x[(start - M + m) * channels + c] : 0.0;"),
    "conv_silu_before_sum": ("if (act == 1) acc = acc / (1.0 + exp(-acc));", "(void)0;"),
    "conv_final_cache_shifted": ("final_cache[(n * channels + c) * M + m] = xe[len + m];",
                                 "final_cache[(n * channels + c) * M + m] = xe[len + m - (m > 0)];"),
}


# planted mistakes in the gated RMSNorm
NORM_MUTANTS = {
    "norm_one_plus_weight": ("y[r * D + i] = orow[i] * inv * w[i] * gate;",
                             "y[r * D + i] = orow[i] * inv * (1.0 + w[i]) * gate;"),
    "norm_eps_outside_sqrt": ("const double inv = 1.0 / sqrt(ms + eps);", "const double inv = 1.0 / (sqrt(ms) + eps);"),
    "norm_sum_not_mean": ("ms /= (double)D;", "(void)0;"),
    "norm_silu_gate": ("const double gate = 1.0 / (1.0 + exp(-g[r * D + i]));",
                       "const double gate = g[r * D + i] / (1.0 + exp(-g[r * D + i]));"),
    "norm_gate_inside_rms": ("    for (int64_t i = 0; i < D; ++i) ms += orow[i] * orow[i];",
                             "    for (int64_t i = 0; i < D; ++i) ms += orow[i] * orow[i] / (1.0 + exp(-g[r * D + i]));"),
    "norm_no_sqrt": ("const double inv = 1.0 / sqrt(ms + eps);", "const double inv = 1.0 / (ms + eps);"),
}


# planted mistakes in the q / k L2 normalisation
L2_MUTANTS = {
    "l2_eps_outside_sqrt": ("static void l2norm_row(", "const double inv = 1.0 / sqrt(ss + eps);",
                            "const double inv = 1.0 / (sqrt(ss) + eps);"),
    "l2_no_sqrt": ("static void l2norm_row(", "const double inv = 1.0 / sqrt(ss + eps);",
                   "const double inv = 1.0 / (ss + eps);"),
    "l2_abs_not_square": ("static void l2norm_row(", "ss += x[i] * x[i];", "ss += fabs(x[i]);"),
    "l2_q_left_as_is": ("int kda_oracle_qk_l2norm(", "l2norm_row(D, eps, q + r * D, qn + r * D);",
                        "for (int64_t i = 0; i < D; ++i) qn[r * D + i] = q[r * D + i];"),
    "l2_k_from_q": ("int kda_oracle_qk_l2norm(", "l2norm_row(D, eps, k + r * D, kn + r * D);",
                    "l2norm_row(D, eps, q + r * D, kn + r * D);"),
    "l2_first_row_only": ("int kda_oracle_qk_l2norm(", "for (int64_t r = 0; r < rows; ++r) {",
                          "for (int64_t r = 0; r < (rows > 0); ++r) {"),
}


def _mutate_in(src, func, old, new, name):
    """Replace `old` by `new` inside the body of the C function starting with
    `func` (up to the next top-level closing brace); `old` must occur exactly
    once there."""
    a = src.index(func)
    e = src.index("\n}\n", a) + 3
    body = src[a:e]
    assert body.count(old) == 1, f"mutation anchor for {name} not unique/found in {func}"
    return src[:a] + body.replace(old, new) + src[e:]


def _pre_update_output(src):
    """Move the output loop before the rank-1 update (output from the pre-update state)."""
    upd = ("    for (int64_t i = 0; i < dk; ++i)\n"
           "      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * delta[j];\n")
    start = src.index("    /* output from the updated state")
    end = src.index("  }\n  if (final_state)")
    out_block = src[start:end]
    assert upd in src
    return src.replace(upd, "").replace(out_block, out_block + upd.replace("    ", "    ", 1))


def _readback_before_decay(src):
    """Read back (and update) before decaying: the printed order says decay first."""
    start = src.index("    /* decay: every key channel")
    mid = src.index("    /* read back the decayed state")
    decay_block = src[start:mid]
    src = src.replace(decay_block, "")
    anchor = "    /* output from the updated state"
    return src.replace(anchor, decay_block + anchor)


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def _run_pins(lib_path, pins="test_oracle_pins.py"):
    env = dict(os.environ, KDA_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def _build(workdir, name, src_text):
    src = os.path.join(workdir, f"{name}.c")
    with open(src, "w") as f:
        f.write(src_text)
    lib = os.path.join(workdir, f"lib_{name}.so")
    oracle.build(out_path=lib, src=src, extra_flags=["-I", os.path.join(ROOT, "oracle"), "-w"])
    return lib


def test_unmutated_copy_passes(workdir):
    lib = _build(workdir, "clean", open(SRC).read())
    for pins in ("test_oracle_pins.py", "test_oracle_bwd_pins.py", "test_oracle_conv_pins.py",
                 "test_oracle_norm_pins.py", "test_oracle_l2_pins.py"):
        rc, out = _run_pins(lib, pins)
        assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS) + ["pre_update_output", "readback_before_decay"])
def test_mutant_is_caught(workdir, name):
    src = open(SRC).read()
    if name in ("pre_update_output", "readback_before_decay"):
        a = src.index("static void run_unit(")
        e = src.index("\n}\n", a) + 3
        edit = _pre_update_output if name == "pre_update_output" else _readback_before_decay
        mutated = src[:a] + edit(src[a:e]) + src[e:]
    else:
        old, new = MUTANTS[name]
        mutated = _mutate_in(src, "static void run_unit(", old, new, name)
    assert mutated != src
    rc, out = _run_pins(_build(workdir, name, mutated))
    assert rc != 0, f"mutant {name} survived the pins:\n{out}"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(workdir, name):
    src = open(SRC).read()
    old, new = BWD_MUTANTS[name]
    mutated = _mutate_in(src, "static int run_unit_bwd(", old, new, name)
    rc, out = _run_pins(_build(workdir, name, mutated), "test_oracle_bwd_pins.py")
    assert rc != 0, f"mutant {name} survived the backward pins:\n{out}"


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(workdir, name):
    src = open(SRC).read()
    old, new = CONV_MUTANTS[name]
    mutated = _mutate_in(src, "int kda_oracle_short_conv(", old, new, name)
    rc, out = _run_pins(_build(workdir, name, mutated), "test_oracle_conv_pins.py")
    assert rc != 0, f"mutant {name} survived the convolution pins:\n{out}"


@pytest.mark.parametrize("name", sorted(NORM_MUTANTS))
def test_norm_mutant_is_caught(workdir, name):
    src = open(SRC).read()
    old, new = NORM_MUTANTS[name]
    mutated = _mutate_in(src, "int kda_oracle_gated_rmsnorm(", old, new, name)
    rc, out = _run_pins(_build(workdir, name, mutated), "test_oracle_norm_pins.py")
    assert rc != 0, f"mutant {name} survived the norm pins:\n{out}"


@pytest.mark.parametrize("name", sorted(L2_MUTANTS))
def test_l2_mutant_is_caught(workdir, name):
    src = open(SRC).read()
    func, old, new = L2_MUTANTS[name]
    mutated = _mutate_in(src, func, old, new, name)
    rc, out = _run_pins(_build(workdir, name, mutated), "test_oracle_l2_pins.py")
    assert rc != 0, f"mutant {name} survived the L2 normalisation pins:\n{out}"
