"""The oracle's pins catch plausible mistakes in it.

Each case below plants one mistake in a copy of the oracle's C core (a sign,
a factor, an index, a threshold or a dropped term that a careful reader could
still miss), builds it with the same flags as the real one into a temporary
directory and runs the pins (`test_oracle_pins.py`, or `test_oracle_depth_pins.py`
for the depth terms) against it in a fresh process: every mutant must fail at
least one pin. An unmutated copy built the
same way must pass them all. The binning, which the oracle writes in numpy,
gets the same treatment: a mutated copy of the oracle package is imported in
place of the real one. Everything runs on the CPU.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "csrc", "gs_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")

# (name, text in the source, replacement); each text occurs exactly once
MUTANTS = [
    ("sigma_cross_term_sign", "- b * q.dx * q.dy;", "+ b * q.dx * q.dy;"),
    ("sigma_missing_half", "-0.5 * (a * q.dx * q.dx + c * q.dy * q.dy)", "-(a * q.dx * q.dx + c * q.dy * q.dy)"),
    ("no_alpha_clamp", "q.alpha = q.ah < ALPHA_MAX ? q.ah : ALPHA_MAX;", "q.alpha = q.ah;"),
    ("no_skip_below_1_255", "if (alpha < ALPHA_MIN) continue;", "if (alpha < 0.0) continue;"),
    ("stop_tested_on_previous_T", "if (test < T_MIN) break;", "if (T < T_MIN) break;"),
    ("T_with_unclamped_alpha", "double test = T * (1.0 - alpha);", "double test = T * (1.0 - ah);"),
    ("behind_not_divided", "S[ch] / (1.0 - al)", "S[ch]"),
    ("dmean_index", "(a_ * q->dx + b_ * q->dy) * ds", "(a_ * q->dx + b_ * q->dx) * ds"),
    ("dconic_b_halved", "o[3] += -q->dx * q->dy * ds;", "o[3] += -0.5 * q->dx * q->dy * ds;"),
    ("dopacity_alpha_for_G", "o[8] += q->G * dal;", "o[8] += q->alpha * dal;"),
    ("dcolour_channel", "o[6] += w * g[1];", "o[6] += w * g[0];"),
    ("behind_accumulates_alpha", "S[1] += col[1] * w;", "S[1] += col[1] * al;"),
    ("clamped_alpha_keeps_sigma_path", "if (q->clamped) return;", ""),
    ("n_contrib_off_by_one", "last = k - start + 1;", "last = k - start;"),
    ("image_without_background", "image[3 * p + 0] = C[0] + T * s.bg[0];", "image[3 * p + 0] = C[0];"),
    ("accum_weight_alpha", "o[9] += w;", "o[9] += al;"),
    # the ambiguity bands and the max-weight continuation bound
    ("alpha_band_ten_times_wider", "static const double K_ALPHA = 4.0;", "static const double K_ALPHA = 40.0;"),
    ("skip_band_dropped", "return fabs(alpha - ALPHA_MIN) <= ea * alpha + 2.0 * U32 * ALPHA_MIN;", "return 0;"),
    ("clamp_band_dropped", "return fabs(ah - ALPHA_MAX) <= ea * ah + 2.0 * U32;", "return 0;"),
    ("stop_band_dropped", "return fabs(test - T_MIN) <= K_T * et * T_MIN + 1e-6 * T_MIN;", "return 0;"),
    ("max_weight_bound_dropped", "double wb = 1.01 * alpha * Tw;", "double wb = 0.0;"),
    ("max_weight_lower_bound_past_ambiguity", "if (buf[e].k < kamb && w > *oc) *oc = w;", "if (w > *oc) *oc = w;"),
    # the admissible-outcome enumeration
    ("outcomes_skip_branch_dropped", "else if (in_skip_band(alpha, ea)) explore(e, k, !skip, -1, -1, T, errT, C, last);",
     ""),
    ("outcomes_stop_branch_dropped", "else if (in_stop_band(test, et)) explore(e, k, 0, clamp, !stop, T, errT, C, last);",
     ""),
]


# mistakes in the depth terms (distortion and median), against the depth pins
DEPTH_MUTANTS = [
    ("dist_pair_cross_sign", "D += w * (u * u * A - 2.0 * u * B + Cs);", "D += w * (u * u * A + 2.0 * u * B + Cs);"),
    ("median_first_not_last", "if (q->T > 0.5) m = e;", "if (q->T > 0.5 && m < 0) m = e;"),
    ("median_pos_off_by_one", "median_pos[p] = m >= 0 ? buf[m].k - start + 1 : 0;",
     "median_pos[p] = m >= 0 ? buf[m].k - start : 0;"),
    ("totals_B_unweighted", "B += w * u;", "B += u;"),
    ("totals_about_zero", "double w = q->alpha * q->T, u = depths[ids[q->k]] - zm;",
     "double w = q->alpha * q->T, u = depths[ids[q->k]];"),
    ("median_band_dropped", "if (amb && fabs(q->T - 0.5) <= K_T * (q->errT + 4.0 * U32) * 0.5 + 1e-6 * 0.5) *amb = 1;",
     ""),
    ("bwd_dist_behind_not_divided", "double dal = gD * (Ti * dw - S / (1.0 - al));",
     "double dal = gD * (Ti * dw - S);"),
    ("bwd_dz_missing_two", "o[9] += gD * 2.0 * w * (u * A - B) + (e == m ? gM : 0.0);",
     "o[9] += gD * w * (u * A - B) + (e == m ? gM : 0.0);"),
    ("bwd_median_to_last_entry", "+ (e == m ? gM : 0.0);", "+ (e == cnt - 1 ? gM : 0.0);"),
    ("bwd_dw_cross_sign", "double dw = u * u * A - 2.0 * u * B + Cs;", "double dw = u * u * A + 2.0 * u * B + Cs;"),
    ("bwd_behind_sum_unweighted", "S += w * dw;", "S += dw;"),
    ("bwd_median_depth_of_first", "int m = median_entry(buf, cnt, NULL);", "int m = cnt > 0 ? 0 : -1;"),
]


def _run(name, text, repl, tmp, pins="test_oracle_pins.py"):
    src = open(SRC).read()
    if text is not None:
        assert src.count(text) == 1, (name, src.count(text))
        src = src.replace(text, repl)
    d = os.path.join(tmp, name)
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, "gs_oracle.c")
    so = os.path.join(d, "gs_oracle.so")
    open(c, "w").write(src)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                    "-o", so, c, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, GS_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", pins), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return p.returncode, p.stdout[-400:]


# mistakes in the numpy binning (oracle/__init__.py)
PY_MUTANTS = [
    ("rect_round_for_floor", "x0 = np.floor((m[:, 0] - r) * inv)", "x0 = np.round((m[:, 0] - r) * inv)"),
    ("rect_end_exclusive_lost", "y1 = np.floor((m[:, 1] + r) * inv) + f(1.0)", "y1 = np.floor((m[:, 1] + r) * inv)"),
    ("depth_ties_by_descending_id", "perm = np.lexsort((ids, dbits[ids], tile))",
     "perm = np.lexsort((-ids, dbits[ids], tile))"),
    ("depth_before_tile", "perm = np.lexsort((ids, dbits[ids], tile))",
     "perm = np.lexsort((ids, tile, dbits[ids]))"),
    ("negative_depth_not_culled", "live = (np.asarray(radii) > 0) & (d > 0) &", "live = (np.asarray(radii) > 0) &"),
    ("tile_ids_column_major", "tile = ty * GX + tx", "tile = tx * GY + ty"),
    # the culling ellipse
    ("cull_threshold_not_doubled", "T = f(2.0) * lnb", "T = lnb"),
    ("cull_log_bound_mantissa_dropped", "lnb = e2 * LN2_F32 + (m2 - f(1.0)) / np.sqrt(m2)", "lnb = e2 * LN2_F32"),
    ("cull_leftmost_v_sign", "vL = (sT * l21) / (l22 * nrm)", "vL = -(sT * l21) / (l22 * nrm)"),
    ("cull_left_end_shear_sign", "xl = mx + (-(l21 * vl) - sl) / l11", "xl = mx + ((l21 * vl) - sl) / l11"),
    ("cull_band_without_half_pixel", "Y0 = ty.astype(f) * f(16.0) + f(0.5)", "Y0 = ty.astype(f) * f(16.0)"),
    ("cull_row_band_one_pixel_short", "v1 = v0 + f(15.0)", "v1 = v0 + f(14.0)"),
    ("cull_not_applied", "kept = np.where(ce[\"cull\"][ids], kept, ~ce[\"dead\"][ids])", "kept = ~ce[\"dead\"][ids]"),
    ("cull_dead_splats_kept", "kept = np.where(ce[\"cull\"][ids], kept, ~ce[\"dead\"][ids])",
     "kept = np.where(ce[\"cull\"][ids], kept, True)"),
]


def _run_py(name, text, repl, tmp, lib):
    """The pins against a copy of the oracle package whose binning carries one
    mistake (its C core: the real build)."""
    d = os.path.join(tmp, "py_" + name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    shutil.copytree(os.path.join(ROOT, "scenes"), os.path.join(d, "scenes"), ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    src = open(PY_SRC).read()
    if text is not None:
        assert src.count(text) == 1, (name, src.count(text))
        src = src.replace(text, repl)
    open(os.path.join(d, "oracle", "__init__.py"), "w").write(src)
    env = dict(os.environ, GS_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(d, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=d, env=env, capture_output=True, text=True,
                       timeout=600)
    return p.returncode, p.stdout[-400:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    import oracle

    lib = oracle.build.build(force=False)  # the real C core, for the binning mutants
    tmp = str(tmp_path_factory.mktemp("oracle_mutants"))
    cases = [("unmutated", None, None)] + MUTANTS
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run, name, t, r, tmp) for name, t, r in cases}
        futs.update({name: ex.submit(_run, name, t, r, tmp, "test_oracle_depth_pins.py")
                     for name, t, r in [("depth_unmutated", None, None)] + DEPTH_MUTANTS})
        futs.update({name: ex.submit(_run_py, name, t, r, tmp, lib)
                     for name, t, r in [("py_unmutated", None, None)] + PY_MUTANTS})
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", ["unmutated", "py_unmutated", "depth_unmutated"])
def test_unmutated_copy_passes(outcomes, name):
    rc, tail = outcomes[name]
    assert rc == 0, tail


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS + PY_MUTANTS + DEPTH_MUTANTS])
def test_pins_catch_mutant(outcomes, name):
    rc, tail = outcomes[name]
    assert rc == 1, f"pins did not fail on mutant {name} (exit {rc}): {tail}"  # 1: tests ran and failed
