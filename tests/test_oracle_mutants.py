"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, plants one plausible mistake (a dropped
term, a wrong sign or index, a swapped operand, a reversed order), builds it on
the CPU and runs the pin suite against that build in a subprocess; the suite
must fail.  The real oracle is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "relu_dropped": ("double relu = x > 0.0 ? x : 0.0;", "double relu = x;"),
    "weight_dropped": ("r += (double)w[j] * relu;", "r += relu;"),
    "q_transposed": ("qd[(int64_t)j * D + d]", "qd[(int64_t)d * H + j]"),
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "fp32_accumulation": ("double x = 0.0;", "float x = 0.0f;"),
    "topk_ascending": ("if (sa > sb) return -1;\n  if (sa < sb) return 1;",
                       "if (sa > sb) return 1;\n  if (sa < sb) return -1;"),
    "topk_tie_high_index": ("  return (ia > ib) - (ia < ib);\n}\n\nstatic int cmp_int_asc",
                            "  return (ia < ib) - (ia > ib);\n}\n\nstatic int cmp_int_asc"),
    "ema_no_seed": ("if (isinf(theta) && theta > 0) return s_k;", ""),
    "ema_weights_swapped": ("float a = alpha * s_k;\n  float b = keep * theta;",
                            "float a = alpha * theta;\n  float b = keep * s_k;"),
    "threshold_not_strict": ("if (sb[s] > th && st->h2g[h] == -1)",
                             "if (sb[s] >= th && st->h2g[h] == -1)"),
    "cap_rounds_down": ("int64_t cap = (ctx + c->cap_div - 1) / c->cap_div;",
                        "int64_t cap = ctx / c->cap_div;"),
    "no_protect": ("      if (g >= 0)\n        st->prio[g] = t;\n      else",
                   "      if (g >= 0)\n        ;\n      else"),
    "evict_newest_first": ("return (*x > *y) - (*x < *y);", "return (*x < *y) - (*x > *y);"),
    "no_reserve": ("int64_t want = n_miss_all + reserve - n_free;",
                   "int64_t want = n_miss_all - n_free;"),
    "alloc_descending": ("install(c, st, h, F[i], host_kv);",
                         "install(c, st, h, F[nF - 1 - i], host_kv);"),
    "prefetch_ignores_offset": ("int32_t g = F[off + r];", "int32_t g = F[r];"),
    "metadata_idxbuf_dropped": ("int64_t per_slot = 1 + 4 + 4 + 4;",
                                "int64_t per_slot = 1 + 4 + 4;"),
    "append_overwrites_last_row": ("const int64_t h = host_id(map, b, ctx[b]);\n    memcpy",
                                   "const int64_t h = host_id(map, b, ctx[b] - 1);\n    memcpy"),
    "gather_ignores_token_map": ("const int64_t h = host_id(map, b, sel_tok[(int64_t)b * k + i]);",
                                 "const int64_t h = sel_tok[(int64_t)b * k + i];"),
    "release_keeps_priority": ("        freef[g] = 1;\n        prio[g] = -1;\n",
                               "        freef[g] = 1;\n"),
    "release_skips_last_token": ("for (int32_t s = 0; s < ctx[b]; ++s) {\n      const int64_t h = "
                                 "host_id(map, b, s);\n      const int32_t g = h2g[h];",
                                 "for (int32_t s = 0; s < ctx[b] - 1; ++s) {\n      const int64_t h = "
                                 "host_id(map, b, s);\n      const int32_t g = h2g[h];"),
    "release_keeps_threshold": ("    theta[b] = INFINITY;\n    if (commit) ctx[b] = 0;\n",
                                "    if (commit) ctx[b] = 0;\n"),
    "admit_ignores_overlap": ("if ((int64_t)base < hi && lo < (int64_t)base + len) return ORC_ECAPACITY;",
                              "(void)lo;\n    (void)hi;"),
    "admit_keeps_threshold": ("  theta[b] = INFINITY;\n  if (commit) {", "  if (commit) {"),
    "f16_ties_away_from_zero": ("double m = nearbyint(a / quantum);", "double m = round(a / quantum);"),
    "f16_subnormal_step": ("e < -14 ? ldexp(1.0, -24)", "e < -14 ? ldexp(1.0, -23)"),
    "bucket_low_byte": ("  return key >> 8;\n", "  return key & 0xFF;\n"),
    "coarse_shift_added": ("const float d = score - pred;", "const float d = score + pred;"),
    "coarse_shift_dropped": ("const float d = score - pred;", "const float d = score;"),
    "coarse_keeps_boundary_bucket": ("if (coarse_bucket(row[s], p) > beta) {",
                                     "if (coarse_bucket(row[s], p) >= beta) {"),
    "prefill_exact_before_early": ("for (int32_t j = 0; j < o->n_cand; ++j) { /* the early transfer */",
                                   "for (int32_t j = 0; j < 0; ++j) { /* the early transfer */"),
    "prefill_no_protect": ("    if (st->h2g[h] >= 0) {\n      st->prio[st->h2g[h]] = t;\n    } else {\n"
                           "      const int32_t g = F[next++];\n      install(c, st, h, g, host_kv);\n"
                           "      o->miss_h",
                           "    if (st->h2g[h] >= 0) {\n      ;\n    } else {\n"
                           "      const int32_t g = F[next++];\n      install(c, st, h, g, host_kv);\n"
                           "      o->miss_h"),
    "append_writes_empty_rows": ("    if (ctx[b] == 0) continue; /* an empty row */\n", ""),
    "append_empty_row_blocks_neighbours": ("      if (o == b || ctx[o] == 0) continue;",
                                           "      if (o == b) continue;"),
    "append_writes_empty_row_bytes": ("  for (int b = 0; b < B; ++b) {\n    if (ctx[b] == 0) continue;\n"
                                      "    const int64_t h = host_id(map, b, ctx[b]);\n    memcpy",
                                      "  for (int b = 0; b < B; ++b) {\n"
                                      "    const int64_t h = host_id(map, b, ctx[b]);\n    memcpy"),
    "append_grows_empty_rows": ("      if (ctx[b] != 0) ctx[b] += 1;", "      ctx[b] += 1;"),
    "append_ignores_neighbours": ("if (h >= hb[o] && h < (int64_t)hb[o] + ctx[o] + 1) return ORC_ECAPACITY;",
                                  "if (0) return ORC_ECAPACITY;"),
    # page tables (R14)
    "page_offset_dropped": ("return 16 * (int64_t)m->pages[(int64_t)b * m->page_stride + s / 16] + s % 16;",
                            "return 16 * (int64_t)m->pages[(int64_t)b * m->page_stride + s / 16];"),
    "page_stride_ignored": ("return 16 * (int64_t)m->pages[(int64_t)b * m->page_stride + s / 16] + s % 16;",
                            "return 16 * (int64_t)m->pages[(int64_t)b + s / 16] + s % 16;"),
    "paged_scores_read_row_order": ("memcpy(rows + s * c->D, kidx + host_id(map, b, s) * c->D, (size_t)c->D);",
                                    "memcpy(rows + s * c->D, kidx + s * c->D, (size_t)c->D);"),
    "paged_prefetch_ignores_pages": ("        int64_t h = host_id(map, b, s);\n        if (sb[s] > th",
                                     "        int64_t h = s;\n        if (sb[s] > th"),
    "admit_ignores_shared_page": ("if (ro[i] == row[j]) return ORC_ECAPACITY;", "(void)ro;"),
    "admit_ignores_repeated_page": ("if (row[i] == row[j]) return ORC_EDEVARG;", "(void)i;"),
    "admit_page_range_unchecked": ("if (row[j] < 0 || 16 * (int64_t)row[j] + 16 > n_host) return ORC_EDEVARG;",
                                   "(void)n_host;"),
    "page_fit_unchecked": ("if (p < 0 || 16 * (int64_t)p + 16 > n_host) return 0;", "(void)p;"),
}


def _build(name, tmp):
    src = open(O.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} is not unique"
    path_c = os.path.join(tmp, f"m_{name}.c")
    path_so = os.path.join(tmp, f"m_{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-std=gnu99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", path_c, "-o", path_so, "-lm"], check=True)
    return path_so


def _run_pins(so):
    env = dict(os.environ, ECHO_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    names = sorted(MUTANTS)
    sos = [_build(n, str(tmp_path)) for n in names]
    with ThreadPoolExecutor(max_workers=6) as ex:
        codes = list(ex.map(_run_pins, sos))
    survivors = [n for n, c in zip(names, codes) if c == 0]
    assert not survivors, f"pins did not notice: {survivors}"


def test_unmutated_oracle_passes_the_pins():
    assert _run_pins(O.build()) == 0
