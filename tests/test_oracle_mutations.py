"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a copy of oracle/gsa_oracle.py (on
the CPU, in a temporary directory) and runs the pin suites against that copy
in a child pytest process: the pins must fail.  A mistake that every pin lets
through would mean that part of the oracle is not pinned.

The planted mistakes cover the layout rules (window inclusivity, sinks,
candidacy), scoring (mean over heads and gists, head groups), selection (tie
order, both levels, which gists score a group, which chunks are candidates),
attention (log-sum-exp) and the block table (stream order, tile codes); for
the gzip masks, the flag threshold, the band, the literal pairs, causality,
the ratio's divisor, the head mapping and the tile codes; for the backward,
each term of the softmax derivative and the head grouping.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# module -> (its pin suites, name -> (exact text in the module, replacement))

GSA_MUTANTS = {
    "window_inclusive": ("vis = vis | ((i - j) < max(lay.window, 1))",
                         "vis = vis | ((i - j) <= max(lay.window, 1))"),
    "no_sinks": ("vis = typ == SINK", "vis = typ == -1"),
    "chunk_candidate_le": ("if len(gp) == lay.gists and gp[-1] < i]",
                           "if len(gp) == lay.gists and gp[-1] <= i]"),
    "sum_not_mean": ("out[m] = float((qg @ kg.T).mean() * scale)",
                     "out[m] = float((qg @ kg.T).sum() * scale)"),
    "tie_to_higher_id": ("order = sorted(scores, key=lambda m: (-scores[m], m))",
                         "order = sorted(scores, key=lambda m: (-scores[m], -m))"),
    "wrong_head_group": ("qg = q[b, r, h * G:(h + 1) * G, :]", "qg = q[b, r, 0:G, :]"),
    "lse_off": ("lse[b, h * G:(h + 1) * G, r] = ls[:, 0]",
                "lse[b, h * G:(h + 1) * G, r] = mx[:, 0]"),
    "tile_code_threshold": ("codes[qt, t] = 0 if cnt == 0 else (2 if cnt == M.shape[0] * len(cols) else 1)",
                            "codes[qt, t] = 0 if cnt == 0 else (2 if cnt >= M.shape[0] * len(cols) - 1 else 1)"),
    "stream_order_one_level": ("kinds = [SINK, GIST, RAW]", "kinds = [SINK, RAW, GIST]"),
    # the two-level branch
    "A_groups_scored_by_l1_gists": ("s2 = gist_scores(qg, kh, tm.group_gists, group_candidates(lay, tm, i),",
                                    "s2 = gist_scores(qg, kh, tm.chunk_gists, group_candidates(lay, tm, i),"),
    "B_group_candidate_le": ("if len(gp) == lay.l2_gists and gp[-1] < i]",
                             "if len(gp) == lay.l2_gists and gp[-1] <= i]"),
    "C_lowest_groups_kept": ("gids, gp2 = top_k(s2, K2)",
                             "gids, gp2 = top_k({x: -y for x, y in s2.items()}, K2)"),
    "D_stream_order_two_levels": ("kinds = [SINK, GIST2, GIST, RAW]", "kinds = [SINK, GIST, GIST2, RAW]"),
    "E_chunks_outside_kept_groups": ("if gr in gids and len(tm.chunk_gists[m]) == lay.gists",
                                     "if gr >= 0 and len(tm.chunk_gists[m]) == lay.gists"),
    # (a chunk of a kept group always precedes the query, since the group's
    # level-2 gists follow its chunks: `<` vs `<=` there is not observable)
    "F_l1_top_k_uses_k2": ("ids, gp = top_k(s1, K1)", "ids, gp = top_k(s1, K2)"),
    "G_all_l1_gists_visible": ("vis = vis | (typ == GIST2) | ((typ == GIST) & np.isin(tm.group, group_ids))",
                               "vis = vis | (typ == GIST2) | (typ == GIST)"),
    "H_l2_gists_hidden": ("vis = vis | (typ == GIST2) | ((typ == GIST) & np.isin(tm.group, group_ids))",
                          "vis = vis | ((typ == GIST) & np.isin(tm.group, group_ids))"),
}

GZIP_MUTANTS = {
    "gz_flags_at_or_above_mean": ("return r > r.mean()", "return r >= r.mean()"),
    "gz_band_strict": ("local = np.abs(i - j) <= w", "local = np.abs(i - j) < w"),
    "gz_literal_either": ("lit = flags[:, None] & flags[None, :]", "lit = flags[:, None] | flags[None, :]"),
    "gz_no_token_causality": ("return bm[blk[:, None], blk[None, :]] & (np.arange(L)[None, :] <= np.arange(L)[:, None])",
                              "return bm[blk[:, None], blk[None, :]]"),
    "gz_ratio_over_own_length": ("mtime=0)) / block", "mtime=0)) / len(x[i * block:(i + 1) * block])"),
    "gz_head_map_modulo": ("h = hq // G", "h = hq % Hkv"),
    "gz_tile_full_threshold": ("codes[qt, t] = 0 if cnt == 0 else (2 if cnt == (r1 - r0) * (c1 - c0) else 1)",
                               "codes[qt, t] = 0 if cnt == 0 else (2 if cnt >= (r1 - r0) * (c1 - c0) - 1 else 1)"),
}

BACKWARD_MUTANTS = {
    "bw_no_delta": ("ds = p * (dp - delta)", "ds = p * dp"),
    "bw_dk_unscaled": ("dk[b, idx, h, :] += scale * np.outer(ds, qr)", "dk[b, idx, h, :] += np.outer(ds, qr)"),
    "bw_dv_from_ds": ("dv[b, idx, h, :] += np.outer(p, dor)", "dv[b, idx, h, :] += np.outer(ds, dor)"),
    "bw_dq_from_v": ("dq[b, r, hq, :] = scale * (ds @ kk)", "dq[b, r, hq, :] = scale * (ds @ vv)"),
    "bw_wrong_head_group": ("for hq in range(h * G, (h + 1) * G):", "for hq in range(h, h + G):"),
    "bw_delta_from_v": ("delta = dor @ orow", "delta = dor @ vv.mean(axis=0)"),
}

SUITES = {
    "gsa_oracle": (["tests/test_oracle_pins.py", "tests/test_oracle_pins_two_level.py"], GSA_MUTANTS),
    "gzip_mask": (["tests/test_oracle_pins_gzip.py"], GZIP_MUTANTS),
    "gsa_backward": (["tests/test_oracle_pins_backward.py"], BACKWARD_MUTANTS),
}
CASES = [(mod, name) for mod, (_, muts) in SUITES.items() for name in sorted(muts)]


@pytest.mark.parametrize("module,name", CASES, ids=[n for _, n in CASES])
def test_planted_mistake_fails_a_pin(module, name, tmp_path):
    pins, muts = SUITES[module]
    old, new = muts[name]
    src = open(os.path.join(ROOT, "oracle", module + ".py")).read()
    assert src.count(old) == 1, f"mutation {name}: its text is not (uniquely) in oracle/{module}.py"
    mutant = tmp_path / (module + ".py")
    mutant.write_text(src.replace(old, new))
    env = dict(os.environ, GSA_ORACLE_MUTANT=str(mutant), GSA_ORACLE_MUTANT_MODULE=module,
               PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          "--hypothesis-seed=0"] + pins, cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 1, (f"mutation {name} passed every pin (rc {res.returncode})\n"
                                 f"{res.stdout[-2000:]}\n{res.stderr[-2000:]}")
