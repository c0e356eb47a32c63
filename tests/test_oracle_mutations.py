"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU) and
check that the pins catch every one of them, while the unmodified source
passes the same pins."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from golden_util import attn_case, expected, load

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "tt_oracle.c")

MUTATIONS = [
    # every loop over the concatenation stops before the block's own tokens
    ("drop_block_keys", "j < N;", "j < (L > 0 ? L : 1);"),
    ("gqa_head_modulo", "const int hk = h / g;", "const int hk = h % Hkv;"),
    ("scale_dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("values_read_token_major",
     "elem(v_pages, (((size_t)page * Hkv + hk) * D + d) * page_size + off, is_bf16)",
     "elem(v_pages, (((size_t)page * Hkv + hk) * page_size + off) * D + d, is_bf16)"),
    ("page_table_ignored", "const int page = page_table[(size_t)b * max_pages + j / page_size];",
     "const int page = j / page_size;"),
    ("block_values_are_keys", "vc[(size_t)(L + j) * D + d] = elem(v_blk, src, is_bf16);",
     "vc[(size_t)(L + j) * D + d] = elem(k_blk, src, is_bf16);"),
    ("max_not_subtracted_sign", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("argmax_last_on_tie", "if ((double)row[v] > m) { m = (double)row[v]; arg = v; }",
     "if ((double)row[v] >= m) { m = (double)row[v]; arg = v; }"),
    ("conf_is_Z", "*conf = 1.0 / Z;", "*conf = Z;"),
    ("commit_tie_higher_slot", "if (cj > cx || (cj == cx && cand[j] < x)) break;",
     "if (cj > cx || (cj == cx && cand[j] > x)) break;"),
    ("commit_unmasked_too", "if (mask[(size_t)b * S + t]) cand[n++] = t;", "cand[n++] = t;"),
    ("remaining_floor", "((long)n + remaining_steps - 1) / remaining_steps", "(long)n / remaining_steps"),
    ("threshold_not_strict", "if (conf[r] > gamma) {", "if (conf[r] >= gamma) {"),
    ("threshold_no_fallback", "if (n > 0 && n_above == 0) commit[(size_t)b * S + best] = 1;", ""),
    ("fallback_higher_slot_on_tie", "if (best < 0 || conf[r] > conf[(size_t)b * S + best]) best = t;",
     "if (best < 0 || conf[r] >= conf[(size_t)b * S + best]) best = t;"),
    ("threshold_ignores_mask", "      if (!mask[r]) continue;\n      ++n;", "      ++n;"),
    ("nsteps_counts_empty", "if (nsteps && n > 0) nsteps[b] += 1;", "if (nsteps) nsteps[b] += 1;"),
    ("chunk_excludes_self", "const int Sk = causal ? t + 1 : S;", "const int Sk = causal ? t : S;"),
    ("chunk_not_causal", "const int Sk = causal ? t + 1 : S;", "const int Sk = S;"),
    ("chunk_anticausal", "const int Sk = causal ? t + 1 : S;", "const int Sk = causal ? S - t : S;"),
    ("lmhead_weight_transposed", "elem(weight, (size_t)v * H + h, 1)", "elem(weight, (size_t)h * V + v, 1)"),
    ("lmhead_drops_last_feature", "for (int h = 0; h < H; ++h)", "for (int h = 0; h < H - 1; ++h)"),
    ("lmhead_rows_ignored", "const int r = rows ? rows[i] : i;", "const int r = i;"),
    ("lmhead_argmax_last_on_tie", "if (row[v] > m) { m = row[v]; arg = v; }",
     "if (row[v] >= m) { m = row[v]; arg = v; }"),
]


def _pins_pass():
    """A compact run of the oracle pins; False as soon as one fails."""
    from test_oracle_attn import sdpa_reference
    from test_oracle_unmask import _brute_force
    try:
        for case in load("attn_hand_cases.json")["cases"]:
            c = attn_case(case, "f32")
            exp = expected(case)
            out = oracle.block_attn(c)
            fixed = ~np.isnan(exp)
            if not np.allclose(out[fixed], exp[fixed], rtol=1e-12, atol=1e-12):
                return False
        rng = np.random.Generator(np.random.PCG64(77))
        c = workloads.make_attn_case(rng, B=2, S=4, Hq=8, Hkv=2, D=16, ctx_lens=[21, 40],
                                     page_size=16, dtype="f32")
        if not np.allclose(oracle.block_attn(c), sdpa_reference(c), rtol=1e-10, atol=1e-12):
            return False
        G = load("unmask_hand_cases.json")
        for row in G["rows"]:
            lg = np.array([float(v) for v in row["logits"]], np.float32)[None]
            ids, _, conf = oracle.unmask(lg, np.ones((1, 1), np.uint8), np.array([1], np.int32))
            if ids[0, 0] != row["id"] or abs(conf[0, 0] - row["conf"]) > 1e-14:
                return False
        cc = G["commit_cases"]
        lg = np.array(cc["logits"], np.float32)
        mask = np.array(cc["mask"], np.uint8)[None]
        for k, want in cc["by_k"]:
            if oracle.unmask(lg, mask, np.array([k], np.int32))[1][0].tolist() != want:
                return False
        for rem, want in cc["by_remaining"]:
            if oracle.unmask(lg, mask, None, rem)[1][0].tolist() != want:
                return False
        rng = np.random.Generator(np.random.PCG64(3))
        for _ in range(4):
            pool = rng.standard_normal((3, 5)).astype(np.float32)
            lg = pool[rng.integers(0, 3, size=8)]
            m = (rng.random((1, 8)) < 0.6).astype(np.uint8)
            k = int(rng.integers(0, 9))
            _, commit, conf = oracle.unmask(lg, m, np.array([k], np.int32))
            if not np.array_equal(commit[0], _brute_force(conf[0], m[0], k)):
                return False
        if not _threshold_pins_pass():
            return False
        if not _chunk_pins_pass():
            return False
        if not _lmhead_pins_pass():
            return False
    except ValueError:
        return False
    return True


def _threshold_pins_pass():
    import test_oracle_threshold as T
    checks = [T.test_hand_sequence_by_gamma, T.test_hand_fallback_tie, T.test_hand_empty_mask,
              T.test_hand_adaptive_loop, T.test_loop_budget_stops_unresolved_blocks]
    checks += [lambda: T.test_gamma_one_is_top1(0), lambda: T.test_negative_gamma_commits_every_masked(0)]
    for f in checks:
        try:
            f()
        except AssertionError:
            return False
    return True


def _chunk_pins_pass():
    import test_oracle_chunk as C
    checks = [lambda case=case: C.test_hand_cases(case) for case in C.G["cases"]]
    checks += [lambda: C.test_against_masked_sdpa([21, 0, 40], 4, 8, 2, 16),
               C.test_future_chunk_tokens_do_not_matter]
    for f in checks:
        try:
            f()
        except AssertionError:
            return False
    return True


def _lmhead_pins_pass():
    import test_oracle_lmhead as M
    checks = [M.test_hand_case, lambda: M.test_identity_head_is_unmask(0),
              lambda: M.test_permuted_head(0), M.test_brute_force_tiny,
              M.test_doubled_weight_doubles_logits, M.test_sequence_selection]
    for f in checks:
        try:
            f()
        except AssertionError:
            return False
    return True


def _build(tmp_path, name, text):
    src = tmp_path / (name + ".c")
    src.write_text(text)
    so = tmp_path / ("lib" + name + ".so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o",
                           str(so), str(src), "-lm"])
    return str(so)


def test_unmodified_source_passes(tmp_path):
    with oracle.library(_build(tmp_path, "control", open(SRC).read())):
        assert _pins_pass()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: " + name
    with oracle.library(_build(tmp_path, name, text.replace(old, new))):
        assert not _pins_pass(), name + " survived every pin"
