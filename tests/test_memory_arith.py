"""The oracle's memory arithmetic against the figures the pages print (CPU only)."""
import json
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "math_path_memory.json")))
UNIT = {"GB": 1e9, "GiB": 2.0 ** 30}


def test_score_matrix_bytes_match_printed():
    for e in GOLD["score_matrix"]:
        got = oracle.math_path_bytes(e["L"], e["Hq"], e["elem_bytes"]) / UNIT[e["unit"]]
        assert round(got, e["decimals"]) == e["printed"], e["cite"]


def test_oom_request_is_one_matrix_near_30k():
    e = GOLD["oom_request"]
    hits = [L for L in range(e["L_low"], e["L_high"] + 1)
            if round(oracle.math_path_bytes(L, e["Hq"], e["elem_bytes"]) / UNIT[e["unit"]], e["decimals"]) == e["printed"]]
    assert hits, e["cite"]
    # and two such matrices would not round to the printed request
    assert all(round(2 * oracle.math_path_bytes(L) / UNIT["GiB"], 2) != e["printed"] for L in hits)


def test_repeated_kv_bytes():
    e = GOLD["repeated_kv"]
    got = oracle.repeat_kv_bytes(e["Hq"], e["L"], e["D"], e["elem_bytes"]) / UNIT[e["unit"]]
    assert round(got, e["decimals"]) == e["printed"], e["cite"]


def test_printed_long_path_memory_is_linear_in_L():
    e = GOLD["long_path_linear"]
    per_token = np.array(e["peak_GiB"]) / np.array(e["L"])
    assert np.ptp(per_token) / per_token.mean() < 0.01, e["cite"]


def test_visible_pair_count_closed_forms():
    # causal, q_offset 0: L(L+1)/2 pairs per head
    for L in (1, 7, 64, 129):
        assert oracle.visible_pairs(L, L) == L * (L + 1) // 2
    # non-causal: Lq * Lk
    assert oracle.visible_pairs(5, 9, causal=False) == 45
    # branch of m rows at offset S over S + m keys: m*S + m(m+1)/2
    S, m = 40, 9
    assert oracle.visible_pairs(m, S + m, q_offset=S) == m * S + m * (m + 1) // 2
    # packed segments: sum of per-segment triangles
    lens = [3, 10, 6]
    seg = np.repeat(np.arange(3), lens)
    assert oracle.visible_pairs(19, 19, seg_q=seg, seg_k=seg) == sum(n * (n + 1) // 2 for n in lens)


def test_product_pair_count_matches_the_oracle_definition():
    """The benchmark's FLOP accounting (package-side, fast) agrees with the
    oracle's dense-mask count on small cases."""
    from long_context_causal_amd import work
    rng = np.random.default_rng(3)
    cases = [dict(Lq=37, Lk=37), dict(Lq=20, Lk=50, q_offset=30), dict(Lq=25, Lk=40, causal=False)]
    seg = np.sort(rng.integers(0, 4, size=60)).astype(np.int32)
    cases.append(dict(Lq=60, Lk=60, seg_q=seg, seg_k=seg))
    cases.append(dict(Lq=60, Lk=60, seg_q=rng.integers(0, 3, 60), seg_k=rng.integers(0, 3, 60), causal=False))
    cases.append(dict(Lq=60, Lk=70, q_offset=10, seg_q=rng.integers(0, 3, 60), seg_k=rng.integers(0, 3, 70)))
    for c in cases:
        c2 = dict(c)
        Lq, Lk = c2.pop("Lq"), c2.pop("Lk")
        assert work.visible_pairs(Lq, Lk, **c2) == oracle.visible_pairs(Lq, Lk, **c2), c
