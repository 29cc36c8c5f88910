"""Host-side checks of bench.py's accounting (no GPU): the algorithmic byte counts the roofline
uses, and the HBM traffic record's binding to the coarse kernel sources."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_head_bytes_draft_slot():
    # packed codes N K / 4, S and ZS 2 N K / 128 bf16 each, x, candidates M NBLK KCAND (4 + 4) bytes
    N, K = 124160, 5120
    b = bench.head_bytes(1, N, K, own_sums=True)
    assert b["coarse"] == N * K // 4 + 4 * N * (K // 128) + 2 * K + (N // 64) * 8 * 8 == 178_924_800
    assert b["xsum"] == 0
    b16 = bench.head_bytes(16, N, K, own_sums=False)
    assert b16["xsum"] == 16 * K * 2 + 16 * 40 * 4
    assert b16["coarse"] == 180_943_360
    assert b16["rerank_topk"] == 16 * 32 * 4 + 16 * 32 * K * 2 + 16 * K * 2 + 16 * 8
    assert b16["total"] == sum(v for k, v in b16.items() if k != "total")


def test_storage_bytes_match_the_page():
    # packed + S + ZS of one rank's slice: 178,790,400 B = 0.1665 GiB (the page's 0.167 GiB per rank)
    N, K = 124160, 5120
    stored = N * K // 4 + 2 * N * (K // 128) * 2
    assert stored == 178_790_400
    assert abs(stored / 2**30 - 0.1665) < 5e-4


def test_traffic_record_is_bound_to_the_sources(tmp_path, monkeypatch):
    rec = {"source_hash": bench.coarse_source_hash(), "per_call_bytes": {"1": 123}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for(1) == 123
    assert bench.traffic_for(16) is None
    rec["source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.traffic_for(1) is None


def test_gpus_other_than_one_exit_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    else:  # pragma: no cover
        raise AssertionError("bench.py --gpus 2 did not exit")
    assert "one GPU" in capsys.readouterr().err


def test_match_classification_on_oracle_outputs():
    """The bench's comparison of final places with the oracle: identical answers match, a token
    far from the oracle's is unexcused, and a selection that swaps the oracle's R-th token for the
    (R+1)-th is excused at the selection edge when their coarse scores are close."""
    import numpy as np

    import oracle
    import synth_inputs as si
    N, K = 4096, 512
    Wb = si.bits(si.gen_weight(N, K, seed=91))
    xb = si.bits(si.gen_x(6, K, seed=92))
    res = oracle.head(xb, Wb, *oracle.pack(Wb), kcand=8, R=32, k=1)
    n = bench.classify(oracle, np, res["idx"].copy(), res["sel"].copy(), res, xb, Wb)
    assert n["match"] == 6 and n["unexcused"] == 0 and n["match_pct"] == 100.0
    idx = res["idx"].copy()
    worst = np.argsort(res["coarse"][0])[0]           # the row's lowest coarse logit: far below the winner
    idx[0, 0] = worst
    n = bench.classify(oracle, np, idx, res["sel"].copy(), res, xb, Wb)
    assert n["match"] == 5 and n["unexcused"] == 1
    # row 1: swap the oracle's 32nd selected token for the best unselected candidate
    c = res["coarse"][1]
    cand = [t for t in res["cand_idx"][1] if t >= 0 and t not in set(res["sel"][1])]
    nxt = max(cand, key=lambda t: (c[t], -t))
    sel = res["sel"].copy()
    sel[1, -1] = nxt
    idx = res["idx"].copy()
    idx[1, 0] = nxt
    n = bench.classify(oracle, np, idx, sel, res, xb, Wb)
    gap = abs(c[nxt] - c[res["sel"][1, -1]]) / np.abs(c).max()
    assert (n["selection_edge"] == 1) == (gap <= bench.COARSE_TIE)
    assert n["match"] == 5
