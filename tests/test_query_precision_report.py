"""The CPU report of how far the E4M3 query quantisation (the fused indexer front's FP8
query, "Fused low-latency decode for DSA layers") moves each stage from a bf16-exact
query.  Runs the report on a small sample and checks that its figures are sane; the
full-size figures are quoted in the design notes."""
import oracle.query_quantisation_report as R


def test_query_quantisation_report_small_sample():
    d = R.report(rows=1, context=8192, topk=256, seed=5)
    assert 0.0 < d["score_dev_over_max_abs_and_A"]["median"] < 0.05
    assert d["score_dev_over_max_abs_and_A"]["max"] < 1.0
    assert 0.8 < d["topk_set_overlap"]["min"] <= 1.0
    assert 0.0 < d["mla_abs_dO"]["max"] < 0.1
    assert 0.0 < d["mla_abs_dLSE"]["max"] < 0.05
