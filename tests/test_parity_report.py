"""The margin-table script on a small synthetic record (host only)."""

from tests.parity_report import report


def test_report_tables():
    recs = [
        {"label": "workload 3 P=-1", "cache": "bf16", "rows": 16, "atol": 5e-3, "rtol": 1e-2,
         "norm": 4e-3, "max_abs": 2e-3, "max_rel": 3e-2, "atol_needed": 1e-3},
        {"label": "full-size step llama3-8b-decode-bf16", "cache": "bf16", "rows": 8, "atol": 5e-3,
         "rtol": 1e-2, "norm": 5e-3, "max_abs": 1e-3, "max_rel": 2e-2, "atol_needed": 4e-3},
        {"label": "x", "cache": "int4", "rows": 4, "atol": 9e-3, "rtol": 1e-2, "norm": 6e-3,
         "max_abs": 1.4e-2, "max_rel": 1e-1, "atol_needed": 4.9e-3},
    ]
    text = report(recs)
    assert "| llama3-70b-decode-bf16 | balanced + merge | 16 |" in text
    assert "| llama3-8b-decode-bf16 | the bench's step" in text
    assert "| bf16 | 2 | 24 | 2.00e-03 | 5.00e-03 | 4.00e-03 | 0.005 |" in text
    assert "| int4 | 1 | 4 |" in text
    # least headroom first: 4e-3 / 5e-3 = 0.80 before 4.9e-3 / 9e-3 = 0.54
    tail = text.split("least headroom")[1]
    assert tail.index("full-size step") < tail.index("| x |")
