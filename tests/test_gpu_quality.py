"""The quality ablation harness on a small synthetic set: every configuration runs end to
end through the C ABI, and the direction the pages report holds (BDR on outlier keys
beats plain INT4; wispaper.ai blog, sections 2 and 4)."""
import math
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def test_quality_ablation_direction():
    import quality
    rows = quality.run(quality.argparse.Namespace(seqs=2, len=512, kv_heads=2, q_heads=8,
                                                  seed=123, json=False))
    assert len(rows) == len(quality.ROTATIONS) * len(quality.OUTLIERS)
    for r in rows:
        assert math.isfinite(r["mean_rel_err"]) and math.isfinite(r["max_rel_err"]), r
    err = {(r["outliers"], r["rotation"]): r["mean_rel_err"] for r in rows}
    # with the outlier recipe of the workloads, the 128 block keeps the error moderate
    assert err[("2% x U(10,30)", "BDR-128 K")] < 0.5, err
    for outl in ("2% x U(10,30)", "2% x U(50,100)"):
        assert err[(outl, "BDR-128 K")] < err[(outl, "plain INT4")], err
    # without outliers INT4 is already accurate; rotation must not make it much worse
    assert err[("none", "BDR-128 K")] < 2 * err[("none", "plain INT4")] + 1e-3, err
    # 2 bits: coarser than 4 bits everywhere, and the rotation still helps on outlier keys
    for outl in ("none", "2% x U(10,30)"):
        assert err[(outl, "BDR-128 K+V 2-bit")] > err[(outl, "BDR-128 K+V")], err
    assert err[("2% x U(10,30)", "BDR-128 K+V 2-bit")] < err[("2% x U(10,30)", "plain 2-bit")], err
