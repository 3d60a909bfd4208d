"""The failing-case record of the parity tests round-trips on the CPU: the
recorded bf16 bits, workload and mode load back unchanged, and the workload
regenerates the same bits."""
import numpy as np

from numerics_safe_softmax_amd import inputs
from tests import parity


def test_dump_and_load_round_trip(tmp_path):
    w = inputs.custom("rr", 1, 2, 37, 64, True, 5, tie_block=4, v_skew_dims=16, v_mu=-2.0, v_sigma=0.5, do_mu=-0.5)
    d = inputs.generate(w)
    path = parity.dump_case(str(tmp_path / "case"), d, w, 2, note="round trip")
    d2, w2, mode = parity.load_case(path)
    assert w2 == w and mode == 2
    assert sorted(d2) == sorted(d)
    for k in d:
        assert d2[k].dtype == np.uint16 and np.array_equal(d2[k], d[k]), k
    d3 = inputs.generate(w2)
    for k in d:
        assert np.array_equal(d3[k], d[k]), k


def test_record_on_failure_records_then_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(parity, "FAIL_DIR", str(tmp_path))
    w = inputs.custom("rr", 1, 1, 8, 64, False, 6)
    d = inputs.generate(w)
    try:
        with parity.record_on_failure("case (1, 1, 8)", d, w, 1):
            assert False, "planted"
    except AssertionError as e:
        assert "planted" in str(e)
    else:
        raise AssertionError("the failure was swallowed")
    d2, w2, mode = parity.load_case(str(tmp_path / "case_1_1_8"))
    assert w2 == w and mode == 1 and np.array_equal(d2["q"], d["q"])
