"""Host logic of bench.py that runs without a GPU: the HBM-traffic lookup
(tied to the profiled kernel source) and the power sampler's parsing."""
import json
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_traffic_only_for_the_profiled_source(monkeypatch):
    """The counters are reported only while attn_fwd.hip matches the digest
    stored with them; any other workload or source gives None."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    key = next(iter(rec["entries"]))
    workload, out = key.split("/")
    entry = rec["entries"][key]
    got = bench.measured_traffic(workload, out)
    if entry["kernel_source_digest"] == bench.kernel_source_digest():
        assert got is not None and got > 0
    else:
        assert got is None
    assert bench.measured_traffic("no_such_workload", out) is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.measured_traffic(workload, out) is None


def _fake_reading(watts, mhz):
    clocks = {"gfx_%d" % i: {"clk": {"value": mhz, "unit": "MHz"}} for i in range(8)}
    clocks["mem_0"] = {"clk": {"value": 1900, "unit": "MHz"}}
    return json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": watts,
                                                                          "unit": "W"}},
                                     "clock": clocks}]})


def test_power_sampler_parses_and_skips_the_first_readings(monkeypatch):
    """A stand-in for amd-smi: an idle reading first, then loaded ones. The
    medians take only samples from LAG_S on; malformed lines are skipped."""
    idle, busy = _fake_reading(250, 200), _fake_reading(1390, 1860)
    cmd = ("printf '%%s %%s\\n' $(date +%%s.%%N) '%s'; echo 'garbage'; sleep 0.7; "
           "for i in 1 2 3; do printf '%%s %%s\\n' $(date +%%s.%%N) '%s'; sleep 0.05; done"
           % (idle, busy))
    monkeypatch.setattr(bench.PowerSampler, "CMD", cmd)
    s = bench.PowerSampler()
    time.sleep(1.2)
    out = s.stop()
    assert len(out["samples_s_w_mhz"]) == 4
    assert out["samples_s_w_mhz"][0][1] == 250.0
    assert out["loaded_samples"] == 3
    assert out["socket_power_w_median"] == 1390.0
    assert out["gfx_clock_mhz_median"] == pytest.approx(1860.0)


def test_digest_ignores_comments_only():
    """The recorded counters stay valid across edits of comments and blank
    lines, and any edit of the code voids them."""
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    same = "/* a note */\nint f(int x) {\n\n  return x + 1;   // another remark\n}\n"
    other = "int f(int x) {\n  return x + 2;  // one more\n}\n"
    assert bench.kernel_source_digest(code) == bench.kernel_source_digest(same)
    assert bench.kernel_source_digest(code) != bench.kernel_source_digest(other)
