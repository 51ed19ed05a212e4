"""bench.py on the host: a request for more than one GPU is refused with a message and exit
status 2 before any device work starts (the benchmark measures one GPU); the GPU clock sampler's
report parsing, and its failure path where amd-smi finds no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_clock_report_parsing():
    """The clock sampler's reader takes the current clock of every gfx / mem domain from amd-smi's
    JSON report, whether the value is a {value, unit} object, a number or a "2400 MHz" string,
    and ignores the other clock fields and domains."""
    sys.path.insert(0, ROOT)
    import bench
    report = [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 2100, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                  "max_clk": {"value": 2400, "unit": "MHz"}},
        "gfx_1": {"clk": 2300},
        "gfx_2": {"clk": "2200 MHz"},
        "gfx_3": {"clk": "N/A"},
        "mem_0": {"clk": {"value": 1900, "unit": "MHz"}},
        "vclk_0": {"clk": {"value": 29, "unit": "MHz"}}}}]
    assert bench._clock_mhz(report, "gfx") == [2100.0, 2300.0, 2200.0]
    assert bench._clock_mhz(report, "mem") == [1900.0]
    assert bench._clock_mhz({"clock": {}}, "gfx") == []


def test_clock_sampler_without_a_gpu_reports_an_error_not_an_exception():
    sys.path.insert(0, ROOT)
    import bench
    out = bench.ClockSampler(period_s=0.05).start().stop()
    assert out["source"].startswith("amd-smi")
    assert out["samples"] >= 0
    if out["samples"] == 0:
        assert "error" in out
