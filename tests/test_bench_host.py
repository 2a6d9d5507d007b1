"""Host-side bookkeeping of bench.py: the traffic figures it reports are the
counter readings of a measurement run, scaled by the copy calibration, and
are withheld once the machine code of the kernels they cover changes.  No
GPU is used."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _pmc(dirpath, rows):
    os.makedirs(dirpath)
    with open(os.path.join(dirpath, "x_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i},"{name}",C,{value}\n')


def test_record_traffic_scales_and_sums(tmp_path):
    run = tmp_path / "run"
    run.mkdir()
    # the copy reads and writes 256 MiB; FETCH_SIZE reads half of it
    _pmc(run / "pmc_copy_fetch", [("copy_kernel(int4 const*)", 131072.0)] * 3)
    _pmc(run / "pmc_copy_write", [("copy_kernel(int4 const*)", 262144.0)] * 3)
    k1, k2 = "void bpt::k1<float>()", "_ZN3bpt2k2IfEEvv"       # profilers print either form
    _pmc(run / "pmc_fetch_w1", [(k1, 100.0), (k1, 300.0), (k2, 10.0), (k2, 10.0)])
    _pmc(run / "pmc_write_w1", [(k1, 50.0), (k1, 50.0), (k2, 4.0), (k2, 4.0)])
    (run / "bench_w1.json").write_text(json.dumps({"config": {"kernel": "variant_a"}}) + "\n")
    # a workload with a bench line but no counter runs is left out
    (run / "bench_w2.json").write_text(json.dumps({"config": {"kernel": "variant_b"}}) + "\n")
    out = tmp_path / "traffic.json"
    table = {"_ZN3bpt2k1IfEEvv": {"code": "c1"}, "_ZN3bpt2k2IfEEvv": {"code": "c2"}}
    bench_table = bench.kernel_table
    bench.kernel_table = lambda: table
    try:
        bench.record_traffic(str(run), str(out))
    finally:
        bench.kernel_table = bench_table
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert list(t["entries"]) == ["w1"]
    e = t["entries"]["w1"]
    assert e["variant"] == "variant_a"
    k = {x["name"]: x for x in e["kernels"]}
    assert k[k1]["fetch_kib"] == 200.0 and k[k1]["write_kib"] == 50.0 and k[k1]["dispatches"] == 2
    assert k[k2]["fetch_kib"] == 10.0 and k[k2]["write_kib"] == 4.0
    # each kernel is stamped with the hash of its template's machine code
    assert k[k1]["code"] == bench.template_code(table, k1) is not None
    assert k[k2]["code"] == bench.template_code(table, k2) != k[k1]["code"]


def test_measured_traffic_requires_matching_variant_and_code(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    table = {"_ZN3bpt1aIfEEvv": {"code": "x1"}, "_ZN3bpt1aIiEEvv": {"code": "x2"},
             "_ZN3bpt1bIfEEvv": {"code": "y1"}}
    monkeypatch.setattr(bench, "kernel_table", lambda: table)
    entry = {"variant": "v",
             "kernels": [{"name": "_ZN3bpt1aIfEEvv", "code": bench.template_code(table, "_ZN3bpt1aIfEEvv"),
                          "fetch_kib": 1.0, "write_kib": 2.0},
                         {"name": "void bpt::b<float>()", "code": bench.template_code(table, "_ZN3bpt1bIfEEvv"),
                          "fetch_kib": 3.0, "write_kib": 0.0}]}

    def write():
        (prof / "traffic.json").write_text(json.dumps(
            {"fetch_scale": 2.0, "write_scale": 1.0, "entries": {"w": entry}}))
    write()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # (1*2 + 2*1) + (3*2 + 0) KiB
    assert bench.measured_traffic("w", "v") == 10 * 1024
    assert bench.measured_traffic("w", "other_variant") is None
    assert bench.measured_traffic("missing", "v") is None
    # another instance of template a changed its code: the reading is dropped
    table["_ZN3bpt1aIiEEvv"] = {"code": "x3"}
    assert bench.measured_traffic("w", "v") is None
    table["_ZN3bpt1aIiEEvv"] = {"code": "x2"}
    assert bench.measured_traffic("w", "v") == 10 * 1024
    # an entry without a code stamp is never used
    del entry["kernels"][1]["code"]
    write()
    assert bench.measured_traffic("w", "v") is None


def test_asm_code_hash_ignores_comments_and_label_numbering():
    from barrier_pipelined_tiled_amd import asm_info
    a = {"lines": [asm_info._normalise(x) for x in
                   ["s_mov_b32 s0, 1 ; a comment", ".LBB44_4:", "s_cbranch_scc1 .LBB44_4"]]}
    b = {"lines": [asm_info._normalise(x) for x in
                   ["s_mov_b32   s0, 1", ".LBB7_4:", "s_cbranch_scc1 .LBB7_4 ; other"]]}
    c = {"lines": [asm_info._normalise(x) for x in
                   ["s_mov_b32 s0, 2", ".LBB7_4:", "s_cbranch_scc1 .LBB7_4"]]}
    assert asm_info.code_hash(a) == asm_info.code_hash(b) != asm_info.code_hash(c)
    assert asm_info.base_name("_ZN3bpt17gemm_apair_kernelIDF16_DF16_Lb0EEEvNS_8GemmArgsE") == "gemm_apair_kernel"
    assert asm_info.base_name("void bpt::gemm_apair_kernel<bool _Accum, false>(bpt::GemmArgs)") == \
        "gemm_apair_kernel"


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_parse_smi_reads_shader_memory_clock_and_power():
    # the shape of `amd-smi metric -g 0 -c -p --json` on ROCm 7.2: one gfx
    # clock per XCD, memory clocks, socket power
    sample = {"gpu_data": [{"gpu": 0,
                            "power": {"socket_power": {"value": 1180, "unit": "W"}},
                            "clock": {**{f"gfx_{i}": {"clk": {"value": 1700 + 10 * i, "unit": "MHz"}}
                                         for i in range(8)},
                                      "mem_0": {"clk": {"value": 2000, "unit": "MHz"}},
                                      "vclk_0": {"clk": {"value": 29, "unit": "MHz"}}}}]}
    r = bench.parse_smi(json.dumps(sample))
    assert r == {"gfx_mhz": 1735, "mem_mhz": 2000, "power_w": 1180}


def test_parse_smi_tolerates_missing_fields():
    r = bench.parse_smi(json.dumps({"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": "N/A"}}}]}))
    assert r == {"gfx_mhz": None, "mem_mhz": None, "power_w": None}


def test_smi_finish_reports_a_bad_reading_instead_of_raising():
    import subprocess
    proc = subprocess.Popen([sys.executable, "-c", "print('not json')"], stdout=subprocess.PIPE, text=True)
    r = bench.smi_finish(proc)
    assert set(r) == {"error"}
    assert bench.smi_finish(None) is None


class _Log:
    """Stand-in for torch in time_steps: events and synchronisations append
    markers to the same log as the steps, and every event pair times 1 ms."""

    def __init__(self):
        self.log = []
        log = self.log

        class Event:
            def __init__(self, enable_timing=False):
                pass

            def record(self, stream=None):
                log.append("event")

            def elapsed_time(self, other):
                return 1.0

        class Cuda:
            pass

        self.cuda = Cuda()
        self.cuda.Event = Event
        self.cuda.synchronize = lambda: log.append("sync")


@pytest.mark.parametrize("unit", [1, 8])
def test_time_steps_times_exactly_k_steps(unit, monkeypatch):
    """The timed block holds exactly K steps between two synchronisations
    (K / unit calls when a call is a replayed graph of `unit` steps), after
    at least W warm-up steps; every figure is per step."""
    t = _Log()
    calls = []

    def step(i):
        calls.append(i)
        t.log.append(("step", i))

    class Args:
        steps, warmup, sleep, settle_ms = 64, 20, 0, 0
    monkeypatch.setattr(bench, "log", lambda *a, **k: None)
    ms, kernel_ms, spread, settle = bench.time_steps(t, step, Args, stream=None, unit=unit)
    # the block: sync, event, K/unit calls, event, sync (the first event pair
    # after the warm-up; settle_ms = 0 leaves no settle phase)
    first_event = t.log.index("event")
    assert t.log[first_event - 1] == "sync"
    second_event = t.log.index("event", first_event + 1)
    timed = [x for x in t.log[first_event:second_event] if isinstance(x, tuple)]
    assert len(timed) == Args.steps // unit
    assert t.log[second_event + 1] == "sync"
    warm = [x for x in t.log[:first_event] if isinstance(x, tuple)]
    assert len(warm) * unit >= Args.warmup
    # step indices advance by unit, so replayed passes and plain calls see the
    # same sequence of rotating sets
    assert [i for _, i in timed] == list(range(timed[0][1], timed[0][1] + Args.steps, unit))
    assert kernel_ms == pytest.approx(1.0 / Args.steps)
    assert spread["median_ms"] == pytest.approx(1.0 / unit)
    assert settle is None


def test_time_steps_refuses_a_step_count_that_splits_a_replay():
    class Args:
        steps, warmup, sleep, settle_ms = 100, 20, 0, 0
    with pytest.raises(SystemExit):
        bench.time_steps(_Log(), lambda i: None, Args, stream=None, unit=8)
