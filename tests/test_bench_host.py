"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts of the prefill shape, and the staleness check that keeps
counter traffic from being reported for changed kernel code."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_ep_get_layout_amd import inputs  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_bytes_match_the_closed_form():
    # dispatch: x read once, K rows written per token, one 4-byte slot read
    # per routed pair; combine: K rows read and the output written per
    # token, a slot and a weight read per routed pair
    w = inputs.WORKLOADS["normal_prefill"]
    M = w.R * w.T * w.K
    assert bench.dispatch_bytes(w, M) == 2 * w.H * (w.N + M) + 4 * M
    assert bench.combine_bytes(w, M) == 2 * w.H * (M + w.N) + 8 * M
    assert bench.dispatch_bytes(w, M) == 4_228_907_008


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {  // add one\n  return x + 1; /* done */\n}\n"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(b.replace("+ 1", "+ 2"))


def test_traffic_is_dropped_when_the_kernel_code_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = {"kernel_hash": bench.kernel_hash("combine_rows"), "hbm_bytes_per_launch": 123}
    (prof / "counters.json").write_text(json.dumps({
        "wl:combine_rows": entry,
        "wl:dispatch_copy": {"kernel_hash": "0" * 16, "hbm_bytes_per_launch": 456},
    }))
    real_root = bench.ROOT
    # counters are read from the temporary folder, sources from the repository
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "combine_ep_get_layout_amd"
    src.symlink_to(os.path.join(real_root, "combine_ep_get_layout_amd"))
    assert bench.traffic_from_profile("combine_rows", "wl") == 123
    assert bench.traffic_from_profile("dispatch_copy", "wl") is None
    assert bench.traffic_from_profile("combine_rows", "other") is None


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_every_profiled_kernel_names_existing_sources(kernel):
    for f in bench.KERNEL_SOURCES[kernel]:
        assert os.path.isfile(os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc", f)), f
    assert len(bench.kernel_hash(kernel)) == 16


def test_host_cpu_reports_count_and_model():
    h = bench.host_cpu()
    assert h["nproc"] == os.cpu_count()
    assert h["model"] is None or isinstance(h["model"], str)


def test_fp8_and_low_latency_bytes_match_the_closed_forms():
    # low-latency decode: x read once, per routed pair H code bytes + 4G
    # scale bytes written and a 4-byte slot read; combine as for bf16
    w = inputs.WORKLOADS["ll_decode"]
    M, N, H, G = w.R * w.T * w.K, w.N, w.H, w.G
    assert bench.dispatch_bytes(w, M) == 2 * H * N + (H + 4 * G) * M + 4 * M
    assert bench.combine_bytes(w, M) == 2 * H * M + 2 * H * N + 8 * M
    # about 75 MB dispatch (x 14.7 + codes 58.7 + scales 1.8) and 132 MB combine
    assert round(bench.dispatch_bytes(w, M) / 1e6, 1) == 75.3
    assert round(bench.combine_bytes(w, M) / 1e6, 1) == 132.2
    # FP8 training shape: UE8M0 scales are one byte per group
    w = inputs.WORKLOADS["fp8_train"]
    M, N, H, G = w.R * w.T * w.K, w.N, w.H, w.G
    assert bench.dispatch_bytes(w, M) == 2 * H * N + (H + G) * M + 4 * M
    assert round(bench.dispatch_bytes(w, M) / 1e9, 2) == 5.41
    assert round(bench.combine_bytes(w, M) / 1e9, 2) == 9.67


def test_mix_ceiling_adds_read_and_write_times_at_the_probe_rates():
    # 7 GB read at 7 TB/s (1 ms) and 2 GB written at 4 TB/s (0.5 ms): a phase
    # measured at 2 ms runs at 0.75 of its mix ceiling
    probes = {"read_GBps": 7000.0, "write_GBps": 4000.0, "copy_GBps": 5000.0}
    assert abs(bench.mix_ceiling((7e9, 2e9), probes) - 1.5) < 1e-12
    res = {"phases": {"a": {"ms_mean": 2.0, "read_bytes": 7e9, "written_bytes": 2e9},
                      "b": {"ms_mean": 1.0, "read_bytes": 0, "written_bytes": 2e9}},
           "bytes_per_step": 11e9, "ms_per_step": 4.0, "GBps": 2750.0,
           "roofline": {"phase": "a"}}
    bench.add_mix_ceiling(res, probes)
    assert res["phases"]["a"]["frac_of_mix_ceiling"] == 0.75
    assert res["phases"]["b"]["frac_of_mix_ceiling"] == 0.5
    assert res["mix_ceiling"]["ms_at_probe_roofs"] == 2.0
    assert res["mix_ceiling"]["frac"] == 0.5
    assert res["roofline"]["frac_of_mix_ceiling"] == 0.75
    assert res["mix_ceiling"]["frac_of_copy_probe"] == 0.55


def test_fanout_fraction_only_for_the_probe_shape():
    """The dispatch and combine phases of a bf16 expert-major workload with
    the fan-out / fan-in probes' shape (rows of 2H bytes, R*T rows, K copies)
    get their rates over the probes'; other workloads do not."""
    from combine_ep_get_layout_amd import inputs

    probes = {"read_GBps": 7000.0, "write_GBps": 6000.0, "copy_GBps": 5500.0,
              "fanout_GBps": 5000.0, "fanin_GBps": 6250.0}

    def res():
        return {"phases": {"dispatch": {"ms_mean": 1.0, "read_bytes": 1e9, "written_bytes": 8e9,
                                        "GBps": 4500.0},
                           "combine": {"ms_mean": 1.0, "read_bytes": 8e9, "written_bytes": 1e9,
                                       "GBps": 5000.0}},
                "bytes_per_step": 18e9, "ms_per_step": 2.0, "GBps": 9000.0,
                "roofline": {"phase": "dispatch"}}

    w = inputs.WORKLOADS["normal_prefill"]
    assert (w.H * 2 // 16, w.N, w.K) == bench.FANOUT_SHAPE
    r = res()
    bench.add_mix_ceiling(r, probes, w)
    assert r["phases"]["dispatch"]["frac_of_fanout_probe"] == 0.9
    assert r["phases"]["combine"]["frac_of_fanin_probe"] == 0.8
    for name in ("rank_prefill", "fp8_train", "ll_decode"):
        r = res()
        bench.add_mix_ceiling(r, probes, inputs.WORKLOADS[name])
        assert "frac_of_fanout_probe" not in r["phases"]["dispatch"], name
        assert "frac_of_fanin_probe" not in r["phases"]["combine"], name


def test_probe_library_rejects_bad_arguments_before_any_launch():
    """The probe entry points check their arguments on the host and return
    -1 before touching the GPU (so these calls run without one)."""
    import ctypes

    if not os.path.exists(bench.PROBE_LIB):
        pytest.skip("libbench_probe.so not built")
    lib = ctypes.CDLL(bench.PROBE_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.bench_probe_launch.argtypes = [ctypes.c_int, vp, vp, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, vp]
    for f in (lib.bench_fanout_launch, lib.bench_fanin_launch):
        f.argtypes = [vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp]
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks
    assert lib.bench_probe_launch(3, p, p, 1 << 20, 1, 0, 64, None) == -1   # kind
    assert lib.bench_probe_launch(2, p, p, 1000, 1, 0, 64, None) == -1      # not 16-byte
    assert lib.bench_probe_launch(2, None, p, 1 << 20, 1, 0, 64, None) == -1
    assert lib.bench_probe_launch(1, None, p, 1 << 20, 3, 0, 64, None) == -1  # unroll
    for f in (lib.bench_fanout_launch, lib.bench_fanin_launch):
        assert f(p, p, 2048, 16, 8, 0, None) == -1    # rows wider than 1024 vectors
        assert f(p, p, 896, 0, 8, 0, None) == -1      # no rows
        assert f(p, p, 896, 16, 65, 0, None) == -1    # too many copies
        assert f(None, p, 896, 16, 8, 0, None) == -1
        assert f(p, p, 100, 16, 8, 1 if f is lib.bench_fanout_launch else 0, None) == -1
        assert f(p, p, 896, 16, 8, 2, None) == -1     # form
