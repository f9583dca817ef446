"""Host logic of bench.py, on the CPU: the algorithmic byte model, the
traffic lookup's source-digest gate, the per-op annotations (share of the
copy ceiling, the backward's reduction plan), the same-size copy rates and
the refusal of more than one GPU.  No GPU is touched: the library calls
are replaced by stand-ins."""
import json
import os
import subprocess
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_alg_bytes_closed_forms():
    # one row of one element: every tensor term is visible on its own
    b = bench.alg_bytes(1, 1, 2)
    assert b["ln_fwd"] == 2 * 2 + 2 * 2 + 8
    assert b["rms_fwd"] == 2 * 2 + 2 + 4
    assert b["fused_add_rms_fwd"] == 4 * 2 + 2 + 4
    assert b["ln_bwd"] == 3 * 2 + 3 * 2 + 8
    assert b["rms_bwd"] == 3 * 2 + 2 * 2 + 4
    assert b["fused_add_rms_bwd"] == 4 * 2 + 2 * 2 + 4
    N, H, e = 32768, 1024, 2
    b = bench.alg_bytes(N, H, e)
    # the unfused pair moves one extra N*H tensor (h written, then read back)
    assert b["unfused_add_rms"] - b["fused_add_rms_fwd"] == N * H * e
    assert b["fused_add_rms_fwd_inplace"] == b["fused_add_rms_fwd"]
    # no bias: one parameter vector fewer; float32 parameters: twice the bytes
    assert b["ln_fwd"] - bench.alg_bytes(N, H, e, beta=False)["ln_fwd"] == H * e
    w = bench.alg_bytes(N, H, e, ep=4)
    assert w["ln_bwd"] - b["ln_bwd"] == 3 * H * (4 - e)
    # the step's five ops at the headline shape
    step = sum(b[k] for k in bench.OPS)
    assert step == 14 * N * H * e + 9 * H * e + 28 * N


def test_counters_traffic_gate(tmp_path, monkeypatch):
    from rmsnorm_row_welford_amd import profsum
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_source_digest": "abc", "traffic_bytes_per_launch": 123.0}
    (prof / "rms_fwd_8x8.counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(profsum, "kernel_source_digest", lambda: "abc")
    assert bench.counters_traffic("rms_fwd", "8x8") == 123.0
    # measured on other kernel sources, missing, or unreadable: no figure
    monkeypatch.setattr(profsum, "kernel_source_digest", lambda: "def")
    assert bench.counters_traffic("rms_fwd", "8x8") is None
    assert bench.counters_traffic("ln_fwd", "8x8") is None
    (prof / "ln_fwd_8x8.counters.json").write_text("{not json")
    assert bench.counters_traffic("ln_fwd", "8x8") is None


def test_annotate_and_plan(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "get_device_properties",
                        lambda dev: types.SimpleNamespace(multi_processor_count=256))
    calls = []

    def partial_rows(N, H, dtype, layernorm, param_dtype=None):
        calls.append((N, H, dtype, layernorm, param_dtype))
        return 256 if N > 512 else 0

    rn = types.SimpleNamespace(bwd_partial_rows=partial_rows)
    table = {"N": 32768, "H": 1024,
             "ln_fwd": {"us": 1.0, "GBps": 3000.0},
             "ln_bwd": {"us": 2.0, "GBps": 4500.0},
             "rms_bwd": {"us": 2.0, "GBps": 6000.0}}
    bench.annotate(rn, None, table, 32768, 1024, "bf16", None, 6000.0)
    assert table["ln_fwd"]["pct_copy_ceiling"] == 50.0
    assert "partial_rows" not in table["ln_fwd"]
    assert table["ln_bwd"]["pct_copy_ceiling"] == 75.0
    assert table["ln_bwd"]["partial_rows"] == 256
    assert table["ln_bwd"]["per_cu"] == 1.0
    assert table["ln_bwd"]["reduction"] == "partial rows + kernel 2"
    assert table["rms_bwd"]["pct_copy_ceiling"] == 100.0
    assert [c[3] for c in calls] == [True, False]
    assert all(c[2] == torch.bfloat16 and c[4] == torch.bfloat16 for c in calls)
    small = {"ln_bwd": {"us": 1.0, "GBps": 600.0}}
    bench.annotate(rn, None, small, 512, 16384, "bf16", "f32", 6000.0)
    assert small["ln_bwd"]["partial_rows"] == 0
    assert small["ln_bwd"]["reduction"].startswith("column sums")
    assert calls[-1][4] == torch.float32


def test_same_size_ceilings(monkeypatch):
    timed = []

    def fake_ceilings(rn, dev, nbytes=0, kinds=("copy", "add"), **kw):
        timed.append((nbytes, kinds))
        return {"copy": {"GBps": 1000.0 + nbytes / (1 << 20)}}

    monkeypatch.setattr(bench, "stream_ceilings", fake_ceilings)
    monkeypatch.setattr(bench, "log", lambda *a: None)
    shapes = {
        "a": {"N": 512, "H": 16384, "dtype": "bf16", "ln_fwd": {"GBps": 508.0}},
        "b": {"N": 2048, "H": 4096, "dtype": "bf16", "rms_fwd": {"GBps": 2032.0}},
        "c": {"N": 1024, "H": 1024, "dtype": "f32", "ln_bwd": {"GBps": 1004.0}},
    }
    bench.same_size_ceilings(None, None, shapes)
    # a and b have the same tensor size (16 MiB): timed once; c is 4 MiB
    assert timed == [(16 << 20, ("copy",)), (4 << 20, ("copy",))]
    assert shapes["a"]["copy_same_size_GBps"] == 1016.0
    assert shapes["a"]["ln_fwd"]["pct_copy_same_size"] == 50.0
    assert shapes["b"]["rms_fwd"]["pct_copy_same_size"] == 200.0
    assert shapes["c"]["ln_bwd"]["pct_copy_same_size"] == 100.0
    bench.same_size_ceilings(None, None, None)   # no shapes timed: nothing to do


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
