"""Host logic of bench.py (no GPU): argument refusals, the HBM-traffic files it
reads, and the CPU-baseline sampler."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import time
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

from workloads import config_by_id, make_layer, scaled  # noqa: E402
from workloads.gen import make_activations  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0 and "one GPU" in r.stderr
    assert not r.stdout.strip()  # no JSON line


def test_route_locality_needs_a_t1_workload():
    r = _run("--workload", "prefill", "--route-locality")
    assert r.returncode != 0 and "T=1" in r.stderr


def _pmc_files():
    return sorted(glob.glob(os.path.join(ROOT, "profiles", "*__pmc.txt")))


def _kv(path):
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_every_workload_kernel_has_its_traffic_file():
    names = {os.path.basename(p) for p in _pmc_files()}
    for wl, spec in bench.WORKLOADS.items():
        assert f"{spec['kernel']}__{wl}__pmc.txt" in names, wl


@pytest.mark.parametrize("path", _pmc_files(), ids=os.path.basename)
def test_traffic_files_are_consistent(path):
    kv = _kv(path)
    kernel = os.path.basename(path).split("__")[0]
    assert kv["kernel"].startswith(kernel)
    fetch, write = float(kv["fetch_kib_per_launch"]), float(kv["write_kib_per_launch"])
    ff, wf = float(kv["fetch_factor"]), float(kv["write_factor"])
    # the factors are the 1 GiB copy's bytes over what the counters read for it
    assert abs(ff - 2 ** 20 / float(kv["copy_1gib_fetch_kib"])) < 1e-3
    assert abs(wf - 2 ** 20 / float(kv["copy_1gib_write_kib"])) < 1e-3
    want = (fetch * ff + write * wf) * 1024
    # the files print about six significant digits
    assert abs(float(kv["hbm_bytes_per_launch"]) - want) <= 2e-4 * want
    d, n = kv["dispatches"].split("/")
    assert int(d) == int(n) > 0


def test_traffic_is_withheld_once_the_source_changes(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    current = bench.source_sha("gate_up_gemm")

    def write(wl, sha):
        (prof / f"gate_up_gemm__{wl}__pmc.txt").write_text(
            f"# synthetic\nkernel: gate_up_gemm_kernel\nsource_sha: {sha}\n"
            f"hbm_bytes_per_launch: 123456\n")

    write("fresh", current)
    write("stale", "0" * len(current))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda k: current)
    assert bench.traffic_from_profile("gate_up_gemm", "fresh") == 123456.0
    assert bench.traffic_from_profile("gate_up_gemm", "stale") is None
    assert bench.traffic_from_profile("gate_up_gemm", "missing") is None


def _standin(cid, mode, **kw):
    cfg = scaled(config_by_id(cid), **kw)
    x, _ = make_activations(cfg)
    return types.SimpleNamespace(cfg=cfg, host_layers=[make_layer(cfg, 0)], x_host=x, mode=mode,
                                 act_quant=0, token_ids=None, ntok=kw.get("T", cfg.T))


class _Clock:
    """A clock that moves only when the stub oracle call runs."""

    def __init__(self):
        self.t = 0.0

    def time(self):
        return self.t


def _fake_oracle(monkeypatch, seconds_per_call):
    from oracle import moe as omoe
    clock = _Clock()
    calls = []

    def block(cfg, layer, x, tokens=None, stats=None, act_quant=0, token_ids=None):
        calls.append((x.shape[0], None if tokens is None else len(tokens)))
        clock.t += seconds_per_call

    monkeypatch.setattr(bench, "time", clock)
    monkeypatch.setattr(omoe, "block_for_config", block)
    return calls


def test_cpu_baseline_runs_the_real_oracle():
    st = _standin(1, "prefill", layers=1)
    t0 = time.time()
    r = bench.cpu_baseline(st, 0.6)
    assert time.time() - t0 >= 0.3
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0


@pytest.mark.parametrize("layers", [1, 3])
def test_cpu_baseline_units_fill_half_the_budget(monkeypatch, layers):
    st = _standin(1, "prefill", layers=layers)  # T = 8: one unit is the whole batch
    calls = _fake_oracle(monkeypatch, 0.25)
    r = bench.cpu_baseline(st, 2.0)
    assert len(calls) == 4 and all(c == (8, 8) for c in calls)  # 4 x 0.25 s reaches 1 s
    assert r["value"] == pytest.approx(4 * 8 / 1.0 / layers)
    assert ("divided by 3 layers" in r["sample"]) == (layers == 3)


def test_cpu_baseline_decode_takes_one_call_per_token(monkeypatch):
    st = _standin(1, "calls", T=1, calls=5)
    calls = _fake_oracle(monkeypatch, 0.3)
    r = bench.cpu_baseline(st, 2.0)
    assert len(calls) == 4 and all(c == (1, None) for c in calls)
    assert r["value"] == pytest.approx(4 / 1.2)
    assert "4 T=1 fp64 oracle calls" in r["sample"]
