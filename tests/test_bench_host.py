"""Host logic of bench.py, on the CPU (no GPU is touched): the one-GPU contract, and the table of
measured HBM traffic keyed by a hash of the kernel sources, so that a changed kernel reports null
traffic instead of counter bytes taken on other code."""
import importlib.util
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line


def test_every_traffic_entry_names_a_workload_and_a_hash():
    bm = _bench()
    import gen
    for name, (nbytes, digest) in bm.MEASURED_TRAFFIC.items():
        assert name in gen.CONFIGS
        assert nbytes > 0 and len(digest) == 16 and int(digest, 16) >= 0


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    bm = _bench()
    src = tmp_path / "block_quantized_int8_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "block_quantized_int8_amd", "csrc"), src)
    here = {k: bm.kernel_source_hash(k) for k in bm.KERNEL_SOURCES}
    monkeypatch.setattr(bm, "ROOT", str(tmp_path))
    assert {k: bm.kernel_source_hash(k) for k in bm.KERNEL_SOURCES} == here   # same bytes, same hash
    name = "q4_0_m2048_n4096_k4096"
    nbytes = bm.MEASURED_TRAFFIC[name][0]
    monkeypatch.setitem(bm.MEASURED_TRAFFIC, name, (nbytes, here["block"]))
    assert bm.measured_traffic(name, "block") == nbytes
    # one changed byte in a source the block kernel is built from: no traffic figure
    f = src / "gemm_block.hip"
    f.write_bytes(f.read_bytes() + b"\n")
    assert bm.kernel_source_hash("block") != here["block"]
    assert bm.measured_traffic(name, "block") is None
    # the W8A8 kernel's own source: its kind's hash changes too
    g = src / "gemm_w8a8.hip"
    g.write_bytes(g.read_bytes() + b"\n")
    assert bm.kernel_source_hash("w8a8") != here["w8a8"]
    assert bm.measured_traffic("no_such_workload", "block") is None
