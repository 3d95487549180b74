"""Host logic of bench.py that runs without a GPU: the refusal of more than one GPU, and the
HBM traffic figure, which is taken from the committed counter summary only while the attention
kernel's sources are the ones the counters were taken on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_committed_traffic_matches_the_current_kernel_sources():
    b = load_bench()
    assert b.measured_traffic() is not None, "profiles/partition_attn_traffic.txt was taken on other kernel sources"


def test_traffic_is_dropped_when_the_sources_change(tmp_path):
    b = load_bench()
    lines = open(b.TRAFFIC_FILE).read().splitlines()
    good = tmp_path / "traffic.txt"
    good.write_text("\n".join(lines) + "\n")
    b.TRAFFIC_FILE = str(good)
    assert b.measured_traffic() == float([l for l in lines if l.startswith("hbm_bytes_per_launch")][0].split(":")[1])
    # one byte more in a copy of a kernel source: another digest, no traffic figure
    src = tmp_path / "attn_kernel.h"
    src.write_bytes(open(b.ATTN_SOURCES[0], "rb").read() + b" ")
    b.ATTN_SOURCES = [str(src)] + b.ATTN_SOURCES[1:]
    b.source_digest.__defaults__ = (b.ATTN_SOURCES,)
    assert b.measured_traffic() is None
    # a summary without the figure, or a missing file: none either
    b.ATTN_SOURCES = load_bench().ATTN_SOURCES
    b.source_digest.__defaults__ = (b.ATTN_SOURCES,)
    bad = tmp_path / "no_figure.txt"
    bad.write_text("\n".join(l for l in lines if not l.startswith("hbm_bytes_per_launch")) + "\n")
    b.TRAFFIC_FILE = str(bad)
    assert b.measured_traffic() is None
    b.TRAFFIC_FILE = str(tmp_path / "missing.txt")
    assert b.measured_traffic() is None
