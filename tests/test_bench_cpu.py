"""The bench's contract on the CPU: one GPU only, and the algorithmic bytes behind
roofline.achieved (codes + scales per packed token and kv head, plus q and out per launch)."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2 and r.stdout == "" and "one GPU" in r.stderr


@pytest.mark.parametrize("wid,per_token", [(1, 68), (2, 100), (3, 68), (4, 116), (5, 84)])
def test_bytes_per_token_and_head(wid, per_token):
    # K3V3: 48 + 2 + 48 + 2; K2V2: 32 + 2 + 32 + 2; affine K4 g32 / V2 g128: 64 + 16 + 32 + 4; K3V2: 48 + 2 + 32 + 2
    assert bench.bytes_per_token_head(synth.WORKLOADS[wid]) == per_token


def test_headline_layer_bytes():
    w = synth.WORKLOADS[2]
    assert bench.layer_bytes(w, w.N) == 2 * 131072 * 100 + 16 * 128 * 2 + 16 * 128 * 4 == 26_226_688
    w5 = synth.WORKLOADS[5]                     # 256 tokens in the fp16 ring cost 2 x 128 x 2 B each
    assert bench.layer_bytes(w5, w5.N) == 2 * (524032 * 84 + 256 * 512) + 16 * 128 * (2 + 4)


def _hbm_summaries():
    d = os.path.join(ROOT, "profiles")
    return sorted(f for f in os.listdir(d) if f.endswith("_hbm_counters.md"))


@pytest.mark.parametrize("name", _hbm_summaries())
def test_hbm_counter_summaries_carry_what_traffic_reads(name):
    # roofline.traffic comes from these files: each names its commands, the kernel source hash it
    # was taken on, and the calibrated bytes per launch
    import re
    text = open(os.path.join(ROOT, "profiles", name)).read()
    kernel = next(k for k in sorted(bench.KERNEL_SOURCES, key=len, reverse=True) if name.startswith(k + "_"))
    tag = name[len(kernel) + 1:-len("_hbm_counters.md")]
    assert tag in bench.WORKLOAD_TAGS.values()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text and "--copy-probe" in text
    assert re.search(r"sha256\s+`[0-9a-f]{64}`", text)
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    assert t and int(t.group(1)) > 0


def test_traffic_is_null_once_the_kernel_source_changes(tmp_path, monkeypatch):
    # a summary taken on other sources is not read
    wid = 2
    name = f"k_decode_gtq_{bench.WORKLOAD_TAGS[wid]}_hbm_counters.md"
    src = open(os.path.join(ROOT, "profiles", name)).read()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / name).write_text(src.replace(bench.kernel_source_sha("k_decode_gtq"), "0" * 64))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda k: "f" * 64)
    assert bench.measured_traffic(wid, "k_decode_gtq") is None
