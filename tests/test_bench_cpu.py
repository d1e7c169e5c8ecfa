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
