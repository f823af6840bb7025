"""The algorithmic bytes bench.py divides by (every roofline figure rests on
them), pinned to the shapes by hand-derived components, and the one-GPU
contract of bench.py.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from autoregressive_codebook_tts_frame_amd import synth  # noqa: E402

# the 28 + 5 layer model: per decoder layer q|k|v 4096 x 1024, o 1024 x 2048,
# gate, up 3072 x 1024 each, down 1024 x 3072
LAYER_PARAMS = 4096 * 1024 + 1024 * 2048 + 3 * 3072 * 1024  # 15,728,640
LAYER_PASSES = 28 + 15 * 5  # talker once, the predictor's 5 layers for each of 15 row passes
HEAD_PARAMS = 16 * 2048 * 1024  # talker head + 15 predictor heads, each read once
KV_ROW = 2 * 8 * 128 * 2  # K and V of 8 heads x 128 dims, bf16: 4,096 bytes per layer-position


def _expected(weight_bytes_per_param: float, batch: int, mean_context: float) -> float:
    weights = (LAYER_PASSES * LAYER_PARAMS + HEAD_PARAMS) * weight_bytes_per_param
    talker_kv = batch * 28 * mean_context * KV_ROW
    predictor_kv = batch * 5 * sum(range(2, 17)) * KV_ROW  # positions 0..1, then 0..j+1 for j = 1..14
    writes = batch * (28 + 5 * 16) * KV_ROW  # one new row per layer pass
    gathers = batch * (16 + 1 + 15) * 1024 * 2  # 16 code rows + the overlay, 15 predictor inputs
    return weights + talker_kv + predictor_kv + writes + gathers


@pytest.mark.parametrize("workload,batch,mean_context,wb,mb", [
    ("bf16_b1", 1, 160.5, 2.0, 3328.9),          # 128-row prompt, 64 frames: keys 129..192
    ("bf16_long_b1", 1, 2048 + 16.5, 2.0, 3547.3),  # 2,048-position prompt, 32 frames
    ("bf16_b32", 32, 1088.5, 2.0, 7406.7),       # 32 streams, mean context 1,088.5
    ("q8_b1", 1, 160.5, 34 / 32, 1778.6),         # 32 int8 + one fp16 scale per 32 weights
    ("q8_b8", 8, 160.5, 34 / 32, 1930.4),
    ("q4_b1", 1, 160.5, 18 / 32, 951.8),          # 32 4-bit codes (16 bytes) + one fp16 scale per 32
    ("q4_b8", 8, 160.5, 18 / 32, 1103.6),
])
def test_frame_bytes_match_the_shapes(workload, batch, mean_context, wb, mb):
    m = synth.WORKLOADS[workload].model
    got = bench.frame_bytes(m, batch, mean_context)
    assert got == pytest.approx(_expected(wb, batch, mean_context), rel=1e-12)
    assert round(got / 1e6, 1) == mb


def test_talker_weight_bytes_of_a_prefill_chunk():
    m = synth.WORKLOADS["bf16_b1"].model
    assert bench.talker_weight_bytes(m) == 28 * LAYER_PARAMS * 2 + 2048 * 1024 * 2


def test_prompt_chunks_of_a_prefill_call():
    # the same positions of every stream still going, a power-of-two bucket,
    # at most 512 rows per chunk, the ring's end cutting the last one
    assert bench.prompt_chunks([2048], 4096) == [(1, 512)] * 4
    assert bench.prompt_chunks([128], 4096) == [(1, 128)]
    assert bench.prompt_chunks([5, 37, 100, 16], 256) == [(4, 128)]
    assert bench.prompt_chunks([600, 40], 4096) == [(2, 256), (1, 512)]
    assert bench.prompt_chunks([300, 40, 129], 4096) == [(3, 128), (2, 256)]
    assert bench.prompt_chunks([4088], 4096) == [(1, 512)] * 8
    assert bench.prompt_chunks([250], 256) == [(1, 256)]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
