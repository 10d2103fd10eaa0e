"""Host-side logic of bench.py, checked without a GPU: the one-GPU guard, the
algorithmic byte and flop accounting behind the roofline figures (against
numbers worked out by hand for a tiny model), and the scaling of rocprofv3
byte counters by a copy of known size."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


TINY = configs.ModelConfig(n_layers=2, hidden=64, n_heads=2, n_kv_heads=1, head_dim=32, n_experts=4, top_k=2,
                           expert_ffn=32, vocab=128, canvas_len=8, window=16, global_layer_mask=0b10,
                           dtype="bf16")
TINY_W = configs.Workload(name="tiny", model=TINY, batch=1, prompt_len=32, n_steps=2, seed=0)


def test_algorithmic_bytes_and_flops_by_hand(bench):
    # M = 8 rows, H = 64, q 64 / kv 32 wide, F = 32, E = 4, k = 2, V = 128, bf16.
    # Per layer: attention-side weights (64*128 + 64*64 + 64*4) * 2 = 25088 B;
    # touched experts + the shared one, 3 matrices of 64 x 32: (t + 1) * 12288 B;
    # prompt K and V of the visible positions (16 on the sliding-window layer 0,
    # all 32 on the global layer 1): 128 B per position; four norm vectors 512 B.
    # Touched 3 and 4: 76800 + 91136 B; the tied head 128*64*2 + 64*2 + 8*64*2.
    byts, flops, gu_bytes, gu_flops = bench.algorithmic(TINY_W, [3, 4])
    assert byts == 76800 + 91136 + 17536
    # GEMMs 2 * 8 * (8192 + 4096 + 256 + 3 * 3 * 2048) per layer, attention
    # 4 * 8 * 2 * 32 * (keys + 8 canvas keys), LM head 2 * 8 * 64 * 128
    assert flops == 2 * 495616 + 2048 * 24 + 2048 * 40 + 131072
    # one gate|up launch: (t + 1) gate|up weights of 2 * 64 * 32, the A rows
    # (8 x 64) and the u rows written (8 * 2 routed + 8 shared, 32 wide), mean
    # over the two layers
    assert gu_bytes == ((4 * 8192 + 1024 + 1536) + (5 * 8192 + 1024 + 1536)) / 2
    assert gu_flops == 2 * 24 * 64 * 2 * 32


def test_mxfp4_experts_count_four_and_a_quarter_bits(bench):
    m = configs.ModelConfig(**{**TINY.__dict__, "expert_format": "mxfp4"})
    w = TINY_W.replace(model=m)
    b_native = bench.algorithmic(TINY_W, [3, 4])[0]
    b_mx = bench.algorithmic(w, [3, 4])[0]
    experts = (4 + 5) * 3 * 64 * 32  # weights of the touched + shared experts over both layers
    assert b_native - b_mx == pytest.approx(experts * (2 - (0.5 + 1 / 32)))


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, counter, value) in enumerate(rows):
            fh.write(f'{i},"{kernel}",{counter},{value}\n')


def test_counter_summary_scales_by_the_copy(bench, tmp_path, monkeypatch):
    gu = "void (anonymous namespace)::k_stream<unsigned short, 2, 2, 1, 8, 32, 0>(StreamArgs, EpiArgs)"
    down = "void (anonymous namespace)::k_stream<unsigned short, 2, 4, 2, 2, 32, 0>(StreamArgs, EpiArgs)"
    # the copy of 512 MiB reads half its bytes in FETCH_SIZE units (scale 2) and
    # writes all of them in WRITE_SIZE units (scale 1); down launches are ignored
    _counter_csv(tmp_path / "cf", [(bench.COPY_KERNEL, "FETCH_SIZE", 262144.0)] * 2)
    _counter_csv(tmp_path / "cw", [(bench.COPY_KERNEL, "WRITE_SIZE", 524288.0)] * 2)
    _counter_csv(tmp_path / "gf", [(gu, "FETCH_SIZE", 1000.0), (gu, "FETCH_SIZE", 3000.0),
                                   (down, "FETCH_SIZE", 99999.0)])
    _counter_csv(tmp_path / "gw", [(gu, "WRITE_SIZE", 10.0), (gu, "WRITE_SIZE", 30.0)])
    out_file = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(out_file))
    bench.summarize_counters(str(tmp_path / "gf"), str(tmp_path / "gw"), str(tmp_path / "cf"),
                             str(tmp_path / "cw"), 512)
    c = json.loads(out_file.read_text())
    assert c["fetch_scale"] == 2.0 and c["write_scale"] == 1.0
    assert c["dispatches"] == [2, 2]
    assert c["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert c["write_bytes_per_launch"] == 20 * 1024
    assert c["traffic_bytes_per_launch"] == 2000 * 1024 * 2 + 20 * 1024
    # the summary is honoured only for the kernel sources it was taken with
    assert bench.measured_traffic() == 2000 * 1024 * 2 + 20 * 1024
    c["kernel_sources_sha256"] = "0" * 64
    out_file.write_text(json.dumps(c))
    assert bench.measured_traffic() is None
