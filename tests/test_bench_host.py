"""Host logic of bench.py (no GPU): the one-GPU refusal and the byte and flop models behind its roofline
objects, checked against hand-counted values."""
import json
import os
import subprocess
import sys

import numpy as np

import hyena_inputs as hi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_algorithmic_bytes_of_the_headline_workload():
    w = hi.WORKLOADS[1]
    T = 4 * 768 * 8192
    # one round trip per order (read u, read x_i, write u_i at 2 bytes) plus the fp32 taps of 768 channels
    assert bench.algorithmic_bytes_per_order(w) == 3 * 2 * T + 4 * 768 * 8192
    assert bench.algorithmic_bytes_per_order(w) * w.order == 352_321_536
    # all orders fused: read v, x_1, x_2, write y, plus both orders' taps
    assert bench.floor_bytes_per_step(w) == 4 * 2 * T + 2 * 4 * 768 * 8192
    assert bench.uses_matrix_cores(w) and not bench.uses_matrix_cores(hi.WORKLOADS[5])


def test_input_dependent_filters_count_one_filter_per_row():
    w = hi.WORKLOADS[7]
    assert bench.algorithmic_bytes_per_order(w) == 3 * 4 * 2 * 128 * 64 ** 3 + 4 * 2 * 128 * 127 ** 3


def test_decode_bytes_per_launch():
    w = hi.WORKLOADS[9]
    rows, N, D = 4 * 768, 2, 768
    # per row: v_t, x_1, x_2 (3 reads), y_t (1 write), 2 history appends, 2 prefix values; per order n
    # history values per row and n taps per channel
    want = 4 * (rows * (3 + 1 + 2 + 2) + N * 128 * (rows + D))
    assert bench.decode_bytes_per_launch(w, 128) == want == 4_030_464


def test_cpu_baseline_runs_on_every_core_of_the_process():
    """The oracle baseline runs on a thread pool over this process's CPU set and says so."""
    w = hi.WORKLOADS[0].with_(B=2, D=8, dims=(1024,))
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    cb = bench.cpu_baseline(w, v, xs, params, budget_s=0.5)
    assert cb["cores"] == len(os.sched_getaffinity(0)) and cb["kind"] == "oracle"
    assert cb["value"] > 0 and isinstance(cb["cpu_model"], str) and cb["cpu_model"]
    assert "rows of the same workload" in cb["sample"]


def test_sampled_parity_of_an_exact_output_is_zero():
    """The bench's own parity check: the oracle's output itself measures (numerically) zero error, and a
    planted mistake in one row shows up in the maximum."""
    from oracle import hyena_oracle as orc
    w = hi.WORKLOADS[0].with_(B=2, D=4, dims=(2048,))
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    hs = [orc.implicit_filter_1d(p, 2048) for p in params]
    y = np.stack([orc.hyena_operator_rows(v[b], [x[b] for x in xs], hs) for b in range(2)])
    rows = [(b, d) for b in range(2) for d in range(4)]
    p = bench.sampled_parity(w, v, xs, params, y, rows)
    assert p["rows"] == 8 and p["max"] < 1e-12
    y[1, 2] *= 1.01
    assert abs(bench.sampled_parity(w, v, xs, params, y, rows)["max"] - 1e-2) < 1e-9
