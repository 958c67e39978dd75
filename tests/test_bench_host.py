"""Host logic of bench.py on the CPU (no kernel is launched).

* More than one GPU is refused with exit status 2 before anything touches a
  device, whether asked for with --gpus or through a launcher's WORLD_SIZE.
* The roofline's algorithmic byte count of the single-layer prefill equals
  the sizes of the buffers the call must read and write, summed from the
  tensors bench.py actually allocates.
* The oracle baseline leg times a bounded sample and reports what it timed.
"""

import os
import subprocess
import sys

import torch

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, extra_env=None):
    env = dict(os.environ, **(extra_env or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2, r.stderr
    assert "single" in r.stderr and r.stdout == ""
    r = run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, r.stderr


def test_prefill_algorithmic_bytes_are_the_buffers_sizes():
    case, args, T, bytes_, _ = bench.prefill_setup(torch.device("cpu"))
    assert T == 8229 and case["H"] == 32 and case["chunk"] == 64

    def nbytes(t):
        return t.numel() * t.element_size()

    reads = sum(nbytes(args[n]) for n in "qkvgb")             # zero initial state: no state read
    state = nbytes(args["pool"][0])                            # one fp32 state, all heads
    writes = nbytes(args["o"]) + state + state + nbytes(args["track_f32"])   # final, snapshot, fp32 snapshot
    assert bytes_ == reads + writes == 343_877_952


def test_cpu_baseline_times_a_bounded_sample():
    cb = bench.cpu_baseline(wl.single_layer_prefill(), seconds_target=0.01)
    want = min(len(os.sched_getaffinity(0)), 16, 32)
    assert cb["kind"] == "oracle" and cb["cores"] == want and cb["unit"] == "tokens/s"
    assert cb["value"] > 0
    assert 0 < cb["single_core_value"] <= cb["value"] * 1.2   # one core is no faster than all of them
    assert cb["sample"].startswith("first 256 of 8229 tokens")


def test_head_subset_draw_matches_full_draw():
    full = wl.token_inputs(50, 6, 16, 16, "bf16", 3)
    part = wl.token_inputs(50, 6, 16, 16, "bf16", 3, heads=[4, 1])
    for n in "qkvgb":
        assert torch.equal(part[n], full[n][:, [4, 1]])


def test_copy_traffic_ratio_is_read_from_the_committed_profile():
    """The fork copy's HBM-traffic ratio comes from the committed counter
    summary: the kernel reads each of its 64 sources once for its four
    children, so the ratio sits at the one-read-per-source floor (0.625 of
    the algorithmic bytes: 64 of 256 source reads plus all 256 writes),
    within counter noise."""
    import bench
    r = bench.committed_copy_traffic_ratio()
    assert r is not None and 0.62 <= r <= 0.65
