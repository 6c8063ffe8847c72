"""A plain C program drives the layer through the C ABI alone.

``tests/c_consumer/moe_layer.c`` is C99 with the HIP runtime's C API for
device memory: no C++, no Python, no torch. Built here with gcc against
``include/`` and the library, it runs on the host without a GPU (version,
workspace query, a rejected shape), and on the GPU the whole forward and
backward of one bf16 layer, whose every output is then held to the same bars
against the fp64 oracle as the layer tests that go through the Python binding.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

from workloads import BF16, bf16_bits_to_f32, make_inputs, small_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "token_dispatch_grouped_amd", "libmoe_mi355x.so")


def _build(tmp_path):
    """A fresh build of the consumer into tmp_path (the host test checks that it compiles cleanly)."""
    if not os.path.exists(LIB):
        pytest.skip("the HIP library is not built")
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    from tests.c_consumer import build as cb
    return cb.build(str(tmp_path / "moe_layer"))


def test_c_consumer_builds_and_runs_on_the_host(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "--host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0].startswith("version moe-mi355x"), lines
    ws = lines[1].split()
    assert ws[0] == "workspace" and ws[1] == "0" and all(int(v) >= 0 for v in ws[2:]), lines
    assert lines[2] == "rejected 1 invalid argument", lines


@pytest.mark.gpu
def test_c_consumer_layer_matches_oracle(tmp_path):
    from tests.test_gpu_parity import compare, oracle_run

    from tests.c_consumer import build as cb
    exe = cb.current()  # built with the library; rebuilt here only if stale
    w = small_workload(600, 256, 8, 2, 192, BF16, "zipf", seed=48, n_empty=2)
    print(f"[c-consumer] T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} {w.dtype}", flush=True)
    inp = make_inputs(w)
    W, mb = inp["weights"], inp["micro"][0]
    T, d, E, k, F = w.T, w.d, w.E, w.k, w.F
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(struct.pack("<qiiii", T, d, E, k, F))
        for arr, dt in ((mb["x"], np.uint16), (mb["logits"], np.float32), (W["w_gu"], np.uint16),
                        (W["w_down"], np.uint16), (mb["dout"], np.uint16)):
            f.write(np.ascontiguousarray(arr, dtype=dt).tobytes())
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    R = T * k
    raw = open(fout, "rb").read()
    pos = 0

    def take(dtype, shape):
        nonlocal pos
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        a = np.frombuffer(raw, dtype=dtype, count=int(np.prod(shape)), offset=pos).reshape(shape)
        pos += n
        return a

    def bf(shape):
        return bf16_bits_to_f32(take(np.uint16, shape)).astype(np.float64)

    g = {}
    g["topk_idx"] = take(np.int32, (T, k))
    g["topk_w"] = take(np.float32, (T, k)).astype(np.float64)
    g["counts"] = take(np.int32, (E,))
    g["offsets"] = take(np.int32, (E + 1,))
    g["row_of_slot"] = take(np.int32, (T, k))
    g["src_of_row"] = take(np.int32, (R,))
    g["x_perm"] = bf((R, d))
    g["h"] = bf((R, 2 * F))
    g["a"] = bf((R, F))
    g["y"] = bf((R, d))
    g["out"] = bf((T, d))
    g["dy"] = bf((R, d))
    g["dtopk_w"] = take(np.float32, (T, k)).astype(np.float64)
    g["dlogits"] = take(np.float32, (T, E)).astype(np.float64)
    g["dx_perm"] = bf((R, d))
    g["dh"] = bf((R, 2 * F))
    g["dx"] = bf((T, d))
    acc = {"dw_gu": take(np.float32, (E, 2 * F, d)).astype(np.float64),
           "dw_down": take(np.float32, (E, d, F)).astype(np.float64)}
    assert pos == len(raw), (pos, len(raw))
    g["dw_unchanged"] = False

    ores, oacc = oracle_run(w, inp)
    compare(w, [g], acc, ores, oacc)
