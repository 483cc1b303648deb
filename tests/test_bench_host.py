"""Host-side logic of bench.py, no GPU: the one-GPU guard, and the HBM-traffic bookkeeping that turns
rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into bytes per launch (scaled by what the same counters
read for a copy of known size) and stops reporting them once a kernel's source changes."""
import csv
import json
import os
import shutil
import subprocess
import sys

import bench

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def write_counters(run_dir, prefix, counter, kernel, per_dispatch):
    """A p_counter_collection.csv as rocprofv3 writes it (only the columns bench.py reads): each dispatch's
    value split over two dimension rows, plus rows of other kernels that must be ignored."""
    d = os.path.join(run_dir, f"{prefix}.{counter}", "host0")
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        did = 1
        for v in per_dispatch:
            for part in (0.25, 0.75):
                w.writerow({"Dispatch_Id": did, "Kernel_Name": kernel, "Counter_Name": counter,
                            "Counter_Value": v * part})
            w.writerow({"Dispatch_Id": did + 1, "Kernel_Name": "__amd_rocclr_fillBufferAligned",
                        "Counter_Name": counter, "Counter_Value": 12345.0})
            did += 2


def test_traffic_bookkeeping(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    sources = sorted({s for _, _, srcs in bench.TRAFFIC_KERNELS.values() for s in srcs})
    for s in sources:
        os.makedirs(root / os.path.dirname(s), exist_ok=True)
        shutil.copy(os.path.join(REPO, s), root / s)
    os.makedirs(root / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(root))
    run = str(tmp_path / "run")
    copy = "void __amd_rocclr_copyBuffer(unsigned char*, unsigned char*)"
    # a 1 GiB copy whose FETCH_SIZE reads half the bytes moved (the factor the hardware shows) and whose
    # WRITE_SIZE reads all of them
    write_counters(run, "copy", "FETCH_SIZE", copy, [2.0 ** 19] * 3)
    write_counters(run, "copy", "WRITE_SIZE", copy, [2.0 ** 20] * 3)
    pk = "void fa::prefill_bf16_kernel<128, true, false, false, false>(fa::PrefillParams)"
    dk = "void fa::decode_split_kernel<128>(fa::DecodeParams)"
    write_counters(run, "prefill", "FETCH_SIZE", pk, [1000.0, 3000.0])
    write_counters(run, "prefill", "WRITE_SIZE", pk, [500.0, 700.0])
    write_counters(run, "decode", "FETCH_SIZE", dk, [8000.0] * 4)
    write_counters(run, "decode", "WRITE_SIZE", dk, [16.0] * 4)
    write_counters(run, "prefill_c4", "FETCH_SIZE", pk, [4000.0])
    write_counters(run, "prefill_c4", "WRITE_SIZE", pk, [800.0])
    bench.write_traffic(run)

    rec = json.load(open(root / "profiles" / "traffic.json"))
    cal = rec["_calibration"]
    assert cal["read_factor"] == 2.0 and cal["write_factor"] == 1.0
    pf, dc = rec["prefill_bf16_c3"], rec["decode_split_c5"]
    assert pf["dispatches"] == 2 and dc["dispatches"] == 4
    assert pf["fetch_kib"] == 2000.0 and pf["write_kib"] == 600.0
    assert pf["read_bytes"] == 2000.0 * 1024 * 2 and pf["write_bytes"] == 600.0 * 1024
    assert pf["bytes_per_launch"] == pf["read_bytes"] + pf["write_bytes"]
    assert dc["bytes_per_launch"] == 8000.0 * 1024 * 2 + 16.0 * 1024
    c4 = rec["prefill_bf16_c4"]
    assert c4["dispatches"] == 1 and c4["bytes_per_launch"] == 4000.0 * 1024 * 2 + 800.0 * 1024
    # algorithmic bytes of the two workloads: Q, K, V read and O, LSE written; K, V, q read
    assert pf["algorithmic_bytes"] == 4 * 32 * 8192 * 128 * 2 + 32 * 8192 * 4
    assert dc["algorithmic_bytes"] == 2 * 64 * 32 * 8192 * 128 * 2 + 64 * 32 * 128 * 2
    assert c4["algorithmic_bytes"] == pf["algorithmic_bytes"]  # same tensors as c3, another query mix

    assert bench.traffic_from_profiles("prefill_bf16_c3") == pf["bytes_per_launch"]
    assert bench.traffic_from_profiles("decode_split_c5") == dc["bytes_per_launch"]
    assert bench.traffic_from_profiles("no_such_kernel") is None
    # a changed prefill source invalidates the prefill's counters only
    with open(root / "exact_tiled_attention_09_amd/csrc/prefill_bf16.hip", "a") as f:
        f.write("\n// edited\n")
    assert bench.traffic_from_profiles("prefill_bf16_c3") is None
    assert bench.traffic_from_profiles("decode_split_c5") == dc["bytes_per_launch"]
    # and a change to a header both include invalidates both
    with open(root / "exact_tiled_attention_09_amd/csrc/common.h", "a") as f:
        f.write("\n// edited\n")
    assert bench.traffic_from_profiles("decode_split_c5") is None
