"""Host-side logic of bench.py (CPU only): the algorithmic byte counts the
roofline uses, the traffic record written from rocprofv3 counter files, the
one-GPU guard, and the workload options' checks and names."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_request_head():
    """K = V = 128, bf16 q/k/v/o, fp32 g and beta, fp32 state: state read and
    written (2 * 4 * 128 * 128 = 131,072 B), q and k 256 B each, v and o
    256 B each, g 512 B and beta 4 B: 132,612 B per (request, head)."""
    assert bench.decode_work(1, 1, 1, 128, 128) == 132612
    assert bench.decode_work(4096, 32, 32, 128, 128) == 132612 * 4096 * 32
    # with raw bf16 gate inputs: g 256 B and b 2 B, plus A_log and dt_bias once
    assert bench.decode_work(1, 1, 1, 128, 128, gate_bytes=2) == 132612 - 258 + 8 * 128
    # GQA: q and k are shared by the value heads of a key head
    assert bench.decode_work(1, 1, 2, 128, 128) == 2 * (132612 - 256)


def test_prefill_bytes_per_token_head():
    """Per (token, head): q, k, v, o 256 B each in bf16, g 512 B, beta 4 B =
    1,540 B; plus the fp32 initial and final state of each (sequence, head)."""
    flops, nbytes = bench.prefill_work([0, 64], 1, 1, 128, 128)
    assert nbytes == 64 * 1540 + 2 * 4 * 128 * 128
    # 6 K V + C (3 K + 2 V) flops per token-head
    assert flops == 64 * (6 * 128 * 128 + 64 * (3 * 128 + 2 * 128))


def test_multi_decode_bytes():
    """One state read per busy request and one written per cached step (the
    pitch caps the cached steps); per token the decode's inputs and o."""
    state = 4 * 128 * 128
    per_tok = 256 + 256 + 256 + 2 * 129 + 256
    assert bench.multi_decode_work([3, 0, 10], 1, 1, 128, 128, 8, False) == \
        (2 * state + (3 + 8) * state + 13 * per_tok) + 8 * 128
    assert bench.multi_decode_work([3], 1, 1, 128, 128, 8, True) == \
        (2 * state + 3 * state + 3 * per_tok) + 8 * 128


def _write_counters(d, counter, rows):
    os.makedirs(os.path.join(d, "host", "1"), exist_ok=True)
    with open(os.path.join(d, "host", "1", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, value in rows:
            w.writerow([name, counter, value])


def test_traffic_record_from_counter_files(tmp_path):
    """Counters scaled by the 4 GiB copy's reading (here fetch counts half the
    bytes, as on MI355X), per launch, with the decode source's hash; the
    bench reports the record only while that hash matches."""
    copy = "__amd_rocclr_copyBuffer"
    dec = "void " + bench.DECODE_KERNEL + "(kda::DecodeArgs)"
    fused = "void " + bench.FUSED_DECODE_KERNEL + "(kda::DecodeArgs)"
    multi = "void " + bench.MULTI_DECODE_KERNEL + "(kda::DecodeArgs)"
    F, Wd = str(tmp_path / "F"), str(tmp_path / "W")
    _write_counters(F, "FETCH_SIZE", [(copy, 2097152), (dec, 1000.0), (fused, 900.0), (fused, 1100.0),
                                      (multi, 300.0)])
    _write_counters(Wd, "WRITE_SIZE", [(copy, 4194304), (dec, 2000.0), (fused, 2000.0), (fused, 2000.0),
                                       (multi, 4000.0)])
    out = str(tmp_path / "rec.json")
    rec = bench.traffic_record("decode", F, Wd, path=out)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes_per_launch"] == (1000.0 * 2 + 2000.0) * 1024
    assert rec["fused_gate_traffic_bytes_per_launch"] == (1000.0 * 2 + 2000.0) * 1024   # mean of launches
    assert rec["multi_decode_traffic_bytes_per_launch"] == (300.0 * 2 + 4000.0) * 1024
    assert bench.measured_traffic(out) == json.load(open(out))
    rec["kernel_source_sha256_16"] = "0" * 16
    json.dump(rec, open(out, "w"))
    assert bench.measured_traffic(out) is None


def test_traffic_record_needs_each_kernel_once(tmp_path):
    F, Wd = str(tmp_path / "F"), str(tmp_path / "W")
    _write_counters(F, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 2097152)])
    _write_counters(Wd, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 4194304)])
    with pytest.raises(SystemExit):
        bench.traffic_record("decode", F, Wd, path=str(tmp_path / "rec.json"))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args", [["--prefill-workload", "long"], ["--prefill-lengths", "64,128"],
                                  ["--prefill-lengths", "64", "--part", "decode"]])
def test_own_prefill_workloads_need_part_prefill(args):
    """The long-prompt and given-lengths prefills are timed on their own; the
    step (prefill + decode) keeps its fixed workloads."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "--part prefill" in r.stderr


def test_workload_names():
    assert bench.workload_name("decode", False, 0, 256).startswith("recurrent decode: B=256,")
    assert "pool 320 slots" in bench.workload_name("decode", False, 0, 256)
    assert "1 sequence of 32768 tokens" in bench.workload_name("prefill", True, 32768)
    name = bench.workload_name("prefill", False, 192, lengths=[64, 128])
    assert "2 sequences of lengths [64, 128] (T=192)" in name and "pool 3 slots" in name
    both = bench.workload_name("both", False, 38632)
    assert "16 seqs" in both and "B=4096" in both
