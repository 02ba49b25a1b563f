"""Host-side checks of the benchmark: its refusal of more than one GPU and the
algorithmic counts it divides by."""
import os
import subprocess
import sys

from mla_latent_decode_amd.inputs import DSV3, TINY
from mla_latent_decode_amd.layout import (append_bytes_per_token, cache_bytes_per_token,
                                          decode_flops_per_token, train_attention_flops)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cache_bytes_match_the_layout():
    assert cache_bytes_per_token(DSV3, True) == 1184      # 1024 + 128 + 8 * 4
    assert cache_bytes_per_token(DSV3, False) == 1152
    assert cache_bytes_per_token(TINY, True) == 4 * (32 + 8) + 4 * 2
    assert append_bytes_per_token(DSV3) == 2 * (512 + 64) + 1184
    assert decode_flops_per_token(DSV3) == 2 * 128 * (512 + 64) + 2 * 128 * 512


def test_training_flops_count_every_causal_pair():
    B, T = 2, 5
    pairs = sum(1 for b in range(B) for h in range(DSV3.n_heads) for i in range(T)
                for j in range(i + 1))
    f, bwd = train_attention_flops(DSV3, B, T)
    assert f == 2 * pairs * (192 + 128)
    assert bwd == 2 * pairs * (3 * 192 + 2 * 128)


def test_traffic_from_pmc_counters(tmp_path):
    """The split-KV kernel's HBM bytes from two counter-collection CSVs: each
    counter is scaled by what it reads for the 1 GiB calibration copy, rows of
    one dispatch are summed and dispatches averaged."""
    import bench
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    dec = "void qkmla::(anonymous namespace)::decode_mfma_kernel<true, 4>(Args)"
    plain = "void qkmla::(anonymous namespace)::decode_mfma_kernel<false, 4>(Args)"
    cp = "__amd_rocclr_copyBuffer"
    conv = "void at::native::vectorized_elementwise_kernel<4, bfloat16_copy_kernel_cuda>(int)"
    gib_kib = (1 << 30) / 1024
    fetch = head + "".join([
        f'0,"{conv}",FETCH_SIZE,7\n', f'0,"{cp}",FETCH_SIZE,5\n',  # set-up copies, other sizes
        f'1,"{dec}",FETCH_SIZE,60000\n', f'1,"{dec}",FETCH_SIZE,20000\n',  # one dispatch, 2 rows
        f'2,"{dec}",FETCH_SIZE,82000\n',
        f'3,"{plain}",FETCH_SIZE,1\n'] +
        [f'{d},"{cp}",FETCH_SIZE,{gib_kib * 1.25}\n' for d in (4, 5, 6)])  # counter reads 25% high
    write = head + "".join([
        f'0,"{conv}",WRITE_SIZE,7\n', f'0,"{cp}",WRITE_SIZE,5\n',
        f'1,"{dec}",WRITE_SIZE,4000\n', f'2,"{dec}",WRITE_SIZE,6000\n'] +
        [f'{d},"{cp}",WRITE_SIZE,{gib_kib}\n' for d in (4, 5, 6)])
    (tmp_path / "f.csv").write_text(fetch)
    (tmp_path / "w.csv").write_text(write)
    t = bench.traffic_from_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "w1", 77594624)
    e = t["w1"]
    assert abs(e["fetch_KiB"] - 81000) < 1e-9 and abs(e["write_KiB"] - 5000) < 1e-9
    expect = 81000 * 1024 / 1.25 + 5000 * 1024
    assert abs(e["hbm_bytes_per_launch"] - expect) <= 1
    assert e["kernel_src_sha256_16"] == bench._kernel_src_hash()


def test_default_run_keeps_the_headline_when_the_next_rows_fail(monkeypatch, capsys):
    """The default run takes the headline and the next-row measurements from
    two child processes; a next-row child that dies leaves an error entry and
    the headline line is still printed."""
    import argparse
    import json

    import bench
    calls = []

    def fake_child(part, args, timeout_s):
        calls.append(part)
        if part == "headline":
            return {"metric": bench.METRIC, "value": 1.0}, None
        return None, "the next part exited with status -11"
    monkeypatch.setattr(bench, "_run_child", fake_child)
    args = argparse.Namespace(no_next=False, no_cpu=True)
    bench.run_parts(args)
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert calls == ["headline", "next"]
    assert line["value"] == 1.0 and "status -11" in line["next_rows"]["error"]


def test_default_run_fails_without_a_gpu_headline(monkeypatch):
    import argparse

    import bench
    monkeypatch.setattr(bench, "_run_child", lambda part, args, t: (None, "exited with status 2"))
    try:
        bench.run_parts(argparse.Namespace(no_next=False, no_cpu=True))
    except SystemExit as e:
        assert e.code == 1
    else:
        raise AssertionError("run_parts returned without a headline")
