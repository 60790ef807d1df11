"""Host-side checks of the benchmark harness (CPU): the one-GPU refusal, the
algorithmic byte counts of every quantize workload, the buffer-rotation
sizing that keeps inputs out of the last-level cache, the rate arithmetic,
the rocprofv3 summary parsers, and the committed HBM-traffic summaries."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_quantize_byte_counts(monkeypatch):
    """Input read once plus every output written once, per workload: codes,
    scales, zero-points and block scales at their storage sizes."""
    import types
    import torch
    import tensor_quantization_amd as tq
    # building the list only reads the launch stream; nothing is allocated or launched
    monkeypatch.setattr(torch.cuda, "current_stream", lambda: types.SimpleNamespace(cuda_stream=0))
    ops = {o[0]: o[2] for o in bench.quantizers(torch, tq, bench.Inputs())}
    n2, n3, na, nw, n5 = 8192 * 4096, 11008 * 4096, 4096 * 7168, 7168 * 7168, 14336 * 4096
    assert ops["per_token_s8"] == n2 * 2 + n2 + 8192 * 4 == 100_696_064
    assert ops["per_group_u4_g128"] == n3 * 2 + n3 // 2 + (n3 // 128) * (4 + 1) == 114_483_200
    assert ops["fp8_1x128"] == na * 2 + na + (na // 128) * 4 == 88_997_888
    assert ops["fp8_128x128"] == nw * 2 + nw + (nw // (128 * 128)) * 4 == 154_153_216
    assert ops["nvfp4_static_global"] == n5 * 2 + n5 // 2 + n5 // 16 + 4 == 150_470_660
    assert ops["mxfp4"] == n5 * 2 + n5 // 2 + n5 // 32 == 148_635_648


@pytest.mark.parametrize("read_bytes,set_size", [(67_108_864, 134_250_496), (90_177_536, 205_660_416),
                                                 (117_440_512, 150_470_660), (65_536, 200_000)])
def test_buffer_rotation_defeats_the_last_level_cache(read_bytes, set_size):
    n = bench.nsets_for(read_bytes, set_size)
    assert 2 <= n <= 64
    if read_bytes > 1 << 20:           # the large workloads: re-read only after 2x the LLC of other reads
        assert (n - 1) * read_bytes >= 2 * bench.LLC_BYTES
        assert n * set_size >= 1.2e9 or n == 64


def test_rate():
    d = bench.rate(100_696_064, 17.78)
    assert d["GBps"] == pytest.approx(100_696_064 / 17.78e-6 / 1e9, rel=1e-3)
    assert d["frac"] == pytest.approx(d["GBps"] / bench.HBM_PEAK_GBPS, abs=1e-4)


def test_summary_parsers(tmp_path, capsys):
    (tmp_path / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n"
        "k_a,1000,3000\nk_a,5000,9000\nk_b,0,1000\n")
    bench.trace_summary(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    ka = [l for l in out if l.startswith("k_a")][0].split()
    assert ka[1] == "2" and float(ka[2]) == pytest.approx(3.0)      # two dispatches of 2 and 4 us
    (tmp_path / "run_counter_collection.csv").write_text(
        "Kernel_Name,Counter_Name,Dispatch_Id,Counter_Value\n"
        "k_a,FETCH_SIZE,1,10\nk_a,FETCH_SIZE,1,5\nk_a,FETCH_SIZE,2,21\n")
    bench.pmc_summary(str(tmp_path))
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("k_a")][0].split()
    assert row[-2] == "2" and float(row[-1]) == pytest.approx(18.0)  # per dispatch: 15 and 21


@pytest.mark.parametrize("op,alg", [("quant_per_token_s8", 100_696_064), ("quant_per_group_u4_g128", 114_483_200)])
def test_committed_hbm_traffic(op, alg):
    """The committed counter summary of a headline kernel: reported only while
    taken from the current sources, and then within a few percent of the
    algorithmic bytes (no re-reads)."""
    t = bench.read_traffic(op)
    if t is None:
        pytest.skip("the counter summary of %s was taken from other kernel sources: re-take it" % op)
    assert 1.0 <= t / alg <= 1.05
