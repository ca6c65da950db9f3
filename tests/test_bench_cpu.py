"""bench.py host logic that needs no GPU: the one-GPU guard, algorithmic
bytes, the counter-file hash check, and the reference streaming library's
exports and argument checks (no kernel is launched here)."""
import ctypes
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    B = bench.algorithmic_bytes(32768, 4096, 2, 4)
    assert B["fwd"] == 536903684 and B["bwd"] == 805355528
    assert B["pass1"] + B["pass2"] == B["bwd"]
    assert bench.algorithmic_bytes(4194304, 32, 2, 4)["fwd"] == 536871172


def test_traffic_is_dropped_when_the_kernels_change(tmp_path, monkeypatch):
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"k:w": {"bytes_per_launch": 5, "source_hash": "not-the-current-one"},
                             "k:v": {"bytes_per_launch": 7, "source_hash": bench.kernel_source_hash()}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic("k:w") is None
    assert bench.load_traffic("k:v")["bytes_per_launch"] == 7
    assert bench.load_traffic("missing") is None


def test_stream_reference_library_exports_and_rejects_bad_arguments():
    import __graft_entry__ as ge
    ge._ensure_built()
    sys.path.insert(0, os.path.join(ROOT, "bwd_dyt_forward_amd"))
    import build
    lib = ctypes.CDLL(build.STREAM_REF_PATH)
    lib.stream_ref_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.stream_ref_2in1out.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p]
    a = 0x10000
    assert lib.stream_ref_copy(None, a, 64, None) == 1
    assert lib.stream_ref_copy(a, a + 0x1000, 63, None) == 1          # not a multiple of 16
    assert lib.stream_ref_copy(a + 4, a + 0x1000, 64, None) == 1      # misaligned
    assert lib.stream_ref_2in1out(a, None, a + 0x1000, 64, None) == 1
    lib.stream_ref_2in2out.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.stream_ref_3in1out.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    assert lib.stream_ref_2in2out(a, a + 0x1000, a + 0x2000, None, 64, 1, None) == 1
    assert lib.stream_ref_2in2out(a, a + 0x1000, a + 0x2000, a + 0x3004, 64, 0, None) == 1
    assert lib.stream_ref_3in1out(a, a + 0x1000, None, a + 0x2000, 64, 1, None) == 1
    assert lib.stream_ref_3in1out(a, a + 0x1000, a + 0x2000, a + 0x3000, 48 + 1, 0, None) == 1


def test_width_case_filter():
    assert bench.parse_width_cases("bf16:2560,f32:4104+1") == [("bf16", 2560, 0), ("f32", 4104, 1)]
    assert bench.parse_width_cases(None) == list(bench.WIDTH_CASES)
    import pytest
    with pytest.raises(ValueError):
        bench.parse_width_cases("f16:2560")
