"""bench.py's host logic on the CPU: the counter-file readers, the kernel name
parsing behind the traffic record, the traffic guard that drops a counter
figure once the profiled kernel's machine code or the library sources that
pick the kernel change, and the refusal to run on more than one GPU.  Nothing here touches
a GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FP4_M1 = "void tern::(anonymous namespace)::gemv_fp4_kernel<1, false, 5, 1>(unsigned short const*, int)"
B16 = "void tern::(anonymous namespace)::gemv_b16_kernel<true, false, 3>(unsigned short const*, int)"
COPY = "void tern::(anonymous namespace)::stream_kernel<true>(unsigned char const*, unsigned long)"
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int)"


def _counter_csv(d, rows):
    os.makedirs(os.path.join(d, "host", "1"), exist_ok=True)
    with open(os.path.join(d, "host", "1", "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, counter, value) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{value}\n')


def test_pmc_average_takes_the_named_kernel_only(tmp_path):
    d = str(tmp_path / "f")
    _counter_csv(d, [(FP4_M1, "FETCH_SIZE", 100.0), (FP4_M1, "FETCH_SIZE", 300.0),
                     (TORCH, "FETCH_SIZE", 9999.0), (COPY, "FETCH_SIZE", 5.0)])
    avg, names = bench._pmc_average(d, "gemv_fp4_kernel")
    assert avg == {"FETCH_SIZE": 200.0}
    assert names == [FP4_M1]


def test_dominant_kernel_ignores_the_copy_and_foreign_kernels(tmp_path):
    d = str(tmp_path / "f")
    rows = [(B16, "FETCH_SIZE", 1.0)] * 3 + [(FP4_M1, "FETCH_SIZE", 1.0)] * 2 + \
           [(COPY, "FETCH_SIZE", 1.0)] * 9 + [(TORCH, "FETCH_SIZE", 1.0)] * 9
    _counter_csv(d, rows)
    assert bench._dominant_kernel(d) == "gemv_b16_kernel"


def test_dominant_kernel_refuses_a_directory_without_library_kernels(tmp_path):
    d = str(tmp_path / "f")
    _counter_csv(d, [(TORCH, "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench._dominant_kernel(d)


@pytest.mark.parametrize("mangled,want", [
    ("_ZN4tern12_GLOBAL__N_115gemv_fp4_kernelILi1ELb0ELi5ELi1EEEvPKtPKhS3_PKaPKfPviii", "<1, false, 5, 1>"),
    ("_ZN4tern12_GLOBAL__N_115gemv_b16_kernelILb1ELb0ELi3EEEvPKtPKhS3_PKaPKfPviiii", "<true, false, 3>"),
])
def test_template_args_of_a_mangled_kernel_name(mangled, want):
    assert bench._template_args(mangled) == want


def test_traffic_guard_drops_a_record_whose_code_hash_differs(tmp_path, monkeypatch):
    """A counter record whose machine-code hash does not match the current
    library (here: a symbol the library does not have) is not reported."""
    rec = {"w M=1 K=128 N=16": {"kernel_symbols": ["_Z_not_a_kernel"], "kernel_code_sha256": "00",
                                "dispatch_sha256": bench.dispatch_sha256(), "hbm_bytes_per_launch": 1,
                                "profile": "p.md"}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    pytest.importorskip("ternary_weight_matmul_amd", reason="libtern.so not built")
    value, why = bench.measured_traffic("w M=1 K=128 N=16")
    assert value is None and "machine code" in why
    assert bench.measured_traffic("absent")[0] is None


def test_traffic_guard_drops_a_record_of_other_library_sources(tmp_path, monkeypatch):
    tern = pytest.importorskip("ternary_weight_matmul_amd", reason="libtern.so not built")
    funcs = bench.device_functions(tern.library_path())
    sym = sorted(s for s in funcs if "gemv_fp4_kernel" in s)[0]
    rec = {"w": {"kernel_symbols": [sym], "kernel_code_sha256": bench.kernel_code_sha256([sym]),
                 "dispatch_sha256": "0" * 64, "hbm_bytes_per_launch": 7, "profile": "p.md"}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    value, why = bench.measured_traffic("w")
    assert value is None and "library sources" in why
    rec["w"]["dispatch_sha256"] = bench.dispatch_sha256()
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == (7, "p.md")


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_library_source_hash_covers_the_kernel_files(tmp_path, monkeypatch):
    """A change in a kernel file (where the launch shape of a shape is chosen),
    not only in the ABI dispatch, changes the source hash."""
    import shutil
    shutil.copytree(os.path.join(ROOT, bench.DISPATCH_SOURCES), tmp_path / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DISPATCH_SOURCES", "csrc")
    before = bench.dispatch_sha256()
    with open(tmp_path / "csrc" / "tern_gemv_fp4.hip", "a") as f:
        f.write("\n")
    assert bench.dispatch_sha256() != before
