"""Host logic of bench.py, on the CPU: the guard that keeps HBM-traffic
counters from being reported for a kernel other than the one profiled (its
whole translation unit and its register schedule), and the multi-GPU
refusal."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

QUANT = "bit_quantized_jl_amd/csrc/k_quantize_mfma.hip"


def test_translation_unit_lists_every_included_header():
    files = [os.path.relpath(p, ROOT) for p in bench.translation_unit_files(bench.QUANT_KERNEL_SRC)]
    assert files[0] == QUANT
    for header in ("bit_quantized_jl_amd/csrc/device_common.h",
                   "bit_quantized_jl_amd/csrc/qjl_internal.h",
                   "bit_quantized_jl_amd/csrc/mfma_image.h", "include/qjl.h"):
        assert header in files, header
    assert len(files) == len(set(files))


def _copy_sources(tmp_path):
    dst = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "bit_quantized_jl_amd", "csrc"),
                    dst / "bit_quantized_jl_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    return dst


@pytest.mark.parametrize("edited", ["bit_quantized_jl_amd/csrc/device_common.h",
                                    "bit_quantized_jl_amd/csrc/qjl_internal.h",
                                    "bit_quantized_jl_amd/csrc/mfma_image.h", "include/qjl.h",
                                    QUANT])
def test_an_edit_anywhere_in_the_unit_changes_its_hash(tmp_path, edited):
    dst = _copy_sources(tmp_path)
    src = str(dst / QUANT)
    before = bench.kernel_tu_hash(src)
    with open(dst / edited, "a") as f:
        f.write("\n// a comment is an edit too\n")
    assert bench.kernel_tu_hash(src) != before


def test_an_edit_outside_the_unit_keeps_its_hash(tmp_path):
    dst = _copy_sources(tmp_path)
    src = str(dst / QUANT)
    before = bench.kernel_tu_hash(src)
    with open(dst / "bit_quantized_jl_amd/csrc/k_score_mfma.hip", "a") as f:
        f.write("\n// another kernel\n")
    assert bench.kernel_tu_hash(src) == before


def _summary(path, tu_hash, schedule=None, nbytes=612986802):
    lines = ["# synthetic summary", "kernel: quantize_mfma_kernel<128, 256, 4, 2, 4, true, false, false>"]
    if schedule is not None:
        lines.append(f"dense_schedule: {schedule}")
    lines += [f"kernel_tu_sha256_16: {tu_hash}", f"hbm_bytes_per_launch: {nbytes}"]
    path.write_text("\n".join(lines) + "\n")


def test_traffic_is_reported_only_for_the_profiled_unit_and_schedule(tmp_path, monkeypatch):
    summary = tmp_path / "pmc.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summary))
    monkeypatch.delenv("QJL_DENSE_SCHEDULE", raising=False)
    current = bench.kernel_tu_hash()
    assert bench.read_traffic() is None  # no summary at all

    _summary(summary, current, "default", 612986802)
    assert bench.read_traffic() == 612986802.0
    _summary(summary, current, None, 612986802)  # older summaries name no schedule: the default
    assert bench.read_traffic() == 612986802.0
    _summary(summary, "0123456789abcdef", "default")  # taken on another version of the unit
    assert bench.read_traffic() is None

    _summary(summary, current, "default")
    for schedule, expect in (("prefetch", None), ("rt4", None), ("immediate", None),
                             ("no such schedule", 612986802.0)):  # unknown value: the default
        monkeypatch.setenv("QJL_DENSE_SCHEDULE", schedule)
        assert bench.dense_schedule() in bench.DENSE_SCHEDULES
        assert bench.read_traffic() == expect, schedule
    _summary(summary, current, "rt4")
    monkeypatch.setenv("QJL_DENSE_SCHEDULE", "rt4")
    assert bench.read_traffic() == 612986802.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_each_schedule_names_the_kernel_its_profile_lists():
    assert set(bench.DENSE_KERNEL_7B) == set(bench.DENSE_SCHEDULES)
    text = open(os.path.join(ROOT, "profiles",
                             "quantize_dense_llama7b_decode_schedules.txt")).read()
    for schedule, kernel in bench.DENSE_KERNEL_7B.items():
        assert f"{schedule:10s} {kernel}" in text, schedule
