"""CPU checks of the rocprofv3 CSV summarizer that writes the profiles and
the traffic figure bench.py reports: names, per-dispatch means, the scaling
by the reference multiply, and the per-code instruction count."""

import csv
import json
import os

from bit_kv_cache_decode_amd import rocprof_summary as rs

DEC = ("void kivi::(anonymous namespace)::decode_kernel<2, 32, false, 2, false, false>"
       "(kivi::(anonymous namespace)::DecodeArgs, kivi::(anonymous namespace)::EncodeArgs)")
MUL = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, "
       "float, at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >")
APPEND = "_ZN4kivi12_GLOBAL__N_113append_kernelEPKDF16_S2_PDF16_S3_PiPjii"


def _csv(path, rows):
    cols = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_short_names():
    assert rs.short_name(APPEND) == "append_kernel"
    assert rs.short_name(DEC).startswith("void decode_kernel<2, 32, false, 2, false, false>(DecodeArgs")


def test_traffic_scales_by_the_reference_dispatch(tmp_path):
    f, w = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    # the reference multiply over 1 MiB: FETCH reads half the bytes, WRITE all
    _csv(f, [(MUL, 1 << 18, 256, "FETCH_SIZE", 512.0), (MUL, 64, 256, "FETCH_SIZE", 1.0),
             (DEC, 131072, 512, "FETCH_SIZE", 100.0), (DEC, 131072, 512, "FETCH_SIZE", 102.0)])
    _csv(w, [(MUL, 1 << 18, 256, "WRITE_SIZE", 1024.0), (DEC, 131072, 512, "WRITE_SIZE", 4.0)])

    class A:
        fetch_csv, write_csv, workload, copy_mb = f, w, "wl", 1
        fetch_command = write_command = "cmd"
        out, json = str(tmp_path / "t.md"), str(tmp_path / "t.json")
    rs.traffic(A)
    t = json.load(open(A.json))
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    assert t["read_bytes_per_launch"] == 101 * 1024 * 2
    assert t["write_bytes_per_launch"] == 4 * 1024
    assert t["kernel_source_sha256"] == rs.kernel_hash() and "step_bytes_per_launch" not in t
    assert os.path.getsize(A.out) > 0


def test_counters_per_code_and_launch_shapes(tmp_path):
    c = str(tmp_path / "c.csv")
    _csv(c, [(DEC, 131072, 512, "SQ_INSTS_VALU", 1000.0), (DEC, 131072, 512, "SQ_WAVES", 10.0),
             (APPEND, 8192, 1024, "SQ_INSTS_VALU", 5.0), (APPEND, 16384, 1024, "SQ_INSTS_VALU", 7.0)])

    class A:
        csv, workload, command, codes, note = c, "wl", "cmd", 6400, ""
        kernel = rs.DECODE
        out = str(tmp_path / "c.md")
    rs.counters(A)
    text = open(A.out).read()
    assert "10.000 lane-level VALU instructions per code" in text   # 64 * 1000 / 6400
    assert "append_kernel [8 workgroups]" in text and "append_kernel [16 workgroups]" in text
    # the per-code figure for another kernel, chosen by name
    A.kernel, A.out = "append_kernel", str(tmp_path / "d.md")
    rs.counters(A)
    assert "append_kernel: 5 wave-level VALU instructions" in open(A.out).read()  # first shape
