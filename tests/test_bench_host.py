"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the HBM
traffic record written from rocprofv3 --pmc counter files (copy calibration,
selection of the roofline kernel's launches, source-hash check)."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, counter, launches):
    """launches: (kernel symbol, grid threads, value) in dispatch order; the
    rows are written shuffled to check that the reader sorts them."""
    os.makedirs(path, exist_ok=True)
    rows = []
    for i, (name, grid, value) in enumerate(launches):
        r = dict.fromkeys(FIELDS, "0")
        r.update(Dispatch_Id=str(i + 1), Correlation_Id=str(i + 1), Grid_Size=str(grid),
                 Kernel_Name=name, Workgroup_Size="256", Counter_Name=counter,
                 Counter_Value=repr(value))
        rows.append(r)
        other = dict(r, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value="1e9")
        rows.append(other)
    rows = rows[1::2] + rows[0::2]
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_record_traffic(bench, tmp_path, monkeypatch):
    key, sources, symbol = bench.TRAFFIC_KERNELS["decode"]
    kern = "void dg::(anonymous namespace)::%s(dg::(anonymous namespace)::SkinnyArgs)" % symbol
    other = "void dg::(anonymous namespace)::gemm_skinny_kernel<16, 2, 1, false, 3, false>(x)"
    sep = "void dg::(anonymous namespace)::transpose_kernel(x)"
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = bench.COPY_BYTES / 1024.0
    write_csv(tmp_path / "copy_FETCH_SIZE", "FETCH_SIZE",
              [("fill", 4096, 1.0), (copy, 4096, gib_kib / 2), (copy, 4096, gib_kib / 2)])
    write_csv(tmp_path / "copy_WRITE_SIZE", "WRITE_SIZE", [(copy, 4096, gib_kib)] * 3)
    # warm-up launches of the same kernel at another grid and at the same grid,
    # the separator, then the roofline launches; a non-library kernel last
    warm = [(kern, 256 * 224, 7.0), (other, 256 * 192, 9.0), (kern, 256 * 256, 5.0)]
    write_csv(tmp_path / "decode_FETCH_SIZE", "FETCH_SIZE",
              warm + [(sep, 256, 1.0)] + [(kern, 256 * 256, 1000.0 + i) for i in range(3)]
              + [("probe", 1024, 3.0)])
    write_csv(tmp_path / "decode_WRITE_SIZE", "WRITE_SIZE",
              warm + [(sep, 256, 1.0)] + [(kern, 256 * 256, 20.0)] * 3)
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"kept": {"bytes_per_launch": 1}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic("decode", str(tmp_path))
    table = json.loads(out.read_text())
    assert table["kept"] == {"bytes_per_launch": 1}
    rec = table[key]
    assert rec["fetch_dispatches"] == 3 and rec["write_dispatches"] == 3
    assert rec["workgroups"] == 256
    assert rec["fetch_calibration"] == pytest.approx(2.0)
    assert rec["write_calibration"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == round(1001.0 * 1024 * 2)
    assert rec["write_bytes"] == 20 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # the record is reported while the sources keep their hash, and only then
    assert bench.recorded_traffic(key, sources) == rec["bytes_per_launch"]
    rec["source_sha256_16"] = "0" * 16
    out.write_text(json.dumps({key: rec}))
    assert bench.recorded_traffic(key, sources) is None


def test_record_traffic_rejects_another_kernel_last(bench, tmp_path, monkeypatch):
    gib_kib = bench.COPY_BYTES / 1024.0
    write_csv(tmp_path / "copy_FETCH_SIZE", "FETCH_SIZE", [("copyBuffer", 1, gib_kib / 2)])
    write_csv(tmp_path / "copy_WRITE_SIZE", "WRITE_SIZE", [("copyBuffer", 1, gib_kib)])
    wrong = "void dg::(anonymous namespace)::gemm_tiled_kernel<256, 1, false, false, false>(x)"
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        write_csv(tmp_path / ("dense_" + c), c, [(wrong, 1024, 5.0)] * 2)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    with pytest.raises(SystemExit, match="expected"):
        bench.record_traffic("dense", str(tmp_path))
    assert not (tmp_path / "traffic.json").exists()
