"""The bench's HBM-traffic summary (bench.pmc_summary) on synthetic rocprofv3
counter files: per-call bytes are the sum over the kernels of one call divided
by the number of calls, each counter scaled by its reading for the calibration
copy.  The parallel form launches two query-block kernels per call (the hi+lo
first blocks and the rest); only the second counts the calls."""
import csv
import os

import bench

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(COLS)
        for i, (kernel, value) in enumerate(rows):
            w.writerow([i, kernel, counter, value])


def _summary(tmp_path, name, fetch_rows, write_rows):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", fetch_rows)
    _write(w, "WRITE_SIZE", write_rows)
    bench.pmc_summary(name, str(f), str(w), ["cmd"], out_dir=str(tmp_path))
    vals = {}
    for line in open(os.path.join(tmp_path, f"traffic_{name}.txt")):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = v.strip()
    return vals


def test_parallel_calls_counted_once(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    main = "void ret::qblock_kernel<256, 512, true, false>(ret::RetArgs, ret::TaskGeom, unsigned short const*)"
    first = "void ret::qblock_kernel<256, 512, true, true>(ret::RetArgs, ret::TaskGeom, unsigned short const*)"
    ncalls = 3
    # fetch: the counter reads half the bytes (factor 2), write reads them all
    fetch = [("void at::native::neg_kernel", copy_kib / 2)]
    write = [("void at::native::neg_kernel", copy_kib)]
    for _ in range(ncalls):
        fetch += [(first, 100.0), (main, 900.0)]
        write += [(first, 10.0), (main, 290.0)]
    vals = _summary(tmp_path, "parallel_2k", fetch, write)
    assert float(vals["fetch_kib_per_call"]) == 1000.0
    assert float(vals["write_kib_per_call"]) == 300.0
    assert abs(float(vals["fetch_factor"]) - 2.0) < 1e-9 and abs(float(vals["write_factor"]) - 1.0) < 1e-9
    assert int(vals["hbm_bytes_per_call"]) == (2 * 1000 + 300) * 1024


def test_chunkwise_three_kernels_per_call(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    ks = ["void ret::seg_state_kernel<128, 256>(ret::RetArgs, ret::TaskGeom, float*)",
          "ret::seg_scan_kernel(ret::RetArgs, ret::TaskGeom, float*, float const*, float*)",
          "void ret::seg_out_kernel<128, 256, false, true>(ret::RetArgs, ret::TaskGeom, float const*)"]
    fetch = [("void at::native::neg_kernel", copy_kib / 2)]
    write = [("void at::native::neg_kernel", copy_kib)]
    for _ in range(2):
        fetch += [(k, v) for k, v in zip(ks, (100.0, 20.0, 300.0))]
        write += [(k, v) for k, v in zip(ks, (30.0, 30.0, 130.0))]
    vals = _summary(tmp_path, "chunkwise_32k", fetch, write)
    assert float(vals["fetch_kib_per_call"]) == 420.0
    assert float(vals["write_kib_per_call"]) == 190.0
