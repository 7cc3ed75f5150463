"""The bench's HBM-traffic summary (bench.pmc_summary) on synthetic rocprofv3
counter files: per-call bytes are the sum over the kernels of one call divided
by the number of calls, each counter scaled by its reading for the calibration
copy.  The parallel form launches the key rotation and two query-block kernels
per call (the hi+lo first blocks and the rest); only the last counts the calls."""
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
    main = ("void ret::qblock_kernel<256, 512, true, false, true>(ret::RetArgs, ret::TaskGeom, unsigned short const*, "
            "unsigned short const*)")
    first = ("void ret::qblock_kernel<256, 512, true, true, false>(ret::RetArgs, ret::TaskGeom, unsigned short const*, "
             "unsigned short const*)")
    rot = "void ret::rotate_keys_kernel<256>(ret::RetArgs, unsigned short*)"
    ncalls = 3
    # fetch: the counter reads half the bytes (factor 2), write reads them all
    fetch = [("void at::native::neg_kernel", copy_kib / 2)]
    write = [("void at::native::neg_kernel", copy_kib)]
    for _ in range(ncalls):
        fetch += [(rot, 50.0), (first, 100.0), (main, 900.0)]
        write += [(rot, 40.0), (first, 10.0), (main, 290.0)]
    vals = _summary(tmp_path, "parallel_2k", fetch, write)
    assert float(vals["fetch_kib_per_call"]) == 1050.0
    assert float(vals["write_kib_per_call"]) == 340.0
    assert abs(float(vals["fetch_factor"]) - 2.0) < 1e-9 and abs(float(vals["write_factor"]) - 1.0) < 1e-9
    assert int(vals["hbm_bytes_per_call"]) == (2 * 1050 + 340) * 1024


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


def test_util_summary_normalisation(tmp_path):
    """bench.util_summary: per-dispatch averages of the utilisation counters and
    the fractions derived from them (cycles per XCD, MFMA busy per SIMD cycle,
    LDS busy per CU cycle, conflict and wait ratios); kernels of other libraries
    are left out."""
    k = "void ret::qblock_kernel<256, 512, true, false>(ret::RetArgs, ret::TaskGeom, unsigned short const*)"
    cyc = 1000.0  # active cycles per XCD in each dispatch
    simds = bench.N_CU * bench.SIMD_PER_CU
    per_dispatch = {"GRBM_GUI_ACTIVE": cyc * bench.N_XCD, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * cyc * simds,
                    "SQ_LDS_IDX_ACTIVE": 0.5 * cyc * bench.N_CU, "SQ_LDS_BANK_CONFLICT": 0.1 * 0.5 * cyc * bench.N_CU,
                    "SQ_WAIT_INST_LDS": 30.0, "SQ_WAVE_CYCLES": 300.0}
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(COLS)
        for d in range(2):  # two dispatches: the second reads twice the first, averaging to 1.5x
            for c, v in per_dispatch.items():
                w.writerow([d, k, c, v * (1 + d) / 1.5])
                w.writerow([d, "at::native::other_kernel", c, 7.0])
    bench.util_summary("t", str(path), ["cmd"], out_dir=str(tmp_path))
    vals = {}
    for line in open(os.path.join(tmp_path, "util_t.txt")):
        if "=" in line and not line.startswith("#"):
            key, v = line.split("=", 1)
            vals[key.strip()] = v.strip()
    assert vals["kernel"] == k[:110]
    assert vals["dispatches"] == "2"
    assert float(vals["cycles_per_xcd"]) == cyc
    assert abs(float(vals["mfma_busy"]) - 0.25) < 1e-3
    assert abs(float(vals["lds_busy"]) - 0.5) < 1e-3
    assert abs(float(vals["lds_bank_conflict"]) - 0.1) < 1e-3
    assert abs(float(vals["lds_wait"]) - 0.1) < 1e-3


def test_layer_legs_count_library_gemms(tmp_path):
    """The gated layer's legs sum this library's kernels and the hipBLASLt GEMMs of a
    call (Cijk...), counting calls by a kernel that runs once per call."""
    copy_kib = bench.COPY_BYTES / 1024
    gemm = "Custom_Cijk_Alik_Bljk_BBS_BH_Bias_HA_S_SAV_NTD_SK3_UserArgs_MT256x256x64_MI16x16x1_shortname0_gfx950"
    scan = "ret::seg_scan_t_kernel(ret::RetArgs, ret::TaskGeom, float const*, unsigned short*, float const*, flo"
    out = "void ret::qblock_kernel<256, 512, false, false>(ret::RetArgs, ret::TaskGeom, unsigned short const*)"
    fetch = [("void at::native::neg_kernel", copy_kib / 2), ("void at::native::fill_kernel", 5000.0)]
    write = [("void at::native::neg_kernel", copy_kib), ("void at::native::fill_kernel", 5000.0)]
    for _ in range(4):
        fetch += [(gemm, 400.0), (scan, 50.0), (out, 300.0), (gemm, 100.0)]
        write += [(gemm, 200.0), (scan, 25.0), (out, 100.0), (gemm, 60.0)]
    vals = _summary(tmp_path, "msr_layer", fetch, write)
    assert float(vals["fetch_kib_per_call"]) == 850.0
    assert float(vals["write_kib_per_call"]) == 385.0
    assert int(vals["algorithmic_bytes_per_call"]) == bench._alg_bytes_msr()
