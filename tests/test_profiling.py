"""Host-side checks of the rocprofv3 counter summaries (no GPU): the copy
kernel's calibration and the attribution of each kernel to its pass."""
import csv
import os

from weight_scans_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]

# one bench step of a segmented run, in dispatch order: the calibration copy,
# the forward (state-only pass, combine, full pass), the backward (segment
# pass, combine, fused kernel, finalize)
DISPATCHES = [
    ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>()", 2.0, 1.0),
    ("void gls::(anonymous namespace)::fwd_mfma<128, false, false>(gls::FwdArgs)", 10.0, 0.5),
    ("gls::(anonymous namespace)::seg_combine(float*, float const*, int, int, int)", 3.0, 3.0),
    ("void gls::(anonymous namespace)::fwd_mfma<128, true, true>(gls::FwdArgs)", 20.0, 15.0),
    ("void gls::(anonymous namespace)::bwd_lam<128>(gls::BwdArgs)", 12.0, 1.0),
    ("gls::(anonymous namespace)::seg_combine(float*, float const*, int, int, int)", 7.0, 7.0),
    ("gls::(anonymous namespace)::bwd_f128(gls::BwdArgs)", 40.0, 20.0),
    ("void gls::(anonymous namespace)::finalize_kernel<float>(gls::FinArgs)", 1.0, 0.25),
]


def _write(dirpath, counter, col):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, d in enumerate(DISPATCHES):
            # values in KiB, in units of the copy kernel's counts
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": d[0], "Counter_Name": counter,
                        "Counter_Value": d[col] * 1024.0})


def test_traffic_calibration_and_pass_attribution(tmp_path):
    fdir, wdir = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write(fdir, "FETCH_SIZE", 1)
    _write(wdir, "WRITE_SIZE", 2)
    res = profiling.traffic(fdir, wdir)
    # the copy reads and writes CALIB_BYTES: fetch counts 2 units, write 1
    unit_f = profiling.CALIB_BYTES / (2.0 * 1024.0 * 1024.0)
    unit_w = profiling.CALIB_BYTES / (1.0 * 1024.0 * 1024.0)
    k = res["kernels"]
    # the two combines are told apart by the dispatch before them
    assert "seg_combine (fwd)" in k and "seg_combine (bwd)" in k
    assert abs(k["seg_combine (fwd)"]["fetch_bytes"] - 3.0 * 1024 * 1024 * unit_f) < 1e-3
    assert abs(k["seg_combine (bwd)"]["write_bytes"] - 7.0 * 1024 * 1024 * unit_w) < 1e-3
    assert abs(k["bwd_f128"]["fetch_bytes"] - 40.0 * 1024 * 1024 * unit_f) < 1e-3
    assert k["bwd_lam<128>"]["dispatches"] == 1
