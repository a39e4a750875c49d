"""The rocprofv3 counter summarizer on synthetic CSVs (CPU): per-call figures,
the copy calibration, and the scaling of instruction counts by the share of
launched waves the SQ counters saw."""
import csv
import os

from selective_state_space_31_amd import counters

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]


def write_pass(d, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for did, name, grid, wg, cname, val in rows:
            w.writerow(dict(Correlation_Id=did, Dispatch_Id=did, Agent_Id=1, Queue_Id=1,
                            Process_Id=1, Thread_Id=1, Grid_Size=grid, Kernel_Id=1,
                            Kernel_Name=name, Workgroup_Size=wg, LDS_Block_Size=0,
                            Scratch_Size=0, VGPR_Count=64, SGPR_Count=32, Counter_Name=cname,
                            Counter_Value=val, Start_Timestamp=0, End_Timestamp=1))


def test_per_call_figures(tmp_path):
    k1 = "void ssm::fwd_sum_kernel<ssm::bf16_t, 16>(ssm::FwdArgs<ssm::bf16_t>)"
    k2 = "void ssm::fwd_out_kernel<ssm::bf16_t, 16>(ssm::FwdArgs<ssm::bf16_t>)"
    other = "void at::native::fill_kernel(float*)"
    # each call launches k1 once and k2 twice; 1024 work-items in groups of
    # 256 = 16 waves per dispatch, of which the SQ saw 12; the two passes
    # make different numbers of calls (3 and 5)
    p1, p2 = str(tmp_path / "p1"), str(tmp_path / "p2")
    rows1, rows2 = [], []
    for c in range(3):
        for i, k in enumerate((k1, k2, k2)):
            did = 10 * c + i
            rows1 += [(did, k, 1024, 256, "SQ_WAVES", 12), (did, k, 1024, 256, "SQ_INSTS_VALU", 1200)]
        rows1.append((10 * c + 5, other, 64, 64, "SQ_INSTS_VALU", 7))
    for c in range(5):
        for i, k in enumerate((k1, k2, k2)):
            did = 10 * c + i
            rows2 += [(did, k, 1024, 256, "FETCH_SIZE", 100.0), (did, k, 1024, 256, "WRITE_SIZE", 50.0)]
    write_pass(p1, rows1)
    write_pass(p2, rows2)
    cal = str(tmp_path / "cal")
    # a 1 GiB copy whose FETCH_SIZE reads half its bytes, WRITE_SIZE all of them
    write_pass(cal, [(1, "void at::native::copy_kernel(float*)", 1 << 28, 256, "FETCH_SIZE",
                      524288.0),
                     (1, "void at::native::copy_kernel(float*)", 1 << 28, 256, "WRITE_SIZE",
                      1048576.0)])
    res = counters.summarize("mamba130m_bf16", [p1, p2], [cal])
    assert res["calls_profiled"] == [3, 5]
    assert abs(res["calibration"]["fetch_scale"] - 2.0) < 1e-12
    assert abs(res["calibration"]["write_scale"] - 1.0) < 1e-12
    # per call: three launches x 100 KiB read (x2) and 50 KiB written
    assert res["hbm_read_bytes_per_call"] == 3 * 100 * 1024 * 2.0
    assert res["hbm_write_bytes_per_call"] == 3 * 50 * 1024 * 1.0
    # 1200 instructions counted on 12 of 16 waves: 1600 per dispatch
    k = res["kernels"]["void fwd_sum_kernel<bf16_t, 16>"]
    assert k["waves_launched"] == 16 and abs(k["sq_wave_coverage"] - 0.75) < 1e-12
    assert res["kernels"]["void fwd_out_kernel<bf16_t, 16>"]["launches_per_call"] == 2
    assert abs(res["valu_insts_per_call"] - 3 * 1600) < 1e-9
    assert "fill_kernel" not in " ".join(res["kernels"])
    assert res["kernel_source_sha256_16"] == counters.source_hash("mamba130m_bf16")


def test_source_hash_families():
    assert counters.family("longctx_bf16") == "fwd"
    assert counters.family("mamba130m_bf16_bwd") == "bwd"
    assert counters.family("ssd_mamba2_2p7b_bf16") == "ssd"
    assert counters.family("conv1d_mamba130m_bf16") == "conv"
    assert counters.family("decode_fp32") == "decode"
    # the forward workloads share one hash; the SSD's differs
    assert counters.source_hash("longctx_bf16") == counters.source_hash("mamba2p8b_bf16")
    assert counters.source_hash("longctx_bf16") != counters.source_hash("ssd_mamba2_2p7b_bf16")
