"""Host-side checks of the rocprofv3 summary helpers bench.py relies on."""
import json

from lora_mixture_experts_amd import profsum


def test_kernel_labels():
    assert profsum.label("void moelora::k_gemm_skinny<true, 4>(moelora::GemmArgs)") == "gemm_gate_up"
    assert profsum.label("void moelora::k_gemm_skinny<false, 4>(moelora::GemmArgs)") == "gemm_down"
    assert profsum.label("void moelora::k_gemm_dma<128, 192, 2, 2, 2, true>(moelora::GemmArgs)") == "gemm_gate_up"
    assert profsum.label("void moelora::k_gemm_tiled<64, 128, 2, 2, false>(moelora::GemmArgs)") == "gemm_down"
    # the 16-row kernel's flag is its first argument, whatever follows it
    assert profsum.label("void moelora::k_gemm_skinny<false, 4, 2, 1, true>(moelora::GemmArgs)") == "gemm_down"
    assert profsum.label("void moelora::k_gemm_skinny<true, 4, 2, 2, false>(moelora::GemmArgs)") == "gemm_gate_up"
    assert profsum.label("void moelora::k_shrink<2>(moelora::ShrinkArgs)") == "shrink"
    assert profsum.label("__amd_rocclr_copyBuffer") is None


def test_traffic_dropped_when_sources_change(tmp_path):
    p = tmp_path / "t.md"
    blob = dict(workload="decode", source_hash=profsum.kernel_source_hash(), kernels={"gemm_gate_up": 123})
    p.write_text("x\n```json\n" + json.dumps(blob) + "\n```\n")
    assert profsum.read_traffic(str(p), "gemm_gate_up") == 123
    blob["source_hash"] = "0" * 16
    p.write_text("x\n```json\n" + json.dumps(blob) + "\n```\n")
    assert profsum.read_traffic(str(p), "gemm_gate_up") is None
    assert profsum.read_traffic(str(tmp_path / "missing.md"), "gemm_gate_up") is None


def test_traffic_summary_scales_by_reference_dispatch(tmp_path):
    hdr = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,"
           "Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,"
           "SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
    neg = '"void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"'
    gemm = '"void moelora::k_gemm_skinny<true, 4>(moelora::GemmArgs)"'

    def rows(counter, ref, val):
        return hdr + "".join(f'{i},{i},"Agent 1",1,1,1,64,1,{n},64,0,0,8,0,16,"{counter}",{v},0,1\n'
                             for i, (n, v) in enumerate([(neg, ref), (gemm, val), (gemm, val)]))
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    f.write_text(rows("FETCH_SIZE", 512.0, 100.0))   # 1 MiB read shows as 512 KiB: x2
    w.write_text(rows("WRITE_SIZE", 1024.0, 10.0))   # writes counted exactly: x1
    text = profsum.traffic_summary(str(f), str(w), 1, "decode", "cmd")
    blob = json.loads(text.split("```json\n")[1].split("\n```")[0])
    assert blob["fetch_factor"] == 2.0 and blob["write_factor"] == 1.0
    assert blob["kernels"]["gemm_gate_up"] == (200 + 10) * 1024
