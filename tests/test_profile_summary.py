"""Host logic of the rocprofv3 summaries: kernel names map to the families bench.py reports."""
import json
import os

from block_scaled_fp4_hadamard_amd.rocprof_summary import kernel_family, sources_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_families():
    cases = {
        "void mx::quant_kernel<32, 0, 0, true, true>(mx::QuantParams)": "quant.rtne",
        "void mx::quant_kernel<32, 0, 1, true, false>(mx::QuantParams)": "quant.sr",
        "void mx::gemm_full_kernel<0, 1, false>(mx::GemmParams, mx::TileMap, int)": "gemm.bf16",
        "void mx::gemm_full_kernel<1, 0, true>(mx::GemmParams, mx::TileMap, int)": "gemm.f32",
        "void mx::gemm_general_kernel<0, 1>(mx::GemmParams, mx::TileMap)": "gemm.bf16",
        "void mx::mxnorm_kernel<0, 0, 2>(mx::MxNormParams)": "mxnorm",
        "void mx::block16_kernel<1, 0, 0, true>(mx::Block16Params, long)": "nvfp4.col",
        "void mx::block16_kernel<0, 1, 1, false>(mx::Block16Params, long)": "mx16.row",
        "void mx::quant_stats_kernel<32>(mx::QuantStatsParams)": None,
    }
    for name, fam in cases.items():
        assert kernel_family(name) == fam, name


def test_committed_traffic_describes_the_current_kernels():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        traffic = json.load(f)
    assert traffic["sources_hash"] == sources_hash()
    for fam in ("gemm.bf16", "gemm.f32", "quant.rtne", "quant.sr", "mxnorm", "nvfp4.row", "nvfp4.col"):
        assert traffic["families"][fam]["bytes_per_launch"] > 0
