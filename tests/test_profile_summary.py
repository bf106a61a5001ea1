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
        "void mx::gemm_full_kernel<1, 0, true>(mx::GemmParams, mx::TileMap, int)": "gemm.e1m2.f32",
        "void mx::gemm_general_kernel<0, 1>(mx::GemmParams, mx::TileMap)": "gemm.bf16",
        "void mx::gemm_full_kernel<0, 1, false, 2, true>(mx::GemmParams, mx::TileMap, int)": "gemm.bf16",
        "void mx::gemm_full_kernel<0, 0, true, 2, false>(mx::GemmParams, mx::TileMap, int)": "gemm.f32",
        "void mx::gemm_full_kernel<1, 1, false, 2, true>(mx::GemmParams, mx::TileMap, int)": "gemm.e1m2.bf16",
        "void mx::gemm_general_kernel<1, 0>(mx::GemmParams, mx::TileMap)": "gemm.e1m2.f32",
        "void mx::mxnorm_kernel<0, 0, 2>(mx::MxNormParams)": "mxnorm",
        "void mx::block16_kernel<1, 0, 0, true>(mx::Block16Params, long)": "nvfp4.col",
        "void mx::block16_kernel<0, 1, 1, false>(mx::Block16Params, long)": "mx16.row",
        "void mx::quant_stats_kernel<32, 0, false, true>(mx::QuantStatsParams)": "diag",
        "void mx::rotate_kernel<32>(mx::RotateParams)": "rotate",
    }
    for name, fam in cases.items():
        assert kernel_family(name) == fam, name


def test_committed_traffic_file_and_staleness():
    """profiles/traffic.json holds positive byte counts per family and the hash of the kernel sources it was
    measured on; bench.py reports its figure only while that hash matches the current sources (traffic null
    otherwise, so a stale counter run is never attached to changed kernels)."""
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        traffic = json.load(f)
    assert len(traffic["sources_hash"]) == 16
    for fam in ("gemm.bf16", "gemm.f32", "quant.rtne", "quant.sr"):
        assert traffic["families"][fam]["bytes_per_launch"] > 0
    got = bench.load_traffic("gemm.bf16")
    if traffic["sources_hash"] == sources_hash():
        assert got == traffic["families"]["gemm.bf16"]["bytes_per_launch"]
    else:
        assert got is None
