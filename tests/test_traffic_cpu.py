"""The counter-traffic tool maps kernel symbols to the library's launch names
(CPU only; no counters are read)."""
from gated_delta_rule_66_amd.traffic import launch_name


def test_state_kernel_classified_by_its_summary_flag():
    # <T, K, waves, tiles, SUMMARY, OUT, GATE>: only the first bool decides
    assert launch_name("_ZN3kda16kda_state_kernelIDF16bLi128ELi4ELi2ELb0ELb1EEEvNS_11StateParamsE") == "state_output"
    assert launch_name("_ZN3kda16kda_state_kernelIDF16bLi128ELi4ELi2ELb0ELb1ELb1EEEvNS_11StateParamsE") == "state_output"
    assert launch_name("_ZN3kda16kda_state_kernelIDF16bLi128ELi4ELi2ELb0ELb0EEEvNS_11StateParamsE") == "state_output"
    assert launch_name("_ZN3kda16kda_state_kernelIDF16bLi128ELi8ELi2ELb1ELb0EEEvNS_11StateParamsE") == "state_summary"
    assert launch_name("void kda::kda_state_kernel<__bf16, 128, 4, 2, false, true, false>(kda::StateParams)") == \
        "state_output"
    assert launch_name("void kda::kda_state_kernel<__bf16, 128, 8, 2, true, false, false>(kda::StateParams)") == \
        "state_summary"


def test_other_kernels():
    assert launch_name("_ZN3kda16kda_intra_kernelIDF16bLi128ELi128EEEvNS_11IntraParamsE") == "intra_chunk"
    assert launch_name("void kda::kda_scan_kernel<128, false>(kda::ScanParams)") == "segment_scan"
    assert launch_name("_ZN3kda16kda_chunk_kernelIDF16bLi128ELi4ELb1EEEvNS_11ChunkParamsE") == "chunk_summary"
    assert launch_name("_ZN3kda16kda_chunk_kernelIDF16bLi128ELi4ELb0EEEvNS_11ChunkParamsE") == "chunk_output"
    assert launch_name("_ZN3kda17kda_decode_kernelIDF16bLi128ELi128ELi64EEEvNS_12DecodeParamsE") == "decode_step"
    assert launch_name("_ZN3kda23kda_decode_multi_kernelIDF16bLi128ELi128ELi64EEEvNS_17MultiDecodeParamsE") == \
        "decode_steps"
    # the output pass <GATE>, gated or not; the summaries run in the first-pass kernel
    assert launch_name("_ZN3kda16kda_fused_kernelILb1EEEvNS_11FusedParamsE") == "fused_output"
    assert launch_name("_ZN3kda16kda_fused_kernelILb0EEEvNS_11FusedParamsE") == "fused_output"
    assert launch_name("void kda::kda_fused_kernel<true>(kda::FusedParams)") == "fused_output"
    assert launch_name("void kda::kda_fused_kernel<false>(kda::FusedParams)") == "fused_output"
    assert launch_name("_ZN3kda22kda_fused_first_kernelILb0EEEvNS_11FusedParamsES1_") == "fused_summary"
    assert launch_name("void kda::kda_fused_first_kernel<true>(kda::FusedParams, kda::FusedParams)") == "fused_summary"
    assert launch_name("void at::native::vectorized_elementwise_kernel<4>(...)") is None
