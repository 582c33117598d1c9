"""CPU tests of the profiler-output helpers (kernel naming and classification)."""
from io_aware_flashattention_flash_amd.profiling import kernel_key, readable_name


def test_mangled_and_demangled_names_classify_alike():
    cases = {
        "_ZN2fa12fwd16_kernelIDF16bLi128ELi64ELi4ELb1ELb0EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<bf16, 128, 64, 4, true, false>", "fwd"),
        "_ZN2fa13bwd_dq_kernelIDF16_Li64ELi64ELi4ELb1EEEvNS_9BwdParamsIT_EE":
            ("fa::bwd_dq_kernel<f16, 64, 64, 4, true>", "bwd_dq"),
        "_ZN2fa15bwd_dkdv_kernelIDF16bLi64ELi4ELi64ELb0EEEvNS_9BwdParamsIT_EE":
            ("fa::bwd_dkdv_kernel<bf16, 64, 4, 64, false>", "bwd_dkdv"),
        "void fa::fwd_fp32_kernel<64, false>(fa::FwdF32Params)": ("fa::fwd_fp32_kernel<64, false>", "fwd_fp32"),
        "void fa::fwd_fp32_split_kernel<64, false, 4>(fa::FwdF32Params)": ("fa::fwd_fp32_split_kernel<64, false, 4>",
                                                                            "fwd_fp32"),
        "_ZN2fa20kvsplit_merge_kernelIDF16bLi128EEEvPKfS2_PT_Pfii": ("fa::kvsplit_merge_kernel<bf16, 128>",
                                                                     "kvsplit_merge"),
        # the forward's last template argument is its launch mode: 0 dense, 1 key-split, 2 masked
        "_ZN2fa12fwd16_kernelIDF16bLi128ELi64ELi4ELb1ELi0EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<bf16, 128, 64, 4, true, 0>", "fwd"),
        "_ZN2fa12fwd16_kernelIDF16bLi128ELi64ELi4ELb0ELi1EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<bf16, 128, 64, 4, false, 1>", "fwd_kvsplit"),
        "_ZN2fa12fwd16_kernelIDF16_Li64ELi64ELi4ELb1ELi2EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<f16, 64, 64, 4, true, 2>", "fwd"),
        # current instances carry one more argument (the split launches of small problems)
        "_ZN2fa12fwd16_kernelIDF16bLi128ELi64ELi4ELb0ELi1ELb0EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<bf16, 128, 64, 4, false, 1, false>", "fwd_kvsplit"),
        "_ZN2fa12fwd16_kernelIDF16bLi64ELi64ELi4ELb1ELi0ELb1EEEvNS_11Fwd16ParamsIT_EE":
            ("fa::fwd16_kernel<bf16, 64, 64, 4, true, 0, true>", "fwd"),
        "_ZN2fa13bwd_dq_kernelIDF16bLi64ELi64ELi4ELb1ELb0ELb0ELb1EEEvNS_9BwdParamsIT_EE":
            ("fa::bwd_dq_kernel<bf16, 64, 64, 4, true, false, false, true>", "bwd_dq"),
        "_ZN2fa15bwd_dkdv_kernelIDF16bLi64ELi4ELi64ELb1ELb0ELb0ELi0ELb0EEEvNS_9BwdParamsIT_EE":
            ("fa::bwd_dkdv_kernel<bf16, 64, 4, 64, true, false, false, 0, false>", "bwd_dkdv"),
        "__amd_rocclr_copyBuffer": ("__amd_rocclr_copyBuffer", None),
    }
    for raw, (pretty, key) in cases.items():
        assert readable_name(raw) == pretty
        assert kernel_key(raw) == key
    assert kernel_key("void fa::fwd16_kernel<__bf16, 64, 64, 4, true, false>(fa::Fwd16Params<__bf16>)") == "fwd"


def test_algorithmic_bytes_move_each_tensor_once():
    from io_aware_flashattention_flash_amd import inputs
    from io_aware_flashattention_flash_amd.profiling import algorithmic_bytes
    w = inputs.WORKLOADS["fwdbwd_bf16_b4h16n2048d64_causal"]
    t = 4 * 16 * 2048 * 64 * 2
    r = 4 * 16 * 2048 * 4
    assert algorithmic_bytes(w, "fwd") == (3 * t, t + r)
    assert sum(algorithmic_bytes(w, "bwd_dkdv")) == 6 * t + 2 * r == sum(algorithmic_bytes(w, "bwd_dq"))
    c1 = inputs.WORKLOADS["fwd_fp32_b1h1n128d64"]
    assert sum(algorithmic_bytes(c1, "fwd_fp32")) == 4 * 128 * 64 * 4 + 128 * 4


def test_decode_algorithmic_bytes():
    """The key-split forward reads Q, K and V once (its fp32 partials are scratch); the merge writes
    O and LSE."""
    from io_aware_flashattention_flash_amd.profiling import DECODE, algorithmic_bytes, workload
    w = workload("decode_bf16_b8h32nq1nk8192d128")
    assert w is DECODE["decode_bf16_b8h32nq1nk8192d128"]
    assert algorithmic_bytes(w, "fwd_kvsplit") == (8 * 32 * (1 + 2 * 8192) * 128 * 2, 0)
    assert algorithmic_bytes(w, "kvsplit_merge") == (0, 8 * 32 * 1 * (128 * 2 + 4))
