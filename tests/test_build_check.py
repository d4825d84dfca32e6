"""The build's scratch check (nvfp4_weight_quantized_qerl_amd/build.py): it
reads hipcc's kernel-resource-usage remarks and rejects kernels that use
scratch memory beyond the allowlist.  Host-only: the remark text is a
fixture in hipcc's format, nothing is compiled."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location(
    "_qerl_build", os.path.join(ROOT, "nvfp4_weight_quantized_qerl_amd", "build.py"))
build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(build)

REMARKS = """\
./decode_m128.h:146:1: remark: Function Name: _ZN4qerl4d12811decode_m128ILb0ELb1EEEvNS0_4ArgsE [-Rpass-analysis=kernel-resource-usage]
./decode_m128.h:146:1: remark:     TotalSGPRs: 94 [-Rpass-analysis=kernel-resource-usage]
./decode_m128.h:146:1: remark:     VGPRs: 254 [-Rpass-analysis=kernel-resource-usage]
./decode_m128.h:146:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
./decode_lds.h:162:1: remark: Function Name: _ZN4qerl4dlds10decode_ldsILi1ELi5ELb1EEEvNS0_4ArgsE [-Rpass-analysis=kernel-resource-usage]
./decode_lds.h:162:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
./decode_lds.h:162:1: remark:     ScratchSize [bytes/lane]: 516 [-Rpass-analysis=kernel-resource-usage]
./prefill_kernel.h:113:1: remark: Function Name: _ZN4qerl7prefill4gemmILi2ELi4ELi128ELi64ELi2EEEvNS0_4ArgsE [-Rpass-analysis=kernel-resource-usage]
./prefill_kernel.h:113:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_parsed():
    assert build._scratch_users(REMARKS) == [
        ("_ZN4qerl4dlds10decode_ldsILi1ELi5ELb1EEEvNS0_4ArgsE", 516),
        ("_ZN4qerl7prefill4gemmILi2ELi4ELi128ELi64ELi2EEEvNS0_4ArgsE", 12),
    ]


def test_allowlist_admits_only_the_prefill_tile():
    bad = [(k, b) for k, b in build._scratch_users(REMARKS)
           if b > build.SCRATCH_ALLOWED.get(k, 0)]
    assert bad == [("_ZN4qerl4dlds10decode_ldsILi1ELi5ELb1EEEvNS0_4ArgsE", 516)]


def test_remarks_requested():
    assert "-Rpass-analysis=kernel-resource-usage" in build.COMMON
