"""The kernel resource report's parsing of the compiler's resource remarks
(no compile here: a fixture in the remarks' format)."""

from moe_grouped_gemm_02_amd import resource_usage as ru

FIXTURE = """\
k.hip:28:1: remark: Function Name: _ZN2dg18quant_1x128_kernelILb1EEEvPKtPhPviili [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     TotalSGPRs: 49 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     VGPRs: 46 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:28:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:90:1: remark: Function Name: _ZN2dg18quant_1x128_kernelILb0EEEvPKtPhPviili [-Rpass-analysis=kernel-resource-usage]
k.hip:90:1: remark:     VGPRs: 43 [-Rpass-analysis=kernel-resource-usage]
k.hip:90:1: remark:     ScratchSize [bytes/lane]: 40 [-Rpass-analysis=kernel-resource-usage]
k.hip:90:1: remark:     VGPRs Spill: 9 [-Rpass-analysis=kernel-resource-usage]
"""


def test_parse_remarks():
    ks = ru.parse(FIXTURE)
    assert set(ks) == {"_ZN2dg18quant_1x128_kernelILb1EEEvPKtPhPviili", "_ZN2dg18quant_1x128_kernelILb0EEEvPKtPhPviili"}
    a = ks["_ZN2dg18quant_1x128_kernelILb1EEEvPKtPhPviili"]
    assert a["VGPRs"] == 46 and a["TotalSGPRs"] == 49 and a["Occupancy [waves/SIMD]"] == 8
    assert "Dynamic Stack" not in a  # not a number
    b = ks["_ZN2dg18quant_1x128_kernelILb0EEEvPKtPhPviili"]
    assert b == {"VGPRs": 43, "ScratchSize [bytes/lane]": 40, "VGPRs Spill": 9}


def test_short_names():
    name = ("void dg::(anonymous namespace)::gemm_kernel<dg::(anonymous namespace)::Tile<128, 128, 2, 4, 4>, "
            "0, true, 0, 0>(dg::GemmParams, dg::Schedule)")
    assert ru.short(name) == "gemm_kernel<Tile<128, 128, 2, 4, 4>, 0, true, 0, 0>"
    assert ru.short("void dg::quant_1x128_kernel<true>(unsigned short const*, int)") == "quant_1x128_kernel<true>"
