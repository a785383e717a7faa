"""The build's check that no kernel spills registers to scratch memory: the
parser of the compiler's resource-usage remarks (no compilation here)."""
from dora_fine_tuning_amd import build as B


def test_spill_parser_names_the_spilling_kernel_and_drops_the_remarks():
    log = "\n".join([
        "x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 120 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 456 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:3: warning: unused variable 'q'",
    ])
    bad, kept = B._spills(log)
    assert bad == ["kern_b: 456 bytes/lane"]
    assert kept == "x.hip:20:3: warning: unused variable 'q'"


def test_spill_parser_accepts_a_clean_log():
    assert B._spills("") == ([], "")
    bad, _ = B._spills("k.hip:3:1: remark: Function Name: k [-Rpass-analysis=kernel-resource-usage]\n"
                       "k.hip:3:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]")
    assert bad == []
