"""CPU checks of the text parsers the measurement records rely on."""
from tree_verification_attention_tsw_amd import profiling

SMI = """GPU: 0
    POWER:
        SOCKET_POWER: 1388 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1927 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1891 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_smi_metric_parse():
    watts, mean, clocks = profiling.parse_smi_metric(SMI)
    assert watts == 1388.0
    assert clocks == [1927.0, 1891.0]          # graphics clocks only, not MEM_0
    assert mean == (1927.0 + 1891.0) / 2


def test_smi_metric_parse_missing_fields():
    assert profiling.parse_smi_metric("") is None
    assert profiling.parse_smi_metric(SMI.replace("SOCKET_POWER: 1388 W", "SOCKET_POWER: N/A")) is None


def test_power_cap_parse():
    text = ("======================================= Power Cap ========================================\n"
            "GPU[0]\t\t: Max Graphics Package Power (W): 1400.0\n")
    assert profiling.parse_power_cap(text) == 1400.0
    assert profiling.parse_power_cap("nothing here") is None
