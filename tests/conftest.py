import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """Per-test parity counts of the GPU tests (set kinds, tokens in the differences,
    the largest mass slack, outputs accepted through the half-ulp allowance)."""
    mod = sys.modules.get("tests._parity")
    if mod is None or not mod.STATS:
        return
    tot = {}
    terminalreporter.write_line("parity counts (exact / band / valid-alt sets; half-ulp outputs):")
    for name, st in sorted(mod.STATS.items()):
        for k, v in st.items():
            tot[k] = max(tot.get(k, 0), v) if k.startswith("max") else tot.get(k, 0) + v
        if st["band"] or st["valid-alt"] or st["half_ulp_outputs"]:
            terminalreporter.write_line(
                f"  {name}: {st['exact']}/{st['band']}/{st['valid-alt']} sets, "
                f"{st['band_tokens']} band + {st['alt_tokens']} run tokens, mass slack "
                f"{st['max_mass_slack']:.2e}, half-ulp outputs {st['half_ulp_outputs']}")
    terminalreporter.write_line(
        f"  all: {tot.get('exact', 0)} exact, {tot.get('band', 0)} band, "
        f"{tot.get('valid-alt', 0)} valid-alt sets; {tot.get('outputs', 0)} outputs, "
        f"{tot.get('half_ulp_outputs', 0)} through the half-ulp allowance, max |err| "
        f"{tot.get('max_out_err', 0.0):.3g}")
    path = os.environ.get("RTP_PARITY_JSON")
    if path:
        import json
        with open(path, "w") as f:
            json.dump({"tests": mod.STATS, "all": tot}, f, indent=1, sort_keys=True)
