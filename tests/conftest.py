import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """One line with what the parity checks compared: attention values (logits and
    outputs) against the oracle, packed codes (with the counted threshold ties) and
    stored norms (bit-exact)."""
    mod = sys.modules.get("gtq_testutil")
    if mod is None:
        return
    s = mod.STATS
    if not (s["attn_checks"] or s["codes"]):
        return
    terminalreporter.write_line(
        f"gtq parity: {s['attn_checks']} attention comparisons ({s['attn_values']} values) within "
        f"1e-4 + 2e-3|ref|; {s['codes']} codes, {s['code_ties']} differing only within 1e-6 of a threshold; "
        f"{s['norms']} norms, {s['norm_mismatches']} not bit-exact")
