"""The layout phase probe (combine_get_dispatch_amd/probes/layout_phases.py)
patches timestamps into a copy of the kernel source at exact anchors.  This
CPU check keeps it in step with the kernels: every anchor must still match
once, and the instrumented copy must hold one mark per phase."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _probe():
    path = os.path.join(ROOT, "combine_get_dispatch_amd", "probes", "layout_phases.py")
    spec = importlib.util.spec_from_file_location("layout_phases", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_layout_phase_probe_anchors_match_the_kernel():
    mod = _probe()
    with open(os.path.join(ROOT, "combine_get_dispatch_amd", "csrc", "ep_kernels.hip")) as f:
        src = f.read()
    out = mod.instrument(src)
    for slot, _, _ in mod.PHASES:
        assert f"s_ts[{slot}] = __builtin_amdgcn_s_memrealtime()" in out, slot
    # Both exits of the layout kernel write the record out.
    assert out.count("FLUSH;") == 2
