"""Every HIP source of the library, compiled for gfx950 to assembly (device
code only, the library's own flags), passes the in-flight-load check of
`isa_waits`: no instruction touches a register that a load issued before it
still owns.  Plus the check itself must catch waits taken out of real code."""
import os
import shutil
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))
import isa_waits  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_build_script():
    # from its file: importing the package would load the built library
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "slm_build_script", os.path.join(ROOT, "bounded_generation_slm_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_build = _load_build_script()

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in _build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = ["hipcc", *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-o", str(out), src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.mark.parametrize("src", _build.sources(), ids=os.path.basename)
def test_no_access_before_wait(src, tmp_path):
    found = isa_waits.hazards(_asm(src, tmp_path))
    assert not found, "\n".join("%s line %d: %s (%s)" % f for f in found[:10])


def test_check_catches_removed_waits(tmp_path):
    """The packed prefill's assembly with its waits taken out must be flagged
    for both counters."""
    src = [s for s in _build.sources() if s.endswith("prefill_attn.hip")][0]
    text = _asm(src, tmp_path)
    no_lgkm = "\n".join(l for l in text.splitlines() if "lgkmcnt" not in l)
    no_vm = "\n".join(l for l in text.splitlines() if "vmcnt" not in l)
    assert any(f[3] == "lgkmcnt" for f in isa_waits.hazards(no_lgkm))
    assert any(f[3] == "vmcnt" for f in isa_waits.hazards(no_vm))
