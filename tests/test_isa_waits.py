"""Every HIP source of the library, compiled for gfx950 to assembly (device
code only, the library's own flags), passes the in-flight-load check of
`isa_waits`: on no path through a kernel does an instruction touch a register
that a load issued before it still owns, and no kernel whose loads are issued
from inline assembly (waits counted by hand) uses scratch memory.  The check
itself must catch waits taken out of real code and a copy or overwrite of an
in-flight register planted at the persistent prefill's loop back-edge."""
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


_CACHE = {}


def _asm(src, tmp_path):
    if src in _CACHE:
        return _CACHE[src]
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in _build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = ["hipcc", *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-o", str(out), src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    _CACHE[src] = out.read_text()
    return _CACHE[src]


@pytest.mark.parametrize("src", _build.sources(), ids=os.path.basename)
def test_no_access_before_wait(src, tmp_path):
    text = _asm(src, tmp_path)
    found = isa_waits.hazards(text)
    assert not found, "\n".join("%s line %d: %s (%s)" % f for f in found[:10])
    spill = isa_waits.asm_memory_kernels(text) & isa_waits.scratch_users(text)
    assert not spill, "kernels with hand-counted waits use scratch: %s" % sorted(spill)


def test_scratch_detection():
    text = "\n".join(["_Zfoo:", ";;#ASMSTART", "global_load_dwordx4 v[0:3], v[4:5], off", ";;#ASMEND",
                      "scratch_store_dword off, v1, s0", "s_endpgm", ".Lfunc_end0:",
                      ".set _Zbar.private_seg_size, 16"])
    assert isa_waits.asm_memory_kernels(text) == {"_Zfoo"}
    assert isa_waits.scratch_users(text) == {"_Zfoo", "_Zbar"}


_PERSISTENT = "_ZN3slm12_GLOBAL__N_125prefill_persistent_kernelILi128ELi2ELb0EEEvNS_13PrefillParamsE"


def _back_edge_and_q(text):
    """Line index of the persistent kernel's loop back-edge branch and the
    registers of its inline-asm Q loads."""
    lines = text.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(_PERSISTENT + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    labels, q, in_asm, back = {}, set(), False, None
    for i in range(start, end):
        s = lines[i].split(";", 1)[0].strip() if not lines[i].lstrip().startswith(";") else lines[i].strip()
        if s.endswith(":"):
            labels[s[:-1]] = i
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and s.startswith("global_load_dwordx4"):
            q |= isa_waits._regs(s.split()[1].rstrip(","))
        parts = s.split()
        if parts and parts[0].startswith(("s_cbranch", "s_branch")) and parts[-1] in labels:
            back = i                                   # a branch to a label above it
    return back, q


def test_check_catches_loop_edge_copy(tmp_path):
    """At the persistent prefill's loop back-edge the Q rows of the next item
    may still be in flight (loaded at the end of the loop's last step).  A
    copy of one of those registers planted just before the back-edge branch,
    and an overwrite of one, must both be flagged; the unmodified code is clean."""
    src = [s for s in _build.sources() if s.endswith("prefill_attn.hip")][0]
    text = _asm(src, tmp_path)
    back, q = _back_edge_and_q(text)
    assert back is not None and len(q) >= 32
    lines = text.splitlines()
    vm, _ = isa_waits.inflight_at(text, _PERSISTENT, back + 1)
    live = sorted(vm & q)
    assert live, "no Q register in flight at the back-edge"
    assert not [f for f in isa_waits.hazards(text) if f[0] == _PERSISTENT]
    for plant in ("v_mov_b32 v255, v%d" % live[0], "v_mov_b32 v%d, 0" % live[-1],
                  "v_accvgpr_write_b32 a0, v%d" % live[0]):
        planted = "\n".join(lines[:back] + ["\t" + plant] + lines[back:])
        found = [f for f in isa_waits.hazards(planted) if f[0] == _PERSISTENT]
        assert any(f[2] == plant and f[3] == "vmcnt" for f in found), plant


def test_check_catches_removed_waits(tmp_path):
    """The packed prefill's assembly with its waits taken out must be flagged
    for both counters."""
    src = [s for s in _build.sources() if s.endswith("prefill_attn.hip")][0]
    text = _asm(src, tmp_path)
    no_lgkm = "\n".join(l for l in text.splitlines() if "lgkmcnt" not in l)
    no_vm = "\n".join(l for l in text.splitlines() if "vmcnt" not in l)
    assert any(f[3] == "lgkmcnt" for f in isa_waits.hazards(no_lgkm))
    assert any(f[3] == "vmcnt" for f in isa_waits.hazards(no_vm))
