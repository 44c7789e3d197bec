"""Static check of compiled gfx950 assembly (built here from this repository's
HIP sources): no instruction reads or overwrites the destination VGPRs of a
load that is still in flight.

LDS loads (and other LGKM-counted operations) complete in issue order and are
covered by `s_waitcnt lgkmcnt(N)`; vector-memory loads and stores likewise by
`s_waitcnt vmcnt(N)`.  Two loads of one counter may target the same register
(the later one lands last); across the two counters they may not.  Loads issued through inline assembly are invisible to
the compiler's own wait insertion, so this is the check that their waits are
where the code assumes.  Tracking is per basic block (any branch or label
resets it), so a load whose wait sits in another block is not followed."""
import re

_VREG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")


def _regs(tok):
    out = set()
    for m in _VREG.finditer(tok):
        if m.group(1) is not None:
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _is_vmem(op):
    return op.startswith(("global_", "buffer_", "flat_", "scratch_"))


def _is_lgkm(op):
    return op.startswith(("ds_", "s_load", "s_buffer_load", "s_memtime", "s_sendmsg"))


def hazards(asm_text):
    """(kernel, line number, instruction, counter) for each access to a
    register an in-flight load still owns."""
    found = []
    kern = None
    lgkm, vm = [], []                    # in-flight ops in issue order: destination registers
    for no, line in enumerate(asm_text.splitlines(), 1):
        s = line.strip()
        if not s or s.startswith(";"):
            continue
        if s.endswith(":") or re.match(r"^[._A-Za-z0-9$]+:", s):
            if re.match(r"^_Z\S+:", s):
                kern = s.split(":")[0]
            lgkm, vm = [], []            # a label: control can enter here from elsewhere
            continue
        if s.startswith("."):
            continue
        parts = [p for p in re.split(r"[\s,]+", s) if p]
        op = parts[0]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                n = int(m.group(1))
                lgkm = lgkm[len(lgkm) - n:] if n else []
            m = re.search(r"vmcnt\((\d+)\)", s)
            if m:
                n = int(m.group(1))
                vm = vm[len(vm) - n:] if n else []
            continue
        if op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_swappc", "s_endpgm")):
            lgkm, vm = [], []
            continue
        dest = _regs(parts[1]) if len(parts) > 1 else set()
        srcs = set()
        for tok in parts[2:]:
            srcs |= _regs(tok)
        is_load = _is_vmem(op) and "load" in op or op.startswith(("ds_read", "ds_bpermute", "ds_permute"))
        touched = srcs | (set() if is_load else dest)
        if _is_vmem(op) and "store" in op or op.startswith("ds_write"):
            touched = srcs | dest        # store data and address are read
        for name, inflight in (("lgkmcnt", lgkm), ("vmcnt", vm)):
            owned = set()
            for d in inflight:
                owned |= d
            if touched & owned:
                found.append((kern, no, s, name))
        if is_load:                      # a new load may not target a register a load of the
            other = vm if op.startswith("ds_") else lgkm    # other counter still owns (loads of one
            owned = set()                                    # counter return in issue order)
            for d in other:
                owned |= d
            if dest & owned:
                found.append((kern, no, s, "vmcnt" if other is vm else "lgkmcnt"))
        if _is_lgkm(op):
            lgkm.append(dest if op.startswith(("ds_read", "ds_bpermute", "ds_permute")) else set())
        elif _is_vmem(op):
            vm.append(dest if "load" in op and "lds" not in s else set())
    return found
