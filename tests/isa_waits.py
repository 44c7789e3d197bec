"""Static check of compiled gfx950 assembly (built here from this repository's
HIP sources): no instruction reads or overwrites the destination VGPRs of a
load that is still in flight.

Loads issued through inline assembly are invisible to the compiler's own wait
insertion: it takes their destination registers as written when the asm
statement ends.  Their waits are counted by hand, and the compiler may still
copy, spill or reuse such a register before that wait (a copy at a loop edge,
made to join two values of a loop-carried variable, is the typical case).
This check follows the in-flight loads through the whole control-flow graph
of every kernel, across branches and loop back-edges, to a fixed point.

Model (the kernels rely on the same one):
  * vector-memory operations (loads, stores, returning atomics, direct-to-LDS
    loads) complete in issue order and are covered by `s_waitcnt vmcnt(N)`;
    LDS operations likewise by `lgkmcnt(N)`.  Scalar-memory loads may complete
    out of order, so they never count towards the age of an LDS load;
  * an in-flight load is kept with its age: how many operations of its counter
    were issued after it on the youngest path.  `vmcnt(N)` retires every
    vector-memory load of age >= N.  Where paths join, a register is in
    flight if it is on any incoming path, with the smallest age;
  * two loads of one counter may target the same register (they land in
    order); across the two counters they may not.

Findings:
  * within the block that issued the load (straight-line code, where the
    hand-counted waits sit), any instruction that reads or writes one of its
    destination registers before the wait retires it;
  * on any path that crosses a block boundary, an instruction that overwrites
    the register, or that copies, moves or spills it (moves, accumulator
    moves, selects, stores) before the wait.  (A consumer such as an MFMA in
    another block is not flagged there: whether its wait ran depends on the
    same run-time conditions as the load, which a path-insensitive analysis
    cannot follow.)

`scratch_users(asm)` lists the kernels that use private (scratch) memory: a
spill of a register that an inline-asm load still owns reads it before the
load lands, so a kernel with hand-issued loads must not spill at all."""
import re

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_LABEL = re.compile(r"^([.$_A-Za-z0-9]+):")
_CAP = 64                            # the 6-bit counters: 64 later operations retire any earlier one


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


def _is_ds(op):
    return op.startswith("ds_")


def _is_smem(op):
    return op.startswith(("s_load", "s_buffer_load", "s_memtime", "s_sendmsg", "s_dcache", "s_scratch_load"))


_BRANCH = ("s_cbranch", "s_branch", "s_setpc", "s_swappc", "s_endpgm")
# what the compiler emits to copy, move or spill a VGPR (lane reads into SGPRs
# are consumers, not copies)
_COPY = ("v_mov_", "v_pk_mov_", "v_accvgpr_", "v_cndmask_", "v_perm_", "v_alignbit", "v_alignbyte")


def _instrs(asm_text):
    """Functions of the listing: name -> [(line number, text)] of labels and
    instructions (directives, comments and blank lines dropped)."""
    funcs, cur, name = {}, None, None
    for no, line in enumerate(asm_text.splitlines(), 1):
        s = line.split(";", 1)[0].strip() if not line.lstrip().startswith(";") else ""
        if not s:
            continue
        m = _LABEL.match(s)
        if m and re.match(r"^_Z\S+$", m.group(1)):
            name = m.group(1)
            cur = funcs.setdefault(name, [])
            continue
        if s.startswith(".Lfunc_end"):
            name, cur = None, None
            continue
        if cur is None:
            continue
        if m:
            cur.append((no, m.group(1) + ":"))
            continue
        if s.startswith("."):
            continue
        cur.append((no, s))
    return funcs


def _blocks(instrs):
    """Basic blocks: [(labels, [(no, text)], successor indices)]."""
    blocks, labels, body = [], [], []
    for no, s in instrs:
        if s.endswith(":"):
            if body:
                blocks.append((labels, body))
                labels, body = [], []
            labels.append(s[:-1])
            continue
        body.append((no, s))
        if s.split()[0].startswith(_BRANCH):
            blocks.append((labels, body))
            labels, body = [], []
    if body or labels:
        blocks.append((labels, body))
    where = {l: i for i, (ls, _) in enumerate(blocks) for l in ls}
    out = []
    for i, (ls, body) in enumerate(blocks):
        succ = []
        last = body[-1][1].split() if body else [""]
        op = last[0]
        if op.startswith("s_branch"):
            succ = [where[last[1]]] if last[1] in where else []
        elif op.startswith("s_cbranch"):
            succ = ([where[last[1]]] if last[1] in where else []) + ([i + 1] if i + 1 < len(blocks) else [])
        elif op.startswith(("s_endpgm", "s_setpc")):
            succ = []
        elif i + 1 < len(blocks):
            succ = [i + 1]
        out.append((ls, body, succ))
    return out


def _parse(s):
    parts = [p for p in re.split(r"[\s,]+", s) if p]
    op = parts[0]
    ret_atomic = _is_vmem(op) and "atomic" in op and re.search(r"\b(sc0|glc)\b", s) is not None
    is_load = (_is_vmem(op) and "load" in op and "lds" not in parts[1:] and "_lds_" not in op) or ret_atomic \
        or op.startswith(("ds_read", "ds_bpermute", "ds_permute", "ds_swizzle"))
    first = _regs(parts[1]) if len(parts) > 1 else set()
    rest = set()
    for tok in parts[2:]:
        rest |= _regs(tok)
    store = (_is_vmem(op) and ("store" in op or ("atomic" in op and not ret_atomic))) or op.startswith(
        ("ds_write", "ds_add", "ds_max", "ds_min", "ds_and", "ds_or", "ds_xor", "ds_inc", "ds_dec"))
    if store or op.startswith("s_"):
        reads, writes = first | rest, set()
    elif op.startswith("v_writelane"):
        reads, writes = first | rest, first       # writes one lane: the rest of the register is kept
    else:
        reads, writes = rest, first
    if op.startswith("v_readlane") or op.startswith("v_readfirstlane"):
        reads, writes = rest, set()               # SGPR destination
    return op, is_load, reads, writes


def _retire(state, n):
    return {r: a for r, a in state.items() if a < n}


def _age(state):
    """One more operation of the entries' counter: every entry ages by one."""
    return {r: a + 1 for r, a in state.items() if a + 1 < _CAP}


def _merge(a, b):
    out = dict(a)
    for r, age in b.items():
        out[r] = min(age, out.get(r, _CAP))
    return out


def _run_block(body, vm, lgkm, kern, found):
    """Transfer over one block.  vm, lgkm: {register: age} inherited from the
    predecessors; returns the state at the block's end.  Registers loaded in
    this block are `local` until the block ends."""
    vm, lgkm = dict(vm), dict(lgkm)
    local = {"vmcnt": set(), "lgkmcnt": set()}
    for no, s in body:
        op, is_load, reads, writes = _parse(s)
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                lgkm = _retire(lgkm, int(m.group(1)))
            m = re.search(r"vmcnt\((\d+)\)", s)
            if m:
                vm = _retire(vm, int(m.group(1)))
            continue
        copy = op.startswith(_COPY) or (not is_load and bool(reads) and (_is_vmem(op) or _is_ds(op)))
        own = "lgkmcnt" if _is_ds(op) else ("vmcnt" if _is_vmem(op) else None)
        for name, st in (("lgkmcnt", lgkm), ("vmcnt", vm)):
            w = writes if not (is_load and name == own) else set()   # same-counter loads land in order
            for r in (reads | w) & set(st):
                if r in local[name] or r in w or copy:
                    found.add((kern, no, s, name))
        if is_load:                          # a load of the other counter may not target an owned register
            other = "vmcnt" if _is_ds(op) else "lgkmcnt"
            if writes & set(vm if other == "vmcnt" else lgkm):
                found.add((kern, no, s, other))
        if _is_ds(op):
            lgkm = _age(lgkm)
            if is_load:
                for r in writes:
                    lgkm[r] = 0
                    local["lgkmcnt"].add(r)
        elif _is_vmem(op):
            vm = _age(vm)
            if is_load:
                for r in writes:
                    vm[r] = 0
                    local["vmcnt"].add(r)
    return vm, lgkm


def _fixpoint(blocks, kern, found):
    """Entry state of every block, to a fixed point over all paths."""
    entry = [None] * len(blocks)
    entry[0] = ({}, {})
    work = [0]
    while work:
        i = work.pop()
        ovm, olg = _run_block(blocks[i][1], *entry[i], kern, found)
        for j in blocks[i][2]:
            new = (dict(ovm), dict(olg)) if entry[j] is None else (_merge(entry[j][0], ovm), _merge(entry[j][1], olg))
            if new != entry[j]:
                entry[j] = new
                if j not in work:
                    work.append(j)
    return entry


def hazards(asm_text):
    """(kernel, line number, instruction, counter) for each access to a
    register an in-flight load still owns, over every path of every kernel."""
    found = set()
    for kern, instrs in _instrs(asm_text).items():
        blocks = _blocks(instrs)
        if blocks:
            _fixpoint(blocks, kern, found)
    return sorted(found, key=lambda f: (f[0] or "", f[1]))


def inflight_at(asm_text, kern, line_no):
    """(vector-memory, LDS) registers that loads may still own just before the
    instruction at `line_no` of kernel `kern`."""
    blocks = _blocks(_instrs(asm_text).get(kern, []))
    if not blocks:
        return set(), set()
    entry = _fixpoint(blocks, kern, set())
    for i, (_, body, _) in enumerate(blocks):
        for k, (no, _) in enumerate(body):
            if no == line_no and entry[i] is not None:
                vm, lg = _run_block(body[:k], *entry[i], kern, set())
                return set(vm), set(lg)
    return set(), set()


def asm_memory_kernels(asm_text):
    """Kernels that issue memory operations from inline assembly (their waits
    are counted by hand)."""
    out, name, in_asm = set(), None, False
    for line in asm_text.splitlines():
        s = line.strip()
        m = _LABEL.match(s)
        if m and re.match(r"^_Z\S+$", m.group(1)):
            name = m.group(1)
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if in_asm and name and s and not s.startswith(";"):
            op = s.split()[0]
            if _is_vmem(op) or _is_ds(op) or _is_smem(op):
                out.add(name)
    return out


def scratch_users(asm_text):
    """Kernels with a private (scratch) segment or scratch instructions."""
    out, name = set(), None
    for line in asm_text.splitlines():
        s = line.strip()
        m = _LABEL.match(s)
        if m and re.match(r"^_Z\S+$", m.group(1)):
            name = m.group(1)
        m = re.match(r"\.set\s+(_Z\S+)\.private_seg_size,\s*(\d+)", s)
        if m and int(m.group(2)) > 0:
            out.add(m.group(1))
        if name and s.split(" ", 1)[0].startswith("scratch_"):
            out.add(name)
    return out
