"""Checks, on the CPU, the generated assembly (without and with the causal
mask) of the 64-rows-per-wavefront forward's tile loop (exact_io_aware_02_amd/gen_fwd_asm.py) against the
rules the generator states for the hazards it handles itself:

  * every LDS read has landed (s_waitcnt lgkmcnt) before an MFMA or VALU
    instruction reads the registers it writes;
  * an MFMA result is not read or overwritten by a non-MFMA instruction
    within 18 wait states, and the U accumulators are read only after the
    48 wait states of three s_nop 15;
  * a transcendental (v_exp_f32, v_rcp_f32) result is not read by the next
    instruction;
  * a lane mask written by a VALU compare is read 2 wait states later at the
    earliest, and so are the operands of v_permlane32_swap;
  * a VALU write reaches an MFMA operand 2 wait states later at the earliest;
  * M0 and EXEC writes precede the buffer load that uses them by at least 1
    and 5 wait states;
  * the register homes do not overlap, and nothing but the output operands
    is written outside the clobbered registers.

Wait states are counted along the straight-line order of the program (an
s_nop N counts N + 1, every other instruction at least 1).  Across the loop's
back edge a score tile is read a step (a workgroup barrier) after it was
written, which this linear count does not see and does not need to.
"""

import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN_PATH = os.path.join(ROOT, "exact_io_aware_02_amd", "gen_fwd_asm.py")


def _gen():
    spec = importlib.util.spec_from_file_location("_gen_fwd_asm", GEN_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


REG = re.compile(r"\b([vas])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for kind, lo, hi, one in REG.findall(text):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    if re.search(r"\bvcc\b", text):
        out.add(("s", "vcc"))
    return out


def _parse(line):
    """(mnemonic, written registers, read registers) of one instruction."""
    if line.endswith(":"):
        return ("label", set(), set())
    op, _, rest = line.partition(" ")
    args = [a.strip() for a in rest.split(",")] if rest else []
    no_dst = op.startswith(("s_cmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier",
                            "ds_write", "s_setprio", "buffer_store"))
    if op.startswith("buffer_load") and rest.endswith("lds"):
        no_dst = True
    if no_dst or not args:
        return (op, set(), _regs(rest))
    dst = _regs(args[0])
    src = set().union(*[_regs(a) for a in args[1:]]) if len(args) > 1 else set()
    if op == "v_permlane32_swap_b32":  # swaps: both operands are read and written
        dst |= src
        src |= dst
    return (op, dst, src)


def _wait_states(op, line):
    if op == "s_nop":
        return int(line.split()[1]) + 1
    return 1


_VARIANTS = [(c, p) for p in (0, 4, 8, 16) for c in (False, True)]


@pytest.fixture(scope="module", params=_VARIANTS,
                ids=[("causal" if c else "non-causal") + (f"-poly{p}" if p else "") for c, p in _VARIANTS])
def program(request):
    """(generator, program) of one kernel variant; the generator's clobbers()
    is bound to the variant's exponential share."""
    g = _gen()
    causal, poly = request.param
    assert poly == 0 or poly in g.POLY_SHARES
    prog = [ln for ln in g.item_asm(causal, poly)]
    base_clobbers = g.clobbers
    g.clobbers = lambda poly=poly: base_clobbers(poly)
    return g, prog


def test_register_homes_are_disjoint(program):
    g, _ = program
    vhomes = {
        "S": set(range(g.S_BUF[0], g.S_BUF[1] + 64)),
        "W": set(range(g.W_BUF[0], g.W_BUF[1] + 32)),
        "tmp": set(range(g.TMP0, g.TMP0 + 16)),
        "state": set(range(g.ST, g.ST + 16)),
    }
    names = list(vhomes)
    for i, a in enumerate(names):
        for b in names[i + 1:]:
            assert not (vhomes[a] & vhomes[b]), (a, b)
    assert g.FRAG0 + 4 * g.NSLOT == 256


def test_writes_stay_inside_the_clobbers(program):
    g, prog = program
    clob = set()
    for name in re.findall(r'"(\w+)"', g.clobbers()):
        m = re.fullmatch(r"([vas])(\d+)", name)
        if m:
            clob.add((m.group(1), int(m.group(2))))
        elif name == "vcc":
            clob.add(("s", "vcc"))
    for line in prog:
        op, dst, _ = _parse(line)
        if "%[" in line.split(",")[0]:
            continue  # the output operands (and M0) are the compiler's
        for r in dst:
            assert r in clob, (line, r)


def lds_violations(prog):
    """Reads or overwrites of registers an outstanding LDS read writes."""
    out, pending = [], []  # registers written by outstanding LDS reads, oldest first
    for line in prog:
        op, dst, src = _parse(line)
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                keep = int(m.group(1))
                pending = pending[len(pending) - keep:] if keep < len(pending) else pending
            continue
        if op == "label":
            continue
        busy = set().union(*pending) if pending else set()
        if (src & busy) or ((dst & busy) and not op.startswith("ds_read")):
            out.append(line)
        if op.startswith("ds_read"):
            pending.append(dst)
        elif op.startswith("ds_write"):
            pending.append(set())
    return out


def mfma_violations(prog):
    """Non-MFMA reads or writes of an MFMA result within 18 wait states (48
    for the U accumulators read by v_accvgpr_read)."""
    out, recent = [], []  # (registers, wait states since the MFMA issued)
    for line in prog:
        op, dst, src = _parse(line)
        if op == "label":
            continue
        if op.startswith("v_mfma"):
            # an MFMA may read (SrcC) and rewrite an accumulator it chains on
            recent = [(r, w) for r, w in recent if not (r & dst)]
        else:
            for regs, w in recent:
                u = any(k == "a" and n < 128 for k, n in regs) and op == "v_accvgpr_read_b32"
                if w < (48 if u else 18) and (regs & (src | dst)):
                    out.append(line)
        ws = _wait_states(op, line)
        recent = [(r, w + ws) for r, w in recent]
        if op.startswith("v_mfma"):
            recent.append((dst, 0))
    return out


def line_writes(line, reg):
    parts = line.split(None, 1)
    return len(parts) == 2 and parts[0].startswith("s_") and parts[1].split(",")[0].strip() == reg


def short_range_violations(prog):
    out = []
    lines = [ln for ln in prog if not ln.endswith(":")]
    parsed = [_parse(ln) for ln in lines]
    for i, (op, dst, src) in enumerate(parsed):
        def gap_to(j):
            return sum(_wait_states(parsed[k][0], lines[k]) for k in range(i + 1, j))
        if op in ("v_exp_f32", "v_rcp_f32", "v_log_f32") and i + 1 < len(parsed) and (parsed[i + 1][2] & dst):
            out.append(lines[i + 1])
        for j in range(i + 1, min(i + 4, len(parsed))):
            opj, dstj, srcj = parsed[j]
            if op.startswith("v_cmp") and (srcj & dst) and gap_to(j) < 2:
                out.append(lines[j])
            if opj == "v_permlane32_swap_b32" and op.startswith("v_") and (dst & srcj) and gap_to(j) < 2:
                out.append(lines[j])
            if (opj.startswith("v_mfma") and op.startswith("v_") and not op.startswith("v_mfma")
                    and (dst & srcj) and gap_to(j) < 2):
                out.append(lines[j])
        for reg, need in (("m0", 1), ("exec", 5)):
            if line_writes(lines[i], reg) and (reg == "m0" or "-1, 0" in lines[i]):
                j = next((k for k in range(i + 1, len(parsed)) if parsed[k][0].startswith("buffer_load")), None)
                if j is not None and gap_to(j) < need:
                    out.append(lines[j])
    return out


def test_lds_reads_land_before_use(program):
    _, prog = program
    assert lds_violations(prog) == []


def test_mfma_results_settle_before_other_use(program):
    _, prog = program
    assert mfma_violations(prog) == []


def test_short_range_hazards(program):
    _, prog = program
    assert short_range_violations(prog) == []


def test_checks_catch_planted_mistakes(program):
    """Each check rejects a copy of the program with one wait taken out or one
    instruction moved too close (the checks are not vacuous)."""
    _, prog = program
    # an LDS wait removed
    i = next(k for k, ln in enumerate(prog) if ln.startswith("s_waitcnt lgkmcnt(") and prog[k + 1].startswith("v_mfma"))
    assert lds_violations(prog[:i] + prog[i + 1:])
    # a score read right after the MFMA that writes it
    i = next(k for k, ln in enumerate(prog) if ln.startswith("v_mfma_f32_32x32x16_bf16 v[0:15]"))
    assert mfma_violations(prog[:i + 1] + ["v_max_f32 v200, v0, v1"] + prog[i + 1:])
    # a U accumulator read 20 wait states after the MFMA that writes it
    i = next(k for k, ln in enumerate(prog) if ln.startswith("v_mfma_f32_32x32x16_bf16 a[0:15]"))
    assert mfma_violations(prog[:i + 1] + ["s_nop 15", "s_nop 3", "v_accvgpr_read_b32 v192, a0"] + prog[i + 1:])
    # the nop between a compare and its mask's reader removed
    i = next(k for k, ln in enumerate(prog) if ln.startswith("v_cmp_gt_f32_e64") and prog[k + 1] == "s_nop 1"
             and prog[k + 2].startswith("s_or_b64"))
    assert short_range_violations(prog[:i + 1] + prog[i + 2:])
    # an exponential's result read at once
    i = next(k for k, ln in enumerate(prog) if ln.startswith("v_exp_f32"))
    dst = prog[i].split()[1].rstrip(",")
    assert short_range_violations(prog[:i + 1] + [f"v_add_f32 v200, v200, {dst}"] + prog[i + 1:])
    # the nops after an EXEC change removed
    i = next(k for k, ln in enumerate(prog) if ln.startswith("s_cselect_b64 exec"))
    assert short_range_violations(prog[:i + 1] + prog[i + 2:])


def test_every_exec_change_is_undone_before_vector_work(program):
    _, prog = program
    masked = False
    for line in prog:
        op, _, _ = _parse(line)
        if line_writes(line, "exec"):
            masked = "-1, 0" in line
            continue
        if masked:
            assert op.startswith(("s_", "buffer_load")), f"vector work with EXEC changed: {line}"


def test_prefetch_wait_counts_only_later_instructions(program):
    """An item waits for the loads its predecessor prefetched with
    s_waitcnt vmcnt(k), where k is the number of VMEM instructions issued
    after them (vmcnt falls in issue order): the predecessor's stores after
    its last prefetch load, plus this item's V_0 loads before the wait,
    counting a load with no lane active as issued or not."""
    g, prog = program
    last = max(i for i, ln in enumerate(prog) if ln.startswith("buffer_load"))
    assert "%[nqrsrc]" in prog[last] or "%[nklo]" in "".join(prog[last - 40:last])
    stores = sum(1 for ln in prog[last + 1:] if ln.startswith("buffer_store"))
    assert not any(ln.startswith("buffer_load") for ln in prog[last + 1:])
    a = prog.index("L_pre_%=:")
    b = next(i for i in range(a, len(prog)) if prog[i].startswith("s_waitcnt vmcnt("))
    v0 = [ln for ln in prog[a:b] if ln.startswith("buffer_load")]
    masked = sum(1 for i in range(a, b) if prog[i].startswith("s_cselect_b64 exec"))
    assert stores == 18 and len(v0) == 5 and masked == 1
    assert g.VM_AFTER_PREFETCH == stores + len(v0) - masked
    assert f"s_waitcnt vmcnt({g.VM_AFTER_PREFETCH})" in prog
    # the first item of a workgroup waits for all but V_0 (4 or 5 loads)
    assert "s_waitcnt vmcnt(4)" in prog


class _Machine:
    """Symbolic execution of one item's program, enough to follow the LDS
    buffers: the scalar arithmetic and branches that choose tiles and
    buffers, the buffer->LDS loads (which tile of which item lands in which
    buffer), the fragment reads and the MFMAs that consume them.  All four
    wavefronts run the same program, so a load is visible to every wavefront
    at the first barrier after this wavefront has waited for it."""

    def __init__(self, g, n, pre, mem, item, wave=0, exec0_counts=True, qw0=0):
        self.g, self.n, self.mem, self.item = g, n, mem, item
        # the last 1 KiB block of a tile is loaded by wavefront 0 only; the
        # others issue that load with EXEC = 0, which may or may not count in
        # vmcnt (both are checked)
        self.exec_on = True
        self.exec0_counts = exec0_counts
        self.vregion = g.KV_LDS[2]          # V buffers follow the K buffers
        self.ops = {"%[n]": n, "%[pre]": pre, "%[wbase]": 0, "%[wave]": wave,
                    "%[kb]": 0, "%[vb]": self.vregion, "%[hb]": n * 16384, "%[nhb]": 1 << 24,
                    "%[klo]": 0, "%[vlo]": 0, "%[nklo]": 1 << 28, "%[nvlo]": 1 << 28, "%[khi]": 0, "%[vhi]": 0,
                    "%[nkhi]": 0, "%[nvhi]": 0, "%[n_keys]": 64 * n, "%[qw0]": qw0, "%[c]": 0, "%[theta]": 0}
        self.s = {}
        self.v = {}
        self.slots = {}   # AGPR slot -> tag of the data read into it
        self.fin = False
        self.barriers = 0      # the item's first block (S_0 = K_0 Q^T) follows its first barrier
        self.pv_tiles = set()  # V tiles multiplied into U
        self.errors = []

    def val(self, x):
        x = x.strip()
        if x in self.ops:
            return self.ops[x]
        if x == "m0":
            return getattr(self, "m0", 0)
        if x.startswith("s") and x[1:].isdigit():
            return self.s.get(int(x[1:]), 0)
        return int(x, 0)

    def run(self, prog):
        labels = {ln[:-1]: i for i, ln in enumerate(prog) if ln.endswith(":")}
        pc, scc, steps = 0, 0, 0
        while pc < len(prog):
            steps += 1
            assert steps < 200000
            ln = prog[pc]
            pc += 1
            if ln.endswith(":"):
                continue
            op, _, rest = ln.partition(" ")
            args = [x.strip() for x in rest.split(",")] if rest else []
            if op in ("s_mov_b32", "s_add_u32", "s_sub_u32", "s_mul_i32", "s_lshl_b32", "s_cselect_b32", "s_addc_u32") \
                    and args[0].startswith("s") and args[0][1:].isdigit():
                d = int(args[0][1:])
                if op == "s_mov_b32":
                    r = self.val(args[1])
                elif op == "s_add_u32":
                    r = self.val(args[1]) + self.val(args[2])
                elif op == "s_sub_u32":
                    r = self.val(args[1]) - self.val(args[2])
                    scc = int(r < 0)
                elif op == "s_mul_i32":
                    r = self.val(args[1]) * self.val(args[2])
                elif op == "s_lshl_b32":
                    r = self.val(args[1]) << self.val(args[2])
                elif op == "s_cselect_b32":
                    r = self.val(args[1]) if scc else self.val(args[2])
                else:
                    r = self.val(args[1])
                self.s[d] = r
            elif op == "s_add_u32" and args[0] == "m0":
                self.m0 = self.val(args[1]) + self.val(args[2])
            elif op.startswith("s_cmp_"):
                a_, b_ = self.val(args[0]), self.val(args[1])
                scc = int({"eq": a_ == b_, "lg": a_ != b_, "lt": a_ < b_, "gt": a_ > b_, "ge": a_ >= b_}[op[6:8]])
            elif op == "s_cselect_b64" and args[0] == "exec":
                self.exec_on = bool(scc)
            elif op == "s_mov_b64" and args[0] == "exec":
                self.exec_on = True
            elif op == "s_cbranch_scc1":
                if scc:
                    pc = labels[args[0]]
            elif op == "s_cbranch_scc0":
                if not scc:
                    pc = labels[args[0]]
            elif op == "s_branch":
                pc = labels[args[0]]
            elif op == "v_add_u32" and args[1].startswith("s") and args[2] in ("%[kb]", "%[vb]"):
                self.v[int(args[0][1:])] = self.val(args[1]) + self.ops[args[2]]
            elif op == "s_waitcnt" and "vmcnt" in rest:
                k = int(rest.split("vmcnt(")[1].split(")")[0])
                self.mem.wait(k)
            elif op == "s_barrier":
                self.mem.barrier()
                self.barriers += 1
            elif op == "buffer_load_dwordx4" and rest.endswith("lds"):
                r = int(args[1][2:].split(":")[0])
                base = self.s[r]
                item = self.item + (base >> 28)
                tile = (base & ((1 << 28) - 1)) >> 14
                kind = "K" if self.m0 < self.vregion else "V"
                region = 0 if kind == "K" else self.vregion
                buf = (self.m0 - region) // self.g.TILE
                assert self.m0 % 1024 == 0 and 0 <= buf < 3, (ln, self.m0)
                if self.exec_on:
                    self.mem.load((kind, buf), (kind, item, tile))
                elif self.exec0_counts:
                    self.mem.vmem()
            elif op.startswith("buffer_load") or op.startswith("buffer_store"):
                self.mem.vmem()
            elif op.startswith("ds_read") and ("%[kb]" in ln or "%[vb]" in ln):
                base = self.ops[args[1].split()[0]]
                off = int(ln.split("offset:")[1])
                kind = "K" if base < self.vregion else "V"
                region = 0 if kind == "K" else self.vregion
                buf = (base + off - region) // self.g.TILE
                slot = int(args[0].split("[")[1].split(":")[0])
                self.slots[slot] = self.mem.read((kind, buf))
            elif op == "v_add_u32" and "%[nqvo]" in ln:   # the final block sets up the next item's loads
                self.fin = True
            elif op.startswith("v_mfma"):
                slot = int(args[1].split("[")[1].split(":")[0])
                j = self.s.get(self.g.S_J, 0) if self.barriers > 1 else -1
                if args[0].startswith("v["):   # S_t = K_t Q^T into S buffer t & 1
                    # step j forms S_{j+1}, or completes S_j with the
                    # products its predecessor deferred (the first block: S_0)
                    par = 0 if int(args[0][2:].split(":")[0]) < self.g.S_BUF[1] else 1
                    want = ("K", self.item, j + 1 if par == (j + 1) % 2 else j)
                else:                           # U += V W: V tile j - 1 (the last block: n - 1)
                    want = ("V", self.item, self.n - 1 if self.fin else j - 1)
                    self.pv_tiles.add(want[2])
                if self.slots.get(slot) != want:
                    self.errors.append((ln, self.slots.get(slot), want))
        return self.errors


class _Memory:
    """LDS buffers of one workgroup: per buffer the loads issued into it, in
    order; a load is complete once this wavefront waited for it, and visible
    to every wavefront after the next barrier."""

    def __init__(self):
        self.vm = []          # VMEM instructions in issue order: (buffer or None, tag)
        self.done = 0         # VMEM instructions known complete
        self.visible = 0      # VMEM instructions visible to all wavefronts
        self.reads_since_barrier = set()
        self.errors = []

    def vmem(self):
        self.vm.append((None, None))

    def load(self, buf, tag):
        if buf in self.reads_since_barrier:
            self.errors.append(("load into a buffer read since the last barrier", buf, tag))
        self.vm.append((buf, tag))

    def wait(self, k):
        self.done = max(self.done, len(self.vm) - k)

    def barrier(self):
        self.visible = self.done
        self.reads_since_barrier = set()

    def read(self, buf):
        self.reads_since_barrier.add(buf)
        pending = [t for b, t in self.vm[self.visible:] if b == buf]
        vis = [t for b, t in self.vm[:self.visible] if b == buf]
        if pending:
            return ("in flight",) + tuple(pending)
        return vis[-1] if vis else None


@pytest.mark.parametrize("wave,exec0_counts", [(0, True), (1, True), (1, False), (2, True), (3, False)])
@pytest.mark.parametrize("causal", [False, True])
def test_lds_buffers_hold_the_tiles_each_product_reads(causal, wave, exec0_counts):
    """Sequences of items of 1 to 9 tiles, in a persistent workgroup's order
    (the first item loads its own tiles, later ones use their predecessor's
    prefetch): every MFMA reads the K or V tile that the forward
    multiplies at that step (S_j = K_j Q^T, then O += V_j P_j), no load targets a buffer read since the last barrier, and no
    read races a load still in flight."""
    g = _gen()
    prog = g.item_asm(causal)
    if causal:
        # query tiles qt of 256 rows: n = 4 qt + 4 tiles, this wavefront's
        # rows start at 256 qt + 64 wave (its diagonal tile is 4 qt + wave)
        runs = [[(4 * qt + 4, 256 * qt + 64 * wave) for qt in qts] for qts in ([0, 3, 1, 2], [7, 0], [2, 2, 5])]
    else:
        runs = [[(n, 0) for n in lengths]
                for lengths in ([1, 1, 1, 1], [2, 3, 4, 5], [9, 1, 2, 7, 3], [5, 5, 5], [3, 8, 6, 2, 1, 4], [7])]
    for items in runs:
        mem = _Memory()
        for i, (n, qw0) in enumerate(items):
            m = _Machine(g, n, int(i > 0), mem, i, wave, exec0_counts, qw0)
            errs = m.run(prog)
            assert not errs, (items, i, errs[:3])
            if causal:
                # every product of a tile up to the diagonal one ran, none after it
                assert m.pv_tiles == set(range(min(n, qw0 // 64 + 1))), (items, i, sorted(m.pv_tiles))
        assert not mem.errors, (items, mem.errors[:3])


def test_buffer_checker_catches_planted_mistakes():
    """The checker is not vacuous: an item that does not wait for its
    predecessor's prefetch, and a step whose K load goes into the buffer it
    is reading, are both rejected."""
    g = _gen()
    prog = g.item_asm(False)
    mem = _Memory()
    assert not _Machine(g, 4, 0, mem, 0).run(prog)
    bad = [ln.replace(f"vmcnt({g.VM_AFTER_PREFETCH})", "vmcnt(40)") for ln in prog]
    assert _Machine(g, 3, 1, mem, 1).run(bad) or mem.errors
    # K_{j+2} into the buffer of K_{j+1}: swap the two K buffers' offsets in
    # the loop's loads
    i = next(k for k, ln in enumerate(prog) if ln.startswith("L_loop_"))
    swapped = prog[:i] + [ln.replace(f"%[wbase], {g.KV_LDS[1]}", "%[wbase], X").replace(
        f"%[wbase], {g.KV_LDS[0]}", f"%[wbase], {g.KV_LDS[1]}").replace("%[wbase], X", f"%[wbase], {g.KV_LDS[0]}")
        for ln in prog[i:]]
    assert swapped != prog
    mem = _Memory()
    assert _Machine(g, 6, 0, mem, 0).run(swapped) or mem.errors


def test_generator_output_is_deterministic(tmp_path):
    g = _gen()
    a, b = tmp_path / "a.inc", tmp_path / "b.inc"
    g.main(str(a))
    g.main(str(b))
    assert a.read_text() == b.read_text()
    assert "FA_ASM_ITEM" in a.read_text() and "FA_ASM_CLOBBERS" in a.read_text()
