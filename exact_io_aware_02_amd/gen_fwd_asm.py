"""Generate the gfx950 assembly of one query tile of the d = 128 bf16
FlashAttention forward (64 query rows per wavefront, one wavefront per SIMD).

    python exact_io_aware_02_amd/gen_fwd_asm.py OUT.inc

The build runs this before compiling fa_fwd_bf16_asm.hip, which includes the
output: the C string macros FA_ASM_ITEM and FA_ASM_ITEM_CAUSAL, the bodies of
inline-asm statements that run Algorithm 1 of "Infra: Flash Attention"
("Tiled computation and forward"), without and with the causal mask, for one
query tile of a wavefront and store its rows of O = U / l (bf16) and
L = m + log l (keys past N are masked).
While its last product block runs, an item loads the next item's Q, K_0 and
K_1, so a persistent workgroup's items follow one another with no wait for
those loads.

Why assembly: a wavefront keeps U^T for 64 queries (128 AGPRs), its Q
fragments (64 AGPRs), two score tiles and two probability tiles (192 VGPRs)
live at once.  The compiler spills and copies such a kernel between the
register files; written out, every value has one home:

  a[0:127]    U^T accumulators, u[db][qb] = a[(2 db + qb) * 16 ...]
  a[128:191]  Q fragments, qf[qb][ds] = a[128 + (8 qb + ds) * 4 ...]
  a[192:255]  16 slots of K / V fragments read from LDS
  v[0:127]    score tiles S_A, S_B: s[cb][qb] = 16 VGPRs at (2 cb + qb) * 16
  v[128:191]  probability tiles W_A, W_B: w[qb][ks] = 4 VGPRs at (4 qb + ks) * 4
  v[192:207]  softmax temporaries
  v[208:223]  per-row state (base m, partial l, alpha, ...)

Each tile step j (64 keys) is one straight-line stream that overlaps, inside
the wavefront, U += V_{j-1}^T W_{j-1}^T and S_{j+1} = K_{j+1} Q^T on the
matrix core with the softmax of S_j on the VALU (the FlashAttention-3
overlap of the blog's FA-3 section as a software pipeline over tiles).  A
wavefront issues independent VALU instructions while its MFMAs run, so the
softmax hides under the products.

Hazards the compiler would otherwise handle are handled here:
  * LDS reads -> MFMA operands: s_waitcnt lgkmcnt counted per read.
  * MFMA results -> VALU reads: score tiles are read one step (a barrier and
    more than 50 instructions) after the MFMAs that wrote them; U is read only
    after 48 wait states.
  * VALU compare -> lane-mask read, VALU -> permlane: 2 wait states.
  * transcendental result -> VALU read: at least 1 wait state.
  * M0 write -> buffer load to LDS: 1 wait state (more are given).

Buffer loads are bounds-checked by the hardware against the size in their
resource through their VGPR and instruction offsets (whether the SGPR offset
counts differs between GPU generations).  So each K or V tile is loaded
through a resource of its own that starts at the tile and ends at the end of
the head (empty past it), and the second query block's rows are addressed
through a VGPR: rows past N read as zeros and no load touches memory past
the head, by construction.
"""

import sys

D = 128
BC = 64
STRIDE = 2 * D + 16          # padded LDS row (bytes)
TILE = BC * STRIDE           # one K or V tile in LDS (17408)
KBUF = [0, TILE]             # K buffer offsets from the K read base
VBUF = [0, TILE]             # V buffer offsets from the V read base
KV_LDS = [0, TILE, 2 * TILE, 3 * TILE]  # K0, K1, V0, V1 from the LDS base
LOADS = TILE // 1024         # 17 x 1 KiB buffer->LDS loads per tile
WAVES = 4

S_BUF = [0, 64]              # VGPR base of S_A, S_B
W_BUF = [128, 160]           # VGPR base of W_A, W_B
TMP0 = 192                   # 16 temporaries v[192:207]
ST = 208                     # state registers v[208:223]
V_M = [ST + 0, ST + 1]       # base m per query block (raw score units)
V_L = [ST + 2, ST + 3]       # partial l per query block (this lane's keys)
V_MC = [ST + 4, ST + 5]      # m * c (VGPR banks 0, 1)
V_AL = [ST + 6, ST + 7]      # alpha
V_MX = [ST + 8, ST + 9]      # tile max
V_NINF = ST + 10             # -inf
V_THR = [ST + 11, ST + 12]   # mask thresholds
V_T = ST + 13                # scratch
V_MC2 = [ST + 14, ST + 15]   # m * c again, in VGPR banks 2, 3
FRAG0 = 192                  # AGPR fragment slots a[192:255]
NSLOT = 16
LOOKAHEAD = 6
# the buffer->LDS loads of a block are issued over its first LOAD_SPREAD of
# MFMAs: they are waited for at the next step's top, and issued late they
# leave too little time to cover the HBM latency
LOAD_SPREAD = 0.5
VALU_LEAD = 8                # softmax instructions issued before a step's first MFMA

# Exponentials given to a polynomial (the share of "Infra: Flash Attention",
# section "FlashAttention-4", that runs on the multiply-add units): with
# poly = k > 0, k of the 64 exponentials per lane of a tile are
# 2^x = 2^floor(x) p(x - floor(x)), p the cubic with p(0) = 1 of least
# maximum relative error against 2^f on [0, 1] (fitted by linear programming
# over 20,001 points; 8.6e-5, checked in float32 Horner order by the CPU
# tests), floor(x) added to the exponent by v_ldexp_f32.  x is clamped at
# -200 first, so masked scores (-inf) give exactly 0, as v_exp_f32 does.
POLY_SHARES = (4, 8, 16)     # variants built besides 0 (v_exp_f32 only)
POLY_C1 = 0x3F31F335         # 0.695117...
POLY_C2 = 0x3E691B63         # 0.227643...
POLY_C3 = 0x3D9DD5D8         # 0.077068...
POLY_CLAMP = 0xC3480000      # -200.0
V_POLY_P = 224               # Horner accumulator (the query blocks' pairs run one after the other)
V_POLY_C2 = 225              # c2 (v_fmamk_f32 takes one literal)

# SGPRs used inside (declared as clobbers)
S_J = 40        # tile index j
S_T1 = 41
S_T2 = 42
S_SOFF = 43     # byte offset of a tile within the head
S_MV = [44, 46]  # moved masks per query block (pairs)
S_ANY = 48      # pair
S_CMP = [50, 52, 54]  # compare masks (pairs)
S_KB = 56       # key base of the masked tile
S_M0 = 58       # the caller's M0, restored at the end
S_C = 70        # c = scale * log2(e)
S_THETA = 71    # rescale threshold (raw score units)
S_256 = 72      # 2^8 as fp32
S_RK = 60       # s[60:63]: resource of the K tile being loaded
S_RV = 64       # s[64:67]: resource of the V tile being loaded
SGPR_CLOBBERS = list(range(40, 59)) + list(range(60, 68)) + [S_C, S_THETA, S_256]


def kfrag_reads(slot, buf, cb, ds):
    f = FRAG0 + 4 * slot
    off = KBUF[buf] + cb * 32 * STRIDE + ds * 32
    return [f"ds_read_b128 a[{f}:{f + 3}], %[kb] offset:{off}"]


def vfrag_reads(slot, buf, db, ks):
    f = FRAG0 + 4 * slot
    out = []
    for t in range(2):
        off = VBUF[buf] + (ks * 16 + 2 * t) * STRIDE + db * 64
        out.append(f"ds_read_b64_tr_b16 a[{f + 2 * t}:{f + 2 * t + 1}], %[vb] offset:{off}")
    return out


def mfma_pv(slot, db, qb, wbuf, ks):
    f = FRAG0 + 4 * slot
    u = (2 * db + qb) * 16
    w = W_BUF[wbuf] + (4 * qb + ks) * 4
    return f"v_mfma_f32_32x32x16_bf16 a[{u}:{u + 15}], a[{f}:{f + 3}], v[{w}:{w + 3}], a[{u}:{u + 15}]"


def mfma_qk(slot, sbuf, cb, qb, ds):
    f = FRAG0 + 4 * slot
    s = S_BUF[sbuf] + (2 * cb + qb) * 16
    q = 128 + (8 * qb + ds) * 4
    c = "0" if ds == 0 else f"v[{s}:{s + 15}]"
    return f"v_mfma_f32_32x32x16_bf16 v[{s}:{s + 15}], a[{f}:{f + 3}], a[{q}:{q + 3}], {c}"


def interleave_lists(lists):
    """Round-robin merge of instruction lists (each list keeps its order)."""
    out = []
    for k in range(max(len(x) for x in lists)):
        for x in lists:
            if k < len(x):
                out.append(x[k])
    return out


def softmax_ops(sbuf, wbuf, fast=False, poly=0):
    """VALU instructions of the softmax of score tile sbuf into W tile wbuf:
    row max, the conditional move of the base (threshold theta in raw score
    units), W = exp2(c S - c m) in bf16, the fp32 row sums, l = alpha l + sum.

    A VALU instruction whose VGPR operands share a bank (register number mod
    4) pays for the conflict, and one wavefront has no other wavefront to
    hide that behind, so operands are placed in distinct banks: c is an SGPR,
    m c has a copy in banks 0/1 and one in 2/3, score pairs use temporaries
    in banks 0/1 and the partial sums live in banks 2/3, and the max chains
    combine scores of banks 0 and 2 (resp. 1 and 3) into an accumulator of
    another bank.  Dependent chains are short and interleaved (eight max
    chains, eight partial sums).

    fast: W relative to the current base without forming the row max; l is
    left alone and the tile's per-lane sums are left in psum[0] and psum[4].
    If no sum exceeds 2^8, no weight did either, and the result is what the
    full version gives when the base does not move (alpha = 1).

    poly: exponentials per 64 given to the polynomial (exp_ops)."""
    sb = S_BUF[sbuf]
    ops = []
    pair_tmp = [(TMP0 + 4 * i, TMP0 + 4 * i + 1) for i in range(4)]          # banks 0, 1
    psum = [TMP0 + 4 * (i // 2) + 2 + (i & 1) for i in range(8)]             # banks 2, 3
    if fast:
        return exp_ops(sb, wbuf, pair_tmp, psum, poly)
    # row max: per (query block, 32-key block) two chains, over the scores in
    # banks {0, 2} (accumulator in bank 1 or 3) and in banks {1, 3}
    # (accumulator in bank 0 or 2)
    acc_even = [TMP0 + 1, TMP0 + 3, TMP0 + 5, TMP0 + 7]   # banks 1, 3
    acc_odd = [TMP0 + 0, TMP0 + 2, TMP0 + 4, TMP0 + 6]    # banks 0, 2
    chains = []
    for qb in range(2):
        for cb in range(2):
            r = sb + (2 * cb + qb) * 16
            i = 2 * qb + cb
            for par, acc in ((0, acc_even[i]), (1, acc_odd[i])):
                vals = [r + t for t in range(par, 16, 2)]
                ch = [f"v_max_f32 v{acc}, v{vals[0]}, v{vals[1]}"]
                for k in range(2, 8, 2):
                    ch.append(f"v_max3_f32 v{acc}, v{acc}, v{vals[k]}, v{vals[k + 1]}")
                chains.append(ch)
    ops += interleave_lists(chains)
    for qb in range(2):
        e0, e1 = acc_even[2 * qb], acc_even[2 * qb + 1]
        o0, o1 = acc_odd[2 * qb], acc_odd[2 * qb + 1]
        ops.append(f"v_max3_f32 v{o0}, v{o0}, v{e0}, v{e1}")
        ops.append(f"v_max_f32 v{V_MX[qb]}, v{o0}, v{o1}")
    for qb in range(2):
        ops.append(f"v_mov_b32 v{acc_even[qb]}, v{V_MX[qb]}")
    ops.append("s_nop 1")
    for qb in range(2):
        ops.append(f"v_permlane32_swap_b32 v{V_MX[qb]}, v{acc_even[qb]}")
    for qb in range(2):
        ops.append(f"v_max_f32 v{V_MX[qb]}, v{V_MX[qb]}, v{acc_even[qb]}")
    thr = []
    for qb in range(2):
        mx, m, mc, mc2, al = V_MX[qb], V_M[qb], V_MC[qb], V_MC2[qb], V_AL[qb]
        mv = S_MV[qb]
        t = acc_odd[2 + qb]
        thr.append([
            f"v_add_f32 v{t}, s{S_THETA}, v{m}",                    # m + theta
            f"v_cmp_gt_f32_e64 s[{mv}:{mv + 1}], v{mx}, v{t}",       # moved
            "s_nop 1",
            f"v_cndmask_b32_e64 v{mx}, v{m}, v{mx}, s[{mv}:{mv + 1}]",  # m_new
            f"v_mul_f32 v{mc}, s{S_C}, v{mx}",                      # c m_new
            f"v_fma_f32 v{t}, v{m}, s{S_C}, -v{mc}",                # c (m_old - m_new)
            f"v_exp_f32 v{t}, v{t}",
            f"v_mov_b32 v{mc2}, v{mc}",
            f"v_mov_b32 v{m}, v{mx}",
            f"v_cndmask_b32_e64 v{al}, 1.0, v{t}, s[{mv}:{mv + 1}]",  # alpha
        ])
    ops += interleave_lists(thr)
    ops += exp_ops(sb, wbuf, pair_tmp, psum, poly)
    for qb in range(2):
        ops.append(f"v_fma_f32 v{V_L[qb]}, v{V_AL[qb]}, v{V_L[qb]}, v{psum[4 * qb]}")
    return ops


def exp2_poly(x, f, p):
    """x <- 2^x on the multiply-add units: clamp, fraction f and floor (in
    place, as an integer), Horner p(f) = 1 + f (c1 + f (c2 + f c3)), then
    p 2^floor by the exponent.  f and p are temporaries."""
    return [
        f"v_max_f32 v{x}, {POLY_CLAMP:#x}, v{x}",
        f"v_fract_f32 v{f}, v{x}",
        f"v_cvt_flr_i32_f32 v{x}, v{x}",
        f"v_fmamk_f32 v{p}, v{f}, {POLY_C3:#x}, v{V_POLY_C2}",
        f"v_fmaak_f32 v{p}, v{p}, v{f}, {POLY_C1:#x}",
        f"v_fma_f32 v{p}, v{p}, v{f}, 1.0",
        f"v_ldexp_f32 v{x}, v{p}, v{x}",
    ]


def exp_ops(sb, wbuf, pair_tmp, psum, poly=0):
    """W = exp2(c S - c m) for a score tile: per pair of scores two FMAs, two
    exponentials (each read at least one instruction later), two adds into
    the partial sum of the pair's 8-key group, one bf16 pack; the two query
    blocks alternate pair by pair.  Leaves the per-lane tile sums in psum[0],
    psum[4].

    poly = k: the second exponential of every (32 / k)-th pair of a query
    block is exp2_poly, with the pair's W register (written only by the
    pack) as its fraction temporary."""
    assert poly == 0 or poly in POLY_SHARES
    every = 32 // poly if poly else 0
    ops = []
    seqs = {0: [], 1: []}
    k_pair = 0
    for ks in range(4):
        cb, h = ks >> 1, ks & 1
        for k in range(4):
            for qb in range(2):
                src = sb + (2 * cb + qb) * 16 + 8 * h + 2 * k   # banks 0, 1 (k even) or 2, 3
                mcx = V_MC2[qb] if k % 2 == 0 else V_MC[qb]
                w = W_BUF[wbuf] + (4 * qb + ks) * 4
                a, b = pair_tmp[k_pair % 4]
                k_pair += 1
                ps = psum[4 * qb + ks]
                by_poly = every and (4 * ks + k) % every == every - 1
                seqs[qb].append([
                    f"v_fma_f32 v{a}, v{src}, s{S_C}, -v{mcx}",
                    f"v_fma_f32 v{b}, v{src + 1}, s{S_C}, -v{mcx}",
                    f"v_exp_f32 v{a}, v{a}",
                    *(exp2_poly(b, w + k, V_POLY_P) if by_poly else [f"v_exp_f32 v{b}, v{b}"]),
                    f"v_add_f32 v{ps}, 0, v{a}" if k == 0 else f"v_add_f32 v{ps}, v{ps}, v{a}",
                    f"v_add_f32 v{ps}, v{ps}, v{b}",
                    f"v_cvt_pk_bf16_f32 v{w + k}, v{a}, v{b}",
                ])
    for c0, c1 in zip(seqs[0], seqs[1]):
        ops += c0 + c1
    for qb in range(2):
        p = psum[4 * qb:4 * qb + 4]
        ops += [f"v_add_f32 v{p[0]}, v{p[0]}, v{p[1]}", f"v_add_f32 v{p[2]}, v{p[2]}, v{p[3]}"]
    for qb in range(2):
        p = psum[4 * qb:4 * qb + 4]
        ops.append(f"v_add_f32 v{p[0]}, v{p[0]}, v{p[2]}")
    return ops


class Stream:
    """Builds one straight-line block: MFMAs with their fragment reads issued
    LOOKAHEAD fragments ahead, lgkmcnt waits counted per read, and VALU
    instructions spread evenly between the MFMAs."""

    def __init__(self, poly=0):
        self.out = []
        self.poly = poly   # exponentials per 64 given to the polynomial

    def emit(self, s):
        self.out.append(s)

    def block(self, frags, valu, valu_first=0, groups=()):
        """frags: list of (read_fn(slot) -> [instr], [mfma_fn(slot) -> instr]);
        groups: instruction groups (buffer->LDS loads) issued one after each
        odd MFMA, so the matrix core runs while the wavefront issues them."""
        issued = []      # per issued DS instruction: fragment index
        n = len(frags)
        nmf = sum(len(m) for _, m in frags)
        next_read = 0
        vi = 0

        def read_upto(k):
            nonlocal next_read
            while next_read < n and next_read <= k:
                rd, _ = frags[next_read]
                for ins in rd(next_read % NSLOT):
                    self.emit(ins)
                    issued.append(next_read)
                next_read += 1

        ready = set()
        gi = 0
        read_upto(LOOKAHEAD - 1)
        while vi < min(valu_first, len(valu)):
            self.emit(valu[vi])
            vi += 1
        done = 0
        for fi, (_, mfs) in enumerate(frags):
            read_upto(fi + LOOKAHEAD - 1)
            if fi not in ready:
                # wait for this fragment and the next one
                upto = fi + 1 if fi + 1 < next_read else fi
                last = max(i for i, f in enumerate(issued) if f == upto)
                after = len(issued) - 1 - last
                self.emit(f"s_waitcnt lgkmcnt({min(after, 15)})")
                ready.update(range(fi, upto + 1))
            for mf in mfs:
                self.emit(mf(fi % NSLOT))
                done += 1
                while gi < len(groups) and done >= max(1, (gi + 1) * int(nmf * LOAD_SPREAD) // (len(groups) + 1)):
                    for ins in groups[gi]:
                        self.emit(ins)
                    gi += 1
                target = valu_first + ((len(valu) - valu_first) * done + nmf - 1) // nmf
                while vi < min(target, len(valu)):
                    self.emit(valu[vi])
                    vi += 1
        while vi < len(valu):
            self.emit(valu[vi])
            vi += 1
        assert gi == len(groups), "load groups left over"


def pv_frags(vbuf, wbuf):
    fr = []
    for ks in range(4):
        for db in range(4):
            fr.append((lambda s, ks=ks, db=db: vfrag_reads(s, vbuf, db, ks),
                       [lambda s, db=db, qb=qb, ks=ks: mfma_pv(s, db, qb, wbuf, ks) for qb in range(2)]))
    return fr


def qk_frags(kbuf, sbuf):
    fr = []
    for ds in range(8):
        for cb in range(2):
            fr.append((lambda s, cb=cb, ds=ds: kfrag_reads(s, kbuf, cb, ds),
                       [lambda s, cb=cb, qb=qb, ds=ds: mfma_qk(s, sbuf, cb, qb, ds) for qb in range(2)]))
    return fr


def interleave(a, b):
    out = []
    for x, y in zip(a, b):
        out += [x, y]
    return out


def tile_rsrc(emit, kind, tile_sgpr, r):
    """s[r:r+3] = resource of K or V tile s[tile_sgpr] of the head: base at
    the tile, size the bytes left in the head (0 past its end)."""
    emit(f"s_lshl_b32 s{S_SOFF}, s{tile_sgpr}, 14")
    emit(f"s_add_u32 s{r}, %[{kind}lo], s{S_SOFF}")
    emit(f"s_addc_u32 s{r + 1}, %[{kind}hi], 0")
    emit(f"s_sub_u32 s{r + 2}, %[hb], s{S_SOFF}")
    emit(f"s_cselect_b32 s{r + 2}, 0, s{r + 2}")
    emit(f"s_mov_b32 s{r + 3}, 0x20000")


def dma_groups(kind, dst_off, r):
    """Buffer->LDS loads of one K or V tile as instruction groups: this
    wavefront's 1 KiB blocks wave, wave + 4, ...; block 16 belongs to
    wavefront 0, so the other wavefronts issue that load with no lane active
    (EXEC = 0: nothing is read or written).  The tile's resource is in
    s[r:r+3]."""
    rs = f"s[{r}:{r + 3}]"
    out = []
    for p in range((LOADS + WAVES - 1) // WAVES):
        g = []
        partial = WAVES * p + WAVES > LOADS
        if partial:
            g += ["s_cmp_eq_u32 %[wave], 0", "s_cselect_b64 exec, -1, 0", "s_nop 4"]
        g += [f"s_add_u32 m0, %[wbase], {dst_off + p * WAVES * 1024}", "s_nop 1",
              f"buffer_load_dwordx4 %[{kind}vo{p}], {rs}, 0 offen lds"]
        if partial:
            g += ["s_mov_b64 exec, -1", "s_nop 4"]
        out.append(g)
    return out


def dma_tile(st, kind, dst_off, tile_sgpr, label):
    """Buffer->LDS loads of one K or V tile: this wavefront's 1 KiB blocks
    wave, wave + 4, ... (block 16 only on wavefront 0)."""
    r = S_RK if kind == "k" else S_RV
    tile_rsrc(st.emit, kind, tile_sgpr, r)
    for p in range((LOADS + WAVES - 1) // WAVES):
        if WAVES * p + WAVES > LOADS:
            st.emit("s_cmp_lg_u32 %[wave], 0")
            st.emit(f"s_cbranch_scc1 {label}_%=")
        st.emit(f"s_add_u32 m0, %[wbase], {dst_off + p * WAVES * 1024}")
        st.emit("s_nop 1")
        st.emit(f"buffer_load_dwordx4 %[{kind}vo{p}], s[{r}:{r + 3}], 0 offen lds")
    st.emit(f"{label}_%=:")


def cmp_mask(st, elems):
    """elems: (score register, threshold register, c): the score becomes -inf
    where c > threshold.  Three compare masks rotate, so that every mask is
    read three instructions after it is written."""
    pend = []
    for k, (reg, thr, c) in enumerate(elems):
        sp = S_CMP[k % 3]
        st.emit(f"v_cmp_lt_i32_e64 s[{sp}:{sp + 1}], v{thr}, {c}")
        pend.append((reg, sp))
        if len(pend) == 3:
            for r, m in pend:
                st.emit(f"v_cndmask_b32_e64 v{r}, v{r}, v{V_NINF}, s[{m}:{m + 1}]")
            pend = []
    for r, m in pend:
        st.emit("s_nop 1")
        st.emit(f"v_cndmask_b32_e64 v{r}, v{r}, v{V_NINF}, s[{m}:{m + 1}]")


def mask_block(st, sbuf, causal, label):
    """Masking of the score tile at key base 64 j (j in s[S_J]) before its
    softmax.  Lane (l32, g) holds, for query block qb, the keys kbase + c + 4 g
    with c = 32 cb + 8 (i >> 2) + (i & 3) for element i of s[cb][qb].
      * a tile reaching past N: every key past the lane's last valid one
        (thresholds %[limg0/1] = lim - 4 g, lim = N - 1 or, causal,
        min(N - 1, query)) is set to -inf;
    causal only (the wavefront's rows are qw0 .. qw0 + 63):
      * the diagonal tile (kbase = qw0): key c + 4 g of query block qb is
        masked against query 32 qb + l32, i.e. the lower-left 32 x 32 block is
        kept, the upper-right one dropped, and the two diagonal blocks compare
        c against %[dg] = l32 - 4 g;
      * a tile wholly after the rows (kbase > qw0): every weight is zero, which
        m c = +inf gives for the whole tile (restored after the step); step
        runs this only for the first such tile, and skips the rest."""
    st.emit(f"s_lshl_b32 s{S_KB}, s{S_J}, 6")
    st.emit(f"s_add_u32 s{S_T1}, s{S_KB}, 64")
    st.emit(f"s_cmp_gt_u32 s{S_T1}, %[n_keys]")
    st.emit(f"s_cbranch_scc1 {label}_gen_%=")
    if causal:
        st.emit(f"s_cmp_eq_u32 s{S_KB}, %[qw0]")
        st.emit(f"s_cbranch_scc1 {label}_diag_%=")
        st.emit(f"s_cmp_gt_u32 s{S_KB}, %[qw0]")
        st.emit(f"s_cbranch_scc1 {label}_full_%=")
    st.emit(f"s_branch {label}_end_%=")
    sb = S_BUF[sbuf]
    # general: thresholds against the tile's key base (the scores were
    # written by MFMAs a step ago; the nops cover the rest of their latency
    # for a tile read right after its product)
    st.emit(f"{label}_gen_%=:")
    st.emit("s_nop 15")
    st.emit("s_nop 15")
    st.emit("s_nop 15")
    for qb in range(2):
        st.emit(f"v_subrev_u32 v{V_THR[qb]}, s{S_KB}, %[limg{qb}]")
    elems = []
    for qb in range(2):
        for cb in range(2):
            for i in range(16):
                elems.append((sb + (2 * cb + qb) * 16 + i, V_THR[qb], 32 * cb + 8 * (i >> 2) + (i & 3)))
    cmp_mask(st, elems)
    if causal:
        st.emit(f"s_branch {label}_end_%=")
        st.emit(f"{label}_diag_%=:")
        st.emit("s_nop 15")
        st.emit("s_nop 15")
        st.emit("s_nop 15")
        for i in range(16):
            st.emit(f"v_mov_b32 v{sb + (2 * 1 + 0) * 16 + i}, v{V_NINF}")
        st.emit(f"v_mov_b32 v{V_THR[0]}, %[dg]")
        elems = []
        for cb, qb in ((0, 0), (1, 1)):
            for i in range(16):
                elems.append((sb + (2 * cb + qb) * 16 + i, V_THR[0], 8 * (i >> 2) + (i & 3)))
        cmp_mask(st, elems)
        st.emit(f"s_branch {label}_end_%=")
        st.emit(f"{label}_full_%=:")
        for r in V_MC + V_MC2:
            st.emit(f"v_mov_b32 v{r}, 0x7f800000")
    st.emit(f"{label}_end_%=:")


def rescale_block(st, label):
    st.emit(f"s_or_b64 s[{S_ANY}:{S_ANY + 1}], s[{S_MV[0]}:{S_MV[0] + 1}], s[{S_MV[1]}:{S_MV[1] + 1}]")
    st.emit(f"s_cbranch_scc0 {label}_%=")
    st.emit("s_nop 15")
    st.emit("s_nop 15")
    st.emit("s_nop 15")
    for base in range(0, 128, 8):
        qb = (base // 16) % 2
        for k in range(8):
            st.emit(f"v_accvgpr_read_b32 v{TMP0 + k}, a{base + k}")
        for k in range(8):
            st.emit(f"v_mul_f32 v{TMP0 + k}, v{TMP0 + k}, v{V_AL[qb]}")
        for k in range(8):
            st.emit(f"v_accvgpr_write_b32 a{base + k}, v{TMP0 + k}")
    st.emit("s_nop 3")
    st.emit(f"{label}_%=:")


def step(st, parity, causal, kind, label):
    """Tile step j (parity = j & 1, j in s[S_J]).  kind: 'full' (PV of j-1,
    QK of j+1, softmax of j), 'last' (PV of j-1, softmax of j), 'first'
    (j = 0: QK of 1, softmax of 0).

    Causal: the wavefront's rows qw0 .. qw0 + 63 end in its diagonal tile
    dj = qw0 / 64, and tiles after it get zero weights ("CMU 10-423 Lecture
    18", section 4.3: work wholly above the diagonal is skipped).  So from
    j = dj on the products with K_{j+1} are skipped, and from j = dj + 2 on
    the whole step (PV of a zero W_{j-1}, the softmax of a masked tile): the
    wavefront then only issues its share of the tile loads and joins the
    barrier, which the other wavefronts of the workgroup still need."""
    j_odd = parity
    # top: own loads landed, every wavefront done with step j-1's buffers.
    # Step 0 reads only K_1, waited for before S_0; V_0 (and the previous
    # item's stores) are left to step 1's wait.
    st.emit("s_waitcnt lgkmcnt(0)" if kind == "first" else "s_waitcnt vmcnt(0) lgkmcnt(0)")
    st.emit("s_barrier")
    groups = []
    if kind in ("full", "first"):
        # K_{j+2} into K buffer j & 1, last read in step j-1.  Past the last
        # tile its resource is empty: zeros into a buffer nobody reads.
        st.emit(f"s_add_u32 s{S_T2}, s{S_J}, 2")
        tile_rsrc(st.emit, "k", S_T2, S_RK)
        groups += dma_groups("k", KV_LDS[j_odd], S_RK)
    if kind in ("full", "last"):
        # V_j into V buffer j & 1, last read (V_{j-2}) in step j-1
        tile_rsrc(st.emit, "v", S_J, S_RV)
        groups += dma_groups("v", KV_LDS[2 + j_odd], S_RV)
    if not causal or kind == "first":
        step_body(st, j_odd, causal, kind, label, groups)
        return
    # 64 j - qw0: >= 128 from j = dj + 2 on, >= 0 from j = dj on
    st.emit(f"s_lshl_b32 s{S_T1}, s{S_J}, 6")
    st.emit(f"s_sub_u32 s{S_T1}, s{S_T1}, %[qw0]")
    st.emit(f"s_cmp_ge_i32 s{S_T1}, 128")
    st.emit(f"s_cbranch_scc1 {label}_dead_%=")
    if kind == "full":
        st.emit(f"s_cmp_ge_i32 s{S_T1}, 0")
        st.emit(f"s_cbranch_scc1 {label}_pvo_%=")
    step_body(st, j_odd, causal, kind, label, groups)
    st.emit(f"s_branch {label}_join_%=")
    if kind == "full":
        st.emit(f"{label}_pvo_%=:")
        step_body(st, j_odd, causal, "last", f"{label}p", groups)
        st.emit(f"s_branch {label}_join_%=")
    st.emit(f"{label}_dead_%=:")
    for g in groups:
        for ins in g:
            st.emit(ins)
    st.emit(f"{label}_join_%=:")


def step_body(st, j_odd, causal, kind, label, groups):
    """A step's mask, products, softmax and conditional rescale (see step)."""
    mask_block(st, j_odd, causal, f"{label}_mask")
    valu = softmax_ops(j_odd, j_odd, fast=(kind != "first"), poly=st.poly)
    if kind == "full":
        frags = interleave(pv_frags(1 - j_odd, 1 - j_odd), qk_frags(1 - j_odd, 1 - j_odd))
    elif kind == "last":
        frags = pv_frags(1 - j_odd, 1 - j_odd)
    else:
        frags = qk_frags(1, 1)
    st.block(frags, valu, valu_first=(40 if kind == "first" else VALU_LEAD), groups=groups)
    if causal:
        # m c again (a tile after the rows set it to +inf)
        for qb in range(2):
            st.emit(f"v_mul_f32 v{V_MC[qb]}, s{S_C}, v{V_M[qb]}")
        for qb in range(2):
            st.emit(f"v_mov_b32 v{V_MC2[qb]}, v{V_MC[qb]}")
    if kind != "first":
        # conditional rescaling ("Invariant of conditional rescaling"): the
        # base moves only if a weight relative to it exceeds 2^8, which only
        # a tile sum above 2^8 can show; then the tile's softmax is redone
        # with its row max, and U and l are rescaled
        t0, t1 = TMP0 + 2, TMP0 + 10   # psum[0], psum[4]
        st.emit(f"v_cmp_gt_f32_e64 s[{S_MV[0]}:{S_MV[0] + 1}], v{t0}, s{S_256}")
        st.emit(f"v_cmp_gt_f32_e64 s[{S_MV[1]}:{S_MV[1] + 1}], v{t1}, s{S_256}")
        st.emit("s_nop 1")
        st.emit(f"s_or_b64 s[{S_ANY}:{S_ANY + 1}], s[{S_MV[0]}:{S_MV[0] + 1}], s[{S_MV[1]}:{S_MV[1] + 1}]")
        st.emit(f"s_cbranch_scc1 {label}_slow_%=")
        st.emit(f"v_add_f32 v{V_L[0]}, v{V_L[0]}, v{t0}")
        st.emit(f"v_add_f32 v{V_L[1]}, v{V_L[1]}, v{t1}")
        st.emit(f"s_branch {label}_done_%=")
        st.emit(f"{label}_slow_%=:")
        for ins in softmax_ops(j_odd, j_odd, poly=st.poly):
            st.emit(ins)
        rescale_block(st, f"{label}_rs")
        st.emit(f"{label}_done_%=:")


LN2 = "0x3f317218"           # ln 2 as fp32


def prefetch_groups():
    """The next item's K_0, K_1 (into K buffers 0, 1) and Q fragments (into
    a[128:191]) as load groups; the caller has set up their resources."""
    q = []
    for qb in range(2):
        for ds in range(8):
            f = 128 + (8 * qb + ds) * 4
            vo = "%[nqvo]" if qb == 0 else f"v{TMP0 + 15}"
            q.append(f"buffer_load_dwordx4 a[{f}:{f + 3}], {vo}, %[nqrsrc], 0 offen offset:{32 * ds}")
    qg = [q[i:i + 2] for i in range(0, 16, 2)]
    return (dma_groups("k", KV_LDS[0], S_RK) + qg[:4] + dma_groups("k", KV_LDS[1], S_RV) + qg[4:])


def prefetch_setup(e):
    """Resources of the next item's K_0 and K_1 (empty if there is none:
    %[nhb] = 0) and the VGPR offset of its second query block."""
    e(f"v_add_u32 v{TMP0 + 15}, 0x2000, %[nqvo]")
    for t, r in ((0, S_RK), (1, S_RV)):
        e(f"s_mov_b32 s{S_T2}, {t}")
        e(f"s_lshl_b32 s{S_SOFF}, s{S_T2}, 14")
        e(f"s_add_u32 s{r}, %[nklo], s{S_SOFF}")
        e(f"s_addc_u32 s{r + 1}, %[nkhi], 0")
        e(f"s_sub_u32 s{r + 2}, %[nhb], s{S_SOFF}")
        e(f"s_cselect_b32 s{r + 2}, 0, s{r + 2}")
        e(f"s_mov_b32 s{r + 3}, 0x20000")


def final_block(st, par, causal, label):
    """U += V_{n-1} W_{n-1} from buffers par (j = n - 1 in s[S_J]) while the
    next item's Q, K_0, K_1 load.  Causal: a wavefront whose rows end before
    tile n - 1 (64 (n - 1) >= qw0 + 64) has W_{n-1} = 0 and only issues the
    loads."""
    e = st.emit
    e("s_waitcnt vmcnt(0) lgkmcnt(0)")
    e("s_barrier")
    prefetch_setup(e)
    if causal:
        e(f"s_lshl_b32 s{S_T1}, s{S_J}, 6")
        e(f"s_sub_u32 s{S_T1}, s{S_T1}, %[qw0]")
        e(f"s_cmp_ge_i32 s{S_T1}, 64")
        e(f"s_cbranch_scc1 {label}_dead_%=")
    st.block(pv_frags(par, par), [], groups=prefetch_groups())
    if causal:
        e(f"s_branch {label}_join_%=")
        e(f"{label}_dead_%=:")
        for g in prefetch_groups():
            for ins in g:
                e(ins)
        e(f"{label}_join_%=:")


# VMEM instructions a wavefront issues between the prefetch of the next
# item's Q, K_0, K_1 and that item's wait for them: the 16 O-row stores and
# 2 L stores of this item, then the next item's V_0 loads (4 or 5: whether
# a load with no lane active counts is not relied on, so 4)
VM_AFTER_PREFETCH = 16 + 2 + 4


def item_asm(causal, poly=0):
    """One query tile of a wavefront: the tile loop, then O and L stored.
    %[pre] = 1: Q, K_0, K_1 were prefetched by the previous item, which
    issued nothing but its stores after them.  Every item prefetches those of
    the next one (%[nq*], %[nk*]; empty resources if there is none).
    poly: exponentials per 64 of a tile computed by exp2_poly (0: none)."""
    st = Stream(poly)
    e = st.emit
    e(f"s_mov_b32 s{S_M0}, m0")
    if poly:
        e(f"v_mov_b32 v{V_POLY_C2}, {POLY_C2:#x}")
    e(f"v_readfirstlane_b32 s{S_C}, %[c]")
    e(f"v_readfirstlane_b32 s{S_THETA}, %[theta]")
    e(f"s_mov_b32 s{S_256}, 0x43800000")
    e(f"v_mov_b32 v{V_NINF}, 0xff800000")
    e(f"v_mov_b32 v{V_M[0]}, 0xff800000")
    e(f"v_mov_b32 v{V_M[1]}, 0xff800000")
    e(f"v_mov_b32 v{V_L[0]}, 0")
    e(f"v_mov_b32 v{V_L[1]}, 0")
    # the first item of a workgroup loads Q (rows past N read as zeros; query
    # block 1 is 32 rows, 8 KiB, further), K_0 and K_1 itself
    e("s_cmp_eq_u32 %[pre], 0")
    e("s_cbranch_scc0 L_pre_%=")
    e(f"v_add_u32 v{TMP0}, 0x2000, %[qvo]")
    for qb in range(2):
        for ds in range(8):
            q = 128 + (8 * qb + ds) * 4
            vo = "%[qvo]" if qb == 0 else f"v{TMP0}"
            e(f"buffer_load_dwordx4 a[{q}:{q + 3}], {vo}, %[qrsrc], 0 offen offset:{32 * ds}")
    e(f"s_mov_b32 s{S_T2}, 0")
    tile_rsrc(e, "k", S_T2, S_RK)
    for g in dma_groups("k", KV_LDS[0], S_RK):
        for ins in g:
            e(ins)
    e(f"s_mov_b32 s{S_T2}, 1")
    tile_rsrc(e, "k", S_T2, S_RK)
    for g in dma_groups("k", KV_LDS[1], S_RK):
        for ins in g:
            e(ins)
    e("L_pre_%=:")
    # V_0
    e(f"s_mov_b32 s{S_J}, 0")
    tile_rsrc(e, "v", S_J, S_RV)
    for g in dma_groups("v", KV_LDS[2], S_RV):
        for ins in g:
            e(ins)
    # wait for Q, K_0, K_1 (not V_0, nor the previous item's stores)
    e("s_cmp_eq_u32 %[pre], 0")
    e("s_cbranch_scc0 L_prew_%=")
    e("s_waitcnt vmcnt(4)")
    e("s_branch L_prewd_%=")
    e("L_prew_%=:")
    e(f"s_waitcnt vmcnt({VM_AFTER_PREFETCH})")
    e("L_prewd_%=:")
    e("s_barrier")
    # S_0 = K_0 Q^T, U = 0 alongside
    st.block(qk_frags(0, 0), [f"v_accvgpr_write_b32 a{k}, 0" for k in range(128)])
    e("s_nop 15")
    e("s_nop 15")
    # step 0
    step(st, 0, causal, "first", "st0")
    e("s_cmp_eq_u32 %[n], 1")
    e("s_cbranch_scc1 L_fin0_%=")
    e(f"s_mov_b32 s{S_J}, 1")
    e("L_loop_%=:")
    e(f"s_add_u32 s{S_T1}, s{S_J}, 1")
    e(f"s_cmp_lt_u32 s{S_T1}, %[n]")
    e("s_cbranch_scc0 L_last1_%=")
    step(st, 1, causal, "full", "sa")
    e(f"s_add_u32 s{S_J}, s{S_J}, 1")
    e(f"s_add_u32 s{S_T1}, s{S_J}, 1")
    e(f"s_cmp_lt_u32 s{S_T1}, %[n]")
    e("s_cbranch_scc0 L_last0_%=")
    step(st, 0, causal, "full", "sb")
    e(f"s_add_u32 s{S_J}, s{S_J}, 1")
    e("s_branch L_loop_%=")
    # last step j = n - 1 (odd), then U += V_{n-1} W_{n-1} from buffers 1
    # while the next item's Q, K_0, K_1 load (no K buffer and no Q fragment
    # is read after step n - 2)
    e("L_last1_%=:")
    step(st, 1, causal, "last", "sl1")
    final_block(st, 1, causal, "fb1")
    e("s_branch L_done_%=")
    e("L_last0_%=:")
    step(st, 0, causal, "last", "sl0")
    e("L_fin0_%=:")
    final_block(st, 0, causal, "fb0")
    e("L_done_%=:")
    # epilogue: every wavefront done with the V buffers (the next item loads
    # V_0 at once); O = U / l into this wavefront's 64 staging rows (l summed
    # over the lane pair first)
    e("s_waitcnt lgkmcnt(0)")
    e("s_barrier")
    for qb in range(2):
        e(f"v_mov_b32 v{V_T}, v{V_L[qb]}")
        e("s_nop 1")
        e(f"v_permlane32_swap_b32 v{V_L[qb]}, v{V_T}")
        e(f"v_add_f32 v{V_L[qb]}, v{V_L[qb]}, v{V_T}")
        e(f"v_rcp_f32 v{V_AL[qb]}, v{V_L[qb]}")
    e("s_nop 15")
    e("s_nop 15")
    e("s_nop 15")
    for qb in range(2):
        for db in range(4):
            u = (2 * db + qb) * 16
            for i4 in range(4):
                for k in range(4):
                    e(f"v_accvgpr_read_b32 v{TMP0 + k}, a{u + 4 * i4 + k}")
                for k in range(4):
                    e(f"v_mul_f32 v{TMP0 + k}, v{TMP0 + k}, v{V_AL[qb]}")
                e(f"v_cvt_pk_bf16_f32 v{TMP0 + 4}, v{TMP0}, v{TMP0 + 1}")
                e(f"v_cvt_pk_bf16_f32 v{TMP0 + 5}, v{TMP0 + 2}, v{TMP0 + 3}")
                off = qb * 32 * STRIDE + 64 * db + 16 * i4
                e(f"ds_write_b64 %[stg], v[{TMP0 + 4}:{TMP0 + 5}] offset:{off}")
    # L = ln l + m scale = (log2 l + c m) ln 2, for rows qw0 + l32 and
    # qw0 + 32 + l32 (both lanes of a pair store the same value)
    for qb in range(2):
        e(f"v_log_f32 v{TMP0 + 8 + qb}, v{V_L[qb]}")
    e(f"v_add_u32 v{TMP0 + 12}, 0x1000, %[ovo]")
    for qb in range(2):
        e(f"v_add_f32 v{TMP0 + 8 + qb}, v{TMP0 + 8 + qb}, v{V_MC[qb]}")
    e(f"v_add_u32 v{TMP0 + 13}, 0x2000, %[ovo]")
    for qb in range(2):
        e(f"v_mul_f32 v{TMP0 + 8 + qb}, {LN2}, v{TMP0 + 8 + qb}")
    e(f"v_add_u32 v{TMP0 + 14}, 0x3000, %[ovo]")
    # the wavefront's 64 rows leave whole: lane (r, ch) = (lane / 16, lane %
    # 16) reads 16 bytes of rows 4 k + r and stores them (rows past N are
    # past the resource's end: dropped)
    e("s_waitcnt lgkmcnt(0)")
    for k in range(16):
        e(f"ds_read_b128 v[{4 * k}:{4 * k + 3}], %[srd] offset:{4 * k * STRIDE}")
    e("s_waitcnt lgkmcnt(0)")
    for k in range(16):
        vo = "%[ovo]" if k < 4 else f"v{TMP0 + 11 + k // 4}"
        e(f"buffer_store_dwordx4 v[{4 * k}:{4 * k + 3}], {vo}, %[orsrc], 0 offen offset:{1024 * (k % 4)}")
    e(f"buffer_store_dword v{TMP0 + 8}, %[lvo], %[lrsrc], 0 offen")
    e(f"buffer_store_dword v{TMP0 + 9}, %[lvo], %[lrsrc], 0 offen offset:128")
    e(f"s_mov_b32 m0, s{S_M0}")
    return st.out


def clobbers(poly=0):
    v = [f'"v{i}"' for i in range(0, ST + 16)]
    if poly:
        v += [f'"v{i}"' for i in (V_POLY_P, V_POLY_C2)]
    a = [f'"a{i}"' for i in range(256)]
    s = [f'"s{i}"' for i in SGPR_CLOBBERS]
    return ", ".join(v + a + s + ['"vcc"', '"scc"', '"memory"'])


def main(out):
    with open(out, "w") as f:
        f.write("// Generated by gen_fwd_asm.py; do not edit.\n#pragma once\n\n")
        for poly in (0, *POLY_SHARES):
            sfx = f"_POLY{poly}" if poly else ""
            for name, causal in (("FA_ASM_ITEM", False), ("FA_ASM_ITEM_CAUSAL", True)):
                body = item_asm(causal, poly)
                f.write(f"#define {name}{sfx} \\\n")
                for ins in body:
                    f.write(f'  "{ins}\\n" \\\n')
                f.write('  ""\n\n')
        f.write(f"#define FA_ASM_CLOBBERS {clobbers()}\n")
        f.write(f"#define FA_ASM_CLOBBERS_POLY {clobbers(1)}\n")


if __name__ == "__main__":
    main(sys.argv[1])
