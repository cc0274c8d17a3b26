"""Write tile_phases.inc: the inner-loop phases of the wide attention kernel as inline-asm
device functions.

    python causal_grouped_query_amd/csrc/gen_tile_phases.py      (rewrites tile_phases.inc)

A wave of the wide kernel owns R = 2 blocks of 32 query rows.  Keys are walked in 32-key
sub-tiles; the phase of sub-tile j issues, in one instruction stream:

  scores   S_r = K(j+1) Q_r^T       8 K fragments from LDS, each the A operand of R MFMAs
  P.V      O_r += V(j-1)^T P_r^T    8 V^T fragments from LDS, each the A operand of R MFMAs
  softmax  p = exp2(S_r(j) * c - m_r), P_r(j) = bf16(p), and two fp32 partial sums of p
           per lane and row block (the common path: no row max, see the kernel)

so that the softmax's VALU instructions issue between the wave's own MFMAs.  On gfx950 a
wave that runs its softmax as a separate phase issues about one VALU instruction per 8
cycles; placed between its 32-cycle MFMAs the same instructions cost a few cycles each.
The MFMAs are v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Layouts are those of the
kernel: S^T tiles hold 16 keys of one query row per lane, which is the B-operand layout of
the P.V MFMA, so P needs no data movement.

The loop's phases (phase_step_up / phase_step_down) also issue this wave's quarter of one
K or V tile (4 x 1 KB LDS-DMA loads between the MFMAs), and begin with a scalar compare of
the sub-tile index against the wave's last one: past it the block branches to the loads
alone.  The two variants differ only in the order of the loads' 16-row steps (up, then back
down), so one VGPR holds the lane's load offset for every piece.

Register use: fragments and softmax temporaries live in fixed registers v[228:255] (inline
asm cannot name part of an operand, and the V^T fragment is two 8-byte transposing reads
into one 16-byte operand); every block takes them as read-write operands pinned to those
registers, and the kernel keeps them live from before the first block to after the last,
so the compiler places nothing of its own there.  Everything else that lives across phases
is a compiler operand; O (MFMA accumulators only) is held in AGPRs.

Hazards (the compiler does not look inside the asm): every LDS read is waited for with
s_waitcnt before the MFMA that uses it and all reads complete inside the block; an LDS read
refills a fragment buffer only two or more MFMAs after the last MFMA reading it (checked,
also across consecutive phases); a transcendental result is read one instruction after it
is written; a block that writes S ends at least 12 instructions after its last score MFMA
(MFMA result -> VALU read); each block issues at least three instructions before its first
MFMA (VALU result -> MFMA operand); an M0 write is followed by one wait state before the
LDS-DMA load that reads it.  Code outside the blocks that reads O waits with s_nop itself.
"""

from __future__ import annotations

import os
import sys

R = 2                      # row blocks per wave
NW = 4                     # waves per workgroup (LDS stage slots of one fill piece)
KBUF, VBUF = 3, 3          # fragment buffers in flight
FIX_BASE = 228             # fixed registers v[228:255]
T_REGS = [FIX_BASE + i for i in range(4)]
FIX_TUPLES = [(FIX_BASE + 4 * i, FIX_BASE + 4 * i + 3) for i in range(7)]   # fx[0..6]
V_REGS = [FIX_BASE + 4 + 4 * i for i in range(VBUF)]
K_REGS = [FIX_BASE + 16 + 4 * i for i in range(KBUF)]
PATTERN = "SPSPSPSPSSPSPSPP"   # order of score (S) and P.V (P) fragment units
AHEAD = 2                  # fragment reads issued ahead of their MFMAs
LEAD = 4                   # softmax instructions issued before the first MFMA
XDL_VALU_WAIT = 12         # wait states between an MFMA result and a VALU read of it
MFMA_TAIL = 12             # instructions a block issues after its last MFMA
FILLS_PER_PHASE = 4        # K/V tile loads (1 KB each, global -> LDS) issued inside a full phase


def _vr(base, n=4):
    return "v[%d:%d]" % (base, base + n - 1)


def fill_piece(k, fills, desc):
    """Issue the k-th fill piece of a phase: 1 KB of K or V rows into this wave's LDS stage
    slot.  Piece p sits p*NW KB further in LDS (M0) and p*16 rows further in HBM.  The lane
    offset steps by 16 rows in place: up through pieces 0..3 in one phase, down through
    3..0 in the next, so one VGPR serves every piece and the buffer range check applies to
    the whole offset."""
    p = fills - 1 - k if desc else k
    ln = []
    if k > 0:
        ln.append(("v_subrev_u32 %[fo], %[fs], %[fo]") if desc else "v_add_u32 %[fo], %[fs], %[fo]")
    ln.append("s_mov_b32 m0, %[fm]" if p == 0 else "s_add_u32 m0, %%[fm], %d" % (p * NW * 1024))
    ln.append("s_nop 0")
    ln.append("buffer_load_dwordx4 %[fo], %[fr], 0 offen lds")
    return ln


def phase_lines(D, do_scores, do_pv, do_softmax, fills=0, desc=False):
    nds, ndb = D // 16, D // 32
    su = [("S", d) for d in range(nds)] if do_scores else []
    pu = [("P", ks, db) for ks in range(2) for db in range(ndb)] if do_pv else []
    units, si, pi = [], 0, 0
    for ch in PATTERN * 2:
        if ch == "S" and si < len(su):
            units.append(su[si]); si += 1
        elif ch == "P" and pi < len(pu):
            units.append(pu[pi]); pi += 1
    units += su[si:] + pu[pi:]
    buf, kc, vc = {}, 0, 0
    for u in units:
        if u[0] == "S":
            buf[u] = K_REGS[kc % KBUF]; kc += 1
        else:
            buf[u] = V_REGS[vc % VBUF]; vc += 1

    lines = ["s_waitcnt lgkmcnt(0)"]
    pending = []   # (unit, lgkm operations), oldest first

    def issue(u):
        r = buf[u]
        if u[0] == "S":
            lines.append("ds_read_b128 %s, %%[ka%d] offset:%%[koff]" % (_vr(r), u[1]))
            pending.append((u, 1))
        else:
            ks, db = u[1], u[2]
            lines.append("ds_read_b64_tr_b16 %s, %%[va%d_0] offset:%%[voff%d]" % (_vr(r, 2), db, ks))
            lines.append("ds_read_b64_tr_b16 %s, %%[va%d_1] offset:%%[voff%d]" % (_vr(r + 2, 2), db, ks))
            pending.append((u, 2))

    valu = []
    if do_softmax:
        t = ["v%d" % x for x in T_REGS]
        k = 0
        for pair in range(8):
            for rb in range(R):
                e0, e1 = 2 * pair, 2 * pair + 1
                ta, tb = t[(2 * k) % 4], t[(2 * k + 1) % 4]
                k += 1
                valu.append("v_fma_f32 %s, %%[sc%d_%d], %%[c], -%%[mx%d]" % (ta, rb, e0, rb))
                valu.append("v_fma_f32 %s, %%[sc%d_%d], %%[c], -%%[mx%d]" % (tb, rb, e1, rb))
                valu.append("v_exp_f32 %s, %s" % (ta, ta))
                valu.append("v_exp_f32 %s, %s" % (tb, tb))
                if pair == 0:
                    valu.append("v_mov_b32 %%[l%d_0], %s" % (rb, ta))
                    valu.append("v_mov_b32 %%[l%d_1], %s" % (rb, tb))
                else:
                    valu.append("v_add_f32 %%[l%d_0], %%[l%d_0], %s" % (rb, rb, ta))
                    valu.append("v_add_f32 %%[l%d_1], %%[l%d_1], %s" % (rb, rb, tb))
                valu.append("v_cvt_pk_bf16_f32 %%[pn%d_%d], %s, %s" % (rb, pair, ta, tb))

    nxt = 0
    while nxt < min(AHEAD, len(units)):
        issue(units[nxt]); nxt += 1
    vi = 0
    lead = min(LEAD, len(valu)) if units else len(valu)
    while vi < lead:
        lines.append(valu[vi]); vi += 1
    if units and len(lines) < 4:
        lines.append("s_nop 1")
    nmf = len(units) * R
    fill_i = 0
    tail = min(MFMA_TAIL, max(0, len(valu) - lead)) if units else 0
    per = (len(valu) - lead - tail) / max(1, nmf)
    mfi = 0
    for u in units:
        idx = [p[0] for p in pending].index(u)
        lines.append("s_waitcnt lgkmcnt(%d)" % sum(c for (_, c) in pending[idx + 1:]))
        del pending[:idx + 1]
        r = buf[u]
        for rb in range(R):
            if u[0] == "S":
                d = u[1]
                lines.append("v_mfma_f32_32x32x16_bf16 %%[sn%d], %s, %%[q%d_%d], %s"
                             % (rb, _vr(r), rb, d, "0" if d == 0 else "%%[sn%d]" % rb))
            else:
                ks, db = u[1], u[2]
                lines.append("v_mfma_f32_32x32x16_bf16 %%[o%d_%d], %s, %%[pp%d_%d], %%[o%d_%d]"
                             % (rb, db, _vr(r), rb, ks, rb, db))
            mfi += 1
            if fills and mfi % (nmf // fills) == nmf // (2 * fills) and fill_i < fills:
                lines += fill_piece(fill_i, fills, desc)
                fill_i += 1
            if rb == 0 and nxt < len(units):
                issue(units[nxt]); nxt += 1
            target = lead + int(round(per * mfi))
            while vi < min(target, len(valu)):
                lines.append(valu[vi]); vi += 1
    while vi < len(valu):
        lines.append(valu[vi]); vi += 1
    assert not pending
    assert fill_i == fills, (fill_i, fills)
    # keep the block going past its last MFMA: softmax work moved to the tail, else s_nop
    if units:
        last_mf = max(i for i, ln in enumerate(lines) if ln.startswith("v_mfma"))
        after = len(lines) - 1 - last_mf
        if after < MFMA_TAIL:
            lines.append("s_nop %d" % (MFMA_TAIL - after - 1))
    if do_scores:
        last = max(i for i, ln in enumerate(lines)
                   if ln.startswith("v_mfma") and ln.split(",")[0].endswith(("%[sn0]", "%[sn1]")))
        after = len(lines) - 1 - last
        if after < XDL_VALU_WAIT:
            lines.append("s_nop %d" % (XDL_VALU_WAIT - after - 1))
    # a transcendental result must not be read by the next instruction
    for i in range(len(lines) - 1):
        if lines[i].startswith("v_exp_f32"):
            dst = lines[i].split()[1].rstrip(",")
            nxt_ops = lines[i + 1].split(None, 1)[1] if " " in lines[i + 1] else ""
            assert dst not in [x.strip() for x in nxt_ops.split(",")][1:], lines[i:i + 2]
    return units, lines


MIN_REUSE_GAP = 2   # MFMAs between an MFMA reading a fragment buffer and an LDS read into it


def check_fragment_reuse(lines):
    """An LDS read may refill a fragment buffer only after MIN_REUSE_GAP further MFMAs have
    issued past the last MFMA that reads it: the read's data can land before a queued MFMA
    has fetched its operand (seen with one MFMA in between: wrong results).  ``lines`` is a
    phase followed by the next phase, so the reuse across the phase boundary is checked
    too (the code between two phases only adds distance)."""
    last_reader = {}      # buffer base register -> MFMA count at its last read
    n_mfma = 0
    for ln in lines:
        if ln.startswith("v_mfma"):
            n_mfma += 1
            a_op = ln.split(",")[1].strip()
            if a_op.startswith("v["):
                last_reader[int(a_op[2:].split(":")[0])] = n_mfma
        elif ln.startswith("ds_read"):
            dst = ln.split()[1].rstrip(",")
            base = int(dst[2:].split(":")[0])
            for b in (base, base - 2):           # a transposing read fills half a buffer
                if b in last_reader:
                    gap = n_mfma - last_reader[b]
                    assert gap >= MIN_REUSE_GAP, (ln, gap)


def emit(D, name, do_scores, do_pv, do_softmax, fills=0, skippable=False, desc=False):
    nds, ndb = D // 16, D // 32
    units, lines = phase_lines(D, do_scores, do_pv, do_softmax, fills, desc)
    if skippable:
        # a wave-uniform test skips the computation; the fill loads are issued either way
        fl = []
        for i in range(fills):
            fl += fill_piece(i, fills, desc)
        lines = (["s_cmp_gt_i32 %[sj], %[sjmax]", "s_cbranch_scc1 .Lfill_only_%="] + lines +
                 ["s_branch .Lphase_end_%=", ".Lfill_only_%=:"] + fl + [".Lphase_end_%=:"])
    params, outs, ins, pre, post = [], [], [], [], []
    if do_pv:
        params.append("f32x16 (&o)[%d][%d]" % (R, ndb))
        outs += ['[o%d_%d] "+a"(o[%d][%d])' % (rb, db, rb, db) for rb in range(R) for db in range(ndb)]
        params.append("const bf16x8 (&pp)[%d][2]" % R)
        ins += ['[pp%d_%d] "v"(pp[%d][%d])' % (rb, ks, rb, ks) for rb in range(R) for ks in range(2)]
        params.append("const unsigned (&va)[%d][2]" % ndb)
        ins += ['[va%d_%d] "v"(va[%d][%d])' % (db, h, db, h) for db in range(ndb) for h in range(2)]
        ins += ['[voff0] "i"(VOFF)', '[voff1] "i"(VOFF + 16 * %d * 2)' % D]
    if do_scores:
        params.append("const bf16x8 (&q)[%d][%d]" % (R, nds))
        ins += ['[q%d_%d] "v"(q[%d][%d])' % (rb, d, rb, d) for rb in range(R) for d in range(nds)]
        params.append("f32x16 (&sn)[%d]" % R)
        outs += ['[sn%d] "=&v"(sn[%d])' % (rb, rb) for rb in range(R)]
        params.append("const unsigned (&ka)[%d]" % nds)
        ins += ['[ka%d] "v"(ka[%d])' % (d, d) for d in range(nds)]
        ins.append('[koff] "i"(KOFF)')
    if do_softmax:
        params.append("const f32x16 (&sc)[%d]" % R)
        ins += ['[sc%d_%d] "v"(sc[%d][%d])' % (rb, e, rb, e) for rb in range(R) for e in range(16)]
        params += ["float c", "const float (&m)[%d]" % R, "bf16x8 (&pn)[%d][2]" % R,
                   "float (&l)[%d][2]" % R]
        ins += ['[c] "s"(c)'] + ['[mx%d] "v"(m[%d])' % (rb, rb) for rb in range(R)]
        pre.append("unsigned pw[%d][8];" % R)
        outs += ['[pn%d_%d] "=&v"(pw[%d][%d])' % (rb, i, rb, i) for rb in range(R) for i in range(8)]
        outs += ['[l%d_%d] "=&v"(l[%d][%d])' % (rb, h, rb, h) for rb in range(R) for h in range(2)]
        for rb in range(R):
            for ks in range(2):
                post.append("pn[%d][%d] = __builtin_bit_cast(bf16x8, u32x4{pw[%d][%d], pw[%d][%d], "
                            "pw[%d][%d], pw[%d][%d]});"
                            % (rb, ks, rb, 4 * ks, rb, 4 * ks + 1, rb, 4 * ks + 2, rb, 4 * ks + 3))
    if fills:
        params += ["__amdgpu_buffer_rsrc_t fr", "unsigned fm", "unsigned& fo", "unsigned fs"]
        outs.append('[fo] "+v"(fo)')
        ins += ['[fr] "s"(fr)', '[fm] "s"(fm)', '[fs] "s"(fs)']
    if skippable:
        # the computation is skipped when j > jmax (two integers: a flag would be materialised
        # in a VGPR by the compiler)
        params += ["int j", "int jmax"]
        ins += ['[sj] "s"(j)', '[sjmax] "s"(jmax)']
    params.append("u32x4 (&fx)[%d]" % len(FIX_TUPLES))
    outs += ['"+{v[%d:%d]}"(fx[%d])' % (a, b, i) for i, (a, b) in enumerate(FIX_TUPLES)]
    clob = ['"memory"'] + (['"m0"', '"scc"'] if fills or skippable else [])
    body = "".join('      "%s\\n"\n' % ln for ln in lines)
    what = [w for w, f in (("scores", do_scores), ("P.V", do_pv), ("softmax", do_softmax)) if f]
    s = ["// %s: %d MFMA, %d instructions" % (" + ".join(what), len(units) * R, len(lines))]
    if do_scores or do_pv:
        s.append("template <int KOFF, int VOFF>")
    s.append("__device__ __forceinline__ void %s(%s) {" % (name, ", ".join(params)))
    s += ["  " + p for p in pre]
    s.append("  asm volatile(\n%s      : %s\n      : %s\n      : %s);"
             % (body, ", ".join(outs), ", ".join(ins), ", ".join(clob)))
    s += ["  " + p for p in post]
    s.append("}")
    return "\n".join(s)


def emit_o_helpers(D):
    """Accesses of O outside the phases.  O (f32x16 tiles o[R][D/32], one per 32-row block
    and 32-wide d block) is only ever an AGPR asm operand, so the compiler never copies it
    into VGPRs; element-wise work names each of the 16 AGPRs of a tile as its own operand."""
    ndb = D // 32
    n = ndb * 16
    out = []
    for rb in range(R):
        outs = ", ".join('"=a"(o[%d][%d][%d])' % (rb, db, e) for db in range(ndb) for e in range(16))
        body = "".join('      "v_accvgpr_write_b32 %%%d, 0\\n"\n' % i for i in range(n))
        out.append("__device__ __forceinline__ void o_zero_%d(f32x16 (&o)[%d][%d]) {\n"
                   "  asm volatile(\n%s      : %s);\n}" % (rb, R, ndb, body, outs))
    for rb in range(R):
        outs = ", ".join('"+a"(o[%d][%d][%d])' % (rb, db, e) for db in range(ndb) for e in range(16))
        body = ""
        for i in range(n):
            t = T_REGS[i % 4]
            body += '      "v_accvgpr_read_b32 v%d, %%%d\\n"\n' % (t, i)
            body += '      "v_mul_f32 v%d, v%d, %%[f]\\n"\n' % (t, t)
            body += '      "v_accvgpr_write_b32 %%%d, v%d\\n"\n' % (i, t)
        outs += ', "+{v[%d:%d]}"(fx0)' % FIX_TUPLES[0]
        out.append("__device__ __forceinline__ void o_scale_%d(f32x16 (&o)[%d][%d], float f, u32x4& fx0) {\n"
                   "  asm volatile(\n%s      : %s\n      : [f] \"v\"(f));\n}"
                   % (rb, R, ndb, body, outs))
    ins = ", ".join('"a"(t[%d])' % e for e in range(16))
    outs = ", ".join('"=v"(x[%d])' % e for e in range(16))
    body = "".join('      "v_accvgpr_read_b32 %%%d, %%%d\\n"\n' % (e, 16 + e) for e in range(16))
    out.append("__device__ __forceinline__ f32x16 o_read(const f32x16& t) {\n  float x[16];\n"
               "  asm volatile(\n%s      : %s\n      : %s);\n  f32x16 r;\n"
               "#pragma unroll\n  for (int e = 0; e < 16; ++e) r[e] = x[e];\n  return r;\n}"
               % (body, outs, ins))
    return "\n\n".join(out)


# the prologue's phases (the loop uses phase_step_up / phase_step_down): scores of sub-tile 0,
# then scores of sub-tile 1 with the softmax of sub-tile 0
VARIANTS = (("scores_softmax", True, False, True), ("scores", True, False, False))


def header():
    out = ["// tile_phases.inc -- generated by gen_tile_phases.py; do not edit by hand.",
           "// The inner-loop phases of the wide attention kernel (gqa_fwd_wide_kernel.hpp):",
           "// for 32-key sub-tile j, scores of sub-tile j+1, P.V of sub-tile j-1 and the",
           "// softmax of sub-tile j in one instruction stream.  See the generator for the",
           "// register and hazard rules.",
           "#pragma once", "", "namespace h3attn {", "namespace wide {", ""]
    for D in (128,):
        out.append("namespace d%d {" % D)
        for name, s, p, x in VARIANTS:
            out.append(emit(D, "phase_" + name, s, p, x))
            out.append("")
        _, up = phase_lines(D, True, True, True, FILLS_PER_PHASE, False)
        _, down = phase_lines(D, True, True, True, FILLS_PER_PHASE, True)
        check_fragment_reuse(up + down)
        check_fragment_reuse(down + up)
        out.append(emit(D, "phase_step_up", True, True, True, fills=FILLS_PER_PHASE, skippable=True))
        out.append("")
        out.append(emit(D, "phase_step_down", True, True, True, fills=FILLS_PER_PHASE,
                        skippable=True, desc=True))
        out.append("")
        out.append(emit_o_helpers(D))
        out.append("")
        out.append("}  // namespace d%d" % D)
    out += ["", "}  // namespace wide", "}  // namespace h3attn", ""]
    return "\n".join(out)


PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tile_phases.inc")

if __name__ == "__main__":
    text = header()
    if "--check" in sys.argv:
        with open(PATH) as f:
            sys.exit(0 if f.read() == text else 1)
    with open(PATH, "w") as f:
        f.write(text)
