"""Checks of the generated gfx950 code (no GPU; compiles the kernels to
assembly with hipcc): the invariant the tiled GEMM's k-pair waits rely on,
and the register / LDS / scratch budget of every kernel instance.

The non-lean tiled kernel issues its epilogue-operand loads at k-pair 0
right behind that iteration's LDS copies, and the waits for stages 1 .. NS-1
leave kEpiLoads = 2 TN + TN RT (+ TM RT when lora_act partial 0 is loaded
early) loads in flight besides the younger stages.  Loads complete in issue
order, so the waits are exact only if the code really issues at least that
many loads between the k-pair-0 copies and the next wait: fewer would let a
wait return before its stage has landed.
"""
import os
import re
import shutil
import subprocess

import pytest

from w4a4_gemm_lora_amd import build as B

NAME = re.compile(r"^(_ZN4w4a417gemm_tiled_kernelI\S*):")
ARGS = re.compile(r"ILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E")


def _epilogue_loads(wm, wn, tm, tn, rt, spl, qout=0):
    late = tm * rt * spl > 16 or tm * rt >= 16 or (qout and tm * rt * spl >= 16)
    return 2 * tn + tn * rt + (tm * rt if (not late and rt > 0) else 0)


HAVE_HIPCC = shutil.which(B.HIPCC) is not None or os.path.exists(B.HIPCC)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """gfx950 assembly of each .hip source, compiled once for this module."""
    if not HAVE_HIPCC:
        pytest.skip("hipcc not installed")
    d = tmp_path_factory.mktemp("asm")
    out = {}
    for src in ("gemm.hip", "quantize.hip"):
        o = d / (src + ".s")
        cmd = [B.HIPCC] + B.COMMON + ["-x", "hip", "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(o)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[src] = o.read_text()
    return out


def test_epilogue_loads_follow_the_first_copies(asm):
    lines = asm["gemm.hip"].split("\n")
    checked = 0
    for i, line in enumerate(lines):
        m = NAME.match(line)
        if not m:
            continue
        wm, wn, tm, tn, rt, ns, spl, glu, occ, ks, psum, qout = map(int, ARGS.search(m.group(1)).groups())
        if occ >= 3:
            continue   # the lean variant loads its epilogue operands after the loop
        if psum:
            continue   # the diagnostic instances load no epilogue operands
        body = []
        for t in lines[i + 1:]:
            if t.startswith(".Lfunc_end"):
                break
            body.append(t.strip())
        barriers = [k for k, t in enumerate(body) if t == "s_barrier"]
        assert len(barriers) >= 2, m.group(1)
        seg = body[barriers[0]:barriers[1]]   # k-pair 0: after its barrier, up to k-pair 1's
        last_copy = max(k for k, t in enumerate(seg) if "global_load_lds" in t)
        loads = [t for t in seg[last_copy:] if t.startswith("global_load_dword") and "lds" not in t]
        want = _epilogue_loads(wm, wn, tm, tn, rt, spl, qout)
        assert len(loads) >= want, (m.group(1), len(loads), want)
        nw = wm * wn
        ops = (wm * tm + wn * tn + nw - 1) // nw + 1
        waits = {int(v) for v in re.findall(r"s_waitcnt vmcnt\((\d+)\)", "\n".join(body))}
        assert want in waits or ops + want in waits or 2 * ops + want in waits, m.group(1)
        checked += 1
    assert checked >= 100   # every non-lean instance of every tile shape, rank and variant


# ---------------------------------------------------------------------------
# Resource budget of every kernel instance ("High-Performance Kernel Design for
# W4A4 ... on Blackwell", sections 4-5: a pipeline depth that overruns the
# on-chip budget fails silently as lost performance, so the budget is checked,
# not assumed).  gfx950: 512 VGPRs (arch + accumulation, 8-register granules)
# per SIMD lane shared by the waves on it, 160 KiB of LDS per CU.
KDESC = re.compile(r"^\s*\.amdhsa_kernel (\S+)$")
TILED = re.compile(r"gemm_tiled_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)"
                   r"ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)E")
WIDE = re.compile(r"gemm_wide_kernelILi(\d+)ELi(\d+)ELb(\d)ELb(\d)E")
DECODE = re.compile(r"gemm_decode_(?:dot_)?kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELi(\d+)ELb(\d)E")
LDS_PER_CU = 160 * 1024


def _descriptors(text):
    """{kernel name: {field: int}} from the .amdhsa_kernel blocks."""
    out, cur = {}, None
    for line in text.split("\n"):
        m = KDESC.match(line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        if cur is not None:
            t = line.split()
            if t and t[0] == ".end_amdhsa_kernel":
                cur = None
            elif len(t) == 2 and t[0].startswith(".amdhsa_"):
                cur[t[0][len(".amdhsa_"):]] = int(t[1])
    return out


def _waves_per_simd(d):
    regs = (d["next_free_vgpr"] + 7) // 8 * 8
    return min(8, 512 // regs)


def test_every_instance_fits_its_occupancy(asm):
    """No instance uses scratch (spills or private arrays), and each fits
    the occupancy its launch bounds promise.  The bound's second argument is
    a minimum of waves per SIMD (the compiler's register budget is 512 / it):
    a tiled instance built for OCC (WM x WN x KS waves per workgroup, KS / 1
    or 2 waves of it on each SIMD) must keep OCC waves on every SIMD by
    registers and OCC / (WM WN KS / 4) workgroups per CU by LDS; a decode
    instance (DW waves, bound 16 / DW) keeps 4 waves per SIMD.  The
    instances with the quantized gated output are held to their tile
    shape's occupancy like the others.  The
    diagnostic (group-sum) instances are built for one workgroup per CU and
    checked against that.  The wide kernel (4 waves) is built for two
    workgroups per CU."""
    seen = {"tiled": 0, "tiled_qout": 0, "wide": 0, "decode": 0, "other": 0}
    for src, text in asm.items():
        for name, d in _descriptors(text).items():
            assert d["private_segment_fixed_size"] == 0, f"{name}: {d['private_segment_fixed_size']} B of scratch"
            lds = d["group_segment_fixed_size"]
            m = TILED.search(name)
            if m:
                wm, wn, tm, tn, rt, ns, spl, glu, occ, ks, psum, qout = map(int, m.groups())
                per_wg = max(1, wm * wn * ks // 4)   # waves of one workgroup on each SIMD
                want = max(per_wg, 1 if psum else occ)
                assert _waves_per_simd(d) >= want, (name, d["next_free_vgpr"], want)
                assert (want // per_wg) * lds <= LDS_PER_CU, (name, lds, want)
                seen["tiled"] += 1
                seen["tiled_qout"] += qout
                continue
            m = WIDE.search(name)
            if m:   # 4 waves, built for 2 workgroups per CU (1 for the diagnostic instance)
                blocks = 1 if int(m.group(4)) else 2
                assert _waves_per_simd(d) >= blocks, (name, d["next_free_vgpr"])
                assert blocks * lds <= LDS_PER_CU, (name, lds)
                seen["wide"] += 1
                continue
            m = DECODE.search(name)
            if m:
                dw, psum = int(m.group(6)), int(m.group(7))
                blocks = 1 if psum else 16 // dw
                assert _waves_per_simd(d) >= max(1, blocks * dw // 4), (name, d["next_free_vgpr"])
                assert blocks * lds <= LDS_PER_CU, (name, lds, dw)
                seen["decode"] += 1
                continue
            assert lds <= LDS_PER_CU, (name, lds)
            seen["other"] += 1
    assert seen["tiled"] >= 100 and seen["wide"] >= 10 and seen["decode"] >= 40 and seen["other"] >= 5, seen
    # the quantized gated output: 128 x 128 and 64 x 128, both occupancies, every rank, 1 or 4 partials
    assert seen["tiled_qout"] == 2 * 2 * 5 * 2, seen


def test_rmsnorm_conversion_keeps_its_fp32_step(asm):
    """The fused RMSNorm pass rounds its fp64 value to fp32 and then to fp16
    (two hardware conversions per value).  Under fp contraction the backend
    may merge the two into one software fp64 -> fp16 rounding, recognisable
    by its extraction of the double's exponent field (bits 20..30 of the
    high dword); that rounding differs from the two-step one at fp16 ties of
    the fp32 value, so no instance may contain it."""
    lines = asm["quantize.hip"].split("\n")
    name, checked = None, 0
    for line in lines:
        m = re.match(r"^(_ZN4w4a420quantize_rows_kernelILi\d+ELi\d+ELb(\d)E\S*):", line)
        if m:
            name = m.group(1) if m.group(2) == "1" else None
            checked += name is not None
            continue
        if name and re.search(r"v_bfe_u32\s+v\d+, v\d+, 20, 11\b", line):
            raise AssertionError(f"{name}: one-step fp64 -> fp16 conversion")
    assert checked >= 15   # every RMSNorm instance (rank 0..64, 2..16 waves)
