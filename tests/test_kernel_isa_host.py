"""Check the generated gfx950 code of the tiled GEMM for the invariant its
k-pair waits rely on (no GPU; compiles gemm.hip to assembly with hipcc).

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
ARGS = re.compile(r"ILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELi(\d+)ELi(\d+)E")


def _epilogue_loads(wm, wn, tm, tn, rt, spl):
    late = tm * rt * spl > 16 or tm * rt >= 16
    return 2 * tn + tn * rt + (tm * rt if (not late and rt > 0) else 0)


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_epilogue_loads_follow_the_first_copies(tmp_path):
    out = tmp_path / "gemm.s"
    cmd = [B.HIPCC] + B.COMMON + ["-x", "hip", "--cuda-device-only", "-S",
                                  os.path.join(B.CSRC, "gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = out.read_text().split("\n")
    checked = 0
    for i, line in enumerate(lines):
        m = NAME.match(line)
        if not m:
            continue
        wm, wn, tm, tn, rt, ns, spl, glu, occ, ks = map(int, ARGS.search(m.group(1)).groups())
        if occ >= 3:
            continue   # the lean variant loads its epilogue operands after the loop
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
        want = _epilogue_loads(wm, wn, tm, tn, rt, spl)
        assert len(loads) >= want, (m.group(1), len(loads), want)
        nw = wm * wn
        ops = (wm * tm + wn * tn + nw - 1) // nw + 1
        waits = {int(v) for v in re.findall(r"s_waitcnt vmcnt\((\d+)\)", "\n".join(body))}
        assert want in waits or ops + want in waits or 2 * ops + want in waits, m.group(1)
        checked += 1
    assert checked >= 100   # every non-lean instance of every tile shape, rank and variant
