"""Register check on the gfx950 code of the kernels (no GPU needed).

v_cvt_scalef32_2xpk16_fp6_f32 packs 32 fp32 values into 6 dwords of E2M3
codes in several passes, and the passes after the first read sources that
the first has already written when the destination overlaps them.  The
compiler does not treat that as a constraint, so the kernels keep the
sources live past the conversion.  This test compiles both kernel sources
to assembly with the library's build flags and checks that no conversion's
destination registers overlap its source or scale registers.  (An overlap
once turned every P block of the d = 64 MX attention into garbage after its
first two elements.)
"""
import os
import re
import subprocess
import tempfile

import pytest

from quantized_attention_video_02_amd import build as bld

CONV = "v_cvt_scalef32_2xpk16_fp6_f32"


def _regs(op: str) -> set:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


def _overlaps(asm: str):
    found, bad = 0, []
    for line in asm.splitlines():
        line = line.split(";")[0].strip()
        if not line.startswith(CONV):
            continue
        found += 1
        ops = [o.strip() for o in line[len(CONV):].split(",")]
        dst, srcs = _regs(ops[0]), set().union(*(_regs(o) for o in ops[1:4]))
        assert len(dst) == 6, line
        if dst & srcs:
            bad.append(line)
    return found, bad


def test_overlap_detector():
    ok = f"\t{CONV} v[174:179], v[130:145], v[146:161], v192\n"
    assert _overlaps(ok) == (1, [])
    for bad in (f"{CONV} v[122:127], v[100:115], v[84:99], v122",      # the scale
                f"{CONV} v[10:15], v[0:15], v[16:31], v40",             # the first source
                f"{CONV} v[30:35], v[0:15], v[16:31], v40"):            # the second source
        assert _overlaps(bad)[0] == 1 and len(_overlaps(bad)[1]) == 1


@pytest.mark.parametrize("src,min_count", [("sage_attn.hip", 4), ("sage_quant.hip", 2)])
def test_fp6_pack_registers_disjoint(src, min_count):
    try:
        cc = bld.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    flags = [f for f in bld.HIPFLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        r = subprocess.run([cc, *flags, "-I", bld.INCLUDE, "--cuda-device-only", "-S",
                            os.path.join(bld.CSRC, src), "-o", out],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            found, bad = _overlaps(f.read())
    assert found >= min_count, found
    assert not bad, bad
