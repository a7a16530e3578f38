"""The direct global-to-LDS loads are written as inline assembly that sets M0 (the instruction's LDS address) and
declares M0 clobbered.  The compiler does not preserve a reserved register across such a statement, so this is safe
only while compiled code keeps no value of its own in M0.  This test compiles every kernel source for gfx950 to
assembly (on the CPU) and checks exactly that: every M0 write is one of those statements (a scalar move into M0
followed by the load), and no instruction that reads M0 implicitly or explicitly (indirect register moves, messages,
GWS / append / consume LDS operations, interpolation) appears anywhere."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

IMPLICIT_M0 = re.compile(r"^\s*(v_movrel|s_movrel|s_set_gpr_idx|s_sendmsg|ds_gws|ds_append|ds_consume|ds_ordered|"
                         r"v_interp|s_ttracedata|lds_param|lds_direct)")


def _asm(src):
    from sparse_attention_kpool_amd import build as B
    flags = [f for f in B.COMPILE_FLAGS if f not in ("-fPIC",)]
    cmd = [B.hipcc(), *flags, *B.FILE_FLAGS.get(os.path.basename(src), []), "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"device assembly unavailable: {r.stderr[-300:]}")
    return r.stdout


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(os.path.join(ROOT, "sparse_attention_kpool_amd", "csrc"))
                                  if f.endswith(".hip")))
def test_m0_holds_only_the_direct_load_address(name):
    try:
        from sparse_attention_kpool_amd import build as B
        B.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    lines = [l.split(";")[0].rstrip() for l in _asm(os.path.join(ROOT, "sparse_attention_kpool_amd", "csrc", name))
             .splitlines()]
    code = [l for l in lines if l.strip() and not l.strip().startswith(".") and not l.strip().endswith(":")]
    for i, l in enumerate(code):
        assert not IMPLICIT_M0.match(l), f"{name}: an instruction that reads M0: {l.strip()}"
        if re.search(r"\bm0\b", l):
            assert re.match(r"^\s*s_mov_b32 m0, s\d+$", l), f"{name}: M0 used outside the direct loads: {l.strip()}"
            nxt = [c.strip() for c in code[i + 1:i + 3]]
            assert nxt[0] == "s_nop 0" and nxt[1].startswith("global_load_lds_dwordx4"), \
                f"{name}: an M0 write not followed by its direct load: {nxt}"
