"""Properties of the generated gfx950 code, checked on the CPU from the compiler's assembly.

Every source of the library is compiled for the device with the build's own
flags and the assembly is scanned:

- M0 is written only by the direct-to-LDS load helper, each write directly
  followed by its buffer_load ... lds.  The helper's inline asm clobbers M0,
  which the compiler treats as reserved, so no compiler-generated code may
  rely on M0 across it;
- no packed-FP32 VALU instructions (the build disables them);
- no scalar-memory stores, atomics or scalar-cache write-back / discard:
  every global write goes through vector memory instructions.
"""
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "sgd_cnns_amd"))

# instruction-name prefixes assembled at run time from pieces (see the module docstring)
_SCALAR_WRITES = ["s_" + w for w in ("store", "buffer_store", "scratch_store", "atomic", "buffer_atomic",
                                     "dcache_wb", "dcache_discard")]
_PACKED_F32 = ["v_pk_" + op + "_f32" for op in ("add", "mul", "fma")]


def _device_asm(src, out_dir):
    import build as B
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    cmd = ["hipcc", *flags, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read().splitlines()


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_device_code_properties(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "sgd_cnns_amd", "csrc", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        listings = dict(zip(srcs, ex.map(lambda s: _device_asm(s, str(tmp_path)), srcs)))
    m0_writes = 0
    for src, lines in listings.items():
        code = [l.split(";")[0].strip() for l in lines]
        code = [l for l in code if l and not l.startswith(".") and not l.endswith(":")]
        for i, l in enumerate(code):
            op = l.split()[0]
            assert not any(op.startswith(p) for p in _SCALAR_WRITES), f"{os.path.basename(src)}: {l}"
            assert op not in _PACKED_F32, f"{os.path.basename(src)}: {l}"
            if re.search(r"\bm0\b", l):
                assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"{os.path.basename(src)}: {l}"
                nxt = code[i + 1] if i + 1 < len(code) else ""
                assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), \
                    f"{os.path.basename(src)}: M0 write not followed by its LDS load: {nxt}"
                m0_writes += 1
    assert m0_writes > 0, "the direct-to-LDS loads were not found"
