"""Checks on the gfx950 assembly of this library's own kernels (CPU only).

The kernels rely on properties the compiler could silently break:

* the global->LDS copies are inline assembly that load M0 themselves, so no
  compiler-generated instruction may write M0 (it would race with them);
* the hot loops count outstanding copies exactly, so no kernel may spill
  registers to scratch (a spill reload inside a loop would also wait for the
  copies in flight);
* packed fp32 VALU instructions are not used on this hardware (the build
  disables them; this checks that none appear).
"""

import os
import re
import subprocess

import pytest

from shared_prefix_tree_amd import build as b

SOURCES = ["fwd.hip", "bwd.hip"]


def assembly(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [b.HIPCC, *b.FLAGS, "-x", "hip", "--cuda-device-only", "-S", os.path.join(b.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernels(asm):
    """(name, body lines) of every kernel function in the assembly."""
    found = []
    for m in re.finditer(r"^(_ZN9tree_attn\w+_kernel\w*):", asm, flags=re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        found.append((name, asm[m.end():end].splitlines()))
    return found


def meta(asm, name, key):
    m = re.search(rf"\.set {re.escape(name)}\.{key}, (\d+)", asm)
    return int(m.group(1)) if m else None


@pytest.fixture(scope="module")
def asms(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("asm")
    return {src: assembly(src, tmp) for src in SOURCES}


@pytest.mark.parametrize("src", SOURCES)
def test_kernels_do_not_spill(asms, src):
    ks = kernels(asms[src])
    assert ks, "no kernels found"
    for name, body in ks:
        assert not any(l.strip().startswith("scratch_") for l in body), f"{name} spills to scratch"
        assert meta(asms[src], name, "private_seg_size") == 0, name


@pytest.mark.parametrize("src", SOURCES)
def test_m0_is_written_only_by_the_copy_assembly(asms, src):
    for name, body in kernels(asms[src]):
        inside = False
        for l in body:
            s = l.strip()
            if s.startswith(";;#ASMSTART"):
                inside = True
            elif s.startswith(";;#ASMEND"):
                inside = False
            elif not inside and re.match(r"s_\w+\s+m0\b", s):
                pytest.fail(f"{name}: compiler-generated write of M0: {s}")


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32_valu(asms, src):
    bad = re.findall(r"\bv_pk_(?:add|mul|fma|mov)_f32\b", asms[src])
    assert not bad, bad[:5]
