"""Host-only checks of the C ABI: the library loads, exports every entry
point declared in include/gla.h, and rejects bad arguments with the
documented status before any HIP call (so these run without a GPU)."""
import ctypes as ct
import os
import re

import pytest

from gated_deltanet_gla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"GLA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert {"gla_chunk_fwd", "gdn_chunk_fwd", "gla_decode_step", "gdn_decode_step",
            "causal_conv1d_fwd"} <= set(names)
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    assert _lib.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5, -6):
        assert _lib.status_string(st) not in ("ok", "unknown status")
    assert _lib.lib().gla_version().decode().count(".") == 2


FAKE = 0x1000   # never dereferenced: validation fails before any launch


def _chunk_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, cu=FAKE, B=2, N=10, H=4, dk=128, dv=128, C=64,
             idt=1, odt=1, pool=FAKE, n_slots=4, slots=FAKE, flags=0, o=FAKE, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return a


def _gla_chunk(a):
    return _lib.lib().gla_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["cu"], a["B"], a["N"],
                                    a["H"], a["dk"], a["dv"], a["C"], a["idt"], a["odt"], a["pool"],
                                    a["n_slots"], a["slots"], a["flags"], a["o"], a["ws"], a["wsb"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.GLA_EPTR), (dict(pool=None), _lib.GLA_EPTR), (dict(cu=None), _lib.GLA_EPTR),
    (dict(dk=96), _lib.GLA_ESHAPE), (dict(dv=256), _lib.GLA_ESHAPE), (dict(H=0), _lib.GLA_ESHAPE),
    (dict(N=-1), _lib.GLA_ESHAPE), (dict(B=-3), _lib.GLA_ESHAPE), (dict(n_slots=0), _lib.GLA_ESHAPE),
    (dict(C=48), _lib.GLA_ECHUNK), (dict(C=128), _lib.GLA_ECHUNK), (dict(idt=2), _lib.GLA_EDTYPE),
    (dict(odt=-1), _lib.GLA_EDTYPE), (dict(flags=8), _lib.GLA_ESHAPE), (dict(B=0), _lib.GLA_ESHAPE),
])
def test_gla_chunk_validation(kw, status):
    assert _gla_chunk(_chunk_args(**kw)) == status


def test_gla_chunk_workspace_contract():
    L = _lib.lib()
    need = L.gla_chunk_workspace_bytes(2, 10, 4, 128, 128, 64)
    assert need > 0                                     # segmented path keeps per-segment states
    assert _gla_chunk(_chunk_args()) == _lib.GLA_EWORKSPACE
    assert _gla_chunk(_chunk_args(ws=FAKE, wsb=need - 1)) == _lib.GLA_EWORKSPACE
    # bound grows with the token count and covers one 128x128 fp32 state per segment and head
    big = L.gla_chunk_workspace_bytes(4, 16384, 16, 128, 128, 64)
    assert big >= (16384 // 1024 + 4 - 1) * 16 * 128 * 128 * 4
    assert L.gla_chunk_workspace_bytes(2, 10, 4, 64, 64, 64) == 0
    assert L.gla_chunk_workspace_bytes(2, 10, 4, 100, 128, 64) == 0


def test_empty_calls_are_noops():
    # nothing to do -> OK without touching any pointer
    assert _gla_chunk(_chunk_args(B=0, N=0, q=None, k=None, v=None, pool=None, cu=None)) == 0
    L = _lib.lib()
    assert L.gla_decode_step(None, None, None, None, 0, 16, 128, 128, 1, 1, None, 4, None, None,
                             None) == 0


def test_gdn_chunk_validation():
    L = _lib.lib()
    a = _chunk_args()
    args = [a["q"], a["k"], a["v"], a["alpha"], None, a["cu"], a["B"], a["N"], a["H"], a["dk"],
            a["dv"], a["C"], a["idt"], a["odt"], a["pool"], a["n_slots"], a["slots"], 0, a["o"],
            None, 0, None]
    assert L.gdn_chunk_fwd(*args) == _lib.GLA_EPTR          # beta missing
    need = L.gdn_chunk_workspace_bytes(2, 10, 4, 128, 128, 64)
    args[4] = FAKE
    if need:
        assert L.gdn_chunk_fwd(*args) == _lib.GLA_EWORKSPACE
        args[19], args[20] = FAKE, need - 1
        assert L.gdn_chunk_fwd(*args) == _lib.GLA_EWORKSPACE
    assert L.gdn_chunk_workspace_bytes(2, 10, 4, 100, 128, 64) == 0


def test_decode_validation():
    L = _lib.lib()
    base = [FAKE, FAKE, FAKE, FAKE, 8, 16, 128, 128, 1, 1, FAKE, 32, FAKE, FAKE, None]
    for i, bad, st in [(0, None, -1), (10, None, -1), (12, None, -1), (13, None, -1),
                       (6, 100, -2), (7, 8, -2), (8, 5, -3), (11, 0, -2), (4, -1, -2)]:
        args = list(base)
        args[i] = bad
        assert L.gla_decode_step(*args) == st, (i, bad)
    gargs = base[:4] + [None] + base[4:]
    assert L.gdn_decode_step(*gargs) == -1


def test_conv_validation():
    L = _lib.lib()
    base = [FAKE, FAKE, FAKE, 2, 10, 2048, 4, FAKE, 8, FAKE, 0, FAKE, 1, None]
    for i, bad, st in [(0, None, -1), (1, None, -1), (5, 12, -2), (6, 5, -2), (6, 1, -2),
                       (12, 3, -3), (8, 0, -2), (10, 4, -2), (11, None, -1)]:
        args = list(base)
        args[i] = bad
        assert L.causal_conv1d_fwd(*args) == st, (i, bad)


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no CPU path."""
    pkg = os.path.join(ROOT, "gated_deltanet_gla_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("no oracle", ""), fn


def test_decode_multi_and_copy_validation():
    L = _lib.lib()
    # q k v alpha R J H dk dv idt odt pool n_slots slots pos o stream
    base = [FAKE, FAKE, FAKE, FAKE, 8, 4, 16, 128, 128, 1, 1, FAKE, 64, FAKE, FAKE, FAKE, None]
    for i, bad, st in [(0, None, -1), (14, None, -1), (15, None, -1), (11, None, -1),
                       (5, -1, -2), (7, 100, -2), (9, 7, -3), (12, 0, -2), (4, -2, -2)]:
        args = list(base)
        args[i] = bad
        assert L.gla_decode_multi(*args) == st, (i, bad)
    gargs = base[:4] + [None] + base[4:]
    assert L.gdn_decode_multi(*gargs) == -1
    # nothing to do: OK without touching pointers
    assert L.gla_decode_multi(None, None, None, None, 0, 4, 16, 128, 128, 1, 1, None, 4, None,
                              None, None, None) == 0
    assert L.gla_decode_multi(FAKE, FAKE, FAKE, FAKE, 8, 0, 16, 128, 128, 1, 1, FAKE, 4, FAKE,
                              None, FAKE, None) == 0
    # pool n_slots H dk dv src dst n stream
    cbase = [FAKE, 64, 16, 128, 128, FAKE, FAKE, 3, None]
    for i, bad, st in [(0, None, -1), (5, None, -1), (6, None, -1), (3, 48, -2), (7, -1, -2),
                       (1, 0, -2), (2, 0, -2)]:
        args = list(cbase)
        args[i] = bad
        assert L.gla_state_copy(*args) == st, (i, bad)
    assert L.gla_state_copy(None, 0, 16, 128, 128, None, None, 0, None) == 0


def test_chunk_ckpt_validation():
    L = _lib.lib()
    a = _chunk_args()
    ws = L.gla_chunk_workspace_bytes(2, 10, 4, 128, 128, 64)

    def gla(interval, slots, stride, C=64):
        return L.gla_chunk_fwd_ckpt(a["q"], a["k"], a["v"], a["alpha"], a["cu"], a["B"], a["N"],
                                    a["H"], a["dk"], a["dv"], C, a["idt"], a["odt"], a["pool"],
                                    a["n_slots"], a["slots"], 0, interval, slots, stride, a["o"],
                                    FAKE, ws, None)
    assert gla(64, FAKE, -1) == _lib.GLA_ESHAPE
    assert gla(96, FAKE, 2) == _lib.GLA_ECHUNK          # not a multiple of the chunk
    assert gla(32, FAKE, 2) == _lib.GLA_ECHUNK          # shorter than the chunk
    assert gla(0, FAKE, 2) == _lib.GLA_ECHUNK
    assert gla(128, None, 2) == _lib.GLA_EPTR
    assert gla(128, FAKE, 1 << 30) == _lib.GLA_ESHAPE
    gargs = [a["q"], a["k"], a["v"], a["alpha"], FAKE, a["cu"], a["B"], a["N"], a["H"], a["dk"],
             a["dv"], 64, a["idt"], a["odt"], a["pool"], a["n_slots"], a["slots"], 0, 100, FAKE, 2,
             a["o"], FAKE, 1 << 40, None]
    assert L.gdn_chunk_fwd_ckpt(*gargs) == _lib.GLA_ECHUNK
    gargs[19] = None
    gargs[18] = 128
    assert L.gdn_chunk_fwd_ckpt(*gargs) == _lib.GLA_EPTR


def test_lin_attn_validation():
    L = _lib.lib()
    # q k v cu B N H dk dv C idt odt pool zpool n_slots slots flags eps o ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 64, 64, 64, 1, 1, FAKE, FAKE, 4, FAKE, 0, 1e-6, FAKE,
            None, 0, None]
    for i, bad, st in [(0, None, -1), (13, None, -1), (12, None, -1), (3, None, -1),
                       (7, 96, -2), (9, 48, -4), (10, 4, -3), (17, -1.0, -2),
                       (17, float("inf"), -2), (17, float("nan"), -2)]:
        args = list(base)
        args[i] = bad
        assert L.lin_attn_chunk_fwd(*args) == st, (i, bad)
    need = L.lin_attn_chunk_workspace_bytes(2, 10, 4, 128, 128, 64)
    assert need == L.gla_chunk_workspace_bytes(2, 10, 4, 128, 128, 64) > 0
    # the generic path with several d_v tiles per head keeps a copy of the
    # entry normalisers (2 sequences x 4 heads x dk floats); one tile needs none
    assert L.lin_attn_chunk_workspace_bytes(2, 10, 4, 32, 64, 32) == 2 * 4 * 32 * 4
    assert L.lin_attn_chunk_workspace_bytes(2, 10, 4, 64, 32, 32) == 0
    args = list(base)
    args[9] = 32
    assert L.lin_attn_chunk_fwd(*args) == _lib.GLA_EWORKSPACE
    args = list(base)
    args[7] = args[8] = 128
    assert L.lin_attn_chunk_fwd(*args) == _lib.GLA_EWORKSPACE
    # q k v R H dk dv idt odt pool zpool n_slots slots eps o stream
    dbase = [FAKE, FAKE, FAKE, 8, 16, 128, 128, 1, 1, FAKE, FAKE, 32, FAKE, 1e-6, FAKE, None]
    for i, bad, st in [(0, None, -1), (10, None, -1), (14, None, -1), (5, 8, -2), (13, -2.0, -2)]:
        args = list(dbase)
        args[i] = bad
        assert L.lin_attn_decode_step(*args) == st, (i, bad)
    assert L.lin_attn_decode_step(None, None, None, 0, 16, 128, 128, 1, 1, None, None, 4, None,
                                  1e-6, None, None) == 0


def test_gdn_prep_run_validation():
    L = _lib.lib()
    need = L.gdn_chunk_workspace_bytes(2, 10, 4, 128, 128, 64)
    # q k alpha beta cu B N H dk dv C idt ws wsb stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 4, 128, 128, 64, 1, FAKE, need, None]
    for i, bad, st in [(0, None, -1), (3, None, -1), (4, None, -1), (12, None, -5), (13, need - 1, -5),
                       (8, 96, -2), (10, 48, -4), (11, 3, -3), (5, 0, -2)]:
        args = list(base)
        args[i] = bad
        assert L.gdn_chunk_prep(*args) == st, (i, bad)
    assert L.gdn_chunk_prep(None, None, None, None, None, 0, 0, 4, 128, 128, 64, 1, None, 0, None) == 0
    a = _chunk_args()
    rargs = [a["q"], a["k"], a["v"], a["alpha"], FAKE, a["cu"], a["B"], a["N"], a["H"], a["dk"],
             a["dv"], a["C"], a["idt"], a["odt"], a["pool"], a["n_slots"], a["slots"], 0, a["o"],
             None, 0, None]
    assert L.gdn_chunk_run(*rargs) == _lib.GLA_EWORKSPACE
    rargs[4] = None
    assert L.gdn_chunk_run(*rargs) == _lib.GLA_EPTR


def test_slot_copy_validation():
    L = _lib.lib()
    # buf slot_bytes n_slots src dst n stream
    base = [FAKE, 12288, 8, FAKE, FAKE, 3, None]
    for i, bad, st in [(0, None, -1), (3, None, -1), (4, None, -1), (1, 0, -2), (1, 20, -2),
                       (2, 0, -2), (5, -1, -2), (0, FAKE + 4, -1)]:
        args = list(base)
        args[i] = bad
        assert L.gla_slot_copy(*args) == st, (i, bad)
    assert L.gla_slot_copy(None, 16, 0, None, None, 0, None) == 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/gla.h compiles as strict C99 and a C program links the library
    and gets validation results from it (no device is touched)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_gla.c"
    src.write_text(
        '#include "gla.h"\n#include <stdio.h>\n'
        "int main(void) {\n"
        "  int a = gla_chunk_fwd(0, 0, 0, 0, 0, 0, 0, 16, 128, 128, 64, GLA_BF16, GLA_BF16, 0, 1, 0,"
        " 0, 0, 0, 0, 0);\n"
        "  int b = gla_decode_step(0, 0, 0, 0, 4, 16, 128, 128, GLA_BF16, GLA_BF16, 0, 8, 0, 0, 0);\n"
        "  int c = gla_slot_copy(0, 20, 4, 0, 0, 1, 0);\n"
        '  printf("%d %d %d %s\\n", a, b, c, gla_version());\n'
        "  return 0;\n}\n")
    exe = tmp_path / "use_gla"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                    os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lgla_mi355x",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out[:3] == ["0", str(_lib.GLA_EPTR), str(_lib.GLA_ESHAPE)]
    assert out[3] == _lib.lib().gla_version().decode()
