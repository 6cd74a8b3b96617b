"""include/forge.h is a C header: a C99 translation unit that includes it and
takes the address of every declared entry point compiles warning-free, and
links against the built library."""
import os
import re
import shutil
import subprocess

import pytest

from weight_gradient_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "forge.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"FORGE_API\s+[\w\s\*]*?\b(forge_\w+)\s*\(", text)))


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_and_links_as_c(tmp_path, std):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = _declared()
    src = tmp_path / "use_forge.c"
    src.write_text(
        "#include \"forge.h\"\n#include <stdint.h>\n#include <stdio.h>\n"
        "typedef void (*fn_t)(void);\n"
        "int main(void) {\n"
        "  const fn_t fns[] = {\n"
        + "".join(f"    (fn_t)&{n},\n" for n in names)
        + "  };\n"
        "  forge_adamw_params p = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1, 0.0};\n"
        "  /* a clip request fails closed before any device work */\n"
        "  p.max_grad_norm = 1.0;\n"
        "  /* fake, 16-byte aligned, disjoint addresses: validation never dereferences them */\n"
        "  const void* X = (const void*)(uintptr_t)0x800000000ULL;\n"
        "  const void* dY = (const void*)(uintptr_t)0xA00000000ULL;\n"
        "  float* W = (float*)(uintptr_t)0x100000ULL;\n"
        "  float* m = (float*)(uintptr_t)0x200000000ULL;\n"
        "  float* v = (float*)(uintptr_t)0x400000000ULL;\n"
        "  forge_status s = forge_wgrad_adamw(X, dY, W, m, v, 8, 8, 8, &p, FORGE_TILE_DEFAULT, 0);\n"
        "  printf(\"%d %s %d\\n\", (int)s, forge_status_string(s), (int)(sizeof fns / sizeof fns[0]));\n"
        "  return 0;\n"
        "}\n")
    exe = tmp_path / "use_forge"
    lib_dir = os.path.dirname(_lib.library_path)
    r = subprocess.run([cc, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        "-L", lib_dir, "-lforge", f"-Wl,-rpath,{lib_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    status, *rest = out.stdout.split()
    assert int(status) == 6                       # FORGE_ERR_CLIP_NOT_FUSABLE
    assert int(rest[-1]) == len(names)


def test_binding_constants_match_the_header(tmp_path):
    """The Python binding's tile ids, element types, status codes and struct
    layouts are the header's: a C program prints the header's values and
    sizes, and they must equal the binding's."""
    import ctypes
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = (["FORGE_TILE_DEFAULT", "FORGE_TILE_256x128", "FORGE_TILE_128x128",
              "FORGE_TILE_256x256", "FORGE_TILE_PERSISTENT", "FORGE_F32", "FORGE_BF16",
              "FORGE_FP8_E4M3", "FORGE_FP8_E5M2"] + sorted(_lib.STATUS.values()))
    src = tmp_path / "consts.c"
    src.write_text(
        "#include \"forge.h\"\n#include <stdio.h>\n#include <stddef.h>\n"
        "int main(void) {\n"
        + "".join(f"  printf(\"{n} %d\\n\", (int){n});\n" for n in names)
        + "  printf(\"adamw_size %d\\n\", (int)sizeof(forge_adamw_params));\n"
          "  printf(\"adamw_step %d\\n\", (int)offsetof(forge_adamw_params, step));\n"
          "  printf(\"adamw_clip %d\\n\", (int)offsetof(forge_adamw_params, max_grad_norm));\n"
          "  printf(\"sgdm_size %d\\n\", (int)sizeof(forge_sgdm_params));\n"
          "  return 0;\n}\n")
    exe = tmp_path / "consts"
    subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = dict((k, int(v)) for k, v in (ln.split() for ln in out.splitlines()))
    for n in names[:9]:
        assert got[n] == getattr(_lib, n), n
    for code, n in _lib.STATUS.items():
        assert got[n] == code, n
    assert got["adamw_size"] == ctypes.sizeof(_lib.AdamWParams)
    assert got["adamw_step"] == _lib.AdamWParams.step.offset
    assert got["adamw_clip"] == _lib.AdamWParams.max_grad_norm.offset
    assert got["sgdm_size"] == ctypes.sizeof(_lib.SgdmParams)
