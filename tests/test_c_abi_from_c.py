"""The C ABI used from C: include/bsa.h compiles as strict C99 and C++11, and a C
program linked against libbsa.so calls the host-only entry points (no device needed).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "block_sparse_tiled_amd")

PROGRAM = r"""
#include <stdio.h>
#include "bsa.h"
int main(void) {
  int ok = 1;
  ok &= bsa_abi_version() == 2;
  ok &= bsa_within_launch_limits(1, BSA_MAX_BATCH_HEADS, 100, 10) == 1;
  ok &= bsa_within_launch_limits(1, BSA_MAX_BATCH_HEADS + 1, 100, 10) == 0;
  ok &= bsa_within_launch_limits(1, 1, BSA_ROWS_LIMIT, 10) == 0;
  ok &= bsa_within_launch_limits(1, 1, 100, BSA_TILES_LIMIT) == 0;
  ok &= bsa_within_launch_limits(-1, 1, 100, 10) == 0;
  /* a 21 x 30 x 52 latent in 4 x 4 x 4 cubes: ceil-divided per axis */
  ok &= bsa_cube_num_tiles(21, 30, 52, 4, 4, 4) == 6 * 8 * 13;
  printf("%s|%s\n", bsa_status_string(BSA_OK), bsa_status_string(BSA_ERR_LAUNCH_LIMITS));
  return ok ? 0 : 1;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


@pytest.mark.parametrize("lang", ["c99", "c++11"])
def test_header_compiles_strictly(tmp_path, lang):
    cc = _compiler("gcc" if lang == "c99" else "g++")
    src = tmp_path / "h.c"
    src.write_text('#include "bsa.h"\nint main(void) { return bsa_abi_version() == 2 ? 0 : 1; }\n')
    cmd = [cc, f"-std={lang}", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{INC}"]
    cmd += (["-x", "c++"] if lang != "c99" else []) + ["-c", str(src), "-o", str(tmp_path / "h.o")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_c_program_calls_the_host_entry_points(tmp_path):
    cc = _compiler("gcc")
    if not os.path.exists(os.path.join(LIBDIR, "libbsa.so")):
        pytest.skip("libbsa.so is not built")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{INC}", str(src),
                          f"-L{LIBDIR}", "-lbsa", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    ok, limits = run.stdout.strip().split("|")
    assert ok == "ok" and limits.startswith("launch limits exceeded")
