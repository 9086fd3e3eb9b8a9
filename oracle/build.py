"""Build the oracle's C library (``oracle/rank_step.c`` -> ``liboracle_step.so``)
with gcc, in place:

    python -m oracle.build

IEEE double arithmetic only: no fused multiply-add contraction and no
fast-math, so the compiled oracle takes the same rounding steps as
``oracle.step``.
"""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Werror", "-ffp-contract=off",
         "-fno-fast-math"]


def build_c(src, out):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found")
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([cc] + FLAGS + [src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build():
    return build_c(os.path.join(HERE, "rank_step.c"), os.path.join(HERE, "liboracle_step.so"))


if __name__ == "__main__":
    print(build())
