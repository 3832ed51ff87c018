"""Build step for the CPU oracle (test infrastructure).

Compiles ``mla_oracle.c`` with gcc into ``oracle/libmla_oracle.so``. A mutant build
(``mutant=k``) plants the k-th known mistake (see ORACLE_MUTANT in the C source) into a
separate library so that the tests can show each pin catches it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mla_oracle.c")
LIB = os.path.join(HERE, "libmla_oracle.so")


def build(out=LIB, mutant=0, quiet=True):
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-DORACLE_MUTANT=%d" % int(mutant), SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
