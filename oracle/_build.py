"""Build step for the CPU oracle (test infrastructure only).

Compiles ``ssm_oracle.c`` with the host C compiler at -O2 and without
fast-math, into ``liboracle.so`` beside this file.  ``build_mutant(k, dir)``
compiles the deliberately wrong variant k used by the pin meta-test.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math"]


def _cc():
    return os.environ.get("CC", "gcc")


def build(out=LIB, mutant=0):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_cc(), *CFLAGS, "-DORACLE_MUTANT=%d" % mutant, SRC, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_mutant(k, directory):
    return build(os.path.join(directory, "liboracle_m%d.so" % k), mutant=k)


if __name__ == "__main__":
    print(build())
