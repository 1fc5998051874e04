"""Compile the CPU oracle (plain C, fp64, OpenMP) into oracle/libpack3d_oracle.so.

Test infrastructure: the oracle is the checker, not part of the product path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pack3d_oracle.c")
LIB = os.path.join(HERE, "libpack3d_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, for
# a CPU pass over the pins (loaded with libasan preloaded into the process)
LIB_SAN = os.path.join(HERE, "libpack3d_oracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized() -> str:
    """The oracle with ASan and UBSan (host code only; gcc, no GPU code)."""
    tmp = LIB_SAN + ".tmp"
    cmd = ["gcc", *SAN_FLAGS, "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_SAN)
    return LIB_SAN


def sanitizer_preload() -> str:
    """Runtime libraries a process must preload to load LIB_SAN."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
        libs.append(os.path.realpath(path))
    return " ".join(libs)


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        print(build(force="--lazy" not in sys.argv))
