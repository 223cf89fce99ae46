"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``bole_oracle.c`` into ``liboracle.so`` next to it with gcc and OpenMP.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bole_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
# host-only sanitizer build (gcc, no GPU code): AddressSanitizer and UndefinedBehaviorSanitizer,
# every report fatal
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the oracle library and return its path (sanitize: the instrumented build,
    liboracle_san.so, which the loader takes when BOLE_ORACLE_LIB names it)."""
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = ["gcc", *(SAN_FLAGS if sanitize else ["-O2"]), "-std=c99", "-fPIC", "-shared",
           "-fopenmp", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
