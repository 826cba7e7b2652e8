"""Build the oracle's shared library with the host C compiler.

Test infrastructure only: the oracle is loaded by the test suite, the smoke
check and the benchmark's CPU-baseline leg, never by the GPU library.  Plain
-O2, no fast-math, no explicit SIMD, so that every floating-point operation is
the one written in paged_attention_ref.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "paged_attention_ref.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile `src` (the oracle source, or a copy of it) into the shared library `lib`."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", src, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
