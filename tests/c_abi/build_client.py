"""Build the plain C client of libgsa (test infrastructure): host C code only,
linked against the in-tree libgsa.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "gsa_c_client.c")
BIN = os.path.join(HERE, "gsa_c_client")


def build() -> str:
    pkg = os.path.join(ROOT, "slot_memory_sequence_amd")
    tmp = BIN + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", SRC, "-L" + pkg, "-lgsa", "-L/opt/rocm/lib",
                           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../slot_memory_sequence_amd",
                           "-Wl,-rpath,/opt/rocm/lib", "-o", tmp])
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
