"""Compile tests/c/c_caller.c (plain C, gcc) against the library and the
oracle, in place.  Test infrastructure; run by __graft_entry__.build() and,
when the binary is missing, by the CPU test."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "c_caller.c")
BIN = os.path.join(HERE, "c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", BIN,
           "-L", os.path.join(ROOT, "delta_rule_linear_amd"), "-ldeltarule",
           "-L", os.path.join(ROOT, "oracle"), "-ldr_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../delta_rule_linear_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build())
