"""Compile the C consumer of the library (tests/c_api/abi_consumer.c).

It includes only include/flash_attn.h and the HIP runtime's C API, links
libflashattn.so and the oracle's liboracle.so through $ORIGIN-relative rpaths
(so it runs wherever the tree is copied), and is built next to its source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.c")
EXE = os.path.join(HERE, "abi_consumer")


def command(out: str = EXE) -> list:
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), SRC, "-o", out,
            "-L", os.path.join(ROOT, "exact_attention_77_amd"), "-lflashattn",
            "-L", os.path.join(ROOT, "oracle"), "-loracle",
            "-L/opt/rocm/lib", "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../exact_attention_77_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
            "-Wl,-rpath,/opt/rocm/lib"]


def build(out: str = EXE) -> str:
    subprocess.run(command(out), check=True)
    return out


if __name__ == "__main__":
    print(build())
