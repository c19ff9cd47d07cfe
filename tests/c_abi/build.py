"""Compile tests/c_abi/c_abi_check (host-only C++ against include/thrift.h,
the HIP runtime and the in-tree libthrift.so; g++, no device code)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "c_abi_check")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    lib_dir = os.path.join(ROOT, "fp16_long_context_amd")
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{os.path.join(ROOT, 'include')}", "-o", EXE + ".tmp", os.path.join(HERE, "c_abi_check.cpp"),
           f"-L{lib_dir}", "-lthrift", "-Wl,-rpath,$ORIGIN/../../fp16_long_context_amd",
           f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
