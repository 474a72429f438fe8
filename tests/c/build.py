"""Build the plain C client of the library (gcc, no hipcc): tests/c/abi_client."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "abi_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    libdir = os.path.join(ROOT, "gradient_aggregation_amd")
    tmp = EXE + ".tmp%d" % os.getpid()
    # hip_runtime_api.h needs the platform named when a plain C compiler reads it
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                           os.path.join(HERE, "abi_client.c"), "-o", tmp, "-L", libdir, "-lgradagg",
                           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + libdir,
                           "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
