"""Builds tests/c_abi/closed_form: a plain C program (gcc, no HIP compiler)
that links libqknorm.so and the HIP runtime and calls the C ABI directly."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "closed_form.c")
BIN = os.path.join(HERE, "closed_form")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC,
           f"-L{os.path.join(ROOT, 'qk_norm_amd')}", "-lqknorm", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../qk_norm_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", BIN + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
