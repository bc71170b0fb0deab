"""Build the C client check (tests/c/h2o_c_check) against include/h2o.h and the
in-tree libh2o.so, with gcc: a C program, not a HIP extension."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "h2o_c_check.c")
EXE = os.path.join(HERE, "h2o_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = EXE) -> list:
    return ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
            f"-I{os.path.join(ROOT, 'include')}", SRC, f"-L{os.path.join(ROOT, 'kv_cache_eviction_h2o_amd')}",
            "-lh2o", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
            "-Wl,-rpath,$ORIGIN/../../kv_cache_eviction_h2o_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", out]


def build(out: str = EXE) -> str:
    subprocess.run(command(out), check=True)
    return out


if __name__ == "__main__":
    print(build())
