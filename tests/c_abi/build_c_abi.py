"""Compile tests/c_abi/abi_main.c against the built libwanattn.so, the oracle
and the seeded generator (run by __graft_entry__.build(); the binary is run
by tests/test_gpu_c_abi.py)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_main")


def build() -> str:
    pkg = os.path.join(ROOT, "video_diffusion_transformer_wanattn_amd")
    dirs = [pkg, os.path.join(ROOT, "oracle"), os.path.join(pkg, "seeded")]
    rpath = ":".join("$ORIGIN/" + os.path.relpath(d, HERE) for d in dirs)
    tmp = BIN + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "abi_main.c"), "-o", tmp]
    cmd += ["-L" + d for d in dirs] + ["-lwanattn", "-loracle", "-lseeded", "-L/opt/rocm/lib", "-lamdhip64",
                                       "-lm", "-lpthread", "-Wl,-rpath," + rpath + ":/opt/rocm/lib"]
    subprocess.check_call(cmd)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
