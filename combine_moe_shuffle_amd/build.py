"""Build libmoe_shuffle.so (gfx950) in-tree with hipcc.

    python -m combine_moe_shuffle_amd.build

Every .hip file under csrc/ is compiled to an object for gfx950 only, then
linked into one shared library next to this file. The library exports only
the C ABI of include/moe_shuffle.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_shuffle.so")
FASTCALL_SRC = os.path.join(ROOT, "_build", "moe_fastcall.c")
CONSUMER_SRC = os.path.join(ROOT, "tests", "c_abi_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "c_abi_consumer")
OBJDIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # every fp32 operation is written out; no contraction into FMA
    "-ffp-contract=off",
    # hipcc makes packed-fp32 instructions on its own; keep them off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if r.stderr.strip() and verbose:
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_fastcall()
    build_consumer()
    return LIB


# CPython argument format of each ctypes argument type of _lib.SIGNATURES
_FORMAT = {"c_void_p": "K", "c_int": "i", "c_long": "L", "c_ulong": "K", "c_uint": "I",
           "c_float": "f"}
_CTYPE = {"K": "unsigned long long", "i": "int", "L": "long long", "I": "unsigned int",
          "f": "float"}


def fastcall_source() -> str:
    """C source of the _moe_fastcall extension: for every entry point of the
    ABI that returns a status, a wrapper that parses plain Python ints (device
    pointers as integers, 0 for NULL) and floats and calls it; plus
    last_error(). Generated from _lib.SIGNATURES, the table the ctypes binding
    uses, so the two cannot drift apart."""
    import ctypes

    sys.path.insert(0, ROOT)
    from combine_moe_shuffle_amd._lib import SIGNATURES

    out = ['#define PY_SSIZE_T_CLEAN', "#include <Python.h>", "#include <stdint.h>",
           '#include "moe_shuffle.h"', ""]
    methods = []
    for name, (res, args) in SIGNATURES.items():
        if res is not ctypes.c_int or not args:
            continue
        fmt = "".join(_FORMAT[a.__name__] for a in args)
        decl = " ".join(f"{_CTYPE[c]} a{i};" for i, c in enumerate(fmt))
        refs = ", ".join(f"&a{i}" for i in range(len(fmt)))
        call = ", ".join(f"(void *)(uintptr_t)a{i}" if c == "K" and args[i] is ctypes.c_void_p
                         else f"a{i}" for i, c in enumerate(fmt))
        out += [f"static PyObject *w_{name}(PyObject *self, PyObject *args) {{",
                f"  (void)self; {decl}",
                f'  if (!PyArg_ParseTuple(args, "{fmt}", {refs})) return NULL;',
                f"  return PyLong_FromLong((long){name}({call}));", "}", ""]
        methods.append(f'  {{"{name}", w_{name}, METH_VARARGS, NULL}},')
    out += ["static PyObject *w_last_error(PyObject *self, PyObject *args) {",
            "  (void)self; (void)args;",
            "  return PyUnicode_FromString(moe_last_error());", "}", "",
            "static PyMethodDef kMethods[] = {", *methods,
            '  {"last_error", w_last_error, METH_NOARGS, NULL},',
            "  {NULL, NULL, 0, NULL}};", "",
            "static struct PyModuleDef kModule = {",
            "    PyModuleDef_HEAD_INIT, \"_moe_fastcall\", NULL, -1, kMethods,",
            "    NULL, NULL, NULL, NULL};",
            "PyMODINIT_FUNC PyInit__moe_fastcall(void) { return PyModule_Create(&kModule); }", ""]
    return "\n".join(out)


def build_fastcall() -> str:
    """The CPython extension the bindings call through (one C call per launch
    instead of ctypes' per-argument conversion), linked to this library."""
    import sysconfig

    os.makedirs(os.path.dirname(FASTCALL_SRC), exist_ok=True)
    with open(FASTCALL_SRC, "w") as f:
        f.write(fastcall_source())
    target = os.path.join(HERE, "_moe_fastcall" + sysconfig.get_config_var("EXT_SUFFIX"))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", "-shared",
           "-fPIC", f"-I{sysconfig.get_paths()['include']}", f"-I{INCLUDE}", FASTCALL_SRC,
           "-o", target + ".tmp", f"-L{HERE}", "-lmoe_shuffle", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the fast-call extension failed:\n{r.stdout}\n{r.stderr}")
    os.replace(target + ".tmp", target)
    return target


def build_consumer() -> str:
    """The plain C consumer of the ABI used by the tests: gcc, the header, the
    HIP runtime API and this library (found through its rpath)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", f"-I{INCLUDE}", CONSUMER_SRC, "-o", CONSUMER + ".tmp",
           f"-L{HERE}", "-lmoe_shuffle", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../combine_moe_shuffle_amd", f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C consumer failed:\n{r.stdout}\n{r.stderr}")
    os.replace(CONSUMER + ".tmp", CONSUMER)
    return CONSUMER


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
