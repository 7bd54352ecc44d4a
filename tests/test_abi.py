"""The C-ABI library on the CPU: it loads, exports what include/kd.h declares, and rejects bad input.

No compute call is made here (this container has no GPU); kd_init only gets as far as its
argument checks or the device query.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import workloads
from bandwidth_bound_transformer_amd import kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = kd.library()
    decl = declared_functions()
    assert decl == sorted(kd.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", kd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kd_[a-z_]+)$", out, flags=re.M))
    for name in decl:
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    src = '#include "kd.h"\nint main(void){ kd_config c; (void)c; return (int)sizeof(kd_weights) > 0 ? 0 : 1; }\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", "/dev/null"],
                         input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_struct_layout_matches_binding():
    """Every field of the ctypes structs sits where a C compiler puts it, given kd.h."""
    structs = {"kd_config": kd.kd_config, "kd_layer_weights": kd.kd_layer_weights, "kd_weights": kd.kd_weights}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "kd.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"kd_layout_{os.getpid()}")
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe],
                         input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    try:
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    finally:
        os.unlink(exe)
    want = {}
    for line in filter(None, out):
        sname, field, val = line.split()
        want[(sname, field)] = int(val)
    for name, cls in structs.items():
        assert ctypes.sizeof(cls) == want[(name, "size")], name
        for field, _ in cls._fields_:
            assert getattr(cls, field).offset == want[(name, field)], (name, field)


def test_header_constants_match_binding():
    """Every numeric KD_* constant of kd.h that the binding defines has the header's value, and the
    binding defines every number format and status code."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    consts = {n: int(v.rstrip("uU"), 0) for n, v in re.findall(r"#define\s+(KD_[A-Z0-9_]+)\s+\(?(-?(?:0x[0-9a-fA-F]+|\d+)[uU]?)\)?", text)}
    assert {"KD_DTYPE_F32", "KD_DTYPE_BF16", "KD_DTYPE_FP8_E4M3", "KD_DTYPE_INT8"} <= set(consts)
    for name, value in consts.items():
        if name.startswith(("KD_DTYPE_", "KD_STATUS_", "KD_ERR_")) or name == "KD_OK":
            assert hasattr(kd, name), name
        if hasattr(kd, name):
            assert getattr(kd, name) == value, (name, getattr(kd, name), value)


def test_strerror_covers_every_code():
    for code in range(-7, 1):
        assert kd.kd_strerror(code) and "unknown" not in kd.kd_strerror(code)
    assert "unknown" in kd.kd_strerror(-99)


def test_kv_layout():
    shape = workloads.get("2b").model
    cfg = kd.make_config(shape, batch=1, max_seq=1000)
    nbytes, strides = kd.kd_kv_layout(cfg)
    s_alloc = 1008  # max_seq + 7 rounded up to a multiple of 16
    assert strides == (2 * 4 * s_alloc * 128, 4 * s_alloc * 128, 4 * s_alloc * 128, s_alloc * 128, 128, 1)
    assert nbytes == 26 * 2 * 4 * s_alloc * 128 * 2
    tiny = workloads.get("tiny")
    n2, st2 = kd.kd_kv_layout(kd.make_config(tiny.model, 1, tiny.max_seq))
    assert n2 == 2 * 2 * 4 * 112 * 64 * 4 and st2[3] == 112 * 64


@pytest.mark.parametrize(
    "field,value",
    [("n_layers", 0), ("d_model", -1), ("n_kv_heads", 3), ("head_dim", 63), ("max_seq", 0), ("batch", 0), ("weight_dtype", 7), ("rope_base", 0.0)],
)
def test_bad_config_rejected(field, value):
    cfg = kd.make_config(workloads.get("tiny").model, 1, 96)
    setattr(cfg, field, value)
    with pytest.raises(kd.KDError) as e:
        kd.kd_kv_layout(cfg)
    assert e.value.code == kd.KD_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert kd.library().kd_init(ctypes.byref(cfg), None, ctypes.byref(h)) == kd.KD_ERR_INVALID_ARG
    assert h.value is None


def test_null_arguments_rejected():
    lib = kd.library()
    cfg = kd.make_config(workloads.get("tiny").model, 1, 96)
    h = ctypes.c_void_p()
    assert lib.kd_init(None, None, ctypes.byref(h)) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_init(ctypes.byref(cfg), None, None) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_init(ctypes.byref(cfg), None, ctypes.byref(h)) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_step(None, None, None, None, None, None) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_step_noalloc(None, None, None, None, None, None) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_stream_read(None, 1 << 20, None) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_generate(None, 4, None, None, None, None, None, None, None) == kd.KD_ERR_INVALID_ARG
    assert lib.kd_control(None, kd.KD_CTRL_CANCEL, 1) == kd.KD_ERR_INVALID_ARG
    bits = ctypes.c_uint32()
    assert lib.kd_device_status(None, ctypes.byref(bits), 0) == kd.KD_ERR_INVALID_ARG
    info = (ctypes.c_int64 * 8)()
    assert lib.kd_get_info(None, info) == kd.KD_ERR_INVALID_ARG
    lib.kd_destroy(None)  # accepted


def test_init_without_gpu_reports_no_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    wl = workloads.get("tiny")
    w = workloads.make_weights(wl.model, seed=0, workers=2)
    with pytest.raises(kd.KDError) as e:
        kd.kd_init(kd.make_config(wl.model, 1, wl.max_seq), w)
    assert e.value.code == kd.KD_ERR_NO_DEVICE
