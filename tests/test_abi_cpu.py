"""The C-ABI library loads on a host without a GPU and exports every entry
point its headers declare; host-only argument checks answer without touching
the device."""
import ctypes
import os
import re

import pytest

from block_draft_model_amd import kdraft

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in ("kdraft.h", "kdraft_debug.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kdraft.LIB_PATH):
        pytest.fail("libkdraft.so is not built (python -m block_draft_model_amd.build)")
    return kdraft.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    missing = [n for n in names if not hasattr(lib, n)]
    assert missing == []
    assert set(names) == set(kdraft.EXPORTS)


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert kdraft.status_string(s) not in ("", "unknown status")
    assert kdraft.status_string(-99) == "unknown status"


def test_default_config_is_the_model_card_shape(lib):
    c = kdraft.default_config()
    assert (c.hidden, c.heads, c.head_dim, c.ffn, c.layers, c.block, c.rank, c.taps) == \
        (2560, 20, 128, 6144, 4, 4, 256, 3)
    assert (c.window, c.draft_vocab, c.full_vocab) == (2048, 60614, 131072)
    assert abs(c.rope_theta - 10000.0) < 1e-3 and abs(c.rms_eps - 1e-6) < 1e-12


def test_host_side_argument_errors(lib):
    h = ctypes.c_void_p()
    assert lib.kd_create(None, None, ctypes.byref(h)) == kdraft.KD_ERR_ARG
    assert lib.kd_create(ctypes.byref(kdraft.default_config()), None, None) == kdraft.KD_ERR_ARG
    for field, val in (("hidden", 4096), ("heads", 32), ("layers", 5), ("rank", 128)):
        cfg = kdraft.default_config(**{field: val})
        assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_UNSUPPORTED
    cfg = kdraft.default_config(head_quant=99)
    assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_UNSUPPORTED
    cfg = kdraft.default_config(body_quant=99)
    assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_UNSUPPORTED
    # every body and head format passes the format check (the window check
    # below still rejects this config before any device work)
    for body in (kdraft.KD_QUANT_FP8_BLOCK64, kdraft.KD_QUANT_BF16, kdraft.KD_QUANT_NVFP4):
        for head in (kdraft.KD_QUANT_NVFP4, kdraft.KD_QUANT_BF16, kdraft.KD_QUANT_FP8_BLOCK64):
            cfg = kdraft.default_config(body_quant=body, head_quant=head, window=0)
            assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_ARG
    cfg = kdraft.default_config(window=0)
    assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_ARG
    cfg = kdraft.default_config(max_streams=1 << 30)
    assert lib.kd_create(ctypes.byref(cfg), None, ctypes.byref(h)) == kdraft.KD_ERR_OOM
    assert lib.kd_round(None, 1, None, None, None, None, None, None, None) == kdraft.KD_ERR_ARG
    assert lib.kd_ingest(None, 1, 1, None, None, None, None) == kdraft.KD_ERR_ARG
    assert lib.kd_load_weights(None, None) == kdraft.KD_ERR_ARG
    assert lib.kd_last_error(None) == b""
    lib.kd_destroy(None)


def test_copy_guard_follows_the_reference(lib):
    """The host-side pause guard against the reference on random outcomes."""
    import numpy as np
    from oracle.copy_draft import PauseGuard
    rng = np.random.default_rng(3)
    for trial in range(20):
        window = int(rng.integers(1, 30))
        pause = int(rng.integers(0, 50))
        ref, got = PauseGuard(window, 0.5, pause), kdraft.CopyGuard(window, 0.5, pause)
        for step in range(400):
            if ref.armed():
                p = int(rng.integers(1, 9))
                a = int(rng.integers(0, p + 1)) if rng.random() < 0.7 else 0
                ref.record(p, a)
                got.record(p, a)
            adv = int(rng.integers(1, 5))
            ref.advance(adv)
            got.advance(adv)
            assert ref.armed() == got.armed(), (trial, step)


def test_copy_draft_argument_errors(lib):
    assert lib.kd_copy_draft(None, 1, None, 0, None, None, 0, 8, None, None) == kdraft.KD_ERR_ARG


def test_ctypes_structs_match_the_c_header(tmp_path):
    """The binding's ctypes structures have the header's sizes and field
    offsets (compiled with the host C compiler from include/kdraft.h)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    checks = {
        "kd_kv": (kdraft.KdKV, ["k", "v", "stride_stream", "capacity", "format", "k_so", "v_so"]),
        "kd_weights": (kdraft.KdWeights, ["fuse", "mask_row", "layer", "final_norm", "head_g",
                                          "embed_table", "kv_rot_signs", "head_bf16", "head_fp8"]),
        "kd_config": (kdraft.KdConfig, ["hidden", "max_streams", "rope_theta", "head_quant"]),
        "kd_copy_guard": (kdraft.KdCopyGuard, ["window", "min_accept", "proposed", "accepted"]),
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kdraft.h"', "int main(void) {"]
    for name, (_, fields) in checks.items():
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({name}));')
        for f in fields:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for name, (cls, fields) in checks.items():
        assert got[(name, "sizeof")] == ctypes.sizeof(cls), name
        for f in fields:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)
