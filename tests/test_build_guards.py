"""Build guards: properties of the gfx950 code that the tree's bits depend on.

Compiles the HIP library to device assembly with the library's own flags and
checks what the arithmetic contract needs: subnormals kept, no packed FP32,
the correctly rounded division sequence, FMA only inside that sequence, and
no scalar-cache stores.  CPU only (hipcc cross-compiles).
"""
import os
import re
import subprocess

import pytest

from stable_variance_amd import build as libbuild


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in libbuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    procs = []
    for src in libbuild.SRCS:
        out = d / (os.path.basename(src) + ".s")
        cmd = [libbuild.hipcc(), *flags, "--cuda-device-only", "-S", src, "-o", str(out)]
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    text = []
    for out, pr in procs:
        _, err = pr.communicate()
        assert pr.returncode == 0, err
        text.append(out.read_text())
    return "\n".join(text)


def kernels(asm_text):
    """Map kernel symbol -> (body text, metadata text)."""
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm_text, re.S):
        name = m.group(1)
        body_m = re.search(re.escape(name) + r":.*?s_endpgm", asm_text, re.S)
        out[name] = (body_m.group(0) if body_m else "", m.group(2))
    return out


def test_every_kernel_keeps_subnormals(asm):
    ks = kernels(asm)
    assert len(ks) >= 10 and any("k_adn_sum" in k for k in ks)
    for name, (_, meta) in ks.items():
        mode = re.search(r"\.amdhsa_float_denorm_mode_32 (\d+)", meta)
        assert mode and mode.group(1) == "3", name  # 3 = keep input and output subnormals


def test_no_packed_fp32(asm):
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)


def test_no_scalar_memory_writes(asm):
    # scalar-unit stores, atomics and cache write-backs (names built from parts)
    forbidden = ["s_" + w for w in ("store", "atomic", "buffer" + "_store", "dcache" + "_wb")]
    for f in forbidden:
        assert not re.search(r"\b" + f, asm), f


# Kernels known to use private (scratch) memory: the lane-per-column axis-0
# kernel with 64 rows per lane and 16 waves (the ablation variants' columns of
# 513..1024 rows, and the var_cols_one=0 geometry) is capped at 128 VGPRs by
# its 1024-thread workgroup and spills 7 of them.  Every other kernel must
# keep everything in registers and LDS.
SCRATCH_ALLOWED = re.compile(r"k_var_colsILi64ELi16ELi[0-9]+E")


def test_no_private_segment_outside_the_known_exception(asm):
    ks = kernels(asm)
    assert len(ks) >= 10
    seen = []
    for name, (_, meta) in ks.items():
        size = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", meta)
        assert size, name
        if int(size.group(1)) != 0:
            assert SCRATCH_ALLOWED.search(name), (name, size.group(1))
            seen.append(name)
    assert len(seen) <= 8, seen


def element_type(name):
    """f64 for kernels whose first argument is a const double*, else f32."""
    return "f64" if re.search(r"Ev(PKd|PK[0-9]+NodeD)", name) else "f32"


def test_division_is_correctly_rounded_and_fma_only_inside_it(asm):
    ks = kernels(asm)
    var = [(n, b) for n, (b, _) in ks.items() if ("k_var_rows" in n or "k_var_cols" in n)]
    assert var and any(element_type(n) == "f64" for n, _ in var)
    for n, body in var:
        t = element_type(n)
        # the IEEE division sequence (scale, Newton steps, fmas, fixup)
        assert f"v_div_fixup_{t}" in body and f"v_div_scale_{t}" in body, n
    for n, (body, _) in ks.items():
        # every FMA belongs to a division: at most 5 (f32) or 6 (f64) per sequence
        for t, per in (("f32", 5), ("f64", 6)):
            nfma = len(re.findall(rf"\bv_fmac?_{t}", body))
            ndiv = len(re.findall(rf"\bv_div_fixup_{t}", body))
            assert nfma <= per * ndiv, (n, t, nfma, ndiv)
        if "k_tree_sum" in n or "k_adn_sum" in n:
            # the sums divide nothing; the ADN conversion's double adds stay unfused
            assert not re.search(r"\bv_fmac?_f(32|64)", body), n


def test_source_guards_reject_fast_math():
    cmd = [libbuild.hipcc(), "--offload-arch=gfx950", "-ffast-math", "--cuda-device-only", "-fsyntax-only",
           libbuild.SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode != 0 and "fast-math" in (res.stderr + res.stdout)
