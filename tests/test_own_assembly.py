"""Checks on the gfx950 assembly of this library's own kernels (CPU only).

  * no scratch memory: the register file of the interpreter and every value
    stays in VGPRs;
  * binary32 data paths contain no fused multiply-add of any form (v_fma*,
    v_fmac*, v_fma_mix*, v_mad*, v_mac*) and no packed binary32 instruction;
  * every kernel keeps FP32 and FP16/FP64 denormals (denorm mode 3, the
    default execution mode the Silk "AMDGPU Backend" page lists under "Code
    Object Format");
  * the linear kernels move data with 128-bit global loads and stores, the
    tiled kernels go through LDS;
  * the linear interpreter loads binary32 inputs straight into LDS and waits
    for those loads (vmcnt 0) before it reads LDS.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
FILES = ["kernels_linear", "kernels_interp", "kernels_rows", "kernels_tiled", "kernels_gather"]


def _asm(name):
    path = os.path.join(BUILD, name + ".s")
    src = os.path.join(ROOT, "elementwise_tensor_commands_amd", "csrc", name + ".hip")
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "ecmd_build", os.path.join(ROOT, "elementwise_tensor_commands_amd", "build.py"))
        B = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(B)
        os.makedirs(BUILD, exist_ok=True)
        subprocess.run([B.HIPCC, *B.FLAGS, "-x", "hip", "--offload-device-only", "-S", src, "-o", path],
                       check=True, capture_output=True)
    return open(path).read()


def _kernels(text):
    """name -> (body text, descriptor directives text)"""
    out = {}
    for m in re.finditer(r"^(_Z\w+):\s*(?:;.*)?$", text, re.M):
        name = m.group(1)
        end = text.find("s_endpgm", m.end())
        body = text[m.end(): end]
        d0 = text.find(".amdhsa_kernel " + name)
        d1 = text.find(".end_amdhsa_kernel", d0)
        out[name] = (body, text[d0:d1])
    return out


@pytest.fixture(scope="module", params=FILES)
def kernels(request):
    k = _kernels(_asm(request.param))
    assert k, request.param
    return request.param, k


FMA = re.compile(r"\b(v_fma\w*|v_fmac\w*|v_mad_f\w*|v_mad_mix\w*|v_mac_f\w*|v_pk_fma\w*|v_pk_add_f32|v_pk_mul_f32)\b(.*)")


def test_no_scratch(kernels):
    fname, ks = kernels
    for name, (body, desc) in ks.items():
        assert "scratch_" not in body, name
        m = re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", desc)
        assert m and int(m.group(1)) == 0, name


def test_no_fused_or_packed_fp32(kernels):
    fname, ks = kernels
    for name, (body, _) in ks.items():
        for m in FMA.finditer(body):
            op, rest = m.group(1), m.group(2)
            # The only tolerated form: the float-reciprocal step of 64-bit
            # integer division in index arithmetic (scale by 2^32 = 0x4f800000).
            ok = op.startswith(("v_fmac_f32", "v_fmamk_f32", "v_fmaak_f32")) and \
                ("0x4f800000" in rest or "0xcf800000" in rest)
            assert ok, "%s: %s%s" % (name, op, rest)


def test_denormals_kept(kernels):
    fname, ks = kernels
    for name, (_, desc) in ks.items():
        assert re.search(r"\.amdhsa_float_denorm_mode_32\s+3", desc), name
        assert re.search(r"\.amdhsa_float_denorm_mode_16_64\s+3", desc), name


def test_linear_uses_128bit_accesses():
    ks = _kernels(_asm("kernels_linear"))
    vec = [n for n in ks if "Lb1E" in n]      # VEC = true instantiations
    assert vec
    for name in vec:
        body = ks[name][0]
        # every vector-path kernel moves data in 64- or 128-bit accesses (binary16
        # groups of 4 elements are 8 bytes); all-32-bit Programs use 128-bit only
        has_loads = "kProgFill" not in name                    # a fill only stores
        assert (not has_loads or re.search(r"global_load_dwordx[24]", body)) and \
            re.search(r"global_store_dwordx[24]", body), name
        if any(p in name for p in ("kProgAddF32", "kProgIntFused", "kProgAxpbyF32", "kProgCopyF32")):
            assert "global_load_dwordx4" in body and "global_store_dwordx4" in body, name


def test_tiled_uses_lds():
    ks = _kernels(_asm("kernels_tiled"))
    for name, (body, _) in ks.items():
        assert "ds_write" in body and "ds_read" in body and "s_barrier" in body, name


def test_interp_waits_for_lds_dma():
    """Direct global-to-LDS loads are not ordered before later LDS reads by the
    compiler: the interpreter waits for them explicitly.  In program order, no
    ds_read may follow a global_load_lds without an s_waitcnt vmcnt(0) between."""
    ks = _kernels(_asm("kernels_interp"))
    assert len(ks) == 34, list(ks)     # linear and rows x K = 1, 2, 4 x nontemporal loads x stores; 5 tiled shapes x 2
    for name, (body, _) in ks.items():
        assert "global_load_lds_dwordx4" in body and "ds_read_b128" in body, name
        pending = False
        for line in body.splitlines():
            t = line.strip()
            if t.startswith("global_load_lds"):
                pending = True
            elif t.startswith("s_waitcnt") and "vmcnt(0)" in t:
                pending = False
            elif t.startswith("ds_read"):
                assert not pending, "%s: LDS read before the LDS loads were waited for" % name
