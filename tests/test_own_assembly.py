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
  * the interpreters load inputs straight into LDS and wait for those loads
    (vmcnt 0) before they read LDS.
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
    csrc = os.path.join(ROOT, "elementwise_tensor_commands_amd", "csrc")
    src = os.path.join(csrc, name + ".hip")
    newest = max(os.path.getmtime(os.path.join(csrc, f)) for f in os.listdir(csrc) if f.endswith(".h"))
    if not os.path.exists(path) or os.path.getmtime(path) < max(os.path.getmtime(src), newest):
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

    def flags(name):
        """(VEC, NTL, NTS) of an instance: k_linear<EV, E, G, VEC, NTL, NTS> or the
        lean k_linear1<EV, E, G, NTL, NTS> (vector accesses only)."""
        f = [b == "1" for b in re.findall(r"Lb([01])E", name)]
        return (True, *f) if "k_linear1I" in name else tuple(f)

    vec = [n for n in ks if flags(n)[0]]                       # VEC = true instantiations
    assert vec and any("k_linear1I" in n for n in vec)
    for name in vec:
        body = ks[name][0]
        nts = flags(name)[2]
        # every vector-path kernel moves data in 64- or 128-bit accesses (binary16
        # groups of 4 elements are 8 bytes); all-32-bit Programs use 128-bit only.
        # Streaming stores go through buffer stores with the nt and sc1 bits.
        store = r"buffer_store_dwordx([24]) v\[\d+:\d+\], v\d+, s\[\d+:\d+\], 0 offen nt sc1" if nts else \
            r"global_store_dwordx([24])"
        has_loads = "kProgFill" not in name                    # a fill only stores
        assert (not has_loads or re.search(r"global_load_dwordx[24]", body)) and re.search(store, body), name
        if any(p in name for p in ("kProgAddF32", "kProgIntFused", "kProgAxpbyF32", "kProgCopyF32")):
            assert "global_load_dwordx4" in body and "4" in re.search(store, body).group(1), name


def test_tiled_uses_lds():
    ks = _kernels(_asm("kernels_tiled"))
    for name, (body, _) in ks.items():
        assert "ds_write" in body and "ds_read" in body and "s_barrier" in body, name


def _blocks(text):
    """Basic blocks of one kernel's assembly: [(label, lines, successors)]."""
    blocks, cur, label = [], [], None
    for line in text.splitlines():
        t = line.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":") and not t.startswith("."):
            continue
        if t.endswith(":"):
            blocks.append([label, cur])
            cur, label = [], t[:-1]
            continue
        cur.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append([label, cur])
            cur, label = [], None
    blocks.append([label, cur])
    out = []
    index = {b[0]: i for i, b in enumerate(blocks) if b[0]}
    for i, (label, lines) in enumerate(blocks):
        succ = []
        last = lines[-1] if lines else ""
        if last.startswith(("s_branch", "s_cbranch")):
            succ.append(index[last.split()[1]])
        if not last.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            succ.append(i + 1)
        out.append((label, lines, succ))
    return out


def test_interp_waits_for_lds_dma():
    """Direct global-to-LDS loads are not ordered before later LDS reads by the
    compiler: the interpreters wait for them explicitly.  On every path of the
    control-flow graph, no ds_read follows a global_load_lds without an
    s_waitcnt vmcnt(0) between."""
    text = _asm("kernels_interp")
    ks = _kernels(text)
    # linear x K = 1, 2, 4 x nontemporal loads x stores; rows the same x 3 row modes; 5 tiled shapes x 2;
    # gather K x 3 modes
    assert len(ks) == 12 + 36 + 10 + 9, list(ks)
    for name in ks:
        start = re.search(r"^%s:.*$" % name, text, re.M).end()
        blocks = _blocks(text[start: text.find(".Lfunc_end", start)])
        body = "\n".join("\n".join(b[1]) for b in blocks)
        if "k_gather_interp" in name:     # one word (binary32) or one 2-byte value per lane into LDS
            assert "global_load_lds_dword " in body and "global_load_lds_ushort" in body, name
        else:
            assert "global_load_lds_dwordx4" in body, name
        assert "ds_read_b128" in body, name
        bad = _read_before_wait(blocks)
        assert bad is None, "%s: LDS read before the LDS loads were waited for: %s" % (name, bad)


def _read_before_wait(blocks):
    """Forward data flow of "a direct load may be outstanding" to a fixed
    point; the first ds_read reached in that state, or None."""
    pend_in = [False] * len(blocks)
    changed = True
    while changed:
        changed = False
        for i, (_, lines, succ) in enumerate(blocks):
            pending = pend_in[i]
            for t in lines:
                if t.startswith("global_load_lds"):
                    pending = True
                elif t.startswith("s_waitcnt") and "vmcnt(0)" in t:
                    pending = False
                elif t.startswith("ds_read") and pending:
                    return t
            for j in succ:
                if pending and not pend_in[j]:
                    pend_in[j] = True
                    changed = True
    return None


def test_wait_check_follows_branches():
    """The check sees a read reached through a branch taken from a block laid
    out after it, and accepts the same code with the wait on that path."""
    bad = """
\ts_branch .LBB0_2
.LBB0_1:
\tds_read_b128 v[0:3], v4
\ts_endpgm
.LBB0_2:
\tglobal_load_lds_dword v[6:7], off
\ts_cbranch_scc1 .LBB0_1
\ts_waitcnt vmcnt(0)
\ts_branch .LBB0_1
"""
    assert _read_before_wait(_blocks(bad)) == "ds_read_b128 v[0:3], v4"
    good = bad.replace("\ts_cbranch_scc1 .LBB0_1\n", "\ts_waitcnt vmcnt(0)\n\ts_cbranch_scc1 .LBB0_1\n")
    assert _read_before_wait(_blocks(good)) is None


def test_linear_input_loads_ordered():
    """The lean linear kernels issue an input's loads only once the previous
    input's have returned where every input access is 16 bytes (the axpby, the
    int32 Command), and the first input's alone otherwise (the mixed-precision
    Command, binary16 inputs read 8 bytes a work-item): in the assembly, a
    vmcnt(0) wait between the loads as the order asks."""
    ks = _kernels(_asm("kernels_linear"))
    for prog, expect in (("kProgAxpbyF32", "LWL"), ("kProgIntFused", "LWLWL"), ("kProgMixedTwoOut", "LWLL")):
        names = [n for n in ks if "k_linear1I" in n and prog + "E" in n and "Li4ELi4ELb1ELb1ELin1E" in n]
        assert len(names) == 1, (prog, names)
        seq = ""
        for line in ks[names[0]][0].splitlines():
            op = line.strip()
            if re.match(r"global_load_dwordx[24]\b", op):
                seq += "L"
            elif re.match(r"s_waitcnt vmcnt\(0\)", op):
                seq += "W"
        assert seq.startswith(expect), (prog, seq)
