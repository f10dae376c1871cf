"""The tile GEMM issues v_mfma_f32_16x16x32_bf16 as inline assembly (the
accumulators stay tied in AGPRs), so the compiler inserts no hazard padding
for it. These host tests compile the kernel source to gfx950 assembly with
the library's own flags and check the rules the kernel keeps instead:

  * every MFMA accumulates in place (destination == accumulator input);
  * an accumulator quad is not the target of two MFMAs closer than 8 apart;
  * after an MFMA, nothing reads or writes an AGPR until 24 wait states of
    padding (three s_nop 7) have been issued;
  * no VALU instruction writes an MFMA's source VGPRs within 4 wait states
    before that MFMA;
  * no scratch (spill) traffic anywhere in the kernel;
  * the float32 epilogue's 16-byte stores keep their streaming policy
    (also inline assembly), and no instruction overwrites the data
    registers of a store wider than 8 bytes in the next wait state.

Each kernel is checked whole, up to its end (it has several s_endpgm).
A change that breaks one of them would produce wrong results only on some
runs, if at all, so it is caught here, on the host, before any GPU run.
"""
import os
import re
import subprocess
import tempfile

import pytest

from local_shard_gemm_amd import build as lib_build

KERNEL = "_ZN7shardmm12_GLOBAL__N_121gemm_bf16_mfma_kernel"


@pytest.fixture(scope="module")
def kernels():
    try:
        hipcc = lib_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(lib_build.CSRC, "gemm_mfma.hip")
    flags = [f for f in lib_build.COMMON if f not in ("-fPIC", "-Wall")]
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "gemm_mfma.s")
        r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    found = {}
    # the whole function: a kernel has several s_endpgm (early exits)
    for m in re.finditer(r"^(" + KERNEL + r"\S+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.S | re.M):
        lines = [l.strip() for l in m.group(2).split("\n")]
        ins = []
        for l in lines:
            if l.endswith(":") or re.match(r"^\.LBB\S*:", l) or l.startswith("s_endpgm"):
                ins.append("<label>")  # a basic block starts (or the wave ends)
            elif l and not l.startswith((";", ".")):
                ins.append(l)
        found[m.group(1)] = ins
    # float32 / bfloat16 out, with / without GeLU, for the 256-row and the
    # 128-row tile
    assert len(found) == 8, sorted(found)
    return found


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", text):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _operands(ins):
    body = ins.split(None, 1)[1] if " " in ins else ""
    return [p.strip() for p in body.split(",")]


def _is_mfma(ins):
    return ins.startswith("v_mfma")


def test_every_mfma_accumulates_in_place(kernels):
    for name, ins in kernels.items():
        mfma = [i for i in ins if _is_mfma(i)]
        assert len(mfma) >= 128, name
        for i in mfma:
            ops = _operands(i)
            assert ops[0] == ops[3] and ops[0].startswith("a["), (name, i)


def test_accumulator_targets_at_least_8_mfmas_apart(kernels):
    """Within each basic block (across blocks the kernel's structure keeps
    them further apart: one MFMA per accumulator per K stage)."""
    for name, ins in kernels.items():
        last = {}
        n = 0
        for i in ins:
            if i == "<label>" or i.startswith(("s_branch", "s_cbranch")):
                last = {}
                continue
            if not _is_mfma(i):
                continue
            dst = _operands(i)[0]
            if dst in last:
                assert n - last[dst] >= 8, (name, i, n - last[dst])
            last[dst] = n
            n += 1


def test_agprs_untouched_until_padding_after_mfma(kernels):
    for name, ins in kernels.items():
        pending, nops = False, 0
        for i in ins:
            if _is_mfma(i):
                pending, nops = True, 0
                continue
            if i.startswith("s_nop 7"):
                nops += 1
                if nops >= 3:
                    pending = False
                continue
            if i == "<label>":
                continue
            nops = 0
            if pending:
                assert not any(r[0] == "a" for r in _regs(i)), (name, i)


def test_no_valu_write_of_mfma_sources_just_before(kernels):
    for name, ins in kernels.items():
        for k, i in enumerate(ins):
            if not _is_mfma(i):
                continue
            srcs = {r for r in _regs(",".join(_operands(i)[1:3])) if r[0] == "v"}
            waits = 0
            for j in range(k - 1, max(-1, k - 16), -1):
                if waits >= 4:
                    break
                p = ins[j]
                if p == "<label>":
                    continue
                op = p.split()[0]
                if op == "s_nop":
                    waits += int(p.split()[1]) + 1
                    continue
                if op.startswith("v_") and not _is_mfma(p):
                    assert not (_regs(_operands(p)[0]) & srcs), (name, p, i)
                waits += 1


def test_no_scratch_traffic(kernels):
    for name, ins in kernels.items():
        assert not [i for i in ins if i.startswith("scratch_")], name


def _fp32_kernels(kernels):
    # template arguments <OUT_BF16 = false, GELU>: float32 output
    return {n: ins for n, ins in kernels.items() if "ILb0E" in n}


def test_float32_tile_stores_stream(kernels):
    """The 256-row tile's float32 epilogue stores its 16-byte vectors with
    the streaming, system-scope policy (a plain store would leave the
    burst's dirty lines in the L2 in the way of the next wave of tiles);
    the 128-row tile's, whose partials a sum reads right after, plainly."""
    fp32 = _fp32_kernels(kernels)
    assert len(fp32) == 4
    for name, ins in fp32.items():
        st = [i for i in ins if i.startswith("global_store_dwordx4")]
        if "Li8E" in name:
            assert sum(1 for i in st if i.endswith("nt sc0 sc1")) >= 64, name  # 16x16 blocks per wave
        else:
            assert sum(1 for i in st if not i.endswith(("nt", "sc0", "sc1"))) >= 32, name
            assert not [i for i in st if i.endswith("nt sc0 sc1")], name


def test_store_data_not_overwritten_in_the_next_wait_state(kernels):
    """A store of more than 8 bytes reads its data registers after issue:
    the next instruction must not write them (one wait state, an s_nop or
    any other instruction, must come first)."""
    for name, ins in kernels.items():
        body = [i for i in ins if i != "<label>"]
        for k, i in enumerate(body[:-1]):
            if not i.startswith(("global_store_dwordx3", "global_store_dwordx4",
                                 "buffer_store_dwordx3", "buffer_store_dwordx4")):
                continue
            data = _regs(_operands(i)[1])
            nxt = body[k + 1]
            if nxt.startswith("s_") or not nxt.startswith("v_"):
                continue
            assert not (_regs(_operands(nxt)[0]) & data), (name, i, nxt)
