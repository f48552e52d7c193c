"""Host-side checks of the generated prefill instruction stream (no GPU): the hazard
checker is pinned on planted violations, the generated text keeps its register contract,
and the compiled gfx950 kernels (the generated prefill, and the backward with its
written-out matrix products) keep every wait-state distance."""
import os
import re
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "attention_forward_03_amd", "csrc")
sys.path.insert(0, HERE)
sys.path.insert(0, CSRC)
import gfx950_hazards as hz  # noqa: E402
import gen_prefill_r2 as gen  # noqa: E402


def _rules(text):
    ins, labels = hz.parse(text.strip().splitlines())
    return sorted({b[0] for b in hz.check(ins, labels)})


@pytest.mark.parametrize("listing,rule", [
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\nv_add_f32 v40, v3, v41",
     "mfma D -> non-mfma access"),
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\ns_nop 7\ns_nop 2\nv_add_f32 v40, v3, v41",
     "mfma D -> non-mfma access"),
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\n"
     "v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[36:39], v[16:31]", "mfma D -> mfma srcA/B"),
    ("v_mov_b32 v33, 0\nv_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]", "valu write -> mfma read"),
    ("v_exp_f32 v40, v41\nv_add_f32 v42, v40, v42", "trans -> read"),
    ("v_permlane32_swap_b32 v1, v2\nv_max_f32 v3, v1, v2", "permlane -> access"),
    ("s_add_u32 m0, s67, 4096\nbuffer_load_dwordx4 v204, s[88:91], 0 offen lds", "m0 write -> lds load"),
    # through a taken branch (the branch itself is one wait state)
    ("v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\ns_branch L1\ns_nop 7\ns_nop 7\nL1:\n"
     "v_add_f32 v40, v3, v41", "mfma D -> non-mfma access"),
])
def test_checker_flags_planted_violations(listing, rule):
    assert rule in _rules(listing)


@pytest.mark.parametrize("listing", [
    "v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\ns_nop 7\ns_nop 3\nv_add_f32 v40, v3, v41",
    "v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\n"
    "v_mfma_f32_32x32x16_bf16 v[0:15], v[40:43], v[36:39], v[0:15]",   # srcC chain is forwarded
    "v_mov_b32 v33, 0\ns_nop 1\nv_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]",
    "v_exp_f32 v40, v41\ns_nop 0\nv_add_f32 v42, v40, v42",
    "s_add_u32 m0, s67, 4096\ns_nop 0\nbuffer_load_dwordx4 v204, s[88:91], 0 offen lds",
])
def test_checker_passes_legal_distances(listing):
    assert _rules(listing) == []


def _stream(bf16, mode):
    return [ln for ln in gen.Gen(bf16, mode).build()]


NO_DEST = ("s_waitcnt", "s_barrier", "s_nop", "s_branch", "s_cbranch", "s_cmp", "global_store", "ds_write",
           "buffer_load")   # buffer_load ... lds: the first operand is the lane offset (read)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_generated_stream_register_contract(bf16, mode):
    lines = _stream(bf16, mode)
    labels = [ln[:-1] for ln in lines if ln.endswith(":")]
    assert len(labels) == len(set(labels)), "a label is defined twice"
    for ln in lines:
        if ln.endswith(":"):
            continue
        op, _, rest = ln.partition(" ")
        if op.startswith(("s_branch", "s_cbranch")):
            assert rest in labels, ln
            continue
        for m in re.finditer(r"offset:(\d+)", ln):
            assert int(m.group(1)) <= 65535, ln
        for r in hz.regs(rest):
            assert r[0] != "v" or r[1] < 256, ln
            assert r[0] != "a" or r[1] < 256, ln
        if op.startswith(NO_DEST) or op.startswith("v_cmp") or not rest:
            continue
        dst = hz.regs(rest.split(",")[0])
        for f, i in dst:
            if f == "v":
                assert gen.S_X <= i < gen.NVGPR, f"writes input or unlisted v{i}: {ln}"
            elif f == "a":
                assert i < 192, ln
            elif f == "s":
                assert gen.NSGPR_LO <= i < gen.NSGPR_HI, f"writes input or unlisted s{i}: {ln}"


def test_clobber_list_covers_the_stream_registers():
    clob = gen.clobbers()
    for i in range(gen.S_X, gen.NVGPR):
        assert f'"v{i}"' in clob
    for i in range(192):
        assert f'"a{i}"' in clob
    for i in range(gen.NSGPR_LO, gen.NSGPR_HI):
        assert f'"s{i}"' in clob
    assert '"vcc"' in clob and '"scc"' in clob


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


def _device_asm_cmd(src, out, extra_includes=()):
    """The library build's compile line for `src` (its common and per-file flags), for the
    device code only and as assembly: the checks below then read the code that ships."""
    sys.path.insert(0, ROOT)
    from attention_forward_03_amd import build
    cmd = [_hipcc(), *build.common_flags(), *build.SOURCE_FLAGS.get(src, []), "-I", CSRC]
    for inc in extra_includes:
        cmd += ["-I", str(inc)]
    return cmd + ["-x", "hip", "-S", "--offload-device-only", os.path.join(CSRC, src), "-o", str(out)]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_compiled_kernels_keep_the_wait_states(tmp_path):
    gen.main(str(tmp_path / "gen"))
    out = tmp_path / "prefill.s"
    cmd = _device_asm_cmd("prefill.hip", out, [tmp_path / "gen"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    funcs = hz.functions(out.read_text())
    names = [n for n in funcs if "fwd_r2_kernel" in n]
    assert len(names) == 6
    for n in names:
        ins, labels = hz.parse(funcs[n])
        bad = hz.check(ins, labels)
        assert not bad, (n, bad[:3])


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_compiled_backward_keeps_the_wait_states(tmp_path):
    out = tmp_path / "backward.s"
    cmd = _device_asm_cmd("backward.hip", out)
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    funcs = hz.functions(out.read_text())
    names = [n for n in funcs if "bwd_main_kernel" in n]
    assert len(names) == 8
    for n in names:
        ins, labels = hz.parse(funcs[n])
        assert sum(op.startswith("v_mfma") for op, _, _ in ins) > 0
        bad = hz.check(ins, labels)
        assert not bad, (n, bad[:3])
