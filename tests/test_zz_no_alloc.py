"""GPU: the allocation-free decode entry point (attn_decode_paged_noalloc, through the C
ABI) against the entry point with a caller-supplied workspace (attn_decode_paged). Both
run the same kernels, so O and LSE must agree bit for bit; each is also held to the
oracle's tolerance. Two calls in a row share the library's scratch array, the second on a
smaller input, so a partial left over from the first call that the second read would show."""
import numpy as np
import pytest
import torch

import attention_forward_03_amd as attn
import workloads
from gpu_support import Guarded, compare, decode_kind, decode_tensors, note, oracle_decode, widen

pytestmark = pytest.mark.gpu


def _both(case):
    t = decode_tensors(case)
    S, hq, _ = t["q"].shape
    outs = []
    for noalloc in (False, True):
        go, gl = Guarded(t["q"].shape, t["q"].dtype), Guarded((S, hq), torch.float32)
        kw = dict(k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), out=go.t, lse_out=gl.t)
        if noalloc:
            attn.decode_paged_noalloc(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                                      case.max_seq_len, **kw)
        else:
            attn.decode_paged(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                              case.max_seq_len, return_lse=True, **kw)
        torch.cuda.synchronize()
        go.check_guards("O")
        gl.check_guards("LSE")
        outs.append((go.t.cpu(), gl.t.cpu()))
    return outs


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_noalloc_decode_equals_workspace_decode(kv):
    cases = [
        workloads.make_decode(lengths=[5000, 1, 2048, 3001, 700, 4099], num_q_heads=8, num_kv_heads=2,
                              head_dim=128, kv_dtype=kv, seed=101),
        # second call: fewer sequences, shorter, another head layout
        workloads.make_decode(lengths=[17, 300], num_q_heads=4, num_kv_heads=4, head_dim=128, kv_dtype=kv,
                              seed=102),
    ]
    for n, case in enumerate(cases):
        note(f"[noalloc] {kv} call {n}: lengths {case.seq_lens.tolist()} Hq={case.num_q_heads} "
             f"Hkv={case.num_kv_heads}")
        (o_ws, l_ws), (o_na, l_na) = _both(case)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), f"call {n}: O differs"
        assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32)), f"call {n}: LSE differs"
        ro, rl = oracle_decode(case)
        compare(widen(o_na, case.q_dtype), ro, decode_kind(case), f"noalloc call {n} O")
        compare(l_na.numpy(), rl, decode_kind(case), f"noalloc call {n} LSE", lse=True)


def test_noalloc_decode_full_workload_sampled():
    """The 64-sequence decode workload (L ~ U[512, 32768], Hq=32 Hkv=8): its 34 MB of partial
    results fit the scratch; equal to the workspace entry point bit for bit."""
    case = workloads.config_decode("bf16")
    (o_ws, l_ws), (o_na, l_na) = _both(case)
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32))
    seqs = np.array([0, int(np.argmin(case.seq_lens)), int(np.argmax(case.seq_lens))])
    ro, rl = oracle_decode(case, seqs)
    compare(widen(o_na[torch.from_numpy(seqs).long()], "bf16"), ro, "bf16", "noalloc full O")
    compare(l_na.numpy()[seqs], rl, "bf16", "noalloc full LSE", lse=True)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    case = workloads.make_decode(lengths=[40], num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype="bf16",
                                 seed=103)
    t = decode_tensors(case)
    out = torch.empty_like(t["q"])
    # a forced plan of 65536 splits of 16 tokens over a claimed 2^20-token bound needs
    # 8 x 65536 x 129 x 4 bytes of partials, beyond 64 MiB: rejected on the host, nothing is
    # launched
    with pytest.raises(attn.AttnError):
        attn.decode_paged_noalloc(t["q"], t["k_cache"], t["v_cache"],
                                  torch.zeros((1, 65536), dtype=torch.int32, device="cuda"), t["seq_lens"],
                                  1 << 20, out=out, num_splits=65536)
