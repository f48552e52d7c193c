"""The measurement probes run on the GPU and report physically plausible figures; the
cache flush really writes zeros over its buffer."""
import numpy as np
import pytest
import torch

import attention_forward_03_amd as attn

pytestmark = pytest.mark.gpu


def _operands(seed):
    # random bf16 bits of N(0,1)-like magnitude, two per 32-bit word
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(256 * 8 * 2).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint32)
    w = (b[0::2] | (b[1::2] << 16)).astype(np.uint32)
    return torch.from_numpy(w.view(np.int32)).cuda()


@pytest.mark.parametrize("valu_mix", [False, True])
def test_probe_mfma_reports_clock_and_rate(valu_mix):
    wg, iters = 256, 2000
    ops = _operands(11)
    clocks = torch.zeros(2 * wg, dtype=torch.int64, device="cuda")
    sink = torch.zeros(256 * wg, dtype=torch.float32, device="cuda")
    print(f"[probe] mfma wg={wg} iters={iters} valu_mix={valu_mix}", flush=True)
    attn.probe_mfma(ops, clocks, sink, workgroups=wg, iters=iters, valu_mix=valu_mix)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    attn.probe_mfma(ops, clocks, sink, workgroups=wg, iters=iters, valu_mix=valu_mix)
    e[1].record()
    torch.cuda.synchronize()
    c = clocks.cpu().numpy().reshape(wg, 2)
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
    ghz = c[:, 0].sum() / (c[:, 1].sum() / 100e6) / 1e9
    tflops = wg * 4 * 32 * iters * 32768 / (e[0].elapsed_time(e[1]) * 1e-3) / 1e12
    print(f"[probe] {ghz:.3f} GHz, {tflops:.0f} TFLOP/s", flush=True)
    assert 0.5 < ghz < 3.0
    assert 200 < tflops < 2600      # below the 2.5 PFLOP/s dense bf16 specification
    # cycles per product per SIMD: at least the 32 a 32x32x16 product occupies
    cyc_per_mfma = c[:, 0].mean() / (32 * iters)
    assert cyc_per_mfma >= 31.0


def test_probe_hbm_read_rate():
    nbytes, wg = 1 << 30, 2048
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(wg, dtype=torch.int32, device="cuda")
    print(f"[probe] hbm read {nbytes} bytes wg={wg}", flush=True)
    attn.probe_hbm_read(buf, sink, workgroups=wg)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    attn.probe_hbm_read(buf, sink, workgroups=wg)
    e[1].record()
    torch.cuda.synchronize()
    gbps = nbytes / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9
    print(f"[probe] {gbps:.0f} GB/s", flush=True)
    assert 1000 < gbps < 8200        # below the 8 TB/s HBM3E specification (+ timer slack)
    # every 16-byte chunk reads ones: the xor of an even number of ones per lane is 0
    assert (sink.cpu().numpy() == 0).all()


def test_flush_writes_zeros():
    buf = torch.full((1 << 22,), 7, dtype=torch.int32, device="cuda")
    attn.flush_caches(buf)
    torch.cuda.synchronize()
    assert int(buf.abs().sum().item()) == 0
