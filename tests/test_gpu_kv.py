"""GPU parity: NVFP4 KV cache quantize-on-write / dequantize-on-read vs the oracle.

Bar: the cache bytes equal the oracle's whole-tensor quantization with the
same static globals, bit for bit, whatever the chunk order; reads equal the
oracle's dequantization bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth
from tests.gpu_util import step, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _caches(tokens, heads, dim, gk, gv):
    kc = nv.NVFP4Tensor.empty(tokens * heads, dim, 1, DEV)
    vc = nv.NVFP4Tensor.empty(tokens * heads, dim, 1, DEV)
    kc.global_.fill_(gk)
    vc.global_.fill_(gv)
    return kc, vc


def _static_global(orc, t):
    b = synth.bits(t).reshape(-1, t.shape[-1])
    return float(orc.global_from_amax(orc.amax_bf16(np.ascontiguousarray(b))))


@pytest.mark.parametrize("order", ["forward", "shuffled"])
def test_chunked_writes_equal_whole_tensor(orc, order):
    kv = synth.KVCache(tokens=8192, chunk=2048)
    k, v = kv.k(), kv.v()
    gk, gv = _static_global(orc, k), _static_global(orc, v)
    kc, vc = _caches(kv.tokens, kv.heads, kv.dim, gk, gv)
    kd, vd = k.to(DEV), v.to(DEV)
    starts = list(range(0, kv.tokens, kv.chunk))
    if order == "shuffled":
        starts = list(np.random.default_rng(5).permutation(starts))
    for c0 in starts:
        step(f"kv write chunk at {c0}")
        nv.nvfp4_kv_quant(kd[c0:c0 + kv.chunk], vd[c0:c0 + kv.chunk], int(c0), kc, vc, kv.heads)
    torch.cuda.synchronize()
    for name, t, cache, g in (("k", k, kc, gk), ("v", v, vc, gv)):
        ref = orc.quantize(np.ascontiguousarray(synth.bits(t).reshape(-1, kv.dim)), static_G=g)
        np.testing.assert_array_equal(u8(cache.scales)[0], ref.scales, err_msg=name)
        np.testing.assert_array_equal(u8(cache.packed)[0], ref.packed, err_msg=name)
        # read back a window and the whole cache
        ko, vo = nv.nvfp4_kv_dequant(kc, vc, kv.heads, 1000, 3000, torch.bfloat16)
        got = synth.bits(ko if name == "k" else vo).reshape(-1, kv.dim)
        _, bref = orc.dequantize(ref.rows(1000 * kv.heads, 4000 * kv.heads), want_bf16=True)
        np.testing.assert_array_equal(got, bref)


def test_chunked_writes_replayed_from_a_graph(orc):
    """The chunk writes captured once in a HIP graph, as a serving loop runs
    them: every replay (caches cleared and unrelated eager work in between)
    leaves exactly the bytes of the eager writes."""
    kv = synth.KVCache(tokens=8192, chunk=2048)
    k, v = kv.k(), kv.v()
    gk, gv = _static_global(orc, k), _static_global(orc, v)
    kd, vd = k.to(DEV), v.to(DEV)
    ke, ve = _caches(kv.tokens, kv.heads, kv.dim, gk, gv)
    kg, vg = _caches(kv.tokens, kv.heads, kv.dim, gk, gv)

    def write_all(kc, vc):
        for c0 in range(0, kv.tokens, kv.chunk):
            nv.nvfp4_kv_quant(kd[c0:c0 + kv.chunk], vd[c0:c0 + kv.chunk], c0, kc, vc, kv.heads)

    step("kv eager writes")
    write_all(ke, ve)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        write_all(kg, vg)
    torch.cuda.current_stream().wait_stream(side)
    step("kv graph capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        write_all(kg, vg)
    for rep in range(3):
        for t in (kg.packed, kg.scales, vg.packed, vg.scales):
            t.zero_()
        nv.nvfp4_kv_dequant(ke, ve, kv.heads, 0, 512, torch.bfloat16)
        step(f"kv graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for a, b in ((kg, ke), (vg, ve)):
            assert torch.equal(a.packed, b.packed) and torch.equal(a.scales, b.scales), rep


def test_full_context_write_read_sampled(orc):
    """262144 tokens x 4 heads x 256, 128 chunk writes then one full read;
    sampled rows checked against the oracle."""
    kv = synth.C5
    k, v = kv.k(DEV), kv.v(DEV)
    gk = orc.global_from_amax(float(k.float().abs().max().item()))
    gv = orc.global_from_amax(float(v.float().abs().max().item()))
    kc, vc = _caches(kv.tokens, kv.heads, kv.dim, gk, gv)
    step("kv full-context writes")
    for c0 in range(0, kv.tokens, kv.chunk):
        nv.nvfp4_kv_quant(k[c0:c0 + kv.chunk], v[c0:c0 + kv.chunk], c0, kc, vc, kv.heads)
    step("kv full-context read")
    ko, vo = nv.nvfp4_kv_dequant(kc, vc, kv.heads, 0, kv.tokens, torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[np.random.default_rng(6).choice(kv.tokens * kv.heads, 64, replace=False),
                           0, kv.tokens * kv.heads - 1])
    for t, cache, g, out in ((k, kc, gk, ko), (v, vc, gv, vo)):
        src = synth.bits(t.reshape(-1, kv.dim)[torch.from_numpy(rows).to(DEV)])
        ref = orc.quantize(np.ascontiguousarray(src), static_G=g)
        np.testing.assert_array_equal(u8(cache.scales)[0][rows], ref.scales)
        np.testing.assert_array_equal(u8(cache.packed)[0][rows], ref.packed)
        f = out.reshape(-1, kv.dim)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        np.testing.assert_array_equal(f.view(np.uint32), orc.dequantize(ref).view(np.uint32))
    counts = nv.nvfp4_audit_scales(kc).cpu().numpy()
    assert counts[0] == kv.tokens * kv.heads * kv.dim // 16
    assert counts[1] == 0 and counts[2] == 0 and counts[3] >= 1


def test_k_only_and_bounds():
    kc, vc = _caches(16, 4, 256, 1.0, 1.0)
    k = torch.zeros((8, 4, 256), dtype=torch.bfloat16, device=DEV)
    nv.nvfp4_kv_quant(k, None, 8, kc, vc, 4)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_kv_quant(k, None, 9, kc, vc, 4)  # past the cache end
