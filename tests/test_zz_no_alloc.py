"""The allocation-free MoE entry point (nvfp4_moe_grouped_gemm_noalloc):
same kernels as nvfp4_moe_grouped_gemm on the library's own device scratch,
for callers that cannot allocate.  Its output must equal the allocating
entry point's bit for bit, on two calls in a row (the second smaller, so it
runs on what the first left in the scratch), and a layer whose workspace
exceeds the scratch is refused before any launch."""
import ctypes

import pytest
import torch

import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import _lib, synth, workloads
from tests.gpu_util import step

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(x, ids, w, W, static_in_globals=None):
    T, H = x.shape
    k = ids.shape[1]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    c13, c2 = W.w13.c(), W.w2.c()
    st = _lib.load().nvfp4_moe_grouped_gemm_noalloc(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(w.data_ptr()), T, k,
        W.w13.batch, ctypes.byref(c13), ctypes.byref(c2),
        None if static_in_globals is None else ctypes.c_void_p(static_in_globals.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out


def test_noalloc_equals_allocating_entry_point_twice():
    cfg = synth.C4_DECODE                       # 384 experts, top-8, T = 64
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("noalloc: 384-expert decode batch T=64")
    st, got = _noalloc(x, ids, w, W)
    assert st == _lib.OK, nv.status_string(st)
    ref = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # second call, smaller batch (the first 16 tokens)
    step("noalloc: second call T=16")
    x2, ids2, w2 = x[:16].contiguous(), ids[:16].contiguous(), w[:16].contiguous()
    st, got2 = _noalloc(x2, ids2, w2, W)
    assert st == _lib.OK
    ref2 = nv.nvfp4_moe_grouped_gemm(x2, ids2, w2, W.w13, W.w2)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2)
    assert nv.nvfp4_get_error() == 0


def test_noalloc_dense_mlp_and_static_globals():
    """The 27B-class MLP as one expert at M = 1 and 32 (K-split gate_up and
    down), with calibrated globals on the second call."""
    c2 = synth.C2
    mlp = workloads.build_dense_mlp(c2, DEV)
    for M, static in ((32, False), (1, True)):
        x = c2.x(M, DEV)
        ids = torch.zeros((M, 1), dtype=torch.int32, device=DEV)
        wt = torch.ones((M, 1), dtype=torch.float32, device=DEV)
        sg = torch.tensor([0.01, 0.002], dtype=torch.float32, device=DEV) if static else None
        step(f"noalloc: dense MLP M={M} static={static}")
        st, got = _noalloc(x, ids, wt, mlp, sg)
        assert st == _lib.OK, nv.status_string(st)
        ref = nv.nvfp4_moe_grouped_gemm(x, ids, wt, mlp.w13, mlp.w2, static_in_globals=sg)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_noalloc_refuses_layers_beyond_the_scratch():
    cfg = synth.MoE(seed=70, E=8, k=2, H=4096, I=1024, T=4096)
    lib = _lib.load()
    need = nv.nvfp4_workspace_size(_lib.OP_MOE, cfg.T, cfg.k, cfg.E, cfg.H, cfg.I)
    assert need > lib.nvfp4_noalloc_scratch_bytes()
    W = workloads.MoEWeights(nv.NVFP4Tensor.empty(2 * cfg.I, cfg.H, cfg.E, DEV),
                             nv.NVFP4Tensor.empty(cfg.H, cfg.I, cfg.E, DEV))
    x = torch.zeros((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    step("noalloc: oversized layer refused")
    st, _ = _noalloc(x, ids, w, W)
    assert st == _lib.WORKSPACE


def test_noalloc_layer_replays_from_a_hip_graph():
    """The allocation-free layer captured in a HIP graph (it records no
    allocation and no memset) and replayed several times, with eager work
    and synchronizations in between: every replay equals the eager call."""
    cfg = synth.C4_DECODE
    W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
    ref = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.nvfp4_moe_grouped_gemm_noalloc(x, ids, w, W.w13, W.w2, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    step("noalloc: capture the 384-expert decode layer")
    with torch.cuda.graph(graph):
        nv.nvfp4_moe_grouped_gemm_noalloc(x, ids, w, W.w13, W.w2, out=out)
    for rep in range(4):
        out.zero_()
        # eager work on the same scratch between replays
        other = nv.nvfp4_moe_grouped_gemm_noalloc(x[:8].contiguous(), ids[:8].contiguous(), w[:8].contiguous(),
                                                  W.w13, W.w2)
        torch.cuda.synchronize()
        step(f"noalloc: graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert other.shape == (8, cfg.H)
    assert nv.nvfp4_get_error() == 0
