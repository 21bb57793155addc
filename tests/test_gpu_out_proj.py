"""The block's tail on the GPU (muse_out_proj: o_proj 4096 -> 6656, the
post-attention RMSNorm with epsilon 1e-8, the residual add; "Chapter 9 - The
Muse Glimmer architecture" 9.8, 9.9 and Figure 9.1) against the oracle, on
seeded synthetic weights.

Tolerance: the bf16 bound, |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise (the
GPU accumulates the bf16 products in f32 and rounds the output to bf16; the
oracle is double throughout).  Token counts cover the few-token kernel (1 to
64 rows: one to four 16-row tiles, full and ragged), the hipBLASLt GEMM above
64 tokens (65, 256, 257, 300, 513), and a prefill-sized batch checked on
sampled rows (rows are independent, so a sample is exact for its rows).
"""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
import oracle
from full_gqa_attention_amd import synth
from parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_case(M, rows=None, config=70, in_place=False):
    inp = synth.out_proj_inputs(M, config=config, device=DEV, backend="numpy" if M <= 4096 else "torch")
    res_before = inp.residual.clone()
    if in_place:
        out = fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual, out=inp.residual)
    else:
        out = fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(M)
    ref = oracle.out_proj_rows(bits(inp.attn), bits(inp.w), inp.gamma.cpu().numpy(), bits(res_before), rows=rows)
    got = out[torch.as_tensor(rows, device=DEV).long()].double().cpu().numpy()
    return assert_close(got, ref, synth.BF16, f"out_proj M={M}")


@pytest.mark.parametrize("M", [1, 4, 16, 17, 32, 33, 48, 64, 65, 256, 257])
def test_out_proj_all_rows(M):
    run_case(M)


def test_out_proj_prefill_sized_sampled_rows():
    """8 x 8,192 tokens (the prefill workload's batch) on sampled rows,
    including the first and last rows and rows around 256-row boundaries."""
    M = 65536
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 257, 4095, 4096, 32767, 65279, 65280, 65535],
                                     np.random.default_rng(3).integers(0, M, 21)]))
    run_case(M, rows=rows, config=71)


@pytest.mark.parametrize("M", [1024, 4096, 16384])
def test_out_proj_mid_sized_sampled_rows(M):
    """Token counts where the GEMM library picks other algorithms than at
    65,536 (at 16,384 its first pick needs a workspace, which the call does
    not pass: only algorithms that need none may run), on sampled rows."""
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1],
                                     np.random.default_rng(M).integers(0, M, 16)]))
    run_case(M, rows=rows, config=76)


def test_out_proj_in_place_residual():
    run_case(300, in_place=True, config=72)


def test_out_proj_deterministic():
    inp = synth.out_proj_inputs(513, config=73, device=DEV)
    a = fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual).clone()
    b = fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_out_proj_few_tokens_reused_workspace():
    """One workspace (filled with junk first) through few-token calls of
    different sizes: the slice partials a previous call left behind must not
    leak into the next."""
    ws = torch.empty(fa.out_proj_workspace_size(64), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)
    for i, M in enumerate([64, 7, 64, 1, 40]):
        inp = synth.out_proj_inputs(M, config=74, step=i, device=DEV, backend="numpy")
        out = fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.out_proj_rows(bits(inp.attn), bits(inp.w), inp.gamma.cpu().numpy(), bits(inp.residual))
        assert_close(out.double().cpu().numpy(), ref, synth.BF16, f"out_proj reused workspace call {i} M={M}")


def test_out_proj_few_tokens_graph_replays_match_eager():
    """A captured few-token call replays with new attn rows copied in and eager
    calls in between; every replay equals the eager result bit for bit."""
    M = 48
    inp = synth.out_proj_inputs(M, config=75, device=DEV)
    ws = torch.empty(fa.out_proj_workspace_size(M), dtype=torch.uint8, device=DEV)
    attn, out = inp.attn.clone(), torch.empty_like(inp.residual)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                         # warm-up outside the capture
        fa.out_proj(attn, inp.w, inp.gamma, inp.residual, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.out_proj(attn, inp.w, inp.gamma, inp.residual, out=out, workspace=ws)
    for rep in range(3):
        attn.copy_(synth.out_proj_inputs(M, config=75, step=10 + rep, device=DEV).attn)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = fa.out_proj(attn, inp.w, inp.gamma, inp.residual)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"
