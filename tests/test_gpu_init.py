"""mi_init (include/mi_normquant.h): after it, the first call of each GEMM
kernel that needs a raised LDS limit (the decode step in one launch and in
two, the stream pair, the TP-shard forms, the wide and the decode GEMMs, fp32
and e8m0 scales)
can be captured into a HIP graph with no ordinary call before it, and the replay
equals an eager call bit for bit.  Run in a fresh process, so that no
earlier test has launched (and thereby prepared) those kernels."""
import os
import subprocess
import sys

import pytest

from helpers import gpu_or_skip

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import rmsnorm_fp8_block_amd as mi

dev = torch.device("cuda:0")
g = torch.Generator(device="cpu").manual_seed(5)


def codes(*shape):
    c = torch.randint(0, 0x78, shape, generator=g, dtype=torch.int32) | (torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 7)
    return c.to(torch.uint8).to(dev)


def fscale(*shape):
    return (torch.rand(shape, generator=g) * 1e-2 + 1e-3).to(dev)


def escale(*shape):
    return torch.randint(118, 127, shape, generator=g, dtype=torch.int32).to(torch.uint8).to(dev)


mi.mi_init()
cases = []
# one-launch decode step, M = 8 (fp32 scales)
M = 8
buf = torch.randn((M, 2048), generator=g).to(torch.bfloat16).to(dev)
gq = (1 + 0.1 * torch.randn(1536, generator=g)).to(torch.bfloat16).to(dev)
gk = (1 + 0.1 * torch.randn(512, generator=g)).to(torch.bfloat16).to(dev)
wa, wb = mi.relayout_weight(codes(24576, 1536)), mi.relayout_weight(codes(8192, 1536))
sa, sb = fscale(192, 12), fscale(64, 12)
def step(o):
    return mi.prepare_fused_normquant_gemm_pair(buf[:, :1536], buf[:, 1536:], gq, gk, 1e-6, True, wa, sa, wb, sb, *o)
def step_outs():
    return (torch.empty((M, 1536), dtype=torch.uint8, device=dev), torch.empty(M * 12, device=dev),
            torch.empty((M, 512), dtype=torch.bfloat16, device=dev), torch.empty((M, 24576), dtype=torch.bfloat16, device=dev),
            torch.empty((M, 8192), dtype=torch.bfloat16, device=dev))
cases.append(("step M=8", step, step_outs))
# the step at M = 48 (two launches: the norm-quant, then the stream pair)
buf48 = torch.randn((48, 2048), generator=g).to(torch.bfloat16).to(dev)
def step48(o):
    return mi.prepare_fused_normquant_gemm_pair(buf48[:, :1536], buf48[:, 1536:], gq, gk, 1e-6, True, wa, sa, wb, sb, *o)
def step48_outs():
    return (torch.empty((48, 1536), dtype=torch.uint8, device=dev), torch.empty(48 * 12, device=dev),
            torch.empty((48, 512), dtype=torch.bfloat16, device=dev), torch.empty((48, 24576), dtype=torch.bfloat16, device=dev),
            torch.empty((48, 8192), dtype=torch.bfloat16, device=dev))
cases.append(("step M=48", step48, step48_outs))
# TP shards at M = 1: the TP-8 pair (split-K, one subtile per CU) and the
# TP-2 pair (stream kernel, one subtile per wave, four per CU)
a1, s1 = codes(1, 1536), fscale(12, 1).T
wa8, wb8 = mi.relayout_weight(codes(3072, 1536)), mi.relayout_weight(codes(1024, 1536))
wa2, wb2 = mi.relayout_weight(codes(12288, 1536)), mi.relayout_weight(codes(4096, 1536))
for tag, x1, x2 in (("TP-8", wa8, wb8), ("TP-2", wa2, wb2)):
    y1, y2 = fscale(x1.N // 128, 12), fscale(x2.N // 128, 12)
    cases.append((f"{tag} pair M=1",
                  lambda o, x1=x1, x2=x2, y1=y1, y2=y2: mi.prepare_block_scaled_fp8_gemm_pair(
                      a1, s1, x1, y1, o[0], x2, y2, o[1]),
                  lambda x1=x1, x2=x2: (torch.empty((1, x1.N), dtype=torch.bfloat16, device=dev),
                                        torch.empty((1, x2.N), dtype=torch.bfloat16, device=dev))))
# stream pair, M = 64, column-major scales
a64, s64 = codes(64, 1536), fscale(12, 64).T
def pair(o):
    return mi.prepare_block_scaled_fp8_gemm_pair(a64, s64, wa, sa, o[0], wb, sb, o[1])
cases.append(("pair M=64", pair, lambda: (torch.empty((64, 24576), dtype=torch.bfloat16, device=dev),
                                          torch.empty((64, 8192), dtype=torch.bfloat16, device=dev))))
# wide GEMM, M = 256, fp32 and e8m0 scales
a256 = codes(256, 1536)
s256, e256 = fscale(256, 12), escale(256, 12)
ea = escale(192, 12)
cases.append(("wide M=256", lambda o: mi.prepare_block_scaled_fp8_gemm(a256, s256, wa, sa, o[0]),
              lambda: (torch.empty((256, 24576), dtype=torch.bfloat16, device=dev),)))
cases.append(("wide e8m0 M=256", lambda o: mi.prepare_block_scaled_fp8_gemm(a256, e256, wa, ea, o[0]),
              lambda: (torch.empty((256, 24576), dtype=torch.bfloat16, device=dev),)))
# decode GEMM: M = 8 over a K = 2048 weight (the stream kernel takes K/128 in {4, 8, 12} only)
w2k = codes(24576, 2048)
a8, s8, sw2k = codes(8, 2048), fscale(8, 16), fscale(192, 16)
cases.append(("decode M=8 K=2048", lambda o: mi.prepare_block_scaled_fp8_gemm(a8, s8, w2k, sw2k, o[0]),
              lambda: (torch.empty((8, 24576), dtype=torch.bfloat16, device=dev),)))

fails = 0
for name, make, outs in cases:
    o_graph = outs()
    call = make(o_graph)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        call()          # the first launch of this kernel in the process
    for _ in range(2):
        gr.replay()
    torch.cuda.synchronize()
    o_eager = outs()
    make(o_eager)()
    torch.cuda.synchronize()
    same = all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(o_graph, o_eager))
    print(name, "replay == eager" if same else "MISMATCH", flush=True)
    fails += not same
print("FAILS", fails, flush=True)
sys.exit(1 if fails else 0)
"""


def test_first_calls_captured_after_init():
    gpu_or_skip()
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "FAILS 0" in r.stdout
