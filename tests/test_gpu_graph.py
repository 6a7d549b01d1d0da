"""HIP-graph capture of one linear's training-step launches, through the C ABI.

Every piece of state the entry points keep between kernels lives in the
device records and changes only inside kernels (the tagged amax word and
its epoch, the saturation count), so a captured graph must replay
correctly. The step (fp8_linear_fwd, fp8_linear_bwd, fp8_wgrad_fp8 with
mu, fp8_amax_scale, and a forward-format GEMM whose tiles are split into
reduction halves over a workspace) is captured once and replayed on new inputs whose
magnitudes shrink and grow from replay to replay, with eager work and
synchronisation between the replays. Every replay must equal the same
calls made eagerly on separate buffers, bit for bit (same kernels, same
inputs), and each published amax must equal the oracle's max of the
replay's own input (a stale maximum from an earlier replay would fail
this)."""
import numpy as np
import pytest
import torch

import oracle
import tensor_scaled_fp8_amd as tsf
from tests.gpu_util import bf16_bits, f32_bits, scale_record
from workloads import draw_normal_bf16

pytestmark = pytest.mark.gpu

M, K, N = 400, 528, 784          # several tiles and ragged edges in every GEMM
RS = 1024                        # reduction of the tail-split GEMM
# (sigma X, sigma W, sigma dY) per replay: the first is the captured run
SIGMAS = [(1.0, 0.02, 1e-5), (1e-3, 0.5, 1e-8), (30.0, 1e-4, 3e-3), (1e-6, 0.02, 1e-5), (2.0, 2.0, 2.0)]


class Step:
    def __init__(self):
        bf = dict(dtype=torch.bfloat16, device="cuda")
        u8 = dict(dtype=torch.uint8, device="cuda")
        self.X, self.W, self.dY = torch.empty((M, K), **bf), torch.empty((K, N), **bf), torch.empty((M, N), **bf)
        self.ws = tsf.LinearWorkspace(M, K, N)
        self.Y, self.dX, self.dW = torch.empty((M, N), **bf), torch.empty((M, K), **bf), torch.empty((K, N), **bf)
        self.dW2, self.dw8, self.dw8t = torch.empty((K, N), **bf), torch.empty((K, N), **u8), torch.empty((N, K), **u8)
        self.s_dw, self.s_a = tsf.new_scale(1)[0], tsf.new_scale(1)[0]
        # tail-split GEMM: A [M, RS], B [N, RS] E4M3 codes, every tile split in two
        self.a8, self.b8 = torch.empty((M, RS), **u8), torch.empty((N, RS), **u8)
        self.sa8, self.sb8 = scale_record(6), scale_record(11)
        self.ws8 = torch.empty(tsf.gemm_workspace_bytes("e4m3", "e4m3", M, N, RS, "tail"), **u8)
        assert self.ws8.numel() > 0
        self.Y3 = torch.empty((M, N), **bf)

    def load(self, i):
        sx, sw, sdy = SIGMAS[i]
        for t, seed, shape, sigma in ((self.X, 1, (M, K), sx), (self.W, 2, (K, N), sw), (self.dY, 3, (M, N), sdy)):
            bits = draw_normal_bf16(100 * i + seed, shape, sigma)
            t.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
        g = np.random.Generator(np.random.PCG64(100 * i + 7))
        self.a8.copy_(torch.from_numpy(oracle.encode(g.standard_normal((M, RS)) * 6, oracle.E4M3)))
        self.b8.copy_(torch.from_numpy(oracle.encode(g.standard_normal((N, RS)) * 40, oracle.E4M3)))

    def run(self):
        tsf.fp8_linear_fwd(self.X, self.W, self.ws, Y=self.Y)
        tsf.fp8_linear_bwd(self.dY, self.ws, mu_log2=1, dX=self.dX, dW=self.dW)
        tsf.fp8_wgrad_fp8(self.ws.x8, self.ws.sx, self.ws.dy8, self.ws.sdy, 0, 2, dW=self.dW2, s_dw=self.s_dw,
                          dw8=self.dw8, dw8t=self.dw8t, transposed=True, x_layout="cols", dy_layout="cols")
        tsf.fp8_amax_scale(self.dY, "e5m2", self.s_a, 0, 1)
        tsf.fp8_gemm(self.a8, "e4m3", self.sa8, self.b8, "e4m3", self.sb8, out=self.Y3, workspace=self.ws8,
                     split="tail")

    def outputs(self):
        ws = self.ws
        return {"Y": self.Y, "dX": self.dX, "dW": self.dW, "dW2": self.dW2, "dw8": self.dw8, "dw8t": self.dw8t,
                "x8": ws.x8, "w8": ws.w8, "dy8": ws.dy8, "Y3": self.Y3}

    def records(self):
        recs = {"sx": self.ws.sx, "sw": self.ws.sw, "sdy": self.ws.sdy, "s_dw": self.s_dw, "s_a": self.s_a}
        return {k: (lambda r: (f32_bits(r["amax"]), r["bias"], r["flags"], r["sat_count"]))(tsf.read_scale(v))
                for k, v in recs.items()}


def test_graph_replays_match_eager():
    eager, cap = Step(), Step()
    cap.load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cap.run()                      # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.run()
    torch.cuda.synchronize()
    for i in range(len(SIGMAS)):
        cap.load(i)
        eager.load(i)
        eager.run()                    # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = cap.outputs(), eager.outputs()
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), (i, k)
        ra, rb = cap.records(), eager.records()
        assert ra == rb, (i, ra, rb)
        # each amax is this replay's own
        for name, t in (("sx", cap.X), ("sw", cap.W), ("sdy", cap.dY), ("s_a", cap.dY)):
            assert ra[name][0] == f32_bits(oracle.amax(bf16_bits(t))), (i, name)
        assert ra["s_dw"][0] == f32_bits(oracle.amax(bf16_bits(cap.dW2))), i
        # the split GEMM of this replay's codes against the oracle
        bits, _, tol = oracle.gemm_nt(cap.a8.cpu().numpy(), oracle.E4M3, 6, cap.b8.cpu().numpy(), oracle.E4M3, 11)
        err = np.abs(oracle.bf16_to_f64(bf16_bits(cap.Y3)) - oracle.bf16_to_f64(bits))
        assert not np.any(~(err <= tol)), (i, float(np.max(err / tol)))
