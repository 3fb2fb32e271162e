"""The library's calls inside a captured HIP graph: every call enqueues kernels
only on the stream it is given (no allocation, no memset, no host sync), so
a graph captured on a side stream replays them.  Each replay is checked
against the eager results, with eager work and synchronisations between the
replays."""
import sys

import numpy as np
import pytest

from ternary_weight_int8_amd import binding as B
from ternary_weight_int8_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def test_graph_replays_match_eager():
    # the stream forward, dW, the skinny forward, the split dX with its
    # workspace and the row quantizer, captured once and replayed three times
    say("graph capture")
    A, Wp = synth.fwd_inputs(3, 2048, 3456, 1280, 3)
    dC = synth.uniform_int8(3, synth.STREAM_DC, 2048, 3456)
    As, Ws = synth.fwd_inputs(4, 27, 4096, 8192, 3)
    dCs, Wxs = synth.dx_inputs(4, 27, 4096, 8192, 3)
    X = synth.float_inputs(5, synth.STREAM_X, 27, 8192, "bf16")
    Ad, Wd, dCd, Asd, Wsd, dCsd, Wxsd = (dev(v) for v in (A, Wp, dC, As, Ws, dCs, Wxs))
    Xd = dev(X).view(torch.bfloat16)
    nws = B.ternary_gemm_dx_workspace(27, 4096, 8192)
    assert nws > 0
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    outs = {
        "fwd": torch.empty((2048, 3456), dtype=torch.int32, device=DEV),
        "dw": torch.empty((1280, 3456), dtype=torch.int32, device=DEV),
        "skinny": torch.empty((27, 4096), dtype=torch.int32, device=DEV),
        "dx_ws": torch.empty((27, 8192), dtype=torch.int32, device=DEV),
        "q": torch.empty((27, 8192), dtype=torch.int8, device=DEV),
        "s": torch.empty((27,), dtype=torch.float32, device=DEV),
    }

    def run(stream):
        B.ternary_gemm_s8(Ad, Wd, C=outs["fwd"], stream=stream)
        B.ternary_gemm_s8_dw(Ad, dCd, dW=outs["dw"], stream=stream)
        B.ternary_gemm_s8(Asd, Wsd, C=outs["skinny"], stream=stream)
        B.ternary_gemm_s8_dx_ws(dCsd, Wxsd, 8192, workspace=ws, dX=outs["dx_ws"], stream=stream)
        B.ternary_quantize_rows(Xd, Q=outs["q"], scale=outs["s"], stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(side)
    side.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run(side)
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        # eager work between the replays on the same buffers' neighbours
        junk = B.ternary_gemm_s8(Asd, Wsd)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager result"
        assert torch.equal(junk, eager["skinny"])
