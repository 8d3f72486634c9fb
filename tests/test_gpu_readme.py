"""README's usage examples run as written (GPU).

The three Python blocks of README.md's Use section -- the forward step
(weight cast, fused quantize, exact FP8 GEMM, state update), the backward of
the same layer (E5M2 cast of the gradient with its transposed codes, the
transposes, dA = dY W, the split-K dW = dY^T A) and the MXFP8 forward
(quantize_mx of the activation and the weight, fp8_gemm_mx) -- are executed
verbatim on seeded GPT-2-shape inputs drawn on the GPU.  Sampled rows of y,
dA, dW and the MX output are compared with the oracle's float64 GEMMs ("FP8
training: what it is and how it works", Step 3; Trade-offs and edge cases for
the 32-value blocks) of the same codes to the plain bound; each per-tensor
cast used its fresh state's first scale, max / (initial_amax * margin)
("Paradigma ...", delayed scaling), and the weight its current scale wsc[1].
"""
import os
import re

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, check_gemm, u8_np

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _blocks():
    return re.findall(r"```python\n(.*?)```", open(README).read(), re.S)


def test_readme_usage_examples():
    blocks = _blocks()
    assert len(blocks) == 3
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    ns = {"h": (torch.randn((16384, 3072), generator=g, device=DEV)).to(torch.bfloat16),
          "w": (torch.randn((768, 3072), generator=g, device=DEV) * 0.02).to(torch.bfloat16)}
    exec(blocks[0], ns)
    ns["dy"] = (torch.randn((16384, 768), generator=g, device=DEV) * 0.01).to(torch.bfloat16)
    exec(blocks[1], ns)
    exec(blocks[2], ns)
    torch.cuda.synchronize()
    s_a = O.State(O.E4M3, 16, 1.25, 1.0).scale
    s_g = O.State(O.E5M2, 16, 1.25, 1.0).scale
    s_w = float(ns["wsc"][1].item())
    a8, w8, dy8, dy8t, a8t, w8t = (u8_np(ns[k]) for k in ("a8", "w8", "dy8", "dy8t", "a8t", "w8t"))
    assert np.array_equal(a8t, a8.T) and np.array_equal(w8t, w8.T)
    rows = np.array([0, 1, 8191, 16382, 16383])
    ref, absref = O.gemm_f64(a8, O.E4M3, w8, O.E4M3, O.PER_TENSOR, s_a, s_w, rows=rows)
    check_gemm(ns["y"].float().cpu().numpy()[rows], ref, absref, "y = A W^T")
    ref, absref = O.gemm_f64(dy8, O.E5M2, w8t, O.E4M3, O.PER_TENSOR, s_g, s_w, rows=rows)
    check_gemm(ns["da"].float().cpu().numpy()[rows], ref, absref, "dA = dY W")
    wrows = np.array([0, 383, 767])
    ref, absref = O.gemm_f64(dy8t, O.E5M2, a8t, O.E4M3, O.PER_TENSOR, s_g, s_a, rows=wrows)
    check_gemm(ns["dw"].float().cpu().numpy()[wrows], ref, absref, "dW = dY^T A")
    ref, absref = O.gemm_mx_f64(u8_np(ns["ma8"]), O.E4M3, u8_np(ns["ma_e"]), u8_np(ns["mw8"]),
                                O.E4M3, u8_np(ns["mw_e"]), rows=rows)
    check_gemm(ns["my"].float().cpu().numpy()[rows], ref, absref, "MX y = A W^T")
