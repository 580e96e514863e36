"""w8a8_linear_noalloc (the K-split scratch in the library's static device
array) against w8a8_linear with a caller workspace: bitwise-equal outputs and
int32 sums on two calls in a row, the second smaller, through the C ABI."""
import numpy as np
import pytest
import torch

import ditsynth
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, dev, say

pytestmark = pytest.mark.gpu


def _pair(M, N, K, seed):
    a, b, sa, sb, bias = ditsynth.int8_operands(M, N, K, seed=seed)
    args = (dev(a, torch.int8), dev(sa), dev(b, torch.int8), dev(sb), dev(bias))
    y_ws = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    acc_ws = torch.empty((M, N), dtype=torch.int32, device=DEV)
    work = torch.empty((dq.w8a8_linear_workspace_bytes(),), dtype=torch.uint8, device=DEV)
    dq.w8a8_linear(*args, y_ws, acc_out=acc_ws, workspace=work)
    y_na = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    acc_na = torch.full((M, N), -5, dtype=torch.int32, device=DEV)
    dq.w8a8_linear_noalloc(*args, y_na, acc_out=acc_na)
    torch.cuda.synchronize()
    return y_ws, acc_ws, y_na, acc_na


def test_noalloc_matches_workspace_variant_two_calls():
    # 1) 272 tiles on 256 CUs: the 16 tiles of the last round split along K
    #    (more K ranges than the 32 MiB scratch holds with a workspace: fewer here)
    # 2) a smaller call after it: 4 tiles, every tile split; the scratch keeps the
    #    first call's contents, which the second call must not read
    for M, N, K in ((4352, 4096, 4096), (300, 512, 4096)):
        say("noalloc", M, N, K)
        y_ws, acc_ws, y_na, acc_na = _pair(M, N, K, seed=M + N)
        assert torch.equal(acc_na, acc_ws)
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
