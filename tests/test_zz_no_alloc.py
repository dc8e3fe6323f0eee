"""The allocation-free grouping entry point (vc_vsmooth_group_static) through the C ABI: the
same results as vc_vsmooth_group bit for bit, on two calls in a row where the second is smaller
(the library's scratch then holds the first call's data), and the size limit enforced on the host.
Collected last: a failure here hides no other test."""
import ctypes

import numpy as np
import pytest
import torch

import bit_attention_video_amd as vc

from gpu_util import DEV, bf16_dev, config_inputs, note

S = vc.STATUS


def test_static_group_size_limit_on_host():
    lib = vc.lib()
    FAKE = ctypes.c_void_p(0x1000)        # never dereferenced: the call fails before any use
    # B*H = 200, N = 65,536, k = 256 needs more than the 16 MiB scratch
    assert lib.vc_group_workspace_size(1, 200, 65536, 256) > 16 << 20
    args = (FAKE, 1, 200, 65536, 128, 256, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert lib.vc_vsmooth_group_static(*args) == S["VC_ERR_WORKSPACE"]
    assert lib.vc_vsmooth_group_static(FAKE, 1, 1, 1000, 128, 8, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == S["VC_ERR_SHAPE"]
    assert lib.vc_vsmooth_group_static(None, 1, 1, 1024, 128, 8, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == S["VC_ERR_NULL"]
    assert lib.vc_vsmooth_group_static(FAKE, 1, 1, 1024, 128, 0, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == S["VC_ERR_K"]
    assert lib.vc_vsmooth_group_static(None, 1, 0, 1024, 128, 8, 3, None, None, None, None, None, None,
                                       None) == S["VC_OK"]
    # the largest workloads fit
    assert lib.vc_group_workspace_size(1, 40, 70016, 128) <= 16 << 20
    assert lib.vc_group_workspace_size(1, 24, 115200, 256) <= 16 << 20


def _same(a, b):
    for key in ("labels", "perm", "offsets", "C", "J"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.gpu
def test_static_group_matches_workspace_call_twice():
    cases = [("video", [0, 1, 2, 3], 128, 4), ("medium", [5], 64, 3)]     # the second call is smaller
    for name, heads, k, iters in cases:
        cfg, Q, K, V = config_inputs(name, heads)
        note(f"static-scratch grouping {name} heads={heads} k={k} iters={iters}")
        Vd = bf16_dev(V)
        got = vc.vc_vsmooth_group_static(Vd, k, iters)
        ref = vc.vc_vsmooth_group(Vd, k, iters)
        torch.cuda.synchronize()
        _same(got, ref)
        assert not vc.vc_validate_perm(got["perm"]).any()
    # warm start through the static path as well
    got_w = vc.vc_vsmooth_group_static(Vd, k, 2, C_init=ref["C"])
    ref_w = vc.vc_vsmooth_group(Vd, k, 2, C_init=ref["C"])
    _same(got_w, ref_w)
