"""The custom-op layer on the host (CPU only): the addrms::* ops register and
their fake implementations give the output shapes and dtypes the kernels
produce, without touching a device."""
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import add_rmsnorm_amd.autograd  # noqa: F401  (registers the ops)


def test_fake_shapes():
    with FakeTensorMode():
        x = torch.empty(3, 5, 96, dtype=torch.bfloat16)
        w = torch.empty(96, dtype=torch.float32)
        y, rstd = torch.ops.addrms.rms_norm_fwd(x, w, 1e-6)
        assert y.shape == x.shape and y.dtype == x.dtype
        assert rstd.shape == (3, 5) and rstd.dtype == torch.float32
        y, res, rstd = torch.ops.addrms.add_rms_norm_fwd(x, x, w, 1e-6)
        assert res.shape == x.shape and res.dtype == x.dtype and rstd.shape == (3, 5)
        dx, dw = torch.ops.addrms.rms_norm_bwd(x, x, w, rstd)
        assert dx.shape == x.shape and dw.shape == (96,) and dw.dtype == torch.float32
        dh, dw = torch.ops.addrms.add_rms_norm_bwd(x, None, x, w, rstd)
        assert dh.shape == x.shape and dw.dtype == torch.float32


def test_fake_shapes_layernorm():
    with FakeTensorMode():
        x = torch.empty(6, 128, dtype=torch.bfloat16)
        w = torch.empty(128, dtype=torch.bfloat16)
        y, mean, rstd = torch.ops.addrms.layer_norm_fwd(x, w, w, 1e-5)
        assert y.shape == x.shape and mean.shape == (6,) and rstd.dtype == torch.float32
        y, res, mean, rstd = torch.ops.addrms.add_layer_norm_fwd(x, x, w, None, 1e-5)
        assert res.shape == x.shape and mean.shape == (6,)
        dh, dw, db = torch.ops.addrms.add_layer_norm_bwd(x, None, x, w, mean, rstd)
        assert dh.shape == x.shape and dw.shape == db.shape == (128,)
