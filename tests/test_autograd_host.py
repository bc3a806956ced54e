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


def test_fake_shapes_fp8_and_rope():
    with FakeTensorMode():
        x = torch.empty(4, 7168, dtype=torch.bfloat16)
        w = torch.empty(7168, dtype=torch.bfloat16)
        q, s = torch.ops.addrms.rms_norm_fp8(x, w, 1e-6, 0)
        assert q.dtype == torch.float8_e4m3fn and q.shape == x.shape and s.shape == (4,)
        q, s, res = torch.ops.addrms.add_rms_norm_fp8(x, x, w, 1e-6, 128)
        assert s.shape == (4, 56) and s.dtype == torch.float32 and res.shape == x.shape
        q, s = torch.ops.addrms.rms_norm_fp8(x, w, 1e-6, 100000)
        assert s.shape == (4, 1)
        qh = torch.empty(8, 32, 128, dtype=torch.bfloat16)
        kh = torch.empty(8, 8, 128, dtype=torch.bfloat16)
        wq = torch.empty(128, dtype=torch.bfloat16)
        cos = torch.empty(64, 64)
        pos = torch.empty(8, dtype=torch.int64)
        qo, ko = torch.ops.addrms.rms_norm_rope_qk(qh, kh, wq, wq, cos, cos, pos, 1e-6, False)
        assert qo.shape == qh.shape and ko.shape == kh.shape and qo.dtype == torch.bfloat16
        assert torch.ops.addrms.rms_norm_rope_qk_(qh, kh, wq, wq, cos, cos, pos, 1e-6, True) is None


def test_fake_shapes_mxfp4():
    with FakeTensorMode():
        x = torch.empty(4, 7168, dtype=torch.bfloat16)
        w = torch.empty(7168, dtype=torch.bfloat16)
        q, s = torch.ops.addrms.rms_norm_mxfp4(x, w, 1e-6)
        assert q.shape == (4, 3584) and q.dtype == torch.float4_e2m1fn_x2
        assert s.shape == (4, 224) and s.dtype == torch.float8_e8m0fnu
        q, s, res = torch.ops.addrms.add_rms_norm_mxfp4(x, x, w, 1e-6)
        assert res.shape == x.shape and s.shape == (4, 224)
