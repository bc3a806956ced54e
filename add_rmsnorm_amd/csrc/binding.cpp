// Native Python binding of the latency-bound forwards (rmsnorm_fwd,
// add_rmsnorm_fwd): the same calls, arguments, checks and results as the
// ctypes binding in __init__.py, with the tensor checks done on at::Tensor
// in C++.  At decode sizes the call is launch-bound, and the checks of five
// tensors through Python attribute lookups cost about as much as the launch.
// Argument marshalling only: every numeric step runs in libaddrms.so's HIP
// kernels, through its C ABI (include/addrms.h).
#include <torch/extension.h>

#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>

#include "addrms.h"

namespace {

// Python's spelling of a dtype ("torch.bfloat16") and of a shape ("(4, 64)",
// "(64,)"), so that messages match the ctypes binding's word for word
std::string dtype_str(at::ScalarType s)
{
    return py::str(reinterpret_cast<PyObject *>(torch::getTHPDtype(s)));
}

std::string shape_str(at::IntArrayRef s)
{
    std::string out = "(";
    for (size_t i = 0; i < s.size(); i++)
        out += (i ? ", " : "") + std::to_string(s[i]);
    return out + (s.size() == 1 ? ",)" : ")");
}

int code_of(const at::Tensor &t, const char *what)
{
    switch (t.scalar_type()) {
    case at::kFloat: return ADDRMS_F32;
    case at::kBFloat16: return ADDRMS_BF16;
    case at::kHalf: return ADDRMS_F16;
    default:
        throw py::type_error(std::string(what) + ": dtype " + dtype_str(t.scalar_type()) +
                             " not supported (float32, bfloat16, float16)");
    }
}

void check_dev(const at::Tensor &t, const char *what)
{
    if (!t.is_cuda())
        throw py::value_error(std::string(what) + " must be a GPU tensor");
    if (!t.is_contiguous())
        throw py::value_error(std::string(what) + " must be contiguous");
}

// t on the GPU, contiguous, of dtype dt and shape `shape`
void check_like(const at::Tensor &t, const char *what, at::ScalarType dt, at::IntArrayRef shape)
{
    check_dev(t, what);
    if (t.scalar_type() != dt)
        throw py::type_error(std::string(what) + " must be " + dtype_str(dt) + ", got " +
                             dtype_str(t.scalar_type()));
    if (t.sizes() != shape)
        throw py::value_error(std::string(what) + " must have shape " + shape_str(shape) +
                              ", got " + shape_str(t.sizes()));
}

void check_w(const at::Tensor &w, int64_t N)
{
    check_dev(w, "w");
    if (w.dim() != 1 || w.size(0) != N)
        throw py::value_error("w must have shape (" + std::to_string(N) + ",), got " +
                              shape_str(w.sizes()));
}

// (M, N) of the rows of x: its last dimension is N
std::pair<int64_t, int64_t> rows(const at::Tensor &x)
{
    if (x.dim() < 1 || x.size(-1) == 0)
        throw py::value_error("input must have a non-empty last dimension");
    const int64_t N = x.size(-1);
    return {x.numel() / N, N};
}

at::Tensor stats_out(const at::Tensor &x, py::object given, bool want, const char *what)
{
    if (!given.is_none()) {
        at::Tensor t = given.cast<at::Tensor>();
        check_like(t, what, at::kFloat, x.sizes().slice(0, x.dim() - 1));
        return t;
    }
    if (want)
        return at::empty(x.sizes().slice(0, x.dim() - 1), x.options().dtype(at::kFloat));
    return at::Tensor();
}

[[noreturn]] void raise_status(int st, const char *what)
{
    py::object err = py::module_::import("add_rmsnorm_amd").attr("AddRmsError")(st, what);
    PyErr_SetObject(err.get_type().ptr(), err.ptr());
    throw py::error_already_set();
}

void *stream_of(const at::Tensor &x)
{
    return static_cast<void *>(c10::hip::getCurrentHIPStream(x.get_device()).stream());
}

py::object py_rmsnorm_fwd(const at::Tensor &x, const at::Tensor &w, double eps, py::object y_arg,
                          py::object rstd_arg, bool return_rstd)
{
    check_dev(x, "x");
    const auto [M, N] = rows(x);
    check_w(w, N);
    at::Tensor y;
    if (y_arg.is_none()) {
        y = at::empty_like(x);
    } else {
        y = y_arg.cast<at::Tensor>();
        check_like(y, "y", x.scalar_type(), x.sizes());
    }
    at::Tensor rstd = stats_out(x, rstd_arg, return_rstd, "rstd");
    const int dt = code_of(x, "x"), wdt = code_of(w, "w");
    int st;
    {
        c10::DeviceGuard guard(x.device());
        st = ::rmsnorm_fwd(x.data_ptr(), w.data_ptr(), y.data_ptr(),
                           rstd.defined() ? rstd.data_ptr<float>() : nullptr, M, N, (float)eps, dt,
                           wdt, stream_of(x));
    }
    if (st != 0)
        raise_status(st, "rmsnorm_fwd");
    if (rstd.defined())
        return py::make_tuple(y, rstd);
    return py::cast(y);
}

py::object py_add_rmsnorm_fwd(const at::Tensor &x, const at::Tensor &r, const at::Tensor &w,
                              double eps, py::object y_arg, py::object res_arg,
                              py::object rstd_arg, bool return_rstd)
{
    check_dev(x, "x");
    const auto [M, N] = rows(x);
    check_like(r, "r", x.scalar_type(), x.sizes());
    check_w(w, N);
    at::Tensor y, res;
    if (y_arg.is_none()) {
        y = at::empty_like(x);
    } else {
        y = y_arg.cast<at::Tensor>();
        check_like(y, "y", x.scalar_type(), x.sizes());
    }
    if (res_arg.is_none()) {
        res = at::empty_like(x);
    } else {
        res = res_arg.cast<at::Tensor>();
        check_like(res, "residual_out", x.scalar_type(), x.sizes());
    }
    at::Tensor rstd = stats_out(x, rstd_arg, return_rstd, "rstd");
    const int dt = code_of(x, "x"), wdt = code_of(w, "w");
    int st;
    {
        c10::DeviceGuard guard(x.device());
        st = ::add_rmsnorm_fwd(x.data_ptr(), r.data_ptr(), w.data_ptr(), y.data_ptr(),
                               res.data_ptr(), rstd.defined() ? rstd.data_ptr<float>() : nullptr, M,
                               N, (float)eps, dt, wdt, stream_of(x));
    }
    if (st != 0)
        raise_status(st, "add_rmsnorm_fwd");
    if (rstd.defined())
        return py::make_tuple(y, res, rstd);
    return py::make_tuple(y, res);
}

} // namespace

PYBIND11_MODULE(_native, m)
{
    m.doc() = "Native binding of the latency-bound forwards of libaddrms.so";
    m.def("rmsnorm_fwd", &py_rmsnorm_fwd, py::arg("x"), py::arg("w"), py::arg("eps") = 1e-6,
          py::kw_only(), py::arg("y") = py::none(), py::arg("rstd") = py::none(),
          py::arg("return_rstd") = false);
    m.def("add_rmsnorm_fwd", &py_add_rmsnorm_fwd, py::arg("x"), py::arg("r"), py::arg("w"),
          py::arg("eps") = 1e-6, py::kw_only(), py::arg("y") = py::none(),
          py::arg("residual_out") = py::none(), py::arg("rstd") = py::none(),
          py::arg("return_rstd") = false);
}
