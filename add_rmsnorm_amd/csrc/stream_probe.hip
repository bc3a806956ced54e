// Measurement aid for the benchmark, built as its own small library
// (libaddrms_probe.so) and never linked into libaddrms.so.
//
// The fused forward reads two streams and writes two.  This kernel does only
// that -- c = a + b, d = a ^ b on 16-byte vectors, with the same 128-bit
// non-temporal accesses as the row kernels and no reduction -- so its
// bandwidth is the practical ceiling of that access mix on the device, which
// the benchmark reports beside the 8 TB/s nominal peak.
//
//   int addrms_probe_stream_2r2w(const void *a, const void *b, void *c, void *d,
//                                size_t bytes_each, void *stream);
//   bytes_each: size of each of the four device buffers, a multiple of 16.
//   Returns the hipError_t of the launch (0 on success).
#include <hip/hip_runtime.h>

#include "device.hpp"

namespace {

using addrms::u32x4;
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(256)
stream_2r2w_kernel(const u32x4 *a, const u32x4 *b, u32x4 *c, u32x4 *d, size_t n)
{
    const size_t stride = (size_t)gridDim.x * 256 * kUnroll;
    for (size_t base = (size_t)blockIdx.x * 256 * kUnroll + threadIdx.x; base < n; base += stride) {
        u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n) {
                va[u] = addrms::ld_stream<3>(a + i);
                vb[u] = addrms::ld_stream<3>(b + i);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * 256;
            if (i < n) {
                addrms::st_stream<3>(c + i, va[u] + vb[u]);
                addrms::st_stream<3>(d + i, va[u] ^ vb[u]);
            }
        }
    }
}

} // namespace

extern "C" int addrms_probe_stream_2r2w(const void *a, const void *b, void *c, void *d,
                                        size_t bytes_each, void *stream)
{
    if (!a || !b || !c || !d || bytes_each % 16 != 0)
        return (int)hipErrorInvalidValue;
    const size_t n = bytes_each / 16;
    const size_t blocks = (n + 256 * kUnroll - 1) / (256 * kUnroll);
    const unsigned grid = (unsigned)(blocks < 0x7fffffffu ? (blocks ? blocks : 1) : 0x7fffffffu);
    hipLaunchKernelGGL(stream_2r2w_kernel, dim3(grid), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4 *>(a),
                       static_cast<const u32x4 *>(b), static_cast<u32x4 *>(c), static_cast<u32x4 *>(d), n);
    return (int)hipGetLastError();
}
