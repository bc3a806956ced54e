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
//                                size_t bytes_each, int shape, void *stream);
//   bytes_each: size of each of the four device buffers, a multiple of 16.
//   shape: 0 = 256-thread blocks, 4 vectors a lane per stream (16 KiB per
//   block and stream); 1 = 512-thread blocks, 2 vectors a lane (the same
//   bytes per block with 8 waves, the row kernels' shape).  Of the shapes
//   swept on MI355X these two stream fastest (6.1-6.3 TB/s); the benchmark
//   reports the better one.
//   Returns the hipError_t of the launch (0 on success).
#include <hip/hip_runtime.h>

#include "device.hpp"

namespace {

using addrms::u32x4;

template <int B, int kUnroll>
__global__ void __launch_bounds__(B)
stream_2r2w_kernel(const u32x4 *a, const u32x4 *b, u32x4 *c, u32x4 *d, size_t n)
{
    const size_t stride = (size_t)gridDim.x * B * kUnroll;
    for (size_t base = (size_t)blockIdx.x * B * kUnroll + threadIdx.x; base < n; base += stride) {
        u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * B;
            if (i < n) {
                va[u] = addrms::ld_stream<3>(a + i);
                vb[u] = addrms::ld_stream<3>(b + i);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * B;
            if (i < n) {
                addrms::st_stream<3>(c + i, va[u] + vb[u]);
                addrms::st_stream<3>(d + i, va[u] ^ vb[u]);
            }
        }
    }
}

template <int B, int U>
hipError_t launch_probe(const void *a, const void *b, void *c, void *d, size_t n, hipStream_t s)
{
    const size_t blocks = (n + B * U - 1) / (B * U);
    const unsigned grid = (unsigned)(blocks < 0x7fffffffu ? (blocks ? blocks : 1) : 0x7fffffffu);
    hipLaunchKernelGGL((stream_2r2w_kernel<B, U>), dim3(grid), dim3(B), 0, s,
                       static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b),
                       static_cast<u32x4 *>(c), static_cast<u32x4 *>(d), n);
    return hipGetLastError();
}

} // namespace

extern "C" int addrms_probe_stream_2r2w(const void *a, const void *b, void *c, void *d,
                                        size_t bytes_each, int shape, void *stream)
{
    if (!a || !b || !c || !d || bytes_each % 16 != 0 || shape < 0 || shape > 1)
        return (int)hipErrorInvalidValue;
    const size_t n = bytes_each / 16;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return (int)(shape == 0 ? launch_probe<256, 4>(a, b, c, d, n, s) : launch_probe<512, 2>(a, b, c, d, n, s));
}
