// Measurement aid for the benchmark, built as its own small library
// (libaddrms_probe.so) and never linked into libaddrms.so.
//
// The fused forward reads two streams and writes two; the backwards read two
// or three and write one.  These kernels do only the streaming -- no
// reduction, one or two integer ops per 16-byte vector -- so their bandwidth
// is the practical ceiling of each access mix on the device, against which
// the row kernels are measured.  The matrix covers:
//   * the access mix: 1 or 2 read-only streams, 1 or 2 write-only streams,
//     1R1W, 2R1W, 2R2W (the fused forward), 3R1W (the fused backward);
//   * the launch shape: threads per block and 16-byte vectors per lane, one
//     block per chunk (as the row kernels launch), so a block reads its
//     whole chunk and then writes it (the read/write phase granularity);
//   * the cache policy of loads and stores (buffer instructions with the
//     sc0, sc1 and nt bits set per variant);
//   * loads through LDS (global_load_lds_dwordx4: the data goes straight to
//     LDS, so a lane keeps more bytes in flight without holding registers);
//   * a persistent grid whose blocks issue the next chunk's loads before the
//     current chunk's stores (software pipelining);
//   * persistent grids with a fixed share of chunks per block (on the grid
//     that fits at once, or 2 or 4 times it), against ones whose blocks take
//     chunks from a work counter;
//   * in-place outputs (the host passes the input buffers as outputs).
//
//   int   addrms_probe_count(void);
//   const char *addrms_probe_name(int id);          static string
//   int   addrms_probe_streams(int id, int *nin, int *nout, int *needs_counter);
//   int   addrms_probe_run(int id, const void *const *in, void *const *out,
//                          size_t bytes_each, unsigned *counter, void *stream);
//     in: nin device buffers of bytes_each bytes (read); out: nout device
//     buffers of bytes_each bytes (written); a read-only probe takes one
//     output buffer of at least 16 bytes as a sink, written only if the data
//     xor to an impossible value.  bytes_each: a multiple of 16, below 4 GiB.
//     counter: a device word that is zero at launch, for the probes that take
//     chunks from a work counter (needs_counter); ignored by the others.
//     Returns the hipError_t of the launch (0 on success), or
//     hipErrorInvalidValue for bad arguments.
//   int   addrms_probe_floor(int kind, const void *in, void *out, void *stream);
//     The launch floor of a one-row call (the decode shapes): kind 0, an empty
//     kernel of one 64-thread block; kind 1, one 1024-thread block that copies
//     16 KiB (one 16-byte vector a thread) from in to out, each of at least
//     16 KiB.  Same return convention.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "device.hpp"

namespace {

using addrms::u32x4;

struct PArgs {
    const u32x4 *in[3];
    u32x4 *out[2];
    size_t n; // 16-byte vectors per stream
};

// Cache-policy bits of the buffer instructions (the aux operand): 1 = sc0,
// 2 = nt, 16 = sc1.  Policy -1 selects the global instructions the row
// kernels use, non-temporal (global_load/store_dwordx4 ... nt).
constexpr int kGlobalNt = -1;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, size_t n)
{
    // raw buffer, no stride; 0x00020000: 32-bit data format, the value used
    // for untyped buffer access on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)(n * 16), 0x00020000);
}

template <int POL>
__device__ __forceinline__ u32x4 ld(const u32x4 *base, size_t n, size_t i)
{
    if constexpr (POL == kGlobalNt) {
        return __builtin_nontemporal_load(base + i);
    } else {
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, n), (int)(i * 16), 0, POL);
    }
}

template <int POL>
__device__ __forceinline__ void st(u32x4 *base, size_t n, size_t i, const u32x4 &v)
{
    if constexpr (POL == kGlobalNt) {
        __builtin_nontemporal_store(v, base + i);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base, n), (int)(i * 16), 0, POL);
    }
}

// Output w of the values read: the sum and the xor of the inputs (a write-only
// probe writes the vector index).
template <int NR>
__device__ __forceinline__ u32x4 out_val(const u32x4 (&v)[NR > 0 ? NR : 1], int w, size_t i)
{
    if constexpr (NR == 0) {
        const unsigned k = (unsigned)i;
        return u32x4{k, k ^ 1u, k ^ 2u, k ^ 3u} + (unsigned)w;
    } else {
        u32x4 s = v[0], x = v[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) {
            s += v[r];
            x ^= v[r];
        }
        return w == 0 ? s : x;
    }
}

// One block per chunk of B * U vectors of each stream: every load of the
// chunk, then every store.
template <int NR, int NW, int B, int U, int LP, int SP>
__global__ void __launch_bounds__(B) mix_kernel(PArgs a, unsigned *)
{
    const size_t base = (size_t)blockIdx.x * B * U + threadIdx.x;
    u32x4 v[U][NR > 0 ? NR : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * B;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            v[u][r] = i < a.n ? ld<LP>(a.in[r], a.n, i) : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (NW == 0) {
        u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r)
                acc ^= v[u][r];
        // inputs hold small values, so the top bits of the xor are clear
        if ((acc[0] & acc[1] & acc[2] & acc[3]) == 0xFFFFFFFFu)
            a.out[0][0] = acc;
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * B;
            if (i < a.n) {
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    st<SP>(a.out[w], a.n, i, out_val<NR>(v[u], w, i));
            }
        }
    }
}

// 2R2W with the loads going straight to LDS (global_load_lds_dwordx4, nt):
// a wave's 64 lanes fill 1 KiB of LDS per instruction, lane l at byte 16*l of
// the wave's region; after every load of the chunk has landed, each lane
// reads its own vectors back and stores them.
template <int B, int U>
__global__ void __launch_bounds__(B) lds_kernel(PArgs a, unsigned *)
{
    __shared__ u32x4 buf[2][U][B];
    const int wbase = threadIdx.x & ~63;
    const size_t base = (size_t)blockIdx.x * B * U + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * B;
        if (i < a.n) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
                __builtin_amdgcn_global_load_lds(
                    (const void *)(a.in[r] + i),
                    (__attribute__((address_space(3))) void *)&buf[r][u][wbase], 16, 0, 2);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * B;
        if (i < a.n) {
            const u32x4 x = buf[0][u][threadIdx.x], y = buf[1][u][threadIdx.x];
            __builtin_nontemporal_store(x + y, a.out[0] + i);
            __builtin_nontemporal_store(x ^ y, a.out[1] + i);
        }
    }
}

// 2R2W on a persistent grid: a block walks chunks of B * U vectors with a
// grid stride and issues the next chunk's loads before the current chunk's
// stores, so reads stay in flight while it writes.
template <int B, int U>
__global__ void __launch_bounds__(B) pipe_kernel(PArgs a, unsigned *)
{
    const size_t chunk = (size_t)B * U;
    const size_t nchunks = (a.n + chunk - 1) / chunk;
    u32x4 cur[U][2], nxt[U][2];
    auto load = [&](size_t c, u32x4 (&v)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
#pragma unroll
            for (int r = 0; r < 2; ++r)
                v[u][r] = i < a.n ? __builtin_nontemporal_load(a.in[r] + i) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    size_t c = blockIdx.x;
    if (c < nchunks)
        load(c, cur);
    for (; c < nchunks; c += gridDim.x) {
        if (c + gridDim.x < nchunks)
            load(c + gridDim.x, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
            if (i < a.n) {
                __builtin_nontemporal_store(cur[u][0] + cur[u][1], a.out[0] + i);
                __builtin_nontemporal_store(cur[u][0] ^ cur[u][1], a.out[1] + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            cur[u][0] = nxt[u][0];
            cur[u][1] = nxt[u][1];
        }
    }
}

// NR reads and NW writes on a persistent grid (as many blocks as fit at once),
// a chunk of B * U vectors per step.  QUEUE = false: block b takes chunks b,
// b + grid, b + 2 grid, ... (a fixed share, as the backward's persistent grid
// does).  QUEUE = true: each step's chunk is the next ticket of a global
// counter (a vector-memory atomic; *ctr is zero at launch), so blocks on
// faster CUs take more chunks, as the hardware dispatcher balances a grid of
// one block per chunk.  Every block leaves once the tickets pass the chunk
// count.
template <int NR, int NW, int B, int U, bool QUEUE>
__global__ void __launch_bounds__(B) pers_kernel(PArgs a, unsigned *ctr)
{
    __shared__ unsigned ticket;
    const size_t chunk = (size_t)B * U;
    const size_t nchunks = (a.n + chunk - 1) / chunk;
    size_t c = blockIdx.x;
    for (;;) {
        if constexpr (QUEUE) {
            if (threadIdx.x == 0)
                ticket = atomicAdd(ctr, 1u);
            __syncthreads();
            c = ticket;
            __syncthreads(); // every lane has read the ticket before the next is written
        }
        if (c >= nchunks)
            break;
        u32x4 v[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                v[u][r] = i < a.n ? __builtin_nontemporal_load(a.in[r] + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
            if (i < a.n) {
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    __builtin_nontemporal_store(out_val<NR>(v[u], w, i), a.out[w] + i);
            }
        }
        if constexpr (!QUEUE)
            c += gridDim.x;
    }
}

// As pers_kernel with QUEUE, but the next chunk's ticket is requested at the
// start of the current step, so the atomic's round trip overlaps the loads;
// thread 0 publishes it through LDS at the step's one barrier.  The first
// chunk of block b is b; tickets count on from gridDim.x.
template <int NR, int NW, int B, int U>
__global__ void __launch_bounds__(B) queue2_kernel(PArgs a, unsigned *ctr)
{
    __shared__ unsigned slot[2];
    const size_t chunk = (size_t)B * U;
    const size_t nchunks = (a.n + chunk - 1) / chunk;
    size_t c = blockIdx.x;
    for (int it = 0; c < nchunks; ++it) {
        unsigned nxt = 0;
        if (threadIdx.x == 0)
            nxt = gridDim.x + atomicAdd(ctr, 1u);
        u32x4 v[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                v[u][r] = i < a.n ? __builtin_nontemporal_load(a.in[r] + i) : u32x4{0u, 0u, 0u, 0u};
        }
        if (threadIdx.x == 0)
            slot[it & 1] = nxt;
        __syncthreads(); // slot[it & 1] is rewritten two steps later, after another barrier
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = c * chunk + threadIdx.x + (size_t)u * B;
            if (i < a.n) {
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    __builtin_nontemporal_store(out_val<NR>(v[u], w, i), a.out[w] + i);
            }
        }
        c = slot[it & 1];
    }
}

struct Probe {
    const char *name;
    const void *fn;
    int block;
    int per_block; // vectors of each stream per block (chunk)
    int nin, nout;
    bool persistent;
    bool queue;     // needs a zeroed counter
    int oversub = 1; // persistent grids: this many times the blocks that fit at once
};

#define MIX(NR, NW, B, U, LP, SP, NAME) \
    Probe{NAME, reinterpret_cast<const void *>(&mix_kernel<NR, NW, B, U, LP, SP>), B, B * U, NR, NW, false, false}
#define PERS(NR, NW, B, U, Q, NAME) \
    Probe{NAME, reinterpret_cast<const void *>(&pers_kernel<NR, NW, B, U, Q>), B, B * U, NR, NW, true, Q}

constexpr int G = kGlobalNt;

const Probe kProbes[] = {
    // access mix, global nt loads and stores, the two shapes the row kernels use
    MIX(1, 0, 256, 4, G, G, "r1_b256_u4"),
    MIX(1, 0, 512, 2, G, G, "r1_b512_u2"),
    MIX(2, 0, 256, 4, G, G, "r2_b256_u4"),
    MIX(2, 0, 512, 2, G, G, "r2_b512_u2"),
    MIX(0, 1, 256, 4, G, G, "w1_b256_u4"),
    MIX(0, 1, 512, 2, G, G, "w1_b512_u2"),
    MIX(0, 2, 256, 4, G, G, "w2_b256_u4"),
    MIX(0, 2, 512, 2, G, G, "w2_b512_u2"),
    MIX(1, 1, 256, 4, G, G, "r1w1_b256_u4"),
    MIX(1, 1, 512, 2, G, G, "r1w1_b512_u2"),
    MIX(2, 1, 256, 4, G, G, "r2w1_b256_u4"),
    MIX(2, 1, 512, 2, G, G, "r2w1_b512_u2"),
    MIX(2, 2, 256, 4, G, G, "r2w2_b256_u4"),
    MIX(2, 2, 512, 2, G, G, "r2w2_b512_u2"),
    MIX(3, 1, 256, 4, G, G, "r3w1_b256_u4"),
    MIX(3, 1, 512, 2, G, G, "r3w1_b512_u2"),
    // 2R2W read/write phase granularity: vectors a lane loads before storing
    MIX(2, 2, 256, 1, G, G, "r2w2_b256_u1"),
    MIX(2, 2, 256, 2, G, G, "r2w2_b256_u2"),
    MIX(2, 2, 256, 8, G, G, "r2w2_b256_u8"),
    MIX(2, 2, 512, 1, G, G, "r2w2_b512_u1"),
    MIX(2, 2, 512, 4, G, G, "r2w2_b512_u4"),
    MIX(2, 2, 1024, 1, G, G, "r2w2_b1024_u1"),
    MIX(2, 2, 1024, 2, G, G, "r2w2_b1024_u2"),
    // 2R2W cache policy (buffer instructions): loads nt; stores none, sc0,
    // sc1, nt, sc0|nt, sc1|nt, sc0|sc1|nt
    MIX(2, 2, 512, 2, 2, 0, "r2w2_b512_u2_ld-nt_st-none"),
    MIX(2, 2, 512, 2, 2, 1, "r2w2_b512_u2_ld-nt_st-sc0"),
    MIX(2, 2, 512, 2, 2, 16, "r2w2_b512_u2_ld-nt_st-sc1"),
    MIX(2, 2, 512, 2, 2, 2, "r2w2_b512_u2_ld-nt_st-nt"),
    MIX(2, 2, 512, 2, 2, 3, "r2w2_b512_u2_ld-nt_st-sc0nt"),
    MIX(2, 2, 512, 2, 2, 18, "r2w2_b512_u2_ld-nt_st-sc1nt"),
    MIX(2, 2, 512, 2, 2, 19, "r2w2_b512_u2_ld-nt_st-sc0sc1nt"),
    MIX(2, 2, 512, 2, 0, 2, "r2w2_b512_u2_ld-none_st-nt"),
    MIX(2, 2, 512, 2, 16, 2, "r2w2_b512_u2_ld-sc1_st-nt"),
    // write-only cache policy
    MIX(0, 2, 512, 2, G, 0, "w2_b512_u2_st-none"),
    MIX(0, 2, 512, 2, G, 16, "w2_b512_u2_st-sc1"),
    MIX(0, 2, 512, 2, G, 18, "w2_b512_u2_st-sc1nt"),
    MIX(0, 2, 512, 2, G, 19, "w2_b512_u2_st-sc0sc1nt"),
    // 2R2W with loads through LDS
    Probe{"r2w2_lds_b256_u4", reinterpret_cast<const void *>(&lds_kernel<256, 4>), 256, 1024, 2, 2, false, false},
    Probe{"r2w2_lds_b256_u8", reinterpret_cast<const void *>(&lds_kernel<256, 8>), 256, 2048, 2, 2, false, false},
    Probe{"r2w2_lds_b512_u2", reinterpret_cast<const void *>(&lds_kernel<512, 2>), 512, 1024, 2, 2, false, false},
    Probe{"r2w2_lds_b512_u4", reinterpret_cast<const void *>(&lds_kernel<512, 4>), 512, 2048, 2, 2, false, false},
    // 2R2W, persistent, next chunk's loads before the current chunk's stores
    Probe{"r2w2_pipe_b256_u2", reinterpret_cast<const void *>(&pipe_kernel<256, 2>), 256, 512, 2, 2, true, false},
    Probe{"r2w2_pipe_b256_u4", reinterpret_cast<const void *>(&pipe_kernel<256, 4>), 256, 1024, 2, 2, true, false},
    Probe{"r2w2_pipe_b512_u2", reinterpret_cast<const void *>(&pipe_kernel<512, 2>), 512, 1024, 2, 2, true, false},
    // persistent grids: a fixed share of chunks per block, or chunks taken
    // from a work counter (the backwards' mixes and the forward's)
    PERS(2, 1, 256, 4, false, "r2w1_pers_b256_u4"),
    PERS(2, 1, 256, 4, true, "r2w1_queue_b256_u4"),
    PERS(2, 1, 512, 2, false, "r2w1_pers_b512_u2"),
    PERS(2, 1, 512, 2, true, "r2w1_queue_b512_u2"),
    PERS(2, 2, 512, 2, false, "r2w2_pers_b512_u2"),
    PERS(2, 2, 512, 2, true, "r2w2_queue_b512_u2"),
    PERS(3, 1, 512, 2, false, "r3w1_pers_b512_u2"),
    PERS(3, 1, 512, 2, true, "r3w1_queue_b512_u2"),
    // the fixed share on 2 and 4 times the resident grid (the dispatcher
    // balances whole blocks), and the work counter with its ticket requested
    // a step ahead
    Probe{"r2w1_pers2x_b512_u2", reinterpret_cast<const void *>(&pers_kernel<2, 1, 512, 2, false>),
          512, 1024, 2, 1, true, false, 2},
    Probe{"r2w1_pers4x_b512_u2", reinterpret_cast<const void *>(&pers_kernel<2, 1, 512, 2, false>),
          512, 1024, 2, 1, true, false, 4},
    Probe{"r2w1_pers4x_b1024_u1", reinterpret_cast<const void *>(&pers_kernel<2, 1, 1024, 1, false>),
          1024, 1024, 2, 1, true, false, 4},
    Probe{"r2w1_queue2_b512_u2", reinterpret_cast<const void *>(&queue2_kernel<2, 1, 512, 2>), 512,
          1024, 2, 1, true, true},
    Probe{"r2w1_queue2_b256_u4", reinterpret_cast<const void *>(&queue2_kernel<2, 1, 256, 4>), 256,
          1024, 2, 1, true, true},
    Probe{"r3w1_queue2_b512_u2", reinterpret_cast<const void *>(&queue2_kernel<3, 1, 512, 2>), 512,
          1024, 3, 1, true, true},
    Probe{"r2w2_queue2_b512_u2", reinterpret_cast<const void *>(&queue2_kernel<2, 2, 512, 2>), 512,
          1024, 2, 2, true, true},
};
constexpr int kNumProbes = (int)(sizeof(kProbes) / sizeof(kProbes[0]));

} // namespace

__global__ void __launch_bounds__(64) floor_empty_kernel() {}

__global__ void __launch_bounds__(1024) floor_row_kernel(const u32x4 *in, u32x4 *out)
{
    out[threadIdx.x] = __builtin_nontemporal_load(in + threadIdx.x);
}

extern "C" {

int addrms_probe_floor(int kind, const void *in, void *out, void *stream)
{
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (kind == 0) {
        void *argv[] = {nullptr};
        return (int)hipLaunchKernel(reinterpret_cast<const void *>(&floor_empty_kernel), dim3(1),
                                    dim3(64), argv, 0, s);
    }
    if (kind != 1 || !in || !out)
        return (int)hipErrorInvalidValue;
    const u32x4 *pi = static_cast<const u32x4 *>(in);
    u32x4 *po = static_cast<u32x4 *>(out);
    void *argv[] = {&pi, &po};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&floor_row_kernel), dim3(1),
                                dim3(1024), argv, 0, s);
}

int addrms_probe_count(void) { return kNumProbes; }

const char *addrms_probe_name(int id) { return id >= 0 && id < kNumProbes ? kProbes[id].name : ""; }

int addrms_probe_streams(int id, int *nin, int *nout, int *needs_counter)
{
    if (id < 0 || id >= kNumProbes || !nin || !nout || !needs_counter)
        return (int)hipErrorInvalidValue;
    *nin = kProbes[id].nin;
    *nout = kProbes[id].nout;
    *needs_counter = kProbes[id].queue ? 1 : 0;
    return 0;
}

int addrms_probe_run(int id, const void *const *in, void *const *out, size_t bytes_each,
                     unsigned *counter, void *stream)
{
    if (id < 0 || id >= kNumProbes || bytes_each == 0 || bytes_each % 16 != 0 ||
        bytes_each >= ((size_t)1 << 32))
        return (int)hipErrorInvalidValue;
    const Probe &p = kProbes[id];
    if (p.queue && !counter)
        return (int)hipErrorInvalidValue;
    PArgs a{};
    for (int r = 0; r < p.nin; ++r) {
        if (!in || !in[r])
            return (int)hipErrorInvalidValue;
        a.in[r] = static_cast<const u32x4 *>(in[r]);
    }
    // a read-only probe writes at most one vector of its sink
    const int nout = p.nout > 0 ? p.nout : 1;
    for (int w = 0; w < nout; ++w) {
        if (!out || !out[w])
            return (int)hipErrorInvalidValue;
        a.out[w] = static_cast<u32x4 *>(out[w]);
    }
    a.n = bytes_each / 16;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    size_t blocks = (a.n + p.per_block - 1) / p.per_block;
    if (p.persistent) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, p.fn, p.block, 0);
        if (e != hipSuccess)
            return (int)e;
        const size_t cap = (size_t)cus * (size_t)(per_cu > 0 ? per_cu : 1) * (size_t)p.oversub;
        if (blocks > cap)
            blocks = cap;
    }
    void *argv[] = {&a, &counter};
    return (int)hipLaunchKernel(p.fn, dim3((unsigned)blocks), dim3(p.block), argv, 0, s);
}

} // extern "C"
