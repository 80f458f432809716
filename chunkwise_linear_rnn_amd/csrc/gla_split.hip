// Slice plumbing for heads wider than the kernels, and the small reshapes of the
// gate forms the kernels do not take directly.
//
// The recurrence of Section 4.1, Eq. 3 acts on each value column of the state
// independently (column j of S_t depends only on column j of v and of S_0), and
// its diagonal gate scales each state row on its own (row i depends only on
// column i of k and g, and o_t = q_t S_t sums over the rows).  A head with wide
// values is therefore several heads that share q, k and g, whose dv and dS_0
// sit side by side and whose dq, dk and dg (the closed form of Section 4.3 is
// linear in the per-slice terms) add; a head with wide keys is several heads
// that share v, whose outputs and dv add.  These kernels gather a slice's
// columns into contiguous buffers and scatter them back (gla_copy_cols), add a
// slice's result into another's (gla_add_into), pad 64-wide heads of the
// general gate to the kernels' 128 with zero columns (gla_pad_cols), repeat a
// scalar gate over the key columns for the fp32 path (gla_bcast_cols) and sum
// that path's per-column gate gradient back to one value per token
// (gla_row_sums).
#include <hip/hip_runtime.h>

#include "gla_device.hpp"
#include "gla_launch.hpp"
#include "gla_timing.hpp"

namespace gla {

// dst[r][off_d + c] = src[r][off_s + c] for c < W, r < rows; W, offsets and row
// strides in elements, all multiples of 16 bytes.
template <typename T>
__global__ void __launch_bounds__(256)
gla_copy_cols(const T* __restrict__ src, long ld_s, long off_s, T* __restrict__ dst, long ld_d, long off_d, long W,
              long rows) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const long per_row = W / VEC;
    const long n = rows * per_row;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const long r = i / per_row, c = (i % per_row) * VEC;
        *reinterpret_cast<u32x4*>(dst + r * ld_d + off_d + c) = *reinterpret_cast<const u32x4*>(src + r * ld_s + off_s + c);
    }
}

// a[i] = a[i] + b[i] in fp32, rounded once to T; n a multiple of 16 bytes' worth of T.
template <typename T>
__global__ void __launch_bounds__(256)
gla_add_into(T* __restrict__ a, const T* __restrict__ b, long n) {
    constexpr int VEC = 16 / (int)sizeof(T);
    for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * VEC; i < n; i += (long)gridDim.x * 256 * VEC) {
        u32x4 x = *reinterpret_cast<const u32x4*>(a + i);
        const u32x4 y = *reinterpret_cast<const u32x4*>(b + i);
        T* xv = reinterpret_cast<T*>(&x);
        const T* yv = reinterpret_cast<const T*>(&y);
#pragma unroll
        for (int e = 0; e < VEC; ++e) xv[e] = Elem<T>::from_f(Elem<T>::to_f(xv[e]) + Elem<T>::to_f(yv[e]));
        *reinterpret_cast<u32x4*>(a + i) = x;
    }
}

// dst[r][c] = c < W_src ? src[r][c] : 0 for c < W_dst (row strides ld_s, ld_d;
// all in elements, multiples of 16 bytes): zero padding of columns or row blocks.
template <typename T>
__global__ void __launch_bounds__(256)
gla_pad_cols(const T* __restrict__ src, long ld_s, long W_src, T* __restrict__ dst, long ld_d, long W_dst,
             long rows) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const long per_row = W_dst / VEC;
    const long n = rows * per_row;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const long r = i / per_row, c = (i % per_row) * VEC;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (c < W_src) x = *reinterpret_cast<const u32x4*>(src + r * ld_s + c);
        *reinterpret_cast<u32x4*>(dst + r * ld_d + c) = x;
    }
}

// dst[r][c] = src[r] for c < W (W a multiple of 4): a per-token gate repeated
// over the key columns.
__global__ void __launch_bounds__(256)
gla_bcast_cols(const float* __restrict__ src, float* __restrict__ dst, long W, long rows) {
    const long per_row = W / 4;
    const long n = rows * per_row;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        const float x = src[i / per_row];
        *reinterpret_cast<f32x4*>(dst + i * 4) = f32x4{x, x, x, x};
    }
}

// dst[r] = sum over c < W of src[r][c], in ascending c, in fp32.
__global__ void __launch_bounds__(256)
gla_row_sums(const float* __restrict__ src, long W, float* __restrict__ dst, long rows) {
    for (long r = (long)blockIdx.x * 256 + threadIdx.x; r < rows; r += (long)gridDim.x * 256) {
        const float* row = src + r * W;
        float acc = 0.f;
        for (long c = 0; c < W; c += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(row + c);
            acc += x[0];
            acc += x[1];
            acc += x[2];
            acc += x[3];
        }
        dst[r] = acc;
    }
}

static unsigned grid_for(long work) {
    const long g = (work + 255) / 256;
    return (unsigned)(g < 2048 ? (g > 0 ? g : 1) : 2048);
}

hipError_t launch_copy_cols(bool bf16, const void* src, long ld_s, long off_s, void* dst, long ld_d, long off_d, long W,
                            long rows, hipStream_t stream) {
    if (rows <= 0 || W <= 0) return hipSuccess;
    const int vec = bf16 ? 8 : 4;
    const unsigned g = grid_for(rows * (W / vec));
    if (bf16)
        GLA_LAUNCH("copy_cols", gla_copy_cols<__bf16>, dim3(g), dim3(256), stream, (const __bf16*)src, ld_s, off_s,
                   (__bf16*)dst, ld_d, off_d, W, rows);
    else
        GLA_LAUNCH("copy_cols", gla_copy_cols<float>, dim3(g), dim3(256), stream, (const float*)src, ld_s, off_s,
                   (float*)dst, ld_d, off_d, W, rows);
    return hipGetLastError();
}

hipError_t launch_add_into(bool bf16, void* a, const void* b, long n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (bf16)
        GLA_LAUNCH("add_halves", gla_add_into<__bf16>, dim3(grid_for(n / 8)), dim3(256), stream, (__bf16*)a,
                   (const __bf16*)b, n);
    else
        GLA_LAUNCH("add_halves", gla_add_into<float>, dim3(grid_for(n / 4)), dim3(256), stream, (float*)a,
                   (const float*)b, n);
    return hipGetLastError();
}

hipError_t launch_pad_cols(bool bf16, const void* src, long ld_s, long W_src, void* dst, long ld_d, long W_dst,
                           long rows, hipStream_t stream) {
    if (rows <= 0 || W_dst <= 0) return hipSuccess;
    const int vec = bf16 ? 8 : 4;
    const unsigned g = grid_for(rows * (W_dst / vec));
    if (bf16)
        GLA_LAUNCH("pad_cols", gla_pad_cols<__bf16>, dim3(g), dim3(256), stream, (const __bf16*)src, ld_s, W_src,
                   (__bf16*)dst, ld_d, W_dst, rows);
    else
        GLA_LAUNCH("pad_cols", gla_pad_cols<float>, dim3(g), dim3(256), stream, (const float*)src, ld_s, W_src,
                   (float*)dst, ld_d, W_dst, rows);
    return hipGetLastError();
}

hipError_t launch_bcast_cols(const float* src, float* dst, long W, long rows, hipStream_t stream) {
    if (rows <= 0 || W <= 0) return hipSuccess;
    GLA_LAUNCH("bcast_gate", gla_bcast_cols, dim3(grid_for(rows * (W / 4))), dim3(256), stream, src, dst, W, rows);
    return hipGetLastError();
}

hipError_t launch_row_sums(const float* src, long W, float* dst, long rows, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    GLA_LAUNCH("gate_row_sums", gla_row_sums, dim3(grid_for(rows)), dim3(256), stream, src, W, dst, rows);
    return hipGetLastError();
}

}  // namespace gla
