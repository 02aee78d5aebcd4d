// Column padding and cropping of row-major [rows, d] tensors: the attention
// kernels are built for head dims 32, 64 and 128; any other head dim up to 128
// runs them on copies widened with zero columns to the next of those sizes.
// Zero columns of q and k add nothing to any q . k, and zero columns of v only
// produce output columns that are cropped away, so the padded problem has the
// same softmax and the same results (dq, dk, dv likewise). Bit copy.
#include "fa2_launch.h"

namespace fa2mi {

namespace {

constexpr int kColsRowsPerBlock = kPadColsRowsPerBlock;

// dst[r][c] = src[r][c] for c < d_src, 0 for d_src <= c < d_dst; each
// workgroup moves kColsRowsPerBlock consecutive rows, which are contiguous on
// both sides, with consecutive threads on consecutive destination elements.
template <typename T>
__global__ __launch_bounds__(256) void pad_cols_kernel(const T *__restrict__ src, T *__restrict__ dst, int64_t rows,
                                                       int d_src, int d_dst) {
    const int64_t row0 = (int64_t)blockIdx.x * kColsRowsPerBlock;
    const int nrow = (int)min<int64_t>(kColsRowsPerBlock, rows - row0);
    const T *s = src + row0 * d_src;
    T *d = dst + row0 * d_dst;
    for (int idx = threadIdx.x; idx < nrow * d_dst; idx += 256) {
        const int r = idx / d_dst, c = idx - r * d_dst;
        d[idx] = c < d_src ? s[r * d_src + c] : T(0);
    }
}

}  // namespace

hipError_t launch_pad_cols(int dt, const void *src, void *dst, int64_t rows, int d_src, int d_dst,
                           hipStream_t stream) {
    const unsigned grid = (unsigned)((rows + kColsRowsPerBlock - 1) / kColsRowsPerBlock);
    if (dt == 0)
        hipLaunchKernelGGL(pad_cols_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream, (const uint32_t *)src,
                           (uint32_t *)dst, rows, d_src, d_dst);
    else
        hipLaunchKernelGGL(pad_cols_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, (const uint16_t *)src,
                           (uint16_t *)dst, rows, d_src, d_dst);
    return hipGetLastError();
}

}  // namespace fa2mi
