// ssd_pad.hip -- zero-padding copies that let the prefill serve any head dimension P and
// state dimension N that are multiples of 16: the inputs are copied into the caller's
// workspace with P and N padded to the next size the kernels are built for (zero channels
// of x and z, zero state columns of B, C and the initial state), the prefill runs on the
// padded problem, and y and the final state are copied back without the padding.  Zero
// channels and zero state columns add exact zeros to every sum of the method, so the
// caller's part of the result is the unpadded problem's ("Mamba-Family State-Space Model
// Kernels on a Programmable CGLA", Sec. III-A: each channel p of the state evolves on its
// own; the output contracts the state with C over N).
#include "ssd_common.h"
#include "ssd_launch.h"

namespace ssd {

// dst[(o * nin_dst + i) * dlen + k] = (i < nin_src && k < slen) ? src[o * so + i * si + k * sk] : 0
// for o < nout, i < nin_dst, k < dlen (sk = 0 repeats one source element dlen times).
template <typename T>
__global__ __launch_bounds__(256) void pad_copy_kernel(const T *__restrict__ src, T *__restrict__ dst, long long nout,
                                                      int nin_src, int nin_dst, int slen, int dlen, long long so,
                                                      long long si, long long sk)
{
    const long long total = nout * nin_dst * dlen;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
        const int k = (int)(e % dlen);
        const long long oi = e / dlen;
        const int i = (int)(oi % nin_dst);
        const long long o = oi / nin_dst;
        T v = T(0);
        if (i < nin_src && k < slen) v = src[o * so + i * si + k * sk];
        dst[e] = v;
    }
}

hipError_t launch_pad_copy(const void *src, void *dst, int elem_bytes, long long nout, int nin_src, int nin_dst,
                           int slen, int dlen, long long so, long long si, long long sk, hipStream_t s)
{
    const long long total = nout * nin_dst * dlen;
    if (total <= 0) return hipSuccess;
    const long long want = (total + 255) / 256;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    if (elem_bytes == 1)  // fp8 e4m3 codes (the zero code is +0)
        launch_kernel("pad_copy_kernel", pad_copy_kernel<uint8_t>, grid, 256, s, static_cast<const uint8_t *>(src),
                      static_cast<uint8_t *>(dst), nout, nin_src, nin_dst, slen, dlen, so, si, sk);
    else if (elem_bytes == 2)
        launch_kernel("pad_copy_kernel", pad_copy_kernel<uint16_t>, grid, 256, s,
                      static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), nout, nin_src, nin_dst,
                      slen, dlen, so, si, sk);
    else if (elem_bytes == 4)
        launch_kernel("pad_copy_kernel", pad_copy_kernel<uint32_t>, grid, 256, s,
                      static_cast<const uint32_t *>(src), static_cast<uint32_t *>(dst), nout, nin_src, nin_dst,
                      slen, dlen, so, si, sk);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ssd
