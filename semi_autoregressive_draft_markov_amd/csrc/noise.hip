// The random numbers of the drafting calls, exposed for checking against an
// independent implementation.  The pages sample x_k from p_k left to right
// (mainlymatmul "DSpark: Wait It's All Autoregressive?", "A parallel backbone
// with autoregressive sampling"; dormouse "DSpark - paper verification",
// section 1, Eq 4) but define no generator; the kernels draw Gumbel-max noise
// from Philox4x32-10 (Salmon et al., SC'11) with the counter layout the C ABI
// documents.  This file runs exactly the device routines the drafting and
// verification kernels call (device_common.h), one element per thread.
#include "device_common.h"
#include "internal.h"

namespace dspark {

__global__ __launch_bounds__(256) void k_noise(uint32_t key0, uint32_t key1, uint32_t ctr1, uint32_t ctr2,
                                               uint32_t ctr3, uint32_t v0, int n,
                                               const uint32_t* __restrict__ words_in, uint32_t* __restrict__ words,
                                               float* __restrict__ gumbel, float* __restrict__ gumbel2) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    uint32_t w;
    if (words_in) {
        w = words_in[i];
    } else {
        const uint32_t v = v0 + static_cast<uint32_t>(i);
        const u32x4 out = philox4x32_10(u32x4{v >> 2, ctr1, ctr2, ctr3}, key0, key1);
        const uint32_t q = v & 3u;
        w = q == 0 ? out[0] : q == 1 ? out[1] : q == 2 ? out[2] : out[3];
    }
    if (words) words[i] = w;
    if (gumbel) gumbel[i] = gumbel_from_word(w);
    if (gumbel2) gumbel2[i] = log2_of_neg_log2_uniform(w);
}

hipError_t launch_noise(uint64_t seed, uint64_t offset, uint32_t ctr1, uint32_t ctr2, uint32_t v0, int n,
                        const uint32_t* words_in, uint32_t* words, float* gumbel, float* gumbel2,
                        hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_noise, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t>(seed),
                       static_cast<uint32_t>(seed >> 32), ctr1, ctr2, static_cast<uint32_t>(offset), v0, n,
                       words_in, words, gumbel, gumbel2);
    return hipGetLastError();
}

}  // namespace dspark
