// kv_prepare.hip -- the key (= value) vector of each compressed entry.
//
// [V4-Pro card, "Hybrid attention"]: RMSNorm on the single compressed KV
// head before the attention dot product, and RoPE on the last 64 dims of each
// KV entry.  Both depend on the entry alone -- its channels, gamma_kv and its
// position j*m + offset -- so they are applied once, when the entry enters
// the cache, and not on every attention call that reads it.
//
// Layout and schedule: one wave per entry row (prepare_row, shared with the
// streaming append so that both write bitwise the same rows).
#include "cakv_internal.hpp"
#include "cakv_rows.hpp"

namespace cakv {

template <typename T>
__global__ __launch_bounds__(256) void kv_prepare_kernel(const T* in, T* out,
                                                         const float* __restrict__ gamma, int64_t N, int D,
                                                         int64_t j0, int64_t n, int64_t rows, int m,
                                                         int rope_dims, double rope_ratio, int pos_off,
                                                         float eps) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const int64_t b = row / n, j = j0 + row % n;
    const int64_t off = (b * N + j) * (int64_t)D;
    prepare_row<T>(in + off, out + off, gamma, D, (double)(j * m + pos_off), rope_dims, rope_ratio, eps,
                   (int)(threadIdx.x & 63));
}

int launch_kv_prepare(const void* in, void* out, int dtype, int64_t B, int64_t N, int64_t D, int64_t j0,
                      int64_t n, const float* gamma, int32_t m, int32_t rope_dims, double rope_ratio,
                      int32_t pos_off, float eps, hipStream_t stream) {
    const int64_t rows = B * n;
    if (rows == 0) return 0;
    if (D > 64 * 8 * kPrepMaxChunks) return -2;
    const int64_t grid = (rows + 3) / 4;
    if (grid > 0x7fffffffLL) return -2;
    prof_mark("kv_prepare_kernel", false, stream);
    if (dtype == 0)
        hipLaunchKernelGGL((kv_prepare_kernel<float>), dim3((unsigned)grid), dim3(256), 0, stream,
                           (const float*)in, (float*)out, gamma, N, (int)D, j0, n, rows, m, rope_dims, rope_ratio,
                           pos_off, eps);
    else
        hipLaunchKernelGGL((kv_prepare_kernel<bf16_t>), dim3((unsigned)grid), dim3(256), 0, stream,
                           (const bf16_t*)in, (bf16_t*)out, gamma, N, (int)D, j0, n, rows, m, rope_dims,
                           rope_ratio, pos_off, eps);
    prof_mark("kv_prepare_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace cakv
