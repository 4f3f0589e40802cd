// norm.hip — batch-invariant RMSNorm for gfx950.
//
// y[t, k] = gamma[k] x[t, k] / sqrt(mean_k x[t, k]^2 + eps)
//
// The pages list RMSNorm among the kernels whose reduction must not depend
// on the batch ("训推一致性与 determinism", section 6 kernel table: a
// batch-invariant RMS with a fixed reduction; "Diagnosing Training
// Inference Mismatch ... (VeXact)", methodology: batch-invariant RMSNorm).
// Here one wave owns one row, whatever N is: lane l folds the squares of
// columns 8 (l + 64 i) + j, i ascending then j ascending, in fp64, and the
// 64 lane sums meet in a fixed butterfly.  The row's bits therefore depend
// on its own values and D only.  The normalised value is formed in fp64 and
// rounded once to the output type (bf16: nearest, ties to even), so the
// only rounding between the definition and the stored value is that last
// one.  The kernel is bound by HBM: it reads x (and gamma, from cache) and
// writes y once; the second read of a row comes from cache.

#include "tim_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace tim {
namespace {

constexpr int kNormWaves = 4;            // rows per workgroup
constexpr int kNormThreads = 64 * kNormWaves;

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
    return (double)__builtin_bit_cast(float, (uint32_t)b << 16);
}

// Nearest bf16 of a double, ties to even, from the double's own bits (no
// intermediate float rounding).  Normal range: round the 52-bit fraction at
// bit 45 (8 significant bits kept); the rounded value is then a float
// exactly, whose upper half is the bf16.  Below 2^-126 the bf16 grid is
// the fixed step 2^-133, and the bits are the step count.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7FC0u);           // NaN
    const double ax = __builtin_bit_cast(double, a);
    if (ax < 0x1p-126) {
        const double q = __builtin_rint(ax * 0x1p133);                           // 0..128
        return (uint16_t)(sign | (uint16_t)q);
    }
    const uint64_t lsb = (a >> 45) & 1ull;
    const uint64_t r = (a + 0x00000FFFFFFFFFFFull + lsb) & ~0x00001FFFFFFFFFFFull;
    const float f = (float)__builtin_bit_cast(double, r);                        // exact, or inf
    return (uint16_t)(sign | (uint16_t)((__builtin_bit_cast(uint32_t, f) >> 16) & 0x7FFFu));
}

template <bool kBf16>
__device__ __forceinline__ double load_x(const void* base, int64_t idx) {
    if constexpr (kBf16) return bf16_to_f64(((const uint16_t*)base)[idx]);
    else return (double)((const float*)base)[idx];
}

// Grid: ceil(n / kNormWaves) workgroups; wave w of workgroup b owns row
// 4 b + w.  kVec: rows and gamma are 16-byte aligned and d % 8 == 0, so
// eight bf16 (or two float4) of a lane's column group load at once; the
// arithmetic is the same either way.
template <bool kBf16, bool kVec>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(const void* __restrict__ x, int64_t ldx, const void* __restrict__ gamma, int64_t n,
               int64_t d, double eps, void* __restrict__ y, int64_t ldy,
               float* __restrict__ rstd_out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (t >= n) return;                                  // whole wave leaves together
    const int64_t groups = (d + 7) / 8;                  // 8-column groups of the row
    const int64_t xrow = t * ldx, yrow = t * ldy;

    auto load8 = [&](const void* base, int64_t off, int64_t c0, double (&v)[8]) {
        if constexpr (kVec) {
            if constexpr (kBf16) {
                const uint4 q = *(const uint4*)((const uint16_t*)base + off + c0);
                const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = bf16_to_f64((uint16_t)(w4[j] & 0xFFFFu));
                    v[2 * j + 1] = bf16_to_f64((uint16_t)(w4[j] >> 16));
                }
            } else {
                const float4 q0 = *(const float4*)((const float*)base + off + c0);
                const float4 q1 = *(const float4*)((const float*)base + off + c0 + 4);
                v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
                v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = c0 + j < d ? load_x<kBf16>(base, off + c0 + j) : 0.0;
        }
    };

    // sum of squares: lane order fixed (group i ascending, column j ascending)
    double ss = 0.0;
    for (int64_t g = lane; g < groups; g += 64) {
        double v[8];
        load8(x, xrow, g * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fma(v[j], v[j], ss);
    }
    // fixed butterfly: every lane ends with the same bits (a + b == b + a)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    if (rstd_out && lane == 0) rstd_out[t] = (float)r;

    for (int64_t g = lane; g < groups; g += 64) {
        double v[8], gm[8];
        load8(x, xrow, g * 8, v);
        load8(gamma, 0, g * 8, gm);
        const int64_t c0 = g * 8;
        if constexpr (kBf16) {
            uint16_t o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = f64_to_bf16_rne(gm[j] * (v[j] * r));
            if constexpr (kVec) {
                uint4 q;
                q.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                q.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                q.z = (uint32_t)o[4] | ((uint32_t)o[5] << 16);
                q.w = (uint32_t)o[6] | ((uint32_t)o[7] << 16);
                *(uint4*)((uint16_t*)y + yrow + c0) = q;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (c0 + j < d) ((uint16_t*)y)[yrow + c0 + j] = o[j];
            }
        } else {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = (float)(gm[j] * (v[j] * r));
            if constexpr (kVec) {
                *(float4*)((float*)y + yrow + c0) = make_float4(o[0], o[1], o[2], o[3]);
                *(float4*)((float*)y + yrow + c0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (c0 + j < d) ((float*)y)[yrow + c0 + j] = o[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* gamma, int64_t n, int64_t d,
                          int dtype, double eps, void* y, int64_t ldy, float* rstd,
                          hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + kNormWaves - 1) / kNormWaves;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const int64_t esz = dtype == 0 ? 2 : 4;
    const bool vec = d % 8 == 0 && (ldx * esz) % 16 == 0 && (ldy * esz) % 16 == 0 &&
                     ((uintptr_t)x % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     ((uintptr_t)gamma % 16) == 0;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kNormThreads), 0, st, x, ldx, gamma,
                           n, d, eps, y, ldy, rstd);
    };
    if (dtype == 0) {
        if (vec) go(rmsnorm_kernel<true, true>);
        else go(rmsnorm_kernel<true, false>);
    } else {
        if (vec) go(rmsnorm_kernel<false, true>);
        else go(rmsnorm_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace tim
