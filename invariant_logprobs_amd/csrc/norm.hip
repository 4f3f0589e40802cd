// norm.hip — batch-invariant RMSNorm for gfx950.
//
// y[t, k] = gamma[k] x[t, k] / sqrt(mean_k x[t, k]^2 + eps)
//
// The pages list RMSNorm among the kernels whose reduction must not depend
// on the batch ("训推一致性与 determinism", section 6 kernel table: a
// batch-invariant RMS with a fixed reduction; "Diagnosing Training
// Inference Mismatch ... (VeXact)", methodology: batch-invariant RMSNorm).
// Here one wave owns one row, whatever N is, and reduces it in an order
// fixed by d alone (below).  The row's bits therefore depend
// on its own values and D only.  The normalised value is formed in fp64 and
// rounded once to the output type (bf16: nearest, ties to even), so the
// only rounding between the definition and the stored value is that last
// one.  Work per element: one fp64 fold, two fp64 products, one conversion
// and three integer steps for the rounding.  Rows of up to 4096 elements
// (8192 in bf16) are held in registers and read once; wider rows are read
// twice (the second time mostly from cache).  y is written once.

#include "tim_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace tim {
namespace {

constexpr int kNormWaves = 4;            // rows per workgroup, one per wave
constexpr int kNormThreads = 64 * kNormWaves;

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
    return (double)__builtin_bit_cast(float, (uint32_t)b << 16);
}

// Nearest bf16 of a double, ties to even (the bits, in the low half).
// f = the nearest float of x first (one hardware conversion).  Every bf16
// midpoint is a float, so rounding x to the float grid cannot carry it
// across a midpoint: f rounds to the same bf16 as x unless f lands exactly
// on a midpoint.  Then x itself decides: equal (a true tie, to even), or
// which side of the midpoint it lies on.  A NaN stays a quiet NaN (the
// conversion gives the canonical one).
__device__ __forceinline__ uint32_t bf16_of_float_rne(uint32_t b) {
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ bool on_bf16_midpoint(uint32_t b) { return (b & 0xFFFFu) == 0x8000u; }
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
    const float f = (float)x;
    const uint32_t b = __builtin_bit_cast(uint32_t, f);
    if (on_bf16_midpoint(b)) {
        const double fd = (double)f;
        if (fd != x) return fabs(x) > fabs(fd) ? (b + 0x8000u) >> 16 : b >> 16;
    }
    return bf16_of_float_rne(b);
}

// Raw storage of one lane's 8-column group: 8 bf16 in one uint4, or 8 fp32 in
// two.  Columns past d hold zero bits (0.0).
template <bool kBf16>
struct Group {
    uint4 q[kBf16 ? 1 : 2];
};

template <bool kBf16, bool kVec>
__device__ __forceinline__ void load_group(const void* base, int64_t off, int64_t c0, int64_t d,
                                           Group<kBf16>& g) {
    if constexpr (kVec) {
        if constexpr (kBf16) {
            g.q[0] = *(const uint4*)((const uint16_t*)base + off + c0);
        } else {
            g.q[0] = *(const uint4*)((const float*)base + off + c0);
            g.q[1] = *(const uint4*)((const float*)base + off + c0 + 4);
        }
    } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool in = c0 + j < d;
            if constexpr (kBf16) e[j] = in ? ((const uint16_t*)base)[off + c0 + j] : 0u;
            else e[j] = in ? __builtin_bit_cast(uint32_t, ((const float*)base)[off + c0 + j]) : 0u;
        }
        if constexpr (kBf16) {
            g.q[0] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                e[6] | (e[7] << 16));
        } else {
            g.q[0] = make_uint4(e[0], e[1], e[2], e[3]);
            g.q[1] = make_uint4(e[4], e[5], e[6], e[7]);
        }
    }
}

template <bool kBf16>
__device__ __forceinline__ void unpack(const Group<kBf16>& g, double (&v)[8]) {
    if constexpr (kBf16) {
        const uint32_t w4[4] = {g.q[0].x, g.q[0].y, g.q[0].z, g.q[0].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_to_f64((uint16_t)(w4[j] & 0xFFFFu));
            v[2 * j + 1] = bf16_to_f64((uint16_t)(w4[j] >> 16));
        }
    } else {
        const uint32_t w8[8] = {g.q[0].x, g.q[0].y, g.q[0].z, g.q[0].w,
                                g.q[1].x, g.q[1].y, g.q[1].z, g.q[1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (double)__builtin_bit_cast(float, w8[j]);
    }
}

// y for one group: gamma * (x * r) in fp64, one rounding, stored.  v and gm
// are the group's x and gamma as doubles.  bf16: the common case rounds
// through the float conversion; if any lane of the wave has a value whose
// float lands on a bf16 midpoint, the whole wave takes the exact path for
// this group (a uniform branch, almost never taken).
template <bool kBf16, bool kVec>
__device__ __forceinline__ void store_group(const double (&v)[8], const double (&gm)[8],
                                            double r, void* y, int64_t off, int64_t c0,
                                            int64_t d) {
    double yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) yv[j] = gm[j] * (v[j] * r);
    if constexpr (kBf16) {
        uint32_t o[8];
        bool mid = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = __builtin_bit_cast(uint32_t, (float)yv[j]);
            mid |= on_bf16_midpoint(b);
            o[j] = bf16_of_float_rne(b);
        }
        if (__builtin_expect(__ballot(mid) != 0, 0)) {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = f64_to_bf16_rne(yv[j]);
        }
        if constexpr (kVec) {
            *(uint4*)((uint16_t*)y + off + c0) =
                make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                           o[6] | (o[7] << 16));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < d) ((uint16_t*)y)[off + c0 + j] = (uint16_t)o[j];
        }
    } else {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (float)yv[j];
        if constexpr (kVec) {
            *(float4*)((float*)y + off + c0) = make_float4(o[0], o[1], o[2], o[3]);
            *(float4*)((float*)y + off + c0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < d) ((float*)y)[off + c0 + j] = o[j];
        }
    }
}

// One wave per row (4 rows per workgroup), no barrier: lane l owns the
// groups l, l + 64, ... and reads its row twice (the second time from
// cache).  Sum of squares: each lane folds its groups in ascending order, a
// column at a time, in fp64, and the 64 lane sums meet in a fixed
// butterfly.
template <bool kBf16, bool kVec>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_wave_kernel(const void* __restrict__ x, int64_t ldx, const void* __restrict__ gamma,
                    int64_t n, int64_t d, double eps, void* __restrict__ y, int64_t ldy,
                    float* __restrict__ rstd_out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (t >= n) return;                                  // whole wave leaves together
    const int64_t groups = (d + 7) / 8;
    double ss = 0.0;
#pragma unroll 2
    for (int64_t g = lane; g < groups; g += 64) {
        Group<kBf16> xg;
        load_group<kBf16, kVec>(x, t * ldx, g * 8, d, xg);
        double v[8];
        unpack<kBf16>(xg, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fma(v[j], v[j], ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    if (rstd_out && lane == 0) rstd_out[t] = (float)r;
    for (int64_t g = lane; g < groups; g += 64) {
        Group<kBf16> xg, gg;
        load_group<kBf16, kVec>(x, t * ldx, g * 8, d, xg);
        load_group<kBf16, kVec>(gamma, 0, g * 8, d, gg);
        double v[8], gm[8];
        unpack<kBf16>(xg, v);
        unpack<kBf16>(gg, gm);
        store_group<kBf16, kVec>(v, gm, r, y, t * ldy, g * 8, d);
    }
}

// The same for rows of at most 64 kPer groups: a lane keeps its groups
// l, l + 64, ... in registers, so all of them are in flight at once and x is
// read once.  Same fold order as above (ascending groups, a column at a
// time, then the butterfly), so the same bits.
template <bool kBf16, bool kVec, int kPer>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_reg_kernel(const void* __restrict__ x, int64_t ldx, const void* __restrict__ gamma,
                   int64_t n, int64_t d, double eps, void* __restrict__ y, int64_t ldy,
                   float* __restrict__ rstd_out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (t >= n) return;                                  // whole wave leaves together
    const int64_t groups = (d + 7) / 8;
    Group<kBf16> xg[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t g = lane + 64 * i;
        if (g < groups) load_group<kBf16, kVec>(x, t * ldx, g * 8, d, xg[i]);
        else xg[i] = Group<kBf16>{};
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        double v[8];
        unpack<kBf16>(xg[i], v);               // groups past the row are zeros: exact no-ops
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fma(v[j], v[j], ss);
    }
    // keep the raw groups, not their fp64 unpacking, alive for the second
    // pass (the unpacking is cheap; holding it would cost 4x the registers)
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
        for (int k = 0; k < (kBf16 ? 1 : 2); ++k)
            asm volatile("" : "+v"(xg[i].q[k].x), "+v"(xg[i].q[k].y), "+v"(xg[i].q[k].z),
                              "+v"(xg[i].q[k].w));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    if (rstd_out && lane == 0) rstd_out[t] = (float)r;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t g = lane + 64 * i;
        if (g >= groups) break;
        Group<kBf16> gg;
        load_group<kBf16, kVec>(gamma, 0, g * 8, d, gg);
        double v[8], gm[8];
        unpack<kBf16>(xg[i], v);
        unpack<kBf16>(gg, gm);
        store_group<kBf16, kVec>(v, gm, r, y, t * ldy, g * 8, d);
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
    const int64_t groups = (d + 7) / 8;
    if (dtype == 0) {
        if (groups <= 64 * 8) {              // D <= 4096: 32 registers of row per lane
            if (vec) go(rmsnorm_reg_kernel<true, true, 8>);
            else go(rmsnorm_reg_kernel<true, false, 8>);
        } else if (groups <= 64 * 16) {      // D <= 8192
            if (vec) go(rmsnorm_reg_kernel<true, true, 16>);
            else go(rmsnorm_reg_kernel<true, false, 16>);
        } else {
            if (vec) go(rmsnorm_wave_kernel<true, true>);
            else go(rmsnorm_wave_kernel<true, false>);
        }
    } else {
        if (groups <= 64 * 8) {              // D <= 4096: 64 registers of row per lane
            if (vec) go(rmsnorm_reg_kernel<false, true, 8>);
            else go(rmsnorm_reg_kernel<false, false, 8>);
        } else {
            if (vec) go(rmsnorm_wave_kernel<false, true>);
            else go(rmsnorm_wave_kernel<false, false>);
        }
    }
    return hipGetLastError();
}

}  // namespace tim
