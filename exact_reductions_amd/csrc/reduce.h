// Lane accumulators, wave and workgroup reductions, records and the
// per-frame combine shared by the stage-1 kernels of libvqx (internal).
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
//
// Every term is an exact integer and every sum an integer sum, so the
// reduction order cannot change a result.  A kernel that uses these must
// keep each lane's share within the budgets stated with the kernel: every
// wave64 total of a lane accumulator (or of its 16-bit halves) must fit
// uint32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plane_stats.h"
#include "terms.h"

#pragma clang fp contract(off)

namespace vqx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // four wave64s
static_assert(kThreads == kChunkThreads, "dispatch-size check");
constexpr int kWaves = kThreads / 64;

// --------------------------------------------------------------- 8-bit terms
struct Acc8 {
    uint32_t r1 = 0, d1 = 0, r2 = 0, d2 = 0, rd = 0;
};

// Four samples of each plane packed in one dword.
__device__ __forceinline__ void add_dword(Acc8 &a, uint32_t r, uint32_t d)
{
    a.r1 = __builtin_amdgcn_sad_u8(r, 0u, a.r1);          // + r0 + r1 + r2 + r3
    a.d1 = __builtin_amdgcn_sad_u8(d, 0u, a.d1);
    a.r2 = __builtin_amdgcn_udot4(r, r, a.r2, false);     // + sum r_i^2
    a.d2 = __builtin_amdgcn_udot4(d, d, a.d2, false);
    a.rd = __builtin_amdgcn_udot4(r, d, a.rd, false);     // + sum r_i*d_i
}

// -------------------------------------------------------------- 16-bit terms
// Each sample is converted to float once; that value serves its own square
// and the difference (left to itself, the compiler squares a sample as an
// integer and converts the product, which converts each sample twice).  The
// three products are integers below 2^32 [MOMENT, Decision].  Two lane
// forms add them exactly, each where it measured faster:
//  * Acc16U64, uint64 lanes (one v_lshl_add_u64 per term, plus a move that
//    zeroes the high half of the term's register pair): the contiguous
//    stage 1, 153.4 us per 3840x2160x32 batch against 155.9 us in binary64;
//  * Acc16F64, binary64 lanes (a widening conversion and an fp64 add per
//    term; a lane adds at most a few hundred terms, so every partial sum is
//    an integer below 2^53, exact, and the total converts to uint64 without
//    loss): the view kernels and the mapped stage 1.  It needs far fewer
//    registers, which the view kernels' sample-by-sample path, bound by
//    load latency, turns into occupancy (368 us against 497 us per batch
//    of rows at mismatched offsets).
// Either way the sums are exact integers.  The kernels run near the HBM
// roofline with their SIMDs also busy, so the work per byte matters.
struct Acc16U64 {
    uint64_t noise = 0, r2 = 0, d2 = 0;
    uint32_t r1 = 0, d1 = 0;
};

struct Acc16F64 {
    double noise = 0, r2 = 0, d2 = 0;
    uint32_t r1 = 0, d1 = 0;
};

// A float product (an integer below 2^32) as a term of a Lane sum: read
// back as uint32 for integer lanes, widened for binary64 lanes.
__device__ __forceinline__ uint32_t lane_term(float p, uint64_t) { return static_cast<uint32_t>(p); }
__device__ __forceinline__ double lane_term(float p, double) { return static_cast<double>(p); }

// Two samples of each plane packed in one dword.
template <class Acc>
__device__ __forceinline__ void add_dword_16(Acc &a, uint32_t r, uint32_t d)
{
    using Lane = decltype(a.noise);
    float r0 = static_cast<float>(r & 0xffffu), r1 = static_cast<float>(r >> 16);
    float d0 = static_cast<float>(d & 0xffffu), d1 = static_cast<float>(d >> 16);
    asm volatile("" : "+v"(r0), "+v"(r1), "+v"(d0), "+v"(d1));  // one conversion each
    // float_psnr: the square of the float difference [PSNR, Decision]
    a.noise += lane_term((r0 - d0) * (r0 - d0), Lane{});
    a.noise += lane_term((r1 - d1) * (r1 - d1), Lane{});
    // float_moment: the float squares of the samples [MOMENT, Decision]
    a.r2 += lane_term(r0 * r0, Lane{});
    a.r2 += lane_term(r1 * r1, Lane{});
    a.d2 += lane_term(d0 * d0, Lane{});
    a.d2 += lane_term(d1 * d1, Lane{});
    // the sample sums: r0 + r1 in one integer dot product
    const u16x2 ones = {1, 1};
    a.r1 = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, r), ones, a.r1, false);
    a.d1 = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, d), ones, a.d1, false);
}

__device__ __forceinline__ void add_dword(Acc16U64 &a, uint32_t r, uint32_t d) { add_dword_16(a, r, d); }
__device__ __forceinline__ void add_dword(Acc16F64 &a, uint32_t r, uint32_t d) { add_dword_16(a, r, d); }

// Acc16's sums with uint64 lanes, and the OR of the terms of each square
// sum, for their low bits: a run of terms all multiples of 2^k rounds
// nowhere in a binade of unit 2^k (the CPU-order mode reads this).
struct Acc16Low {
    uint64_t noise = 0, r2 = 0, d2 = 0;
    uint32_t r1 = 0, d1 = 0;
    uint32_t or_noise = 0, or_r2 = 0, or_d2 = 0;
};

__device__ __forceinline__ void add_dword(Acc16Low &a, uint32_t r, uint32_t d)
{
    float r0 = static_cast<float>(r & 0xffffu), r1 = static_cast<float>(r >> 16);
    float d0 = static_cast<float>(d & 0xffffu), d1 = static_cast<float>(d >> 16);
    asm volatile("" : "+v"(r0), "+v"(r1), "+v"(d0), "+v"(d1));  // one conversion each
    const uint32_t n0 = float_square(r0 - d0), n1 = float_square(r1 - d1);
    const uint32_t a0 = float_square(r0), a1 = float_square(r1);
    const uint32_t b0 = float_square(d0), b1 = float_square(d1);
    a.noise += n0;
    a.noise += n1;
    a.r2 += a0;
    a.r2 += a1;
    a.d2 += b0;
    a.d2 += b1;
    a.or_noise |= n0 | n1;
    a.or_r2 |= a0 | a1;
    a.or_d2 |= b0 | b1;
    const u16x2 ones = {1, 1};
    a.r1 = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, r), ones, a.r1, false);
    a.d1 = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, d), ones, a.d1, false);
}

// A lane's sum as uint64 (a double lane sum is an exact integer below 2^53).
__device__ __forceinline__ uint64_t lane_total(double x) { return static_cast<uint64_t>(x); }
__device__ __forceinline__ uint64_t lane_total(uint64_t x) { return x; }

template <class Acc>
__device__ __forceinline__ void add_vec(Acc &a, const u32x4 &r, const u32x4 &d)
{
    add_dword(a, r.x, d.x);
    add_dword(a, r.y, d.y);
    add_dword(a, r.z, d.z);
    add_dword(a, r.w, d.w);
}

// ---------------------------------------------------------- wave64 reduction
// Sum of v over the 64 lanes, returned to every lane.  Four DPP steps add
// within each row of 16 lanes; row_bcast:15 and row_bcast:31 carry rows into
// rows 1..3, so lane 63 ends with the total, which readlane broadcasts.
__device__ __forceinline__ uint32_t dpp_step(uint32_t v, int ctrl_sel)
{
    switch (ctrl_sel) {
    case 0: return __builtin_amdgcn_update_dpp(0u, v, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    case 1: return __builtin_amdgcn_update_dpp(0u, v, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    case 2: return __builtin_amdgcn_update_dpp(0u, v, 0x124, 0xf, 0xf, false);  // row_ror:4
    case 3: return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false);  // row_ror:8
    case 4: return __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    default: return __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
    }
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    v += dpp_step(v, 0);
    v += dpp_step(v, 1);
    v += dpp_step(v, 2);
    v += dpp_step(v, 3);
    v += dpp_step(v, 4);
    v += dpp_step(v, 5);
    return __builtin_amdgcn_readlane(v, 63);
}

// OR of v over the 64 lanes (the wave_sum steps with | for +).
__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    v |= dpp_step(v, 0);
    v |= dpp_step(v, 1);
    v |= dpp_step(v, 2);
    v |= dpp_step(v, 3);
    v |= dpp_step(v, 4);
    v |= dpp_step(v, 5);
    return __builtin_amdgcn_readlane(v, 63);
}

// OR of v over the workgroup, in every thread.  All threads must call it.
__device__ __forceinline__ uint32_t workgroup_or(uint32_t v)
{
    __shared__ uint32_t lds[kWaves];
    const uint32_t w = wave_or(v);
    if ((threadIdx.x & 63) == 0)
        lds[threadIdx.x / 64] = w;
    __syncthreads();
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
        o |= lds[i];
    return o;
}

// Adds every lane's accumulators of the workgroup: every thread gets the N
// totals in uint64.  All threads must call it.
template <int N>
__device__ __forceinline__ void workgroup_sums(const uint32_t (&v)[N], uint64_t (&out)[N])
{
    __shared__ uint32_t lds[kWaves][N];
    const int wave = threadIdx.x / 64;
    uint32_t w[N];
#pragma unroll
    for (int k = 0; k < N; ++k)
        w[k] = wave_sum(v[k]);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k)
            lds[wave][k] = w[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        uint64_t s = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
            s += lds[i][k];
        out[k] = s;
    }
}

// Thread 0 writes the workgroup's record; the combine kernel that follows
// in the stream reads it.
__device__ __forceinline__ void write_record(uint64_t *part, int64_t wg,
                                             const uint64_t (&rec)[kSums])
{
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < kSums; ++k)
            part[wg * kRecordStride + k] = rec[k];
    }
}

// One sample of each plane as the low lane of a dword (the other lanes zero,
// which add nothing to any sum: q(0) = 0).
template <int kBytes>
__device__ __forceinline__ uint32_t load_sample(const void *plane, int64_t i)
{
    if constexpr (kBytes == 1)
        return static_cast<const uint8_t *>(plane)[i];
    else
        return static_cast<const uint16_t *>(plane)[i];
}


// ------------------------------------------------------------- combine
// Adds frame `frame`'s records in uint64 and writes its five sums.  All
// kThreads threads of the workgroup must call it.
__device__ __forceinline__ void combine_frame(const uint64_t *part, int chunks, int64_t frame, uint64_t *out_noise,
                                              uint64_t *out_moments)
{
    __shared__ uint64_t lds[kSums][kThreads];
    const int t = threadIdx.x;
    uint64_t s[kSums] = {0, 0, 0, 0, 0};
    for (int c = t; c < chunks; c += kThreads) {
#pragma unroll
        for (int k = 0; k < kSums; ++k)
            s[k] += part[(frame * chunks + c) * kRecordStride + k];
    }
#pragma unroll
    for (int k = 0; k < kSums; ++k)
        lds[k][t] = s[k];
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (t < off) {
#pragma unroll
            for (int k = 0; k < kSums; ++k)
                lds[k][t] += lds[k][t + off];
        }
        __syncthreads();
    }
    if (t == 0) {
        out_noise[frame] = lds[kNoise][0];
        if (out_moments) {  // null where only the noise is wanted
            out_moments[4 * frame + 0] = lds[kRef1][0];
            out_moments[4 * frame + 1] = lds[kDist1][0];
            out_moments[4 * frame + 2] = lds[kRef2][0];
            out_moments[4 * frame + 3] = lds[kDist2][0];
        }
    }
}

}  // namespace
}  // namespace vqx
