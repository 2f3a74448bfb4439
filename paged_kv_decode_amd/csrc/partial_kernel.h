// partial_kernel.h -- the partial kernel of paged-KV GQA decode attention
// (gfx950 device code), included by the translation units that instantiate it.
//
// Partial kernel: one workgroup of NW wave64s per (partition, KV head,
// sequence).  The partition's pages are dealt to the waves in blocks of NB
// pages (4 KiB of K and 4 KiB of V per block where a page allows it; one
// 8 KiB page at head_dim 256).  For each block a wave
//   1. reads the block's page ids from a page-id vector (one scalar readlane
//      per page) and issues 16-byte loads of whole 128-byte lines of every K
//      and V row of those pages;
//   2. copies the rows into per-wave LDS tiles (row-swizzled) as soon as they
//      land, and requests the next block's rows into the freed registers;
//   3. forms the scores of all G query heads of the group against each
//      16-token page with one MFMA chain: the page's key rows (from the K
//      tile) are the A operand, the G query rows (zero-padded to 16) the B
//      operand, head_dim the reduction axis, so each K byte is read once per
//      group;
//   4. updates the per-head online-softmax state (running max, denominator):
//      each lane holds one head and four tokens, so the block maximum is an
//      in-lane max plus two cross-lane steps;
//   5. accumulates P.V on the matrix cores: the probabilities are already in
//      the A-operand layout, V comes from the V tile through the LDS
//      transpose read, and the output block sits in VGPRs.
// The waves' states are then combined in LDS (running max first, then the
// rescaled denominators and outputs) and the workgroup writes either the
// partition state (o normalised, max, denominator) for the merge kernel or,
// when one partition covers the context, out and lse directly.
//
// Exponentials are base 2 throughout (scores pre-multiplied by log2(e));
// lse is converted back to the natural logarithm on output.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "pa_decode.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kPage = 16;
constexpr float kLn2 = 0.693147180559945309f;
// Headroom (log2 units) of the softmax reference value over the running max.
constexpr float kSlack = 8.f;

template <int DT> struct Elt;
template <> struct Elt<PA_DTYPE_F32> { static constexpr int bytes = 4; };
template <> struct Elt<PA_DTYPE_F16> { static constexpr int bytes = 2; };
template <> struct Elt<PA_DTYPE_BF16> { static constexpr int bytes = 2; };

// ---- cross-lane helpers (wave64, DPP within 16-lane rows) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max / sum over the 16 lanes of each DPP row (xor 1, xor 2, half mirror, mirror).
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// Max / sum over the four 16-lane rows of the wave, for each lane % 16:
// permlane32_swap pairs rows {0,1} with {2,3}, permlane16_swap row 0 with 1
// and row 2 with 3 (VALU lane swaps, no LDS round trip).
__device__ __forceinline__ float rows4_max(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows4_sum(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum over the 64 lanes: within each 16-lane row by DPP
// row shifts (a lane whose source lies before its row reads 0), then each
// row adds the totals of the rows before it.
__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
    x += __builtin_amdgcn_mov_dpp(x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_mov_dpp(x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_mov_dpp(x, 0x118, 0xF, 0xF, true);   // row_shr:8
    const int t0 = __builtin_amdgcn_readlane(x, 15);
    const int t1 = __builtin_amdgcn_readlane(x, 31);
    const int t2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane >> 4;
    return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// floor(num / den) for num >= 0, den > 0, num + den < 2^53 and a quotient
// below 2^31.  A quotient q = num / den that is not an integer lies at least
// 1 / den below the next integer k + 1, while rounding q to double moves it
// by at most half an ulp of k + 1, i.e. (k + 1) 2^-53 < 1 / den when
// num + den < 2^53; so the correctly rounded double quotient never reaches
// k + 1 and truncating it is exact.  Much cheaper than the 64-bit integer
// division sequence.
__device__ __forceinline__ int floor_div(int64_t num, int den)
{
    return int(double(num) / double(den));
}

__device__ __forceinline__ void wave_lds_sync()
{
    // LDS traffic of one wave is ordered; this keeps the compiler from moving
    // LDS accesses across the exchange point and waits for them to land.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Compiler-only memory barrier: keeps prefetch loads where they are written
// (otherwise they are sunk next to their first use, which undoes the
// software pipeline); emits no instruction.
__device__ __forceinline__ void pin_loads() { asm volatile("" ::: "memory"); }

// ---- score MFMA over one 16-byte chunk of head_dim ----
template <int DT> struct Chunk;

template <> struct Chunk<PA_DTYPE_F16> {
    __device__ static f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

template <> struct Chunk<PA_DTYPE_BF16> {
    __device__ static f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <> struct Chunk<PA_DTYPE_F32> {
    __device__ static f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
    {
        // Four K=4 steps, one per float of the chunk (same k slot in A and B).
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c,
                                                     0, 0, 0);
        return c;
    }
};

// sin and cos of 2 pi x for |x| <= 1/2 (x in revolutions, already reduced):
// the nearest quarter turn q/4 is split off, the rest |a| <= pi/4 goes
// through the Taylor series of sin (to degree 9) and cos (to degree 10),
// whose truncation error on |a| <= pi/4 is below 2e-9, and the result is
// turned by q quarter turns.
__device__ __forceinline__ void sincos_rev(float x, float* s, float* c)
{
    const float q = rintf(4.f * x);
    const float a = (x - 0.25f * q) * 6.28318530717958648f;
    const float a2 = a * a;
    const float sp =
        a * (1.f + a2 * (-1.f / 6.f + a2 * (1.f / 120.f + a2 * (-1.f / 5040.f + a2 * (1.f / 362880.f)))));
    const float cp =
        1.f + a2 * (-0.5f + a2 * (1.f / 24.f + a2 * (-1.f / 720.f +
                                                     a2 * (1.f / 40320.f + a2 * (-1.f / 3628800.f)))));
    const int k = int(q) & 3;
    // sin(a + k pi/2), cos(a + k pi/2)
    *s = k == 0 ? sp : k == 1 ? cp : k == 2 ? -sp : -cp;
    *c = k == 0 ? cp : k == 1 ? -sp : k == 2 ? -cp : sp;
}

// ---- turned (rotary-embedded) key chunks ----
// widen(): a key chunk as EPC floats.  mfma(): the score MFMA of a turned
// chunk (floats) against q.  A turned key is no longer a 16-bit value, so
// f16 / bf16 keys enter as two parts, hi = round(x) and lo = round(x - hi)
// (about 22 / 18 significant bits together, two MFMAs); rounding the turned
// key once would move each score by ~2^-12 (f16) or ~2^-9 (bf16) relative.
template <int DT> struct TurnedKey;


template <> struct TurnedKey<PA_DTYPE_F16> {
    static constexpr int EPC = 8;
    __device__ static void widen(u32x4 c, float (&x)[8])
    {
        const f16x8 h = __builtin_bit_cast(f16x8, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)h[e];
    }
    __device__ static f32x4 mfma(const float (&x)[8], u32x4 q, f32x4 acc)
    {
        f16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = (_Float16)x[e];
            lo[e] = (_Float16)(x[e] - (float)hi[e]);
        }
        acc = Chunk<PA_DTYPE_F16>::mfma(__builtin_bit_cast(u32x4, hi), q, acc);
        return Chunk<PA_DTYPE_F16>::mfma(__builtin_bit_cast(u32x4, lo), q, acc);
    }
    // Turn the pair chunks (x, y) (first / second half of head_dim) by the
    // angles (cs, sn) and add both score MFMAs.  The f16 keys enter the
    // mixed-precision FMAs directly; hi is the pair-wise round toward zero of
    // the turned value and lo = fma(hi, m1, turned) rounded to f16, one mixed
    // FMA.  m1 is -1 from a kernel argument: with a literal -1 the compiler
    // rewrites the FMA as a subtraction with conversions around it.
    __device__ static f32x4 turn_mfma(u32x4 xc, u32x4 yc, const float (&cs)[8],
                                      const float (&sn)[8], u32x4 qx, u32x4 qy, f32x4 acc,
                                      float m1)
    {
        typedef __fp16 h2 __attribute__((ext_vector_type(2)));
        const f16x8 x = __builtin_bit_cast(f16x8, xc), y = __builtin_bit_cast(f16x8, yc);
        float xr[8], yr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ys = __builtin_fmaf((float)y[e], sn[e], 0.f);
            const float xs = __builtin_fmaf((float)x[e], sn[e], 0.f);
            xr[e] = __builtin_fmaf((float)x[e], cs[e], -ys);
            yr[e] = __builtin_fmaf((float)y[e], cs[e], xs);
        }
        u32x4 xh, xl, yh, yl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h2 a = __builtin_amdgcn_cvt_pkrtz(xr[2 * j], xr[2 * j + 1]);
            const h2 b = __builtin_amdgcn_cvt_pkrtz(yr[2 * j], yr[2 * j + 1]);
            xh[j] = __builtin_bit_cast(uint32_t, a);
            yh[j] = __builtin_bit_cast(uint32_t, b);
            const f16x2 lx = {(_Float16)__builtin_fmaf((float)a[0], m1, xr[2 * j]),
                              (_Float16)__builtin_fmaf((float)a[1], m1, xr[2 * j + 1])};
            const f16x2 ly = {(_Float16)__builtin_fmaf((float)b[0], m1, yr[2 * j]),
                              (_Float16)__builtin_fmaf((float)b[1], m1, yr[2 * j + 1])};
            xl[j] = __builtin_bit_cast(uint32_t, lx);
            yl[j] = __builtin_bit_cast(uint32_t, ly);
        }
        acc = Chunk<PA_DTYPE_F16>::mfma(xh, qx, acc);
        acc = Chunk<PA_DTYPE_F16>::mfma(xl, qx, acc);
        acc = Chunk<PA_DTYPE_F16>::mfma(yh, qy, acc);
        return Chunk<PA_DTYPE_F16>::mfma(yl, qy, acc);
    }
};

template <> struct TurnedKey<PA_DTYPE_BF16> {
    static constexpr int EPC = 8;
    __device__ static void widen(u32x4 c, float (&x)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(c[j] << 16);
            x[2 * j + 1] = __uint_as_float(c[j] & 0xffff0000u);
        }
    }
    __device__ static f32x4 mfma(const float (&x)[8], u32x4 q, f32x4 acc)
    {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = (__bf16)x[e];
            lo[e] = (__bf16)(x[e] - (float)hi[e]);
        }
        acc = Chunk<PA_DTYPE_BF16>::mfma(__builtin_bit_cast(u32x4, hi), q, acc);
        return Chunk<PA_DTYPE_BF16>::mfma(__builtin_bit_cast(u32x4, lo), q, acc);
    }
    // As TurnedKey<F16>::turn_mfma.  hi: the pair rounded to nearest bf16
    // (one packed conversion); lo = turned - hi, exact in f32, truncated to
    // bf16 (a byte permute keeps the upper halves): |error| < 2^-16 |turned|.
    __device__ static f32x4 turn_mfma(u32x4 xc, u32x4 yc, const float (&cs)[8],
                                      const float (&sn)[8], u32x4 qx, u32x4 qy, f32x4 acc,
                                      float)
    {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        u32x4 xh, xl, yh, yl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x0 = __uint_as_float(xc[j] << 16), x1 = __uint_as_float(xc[j] & 0xffff0000u);
            const float y0 = __uint_as_float(yc[j] << 16), y1 = __uint_as_float(yc[j] & 0xffff0000u);
            const float c0 = cs[2 * j], c1 = cs[2 * j + 1], s0 = sn[2 * j], s1 = sn[2 * j + 1];
            const f2 xr = {x0 * c0 - y0 * s0, x1 * c1 - y1 * s1};
            const f2 yr = {y0 * c0 + x0 * s0, y1 * c1 + x1 * s1};
            const uint32_t hx = __builtin_bit_cast(uint32_t, __builtin_convertvector(xr, b2));
            const uint32_t hy = __builtin_bit_cast(uint32_t, __builtin_convertvector(yr, b2));
            xh[j] = hx;
            yh[j] = hy;
            const float lx0 = xr[0] - __uint_as_float(hx << 16);
            const float lx1 = xr[1] - __uint_as_float(hx & 0xffff0000u);
            const float ly0 = yr[0] - __uint_as_float(hy << 16);
            const float ly1 = yr[1] - __uint_as_float(hy & 0xffff0000u);
            xl[j] = __builtin_amdgcn_perm(__float_as_uint(lx1), __float_as_uint(lx0), 0x07060302u);
            yl[j] = __builtin_amdgcn_perm(__float_as_uint(ly1), __float_as_uint(ly0), 0x07060302u);
        }
        acc = Chunk<PA_DTYPE_BF16>::mfma(xh, qx, acc);
        acc = Chunk<PA_DTYPE_BF16>::mfma(xl, qx, acc);
        acc = Chunk<PA_DTYPE_BF16>::mfma(yh, qy, acc);
        return Chunk<PA_DTYPE_BF16>::mfma(yl, qy, acc);
    }
};

template <> struct TurnedKey<PA_DTYPE_F32> {
    static constexpr int EPC = 4;
    __device__ static void widen(u32x4 c, float (&x)[4])
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(c[e]);
    }
    __device__ static f32x4 mfma(const float (&x)[4], u32x4 q, f32x4 acc)
    {
        const u32x4 a = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                         __float_as_uint(x[3])};
        return Chunk<PA_DTYPE_F32>::mfma(a, q, acc);
    }
};

template <int DT> __device__ __forceinline__ void store_out(void* out, size_t idx, float x);
template <> __device__ __forceinline__ void store_out<PA_DTYPE_F32>(void* out, size_t idx, float x)
{
    static_cast<float*>(out)[idx] = x;
}
template <> __device__ __forceinline__ void store_out<PA_DTYPE_F16>(void* out, size_t idx, float x)
{
    static_cast<_Float16*>(out)[idx] = (_Float16)x;
}
template <> __device__ __forceinline__ void store_out<PA_DTYPE_BF16>(void* out, size_t idx, float x)
{
    static_cast<__bf16*>(out)[idx] = (__bf16)x;
}
// Four consecutive output elements (16-byte aligned for f32, 8-byte for
// f16/bf16: out is 16-byte aligned and idx a multiple of 4), rounded to the
// output type as store_out does.
template <int DT> __device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 x);
template <> __device__ __forceinline__ void store_out4<PA_DTYPE_F32>(void* out, size_t idx, f32x4 x)
{
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = x;
}
template <> __device__ __forceinline__ void store_out4<PA_DTYPE_F16>(void* out, size_t idx, f32x4 x)
{
    const f16x4 h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(out) + idx) = h;
}
template <> __device__ __forceinline__ void store_out4<PA_DTYPE_BF16>(void* out, size_t idx, f32x4 x)
{
    const bf16x4 h = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + idx) = h;
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

// K/V are streamed and read once per step: non-temporal loads (measured on
// MI355X: random 8 KiB page tiles gather at ~6.9 TB/s this way against ~6.0
// TB/s with default loads).
__device__ __forceinline__ u32x4 load16_stream(const void* p)
{
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}


// ---- P.V on the matrix cores ----
// One 16x16 output block (16 query-head rows x 16 head_dim columns) gains
// p[head][token] * V[token][column] over the 16 tokens of a page.  Lane l
// holds p of head l % 16 for tokens 4*(l/16) + j (the score MFMA leaves them
// there) and reads V[tokens 4*(l/16) + j][column l % 16] from the LDS tile.
template <int DT> struct PV;

template <> struct PV<PA_DTYPE_F16> {
    // p = hi + lo in two f16 parts (22 significant bits): f16 p alone leaves
    // a relative error near 2^-12 per probability, which alone would use a
    // third of the output tolerance after rounding to f16.
    __device__ static f32x4 mma(const float p[4], s16x4 v, f32x4 c)
    {
        const f16x4 hi = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
        const f16x4 lo = {(_Float16)(p[0] - (float)hi[0]), (_Float16)(p[1] - (float)hi[1]),
                          (_Float16)(p[2] - (float)hi[2]), (_Float16)(p[3] - (float)hi[3])};
        const f16x4 vh = __builtin_bit_cast(f16x4, v);
        c = __builtin_amdgcn_mfma_f32_16x16x16f16(hi, vh, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x16f16(lo, vh, c, 0, 0, 0);
    }
};

// Two pages at once (16x16x32): k slots 0..3 of a lane group are page a's
// tokens 4*grp + j, slots 4..7 page b's; the V operand is the two transpose
// reads side by side.
template <int DT> struct PV2;

template <> struct PV2<PA_DTYPE_F16> {
    __device__ static f32x4 mma(const float pa[4], const float pb[4], s16x4 va, s16x4 vb, f32x4 c)
    {
        f16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hi[j] = (_Float16)pa[j];
            hi[4 + j] = (_Float16)pb[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo[j] = (_Float16)(pa[j] - (float)hi[j]);
            lo[4 + j] = (_Float16)(pb[j] - (float)hi[4 + j]);
        }
        const f16x8 v = __builtin_bit_cast(f16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, v, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, v, c, 0, 0, 0);
    }
};

template <> struct PV2<PA_DTYPE_BF16> {
    __device__ static f32x4 mma(const float pa[4], const float pb[4], s16x4 va, s16x4 vb, f32x4 c)
    {
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hi[j] = (__bf16)pa[j];
            hi[4 + j] = (__bf16)pb[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo[j] = (__bf16)(pa[j] - (float)hi[j]);
            lo[4 + j] = (__bf16)(pb[j] - (float)hi[4 + j]);
        }
        const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, v, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, v, c, 0, 0, 0);
    }
};

template <> struct PV<PA_DTYPE_BF16> {
    // p = hi + lo in two bf16 parts (16 significant bits): one bf16 part alone
    // would leave a relative error near 2^-9 in every probability.
    __device__ static f32x4 mma(const float p[4], s16x4 v, f32x4 c)
    {
        const bf16x4 hi = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
        const bf16x4 lo = {(__bf16)(p[0] - (float)hi[0]), (__bf16)(p[1] - (float)hi[1]),
                           (__bf16)(p[2] - (float)hi[2]), (__bf16)(p[3] - (float)hi[3])};
        const bf16x4 vb = __builtin_bit_cast(bf16x4, v);
        c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, vb, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, vb, c, 0, 0, 0);
    }
};

// ---- q.k on the vector ALUs (comparison build only) ----
// A library built with PA_QK_VALU=1 forms the scores with packed dot
// products instead of the score MFMA, for measuring one against the other;
// the shipped library uses the MFMA.
#ifndef PA_QK_VALU
#define PA_QK_VALU 0
#endif

// ---- fused merge (comparison build only) ----
// A library built with PA_FUSED_MERGE=1 launches no merge kernel for the fixed
// schedule: the partial kernel writes its partition states with agent-scope
// stores (written through to memory), then the last workgroup of each
// (sequence, KV head), found with an agent-scope counter in the workspace,
// merges that group's states itself.  The shipped library keeps the merge
// kernel.
#ifndef PA_FUSED_MERGE
#define PA_FUSED_MERGE 0
#endif
__device__ __forceinline__ void st_state(float* p, float v)
{
#if PA_FUSED_MERGE
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
    *p = v;
#endif
}
__device__ __forceinline__ void st_state4(float* p, f32x4 v)
{
#if PA_FUSED_MERGE
#pragma unroll
    for (int k = 0; k < 4; ++k) __hip_atomic_store(p + k, v[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
    *reinterpret_cast<f32x4*>(p) = v;
#endif
}

// Dot product of two 16-byte chunks (8 f16 / 8 bf16 / 4 f32 elements),
// accumulated in f32.  Each 32-bit element is copied to a scalar before the
// bit cast: hipcc (ROCm 7.2) compiles __builtin_bit_cast of a vector element
// expression, v[j], as a cast of element 0 for every j.
template <int DT> struct Dot;
template <> struct Dot<PA_DTYPE_F16> {
    __device__ static float dot(u32x4 a, u32x4 b, float c)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = a[j], y = b[j];
            c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), c,
                                       false);
        }
        return c;
    }
};
template <> struct Dot<PA_DTYPE_BF16> {
    __device__ static float dot(u32x4 a, u32x4 b, float c)
    {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = a[j], y = b[j];
            c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, x), __builtin_bit_cast(b2, y), c,
                                                false);
        }
        return c;
    }
};
template <> struct Dot<PA_DTYPE_F32> {
    __device__ static float dot(u32x4 a, u32x4 b, float c)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_fmaf(__uint_as_float(a[j]), __uint_as_float(b[j]), c);
        return c;
    }
};

// ---------------------------------------------------------------------------
// Partial kernel.
//   DT: element type; D: head_dim; G: instantiated group size (>= actual);
//   NB: pages per block; ROT: rotary embedding of q and keys (rotary_mode 1);
//   BAL: the length-balanced schedule.
// Workgroup (fixed schedule): blockDim.x / 64 waves split into partition
// slots of prm.waves_per_partition waves; slot j of workgroup x handles
// partition x * slots + j of KV head blockIdx.y of sequence blockIdx.z.
// Balanced schedule: wave j of workgroup x is wave x * waves + j of KV head
// blockIdx.y; it finds its range of the batch's visible pages from the
// lengths (see the prologue) and computes one partition state per sequence
// piece of that range.
// Lane maps (lane = 0..63, i16 = lane % 16, grp = lane / 16):
//   loads:   K and V alike: load instruction i of a page reads chunks
//            64*i .. 64*i + 63 of the page's 16 x CH chunk grid, lane l chunk
//            x = 64*i + l, i.e. row x / CH, chunk x % CH (for CH a power of
//            two: chunk c = l % CH of rows l / CH + (64 / CH) * i), so each
//            load instruction reads whole 128-byte lines; the rows go to
//            per-wave LDS tiles (16-byte chunks XOR-swizzled by row so that
//            the reads below are bank-conflict free);
//   scores:  MFMA with the page's 16 key rows as A and the G query rows
//            (zero-padded to 16) as B, head_dim the reduction axis: lane reads
//            chunk 4*ks + grp of key row i16 and of query row i16; result
//            element r of the lane is the score of query head i16 against
//            token 4*grp + r, so each K byte is read once per group;
//   P.V:     MFMA with those probabilities as A (no data movement) and V as
//            B, read from the V tile with the LDS transpose read; output
//            element r of the lane is head 4*grp + r, column 16*db + i16.
// The MFMA operand layout read straight from memory would fetch 16 rows x 64
// bytes per instruction: twice the L1 tag lookups of whole lines, and with
// non-temporal loads two L2 requests per line.
// LDS: per wave [K tile, V tile, rotary base table (ROT only)], then (ROT
// only) the workgroup's rotary offset table; after the main loop the wave
// areas are reused for the combine of the slot's waves.
// ---------------------------------------------------------------------------
template <int DT, int D, int G, int NB, bool ROT, bool BAL>
__global__ __launch_bounds__(256) void partial_kernel(const PartialParams prm)
{
    constexpr int EB = Elt<DT>::bytes;
    constexpr int CH = D * EB / 16;   // 16-byte chunks per key row
    constexpr int EPC = 16 / EB;      // elements per chunk
    constexpr int KS = CH / 4;        // load instructions per page = MFMA k-steps per page
    constexpr bool POW2 = (CH & (CH - 1)) == 0;
    constexpr int R = POW2 ? kWave / CH : 0;  // token rows per load instruction (power of two)
    constexpr int CHP = POW2 ? CH : CH + 1;   // tile row stride in chunks (odd when padded)
    constexpr int NDB = D / 16;       // 16-column blocks of the output
    constexpr int GP4 = (G + 3) / 4 * 4;
    constexpr int IPV = kWave / NB;   // loop iterations one page-id vector covers
    constexpr int KT = NB * kPage * CHP;  // 16-byte slots of one block's K (or V) tile
    constexpr int HD = D / 2;         // rotary frequencies
    constexpr int NE = ROT ? (NB * HD + kWave - 1) / kWave : 1;  // base-table entries per lane
    // Comparison build (PA_QK_VALU): scores on the vector ALUs; q in VGPRs
    // when G x KS chunks fit in 96 VGPRs, else in a per-wave LDS copy; the
    // scores pass through a per-wave [NB][16][16] LDS buffer on their way to
    // the P.V operand layout.
    constexpr bool QKV = PA_QK_VALU != 0 && !ROT;
    constexpr bool QREG = QKV && G * KS <= 24;
    constexpr int QW = QKV ? (QREG ? 0 : G * CH * 4) + NB * 256 : 0;   // floats
    constexpr int WS = 8 * KT + (ROT ? NB * D : 0) + QW;  // floats of LDS per wave
    static_assert(KS * 4 == CH && KS * kWave == kPage * CH, "lane map");
    static_assert(CH == 8 || CH == 12 || CH == 16 || CH == 32, "tiles");
    static_assert(G <= 16, "one 16-row MFMA block of query heads");

    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int lane = threadIdx.x & (kWave - 1);
    // Wave index and count are wave-uniform: keep them in scalar registers so
    // that page ids and loop bounds are scalar too.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nw = blockDim.x / kWave;
    // The balanced schedule gives every wave its own range (one wave per
    // partition slot).
    const int wpp = BAL ? 1 : prm.waves_per_partition;
    const int slot = wave / wpp, wi = wave % wpp;
    const int nslots = nw / wpp;
    const int prel = blockIdx.x * nslots + slot;
    const int kvh = blockIdx.y;
    const int Gact = prm.group;
    const int S = prm.partition_size;
    // The violation bits are reported after the main loop (fixed schedule;
    // wave-uniform) or after the last segment (balanced schedule).
    int violation = 0;
    // Page-table row and context length of sequence j: dense rows of
    // pt_stride entries with context_lens, or CSR rows (page_indptr,
    // last_page_len; first entry *i0).  *row_len bounds the entries a row
    // may be read at.  Values outside the contract are clamped (and
    // reported), so that no address ever comes from them.  Clamps without
    // branches: a branch on a loaded value would hold back the page-id and q
    // loads until that value arrives.
    auto seq_view = [&](int j, int* i0_out, int* row_len_out, int* n_out) {
        int nn;
        if (prm.page_indptr) {
            const int r0 = prm.page_indptr[j], r1 = prm.page_indptr[j + 1];
            const int i0 = min(max(r0, 0), prm.nnz_pages);
            const int i1 = min(max(r1, i0), prm.nnz_pages);
            violation |= (i0 != r0 || i1 != r1) ? PA_DECODE_VIOLATION_ROW : 0;
            *i0_out = i0;
            *row_len_out = i1 - i0;
            const int last = min(max(prm.last_page_len[j], 0), kPage);
            nn = i1 > i0 ? (i1 - i0 - 1) * kPage + last : 0;
        } else {
            *i0_out = 0;
            *row_len_out = prm.pt_stride;
            nn = prm.context_lens[j];
        }
        const int nc = min(max(nn, 0), prm.max_context_len);
        violation |= nc != nn ? PA_DECODE_VIOLATION_LENGTH : 0;
        *n_out = nc;
    };
    // The segment being computed: sequence b, its row, its clamped length.
    int b, row_len, n;
    const int32_t* pt_row;
    const int i16 = lane & 15, grp = lane >> 4;
    // Load map: row and chunk of instruction i's chunk for this lane.
    auto lrow = [&](int i) { if constexpr (POW2) return R * i + lane / CH; else return (kWave * i + lane) / CH; };
    auto lchk = [&](int i) { if constexpr (POW2) return lane % CH; else return (kWave * i + lane) % CH; };

    // Page ids of this wave's pages, one per lane: lane j holds the page of
    // block (wi + wpp * (it0 + j / NB)), page j % NB of the partition that
    // starts at page pg_first; entries at or past pg_end are not read.
    auto load_ids = [&](int pg_first, int pg_end, int it0) {
        const int it = it0 + lane / NB;
        const int pg = pg_first + (wi + wpp * it) * NB + lane % NB;
        return pg < pg_end ? pt_row[pg] : 0;
    };
    int ids = 0;

    // Balanced schedule.  Lane j < batch holds sequence j's clamped view and
    // visible pages (window start lo_j to the last page).  Each sequence
    // with pages is charged C = bal_start extra "start" pages in front of
    // them (a segment's start costs a page-id and q fetch before its first
    // block), which no wave reads; vv_j is that charged count, vincl the
    // inclusive prefix sum, T the total.  With Weff = min(bal_waves, T)
    // waves (so that each has at least one charged page), wave w takes the
    // charged pages [w T / Weff, (w + 1) T / Weff) of the concatenation in
    // sequence order, so page x lies in wave ((x + 1) Weff - 1) / T.  The
    // visible pages of the wave's range, cut at sequence ends, are its
    // segments; the segment of sequence b in wave w is that sequence's state
    // row w - w0(b), w0(b) being the wave of its first visible page.
    int sb = 0;                       // first sequence of the range
    int vincl = 0, vpages = 0, vv = 0, vn = 0, vlo = 0, vi0 = 0, vrl = 0;
    const int C = prm.bal_start;
    int T = 0, Weff = 0;
    int64_t rA = 0, rE = 0;           // the wave's page range
    uint64_t nonempty = 0;
    // The next segment (sequence nx_b, pages [nx_pg0, nx_pg1)) and its page
    // ids, fetched one segment ahead.
    bool nx = false;
    int nx_b = 0, nx_pg0 = 0, nx_pg1 = 0, nx_ids = 0;
    auto seq_row = [&](int j) {
        return prm.page_table + (prm.page_indptr ? size_t(__builtin_amdgcn_readlane(vi0, j))
                                                 : size_t(j) * prm.pt_stride);
    };
    // From sequence s on, the first sequence with visible pages in the
    // range: sets nx_b, nx_pg0, nx_pg1 and issues the load of its first
    // page ids; false when none is left (or the next starts past the range).
    auto find_seg = [&](int s) -> bool {
        for (;;) {
            const uint64_t rest = s < kWave ? nonempty & (~0ull << s) : 0ull;
            if (rest == 0)
                return false;
            s = __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(rest)));
            const int in = __builtin_amdgcn_readlane(vincl, s);
            const int ex = in - __builtin_amdgcn_readlane(vv, s);
            if (ex >= rE)
                return false;
            // The visible part of the range in sequence s (empty when the
            // range holds only its start charge).
            const int64_t r0 = max(rA, int64_t(ex) + C), r1 = min(rE, int64_t(in));
            if (r0 < r1) {
                const int fp = __builtin_amdgcn_readlane(vlo, s) / kPage;
                nx_b = s;
                nx_pg0 = fp + int(r0 - ex - C);
                nx_pg1 = fp + int(r1 - ex - C);
                const int32_t* row = seq_row(s);
                nx_ids = nx_pg0 + lane < nx_pg1 ? row[nx_pg0 + lane] : 0;
                return true;
            }
            ++s;
        }
    };
    if constexpr (BAL) {
        const int B = min(prm.batch, kWave);
        if (lane < B) {
            seq_view(lane, &vi0, &vrl, &vn);
            vlo = (prm.window > 0 && vn > prm.window) ? vn - prm.window : 0;
            vpages = vn > vlo ? (vn + kPage - 1) / kPage - vlo / kPage : 0;
        }
        violation = (__ballot(violation & PA_DECODE_VIOLATION_ROW) ? PA_DECODE_VIOLATION_ROW : 0) |
                    (__ballot(violation & PA_DECODE_VIOLATION_LENGTH) ? PA_DECODE_VIOLATION_LENGTH : 0);
        vv = vpages > 0 ? vpages + C : 0;
        vincl = wave_incl_scan(vv, lane);
        T = __builtin_amdgcn_readlane(vincl, kWave - 1);
        Weff = min(prm.bal_waves, T);
        if (prel < Weff) {
            rA = floor_div(int64_t(prel) * T, Weff);
            rE = floor_div(int64_t(prel + 1) * T, Weff);
        } else {
            rA = rE = T;
        }
        nonempty = __ballot(vpages > 0);
        // Sequences that end at or before the range start.
        sb = __popcll(__ballot(lane < B && vincl <= rA));
        // Row counts of the KV head's query heads (written by its first
        // wave): the waves from the one holding a sequence's first visible
        // page to the one holding its last.
        if (prel == 0 && lane < B) {
            int c = 0;
            if (vpages > 0) {
                const int64_t ex = vincl - vv;
                c = floor_div(int64_t(vincl) * Weff - 1, T) - floor_div((ex + C + 1) * Weff - 1, T) + 1;
            }
            int32_t* cr = prm.ws_cnt + size_t(lane) * prm.num_q_heads + size_t(kvh) * Gact;
            for (int g = 0; g < Gact; ++g) cr[g] = c;
        }
        nx = find_seg(sb);
    } else {
        // Sequence blockIdx.z, read as seq_view does, but with the row
        // address formed in each branch: a scalar wait for the row stride
        // after the length load is issued would also wait for the length.
        b = blockIdx.z;
        if (prm.page_indptr) {
            const int r0 = prm.page_indptr[b], r1 = prm.page_indptr[b + 1];
            const int i0 = min(max(r0, 0), prm.nnz_pages);
            const int i1 = min(max(r1, i0), prm.nnz_pages);
            violation |= (i0 != r0 || i1 != r1) ? PA_DECODE_VIOLATION_ROW : 0;
            pt_row = prm.page_table + i0;
            row_len = i1 - i0;
            const int last = min(max(prm.last_page_len[b], 0), kPage);
            n = row_len > 0 ? (row_len - 1) * kPage + last : 0;
        } else {
            pt_row = prm.page_table + size_t(b) * prm.pt_stride;
            row_len = prm.pt_stride;
            n = prm.context_lens[b];
        }
        {
            const int nc = min(max(n, 0), prm.max_context_len);
            violation |= nc != n ? PA_DECODE_VIOLATION_LENGTH : 0;
            n = nc;
        }
        // Without a window the partition's first page does not depend on the
        // context length: fetch the page ids together with the length and q.
        if (prm.window <= 0 && prel < prm.num_partitions) {
            const int pgs = prel * (S / kPage);
            ids = load_ids(pgs, min(pgs + S / kPage, row_len), 0);
        }
    }

    // Rotary embedding, relative form.  With q turned to its position m =
    // n - 1 and key j to position j, the score is q . R((j - m) theta) k_j:
    // the key turned by its distance to the query, q as it is.  The lane's
    // token is j = 16 P + i16 for page P, so the angle of frequency i is the
    // page's base (16 P - m) theta_i plus the in-page offset i16 theta_i:
    // for each block the wave writes the bases of its pages to rtab (angle
    // reduced to one turn in f64, then sincos_rev), and the workgroup keeps the (cos, sin)
    // of every offset t theta_i (t < 16) in otab.  Element e of key chunk c
    // (c < CH/2) pairs with element e of chunk c + CH/2; both use frequency
    // i = EPC * c + e.
    constexpr int TS = D + 4;   // otab row stride in floats (16-byte rows, spread banks)
    float* otab = smem + nw * WS;
    double* ftab = reinterpret_cast<double*>(otab + kPage * TS);   // [HD] revolutions per position
    // Revolutions per position of frequency i: theta_i / (2 pi) =
    // rope_f0 * rope_rho^i, by binary powering in f64 (i < 128).
    auto rev_per_pos = [&](int i) {
        double r = prm.rope_f0, x = prm.rope_rho;
#pragma unroll
        for (int bit = 0; bit < 7; ++bit) {
            r = ((i >> bit) & 1) ? r * x : r;
            x *= x;
        }
        return r;
    };
    // Every wave of the workgroup runs this exactly once (it holds the one
    // barrier that publishes otab).  Each thread takes one frequency i
    // (rev_per_pos once) and every T-th offset t of it, T = threads per
    // frequency; with fewer threads than frequencies, several frequencies and
    // all 16 offsets.  The fixed schedule runs it while the wave's first K/V
    // loads are in flight; the balanced schedule before its segments.
    auto rotary_setup = [&]() {
        const int T = int(blockDim.x) >= HD ? int(blockDim.x) / HD : 1;
        const int i0 = int(threadIdx.x) % (T * HD) % HD;
        const int j = int(threadIdx.x) < T * HD ? int(threadIdx.x) / HD : T;
        const int istep = int(blockDim.x) >= HD ? HD : int(blockDim.x);
#pragma unroll 1
        for (int i = i0; j < T && i < HD; i += istep) {
            const double f = rev_per_pos(i);
            if (j == 0)
                ftab[i] = f;
#pragma unroll 1
            for (int t = j; t < kPage; t += T) {
                double x = t * f;
                x -= rint(x);
                float sn, c;
                sincos_rev(float(x), &sn, &c);
                otab[t * TS + 2 * i] = c;
                otab[t * TS + 2 * i + 1] = sn;
            }
        }
        __syncthreads();
    };
    // Rotary tables not yet built by this wave.  Every wave takes part in
    // the build exactly once, before any other barrier of the workgroup:
    // fixed schedule, in its one pass, after its first loads if it has
    // blocks; balanced schedule (no other barrier), after the first loads of
    // its first segment (every segment has blocks), or after the segment
    // loop when it has no segment.
    bool tables_pending = ROT;

    // One segment per pass; the fixed schedule makes exactly one pass.
    for (;;) {
        int t0, t1, pg0, pg1, srow;   // srow: the segment's partition (state row) index
        bool active;
        if constexpr (BAL) {
            // The segment whose page ids were fetched ahead; then the ids of the
            // one after it go out, so that they are in by the time its blocks
            // start.
            if (!nx)
                break;
            b = nx_b;
            pg0 = nx_pg0;
            pg1 = nx_pg1;
            ids = nx_ids;
            n = __builtin_amdgcn_readlane(vn, b);
            row_len = __builtin_amdgcn_readlane(vrl, b);
            pt_row = seq_row(b);
            const int lo = __builtin_amdgcn_readlane(vlo, b);
            t0 = max(pg0 * kPage, lo);
            t1 = min(pg1 * kPage, n);
            active = true;
            const int ex = __builtin_amdgcn_readlane(vincl, b) - __builtin_amdgcn_readlane(vv, b);
            srow = prel - floor_div((int64_t(ex) + C + 1) * Weff - 1, T);
            nx = find_seg(b + 1);
        }
        // q as the MFMA B operand, held in VGPRs: column i16 = query head
        // kvh*G + i16 (zero past G), chunk 4*ks + grp of head_dim.
        u32x4 qa[KS];
        if constexpr (!QKV) {
            const bool real = i16 < Gact;
            const char* qrow = static_cast<const char*>(prm.q) +
                               (size_t(b) * prm.num_q_heads + size_t(kvh) * Gact + (real ? i16 : 0)) * D * EB;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 z = {0u, 0u, 0u, 0u};
                qa[ks] = real ? load16(qrow + (4 * ks + grp) * 16) : z;
            }
        }
        // Comparison build: lane (token i16, group grp) takes chunks 4 ks +
        // grp of every query row of the group (zero rows past G).
        [[maybe_unused]] u32x4 qv[QREG ? G : 1][QREG ? KS : 1];
        [[maybe_unused]] u32x4* qcopy =
            reinterpret_cast<u32x4*>(smem + wave * WS + 8 * KT + (ROT ? NB * D : 0));
        [[maybe_unused]] float* sbuf =
            smem + wave * WS + 8 * KT + (ROT ? NB * D : 0) + (QREG ? 0 : G * CH * 4);
        if constexpr (QKV) {
            const char* q0 = static_cast<const char*>(prm.q) +
                             (size_t(b) * prm.num_q_heads + size_t(kvh) * Gact) * D * EB;
            const u32x4 z = {0u, 0u, 0u, 0u};
            if constexpr (QREG) {
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        qv[g][ks] = g < Gact ? load16(q0 + (size_t(g) * CH + 4 * ks + grp) * 16) : z;
            } else {
                for (int x = lane; x < G * CH; x += kWave)
                    qcopy[x] = x / CH < Gact ? load16(q0 + size_t(x) * 16) : z;
                wave_lds_sync();
            }
        }

        if constexpr (!BAL) {
            const int lo = (prm.window > 0 && n > prm.window) ? n - prm.window : 0;
            const int pabs = lo / S + prel;
            t0 = max(pabs * S, lo);
            t1 = min(pabs * S + S, n);
            active = prel < prm.num_partitions && t0 < t1;
            pg0 = t0 / kPage;
            pg1 = (t1 + kPage - 1) / kPage;
            srow = prel;
            if (prm.window > 0 && active)
                ids = load_ids(pg0, pg1, 0);
        }

        const int64_t ss = prm.stride_slot;
        const char* kbase = static_cast<const char*>(prm.k) + int64_t(kvh) * prm.stride_head * EB;
        const char* vbase = static_cast<const char*>(prm.v) + int64_t(kvh) * prm.stride_head * EB;

        // Online-softmax state of head i16 (the same in the four lane groups;
        // the denominator holds the lane's own tokens until the end).
        float m_run = -INFINITY, l_run = 0.f;
        f32x4 acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4* ktile = reinterpret_cast<u32x4*>(smem + wave * WS);
        u32x4* vtile = ktile + KT;
        float2* rtab = reinterpret_cast<float2*>(vtile + KT);   // ROT: [NB][HD] (cos, sin)
        // Tile layout (K and V alike): chunk j of tile row r (page r / 16, token
        // r % 16) sits at slot tix(r, j).  Power-of-two rows: r * CH + (j ^
        // swz(r)), where swz permutes within aligned groups of 8 chunks, so a
        // 128-byte line still lands whole, and the 16 rows one read touches fall
        // in distinct 16-byte bank groups.  12-chunk rows (head_dim 96): rows
        // padded to an odd 13 slots, which spreads 16 consecutive rows over all
        // 16 bank groups without a swizzle.
        auto swz = [](int r) { return CH >= 16 ? (r & 15) : ((r >> 1) & 7); };
        auto tix = [&](int r, int j) {
            if constexpr (POW2) return r * CH + (j ^ swz(r));
            else return r * CHP + j;
        };

        // Bases of the block's pages: entry nb * HD + i of rtab.
        auto fill_bases = [&](int pgb) {
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                const int e = lane + kWave * k;
                if (NE * kWave == NB * HD || e < NB * HD) {
                    const int pos = (pgb + e / HD) * kPage - (n - 1);
                    double x = double(pos) * ftab[e % HD];
                    x -= rint(x);
                    float sn, c;
                    sincos_rev(float(x), &sn, &c);
                    rtab[e] = make_float2(c, sn);
                }
            }
        };
        // The score MFMAs of page nb with turned keys.
        auto turned_scores = [&](int nb) {
            using TK = TurnedKey<DT>;
            static_assert(TK::EPC == EPC, "turned-key chunk width");
            const int row = nb * kPage + i16;
            const float2* bt = rtab + nb * HD;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            const float2* ot = reinterpret_cast<const float2*>(otab + i16 * TS);
            auto angle = [&](int i0, float (&cs)[EPC], float (&sn)[EPC]) {
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const float2 bb = bt[i0 + e], oo = ot[i0 + e];
                    cs[e] = bb.x * oo.x - bb.y * oo.y;
                    sn[e] = bb.y * oo.x + bb.x * oo.y;
                }
            };
            if constexpr (KS % 2 == 0) {
                // Chunk fs (first half) and fs + KS/2 (second half) of the lane.
#pragma unroll
                for (int fs = 0; fs < KS / 2; ++fs) {
                    if constexpr (KS >= 8) {
                        if (fs > 0)
                            pin_loads();   // head_dim 256: one chunk pair at a time
                    }
                    float cs[EPC], sn[EPC];
                    angle(EPC * (4 * fs + grp), cs, sn);
                    const u32x4 xc = ktile[tix(row, 4 * fs + grp)];
                    const u32x4 yc = ktile[tix(row, 4 * (fs + KS / 2) + grp)];
                    if constexpr (DT != PA_DTYPE_F32) {
                        d = TK::turn_mfma(xc, yc, cs, sn, qa[fs], qa[fs + KS / 2], d, prm.minus_one);
                    } else {
                        float x[EPC], y[EPC], xr[EPC], yr[EPC];
                        TK::widen(xc, x);
                        TK::widen(yc, y);
#pragma unroll
                        for (int e = 0; e < EPC; ++e) {
                            xr[e] = x[e] * cs[e] - y[e] * sn[e];
                            yr[e] = y[e] * cs[e] + x[e] * sn[e];
                        }
                        d = TK::mfma(xr, qa[fs], d);
                        d = TK::mfma(yr, qa[fs + KS / 2], d);
                    }
                }
            } else {
                // Odd chunk count (head_dim 96): the partner chunk of the other
                // half is a second LDS read.
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c = 4 * ks + grp;
                    const bool first = c < CH / 2;
                    float cs[EPC], sn[EPC], x[EPC], y[EPC], xr[EPC];
                    angle(EPC * (first ? c : c - CH / 2), cs, sn);
                    TK::widen(ktile[tix(row, c)], x);
                    TK::widen(ktile[tix(row, first ? c + CH / 2 : c - CH / 2)], y);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) xr[e] = x[e] * cs[e] + (first ? -y[e] : y[e]) * sn[e];
                    d = TK::mfma(xr, qa[ks], d);
                }
            }
            return d;
        };

        const int nblk = active ? (pg1 - pg0 + NB - 1) / NB : 0;
        const int nit = nblk > wi ? (nblk - wi + wpp - 1) / wpp : 0;

        // Software pipeline over the wave's blocks: as soon as block it's K and V
        // rows are in the LDS tiles, the registers take block it+1's loads, so the
        // loads of one block are in flight while the previous block is computed.
        // Every phase issues exactly 2*NB*KS loads, with no branch around the
        // individual pages, so that each wait leaves the younger loads in flight:
        // a page past the end of a short block gets a zero lane offset, i.e. all
        // lanes read one 16-byte piece of a page.  The last step of a chunk
        // issues nothing (one wave-uniform branch), which shortens the
        // single-block waves of short contexts.
        u32x4 kr[NB][KS], vr[NB][KS];
        int64_t page[NB];
        uint32_t pmask[NB];
        // Byte offset of this lane's chunk of load instruction i in a page.  For
        // power-of-two rows it is loff[0] + i * lstep, with a wave-uniform step
        // (instruction i reads rows R*i + lane/CH), so one VGPR holds them all.
        uint32_t loff[POW2 ? 1 : KS];
#pragma unroll
        for (int i = 0; i < (POW2 ? 1 : KS); ++i)
            loff[i] = uint32_t((int64_t(lrow(i)) * ss + int64_t(lchk(i)) * EPC) * EB);
        const uint32_t lstep = uint32_t(int64_t(R) * ss * EB);
        auto fetch_ids = [&](int itn, int it0, int it1) {
            // Page ids of block `itn` into scalar registers (ids holds the blocks
            // it0 .. it0 + IPV - 1).
            const int itc = min(itn, it1 - 1);
            const int nbv_ = itn < it1 ? min(NB, pg1 - (pg0 + (wi + wpp * itn) * NB)) : 0;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // A page id outside the pool reads page 0 instead (reported
                // when it belongs to the block; ids past the block are padding).
                const int id = __builtin_amdgcn_readlane(ids, (itc - it0) * NB + nb);
                const bool ok = uint32_t(id) < uint32_t(prm.num_pages);
                violation |= (ok || nb >= nbv_) ? 0 : PA_DECODE_VIOLATION_PAGE;
                page[nb] = ok ? id : 0;
                uint32_t m = __builtin_amdgcn_readfirstlane(nb < nbv_ ? ~0u : 0u);
                asm volatile("" : "+s"(m));  // an opaque mask, not a branch condition
                pmask[nb] = m;
            }
        };
        auto issue = [&](const char* base, u32x4 (&r)[NB][KS]) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const char* pb = base + page[nb] * prm.stride_page * EB;
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    if constexpr (POW2)
                        r[nb][i] = load16_stream(pb + ((uint32_t(i) * lstep) & pmask[nb]) +
                                                 (loff[0] & pmask[nb]));
                    else
                        r[nb][i] = load16_stream(pb + (loff[i] & pmask[nb]));
                }
            }
        };
        // Registers -> swizzled tile; V rows of tokens outside [t0, t1) (or of
        // pages past the block's end) become zero, so that slots the method must
        // not read never reach the output (their probabilities are already 0).
        auto stage = [&](u32x4* tile, const u32x4 (&r)[NB][KS], bool zero_invalid, int pgb, int nbv) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    const int row = nb * kPage + lrow(i);
                    u32x4 x = r[nb][i];
                    if (zero_invalid) {
                        const int tok = (pgb + nb) * kPage + lrow(i);
                        const u32x4 z = {0u, 0u, 0u, 0u};
                        x = (nb < nbv && tok >= t0 && tok < t1) ? x : z;
                    }
                    tile[tix(row, lchk(i))] = x;
                }
        };

        // One pipeline step: block it's rows go from the registers to the tiles,
        // the registers take block it+1's loads, then block it is computed.
        auto step = [&](int it, int it0, int it1) {
            const int pgb = pg0 + (wi + wpp * it) * NB;
            const int nbv = min(NB, pg1 - pgb);
            // Edge blocks only (partition or window ends, short blocks) need
            // the V mask (wave-uniform).
            const bool edge = nbv < NB || pgb * kPage < t0 || (pgb + NB) * kPage > t1;

            if constexpr (ROT)
                fill_bases(pgb);
            stage(ktile, kr, false, pgb, nbv);
            if (edge)
                stage(vtile, vr, true, pgb, nbv);
            else
                stage(vtile, vr, false, pgb, nbv);
            wave_lds_sync();
            if (it + 1 < it1) {
                // The next block of this chunk (the loads of a following chunk
                // are issued once its page ids are in).
                fetch_ids(it + 1, it0, it1);
                issue(kbase, kr);
                pin_loads();
                issue(vbase, vr);
                pin_loads();
            }

            // Without rotary, every K tile read of the block goes out before
            // the first score MFMA, and every V transpose read (P.V operand)
            // right after the score MFMAs, so that each LDS latency is paid
            // once per block rather than once per page (32 VGPRs each).
            constexpr bool PRE = !ROT && !QKV && DT != PA_DTYPE_F32;
            [[maybe_unused]] u32x4 kt[PRE ? NB : 1][PRE ? KS : 1];
            if constexpr (PRE) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) kt[nb][ks] = ktile[tix(nb * kPage + i16, 4 * ks + grp)];
                pin_loads();
            }

            // Scores (base 2) of head i16 against token 4*grp + r of each page.
            float s[NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
                if constexpr (ROT) {
                    // One page at a time: the turned keys of a page take ~90
                    // VGPRs while they are formed.
                    pin_loads();
                    d = turned_scores(nb);
                } else if constexpr (QKV) {
                    // Lane (token i16, group grp): partial dots of its key row's
                    // chunks 4 ks + grp with every query row, summed over the four
                    // groups by lane swaps, then written [head][token] and read back
                    // as (head i16, tokens 4 grp .. 4 grp + 3).
                    float part[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) part[g] = 0.f;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const u32x4 kc = ktile[tix(nb * kPage + i16, 4 * ks + grp)];
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            u32x4 qc;
                            if constexpr (QREG) qc = qv[g][ks];
                            else qc = qcopy[g * CH + 4 * ks + grp];
                            part[g] = Dot<DT>::dot(kc, qc, part[g]);
                        }
                    }
                    float* sb = sbuf + nb * 256;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        part[g] = rows4_sum(part[g]);
                        if (grp == 0) sb[g * 16 + i16] = part[g];
                    }
                    wave_lds_sync();
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    d = i16 < G ? *reinterpret_cast<const f32x4*>(sb + i16 * 16 + 4 * grp) : z;
                } else if constexpr (PRE) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) d = Chunk<DT>::mfma(kt[nb][ks], qa[ks], d);
                } else {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        d = Chunk<DT>::mfma(ktile[tix(nb * kPage + i16, 4 * ks + grp)], qa[ks], d);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) s[nb][r] = d[r] * prm.scale_log2;
            }

            // P.V operand reads: V rows 4*grp + i16/4 of each page, columns
            // 16*db + 4*(i16%4) .. +3 through the LDS transpose read.
            auto tr_read = [&](int nb, int db) -> s16x4 {
                const int vrow = nb * kPage + 4 * grp + (i16 >> 2);
                const int j = 2 * db + ((i16 & 3) >> 1);
                const char* addr = reinterpret_cast<const char*>(vtile + tix(vrow, j)) + (i16 & 1) * 8;
                return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(addr));
            };
            [[maybe_unused]] s16x4 vt[PRE ? NB : 1][PRE ? NDB : 1];
            if constexpr (PRE) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) vt[nb][db] = tr_read(nb, db);
                pin_loads();
            }
            auto vop = [&](int nb, int db) -> s16x4 {
                if constexpr (PRE) return vt[nb][db];
                else return tr_read(nb, db);
            };
            // Tokens outside [t0, t1) and pages past the block's end score
            // -inf; only edge blocks have any (wave-uniform branch).
            if (edge) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tok = (pgb + nb) * kPage + 4 * grp + r;
                        const bool ok = nb < nbv && tok >= t0 && tok < t1;
                        s[nb][r] = ok ? s[nb][r] : -INFINITY;
                    }
            }

            // Block maximum of head i16: the lane's own 4*NB scores, then the
            // four lane groups.
            float bm = s[0][0];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[nb][r]);
            bm = rows4_max(bm);
            // The reference value m_run the exponentials are taken against
            // moves only when the block maximum passes it by more than
            // kSlack (so p <= 2^kSlack, exact in f16 / bf16 hi+lo and f32);
            // the state (m, l, acc) is exact for any reference, since the
            // result is acc / l and m + log2(l).  The output accumulators
            // then need rescaling only on those rare moves (wave-uniform
            // decision).
            const bool grow = bm > m_run + kSlack;
            const float mnew = grow ? bm : m_run;
            const float alpha = grow ? fast_exp2(m_run - bm) : 1.f;
            const bool any_rescale = __any(grow && i16 < G);
            float ps = 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    s[nb][r] = fast_exp2(s[nb][r] - mnew);
                    ps += s[nb][r];
                }
            l_run = alpha * l_run + ps;
            m_run = mnew;

            if (any_rescale) {
                // Row 4*grp + r of the output blocks is head 4*grp + r, whose
                // alpha sits in lane 4*grp + r.
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = __shfl(alpha, 4 * grp + r);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db][r] *= a;
                }
            }

            // P.V on the matrix cores.
            if constexpr (DT == PA_DTYPE_F32) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    // 16x16x4 f32 steps: step r takes token 4*grp + r of every
                    // lane group (k index grp).
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = nb * kPage + 4 * grp + r;
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int col = 16 * db + i16;
                            const float v = reinterpret_cast<const float*>(vtile + tix(row, col >> 2))[col & 3];
                            acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(s[nb][r], v, acc[db], 0, 0, 0);
                        }
                    }
                }
            } else if constexpr (NB % 2 == 0) {
                // Pages in pairs: 32 tokens per MFMA (the same issue cost as 16).
#pragma unroll
                for (int nb = 0; nb < NB; nb += 2) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        acc[db] = PV2<DT>::mma(s[nb], s[nb + 1], vop(nb, db), vop(nb + 1, db), acc[db]);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db] = PV<DT>::mma(s[nb], vop(nb, db), acc[db]);
                }
            }
        };

        // Outer loop over chunks of IPV blocks (one page-id vector each); the
        // pipelined inner loop itself issues no load but K/V.  With rotary
        // (fixed schedule) the first chunk's first loads go out before the
        // workgroup builds its rotary tables, so the two overlap.
        bool first_issued = false;
        if constexpr (ROT) {
            if (tables_pending) {
                if (nit > 0) {
                    fetch_ids(0, 0, min(nit, IPV));
                    issue(kbase, kr);
                    pin_loads();
                    issue(vbase, vr);
                    pin_loads();
                    first_issued = true;
                }
                rotary_setup();
                tables_pending = false;
            }
        }
        for (int it0 = 0; it0 < nit; it0 += IPV) {
            const int it1 = min(nit, it0 + IPV);
            if (it0 > 0 || !first_issued) {
                if (it0 > 0)
                    ids = load_ids(pg0, pg1, it0);
                fetch_ids(it0, it0, it1);
                issue(kbase, kr);
                pin_loads();
                issue(vbase, vr);
                pin_loads();
            }
            for (int it = it0; it < it1; ++it) step(it, it0, it1);
        }  // chunks of IPV blocks

        if constexpr (!BAL) {
            if (prm.status && violation != 0 && lane == 0)
                __hip_atomic_fetch_or(prm.status, violation, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // Denominator of head i16 over the four lane groups.
        l_run = rows4_sum(l_run);

        // Results: per (query head g of the group, partition) the partition
        // state (o normalised, max, denominator) for the merge, or, when one
        // partition covers the context, out and lse (an empty context gives
        // out = 0, lse = -inf).  Head g's rows: ws_o + (h0 + g) P D + p D,
        // ws_m / ws_l + (h0 + g) P + p, out + (h0 + g) D.  The split / out
        // choice is one uniform branch around each store sequence, and the
        // stores run from one base address with constant offsets.
        const size_t h0 = size_t(b) * prm.num_q_heads + size_t(kvh) * Gact;
        const int P = prm.num_partitions;
#if PA_FUSED_MERGE
        // Comparison build: once every thread's state stores (written through
        // to memory) have completed, one agent-scope add per workgroup on the
        // (sequence, KV head) counter; the workgroup that completes the count
        // takes an agent-scope acquire fence (the L2 lines it may hold of
        // the states are dropped), stages the group's maxima and denominators
        // in LDS, forms each partition's weight 2^(m_p - M) l_p once, and
        // sums the weighted state rows with float4 loads, as the merge kernels
        // do; then it clears the counter for the next call.
        auto fused_tail = [&]() {
            if (!prm.split)
                return;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            int* flag = reinterpret_cast<int*>(smem);
            int32_t* cnt = prm.ws_cnt + size_t(b) * gridDim.y + kvh;
            if (threadIdx.x == 0) {
                const int valid = min(nslots, P - int(blockIdx.x) * nslots);
                const int old = __hip_atomic_fetch_add(cnt, valid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                *flag = old + valid == P;
            }
            __syncthreads();
            if (!*flag)
                return;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const int GP = Gact * P, bd = blockDim.x, tid = threadIdx.x;
            float* wm = smem + 4;          // [Gact][P]: maxima, then weights
            float* wl = wm + GP;           // [Gact][P]: denominators
            float* hM = wl + GP;           // [Gact]
            float* hL = hM + 16;           // [Gact]
            for (int e = tid; e < GP; e += bd) {
                const size_t row = (h0 + e / P) * P + e % P;
                wm[e] = prm.ws_m[row];
                wl[e] = prm.ws_l[row];
            }
            __syncthreads();
            for (int g = tid; g < Gact; g += bd) {
                float M = -INFINITY;
                for (int p = 0; p < P; ++p) M = fmaxf(M, wm[g * P + p]);
                hM[g] = M;
            }
            __syncthreads();
            for (int e = tid; e < GP; e += bd) {
                const float M = hM[e / P], l = wl[e];
                wm[e] = (M != -INFINITY && l > 0.f) ? fast_exp2(wm[e] - M) * l : 0.f;
            }
            __syncthreads();
            for (int g = tid; g < Gact; g += bd) {
                float L = 0.f;
                for (int p = 0; p < P; ++p) L += wm[g * P + p];
                hL[g] = L;
            }
            __syncthreads();
            constexpr int D4 = D / 4;
            for (int e = tid; e < Gact * D4; e += bd) {
                const int g = e / D4, c = 4 * (e % D4);
                const size_t h = h0 + g;
                const float* orow = prm.ws_o + h * P * D + c;
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
                for (int p = 0; p < P; ++p)
                    o += wm[g * P + p] * *reinterpret_cast<const f32x4*>(orow + size_t(p) * D);
                const float M = hM[g], L = hL[g];
                if (M != -INFINITY)
                    o *= 1.f / L;
                store_out4<DT>(prm.out, h * D + c, o);
                if (c == 0 && prm.lse)
                    prm.lse[h] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
            }
            if (tid == 0)
                __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
#endif

        if (wpp == 1) {
            // Every wave owns its partition: write straight from the output
            // blocks (row 4*grp + r of block db is head 4*grp + r, column
            // 16*db + i16); the max and denominator of head 4*grp + r sit in
            // lane 4*grp + r.  No LDS, no barrier.
            if (uint32_t(srow) < uint32_t(P)) {
                float Mr[4], Lr[4], inv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Mr[r] = __shfl(m_run, 4 * grp + r);
                    Lr[r] = __shfl(l_run, 4 * grp + r);
                    inv[r] = Mr[r] == -INFINITY ? 0.f : __builtin_amdgcn_rcpf(Lr[r]);
                }
                if (prm.split) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int g = 4 * grp + r;
                        if (g < Gact) {
                            float* o = prm.ws_o + ((h0 + g) * P + srow) * D + i16;
#pragma unroll
                            for (int db = 0; db < NDB; ++db) st_state(o + 16 * db, acc[db][r] * inv[r]);
                            if (i16 == 0) {
                                st_state(prm.ws_m + (h0 + g) * P + srow, Mr[r]);
                                st_state(prm.ws_l + (h0 + g) * P + srow, Lr[r]);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int g = 4 * grp + r;
                        if (g < Gact) {
#pragma unroll
                            for (int db = 0; db < NDB; ++db)
                                store_out<DT>(prm.out, (h0 + g) * D + 16 * db + i16, acc[db][r] * inv[r]);
                            if (i16 == 0 && prm.lse)
                                prm.lse[h0 + g] = Mr[r] == -INFINITY ? -INFINITY : (Mr[r] + log2f(Lr[r])) * kLn2;
                        }
                    }
                }
            }
            if constexpr (BAL)
                continue;
#if PA_FUSED_MERGE
            fused_tail();
#endif
            return;
        }

        // Several waves share each partition: combine them in LDS, maximum
        // first, then the rescaled denominators and outputs.  A wave without
        // blocks holds max = -inf, denominator 0 and contributes nothing; a slot
        // whose partition is empty ends with max = -inf.
        __syncthreads();
        float* cm = smem;               // [nw][GP4]
        float* cl = cm + nw * GP4;      // [nw][GP4]
        float* ca = cl + nw * GP4;      // [nw][G][D]
        if (grp == 0 && i16 < G) {
            cm[wave * GP4 + i16] = m_run;
            cl[wave * GP4 + i16] = l_run;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int g = 4 * grp + r;
            if (g < G) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) ca[(wave * G + g) * D + 16 * db + i16] = acc[db][r];
            }
        }
        __syncthreads();

        // One thread per (slot, head, 4 consecutive columns): the slot's
        // waves' weights 2^(m_w - M), the denominator, then a float4 of the
        // output from float4 LDS reads and one 16-byte (8-byte) store.
        constexpr int D4 = D / 4;
        const int items = nslots * Gact * D4;
        for (int e = threadIdx.x; e < items; e += blockDim.x) {
            const int sl = e / (Gact * D4);
            const int g = (e / D4) % Gact;
            const int c = 4 * (e % D4);
            const int p_rel = blockIdx.x * nslots + sl;
            if (p_rel >= P)
                continue;
            const int w0 = sl * wpp;
            float M = -INFINITY;
            for (int w = w0; w < w0 + wpp; ++w) M = fmaxf(M, cm[w * GP4 + g]);
            float L = 0.f;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            if (M != -INFINITY) {
                for (int w = w0; w < w0 + wpp; ++w) {
                    const float sc = fast_exp2(cm[w * GP4 + g] - M);
                    L += sc * cl[w * GP4 + g];
                    o += sc * *reinterpret_cast<const f32x4*>(ca + (w * G + g) * D + c);
                }
                o *= __builtin_amdgcn_rcpf(L);
            }
            if (prm.split) {
                st_state4(prm.ws_o + ((h0 + g) * P + p_rel) * D + c, o);
                if (c == 0) {
                    st_state(prm.ws_m + (h0 + g) * P + p_rel, M);
                    st_state(prm.ws_l + (h0 + g) * P + p_rel, L);
                }
            } else {
                store_out4<DT>(prm.out, (h0 + g) * D + c, o);
                if (c == 0 && prm.lse)
                    prm.lse[h0 + g] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
            }
        }
#if PA_FUSED_MERGE
        fused_tail();
#endif
        return;
    }  // segments

    if constexpr (ROT && BAL) {
        if (tables_pending)
            rotary_setup();   // a wave without segments still joins the build's barrier
    }
    if (prm.status && violation != 0 && lane == 0)
        __hip_atomic_fetch_or(prm.status, violation, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Launch through hipExtLaunchKernelGGL so optional start/stop events bracket
// the kernel itself.
template <typename K, typename... Args>
hipError_t launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  LaunchEvents ev, const Args&... args)
{
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds), stream, ev.start, ev.stop, 0,
                              args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    return hipGetLastError();
}

// Pages per block: the planner's rule (pages_per_block_for_row).
template <int DT, int D>
constexpr int pages_per_block_t()
{
    return pages_per_block_for_row(D * Elt<DT>::bytes);
}

template <bool BAL, int DT, int D, int G>
hipError_t launch_partial_t(bool rot, const PartialParams& p, dim3 grid, dim3 block, size_t lds,
                            hipStream_t stream, LaunchEvents ev)
{
    constexpr int NB = pages_per_block_t<DT, D>();
    if (rot)
        return launch(partial_kernel<DT, D, G, NB, true, BAL>, grid, block, lds, stream, ev, p);
    return launch(partial_kernel<DT, D, G, NB, false, BAL>, grid, block, lds, stream, ev, p);
}

template <bool BAL, int DT, int D, int G>
int waves_per_cu_t(bool rot, int waves, size_t lds)
{
    constexpr int NB = pages_per_block_t<DT, D>();
    const void* k = rot ? reinterpret_cast<const void*>(partial_kernel<DT, D, G, NB, true, BAL>)
                        : reinterpret_cast<const void*>(partial_kernel<DT, D, G, NB, false, BAL>);
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, waves * kWave, lds) != hipSuccess)
        return 0;
    return blocks * waves;
}

template <bool BAL, int DT, int D>
int waves_per_cu_g(int group_t, bool rot, int waves, size_t lds)
{
    switch (group_t) {
    case 1: return waves_per_cu_t<BAL, DT, D, 1>(rot, waves, lds);
    case 2: return waves_per_cu_t<BAL, DT, D, 2>(rot, waves, lds);
    case 4: return waves_per_cu_t<BAL, DT, D, 4>(rot, waves, lds);
    case 6: return waves_per_cu_t<BAL, DT, D, 6>(rot, waves, lds);
    case 8: return waves_per_cu_t<BAL, DT, D, 8>(rot, waves, lds);
    case 16: return waves_per_cu_t<BAL, DT, D, 16>(rot, waves, lds);
    default: return 0;
    }
}

template <bool BAL, int DT, int D>
hipError_t launch_partial_g(int group_t, bool rot, const PartialParams& p, dim3 grid, dim3 block,
                            size_t lds, hipStream_t stream, LaunchEvents ev)
{
    switch (group_t) {
    case 1: return launch_partial_t<BAL, DT, D, 1>(rot, p, grid, block, lds, stream, ev);
    case 2: return launch_partial_t<BAL, DT, D, 2>(rot, p, grid, block, lds, stream, ev);
    case 4: return launch_partial_t<BAL, DT, D, 4>(rot, p, grid, block, lds, stream, ev);
    case 6: return launch_partial_t<BAL, DT, D, 6>(rot, p, grid, block, lds, stream, ev);
    case 8: return launch_partial_t<BAL, DT, D, 8>(rot, p, grid, block, lds, stream, ev);
    case 16: return launch_partial_t<BAL, DT, D, 16>(rot, p, grid, block, lds, stream, ev);
    default: return hipErrorInvalidValue;
    }
}

template <bool BAL>
hipError_t launch_partial_any(int dtype, int head_dim, int group_t, const PartialParams& p,
                              dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                              LaunchEvents ev)
{
    const bool rot = p.rotary != 0;
#define PA_PARTIAL(DT, D) return launch_partial_g<BAL, DT, D>(group_t, rot, p, grid, block, lds, stream, ev);
    if (dtype == PA_DTYPE_F32 && head_dim == 64) { PA_PARTIAL(PA_DTYPE_F32, 64) }
    if (dtype == PA_DTYPE_F16) {
        if (head_dim == 64) { PA_PARTIAL(PA_DTYPE_F16, 64) }
        if (head_dim == 96) { PA_PARTIAL(PA_DTYPE_F16, 96) }
        if (head_dim == 128) { PA_PARTIAL(PA_DTYPE_F16, 128) }
        if (head_dim == 256) { PA_PARTIAL(PA_DTYPE_F16, 256) }
    }
    if (dtype == PA_DTYPE_BF16) {
        if (head_dim == 64) { PA_PARTIAL(PA_DTYPE_BF16, 64) }
        if (head_dim == 96) { PA_PARTIAL(PA_DTYPE_BF16, 96) }
        if (head_dim == 128) { PA_PARTIAL(PA_DTYPE_BF16, 128) }
        if (head_dim == 256) { PA_PARTIAL(PA_DTYPE_BF16, 256) }
    }
#undef PA_PARTIAL
    return hipErrorInvalidValue;
}

template <bool BAL>
int partial_waves_any(int dtype, int head_dim, int group_t, bool rotary, int waves, size_t lds)
{
#define PA_OCC(DT, D) return waves_per_cu_g<BAL, DT, D>(group_t, rotary, waves, lds);
    if (dtype == PA_DTYPE_F32 && head_dim == 64) { PA_OCC(PA_DTYPE_F32, 64) }
    if (dtype == PA_DTYPE_F16) {
        if (head_dim == 64) { PA_OCC(PA_DTYPE_F16, 64) }
        if (head_dim == 96) { PA_OCC(PA_DTYPE_F16, 96) }
        if (head_dim == 128) { PA_OCC(PA_DTYPE_F16, 128) }
        if (head_dim == 256) { PA_OCC(PA_DTYPE_F16, 256) }
    }
    if (dtype == PA_DTYPE_BF16) {
        if (head_dim == 64) { PA_OCC(PA_DTYPE_BF16, 64) }
        if (head_dim == 96) { PA_OCC(PA_DTYPE_BF16, 96) }
        if (head_dim == 128) { PA_OCC(PA_DTYPE_BF16, 128) }
        if (head_dim == 256) { PA_OCC(PA_DTYPE_BF16, 256) }
    }
#undef PA_OCC
    return 0;
}

}  // namespace
}  // namespace pa
