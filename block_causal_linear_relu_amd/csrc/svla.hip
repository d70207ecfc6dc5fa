// libsvla -- block-causal ReLU linear attention for AMD Instinct MI355X (gfx950).
//
// The C ABI is declared in include/svla.h, which states the method and cites
// the SANA-Video pages that define it.  This file holds the three kernels of
// the path and the host code around them:
//
//   svla_state_build   per (b,h,block,split): S_part = sum_j R_j phi(k_j) (x) v_j
//                      and z_part = sum_j phi(k_j) on bf16 (or fp32) MFMA with
//                      fp32 accumulation; K/V tiles staged in LDS from
//                      coalesced 128-bit buffer loads.
//   svla_state_scan    per (b,h,state tile): sums the split partials and takes
//                      the inclusive, optionally decayed prefix over blocks;
//                      writes each block's state in the register layout the
//                      apply kernel feeds to the matrix cores, and the final
//                      state.
//   svla_apply         per (b,h,block,token tile): O = phi~(Q) S / (phi(Q) z + eps)
//                      with O^T = S^T phi~(Q)^T on MFMA, the denominator on the
//                      vector ALU, RoPE on the numerator operand only.
//
// Every global access of the hot kernels goes through a buffer resource
// sized to the (b,h) slice it belongs to: a lane whose token lies past the
// end of its range is given an offset past the resource and reads zeros /
// drops its store.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <type_traits>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/svla.h"

// Tuning knobs (compile-time; the defaults are the measured choices).
#ifndef SVLA_DMA_WGS
#define SVLA_DMA_WGS 420           // state build without RoPE: workgroups wanted per launch
#endif
#ifndef SVLA_DMA_U32
#define SVLA_DMA_U32 1             // ... d = 32: 16-byte loads per thread per tensor per stage
#endif
#ifndef SVLA_DMA_R32
#define SVLA_DMA_R32 3             // ... and LDS ring depth
#endif
#ifndef SVLA_DMA_U
#define SVLA_DMA_U 1               // the same for d = 64, 128
#endif
#ifndef SVLA_DMA_R
#define SVLA_DMA_R 4               // ... ring depth for d = 64
#endif
#ifndef SVLA_DMA_R128
#define SVLA_DMA_R128 3            // ... and for d = 128
#endif
#ifndef SVLA_DMA_U128
#define SVLA_DMA_U128 SVLA_DMA_U   // ... 16-byte loads per thread per tensor per stage at d = 128
#endif
#ifndef SVLA_MIN_SPLIT_ROPE
#define SVLA_MIN_SPLIT_ROPE 5      // builds with RoPE: tokens per split >= this * d
#endif
#ifndef SVLA_MIN_SPLIT_128
#define SVLA_MIN_SPLIT_128 1       // d = 128 build without RoPE: tokens per split >= this * d
#endif
#ifndef SVLA_FOLD_MAX_PARTS
#define SVLA_FOLD_MAX_PARTS 8      // one-block calls: partials the apply sums itself (no scan) at most
#endif
#ifndef SVLA_FOLD_MAX_PARTS_ROPE
#define SVLA_FOLD_MAX_PARTS_ROPE 8 // ... with RoPE
#endif
#ifndef SVLA_ROPE_PF
#define SVLA_ROPE_PF 3             // state build with RoPE: stages in flight per wave
#endif
#ifndef SVLA_ROPE_U
#define SVLA_ROPE_U 1              // ... 16-byte loads per lane per tensor per stage (2 at d >= 64)
#endif
#ifndef SVLA_ROPE_WGS
#define SVLA_ROPE_WGS 2048         // ... (and fp32 builds): workgroups wanted per launch
#endif
#ifndef SVLA_F8_WGS
#define SVLA_F8_WGS 420            // fp8 state build without RoPE: workgroups wanted per launch
#endif
#ifndef SVLA_MIN_SPLIT_PER_D
#define SVLA_MIN_SPLIT_PER_D 8     // tokens per build workgroup and block >= this * d
#endif
#ifndef SVLA_APPLY_TILE32
#define SVLA_APPLY_TILE32 256      // apply: tokens per workgroup for bf16 d = 32 and fp32 d = 32, 64
#endif
#ifndef SVLA_APPLY_TILE_FOLD
#define SVLA_APPLY_TILE_FOLD 512   // ... bf16 d = 32 with the scan folded in (one-block calls)
#endif
#ifndef SVLA_APPLY_TILE_FOLD_ROPE
#define SVLA_APPLY_TILE_FOLD_ROPE 192   // ... and with RoPE (latency-bound block steps: more workgroups)
#endif
#ifndef SVLA_APPLY_TILE_ROPE
#define SVLA_APPLY_TILE_ROPE 512   // ... with RoPE (amortises the per-workgroup angle table)
#endif
#ifndef SVLA_APPLY_TILE128
#define SVLA_APPLY_TILE128 128     // ... fp32, d = 128
#endif
#ifndef SVLA_APPLY32_PF
#define SVLA_APPLY32_PF 4          // ... d = 32: 16-token groups of Q loads in flight per wave
#endif
#ifndef SVLA_APPLY32_PF_ROPE
#define SVLA_APPLY32_PF_ROPE 4     // ... and with RoPE
#endif
#ifndef SVLA_APPLY_TILE_LDS
#define SVLA_APPLY_TILE_LDS 256    // bf16 apply with the state in LDS (d >= 64): tokens per workgroup
#endif
#ifndef SVLA_APPLY_RING_PF
#define SVLA_APPLY_RING_PF 2       // bf16 apply, d >= 64: groups of Q in flight per wave (LDS slots)
#endif
#ifndef SVLA_APPLY_XCD
#define SVLA_APPLY_XCD 1           // apply: the token tiles of one block on one XCD
#endif
#ifndef SVLA_TCONV_MAXF
#define SVLA_TCONV_MAXF 4          // temporal convolution: frames per chunk (loads in flight per thread)
#endif
#ifndef SVLA_TCONV_XAUX
#define SVLA_TCONV_XAUX 2          // ... cache policy of the X loads (non-temporal: read once)
#endif
#ifndef SVLA_TCONV_YAUX
#define SVLA_TCONV_YAUX 2          // ... and of the Y stores (non-temporal)
#endif
#ifndef SVLA_FUSED_MAX_N
#define SVLA_FUSED_MAX_N 3072      // one-launch block step (bf16, d = 32): longest block
#endif
#ifndef SVLA_FUSED_WGS
#define SVLA_FUSED_WGS 256         // ... workgroups per launch at most (one per CU), unless B*H is larger
#endif
#ifndef SVLA_FUSED_W
#define SVLA_FUSED_W 16            // ... waves per workgroup
#endif
#ifndef SVLA_FUSED_PF
#define SVLA_FUSED_PF 3            // ... K/V stages in flight per wave (without RoPE)
#endif
#ifndef SVLA_FUSED_PF_ROPE
#define SVLA_FUSED_PF_ROPE 2       // ... and with RoPE
#endif
#ifndef SVLA_FUSED_PRE
#define SVLA_FUSED_PRE 2           // ... stages of K/V loads issued before the RoPE table is filled
#endif
#ifndef SVLA_FUSED_QLATE
#define SVLA_FUSED_QLATE 0         // ... Q rows issued after the build (1) or after the RoPE table (0)
#endif
#ifndef SVLA_FUSED_QG
#define SVLA_FUSED_QG 4            // ... Q groups of 16 tokens per wave at most (tile <= 16 * W * QG);
                                   // tiles of up to 16 * W * 2 tokens take an instance with 2
#endif
#ifndef SVLA_BWD_HOLD_Q
#define SVLA_BWD_HOLD_Q 1          // backward query side: state operands in registers (1) or LDS (0)
#endif
#ifndef SVLA_BWD_BF16
#define SVLA_BWD_BF16 1            // backward query side, bf16 inputs at d = 32: bf16 hi + lo products
#endif
#ifndef SVLA_BWD_WGS
#define SVLA_BWD_WGS 2048          // backward query/key kernels: workgroups wanted per launch
#endif
// Cache-policy bits of the streaming accesses (gfx950 buffer instructions:
// bit 1 = nt, non-temporal).  Measured: nt pays for K/V (read once by the
// state build), for Q (read once by the apply) and not for O.
#ifndef SVLA_KV_AUX
#define SVLA_KV_AUX 2
#endif
#ifndef SVLA_Q_AUX
#define SVLA_Q_AUX 2
#endif
#ifndef SVLA_O_AUX
#define SVLA_O_AUX 0
#endif

// ---------------------------------------------------------------------------
// types and small device helpers
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) short i16x2_t;

namespace {

constexpr int kThreads = 256;                 // build and apply: 4 waves of 64
constexpr int kFoldMaxParts = SVLA_FOLD_MAX_PARTS;           // partials a scan folded into the apply sums at most
constexpr int kFoldMaxPartsRope = SVLA_FOLD_MAX_PARTS_ROPE;  // ... with RoPE (block steps cut into more splits)
constexpr int kScanLongChain = 16;            // scan: blocks from which the chain is cut four ways
constexpr uint32_t kOOB = 0x80000000u;        // an offset past every resource
constexpr int kMaxRopeEntries = 4096;         // (cos, sin) pairs per workgroup

// gfx9 raw buffer: stride 0, range check on bytes, 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Streaming accesses with an explicit cache policy.
template <int AUX>
__device__ __forceinline__ u32x4_t load16p(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void store16p(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, AUX);
}

// Reinterpretation helpers.  They take their operand by value on purpose:
// this compiler folds a bit cast applied directly to a vector element
// subscript (v[e]) to element 0, so element reads always go through these.
__device__ __forceinline__ float as_f32(unsigned int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ unsigned int as_u32(float x) { return __builtin_bit_cast(unsigned int, x); }

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(as_u32(v), r, (int)off, 0, 0);
}

// phi on two packed bf16: a bf16 with its sign bit set is negative as an
// int16 as well, so max(x, 0) in int16 arithmetic is the ReLU (-0 -> +0).
__device__ __forceinline__ unsigned int relu_bf16x2(unsigned int x)
{
    i16x2_t v = __builtin_bit_cast(i16x2_t, x);
    v = __builtin_elementwise_max(v, (i16x2_t){0, 0});
    return __builtin_bit_cast(unsigned int, v);
}

__device__ __forceinline__ float bf16lo(unsigned int x) { return as_f32(x << 16); }
__device__ __forceinline__ float bf16hi(unsigned int x) { return as_f32(x & 0xFFFF0000u); }

// round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950)
__device__ __forceinline__ unsigned short f2bf(float x)
{
    return __builtin_bit_cast(unsigned short, (__bf16)x);
}

// two fp32 -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Input element types of the bf16 kernels: bf16 (IN = 2 bytes) or OCP FP8
// E4M3 (IN = 1).  A lane handles 8 consecutive features: 16 bytes of bf16 or
// 8 bytes of fp8, kept in the low half of a u32x4_t.
template <int IN, int AUX>
__device__ __forceinline__ u32x4_t load8f(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (IN == 2) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
    } else {
        typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
        return (u32x4_t){v[0], v[1], 0u, 0u};
    }
}

// The 8 features as fp32 values, phi applied when RELU.  fp8 decodes on the
// hardware converter (two values per instruction), exactly.
template <int IN, bool RELU>
__device__ __forceinline__ void feat8(const u32x4_t &v, float *f)
{
    if constexpr (IN == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned int w = RELU ? relu_bf16x2(v[e]) : v[e];
            f[2 * e] = bf16lo(w);
            f[2 * e + 1] = bf16hi(w);
        }
    } else {
        typedef __attribute__((ext_vector_type(2))) float f32x2_t;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], false);
            const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], true);
            f[4 * e] = lo[0];
            f[4 * e + 1] = lo[1];
            f[4 * e + 2] = hi[0];
            f[4 * e + 3] = hi[1];
        }
        if constexpr (RELU) {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = fmaxf(f[e], 0.f);
        }
    }
}

// The 8 features as packed bf16 (phi applied when RELU); exact, since every
// fp8 E4M3 value is a bf16 value.
template <int IN, bool RELU>
__device__ __forceinline__ u32x4_t bf16x8_of(const u32x4_t &v)
{
    u32x4_t o;
    if constexpr (IN == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = RELU ? relu_bf16x2(v[e]) : v[e];
    } else {
        float f[8];
        feat8<IN, RELU>(v, f);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16(f[2 * e], f[2 * e + 1]);
    }
    return o;
}

// Barrier for LDS hand-offs inside a workgroup.  __syncthreads() also
// fences global memory, which on this architecture waits for every load in
// flight (loads and stores share one counter), so it would drain the
// prefetched stages; this waits for this wave's LDS operations only.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Output feature of row 4 (rho / 4) + rho % 4 of m-tile m in the apply's
// O^T MFMA (the column of S that packed-operand row (m, rho) holds).
__host__ __device__ constexpr int op_col(int m, int rho)
{
    return 32 * (m / 2) + 8 * (rho / 4) + 4 * (m % 2) + rho % 4;
}

// Unsigned division by a divisor fixed per launch (multiply-high method of
// Granlund and Montgomery): q = (t + ((x - t) >> s1)) >> s2, t = mulhi(x, mul).
struct FastDiv {
    uint32_t div, mul, s1, s2;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv &f)
{
    uint32_t t = __umulhi(x, f.mul);
    return (t + ((x - t) >> f.s1)) >> f.s2;
}

// ---------------------------------------------------------------------------
// 3D RoPE: per-workgroup (cos, sin) table in LDS, and the rotation of one
// thread's 16-byte chunk of features.
// ---------------------------------------------------------------------------
struct RopeK {
    int on;
    int dt, dh, dw;          // dims per axis (even)
    int gh, gw;              // latent grid
    int t0;                  // absolute frame of the call's first token
    float base;
    FastDiv div_hw, div_w;   // p / (gh*gw), q / gw
    int tab_bytes;           // LDS reserved for the table in front of the stage buffers
    // per axis (t, h, w): the frequency of pair 0 in turns per position,
    // 1 / (2 pi), and the ratio base^(-2/width) between successive pairs
    // (host fp64), so pair m's frequency is freq0 * ratio^m
    double freq0[3], ratio[3];
};

// Table layout (float2 cos, sin), position fastest: [dt/2 pairs][nf frames],
// then [dh/2 pairs][gh rows], then [dw/2 pairs][gw columns], then one
// identity entry (cos 1, sin 0) for the unrotated dims.
__device__ __forceinline__ int rope_entries(const RopeK &r, int nf)
{
    return nf * (r.dt / 2) + r.gh * (r.dh / 2) + r.gw * (r.dw / 2);
}

// Angles pos * theta_m with theta_m = base^(-2m/width): pair m's frequency
// in turns per position is freq0 * ratio^m (fp64, by squaring: m < 64), each
// entry's angle is reduced to a fraction of a turn in fp64 (so large frame
// indices keep their accuracy) and only then goes through an fp32 sin/cos
// of pi times that small argument.
// A kernel-argument double held in scalar registers (read once per wave).
__device__ __forceinline__ double sreg_f64(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double rope_freq(double f, double q, int m)
{
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        if ((m >> b) & 1) f *= q;
        q *= q;
    }
    return f;
}

// (cos, sin) of pair m at position pos: the angle in turns reduced in fp64,
// then an fp32 sin/cos of pi times twice the fraction.
__device__ __forceinline__ float2 rope_cs(double freq0, double ratio, int pos, int m)
{
    double turns = (double)pos * rope_freq(freq0, ratio, m);
    turns -= floor(turns);
    float s, c;
    sincospif(2.0f * (float)turns, &s, &c);
    return make_float2(c, s);
}

__device__ void rope_fill(float2 *tab, const RopeK &r, int f0, int nf)
{
    const int pt = r.dt / 2, ph = r.dh / 2;
    const int nT = nf * pt, nH = r.gh * ph, total = rope_entries(r, nf);
    // per-axis values in scalar registers, chosen by value below: an index
    // into the kernel argument that differs across lanes would become a
    // vector memory load, whose wait (loads complete in order) would also wait
    // for every K/V/Q load the kernel issued before the table
    const double fT = sreg_f64(r.freq0[0]), fH = sreg_f64(r.freq0[1]), fW = sreg_f64(r.freq0[2]);
    const double qT = sreg_f64(r.ratio[0]), qH = sreg_f64(r.ratio[1]), qW = sreg_f64(r.ratio[2]);
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        int pos, m, a;
        if (e < nT) {
            m = e / nf; pos = f0 + (e - m * nf); a = 0;
        } else if (e < nT + nH) {
            const int x = e - nT; m = x / r.gh; pos = x - m * r.gh; a = 1;
        } else {
            const int x = e - nT - nH; m = x / r.gw; pos = x - m * r.gw; a = 2;
        }
        const double fa = a == 0 ? fT : a == 1 ? fH : fW, qa = a == 0 ? qT : a == 1 ? qH : qW;
        tab[e] = rope_cs(fa, qa, pos, m);
    }
    if (threadIdx.x == 0) tab[total] = make_float2(1.f, 0.f);   // identity, for unrotated dims
}

// Table of the one-launch step: the same angles with the pair index fastest,
// [nf frames][dt/2 pairs], then [gh rows][dh/2 pairs], then [gw columns][dw/2
// pairs], then two identity entries.  With dt, dh and dw multiples of 4, the
// two pairs of a 4-feature group belong to one axis and are one 16-byte read.
__device__ void gtab_fill(float2 *tab, const RopeK &r, int nf)
{
    const int pt = r.dt / 2, ph = r.dh / 2, pw = r.dw / 2;
    const int nT = nf * pt, nH = r.gh * ph, total = nT + nH + r.gw * pw;
    const double fT = sreg_f64(r.freq0[0]), fH = sreg_f64(r.freq0[1]), fW = sreg_f64(r.freq0[2]);
    const double qT = sreg_f64(r.ratio[0]), qH = sreg_f64(r.ratio[1]), qW = sreg_f64(r.ratio[2]);
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        int pos, m, a;
        if (e < nT) {
            pos = e / pt; m = e - pos * pt; pos += r.t0; a = 0;
        } else if (e < nT + nH) {
            const int x = e - nT; pos = x / ph; m = x - pos * ph; a = 1;
        } else {
            const int x = e - nT - nH; pos = x / pw; m = x - pos * pw; a = 2;
        }
        const double fa = a == 0 ? fT : a == 1 ? fH : fW, qa = a == 0 ? qT : a == 1 ? qH : qW;
        tab[e] = rope_cs(fa, qa, pos, m);
    }
    if (threadIdx.x < 2) tab[total + threadIdx.x] = make_float2(1.f, 0.f);
}

// LDS byte offset of a lane's two 4-feature groups (features 8 c + 4 G .. + 3
// of chunk c) for a token at (frame, row, column): base + frame st + row sh +
// column sw, at most one of st, sh, sw nonzero (none: the identity entries).
struct GroupAddr {
    int base[2], st[2], sh[2], sw[2];
};

__device__ __forceinline__ GroupAddr gtab_groups(const RopeK &r, int chunk, int nf)
{
    GroupAddr g;
    const int pt = r.dt / 2, ph = r.dh / 2, pw = r.dw / 2;
    const int offH = nf * pt, offW = offH + r.gh * ph, offI = offW + r.gw * pw;
#pragma unroll
    for (int G = 0; G < 2; ++G) {
        const int P = 4 * chunk + 2 * G;           // the group's first pair
        int e = offI, st = 0, sh = 0, sw = 0;
        if (P < pt) {
            e = P; st = pt;
        } else if (P < pt + ph) {
            e = offH + P - pt; sh = ph;
        } else if (P < pt + ph + pw) {
            e = offW + P - pt - ph; sw = pw;
        }
        g.base[G] = 8 * e; g.st[G] = 8 * st; g.sh[G] = 8 * sh; g.sw[G] = 8 * sw;
    }
    return g;
}

__device__ __forceinline__ int gtab_off(const GroupAddr &g, int G, int fr, int row, int col)
{
    return g.base[G] + fr * g.st[G] + row * g.sh[G] + col * g.sw[G];
}

// Rotate features x[0..3] (two pairs) by the group's (cos, sin, cos, sin).
__device__ __forceinline__ void rot_group(float *x, const f32x4_t cs)
{
    const float x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
    x[0] = x0 * cs[0] - x1 * cs[1];
    x[1] = x0 * cs[1] + x1 * cs[0];
    x[2] = x2 * cs[2] - x3 * cs[3];
    x[3] = x2 * cs[3] + x3 * cs[2];
}

// A lane's token walk through the grid: the token advances by a fixed count
// (dF frames, dR < gh rows, dC < gw columns) per step, the row and column
// carry, and the table offsets of the lane's two groups follow by adds: per
// step k0, plus k1 when the column wraps, plus k2 when the row wraps.
struct GroupWalk {
    int off[2], k0[2], k1[2], k2[2];
    int row, col, dR, dC, gh, gw;
};

__device__ __forceinline__ GroupWalk group_walk(const GroupAddr &g, const RopeK &r, uint32_t tok0, uint32_t step)
{
    GroupWalk w;
    const uint32_t hw = (uint32_t)(r.gh * r.gw);
    const uint32_t f0 = fdiv(tok0, r.div_hw), r0 = tok0 - f0 * hw, y0 = fdiv(r0, r.div_w);
    const uint32_t df = fdiv(step, r.div_hw), dr = step - df * hw, dy = fdiv(dr, r.div_w);
    w.row = (int)y0; w.col = (int)(r0 - y0 * (uint32_t)r.gw);
    w.dR = (int)dy; w.dC = (int)(dr - dy * (uint32_t)r.gw);
    w.gh = r.gh; w.gw = r.gw;
#pragma unroll
    for (int G = 0; G < 2; ++G) {
        w.off[G] = g.base[G] + (int)f0 * g.st[G] + w.row * g.sh[G] + w.col * g.sw[G];
        w.k0[G] = (int)df * g.st[G] + w.dR * g.sh[G] + w.dC * g.sw[G];
        w.k1[G] = g.sh[G] - r.gw * g.sw[G];
        w.k2[G] = g.st[G] - r.gh * g.sh[G];
    }
    return w;
}

__device__ __forceinline__ void walk_step(GroupWalk &w)
{
    int c = w.col + w.dC;
    const bool cc = c >= w.gw;
    c = cc ? c - w.gw : c;
    int r = w.row + w.dR + (cc ? 1 : 0);
    const bool cr = r >= w.gh;
    r = cr ? r - w.gh : r;
    w.row = r; w.col = c;
#pragma unroll
    for (int G = 0; G < 2; ++G) w.off[G] += w.k0[G] + (cc ? w.k1[G] : 0) + (cr ? w.k2[G] : 0);
}

// Per-thread description of the 4 (bf16 chunk) or 2 (fp32 chunk) pairs of
// its fixed feature chunk.  A pair's table index for a token at (frame
// offset fr, row, col) is base + (fr & mt) + (row & mh) + (col & mw): the
// mask of the pair's axis is all ones and the other two are zero (no
// multiply on the way); a pair outside the three slices has three zero
// masks and points at the identity entry, so the rotation has no branches.
template <int PAIRS>
struct RopePairs {
    int base[PAIRS], mt[PAIRS], mh[PAIRS], mw[PAIRS];
};

template <int PAIRS>
__device__ __forceinline__ RopePairs<PAIRS> rope_pairs(const RopeK &r, int first_feature, int nf)
{
    RopePairs<PAIRS> p;
    const int pt = r.dt / 2, ph = r.dh / 2;
    const int offH = nf * pt, offW = offH + r.gh * ph;
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
        const int f = first_feature + 2 * j;
        p.mt[j] = p.mh[j] = p.mw[j] = 0;
        if (f < r.dt) {
            p.base[j] = (f / 2) * nf; p.mt[j] = -1;
        } else if (f < r.dt + r.dh) {
            p.base[j] = offH + ((f - r.dt) / 2) * r.gh; p.mh[j] = -1;
        } else if (f < r.dt + r.dh + r.dw) {
            p.base[j] = offW + ((f - r.dt - r.dh) / 2) * r.gw; p.mw[j] = -1;
        } else {
            p.base[j] = rope_entries(r, nf);       // the identity entry
        }
    }
    return p;
}

// Position of call token p: frame offset from the table's first frame, grid
// row, grid column.
struct RopePos {
    int fr, row, col;
};

__device__ __forceinline__ RopePos rope_pos(uint32_t p, uint32_t frame_lo, const RopeK &r)
{
    const uint32_t fr = fdiv(p, r.div_hw);
    const uint32_t rem = p - fr * (uint32_t)(r.gh * r.gw);
    const uint32_t row = fdiv(rem, r.div_w);
    return RopePos{(int)(fr - frame_lo), (int)row, (int)(rem - row * (uint32_t)r.gw)};
}

// Rotate x[2j], x[2j+1] by the angles of the token at `pos`.
template <int PAIRS>
__device__ __forceinline__ void rope_rotate(float *x, const RopePos &pos,
                                            const RopePairs<PAIRS> &pp, const float2 *tab)
{
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
        const int idx = pp.base[j] + (pos.fr & pp.mt[j]) + (pos.row & pp.mh[j]) + (pos.col & pp.mw[j]);
        const float2 cs = tab[idx];
        const float x0 = x[2 * j], x1 = x[2 * j + 1];
        x[2 * j] = x0 * cs.x - x1 * cs.y;
        x[2 * j + 1] = x0 * cs.y + x1 * cs.x;
    }
}

// Workgroup w of a launch is dispatched to XCD w % 8 (round-robin over the
// eight XCDs, each with its own L2).  Logical id (w % 8) * ceil(G / 8) + w / 8
// gives each XCD one contiguous range of the G logical ids, so neighbouring
// logical workgroups (the token tiles of one block, which read the same
// block state) share an L2.  The grid is G rounded up to a multiple of 8;
// a logical id >= G has no work.
__device__ __forceinline__ long xcd_logical(long G)
{
    const long w = blockIdx.x;
    return SVLA_APPLY_XCD ? (w % 8) * ((G + 7) / 8) + w / 8 : w;
}

inline unsigned xcd_grid(long G) { return (unsigned)(SVLA_APPLY_XCD ? (G + 7) / 8 * 8 : G); }

// ---------------------------------------------------------------------------
// kernel arguments
// ---------------------------------------------------------------------------
struct ScanArgs {
    const float *S_part, *z_part;  // split partials (or local states, or prefix states)
    const float *g;                // [BH][nb] or null
    const float *S_in, *z_in;      // state entering block 0, or null
    void *S_op;                    // packed operand [BH*nb][d*d] (bf16 or fp32)
    float *z_pre;                  // [BH*nb][d]
    float *S_pre;                  // fp32 prefix states [BH*nb][d*d] (export mode)
    float *S_fin, *z_fin;          // final state or null
    int nb, splits;                // blocks, partial states per block
};

struct BuildArgs {
    const void *K, *V;
    float *S_part, *z_part;        // [BH*nb][slots][d*d], [BH*nb][slots][d]
    int N, n, nb;
    int splits, chunk;             // workgroups per block, tokens per workgroup
    int slots;                     // partials per block: splits (+ 1 for the carried state)
    long BH;
    RopeK rope;
    // one block whose scan is folded into the apply: split 0 also stores
    // g * S_in, g * z_in as partial number `splits` (g: [BH] or null)
    const float *S_in, *z_in, *g;
};

// Partial number `splits` of a one-block (b,h): the carried state, scaled
// by its gate, so the apply never reads S_in (which the final state may
// overwrite in place).
__device__ __forceinline__ void carry_in(const BuildArgs &a, long bh, int D)
{
    const float gb = a.g ? a.g[bh] : 1.f;
    float *dS = a.S_part + (bh * a.slots + a.splits) * D * D;
    float *dz = a.z_part + (bh * a.slots + a.splits) * D;
    for (int e = threadIdx.x * 4; e < D * D; e += kThreads * 4)
        *(f32x4_t *)(dS + e) = gb * *(const f32x4_t *)(a.S_in + bh * D * D + e);
    for (int e = threadIdx.x * 4; e < D; e += kThreads * 4)
        *(f32x4_t *)(dz + e) = gb * *(const f32x4_t *)(a.z_in + bh * D + e);
}

struct ApplyArgs {
    const void *Q;
    void *O;
    const void *S_op;              // packed operand [BH*nb][d*d]
    const float *z_pre;            // [BH*nb][d]
    int N, n, nb, tile, tiles;     // tile: tokens per workgroup; tiles per block
    long groups;                   // logical workgroups: B*H*nb*tiles
    float eps;
    RopeK rope;
    // one block with the scan folded in (svla_apply_bf16<.., true>): the
    // state is the sum of the build's partials (the last one the carried,
    // decayed state when there is one)
    const float *S_part, *z_part;  // [BH][splits][d*d], [BH][splits][d]
    int splits;
    float *S_fin, *z_fin;          // final state or null (written by tile 0)
};

// SCAN_FORWARD: partials -> packed operands, prefix z and the final state;
// SCAN_EXPORT: local states -> fp32 prefix states; SCAN_PACK: prefix states
// -> packed operands.
enum ScanMode { SCAN_FORWARD = 0, SCAN_EXPORT = 1, SCAN_PACK = 2 };

// ---------------------------------------------------------------------------
// svla_state_scan: per (bh, element tile), the inclusive, optionally decayed
// prefix over blocks, S_c = g_c S_{c-1} + (sum of block c's split partials).
//
// Packed operand layout read by svla_apply (per (bh, block), d*d entries):
// bf16: fragment (m, ks) = 64 lanes x 8 values; lane (rho + 16 kg), value i
//       holds S[32 ks + 8 kg + i][f(m, rho)]
// fp32: fragment (m, kq) = 64 lanes x 4 values; lane (rho + 16 kg), value i
//       holds S[16 kq + 4 kg + i][f(m, rho)]
// with f(m, rho) = op_col(m, rho) = 32 (m / 2) + 8 (rho / 4) + 4 (m % 2) + rho % 4:
// the output rows of the MFMA land so that the lanes of one token hold
// O features 32 h + 8 kg + [0, 8) in m-tiles 2h and 2h + 1, and each store
// instruction of the apply writes whole 64-byte row segments.
//
// Element tiles: lane -> column v0 + lane % CW and RL consecutive rows
// k0 + RL (lane / CW) of an 8-row x CW-column tile, so each lane's values
// are contiguous in the packed operand (one store per block) and every
// load instruction reads whole row segments.  The last tile of a (bh) is z.
// For long chains of blocks the NSEG waves of a workgroup take the same
// tile and 1/NSEG of the blocks each, which cuts the serial chain NSEG ways
// (the prefix over blocks is associative: (G1, P1) then (G2, P2) is
// (G1 G2, G2 P1 + P2)):
//   1. each wave sums its blocks from a zero state: its product of gates G
//      and its partial prefix P;
//   2. through LDS, each wave composes the (G, P) of the waves before it
//      onto the incoming state (S_in or 0), in wave order;
//   3. each wave walks its blocks again from that state and writes every
//      block's prefix; the last wave's state is the final state.
// With NSEG = 1 the one wave skips steps 1 and 2.
// The partials of a wave's blocks are read in chunks of LA, all loads of a
// chunk issued before any is used.  Everything is summed in a fixed order,
// so the result repeats bit for bit.
// ---------------------------------------------------------------------------
template <int D>
struct ScanShape {
    static constexpr int RL = D == 32 ? 2 : 4;          // rows per lane
    static constexpr int CW = 8 * RL;                   // columns per tile
    static constexpr int STILES = (D / 8) * (D / CW);   // S tiles per (bh)
};

// Walk partials [lo, hi) of one (bh) (block-major, split-minor) in chunks
// of LA: fetch(idx, values) loads one (idx clamped into [lo, hi), so every
// load is in bounds; a value past hi is never used), consume(values) adds it.
template <int LA, int W, typename Fetch, typename Consume>
__device__ __forceinline__ void scan_walk(int lo, int hi, Fetch fetch, Consume consume)
{
    static_assert(LA * W < 64, "the loads of a chunk must fit the vmcnt counter");
    for (int base = lo; base < hi; base += LA) {
        float buf[LA][W];
#pragma unroll
        for (int j = 0; j < LA; ++j) fetch(min(base + j, hi - 1), buf[j]);
        wait_vmcnt<0>();      // once per chunk: the stores of consume() then wait for nothing
#pragma unroll
        for (int j = 0; j < LA; ++j)
            if (base + j < hi) consume(buf[j]);
    }
}

// The segmented scan of W values per lane.  fetch(idx, values) loads
// partial idx of this (bh); emit(c, values) writes block c's prefix;
// `acc` holds the incoming state on entry and, in the last wave, the final
// state on exit.  red: LDS of NSEG * W * 64 + NSEG floats.
template <int W, int MODE, int NSEG, typename Fetch, typename Emit>
__device__ __forceinline__ void scan_blocks(const ScanArgs &a, long bh, float *acc, float *red,
                                            Fetch fetch, Emit emit)
{
    constexpr int LA = 63 / W;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per = (a.nb + NSEG - 1) / NSEG;
    const int c0 = min(wave * per, a.nb), c1 = min(c0 + per, a.nb);
    const int lo = c0 * a.splits, hi = c1 * a.splits;
    const int hi0 = min(hi, lo + LA);      // the first chunk, loaded once for both passes
    const float *g = a.g ? a.g + bh * a.nb : nullptr;

    float first[LA][W];
    if (lo < hi) {
#pragma unroll
        for (int j = 0; j < LA; ++j) fetch(min(lo + j, hi - 1), first[j]);
        wait_vmcnt<0>();
    }
    // walk this wave's partials: the first chunk from registers, the rest loaded
    auto walk = [&](auto consume) {
#pragma unroll
        for (int j = 0; j < LA; ++j)
            if (lo + j < hi0) consume(first[j]);
        scan_walk<LA, W>(hi0, hi, fetch, consume);
    };

    if constexpr (MODE != SCAN_PACK && NSEG > 1) {
        // 1. this wave's (G, P) from a zero state
        float P[W], G = 1.f;
#pragma unroll
        for (int r = 0; r < W; ++r) P[r] = 0.f;
        int c = c0, sp = 0;
        walk([&](const float *x) {
            if (sp == 0 && g) {
                const float gc = g[c];
                G *= gc;
#pragma unroll
                for (int r = 0; r < W; ++r) P[r] *= gc;
            }
#pragma unroll
            for (int r = 0; r < W; ++r) P[r] += x[r];
            if (++sp == a.splits) { sp = 0; ++c; }
        });
        if (a.splits == 0 && g) {   // no tokens: the blocks only decay
            for (int cc = c0; cc < c1; ++cc) G *= g[cc];
        }
#pragma unroll
        for (int r = 0; r < W; ++r) red[(wave * W + r) * 64 + lane] = P[r];
        if (lane == 0) red[NSEG * W * 64 + wave] = G;
        __syncthreads();
        // 2. compose the earlier waves onto the incoming state
        for (int w = 0; w < wave; ++w) {
            const float gw = red[NSEG * W * 64 + w];
#pragma unroll
            for (int r = 0; r < W; ++r) acc[r] = gw * acc[r] + red[(w * W + r) * 64 + lane];
        }
    }
    // 3. this wave's blocks from its incoming state
    int c = c0, sp = 0;
    if (a.splits == 0) {
        for (; c < c1; ++c) {
            if (g) {
#pragma unroll
                for (int r = 0; r < W; ++r) acc[r] *= g[c];
            }
            emit(c, acc);
        }
    } else {
        walk([&](const float *x) {
            if (sp == 0) {
                const float gc = MODE == SCAN_PACK ? 0.f : (g ? g[c] : 1.f);
#pragma unroll
                for (int r = 0; r < W; ++r) acc[r] *= gc;
            }
#pragma unroll
            for (int r = 0; r < W; ++r) acc[r] += x[r];
            if (++sp == a.splits) {
                emit(c, acc);
                sp = 0;
                ++c;
            }
        });
    }
}

template <int D, int MODE, bool OPBF16, int NSEG>
__device__ __forceinline__ void scan_s_tile(const ScanArgs &a, long bh, int tile, float *red)
{
    using SH = ScanShape<D>;
    constexpr int RL = SH::RL, CW = SH::CW;
    const int lane = threadIdx.x & 63;
    const int v = (tile % (D / CW)) * CW + lane % CW;
    const int k = (tile / (D / CW)) * 8 + RL * (lane / CW);
    // operand position of (k .. k + RL - 1, v)
    const int m = 2 * (v / 32) + (v % 8) / 4, rho = 4 * ((v % 32) / 8) + v % 4;   // op_col(m, rho) == v
    long opos;
    if constexpr (OPBF16)
        opos = ((long)((m * (D / 32) + k / 32) * 64 + rho + 16 * ((k % 32) / 8)) * 8 + k % 8);
    else
        opos = ((long)((m * (D / 16) + k / 16) * 64 + rho + 16 * ((k % 16) / 4)) * 4 + k % 4);

    float acc[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r)
        acc[r] = (MODE != SCAN_PACK && a.S_in) ? a.S_in[bh * D * D + (k + r) * D + v] : 0.f;
    const float *part = a.S_part + bh * (long)a.nb * a.splits * D * D + k * D + v;
    auto fetch = [&](int idx, float *dst) {
        const float *src = part + (long)idx * D * D;
#pragma unroll
        for (int r = 0; r < RL; ++r) dst[r] = src[r * D];
    };
    auto emit = [&](int c, const float *x) {
        const long unit = bh * a.nb + c;
        if constexpr (MODE == SCAN_EXPORT) {
#pragma unroll
            for (int r = 0; r < RL; ++r) a.S_pre[unit * D * D + (k + r) * D + v] = x[r];
        } else if constexpr (OPBF16) {
            unsigned short *op = (unsigned short *)a.S_op + unit * D * D + opos;
            if constexpr (RL == 2) *(unsigned int *)op = pack_bf16(x[0], x[1]);
            else *(uint2 *)op = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
        } else {
            float *op = (float *)a.S_op + unit * D * D + opos;
            if constexpr (RL == 2) *(float2 *)op = make_float2(x[0], x[1]);
            else *(float4 *)op = make_float4(x[0], x[1], x[2], x[3]);
        }
    };
    scan_blocks<RL, MODE, NSEG>(a, bh, acc, red, fetch, emit);
    if (MODE != SCAN_PACK && a.S_fin && (threadIdx.x >> 6) == NSEG - 1) {
#pragma unroll
        for (int r = 0; r < RL; ++r) a.S_fin[bh * D * D + (k + r) * D + v] = acc[r];
    }
}

// z of one (bh): lane -> z[lane], z[lane + 64]
template <int D, int MODE, int NSEG>
__device__ __forceinline__ void scan_z_tile(const ScanArgs &a, long bh, float *red)
{
    constexpr int ZL = (D + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int e0 = min(lane, D - 1);    // lanes past d read a valid element and write nothing
    float acc[ZL];
#pragma unroll
    for (int r = 0; r < ZL; ++r) acc[r] = (a.z_in && lane + 64 * r < D) ? a.z_in[bh * D + e0 + 64 * r] : 0.f;
    const float *part = a.z_part + bh * (long)a.nb * a.splits * D + e0;
    auto fetch = [&](int idx, float *dst) {
        const float *src = part + (long)idx * D;
#pragma unroll
        for (int r = 0; r < ZL; ++r) dst[r] = src[64 * r];
    };
    auto emit = [&](int c, const float *x) {
#pragma unroll
        for (int r = 0; r < ZL; ++r)
            if (lane + 64 * r < D) a.z_pre[(bh * a.nb + c) * D + lane + 64 * r] = x[r];
    };
    scan_blocks<ZL, MODE, NSEG>(a, bh, acc, red, fetch, emit);
    if (a.z_fin && (threadIdx.x >> 6) == NSEG - 1) {
#pragma unroll
        for (int r = 0; r < ZL; ++r)
            if (lane + 64 * r < D) a.z_fin[bh * D + lane + 64 * r] = acc[r];
    }
}

template <int D, int MODE, bool OPBF16, int NSEG>
__global__ void __launch_bounds__(64 * NSEG)
svla_state_scan_k(const ScanArgs a)
{
    constexpr int STILES = ScanShape<D>::STILES;
    __shared__ float red[NSEG > 1 ? NSEG * 4 * 64 + NSEG : 1];
    const long bh = blockIdx.x / (STILES + 1);
    const int tile = (int)(blockIdx.x % (STILES + 1));
    if (tile < STILES) scan_s_tile<D, MODE, OPBF16, NSEG>(a, bh, tile, red);
    else if (MODE != SCAN_PACK) scan_z_tile<D, MODE, NSEG>(a, bh, red);
}

// ---------------------------------------------------------------------------
// svla_state_build, bf16 inputs without RoPE, loads straight to LDS.
//
// Workgroup = (bh, block c, split s): it walks its token range in
// stages of TT tokens.  K and V travel from global memory into an R-deep
// ring of LDS stages with buffer_load ... lds (16 bytes per lane, one
// kilobyte per wave instruction), so R - 1 stages of loads stay in flight
// without holding registers.  The contraction S = phi(K)^T V runs on
// v_mfma_f32_32x32x16_bf16 over tokens: each lane needs 8 tokens of one
// feature from the staged rows (which token feeds which k-slot does not
// matter for a sum over tokens, as long as A and B agree): 16-bit gathers
// for d = 32, transposing reads (ds_read_b64_tr_b16) for d >= 64.  phi is applied
// to the K fragments, and z comes out of the same matrix cores as phi(K)
// times a ones operand.  Rows of the last stage past the range are
// overwritten with zeros by the lanes that loaded them.  Each stage buffer
// is its own LDS object, which lets the compiler tell the loads of
// different stages apart instead of waiting for all of them.
//   d = 32 : one 32x32 output tile; the 4 waves split the stage's tokens and
//            their tiles are summed through LDS at the end.
//   d = 64 : 2x2 tiles, one per wave; every wave sees every token.
//   d = 128: 4x4 tiles, 2x2 per wave; every wave sees every token.  (Four
//            workgroups per unit, one 64 x 64 quadrant each, read the K and
//            V half-rows twice through L2 and lost more to L2 misses than
//            the extra split partials of whole rows cost.)
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;

template <int D>
__device__ __forceinline__ int swz16(int t, int chunk)
{
    // rows of d >= 64 span every LDS bank: odd rows swap chunk halves so
    // the two half-waves (even/odd tokens) read disjoint banks.
    return (D >= 64) ? (chunk ^ ((t & 1) << 2)) : chunk;
}

// Token-contraction operand of v_mfma_f32_32x32x16_bf16 from a row-major
// [token][D] bf16 tile (16-byte chunks swizzled by swz16): lane l needs 8
// tokens of feature f0 + l % 32.  ds_read_b64_tr_b16 hands lane 4a + k of
// each 16-lane group element k of the 8-byte pieces addressed by lanes a,
// a + 4, a + 8, a + 12 of that group, so two such reads, with lane i of the
// group addressing token 4 r + i / 4 and features 4 (i % 4) .. + 3 of the
// group's 16-feature half, give lane l tokens 8 (l / 32) + 0 .. 7 of its
// feature: k-slot 8 (l / 32) + j is token 8 (l / 32) + j of the 16-token group.
// trb_offset: the lane's byte offset for read r = 0 (r = 1 adds 4 rows).
template <int D>
__device__ __forceinline__ int trb_offset(int lane, int f0)
{
    const int i = lane & 15, G = lane >> 4;
    const int row = 8 * (G >> 1) + (i >> 2);
    const int c = (f0 >> 3) + 2 * (G & 1) + ((i & 3) >> 1);
    return row * D * 2 + swz16<D>(row, c) * 16 + 8 * (i & 1);
}

// One operand by the builtin, for kernels with no loads to LDS in flight.
template <int D>
__device__ __forceinline__ bf16x8_t trb_load(const unsigned char *grp, int off)
{
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4_t *lp;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(grp + off));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(grp + off + 4 * D * 2));
    const u32x4_t x = {__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                       __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
    return __builtin_bit_cast(bf16x8_t, x);
}

// Both operands of one 16-token group: four transposing reads in one asm
// block that also waits for them (the compiler sees no LDS read here, so it
// adds no wait for the stage loads in flight, which write other buffers;
// the ring's own waits and barriers order these reads).
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int D>
__device__ __forceinline__ void trb_load2(const unsigned char *kgrp, int koff, const unsigned char *vgrp,
                                          int voff, bf16x8_t &av, bf16x8_t &bv)
{
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
    u32x2_t k0, k1, v0, v1;
    asm volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                 "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
                 "ds_read_b64_tr_b16 %2, %5\n\t"
                 "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(k0), "=&v"(k1), "=&v"(v0), "=&v"(v1)
                 : "v"(lds_addr(kgrp + koff)), "v"(lds_addr(vgrp + voff)), "i"(4 * D * 2));
    const u32x4_t a = {k0[0], k0[1], k1[0], k1[1]};
    const u32x4_t b = {v0[0], v0[1], v1[0], v1[1]};
    av = __builtin_bit_cast(bf16x8_t, a);
    bv = __builtin_bit_cast(bf16x8_t, b);
}

template <int D, int U, int R>
__global__ void __launch_bounds__(kThreads)
svla_state_build_dma(const BuildArgs a)
{
    constexpr int CPR = D / 8;            // 16-byte chunks per token row
    constexpr int RPW = 64 / CPR;         // rows one wave instruction covers
    constexpr int RPS = kThreads / CPR;   // rows one pass of the 4 waves covers
    constexpr int TT = U * RPS;           // tokens per stage
    constexpr int ROWB = D * 2;
    constexpr int TILEB = TT * ROWB;      // U * 4096
    constexpr int STAGEB = 2 * TILEB;     // K tile, then V tile
    constexpr bool SPLITK = (D == 32);
    constexpr int TPW = SPLITK ? 1 : D / 64;
    static_assert(TPW <= 2, "at most 2 x 2 tiles of 32 x 32 per wave");
    constexpr int GPS = TT / 16;
    constexpr int L = 2 * U;              // loads per thread per stage
    static_assert(R >= 3 && R <= 4, "ring depth");
    static_assert(!SPLITK || STAGEB >= 8192, "epilogue reuses two stage buffers");

    __shared__ __attribute__((aligned(16))) unsigned char b0[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b1[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b2[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b3[R > 3 ? STAGEB : 16];
    __shared__ float zred[4 * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long wid = blockIdx.x;
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = wid / per_bh;
    const int rest = (int)(wid - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    const uint32_t slice = (uint32_t)a.N * D * 2;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);

    auto buf = [&](int j) -> unsigned char * {
        return j == 0 ? b0 : j == 1 ? b1 : j == 2 ? b2 : b3;
    };
    // stage `st` into buffer `dst`: lane -> (row lane / CPR, LDS slot lane % CPR),
    // the slot holding global chunk slot ^ swizzle(row)
    auto issue = [&](unsigned char *dst, int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = (u * 4 + wave) * RPW + lane / CPR;
            const int t = tok_lo + st * TT + r;
            const int cg = swz16<D>(r, lane % CPR);
            const bool in = t < tok_hi;
            const uint32_t off = in ? (uint32_t)(t * D + cg * 8) * 2u : kOOB;
            unsigned char *kd = dst + (u * 4 + wave) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr_t)kd, 16, off, 0, 0, SVLA_KV_AUX);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr_t)(kd + TILEB), 16, off, 0, 0, SVLA_KV_AUX);
        }
    };

    f32x16_t zt[TPW];                     // phi(K) x ones: every column holds z
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) zt[i][r] = 0.f;
    u16x8_t ones16;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones16[i] = 0x3F80;   // bf16 1.0
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones16);
    f32x16_t acc[TPW][TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int m = lane & 31, g = lane >> 5;
    const int mt0 = SPLITK ? 0 : (wave >> 1) * TPW;
    const int nt0 = SPLITK ? 0 : (wave & 1) * TPW;
    const bool zwave = SPLITK || nt0 == 0;     // one wave per K fragment sums z
    constexpr int GPW = SPLITK ? GPS / 4 : GPS;  // 16-token groups per wave per stage
    // d = 32 (64-byte rows): lane (m, g) gathers k-slot i of a group from row
    // 16 gi + g + 2 i, 16-bit reads (the row's parity (= g) fixes the
    // swizzle; these were measured faster here than the transposing reads).
    // Half-rows of d = 128: the lane's byte offsets of its transposing reads.
    constexpr bool TR = D >= 64;
    int kl[TPW], vl[TPW];
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int f = 32 * (mt0 + tm) + m;
        kl[tm] = TR ? trb_offset<D>(lane, 32 * (mt0 + tm)) : g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
    }
#pragma unroll
    for (int tn = 0; tn < TPW; ++tn) {
        const int f = 32 * (nt0 + tn) + m;
        vl[tn] = TR ? trb_offset<D>(lane, 32 * (nt0 + tn)) : g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
    }

    const int ntiles = tok_hi > tok_lo ? (tok_hi - tok_lo + TT - 1) / TT : 0;
    const int nst = (ntiles + R - 1) / R * R;
#pragma unroll
    for (int j = 0; j < R - 1; ++j) issue(buf(j), j);

    for (int it0 = 0; it0 < nst; it0 += R) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int it = it0 + j;
            wait_vmcnt<(R - 2) * L>();     // this wave's loads of stage `it` have landed
            // Rows past the range (only in a workgroup's last stages): the lane
            // that loaded a slot overwrites it with zeros, so they add nothing
            // whatever an out-of-range load left there.
            if (tok_lo + (it + 1) * TT > tok_hi) {
                const int vrows = tok_hi - (tok_lo + it * TT);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int r = (u * 4 + wave) * RPW + lane / CPR;
                    if (r >= vrows) {
                        unsigned char *slot = buf(j) + (u * 4 + wave) * 1024 + lane * 16;
                        *(u32x4_t *)slot = (u32x4_t){0u, 0u, 0u, 0u};
                        *(u32x4_t *)(slot + TILEB) = (u32x4_t){0u, 0u, 0u, 0u};
                    }
                }
            }
            lds_barrier();                 // ... everyone's have; stage it-1 is consumed
            issue(buf((j + R - 1) % R), it + R - 1);
            const unsigned char *Ks = buf(j);
            const unsigned char *Vs = Ks + TILEB;
#pragma unroll
            for (int gg = 0; gg < GPW; ++gg) {
                const int gi = SPLITK ? wave + 4 * gg : gg;
                bf16x8_t av[TPW], bv[TPW];
                if constexpr (TR) {
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
                        trb_load2<D>(Ks + 16 * gi * ROWB, kl[t], Vs + 16 * gi * ROWB, vl[t], av[t], bv[t]);
                } else {
                    const unsigned short *pk = (const unsigned short *)Ks + 16 * gi * D + kl[0];
                    const unsigned short *pv = (const unsigned short *)Vs + 16 * gi * D + vl[0];
                    u16x8_t x, y;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x[i] = pk[2 * i * D];
                        y[i] = pv[2 * i * D];
                    }
                    av[0] = __builtin_bit_cast(bf16x8_t, x);
                    bv[0] = __builtin_bit_cast(bf16x8_t, y);
                }
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
                    u32x4_t w = __builtin_bit_cast(u32x4_t, av[tm]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = relu_bf16x2(w[e]);
                    av[tm] = __builtin_bit_cast(bf16x8_t, w);
                    // z on the matrix cores: phi(K) times a ones operand
                    if (zwave) zt[tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], ones, zt[tm], 0, 0, 0);
                }
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TPW; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();      // the trailing out-of-range loads target the ring too
    __syncthreads();

    // ---- epilogue: S_part (row-major [k][v]) and z_part
    const long unit = (bh * a.nb + c) * a.slots + s;
    const auto rS = make_rsrc(a.S_part + unit * D * D, D * D * 4);
    const auto rz = make_rsrc(a.z_part + unit * D, D * 4);
    // z: column 0 of each zt tile, held by lanes 0 (rows 8q + r, r < 4) and 32 (rows 8q + 4 + r)
    if constexpr (SPLITK) {
        float *red = (float *)(wave < 2 ? b0 : b1);   // 2 waves x 16 x 64 floats each
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wave & 1) * 16 + r) * 64 + lane] = acc[0][0][r];
        if ((lane & 31) == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) zred[wave * 32 + 8 * (r >> 2) + 4 * g + (r & 3)] = zt[0][r];
        }
    } else {
        if (zwave && (lane & 31) == 0) {
#pragma unroll
            for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r) zred[32 * (mt0 + tm) + 8 * (r >> 2) + 4 * g + (r & 3)] = zt[tm][r];
        }
    }
    __syncthreads();
    if constexpr (SPLITK) {
        const int e0 = tid * 4, rr = e0 / 32, c0 = e0 % 32;
        const float *r01 = (const float *)b0, *r23 = (const float *)b1;
        u32x4_t out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ln = (c0 + j) + 32 * ((rr >> 2) & 1);
            const int r = 4 * (rr >> 3) + (rr & 3);
            float v = r01[(0 * 16 + r) * 64 + ln];
            v += r01[(1 * 16 + r) * 64 + ln];
            v += r23[(0 * 16 + r) * 64 + ln];
            v += r23[(1 * 16 + r) * 64 + ln];
            out[j] = as_u32(v);
        }
        store16(rS, (uint32_t)(rr * D + c0) * 4u, out);
        if (tid < D) {
            float v = zred[tid];
            v += zred[32 + tid];
            v += zred[64 + tid];
            v += zred[96 + tid];
            store4(rz, (uint32_t)tid * 4u, v);
        }
    } else {
#pragma unroll
        for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
            for (int tn = 0; tn < TPW; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 32 * (mt0 + tm) + 8 * (r >> 2) + 4 * g + (r & 3);
                    const int cc = 32 * (nt0 + tn) + m;
                    store4(rS, (uint32_t)(rr * D + cc) * 4u, acc[tm][tn][r]);
                }
        if (tid < D) store4(rz, (uint32_t)tid * 4u, zred[tid]);
    }
    if (a.S_in && s == 0) carry_in(a, bh, D);
}

// ---------------------------------------------------------------------------
// svla_state_build, bf16 inputs with RoPE: wave-private streams.
//
// Workgroup = (bh, block c, split s[, quadrant]).  Its token range is cut
// into wave stages of TW tokens and wave w takes stages w, w + 4, w + 8, ...
// Each wave keeps PF stages of K/V loads in flight in registers, applies phi,
// the rotation and the bf16 hi/lo split to its K chunks (one token, 8
// features per lane), writes the stage into an LDS slot of its own and
// contracts it from there on v_mfma_f32_32x32x16_bf16, which sums over
// tokens: each lane takes 8 tokens of one feature from the slot rows with
// two transposing reads (ds_read_b64_tr_b16, see trb_offset); the hi and lo
// parts make two MFMAs, so the state keeps about 16 bits of the rotated
// key.  z sums the unrotated phi(k) on the vector ALU.
// No wave reads another wave's slot, and the LDS operations of one wave
// execute in program order, so the main loop needs no barrier and the slot
// can be overwritten by the next stage right after it was read.  Every wave
// accumulates the whole tile; the four tiles are summed through LDS at the
// end, in wave order.  Rows past the range load zeros (buffer range
// check), which add nothing.
//   D = DG     : the whole d x d state (d = 32, 64).
//   DG = 128   : D = 64 quadrant split; four workgroups per unit, each
//                one 64 x 64 quadrant of S from K and V half-rows.
// ---------------------------------------------------------------------------
template <int D, int DG, int PF, int U, bool ROPE = true, int IN = 2>
__global__ void __launch_bounds__(kThreads)
svla_state_build_rope(const BuildArgs a)
{
    constexpr int CPR = D / 8;            // 8-feature chunks per (half-)row
    constexpr int RPW = 64 / CPR;         // rows one wave load instruction covers
    constexpr int TW = U * RPW;           // tokens per wave stage
    constexpr int GPW = TW / 16;          // 16-token groups per wave stage
    constexpr int ROWB = D * 2;           // bytes of a staged (bf16) row
    constexpr int TILEB = TW * ROWB;
    constexpr int NK = ROPE ? 2 : 1;      // K tiles: (rotated) hi, and lo with RoPE
    static_assert(IN == 2 || (D == 32 && DG == 32), "fp8 inputs at d = 32 only");
    constexpr int SLOTB = (NK + 1) * TILEB;
    constexpr int TPW = D / 32;           // 32 x 32 tiles per side
    constexpr bool QUAD = DG != D;
    static_assert(TW % 16 == 0, "a wave stage holds whole 16-token groups");
    static_assert(!QUAD || (DG == 128 && D == 64), "the quadrant split is for d = 128");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    long wid = blockIdx.x;
    int qm = 0, qn = 0;
    if constexpr (QUAD) {
        // Quadrants of one unit get workgroup ids 8 apart, so the round-robin
        // dispatch puts all four on one XCD and its L2 serves the K/V
        // half-rows they share.
        const long x = wid % 8, r = wid / 8;
        const int q = (int)(r % 4);
        qm = q >> 1;
        qn = q & 1;
        wid = (r / 4) * 8 + x;
        if (wid >= (long)a.nb * a.splits * a.BH) return;
    }
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = wid / per_bh;
    const int rest = (int)(wid - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    const uint32_t slice = (uint32_t)a.N * DG * IN;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);
    const int kcol = 64 * qm, vcol = 64 * qn;   // first feature of this tile in K / V

    // lane -> (row lane / CPR + u RPW of the wave stage, chunk q of the row)
    const int row = lane / CPR, q = lane % CPR;

    // this wave's stages: st = wave + 4 i, i < nw
    const int nst = tok_hi > tok_lo ? (tok_hi - tok_lo + TW - 1) / TW : 0;
    const int nw = nst > wave ? (nst - wave + 3) / 4 : 0;
    auto offset = [&](int i, int u, int col) -> uint32_t {
        const int t = tok_lo + (wave + 4 * i) * TW + u * RPW + row;
        return t < tok_hi ? (uint32_t)(t * DG + col + q * 8) * (uint32_t)IN : kOOB;
    };
    // Register slot p holds stage i with i % PF == p.  The scheduling
    // barriers keep the slots' loads in slot order, the order the loop
    // consumes them in, so a wait for the oldest slot leaves the younger
    // slots' loads in flight.
    u32x4_t kreg[PF][U], vreg[PF][U];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kreg[p][u] = load8f<IN, SVLA_KV_AUX>(rK, offset(p, u, kcol));
            vreg[p][u] = load8f<IN, SVLA_KV_AUX>(rV, offset(p, u, vcol));
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // the RoPE table is built while the first stages load
    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<4> pp;
    unsigned char *const work = lds + (ROPE ? a.rope.tab_bytes : 0);   // slots, then the epilogue
    if constexpr (ROPE) {
        frame_lo = tok_lo < tok_hi ? fdiv((uint32_t)tok_lo, a.rope.div_hw) : 0;
        const uint32_t frame_hi = tok_lo < tok_hi ? fdiv((uint32_t)(tok_hi - 1), a.rope.div_hw) : 0;
        const int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
        pp = rope_pairs<4>(a.rope, kcol + q * 8, nf);
        lds_barrier();
    }
    unsigned char *slot = work + wave * SLOTB;

    f32x16_t acc[TPW][TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    float zacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[e] = 0.f;

    const int m = lane & 31, g = lane >> 5;
    // the lane's byte offsets of its transposing reads within a 16-token group
    int fl[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) fl[t] = trb_offset<D>(lane, 32 * t);

    // The loop is kept regular so the compiler can count the loads in flight:
    // the stage count is rounded up to a multiple of PF (the extra stages
    // load nothing and add zeros) and every register slot is refilled.
    const int nwr = (nw + PF - 1) / PF * PF;
    for (int i0 = 0; i0 < nwr; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int i = i0 + p;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = u * RPW + row;              // row within the stage
                const int cpos = swz16<D>(r, q);
                float kf[8];
                feat8<IN, true>(kreg[p][u], kf);
#pragma unroll
                for (int e = 0; e < 8; ++e) zacc[e] += kf[e];
                if constexpr (ROPE) {
                    const int tok = tok_lo + (wave + 4 * i) * TW + r;
                    rope_rotate<4>(kf, rope_pos((uint32_t)tok, frame_lo, a.rope), pp, tab);
                    u32x4_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hi[e] = pack_bf16(kf[2 * e], kf[2 * e + 1]);
                        lo[e] = pack_bf16(kf[2 * e] - bf16lo(hi[e]), kf[2 * e + 1] - bf16hi(hi[e]));
                    }
                    *(u32x4_t *)(slot + r * ROWB + cpos * 16) = hi;
                    *(u32x4_t *)(slot + TILEB + r * ROWB + cpos * 16) = lo;
                } else {
                    *(u32x4_t *)(slot + r * ROWB + cpos * 16) = bf16x8_of<IN, true>(kreg[p][u]);
                }
                *(u32x4_t *)(slot + NK * TILEB + r * ROWB + cpos * 16) = bf16x8_of<IN, false>(vreg[p][u]);
            }
            // refill this register slot with the stage PF ahead
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                kreg[p][u] = load8f<IN, SVLA_KV_AUX>(rK, offset(i + PF, u, kcol));
                vreg[p][u] = load8f<IN, SVLA_KV_AUX>(rV, offset(i + PF, u, vcol));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
                bf16x8_t av[TPW], al[TPW], bv[TPW];
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    av[t] = trb_load<D>(slot + 16 * gi * ROWB, fl[t]);
                    if constexpr (ROPE) al[t] = trb_load<D>(slot + TILEB + 16 * gi * ROWB, fl[t]);
                    bv[t] = trb_load<D>(slot + NK * TILEB + 16 * gi * ROWB, fl[t]);
                }
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TPW; ++tn) {
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
                        if constexpr (ROPE)
                            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[tm], bv[tn], acc[tm][tn], 0, 0, 0);
                    }
            }
        }
    }

    if constexpr (D == 32 && !QUAD) {
        // ---- epilogue (d = 32): each wave's tile in an LDS region of its
        // own, then every thread sums four values in wave order (the same
        // order as the pass-by-pass sum below); z is summed within each wave
        // over the 16 lanes that share a chunk, then over the waves
        float *red = (float *)work;                                // 4 x D x D floats
        float *zw = red + 4 * D * D;                               // 4 x D floats
        __syncthreads();          // every wave is done with its slot
#pragma unroll
        for (int r = 0; r < 16; ++r)
            red[wave * D * D + (8 * (r >> 2) + 4 * g + (r & 3)) * D + m] = acc[0][0][r];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = zacc[e];
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            zacc[e] = v;
        }
        if (lane < CPR) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zw[wave * D + lane * 8 + e] = zacc[e];
        }
        __syncthreads();
        static_assert(D * D == 4 * kThreads, "four values per thread");
        const long unit = (bh * a.nb + c) * a.slots + s;
        const auto rS = make_rsrc(a.S_part + unit * DG * DG, DG * DG * 4);
        const auto rz = make_rsrc(a.z_part + unit * DG, DG * 4);
        const int e0 = tid * 4;
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = red[e0 + i];
#pragma unroll
        for (int w = 1; w < 4; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] += red[w * D * D + e0 + i];
        u32x4_t out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = as_u32(t[i]);
        store16(rS, (uint32_t)e0 * 4u, out);
        if (tid < D) store4(rz, (uint32_t)tid * 4u, ((zw[tid] + zw[D + tid]) + zw[2 * D + tid]) + zw[3 * D + tid]);
        if (a.S_in && s == 0) carry_in(a, bh, D);
        return;
    }

    // ---- epilogue: the four waves' tiles summed in wave order, then
    // S_part (row-major [k][v], row stride DG) and z_part
    float *red = (float *)work;                                    // D x D floats
    float *zred = red + D * D;                                     // 256 x 8 floats
    __syncthreads();          // every wave is done with its slot
#pragma unroll 1
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
                for (int tn = 0; tn < TPW; ++tn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rr = 32 * tm + 8 * (r >> 2) + 4 * g + (r & 3);
                        const int cc = 32 * tn + m;
                        float *p = red + rr * D + cc;
                        *p = w == 0 ? acc[tm][tn][r] : *p + acc[tm][tn][r];
                    }
        }
        __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[D + tid * 8 + e] = zacc[e];
    __syncthreads();
    if (tid < D) {
        // feature tid = 8 qq + e: summed over the threads that hold chunk qq
        const int qq = tid >> 3, e = tid & 7;
        float v = 0.f;
        for (int j = 0; j < kThreads / CPR; ++j) v += zred[D + (qq + CPR * j) * 8 + e];
        zred[tid] = v;
    }
    __syncthreads();
    const long unit = (bh * a.nb + c) * a.slots + s;
    const auto rS = make_rsrc(a.S_part + unit * DG * DG, DG * DG * 4);
    const auto rz = make_rsrc(a.z_part + unit * DG, DG * 4);
#pragma unroll
    for (int e0 = tid * 4; e0 < D * D; e0 += kThreads * 4) {
        const int rr = e0 / D, c0 = e0 % D;
        store16(rS, (uint32_t)((kcol + rr) * DG + vcol + c0) * 4u, *(const u32x4_t *)(red + e0));
    }
    if (tid < D && qn == 0) store4(rz, (uint32_t)(kcol + tid) * 4u, zred[tid]);
    if constexpr (!QUAD) {
        if (a.S_in && s == 0) carry_in(a, bh, D);
    }
}

// ---------------------------------------------------------------------------
// svla_state_build, fp32 inputs: the same walk with fp32 rows staged and
// v_mfma_f32_32x32x2_f32 (one token per half-wave per instruction).
// ---------------------------------------------------------------------------
template <int D, bool ROPE>
__global__ void __launch_bounds__(kThreads)
svla_state_build_f32(const BuildArgs a)
{
    constexpr int CPR = D / 4;            // 16-byte chunks (4 floats) per row
    constexpr int TT = kThreads / CPR;    // 32, 16, 8 tokens per stage
    constexpr int ROWB = D * 4;
    constexpr int TILEB = TT * ROWB;      // 4096
    constexpr int STAGEB = 2 * TILEB;
    constexpr bool SPLITK = (D == 32);
    constexpr int TPW = SPLITK ? 1 : D / 64;
    constexpr int PPS = TT / 2;           // token pairs per stage

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = blockIdx.x / per_bh;
    const int rest = (int)(blockIdx.x - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    const uint32_t slice = (uint32_t)a.N * D * 4;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);

    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<2> pp;
    const int row = tid / CPR, q = tid % CPR;
    if constexpr (ROPE) {
        frame_lo = tok_lo < tok_hi ? fdiv((uint32_t)tok_lo, a.rope.div_hw) : 0;
        uint32_t frame_hi = tok_lo < tok_hi ? fdiv((uint32_t)(tok_hi - 1), a.rope.div_hw) : 0;
        int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
        pp = rope_pairs<2>(a.rope, q * 4, nf);
        __syncthreads();
    }
    unsigned char *stage = lds + (ROPE ? a.rope.tab_bytes : 0);

    float zacc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x16_t acc[TPW][TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ntiles = tok_hi > tok_lo ? (tok_hi - tok_lo + TT - 1) / TT : 0;
    int tok = tok_lo + row;
    uint32_t off = tok < tok_hi ? (uint32_t)(tok * D + q * 4) * 4u : kOOB;
    u32x4_t kreg = load16(rK, off);
    u32x4_t vreg = load16(rV, off);
    const int m = lane & 31, g = lane >> 5;
    const int mt0 = SPLITK ? 0 : (wave >> 1) * TPW;
    const int nt0 = SPLITK ? 0 : (wave & 1) * TPW;

    for (int it = 0; it < ntiles; ++it) {
        unsigned char *st = stage + (it & 1) * STAGEB;
        float kf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kf[e] = fmaxf(as_f32(kreg[e]), 0.f);
            zacc[e] += kf[e];
        }
        if constexpr (ROPE) rope_rotate<2>(kf, rope_pos((uint32_t)tok, frame_lo, a.rope), pp, tab);
        u32x4_t kw;
#pragma unroll
        for (int e = 0; e < 4; ++e) kw[e] = as_u32(kf[e]);
        *(u32x4_t *)(st + row * ROWB + q * 16) = kw;
        *(u32x4_t *)(st + TILEB + row * ROWB + q * 16) = vreg;
        __syncthreads();
        if (it + 1 < ntiles) {
            tok += TT;
            off = tok < tok_hi ? (uint32_t)(tok * D + q * 4) * 4u : kOOB;
            kreg = load16(rK, off);
            vreg = load16(rV, off);
        }
        const float *Ks = (const float *)st;
        const float *Vs = (const float *)(st + TILEB);
        constexpr int PPW = SPLITK ? PPS / 4 : PPS;     // pairs per wave
        const int p0 = SPLITK ? wave * PPW : 0;
#pragma unroll
        for (int pi = 0; pi < PPW; ++pi) {
            const int t = 2 * (p0 + pi) + g;
            float av[TPW], bv[TPW];
#pragma unroll
            for (int tm = 0; tm < TPW; ++tm) av[tm] = Ks[t * D + 32 * (mt0 + tm) + m];
#pragma unroll
            for (int tn = 0; tn < TPW; ++tn) bv[tn] = Vs[t * D + 32 * (nt0 + tn) + m];
#pragma unroll
            for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
                for (int tn = 0; tn < TPW; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
        }
    }
    __syncthreads();

    const long unit = (bh * a.nb + c) * a.slots + s;
    const auto rS = make_rsrc(a.S_part + unit * D * D, D * D * 4);
    const auto rz = make_rsrc(a.z_part + unit * D, D * 4);
    float *red = (float *)stage;
    float *zred = (float *)(stage + (SPLITK ? 4 * 16 * 64 * 4 : 0));
    if constexpr (SPLITK) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[0][0][r];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) zred[tid * 4 + e] = zacc[e];
    __syncthreads();
    if constexpr (SPLITK) {
        const int e0 = tid * 4, rr = e0 / 32, c0 = e0 % 32;
        u32x4_t out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ln = (c0 + j) + 32 * ((rr >> 2) & 1);
            const int r = 4 * (rr >> 3) + (rr & 3);
            float v = red[(0 * 16 + r) * 64 + ln];
            v += red[(1 * 16 + r) * 64 + ln];
            v += red[(2 * 16 + r) * 64 + ln];
            v += red[(3 * 16 + r) * 64 + ln];
            out[j] = as_u32(v);
        }
        store16(rS, (uint32_t)(rr * D + c0) * 4u, out);
    } else {
#pragma unroll
        for (int tm = 0; tm < TPW; ++tm)
#pragma unroll
            for (int tn = 0; tn < TPW; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 32 * (mt0 + tm) + 8 * (r >> 2) + 4 * g + (r & 3);
                    const int cc = 32 * (nt0 + tn) + m;
                    store4(rS, (uint32_t)(rr * D + cc) * 4u, acc[tm][tn][r]);
                }
    }
    if (tid < D) {
        const int qq = tid >> 2, e = tid & 3;
        float v = 0.f;
        for (int j = 0; j < kThreads / CPR; ++j) v += zred[(qq + CPR * j) * 4 + e];
        store4(rz, (uint32_t)tid * 4u, v);
    }
}

// ---------------------------------------------------------------------------
// svla_apply, bf16 inputs, d = 32.  Workgroup = (bh, block c, token tile);
// the tiles of one block run on one XCD.
// O^T = S^T phi~(Q)^T on v_mfma_f32_16x16x32_bf16: the state is the A
// operand (kept in registers for the whole tile), phi~(q) the B operand
// straight from a 16-byte load per lane (token = lane % 16, 8 features of
// chunk lane / 16).  The denominator phi(q) . z is a per-lane partial dot
// product reduced over the 4 lanes that share a token.  Each wave takes
// every 4th 16-token group, with all output features, and keeps PF groups
// of Q loads in flight.
// FOLD (one block, no scan kernel): the state is the sum of the build's
// partials, formed in LDS by every workgroup of the (b,h) while its first
// Q loads are in flight; tile 0 also writes it out as the final state.
// Otherwise the state comes from the scan's packed operand and prefix z.
// ---------------------------------------------------------------------------
template <int D, bool ROPE, bool FOLD, int IN = 2>
__global__ void __launch_bounds__(kThreads)
svla_apply_bf16(const ApplyArgs a)
{
    static_assert(IN == 2 || D == 32, "fp8 inputs at d = 32 only");
    constexpr int MT = D / 16;
    constexpr int KS = D / 32;
    constexpr int PF = ROPE ? SVLA_APPLY32_PF_ROPE : SVLA_APPLY32_PF;
    constexpr int MAXP = ROPE ? kFoldMaxPartsRope : kFoldMaxParts;
    static_assert(D == 32, "laid out for d = 32");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const long lid = xcd_logical(a.groups);
    if (lid >= a.groups) return;
    const int tile = (int)(lid % a.tiles);
    const int c = (int)((lid / a.tiles) % a.nb);
    const long bh = lid / ((long)a.tiles * a.nb);
    const int t_lo = c * a.n + tile * a.tile;
    const int t_hi = min(t_lo + a.tile, (c + 1) * a.n);
    const long unit = bh * a.nb + c;

    const uint32_t slice = (uint32_t)a.N * D * 2;              // O: bf16
    const uint32_t qslice = (uint32_t)a.N * D * IN;
    const auto rQ = make_rsrc((const char *)a.Q + bh * qslice, qslice);
    const auto rO = make_rsrc((char *)a.O + bh * slice, slice);
    const int kg = lane >> 4, tl = lane & 15;

    // 1. the state's loads: this thread's four floats of S (and of z for
    // threads < d / 4) from every partial, or the packed operand and z
    f32x4_t part[FOLD ? MAXP : 1][2];
    u32x4_t sop[MT][KS], zr[KS][2];
    const int e0 = tid * 4;
    if constexpr (FOLD) {
        const float *pS = a.S_part + bh * a.splits * D * D + e0;
        const float *pz = a.z_part + bh * a.splits * D + min(e0, D - 4);
#pragma unroll
        for (int sp = 0; sp < MAXP; ++sp) {
            if (sp < a.splits) {                     // (uniform)
                part[sp][0] = *(const f32x4_t *)(pS + sp * D * D);
                part[sp][1] = *(const f32x4_t *)(pz + sp * D);
            } else {
                part[sp][0] = part[sp][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
        }
    } else {
        const auto rS = make_rsrc((const char *)a.S_op + unit * D * D * 2, D * D * 2);
        const auto rz = make_rsrc(a.z_pre + unit * D, D * 4);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sop[mi][ks] = load16(rS, (uint32_t)(((mi * KS + ks) * 64 + lane) * 16));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            zr[ks][0] = load16(rz, (uint32_t)(8 * (4 * ks + kg)) * 4u);
            zr[ks][1] = load16(rz, (uint32_t)(8 * (4 * ks + kg) + 4) * 4u);
        }
    }

    // 2. the first PF groups of Q, issued before the state is formed so they
    // land meanwhile (slot p holds this wave's group i, i % PF == p; the
    // scheduling barriers keep the loads in slot order)
    const int ngroups = t_hi > t_lo ? (t_hi - t_lo + 15) / 16 : 0;
    const int nw = ngroups > wave ? (ngroups - wave + 3) / 4 : 0;
    auto qoff = [&](int i, int ks) -> uint32_t {
        const int tok = t_lo + 16 * (wave + 4 * i) + tl;
        return tok < t_hi ? (uint32_t)(tok * D + 8 * (4 * ks + kg)) * (uint32_t)IN : kOOB;
    };
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t qreg[PF][KS];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[p][ks] = load8f<IN, SVLA_Q_AUX>(rQ, qoff(p, ks));
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. the state in registers: A fragments sf (lane (rho + 16 kg), value i
    // = S[32 ks + 8 kg + i][op_col(mi, rho)])
    // and z for this lane's features
    bf16x8_t sf[MT][KS];
    float zf[KS][8];
    unsigned char *lds_free = lds;
    if constexpr (ROPE) lds_free += a.rope.tab_bytes;
    if constexpr (FOLD) {
        // summed in partial order, so every workgroup of the (b,h) gets the same bits
        float *st = (float *)lds_free;      // S[k][v] at [0, d*d), z at [d*d, d*d + d)
        f32x4_t vs = part[0][0], vz = part[0][1];
#pragma unroll
        for (int sp = 1; sp < MAXP; ++sp) {
            if (sp < a.splits) {
                vs += part[sp][0];
                vz += part[sp][1];
            }
        }
        *(f32x4_t *)(st + e0) = vs;
        if (e0 < D) *(f32x4_t *)(st + D * D + e0) = vz;
        if (tile == 0 && a.S_fin) {
            *(f32x4_t *)(a.S_fin + bh * D * D + e0) = vs;
            if (e0 < D) *(f32x4_t *)(a.z_fin + bh * D + e0) = vz;
        }
        lds_barrier();
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int f = op_col(mi, tl);
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16(st[(32 * ks + 8 * kg + 2 * e) * D + f],
                                     st[(32 * ks + 8 * kg + 2 * e + 1) * D + f]);
                sf[mi][ks] = __builtin_bit_cast(bf16x8_t, w);
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) zf[ks][e] = st[D * D + 8 * (4 * ks + kg) + e];
    } else {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sf[mi][ks] = __builtin_bit_cast(bf16x8_t, sop[mi][ks]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                zf[ks][e] = as_f32(zr[ks][0][e]);
                zf[ks][4 + e] = as_f32(zr[ks][1][e]);
            }
    }

    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<4> pp[KS];
    if constexpr (ROPE) {
        frame_lo = t_lo < t_hi ? fdiv((uint32_t)t_lo, a.rope.div_hw) : 0;
        const uint32_t frame_hi = t_lo < t_hi ? fdiv((uint32_t)(t_hi - 1), a.rope.div_hw) : 0;
        const int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pp[ks] = rope_pairs<4>(a.rope, 8 * (4 * ks + kg), nf);
        lds_barrier();
    }

    // 4. the groups: wave group i covers tokens t_lo + 16 (wave + 4 i) ...
    auto group = [&](int i, const u32x4_t *qr) {
        const int tok = t_lo + 16 * (wave + 4 * i) + tl;
        const bool valid = tok < t_hi;
        float den = 0.f;
        bf16x8_t qf[KS];
        RopePos rp{0, 0, 0};
        if constexpr (ROPE) rp = rope_pos((uint32_t)tok, frame_lo, a.rope);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t pq = {0u, 0u, 0u, 0u};
            if constexpr (IN == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = relu_bf16x2(qr[ks][e]);
            }
            float pf[8];
            feat8<IN, true>(qr[ks], pf);
#pragma unroll
            for (int e = 0; e < 8; ++e) den = fmaf(pf[e], zf[ks][e], den);
            if constexpr (ROPE) rope_rotate<4>(pf, rp, pp[ks], tab);
            if constexpr (ROPE || IN != 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = pack_bf16(pf[2 * e], pf[2 * e + 1]);
            }
            qf[ks] = __builtin_bit_cast(bf16x8_t, pq);
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        den += a.eps;
        const float inv = den != 0.f ? 1.0f / den : 0.f;

        f32x4_t acc[MT];
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            acc[mi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[mi][ks], qf[ks], acc[mi], 0, 0, 0);
        }
        // m-tiles 2h, 2h + 1 hold O[tok][op_col(2h, 4 kg) + 0 .. 7]
#pragma unroll
        for (int h = 0; h < MT / 2; ++h) {
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                o[2 * e] = pack_bf16(acc[2 * h + e][0] * inv, acc[2 * h + e][1] * inv);
                o[2 * e + 1] = pack_bf16(acc[2 * h + e][2] * inv, acc[2 * h + e][3] * inv);
            }
            const int v0 = op_col(2 * h, 4 * kg);
            store16p<SVLA_O_AUX>(rO, valid ? (uint32_t)(tok * D + v0) * 2u : kOOB, o);
        }
    };
    if constexpr (ROPE) {
        // the rotation makes this loop bound by the vector ALU: batches of PF
        // groups, loaded together, keep the register count (and occupancy) up;
        // the first batch was issued before the state was formed
        for (int i0 = 0; i0 < nw; i0 += PF) {
            u32x4_t qb[PF][KS];
            if (i0 == 0) {
#pragma unroll
                for (int p = 0; p < PF; ++p)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) qb[p][ks] = qreg[p][ks];
            } else {
#pragma unroll
                for (int p = 0; p < PF; ++p)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) qb[p][ks] = load8f<IN, SVLA_Q_AUX>(rQ, qoff(i0 + p, ks));
            }
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                if (i0 + p >= nw) break;
                group(i0 + p, qb[p]);
            }
        }
    } else {
        // a ring of PF groups in flight; the count is rounded up to a multiple
        // of PF (the extra groups load nothing and store nothing) so the loop
        // stays regular for the wait counts
        const int nwr = (nw + PF - 1) / PF * PF;
        for (int i0 = 0; i0 < nwr; i0 += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                const int i = i0 + p;
                u32x4_t qr[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qr[ks] = qreg[p][ks];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qreg[p][ks] = load8f<IN, SVLA_Q_AUX>(rQ, qoff(i + PF, ks));
                __builtin_amdgcn_sched_barrier(0);
                group(i, qr);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// svla_apply, bf16 inputs, d = 64 and 128: the block state and the token
// rows in LDS.
//
// Workgroup = (bh, block c, token tile); the tiles of one block run on one
// XCD.  The packed state operand of the block (d*d bf16, 1 KB per MFMA
// fragment) is copied to LDS once per workgroup, and the waves split the
// tile's 16-token groups (wave w takes groups w, w + 4, ...), so each Q
// element is loaded and prepared once.  Per group, O^T = S^T phi~(Q)^T on
// v_mfma_f32_16x16x32_bf16: the A fragments come from LDS, phi~(q) is the
// B operand (token = lane % 16, features 8 (4 ks + lane / 16) ...).  The
// denominator runs on the matrix cores too: one more A tile whose rows 4j
// and 4j + 1 hold z split into bf16 hi and lo parts (zero elsewhere),
// against the unrotated phi(q), puts phi(q) . z (to ~16 bits of z) in the
// first two accumulator values of every lane of the token.
//
// Memory accesses are whole rows: each wave owns a ring of PF slots, one
// 16-token group each.  A group's Q
// rows land in its slot straight from memory (buffer_load ... lds, every
// wave instruction one contiguous kilobyte of whole rows); the 16-byte
// chunks of row r sit at position chunk ^ (r mod chunks per row), so the
// MFMA operand reads (16 rows, one chunk each) hit distinct banks.  The
// output of the group goes back into the same slot in the same layout and
// leaves it as whole rows, one contiguous kilobyte per store instruction.
// No wave touches another wave's slots and the LDS operations of one wave
// execute in program order, so the ring needs no barrier.
// ---------------------------------------------------------------------------
template <int D, bool ROPE, int PF>
__global__ void __launch_bounds__(kThreads)
svla_apply_ring(const ApplyArgs a)
{
    constexpr int MT = D / 16;            // 16-feature m-tiles of the output
    constexpr int KS = D / 32;            // 32-deep k-steps
    constexpr int NFRAG = MT * KS;        // 1 KB fragments of the packed state
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int ROWB = D * 2;
    constexpr int RPI = 64 / CPR;         // rows one wave instruction covers
    constexpr int NI = 16 / RPI;          // wave instructions per group
    constexpr int SLOTB = 16 * ROWB;
    static_assert(NFRAG % 4 == 0, "the four waves copy the state in equal shares");
    static_assert(NI == KS, "one kilobyte per k-step");
    static_assert(PF >= 1 && PF <= 3, "ring depth");
    __shared__ __attribute__((aligned(16))) unsigned char sS[NFRAG * 1024];
    // ring position p of the four waves: an LDS object of its own, so the
    // compiler can tell a slot's reads from the loads in flight into the
    // other positions
    __shared__ __attribute__((aligned(16))) unsigned char r0[4 * SLOTB];
    __shared__ __attribute__((aligned(16))) unsigned char r1[PF > 1 ? 4 * SLOTB : 16];
    __shared__ __attribute__((aligned(16))) unsigned char r2[PF > 2 ? 4 * SLOTB : 16];
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];   // RoPE table

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const long lid = xcd_logical(a.groups);
    if (lid >= a.groups) return;
    const int tile = (int)(lid % a.tiles);
    const int c = (int)((lid / a.tiles) % a.nb);
    const long bh = lid / ((long)a.tiles * a.nb);
    const int t_lo = c * a.n + tile * a.tile;
    const int t_hi = min(t_lo + a.tile, (c + 1) * a.n);
    const long unit = bh * a.nb + c;

    const uint32_t slice = (uint32_t)a.N * D * 2;
    const auto rQ = make_rsrc((const char *)a.Q + bh * slice, slice);
    const auto rO = make_rsrc((char *)a.O + bh * slice, slice);
    const auto rS = make_rsrc((const char *)a.S_op + unit * D * D * 2, D * D * 2);
    const auto rz = make_rsrc(a.z_pre + unit * D, D * 4);
    const int kg = lane >> 4, tl = lane & 15;
    auto slot_of = [&](int p) -> unsigned char * {
        return (p == 0 ? r0 : p == 1 ? r1 : r2) + wave * SLOTB;
    };

    // 1. the state operand -> LDS, one fragment per wave instruction
    constexpr int FPW = NFRAG / 4;
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
        const int f = wave + 4 * j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_ptr_t)(sS + f * 1024), 16,
                                                 (uint32_t)(f * 1024 + lane * 16), 0, 0, 0);
    }
    // 2. z for this lane's k positions
    u32x4_t zr[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        zr[ks][0] = load16(rz, (uint32_t)(8 * (4 * ks + kg)) * 4u);
        zr[ks][1] = load16(rz, (uint32_t)(8 * (4 * ks + kg) + 4) * 4u);
    }
    // 3. the first PF groups of Q: this wave's group i -> slot i % PF; lane l
    // of instruction j brings row RPI j + l / CPR, chunk (l % CPR) ^ (row % CPR)
    const int ngroups = t_hi > t_lo ? (t_hi - t_lo + 15) / 16 : 0;
    const int nw = ngroups > wave ? (ngroups - wave + 3) / 4 : 0;
    const int nwr = (nw + PF - 1) / PF * PF;
    const int lrow = lane / CPR, lpos = lane % CPR;
    auto row_off = [&](int i, int j) -> uint32_t {      // global byte offset of lane's chunk, or kOOB
        const int row = RPI * j + lrow;
        const int tok = t_lo + 16 * (wave + 4 * i) + row;
        return tok < t_hi ? (uint32_t)(tok * D + ((lpos ^ (row & (CPR - 1))) * 8)) * 2u : kOOB;
    };
    auto issue = [&](int i, unsigned char *slot) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // (the offset in a variable of its own: with a lambda call as the
            // builtin's argument this compiler drops the kernel's host stub)
            const uint32_t off = row_off(i, j);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_ptr_t)(slot + j * 1024), 16, off, 0, 0, SVLA_Q_AUX);
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) issue(p, slot_of(p));

    // the z tile: lane (rho + 16 kg), k = 32 ks + 8 kg + i holds z_hi[k] in
    // rows rho = 4j, z_lo[k] in rows 4j + 1, 0 in the others
    wait_vmcnt<PF * NI>();
    bf16x8_t zt[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u16x8_t h;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = as_f32(zr[ks][i >> 2][i & 3]);
            const unsigned short hi = f2bf(v);
            const unsigned short lo = f2bf(v - as_f32((unsigned int)hi << 16));
            h[i] = (tl & 3) == 0 ? hi : (tl & 3) == 1 ? lo : (unsigned short)0;
        }
        zt[ks] = __builtin_bit_cast(bf16x8_t, h);
    }

    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<4> pp[KS];
    if constexpr (ROPE) {
        frame_lo = t_lo < t_hi ? fdiv((uint32_t)t_lo, a.rope.div_hw) : 0;
        const uint32_t frame_hi = t_lo < t_hi ? fdiv((uint32_t)(t_hi - 1), a.rope.div_hw) : 0;
        const int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pp[ks] = rope_pairs<4>(a.rope, 8 * (4 * ks + kg), nf);
    }
    lds_barrier();         // every wave's state fragments (and the table) are in LDS

    // the lane's operand row tl: chunk c sits at position c ^ (tl % CPR)
    const int rsw = tl & (CPR - 1);
    for (int i0 = 0; i0 < nwr; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int i = i0 + p;
            unsigned char *slot = slot_of(p);
            // this group's rows have landed: the loads of the PF - 1 later
            // groups may still be in flight.  Loads complete in order among
            // themselves, but the output stores between them may complete
            // before or after them, so the count admits no store.
            wait_vmcnt<(PF - 1) * NI>();
            const int tok = t_lo + 16 * (wave + 4 * i) + tl;
            u32x4_t qr[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qr[ks] = *(const u32x4_t *)(slot + tl * ROWB + (((4 * ks + kg) ^ rsw) * 16));

            bf16x8_t qu[KS], qf[KS];
            RopePos rp{0, 0, 0};
            if constexpr (ROPE) rp = rope_pos((uint32_t)tok, frame_lo, a.rope);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4_t pq;
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = relu_bf16x2(qr[ks][e]);
                qu[ks] = __builtin_bit_cast(bf16x8_t, pq);
                if constexpr (ROPE) {
                    float pf[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pf[2 * e] = bf16lo(pq[e]);
                        pf[2 * e + 1] = bf16hi(pq[e]);
                    }
                    rope_rotate<4>(pf, rp, pp[ks], tab);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pq[e] = pack_bf16(pf[2 * e], pf[2 * e + 1]);
                    qf[ks] = __builtin_bit_cast(bf16x8_t, pq);
                } else {
                    qf[ks] = qu[ks];
                }
            }
            f32x4_t dz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                dz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zt[ks], qu[ks], dz, 0, 0, 0);
            f32x4_t acc[MT];
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) acc[mi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8_t sf[MT];
#pragma unroll
                for (int mi = 0; mi < MT; ++mi)
                    sf[mi] = *(const bf16x8_t *)(sS + (mi * KS + ks) * 1024 + lane * 16);
#pragma unroll
                for (int mi = 0; mi < MT; ++mi)
                    acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[mi], qf[ks], acc[mi], 0, 0, 0);
            }
            const float den = dz[0] + dz[1] + a.eps;
            const float inv = den != 0.f ? 1.0f / den : 0.f;
            // m-tiles 2h, 2h + 1 hold O[tok][op_col(2h, 4 kg) + 0 .. 7], that is
            // chunk 4 h + kg of the output row: into the slot, over this group's Q
#pragma unroll
            for (int h = 0; h < MT / 2; ++h) {
                u32x4_t o;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    o[2 * e] = pack_bf16(acc[2 * h + e][0] * inv, acc[2 * h + e][1] * inv);
                    o[2 * e + 1] = pack_bf16(acc[2 * h + e][2] * inv, acc[2 * h + e][3] * inv);
                }
                *(u32x4_t *)(slot + tl * ROWB + (((4 * h + kg) ^ rsw) * 16)) = o;
            }
            // whole rows out, then the next group PF ahead into the slot.  The
            // slot's reads must have returned before its loads are issued: a
            // load writes LDS when its data arrives, which for a row past the
            // range (zeros, no memory access) can be almost at once.
            u32x4_t orow[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j) orow[j] = *(const u32x4_t *)(slot + j * 1024 + lane * 16);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int j = 0; j < NI; ++j) store16p<SVLA_O_AUX>(rO, row_off(i, j), orow[j]);
            issue(i + PF, slot);
        }
    }
    wait_vmcnt<0>();      // the trailing out-of-range loads target the ring too
}

// ---------------------------------------------------------------------------
// svla_apply, fp32 inputs: v_mfma_f32_16x16x4_f32, lane chunk = 4 features
// of chunk 4 kq + lane / 16; the state operand stays fp32.
// ---------------------------------------------------------------------------
template <int D, bool ROPE>
__global__ void __launch_bounds__(kThreads)
svla_apply_f32(const ApplyArgs a)
{
    constexpr int MT = D / 16;
    constexpr int KQ = D / 16;
    constexpr bool SPLITM = (D == 128);
    constexpr int MW = SPLITM ? 2 : MT;

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long lid = xcd_logical(a.groups);
    if (lid >= a.groups) return;
    const int tile = (int)(lid % a.tiles);
    const int c = (int)((lid / a.tiles) % a.nb);
    const long bh = lid / ((long)a.tiles * a.nb);
    const int t_lo = c * a.n + tile * a.tile;
    const int t_hi = min(t_lo + a.tile, (c + 1) * a.n);
    const long unit = bh * a.nb + c;

    const uint32_t slice = (uint32_t)a.N * D * 4;
    const auto rQ = make_rsrc((const char *)a.Q + bh * slice, slice);
    const auto rO = make_rsrc((char *)a.O + bh * slice, slice);
    const auto rS = make_rsrc((const char *)a.S_op + unit * D * D * 4, D * D * 4);
    const auto rz = make_rsrc(a.z_pre + unit * D, D * 4);

    const int kg = lane >> 4, tl = lane & 15;
    const int m0 = SPLITM ? 2 * wave : 0;

    f32x4_t sf[MW][KQ];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
            sf[mi][kq] = __builtin_bit_cast(f32x4_t,
                load16(rS, (uint32_t)((((m0 + mi) * KQ + kq) * 64 + lane) * 16)));
    f32x4_t zf[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
        zf[kq] = __builtin_bit_cast(f32x4_t, load16(rz, (uint32_t)(4 * (4 * kq + kg)) * 4u));

    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<2> pp[KQ];
    if constexpr (ROPE) {
        frame_lo = t_lo < t_hi ? fdiv((uint32_t)t_lo, a.rope.div_hw) : 0;
        uint32_t frame_hi = t_lo < t_hi ? fdiv((uint32_t)(t_hi - 1), a.rope.div_hw) : 0;
        int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) pp[kq] = rope_pairs<2>(a.rope, 4 * (4 * kq + kg), nf);
        __syncthreads();
    }

    const int ngroups = t_hi > t_lo ? (t_hi - t_lo + 15) / 16 : 0;
    const int g_first = SPLITM ? 0 : wave, g_step = SPLITM ? 1 : 4;
    for (int gi = g_first; gi < ngroups; gi += g_step) {
        const int tok = t_lo + 16 * gi + tl;
        const bool valid = tok < t_hi;
        float qv[KQ][4];
        float den = 0.f;
        RopePos rp{0, 0, 0};
        if constexpr (ROPE) rp = rope_pos((uint32_t)tok, frame_lo, a.rope);
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
            u32x4_t r = load16(rQ, valid ? (uint32_t)(tok * D + 4 * (4 * kq + kg)) * 4u : kOOB);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qv[kq][e] = fmaxf(as_f32(r[e]), 0.f);
                den = fmaf(qv[kq][e], zf[kq][e], den);
            }
            if constexpr (ROPE) rope_rotate<2>(qv[kq], rp, pp[kq], tab);
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        den += a.eps;
        const float inv = den != 0.f ? 1.0f / den : 0.f;
        f32x4_t acc[MW];
#pragma unroll
        for (int mi = 0; mi < MW; ++mi) {
            acc[mi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[mi] = __builtin_amdgcn_mfma_f32_16x16x4f32(sf[mi][kq][i], qv[kq][i], acc[mi], 0, 0, 0);
        }
#pragma unroll
        for (int mi = 0; mi < MW; ++mi) {
            u32x4_t o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = as_u32(acc[mi][r] * inv);
            const int v0 = op_col(m0 + mi, 4 * kg);
            store16(rO, valid ? (uint32_t)(tok * D + v0) * 4u : kOOB, o);
        }
    }
}

// ---------------------------------------------------------------------------
// svla_step_fused: a one-block call (a block step, or a non-causal call over
// a short sequence) of bf16 or fp8 inputs at d = 32 in one launch, with no
// hand-off between workgroups.
//
// Workgroup = (bh, tile t), `tiles` workgroups per (bh), all on one XCD (the
// tiles of a bh are 8 workgroup ids apart and the dispatch is round-robin over
// the eight XCDs).  Every workgroup builds the block's whole state itself:
// the workgroups of one bh read the same K and V rows, which their shared L2
// serves after the first miss, and sum them in the same fixed order, so they
// all hold the same bits.  Each adds the decayed carried state and reads out
// the Q rows of its own tile; tile 0 writes the new state.  The host takes
// this path only when the new state does not overlap the carried one, so no
// workgroup of a launch reads memory that another one writes, and nothing
// waits on another workgroup.
//
// Order: every wave issues the K/V loads of its first PRE (2) 16-token
// stages, the RoPE table is filled (the one barrier before the build), then
// the other prefetched stages, the tile's Q rows and the carried state are
// issued, so the build starts while the loads still stream in.  With RoPE
// two stages are in flight per wave, without it three.  (Measured on the
// minute-long step, us per step: 3 in flight with 1 before the table 11.3,
// with 2 10.9, with 3 10.9; 2 in flight with 2 before the table 10.5, with
// 1 10.8; 1 in flight 11.0; 4 in flight 11.4 - 11.5; every prefetched load
// including Q before the table was slower, and so was Q issued only after
// the build, 10.7.  On the 720p step without RoPE, 3 in flight beat 2 by
// 1.5 %.)
//
// Build: W waves, wave w takes stages w, w + W, ... of the block (one token
// row chunk of 16 bytes per lane and tensor, PF stages in flight in
// registers, exactly the stages the wave owns); phi (and with RoPE the
// rotation, the key split into bf16 hi + lo) is applied in registers, the
// stage goes through a wave-private LDS slot, and the token contraction runs
// on v_mfma_f32_32x32x16_bf16 from transposing reads; z sums the unrotated
// phi(k) on the vector ALU.  A lane's token advances by 16 W per stage, so its
// grid position is stepped with carries instead of divided out, and its two
// 4-feature groups read their (cos, sin) pairs as two 16-byte entries.
// Epilogue: each wave stores its 32x32 tile and its z sums (reduced across
// the wave by DPP and lane swaps) in an LDS area of its own, so it does not
// wait for the other waves' stage slots; after one barrier thread e sums
// element e of the W tiles in wave order, adds the decayed carried state and
// writes a transposed copy for the read-out (tile 0 also the new state).
// Read-out: O^T = S^T phi~(Q)^T on v_mfma_f32_16x16x32_bf16 with the state
// as the A operand in registers.
// ---------------------------------------------------------------------------
struct StepArgs {
    const void *Q, *K, *V;
    void *O;
    const float *S_in, *z_in;      // carried state or null
    const float *g;                // [BH] decay of the carried state, or null
    float *S_out, *z_out;          // new state or null
    int n;                         // tokens of the block
    int tiles, tile;               // workgroups per bh, tokens per workgroup (multiple of 16)
    int work_bytes;                // dynamic LDS after the RoPE table (stage slots, tiles, state)
    long BH;
    float eps;
    RopeK rope;
};

// Sum over the lanes of a wave that share lane % 4: rotations by 4 and 8
// inside each row of 16 lanes, then swaps of rows and of halves.
__device__ __forceinline__ float wave_sum_mod4(float v)
{
    v += as_f32((unsigned int)__builtin_amdgcn_update_dpp(0, (int)as_u32(v), 0x124, 0xF, 0xF, false));
    v += as_f32((unsigned int)__builtin_amdgcn_update_dpp(0, (int)as_u32(v), 0x128, 0xF, 0xF, false));
    const auto r16 = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
    v = as_f32(r16[0]) + as_f32(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return as_f32(r32[0]) + as_f32(r32[1]);
}

// LDS bytes of the one-launch step after the RoPE table: W stage slots, W
// tiles of 32 x 32 floats, W z sums, the transposed state and z.
constexpr int fused_slot_bytes(bool rope) { return (rope ? 3 : 2) * 1024; }
constexpr int kFusedSLD = 36;                 // row stride (floats) of the transposed state
constexpr int fused_work_bytes(bool rope, int W)
{
    return W * fused_slot_bytes(rope) + W * 4096 + W * 128 + (32 * kFusedSLD + 32) * 4;
}

template <bool ROPE, int W, int PF, int QG, int IN = 2>
__global__ void __launch_bounds__(64 * W)
svla_step_fused(const StepArgs a)
{
    constexpr int D = 32;
    constexpr int ROWB = D * 2;           // 64 bytes per token row
    constexpr int TILEB = 16 * ROWB;      // one 16-token stage of one tensor
    constexpr int NK = ROPE ? 2 : 1;      // K tiles per stage: (rotated) hi, lo
    constexpr int SLOTB = (NK + 1) * TILEB;
    constexpr int SLD = kFusedSLD;
    constexpr int EPT = 1024 / (64 * W);  // state elements per thread in the epilogue
    static_assert(SLOTB == fused_slot_bytes(ROPE), "slot size");
    static_assert(16 % W == 0, "W divides 16");
    static_assert(2 * PF + QG + EPT + 1 < 64, "the loads issued together must fit the vmcnt counter");

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int k8 = (int)(blockIdx.x >> 3);
    const long bh = 8L * (k8 / a.tiles) + (blockIdx.x & 7);
    const int tile = k8 % a.tiles;
    if (bh >= a.BH) return;
    const int n = a.n;
    const int t_lo = tile * a.tile, t_hi = min(t_lo + a.tile, n);

    const uint32_t slice = (uint32_t)n * D * 2;                 // O: bf16
    const uint32_t islice = (uint32_t)n * D * IN;               // Q, K, V: bf16 or fp8
    const auto rK = make_rsrc((const char *)a.K + bh * islice, islice);
    const auto rV = make_rsrc((const char *)a.V + bh * islice, islice);
    const auto rQ = make_rsrc((const char *)a.Q + bh * islice, islice);
    const auto rO = make_rsrc((char *)a.O + bh * slice, slice);

    unsigned char *tabp = lds;
    unsigned char *work = lds + (ROPE ? a.rope.tab_bytes : 0);
    float *red = (float *)(work + W * SLOTB);              // W tiles, [c][lane][4] each
    float *zred = red + W * 1024;                          // W x D z sums
    float *stT = zred + W * D;                             // S^T [v][SLD], then z

    // 1. the K/V loads of this wave's first PRE stages: stage st = wave + W i;
    // lane -> row lane / 4 of the stage, chunk lane % 4
    const int row = lane >> 2, q = lane & 3;
    const int nst = (n + 15) / 16;
    const int nw = nst > wave ? (nst - wave + W - 1) / W : 0;
    auto kv_off = [&](int i) -> uint32_t {
        const int t = 16 * (wave + W * i) + row;
        return t < n ? (uint32_t)(t * D + q * 8) * (uint32_t)IN : kOOB;
    };
    u32x4_t kreg[PF], vreg[PF];
    constexpr int PRE = SVLA_FUSED_PRE < PF ? SVLA_FUSED_PRE : PF;   // stages issued before the table
#pragma unroll
    for (int p = 0; p < PRE; ++p) {
        kreg[p] = load8f<IN, 0>(rK, kv_off(p));
        vreg[p] = load8f<IN, 0>(rV, kv_off(p));
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. the RoPE table, frames of every row of the padded stages
    const int nf = ROPE ? (16 * nst - 1) / (a.rope.gh * a.rope.gw) + 1 : 1;
    if constexpr (ROPE) {
        gtab_fill((float2 *)tabp, a.rope, nf);
        lds_barrier();
    }

    // 3. the other prefetched stages, this wave's Q groups of the tile (in
    // the read-out's operand layout: token lane % 16 of the group, features
    // 8 (lane / 16) ..), the carried state elements of this thread
#pragma unroll
    for (int p = PRE; p < PF; ++p) {
        kreg[p] = load8f<IN, 0>(rK, kv_off(p));
        vreg[p] = load8f<IN, 0>(rV, kv_off(p));
        __builtin_amdgcn_sched_barrier(0);
    }
    const int kg = lane >> 4, tl = lane & 15;
    u32x4_t qreg[QG];
    auto load_q = [&]() {
#pragma unroll
        for (int j = 0; j < QG; ++j) {
            const int tok = t_lo + 16 * (wave + W * j) + tl;
            qreg[j] = load8f<IN, SVLA_Q_AUX>(rQ, tok < t_hi ? (uint32_t)(tok * D + 8 * kg) * (uint32_t)IN : kOOB);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (!SVLA_FUSED_QLATE) load_q();
    // element e = c 256 + l 4 + r' of the epilogue is register 4 c + r' of
    // lane l of a tile: S[8 c + 4 (l / 32) + r'][l % 32]
    auto elem_k = [](int e) { return 8 * (e >> 8) + 4 * ((e >> 7) & 1) + (e & 3); };
    auto elem_v = [](int e) { return (e >> 2) & 31; };
    const float gb = a.g ? a.g[bh] : 1.f;
    float s_in[EPT], z_in = 0.f;
#pragma unroll
    for (int u = 0; u < EPT; ++u) s_in[u] = 0.f;
    if (a.S_in) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + 64 * W * u;
            s_in[u] = a.S_in[bh * D * D + elem_k(e) * D + elem_v(e)];
        }
        if (tid < D) z_in = a.z_in[bh * D + tid];
    }

    // RoPE: this lane's table groups, walked from its first token by 16 W
    // tokens per stage
    GroupWalk walk{};
    if constexpr (ROPE) walk = group_walk(gtab_groups(a.rope, q, nf), a.rope, (uint32_t)(16 * wave + row), 16u * W);
    unsigned char *slot = work + wave * SLOTB;

    // 4. the block's state, this wave's stages
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float zacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[e] = 0.f;
    const int fl = trb_offset<D>(lane, 0);
    // stage i (ring slot p = i % PF): phi, rotation, split, the slot, the
    // refill with stage i + PF (past the wave's last stage: an offset out of
    // range, read as zeros), the contraction
    auto stage = [&](int i, u32x4_t &kr, u32x4_t &vr) {
        float kf[8];
        feat8<IN, true>(kr, kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) zacc[e] += kf[e];
        if constexpr (ROPE) {
            rot_group(kf, *(const f32x4_t *)(tabp + walk.off[0]));
            rot_group(kf + 4, *(const f32x4_t *)(tabp + walk.off[1]));
            walk_step(walk);
            u32x4_t hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = pack_bf16(kf[2 * e], kf[2 * e + 1]);
                lo[e] = pack_bf16(kf[2 * e] - bf16lo(hi[e]), kf[2 * e + 1] - bf16hi(hi[e]));
            }
            *(u32x4_t *)(slot + row * ROWB + q * 16) = hi;
            *(u32x4_t *)(slot + TILEB + row * ROWB + q * 16) = lo;
        } else {
            *(u32x4_t *)(slot + row * ROWB + q * 16) = bf16x8_of<IN, true>(kr);
        }
        *(u32x4_t *)(slot + NK * TILEB + row * ROWB + q * 16) = bf16x8_of<IN, false>(vr);
        __builtin_amdgcn_sched_barrier(0);
        kr = load8f<IN, 0>(rK, kv_off(i + PF));
        vr = load8f<IN, 0>(rV, kv_off(i + PF));
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8_t av = trb_load<D>(slot, fl);
        const bf16x8_t bv = trb_load<D>(slot + NK * TILEB, fl);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
        if constexpr (ROPE) {
            const bf16x8_t al = trb_load<D>(slot + TILEB, fl);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, acc, 0, 0, 0);
        }
    };
    // whole rounds of PF stages (no exit inside a round, so every wait in the
    // loop counts the same PF - 1 stages of loads behind it), then the rest
    const int rounds = nw / PF;
    for (int i0 = 0; i0 < rounds * PF; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) stage(i0 + p, kreg[p], vreg[p]);
    }
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p)
        if (rounds * PF + p < nw) stage(rounds * PF + p, kreg[p], vreg[p]);

    if constexpr (SVLA_FUSED_QLATE) load_q();

    // 5. this wave's tile and z sums into its own LDS area
    {
        f32x4_t *dst = (f32x4_t *)(red + wave * 1024) + lane;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dst[64 * c] = (f32x4_t){acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[e] = wave_sum_mod4(zacc[e]);
    if (lane < 4) {
        f32x4_t *zd = (f32x4_t *)(zred + wave * D + 8 * lane);
        zd[0] = (f32x4_t){zacc[0], zacc[1], zacc[2], zacc[3]};
        zd[1] = (f32x4_t){zacc[4], zacc[5], zacc[6], zacc[7]};
    }
    lds_barrier();

    // 6. element e summed over the W tiles in wave order, plus the decayed
    // carried state; the transposed copy for the read-out, the new state
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int e = tid + 64 * W * u;
        float t = red[e];
#pragma unroll
        for (int w = 1; w < W; ++w) t += red[w * 1024 + e];
        const float s = gb * s_in[u] + t;
        const int k = elem_k(e), v = elem_v(e);
        stT[v * SLD + k] = s;
        if (tile == 0 && a.S_out) a.S_out[bh * D * D + k * D + v] = s;
    }
    if (tid < D) {
        float t = zred[tid];
#pragma unroll
        for (int w = 1; w < W; ++w) t += zred[w * D + tid];
        const float z = gb * z_in + t;
        stT[D * SLD + tid] = z;
        if (tile == 0 && a.z_out) a.z_out[bh * D + tid] = z;
    }
    lds_barrier();

    // 7. the state as A fragments: lane (rho + 16 kg), value i = S[8 kg + i][op_col(mi, rho)]
    bf16x8_t sf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const float *col = stT + op_col(mi, tl) * SLD + 8 * kg;
        const f32x4_t lo = *(const f32x4_t *)col, hi = *(const f32x4_t *)(col + 4);
        const u32x4_t w = {pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(hi[0], hi[1]),
                           pack_bf16(hi[2], hi[3])};
        sf[mi] = __builtin_bit_cast(bf16x8_t, w);
    }
    float zf[8];
    {
        const f32x4_t z0 = *(const f32x4_t *)(stT + D * SLD + 8 * kg);
        const f32x4_t z1 = *(const f32x4_t *)(stT + D * SLD + 8 * kg + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { zf[e] = z0[e]; zf[4 + e] = z1[e]; }
    }
    GroupAddr gq{};
    if constexpr (ROPE) gq = gtab_groups(a.rope, kg, nf);

    // 8. read-out of this wave's groups of the tile
    const int ngroups = t_hi > t_lo ? (t_hi - t_lo + 15) / 16 : 0;
    const int nq = ngroups > wave ? (ngroups - wave + W - 1) / W : 0;
#pragma unroll
    for (int j = 0; j < QG; ++j) {
        if (j >= nq) break;                     // (uniform)
        const int tok = t_lo + 16 * (wave + W * j) + tl;
        const bool valid = tok < t_hi;
        const u32x4_t qr = qreg[j];
        u32x4_t pq = {0u, 0u, 0u, 0u};
        if constexpr (IN == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) pq[e] = relu_bf16x2(qr[e]);
        }
        float pf[8];
        feat8<IN, true>(qr, pf);
        float den = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) den = fmaf(pf[e], zf[e], den);
        if constexpr (ROPE) {
            const uint32_t hw = (uint32_t)(a.rope.gh * a.rope.gw);
            const uint32_t fr = fdiv((uint32_t)tok, a.rope.div_hw), rem = (uint32_t)tok - fr * hw;
            const uint32_t rw = fdiv(rem, a.rope.div_w), cl = rem - rw * (uint32_t)a.rope.gw;
            rot_group(pf, *(const f32x4_t *)(tabp + gtab_off(gq, 0, (int)fr, (int)rw, (int)cl)));
            rot_group(pf + 4, *(const f32x4_t *)(tabp + gtab_off(gq, 1, (int)fr, (int)rw, (int)cl)));
        }
        if constexpr (ROPE || IN != 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) pq[e] = pack_bf16(pf[2 * e], pf[2 * e + 1]);
        }
        const bf16x8_t qf = __builtin_bit_cast(bf16x8_t, pq);
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        den += a.eps;
        const float inv = den != 0.f ? 1.0f / den : 0.f;
        f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
        o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[0], qf, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[1], qf, o1, 0, 0, 0);
        // m-tiles 0 and 1 hold O[tok][8 kg .. 8 kg + 7]
        u32x4_t o;
        o[0] = pack_bf16(o0[0] * inv, o0[1] * inv);
        o[1] = pack_bf16(o0[2] * inv, o0[3] * inv);
        o[2] = pack_bf16(o1[0] * inv, o1[1] * inv);
        o[3] = pack_bf16(o1[2] * inv, o1[3] * inv);
        store16p<SVLA_O_AUX>(rO, valid ? (uint32_t)(tok * D + op_col(0, 4 * kg)) * 2u : kOOB, o);
    }
}
// ---------------------------------------------------------------------------
// svla_temporal_conv: the Mix-FFN's temporal convolution made causal across
// blocks.  y[t,p,c] = bias[c] + w[c][0] x[t-1,p,c] + w[c][1] x[t,p,c] +
// w[c][2] x[t+1,p,c], where a block's first frame reads the previous block's
// last frame (the cache before the call's first frame) and a block's last
// frame reads zero in place of the next frame.
//
// Thread = (b, grid position p, chunk of 8 channels), the chunk fastest, so
// every load or store instruction of a wave covers 64 consecutive 16-byte
// (bf16) or 32-byte (fp32) pieces of a row of channels.  Each thread walks
// all T frames in chunks of MAXF frames, all loads of a chunk issued before
// any is used, carrying the previous frame in registers: every element of X
// is read once (plus one look-ahead frame per chunk boundary, which the L2
// serves) and every element of Y written once.  The thread that reads its
// cache element is the one that writes the new cache element, after it, so
// the cache may be committed in place.
// ---------------------------------------------------------------------------
struct ConvArgs {
    const void *X;
    void *Y;
    const float *w, *bias;          // [C][3], [C] or null
    const void *cache_in;           // [B][P][C] or null (zero)
    void *cache_out;                // [B][P][C] or null
    int T, F, P, C8;                // frames, frames per block, positions, 8-channel chunks
    long units;                     // B * P * C8
};

template <int ES>                   // bytes per element: 2 (bf16) or 4 (fp32)
struct Chunk8 {
    static constexpr int NL = ES / 2;            // 16-byte loads per 8 channels
    u32x4_t q[NL];
};

template <int ES, int AUX = 0>
__device__ __forceinline__ Chunk8<ES> chunk_load(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    Chunk8<ES> c;
#pragma unroll
    for (int i = 0; i < Chunk8<ES>::NL; ++i) c.q[i] = load16p<AUX>(r, off == kOOB ? kOOB : off + 16u * i);
    return c;
}

template <int ES>
__device__ __forceinline__ void chunk_floats(const Chunk8<ES> &c, float *f)
{
    if constexpr (ES == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = bf16lo(c.q[0][e]);
            f[2 * e + 1] = bf16hi(c.q[0][e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = as_f32(c.q[e >> 2][e & 3]);
    }
}

template <int ES, int MAXF>
__global__ void __launch_bounds__(kThreads)
svla_temporal_conv_k(const ConvArgs a)
{
    const long u = (long)blockIdx.x * kThreads + threadIdx.x;
    if (u >= a.units) return;
    const int c8 = (int)(u % a.C8);
    const long r = u / a.C8;
    const int p = (int)(r % a.P);
    const long b = r / a.P;
    const uint32_t rowb = (uint32_t)a.C8 * 8u * ES;             // bytes per (t, p) row of channels
    const uint32_t slice = (uint32_t)a.T * (uint32_t)a.P * rowb;
    const auto rX = make_rsrc((const char *)a.X + b * slice, slice);
    const auto rY = make_rsrc((char *)a.Y + b * slice, slice);
    const uint32_t col = (uint32_t)p * rowb + (uint32_t)c8 * 8u * ES;   // (p, chunk) within a frame
    auto off = [&](int t) -> uint32_t { return t < a.T ? (uint32_t)t * (uint32_t)a.P * rowb + col : kOOB; };

    // the taps and bias of this thread's 8 channels
    float w0[8], w1[8], w2[8], bs[8];
    {
        const f32x4_t *wp = (const f32x4_t *)(a.w + (long)c8 * 24);
        float wv[24];
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const f32x4_t v = wp[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[4 * i + e] = v[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            w0[e] = wv[3 * e];
            w1[e] = wv[3 * e + 1];
            w2[e] = wv[3 * e + 2];
        }
        f32x4_t b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
        if (a.bias) {
            b0 = *(const f32x4_t *)(a.bias + (long)c8 * 8);
            b1 = *(const f32x4_t *)(a.bias + (long)c8 * 8 + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bs[e] = b0[e];
            bs[4 + e] = b1[e];
        }
    }
    const uint32_t coff = (uint32_t)(b * a.P + p) * rowb + (uint32_t)c8 * 8u * ES;   // cache offset
    const uint32_t cbytes = (uint32_t)a.units * 8u * ES;
    float prev[8];
    {
        Chunk8<ES> pc;
#pragma unroll
        for (int i = 0; i < Chunk8<ES>::NL; ++i) pc.q[i] = (u32x4_t){0u, 0u, 0u, 0u};
        if (a.cache_in) pc = chunk_load<ES>(make_rsrc(a.cache_in, cbytes), coff);
        chunk_floats<ES>(pc, prev);
    }
    float last[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) last[e] = prev[e];
    int phase = 0;                                              // t % F
    for (int t0 = 0; t0 < a.T; t0 += MAXF) {
        // this chunk's frames and, when the chunk ends inside a block, the next frame
        Chunk8<ES> v[MAXF + 1];
#pragma unroll
        for (int j = 0; j < MAXF; ++j) v[j] = chunk_load<ES, SVLA_TCONV_XAUX>(rX, off(t0 + j));
        const int end = t0 + MAXF < a.T ? t0 + MAXF : a.T;
        const bool look = end < a.T && (end % a.F) != 0;       // frame end - 1 is not a block end
        v[MAXF] = chunk_load<ES>(rX, look ? off(end) : kOOB);
#pragma unroll
        for (int j = 0; j < MAXF; ++j) {
            const int t = t0 + j;
            if (t >= a.T) break;
            float cur[8], nxt[8];
            chunk_floats<ES>(v[j], cur);
            chunk_floats<ES>(v[j + 1], nxt);
            const bool block_end = phase == a.F - 1;            // then the next frame reads as zero
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                y[e] = fmaf(w2[e], block_end ? 0.f : nxt[e], fmaf(w1[e], cur[e], fmaf(w0[e], prev[e], bs[e])));
            if constexpr (ES == 2) {
                u32x4_t o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = pack_bf16(y[2 * e], y[2 * e + 1]);
                store16p<SVLA_TCONV_YAUX>(rY, off(t), o);
            } else {
                u32x4_t o0, o1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = as_u32(y[e]);
                    o1[e] = as_u32(y[4 + e]);
                }
                store16p<SVLA_TCONV_YAUX>(rY, off(t), o0);
                store16p<SVLA_TCONV_YAUX>(rY, off(t) + 16u, o1);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                prev[e] = cur[e];
                last[e] = cur[e];
            }
            phase = phase == a.F - 1 ? 0 : phase + 1;
        }
    }
    if (a.cache_out) {
        const auto rC = make_rsrc(a.cache_out, cbytes);
        if constexpr (ES == 2) {
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_bf16(last[2 * e], last[2 * e + 1]);   // exact: bf16 values
            store16(rC, coff, o);
        } else {
            u32x4_t o0, o1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o0[e] = as_u32(last[e]);
                o1[e] = as_u32(last[4 + e]);
            }
            store16(rC, coff, o0);
            store16(rC, coff + 16u, o1);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward pass: the gradients of the block-causal forward, for block-causal
// training (SANA-Video talk, the passage on causal training: a block cannot
// see the next one).  Per (b,h), with p = phi(q), a = phi(k), p~ = R p,
// a~ = R a, S_c / z_c the inclusive state of block c and, for token i of
// block c, num_i = S_c^T p~_i, den_i = p_i . z_c + eps, O_i = num_i / den_i:
//   dnum_i = dO_i / den_i, dden_i = -(dO_i . O_i) / den_i
//   dq_i = [q_i > 0] (R_i^T S_c dnum_i + dden_i z_c)
//   G_c = sum_{i in c} p~_i dnum_i^T + g_{c+1} G_{c+1},
//   H_c = sum_{i in c} dden_i p_i + g_{c+1} H_{c+1}   (the gradient reaching S_c, z_c)
//   dv_j = G_c^T a~_j, dk_j = [k_j > 0] (R_j^T G_c v_j + H_c)
//   dg_c = <G_c, S_{c-1}> + <H_c, z_{c-1}>, dS0 = g_0 G_0, dz0 = g_0 H_0.
// Three kernels after the forward state is rebuilt (state build + export
// scan): the query side (dq and each split's share of the sums of G and H),
// the reverse scan over blocks (G_c, H_c, dS0, dz0) and the key side (dk,
// dv, dg).  All sums are fp32.  Every product over features or tokens runs
// on v_mfma_f32_16x16x4f32, except for bf16 inputs at d = 32: there the
// fp32 operands are split into bf16 hi + lo and the products run on the
// bf16 matrix instructions (hi hi + hi lo + lo hi, about 2^-16 relative; a
// bf16 value's lo part is zero and its products are skipped).
//
// Lane layout of the per-token work: the kernels run on
// v_mfma_f32_16x16x4f32 with the MFMA's output rows as features and its
// columns as tokens.  In a 16-token group of a wave, lane (n = lane % 16,
// q = lane / 16) owns token n and the d/4 consecutive features
// F(q, L) = (d/4) q + L, L < d/4: register i of output tile t is local
// feature L = 4 t + i.  The state operand picks the feature order: tile t's
// row m holds feature pi(t, m) = (d/4) (m / 4) + 4 t + m % 4, which is the
// feature that row lands on in lane group m / 4.  A contraction over features
// takes its k-slots in any order as long as both operands agree, so at step s
// the k-slot of lane group q is feature F(q, s): the B operand is then a
// register the lane already holds (its own p~, dnum, a~ or v) and only the
// state operand is read.  Every per-token vector (q, dO, num, dnum, dp~, k, v,
// dv, da~) lives in this layout, so the element-wise steps and RoPE's pairs
// need no data exchange, and a lane's features are contiguous in memory: one
// wave instruction of 16-byte accesses covers whole 64-byte rows of 16
// tokens (bf16, d = 32).  The four lanes of a token meet through two lane
// swaps for each dot product over features.  The sum over tokens of
// p~ dnum^T goes through a per-wave LDS tile (rows padded to d + 16 floats,
// which spreads the four token rows a step reads over the banks, and 4-float
// chunks swapped per row, which spreads the 16 rows a write touches).
// ---------------------------------------------------------------------------
struct BwdArgs {
    const void *Q, *K, *V, *dO;
    void *dQ, *dK, *dV;
    const float *S_pre, *z_pre;    // inclusive forward states [BH*nb][d*d], [BH*nb][d]
    float *dS_part, *dz_part;      // query side: [BH*nb][splits][d*d], [BH*nb][splits][d]
    float *G, *Hz;                 // reverse scan: [BH*nb][d*d], [BH*nb][d]
    const float *g, *S0, *z0;      // gate [BH][nb], state entering block 0 (each nullable)
    float *dg, *dS0, *dz0;         // [BH][nb], [BH][d*d], [BH][d] (each nullable)
    int N, n, nb, splits, chunk;   // splits of a block's tokens, tokens per split (a multiple of 16)
    long BH;
    float eps;
    RopeK rope;
};

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// A lane's d/4 features of one token, as stored (bf16 when ES == 2, fp32 when 4).
template <int D, int ES>
struct LaneRaw {
    static constexpr int NC = D / 4 * ES / 16;     // 16-byte chunks
    u32x4_t c[NC];
};

template <int D, int ES>
__device__ __forceinline__ void bwd_load(LaneRaw<D, ES> &v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
#pragma unroll
    for (int i = 0; i < LaneRaw<D, ES>::NC; ++i)
        v.c[i] = load16(r, off == kOOB ? kOOB : off + 16u * i);
}

template <int D, int ES>
__device__ __forceinline__ void bwd_floats(const LaneRaw<D, ES> &v, float *f)
{
#pragma unroll
    for (int i = 0; i < LaneRaw<D, ES>::NC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ES == 2) {
                f[8 * i + 2 * e] = bf16lo(v.c[i][e]);
                f[8 * i + 2 * e + 1] = bf16hi(v.c[i][e]);
            } else {
                f[4 * i + e] = as_f32(v.c[i][e]);
            }
        }
}

template <int D, int ES>
__device__ __forceinline__ void bwd_pack(LaneRaw<D, ES> &v, const float *f)
{
#pragma unroll
    for (int i = 0; i < LaneRaw<D, ES>::NC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ES == 2) v.c[i][e] = pack_bf16(f[8 * i + 2 * e], f[8 * i + 2 * e + 1]);
            else v.c[i][e] = as_u32(f[4 * i + e]);
        }
}

// Stores are not ordered with loads in the wait counter, so a wait for a load
// also waits for every store issued before it.  The kernels therefore hold a
// group's results and store them one group later, just before the next loads
// go out: by the time those loads are waited for, the stores have had a whole
// group's work to complete.
template <int D, int ES>
struct Pending {
    LaneRaw<D, ES> v;
    uint32_t off = kOOB;        // byte offset of the lane's features; kOOB: nothing pending
};

template <int D, int ES>
__device__ __forceinline__ void bwd_flush(__amdgpu_buffer_rsrc_t r, const Pending<D, ES> &p)
{
#pragma unroll
    for (int i = 0; i < LaneRaw<D, ES>::NC; ++i)
        store16(r, p.off == kOOB ? kOOB : p.off + 16u * i, p.v.c[i]);
}

// x <- R^T x for the pairs (x[2j], x[2j+1]) of a token at `pos` (the inverse
// rotation: the angles of rope_rotate, negated).
template <int PAIRS>
__device__ __forceinline__ void rope_rotate_t(float *x, const RopePos &pos,
                                              const RopePairs<PAIRS> &pp, const float2 *tab)
{
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
        const int idx = pp.base[j] + (pos.fr & pp.mt[j]) + (pos.row & pp.mh[j]) + (pos.col & pp.mw[j]);
        const float2 cs = tab[idx];
        const float x0 = x[2 * j], x1 = x[2 * j + 1];
        x[2 * j] = x0 * cs.x + x1 * cs.y;
        x[2 * j + 1] = x1 * cs.x - x0 * cs.y;
    }
}

// The state (S_c or G_c) of one block into LDS twice: M[k][j] row-major and
// its transpose Mt[j][k] (rows of d floats), and the vector (z_c or H_c).
template <int D>
__device__ __forceinline__ void bwd_state_to_lds(const float *S, const float *z, float *M, float *Mt,
                                                 float *vec)
{
    for (int e = threadIdx.x * 4; e < D * D; e += kThreads * 4) {
        const f32x4_t v = *(const f32x4_t *)(S + e);
        *(f32x4_t *)(M + e) = v;
        const int k = e / D, j = e % D;
#pragma unroll
        for (int i = 0; i < 4; ++i) Mt[(j + i) * D + k] = v[i];
    }
    if (threadIdx.x < D) vec[threadIdx.x] = z[threadIdx.x];
}

// Feature held by row m of output tile t (see the lane layout above).
template <int D>
__device__ __forceinline__ int bwd_pi(int t, int m) { return D / 4 * (m >> 2) + 4 * t + (m & 3); }

// The state operands of the two feature contractions, for lane (m, q):
// fwd[t][s] = M[F(q, s)][pi(t, m)] (output rows pi, k-slots F) and
// bwd[t][s] = M[pi(t, m)][F(q, s)] = Mt[F(q, s)][pi(t, m)].  With HOLD (d = 32
// only) they are read once per workgroup into registers, otherwise from LDS
// per instruction (fewer registers, more waves per SIMD).
template <int D, bool HOLD>
struct StateOps {
    static constexpr bool REG = HOLD && D == 32;
    float fwd[REG ? D / 16 : 1][REG ? D / 4 : 1], bwd[REG ? D / 16 : 1][REG ? D / 4 : 1];
    const float *M, *Mt;
    int q, m;
    __device__ __forceinline__ void init(const float *M_, const float *Mt_, int q_, int m_)
    {
        M = M_; Mt = Mt_; q = q_; m = m_;
        if constexpr (REG) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
#pragma unroll
                for (int s = 0; s < D / 4; ++s) {
                    fwd[t][s] = M[(D / 4 * q + s) * D + bwd_pi<D>(t, m)];
                    bwd[t][s] = Mt[(D / 4 * q + s) * D + bwd_pi<D>(t, m)];
                }
        }
    }
    __device__ __forceinline__ float f(int t, int s) const
    {
        if constexpr (REG) return fwd[t][s];
        else return M[(D / 4 * q + s) * D + bwd_pi<D>(t, m)];
    }
    __device__ __forceinline__ float b(int t, int s) const
    {
        if constexpr (REG) return bwd[t][s];
        else return Mt[(D / 4 * q + s) * D + bwd_pi<D>(t, m)];
    }
};

// An fp32 operand as bf16 hi + lo (hi = the value rounded to bf16, lo = the
// remainder rounded to bf16): hi + lo keeps about 16 bits of the value, and a
// product of two such operands taken as hi hi + hi lo + lo hi on the bf16
// matrix instructions (exact products, fp32 sums) is accurate to about 2^-16
// relative, against the bf16 output rounding of 2^-9.
__device__ __forceinline__ void split_bf16x8(const float *x, bf16x8_t &hi, bf16x8_t &lo)
{
    u32x4_t h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
        l[e] = pack_bf16(x[2 * e] - bf16lo(h[e]), x[2 * e + 1] - bf16hi(h[e]));
    }
    hi = __builtin_bit_cast(bf16x8_t, h);
    lo = __builtin_bit_cast(bf16x8_t, l);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void split_bf16x4(const float *x, i16x4_t &hi, i16x4_t &lo)
{
    typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
    u32x2_t h, l;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        h[e] = pack_bf16(x[2 * e], x[2 * e + 1]);
        l[e] = pack_bf16(x[2 * e] - bf16lo(h[e]), x[2 * e + 1] - bf16hi(h[e]));
    }
    hi = __builtin_bit_cast(i16x4_t, h);
    lo = __builtin_bit_cast(i16x4_t, l);
}

// Sum of x over the four lanes (q = 0..3) of a token.
__device__ __forceinline__ float token_sum(float x)
{
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Query side.  Workgroup = (bh, block c, split s); wave w takes the 16-token
// groups w, w + 4, ... of the split and keeps the next group's loads in
// flight while it works on one.  Per group: num^T = S_c^T p~^T (MFMA), den,
// O, dnum, dden, dp~^T = S_c dnum^T (MFMA), dq = [q > 0] (R^T dp~ + dden z_c)
// stored one group later, and p~^T dnum accumulated over the wave's tokens
// (MFMA over the LDS tile); dden p is summed per lane.  At the end the four
// waves' sums are added through LDS and written as split s's partial of
// block c.
template <int D, int ES, bool ROPE>
__global__ void __launch_bounds__(kThreads)
svla_bwd_query(const BwdArgs a)
{
    constexpr int T = D / 16;               // 16-row output tiles
    constexpr int FPL = D / 4;              // features per lane
    constexpr int LD = D + 16;              // LDS tile row (floats)
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, q = lane >> 4;
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = blockIdx.x / per_bh;
    const int rest = (int)(blockIdx.x - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const long unit = bh * a.nb + c;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    float2 *tab = (float2 *)lds;
    float *Ss = (float *)(lds + (ROPE ? a.rope.tab_bytes : 0));
    float *St = Ss + D * D;
    float *zs = St + D * D;
    float *work = zs + 64;
    float *Pt = work + wave * 2 * 16 * LD, *Dn = Pt + 16 * LD;

    const uint32_t slice = (uint32_t)a.N * D * ES;
    const auto rQ = make_rsrc((const char *)a.Q + bh * slice, slice);
    const auto rO = make_rsrc((const char *)a.dO + bh * slice, slice);
    const auto rdQ = make_rsrc((char *)a.dQ + bh * slice, slice);

    const int ngroups = (tok_hi - tok_lo + 15) / 16;
    // byte offset of the lane's features in group grp (kOOB past the split)
    auto lane_off = [&](int grp) -> uint32_t {
        const int tok = tok_lo + grp * 16 + m;
        return grp < ngroups && tok < tok_hi ? (uint32_t)(tok * D + FPL * q) * ES : kOOB;
    };
    // the first group's loads go out before the state and table are set up
    LaneRaw<D, ES> qr, orw;
    int grp = wave;
    bwd_load<D, ES>(qr, rQ, lane_off(grp));
    bwd_load<D, ES>(orw, rO, lane_off(grp));
    bwd_state_to_lds<D>(a.S_pre + unit * D * D, a.z_pre + unit * D, Ss, St, zs);
    uint32_t frame_lo = 0;
    RopePairs<FPL / 2> pp;
    if constexpr (ROPE) {
        frame_lo = fdiv((uint32_t)tok_lo, a.rope.div_hw);
        const uint32_t frame_hi = fdiv((uint32_t)(tok_hi - 1), a.rope.div_hw);
        const int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
        pp = rope_pairs<FPL / 2>(a.rope, FPL * q, nf);
    }
    __syncthreads();
    StateOps<D, SVLA_BWD_HOLD_Q> so;
    so.init(Ss, St, q, m);
    float zr[FPL];
#pragma unroll
    for (int L = 0; L < FPL; ++L) zr[L] = zs[FPL * q + L];
    // bf16 inputs at d = 32: the three products on the bf16 matrix
    // instructions with hi + lo operands (split_bf16x8).  A lane's 8
    // features are one k-group of v_mfma_f32_16x16x32_bf16 (k-slot i of lane
    // group q is feature F(q, i), in A and B alike), and the state operand of
    // tile t holds the same entries as the fp32 path's 8 steps.
    constexpr bool BF = SVLA_BWD_BF16 && ES == 2 && D == 32;
    bf16x8_t afh[BF ? T : 1], afl[BF ? T : 1], abh[BF ? T : 1], abl[BF ? T : 1];
    if constexpr (BF) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float xf[8], xb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xf[i] = so.f(t, i);
                xb[i] = so.b(t, i);
            }
            split_bf16x8(xf, afh[t], afl[t]);
            split_bf16x8(xb, abh[t], abl[t]);
        }
    }

    f32x4_t dS[T][T];
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
        for (int j = 0; j < T; ++j) dS[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float dz[FPL];
#pragma unroll
    for (int L = 0; L < FPL; ++L) dz[L] = 0.f;

    Pending<D, ES> pq;
    for (; grp < ngroups; grp += 4) {
        const uint32_t off = lane_off(grp);
        float p[FPL], dO[FPL];
        bwd_floats<D, ES>(qr, p);
        bwd_floats<D, ES>(orw, dO);
        bwd_flush<D, ES>(rdQ, pq);              // the previous group's dq
        bwd_load<D, ES>(qr, rQ, lane_off(grp + 4));
        bwd_load<D, ES>(orw, rO, lane_off(grp + 4));
        // keep those loads here, ahead of this group's work (the scheduler
        // would otherwise sink them to the end of the loop body)
        __builtin_amdgcn_sched_barrier(0);
        float denp = 0.f, pt[FPL];
#pragma unroll
        for (int L = 0; L < FPL; ++L) {
            p[L] = fmaxf(p[L], 0.f);               // p > 0 exactly where q > 0
            denp += p[L] * zr[L];
            pt[L] = p[L];
        }
        RopePos pos{0, 0, 0};
        if constexpr (ROPE) {
            pos = rope_pos((uint32_t)min(tok_lo + grp * 16 + m, tok_hi - 1), frame_lo, a.rope);
            rope_rotate<FPL / 2>(pt, pos, pp, tab);
        }
        // num^T = S^T p~^T
        f32x4_t num[T];
#pragma unroll
        for (int t = 0; t < T; ++t) num[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
            bf16x8_t bh, bl;
            split_bf16x8(pt, bh, bl);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                // (without RoPE p~ = phi(q) is a bf16 value: its lo part vanishes)
                num[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afh[t], bh, num[t], 0, 0, 0);
                if constexpr (ROPE) num[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afh[t], bl, num[t], 0, 0, 0);
                num[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afl[t], bh, num[t], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < FPL; ++st)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    num[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(so.f(t, st), pt[st], num[t], 0, 0, 0);
        }
        const float den = token_sum(denp) + a.eps;
        const float inv = den != 0.f ? 1.f / den : 0.f;
        float dotp = 0.f;
#pragma unroll
        for (int L = 0; L < FPL; ++L) dotp += dO[L] * (num[L / 4][L % 4] * inv);
        const float dden = -token_sum(dotp) * inv;
        float dn[FPL];
#pragma unroll
        for (int L = 0; L < FPL; ++L) dn[L] = dO[L] * inv;
        // dp~^T = S dnum^T
        f32x4_t dpt[T];
#pragma unroll
        for (int t = 0; t < T; ++t) dpt[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
            bf16x8_t bh, bl;
            split_bf16x8(dn, bh, bl);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                dpt[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abh[t], bh, dpt[t], 0, 0, 0);
                dpt[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abh[t], bl, dpt[t], 0, 0, 0);
                dpt[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abl[t], bh, dpt[t], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < FPL; ++st)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    dpt[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(so.b(t, st), dn[st], dpt[t], 0, 0, 0);
        }
        // the wave's token tile for p~^T dnum (4-float chunks of row r swapped
        // within their 16-float group by 4 ((r / 4) % 4): the 16 rows one
        // write instruction touches then cover all 64 banks)
        const int swm = 4 * ((m >> 2) & 3);
#pragma unroll
        for (int L = 0; L < FPL; L += 4) {
            *(f32x4_t *)(Pt + m * LD + ((FPL * q + L) ^ swm)) = (f32x4_t){pt[L], pt[L + 1], pt[L + 2], pt[L + 3]};
            *(f32x4_t *)(Dn + m * LD + ((FPL * q + L) ^ swm)) = (f32x4_t){dn[L], dn[L + 1], dn[L + 2], dn[L + 3]};
        }
        // dq = [q > 0] (R^T dp~ + dden z), held until the next group; dz += dden p
        float v[FPL];
#pragma unroll
        for (int L = 0; L < FPL; ++L) v[L] = dpt[L / 4][L % 4];
        if constexpr (ROPE) rope_rotate_t<FPL / 2>(v, pos, pp, tab);
#pragma unroll
        for (int L = 0; L < FPL; ++L) {
            v[L] = p[L] > 0.f ? v[L] + dden * zr[L] : 0.f;
            dz[L] += dden * p[L];
        }
        bwd_pack<D, ES>(pq.v, v);
        pq.off = off;
        if constexpr (BF) {
            // the group's 16 tokens as the k-slots of v_mfma_f32_16x16x16_bf16:
            // lane (m, q) holds tokens 4 st + q, st < 4, of feature 16 t + m
            float av[T][4], bv[T][4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int tt = 4 * st + q, swr = 4 * (st & 3);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    av[t][st] = Pt[tt * LD + ((16 * t + m) ^ swr)];
                    bv[t][st] = Dn[tt * LD + ((16 * t + m) ^ swr)];
                }
            }
            i16x4_t ah[T], al[T], bh[T], bl[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                split_bf16x4(av[t], ah[t], al[t]);
                split_bf16x4(bv[t], bh[t], bl[t]);
            }
#pragma unroll
            for (int i = 0; i < T; ++i)
#pragma unroll
                for (int j = 0; j < T; ++j) {
                    dS[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah[i], bh[j], dS[i][j], 0, 0, 0);
                    dS[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah[i], bl[j], dS[i][j], 0, 0, 0);
                    if constexpr (ROPE)        // (p~ unrotated is a bf16 value)
                        dS[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al[i], bh[j], dS[i][j], 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int tt = 4 * st + q, swr = 4 * (st & 3);     // the swap of row tt
                float av[T], bv[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    av[t] = Pt[tt * LD + ((16 * t + m) ^ swr)];
                    bv[t] = Dn[tt * LD + ((16 * t + m) ^ swr)];
                }
#pragma unroll
                for (int i = 0; i < T; ++i)
#pragma unroll
                    for (int j = 0; j < T; ++j)
                        dS[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], dS[i][j], 0, 0, 0);
            }
        }
    }
    bwd_flush<D, ES>(rdQ, pq);
    // this split's partials: the four waves' p~^T dnum tiles, then dden p
    __syncthreads();
    float *red = work;
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
        for (int j = 0; j < T; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((wave * T * T + i * T + j) * 4 + r) * 64 + lane] = dS[i][j][r];
    __syncthreads();
    const auto rS = make_rsrc(a.dS_part + (unit * a.splits + s) * D * D, D * D * 4);
    for (int e = tid * 4; e < D * D; e += kThreads * 4) {
        const int k = e / D, j0 = e % D;
        const int tile = (k / 16) * T + j0 / 16;
        const int r = k % 4, qq = (k % 16) / 4;
        u32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ln = (j0 + i) % 16 + 16 * qq;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) v += red[((w * T * T + tile) * 4 + r) * 64 + ln];
            o[i] = as_u32(v);
        }
        store16(rS, (uint32_t)e * 4u, o);
    }
    __syncthreads();
#pragma unroll
    for (int L = 0; L < FPL; ++L) red[(wave * 64 + lane) * FPL + L] = dz[L];
    __syncthreads();
    // feature f = FPL qq + L sits in register L of the lanes of group qq;
    // 256 / D threads per feature each add a share of the 4 x 16 lanes, then one adds those
    float *red2 = red + 4 * 64 * FPL;
    {
        constexpr int PARTS = kThreads / D;
        const int f = tid % D, part = tid / D;
        const int qq = f / FPL, L = f % FPL;
        float v = 0.f;
        for (int i = part; i < 64; i += PARTS) {
            const int w = i / 16, ln = i % 16 + 16 * qq;
            v += red[(w * 64 + ln) * FPL + L];
        }
        red2[part * D + f] = v;
    }
    __syncthreads();
    if (tid < D) {
        float v = 0.f;
        for (int part = 0; part < kThreads / D; ++part) v += red2[part * D + tid];
        a.dz_part[(unit * a.splits + s) * D + tid] = v;
    }
}

// Reverse scan over blocks: G_c = (sum of block c's split partials) +
// g_{c+1} G_{c+1} (H likewise), from the last block back; dS0 = g_0 G_0,
// dz0 = g_0 H_0.  Each thread owns 4 consecutive entries of [S | z] of one
// (bh) and walks the blocks in chunks of 4, all loads of a chunk issued
// before any is added.  With no tokens (splits = 0) every G, H is zero.
template <int D>
__global__ void __launch_bounds__(kThreads)
svla_bwd_scan(const BwdArgs a)
{
    constexpr int E4 = (D * D + D) / 4;
    constexpr int TILES = (E4 + kThreads - 1) / kThreads;
    constexpr int MS = 4;                    // split partials per block at most
    const long bh = blockIdx.x / TILES;
    const int idx = (int)(blockIdx.x % TILES) * kThreads + threadIdx.x;
    if (a.splits == 0 && a.dg && blockIdx.x % TILES == 0) {
        // no tokens: no key-side kernel forms the gate gradient, which is zero
        for (int c = threadIdx.x; c < a.nb; c += kThreads) a.dg[bh * a.nb + c] = 0.f;
    }
    if (idx >= E4) return;
    const int e = idx * 4;
    const bool isz = e >= D * D;
    const int off = isz ? e - D * D : e;
    const int stride = isz ? D : D * D;
    const float *part = (isz ? a.dz_part : a.dS_part) + bh * (long)a.nb * a.splits * stride + off;
    float *out = (isz ? a.Hz : a.G) + bh * (long)a.nb * stride + off;
    const float *g = a.g ? a.g + bh * a.nb : nullptr;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int sp = a.splits;
    for (int c0 = a.nb - 1; c0 >= 0; c0 -= 4) {
        f32x4_t L[4][MS];
        if (sp > 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = max(c0 - j, 0);
#pragma unroll
                for (int q = 0; q < MS; ++q)
                    L[j][q] = *(const f32x4_t *)(part + ((long)c * sp + min(q, sp - 1)) * stride);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = c0 - j;
            if (c < 0) break;
            const float gn = c + 1 < a.nb ? (g ? g[c + 1] : 1.f) : 0.f;
            acc *= gn;
#pragma unroll
            for (int q = 0; q < MS; ++q)
                if (q < sp) acc += L[j][q];
            *(f32x4_t *)(out + (long)c * stride) = acc;
        }
    }
    const float g0 = g ? g[0] : 1.f;
    float *d0 = isz ? a.dz0 : a.dS0;
    if (d0 && a.nb > 0) *(f32x4_t *)(d0 + bh * (long)stride + off) = g0 * acc;
}

// Key side.  Workgroup = (bh, block c, split s): G_c, H_c in LDS; per
// 16-token group dv^T = G^T a~^T and da~^T = G v^T (MFMA), dk = [k > 0]
// (R^T da~ + H), stored one group later.  Split 0 also forms
// dg_c = <G_c, S_{c-1}> + <H_c, z_{c-1}>.
template <int D, int ES, bool ROPE>
__global__ void __launch_bounds__(kThreads)
svla_bwd_key(const BwdArgs a)
{
    constexpr int T = D / 16;
    constexpr int FPL = D / 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, q = lane >> 4;
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = blockIdx.x / per_bh;
    const int rest = (int)(blockIdx.x - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const long unit = bh * a.nb + c;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    float2 *tab = (float2 *)lds;
    float *Gs = (float *)(lds + (ROPE ? a.rope.tab_bytes : 0));
    float *Gt = Gs + D * D;
    float *hs = Gt + D * D;
    float *red = hs + 64;

    const uint32_t slice = (uint32_t)a.N * D * ES;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);
    const auto rdK = make_rsrc((char *)a.dK + bh * slice, slice);
    const auto rdV = make_rsrc((char *)a.dV + bh * slice, slice);

    const int ngroups = (tok_hi - tok_lo + 15) / 16;
    auto lane_off = [&](int grp) -> uint32_t {
        const int tok = tok_lo + grp * 16 + m;
        return grp < ngroups && tok < tok_hi ? (uint32_t)(tok * D + FPL * q) * ES : kOOB;
    };
    LaneRaw<D, ES> kr, vr;
    int grp = wave;
    bwd_load<D, ES>(kr, rK, lane_off(grp));
    bwd_load<D, ES>(vr, rV, lane_off(grp));
    bwd_state_to_lds<D>(a.G + unit * D * D, a.Hz + unit * D, Gs, Gt, hs);
    uint32_t frame_lo = 0;
    RopePairs<FPL / 2> pp;
    if constexpr (ROPE) {
        frame_lo = fdiv((uint32_t)tok_lo, a.rope.div_hw);
        const uint32_t frame_hi = fdiv((uint32_t)(tok_hi - 1), a.rope.div_hw);
        const int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
        pp = rope_pairs<FPL / 2>(a.rope, FPL * q, nf);
    }
    __syncthreads();
    if (s == 0 && a.dg) {
        // dg_c: the state before block c is S_{c-1}, S0 for block 0 (zero without it)
        const float *Sp = c > 0 ? a.S_pre + (unit - 1) * D * D : a.S0 ? a.S0 + bh * D * D : nullptr;
        const float *zp = c > 0 ? a.z_pre + (unit - 1) * D : a.z0 ? a.z0 + bh * D : nullptr;
        float v = 0.f;
        if (Sp) {
            for (int e = tid; e < D * D; e += kThreads) v += Gs[e] * Sp[e];
            if (tid < D) v += hs[tid] * zp[tid];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
        if (lane == 0) red[wave] = v;
        __syncthreads();
        if (tid == 0) a.dg[unit] = red[0] + red[1] + red[2] + red[3];
    }
    // G's operands: dv^T = G^T a~^T reads G[F(q, s)][pi(t, m)] (the forward
    // form), da~^T = G v^T reads G[pi(t, m)][F(q, s)] (the transposed form)
    StateOps<D, true> go;
    go.init(Gs, Gt, q, m);
    float hr[FPL];
#pragma unroll
    for (int L = 0; L < FPL; ++L) hr[L] = hs[FPL * q + L];
    // bf16 inputs at d = 32: both products on v_mfma_f32_16x16x32_bf16 with G
    // as bf16 hi + lo (as on the query side); v, and a~ without RoPE, are
    // bf16 values, so their lo parts vanish and two products suffice
    constexpr bool BF = SVLA_BWD_BF16 && ES == 2 && D == 32;
    bf16x8_t gfh[BF ? T : 1], gfl[BF ? T : 1], gbh[BF ? T : 1], gbl[BF ? T : 1];
    if constexpr (BF) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float xf[8], xb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xf[i] = go.f(t, i);
                xb[i] = go.b(t, i);
            }
            split_bf16x8(xf, gfh[t], gfl[t]);
            split_bf16x8(xb, gbh[t], gbl[t]);
        }
    }

    Pending<D, ES> pv, pk;
    for (; grp < ngroups; grp += 4) {
        const uint32_t off = lane_off(grp);
        float at[FPL], v[FPL];
        bwd_floats<D, ES>(kr, at);
        bwd_floats<D, ES>(vr, v);
        bwd_flush<D, ES>(rdV, pv);             // the previous group's dv, dk
        bwd_flush<D, ES>(rdK, pk);
        bwd_load<D, ES>(kr, rK, lane_off(grp + 4));
        bwd_load<D, ES>(vr, rV, lane_off(grp + 4));
        __builtin_amdgcn_sched_barrier(0);     // those loads stay ahead of this group's work
        unsigned live = 0u;                    // bit L: k > 0 (the ReLU's mask)
#pragma unroll
        for (int L = 0; L < FPL; ++L) {
            live |= (at[L] > 0.f ? 1u : 0u) << L;
            at[L] = fmaxf(at[L], 0.f);
        }
        RopePos pos{0, 0, 0};
        if constexpr (ROPE) {
            pos = rope_pos((uint32_t)min(tok_lo + grp * 16 + m, tok_hi - 1), frame_lo, a.rope);
            rope_rotate<FPL / 2>(at, pos, pp, tab);
        }
        f32x4_t dv[T], da[T];
#pragma unroll
        for (int t = 0; t < T; ++t) dv[t] = da[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
            bf16x8_t ah, al, vh, vl;
            split_bf16x8(at, ah, al);
            split_bf16x8(v, vh, vl);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gfh[t], ah, dv[t], 0, 0, 0);
                if constexpr (ROPE) dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gfh[t], al, dv[t], 0, 0, 0);
                dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gfl[t], ah, dv[t], 0, 0, 0);
                da[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gbh[t], vh, da[t], 0, 0, 0);
                da[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gbl[t], vh, da[t], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int st = 0; st < FPL; ++st)
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    dv[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(go.f(t, st), at[st], dv[t], 0, 0, 0);
                    da[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(go.b(t, st), v[st], da[t], 0, 0, 0);
                }
        }
        float x[FPL], y[FPL];
#pragma unroll
        for (int L = 0; L < FPL; ++L) {
            x[L] = dv[L / 4][L % 4];
            y[L] = da[L / 4][L % 4];
        }
        if constexpr (ROPE) rope_rotate_t<FPL / 2>(y, pos, pp, tab);
#pragma unroll
        for (int L = 0; L < FPL; ++L) y[L] = (live >> L) & 1u ? y[L] + hr[L] : 0.f;
        bwd_pack<D, ES>(pv.v, x);
        bwd_pack<D, ES>(pk.v, y);
        pv.off = pk.off = off;
    }
    bwd_flush<D, ES>(rdV, pv);
    bwd_flush<D, ES>(rdK, pk);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local char g_err[512] = "";
thread_local void *const *t_events = nullptr;   // svla_set_timing_events
thread_local int t_nev = 0;

enum Slot {
    SLOT_BUILD = 0, SLOT_SCAN = 1, SLOT_APPLY = 2, SLOT_STEP = 3, SLOT_CONV = 4,
    SLOT_BWD_QUERY = 5, SLOT_BWD_SCAN = 6, SLOT_BWD_KEY = 7
};
constexpr int kSlots = 8;

// Every kernel goes through here.  With timing events set, the launch
// carries a start/stop event pair that the runtime records around the
// kernel's own execution.
// svla_describe: while set, launch() records what it would launch instead.
struct LaunchDesc {
    char name[kSlots][96];
    unsigned grid[kSlots], block[kSlots];
    size_t lds[kSlots];
    bool used[kSlots];
};
thread_local LaunchDesc *t_desc = nullptr;

template <typename Arg>
void launch(void (*kernel)(Arg), unsigned grid, size_t lds, hipStream_t s, Slot slot, const Arg &a,
            const char *name, unsigned threads = kThreads)
{
    if (t_desc) {
        snprintf(t_desc->name[slot], sizeof t_desc->name[slot], "%s", name);
        t_desc->grid[slot] = grid;
        t_desc->block[slot] = threads;
        t_desc->lds[slot] = lds;
        t_desc->used[slot] = true;
        return;
    }
    const int e = 2 * (int)slot;
    if (t_events && e + 1 < t_nev)
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), (uint32_t)lds, s,
                              (hipEvent_t)t_events[e], (hipEvent_t)t_events[e + 1], 0, a);
    else
        kernel<<<dim3(grid), dim3(threads), lds, s>>>(a);
}

svla_status fail(svla_status s, const char *fn, const char *fmt, ...) __attribute__((format(printf, 3, 4)));
svla_status fail(svla_status s, const char *fn, const char *fmt, ...)
{
    char msg[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    snprintf(g_err, sizeof g_err, "%s: %s", fn, msg);
    return s;
}

FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.div = d;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;                  // l = ceil(log2 d)
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.s1 = l ? 1 : 0;
    f.s2 = l ? l - 1 : 0;
    return f;
}

struct Plan {
    int B, H, nb, n, d;
    long BH;
    int esize;                 // bytes per Q/K/V/O element
    bool dma;                  // build straight to LDS (bf16 without RoPE)
    bool fold;                 // one block, bf16, d = 32: the apply sums the partials (no scan)
    int splits, chunk;         // build: workgroups per block, tokens per workgroup
    int tile, tiles;           // apply
    int oesize;                // bytes per O element and per packed state operand element
    size_t lds_build, lds_apply;
    size_t off_spart, off_zpart, off_sop, off_zpre, total;
    RopeK rope;
    // one-launch block step (svla_step_fused), taken when the new state does
    // not overlap the carried one
    bool fused;
    int ftiles, ftile;         // workgroups per bh, tokens per workgroup
    int fwork, ftab;           // LDS bytes: stage slots / epilogue, RoPE table
    size_t lds_fused;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// RoPE build (svla_state_build_rope): stages in flight per wave and 16-byte
// loads per lane per tensor per stage (at least one 16-token group per stage:
// a wave load covers 64 / (d / 8) rows, 8 rows for the 64-feature rows and
// half-rows of d >= 64)
constexpr int rope_pf() { return SVLA_ROPE_PF; }
constexpr int rope_u(int d) { return d == 32 || SVLA_ROPE_U >= 2 ? SVLA_ROPE_U : 2; }
constexpr int rope_tokens(int d) { return rope_u(d) * 64 / ((d == 128 ? 64 : d) / 8); }

// Splits of a block's tokens over workgroups: about `target` workgroups per
// launch, but never fewer than min_per_d * d tokens per split, so the fp32
// partial state (4 d^2 bytes) stays a small fraction of the K/V bytes it
// summarises (1/8 at the default).  The d = 128 build without RoPE takes
// min_per_d = 1: with many blocks the target binds first (three splits per
// block at 20 heads x 8 blocks), and a call with few blocks (a block step of
// 20 heads) is bound by how many workgroups stream its K and V, not by the
// partials' bytes (measured: 23.1 -> 13.6 us for the 1760-token gated step).
// Measured: the build without RoPE runs best with one or two long-lived
// workgroups per CU, the RoPE build with many.
int pick_splits(long units, int n, int d, long target, int *chunk_out,
                int min_per_d = SVLA_MIN_SPLIT_PER_D)
{
    constexpr int G = 64;   // chunk granularity; independent of the stage size
    if (n <= 0 || units <= 0) { *chunk_out = G; return 0; }
    long want = (target + units - 1) / units;
    long cap = n / (min_per_d * d);
    if (cap < 1) cap = 1;
    long s = want < cap ? want : cap;
    if (s < 1) s = 1;
    int chunk = (int)((n + s - 1) / s);
    chunk = (chunk + G - 1) / G * G;
    *chunk_out = chunk;
    return (n + chunk - 1) / chunk;
}

int frames_spanned_max(int tokens, int hw) { return tokens <= 0 ? 1 : (tokens - 1) / hw + 2; }

svla_status check_rope(const char *fn, const svla_rope *r, int d, RopeK *out)
{
    memset(out, 0, sizeof *out);
    if (!r) return SVLA_OK;
    if (r->dt_dims < 0 || r->dh_dims < 0 || r->dw_dims < 0 || (r->dt_dims & 1) ||
        (r->dh_dims & 1) || (r->dw_dims & 1))
        return fail(SVLA_ERR_VALUE, fn, "rope dims must be even and >= 0 (got %d/%d/%d)",
                    r->dt_dims, r->dh_dims, r->dw_dims);
    if (r->dt_dims + r->dh_dims + r->dw_dims > d)
        return fail(SVLA_ERR_VALUE, fn, "rope dims %d+%d+%d exceed d=%d", r->dt_dims,
                    r->dh_dims, r->dw_dims, d);
    if (r->grid_h < 1 || r->grid_w < 1 || (long)r->grid_h * r->grid_w > (1L << 30))
        return fail(SVLA_ERR_VALUE, fn, "rope grid %dx%d invalid", r->grid_h, r->grid_w);
    if (r->t0 < 0) return fail(SVLA_ERR_VALUE, fn, "rope t0 must be >= 0 (got %d)", r->t0);
    if (!(r->base > 0.f) || !isfinite(r->base))
        return fail(SVLA_ERR_VALUE, fn, "rope base must be finite and > 0");
    out->on = 1;
    out->dt = r->dt_dims; out->dh = r->dh_dims; out->dw = r->dw_dims;
    out->gh = r->grid_h; out->gw = r->grid_w; out->t0 = r->t0; out->base = r->base;
    out->div_hw = make_fastdiv((uint32_t)(r->grid_h * r->grid_w));
    out->div_w = make_fastdiv((uint32_t)r->grid_w);
    const int widths[3] = {r->dt_dims, r->dh_dims, r->dw_dims};
    for (int ax = 0; ax < 3; ++ax) {
        out->freq0[ax] = 0.5 / M_PI;
        out->ratio[ax] = widths[ax] > 0 ? pow((double)r->base, -2.0 / widths[ax]) : 1.0;
    }
    return SVLA_OK;
}

svla_status check_sizes(const char *fn, svla_dtype dt, int B, int H, int nb, int n, int d)
{
    if (dt != SVLA_F32 && dt != SVLA_BF16 && dt != SVLA_FP8)
        return fail(SVLA_ERR_DTYPE, fn, "dtype %d is not SVLA_F32, SVLA_BF16 or SVLA_FP8", (int)dt);
    if (B < 0 || H < 0 || nb < 0 || n < 0)
        return fail(SVLA_ERR_SHAPE, fn, "negative size (B=%d H=%d nb=%d n=%d)", B, H, nb, n);
    if (d != 32 && d != 64 && d != 128)
        return fail(SVLA_ERR_UNSUPPORTED, fn, "d=%d not in {32, 64, 128}", d);
    if (dt == SVLA_FP8 && d != 32)
        return fail(SVLA_ERR_UNSUPPORTED, fn, "fp8 inputs are supported at d = 32 only (got d=%d)", d);
    const int es = dt == SVLA_F32 ? 4 : 2;          // the larger of the input and output element
    if ((long long)nb * n * d * es >= (1LL << 31))
        return fail(SVLA_ERR_SHAPE, fn, "one (b,h) slice of %lld tokens x d=%d exceeds 2 GiB",
                    (long long)nb * n, d);
    if ((long long)B * H * nb >= (1LL << 31) / 64)
        return fail(SVLA_ERR_SHAPE, fn, "B*H*nb=%lld too large", (long long)B * H * nb);
    return SVLA_OK;
}

svla_status make_plan(const char *fn, svla_op op, svla_dtype dt, int B, int H, int nb, int n,
                      int d, const svla_rope *rope, Plan *p)
{
    svla_status st = check_sizes(fn, dt, B, H, nb, n, d);
    if (st) return st;
    memset(p, 0, sizeof *p);
    p->B = B; p->H = H; p->nb = nb; p->n = n; p->d = d;
    p->BH = (long)B * H;
    p->esize = dt == SVLA_BF16 ? 2 : dt == SVLA_FP8 ? 1 : 4;
    p->oesize = dt == SVLA_F32 ? 4 : 2;               // fp8 inputs give a bf16 output
    st = check_rope(fn, rope, d, &p->rope);
    if (st) return st;
    p->dma = p->esize == 2 && !p->rope.on;
    const long units = p->BH * nb;
    int chunk_dma = 0, chunk_other = 0;
    const int splits_dma = pick_splits(units, n, d, SVLA_DMA_WGS, &chunk_dma,
                                       d == 128 ? SVLA_MIN_SPLIT_128 : SVLA_MIN_SPLIT_PER_D);
    // (the RoPE builds take shorter splits; the workspace holds either plan's
    // partials, since its size must not depend on RoPE)
    int chunk_rope = 0;
    const int splits_plain = pick_splits(units, n, d, SVLA_ROPE_WGS, &chunk_other);
    const int splits_rope = pick_splits(units, n, d, SVLA_ROPE_WGS, &chunk_rope, SVLA_MIN_SPLIT_ROPE);
    // fp8 without RoPE (the register build): fewer, longer splits, so a
    // one-block call's partials fit the read-out that sums them
    int chunk_f8 = 0;
    const int splits_f8 = pick_splits(units, n, d, SVLA_F8_WGS, &chunk_f8);
    const bool f8plain = p->esize == 1 && !p->rope.on;
    const int splits_other = p->rope.on ? splits_rope : f8plain ? splits_f8 : splits_plain;
    if (p->rope.on) chunk_other = chunk_rope;
    if (f8plain) chunk_other = chunk_f8;
    if (op == SVLA_OP_STATE_BUILD) {
        // one workgroup per block: its partial is the block's local state
        p->splits = n > 0 ? 1 : 0;
        p->chunk = n > 0 ? n : 1;
    } else {
        p->splits = p->dma ? splits_dma : splits_other;
        p->chunk = p->dma ? chunk_dma : chunk_other;
    }
    p->fold = (op == SVLA_OP_NONCAUSAL || op == SVLA_OP_BLOCK_CAUSAL || op == SVLA_OP_BLOCK_STEP) &&
              p->esize <= 2 && d == 32 && nb == 1 && n > 0 &&
              p->splits + 1 <= (p->rope.on ? kFoldMaxPartsRope : kFoldMaxParts);
    // the one-launch step: one block of bf16 or fp8 at d = 32, short enough for every
    // workgroup of a (b,h) to build the whole block state itself
    // (with RoPE: axis widths that are multiples of 4, so each 4-feature group
    // of the step's table reads lies on one axis)
    p->fused = (op == SVLA_OP_NONCAUSAL || op == SVLA_OP_BLOCK_CAUSAL || op == SVLA_OP_BLOCK_STEP) &&
               p->esize <= 2 && d == 32 && nb == 1 && n > 0 && n <= SVLA_FUSED_MAX_N && p->BH > 0 &&
               (!p->rope.on || (p->rope.dt % 4 == 0 && p->rope.dh % 4 == 0 && p->rope.dw % 4 == 0));
    if (p->fused) {
        // at most one workgroup per CU: (a second round of workgroups would
        // repeat the whole build); at least one per (b,h)
        const int ngr = (n + 15) / 16;                       // 16-token groups
        long T = SVLA_FUSED_WGS / p->BH;
        if (T > ngr) T = ngr;
        if (T < 1) T = 1;
        const int maxg = SVLA_FUSED_W * SVLA_FUSED_QG;        // groups one workgroup reads out
        if ((ngr + T - 1) / T > maxg) T = (ngr + maxg - 1) / maxg;
        const int gpt = (int)((ngr + T - 1) / T);
        p->ftile = 16 * gpt;
        p->ftiles = (ngr + gpt - 1) / gpt;
        p->fwork = fused_work_bytes(p->rope.on, SVLA_FUSED_W);
        p->ftab = 0;
        if (p->rope.on) {
            // frames of every row of the padded 16-token stages, two identity entries
            const long nf = (16L * ngr - 1) / ((long)p->rope.gh * p->rope.gw) + 1;
            const long e = nf * (p->rope.dt / 2) + (long)p->rope.gh * (p->rope.dh / 2) +
                           (long)p->rope.gw * (p->rope.dw / 2) + 2;
            if (e > kMaxRopeEntries) p->fused = false;          // (the split build takes it)
            p->ftab = (int)((e * 8 + 255) & ~255L);
        }
        p->lds_fused = (size_t)p->ftab + p->fwork;
    }
    p->tile = (p->esize == 2 && d >= 64) ? SVLA_APPLY_TILE_LDS
              : d == 128 ? SVLA_APPLY_TILE128
              : p->rope.on ? (p->fold ? SVLA_APPLY_TILE_FOLD_ROPE : SVLA_APPLY_TILE_ROPE)
              : p->fold ? SVLA_APPLY_TILE_FOLD : SVLA_APPLY_TILE32;
    p->tiles = n > 0 ? (n + p->tile - 1) / p->tile : 0;

    // dynamic LDS: [RoPE table][stage buffers | epilogue] (the direct-to-LDS
    // build has static LDS only)
    if (p->esize <= 2) {
        const int td = d == 128 ? 64 : d;                 // tile side (quadrants for d = 128)
        const size_t slots = (size_t)4 * 3 * rope_tokens(d) * td * 2;
        // (the register build's d = 32 epilogue sums the four wave tiles in one
        // pass; at d >= 64 it sums them pass by pass)
        const size_t epi = td == 32 ? ((size_t)4 * td * td + 4 * td) * 4
                                    : ((size_t)td * td + td + 2048) * 4;
        p->lds_build = p->dma ? 0 : (slots > epi ? slots : epi);
    } else {
        const size_t stage = (size_t)2 * 2 * 4096;
        const size_t epi = (d == 32 ? 16384 : 0) + 8192;
        p->lds_build = stage > epi ? stage : epi;
    }
    p->lds_apply = 0;
    if (p->rope.on) {
        const int hw = p->rope.gh * p->rope.gw;
        const long eb = (long)frames_spanned_max(p->chunk, hw) * (p->rope.dt / 2) +
                        (long)p->rope.gh * (p->rope.dh / 2) + (long)p->rope.gw * (p->rope.dw / 2);
        const long ea = (long)frames_spanned_max(p->tile, hw) * (p->rope.dt / 2) +
                        (long)p->rope.gh * (p->rope.dh / 2) + (long)p->rope.gw * (p->rope.dw / 2);
        if (eb >= kMaxRopeEntries || ea >= kMaxRopeEntries)
            return fail(SVLA_ERR_UNSUPPORTED, fn,
                        "RoPE table of %ld entries exceeds %d (grid %dx%d too large)",
                        eb > ea ? eb : ea, kMaxRopeEntries, p->rope.gh, p->rope.gw);
        // the table takes only what the largest range of this call needs
        // (build and apply share it: the larger of the two)
        const long e = (eb > ea ? eb : ea) + 1;   // + the identity entry
        p->rope.tab_bytes = (int)((e * 8 + 255) & ~255L);
        p->lds_build += (size_t)p->rope.tab_bytes;
        p->lds_apply = (size_t)p->rope.tab_bytes;
    }
    if (p->fold) p->lds_apply += (size_t)(d * d + d) * 4;   // the summed state

    // workspace: partial states (as many per block as either build writes,
    // so the size does not depend on RoPE), packed prefix operands, prefix z
    size_t off = 0;
    const bool fused = op == SVLA_OP_NONCAUSAL || op == SVLA_OP_BLOCK_CAUSAL || op == SVLA_OP_BLOCK_STEP;
    if (fused) {
        // (+ 1: a one-block call whose scan is folded into the apply keeps
        // the carried state there)
        int most = splits_dma > splits_plain ? splits_dma : splits_plain;
        if (splits_rope > most) most = splits_rope;
        if (splits_f8 > most) most = splits_f8;
        const size_t slots = (size_t)most + 1;
        p->off_spart = off; off = align256(off + (size_t)units * slots * d * d * 4);
        p->off_zpart = off; off = align256(off + (size_t)units * slots * d * 4);
    }
    if (fused || op == SVLA_OP_APPLY) {
        p->off_sop = off; off = align256(off + (size_t)units * d * d * p->oesize);
    }
    if (fused) {
        p->off_zpre = off; off = align256(off + (size_t)units * d * 4);
    }
    p->total = off;
    return SVLA_OK;
}

inline bool misaligned(const void *ptr) { return ((uintptr_t)ptr & 15) != 0; }

// ---- launchers ---------------------------------------------------------------

template <int D>
void launch_build(const Plan &p, const BuildArgs &args, hipStream_t s)
{
    BuildArgs a = args;
    a.splits = p.splits;
    a.chunk = p.chunk;
    a.slots = p.splits + (a.S_in ? 1 : 0);
    const unsigned grid = (unsigned)(p.BH * p.nb * p.splits);
    const unsigned qgrid = (unsigned)((grid + 7) / 8 * 8 * 4);   // RoPE build at d = 128: four quadrants
    char nm[96];
    if (p.dma) {
        constexpr int U = D == 32 ? SVLA_DMA_U32 : D == 64 ? SVLA_DMA_U : SVLA_DMA_U128;
        constexpr int R = D == 32 ? SVLA_DMA_R32 : D == 64 ? SVLA_DMA_R : SVLA_DMA_R128;
        snprintf(nm, sizeof nm, "void svla_state_build_dma<%d, %d, %d>", D, U, R);
        launch(svla_state_build_dma<D, U, R>, grid, 0, s, SLOT_BUILD, a, nm);
    } else if (p.esize <= 2) {
        constexpr int PF = rope_pf(), U = rope_u(D);
        if constexpr (D == 128) {
            snprintf(nm, sizeof nm, "void svla_state_build_rope<64, 128, %d, %d, true, 2>", PF, U);
            launch(svla_state_build_rope<64, 128, PF, U>, qgrid, p.lds_build, s, SLOT_BUILD, a, nm);
        } else {
            const bool r = p.rope.on;
            snprintf(nm, sizeof nm, "void svla_state_build_rope<%d, %d, %d, %d, %s, %d>", D, D, PF, U,
                     r ? "true" : "false", p.esize);
            if constexpr (D == 32) {
                if (p.esize == 1 && r) launch(svla_state_build_rope<D, D, PF, U, true, 1>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
                else if (p.esize == 1) launch(svla_state_build_rope<D, D, PF, U, false, 1>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
                else launch(svla_state_build_rope<D, D, PF, U>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
            } else {
                launch(svla_state_build_rope<D, D, PF, U>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
            }
        }
    } else {
        snprintf(nm, sizeof nm, "void svla_state_build_f32<%d, %s>", D, p.rope.on ? "true" : "false");
        if (p.rope.on) launch(svla_state_build_f32<D, true>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
        else launch(svla_state_build_f32<D, false>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
    }
}

template <int D, int MODE>
void launch_scan_d(const Plan &p, const ScanArgs &a, hipStream_t s)
{
    const unsigned grid = (unsigned)(p.BH * (ScanShape<D>::STILES + 1));
    const bool bf = p.oesize == 2;
    char nm[96];
    if (MODE != SCAN_PACK && p.nb >= kScanLongChain) {
        snprintf(nm, sizeof nm, "void svla_state_scan_k<%d, %d, %s, 4>", D, MODE, bf ? "true" : "false");
        if (bf) launch(svla_state_scan_k<D, MODE, true, 4>, grid, 0, s, SLOT_SCAN, a, nm, 256);
        else launch(svla_state_scan_k<D, MODE, false, 4>, grid, 0, s, SLOT_SCAN, a, nm, 256);
    } else {
        snprintf(nm, sizeof nm, "void svla_state_scan_k<%d, %d, %s, 1>", D, MODE, bf ? "true" : "false");
        if (bf) launch(svla_state_scan_k<D, MODE, true, 1>, grid, 0, s, SLOT_SCAN, a, nm, 64);
        else launch(svla_state_scan_k<D, MODE, false, 1>, grid, 0, s, SLOT_SCAN, a, nm, 64);
    }
}

template <int D>
void launch_apply(const Plan &p, const ApplyArgs &args, hipStream_t s)
{
    ApplyArgs a = args;
    a.groups = p.BH * p.nb * p.tiles;
    const unsigned grid = xcd_grid(a.groups);
    char nm[96];
    snprintf(nm, sizeof nm, "void svla_apply_%s<%d, %s>", p.esize <= 2 ? "bf16" : "f32", D,
             p.rope.on ? "true" : "false");
    if (p.esize <= 2) {
        if constexpr (D >= 64) {
            constexpr int PF = SVLA_APPLY_RING_PF;
            snprintf(nm, sizeof nm, "void svla_apply_ring<%d, %s, %d>", D, p.rope.on ? "true" : "false", PF);
            if (p.rope.on) launch(svla_apply_ring<D, true, PF>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
            else launch(svla_apply_ring<D, false, PF>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
        } else {
            const bool r = p.rope.on, f = p.fold;
            snprintf(nm, sizeof nm, "void svla_apply_bf16<%d, %s, %s, %d>", D, r ? "true" : "false",
                     f ? "true" : "false", p.esize);
            if (p.esize == 2) {
                if (r && f) launch(svla_apply_bf16<D, true, true>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else if (r) launch(svla_apply_bf16<D, true, false>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else if (f) launch(svla_apply_bf16<D, false, true>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else launch(svla_apply_bf16<D, false, false>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
            } else {
                if (r && f) launch(svla_apply_bf16<D, true, true, 1>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else if (r) launch(svla_apply_bf16<D, true, false, 1>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else if (f) launch(svla_apply_bf16<D, false, true, 1>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
                else launch(svla_apply_bf16<D, false, false, 1>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
            }
        }
    } else {
        if (p.rope.on) launch(svla_apply_f32<D, true>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
        else launch(svla_apply_f32<D, false>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
    }
}

void build_any(const Plan &p, const BuildArgs &a, hipStream_t s)
{
    if (p.d == 32) launch_build<32>(p, a, s);
    else if (p.d == 64) launch_build<64>(p, a, s);
    else launch_build<128>(p, a, s);
}

template <int MODE>
void scan_any(const Plan &p, const ScanArgs &a, hipStream_t s)
{
    if (p.d == 32) launch_scan_d<32, MODE>(p, a, s);
    else if (p.d == 64) launch_scan_d<64, MODE>(p, a, s);
    else launch_scan_d<128, MODE>(p, a, s);
}

void apply_any(const Plan &p, const ApplyArgs &a, hipStream_t s)
{
    if (p.d == 32) launch_apply<32>(p, a, s);
    else if (p.d == 64) launch_apply<64>(p, a, s);
    else launch_apply<128>(p, a, s);
}

void launch_fused(const Plan &p, const StepArgs &args, hipStream_t s)
{
    StepArgs a = args;
    a.tiles = p.ftiles;
    a.tile = p.ftile;
    a.work_bytes = p.fwork;
    a.BH = p.BH;
    a.rope = p.rope;
    a.rope.tab_bytes = p.ftab;
    const unsigned grid = (unsigned)(8L * p.ftiles * ((p.BH + 7) / 8));
    constexpr int W = SVLA_FUSED_W, PF = SVLA_FUSED_PF, PFR = SVLA_FUSED_PF_ROPE, QG = SVLA_FUSED_QG;
    // a tile of at most 2 groups per wave takes the instance with 2 Q
    // registers (measured: the minute-long step is 1 % slower with 4)
    const bool q2 = QG > 2 && p.ftile <= 16 * W * 2;
    char nm[96];
    snprintf(nm, sizeof nm, "void svla_step_fused<%s, %d, %d, %d, %d>", p.rope.on ? "true" : "false", W,
             p.rope.on ? PFR : PF, q2 ? 2 : QG, p.esize);
    auto go = [&](auto k) { launch(k, grid, p.lds_fused, s, SLOT_STEP, a, nm, 64 * W); };
    if (p.esize == 2) {
        if (p.rope.on) q2 ? go(svla_step_fused<true, W, PFR, 2>) : go(svla_step_fused<true, W, PFR, QG>);
        else q2 ? go(svla_step_fused<false, W, PF, 2>) : go(svla_step_fused<false, W, PF, QG>);
    } else {
        if (p.rope.on) q2 ? go(svla_step_fused<true, W, PFR, 2, 1>) : go(svla_step_fused<true, W, PFR, QG, 1>);
        else q2 ? go(svla_step_fused<false, W, PF, 2, 1>) : go(svla_step_fused<false, W, PF, QG, 1>);
    }
}

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte (null: no).
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

svla_status check_launch(const char *fn)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SVLA_ERR_HIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
    return SVLA_OK;
}

// The fused forward shared by the non-causal call, the one-shot block-causal
// calls and the block steps: build -> scan -> apply on one stream.
svla_status forward(const char *fn, svla_op op, svla_dtype dt, int B, int H, int nb, int n,
                    int d, const void *Q, const void *K, const void *V, void *O,
                    const float *S0, const float *z0, float *S_fin, float *z_fin,
                    const float *g, const svla_rope *rope, float eps, void *ws,
                    size_t ws_bytes, svla_stream stream, bool dry = false)
{
    Plan p;
    svla_status st = make_plan(fn, op, dt, B, H, nb, n, d, rope, &p);
    if (st) return st;
    if (!(eps >= 0.f) || !isfinite(eps))
        return fail(SVLA_ERR_VALUE, fn, "eps must be finite and >= 0");
    if (p.BH == 0) return SVLA_OK;
    const bool tokens = (long)nb * n > 0;
    if (tokens && (!Q || !K || !V || !O)) return fail(SVLA_ERR_NULL, fn, "Q, K, V and O are required");
    if ((S0 == nullptr) != (z0 == nullptr)) return fail(SVLA_ERR_NULL, fn, "pass both S0 and z0, or neither");
    if ((S_fin == nullptr) != (z_fin == nullptr))
        return fail(SVLA_ERR_NULL, fn, "pass both final-state outputs, or neither");
    if (op == SVLA_OP_BLOCK_STEP && !S_fin) return fail(SVLA_ERR_NULL, fn, "S_out and z_out are required");
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) || misaligned(S0) ||
        misaligned(z0) || misaligned(S_fin) || misaligned(z_fin) || misaligned(g) || misaligned(ws))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    if (p.total > 0 && !ws) return fail(SVLA_ERR_NULL, fn, "workspace of %zu bytes required", p.total);
    if (ws_bytes < p.total)
        return fail(SVLA_ERR_WORKSPACE, fn, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, p.total);
    if (dry) return SVLA_OK;           // validation only (no HIP call made)

    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    (void)hipGetLastError();
    const size_t sb = (size_t)p.BH * d * d * 4, zb = (size_t)p.BH * d * 4;
    if (p.fused && !overlap(S0, sb, S_fin, sb) && !overlap(S0, sb, z_fin, zb) &&
        !overlap(z0, zb, S_fin, sb) && !overlap(z0, zb, z_fin, zb)) {
        StepArgs fa;
        memset(&fa, 0, sizeof fa);
        fa.Q = Q; fa.K = K; fa.V = V; fa.O = O;
        fa.S_in = S0; fa.z_in = z0; fa.g = g; fa.S_out = S_fin; fa.z_out = z_fin;
        fa.n = n; fa.eps = eps;
        launch_fused(p, fa, s);
        return check_launch(fn);
    }
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    sa.S_part = (const float *)(w + p.off_spart);
    sa.z_part = (const float *)(w + p.off_zpart);
    sa.g = g; sa.S_in = S0; sa.z_in = z0;
    sa.S_op = w + p.off_sop;
    sa.z_pre = (float *)(w + p.off_zpre);
    sa.S_fin = S_fin; sa.z_fin = z_fin;
    sa.nb = nb; sa.splits = p.splits;
    if (tokens) {
        BuildArgs ba;
        memset(&ba, 0, sizeof ba);
        ba.K = K; ba.V = V;
        ba.S_part = (float *)(w + p.off_spart);
        ba.z_part = (float *)(w + p.off_zpart);
        ba.N = nb * n; ba.n = n; ba.nb = nb; ba.splits = p.splits; ba.chunk = p.chunk;
        ba.BH = p.BH;
        ba.rope = p.rope;
        if (p.fold && S0) { ba.S_in = S0; ba.z_in = z0; ba.g = g; }
        build_any(p, ba, s);
        if ((st = check_launch(fn))) return st;
    }
    if (!p.fold) {
        scan_any<SCAN_FORWARD>(p, sa, s);
        if ((st = check_launch(fn))) return st;
    }
    if (tokens) {
        ApplyArgs aa;
        memset(&aa, 0, sizeof aa);
        aa.Q = Q; aa.O = O; aa.S_op = w + p.off_sop; aa.z_pre = (const float *)(w + p.off_zpre);
        aa.N = nb * n; aa.n = n; aa.nb = nb; aa.tile = p.tile; aa.tiles = p.tiles; aa.eps = eps;
        aa.rope = p.rope;
        if (p.fold) {
            aa.S_part = sa.S_part; aa.z_part = sa.z_part; aa.splits = p.splits + (S0 ? 1 : 0);
            aa.S_fin = S_fin; aa.z_fin = z_fin;
        }
        apply_any(p, aa, s);
        if ((st = check_launch(fn))) return st;
    }
    return SVLA_OK;
}


// ---- backward ---------------------------------------------------------------

constexpr int kBwdMaxSplits = 4;     // query/key splits per block (the reverse scan reads this many)
constexpr long kBwdWgs = SVLA_BWD_WGS;
constexpr int kBwdMinChunk = 128;    // ... but at least two 16-token groups per wave

struct BwdPlan {
    Plan fwd;                        // the forward state rebuild: state build + export scan
    int splits, chunk;               // query/key workgroups per block, tokens per workgroup
    int tab_bytes;                   // LDS of the RoPE table (query and key kernels)
    size_t lds_query, lds_key;
    size_t off_spre, off_zpre, off_dsp, off_dzp, off_G, off_H, total;
};

svla_status make_bwd_plan(const char *fn, svla_dtype dt, int B, int H, int nb, int n, int d,
                          const svla_rope *rope, BwdPlan *bp)
{
    memset(bp, 0, sizeof *bp);
    if (dt == SVLA_FP8) return fail(SVLA_ERR_UNSUPPORTED, fn, "the backward pass takes SVLA_F32 or SVLA_BF16");
    svla_status st = make_plan(fn, SVLA_OP_BLOCK_CAUSAL, dt, B, H, nb, n, d, rope, &bp->fwd);
    if (st) return st;
    if (d == 128) return fail(SVLA_ERR_UNSUPPORTED, fn, "the backward pass takes d = 32 or 64 (got 128)");
    const Plan &p = bp->fwd;
    const long units = p.BH * nb;
    if (n > 0 && units > 0) {
        long sp = (kBwdWgs + units - 1) / units;
        if (sp > kBwdMaxSplits) sp = kBwdMaxSplits;
        int chunk = (int)((n + sp - 1) / sp);
        chunk = (chunk + 31) / 32 * 32;
        if (chunk < kBwdMinChunk) chunk = kBwdMinChunk;
        bp->chunk = chunk;
        bp->splits = (n + chunk - 1) / chunk;
    }
    if (p.rope.on) {
        const long e = (long)frames_spanned_max(bp->chunk, p.rope.gh * p.rope.gw) * (p.rope.dt / 2) +
                       (long)p.rope.gh * (p.rope.dh / 2) + (long)p.rope.gw * (p.rope.dw / 2) + 1;
        if (e > kMaxRopeEntries)
            return fail(SVLA_ERR_UNSUPPORTED, fn, "RoPE table of %ld entries exceeds %d (grid %dx%d too large)",
                        e, kMaxRopeEntries, p.rope.gh, p.rope.gw);
        bp->tab_bytes = (int)((e * 8 + 255) & ~255L);
    }
    // query side: state twice, z, then the per-wave token tiles (2 x 16 rows of
    // d + 16 floats) or the end-of-workgroup reductions, whichever is larger
    const size_t tiles = (size_t)128 * (d + 16), red_s = (size_t)1024 * (d / 16) * (d / 16),
                 red_z = (size_t)64 * d + 256;
    const size_t work = tiles > red_s ? (tiles > red_z ? tiles : red_z) : (red_s > red_z ? red_s : red_z);
    bp->lds_query = (size_t)bp->tab_bytes + ((size_t)2 * d * d + 64 + work) * 4;
    bp->lds_key = (size_t)bp->tab_bytes + ((size_t)2 * d * d + 64 + 64) * 4;
    // workspace: the forward's split partials, then the rebuilt prefix states,
    // the query side's partials and the reverse scan's G, H
    size_t off = p.off_sop;
    bp->off_spre = off; off = align256(off + (size_t)units * d * d * 4);
    bp->off_zpre = off; off = align256(off + (size_t)units * d * 4);
    bp->off_dsp = off; off = align256(off + (size_t)units * kBwdMaxSplits * d * d * 4);
    bp->off_dzp = off; off = align256(off + (size_t)units * kBwdMaxSplits * d * 4);
    bp->off_G = off; off = align256(off + (size_t)units * d * d * 4);
    bp->off_H = off; off = align256(off + (size_t)units * d * 4);
    bp->total = off;
    return SVLA_OK;
}

template <int D, int ES>
void launch_bwd_d(const BwdPlan &bp, const BwdArgs &a, bool tokens, hipStream_t s)
{
    const Plan &p = bp.fwd;
    const bool r = p.rope.on;
    const unsigned grid = (unsigned)(p.BH * p.nb * bp.splits);
    char nm[96];
    if (tokens) {
        snprintf(nm, sizeof nm, "void svla_bwd_query<%d, %d, %s>", D, ES, r ? "true" : "false");
        if (r) launch(svla_bwd_query<D, ES, true>, grid, bp.lds_query, s, SLOT_BWD_QUERY, a, nm);
        else launch(svla_bwd_query<D, ES, false>, grid, bp.lds_query, s, SLOT_BWD_QUERY, a, nm);
        if (hipPeekAtLastError() != hipSuccess) return;
    }
    constexpr int E4 = (D * D + D) / 4;
    const unsigned sgrid = (unsigned)(p.BH * ((E4 + kThreads - 1) / kThreads));
    snprintf(nm, sizeof nm, "void svla_bwd_scan<%d>", D);
    launch(svla_bwd_scan<D>, sgrid, 0, s, SLOT_BWD_SCAN, a, nm);
    if (hipPeekAtLastError() != hipSuccess) return;
    if (tokens) {
        snprintf(nm, sizeof nm, "void svla_bwd_key<%d, %d, %s>", D, ES, r ? "true" : "false");
        if (r) launch(svla_bwd_key<D, ES, true>, grid, bp.lds_key, s, SLOT_BWD_KEY, a, nm);
        else launch(svla_bwd_key<D, ES, false>, grid, bp.lds_key, s, SLOT_BWD_KEY, a, nm);
    }
}

void bwd_any(const BwdPlan &bp, const BwdArgs &a, bool tokens, hipStream_t s)
{
    const int d = bp.fwd.d, es = bp.fwd.esize;
    if (d == 32 && es == 2) launch_bwd_d<32, 2>(bp, a, tokens, s);
    else if (d == 32) launch_bwd_d<32, 4>(bp, a, tokens, s);
    else if (es == 2) launch_bwd_d<64, 2>(bp, a, tokens, s);
    else launch_bwd_d<64, 4>(bp, a, tokens, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// The scratch of svla_block_step_noalloc: device memory that the library holds
// for callers that cannot allocate (one copy per GPU, from module load until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// the device address: the address comes from hipGetSymbolAddress, resolved
// once per device with that device current and kept in g_scratch_ptr.
// Every call on a GPU shares that GPU's copy and leaves its content behind;
// the block step needs nothing in it to start at zero.  Calls that overlap on
// one GPU race on it.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device of `stream` (which must be the current
// device: its copy of `scratch` is resolved with that device current).
svla_status scratch_for(const char *fn, svla_stream stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SVLA_ERR_HIP, fn, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (stream) {
        hipDevice_t sd = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sd);
        if (e != hipSuccess)
            return fail(SVLA_ERR_HIP, fn, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
        if ((int)sd != dev)
            return fail(SVLA_ERR_VALUE, fn, "the stream belongs to device %d, the current device is %d",
                        (int)sd, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SVLA_ERR_UNSUPPORTED, fn, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SVLA_ERR_HIP, fn, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SVLA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int svla_abi_version(void) { return SVLA_ABI_VERSION; }

const char *svla_status_string(svla_status s)
{
    switch (s) {
    case SVLA_OK: return "SVLA_OK";
    case SVLA_ERR_NULL: return "SVLA_ERR_NULL";
    case SVLA_ERR_SHAPE: return "SVLA_ERR_SHAPE";
    case SVLA_ERR_DTYPE: return "SVLA_ERR_DTYPE";
    case SVLA_ERR_ALIGN: return "SVLA_ERR_ALIGN";
    case SVLA_ERR_UNSUPPORTED: return "SVLA_ERR_UNSUPPORTED";
    case SVLA_ERR_WORKSPACE: return "SVLA_ERR_WORKSPACE";
    case SVLA_ERR_VALUE: return "SVLA_ERR_VALUE";
    case SVLA_ERR_HIP: return "SVLA_ERR_HIP";
    default: break;
    }
    return "SVLA_ERR_UNKNOWN";
}

const char *svla_last_error(void) { return g_err; }

svla_status svla_set_timing_events(void *const *events, int n)
{
    if (events && n < 0) return fail(SVLA_ERR_VALUE, "svla_set_timing_events", "n must be >= 0");
    t_events = (events && n > 0) ? events : nullptr;
    t_nev = t_events ? n : 0;
    return SVLA_OK;
}

svla_status svla_describe(svla_op op, svla_dtype dt, int B, int H, int nb, int n, int d,
                          const svla_rope *rope, char *buf, size_t len)
{
    const char *fn = "svla_describe";
    if (!buf || len == 0) return fail(SVLA_ERR_NULL, fn, "buf is NULL or empty");
    if (op != SVLA_OP_NONCAUSAL && op != SVLA_OP_BLOCK_CAUSAL && op != SVLA_OP_BLOCK_STEP)
        return fail(SVLA_ERR_VALUE, fn, "only the fused calls are described (op %d)", (int)op);
    Plan p;
    svla_status st = make_plan(fn, op, dt, B, H, nb, n, d, rope, &p);
    if (st) return st;
    // the plan the call takes, and (for a call that can take the one-launch
    // step) the two-kernel plan it takes when the new state overlaps the old
    LaunchDesc desc[2];
    memset(desc, 0, sizeof desc);
    BuildArgs ba;
    memset(&ba, 0, sizeof ba);
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    ApplyArgs aa;
    memset(&aa, 0, sizeof aa);
    StepArgs fa;
    memset(&fa, 0, sizeof fa);
    if (p.BH > 0) {
        t_desc = &desc[0];
        if (p.fused) launch_fused(p, fa, nullptr);
        t_desc = &desc[p.fused ? 1 : 0];
        if ((long)nb * n > 0) build_any(p, ba, nullptr);
        if (!p.fold) scan_any<SCAN_FORWARD>(p, sa, nullptr);
        if ((long)nb * n > 0) apply_any(p, aa, nullptr);
        t_desc = nullptr;
    }
    static const char *slot_name[kSlots] = {"build", "scan", "apply", "step", "conv",
                                            "bwd_query", "bwd_scan", "bwd_key"};
    int w = snprintf(buf, len, "{\"fused\": %s, \"step_tiles\": %d, \"step_tile\": %d, \"splits\": %d, "
                     "\"chunk\": %d, \"apply_tile\": %d, \"workspace\": %zu",
                     p.fused ? "true" : "false", p.fused ? p.ftiles : 0, p.fused ? p.ftile : 0,
                     p.splits, p.chunk, p.tile, p.total);
    for (int pl = 0; pl < (p.fused ? 2 : 1); ++pl) {
        if (w < 0 || (size_t)w >= len) break;
        w += snprintf(buf + w, len - w, ", \"%s\": [", pl == 0 ? "kernels" : "in_place_kernels");
        bool first = true;
        for (int k = 0; k < kSlots; ++k) {
            if (!desc[pl].used[k] || w < 0 || (size_t)w >= len) continue;
            w += snprintf(buf + w, len - w, "%s{\"slot\": \"%s\", \"name\": \"%s\", \"grid\": %u, \"block\": %u, \"lds\": %zu}",
                          first ? "" : ", ", slot_name[k], desc[pl].name[k], desc[pl].grid[k],
                          desc[pl].block[k], desc[pl].lds[k]);
            first = false;
        }
        if (w >= 0 && (size_t)w < len) w += snprintf(buf + w, len - w, "]");
    }
    if (w >= 0 && (size_t)w < len) w += snprintf(buf + w, len - w, "}");
    if (w < 0 || (size_t)w >= len) return fail(SVLA_ERR_VALUE, fn, "buffer of %zu bytes too small", len);
    return SVLA_OK;
}

svla_status svla_workspace_size(svla_op op, svla_dtype dt, int B, int H, int nb, int n, int d,
                                size_t *bytes)
{
    const char *fn = "svla_workspace_size";
    if (!bytes) return fail(SVLA_ERR_NULL, fn, "bytes is NULL");
    if ((int)op < SVLA_OP_NONCAUSAL || (int)op > SVLA_OP_BACKWARD)
        return fail(SVLA_ERR_VALUE, fn, "unknown op %d", (int)op);
    if (op == SVLA_OP_BACKWARD) {
        BwdPlan bp;
        svla_status st = make_bwd_plan(fn, dt, B, H, nb, n, d, nullptr, &bp);
        if (st) return st;
        *bytes = bp.total;
        return SVLA_OK;
    }
    Plan p;
    svla_status st = make_plan(fn, op, dt, B, H, nb, n, d, nullptr, &p);
    if (st) return st;
    *bytes = p.total;
    return SVLA_OK;
}

svla_status svla_noncausal(svla_dtype dt, int B, int H, int N, int d, const void *Q,
                           const void *K, const void *V, void *O, float eps, float *S_out,
                           float *z_out, void *ws, size_t ws_bytes, svla_stream stream)
{
    return forward("svla_noncausal", SVLA_OP_NONCAUSAL, dt, B, H, 1, N, d, Q, K, V, O, nullptr,
                   nullptr, S_out, z_out, nullptr, nullptr, eps, ws, ws_bytes, stream);
}

svla_status svla_block_causal(svla_dtype dt, int B, int H, int nb, int n, int d, const void *Q,
                              const void *K, const void *V, void *O, const float *S0,
                              const float *z0, float *S_final, float *z_final,
                              const svla_rope *rope, float eps, void *ws, size_t ws_bytes,
                              svla_stream stream)
{
    return forward("svla_block_causal", SVLA_OP_BLOCK_CAUSAL, dt, B, H, nb, n, d, Q, K, V, O, S0,
                   z0, S_final, z_final, nullptr, rope, eps, ws, ws_bytes, stream);
}

svla_status svla_block_causal_gated(svla_dtype dt, int B, int H, int nb, int n, int d,
                                    const void *Q, const void *K, const void *V, void *O,
                                    const float *S0, const float *z0, float *S_final,
                                    float *z_final, const float *g, const svla_rope *rope,
                                    float eps, void *ws, size_t ws_bytes, svla_stream stream)
{
    const char *fn = "svla_block_causal_gated";
    if (!g && (long)B * H * nb > 0) return fail(SVLA_ERR_NULL, fn, "g is required");
    return forward(fn, SVLA_OP_BLOCK_CAUSAL, dt, B, H, nb, n, d, Q, K, V, O, S0, z0, S_final,
                   z_final, g, rope, eps, ws, ws_bytes, stream);
}

svla_status svla_block_step(svla_dtype dt, int B, int H, int n, int d, const void *Q,
                            const void *K, const void *V, void *O, const float *S_in,
                            const float *z_in, float *S_out, float *z_out,
                            const svla_rope *rope, float eps, void *ws, size_t ws_bytes,
                            svla_stream stream)
{
    return forward("svla_block_step", SVLA_OP_BLOCK_STEP, dt, B, H, 1, n, d, Q, K, V, O, S_in,
                   z_in, S_out, z_out, nullptr, rope, eps, ws, ws_bytes, stream);
}

svla_status svla_block_step_gated(svla_dtype dt, int B, int H, int n, int d, const void *Q,
                                  const void *K, const void *V, void *O, const float *S_in,
                                  const float *z_in, float *S_out, float *z_out,
                                  const float *g, const svla_rope *rope, float eps, void *ws,
                                  size_t ws_bytes, svla_stream stream)
{
    const char *fn = "svla_block_step_gated";
    if (!g && (long)B * H > 0) return fail(SVLA_ERR_NULL, fn, "g is required");
    return forward(fn, SVLA_OP_BLOCK_STEP, dt, B, H, 1, n, d, Q, K, V, O, S_in, z_in, S_out,
                   z_out, g, rope, eps, ws, ws_bytes, stream);
}

svla_status svla_block_step_noalloc(svla_dtype dt, int B, int H, int n, int d, const void *Q,
                                    const void *K, const void *V, void *O, const float *S_in,
                                    const float *z_in, float *S_out, float *z_out,
                                    const float *g, const svla_rope *rope, float eps,
                                    svla_stream stream)
{
    const char *fn = "svla_block_step_noalloc";
    Plan p;
    svla_status st = make_plan(fn, SVLA_OP_BLOCK_STEP, dt, B, H, 1, n, d, rope, &p);
    if (st) return st;
    if (p.total > kScratchBytes)
        return fail(SVLA_ERR_WORKSPACE, fn, "this step needs %zu bytes of scratch; the library holds %zu "
                    "per device", p.total, kScratchBytes);
    // every check of the call first (an aligned stand-in for the scratch
    // address, which is only checked, never used), then the first HIP call
    void *const stand_in = (void *)(uintptr_t)256;
    st = forward(fn, SVLA_OP_BLOCK_STEP, dt, B, H, 1, n, d, Q, K, V, O, S_in, z_in, S_out, z_out, g,
                 rope, eps, stand_in, kScratchBytes, stream, true);
    if (st || p.BH == 0) return st;
    void *ws = nullptr;
    if ((st = scratch_for(fn, stream, &ws))) return st;
    return forward(fn, SVLA_OP_BLOCK_STEP, dt, B, H, 1, n, d, Q, K, V, O, S_in, z_in, S_out, z_out, g,
                   rope, eps, ws, kScratchBytes, stream);
}

svla_status svla_temporal_conv(svla_dtype dt, int B, int nb, int F, int P, int C, const void *X,
                               void *Y, const float *w, const float *bias, const void *cache_in,
                               void *cache_out, svla_stream stream)
{
    const char *fn = "svla_temporal_conv";
    if (dt != SVLA_F32 && dt != SVLA_BF16)
        return fail(SVLA_ERR_DTYPE, fn, "dtype %d is not SVLA_F32 or SVLA_BF16", (int)dt);
    if (B < 0 || nb < 0 || F < 1 || P < 0 || C < 0)
        return fail(SVLA_ERR_SHAPE, fn, "bad size (B=%d nb=%d F=%d P=%d C=%d; F >= 1)", B, nb, F, P, C);
    if (C % 8) return fail(SVLA_ERR_UNSUPPORTED, fn, "C=%d is not a multiple of 8", C);
    const long long es = dt == SVLA_BF16 ? 2 : 4;
    const long long T = (long long)nb * F;
    if (T * P * C * es >= (1LL << 31) || (long long)B * P * C * es >= (1LL << 31) || T >= (1LL << 31))
        return fail(SVLA_ERR_SHAPE, fn, "one batch's frames or the cache exceed 2 GiB");
    const long long units = (long long)B * P * (C / 8);
    if (units == 0) return SVLA_OK;
    if (T > 0 && (!X || !Y || !w)) return fail(SVLA_ERR_NULL, fn, "X, Y and w are required");
    if (T == 0 && !cache_out) return SVLA_OK;                       // no frame and no cache: nothing to do
    if (T == 0 && !w) return fail(SVLA_ERR_NULL, fn, "w is required");
    if (misaligned(X) || misaligned(Y) || misaligned(w) || misaligned(bias) || misaligned(cache_in) ||
        misaligned(cache_out))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    const size_t xb = (size_t)(B * T * P * C * es), cb = (size_t)(B * P * C * es);
    if (overlap(X, xb, Y, xb) || overlap(cache_out, cb, X, xb) || overlap(cache_out, cb, Y, xb) ||
        (cache_in && cache_out && cache_in != cache_out && overlap(cache_in, cb, cache_out, cb)))
        return fail(SVLA_ERR_VALUE, fn, "Y overlaps X, or the cache out overlaps X, Y or (other than "
                    "in place) the cache in");
    ConvArgs a;
    memset(&a, 0, sizeof a);
    a.X = X; a.Y = Y; a.w = w; a.bias = bias; a.cache_in = cache_in; a.cache_out = cache_out;
    a.T = (int)T; a.F = F; a.P = P; a.C8 = C / 8; a.units = units;
    const unsigned grid = (unsigned)((units + kThreads - 1) / kThreads);
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    constexpr int MF = SVLA_TCONV_MAXF;
    char nm[96];
    snprintf(nm, sizeof nm, "void svla_temporal_conv_k<%d, %d>", dt == SVLA_BF16 ? 2 : 4, MF);
    if (dt == SVLA_BF16) launch(svla_temporal_conv_k<2, MF>, grid, 0, s, SLOT_CONV, a, nm);
    else launch(svla_temporal_conv_k<4, MF>, grid, 0, s, SLOT_CONV, a, nm);
    return check_launch(fn);
}

svla_status svla_block_causal_backward(svla_dtype dt, int B, int H, int nb, int n, int d,
                                       const void *Q, const void *K, const void *V, const void *dO,
                                       const float *S0, const float *z0, const float *g,
                                       const svla_rope *rope, float eps, void *dQ, void *dK,
                                       void *dV, float *dg, float *dS0, float *dz0, void *ws,
                                       size_t ws_bytes, svla_stream stream)
{
    const char *fn = "svla_block_causal_backward";
    BwdPlan bp;
    svla_status st = make_bwd_plan(fn, dt, B, H, nb, n, d, rope, &bp);
    if (st) return st;
    const Plan &p = bp.fwd;
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(SVLA_ERR_VALUE, fn, "eps must be finite and >= 0");
    if (p.BH * nb == 0) return SVLA_OK;
    const bool tokens = n > 0;
    if (tokens && (!Q || !K || !V || !dO || !dQ || !dK || !dV))
        return fail(SVLA_ERR_NULL, fn, "Q, K, V, dO, dQ, dK and dV are required");
    if ((S0 == nullptr) != (z0 == nullptr)) return fail(SVLA_ERR_NULL, fn, "pass both S0 and z0, or neither");
    if ((dS0 == nullptr) != (dz0 == nullptr)) return fail(SVLA_ERR_NULL, fn, "pass both dS0 and dz0, or neither");
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) || misaligned(dQ) ||
        misaligned(dK) || misaligned(dV) || misaligned(S0) || misaligned(z0) || misaligned(g) ||
        misaligned(dg) || misaligned(dS0) || misaligned(dz0) || misaligned(ws))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    if (tokens) {
        // every gradient is written while some input is still to be read
        const size_t tb = (size_t)p.BH * nb * n * d * p.esize;
        const void *in[4] = {Q, K, V, dO};
        void *out[3] = {dQ, dK, dV};
        for (int i = 0; i < 3; ++i) {
            for (int j = 0; j < 4; ++j)
                if (overlap(out[i], tb, in[j], tb))
                    return fail(SVLA_ERR_VALUE, fn, "dQ, dK and dV must not overlap Q, K, V or dO");
            for (int j = i + 1; j < 3; ++j)
                if (overlap(out[i], tb, out[j], tb))
                    return fail(SVLA_ERR_VALUE, fn, "dQ, dK and dV must not overlap each other");
        }
    }
    if (!ws) return fail(SVLA_ERR_NULL, fn, "workspace of %zu bytes required", bp.total);
    if (ws_bytes < bp.total)
        return fail(SVLA_ERR_WORKSPACE, fn, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, bp.total);
    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    (void)hipGetLastError();
    if (tokens) {
        // the forward's inclusive states, block by block
        BuildArgs ba;
        memset(&ba, 0, sizeof ba);
        ba.K = K; ba.V = V;
        ba.S_part = (float *)(w + p.off_spart);
        ba.z_part = (float *)(w + p.off_zpart);
        ba.N = nb * n; ba.n = n; ba.nb = nb; ba.splits = p.splits; ba.chunk = p.chunk;
        ba.BH = p.BH;
        ba.rope = p.rope;
        build_any(p, ba, s);
        if ((st = check_launch(fn))) return st;
        ScanArgs sa;
        memset(&sa, 0, sizeof sa);
        sa.S_part = ba.S_part; sa.z_part = ba.z_part; sa.g = g; sa.S_in = S0; sa.z_in = z0;
        sa.S_pre = (float *)(w + bp.off_spre); sa.z_pre = (float *)(w + bp.off_zpre);
        sa.nb = nb; sa.splits = p.splits;
        scan_any<SCAN_EXPORT>(p, sa, s);
        if ((st = check_launch(fn))) return st;
    }
    BwdArgs a;
    memset(&a, 0, sizeof a);
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.dQ = dQ; a.dK = dK; a.dV = dV;
    a.S_pre = (const float *)(w + bp.off_spre); a.z_pre = (const float *)(w + bp.off_zpre);
    a.dS_part = (float *)(w + bp.off_dsp); a.dz_part = (float *)(w + bp.off_dzp);
    a.G = (float *)(w + bp.off_G); a.Hz = (float *)(w + bp.off_H);
    a.g = g; a.S0 = S0; a.z0 = z0; a.dg = dg; a.dS0 = dS0; a.dz0 = dz0;
    a.N = nb * n; a.n = n; a.nb = nb; a.splits = bp.splits; a.chunk = bp.chunk;
    a.BH = p.BH; a.eps = eps;
    a.rope = p.rope;
    a.rope.tab_bytes = bp.tab_bytes;
    bwd_any(bp, a, tokens, s);
    return check_launch(fn);
}

svla_status svla_state_build(svla_dtype dt, int B, int H, int nb, int n, int d, const void *K,
                             const void *V, const svla_rope *rope, float *S_local,
                             float *z_local, void *ws, size_t ws_bytes, svla_stream stream)
{
    const char *fn = "svla_state_build";
    Plan p;
    svla_status st = make_plan(fn, SVLA_OP_STATE_BUILD, dt, B, H, nb, n, d, rope, &p);
    if (st) return st;
    (void)ws; (void)ws_bytes;
    if (p.BH * nb == 0) return SVLA_OK;
    if (!S_local || !z_local) return fail(SVLA_ERR_NULL, fn, "S_local and z_local are required");
    if (n > 0 && (!K || !V)) return fail(SVLA_ERR_NULL, fn, "K and V are required");
    if (misaligned(K) || misaligned(V) || misaligned(S_local) || misaligned(z_local))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (n == 0) {
        // no tokens: every local contribution is zero
        ScanArgs sa;
        memset(&sa, 0, sizeof sa);
        sa.nb = nb; sa.splits = 0; sa.S_pre = S_local; sa.z_pre = z_local;
        // an export scan over zero partials writes a zero state for every block
        scan_any<SCAN_EXPORT>(p, sa, s);
        return check_launch(fn);
    }
    BuildArgs ba;
    memset(&ba, 0, sizeof ba);
    ba.K = K; ba.V = V; ba.S_part = S_local; ba.z_part = z_local;
    ba.N = nb * n; ba.n = n; ba.nb = nb; ba.splits = p.splits; ba.chunk = p.chunk; ba.rope = p.rope;
    ba.BH = p.BH;
    build_any(p, ba, s);
    return check_launch(fn);
}

svla_status svla_state_scan(int B, int H, int nb, int d, const float *S_local,
                            const float *z_local, const float *g, const float *S0,
                            const float *z0, float *S_prefix, float *z_prefix,
                            svla_stream stream)
{
    const char *fn = "svla_state_scan";
    Plan p;
    svla_status st = make_plan(fn, SVLA_OP_STATE_SCAN, SVLA_F32, B, H, nb, 1, d, nullptr, &p);
    if (st) return st;
    if (p.BH * nb == 0) return SVLA_OK;
    if (!S_local || !z_local || !S_prefix || !z_prefix)
        return fail(SVLA_ERR_NULL, fn, "S_local, z_local, S_prefix and z_prefix are required");
    if ((S0 == nullptr) != (z0 == nullptr)) return fail(SVLA_ERR_NULL, fn, "pass both S0 and z0, or neither");
    if (misaligned(S_local) || misaligned(z_local) || misaligned(S_prefix) ||
        misaligned(z_prefix) || misaligned(S0) || misaligned(z0) || misaligned(g))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    sa.S_part = S_local; sa.z_part = z_local; sa.g = g; sa.S_in = S0; sa.z_in = z0;
    sa.S_pre = S_prefix; sa.z_pre = z_prefix; sa.nb = nb; sa.splits = 1;
    (void)hipGetLastError();
    scan_any<SCAN_EXPORT>(p, sa, (hipStream_t)stream);
    return check_launch(fn);
}

svla_status svla_apply(svla_dtype dt, int B, int H, int nb, int n, int d, const void *Q,
                       const float *S_prefix, const float *z_prefix, const svla_rope *rope,
                       float eps, void *O, void *ws, size_t ws_bytes, svla_stream stream)
{
    const char *fn = "svla_apply";
    Plan p;
    svla_status st = make_plan(fn, SVLA_OP_APPLY, dt, B, H, nb, n, d, rope, &p);
    if (st) return st;
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(SVLA_ERR_VALUE, fn, "eps must be finite and >= 0");
    if (p.BH * nb * n == 0) return SVLA_OK;
    if (!Q || !O || !S_prefix || !z_prefix)
        return fail(SVLA_ERR_NULL, fn, "Q, O, S_prefix and z_prefix are required");
    if (!ws) return fail(SVLA_ERR_NULL, fn, "workspace of %zu bytes required", p.total);
    if (misaligned(Q) || misaligned(O) || misaligned(S_prefix) || misaligned(z_prefix) || misaligned(ws))
        return fail(SVLA_ERR_ALIGN, fn, "device pointers must be 16-byte aligned");
    if (ws_bytes < p.total)
        return fail(SVLA_ERR_WORKSPACE, fn, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, p.total);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    sa.S_part = S_prefix; sa.nb = nb; sa.splits = 1; sa.S_op = ws;
    scan_any<SCAN_PACK>(p, sa, s);
    if ((st = check_launch(fn))) return st;
    ApplyArgs aa;
    memset(&aa, 0, sizeof aa);
    aa.Q = Q; aa.O = O; aa.S_op = ws; aa.z_pre = z_prefix;
    aa.N = nb * n; aa.n = n; aa.nb = nb; aa.tile = p.tile; aa.tiles = p.tiles; aa.eps = eps;
    aa.rope = p.rope;
    apply_any(p, aa, s);
    return check_launch(fn);
}

}  // extern "C"
