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
#include <type_traits>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/svla.h"

// Tuning knobs (compile-time; the defaults are the measured choices).
#ifndef SVLA_BUILD_PF
#define SVLA_BUILD_PF 2            // stages of K/V loads in flight in the state build
#endif
#ifndef SVLA_BUILD_U
#define SVLA_BUILD_U 2             // 16-byte K and V chunks per thread per stage
#endif
#ifndef SVLA_BUILD_PF_ROPE
#define SVLA_BUILD_PF_ROPE 2       // the same two knobs for the RoPE build
#endif
#ifndef SVLA_BUILD_U_ROPE
#define SVLA_BUILD_U_ROPE 1
#endif
#ifndef SVLA_DMA_U32
#define SVLA_DMA_U32 1             // direct-to-LDS build, d = 32: chunks per thread per stage
#endif
#ifndef SVLA_DMA_R32
#define SVLA_DMA_R32 3             // ... and LDS ring depth
#endif
#ifndef SVLA_DMA_U
#define SVLA_DMA_U 1               // the same for d = 64, 128
#endif
#ifndef SVLA_DMA_R
#define SVLA_DMA_R 4
#endif
#ifndef SVLA_QUAD128
#define SVLA_QUAD128 1             // d = 128 build: one workgroup per 64 x 64 quadrant of S
#endif
#ifndef SVLA_APPLY_TILE32
#define SVLA_APPLY_TILE32 256      // apply: tokens per workgroup for d = 32, 64
#endif
#ifndef SVLA_APPLY_TILE_ROPE
#define SVLA_APPLY_TILE_ROPE 512   // ... with RoPE (amortises the per-workgroup angle table)
#endif
#ifndef SVLA_APPLY_TILE128
#define SVLA_APPLY_TILE128 128     // ... and for d = 128
#endif
#ifndef SVLA_USE_DMA
#define SVLA_USE_DMA 1             // non-RoPE bf16 builds load straight to LDS
#endif
// Cache-policy bits of the streaming accesses (gfx950 buffer instructions:
// bit 1 = nt, non-temporal).  Measured: nt pays for K/V (read once by the
// state build) and for Q when every element is read once (d <= 64); the
// d = 128 apply re-reads Q from four waves and wants it cached.
#ifndef SVLA_KV_AUX
#define SVLA_KV_AUX 2
#endif
#ifndef SVLA_Q_AUX
#define SVLA_Q_AUX 2
#endif
#ifndef SVLA_O_AUX
#define SVLA_O_AUX 0
#endif
#ifndef SVLA_SCAN_LA
#define SVLA_SCAN_LA 16            // partial-state loads in flight per scan thread
#endif
#ifndef SVLA_TARGET_WGS
#define SVLA_TARGET_WGS 2048       // state-build workgroups wanted per launch
#endif
#ifndef SVLA_MIN_SPLIT_PER_D
#define SVLA_MIN_SPLIT_PER_D 8     // tokens per split >= this * d
#endif
#ifndef SVLA_FUSE_MAX_D
#define SVLA_FUSE_MAX_D 0          // fuse the scan into the build for d <= this
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
constexpr int kScanThreads = 64;              // scan: one wave, 256 state elements per workgroup
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

__device__ __forceinline__ unsigned int pack_bf16(float lo, float hi)
{
    return (unsigned int)f2bf(lo) | ((unsigned int)f2bf(hi) << 16);
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
};

// Table layout: [frames nf x dt/2][rows gh x dh/2][cols gw x dw/2] of float2.
__device__ __forceinline__ int rope_entries(const RopeK &r, int nf)
{
    return nf * (r.dt / 2) + r.gh * (r.dh / 2) + r.gw * (r.dw / 2);
}

// Angles pos * theta_m with theta_m = base^(-2m/width): the per-pair
// frequencies (in turns, theta_m / 2 pi) are computed once per workgroup in
// fp64, each entry's angle is reduced to a fraction of a turn in fp64 (so
// large frame indices keep their accuracy) and only then goes through an
// fp32 sin/cos of pi times that small argument.
constexpr int kMaxRopePairs = 64;

__device__ void rope_fill(float2 *tab, const RopeK &r, int f0, int nf)
{
    __shared__ double turns_per_pos[3 * kMaxRopePairs];
    const int pt = r.dt / 2, ph = r.dh / 2, pw = r.dw / 2;
    for (int e = threadIdx.x; e < pt + ph + pw; e += blockDim.x) {
        const int a = e < pt ? 0 : e < pt + ph ? 1 : 2;
        const int m = a == 0 ? e : a == 1 ? e - pt : e - pt - ph;
        const int width = a == 0 ? r.dt : a == 1 ? r.dh : r.dw;
        turns_per_pos[a * kMaxRopePairs + m] =
            pow((double)r.base, -2.0 * (double)m / (double)width) * (0.5 / M_PI);
    }
    __syncthreads();
    const int nT = nf * pt, nH = r.gh * ph, total = rope_entries(r, nf);
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        int pos, m, a;
        if (e < nT) {
            pos = f0 + e / pt; m = e % pt; a = 0;
        } else if (e < nT + nH) {
            int x = e - nT; pos = x / ph; m = x % ph; a = 1;
        } else {
            int x = e - nT - nH; pos = x / pw; m = x % pw; a = 2;
        }
        double turns = (double)pos * turns_per_pos[a * kMaxRopePairs + m];
        turns -= floor(turns);
        float s, c;
        sincospif(2.0f * (float)turns, &s, &c);
        tab[e] = make_float2(c, s);
    }
    if (threadIdx.x == 0) tab[total] = make_float2(1.f, 0.f);   // identity, for unrotated dims
}

// Per-thread description of the 4 (bf16 chunk) or 2 (fp32 chunk) pairs of
// its fixed feature chunk.  A pair's table index for a token at (frame
// offset fr, row, col) is base + fr * mt + row * mh + col * mw, with exactly
// one multiplier non-zero for a rotated pair; a pair outside the three
// slices points at the identity entry (cos 1, sin 0) that ends the table, so
// the rotation has no branches.
template <int PAIRS>
struct RopePairs {
    int base[PAIRS], mt[PAIRS], mh[PAIRS], mw[PAIRS];
};

template <int PAIRS>
__device__ __forceinline__ RopePairs<PAIRS> rope_pairs(const RopeK &r, int first_feature, int nf)
{
    RopePairs<PAIRS> p;
    const int pt = r.dt / 2, ph = r.dh / 2, pw = r.dw / 2;
    const int offH = nf * pt, offW = offH + r.gh * ph;
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
        int f = first_feature + 2 * j;
        p.mt[j] = p.mh[j] = p.mw[j] = 0;
        if (f < r.dt) {
            p.base[j] = f / 2; p.mt[j] = pt;
        } else if (f < r.dt + r.dh) {
            p.base[j] = offH + (f - r.dt) / 2; p.mh[j] = ph;
        } else if (f < r.dt + r.dh + r.dw) {
            p.base[j] = offW + (f - r.dt - r.dh) / 2; p.mw[j] = pw;
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
        const int idx = pp.base[j] + pos.fr * pp.mt[j] + pos.row * pp.mh[j] + pos.col * pp.mw[j];
        const float2 cs = tab[idx];
        const float x0 = x[2 * j], x1 = x[2 * j + 1];
        x[2 * j] = x0 * cs.x - x1 * cs.y;
        x[2 * j + 1] = x0 * cs.y + x1 * cs.x;
    }
}

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
    int nb, splits;
};

struct BuildArgs {
    const void *K, *V;
    float *S_part, *z_part;        // [BH*nb*splits][d*d], [BH*nb*splits][d]
    int N, n, nb, splits, chunk;   // chunk: tokens per split (multiple of the stage)
    long BH;
    RopeK rope;
    unsigned long long *counters;  // [BH] arrival counters of the fused scan
    unsigned epoch;                // distinct per call (see arrive())
    ScanArgs scan;                 // what the last workgroup of a (b,h) runs
};

struct ApplyArgs {
    const void *Q;
    void *O;
    const void *S_op;              // packed operand [BH*nb][d*d]
    const float *z_pre;            // [BH*nb][d]
    int N, n, nb, tile, tiles;     // tile: tokens per workgroup; tiles per block
    float eps;
    RopeK rope;
};

enum ScanMode { SCAN_FUSED = 0, SCAN_EXPORT = 1, SCAN_PACK = 2 };

// ---------------------------------------------------------------------------
// The scan of one (bh, tile): tile < d*d/1024 is a 1024-element slice of S
// (each thread owns 4 consecutive elements of S[k][v]), tile == d*d/1024 is
// z.  Blocks are walked in order, acc = g_c * acc + sum over splits, with the
// splits added in index order, so the result repeats bit for bit.
//
// Packed operand layout read by svla_apply (per (bh, block), d*d entries):
// bf16: fragment (m, ks) = 64 lanes x 8 values; lane (rho + 16 kg), value i
//       holds S[32 ks + 8 kg + i][f(m, rho)]
// fp32: fragment (m, kq) = 64 lanes x 4 values; lane (rho + 16 kg), value i
//       holds S[16 kq + 4 kg + i][f(m, rho)]
// with f(m, rho) = (d/4) (rho / 4) + 4 m + rho % 4: the output rows of the
// MFMA land so that each lane ends up with consecutive O features.
// ---------------------------------------------------------------------------
template <int D, int MODE, bool OPBF16, int NT>
__device__ __forceinline__ void scan_tile(const ScanArgs &a, long bh, int tile, int tid)
{
    constexpr int STILES = D * D / (NT * 4);
    if (tile < STILES) {
        const int e0 = tile * (NT * 4) + tid * 4;
        const int k = e0 / D, v = e0 % D;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (MODE != SCAN_PACK && a.S_in) acc = *(const f32x4_t *)(a.S_in + bh * D * D + e0);
        // operand positions of the 4 elements (k, v..v+3)
        const int m = (v % (D / 4)) / 4, rho0 = 4 * (v / (D / 4));
        int opos[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (OPBF16) {
                const int ks = k / 32, kg = (k % 32) / 8, i = k % 8;
                opos[j] = (((m * (D / 32) + ks) * 64 + rho0 + j + 16 * kg) * 8 + i);
            } else {
                const int kq = k / 16, kg = (k % 16) / 4, i = k % 4;
                opos[j] = (((m * (D / 16) + kq) * 64 + rho0 + j + 16 * kg) * 4 + i);
            }
        }
        // The partials of (block c, split sp) form one stream, idx = c*splits + sp,
        // read through a ring of LA loads in flight; a refill past the end
        // re-reads the last partial (always in bounds) and is never used.
        constexpr int LA = SVLA_SCAN_LA;
        const int total = a.nb * a.splits;
        const float *base = a.S_part + bh * (long)total * D * D + e0;
        f32x4_t ring[LA];
#pragma unroll
        for (int j = 0; j < LA; ++j)
            ring[j] = total > 0 ? *(const f32x4_t *)(base + (long)min(j, total - 1) * D * D)
                                : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        int c = 0, sp = 0;
        if (a.splits == 0) {
            // no tokens: each block only decays the carried state
            for (; c < a.nb; ++c) {
                const long unit = bh * a.nb + c;
                if (a.g) acc *= a.g[unit];
                if (MODE == SCAN_EXPORT) *(f32x4_t *)(a.S_pre + unit * D * D + e0) = acc;
            }
        }
        for (int idx0 = 0; idx0 < total; idx0 += LA) {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int idx = idx0 + j;
                if (idx < total) {
                    const long unit = bh * a.nb + c;
                    if (sp == 0) {
                        if (MODE == SCAN_PACK) acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                        else if (a.g) acc *= a.g[unit];
                    }
                    acc += ring[j];
                    if (sp == a.splits - 1) {
                        if (MODE == SCAN_EXPORT) {
                            *(f32x4_t *)(a.S_pre + unit * D * D + e0) = acc;
                        } else if constexpr (OPBF16) {
                            unsigned short *op = (unsigned short *)a.S_op + unit * D * D;
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) op[opos[jj]] = f2bf(acc[jj]);
                        } else {
                            float *op = (float *)a.S_op + unit * D * D;
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) op[opos[jj]] = acc[jj];
                        }
                        sp = 0;
                        ++c;
                    } else {
                        ++sp;
                    }
                }
                ring[j] = *(const f32x4_t *)(base + (long)min(idx + LA, total - 1) * D * D);
            }
        }
        if (MODE != SCAN_PACK && a.S_fin) *(f32x4_t *)(a.S_fin + bh * D * D + e0) = acc;
    } else if (MODE != SCAN_PACK && tid < D / 4) {
        const int e0 = tid * 4;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (a.z_in) acc = *(const f32x4_t *)(a.z_in + bh * D + e0);
        constexpr int LA = SVLA_SCAN_LA;   // same look-ahead ring as for S
        const int total = a.nb * a.splits;
        const float *base = a.z_part + bh * (long)total * D + e0;
        f32x4_t ring[LA];
#pragma unroll
        for (int j = 0; j < LA; ++j)
            ring[j] = total > 0 ? *(const f32x4_t *)(base + (long)min(j, total - 1) * D)
                                : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        int c = 0, sp = 0;
        if (a.splits == 0) {
            for (; c < a.nb; ++c) {
                const long unit = bh * a.nb + c;
                if (a.g) acc *= a.g[unit];
                *(f32x4_t *)(a.z_pre + unit * D + e0) = acc;
            }
        }
        for (int idx0 = 0; idx0 < total; idx0 += LA) {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int idx = idx0 + j;
                if (idx < total) {
                    const long unit = bh * a.nb + c;
                    if (sp == 0 && a.g) acc *= a.g[unit];
                    acc += ring[j];
                    if (sp == a.splits - 1) {
                        *(f32x4_t *)(a.z_pre + unit * D + e0) = acc;
                        sp = 0;
                        ++c;
                    } else {
                        ++sp;
                    }
                }
                ring[j] = *(const f32x4_t *)(base + (long)min(idx + LA, total - 1) * D);
            }
        }
        if (a.z_fin) *(f32x4_t *)(a.z_fin + bh * D + e0) = acc;
    }
}

template <int D, int MODE, bool OPBF16>
__global__ void __launch_bounds__(kScanThreads)
svla_state_scan_k(const ScanArgs a)
{
    constexpr int STILES = D * D / (kScanThreads * 4);
    const long bh = blockIdx.x / (STILES + 1);
    scan_tile<D, MODE, OPBF16, kScanThreads>(a, bh, blockIdx.x % (STILES + 1), threadIdx.x);
}

// Arrival of one workgroup at a (b,h) counter; true for the last of `total`.
// The counter holds (epoch << 32 | count).  A count left by any other call
// (a different epoch), or whatever an unused workspace held, is restarted,
// so the workspace needs no initialisation; the last arrival rewinds the
// count to 0 under the same epoch, so replaying a captured launch works too.
// The loop ends: a failed compare-and-swap means another workgroup's swap
// succeeded, and at most `total` workgroups arrive per launch.
__device__ bool arrive(unsigned long long *ctr, unsigned epoch, unsigned total)
{
    const unsigned long long tag = (unsigned long long)epoch << 32;
    unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const unsigned long long nw = ((old >> 32) == epoch) ? old + 1 : (tag | 1ull);
        const unsigned long long prev = atomicCAS(ctr, old, nw);
        if (prev == old) {
            if ((unsigned)(nw & 0xffffffffull) == total) {
                __hip_atomic_store(ctr, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return true;
            }
            return false;
        }
        old = prev;
    }
}

// After a build workgroup has written its partials: the last workgroup of the
// (b,h) runs the scan of every tile of that (b,h) (the inclusive prefix over
// blocks, the packed operands, the final state).
template <int D, bool OPBF16>
__device__ __forceinline__ void fused_scan(const BuildArgs &a, long bh, int tid)
{
    __shared__ int s_last;
    __threadfence();                 // release this workgroup's partial stores
    __syncthreads();
    if (tid == 0) s_last = arrive(a.counters + bh, a.epoch, (unsigned)(a.nb * a.splits));
    __syncthreads();
    if (!s_last) return;
    __threadfence();                 // acquire every other workgroup's partials
#pragma unroll 1
    for (int tile = 0; tile <= D * D / 1024; ++tile) scan_tile<D, SCAN_FUSED, OPBF16, kThreads>(a.scan, bh, tile, tid);
}

// ---------------------------------------------------------------------------
// svla_state_build, bf16 inputs.
//
// Workgroup = (bh, block c, split s); it walks its token range in stages of
// TT tokens.  Per stage every thread loads one 16-byte chunk of K and of V
// (8 features of one token), applies phi to K, adds phi(k) to its running z,
// and writes both chunks to LDS rows.  PF stages of loads are in flight while
// the current stage is contracted.  The MFMA v_mfma_f32_32x32x16_bf16
// contracts over tokens, so each lane gathers 8 tokens of one feature from
// the staged rows.  Which token feeds which k-slot does not matter for a
// sum over tokens, as long as A and B use the same assignment; lanes 32-63
// take the odd tokens so the two half-waves hit disjoint LDS banks.
//   d = 32 : one 32x32 output tile; the 4 waves split the stage's tokens and
//            their accumulators are summed through LDS at the end.
//   d = 64 : 2x2 tiles, one per wave, every wave sees every token.
//   d = 128: 4x4 tiles, 2x2 per wave.
// With RoPE the rotated phi(k) is split into bf16 hi + lo parts, two MFMAs,
// so the state keeps ~16 bits of the rotated key.
// FUSE: the last workgroup of each (b,h) also runs the scan (fused_scan).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz16(int t, int chunk)
{
    // rows of d >= 64 span every LDS bank: odd rows swap chunk halves so
    // the two half-waves (even/odd tokens) read disjoint banks.
    return (D >= 64) ? (chunk ^ ((t & 1) << 2)) : chunk;
}

template <int D, bool ROPE, int PF, int U, bool FUSE>
__global__ void __launch_bounds__(kThreads)
svla_state_build_bf16(const BuildArgs a)
{
    constexpr int CPR = D / 8;            // 16-byte chunks per token row
    constexpr int RPS = kThreads / CPR;   // token rows one pass of the threads covers
    constexpr int TT = U * RPS;           // tokens per stage (U chunks per thread per tensor)
    constexpr int ROWB = D * 2;
    constexpr int TILEB = TT * ROWB;      // U * 4096 bytes
    constexpr int NK = ROPE ? 2 : 1;
    constexpr int STAGEB = (NK + 1) * TILEB;
    constexpr bool SPLITK = (D == 32);
    constexpr int TPW = SPLITK ? 1 : D / 64;
    constexpr int GPS = TT / 16;          // 16-token groups per stage

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned per_bh = (unsigned)(a.splits * a.nb);
    const long bh = blockIdx.x / per_bh;
    const int rest = (int)(blockIdx.x - bh * per_bh);
    const int c = rest / a.splits, s = rest % a.splits;
    const int tok_lo = c * a.n + s * a.chunk;
    const int tok_hi = min(tok_lo + a.chunk, (c + 1) * a.n);

    const uint32_t slice = (uint32_t)a.N * D * 2;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);

    // RoPE table (lives before the stage buffers)
    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<4> pp;
    const int row = tid / CPR, q = tid % CPR;
    if constexpr (ROPE) {
        frame_lo = tok_lo < tok_hi ? fdiv((uint32_t)tok_lo, a.rope.div_hw) : 0;
        uint32_t frame_hi = tok_lo < tok_hi ? fdiv((uint32_t)(tok_hi - 1), a.rope.div_hw) : 0;
        int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
        pp = rope_pairs<4>(a.rope, q * 8, nf);
        __syncthreads();
    }
    unsigned char *stage = lds + (ROPE ? a.rope.tab_bytes : 0);

    float zacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zacc[e] = 0.f;

    f32x16_t acc[TPW][TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < TPW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // The stage loop is kept regular so the compiler can count the loads in
    // flight: the stage count is rounded up to a multiple of PF (extra stages
    // load nothing and add zeros) and every slot is refilled unconditionally
    // (a refill past the range gets the out-of-range offset).
    const int ntiles = tok_hi > tok_lo ? (tok_hi - tok_lo + TT - 1) / TT : 0;
    const int nstages = (ntiles + PF - 1) / PF * PF;
    auto offset = [&](int t) -> uint32_t {
        return t < tok_hi ? (uint32_t)(t * D + q * 8) * 2u : kOOB;
    };
    u32x4_t kreg[PF][U], vreg[PF][U];
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = offset(tok_lo + row + u * RPS + p * TT);
            kreg[p][u] = load16p<SVLA_KV_AUX>(rK, off);
            vreg[p][u] = load16p<SVLA_KV_AUX>(rV, off);
        }

    const int m = lane & 31, g = lane >> 5;
    const int mt0 = SPLITK ? 0 : (wave >> 1) * TPW;
    const int nt0 = SPLITK ? 0 : (wave & 1) * TPW;
    constexpr int GPW = SPLITK ? GPS / 4 : GPS;  // 16-token groups per wave per stage
    // lane part of a fragment element's LDS index (k-slot i reads row 16 gi + g + 2 i)
    int kl[TPW], vl[TPW];
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int f = 32 * (mt0 + tm) + m;
        kl[tm] = g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
    }
#pragma unroll
    for (int tn = 0; tn < TPW; ++tn) {
        const int f = 32 * (nt0 + tn) + m;
        vl[tn] = g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
    }

    for (int it0 = 0; it0 < nstages; it0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int it = it0 + p;
            unsigned char *st = stage + (it & 1) * STAGEB;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = row + u * RPS;              // row within the stage
                const int tok = tok_lo + r + it * TT;
                // phi(k), z, (rotation), stage to LDS
                u32x4_t kr;
#pragma unroll
                for (int e = 0; e < 4; ++e) kr[e] = relu_bf16x2(kreg[p][u][e]);
                float kf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = bf16lo(kr[e]);
                    kf[2 * e + 1] = bf16hi(kr[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) zacc[e] += kf[e];
                const int cpos = swz16<D>(r, q);
                if constexpr (ROPE) {
                    rope_rotate<4>(kf, rope_pos((uint32_t)tok, frame_lo, a.rope), pp, tab);
                    u32x4_t hi, lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        unsigned short h0 = f2bf(kf[2 * e]), h1 = f2bf(kf[2 * e + 1]);
                        float r0 = kf[2 * e] - as_f32((unsigned int)h0 << 16);
                        float r1 = kf[2 * e + 1] - as_f32((unsigned int)h1 << 16);
                        hi[e] = (unsigned int)h0 | ((unsigned int)h1 << 16);
                        lo[e] = pack_bf16(r0, r1);
                    }
                    *(u32x4_t *)(st + r * ROWB + cpos * 16) = hi;
                    *(u32x4_t *)(st + TILEB + r * ROWB + cpos * 16) = lo;
                } else {
                    *(u32x4_t *)(st + r * ROWB + cpos * 16) = kr;
                }
                *(u32x4_t *)(st + NK * TILEB + r * ROWB + cpos * 16) = vreg[p][u];
            }
            lds_barrier();

            // refill this register slot with the stage PF ahead
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t off = offset(tok_lo + row + u * RPS + (it + PF) * TT);
                kreg[p][u] = load16p<SVLA_KV_AUX>(rK, off);
                vreg[p][u] = load16p<SVLA_KV_AUX>(rV, off);
            }

            const unsigned short *Kh = (const unsigned short *)st;
            const unsigned short *Kl = (const unsigned short *)(st + TILEB);
            const unsigned short *Vs = (const unsigned short *)(st + NK * TILEB);
#pragma unroll
            for (int gg = 0; gg < GPW; ++gg) {
                const int gi = SPLITK ? wave + 4 * gg : gg;
                bf16x8_t av[TPW], al[TPW], bv[TPW];
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
                    const unsigned short *ph = Kh + 16 * gi * D + kl[tm];
                    const unsigned short *pl = Kl + 16 * gi * D + kl[tm];
                    u16x8_t x, y;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        x[i] = ph[2 * i * D];
                        if constexpr (ROPE) y[i] = pl[2 * i * D];
                    }
                    av[tm] = __builtin_bit_cast(bf16x8_t, x);
                    if constexpr (ROPE) al[tm] = __builtin_bit_cast(bf16x8_t, y);
                }
#pragma unroll
                for (int tn = 0; tn < TPW; ++tn) {
                    const unsigned short *pv = Vs + 16 * gi * D + vl[tn];
                    u16x8_t x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = pv[2 * i * D];
                    bv[tn] = __builtin_bit_cast(bf16x8_t, x);
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
    __syncthreads();   // every wave is done with the stage buffers

    // ---- epilogue: write S_part (row-major [k][v]) and z_part
    const long unit = (bh * a.nb + c) * a.splits + s;
    const auto rS = make_rsrc(a.S_part + unit * D * D, D * D * 4);
    const auto rz = make_rsrc(a.z_part + unit * D, D * 4);
    float *red = (float *)stage;
    float *zred = (float *)(stage + (SPLITK ? 4 * 16 * 64 * 4 : 0));
    if constexpr (SPLITK) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[0][0][r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[tid * 8 + e] = zacc[e];
    __syncthreads();
    if constexpr (SPLITK) {
        // thread -> 4 consecutive columns of one row; fixed summation order
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
        const int qq = tid >> 3, e = tid & 7;
        float v = 0.f;
        for (int j = 0; j < kThreads / CPR; ++j) v += zred[(qq + CPR * j) * 8 + e];
        store4(rz, (uint32_t)tid * 4u, v);
    }
    if constexpr (FUSE) fused_scan<D, true>(a, bh, tid);
    (void)RPS;
}

// ---------------------------------------------------------------------------
// svla_state_build, bf16 inputs without RoPE, loads straight to LDS.
//
// The same contraction as svla_state_build_bf16, but K and V travel from
// global memory into an R-deep ring of LDS stages with buffer_load ... lds
// (16 bytes per lane, one kilobyte per wave instruction), so R - 1 stages of
// loads stay in flight without holding registers.  phi is applied to the
// K fragments after they are read from LDS, and z is summed from those
// fragments.  Rows past the end of the range are masked when fragments are
// read, so whatever an out-of-range load leaves in LDS never enters a sum.
// Each stage buffer is its own LDS object, which lets the compiler tell the
// loads of different stages apart instead of waiting for all of them.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D, int U, int R, int DG>
__global__ void __launch_bounds__(kThreads)
svla_state_build_dma(const BuildArgs a)
{
    // D: width of the tile this workgroup contracts; DG: feature count of the
    // data.  DG == 2 D is the quadrant split for d = 128: four workgroups per
    // (b,h,block,split), each computing one 64 x 64 quadrant of S.
    constexpr int CPR = D / 8;            // 16-byte chunks per token row
    constexpr int RPW = 64 / CPR;         // rows one wave instruction covers
    constexpr int RPS = kThreads / CPR;   // rows one pass of the 4 waves covers
    constexpr int TT = U * RPS;           // tokens per stage
    constexpr int ROWB = D * 2;
    constexpr int TILEB = TT * ROWB;      // U * 4096
    constexpr int STAGEB = 2 * TILEB;     // K tile, then V tile
    constexpr bool SPLITK = (D == 32);
    constexpr int TPW = SPLITK ? 1 : D / 64;
    constexpr int GPS = TT / 16;
    constexpr int L = 2 * U;              // loads per thread per stage
    constexpr bool QUAD = DG != D;
    static_assert(R >= 3 && R <= 4, "ring depth");
    static_assert(!SPLITK || STAGEB >= 8192, "epilogue reuses two stage buffers");
    static_assert(!QUAD || (DG == 128 && D == 64), "quadrant split is for d = 128");

    __shared__ __attribute__((aligned(16))) unsigned char b0[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b1[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b2[STAGEB];
    __shared__ __attribute__((aligned(16))) unsigned char b3[R > 3 ? STAGEB : 16];
    __shared__ float zred[4 * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Quadrants of one unit get workgroup ids 8 apart, so the round-robin
    // dispatch puts all four on the same XCD and its L2 serves the shared
    // K/V half-rows.
    long wid = blockIdx.x;
    int qm = 0, qn = 0;
    if constexpr (QUAD) {
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

    const uint32_t slice = (uint32_t)a.N * DG * 2;
    const auto rK = make_rsrc((const char *)a.K + bh * slice, slice);
    const auto rV = make_rsrc((const char *)a.V + bh * slice, slice);
    const int kcol = 64 * qm, vcol = 64 * qn;   // first feature of this tile in K / V

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
            const uint32_t offk = in ? (uint32_t)(t * DG + kcol + cg * 8) * 2u : kOOB;
            const uint32_t offv = in ? (uint32_t)(t * DG + vcol + cg * 8) * 2u : kOOB;
            unsigned char *kd = dst + (u * 4 + wave) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr_t)kd, 16, offk, 0, 0, SVLA_KV_AUX);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr_t)(kd + TILEB), 16, offv, 0, 0, SVLA_KV_AUX);
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
    // Lane part of a fragment element's LDS index: k-slot i of a group reads
    // row 16 gi + g + 2 i, and the row's parity (= g) fixes the swizzle.
    int kl[TPW], vl[TPW];
#pragma unroll
    for (int tm = 0; tm < TPW; ++tm) {
        const int f = 32 * (mt0 + tm) + m;
        kl[tm] = g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
    }
#pragma unroll
    for (int tn = 0; tn < TPW; ++tn) {
        const int f = 32 * (nt0 + tn) + m;
        vl[tn] = g * D + swz16<D>(g, f >> 3) * 8 + (f & 7);
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
            const unsigned short *Ks = (const unsigned short *)buf(j);
            const unsigned short *Vs = Ks + TT * D;
#pragma unroll
            for (int gg = 0; gg < GPW; ++gg) {
                const int gi = SPLITK ? wave + 4 * gg : gg;
                bf16x8_t av[TPW], bv[TPW];
#pragma unroll
                for (int tm = 0; tm < TPW; ++tm) {
                    const unsigned short *pk = Ks + 16 * gi * D + kl[tm];
                    u16x8_t x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = pk[2 * i * D];
                    u32x4_t w = __builtin_bit_cast(u32x4_t, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = relu_bf16x2(w[e]);
                    av[tm] = __builtin_bit_cast(bf16x8_t, w);
                    // z on the matrix cores: phi(K) times a ones operand
                    if (zwave) zt[tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], ones, zt[tm], 0, 0, 0);
                }
#pragma unroll
                for (int tn = 0; tn < TPW; ++tn) {
                    const unsigned short *pv = Vs + 16 * gi * D + vl[tn];
                    u16x8_t x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = pv[2 * i * D];
                    bv[tn] = __builtin_bit_cast(bf16x8_t, x);
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
    const long unit = (bh * a.nb + c) * a.splits + s;
    const auto rS = make_rsrc(a.S_part + unit * DG * DG, DG * DG * 4);
    const auto rz = make_rsrc(a.z_part + unit * DG, DG * 4);
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
                    const int rr = kcol + 32 * (mt0 + tm) + 8 * (r >> 2) + 4 * g + (r & 3);
                    const int cc = vcol + 32 * (nt0 + tn) + m;
                    store4(rS, (uint32_t)(rr * DG + cc) * 4u, acc[tm][tn][r]);
                }
        if (tid < D && qn == 0) store4(rz, (uint32_t)(kcol + tid) * 4u, zred[tid]);
    }
}

// ---------------------------------------------------------------------------
// svla_state_build, fp32 inputs: the same walk with fp32 rows staged and
// v_mfma_f32_32x32x2_f32 (one token per half-wave per instruction).
// ---------------------------------------------------------------------------
template <int D, bool ROPE, bool FUSE>
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

    const long unit = (bh * a.nb + c) * a.splits + s;
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
    if constexpr (FUSE) fused_scan<D, false>(a, bh, tid);
}

// ---------------------------------------------------------------------------
// svla_apply, bf16 inputs.  Workgroup = (bh, block c, token tile).
// O^T = S^T phi~(Q)^T on v_mfma_f32_16x16x32_bf16: the state is the A
// operand (kept in registers for the whole tile, loaded once from the
// packed layout), phi~(q) the B operand straight from a 16-byte load per
// lane (token = lane % 16, 8 features of chunk 4 ks + lane / 16).  The
// denominator phi(q) . z is a per-lane partial dot product reduced over the
// 4 lanes that share a token.
//   d = 32, 64: each wave takes every 4th 16-token group, all output features.
//   d = 128   : every wave takes every group, for its own 32 output features.
// ---------------------------------------------------------------------------
template <int D, bool ROPE>
__global__ void __launch_bounds__(kThreads)
svla_apply_bf16(const ApplyArgs a)
{
    constexpr int MT = D / 16;
    constexpr int KS = D / 32;
    constexpr bool SPLITM = (D == 128);
    constexpr int MW = SPLITM ? 2 : MT;

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x % a.tiles;
    const int c = (blockIdx.x / a.tiles) % a.nb;
    const long bh = blockIdx.x / ((long)a.tiles * a.nb);
    const int t_lo = c * a.n + tile * a.tile;
    const int t_hi = min(t_lo + a.tile, (c + 1) * a.n);
    const long unit = bh * a.nb + c;

    const uint32_t slice = (uint32_t)a.N * D * 2;
    const auto rQ = make_rsrc((const char *)a.Q + bh * slice, slice);
    const auto rO = make_rsrc((char *)a.O + bh * slice, slice);
    const auto rS = make_rsrc((const char *)a.S_op + unit * D * D * 2, D * D * 2);
    const auto rz = make_rsrc(a.z_pre + unit * D, D * 4);

    const int kg = lane >> 4, tl = lane & 15;
    const int m0 = SPLITM ? 2 * wave : 0;

    bf16x8_t sf[MW][KS];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sf[mi][ks] = __builtin_bit_cast(bf16x8_t,
                load16(rS, (uint32_t)((((m0 + mi) * KS + ks) * 64 + lane) * 16)));
    float zf[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4_t z0 = load16(rz, (uint32_t)(8 * (4 * ks + kg)) * 4u);
        u32x4_t z1 = load16(rz, (uint32_t)(8 * (4 * ks + kg) + 4) * 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            zf[ks][e] = as_f32(z0[e]);
            zf[ks][4 + e] = as_f32(z1[e]);
        }
    }

    float2 *tab = (float2 *)lds;
    uint32_t frame_lo = 0;
    RopePairs<4> pp[KS];
    if constexpr (ROPE) {
        frame_lo = t_lo < t_hi ? fdiv((uint32_t)t_lo, a.rope.div_hw) : 0;
        uint32_t frame_hi = t_lo < t_hi ? fdiv((uint32_t)(t_hi - 1), a.rope.div_hw) : 0;
        int nf = (int)(frame_hi - frame_lo) + 1;
        rope_fill(tab, a.rope, a.rope.t0 + (int)frame_lo, nf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pp[ks] = rope_pairs<4>(a.rope, 8 * (4 * ks + kg), nf);
        __syncthreads();
    }

    // groups of this wave: g_first, g_first + g_step, ...; the loads of GB
    // groups are issued together before any of them is used.
    constexpr int GB = SPLITM ? 2 : 4;
    const int ngroups = t_hi > t_lo ? (t_hi - t_lo + 15) / 16 : 0;
    const int g_first = SPLITM ? 0 : wave, g_step = SPLITM ? 1 : 4;
    for (int gb = g_first; gb < ngroups; gb += GB * g_step) {
    u32x4_t qb[GB][KS];
#pragma unroll
    for (int j = 0; j < GB; ++j) {
        const int tok = t_lo + 16 * (gb + j * g_step) + tl;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[j][ks] = load16p<SPLITM ? 0 : SVLA_Q_AUX>(rQ, tok < t_hi ? (uint32_t)(tok * D + 8 * (4 * ks + kg)) * 2u : kOOB);
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
        const int gi = gb + j * g_step;
        if (gi >= ngroups) break;
        const int tok = t_lo + 16 * gi + tl;
        const bool valid = tok < t_hi;
        const u32x4_t *qr = qb[j];
        float den = 0.f;
        bf16x8_t qf[KS];
        RopePos rp{0, 0, 0};
        if constexpr (ROPE) rp = rope_pos((uint32_t)tok, frame_lo, a.rope);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t p;
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = relu_bf16x2(qr[ks][e]);
            float pf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pf[2 * e] = bf16lo(p[e]);
                pf[2 * e + 1] = bf16hi(p[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) den = fmaf(pf[e], zf[ks][e], den);
            if constexpr (ROPE) {
                rope_rotate<4>(pf, rp, pp[ks], tab);
#pragma unroll
                for (int e = 0; e < 4; ++e) p[e] = pack_bf16(pf[2 * e], pf[2 * e + 1]);
            }
            qf[ks] = __builtin_bit_cast(bf16x8_t, p);
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
            for (int ks = 0; ks < KS; ++ks)
                acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[mi][ks], qf[ks], acc[mi], 0, 0, 0);
        }
        // lane holds O[tok][4 MT kg + 4 (m0 + mi) + r], consecutive in (mi, r)
#pragma unroll
        for (int h = 0; h < MW / 2; ++h) {
            u32x4_t o;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                o[2 * e] = pack_bf16(acc[2 * h + e][0] * inv, acc[2 * h + e][1] * inv);
                o[2 * e + 1] = pack_bf16(acc[2 * h + e][2] * inv, acc[2 * h + e][3] * inv);
            }
            const int v0 = 4 * MT * kg + 4 * (m0 + 2 * h);
            store16p<SVLA_O_AUX>(rO, valid ? (uint32_t)(tok * D + v0) * 2u : kOOB, o);
        }
    }
    }
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
    const int tile = blockIdx.x % a.tiles;
    const int c = (blockIdx.x / a.tiles) % a.nb;
    const long bh = blockIdx.x / ((long)a.tiles * a.nb);
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
            const int v0 = 4 * MT * kg + 4 * (m0 + mi);
            store16(rO, valid ? (uint32_t)(tok * D + v0) * 4u : kOOB, o);
        }
    }
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local char g_err[512] = "";
thread_local void *const *t_events = nullptr;   // svla_set_timing_events
thread_local int t_nev = 0;

enum Slot { SLOT_BUILD = 0, SLOT_SCAN = 1, SLOT_APPLY = 2 };

// Every kernel goes through here.  With timing events set, the launch
// carries a start/stop event pair that the runtime records around the
// kernel's own execution.
// svla_describe: while set, launch() records what it would launch instead.
struct LaunchDesc {
    char name[3][96];
    unsigned grid[3], block[3];
    size_t lds[3];
    bool used[3];
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
    int splits, chunk;         // build
    int tile, tiles;           // apply
    bool fuse;                 // scan runs in the build's last workgroup per (b,h)
    size_t lds_build, lds_apply;
    size_t off_ctr, off_spart, off_zpart, off_sop, off_zpre, total;
    RopeK rope;
};

// A value that differs between any two calls of the process (see arrive()).
unsigned next_epoch()
{
    static std::atomic<unsigned> e{(unsigned)std::chrono::steady_clock::now().time_since_epoch().count()};
    return e.fetch_add(1, std::memory_order_relaxed);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16 state build: chunks per thread per stage and stages of loads in flight
constexpr int build_u(bool rope) { return rope ? SVLA_BUILD_U_ROPE : SVLA_BUILD_U; }
constexpr int build_pf(bool rope) { return rope ? SVLA_BUILD_PF_ROPE : SVLA_BUILD_PF; }


// Splits of a block's tokens over workgroups: enough workgroups to fill the
// chip (about SVLA_TARGET_WGS), but never fewer than SVLA_MIN_SPLIT_PER_D * d
// tokens per split, so the fp32 partial state (4 d^2 bytes) stays a small
// fraction of the K/V bytes it summarises (1/8 at the default).
int pick_splits(long units, int n, int d, int *chunk_out)
{
    constexpr int G = 64;   // chunk granularity; independent of the stage size, so the
                            // workspace size does not depend on RoPE or tuning
    if (n <= 0 || units <= 0) { *chunk_out = G; return 0; }
    long want = (SVLA_TARGET_WGS + units - 1) / units;
    long cap = n / (SVLA_MIN_SPLIT_PER_D * d);
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
    return SVLA_OK;
}

svla_status check_sizes(const char *fn, svla_dtype dt, int B, int H, int nb, int n, int d)
{
    if (dt != SVLA_F32 && dt != SVLA_BF16)
        return fail(SVLA_ERR_DTYPE, fn, "dtype %d is not SVLA_F32 or SVLA_BF16", (int)dt);
    if (B < 0 || H < 0 || nb < 0 || n < 0)
        return fail(SVLA_ERR_SHAPE, fn, "negative size (B=%d H=%d nb=%d n=%d)", B, H, nb, n);
    if (d != 32 && d != 64 && d != 128)
        return fail(SVLA_ERR_UNSUPPORTED, fn, "d=%d not in {32, 64, 128}", d);
    const int es = dt == SVLA_BF16 ? 2 : 4;
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
    p->esize = dt == SVLA_BF16 ? 2 : 4;
    st = check_rope(fn, rope, d, &p->rope);
    if (st) return st;
    if (op == SVLA_OP_STATE_BUILD) {
        p->splits = n > 0 ? 1 : 0;
        p->chunk = n > 0 ? n : 1;
    } else {
        p->splits = pick_splits(p->BH * nb, n, d, &p->chunk);
    }
    p->tile = d == 128 ? SVLA_APPLY_TILE128 : (p->rope.on ? SVLA_APPLY_TILE_ROPE : SVLA_APPLY_TILE32);
    p->tiles = n > 0 ? (n + p->tile - 1) / p->tile : 0;

    // LDS: [RoPE table][stage buffers | epilogue]
    const size_t stage = (size_t)2 * ((p->esize == 2 && p->rope.on) ? 3 : 2) * 4096 *
                         (p->esize == 2 ? build_u(p->rope.on) : 1);
    const size_t epi = (d == 32 ? 16384 : 0) + 8192;
    p->lds_build = stage > epi ? stage : epi;
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

    // workspace
    size_t off = 0;
    const size_t units = (size_t)p->BH * nb;
    const bool fused = op == SVLA_OP_NONCAUSAL || op == SVLA_OP_BLOCK_CAUSAL || op == SVLA_OP_BLOCK_STEP;
    p->fuse = fused && d <= SVLA_FUSE_MAX_D && p->splits > 0 && nb > 0;
    if (fused) {
        p->off_ctr = off; off = align256(off + (size_t)p->BH * 8);
        p->off_spart = off; off = align256(off + units * p->splits * d * d * 4);
        p->off_zpart = off; off = align256(off + units * p->splits * d * 4);
    }
    if (fused || op == SVLA_OP_APPLY) {
        p->off_sop = off; off = align256(off + units * d * d * p->esize);
    }
    if (fused) {
        p->off_zpre = off; off = align256(off + units * d * 4);
    }
    p->total = off;
    return SVLA_OK;
}

inline bool misaligned(const void *ptr) { return ((uintptr_t)ptr & 15) != 0; }

// ---- launchers ---------------------------------------------------------------

template <int D, bool FUSE>
void launch_build_f(const Plan &p, const BuildArgs &a, hipStream_t s)
{
    const unsigned grid = (unsigned)(p.BH * p.nb * p.splits);
    const char *fz = FUSE ? "true" : "false";
    char nm[96];
    if (SVLA_USE_DMA && p.esize == 2 && !p.rope.on && !FUSE) {
        constexpr int U = D == 32 ? SVLA_DMA_U32 : SVLA_DMA_U;
        constexpr int R = D == 32 ? SVLA_DMA_R32 : SVLA_DMA_R;
        if constexpr (D == 128 && SVLA_QUAD128) {
            const unsigned qgrid = (unsigned)((grid + 7) / 8 * 8 * 4);
            snprintf(nm, sizeof nm, "void svla_state_build_dma<64, %d, %d, 128>", U, R);
            launch(svla_state_build_dma<64, U, R, 128>, qgrid, 0, s, SLOT_BUILD, a, nm);
        } else {
            snprintf(nm, sizeof nm, "void svla_state_build_dma<%d, %d, %d, %d>", D, U, R, D);
            launch(svla_state_build_dma<D, U, R, D>, grid, 0, s, SLOT_BUILD, a, nm);
        }
        return;
    }
    if (p.esize == 2) {
        if (p.rope.on) {
            snprintf(nm, sizeof nm, "void svla_state_build_bf16<%d, true, %d, %d, %s>", D,
                     build_pf(true), build_u(true), fz);
            launch(svla_state_build_bf16<D, true, build_pf(true), build_u(true), FUSE>, grid,
                   p.lds_build, s, SLOT_BUILD, a, nm);
        } else {
            snprintf(nm, sizeof nm, "void svla_state_build_bf16<%d, false, %d, %d, %s>", D,
                     build_pf(false), build_u(false), fz);
            launch(svla_state_build_bf16<D, false, build_pf(false), build_u(false), FUSE>, grid,
                   p.lds_build, s, SLOT_BUILD, a, nm);
        }
    } else {
        snprintf(nm, sizeof nm, "void svla_state_build_f32<%d, %s, %s>", D,
                 p.rope.on ? "true" : "false", fz);
        if (p.rope.on) launch(svla_state_build_f32<D, true, FUSE>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
        else launch(svla_state_build_f32<D, false, FUSE>, grid, p.lds_build, s, SLOT_BUILD, a, nm);
    }
}

template <int D>
void launch_build(const Plan &p, const BuildArgs &a, hipStream_t s)
{
    if constexpr (D <= SVLA_FUSE_MAX_D) {
        if (p.fuse) { launch_build_f<D, true>(p, a, s); return; }
    }
    launch_build_f<D, false>(p, a, s);
}

template <int D, int MODE>
void launch_scan_d(const Plan &p, const ScanArgs &a, hipStream_t s)
{
    const unsigned grid = (unsigned)(p.BH * (D * D / (kScanThreads * 4) + 1));
    char nm[96];
    snprintf(nm, sizeof nm, "void svla_state_scan_k<%d, %d, %s>", D, MODE, p.esize == 2 ? "true" : "false");
    if (p.esize == 2) launch(svla_state_scan_k<D, MODE, true>, grid, 0, s, SLOT_SCAN, a, nm, kScanThreads);
    else launch(svla_state_scan_k<D, MODE, false>, grid, 0, s, SLOT_SCAN, a, nm, kScanThreads);
}

template <int D>
void launch_apply(const Plan &p, const ApplyArgs &a, hipStream_t s)
{
    const unsigned grid = (unsigned)(p.BH * p.nb * p.tiles);
    char nm[96];
    snprintf(nm, sizeof nm, "void svla_apply_%s<%d, %s>", p.esize == 2 ? "bf16" : "f32", D,
             p.rope.on ? "true" : "false");
    if (p.esize == 2) {
        if (p.rope.on) launch(svla_apply_bf16<D, true>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
        else launch(svla_apply_bf16<D, false>, grid, p.lds_apply, s, SLOT_APPLY, a, nm);
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
                    size_t ws_bytes, svla_stream stream)
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

    hipStream_t s = (hipStream_t)stream;
    char *w = (char *)ws;
    (void)hipGetLastError();
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    sa.S_part = (const float *)(w + p.off_spart);
    sa.z_part = (const float *)(w + p.off_zpart);
    sa.g = g; sa.S_in = S0; sa.z_in = z0;
    sa.S_op = w + p.off_sop;
    sa.z_pre = (float *)(w + p.off_zpre);
    sa.S_fin = S_fin; sa.z_fin = z_fin;
    sa.nb = nb; sa.splits = p.splits;
    if (p.splits > 0 && nb > 0) {
        BuildArgs ba;
        memset(&ba, 0, sizeof ba);
        ba.K = K; ba.V = V;
        ba.S_part = (float *)(w + p.off_spart);
        ba.z_part = (float *)(w + p.off_zpart);
        ba.N = nb * n; ba.n = n; ba.nb = nb; ba.splits = p.splits; ba.chunk = p.chunk;
        ba.BH = p.BH;
        ba.rope = p.rope;
        if (p.fuse) {
            ba.counters = (unsigned long long *)(w + p.off_ctr);
            ba.epoch = next_epoch();
            ba.scan = sa;
        }
        build_any(p, ba, s);
        if ((st = check_launch(fn))) return st;
    }
    if (!p.fuse) {
        scan_any<SCAN_FUSED>(p, sa, s);
        if ((st = check_launch(fn))) return st;
    }
    if (tokens) {
        ApplyArgs aa;
        aa.Q = Q; aa.O = O; aa.S_op = w + p.off_sop; aa.z_pre = (const float *)(w + p.off_zpre);
        aa.N = nb * n; aa.n = n; aa.nb = nb; aa.tile = p.tile; aa.tiles = p.tiles; aa.eps = eps;
        aa.rope = p.rope;
        apply_any(p, aa, s);
        if ((st = check_launch(fn))) return st;
    }
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
    LaunchDesc desc;
    memset(&desc, 0, sizeof desc);
    t_desc = &desc;
    BuildArgs ba;
    memset(&ba, 0, sizeof ba);
    ScanArgs sa;
    memset(&sa, 0, sizeof sa);
    ApplyArgs aa;
    memset(&aa, 0, sizeof aa);
    if (p.BH > 0) {
        if (p.splits > 0 && nb > 0) build_any(p, ba, nullptr);
        if (!p.fuse) scan_any<SCAN_FUSED>(p, sa, nullptr);
        if ((long)nb * n > 0) apply_any(p, aa, nullptr);
    }
    t_desc = nullptr;
    static const char *slot_name[3] = {"build", "scan", "apply"};
    int w = snprintf(buf, len, "{\"splits\": %d, \"chunk\": %d, \"apply_tile\": %d, \"workspace\": %zu, \"kernels\": [",
                     p.splits, p.chunk, p.tile, p.total);
    bool first = true;
    for (int k = 0; k < 3; ++k) {
        if (!desc.used[k] || w < 0 || (size_t)w >= len) continue;
        w += snprintf(buf + w, len - w, "%s{\"slot\": \"%s\", \"name\": \"%s\", \"grid\": %u, \"block\": %u, \"lds\": %zu}",
                      first ? "" : ", ", slot_name[k], desc.name[k], desc.grid[k], desc.block[k], desc.lds[k]);
        first = false;
    }
    if (w >= 0 && (size_t)w < len) w += snprintf(buf + w, len - w, "]}");
    if (w < 0 || (size_t)w >= len) return fail(SVLA_ERR_VALUE, fn, "buffer of %zu bytes too small", len);
    return SVLA_OK;
}

svla_status svla_workspace_size(svla_op op, svla_dtype dt, int B, int H, int nb, int n, int d,
                                size_t *bytes)
{
    const char *fn = "svla_workspace_size";
    if (!bytes) return fail(SVLA_ERR_NULL, fn, "bytes is NULL");
    if ((int)op < SVLA_OP_NONCAUSAL || (int)op > SVLA_OP_APPLY)
        return fail(SVLA_ERR_VALUE, fn, "unknown op %d", (int)op);
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
        // an export scan over zero splits writes a zero state for every block
        scan_any<SCAN_EXPORT>(p, sa, s);
        return check_launch(fn);
    }
    BuildArgs ba;
    memset(&ba, 0, sizeof ba);
    ba.K = K; ba.V = V; ba.S_part = S_local; ba.z_part = z_local;
    ba.N = nb * n; ba.n = n; ba.nb = nb; ba.splits = 1; ba.chunk = p.chunk; ba.rope = p.rope;
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
    aa.Q = Q; aa.O = O; aa.S_op = ws; aa.z_pre = z_prefix;
    aa.N = nb * n; aa.n = n; aa.nb = nb; aa.tile = p.tile; aa.tiles = p.tiles; aa.eps = eps;
    aa.rope = p.rope;
    apply_any(p, aa, s);
    return check_launch(fn);
}

}  // extern "C"
