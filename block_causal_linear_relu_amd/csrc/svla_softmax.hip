// svla_softmax_attention: the softmax "anchor" layers of the SANA-Video 2.0
// hybrid (2.0 news page, the hybrid linear-softmax attention paragraph:
// periodic softmax layers among gated linear ones, three to one; comfyui-wiki
// model page, the 2.0 section: dense softmax anchors), on the block schedule
// of the linear layers (talk, block-by-block generation): queries of nb blocks
// of n tokens against Nk >= nb*n cached keys; query i (block c = i / n) sees
// keys 0 .. Nk - nb*n + (c+1)*n - 1, and
//     O_i = sum_j softmax_j(scale * q_i . k_j) v_j.
// bf16 Q, K, V, O; fp32 logits, weights and sums.  The kernel is kept in a
// source of its own.
//
// Workgroup = (b,h, tile of 32 W queries), W waves of 32 queries each (W = 8
// at d = 128, 4 at d = 64); the tiles are launched heaviest first (the last
// query tiles see the most keys).
// The keys stream through two LDS stages in tiles of 64; each tile's K and V
// are loaded into registers one tile ahead.  Per 32-key half, on
// v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   rows = keys, columns = queries: the K tile is the A operand
//                 (16-byte LDS reads of its rows), the wave's Q rows the B
//                 operand, held in registers for the whole kernel; lane
//                 (n, h) ends with 16 of the 32 keys' logits of query n, so a
//                 query's running max and sum need one lane swap.
//   O^T += V^T P^T  rows = features, columns = queries: P is the B operand
//                 straight from the lane's own registers (the k-slots of a
//                 contraction over keys may be taken in any order as long as
//                 both operands agree), V^T the A operand from a transposed
//                 LDS copy of the V tile; the A operand's rows are ordered so
//                 that lane (n, h) accumulates 16 contiguous features of its
//                 query per output tile (two 16-byte stores at the end).
// Online softmax in base 2 (logits scaled by scale * log2 e): running max m
// and per-lane partial sum l per query; the accumulator is rescaled only when
// some query of the wave raised its max.  The weights use the hardware's
// 2^x (v_exp_f32) directly: its arguments are <= 0, and a weight below 2^-126
// (flushed to zero) is below bf16's resolution of the sum it enters.  Keys past a query's visible range
// (only in the last tiles of a workgroup) get weight zero.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/svla.h"

#ifndef SVLA_SM_WAVES
#define SVLA_SM_WAVES 2            // waves per SIMD the register allocation must allow
#endif
#ifndef SVLA_SM_W128
#define SVLA_SM_W128 8             // waves per workgroup at d = 128 (32 queries each)
#endif

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

constexpr int kKTile = 64;             // keys per LDS tile
constexpr uint32_t kSmOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sm_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_t sm_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ unsigned int sm_pack_bf16(float lo, float hi)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

struct SoftmaxArgs {
    const void *Q, *K, *V;
    void *O;
    int Nq, Nk, n;                 // queries (nb * n), keys, tokens per block
    int qtiles;                    // query tiles per (b,h)
    long BH;
    float c2;                      // scale * log2(e)
};

// Feature that row m of output tile t holds (see the header comment): lane
// (n, h) register r of tile t is feature 32 t + 16 h + r.
__device__ __forceinline__ int sm_feat(int t, int m)
{
    return 32 * t + 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// LDS hand-off barrier that waits for this wave's LDS operations only (a
// __syncthreads() would also wait for every global load in flight, i.e. for
// the prefetched key tiles).
__device__ __forceinline__ void sm_lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waves per workgroup (32 queries each): eight at d = 128, so a key tile
// staged in LDS serves 256 queries; four at d = 64.
template <int D>
constexpr int sm_waves() { return D == 128 ? SVLA_SM_W128 : 4; }

template <int D>
struct SmTile {                                 // one key tile's K and V chunks in registers
    static constexpr int CPT = kKTile * D / 8 / (64 * sm_waves<D>());
    u32x4_t k[CPT], v[CPT];
};

template <int D>
__global__ void __launch_bounds__(64 * sm_waves<D>(), SVLA_SM_WAVES)
svla_softmax_fwd(const SoftmaxArgs a)
{
    constexpr int kSmThreads = 64 * sm_waves<D>();
    constexpr int kQTile = 32 * sm_waves<D>();   // queries per workgroup
    constexpr int KK = D / 16;                 // 16-feature steps of the logit product
    constexpr int T = D / 32;                  // output tiles of 32 features
    constexpr int LDK = D + 8;                 // K tile row, bf16 elements
    constexpr int LDV = kKTile + 8;            // V^T tile row, bf16 elements
    constexpr int CPT = SmTile<D>::CPT;        // 16-byte chunks per thread per tensor
    constexpr int KSZ = kKTile * LDK, VSZ = D * LDV;
    // two LDS stages of [K tile | V^T tile]
    extern __shared__ __attribute__((aligned(16))) unsigned short sm_lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 31, h = lane >> 5;
    const long bh = blockIdx.x % a.BH;
    const int qt = a.qtiles - 1 - (int)(blockIdx.x / a.BH);     // heaviest tiles first
    const int q0 = qt * kQTile;
    const uint32_t qslice = (uint32_t)a.Nq * D * 2, kslice = (uint32_t)a.Nk * D * 2;
    const auto rQ = sm_rsrc((const char *)a.Q + bh * qslice, qslice);
    const auto rO = sm_rsrc((char *)a.O + bh * qslice, qslice);
    const auto rK = sm_rsrc((const char *)a.K + bh * kslice, kslice);
    const auto rV = sm_rsrc((const char *)a.V + bh * kslice, kslice);

    // visible keys of a query row: Nk - Nq + (block + 1) n; rows past Nq see none
    auto limit_of = [&](int row) -> int {
        return row < a.Nq ? a.Nk - a.Nq + (row / a.n + 1) * a.n : 0;
    };
    const int qrow = q0 + 32 * wave + m;          // this lane's query
    const int lim = limit_of(qrow);
    // the workgroup's key range: up to the largest limit of its rows; tiles
    // below the smallest limit need no mask
    const int last_row = min(q0 + kQTile, a.Nq) - 1;
    const int kmax = limit_of(last_row);
    const int kmin = limit_of(q0);
    const int ntiles = (kmax + kKTile - 1) / kKTile;

    // K: thread -> 16-byte chunk (key, ch), consecutive lanes along a row.
    // V: thread -> (key pair j, chunk ch) with j fastest: the rows 2j and 2j+1
    // of the chunk, written to V^T as one 4-byte word (keys 2j, 2j+1) per
    // feature, so the 32 lanes of a half-wave fill one V^T row segment and
    // the two half-waves rows 8 features apart (32 banks apart).
    auto issue = [&](SmTile<D> &r, int tile) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = tid + c * kSmThreads;            // chunk index in the tile
            const int key = idx / (D / 8), ch = idx % (D / 8);
            const int kg = tile * kKTile + key;
            const uint32_t off = tile < ntiles && kg < kmax ? ((uint32_t)kg * D + ch * 8) * 2 : kSmOOB;
            r.k[c] = sm_load16(rK, off);
        }
#pragma unroll
        for (int c = 0; c < CPT / 2; ++c) {
            const int idx = tid + c * kSmThreads;
            const int j = idx % (kKTile / 2), ch = idx / (kKTile / 2);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int kg = tile * kKTile + 2 * j + e;
                const uint32_t off = tile < ntiles && kg < kmax ? ((uint32_t)kg * D + ch * 8) * 2 : kSmOOB;
                r.v[2 * c + e] = sm_load16(rV, off);
            }
        }
    };
    auto stage = [&](const SmTile<D> &r, int buf) {
        unsigned short *Ks = sm_lds + buf * (KSZ + VSZ), *Vt = Ks + KSZ;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = tid + c * kSmThreads;
            const int key = idx / (D / 8), ch = idx % (D / 8);
            *(u32x4_t *)(Ks + key * LDK + ch * 8) = r.k[c];
        }
#pragma unroll
        for (int c = 0; c < CPT / 2; ++c) {
            const int idx = tid + c * kSmThreads;
            const int j = idx % (kKTile / 2), ch = idx / (kKTile / 2);
            const u32x4_t v0 = r.v[2 * c], v1 = r.v[2 * c + 1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // features ch*8 + 2e (low halves) and ch*8 + 2e + 1 (high halves)
                *(unsigned int *)(Vt + (ch * 8 + 2 * e) * LDV + 2 * j) =
                    (v0[e] & 0xFFFFu) | (v1[e] << 16);
                *(unsigned int *)(Vt + (ch * 8 + 2 * e + 1) * LDV + 2 * j) =
                    (v0[e] >> 16) | (v1[e] & 0xFFFF0000u);
            }
        }
    };

    // the first key tile's loads, then the wave's Q rows (B operand of
    // S^T = K Q^T, 16 features per step), held for the whole kernel
    SmTile<D> ra;
    issue(ra, 0);
    u32x4_t qv[KK];
    {
        const uint32_t off = qrow < a.Nq ? (uint32_t)qrow * D * 2 : kSmOOB;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qv[kk] = sm_load16(rQ, off == kSmOOB ? kSmOOB : off + (uint32_t)(16 * kk + 8 * h) * 2);
    }

    f32x16_t acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float mrun = -INFINITY, lsum = 0.f;

    // key tile it from LDS stage `buf`
    auto compute = [&](int it, int buf) {
        const unsigned short *Ks = sm_lds + buf * (KSZ + VSZ), *Vt = Ks + KSZ;
        const int k0 = it * kKTile;
        // logits of the two 32-key halves: lane (n, h) holds keys
        // 32 half + 8 (r / 4) + 4 h + r % 4 of query n
        f32x16_t s[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[hf][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const u32x4_t kv = *(const u32x4_t *)(Ks + (32 * hf + m) * LDK + 16 * kk + 8 * h);
                s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                                __builtin_bit_cast(bf16x8_t, qv[kk]),
                                                                s[hf], 0, 0, 0);
            }
        }
        // mask, running max (of the raw logits: the scale is positive, so it
        // is applied once, inside the exponent's fused multiply-add)
        if (k0 + kKTile > kmin) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * hf + 8 * (r >> 2) + 4 * h + (r & 3);
                    s[hf][r] = key < lim ? s[hf][r] : -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[hf][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * a.c2;
        const float mnew = fmaxf(mrun, tmax);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrun - muse);
        mrun = mnew;
        // the weights 2^(c2 s - m), their sum, and P as bf16 (the B operand of
        // O^T += V^T P^T)
        unsigned int pw[2][8];
        float psum = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[hf][r], a.c2, -muse));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[hf][r + 1], a.c2, -muse));
                psum += p0 + p1;
                pw[hf][r / 2] = sm_pack_bf16(p0, p1);
            }
        lsum = lsum * alpha + psum;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
        }
        // O^T += V^T P^T: per 32-key half two 16-key steps; k-slot i of lane
        // half h in step st is the lane's register 8 st + i, i.e. key
        // 32 hf + 16 st + 8 (i / 4) + 4 h + i % 4
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const u32x4_t pb = {pw[hf][4 * st], pw[hf][4 * st + 1], pw[hf][4 * st + 2], pw[hf][4 * st + 3]};
                const int kb = 32 * hf + 16 * st + 4 * h;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const unsigned short *row = Vt + sm_feat(t, m) * LDV + kb;
                    const u32x2_t lo = *(const u32x2_t *)row;
                    const u32x2_t hi = *(const u32x2_t *)(row + 8);
                    const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                                     __builtin_bit_cast(bf16x8_t, pb),
                                                                     acc[t], 0, 0, 0);
                }
            }
    };
    // Tile t is loaded into registers during tile t - 1 and staged into LDS
    // stage t % 2 at the start of its own turn; one barrier per tile publishes
    // it, and (every wave having passed it only after its previous tile's
    // work) frees the stage the next tile overwrites.
    for (int it = 0; it < ntiles; ++it) {
        stage(ra, it & 1);
        issue(ra, it + 1);
        sm_lds_barrier();
        __builtin_amdgcn_sched_barrier(0);    // the next tile's loads stay ahead of this tile's work
        compute(it, it & 1);
    }
    // O = acc / l: lane (n, h) holds features 32 t + 16 h + r of its query
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < a.Nq) {
        const uint32_t off = (uint32_t)qrow * D * 2;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4_t o;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = sm_pack_bf16(acc[t][8 * c + 2 * e] * inv, acc[t][8 * c + 2 * e + 1] * inv);
                __builtin_amdgcn_raw_buffer_store_b128(o, rO, (int)(off + (uint32_t)(32 * t + 16 * h + 8 * c) * 2), 0, 0);
            }
    }
}

template <int D>
constexpr size_t sm_lds_bytes() { return (size_t)2 * (kKTile * (D + 8) + D * (kKTile + 8)) * 2; }

bool sm_overlap(const void *x, size_t nx, const void *y, size_t ny)
{
    if (!x || !y) return false;
    const uintptr_t a = (uintptr_t)x, b = (uintptr_t)y;
    return a < b + ny && b < a + nx;
}

}  // namespace

extern "C" svla_status svla_softmax_attention(svla_dtype dt, int B, int H, int nb, int n, int Nk,
                                              int d, const void *Q, const void *K, const void *V,
                                              void *O, float scale, svla_stream stream)
{
    if (dt != SVLA_BF16) return SVLA_ERR_DTYPE;
    if (B < 0 || H < 0 || nb < 0 || n < 0 || Nk < 0) return SVLA_ERR_SHAPE;
    if (d != 64 && d != 128) return SVLA_ERR_UNSUPPORTED;
    const long long Nq = (long long)nb * n;
    if (Nk < Nq) return SVLA_ERR_SHAPE;
    if ((long long)Nk * d * 2 >= (1LL << 31)) return SVLA_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return SVLA_ERR_VALUE;
    const long long BH = (long long)B * H;
    if (BH == 0 || Nq == 0) return SVLA_OK;
    if (!Q || !K || !V || !O) return SVLA_ERR_NULL;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return SVLA_ERR_ALIGN;
    const size_t qb = (size_t)(BH * Nq * d * 2), kb = (size_t)(BH * Nk * d * 2);
    if (sm_overlap(O, qb, Q, qb) || sm_overlap(O, qb, K, kb) || sm_overlap(O, qb, V, kb))
        return SVLA_ERR_VALUE;
    const int qtile = 32 * (d == 128 ? sm_waves<128>() : sm_waves<64>());
    const int qtiles = (int)((Nq + qtile - 1) / qtile);
    if (BH * qtiles >= (1LL << 31)) return SVLA_ERR_SHAPE;
    SoftmaxArgs a;
    memset(&a, 0, sizeof a);
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    a.Nq = (int)Nq; a.Nk = Nk; a.n = n; a.qtiles = qtiles; a.BH = BH;
    a.c2 = scale * 1.4426950408889634f;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const unsigned grid = (unsigned)(BH * qtiles);
    if (d == 128) svla_softmax_fwd<128><<<grid, 64 * sm_waves<128>(), sm_lds_bytes<128>(), s>>>(a);
    else svla_softmax_fwd<64><<<grid, 64 * sm_waves<64>(), sm_lds_bytes<64>(), s>>>(a);
    return hipGetLastError() == hipSuccess ? SVLA_OK : SVLA_ERR_HIP;
}
