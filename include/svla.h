/*
 * svla.h -- C ABI of libsvla: block-causal ReLU linear attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (SANA-Video, "Efficient Video Generation with Block Linear
 * Diffusion Transformer"):
 *   - linear attention is the core operation of the Linear DiT (abstract,
 *     design (1) "Linear DiT");
 *   - its state is a d x d matrix whose shape does not depend on the
 *     sequence length, cached after each block and increased by the next
 *     block's KV contribution (ICLR 2026 oral talk, "block KV cache"
 *     review; abstract, design (2) "Constant-Memory KV cache");
 *   - video is generated block by block, causally across blocks and
 *     bidirectionally inside a block (talk, the description of the hybrid
 *     schedule: autoregressive over blocks, diffusion inside each block);
 *   - SANA-Video 2.0 uses gated linear attention layers (SANA-Video 2.0
 *     news page, "Hybrid Linear-Softmax Attention"; comfyui-wiki model page,
 *     2.0 section);
 *   - the linear attention carries 3D RoPE (talk, architecture section on
 *     the changes made to the linear attention; comfyui-wiki model page,
 *     rotary position embeddings).
 *
 * Definitions used by every call, per (batch b, head h):
 *   phi(x)  = max(x, 0), elementwise, on Q and K only.
 *   local_c = sum over tokens j of block c of  R_j phi(k_j) (x) v_j   (d x d)
 *   zloc_c  = sum over tokens j of block c of  phi(k_j)               (d)
 *   S_c     = g_c * S_{c-1} + local_c,   z_c = g_c * z_{c-1} + zloc_c,
 *             S_{-1} = S0 (or 0), g_c = 1 when ungated.
 *   O_i     = (R_i phi(q_i))^T S_c / (phi(q_i) . z_c + eps) for i in block c.
 * R_j is the identity without RoPE.  With RoPE, R_j rotates adjacent pairs
 * (2m, 2m+1) of three dimension slices by +pos*theta_m, theta_m =
 * base^(-2m/width): dims [0,dt) by the frame index t, [dt,dt+dh) by the
 * grid row, [dt+dh,dt+dh+dw) by the grid column; dims past dt+dh+dw are not
 * rotated.  Token p of a call (p counts from 0 over the call's tokens) sits at
 * frame t0 + p/(grid_h*grid_w), row (p/grid_w)%grid_h, column p%grid_w.
 * The rotation touches the numerator only: z and the denominator use phi(.)
 * unrotated.
 *
 * Conventions shared by every entry point:
 *   Layout   Q, K, V, O: contiguous [B,H,N,d] (d fastest), one dtype (with
 *            SVLA_FP8, Q, K, V are fp8 and O is bf16).
 *            S: [B,H,d,d] fp32, S[k][v] (row = key feature, column = value
 *            feature).  z: [B,H,d] fp32.  g: fp32.
 *   Memory   All pointers except `rope` are device pointers (HIP), 16-byte
 *            aligned.  The caller owns every buffer.  The library never
 *            allocates or frees memory and never synchronises: it only
 *            enqueues kernels on `stream` (NULL = the default stream).
 *            O must not overlap Q, K, V or the workspace.
 *   Sizes    d in {32, 64, 128}; B, H, nb, n >= 0.  One (b,h) slice of Q
 *            must stay below 2 GiB.  Empty inputs (B*H == 0) return SVLA_OK
 *            without launching anything.
 *   Errors   Every call returns a status.  All validation runs on the host
 *            before any HIP call; on any error nothing is launched and no
 *            output is written.  svla_last_error() returns a thread-local
 *            message for the last failing call of the thread.
 *            SVLA_ERR_HIP reports a launch failure only; faults during
 *            execution surface at the caller's next synchronisation.
 *   Workspace  Scratch device memory of at least svla_workspace_size()
 *            bytes for the same op and sizes.  Its content on entry does
 *            not matter; the size does not depend on how many blocks came
 *            before (the state is the only thing carried).
 *   Threads  Calls are re-entrant.  Two calls that share a workspace must be
 *            ordered on one stream.
 */
#ifndef SVLA_H
#define SVLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVLA_ABI_VERSION 1

typedef enum svla_status {
    SVLA_OK = 0,
    SVLA_ERR_NULL = 1,        /* a required pointer is NULL                   */
    SVLA_ERR_SHAPE = 2,       /* negative size, slice too large, N % nb != 0  */
    SVLA_ERR_DTYPE = 3,       /* dtype not SVLA_F32 / SVLA_BF16 / SVLA_FP8    */
    SVLA_ERR_ALIGN = 4,       /* a device pointer not 16-byte aligned         */
    SVLA_ERR_UNSUPPORTED = 5, /* d not in {32,64,128}; RoPE split or grid too large */
    SVLA_ERR_WORKSPACE = 6,   /* workspace smaller than svla_workspace_size() */
    SVLA_ERR_VALUE = 7,       /* eps < 0 or not finite; bad RoPE parameters   */
    SVLA_ERR_HIP = 8,         /* a kernel launch failed                       */
    /* not statuses: they make the type hold every int, so a C caller's
       out-of-range value is an unknown status, never undefined in C++ */
    SVLA_STATUS_INT_MIN_ = -2147483647 - 1,
    SVLA_STATUS_INT_MAX_ = 2147483647
} svla_status;

typedef enum svla_dtype {
    SVLA_F32 = 0,   /* IEEE binary32 Q/K/V/O */
    SVLA_BF16 = 1,  /* bfloat16 Q/K/V/O; arithmetic accumulates in fp32 */
    SVLA_FP8 = 2,   /* OCP FP8 E4M3 Q/K/V (1 byte per element; d = 32 only) with a
                       bfloat16 O: the low-precision inputs that the abstract's
                       NVFP4 deployment points to; arithmetic as for bf16 */
    SVLA_DTYPE_INT_MIN_ = -2147483647 - 1,   /* range markers, as for svla_status */
    SVLA_DTYPE_INT_MAX_ = 2147483647
} svla_dtype;

/* Which call a workspace is sized for. */
typedef enum svla_op {
    SVLA_OP_NONCAUSAL = 0,
    SVLA_OP_BLOCK_CAUSAL = 1,   /* also the gated variant */
    SVLA_OP_BLOCK_STEP = 2,     /* also the gated variant */
    SVLA_OP_STATE_BUILD = 3,
    SVLA_OP_STATE_SCAN = 4,
    SVLA_OP_APPLY = 5,
    SVLA_OP_BACKWARD = 6,       /* svla_block_causal_backward */
    SVLA_OP_INT_MIN_ = -2147483647 - 1,      /* range markers, as for svla_status */
    SVLA_OP_INT_MAX_ = 2147483647
} svla_op;

/* 3D RoPE on the numerator (host struct; may live on the stack).
 * dt_dims/dh_dims/dw_dims: even, >= 0, sum <= d.  grid_h, grid_w >= 1.
 * t0 >= 0: absolute frame index of the call's first token.  base > 0. */
typedef struct svla_rope {
    int dt_dims, dh_dims, dw_dims;
    int grid_h, grid_w;
    int t0;
    float base;
} svla_rope;

/* A hipStream_t; NULL means the default stream. */
typedef void *svla_stream;

/* ---- versioning and errors ------------------------------------------------ */

int svla_abi_version(void);                       /* == SVLA_ABI_VERSION */
const char *svla_status_string(svla_status s);    /* static string */
const char *svla_last_error(void);                /* thread-local; "" if none */

/* Bytes of workspace the call `op` needs for these sizes (nb = 1 for the
 * non-causal call and the block step; N = nb*n), with or without RoPE and
 * a gate (the size covers every launch plan the call can pick).  *bytes is
 * written on SVLA_OK only. */
svla_status svla_workspace_size(svla_op op, svla_dtype dt, int B, int H,
                                int nb, int n, int d, size_t *bytes);

/* The launch plan of a fused call (SVLA_OP_NONCAUSAL, _BLOCK_CAUSAL,
 * _BLOCK_STEP) for these sizes, as a JSON object written to buf (host
 * memory, `len` bytes including the terminating zero): split count, tokens
 * per split, apply tile, workspace bytes, and for each kernel its name (as
 * profilers report it), grid, block and dynamic LDS ("kernels").  A one-block
 * call of bf16 at d = 32 up to 3072 tokens runs as one launch ("fused": true,
 * "step_tiles" workgroups of "step_tile" tokens per (b,h)) unless its new
 * state overlaps the state it reads; "in_place_kernels" then lists the launches
 * of that case.  Launches nothing.  SVLA_ERR_VALUE if the text does not fit. */
svla_status svla_describe(svla_op op, svla_dtype dt, int B, int H, int nb, int n, int d,
                          const svla_rope *rope, char *buf, size_t len);

/* ---- the method ------------------------------------------------------------ */

/* Non-causal linear attention over one block of N tokens (the base Linear
 * DiT: abstract, design (1)).  O = phi(Q) S / (phi(Q) z + eps) with
 * S = phi(K)^T V, z = sum phi(K) over all N tokens.
 * S_out [B,H,d,d] and z_out [B,H,d] (nullable, both or neither) receive S, z. */
svla_status svla_noncausal(svla_dtype dt, int B, int H, int N, int d,
                           const void *Q, const void *K, const void *V, void *O,
                           float eps, float *S_out, float *z_out,
                           void *ws, size_t ws_bytes, svla_stream stream);

/* Block-causal linear attention over nb blocks of n tokens in one call
 * (talk, block KV cache and block-causal schedule).  Tokens of block c read
 * the inclusive state S_c.  S0/z0 (nullable, both or neither): state that
 * enters block 0.  S_final/z_final (nullable, both or neither): S_{nb-1}.
 * rope: NULL for none. */
svla_status svla_block_causal(svla_dtype dt, int B, int H, int nb, int n, int d,
                              const void *Q, const void *K, const void *V, void *O,
                              const float *S0, const float *z0,
                              float *S_final, float *z_final,
                              const svla_rope *rope, float eps,
                              void *ws, size_t ws_bytes, svla_stream stream);

/* As svla_block_causal with a decay g [B,H,nb] (fp32, device) applied to the
 * state entering each block (SANA-Video 2.0 gated layers):
 * S_c = g[b,h,c] * S_{c-1} + local_c, and likewise for z. */
svla_status svla_block_causal_gated(svla_dtype dt, int B, int H, int nb, int n, int d,
                                    const void *Q, const void *K, const void *V, void *O,
                                    const float *S0, const float *z0,
                                    float *S_final, float *z_final,
                                    const float *g, const svla_rope *rope, float eps,
                                    void *ws, size_t ws_bytes, svla_stream stream);

/* One streaming block step (talk: cache the state, add the next block's KV
 * contribution): Q, K, V, O are [B,H,n,d] for this block only.
 * S_out = S_in + phi(K)^T V, z_out = z_in + sum phi(K); O reads S_out.
 * S_in/z_in nullable (zero state).  S_out/z_out required; S_out may equal
 * S_in (commit in place) or differ (evaluate without committing, as a
 * denoising loop does before a block is final, or commit into the other of
 * two state buffers).  With RoPE, rope->t0 is the absolute frame index of
 * this block's first token.
 * Launches: bf16 at d = 32 with n <= 3072 and S_out/z_out sharing no byte
 * with S_in/z_in runs as one kernel (every workgroup of a (b,h) builds the
 * block state itself, nothing waits on another workgroup); otherwise, and
 * always when the new state overlaps the old one, a state build and a read-out
 * that folds the scan in (two kernels, for bf16 or fp8 at d = 32 whose block
 * is cut into at most 7 splits; otherwise build, scan and read-out). */
svla_status svla_block_step(svla_dtype dt, int B, int H, int n, int d,
                            const void *Q, const void *K, const void *V, void *O,
                            const float *S_in, const float *z_in,
                            float *S_out, float *z_out,
                            const svla_rope *rope, float eps,
                            void *ws, size_t ws_bytes, svla_stream stream);

/* As svla_block_step with decay g [B,H] (fp32, device):
 * S_out = g * S_in + phi(K)^T V, z_out = g * z_in + sum phi(K). */
svla_status svla_block_step_gated(svla_dtype dt, int B, int H, int n, int d,
                                  const void *Q, const void *K, const void *V, void *O,
                                  const float *S_in, const float *z_in,
                                  float *S_out, float *z_out,
                                  const float *g, const svla_rope *rope, float eps,
                                  void *ws, size_t ws_bytes, svla_stream stream);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): svla_block_step (g NULL) or svla_block_step_gated (g [B,H]
 * non-NULL) with the library's own scratch instead of a caller workspace.
 * The scratch is 32 MiB per GPU, held from the library's load until the
 * process ends; a step whose svla_workspace_size(SVLA_OP_BLOCK_STEP, ...) is
 * larger returns SVLA_ERR_WORKSPACE.  The call allocates nothing.  `stream`
 * must belong to the current device (NULL = its default stream), otherwise
 * SVLA_ERR_VALUE.  Every call on a GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  Validation runs before any HIP call, as elsewhere. */
svla_status svla_block_step_noalloc(svla_dtype dt, int B, int H, int n, int d,
                                    const void *Q, const void *K, const void *V, void *O,
                                    const float *S_in, const float *z_in,
                                    float *S_out, float *z_out,
                                    const float *g, const svla_rope *rope, float eps,
                                    svla_stream stream);

/* ---- the three kernels, one by one ------------------------------------------ */

/* Each block's own contribution: S_local [B,H,nb,d,d] = sum_j R_j phi(k_j) (x) v_j,
 * z_local [B,H,nb,d] = sum_j phi(k_j) (talk: the current block's KV
 * contribution).  K, V: [B,H,nb*n,d]. */
svla_status svla_state_build(svla_dtype dt, int B, int H, int nb, int n, int d,
                             const void *K, const void *V, const svla_rope *rope,
                             float *S_local, float *z_local,
                             void *ws, size_t ws_bytes, svla_stream stream);

/* Inclusive (optionally decayed) prefix over blocks (talk: the cached state
 * plus the current block's contribution):
 * S_prefix[b,h,c] = g[b,h,c] * S_prefix[b,h,c-1] + S_local[b,h,c], starting
 * from S0 (nullable = 0); z likewise.  g nullable (= 1).
 * S_local, S_prefix: [B,H,nb,d,d]; z_local, z_prefix: [B,H,nb,d]. */
svla_status svla_state_scan(int B, int H, int nb, int d,
                            const float *S_local, const float *z_local,
                            const float *g, const float *S0, const float *z0,
                            float *S_prefix, float *z_prefix, svla_stream stream);

/* Read-out of every token against its block's state:
 * O_i = (R_i phi(q_i))^T S_prefix[c] / (phi(q_i) . z_prefix[c] + eps).
 * Q, O: [B,H,nb*n,d]; S_prefix [B,H,nb,d,d]; z_prefix [B,H,nb,d].
 * With dt == SVLA_BF16 the state enters the matrix cores rounded to bf16. */
svla_status svla_apply(svla_dtype dt, int B, int H, int nb, int n, int d,
                       const void *Q, const float *S_prefix, const float *z_prefix,
                       const svla_rope *rope, float eps, void *O,
                       void *ws, size_t ws_bytes, svla_stream stream);

/* ---- the FFN's temporal convolution, causal across blocks -------------------- */

/* The Mix-FFN's temporal 1-D convolution made causal across blocks (talk, the
 * passage on a causal FFN with temporal convolution: a zero token separates
 * two blocks in training so a block cannot see the next one, and the previous
 * block's last token is cached as the first token of the next block so it can
 * see the previous one; comfyui-wiki model page, the temporal 1-D convolution
 * added to Mix-FFN).  Depthwise, 3 taps over latent frames:
 *   y[t,p,c] = bias[c] + w[c][0] x[t-1,p,c] + w[c][1] x[t,p,c] + w[c][2] x[t+1,p,c]
 * where x[t-1] of the call's first frame is cache_in (zero when NULL), later
 * blocks' first frames read the previous frame (the previous block's last
 * frame), and x[t+1] reads zero for the last frame of every block.
 *   X, Y       [B, T, P, C] contiguous, C fastest, one dtype; T = nb * F frames
 *              in nb blocks of F; P = grid_h * grid_w positions; C % 8 == 0.
 *   w          [C][3] fp32 (taps for t-1, t, t+1); bias [C] fp32 or NULL.
 *   cache_in   [B, P, C] in X's dtype, or NULL: the frame before X's first.
 *   cache_out  [B, P, C] in X's dtype, or NULL: receives X's last frame (the
 *              next call's cache_in; with nb = 0, cache_in or zeros).  It may
 *              equal cache_in (commit in place) but not overlap it otherwise,
 *              and must not overlap X or Y.  Y must not overlap X.
 * A stream of block steps (nb = 1, the cache carried) gives the same Y as
 * one call over all blocks.  One batch's frames and the cache must each stay
 * below 2 GiB.  Errors as elsewhere; overlaps are SVLA_ERR_VALUE. */
svla_status svla_temporal_conv(svla_dtype dt, int B, int nb, int F, int P, int C,
                               const void *X, void *Y, const float *w, const float *bias,
                               const void *cache_in, void *cache_out, svla_stream stream);

/* ---- training: the backward pass ----------------------------------------------- */

/* Gradients of svla_block_causal / svla_block_causal_gated for block-causal
 * training (talk, the causal-training passage: block c cannot see block c+1,
 * so its tokens read only the states of blocks 0 .. c).  Given the forward's
 * inputs and dO = dLoss/dO [B,H,nb*n,d], writes
 *   dQ, dK, dV [B,H,nb*n,d] in the input dtype (required when n > 0);
 *   dg  [B,H,nb] fp32: dLoss/dg[b,h,c] (nullable; with g NULL it is the
 *       gradient with respect to a gate of 1 on every block);
 *   dS0 [B,H,d,d], dz0 [B,H,d] fp32: dLoss/dS0, dLoss/dz0 (nullable, both or
 *       neither; zero when nothing reaches them).
 * The forward's block states are rebuilt from K, V (and S0, z0, g) inside the
 * call; nothing from the forward call is kept.  With num = S_c^T R phi(q),
 * den = phi(q) . z_c + eps: dq = [q > 0] (R^T S_c dnum + dden z_c) with
 * dnum = dO / den, dden = -(dO . O) / den; G_c = sum over block c of
 * (R phi(q)) dnum^T + g_{c+1} G_{c+1} (H_c likewise with dden phi(q)) is the
 * gradient reaching S_c; dv = G_c^T R phi(k), dk = [k > 0] (R^T G_c v + H_c);
 * dg_c = <G_c, S_{c-1}> + <H_c, z_{c-1}>.  The derivative of phi at 0 is 0, and
 * a token whose denominator is 0 passes no gradient.  Sums are fp32 and the
 * gradients are rounded once, to the output dtype; for SVLA_BF16 at d = 32 the
 * products take their fp32 operands as bf16 hi + lo pairs (about 2^-16
 * relative), otherwise they are fp32 products.
 * dt: SVLA_F32 or SVLA_BF16 (SVLA_FP8: SVLA_ERR_UNSUPPORTED); d: 32 or 64
 * (128: SVLA_ERR_UNSUPPORTED).  dQ, dK, dV must not overlap each other or the
 * inputs (SVLA_ERR_VALUE).  Workspace: svla_workspace_size(SVLA_OP_BACKWARD).
 * Launches: state build, export scan, query side, reverse scan, key side. */
svla_status svla_block_causal_backward(svla_dtype dt, int B, int H, int nb, int n, int d,
                                       const void *Q, const void *K, const void *V,
                                       const void *dO, const float *S0, const float *z0,
                                       const float *g, const svla_rope *rope, float eps,
                                       void *dQ, void *dK, void *dV, float *dg,
                                       float *dS0, float *dz0, void *ws, size_t ws_bytes,
                                       svla_stream stream);

/* ---- the 2.0 hybrid's softmax anchors -------------------------------------------- */

/* Softmax attention on the block schedule of the linear layers: the dense
 * softmax "anchor" layers that SANA-Video 2.0 interleaves with its gated linear
 * layers ([2.0 news], the hybrid linear-softmax attention paragraph; [Model
 * page], the 2.0 section), bidirectional inside a block and causal across
 * blocks ([Talk], block-by-block generation).  Queries of nb blocks of n tokens
 * (Q, O [B,H,nb*n,d]) attend Nk >= nb*n keys (K, V [B,H,Nk,d]) whose first
 * Nk - nb*n come before the queries' first block (a KV cache): query i, in
 * block c = i / n, sees keys 0 .. Nk - nb*n + (c+1)*n - 1, and
 *     O_i = sum_j softmax_j(scale * q_i . k_j) v_j.
 * One call over all blocks is Nk = nb*n; a streaming step of block c is nb = 1,
 * Nk = (c+1)*n.  bf16 only (SVLA_ERR_DTYPE otherwise); d = 64 or 128
 * (SVLA_ERR_UNSUPPORTED otherwise); scale > 0 and finite (SVLA_ERR_VALUE; the
 * usual choice is 1/sqrt(d)); O must not overlap Q, K or V (SVLA_ERR_VALUE);
 * one (b,h) slice of K below 2 GiB.  Logits, weights and sums are fp32; O is
 * rounded once to bf16.  No workspace; one kernel on `stream`. */
svla_status svla_softmax_attention(svla_dtype dt, int B, int H, int nb, int n, int Nk, int d,
                                   const void *Q, const void *K, const void *V, void *O,
                                   float scale, svla_stream stream);

/* ---- instrumentation ----------------------------------------------------------- */

/* For benchmarks that time each kernel with HIP events.  While set, every
 * kernel that a call made by this thread launches for slot k (0 = state
 * build, 1 = scan, 2 = apply, 3 = one-launch block step, 4 = temporal
 * convolution, 5 / 6 / 7 = the backward's query side / reverse scan / key side) is launched with the start/stop pair
 * events[2k], events[2k+1], which the runtime records around that kernel's
 * execution (a kernel a call does not need is not launched and leaves its
 * pair alone; pairs past n are not used).  `events` are hipEvent_t handles
 * created by the caller and must stay valid while set; the array is not
 * copied.  Pass NULL (or n = 0) to stop.  Timing adds no other work. */
svla_status svla_set_timing_events(void *const *events, int n);

/* HBM bandwidth probes for a benchmark's ceiling measurement (not part of the
 * method): mode 0 streams `bytes` of src through 16-byte non-temporal loads
 * (sink: `workgroups` unsigned ints, written only in a case that does not
 * occur; required), mode 1 copies src to dst (non-overlapping) the same way.
 * `workgroups` workgroups of 256 threads each take one contiguous range;
 * bytes must be a multiple of workgroups * 16 KiB, each range below 2 GiB,
 * pointers 16-byte aligned.  Launches one kernel on `stream`; allocates
 * nothing.  SVLA_ERR_VALUE (mode, workgroups), _NULL, _SHAPE, _ALIGN, _HIP. */
svla_status svla_hbm_probe(int mode, const void *src, void *dst, size_t bytes,
                           unsigned int *sink, int workgroups, svla_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* SVLA_H */
