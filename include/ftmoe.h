/*
 * ftmoe.h -- C ABI of libftmoe.so: the NVFP4-weight mixture-of-experts layer
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer (FreeToken commit log, page 2: the 288-expert NVFP4 MoE entry, and
 * the entry with 512 routed experts, top-10, plus a gated shared expert; the
 * clamped-SwiGLU entry; the MoE router / shared gate kernels and the
 * top-k router entry (k not a power of two).  FreeToken fork PR #84, page 1: the
 * bullet on #631, the NVFP4 MoE decode GEMV on the per-token path of each layer,
 * and the bullet on #578, NVFP4 prefill experts):
 *
 *   logit[t,e] = sum_h Wr[e,h] x[t,h] (+ bias[e])          router, fp64 sum, one fp32 rounding
 *   ids[t,:]   = top-k experts by (logit desc, index asc)   a NaN logit ranks below every number
 *   w[t,i]     = softmax over the k selected logits          fp32
 *   for each selected expert e (NVFP4 weights, see below):
 *     gate_r = sum_h Wg[r,h] x_h,  up_r = sum_h Wu[r,h] x_h
 *     h_r    = silu(gate_r) * up_r                                       (act 0)
 *            = silu(min(gate_r, gate_max)) * clamp(up_r, -up_absmax, up_absmax)  (act 1)
 *     o_c    = sum_r Wd[c,r] h_r
 *   y[t,c] = bf16( sum_i w[t,i] o_{ids[t,i]}[c]  +  sigmoid(sum_h gs[h] x[t,h]) o_shared[c] )
 *
 * NVFP4 weights: each element is a 4-bit e2m1 code (OCP Microscaling v1.0), each
 * run of 16 consecutive K elements of a row shares one e4m3 scale byte (OCP 8-bit
 * Floating Point), and each tensor (gate, up, down of each expert) has one fp32
 * global scale.  The dequantised weight is fp32(fp32(e2m1 * e4m3) * global).
 *
 * Canonical layout (the input of ft_nvfp4_repack), per bank of n experts with
 * hidden size H and intermediate size I:
 *   w13 codes   u8  [n][2I][H/2]   rows 0..I-1 are gate, rows I..2I-1 are up;
 *                                  byte k/2 of a row holds element k in its low
 *                                  nibble when k is even, in its high nibble when odd
 *   w13 scales  u8  [n][2I][H/16]  e4m3, scale of elements 16j..16j+15 at byte j
 *   w2 codes    u8  [n][H][I/2]
 *   w2 scales   u8  [n][H][I/16]
 *   global      f32 [n][3]         (gate, up, down)
 * The repacked layout that the compute entry points read is private to the
 * library; its sizes come from ft_nvfp4_repacked_bytes.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says host.  The caller
 *    allocates every buffer and keeps it alive until the work enqueued on the
 *    stream has finished; the library keeps no pointer after it returns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every compute call only
 *    enqueues work on it: it never synchronises, never copies between host and
 *    device and never allocates, so it may be captured into a HIP graph.
 *  - Return value: FT_OK, or a negative ft_status; ft_last_error() then holds a
 *    message (thread-local, valid until the next call on the same thread).
 *    Arguments are checked on the host before anything is enqueued; values that
 *    live in device memory (for example ids passed to ft_moe_nvfp4_prefill) are
 *    the caller's responsibility (see ft_moe_nvfp4_prefill for bad ids).
 *  - Every device pointer must be 16-byte aligned; the workspace 256-byte aligned.
 *  - Identical inputs give identical output bits, independent of buffer
 *    addresses, stream and graph replay (no floating-point atomics).
 *  - Supported shapes: hidden % 256 == 0 and hidden <= 8192; inter % 64 == 0 and
 *    inter <= 4096 (shared_inter likewise, or 0); 1 <= top_k <= min(E, 16);
 *    E <= 1024.  Other shapes return FT_EUNSUPPORTED.
 */
#ifndef FTMOE_H
#define FTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FT_ABI_VERSION 1

typedef int32_t ft_status;
#define FT_OK 0
#define FT_EINVAL (-1)        /* null pointer, negative size, inconsistent arguments */
#define FT_EUNSUPPORTED (-2)  /* valid but outside the supported shapes */
#define FT_EWORKSPACE (-3)    /* workspace missing or smaller than ft_moe_workspace_bytes */
#define FT_EHIP (-4)          /* a HIP runtime call failed; the message names it */

typedef struct ft_moe_desc {
    int32_t num_experts;   /* E, routed experts */
    int32_t hidden;        /* H */
    int32_t inter;         /* I, intermediate size of each routed expert */
    int32_t top_k;         /* k */
    int32_t act;           /* 0 = SwiGLU, 1 = clamped SwiGLU */
    float gate_max;        /* act 1: gate is clamped above at gate_max (7.0 in the workloads) */
    float up_absmax;       /* act 1: up is clamped to [-up_absmax, up_absmax] (7.0) */
    int32_t shared_inter;  /* intermediate size of the gated shared expert; 0 = none */
} ft_moe_desc;

/* One repacked NVFP4 expert bank (routed: n = num_experts; shared: n = 1). */
typedef struct ft_nvfp4_experts {
    const uint8_t *w13;        /* repacked gate|up codes */
    const uint8_t *w13_scale;  /* repacked gate|up e4m3 scales */
    const uint8_t *w2;         /* repacked down codes */
    const uint8_t *w2_scale;   /* repacked down e4m3 scales */
    const float *global_scale; /* f32 [n][3]: gate, up, down */
} ft_nvfp4_experts;

/* One repacked block-fp8 expert bank (routed: n = num_experts; shared: n = 1): e4m3
 * weights with one fp32 scale per 128 x 128 block (see ft_fp8_repack). */
typedef struct ft_fp8_experts {
    const uint8_t *w13;       /* repacked gate|up e4m3 codes */
    const float *w13_scale;   /* f32 [n][2I/128][H/128] block scales */
    const uint8_t *w2;        /* repacked down e4m3 codes */
    const float *w2_scale;    /* f32 [n][H/128][I/128] block scales */
} ft_fp8_experts;

/* A KV-cache prefix of one sequence for ft_attn_extend. */
typedef struct ft_kv_cache {
    int32_t format;                 /* 0 bf16, 1 fp8 (e4m3), 2 NVFP4 */
    int32_t prefix;                 /* cached positions (0 = none) */
    const void *k, *v;              /* bf16 [prefix][Hkv][d] | u8 [prefix][Hkv][d] |
                                       e2m1 codes u8 [prefix][Hkv][d/2] (low nibble first) */
    const uint8_t *k_block_scale;   /* NVFP4: e4m3 [prefix][Hkv][d/16]; else unused */
    const uint8_t *v_block_scale;
    float k_scale, v_scale;         /* fp8 / NVFP4: per-tensor scales, positive and finite
                                       (else FT_EINVAL); bf16: unused */
} ft_kv_cache;

/* FT_ABI_VERSION of the library that was loaded. */
int32_t ft_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Host string. */
const char *ft_last_error(void);

/* Makes `device` current and caches its properties (CU count); checks that the
 * one-launch decode kernel can keep a block resident on each CU.  Call once per
 * device before the compute calls, outside stream capture. */
ft_status ft_init(int32_t device);

/* Bytes of repacked part `part` (0 w13 codes, 1 w13 scales, 2 w2 codes,
 * 3 w2 scales) for a bank of n experts of size (hidden, inter).  Returns 0 for
 * invalid arguments. */
size_t ft_nvfp4_repacked_bytes(int32_t hidden, int32_t inter, int32_t n_experts, int32_t part);

/* Load-time layout conversion, from the canonical layout above into the layout
 * the compute entry points read (FreeToken fork PR #84, page 1, bullet on #631:
 * the decode GEMV stops converting layouts per call; here the conversion moves
 * to load time).  Byte-preserving: every code and scale byte is moved, none is
 * changed.  The gate|up tensors stay row-major (one wave reads a row's codes as
 * contiguous 16-byte lanes); the down tensors become K-chunk-major, [n][I/32][H]
 * records of 16 code bytes and [n][I/32][H] records of 2 scale bytes, so that 64
 * lanes reading 64 consecutive output rows read 1 KiB contiguous.
 * Inputs are canonical device buffers; outputs are device buffers of
 * ft_nvfp4_repacked_bytes() bytes each (no overlap with the inputs). */
ft_status ft_nvfp4_repack(int32_t hidden, int32_t inter, int32_t n_experts,
                          const uint8_t *w13, const uint8_t *w13_scale,
                          const uint8_t *w2, const uint8_t *w2_scale,
                          uint8_t *out_w13, uint8_t *out_w13_scale,
                          uint8_t *out_w2, uint8_t *out_w2_scale, void *stream);

/* Workspace bytes needed by ft_moe_route (path 0), ft_moe_nvfp4_decode (path 1)
 * or ft_moe_nvfp4_prefill (path 2) for `tokens` tokens; a workspace sized for T
 * tokens serves every smaller token count of the same path.  Returns 0 for
 * invalid arguments.  Ownership: the caller allocates it (device memory) and
 * zero-fills it once before its first use; every call that returned FT_OK leaves
 * it ready for the next call of the same path (counters are reset by the kernels
 * that use them, never by a memset).  Use one workspace per path, on one device;
 * calls that share a workspace must not run concurrently. */
size_t ft_moe_workspace_bytes(const ft_moe_desc *desc, int64_t tokens, int32_t path);

/* Router only (FreeToken commit log, page 2: the MoE router / shared gate kernels
 * entry and the top-k router entry for k not a power of two): logits with exact fp32 x bf16
 * products summed in fp64 and rounded once to fp32 (from 24 tokens on the fp64
 * MFMA units, split along K below 1024 tokens; the splits summed in a fixed
 * order), top-k (ties to the lower index) and softmax weights of the selected
 * logits.
 *   x         bf16 [T][H]      w_router f32 [E][H]      bias f32 [E] or NULL
 *   topk_ids  i32  [T][k]      topk_w   f32 [T][k]      (outputs, rank order)
 * 0 <= T <= 2^21 (T == 0 enqueues nothing). */
ft_status ft_moe_route(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                       const float *w_router, const float *bias, int32_t *topk_ids,
                       float *topk_w, void *workspace, size_t workspace_bytes, void *stream);

/* The whole layer for decode batches (1 <= T <= 64; FreeToken fork PR #84,
 * page 1, the bullet on #631): routing, the gate|up GEMV with in-register
 * dequantisation and (clamped) SwiGLU, the down GEMV, the weighted combine and
 * the gated shared expert.  T < 8 runs as one persistent kernel; T >= 8 routes,
 * selects and groups the (token, slot) pairs by expert in one persistent kernel
 * (one block per CU, fp64 MFMA router split along K; the top-k and the grouping
 * as in ft_moe_route and ft_moe_nvfp4_prefill) and then runs the grouped kernels
 * of ft_moe_nvfp4_prefill, so each selected expert's weights are read once for
 * all of its tokens.
 *   x bf16 [T][H]; w_router f32 [E][H]; bias f32 [E] or NULL
 *   routed: repacked bank of E experts; shared: repacked bank of 1 expert, or
 *   NULL when desc->shared_inter == 0; shared_gate bf16 [H] (NULL when no shared)
 *   topk_ids_out i32 [T][k], topk_w_out f32 [T][k]: optional side outputs (NULL ok)
 *   y bf16 [T][H] (output) */
ft_status ft_moe_nvfp4_decode(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                              const float *w_router, const float *bias,
                              const ft_nvfp4_experts *routed, const ft_nvfp4_experts *shared,
                              const uint16_t *shared_gate, int32_t *topk_ids_out,
                              float *topk_w_out, uint16_t *y, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Block-fp8 experts, the second routed-expert codec of the 512-expert layer
 * (FreeToken commit log, page 2: the entry with NVFP4 / block-fp8 routed experts and
 * its fp8 scale-bank padding rule).  The pages give no block shape; this library
 * reads it as: one OCP e4m3 byte per weight and one fp32 scale per 128 x 128 block of
 * each [rows][K] matrix, dequantised weight = fp32(e4m3 * scale) (one rounding), no
 * separate global scale.  Canonical layout (the input of ft_fp8_repack):
 *   w13 codes   u8  [n][2I][H]          gate rows 0..I-1, then up rows
 *   w13 scales  f32 [n][2I/128][H/128]
 *   w2 codes    u8  [n][H][I]
 *   w2 scales   f32 [n][H/128][I/128]
 * Needs hidden % 256 == 0 and inter % 128 == 0 (shared_inter likewise).
 * ft_fp8_repacked_bytes: bytes of part 0..3 (codes, scales, codes, scales) of the
 * repacked bank (0 for invalid arguments).  ft_fp8_repack: gate|up codes and every
 * scale are copied; down codes become K-chunk-major [n][I/32][H] records of 32 bytes
 * (64 lanes reading 64 consecutive rows read 2 KiB contiguous). */
size_t ft_fp8_repacked_bytes(int32_t hidden, int32_t inter, int32_t n_experts, int32_t part);
ft_status ft_fp8_repack(int32_t hidden, int32_t inter, int32_t n_experts, const uint8_t *w13,
                        const float *w13_scale, const uint8_t *w2, const float *w2_scale,
                        uint8_t *out_w13, float *out_w13_scale, uint8_t *out_w2,
                        float *out_w2_scale, void *stream);

/* The decode layer (as ft_moe_nvfp4_decode: routing, fused gate|up GEMV with in-register
 * e4m3 -> bf16 conversion and the block scale applied per 32-element chunk, (clamped)
 * SwiGLU, down GEMV, weighted combine, gated shared expert) over block-fp8 banks, for
 * 1 <= tokens <= 7 (the one-launch kernel; 8 or more return FT_EUNSUPPORTED).  The
 * shared expert, when desc->shared_inter > 0, is a block-fp8 bank of one expert.  The
 * workspace is a decode workspace (ft_moe_workspace_bytes, path 1); its give-up status
 * is read with ft_moe_device_status. */
ft_status ft_moe_fp8_decode(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                            const float *w_router, const float *bias, const ft_fp8_experts *routed,
                            const ft_fp8_experts *shared, const uint16_t *shared_gate,
                            int32_t *topk_ids_out, float *topk_w_out, uint16_t *y,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Test export: tensor `tensor` (0 gate, 1 up, 2 down) of expert `expert` of a repacked
 * block-fp8 bank as fp32 [rows][K] (out 16-byte aligned), through the decode kernel's
 * routines: mode 0 decodes codes as its down GEMV does (e4m3 pair -> fp32 pair), mode 1
 * as its gate|up GEMV does (e4m3 pair -> bf16 pair); both multiply by the block scale. */
ft_status ft_fp8_dequant(int32_t hidden, int32_t inter, int32_t n_experts,
                         const ft_fp8_experts *bank, int32_t expert, int32_t tensor, int32_t mode,
                         float *out, void *stream);

/* Per-tensor FP8 W8A8 projection (FreeToken commit log, page 2, the paragraph on
 * row-wise FP8 scaled matrix products: a fused projection stacks parts such as q, k
 * and v along its output rows, each part with its own per-tensor weight scale; it
 * runs as one row-wise-scaled GEMM or, as a fallback, one tensor-wise GEMM per part
 * over its row slice, the parts taken at load time from the run-lengths of the
 * per-row weight scales).
 *   s_x = amax|x| / 448 (fp32, correctly rounded; 1 for x == 0)
 *   xq  = e4m3(x / s_x) (fp32 quotient, round to nearest even)
 *   y   = bf16( s_x * s_w[n] * sum_k xq[m,k] * w[n,k] ), fp32 accumulation
 *   x   bf16 [M][K]; w e4m3 [N][K] row-major; y bf16 [M][N]; K % 64 == 0.
 * ft_fp8_linear_workspace_bytes: device workspace for M x K activations (0 for
 * unsupported sizes); no zero fill needed; calls sharing one must not overlap.
 * ft_fp8_quantize: the activation step alone (codes u8 [M][K] and s_x, device).
 * ft_fp8_linear: the row-wise form, w_scale_rows f32 [N] (device), one GEMM launch.
 * ft_fp8_linear_parts: the per-part form; part_rows (HOST, [n_parts + 1], 0 first,
 * strictly increasing, N last) and part_scales (HOST, [n_parts]); one GEMM launch
 * per part, writing y's columns of that part (row stride N).  Both forms give the
 * same bits for the same per-row scales.
 * ft_fp8_scale_runs: HOST helper for load time: splits a host per-row scale vector
 * into runs of equal bit patterns (part_rows [max_parts + 1], part_scales
 * [max_parts]); returns the number of parts, or -1 (bad arguments, too many runs). */
size_t ft_fp8_linear_workspace_bytes(int64_t M, int64_t K);
ft_status ft_fp8_quantize(int64_t M, int64_t K, const uint16_t *x, uint8_t *xq, float *x_scale,
                          void *workspace, size_t workspace_bytes, void *stream);
ft_status ft_fp8_linear(int64_t M, int64_t N, int64_t K, const uint16_t *x, const uint8_t *w,
                        const float *w_scale_rows, uint16_t *y, void *workspace,
                        size_t workspace_bytes, void *stream);
ft_status ft_fp8_linear_parts(int64_t M, int64_t K, const uint16_t *x, const uint8_t *w,
                              int32_t n_parts, const int64_t *part_rows, const float *part_scales,
                              uint16_t *y, void *workspace, size_t workspace_bytes,
                              void *stream);
int32_t ft_fp8_scale_runs(const float *w_scale_rows, int64_t N, int64_t *part_rows,
                          float *part_scales, int32_t max_parts);

/* Extend attention over a quantised KV cache (FreeToken fork PR #84, page 1, the
 * bullet on the extend-attention kernel of the NVFP4 KV-cache step: the cache loops
 * use a quantised twin of the attention tile with the per-tensor scales on the dot
 * outputs and the softmax normaliser over the unscaled probabilities; the loops over
 * the new tokens stay 16-bit).  For one sequence: n_new query tokens at positions
 * prefix .. prefix + n_new - 1 attend to the cached positions and to the new tokens,
 * key position p visible to query position t iff p <= t and (window == 0 or
 * t - p < window); scores q.k / sqrt(head_dim); query head h reads kv head
 * h / (q_heads / kv_heads).  A cached value is code x tensor scale (fp8) or
 * e2m1 code x e4m3 block scale x tensor scale (NVFP4).
 *   q bf16 [n_new][q_heads][d]; k_new, v_new bf16 [n_new][kv_heads][d];
 *   out bf16 [n_new][q_heads][d]; head_dim 64 or 128. */
ft_status ft_attn_extend(int32_t n_new, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                         int32_t window, const uint16_t *q, const uint16_t *k_new,
                         const uint16_t *v_new, const ft_kv_cache *cache, uint16_t *out,
                         void *stream);

/* ft_moe_nvfp4_decode with the routed experts held in a bank of expert SLOTS
 * (FreeToken fork PR #84, page 1, the interleaved A/B table: the deployment keeps
 * a fixed number of expert slots and counts expert-cache misses per token;
 * FreeToken commit log, page 2: the expert banks plan their residency).
 *   slots     repacked bank of n_slots experts (any n_slots >= 1 for 1..7 tokens;
 *             n_slots <= num_experts for 8..64 tokens, else FT_EUNSUPPORTED)
 *   slot_of   i32 [E] device: the slot holding expert e, or any value outside
 *             [0, n_slots) when expert e is not resident
 *   miss_out  i32 [T][k] device, optional: for each selected place, the expert id
 *             when that expert is not resident, else -1
 * Routing is computed as by ft_moe_nvfp4_decode (topk_ids_out holds expert ids).
 * A selected expert that is not resident contributes nothing to y (the routing
 * weights of the others are not renormalised): the caller sees it in miss_out and
 * may page the expert in and call again.  Other arguments as ft_moe_nvfp4_decode
 * (the workspace is sized by ft_moe_workspace_bytes for path 1). */
ft_status ft_moe_nvfp4_decode_slots(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                                    const float *w_router, const float *bias,
                                    const ft_nvfp4_experts *slots, int32_t n_slots,
                                    const int32_t *slot_of, const ft_nvfp4_experts *shared,
                                    const uint16_t *shared_gate, int32_t *topk_ids_out,
                                    float *topk_w_out, int32_t *miss_out, uint16_t *y,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* The expert part of the layer for prefill chunks (FreeToken fork PR #84,
 * page 1, the bullet on #578), given routes (for example from ft_moe_route):
 * pairs grouped by expert, gate|up and down as grouped bf16 MFMA GEMMs (exact
 * bf16 code x scale tiles, fp32 accumulation, h carried as a bf16 hi + lo pair),
 * combine in slot order.  0 <= T <= 65535.  Ids live in device memory and are not
 * checked on the host; a token whose ids include a value outside [0, E) gets NaN
 * outputs (the kernels never read outside the bank).
 *   x bf16 [T][H]; topk_ids i32 [T][k]; topk_w f32 [T][k]; y bf16 [T][H] (output)
 *   shared / shared_gate as for decode. */
ft_status ft_moe_nvfp4_prefill(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                               const int32_t *topk_ids, const float *topk_w,
                               const ft_nvfp4_experts *routed, const ft_nvfp4_experts *shared,
                               const uint16_t *shared_gate, uint16_t *y, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Status of the device-side waits of ft_moe_nvfp4_decode on this workspace.
 * The one-launch decode path (T < 8) and the routing kernel of a decode batch
 * (T >= 8) run one block per compute unit whose blocks hand values to each other;
 * they therefore need every block resident at once (one per CU: ft_init checks
 * that the device can hold one, and work from other streams that occupies whole
 * CUs breaks the assumption).  Every wait is bounded: a wait
 * that gives up lets the kernel finish, leaves that call's y (and side outputs)
 * invalid, and records why in the workspace.  This call enqueues one tiny kernel
 * that copies the recorded reasons to *status (device int32) and clears them, so
 * the hot call itself never synchronises; read *status after the stream reaches
 * it.  0 = no give-up since the last read; otherwise an OR of 1 (router logits),
 * 2 (shared gate), 4 (intermediate h values), 8 (partial output sums), 16 (the
 * routes of a decode batch, T >= 8, awaited by its grouping).
 * `workspace` is a decode (path 1) workspace; graph-capturable. */
ft_status ft_moe_device_status(void *workspace, size_t workspace_bytes, int32_t *status,
                               void *stream);

/* ft_moe_nvfp4_decode for callers that cannot allocate device memory (code under
 * HIP graph capture that may not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as ft_moe_nvfp4_decode for
 * 1 <= tokens <= 7 (the one-launch kernel), without a workspace: the call uses a
 * fixed 4 MiB array of device memory that the library holds on each GPU it runs
 * on until the process ends, located and zero-filled by ft_init (call it first on
 * each device; otherwise FT_EINVAL).  Shapes whose decode workspace
 * (ft_moe_workspace_bytes, path 1) exceeds 4 MiB return FT_EWORKSPACE; 8 or more
 * tokens return FT_EUNSUPPORTED.  It allocates nothing and only enqueues work on
 * `stream` (capturable).  Every call on one GPU shares that array and it keeps
 * the last call's contents: calls on one GPU must not overlap (two streams
 * running this call at once race).  status: optional device int32 that receives
 * what ft_moe_device_status would report for the call's waits (NULL = not read). */
ft_status ft_moe_nvfp4_decode_noalloc(const ft_moe_desc *desc, int64_t tokens, const uint16_t *x,
                                      const float *w_router, const float *bias,
                                      const ft_nvfp4_experts *routed,
                                      const ft_nvfp4_experts *shared,
                                      const uint16_t *shared_gate, int32_t *topk_ids_out,
                                      float *topk_w_out, uint16_t *y, int32_t *status,
                                      void *stream);

/* Test and diagnostic hook: the number of polls after which a device-side wait of
 * ft_moe_nvfp4_decode gives up (0 restores the default, about one second).  It is
 * process-wide and applies to calls enqueued afterwards.  A call in which one wait
 * gives up makes its other waits stop within 16 polls. */
ft_status ft_set_wait_limit(int32_t polls);

/* Test export: dequantise tensor `tensor` (0 gate [I][H], 1 up [I][H],
 * 2 down [H][I]) of expert `expert` of a repacked bank into a row-major matrix
 * `out` (16-byte aligned), through the device routines the compute kernels use.
 * `inter` is the bank's intermediate size.  out_dtype selects the routine:
 *   0  fp32 code x scale x global (the codes decoded as the one-launch decode
 *      kernel's down GEMV decodes them);
 *   1  the value of 0 rounded to bf16 (nearest-even);
 *   2  bf16 code x scale WITHOUT the global scale, exactly as the grouped decode
 *      and prefill kernels build their bf16 MFMA tiles (every such product is
 *      exact in bf16);
 *   3  fp32 code x scale x global with the codes decoded as the one-launch decode
 *      kernel's gate|up GEMV decodes them (e2m1 pair -> bf16 pair);
 *   4  fp16 code x scale WITHOUT the global scale, exactly as the grouped and
 *      prefill down GEMMs build their fp16 MFMA tiles when h travels in fp16
 *      (every such product is exact in fp16: at most 6 significant bits, and
 *      within [2^-10, 2688] in magnitude, or zero).
 * Every mode is exact: 0 and 3 equal one fp32 rounding of code x scale x global. */
ft_status ft_nvfp4_dequant(int32_t hidden, int32_t inter, int32_t n_experts,
                           const ft_nvfp4_experts *bank, int32_t expert, int32_t tensor,
                           int32_t out_dtype, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FTMOE_H */
