/*
 * pq.h — C ABI of the MI355X (gfx950) quantized-weight decode library.
 *
 * The library implements the weight-streaming hot path of batch-1 and small-M
 * (speculative-verify) decode through quantized MoE expert weights:
 *
 *   - Sionic AI blog, "GPU 커널부터 새로 짜서 GLM-5.2 속도 10배 올리기"
 *     (GLM-5.2 made ten times faster by rewriting the GPU kernels), cited
 *     below as [Sionic]: intro (decode streams every active weight from HBM
 *     once, so it is bandwidth bound), §1 (a batch-1 gate_up launches too few
 *     blocks; live FP8 activation quantisation must overlap the weight loads;
 *     split-K across the chip), §2 (one scale per K block must not stall the
 *     load pipeline), §4 (quantisation fused into the GEMM, few kernels),
 *     §5-6 (one weight read serves several verified tokens).
 *   - aiwitness post "GLM 5.3 Flash Q4 @ 60tps / 550tps on M3 Ultra" ([M3]):
 *     Q4 weight-streaming decode; merging small kernels into few dispatches.
 *   - rbeckner.com "Qwen 3.8-27B M1 Ultra에서 ..." ([M1]): a 256-expert MoE is
 *     dispatch bound when each expert op is its own launch.
 *
 * Conventions for every call:
 *   - Data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *     16-byte aligned, contiguous, row-major.  bf16 and fp16 values are passed
 *     as their 16-bit patterns (uint16_t).  FP8 is OCP E4M3FN (max 448).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Every compute call is asynchronous on that stream.
 *   - The caller owns all buffers (inputs, outputs, workspace).  Outside of
 *     pq_workspace_init the library allocates nothing and keeps no per-call
 *     state; distinct workspaces may be used from different threads.  One
 *     workspace must not be used by two calls that can overlap in time.  The
 *     one exception: the first pq_gemv_q4_group call on a device that makes
 *     two launches or more creates one stream and two events for it, kept
 *     until the process ends.
 *   - Arguments are validated on the host before anything is launched.  On a
 *     validation failure the call returns a negative pq_status, launches
 *     nothing and leaves every output untouched.  A failing HIP launch returns
 *     PQ_ERR_HIP and the HIP error code is kept per thread
 *     (pq_last_hip_error).  Errors raised while a kernel runs (a bad expert id
 *     in device memory, the spin-wait watchdog) are recorded in the workspace
 *     and reported by pq_workspace_check.
 *   - Workspaces must be zeroed once with pq_workspace_init before first use.
 *     Kernels leave every counter they touch at zero when they finish, so no
 *     per-call clearing is needed.
 */
#ifndef PQ_H
#define PQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PQ_OK = 0,
  PQ_ERR_NULL = -1,        /* a required pointer is NULL                         */
  PQ_ERR_SHAPE = -2,       /* a size is out of range or not a required multiple  */
  PQ_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned                   */
  PQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than *_workspace()    */
  PQ_ERR_UNSUPPORTED = -5, /* the current device is not gfx950, or no device     */
  PQ_ERR_HIP = -6,         /* a HIP runtime call failed (see pq_last_hip_error)  */
  PQ_ERR_TIMEOUT = -7,     /* a kernel's bounded spin-wait gave up (workspace)   */
  PQ_ERR_BAD_EXPERT = -8,  /* a top-k expert id in device memory was out of range */
  PQ_ERR_SCRATCH = -9      /* the call needs more than the static scratch holds  */
} pq_status;

typedef enum {
  PQ_EPI_NONE = 0,
  /* N = 2*Nh weight rows, rows [0,Nh) gate and [Nh,N) up; the output is
   * h[m,i] = silu(gate[m,i]) * up[m,i], bf16 [M,Nh]  (fused gate_up epilogue) */
  PQ_EPI_SILU_MUL = 1
} pq_epilogue;

/* ------------------------------------------------------------------------- */
/* Block quantisers (weight preparation and the live activation rule).        */
/* ------------------------------------------------------------------------- */

/* FP8 block quantisation of `rows` rows of K values, one fp32 scale per 128
 * consecutive values of a row ([Sionic] §1 live FP8 activation quantisation;
 * §2 one scale per K block).  For every block: s = fp32(amax / 448) by IEEE
 * division (s = 1 if amax = 0), code = E4M3(fp32(v / s)) rounded to nearest
 * even with saturation to +-448; NaN -> 0x7F.
 *   in      : bf16 [rows,K] if in_is_f32 == 0, fp32 [rows,K] otherwise
 *   codes   : uint8 [rows,K] (output)       scales : fp32 [rows,K/128] (output)
 * Constraints: rows >= 1, K >= 128, K % 128 == 0.  Inputs must be finite. */
int pq_quantize_fp8(const void* in, int in_is_f32, int rows, int K,
                    uint8_t* codes, float* scales, void* stream);

/* Symmetric int4 quantisation with one fp16 scale per 32 consecutive values
 * of a row ([M3] Q4 weight-streaming decode).  s = fp16_rne(fp32(amax / 7)),
 * q = clamp(rne(fp32(w / fp32(s))), -8, 7), q = 0 where s == 0; stored as
 * offset-binary nibbles u = q + 8, low nibble = even k.
 *   w      : fp32 [N,K]           packed : uint8 [N,K/2] (output)
 *   scales : fp16 [N,K/32] (output)
 * Constraints: N >= 1, K >= 32, K % 32 == 0.  Inputs must be finite. */
int pq_quantize_q4(const float* w, int N, int K, uint8_t* packed, uint16_t* scales,
                   void* stream);

/* ------------------------------------------------------------------------- */
/* Block-scaled FP8 weight-streaming GEMV / skinny GEMM with live activation   */
/* quantisation fused in ([Sionic] §1 and §4; §2 scales per K block).         */
/* ------------------------------------------------------------------------- */

/* Workspace bytes pq_gemv_fp8 needs for this shape on the current device:
 * 0 where the vector kernel runs (a row's K range cut between waves is
 * reduced on chip), else the arrival counters and partial sums of the
 * matrix-core kernel; 0 for invalid shapes (pq_gemv_fp8 then reports the
 * error). */
size_t pq_gemv_fp8_workspace(int M, int K, int N, int epi);

/* y = epi(bf16( sum_b s_x[m,b] s_w[n,b] sum_{k in b} q_x[m,k] q_w[n,k] ))
 * where (q_x, s_x) is the live FP8 quantisation of x (rule of
 * pq_quantize_fp8), accumulated in fp32.
 *   x       : bf16 [M,K]                  w : E4M3 [N,K]   w_scale : fp32 [N,K/128]
 *   y       : bf16 [M,N] (PQ_EPI_NONE) or bf16 [M,N/2] (PQ_EPI_SILU_MUL)
 *   xq_dbg  : nullable, E4M3 [M,K]  — the quantised activation codes
 *   xs_dbg  : nullable, fp32 [M,K/128] — the activation scales
 *   ws, ws_bytes : device workspace of pq_gemv_fp8_workspace() bytes, set up
 *            once by pq_workspace_init (may be NULL / 0 when that is 0);
 *            too small: PQ_ERR_WORKSPACE.
 * Constraints: 1 <= M <= 8, K % 128 == 0, 128 <= K <= 16384, N >= 1,
 * N*K < 2^31, N even under PQ_EPI_SILU_MUL; PQ_ERR_SHAPE otherwise.
 * Two kernels: a vector kernel (each output row computed by one block) and,
 * for M >= 3 on weight matrices of at least 128 MB, a matrix-core kernel
 * (v_mfma_f32_16x16x128_f8f6f4 per 128-wide K block, tiles of 16 rows split
 * over the whole grid).  In either kernel an output's bits depend on the
 * shape and the device's CU count only (not on the other tokens); the two
 * kernels round differently.  PQ_FP8_PATH=valu|mfma forces one kernel;
 * PQ_BLOCKS_PER_CU (default 1) sets the number of blocks per CU. */
int pq_gemv_fp8(const uint16_t* x, int M, int K,
                const uint8_t* w, const float* w_scale, int N,
                int epi, uint16_t* y,
                uint8_t* xq_dbg, float* xs_dbg,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Prefill / large-M block-scaled FP8 GEMM on the matrix cores ([M3]: prefill */
/* reuses each prepared weight for many tokens).                              */
/* ------------------------------------------------------------------------- */

/* Workspace bytes pq_gemm_fp8 needs: the data-region offset of the shared
 * workspace layout plus M*K + 4*M*K/128 bytes (rounded up) for the quantised
 * activation; 0 for invalid shapes. */
size_t pq_gemm_fp8_workspace(int M, int K, int N, int epi);

/* The contraction of pq_gemv_fp8 for any M >= 1 (no upper bound):
 *   y = epi(bf16( sum_b s_x[m,b] s_w[n,b] sum_{k in b} q_x[m,k] q_w[n,k] ))
 * Two launches on `stream`: the live FP8 quantisation of x (the rule of
 * pq_quantize_fp8) into the workspace's data region, then the GEMM
 * (v_mfma_f32_16x16x128_f8f6f4 per 128-wide K block, 128 x 128 tiles, both
 * block scales applied per K block in fp32).
 *   x : bf16 [M,K]     w : E4M3 [N,K]     w_scale : fp32 [N,K/128]
 *   y : bf16 [M,N] (PQ_EPI_NONE) or [M,N/2] (PQ_EPI_SILU_MUL, gate rows then
 *       up rows as in pq_gemv_fp8)
 *   ws, ws_bytes : workspace of pq_gemm_fp8_workspace() bytes (the counters
 *       and the zeroed region of the other entry points are not touched, so
 *       the workspace may be theirs); too small: PQ_ERR_WORKSPACE.
 * Constraints: K % 128 == 0, N >= 1, N*K < 2^31, M*K < 2^31, N even under
 * PQ_EPI_SILU_MUL; PQ_ERR_SHAPE otherwise.  An output's bits do not depend on
 * the other tokens of the call. */
int pq_gemm_fp8(const uint16_t* x, int M, int K,
                const uint8_t* w, const float* w_scale, int N,
                int epi, uint16_t* y,
                void* ws, size_t ws_bytes, void* stream);

/* The GEMM launch of pq_gemm_fp8 alone, on an activation already quantised by
 * the rule of pq_quantize_fp8 (for a caller whose previous step produced it):
 *   xq : E4M3 [M,K]     xs : fp32 [M,K/128]
 * Other arguments, constraints and results as pq_gemm_fp8; no workspace. */
int pq_gemm_fp8_prequant(const uint8_t* xq, const float* xs, int M, int K,
                         const uint8_t* w, const float* w_scale, int N,
                         int epi, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------- */
/* int4 g32 weight-streaming GEMV (W4A16): [M3] Q4 decode.                    */
/* ------------------------------------------------------------------------- */

/* Workspace bytes pq_gemv_q4 needs for this shape on the current device
 * (arrival counters and the partial sums of row tiles cut between waves);
 * 0 when none is needed, and 0 for invalid shapes (pq_gemv_q4 then reports
 * the error). */
size_t pq_gemv_q4_workspace(int M, int K, int N, int epi);

/* y = epi(bf16( sum_g s[n,g] sum_{k in g} x[m,k] q[n,k] )), fp32 accumulation.
 *   x : bf16 [M,K]    w : nibbles [N,K/2] (layout of pq_quantize_q4)
 *   w_scale : fp16 [N,K/32]    y : bf16 [M,N] or [M,N/2] under PQ_EPI_SILU_MUL
 *   ws : device workspace of ws_bytes >= pq_gemv_q4_workspace(...) (may be
 *        NULL when that is 0), zeroed once by pq_workspace_init; calls that
 *        share a workspace must be ordered (one stream).
 * Constraints: 1 <= M <= 8, K % 32 == 0, K >= 32, N >= 1, N even under
 * PQ_EPI_SILU_MUL, N*K/2 < 2^31, and M*K <= 69632 (the bf16 activation and
 * its staging live in one CU's LDS; e.g. K = 17408 at M <= 4, K = 8704 at
 * M = 8); PQ_ERR_SHAPE otherwise.
 * With K % 256 == 0, M >= 5 (and M == 4 when (N or N/2 under SiLU) * K >=
 * 48 Mi) runs on the matrix cores (bf16 MFMA on unpacked nibbles), everything
 * else on the vector units; PQ_Q4_PATH=valu or =mfma
 * forces one kernel (mfma only where K % 256 == 0).  For a given kernel the
 * output bits depend on the shape and the device's CU count only (not on M
 * or on other rows); PQ_BLOCKS_PER_CU (default 1) sets the blocks per CU. */
int pq_gemv_q4(const uint16_t* x, int M, int K,
               const uint8_t* w, const uint16_t* w_scale, int N,
               int epi, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* One int4 linear of a grouped call (the arguments of pq_gemv_q4). */
typedef struct {
  const uint16_t* x;        /* bf16 [M,K]                                   */
  const uint8_t* w;         /* nibbles [N,K/2] (layout of pq_quantize_q4)   */
  const uint16_t* w_scale;  /* fp16 [N,K/32]                                */
  uint16_t* y;              /* bf16 [M,N], or [M,N/2] under PQ_EPI_SILU_MUL */
  int K, N, epi;
} pq_q4_linear;

/* Several independent int4 g32 GEMVs, all with M tokens, in as few launches
 * as possible ([M3]: merging the small kernels of a decode step raised it from
 * 59% to 81% of measured bandwidth): linears[i] computes exactly what
 * pq_gemv_q4 computes for those arguments on its vector kernel, and every
 * output bit equals that call's (each linear's work is split over the grid
 * and the waves as if it ran alone; it does not depend on the other linears
 * of the call, nor on M).  The linears are packed in order into launches of
 * at most 12 whose activations (M*K*2.125 bytes each, plus partial sums) fit
 * one CU's 160 KB of LDS; each launch streams all of its linears' weights
 * back to back from one persistent grid, so start-up and ring fill are paid
 * once per launch instead of once per linear.
 *   linears : host array of n descriptors (device pointers inside)
 *   launches: nullable host int; receives the number of kernel launches made
 * Constraints per linear as pq_gemv_q4 (PQ_ERR_SHAPE etc.; nothing is
 * launched if any linear is invalid); n = 0 is a no-op.  No workspace.
 * The outputs must not overlap any input of the same call.  When the call
 * makes two launches or more and no two outputs overlap, the launches
 * alternate between `stream` and a second stream of the device, forked from
 * `stream` at the call and joined back into it at the end, so that a launch
 * starts on the CUs the previous one frees while its last blocks still run;
 * work queued on `stream` after the call waits for all of it.  With
 * overlapping outputs, or PQ_Q4_STREAMS=1, every launch goes to `stream` in
 * order (the later linear's values win). */
int pq_gemv_q4_group(const pq_q4_linear* linears, int n, int M, int* launches, void* stream);

/* ------------------------------------------------------------------------- */
/* Routed MoE decode layer in ONE kernel launch ([Sionic] intro, §4, §5;      */
/* [M1] dispatch-bound MoE; [M3] merging small kernels).                      */
/* ------------------------------------------------------------------------- */

size_t moe_decode_layer_workspace(int M, int H, int I, int E, int top_k);

/* For each token m (1 <= M <= 8):
 *   route  : if router_logits != NULL, take the top_k experts of the fp32
 *            logits [M,E] in descending order (ties to the lower id) and
 *            softmax weights over the selected logits; they are WRITTEN to
 *            topk_ids / topk_w.  If router_logits == NULL, topk_ids int32
 *            [M,top_k] and topk_w fp32 [M,top_k] are READ as inputs.
 *   per slot j with expert e:
 *            h  = silu(gate_e(q(x_m))) * up_e(q(x_m))      -> bf16 [I]
 *            y  = down_e(q(h))                             fp32 [H]
 *   out[m] = bf16( sum_j w[m,j] * y_j ), j in slot order.
 *   q(.) is the live FP8 quantisation of pq_quantize_fp8.  Every distinct
 *   expert of the call is streamed from HBM once for all tokens routed to it.
 *   x   : bf16 [M,H]
 *   w13 : E4M3 [E,2I,H] (gate rows then up rows)   s13 : fp32 [E,2I,H/128]
 *   w2  : E4M3 [E,H,I]                              s2  : fp32 [E,H,I/128]
 *   out : bf16 [M,H]
 *   h_dbg, hq_dbg, hs_dbg : nullable bf16 [M,top_k,I], E4M3 [M,top_k,I],
 *            fp32 [M,top_k,I/128] — the intermediate h and its quantisation.
 *   ws  : workspace of ws_bytes >= moe_decode_layer_workspace(...)
 * Constraints: 1 <= M <= 8, 1 <= top_k <= 8, top_k <= E <= 1024,
 * H % 128 == 0, I % 128 == 0, 128 <= H <= 16384, 128 <= I <= 16384.
 * Router logits must be finite.  The kernel needs the whole GPU while it runs:
 * its blocks (one per CU) wait on each other, so every block must be resident
 * at once.  Another kernel running concurrently on the device can keep a block
 * from starting; the waits are bounded, and a wait that gives up records
 * PQ_ERR_TIMEOUT in the workspace.  The outputs of a call are therefore
 * defined only if pq_workspace_check on its workspace returns PQ_OK (callers
 * that cannot guarantee an idle device check it, or set
 * PQ_MOE_LAUNCH=cooperative, which makes the runtime guarantee co-residency or
 * refuse the launch with PQ_ERR_HIP).
 * Two kernels implement the call with bitwise equal results: for M = 1 one
 * whose blocks start the down projection once every h row of the call is
 * there (a grid-wide barrier on the h values themselves), for M >= 2 one that
 * starts each union entry's down rows once that entry's h is there (the
 * environment variable PQ_MOE_PATH=barrier|stream forces one;
 * PQ_MOE_SCALES=step makes the first load every gate_up step's block scales
 * with its weights instead of once per h row through LDS, with equal bits).
 * The workspace (zeroed once by pq_workspace_init) may be shared with the
 * other entry points; the call leaves its counters and its h exchange region
 * at zero, as it found them. */
int moe_decode_layer(const uint16_t* x, int M, int H,
                     const float* router_logits,
                     int32_t* topk_ids, float* topk_w,
                     int E, int top_k, int I,
                     const uint8_t* w13, const float* s13,
                     const uint8_t* w2, const float* s2,
                     uint16_t* out,
                     uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg,
                     void* ws, size_t ws_bytes, void* stream);

/* Which kernel and LDS layout moe_decode_layer / moe_decode_layer_ex use for
 * a call of this shape on the current device (the same rule, including the
 * PQ_MOE_PATH override): *kernel = 0 for the kernel with a grid-wide barrier
 * before the down projection, 1 for the one without; *alias = 1 when the
 * re-quantised h reuses the LDS region of the quantised x (always in kernel 0,
 * which stages h once every wave of the block is past gate_up; in kernel 1
 * when x, h and the output
 * partials do not fit side by side, and h is then staged only once every
 * wave of the block is past gate_up);
 * *lds_bytes = the dynamic LDS per block.  shared: 1 with a shared expert.
 * Returns PQ_OK, or the status the call itself would return for this shape
 * (PQ_ERR_SHAPE, PQ_ERR_UNSUPPORTED without a gfx950 device); PQ_ERR_NULL if
 * an output pointer is NULL.  Host pointers; launches nothing. */
int moe_decode_layer_config(int M, int H, int I, int E, int top_k, int shared,
                            int* kernel, int* alias, size_t* lds_bytes);

/* The same layer with the steps either side of it in the launch ([CMP], on
 * the 3.05bpw quality: the router kept at native precision, shared experts
 * beside the routed ones):
 *   router_w : nullable bf16 [E,H].  When given, the router GEMV runs in the
 *            launch: l[m,e] = sum_k x[m,k] router_w[e,k] (bf16 products, fp32
 *            accumulation), each block computing a slice of the rows and
 *            publishing it through the workspace; routing then follows
 *            moe_decode_layer's rule on these logits, which are written to
 *            router_logits (nullable, fp32 [M,E]) and the ids and weights to
 *            topk_ids / topk_w.  When router_w is NULL, router_logits and
 *            topk_ids / topk_w mean what they mean in moe_decode_layer.
 *   sh_w13, sh_s13, sh_w2, sh_s2 : a shared expert with the routed experts'
 *            shapes ([2I,H], [2I,H/128], [H,I], [H,I/128]), all four or none
 *            (else PQ_ERR_NULL).  Every token runs it like a routed slot and
 *            its output is added with weight 1 after the routed slots:
 *            out[m] = bf16( sum_j w[m,j] y_j + y_shared ).  Its weights are
 *            streamed first, while the routing is still being decided.
 *   h_dbg, hq_dbg, hs_dbg : nullable [M*top_k + M*sh, I] (and [.., I/128]):
 *            the (token, slot) pairs, then the shared expert's pair per token.
 * Everything else as moe_decode_layer (which is this call with router_w and
 * the shared expert NULL).  The same workspace size serves both. */
int moe_decode_layer_ex(const uint16_t* x, int M, int H,
                        const uint16_t* router_w, float* router_logits,
                        int32_t* topk_ids, float* topk_w,
                        int E, int top_k, int I,
                        const uint8_t* w13, const float* s13,
                        const uint8_t* w2, const float* s2,
                        const uint8_t* sh_w13, const float* sh_s13,
                        const uint8_t* sh_w2, const float* sh_s2,
                        uint16_t* out,
                        uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg,
                        void* ws, size_t ws_bytes, void* stream);

/* Allocation-free form of moe_decode_layer_ex, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and constraints as
 * moe_decode_layer_ex, except:
 *   - there is no workspace argument: the layer's workspace is a static
 *     device array inside the library (4 MiB, one copy per GPU the library
 *     runs on, held until the process ends; the first call on a device looks
 *     it up and zeroes it with one extra kernel launch on `stream`).  A call
 *     whose layer needs more (moe_decode_layer_workspace() > 4 MiB, e.g.
 *     M = 8, top_k = 8 at I >= 14208) returns PQ_ERR_SCRATCH and launches
 *     nothing.  The call allocates nothing (no hipMalloc, no allocating
 *     library routine).
 *   - every call on one GPU shares that GPU's array: calls that can overlap
 *     in time on one GPU (other streams, other threads) race and must not be
 *     issued; calls ordered on one stream are safe (each leaves the array's
 *     counters and exchange regions at zero, as the workspace form does).
 *   - status: nullable device int32.  When given, the kernel writes the call's
 *     device-side status there as it ends (PQ_OK, PQ_ERR_TIMEOUT or
 *     PQ_ERR_BAD_EXPERT) and clears the record; a status recorded by a call
 *     given NULL stays until a later call with a status pointer reports it.
 *     16-byte aligned.
 * Host-side validation errors are returned as by moe_decode_layer_ex. */
int moe_decode_layer_noalloc(const uint16_t* x, int M, int H,
                             const uint16_t* router_w, float* router_logits,
                             int32_t* topk_ids, float* topk_w,
                             int E, int top_k, int I,
                             const uint8_t* w13, const float* s13,
                             const uint8_t* w2, const float* s2,
                             const uint8_t* sh_w13, const float* sh_s13,
                             const uint8_t* sh_w2, const float* sh_s2,
                             uint16_t* out,
                             uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg,
                             int32_t* status, void* stream);

/* ------------------------------------------------------------------------- */
/* Workspace and error helpers.                                               */
/* ------------------------------------------------------------------------- */

/* Zero a workspace (asynchronously on `stream`); call once per allocation. */
int pq_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Synchronise `stream` and return the error recorded in the workspace by a
 * kernel (PQ_OK, PQ_ERR_TIMEOUT or PQ_ERR_BAD_EXPERT); the record is cleared. */
int pq_workspace_check(void* ws, void* stream);

/* Human-readable name of a pq_status. */
const char* pq_strerror(int status);

/* HIP error code of the last PQ_ERR_HIP returned on the calling thread. */
int pq_last_hip_error(void);

/* Kernel launches one call of the named entry point makes ("pq_gemm_fp8": 2,
 * the activation quantisation and the GEMM; every other compute entry point:
 * 1, including the whole MoE layer; moe_decode_layer_noalloc adds one
 * zeroing launch on the first call on each device).  PQ_ERR_NULL for NULL,
 * PQ_ERR_UNSUPPORTED for a name that is not a compute entry point. */
int pq_launches_per_call(const char* entry_point);

/* Measurement helper: stream `bytes` of device memory at `src` through the
 * load path of the weight streams (128-bit non-temporal loads, one persistent
 * block per CU, a contiguous share each) and store a checksum per wave into
 * `sink` (device, 16-byte aligned, at least 65536 bytes).  Timing a call
 * gives the achievable HBM read bandwidth that the kernels' roofline fraction
 * can be compared with.  bytes % 16 == 0; a CU's share must stay below 2 GB
 * (PQ_ERR_SHAPE).  Asynchronous on `stream`. */
int pq_stream_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ_H */
