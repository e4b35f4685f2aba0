/*
 * fmlp.h -- C ABI of the fused transformer feed-forward library for AMD
 * MI355X (CDNA4, gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 *  Data:       all matrices are dense, row-major and contiguous.  Weights are
 *              stored [out, in] as nn.Linear stores them, and are read as
 *              stored: the GEMM walks both operands along K, so no transpose
 *              copy ever runs ("Profiling in PyTorch (Part 2): From nn.Linear
 *              to a Fused MLP", section "Where did the transpose go? Kernel
 *              layouts and pre-ops": a transpose only rewrites strides and the
 *              GEMM variant that reads the weight in transposed order is picked).
 *              Leading dims of activations are flattened by the caller:
 *              M = batch * seq (same page, section "Why are there two kinds of
 *              GEMM kernels?").
 *  Types:      activations, weights, biases and outputs are bf16, passed as raw
 *              16-bit patterns (fmlp_bf16).  Accumulation is fp32; the output is
 *              rounded to bf16 round-to-nearest-even.  Hidden activations that
 *              feed a second GEMM (h, m) are rounded to bf16 once.
 *  Pointers:   device pointers (hipMalloc / torch CUDA tensors) on the current
 *              HIP device, 16-byte aligned.  The caller owns every buffer,
 *              including outputs and workspaces; the library never allocates
 *              on a call and keeps no pointer after it returns.  Outputs must
 *              not alias inputs.  With no tokens (M or T == 0) the token-sized
 *              buffers (activations, outputs, routes) may be NULL: nothing is
 *              read or written; weights are still checked.
 *  Shapes:     every inner dimension (K, H, N, D) must be a positive multiple
 *              of 8 (16-byte rows), the analogue of the "align8" GEMM variants
 *              named on the page above, and below 2^22 (kernels address a
 *              256-row tile of an operand with 32-bit byte offsets); the token
 *              count M (or T) may be any value >= 0 below 2^31 (M == 0 is a
 *              no-op).
 *  Streams:    fmlp_stream is a hipStream_t (NULL = the null stream).  Every
 *              call only enqueues work on that stream and returns; FMLP_OK means
 *              "enqueued".  Device faults surface at the caller's next sync.
 *  Errors:     a call validates every argument before it enqueues anything; on
 *              an error nothing is enqueued and the outputs are untouched.  A
 *              failed launch returns FMLP_E_HIP.  fmlp_last_error() gives a
 *              thread-local detail string for the last failing call.
 *  Threads:    calls are thread-safe.  Calls that share a workspace must be
 *              ordered on one stream.
 */
#ifndef FMLP_H_
#define FMLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t fmlp_bf16;  /* raw bf16 bit pattern */
typedef void* fmlp_stream;   /* a hipStream_t */

typedef enum {
  FMLP_ACT_NONE = 0,
  FMLP_ACT_GELU_ERF = 1,   /* exact GELU  z*Phi(z) */
  FMLP_ACT_GELU_TANH = 2,  /* z/2 * (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
  FMLP_ACT_RELU = 3,       /* max(z, 0): the two-layer MLP of ainews.cool "PyTorch fused
                              MLP efficiency", section "technical deep dive" */
  FMLP_ACT_SILU = 4        /* z * sigmoid(z) (swish); as a gate: SwiGLU */
} fmlp_act;

typedef enum {
  FMLP_OK = 0,
  FMLP_E_NULL = 1,       /* a required pointer is NULL */
  FMLP_E_SHAPE = 2,      /* a dimension is negative/zero or too large */
  FMLP_E_ALIGN = 3,      /* an inner dim is not a multiple of 8, or a pointer is not 16-B aligned */
  FMLP_E_ARG = 4,        /* bad enum / top_k / expert count / path */
  FMLP_E_WORKSPACE = 5,  /* workspace NULL or smaller than the *_workspace_size() value */
  FMLP_E_DEVICE = 6,     /* no usable gfx950 device current */
  FMLP_E_HIP = 7         /* a HIP launch failed; see fmlp_last_error() */
} fmlp_status;

/*
 * y[M,N] = act(x[M,K] . W[N,K]^T + b[N])
 *
 * One nn.Linear forward with its epilogue: bias add and activation run on the
 * fp32 accumulator in registers, and only the final tile is written to HBM
 * ("Profiling in PyTorch (Part 2)", sections "From matmul-add to Linear" and
 * "Why are there no separate mul and add kernels?").  b may be NULL (no bias;
 * the page's bias-free Linears).  act is an fmlp_act.  Exactly one kernel
 * launch.  No workspace.
 */
fmlp_status fmlp_linear(const fmlp_bf16* x, const fmlp_bf16* W, const fmlp_bf16* b, int act,
                        int64_t M, int64_t K, int64_t N, fmlp_bf16* y, fmlp_stream stream);

/*
 * y[M,N] = act(x[M,K] . W1[H,K]^T + b1[H]) . W2[N,H]^T + b2[N]
 *
 * The two-layer MLP with the activation between the layers only (ainews.cool
 * "PyTorch fused MLP efficiency", section "technical deep dive": W1*X+b1,
 * activation, W2*(.)+b2).  b1 and/or b2 may be NULL.  The hidden activation h
 * is rounded to bf16 once before the second GEMM.
 * Paths (chosen from the shape): M <= 16: one persistent decode launch;
 * K, H, N <= 128: one fused small-MLP launch; otherwise two GEMM launches with
 * h in the workspace.  workspace must hold fmlp_mlp2_workspace_size(M,K,H,N)
 * bytes (it may be NULL when that size is 0).  Its first 8192 bytes are the
 * decode kernel's header: 32-bit word 0 (fmlp_decode_generation_offset) is a
 * generation that each one-launch decode call advances by exactly one, word 2
 * (fmlp_decode_timeout_offset) counts device-wide barrier waits that gave up,
 * and the rest holds per-block arrival flags.  Zero the header once before the
 * first call (the timeout count starts there).  After that nothing else is
 * required: every launch tags what it publishes (h words, flags) with an epoch
 * mixed from the next generation and a per-launch salt, so neither a header
 * zeroed again between calls, nor recycled memory, nor words left by an
 * earlier call are ever taken for this call's h.  The same workspace may be
 * shared, in stream order, by every call of this header (the FP8 calls,
 * fmlp_geglu/fmlp_glu and the backward calls keep their data after the
 * 8192-byte header too; the one-token FP8 two-layer launch advances the same
 * generation).
 * The one-launch decode form needs every block resident at once: its grid is
 * at most one block per CU, so on a device not shared with long-running work
 * it always is.  A barrier wait that gives up (after 2^20 polls of the flags)
 * leaves y wrong; it is counted in word 2, which a caller checks after a sync.
 */
fmlp_status fmlp_mlp2(const fmlp_bf16* x, const fmlp_bf16* W1, const fmlp_bf16* b1,
                      const fmlp_bf16* W2, const fmlp_bf16* b2, int act,
                      int64_t M, int64_t K, int64_t H, int64_t N,
                      fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_mlp2_workspace_size(int64_t M, int64_t K, int64_t H, int64_t N);

/*
 * y[M,D] = (gelu_tanh(x[M,D] . Wg[H,D]^T) * (x . Wu[H,D]^T)) . Wd[D,H]^T
 *
 * The GeGLU feed-forward block, all projections bias-free ("Profiling in
 * PyTorch (Part 2)", section "Stacking three Linears: the MLP").  The gate and
 * up projections share each x tile and apply gelu(g)*u in registers, so g and
 * u never reach HBM; m is rounded to bf16 once.  Paths: M <= 16: one
 * persistent decode launch; otherwise a fused gate+up launch writing m to the
 * workspace and a down-projection launch.  Workspace rules as fmlp_mlp2.
 *
 * A third path, chosen only by fmlp_set_path(4) (it is not faster on
 * MI355X, see below), runs the whole block as ONE launch with m kept on chip
 * (section "The fused Triton kernel": the intermediate's round trip through
 * global memory): for D <= 1024, a block owns 64 tokens and a range of the
 * hidden units, computes m 128 units at a time into LDS and accumulates y in
 * registers; the ranges' fp32 partial y go to the workspace and the block
 * that finishes a token tile last adds them in a fixed order (bitwise
 * deterministic).  Measured on the 8192-token 768/3072 GeGLU: 197 us against
 * 122 us for the two launches, with 19 % less L2-miss traffic; the 64-token
 * tile that a 64 x D fp32 accumulator allows makes it bound by L2-to-LDS
 * loads.  Its workspace needs no initialisation; fmlp_geglu_workspace_size
 * covers both forms.  D > 1024 with path 4 is FMLP_E_ARG.
 */
fmlp_status fmlp_geglu(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                       const fmlp_bf16* Wd, int64_t M, int64_t D, int64_t H,
                       fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_geglu_workspace_size(int64_t M, int64_t D, int64_t H);

/*
 * y[M,D] = (gate_act(x[M,D] . Wg[H,D]^T) * (x . Wu[H,D]^T)) . Wd[D,H]^T
 *
 * The gated feed-forward block with the gate's activation as an argument:
 * gate_act = FMLP_ACT_GELU_TANH is fmlp_geglu; FMLP_ACT_SILU gives SwiGLU,
 * FMLP_ACT_RELU ReGLU, FMLP_ACT_GELU_ERF GeGLU with the exact GELU and
 * FMLP_ACT_NONE the bilinear form.  The three-Linear MLP blocks of the models
 * ainews.cool "PyTorch fused MLP efficiency" names (section "technical deep
 * dive": LLaMA-3; section "architectural impact": Mixtral experts) have this
 * shape; the page does not name their gate activation.  Same kernels, paths,
 * workspace (fmlp_glu_workspace_size == fmlp_geglu_workspace_size) and errors
 * as fmlp_geglu; a gate_act that is not an fmlp_act is FMLP_E_ARG.
 */
fmlp_status fmlp_glu(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                     const fmlp_bf16* Wd, int gate_act, int64_t M, int64_t D, int64_t H,
                     fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_glu_workspace_size(int64_t M, int64_t D, int64_t H);

/*
 * Backward pass (training)
 *
 * The gradients of fmlp_linear and fmlp_glu for an upstream gradient dy: the
 * chain rule on the forward definitions.  The pages profile the forward only;
 * the fused gelu*mul of "Profiling in PyTorch (Part 2)", section "Let's use
 * hand tuned kernels" (LigerGELUMulFunction) is an autograd Function whose
 * backward the page does not describe.  Activations' derivatives:
 *   gelu_erf   Phi(z) + z phi(z)
 *   gelu_tanh  (1 + tanh u)/2 + z/2 (1 - tanh^2 u) sqrt(2/pi)(1 + 3*0.044715 z^2),
 *              u = sqrt(2/pi)(z + 0.044715 z^3)
 *   relu       1 for z > 0, else 0;   silu  sigmoid(z)(1 + z(1 - sigmoid(z)))
 * Pre-activations are recomputed by the forward GEMM with a derivative
 * epilogue (nothing of the forward is saved).  Every gradient is accumulated
 * in fp32 and written as bf16 once; the intermediate dz (or dm, m, dg, du) is
 * rounded to bf16 once before the GEMM that consumes it, as eager PyTorch
 * stores it.  Results are bitwise deterministic.  Operands that a backward
 * GEMM contracts over their rows are read in place (k-major, through LDS
 * transpose reads) where the GEMM runs on 256x256 tiles, and otherwise first
 * written transposed into the workspace, as is dz for the bias gradient's row
 * sum.  Outputs are caller-owned bf16, must not alias inputs, and
 * M < 2^22; with M == 0 the weight and bias gradients are written as zeros.
 * Workspace: the *_bwd_workspace_size bytes, no initialisation needed; the
 * first 8192 bytes (the decode header of fmlp_mlp2 / fmlp_glu) are never
 * written, so one workspace can serve forward and backward calls in turn.
 */

/* Linear + activation, y = act(x[M,K] . W[N,K]^T + b[N]):
 *   dz = dy[M,N] * act'(x W^T + b),  dx[M,K] = dz W,  dW[N,K] = dz^T x,
 *   db[N] = sum over tokens of dz.
 * b may be NULL (no bias in the forward); db may be NULL (not computed). */
fmlp_status fmlp_linear_bwd(const fmlp_bf16* x, const fmlp_bf16* W, const fmlp_bf16* b, int act,
                            const fmlp_bf16* dy, int64_t M, int64_t K, int64_t N,
                            fmlp_bf16* dx, fmlp_bf16* dW, fmlp_bf16* db,
                            void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_linear_bwd_workspace_size(int64_t M, int64_t K, int64_t N);

/* The gated block, y = (gate_act(x Wg^T) * (x Wu^T)) Wd^T (FMLP_ACT_GELU_TANH:
 * GeGLU), x [M,D], Wg, Wu [H,D], Wd [D,H], dy [M,D]:
 *   g = x Wg^T, u = x Wu^T, m = act(g) * u, dWd[D,H] = dy^T m, dm = dy Wd,
 *   dg = dm * u * act'(g), du = dm * act(g),
 *   dx[M,D] = dg Wg + du Wu,  dWg[H,D] = dg^T x,  dWu[H,D] = du^T x.
 * 2H must be below 2^22. */
fmlp_status fmlp_glu_bwd(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd,
                         int gate_act, const fmlp_bf16* dy, int64_t M, int64_t D, int64_t H,
                         fmlp_bf16* dx, fmlp_bf16* dWg, fmlp_bf16* dWu, fmlp_bf16* dWd,
                         void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_glu_bwd_workspace_size(int64_t M, int64_t D, int64_t H);

/*
 * fmlp_glu without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels, paths, results and errors
 * as fmlp_glu; the workspace is instead a device array inside this library of
 * FMLP_GLU_NOALLOC_SCRATCH_BYTES (64 MiB), one per device the library runs on,
 * held until the process ends.  A shape whose fmlp_glu_workspace_size exceeds
 * it is FMLP_E_WORKSPACE (the 8192-token 768/3072 block and every shape of up
 * to 16 tokens fit).  No call allocates anything: the first call on a device
 * looks up the array's device address once (with that device current) and
 * clears its 8 KB decode header with a small kernel on `stream`; make that
 * first call outside graph capture.  Every call on a device shares that
 * device's array, which keeps the last call's contents: calls that overlap on
 * one device (on different streams, or from different threads without
 * ordering) race and give wrong results; order them on one stream.
 */
#define FMLP_GLU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fmlp_status fmlp_glu_noalloc(const fmlp_bf16* x, const fmlp_bf16* Wg, const fmlp_bf16* Wu,
                             const fmlp_bf16* Wd, int gate_act, int64_t M, int64_t D, int64_t H,
                             fmlp_bf16* y, fmlp_stream stream);

/*
 * FP8 weights for decode (1 <= M <= 16 tokens)
 *
 * At a few tokens a feed-forward layer is bound by reading its weights once
 * (ainews.cool "PyTorch fused MLP efficiency", section "architectural impact":
 * decode is memory-bandwidth bound); one byte per weight halves those bytes.
 * Each weight matrix is passed as OCP FP8 E4M3 codes (fmlp_fp8: sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F and 0xFF
 * are NaN; largest finite value 448) with one fp32 scale per output row:
 *     W[n, k] = scale[n] * e4m3(q[n, k]).
 * The calls compute exactly what fmlp_linear / fmlp_mlp2 / fmlp_glu compute on
 * that W: x . e4m3(q)^T is accumulated in fp32 (the codes convert to bf16
 * exactly), multiplied by the row's scale, then bias and activation; h (or m)
 * is rounded to bf16 once.  Activations, biases and outputs are bf16 as above.
 * Besides the shared rules: M <= 16 (larger M is FMLP_E_ARG; M == 0 is a
 * no-op), every dimension a layer contracts over (K, H, D) a multiple of 16
 * (FMLP_E_ALIGN; an output-only N keeps the multiple of 8), code arrays
 * 16-byte aligned, scale arrays [N] fp32, 4-byte aligned and finite.
 * Launches: at one token with H <= 4096 (and 2 K <= 65536) the two-layer forms
 * run as ONE persistent launch with the one-launch decode's protocol (ainews,
 * section "technical deep dive": the fused MLP is one kernel): h is published
 * as epoch-tagged words after the workspace's 8192-byte header, every block
 * gathers it, and the header's generation advances by one and its timeout
 * count works as described for fmlp_mlp2 (same header, same residency
 * assumption).  Otherwise one launch per layer, writing h or m [M, H] bf16
 * after the header and never touching the header.  fmlp_set_path(2) forces
 * the launch-per-layer form.  The workspace: fmlp_w8_workspace_size bytes;
 * zero its header once, as for fmlp_mlp2.
 */
typedef uint8_t fmlp_fp8;  /* OCP FP8 E4M3 ("e4m3fn") code */

/* y[M,N] = act(x[M,K] . (w_scale[N] * e4m3(Wq[N,K]))^T + b[N]); b may be NULL. */
fmlp_status fmlp_linear_w8(const fmlp_bf16* x, const fmlp_fp8* Wq, const float* w_scale,
                           const fmlp_bf16* b, int act, int64_t M, int64_t K, int64_t N,
                           fmlp_bf16* y, fmlp_stream stream);

/* fmlp_mlp2 with W1 = s1 * e4m3(W1q) [H,K] and W2 = s2 * e4m3(W2q) [N,H]. */
fmlp_status fmlp_mlp2_w8(const fmlp_bf16* x, const fmlp_fp8* W1q, const float* s1,
                         const fmlp_bf16* b1, const fmlp_fp8* W2q, const float* s2,
                         const fmlp_bf16* b2, int act, int64_t M, int64_t K, int64_t H, int64_t N,
                         fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);

/* fmlp_glu with Wg = sg * e4m3(Wgq), Wu = su * e4m3(Wuq) [H,D], Wd = sd * e4m3(Wdq) [D,H].
 * The gate and up rows of each tile are read together and act(g) * u is
 * applied in registers, as in fmlp_glu. */
fmlp_status fmlp_glu_w8(const fmlp_bf16* x, const fmlp_fp8* Wgq, const float* sg,
                        const fmlp_fp8* Wuq, const float* su, const fmlp_fp8* Wdq, const float* sd,
                        int gate_act, int64_t M, int64_t D, int64_t H, fmlp_bf16* y,
                        void* workspace, size_t workspace_bytes, fmlp_stream stream);

/* bytes of workspace the two-layer FP8 calls need: the 8192-byte decode
 * header, then h or m, M x H bf16, or at one token H / 2 words of 8 bytes,
 * whichever is larger (0 for M == 0) */
size_t fmlp_w8_workspace_size(int64_t M, int64_t H);

/*
 * y[t,:] = sum_{j<top_k} gate_w[t,j] * geglu_{expert_ids[t,j]}(x[t,:])
 *
 * Mixture of GeGLU experts (ainews.cool "PyTorch fused MLP efficiency",
 * section "architectural impact": tokens are routed to several experts, each an
 * MLP).  x [T,D]; expert_ids int32 [T,top_k] and gate_w fp32 [T,top_k] are
 * device arrays; Wg, Wu are stacked [E,H,D] and Wd is [E,D,H].  1 <= top_k <= 8,
 * 1 <= E <= 1024.  Routed pairs are bucketed per expert (stable in token
 * order), each expert runs the fused gate+up and down GEMMs over its rows, and
 * the weighted combine sums the top_k contributions of a token in slot order in
 * fp32 (deterministic; no atomics).  An expert id outside [0,E) contributes
 * nothing and is counted in the workspace error word (fmlp_moe_error_count
 * documents where).  Workspace: fmlp_moe_workspace_size(T,D,H,E,top_k) bytes.
 * x must hold fewer than 2^30 elements (T*D < 2^30): routed rows are gathered
 * from it with 32-bit byte offsets; a larger x is FMLP_E_SHAPE.
 */
fmlp_status fmlp_moe_geglu(const fmlp_bf16* x, const int32_t* expert_ids, const float* gate_w,
                           const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd,
                           int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k,
                           fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);
size_t fmlp_moe_workspace_size(int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k);

/*
 * fmlp_moe_geglu with the experts' gate activation as an argument (as
 * fmlp_glu; FMLP_ACT_SILU gives SwiGLU experts).  fmlp_moe_geglu is this call
 * with FMLP_ACT_GELU_TANH.  Same workspace and errors.
 */
fmlp_status fmlp_moe_glu(const fmlp_bf16* x, const int32_t* expert_ids, const float* gate_w,
                         const fmlp_bf16* Wg, const fmlp_bf16* Wu, const fmlp_bf16* Wd, int gate_act,
                         int64_t T, int64_t D, int64_t H, int32_t E, int32_t top_k,
                         fmlp_bf16* y, void* workspace, size_t workspace_bytes, fmlp_stream stream);
/*
 * The routes on the device: logits[t,e] = x[t,:] . Wr[e,:] (fp32 accumulation),
 * expert_ids[t,:] = the top_k experts by logit in descending order (a tie goes
 * to the lower expert id), gate_w[t,:] = softmax over those top_k logits.
 * The router of the MoE layer in ainews.cool "PyTorch fused MLP efficiency",
 * section "architectural impact" (tokens routed to several experts); the page
 * gives no router formula, and this is the plain linear router with top-k and a
 * softmax over the chosen logits.  Its outputs are the routes fmlp_moe_glu /
 * fmlp_moe_geglu take.
 * x [T,D] bf16 and Wr [E,D] bf16 (16-byte aligned); expert_ids int32 [T,top_k],
 * gate_w fp32 [T,top_k] and logits fp32 [T,E] (may be NULL: not written) are
 * caller-owned device arrays, 4-byte aligned.  1 <= E <= 64,
 * 1 <= top_k <= min(8, E).  One launch; no workspace; deterministic.
 */
fmlp_status fmlp_moe_route(const fmlp_bf16* x, const fmlp_bf16* Wr, int64_t T, int64_t D, int32_t E,
                           int32_t top_k, int32_t* expert_ids, float* gate_w, float* logits,
                           fmlp_stream stream);

/* Byte offset, inside the MoE workspace, of the int32 count of invalid expert ids
 * seen by the last call (read it after a stream sync). */
size_t fmlp_moe_error_offset(void);

/* Byte offsets, inside an fmlp_mlp2 / fmlp_geglu / fmlp_glu workspace, of the
 * one-launch decode kernel's uint32 words: the count of device-wide barrier
 * waits that gave up (cumulative; nonzero means a decode result written since
 * it was last seen is wrong), and the generation (advanced by one per
 * one-launch decode call).  Read them after a stream sync. */
size_t fmlp_decode_timeout_offset(void);
size_t fmlp_decode_generation_offset(void);

/*
 * Path override for tests and benchmarks (thread-local; applies to the calling
 * thread's later fmlp_mlp2 / fmlp_geglu calls):
 *   0 = automatic (default), 1 = force the decode path (needs M <= 16),
 *   2 = force the two-GEMM path, 3 = force the fused small-MLP path (mlp2 only),
 *   4 = the gated block in one launch with m on chip (fmlp_geglu / fmlp_glu
 *       only, D <= 1024).
 * A forced path that does not apply to a call makes it return FMLP_E_ARG.
 */
fmlp_status fmlp_set_path(int path);

/*
 * Cooperative launch of the one-launch decode forms (thread-local; applies to
 * the calling thread's later fmlp_mlp2 / fmlp_geglu / fmlp_glu decode calls and
 * the one-token FP8 two-layer calls).  on = 1: those kernels go through
 * hipLaunchCooperativeKernel, so a grid that cannot be resident at once is
 * refused (FMLP_E_HIP) instead of a barrier wait timing out with y wrong;
 * measured to add about 18 us per call on MI355X.  on = 0 (default): the
 * plain launch, with the timeout count in the workspace header.  Other values
 * are FMLP_E_ARG.
 */
fmlp_status fmlp_set_cooperative_decode(int on);

const char* fmlp_status_string(fmlp_status s);
const char* fmlp_last_error(void);
int fmlp_version(void);  /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* FMLP_H_ */
