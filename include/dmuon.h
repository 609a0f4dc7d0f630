/*
 * dmuon.h -- batched Muon optimizer step for AMD Instinct MI355X (gfx950).
 *
 * One call runs the Muon update over a whole set of 2-D weight matrices on one
 * GPU stream:
 *
 *   buf <- mu * buf + grad                          momentum (fp32 state)
 *   Y   <- grad + mu * buf   (Nesterov)  or  buf    Newton-Schulz input
 *   U   <- NS_k(Y)                                  numel >= 100000
 *   U   <- Y                                        numel <  100000
 *   p   <- p - lr * lr_scale_i * U
 *
 * where NS_k normalises by the Frobenius norm (+1e-7), iterates on the wide
 * orientation (the transpose when rows > cols) and applies k times the cubic
 * map X <- 1.5 X - 0.5 (X X^T) X, or a custom odd polynomial (dmuon_ns_config).
 * With weight decay wd the update is p <- p (1 - lr wd) - lr s_i U.
 *
 * Sources: DMuon blog post "DMuon：让矩阵正交化优化器达到接近 AdamW 的分布式训练开销",
 * sections "Muon 核心：Newton-Schulz 迭代" (normalisation, cubic map, transpose
 * to the wide side) and "代码实现" (VanillaMuon: momentum, non-matrix branch,
 * update); DMuon training guide "训练指南", table "超参数指南" (lr, momentum,
 * ns_steps, nesterov: ns_input = grad + mu * buf) and section "编写 Predicate"
 * (numel < 100_000 is too small for NS).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are dense, row-major, contiguous: element (r, c) of matrix i is at
 *   offset r * cols[i] + c.  rows[i], cols[i] >= 1 and <= DMUON_MAX_DIM.
 * - Tensor pointers are device pointers; the pointer arrays themselves, the
 *   shape arrays and lr_scale are host arrays, read only during the call.
 * - All tensors and the workspace are owned by the caller.  The library
 *   allocates no device memory at run time; its only device memory is the
 *   static scratch of dmuon_muon_step_noalloc, which comes with the library's
 *   code on each GPU.  It keeps no state between calls other than per-device
 *   capability checks, the scratch addresses and the optional profiler record.
 * - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *   and the call returns without synchronising.  Inputs must stay valid and
 *   unmodified until the stream reaches the end of the enqueued work.
 * - The workspace must hold at least the queried number of bytes and must not
 *   be used by anything else until the enqueued work completes.  Two calls may
 *   run concurrently only with distinct workspaces and disjoint outputs.
 * - The calls cannot be recorded into a HIP graph: each uploads its
 *   descriptors from host memory that lives only for the call.  A call on a
 *   stream that is capturing returns DMUON_ERR_INVALID_ARG.
 * - Argument errors are detected before anything is enqueued; nothing is
 *   modified in that case.  A later DMUON_ERR_HIP means a launch failed and the
 *   outputs are unspecified.
 * - Results are bitwise reproducible for the same inputs, and a matrix's result
 *   does not depend on the other matrices in the batch or their order.
 * - Environment (read at each call): DMUON_NS_KERNEL=gemm selects the
 *   DMUON_NS_DIRECT backend whatever ns_config says: every tile of each Gram
 *   product instead of its lower triangle plus a mirrored copy.  It is a
 *   measurement ablation that shows what the triangle saves; results match the
 *   default to rounding.  Every other value, or no value, changes nothing.
 */
#ifndef DMUON_H
#define DMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of gradients, parameters and Newton-Schulz operands.  The blog's
 * newton_schulz accepts float32 or bfloat16.  Momentum is always float32. */
#define DMUON_F32 0
#define DMUON_BF16 1

/* Status codes. */
#define DMUON_OK 0
#define DMUON_ERR_INVALID_ARG 1        /* bad count, shape, pointer, step count, ... */
#define DMUON_ERR_UNSUPPORTED_DTYPE 2  /* dtype is neither DMUON_F32 nor DMUON_BF16 */
#define DMUON_ERR_WORKSPACE 3          /* workspace NULL or smaller than the query */
#define DMUON_ERR_NO_DEVICE 4          /* no HIP device visible */
#define DMUON_ERR_UNSUPPORTED_ARCH 5   /* current device is not gfx950 */
#define DMUON_ERR_HIP 6                /* a HIP runtime call or launch failed */

/* Training guide, "编写 Predicate": matrices with numel < 100_000 skip NS. */
#define DMUON_MIN_NS_NUMEL 100000
/* Largest accepted rows or cols. */
#define DMUON_MAX_DIM 65536
/* Largest accepted ns_steps. */
#define DMUON_MAX_NS_STEPS 64

/*
 * Newton-Schulz configuration: the training guide's `ns_backend` ("超参数指南":
 * "gram" or "direct", or a NewtonSchulz object with custom coefficients; the
 * pages print no coefficients).  Each step maps the iterate X (wide side) to
 *
 *   X <- c0 X + c1 A X + c2 A^2 X,    A = X X^T,
 *
 * an odd polynomial in X; (c0, c1) = (1.5, -0.5) with no c2 is the blog's
 * cubic map ("Muon 核心：Newton-Schulz 迭代").  A NULL config pointer means
 * { DMUON_NS_GRAM, 0, 0, NULL }.
 */
#define DMUON_NS_GRAM 0       /* Gram products on lower-triangle tiles, mirrored (default) */
#define DMUON_NS_DIRECT 1     /* Gram products on every tile */
#define DMUON_MAX_NS_TERMS 3  /* c0, c1, c2 */
typedef struct {
    int backend;          /* DMUON_NS_GRAM or DMUON_NS_DIRECT */
    int num_terms;        /* 0: the cubic map (1.5, -0.5); 2 or 3: coefficients from `coeffs` */
    int per_step;         /* 0: one coefficient set for every step; 1: one set per step (ns_steps sets) */
    const float* coeffs;  /* host; sets of num_terms floats (c0 first), one after another; read during
                             the call; every value finite.  Ignored when num_terms is 0. */
} dmuon_ns_config;

/* Learning-rate scale modes of dmuon_muon_step (s_i below). */
#define DMUON_LR_SCALE_ONE 0        /* s_i = lr_scale[i], or 1 when lr_scale is NULL */
#define DMUON_LR_SCALE_MOONLIGHT 1  /* s_i = 0.2 * sqrt(max(rows_i, cols_i)) * (lr_scale[i], or 1) --
                                       the training guide's per-parameter scaling ("超参数指南", lr) */

/*
 * Workspace size for dmuon_ns_batched over the given shapes and configuration
 * (NULL = default), in bytes.  The blog post's "什么时候用 / 不用？" notes that
 * Newton-Schulz needs temporary matrices; here they are the iterate (two
 * operand copies plus, for bf16, its low half) and the m' x m' Gram matrix per
 * matrix, in the caller's workspace.  Writes *bytes_out and returns DMUON_OK,
 * or an argument error (the shape rules of dmuon_ns_batched, whose
 * newton_schulz in "代码实现" accepts 2-D matrices only).  Needs no GPU.  A
 * three-term polynomial needs an extra m' x m' buffer per matrix.
 */
int dmuon_ns_workspace_bytes(int count, const int64_t* rows, const int64_t* cols, int dtype,
                             const dmuon_ns_config* ns_config, size_t* bytes_out);

/*
 * Newton-Schulz orthogonalisation of `count` independent matrices
 * (blog post, "Muon 核心：Newton-Schulz 迭代" and the newton_schulz listing of
 * "代码实现"):
 *
 *   out_i = NS_{ns_steps}(x_i)
 *
 * x_in[i]  : device, rows[i] x cols[i], `dtype`, read only.
 * x_out[i] : device, rows[i] x cols[i], `dtype`, written (RNE for bf16).  May
 *            equal x_in[i]; must not overlap any other input or output.
 * ns_steps : 0 .. DMUON_MAX_NS_STEPS; 0 returns the normalised input.
 * ns_config: NULL (the cubic map, gram backend) or a host configuration, read
 *            during the call; the workspace must be sized for the same one.
 * Every matrix is orthogonalised, whatever its size.  bf16 inputs run the
 * contractions on bf16 operands with fp32 accumulation; between steps the
 * iterate is kept as a bf16 pair hi + lo (16 significant bits), and all
 * epilogue arithmetic is fp32.
 */
int dmuon_ns_batched(int count, const void* const* x_in, void* const* x_out,
                     const int64_t* rows, const int64_t* cols, int dtype, int ns_steps,
                     const dmuon_ns_config* ns_config,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Workspace size for dmuon_muon_step over the given shapes and Newton-Schulz
 * configuration (NULL = default), in bytes: the Newton-Schulz temporaries of
 * the matrices that take that route (blog post, "什么时候用 / 不用？"; matrices
 * below DMUON_MIN_NS_NUMEL need none), plus descriptors and the per-block norm
 * partials.  Same errors as dmuon_ns_workspace_bytes.  Needs no GPU.
 */
int dmuon_muon_step_workspace_bytes(int count, const int64_t* rows, const int64_t* cols, int dtype,
                                    const dmuon_ns_config* ns_config, size_t* bytes_out);

/*
 * One Muon step over `count` matrices (blog post VanillaMuon.step with the
 * training guide's Nesterov input; equations at the top of this header).
 *
 * params[i]     : device, rows x cols, `dtype`; updated in place (RNE for bf16).
 * grads[i]      : device, rows x cols, `dtype`; read only.
 * momentum[i]   : device, rows x cols, float32; updated in place.  Start from
 *                 zeros for a fresh optimizer.
 * mu            : momentum coefficient (0.95 in the pages' defaults).
 * nesterov      : nonzero -> Y = grad + mu * buf (with the updated buf).
 * ns_steps      : 0 .. DMUON_MAX_NS_STEPS (5 in the pages' defaults).
 * ns_config     : NULL (cubic map, gram backend) or a host configuration; the
 *                 workspace must be sized for the same one.
 * lr            : learning rate (0.02 in the pages' defaults).
 * weight_decay  : decoupled decay (training guide, creating the optimizer:
 *                 `weight_decay`, default 0): p <- p (1 - lr wd) - lr s_i U,
 *                 with the unscaled lr in the decay.  Finite.
 * lr_scale_mode : DMUON_LR_SCALE_ONE or DMUON_LR_SCALE_MOONLIGHT.
 * lr_scale      : host array of `count` finite floats multiplying lr per
 *                 matrix, or NULL for 1.0.
 * update_out    : NULL, or a host array of `count` device pointers (entries
 *                 may be NULL) receiving U_i as float32, rows x cols.
 * norms_out     : NULL, or a device float32 array of `count` entries receiving
 *                 ||Y_i||_F.
 * params, grads, momentum and non-NULL update_out entries must be distinct
 * non-overlapping buffers.
 * Range: the 1/(||Y|| + 1e-7) scale is folded into the first Newton-Schulz
 * step, whose Gram product accumulates the unnormalised Y Y^T in fp32.  A
 * matrix with ||Y||_F >= 2^63 (about 9.2e18; its norms_out entry may be inf)
 * is outside that range and gets a NaN update, as a non-finite gradient does;
 * the other matrices of the call are unaffected.
 */
int dmuon_muon_step(int count, void* const* params, const void* const* grads, float* const* momentum,
                    const int64_t* rows, const int64_t* cols, int dtype,
                    int ns_steps, const dmuon_ns_config* ns_config,
                    float mu, int nesterov, float lr, float weight_decay,
                    int lr_scale_mode, const float* lr_scale,
                    float* const* update_out, float* norms_out,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Workspace size for dmuon_muon_step_clipped, in bytes: that of
 * dmuon_muon_step for the same shapes and configuration, plus the clip's
 * per-tile partial sums and per-segment coefficients.  Needs no GPU.
 */
int dmuon_muon_step_clip_workspace_bytes(int count, const int64_t* rows, const int64_t* cols, int dtype,
                                         const dmuon_ns_config* ns_config, int num_segments, size_t* bytes_out);

/*
 * dmuon_muon_step with per-segment global p-norm gradient clipping folded in
 * (training guide, "梯度裁剪": the Muon clip runs on the reduced gradients
 * before momentum and Newton-Schulz; "regular / Muon / AdamW 的融合 CUDA 裁剪":
 * per-segment norms and coefficients computed in one fused pass).  The clip is
 * dmuon_clip_grad_norm's rule with the matrices as its tensors:
 *
 *   total_s = || gradients of segment s ||_p
 *   coef_s  = min(max_norm[s] / (total_s + 1e-6), 1)
 *
 * and the step then runs on coef_{segment[i]} * grads[i], formed in fp32 as
 * each gradient element is read and never rounded to the gradient dtype.  The
 * caller's gradients are not rewritten (unlike dmuon_clip_grad_norm), which
 * saves that pass: clipping costs one extra read of the gradients.
 *
 * segment[i]   : host, the clipping segment of matrix i, in [0, num_segments).
 * num_segments, max_norm (host, finite, >= 0), norm_type (p > 0 or +inf),
 * totals_out (NULL or device float32[num_segments]): as in
 * dmuon_clip_grad_norm.  Every other argument as in dmuon_muon_step; the
 * workspace is sized by dmuon_muon_step_clip_workspace_bytes.  A segment whose
 * coefficient is 1 gets bitwise the result of dmuon_muon_step.
 */
int dmuon_muon_step_clipped(int count, void* const* params, const void* const* grads, float* const* momentum,
                            const int64_t* rows, const int64_t* cols, int dtype,
                            int ns_steps, const dmuon_ns_config* ns_config,
                            float mu, int nesterov, float lr, float weight_decay,
                            int lr_scale_mode, const float* lr_scale,
                            float* const* update_out, float* norms_out,
                            const int* segment, int num_segments, const float* max_norm, float norm_type,
                            float* totals_out, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Scratch held by the library for dmuon_muon_step_noalloc: 64 MiB on each GPU
 * the library is loaded on, from the load until the process ends. */
#define DMUON_NOALLOC_SCRATCH_BYTES 67108864

/*
 * dmuon_muon_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as dmuon_muon_step (bitwise: the same kernels),
 * but the scratch is the library's own static device array of
 * DMUON_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace; the call
 * allocates nothing.  A set whose dmuon_muon_step_workspace_bytes exceeds
 * DMUON_NOALLOC_SCRATCH_BYTES is rejected with DMUON_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams or threads) race and give undefined
 * results; calls ordered on one stream are safe.  The array needs no clearing
 * between calls (every stage writes what it later reads).  The stream-capture
 * restriction of dmuon_muon_step applies as well (host-side descriptors).
 */
int dmuon_muon_step_noalloc(int count, void* const* params, const void* const* grads, float* const* momentum,
                            const int64_t* rows, const int64_t* cols, int dtype,
                            int ns_steps, const dmuon_ns_config* ns_config,
                            float mu, int nesterov, float lr, float weight_decay,
                            int lr_scale_mode, const float* lr_scale,
                            float* const* update_out, float* norms_out, void* hip_stream);

/*
 * Workspace size for dmuon_clip_grad_norm, in bytes.  Needs no GPU.
 */
int dmuon_clip_grad_norm_workspace_bytes(int count, const int64_t* numel, int num_segments, size_t* bytes_out);

/*
 * Per-segment global p-norm gradient clipping, in place (training guide,
 * "梯度裁剪": the Muon clip before momentum and Newton-Schulz, and the fused
 * bucketed clip that keeps per-segment semantics; the rule of PyTorch's
 * clip_grad_norm_, which the guide names for the other parameters):
 *
 *   total_s = (sum over i with segment[i] == s of sum |g_i|^p)^(1/p)   (max |g_i| for p = +inf)
 *   coef_s  = min(max_norm[s] / (total_s + 1e-6), 1)
 *   g_i    <- coef_s * g_i     (a segment with coef_s == 1 is not rewritten)
 *
 * grads[i]     : device, numel[i] contiguous elements of `dtype`, updated in
 *                place (RNE for bf16); distinct buffers.
 * numel[i]     : >= 0 (0 = an empty tensor, ignored).
 * segment[i]   : host, in [0, num_segments).
 * max_norm[s]  : host, finite, >= 0.
 * norm_type    : p > 0 or +inf.  Totals accumulate in fp32 in a fixed order,
 *                so results are bitwise reproducible.  A non-finite total
 *                gives a coefficient of 0 (total +inf) or NaN (total NaN),
 *                as the reference rule does.
 * totals_out   : NULL or device float32[num_segments] receiving total_s.
 * count == 0 enqueues nothing.
 */
int dmuon_clip_grad_norm(int count, void* const* grads, const int64_t* numel, int dtype, const int* segment,
                         int num_segments, const float* max_norm, float norm_type, float* totals_out,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Workspace size for dmuon_adamw_step, in bytes.  Needs no GPU.
 */
int dmuon_adamw_step_workspace_bytes(int count, const int64_t* numel, size_t* bytes_out);

/*
 * One AdamW step over `count` non-matrix parameters, in place (training
 * guide, "第 4 步：创建优化器": the parameters Muon does not take form a
 * standard AdamW group with adamw_lr, adamw_betas, adamw_eps and
 * adamw_weight_decay; blog post, section "为什么需要矩阵感知优化器": the
 * update subtracts alpha m_hat / (sqrt(v_hat) + eps) with bias-corrected
 * moments).  Read as PyTorch's AdamW, per element in fp32:
 *
 *   p <- p (1 - lr weight_decay)
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - (lr / (1 - beta1^step)) m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 *
 * params[i]     : device, numel[i] contiguous elements of `dtype`; updated in
 *                 place (RNE for bf16).
 * grads[i]      : device, numel[i] elements of `dtype`; read only.
 * exp_avg[i], exp_avg_sq[i] : device, numel[i] float32 moments, updated in
 *                 place.  Start both from zeros.
 * numel[i]      : >= 0 (0 = an empty tensor, ignored; its pointers may be NULL).
 * step          : the step counter t >= 1 of this update (1 on the first call).
 * lr, weight_decay : finite.  beta1, beta2 in [0, 1).  eps finite, >= 0.
 *                 The pages' defaults: lr 1e-3, betas (0.9, 0.999), eps 1e-8,
 *                 weight_decay 0.01.
 * All buffers must be distinct and aligned to their element size; 16-byte
 * alignment (8-byte for bf16 parameters and gradients) takes the vector path.
 * The bias corrections and 1 - lr weight_decay are formed in double on the
 * host and rounded to float once.  count == 0 enqueues nothing.
 */
int dmuon_adamw_step(int count, void* const* params, const void* const* grads, float* const* exp_avg,
                     float* const* exp_avg_sq, const int64_t* numel, int dtype, int step, float lr, float beta1,
                     float beta2, float eps, float weight_decay, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/*
 * The plan of a call as text: routes (numel < DMUON_MIN_NS_NUMEL goes
 * elementwise when muon_step is nonzero), shape groups with their transposed
 * count, tiles and K slices, launches per Newton-Schulz step, algorithmic
 * flops and the workspace size -- the analogue of the training guide's INFO
 * summary of how parameters were assigned ("日志与调试", "验证参数分配").
 * Writes at most buf_len bytes including the terminating NUL (buf may be NULL
 * when buf_len is 0) and sets *needed (if not NULL) to the full length + 1.
 * Needs no GPU.  With the environment variable DMUON_LOG set (to anything but
 * "" or "0"), every call prints this text to stderr when its plan differs from
 * the last one printed.
 */
int dmuon_plan_summary(int count, const int64_t* rows, const int64_t* cols, int dtype,
                       const dmuon_ns_config* ns_config, int ns_steps, int muon_step, char* buf, size_t buf_len,
                       size_t* needed);

/* Static text for a status code.  The codes translate the pages' error
 * conventions to return values: the blog's newton_schulz asserts a 2-D input
 * ("代码实现", and "常见错误" 2: a bias vector must not reach NS) and accepts
 * float32 or bfloat16 only; the training guide's optimizer rejects bad
 * parameter lists when it is built ("第 4 步：创建优化器"). */
const char* dmuon_status_string(int status);

/* Details of the last error returned on the calling thread ("" if none). */
const char* dmuon_last_error(void);

/* Build and kernel description, the analogue of the pages' get_ns_backend()
 * string (training guide, "检查 NS 后端"). */
const char* dmuon_backend_info(void);

/*
 * Kernel-level timing.  While enabled, every kernel the library enqueues is
 * bracketed by a pair of HIP events on its stream.  dmuon_profile_read waits
 * for those events, returns per-kernel totals and clears the record.
 */
typedef struct {
    char name[40];      /* kernel family, e.g. "ns_gemm" */
    int64_t launches;   /* launches recorded */
    double total_ms;    /* sum of event-measured launch durations */
    double flops;       /* algorithmic flops summed over those launches */
    double bytes;       /* algorithmic HBM bytes summed over those launches */
} dmuon_kernel_stat;

int dmuon_profile_enable(int on);
/* Fills up to `max_stats` entries and sets *n_stats; returns a status. */
int dmuon_profile_read(dmuon_kernel_stat* stats, int max_stats, int* n_stats);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_H */
