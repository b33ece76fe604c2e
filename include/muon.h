/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer-step library.
 *
 * The operation (sources: Keller Jordan's "new optimizer" X thread,
 * xunroll.com/thread/1842300916864844014, tweets 2/8, 5/8 and 6/8; the
 * momentum convention from "07. Training neural networks", section
 * "Momentum"):
 *
 *   for every 2-D parameter matrix W (rows x cols, fp32) with gradient G and
 *   momentum buffer M:
 *     M  <- beta * M + G                      SGD momentum buffer
 *     U  <- G + beta * M                      Nesterov look-ahead
 *     X0 <- bf16( U / (||U||_F + 1e-7) )      transposed first if rows > cols
 *     repeat ns_steps times (quintic Newton-Schulz, in bfloat16):
 *        A <- bf16(X X^T);  B <- bf16(b A + c A A);  X <- bf16(a X + B X)
 *     W  <- W - lr * X                        (X transposed back)
 *
 * The thread states the design: orthogonalise each parameter's update after
 * Nesterov momentum, with a quintic Newton-Schulz iteration run in bfloat16,
 * whose coefficients maximise the slope at zero at the cost of exact
 * convergence.  The normalisation, the epsilon, the coefficient values and the
 * bf16 storage points are readings of those statements, not quotes: every
 * product accumulates in fp32 from bf16 operands; A, B and each new X are
 * rounded to bf16 (round to nearest even); the epilogue combinations
 * b*A + c*(AA) and a*X + (BX) are two fp32 products and one fp32 sum, not
 * fused.  No weight decay (the thread's replies report it as worse).  Only
 * 2-D matrices belong here; 1-D parameters go to another optimizer.
 *
 * Conventions for every entry point:
 *   - All matrix pointers are device pointers (HIP device memory, e.g. from
 *     PyTorch), row-major, contiguous, 4-byte aligned, caller-owned, and do
 *     not alias one another.  Arrays of pointers and shapes are host arrays,
 *     read only during the call.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Kernel faults surface at the caller's next synchronisation.  The
 *     calls made on one device must be ordered on the GPU: make them on one
 *     stream, or order the streams yourself (events).  They share the
 *     library's workspace and plan tables, which each call writes in its
 *     stream's order.
 *   - Plans are cached per device and keyed on the shapes (and the entry
 *     point), not on the pointers.  The first call with a set of shapes
 *     builds its plan: it allocates the plan's device table block
 *     (descriptors and work lists, a few hundred KB at most for GPT-2-sized
 *     sets) and enqueues its upload; it does not synchronise.  A call whose
 *     pointers differ from the previous call's on that plan enqueues one
 *     small kernel per 40 matrices that writes them into the descriptors;
 *     otherwise a call only enqueues the step's kernels.  Up to 8 plans are
 *     kept; evicting the least recently used one, or growing the library's
 *     workspace, waits for the device (hipDeviceSynchronize).
 *   - HIP graph capture: a call made while `stream` is capturing must find
 *     its plan and a large enough workspace already there (make one call
 *     with the same shapes first; otherwise it fails with MUON_EINVAL and
 *     enqueues nothing).  It allocates nothing and records only kernel
 *     launches: the pointer write and the step.  Its plan, and the workspace
 *     that plan uses, are then kept until muon_release(): neither eviction
 *     nor a later, larger call frees them, so the graph can be replayed
 *     between other calls.  Graphs must not be replayed after
 *     muon_release(), or after muon_set_workspace() replaced a caller-owned
 *     workspace they use.
 *   - Arguments are validated on the host before any HIP call; on failure
 *     the call returns a negative code, enqueues nothing and
 *     muon_last_error() describes the problem.
 *   - Return codes: MUON_OK (0), MUON_EINVAL (bad argument), MUON_ENOMEM
 *     (workspace allocation failed or caller workspace too small),
 *     MUON_EHIP (a HIP runtime call or launch failed; the HIP error string is
 *     in muon_last_error()).
 */
#ifndef MUON_H_
#define MUON_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_OK 0
#define MUON_EINVAL (-1)
#define MUON_ENOMEM (-2)
#define MUON_EHIP (-3)

/* Largest accepted ns_steps and matrix count per call. */
#define MUON_MAX_NS_STEPS 64
#define MUON_MAX_MATRICES 65536

/* Matrix shape in the caller's orientation. */
typedef struct {
  int64_t rows;
  int64_t cols;
} muon_shape_t;

/*
 * One Muon step over n independent matrices.
 *   params[i]   fp32 rows x cols, updated in place
 *   grads[i]    fp32 rows x cols, read only
 *   momentum[i] fp32 rows x cols, updated in place (zero before the first step)
 *   shapes[i]   rows, cols >= 1; rows * cols < 2^31
 *   lr          finite
 *   beta        in [0, 1)
 *   ns_steps    0 .. MUON_MAX_NS_STEPS (0 applies the normalised bf16 X0)
 *   coeffs      host array {a, b, c}, finite; the same triple every iteration
 * n == 0 is a no-op.  A zero gradient with a zero buffer leaves W unchanged.
 * NaN/Inf in the inputs propagate; nothing checks for them.
 */
int muon_step(float* const* params, const float* const* grads, float* const* momentum,
              const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
              const float* coeffs, hipStream_t stream);

/*
 * Same as muon_step, and additionally writes the bf16 update X (the value
 * applied as W -= lr * X) to updates[i] (uint16 bf16 bit patterns,
 * rows x cols, caller orientation).  updates may be NULL, or any element may
 * be NULL, to skip that output.
 */
int muon_step_ex(float* const* params, const float* const* grads, float* const* momentum,
                 const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
                 const float* coeffs, uint16_t* const* updates, hipStream_t stream);

/*
 * muon_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, same kernels and bit-identical results as muon_step, but
 * the workspace and the plan tables live in a static device array of
 * MUON_NOALLOC_SCRATCH_BYTES (128 MiB) that every device the library runs on
 * holds from the library's load until the process ends; no hipMalloc,
 * hipFree, pinned host memory or copy-engine transfer is used (the tables
 * and pointers reach the device as kernel arguments; host bookkeeping uses
 * the C++ heap).  A call whose workspace and tables exceed the array (one
 * GPT-2-124M block, 55.4 MiB, fits; the whole 48-matrix hidden set does not)
 * fails with MUON_ENOMEM and enqueues nothing.  Every call on a device
 * shares that device's array and leaves its contents behind; no call
 * depends on them (every value a kernel reads there was written earlier in
 * the same call), but calls whose GPU work overlaps in time on one device
 * race on the array: order them (one stream).
 */
#define MUON_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int muon_step_noalloc(float* const* params, const float* const* grads, float* const* momentum,
                      const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
                      const float* coeffs, hipStream_t stream);

/*
 * muon_step_ex with a coefficient schedule: coeffs is a host array of
 * 3 * ns_steps floats, iteration k (0-based) using coeffs[3k .. 3k+2] as
 * {a, b, c}; all must be finite; it may be NULL when ns_steps = 0.  (The
 * thread's tweet 6/8 presents the coefficients as a trade-off between the
 * slope at zero and closeness to 1; a schedule makes that choice per
 * iteration.)  A schedule repeating one triple gives exactly muon_step_ex's
 * result.  updates as in muon_step_ex (may be NULL).
 */
int muon_step_sched(float* const* params, const float* const* grads, float* const* momentum,
                    const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
                    const float* coeffs, uint16_t* const* updates, hipStream_t stream);

/*
 * The Newton-Schulz core alone: out[i] = iterate(x[i]) with the same
 * storage points as muon_step, no normalisation, no momentum.  x[i] and out[i]
 * are bf16 bit patterns (uint16), rows x cols in the caller's orientation
 * (tall matrices are transposed internally); out may equal x.  ns_steps = 0
 * copies.
 */
int muon_newton_schulz(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes,
                       int n, int ns_steps, const float* coeffs, hipStream_t stream);

/* muon_newton_schulz with a coefficient schedule (3 * ns_steps floats, as in
 * muon_step_sched). */
int muon_newton_schulz_sched(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes,
                             int n, int ns_steps, const float* coeffs, hipStream_t stream);

/*
 * Multi-tensor AdamW step, for the parameters that are not hidden 2-D
 * matrices (embeddings, biases, norm gains).  The update (the "07. Training
 * neural networks" page, section "Adam, weight decay and AdamW" and its
 * derivation of the bias correction and of the decoupled decay), for every
 * element of tensor i, with t = step:
 *   p <- p * (1 - lr * weight_decay[i])           decay first (decoupled)
 *   u <- beta1 * u + (1 - beta1) * g
 *   v <- beta2 * v + (1 - beta2) * g * g
 *   p <- p - lr * (u / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * fp32 throughout, one IEEE rounding per operation in the order written
 * (no fused multiply-add; division and square root correctly rounded);
 * 1 - beta_k and 1 - beta_k^t are evaluated in double from the fp32
 * arguments and rounded once to fp32; the decay factor is
 * fp32(1 - fp32(lr * weight_decay[i])).
 *   params[i], exp_avg[i], exp_avg_sq[i]  fp32, numels[i] contiguous elements,
 *               updated in place (exp_avg, exp_avg_sq zero before step 1)
 *   grads[i]    fp32, numels[i] elements, read only
 *   numels[i]   >= 0; a tensor with 0 elements is skipped (its pointers may be NULL)
 *   weight_decay  host array of n finite values >= 0, or NULL for 0 everywhere
 *   lr          finite;  beta1, beta2 in [0, 1);  eps finite, >= 0
 *   step        >= 1 (t of the bias corrections: 1 on the first step)
 * Pointers as for muon_step (device, 4-byte aligned, no two arrays
 * overlapping).  n == 0 is a no-op; n <= MUON_ADAMW_MAX_TENSORS.  Uses no
 * workspace; its work list is cached per pointer set like the Muon plans.
 * lr, the betas, eps and step are launch arguments, and so is the first
 * non-zero weight_decay value, shared by every tensor that uses it: a
 * schedule of those values reuses the cached list.  Only a tensor whose
 * non-zero lambda differs from that shared value has its lambda cached with
 * the list.
 */
#define MUON_ADAMW_MAX_TENSORS 65536
int muon_adamw_step(float* const* params, const float* const* grads, float* const* exp_avg,
                    float* const* exp_avg_sq, const int64_t* numels, const float* weight_decay, int n,
                    float lr, float beta1, float beta2, float eps, int64_t step, hipStream_t stream);

/*
 * Delayed untying of a shared parameter (the "nanoGPT Speedrun Techniques:
 * How Delayed Untying Solves the Sparse Gradient Problem" page, section
 * "Option B: Delayed Untying"): the parameter and both of its AdamW moments
 * (rows x cols fp32 each, row-major) are copied into new buffers, so that the
 * new parameter's trajectory continues from the shared point instead of
 * restarting its moments.  transpose = 1 writes the copies as cols x rows
 * (an output layer stored d_model x vocab against a vocab x d_model
 * embedding); transpose = 0 copies as is.  rows, cols >= 1 with
 * rows * cols <= 2^40; all six pointers device, 4-byte aligned, no
 * destination overlapping another array.  Bit-exact copies.
 */
int muon_adamw_untie(const float* param, const float* exp_avg, const float* exp_avg_sq, float* new_param,
                     float* new_exp_avg, float* new_exp_avg_sq, int64_t rows, int64_t cols, int transpose,
                     hipStream_t stream);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* muon_last_error(void);

/*
 * Device workspace bytes a call over these shapes needs (bf16 iterates,
 * Gram and polynomial matrices, norm partials, fp32 partial tiles when a
 * long-K Gram product is cut into K chunks).  The plan's table block
 * (descriptors and work lists) is not part of it: each cached plan holds
 * its own small device allocation.  Pure host computation.  Returns 0 and
 * sets the error text for invalid shapes.
 */
size_t muon_workspace_bytes(const muon_shape_t* shapes, int n);

/*
 * Hand the library a caller-owned device workspace for the current device
 * (NULL/0 returns to library-owned workspace, allocated at the next call).
 * The caller keeps it alive until muon_release() or another
 * muon_set_workspace() call; calls that need more than `bytes` fail with
 * MUON_ENOMEM.  Waits for the device; plans on the previous workspace that
 * no captured graph uses are dropped.
 */
int muon_set_workspace(void* dev_ptr, size_t bytes);

/* Free the library's cached workspace and plans on all devices (synchronises). */
void muon_release(void);

/*
 * Counters of the current device's plan cache since it was created (or
 * since muon_release()), for diagnostics: out[0] plans built, out[1] table
 * uploads, out[2] pointer-write launches, out[3] device synchronisations,
 * out[4] plans evicted, out[5] workspace allocations.  out is a host array
 * of 6.  Never touches the device.
 */
int muon_plan_stats(int64_t out[6]);

/*
 * Concurrency of one call (1 .. 4, default 1; the setting is process-wide).
 * Matrices of one canonical shape (m x n, m <= n) form a group; with more
 * than one lane the groups are spread over up to `lanes` lanes, and each
 * lane runs its matrices' whole step on an internal stream of the library,
 * forked from the caller's stream (after everything enqueued there before the
 * call) and joined back to it, so that one group's kernels fill the GPU while
 * another's tail off.  1 keeps every kernel on the caller's stream.  Results
 * are bit-identical for any setting; under graph capture the lanes run one
 * after another on the capturing stream.  Kernel timing (below) brackets
 * each lane's launches on that lane's stream.
 */
int muon_set_lanes(int lanes);

/*
 * Kernel timing for measurement.  muon_timing_enable(k) brackets every
 * subsequent launch of kernel family k with HIP events on the launch stream;
 * k = -1 stops.  muon_timing_read waits for the recorded events and returns
 * the summed kernel time and the number of launches since the last read.
 */
#define MUON_KERNEL_MOMENTUM 0 /* momentum update + norm partial sums */
#define MUON_KERNEL_CAST 1     /* normalise + transpose + cast to bf16 */
#define MUON_KERNEL_GRAM 2     /* A = X X^T */
#define MUON_KERNEL_POLY 3     /* B = b A + c A A */
#define MUON_KERNEL_UPDATE 4   /* X <- a X + B X */
#define MUON_KERNEL_APPLY 5    /* W -= lr X */
#define MUON_KERNEL_ADAMW 6    /* multi-tensor AdamW (muon_adamw_step) */
int muon_timing_enable(int kernel);
int muon_timing_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H_ */
