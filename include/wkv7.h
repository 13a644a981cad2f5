/*
 * wkv7.h -- C ABI of libwkv7: the WKV7 (RWKV-7) matrix-state recurrence and
 * its reverse (backward-through-time) scan on MI355X (gfx950).
 *
 * The operation (Foundry page "rwkvx/rx_pretrain.c": rx_wkv7_forward_seq for
 * the forward, rx_wkv7_backward and the comment block above it for the
 * reverse scan; the flat index helpers vx/sx there fix the layouts).  For
 * every batch b and head h independently, with S[i][j] (i = value row,
 * j = key column) starting at s0:
 *
 *     sa_t = S_{t-1} a_t
 *     S_t  = S_{t-1} diag(w_t) + v_t k_t^T + sa_t b_t^T
 *     y_t  = S_t r_t
 *
 * The backward returns the exact gradient of
 *     L = sum_t <dy_t, y_t> + <dsT, S_{T-1}>
 * with respect to r, w, k, v, a, b and s0.  (The page seeds the reverse scan
 * with a zero state gradient; the dsT input is the extension the burn_mamba
 * serial_recalculated backward.rs page makes with its d_final_state input.)
 * w is the multiplicative decay itself and dw is dL/dw for that multiplier.
 *
 * Layouts (all row-major, contiguous):
 *   vectors r, w, k, v, a, b, dy, y, dr, dw, dk, dv, da, db : [B][T][H][N]
 *   states  s0, sT, dsT, ds0                                 : [B][H][N][N] fp32
 *   checkpoint record ckpt (wkv7_checkpoint_bytes bytes, fp32):
 *     states  [B][H][ceil(T/C)][N][N] at offset 0; slot c holds the state
 *             before step c*C (slot 0 = s0, or zeros);
 *     sa tape [B][T][H][N] at byte offset roundup(states bytes, 256): the
 *             forward's sa_t = S_{t-1} a_t, so the backward regenerates
 *             states without recomputing these dot products.
 * Inputs r..b and dy are fp32 or bf16 (wkv7_shape.dtype); everything else,
 * including y and all gradients, is fp32.
 *
 * Ownership and execution: every pointer is caller-owned DEVICE memory,
 * 16-byte aligned.  Calls only enqueue work on `stream` (NULL = the default
 * stream) and return; the library never allocates, frees or synchronises.
 * Results are deterministic (fixed reduction order, no float atomics).
 * Apart from one fault word per device (wkv7_fault_status) and the test
 * hooks, there is no global mutable state: concurrent calls on different
 * streams are safe when their output buffers do not overlap.
 *
 * Errors: every argument is validated before anything is enqueued; a
 * negative status means nothing was written.  WKV7_ERR_HIP reports a launch
 * failure (from hipGetLastError) after validation passed.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of the inputs r, w, k, v, a, b and dy. */
typedef enum {
    WKV7_F32 = 0,
    WKV7_BF16 = 1
} wkv7_dtype;

/* How wkv7_backward computes the gradients (the results agree to rounding).
 *   AUTO    : the chunk form where it applies (N = 64, C = 64 and
 *             T*H*64*4 < 2^31 bytes), the step scan elsewhere.
 *   SCAN    : the step-by-step reverse scan: regenerate the states of a
 *             chunk from its checkpoint, then run the reverse recurrence.
 *   CHUNKED : the chunk form (WKV7_ERR_UNSUPPORTED where it does not apply,
 *             and where T*H*64*4 bytes, one batch row of a vector tensor,
 *             reach 2^31).
 *             Per 64-step chunk it runs only dsa = G b step by step and forms
 *             every gradient from dense products of the chunk's vectors with
 *             the checkpointed state and the incoming state gradient.  It
 *             takes decays w in [1/16, 1] whose product over a chunk stays
 *             above 2^-60; for a head whose inputs leave that range it falls
 *             back to SCAN for that head by itself.
 * The forward ignores this field. */
typedef enum {
    WKV7_ALGO_AUTO = 0,
    WKV7_ALGO_SCAN = 1,
    WKV7_ALGO_CHUNKED = 2
} wkv7_algo;

/* Bits of wkv7_shape.flags.
 *   WKV7_FUSED_INPUTS : the w, a, b arguments carry the time-mix values the
 *     Foundry rx_pretrain.c page forms them from in tm_pre_forward, and the
 *     library forms them itself: w holds the decay pre-activation omega
 *     (w = exp(-c * sigmoid(omega)), c = RX_WDECAY_COEFF = exp(-0.5)), a the
 *     normalised key kk (a = -kk) and b the gate ag (b = kk * ag).  The
 *     backward then returns d omega, d kk and d ag (the page's time-mix
 *     backward: dw * w * (-c) * sigmoid * (1 - sigmoid), -da + ag * db,
 *     kk * db) in the places of dw, da and db, saving the element-wise
 *     passes over those tensors before and after the scan.  Needs N = 64,
 *     C = 64 and, for T > 1, T*H*64*4 < 2^31 bytes, with algo AUTO or
 *     CHUNKED (WKV7_ERR_UNSUPPORTED otherwise); the checkpoint record of a
 *     fused forward is for a fused backward. */
enum {
    WKV7_FUSED_INPUTS = 1
};

typedef struct {
    int64_t B;      /* batch, >= 0 */
    int64_t T;      /* time steps, >= 0 */
    int64_t H;      /* heads, >= 0 */
    int64_t N;      /* head size; 16 and 64 are supported */
    int32_t dtype;  /* wkv7_dtype */
    int32_t chunk;  /* checkpoint interval C: 0 means 64; else a multiple of
                       8 in [8, 4096] */
    int32_t algo;   /* wkv7_algo (backward only) */
    int32_t flags;  /* 0 or WKV7_FUSED_INPUTS; other bits must be 0 */
} wkv7_shape;

enum {
    WKV7_OK = 0,
    WKV7_ERR_INVALID = -1,      /* NULL/misaligned pointer, negative size,
                                   bad dtype, chunk or algo, size overflow */
    WKV7_ERR_UNSUPPORTED = -2,  /* N not in {16, 64}; CHUNKED or fused
                                   inputs where they do not apply */
    WKV7_ERR_WORKSPACE = -3,    /* workspace missing or too small */
    WKV7_ERR_HIP = -4           /* a kernel launch failed */
};

/* Bytes of the checkpoint record for `shape`.  The record replaces the
 * page's cache of every state in rx_wkv7_backward with the state at the
 * start of every C-step chunk, from which the backward recomputes the
 * chunk (the per-chunk start states of the burn_dragon_kernel
 * src/sequence/rwkv8/backward.rs page, chunk_rho_start, are the prior art):
 * roundup(B*H*ceil(T/C)*N*N*4, 256) + B*T*H*N*4 bytes; 0 when the shape
 * is invalid.
 * Shapes of few, long sequences run split into segments (N = 64, C = 64,
 * T*H*64*4 < 2^31, B*H <= 64, at least 4 chunks; the count, up to 8, and
 * the segment length follow from the shape): their record rounds the sa
 * part up to 256 bytes and adds the segments' transition products,
 * B*H*nseg*N*N*4 bytes.  A wkv7_forward with no record runs split when it
 * writes y and the last segment has at least N steps, keeping the carries
 * between segments in y's own rows until the segments overwrite them with
 * their outputs. */
size_t wkv7_checkpoint_bytes(const wkv7_shape *shape);

/* Bytes of device workspace wkv7_backward needs (this library's own
 * layout; the pages have no such buffer): the per-(b,h) state
 * sub-checkpoints of one chunk and one int per (b,h) (for a split shape
 * also one int and one N x N fp32 state gradient per (b,h) and segment),
 * plus room for the checkpoint record itself when `ckpt_provided` is 0.
 * 0 when the shape is invalid or empty. */
size_t wkv7_backward_workspace_bytes(const wkv7_shape *shape, int ckpt_provided);

/* Forward scan (rx_wkv7_forward_seq on the Foundry rx_pretrain.c page).
 *   r, w, k, v, a, b : inputs, [B][T][H][N], dtype per shape->dtype; required
 *                      unless B*T*H == 0.
 *   s0   : initial state, fp32 [B][H][N][N]; NULL means zeros.
 *   y    : output, fp32 [B][T][H][N]; NULL skips it.
 *   sT   : final state, fp32 [B][H][N][N]; NULL skips it.
 *   ckpt : checkpoint record for wkv7_backward, wkv7_checkpoint_bytes(shape)
 *          bytes (states every C steps and the per-step sa); NULL skips it.
 * With T == 0, sT receives s0 (or zeros).  T == 1 (one decode step of
 * batched inference from a carry-in state) runs a single-step kernel that
 * streams each (b, h)'s state through once; there sT may be s0 itself (the
 * state is updated in place).  Otherwise no output may overlap an input. */
int wkv7_forward(const wkv7_shape *shape,
                 const void *r, const void *w, const void *k, const void *v,
                 const void *a, const void *b, const float *s0,
                 float *y, float *sT, float *ckpt, hipStream_t stream);

/* Reverse scan (rx_wkv7_backward on the Foundry rx_pretrain.c page, seeded
 * with dsT).
 *   r..b, dy : inputs as for the forward; dy is dL/dy, [B][T][H][N].
 *   s0   : the forward's initial state (NULL = zeros); read only when
 *          ckpt is NULL.
 *   dsT  : dL/d(final state), fp32 [B][H][N][N]; NULL means zeros.
 *   ckpt : the checkpoint record a wkv7_forward call with the same inputs,
 *          s0 and chunk wrote; NULL makes the backward recompute it into the
 *          workspace first.
 *   dr, dw, dk, dv, da, db : outputs, fp32 [B][T][H][N], all required.
 *   ds0  : dL/ds0, fp32 [B][H][N][N]; NULL skips it.
 *   workspace, workspace_bytes : device scratch of at least
 *          wkv7_backward_workspace_bytes(shape, ckpt != NULL) bytes; its
 *          contents on entry do not matter.
 * With T == 0, ds0 receives dsT (or zeros). */
int wkv7_backward(const wkv7_shape *shape,
                  const void *r, const void *w, const void *k, const void *v,
                  const void *a, const void *b, const float *s0,
                  const void *dy, const float *dsT, const float *ckpt,
                  float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                  float *ds0, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* wkv7_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results (bit
 * for bit) and errors as wkv7_backward, except that the workspace is the
 * library's own fixed device array of WKV7_NOALLOC_SCRATCH_BYTES bytes per
 * GPU, which each GPU the library runs on holds until the process ends.  A
 * shape whose workspace (wkv7_backward_workspace_bytes(shape, ckpt != NULL))
 * exceeds that size returns WKV7_ERR_WORKSPACE before anything is enqueued.
 * The call allocates and frees nothing.  Calls that overlap on one GPU (on
 * different streams, or from different threads) share the array and race:
 * order them on one stream. */
#define WKV7_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int wkv7_backward_noalloc(const wkv7_shape *shape,
                          const void *r, const void *w, const void *k, const void *v,
                          const void *a, const void *b, const float *s0,
                          const void *dy, const float *dsT, const float *ckpt,
                          float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                          float *ds0, hipStream_t stream);

/* The time-mix epilogue after the scan, N = 64 (Foundry page
 * "rwkvx/rx_pretrain.c": gn_forward, the bonus term and the gate g applied
 * to the scan's output in rx_timemix_forward_seq, and the per-token
 * post-processing backward of its backward), per (b, t, h) over the head's
 * 64 entries:
 *   z = ((y - mean) * rstd * ln_w + ln_b + s * v) * g,
 *   rstd = 1 / sqrt(var + 64e-5),  s = sum_j r_j * k_j * r_k[j].
 * One pass over the tensors each way.  The output projection that follows on
 * the page is not part of it.
 *   y, dz      : fp32 [B][T][H][64]; r, k, v, g: [B][T][H][64], dtype per
 *                shape->dtype (the scan's r, k, v and the gate).
 *   ln_w, ln_b, r_k : fp32 [H][64] per-channel parameters.
 *   z          : fp32 [B][T][H][64] output.
 * The backward returns dy (the scan's output gradient, to hand to
 * wkv7_backward), dg, the bonus term's shares of dr, dk, dv (to add to the
 * scan's), all fp32 [B][T][H][64], and dln_w, dln_b, dr_k (fp32 [H][64],
 * summed over b and t in a fixed order: reproducible bit for bit), with a
 * workspace of wkv7_epilogue_workspace_bytes(shape) bytes, 256-byte
 * aligned.  The shape's chunk, algo and flags fields must be valid and are
 * otherwise unused.  N != 64 is WKV7_ERR_UNSUPPORTED; no output may overlap
 * an input; B*T == 0 gives zero parameter gradients. */
size_t wkv7_epilogue_workspace_bytes(const wkv7_shape *shape);
int wkv7_epilogue_forward(const wkv7_shape *shape, const float *y, const void *r, const void *k,
                          const void *v, const void *g, const float *ln_w, const float *ln_b,
                          const float *r_k, float *z, hipStream_t stream);
int wkv7_epilogue_backward(const wkv7_shape *shape, const float *dz, const float *y, const void *r,
                           const void *k, const void *v, const void *g, const float *ln_w,
                           const float *ln_b, const float *r_k, float *dy, float *dg, float *dr,
                           float *dk, float *dv, float *dln_w, float *dln_b, float *dr_k,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char *wkv7_status_string(int status);

/* Fault bits of the current device.  The N = 64 forward's helper waves wait
 * for each other with a bounded poll (about 30 ms per wait; a correct build
 * never reaches the bound).  A wait that gives up makes its workgroup
 * overwrite every output it wrote (its y and sa-tape rows, checkpoint slots
 * and final state) with NaN and sets bit 0 of a per-device fault word, so
 * that no finite wrong value is returned silently.  This call waits for
 * `stream` (the only call in the library that synchronises), stores the bits
 * in *faults and clears them when `clear` is non-zero.  Returns WKV7_OK,
 * WKV7_ERR_INVALID (faults NULL) or WKV7_ERR_HIP. */
enum {
    WKV7_FAULT_HELPER_WAIT = 1
};
int wkv7_fault_status(unsigned *faults, int clear, hipStream_t stream);

/* Test hooks, for the library's own tests only (process-global, not
 * thread-safe, never needed by a caller):
 *   WKV7_HOOK_FAULT_INJECT, value 0 or 1: with 1, every workgroup of the
 *     N = 64 forward reports a given-up helper wait (NaN outputs, fault bit)
 *     although every wait still completes normally;
 *   WKV7_HOOK_FAIL_LAUNCHES, value n >= 0: the next n calls that enqueue
 *     work return WKV7_ERR_HIP as if their launch had failed (their work is
 *     still enqueued).
 * Returns WKV7_OK, or WKV7_ERR_INVALID for an unknown hook or value. */
enum {
    WKV7_HOOK_FAULT_INJECT = 1,
    WKV7_HOOK_FAIL_LAUNCHES = 2
};
int wkv7_test_hook(int hook, int64_t value);

/* ABI version (major * 100 + minor). */
int wkv7_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
