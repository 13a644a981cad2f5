/*
 * rwkv8.h -- C ABI of the RWKV-8 rho / rho_norm recurrence in libwkv7, on
 * MI355X (gfx950): a second, diagonal-decay linear recurrence with a
 * normalised readout of the state before each step.
 *
 * The operation (burn_dragon_kernel page src/sequence/rwkv8/backward.rs:
 * compute_chunk_traces runs the "before" recurrences of rho and rho_norm on
 * delta = query (x) value; backward_chunk_impl's gradients fix the readout).
 * For every batch b and head h independently, with rho R[l][e] (l latent,
 * e embedding), rho_norm n[l] and the head's decay d[l], EPS = 1e-6:
 *
 *     y_t     = sum_l (q_t[l] / (sum_l' q_t[l'] + EPS)) R_t[l][:] / (n_t[l] + EPS)
 *     R_{t+1} = diag(d) R_t + q_t v_t^T
 *     n_{t+1} = d * n_t + q_t
 *
 * The backward returns the exact gradient of
 *     L = sum_t <dy_t, y_t> + <dR_T, R_T> + <dn_T, n_T>
 * with respect to q, v, the decay (summed over batch and time, as the page's
 * grad_decay) and the initial states.  (The page starts the reverse pass
 * from zero boundary gradients and drops the initial-state gradients; the
 * final-state gradient inputs and initial-state gradient outputs are the
 * extension the burn_mamba serial_recalculated backward.rs page makes with
 * d_final_state / d_initial_state.)
 *
 * Layouts, as on the page (fp32, row-major, contiguous, 16-byte aligned):
 *   q    [B][H][T][64]    (latent size L = 64)
 *   v    [B][Hv][T][64]   (embedding size E = 64; Hv = 1 shares one value
 *                          across the heads, as the page allows, else Hv = H)
 *   y, dy [B][H][T][64]
 *   rho  [B][H][64][64],  rho_norm [B][H][64],  decay [H][64]
 *   checkpoint record (rwkv8_checkpoint_bytes): [B][H][ceil(T/64)] blocks of
 *     64*64 + 64 floats, the rho and rho_norm before every 64th step (the
 *     page's per-chunk start states chunk_rho_start, chunk_rho_norm_start).
 *
 * Decay domain: the kernels form the recurrence over 16-step tiles with
 * decay powers relative to each tile's start, which needs every decay of a
 * head in [2^-7, 1].  A head with a decay outside that range (or NaN) gets
 * NaN in every output it owns and sets bit WKV7_FAULT_RWKV8_DECAY of the
 * device's fault word (wkv7_fault_status), so no finite wrong value is
 * returned.
 *
 * Ownership, execution and errors as for wkv7.h: device pointers owned by
 * the caller, work enqueued on `stream`, nothing allocated or synchronised,
 * every argument validated before anything is enqueued (WKV7_* statuses),
 * deterministic results (fixed summation orders, no float atomics).
 */
#ifndef RWKV8_H
#define RWKV8_H

#include "wkv7.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t B;     /* batch, >= 0 */
    int64_t T;     /* time steps, >= 0 */
    int64_t H;     /* heads, >= 0 */
    int64_t Hv;    /* value heads: 1 or H */
    int64_t L;     /* latent size: 64 */
    int64_t E;     /* embedding size: 64 */
} rwkv8_shape;

enum {
    WKV7_FAULT_RWKV8_DECAY = 2   /* fault bit: an RWKV-8 decay outside [2^-7, 1] */
};

/* Bytes of the checkpoint record: B*H*ceil(T/64)*(64*64 + 64)*4; 0 when the
 * shape is invalid. */
size_t rwkv8_checkpoint_bytes(const rwkv8_shape *shape);

/* Bytes of device workspace rwkv8_backward needs: the per-(b,h) decay
 * gradients (B*H*64 floats), the per-head value gradients when Hv = 1
 * (B*H*T*64 floats, summed over the heads in a fixed order), and the
 * checkpoint record when ckpt_provided is 0; each part 256-byte aligned.
 * 0 when the shape is invalid or empty. */
size_t rwkv8_backward_workspace_bytes(const rwkv8_shape *shape, int ckpt_provided);

/* Forward.  q, v, decay required (unless B*H*T == 0); rho0, norm0: carry-in
 * states, NULL = zeros; y, rhoT, normT, ckpt: outputs, each NULL to skip.
 * T == 0 copies the carry-in states to rhoT, normT.  No output may overlap an
 * input. */
int rwkv8_forward(const rwkv8_shape *shape, const float *q, const float *v, const float *decay,
                  const float *rho0, const float *norm0, float *y, float *rhoT, float *normT,
                  float *ckpt, hipStream_t stream);

/* Backward.  dy required; drhoT, dnormT: final-state gradients, NULL =
 * zeros; ckpt: the record a rwkv8_forward with the same inputs wrote, or NULL
 * to recompute it into the workspace (rho0, norm0 are read only then).
 * Outputs dq [B][H][T][64], dv [B][Hv][T][64] and ddecay [H][64] are
 * required; drho0 [B][H][64][64] and dnorm0 [B][H][64] may be NULL.  T == 0
 * gives drho0 = drhoT, dnorm0 = dnormT and a zero ddecay. */
int rwkv8_backward(const rwkv8_shape *shape, const float *q, const float *v, const float *decay,
                   const float *rho0, const float *norm0, const float *dy, const float *drhoT,
                   const float *dnormT, const float *ckpt, float *dq, float *dv, float *ddecay,
                   float *drho0, float *dnorm0, void *workspace, size_t workspace_bytes,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RWKV8_H */
