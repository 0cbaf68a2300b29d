/*
 * rwkv_wkv.h -- C ABI of librwkv_wkv, the RWKV-4 time-mixing WKV operator on gfx950.
 *
 * Operator. For one sequence b and one channel c, with 0-based token index t:
 *
 *     y_t = ( sum_{i<t} e^{-(t-1-i) w + k_i} v_i  +  e^{u + k_t} v_t )
 *         / ( sum_{i<t} e^{-(t-1-i) w + k_i}      +  e^{u + k_t}     )
 *
 * a weighted average of v in which older tokens decay with their distance through one
 * per-channel rate w, the current token gets a per-channel bonus u, and channels are
 * independent ("RWKV解读：在Transformer的时代的新RNN", section 二.3 "RWKV的网络架构",
 * formula (8); "RWKV についての調査記録", section 【wkvとは】). The same values have a
 * recursive form (formula (8) remark on the first page), which is what the decode entry
 * point advances one token at a time ("RWKV についての調査記録", section "RWKVとは？":
 * at inference the model takes a token and a state and returns the new state).
 *
 * Conventions shared by every entry point:
 *   - All tensors are fp32, dense, row-major, and live in device memory owned by the
 *     caller. k, v, y, dy, dk, dv are [B][T][C] with C fastest; decode tensors and the
 *     state are [B][C]; w, u, dw, du are [C].
 *   - w is the positive decay rate itself (weight of a token i steps back beyond the
 *     previous one is e^{-i w}); it is not log w and not -w. Results are unspecified for
 *     w < 0, for non-finite inputs, and for |v| > 1e20.
 *   - Outputs must not alias inputs, except the decode state, which is updated in place.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call
 *     validates its arguments on the host, enqueues its kernels on `stream` and returns
 *     without synchronizing; a kernel fault surfaces at the caller's next synchronization.
 *   - Every call returns WKV_OK (0) or an error code. Argument errors are detected before
 *     any HIP call and launch nothing; the message of the last failing call on the
 *     calling thread is available from wkv_last_error(). A zero-sized dimension is a
 *     successful no-op (dw and du are zero-filled when C > 0 and B*T == 0).
 *   - The library allocates no device memory, with one exception: wkv_forward, whose
 *     signature has no workspace, takes its scan's scratch from the current device's
 *     stream-ordered memory pool (hipMallocAsync) and returns it (hipFreeAsync), both on
 *     `stream`, within the call. Every other entry point uses only memory the caller passes,
 *     except wkv_forward_noalloc, whose scratch is a static array of the library's code
 *     object (64 MiB on each GPU it is loaded on, held until the process ends).
 *
 * Entry points. wkv_forward, wkv_backward_workspace_size, wkv_backward and wkv_decode_step
 * are the operator's three calls with the plainest boundary: a forward that writes y, a
 * backward that needs nothing from the forward (it recomputes what it needs into its
 * workspace), and a decode step. Training code that runs a backward after every forward
 * should use the pair wkv_forward_train / wkv_backward_train instead, which hands the
 * window states from the forward to the backward through a workspace and so saves the
 * backward a pass over k and v. The other entry points add the gate, 16-bit storage, a
 * state in and out, and the token-shift mix.
 */
#ifndef RWKV_WKV_H
#define RWKV_WKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV_OK 0
#define WKV_ERR_INVALID_ARG 1 /* null pointer with a nonzero size, negative or too large dim, short buffer */
#define WKV_ERR_UNSUPPORTED 2 /* the current device is not gfx950 */
#define WKV_ERR_HIP 3         /* a HIP runtime call or kernel launch failed */

/* Storage formats of the [B][T][C] tensors for the *_typed entry points. */
#define WKV_F32 0  /* IEEE binary32 */
#define WKV_BF16 1 /* bfloat16: the upper half of a binary32 */
#define WKV_F16 2  /* IEEE binary16 */

/* Library version, as 10000*major + 100*minor + patch. */
int wkv_version(void);

/* The look-back's patience, for every later call from any thread: how many times a
 * workgroup re-reads the flag of a window that has published nothing yet (an earlier
 * window in the forward, a later one in the backward) before it recomputes that window's
 * aggregate from the inputs itself. The scan is canonical, so results are bitwise the same
 * whatever the value; it trades waiting for recomputation. `tries` >= 0 (default 2000; 0
 * recomputes whenever a flag is not already there, which tests use to drive that path).
 * Returns WKV_OK, or WKV_ERR_INVALID_ARG for a negative count. */
int wkv_set_poll_limit(int tries);
int wkv_poll_limit(void);

/* Static description of a status code ("ok", "invalid argument", ...). Never NULL. */
const char *wkv_status_string(int status);

/* Message of the last failing call made by this thread ("" if none). Never NULL. */
const char *wkv_last_error(void);

/* Forward: y [B][T][C] from k, v [B][T][C] and w, u [C], starting from the empty state
 * (formula (8) of "RWKV解读：在Transformer的时代的新RNN", section 二.3). The scan's scratch
 * (publication flags and per-window records, fwd_scan_bytes: 48 bytes per 64 tokens and
 * channel plus 8 per window and 64 channels) comes from the stream-ordered pool for the
 * duration of the call; an allocation failure returns WKV_ERR_HIP. Keeps nothing for a
 * backward (see wkv_forward_train). Requires C <= 2^24 and B*ceil(C/64)*ceil(T/64) < 2^31. */
int wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                const float *k, const float *v, float *y, void *stream);

/* wkv_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same scan and bitwise the
 * same y, with its scratch (the flags and window records, wkv_forward_noalloc_scratch_bytes
 * bytes) in an array of wkv_forward_noalloc_max_scratch() bytes (64 MiB) that the library
 * holds on every GPU it runs on until the process ends. No allocation of any kind happens
 * in the call. Sizes whose scratch exceeds the array are refused with WKV_ERR_INVALID_ARG
 * before any launch (the 3B-class layer, B=8 T=4096 C=2560, needs 63 MB). Calls on one GPU
 * share the array: two such calls that overlap in time on the same GPU (different streams,
 * or concurrent host threads) race and must not be made; calls one after another on a
 * stream are fine (nothing needs clearing between them). */
int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                        const float *k, const float *v, float *y, void *stream);
/* Scratch wkv_forward_noalloc needs for (B, T, C) (0 for invalid dims), and the most it can
 * take. */
size_t wkv_forward_noalloc_scratch_bytes(int64_t B, int64_t T, int64_t C);
size_t wkv_forward_noalloc_max_scratch(void);

/* Bytes of device scratch that wkv_forward_train and wkv_forward_state need for (B, T, C):
 * a 256-byte stamp, publication flags plus, for every (b, c) sequence and every 64-token
 * window, the window's aggregate and the recurrent state after it, the state entering the
 * window's second 32-token chunk (each: the two sums of the recursive form, their
 * age-weighted counterparts and their scale, 40 bytes), and per (b, c) the state before
 * token 0 and the final state. Returns 0 for invalid dims. */
size_t wkv_forward_workspace_size(int64_t B, int64_t T, int64_t C);

/* The training forward: y as wkv_forward, plus the window states a backward reads, left in
 * `workspace` (16-byte aligned, at least wkv_forward_workspace_size(B, T, C) bytes given in
 * `workspace_bytes`; required whenever B*T*C > 0; its previous content is ignored). Pass
 * the same workspace to wkv_backward_train (or wkv_backward_gated/typed) for the same
 * inputs; it must not be used by two calls at the same time. The workspace is stamped with
 * what the call left in it, which the backward checks. */
int wkv_forward_train(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, float *y, void *workspace,
                      size_t workspace_bytes, void *stream);

/* Forward from a given state, leaving the state after the last token: the T tokens run as
 * in wkv_forward, but the scan starts from the decode state (a, b, p) [B][C] (same meaning
 * as in wkv_decode_step: A = a e^p, B = b e^p) instead of the empty one, and a, b, p are
 * overwritten with the state after token T-1, ready for wkv_decode_step. This is the
 * prompt-then-generate use of the recursive form ("RWKV についての調査記録", section
 * "コードを見ながらRWKVの構造を把握": the prompt's tokens go through the layer one after
 * another, each updating the state, before the next token is predicted), with the prompt
 * run in parallel. y and the workspace are as for wkv_forward_train (same size); a
 * wkv_backward_train given this workspace treats the initial state as a constant,
 * wkv_backward_state also gives the gradient with respect to it (and takes one for the
 * final state).
 * The final state is accurate to fp32 (p is rounded first, a and b rescaled to match).
 * a, b, p must not overlap each other, k, v, y, w, u or the workspace. A zero-sized
 * dimension is a no-op that leaves the state unchanged. */
int wkv_forward_state(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, float *y, float *a, float *b, float *p,
                      void *workspace, size_t workspace_bytes, void *stream);

/* The gated forward: out = sigma(r) * y elementwise, sigma(x) = 1 / (1 + e^{-x}), with y as in
 * wkv_forward and r [B][T][C] the receptance: the time-mixing block passes the WKV result
 * through a sigmoid gate of r ("RWKV解读：在Transformer的时代的新RNN", section 二.3: R is
 * sigmoid-activated, a forgetting mechanism, formula (9); "RWKV についての調査記録", section
 * "コードを見ながらRWKVの構造を把握": wkv is computed, then gated by sigma). y itself is
 * not written. The workspace is as for wkv_forward_train and serves wkv_backward_gated (or
 * wkv_backward_train) the same way. out must not overlap any input. */
int wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, const float *r, float *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* wkv_forward_train (r == NULL) or wkv_forward_gated (r != NULL) with k, v, r and y/out in the
 * storage format `dtype` (WKV_F32, WKV_BF16 or WKV_F16); w and u stay fp32. Values are
 * widened to fp32 on load; every sum, carry and state is kept in fp32/fp64 as in the fp32
 * entry points, and only the outputs are rounded to the format (to nearest even). 16-bit
 * tensors must be 2-byte aligned. The workspace is the same as wkv_forward_train's. */
int wkv_forward_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                      const float *u, const void *k, const void *v, const void *r, void *y,
                      void *workspace, size_t workspace_bytes, void *stream);

/* The forward for inference, where no backward follows: wkv_forward_typed (r == NULL) or
 * its gated form (r != NULL), from a given state if a, b, p are given (all three, as in
 * wkv_forward_state, overwritten with the state after token T-1) or from the empty state if
 * all three are NULL. Outputs and final state are bitwise those of the training entry
 * points; the workspace (wkv_forward_workspace_size bytes) is left without the states a
 * backward reads (their age-weighted sums are never formed and the carries entering the
 * windows' second chunks and token 0 are not stored), so it must not be passed to
 * a backward: a backward given it is refused (WKV_ERR_INVALID_ARG when this process filled
 * it; otherwise its dw, du come out NaN, from the workspace's stamp). This is the prompt
 * prefill of "RWKV についての調査記録", section "コードを見ながらRWKVの構造を把握" (the
 * prompt's tokens update the state in order) run in parallel, with 1.1 bytes per element
 * less workspace traffic than wkv_forward_state. */
int wkv_forward_infer(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                      const float *u, const void *k, const void *v, const void *r, void *y,
                      float *a, float *b, float *p, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Bytes of device scratch that wkv_backward needs for (B, T, C): its own records (flags,
 * reverse window records, per-window dw/du partials) plus room for the forward window
 * states it recomputes. Returns 0 for invalid dims. */
size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C);

/* Backward of L = sum_{b,t,c} dy[b,t,c] * y[b,t,c] ("RWKV についての調査記録", section
 * "Trainingについて": all parameters get gradients): dk, dv [B][T][C] and dw, du [C],
 * where dw and du are summed over b and t and overwritten (not accumulated). dw is the
 * gradient with respect to w itself (a caller that stores d = log w uses w * dw). Needs
 * nothing from a forward: the window states are recomputed from k, v into `workspace`
 * (16-byte aligned, wkv_backward_workspace_size(B, T, C) bytes given in `workspace_bytes`),
 * which is clobbered. dw and du are summed in a fixed order and are bitwise reproducible
 * run to run. */
int wkv_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                 const float *k, const float *v, const float *dy, float *dk, float *dv,
                 float *dw, float *du, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device scratch that wkv_backward_train needs (its own records only: the forward
 * window states come from the forward's workspace). Returns 0 for invalid dims. */
size_t wkv_backward_train_workspace_size(int64_t B, int64_t T, int64_t C);

/* wkv_backward after wkv_forward_train: `fwd_workspace` is the workspace that call filled
 * for the same B, T, C, w, u, k, v (only read; required). Its window states replace the
 * backward's own pass over k and v, and `workspace` needs only
 * wkv_backward_train_workspace_size(B, T, C) bytes. Results are bitwise those of
 * wkv_backward. A workspace that an inference forward (wkv_forward_infer) or a forward of
 * other sizes last filled is refused with WKV_ERR_INVALID_ARG when this process filled it;
 * a mismatch the library cannot see on the host (a workspace filled elsewhere) makes dw and
 * du NaN through the workspace's stamp. */
int wkv_backward_train(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *dy,
                       const void *fwd_workspace, float *dk, float *dv, float *dw, float *du,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes that wkv_backward_gated, wkv_backward_typed, wkv_backward_state and their typed
 * forms need: with have_fwd_workspace != 0 the caller passes the workspace a state-keeping
 * forward filled for the same inputs (= wkv_backward_train_workspace_size); with 0 the window
 * states are recomputed into this workspace (= wkv_backward_workspace_size). */
size_t wkv_backward_workspace_size_ex(int64_t B, int64_t T, int64_t C, int have_fwd_workspace);

/* wkv_backward for a forward from a state (wkv_forward_state, whose workspace must be
 * given as `fwd_workspace`: it records the state the forward started from and the one it
 * returned, so the caller need not keep them), for a sequence trained in pieces, each
 * resuming from the state the previous one left ("RWKV についての調査記録", section
 * "RWKVとは？": the state carries the past; the recursive form of formula (8) of
 * "RWKV解读：在Transformer的时代的新RNN", section 二.3, run over the pieces in turn).
 *
 * L = sum_{b,t,c} dy[b,t,c] y[b,t,c] + sum_{b,c} (dfa[b,c] a_T[b,c] + dfb[b,c] b_T[b,c]),
 * where (a_T, b_T, p_T) is the state the forward returned (p_T held fixed; A_T = a_T e^{p_T})
 * and dfa, dfb [B][C] its cotangent from the next piece (that piece's da, db), or both NULL
 * (then L is wkv_backward's). Outputs: dk, dv, dw, du as in wkv_backward, and da, db, dp
 * [B][C] fp32 (overwritten), the gradient with respect to the state (a, b, p) the forward
 * started from. The state before token 0 reaches token t only through A0 e^{-t w} and
 * B0 e^{-t w}, so with the future sums G = sum_t e^{-t w} dy_t / D_t and H = sum_t e^{-t w}
 * dy_t y_t / D_t (D_t the denominator at token t): da = G e^p, db = -H e^p, dp = (a G -
 * b H) e^p, plus with dfa, dfb the path through the final state (A_T holds e^{-T w} A0).
 * dp = a da + b db always (L depends on a, p only through a e^p). A forward from the empty
 * state (wkv_forward_train, or a = b = 0) gives da = db = dp = 0. Without dfa, dfb: dk,
 * dv, dw, du are bitwise those of wkv_backward_train with the same arguments; with them the final
 * state acts as one more token at T in the future sums of all earlier tokens (the reverse
 * scan starts from it), at about 3% more time. T == 0 writes zero da, db,
 * dp, dw, du, but is refused with dfa, dfb (a zero-length piece records no state: its
 * final state's cotangent is its initial state's, which the caller passes on). Outputs
 * must not overlap each other or any input. */
int wkv_backward_state(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *dy, const float *dfa,
                       const float *dfb, const void *fwd_workspace, float *dk, float *dv,
                       float *dw, float *du, float *da, float *db, float *dp,
                       void *workspace, size_t workspace_bytes, void *stream);

/* wkv_forward_state and wkv_backward_state for the other storage formats and the gate, as
 * wkv_forward_typed / wkv_backward_typed are for the training pair: k, v, dy, r,
 * y, dk, dv, dr in the format `dtype` (WKV_F32, WKV_BF16 or WKV_F16), with r == NULL (and
 * dr == NULL) for the plain operator or the receptance gate out = sigma(r) * y (dy then the
 * cotangent of out). w, u, the state a, b, p, its cotangent dfa, dfb, and dw, du, da, db,
 * dp stay fp32. wkv_forward_state_typed keeps the states its backward reads (unlike
 * wkv_forward_infer, whose outputs it shares bitwise); a, b, p all or none. Arithmetic,
 * workspaces and errors as in the fp32 entry points. */
int wkv_forward_state_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                            const float *u, const void *k, const void *v, const void *r,
                            void *y, float *a, float *b, float *p, void *workspace,
                            size_t workspace_bytes, void *stream);
int wkv_backward_state_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                             const float *u, const void *k, const void *v, const void *dy,
                             const void *r, const float *dfa, const float *dfb,
                             const void *fwd_workspace, void *dk, void *dv, void *dr,
                             float *dw, float *du, float *da, float *db, float *dp,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Backward of the gated forward, L = sum dout * sigma(r) * y: as wkv_backward with the
 * cotangent dy = dout * sigma(r) formed on the fly, plus dr [B][T][C] =
 * dout * sigma(r) * (1 - sigma(r)) * y (y recomputed, never read). `fwd_workspace` is NULL
 * (states recomputed; workspace as for wkv_backward) or the workspace wkv_forward_gated (or
 * wkv_forward_train) filled for the same inputs (workspace as for wkv_backward_train). */
int wkv_backward_gated(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *r, const float *dout,
                       const void *fwd_workspace, float *dk, float *dv, float *dr, float *dw,
                       float *du, void *workspace, size_t workspace_bytes, void *stream);

/* wkv_backward / wkv_backward_train (r == dr == NULL; dy is the cotangent of y;
 * fwd_workspace NULL or not) or wkv_backward_gated (r, dr given; dy is the cotangent of the
 * gated output) with k, v, dy, r, dk, dv, dr in the storage format `dtype`; w, u, dw, du
 * stay fp32. Arithmetic as in the fp32 entry points; dk, dv, dr are rounded to the format on
 * store. Workspace size: wkv_backward_workspace_size_ex(B, T, C, fwd_workspace != NULL). */
int wkv_backward_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                       const float *u, const void *k, const void *v, const void *dy,
                       const void *r, const void *fwd_workspace, void *dk, void *dv, void *dr,
                       float *dw, float *du, void *workspace, size_t workspace_bytes,
                       void *stream);

/* One decode step for B sequences (the recursive form; "RWKV についての調査記録",
 * section "RWKVとは？"). k, v, y are [B][C]; the state is three [B][C] arrays a, b, p
 * meaning A = a e^p, B = b e^p, where A and B are the decayed sums of e^{k_i} v_i and
 * e^{k_i} over the tokens seen so far; the empty state is a = b = 0, p = -1e38.
 * y is computed from the state before the update, then the state is advanced by the
 * token in place. Any rescaled equivalent (a e^d, b e^d, p - d) is the same state. */
int wkv_decode_step(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                    const float *v, float *a, float *b, float *p, float *y, void *stream);

/* wkv_decode_step with k, v and y [B][C] in the storage format `dtype` (WKV_F32, WKV_BF16 or
 * WKV_F16; 16-bit tensors 2-byte aligned): k, v are widened to fp32 on load and y is rounded
 * to the format (to nearest even) on store; w, u and the state a, b, p stay fp32, so the
 * state carries the same precision as in wkv_decode_step (a serving loop whose activations
 * are 16-bit decodes with 30 instead of 36 bytes per element). Same recursive form ("RWKV
 * についての調査記録", section "RWKVとは？"), validation and errors. */
int wkv_decode_step_typed(int dtype, int64_t B, int64_t C, const float *w, const float *u,
                          const void *k, const void *v, float *a, float *b, float *p, void *y,
                          void *stream);

/* Token-shift mix, the step that produces the inputs of the R, K, V projections
 * ("RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (7): they are computed from a
 * weighted sum of the current and the previous token's input, one trained per-channel weight
 * each): for x [B][T][C] and mu [3][C] (rows r, k, v),
 *     out_m[b][t][c] = mu[m][c] x[b][t][c] + (1 - mu[m][c]) x[b][t-1][c],   m = r, k, v,
 * where x[b][-1] is x_prev[b] ([B][C]; NULL means zeros, a fresh sequence). x_last ([B][C])
 * receives x[b][T-1] (the next call's x_prev) unless NULL. Outputs must not overlap inputs. */
int wkv_token_shift(int64_t B, int64_t T, int64_t C, const float *x, const float *x_prev,
                    const float *mu, float *out_r, float *out_k, float *out_v, float *x_last,
                    void *stream);

/* Bytes of device scratch wkv_token_shift_backward needs (fp64 partials of dmu). */
size_t wkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C);

/* Backward of L = sum_m sum dout_m * out_m: dx [B][T][C], dx_prev [B][C] (unless NULL) and
 * dmu [3][C], the last summed over b and t in a fixed order and overwritten. */
int wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, const float *x,
                             const float *x_prev, const float *mu, const float *dout_r,
                             const float *dout_k, const float *dout_v, float *dx, float *dx_prev,
                             float *dmu, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RWKV_WKV_H */
