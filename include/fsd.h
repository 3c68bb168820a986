/*
 * fsd.h — C ABI of the hot path of a three-step video refiner on AMD MI355X
 * (gfx950): the LoRA-fused linear that every refinement step evaluates, and
 * the renoise / Euler arithmetic on the latent around it.
 *
 * Sources (the method's definition):
 *   [EN]  "Open-H3-Regenerate-2K: High-Resolution Video Refinement with
 *          Few-Step Diffusion" (agientry.com, English article)
 *   [CW]  "Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案"
 *          (comfyui-wiki.com news page)
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers (hipMalloc'd or equivalent), except
 *     where a parameter says "host".  The caller owns every buffer, including
 *     the workspace; the library never allocates, frees or synchronises and
 *     keeps no state between calls (calls are reentrant).
 *   - bf16 means IEEE binary32 truncated to its top 16 bits (bfloat16), stored
 *     as 2-byte little-endian words.  fp32 is IEEE binary32.
 *   - Matrices are row-major.  "ld" is the row stride in ELEMENTS.
 *   - Every bf16 matrix pointer must be 16-byte aligned and every ld a
 *     multiple of 8 elements, so each row starts on a 16-byte boundary;
 *     fp32 vectors of the sampler must be 16-byte aligned.
 *   - stream is a hipStream_t; NULL means the default stream.  Calls enqueue
 *     and return.  The returned status covers argument validation (done before
 *     any HIP call) and the launch itself (FSD_EHIP if the launch failed).
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Nothing is printed and no exception crosses the boundary.
 *   - All kernels are deterministic: the same inputs give bitwise-identical
 *     outputs (no atomics, no split reductions whose order varies).
 */
#ifndef FSD_H
#define FSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSD_ABI_VERSION 1

typedef enum {
  FSD_OK = 0,
  FSD_EINVAL = 1,        /* null pointer, bad size, bad ld, illegal aliasing, non-finite sigma */
  FSD_EALIGN = 2,        /* pointer or ld not 16-byte aligned                                   */
  FSD_EUNSUPPORTED = 3,  /* valid request that this library does not implement                  */
  FSD_EWORKSPACE = 4,    /* workspace null or too small                                         */
  FSD_EHIP = 5           /* the HIP runtime reported an error when launching                    */
} fsd_status;

typedef enum {
  FSD_EPI_NONE = 0,      /* Y = acc (+ bias) (+ residual)                                   */
  FSD_EPI_SWIGLU = 1     /* Y[:, j] = silu(acc[:, j]) * acc[:, F + j], F = N / 2 (see below) */
} fsd_epilogue;

/* Version of this header's ABI (FSD_ABI_VERSION). */
int fsd_abi_version(void);

/* Static, NUL-terminated name of a status code ("FSD_OK", ...); never NULL
 * (values outside fsd_status give "FSD_UNKNOWN"). */
const char* fsd_status_str(fsd_status status);

/* ------------------------------------------------------------------------ *
 * a0. Rank-axis merge of several LoRA adapters into one                      *
 * ------------------------------------------------------------------------ *
 * [CW] section "三个步如何完成工作": the refiner (rank 384), the Turbo
 * adapter (rank 128) and the Sharp adapter (rank 64) are merged into one
 * rank-576 LoRA by concatenating their factors along the rank axis, stored in
 * fp32.  Concatenation along rank makes B·A equal the sum of the adapters'
 * B_i·A_i, which is what the merge check on that page verifies.
 *
 *   A = [A_0; A_1; ...]              (rows stacked)      -> bf16 [R, K]
 *   B = [s_0·B_0 | s_1·B_1 | ...]    (columns stacked)   -> bf16 [N, R]
 *   R = sum of ranks[i]
 *
 * A_list, B_list, ranks, scales: HOST arrays of n_adapters entries.
 *   A_list[i]: device fp32 [ranks[i], K] row-major (ld = K).
 *   B_list[i]: device fp32 [N, ranks[i]] row-major (ld = ranks[i]).
 *   scales:    per-adapter strength s_i folded into B_i; NULL means all 1.
 * A_out: device bf16 [R, K]; B_out: device bf16 [N, R].
 * Each output element is s_i·b rounded once to fp32 (exact when s_i = 1) and
 * then to bf16 by round-to-nearest-even: the result is bit-exact.
 * Requirements: 1 <= n_adapters <= 16, ranks[i] >= 1, K >= 1, N >= 1,
 * A_out/B_out 16-byte aligned; outputs must not overlap inputs.
 */
int fsd_lora_merge(int n_adapters, const float* const* A_list,
                   const float* const* B_list, const int64_t* ranks,
                   const float* scales, int64_t K, int64_t N,
                   void* A_out, void* B_out, void* stream);

/* ------------------------------------------------------------------------ *
 * a2 + a3 (+ a4). LoRA-fused linear                                         *
 * ------------------------------------------------------------------------ *
 * [CW] section "三个步如何完成工作": each of the transformer's adapted linear
 * layers carries the merged rank-576 LoRA; [EN] section "Three steps instead
 * of dozens": every refinement step is one call of that transformer.  A linear
 * layer with a LoRA computes
 *
 *   Y = X·W0ᵀ + s·(X·Aᵀ)·Bᵀ (+ bias) (+ residual)
 *
 * evaluated here as two kernels:
 *   phase A (fsd_lora_down):  T = bf16(s · X·Aᵀ)                [M, r]
 *   phase B (fsd_lora_up):    Y = [X | T]·[W0 | B]ᵀ + bias ...  one MFMA
 *                             K-loop over K + r columns, then the epilogue.
 * T is the only intermediate; it lives in the caller's workspace.
 *
 * Operands (all bf16 unless noted):
 *   X   [M, K]  row stride ldx >= K            (tokens x in_features)
 *   W0  [N, K]  row stride K                   (out_features x in_features)
 *   A   [r, K]  row stride K                   (merged down-projection)
 *   B   [N, r]  row stride r                   (merged up-projection)
 *   bias fp32 [N] or NULL
 *   residual [M, Nout] row stride ldr, or NULL; may be the SAME pointer as Y
 *            with ldr == ldy (in-place residual add).  Not allowed with SWIGLU.
 *   Y   [M, Nout] row stride ldy >= Nout;  Nout = N, or N/2 with SWIGLU.
 *   scale: s (fp32, finite).  Applied to T before T is rounded to bf16.
 *   epilogue FSD_EPI_SWIGLU: the N accumulator columns are read as [G | U]
 *            halves (gate first, F = N/2) and Y = silu(G)·U elementwise,
 *            silu(g) = g / (1 + exp(-g)); bias is added to both halves before
 *            the activation.
 * Accumulation is fp32; Y is rounded to bf16 (round-to-nearest-even).
 * Sizes: M >= 0 (M == 0 is a no-op), K >= 8, N >= 8, r >= 0 (r == 0 gives the
 * plain GEMM), K, N, r multiples of 8, SWIGLU needs N a multiple of 16.
 * Buffer offsets are 32-bit: (N + 256)·K·2, (N + 256)·r·2 and 256·ld·2 for
 * each of ldx, ldt and ldr must stay below 2^31 (else FSD_EUNSUPPORTED).
 * Aliasing: Y must not overlap X, W0, A, B, bias or the workspace.
 */

/* Bytes of workspace with which fsd_lora_linear runs its preferred schedule
 * for M rows at rank r: min(M, 43,520)·r·2 (50.1 MB at r = 576, all rows of T
 * when M <= 43,520).  0 when M <= 0 or r <= 0. */
size_t fsd_lora_linear_workspace_bytes(int64_t M, int64_t r);

/* Phase A alone.  T: bf16 [M, r] with row stride ldt >= r. */
int fsd_lora_down(const void* X, int64_t ldx, const void* A, float scale,
                  void* T, int64_t ldt, int64_t M, int64_t K, int64_t r,
                  void* stream);

/* Phase B alone: Y = epi([X | T]·[W0 | B]ᵀ + bias) (+ residual), T as written
 * by fsd_lora_down (ldt >= r).  With r == 0, T and B are ignored. */
int fsd_lora_up(const void* X, int64_t ldx, const void* W0, const void* T,
                int64_t ldt, const void* B, const float* bias,
                const void* residual, int64_t ldr, void* Y, int64_t ldy,
                int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                void* stream);

/* Phase A then phase B, chunked over M so that T stays in a small workspace
 * (bf16, T of a chunk at row stride r).  workspace_bytes must hold at least
 * min(M, 256) rows of T (fsd_lora_linear_workspace_bytes(min(M, 256), r),
 * else FSD_EWORKSPACE); with r == 0 the workspace may be NULL.  Schedule,
 * from the rows of T that fit ("fit"):
 *   fit >= M: phase A over all rows, then phase B (two launches);
 *   fit >= 512: chunks of R rows, R = min(21,760, 256·floor(fit/512)), through
 *     two alternating halves of the workspace: launch 0 is phase A of chunk 0,
 *     launch c + 1 is phase B of chunk c together with phase A of chunk c + 1
 *     in one grid, so phase A's tiles fill the CUs that phase B's last wave
 *     leaves idle (21,760 rows = 85 row tiles: its 255 phase-A tiles fill one
 *     wave of 256 CUs);
 *   otherwise: 256-row chunks, phase A then phase B each.
 * Chunks start on 256-row boundaries, so the result is bitwise identical to
 * the unchunked one whatever the workspace size.  The workspace is read and
 * written only by this call's kernels; it need not be initialised. */
int fsd_lora_linear(const void* X, int64_t ldx, const void* W0, const void* A,
                    const void* B, const float* bias, const void* residual,
                    int64_t ldr, float scale, void* Y, int64_t ldy, int64_t M,
                    int64_t N, int64_t K, int64_t r, int epilogue,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The schedule of fsd_lora_linear for M rows at rank r and a workspace of
 * workspace_bytes bytes: returns its number of kernel launches (0 when
 * M == 0; -1 for M < 0 or r < 0) and stores the rows per chunk in *chunk_rows
 * and the schedule in *schedule (0: phase A then phase B over all rows;
 * 1: pipelined pairs; 2: chunks of phase A then phase B), each when non-NULL.
 * Host-only arithmetic: no HIP call. */
int64_t fsd_lora_linear_plan(int64_t M, int64_t r, size_t workspace_bytes,
                             int64_t* chunk_rows, int* schedule);

/* Launch number `index` (0 <= index < fsd_lora_linear_plan(...)) of
 * fsd_lora_linear with the same arguments; calling every index in order, on one
 * stream, is exactly fsd_lora_linear.  Lets a caller place its own work (timing
 * events, captures) between the launches.  Same validation and errors as
 * fsd_lora_linear, plus FSD_EINVAL for an index out of range (index 0 with
 * M == 0 is a no-op). */
int fsd_lora_linear_launch(const void* X, int64_t ldx, const void* W0,
                           const void* A, const void* B, const float* bias,
                           const void* residual, int64_t ldr, float scale,
                           void* Y, int64_t ldy, int64_t M, int64_t N,
                           int64_t K, int64_t r, int epilogue, void* workspace,
                           size_t workspace_bytes, int64_t index, void* stream);

/* ------------------------------------------------------------------------ *
 * The LoRA-fused linear without an allocation                               *
 * ------------------------------------------------------------------------ *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fsd_lora_linear with T kept in a scratch array that the library holds on
 * each GPU it runs on, FSD_NOALLOC_SCRATCH_BYTES bytes (two 21,760-row chunks
 * of T at rank 576), instead of a caller's workspace.  Same arguments (minus
 * the workspace), results (bitwise those of fsd_lora_linear with a workspace
 * of that size) and errors as fsd_lora_linear, and:
 *   - r > FSD_NOALLOC_SCRATCH_BYTES / 512 (256 rows of T must fit) gives
 *     FSD_EUNSUPPORTED, before any HIP call;
 *   - the first call on a device looks up that device's scratch address
 *     (hipGetDevice, hipGetSymbolAddress; FSD_EHIP if that fails) before the
 *     remaining validation; later calls only query the current device;
 *   - no allocation, no free, no synchronisation; the scratch needs no
 *     clearing (T is written before it is read);
 *   - every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents: calls that overlap on one GPU (several streams, several
 *     host threads) race and must be ordered by the caller. */
#define FSD_NOALLOC_SCRATCH_BYTES ((size_t)50135040)
int fsd_lora_linear_noalloc(const void* X, int64_t ldx, const void* W0,
                            const void* A, const void* B, const float* bias,
                            const void* residual, int64_t ldr, float scale,
                            void* Y, int64_t ldy, int64_t M, int64_t N,
                            int64_t K, int64_t r, int epilogue, void* stream);

/* ------------------------------------------------------------------------ *
 * a1. Partial renoise                                                        *
 * ------------------------------------------------------------------------ *
 * [EN] section "Three steps instead of dozens", renoise equation: the
 * upscaled latent is re-noised to sigma_0 with standard Gaussian noise,
 *   z = (1 - sigma)·u + sigma·eps        (elementwise, fp32, n elements)
 * u, eps, z: fp32 [n], 16-byte aligned.  z may be the same pointer as u or
 * eps; no other overlap.  sigma finite.  n >= 0 (0 is a no-op).
 */
int fsd_renoise(const float* u, const float* eps, float sigma, float* z,
                int64_t n, void* stream);

/* ------------------------------------------------------------------------ *
 * a5. One Euler step of the sampler                                          *
 * ------------------------------------------------------------------------ *
 * [EN] section "Three steps instead of dozens", schedule and update:
 *   z <- z + (sigma_next - sigma)·v      (in place, fp32, n elements)
 * with sigma 0.909 -> 0.857 -> 0.667 -> 0 passed by the caller.  The step
 * (sigma_next - sigma) is formed in fp32.  z, v: fp32 [n], 16-byte aligned;
 * v must not partially overlap z.  sigma, sigma_next finite.  n >= 0.
 */
int fsd_euler_step(float* z, const float* v, float sigma, float sigma_next,
                   int64_t n, void* stream);

/* ------------------------------------------------------------------------ *
 * Token embed / head of the velocity stand-in (2K three-step sweep)          *
 * ------------------------------------------------------------------------ *
 * The pages give neither the transformer's widths nor its input and output
 * projections; these two calls carry a synthetic stand-in's projections
 * between the 24-channel latent (channel-last, one token per latent voxel;
 * [EN] section "Why upscaling happens in latent space", shape equation) and
 * the model width D.
 *
 * fsd_token_embed:  X[m, n] = bf16( sum_c z[m, c]·E[n, c] ),  fp32 sums
 *   (z enters as the bf16 pair hi + lo, within 2^-16 relative of z).
 *   z fp32 [M, C] (row stride C), E bf16 [D, C] (row stride C),
 *   X bf16 [M, D] row stride ldx >= D.  1 <= C <= 32, D multiple of 8,
 *   C·D·2 < 2^31 (else FSD_EUNSUPPORTED).
 * fsd_token_head:   v[m, c] = sum_n H[m, n]·P[c, n],  fp32 sums, fp32 out.
 *   H bf16 [M, D] row stride ldh >= D, P bf16 [C, D] (row stride D),
 *   v fp32 [M, C] (row stride C).  1 <= C <= 32, D multiple of 64.
 */
int fsd_token_embed(const float* z, const void* E, void* X, int64_t ldx,
                    int64_t M, int64_t C, int64_t D, void* stream);
int fsd_token_head(const void* H, int64_t ldh, const void* P, float* v,
                   int64_t M, int64_t D, int64_t C, void* stream);

/* fsd_token_head_euler: the head with the sampler's Euler update fused in,
 *   z[m, c] <- z[m, c] + (sigma_next - sigma)·sum_n H[m, n]·P[c, n]
 * ([EN] section "Three steps instead of dozens", Euler update equation,
 * with v the head's output).  v is never written: the sums stay in
 * registers and each z element is updated with the same fp32 fma as
 * fsd_euler_step applies to a stored v, so the two routes agree bit for bit.
 * H, P, C, D as for fsd_token_head; z fp32 [M, C] (row stride C), updated in
 * place, 4-byte aligned, must not overlap H or P; sigma, sigma_next finite
 * (else FSD_EINVAL); (sigma_next - sigma) is formed in fp32. */
int fsd_token_head_euler(const void* H, int64_t ldh, const void* P, float* z,
                         int64_t M, int64_t D, int64_t C, float sigma,
                         float sigma_next, void* stream);

/* ------------------------------------------------------------------------ *
 * MXFP8 linears (NEXT step of the pages' own optimisation)                   *
 * ------------------------------------------------------------------------ *
 * The pages run the linears as MXFP8 FP8 GEMMs, quantized again per stage, with
 * SwiGLU fused into a one-pass activation quantizer ([EN] section "Where the
 * 3.9x speedup comes from", inference-configuration table).  Format (OCP MX
 * v1.0, the pages fix none of it): blocks of 32 elements along K, shared
 * E8M0 scale 2^(floor(log2 amax) - 8), E4M3 elements rounded to nearest-even
 * and saturated at 448.
 *
 * Layout: elements Q as bytes [M, Kp], Kp = K rounded up to 128, row stride
 * ldq >= Kp (multiple of 16), columns K..Kp-1 zero.  Scales S, Mp = M rounded
 * up to 256: for each 128-element step t < Kp/128 and 64-row group g < Mp/64,
 * 64 consecutive 32-bit words; byte i (0..3, little-endian) of word 16·b + r
 * (b < 4, r < 16) is the E8M0 scale of row 64g + 16i + r over elements
 * 128t + 32b .. +31.  That is the order in which the MXFP8 GEMM's lanes take
 * the scales of a 16-row block, one word serving four blocks.  Padding rows
 * and blocks hold 127 (a scale of 1) and zero elements.  S is 4-byte aligned.
 *
 * fsd_mx_scale_bytes: size of S for M rows of K elements.
 * fsd_mx_quantize: X bf16 [M, K] (row stride ldx >= K, multiple of 8, 16-byte
 *   aligned), K a multiple of 32 -> Q, S as above.  Q 16-byte aligned; Q and S
 *   must not overlap X or each other.  Errors: FSD_EINVAL, FSD_EALIGN.
 *
 * fsd_mx_lora_down: phase A on MXFP8 operands,
 *   T = bf16(scale · deq(Xq, Xs) · deq(Aq, As)ᵀ), fp32 accumulation.
 *   Xq [M, Kp] (row stride ldxq) with scales Xs for M rows; Aq [r, Kp] (row
 *   stride Kp) with scales As for r rows; K a multiple of 32, r a multiple of
 *   8; T bf16 [M, r] (row stride ldt >= r, multiple of 8, 16-byte aligned),
 *   not overlapping any input.
 * fsd_mx_lora_up: phase B on MXFP8 operands,
 *   Y = epi(deq(Xq)·deq(W0q)ᵀ + deq(Tq)·deq(Bq)ᵀ + bias) (+ residual), with
 *   W0q [N, Kp] (row stride Kp, scales W0s for N rows), Tq [M, rp] (row stride
 *   ldtq, scales Ts for M rows) and Bq [N, rp] (row stride rp, scales Bs for
 *   N rows), rp = r rounded up to 128.  r a multiple of 32 (0: no LoRA term;
 *   Tq, Ts, Bq, Bs unused).  bias, residual, Y, ldy, epilogue as for
 *   fsd_lora_up; SwiGLU needs N a multiple of 128 (else FSD_EUNSUPPORTED).
 * fsd_mx_lora_up_swiglu_mx: fsd_mx_lora_up with the SwiGLU epilogue whose
 *   output leaves as MXFP8 in the same pass: H = SwiGLU(...) is rounded to
 *   bf16 (exactly what fsd_mx_lora_up writes) and quantized as
 *   fsd_mx_quantize would quantize it, so the bytes equal those of the two
 *   calls in sequence.  Hq [M, F] E4M3 (F = N/2, row stride ldhq >= F,
 *   multiple of 16), Hs its scales for M rows of F; N a multiple of 256
 *   (else FSD_EUNSUPPORTED); no residual.  The pages fuse SwiGLU with the
 *   activation quantizer ([EN] inference-configuration table, "Fused SwiGLU +
 *   MXFP8 quantizer").
 * In all three, code arrays are 16-byte aligned with row strides multiples of 16,
 * scale arrays 4-byte aligned; a weight operand must span less than 2 GiB with
 * 256 extra rows, an activation operand's 256-row tile likewise (and 256
 * rows of the residual, 256·ldr·2 bytes), and every scale array less than
 * 2 GiB (else FSD_EUNSUPPORTED). */
size_t fsd_mx_scale_bytes(int64_t M, int64_t K);
int fsd_mx_quantize(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q,
                    int64_t ldq, void* S, void* stream);
int fsd_mx_lora_down(const void* Xq, int64_t ldxq, const void* Xs, const void* Aq,
                     const void* As, float scale, void* T, int64_t ldt, int64_t M,
                     int64_t K, int64_t r, void* stream);
int fsd_mx_lora_up(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                   const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                   const void* Bq, const void* Bs, const float* bias,
                   const void* residual, int64_t ldr, void* Y, int64_t ldy,
                   int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                   void* stream);
int fsd_mx_lora_up_swiglu_mx(const void* Xq, int64_t ldxq, const void* Xs,
                             const void* W0q, const void* W0s, const void* Tq,
                             int64_t ldtq, const void* Ts, const void* Bq,
                             const void* Bs, const float* bias, void* Hq,
                             int64_t ldhq, void* Hs, int64_t M, int64_t N,
                             int64_t K, int64_t r, void* stream);

/* One-pass activation quantization: the producer of an activation emits its
 * MXFP8 form in the same pass, so no separate quantizer pass reads it back
 * (the pages list "one-pass activation quantization" among their kernels,
 * [EN] "Where the 3.9x speedup comes from", inference-configuration table).
 * Each one writes the bytes that the unfused route (the bf16 result, then
 * fsd_mx_quantize of it) writes: the value is rounded to bf16 first, then
 * quantized.  Code arrays 16-byte aligned with row strides multiples of 16,
 * scale arrays 4-byte aligned and sized by fsd_mx_scale_bytes; outputs must
 * not overlap any input or each other (else FSD_EINVAL).
 *
 * fsd_mx_lora_down_mx: fsd_mx_lora_down whose T leaves only as MXFP8: Tq
 *   [M, rp] (rp = r rounded up to 128, row stride ldtq >= rp) and Ts for M
 *   rows of r; r a multiple of 32.  Tq, Ts are what fsd_mx_lora_up takes.
 * fsd_mx_lora_up_q: fsd_mx_lora_up (plain epilogue: bias, residual) that
 *   writes Y and also the MXFP8 form of Y's columns [q0, q1) as a matrix of
 *   q1 - q0 columns: Yq (row stride ldyq >= (q1 - q0) rounded up to 128) and
 *   Ys.  q0, q1 multiples of 32 with 0 <= q0 < q1 <= N.  Used for the V slice
 *   of the QKV output (the O projection's input) and for the residual stream
 *   after the O projection (the gate/up input).
 * fsd_token_embed_mx: fsd_token_embed that also writes the MXFP8 form of X
 *   (Xq [M, D], row stride ldxq >= D, and Xs); D a multiple of 128 (else
 *   FSD_EUNSUPPORTED). */
int fsd_mx_lora_down_mx(const void* Xq, int64_t ldxq, const void* Xs,
                        const void* Aq, const void* As, float scale, void* Tq,
                        int64_t ldtq, void* Ts, int64_t M, int64_t K, int64_t r,
                        void* stream);
int fsd_mx_lora_up_q(const void* Xq, int64_t ldxq, const void* Xs,
                     const void* W0q, const void* W0s, const void* Tq,
                     int64_t ldtq, const void* Ts, const void* Bq, const void* Bs,
                     const float* bias, const void* residual, int64_t ldr,
                     void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                     int64_t r, int64_t q0, int64_t q1, void* Yq, int64_t ldyq,
                     void* Ys, void* stream);
int fsd_token_embed_mx(const float* z, const void* E, void* X, int64_t ldx,
                       int64_t M, int64_t C, int64_t D, void* Xq, int64_t ldxq,
                       void* Xs, void* stream);

/* The whole MXFP8 LoRA linear in row chunks, with T kept small and quantized:
 * the schedule of fsd_lora_linear ([CW] section "三个步如何完成工作": the
 * rank-576 merged adapter on every adapted linear) on MXFP8 operands.  Chunks of
 * R rows (a multiple of 256, at most 21,760) pass through two halves of the
 * workspace; launch 0 is phase A of chunk 0, launch c + 1 is phase B of chunk c
 * together with phase A of chunk c + 1 in one grid.  Phase A writes its chunk
 * of T as MXFP8 (fsd_mx_lora_down_mx's bytes); phase B is fsd_mx_lora_up (or
 * its quantizing forms) over the chunk's rows, so every output byte equals the
 * unchunked route's.
 *   Xq, ldxq, Xs: the input, MXFP8 [M, Kp] with scales for M rows, K a
 *     multiple of 32; Aq, As: the merged down projection [r, Kp], r a multiple
 *     of 32; W0q, W0s [N, Kp] and Bq, Bs [N, rp]: as for fsd_mx_lora_up;
 *     scale: applied to T before its bf16 rounding.
 *   epilogue FSD_EPI_NONE: Y bf16 [M, N] (row stride ldy), bias and residual
 *     as for fsd_mx_lora_up; with Yq != NULL also the MXFP8 of Y's columns
 *     [q0, q1) as fsd_mx_lora_up_q writes it.
 *   epilogue FSD_EPI_SWIGLU: either Y bf16 [M, N/2] (N a multiple of 128) or,
 *     with Y == NULL, Yq/Ys = the MXFP8 of H as fsd_mx_lora_up_swiglu_mx writes
 *     it (q0 = 0, q1 = N/2, N a multiple of 256); no residual.
 *   workspace: 16-byte aligned, owned by the caller, read and written only by
 *     this call's kernels; it must hold two chunks of at least 256 rows of T
 *     (rp + rp/32 bytes per row), else FSD_EWORKSPACE.  Outputs must overlap
 *     neither an input, the workspace nor each other (the residual may be Y).
 * fsd_mx_lora_linear_workspace_bytes: the preferred size: two chunks of
 *   min(M rounded up to 256, 21,760) rows (28.7 MB at r = 576); at ranks above
 *   about 3.1 million the chunk is further capped so that its T scales
 *   (R·rp/32 bytes) stay below 2^31 bytes.
 * fsd_mx_lora_linear_plan: the number of launches and the chunk rows for M
 *   rows at rank r through workspace_bytes (FSD_EWORKSPACE if too small).
 * fsd_mx_lora_linear_launch: launch `index` (0 <= index < launches) alone,
 *   e.g. to put timing events between launches; issuing every index in order
 *   on one stream is fsd_mx_lora_linear. */
size_t fsd_mx_lora_linear_workspace_bytes(int64_t M, int64_t r);
int fsd_mx_lora_linear_plan(int64_t M, int64_t r, size_t workspace_bytes,
                            int64_t* launches, int64_t* chunk_rows);
int fsd_mx_lora_linear(const void* Xq, int64_t ldxq, const void* Xs,
                       const void* Aq, const void* As, float scale,
                       const void* W0q, const void* W0s, const void* Bq,
                       const void* Bs, const float* bias, const void* residual,
                       int64_t ldr, void* Y, int64_t ldy, int64_t M, int64_t N,
                       int64_t K, int64_t r, int epilogue, int64_t q0, int64_t q1,
                       void* Yq, int64_t ldyq, void* Ys, void* workspace,
                       size_t workspace_bytes, void* stream);
int fsd_mx_lora_linear_launch(const void* Xq, int64_t ldxq, const void* Xs,
                              const void* Aq, const void* As, float scale,
                              const void* W0q, const void* W0s, const void* Bq,
                              const void* Bs, const float* bias,
                              const void* residual, int64_t ldr, void* Y,
                              int64_t ldy, int64_t M, int64_t N, int64_t K,
                              int64_t r, int epilogue, int64_t q0, int64_t q1,
                              void* Yq, int64_t ldyq, void* Ys, void* workspace,
                              size_t workspace_bytes, int64_t index, void* stream);

/* ------------------------------------------------------------------------ *
 * Dense attention (NEXT step: the refine path's baseline attention)          *
 * ------------------------------------------------------------------------ *
 * The pages' baseline refine runs the transformer's attention densely in
 * bf16 ([EN] "Where the 3.9x speedup comes from", dense-BF16 baseline row);
 * the operation is textbook scaled dot-product attention, per head h:
 *   O_h = softmax(Q_h · K_hᵀ · scale) · V_h,
 * the softmax over all S keys of the sequence, fp32 statistics, P rounded to
 * bf16 before the P·V product, O rounded to bf16.
 *
 * fsd_attention_workspace_bytes: bytes of the workspace (V transposed per
 *   head, H·D·round_up(S, 64)·2).
 * fsd_attention: Q, K, V bf16 [S, H·D] (head h in columns h·D .. h·D+D-1; the
 *   Q, K and V slices of a QKV projection output can be passed in place), row
 *   stride ld >= H·D (multiple of 8); O bf16 [S, H·D], row stride ldo >= H·D
 *   (multiple of 8).  D must be 128 (else FSD_EUNSUPPORTED); scale finite and
 *   > 0 (1/sqrt(D) for the standard form).  All pointers 16-byte aligned; O
 *   and the workspace must not overlap the inputs or each other.  Errors:
 *   FSD_EINVAL, FSD_EALIGN, FSD_EUNSUPPORTED (also for a 256-row tile or one
 *   transposed head spanning 2 GiB), FSD_EWORKSPACE. */
size_t fsd_attention_workspace_bytes(int64_t S, int64_t H, int64_t D);
int fsd_attention(const void* Q, const void* K, const void* V, int64_t ld,
                  void* O, int64_t ldo, int64_t S, int64_t H, int64_t D,
                  float scale, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ------------------------------------------------------------------------ *
 * One HIP graph per refinement step                                          *
 * ------------------------------------------------------------------------ *
 * [EN] "Where the 3.9x speedup comes from": the refine runs each of its steps
 * as one captured graph.  These calls record the launches that this library's
 * entry points enqueue on a stream into one graph and replay it:
 *   fsd_graph_begin(stream): start capturing the launches enqueued on `stream`
 *     (a created stream, not NULL) by this thread (thread-local capture mode).
 *   fsd_graph_end(stream, &graph): end the capture and instantiate it; *graph
 *     receives the executable graph (owned by the caller, NULL on failure).
 *   fsd_graph_launch(graph, stream): replay it on `stream`, asynchronously.
 *   fsd_graph_destroy(graph): release it (NULL is a no-op).
 * The replay repeats the captured launches with the pointers, sizes and scalars
 * they were given: the buffers must stay allocated and in place.  No entry
 * point of this library records a memset or an allocation, so every replay is
 * exactly the captured launches.  Errors: FSD_EINVAL (NULL stream or graph
 * pointer), FSD_EHIP (the HIP runtime refused: e.g. the stream was not being
 * captured, or a launch between begin and end failed). */
int fsd_graph_begin(void* stream);
int fsd_graph_end(void* stream, void** graph);
int fsd_graph_launch(void* graph, void* stream);
int fsd_graph_destroy(void* graph);

#ifdef __cplusplus
}
#endif

#endif /* FSD_H */
