/*
 * svdq.h - C ABI of libsvdq: the SVDQuant W4A4 + low-rank linear on MI355X (gfx950).
 *
 * The layer (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
 * Nunchaku 4-Bit-Quantisierung", section "Nunchaku und SVDQuant"): activation
 * outliers are moved into the weights by a per-input-channel smoothing vector
 * lambda, the hardest part of each smoothed weight matrix W' = W diag(lambda) is
 * kept in a 16-bit rank-r branch (L1 [K,r], L2 [r,N]), and the residual R runs as
 * 4-bit weights against 4-bit activations:
 *
 *     Y = X W^T + b  ~=  dequant(Q(X_hat) . Q(R)^T) + (X_hat L1) L2 + b,
 *     X_hat = X diag(lambda)^-1.
 *
 * The online work is split into the two fused calls named by the charmloop.ai
 * news item on Nunchaku in Diffusers (paragraph on the 16-bit branch): the
 * low-rank down-projection runs inside the activation-quantization kernel, the
 * low-rank up-projection inside the 4-bit compute kernel.  Composed, they are a
 * drop-in for an nn.Linear(K, N) forward (mind-verse.de, section "Native
 * Ladefunktion in Diffusers": the module tree stays that of the dense model).
 *
 * Conventions common to every call
 *  - Layouts follow nn.Linear: X [M,K], W [N,K], Y [M,N]; lora_down = L1^T [r,K];
 *    lora_up = L2^T [N,r].  Every array is dense, row-major, no padding.
 *  - bf16 arrays are passed as raw 16-bit patterns (IEEE bfloat16).
 *  - int4 codes: two per byte along K, element 2i in the low nibble of byte i,
 *    two's complement, values in [-7, 7].  Codes are [rows, K/2] bytes in the
 *    storage order: in every row whose index in the array has bit 3 set (rows
 *    8-15 of each 16), the two 8-byte halves of every 16-byte piece of the row
 *    are exchanged (byte j of the row sits at j ^ 8); rows 0-7 of each 16 are
 *    in the plain order.  Call 1 writes and call 2 reads this order, and
 *    svdq_pack_weights writes it, so a view of a codes array must start at a
 *    multiple of 16 rows.  (It lets call 2 read its LDS fragments without bank
 *    conflicts.)  MXFP4 and AWQ codes keep the plain order.
 *  - Scales: bf16 [rows, K/group_size], one per row per group of group_size
 *    consecutive k.  Only group_size == 64 and int4 are supported (the int4
 *    scheme's group size in the quantization config on mind-verse.de, section
 *    "Native Ladefunktion in Diffusers").
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    device workspace some calls need (below); the library allocates no device
 *    memory and keeps no state besides a per-device capability cache and the
 *    test hooks' settings.  Device pointers must be 16-byte aligned.  An output
 *    must not overlap an input, another output or the workspace
 *    (INVALID_VALUE); inputs may share memory.
 *  - Workspace: calls 1 and 2 may split K over several workgroups whose fp32
 *    partial sums meet in device memory.  svdq_*_workspace_size gives the
 *    bytes a shape needs on the current device (0: none; NULL may then be
 *    passed).  A workspace starts with a fixed 1 MiB region of arrival
 *    counters, then scratch.  The caller zero-fills a workspace once, before
 *    its first use; every call leaves its counters back at zero and writes
 *    scratch before reading it, so one workspace serves any later call, of any
 *    shape whose query fits its capacity, that is ordered after the previous
 *    one (same stream, or an explicit dependency).  Calls that may run at the same time need distinct
 *    workspaces.  The caller must not write to it between calls.  A call whose
 *    workspace is NULL or smaller than the query returns INVALID_VALUE before
 *    any launch.  The size depends on the test hooks below; query after
 *    setting them.
 *  - Empty batch: M == 0 is a successful no-op once the dimensions are valid;
 *    nothing is read or written, so the pointers may be NULL.
 *  - Errors: argument and shape errors are returned synchronously, before any
 *    HIP call.  Kernels run asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream) on the current HIP device; a launch failure returns
 *    SVDQ_STATUS_HIP_ERROR, device faults surface at the caller's next
 *    synchronisation.  svdq_last_error() gives a thread-local message for the
 *    last failing call.  No C++ exception crosses this boundary.
 *  - Calls on distinct streams may run concurrently from several threads.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
  SVDQ_STATUS_SUCCESS = 0,
  SVDQ_STATUS_INVALID_VALUE = 1,   /* null required pointer, negative dim, misalignment,
                                      overlapping output, missing or short workspace */
  SVDQ_STATUS_NOT_SUPPORTED = 2,   /* group_size != 64, K % 64, N % 64, r not in {0,16,...,128} */
  SVDQ_STATUS_ARCH_MISMATCH = 3,   /* current device is not gfx950 */
  SVDQ_STATUS_NO_DEVICE = 4,       /* no HIP device visible */
  SVDQ_STATUS_HIP_ERROR = 5,       /* the HIP runtime reported an error */
  SVDQ_STATUS_INTERNAL = 6
} svdq_status;

/* Static name of a status code. */
const char* svdq_status_string(svdq_status status);

/* Thread-local message describing the last failing call on this thread ("" if none). */
const char* svdq_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int svdq_version(void);

/*
 * Checks that HIP device `device` is a gfx950 (MI355X).  The result is cached per
 * device.  The loader of the pages validates the GPU generation when a
 * checkpoint is loaded and errors out on unsupported ones (mind-verse.de,
 * section "Hardware-Unterstützung"); this is that check for this library.
 * Returns SUCCESS, NO_DEVICE, ARCH_MISMATCH or INVALID_VALUE (bad index).
 */
svdq_status svdq_check_device(int device);

/*
 * Call 1 - smoothing, per-token per-group int4 quantization, packing, and the
 * fused low-rank down-projection (charmloop.ai item, fusion paragraph;
 * ai2day.live, "AI-Bildmodelle auf normalen GPUs ausführen", section "Was ist
 * Nunchaku Lite und was macht es genau?": 4 bits also for the live activations).
 *
 *   mu_k      = fl32(1 / lambda_k)
 *   x_hat     = bf16(fl32(X * mu))                     (one canonical bf16 X_hat)
 *   per row m and group g of 64 k:
 *     s       = bf16(fl32(max|x_hat| / 7))
 *     q       = clamp(rint_even(x_hat * fl32(1/s)), -7, 7)
 *               (s == 0, or fl32(1/s) overflowing (s < 2^-128): q = 0)
 *   lora_act  = bf16(x_hat @ lora_down^T)              (fp32 accumulation)
 *
 *   x          device, bf16 [M, K]
 *   smooth     device, fp32 [K]   lambda (X is divided by it, W multiplied)
 *   lora_down  device, bf16 [r, K]; may be NULL iff r == 0
 *   M >= 0 (M == 0 is a no-op), K > 0 with K % 64 == 0, r in {0,16,...,128},
 *   group_size == 64; M <= 2^24 and M * K <= 2^40, and M <= 2^22 when r > 0
 *   and K > 4096 (NOT_SUPPORTED beyond)
 *   act_codes  device out, u8   [M, K/2]
 *   act_scales device out, bf16 [M, K/64]
 *   lora_act   device out, bf16 [M, r]; may be NULL iff r == 0
 *   workspace  device scratch of svdq_quantize_act_workspace_size(M, K, r) bytes
 *              (see Conventions; may be NULL when that is 0), workspace_bytes its size
 *   stream     hipStream_t or NULL
 * Codes and scales are exactly defined (bit-exact to the rule above); lora_act
 * may differ from a float64 evaluation by one bf16 ulp (summation order).  When
 * K is split over several workgroups, their fp32 partial sums of lora_act meet
 * in the workspace and are added in a fixed order, so the result does not
 * depend on timing.
 */
svdq_status svdq_quantize_act_lora_down(
    const void* x, const float* smooth, const void* lora_down,
    int64_t M, int64_t K, int64_t r, int64_t group_size,
    void* act_codes, void* act_scales, void* lora_act,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes call 1 (either element format) needs for (M, K, r) on the
 * current device, with the current test hooks; 0 when it needs none and for
 * shapes the call rejects (the call reports those).  Host only, no launch.
 */
size_t svdq_quantize_act_workspace_size(int64_t M, int64_t K, int64_t r);

/*
 * Test hook for call 1: forces its work split for every later call in this
 * process.  k_blocks = number of K-blocks (each a run of consecutive groups of
 * 64; clipped to K/64), tiles_per_wg = row tiles of 16 per workgroup (1..12);
 * 0 keeps the automatic choice for that parameter.  A forced split whose
 * K-block would not fit in LDS is ignored.  Codes and scales do not depend on
 * the split; lora_act may change by a bf16 ulp (its fp32 partial sums change).
 * Returns INVALID_VALUE for negative values or tiles_per_wg > 12.
 */
svdq_status svdq_debug_set_quant_plan(int k_blocks, int tiles_per_wg);

/*
 * Test hook for call 1: picks its kernel for every later call in this process.
 * 0 chooses by shape; 1 forces the kernel with one wave per row tile of 16
 * tokens; 2..8 force the row-tile kernel, in which a workgroup owns one row
 * tile and that many waves split each K-block's groups, their lora_down
 * partials added in LDS (k_blocks of svdq_debug_set_quant_plan still sets the
 * K-blocks, tiles_per_wg is not used).  Codes and scales do not change;
 * lora_act may change by a bf16 ulp.  Returns INVALID_VALUE outside 0..8.
 */
svdq_status svdq_debug_set_quant_waves(int waves);

/*
 * Test hook for call 2 (and svdq_w4a4_group_acc_debug): 0 chooses the kernel
 * by shape (the few-token kernel, whose waves split K, for up to 64 tokens,
 * and up to 160 for layers of at most 2^24 weights; the tiled kernel
 * otherwise), 1 forces the tiled kernel, 2 the few-token kernel
 * wherever it is supported.  Both compute the same integers and the same
 * dequantization; Y may differ in fp32 rounding order.  Returns INVALID_VALUE
 * for other values.
 */
svdq_status svdq_debug_set_gemm_path(int path);

/*
 * Test hook for call 2's tiled kernel: the number of K-splits per output tile
 * for every later call in this process (0 = chosen by shape; clipped to the
 * number of group pairs K/128, rounded up).  With splits > 1 each workgroup
 * runs a run of whole quant groups of its tile and the fp32 partial tiles are
 * added in split order through the caller's workspace (query its size after
 * setting the hook), so Y may differ from the unsplit result in fp32 rounding
 * order but not between runs.  Ignored by
 * the QKV epilogue and the accumulator dump.  Returns INVALID_VALUE outside
 * 0..64.
 */
svdq_status svdq_debug_set_gemm_splits(int splits);

/*
 * Test hook for svdq_fp4_gemm_lora_up: the output tile edge for every later
 * call in this process.  0 chooses by shape (256 x 256 tiles, one workgroup
 * per CU and no workspace, when K % 1024 == 0 and there are at least a
 * quarter as many of those tiles as CUs; otherwise 128 x 128 tiles with
 * K-splits), 128 forces the
 * 128 x 128 kernel, 256 the 256 x 256 kernel wherever K % 1024 == 0.  A split
 * count forced by svdq_debug_set_gemm_splits also selects the 128 x 128
 * kernel.  Query the workspace size after setting the hook.  Returns
 * INVALID_VALUE for other values.
 */
svdq_status svdq_debug_set_fp4_tile(int tile);

/*
 * Call 2 - W4A4 GEMM with per-group int32 accumulation, per-group
 * dequantization, the fused low-rank up-projection and the bias
 * (mind-verse.de, section "Nunchaku und SVDQuant": fused kernels for the 4-bit
 * path and the low-rank branch; charmloop.ai item, fusion paragraph).
 *
 *   acc_g[m,n] = sum_{k in g} q_x[m,k] * q_w[n,k]     (exact int32)
 *   Y[m,n]     = bf16( sum_g s_x[m,g] s_w[n,g] acc_g[m,n]
 *                      + lora_act[m,:] . lora_up[n,:] + bias[n] )  (fp32 accumulation)
 *
 *   act_codes, act_scales  device, as produced by call 1 ([M,K/2] u8, [M,K/64] bf16)
 *   w_codes    device, u8   [N, K/2]   packed residual codes (svdq_pack_weights)
 *   w_scales   device, bf16 [N, K/64]
 *   lora_act   device, bf16 [M, r]; NULL iff r == 0
 *   lora_up    device, bf16 [N, r]; NULL iff r == 0
 *   bias       device, bf16 [N] or NULL (no bias)
 *   M >= 0 (0 is a no-op), N > 0 with N % 64 == 0, K > 0 with K % 64 == 0,
 *   r in {0,16,...,128}, group_size == 64
 *   y          device out, bf16 [M, N]
 *   workspace  device scratch of svdq_w4a4_gemm_workspace_size(M, N, K, r) bytes
 *              (see Conventions; may be NULL when that is 0), workspace_bytes its size
 * With few output tiles (fewer than two 128 x 128 tiles per compute unit) the
 * tiled kernel splits K over several workgroups per tile; their fp32 partial
 * tiles meet in the workspace and are added in a fixed order, so Y does not
 * depend on timing.
 */
svdq_status svdq_w4a4_gemm_lora_up(
    const void* act_codes, const void* act_scales,
    const void* w_codes, const void* w_scales,
    const void* lora_act, const void* lora_up, const void* bias,
    int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
    void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes call 2 (svdq_w4a4_gemm_lora_up and _ex, any epilogue) needs
 * for (M, N, K, r) on the current device, with the current test hooks; 0 when
 * it needs none and for shapes the call rejects.  Host only, no launch.
 */
size_t svdq_w4a4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * Output epilogues of call 2, applied to y + b before the bf16 rounding.
 * SVDQ_EPILOGUE_GELU_TANH is GELU with the tanh approximation (Hendrycks and
 * Gimpel, 2016): 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), as in the MLP
 * up-projection of a diffusion transformer block; the W4A4 layer serves the
 * attention and MLP projections (mind-verse.de, "Effiziente Optimierung von
 * Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku
 * Lite: Nahtlose Integration in Diffusers").  Evaluated in fp32 from
 * exp(2u): relative error a few fp32 ulp, far below the bf16 output rounding.
 */
typedef enum {
  SVDQ_EPILOGUE_NONE = 0,
  SVDQ_EPILOGUE_GELU_TANH = 1
} svdq_epilogue;

/*
 * Call 2 with an output epilogue (svdq_epilogue); arguments and errors as for
 * svdq_w4a4_gemm_lora_up, plus INVALID_VALUE for an unknown epilogue.  With
 * SVDQ_EPILOGUE_NONE it is svdq_w4a4_gemm_lora_up.  An MLP pair chains
 * call 2 (GELU) -> call 1 on its bf16 output -> call 2 of the down-projection
 * on one stream, with no host round trip.
 */
svdq_status svdq_w4a4_gemm_lora_up_ex(
    const void* act_codes, const void* act_scales,
    const void* w_codes, const void* w_scales,
    const void* lora_act, const void* lora_up, const void* bias,
    int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
    int epilogue, void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Call 2 (svdq_w4a4_gemm_lora_up_ex) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid allocation.  It takes no workspace and allocates nothing: when
 * the shape splits K, the partial sums go through a fixed device scratch the
 * library holds on each device from its first use until the process ends (64
 * MiB, the first MiB arrival counters).  The first call on a device clears
 * those counters with a small fill kernel on `stream`; every call leaves them
 * at zero.  All calls on one device share that scratch: calls that may run at
 * the same time on one device (different streams, concurrent graphs) race
 * and give wrong results; order them.  A shape whose plan needs more scratch
 * than the fixed size (svdq_w4a4_gemm_workspace_size above 64 MiB) returns
 * NOT_SUPPORTED before any launch.  Arguments, results and other errors as for
 * svdq_w4a4_gemm_lora_up_ex; the result is bit-identical to it.
 */
svdq_status svdq_w4a4_gemm_lora_up_noalloc(
    const void* act_codes, const void* act_scales,
    const void* w_codes, const void* w_scales,
    const void* lora_act, const void* lora_up, const void* bias,
    int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
    int epilogue, void* y, void* stream);

/*
 * Call 2 with the fused QKV epilogue of a diffusion transformer's attention:
 * for FLUX.1-dev the Q, K and V projections are one quantized to_qkv linear
 * whose fused operator also does the Q/K normalization and the rotary
 * embeddings (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen
 * durch Nunchaku 4-Bit-Quantisierung", section "Quantisierung von Modellen mit
 * strukturellen Umschreibungen").  With v = Y*[m, :] + b (Y* as in call 2) and
 * Y = [Q | K | V] along N (thirds of N/3 columns, heads of head_dim channels):
 *   Q, K heads:  z = v_h / sqrt(mean(v_h^2) + eps) * w     (RMSNorm, per head;
 *                w = q_norm for Q, k_norm for K)
 *                (z[2i], z[2i+1]) -> (z[2i] c - z[2i+1] s, z[2i] s + z[2i+1] c)
 *                with c = rope_cos[m, i], s = rope_sin[m, i] (RoFormer rotation
 *                of adjacent channel pairs, the same angles for every head)
 *   V:           v
 * all in fp32 from the unrounded v, rounded to bf16 once.
 *
 *   head_dim   == 128; N must be a multiple of 3 * head_dim
 *   q_norm, k_norm   device, bf16 [head_dim]
 *   eps        finite, >= 0 (FLUX uses 1e-6)
 *   rope_cos, rope_sin   device, fp32 [M, head_dim/2]
 *   y          device out, bf16 [M, N]
 * Other arguments, errors and the M == 0 rule as for svdq_w4a4_gemm_lora_up;
 * NOT_SUPPORTED for another head_dim or N, INVALID_VALUE for a bad eps or a
 * null or misaligned table.  Runs unsplit on the tiled kernel for every M, so
 * it takes no workspace.
 */
svdq_status svdq_w4a4_gemm_qkv_norm_rope(
    const void* act_codes, const void* act_scales,
    const void* w_codes, const void* w_scales,
    const void* lora_act, const void* lora_up, const void* bias,
    int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
    int64_t head_dim, const void* q_norm, const void* k_norm, float eps,
    const float* rope_cos, const float* rope_sin, void* y, void* stream);

/*
 * Test hook for call 2: runs the same main loop as svdq_w4a4_gemm_lora_up (the
 * kernel the shape and the path hook select) over the rows [m0, m0 + mc) and
 * the 64-aligned column range around [n0, n0 + nc), and writes the int32 group
 * accumulators of that window (the exact integer sums sum_{k in g} q_x q_w,
 * any internal scaling removed) instead of Y:
 *   acc  device out, int32 [mc, nc, K/64]:  acc[(i * nc + j) * K/64 + g]
 *        = acc_g[m0 + i, n0 + j]
 * Same shape rules as call 2; the window must lie inside [0, M) x [0, N)
 * (INVALID_VALUE otherwise); an empty window is a no-op; mc * nc * K/64 above
 * 2^31 is NOT_SUPPORTED.  No scales, lora or bias are read; no workspace.
 */
svdq_status svdq_w4a4_group_acc_debug(
    const void* act_codes, const void* w_codes,
    int64_t M, int64_t N, int64_t K,
    int64_t m0, int64_t mc, int64_t n0, int64_t nc,
    int32_t* acc, void* stream);

/*
 * FP4 variant of calls 1 and 2.  The svdq_w4a4 family also comes in a 4-bit
 * floating-point precision (mind-verse.de, "Effiziente Optimierung von
 * Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", sections "Nunchaku
 * Lite: Nahtlose Integration in Diffusers" and "Hardware-Unterstützung"; named
 * nvfp4 there, group size 16, for Blackwell).  Here the element format is the
 * one CDNA4's matrix cores compute on natively, OCP MXFP4 (Microscaling
 * Formats v1.0): blocks of 32 along K share an E8M0 scale 2^e with
 * e = floor(log2 max|v|) - 2 clamped to [-127, 127] (-127 for a zero block),
 * elements are E2M1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; sign bit 3) rounded
 * to nearest, a midpoint to the even code, above 6 saturating, zero unsigned.
 * Smoothing and the low-rank branch are those of the int4 path.
 *
 * Call 1 (svdq_quantize_act_lora_down_fp4): as svdq_quantize_act_lora_down
 * with x_hat quantized to MXFP4 per token and 32-block:
 *   act_codes  device out, u8 [M, K/2] E2M1 codes, element 2i in the low nibble
 *   act_scales device out, u8 [M, K/32] biased exponents e + 127
 *   K % 128 == 0, group size fixed (32-blocks); other arguments and errors as
 *   for the int4 call.  Codes and exponents are exactly defined.
 * Call 2 (svdq_fp4_gemm_lora_up):
 *   Y = bf16( sum_k deq(act)[m,k] deq(w)[n,k] + lora_act . lora_up^T + bias )
 *   with deq(code, e) = E2M1(code) * 2^(e - 127), fp32 accumulation inside the
 *   matrix core (v_mfma_scale_f32_16x16x128_f8f6f4, the block scales applied
 *   there); w_codes u8 [N, K/2] and w_scales u8 [N, K/32] from
 *   svdq_pack_weights_fp4; epilogue SVDQ_EPILOGUE_NONE or _GELU_TANH; K % 128
 *   == 0; workspace of svdq_fp4_gemm_workspace_size(M, N, K, r) bytes; other
 *   arguments and errors as for svdq_w4a4_gemm_lora_up_ex.
 * Call 1's workspace is svdq_quantize_act_workspace_size(M, K, r), as for the
 * int4 call.
 */
svdq_status svdq_quantize_act_lora_down_fp4(
    const void* x, const float* smooth, const void* lora_down,
    int64_t M, int64_t K, int64_t r,
    void* act_codes, void* act_scales, void* lora_act,
    void* workspace, size_t workspace_bytes, void* stream);
svdq_status svdq_fp4_gemm_lora_up(
    const void* act_codes, const void* act_scales,
    const void* w_codes, const void* w_scales,
    const void* lora_act, const void* lora_up, const void* bias,
    int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
    void* y, void* workspace, size_t workspace_bytes, void* stream);
size_t svdq_fp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * AWQ W4A16 linear: 4-bit weights with 16-bit activations, the second kernel
 * family of the Nunchaku Lite integration, used for the adaptive-normalization
 * and modulation projections (mind-verse.de, "Effiziente Optimierung von
 * Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku
 * Lite: Nahtlose Integration in Diffusers"; precision int4, group_size 64 in
 * the config of section "Native Ladefunktion in Diffusers").  Quantization as
 * in AWQ (Lin et al., 2023); weights from svdq_awq_pack_weights.
 *
 *   x_hat  = bf16(fl32(x * fl32(1/smooth)))
 *   Y[m,n] = bf16( sum_g Delta[n,g] * sum_{k in g} x_hat[m,k] (q[n,k] - z[n,g]) + bias[n] )
 *            (exact products, fp32 accumulation)
 *
 *   x         device, bf16 [M, K]
 *   smooth    device, fp32 [K]   activation-aware scale s (x is divided by it)
 *   w_codes   device, u8   [N, K/2]  unsigned 4-bit codes q, element 2i in the low nibble
 *   w_scales  device, bf16 [N, K/64] Delta
 *   w_zeros   device, u8   [N, K/64] z in 0..15
 *   bias      device, bf16 [N] or NULL
 *   M >= 0 (0 is a no-op), N % 32 == 0, K % 64 == 0, group_size == 64, and
 *   K <= 16384 for M == 1, K <= 8192 for M <= 4, K <= 4096 for larger M (the
 *   x_hat staged in LDS per 16-token tile; NOT_SUPPORTED beyond)
 *   y         device out, bf16 [M, N]
 * Built for few tokens (a conditioning vector per image): the packed weights
 * are streamed once per 16 rows of x, codes and x_hat staged in LDS.  Errors as for svdq_w4a4_gemm_lora_up.
 */
svdq_status svdq_awq_w4a16_gemm(
    const void* x, const float* smooth, const void* w_codes, const void* w_scales,
    const void* w_zeros, const void* bias, int64_t M, int64_t N, int64_t K, int64_t group_size,
    void* y, void* stream);

/*
 * L AWQ W4A16 linears of the same shape that take the same input, in one
 * launch: Y_l = the linear above with layer l's smoothing vector, codes,
 * Delta, z and bias, for l = 0..L-1.  The modulation projections of a
 * diffusion transformer are such a set: every block's adaptive-normalization
 * projection reads the same conditioning vector (mind-verse.de, section
 * "Nunchaku Lite: Nahtlose Integration in Diffusers", modulation layers kept
 * at awq_w4a16), so a step's projections of one shape can run together
 * instead of one launch per block.  Every layer's result is bit-identical to
 * svdq_awq_w4a16_gemm on that layer's arrays.
 *   x         device, bf16 [M, K]            shared by all layers
 *   smooth    device, fp32 [L, K]
 *   w_codes   device, u8   [L, N, K/2]
 *   w_scales  device, bf16 [L, N, K/64]
 *   w_zeros   device, u8   [L, N, K/64]
 *   bias      device, bf16 [L, N] or NULL
 *   y         device out, bf16 [L, M, N]
 *   0 <= L <= 65535 (0 is a no-op, above NOT_SUPPORTED); M, N, K and
 *   group_size as for svdq_awq_w4a16_gemm.  Errors as for that call.
 */
svdq_status svdq_awq_w4a16_gemm_stacked(
    const void* x, const float* smooth, const void* w_codes, const void* w_scales,
    const void* w_zeros, const void* bias, int64_t L, int64_t M, int64_t N, int64_t K,
    int64_t group_size, void* y, void* stream);

/*
 * Host-side packer, step 1: the smoothing vector (mind-verse.de, section
 * "Nunchaku und SVDQuant": outliers of the activations are shifted into the
 * weights).  lambda_j = fl32(sqrt(max(a_j, 1e-5) / max(max_n |W_nj|, 1e-5))),
 * evaluated in double and rounded once.
 *   x_absmax  host, fp32 [K]   per-channel max |X| from calibration
 *   w         host, bf16 [N, K]
 *   smooth    host out, fp32 [K]
 * CPU only; never touches a GPU.
 */
svdq_status svdq_smooth_from_absmax(const float* x_absmax, const uint16_t* w,
                                    int64_t N, int64_t K, float* smooth);

/*
 * Host-side packer, step 2: offline packing of one linear (mind-verse.de,
 * section "Nunchaku und SVDQuant"; config example with rank 32 in section
 * "Native Ladefunktion in Diffusers"; ai2day.live section "Was ist Nunchaku
 * Lite und was macht es genau?" for the SVD).
 *   W' = W diag(lambda) in double; a rank-r truncated SVD W' ~= U S V^T by
 *   randomized subspace iteration (seeded by `seed`), singular values shared
 *   evenly: lora_up = bf16(U S^1/2) [N,r], lora_down = bf16(S^1/2 V^T) [r,K];
 *   R = W' - lora_up lora_down (with the rounded factors, in double);
 *   per row n and group g: s = bf16(max|R| / 7) (one rounding),
 *   q = clamp(rint_even(R / s), -7, 7), packed as described above.
 *   w         host, bf16 [N, K];  smooth  host, fp32 [K]
 *   N > 0, K > 0 with K % 64 == 0, r in {0,...,min(N,K,128)} (any r here),
 *   group_size == 64
 *   w_codes   host out, u8   [N, K/2]
 *   w_scales  host out, bf16 [N, K/64]
 *   lora_down host out, bf16 [r, K]  (may be NULL iff r == 0)
 *   lora_up   host out, bf16 [N, r]  (may be NULL iff r == 0)
 * CPU only (threads); deterministic for a given seed and thread count.
 */
svdq_status svdq_pack_weights(const uint16_t* w, const float* smooth,
                              int64_t N, int64_t K, int64_t r, int64_t group_size,
                              uint64_t seed,
                              uint8_t* w_codes, uint16_t* w_scales,
                              uint16_t* lora_down, uint16_t* lora_up);

/*
 * Host packer of the FP4 variant: smoothing and rank-r split as
 * svdq_pack_weights (same seed, same factors), the residual quantized to
 * MXFP4 per row and 32-block: w_codes u8 [N, K/2], w_scales u8 [N, K/32].
 * K % 128 == 0; errors as svdq_pack_weights.
 */
svdq_status svdq_pack_weights_fp4(const uint16_t* w, const float* smooth, int64_t N, int64_t K, int64_t r,
                                  uint64_t seed, uint8_t* w_codes, uint8_t* w_scales, uint16_t* lora_down,
                                  uint16_t* lora_up);

/*
 * Host AWQ packer (CPU, caller-owned host buffers): the offline step of the
 * AWQ W4A16 linear.  s_x[k] = mean over the Mc calibration rows of |x[m,k]|;
 * for alpha = i / n_grid (i = 0..n_grid-1), s = clamp(s_x^alpha, 1e-4) /
 * sqrt(max s * min s) rounded to fp32, W * s quantized per 64-wide group
 * (Delta = bf16(max(max - min, 1e-5) / 15), z = clamp(rint(-min / Delta), 0, 15),
 * q = clamp(rint(w / Delta) + z, 0, 15)); the alpha with the least mean squared
 * output error on the calibration rows wins (the first on ties).  Outputs the
 * winning s and the codes, scales and zeros of svdq_awq_w4a16_gemm, and alpha
 * (alpha_out may be NULL).  Deterministic for any thread count.
 *   w bf16 [N, K], x_calib bf16 [Mc, K]; Mc, N > 0, K % 64 == 0, group_size == 64,
 *   1 <= n_grid <= 1000.
 */
svdq_status svdq_awq_pack_weights(const uint16_t* w, const uint16_t* x_calib, int64_t Mc, int64_t N,
                                  int64_t K, int64_t group_size, int n_grid, float* smooth,
                                  uint8_t* w_codes, uint16_t* w_scales, uint8_t* w_zeros,
                                  float* alpha_out);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
