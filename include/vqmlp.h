/*
 * vqmlp.h -- C ABI of the VQ3 quantized-MLP forward for AMD MI355X (gfx950).
 *
 * The operation (web page: model card "anemll/anemll-forge-qwen3.8-27B"):
 *   - every MLP matrix (gate, up, down) is a three-bit vector lookup table "2x64": 64
 *     two-component FP16 centroids, one six-bit index per pair of output channels, per-channel
 *     scales (section "Release 0.2: three-bit MLP, token-mixer rotations, distilled weights",
 *     format table and first bullet).  This library stores one 64-entry codebook per group of 8
 *     output rows; code[p][j] selects (W[2p][j], W[2p+1][j]); the row scale multiplies the row;
 *   - the MLP input is scaled per channel and rotated online by block-Hadamard matrices with
 *     seeded signs, the weights living in the rotated basis (same section, second bullet; section
 *     "Files and runtime compatibility", first bullet);
 *   - the activation is silu(g) = g*sigmoid(g) ("ANEMLL ANE LLM conversion pipeline", Facts, item
 *     on Forge numerics), applied as silu(gate) * up, followed by the rotated down projection.
 *
 * So, for x [T][H]:
 *   x~ = R_H(x . s),  a = silu(W_gate x~) . (W_up x~),  y = W_down R_I(a),
 *   R_n = (I (x) H_b / sqrt(b)) diag(sign),  H_b the Sylvester Hadamard matrix of order b,
 *   W[r][j] = cb[r/8][code[r/2][j]][r%2] * sc[r].
 * y is rounded to FP16 (round to nearest even); everything before it accumulates in FP32, with
 * x~ and the rotated activation held in FP16 as matrix-core operands.
 *
 * Conventions: every entry point returns a vqmlp_status (0 = OK); no C++ exception crosses the
 * ABI.  On failure nothing has been launched and vqmlp_last_error() (per thread) explains why.
 * "DEVICE" pointers are HIP device allocations owned by the caller; "HOST" pointers are plain
 * host memory owned by the caller.  `stream` is a hipStream_t (NULL = the legacy default
 * stream); device work is only enqueued, never waited for, and asynchronous device faults
 * surface at the caller's next synchronisation.
 *
 * Tracing: with the environment variable VQMLP_TRACE set to anything but "0", every forward
 * (MLP, 2x16, scalar-LUT, argmax head) writes one line to stderr that names the kernels its
 * dispatch chose and their K splits.  The variable is read on each call.
 */
#ifndef VQMLP_H
#define VQMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQMLP_ABI_VERSION 1
#define VQMLP_LAYOUT_VERSION 1

typedef enum {
    VQMLP_OK = 0,
    VQMLP_ERR_INVALID_ARG = 1, /* null pointer, bad shape, bad code, bad header, misalignment  */
    VQMLP_ERR_UNSUPPORTED = 2, /* valid but not handled: shape limits, non-gfx950 device       */
    VQMLP_ERR_WORKSPACE = 3,   /* workspace too small                                         */
    VQMLP_ERR_HIP = 4          /* a HIP runtime call or launch failed                         */
} vqmlp_status;

int vqmlp_abi_version(void);
/* Text of the last failure on the calling thread ("" if none).  Valid until the next call. */
const char *vqmlp_last_error(void);

/* ------------------------------------------------------------------ one VQ3 matrix W[N][K]
 * Requirements: N % 32 == 0 (16 row pairs per tile), K % 64 == 0, N, K <= 1<<20.
 *
 * Packed layout (version 1), one contiguous buffer:
 *   [0, 256)      header: u32 magic 'VQ3P', u32 layout version, u32 N, u32 K, u32 group rows (8),
 *                 u32 codebook entries (64), u32 kind (0 = VQ3), u32 reserved,
 *                 u64 codes offset, u64 codes bytes, u64 codebook offset, u64 codebook bytes,
 *                 u64 scale offset, u64 scale bytes, u64 total bytes; the rest zero.
 *   codes         (N/32) x (K/64) tiles of 768 bytes, tile (m, k) at (m*(K/64) + k)*768.  A tile
 *                 covers row pairs 16m..16m+15 and columns 64k..64k+63.  Bytes 12*l..12*l+11 of
 *                 the tile form a 96-bit little-endian word for lane l = 0..63 holding 16 six-bit
 *                 codes: code q = 4s+i (bits 6q..6q+5) belongs to pair 16m + (l % 16) and column
 *                 64k + 16s + 4*(l / 16) + i.  (This is the order in which a 64-lane wave consumes
 *                 them as matrix-core operands, so every wave load is one contiguous 768-byte run.)
 *   codebook      [N/8][64][2] binary16, natural order, 256-byte aligned.
 *   scale         [N] binary16, 256-byte aligned.
 */
vqmlp_status vqmlp_packed_bytes(int N, int K, size_t *bytes);

/* Pack HOST arrays into a HOST buffer of at least vqmlp_packed_bytes() bytes.
 *   codes     [N/2][K] uint8, values 0..63 (row p covers output rows 2p, 2p+1)
 *   codebook  [N/8][64][2] binary16 bits; [g][c][0] goes to the even row, [g][c][1] to the odd
 *   row_scale [N] binary16 bits
 * Returns INVALID_ARG for a code above 63, a short buffer or a bad shape. */
vqmlp_status vqmlp_pack(int N, int K, const uint8_t *codes, const uint16_t *codebook,
                        const uint16_t *row_scale, void *packed, size_t packed_bytes);

/* Inverse of vqmlp_pack (HOST to HOST); validates the header first. */
vqmlp_status vqmlp_unpack(int N, int K, const void *packed, size_t packed_bytes, uint8_t *codes,
                          uint16_t *codebook, uint16_t *row_scale);

/* Test hook: w[r][j] = float(cb) * float(sc), exactly (an FP16 x FP16 product fits FP32), for a
 * DEVICE packed buffer; w is DEVICE float [N][K]. */
vqmlp_status vqmlp_dequant(int N, int K, const void *packed, float *w, void *stream);

/* ------------------------------------------------------------------ the MLP plan */
typedef struct {
    int H, I;           /* hidden and intermediate sizes                                    */
    int had_block_h;    /* Hadamard block of the input rotation, power of two in [2, 1024];
                           0 = the largest power of two <= 128 dividing H                    */
    int had_block_i;    /* same for the down projection's input (64 for I = 704)            */
    int t_max;          /* largest T a forward may pass (sizes the workspace)               */
    const void *gate;   /* DEVICE packed VQ3 buffer, N = I, K = H                           */
    const void *up;     /* DEVICE packed VQ3 buffer, N = I, K = H                           */
    const void *down;   /* DEVICE packed VQ3 buffer, N = H, K = I                           */
    const uint16_t *s_in;   /* DEVICE binary16 [H] per-channel input scale                  */
    const int8_t *sign_h;   /* DEVICE int8 [H] +-1, or NULL for all +1                      */
    const int8_t *sign_i;   /* DEVICE int8 [I] +-1, or NULL for all +1                      */
} vqmlp_desc;

typedef struct vqmlp_plan vqmlp_plan;

/* Validate the description (shapes, alignment, gfx950 device, and each packed header through
 * one synchronous device-to-host copy) and build an immutable host-side plan.  The plan keeps
 * the pointers only: it allocates no device memory and the caller keeps every buffer alive. */
vqmlp_status vqmlp_create(const vqmlp_desc *desc, vqmlp_plan **out);
vqmlp_status vqmlp_destroy(vqmlp_plan *plan);

/* Workspace a forward with T rows needs (DEVICE bytes, 256-byte aligned).  The workspace must
 * be zero-filled before its first use; every forward leaves its control words zero again. */
vqmlp_status vqmlp_workspace_bytes(const vqmlp_plan *plan, int T, size_t *bytes);

/* y = MLP(x).  x, y: DEVICE binary16 [T][H], 16-byte aligned, may not overlap the workspace.
 * T == 0 is a no-op.  T <= 8 runs the bandwidth-bound fused kernel (H <= 5120; larger H takes
 * the tiled kernels), T > 8 the matrix-core tiled kernels.  Calls that share a workspace must
 * not overlap in time.
 *
 * The fused T <= 8 kernel is persistent: one workgroup per compute unit, handing operands and
 * partial sums to one another through the workspace.  It needs all of its workgroups resident
 * at once, i.e. no other kernel holding compute units for long while it runs.  Every wait for a
 * hand-off is bounded (about 2^18 short sleeps, milliseconds); a wait that runs out sets a bit
 * in the workspace's error word and the call completes with wrong values in y instead of
 * hanging.  vqmlp_workspace_errors reads (and clears) that word. */
vqmlp_status vqmlp_forward(const vqmlp_plan *plan, int T, const void *x, void *y, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Same as vqmlp_forward with the kernel family chosen by the caller: path 0 = automatic
 * (T <= 8 and H <= 5120: path 1; otherwise path 2), 1 = the fused single-launch T <= 8 kernel
 * (T <= 8, H <= 5120), 2 = the tiled matrix-core kernels (any T; H and I multiples of 64).
 * Path 1 keeps its queue, counters, error word and epoch in the first 64 bytes of the
 * workspace: the caller zero-fills the workspace once, and every call leaves that control block
 * ready for the next call.  VQMLP_ERR_INVALID_ARG for another path number,
 * VQMLP_ERR_UNSUPPORTED when the chosen path does not take the shape or T. */
vqmlp_status vqmlp_forward_path(const vqmlp_plan *plan, int T, const void *x, void *y,
                                void *workspace, size_t workspace_bytes, int path, void *stream);

/* vqmlp_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels with the workspace in a
 * fixed 16 MiB device array that the library holds, one per GPU, until the process ends.  This
 * call allocates nothing and frees nothing.  The array is set up (address fetched, zero-filled)
 * by the first vqmlp_create made with that device current; without one this returns
 * VQMLP_ERR_UNSUPPORTED.  A forward whose workspace (vqmlp_workspace_bytes) exceeds 16 MiB
 * returns VQMLP_ERR_WORKSPACE without launching anything: at H = 5120, I = 17408 every T <= 8
 * fits, larger T only while its tiled-path buffers do.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; serialise them.  The fused kernel's
 * error word (see vqmlp_forward) lives in the array, out of the caller's reach.  Other
 * arguments and errors as vqmlp_forward. */
vqmlp_status vqmlp_forward_noalloc(const vqmlp_plan *plan, int T, const void *x, void *y,
                                   void *stream);

/* Error bits that the fused kernel's bounded waits left in a workspace (see vqmlp_forward):
 * 1 = a projection's operand never arrived, 2 = a rotation block of the gated intermediate never
 * completed, 4 = a partial sum of the down projection never arrived.  0 means every wait of
 * every call since the last clear ended normally.  Waits for `stream` (a host-device
 * synchronisation: not for use inside graph capture), copies the word to *bits and, when
 * clear != 0, zeroes it on `stream` and waits again.  workspace: the DEVICE workspace of
 * vqmlp_forward (256-byte aligned, workspace_bytes >= 64).  VQMLP_ERR_INVALID_ARG for null or
 * unaligned pointers or a short workspace, VQMLP_ERR_HIP when a HIP call fails. */
vqmlp_status vqmlp_workspace_errors(void *workspace, size_t workspace_bytes, int clear,
                                    uint32_t *bits, void *stream);

/* Test hook for the rotation kernels: out[t][.] = R_n(x[t][.] . s) with block b (power of two,
 * 2..1024), FP32 output.  x DEVICE binary16 [T][n]; s DEVICE binary16 [n] or NULL (all 1);
 * sign DEVICE int8 [n] or NULL; out DEVICE float [T][n]. */
vqmlp_status vqmlp_rotate(int T, int n, int b, const uint16_t *x, const uint16_t *s,
                          const int8_t *sign, float *out, void *stream);

/* Measurement hook: reads `bytes` of the DEVICE buffer buf once (16-byte loads, each workgroup a
 * contiguous share, one pass), the plainest weight stream there is: its rate is the HBM read
 * rate that the weight-streaming kernels above can be compared with.  buf 16-byte aligned,
 * bytes a multiple of 16; sink: DEVICE uint32, written only in the unlikely case that the XOR of
 * all words equals one fixed value (so the loads cannot be dropped).  Asynchronous on stream.
 * VQMLP_ERR_INVALID_ARG for null or unaligned arguments, VQMLP_ERR_HIP for a failed launch. */
vqmlp_status vqmlp_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* ------------------------------------------------------------------ scalar-LUT projection
 * Token-mixer format of the same model card (format table, "Token mixers" row; rotation bullet):
 * bits in {2, 4}, one table of 2^bits binary16 scalars per 8 output rows, a binary16 scale per
 * output row, optional rank-r binary16 factors U [N][r] and V [r][K]:
 *   y = W x~ + U (V x~),  x~ = R_K(x . s) with 1024-wide (or had_block) Hadamard blocks.
 * Requirements: N % 64 == 0, K % 64 == 0, r <= 256.
 * Packed layout (version 1): 256-byte header as above (kind 2 for 2-bit, 4 for 4-bit), then
 * codes as [N][K/ (32/bits)] little-endian 32-bit words (code j of row n at bits
 * bits*(j % (32/bits)) of word j / (32/bits)), then the tables [N/8][2^bits] binary16, then the
 * scales [N] binary16, each section 256-byte aligned. */
vqmlp_status vqmlp_lut_packed_bytes(int bits, int N, int K, size_t *bytes);
vqmlp_status vqmlp_lut_pack(int bits, int N, int K, const uint8_t *codes /* [N][K] */,
                            const uint16_t *lut /* [N/8][1<<bits] */,
                            const uint16_t *row_scale /* [N] */, void *packed, size_t bytes);
vqmlp_status vqmlp_lut_unpack(int bits, int N, int K, const void *packed, size_t bytes,
                              uint8_t *codes, uint16_t *lut, uint16_t *row_scale);
vqmlp_status vqmlp_lut_workspace_bytes(int N, int K, int T, int r, size_t *bytes);
/* x DEVICE binary16 [T][K] -> y DEVICE binary16 [T][N].  packed, U, V, s, sign DEVICE; x, y,
 * U, V 16-byte aligned, the workspace 256-byte aligned (no zero fill needed).  r == 0: no
 * factors (U, V ignored); r > 0 needs both.  s, sign NULL: all 1.  had_block 0: no rotation,
 * else a power of two in 2..1024 dividing K.  Returns VQMLP_ERR_INVALID_ARG for bad shapes,
 * pointers or a packed buffer whose header does not match (bits, N, K), VQMLP_ERR_WORKSPACE
 * when workspace_bytes is below vqmlp_lut_workspace_bytes, VQMLP_ERR_HIP for launch errors. */
vqmlp_status vqmlp_lut_forward(int bits, int N, int K, int T, const void *packed,
                               const uint16_t *U, const uint16_t *V, int r, const uint16_t *s,
                               const int8_t *sign, int had_block, const void *x, void *y,
                               void *workspace, size_t workspace_bytes, void *stream);

/* The same projection with its validation done once.  vqmlp_lut_forward checks the device and
 * reads the packed header through a synchronous device-to-host copy on every call, which stalls
 * the host until earlier work has drained; a plan does those checks at creation (same
 * arguments and errors as vqmlp_lut_forward) and keeps the pointers only (no device memory;
 * the caller keeps every buffer alive).  vqmlp_lut_plan_forward then issues no host-device
 * synchronisation: same x, y, workspace rules and errors as vqmlp_lut_forward. */
typedef struct vqmlp_lut_plan vqmlp_lut_plan;
vqmlp_status vqmlp_lut_create(int bits, int N, int K, const void *packed, const uint16_t *U,
                              const uint16_t *V, int r, const uint16_t *s, const int8_t *sign,
                              int had_block, vqmlp_lut_plan **out);
vqmlp_status vqmlp_lut_destroy(vqmlp_lut_plan *plan);
vqmlp_status vqmlp_lut_plan_forward(const vqmlp_lut_plan *plan, int T, const void *x, void *y,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Greedy next token from a scalar-LUT output head (the model card's four-bit LUT head; in-model
 * argmax of the conversion pipeline page, "Facts": the head returns, per token, the index of the
 * largest logit and its value instead of the vocabulary's logits).  plan: a vqmlp_lut_create plan
 * with r == 0 (no factors), K <= 5120, s 16-byte and sign 8-byte aligned (the head's norm gain
 * goes in s; had_block 0: no rotation).  For T <= 8 rows of x (DEVICE binary16 [T][K], 16-byte
 * aligned) writes index[t] (DEVICE int32) = the lowest row n among the largest logits
 * sc[n] * (W_lut x~)[t][n] (FP32 accumulation, no rank term) and, when value is not NULL,
 * value[t] (DEVICE float) = that logit.  Workspace: vqmlp_lut_workspace_bytes(N, K, T, 0), 256-byte
 * aligned, no zero fill.  Errors: VQMLP_ERR_UNSUPPORTED for T > 8, r != 0, K > 5120 or unaligned
 * s / sign; VQMLP_ERR_INVALID_ARG, VQMLP_ERR_WORKSPACE, VQMLP_ERR_HIP as vqmlp_lut_forward.
 * T == 0 is a no-op. */
vqmlp_status vqmlp_lut_plan_argmax(const vqmlp_lut_plan *plan, int T, const void *x,
                                   int32_t *index, float *value, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ 2x16 vector LUT
 * The two-bit vector lookup table "2x16" of the previous packages' MLP (model card, section
 * "Release 0.2: three-bit MLP, token-mixer rotations, distilled weights", format table): 16
 * two-component centroids per group of 8 output rows, one four-bit index per pair of output
 * channels, per-channel scales.  W[r][j] = cb[r/8][code[r/2][j]][r%2] * sc[r], the conventions
 * of the three-bit form with 16 entries.  N and K multiples of 32.
 *
 * vqmlp_vq2_packed_bytes: size of the packed buffer (header, codes [N/2][K/8] words with code j
 * at bits 4 (j % 8) of word j / 8, centroids [N/8][16] words (component 0 in the low half), row
 * scales [N]; sections 256-byte aligned).
 * vqmlp_vq2_pack / vqmlp_vq2_unpack: HOST to HOST; codes [N/2][K] uint8 (0..15, INVALID_ARG
 * above), codebook [N/8][16][2] binary16 bits, row_scale [N] binary16 bits; unpack validates
 * the header first. */
vqmlp_status vqmlp_vq2_packed_bytes(int N, int K, size_t *bytes);
vqmlp_status vqmlp_vq2_pack(int N, int K, const uint8_t *codes, const uint16_t *codebook,
                            const uint16_t *row_scale, void *packed, size_t packed_bytes);
vqmlp_status vqmlp_vq2_unpack(int N, int K, const void *packed, size_t packed_bytes,
                              uint8_t *codes, uint16_t *codebook, uint16_t *row_scale);

/* Projection plan at T <= 8 tokens: y[t][r] = sum_j W[r][j] x[t][j] (x used as given: an input
 * scale or rotation is the caller's), FP32 accumulation, one rounding to binary16.
 * vqmlp_vq2_create: packed is a DEVICE buffer written by vqmlp_vq2_pack (256-byte aligned; its
 * header is read once here, so create synchronises); the plan keeps the pointer only.  Errors:
 * VQMLP_ERR_INVALID_ARG for a bad shape, null or mismatched buffer; VQMLP_ERR_UNSUPPORTED for
 * K > 5120 or a device other than gfx950.
 * vqmlp_vq2_plan_forward: x DEVICE binary16 [T][K] (16-byte aligned), y DEVICE binary16 [T][N];
 * no workspace, no allocation, no host-device synchronisation (stream: a hipStream_t, NULL =
 * default).  Errors: VQMLP_ERR_UNSUPPORTED for T > 8; VQMLP_ERR_INVALID_ARG for null or
 * unaligned pointers; VQMLP_ERR_HIP if the launch fails.  T == 0 is a no-op. */
/* The MLP of the previous packages (same card, format table, "Previous packages" column: gate, up
 * and down as 2x16 vector LUTs): vqmlp_create with every matrix a DEVICE buffer written by
 * vqmlp_vq2_pack (gate and up N = I, K = H; down N = H, K = I).  Same description, rotations,
 * activation, plan rules and errors as vqmlp_create; H and I multiples of 64.  The plan works with
 * vqmlp_workspace_bytes, vqmlp_forward, vqmlp_forward_path, vqmlp_forward_noalloc and
 * vqmlp_destroy: T <= 8 (with I a multiple of 128) runs the 2x16 projection kernel (path 1:
 * gate and up as FP32 planes in K slices of at most 5120 columns, one pass for SiLU, sign and
 * the 128-wide rotation, the down product in K slices, one pass summing the slices), any T the
 * matrix-core kernels with a 2x16 decoder (path 2: the tiled kernels up to T = 32, the
 * register-decode kernels of the three-bit form from T = 33). */
vqmlp_status vqmlp_create_vq2(const vqmlp_desc *desc, vqmlp_plan **out);

typedef struct vqmlp_vq2_plan vqmlp_vq2_plan;
vqmlp_status vqmlp_vq2_create(int N, int K, const void *packed, vqmlp_vq2_plan **out);
vqmlp_status vqmlp_vq2_destroy(vqmlp_vq2_plan *plan);
vqmlp_status vqmlp_vq2_plan_forward(const vqmlp_vq2_plan *plan, int T, const void *x, void *y,
                                    void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VQMLP_H */
