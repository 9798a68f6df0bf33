/*
 * sbn.h -- C ABI of the Sparse-BitLinear hot path for AMD Instinct MI355X (gfx950).
 *
 * The operator is the Sparse-BitLinear layer of "Sparse-BitNet: 1.58-bit LLMs
 * are Naturally Friendly to Semi-Structured Sparsity" (arXiv 2603.05168), as
 * summarised on the gist.science pages (Japanese "技術概要" §2.1, German
 * "Technische Zusammenfassung" §2, Korean "기술 요약" §2.1-2.2, French
 * "Résumé technique" §2) and the fugumt.com abstract page.  It replaces a
 * linear layer: BF16 master weights W [R x K] get an N:M mask from their
 * magnitudes, are ternarized to {-1, 0, +1} with one per-tensor scale and
 * masked (quantize, then mask), and multiply int8 activations.  The backward
 * pass is a straight-through estimator on both quantizers with a dense
 * gradient through the mask.
 *
 * Shapes: T tokens, R output features, K input features.  N:M groups run
 * along K inside each output row.  Supported ratios: m in {4, 8} and
 * 1 <= n <= m (n == m is the dense-ternary control).  K must be a multiple
 * of 64.
 *
 * Packed weight format ("SBN-v1", the explicit N:M metadata of the
 * quantize-then-mask order; the pages do not print a layout):
 *   meta  : per row a K-bit bitmap, bit (g*m + p) set iff position p of
 *           group g survives; bit b is bit (b & 7) of byte (b >> 3).
 *           Row stride K/8 bytes.  Absent (may be NULL, 0 bytes) when n == m.
 *   codes : per row the 2-bit codes of the survivors in increasing k; the
 *           j-th survivor uses bits 2j and 2j+1, same bit order.
 *           00 = 0, 01 = +1, 11 = -1.  Row stride K*n/(4*m) bytes.
 *   s_w   : one float, the per-tensor scale (device memory).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps them.  bf16 tensors are passed as
 *     uint16_t bit patterns.  All tensors are row-major; leading dimensions
 *     (ld*) are in elements.  Device pointers must be 16-byte aligned and
 *     leading dimensions multiples of 8 elements.
 *   - Scales s_w and s_x stay on the device; no call synchronises the host.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *   - Scratch memory is the caller's workspace `ws` of at least
 *     sbn_workspace_bytes() bytes (ws may be NULL when that size is 0).
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error nothing is launched, outputs are untouched, and a message is
 *     available from sbn_last_error() (per thread).  No C++ exception or
 *     abort crosses the ABI.
 *   - Inputs with NaN or Inf are outside the contract.  Activations with
 *     |x| >= 2^120 are outside the contract (127*x must not overflow).
 *     With the environment variable SBN_CHECK_FINITE=1 (read on every call),
 *     the calls that take bf16 or fp32 inputs (W, G, X, dY) scan them first
 *     and return SBN_ERR_VALUE, launching nothing else, if one holds a NaN or
 *     Inf.  The scan synchronises the stream (a diagnostic mode) and is
 *     skipped while the stream is being captured into a graph.
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef SBN_H
#define SBN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SBN_ABI_VERSION 2

typedef enum sbn_status {
  SBN_OK = 0,
  SBN_ERR_NULL = 1,            /* a required pointer is NULL */
  SBN_ERR_SHAPE = 2,           /* T, R, K < 1; K % 64 != 0; ld < row length; T > 16 for the GEMV */
  SBN_ERR_UNSUPPORTED_NM = 3,  /* m not in {4, 8} or n not in [1, m] */
  SBN_ERR_ALIGN = 4,           /* pointer not 16-byte aligned or ld not a multiple of 8 */
  SBN_ERR_WORKSPACE = 5,       /* ws_bytes smaller than sbn_workspace_bytes() */
  SBN_ERR_DTYPE = 6,           /* output dtype not allowed for this call */
  SBN_ERR_HIP = 7,             /* a HIP launch or runtime call failed */
  SBN_ERR_FLAGS = 8,           /* a flag bit this call does not accept */
  SBN_ERR_VALUE = 9            /* a scalar argument out of range (e.g. a non-finite lr), or a
                                  non-finite input under SBN_CHECK_FINITE=1 */
} sbn_status;

typedef enum sbn_dtype {
  SBN_F32 = 0,                 /* float32 */
  SBN_BF16 = 1,                /* bfloat16, round to nearest even from float32 */
  SBN_I32_ACC = 2              /* raw int32 accumulator sum_k Xq*Wt, unscaled */
} sbn_dtype;

/*
 * Variant flags.  The two ablations the pages report (gist.science de §4
 * "Ablationsstudien", fr §5 "Importance de la Stratégie d'Optimisation": both
 * make training worse) are kept as switches of the method's own calls, for
 * that comparison:
 *   SBN_MASK_FROM_TERNARY  pack: the mask keeps, per group, the n largest |q|
 *                          of the ternary weights q = RoundClip(w / s_w)
 *                          (0 or 1) instead of the n largest |w| of the master
 *                          weights; ties go to the lower index as before.
 *   SBN_GRAD_W_MASKED      backward: dW is 0 wherever the meta bit of (r, k)
 *                          is clear (gradients blocked for pruned weights)
 *                          instead of the dense gradient.  No effect at n == m.
 */
typedef enum sbn_flags {
  SBN_FLAGS_NONE = 0,
  SBN_MASK_FROM_TERNARY = 1,
  SBN_GRAD_W_MASKED = 2
} sbn_flags;

typedef enum sbn_op {
  SBN_OP_PACK = 0,
  SBN_OP_ACT_QUANT = 1,
  SBN_OP_GEMM = 2,
  SBN_OP_GEMV = 3,
  SBN_OP_BACKWARD = 4,
  SBN_OP_FORWARD = 5,
  SBN_OP_GEMM_PREPARED = 6
} sbn_op;

/* ABI version of the loaded library (SBN_ABI_VERSION). */
int sbn_abi_version(void);

/* Static English text for a status code. */
const char* sbn_status_string(sbn_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* sbn_last_error(void);

/*
 * Allocation sizes of the packed planes for an R x K weight at ratio n:m:
 * codes_bytes = R*K*n/(4*m) and meta_bytes = R*K/8 (0 when n == m), each
 * rounded up to a multiple of 16 bytes.  The data fill the first
 * R*K*n/(4*m) and R*K/8 bytes; readers load whole aligned words, so the
 * buffers must have the rounded sizes.
 * Host-only; errors: SBN_ERR_NULL, SBN_ERR_SHAPE, SBN_ERR_UNSUPPORTED_NM.
 */
sbn_status sbn_packed_bytes(int64_t R, int64_t K, int n, int m,
                            size_t* codes_bytes, size_t* meta_bytes);

/*
 * Workspace bytes needed by `op` at these sizes (0 if none).  Host-only.
 * Arguments that do not apply to `op` are ignored (pass 0).
 */
sbn_status sbn_workspace_bytes(sbn_op op, int64_t T, int64_t R, int64_t K,
                               int n, int m, size_t* bytes);

/*
 * Mask, ternarize and pack the master weights.
 *
 * Mask (gist.science de §2 "Methodik", ko §2.1, fr §2, ja §2.1): in every
 * group of m consecutive weights along K, keep the n largest |w| of the
 * BF16 master weights; equal magnitudes go to the lower index.  The mask is
 * recomputed from W on every call (ja §2.1, ko §2.2: every training step).
 * Scale: s_w = max(fp32(mean |W|), 1e-5), the mean taken exactly over all
 * R*K entries before masking (quantize-then-mask order, ja §2.1, fr §2) and
 * rounded once to fp32.
 * Ternarize: q = RoundClip(w / s_w, -1, 1), round half to even, i.e.
 * q = sign(w) if |w| > s_w/2 else 0; pruned positions are 0.
 *
 *   W      [R x K] bf16, row stride ldw >= K                         (in)
 *   codes  [R x K*n/(4m)] bytes                                     (out)
 *   meta   [R x K/8] bytes; ignored and may be NULL when n == m     (out)
 *   s_w    1 float                                                  (out)
 *   ws     workspace of sbn_workspace_bytes(SBN_OP_PACK, 0, R, K, n, m); needs
 *          no initialisation (it holds per-block partial sums of |w|).
 *
 * Limits: K <= 2^18 and R*K < 2^37.
 * The result is bit-for-bit independent of launch geometry (the sum of
 * |w| is formed exactly in integer arithmetic).
 */
sbn_status sbn_mask_ternarize_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw,
                                   int n, int m, uint8_t* codes, uint8_t* meta, float* s_w,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * sbn_mask_ternarize_pack with variant flags: 0 or SBN_MASK_FROM_TERNARY.
 * Other flag bits: SBN_ERR_FLAGS.  Arguments and limits as above.
 */
sbn_status sbn_mask_ternarize_pack_ex(const uint16_t* W, int64_t R, int64_t K, int64_t ldw,
                                      int n, int m, uint32_t flags, uint8_t* codes, uint8_t* meta,
                                      float* s_w, void* ws, size_t ws_bytes, void* stream);

/*
 * sbn_mask_ternarize_pack without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): same arguments and results bit for
 * bit, no flags.  Its scratch is a fixed 528 KiB array inside the library, one
 * per GPU, kept until the process ends; the call allocates and frees nothing.
 * Limit: R*K <= 2^28 (larger weights return SBN_ERR_WORKSPACE and launch
 * nothing; use sbn_mask_ternarize_pack with a workspace).  All calls on one GPU
 * share that scratch: calls that overlap on one GPU (different streams, or
 * threads, without ordering) race and are outside the contract; calls ordered
 * on one stream are fine.  SBN_CHECK_FINITE is not applied.
 */
sbn_status sbn_mask_ternarize_pack_noalloc(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                                           uint8_t* codes, uint8_t* meta, float* s_w, void* stream);

/*
 * One optimizer step on the BF16 master weights followed by the next
 * step's mask/ternarize/pack of the updated weights, in two passes over W.
 * The pages keep BF16 master weights that receive the gradients and
 * recompute the mask from them at every step (ja §2.1, ko §2.2) but name no
 * optimizer; this is plain SGD:
 *   W[r,k] <- bf16(fma(-lr, G[r,k], W[r,k]))   (one float32 rounding of the
 *             exact value, then round half to even to bf16), in place;
 * then exactly sbn_mask_ternarize_pack_ex(W, ...) of the new W.  Pass 1
 * updates W and sums |W| from the values it writes; pass 2 masks and packs,
 * so W is read twice and written once (an update followed by a separate
 * pack reads it three times).
 *
 *   W      [R x K] bf16, row stride ldw >= K        (in/out, updated in place)
 *   G      [R x K] float32, row stride ldg >= K     (in, e.g. dW of sbn_backward)
 *   lr     learning rate, finite (else SBN_ERR_VALUE)
 *   flags  0 or SBN_MASK_FROM_TERNARY
 *   codes, meta, s_w, ws: as sbn_mask_ternarize_pack (workspace of
 *          sbn_workspace_bytes(SBN_OP_PACK, 0, R, K, n, m))
 * An update that overflows bf16 is outside the contract.
 */
sbn_status sbn_sgd_update_pack(uint16_t* W, int64_t R, int64_t K, int64_t ldw, const float* G,
                               int64_t ldg, float lr, int n, int m, uint32_t flags, uint8_t* codes,
                               uint8_t* meta, float* s_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-token absmax int8 quantization of the activations (the pages leave
 * the activation path open; this is the 1.58-bit BitNet convention):
 *   a = max(max_k |x[t,k]|, 1e-5); Xq = rint((127*x) / a) in float32,
 *   round half to even, in [-127, 127]; s_x[t] = a / 127 (float32).
 *
 *   X   [T x K] bf16, row stride ldx >= K   (in)
 *   Xq  [T x K] int8, contiguous            (out)
 *   s_x [T] float                           (out)
 */
sbn_status sbn_act_quant(const uint16_t* X, int64_t T, int64_t K, int64_t ldx,
                         int8_t* Xq, float* s_x, void* stream);

/*
 * Sparse ternary matmul, the forward of Sparse-BitLinear (ja §2.1, de §2;
 * the pages run it on a custom 6:8 sparse kernel, ja §3.2, de §4):
 *   acc[t,r] = sum_k Xq[t,k] * Wt[r,k]   (exact int32)
 *   Y[t,r]   = fl32(fl32(acc) * fl32(s_w * s_x[t]))   for SBN_F32,
 *              that value rounded to bf16            for SBN_BF16,
 *              acc                                   for SBN_I32_ACC.
 *
 *   Xq [T x K] int8 contiguous, s_x [T] float             (in)
 *   codes, meta, s_w: packed weight from sbn_mask_ternarize_pack (in)
 *   Y  [T x R] of dtype ydt, row stride ldy >= R          (out)
 *   ws workspace of sbn_workspace_bytes(SBN_OP_GEMM, T, R, K, n, m)
 *
 * 2:4 runs on the gfx950 structured-sparse int8 matrix instructions; other
 * ratios expand to dense int8 tiles and run on dense int8 matrix cores.
 */
sbn_status sbn_sparse_ternary_gemm(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                   const uint8_t* codes, const uint8_t* meta, const float* s_w,
                                   int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * For weights that serve many GEMM calls (inference): the weight operand the
 * GEMM builds from the packed planes on every call, built once.
 * sbn_gemm_weight_bytes: its size (host-only).
 * sbn_prepare_gemm_weight: packed planes (meta NULL when n == m) -> prepared
 *   operand (device, sbn_gemm_weight_bytes(R, K, n, m) bytes, opaque layout).
 * sbn_sparse_ternary_gemm_prepared: the sparse_ternary_gemm on it, same
 *   results bit for bit; ws of sbn_workspace_bytes(SBN_OP_GEMM_PREPARED, T, R,
 *   K, n, m) bytes (0 for every ratio in this version: the activations are
 *   read in place; ws may then be NULL).
 * Errors: as sbn_sparse_ternary_gemm.
 */
sbn_status sbn_gemm_weight_bytes(int64_t R, int64_t K, int n, int m, size_t* bytes);
sbn_status sbn_prepare_gemm_weight(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                                   uint8_t* prepared, void* stream);
sbn_status sbn_sparse_ternary_gemm_prepared(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                            const uint8_t* prepared, const float* s_w, int64_t R, int n, int m,
                                            void* Y, sbn_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                                            void* stream);

/*
 * The whole forward of one Sparse-BitLinear call in one entry point:
 *   sbn_mask_ternarize_pack_ex(W, ..., flags) ; sbn_act_quant(X, ...) ;
 *   sbn_sparse_ternary_gemm(Xq, s_x, ..., Y)
 * with the same results, bit for bit.  The activation quantizer does not
 * depend on the weight pack; at 2:4 it runs in the same launch as the pack's
 * second pass, side by side, which saves a launch and overlaps their memory
 * traffic.  At 2:4 with flags 0, where the GEMM takes its wide tiles, that
 * second pass also writes the GEMM's weight operand into ws and the GEMM
 * reads it and Xq in place (three launches, no layout launch); ws keeps the
 * same size either way.
 *
 *   W      [R x K] bf16, row stride ldw >= K                    (in)
 *   X      [T x K] bf16, row stride ldx >= K                    (in)
 *   flags  0 or SBN_MASK_FROM_TERNARY
 *   codes, meta, s_w                                            (out, as the pack)
 *   Xq [T x K] int8 contiguous, s_x [T] float                   (out, as act_quant)
 *   Y  [T x R] of dtype ydt, row stride ldy >= R                (out, as the GEMM)
 *   ws workspace of sbn_workspace_bytes(SBN_OP_FORWARD, T, R, K, n, m)
 * Limits and errors: those of the three calls.
 */
sbn_status sbn_forward(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, const uint16_t* X, int64_t T,
                       int64_t ldx, int n, int m, uint32_t flags, uint8_t* codes, uint8_t* meta, float* s_w,
                       int8_t* Xq, float* s_x, void* Y, sbn_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Same operation as sbn_sparse_ternary_gemm for decode batches, 1 <= T <= 16:
 * streams the packed weight once from memory and unpacks it in registers.
 * ws: sbn_workspace_bytes(SBN_OP_GEMV, ...) (currently 0).
 */
sbn_status sbn_sparse_ternary_gemv(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                   const uint8_t* codes, const uint8_t* meta, const float* s_w,
                                   int64_t R, int n, int m, void* Y, sbn_dtype ydt, int64_t ldy,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * sbn_sparse_ternary_gemv over `count` weights that share the activations
 * (e.g. the projections of one layer that read the same tokens), in one
 * launch where the shapes allow (2:4 and 6:8 with K a multiple of 1024 up to
 * 4096; otherwise one launch per weight):
 *   Y_b = that call's result for (Xq, s_x, codes[b], meta[b], s_w[b])
 * for b < count.  codes, meta, s_w and Y are HOST arrays of `count` device
 * pointers (meta may be NULL, or hold NULLs, when n == m); every weight is
 * R x K at ratio n:m, every Y_b is [T x R] of dtype ydt with row stride ldy.
 * The pointer arrays are read during the call and not kept.
 * Errors: as sbn_sparse_ternary_gemv, and SBN_ERR_SHAPE for count < 1 or
 * count > SBN_GEMV_MAX_BATCH.
 */
#define SBN_GEMV_MAX_BATCH 64
sbn_status sbn_sparse_ternary_gemv_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                           const uint8_t* const* codes, const uint8_t* const* meta,
                                           const float* const* s_w, int64_t R, int n, int m,
                                           void* const* Y, sbn_dtype ydt, int64_t ldy, int64_t count,
                                           void* stream);

/*
 * One weight of a decode GEMV table: the device pointers of sbn_sparse_ternary_
 * gemv's per-weight arguments (for a decode plane: codes = the plane, meta
 * unused).  Four pointers, 32 bytes, 8-byte aligned.
 */
typedef struct sbn_gemv_entry {
  const uint8_t* codes;
  const uint8_t* meta;
  const float* s_w;
  void* Y;
} sbn_gemv_entry;

/*
 * sbn_sparse_ternary_gemv over `count` weights sharing the activations, with
 * the weights listed in a table in DEVICE memory, in one launch whatever the
 * count (decode over a whole pool of weights: the launch's start-up and drain
 * are paid once, and the caller builds the table once and reuses it across
 * steps and graph replays):
 *   Y_b = that call's result for (Xq, s_x, table[b].codes, table[b].meta,
 *         table[b].s_w), written to table[b].Y, for b < count.
 * Every weight is R x K at ratio n:m; every Y_b is [T x R] of dtype ydt with
 * row stride ldy.  Covered shapes: 1 <= T <= 16, K a multiple of 1024 up to
 * 4096, n:m 2:4 or 6:8; others return SBN_ERR_SHAPE / SBN_ERR_UNSUPPORTED_NM
 * (use the batched call).  count * ceil(R / 16) <= 2^40.
 * The table and every pointer in it are read by the kernel, not by the host:
 * they must stay valid and unchanged until the launch completes, and the
 * library cannot check them.  sbn_gemv_table_check checks a host copy of a
 * table (each entry as sbn_sparse_ternary_gemv checks its arguments); an
 * entry that would fail it gives undefined results (a misaligned or dangling
 * pointer can fault the device).  Only `table` itself is checked here
 * (non-NULL, 16-byte aligned).
 */
sbn_status sbn_sparse_ternary_gemv_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                         const sbn_gemv_entry* table, int64_t count, int64_t R, int n, int m,
                                         sbn_dtype ydt, int64_t ldy, void* stream);

/*
 * Host-only check of a GEMV table before it is copied to the device: every
 * entry of the HOST array `table` (count entries) against the arguments of a
 * later table call of the given form: SBN_FORM_PACKED for
 * sbn_sparse_ternary_gemv_table, SBN_FORM_D2 for sbn_ternary_gemv_d2_table,
 * SBN_FORM_J6 for sbn_ternary_gemv_j6_table (n, m ignored for the last two).
 * Returns the first failure, naming the entry; SBN_ERR_VALUE for an unknown form.
 */
#define SBN_FORM_PACKED 0
#define SBN_FORM_D2 1
#define SBN_FORM_J6 2
sbn_status sbn_gemv_table_check(const sbn_gemv_entry* table, int64_t count, int64_t T, int64_t K, int64_t R,
                                int n, int m, int form, sbn_dtype ydt, int64_t ldy);

/*
 * Decode plane: a byte-lean form of a packed weight for memory-bound decode
 * (not a format of the pages; at 6:8 the packed planes hold 2.5 bits per
 * weight, the decode plane 2).  It holds the effective ternary weights (pruned
 * positions 0) at one 2-bit code per position (00 = 0, 01 = +1, 11 = -1), no
 * bitmap: row r is K/16 little-endian 32-bit words, word w holds positions
 * 16w .. 16w+15, position 16w + 4k + b (k, b in 0..3) in bits 8b + 6 - 2k
 * (low) and 8b + 7 - 2k (high).  Row stride K/4 bytes.
 *
 * sbn_decode_plane_bytes: R*K/4 rounded up to 16 (host-only).
 * sbn_repack_d2: packed planes (codes, meta of an n:m weight; meta NULL when
 *   n == m) -> decode plane d2 of sbn_decode_plane_bytes(R, K) bytes.
 * sbn_ternary_gemv_d2: the decode GEMV of sbn_sparse_ternary_gemv on a decode
 *   plane, 1 <= T <= 16, same results (Y as there; s_w the weight's scale).
 * sbn_ternary_gemv_d2_batched: the same over `count` planes sharing the
 *   activations, one launch (K a multiple of 1024 up to 4096; else one launch
 *   per plane); d2, s_w and Y are HOST arrays of device pointers.
 * Errors: as the packed-weight calls; SBN_ERR_SHAPE for count outside
 * [1, SBN_GEMV_MAX_BATCH].
 */
sbn_status sbn_decode_plane_bytes(int64_t R, int64_t K, size_t* bytes);
sbn_status sbn_repack_d2(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, int n, int m,
                         uint8_t* d2, void* stream);
sbn_status sbn_ternary_gemv_d2(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* d2,
                               const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy, void* stream);
sbn_status sbn_ternary_gemv_d2_batched(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                       const uint8_t* const* d2, const float* const* s_w, int64_t R,
                                       void* const* Y, sbn_dtype ydt, int64_t ldy, int64_t count, void* stream);
/*
 * sbn_ternary_gemv_d2_table: sbn_ternary_gemv_d2 over a DEVICE table of
 * `count` planes (table[b].codes = plane b; meta unused) sharing the
 * activations, one launch, as sbn_sparse_ternary_gemv_table (K a multiple of
 * 1024 up to 4096, 1 <= T <= 16, count * ceil(R / 16) <= 2^40; the entries
 * are the caller's to keep valid and are not checked here).
 */
sbn_status sbn_ternary_gemv_d2_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                     const sbn_gemv_entry* table, int64_t count, int64_t R, sbn_dtype ydt,
                                     int64_t ldy, void* stream);

/*
 * Joint 2:4 code: a byte-lean form of a 2:4 packed weight for memory-bound
 * decode (not a format of the pages; the pages benchmark 2:4 decode,
 * gist.science/ja 技術概要 §3.2, gist.science/de Technische Zusammenfassung §4).
 * Each group of four effective ternary weights (at most two nonzeros) is one
 * 6-bit code, 1.5 bits per weight against the packed planes' 2:
 *   code = nib | h << 4, nib = i1 | i2 << 2 (positions of two slots);
 *   i1 != i2: slot values v1 = h & 1 ? -1 : +1, v2 = h & 2 ? -1 : +1;
 *   i1 == i2: v1 = 0, +1, -1 for h = 0, 1, 3, v2 = 0;
 *   the group's weights are v1 at i1 plus v2 at i2.
 * Canonical code (what sbn_repack_j6 writes): two nonzeros at i < j ->
 * (i, j) with their signs; one nonzero at p -> (p, p) with its code; none -> 0.
 * Two planes, row-major:
 *   nibble plane, K/8 bytes per row: nib of group g in bits 4(g % 2) of byte
 *     g / 2 (32-bit little-endian word v holds groups 8v .. 8v+7 at bits
 *     4(g % 8): the 2:4 matrix instruction's index word for those positions);
 *   h plane, K/16 bytes per row: 32-bit little-endian word u holds groups
 *     16u .. 16u+15, group 16u + 8b + 2k + o (b, o in 0..1, k in 0..3) in
 *     byte k at bits 2(2b + o) and 2(2b + o) + 1.
 *
 * sbn_j6_bytes: nibble- and h-plane bytes, R*K/8 and R*K/16 each rounded up
 *   to 16 (host-only).  K a multiple of 64.
 * sbn_repack_j6: 2:4 packed planes (codes, meta) -> the two planes.  K a
 *   multiple of 64.  The inputs must be 2:4 planes as sbn_mask_ternarize_pack
 *   writes them (two survivors per group).
 * sbn_ternary_gemv_j6: the decode GEMV of sbn_sparse_ternary_gemv on the
 *   joint code (same results bit for bit; s_w the weight's scale), 1 <= T <=
 *   16, K a multiple of 1024 up to 4096 (else SBN_ERR_SHAPE).
 * sbn_ternary_gemv_j6_table: the same over a DEVICE table of weights
 *   (table[b].codes = nibble plane, table[b].meta = h plane), one launch, as
 *   sbn_sparse_ternary_gemv_table.
 * Errors: as the packed-weight calls.
 */
sbn_status sbn_j6_bytes(int64_t R, int64_t K, size_t* nib_bytes, size_t* h_bytes);
sbn_status sbn_repack_j6(const uint8_t* codes, const uint8_t* meta, int64_t R, int64_t K, uint8_t* nib,
                         uint8_t* hpl, void* stream);
sbn_status sbn_ternary_gemv_j6(const int8_t* Xq, const float* s_x, int64_t T, int64_t K, const uint8_t* nib,
                               const uint8_t* hpl, const float* s_w, int64_t R, void* Y, sbn_dtype ydt, int64_t ldy,
                               void* stream);
sbn_status sbn_ternary_gemv_j6_table(const int8_t* Xq, const float* s_x, int64_t T, int64_t K,
                                     const sbn_gemv_entry* table, int64_t count, int64_t R, sbn_dtype ydt,
                                     int64_t ldy, void* stream);

/*
 * Dual-STE backward of Sparse-BitLinear (ja §2.1, de §2 "Dual STE",
 * ko §2.2, fr §2): identity Jacobian through both quantizers and a dense
 * gradient through the mask, so every master weight receives a gradient.
 *   dX[t,k] = sum_r dY[t,r] * s_w * Wt[r,k]       (through the sparse ternary W)
 *   dW[r,k] = sum_t dY[t,r] * s_x[t] * Xq[t,k]    (dense, every (r,k))
 * No derivative of s_w or s_x is taken.  Accumulation is float32.
 *
 *   dY [T x R] bf16 contiguous                     (in)
 *   Xq [T x K] int8 contiguous, s_x [T] float      (in, from sbn_act_quant)
 *   codes, meta, s_w: packed weight                (in)
 *   dX [T x K] of dtype dxdt (SBN_F32 or SBN_BF16), contiguous; may be NULL (out)
 *   dW [R x K] float, contiguous; may be NULL      (out)
 *   ws workspace of sbn_workspace_bytes(SBN_OP_BACKWARD, T, R, K, n, m)
 * R must be a multiple of 8 (dY rows are read in 16-byte units).
 */
sbn_status sbn_backward(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                        const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                        const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * sbn_backward with variant flags: 0 or SBN_GRAD_W_MASKED (then meta is
 * required when n < m, and dW at pruned positions is written as 0).
 * Other flag bits: SBN_ERR_FLAGS.  Arguments as sbn_backward.
 */
sbn_status sbn_backward_ex(const uint16_t* dY, int64_t T, int64_t R, const int8_t* Xq,
                           const float* s_x, int64_t K, const uint8_t* codes, const uint8_t* meta,
                           const float* s_w, int n, int m, void* dX, sbn_dtype dxdt, float* dW,
                           uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel timing (diagnostics; not part of the operator).  While enabled,
 * every kernel the library launches whose name equals `kernel` (or every
 * kernel, when `kernel` is NULL) is bracketed by two HIP events recorded on
 * the stream it runs on.  sbn_profile_dump waits for the recorded events
 * and writes one line per kernel name, "name launches total_ms\n", into buf
 * (NUL-terminated, truncated to buf_bytes); sbn_profile_reset forgets them.
 * Kernel names: abs_sum, sgd_abs_sum, mask_pack, mask_pack_quant, act_quant, layout_sparse, layout_dense,
 * gemm_smfmac, gemm_mfma, gemv, gemv_stream_24, gemv_stream_68, repack_d2, gemv_stream_d2, gemv_d2, expand_wt,
 * prep_u, prep_xq, gemm_dx, gemm_dw.
 * Errors: SBN_ERR_NULL (buf), SBN_ERR_HIP.
 */
sbn_status sbn_profile_enable(int on, const char* kernel);
sbn_status sbn_profile_reset(void);
sbn_status sbn_profile_dump(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif

#endif /* SBN_H */
