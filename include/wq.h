/*
 * wq.h -- C ABI of libwq: the weight-streaming skinny GEMM of a
 * speculative-decoding verify pass, on AMD MI355X (gfx950).
 *
 * Operation (every entry point):
 *     Y[n][m] = sum_k W[m][k] * X[n][k],   0 <= n < N <= 8, 0 <= m < M
 * with X in BF16, Y in FP32 (FP32 accumulation) and W in one of two stored
 * formats.  This is the product the crit-hub engine card
 * "mtp7-device-confidence" runs for its verify pass (section "Design", rows
 * "Decode" and "GEMVs": one target pass over the drafted columns, 2-8 of
 * them, reading FP8 and NVFP4 weight bytes directly; N = 1 is plain
 * decode), and which its section "Measured" prices by the bytes it reads.
 *
 * Conventions shared by all calls
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees, copies to the host or synchronizes;
 *    a call only enqueues work on `stream` (a hipStream_t; NULL means the
 *    default stream).  The caller keeps every buffer alive until that
 *    work has completed.
 *  - Inputs are read-only.  Y must not alias any input.  Y is overwritten
 *    (never accumulated into).
 *  - Arguments are validated on the host before anything is enqueued; on
 *    any error the call returns a status other than WQ_SUCCESS and has
 *    launched nothing.  Faults during execution surface at the caller's
 *    next synchronization of `stream`.
 *  - Results are deterministic: the same inputs give the same bits on
 *    every call, and column n of Y does not depend on N or on the other
 *    columns of X (the crit-hub card's section "Checks" asks for GEMVs at
 *    1-8 columns "with column invariance"; the crit README's "Kernel
 *    workbench" asks for the same bits on a repeat).  How K is split
 *    depends only on (M, K) and the device, never on N.
 *  - Workspace: some shapes split their work across workgroups and need
 *    scratch memory.  Query its size with the matching *_workspace_bytes
 *    call; pass a device buffer at least that large (16-byte aligned), or
 *    NULL/0 when the query returns 0.  Single-matrix calls (wq_gemm_*): the
 *    buffer must be all zero before its first use (torch.zeros, hipMemset);
 *    its first 16 KiB hold arrival counters that every call leaves zero
 *    again, and the rest is scratch, so any later single-matrix call may
 *    reuse it without clearing (a buffer used by wq_verify_pass or anything
 *    else in between must be zeroed again).  wq_verify_pass's workspace
 *    needs no initialization (its prepare call writes what it needs).
 *    Calls that share one workspace must not overlap in time (same stream
 *    is fine).
 *  - Threading: the library keeps no state besides a per-device cache of
 *    the compute-unit count; calls are reentrant on different streams with
 *    different workspaces.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wq_status {
  WQ_SUCCESS = 0,
  WQ_ERROR_INVALID_VALUE = 1,     /* NULL pointer, N outside 1..8, M or K < 1, count < 1, bad format */
  WQ_ERROR_UNSUPPORTED_SHAPE = 2, /* K not a multiple of 32 (NVFP4) or 16 (FP8-row), or too large */
  WQ_ERROR_MISALIGNED = 3,        /* an array pointer not 16-byte aligned */
  WQ_ERROR_WORKSPACE = 4,         /* workspace NULL or smaller than the query returned */
  WQ_ERROR_LAUNCH = 5,            /* the HIP runtime refused a launch or a copy */
  WQ_ERROR_DEVICE = 6,            /* no current HIP device, or not a gfx950 device */
  WQ_ERROR_SCRATCH_LIMIT = 7      /* wq_gemm_nvfp4_tiled_noalloc: the shape needs more scratch than
                                     the library's static buffer holds */
} wq_status;

enum { WQ_FMT_NVFP4 = 0, WQ_FMT_FP8ROW = 1, WQ_FMT_NVFP4_TILED = 2, WQ_FMT_FP8ROW_TILED = 3 };

/* Human-readable name of a status code (static string, never NULL). */
const char* wq_status_string(wq_status s);

/* Bytes of workspace the single-matrix call of format `fmt` needs
 * (wq_gemm_nvfp4, wq_gemm_fp8row, wq_gemm_nvfp4_tiled or
 * wq_gemm_fp8row_tiled) for this shape on the current device; 0 when
 * the shape is computed without splitting K.  Returns 0 for invalid
 * arguments too (the GEMM call then reports the error). */
size_t wq_gemm_workspace_bytes(int fmt, int M, int K, int N);

/* The K split a call will use: K is cut into *n_chunks chunks of *k_chunk
 * (the last may be shorter).  in_verify_pass = 0 asks about the
 * single-matrix calls (wq_gemm_*) on the current device, 1 about a matrix
 * inside wq_verify_pass, 2 about a matrix that wq_verify_pass computes in
 * blocks (a large split matrix of a pass of tiled matrices only; see
 * wq_verify_pass).  Two calls that report the same split compute
 * bit-identical results for the same matrix and columns.
 * *k_chunk = 0 (single calls on the tiled formats with fewer than 8 row
 * tiles of 16 per compute unit) reports the split-tile mode: the steps of
 * the *n_chunks K chunks are cut into one equal run per workgroup and one
 * equal piece per wave, each tile's pieces are added in k order (in LDS,
 * then across workgroups by the last one to arrive), so every compute unit
 * streams the same bytes; the cut depends on (M, K) and the device, never on
 * N, and the rounding differs from that of the chunked calls. */
wq_status wq_gemm_split(int fmt, int M, int K, int in_verify_pass, int* k_chunk, int* n_chunks);

/* NVFP4 weights.
 *   codes  [M][K/2] uint8: two E2M1 codes per byte; byte j of row m holds
 *          k = 2j in its low nibble and k = 2j+1 in its high nibble.
 *          E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.
 *   scales [M][K/16] uint8: one E4M3 (FN) scale per 16 consecutive k;
 *          scale b of row m covers k in [16b, 16b+16).  NaN scales
 *          propagate to the outputs they touch.
 *   global_scale  FP32 per-tensor multiplier (not its reciprocal).
 *   x      [N][K] BF16 bit patterns, row-major (row n = column n of X).
 *   y      [N][M] FP32, row-major, overwritten.
 *   W[m][k] = e2m1(code) * e4m3(scale) * global_scale.
 * Requirements: 1 <= N <= 8, M >= 1, K >= 32, K % 32 == 0, M*K/2 < 2^40,
 * codes/scales/x/y 16-byte aligned (x's row stride K*2 bytes is then a
 * multiple of 64; scales' row stride K/16 bytes need only be a multiple
 * of 2, which K % 32 == 0 gives). */
wq_status wq_gemm_nvfp4(const uint8_t* codes, const uint8_t* scales, float global_scale,
                        const uint16_t* x, float* y, int M, int K, int N,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Tiled NVFP4: the same codes and scales, permuted once at load time into
 * the order the NVFP4 kernels stream (the card's section "Design", row
 * "Weights", likewise keeps NVFP4 scales in a kernel-specific tile order).
 * For T = ceil(M/16) row tiles and S = ceil(K/256) steps, block (t, s) is
 * 2304 bytes at offset (t*S + s)*2304 and covers rows 16t..16t+15 and
 * k = 256s..256s+255 (rows >= M and k >= K are zero codes with zero
 * scales).  Inside it, with lane l = c + 16g (c = 0..15, g = 0..3),
 * h = 0..1 and j = 0..3:
 *   bytes [1024h + 16l + 4j, +4) = plain code bytes
 *       [128s + 64h + 16j + 4g, +4) of row 16t + c;
 *   byte 2048 + 8(16p + c) + 4h + j (p = 0..1) = the scale of row 16t + c
 *       for scale block 16s + 8h + 2j + p.
 * wq_nvfp4_tiled_bytes: size of the tiled buffer (0 for an invalid shape).
 * wq_nvfp4_tile / wq_nvfp4_untile: convert on the GPU (enqueue only; all
 *   buffers 16-byte aligned, shapes as for wq_gemm_nvfp4).  untile(tile(w))
 *   reproduces codes and scales bit for bit.
 * wq_gemm_nvfp4_tiled: the product on tiled weights; same results as
 *   wq_gemm_nvfp4 on the plain weights (bit for bit when wq_gemm_split
 *   reports the same split for WQ_FMT_NVFP4 and WQ_FMT_NVFP4_TILED). */
size_t wq_nvfp4_tiled_bytes(int M, int K);
wq_status wq_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, int M, int K,
                        uint8_t* tiled, void* stream);
wq_status wq_nvfp4_untile(const uint8_t* tiled, int M, int K,
                          uint8_t* codes, uint8_t* scales, void* stream);
wq_status wq_gemm_nvfp4_tiled(const uint8_t* tiled, float global_scale,
                              const uint16_t* x, float* y, int M, int K, int N,
                              void* workspace, size_t workspace_bytes, void* stream);

/* wq_gemm_nvfp4_tiled without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace (arrival counters and
 * partial sums) lives in a static device buffer of WQ_NOALLOC_SCRATCH_BYTES
 * inside the library: one per GPU, located on the first call on that GPU
 * and held until the process ends.  That first call also clears the
 * counters, with a small kernel on `stream` ahead of the product; every
 * product leaves them zero again.  The call allocates nothing, on the host
 * or the device.
 * Results are those of wq_gemm_nvfp4_tiled with a workspace, bit for bit.
 * Errors: as wq_gemm_nvfp4_tiled, plus WQ_ERROR_SCRATCH_LIMIT (nothing
 * launched) when wq_gemm_workspace_bytes(WQ_FMT_NVFP4_TILED, M, K, N) exceeds
 * WQ_NOALLOC_SCRATCH_BYTES.  Every call on one GPU shares that GPU's
 * buffer: calls that may overlap in time on one GPU (different streams, or
 * threads without ordering) race and give undefined results; calls ordered
 * on one stream are safe. */
#define WQ_NOALLOC_SCRATCH_BYTES (4u << 20)
wq_status wq_gemm_nvfp4_tiled_noalloc(const uint8_t* tiled, float global_scale,
                                      const uint16_t* x, float* y, int M, int K, int N, void* stream);

/* Row-scaled FP8-E4M3 weights (the card's section "Model": projections and
 * output head stored or re-encoded as FP8 with one scale per output row).
 *   w         [M][K] uint8 E4M3 (FN) codes.
 *   row_scale [M] FP32; W[m][k] = e4m3(w[m][k]) * row_scale[m].
 *   x, y      as for wq_gemm_nvfp4.
 * Requirements: 1 <= N <= 8, M >= 1, K >= 16, K % 16 == 0, M*K < 2^40,
 * w/row_scale/x/y 16-byte aligned. */
wq_status wq_gemm_fp8row(const uint8_t* w, const float* row_scale,
                         const uint16_t* x, float* y, int M, int K, int N,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Tiled FP8-row: the same E4M3 bytes, permuted once at load time so that
 * every wave load is one contiguous kilobyte.  For T = ceil(M/16) row tiles
 * and S = ceil(K/128) steps, block (t, s) is 2048 bytes at offset
 * (t*S + s)*2048 and covers rows 16t..16t+15 and k = 128s..128s+127 (rows
 * >= M and k >= K are zero bytes).  Inside it, with lane l = c + 16g
 * (c = 0..15, g = 0..3) and h = 0..1:
 *   bytes [1024h + 16l, +16) = plain bytes [128s + 64h + 16g, +16) of
 *       row 16t + c.
 * The row scales stay a separate FP32 array [M].
 * wq_fp8_tiled_bytes: size of the tiled buffer (0 for an invalid shape).
 * wq_fp8_tile / wq_fp8_untile: convert on the GPU (enqueue only; buffers
 *   16-byte aligned, shapes as for wq_gemm_fp8row).  untile(tile(w))
 *   reproduces w bit for bit.
 * wq_gemm_fp8row_tiled: the product on tiled weights; same results as
 *   wq_gemm_fp8row on the plain weights (bit for bit when wq_gemm_split
 *   reports the same split for WQ_FMT_FP8ROW and WQ_FMT_FP8ROW_TILED). */
size_t wq_fp8_tiled_bytes(int M, int K);
wq_status wq_fp8_tile(const uint8_t* w, int M, int K, uint8_t* tiled, void* stream);
wq_status wq_fp8_untile(const uint8_t* tiled, int M, int K, uint8_t* w, void* stream);
wq_status wq_gemm_fp8row_tiled(const uint8_t* tiled, const float* row_scale,
                               const uint16_t* x, float* y, int M, int K, int N,
                               void* workspace, size_t workspace_bytes, void* stream);

/* One matrix of a verify pass (host-side descriptor).  For WQ_FMT_NVFP4,
 * `w` = codes, `scales` = block scales, `global_scale` used; for
 * WQ_FMT_NVFP4_TILED, `w` = the tiled buffer, `scales` unused (may be
 * NULL), `global_scale` used; for WQ_FMT_FP8ROW, `w` = E4M3 codes,
 * `scales` = the FP32 row scales (reinterpreted), `global_scale` ignored;
 * for WQ_FMT_FP8ROW_TILED, `w` = the tiled buffer, `scales` = the row
 * scales, `global_scale` ignored.
 * x [N][K], y [N][M] as above. */
typedef struct wq_matrix {
  int32_t fmt;
  int32_t M;
  int32_t K;
  float global_scale;
  const void* w;
  const void* scales;
  const uint16_t* x;
  float* y;
} wq_matrix;

/* Workspace bytes wq_verify_pass needs for these descriptors (the
 * device-side copy of the descriptor table plus split-K scratch). */
size_t wq_verify_workspace_bytes(const wq_matrix* descs, int count, int N);

/* A whole verify pass: `count` independent products, all at the same N,
 * in ONE persistent kernel launch, so that small matrices do not leave
 * HBM idle between launches (the card's section "Decode": the verify pass
 * for the drafts made runs as one node of the round's graph).  `descs` is
 * a HOST array; it is validated, then copied into `workspace` with an
 * asynchronous host-to-device copy on `stream` (so the call is not
 * capture-safe unless the host array is pinned).  Each matrix obeys the
 * requirements of its format's GEMM call; matrices may differ in format
 * and shape.  Results equal, bit for bit, those of the single-matrix
 * calls whenever wq_gemm_split reports the same split for both; otherwise
 * they agree to FP32 rounding of the sums.  In a pass of tiled matrices
 * only, a matrix split in K that is large next to a workgroup's share of
 * the pass (32 or more of its 16-row tiles per workgroup) is computed in
 * blocks of tiles whose chunk sums stay in the workgroup's LDS and are
 * added in chunk order, as the separate reduction adds them: the same bits,
 * no partial sums written, no reduction launch for it. */
wq_status wq_verify_pass(const wq_matrix* descs, int count, int N,
                         void* workspace, size_t workspace_bytes, void* stream);

/* A verify pass split in two, for callers that run the same pass many
 * times (every decode round of an engine) or capture it in a HIP graph:
 * wq_verify_prepare validates the descriptors and writes the device-side
 * table into `workspace` (one asynchronous host-to-device copy on
 * `stream`), filling `plan`; wq_verify_launch then only launches the
 * kernel and can be called any number of times, on any stream ordered
 * after the copy, for as long as the workspace and every matrix buffer
 * stay alive and unchanged in place (apart from the claim counter of the
 * pass's dynamic tail, which each launch advances and none resets).
 * Launches of one plan share that counter: they must run one after
 * another (one stream, or ordered by events), never at the same time.
 * wq_verify_pass is prepare + launch.
 * The plan's fields are owned by the library; callers only keep it
 * (reduce_runs: reduction blocks launched after the pass, 0 when there are
 * none; lds_extra: LDS bytes per workgroup for blocked chunk sums). */
typedef struct wq_verify_plan {
  void* workspace;
  size_t workspace_bytes;
  int32_t count;
  int32_t N;
  int32_t mode;
  int32_t grid;
  size_t ranges_offset;
  size_t reduce_offset;
  int32_t reduce_runs;
  int32_t lds_extra;
} wq_verify_plan;

wq_status wq_verify_prepare(const wq_matrix* descs, int count, int N,
                            void* workspace, size_t workspace_bytes, void* stream,
                            wq_verify_plan* plan);
wq_status wq_verify_launch(const wq_verify_plan* plan, void* stream);

/* The verify pass with its column count read from device memory when the
 * kernels run (the crit-hub engine card, section "Design", row "Decode":
 * the round's graph runs the verify pass for the drafts made, 2-8 columns,
 * a number known only on the device).  `plan` must come from
 * wq_verify_prepare with N = 8 over tiled matrices only (WQ_FMT_NVFP4_TILED
 * and/or WQ_FMT_FP8ROW_TILED; the plan's x and y buffers hold 8 columns);
 * `n_device` is an int32 in device memory, 4-byte aligned, read as
 * n = min(max(*n_device, 1), 8).  Each matrix then gets y[0..n-1] =
 * x[0..n-1] . W^T, bit for bit what a plan prepared for N = n computes;
 * rows n..7 of y are left untouched.  Launch only (capture-safe). */
wq_status wq_verify_launch_n(const wq_verify_plan* plan, const int32_t* n_device, void* stream);

/* The same prepared pass with every NVFP4 step computed on the vector ALUs
 * (BF16 dot-2 instructions, FP32 sums) instead of the matrix cores; tiled
 * FP8-row matrices of the plan keep the matrix-core step.  It exists to
 * price that choice: at these column counts the product streams weights,
 * and the matrix cores are used only because they are measured faster
 * (the crit-hub engine card, section "Design", row "GEMVs", reads the
 * weights into tensor-core fragments on its GPU).  `plan` must come from
 * wq_verify_prepare over tiled matrices only.  Results agree with
 * wq_verify_launch within the products' tolerance (not bit for bit: the
 * sums are grouped differently); column n still has the same bits for every
 * N.  Launch only. */
wq_status wq_verify_launch_valu(const wq_verify_plan* plan, void* stream);

/* Greedy draft acceptance fused onto the output-head product (the crit
 * README, section "Core": greedy draft acceptance is part of sampling;
 * section "Inference": speculative decoding verifies a proposed
 * continuation and keeps the accepted tokens; the crit-hub engine card,
 * section "Design", rows "Decode" and "Exactness": the verify pass runs
 * inside the round's device graph, so the host never waits mid-round, and
 * the output equals plain greedy decoding).
 *   fmt        WQ_FMT_FP8ROW_TILED (w = tiled head, row_scale = FP32 [M]) or
 *              WQ_FMT_NVFP4_TILED (w = tiled head, global_scale used,
 *              row_scale may be NULL).  M = vocabulary rows, K = hidden size.
 *   x          [N][K] BF16: column 0 the hidden state after the last
 *              accepted token, columns 1..N-1 after drafts 1..N-1.
 *   drafts     [N-1] int32, device (may be NULL when N = 1): the drafted
 *              token ids, draft j = drafts[j-1].
 *   logits     [N][M] FP32, device, or NULL: if given, the head's output,
 *              as wq_gemm_*_tiled writes it.
 *   tokens     [N] int32, device: tokens[n] = the row m with the largest
 *              logits[n][m]; the lowest such m on ties; a NaN logit counts
 *              as larger than any number (the lowest NaN row wins); -0 and
 *              +0 are equal.
 *   accepted   [1] int32, device: the number a of leading drafts with
 *              draft j == tokens[j-1] for j = 1..a (0 <= a <= N-1); the
 *              round's output tokens are tokens[0..a].
 * Requirements: as wq_gemm_*_tiled, with K in one K chunk (K <= 8704:
 * wq_gemm_split(fmt, M, K, 1, ...) reports one chunk); tokens, accepted,
 * drafts 4-byte aligned.  The workspace (wq_head_accept_workspace_bytes;
 * no initialization needed) holds one key per workgroup and column.
 * Enqueues two kernels on `stream`; nothing is read back to the host. */
size_t wq_head_accept_workspace_bytes(int fmt, int M, int K, int N);
wq_status wq_head_accept(int fmt, const uint8_t* w, const float* row_scale, float global_scale,
                         const uint16_t* x, int M, int K, int N, const int32_t* drafts,
                         float* logits, int32_t* tokens, int32_t* accepted,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Load-time round-to-nearest quantizers on the GPU (the crit landing page,
 * section on Models: post-training quantization to FP8 or NVFP4 by
 * round-to-nearest; its Gemma case study re-encodes BF16 projections and
 * the output head to FP8 at load; the crit-hub engine card, section
 * "Model", re-encodes the draft layer as row-scaled FP8 and the output
 * head as NVFP4).  Input w [M][K] BF16 bits, finite, row-major.
 *  wq_quantize_fp8row: per row m, row_scale[m] = fp32(max_k |w| / 448) and
 *    q[m][k] = E4M3(fp32(w[m][k] / row_scale[m])); a zero row gives scale 0
 *    and zero bytes.  K % 16 == 0.
 *  wq_quantize_nvfp4: with tensor scale g (finite, > 0; g = amax / (6*448)
 *    uses the full scale range), per block of 16 k: scale byte
 *    s = E4M3(fp32(max |w| / fp32(6 g))), d = fp32(e4m3(s) * g), and
 *    code = E2M1(fp32(w / d)), all zero when d = 0; codes/scales in the
 *    layout wq_gemm_nvfp4 takes.  K % 32 == 0.
 * E4M3 and E2M1 round to nearest, ties to the even code, saturate at 448
 * and 6, and keep the sign bit (a negative value that rounds to zero gives
 * the negative-zero code).  Divisions are correctly rounded FP32.  All
 * buffers 16-byte aligned; enqueue only. */
wq_status wq_quantize_fp8row(const uint16_t* w, int M, int K, uint8_t* q, float* row_scale, void* stream);
wq_status wq_quantize_nvfp4(const uint16_t* w, int M, int K, float global_scale,
                            uint8_t* codes, uint8_t* scales, void* stream);

/* Chained MLP layers over the verify columns.  The crit-hub engine card
 * "mtp7-device-confidence" (section "Limits") traces its short-prompt
 * latency to the many small kernels each layer launches, and (section
 * "Design", row "Decode") runs a decode round as one device graph; the
 * pages give no layer equations, so the layer is a pre-norm dense MLP block
 * on the N columns of an FP32 residual stream h [N][D]:
 *     r[n] = 1 / sqrt(sum_k h[n][k]^2 / D + eps)
 *     a    = BF16(h * r * gamma)                (gamma: BF16 [D])
 *     s    = BF16(silu(a . Wg^T) * (a . Wu^T))  (Wg, Wu: NVFP4 [F][D])
 *     h   += s . Wd^T                           (Wd: NVFP4 [D][F])
 * with silu(v) = v / (1 + e^-v), BF16 rounding to nearest-even, and FP32
 * sums as in the GEMM calls.  Layers run in order, three kernels each
 * (gate/up with the RMSNorm made while staging its input and SwiGLU in its
 * epilogue; down, split in K; the residual update, which also makes the
 * next layer's sums of squares) plus one small kernel in front: no host
 * work between layers, and capture-safe once prepared.
 *
 * wq_nvfp4_tile_glu: the gate/up weights in the interleaved tiled layout
 *   the chain reads (tile t = gate rows 8t..8t+7 then up rows 8t..8t+7);
 *   gate/up codes [F][D/2] and scales [F][D/16] as wq_gemm_nvfp4 takes
 *   them, F % 8 == 0, D % 32 == 0; `tiled` holds wq_nvfp4_tiled_bytes(2F, D)
 *   bytes.  The down weights use wq_nvfp4_tile (M = D, K = F).
 * wq_mlp_layer: one layer's device buffers (HOST array of them).
 * wq_mlp_chain_prepare: checks the shapes (N 1..8, D % 32 == 0 and
 *   D <= 8704, F % 32 == 0, eps finite >= 0, all pointers non-null and
 *   16-byte aligned) and writes the descriptor table into `workspace`
 *   (>= wq_mlp_chain_workspace_bytes(layers, D, F, N) bytes, 16-byte
 *   aligned; one asynchronous host-to-device copy on `stream`), filling
 *   `plan`.  h [N][D] FP32 (in/out), a [N][D] and s [N][F] (BF16 outputs:
 *   the last layer's normalized input and gated product) are device
 *   buffers that must not overlap each other, the workspace or a weight.
 * wq_mlp_chain_launch: runs the layers (launch only; any number of times,
 *   on a stream ordered after the prepare's copy, while every buffer stays
 *   alive).  Each run updates h in place.  Results are deterministic, and
 *   running the layers in one call or one layer per call gives the same
 *   bits.  An all-zero column with eps = 0 gives NaN (0 * inf), as the
 *   formula does.
 * wq_mlp_chain_launch_persistent: the same layers, phases and bits in ONE
 *   cooperative launch (every workgroup resident), whose phases are
 *   separated by grid barriers in the workspace instead of kernel
 *   boundaries, so that each phase's first weight loads are in flight
 *   while the previous phase finishes (the card's "Decode" row: a round as
 *   one device-side program).  Returns WQ_ERROR_UNSUPPORTED_SHAPE when the
 *   device cannot keep the grid resident (plan->grid_chain == 0).  A wait
 *   that gives up (a workgroup that never arrives, which a correct launch
 *   does not produce) sets the uint32 at workspace + plan->ctl_offset + 8
 *   to nonzero instead of hanging; the outputs are then undefined and the
 *   plan must be prepared again.  Launches of one plan must not overlap.
 *   Not for stream capture. */
typedef struct wq_mlp_layer {
  const void* gate_up;    /* from wq_nvfp4_tile_glu */
  const void* down;       /* from wq_nvfp4_tile, D x F */
  const uint16_t* gamma;  /* BF16 [D] */
  float gate_scale;       /* tensor scales of Wg, Wu, Wd */
  float up_scale;
  float down_scale;
  int32_t reserved;
} wq_mlp_layer;

typedef struct wq_mlp_plan {
  void* workspace;
  size_t workspace_bytes;
  float* h;
  int32_t layers;
  int32_t D;
  int32_t F;
  int32_t N;
  int32_t grid_gate_up;
  int32_t grid_down;
  int32_t down_chunks;
  int32_t grid_chain;
  size_t ranges_gate_up_offset;
  size_t ranges_down_offset;
  size_t ssp_offset;
  size_t ctl_offset;
} wq_mlp_plan;

wq_status wq_nvfp4_tile_glu(const uint8_t* gate_codes, const uint8_t* gate_scales, const uint8_t* up_codes,
                            const uint8_t* up_scales, int F, int D, uint8_t* tiled, void* stream);
size_t wq_mlp_chain_workspace_bytes(int layers, int D, int F, int N);
/* How the chain splits the down product's K = F: chunk length and count. */
wq_status wq_mlp_chain_split(int D, int F, int* k_chunk, int* n_chunks);
wq_status wq_mlp_chain_prepare(const wq_mlp_layer* layers, int count, int D, int F, int N, float eps,
                               float* h, uint16_t* a, uint16_t* s, void* workspace, size_t workspace_bytes,
                               void* stream, wq_mlp_plan* plan);
wq_status wq_mlp_chain_launch(const wq_mlp_plan* plan, void* stream);
wq_status wq_mlp_chain_launch_persistent(const wq_mlp_plan* plan, void* stream);

/* Measurement kernels (not part of the product; they price it).  The crit
 * README's Eval turns the GPU's measured bandwidth into a floor for each
 * kernel, and the NInfer README ships a standalone bandwidth probe; these
 * are the MI355X equivalents.
 *  wq_probe_read: streams `bytes` (multiple of 16, src 16-byte aligned)
 *    with the 16-byte non-temporal loads the weight stream uses, writing one
 *    word per thread to `sink`, which must hold wq_probe_sink_words() words.
 *    One workgroup of 8 waves per CU; each wave reads its own contiguous
 *    share in whole 1 KB requests, 8 in flight.
 *  wq_probe_read_write: the same read stream, plus, every `every_kb` KB a
 *    wave reads (a multiple of 8), one 256-byte store of that wave to its own
 *    consecutive slice of `dst`, written through to memory as the verify
 *    pass writes its outputs: it prices output writes mixed into a weight
 *    stream.  `dst` must hold wq_probe_read_write_bytes(bytes, every_kb)
 *    bytes (16-byte aligned); a call writes at most that, and exactly that
 *    when the waves' shares are of equal length (bytes a multiple of 16 x
 *    the wave count, e.g. 4 GiB on 256 CUs).
 *  wq_probe_copy: copies `bytes` from src to dst (both 16-byte aligned,
 *    not overlapping): a kernel that reads and writes exactly `bytes`, for
 *    scaling hardware byte counters.
 * All only enqueue on `stream`; the read probes need a current device
 * (WQ_ERROR_DEVICE otherwise) and return WQ_ERROR_UNSUPPORTED_SHAPE when a
 * wave's share would reach 2 GiB. */
size_t wq_probe_sink_words(void);
wq_status wq_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
size_t wq_probe_read_write_bytes(size_t bytes, int every_kb);
wq_status wq_probe_read_write(const void* src, size_t bytes, void* dst, int every_kb, uint32_t* sink, void* stream);
wq_status wq_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
