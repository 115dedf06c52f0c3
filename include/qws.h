/*
 * qws.h -- C ABI of libqws: the batch-size-1 decode step of a sparse MoE model on one MI355X
 * (gfx950). Two weight streams dominate that step: the routed experts and the vocabulary LM head
 * (runbyai.xyz/posts/593 paragraph 2; Netics Labs, "Three MoE Inference Optimizations NVIDIA
 * Measured on DGX Spark", section "Decoding was memory-bound on a 124-billion-parameter model at
 * batch size 1"). This library streams both.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Buffers are DEVICE pointers the caller owns (allocated by the caller, for example as torch
 *    tensors). Descriptors are non-owning views; they must stay valid until the enqueued work ends.
 *  - Every call checks its arguments on the host first. On any error it returns a negative status
 *    and enqueues nothing. On success it enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    default stream) and returns QWS_OK without synchronising, except qws_selfcheck.
 *  - Weight and activation base pointers must be 16-byte aligned (QWS_ERR_ALIGN otherwise).
 *  - bf16 is passed as 16-bit patterns; float32 logits and outputs are IEEE binary32.
 *  - Calls are re-entrant and thread-safe; calls that share a workspace must not overlap in time.
 *  - No call allocates or frees memory.
 */
#ifndef QWS_H
#define QWS_H

#ifndef __HIPCC_RTC__   /* hipRTC (run-time compilation of the kernels) has size_t built in */
#include <stddef.h>
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define QWS_ABI_VERSION 1

typedef void* qws_stream_t; /* hipStream_t */

enum qws_status {
  QWS_OK = 0,
  QWS_ERR_ARG = -1,       /* NULL pointer where one is required, bad enum value, both outputs NULL */
  QWS_ERR_SHAPE = -2,     /* a size outside the supported range (see each call) */
  QWS_ERR_ALIGN = -3,     /* a base pointer that is not 16-byte aligned */
  QWS_ERR_FORMAT = -4,    /* a descriptor whose format tag does not match the entry point */
  QWS_ERR_WORKSPACE = -5, /* workspace NULL or smaller than the matching *_workspace_bytes() */
  QWS_ERR_DEVICE = -6,    /* the HIP runtime refused a launch; qws_strerror appends its message */
  QWS_ERR_SELFCHECK = -7, /* the device decoded a format differently from the host tables */
  QWS_ERR_COMPILE = -8    /* run-time compilation failed; qws_strerror appends the compiler log */
};

/* Format tags carried by descriptors. A descriptor tagged with one format is refused by an entry
 * point that expects another, so quantised bytes are never read as a different type: the pages
 * report that exact silent failure, FP8 head weights read as BF16 by a draft model, and advise
 * asserting the configuration at startup (posts/593 paragraph 9; Netics, section "One missing
 * interface makes the stack slower than baseline"). */
enum qws_format {
  QWS_FMT_MXFP4_E2M1_E8M0_B32 = 0x4D584634, /* e2m1 nibbles + one E8M0 scale per 32 elements */
  QWS_FMT_FP8_E4M3FN_ROWSCALE = 0x46503845, /* E4M3 (OCP "FN") codes, row-major, + one fp32 scale per row */
  QWS_FMT_BF16 = 0x42463136,                /* plain bf16 */
  QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR = 0x4D584655, /* MXFP4 experts, task-major (moe_pack_mxfp4) */
  QWS_FMT_FP8_E4M3FN_ROWSCALE_T16 = 0x46503854 /* E4M3 codes in 16-row tiles (below) + fp32 row scales */
};

/* Text for a status code. For QWS_ERR_DEVICE the text of the calling thread's last HIP error is
 * appended. The returned pointer stays valid until the next call on the same thread. */
const char* qws_strerror(int status);

/* QWS_ABI_VERSION of the loaded library. */
int qws_abi_version(void);

/* Startup validation (Netics, "One missing interface ...": validate at startup that each
 * optimisation is active rather than infer it from throughput). Decodes every e2m1 code under
 * several E8M0 scales through both device dequantisation routines, every E4M3 code, and encodes a
 * fixed set of float32 values to E4M3 on the device, then compares with tables built on the host.
 * Synchronises `stream`. Returns QWS_OK or QWS_ERR_SELFCHECK (or QWS_ERR_DEVICE). */
int qws_selfcheck(qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * MoE router: logits, top-k, renormalised softmax gate weights.
 *   logits[m, e] = sum_k x[m, k] * w_router[e, k] + bias[m, e]
 *   topk_idx[m, :] = the K largest logits, ordered by (logit descending, expert index
 *                    ascending): ties go to the lower index; -0.0 equals +0.0; NaN ranks as
 *                    -inf (below every other value; ties with -inf by index).
 *   topk_w[m, i]   = exp(l_i - l_max) / sum_j exp(l_j - l_max) over the K selected logits.
 * Each MoE layer routes a token to eight of 512 routed experts plus one shared expert
 * (posts/593 paragraph 2); the score function is not stated on the pages, softmax over the
 * selected logits is this library's reading.
 *
 *   x_bf16          [M, H] bf16, rows contiguous.            1 <= M <= 4, H % 8 == 0, 8 <= H <= 2560
 *   w_router_bf16   [E, H] bf16, row-major.                  1 <= E <= 1024
 *   bias            NULL, [E] (bias_row_stride 0) or [M, E] (bias_row_stride E), fp32.
 *   K               1 <= K <= min(8, E).
 *   topk_idx        [M, K] int32 out.  topk_w [M, K] fp32 out.
 *   logits_out      NULL or [M, E] fp32 out (the logits including bias).
 *   workspace       device memory of moe_route_workspace_bytes(M, E) bytes, ZERO-FILLED before
 *                   its first use; every call leaves it zero-filled again.
 * -------------------------------------------------------------------------------------------*/
size_t moe_route_workspace_bytes(int M, int E);
int moe_route_topk(const void* x_bf16, int M, int H, const void* w_router_bf16, int E,
                   const float* bias, long long bias_row_stride, int K, int* topk_idx,
                   float* topk_w, float* logits_out, void* workspace, size_t workspace_bytes,
                   qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * MXFP4 expert bank (non-owning view). Expert e < n_routed is a routed expert; if has_shared,
 * the shared expert is stored at index n_routed. Per expert, canonical row-major layout:
 *   gate_up_q [2I, H/2] bytes: byte j of a row holds element 2j in bits 3:0, 2j+1 in bits 7:4
 *   gate_up_s [2I, H/32] E8M0 bytes: scale of elements 32b .. 32b+31 of the row is 2^(s-127)
 *   down_q    [H, I/2],  down_s [H, I/32], same encoding.
 * gate_up rows [0, I) are the gate projection, rows [I, 2I) the up projection. Consecutive
 * experts are contiguous (expert e starts at e * rows * row_bytes). Scale bytes must be in 1..254.
 * MXFP4 is the experts' format on the pages (posts/593 paragraph 4; Netics, "Humming MXFP4
 * kernels compile at run time ..."); element and scale encodings are OCP MX v1.0.
 * -------------------------------------------------------------------------------------------*/
typedef struct {
  unsigned format; /* QWS_FMT_MXFP4_E2M1_E8M0_B32, or ..._TASKMAJOR after moe_pack_mxfp4 */
  int n_routed;    /* 1 .. 1024 */
  int has_shared;  /* 0 or 1 */
  int hidden;      /* H: multiple of 32, 32 .. 2560 */
  int inter;       /* I: multiple of 32, 32 .. 1024 */
  const unsigned char* gate_up_q;
  const unsigned char* gate_up_s;
  const unsigned char* down_q;
  const unsigned char* down_s;
} qws_mxfp4_experts;

/* ------------------------------------------------------------------------------------------
 * Routed-expert FFN with the expert union of a verification window (posts/593 paragraph 5:
 * verifying four positions can touch up to 32 experts; each expert is read once for all of
 * them):
 *   y[m] = shared(x[m]) + sum_i topk_w[m, i] * expert_{topk_idx[m, i]}(x[m])
 *   expert(x) = W_down . (silu(W_gate . x) * (W_up . x)),  silu(g) = g / (1 + e^-g)
 * float32 accumulation throughout; the SwiGLU activation stays float32.
 *
 *   x_bf16       [M, H] bf16.  1 <= M <= 4.
 *   topk_idx     [M, K] int32, topk_w [M, K] fp32 (device-resident, e.g. from moe_route_topk).
 *                1 <= K <= 8. A token holding an id outside [0, n_routed) gets a NaN row.
 *                A token listing an expert twice adds both weights.
 *   y_bf16       NULL or [M, H] bf16 out: round-to-nearest-even of y_f32.
 *   y_f32        NULL or [M, H] fp32 out. At least one of y_bf16, y_f32 must be given.
 *   workspace    moe_expert_workspace_bytes(M, K, H, I) bytes, ZERO-FILLED before first use;
 *                every call leaves its counters zero again.
 * -------------------------------------------------------------------------------------------*/
size_t moe_expert_workspace_bytes(int M, int K, int hidden, int inter);
int moe_expert_gemv_mxfp4(const qws_mxfp4_experts* w, const void* x_bf16, int M,
                          const int* topk_idx, const float* topk_w, int K, void* y_bf16,
                          float* y_f32, void* workspace, size_t workspace_bytes,
                          qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Task-major copy of an MXFP4 bank for the fused entry points (a one-off conversion at load
 * time, like lmhead_quantize_fp8; the codes and scales are moved, never changed). The fused layer
 * splits each expert's FFN into tasks of 32 activations: task (e, j) needs gate rows 32j .. 32j+31,
 * up rows I+32j .. I+32j+31 and columns 32j .. 32j+31 of every down-projection row. The copy stores
 * each task as one record of QWS_TASK_BYTES bytes, in the order in which the 16 waves x 64 lanes
 * of a workgroup read it, so that every load instruction of a wave reads 1 KB of consecutive
 * bytes:
 *   out[(e * I/32 + j) * QWS_TASK_BYTES + ((p * 16 + w) * 64 + l) * 16 + b],  p < 8 pieces,
 * with w = 4 rg + ks, l = 16 g + i:
 * The down projection is cut into the 16-row tiles q = 0 .. 9 of each wave: tile q of wave w is
 * down rows 16 (w + 16 q) .. +15, and "row i of tile q" means those rows' 16 bytes (32 codes) in
 * columns 32j .. 32j+31:
 *   p 0     bytes 0..7: bytes 8 (g >> 1) .. 8 (g >> 1) + 7 of row i of tile 8 + (g & 1); bytes
 *           8..12: the scales of the five gate/up chunks of p 1..5; byte 13 + Q, Q < 3: the
 *           scale of row i of tile 4 Q + g in block j (zero for 4 Q + g > 9);
 *   p 1..5  gate/up codes: row i of row group rg (gate 32j + 16 rg + i for rg < 2, else up
 *           I + 32j + 16 (rg - 2) + i), 16-byte chunk 20 ks + 4 (p - 1) + g of the row;
 *   p 6, 7  row i of tile 4 (p - 6) + g.
 * Chunks, rows and scales past H are zero. n = n_routed + has_shared; H <= 2560 (16 x 5 x 32
 * elements per row), I a multiple of 32. desc_out receives `src` with format
 * QWS_FMT_MXFP4_E2M1_E8M0_B32_TASKMAJOR, gate_up_q = out and the other three pointers NULL.
 * src must be canonical (QWS_ERR_FORMAT otherwise); out 16-byte aligned, out_bytes at least
 * moe_pack_mxfp4_bytes(n, H, I), not overlapping the bank.
 * -------------------------------------------------------------------------------------------*/
#define QWS_TASK_BYTES 131072
size_t moe_pack_mxfp4_bytes(int n_experts, int hidden, int inter); /* 0 for an unsupported shape */
int moe_pack_mxfp4(const qws_mxfp4_experts* src, unsigned char* out, size_t out_bytes, qws_mxfp4_experts* desc_out,
                   qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * One MoE layer in ONE launch: router GEMV, top-K, softmax, expert union, MXFP4 gate_up + SwiGLU,
 * MXFP4 down + gate-weighted combine with the shared expert -- the same arithmetic as
 * moe_route_topk followed by moe_expert_gemv_mxfp4, without the kernel boundaries between them
 * (each costs ~1.7 us on MI355X, a third of a layer's streaming time at M = 1). The grid is one
 * persistent workgroup per compute unit. Its hand-offs are 64-bit words that carry a 32-bit value
 * with a tag unique to (launch, layer, kind), so a reader polls the data itself. Experts must be
 * packed by moe_pack_mxfp4 (QWS_ERR_FORMAT otherwise). The expert products run on the matrix
 * cores: gate/up on the scaled FP4 x FP8 instruction, the e2m1 codes and E8M0 scales as stored
 * against x written as two E4M3 parts per element with one E8M0 scale per 32 (exact for every
 * element within 2^13 of its block's largest magnitude, smaller ones rounded at 2^-16 of it);
 * down on the same instruction with the formats swapped, the codes as stored against the fp32
 * SwiGLU activation written as four E4M3 parts per element (the next four significant bits each,
 * the last rounded; one E8M0 scale per part and 32 activations: the sum is the activation to
 * ~2^-16 of its block's largest). The instruction's internal accumulation is a little coarser
 * than float32 (about 1e-4 of one op's largest output, measured), so results agree with
 * moe_expert_gemv_mxfp4 to ~1e-5 of max|y|, not bit for bit; the order is fixed, so repeated
 * launches agree bit for bit. Non-finite activations are not supported.
 * -------------------------------------------------------------------------------------------*/
typedef struct {
  const void* x_bf16;         /* [M, H] bf16, ready before the launch                               */
  const void* w_router_bf16;  /* [E, H] bf16, E = experts.n_routed                                  */
  const float* bias;          /* NULL, [E] (bias_row_stride 0) or [M, E] (bias_row_stride E)         */
  long long bias_row_stride;
  qws_mxfp4_experts experts;  /* the layer's bank; shapes must be equal across the layers of a call */
  int* topk_idx;              /* NULL or [M, K] int32 out                                            */
  float* topk_w;              /* NULL or [M, K] fp32 out                                             */
  float* logits_out;          /* NULL or [M, E] fp32 out                                             */
  void* y_bf16;               /* NULL or [M, H] bf16 out (RNE of y_f32)                              */
  float* y_f32;               /* NULL or [M, H] fp32 out; at least one of y_bf16, y_f32             */
} qws_moe_layer;

/* Workspace for moe_layer_mxfp4 / moe_layers_mxfp4: ZERO-FILLED before its first use and then
 * reused as is (counters only increase and tags change per launch; nothing needs resetting, so a
 * launch may be captured in a HIP graph and replayed; every 2^20 launches the kernel clears the
 * tagged words itself before the tags repeat). One workspace per device and stream; calls sharing
 * it must not overlap in time. E <= 1024, H <= 2560, I <= 1024, K <= 8, M <= 4. The size covers
 * grids of up to 512 compute units. */
size_t moe_layer_workspace_bytes(int M, int K, int E, int hidden, int inter);

/* One layer; `layer` is host memory. Same contract as the two-call path above. */
int moe_layer_mxfp4(const qws_moe_layer* layer, int M, int K, void* workspace, size_t workspace_bytes,
                    qws_stream_t stream);

/* n_layers (<= 1024) layers in stream order in one launch: layer l+1 starts its x-dependent work
 * only after layer l's output is written. layers_host (host memory) is validated; layers_device
 * must be an identical copy in device memory (read by the kernel for layers 1 .. n_layers-1).
 * When every layer's x_bf16 is the previous layer's y_bf16 (a decode step's chain), layer l+1
 * reads its x from tagged copies that layer l's row owners publish, with no barrier between the
 * layers; otherwise the layers are separated by a grid barrier. The results are the same. Weight
 * loads that do not depend on x (router rows, the shared expert) are issued before x is ready. */
int moe_layers_mxfp4(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                     int M, int K, void* workspace, size_t workspace_bytes, qws_stream_t stream);

/* W4A8 variants of the two calls above: MXFP4 weights x MXFP8 activations (the baseline's W4A8
 * recipe: Netics Labs, "Three MoE Inference Optimizations NVIDIA Measured on DGX Spark", section on
 * the Humming MXFP4 kernels; the pages give no activation format, and the one used is MXFP8 from
 * the same OCP Microscaling family as the weights). Same arguments, validation, workspace, errors
 * and outputs as moe_layer_mxfp4 / moe_layers_mxfp4 on the same task-major banks; only the
 * arithmetic of the experts differs: x is quantised per token and per 32 elements to E4M3 codes
 * with one E8M0 scale 2^(floor(log2 max|x|) - 8) (OCP MX v1.0 conversion: nearest E4M3 value,
 * ties to even, magnitudes past 448 clamped; scale exponent at least -127), the gate/up products
 * run on the scaled FP4 x FP8 instruction, and each expert's SwiGLU output a (float32) is
 * quantised the same way in blocks of 32 along the intermediate dimension (the down weights' MX
 * blocks) before the down products, which also run on that instruction. Router, top-K, gate
 * weights, combine and the shared expert are those of the bf16 layer. An element of a that lies
 * within float32 rounding of an E4M3 rounding point may round differently than in an exact
 * computation. */
int moe_layer_w4a8(const qws_moe_layer* layer, int M, int K, void* workspace, size_t workspace_bytes,
                   qws_stream_t stream);
int moe_layers_w4a8(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers,
                    int M, int K, void* workspace, size_t workspace_bytes, qws_stream_t stream);

/* Timeouts of bounded in-kernel waits so far in this workspace: a count that only increases (0
 * when healthy). A wait times out only if the grid was not co-resident; the launch it belongs to
 * then ends all of its waits and its outputs are not valid. Later launches are not affected: they
 * wait normally and add to the count only for their own timeouts, so a count that is unchanged
 * across a launch means that launch's outputs are valid. Synchronises `stream`; errors_out is host
 * memory. */
int moe_workspace_errors(const void* workspace, int M, int K, int E, int inter, unsigned* errors_out,
                         qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Vocabulary LM head (non-owning view). The head projects H = 2,560 onto 157,184 tokens and
 * every generated token reads all of it: ~805 MB per token in bf16, half in FP8 (posts/593
 * paragraph 3).
 *   format QWS_FMT_BF16:                    w = bf16 [rows, cols], row_scale NULL.
 *   format QWS_FMT_FP8_E4M3FN_ROWSCALE_T16: w = E4M3 codes u8, tile-major (below), row_scale fp32
 *                                           [rows]; weight[r, k] = e4m3(q[r, k]) * row_scale[r].
 *   format QWS_FMT_FP8_E4M3FN_ROWSCALE:     the same codes row-major, w = u8 [rows, cols]. The FP8
 *                                           GEMVs read only tile-major codes and refuse this tag
 *                                           (QWS_ERR_FORMAT): lmhead_fp8_tile_major converts.
 * rows >= 1; cols multiple of 32, 32 .. 2560.
 * Tile-major FP8 codes (lmhead_fp8_codes_bytes(rows, cols) bytes): the rows in tiles of 16, the
 * last one padded with zero-code rows; tile t starts at byte 16 t cols; inside it, the 16 codes
 * q[16 t + i, 16 c .. 16 c + 15] (chunk c of tile row i) are at byte 16 (16 c + i). A wave of the
 * GEMV then reads 1 KB of consecutive bytes per load instruction: 4 chunks of 16 rows, the
 * operand of one matrix-core product each. The layout is part of the tag, so row-major codes are
 * never read as tiles (the pages' silent failure is a head read in the wrong format: posts/593
 * paragraph 9).
 * -------------------------------------------------------------------------------------------*/
typedef struct {
  unsigned format;
  long long rows;
  long long cols;
  const void* w;
  const float* row_scale;
} qws_lmhead;

/* Fill a bf16 head descriptor (no device work). */
int lmhead_bf16_desc(const void* w_bf16, long long rows, long long cols, qws_lmhead* desc_out);

/* Online FP8 quantisation of a bf16 head, done once when the head is constructed (Netics,
 * "Online FP8 quantization halves the LM head weight reads"):
 *   s_r = fl32(max_k |W[r, k]| / 448)  (s_r = 1 for an all-zero row)
 *   q[r, k] = E4M3(fl32(W[r, k] / s_r)), round to nearest even, saturating at +-448
 * Both divisions are IEEE float32 round-to-nearest-even.
 *   w_bf16 [rows, cols] in; codes_out u8, lmhead_fp8_codes_bytes(rows, cols) bytes (tile-major,
 *   pad rows written as zero codes) and row_scale_out fp32 [rows] out, all device memory owned by
 *   the caller. desc_out (host memory) is filled with a QWS_FMT_FP8_E4M3FN_ROWSCALE_T16
 *   descriptor of the outputs.
 * Errors: QWS_ERR_ARG for a missing pointer, QWS_ERR_SHAPE for rows or cols out of range,
 * QWS_ERR_ALIGN for w_bf16 or codes_out not 16-byte aligned.                                 */
int lmhead_quantize_fp8(const void* w_bf16, long long rows, long long cols,
                        unsigned char* codes_out, float* row_scale_out, qws_lmhead* desc_out,
                        qws_stream_t stream);

/* Bytes of the tile-major FP8 codes of a rows x cols head: ceil(rows / 16) * 16 * cols; 0 for
 * rows or cols out of range. */
size_t lmhead_fp8_codes_bytes(long long rows, long long cols);

/* Tile-major copy of a head whose E4M3 codes are row-major (for example quantised elsewhere): the
 * codes are moved into the layout above (pad rows zero), never changed. src must be tagged
 * QWS_FMT_FP8_E4M3FN_ROWSCALE (QWS_ERR_FORMAT otherwise), with row_scale set; codes_out holds
 * codes_bytes >= lmhead_fp8_codes_bytes(rows, cols) bytes of device memory, 16-byte aligned and
 * not overlapping src->w (QWS_ERR_WORKSPACE, QWS_ERR_ALIGN, QWS_ERR_ARG otherwise). desc_out
 * (host memory) receives a QWS_FMT_FP8_E4M3FN_ROWSCALE_T16 descriptor of codes_out with src's
 * row_scale pointer. */
int lmhead_fp8_tile_major(const qws_lmhead* src, unsigned char* codes_out, size_t codes_bytes,
                          qws_lmhead* desc_out, qws_stream_t stream);

/* logits[m, r] = row_scale[r] * sum_k e4m3(q[r, k]) * x[m, k]   (head must be tagged
 * QWS_FMT_FP8_E4M3FN_ROWSCALE_T16; QWS_ERR_FORMAT for any other tag, row-major FP8 included)
 *   x_bf16 [M, cols], 1 <= M <= 4; logits_out fp32 [M, rows]. Each token gets the same logits,
 *   bit for bit, whatever M and its place in the window.                                    */
int lmhead_gemv_fp8(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                    qws_stream_t stream);

/* Greedy verification of a speculative window after the FP8 head. The configuration drafts
 * three tokens and verifies a four-position window at once, accepting the correct prefix
 * (runbyai.xyz/signal/190, the paragraph on speculative decoding; Netics post, "Speculative
 * decoding reduces the number of steps"); greedy decoding is the pages' synthetic run.
 *   x_bf16 [M, cols], 1 <= M <= 4 (the window's positions); draft [M - 1] int32 (NULL allowed
 *   when M = 1); logits_out NULL or fp32 [M, rows] (the same values as lmhead_gemv_fp8);
 *   target_out [M]: each position's argmax (ties to the lower row; NaN below every number);
 *   emitted_out [M] and n_out [1]: draft i (i < M - 1) is accepted while it equals target i, then
 *   the target of the first position not accepted: emitted[0 .. n) with n in 1 .. M, emitted[i]
 *   = -1 for i >= n. All of these are device memory owned by the caller.
 *   workspace: lmhead_verify_workspace_bytes(M) bytes, 16-byte aligned, zero-filled before its
 *   first use and left ready for the next call; calls that share it must not overlap.
 * Two launches: the head GEMV (logits, and each workgroup's largest key per position), then one
 * workgroup that reduces the keys and forms the window.
 * Errors: QWS_ERR_FORMAT for a head not tagged QWS_FMT_FP8_E4M3FN_ROWSCALE_T16, QWS_ERR_ARG for a missing pointer,
 * QWS_ERR_SHAPE for M outside 1 .. 4, QWS_ERR_WORKSPACE / QWS_ERR_ALIGN as elsewhere. */
size_t lmhead_verify_workspace_bytes(int M);
int lmhead_verify_greedy_fp8(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                             float* logits_out, int* target_out, int* emitted_out, int* n_out,
                             void* workspace, size_t workspace_bytes, qws_stream_t stream);

/* lmhead_verify_greedy_fp8 without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The same two launches and results; the head workgroups' keys go to a 64 KB device array of the
 * library instead (one per GPU, held until the process ends; its device address is looked up on
 * the first call on each device). No call allocates or frees memory. Every call on one GPU shares
 * that array: calls that overlap in time on one GPU (other streams, other threads) race and must
 * be serialised by the caller. Nothing in it needs clearing: each call writes every key it reads.
 * Errors: as lmhead_verify_greedy_fp8 (a window of more than 4 positions, which the array could
 * not hold, is QWS_ERR_SHAPE), plus QWS_ERR_DEVICE if the array's address cannot be found. */
int lmhead_verify_greedy_fp8_noalloc(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                                     float* logits_out, int* target_out, int* emitted_out, int* n_out,
                                     qws_stream_t stream);

/* Sampled verification of a speculative window after the FP8 head, for the pages' sampled run
 * (temperature 0.6, top_p 0.95, top_k 29: Netics post, "GSM8K measured a 42.5% throughput gain").
 * Per position m: the logits divided by the temperature, the top_k largest (ties to the lower row;
 * NaN below every number), their softmax, the shortest prefix of that order whose probability
 * reaches top_p, and token[m] = the first of that prefix whose running probability exceeds
 * u[m] times the prefix's total (the last of it when none does). Draft i is accepted while it
 * equals token[i]; emitted / n as for lmhead_verify_greedy_fp8. (The pages give no acceptance rule
 * for sampled drafts and no draft probabilities, so a draft counts when it is the token the target
 * samples with the caller's uniform; u[m] is drawn by the caller, in [0, 1).)
 *   x_bf16 [M, cols], 1 <= M <= 4; draft [M - 1] int32 (NULL allowed when M = 1);
 *   temperature > 0, finite; 1 <= top_k <= 32; 0 < top_p <= 1; u fp32 [M] (device);
 *   logits_out fp32 [M, rows] (required: the same values as lmhead_gemv_fp8); token_out int32 [M];
 *   topk_out NULL or int32 [M, top_k]: the rows of the top_k in order (-1 past min(top_k, rows));
 *   emitted_out int32 [M], n_out int32 [1]; all device memory owned by the caller.
 *   workspace: lmhead_verify_workspace_bytes(M) bytes, shared with lmhead_verify_greedy_fp8 (the
 *   same conditions: zero-filled before first use, calls that share it must not overlap).
 * Two launches: the head GEMV (logits and each head workgroup's four largest keys per position),
 * then one workgroup per position.
 * Errors: as lmhead_verify_greedy_fp8, plus QWS_ERR_ARG for u or logits_out missing, temperature or
 * top_p out of range, QWS_ERR_SHAPE for top_k outside 1 .. 32 or more than 262,144 rows. */
int lmhead_verify_sample_fp8(const qws_lmhead* head, const void* x_bf16, int M, const int* draft,
                             float temperature, int top_k, float top_p, const float* u,
                             float* logits_out, int* token_out, int* topk_out, int* emitted_out,
                             int* n_out, void* workspace, size_t workspace_bytes, qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Run-time specialisation (hipRTC). The pages' first optimisation compiles kernels at run time
 * for the real shapes, data types and architecture and caches them on disk, so that a kernel
 * builds in seconds (runbyai.xyz/posts/593 paragraph 4; Netics post, "Humming MXFP4 kernels
 * compile at run time for the model's real shapes"). Here: the FP8 head GEMV, compiled from the
 * same source as lmhead_gemv_fp8 with rows and cols as constants, for the current device's
 * architecture (gcnArchName) and M; and the fused MoE layers with the layer shape as constants.
 * Key: the kernel and its constants, the architecture, a hash of the sources, and a digest of the
 * compile options and the hipRTC version. The disk cache is `cache_dir` (NULL: $QWS_RTC_CACHE,
 * else $XDG_CACHE_HOME/qws_rtc, else $HOME/.cache/qws_rtc; none of these set: no disk cache),
 * created with mode 0700 and used only while it is a directory owned by the calling user that no
 * one else may write; one file per key, written to a fresh temporary file (mkstemp) and renamed,
 * so that concurrent processes never read half a file; a file is read only if it is a regular file
 * owned by the user (not followed through a link) whose stored code hash matches. Any failed check
 * means a compile instead.
 * -------------------------------------------------------------------------------------------*/
typedef struct {
  unsigned long long compiles;    /* hipRTC compilations */
  unsigned long long disk_hits;   /* code objects read from the disk cache */
  unsigned long long memory_hits; /* launches that found their module already loaded */
  double compile_ms;              /* wall time spent compiling (and writing the cache) */
  double load_ms;                 /* wall time spent reading cache files and loading modules */
} qws_rtc_stats;

/* Same result as lmhead_gemv_fp8, bit for bit (same source, same arithmetic); the first call for a
 * key compiles or reads the cache, later calls launch the loaded module. Errors: as
 * lmhead_gemv_fp8, plus QWS_ERR_COMPILE (compiler log in qws_strerror) and QWS_ERR_DEVICE for a
 * module that does not load. Thread-safe (one lock around the cache). */
int lmhead_gemv_fp8_rtc(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                        const char* cache_dir, qws_stream_t stream);
/* Compile (or find in the disk cache) the GEMV for an architecture name such as "gfx950" or
 * "gfx950:sramecc+:xnack-", without a device: for building a cache ahead of time. QWS_ERR_ARG for an
 * arch name not of that form, QWS_ERR_SHAPE as lmhead_gemv_fp8, QWS_ERR_COMPILE (e.g. an
 * architecture without the gfx950 conversions the kernel uses). */
int qws_rtc_compile_head_fp8(int M, long long rows, long long cols, const char* arch, const char* cache_dir);
/* The fused MoE layers (moe_layers_mxfp4, or moe_layers_w4a8 when w4a8 = 1) compiled at run time
 * for the layers' shape: the same kernel source with E, K, hidden, inter and the shared expert as
 * constants and M, the precision and the kind of sequence (chained or not) as template arguments,
 * for the current device's architecture. Key: (M, precision, E, hidden, inter, K, shared, chained,
 * architecture, source hash, options and hipRTC version). Same arguments, validation, workspace and results as the template entry
 * points, bit for bit; QWS_ERR_ARG for w4a8 outside {0, 1}, plus the errors of
 * lmhead_gemv_fp8_rtc. A compile takes seconds: the first call for a key blocks the calling
 * thread until it is done (qws_rtc_compile_moe builds the cache ahead of time). */
int moe_layers_rtc(const qws_moe_layer* layers_host, const qws_moe_layer* layers_device, int n_layers, int M,
                   int K, int w4a8, void* workspace, size_t workspace_bytes, const char* cache_dir,
                   qws_stream_t stream);
/* Compile (or find in the disk cache) the fused MoE kernels for a shape and an architecture name,
 * without a device: the kernel for separate layers and the one for chained sequences. QWS_ERR_ARG
 * for a bad arch name or w4a8 outside {0, 1}; QWS_ERR_SHAPE for M, K, E, hidden, inter or
 * has_shared outside the ranges of moe_layer_mxfp4. */
int qws_rtc_compile_moe(int M, int K, int E, int hidden, int inter, int has_shared, int w4a8, const char* arch,
                        const char* cache_dir);
/* Counters since load or the last qws_rtc_reset (stats_out: host memory). */
int qws_rtc_stats_get(qws_rtc_stats* stats_out);
/* Unload the modules and zero the counters; the disk cache is kept. */
int qws_rtc_reset(void);

/* logits[m, r] = sum_k W[r, k] * x[m, k]   (head must be BF16-tagged; an FP8 head is refused
 * with QWS_ERR_FORMAT instead of being read as bf16). Same shapes as lmhead_gemv_fp8.       */
int lmhead_gemv_bf16(const qws_lmhead* head, const void* x_bf16, int M, float* logits_out,
                     qws_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Diagnostics (not on the hot path)
 * -------------------------------------------------------------------------------------------*/
/* Dequantise an MXFP4 matrix [rows, cols] (canonical layout above) into fp32 out [rows, cols]
 * with the device routine of the down projection (path 0: e2m1 -> fp32 with the block scale)
 * or of the gate/up projection (path 1: e2m1 -> bf16 with the block scale, widened to fp32).
 * cols multiple of 32, 32 .. 65536. Exact for scale bytes 2 .. 252.                        */
int qws_debug_dequant_mxfp4(const unsigned char* q, const unsigned char* s, long long rows,
                            int cols, int path, float* out, qws_stream_t stream);

/* out[r, k] = fl32(e4m3(q[r, k]) * row_scale[r]) for a QWS_FMT_FP8_E4M3FN_ROWSCALE_T16 head,
 * fp32 [rows, cols] row-major.                                                              */
int qws_debug_dequant_fp8(const qws_lmhead* head, float* out, qws_stream_t stream);

/* Tracing of the fused MoE launches on the current device: while `buf` is registered (device
 * memory, 16-byte aligned), every moe_layer_mxfp4 / moe_layers_mxfp4 launch whose trace fits in
 * `bytes` writes, per layer and workgroup, 16 timestamps of the device wall clock (100 MHz,
 * uint64): [0] layer start, [1] x staged, [2] router rows done, [3] shared-expert task done,
 * [4] logits received, [10] selection threshold found, [11] candidates above it compacted,
 * [12] candidate ranks done, [5] selection and union done, [15] the last task's record has
 * arrived (thread 0; taking it makes wave 0 wait there), [6] routed tasks done, [7] partial
 * sums received (row owners), [13] row sums done, [8] output written, [14] layer-end stores
 * acknowledged, [9] layer barrier passed (sequences that are not chained); layout [n_layers][grid][16]. NULL unregisters.
 * Diagnostics only. */
int qws_debug_trace_buffer(void* buf, size_t bytes);

/* Activations of the W4A8 layer on the current device: while `buf` is registered (device memory,
 * 16-byte aligned), every moe_layer_w4a8 launch (one layer) whose record fits in `bytes` writes,
 * for each (expert e, token m) it computes (e = E: the shared expert), the float32 SwiGLU output
 * a[e][m][k] (k < I) at float offset (e * M + m) * I + k, its E4M3 code at byte offset
 * (E+1) * M * I * 4 + (e * M + m) * I + k and the block's E8M0 scale byte at byte offset
 * (E+1) * M * I * 5 + ((e * M + m) * I + k) / 32; needs (E+1) * M * I * 5 + (E+1) * M * I / 32 bytes.
 * Entries of experts the launch does not run are left as they were. NULL unregisters.
 * Diagnostics only (the parity test compares these with the oracle's). */
int qws_debug_w4a8_act_buffer(void* buf, size_t bytes);

/* Streaming-read probe: reads `bytes` (multiple of 16, 16-byte aligned) with 128-bit loads and
 * writes one checksum word per workgroup into sink[0 .. blocks) (blocks <= 65536). Measures the
 * device's practical read bandwidth.                                                        */
int qws_probe_read(const void* buf, size_t bytes, unsigned* sink, int blocks, qws_stream_t stream);

/* Non-temporal streaming-read probe: same arguments and errors as qws_probe_read. Workgroup b
 * reads its own contiguous share (bytes / blocks, rounded up to 16-byte words; the last share
 * ends at the buffer's end) with non-temporal 128-bit loads and writes the XOR of the share's
 * 32-bit words into sink[b] (0 for an empty share). The faster streaming shape; its lines are not
 * kept in the caches, so unlike qws_probe_read it is no cache flush.                          */
int qws_probe_read_nt(const void* buf, size_t bytes, unsigned* sink, int blocks, qws_stream_t stream);

/* Copy probe: copies `bytes` (multiple of 16; both buffers 16-byte aligned, not overlapping) from
 * `src` to `dst` with 128-bit loads and stores, grid-strided over `blocks` workgroups (<= 65536).
 * A kernel of known traffic (reads and writes `bytes` each) against which HBM traffic counters
 * are scaled.                                                                                 */
int qws_probe_copy(const void* src, void* dst, size_t bytes, int blocks, qws_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QWS_H */
