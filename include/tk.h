/*
 * tk.h -- C ABI of the fused SwiGLU + MoE top-k weight + FP8/FP4 cast for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (one launch, one HBM read of the input, one HBM write of the
 * output) follows DeepSeek's TileKernels kernel
 * swiglu_forward_and_per_token_cast as described in
 *   "【DeepSeek】TileKernels从入门到精通" (zhichai.net/topic/177618752),
 *   ch.2 "解剖麻雀（SwiGLU与Quant的单次Kernel融合）":
 *     - "内存的“连体双胞胎”：布局的艺术": the input is one packed bf16 tensor
 *       [num_expanded_tokens, 2*hidden]; gate = left half, up = right half
 *       at column offset hidden;
 *     - "算子融合的“三重境界”": sigmoid(gate)*gate, times up, times the
 *       row's top-k routing weight, then the abs-max of the result gives the
 *       scale factor and the values are cast to FP8 in registers;
 *     - "守门员 Clamp": optional clamp of the gate against a limit, with an
 *       atomically accumulated count of clamped values;
 *   and "TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式"
 *   (zhichai.net/topic/177618740), "3. Quantization": FP8 E4M3 per-token or
 *   per-block, FP4 E2M1, and UE8M0 (power-of-two) scale factors.
 *
 * Per row r (j < hidden, g = x[r, j], u = x[r, hidden + j], both bf16):
 *   clamp (if clamp_limit is finite): count g > L; g = min(g, L);
 *                                     u = min(max(u, -L), L)
 *   a = RN(g * sigma(g))   sigma(g) = 1/(1+e^-g), correctly rounded to fp32
 *   b = RN(a * u);  y = RN(b * topk_weight[r])   (fp32, no fused multiply-add)
 *   per group of G consecutive columns (G = hidden when group_size == 0):
 *     amax = max |y|
 *     TK_SCALE_FP32 : scale = RN(amax / fmt_max), inv = min(RN(fmt_max/amax), FLT_MAX)
 *     TK_SCALE_UE8M0: k = smallest integer with fmt_max * 2^k >= amax
 *                     (at least -127); scale byte = k + 127, inv = 2^-k
 *     code = cast(RN(y * inv)), round to nearest even, saturating
 *   fmt_max = 448 (FP8 E4M3, OCP "FN" encoding) or 6 (FP4 E2M1).
 *   Dequantisation is code * scale (scale = 2^(byte-127) for UE8M0).
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is DEVICE memory owned by the caller.  The library
 *    allocates nothing per call; it keeps per device a CU count and a
 *    32 KiB sigmoid table in static device memory, set up by tk_init or by
 *    the first call on that device.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and return after the launch is enqueued.
 *  - Outputs must not overlap inputs.
 *  - n == 0 (tokens == 0) returns TK_OK and launches nothing; the one
 *    exception is tk_topk_to_pos, which still writes its all-zero offsets.
 *  - Errors are returned, never thrown; on any error nothing is launched
 *    except for TK_ERR_HIP, which reports a failed launch or device query.
 *  - Inputs are expected to be finite.  A NaN or infinite input gives codes
 *    and scales the ABI does not specify; in particular, with the clamp on a
 *    NaN gate or up value comes out as a finite clamped value (the clamp is a
 *    min / max that does not propagate NaN), so it does not show in the codes.
 */
#ifndef TK_H_
#define TK_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Scale format and layout.  n = rows, G = groups per row (hidden / group size,
 * 1 per-token).  The column-major and packed layouts are the "TMA-aligned
 * column-major" scale storage and the "UE8M0 packed" scale compression named in
 * "TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式" "3. Quantization", laid out
 * for a GEMM that reads one group's scales for consecutive rows:
 *   TK_SCALE_FP32            fp32  [n][G] row-major
 *   TK_SCALE_UE8M0           uint8 [n][G] row-major
 *   TK_SCALE_FP32_COLMAJOR   fp32  [G][ld], ld = n rounded up to 4; element (r, k) at k*ld + r
 *   TK_SCALE_UE8M0_COLMAJOR  uint8 [G][ld], ld = n rounded up to 16; element (r, k) at k*ld + r
 *   TK_SCALE_UE8M0_PACKED    uint32 [ceil(G/4)][ld], ld = n rounded up to 4; word (j, r) holds the
 *                            bytes of groups 4j..4j+3 of row r, group 4j in the low byte
 * Column-major and packed buffers must be 16-byte aligned; rows r >= n of a
 * column and bytes of groups k >= G of the last packed word are not written.
 */
typedef enum {
    TK_SCALE_FP32 = 0,
    TK_SCALE_UE8M0 = 1,
    TK_SCALE_FP32_COLMAJOR = 2,
    TK_SCALE_UE8M0_COLMAJOR = 3,
    TK_SCALE_UE8M0_PACKED = 4
} tk_scale_fmt;

typedef enum {
    TK_DTYPE_BF16 = 0,  /* bf16 elements (2 bytes) */
    TK_DTYPE_FP32 = 1   /* fp32 elements (4 bytes) */
} tk_dtype;

typedef enum {
    TK_OK = 0,
    TK_ERR_INVALID_ARG = 1, /* a documented precondition does not hold */
    TK_ERR_UNSUPPORTED = 2, /* valid request outside the shapes the kernels cover */
    TK_ERR_HIP = 3          /* HIP runtime error (launch, device query) */
} tk_status;

/*
 * tk_init: one-time set-up of `device` (its CU count and the sigmoid table).
 * The first tk_swiglu_cast_* call on a device does this itself and blocks
 * until it is finished; call tk_init beforehand to take that cost out of the
 * first call (required before capturing calls into a HIP graph).
 * Thread-safe.  The caller's current device is left unchanged.
 * Errors: TK_ERR_INVALID_ARG for a device index out of range, TK_ERR_HIP.
 */
tk_status tk_init(int device);

/*
 * tk_swiglu_cast_fp8: the fused step with FP8 E4M3 codes.
 *
 *  x             bf16 [n, 2*hidden], row-major; columns [0, hidden) are the
 *                gate, [hidden, 2*hidden) the up projection.  16-byte aligned.
 *  topk_weight   fp32 [n], the routing weight of each expanded row, 4-byte
 *                aligned; NULL means weight 1 (the last product is skipped).
 *  n             rows (num_expanded_tokens), 0 <= n < 2^31.
 *  hidden        columns per half; > 0 and a multiple of 8.
 *  group_size    0 = one scale per row (per-token); otherwise the width of a
 *                column group with its own scale: a multiple of 8 dividing
 *                hidden.
 *  clamp_limit   L > 0; +INFINITY disables the clamp (the count is then 0).
 *  scale_fmt     a tk_scale_fmt value (value kind and layout).
 *  codes         uint8 [n, hidden], E4M3 codes, 8-byte aligned.
 *  scales        one scale per group in the tk_scale_fmt layout (G = 1 when
 *                group_size == 0): row-major fp32 (4-byte aligned) or uint8,
 *                or a 16-byte aligned column-major / packed layout.
 *  clamped_count int64 on the device, or NULL.  The number of gate values
 *                strictly above L is ADDED to it (the caller zeroes it).
 *  stream        hipStream_t to launch on.
 *
 * Returns TK_ERR_INVALID_ARG when: n < 0 or n >= 2^31; hidden <= 0 or not a
 * multiple of 8; group_size < 0, not a multiple of 8 or not dividing hidden;
 * clamp_limit is NaN or <= 0; scale_fmt is unknown; n > 0 and x, codes or
 * scales is NULL; a pointer breaks its alignment; an output overlaps an input.
 * Every group_size that is valid has a kernel: groups of 2^j * 8 columns up to
 * 512 are reduced inside one 512-column step, groups of whole steps over one
 * to four waves, other widths up to 8192 columns as runs of whole groups per
 * wave reduced through LDS, and the remaining ones (wider than 8192 columns
 * and not split evenly over 2 or 4 waves, or wider than 32768) by one wave
 * per group that reads the group twice.  TK_ERR_UNSUPPORTED is returned only
 * when the plan would need 2^31 or more units of work (n times the units per
 * row).
 */
tk_status tk_swiglu_cast_fp8(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                             int64_t group_size, float clamp_limit, tk_scale_fmt scale_fmt,
                             void* codes, void* scales, int64_t* clamped_count, void* stream);

/*
 * tk_swiglu_cast_fp4: the same step with FP4 E2M1 codes (fmt_max = 6).
 * codes is uint8 [n, hidden/2], 4-byte aligned: element 2i of a row is the
 * low nibble of byte i, element 2i+1 the high nibble; each nibble is
 * sign(1) | exponent(2) | mantissa(1).  Everything else as tk_swiglu_cast_fp8.
 */
tk_status tk_swiglu_cast_fp4(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                             int64_t group_size, float clamp_limit, tk_scale_fmt scale_fmt,
                             void* codes, void* scales, int64_t* clamped_count, void* stream);

/*
 * tk_swiglu_forward: the first stage of the same operation on its own, the
 * "swiglu_forward" of the unfused reference in "【DeepSeek】TileKernels从入门到
 * 精通" ch.5 "越过性能红线" (swiglu_forward, then cast): writes
 * y = RN(RN(RN(g*sigma(g))*u)*topk_weight) in fp32 with the same clamp and
 * counter, and no cast.  Exposes every bit of the fused kernel's activation
 * (same device code) and is the first kernel of the unfused two-pass path.
 *
 *  y  fp32 [n, hidden], row-major, 16-byte aligned, caller-owned device memory.
 *  Other arguments, conventions and errors as tk_swiglu_cast_fp8 (there is no
 *  group, format or scale, so TK_ERR_UNSUPPORTED never occurs).
 */
tk_status tk_swiglu_forward(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                            float clamp_limit, float* y, int64_t* clamped_count, void* stream);

/*
 * tk_cast_fp8: the stand-alone cast of rows to FP8 E4M3 codes with per-token
 * or per-block scales -- TileKernels' per_token_cast ("【DeepSeek】TileKernels从
 * 入门到精通" ch.1 "透视底层"/"闭环"), and the "cast" of the unfused reference in
 * ch.5 "越过性能红线".  Per row r and group of G columns:
 *   amax = max |y|; scale and inv as in tk_swiglu_cast_fp8; code = cast(RN(y*inv))
 * with y the input value (bf16 widened exactly to fp32, or fp32).  The same
 * value gets the same code and scale as on the fused path.
 *
 *  x          [n, hidden] row-major, in_dtype elements, 16-byte aligned.
 *  in_dtype   TK_DTYPE_BF16 or TK_DTYPE_FP32.
 *  n, hidden, group_size, scale_fmt, codes, scales, stream: as
 *             tk_swiglu_cast_fp8.
 * Returns TK_ERR_INVALID_ARG for the same conditions as tk_swiglu_cast_fp8
 * (without weight, clamp and counter) and for an unknown in_dtype;
 * TK_ERR_UNSUPPORTED only when the plan would need 2^31 or more units of work,
 * as for tk_swiglu_cast_fp8 (every valid group_size has a kernel).
 */
tk_status tk_cast_fp8(const void* x, tk_dtype in_dtype, int64_t n, int64_t hidden, int64_t group_size,
                      tk_scale_fmt scale_fmt, void* codes, void* scales, void* stream);

/* tk_cast_fp4: the stand-alone cast to FP4 E2M1 codes packed two per byte
 * (element 2i in the low nibble), fmt_max 6.  Otherwise as tk_cast_fp8. */
tk_status tk_cast_fp4(const void* x, tk_dtype in_dtype, int64_t n, int64_t hidden, int64_t group_size,
                      tk_scale_fmt scale_fmt, void* codes, void* scales, void* stream);

/*
 * tk_topk_gate: deterministic top-k expert selection per token -- the Gating
 * module of "TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式" ("1. Gating":
 * top-k of [num_tokens, num_experts] scores, equal scores to the smaller
 * index) with the grouped step of "【DeepSeek】TileKernels从入门到精通" ch.3
 * ("导诊台的“工号制度”": groups ranked by the sum of their two best scores,
 * equal sums to the smaller group index).
 *
 *   "a beats b": score_a > score_b, or equal scores (-0 == +0) and a < b.
 *   n_group > 1: the experts form n_group consecutive groups; a group's score
 *   is RN(best + second best) of its members; only the topk_group best groups'
 *   members are candidates.  Then k times: the best remaining candidate.
 *
 *  scores       fp32 [tokens, experts], row-major, 4-byte aligned (device);
 *               +-inf allowed, NaN not (a NaN score's rank is unspecified).
 *  tokens       0 <= tokens < 2^31.
 *  experts      1..512;  k: 1..64 and at most the number of candidates.
 *  n_group      divides experts (1 = no groups); topk_group in 1..n_group;
 *               with groups, each group has at least 2 experts.
 *  normalise    0: weights are the chosen scores; 1: each chosen score divided
 *               by the fp32 sum of the chosen scores added best first (a zero
 *               sum leaves the scores as they are).
 *  topk_idx     int32 [tokens, k] (device), best first.
 *  topk_weight  fp32 [tokens, k] (device), in the same order.
 * Returns TK_ERR_INVALID_ARG for violated preconditions, overlapping outputs or
 * misaligned pointers; TK_ERR_UNSUPPORTED when experts > 512 or k > 64, or when
 * groups cannot be laid out as blocks of 2^j whole lanes: a token takes 32
 * lanes when experts <= 256 and k <= 32, else 64, each lane C consecutive
 * experts, and some C from ceil(experts / lanes) to 8 must divide
 * experts / n_group with a power-of-two quotient (the 32-lane layout is tried
 * first).  Example: 160 experts in 8 groups take C = 5, 4 lanes per group.
 */
tk_status tk_topk_gate(const float* scores, int64_t tokens, int64_t experts, int64_t k, int64_t n_group,
                       int64_t topk_group, int normalise, int32_t* topk_idx, float* topk_weight, void* stream);

/*
 * tk_moe_reduce: the weighted top-k reduce of the experts' output rows -- the
 * fused reduce of "【DeepSeek】TileKernels从入门到精通" ch.3, sections
 * "结算中心的“减法工程”" (routing weights, quantisation scale factors and a
 * global scale applied in one pass: the expert outputs are read once and the
 * result written once) and "动态寻址" (rows found through a token/top-k ->
 * position map).
 *
 *   Per token t and column c, over the present slots j = 0..k-1 in order
 *   (slot j is present when 0 <= pos[t,j] < n_rows; any other entry, such as
 *   -1 for a dropped slot, contributes nothing and its row is never read):
 *     f   = RN(topk_weight[t,j] * row_scale[p])   (f = topk_weight[t,j] when
 *                                                  row_scale is NULL)
 *     acc = RN(acc + RN(f * x[p,c]))              from acc = +0
 *     out[t,c] = RN(acc * global_scale), then rounded to the nearest bf16
 *     (ties to even) for TK_DTYPE_BF16, or kept as fp32 for TK_DTYPE_FP32.
 *   Every operation is one IEEE fp32 operation, round to nearest even.
 *
 *  x            bf16 [n_rows, hidden], row-major, 16-byte aligned (device); may
 *               be NULL when n_rows == 0.
 *  row_scale    fp32 [n_rows] (device), 4-byte aligned, or NULL.
 *  pos          int32 [tokens, k] (device), 4-byte aligned: the row of each
 *               (token, slot), as tk_topk_to_pos builds it from top-k indices.
 *               Entries are range-checked on the device, so a bad entry drops
 *               its slot instead of reading out of bounds.
 *  topk_weight  fp32 [tokens, k] (device), 4-byte aligned.
 *  global_scale a finite fp32 factor applied once to each sum.
 *  tokens       0 <= tokens < 2^31;  k: 1..64 (k > 64: TK_ERR_UNSUPPORTED).
 *  hidden       a positive multiple of 8, at most (2^31-1)/8.
 *  n_rows       0 <= n_rows < 2^31.
 *  out_dtype    TK_DTYPE_BF16 or TK_DTYPE_FP32.
 *  out          [tokens, hidden] of out_dtype (device), 16-byte aligned; it must
 *               not overlap x, row_scale, pos or topk_weight.
 * The caller owns every buffer; the call keeps no pointer after it returns and
 * allocates nothing.  Returns TK_ERR_INVALID_ARG for violated preconditions,
 * overlapping buffers or misaligned pointers (before any HIP call), TK_OK
 * without a launch when tokens == 0, TK_ERR_HIP if the launch fails.
 */
tk_status tk_moe_reduce(const void* x, const float* row_scale, const int32_t* pos, const float* topk_weight,
                        float global_scale, int64_t tokens, int64_t k, int64_t hidden, int64_t n_rows,
                        tk_dtype out_dtype, void* out, void* stream);

/*
 * tk_topk_to_pos: the token/top-k -> expert-row map that tk_moe_reduce gathers
 * through -- the position map of "【DeepSeek】TileKernels从入门到精通" ch.3, section
 * "动态寻址".  The expanded rows are laid out as a grouped expert GEMM reads
 * them: expert 0's rows first, then expert 1's, ...; within an expert, in
 * token order.
 *
 *   Slot (t, j) is present when 0 <= e = topk_idx[t,j] < experts and no earlier
 *   slot of token t names e (a top-k never repeats an expert; a repeat, like a
 *   negative entry for a dropped slot, is absent).
 *   expert_offsets[e] = the number of present slots naming an expert below e;
 *   expert_offsets[experts] = the number of present slots (rows in all).
 *   pos[t,j] = expert_offsets[e] + the number of tokens t' < t with a present
 *   slot naming e, for a present slot; -1 otherwise.
 *
 *  topk_idx        int32 [tokens, k] (device), 4-byte aligned.
 *  tokens          0 <= tokens < 2^31, with tokens * k < 2^31.
 *  k               1..64 (k > 64: TK_ERR_UNSUPPORTED).
 *  experts         1..512 (more: TK_ERR_UNSUPPORTED).
 *  pos             int32 [tokens, k] (device), 4-byte aligned; also the call's
 *                  working storage (each block of 1024 tokens keeps its
 *                  per-expert counts there until it writes its rows).
 *  expert_offsets  int32 [experts + 1] (device), 4-byte aligned; also working
 *                  storage during the call.  All zero when tokens == 0.
 * The three buffers must not overlap.  Three kernel launches on `stream`
 * (one when tokens == 0); the call keeps no pointer after it returns and
 * allocates nothing.  Returns TK_ERR_INVALID_ARG for violated preconditions,
 * overlapping buffers or misaligned pointers (before any HIP call), TK_ERR_HIP
 * if a launch fails.
 */
tk_status tk_topk_to_pos(const int32_t* topk_idx, int64_t tokens, int64_t k, int64_t experts, int32_t* pos,
                         int32_t* expert_offsets, void* stream);

/* tk_status_str: a static, human-readable name for a status code. */
const char* tk_status_str(tk_status status);

#ifdef __cplusplus
}
#endif

#endif /* TK_H_ */
