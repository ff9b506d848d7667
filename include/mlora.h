/*
 * mlora.h -- C interface of the packed multi-LoRA linear layer for AMD MI355X
 * (gfx950).
 *
 * What it computes.  Many LoRA adapters share one frozen base weight W0.  The
 * packed token axis (sequence length x batch, PLoRA: Efficient Concurrent LoRA
 * Training for Large Language Models, §9.2) is split into contiguous
 * segments: rows [o_i, o_{i+1}) belong to adapter i.  Each adapter computes
 * exactly standard LoRA on its rows (same page, §2.4), with the shapes of
 * §2.1 (W0: d_in x d_out, A_i: d_in x r_i, B_i: r_i x d_out; the page's
 * product "B x A" is read as A.B, the only order the shapes allow):
 *
 *   forward :  Z'_i = s_i X_i A_i                      (saved activation)
 *              Y_i  = X_i W0 + Z'_i B_i
 *   backward:  dZ_i = s_i dY_i B_i^T                   (PLoRA §9.2 Case 2)
 *              dB_i = Z'_i^T dY_i  (= s_i Z_i^T dY_i)  (Case 1)
 *              dA_i = X_i^T dZ_i                       (Case 3)
 *              dX_i = dY_i W0^T + dZ_i A_i^T           (Case 4 plus the base)
 *
 * W0 is frozen and gets no gradient.  An adapter with no rows gets dA_i = 0
 * and dB_i = 0.  Gradients are written, never accumulated.
 *
 * Precision.  MLORA_BF16: X, W0, A_i, B_i, dY, Y, dX, Z' and the internal
 * dZ are bf16 (round to nearest even); every product accumulates in fp32;
 * dA_i and dB_i are fp32.  MLORA_FP32: every tensor fp32, fp32 arithmetic,
 * no reduced-precision step anywhere.
 *
 * Layouts.  Row-major, densely packed: X [T][d_in], Y [T][d_out],
 * dY [T][d_out], dX [T][d_in], A_i [d_in][r_i], B_i [r_i][d_out],
 * dA_i [d_in][r_i] fp32, dB_i [r_i][d_out] fp32.  W0 is [d_in][d_out]
 * (MLORA_W0_KN, the math layout) or [d_out][d_in] (MLORA_W0_NK, the layout of
 * an nn.Linear weight), or both (MLORA_W0_BOTH): one buffer holding
 * [d_in][d_out] followed by its transpose [d_out][d_in].  The base is
 * frozen, so a caller with memory to spare keeps both once
 * (mlora_base_transpose builds the second half).  The forward then reads
 * [d_out][d_in] and the backward's dX [d_in][d_out]: in both products both
 * GEMM operands are contiguous along the reduction, the base GEMM's faster
 * case.  Results are bit-identical to either single layout.  The saved activation Z' is plan-defined: adapter i
 * occupies plan.zoff[i] .. + n_i*r_pad(i) elements as [n_i][r_pad(i)], the
 * padding columns zero.
 *
 * Memory and ownership.  Every device buffer belongs to the caller: tensors,
 * the saved activation (mlora_plan_info.z_bytes) and the workspace
 * (mlora_plan_info.workspace_bytes).  Per-adapter pointers and scales are
 * passed as DEVICE arrays (as batched BLAS interfaces take them): the caller
 * uploads the n pointers / floats once and reuses them while the adapter set
 * is unchanged.  Device pointers must be 16-byte aligned.  The plan owns only
 * host tables and, when it uses more than one stream, its internal streams
 * and events.
 *
 * Streams.  Work is enqueued on the caller's stream (a hipStream_t passed as
 * void*, NULL = the null stream) and the calls return without waiting.  The
 * plan's internal side stream, forked from the caller's stream and joined
 * back to it with events before a call returns (so the caller sees ordinary
 * single-stream ordering), runs the HBM-bound LoRA work beside the base
 * GEMMs: with n_streams > 1 adapter groups, every group's shrink and dZ,
 * group by group, while each group's base GEMM (its row tiles, rule 7 of
 * mlora_plan) runs on the caller's stream once its own group's shrink or dZ
 * is done; and the backward's weight
 * gradients (dA, dB) beside the dX GEMMs when wg_overlap resolves to
 * MLORA_WG_SIDE (otherwise they follow the last dX GEMM on the caller's
 * stream).  The GEMMs of different groups never run at the same time, so
 * each has the chip and its caches to itself.
 *
 * Graph capture.  forward, backward and mlora_adamw_step enqueue only
 * kernels and stream-ordering events (no allocation, no memset), so a plan
 * with one stream group can be captured into a HIP graph and replayed.  A
 * plan with several stream groups returns MLORA_ERR_UNSUPPORTED on a
 * capturing stream (ending such a capture faulted in the runtime).
 *
 * Errors.  Every call validates its arguments on the host before launching
 * anything; on failure it returns a negative status, launches nothing and
 * writes no output.  mlora_last_error() gives a thread-local message.  No call
 * aborts or throws.  Calls on one plan are not thread-safe.
 */
#ifndef MLORA_H
#define MLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLORA_OK = 0,
  MLORA_ERR_INVALID_ARG = -1, /* malformed offsets/ranks/pointers/sizes   */
  MLORA_ERR_UNSUPPORTED = -2, /* rank > 256, dims not multiples of 64, device not gfx950 */
  MLORA_ERR_HIP = -3,         /* a HIP runtime call failed (message has the hipError_t) */
  MLORA_ERR_WORKSPACE = -4,   /* workspace too small or plan tables not uploaded to it */
  MLORA_ERR_NOMEM = -5        /* host allocation failed                    */
} mlora_status;

typedef enum { MLORA_FP32 = 0, MLORA_BF16 = 1 } mlora_dtype;
typedef enum { MLORA_W0_KN = 0, MLORA_W0_NK = 1, MLORA_W0_BOTH = 2 } mlora_w0_layout;
typedef enum { MLORA_W0_BF16 = 0, MLORA_W0_MXFP8 = 1, MLORA_W0_MXFP4 = 2 } mlora_w0_format;
typedef enum { MLORA_ACT_BF16 = 0, MLORA_ACT_MXFP8 = 1 } mlora_act_format;

/* The backward's weight gradients (dA, dB) run on the side stream beside the
 * dX GEMM(s) (SIDE), or after them on the caller's stream (AFTER).  AUTO:
 * SIDE when the dX GEMMs of all stream groups together have at most 16
 * rounds of 256 output tiles (their last round leaves CUs idle that the
 * reductions fill), AFTER when they have more (the HBM-bound reductions then
 * mostly compete with the GEMM for CUs and memory bandwidth: on the
 * 70B-shaped MLP pair beside costs the dX GEMMs 7.6 ms a step, after costs
 * 3.7 ms).  bf16 plans; the fp32 path runs everything on the caller's
 * stream.  Results are bitwise identical either way. */
typedef enum { MLORA_WG_AUTO = 0, MLORA_WG_SIDE = 1, MLORA_WG_AFTER = 2 } mlora_wg_overlap;

#define MLORA_MAX_RANK 256
#define MLORA_MAX_ADAPTERS 65536
#define MLORA_MAX_STREAMS 4
#define MLORA_MAX_PROJECTIONS 8

/* Plan options.  A zero field takes its default. */
typedef struct {
  int32_t nano_rows;      /* NB, rows per nano-batch (16..256, multiple of 16; bf16: of 32);
                             default: 128 when T * n_proj >= 65536, 64 when >= 32768, else 32 */
  int32_t gemm_rows;      /* BM, rows per GEMM tile; default 256 (bf16 requires 256)        */
  int32_t n_streams;      /* adapter groups on separate streams, 1..4; default 1            */
  int32_t chunk_min;      /* reduction chunk rows, KC_i = min(chunk_max,                    */
  int32_t chunk_max;      /*   max(chunk_min, chunk_per_rank * r_pad(i)));                  */
  int32_t chunk_per_rank; /*   defaults 256, 2048, 8                                        */
  int32_t w0_layout;      /* mlora_w0_layout; default MLORA_W0_KN (BOTH: bf16/fp32 W0 only)  */
  int32_t w0_format;      /* mlora_w0_format; default MLORA_W0_BF16 (MXFP8, MXFP4: bf16 plans only) */
  int32_t act_format;     /* mlora_act_format of the activations in the forward's base product;
                             MLORA_ACT_MXFP8 needs w0_format MXFP8 or MXFP4, w0_layout NK and
                             d_in a multiple of 128 (see "Activations on the MXFP8 matrix cores") */
  int32_t wg_overlap;     /* mlora_wg_overlap: where the backward's weight gradients run
                             (see "Streams"); default MLORA_WG_AUTO */
  int32_t grad_accumulate;/* 0 (default): mlora_backward overwrites dA_i and dB_i (an adapter
                             with no rows gets zeros); 1: it adds this call's gradients to
                             what dA_i and dB_i hold (accumulation over micro-batches; an
                             adapter with no rows keeps its values) */
} mlora_plan_opts;

typedef struct mlora_plan_s *mlora_plan_t;

/*
 * mlora_plan -- build the host plan for one packed layer (no HIP call).
 *
 * seg_offsets: host, n+1 entries, seg_offsets[0] = 0, non-decreasing,
 *   T = seg_offsets[n] < 2^31.  ranks: host, n entries in [1, 256].
 *   1 <= n <= MLORA_MAX_ADAPTERS; d_in, d_out positive multiples of 64.
 * The rule (tLoRA: Efficient Multi-LoRA Training with Elastic Shared
 * Super-Models, abstract: low-rank tiles re-formed per rank, rank-aware
 * nano-batches; PLoRA §9.2: tile tokens and hidden dims, never the rank):
 *  1. r_pad(i) = max(32, next power of two >= r_i).
 *  2. zoff(i) = sum_{j<i} n_j r_pad(j); roff(i) = sum_{j<i} r_pad(j).
 *  3. S' = min(n_streams, n) groups of consecutive adapters: g_0 = 0,
 *     g_S' = n, g_s = max(g_{s-1}, first a with o_a >= ceil(s T / S')).
 *  4. Inside a group adapters are visited by r_pad descending, index
 *     ascending.
 *  5. Nano-batches: each adapter's rows cut into pieces of NB rows (NB from
 *     the options, else 128, 64 or 32 as T * n_proj reaches 65536, 32768
 *     or neither: larger pieces share the rank operand over more rows while
 *     a small layer keeps enough pieces to fill the chip).
 *  6. Reduction chunks: pieces of KC_i rows; chunk c's partial sums sit at
 *     rank-row prefix cpref(c) = sum of r_pad over earlier chunks.
 *  7. GEMM row tiles of BM rows from row 0, M = ceil(T / BM) of them (the
 *     last one partial).  Group s's GEMMs take tiles [a_s, a_{s+1}): a_0 = 0,
 *     a_S' = M, a_s = max(a_{s-1}, G floor(floor(o_{g_s} / BM) / G)), G = 16
 *     when M >= 32 S' and 1 otherwise.  A group's GEMM thus holds rows of
 *     its own and earlier groups only (whose shrink and dZ have run), and
 *     with G = 16 it covers whole rounds of 256 output tiles for any output
 *     width that is a multiple of 4096.  Each tile lists extension steps
 *     (adapter j of any group, rows [lo,hi) of j in the tile,
 *     k0 = 0,32,..<r_pad(j)).
 *  8. Optimizer work items (see OPT_BLOCKS below).
 *  9. bf16 only: a group's GEMM with t = (row tiles) x ceil(N / 256) output
 *     tiles and nk = K / 32 K-steps (forward: N = d_out, K = d_in; dX:
 *     N = d_in, K = d_out) splits K into S parts when t < 128 and nk >= 16:
 *     S = min(floor(256 / t), floor(nk / 8), 16), then with kper =
 *     ceil(nk / S), S = ceil(nk / kper); S < 2 means no split.  The parts'
 *     fp32 sums are added in part order, so results stay bitwise
 *     repeatable.
 * The copies of seg_offsets/ranks are the plan's; the caller's arrays may be
 * freed on return.  On error *out is left untouched.
 */
mlora_status mlora_plan(int32_t n, const int64_t *seg_offsets, const int32_t *ranks, int64_t d_in,
                        int64_t d_out, mlora_dtype dtype, const mlora_plan_opts *opts,
                        mlora_plan_t *out);

/*
 * mlora_plan_from_ids -- the same for rows in the caller's order, each
 * token naming its adapter: token t belongs to adapter token_adapter[t]
 * (host, T entries, each in [0, n); T may be 0).  A stable counting sort by
 * id groups the rows (each adapter's rows keep the caller's order); the
 * resulting segments get the plan of mlora_plan, and the permutation
 * (MLORA_TAB_PERM: grouped row -> caller row) is applied inside forward and
 * backward: X, dY, Y and dX stay in the caller's row order, Z' is in grouped
 * order.  The PLoRA page (§2.4) gives every packed adapter its own inputs;
 * ids are another way for a caller to name them.  Errors as mlora_plan, plus
 * MLORA_ERR_INVALID_ARG for an id out of range.
 */
mlora_status mlora_plan_from_ids(int32_t n, int64_t T, const int32_t *token_adapter,
                                 const int32_t *ranks, int64_t d_in, int64_t d_out, mlora_dtype dtype,
                                 const mlora_plan_opts *opts, mlora_plan_t *out);

/*
 * mlora_plan_multi -- one packed layer over several projections that share
 * the same input, e.g. Q, K and V of an attention block or gate and up of an
 * MLP block (PLoRA §8: an adapter can target each of these matrices; they
 * all read the block's input).  Projection q has output width widths[q];
 * the projections are concatenated along the output: q owns columns
 * [c_q, c_q + widths[q]) of Y, dY and W0 (c_q = sum of earlier widths,
 * d_out = sum of all widths), so W0 is the concatenated frozen weight
 * [d_in][d_out] (KN) or [d_out][d_in] (NK).  Adapter i has, for every
 * projection q, its own rank ranks[i * n_proj + q] in [1, 256], A_iq
 * [d_in][r_iq], B_iq [r_iq][widths[q]] and scale; forward, backward and
 * mlora_adamw_step take the per-adapter device arrays (A, B, scales, dA, dB,
 * and the optimizer's) with n * n_proj entries in that order.  Per pair
 * (i, q) the layer computes standard LoRA on adapter i's rows and columns of
 * q; dX sums every projection:
 *   Y_i[:, cols_q] = X_i W0_q + s_iq X_i A_iq B_iq
 *   dX_i = sum_q (dY_i[:, cols_q] W0_q^T + s_iq dY_i[:, cols_q] B_iq^T A_iq^T)
 * The plan is mlora_plan's rule over the pairs v = i * n_proj + q (the
 * tables indexed per adapter have one entry per pair), with buckets ordered
 * by padded rank, then projection, then adapter, and each GEMM row tile
 * listing its extension steps projection by projection (TILE_EXT_START has
 * n_tiles * n_proj + 1 entries).  1 <= n_proj <= MLORA_MAX_PROJECTIONS; with
 * n_proj > 1 every width must be a multiple of 256 (bf16) or 64 (fp32), so
 * no GEMM column tile straddles two projections.  n_proj = 1 is mlora_plan.
 */
mlora_status mlora_plan_multi(int32_t n, const int64_t *seg_offsets, int32_t n_proj,
                              const int64_t *widths, const int32_t *ranks, int64_t d_in,
                              mlora_dtype dtype, const mlora_plan_opts *opts, mlora_plan_t *out);

/*
 * mlora_plan_multi_from_ids -- mlora_plan_multi for rows in the caller's
 * order: token t belongs to adapter token_adapter[t] (as mlora_plan_from_ids;
 * the stable counting sort gives the segments and MLORA_TAB_PERM), and every
 * adapter has a rank per projection (ranks[i * n_proj + q]).  Errors as
 * mlora_plan_multi plus MLORA_ERR_INVALID_ARG for an id out of range.
 */
mlora_status mlora_plan_multi_from_ids(int32_t n, int64_t T, const int32_t *token_adapter,
                                       int32_t n_proj, const int64_t *widths, const int32_t *ranks,
                                       int64_t d_in, mlora_dtype dtype, const mlora_plan_opts *opts,
                                       mlora_plan_t *out);

void mlora_plan_destroy(mlora_plan_t plan);

typedef struct {
  int64_t T, n, d_in, d_out;
  int32_t dtype, n_groups;
  int64_t z_elems, z_bytes;  /* saved activation Z' size                        */
  int64_t workspace_bytes;   /* device workspace for forward and backward       */
  int64_t table_bytes;       /* leading part of the workspace holding the tables */
  int64_t rpad_total, partial_rows;
  int64_t n_nano, n_chunks, n_tiles, n_ext;
  int64_t n_opt_blocks;      /* optimizer work items (0: layer too large, see mlora_adamw_step) */
  int64_t n_proj;            /* projections sharing the input (1 unless mlora_plan_multi) */
  int64_t act_offset;        /* act_format MLORA_ACT_MXFP8: byte offset in the workspace of the
                                last forward's MXFP8 activations, T * d_in E4M3 codes [T][d_in]
                                (rows in the caller's order), then T * d_in / 32 E8M0 scale
                                codes [T][d_in / 32]; -1 otherwise */
  int64_t dz_offset;         /* byte offset in the workspace of dZ = s dY B^T (PLoRA §9.2,
                                Case 2) as the last backward left it: z_elems elements in
                                the layout of Z' (plan dtype), padding columns zero */
  int32_t wg_side;           /* 1: the backward's weight gradients run beside the dX GEMM
                                on the side stream (wg_overlap resolved); 0: after it */
  int32_t reserved;
} mlora_plan_info;

mlora_status mlora_plan_get_info(mlora_plan_t plan, mlora_plan_info *info);

/* Plan tables, for inspection and bit-exact testing.  All int32 except
 * MLORA_TAB_ZOFF and MLORA_TAB_OFFSETS (int64).  Shapes:
 *   RPAD[n], ZOFF[n], ROFF[n], GROUPS[S'+1] (first adapter of each group),
 *   NANO[n_nano][3] (adapter, row0, rows), NANO_START[S'+1],
 *   CHUNKS[n_chunks][3], CHUNK_START[S'+1], CHUNK_RPREF[n_chunks],
 *   ADAPTER_CHUNK_FIRST[n], ADAPTER_CHUNK_COUNT[n],
 *   TILES[n_tiles][2] (row0, rows), TILE_START[S'+1],
 *   EXT[n_ext][4] (adapter, lo, hi, k0), TILE_EXT_START[n_tiles+1],
 *   OFFSETS[n+1], RANKS[n], PERM[T] (plans from ids; empty otherwise),
 *   OPT_BLOCKS[n_opt_blocks][2] (tensor, piece): the work items of
 *   mlora_adamw_step, for every adapter i ascending A_i (tensor 2i) then B_i
 *   (tensor 2i+1), each cut into pieces of 2048 elements,
 *   PROJ_COLS[n_proj+1] (first output column of each projection, then
 *   d_out), SEG_START[n*n_proj] (int64: first row of each pair's adapter),
 *   CHUNK_BOFF[n_chunks] (int64: element offset of each chunk's dB partial
 *   sums, rows of the chunk's projection width), KSPLIT[S'][2] (K-split of
 *   each group's forward and dX GEMM, rule 9 of mlora_plan), OPT_FIRST[n+1]
 *   (first OPT_BLOCKS entry of each adapter).
 * With mlora_plan_multi, "adapter" above means the (adapter, projection)
 * pair v = i * n_proj + q: RANKS, RPAD, ZOFF, ROFF and the per-adapter chunk
 * tables have n * n_proj entries; OFFSETS and GROUPS are over adapters. */
typedef enum {
  MLORA_TAB_RPAD = 0,
  MLORA_TAB_ZOFF,
  MLORA_TAB_ROFF,
  MLORA_TAB_GROUPS,
  MLORA_TAB_NANO,
  MLORA_TAB_NANO_START,
  MLORA_TAB_CHUNKS,
  MLORA_TAB_CHUNK_START,
  MLORA_TAB_CHUNK_RPREF,
  MLORA_TAB_ADAPTER_CHUNK_FIRST,
  MLORA_TAB_ADAPTER_CHUNK_COUNT,
  MLORA_TAB_TILES,
  MLORA_TAB_TILE_START,
  MLORA_TAB_EXT,
  MLORA_TAB_TILE_EXT_START,
  MLORA_TAB_OFFSETS,
  MLORA_TAB_RANKS,
  MLORA_TAB_PERM,
  MLORA_TAB_OPT_BLOCKS,
  MLORA_TAB_PROJ_COLS,
  MLORA_TAB_SEG_START,
  MLORA_TAB_CHUNK_BOFF,
  MLORA_TAB_KSPLIT,
  MLORA_TAB_OPT_FIRST,
  MLORA_TAB_COUNT
} mlora_table;

/* Copies table `table` into host buffer dst.  *bytes_inout: capacity in,
 * bytes written out.  Capacity too small -> MLORA_ERR_INVALID_ARG with
 * *bytes_inout set to the size needed.  dst may be NULL to query the size. */
mlora_status mlora_plan_export(mlora_plan_t plan, int32_t table, void *dst, size_t *bytes_inout);

/* Copies the plan tables into the leading table_bytes of `workspace` on
 * `stream` and remembers the workspace address.  Needed once per (plan,
 * workspace) pair before forward/backward; they refuse any other workspace
 * with MLORA_ERR_WORKSPACE.  The copy is asynchronous from plan-owned host
 * memory that stays valid until the plan is destroyed. */
mlora_status mlora_plan_upload(mlora_plan_t plan, void *workspace, size_t ws_bytes, void *stream);

/*
 * A frozen base in MXFP8 (w0_format = MLORA_W0_MXFP8; the PLoRA page, §5 and
 * §11.3, trains adapters over bases that QLoRA-style methods keep in a low
 * precision, since the base is only read).  W0 then points at one buffer:
 * d_in * d_out E4M3 element codes (OCP FP8: S.EEEE.MMM, bias 7, S.1111.111
 * NaN, largest 448) laid out as the bf16 W0 of the same w0_layout would be,
 * followed at byte offset d_in * d_out by d_out * (d_in / 32) E8M0 scale
 * codes [d_out][d_in / 32] (2^(X - 127), 255 NaN), one per 32 consecutive
 * inputs of an output column.  The weight the layer multiplies is element x
 * scale rounded to bf16 (nearest even; exact unless below bf16's normal
 * range).  forward, and backward when it computes dX, first decode W0 into
 * the workspace (2 * d_in * d_out bytes, counted in workspace_bytes) with
 * one HBM-bound kernel (MLORA_K_DEQUANT), then run the bf16 path.  The
 * resident base takes 1 + 1/32 bytes per weight instead of 2.
 *
 * A 4-bit base (QLoRA's setting in §11.3 of the page), taken as MXFP4
 * (w0_format = MLORA_W0_MXFP4): the same except that the elements are E2M1
 * codes (OCP FP4: S.EE.M, bias 1, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, no
 * NaN or infinity), two to a byte along the rows of the layout with the
 * even element in the low four bits: d_in * d_out / 2 code bytes, the scale
 * codes following at that byte offset.  Products from 2^128 up decode to
 * infinity.  The resident base takes 0.5 + 1/32 bytes per weight.
 *
 * Activations on the MXFP8 matrix cores (act_format = MLORA_ACT_MXFP8, with
 * an MXFP8 or MXFP4 base held as [d_out][d_in]): the forward's base product
 * runs on gfx950's scaled matrix instruction (v_mfma_scale_f32_32x32x64_
 * f8f6f4: E4M3 x E4M3, or an E2M1 base against E4M3 activations) with no
 * bf16 copy of W0.  X is first quantized to MXFP8 by the OCP
 * microscaling conversion, per row in blocks of 32 inputs along d_in: the
 * block's shared exponent is floor(log2 max|x|) - 8, clamped to [-127, 127]
 * (-127 for a block of zeros); elements x 2^-exponent are rounded to the
 * nearest E4M3 value, ties to even, saturating at 448 (one HBM-bound
 * kernel, MLORA_K_QUANT_ACT; the result stays in the workspace,
 * mlora_plan_info.act_offset).  The forward then computes
 *   Y = Q(X) W0 + Z' B,  Z' = s X A
 * with the LoRA terms on X itself, as bf16 extension steps of the same
 * GEMM.  The backward is unchanged (dX = dY W0^T + dZ A^T over the decoded
 * base: the straight-through reading of the activation quantizer).  The
 * forward over a large K split into parts (rule 9) is not split on this
 * path.
 */

/*
 * mlora_forward -- Y = X W0 + Z' B per adapter, and Z' = s X A saved.
 * X [T][d_in]; W0 per w0_layout; A, B: device arrays of n device pointers;
 * scales: device array of n floats (any value, 0 and negatives allowed).
 * Y [T][d_out] and Z (z_elems) are overwritten.  Kernels: grouped rank-padded
 * shrink (PLoRA §9.2: split the input dimension for A), then the base GEMM
 * with the LoRA expand as extra K-steps on the same accumulators (split the
 * output dimension for B).
 */
mlora_status mlora_forward(mlora_plan_t plan, const void *X, const void *W0, const void *const *A,
                           const void *const *B, const float *scales, void *Y, void *Z,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * mlora_forward_noalloc -- mlora_forward without a workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The same kernels in the
 * same order, so Y and Z are bit-identical to mlora_forward's.  The work
 * buffers (the plan tables, the rank-padded concatenations of A_i and B_i,
 * split-K partial tiles, a microscaled base's bf16 decoding) live in a
 * static device array of 64 MiB per GPU, held until the process ends; no
 * call allocates or frees anything.  Every call copies the plan tables in
 * first (an asynchronous host-to-device copy on `stream`), and writes every
 * other scratch byte it reads earlier in the same call, so nothing carries
 * over from the previous call.  All calls on one GPU share that array:
 * calls that overlap on one GPU (several streams, several threads) race and
 * must be ordered by the caller.  A layer whose buffers exceed the scratch
 * returns MLORA_ERR_UNSUPPORTED with nothing launched (mlora_forward has no
 * such limit).  Arguments and errors otherwise as mlora_forward; no
 * mlora_plan_upload is needed.
 */
mlora_status mlora_forward_noalloc(mlora_plan_t plan, const void *X, const void *W0, const void *const *A,
                                   const void *const *B, const float *scales, void *Y, void *Z,
                                   void *stream);

/*
 * mlora_backward -- dX (optional, NULL skips it), dA_i, dB_i (fp32).
 * Inputs as in forward plus dY [T][d_out] and the Z' saved by forward.
 * dA, dB: device arrays of n device pointers to fp32 buffers.  Case 2 (dZ)
 * reduces over d_out inside one workgroup; Cases 1 and 3 reduce over tokens in
 * fixed-size chunks whose partial sums are added in a fixed order (no float
 * atomics: results are bitwise repeatable for a given plan); Case 4 runs as
 * extra K-steps of the dX GEMM.  dA_i and dB_i are overwritten, or, with the
 * plan option grad_accumulate, this call's gradients are added to them (one
 * fp32 rounding per element; dX is overwritten either way).
 */
mlora_status mlora_backward(mlora_plan_t plan, const void *dY, const void *X, const void *W0,
                            const void *const *A, const void *const *B, const float *scales,
                            const void *Z, void *dX, void *const *dA, void *const *dB,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * Per-adapter optimizer hyperparameters for mlora_adamw_step.  step is the
 * number of this update for the adapter (1 for its first), used in the bias
 * corrections; an adapter with step <= 0 is skipped: its weights, moments and
 * copies are left untouched.  Useful ranges: lr >= 0, 0 <= beta1, beta2 < 1,
 * eps > 0; the values live in device memory and are not checked (a beta of 1
 * gives that adapter a zero bias correction and IEEE inf/NaN weights, never
 * a fault).
 */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t step;
  float max_grad_norm; /* > 0: clip the adapter's gradients to this 2-norm (used when clip_grads = 1) */
} mlora_adamw_hparams;

/*
 * mlora_adamw_step -- one AdamW update of every adapter's A_i and B_i, each
 * adapter with its own hyperparameters and state (PLoRA §2.4: every packed
 * adapter keeps its own parameters and optimizer state; §8: AdamW keeps a
 * momentum and a velocity per trained parameter; §2.2 and §11.1: learning
 * rate and the other knobs differ per configuration).  The pages do not
 * write AdamW out; the update is Adam with decoupled weight decay scaled by
 * the learning rate (the torch.optim.AdamW form), per element:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *   p <- p - (lr / (1 - b1^step)) m / (sqrt(v / (1 - b2^step)) + eps)
 * in fp32.
 *
 * Clipping (clip_grads = 1): an adapter with max_grad_norm > 0 first has all
 * its gradients multiplied by min(1, max_grad_norm / (||g|| + 1e-6)), ||g||
 * the 2-norm over its dA and dB together (the rule of PyTorch's
 * clip_grad_norm_, per adapter: every packed job clips on its own).  The
 * norms are fp32 sums in a fixed order (bitwise repeatable); two extra
 * launches.  clip_grads = 0 ignores max_grad_norm.
 *
 * hparams: device array of n mlora_adamw_hparams.  A, B: device arrays of n
 * device pointers to the fp32 master weights ([d_in][r_i] and [r_i][d_out]),
 * updated in place.  dA, dB: fp32 gradients as mlora_backward writes them.
 * mA, vA, mB, vB: fp32 first and second moments, same shapes, updated in
 * place (zero them before an adapter's first step).  A_copy, B_copy: for a
 * bf16 plan, NULL or device arrays of pointers to the bf16 weights the
 * forward and backward read, overwritten with the updated masters rounded to
 * nearest even (both or neither); for an fp32 plan both must be NULL (the
 * masters are the weights).  No two of the buffers may overlap.  The work
 * items are the plan's OPT_BLOCKS table, so the workspace must hold the
 * uploaded tables; the call writes nothing else in it.  MLORA_ERR_UNSUPPORTED
 * when the layer has more than 2^27 work items (n_opt_blocks = 0).
 */
mlora_status mlora_adamw_step(mlora_plan_t plan, const mlora_adamw_hparams *hparams,
                              void *const *A, void *const *B, const void *const *dA,
                              const void *const *dB, void *const *mA, void *const *vA,
                              void *const *mB, void *const *vB, void *const *A_copy,
                              void *const *B_copy, int32_t clip_grads, void *workspace,
                              size_t ws_bytes, void *stream);

/*
 * mlora_base_transpose -- out[c][r] = in[r][c] for a rows x cols matrix of
 * bf16 (dtype MLORA_BF16) or fp32 (MLORA_FP32) elements, enqueued on
 * `stream`.  Builds the second half of an MLORA_W0_BOTH base: in = the
 * [d_in][d_out] half (rows = d_in, cols = d_out), out = in + d_in * d_out
 * elements.  Device pointers, 16-byte aligned, not overlapping; rows and
 * cols positive multiples of 64 (the layer's dimensions are).
 * MLORA_ERR_INVALID_ARG otherwise, with nothing launched.  Not part of any
 * step: the base is frozen, so it runs once.
 */
mlora_status mlora_base_transpose(const void *in, void *out, int64_t rows, int64_t cols,
                                  mlora_dtype dtype, void *stream);

/* Per-kernel timing.  Launches of the selected kinds are bracketed by HIP
 * events on the stream they run on; mlora_profile_read waits for them, adds
 * their durations to the totals of kernel `kind` and returns them, then
 * clears.  Each pair of events costs a few microseconds of stream time, so a
 * caller timing whole steps selects only the kernels it needs. */
typedef enum {
  MLORA_K_SHRINK = 0,    /* Z' = s X A (F1)                                  */
  MLORA_K_GEMM_FWD,      /* Y = X W0 + Z' B (F2)                             */
  MLORA_K_DZ,            /* dZ = s dY B^T (B1)                               */
  MLORA_K_TOKEN_REDUCE,  /* chunk partials of dB (B2) and dA (B3), one launch */
  MLORA_K_REDUCE,        /* fixed-order sum of the chunk partials            */
  MLORA_K_GEMM_DX,       /* dX = dY W0^T + dZ A^T (B4)                       */
  MLORA_K_PREP,          /* rank-padded concatenations of A and B            */
  MLORA_K_ADAMW,         /* per-adapter AdamW step (mlora_adamw_step)        */
  MLORA_K_DEQUANT,       /* decode of an MXFP8/MXFP4 base weight into bf16   */
  MLORA_K_GRAD_NORM,     /* per-adapter gradient norms and clip factors      */
  MLORA_K_QUANT_ACT,     /* activations to MXFP8 (act_format MLORA_ACT_MXFP8) */
  MLORA_K_COUNT
} mlora_kernel_kind;

/* mask: bit k selects kind k (1 << MLORA_K_GEMM_FWD, ...); 0 disables
 * timing; MLORA_PROFILE_ALL selects every kind. */
#define MLORA_PROFILE_ALL (-1)
mlora_status mlora_profile_enable(mlora_plan_t plan, int32_t mask);
mlora_status mlora_profile_read(mlora_plan_t plan, double *total_ms /*[MLORA_K_COUNT]*/,
                                int64_t *launches /*[MLORA_K_COUNT]*/);

/* MLORA_OK when the current device is gfx950, else MLORA_ERR_UNSUPPORTED. */
mlora_status mlora_device_check(void);

const char *mlora_status_string(mlora_status s);
const char *mlora_last_error(void);
const char *mlora_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLORA_H */
