/*
 * moe.h -- C ABI of the MI355X (gfx950) fused mixture-of-experts FFN forward.
 *
 *   y_t = sum_{e in TopK(t)} alpha_{t,e} * ( W2_e^T ( SiLU(x_t W13_e[:, :I] + b13_e[:I])
 *                                                  * (x_t W13_e[:, I:] + b13_e[I:]) ) + b2_e )
 *
 * Sources (the pages on fused MoE):
 *   - the math: FlagGems "fused_moe.py" walkthrough, sec. 1.1 (MoE definition)
 *     and sec. 1.2 (routed-item form h_r, z_r, o_r, y_t);
 *   - the argument list and its constraints: MindIE-SD "Fused MoE" page,
 *     function signature, parameter table and routing-selection section;
 *   - the two activation formats (contiguous (M, K) + topk ids/weights, and
 *     batched (E, max_tokens, K) + expert_num_tokens) and the
 *     workspace_shapes / apply split: vLLM "Fused MoE Modular Kernel" page,
 *     introduction and the workspace_shapes() section;
 *   - the align metadata (sorted_token_ids, expert_ids, num_tokens_post_padded):
 *     FlagGems walkthrough, "moe_align_block_size" section;
 *   - fp8 W8A8 scales: FlagGems walkthrough, "FP8 W8A8" section.
 *
 * Conventions shared by every entry point:
 *   - Every buffer is caller-owned device memory (except the two structs,
 *     which are host memory read during the call).  The library allocates
 *     nothing, keeps no pointer after returning, and enqueues all work on the
 *     caller's stream; it never synchronises the host.  A call can therefore
 *     be captured into a HIP graph.
 *   - Row-major, contiguous tensors with a stride-1 last dimension.  Leading
 *     dims of a [..., H] activation are flattened into M by the caller.
 *   - Expert ids are int32, routing weights float32.
 *   - All argument checks run on the host before anything is enqueued; on
 *     error nothing is enqueued.  Device-side data cannot be checked on the
 *     host; the kernels handle it safely and report it in the workspace's
 *     device status word (moe_device_status): precomputed topk ids outside
 *     [0, E) (or [0, global_experts)) and expert_map values outside [-1, E)
 *     contribute nothing, expert_num_tokens values outside [0, max_tokens]
 *     are clamped, token_map entries that name no valid row are skipped.
 *   - Thread safety: concurrent calls are safe when they use distinct
 *     workspaces and outputs.  The library's only process state is a
 *     per-device cache of device attributes (compute units, kernel
 *     occupancy), filled on first use with atomic stores.
 *   - The library reads no environment variables.
 *   - Two builds export this same ABI: libmoe.so, and libmoe_checked.so, a
 *     bounds-checked build for debugging (moe_version() ends in "checked").
 *     In the latter every index the kernels take from device data (the GEMM
 *     tile table, sorted ids behind row gathers and output rows, the reduce's
 *     row map) is checked against its buffer first; an index outside it is
 *     not used and sets MOE_DEV_BOUNDS.  With valid inputs both builds give
 *     the same results bit for bit.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* shape / range / null-pointer violation            */
    MOE_ERR_UNSUPPORTED = -2, /* valid request this build does not implement        */
    MOE_ERR_WORKSPACE = -3,   /* workspace null, misaligned (256 B) or too small    */
    MOE_ERR_LAUNCH = -4,      /* a kernel launch failed (hipGetLastError)           */
    MOE_ERR_STATIC_LIMIT = -5 /* moe_forward_static: the problem's workspace exceeds
                                 MOE_STATIC_WORKSPACE_BYTES                        */
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_FP8_E4M3FN = 2,
    MOE_U8 = 3,               /* weights only: unsigned 8-bit codes (WNA16, int8_w8a16)  */
    MOE_U4 = 4                /* weights only: unsigned 4-bit codes, two per byte (int4_w4a16) */
} moe_dtype;

typedef enum {
    MOE_ROUTE_SOFTMAX = 0,    /* scores = softmax(logits) over all E              */
    MOE_ROUTE_SIGMOID = 1,    /* scores = sigmoid(logits); weights always normalised */
    MOE_ROUTE_PRECOMPUTED = 2 /* caller passes topk_ids / topk_weights (the pages'
                                 custom_routing_function output)                   */
} moe_routing;

typedef enum {
    MOE_FMT_CONTIGUOUS = 0,   /* hidden [M, H], one routed item per (token, slot)  */
    MOE_FMT_BATCHED = 1       /* hidden [E, max_tokens, H] + expert_num_tokens[E]  */
} moe_format;

/* GEMM tile family of the bf16 (and WNA16) expert GEMMs, for moe_problem's
 * tile_hint.  MOE_TILE_AUTO lets the library choose from the average routed
 * rows per expert; the others force one family (tests and tuning sweeps). */
typedef enum {
    MOE_TILE_AUTO = 0,
    MOE_TILE_DMA_160 = 1,     /* 160-row LDS-DMA ring (prefill-sized loads)       */
    MOE_TILE_REG_64 = 2,      /* 64-row register-staged tile (bf16 only)          */
    MOE_TILE_REG_16 = 3,      /* 16-row register-staged tile (bf16 only)          */
    MOE_TILE_DMA_32 = 5,      /* 32-row LDS-DMA ring (decode-sized loads)         */
    MOE_TILE_DMA_64 = 6,      /* 64-row LDS-DMA ring                              */
    MOE_TILE_DMA_256 = 7      /* 256-row LDS-DMA ring (bf16 only; compute-bound)  */
} moe_tile_hint;

/* Bits of the device status word (moe_workspace_info.off_status).  Device-side
 * data that the host cannot check is handled safely on the device, and the
 * forward records here what it found; the word is rewritten by every forward
 * (its align / tile-list kernel stores it, later kernels only OR bits in). */
typedef enum {
    MOE_DEV_ID_RANGE = 1,       /* a precomputed topk id outside [0, experts routed
                                   over), or an expert_map value outside [-1, E):
                                   that routed item got no row                    */
    MOE_DEV_COUNT_CLAMPED = 2,  /* an expert_num_tokens value outside
                                   [0, max_tokens], clamped into that range       */
    MOE_DEV_ROWS_OVERFLOW = 4,  /* batched slabs hold more valid rows than M *
                                   top_k (with M > 0): nothing was computed       */
    MOE_DEV_TOKEN_MAP = 8,      /* a token_map entry (other than -1) that names no
                                   valid slab row contributed nothing             */
    MOE_DEV_BOUNDS = 16         /* bounds-checked build (libmoe_checked.so) only:
                                   a GEMM tile, gathered row or reduce row taken
                                   from device data fell outside its buffer; that
                                   tile or row was skipped                        */
} moe_device_status;

/* Memory layout of w13 / w2 (see moe_pack_weights). */
typedef enum {
    MOE_W_PLAIN = 0,          /* w13 [E, H, 2I], w2 [E, I, H], row-major          */
    MOE_W_PACKED = 1          /* bf16 / fp8: the blocked layouts of moe_pack_weights */
} moe_weight_layout;

/* Problem description (host struct).
 *
 *   format       MOE_FMT_CONTIGUOUS or MOE_FMT_BATCHED.
 *   M            tokens.  Contiguous: rows of hidden/out.  Batched: the tokens
 *                behind the slabs: rows of the token map and of out when
 *                batched_reduce is set.  In the batched format M > 0 promises
 *                that the slabs hold at most M * top_k valid rows in total
 *                (each valid slab row is one routed copy of a token); it sizes
 *                the workspace and guides the tile choice.  M = 0 (only without
 *                batched_reduce) allows up to E * max_tokens rows.  Slabs that
 *                break the promise are not computed: the status word gets
 *                MOE_DEV_ROWS_OVERFLOW, out is zero with batched_reduce and
 *                left unwritten without.
 *   H, I         hidden and intermediate sizes; w13 is [E, H, 2I], w2 [E, I, H].
 *                Both must be multiples of 16; the fp8 path needs I % 128 == 0.
 *   E, top_k     experts (1..1024) and experts per token (1..E, <= 32).
 *   max_tokens   batched: rows per expert slab.
 *   act_dtype    hidden: MOE_F32 or MOE_BF16 (MOE_FP8_E4M3FN: batched only,
 *                pre-quantised codes with a_scale).
 *   w_dtype      weights: same as act_dtype for f32/bf16, or MOE_FP8_E4M3FN
 *                (float scales per output channel, or per block with
 *                fp8_block; activations are then quantised per token, or per
 *                token and 128 columns, on the fly unless already fp8), or
 *                MOE_U8 / MOE_U4: WNA16 weights (the walkthrough's "WNA16"
 *                section, int8_w8a16 / int4_w4a16) with bf16 activations:
 *                weight = (q - z) * s, q the unsigned code, one float scale s
 *                and one zero point z per group of wq_group K rows and output
 *                column (z = 2^(bits-1) when no zero points are given); the
 *                weights are dequantised to bf16 inside the GEMMs, which
 *                accumulate in float32.  Needs w_layout = MOE_W_PACKED.
 *                GPTQ / AWQ checkpoints: moe_repack_wna16 first.
 *   out_dtype    MOE_F32 or MOE_BF16.  f32 activations need f32 out.
 *   logits_dtype MOE_F32 or MOE_BF16 (contiguous, routing != PRECOMPUTED).
 *   routing, renormalize, group_count, k_group, group_select_mode,
 *   routed_scaling_factor
 *                the routing parameters of the MindIE-SD page: grouped
 *                selection picks k_group of group_count contiguous expert
 *                groups by their largest score (mode 0) or the sum of their
 *                two largest scores (mode 1), then top_k experts inside them;
 *                renormalize divides softmax weights by their sum (sigmoid
 *                weights are always divided by their sum); the final weights
 *                are multiplied by routed_scaling_factor.
 *                Constraints: E % group_count == 0, 1 <= k_group <= group_count,
 *                top_k <= k_group * E / group_count, mode 1 needs >= 2 experts
 *                per group.  Ties break toward the lower expert (group) index.
 *   has_w13_bias, has_w2_bias
 *                biases [E, 2I] / [E, H], same dtype as the activations (bf16
 *                for fp8 weights).  b13 is added before the activation; b2 is
 *                added to each expert output, so it is scaled by the weight.
 *   batched_reduce
 *                batched only: also reduce the expert rows into out [M, H] with
 *                token_map / token_map_w (the pages' naive batched
 *                weight-and-reduce); 0 writes the expert rows to out
 *                [E, max_tokens, H] instead.
 *   w_layout     MOE_W_PLAIN, or MOE_W_PACKED when w13 / w2 hold the output of
 *                moe_pack_weights (bf16 or fp8 weights; else MOE_ERR_UNSUPPORTED).
 *   global_experts
 *                contiguous only.  0: the E experts of w13 / w2 are all the
 *                experts.  > 0: routing runs over global_experts experts
 *                (logits [M, global_experts], topk ids in [0, global_experts))
 *                of which this device holds the E of w13 / w2, named by
 *                args->expert_map [global_experts]: the local index of each
 *                global expert, or -1 for an expert held elsewhere (the
 *                expert-parallel shard of the FlagGems walkthrough, whose
 *                kernel writes zeros for an expert id of -1, and of the vLLM
 *                page's expert map).  Routed items of unmapped experts add
 *                nothing to out, which then holds this shard's partial sum;
 *                the workspace topk ids stay global, align counts, sorted ids
 *                and expert ids are local.  Needs global_experts >= E; the
 *                routing constraints apply to global_experts.
 *   apply_weight_on_input
 *                contiguous only.  0: the routing weight scales each expert
 *                output o_r (b2 included).  1: it scales the expert's
 *                intermediate z_r = SiLU(gate) * up before the second GEMM
 *                and the outputs are summed unweighted (the walkthrough's
 *                apply_router_weight_on_input switch, sec. 1.2; equal to 0
 *                when there is no b2, since W2^T (a z) = a W2^T z).
 *   chunk_tokens contiguous only.  0: one pass over all M tokens.  > 0: the
 *                tokens are processed in chunks of chunk_tokens rows, one
 *                after another on the stream (the walkthrough's CHUNK_SIZE
 *                execution), and the workspace is sized for one chunk; its
 *                regions then hold the last chunk's intermediates.
 *   fp8_block    fp8 weights only.  0: per-output-channel weight scales and
 *                per-token activation scales.  128: block-wise scales (the
 *                walkthrough's "FP8 W8A8" block-wise granularity: every
 *                128-deep K block of a product is scaled by its activation
 *                block's and weight block's scales): one weight scale per
 *                128 x 128 block and one activation scale per token and 128
 *                columns (see moe_args).  Needs w_layout = MOE_W_PACKED.
 *                Other block sizes: MOE_ERR_UNSUPPORTED.
 *   tile_hint    a moe_tile_hint.  MOE_TILE_AUTO (0): the library's choice.
 *                Other values force one GEMM tile family (for tests and tuning
 *                sweeps): bf16 weights take any family, WNA16 weights the
 *                LDS-DMA ones (MOE_TILE_DMA_*); f32 and fp8 weights need 0
 *                (MOE_ERR_UNSUPPORTED otherwise).  Unknown values:
 *                MOE_ERR_INVALID_ARG.  Results stay within the tolerances
 *                whatever the family; the workspace size may change with it.
 *   gemm1_wave_cols
 *                0: the library's choice.  2 or 4: the width of the first GEMM's
 *                tile in the 160-row bf16 family (2 x 64 or 4 x 64 weight
 *                columns a wave row); ignored by the other families.  Other
 *                values: MOE_ERR_INVALID_ARG.
 *   wq_group     MOE_U8 / MOE_U4 weights: K rows per scale group, 32, 64 or 128
 *                (0 means 128; the group sizes of GPTQ / AWQ checkpoints).
 *                Other values MOE_ERR_UNSUPPORTED; other weight types need 0
 *                (MOE_ERR_INVALID_ARG).
 */
typedef struct {
    int32_t format;
    int32_t M, H, I, E, top_k;
    int32_t max_tokens;
    int32_t act_dtype, w_dtype, out_dtype, logits_dtype;
    int32_t routing, renormalize, group_count, k_group, group_select_mode;
    float routed_scaling_factor;
    int32_t has_w13_bias, has_w2_bias;
    int32_t batched_reduce;
    int32_t w_layout;
    int32_t global_experts;
    int32_t apply_weight_on_input;
    int32_t chunk_tokens;
    int32_t fp8_block;
    int32_t tile_hint;
    int32_t gemm1_wave_cols;
    int32_t wq_group;
} moe_problem;

/* Workspace layout chosen by the library for one problem.  All offsets are
 * in bytes from the workspace base and 256-byte aligned.  The regions hold
 * the path's intermediates and stay readable after the stream work is done
 * (tests compare them with the CPU definition):
 *   topk_ids [M, top_k] int32, topk_weights [M, top_k] float  (contiguous)
 *   expert_counts [E] int32
 *   expert_offsets [E + 1] int32: start of each expert's padded run in
 *       sorted_ids (entry E = num_post_padded)
 *   sorted_ids [max_sorted_len] int32: positions [0, num_post_padded) hold
 *       the routed items grouped by expert, ascending within an expert, each
 *       expert's run padded to a multiple of block_m with a sentinel
 *       (contiguous: r = t*top_k + j, sentinel M*top_k; batched:
 *       r = e*max_tokens + i, sentinel E*max_tokens)
 *   expert_ids [max_blocks] int32: the expert of each block_m-row block
 *   num_post_padded [1] int32
 *   aq / aq_scale: fp8 activation codes and per-row scales (fp8 weights)
 *   z [max_sorted_len, I]: SiLU(gate)*up per padded row (bf16 or f32; fp8
 *       codes on the fp8 path, with float scales per (row, 128 columns) in
 *       z_scale [I / 128][max_sorted_len + 256], group-major)
 *   o [max_sorted_len, H] (contiguous, and batched with batched_reduce):
 *       each routed item's expert output at its padded position, float
 *   o2 [max_sorted_len, H]: when the second GEMM runs as two K halves, the
 *       second half's partial outputs (the item's output is then o + o2);
 *       off_o2 = 0 when it does not
 *   status [1] int32: the device status word, an OR of moe_device_status
 *       bits, 0 when the device found nothing to report.
 * The layout depends on the problem and on the compute-unit count of the
 * device (a device attribute query; no device work).  */
typedef struct {
    size_t bytes;
    int32_t block_m;
    int32_t max_blocks;
    int64_t max_sorted_len;
    size_t off_topk_ids, off_topk_weights, off_expert_counts, off_expert_offsets, off_sorted_ids,
        off_expert_ids, off_num_post_padded, off_aq, off_aq_scale, off_z, off_z_scale, off_o;
    size_t off_o2, off_status;
} moe_workspace_info;

/* Fills *info for problem *p (host only, no device work; reads the current
 * device's compute-unit count).  The caller then provides a device buffer of
 * info->bytes, 256-byte aligned.  Returns MOE_OK, MOE_ERR_INVALID_ARG or
 * MOE_ERR_UNSUPPORTED (same checks as moe_forward). */
int moe_workspace_shapes(const moe_problem* p, moe_workspace_info* info);

/* Device pointers of one forward (host struct; NULL where unused).  A
 * contiguous forward with M = 0 reads and writes no token array: hidden,
 * out, router_logits and topk_ids / topk_weights may then be NULL, and it
 * returns MOE_OK with nothing enqueued.
 *   hidden            contiguous [M, H]; batched [E, max_tokens, H]
 *                     (rows past expert_num_tokens[e] are never read).
 *   a_scale           batched fp8 activations: [E, max_tokens] per-row scales,
 *                     or [E, max_tokens, ceil(H / 128)] with fp8_block = 128.
 *   router_logits     [M, E] (routing SOFTMAX / SIGMOID).
 *   topk_ids, topk_weights
 *                     [M, top_k] int32 / float (routing PRECOMPUTED).
 *   expert_num_tokens batched: [E] int32 valid rows per slab.
 *   token_map, token_map_w
 *                     batched_reduce: [M, top_k] flat slab row e*max_tokens+i
 *                     holding token t's j-th routed copy, and its weight; -1
 *                     for a copy that has no row here (served by another
 *                     expert-parallel rank), which contributes nothing.  Other
 *                     entries that name no valid slab row (outside
 *                     [0, E*max_tokens), or i >= expert_num_tokens[e])
 *                     contribute nothing and set MOE_DEV_TOKEN_MAP.
 *   w13, w2           [E, H, 2I] (gate = columns [0, I), up = [I, 2I)), [E, I, H];
 *                     MOE_U4 codes two per byte along the last dimension, the
 *                     even column in the low nibble: [E, H, I], [E, I, H / 2].
 *   w13_bias, w2_bias [E, 2I], [E, H] when has_*_bias.
 *   w13_scale, w2_scale
 *                     MOE_U8 / MOE_U4 weights: float per K group (G = wq_group
 *                     rows) and column, [E, ceil(H / G), 2I] and
 *                     [E, ceil(I / G), H].
 *                     fp8 weights: float per output channel, [E, 2I] and [E, H];
 *                     with fp8_block = 128 one float per 128 x 128 block,
 *                     [E, 2I / 128, ceil(H / 128)] and [E, ceil(H / 128), I / 128]
 *                     (output-column block, then K block), the layout of the
 *                     [N / 128, K / 128] per-expert scale grids of block-wise
 *                     fp8 checkpoints.
 *   out               contiguous / batched_reduce: [M, H]; batched: [E, max_tokens, H]
 *                     (only valid rows written).  out may alias hidden in the
 *                     contiguous format (in-place): every read of hidden
 *                     precedes the first write of out on the stream (per
 *                     chunk, when chunk_tokens is set).
 *   expert_map        global_experts > 0: [global_experts] int32, each value
 *                     in [-1, E).
 *   w13_zero, w2_zero MOE_U8 / MOE_U4 weights: uint8 zero points, the shapes of
 *                     w13_scale / w2_scale (one per group and column, values
 *                     below 2^bits), or NULL for the symmetric 2^(bits-1). */
typedef struct {
    const void* hidden;
    const float* a_scale;
    const void* router_logits;
    const int32_t* topk_ids;
    const float* topk_weights;
    const int32_t* expert_num_tokens;
    const int32_t* token_map;
    const float* token_map_w;
    const void* w13;
    const void* w2;
    const void* w13_bias;
    const void* w2_bias;
    const float* w13_scale;
    const float* w2_scale;
    void* out;
    const int32_t* expert_map;
    const uint8_t* w13_zero;
    const uint8_t* w2_zero;
} moe_args;

/* Enqueues one fused MoE forward on `stream` (a hipStream_t; NULL = the
 * default stream): router -> align -> [fp8 activation quant] -> grouped
 * GEMM W13 + bias + SiLU*up [+ fp8 requant] -> grouped GEMM W2 + bias ->
 * top-k weight-and-reduce (unpermute).  `workspace` is a device buffer of at
 * least moe_workspace_shapes(p)->bytes, 256-byte aligned.  Returns MOE_OK
 * after enqueueing, or an error code with nothing enqueued (MOE_ERR_LAUNCH:
 * a launch failed after earlier kernels of the call were enqueued). */
int moe_forward(const moe_problem* p, const moe_args* a, void* workspace, size_t workspace_bytes,
                void* stream);

/* Kernel stages of one forward, in launch order (for moe_forward_timed). */
typedef enum {
    MOE_STAGE_ROUTER = 0,  /* top-k routing (skipped for PRECOMPUTED and batched) */
    MOE_STAGE_ALIGN = 1,   /* align (contiguous) or tile list (batched)           */
    MOE_STAGE_QUANT = 2,   /* per-row fp8 activation quantisation (fp8 weights)   */
    MOE_STAGE_GEMM1 = 3,   /* grouped W13 GEMM + bias + SiLU*up (+ fp8 requant)   */
    MOE_STAGE_GEMM2 = 4,   /* grouped W2 GEMM + bias                              */
    MOE_STAGE_REDUCE = 5,  /* top-k weight-and-reduce (unpermute)                 */
    MOE_NUM_STAGES = 6
} moe_stage;

/* moe_forward with instrumentation for kernel timing: events[2*s] and
 * events[2*s + 1] (hipEvent_t handles created by the caller, may be NULL)
 * are recorded on `stream` immediately before and after the launch of stage
 * s; stages a problem does not run leave their events unrecorded.  `events`
 * points at 2 * MOE_NUM_STAGES handles.  Same work, arguments and errors as
 * moe_forward. */
int moe_forward_timed(const moe_problem* p, const moe_args* a, void* workspace,
                      size_t workspace_bytes, void* stream, void** events);

/* Checkpoint layouts of WNA16 codes, for moe_repack_wna16. */
typedef enum {
    MOE_WQ_GPTQ = 1,          /* codes packed along K into int32 words            */
    MOE_WQ_AWQ = 2            /* codes packed along N, interleaved (4-bit only)   */
} moe_wq_format;

/* Converts the int32-packed codes of a GPTQ or AWQ checkpoint (the
 * walkthrough's "WNA16" section names both layouts) into the plain WNA16
 * layout that moe_pack_weights takes, for E experts of one K x N weight
 * (w13: K = H, N = 2I; w2: K = I, N = H).  per = 32 / bits codes share a
 * word; code slot i of a word is bits [bits * i, bits * (i + 1)).
 *   MOE_WQ_GPTQ (bits 4 or 8): qweight [E, K / per, N], word (r, n) holding
 *     rows per * r + i of column n; qzeros [E, ceil(K / group), N / per],
 *     word (g, c) holding columns per * c + i.
 *   MOE_WQ_AWQ (bits 4): qweight [E, K, N / 8], word (k, c) holding column
 *     8 c + {0, 2, 4, 6, 1, 3, 5, 7}[i] of row k in slot i; qzeros
 *     [E, ceil(K / group), N / 8] the same way.
 * Writes `codes` (bits 8: [E, K, N] bytes; bits 4: [E, K, N / 2], two codes
 * a byte along N, the even column in the low nibble) and, when qzeros is
 * given, `zeros` [E, ceil(K / group), N] uint8: each stored zero point plus
 * zero_adjust, modulo 2^bits (1 for checkpoints that store z - 1, else 0).
 * The checkpoints' scales are already [E, ceil(K / group), N] (convert them
 * to float32); act-order permutations (g_idx) are not taken.  Device
 * buffers, caller-owned, not overlapping; enqueued on `stream`.  Returns
 * MOE_OK; MOE_ERR_INVALID_ARG for a null pointer (zeros null with qzeros
 * given), a non-positive size, K not a multiple of per (GPTQ), N not a
 * multiple of 8 (AWQ) or of per (GPTQ zero points), N odd with 4 bits;
 * MOE_ERR_UNSUPPORTED for bits other than 4 / 8, AWQ with 8 bits, a group
 * other than 32 / 64 / 128, or an unknown format; MOE_ERR_LAUNCH. */
int moe_repack_wna16(int format, int bits, int E, int K, int N, int group,
                     const int32_t* qweight, const int32_t* qzeros, int zero_adjust,
                     uint8_t* codes, uint8_t* zeros, void* stream);

/* Packed weights.  The expert weights are constant across calls, so a caller
 * can re-lay them out once, at load time, into the order in which the grouped
 * GEMMs stream them (the walkthrough's "fused_moe_kernel" section reads each
 * weight tile as a K x BLOCK_SIZE_N block; packing makes every such block of
 * one K stage contiguous in memory).  The packed layout is a sequence of
 * 16 KiB blocks.
 *
 * bf16 weights: each block is 64 weight rows (K) x 128 weight columns (N):
 *   row k of a block is 256 bytes = 16 slots of 16 bytes; slot s holds the
 *   8-column chunk c = s ^ (2 * ((k & 3) | ((k >> 1) & 4))) of that row.
 *   w13: block (e, kt, j), kt < ceil(H / 64), j < ceil(I / 64), in that order
 *        (j fastest: the blocks of one K stage are adjacent); chunks 0-7 are
 *        gate columns 64 j + 8 c .., chunks 8-15 the up columns
 *        I + 64 j + 8 (c - 8) .., of weight rows 64 kt + k.
 *   w2:  block (e, kt, j), kt < ceil(I / 64), j < ceil(H / 128); chunk c holds
 *        columns 128 j + 8 c .. of weight rows 64 kt + k.
 * fp8 weights (K-contiguous): each block is 128 weight columns (N) x 128
 *   weight rows (K) of one-byte codes: column n of a block is 128 bytes =
 *   8 slots of 16 bytes; slot s holds the codes of weight rows
 *   128 kt + 16 q .. + 15 with p = s ^ ((n >> 1) & 7), q = 2 (p & 3) + (p >> 2)
 *   (the even 16-row chunks before the odd ones, then the column's XOR).
 *   w13: block (e, kt, j), kt < ceil(H / 128), j < I / 64, j fastest; block
 *        columns 0-63 hold gate columns 64 j .., 64-127 the up columns
 *        I + 64 j .., each half in 32-column groups: block column
 *        32 h + 16 f + s (f < 2, s < 16) of a half is its column 32 h + 2 s + f.
 *   w2:  block (e, kt, j), kt < I / 128, j < ceil(H / 128); block column n
 *        is weight column 128 j + n.
 *   The per-channel scales are not packed.
 * MOE_U8 / MOE_U4 codes: each block is 128 weight columns x 64 weight rows
 *   (K), 8 KiB of 8-bit or 4 KiB of 4-bit codes, in the order the GEMM's
 *   bf16 MFMA fragments read them: for column group f (16 columns), K half h
 *   (32 rows) and lane l = 16 a + c (column 16 f + c, rows 32 h + 8 a ..
 *   + 7), the lane's 8 codes are one 8-byte (U8: code i in byte i) or 4-byte
 *   (U4: code i in nibble i / 2 + 4 (i & 1) of the little-endian word, so
 *   bytes 0-3 hold codes (0, 2), (4, 6), (1, 3), (5, 7), low nibble first)
 *   run at offset ((2 f + h) * 64 + l) * 8 or * 4.
 *   w13: block (e, kt, j), kt < ceil(H / 64), j < ceil(I / 64), j fastest;
 *        block columns 0-63 are gate columns 64 j .., 64-127 up columns
 *        I + 64 j ...
 *   w2:  block (e, kt, j), kt < ceil(I / 64), j < ceil(H / 128); block
 *        column n is weight column 128 j + n.
 *   Scales and zero points are not packed.
 * In all, rows past H (w13) / I (w2) and columns past I (w13) / H (w2) are
 * zero.
 *
 * moe_packed_weight_bytes: sizes of the two packed buffers for *p (host
 * only).  Returns MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED (the
 * weights are not bf16, fp8, MOE_U8 or MOE_U4).
 * moe_pack_weights: enqueues the re-layout of w13 / w2 (plain layout, device
 * pointers) into w13_packed / w2_packed (device buffers of the sizes above,
 * caller-owned, must not overlap the inputs) on `stream`.  The forward then
 * takes w13_packed / w2_packed as w13 / w2 with p->w_layout = MOE_W_PACKED.
 * Errors as moe_packed_weight_bytes, MOE_ERR_INVALID_ARG for null pointers,
 * MOE_ERR_LAUNCH if a launch failed. */
int moe_packed_weight_bytes(const moe_problem* p, size_t* w13_bytes, size_t* w2_bytes);
int moe_pack_weights(const moe_problem* p, const void* w13, const void* w2, void* w13_packed,
                     void* w2_packed, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * or hand over a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The same path and results as
 * moe_forward, with the workspace in a device array that the library holds
 * on every GPU it runs on (MOE_STATIC_WORKSPACE_BYTES each, until the process
 * ends).  The caller passes inputs and outputs only; the call allocates and
 * frees nothing.  Its first call on a device looks up that device's copy of
 * the array (a symbol query with the stream's device made current, then
 * restored); later calls only launch kernels.
 *   - Problems whose workspace (moe_workspace_shapes) exceeds
 *     MOE_STATIC_WORKSPACE_BYTES return MOE_ERR_STATIC_LIMIT with nothing
 *     enqueued; chunk_tokens bounds the workspace of a long batch.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; no region needs to start at zero (each kernel writes
 *     what a later kernel of the same call reads).  Calls that overlap on
 *     one GPU (different streams, or different host threads) race on the
 *     array: serialise them.  The intermediates are not handed out.
 *   - Other errors as moe_forward; MOE_ERR_LAUNCH also when the array's
 *     device address cannot be obtained. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
int moe_forward_static(const moe_problem* p, const moe_args* a, void* stream);

/* Static English description of a status code. */
const char* moe_status_string(int status);

/* Library version, "major.minor.patch". */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
