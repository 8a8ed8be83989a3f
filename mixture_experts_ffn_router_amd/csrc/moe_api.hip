// C ABI of libmoe: argument validation, workspace layout, kernel sequence.
//
// Entry points and their constraints follow the MindIE-SD "Fused MoE" page
// (signature, parameter table, grouped-routing constraints) and the
// FlagGems walkthrough's parameter checks (fused_experts_impl, "parameter
// validation"); the workspace_shapes / apply split follows the vLLM
// "Fused MoE Modular Kernel" page.  All checks run on the host before
// anything is enqueued.
#include <atomic>
#include <cmath>
#include <mutex>

#include "moe_internal.h"

namespace moe {

static constexpr size_t ALIGN = 256;

static size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Tokens per pass of the contiguous forward (all M unless chunked).
static int chunk_rows(const moe_problem* p)
{
    return (p->chunk_tokens > 0 && p->chunk_tokens < p->M) ? p->chunk_tokens : p->M;
}

static int validate(const moe_problem* p)
{
    if (!p)
        return MOE_ERR_INVALID_ARG;
    if (p->format != MOE_FMT_CONTIGUOUS && p->format != MOE_FMT_BATCHED)
        return MOE_ERR_INVALID_ARG;
    if (p->M < 0 || p->H <= 0 || p->I <= 0 || p->E < 1 || p->top_k < 1)
        return MOE_ERR_INVALID_ARG;
    if (p->E > 1024)
        return MOE_ERR_UNSUPPORTED;
    if (p->top_k > (p->global_experts > p->E ? p->global_experts : p->E))
        return MOE_ERR_INVALID_ARG;          // top_k in [1, num_experts]
    if (p->top_k > 32)
        return MOE_ERR_UNSUPPORTED;
    if (p->H % 16 || p->I % 16)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)p->M * p->top_k >= (1ll << 30) || (int64_t)p->H * p->I >= (1ll << 40))
        return MOE_ERR_UNSUPPORTED;
    const int Er = p->global_experts > 0 ? p->global_experts : p->E;   // experts routed over

    // dtype combinations built here
    const int act = p->act_dtype, w = p->w_dtype, out = p->out_dtype;
    if (out != MOE_F32 && out != MOE_BF16)
        return MOE_ERR_UNSUPPORTED;
    if (act == MOE_F32) {
        if (w != MOE_F32 || out != MOE_F32)
            return MOE_ERR_UNSUPPORTED;
    } else if (act == MOE_BF16) {
        if (w != MOE_BF16 && w != MOE_FP8_E4M3FN && w != MOE_U8 && w != MOE_U4)
            return MOE_ERR_UNSUPPORTED;
    } else if (act == MOE_FP8_E4M3FN) {
        if (w != MOE_FP8_E4M3FN || p->format != MOE_FMT_BATCHED)
            return MOE_ERR_UNSUPPORTED;
    } else {
        return MOE_ERR_UNSUPPORTED;
    }
    if (w == MOE_FP8_E4M3FN && p->I % 128)
        return MOE_ERR_UNSUPPORTED;
    if (p->w_layout != MOE_W_PLAIN && p->w_layout != MOE_W_PACKED)
        return MOE_ERR_INVALID_ARG;
    if (p->w_layout == MOE_W_PACKED && w != MOE_BF16 && w != MOE_FP8_E4M3FN && w != MOE_U8 &&
        w != MOE_U4)
        return MOE_ERR_UNSUPPORTED;
    // WNA16 weights are dequantised inside the packed-layout GEMMs
    if ((w == MOE_U8 || w == MOE_U4) && p->w_layout != MOE_W_PACKED)
        return MOE_ERR_UNSUPPORTED;
    // block-wise fp8 scales: 128 x 128 weight blocks, on the packed fp8 kernels
    if (p->fp8_block < 0)
        return MOE_ERR_INVALID_ARG;
    if (p->fp8_block != 0 &&
        (p->fp8_block != 128 || w != MOE_FP8_E4M3FN || p->w_layout != MOE_W_PACKED))
        return MOE_ERR_UNSUPPORTED;

    // WNA16 scale groups of 32, 64 or 128 K rows (0: 128)
    if (p->wq_group != 0) {
        if (w != MOE_U8 && w != MOE_U4)
            return MOE_ERR_INVALID_ARG;
        if (p->wq_group != 32 && p->wq_group != 64 && p->wq_group != 128)
            return MOE_ERR_UNSUPPORTED;
    }

    // per-call tuning hints (tile family, GEMM1 width); 0 = the library's choice
    const int th = p->tile_hint;
    if (th != MOE_TILE_AUTO && th != MOE_TILE_DMA_160 && th != MOE_TILE_REG_64 &&
        th != MOE_TILE_REG_16 && th != MOE_TILE_DMA_32 && th != MOE_TILE_DMA_64 &&
        th != MOE_TILE_DMA_256)
        return MOE_ERR_INVALID_ARG;
    if (p->gemm1_wave_cols != 0 && p->gemm1_wave_cols != 2 && p->gemm1_wave_cols != 4)
        return MOE_ERR_INVALID_ARG;
    if (th != MOE_TILE_AUTO) {
        if (w != MOE_BF16 && w != MOE_U8 && w != MOE_U4)
            return MOE_ERR_UNSUPPORTED;
        if (w != MOE_BF16 &&
            (th == MOE_TILE_REG_64 || th == MOE_TILE_REG_16 || th == MOE_TILE_DMA_256))
            return MOE_ERR_UNSUPPORTED;   // WNA16 runs the 32 / 64 / 160-row DMA families
    }

    if (p->global_experts < 0 || p->chunk_tokens < 0 || p->apply_weight_on_input < 0 ||
        p->apply_weight_on_input > 1)
        return MOE_ERR_INVALID_ARG;
    if (p->global_experts > 0) {
        if (p->global_experts < p->E)
            return MOE_ERR_INVALID_ARG;
        if (p->global_experts > 1024)
            return MOE_ERR_UNSUPPORTED;
    }
    if (p->format == MOE_FMT_BATCHED) {
        // expert maps, input-side routing weights and chunking are contiguous-format features
        if (p->global_experts || p->apply_weight_on_input || p->chunk_tokens)
            return MOE_ERR_UNSUPPORTED;
        if (p->max_tokens < 1)
            return MOE_ERR_INVALID_ARG;
        if ((int64_t)p->E * p->max_tokens >= (1ll << 30))
            return MOE_ERR_UNSUPPORTED;
        if (p->batched_reduce != 0 && p->batched_reduce != 1)
            return MOE_ERR_INVALID_ARG;
        return MOE_OK;                        // routing happened upstream
    }

    if (p->routing != MOE_ROUTE_SOFTMAX && p->routing != MOE_ROUTE_SIGMOID &&
        p->routing != MOE_ROUTE_PRECOMPUTED)
        return MOE_ERR_INVALID_ARG;
    if (p->routing == MOE_ROUTE_PRECOMPUTED)
        return MOE_OK;
    if (p->logits_dtype != MOE_F32 && p->logits_dtype != MOE_BF16)
        return MOE_ERR_UNSUPPORTED;
    if (!std::isfinite(p->routed_scaling_factor))
        return MOE_ERR_INVALID_ARG;
    // grouped routing constraints (MindIE-SD page, routing-selection section)
    const int G = p->group_count, kg = p->k_group;
    if (G < 1 || kg < 1 || kg > G)
        return MOE_ERR_INVALID_ARG;
    if (Er % G)
        return MOE_ERR_INVALID_ARG;
    if (p->group_select_mode != 0 && p->group_select_mode != 1)
        return MOE_ERR_INVALID_ARG;
    if (G > 1) {
        if (G > 64)
            return MOE_ERR_UNSUPPORTED;
        if (p->top_k > kg * (Er / G))
            return MOE_ERR_INVALID_ARG;
        if (p->group_select_mode == 1 && Er / G < 2)
            return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

// GEMM tile family from the average rows per expert: decode-sized loads use
// 32-row DMA tiles, mid-sized loads 64-row tiles, prefill-sized loads 160-row
// tiles so that one tile holds a whole expert of about 128 rows.  A caller's
// tile_hint (validated above) forces the family.
static int choose_tile(const moe_problem* p, int64_t rows_cap)
{
    if (p->w_dtype == MOE_FP8_E4M3FN)
        return p->w_layout == MOE_W_PACKED ? TILE_FP8_DMA : TILE_FP8;
    if (p->w_dtype == MOE_F32)
        return TILE_DECODE;
    switch (p->tile_hint) {
    case MOE_TILE_DMA_160: return TILE_PREFILL;
    case MOE_TILE_REG_64: return TILE_MID;
    case MOE_TILE_REG_16: return TILE_DECODE;
    case MOE_TILE_DMA_32: return TILE_DECODE_DMA;
    case MOE_TILE_DMA_64: return TILE_MID_DMA;
    case MOE_TILE_DMA_256: return TILE_PREFILL_BIG;
    default: break;
    }
    const double avg = (double)rows_cap / p->E;
    if (p->w_dtype == MOE_U8 || p->w_dtype == MOE_U4)     // DMA families only
        return avg <= 12 ? TILE_DECODE_DMA : avg <= 48 ? TILE_MID_DMA : TILE_PREFILL;
    if (avg <= 12)
        return TILE_DECODE_DMA;
    if (avg <= 48)
        return TILE_MID;
    // a few hundred rows per expert or more: compute-bound, 256-row tiles
    return avg >= 384 ? TILE_PREFILL_BIG : TILE_PREFILL;
}

// Internal workspace regions beyond moe_workspace_info: chunk tables and the
// position of every routed item in the sorted order.
enum { INT_CHUNK_OFF = 0, INT_CHUNK_EXPERT = 1, INT_INV = 2, INT_O2 = 3, INT_REGIONS = 4 };

// Workspace layout of problem p on a device with `cus` compute units (the
// GEMM2 K-split choice, and so the o2 region, depends on it).
static int layout(const moe_problem* p, int cus, moe_workspace_info* info,
                  size_t* chunk_offs = nullptr, int* cfg_out = nullptr)
{
    size_t off_chunk_off = 0, off_chunk_expert = 0, off_inv = 0, off_o2 = 0;
    const int rc = validate(p);
    if (rc != MOE_OK)
        return rc;
    moe_workspace_info w{};
    const bool batched = p->format == MOE_FMT_BATCHED;
    const int64_t MK = (int64_t)chunk_rows(p) * p->top_k;
    int64_t rows_cap = MK;
    if (batched) {
        rows_cap = (int64_t)p->E * p->max_tokens;
        // M > 0 promises at most M * top_k valid slab rows (each one routed
        // copy of a token); the tile-list kernel checks the promise on the device
        if (p->M > 0 && MK < rows_cap)
            rows_cap = MK;
    }
    const int BM = ALIGN_BM;
    const int64_t max_sorted = rows_cap + (int64_t)p->E * (BM - 1);
    const bool fp8 = p->w_dtype == MOE_FP8_E4M3FN;
    const int zes = fp8 ? 1 : (p->act_dtype == MOE_F32 ? 4 : 2);

    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    w.block_m = BM;
    w.max_sorted_len = max_sorted;
    w.max_blocks = (int32_t)(max_sorted / BM);
    w.off_topk_ids = take(batched ? 0 : MK * 4);
    w.off_topk_weights = take(batched ? 0 : MK * 4);
    w.off_expert_counts = take((size_t)p->E * 4);
    w.off_expert_offsets = take((size_t)(p->E + 1) * 4);
    w.off_sorted_ids = take((size_t)max_sorted * 4);
    w.off_expert_ids = take((size_t)w.max_blocks * 4);
    w.off_num_post_padded = take(4);
    w.off_status = take(4);
    off_chunk_off = take((size_t)(p->E + 1) * 4);
    off_chunk_expert = take((size_t)w.max_blocks * 4);
    off_inv = take(batched ? 0 : (size_t)MK * 4);
    const bool quant = fp8 && p->act_dtype != MOE_FP8_E4M3FN;
    const int64_t qrows = batched ? max_sorted : chunk_rows(p);
    w.off_aq = take(quant ? (size_t)qrows * p->H : 0);
    // one scale per row, or per row and 128 columns (block-wise)
    const int64_t qgroups = p->fp8_block ? (p->H + 127) / 128 : 1;
    w.off_aq_scale = take(quant ? (size_t)qrows * qgroups * 4 : 0);
    w.off_z = take((size_t)max_sorted * p->I * zes);
    // fp8 z scales, group-major: [I/128][zs_ld]; the row padding lets a GEMM
    // tile read the scales of all its rows as one block
    w.off_z_scale = take(fp8 ? (size_t)zs_ld(max_sorted) * (p->I / 128) * 4 : 0);
    const int64_t orows = (batched && !p->batched_reduce) ? 0 : max_sorted;
    w.off_o = take((size_t)orows * p->H * 4);
    const int cfg = choose_tile(p, rows_cap);
    // (WNA16 GEMM2 runs whole-K tiles)
    const bool split = p->w_dtype != MOE_U8 && p->w_dtype != MOE_U4 && gemm2_k_split(
        cfg, p->format, p->batched_reduce,
        expected_chunks(p->format, chunk_rows(p), p->top_k, p->E, p->max_tokens, tile_rows(cfg)),
        p->H, p->I, cus);
    off_o2 = take(split ? (size_t)orows * p->H * 4 : 0);
    w.off_o2 = split ? off_o2 : 0;
    w.bytes = off;
    *info = w;
    if (chunk_offs) {
        chunk_offs[INT_CHUNK_OFF] = off_chunk_off;
        chunk_offs[INT_CHUNK_EXPERT] = off_chunk_expert;
        chunk_offs[INT_INV] = off_inv;
        chunk_offs[INT_O2] = split ? off_o2 : 0;
    }
    if (cfg_out)
        *cfg_out = cfg;
    return MOE_OK;
}

static Plan make_plan(const moe_problem* p, const moe_workspace_info& w, char* ws,
                      const size_t* chunk_offs, int cfg)
{
    Plan P{};
    P.fmt = p->format;
    P.M = chunk_rows(p);
    P.Er = p->global_experts > 0 ? p->global_experts : p->E;
    P.w_on_input = p->apply_weight_on_input ? 1 : 0;
    P.H = p->H;
    P.I = p->I;
    P.E = p->E;
    P.K = p->top_k;
    P.T = p->max_tokens;
    P.act = p->act_dtype;
    P.wdt = p->w_dtype;
    P.outdt = p->out_dtype;
    P.lgdt = p->logits_dtype;
    P.routing = p->routing;
    P.renorm = p->renormalize ? 1 : 0;
    P.G = p->group_count < 1 ? 1 : p->group_count;
    P.kg = p->k_group;
    P.gmode = p->group_select_mode;
    P.rsf = p->routed_scaling_factor;
    P.has_b13 = p->has_w13_bias ? 1 : 0;
    P.has_b2 = p->has_w2_bias ? 1 : 0;
    P.breduce = p->batched_reduce ? 1 : 0;
    P.wpacked = p->w_layout == MOE_W_PACKED ? 1 : 0;
    P.blk = p->fp8_block ? 1 : 0;
    P.wq = (p->w_dtype == MOE_U8) ? 8 : (p->w_dtype == MOE_U4) ? 4 : 0;
    P.wq_gsh = (p->wq_group == 32) ? 0 : (p->wq_group == 64) ? 1 : 2;
    P.BM = w.block_m;
    P.cfg = cfg;
    P.g1wc = p->gemm1_wave_cols;
    P.CH = tile_rows(cfg);
    P.chunk_off = (int32_t*)(ws + chunk_offs[INT_CHUNK_OFF]);
    P.chunk_expert = (int32_t*)(ws + chunk_offs[INT_CHUNK_EXPERT]);
    P.inv = (int32_t*)(ws + chunk_offs[INT_INV]);
    P.max_sorted = w.max_sorted_len;
    P.max_blocks = w.max_blocks;
    P.rows_cap = w.max_sorted_len - (int64_t)p->E * (w.block_m - 1);
    P.sentinel = (p->format == MOE_FMT_BATCHED) ? (int64_t)p->E * p->max_tokens
                                                 : (int64_t)P.M * p->top_k;
    P.topk_ids = (int32_t*)(ws + w.off_topk_ids);
    P.topk_w = (float*)(ws + w.off_topk_weights);
    P.counts = (int32_t*)(ws + w.off_expert_counts);
    P.offsets = (int32_t*)(ws + w.off_expert_offsets);
    P.sorted_ids = (int32_t*)(ws + w.off_sorted_ids);
    P.expert_ids = (int32_t*)(ws + w.off_expert_ids);
    P.npp = (int32_t*)(ws + w.off_num_post_padded);
    P.aq = (uint8_t*)(ws + w.off_aq);
    P.aq_scale = (float*)(ws + w.off_aq_scale);
    P.z = ws + w.off_z;
    P.z_scale = (float*)(ws + w.off_z_scale);
    P.zs_ld = zs_ld(w.max_sorted_len);
    P.o = (float*)(ws + w.off_o);
    P.g2split = chunk_offs[INT_O2] != 0;
    P.o2 = P.g2split ? (float*)(ws + chunk_offs[INT_O2]) : nullptr;
    P.status = (int32_t*)(ws + w.off_status);
    P.status_or = 0;
    return P;
}

static int check_args(const moe_problem* p, const moe_args* a)
{
    if (!a || !a->w13 || !a->w2)
        return MOE_ERR_INVALID_ARG;
    // a contiguous forward of no tokens touches no token array (they have no
    // rows and may be null)
    const bool no_tokens = p->format == MOE_FMT_CONTIGUOUS && p->M == 0;
    if (!no_tokens && (!a->out || !a->hidden))
        return MOE_ERR_INVALID_ARG;
    if ((p->has_w13_bias && !a->w13_bias) || (p->has_w2_bias && !a->w2_bias))
        return MOE_ERR_INVALID_ARG;
    if ((p->w_dtype == MOE_FP8_E4M3FN || p->w_dtype == MOE_U8 || p->w_dtype == MOE_U4) &&
        (!a->w13_scale || !a->w2_scale))
        return MOE_ERR_INVALID_ARG;
    // zero points of WNA16 weights: both or neither
    if ((p->w_dtype == MOE_U8 || p->w_dtype == MOE_U4) && (!a->w13_zero != !a->w2_zero))
        return MOE_ERR_INVALID_ARG;
    if (p->act_dtype == MOE_FP8_E4M3FN && !a->a_scale)
        return MOE_ERR_INVALID_ARG;
    if (p->format == MOE_FMT_BATCHED) {
        if (!a->expert_num_tokens)
            return MOE_ERR_INVALID_ARG;
        if (p->batched_reduce && (!a->token_map || !a->token_map_w))
            return MOE_ERR_INVALID_ARG;
        return MOE_OK;
    }
    if (p->global_experts > 0 && !a->expert_map)
        return MOE_ERR_INVALID_ARG;
    if (no_tokens)
        return MOE_OK;
    if (p->routing == MOE_ROUTE_PRECOMPUTED) {
        if (!a->topk_ids || !a->topk_weights)
            return MOE_ERR_INVALID_ARG;
    } else if (!a->router_logits) {
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_workspace_shapes(const moe_problem* p, moe_workspace_info* info)
{
    if (!info)
        return MOE_ERR_INVALID_ARG;
    int dev = 0;
    (void)hipGetDevice(&dev);
    return layout(p, device_cus(dev), info);
}

static int run_path(const moe_problem* p, const Plan& P, const moe_args& A, hipStream_t s,
                    void** events);

static int forward(const moe_problem* p, const moe_args* a, void* workspace,
                   size_t workspace_bytes, void* stream, void** events)
{
    moe_workspace_info w;
    size_t chunk_offs[INT_REGIONS];
    int cfg = 0;
    const hipStream_t s = (hipStream_t)stream;
    const int dev = stream_device(s), cus = device_cus(dev);
    int rc = layout(p, cus, &w, chunk_offs, &cfg);
    if (rc != MOE_OK)
        return rc;
    rc = check_args(p, a);
    if (rc != MOE_OK)
        return rc;
    if (!workspace || ((uintptr_t)workspace % ALIGN) || workspace_bytes < w.bytes)
        return MOE_ERR_WORKSPACE;

    Plan P = make_plan(p, w, (char*)workspace, chunk_offs, cfg);
    P.dev = dev;
    P.cus = cus;
    P.emap = a->expert_map;
    const bool batched = p->format == MOE_FMT_BATCHED;
    if (!batched && p->M == 0)
        return MOE_OK;                                   // nothing routed
    if (batched && p->batched_reduce && p->M == 0)
        return MOE_OK;

    // hipGetLastError reports the calling thread's last runtime error, which
    // may come from an unrelated earlier call of the caller; clear it so the
    // checks below see only this call's launches
    (void)hipGetLastError();
    if (batched || P.M == p->M)
        return run_path(p, P, *a, s, events);
    // chunked contiguous forward: the same path over token rows [c0, c0 + n)
    const size_t aes = p->act_dtype == MOE_F32 ? 4 : 2;
    const size_t oes = p->out_dtype == MOE_F32 ? 4 : 2;
    const size_t les = p->logits_dtype == MOE_F32 ? 4 : 2;
    for (int c0 = 0; c0 < p->M; c0 += P.M) {
        Plan Pc = P;
        Pc.M = (p->M - c0 < P.M) ? p->M - c0 : P.M;
        Pc.status_or = c0 > 0;            // later chunks add their findings
        moe_args ac = *a;
        ac.hidden = (const char*)a->hidden + (size_t)c0 * p->H * aes;
        ac.out = (char*)a->out + (size_t)c0 * p->H * oes;
        if (p->routing == MOE_ROUTE_PRECOMPUTED) {
            ac.topk_ids = a->topk_ids + (size_t)c0 * p->top_k;
            ac.topk_weights = a->topk_weights + (size_t)c0 * p->top_k;
        } else {
            ac.router_logits = (const char*)a->router_logits + (size_t)c0 * P.Er * les;
        }
        const int rc2 = run_path(p, Pc, ac, s, events);
        if (rc2 != MOE_OK)
            return rc2;
    }
    return MOE_OK;
}

// The kernel sequence of one pass (P.M tokens of the contiguous format, or
// the batched slabs).
static int run_path(const moe_problem* p, const Plan& P, const moe_args& A, hipStream_t s,
                    void** events)
{
    const moe_args* a = &A;
    const bool batched = p->format == MOE_FMT_BATCHED;
    hipError_t err;
    int stage = 0;
    auto mark = [&](int st, int end) {
        if (events && events[2 * st + end])
            (void)hipEventRecord((hipEvent_t)events[2 * st + end], s);
    };
#define MOE_TRY(st, call)              \
    do {                               \
        stage = (st);                  \
        mark(stage, 0);                \
        err = (call);                  \
        mark(stage, 1);                \
        if (err != hipSuccess)         \
            return MOE_ERR_LAUNCH;     \
    } while (0)

    const float* weights = nullptr;
    if (!batched) {
        const int32_t* ids;
        if (p->routing == MOE_ROUTE_PRECOMPUTED) {
            ids = a->topk_ids;
            weights = a->topk_weights;
            MOE_TRY(MOE_STAGE_ALIGN, launch_align(P, ids, s));
        } else {
            MOE_TRY(MOE_STAGE_ROUTER, launch_router(P, a->router_logits, s));
            ids = P.topk_ids;
            weights = P.topk_w;
            MOE_TRY(MOE_STAGE_ALIGN, launch_align(P, ids, s));
        }
    } else {
        MOE_TRY(MOE_STAGE_ALIGN, launch_tilelist(P, a->expert_num_tokens, s));
    }
    if (p->w_dtype == MOE_FP8_E4M3FN && p->act_dtype != MOE_FP8_E4M3FN)
        MOE_TRY(MOE_STAGE_QUANT, launch_quant_rows(P, a->hidden, s));
    MOE_TRY(MOE_STAGE_GEMM1, launch_gemm1(P, *a, P.w_on_input ? weights : nullptr, s));
    MOE_TRY(MOE_STAGE_GEMM2, launch_gemm2(P, *a, s));
    if (!batched || p->batched_reduce)
        MOE_TRY(MOE_STAGE_REDUCE, launch_reduce(P, *a, P.w_on_input ? nullptr : weights, s));
#undef MOE_TRY
    (void)stage;
    return MOE_OK;
}

extern "C" int moe_forward(const moe_problem* p, const moe_args* a, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    return forward(p, a, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int moe_forward_timed(const moe_problem* p, const moe_args* a, void* workspace,
                                 size_t workspace_bytes, void* stream, void** events)
{
    return forward(p, a, workspace, workspace_bytes, stream, events);
}

// ---------------------------------------------------------------- allocation-free forward
// The workspace of moe_forward_static: one array per device, loaded with the
// library's code object.  Host code never uses its name as an address (on
// the host it is only a handle); the device address comes from a symbol
// query, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];

static std::atomic<void*> g_scratch[MAX_DEVICES];
static std::mutex g_scratch_mu;

// Device address of `scratch` on device dev (queried on first use).
static int scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= MAX_DEVICES)
        return MOE_ERR_UNSUPPORTED;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            int prev = -1;
            if (hipGetDevice(&prev) != hipSuccess || (prev != dev && hipSetDevice(dev) != hipSuccess)) {
                (void)hipGetLastError();
                return MOE_ERR_LAUNCH;
            }
            const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (prev != dev)
                (void)hipSetDevice(prev);
            if (e != hipSuccess || !ptr || (uintptr_t)ptr % ALIGN) {
                (void)hipGetLastError();
                return MOE_ERR_LAUNCH;
            }
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return MOE_OK;
}

extern "C" int moe_forward_static(const moe_problem* p, const moe_args* a, void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    const int dev = stream_device(s);
    moe_workspace_info w;
    int rc = layout(p, device_cus(dev), &w);
    if (rc != MOE_OK)
        return rc;
    rc = check_args(p, a);
    if (rc != MOE_OK)
        return rc;
    if (w.bytes > MOE_STATIC_WORKSPACE_BYTES)
        return MOE_ERR_STATIC_LIMIT;
    void* ws = nullptr;
    rc = scratch_address(dev, &ws);
    if (rc != MOE_OK)
        return rc;
    return forward(p, a, ws, MOE_STATIC_WORKSPACE_BYTES, stream, nullptr);
}

// Packed weight sizes: 16 KiB blocks.  bf16: 64 weight rows x 128 weight
// columns (w13: 64 gate + 64 up columns per block); fp8: 128 weight columns x
// 128 K values (w13: 64 gate + 64 up columns).
static int packed_sizes(const moe_problem* p, size_t* b13, size_t* b2)
{
    if (!p)
        return MOE_ERR_INVALID_ARG;
    // the sizes do not depend on the layout the problem names (a caller may
    // size the packed buffers from the problem of the plain weights)
    moe_problem q = *p;
    q.w_layout = MOE_W_PACKED;
    const int rc = validate(&q);
    if (rc != MOE_OK)
        return rc;
    const size_t blk = 64 * 256;
    if (p->w_dtype == MOE_BF16) {
        *b13 = (size_t)p->E * ((p->I + 63) / 64) * ((p->H + 63) / 64) * blk;
        *b2 = (size_t)p->E * ((p->H + 127) / 128) * ((p->I + 63) / 64) * blk;
        return MOE_OK;
    }
    if (p->w_dtype == MOE_FP8_E4M3FN) {          // I is a multiple of 128 (validated)
        *b13 = (size_t)p->E * (p->I / 64) * ((p->H + 127) / 128) * blk;
        *b2 = (size_t)p->E * ((p->H + 127) / 128) * (p->I / 128) * blk;
        return MOE_OK;
    }
    if (p->w_dtype == MOE_U8 || p->w_dtype == MOE_U4) {   // 128 columns x 64 K codes a block
        const size_t qb = (p->w_dtype == MOE_U8) ? 8192 : 4096;
        *b13 = (size_t)p->E * ((p->H + 63) / 64) * ((p->I + 63) / 64) * qb;
        *b2 = (size_t)p->E * ((p->I + 63) / 64) * ((p->H + 127) / 128) * qb;
        return MOE_OK;
    }
    return MOE_ERR_UNSUPPORTED;
}

extern "C" int moe_packed_weight_bytes(const moe_problem* p, size_t* w13_bytes, size_t* w2_bytes)
{
    if (!w13_bytes || !w2_bytes)
        return MOE_ERR_INVALID_ARG;
    return packed_sizes(p, w13_bytes, w2_bytes);
}

extern "C" int moe_pack_weights(const moe_problem* p, const void* w13, const void* w2,
                                void* w13_packed, void* w2_packed, void* stream)
{
    size_t b13 = 0, b2 = 0;
    const int rc = packed_sizes(p, &b13, &b2);
    if (rc != MOE_OK)
        return rc;
    if (!w13 || !w2 || !w13_packed || !w2_packed)
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();   // a stale error of an earlier, unrelated call
    hipError_t err;
    if (p->w_dtype == MOE_FP8_E4M3FN)
        err = launch_pack_weights_fp8(p->E, p->H, p->I, w13, w2, w13_packed, w2_packed,
                                      (hipStream_t)stream);
    else if (p->w_dtype == MOE_U8 || p->w_dtype == MOE_U4)
        err = launch_pack_weights_wq(p->w_dtype == MOE_U8 ? 8 : 4, p->E, p->H, p->I, w13, w2,
                                     w13_packed, w2_packed, (hipStream_t)stream);
    else
        err = launch_pack_weights(p->E, p->H, p->I, w13, w2, w13_packed, w2_packed,
                                  (hipStream_t)stream);
    return err == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

extern "C" int moe_repack_wna16(int format, int bits, int E, int K, int N, int group,
                                const int32_t* qweight, const int32_t* qzeros, int zero_adjust,
                                uint8_t* codes, uint8_t* zeros, void* stream)
{
    if (format != MOE_WQ_GPTQ && format != MOE_WQ_AWQ)
        return MOE_ERR_UNSUPPORTED;
    if ((bits != 4 && bits != 8) || (format == MOE_WQ_AWQ && bits != 4))
        return MOE_ERR_UNSUPPORTED;
    if (group != 32 && group != 64 && group != 128)
        return MOE_ERR_UNSUPPORTED;
    if (E < 1 || K < 1 || N < 1 || !qweight || !codes || (qzeros && !zeros))
        return MOE_ERR_INVALID_ARG;
    const int per = 32 / bits;
    if ((format == MOE_WQ_GPTQ && K % per) || (format == MOE_WQ_AWQ && N % 8) ||
        (qzeros && N % per) || (bits == 4 && N % 2))
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();   // a stale error of an earlier, unrelated call
    const hipError_t e = launch_repack_wq(format, bits, E, K, N, (K + group - 1) / group, qweight,
                                          qzeros, zero_adjust, codes, zeros, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

extern "C" const char* moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "success";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_STATIC_LIMIT: return "problem needs more workspace than the static array holds";
    default: return "unknown status";
    }
}

extern "C" const char* moe_version(void) { return CHECKED ? "0.1.0 checked" : "0.1.0"; }
