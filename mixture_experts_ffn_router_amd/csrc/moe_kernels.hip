// Bandwidth kernels of the fused MoE forward for gfx950: router (top-k),
// align (permute metadata), batched tile list, per-row fp8 quantisation and
// the top-k weight-and-reduce (unpermute).  None of them uses MFMA.
#include "moe_internal.h"

namespace moe {

// ============================================================ router
// Routing of the MindIE-SD "Fused MoE" page (routing-selection section and
// parameter table): scores by softmax or sigmoid, optional grouped selection
// (k_group of group_count contiguous groups, keyed by the group's largest
// score or by the sum of its two largest), top-k inside the chosen groups,
// renormalisation, routed_scaling_factor.  Expert and group choices compare
// logits (softmax / sigmoid are strictly increasing) with ties to the lower
// index, so they are exact; only the mode-1 group key needs the score values,
// and it is formed as float32(score_a) + float32(score_b) with each score
// evaluated in double and rounded once.
//
// One wavefront per token; lane l holds experts [l*EPL, (l+1)*EPL).

// Orders float bit patterns as unsigned integers (monotone for non-NaN).
__device__ __forceinline__ uint32_t ord_f32(float f)
{
    uint32_t u = __float_as_uint(f + 0.0f);   // -0 -> +0: equal logits tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int EPL>
__global__ void __launch_bounds__(256) k_router(const void* __restrict__ logits, int lgdt, int M,
                                                int E, int K, int scoring, int renorm, int G,
                                                int kg, int gmode, float rsf,
                                                int32_t* __restrict__ topk_ids,
                                                float* __restrict__ topk_w)
{
    __shared__ float sh_logit[4][EPL * 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= M)
        return;

    float s[EPL];
    bool valid[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        valid[i] = e < E;
        float v = -INFINITY;
        if (valid[i])
            v = (lgdt == MOE_BF16) ? bf16_to_f32(((const u16*)logits)[(int64_t)t * E + e])
                                   : ((const float*)logits)[(int64_t)t * E + e];
        s[i] = v;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        mx = fmaxf(mx, s[i]);
    mx = wave_max(mx);

    float p[EPL];
    if (scoring == MOE_ROUTE_SOFTMAX) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            p[i] = valid[i] ? expf(s[i] - mx) : 0.0f;
            sum += p[i];
        }
        sum = wave_sum(sum);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            p[i] = p[i] / sum;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            p[i] = 1.0f / (1.0f + expf(-s[i]));
    }

    bool cand[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        cand[i] = valid[i];

    if (G > 1) {
        const int per = E / G;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (valid[i])
                sh_logit[wave][lane * EPL + i] = s[i];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        // lane g < G forms the key of group g
        unsigned long long gkey = 0;
        if (lane < G) {
            const float* sg = &sh_logit[wave][lane * per];
            float a = -INFINITY, b = -INFINITY;
            for (int i = 0; i < per; ++i) {
                const float v = sg[i];
                if (v > a) {
                    b = a;
                    a = v;
                } else if (v > b) {
                    b = v;
                }
            }
            float key;
            if (gmode == 0) {
                key = a;
            } else if (scoring == MOE_ROUTE_SIGMOID) {
                key = (float)(1.0 / (1.0 + exp(-(double)a))) + (float)(1.0 / (1.0 + exp(-(double)b)));
            } else {
                key = (float)exp((double)a - (double)mx) + (float)exp((double)b - (double)mx);
            }
            gkey = ((unsigned long long)ord_f32(key) << 32) | (uint32_t)(0xffffffffu - lane);
        }
        unsigned long long chosen = 0;
        for (int r = 0; r < kg; ++r) {
            const unsigned long long best = wave_max_u64(gkey);
            const int g = (int)(0xffffffffu - (uint32_t)best);
            chosen |= 1ull << g;
            if (lane == g)
                gkey = 0;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            cand[i] = valid[i] && ((chosen >> ((lane * EPL + i) / per)) & 1ull);
    }

    // top-k by (logit desc, index asc)
    float wsel = 0.0f;   // lane j keeps the score of the j-th pick
    int idsel = 0;
    for (int j = 0; j < K; ++j) {
        unsigned long long mine = 0;
        float pmine = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (cand[i]) {
                const unsigned long long k = ((unsigned long long)ord_f32(s[i]) << 32) |
                                             (uint32_t)(0xffffffffu - (lane * EPL + i));
                if (k > mine) {
                    mine = k;
                    pmine = p[i];
                }
            }
        }
        const unsigned long long best = wave_max_u64(mine);
        const int e = (int)(0xffffffffu - (uint32_t)best);
        const int owner = e / EPL;
        const float pe = __shfl(pmine, owner, 64);
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane * EPL + i == e)
                    cand[i] = false;
        }
        if (lane == j) {
            wsel = pe;
            idsel = e;
        }
    }
    if ((scoring == MOE_ROUTE_SOFTMAX && renorm) || scoring == MOE_ROUTE_SIGMOID) {
        const float tot = wave_sum(lane < K ? wsel : 0.0f);
        wsel = wsel / tot;
    }
    if (lane < K) {
        topk_ids[(int64_t)t * K + lane] = idsel;
        topk_w[(int64_t)t * K + lane] = wsel * rsf;
    }
}

hipError_t launch_router(const Plan& P, const void* logits, hipStream_t s)
{
    const dim3 grid((P.M + 3) / 4), block(256);
    const int scoring = P.routing;
#define MOE_ROUTER(EPL)                                                                          \
    hipLaunchKernelGGL(k_router<EPL>, grid, block, 0, s, logits, P.lgdt, P.M, P.E, P.K, scoring, \
                       P.renorm, P.G, P.kg, P.gmode, P.rsf, P.topk_ids, P.topk_w)
    if (P.E <= 64)
        MOE_ROUTER(1);
    else if (P.E <= 128)
        MOE_ROUTER(2);
    else if (P.E <= 256)
        MOE_ROUTER(4);
    else if (P.E <= 512)
        MOE_ROUTER(8);
    else
        MOE_ROUTER(16);
#undef MOE_ROUTER
    return hipGetLastError();
}

// ============================================================ align
// moe_align_block_size of the FlagGems walkthrough ("moe_align_block_size"
// section): group the M*top_k routed items by expert, pad each expert's run
// to a multiple of BM.  Items keep ascending order inside an expert (a stable
// sort, as the MoonEP page's build_permutation), so the result is unique and
// independent of scheduling.  One workgroup of 16 waves; each wave owns a
// contiguous chunk of items.  Equal-expert lanes of a wave are matched with
// ballots over the id bits, which gives each item its rank without atomics.

constexpr int ALIGN_WAVES = 16;
constexpr int ALIGN_UNROLL = 16;   // 64-item steps loaded per batch

__device__ __forceinline__ unsigned long long match_mask(int e, bool valid, int nbits)
{
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// exclusive scan of v over the 1024 threads of the block; returns the total
__device__ int block_exclusive_scan_1024(int v, int* sh_tot, int* out_prefix)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(incl, o, 64);
        if (lane >= o)
            incl += n;
    }
    if (lane == 63)
        sh_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < ALIGN_WAVES; ++w) {
        const int tw = sh_tot[w];
        if (w < wave)
            base += tw;
        total += tw;
    }
    *out_prefix = base + incl - v;
    return total;
}


// GEMM work unit lists: expert e's padded run is cut into chunks of CH rows
// (the row height of one GEMM tile).  chunk_off[e] = chunks of experts < e,
// chunk_off[E] = all chunks, chunk_expert[c] = expert of chunk c.  Called by
// all 1024 threads; `padded` is this thread's expert run (0 for e >= E).
__device__ void write_chunks(int padded, int CH, int E, int* sh_tot, int32_t* chunk_off,
                             int32_t* chunk_expert)
{
    const int e = threadIdx.x;
    __syncthreads();   // sh_tot is reused from the previous scan
    const int nch = (e < E) ? (padded + CH - 1) / CH : 0;
    int cstart;
    const int ctotal = block_exclusive_scan_1024(nch, sh_tot, &cstart);
    if (e < E) {
        chunk_off[e] = cstart;
        for (int j = 0; j < nch; ++j)
            chunk_expert[cstart + j] = e;
    }
    if (e == 0)
        chunk_off[E] = ctotal;
}

__global__ void __launch_bounds__(1024) k_align(const int32_t* __restrict__ ids, int Mk, int E,
                                                int BM, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted,
                                                int32_t* __restrict__ expert_ids,
                                                int32_t* __restrict__ npp, int sentinel,
                                                int64_t max_sorted, int max_blocks, int CH,
                                                int32_t* __restrict__ chunk_off,
                                                int32_t* __restrict__ chunk_expert,
                                                int32_t* __restrict__ inv)
{
    extern __shared__ int sh[];
    int* cnt = sh;                               // [ALIGN_WAVES][E]
    int* offs = sh + ALIGN_WAVES * E;            // [E]
    int* tot = offs + E;                         // [ALIGN_WAVES]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
    const int chunk = ((Mk + ALIGN_WAVES - 1) / ALIGN_WAVES + 63) / 64 * 64;
    const int beg = wave * chunk, end = min(Mk, beg + chunk);

    for (int i = threadIdx.x; i < ALIGN_WAVES * E; i += blockDim.x)
        cnt[i] = 0;
    __syncthreads();

    // pass 1: per-wave, per-expert counts
    for (int b0 = beg; b0 < end; b0 += 64 * ALIGN_UNROLL) {
        int ev[ALIGN_UNROLL];
#pragma unroll
        for (int u = 0; u < ALIGN_UNROLL; ++u) {
            const int r = b0 + u * 64 + lane;
            ev[u] = (r < end) ? ids[r] : -1;
            if (ev[u] >= E)
                ev[u] = -1;
        }
#pragma unroll
        for (int u = 0; u < ALIGN_UNROLL; ++u) {
            const bool valid = ev[u] >= 0;
            const unsigned long long m = match_mask(ev[u], valid, nbits);
            if (valid && lane == (int)__builtin_ctzll(m))
                cnt[wave * E + ev[u]] += __popcll(m);
        }
    }
    __syncthreads();

    // per-expert totals, wave prefixes, padded offsets
    int run = 0, padded = 0;
    const int e = threadIdx.x;
    if (e < E) {
        for (int w = 0; w < ALIGN_WAVES; ++w) {
            const int c = cnt[w * E + e];
            cnt[w * E + e] = run;
            run += c;
        }
        padded = (run + BM - 1) / BM * BM;
    }
    int start;
    const int total = block_exclusive_scan_1024(padded, tot, &start);
    if (e < E) {
        counts[e] = run;
        offsets[e] = start;
        offs[e] = start;
        for (int b = start / BM; b < (start + padded) / BM && b < max_blocks; ++b)
            expert_ids[b] = e;
        for (int q = start + run; q < start + padded && q < max_sorted; ++q)
            sorted[q] = sentinel;
    }
    if (threadIdx.x == 0) {
        offsets[E] = total;
        *npp = total;
    }
    write_chunks(padded, CH, E, tot, chunk_off, chunk_expert);
    __syncthreads();

    // pass 2: stable scatter
    for (int b0 = beg; b0 < end; b0 += 64 * ALIGN_UNROLL) {
        int ev[ALIGN_UNROLL];
#pragma unroll
        for (int u = 0; u < ALIGN_UNROLL; ++u) {
            const int r = b0 + u * 64 + lane;
            ev[u] = (r < end) ? ids[r] : -1;
            if (ev[u] >= E)
                ev[u] = -1;
        }
#pragma unroll
        for (int u = 0; u < ALIGN_UNROLL; ++u) {
            const bool valid = ev[u] >= 0;
            const unsigned long long m = match_mask(ev[u], valid, nbits);
            const int r = b0 + u * 64 + lane;
            if (valid) {
                const int rank = __popcll(m & ((1ull << lane) - 1ull));
                const int base = offs[ev[u]] + cnt[wave * E + ev[u]];
                const int64_t pos = (int64_t)base + rank;
                if (pos < max_sorted)
                    sorted[pos] = r;
                inv[r] = (pos < max_sorted) ? (int)pos : -1;
            } else if (r < end) {
                inv[r] = -1;                        // expert id out of range: no row
            }
            // every lane has read its base before the leader moves it on
            __builtin_amdgcn_wave_barrier();
            if (valid && lane == (int)__builtin_ctzll(m))
                cnt[wave * E + ev[u]] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

hipError_t launch_align(const Plan& P, const int32_t* ids, hipStream_t s)
{
    const size_t lds = sizeof(int) * ((size_t)ALIGN_WAVES * P.E + P.E + ALIGN_WAVES);
    hipLaunchKernelGGL(k_align, dim3(1), dim3(1024), lds, s, ids, P.M * P.K, P.E, P.BM, P.counts,
                       P.offsets, P.sorted_ids, P.expert_ids, P.npp, (int)P.sentinel, P.max_sorted,
                       P.max_blocks, P.CH, P.chunk_off, P.chunk_expert, P.inv);
    return hipGetLastError();
}

// ============================================================ batched tile list
// Batched format (vLLM "Fused MoE Modular Kernel" introduction): slab e holds
// expert_num_tokens[e] valid rows.  Builds the same metadata as align with
// item r = e*max_tokens + i, so the GEMMs are shared by both formats.  Counts
// beyond max_tokens are clamped, and runs that would pass the workspace
// capacity are dropped, so a bad count can never drive an access out of bounds.
__global__ void __launch_bounds__(1024) k_tilelist(const int32_t* __restrict__ ent, int E, int T,
                                                   int BM, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted,
                                                   int32_t* __restrict__ expert_ids,
                                                   int32_t* __restrict__ npp, int sentinel,
                                                   int64_t max_sorted, int max_blocks, int CH,
                                                   int32_t* __restrict__ chunk_off,
                                                   int32_t* __restrict__ chunk_expert)
{
    __shared__ int tot[ALIGN_WAVES];
    __shared__ int sh_start[1024], sh_cnt[1024];
    const int e = threadIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int c = 0, padded = 0;
    if (e < E) {
        c = min(max(ent[e], 0), T);
        padded = (c + BM - 1) / BM * BM;
    }
    int start;
    const int total = block_exclusive_scan_1024(padded, tot, &start);
    // more rows than the workspace was sized for: process nothing
    const bool fits = (int64_t)total <= max_sorted && total / BM <= max_blocks;
    if (e < E) {
        counts[e] = c;
        offsets[e] = fits ? start : 0;
        sh_start[e] = start;
        sh_cnt[e] = c;
        if (fits)
            for (int b = start / BM; b < (start + padded) / BM; ++b)
                expert_ids[b] = e;
    }
    if (threadIdx.x == 0) {
        offsets[E] = fits ? total : 0;
        *npp = fits ? total : 0;
    }
    write_chunks(fits ? padded : 0, CH, E, tot, chunk_off, chunk_expert);
    if (!fits)
        return;
    __syncthreads();
    // each wave fills the runs of experts wave, wave+16, ...
    for (int x = wave; x < E; x += ALIGN_WAVES) {
        const int st = sh_start[x], cx = sh_cnt[x];
        const int pe = (cx + BM - 1) / BM * BM;
        for (int i = lane; i < pe; i += 64)
            sorted[st + i] = (i < cx) ? x * T + i : sentinel;
    }
}

hipError_t launch_tilelist(const Plan& P, const int32_t* ent, hipStream_t s)
{
    hipLaunchKernelGGL(k_tilelist, dim3(1), dim3(1024), 0, s, ent, P.E, P.T, P.BM, P.counts,
                       P.offsets, P.sorted_ids, P.expert_ids, P.npp, (int)P.sentinel,
                       P.max_sorted, P.max_blocks, P.CH, P.chunk_off, P.chunk_expert);
    return hipGetLastError();
}

// ============================================================ fp8 activation quant
// Dynamic per-row quantisation before the first expert GEMM (FlagGems
// walkthrough, "FP8 W8A8": activations are quantised before each GEMM):
// scale = amax / 448 (1 for an all-zero row), code = RNE(x / scale),
// all in float32 with IEEE division.  One wave per row.
//   ident == 0: rows t in [0, M) of hidden -> aq[t]         (contiguous)
//   ident == 1: padded positions p < npp, source row sorted[p] -> aq[p] (batched)
template <typename TIn>
__global__ void __launch_bounds__(256) k_quant_rows(const TIn* __restrict__ x, int64_t rows, int H,
                                                    int ident, const int32_t* __restrict__ sorted,
                                                    const int32_t* __restrict__ npp, int sentinel,
                                                    uint8_t* __restrict__ aq,
                                                    float* __restrict__ aq_scale)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    int64_t src = r;
    if (ident) {
        if (r >= *npp)
            return;
        const int sid = sorted[r];
        if (sid >= sentinel) {          // padding row: zeros
            for (int k = lane * 16; k < H; k += 64 * 16)
                *(i32x4*)(aq + r * H + k) = i32x4{0, 0, 0, 0};
            if (lane == 0)
                aq_scale[r] = 1.0f;
            return;
        }
        src = sid;
    } else if (r >= rows) {
        return;
    }
    const TIn* row = x + src * (int64_t)H;
    float amax = 0.0f;
    for (int k = lane; k < H; k += 64) {
        float v;
        if constexpr (sizeof(TIn) == 2)
            v = bf16_to_f32(row[k]);
        else
            v = row[k];
        amax = fmaxf(amax, fabsf(v));
    }
    amax = wave_max(amax);
    const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    for (int k = lane * 4; k < H; k += 64 * 4) {
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v;
            if constexpr (sizeof(TIn) == 2)
                v = bf16_to_f32(row[k + i]);
            else
                v = row[k + i];
            packed |= (uint32_t)f32_to_fp8(v / scale) << (8 * i);
        }
        *(uint32_t*)(aq + r * H + k) = packed;
    }
    if (lane == 0)
        aq_scale[r] = scale;
}

hipError_t launch_quant_rows(const Plan& P, const void* hidden, hipStream_t s)
{
    const int ident = (P.fmt == MOE_FMT_BATCHED) ? 1 : 0;
    const int64_t rows = ident ? P.max_sorted : P.M;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (P.act == MOE_BF16)
        hipLaunchKernelGGL(k_quant_rows<u16>, grid, block, 0, s, (const u16*)hidden, rows, P.H,
                           ident, P.sorted_ids, P.npp, (int)P.sentinel, P.aq, P.aq_scale);
    else
        hipLaunchKernelGGL(k_quant_rows<float>, grid, block, 0, s, (const float*)hidden, rows,
                           P.H, ident, P.sorted_ids, P.npp, (int)P.sentinel, P.aq, P.aq_scale);
    return hipGetLastError();
}

// ============================================================ weight-and-reduce
// Unpermute + top-k weight-and-reduce (vLLM page, TopKWeightAndReduce;
// FlagGems moe_sum): y[t] = sum_{j ascending} w[t,j] * o[row(t,j)] in float32,
// rounded once to the output type.  o holds each routed item's expert output
// at its padded position: contiguous, row = inv[t*top_k + j] (the align
// kernel's inverse permutation; -1 contributes nothing); batched,
// row = offsets[e] + i for the slab row e*T + i named by token_map.  When
// GEMM2 ran as two K halves, an item's output is o[row] + o2[row] (that
// order).  One thread per 4 consecutive columns of one token; no atomics.
template <typename TOut>
__global__ void __launch_bounds__(256) k_reduce(const float* __restrict__ o, int M, int H, int K,
                                                const float* __restrict__ w,
                                                const int32_t* __restrict__ tmap, int T,
                                                const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ inv,
                                                const float* __restrict__ o2,
                                                TOut* __restrict__ out)
{
    const int cpr = H / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)M * cpr)
        return;
    const int t = (int)(gid / cpr), c = (int)(gid % cpr) * 4;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < K; ++j) {
        int64_t row;
        if (tmap) {
            const int flat = tmap[(int64_t)t * K + j];
            row = (int64_t)offsets[flat / T] + flat % T;
        } else {
            row = inv[(int64_t)t * K + j];
            if (row < 0)
                continue;
        }
        const float wj = w[(int64_t)t * K + j];
        f32x4 v = *(const f32x4*)(o + row * H + c);
        if (o2) {
            const f32x4 v2 = *(const f32x4*)(o2 + row * H + c);
            v = f32x4{v[0] + v2[0], v[1] + v2[1], v[2] + v2[2], v[3] + v2[3]};
        }
        acc[0] += wj * v[0];
        acc[1] += wj * v[1];
        acc[2] += wj * v[2];
        acc[3] += wj * v[3];
    }
    if constexpr (sizeof(TOut) == 2) {
        const uint32_t lo = f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
        const uint32_t hi = f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
        *(i32x2*)(out + (int64_t)t * H + c) = i32x2{(int)lo, (int)hi};
    } else {
        *(f32x4*)(out + (int64_t)t * H + c) = acc;
    }
}

hipError_t launch_reduce(const Plan& P, const moe_args& A, const float* topk_w, hipStream_t s)
{
    const bool batched = P.fmt == MOE_FMT_BATCHED;
    const float* w = batched ? A.token_map_w : topk_w;
    const int32_t* tmap = batched ? A.token_map : nullptr;
    const int64_t n = (int64_t)P.M * (P.H / 4);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (P.outdt == MOE_BF16)
        hipLaunchKernelGGL(k_reduce<u16>, grid, block, 0, s, P.o, P.M, P.H, P.K, w, tmap, P.T,
                           P.offsets, P.inv, P.o2, (u16*)A.out);
    else
        hipLaunchKernelGGL(k_reduce<float>, grid, block, 0, s, P.o, P.M, P.H, P.K, w, tmap, P.T,
                           P.offsets, P.inv, P.o2, (float*)A.out);
    return hipGetLastError();
}

}  // namespace moe
