// Bandwidth kernels of the fused MoE forward for gfx950: router (top-k),
// align (permute metadata), batched tile list, per-row fp8 quantisation and
// the top-k weight-and-reduce (unpermute).  None of them uses MFMA.
#include <atomic>

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
// A token is routed by a group of LPT lanes of one wave (LPT = 64, or the
// power of two >= E when E is small, so that several tokens share a wave);
// lane `sub` of the group holds experts [sub*EPL, (sub+1)*EPL).  Grouped
// selection always uses whole waves (LPT = 64).

// Orders float bit patterns as unsigned integers (monotone for non-NaN).
__device__ __forceinline__ uint32_t ord_f32(float f)
{
    uint32_t u = __float_as_uint(f + 0.0f);   // -0 -> +0: equal logits tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (key, value) pair: the largest key wins and carries its value along
struct KeyVal {
    uint32_t hi, lo;
    float val;
};

__device__ __forceinline__ KeyVal kv_max(const KeyVal& a, const KeyVal& b)
{
    const bool take = b.hi > a.hi || (b.hi == a.hi && b.lo > a.lo);
    return take ? b : a;
}

template <int CTRL>
__device__ __forceinline__ KeyVal xchg(const KeyVal& v)
{
    return KeyVal{dpp_u32<CTRL>(v.hi), dpp_u32<CTRL>(v.lo), xchg<CTRL>(v.val)};
}
__device__ __forceinline__ KeyVal rdlane(const KeyVal& v, int l)
{
    return KeyVal{(uint32_t)__builtin_amdgcn_readlane((int)v.hi, l),
                  (uint32_t)__builtin_amdgcn_readlane((int)v.lo, l), rdlane(v.val, l)};
}

template <int LPT>
__device__ __forceinline__ KeyVal grp_max_kv(const KeyVal& v)
{
    return grp_reduce<LPT>(v, kv_max);
}

struct RouteArgs {
    int E, K, scoring, renorm, G, kg, gmode;
    float rsf;
};

// Routes one token.  s: this lane's EPL logits (-inf past E).  grow: the
// token's E logits as floats in LDS (read by the grouped selection only).
// Lanes sub < K return pick `sub` (expert id, final weight).
template <int EPL, int LPT>
__device__ __forceinline__ void route_token(const RouteArgs& R, const float (&s)[EPL], int sub,
                                            const float* grow, int& id_out, float& w_out)
{
    const int lane = threadIdx.x & 63;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        mx = fmaxf(mx, s[i]);
    mx = grp_max<LPT>(mx);

    float p[EPL];
    bool cand[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        cand[i] = sub * EPL + i < R.E;
    if (R.scoring == MOE_ROUTE_SOFTMAX) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            p[i] = cand[i] ? expf(s[i] - mx) : 0.0f;
            sum += p[i];
        }
        sum = grp_sum<LPT>(sum);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            p[i] = p[i] / sum;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            p[i] = 1.0f / (1.0f + expf(-s[i]));
    }

    if constexpr (LPT == 64) {
        if (R.G > 1) {
            const int per = R.E / R.G;
            // the two largest logits of each group (a >= b, as a multiset):
            // Q lanes per group (a power of two, G Q <= 64) each scan every
            // Q-th logit of it, then the Q pairs merge by shuffles; lane g then
            // takes group g's pair and forms its key
            int qs = 0;
            while ((R.G << (qs + 1)) <= 64)
                ++qs;
            const int Q = 1 << qs;
            float a = -INFINITY, b = -INFINITY;
            if (lane < (R.G << qs)) {
                const float* sg = grow + (lane >> qs) * per;
                for (int i = lane & (Q - 1); i < per; i += Q) {
                    const float v = sg[i];
                    if (v > a) {
                        b = a;
                        a = v;
                    } else if (v > b) {
                        b = v;
                    }
                }
            }
            for (int o = 1; o < Q; o <<= 1) {
                const float a2 = __shfl_xor(a, o, 64), b2 = __shfl_xor(b, o, 64);
                b = fmaxf(fminf(a, a2), fmaxf(b, b2));
                a = fmaxf(a, a2);
            }
            a = __shfl(a, (lane << qs) & 63, 64);
            b = __shfl(b, (lane << qs) & 63, 64);
            KeyVal gkey{0u, 0u, 0.0f};
            if (lane < R.G) {
                float key;
                if (R.gmode == 0) {
                    key = a;
                } else if (R.scoring == MOE_ROUTE_SIGMOID) {
                    key = (float)(1.0 / (1.0 + exp(-(double)a))) +
                          (float)(1.0 / (1.0 + exp(-(double)b)));
                } else {
                    key = (float)exp((double)a - (double)mx) + (float)exp((double)b - (double)mx);
                }
                gkey = KeyVal{ord_f32(key), 0xffffffffu - lane, 0.0f};
            }
            unsigned long long chosen = 0;
            for (int r = 0; r < R.kg; ++r) {
                const KeyVal best = grp_max_kv<64>(gkey);
                const int g = (int)(0xffffffffu - best.lo);
                chosen |= 1ull << g;
                if (lane == g)
                    gkey = KeyVal{0u, 0u, 0.0f};
            }
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                cand[i] = cand[i] && ((chosen >> ((sub * EPL + i) / per)) & 1ull);
        }
    }

    // top-k by (logit desc, index asc); the winner's score travels with its key
    float wsel = 0.0f;
    int idsel = 0;
    for (int j = 0; j < R.K; ++j) {
        KeyVal mine{0u, 0u, 0.0f};
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (cand[i]) {
                const KeyVal k{ord_f32(s[i]), 0xffffffffu - (uint32_t)(sub * EPL + i), p[i]};
                mine = kv_max(mine, k);
            }
        }
        const KeyVal best = grp_max_kv<LPT>(mine);
        const int e = (int)(0xffffffffu - best.lo);
        if (sub == e / EPL) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (sub * EPL + i == e)
                    cand[i] = false;
        }
        if (sub == j) {
            wsel = best.val;
            idsel = e;
        }
    }
    if ((R.scoring == MOE_ROUTE_SOFTMAX && R.renorm) || R.scoring == MOE_ROUTE_SIGMOID) {
        const float tot = grp_sum<LPT>(sub < R.K ? wsel : 0.0f);
        wsel = wsel / tot;
    }
    id_out = idsel;
    w_out = wsel * R.rsf;
}

__device__ __forceinline__ float load_logit(const void* lg, int lgdt, int64_t i)
{
    return (lgdt == MOE_BF16) ? bf16_to_f32(((const u16*)lg)[i]) : ((const float*)lg)[i];
}

// Router for many tokens: 4 waves of 64 / LPT tokens each per workgroup.
template <int EPL, int LPT>
__global__ void __launch_bounds__(256) k_router(const void* __restrict__ logits, int lgdt, int M,
                                                RouteArgs R, int32_t* __restrict__ topk_ids,
                                                float* __restrict__ topk_w)
{
    constexpr int TPW = 64 / LPT;
    __shared__ float sh_logit[4][EPL * 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sub = lane & (LPT - 1);
    const int t = (blockIdx.x * 4 + wave) * TPW + lane / LPT;
    if (t >= M)
        return;                                 // whole groups leave together
    float s[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = sub * EPL + i;
        s[i] = (e < R.E) ? load_logit(logits, lgdt, (int64_t)t * R.E + e) : -INFINITY;
    }
    if constexpr (LPT == 64) {
        if (R.G > 1) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (sub * EPL + i < R.E)
                    sh_logit[wave][sub * EPL + i] = s[i];
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        }
    }
    int id;
    float w;
    route_token<EPL, LPT>(R, s, sub, sh_logit[wave], id, w);
    if (sub < R.K) {
        topk_ids[(int64_t)t * R.K + sub] = id;
        topk_w[(int64_t)t * R.K + sub] = w;
    }
}

static RouteArgs route_args(const Plan& P)
{
    return RouteArgs{P.Er, P.K, P.routing, P.renorm, P.G, P.kg, P.gmode, P.rsf};
}

// Lanes per token and experts per lane for E experts (grouped: whole waves).
static void route_shape(int E, int G, int& epl, int& lpt)
{
    epl = E <= 64 ? 1 : (E + 63) / 64;
    epl = epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : epl <= 8 ? 8 : 16;
    lpt = 64;
    if (G <= 1 && E <= 32)
        lpt = E <= 8 ? 8 : E <= 16 ? 16 : 32;
}

#define MOE_ROUTE_SHAPES(X) \
    X(1, 8) X(1, 16) X(1, 32) X(1, 64) X(2, 64) X(4, 64) X(8, 64) X(16, 64)

hipError_t launch_router(const Plan& P, const void* logits, hipStream_t s)
{
    int epl, lpt;
    route_shape(P.Er, P.G, epl, lpt);
    const int tpb = 4 * (64 / lpt);
    const dim3 grid((P.M + tpb - 1) / tpb), block(256);
    const RouteArgs R = route_args(P);
#define MOE_ROUTER(EPL, LPT)                                                                  \
    if (epl == EPL && lpt == LPT) {                                                           \
        hipLaunchKernelGGL((k_router<EPL, LPT>), grid, block, 0, s, logits, P.lgdt, P.M, R,   \
                           P.topk_ids, P.topk_w);                                             \
        return hipGetLastError();                                                             \
    }
    MOE_ROUTE_SHAPES(MOE_ROUTER)
#undef MOE_ROUTER
    return hipErrorInvalidValue;
}

// ============================================================ align
// moe_align_block_size of the FlagGems walkthrough ("moe_align_block_size"
// section): group the M*top_k routed items by expert, pad each expert's run
// to a multiple of BM.  Items keep ascending order inside an expert (a stable
// sort, as the MoonEP page's build_permutation), so the result is unique and
// independent of scheduling.  One workgroup of 16 waves.  The items sit in
// LDS (in batches of ALIGN_CAP when there are more); each wave owns a
// contiguous range of a batch.  Counting uses LDS atomics; the scatter ranks
// equal-expert lanes of a wave with ballots over the id bits, so every item's
// position is fixed without global atomics.

constexpr int ALIGN_WAVES = 16;
constexpr int ALIGN_CAP = 8192;        // items per LDS batch of the standalone align

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
#pragma unroll
    for (int w = 0; w < ALIGN_WAVES; ++w) {
        const int tw = sh_tot[w];
        if (w < wave)
            base += tw;
        total += tw;
    }
    *out_prefix = base + incl - v;
    return total;
}

// Largest e in [0, n) with a[e] <= x (a non-decreasing, a[0] <= x).
__device__ __forceinline__ int upper_index(const int* a, int n, int x)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// GEMM work unit lists: expert e's rows need ceil(rows / CH) chunks of at
// most CH rows (the row height of one GEMM tile); how the rows are dealt out
// to the chunks is the GEMM schedule's business.  Counting the real rows, not
// the BM-padded run, matters: a chunk made only of padding would still stream
// the expert's whole weight tile.  chunk_off[e] = chunks of experts < e,
// chunk_off[E] = all chunks, chunk_expert[c] = expert of chunk c.  Called by
// all 1024 threads; `rows` is this thread's expert's row count (0 for e >= E);
// choff: E + 1 ints of LDS scratch.
__device__ void write_chunks(int rows, int CH, int E, int* sh_tot, int* choff,
                             int32_t* chunk_off, int32_t* chunk_expert)
{
    const int e = threadIdx.x;
    __syncthreads();   // sh_tot is reused from the previous scan
    const int nch = (e < E) ? (rows + CH - 1) / CH : 0;
    int cstart;
    const int ctotal = block_exclusive_scan_1024(nch, sh_tot, &cstart);
    if (e < E) {
        chunk_off[e] = cstart;
        choff[e] = cstart;
    }
    if (e == 0)
        chunk_off[E] = ctotal;
    __syncthreads();
    for (int c = threadIdx.x; c < ctotal; c += 1024)
        chunk_expert[c] = upper_index(choff, E, c);
}

struct AlignOut {
    int32_t *counts, *offsets, *sorted, *expert_ids, *npp, *chunk_off, *chunk_expert, *inv;
    int E, BM, CH, sentinel, max_blocks;
    int64_t max_sorted;
    const int32_t* emap;        // [Er] global -> local expert (-1: elsewhere), or null
    int Er;                     // range of the routed ids
    int32_t* status;            // device status word
    int status_or;              // 0: store the align's findings; 1: OR them in
};

// The align stage's findings -> the device status word (one thread).
__device__ __forceinline__ void align_status(const AlignOut& O, int bits)
{
    if (O.status_or)
        *O.status |= bits;      // a later chunk: stream order leaves no other writer
    else
        *O.status = bits;
}

// LDS scratch of align_items (ints), after the item batch: per-wave counts,
// three prefix arrays, scan totals, and one flag word.
__host__ __device__ constexpr int align_scratch_ints(int E)
{
    return ALIGN_WAVES * E + 3 * (E + 1) + ALIGN_WAVES + 1;
}

// Item i of ids_g[b0 ..) -> ids_s[i] as a local expert id: through the
// expert map when there is one.  Unmapped experts (map value -1) become -1
// (no row); so do ids outside the routed range and map values outside
// [-1, E), for which the function returns true (in the threads that saw
// one).  All threads.
__device__ bool align_load(const int32_t* __restrict__ ids_g, int b0, int len, int* ids_s,
                           const AlignOut& O)
{
    const int tid = threadIdx.x, E = O.E;
    bool bad = false;
    for (int i0 = 0; i0 < len; i0 += 1024 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 1024 + tid;
            v[u] = (i < len) ? ids_g[b0 + i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 1024 + tid;
            if (i < len && (v[u] < 0 || v[u] >= O.Er)) {
                bad = true;
                v[u] = -1;
            }
        }
        if (O.emap) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * 1024 + tid;
                if (i < len && v[u] >= 0) {
                    v[u] = O.emap[v[u]];
                    if (v[u] < -1 || v[u] >= E) {
                        bad = true;
                        v[u] = -1;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 1024 + tid;
            if (i < len)
                ids_s[i] = v[u];
        }
    }
    return bad;
}

// Per-wave counts of ids_s[0, len): wave w owns [w ch, (w+1) ch) and
// cnt[w][e] counts its items of expert e.  Starts and ends with a barrier.
__device__ void align_count_waves(const int* ids_s, int len, int* cnt, int E)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < ALIGN_WAVES * E; i += 1024)
        cnt[i] = 0;
    __syncthreads();
    const int ch = (len + ALIGN_WAVES - 1) / ALIGN_WAVES;
    const int end = min(len, (wave + 1) * ch);
    for (int i = wave * ch + lane; i < end; i += 64) {
        const int e = ids_s[i];
        if (e >= 0)
            atomicAdd(&cnt[wave * E + e], 1);
    }
    __syncthreads();
}

// From per-expert totals (thread e < E holds total_e): counts, padded
// offsets, sentinel padding, num_post_padded, GEMM row chunks and block
// expert ids; offs[e] = run[e] = the expert's first padded position.
__device__ void align_layout(int total_e, int* offs, int* run, int* choff, int* tot,
                             const AlignOut& O)
{
    const int tid = threadIdx.x, E = O.E, BM = O.BM;
    const int e = tid;
    const int padded = (e < E) ? (total_e + BM - 1) / BM * BM : 0;
    int start;
    const int total = block_exclusive_scan_1024(padded, tot, &start);
    if (e < E) {
        O.counts[e] = total_e;
        O.offsets[e] = start;
        offs[e] = start;
        run[e] = start;
        for (int q = start + total_e; q < start + padded && q < O.max_sorted; ++q)
            O.sorted[q] = O.sentinel;
    }
    if (tid == 0) {
        O.offsets[E] = total;
        offs[E] = total;
        *O.npp = total;
    }
    write_chunks((e < E) ? total_e : 0, O.CH, E, tot, choff, O.chunk_off, O.chunk_expert);
    for (int b = tid; b < total / BM && b < O.max_blocks; b += 1024)
        O.expert_ids[b] = upper_index(offs, E, b * BM);
}

// Stable scatter of ids_s[0, len) (routed items b0 ..): with cnt holding
// the per-wave counts and run[e] the next free position of expert e, wave
// w's items of expert e go to run[e] + (items of e in waves < w) + their
// rank; run advances past the batch.  Writes sorted ids and inv.
__device__ void align_scatter(const int* ids_s, int b0, int len, int* cnt, int* run,
                              const AlignOut& O)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, E = O.E;
    const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
    // cnt[w][e] <- first position of wave w's items of expert e
    if (tid < E) {
        int base = run[tid];
        for (int w = 0; w < ALIGN_WAVES; ++w) {
            const int c = cnt[w * E + tid];
            cnt[w * E + tid] = base;
            base += c;
        }
        run[tid] = base;
    }
    __syncthreads();
    const int ch = (len + ALIGN_WAVES - 1) / ALIGN_WAVES;
    const int end = min(len, (wave + 1) * ch);
    for (int i0 = wave * ch; i0 < end; i0 += 64) {
        const int i = i0 + lane;
        const int ev = (i < end) ? ids_s[i] : -1;
        const bool valid = ev >= 0;
        const unsigned long long m = match_mask(ev, valid, nbits);
        const int r = b0 + i;
        if (valid) {
            const int rank = __popcll(m & ((1ull << lane) - 1ull));
            const int64_t pos = (int64_t)cnt[wave * E + ev] + rank;
            if (pos < O.max_sorted)
                O.sorted[pos] = r;
            O.inv[r] = (pos < O.max_sorted) ? (int)pos : -1;
        } else if (i < end) {
            O.inv[r] = -1;                          // expert id out of range: no row
        }
        // every lane has read its base before the leader moves it on
        __builtin_amdgcn_wave_barrier();
        if (valid && lane == (int)__builtin_ctzll(m))
            cnt[wave * E + ev] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

// The align proper over the n routed items, in one workgroup.  ids_s: LDS
// batch of up to cap items; if ids_g is non-null the batches are loaded from
// it, otherwise ids_s already holds all n <= cap items.  All 1024 threads.
__device__ void align_items(const int32_t* __restrict__ ids_g, int n, int* ids_s, int cap,
                           int* scratch, const AlignOut& O)
{
    const int E = O.E;
    int* cnt = scratch;                         // [ALIGN_WAVES][E]
    int* offs = cnt + ALIGN_WAVES * E;          // [E + 1] padded start per expert
    int* run = offs + (E + 1);                  // [E + 1] next free position (pass 2)
    int* choff = run + (E + 1);                 // [E + 1] chunk prefix
    int* tot = choff + (E + 1);                 // [ALIGN_WAVES]
    int* bad = tot + ALIGN_WAVES;               // [1] an out-of-range id was seen
    const int tid = threadIdx.x;
    const int nb = (n + cap - 1) / cap;
    if (tid == 0)
        *bad = 0;
    __syncthreads();

    // pass 1: per-expert totals
    int total_e = 0;
    if (nb <= 1) {
        if (ids_g && align_load(ids_g, 0, n, ids_s, O))
            atomicOr(bad, 1);
        __syncthreads();
        align_count_waves(ids_s, n, cnt, E);
        if (tid < E)
            for (int w = 0; w < ALIGN_WAVES; ++w)
                total_e += cnt[w * E + tid];
    } else {
        for (int i = tid; i < E; i += 1024)
            run[i] = 0;
        for (int b = 0; b < nb; ++b) {
            const int b0 = b * cap, len = min(cap, n - b0);
            __syncthreads();
            if (align_load(ids_g, b0, len, ids_s, O))
                atomicOr(bad, 1);
            __syncthreads();
            for (int i = tid; i < len; i += 1024) {
                const int e = ids_s[i];
                if (e >= 0)
                    atomicAdd(&run[e], 1);
            }
        }
        __syncthreads();
        if (tid < E)
            total_e = run[tid];
    }

    align_layout(total_e, offs, run, choff, tot, O);

    // pass 2: stable scatter, batch by batch
    for (int b = 0; b < nb; ++b) {
        const int b0 = b * cap, len = min(cap, n - b0);
        if (nb > 1) {
            __syncthreads();
            align_load(ids_g, b0, len, ids_s, O);
            __syncthreads();
            align_count_waves(ids_s, len, cnt, E);
        }
        align_scatter(ids_s, b0, len, cnt, run, O);
    }
    __syncthreads();
    if (tid == 0)
        align_status(O, *bad ? MOE_DEV_ID_RANGE : 0);
}

// ---- the same align over many workgroups, for large batches of routed
// items: block b of the grid owns items [b ALIGN_BLOCK, (b+1) ALIGN_BLOCK).
// (1) k_align_count: hist[b][e] = block b's items of expert e; (2)
// k_align_layout (one workgroup): totals, the padded layout, and hist[b][e]
// <- first position of block b's items of expert e (blocks in order); (3)
// k_align_scatter: each block's stable scatter from those bases.  Blocks are
// consecutive ranges and the layout takes them in order, so the result is
// the one-workgroup align's, bit for bit.
constexpr int ALIGN_BLOCK = 8192;

__global__ void __launch_bounds__(1024) k_align_count(const int32_t* __restrict__ ids, int Mk,
                                                      AlignOut O, int32_t* __restrict__ hist)
{
    extern __shared__ int sh[];
    int* ids_s = sh;                            // [ALIGN_BLOCK]
    int* cnt = sh + ALIGN_BLOCK;                // [E + 1]: counts, then the block's flag
    const int b0 = blockIdx.x * ALIGN_BLOCK, len = min(ALIGN_BLOCK, Mk - b0);
    for (int i = threadIdx.x; i <= O.E; i += 1024)
        cnt[i] = 0;
    __syncthreads();
    if (align_load(ids, b0, len, ids_s, O))
        atomicOr(&cnt[O.E], 1);
    __syncthreads();
    for (int i = threadIdx.x; i < len; i += 1024) {
        const int e = ids_s[i];
        if (e >= 0)
            atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= O.E; e += 1024)
        hist[(int64_t)blockIdx.x * (O.E + 1) + e] = cnt[e];
}

__global__ void __launch_bounds__(1024) k_align_layout(int nblk, AlignOut O,
                                                       int32_t* __restrict__ hist)
{
    extern __shared__ int sh[];
    const int E = O.E, e = threadIdx.x;
    int* offs = sh;                             // [E + 1]
    int* run = offs + (E + 1);                  // [E + 1]
    int* choff = run + (E + 1);                 // [E + 1]
    int* tot = choff + (E + 1);                 // [ALIGN_WAVES]
    int total_e = 0;
    if (e < E)
        for (int b = 0; b < nblk; ++b)
            total_e += hist[(int64_t)b * (E + 1) + e];
    align_layout(total_e, offs, run, choff, tot, O);
    if (e < E) {
        int base = run[e];
        for (int b = 0; b < nblk; ++b) {
            const int c = hist[(int64_t)b * (E + 1) + e];
            hist[(int64_t)b * (E + 1) + e] = base;
            base += c;
        }
    }
    if (e == 0) {
        int bad = 0;
        for (int b = 0; b < nblk; ++b)
            bad |= hist[(int64_t)b * (E + 1) + E];
        align_status(O, bad ? MOE_DEV_ID_RANGE : 0);
    }
}

__global__ void __launch_bounds__(1024) k_align_scatter(const int32_t* __restrict__ ids, int Mk,
                                                        AlignOut O,
                                                        const int32_t* __restrict__ hist)
{
    extern __shared__ int sh[];
    const int E = O.E;
    int* ids_s = sh;                            // [ALIGN_BLOCK]
    int* cnt = sh + ALIGN_BLOCK;                // [ALIGN_WAVES][E]
    int* run = cnt + ALIGN_WAVES * E;           // [E]
    const int b0 = blockIdx.x * ALIGN_BLOCK, len = min(ALIGN_BLOCK, Mk - b0);
    for (int e = threadIdx.x; e < E; e += 1024)
        run[e] = hist[(int64_t)blockIdx.x * (E + 1) + e];
    (void)align_load(ids, b0, len, ids_s, O);   // k_align_count reported its findings
    __syncthreads();
    align_count_waves(ids_s, len, cnt, E);
    align_scatter(ids_s, b0, len, cnt, run, O);
}

static AlignOut align_out(const Plan& P)
{
    return AlignOut{P.counts,     P.offsets,       P.sorted_ids,  P.expert_ids, P.npp,
                    P.chunk_off,  P.chunk_expert,  P.inv,         P.E,          P.BM,
                    P.CH,         (int)P.sentinel, P.max_blocks,  P.max_sorted, P.emap,
                    P.Er,         P.status,        P.status_or};
}

__global__ void __launch_bounds__(1024) k_align(const int32_t* __restrict__ ids, int Mk, int cap,
                                                AlignOut O)
{
    extern __shared__ int sh[];
    align_items(ids, Mk, sh, cap, sh + cap, O);
}

// Kernels launched with more than 64 KiB of dynamic LDS need the limit
// raised first.  It is raised once per kernel and device to the most a
// workgroup may hold (160 KiB on gfx950), so a forward makes no attribute
// call once the device has seen one (graph capture included).
constexpr int LDS_MAX = 160 * 1024;

static hipError_t set_lds(const void* kernel, size_t bytes, int dev, std::atomic<int>* done)
{
    if (bytes <= 65536)
        return hipSuccess;
    if (bytes > (size_t)LDS_MAX)
        return hipErrorInvalidValue;
    const int slot = (dev >= 0 && dev < MAX_DEVICES) ? dev : 0;
    if (done[slot].load(std::memory_order_acquire))
        return hipSuccess;
    const hipError_t e =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_MAX);
    if (e == hipSuccess)
        done[slot].store(1, std::memory_order_release);
    return e;
}

hipError_t launch_align(const Plan& P, const int32_t* ids, hipStream_t s)
{
    const int Mk = P.M * P.K;
    if (Mk > 2 * ALIGN_BLOCK) {
        // many workgroups; block histograms in the o region, which only GEMM2 writes
        const int nblk = (Mk + ALIGN_BLOCK - 1) / ALIGN_BLOCK;
        int32_t* hist = (int32_t*)P.o;
        const AlignOut O = align_out(P);
        const size_t l1 = sizeof(int) * ((size_t)ALIGN_BLOCK + P.E + 1);
        const size_t l2 = sizeof(int) * (3 * ((size_t)P.E + 1) + ALIGN_WAVES);
        const size_t l3 = sizeof(int) * ((size_t)ALIGN_BLOCK + (size_t)(ALIGN_WAVES + 1) * P.E);
        static std::atomic<int> d1[MAX_DEVICES], d2[MAX_DEVICES], d3[MAX_DEVICES];
        hipError_t e = set_lds((const void*)k_align_count, l1, P.dev, d1);
        if (e == hipSuccess)
            e = set_lds((const void*)k_align_layout, l2, P.dev, d2);
        if (e == hipSuccess)
            e = set_lds((const void*)k_align_scatter, l3, P.dev, d3);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_align_count, dim3(nblk), dim3(1024), l1, s, ids, Mk, O, hist);
        hipLaunchKernelGGL(k_align_layout, dim3(1), dim3(1024), l2, s, nblk, O, hist);
        hipLaunchKernelGGL(k_align_scatter, dim3(nblk), dim3(1024), l3, s, ids, Mk, O, hist);
        return hipGetLastError();
    }
    const int cap = Mk < ALIGN_CAP ? (Mk > 0 ? Mk : 1) : ALIGN_CAP;
    const size_t lds = sizeof(int) * ((size_t)cap + align_scratch_ints(P.E));
    static std::atomic<int> d0[MAX_DEVICES];
    const hipError_t e = set_lds((const void*)k_align, lds, P.dev, d0);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_align, dim3(1), dim3(1024), lds, s, ids, Mk, cap, align_out(P));
    return hipGetLastError();
}

// ============================================================ batched tile list
// Batched format (vLLM "Fused MoE Modular Kernel" introduction): slab e holds
// expert_num_tokens[e] valid rows.  Builds the same metadata as align with
// item r = e*max_tokens + i, so the GEMMs are shared by both formats.  Counts
// outside [0, max_tokens] are clamped (MOE_DEV_COUNT_CLAMPED).  Slabs whose
// runs would pass the workspace capacity (more valid rows than the caller
// promised) get no rows at all (counts 0, MOE_DEV_ROWS_OVERFLOW), so a bad
// count can never drive an access out of bounds and a reduce yields zeros.
__global__ void __launch_bounds__(1024) k_tilelist(const int32_t* __restrict__ ent, int E, int T,
                                                   int BM, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted,
                                                   int32_t* __restrict__ expert_ids,
                                                   int32_t* __restrict__ npp, int sentinel,
                                                   int64_t max_sorted, int max_blocks, int CH,
                                                   int32_t* __restrict__ chunk_off,
                                                   int32_t* __restrict__ chunk_expert,
                                                   int32_t* __restrict__ status)
{
    __shared__ int tot[ALIGN_WAVES];
    __shared__ int sh_start[1025], sh_cnt[1024], choff[1025];
    __shared__ int sh_clamped;
    const int e = threadIdx.x;
    if (threadIdx.x == 0)
        sh_clamped = 0;
    __syncthreads();
    int c = 0, padded = 0;
    if (e < E) {
        const int raw = ent[e];
        c = min(max(raw, 0), T);
        if (c != raw)
            atomicOr(&sh_clamped, 1);
        padded = (c + BM - 1) / BM * BM;
    }
    int start;
    const int total = block_exclusive_scan_1024(padded, tot, &start);   // (its barrier orders sh_clamped)
    // more rows than the workspace was sized for: process nothing
    const bool fits = (int64_t)total <= max_sorted && total / BM <= max_blocks;
    if (e < E) {
        sh_start[e] = start;
        sh_cnt[e] = c;
    }
    if (threadIdx.x == 0)
        sh_start[E] = total;
    // workgroup 0 writes the per-expert metadata and the chunk tables
    if (blockIdx.x == 0) {
        if (e < E) {
            counts[e] = fits ? c : 0;
            offsets[e] = fits ? start : 0;
        }
        if (threadIdx.x == 0) {
            offsets[E] = fits ? total : 0;
            *npp = fits ? total : 0;
            *status = (sh_clamped ? MOE_DEV_COUNT_CLAMPED : 0) | (fits ? 0 : MOE_DEV_ROWS_OVERFLOW);
        }
        write_chunks(fits ? c : 0, CH, E, tot, choff, chunk_off, chunk_expert);
    }
    __syncthreads();
    if (!fits)
        return;
    if (blockIdx.x == 0)
        for (int b = threadIdx.x; b < total / BM; b += 1024)
            expert_ids[b] = upper_index(sh_start, E, b * BM);
    // the sorted ids: every workgroup fills its share of the padded positions,
    // each position finding its expert run by a binary search of the starts
    const int per = (total + gridDim.x - 1) / gridDim.x;
    const int p1 = min(total, (int)(blockIdx.x + 1) * per);
    for (int p = blockIdx.x * per + threadIdx.x; p < p1; p += 1024) {
        const int x = upper_index(sh_start, E, p), i = p - sh_start[x];
        sorted[p] = (i < sh_cnt[x]) ? x * T + i : sentinel;
    }
}

hipError_t launch_tilelist(const Plan& P, const int32_t* ent, hipStream_t s)
{
    // one workgroup per 4096 padded positions the workspace holds (up to 64):
    // each recomputes the layout from the counts and fills its share
    const int64_t nb = (P.max_sorted + 4095) / 4096;
    const dim3 grid((unsigned)(nb < 1 ? 1 : nb > 64 ? 64 : nb));
    hipLaunchKernelGGL(k_tilelist, grid, dim3(1024), 0, s, ent, P.E, P.T, P.BM, P.counts,
                       P.offsets, P.sorted_ids, P.expert_ids, P.npp, (int)P.sentinel,
                       P.max_sorted, P.max_blocks, P.CH, P.chunk_off, P.chunk_expert, P.status);
    return hipGetLastError();
}

// ============================================================ fp8 activation quant
// Dynamic per-row quantisation before the first expert GEMM (FlagGems
// walkthrough, "FP8 W8A8": activations are quantised before each GEMM):
// scale = amax / 448 (1 for an all-zero row), code = RNE(x / scale),
// all in float32 with IEEE division.  One wave per row, 16-byte loads: a
// first pass forms the amax, then the codes are written from the registers
// (rows of up to 256 chunks) or from a second pass over the row (from L2).
//   ident == 0: rows t in [0, M) of hidden -> aq[t]         (contiguous)
//   ident == 1: padded positions p < npp, source row sorted[p] -> aq[p] (batched)
template <typename TIn>
__global__ void __launch_bounds__(256) k_quant_rows(const TIn* __restrict__ x, int64_t rows, int H,
                                                    int ident, const int32_t* __restrict__ sorted,
                                                    const int32_t* __restrict__ npp, int sentinel,
                                                    uint8_t* __restrict__ aq,
                                                    float* __restrict__ aq_scale)
{
    constexpr int VE = 16 / sizeof(TIn);            // elements per 16-byte chunk
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    const int nch = H / VE;                          // H is a multiple of 16
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
    const i32x4* row = (const i32x4*)(x + src * (int64_t)H);
    auto val = [&](const i32x4& c, int i) {
        if constexpr (sizeof(TIn) == 2)
            return bf16_to_f32((u16)((uint32_t)c[i >> 1] >> (16 * (i & 1))));
        else
            return __int_as_float(c[i]);
    };
    float amax = 0.0f;
    i32x4 v[4];                                      // the last 256 chunks read
    for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c0 + u * 64 + lane;
            v[u] = (c < nch) ? row[c] : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < VE; ++i)
                amax = fmaxf(amax, fabsf(val(v[u], i)));
    }
    amax = wave_max(amax);
    const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    auto emit = [&](int c, const i32x4& cv) {
        uint32_t w[VE / 4];
#pragma unroll
        for (int q = 0; q < VE / 4; ++q)
            w[q] = cvt_fp8x2(val(cv, 4 * q) / scale, val(cv, 4 * q + 1) / scale) |
                   (cvt_fp8x2(val(cv, 4 * q + 2) / scale, val(cv, 4 * q + 3) / scale) << 16);
        if constexpr (VE == 8)
            *(i32x2*)(aq + r * H + c * 8) = i32x2{(int)w[0], (int)w[1]};
        else
            *(uint32_t*)(aq + r * H + c * 4) = w[0];
    };
    if (nch <= 64 * 4) {
        // the whole row is still in registers (up to 2048 bf16 / 1024 f32 columns)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = u * 64 + lane;
            if (c < nch)
                emit(c, v[u]);
        }
    } else {
        for (int c = lane; c < nch; c += 64)        // second pass, from L2
            emit(c, row[c]);
    }
    if (lane == 0)
        aq_scale[r] = scale;
}

// Block-wise variant (the "FP8 W8A8" section's block-wise granularity): one
// scale per row and 128 columns (amax / 448 over the group, 1 for an all-zero
// group; a short last group covers the rest of the row), codes as above,
// scales row-major [rows][ceil(H / 128)].  One wave per row, one pass: the
// GL lanes that hold one 128-column group's chunks reduce its amax among
// themselves.
template <typename TIn>
__global__ void __launch_bounds__(256) k_quant_groups(const TIn* __restrict__ x, int64_t rows, int H,
                                                      int ident, const int32_t* __restrict__ sorted,
                                                      const int32_t* __restrict__ npp, int sentinel,
                                                      uint8_t* __restrict__ aq,
                                                      float* __restrict__ aq_scale)
{
    constexpr int VE = 16 / sizeof(TIn);            // elements per 16-byte chunk
    constexpr int GL = 128 / VE;                     // lanes (chunks) per 128-column group
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    const int nch = H / VE, ng = (H + 127) / 128;
    int64_t src = r;
    if (ident) {
        if (r >= *npp)
            return;
        const int sid = sorted[r];
        if (sid >= sentinel) {          // padding row: zeros, unit scales
            for (int k = lane * 16; k < H; k += 64 * 16)
                *(i32x4*)(aq + r * H + k) = i32x4{0, 0, 0, 0};
            for (int gi = lane; gi < ng; gi += 64)
                aq_scale[r * ng + gi] = 1.0f;
            return;
        }
        src = sid;
    } else if (r >= rows) {
        return;
    }
    const i32x4* row = (const i32x4*)(x + src * (int64_t)H);
    auto val = [&](const i32x4& c, int i) {
        if constexpr (sizeof(TIn) == 2)
            return bf16_to_f32((u16)((uint32_t)c[i >> 1] >> (16 * (i & 1))));
        else
            return __int_as_float(c[i]);
    };
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        const i32x4 v = (c < nch) ? row[c] : i32x4{0, 0, 0, 0};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < VE; ++i)
            amax = fmaxf(amax, fabsf(val(v, i)));
        amax = grp_max<GL>(amax);                    // the lanes of one group, all active
        const float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        if (c < nch) {
            uint32_t w[VE / 4];
#pragma unroll
            for (int q = 0; q < VE / 4; ++q)
                w[q] = cvt_fp8x2(val(v, 4 * q) / scale, val(v, 4 * q + 1) / scale) |
                       (cvt_fp8x2(val(v, 4 * q + 2) / scale, val(v, 4 * q + 3) / scale) << 16);
            if constexpr (VE == 8)
                *(i32x2*)(aq + r * H + c * 8) = i32x2{(int)w[0], (int)w[1]};
            else
                *(uint32_t*)(aq + r * H + c * 4) = w[0];
            if (lane % GL == 0)
                aq_scale[r * ng + c / GL] = scale;
        }
    }
}

hipError_t launch_quant_rows(const Plan& P, const void* hidden, hipStream_t s)
{
    const int ident = (P.fmt == MOE_FMT_BATCHED) ? 1 : 0;
    const int64_t rows = ident ? P.max_sorted : P.M;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (P.blk) {
        if (P.act == MOE_BF16)
            hipLaunchKernelGGL(k_quant_groups<u16>, grid, block, 0, s, (const u16*)hidden, rows,
                               P.H, ident, P.sorted_ids, P.npp, (int)P.sentinel, P.aq, P.aq_scale);
        else
            hipLaunchKernelGGL(k_quant_groups<float>, grid, block, 0, s, (const float*)hidden,
                               rows, P.H, ident, P.sorted_ids, P.npp, (int)P.sentinel, P.aq,
                               P.aq_scale);
        return hipGetLastError();
    }
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
// FlagGems moe_sum): y[t] = sum_{j ascending} w[t,j] * o[row(t,j)] in float32
// (w null: weights of 1, when the routing weight was applied to z),
// rounded once to the output type.  o holds each routed item's expert output
// at its padded position: contiguous, row = inv[t*top_k + j] (the align
// kernel's inverse permutation; -1 contributes nothing); batched,
// row = offsets[e] + i for the slab row e*T + i named by token_map (-1, or
// an entry that names no valid slab row, contributes nothing; the latter
// sets MOE_DEV_TOKEN_MAP).  When
// GEMM2 ran as two K halves, an item's output is o[row] + o2[row] (that
// order).  One workgroup per token: the token's item rows and weights are
// the same for every thread (scalar loads), items without a row are skipped
// by a uniform branch.  A thread holds CPT 4-column chunks (256 apart) of
// the row and loads them for 8 / CPT items at once before accumulating, so
// eight loads are in flight whatever H; every output element still sums its
// items in ascending j.  No atomics.
template <typename TOut, int CPT>
__global__ void __launch_bounds__(256) k_reduce(const float* __restrict__ o, int H, int K,
                                                const float* __restrict__ w,
                                                const int32_t* __restrict__ tmap, int T, int E,
                                                const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ inv,
                                                const float* __restrict__ o2,
                                                TOut* __restrict__ out,
                                                int32_t* __restrict__ status, int64_t cap)
{
    constexpr int IU = 8 / CPT;             // items in flight together: IU x CPT loads a thread
    const int64_t t = blockIdx.x;
    const int cpr = H / 4;
    for (int c0 = 0; c0 < cpr; c0 += 256 * CPT) {
        f32x4 acc[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int j0 = 0; j0 < K; j0 += IU) {
            int64_t row[IU];
            float wj[IU];
#pragma unroll
            for (int u = 0; u < IU; ++u) {
                const int j = j0 + u;
                row[u] = -1;
                wj[u] = 0.0f;
                if (j < K) {
                    if (tmap) {
                        // the same entry in every thread: a uniform branch
                        const int flat = tmap[t * K + j];
                        const int e = (flat >= 0) ? flat / T : 0, i = flat - e * T;
                        if (flat >= 0 && e < E && i < counts[e])
                            row[u] = (int64_t)offsets[e] + i;
                        else if (flat != -1 && c0 == 0 && threadIdx.x == 0 &&
                                 !(*status & MOE_DEV_ROWS_OVERFLOW))   // (then no row is valid)
                            atomicOr(status, MOE_DEV_TOKEN_MAP);
                    } else {
                        row[u] = inv[t * K + j];
                    }
                    // (checked build: a row outside o contributes nothing)
                    if (row[u] >= 0 && !in_bounds(row[u], cap, status))
                        row[u] = -1;
                    wj[u] = w ? w[t * K + j] : 1.0f;
                }
            }
            f32x4 v[IU][CPT];
#pragma unroll
            for (int u = 0; u < IU; ++u) {
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int q = c0 + threadIdx.x + 256 * i;
                    v[u][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    if (row[u] >= 0 && q < cpr) {   // no row: nothing loaded
                        v[u][i] = *(const f32x4*)(o + row[u] * H + 4 * q);
                        if (o2) {
                            const f32x4 v2 = *(const f32x4*)(o2 + row[u] * H + 4 * q);
                            v[u][i] = f32x4{v[u][i][0] + v2[0], v[u][i][1] + v2[1],
                                            v[u][i][2] + v2[2], v[u][i][3] + v2[3]};
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < IU; ++u) {
                if (row[u] < 0)
                    continue;                       // contributes nothing
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    acc[i][0] += wj[u] * v[u][i][0];
                    acc[i][1] += wj[u] * v[u][i][1];
                    acc[i][2] += wj[u] * v[u][i][2];
                    acc[i][3] += wj[u] * v[u][i][3];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int q = c0 + threadIdx.x + 256 * i;
            if (q >= cpr)
                continue;
            if constexpr (sizeof(TOut) == 2) {
                const uint32_t lo = f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16);
                const uint32_t hi = f32_to_bf16(acc[i][2]) | ((uint32_t)f32_to_bf16(acc[i][3]) << 16);
                *(i32x2*)(out + t * H + 4 * q) = i32x2{(int)lo, (int)hi};
            } else {
                *(f32x4*)(out + t * H + 4 * q) = acc[i];
            }
        }
    }
}

template <typename TOut>
static void reduce_launch(const Plan& P, const float* w, const int32_t* tmap, void* out,
                          hipStream_t s)
{
    // chunks a thread holds: enough to cover the row in one pass, at most 8
    const int per = (P.H / 4 + 255) / 256;
    const dim3 grid((unsigned)P.M), block(256);
#define MOE_REDUCE(C)                                                                           \
    hipLaunchKernelGGL((k_reduce<TOut, C>), grid, block, 0, s, P.o, P.H, P.K, w, tmap, P.T,    \
                       P.E, P.offsets, P.counts, P.inv, P.o2, (TOut*)out, P.status,        \
                       P.max_sorted)
    if (per <= 1)
        MOE_REDUCE(1);
    else if (per <= 2)
        MOE_REDUCE(2);
    else if (per <= 4)
        MOE_REDUCE(4);
    else
        MOE_REDUCE(8);
#undef MOE_REDUCE
}

hipError_t launch_reduce(const Plan& P, const moe_args& A, const float* topk_w, hipStream_t s)
{
    const bool batched = P.fmt == MOE_FMT_BATCHED;
    const float* w = batched ? A.token_map_w : topk_w;
    const int32_t* tmap = batched ? A.token_map : nullptr;
    if (P.outdt == MOE_BF16)
        reduce_launch<u16>(P, w, tmap, A.out, s);
    else
        reduce_launch<float>(P, w, tmap, A.out, s);
    return hipGetLastError();
}

}  // namespace moe
