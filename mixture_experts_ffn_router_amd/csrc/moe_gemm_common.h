// Shared pieces of the grouped expert GEMMs (bf16 / f32 in moe_gemm.hip,
// fp8 in moe_gemm_fp8.hip): launch arguments, the persistent tile schedule,
// LDS-DMA helpers and the DMA ring loop.  gfx950 only.
#pragma once

#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int PACK_BLOCK = 64 * 256;     // bytes of one packed weight block

// sched_group_barrier instruction classes
constexpr int SCHED_MFMA = 0x008, SCHED_DS_READ = 0x100;

__device__ __forceinline__ float load_bias(const void* b, int dt, int64_t idx)
{
    return (dt == MOE_BF16) ? bf16_to_f32(((const u16*)b)[idx]) : ((const float*)b)[idx];
}

// SiLU(g) * u = g / (1 + e^-g) * u with the hardware exponential and
// reciprocal (v_exp_f32 on a prescaled argument, v_rcp_f32; a few ulp): the
// epilogue's cost matters where the MFMAs are fast.
__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// fp8 requantisation of z per (row, 128 columns): scale = amax / 448 (1 for
// an all-zero group), formed as amax times the float nearest 1 / 448 (within
// an ulp of the quotient; GEMM2 dequantises with the same stored scale); the
// codes are RNE(z * rcp(scale)) with the hardware reciprocal (1 ulp), one per
// group: against exact arithmetic this can move a code by one step only where
// z / scale lies within an ulp or two of a rounding tie, and the group's
// largest value still lands on code 448 (the codes there are 32 apart).
__device__ __forceinline__ float zq_scale(float amax)
{
    return (amax > 0.0f) ? amax * (1.0f / 448.0f) : 1.0f;
}

// 4 x 4 transpose inside each quad of lanes (two DPP butterflies): lane
// 4a + q holding v[r] = X[r][q] (column q of the quad's 4 x 4 block, row r)
// ends up holding v[c] = X[q][c] (row q, columns c).  A 16 x 16 MFMA result
// fragment then gives every lane four consecutive columns of one row, which
// it stores as one 16-byte (float) or 8-byte (bf16) row piece.  Every lane
// of the quad must be active.
__device__ __forceinline__ float dpp_xor1(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ void quad_transpose(f32x4& v, int lane)
{
    const bool odd = lane & 1, hi = lane & 2;
    // lanes q, q ^ 1 swap the elements whose index parity differs from theirs
    float r0 = dpp_xor1(odd ? v[0] : v[1]), r1 = dpp_xor1(odd ? v[2] : v[3]);
    v[0] = odd ? r0 : v[0];
    v[1] = odd ? v[1] : r0;
    v[2] = odd ? r1 : v[2];
    v[3] = odd ? v[3] : r1;
    // lanes q, q ^ 2 the same for bit 1
    r0 = dpp_xor2(hi ? v[0] : v[2]);
    r1 = dpp_xor2(hi ? v[1] : v[3]);
    v[0] = hi ? r0 : v[0];
    v[2] = hi ? v[2] : r0;
    v[1] = hi ? r1 : v[1];
    v[3] = hi ? v[3] : r1;
}

// Four consecutive output values of one row: 16 bytes of float, or 8 bytes
// of bf16 (round to nearest even), at element index o of out.
__device__ __forceinline__ void store_row4(void* out, int64_t o, bool bf16, const f32x4& v)
{
    if (bf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(i32x2*)((u16*)out + o) = i32x2{(int)lo, (int)hi};
    } else {
        *(f32x4*)((float*)out + o) = v;
    }
}

// ---------------------------------------------------------------- arguments
struct Sched {
    const int32_t* counts;      // [E] real rows per expert
    const int32_t* offsets;     // [E + 1] start of each expert's padded run
    const int32_t* chunk_off;   // [E + 1] chunk prefix per expert
    const int32_t* chunk_expert;
    const int32_t* sorted;
    int sentinel;
    int E, n_tiles;
    int64_t cap;                // padded positions in the workspace (checked build)
    int max_chunks;             // entries of chunk_expert (checked build)
    int32_t* status;            // device status word (checked build)
};

struct Gemm1Args {
    Sched s;
    const void* a;              // activation rows [*, H] (f32 / bf16 / fp8 codes)
    const float* a_scale;       // fp8: per activation row, or [row][a_sld] block scales
    int a_sld;                  // block-wise: floats per activation scale row (ceil(H / 128))
    int blk;                    // fp8: block-wise scales (128 x 128 weight blocks)
    int a_ident;                // 1: A row = padded position p; 0: sorted[p] / a_div
    int a_div;
    const void* w13;            // [E, H, 2I], or packed blocks (bf16 / fp8 block layouts)
    int w_packed;               // 1: w13 is in the packed block layout
    const float* w13_scale;     // fp8: [E, 2I], or block-wise [E][2I/128][ceil(H/128)];
                                // WNA16: [E][ceil(H/G)][2I] group scales
    const uint8_t* w13_zero;    // WNA16: zero points like w13_scale, or null
    int wq_gsh;                 // WNA16: log2(K rows per scale group / 32)
    const void* b13;            // [E, 2I] or null
    int bias_dt;
    int H, I;
    void* z;                    // [max_sorted, I]
    float* z_scale;             // fp8: [I/128][zs_ld] (group-major)
    int64_t zs_ld;              // fp8: floats from one z scale group to the next
    const float* row_w;         // routing weight per routed item r (scales z), or null
};

// Routing weight of padded row p (1 without row weights; padding rows 0).
__device__ __forceinline__ float gemm1_row_w(const Gemm1Args& g, int64_t p)
{
    if (!g.row_w)
        return 1.0f;
    const int sid = g.s.sorted[p];
    return (sid < g.s.sentinel && in_bounds(sid, g.s.sentinel, g.s.status)) ? g.row_w[sid] : 0.0f;
}

struct Gemm2Args {
    Sched s;
    const void* z;
    const float* z_scale;       // fp8: [I/128][zs_ld] (group-major)
    int64_t zs_ld;
    const void* w2;             // [E, I, H], or packed blocks (bf16 / fp8 block layouts)
    int w_packed;               // 1: w2 is in the packed block layout
    const float* w2_scale;      // fp8: [E, H], or block-wise [E][ceil(H/128)][I/128];
                                // WNA16: [E][ceil(I/G)][H] group scales
    const uint8_t* w2_zero;     // WNA16: zero points like w2_scale, or null
    int wq_gsh;                 // WNA16: log2(K rows per scale group / 32)
    int blk;                    // fp8: block-wise scales
    const void* b2;             // [E, H] or null
    int bias_dt;
    int H, I;
    int out_mode;               // 1: out[sorted[p]] (out_dt, batched slabs); 2: float o[p]
    int out_dt;
    int T;                      // batched: rows per expert slab
    void* out;
    int ksplit;                 // 2: column block ntile = 2 c + h covers K half h;
    float* out2;                //    half 1 writes its float partials here, without bias
    int vec_out;                // bf16 out rows stored as 8-byte pieces of 4 values
                                // (quad_transpose) instead of one value a lane
};

// ---------------------------------------------------------------- tile schedule
// Persistent, XCD-aware schedule.  Workgroups are dealt round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8), so XCD x is given a contiguous
// eighth of the R logical tiles (whole row chunks when there are many) and
// walks it with its own workgroups: neighbouring tiles run together on one
// XCD and share its L2.
//
// Sharing through L2 only works between tiles that stream the same operand
// within a few K stages of each other (at full HBM rate an XCD's 4 MB L2
// turns over in a few microseconds).  Two rules keep the tiles that share an
// operand in step:
//  - an expert's rows are split into its nch chunks as evenly as 16-row
//    strips allow (rather than full chunks plus a ragged tail), so the
//    chunks that share a weight tile have the same work and run at the same
//    speed;
//  - within an expert, tiles are ordered by groups of up to 8 chunks, then
//    column block, then the chunk in the group, so the tiles running at once
//    on an XCD form a block of about 8 chunks x 8 column blocks: each weight
//    tile is read by the group's chunks together and each activation chunk by
//    the neighbouring column blocks together.
struct TileRef {
    int e, r0, rows, ntile;     // expert, first padded row, real rows (>= 1), column block
    int base;                   // first padded row of the expert's run
    int nch;                    // row chunks of the expert (1: this tile alone reads its weights)
};

constexpr int TILE_GROUP = 8;   // chunks walked together over the column blocks

template <int CH>
struct TileIter {
    int L, hi, per, nt;

    __device__ __forceinline__ explicit TileIter(const Sched& s)
    {
        nt = s.n_tiles;
        const int C = s.chunk_off[s.E];
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        per = gridDim.x >> 3;
        // when an XCD's workgroups are a multiple of the column tiles (the
        // DeepSeek-like layer's W13 GEMM: 32 and 16) and there are 64 row
        // chunks or more, XCD x takes whole chunks: a chunk's column tiles
        // then run in one round of one XCD, and its activation rows are
        // fetched once.  Otherwise the tiles are shared out one by one (a
        // decode-sized load measured 17% slower on whole chunks).
        int lo;
        if (C >= 64 && per % nt == 0) {
            lo = (int)(((int64_t)C * xcd) >> 3) * nt;
            hi = (int)(((int64_t)C * (xcd + 1)) >> 3) * nt;
        } else {
            const int R = C * nt;
            lo = (int)(((int64_t)R * xcd) >> 3);
            hi = (int)(((int64_t)R * (xcd + 1)) >> 3);
        }
        L = lo + slot;
    }

    __device__ __forceinline__ bool next(const Sched& s, TileRef& t)
    {
        // the checked build skips a tile whose expert or rows lie outside the
        // workspace (the release build's tile table comes from align itself)
        while (!next_tile(s, t)) {
        }
        return t.rows > 0;
    }

    // false: tile skipped, try the next; true with t.rows == 0: no tiles left
    __device__ __forceinline__ bool next_tile(const Sched& s, TileRef& t)
    {
        if (L >= hi) {
            t.rows = 0;
            return true;
        }
        if (!in_bounds(L / nt, s.max_chunks, s.status)) {
            L += per;
            return false;
        }
        const int e = s.chunk_expert[L / nt];
        if (!in_bounds(e, s.E, s.status)) {
            L += per;
            return false;
        }
        const int c0 = s.chunk_off[e], nch = s.chunk_off[e + 1] - c0;
        const int local = L - c0 * nt;
        // chunk group: full groups of TILE_GROUP chunks, then the remainder
        const int full = nch / TILE_GROUP;
        int j, ntile;
        if (local < full * TILE_GROUP * nt) {
            const int grp = local / (TILE_GROUP * nt), rem = local - grp * TILE_GROUP * nt;
            ntile = rem / TILE_GROUP;
            j = grp * TILE_GROUP + rem % TILE_GROUP;
        } else {
            const int rem = local - full * TILE_GROUP * nt, gc = nch - full * TILE_GROUP;
            ntile = rem / gc;
            j = full * TILE_GROUP + rem % gc;
        }
        // chunk j's rows: U = ceil(count / 16) strips dealt out evenly, the
        // first U % nch chunks one strip more.  nch = ceil(count / CH) makes
        // every chunk hold between 1 and CH rows, and starts stay 16-row aligned.
        const int cnt = s.counts[e], U = (cnt + 15) >> 4, q = U / nch, extra = U - q * nch;
        const int u0 = j * q + min(j, extra);
        const int base = s.offsets[e];
        t = TileRef{e, base + 16 * u0, min(16 * (q + (j < extra)), cnt - 16 * u0), ntile, base,
                    nch};
        L += per;
        if constexpr (CHECKED) {
            if (!(t.rows > 0 && in_bounds(t.r0, s.cap, s.status) &&
                  in_bounds((int64_t)t.r0 + t.rows - 1, s.cap, s.status)))
                return false;
        }
        return true;
    }
};

// f(e, row0, rows, ntile) for every tile of this workgroup.
template <int CH, typename F>
__device__ __forceinline__ void for_each_tile(const Sched& s, F&& f)
{
    TileIter<CH> it(s);
    TileRef t;
    while (it.next(s, t))
        f(t.e, t.r0, t.rows, t.ntile);
}

// ---------------------------------------------------------------- LDS DMA
// 16 zero bytes: the DMA source of padding rows and out-of-range chunks
static __device__ __attribute__((aligned(16))) int32_t g_zero16[4] = {0, 0, 0, 0};

__device__ __forceinline__ uint32_t lds_u32(const void* p)
{
    return (uint32_t)(uintptr_t)LDS_PTR(const char, p);
}

// M0 is a reserved register: the compiler never allocates it, and in these
// kernels no other instruction reads it, so it needs no clobber.
__device__ __forceinline__ void dma16(const char* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
                 : "memory");
}

// The same with the non-temporal cache policy: for weights that no other
// tile reads, so that streaming them does not evict the operands that
// neighbouring tiles share through L2.
__device__ __forceinline__ void dma16_nt(const char* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
                 : "memory");
}

// 4 bytes a lane: LDS byte lds + 4 l receives lane l's word.
__device__ __forceinline__ void dma4(const char* g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    // vmcnt[3:0], expcnt[6:4] (7: no wait), lgkmcnt[11:8] (15: no wait), vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The DMA ring over the K stages of one tile.  dma_prologue issues stages
// 0 .. NS-2; dma_mainloop then, per stage, waits for it, refills the slot
// freed one iteration earlier and hands the stage to compute().  Every
// iteration issues exactly one stage (a zero-page filler once the real stages
// run out), so when stage kt is awaited exactly NS - 2 stages of D DMAs per
// wave were issued after it: one constant wait serves every iteration and the
// loop body stays one basic block (branches in it make the register
// allocator copy the accumulators between VGPRs and AGPRs).  The loop ends
// drained, with every wave past its last LDS read, so the next tile's
// prologue may refill the ring at once.
// The stages run over [kb, ke) (K / 64 rounded up; a K-split half covers part).
template <typename S, typename Src>
__device__ __forceinline__ void dma_prologue(const Src& src, char* ring, int kb, int ke, int wave)
{
    const uint32_t ring_lds = lds_u32(ring);
#pragma unroll
    for (int st = 0; st < S::NS - 1; ++st)
        src.issue(kb + st, ring_lds + st * S::STAGE, ring_lds + S::NS * S::STAGE, wave,
                  kb + st < ke);
}

template <typename S, typename Src, typename F>
__device__ __forceinline__ void dma_mainloop(const Src& src, char* ring, int kb, int ke, int wave,
                                             F&& compute)
{
    const uint32_t ring_lds = lds_u32(ring);
    int slot = 0;                                   // (kt - kb) % NS
    for (int kt = kb; kt < ke; ++kt) {
        wait_vmcnt<(S::NS - 2) * S::D>();
        __syncthreads();
        // the slot refilled here was last read in iteration kt - 1, which every
        // wave finished before the barrier
        const int nx = kt + S::NS - 1;
        const int nslot = (slot == 0) ? S::NS - 1 : slot - 1;   // (nx - kb) % NS
        src.issue(nx, ring_lds + nslot * S::STAGE, ring_lds + S::NS * S::STAGE, wave, nx < ke);
        compute(ring + slot * S::STAGE);
        slot = (slot == S::NS - 1) ? 0 : slot + 1;
    }
    wait_vmcnt<0>();                                // the fillers land before the ring is reused
    __syncthreads();
}

// A compile-time int argument (the bounds of a DMA range).
template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<i>{}) for i = B .. E - 1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// The same ring with the refill handed to compute(stage, issue): compute
// calls issue(IC<lo>{}, IC<hi>{}) for consecutive ranges that cover the D
// DMAs of the refill exactly once, where it wants them among its fragment
// reads and MFMAs.  The refill is the same as dma_mainloop's, only later in
// the iteration, so one constant wait still serves every iteration.
template <typename S, typename Src, typename F>
__device__ __forceinline__ void dma_mainloop_split(const Src& src, char* ring, int kb, int ke,
                                                   int wave, F&& compute)
{
    const uint32_t ring_lds = lds_u32(ring);
    int slot = 0;                                   // (kt - kb) % NS
    for (int kt = kb; kt < ke; ++kt) {
        wait_vmcnt<(S::NS - 2) * S::D>();
        __syncthreads();
        const int nx = kt + S::NS - 1;
        const int nslot = (slot == 0) ? S::NS - 1 : slot - 1;   // (nx - kb) % NS
        const uint32_t dst = ring_lds + nslot * S::STAGE;
        const bool live = nx < ke;
        auto issue = [&](auto lo, auto hi) {
            src.template issue_part<decltype(lo)::value, decltype(hi)::value>(
                nx, dst, ring_lds + S::NS * S::STAGE, wave, live);
        };
        compute(ring + slot * S::STAGE, issue);
        slot = (slot == S::NS - 1) ? 0 : slot + 1;
    }
    wait_vmcnt<0>();
    __syncthreads();
}

// Source row of real tile row `row` (< rows) for GEMM1's A (activations):
// the routed token's row, or the padded position itself (a_ident).
__device__ __forceinline__ int64_t gemm1_src_row(const Gemm1Args& g, int r0, int row)
{
    const int64_t p = (int64_t)r0 + row;
    if (g.a_ident)
        return p;
    const int sid = g.s.sorted[p];
    return in_bounds(sid, g.s.sentinel, g.s.status) ? (int64_t)(sid / g.a_div) : -1;
}

// Makes the compiler hold v in a register here.  Values loaded from global
// memory ahead of time are pinned this way right after the ring has drained,
// so that the compiler's wait for them (it does not see the DMAs) costs
// nothing instead of stalling behind the next tile's DMAs.
template <typename T>
__device__ __forceinline__ void pin(const T& v)
{
    asm volatile("" : : "v"(v));
}

// Persistent grid: every workgroup the device holds at once (a multiple of
// the 8 XCDs), capped by the largest possible tile count.  Each kernel
// instance queries its occupancy once per device; `cache` is that instance's
// per-device slot array (zero = not yet known).  Two threads may both query
// and store: they store the same value.
template <typename K>
static unsigned persistent_grid(K kernel, int64_t max_tiles, std::atomic<int>* cache,
                                const Plan& P, int threads = 256)
{
    const int slot = (P.dev >= 0 && P.dev < MAX_DEVICES) ? P.dev : 0;
    int per_cu = cache[slot].load(std::memory_order_relaxed);
    if (per_cu == 0) {
        int occ = 0;
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0);
        per_cu = occ > 0 ? occ : 1;
        cache[slot].store(per_cu, std::memory_order_relaxed);
    }
    int64_t g = (int64_t)P.cus * per_cu;
    const int64_t cap = (max_tiles + 7) / 8 * 8;
    if (g > cap)
        g = cap;
    g = (g + 7) / 8 * 8;
    return (unsigned)(g < 8 ? 8 : g);
}


// fp8 GEMMs on packed fp8 weights (moe_gemm_fp8.hip)
hipError_t launch_gemm1_fp8(const Gemm1Args& a, const Plan& P, hipStream_t s);
hipError_t launch_gemm2_fp8(const Gemm2Args& a, const Plan& P, hipStream_t s);

}  // namespace moe
