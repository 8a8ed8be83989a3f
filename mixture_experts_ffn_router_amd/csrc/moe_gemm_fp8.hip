// fp8 (OCP E4M3FN) grouped expert GEMMs on packed fp8 weights, gfx950.
//
// Same organisation as the bf16 path (FlagGems walkthrough, "fused_moe_kernel"
// section; its "FP8 W8A8" section for the scales): one workgroup computes one
// tile of one expert's sorted rows x a block of output columns, float32
// accumulation, dequant / bias / activation / requant in the epilogue.
//
//   GEMM1: h = (sum_k qa[row, k] qw13[e, k, n]) * sa[row] * sw13[e, n] + b13[e, n]
//          z = SiLU(h_gate) * h_up, requantised per (row, 128 z columns)
//   GEMM2: o = (sum_g sz[row, g] sum_{k in g} qz[row, k] qw2[e, k, c]) * sw2[e, c] + b2
// Block-wise scales (BW; the same section's block-wise granularity): each
// 128-deep K block g of a product is scaled by its own activation and weight
// block scales, h = sum_g sa[row, g] sw13[e, n / 128, g] sum_{k in g} qa qw13,
// and likewise in GEMM2 with sz[row, g] sw2[e, c / 128, g].  A K stage is one
// such block, so each stage's MFMA products are scaled before they are
// accumulated; the scales of the stage arrive by DMA with its operands.
//
// With about 770 rows per expert these contractions are MFMA-bound.  A tile is
// F8_ROWS rows x 256 weight columns on 8 waves (2 x 4), each wave F8_ROWS / 2
// rows x 64 columns: (F8_ROWS / 32) x 4 MFMA tiles of
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales) sharing their A and B
// fragments within a 128-deep K stage.  One workgroup per CU; the ring holds
// as many stages as fit in LDS.
//
// Both operands are K-contiguous in LDS (128 bytes = one K stage per row or
// column), so A and B fragments are read the same way: lane l takes row /
// column l % 16 and the 32 K bytes (l / 16) * 32 .. as two 16-byte reads.
// The 16-byte chunk q of row / column r sits in slot
// (q / 2 + 4 (q % 2)) ^ ((r >> 1) & 7): the even chunks (the first reads of
// the four lane groups) fill slots 0-3 and the odd ones slots 4-7 before the
// row's XOR.  Measured with the LDS bank-conflict counter on gfx950, each of
// the two fragment reads is then conflict free (q ^ ((r >> 1) & 7) costs 4
// extra cycles per read).  Activations arrive that way by DMA of their
// natural [rows, K] layout; the weights are packed once into blocks that
// hold them that way (moe_pack_weights).
#include "moe_gemm_common.h"

namespace moe {

// Packed fp8 weight block: 128 weight columns x 128 K values (16 KiB); column
// c is 128 contiguous K bytes whose 16-byte chunk q sits in slot f8_slot(q, c).
constexpr int F8_BLOCK = 128 * 128;

// Slot of 16-byte K chunk q of row / column r, and its inverse: the chunk in slot sl.
__device__ __forceinline__ int f8_slot(int q, int r)
{
    return ((q >> 1) | ((q & 1) << 2)) ^ ((r >> 1) & 7);
}
__device__ __forceinline__ int f8_chunk(int sl, int r)
{
    const int p = sl ^ ((r >> 1) & 7);
    return ((p & 3) << 1) | (p >> 2);
}

template <bool ZS, bool BW = false>
struct F8S {
    static constexpr int NW = 8, NT = 64 * NW;   // 2 x 4 waves
    static constexpr int CG = 4;                  // column groups of waves
    static constexpr int FMW = F8_ROWS / 32;      // 16-row strips per wave
    static constexpr int FN = 4;                  // 16-column fragments per wave
    static constexpr int CH = 2 * FMW * 16;       // rows per tile
    static constexpr int BN = CG * FN * 16;       // 256 weight columns
    static constexpr int NB = BN / 128;           // weight blocks per K stage
    static constexpr int A_BYTES = CH * 128, B_BYTES = NB * F8_BLOCK;
    // per-stage scales after the operands:
    //   GEMM2: the z scales of the stage's rows, one 1 KiB DMA (256 rows' worth;
    //     the scale rows are padded so that the read stays in bounds);
    //   BW GEMM1: the rows' activation block scales (2 x 256 B, one float per
    //     lane), then the gate / up weight block scales (256 B);
    //   BW GEMM2: the two weight block scales of the tile's columns (256 B).
    static constexpr int SA_OFF = 0, SW_OFF = ZS ? 1024 : 512;
    static constexpr int S_BYTES = ZS ? (BW ? 1280 : 1024) : (BW ? 768 : 0);
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int NS = (3 * STAGE <= 150 * 1024) ? 3 : 2;   // ring stages
    static constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;
    // DMAs per wave per stage; wave 0 also issues the z-scale DMA of GEMM2,
    // so with 3 stages GEMM2 waits on a count that covers wave 0's extra one
    static constexpr int D = A_PW + B_PW;
    static constexpr int RING = NS * STAGE;
    static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "DMA split");
    static_assert(CH * 4 <= 1024, "z scales of a stage are one DMA");
};

// DMA sources of one fp8 tile.  Wave w issues A DMAs i = w + 8 j (tile rows
// 8i .. 8i+7, lane l: row 8i + l/8, K chunk f8_chunk(l % 8, row)), weight DMAs
// i = w + 8 j (block i / 16, its KiB i % 16, linear) and, for GEMM2, wave 0
// one DMA of the stage's z scales.  BW: GEMM1 waves 0 and 1 gather the
// activation block scales of tile rows 64 w + l (4 bytes a lane) and wave 2
// the gate / up weight block scales (lanes 0, 1); GEMM2 wave 1 the weight
// block scales of the tile's two 128-column blocks (lanes 0, 1).  Those waves
// issue one DMA more than the others; each wave waits on its own count, and
// the shared constant (the others' count) only makes them wait a little
// longer, never too little.
template <bool ZS, bool BW = false>
struct F8Src {
    typedef F8S<ZS, BW> S;
    const char* ap[S::A_PW];    // this lane's A chunk at K stage 0, null: padding row
    const char* wb[S::NB];      // packed block of K stage 0 per tile block, null past N
    int64_t w_stage;            // bytes from one K stage's blocks to the next
    const char* zs;             // GEMM2: this lane's 16 bytes of the stage-0 z scales
    int64_t zs_stage;           // bytes from one z scale group to the next
    const char* as;             // BW GEMM1: this lane's activation scale at stage 0 (null: none)
    const char* bs;             // BW: this lane's weight block scale at stage 0 (null: none)
    int K;                      // contraction length
    bool nt;                    // the weights are read by this tile alone: non-temporal DMAs

    __device__ __forceinline__ void issue(int kt, uint32_t lds, uint32_t spare, int wave,
                                          bool live) const
    {
        issue_p<false>(kt, lds, spare, wave, live);
    }

    // NT: the weight DMAs with the non-temporal policy
    template <bool NT>
    __device__ __forceinline__ void issue_p(int kt, uint32_t lds, uint32_t spare, int wave,
                                            bool live) const
    {
        issue_part_p<NT, 0, S::D>(kt, lds, spare, wave, live);
    }

    template <int J0, int J1>
    __device__ __forceinline__ void issue_part(int kt, uint32_t lds, uint32_t spare, int wave,
                                               bool live) const
    {
        issue_part_p<false, J0, J1>(kt, lds, spare, wave, live);
    }

    // DMAs [J0, J1) of the wave's D for stage kt: the A DMAs first, then the
    // weight DMAs; the range that ends at D also carries the scale DMAs
    template <bool NT, int J0, int J1>
    __device__ __forceinline__ void issue_part_p(int kt, uint32_t lds, uint32_t, int wave,
                                                 bool live) const
    {
        static_assert(0 <= J0 && J0 <= J1 && J1 <= S::D, "DMA range");
        const int lane = threadIdx.x & 63;
        const char* zero = (const char*)g_zero16;
#pragma unroll
        for (int j = J0; j < J1 && j < S::A_PW; ++j) {
            const int i = wave + S::NW * j;
            const int row = 8 * i + (lane >> 3);
            const int c = f8_chunk(lane & 7, row);
            const bool ok = live && ap[j] && kt * 128 + c * 16 < K;
            dma16(ok ? ap[j] + kt * 128 : zero, lds + i * 1024);
        }
#pragma unroll
        for (int jb = (J0 > S::A_PW ? J0 : S::A_PW); jb < J1; ++jb) {
            const int j = jb - S::A_PW;
            const int i = wave + S::NW * j;          // block i >> 4 == j >> 1 (wave < 8)
            const char* w = wb[(j * S::NW) >> 4];
            const char* p = (live && w) ? w + kt * w_stage + (i & 15) * 1024 + lane * 16 : zero;
            if constexpr (NT)
                dma16_nt(p, lds + S::A_BYTES + i * 1024);
            else
                dma16(p, lds + S::A_BYTES + i * 1024);
        }
        if constexpr (J1 < S::D)
            return;
        if constexpr (ZS) {
            if (wave == 0)
                dma16(live ? zs + kt * zs_stage : zero, lds + S::A_BYTES + S::B_BYTES);
        }
        if constexpr (BW) {
            // block scales: consecutive K blocks are consecutive floats
            const uint32_t sl = lds + S::A_BYTES + S::B_BYTES;
            if constexpr (!ZS) {
                if (wave < 2)
                    dma4((live && as) ? as + kt * 4 : zero, sl + S::SA_OFF + wave * 256);
                else if (wave == 2)
                    dma4((live && bs) ? bs + kt * 4 : zero, sl + S::SW_OFF);
            } else {
                if (wave == 1)
                    dma4((live && bs) ? bs + kt * 4 : zero, sl + S::SW_OFF);
            }
        }
    }
};

// 32 K bytes of row / column r (l % 16 of a fragment) for lane group g = l / 16.
__device__ __forceinline__ i32x8 f8_frag(const char* base, int r, int g)
{
    const char* p = base + r * 128;
    const i32x4 lo = *(const i32x4*)(p + 16 * f8_slot(2 * g, r));
    const i32x4 hi = *(const i32x4*)(p + 16 * f8_slot(2 * g + 1, r));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f32x4 mma_f8(const i32x8& a, const i32x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One K stage for wave (rg, cg): B fragment fn is column bcol[fn] (a multiple
// of 16) of the stage's weight tile; the first NM strips of the wave's four
// hold real rows.  ZS: every product is scaled by its row's z scale before
// it is accumulated (one MFMA spans exactly one 128-column z group).  BW:
// scaled by the row's activation block scale times the weight block scale
// of its columns (GEMM1: fragments 0, 1 are gate columns, 2, 3 up columns;
// GEMM2: the wave's 64 columns lie in block bcol[0] / 128 of the tile).
// The D DMAs of the ring's refill go out through issue(lo, hi), one share
// after each strip's MFMAs, so that their issue overlaps MFMA work instead
// of delaying the stage's fragment reads.
template <bool ZS, bool BW, int NM, typename Issue>
__device__ __forceinline__ void f8_stage(const char* st, int rg, const int (&bcol)[4], int lane,
                                         f32x4 (&acc)[F8_ROWS / 32][4], Issue&& issue)
{
    typedef F8S<ZS, BW> S;
    const int s16 = lane & 15, g = lane >> 4;
    const char* As = st + rg * (S::FMW * 16 * 128);
    const char* Bs = st + S::A_BYTES;
    const char* Ss = st + S::A_BYTES + S::B_BYTES;
    i32x8 b[S::FN];
#pragma unroll
    for (int fn = 0; fn < S::FN; ++fn)
        b[fn] = f8_frag(Bs + bcol[fn] * 128, s16, g);
    // strip fm's A fragment is read before strip fm - 1's MFMAs (two held at a time)
    i32x8 a[2];
    a[0] = f8_frag(As, s16, g);
    auto next_a = [&](auto fmc) {
        constexpr int fm = decltype(fmc)::value;
        if constexpr (fm + 1 < NM)
            a[(fm + 1) & 1] = f8_frag(As + (fm + 1) * 2048, s16, g);
    };
    // one share of the refill after strip fm's MFMAs (SPREAD: the plain
    // GEMM1), else the whole refill first: the scaled stages run out of
    // registers holding the DMA addresses across their MFMAs, and GEMM2
    // measured no faster spread
    constexpr bool SPREAD = !BW && !ZS;
    if constexpr (!SPREAD)
        issue(IC<0>{}, IC<S::D>{});
    auto share = [&](auto fmc) {
        constexpr int fm = decltype(fmc)::value;
        constexpr int lo = fm * S::D / NM, hi = (fm + 1) * S::D / NM;
        if constexpr (SPREAD && hi > lo)
            issue(IC<lo>{}, IC<hi>{});
        if constexpr (SPREAD)
            __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (ZS) {
        // GEMM2's scaled products: strip fm's are scaled and accumulated after
        // strip fm + 1's MFMAs are issued, so the VALU never waits on a
        // product just made (each accumulator still takes one scaled product
        // per stage).  s0 scales fragments fn < FN / 2, s1 the others.  (The
        // block-scaled GEMM1 keeps the direct order: the extra products
        // would not fit its registers.)
        f32x4 tp[S::FN], s0p, s1p;
        static_for<0, NM>([&](auto fmc) {
            constexpr int fm = decltype(fmc)::value;
            const int row0 = rg * S::FMW * 16 + fm * 16 + g * 4;
            f32x4 sz = *(const f32x4*)(Ss + row0 * 4);
            if constexpr (BW) {
                const float sw = *(const float*)(Ss + S::SW_OFF + (bcol[0] >> 7) * 4);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sz[r] *= sw;
            }
            next_a(fmc);
            f32x4 t[S::FN];
#pragma unroll
            for (int fn = 0; fn < S::FN; ++fn)
                t[fn] = mma_f8(a[fm & 1], b[fn], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            if constexpr (fm > 0) {
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[fm - 1][fn][r] += tp[fn][r] * (fn < S::FN / 2 ? s0p[r] : s1p[r]);
            }
#pragma unroll
            for (int fn = 0; fn < S::FN; ++fn)
                tp[fn] = t[fn];
            s0p = sz;
            s1p = sz;
            share(fmc);
        });
#pragma unroll
        for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[NM - 1][fn][r] += tp[fn][r] * (fn < S::FN / 2 ? s0p[r] : s1p[r]);
    } else if constexpr (BW) {
        static_for<0, NM>([&](auto fmc) {
            constexpr int fm = decltype(fmc)::value;
            const int row0 = rg * S::FMW * 16 + fm * 16 + g * 4;
            const f32x4 sa = *(const f32x4*)(Ss + S::SA_OFF + row0 * 4);
            const float swg = *(const float*)(Ss + S::SW_OFF);
            const float swu = *(const float*)(Ss + S::SW_OFF + 4);
            f32x4 fg, fu;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fg[r] = sa[r] * swg;
                fu[r] = sa[r] * swu;
            }
            next_a(fmc);
#pragma unroll
            for (int fn = 0; fn < S::FN; ++fn) {
                const f32x4 t = mma_f8(a[fm & 1], b[fn], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[fm][fn][r] += t[r] * (fn < S::FN / 2 ? fg[r] : fu[r]);
            }
            share(fmc);
        });
    } else {
        static_for<0, NM>([&](auto fmc) {
            constexpr int fm = decltype(fmc)::value;
            next_a(fmc);
#pragma unroll
            for (int fn = 0; fn < S::FN; ++fn)
                acc[fm][fn] = mma_f8(a[fm & 1], b[fn], acc[fm][fn]);
            share(fmc);
        });
    }
}

// A tile's DMA source with its weight DMAs non-temporal.
template <typename Src>
struct F8NtSrc {
    const Src& s;
    __device__ __forceinline__ void issue(int kt, uint32_t lds, uint32_t spare, int wave,
                                          bool live) const
    {
        s.template issue_p<true>(kt, lds, spare, wave, live);
    }
    template <int J0, int J1>
    __device__ __forceinline__ void issue_part(int kt, uint32_t lds, uint32_t spare, int wave,
                                               bool live) const
    {
        s.template issue_part_p<true, J0, J1>(kt, lds, spare, wave, live);
    }
};

// The first stages of a tile's ring, with the tile's weight cache policy.
template <typename S, typename Src>
__device__ __forceinline__ void f8_prologue(const Src& src, char* ring, int nk, int wave)
{
    if (__builtin_amdgcn_readfirstlane(src.nt))
        dma_prologue<S>(F8NtSrc<Src>{src}, ring, 0, nk, wave);
    else
        dma_prologue<S>(src, ring, 0, nk, wave);
}

// The ring over [0, nk) with the MFMAs of the wave's first `live` strips;
// one instantiation per count and weight cache policy keeps the loop body
// branch free.
template <bool ZS, bool BW, int NM = F8_ROWS / 32>
__device__ __forceinline__ void f8_run(const F8Src<ZS, BW>& src, char* ring, int nk, int wave,
                                       int rg, const int (&bcol)[4], int lane,
                                       f32x4 (&acc)[F8_ROWS / 32][4], int live)
{
    typedef F8S<ZS, BW> S;
    auto loop = [&](const auto& ss) {
        if constexpr (NM == 0)
            dma_mainloop_split<S>(ss, ring, 0, nk, wave,
                                  [](const char*, auto&& issue) { issue(IC<0>{}, IC<S::D>{}); });
        else
            dma_mainloop_split<S>(ss, ring, 0, nk, wave, [&](const char* st, auto&& issue) {
                f8_stage<ZS, BW, NM>(st, rg, bcol, lane, acc, issue);
            });
    };
    if constexpr (NM > 0) {
        if (live < NM) {
            f8_run<ZS, BW, NM - 1>(src, ring, nk, wave, rg, bcol, lane, acc, live);
            return;
        }
    }
    if (__builtin_amdgcn_readfirstlane(src.nt))
        loop(F8NtSrc<F8Src<ZS, BW>>{src});
    else
        loop(src);
}

__device__ __forceinline__ void f8_zero(f32x4 (&acc)[F8_ROWS / 32][4])
{
#pragma unroll
    for (int fm = 0; fm < F8_ROWS / 32; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
            acc[fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// ---------------------------------------------------------------- GEMM1
// Tile (expert, row chunk, ntile): z columns 128 ntile .. +127, i.e. the
// gate and up columns of packed blocks 2 ntile and 2 ntile + 1 (each 64 gate
// + 64 up columns).  Wave (rg, cg) owns z columns 32 cg .. +31: gate
// fragments fn = 0, 1 and the matching up fragments fn = 2, 3.  The packing
// orders each 32 columns so that lane l of fragment f holds column
// 32 cg + 2 (l % 16) + f: a lane's two z columns of a row are adjacent.
struct F8G1Src {
    int srow[F8S<false>::A_PW];     // per-lane A source rows, -1: padding
    int sa_row;                     // thread t < CH: source row of tile row t, -1: none
    float rw;                       // thread t < CH: routing weight of tile row t (z scale)
};

__device__ __forceinline__ void f8_gemm1_rows(const Gemm1Args& g, const TileRef& t, int wave,
                                              int lane, F8G1Src& r)
{
    typedef F8S<false> S;
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        const int row = 8 * (wave + S::NW * j) + (lane >> 3);
        r.srow[j] = (row < t.rows) ? (int)gemm1_src_row(g, t.r0, row) : -1;
    }
    const int tr = threadIdx.x;
    r.sa_row = (tr < S::CH && tr < t.rows) ? (int)gemm1_src_row(g, t.r0, tr) : -1;
    r.rw = (tr < S::CH && tr < t.rows) ? gemm1_row_w(g, (int64_t)t.r0 + tr) : 0.0f;
}

template <bool BW>
__device__ __forceinline__ void f8_gemm1_src(const Gemm1Args& g, const TileRef& t,
                                             const F8G1Src& r, F8Src<false, BW>& d)
{
    typedef F8S<false, BW> S;
    const int H = g.H, I = g.I;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nblk = I / 64, nks = (H + 127) / 128;
    d.K = H;
    d.nt = __builtin_amdgcn_readfirstlane(t.nch) == 1;
    d.w_stage = nblk * F8_BLOCK;
    d.zs = nullptr;
    d.zs_stage = 0;
    d.as = d.bs = nullptr;
    if constexpr (BW) {
        // waves 0, 1: activation scales of tile rows 64 wave + lane (thread
        // index = tile row); wave 2, lanes 0 / 1: the gate / up weight blocks
        // of z columns 128 ntile .. (2I / 128 column blocks, nks K blocks)
        if (r.sa_row >= 0)
            d.as = (const char*)(g.a_scale + (int64_t)r.sa_row * g.a_sld);
        if (lane < 2) {
            const int64_t nb = (lane == 0) ? t.ntile : I / 128 + t.ntile;
            d.bs = (const char*)(g.w13_scale + ((int64_t)t.e * (2 * I / 128) + nb) * nks);
        }
    }
#pragma unroll
    for (int bb = 0; bb < S::NB; ++bb)
        d.wb[bb] = (const char*)g.w13 +
                   ((int64_t)t.e * nks * nblk + (int64_t)t.ntile * S::NB + bb) * F8_BLOCK;
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        const int row = 8 * (wave + S::NW * j) + (lane >> 3);
        const int c = f8_chunk(lane & 7, row);
        d.ap[j] = (r.srow[j] >= 0) ? (const char*)g.a + (int64_t)r.srow[j] * H + c * 16
                                   : nullptr;
    }
}

template <bool BW>
__global__ void __launch_bounds__(512, 1) k_gemm1_f8(Gemm1Args g)
{
    typedef F8S<false, BW> S;
    __shared__ __attribute__((aligned(16))) char ring[S::RING];
    __shared__ __attribute__((aligned(16))) float rs[2][S::CH];    // activation row scales, by
                                                                    // tile parity
    __shared__ __attribute__((aligned(16))) float rws[2][S::CH];   // routing weights of the rows
                                                                    // (z scale; 1 without)
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / S::CG, cg = wave % S::CG;
    const int I = g.I, N = 2 * I;
    const int s16 = lane & 15, g4 = lane >> 4;
    const int nk = (g.H + 127) / 128;

    TileIter<S::CH> it(g.s);
    TileRef cur;
    if (!it.next(g.s, cur))
        return;
    F8G1Src rows;
    f8_gemm1_rows(g, cur, wave, lane, rows);
    F8Src<false, BW> src;
    f8_gemm1_src<BW>(g, cur, rows, src);
    // per-row activation scale for the epilogue (block-wise: applied per stage)
    if (tid < S::CH) {
        rs[0][tid] = BW ? 1.0f : (rows.sa_row >= 0 ? g.a_scale[rows.sa_row] : 0.0f);
        rws[0][tid] = rows.rw;
    }
    f8_prologue<S>(src, ring, nk, wave);

    // B fragment columns within the stage's 256-column weight tile
    int bcol[4];
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
        const int zl = cg * 32 + (fn & 1) * 16;             // z column within the tile
        bcol[fn] = (zl / 64) * 128 + (fn >= 2 ? 64 : 0) + zl % 64;
    }

    int parity = 0;
    for (;;) {
        TileRef nxt;
        const bool more = it.next(g.s, nxt);
        if (more)
            f8_gemm1_rows(g, nxt, wave, lane, rows);
        float sn = BW ? 1.0f : 0.0f;               // the next tile's row scale (tid < CH)
        if (!BW && more && tid < S::CH && rows.sa_row >= 0)
            sn = g.a_scale[rows.sa_row];
        const int z0 = cur.ntile * 128;
        float sg[2], su[2], bg[2], bu[2];
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
            const int n = z0 + cg * 32 + 2 * s16 + fn;
            sg[fn] = BW ? 1.0f : g.w13_scale[(int64_t)cur.e * N + n];
            su[fn] = BW ? 1.0f : g.w13_scale[(int64_t)cur.e * N + I + n];
            bg[fn] = bu[fn] = 0.0f;
            if (g.b13) {
                bg[fn] = load_bias(g.b13, g.bias_dt, (int64_t)cur.e * N + n);
                bu[fn] = load_bias(g.b13, g.bias_dt, (int64_t)cur.e * N + I + n);
            }
        }
        f32x4 acc[F8_ROWS / 32][4];
        f8_zero(acc);
        const int strips = (cur.rows + 15) >> 4;
        f8_run<false, BW>(src, ring, nk, wave, rg, bcol, lane, acc,
                          min(max(strips - rg * S::FMW, 0), S::FMW));
        pin(sn);
        pin(rows.rw);
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
            pin(sg[fn]);
            pin(su[fn]);
            pin(bg[fn]);
            pin(bu[fn]);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < S::A_PW; ++j)
                pin(rows.srow[j]);
            f8_gemm1_src<BW>(g, nxt, rows, src);
            f8_prologue<S>(src, ring, nk, wave);
            if (tid < S::CH) {
                rs[parity ^ 1][tid] = sn;
                rws[parity ^ 1][tid] = rows.rw;
            }
        }

        // epilogue: z in registers, row amax across the 4 column waves through
        // LDS, fp8 codes staged in the ring slot no DMA touches before the next
        // tile's first barrier, then 16-byte row stores
        uint8_t* zst = (uint8_t*)(ring + (S::NS - 1) * S::STAGE);           // [CH][128]
        float* amx = (float*)(ring + (S::NS - 1) * S::STAGE + S::CH * 128);  // [CH][4 cg]
        static_assert(S::CH * 128 + S::CH * 16 + S::NW * 64 * 4 <= S::STAGE, "epilogue LDS");
        // pass 1: z of (strip fm, fragment fn < 2, row r) replaces the gate
        // accumulator (the routing weight is 1 without row weights); mb[v],
        // v = 4 fm + r, is the largest |z| of that row among this lane's two
        // columns, as float bits (non-negative floats order like their bits)
        static_assert(S::FMW == 4, "16 row values a lane");
        uint32_t mb[16];
#pragma unroll
        for (int fm = 0; fm < S::FMW; ++fm) {
            const int row0 = rg * S::FMW * 16 + fm * 16 + g4 * 4;
            const f32x4 sa = *(const f32x4*)&rs[parity][row0];
            const f32x4 rw = *(const f32x4*)&rws[parity][row0];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t m = 0;
#pragma unroll
                for (int fn = 0; fn < 2; ++fn) {
                    const float hg = acc[fm][fn][r] * sa[r] * sg[fn];
                    const float hu = acc[fm][fn + 2][r] * sa[r] * su[fn];
                    acc[fm][fn][r] = silu_mul(hg + bg[fn], hu + bu[fn]) * rw[r];
                    m = max(m, __float_as_uint(fabsf(acc[fm][fn][r])));
                }
                mb[fm * 4 + r] = m;
            }
        }
        // the 16 lanes of each lane row share rows: a reduce-scatter over them
        // (partners 15 - i, 7 - i, i ^ 2, i ^ 1) leaves lane i with the row
        // maximum of value v = i over this wave's 32 columns
        {
            const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t keep = b3 ? mb[k + 8] : mb[k], send = b3 ? mb[k] : mb[k + 8];
                mb[k] = max(keep, dpp_u32<DPP_MIRROR16>(send));
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t keep = b2 ? mb[k + 4] : mb[k], send = b2 ? mb[k] : mb[k + 4];
                mb[k] = max(keep, dpp_u32<DPP_MIRROR8>(send));
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t keep = b1 ? mb[k + 2] : mb[k], send = b1 ? mb[k] : mb[k + 2];
                mb[k] = max(keep, dpp_u32<DPP_XOR2>(send));
            }
            const uint32_t keep = b0 ? mb[1] : mb[0], send = b0 ? mb[0] : mb[1];
            const uint32_t m = max(keep, dpp_u32<DPP_XOR1>(send));
            // value v = s16: strip v / 4, row v % 4 of the lane row g4
            amx[(rg * S::FMW * 16 + (s16 >> 2) * 16 + g4 * 4 + (s16 & 3)) * 4 + cg] =
                __uint_as_float(m);
        }
        __syncthreads();
        // pass 2: lane i of each lane row forms the scale of value v = i (the
        // row whose maxima it holds) and passes the reciprocal to its lane row
        // through the wave's own LDS slots; then the codes, the lane's two
        // adjacent columns of a row as one 16-bit write
        float* rcs = amx + S::CH * 4 + wave * 64;                           // [4 g4][16 v]
        {
            const int row = rg * S::FMW * 16 + (s16 >> 2) * 16 + g4 * 4 + (s16 & 3);
            const f32x4 a4 = *(const f32x4*)(amx + row * 4);
            const float amax = fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3]));
            const float sc = zq_scale(amax);
            rcs[g4 * 16 + s16] = __builtin_amdgcn_rcpf(sc);
            if (cg == 0 && row < cur.rows)
                g.z_scale[(int64_t)cur.ntile * g.zs_ld + cur.r0 + row] = sc;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int fm = 0; fm < S::FMW; ++fm) {
            const f32x4 rc = *(const f32x4*)(rcs + g4 * 16 + fm * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rg * S::FMW * 16 + fm * 16 + g4 * 4 + r;
                *(uint16_t*)(zst + row * 128 + cg * 32 + 2 * s16) =
                    (uint16_t)cvt_fp8x2(acc[fm][0][r] * rc[r], acc[fm][1][r] * rc[r]);
            }
        }
        __syncthreads();
        for (int q = tid; q < cur.rows * 8; q += S::NT) {
            const int row = q >> 3, c = q & 7;
            *(i32x4*)((uint8_t*)g.z + ((int64_t)cur.r0 + row) * I + z0 + c * 16) =
                *(const i32x4*)(zst + row * 128 + c * 16);
        }
        if (!more)
            break;
        cur = nxt;
        parity ^= 1;
    }
}

// ---------------------------------------------------------------- GEMM2
// Tile (expert, row chunk, ntile): output columns 256 ntile .. +255 =
// packed blocks 2 ntile, 2 ntile + 1; wave (rg, cg) owns columns 64 cg .. +63.
// A rows are the padded positions (z written by GEMM1); the stage's z scales
// (group kt of the tile's rows) arrive with it.
template <bool BW>
__device__ __forceinline__ void f8_gemm2_src(const Gemm2Args& g, const TileRef& t, int wave,
                                             F8Src<true, BW>& d)
{
    typedef F8S<true, BW> S;
    const int H = g.H, I = g.I;
    const int lane = threadIdx.x & 63;
    const int64_t nblk = (H + 127) / 128, nks = I / 128;
    d.K = I;
    d.nt = __builtin_amdgcn_readfirstlane(t.nch) == 1;
    d.w_stage = nblk * F8_BLOCK;
    d.zs = (const char*)(g.z_scale + t.r0) + lane * 16;
    d.zs_stage = g.zs_ld * 4;
    d.as = d.bs = nullptr;
    if constexpr (BW) {
        // lanes 0 / 1: weight blocks 2 ntile, 2 ntile + 1 (none past H)
        const int64_t nb = 2 * (int64_t)t.ntile + lane;
        if (lane < 2 && nb < nblk)
            d.bs = (const char*)(g.w2_scale + ((int64_t)t.e * nblk + nb) * nks);
    }
#pragma unroll
    for (int bb = 0; bb < S::NB; ++bb) {
        const int64_t jb = (int64_t)t.ntile * S::NB + bb;
        d.wb[bb] = (jb < nblk) ? (const char*)g.w2 + ((int64_t)t.e * nks * nblk + jb) * F8_BLOCK
                               : nullptr;
    }
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        const int row = 8 * (wave + S::NW * j) + (lane >> 3);
        const int c = f8_chunk(lane & 7, row);
        d.ap[j] = (row < t.rows) ? (const char*)g.z + ((int64_t)t.r0 + row) * I + c * 16
                                 : nullptr;
    }
}

template <bool BW>
__global__ void __launch_bounds__(512, 1) k_gemm2_f8(Gemm2Args g)
{
    typedef F8S<true, BW> S;
    __shared__ __attribute__((aligned(16))) char ring[S::RING];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / S::CG, cg = wave % S::CG;
    const int H = g.H;
    const int s16 = lane & 15, g4 = lane >> 4;
    const int nk = g.I / 128;

    TileIter<S::CH> it(g.s);
    TileRef cur;
    if (!it.next(g.s, cur))
        return;
    F8Src<true, BW> src;
    f8_gemm2_src<BW>(g, cur, wave, src);
    f8_prologue<S>(src, ring, nk, wave);
    int bcol[4];
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
        bcol[fn] = cg * 64 + fn * 16;

    for (;;) {
        TileRef nxt;
        const bool more = it.next(g.s, nxt);
        const int c0 = cur.ntile * S::BN;
        const int strips = (cur.rows + 15) >> 4;
        const int64_t dst0 = (g.out_mode == 2) ? (int64_t)cur.r0
                                               : (int64_t)cur.e * g.T + (cur.r0 - cur.base);
        // (checked build: the output rows must lie in o, or in the slabs)
        const bool dst_ok =
            in_bounds(dst0, g.out_mode == 2 ? g.s.cap : (int64_t)g.s.E * g.T, g.s.status) &&
            in_bounds(dst0 + cur.rows - 1, g.out_mode == 2 ? g.s.cap : (int64_t)g.s.E * g.T,
                      g.s.status);
        float sw[4], bias[4];
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
            const int c = c0 + bcol[fn] + s16;
            sw[fn] = (c >= H) ? 0.0f : BW ? 1.0f : g.w2_scale[(int64_t)cur.e * H + c];
            bias[fn] = (g.b2 && c < H) ? load_bias(g.b2, g.bias_dt, (int64_t)cur.e * H + c) : 0.0f;
        }
        f32x4 acc[F8_ROWS / 32][4];
        f8_zero(acc);
        f8_run<true, BW>(src, ring, nk, wave, rg, bcol, lane, acc,
                         min(max(strips - rg * S::FMW, 0), S::FMW));
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
            pin(sw[fn]);
            pin(bias[fn]);
        }
        if (more) {
            f8_gemm2_src<BW>(g, nxt, wave, src);
            f8_prologue<S>(src, ring, nk, wave);
        }
        // epilogue straight from the accumulators: one strip at a time
        const bool obf = g.out_mode == 1 && g.out_dt == MOE_BF16;
        if (g.vec_out) {
            // each fragment's 4 x 4 lane quads transposed: lane (g4, 4a + q)
            // stores row 4 g4 + q of the strip, columns 4a .. 4a + 3
            const int q = s16 & 3;
#pragma unroll
            for (int fm = 0; fm < S::FMW; ++fm) {
                const int strip = rg * S::FMW + fm;
                if (strip >= strips || !dst_ok)
                    continue;
                const int row = strip * 16 + g4 * 4 + q;
                const int64_t base = (dst0 + row) * H + c0 + (s16 & ~3);
#pragma unroll
                for (int fn = 0; fn < 4; ++fn) {
                    if (c0 + bcol[fn] >= H)
                        continue;
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = acc[fm][fn][r] * sw[fn] + bias[fn];
                    quad_transpose(v, lane);
                    if (row < cur.rows)
                        store_row4(g.out, base + bcol[fn], obf, v);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
        for (int fm = 0; fm < S::FMW; ++fm) {
            const int strip = rg * S::FMW + fm;
            if (strip >= strips || !dst_ok)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = strip * 16 + g4 * 4 + r;
                if (row >= cur.rows)
                    continue;
                const int64_t base = (dst0 + row) * H;
#pragma unroll
                for (int fn = 0; fn < 4; ++fn) {
                    const int c = c0 + bcol[fn] + s16;
                    if (c >= H)
                        continue;
                    const float v = acc[fm][fn][r] * sw[fn] + bias[fn];
                    if (obf)
                        ((u16*)g.out)[base + c] = f32_to_bf16(v);
                    else
                        ((float*)g.out)[base + c] = v;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
        if (!more)
            break;
        cur = nxt;
    }
}

// ---------------------------------------------------------------- packing
// One-time re-layout of fp8 expert weights into the K-contiguous blocks
// above.  One thread per 16-byte slot of the output: it gathers 16 K values
// of one weight column; rows past K and columns past N are zeros.
//   w13 [E, H, 2I]: block (e, kt, j), kt < ceil(H/128), j < I/64: columns
//     0-63 = gate columns 64 j .., 64-127 = up columns I + 64 j .., each half
//     in 32-column groups whose column 16 f + s is the group's column 2 s + f
//   w2 [E, I, H]: block (e, kt, j), kt < I/128, j < ceil(H/128): columns 128 j ..
template <bool W13>
__global__ void __launch_bounds__(256) k_pack_f8(const uint8_t* __restrict__ w, int H, int I,
                                                 i32x4* __restrict__ out, int64_t slots)
{
    const int K = W13 ? H : I, ncol = W13 ? 2 * I : H;
    const int64_t nblk = W13 ? I / 64 : (H + 127) / 128, nks = (K + 127) / 128;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < slots;
         q += (int64_t)gridDim.x * 256) {
        const int sl = (int)(q & 7), c = (int)((q >> 3) & 127);
        const int64_t b = q >> 10;                      // block (e, kt, j)
        const int j = (int)(b % nblk);
        const int kt = (int)((b / nblk) % nks);
        const int64_t e = b / nblk / nks;
        const int chunk = f8_chunk(sl, c);             // the K chunk slot sl holds
        int col;
        bool valid;
        if constexpr (W13) {
            // within each 32 columns of a half, block column 16 f + s holds
            // weight column 2 s + f (see the GEMM1 epilogue)
            const int h = c & 63, pc = (h & 32) | ((h & 15) << 1) | ((h >> 4) & 1);
            col = (c < 64) ? 64 * j + pc : I + 64 * j + pc;
            valid = true;
        } else {
            col = 128 * j + c;
            valid = col < H;
        }
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        if (valid) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int row = kt * 128 + chunk * 16 + k;
                const uint32_t byte =
                    (row < K) ? w[((int64_t)e * K + row) * ncol + col] : 0u;
                v[k >> 2] |= byte << (8 * (k & 3));
            }
        }
        out[q] = i32x4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
    }
}

hipError_t launch_pack_weights_fp8(int E, int H, int I, const void* w13, const void* w2,
                                   void* p13, void* p2, hipStream_t s)
{
    const int64_t s13 = (int64_t)E * ((H + 127) / 128) * (I / 64) * (F8_BLOCK / 16);
    const int64_t s2 = (int64_t)E * (I / 128) * ((H + 127) / 128) * (F8_BLOCK / 16);
    auto grid = [](int64_t slots) {
        const int64_t b = (slots + 255) / 256;
        return (unsigned)(b < 16384 ? b : 16384);
    };
    hipLaunchKernelGGL(k_pack_f8<true>, dim3(grid(s13)), dim3(256), 0, s, (const uint8_t*)w13, H,
                       I, (i32x4*)p13, s13);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(k_pack_f8<false>, dim3(grid(s2)), dim3(256), 0, s, (const uint8_t*)w2, H,
                       I, (i32x4*)p2, s2);
    return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
template <bool BW>
static hipError_t run_gemm1_f8(const Gemm1Args& a, const Plan& P, hipStream_t s)
{
    typedef F8S<false, BW> S;
    Gemm1Args g = a;
    g.s.n_tiles = a.I / 128;
    auto kern = k_gemm1_f8<BW>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P, S::NT)),
        block(S::NT);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

template <bool BW>
static hipError_t run_gemm2_f8(const Gemm2Args& a, const Plan& P, hipStream_t s)
{
    typedef F8S<true, BW> S;
    Gemm2Args g = a;
    g.s.n_tiles = (a.H + S::BN - 1) / S::BN;
    auto kern = k_gemm2_f8<BW>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P, S::NT)),
        block(S::NT);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

hipError_t launch_gemm1_fp8(const Gemm1Args& a, const Plan& P, hipStream_t s)
{
    return a.blk ? run_gemm1_f8<true>(a, P, s) : run_gemm1_f8<false>(a, P, s);
}

hipError_t launch_gemm2_fp8(const Gemm2Args& a, const Plan& P, hipStream_t s)
{
    return a.blk ? run_gemm2_f8<true>(a, P, s) : run_gemm2_f8<false>(a, P, s);
}

}  // namespace moe
