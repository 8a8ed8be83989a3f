// Grouped expert GEMMs of the fused MoE forward on gfx950 MFMA.
//
// The organisation follows the FlagGems walkthrough ("fused_moe_kernel"
// section and sec. 1.3): routed items are sorted by expert and padded
// (align kernel); one workgroup computes one tile of one expert's rows x a
// block of output columns; the accumulator is float32 and is cast at the
// output; dequant, bias and activation are fused into the epilogue.
//
//   GEMM1: h[p, n] = sum_k A[row(p), k] * w13[e, k, n] (+ b13[e, n]);
//          z[p, i] = SiLU(h[p, i]) * h[p, I + i]            (gate | up halves)
//   GEMM2: o[p, c] = sum_i z[p, i] * w2[e, i, c] (+ b2[e, c])
//
// Tiles.  An expert's rows (padded to 16) are cut into chunks of CH rows;
// a tile is (expert, chunk, column block).  The four waves share the tile's
// rows and split its columns.  Rows past the expert's count are staged as
// zeros rather than skipped, which keeps the MFMA loop free of branches so
// the fragment reads pipeline; their outputs are never stored.  With CH = 160
// an expert of up to 160 rows is one tile per column block, and each weight
// tile crosses HBM and LDS once.
//
// Data movement (gfx950).  LDS writes are the scarce resource (a b128 write
// moves about half the bytes per clock of a b128 read), so every weight byte
// is written to LDS once and read back once: the four waves split the
// columns of a tile and share its rows.
//   * A (activation rows for GEMM1, z rows for GEMM2, K-contiguous) and B
//     (weights [K, N], N-contiguous) go global -> registers -> LDS in
//     coalesced 16-byte chunks, double buffered: the next K stage's chunks
//     are in flight while the current stage feeds the MFMAs.
//   * A fragments are K-contiguous LDS reads (lane l: row l%16, K elements
//     (l/16)*EPL ..); B fragments use the transposing LDS reads
//     (ds_read_b64_tr_b16 / _b8) that hand each lane consecutive K values of
//     one column.  Row strides are padded by 16 bytes against bank conflicts.
//   * A K stage is 128 bytes of each A row (64 bf16 / 128 fp8 / 32 f32);
//     outputs are staged through LDS so global stores are 16-byte vectors.
#include "moe_gemm_common.h"

namespace moe {


// element size, K per MFMA, K elements per lane per MFMA, K per LDS stage
template <int DT>
struct GT;
template <>
struct GT<MOE_F32> {
    static constexpr int ES = 4, KM = 4, EPL = 1, BK = 32;
    typedef float Frag;
};
template <>
struct GT<MOE_BF16> {
    static constexpr int ES = 2, KM = 32, EPL = 8, BK = 64;
    typedef bf16x8 Frag;
};
template <>
struct GT<MOE_FP8_E4M3FN> {
    static constexpr int ES = 1, KM = 128, EPL = 32, BK = 128;
    typedef i32x8 Frag;
};

// B fragment of a 16-column strip starting at column `col` of the LDS tile
// (row stride bstride bytes): lane l holds column col + l%16, K elements
// [(l/16)*EPL, +EPL) of MFMA step ks.  For 16- and 8-bit data the
// transposing reads deliver that directly: within each 16-lane group, the
// tr16 read gives lane j element j%4 of the 8-byte chunks addressed by lanes
// j/4 + 4i, and the tr8 read gives lane j byte j%8 of the chunks addressed by
// lanes j/8 + 2i; each lane addresses the chunk that must land there.
template <int DT>
__device__ __forceinline__ typename GT<DT>::Frag load_b_frag(const char* Bs, int bstride, int ks,
                                                             int col, int lane)
{
    const int g = lane >> 4, s = lane & 15;
    if constexpr (DT == MOE_F32) {
        return *(const float*)(Bs + (ks * 4 + g) * bstride + (col + s) * 4);
    } else if constexpr (DT == MOE_BF16) {
        const char* p0 = Bs + (ks * 32 + 8 * g + (s >> 2)) * bstride + (col + 4 * (s & 3)) * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p0 + 4 * bstride));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, v);
    } else {
        const char* p0 = Bs + (ks * 128 + 32 * g + (s >> 1)) * bstride + col + 8 * (s & 1);
        const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, p0));
        const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, p0 + 8 * bstride));
        const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, p0 + 16 * bstride));
        const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, p0 + 24 * bstride));
        return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    }
}

// Weight-row swizzle of the packed weight layout and of the LDS weight tiles
// of the DMA path: slot s of weight row k (within a 64-row K stage, 16 slots
// of 16 bytes per 256-byte row) holds 8-column chunk s ^ swz_b(k).  A
// transposing fragment read touches 16 rows x 32 bytes; swz_b sends the 8
// rows each half-wave reads to 8 distinct 32-byte bank groups.
__device__ __forceinline__ int swz_b(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }


template <int DT>
__device__ __forceinline__ f32x4 mma(typename GT<DT>::Frag a, typename GT<DT>::Frag b, f32x4 c)
{
    if constexpr (DT == MOE_F32)
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    else if constexpr (DT == MOE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else   // e4m3 x e4m3, unit block scales (E8M0 127 = 2^0)
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------- tile shapes
// A tile is CH = 16*FM rows (shared by the four waves) x BN weight columns
// (WN per wave per half).  GEMM1 (NH = 2) pairs a gate block and an up block
// of BNZ columns each; every wave owns matching gate and up columns, so the
// epilogue pairs them in registers.
constexpr int A_STRIDE = 128 + 16;   // LDS bytes per A row (one K stage = 128 B)

template <int DT, int FM, int WN, int NH, bool ZSCALE = false>
struct Shape {
    static constexpr int ES = GT<DT>::ES, KM = GT<DT>::KM, EPL = GT<DT>::EPL, BK = GT<DT>::BK;
    static constexpr int KS = BK / KM;                    // MFMA steps per stage
    static constexpr int CH = FM * 16;                    // rows per tile
    static constexpr int FN = WN / 16;
    static constexpr int BNZ = 4 * WN;                    // columns per half
    static constexpr int BN = NH * BNZ;                   // weight columns per tile
    static constexpr int B_STRIDE = BN * ES + 16;         // padded LDS row, bytes
    static constexpr int B_CPR = BN * ES / 16;            // 16-B chunks per weight row
    static constexpr int B_PER_T = BK * B_CPR / 256;
    static constexpr int A_CHUNKS = CH * 8;               // 16-B chunks of one A stage
    static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
    static constexpr int A_BYTES = CH * A_STRIDE;
    static constexpr int B_BYTES = BK * B_STRIDE;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + (ZSCALE ? CH * 4 : 0);
    static constexpr int O_STRIDE = BNZ + 4;              // floats per staged output row
    static constexpr int EPI_BYTES = CH * O_STRIDE * 4;
    static constexpr int LDS_BYTES =
        (2 * STAGE_BYTES > EPI_BYTES) ? 2 * STAGE_BYTES : EPI_BYTES;
    static_assert((BK * B_CPR) % 256 == 0 && B_PER_T >= 1, "weight tile must split over 256 threads");
    static_assert(FN >= 1, "wave tile narrower than one MFMA tile");
    static_assert(BK * ES == 128, "one K stage is 128 bytes of an A row");
};

// A fragment of a 16-row strip from LDS: lane l holds row l%16, K elements
// [(l/16)*EPL, +EPL) of MFMA step ks.
template <int DT>
__device__ __forceinline__ typename GT<DT>::Frag load_a_frag(const char* strip, int ks, int lane)
{
    constexpr int ES = GT<DT>::ES, KM = GT<DT>::KM, EPL = GT<DT>::EPL;
    const char* p = strip + (lane & 15) * A_STRIDE + (ks * KM + (lane >> 4) * EPL) * ES;
    if constexpr (DT == MOE_F32) {
        return *(const float*)p;
    } else if constexpr (DT == MOE_BF16) {
        return __builtin_bit_cast(bf16x8, *(const i32x4*)p);
    } else {
        const i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// Global -> register -> LDS staging of one tile's A rows and weight columns.
// Thread tid owns A chunks q = tid + 256 i (row q/8, 16-byte column q%8) and
// weight chunks q (row q/B_CPR, column chunk q%B_CPR).  Rows past the real
// ones (the padding of the last strip) and columns past N stage zeros.
template <typename S>
struct Stager {
    int a_row[S::A_PER_T], a_kc[S::A_PER_T];
    int64_t a_off[S::A_PER_T];          // byte offset of the source row, -1: zeros
    int b_kk[S::B_PER_T], b_lds[S::B_PER_T];
    int64_t b_off[S::B_PER_T];          // byte column in a weight row, -1: zeros
    i32x4 ra[S::A_PER_T], rb[S::B_PER_T];
    float rs;                           // fp8 z: this thread's row scale (tid < CH)

    // weights: row kk of K stage kt at wbase + kt * w_stage + kk * w_ld + column byte
    __device__ __forceinline__ void load(int kt, const char* abase, int64_t a_k_bytes,
                                         const char* wbase, int64_t w_ld, int64_t w_stage, int K)
    {
        const int k0 = kt * S::BK;
#pragma unroll
        for (int i = 0; i < S::A_PER_T; ++i) {
            ra[i] = i32x4{0, 0, 0, 0};
            const int kb = k0 * S::ES + a_kc[i] * 16;
            if (a_off[i] >= 0 && kb < a_k_bytes)
                ra[i] = *(const i32x4*)(abase + a_off[i] + kb);
        }
#pragma unroll
        for (int i = 0; i < S::B_PER_T; ++i) {
            rb[i] = i32x4{0, 0, 0, 0};
            const int k = k0 + b_kk[i];
            if (b_off[i] >= 0 && k < K)
                rb[i] = *(const i32x4*)(wbase + kt * w_stage + (int64_t)b_kk[i] * w_ld + b_off[i]);
        }
    }
    __device__ __forceinline__ void store(char* stage) const
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < S::A_PER_T; ++i)
            if (tid + 256 * i < S::A_CHUNKS)
                *(i32x4*)(stage + a_row[i] * A_STRIDE + a_kc[i] * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < S::B_PER_T; ++i)
            *(i32x4*)(stage + S::A_BYTES + b_lds[i]) = rb[i];
    }
};

// ---------------------------------------------------------------- GEMM1 tile
template <int DT, int FM, int WN>
__device__ __forceinline__ void gemm1_tile(const Gemm1Args& g, char* smem, int e, int r0,
                                           int rows, int ntile)
{
    typedef Shape<DT, FM, WN, 2> S;
    typedef typename GT<DT>::Frag Frag;
    constexpr int ES = S::ES, FN = S::FN, KS = S::KS, BNZ = S::BNZ;
    constexpr int LDS_READS_PER_B = (DT == MOE_FP8_E4M3FN) ? 4 : (DT == MOE_BF16) ? 2 : 1;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = g.H, I = g.I, N = 2 * I;
    const int n0 = ntile * BNZ;
    const int strips = (rows + 15) >> 4;

    Stager<S> st;
#pragma unroll
    for (int i = 0; i < S::A_PER_T; ++i) {
        const int q = tid + 256 * i;
        st.a_row[i] = q / 8;
        st.a_kc[i] = q % 8;
        st.a_off[i] = -1;
        if (st.a_row[i] < rows) {
            const int64_t p = (int64_t)r0 + st.a_row[i];
            int64_t src = -1;
            if (g.a_ident) {
                src = p;
            } else {
                const int sid = g.s.sorted[p];
                if (sid < g.s.sentinel && in_bounds(sid, g.s.sentinel, g.s.status))
                    src = sid / g.a_div;
            }
            if (src >= 0)
                st.a_off[i] = src * (int64_t)H * ES;
        }
    }
#pragma unroll
    for (int i = 0; i < S::B_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int kk = q / S::B_CPR, cc = q % S::B_CPR;
        const int col = cc * 16 / ES;
        const int zc = (col < BNZ) ? col : col - BNZ;
        const int gcol = (col < BNZ) ? n0 + zc : I + n0 + zc;
        st.b_kk[i] = kk;
        st.b_lds[i] = kk * S::B_STRIDE + cc * 16;
        if (g.w_packed)   // one packed block per tile: chunk cc sits in slot cc ^ swz_b(kk)
            st.b_off[i] = (n0 + zc < I) ? (int64_t)((cc ^ swz_b(kk)) * 16) : -1;
        else
            st.b_off[i] = (n0 + zc < I) ? (int64_t)gcol * ES : -1;
    }
    const char* abase = (const char*)g.a;
    const char* wbase = (const char*)g.w13 + (int64_t)e * H * N * ES;
    int64_t w_ld = (int64_t)N * ES, w_stage = S::BK * w_ld;
    if constexpr (DT == MOE_BF16) {
        static_assert(DT != MOE_BF16 || BNZ == 64, "packed w13 blocks pair 64 gate and 64 up columns");
        if (g.w_packed) {   // block (e, kt, ntile): 64 rows of 256 bytes
            const int64_t nblk = (I + 63) / 64, nks = (H + 63) / 64;
            wbase = (const char*)g.w13 + ((int64_t)e * nks * nblk + ntile) * PACK_BLOCK;
            w_ld = 256;
            w_stage = nblk * PACK_BLOCK;
        }
    }

    f32x4 acc[2][FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[0][fm][fn] = acc[1][fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (H + S::BK - 1) / S::BK;
    st.load(0, abase, (int64_t)H * ES, wbase, w_ld, w_stage, H);
    st.store(smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more)
            st.load(kt + 1, abase, (int64_t)H * ES, wbase, w_ld, w_stage, H);
        const char* As = smem + (kt & 1) * S::STAGE_BYTES;
        const char* Bs = As + S::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // issue every LDS read of this MFMA step before the first MFMA, so
            // the reads stream while the MFMAs consume them in order
            Frag bg[FN], bu[FN], a[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int col = wave * WN + fn * 16;
                bg[fn] = load_b_frag<DT>(Bs, S::B_STRIDE, ks, col, lane);
                bu[fn] = load_b_frag<DT>(Bs, S::B_STRIDE, ks, BNZ + col, lane);
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                a[fm] = load_a_frag<DT>(As + fm * 16 * A_STRIDE, ks, lane);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    acc[0][fm][fn] = mma<DT>(a[fm], bg[fn], acc[0][fm][fn]);
                    acc[1][fm][fn] = mma<DT>(a[fm], bu[fn], acc[1][fm][fn]);
                }
            // keep that order: the reads first, then the MFMAs
            __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, FM + 2 * FN * LDS_READS_PER_B, 0);
            __builtin_amdgcn_sched_group_barrier(SCHED_MFMA, 2 * FM * FN, 0);
        }
        if (more)
            st.store(smem + ((kt + 1) & 1) * S::STAGE_BYTES);
        __syncthreads();
    }

    // epilogue: dequant, bias, SiLU(gate)*up -> LDS (float), then vector stores
    float* Zs = (float*)smem;
    const int g4 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int zc = wave * WN + fn * 16 + s16;
        const int n = n0 + zc;
        float bg = 0.0f, bu = 0.0f, sg = 1.0f, su = 1.0f;
        if (n < I) {
            if (g.b13) {
                bg = load_bias(g.b13, g.bias_dt, (int64_t)e * N + n);
                bu = load_bias(g.b13, g.bias_dt, (int64_t)e * N + I + n);
            }
            if constexpr (DT == MOE_FP8_E4M3FN) {
                sg = g.w13_scale[(int64_t)e * N + n];
                su = g.w13_scale[(int64_t)e * N + I + n];
            }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (fm >= strips)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = fm * 16 + g4 * 4 + r;
                float hg = acc[0][fm][fn][r], hu = acc[1][fm][fn][r];
                if constexpr (DT == MOE_FP8_E4M3FN) {
                    float sa = 0.0f;
                    const int64_t p = (int64_t)r0 + row;
                    if (g.a_ident) {
                        sa = g.a_scale[p];
                    } else {
                        const int sid = g.s.sorted[p];
                        if (sid < g.s.sentinel && in_bounds(sid, g.s.sentinel, g.s.status))
                            sa = g.a_scale[sid / g.a_div];
                    }
                    hg = hg * sa * sg;
                    hu = hu * sa * su;
                }
                Zs[row * S::O_STRIDE + zc] = silu_mul(hg + bg, hu + bu);
            }
        }
    }
    __syncthreads();

    const int nrows = strips * 16;
    if constexpr (DT == MOE_FP8_E4M3FN) {
        // requantise per (row, 128 columns): 8 threads per row, 16 columns each
        static_assert(BNZ == 128, "fp8 z groups are 128 columns");
        for (int rb = 0; rb < nrows; rb += 32) {
            const int row = rb + tid / 8, c0 = (tid % 8) * 16;
            if (row >= nrows)
                continue;                                // whole 8-lane groups skip together
            const float rw = (row < rows) ? gemm1_row_w(g, (int64_t)r0 + row) : 1.0f;
            float v[16], amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                v[c] = Zs[row * S::O_STRIDE + c0 + c] * rw;
                amax = fmaxf(amax, fabsf(v[c]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
            const float sc = zq_scale(amax), rc = __builtin_amdgcn_rcpf(sc);
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = cvt_fp8x2(v[4 * q] * rc, v[4 * q + 1] * rc) |
                       (cvt_fp8x2(v[4 * q + 2] * rc, v[4 * q + 3] * rc) << 16);
            const int64_t p = (int64_t)r0 + row;
            *(i32x4*)((uint8_t*)g.z + p * I + n0 + c0) =
                i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            if ((tid % 8) == 0)
                g.z_scale[(int64_t)(n0 / 128) * g.zs_ld + p] = sc;
        }
    } else {
        constexpr int VE = 16 / ES;                 // z elements per 16-B store
        constexpr int CPR = BNZ / VE;
        for (int q = tid; q < nrows * CPR; q += 256) {
            const int row = q / CPR, c0 = (q % CPR) * VE;
            if (n0 + c0 >= I)
                continue;
            const int64_t p = (int64_t)r0 + row;
            const float* src = Zs + row * S::O_STRIDE + c0;
            const float rw = (row < rows) ? gemm1_row_w(g, p) : 1.0f;
            if constexpr (DT == MOE_BF16) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w[k] = f32_to_bf16(src[2 * k] * rw) |
                           ((uint32_t)f32_to_bf16(src[2 * k + 1] * rw) << 16);
                *(i32x4*)((u16*)g.z + p * I + n0 + c0) =
                    i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            } else {
                *(f32x4*)((float*)g.z + p * I + n0 + c0) =
                    f32x4{src[0] * rw, src[1] * rw, src[2] * rw, src[3] * rw};
            }
        }
    }
}

// ---------------------------------------------------------------- GEMM2 tile
template <int DT, int FM, int WN>
__device__ __forceinline__ void gemm2_tile(const Gemm2Args& g, char* smem, int e, int r0,
                                           int rows, int ntile)
{
    constexpr bool FP8 = DT == MOE_FP8_E4M3FN;
    typedef Shape<DT, FM, WN, 1, FP8> S;
    typedef typename GT<DT>::Frag Frag;
    constexpr int ES = S::ES, FN = S::FN, KS = S::KS, BN = S::BN;
    constexpr int LDS_READS_PER_B = FP8 ? 4 : (DT == MOE_BF16) ? 2 : 1;
    constexpr int LDS_READS_PER_A = FP8 ? 3 : 1;   // fp8: 2 b128 + the row scales

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = g.H, I = g.I;
    const int c0 = ntile * BN;
    const int strips = (rows + 15) >> 4;

    // z rows are the padded positions themselves (written by GEMM1)
    Stager<S> st;
#pragma unroll
    for (int i = 0; i < S::A_PER_T; ++i) {
        const int q = tid + 256 * i;
        st.a_row[i] = q / 8;
        st.a_kc[i] = q % 8;
        st.a_off[i] = (st.a_row[i] < strips * 16) ? ((int64_t)r0 + st.a_row[i]) * I * ES : -1;
    }
#pragma unroll
    for (int i = 0; i < S::B_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int kk = q / S::B_CPR, cc = q % S::B_CPR;
        const int col = c0 + cc * 16 / ES;
        st.b_kk[i] = kk;
        st.b_lds[i] = kk * S::B_STRIDE + cc * 16;
        if (g.w_packed)   // one packed block per tile: chunk cc sits in slot cc ^ swz_b(kk)
            st.b_off[i] = (col < H) ? (int64_t)((cc ^ swz_b(kk)) * 16) : -1;
        else
            st.b_off[i] = (col < H) ? (int64_t)col * ES : -1;
    }
    const char* zbase = (const char*)g.z;
    const char* wbase = (const char*)g.w2 + (int64_t)e * I * H * ES;
    int64_t w_ld = (int64_t)H * ES, w_stage = S::BK * w_ld;
    if constexpr (DT == MOE_BF16) {
        static_assert(DT != MOE_BF16 || BN == 128, "packed w2 blocks are 128 columns");
        if (g.w_packed) {   // block (e, kt, ntile)
            const int64_t nblk = (H + 127) / 128, nks = (I + 63) / 64;
            wbase = (const char*)g.w2 + ((int64_t)e * nks * nblk + ntile) * PACK_BLOCK;
            w_ld = 256;
            w_stage = nblk * PACK_BLOCK;
        }
    }
    auto load = [&](int kt) {
        st.load(kt, zbase, (int64_t)I * ES, wbase, w_ld, w_stage, I);
        if constexpr (FP8)
            st.rs = (tid < strips * 16) ? g.z_scale[(int64_t)kt * g.zs_ld + r0 + tid] : 0.0f;
    };
    auto store = [&](int stage) {
        char* base = smem + stage * S::STAGE_BYTES;
        st.store(base);
        if constexpr (FP8) {
            if (tid < S::CH)
                ((float*)(base + S::A_BYTES + S::B_BYTES))[tid] = st.rs;
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (I + S::BK - 1) / S::BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more)
            load(kt + 1);
        const char* As = smem + (kt & 1) * S::STAGE_BYTES;
        const char* Bs = As + S::A_BYTES;
        const float* Ss = (const float*)(Bs + S::B_BYTES);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag bf[FN], af[FM];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[fn] = load_b_frag<DT>(Bs, S::B_STRIDE, ks, wave * WN + fn * 16, lane);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                af[fm] = load_a_frag<DT>(As + fm * 16 * A_STRIDE, ks, lane);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const Frag a = af[fm];
                if constexpr (FP8) {
                    // one MFMA covers exactly one 128-wide scale group of z
                    const f32x4 sz = *(const f32x4*)(Ss + fm * 16 + (lane >> 4) * 4);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const f32x4 t = mma<DT>(a, bf[fn], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[fm][fn][r] += t[r] * sz[r];
                    }
                } else {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = mma<DT>(a, bf[fn], acc[fm][fn]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, FM * LDS_READS_PER_A + FN * LDS_READS_PER_B, 0);
            __builtin_amdgcn_sched_group_barrier(SCHED_MFMA, FM * FN, 0);
        }
        if (more)
            store((kt + 1) & 1);
        __syncthreads();
    }

    // epilogue: per-channel dequant, bias -> LDS, then row stores
    float* Os = (float*)smem;
    const int g4 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = wave * WN + fn * 16 + s16;
        const int c = c0 + cl;
        float bias = 0.0f, sw = 1.0f;
        if (c < H) {
            if (g.b2)
                bias = load_bias(g.b2, g.bias_dt, (int64_t)e * H + c);
            if constexpr (FP8)
                sw = g.w2_scale[(int64_t)e * H + c];
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            if (fm >= strips)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = fm * 16 + g4 * 4 + r;
                Os[row * S::O_STRIDE + cl] = acc[fm][fn][r] * sw + bias;
            }
        }
    }
    __syncthreads();

    constexpr int CPR = BN / 4;   // 4 floats per chunk
    for (int q = tid; q < rows * CPR; q += 256) {
        const int row = q / CPR, cl = (q % CPR) * 4;
        const int c = c0 + cl;
        if (c >= H)
            continue;
        const int64_t p = (int64_t)r0 + row;
        const int sid = g.s.sorted[p];
        if (sid >= g.s.sentinel || !in_bounds(sid, g.s.sentinel, g.s.status))
            continue;
        const float* src = Os + row * S::O_STRIDE + cl;
        const int64_t dst_row = (g.out_mode == 2) ? p : (int64_t)sid;
        if (g.out_mode == 1 && g.out_dt == MOE_BF16) {
            const uint32_t lo = f32_to_bf16(src[0]) | ((uint32_t)f32_to_bf16(src[1]) << 16);
            const uint32_t hi = f32_to_bf16(src[2]) | ((uint32_t)f32_to_bf16(src[3]) << 16);
            *(i32x2*)((u16*)g.out + dst_row * H + c) = i32x2{(int)lo, (int)hi};
        } else {
            *(f32x4*)((float*)g.out + dst_row * H + c) = f32x4{src[0], src[1], src[2], src[3]};
        }
    }
}

// ---------------------------------------------------------------- kernels
template <int DT, int FM, int WN>
__global__ void __launch_bounds__(256) k_gemm1(Gemm1Args g)
{
    typedef Shape<DT, FM, WN, 2> S;
    __shared__ __attribute__((aligned(16))) char smem[S::LDS_BYTES];
    for_each_tile<S::CH>(g.s, [&](int e, int r0, int rows, int ntile) {
        gemm1_tile<DT, FM, WN>(g, smem, e, r0, rows, ntile);
        __syncthreads();   // the next tile's prologue reuses the LDS
    });
}

template <int DT, int FM, int WN>
__global__ void __launch_bounds__(256) k_gemm2(Gemm2Args g)
{
    typedef Shape<DT, FM, WN, 1, DT == MOE_FP8_E4M3FN> S;
    __shared__ __attribute__((aligned(16))) char smem[S::LDS_BYTES];
    for_each_tile<S::CH>(g.s, [&](int e, int r0, int rows, int ntile) {
        gemm2_tile<DT, FM, WN>(g, smem, e, r0, rows, ntile);
        __syncthreads();
    });
}

// ================================================================ LDS-DMA bf16 tiles
// The large-tile bf16 path moves A and weight tiles with LDS DMA
// (global_load_lds_dwordx4): each lane names one 16-byte global chunk and the
// 64 chunks of a wave land at M0 + 16 * lane, so the loads need no staging
// registers and a ring of NS stages keeps up to NS - 1 K stages in flight.
// The loads come from inline asm, outside the compiler's wait-count
// bookkeeping: the ring waits on them itself with s_waitcnt vmcnt(N).  Vector
// memory loads complete in issue order, so "at most N outstanding" means
// every load older than the last N has landed in LDS; the compiler's own
// waits on its loads only ever see a lower count and so stay correct.
//
// Tile: CH = 32 * FMW rows x BN = 64 * WC weight columns, one K stage = 64
// rows of K.  The 2 * WC waves form a 2 x WC grid: wave (rg, cg) owns FMW
// 16-row strips (rows rg * 16 FMW ..) and four 16-column fragments (64
// weight columns).  Each A fragment is read from LDS by WC waves and each
// weight fragment by two.  WC = 2: 128 columns, 4 waves, two workgroups per
// CU; WC = 4: 256 columns, 8 waves, one workgroup per CU with a deeper ring
// and half the activation traffic per weight byte.
// Layout L = 1 (decode-sized loads, a row or two per expert): one row group
// of WC waves, each with FMW strips (CH = 16 * FMW rows) and two fragments
// (BN = 32 * WC columns), so every wave shares the single live strip's work
// instead of the second row group's waves idling.
//
// LDS layout of a stage (no padding: a DMA fills 1024 contiguous bytes):
//   A  [CH rows][128 B]: 16-byte slot s of row r holds K chunk s ^ ((r>>1)&7),
//      so the 16 rows of a fragment read hit 16 distinct bank groups.
//   B  [64 rows][256 B]: slot s of row k holds column chunk s ^ fB(k), with
//      fB(k) = 2 * ((k & 3) | ((k >> 1) & 4)); a transposing read touches 16
//      rows x 32 bytes and fB sends the 8 rows of each half-wave to 8
//      distinct 32-byte bank groups.
// Out-of-range chunks (K tail, columns past N) and rows past the tile's real
// rows are DMA'd from a zero page; strips that hold only padding skip their
// fragment reads and MFMAs.
//
// WNA16 (Q = 8 or 4 code bits; the walkthrough's "WNA16" section): the
// weight block of a stage is 128 columns x 64 K of codes in fragment order
// (8 or 4 KiB, see the packed layout in moe.h), followed by the stage's
// group scales (1 KiB slot) and zero points (1 KiB slot), DMA'd from the
// plain [E, ceil(K / G), N] grids.  With groups of 64 or 128 K rows the
// stage lies inside one group (128 floats, 128 bytes); with groups of 32
// (G2) it spans two, one per MFMA step, and the slots hold both (the second
// at +512 / +128 bytes).  The 160-row tile dequantises its B fragments to
// bf16 right after their LDS read (w = (q - z) * s as one FMA q * s + (-z s)
// on the float code, then a packed RNE conversion); the small-row tiles feed
// the raw codes to the MFMAs and apply s and z per group
// (DmaFrag::raw_codes).
template <int FMW_, int WC_, int NS_, int Q_ = 0, int G2_ = 0, int L_ = 0>
struct DS {
    static constexpr int FMW = FMW_, WC = WC_, NS = NS_, Q = Q_;
    static constexpr int G2 = G2_;                       // WNA16: two scale groups a stage
    static constexpr int L = L_;                         // wave layout (see above)
    static constexpr int RG = L ? 1 : 2;                 // row groups of waves
    static constexpr int NW = RG * WC, NT = 64 * NW;     // waves, threads
    static constexpr int FN = L ? 2 : 4;                 // 16-column fragments per wave
    static constexpr int CH = 16 * FMW * RG;             // rows per tile
    static constexpr int BN = 16 * FN * WC;              // weight columns per tile
    static constexpr int NB = BN / 128;                  // 128-column weight blocks per tile
    static constexpr int RB = 256;                       // bytes per weight row of a block
    // bytes of one 128-column weight block per K stage: bf16 rows, or codes
    static constexpr int QB = Q ? 128 * 64 * Q / 8 : PACK_BLOCK;
    static constexpr int IPB = QB / 1024;                // 1 KiB DMAs per weight block
    static constexpr int A_BYTES = CH * 128, B_BYTES = NB * QB;
    static constexpr int SZ_OFF = A_BYTES + B_BYTES;     // WNA16: scales, then zero points
    static constexpr int SZ_BYTES = Q ? 2048 : 0;
    static constexpr int STAGE = A_BYTES + B_BYTES + SZ_BYTES;
    static constexpr int A_INS = A_BYTES / 1024, B_INS = B_BYTES / 1024;   // 1 KiB DMAs a stage
    static constexpr int A_PW = (A_INS + NW - 1) / NW;   // A DMA slots per wave
    static constexpr int B_PW = B_INS / NW;
    static constexpr int D = A_PW + B_PW;                // DMAs per wave per stage
    // when NW does not divide A_INS, the spare A slots DMA the zero page into
    // a scratch KiB past the ring, so every wave issues D DMAs a stage
    static constexpr bool A_SPARE = A_PW * NW > A_INS;
    static constexpr int RING = NS * STAGE + (A_SPARE ? 1024 : 0);
    static_assert(WC == 2 || WC == 4, "2 x 2 or 2 x 4 waves");
    static_assert(B_INS % NW == 0, "weight DMAs split evenly");
    static_assert(NS >= 2 && NS <= 4, "ring depth");
    static_assert((NS - 2) * D < 64, "vmcnt range");
    static_assert(Q == 0 || Q == 8 || Q == 4, "code width");
    static_assert(Q == 0 || NB == 1, "a WNA16 tile holds one weight block");
    static_assert(G2 == 0 || Q != 0, "scale groups are a WNA16 notion");
};

// DMA sources of one tile.  Wave w issues the A DMAs i = w + NW j (tile rows
// 8i .. 8i+7; lane l: row 8i + l/8, 16-byte K chunk (l%8) ^ ((row>>1)&7)) and
// the B DMAs i = w + NW j (weight block i / IPB, its KiB i % IPB; plain bf16:
// K rows 4(i%16) + l/16, slot l%16).  WNA16: wave 0 also DMAs the stage's
// group scales, wave 1 its zero points (one group spans two stages); those
// waves wait on the shared count, which only makes them wait a little longer.
// A lane keeps a pointer per A DMA; weight addresses are recomputed per issue
// from uniform bases.  PACKED: each weight block of a K stage is one
// contiguous 16 KiB block of the packed layout; plain: the weights are read
// in place (W13: [H, 2I] gate | up; else [I, H]).
template <typename S, bool PACKED, bool W13>
struct DmaTile {
    const char* wb[S::NB];      // PACKED: block (stage 0) per tile block, null past N;
                                //   plain: wb[0] = the expert's weight matrix
    int64_t w_ld;               // plain: bytes per weight row
    int64_t w_stage;            // PACKED: bytes from one K stage's blocks to the next
    int n0;                     // plain: first column of the tile (z column for W13)
    int ncols;                  // plain: columns (I for W13, H otherwise)
    int K;                      // contraction length
    const char* ap[S::A_PW];    // this lane's A chunk (K stage 0), null: padding row
    const char* qs;             // WNA16: this lane's 16 scale bytes of group 0, or null
    const char* qz;             //   and its 16 zero-point bytes, or null
    int64_t qs_g, qz_g;         //   bytes from one K group to the next
    int gsh;                    //   log2(group / 32): the stage's first group is (2 kt) >> gsh

    bool nt;                    // the weights are read by this tile alone: non-temporal DMAs

    // spare: LDS address of the scratch KiB for spare A slots
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

    // DMAs [J0, J1) of the wave's D for stage kt: the A DMAs first, then the
    // weight DMAs; the range that ends at D also carries the WNA16 scale DMAs
    template <int J0, int J1>
    __device__ __forceinline__ void issue_part(int kt, uint32_t lds, uint32_t spare, int wave,
                                               bool live) const
    {
        issue_part_p<false, J0, J1>(kt, lds, spare, wave, live);
    }

    template <bool NT, int J0, int J1>
    __device__ __forceinline__ void issue_part_p(int kt, uint32_t lds, uint32_t spare, int wave,
                                                 bool live) const
    {
        static_assert(0 <= J0 && J0 <= J1 && J1 <= S::D, "DMA range");
        const int lane = threadIdx.x & 63;
        const char* zero = (const char*)g_zero16;
#pragma unroll
        for (int j = J0; j < J1 && j < S::A_PW; ++j) {
            const int i = wave + S::NW * j;
            const int row = 8 * i + (lane >> 3);
            const int c = (lane & 7) ^ ((row >> 1) & 7);
            const bool ok = live && ap[j] && kt * 64 + c * 8 < K;
            const char* p = ok ? ap[j] + kt * 128 : zero;
            dma16(p, (!S::A_SPARE || i < S::A_INS) ? lds + i * 1024 : spare);
        }
#pragma unroll
        for (int jb = (J0 > S::A_PW ? J0 : S::A_PW); jb < J1; ++jb) {
            const int j = jb - S::A_PW;
            const int i = wave + S::NW * j;
            const int bb = i / S::IPB, k = 4 * (i & 15) + (lane >> 4);
            const char* p = zero;
            if constexpr (PACKED) {
                // a select, not wb[bb]: bb depends on the wave index, and a
                // runtime index would put wb in scratch memory
                const char* w = (S::NB == 1 || bb == 0) ? wb[0] : wb[S::NB - 1];
                if (live && w)
                    p = w + kt * w_stage + (i % S::IPB) * 1024 + lane * 16;
            } else {
                static_assert(S::Q == 0, "WNA16 weights are packed");
                const int c = (lane & 15) ^ swz_b(k);
                int col, valid;
                if constexpr (W13) {
                    const int zc = n0 + 64 * bb + 8 * (c & 7);
                    valid = zc < ncols;
                    col = (c < 8) ? zc : ncols + zc;
                } else {
                    col = n0 + 128 * bb + 8 * c;
                    valid = col < ncols;
                }
                if (live && valid && kt * 64 + k < K)
                    p = wb[0] + (int64_t)(kt * 64 + k) * w_ld + (int64_t)col * 2;
            }
            if constexpr (NT)
                dma16_nt(p, lds + S::A_BYTES + i * 1024);
            else
                dma16(p, lds + S::A_BYTES + i * 1024);
        }
        if constexpr (S::Q != 0 && J1 == S::D) {
            // the group of the stage's first 32 K rows; with G2 the lanes of
            // the second half of each DMA (scales: 32-63, zero points: 8-15)
            // point one group further, which exists while its rows start inside K
            const int grp = (2 * kt) >> gsh;
            const bool second_ok = !S::G2 || kt * 64 + 32 < K;
            if (wave == 0)
                dma16((live && qs && (lane < 32 || second_ok)) ? qs + grp * qs_g : zero,
                      lds + S::SZ_OFF);
            else if (wave == 1)
                dma16((live && qz && (lane < 8 || second_ok)) ? qz + grp * qz_g : zero,
                      lds + S::SZ_OFF + 1024);
        }
    }
};

// Tile row and K chunk of this lane's j-th A DMA (row >= CH: a spare slot).
template <typename S>
__device__ __forceinline__ void dma_a_slot(int j, int wave, int lane, int& row, int& chunk)
{
    const int i = wave + S::NW * j;
    row = 8 * i + (lane >> 3);
    chunk = (lane & 7) ^ ((row >> 1) & 7);
}

// Fragment reads and MFMAs of one stage for wave (rg, cg).  Fragment fn's
// columns start at 8-column chunk bchunk[fn] of weight block bblk[fn].
template <typename S>
struct DmaFrag {
    int a_off[2];               // A fragment byte offset within a strip, per MFMA step
    int b_off[S::FN];           // B fragment byte offset (MFMA step 0, low half); WNA16:
                                //   this lane's codes of MFMA step 0
    int s_off[S::FN];           // WNA16: this lane's column scale (+ 1024: zero point)
    int hz;                     // WNA16: zero points given (else 2^(Q-1))

    __device__ __forceinline__ void init(int lane, const int (&bblk)[S::FN], const int (&bchunk)[S::FN])
    {
        const int s = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            a_off[ks] = s * 128 + (((ks * 4 + g) ^ (s >> 1)) * 16);
        // this lane's K rows are 32 ks + 8 g + s/4 (+4): the swizzle depends on g and s only
        const int x = ((s & 3) >> 1) ^ swz_b(8 * g + (s >> 2));
#pragma unroll
        for (int fn = 0; fn < S::FN; ++fn)
            b_off[fn] = bblk[fn] * PACK_BLOCK + (8 * g + (s >> 2)) * S::RB + ((bchunk[fn] ^ x) * 16) +
                        8 * (s & 1);
    }

    // WNA16: fragment fn is block column group bchunk[fn] / 2 (16 columns);
    // the lane's 8 codes of MFMA step ks sit at ((2 f + ks) * 64 + lane) * Q bytes
    __device__ __forceinline__ void init_q(int lane, const int (&bchunk)[S::FN], bool zeros)
    {
        const int s = lane & 15, g = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            a_off[ks] = s * 128 + (((ks * 4 + g) ^ (s >> 1)) * 16);
#pragma unroll
        for (int fn = 0; fn < S::FN; ++fn) {
            const int f = bchunk[fn] >> 1;
            b_off[fn] = S::A_BYTES + (2 * f * 64 + lane) * S::Q;
            s_off[fn] = S::SZ_OFF + (16 * f + s) * 4;
        }
        hz = zeros ? 1 : 0;
    }

    // Raw form of a WNA16 fragment for the small-row tiles: the 8 codes as
    // exact bf16 integers, 4-bit ones offset by 128 (bf16 bits 0x4300 | q are
    // 128 + q: after one mask of the low and one of the high nibbles, each
    // pair is one byte permute of the codes with a register of 0x43 bytes),
    // 8-bit ones converted through float.  A 64-row K stage lies inside one
    // 128-row scale group, so the stage's products are exactly
    // s (A Q - (z + offset) A 1): P = A Q and the row sums R = A 1 run on the
    // MFMAs and the scale / zero point are applied per stage to the
    // accumulators, instead of to every weight.
    static constexpr float RAW_OFF = (S::Q == 4) ? 128.0f : 0.0f;
    __device__ __forceinline__ static bf16x8 raw_codes(const char* p)
    {
        if constexpr (S::Q == 4) {
            // packed order: code i in nibble i / 2 + 4 (i & 1), so lo's bytes
            // are codes (0, 4, 1, 5) and hi's (2, 6, 3, 7)
            const uint32_t c = *(const uint32_t*)p;
            const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
            const uint32_t k43 = 0x43434343u;
            // word q = bytes (code 2q, 0x43, code 2q + 1, 0x43); selector bytes
            // 0-3 pick the code register's bytes, 4 a 0x43 byte
            i32x4 v;
            v[0] = (int)__builtin_amdgcn_perm(k43, lo, 0x04020400u);
            v[1] = (int)__builtin_amdgcn_perm(k43, hi, 0x04020400u);
            v[2] = (int)__builtin_amdgcn_perm(k43, lo, 0x04030401u);
            v[3] = (int)__builtin_amdgcn_perm(k43, hi, 0x04030401u);
            return __builtin_bit_cast(bf16x8, v);
        } else {
            const i32x2 c = *(const i32x2*)p;
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = (__bf16)(float)(((uint32_t)c[i >> 2] >> (8 * (i & 3))) & 255u);
            return v;
        }
    }

    // the 8 bf16 weights of a WNA16 fragment: w = q * sc + bz, bz = -z * sc
    __device__ __forceinline__ static bf16x8 dequant(const char* p, float sc, float bz)
    {
        float w[8];
        if constexpr (S::Q == 8) {
            const i32x2 c = *(const i32x2*)p;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[i] = fmaf((float)(((uint32_t)c[i >> 2] >> (8 * (i & 3))) & 255u), sc, bz);
        } else {
            // code i is nibble i / 2 + 4 (i & 1): lo's bytes hold codes
            // (0, 4, 1, 5), hi's (2, 6, 3, 7)
            const uint32_t c = *(const uint32_t*)p;
            const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
            constexpr int LO_CODE[4] = {0, 4, 1, 5}, HI_CODE[4] = {2, 6, 3, 7};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                w[LO_CODE[b]] = fmaf((float)((lo >> (8 * b)) & 255u), sc, bz);
                w[HI_CODE[b]] = fmaf((float)((hi >> (8 * b)) & 255u), sc, bz);
            }
        }
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = (__bf16)w[i];
        return v;
    }

    // the MFMAs of the wave's first NM strips (the others hold only padding),
    // with the D DMAs of the ring's refill issued through issue(lo, hi)
    template <int NM, typename Issue>
    __device__ __forceinline__ void stage(const char* st, int rg, f32x4 (&acc)[S::FMW][S::FN],
                                          Issue&& issue) const
    {
        const char* As = st + rg * S::FMW * 2048;
        const char* Bs = st + S::A_BYTES;
        // where the refill goes out: a two-stage ring leaves a refill just one
        // stage to land, and the decode layout is bound by that latency, so
        // there it goes first; the deeper bf16 prefill rings spread it over the
        // first half's MFMAs, so that the DMA issue overlaps MFMA work instead
        // of delaying the stage's first fragment reads
        constexpr bool SPREAD = S::Q == 0 && S::NS >= 3 && S::L == 0;
        if constexpr (!SPREAD)
            issue(IC<0>{}, IC<S::D>{});
        if constexpr (S::Q != 0 && S::FMW <= 2) {
            constexpr float ZDEF = (S::Q == 8) ? 128.0f : 8.0f;
            constexpr int NG = S::G2 ? 2 : 1;            // scale groups in the stage
            float sc[NG][S::FN], szn[NG][S::FN];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn) {
                    sc[gi][fn] = *(const float*)(st + s_off[fn] + gi * 512);
                    const float z = hz ? (float)*(const uint8_t*)(st + S::SZ_OFF + 1024 + gi * 128 +
                                                                  (s_off[fn] - S::SZ_OFF) / 4)
                                       : ZDEF;
                    szn[gi][fn] = -(z + RAW_OFF) * sc[gi][fn];
                }
            const i32x4 ones_bits = {0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80};
            const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_bits);
            f32x4 pq[NM][S::FN], rs[NM];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 0 || S::G2) {
#pragma unroll
                    for (int fm = 0; fm < NM; ++fm) {
                        rs[fm] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int fn = 0; fn < S::FN; ++fn)
                            pq[fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    }
                }
                bf16x8 a[NM], b[S::FN];
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn)
                    b[fn] = raw_codes(st + b_off[fn] + ks * 64 * S::Q);
#pragma unroll
                for (int fm = 0; fm < NM; ++fm)
                    a[fm] = __builtin_bit_cast(bf16x8, *(const i32x4*)(As + fm * 2048 + a_off[ks]));
#pragma unroll
                for (int fm = 0; fm < NM; ++fm) {
                    rs[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], ones, rs[fm], 0, 0, 0);
#pragma unroll
                    for (int fn = 0; fn < S::FN; ++fn)
                        pq[fm][fn] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[fn], pq[fm][fn], 0, 0, 0);
                }
                if (ks == 1 || S::G2) {                  // a scale group is complete
                    const int gi = S::G2 ? ks : 0;
#pragma unroll
                    for (int fm = 0; fm < NM; ++fm)
#pragma unroll
                        for (int fn = 0; fn < S::FN; ++fn)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[fm][fn][r] += sc[gi][fn] * pq[fm][fn][r] + szn[gi][fn] * rs[fm][r];
                }
            }
            return;
        } else if constexpr (S::Q != 0) {
            constexpr float ZDEF = (S::Q == 8) ? 128.0f : 8.0f;
            constexpr int NG = S::G2 ? 2 : 1;            // scale groups in the stage
            float sc[NG][S::FN], bz[NG][S::FN];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn) {
                    sc[gi][fn] = *(const float*)(st + s_off[fn] + gi * 512);
                    const float z = hz ? (float)*(const uint8_t*)(st + S::SZ_OFF + 1024 + gi * 128 +
                                                                  (s_off[fn] - S::SZ_OFF) / 4)
                                       : ZDEF;
                    bz[gi][fn] = -z * sc[gi][fn];
                }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int gi = S::G2 ? ks : 0;
                bf16x8 a[NM], b[S::FN];
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn)
                    b[fn] = dequant(st + b_off[fn] + ks * 64 * S::Q, sc[gi][fn], bz[gi][fn]);
#pragma unroll
                for (int fm = 0; fm < NM; ++fm)
                    a[fm] = __builtin_bit_cast(bf16x8, *(const i32x4*)(As + fm * 2048 + a_off[ks]));
#pragma unroll
                for (int fm = 0; fm < NM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < S::FN; ++fn)
                        acc[fm][fn] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[NM], b[S::FN];
#pragma unroll
            for (int fn = 0; fn < S::FN; ++fn) {
                const char* p = Bs + b_off[fn] + ks * 32 * S::RB;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 4 * S::RB));
                const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                b[fn] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int fm = 0; fm < NM; ++fm)
                a[fm] = __builtin_bit_cast(bf16x8, *(const i32x4*)(As + fm * 2048 + a_off[ks]));
            if constexpr (SPREAD) {
                if (ks == 0) {
                    // one share of the DMAs after each strip's MFMAs
                    static_for<0, NM>([&](auto fmc) {
                        constexpr int fm = decltype(fmc)::value;
#pragma unroll
                        for (int fn = 0; fn < S::FN; ++fn)
                            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
                        constexpr int lo = fm * S::D / NM, hi = (fm + 1) * S::D / NM;
                        if constexpr (hi > lo)
                            issue(IC<lo>{}, IC<hi>{});
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    continue;
                }
            }
#pragma unroll
            for (int fm = 0; fm < NM; ++fm)
#pragma unroll
                for (int fn = 0; fn < S::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, NM + 2 * S::FN, 0);
            __builtin_amdgcn_sched_group_barrier(SCHED_MFMA, NM * S::FN, 0);
        }
    }
};

// A tile's DMA source with its weight DMAs non-temporal.
template <typename Src>
struct NtSrc {
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
__device__ __forceinline__ void dma_prologue_p(const Src& src, char* ring, int kb, int ke, int wave)
{
    if (__builtin_amdgcn_readfirstlane(src.nt))
        dma_prologue<S>(NtSrc<Src>{src}, ring, kb, ke, wave);
    else
        dma_prologue<S>(src, ring, kb, ke, wave);
}

// The mainloop with the MFMAs of the wave's first `live` strips (wave
// uniform): one instantiation per count and weight cache policy, so the loop
// body stays branch free; every wave still issues its DMAs and meets every
// barrier.
template <typename S, int NM = S::FMW, typename Src>
__device__ __forceinline__ void dma_run(const Src& src, char* ring, int kb, int ke, int wave,
                                        int rg, const DmaFrag<S>& fr,
                                        f32x4 (&acc)[S::FMW][S::FN], int live)
{
    auto loop = [&](const auto& ss) {
        if constexpr (NM == 0)
            dma_mainloop_split<S>(ss, ring, kb, ke, wave,
                                  [](const char*, auto&& issue) { issue(IC<0>{}, IC<S::D>{}); });
        else
            dma_mainloop_split<S>(ss, ring, kb, ke, wave, [&](const char* st, auto&& issue) {
                fr.template stage<NM>(st, rg, acc, issue);
            });
    };
    if constexpr (NM > 0) {
        if (live < NM) {
            dma_run<S, NM - 1>(src, ring, kb, ke, wave, rg, fr, acc, live);
            return;
        }
    }
    if (__builtin_amdgcn_readfirstlane(src.nt))
        loop(NtSrc<Src>{src});
    else
        loop(src);
}

// Per-lane source rows of one GEMM1 tile's A DMAs (-1: padding row); loaded
// one tile ahead.
template <typename S>
__device__ __forceinline__ void gemm1_rows(const Gemm1Args& g, const TileRef& t, int wave, int lane,
                                           int (&src)[S::A_PW])
{
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        int row, c;
        dma_a_slot<S>(j, wave, lane, row, c);
        src[j] = (row < t.rows) ? (int)gemm1_src_row(g, t.r0, row) : -1;
    }
}

// DMA sources of a GEMM1 tile: BN/2 gate columns n0.. and the matching BN/2
// up columns I + n0..; weight block bb holds z columns n0 + 64 bb .. +63
// (chunks 0-7 gate, 8-15 up), packed it is block (e, kt, n0 / 64 + bb).
template <typename S, bool PACKED>
__device__ __forceinline__ void gemm1_src(const Gemm1Args& g, const TileRef& t,
                                          const int (&srow)[S::A_PW], DmaTile<S, PACKED, true>& d)
{
    const int H = g.H, I = g.I, N = 2 * I;
    const int n0 = t.ntile * (S::BN / 2);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    d.n0 = n0;
    d.ncols = I;
    d.K = H;
    d.w_ld = (int64_t)N * 2;
    d.qs = d.qz = nullptr;
    d.qs_g = d.qz_g = 0;
    d.nt = __builtin_amdgcn_readfirstlane(t.nch) == 1;
    if constexpr (PACKED) {
        const int64_t nblk = (I + 63) / 64, nks = (H + 63) / 64;
        d.w_stage = nblk * S::QB;
#pragma unroll
        for (int bb = 0; bb < S::NB; ++bb) {
            const int64_t jb = n0 / 64 + bb;
            d.wb[bb] = (jb < nblk) ? (const char*)g.w13 + (t.e * nks * nblk + jb) * S::QB
                                   : nullptr;
        }
        if constexpr (S::Q != 0) {
            // the block's group scales / zero points: gate z columns n0 .. n0 + 63
            // (block columns 0-63), then the up ones (64-127); lanes 0-31 take 4
            // scales each, lanes 0-7 16 zero points each; with G2 lanes 32-63 and
            // 8-15 take the same columns of the next group
            const int G = 32 << g.wq_gsh;
            const int64_t ngk = (H + G - 1) / G, base = (int64_t)t.e * ngk * N;
            d.gsh = g.wq_gsh;
            d.qs_g = (int64_t)N * 4;
            d.qz_g = N;
            if (lane < 32 || S::G2) {
                const int l = lane & 31, c = n0 + 4 * (l & 15);
                if (c < I)
                    d.qs = (const char*)(g.w13_scale + base + (l < 16 ? c : I + c) +
                                         (lane >= 32 ? N : 0));
            }
            if ((lane < 8 || (S::G2 && lane < 16)) && g.w13_zero) {
                const int l = lane & 7, c = n0 + 16 * (l & 3);
                if (c < I)
                    d.qz = (const char*)(g.w13_zero + base + (l < 4 ? c : I + c) +
                                         (lane >= 8 ? N : 0));
            }
        }
    } else {
        d.wb[0] = (const char*)g.w13 + (int64_t)t.e * H * N * 2;
    }
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        const int row = 8 * (wave + S::NW * j) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        d.ap[j] = (srow[j] >= 0) ? (const char*)g.a + (int64_t)srow[j] * H * 2 + c * 16 : nullptr;
    }
}

// DMA sources of a GEMM2 tile: BN output columns c0..; A rows are the padded
// positions (z written by GEMM1); weight block bb holds columns c0 + 128 bb ..,
// packed it is block (e, kt, c0 / 128 + bb).
template <typename S, bool PACKED>
__device__ __forceinline__ void gemm2_src(const Gemm2Args& g, const TileRef& t, int wave,
                                          DmaTile<S, PACKED, false>& d)
{
    const int H = g.H, I = g.I;
    const int c0 = t.ntile * S::BN;
    const int lane = threadIdx.x & 63;
    d.n0 = c0;
    d.ncols = H;
    d.K = I;
    d.w_ld = (int64_t)H * 2;
    d.qs = d.qz = nullptr;
    d.qs_g = d.qz_g = 0;
    d.nt = __builtin_amdgcn_readfirstlane(t.nch) == 1;
    if constexpr (PACKED) {
        const int64_t nblk = (H + 127) / 128, nks = (I + 63) / 64;
        d.w_stage = nblk * S::QB;
#pragma unroll
        for (int bb = 0; bb < S::NB; ++bb) {
            const int64_t jb = c0 / 128 + bb;
            d.wb[bb] = (jb < nblk) ? (const char*)g.w2 + (t.e * nks * nblk + jb) * S::QB
                                   : nullptr;
        }
        if constexpr (S::Q != 0) {
            // the block's group scales / zero points: columns c0 .. c0 + 127
            // (with G2 the upper lanes take the next group's)
            const int G = 32 << g.wq_gsh;
            const int64_t ngi = (I + G - 1) / G, base = (int64_t)t.e * ngi * H;
            d.gsh = g.wq_gsh;
            d.qs_g = (int64_t)H * 4;
            d.qz_g = H;
            const int ls = lane & 31, lz = lane & 7;
            if ((lane < 32 || S::G2) && c0 + 4 * ls < H)
                d.qs = (const char*)(g.w2_scale + base + c0 + 4 * ls + (lane >= 32 ? H : 0));
            if ((lane < 8 || (S::G2 && lane < 16)) && g.w2_zero && c0 + 16 * lz < H)
                d.qz = (const char*)(g.w2_zero + base + c0 + 16 * lz + (lane >= 8 ? H : 0));
        }
    } else {
        d.wb[0] = (const char*)g.w2 + (int64_t)t.e * I * H * 2;
    }
#pragma unroll
    for (int j = 0; j < S::A_PW; ++j) {
        const int row = 8 * (wave + S::NW * j) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        d.ap[j] = (row < t.rows) ? (const char*)g.z + ((int64_t)t.r0 + row) * I * 2 + c * 16
                                 : nullptr;
    }
}

template <typename S>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[S::FMW][S::FN])
{
#pragma unroll
    for (int fm = 0; fm < S::FMW; ++fm)
#pragma unroll
        for (int fn = 0; fn < S::FN; ++fn)
            acc[fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// The DMA kernels are compiled for two waves per SIMD (at most 256 registers
// a lane): two 4-wave workgroups or one 8-wave workgroup per CU, or one
// 4-wave workgroup where the ring's LDS allows no more; with a larger budget
// the compiler moves the accumulators into AGPRs and copies them back and
// forth around the loops.
//
// Persistent GEMM1 over this workgroup's tiles.  The next tile's A source
// rows are loaded while the current tile streams; once its ring has drained
// the next tile's first stages are issued and the current tile's epilogue
// (bias, SiLU(gate) * up, bf16 z stores straight from the accumulators) runs
// while they are in flight.
template <int FMW, int WC, int NS, bool PACKED, int Q = 0, int G2 = 0, int L = 0>
__global__ void __launch_bounds__((DS<FMW, WC, NS, Q, G2, L>::NT), 2)
    k_gemm1_dma(Gemm1Args g)
{
    typedef DS<FMW, WC, NS, Q, G2, L> S;
    constexpr int FN = S::FN;
    constexpr int FH = FN / 2;
    __shared__ __attribute__((aligned(16))) char ring[S::RING];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / S::WC, cg = wave % S::WC;
    const int I = g.I, N = 2 * I;

    TileIter<S::CH> it(g.s);
    TileRef cur;
    if (!it.next(g.s, cur))
        return;
    int srow[S::A_PW];
    gemm1_rows<S>(g, cur, wave, lane, srow);
    DmaTile<S, PACKED, true> src;
    const int nk1 = (g.H + 63) / 64;
    gemm1_src<S, PACKED>(g, cur, srow, src);
    dma_prologue_p<S>(src, ring, 0, nk1, wave);

    // wave (rg, cg): gate fragments fn < FN/2 at z columns (cg FN/2 + fn) 16,
    // up fragments fn >= FN/2 at the same z columns of the up half
    int bblk[FN], bchunk[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int zc = (cg * FH + (fn < FH ? fn : fn - FH)) * 16;
        bblk[fn] = zc / 64;
        bchunk[fn] = (fn < FH ? 0 : 8) + (zc % 64) / 8;
    }
    DmaFrag<S> fr;
    if constexpr (Q != 0)
        fr.init_q(lane, bchunk, g.w13_zero != nullptr);
    else
        fr.init(lane, bblk, bchunk);
    const int g4 = lane >> 4, s16 = lane & 15;

    for (;;) {
        TileRef nxt;
        const bool more = it.next(g.s, nxt);
        if (more)
            gemm1_rows<S>(g, nxt, wave, lane, srow);
        const int n0 = cur.ntile * (S::BN / 2);
        float bg[FH], bu[FH];
#pragma unroll
        for (int fn = 0; fn < FH; ++fn) {
            const int n = n0 + (cg * FH + fn) * 16 + s16;
            bg[fn] = bu[fn] = 0.0f;
            if (g.b13 && n < I) {
                bg[fn] = load_bias(g.b13, g.bias_dt, (int64_t)cur.e * N + n);
                bu[fn] = load_bias(g.b13, g.bias_dt, (int64_t)cur.e * N + I + n);
            }
        }
        f32x4 acc[FMW][FN];
        zero_acc<S>(acc);
        const int strips = (cur.rows + 15) >> 4;
        dma_run<S>(src, ring, 0, nk1, wave, rg, fr, acc, min(max(strips - rg * FMW, 0), FMW));
#pragma unroll
        for (int fn = 0; fn < FH; ++fn) {
            pin(bg[fn]);
            pin(bu[fn]);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < S::A_PW; ++j)
                pin(srow[j]);
            gemm1_src<S, PACKED>(g, nxt, srow, src);
            dma_prologue_p<S>(src, ring, 0, nk1, wave);
        }
        // epilogue: bf16 z of the real rows, staged in the ring slot that no
        // DMA touches before the next tile's first barrier (the prologue
        // above fills slots 0 .. NS-2), then written as 16-byte row chunks.
        // A tile whose z does not fit one slot (256 rows) stages it one row
        // group at a time.
        constexpr int ZS = S::BN / 2 + 8;               // staged row, bf16 elements
        constexpr int ZP = (S::CH * ZS * 2 + S::CH * 4 <= S::STAGE) ? 1 : 2;   // passes
        constexpr int ZR = S::CH / ZP;                  // rows staged per pass
        static_assert(ZR * ZS * 2 + S::CH * 4 <= S::STAGE, "z staging fits in one ring slot");
        static_assert(ZP == 1 || ZR == S::FMW * 16, "a pass stages one row group");
        u16* Zs = (u16*)(ring + (S::NS - 1) * S::STAGE);
        float* rws = (float*)(ring + (S::NS - 1) * S::STAGE + ZR * ZS * 2);
        if (g.row_w) {          // routing weights of the tile's rows, applied to z
            for (int t = threadIdx.x; t < S::CH; t += S::NT)
                rws[t] = (t < cur.rows) ? gemm1_row_w(g, (int64_t)cur.r0 + t) : 0.0f;
            __syncthreads();
        }
        constexpr int CPR = S::BN / 16;                 // 16-byte chunks per z row
#pragma unroll
        for (int pass = 0; pass < ZP; ++pass) {
            if (ZP == 1 || rg == pass) {
#pragma unroll
                for (int fn = 0; fn < FH; ++fn) {
                    const int zc = (cg * FH + fn) * 16 + s16;
#pragma unroll
                    for (int fm = 0; fm < FMW; ++fm) {
                        if (rg * FMW + fm >= strips)
                            continue;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = (rg * FMW + fm) * 16 + g4 * 4 + r;
                            float zv = silu_mul(acc[fm][fn][r] + bg[fn],
                                                acc[fm][fn + FH][r] + bu[fn]);
                            if (g.row_w)
                                zv *= rws[row];
                            Zs[(row - pass * ZR) * ZS + zc] = f32_to_bf16(zv);
                        }
                    }
                }
            }
            __syncthreads();
            const int r_lo = pass * ZR, nr = min(cur.rows - r_lo, ZR);
            for (int q = threadIdx.x; q < nr * CPR; q += S::NT) {
                const int row = q / CPR, c8 = (q % CPR) * 8;
                if (n0 + c8 < I)
                    *(i32x4*)((u16*)g.z + ((int64_t)cur.r0 + r_lo + row) * I + n0 + c8) =
                        *(const i32x4*)(Zs + row * ZS + c8);
            }
            if (pass + 1 < ZP)
                __syncthreads();                        // the next pass reuses the staging rows
        }
        if (!more)
            break;
        cur = nxt;
    }
}

// Persistent GEMM2 over this workgroup's tiles, pipelined across tiles like
// GEMM1; the epilogue (bias, output rows) runs straight from the accumulators.
template <int FMW, int WC, int NS, bool PACKED, int Q = 0, int G2 = 0, int L = 0>
__global__ void __launch_bounds__((DS<FMW, WC, NS, Q, G2, L>::NT), 2)
    k_gemm2_dma(Gemm2Args g)
{
    typedef DS<FMW, WC, NS, Q, G2, L> S;
    constexpr int FN = S::FN;
    __shared__ __attribute__((aligned(16))) char ring[S::RING];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / S::WC, cg = wave % S::WC;
    const int H = g.H;

    // with a K split, logical column block ntile = 2 c + h is block c over the
    // K half h; unit() splits it
    const int nk2 = (g.I + 63) / 64, kmid = nk2 / 2;
    auto unit = [&](TileRef t, int& kb, int& ke, int& part) {
        part = (g.ksplit == 2) ? (t.ntile & 1) : 0;
        if (g.ksplit == 2)
            t.ntile >>= 1;
        kb = (g.ksplit == 2 && part) ? kmid : 0;
        ke = (g.ksplit == 2 && !part) ? kmid : nk2;
        return t;
    };
    TileIter<S::CH> it(g.s);
    TileRef cur;
    if (!it.next(g.s, cur))
        return;
    int kb, ke, part;
    cur = unit(cur, kb, ke, part);
    DmaTile<S, PACKED, false> src;
    gemm2_src<S, PACKED>(g, cur, wave, src);
    dma_prologue_p<S>(src, ring, kb, ke, wave);

    int bblk[FN], bchunk[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int cl = (cg * FN + fn) * 16;
        bblk[fn] = cl / 128;
        bchunk[fn] = (cl % 128) / 8;
    }
    DmaFrag<S> fr;
    if constexpr (Q != 0)
        fr.init_q(lane, bchunk, g.w2_zero != nullptr);
    else
        fr.init(lane, bblk, bchunk);
    const int g4 = lane >> 4, s16 = lane & 15;

    for (;;) {
        TileRef nxt;
        const bool more = it.next(g.s, nxt);
        int nkb = 0, nke = 0, npart = 0;
        if (more)
            nxt = unit(nxt, nkb, nke, npart);
        const int c0 = cur.ntile * S::BN;
        const int strips = (cur.rows + 15) >> 4;
        // output row r0 + row goes to o[r0 + row] (padded position) or, for the
        // batched slabs, to out[e * T + (r0 - base) + row]
        const int64_t dst0 = (g.out_mode == 2) ? (int64_t)cur.r0
                                               : (int64_t)cur.e * g.T + (cur.r0 - cur.base);
        // (checked build: the output rows must lie in o, or in the slabs)
        const bool dst_ok =
            in_bounds(dst0, g.out_mode == 2 ? g.s.cap : (int64_t)g.s.E * g.T, g.s.status) &&
            in_bounds(dst0 + cur.rows - 1, g.out_mode == 2 ? g.s.cap : (int64_t)g.s.E * g.T,
                      g.s.status);
        float bias[FN];   // the bias belongs to the first K half only
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int c = c0 + (cg * FN + fn) * 16 + s16;
            bias[fn] = (g.b2 && c < H && part == 0)
                           ? load_bias(g.b2, g.bias_dt, (int64_t)cur.e * H + c)
                           : 0.0f;
        }
        f32x4 acc[FMW][FN];
        zero_acc<S>(acc);
        dma_run<S>(src, ring, kb, ke, wave, rg, fr, acc, min(max(strips - rg * FMW, 0), FMW));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            pin(bias[fn]);
        float* const outf = part ? g.out2 : (float*)g.out;
        if (more) {
            gemm2_src<S, PACKED>(g, nxt, wave, src);
            dma_prologue_p<S>(src, ring, nkb, nke, wave);
        }
        const bool obf = g.out_mode == 1 && g.out_dt == MOE_BF16;
        if (g.vec_out) {
            // each fragment's 4 x 4 lane quads transposed: lane (g4, 4a + q)
            // stores row 4 g4 + q of the strip, columns 4a .. 4a + 3
            const int q = s16 & 3;
            const int col_off = c0 + cg * FN * 16 + (s16 & ~3);
#pragma unroll
            for (int fm = 0; fm < FMW; ++fm) {
                const int strip = rg * FMW + fm;
                if (strip >= strips || !dst_ok)
                    continue;
                const int row = strip * 16 + g4 * 4 + q;
                const int64_t base = (dst0 + row) * H + col_off;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    if (c0 + (cg * FN + fn) * 16 >= H)
                        continue;
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = acc[fm][fn][r] + bias[fn];
                    quad_transpose(v, lane);
                    if (row < cur.rows)
                        store_row4(obf ? g.out : (void*)outf, base + fn * 16, obf, v);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
        // row (strip, g4*4 + r): uniform base of the strip's 16 rows plus this
        // lane's offset, one strip at a time (keeps the addresses out of registers)
        const int lane_off = g4 * 4 * H + c0 + cg * FN * 16 + s16;
#pragma unroll
        for (int fm = 0; fm < FMW; ++fm) {
            const int strip = rg * FMW + fm;
            if (strip >= strips || !dst_ok)
                continue;
            const int64_t base = (dst0 + strip * 16) * H;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (strip * 16 + g4 * 4 + r >= cur.rows)
                    continue;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    if (c0 + (cg * FN + fn) * 16 + s16 >= H)
                        continue;
                    const float v = acc[fm][fn][r] + bias[fn];
                    const int64_t o = base + lane_off + r * H + fn * 16;
                    if (obf)
                        ((u16*)g.out)[o] = f32_to_bf16(v);
                    else
                        outf[o] = v;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
        if (!more)
            break;
        cur = nxt;
        kb = nkb;
        ke = nke;
        part = npart;
    }
}

// ================================================================ weight packing
// One-time re-layout of bf16 expert weights into 16 KiB blocks of 64 weight
// rows x 128 weight columns, each row's 16-byte chunks swizzled by swz_b, so
// that one K stage of a GEMM tile is one contiguous block and a DMA of it is
// a linear copy (the layout is spelled out next to moe_pack_weights in
// moe.h).  One thread per 16-byte slot of the output; out-of-range rows and
// columns are written as zeros.
__global__ void __launch_bounds__(256) k_pack_w13(const u16* __restrict__ w, int H, int I,
                                                  i32x4* __restrict__ out, int64_t slots)
{
    const int64_t nblk = (I + 63) / 64, nks = (H + 63) / 64;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < slots;
         q += (int64_t)gridDim.x * 256) {
        const int sl = (int)(q & 15), k = (int)((q >> 4) & 63);
        const int64_t b = q >> 10;                      // block (e, kt, j)
        const int j = (int)(b % nblk);
        const int kt = (int)((b / nblk) % nks);
        const int64_t e = b / nblk / nks;
        const int c = sl ^ swz_b(k);
        const int row = kt * 64 + k, zc = 64 * j + 8 * (c & 7);
        i32x4 v = {0, 0, 0, 0};
        if (row < H && zc < I)
            v = *(const i32x4*)(w + (e * H + row) * 2 * I + (c < 8 ? zc : I + zc));
        out[q] = v;
    }
}

__global__ void __launch_bounds__(256) k_pack_w2(const u16* __restrict__ w, int H, int I,
                                                 i32x4* __restrict__ out, int64_t slots)
{
    const int64_t nblk = (H + 127) / 128, nks = (I + 63) / 64;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < slots;
         q += (int64_t)gridDim.x * 256) {
        const int sl = (int)(q & 15), k = (int)((q >> 4) & 63);
        const int64_t b = q >> 10;                      // block (e, kt, j)
        const int j = (int)(b % nblk);
        const int kt = (int)((b / nblk) % nks);
        const int64_t e = b / nblk / nks;
        const int c = sl ^ swz_b(k);
        const int row = kt * 64 + k, col = 128 * j + 8 * c;
        i32x4 v = {0, 0, 0, 0};
        if (row < I && col < H)
            v = *(const i32x4*)(w + (e * I + row) * H + col);
        out[q] = v;
    }
}

hipError_t launch_pack_weights(int E, int H, int I, const void* w13, const void* w2, void* p13,
                               void* p2, hipStream_t s)
{
    const int64_t s13 = (int64_t)E * ((I + 63) / 64) * ((H + 63) / 64) * (PACK_BLOCK / 16);
    const int64_t s2 = (int64_t)E * ((H + 127) / 128) * ((I + 63) / 64) * (PACK_BLOCK / 16);
    auto grid = [](int64_t slots) {
        const int64_t b = (slots + 255) / 256;
        return (unsigned)(b < 16384 ? b : 16384);
    };
    hipLaunchKernelGGL(k_pack_w13, dim3(grid(s13)), dim3(256), 0, s, (const u16*)w13, H, I,
                       (i32x4*)p13, s13);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(k_pack_w2, dim3(grid(s2)), dim3(256), 0, s, (const u16*)w2, H, I,
                       (i32x4*)p2, s2);
    return hipGetLastError();
}

// One-time re-layout of WNA16 weight codes (Q = 8: one byte per weight; Q = 4:
// two per byte along N, the even column in the low nibble) into blocks of
// 128 columns x 64 K in MFMA fragment order (the layout in moe.h): one
// thread per lane group of 8 codes of one column.  Codes past K or N are 0.
//   w13 [E, H, 2I]: block (e, kt, j), j < ceil(I / 64): block columns 0-63 =
//     gate columns 64 j .., 64-127 = up columns I + 64 j ..
//   w2 [E, I, H]: block (e, kt, j), j < ceil(H / 128): columns 128 j ..
template <bool W13, int Q>
__global__ void __launch_bounds__(256) k_pack_wq(const uint8_t* __restrict__ w, int H, int I,
                                                 uint8_t* __restrict__ out, int64_t groups)
{
    const int K = W13 ? H : I, N = W13 ? 2 * I : H;
    const int64_t nblk = W13 ? (I + 63) / 64 : (H + 127) / 128, nks = (K + 63) / 64;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < groups;
         q += (int64_t)gridDim.x * 256) {
        const int l = (int)(q & 63), ks = (int)((q >> 6) & 1), f = (int)((q >> 7) & 7);
        const int64_t b = q >> 10;                      // block (e, kt, j)
        const int j = (int)(b % nblk);
        const int kt = (int)((b / nblk) % nks);
        const int64_t e = b / nblk / nks;
        const int c = 16 * f + (l & 15);                // block column
        int col;
        bool valid;
        if constexpr (W13) {
            const int zc = 64 * j + (c & 63);
            valid = zc < I;
            col = (c < 64) ? zc : I + zc;
        } else {
            col = 128 * j + c;
            valid = col < H;
        }
        const int k0 = 64 * kt + 32 * ks + 8 * (l >> 4);
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = k0 + i;
            code[i] = 0;
            if (valid && row < K) {
                const int64_t r = e * K + row;
                if constexpr (Q == 8)
                    code[i] = w[r * N + col];
                else
                    code[i] = (w[r * (N / 2) + col / 2] >> (4 * (col & 1))) & 15u;
            }
        }
        if constexpr (Q == 8) {
            const uint32_t lo = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
            const uint32_t hi = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
            *(i32x2*)(out + q * 8) = i32x2{(int)lo, (int)hi};
        } else {
            // code i in nibble i / 2 + 4 (i & 1): the low nibbles of bytes
            // 0 and 2 are codes 0 and 1, their high nibbles codes 2 and 3,
            // bytes 1 and 3 the same for codes 4-7 (one byte permute then
            // lays a pair of codes out as two bf16 values, see raw_codes)
            uint32_t v = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v |= code[i] << (4 * (i / 2 + 4 * (i & 1)));
            *(uint32_t*)(out + q * 4) = v;
        }
    }
}

template <int Q>
static hipError_t pack_wq(int E, int H, int I, const void* w13, const void* w2, void* p13,
                          void* p2, hipStream_t s)
{
    const int64_t g13 = (int64_t)E * ((H + 63) / 64) * ((I + 63) / 64) * 1024;
    const int64_t g2 = (int64_t)E * ((I + 63) / 64) * ((H + 127) / 128) * 1024;
    auto grid = [](int64_t n) {
        const int64_t b = (n + 255) / 256;
        return (unsigned)(b < 16384 ? b : 16384);
    };
    hipLaunchKernelGGL((k_pack_wq<true, Q>), dim3(grid(g13)), dim3(256), 0, s,
                       (const uint8_t*)w13, H, I, (uint8_t*)p13, g13);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL((k_pack_wq<false, Q>), dim3(grid(g2)), dim3(256), 0, s,
                       (const uint8_t*)w2, H, I, (uint8_t*)p2, g2);
    return hipGetLastError();
}

hipError_t launch_pack_weights_wq(int bits, int E, int H, int I, const void* w13, const void* w2,
                                  void* p13, void* p2, hipStream_t s)
{
    return bits == 8 ? pack_wq<8>(E, H, I, w13, w2, p13, p2, s)
                     : pack_wq<4>(E, H, I, w13, w2, p13, p2, s);
}

// ---------------------------------------------------------------- GPTQ / AWQ codes
// Checkpoint int32 words -> the plain WNA16 codes (the layouts are spelled
// out next to moe_repack_wna16 in moe.h).  One thread per output byte (one
// 8-bit code, or the two 4-bit codes of columns 2p, 2p + 1), then one per
// zero point.  In an AWQ word, column 8c + j sits in slot (j >> 1) + 4 (j & 1).
template <int BITS, bool AWQ>
__device__ __forceinline__ int wq_checkpoint_code(const int32_t* __restrict__ qw, int64_t e,
                                                  int64_t K, int64_t N, int64_t k, int64_t n)
{
    constexpr int PER = 32 / BITS;
    uint32_t w;
    int slot;
    if constexpr (AWQ) {
        w = (uint32_t)qw[(e * K + k) * (N / 8) + n / 8];
        slot = (int)((n & 7) >> 1) + 4 * (int)(n & 1);
    } else {
        w = (uint32_t)qw[(e * (K / PER) + k / PER) * N + n];
        slot = (int)(k % PER);
    }
    return (int)((w >> (BITS * slot)) & ((1u << BITS) - 1u));
}

template <int BITS, bool AWQ>
__global__ void __launch_bounds__(256) k_repack_wq(const int32_t* __restrict__ qw,
                                                   const int32_t* __restrict__ qz, int zero_adjust,
                                                   int64_t E, int64_t K, int64_t N, int64_t ng,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ zeros)
{
    constexpr int PER = 32 / BITS;
    const int64_t per_row = (BITS == 8) ? N : N / 2;        // output bytes per K row
    const int64_t nc = E * K * per_row, nz = qz ? E * ng * N : 0;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < nc + nz;
         q += (int64_t)gridDim.x * 256) {
        if (q < nc) {
            const int64_t row = q / per_row, b = q % per_row;
            const int64_t e = row / K, k = row % K;
            if constexpr (BITS == 8) {
                codes[q] = (uint8_t)wq_checkpoint_code<8, AWQ>(qw, e, K, N, k, b);
            } else {
                const int lo = wq_checkpoint_code<4, AWQ>(qw, e, K, N, k, 2 * b);
                const int hi = wq_checkpoint_code<4, AWQ>(qw, e, K, N, k, 2 * b + 1);
                codes[q] = (uint8_t)(lo | (hi << 4));
            }
        } else {
            const int64_t zq = q - nc, n = zq % N, eg = zq / N;    // eg = e * ng + g
            uint32_t w;
            int slot;
            if constexpr (AWQ) {
                w = (uint32_t)qz[eg * (N / 8) + n / 8];
                slot = (int)((n & 7) >> 1) + 4 * (int)(n & 1);
            } else {
                w = (uint32_t)qz[eg * (N / PER) + n / PER];
                slot = (int)(n % PER);
            }
            const int z = (int)((w >> (BITS * slot)) & ((1u << BITS) - 1u));
            zeros[zq] = (uint8_t)((z + zero_adjust) & ((1 << BITS) - 1));
        }
    }
}

hipError_t launch_repack_wq(int format, int bits, int64_t E, int64_t K, int64_t N, int64_t ng,
                            const int32_t* qw, const int32_t* qz, int zero_adjust,
                            uint8_t* codes, uint8_t* zeros, hipStream_t s)
{
    const int64_t n = E * K * (bits == 8 ? N : N / 2) + (qz ? E * ng * N : 0);
    const int64_t b = (n + 255) / 256;
    const dim3 grid((unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536)), block(256);
    const bool awq = format == MOE_WQ_AWQ;
    if (bits == 8)
        hipLaunchKernelGGL((k_repack_wq<8, false>), grid, block, 0, s, qw, qz, zero_adjust, E, K,
                           N, ng, codes, zeros);
    else if (awq)
        hipLaunchKernelGGL((k_repack_wq<4, true>), grid, block, 0, s, qw, qz, zero_adjust, E, K,
                           N, ng, codes, zeros);
    else
        hipLaunchKernelGGL((k_repack_wq<4, false>), grid, block, 0, s, qw, qz, zero_adjust, E, K,
                           N, ng, codes, zeros);
    return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
template <int DT, int FM, int WN>
static hipError_t run_gemm1(const Gemm1Args& a, const Plan& P, hipStream_t s)
{
    typedef Shape<DT, FM, WN, 2> S;
    Gemm1Args g = a;
    g.s.n_tiles = (a.I + S::BNZ - 1) / S::BNZ;
    auto kern = k_gemm1<DT, FM, WN>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P)),
        block(256);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

template <int DT, int FM, int WN>
static hipError_t run_gemm2(const Gemm2Args& a, const Plan& P, hipStream_t s)
{
    typedef Shape<DT, FM, WN, 1, DT == MOE_FP8_E4M3FN> S;
    Gemm2Args g = a;
    g.s.n_tiles = (a.H + S::BN - 1) / S::BN;
    auto kern = k_gemm2<DT, FM, WN>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P)),
        block(256);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

template <int FMW, int WC, int NS, bool PACKED, int Q = 0, int G2 = 0, int L = 0>
static hipError_t run_gemm1_dma(const Gemm1Args& a, const Plan& P, hipStream_t s)
{
    typedef DS<FMW, WC, NS, Q, G2, L> S;
    constexpr int BNZ = S::BN / 2;
    Gemm1Args g = a;
    g.s.n_tiles = (a.I + BNZ - 1) / BNZ;
    auto kern = k_gemm1_dma<FMW, WC, NS, PACKED, Q, G2, L>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P, S::NT)),
        block(S::NT);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

template <int FMW, int WC, int NS, bool PACKED, int Q = 0, int G2 = 0, int L = 0>
static hipError_t run_gemm2_dma(const Gemm2Args& a, const Plan& P, hipStream_t s)
{
    typedef DS<FMW, WC, NS, Q, G2, L> S;
    Gemm2Args g = a;
    g.s.n_tiles = (a.H + S::BN - 1) / S::BN * g.ksplit;
    auto kern = k_gemm2_dma<FMW, WC, NS, PACKED, Q, G2, L>;
    static std::atomic<int> cached[MAX_DEVICES];
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached, P, S::NT)),
        block(S::NT);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

// Expected number of GEMM row chunks: every active expert has at least one,
// and the routed rows fill at least rows / CH of them.
static int64_t expected_chunks(const Plan& P)
{
    return expected_chunks(P.fmt, P.M, P.K, P.E, P.T, P.CH);
}

// Routed rows per expert at most one tile height on average (over the
// global experts of a shard, whose items spread over all of them).
static bool about_one_chunk(const Plan& P)
{
    const int64_t rows = (P.fmt == MOE_FMT_BATCHED) ? (int64_t)P.E * P.T : (int64_t)P.M * P.K;
    const int64_t experts = P.Er > P.E ? P.Er : P.E;
    return rows <= experts * P.CH;
}

// Wave columns of the large bf16 GEMM1 tile: 4 (256 columns, 8 waves) when
// there are a few tiles per CU, or when experts hold about one row chunk on
// average (their weights are read once, and the wide tile halves the column
// tiles that re-read each chunk's activation rows through L2), else 2.  A
// caller's gemm1_wave_cols (2 or 4) overrides the choice.
static int gemm1_wave_cols(const Plan& P)
{
    if (P.g1wc == 2 || P.g1wc == 4)
        return P.g1wc;
    if (about_one_chunk(P))
        return 4;
    return expected_chunks(P) * ((P.I + 127) / 128) <= 8 * (int64_t)P.cus ? 4 : 2;
}

int stream_device(hipStream_t s)
{
    int dev = 0;
    if (s) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(s, &d) == hipSuccess)
            return (int)d;
        (void)hipGetLastError();
    }
    (void)hipGetDevice(&dev);
    return dev;
}

int device_cus(int dev)
{
    static std::atomic<int> cache[MAX_DEVICES];
    const int slot = (dev >= 0 && dev < MAX_DEVICES) ? dev : -1;
    int cus = slot >= 0 ? cache[slot].load(std::memory_order_relaxed) : 0;
    if (cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            (void)hipGetLastError();
        cus = n > 0 ? n : 256;
        if (slot >= 0)
            cache[slot].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

static Sched make_sched(const Plan& P)
{
    Sched s{};
    s.counts = P.counts;
    s.offsets = P.offsets;
    s.chunk_off = P.chunk_off;
    s.chunk_expert = P.chunk_expert;
    s.sorted = P.sorted_ids;
    s.sentinel = (int)P.sentinel;
    s.E = P.E;
    s.cap = P.max_sorted;
    s.max_chunks = P.max_blocks;
    s.status = P.status;
    return s;
}

// Tile families (Plan::cfg) and their rows per tile CH (Plan::CH):
//   TILE_PREFILL  10 strips, CH 160: one tile holds a whole expert at ~128 rows/expert
//   TILE_MID       4 strips, CH 64
//   TILE_DECODE    1 strip,  CH 16: a few rows per expert
//   TILE_FP8       8 strips, CH 128, 128-column z groups
// WNA16 (Q code bits) runs the DMA tile families with one weight block a
// tile; G2: groups of 32 K rows, two to a 64-row stage.
template <int Q, int G2>
static hipError_t launch_gemm1_wq(const Gemm1Args& g, const Plan& P, hipStream_t s)
{
    switch (P.cfg) {
    case TILE_DECODE_DMA: return run_gemm1_dma<2, 4, 4, true, Q, G2, 1>(g, P, s);
    case TILE_MID_DMA: return run_gemm1_dma<2, 2, 3, true, Q, G2>(g, P, s);
    default: return run_gemm1_dma<5, 2, 2, true, Q, G2>(g, P, s);
    }
}

template <int Q, int G2>
static hipError_t launch_gemm2_wq(const Gemm2Args& g, const Plan& P, hipStream_t s)
{
    switch (P.cfg) {
    case TILE_DECODE_DMA: return run_gemm2_dma<2, 4, 4, true, Q, G2, 1>(g, P, s);
    case TILE_MID_DMA: return run_gemm2_dma<2, 2, 3, true, Q, G2>(g, P, s);
    default: return run_gemm2_dma<5, 2, 2, true, Q, G2>(g, P, s);
    }
}

hipError_t launch_gemm1(const Plan& P, const moe_args& A, const float* row_w, hipStream_t s)
{
    Gemm1Args g{};
    g.s = make_sched(P);
    g.row_w = row_w;
    const bool fp8 = P.wdt == MOE_FP8_E4M3FN;
    if (fp8) {
        if (P.act == MOE_FP8_E4M3FN) {           // batched, pre-quantised codes
            g.a = A.hidden;
            g.a_scale = A.a_scale;
            g.a_ident = 0;
            g.a_div = 1;
        } else {                                 // quantised by k_quant_rows
            g.a = P.aq;
            g.a_scale = P.aq_scale;
            g.a_ident = (P.fmt == MOE_FMT_BATCHED) ? 1 : 0;
            g.a_div = P.K;
        }
    } else {
        g.a = A.hidden;
        g.a_ident = 0;
        g.a_div = (P.fmt == MOE_FMT_BATCHED) ? 1 : P.K;
    }
    g.w13 = A.w13;
    g.w_packed = P.wpacked;
    g.w13_scale = A.w13_scale;
    g.w13_zero = A.w13_zero;
    g.blk = P.blk;
    g.a_sld = P.blk ? (P.H + 127) / 128 : 1;
    g.b13 = P.has_b13 ? A.w13_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    g.z = P.z;
    g.z_scale = P.z_scale;
    g.zs_ld = P.zs_ld;
    if (fp8)
        return P.wpacked ? launch_gemm1_fp8(g, P, s) : run_gemm1<MOE_FP8_E4M3FN, 8, 32>(g, P, s);
    if (P.wdt == MOE_F32)
        return run_gemm1<MOE_F32, 1, 16>(g, P, s);
    g.wq_gsh = P.wq_gsh;
    if (P.wq == 8)
        return P.wq_gsh ? launch_gemm1_wq<8, 0>(g, P, s) : launch_gemm1_wq<8, 1>(g, P, s);
    if (P.wq == 4)
        return P.wq_gsh ? launch_gemm1_wq<4, 0>(g, P, s) : launch_gemm1_wq<4, 1>(g, P, s);
    switch (P.cfg) {
    case TILE_PREFILL_BIG:
        // about a thousand rows per expert: 256 x 256 tiles, 8 waves of
        // 128 x 64, a 2-stage ring (half the fragment reads per MFMA of the
        // 160-row tiles)
        return P.wpacked ? run_gemm1_dma<8, 4, 2, true>(g, P, s)
                         : run_gemm1_dma<8, 4, 2, false>(g, P, s);
    case TILE_PREFILL:
        // a few tiles per CU (few experts, wide I): 256-column tiles, 8 waves and
        // a 3-stage ring at one workgroup per CU stream the weights fastest;
        // with many tiles per CU two 4-wave workgroups per CU hide the tile
        // transitions better
        if (gemm1_wave_cols(P) == 4)
            return P.wpacked ? run_gemm1_dma<5, 4, 3, true>(g, P, s)
                             : run_gemm1_dma<5, 4, 3, false>(g, P, s);
        return P.wpacked ? run_gemm1_dma<5, 2, 2, true>(g, P, s)
                         : run_gemm1_dma<5, 2, 2, false>(g, P, s);
    case TILE_MID: return run_gemm1<MOE_BF16, 4, 16>(g, P, s);
    case TILE_DECODE_DMA:
        return P.wpacked ? run_gemm1_dma<2, 4, 4, true, 0, 0, 1>(g, P, s)
                         : run_gemm1_dma<2, 4, 4, false, 0, 0, 1>(g, P, s);
    case TILE_MID_DMA:
        return P.wpacked ? run_gemm1_dma<2, 2, 3, true>(g, P, s)
                         : run_gemm1_dma<2, 2, 3, false>(g, P, s);
    default: return run_gemm1<MOE_BF16, 1, 16>(g, P, s);
    }
}

hipError_t launch_gemm2(const Plan& P, const moe_args& A, hipStream_t s)
{
    Gemm2Args g{};
    g.s = make_sched(P);
    g.z = P.z;
    g.z_scale = P.z_scale;
    g.zs_ld = P.zs_ld;
    g.w2 = A.w2;
    g.w_packed = P.wpacked;
    g.w2_scale = A.w2_scale;
    g.w2_zero = A.w2_zero;
    g.blk = P.blk;
    g.b2 = P.has_b2 ? A.w2_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    g.T = P.T;
    g.ksplit = 1;
    g.out2 = P.o2;
    if (P.fmt == MOE_FMT_CONTIGUOUS) {
        g.out_mode = 2;
        g.out = P.o;
        g.out_dt = MOE_F32;
    } else if (P.breduce) {
        g.out_mode = 2;
        g.out = P.o;
        g.out_dt = MOE_F32;
    } else {
        g.out_mode = 1;
        g.out = A.out;
        g.out_dt = P.outdt;
    }
    // bf16 output rows are stored as 8-byte row pieces after a lane-quad
    // transpose (one value a lane would store 2 bytes; batched fp8 W2 GEMM
    // 291 -> 271 us).  Float rows keep one value a lane: 16 lanes already
    // store 64 contiguous bytes, and the transpose measured 1-2% slower
    // there.  The pieces need 8-byte aligned rows: H is a multiple of 16, so
    // the base pointer decides.
    g.vec_out = g.out_mode == 1 && g.out_dt == MOE_BF16 && (uintptr_t)g.out % 8 == 0;
    if (P.wdt == MOE_FP8_E4M3FN)
        return P.wpacked ? launch_gemm2_fp8(g, P, s) : run_gemm2<MOE_FP8_E4M3FN, 8, 32>(g, P, s);
    if (P.wdt == MOE_F32)
        return run_gemm2<MOE_F32, 1, 16>(g, P, s);
    g.wq_gsh = P.wq_gsh;
    if (P.wq == 8)
        return P.wq_gsh ? launch_gemm2_wq<8, 0>(g, P, s) : launch_gemm2_wq<8, 1>(g, P, s);
    if (P.wq == 4)
        return P.wq_gsh ? launch_gemm2_wq<4, 0>(g, P, s) : launch_gemm2_wq<4, 1>(g, P, s);
    switch (P.cfg) {
    case TILE_PREFILL_BIG:
        return P.wpacked ? run_gemm2_dma<8, 4, 2, true>(g, P, s)
                         : run_gemm2_dma<8, 4, 2, false>(g, P, s);
    case TILE_PREFILL:
        if (P.g2split) {   // 256-column tiles over two K halves
            g.ksplit = 2;
            return P.wpacked ? run_gemm2_dma<5, 4, 3, true>(g, P, s)
                             : run_gemm2_dma<5, 4, 3, false>(g, P, s);
        }
        // experts of about one row chunk on average: 256-column tiles, so half
        // as many column tiles re-read each chunk's z rows through L2
        if (about_one_chunk(P))
            return P.wpacked ? run_gemm2_dma<5, 4, 3, true>(g, P, s)
                             : run_gemm2_dma<5, 4, 3, false>(g, P, s);
        // about one tile per CU: one workgroup per CU with a 4-stage ring keeps
        // three K stages in flight; otherwise two workgroups per CU overlap
        // each other's prologues and epilogues
        if (expected_chunks(P) * ((P.H + 127) / 128) <= (int64_t)P.cus * 5 / 4)
            return P.wpacked ? run_gemm2_dma<5, 2, 4, true>(g, P, s)
                             : run_gemm2_dma<5, 2, 4, false>(g, P, s);
        return P.wpacked ? run_gemm2_dma<5, 2, 2, true>(g, P, s)
                         : run_gemm2_dma<5, 2, 2, false>(g, P, s);
    case TILE_MID: return run_gemm2<MOE_BF16, 4, 32>(g, P, s);
    case TILE_DECODE_DMA:
        return P.wpacked ? run_gemm2_dma<2, 4, 4, true, 0, 0, 1>(g, P, s)
                         : run_gemm2_dma<2, 4, 4, false, 0, 0, 1>(g, P, s);
    case TILE_MID_DMA:
        return P.wpacked ? run_gemm2_dma<2, 2, 3, true>(g, P, s)
                         : run_gemm2_dma<2, 2, 3, false>(g, P, s);
    default: return run_gemm2<MOE_BF16, 1, 32>(g, P, s);
    }
}

}  // namespace moe
