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
#include "moe_internal.h"

namespace moe {

typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

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

// sched_group_barrier instruction classes
constexpr int SCHED_MFMA = 0x008, SCHED_DS_READ = 0x100;

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

__device__ __forceinline__ float load_bias(const void* b, int dt, int64_t idx)
{
    return (dt == MOE_BF16) ? bf16_to_f32(((const u16*)b)[idx]) : ((const float*)b)[idx];
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------------- arguments
struct Sched {
    const int32_t* counts;      // [E] real rows per expert
    const int32_t* offsets;     // [E + 1] start of each expert's padded run
    const int32_t* chunk_off;   // [E + 1] chunk prefix per expert
    const int32_t* chunk_expert;
    const int32_t* sorted;
    int sentinel;
    int E, n_tiles;
};

struct Gemm1Args {
    Sched s;
    const void* a;              // activation rows [*, H] (f32 / bf16 / fp8 codes)
    const float* a_scale;       // fp8: per activation row
    int a_ident;                // 1: A row = padded position p; 0: sorted[p] / a_div
    int a_div;
    const void* w13;            // [E, H, 2I]
    const float* w13_scale;     // fp8: [E, 2I]
    const void* b13;            // [E, 2I] or null
    int bias_dt;
    int H, I;
    void* z;                    // [max_sorted, I]
    float* z_scale;             // fp8: [max_sorted, I/128]
};

struct Gemm2Args {
    Sched s;
    const void* z;
    const float* z_scale;
    const void* w2;             // [E, I, H]
    const float* w2_scale;      // fp8: [E, H]
    const void* b2;             // [E, H] or null
    int bias_dt;
    int H, I;
    int out_mode;               // 0: float o[sorted[p]]; 1: out[sorted[p]] (out_dt); 2: float o[p]
    int out_dt;
    void* out;
};

// ---------------------------------------------------------------- tile schedule
// Persistent, XCD-aware schedule.  Logical tiles are ordered by expert, then
// column block, then the expert's row chunks, so the chunks of one expert
// that share a weight tile are neighbours.  Workgroups are dealt round-robin
// over the 8 XCDs (workgroup b runs on XCD b % 8), so XCD x is given the
// contiguous range [x R/8, (x+1) R/8) of the R tiles and walks it with its own
// workgroups: neighbouring tiles run together on one XCD and share its L2.
// f(e, row0, rows, ntile): rows = real rows of the chunk (>= 1).
template <int CH, typename F>
__device__ __forceinline__ void for_each_tile(const Sched& s, F&& f)
{
    const int nt = s.n_tiles;
    const int R = s.chunk_off[s.E] * nt;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = gridDim.x >> 3;
    const int lo = (int)(((int64_t)R * xcd) >> 3), hi = (int)(((int64_t)R * (xcd + 1)) >> 3);
    for (int L = lo + slot; L < hi; L += per) {
        const int e = s.chunk_expert[L / nt];
        const int c0 = s.chunk_off[e], nch = s.chunk_off[e + 1] - c0;
        const int local = L - c0 * nt;
        const int j = local % nch;
        f(e, s.offsets[e] + j * CH, min(CH, s.counts[e] - j * CH), local / nch);
    }
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

    __device__ __forceinline__ void load(int kt, const char* abase, int64_t a_k_bytes,
                                         const char* wbase, int64_t w_ld_bytes, int K)
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
                rb[i] = *(const i32x4*)(wbase + (int64_t)k * w_ld_bytes + b_off[i]);
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
                if (sid < g.s.sentinel)
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
        st.b_off[i] = (n0 + zc < I) ? (int64_t)gcol * ES : -1;
    }
    const char* abase = (const char*)g.a;
    const char* wbase = (const char*)g.w13 + (int64_t)e * H * N * ES;

    f32x4 acc[2][FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[0][fm][fn] = acc[1][fm][fn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (H + S::BK - 1) / S::BK;
    st.load(0, abase, (int64_t)H * ES, wbase, (int64_t)N * ES, H);
    st.store(smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more)
            st.load(kt + 1, abase, (int64_t)H * ES, wbase, (int64_t)N * ES, H);
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
                        if (sid < g.s.sentinel)
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
        const int ngrp = I / 128;
        for (int rb = 0; rb < nrows; rb += 32) {
            const int row = rb + tid / 8, c0 = (tid % 8) * 16;
            if (row >= nrows)
                continue;                                // whole 8-lane groups skip together
            float v[16], amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                v[c] = Zs[row * S::O_STRIDE + c0 + c];
                amax = fmaxf(amax, fabsf(v[c]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
            const float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = (uint32_t)f32_to_fp8(v[4 * q] / sc) |
                       ((uint32_t)f32_to_fp8(v[4 * q + 1] / sc) << 8) |
                       ((uint32_t)f32_to_fp8(v[4 * q + 2] / sc) << 16) |
                       ((uint32_t)f32_to_fp8(v[4 * q + 3] / sc) << 24);
            const int64_t p = (int64_t)r0 + row;
            *(i32x4*)((uint8_t*)g.z + p * I + n0 + c0) =
                i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            if ((tid % 8) == 0)
                g.z_scale[p * ngrp + n0 / 128] = sc;
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
            if constexpr (DT == MOE_BF16) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w[k] = f32_to_bf16(src[2 * k]) | ((uint32_t)f32_to_bf16(src[2 * k + 1]) << 16);
                *(i32x4*)((u16*)g.z + p * I + n0 + c0) =
                    i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            } else {
                *(f32x4*)((float*)g.z + p * I + n0 + c0) = f32x4{src[0], src[1], src[2], src[3]};
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
    const int ngrp = I / 128;
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
        st.b_off[i] = (col < H) ? (int64_t)col * ES : -1;
    }
    const char* zbase = (const char*)g.z;
    const char* wbase = (const char*)g.w2 + (int64_t)e * I * H * ES;
    auto load = [&](int kt) {
        st.load(kt, zbase, (int64_t)I * ES, wbase, (int64_t)H * ES, I);
        if constexpr (FP8)
            st.rs = (tid < strips * 16) ? g.z_scale[((int64_t)r0 + tid) * ngrp + kt] : 0.0f;
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
        if (sid >= g.s.sentinel)
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

// ---------------------------------------------------------------- launchers
// Persistent grid: every workgroup the device holds at once (a multiple of
// the 8 XCDs), capped by the largest possible tile count.  Each kernel
// instance queries its occupancy once; `cached` is that instance's slot.
template <typename K>
static unsigned persistent_grid(K kernel, int64_t max_tiles, int& cached)
{
    if (cached == 0) {
        int dev = 0, cus = 0, occ = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 256, 0);
        cached = (cus > 0 ? cus : 256) * (occ > 0 ? occ : 1);
    }
    int64_t g = cached;
    const int64_t cap = (max_tiles + 7) / 8 * 8;
    if (g > cap)
        g = cap;
    g = (g + 7) / 8 * 8;
    return (unsigned)(g < 8 ? 8 : g);
}

template <int DT, int FM, int WN>
static hipError_t run_gemm1(const Gemm1Args& a, const Plan& P, hipStream_t s)
{
    typedef Shape<DT, FM, WN, 2> S;
    Gemm1Args g = a;
    g.s.n_tiles = (a.I + S::BNZ - 1) / S::BNZ;
    auto kern = k_gemm1<DT, FM, WN>;
    static int cached = 0;
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached)),
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
    static int cached = 0;
    const dim3 grid(persistent_grid(kern, (int64_t)P.max_blocks * g.s.n_tiles, cached)),
        block(256);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
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
    return s;
}

// Tile families (Plan::cfg) and their rows per tile CH (Plan::CH):
//   TILE_PREFILL  10 strips, CH 160: one tile holds a whole expert at ~128 rows/expert
//   TILE_MID       4 strips, CH 64
//   TILE_DECODE    1 strip,  CH 16: a few rows per expert
//   TILE_FP8       8 strips, CH 128, 128-column z groups
hipError_t launch_gemm1(const Plan& P, const moe_args& A, hipStream_t s)
{
    Gemm1Args g{};
    g.s = make_sched(P);
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
    g.w13_scale = A.w13_scale;
    g.b13 = P.has_b13 ? A.w13_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    g.z = P.z;
    g.z_scale = P.z_scale;
    if (fp8)
        return run_gemm1<MOE_FP8_E4M3FN, 8, 32>(g, P, s);
    if (P.wdt == MOE_F32)
        return run_gemm1<MOE_F32, 1, 16>(g, P, s);
    switch (P.cfg) {
    case TILE_PREFILL: return run_gemm1<MOE_BF16, 10, 16>(g, P, s);
    case TILE_MID: return run_gemm1<MOE_BF16, 4, 16>(g, P, s);
    default: return run_gemm1<MOE_BF16, 1, 16>(g, P, s);
    }
}

hipError_t launch_gemm2(const Plan& P, const moe_args& A, hipStream_t s)
{
    Gemm2Args g{};
    g.s = make_sched(P);
    g.z = P.z;
    g.z_scale = P.z_scale;
    g.w2 = A.w2;
    g.w2_scale = A.w2_scale;
    g.b2 = P.has_b2 ? A.w2_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    if (P.fmt == MOE_FMT_CONTIGUOUS) {
        g.out_mode = 0;
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
    if (P.wdt == MOE_FP8_E4M3FN)
        return run_gemm2<MOE_FP8_E4M3FN, 8, 32>(g, P, s);
    if (P.wdt == MOE_F32)
        return run_gemm2<MOE_F32, 1, 16>(g, P, s);
    switch (P.cfg) {
    case TILE_PREFILL: return run_gemm2<MOE_BF16, 10, 32>(g, P, s);
    case TILE_MID: return run_gemm2<MOE_BF16, 4, 32>(g, P, s);
    default: return run_gemm2<MOE_BF16, 1, 32>(g, P, s);
    }
}

}  // namespace moe
