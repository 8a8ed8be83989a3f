// Grouped expert GEMMs of the fused MoE forward on gfx950 MFMA.
//
// The organisation follows the FlagGems walkthrough ("fused_moe_kernel"
// section and sec. 1.3): routed items are sorted by expert and padded to
// BM-row blocks (align kernel); one workgroup computes one (BM-row block of
// one expert) x (column block) tile; the accumulator is float32 and is cast
// at the output; dequant, bias and activation are fused into the epilogue.
//
//   GEMM1: h[p, n] = sum_k A[row(p), k] * w13[e, k, n] (+ b13[e, n]);
//          z[p, i] = SiLU(h[p, i]) * h[p, I + i]            (gate | up halves)
//   GEMM2: o[p, c] = sum_i z[p, i] * w2[e, i, c] (+ b2[e, c])
//
// Data movement: both operands are copied global -> LDS as-is in 16-byte
// chunks (activations/z are K-contiguous rows, weights are N-contiguous
// rows).  A fragments are K-contiguous LDS reads; B fragments use the gfx950
// transposing LDS reads (ds_read_b64_tr_b16 / _b8), which hand each lane
// consecutive K values of one column straight from the N-contiguous tile.
// Two LDS stages; the next stage's global loads are in flight while the
// current one feeds the MFMAs.  Outputs are staged through LDS so global
// stores are full 16-byte vectors.
#include "moe_internal.h"

namespace moe {

typedef short i16x8 __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int DT>
struct GT;
template <>
struct GT<MOE_F32> {
    static constexpr int ES = 4, KM = 4, BK = 32, EPL = 1;
};
template <>
struct GT<MOE_BF16> {
    static constexpr int ES = 2, KM = 32, BK = 64, EPL = 8;
};
template <>
struct GT<MOE_FP8_E4M3FN> {
    static constexpr int ES = 1, KM = 128, BK = 128, EPL = 32;
};

constexpr int A_STRIDE = 128 + 16;   // bytes per A row in LDS (one K stage = 128 B)

template <int DT>
struct Frag;
template <>
struct Frag<MOE_F32> {
    typedef float A;
    typedef float B;
};
template <>
struct Frag<MOE_BF16> {
    typedef bf16x8 A;
    typedef bf16x8 B;
};
template <>
struct Frag<MOE_FP8_E4M3FN> {
    typedef i32x8 A;
    typedef i32x8 B;
};

// A fragment of a 16-row strip: lane l holds row l%16, K elements
// [(l/16)*EPL, +EPL) of the current MFMA step.
template <int DT>
__device__ __forceinline__ typename Frag<DT>::A load_a_frag(const char* As_row_base, int ks,
                                                            int lane)
{
    constexpr int ES = GT<DT>::ES, KM = GT<DT>::KM, EPL = GT<DT>::EPL;
    const char* p = As_row_base + (lane & 15) * A_STRIDE + (ks * KM + (lane >> 4) * EPL) * ES;
    if constexpr (DT == MOE_F32) {
        return *(const float*)p;
    } else if constexpr (DT == MOE_BF16) {
        return __builtin_bit_cast(bf16x8, *(const i32x4*)p);
    } else {
        const i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// B fragment of a 16-column strip starting at column `col` of the LDS tile
// (row stride bstride bytes): lane l holds column col + l%16, K elements
// [(l/16)*EPL, +EPL).  For 16- and 8-bit data the transposing reads deliver
// that directly: within each 16-lane group, the tr16 read gives lane j
// element j%4 of the 8-byte chunks read by lanes j/4 + 4i, and the tr8 read
// gives lane j byte j%8 of the chunks read by lanes j/8 + 2i, so each lane
// points at the chunk of the row/column block that lands where the MFMA
// expects it.
template <int DT>
__device__ __forceinline__ typename Frag<DT>::B load_b_frag(const char* Bs, int bstride, int ks,
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

template <int DT>
__device__ __forceinline__ f32x4 mma(typename Frag<DT>::A a, typename Frag<DT>::B b, f32x4 c)
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
struct Gemm1Args {
    const void* a;              // activation rows [*, H] (f32 / bf16 / fp8 codes)
    const float* a_scale;       // fp8: per activation row
    int a_ident;                // 1: A row = padded position p; 0: sorted[p] / a_div
    int a_div;
    const int32_t* sorted;
    const int32_t* expert_ids;
    const int32_t* offsets;     // [E + 1] padded run starts
    const int32_t* npp;
    int sentinel;
    const void* w13;            // [E, H, 2I]
    const float* w13_scale;     // fp8: [E, 2I]
    const void* b13;            // [E, 2I] or null
    int bias_dt;
    int H, I;
    int max_blocks, n_tiles;
    void* z;                    // [max_sorted, I]
    float* z_scale;             // fp8: [max_sorted, I/128]
};

struct Gemm2Args {
    const void* z;
    const float* z_scale;
    const int32_t* sorted;
    const int32_t* expert_ids;
    const int32_t* offsets;
    const int32_t* npp;
    int sentinel;
    const void* w2;             // [E, I, H]
    const float* w2_scale;      // fp8: [E, H]
    const void* b2;             // [E, H] or null
    int bias_dt;
    int H, I;
    int max_blocks, n_tiles;
    int out_mode;               // 0: float o[sorted[p]]; 1: out[sorted[p]] (out_dt); 2: float o[p]
    int out_dt;
    void* out;
};

// ---------------------------------------------------------------- tile schedule
// Persistent, XCD-aware schedule.  Logical tiles are ordered by expert, then
// column tile, then the expert's row blocks, so the row blocks of one expert
// that share a weight tile are neighbours, and one expert's activation rows
// are reused across its column tiles.  Workgroups are dealt round-robin over
// the 8 XCDs (workgroup b runs on XCD b % 8), so XCD x is given the contiguous
// chunk [x R/8, (x+1) R/8) of the R real tiles and walks it with its own
// workgroups: neighbouring tiles run together on one XCD and share its L2.
template <typename F>
__device__ __forceinline__ void for_each_tile(const int32_t* npp, const int32_t* expert_ids,
                                              const int32_t* offsets, int BM, int nt, F&& f)
{
    const int R = (*npp / BM) * nt;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = gridDim.x >> 3;
    const int lo = (int)(((int64_t)R * xcd) >> 3), hi = (int)(((int64_t)R * (xcd + 1)) >> 3);
    for (int L = lo + slot; L < hi; L += per) {
        const int e = expert_ids[L / nt];
        const int b0 = offsets[e] / BM, nb = offsets[e + 1] / BM - b0;
        const int local = L - b0 * nt;
        f(b0 + local % nb, local / nb);
    }
}

// ---------------------------------------------------------------- GEMM1
template <int DT, int BM, int BNZ, int WAVES_M>
struct G1Cfg {
    static constexpr int ES = GT<DT>::ES, BK = GT<DT>::BK, KM = GT<DT>::KM;
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int WM = BM / WAVES_M, WNZ = BNZ / WAVES_N;
    static constexpr int FM = WM / 16, FN = WNZ / 16;
    static constexpr int BN = 2 * BNZ;                     // gate block | up block
    static constexpr int B_STRIDE = BN * ES + 16;
    static constexpr int A_CHUNKS = BM * 8;                // 16-B chunks per stage
    static constexpr int B_CPR = BN * ES / 16;             // chunks per B row
    static constexpr int B_CHUNKS = BK * B_CPR;
    static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
    static constexpr int B_PER_T = B_CHUNKS / 256;
    static constexpr int STAGE_BYTES = BM * A_STRIDE + BK * B_STRIDE;
    static constexpr int PIPE_BYTES = 2 * STAGE_BYTES + BM * 4;
    static constexpr int Z_STRIDE = BNZ + 4;               // floats
    static constexpr int EPI_BYTES = BM * Z_STRIDE * 4;
    static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
    static_assert(B_CHUNKS % 256 == 0, "B tile must split evenly over 256 threads");
    static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA tile");
};

template <int DT, int BM, int BNZ, int WAVES_M>
__device__ __forceinline__ void gemm1_tile(const Gemm1Args& g, char* smem, int mblk, int ntile)
{
    typedef G1Cfg<DT, BM, BNZ, WAVES_M> C;
    constexpr int ES = C::ES, BK = C::BK, KM = C::KM;
    float* a_rowscale = (float*)(smem + 2 * C::STAGE_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / C::WAVES_N, wave_n = wave % C::WAVES_N;
    const int e = g.expert_ids[mblk];
    const int H = g.H, I = g.I, N = 2 * I;
    const int n0 = ntile * BNZ;
    const int64_t p0 = (int64_t)mblk * BM;

    // activation rows of this block (fixed over the K loop)
    int64_t a_off[C::A_PER_T];
    int a_kc[C::A_PER_T], a_row[C::A_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int q = tid + 256 * i;
        a_row[i] = q / 8;
        a_kc[i] = q % 8;
        a_off[i] = -1;
        if (q < C::A_CHUNKS) {
            const int64_t p = p0 + a_row[i];
            int64_t src = -1;
            if (g.a_ident) {
                src = p;
            } else {
                const int sid = g.sorted[p];
                if (sid < g.sentinel)
                    src = sid / g.a_div;
            }
            if (src >= 0)
                a_off[i] = src * (int64_t)H * ES;
        }
    }
    if constexpr (DT == MOE_FP8_E4M3FN) {
        for (int r = tid; r < BM; r += 256) {
            const int64_t p = p0 + r;
            float sc = 0.0f;
            if (g.a_ident) {
                sc = g.a_scale[p];
            } else {
                const int sid = g.sorted[p];
                if (sid < g.sentinel)
                    sc = g.a_scale[sid / g.a_div];
            }
            a_rowscale[r] = sc;
        }
    }
    // weight chunks: row kk, column chunk cc of the [BK, gate|up] tile
    int64_t b_col_off[C::B_PER_T];
    int b_kk[C::B_PER_T], b_lds[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int kk = q / C::B_CPR, cc = q % C::B_CPR;
        const int col = cc * 16 / ES;
        const int zc = (col < BNZ) ? col : col - BNZ;
        const int gcol = (col < BNZ) ? n0 + zc : I + n0 + zc;
        b_kk[i] = kk;
        b_lds[i] = kk * C::B_STRIDE + cc * 16;
        b_col_off[i] = (n0 + zc < I) ? (int64_t)gcol * ES : -1;
    }
    const char* abase = (const char*)g.a;
    const char* wbase = (const char*)g.w13 + (int64_t)e * H * N * ES;

    i32x4 ra[C::A_PER_T], rb[C::B_PER_T];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            ra[i] = i32x4{0, 0, 0, 0};
            const int kb = k0 * ES + a_kc[i] * 16;
            if (a_off[i] >= 0 && kb < H * ES)
                ra[i] = *(const i32x4*)(abase + a_off[i] + kb);
        }
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i) {
            rb[i] = i32x4{0, 0, 0, 0};
            const int k = k0 + b_kk[i];
            if (b_col_off[i] >= 0 && k < H)
                rb[i] = *(const i32x4*)(wbase + (int64_t)k * N * ES + b_col_off[i]);
        }
    };
    auto lstore = [&](int stage) {
        char* As = smem + stage * C::STAGE_BYTES;
        char* Bs = As + BM * A_STRIDE;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i)
            if (tid + 256 * i < C::A_CHUNKS)
                *(i32x4*)(As + a_row[i] * A_STRIDE + a_kc[i] * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i)
            *(i32x4*)(Bs + b_lds[i]) = rb[i];
    };

    f32x4 acc[2][C::FM][C::FN];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[h][i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (H + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
        const char* As = smem + cur * C::STAGE_BYTES;
        const char* Bs = As + BM * A_STRIDE;
#pragma unroll
        for (int ks = 0; ks < BK / KM; ++ks) {
            typename Frag<DT>::A af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
                af[i] = load_a_frag<DT>(As + (wave_m * C::WM + i * 16) * A_STRIDE, ks, lane);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int col = h * BNZ + wave_n * C::WNZ + j * 16;
                    const typename Frag<DT>::B bf = load_b_frag<DT>(Bs, C::B_STRIDE, ks, col, lane);
#pragma unroll
                    for (int i = 0; i < C::FM; ++i)
                        acc[h][i][j] = mma<DT>(af[i], bf, acc[h][i][j]);
                }
        }
        if (kt + 1 < nk)
            lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: dequant, bias, SiLU(gate)*up -> LDS (float), then vector stores
    float* Zs = (float*)smem;
    const int g4 = lane >> 4, s16 = lane & 15;
    const float* w13s = (DT == MOE_FP8_E4M3FN) ? g.w13_scale + (int64_t)e * N : nullptr;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const int zc = wave_n * C::WNZ + j * 16 + s16;
        const int n = n0 + zc;
        float bg = 0.0f, bu = 0.0f, sg = 1.0f, su = 1.0f;
        if (n < I) {
            if (g.b13) {
                bg = load_bias(g.b13, g.bias_dt, (int64_t)e * N + n);
                bu = load_bias(g.b13, g.bias_dt, (int64_t)e * N + I + n);
            }
            if constexpr (DT == MOE_FP8_E4M3FN) {
                sg = w13s[n];
                su = w13s[I + n];
            }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wave_m * C::WM + i * 16 + g4 * 4 + r;
                float hg = acc[0][i][j][r], hu = acc[1][i][j][r];
                if constexpr (DT == MOE_FP8_E4M3FN) {
                    const float sa = a_rowscale[row];
                    hg = hg * sa * sg;
                    hu = hu * sa * su;
                }
                Zs[row * C::Z_STRIDE + zc] = silu_mul(hg + bg, hu + bu);
            }
    }
    __syncthreads();

    if constexpr (DT == MOE_FP8_E4M3FN) {
        // requantise per (row, 128 columns): 8 threads per row, 16 columns each
        static_assert(BNZ == 128, "fp8 z groups are 128 columns");
        const int ngrp = I / 128;
        for (int r0 = 0; r0 < BM; r0 += 32) {
            const int row = r0 + tid / 8, c0 = (tid % 8) * 16;
            float v[16], amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                v[c] = Zs[row * C::Z_STRIDE + c0 + c];
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
            const int64_t p = p0 + row;
            *(i32x4*)((uint8_t*)g.z + p * I + n0 + c0) =
                i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            if ((tid % 8) == 0)
                g.z_scale[p * ngrp + n0 / 128] = sc;
        }
    } else {
        constexpr int VE = 16 / ES;                 // z elements per 16-B store
        constexpr int CPR = BNZ / VE;
        for (int q = tid; q < BM * CPR; q += 256) {
            const int row = q / CPR, c0 = (q % CPR) * VE;
            if (n0 + c0 >= I)
                continue;
            const int64_t p = p0 + row;
            const float* src = Zs + row * C::Z_STRIDE + c0;
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

template <int DT, int BM, int BNZ, int WAVES_M>
__global__ void __launch_bounds__(256) k_gemm1(Gemm1Args g)
{
    __shared__ __attribute__((aligned(16))) char smem[G1Cfg<DT, BM, BNZ, WAVES_M>::LDS_BYTES];
    for_each_tile(g.npp, g.expert_ids, g.offsets, BM, g.n_tiles, [&](int mblk, int ntile) {
        gemm1_tile<DT, BM, BNZ, WAVES_M>(g, smem, mblk, ntile);
        __syncthreads();   // the next tile's prologue reuses the LDS
    });
}

// ---------------------------------------------------------------- GEMM2
template <int DT, int BM, int BN, int WAVES_M>
struct G2Cfg {
    static constexpr int ES = GT<DT>::ES, BK = GT<DT>::BK, KM = GT<DT>::KM;
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int B_STRIDE = BN * ES + 16;
    static constexpr int A_CHUNKS = BM * 8;
    static constexpr int B_CPR = BN * ES / 16;
    static constexpr int B_CHUNKS = BK * B_CPR;
    static constexpr int A_PER_T = (A_CHUNKS + 255) / 256;
    static constexpr int B_PER_T = B_CHUNKS / 256;
    static constexpr int STAGE_BYTES = BM * A_STRIDE + BK * B_STRIDE + BM * 4;
    static constexpr int PIPE_BYTES = 2 * STAGE_BYTES;
    static constexpr int O_STRIDE = BN + 4;
    static constexpr int EPI_BYTES = BM * O_STRIDE * 4;
    static constexpr int LDS_BYTES = PIPE_BYTES > EPI_BYTES ? PIPE_BYTES : EPI_BYTES;
    static_assert(B_CHUNKS % 256 == 0, "B tile must split evenly over 256 threads");
    static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA tile");
};

template <int DT, int BM, int BN, int WAVES_M>
__device__ __forceinline__ void gemm2_tile(const Gemm2Args& g, char* smem, int mblk, int ntile)
{
    typedef G2Cfg<DT, BM, BN, WAVES_M> C;
    constexpr int ES = C::ES, BK = C::BK, KM = C::KM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / C::WAVES_N, wave_n = wave % C::WAVES_N;
    const int e = g.expert_ids[mblk];
    const int H = g.H, I = g.I;
    const int c0 = ntile * BN;
    const int64_t p0 = (int64_t)mblk * BM;
    const int ngrp = I / 128;

    int a_kc[C::A_PER_T], a_row[C::A_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        const int q = tid + 256 * i;
        a_row[i] = q / 8;
        a_kc[i] = q % 8;
    }
    int64_t b_col_off[C::B_PER_T];
    int b_kk[C::B_PER_T], b_lds[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int kk = q / C::B_CPR, cc = q % C::B_CPR;
        const int col = c0 + cc * 16 / ES;
        b_kk[i] = kk;
        b_lds[i] = kk * C::B_STRIDE + cc * 16;
        b_col_off[i] = (col < H) ? (int64_t)col * ES : -1;
    }
    const char* zbase = (const char*)g.z + p0 * I * ES;
    const char* wbase = (const char*)g.w2 + (int64_t)e * I * H * ES;

    i32x4 ra[C::A_PER_T], rb[C::B_PER_T];
    float rs = 0.0f;
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            ra[i] = i32x4{0, 0, 0, 0};
            const int kb = k0 * ES + a_kc[i] * 16;
            if (tid + 256 * i < C::A_CHUNKS && kb < I * ES)
                ra[i] = *(const i32x4*)(zbase + (int64_t)a_row[i] * I * ES + kb);
        }
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i) {
            rb[i] = i32x4{0, 0, 0, 0};
            const int k = k0 + b_kk[i];
            if (b_col_off[i] >= 0 && k < I)
                rb[i] = *(const i32x4*)(wbase + (int64_t)k * H * ES + b_col_off[i]);
        }
        if constexpr (DT == MOE_FP8_E4M3FN) {
            if (tid < BM)
                rs = g.z_scale[(p0 + tid) * ngrp + kt];
        }
    };
    auto lstore = [&](int stage) {
        char* As = smem + stage * C::STAGE_BYTES;
        char* Bs = As + BM * A_STRIDE;
        float* Ss = (float*)(Bs + BK * C::B_STRIDE);
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i)
            if (tid + 256 * i < C::A_CHUNKS)
                *(i32x4*)(As + a_row[i] * A_STRIDE + a_kc[i] * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i)
            *(i32x4*)(Bs + b_lds[i]) = rb[i];
        if constexpr (DT == MOE_FP8_E4M3FN) {
            if (tid < BM)
                Ss[tid] = rs;
        }
    };

    f32x4 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nk = (I + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
        const char* As = smem + cur * C::STAGE_BYTES;
        const char* Bs = As + BM * A_STRIDE;
        const float* Ss = (const float*)(Bs + BK * C::B_STRIDE);
#pragma unroll
        for (int ks = 0; ks < BK / KM; ++ks) {
            typename Frag<DT>::A af[C::FM];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
                af[i] = load_a_frag<DT>(As + (wave_m * C::WM + i * 16) * A_STRIDE, ks, lane);
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const typename Frag<DT>::B bf =
                    load_b_frag<DT>(Bs, C::B_STRIDE, ks, wave_n * C::WN + j * 16, lane);
#pragma unroll
                for (int i = 0; i < C::FM; ++i) {
                    if constexpr (DT == MOE_FP8_E4M3FN) {
                        // one MFMA spans exactly one 128-wide scale group of z
                        const f32x4 t = mma<DT>(af[i], bf, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                        const f32x4 sz =
                            *(const f32x4*)(Ss + wave_m * C::WM + i * 16 + (lane >> 4) * 4);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[i][j][r] += t[r] * sz[r];
                    } else {
                        acc[i][j] = mma<DT>(af[i], bf, acc[i][j]);
                    }
                }
            }
        }
        if (kt + 1 < nk)
            lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: per-channel dequant, bias -> LDS, then row stores
    float* Os = (float*)smem;
    const int g4 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
        const int cl = wave_n * C::WN + j * 16 + s16;
        const int c = c0 + cl;
        float bias = 0.0f, sw = 1.0f;
        if (c < H) {
            if (g.b2)
                bias = load_bias(g.b2, g.bias_dt, (int64_t)e * H + c);
            if constexpr (DT == MOE_FP8_E4M3FN)
                sw = g.w2_scale[(int64_t)e * H + c];
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wave_m * C::WM + i * 16 + g4 * 4 + r;
                Os[row * C::O_STRIDE + cl] = acc[i][j][r] * sw + bias;
            }
    }
    __syncthreads();

    constexpr int CPR = BN / 4;   // 4 floats per chunk
    for (int q = tid; q < BM * CPR; q += 256) {
        const int row = q / CPR, cl = (q % CPR) * 4;
        const int c = c0 + cl;
        if (c >= H)
            continue;
        const int64_t p = p0 + row;
        const int sid = g.sorted[p];
        if (sid >= g.sentinel)
            continue;
        const float* src = Os + row * C::O_STRIDE + cl;
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

template <int DT, int BM, int BN, int WAVES_M>
__global__ void __launch_bounds__(256) k_gemm2(Gemm2Args g)
{
    __shared__ __attribute__((aligned(16))) char smem[G2Cfg<DT, BM, BN, WAVES_M>::LDS_BYTES];
    for_each_tile(g.npp, g.expert_ids, g.offsets, BM, g.n_tiles, [&](int mblk, int ntile) {
        gemm2_tile<DT, BM, BN, WAVES_M>(g, smem, mblk, ntile);
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

template <int DT, int BM, int BNZ, int WAVES_M>
static hipError_t run_gemm1(const Gemm1Args& a, hipStream_t s)
{
    Gemm1Args g = a;
    g.n_tiles = (a.I + BNZ - 1) / BNZ;
    auto kern = k_gemm1<DT, BM, BNZ, WAVES_M>;
    static int cached = 0;
    const dim3 grid(persistent_grid(kern, (int64_t)g.max_blocks * g.n_tiles, cached)), block(256);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

template <int DT, int BM, int BN, int WAVES_M>
static hipError_t run_gemm2(const Gemm2Args& a, hipStream_t s)
{
    Gemm2Args g = a;
    g.n_tiles = (a.H + BN - 1) / BN;
    auto kern = k_gemm2<DT, BM, BN, WAVES_M>;
    static int cached = 0;
    const dim3 grid(persistent_grid(kern, (int64_t)g.max_blocks * g.n_tiles, cached)), block(256);
    hipLaunchKernelGGL(kern, grid, block, 0, s, g);
    return hipGetLastError();
}

hipError_t launch_gemm1(const Plan& P, const moe_args& A, hipStream_t s)
{
    Gemm1Args g{};
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
    g.sorted = P.sorted_ids;
    g.expert_ids = P.expert_ids;
    g.offsets = P.offsets;
    g.npp = P.npp;
    g.sentinel = (int)P.sentinel;
    g.w13 = A.w13;
    g.w13_scale = A.w13_scale;
    g.b13 = P.has_b13 ? A.w13_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    g.max_blocks = P.max_blocks;
    g.z = P.z;
    g.z_scale = P.z_scale;
    if (fp8)
        return run_gemm1<MOE_FP8_E4M3FN, 128, 128, 2>(g, s);   // block fixed at 128 rows
    if (P.wdt == MOE_F32) {
        switch (P.BM) {
        case 16: return run_gemm1<MOE_F32, 16, 64, 1>(g, s);
        case 32: return run_gemm1<MOE_F32, 32, 64, 2>(g, s);
        case 64: return run_gemm1<MOE_F32, 64, 64, 2>(g, s);
        default: return run_gemm1<MOE_F32, 128, 64, 2>(g, s);
        }
    }
    switch (P.BM) {
    case 16: return run_gemm1<MOE_BF16, 16, 64, 1>(g, s);
    case 32: return run_gemm1<MOE_BF16, 32, 64, 2>(g, s);
    case 64: return run_gemm1<MOE_BF16, 64, 64, 2>(g, s);
    default: return run_gemm1<MOE_BF16, 128, 64, 2>(g, s);
    }
}

hipError_t launch_gemm2(const Plan& P, const moe_args& A, hipStream_t s)
{
    Gemm2Args g{};
    g.z = P.z;
    g.z_scale = P.z_scale;
    g.sorted = P.sorted_ids;
    g.expert_ids = P.expert_ids;
    g.offsets = P.offsets;
    g.npp = P.npp;
    g.sentinel = (int)P.sentinel;
    g.w2 = A.w2;
    g.w2_scale = A.w2_scale;
    g.b2 = P.has_b2 ? A.w2_bias : nullptr;
    g.bias_dt = (P.act == MOE_F32) ? MOE_F32 : MOE_BF16;
    g.H = P.H;
    g.I = P.I;
    g.max_blocks = P.max_blocks;
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
        return run_gemm2<MOE_FP8_E4M3FN, 128, 128, 2>(g, s);
    if (P.wdt == MOE_F32) {
        switch (P.BM) {
        case 16: return run_gemm2<MOE_F32, 16, 64, 1>(g, s);
        case 32: return run_gemm2<MOE_F32, 32, 64, 2>(g, s);
        case 64: return run_gemm2<MOE_F32, 64, 64, 2>(g, s);
        default: return run_gemm2<MOE_F32, 128, 64, 2>(g, s);
        }
    }
    switch (P.BM) {
    case 16: return run_gemm2<MOE_BF16, 16, 128, 1>(g, s);
    case 32: return run_gemm2<MOE_BF16, 32, 128, 2>(g, s);
    case 64: return run_gemm2<MOE_BF16, 64, 128, 2>(g, s);
    default: return run_gemm2<MOE_BF16, 128, 128, 2>(g, s);
    }
}

}  // namespace moe
