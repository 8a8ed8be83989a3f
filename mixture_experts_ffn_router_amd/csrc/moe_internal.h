// Internal declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ------------------------------------------------------------------ vector types
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16;

// ------------------------------------------------------------------ scalar formats
__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bf16 (NaN stays NaN).
__device__ __forceinline__ u16 f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u16)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

// E4M3FN code -> float (exact).
__device__ __forceinline__ float fp8_to_f32(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7)
        return __uint_as_float(0x7fc00000u);
    v = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return s ? -v : v;
}

// float -> E4M3FN, round to nearest even, saturating at +-448.  Integer
// arithmetic on the float's bits, so the result does not depend on any
// hardware conversion mode.
__device__ __forceinline__ uint8_t f32_to_fp8(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)
        return 0x7f;                                    // NaN
    if (a >= 0x43e00000u)                               // |x| >= 448 (incl. inf)
        return (uint8_t)(sign | 0x7e);
    const int exp = (int)(a >> 23) - 127;               // unbiased exponent of |x|
    uint32_t code;
    if (exp < -6) {
        // subnormal range: value = m * 2^-9, m = round(|x| * 2^9)
        // |x| * 2^9 as a fixed-point number with 23+... fractional bits:
        // mantissa with hidden bit, shifted so that the unit is 2^-9.
        if (exp < -10)                                  // below half the smallest step
            return (uint8_t)sign;                       // |x| < 2^-10 rounds to 0
        const uint32_t mant = (a & 0x7fffffu) | 0x800000u;   // |x| = mant * 2^(exp-23)
        const int shift = 23 - 9 - exp;                 // mant >> shift = |x| * 2^9
        const uint32_t q = mant >> shift;
        const uint32_t rem = mant & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        code = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);   // may carry to 8 = 2^-6
    } else {
        // normal: keep 3 mantissa bits, round the dropped 20 bits to nearest even
        const uint32_t mant = a & 0x7fffffu;
        const uint32_t q = ((uint32_t)(exp + 7) << 3) | (mant >> 20);
        const uint32_t rem = mant & 0xfffffu;
        code = q + ((rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u);
        if (code > 0x7eu)
            code = 0x7eu;
    }
    return (uint8_t)(sign | code);
}

// Two floats -> E4M3FN codes (a in bits 0-7, b in bits 8-15) by the hardware
// conversion, which rounds to nearest even and equals f32_to_fp8 wherever
// |x| <= 464 (the midpoint between 448 and the next binade step).  Callers
// pass x / scale with scale = amax / 448, so |x| <= 448 up to one rounding.
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o, 64);
        v = (w > v) ? w : v;
    }
    return v;
}

// Reductions over aligned groups of LPT lanes; every lane of a group gets
// the same result.  Inside a row of 16 lanes the partners are reached with
// DPP (lane i reads lane i^1, i^2 (quad_perm), 7-i within its 8, 15-i within
// its 16), which costs a few cycles where a shuffle through the LDS crossbar
// costs about a hundred; rows are then combined from v_readlane values.
// Each step combines a lane's value with its partner's and the partner
// combines the same two values, so with a commutative op every lane of the
// group ends with identical bits.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_MIRROR8 = 0x141, DPP_MIRROR16 = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float xchg(float v)
{
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ float rdlane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
template <int LPT, typename T, typename Op>
__device__ __forceinline__ T grp_reduce(T v, Op op)
{
    static_assert(LPT == 8 || LPT == 16 || LPT == 32 || LPT == 64, "group width");
    v = op(v, xchg<DPP_XOR1>(v));
    v = op(v, xchg<DPP_XOR2>(v));
    v = op(v, xchg<DPP_MIRROR8>(v));
    if constexpr (LPT >= 16)
        v = op(v, xchg<DPP_MIRROR16>(v));
    if constexpr (LPT == 32) {
        const T a = op(rdlane(v, 0), rdlane(v, 16)), b = op(rdlane(v, 32), rdlane(v, 48));
        v = (threadIdx.x & 32) ? b : a;
    } else if constexpr (LPT == 64) {
        v = op(op(rdlane(v, 0), rdlane(v, 16)), op(rdlane(v, 32), rdlane(v, 48)));
    }
    return v;
}

template <int LPT>
__device__ __forceinline__ float grp_max(float v)
{
    return grp_reduce<LPT>(v, [](float a, float b) { return fmaxf(a, b); });
}

template <int LPT>
__device__ __forceinline__ float grp_sum(float v)
{
    return grp_reduce<LPT>(v, [](float a, float b) { return a + b; });
}

// ------------------------------------------------------------------ execution plan
// GEMM tile families; each fixes the rows per tile (chunk height).
enum {
    TILE_PREFILL = 0,      // LDS-DMA ring, 160 rows
    TILE_MID = 1,          // register-staged, 64 rows
    TILE_DECODE = 2,       // register-staged, 16 rows
    TILE_FP8 = 3,          // fp8 register-staged, 128 rows
    TILE_DECODE_DMA = 4,   // LDS-DMA ring, 32 rows
    TILE_MID_DMA = 5,      // LDS-DMA ring, 64 rows
    TILE_FP8_DMA = 6,      // fp8 LDS-DMA ring on packed fp8 weights, F8_ROWS rows
    TILE_PREFILL_BIG = 7   // LDS-DMA ring, 256 rows x 256 columns (compute-bound loads)
};
constexpr int ALIGN_BM = 16;                 // expert runs are padded to 16 rows
constexpr int F8_ROWS = 128;                 // rows per tile of the fp8 LDS-DMA GEMMs
inline int tile_rows(int cfg)
{
    switch (cfg) {
    case TILE_PREFILL: return 160;
    case TILE_MID: return 64;
    case TILE_FP8: return 128;
    case TILE_DECODE_DMA: return 32;
    case TILE_MID_DMA: return 64;
    case TILE_FP8_DMA: return F8_ROWS;
    case TILE_PREFILL_BIG: return 256;
    default: return 16;
    }
}

// Host-computed description of one call: problem, tile choice, device pointers.
struct Plan {
    int fmt, M, H, I, E, K, T;      // M: tokens of one pass, K = top_k, T = max_tokens
    int Er;                         // experts routed over (global experts of a shard, else E)
    const int32_t* emap;            // [Er] global -> local expert, -1: held elsewhere (or null)
    int w_on_input;                 // routing weight scales z (GEMM1) instead of o (reduce)
    int act, wdt, outdt, lgdt, routing;
    int renorm, G, kg, gmode;
    float rsf;
    int has_b13, has_b2, breduce;
    int wpacked;                    // weights in the packed block layout (bf16 / fp8)
    int blk;                        // fp8: block-wise scales (128 x 128 weight blocks,
                                    // activation scales per row and 128 columns)
    int wq;                         // WNA16 weight code bits (8 or 4), 0 otherwise
    int wq_gsh;                     // WNA16: log2(K rows per scale group / 32): 0, 1 or 2
    int BM;                         // align granularity: each expert run padded to BM rows
    int CH;                         // rows per GEMM tile (a multiple of BM)
    int cfg;                        // GEMM tile family (see moe_gemm.hip)
    int g1wc;                       // 160-row bf16 family: GEMM1 wave columns (2 | 4)
    int dev, cus;                   // device of the launch stream and its compute units
    int64_t rows_cap;               // upper bound of valid routed rows
    int64_t max_sorted;             // rows_cap + E * (BM - 1)
    int max_blocks;                 // max_sorted / BM
    int64_t sentinel;               // sorted-id value of padding rows
    // workspace
    int32_t* topk_ids;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;               // [E + 1] padded prefix (P_e)
    int32_t* sorted_ids;
    int32_t* expert_ids;
    int32_t* npp;
    int32_t* chunk_off;             // [E + 1] GEMM row-chunk prefix per expert
    int32_t* chunk_expert;          // [max_blocks] expert of each chunk
    int32_t* inv;                   // contiguous: [M*K] padded position of routed item r (-1: none)
    uint8_t* aq;
    float* aq_scale;
    void* z;
    float* z_scale;                 // fp8: [I/128][zs_ld], group-major
    int64_t zs_ld;
    float* o;
    float* o2;                      // GEMM2 split in K: the second half's partial outputs
    int g2split;                    // GEMM2 runs as two K halves (o + o2)
    int32_t* status;                // device status word (moe_device_status bits)
    int status_or;                  // 0: the align stage stores the word; 1: ORs into it
                                    // (later chunks of a chunked forward)
};

// Bounds-checked build (compiled with MOE_CHECKED into libmoe_checked.so):
// indices that kernels take from device data (the tile table, sorted ids, the
// reduce's row map) are checked against their buffers, and one outside is
// skipped and reported in the status word (MOE_DEV_BOUNDS) instead of being
// accessed.  The release build compiles the checks away: there these indices
// come from the library's own align and tile-list kernels.
#ifdef MOE_CHECKED
constexpr bool CHECKED = true;
#else
constexpr bool CHECKED = false;
#endif

#ifdef __HIPCC__
// v in [0, n); in the checked build a miss sets MOE_DEV_BOUNDS
__device__ __forceinline__ bool in_bounds(int64_t v, int64_t n, int32_t* status)
{
    if constexpr (!CHECKED) {
        return true;
    } else {
        if (v >= 0 && v < n)
            return true;
        if (status)
            atomicOr(status, (int32_t)MOE_DEV_BOUNDS);
        return false;
    }
}
#endif

// Row stride of the group-major fp8 z scales: every padded position plus one
// GEMM tile of rows, so a tile may read its rows' scales as one block.
inline int64_t zs_ld(int64_t max_sorted) { return max_sorted + 256; }

// WNA16 packed weight codes (moe_gemm.hip): bits 8 or 4
hipError_t launch_pack_weights_wq(int bits, int E, int H, int I, const void* w13, const void* w2,
                                  void* p13, void* p2, hipStream_t s);

// GPTQ / AWQ checkpoint codes -> plain WNA16 codes (moe_gemm.hip)
hipError_t launch_repack_wq(int format, int bits, int64_t E, int64_t K, int64_t N, int64_t ng,
                            const int32_t* qw, const int32_t* qz, int zero_adjust,
                            uint8_t* codes, uint8_t* zeros, hipStream_t s);

// fp8 packed weights (moe_gemm_fp8.hip)
hipError_t launch_pack_weights_fp8(int E, int H, int I, const void* w13, const void* w2,
                                   void* p13, void* p2, hipStream_t s);

// Host-side helpers shared by the workspace layout and the GEMM launchers.
// Expected number of GEMM row chunks: every active expert has at least one,
// and the routed rows fill at least rows / CH of them.
inline int64_t expected_chunks(int fmt, int64_t M, int K, int E, int T, int CH)
{
    const int64_t rows = (fmt == MOE_FMT_BATCHED) ? (int64_t)E * T : M * K;
    const int64_t active = rows < E ? rows : E;
    const int64_t fill = (rows + CH - 1) / CH;
    return active > fill ? active : fill;
}

// Devices whose attributes the library caches (device ordinals below this).
constexpr int MAX_DEVICES = 64;

// Device of a launch stream (the current device for the null stream).
int stream_device(hipStream_t s);

// Compute units of device `dev` (queried once per device, then cached).
int device_cus(int dev);

// GEMM2 of the 160-row bf16 family runs with 256-column tiles split in two K
// halves when whole tiles would not cover the CUs and K is long: the halves
// write separate float partials that the reduce kernel adds.
inline bool gemm2_k_split(int cfg, int fmt, int breduce, int64_t chunks, int H, int I, int cus)
{
    if (cfg != TILE_PREFILL || (fmt == MOE_FMT_BATCHED && !breduce))
        return false;
    return chunks * ((H + 255) / 256) < cus && I >= 1024;
}

// launchers (each returns hipGetLastError() of its launch)
hipError_t launch_router(const Plan& P, const void* logits, hipStream_t s);
hipError_t launch_align(const Plan& P, const int32_t* ids, hipStream_t s);
hipError_t launch_tilelist(const Plan& P, const int32_t* expert_num_tokens, hipStream_t s);
hipError_t launch_quant_rows(const Plan& P, const void* hidden, hipStream_t s);
// row_w: routing weight per routed item, applied to z in GEMM1's epilogue (or null)
hipError_t launch_gemm1(const Plan& P, const moe_args& A, const float* row_w, hipStream_t s);
hipError_t launch_gemm2(const Plan& P, const moe_args& A, hipStream_t s);
hipError_t launch_reduce(const Plan& P, const moe_args& A, const float* topk_w, hipStream_t s);
hipError_t launch_pack_weights(int E, int H, int I, const void* w13, const void* w2, void* p13,
                               void* p2, hipStream_t s);

}  // namespace moe
