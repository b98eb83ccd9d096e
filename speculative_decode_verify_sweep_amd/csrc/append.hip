// Paged KV append: write the W window tokens' K and V into their pool slots,
// the step right before a verify call reads them.
//
// "perf(dflash): widen the verify window past the compact graph's four-row
// limit", section What changed: the window's K/V rows are written into the
// paged cache (stale slots past a request's length are later overwritten and
// never read); "DFlash2 leaves the paged graph fast path ...", section Scope:
// one shared pool addressed by a batched block table and per-request lengths.
// Token i of request p sits at position L_p - W + i; its K row goes to slot
// pos % 16 of pool page block_table[p][pos / 16] and its V row to the same
// slot of the transposed (d-major) value page, or, for a bf16 pool laid out
// token-major, to row pos % 16 of the value page like K.  For e4m3 pools each (token,
// KV head) row gets scale = amax|x| / 448 (1 when the row is all zero) and
// codes = round-to-nearest-even of x / scale on the OCP e4m3fn grid, all in
// fp32 (IEEE division), so the codes are exactly reproducible.  For MXFP4
// pools (OCP Microscaling Formats v1.0 conversion, E2M1 elements and an E8M0
// scale per 32 elements of a row) each block gets X = floor(log2 amax) - 2,
// clamped to [-127, 127] (an all-zero block -127), stored as X + 127, and each
// element the E2M1 code nearest x / 2^X, ties to the even code, past 6
// saturating to 6, with the sign bit of x.  Two tokens share each byte of the
// transposed value page, so V nibbles are written with word atomics (clear,
// then set) and waves writing the two halves of a byte cannot race.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "plan_internal.h"

namespace {

struct AppendParams {
    const uint16_t* k_new;  // bf16 [P][W][Hkv][D]
    const uint16_t* v_new;
    uint8_t* k_pool;
    uint8_t* v_pool;
    float* k_scale;
    float* v_scale;
    const int32_t* bt;
    const int32_t* seq;
    int32_t P, W, Hkv, bt_stride, num_pages;
    int32_t v_tok;  // bf16 pools only: V pages token-major [16][D] like K
};

constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, uint32_t(b) << 16);
}

// A DPP move inside 16-lane rows (VALU, no LDS permute): 0xB1 and 0x4E swap
// lanes at distance 1 and 2 within each quad, 0x141 mirrors each 8-lane half,
// 0x140 each 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of N lanes (N = 2, 4, 8 or 16).  After the quad
// swaps a lane holds its quad's max; the half mirror pairs it with a lane of
// the other quad of its 8, the row mirror with one of the other half of its
// 16.  max is exact and ignores NaN in any order, so the tree's shape does not
// change the result.
template <int N>
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
    return x;
}

// Max over the wave: 16-lane rows by DPP, then rows and halves by the VALU
// lane swaps (a register swapped with itself leaves each lane its own value
// and its partner's).
__device__ __forceinline__ float wave_max(float x) {
    x = group_max<16>(x);
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// One wave per (p, i, kvh); lane l owns elements [E*l, E*l + E) of the row.
// E2M1 code of y (|y| < 8 after the block scaling): count the rounding
// boundaries passed.  A tie between codes c and c+1 goes to the even one, so
// the boundary above an even code is strict and the one above an odd code is
// not.  The sign bit is the sign of y (so of x), also when y rounds to 0.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float v = fabsf(y);
    const uint32_t c = uint32_t(v > 0.25f) + uint32_t(v >= 0.75f) + uint32_t(v > 1.25f) +
                       uint32_t(v >= 1.75f) + uint32_t(v > 2.5f) + uint32_t(v >= 3.5f) +
                       uint32_t(v > 5.0f);
    return c | ((__builtin_bit_cast(uint32_t, y) >> 31) << 3);
}

// Shared exponent X of an MX block with largest magnitude m: floor(log2 m) - 2
// (2 is E2M1's largest exponent), clamped to E8M0's range; -127 for m = 0.
__device__ __forceinline__ int mx_exponent(float m) {
    if (!(m > 0.f)) return -127;
    int e = 0;
    (void)frexpf(m, &e);  // m = f 2^e, f in [0.5, 1): floor(log2 m) = e - 1
    return min(max(e - 3, -127), 127);
}

template <int D, int KV>
__global__ __launch_bounds__(64) void append_kernel(AppendParams a) {
    constexpr bool FP8 = KV == SMALLW_KV_FP8_E4M3;
    constexpr bool FP4 = KV == SMALLW_KV_MXFP4;
    constexpr int E = D / 64;
    const int b = blockIdx.x;
    const int kvh = b % a.Hkv;
    const int i = (b / a.Hkv) % a.W;
    const int p = b / (a.Hkv * a.W);
    const int l = threadIdx.x;
    // the window row first: its address does not depend on the slot, so its
    // load overlaps the dependent length -> block-table -> slot lookup
    const int64_t row = ((int64_t(p) * a.W + i) * a.Hkv + kvh) * D + E * l;
    uint16_t kb[E], vb[E];  // raw bf16 bits, loaded once before any store
    float kx[E], vx[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kb[e] = a.k_new[row + e];
        vb[e] = a.v_new[row + e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kx[e] = bf16_to_f32(kb[e]);
        vx[e] = bf16_to_f32(vb[e]);
    }
    int L = a.seq[p];
    const int cap = a.bt_stride * SMALLW_PAGE_SIZE;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int pos = L - a.W + i;
    if (pos < 0) return;  // the request is shorter than the window: no slot
    int page = a.bt[int64_t(p) * a.bt_stride + (pos >> 4)];
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    const int slot = pos & 15;
    const int64_t ph = int64_t(page) * a.Hkv + kvh;  // page-head index
    if constexpr (FP4) {
        // lane l holds elements E l .. E l + E - 1; a 32-element block is 32/E lanes
        constexpr int BL = 32 / E;
        float km = 0.f, vm = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            km = fmaxf(km, fabsf(kx[e]));
            vm = fmaxf(vm, fabsf(vx[e]));
        }
        km = group_max<BL>(km);
        vm = group_max<BL>(vm);
        const int kX = mx_exponent(km), vX = mx_exponent(vm);
        uint32_t kc = 0;
        uint8_t* kp = a.k_pool + (ph * 16 + slot) * (D / 2) + (E * l) / 2;
#pragma unroll
        for (int e = 0; e < E; ++e) kc |= e2m1_code(ldexpf(kx[e], -kX)) << (4 * e);
#pragma unroll
        for (int e = 0; e < E / 2; ++e) kp[e] = uint8_t(kc >> (8 * e));
        // V^T byte (d, slot / 2), nibble slot & 1; as a word: word 2d + slot / 8,
        // bits 8 ((slot / 2) & 3) + 4 (slot & 1)
        uint32_t* vw = reinterpret_cast<uint32_t*>(a.v_pool + ph * D * 8);
        const int sh = 8 * ((slot >> 1) & 3) + 4 * (slot & 1);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = E * l + e;
            uint32_t* w = vw + 2 * d + (slot >> 3);
            atomicAnd(w, ~(0xFu << sh));
            atomicOr(w, e2m1_code(ldexpf(vx[e], -vX)) << sh);
        }
        if (l % BL == 0) {
            const int blk = (E * l) / 32;
            uint8_t* ks8 = reinterpret_cast<uint8_t*>(a.k_scale);
            uint8_t* vs8 = reinterpret_cast<uint8_t*>(a.v_scale);
            ks8[(ph * 16 + slot) * (D / 32) + blk] = uint8_t(kX + 127);
            vs8[(ph * (D / 32) + blk) * 16 + slot] = uint8_t(vX + 127);  // block-major
        }
    } else if constexpr (!FP8) {
        uint16_t* kp = reinterpret_cast<uint16_t*>(a.k_pool) + (ph * 16 + slot) * D + E * l;
        if (a.v_tok) {
            uint16_t* vp = reinterpret_cast<uint16_t*>(a.v_pool) + (ph * 16 + slot) * D + E * l;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kp[e] = kb[e];
                vp[e] = vb[e];
            }
        } else {
            uint16_t* vp = reinterpret_cast<uint16_t*>(a.v_pool) + ph * D * 16 + slot;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kp[e] = kb[e];
                vp[int64_t(E * l + e) * 16] = vb[e];
            }
        }
    } else {
        float km = 0.f, vm = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            km = fmaxf(km, fabsf(kx[e]));
            vm = fmaxf(vm, fabsf(vx[e]));
        }
        km = wave_max(km);
        vm = wave_max(vm);
        const float ks = km > 0.f ? km / kE4m3Max : 1.f;
        const float vs = vm > 0.f ? vm / kE4m3Max : 1.f;
        uint8_t* kp = a.k_pool + (ph * 16 + slot) * D + E * l;
        uint8_t* vp = a.v_pool + ph * D * 16 + slot;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float kq = fminf(fmaxf(kx[e] / ks, -kE4m3Max), kE4m3Max);
            const float vq = fminf(fmaxf(vx[e] / vs, -kE4m3Max), kE4m3Max);
            // v_cvt_pk_fp8_f32: round to nearest even onto the OCP e4m3fn grid
            const uint32_t kc = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(kq, kq, 0, false));
            const uint32_t vc = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(vq, vq, 0, false));
            kp[e] = uint8_t(kc & 0xFF);
            vp[int64_t(E * l + e) * 16] = uint8_t(vc & 0xFF);
        }
        if (l == 0) {
            a.k_scale[ph * 16 + slot] = ks;
            a.v_scale[ph * 16 + slot] = vs;
        }
    }
}

template <int D>
hipError_t launch_append(const smallw_plan* pl, const AppendParams& a, hipStream_t st) {
    const unsigned blocks = unsigned(int64_t(a.P) * a.W * a.Hkv);
    if (pl->prob.kv_dtype == SMALLW_KV_FP8_E4M3)
        hipLaunchKernelGGL((append_kernel<D, SMALLW_KV_FP8_E4M3>), dim3(blocks), dim3(64), 0, st, a);
    else if (pl->prob.kv_dtype == SMALLW_KV_MXFP4) {
        if constexpr (D != 64)  // the planner rejects MXFP4 at D = 64
            hipLaunchKernelGGL((append_kernel<D, SMALLW_KV_MXFP4>), dim3(blocks), dim3(64), 0, st, a);
    } else
        hipLaunchKernelGGL((append_kernel<D, SMALLW_KV_BF16>), dim3(blocks), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace

extern "C" int small_w_kv_append(const smallw_plan* pl, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 void* stream) {
    if (!pl || !k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens)
        return SMALLW_EINVAL;
    const bool scaled = pl->prob.kv_dtype != SMALLW_KV_BF16;
    if (scaled && (!k_scale || !v_scale)) return SMALLW_EINVAL;
    AppendParams a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k_pool = static_cast<uint8_t*>(k_pool);
    a.v_pool = static_cast<uint8_t*>(v_pool);
    a.k_scale = static_cast<float*>(k_scale);
    a.v_scale = static_cast<float*>(v_scale);
    a.bt = block_table;
    a.seq = seq_lens;
    a.P = pl->prob.num_reqs;
    a.W = pl->prob.window;
    a.Hkv = pl->prob.num_kv_heads;
    a.bt_stride = pl->prob.max_pages_per_req;
    a.num_pages = pl->prob.num_pages;
    a.v_tok = pl->prob.v_layout == SMALLW_V_TOKEN_MAJOR;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (pl->prob.head_dim) {
        case 64: e = launch_append<64>(pl, a, st); break;
        case 128: e = launch_append<128>(pl, a, st); break;
        case 256: e = launch_append<256>(pl, a, st); break;
        default: return SMALLW_EUNSUPPORTED;
    }
    if (e != hipSuccess) {
        smallw::set_device_error("append kernel launch", int(e));
        return SMALLW_EDEVICE;
    }
    return SMALLW_OK;
}
