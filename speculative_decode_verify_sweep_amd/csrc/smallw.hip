// Small-window paged attention for MI355X (gfx950): split-K sweep, log-sum-exp
// combine, page-trace export, and the C entry points that launch them.
//
// Method (see "ChunkedSmallT re-streams full KV per query chunk", section
// Finding): all W window rows of a request attend its visible keys; the key
// range is split across work units and the partial softmax results are merged
// by a reduce step.  Unlike the chunked route that page describes, one work
// unit holds ALL W*G query rows of its KV head, so every K/V byte of the
// visible context is streamed from HBM exactly once per call.
//
// Work unit u = (request p, KV head kvh, key split s), one 512-thread
// workgroup (8 wave64s).  The unit walks its pages two at a time ("chunks" of
// 32 tokens) through an NS-deep ring of LDS buffers that the eight waves fill
// with 16-byte global->LDS DMA loads, each load instruction moving 1 KiB of
// one page-head.  Rows are the N side of the MFMAs:
//   S^T[token][row]  = K[token][:] . Q[row][:]       (v_mfma_f32_16x16x32_bf16)
//   O^T[d][row]     += V^T[d][token] . P^T[token][row]
// In this orientation a lane's accumulator registers all belong to one query
// row, so the online-softmax max/sum and the rescale factor are per-lane
// scalars, and the S^T accumulator registers of two 16-token tiles are
// exactly the B operand of the PV MFMA (no shuffle through LDS).  That is the
// bf16 sweep; e4m3 and MXFP4 pools have sweeps of their own (sweep8_kernel,
// sweep4_kernel) with the same units, orientation and epilogue, 128-token
// steps, and the scores on the scaled 16x16x128 MFMA straight from the codes.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "plan_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s2_t __attribute__((ext_vector_type(2)));  // packed fp8 pair results
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kPage = SMALLW_PAGE_SIZE;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Page-table window staged in LDS (pool page ids of one work unit).
constexpr int kPtab = 512;
// Lazy rescale: the running max is only moved when a chunk's max exceeds it
// by more than this (base-2 units), so exp2(s - m) <= 2^8 stays well inside
// fp32/bf16 range; final normalisation by the same sum keeps the result exact.
constexpr float kRescaleSlack = 8.0f;
// s_waitcnt immediate for gfx9: vmcnt(0), expcnt/lgkmcnt untouched.  The
// compiler's wait-count pass understands this builtin, so after it no
// compiler-issued vector load is considered in flight.
constexpr int kWaitVmcnt0 = 0x0F70;

struct Params {
    const uint16_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const float* k_scale;
    const float* v_scale;
    const int32_t* bt;
    const int32_t* seq;
    uint16_t* out;
    float* lse;
    uint16_t* part_o;  // split partials: fp16, lane-native blocks, rows scaled by 2^-e
    float2* part_rec;  // per (unit, row): {base-2 lse, 2^e}, [unit group][row][split]
    int32_t P, W, Hq, Hkv, G, R, bt_stride, num_pages, causal;
    int32_t split_pages;  // > 0: row-exact splits at multiples of this many pages
    int32_t combine;      // 1: every row goes through partials and the combine
    int32_t window_left;  // > 0: sliding window of this many keys per row
    int32_t piece_align;  // row-exact first pieces start on multiples of this many pages
    float scale_log2;  // softmax scale * log2(e): scores are kept in base 2
    int32_t unit_off[SMALLW_MAX_REQS + 1];
};

struct Unit {
    int p, kvh, s, S, L;
    int pb, pe;  // logical page range [pb, pe)
};

// Work unit u -> (p, kvh, s) and its page range.  Shared by the sweep and the
// page-trace kernel so the trace shows exactly what the sweep addresses.
__device__ __forceinline__ Unit decode_unit(const Params& a, int u) {
    int lo = 0, hi = a.P;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.unit_off[mid] <= u) lo = mid;
        else hi = mid;
    }
    Unit r;
    r.p = lo;
    r.S = (a.unit_off[lo + 1] - a.unit_off[lo]) / a.Hkv;
    const int rem = u - a.unit_off[lo];
    r.kvh = rem / r.S;
    r.s = rem - r.kvh * r.S;
    int L = a.seq[lo];
    const int cap = a.bt_stride * kPage;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    r.L = L;
    const int64_t n = (L + kPage - 1) / kPage;
    // first page any row needs: row 0's window start (0 without a window)
    int64_t n_lo = 0;
    if (a.window_left > 0 && L > 0) {
        const int64_t k0 = (a.causal ? L - a.W : L - 1) - a.window_left + 1;
        n_lo = k0 > 0 ? k0 / kPage : 0;
    }
    if (a.split_pages > 0) {  // row-exact: absolute grid of pieces; the first one
        // starts at n_lo moved down to its grouping grid, the last ends at n
        const int64_t k = n_lo / a.split_pages + r.s;
        const int64_t b0 = k * a.split_pages;
        r.pb = int(min(r.s == 0 ? b0 + ((n_lo - b0) & ~int64_t(a.piece_align - 1)) : b0, n));
        r.pe = r.s + 1 == r.S ? int(n) : int(min((k + 1) * a.split_pages, n));
    } else {
        r.pb = int(n_lo + (int64_t(r.s) * (n - n_lo)) / r.S);
        r.pe = int(n_lo + (int64_t(r.s + 1) * (n - n_lo)) / r.S);
    }
    return r;
}

// Pool page holding logical page n of request p; clamped so a bad table
// entry can never address outside the pool.
__device__ __forceinline__ int phys_page(const Params& a, int p, int n) {
    int pg = a.bt[int64_t(p) * a.bt_stride + n];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    return pg;
}

// 16-byte global -> LDS DMA.  Lane l's 16 bytes land at lds_addr + 16*l.
// Issued through inline asm so the compiler does not guard every later LDS
// read with a full vmcnt(0) wait; completion is tracked by hand with vmcnt.
// The s_nop is the wait state an M0 write needs before an LDS DMA reads it.
// M0 is written inside the statement but not listed as clobbered (the
// compiler reserves it and ignores such a clobber); no compiled code of these
// kernels reads M0 apart from these statements, so no compiler value is lost.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gaddr), "s"(lds_addr)
                 : "memory");
}

// Split partials are written through L2 (sc1): the combine kernel reads them
// right after, and dirty lines left in the eight L2s would otherwise be written
// back in one burst when the sweep kernel ends.  Nothing in the sweep kernel
// reads them, so the stores need no wait; the kernel's end orders them.  A
// store wider than 8 bytes may still be reading its data registers after it
// issues, and the compiler does not see stores inside asm, so the s_nop keeps
// the next instruction from overwriting them too early.
__device__ __forceinline__ void store_wt(void* gaddr, uint2 v) {
    asm volatile("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" : : "v"(gaddr), "v"(v) : "memory");
}
__device__ __forceinline__ void store_wt(void* gaddr, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(gaddr), "v"(v) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) by the
// VALU lane swaps: swapping a register with itself across 16-lane rows (or
// 32-lane halves) leaves every lane its own value in one result and its
// partner's in the other, so a commutative max or sum of the pair is the
// butterfly step with no LDS permute on the path.
__device__ __forceinline__ float pair16(float x, bool take_max) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const float a = __uint_as_float(s[0]), b = __uint_as_float(s[1]);
    return take_max ? fmaxf(a, b) : a + b;
}

__device__ __forceinline__ float pair32(float x, bool take_max) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const float a = __uint_as_float(s[0]), b = __uint_as_float(s[1]);
    return take_max ? fmaxf(a, b) : a + b;
}

__device__ __forceinline__ float wave_max_groups(float x) { return pair32(pair16(x, true), true); }

__device__ __forceinline__ float wave_sum_groups(float x) {
    return pair32(pair16(x, false), false);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// ----------------------------------------------------------------------------
// Split-K sweep kernel for bf16 pools (e4m3 pools: sweep8_kernel, MXFP4
// pools: sweep4_kernel, below).  512 threads = 8 wave64s; wave w owns the
// 16-row MFMA tile w of the unit's W*G rows (W*G <= 128), and the waves share
// the DMA work.
//   D    head dim (64/128/256)
//   NS   LDS ring depth in chunks (2 pages each)
//   VT   V pages token-major ([16][D], like K) instead of d-major
// LDS chunk layout of a bf16 ring stage (bytes): [K page0 | K page1 | V^T page0
// | V^T page1], each a page-head of 16*D*2 bytes.
// K rows are 16-byte-chunk swizzled: token row tau stores global chunk c at
// slot c ^ h(tau), h(tau) = ((tau>>1)&12)|(tau&3) (masked to the row), so the
// 16 lanes of one MFMA operand read hit distinct banks.  A bf16 V^T page
// (rows d of 16 tokens, 32 bytes) is stored in 512-byte groups of 16 rows:
// tokens 0..7 of rows 16k..16k+15 at 512k + 16*(d&15), tokens 8..15 256 bytes
// later.  The two halves of a row then share a bank slot, so a lane's bank
// depends only on its row, as in a linear read, and each 1 KiB DMA instruction
// still reads 1 KiB of contiguous HBM.
// VT (bf16 pools laid out token-major, V pages [16][D] like K): V rows are
// swizzled like K, with hv(tau) = 2*((tau&3)|(((tau>>3)&1)<<2)) (masked to the
// row), and the PV operand comes from ds_read_b64_tr_b16 transpose reads: in
// each 16-lane group, lane 4q+e gets element e of the 8-byte piece lane 4j+q
// addresses (j = 0..3), so lanes 4j..4j+3 address tokens 8g+4*a2+j of four
// d-quads and one read returns four tokens of one d column per lane.
// ----------------------------------------------------------------------------
constexpr int kSweepWaves = 8;
constexpr int kSweepThreads = 64 * kSweepWaves;

__device__ __forceinline__ void dma4(const void* gaddr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gaddr), "s"(lds_addr)
                 : "memory");
}

// The value among p0..p3 that a per-lane index k in [0, 4) selects (selects,
// not an indexed array, which the compiler would put in private memory).
__device__ __forceinline__ int pick4(int k, int p0, int p1, int p2, int p3) {
    return k == 0 ? p0 : k == 1 ? p1 : k == 2 ? p2 : p3;
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 24]
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n) {
#define SMALLW_WAIT_CASE(k) case k: wait_vmcnt<k>(); break;
        SMALLW_WAIT_CASE(0) SMALLW_WAIT_CASE(1) SMALLW_WAIT_CASE(2) SMALLW_WAIT_CASE(3)
        SMALLW_WAIT_CASE(4) SMALLW_WAIT_CASE(5) SMALLW_WAIT_CASE(6) SMALLW_WAIT_CASE(7)
        SMALLW_WAIT_CASE(8) SMALLW_WAIT_CASE(9) SMALLW_WAIT_CASE(10) SMALLW_WAIT_CASE(11)
        SMALLW_WAIT_CASE(12) SMALLW_WAIT_CASE(13) SMALLW_WAIT_CASE(14) SMALLW_WAIT_CASE(15)
        SMALLW_WAIT_CASE(16) SMALLW_WAIT_CASE(17) SMALLW_WAIT_CASE(18) SMALLW_WAIT_CASE(19)
        SMALLW_WAIT_CASE(20) SMALLW_WAIT_CASE(21) SMALLW_WAIT_CASE(22) SMALLW_WAIT_CASE(23)
#undef SMALLW_WAIT_CASE
        default: wait_vmcnt<24>(); break;
    }
}

// The convert's scale operand for E8M0 byte K of the word s.  The convert reads
// only the exponent field (bits 23..30) of its fp32 scale operand (measured:
// the sign and mantissa bits change nothing, and 0 gives 2^-127, 0xFF NaN), so
// byte K shifted into that field is the scale 2^(e-127) exactly, whatever the
// neighbouring bytes put around it: one shift per scale.
template <int K>
__device__ __forceinline__ float e8m0_operand(uint32_t s) {
    if constexpr (K == 3) return __builtin_bit_cast(float, s >> 1);
    else return __builtin_bit_cast(float, s << (23 - 8 * K));
}
// Byte J of w (two E2M1 codes, the low nibble first) -> 2 bf16, each times the
// scale sc.  The pair is moved as a whole word: reading an element out of the
// convert's 2 x bf16 result can lose its upper half.
template <int J>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16(uint32_t w, float sc) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, J));
}

// Epilogue of a work unit, on a wave that owns row tile w: normalise the
// rows, then write the final bf16 output and LSE (an unsplit request) or the
// fp16 split partial and its {lse, scale} record.  acc holds O^T tiles: lane
// l = 16g + ln, tile dt, element i is row r = 16w + ln, d = 16dt + 4g + i.
template <int D>
__device__ __forceinline__ void finish_unit(const Params& a, const f32x4 (&acc)[D / 16],
                                            float m_run, float l_run, int u, const Unit& un,
                                            int w, int l, int g, int r, int qi, int T) {
    constexpr int DT = D / 16;
    const int p = un.p, kvh = un.kvh;
    const float lsum = wave_sum_groups(l_run);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? m_run + __log2f(lsum) : -INFINITY;  // base 2
    // largest |o| of the row (its four lanes), for the split partial's scale
    float mabs = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mabs = fmaxf(mabs, fabsf(acc[dt][i]));
    mabs = wave_max_groups(mabs) * inv;
    if (r >= a.R) return;
    const int h = kvh * a.G + (r - qi * a.G);
    if (un.S == 1 && !a.combine) {
        uint16_t* orow = a.out + ((int64_t(p) * a.W + qi) * a.Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 o = acc[dt] * inv;
            uint2 pk;
            pk.x = uint32_t(f32_to_bf16_bits(o[0])) | (uint32_t(f32_to_bf16_bits(o[1])) << 16);
            pk.y = uint32_t(f32_to_bf16_bits(o[2])) | (uint32_t(f32_to_bf16_bits(o[3])) << 16);
            *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = pk;
        }
        if (g == 0) a.lse[(int64_t(p) * a.W + qi) * a.Hq + h] = lse2 * kLn2;
    } else {
        // split partial in fp16, the row divided by 2^e (e the exponent of its
        // largest |o|, so every value lies in (-1, 1) and keeps 11 significant
        // bits relative to the row's largest); the combine multiplies 2^e back.
        // Stored lane-native: block (u, tile w, k) is 64 lanes x 8 halves, lane
        // l = 16g + ln holding d tiles 2k and 2k+1 of its row, so each store
        // instruction writes 1 KiB of contiguous memory.
        int e = 0;
        (void)frexpf(mabs, &e);
        e = min(max(e, -100), 127);
        const float c = ldexpf(inv, -e);
        uint16_t* ob = a.part_o + ((int64_t(u) * T + w) * (DT / 2)) * 512 + l * 8;
#pragma unroll
        for (int k = 0; k < DT / 2; ++k) {
            const f32x4 x0 = acc[2 * k] * c, x1 = acc[2 * k + 1] * c;
            uint16_t hb[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hb[i] = __builtin_bit_cast(uint16_t, (_Float16)x0[i]);
                hb[4 + i] = __builtin_bit_cast(uint16_t, (_Float16)x1[i]);
            }
            store_wt(ob + k * 512, u32x4{uint32_t(hb[0]) | (uint32_t(hb[1]) << 16),
                                         uint32_t(hb[2]) | (uint32_t(hb[3]) << 16),
                                         uint32_t(hb[4]) | (uint32_t(hb[5]) << 16),
                                         uint32_t(hb[6]) | (uint32_t(hb[7]) << 16)});
        }
        // the S records of one row are contiguous: [unit group][row][split]
        if (g == 0) {
            const float2 rec = {lse2, ldexpf(1.f, e)};
            store_wt(a.part_rec + int64_t(u - un.s) * a.R + int64_t(r) * un.S + un.s,
                     __builtin_bit_cast(uint2, rec));
        }
    }
}

template <int D, int NS, bool VT = false>
__global__ __launch_bounds__(kSweepThreads, 1) void sweep_kernel(Params a) {
    constexpr int KS = D / 32;                     // MFMA k-steps over the head dim
    constexpr int DT = D / 16;                     // 16-wide d tiles of the output
    constexpr int BF_PAGE = 32 * D;                // bf16 page-head of K (or V^T) in LDS
    constexpr int ST_PAGE = BF_PAGE;               // one ring region (a page-head)
    constexpr int ST_STAGE = 4 * ST_PAGE;
    constexpr int RING = NS * ST_STAGE;            // DMA ring
    constexpr int REG_INST = ST_PAGE / 1024;       // DMA instructions per region
    constexpr bool SPLIT = REG_INST >= 2;          // region shared by waves w, w+4
    constexpr int LPW = SPLIT ? REG_INST / 2 : 1;  // DMA instructions per issuing wave
    constexpr int CPR = D / 8;                     // 16-byte bf16 chunks per K token row
    constexpr int AHEAD = NS - 1;                  // chunks in flight ahead of the one computed
    static_assert(REG_INST >= 1 && NS >= 2, "config");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[RING];
    __shared__ int32_t ptab[kPtab];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int l = tid & 63;
    const int g = l >> 4;   // lane group: MFMA k-slot group
    const int ln = l & 15;  // MFMA row/column index within a 16-tile

    const Unit un = decode_unit(a, blockIdx.x);
    const int u = blockIdx.x;
    const int p = un.p, kvh = un.kvh, L = un.L;
    const int npages = un.pe - un.pb;
    const int nchunks = (npages + 1) >> 1;
    const int jend = min(L, un.pe * kPage);            // keys past this: not in the unit
    const int lim_lo = a.causal ? (L - a.W + 1) : L;  // first key some row may not see
    const int first_masked = min(jend, lim_lo);
    // sliding window: keys below L - window_left are outside some row's window
    const int win_hi = a.window_left > 0 ? L - a.window_left : INT_MIN;

    // ---- this wave's query rows (tile w)
    const int T = (a.R + 15) >> 4;
    const bool has_tile = w < T;
    const int r = 16 * w + ln;
    const int qi = r / a.G;
    const int hi_row = a.causal ? (L - a.W + qi) : (L - 1);  // this row's last key
    const int hi_tok = min(jend - 1, hi_row);
    const int lo_tok = a.window_left > 0 ? hi_row - a.window_left + 1 : INT_MIN;
    // Q fragments: KS bf16 k-steps
    bf16x8_t qf[KS];

    // ---- pool page ids of this unit, staged in LDS (window of kPtab pages)
    int tbase = 0;  // unit-relative page index of ptab[0]
    auto fill_ptab = [&](int base) {
        for (int k = tid; k < kPtab; k += kSweepThreads)
            if (base + k < npages) ptab[k] = phys_page(a, p, un.pb + base + k);
    };
    fill_ptab(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // ---- DMA work of this wave: part (w>>2) of region (w&3) of each chunk
    const int region = w & 3;
    const int region_pg = region & 1;
    const bool region_v = region >= 2;
    const bool issues_kv = SPLIT || w < 4;
    const int nload = issues_kv ? LPW : 0;  // DMA instructions per chunk
    const int ibase = SPLIT ? (w >> 2) * LPW : 0;
    uint32_t goff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int qc = 64 * (ibase + i) + l;  // 16-byte chunk index inside the page-head
        if (!region_v) {
            const int tr = qc / CPR, slot = qc % CPR;
            const int tau = 16 * region_pg + tr;
            const int hsw = (((tau >> 1) & 12) | (tau & 3)) & (CPR - 1);
            goff[i] = uint32_t(tr * (2 * D) + (slot ^ hsw) * 16);
        } else if constexpr (VT) {
            const int tr = qc / CPR, slot = qc % CPR;
            const int tau = 16 * region_pg + tr;
            const int hv = (2 * ((tau & 3) | (((tau >> 3) & 1) << 2))) & (CPR - 1);
            goff[i] = uint32_t(tr * (2 * D) + (slot ^ hv) * 16);
        } else {
            // LDS slot qc = 32*a + 16*h + r of its 1 KiB block holds half h of
            // row 16*(2*block + a) + r
            const int d = (qc & ~31) / 2 + (qc & 15), h = (qc >> 4) & 1;
            goff[i] = uint32_t(d * 32 + h * 16);
        }
    }
    const uint32_t smem_base = uint32_t(reinterpret_cast<uintptr_t>(smem));
    const uint8_t* const pool = region_v ? a.v : a.k;

    auto issue_chunk = [&](int c) {
        if (issues_kv) {
            int n = 2 * c + region_pg;
            if (n >= npages) n = 2 * c;  // absent second page: reload the first, masked later
            const int phys = __builtin_amdgcn_readfirstlane(ptab[n - tbase]);
            const uint8_t* base = pool + (int64_t(phys) * a.Hkv + kvh) * int64_t(ST_PAGE);
            const uint32_t lds =
                smem_base + uint32_t((c % NS) * ST_STAGE + region * ST_PAGE + ibase * 1024);
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                dma16(base + goff[i], __builtin_amdgcn_readfirstlane(lds + 1024u * i));
        }
    };

    // ---- prologue: start the ring, then load Q while the first chunks are in
    // flight (one memory round trip for both), and wait for all of it here so
    // that no compiler-visible vector load is pending inside the loop
    const int pro = min(AHEAD, nchunks);
    for (int c = 0; c < pro; ++c) issue_chunk(c);
    {
        const bool valid = has_tile && r < a.R;
        const int gq = r - qi * a.G;
        const uint16_t* qrow =
            a.q + ((int64_t(p) * a.W + (valid ? qi : 0)) * a.Hq + kvh * a.G + (valid ? gq : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            // k-step ks, lane group g: elements 32ks + 8g ..
            if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g);
            qf[ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---- LDS read addressing (per lane, constant over chunks), bf16 layout
    // K operand for QK tile t: M-row ln holds chunk token tau = 8*(ln>>2) + 4t + (ln&3),
    // so lane group g of the S^T accumulators covers chunk tokens 8g+4t+j and the PV
    // B operand of lane group g is chunk tokens 8g..8g+7 -- one 16-byte V^T read.
    uint32_t kaddr[2][4];
    {
        const int mh = (ln >> 2) & (KS - 1 < 3 ? KS - 1 : 3);
        const int ml = ln & 3;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tau = 8 * (ln >> 2) + 4 * t + (ln & 3);
            const int row_base = (tau >> 4) * BF_PAGE + (tau & 15) * (2 * D);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                kaddr[t][b] = uint32_t(row_base + 64 * ((b ^ mh) & (KS - 1)) + 16 * (g ^ ml));
        }
    }
    const uint32_t vaddr = uint32_t(2 * BF_PAGE + (g >> 1) * BF_PAGE + (g & 1) * 256 + ln * 16);
    // VT: the two transpose-read addresses of d tile 0 (tile dt: xor 32 dt);
    // read a2 covers tokens 8g + 4a2 .. 8g + 4a2 + 3 of the chunk
    uint32_t vtA[2] = {};
    if constexpr (VT) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
            const int tau = 8 * g + 4 * a2 + (ln >> 2);
            const int q = ln & 3;
            const int y = (tau & 3) | (((tau >> 3) & 1) << 2);
            vtA[a2] = uint32_t(2 * BF_PAGE + (tau >> 4) * BF_PAGE + (tau & 15) * (2 * D)) |
                      uint32_t((32 * y + 16 * (q >> 1) + 8 * (q & 1)) & (2 * D - 1));
        }
    }
    // one d tile of the PV operand (8 tokens x this lane's d column)
    typedef short v4s_t __attribute__((ext_vector_type(4)));
    auto vread = [&](const uint8_t* vst, int dt) -> u32x4 {
        if constexpr (VT) {
            const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t*)(vst + (vtA[0] ^ uint32_t(32 * dt))));
            const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t*)(vst + (vtA[1] ^ uint32_t(32 * dt))));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            return u32x4{l2.x, l2.y, h2.x, h2.y};
        } else {
            return *reinterpret_cast<const u32x4*>(vst + vaddr + 512 * dt);
        }
    };

    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    auto process = [&](int c, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const uint8_t* st = smem + (c % NS) * ST_STAGE;
        const uint8_t* vst = st;  // V^T operand rows
        const int j0 = (un.pb + 2 * c) * kPage;  // absolute position of chunk token 0
        // S^T = K . Q^T over the chunk's 32 tokens (two 16-token tiles), four
        // independent accumulation chains for MFMA pipelining.  All K operand
        // reads are issued before the first MFMA so LDS latency overlaps.
        f32x4 s4[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) s4[t][0] = s4[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            bf16x8_t kop[KS][2];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    kop[ks][t] =
                        *reinterpret_cast<const bf16x8_t*>(st + kaddr[t][ks & 3] + 256 * (ks >> 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    s4[t][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks][t], qf[ks],
                                                                              s4[t][ks & 1], 0, 0, 0);
        }
        // V^T operands do not depend on the softmax: at D = 256 issue their reads
        // now so their latency hides behind it (at smaller heads the registers
        // are worth more: D = 128 would drop to one workgroup per CU)
        constexpr bool VPRE = D == 256;
        u32x4 vraw[VPRE ? DT : 1];
        if constexpr (VPRE) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                vraw[dt] = vread(vst, dt);
            __builtin_amdgcn_sched_barrier(0);
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = e >> 2, j = e & 3;
            x[e] = s4[t][0][j] + s4[t][1][j];  // the softmax scale goes in the exponent
            if (TAIL) {
                const int j = j0 + 8 * g + e;
                x[e] = (j <= hi_tok && j >= lo_tok) ? x[e] : -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = wave_max_groups(mx) * a.scale_log2;  // base 2 (the scale is positive)
        // row-uniform: the four lanes of a row hold the same mx and m_run
        const bool grow = mx > m_run + kRescaleSlack;
        if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
            m_run = grow ? mx : m_run;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(x[e], a.scale_log2, -m_use));
        l_run += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        // tokens past the unit's keys may hold anything (even NaN): zero their
        // V^T elements
        const int vcnt = TAIL ? min(max(jend - (j0 + 8 * g), 0), 8) : 8;
        const bf16x8_t pf = bf16x8_t{(__bf16)pe[0], (__bf16)pe[1], (__bf16)pe[2], (__bf16)pe[3],
                                     (__bf16)pe[4], (__bf16)pe[5], (__bf16)pe[6], (__bf16)pe[7]};
        // O^T += V^T . P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x4 raw;
            if constexpr (VPRE) raw = vraw[dt];
            else raw = vread(vst, dt);
            if constexpr (TAIL) {
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2)
                    raw[k2] &= (2 * k2 + 1 < vcnt) ? 0xffffffffu : (2 * k2 < vcnt ? 0x0000ffffu : 0u);
            }
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, raw), pf,
                                                              acc[dt], 0, 0, 0);
        }
    };

    // ---- ring step for iteration c: wait for chunk c, then refill the slot
    // freed by chunk c-1 with chunk c+NS-1
    auto ring_step = [&](int c) {
        // chunks younger than c left in flight: all issued up to c+NS-2
        wait_vmcnt_dyn(min(NS - 2, nchunks - 1 - c) * nload);
        __syncthreads();
        const int cn = c + AHEAD;
        if (cn < nchunks) {
            if (2 * cn - tbase >= kPtab) {  // slide the page-table window (long units only)
                tbase = 2 * cn;
                fill_ptab(tbase);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                __syncthreads();
            }
            issue_chunk(cn);
        }
    };
    // Chunks that need no mask come first: the masked ones (keys past the
    // unit's end, or past some row's causal limit) are always a suffix.
    int c_tail = nchunks;
    while (c_tail > 0 && (un.pb + 2 * (c_tail - 1)) * kPage + 32 > first_masked) --c_tail;
    // with a sliding window the chunks holding keys below some row's window
    // start are a prefix, also run masked
    int c_head = 0;
    while (c_head < c_tail && (un.pb + 2 * c_head) * kPage < win_hi) ++c_head;

    // one iteration: the ring step, then the row-tile waves' scores, softmax
    // and PV of chunk c
    auto step = [&](int c, auto tail_tag) {
        ring_step(c);
        if (has_tile) process(c, tail_tag);
    };
    int c = 0;
    for (; c < c_head; ++c) step(c, std::true_type{});
    for (; c < c_tail; ++c) step(c, std::false_type{});
    for (; c < nchunks; ++c) step(c, std::true_type{});

    // ---- epilogue: normalise, write the final output or the split partial
    if (!has_tile) return;
    finish_unit<D>(a, acc, m_run, l_run, u, un, w, l, g, r, qi, T);
}

// Q rows of a work unit as the B operand of the scaled fp8 MFMA: loaded in the
// operand's contraction order, then split per 32-element block into two e4m3
// parts q = hi 2^X + lo 2^(X-4), X = floor(log2 amax) - 7, which hold a bf16 q
// exactly (4 + 4 significant bits).  Block b of a 128-deep k-step is run b >> 1
// of lane groups 2(b & 1), 2(b & 1) + 1; lane group g supplies the scale of
// block g (byte k of shi / slo for k-step k).  Shared by the e4m3 and MXFP4
// sweeps; it waits for all of this wave's loads.
template <int D>
__device__ __forceinline__ void load_split_q(const Params& a, int p, int kvh, bool valid, int qi,
                                             int gq, int g, int ln,
                                             i32x8 (&qhi)[D < 128 ? 1 : D / 128],
                                             i32x8 (&qlo)[D < 128 ? 1 : D / 128], uint32_t& shi,
                                             uint32_t& slo) {
    constexpr int KS4 = D < 128 ? 1 : D / 128;
    bf16x8_t qf[4 * KS4];
    {
        const uint16_t* qrow =
            a.q + ((int64_t(p) * a.W + (valid ? qi : 0)) * a.Hq + kvh * a.G + (valid ? gq : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < 4 * KS4; ++ks) {
            // qf[4k + 2r + h]: contraction positions 128k + 64r + 16g + 8h .. (zero past D)
            const int d0 = 128 * (ks >> 2) + 64 * ((ks >> 1) & 1) + 16 * g + 8 * (ks & 1);
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (valid && d0 < D) raw = *reinterpret_cast<const u32x4*>(qrow + d0);
            qf[ks] = __builtin_bit_cast(bf16x8_t, raw);
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

#pragma unroll
    for (int k = 0; k < KS4; ++k) {
        int X[2];
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
            float m = 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    m = fmaxf(m, fabsf(float(qf[4 * k + 2 * r4 + hh][e])));
            m = pair16(m, true);
            int ex = 0;
            (void)frexpf(m, &ex);
            X[r4] = m > 0.f ? min(max(ex - 8, -123), 127) : 0;
        }
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 8; e += 4) {
                    float x4[4], y4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        x4[i] = ldexpf(float(qf[4 * k + 2 * r4 + hh][e + i]), -X[r4]);
                    int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x4[0], x4[1], 0, false);
                    hw = __builtin_amdgcn_cvt_pk_fp8_f32(x4[2], x4[3], hw, true);
                    const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
                    const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
                    y4[0] = (x4[0] - h01[0]) * 16.f;
                    y4[1] = (x4[1] - h01[1]) * 16.f;
                    y4[2] = (x4[2] - h23[0]) * 16.f;
                    y4[3] = (x4[3] - h23[1]) * 16.f;
                    int lw = __builtin_amdgcn_cvt_pk_fp8_f32(y4[0], y4[1], 0, false);
                    lw = __builtin_amdgcn_cvt_pk_fp8_f32(y4[2], y4[3], lw, true);
                    const int wi = 4 * r4 + 2 * hh + e / 4;  // byte 16 r4 + 8 hh + e
                    qhi[k][wi] = hw;
                    qlo[k][wi] = lw;
                }
        const int src = 16 * 2 * (g & 1) + ln;
        const int x0 = __shfl(X[0], src), x1 = __shfl(X[1], src);
        const int xs = (g >> 1) ? x1 : x0;
        shi |= uint32_t(xs + 127) << (8 * k);
        slo |= uint32_t(xs - 4 + 127) << (8 * k);
    }

}

// ----------------------------------------------------------------------------
// e4m3 sweep (fp8 KV).  The scores run on the scaled fp8 MFMA as in the other
// low-precision path, and so does the PV product: the e4m3 V^T codes go from
// the LDS ring straight into the MFMA's A operand (no decode, no staging), and
// the weights are split into two e4m3 parts per 32-token block and row,
//   p = hi 2^X + lo 2^(X-4),  X = floor(log2 max_block p) - 7,
// which holds every weight to about 2^-8 of itself (the unit roundoff of the
// bf16 weights of the other paths).  Chunks are 64 tokens (4 pages); two
// chunks (128 tokens, the MFMA's depth) make one PV step.
//
// K and V^T each stream through a 4-chunk LDS ring (two PV steps): the next
// step's chunks load while the current one computes, issued by the waves
// that hold no row tile (by all eight when fewer than two are free).
//
// Token layout.  Score tile tt (16 tokens) of a chunk puts page g of the
// chunk in MFMA rows 4g..4g+3 at tokens 4tt..4tt+3, so lane group g ends up
// holding all 16 scores of page g of the chunk for its row.  That is exactly
// the PV B operand: k = 16g + e (run 0) is page g, token e of the step's first
// chunk, k = 64 + 16g + e (run 1) page g, token e of its second.  The A
// operand (V^T) of lane (g, d-row ln) is then row d of page g of each chunk:
// two 16-byte LDS reads, the d-major page layout as stored in HBM.
//
// The running max only moves to whole numbers, so every rescale is an exact
// power of two; the running sum and the output accumulator are rescaled once
// per step, before that step's PV MFMAs.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kSweepThreads, 1) void sweep8_kernel(Params a) {
    constexpr int KS4 = D < 128 ? 1 : D / 128;  // 128-deep k-steps of the scores
    constexpr int DT = D / 16;                  // 16-wide d tiles of the output
    constexpr int PGB = 16 * D;                 // one page-head of codes, K or V^T
    constexpr int CHB = 4 * PGB;                // one 64-token chunk of K or V^T
    constexpr int NK = 4, NV = 4;               // ring slots (chunks)
    constexpr int IPP = PGB / 1024;             // 1 KiB DMA instructions per page
    constexpr int KI = 4 * IPP;                 // ... per chunk, for K and for V^T
    constexpr int SPR = D / 16;                 // 16-byte slots per K row
    constexpr int DH = DT / 2;                  // d tiles per half PV step
    static_assert(IPP >= 1 && KI <= 16 && DT % 2 == 0, "config");

    __shared__ __attribute__((aligned(1024))) uint8_t kring[NK * CHB];
    __shared__ __attribute__((aligned(1024))) uint8_t vring[NV * CHB];
    // per K slot: K scales [page][token] (64), then V scales (64)
    __shared__ __attribute__((aligned(16))) float scl[NK][128];
    __shared__ int32_t ptab[kPtab];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int g = l >> 4;
    const int ln = l & 15;

    const Unit un = decode_unit(a, blockIdx.x);
    const int u = blockIdx.x;
    const int p = un.p, kvh = un.kvh, L = un.L;
    const int npages = un.pe - un.pb;
    const int nchunks = (npages + 3) >> 2;
    const int jend = min(L, un.pe * kPage);
    const int lim_lo = a.causal ? (L - a.W + 1) : L;
    const int first_masked = min(jend, lim_lo);
    const int win_hi = a.window_left > 0 ? L - a.window_left : INT_MIN;

    const int T = (a.R + 15) >> 4;
    const bool has_tile = w < T;
    const int r = 16 * w + ln;
    const int qi = r / a.G;
    const int hi_row = a.causal ? (L - a.W + qi) : (L - 1);
    const int hi_tok = min(jend - 1, hi_row);
    const int lo_tok = a.window_left > 0 ? hi_row - a.window_left + 1 : INT_MIN;

    int tbase = 0;
    auto fill_ptab = [&](int base) {
        for (int k = tid; k < kPtab; k += kSweepThreads)
            if (base + k < npages) ptab[k] = phys_page(a, p, un.pb + base + k);
    };
    fill_ptab(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // ---- DMA work.  The eight pages of a PV step (two chunks of four) are
    // dealt to the issuing waves: the waves without a row tile when there are
    // at least two of them, else all eight.  Issuer e takes pages e, e + NF,
    // ... of the step; for each it reads the pool page id once and moves the
    // page's K and V^T codes, IPP 1 KiB instructions each.  K rows are
    // swizzled so that a lane's 16-byte slot sigma of row (page, token) sits
    // at sigma ^ h, h = (page << 2 | token & 3) masked to the row: the 8 and 16
    // lanes of one operand read then hit distinct banks.  V^T is a raw copy.
    // A chunk's K scales go to issuer 2q mod NF and its V scales to issuer
    // 2q + 1 mod NF (chunk q of the step; lane l: page l >> 4, token l & 15).
    // Measured: a row-tile wave that also issued loads spent about a fifth of
    // each step on them, one page-id read and wait per instruction.
    const int n_free = 8 - T;
    const int NF = n_free >= 2 ? n_free : 8;
    const int e_iss = n_free >= 2 ? w - T : w;  // issuer index; negative: issues nothing
    const uint32_t kr_base = uint32_t(reinterpret_cast<uintptr_t>(kring));
    const uint32_t vr_base = uint32_t(reinterpret_cast<uintptr_t>(vring));
    const uint32_t scl_base = uint32_t(reinterpret_cast<uintptr_t>(&scl[0][0]));
    const float* kscale = a.k_scale;
    const float* vscale = a.v_scale;
    asm volatile("" : "+s"(kscale), "+s"(vscale));

    // chunk t, which is chunk q (0 or 1) of its PV step; pages past the
    // unit's end are replaced by the chunk's first page (always present),
    // their tokens are masked
    auto issue_chunk = [&](int t, int q) {
        if (e_iss < 0) return;
        const uint32_t kslot = uint32_t((t % NK) * CHB), vslot = uint32_t((t % NV) * CHB);
#pragma unroll 1
        for (int p8 = e_iss; p8 < 4 * q + 4; p8 += NF) {
            const int pg = p8 - 4 * q;
            if (pg < 0) continue;
            int n = 4 * t + pg;
            if (n >= npages) n = 4 * t;
            const int phys = __builtin_amdgcn_readfirstlane(ptab[n - tbase]);
            const uint8_t* kp = a.k + (int64_t(phys) * a.Hkv + kvh) * PGB;
            const uint8_t* vp = a.v + (int64_t(phys) * a.Hkv + kvh) * PGB;
            // the lane offsets are recomputed per page from an opaque copy of the
            // lane index: hoisted out of the loop they cost registers the row
            // tiles need (the issuing waves have time to spare)
            int lane = l;
            asm volatile("" : "+v"(lane));
#pragma unroll
            for (int m = 0; m < IPP; ++m) {
                const int i = pg * IPP + m;
                const int qc = 64 * m + lane;
                const int tr = qc / SPR, ps = qc % SPR;
                const int h = ((pg << 2) | (tr & 3)) & (SPR - 1);
                dma16(kp + tr * D + 16 * (ps ^ h),
                      __builtin_amdgcn_readfirstlane(kr_base + kslot + 1024u * uint32_t(i)));
                dma16(vp + 16 * qc,
                      __builtin_amdgcn_readfirstlane(vr_base + vslot + 1024u * uint32_t(i)));
            }
        }
        const bool ks_mine = e_iss == (2 * q) % NF, vs_mine = e_iss == (2 * q + 1) % NF;
        if (ks_mine || vs_mine) {
            int n = 4 * t + (l >> 4);
            if (n >= npages) n = 4 * t;
            const int64_t off = (int64_t(ptab[n - tbase]) * a.Hkv + kvh) * kPage + (l & 15);
            const uint32_t dst = scl_base + uint32_t((t % NK) * 128 * 4);
            if (ks_mine) dma4(kscale + off, __builtin_amdgcn_readfirstlane(dst));
            if (vs_mine) dma4(vscale + off, __builtin_amdgcn_readfirstlane(dst + 256u));
        }
    };

    // ---- prologue: step 0's K and V^T, then Q (one round trip for all of it).
    // Each step then issues the next step's loads right after its barrier, so
    // one step is in flight while the current one computes.
    for (int t = 0; t < min(2, nchunks); ++t) issue_chunk(t, t);
    // Q as two e4m3 parts (its loads overlap the DMA issued above)
    i32x8 qhi[KS4], qlo[KS4];
    uint32_t shi = 0, slo = 0;
    load_split_q<D>(a, p, kvh, has_tile && r < a.R, qi, r - qi * a.G, g, ln, qhi, qlo, shi, slo);

    // K operand reads: lane row (page ln >> 2, token 4 tt + (ln & 3)), run r of
    // k-step k = 16-byte slot 8k + 4r + g of the row, stored at slot ^ (ln & (SPR-1))
    uint32_t k8a[KS4][2];
#pragma unroll
    for (int k = 0; k < KS4; ++k)
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
            const int slot = (8 * k + 4 * r4 + g) & (SPR - 1);
            k8a[k][r4] = uint32_t((ln >> 2) * PGB + (ln & 3) * D + 16 * (slot ^ (ln & (SPR - 1))));
        }
    // V^T operand reads: page g of a chunk, row d = 16 dt + ln
    const uint32_t v8a = uint32_t(g * PGB + 16 * ln);

    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    float m_acc = -INFINITY;  // the running max acc is expressed against

    // ---- scores of chunk t on the scaled MFMA: s4[tt][i] = page g, token 4tt + i
    auto qk = [&](int t, f32x4 (&s4)[4]) {
        const uint8_t* ks = kring + (t % NK) * CHB;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) s4[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two tiles and one k-step at a time: their K operands, then the hi and
        // lo MFMAs of both tiles
#pragma unroll
        for (int t2 = 0; t2 < 4; t2 += 2)
#pragma unroll
            for (int k = 0; k < KS4; ++k) {
                i32x8 ka[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int off = 4 * (t2 + tt) * D;
                    const u32x4 r0 = *reinterpret_cast<const u32x4*>(ks + k8a[k][0] + off);
                    u32x4 r1 = {0u, 0u, 0u, 0u};
                    if constexpr (D >= 128)
                        r1 = *reinterpret_cast<const u32x4*>(ks + k8a[k][1] + off);
                    ka[tt] = i32x8{int(r0[0]), int(r0[1]), int(r0[2]), int(r0[3]),
                                   int(r1[0]), int(r1[1]), int(r1[2]), int(r1[3])};
                }
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    s4[t2 + tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        ka[tt], qhi[k], s4[t2 + tt], 0, 0, 0, 0x7F7F7F7F, 0, int(shi >> (8 * k)));
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    s4[t2 + tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        ka[tt], qlo[k], s4[t2 + tt], 0, 0, 0, 0x7F7F7F7F, 0, int(slo >> (8 * k)));
            }
    };

    // ---- softmax of one PV step (branch-free): the scores of its two chunks
    // share one running max; then each chunk's weights (row ln, page g, tokens
    // 0..15, times the V scales) are split into e4m3 parts of their 32-token
    // block, p = hi 2^X + lo 2^(X-4): chunk A's into dwords 0..3 of the MFMA's
    // B operands with exponent XA, chunk B's into dwords 4..7 with XB.  A
    // masked step may lack chunk B (hasB false): its scores are masked out.
    auto softmax_step = [&](int tA, const f32x4 (&sa)[4], const f32x4 (&sb)[4], bool hasB,
                            i32x8& hi, i32x8& lo, int& XA, int& XB, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const f32x4* spa = reinterpret_cast<const f32x4*>(&scl[tA % NK][0]);
        const f32x4* spb = reinterpret_cast<const f32x4*>(&scl[(tA + 1) % NK][0]);
        const int j0 = (un.pb + 4 * tA + g) * kPage;  // absolute position of token 0 of page g
        // x[e]: chunk A, page g, token e; x[16 + e]: chunk B (64 tokens later).
        // K scales only: the softmax scale goes in the exponent's FMA
        float x[32];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 ka = spa[4 * g + tt], kb = spb[4 * g + tt];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * tt + i;
                x[e] = sa[tt][i] * ka[i];
                x[16 + e] = sb[tt][i] * kb[i];
                if (TAIL) {
                    x[e] = (j0 + e <= hi_tok && j0 + e >= lo_tok) ? x[e] : -INFINITY;
                    x[16 + e] = (hasB && j0 + 64 + e <= hi_tok && j0 + 64 + e >= lo_tok)
                                    ? x[16 + e] : -INFINITY;
                }
            }
        }
        float mx = fmaxf(x[0], x[16]);
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(x[e], x[16 + e]));
        mx = wave_max_groups(mx) * a.scale_log2;  // base 2 (the scale is positive)
        const bool grow = mx > m_run + kRescaleSlack;
        const float m_new = grow ? ceilf(mx) : m_run;
        l_run *= grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // a power of two, or 0
        m_run = m_new;
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float la = 0.f, lb = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], a.scale_log2, -m_use));
            x[16 + e] = __builtin_amdgcn_exp2f(fmaf(x[16 + e], a.scale_log2, -m_use));
            la += x[e];
            lb += x[16 + e];
        }
        l_run += la + lb;
        const int ca = TAIL ? min(max(jend - j0, 0), 16) : 16;
        const int cb = TAIL ? (hasB ? min(max(jend - j0 - 64, 0), 16) : 0) : 16;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f32x4 va = spa[16 + 4 * g + tt], vb = spb[16 + 4 * g + tt];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * tt + i;
                // stale tokens (past the unit's keys) may carry NaN scales
                x[e] = (!TAIL || e < ca) ? x[e] * va[i] : 0.f;
                x[16 + e] = (!TAIL || e < cb) ? x[16 + e] * vb[i] : 0.f;
            }
        }
        // block maxima over lanes l and l ^ 16 (one 32-token block each)
        float ma = x[0], mb = x[16];
#pragma unroll
        for (int e = 1; e < 16; ++e) {
            ma = fmaxf(ma, x[e]);
            mb = fmaxf(mb, x[16 + e]);
        }
        ma = pair16(ma, true);
        mb = pair16(mb, true);
        auto expo = [](float m) {
            int ex = 0;
            (void)frexpf(m, &ex);
            // >= -119 keeps both conversion scales below normal floats
            return m > 0.f ? min(max(ex - 8, -119), 127) : 0;
        };
        XA = expo(ma);
        XB = expo(mb);
        // hi = RNE(p / 2^X), lo = RNE((p - hi 2^X) / 2^(X-4)): the scaled converts
        // divide by (and the reverse one multiplies by) an exact power of two,
        // and p - hi 2^X is exact, so this is the plain split without separate
        // scalings
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int X = c ? XB : XA;
            const float s_hi = __uint_as_float(uint32_t(X + 127) << 23);
            const float s_lo = __uint_as_float(uint32_t(X + 123) << 23);
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const float* pw = x + 16 * c + e;
                s2_t h2 = {0, 0}, l2 = {0, 0};
                h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, pw[0], pw[1], s_hi, false);
                h2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h2, pw[2], pw[3], s_hi, true);
                const int hw = __builtin_bit_cast(int, h2);
                const auto h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, s_hi, false);
                const auto h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, s_hi, true);
                l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, pw[0] - h01[0], pw[1] - h01[1],
                                                              s_lo, false);
                l2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l2, pw[2] - h23[0], pw[3] - h23[1],
                                                              s_lo, true);
                hi[4 * c + e / 4] = hw;
                lo[4 * c + e / 4] = __builtin_bit_cast(int, l2);
            }
        }
    };

    // ---- the previous PV step, carried through the pipeline: its split
    // weights (the MFMA's B operands: dwords 0..3 the first chunk, 4..7 the
    // second), exponents, first chunk and valid-token counts per run
    struct Step {
        i32x8 bhi, blo;
        int XA, XB, tA, c0, c1;
    };
    // half H (d tiles H*DH ..) of the PV MFMAs of step s
    auto pv_half = [&](const Step& s, auto half_tag, auto tail_tag) {
        constexpr int H = decltype(half_tag)::value;
        constexpr bool TAIL = decltype(tail_tag)::value;
        // run 0 of lane group g lies in 32-token block g >> 1, run 1 in block
        // 2 + (g >> 1); lane group g supplies block g's scale: its own run 0
        // (g = 0) or run 1 (g = 3); lane group 1 takes lane group 3's run 0 and
        // lane group 2 lane group 0's run 1, across the 32-lane halves
        const int send = g == 0 ? s.XB : s.XA;
        const auto sw = __builtin_amdgcn_permlane32_swap(uint32_t(send), uint32_t(send), false, false);
        const int other = int(sw[0]) == send ? int(sw[1]) : int(sw[0]);
        const int xs = g == 0 ? s.XA : g == 3 ? s.XB : other;
        const int sc_hi = xs + 127, sc_lo = xs - 4 + 127;
        const uint8_t* va = vring + (s.tA % NV) * CHB + v8a;
        const uint8_t* vb = vring + ((s.tA + 1) % NV) * CHB + v8a;
        uint32_t mask0[4], mask1[4];
        if constexpr (TAIL) {
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const int n0 = min(max(s.c0 - 4 * k2, 0), 4), n1 = min(max(s.c1 - 4 * k2, 0), 4);
                mask0[k2] = n0 == 4 ? ~0u : (1u << (8 * n0)) - 1u;
                mask1[k2] = n1 == 4 ? ~0u : (1u << (8 * n1)) - 1u;
            }
        }
        // d tiles per MFMA group (their V^T reads first)
        constexpr int DG = DH < 4 ? DH : 4;
        static_assert(DH % DG == 0, "whole groups per half");
#pragma unroll
        for (int d0 = H * DH; d0 < (H + 1) * DH; d0 += DG) {
            i32x8 vop[DG];
#pragma unroll
            for (int j = 0; j < DG; ++j) {
                u32x4 x0 = *reinterpret_cast<const u32x4*>(va + 256 * (d0 + j));
                // an absent second chunk reads a stale slot, masked to zero
                u32x4 x1 = *reinterpret_cast<const u32x4*>(vb + 256 * (d0 + j));
                if constexpr (TAIL) {
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        x0[k2] &= mask0[k2];
                        x1[k2] &= mask1[k2];
                    }
                }
                vop[j] = i32x8{int(x0[0]), int(x0[1]), int(x0[2]), int(x0[3]),
                               int(x1[0]), int(x1[1]), int(x1[2]), int(x1[3])};
            }
#pragma unroll
            for (int j = 0; j < DG; ++j)
                acc[d0 + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    vop[j], s.bhi, acc[d0 + j], 0, 0, 0, 0x7F7F7F7F, 0, sc_hi);
#pragma unroll
            for (int j = 0; j < DG; ++j)
                acc[d0 + j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    vop[j], s.blo, acc[d0 + j], 0, 0, 0, 0x7F7F7F7F, 0, sc_lo);
        }
    };
    // the accumulator follows the running max before a step's PV MFMAs
    auto rescale_acc = [&]() {
        if (__any(m_acc != m_run)) {
            // a power of two, or 0 from -inf; rows whose max did not move keep 1
            const float alpha = m_acc == m_run ? 1.f : __builtin_amdgcn_exp2f(m_acc - m_run);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            m_acc = m_run;
        }
    };

    // ---- ring step of PV step j: every load this wave has in flight is step
    // j's (issued right after the previous step's barrier), so wait for all of
    // them; the barrier then also frees the slots step j - 1 used, and the
    // next step's K (chunks 2j + 2, 2j + 3) and V^T go into them
    auto ring_step = [&](int j) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        const int tn = 2 * j + 2;
        if (tn < nchunks) {
            const int lo_need = 4 * tn, hi_need = min(4 * tn + 7, npages - 1);
            if (hi_need - tbase >= kPtab) {  // slide the page-table window (long units only)
                tbase = lo_need;
                fill_ptab(tbase);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                __syncthreads();
            }
            issue_chunk(tn, 0);
            if (tn + 1 < nchunks) issue_chunk(tn + 1, 1);
        }
    };

    // ---- step j: scores of chunks 2j and 2j + 1 (the second may be absent in
    // a masked step), their softmax, then the step's PV MFMAs
    auto step = [&](int j, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int tA = 2 * j;
        const bool hasB = tA + 1 < nchunks;
        Step cur;
        cur.tA = tA;
        cur.c0 = min(max(jend - (un.pb + tA * 4 + g) * kPage, 0), 16);
        cur.c1 = hasB ? min(max(jend - (un.pb + tA * 4 + 4 + g) * kPage, 0), 16) : 0;
        ring_step(j);
        if (has_tile) {
            f32x4 sa[4], sb[4];
            qk(tA, sa);
            if (!TAIL || hasB) {
                qk(tA + 1, sb);
            } else {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) sb[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            softmax_step(tA, sa, sb, hasB, cur.bhi, cur.blo, cur.XA, cur.XB, tail_tag);
            rescale_acc();
            pv_half(cur, std::integral_constant<int, 0>{}, tail_tag);
            pv_half(cur, std::integral_constant<int, 1>{}, tail_tag);
        }
    };

    // Chunks that need a mask (keys past the unit's end or some row's causal
    // limit) are a suffix, those below some row's sliding window a prefix; a
    // step with any of them, or with one chunk only, runs the masked code.
    // Three loops, so that no loop body carries both variants.
    int c_tail = nchunks;
    while (c_tail > 0 && (un.pb + 4 * (c_tail - 1)) * kPage + 64 > first_masked) --c_tail;
    int c_head = 0;
    while (c_head < c_tail && (un.pb + 4 * c_head) * kPage < win_hi) ++c_head;
    const int ngroups = (nchunks + 1) >> 1;
    const int g_head = (c_head + 1) >> 1, g_tail = c_tail >> 1;  // unmasked steps [g_head, g_tail)
    int j = 0;
    for (; j < g_head; ++j) step(j, std::true_type{});
    for (; j < g_tail; ++j) step(j, std::false_type{});
    for (; j < ngroups; ++j) step(j, std::true_type{});

    if (!has_tile) return;
    finish_unit<D>(a, acc, m_run, l_run, u, un, w, l, g, r, qi, T);
}

// ----------------------------------------------------------------------------
// MXFP4 sweep.  Steps of 128 tokens (two 64-token chunks of 4 pages each) with
// one softmax per step, as in the e4m3 sweep.  Scores run on the scaled MFMA:
// the E2M1 K codes are its A operand and their E8M0 bytes its A scales, Q
// split into two e4m3 parts (load_split_q) its B operand.  The V^T codes of a
// step are decoded by all eight waves into a bf16 staging tile, the V scales
// exact in it, and the PV product runs on the bf16 MFMA over four 32-token
// blocks.
//
// One step: barrier (the step's loads have landed and every read of the
// previous step is done) -> loads of the next step into the slots the previous
// step used -> decode of this step's V -> scores and softmax -> barrier (the
// staging tile is complete) -> PV.
//
// Token map: MFMA row m of score tile tt (0..3) of a chunk is chunk token
// 32 (tt >> 1) + 8 (m >> 2) + 4 (tt & 1) + (m & 3), so the S^T accumulators of
// tiles 2b and 2b + 1 give lane group g the chunk tokens 32b + 8g .. 32b + 8g
// + 7: the B operand of the bf16 PV MFMA over 32-token block b of the chunk.
//
// LDS layouts are operand-major: every 16-byte operand piece a lane reads
// sits at 16 l of a 1 KiB block, so the 16 lanes of a group read 256
// contiguous bytes (measured on gfx950: ds_read_b128 with each lane in its
// own row reaches about 60% of the rate of such contiguous reads, whatever
// the bank swizzle).  The DMA places every piece there from its own source.
// LDS ring slot of a chunk (bytes):
//   [0, 32D)    K codes: block (tt, k) of 1 KiB = the A operand of score tile
//               tt, k-step k: piece 16g + m = bytes 64k + 16g .. of the K row
//               of MFMA row m (chunk token 32 (tt >> 1) + 8 (m >> 2) +
//               4 (tt & 1) + (m & 3))
//   [32D, 64D)  V^T codes of the chunk's 4 page-heads as stored ([D][8] each)
//   [64D, 66D)  K scales of the 4 page-heads ([16][D/32] each: [token][D/32])
//   [66D, 68D)  V scales of the 4 page-heads ([D/32][16] each)
// Staging (bf16 V^T of a step): block (32-token block b, d tile dt) of 1 KiB
// = the A operand of the PV MFMA: piece 16c + m = tokens 8c .. 8c + 7 of
// block b, row d = 16 dt + m.
// ----------------------------------------------------------------------------

template <int D, bool SPARE>
__global__ __launch_bounds__(kSweepThreads, 1) void sweep4_kernel(Params a) {
    static_assert(D == 128 || D == 256, "MXFP4 serves D = 128 and 256");
    constexpr int KS4 = D / 128;               // 128-deep k-steps of the scores
    constexpr int DT = D / 16;                 // 16-wide d tiles of the output
    constexpr int PGB = 8 * D;                 // codes of one page-head, K or V^T
    constexpr int SPB = D / 2;                 // E8M0 scales of one page-head
    constexpr int OFF_V = 4 * PGB;             // ring slot: V^T codes
    constexpr int OFF_KS = 8 * PGB;            // ring slot: K scales
    constexpr int OFF_VS = OFF_KS + 4 * SPB;   // ring slot: V scales
    constexpr int CHB = OFF_VS + 4 * SPB;      // one chunk's ring slot
    constexpr int NR = 4;                      // ring slots: two steps
    constexpr int N16 = CHB / 16;              // 16-byte pieces of a chunk
    constexpr int NI = (N16 + 63) / 64;        // DMA instructions per chunk
    constexpr int MI = SPARE ? 1 : (2 * NI + kSweepWaves - 1) / kSweepWaves;  // per wave and step
    constexpr int BLK = 64 * D;                // staging bytes of one 32-token block
    constexpr int NDEC = 8 * D / kSweepThreads;  // decode items per thread and step
    // score tiles whose K operands are read together, (block, d tile) PV
    // products per operand-read group (measured: 4 and 4 are faster at D = 128)
    constexpr int QB = D == 256 ? 8 : 4;
    constexpr int PG = D == 256 ? 8 : 4;
    static_assert(CHB % 256 == 0 && NDEC * kSweepThreads == 8 * D, "config");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NR * CHB];
    __shared__ __attribute__((aligned(1024))) uint8_t stg[4 * BLK];
    __shared__ int32_t ptab[kPtab];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int g = l >> 4;
    const int ln = l & 15;

    const Unit un = decode_unit(a, blockIdx.x);
    const int u = blockIdx.x;
    const int p = un.p, kvh = un.kvh, L = un.L;
    const int npages = un.pe - un.pb;
    const int nchunks = (npages + 3) >> 2;
    const int jend = min(L, un.pe * kPage);
    const int lim_lo = a.causal ? (L - a.W + 1) : L;
    const int first_masked = min(jend, lim_lo);
    const int win_hi = a.window_left > 0 ? L - a.window_left : INT_MIN;

    const int T = (a.R + 15) >> 4;
    const bool has_tile = w < T;
    const int r = 16 * w + ln;
    const int qi = r / a.G;
    const int hi_row = a.causal ? (L - a.W + qi) : (L - 1);
    const int hi_tok = min(jend - 1, hi_row);
    const int lo_tok = a.window_left > 0 ? hi_row - a.window_left + 1 : INT_MIN;

    int tbase = 0;
    auto fill_ptab = [&](int base) {
        for (int k = tid; k < kPtab; k += kSweepThreads)
            if (base + k < npages) ptab[k] = phys_page(a, p, un.pb + base + k);
    };
    fill_ptab(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // ---- DMA work.  Instruction i of a chunk (NI of them) moves pieces
    // q = 64 i + l: K codes (placed operand-major, gathered from the chunk's
    // four pages), then V^T codes, then K and V scales.
    // SPARE (five or six row tiles, chosen at launch): the V^T code
    // instructions come from waves 0..3, the K code and scale instructions
    // from the waves without a row tile, and none from the second row-tile
    // waves of SIMDs 0 and 1 (waves 4 and 5), whose chain is each step's
    // longest.  Per-wave timestamps at 64K W = 16 showed every issuing wave
    // spending 1500-2000 cycles of a ~9000-cycle step on its loads, most of it
    // on the gathered K instructions; the waves without a row tile have that
    // time to spare, the V^T copies are cheap.  64K W = 16: 53.9 -> 49.7 us.
    // Otherwise every wave issues the instructions I = w + 8 m of a step's
    // 2 NI, I = NI c + i being instruction i of the step's chunk c.  Lane l of
    // instruction i moves piece q = 64 i + l of the chunk; its source array
    // (0 K codes, 1 V^T codes, 2 K scales, 3 V scales), page of the chunk and
    // byte offset in that page-head are packed as off | pg << 12 | arr << 14,
    // bit 16 set for a piece inside the chunk.
    uint32_t dsc[MI];
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int q = 64 * ((w + kSweepWaves * m) % NI) + l;
        int arr = 0, pg = 0, off = 0;
        if (q < 2 * D) {  // block (tt, k) = q >> 6, piece 16g + m = q & 63
            const int tt = (q >> 6) / KS4, k = (q >> 6) % KS4, gg = (q >> 4) & 3, m = q & 15;
            const int row = 32 * (tt >> 1) + 8 * (m >> 2) + 4 * (tt & 1) + (m & 3);
            pg = row >> 4;
            off = (row & 15) * (D / 2) + 16 * (4 * k + gg);
        } else if (q < 4 * D) {
            const int o = 16 * (q - 2 * D);
            arr = 1;
            pg = o / PGB;
            off = o % PGB;
        } else {
            const int o = 16 * (q - 4 * D);
            arr = o >= 4 * SPB ? 3 : 2;
            pg = (o % (4 * SPB)) / SPB;
            off = o % SPB;
        }
        dsc[m] = uint32_t(off) | uint32_t(pg) << 12 | uint32_t(arr) << 14 |
                 (q < N16 ? 1u << 16 : 0u);
    }
    const uint32_t ring_base = uint32_t(reinterpret_cast<uintptr_t>(ring));
    // Source addresses as integers: the array is a base plus a uniform
    // (code instructions) or per-lane (the scale instruction) difference.  A
    // select among the four pointers would be compiled as a per-lane lookup
    // in a private table, a memory load in front of every DMA.
    const uint64_t kcb = reinterpret_cast<uint64_t>(a.k);
    const uint64_t vcd = reinterpret_cast<uint64_t>(a.v) - kcb;
    const uint64_t ksb = reinterpret_cast<uint64_t>(a.k_scale);
    const uint64_t vsd = reinterpret_cast<uint64_t>(a.v_scale) - ksb;

    // loads of step j: chunks 2j and 2j + 1, those that exist; pages past the
    // unit's end are replaced by the chunk's first page and masked later.
    // SPARE: chunk c's K code and scale instructions are dealt over the 8 - T
    // waves without a row tile, its V^T code instructions over waves 0..3;
    // the four page ids of a chunk are read once, and each lane selects its
    // page (the K pieces of one instruction come from all four pages).
    auto issue_spare = [&](int j) {
        const bool k_issuer = w >= T;  // a wave without a row tile
        if (!k_issuer && w >= 4) return;
        const int nk = 8 - T, ek = w - T;
        constexpr int NKI = 2 * D / 64, NVI = 2 * D / 64, NSI = NI - NKI - NVI;
        const int mm = l & 15, gg = (l >> 4) & 3;
        const int lrow = 8 * (mm >> 2) + (mm & 3);
#pragma unroll 1
        for (int c = 0; c < 2; ++c) {
            const int t = 2 * j + c;
            if (t >= nchunks) break;
            int pid[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int n = 4 * t + k < npages ? 4 * t + k : 4 * t;
                pid[k] = __builtin_amdgcn_readfirstlane(ptab[n - tbase]);
            }
            const uint32_t slot = ring_base + uint32_t((t % NR) * CHB);
            if (k_issuer) {
#pragma unroll
                for (int idx = 0; idx < NKI + NSI; ++idx) {
                    const int n = c * (NKI + NSI) + idx;
                    if (n % nk != ek) continue;
                    if (idx < NKI) {  // K codes: operand block (tt, k)
                        const int tt = idx / KS4, k = idx % KS4;
                        const int row = 32 * (tt >> 1) + 4 * (tt & 1) + lrow;
                        const int off = (row & 15) * (D / 2) + 16 * (4 * k + gg);
                        const int ph = pick4(row >> 4, pid[0], pid[1], pid[2], pid[3]);
                        const uint64_t src = kcb + uint64_t(int64_t(ph) * a.Hkv + kvh) * PGB + off;
                        dma16(reinterpret_cast<const void*>(src),
                              __builtin_amdgcn_readfirstlane(slot + 1024u * uint32_t(idx)));
                    } else {  // K scales, then V scales
                        const int i = NKI + NVI + (idx - NKI);
                        const int q = 64 * i + l;
                        const int o = 16 * (q - 4 * D);
                        const int ph = pick4((o % (4 * SPB)) / SPB, pid[0], pid[1], pid[2], pid[3]);
                        const uint64_t src = ksb + (o >= 4 * SPB ? vsd : 0) +
                                             uint64_t(int64_t(ph) * a.Hkv + kvh) * SPB + o % SPB;
                        if (q < N16)
                            dma16(reinterpret_cast<const void*>(src),
                                  __builtin_amdgcn_readfirstlane(slot + 1024u * uint32_t(i)));
                    }
                }
            } else {
#pragma unroll
                for (int iv = 0; iv < NVI; ++iv) {  // V^T codes, 1 KiB of one page each
                    if (((c * NVI + iv) & 3) != w) continue;
                    const int pg = (1024 * iv) / PGB;
                    const uint64_t src = kcb + vcd + uint64_t(int64_t(pid[pg]) * a.Hkv + kvh) * PGB +
                                         (1024 * iv) % PGB + 16 * l;
                    dma16(reinterpret_cast<const void*>(src),
                          __builtin_amdgcn_readfirstlane(slot + 1024u * uint32_t(NKI + iv)));
                }
            }
        }
    };
    // otherwise: every page id of this wave's instructions is read first (a DMA
    // statement carries a memory clobber, so an LDS read placed between two of
    // them would make the second wait for the first's page id to arrive)
    auto issue_step = [&](int j) {
        if constexpr (SPARE) {
            issue_spare(j);
            return;
        }
        int phys[MI];
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            const int t = 2 * j + (w + kSweepWaves * m) / NI;
            int n = 4 * t + (int(dsc[m] >> 12) & 3);
            if (n >= npages) n = 4 * t;
            phys[m] = ptab[min(max(n - tbase, 0), kPtab - 1)];
        }
#pragma unroll
        for (int m = 0; m < MI; ++m) {
            const int I = w + kSweepWaves * m;
            if (I >= 2 * NI) break;  // wave-uniform
            const int c = I / NI, i = I % NI;
            const int t = 2 * j + c;
            if (t < nchunks) {
                const uint32_t ds = dsc[m];
                const int64_t ph = int64_t(phys[m]) * a.Hkv + kvh;
                // one array per code instruction (i is uniform); the scale
                // instruction holds K scales, then V scales (bit 14)
                const uint64_t src =
                    i < 4 * D / 64
                        ? kcb + (i >= 2 * D / 64 ? vcd : 0) + uint64_t(ph) * PGB
                        : ksb + ((ds >> 14) & 1 ? vsd : 0) + uint64_t(ph) * SPB;
                const uint32_t lds = ring_base + uint32_t((t % NR) * CHB + 1024 * i);
                if (ds & (1u << 16))
                    dma16(reinterpret_cast<const void*>(src + (ds & 0xFFFu)),
                          __builtin_amdgcn_readfirstlane(lds));
            }
        }
    };

    // ---- prologue: step 0's loads, then Q (one round trip for both)
    if (nchunks > 0) issue_step(0);
    i32x8 qhi[KS4], qlo[KS4];
    uint32_t shi = 0, slo = 0;
    load_split_q<D>(a, p, kvh, has_tile && r < a.R, qi, r - qi * a.G, g, ln, qhi, qlo, shi, slo);

    // K scales: the E8M0 byte of the lane's K row r = 32 (tt >> 1) + 4 (tt & 1)
    // + rl, rl = 8 (ln >> 2) + (ln & 3), for its k-block g of k-step k: byte
    // 4k + g of the row's scales
    const int rl = 8 * (ln >> 2) + (ln & 3);
    const uint32_t ksof = uint32_t(OFF_KS + rl * (D / 32) + g);

    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    auto ring_step = [&](int j) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        const int tn = 2 * j + 2;
        if (tn < nchunks) {
            const int lo_need = 4 * tn, hi_need = min(4 * tn + 7, npages - 1);
            if (hi_need - tbase >= kPtab) {  // slide the page-table window (long units only)
                tbase = lo_need;
                fill_ptab(tbase);
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                __syncthreads();
            }
            issue_step(j + 1);
        }
    };

    // ---- decode of step j's V^T codes.  Item (chunk c, page pg, rows d and
    // d + 16 of one 32-row block): the two rows' 16 codes each (8 bytes, the
    // even token in the low nibble) and the 16 tokens' E8M0 bytes of their
    // block, which both rows share.  The rows' nibbles are re-paired so that
    // byte i of E (O) holds token 2i (2i + 1) of row d in its low nibble and of
    // row d + 16 in its high one: both codes of a byte then take one token's
    // scale, one convert per byte, and the two rows' values are sorted back
    // into their rows by byte permutes.  Tokens past the unit's keys (stale
    // slots, pages past the end) are written as zeros.
    auto decode = [&](int j, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        constexpr int NP = NDEC / 2;  // row pairs per thread and step
        uint2 ca[NP], cb[NP];
        u32x4 sv[NP];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const int it = tid + kSweepThreads * n;
            const int dl = it % (D / 2), pg = (it / (D / 2)) & 3, c = it / (2 * D);
            const int d = 32 * (dl >> 4) + (dl & 15);
            const uint8_t* src = ring + ((2 * j + c) % NR) * CHB;
            ca[n] = *reinterpret_cast<const uint2*>(src + OFF_V + pg * PGB + d * 8);
            cb[n] = *reinterpret_cast<const uint2*>(src + OFF_V + pg * PGB + (d + 16) * 8);
            sv[n] = *reinterpret_cast<const u32x4*>(src + OFF_VS + pg * SPB + (d >> 5) * 16);
        }
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const int it = tid + kSweepThreads * n;
            const int dl = it % (D / 2), pg = (it / (D / 2)) & 3, c = it / (2 * D);
            const int d = 32 * (dl >> 4) + (dl & 15);
            const u32x4 sc = sv[n];
            const int vc = TAIL ? min(max(jend - (un.pb + 4 * (2 * j + c) + pg) * kPage, 0), 16) : 16;
            // row d: pieces 2 (pg & 1) + h of block 2c + (pg >> 1); row d + 16 one
            // d tile (1 KiB) further
            uint8_t* dst = stg + (2 * c + (pg >> 1)) * BLK + (d >> 4) * 1024 + (pg & 1) * 512 +
                           (d & 15) * 16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // tokens 8h .. 8h + 7
                const uint32_t a = h ? ca[n].y : ca[n].x, b = h ? cb[n].y : cb[n].x;
                const uint32_t E = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
                const uint32_t O = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
                u32x4 ra, rb;  // rows d and d + 16: word i = tokens 8h + 2i, 8h + 2i + 1
                auto pair = [&](auto i_tag) {
                    constexpr int i = decltype(i_tag)::value;
                    // token 8h + 2i: scale byte 2i of word 2h + (i >> 1) of sc
                    const uint32_t sw = sc[2 * h + (i >> 1)];
                    const uint32_t te = e2m1x2_to_bf16<i>(E, e8m0_operand<2 * (i & 1)>(sw));
                    const uint32_t to = e2m1x2_to_bf16<i>(O, e8m0_operand<2 * (i & 1) + 1>(sw));
                    uint32_t wa = (te & 0xFFFFu) | (to << 16);
                    uint32_t wb = (te >> 16) | (to & 0xFFFF0000u);
                    if constexpr (TAIL) {
                        const int t = 8 * h + 2 * i;
                        const uint32_t m = t + 1 < vc ? 0xffffffffu : (t < vc ? 0x0000ffffu : 0u);
                        wa &= m;
                        wb &= m;
                    }
                    ra[i] = wa;
                    rb[i] = wb;
                };
                pair(std::integral_constant<int, 0>{});
                pair(std::integral_constant<int, 1>{});
                pair(std::integral_constant<int, 2>{});
                pair(std::integral_constant<int, 3>{});
                *reinterpret_cast<u32x4*>(dst + 256 * h) = ra;
                *reinterpret_cast<u32x4*>(dst + 1024 + 256 * h) = rb;
            }
        }
    };

    // ---- scores of step j: s[4c + tt] = tile tt of chunk 2j + c (chunk B
    // only if present); per k-step all tiles' K operands, then the hi MFMAs,
    // then the lo MFMAs
    auto qk = [&](int j, bool hasB, f32x4 (&s)[8]) {
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) s[t8] = f32x4{0.f, 0.f, 0.f, 0.f};
        // tiles t0 .. t0 + QB - 1, k-step k
        auto kstep = [&](int t0, auto k_tag) {
            constexpr int k = decltype(k_tag)::value;
            u32x4 kw[QB];
            uint32_t sa[QB];
#pragma unroll
            for (int e = 0; e < QB; ++e) {
                const int t8 = t0 + e;
                const uint8_t* sl = ring + ((2 * j + (t8 >> 2)) % NR) * CHB;
                const int tt = t8 & 3, r0 = 32 * (tt >> 1) + 4 * (tt & 1);
                kw[e] = *reinterpret_cast<const u32x4*>(sl + (tt * KS4 + k) * 1024 + 16 * l);
                sa[e] = sl[ksof + r0 * (D / 32) + 4 * k];
            }
#pragma unroll
            for (int e = 0; e < QB; ++e) {
                if (t0 + e >= 4 && !hasB) break;
                const i32x8 ka = {int(kw[e][0]), int(kw[e][1]), int(kw[e][2]), int(kw[e][3]),
                                  0, 0, 0, 0};
                s[t0 + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    ka, qhi[k], s[t0 + e], 4, 0, 0, int(sa[e]), k, int(shi));
            }
#pragma unroll
            for (int e = 0; e < QB; ++e) {
                if (t0 + e >= 4 && !hasB) break;
                const i32x8 ka = {int(kw[e][0]), int(kw[e][1]), int(kw[e][2]), int(kw[e][3]),
                                  0, 0, 0, 0};
                s[t0 + e] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    ka, qlo[k], s[t0 + e], 4, 0, 0, int(sa[e]), k, int(slo));
            }
        };
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += QB) {
            kstep(t0, std::integral_constant<int, 0>{});
            if constexpr (KS4 > 1) kstep(t0, std::integral_constant<int, 1>{});
        }
    };

    // ---- softmax of step j: one running max over the step's 32 scores per
    // lane (the softmax scale goes in the exponent), lazy rescale as in the
    // bf16 sweep, then the weights of 32-token block b as bf16 PV operands
    auto softmax = [&](int j, const f32x4 (&s)[8], bf16x8_t (&pf)[4], auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int j0 = (un.pb + 8 * j) * kPage + 8 * g;  // tile 0, element 0 of lane group g
        float x[32];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = s[t8][i];
                if (TAIL) {
                    const int tt = t8 & 3;
                    const int jj = j0 + 64 * (t8 >> 2) + 32 * (tt >> 1) + 4 * (tt & 1) + i;
                    v = (jj <= hi_tok && jj >= lo_tok) ? v : -INFINITY;
                }
                x[4 * t8 + i] = v;
            }
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
        mx = wave_max_groups(mx) * a.scale_log2;
        const bool grow = mx > m_run + kRescaleSlack;
        if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
            m_run = grow ? mx : m_run;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], a.scale_log2, -m_use));
            ls += x[e];
        }
        l_run += ls;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            pf[b] = bf16x8_t{(__bf16)x[8 * b], (__bf16)x[8 * b + 1], (__bf16)x[8 * b + 2],
                             (__bf16)x[8 * b + 3], (__bf16)x[8 * b + 4], (__bf16)x[8 * b + 5],
                             (__bf16)x[8 * b + 6], (__bf16)x[8 * b + 7]};
    };

    // ---- O^T += V^T . P^T over the step's four 32-token blocks, in groups
    // of PG (block, d tile) products: the operand reads of group n + 1 are
    // issued before the MFMAs of group n, so LDS latency hides behind them
    auto pv = [&](const bf16x8_t (&pf)[4]) {
        constexpr int NG = 4 * DT / PG;
        u32x4 vb[2][PG];
        auto rd = [&](int n, u32x4 (&dst)[PG]) {
#pragma unroll
            for (int e = 0; e < PG; ++e) {
                const int x = PG * n + e, b = x / DT, dt = x % DT;
                dst[e] = *reinterpret_cast<const u32x4*>(stg + b * BLK + dt * 1024 + 16 * l);
            }
        };
        rd(0, vb[0]);
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            if (n + 1 < NG) rd(n + 1, vb[(n + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < PG; ++e) {
                const int x = PG * n + e, b = x / DT, dt = x % DT;
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, vb[n & 1][e]), pf[b], acc[dt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto step = [&](int j, auto tail_tag) {
        const bool hasB = 2 * j + 1 < nchunks;
        ring_step(j);
        decode(j, tail_tag);
        f32x4 s[8];
        bf16x8_t pf[4];
        if (has_tile) {
            qk(j, hasB, s);
            softmax(j, s, pf, tail_tag);
        }
        __syncthreads();
        if (has_tile) pv(pf);
    };

    // masked steps as in the e4m3 sweep: a suffix (keys past the unit's end or
    // some row's causal limit), a prefix (below some row's sliding window)
    int c_tail = nchunks;
    while (c_tail > 0 && (un.pb + 4 * (c_tail - 1)) * kPage + 64 > first_masked) --c_tail;
    int c_head = 0;
    while (c_head < c_tail && (un.pb + 4 * c_head) * kPage < win_hi) ++c_head;
    const int nsteps = (nchunks + 1) >> 1;
    const int g_head = (c_head + 1) >> 1, g_tail = c_tail >> 1;
    int j = 0;
    for (; j < g_head; ++j) step(j, std::true_type{});
    for (; j < g_tail; ++j) step(j, std::false_type{});
    for (; j < nsteps; ++j) step(j, std::true_type{});

    if (!has_tile) return;
    finish_unit<D>(a, acc, m_run, l_run, u, un, w, l, g, r, qi, T);
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine over the S_p key splits of every (p, kvh, row).
// One workgroup per (p, kvh, 16-row tile t, d block k): the 1 KiB lane-native
// partial block (t, k) of each split, read whole by one wave.  In base 2, with
// the stored partial o_s = 2^e_s * h_s:
//   M = max_s lse_s;  lse = M + log2 sum_s 2^(lse_s - M);
//   o = sum_s 2^(lse_s - lse) * 2^e_s * h_s
// Row phase: 16 threads per row load that row's records (contiguous), fold
// them into a running (max, sum), merge by shuffles and leave the weights
// 2^(lse_s - lse) * 2^e_s in LDS.  Column phase: lane l = 16g + ln of wave v
// owns row 16t + ln, its 8 columns of block k and the splits s = v (mod 4).
// Every lane issues its partial-block loads right after the record loads, so
// both are in flight together (one memory round trip when S <= 64).  The
// waves' sums meet in LDS in a fixed order: repeated calls are bitwise equal.
// ----------------------------------------------------------------------------
// Value of another lane of the same 16-lane row, by DPP: step 0 rotates the
// row by 8, step 1 by 4, step 2 swaps lanes at distance 2 in each quad, step 3
// at distance 1 (dpp_ctrl row_ror:8, row_ror:4, quad_perm [2,3,0,1], [1,0,3,2]).
__device__ __forceinline__ float dpp_row_step(float x, int step) {
    const int v = __float_as_int(x);
    int r;
    switch (step) {
        case 0: r = __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false); break;
        case 1: r = __builtin_amdgcn_update_dpp(v, v, 0x124, 0xF, 0xF, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); break;
        default: r = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); break;
    }
    return __int_as_float(r);
}

__device__ __forceinline__ void lse_fold(float& m, float& sm, float v) {
    if (v == -INFINITY) return;
    if (v > m) {
        sm = sm * __builtin_amdgcn_exp2f(m - v) + 1.f;
        m = v;
    } else {
        sm += __builtin_amdgcn_exp2f(v - m);
    }
}

template <int D, bool FEW>
__global__ __launch_bounds__(kThreads) void combine_kernel(Params a) {
    constexpr int KP = D / 32;    // d blocks of two 16-wide tiles
    constexpr int KPF = 16;       // partial blocks per lane per batch
    constexpr int BATCH = 4 * KPF;  // splits per batch
    static_assert(BATCH == 64, "the launch picks FEW for at most 32 splits");
    constexpr int RPT = BATCH / 16;  // records per row-phase thread per batch
    static_assert(kThreads == 256, "four waves");
    __shared__ float wts[16][BATCH + 1];
    __shared__ float lse_row[16];
    __shared__ f32x4 part[3][2][64];

    const int T = (a.R + 15) >> 4;
    int b = blockIdx.x;
    const int k = b % KP;
    b /= KP;
    const int t = b % T;
    b /= T;
    const int kvh = b % a.Hkv;
    const int p = b / a.Hkv;
    const int S = (a.unit_off[p + 1] - a.unit_off[p]) / a.Hkv;
    if (S <= 1 && !a.combine) return;
    const int64_t u0 = a.unit_off[p] + int64_t(kvh) * S;
    const int tid = threadIdx.x;

    // row phase mapping: row pr of the tile, records s = pj (mod 16)
    const int pr = tid >> 4, pj = tid & 15;
    const bool pvalid = 16 * t + pr < a.R;
    const float2* prow = a.part_rec + u0 * a.R + int64_t(pvalid ? 16 * t + pr : 0) * S;
    // column phase mapping
    const int lane = tid & 63, v = tid >> 6;
    const int ln = lane & 15, g = lane >> 4;
    const int r = 16 * t + ln;
    const bool valid = r < a.R;
    const uint16_t* pb = a.part_o + (int64_t(t) * KP + k) * 512 + lane * 8;
    const int64_t ustride = int64_t(T) * KP * 512;

    // records of the first batch, then partial blocks: all in flight together.
    // With FEW (chosen at launch when no request has more than 32 splits)
    // slots past S are not loaded (zero weight, zero block), so a request with
    // few splits makes few memory requests.
    float2 rv[RPT];
    u32x4 o[KPF];
    if constexpr (FEW) {  // every request has fewer splits than a batch
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            rv[q] = pj + 16 * q < S ? prow[pj + 16 * q] : float2{-INFINITY, 0.f};
#pragma unroll
        for (int q = 0; q < KPF; ++q)
            o[q] = v + 4 * q < S ? *reinterpret_cast<const u32x4*>(pb + (u0 + v + 4 * q) * ustride)
                                 : u32x4{0u, 0u, 0u, 0u};
    } else {  // indices clamped to a written split; weights past S are zero
#pragma unroll
        for (int q = 0; q < RPT; ++q) rv[q] = prow[min(pj + 16 * q, S - 1)];
#pragma unroll
        for (int q = 0; q < KPF; ++q)
            o[q] = *reinterpret_cast<const u32x4*>(pb + (u0 + min(v + 4 * q, S - 1)) * ustride);
    }

    // the row's lse over all S records
    float m = -INFINITY, sm = 0.f;
    if (pvalid) {
#pragma unroll
        for (int q = 0; q < RPT; ++q)
            if (pj + 16 * q < S) lse_fold(m, sm, rv[q].x);
        for (int s = pj + BATCH; s < S; s += 16) lse_fold(m, sm, prow[s].x);
    }
    // merge the row's 16 lanes with DPP moves inside each 16-lane row (VALU,
    // no LDS permute): rotate by 8 (the lane l^8), by 4, then swap lane pairs
    // at distance 2 and 1 within quads.  The merge is commutative, so after
    // each step the lanes that hold the same set of records agree bitwise, and
    // after the last one all 16 do.
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        const float m2 = dpp_row_step(m, step), s2 = dpp_row_step(sm, step);
        const float mn = fmaxf(m, m2);
        if (mn != -INFINITY) {
            sm = (m == -INFINITY ? 0.f : sm * __builtin_amdgcn_exp2f(m - mn)) +
                 (m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f(m2 - mn));
            m = mn;
        }
    }
    const float lse_p = (m == -INFINITY || !(sm > 0.f)) ? -INFINITY : m + __log2f(sm);
    if (pj == 0) lse_row[pr] = lse_p;
    auto weight = [&](float2 rec, int s) {
        return (pvalid && s < S && lse_p != -INFINITY)
                   ? __builtin_amdgcn_exp2f(rec.x - lse_p) * rec.y : 0.f;
    };
#pragma unroll
    for (int q = 0; q < RPT; ++q) wts[pr][pj + 16 * q] = weight(rv[q], pj + 16 * q);
    __syncthreads();
    const float lse = lse_row[ln];

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += BATCH) {
        if (s0 > 0) {  // more than one batch of splits: refill weights and blocks
            __syncthreads();
#pragma unroll
            for (int q = 0; q < RPT; ++q) {
                const int s = s0 + pj + 16 * q;
                wts[pr][pj + 16 * q] = weight(prow[min(s, S - 1)], s);
            }
#pragma unroll
            for (int q = 0; q < KPF; ++q)
                o[q] = *reinterpret_cast<const u32x4*>(pb + (u0 + min(s0 + v + 4 * q, S - 1)) *
                                                                ustride);
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < KPF; ++q) {
            const float wgt = wts[ln][v + 4 * q];
            f32x4 h0, h1;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                h0[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(o[q][i])));
                h0[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(o[q][i] >> 16)));
                h1[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(o[q][2 + i])));
                h1[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(o[q][2 + i] >> 16)));
            }
            acc0 += wgt * h0;
            acc1 += wgt * h1;
        }
    }

    // ---- waves 1..3 hand their sums to wave 0, which writes the row
    if (v > 0) {
        part[v - 1][0][lane] = acc0;
        part[v - 1][1][lane] = acc1;
    }
    __syncthreads();
    if (v > 0 || !valid) return;
#pragma unroll
    for (int vv = 0; vv < 3; ++vv) {
        acc0 += part[vv][0][lane];
        acc1 += part[vv][1][lane];
    }
    const int i = r / a.G;
    const int h = kvh * a.G + (r - i * a.G);
    uint16_t* orow = a.out + ((int64_t(p) * a.W + i) * a.Hq + h) * D + 32 * k + 4 * g;
    uint2 pk;
    pk.x = uint32_t(f32_to_bf16_bits(acc0[0])) | (uint32_t(f32_to_bf16_bits(acc0[1])) << 16);
    pk.y = uint32_t(f32_to_bf16_bits(acc0[2])) | (uint32_t(f32_to_bf16_bits(acc0[3])) << 16);
    *reinterpret_cast<uint2*>(orow) = pk;
    pk.x = uint32_t(f32_to_bf16_bits(acc1[0])) | (uint32_t(f32_to_bf16_bits(acc1[1])) << 16);
    pk.y = uint32_t(f32_to_bf16_bits(acc1[2])) | (uint32_t(f32_to_bf16_bits(acc1[3])) << 16);
    *reinterpret_cast<uint2*>(orow + 16) = pk;
    if (k == 0 && g == 0) a.lse[(int64_t(p) * a.W + i) * a.Hq + h] = lse * kLn2;
}

// Page-trace export: the pool pages each work unit streams, in order.
__global__ void trace_kernel(Params a, int32_t* out, int64_t maxp) {
    const int u = blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= a.unit_off[a.P]) return;
    const Unit un = decode_unit(a, u);
    int64_t k = 0;
    for (int n = un.pb; n < un.pe && k < maxp; ++n, ++k) out[u * maxp + k] = phys_page(a, un.p, n);
    for (; k < maxp; ++k) out[u * maxp + k] = -1;
}

// Table check, one workgroup per request p: how many of the block-table entries
// a call reads for p (the pages from the first split's first page to the last
// split's end, as decode_unit gives them to the sweep) lie outside
// [0, num_pages); -1 when the device length breaks the rules the plan's host
// lengths were checked against.  Integer work only; a fixed reduction order.
__global__ __launch_bounds__(kThreads) void check_kernel(Params a, int32_t* bad) {
    const int p = blockIdx.x;
    const int L = a.seq[p];
    if (L < 0 || L > a.bt_stride * kPage || (a.causal && L > 0 && L < a.W)) {
        if (threadIdx.x == 0) bad[p] = -1;
        return;
    }
    const int S = (a.unit_off[p + 1] - a.unit_off[p]) / a.Hkv;
    const int pb = decode_unit(a, a.unit_off[p]).pb;
    const int pe = decode_unit(a, a.unit_off[p] + S - 1).pe;
    int cnt = 0;
    for (int n = pb + int(threadIdx.x); n < pe; n += kThreads) {
        const int pg = a.bt[int64_t(p) * a.bt_stride + n];
        cnt += (pg < 0 || pg >= a.num_pages) ? 1 : 0;
    }
    __shared__ int part[kThreads];
    part[threadIdx.x] = cnt;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (int(threadIdx.x) < h) part[threadIdx.x] += part[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) bad[p] = part[0];
}

// ==== host side: launches, events, error text (device code ends above) ====
thread_local char g_err[256] = "";

}  // namespace

// Scratch for small_w_attention_run_noalloc: the split partials and their
// records of one call, in device memory the library owns from module load to
// process end (each GPU holds its own copy).  In host code `scratch` names a
// host-side stand-in, not the device address: the address is fetched once per
// device with hipGetSymbolAddress and only that value is handed to kernels.
static __device__ __align__(256) uint8_t scratch[SMALLW_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr and a device error
// on failure); resolved on the first call made with that device current.
void* scratch_address() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        smallw::set_device_error("hipGetDevice", int(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        smallw::set_device_error("device index beyond the scratch table", int(hipErrorInvalidDevice));
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            smallw::set_device_error("hipGetSymbolAddress(scratch)", int(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

namespace smallw {
void set_device_error(const char* what, int hip_status) {
    snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(hipError_t(hip_status)));
}
}  // namespace smallw

namespace {

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        smallw::set_device_error(what, int(e));
        return SMALLW_EDEVICE;
    }
    return SMALLW_OK;
}

void fill_params(Params& a, const smallw_plan* pl) {
    const smallw_problem& pr = pl->prob;
    a.P = pr.num_reqs;
    a.W = pr.window;
    a.Hq = pr.num_q_heads;
    a.Hkv = pr.num_kv_heads;
    a.G = pl->G;
    a.R = pl->R;
    a.bt_stride = pr.max_pages_per_req;
    a.num_pages = pr.num_pages;
    a.causal = pr.causal;
    a.scale_log2 = pr.scale * kLog2e;
    a.split_pages = pr.split_pages;
    a.combine = pl->combine ? 1 : 0;
    a.window_left = pr.window_left;
    a.piece_align = smallw::piece_align(pr.kv_dtype);
    for (int p = 0; p <= pr.num_reqs; ++p) a.unit_off[p] = pl->unit_off[p];
}

// Launch through hipExtLaunchKernel so optional events take the kernel's own
// start and end timestamps (no marker packets between the kernels).
template <typename K>
int launch(K kernel, int64_t blocks, int threads, const Params& a, hipStream_t st, void* ev0,
           void* ev1, const char* what) {
    Params arg = a;
    void* args[] = {&arg};
    const hipError_t e =
        hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(unsigned(blocks)),
                           dim3(unsigned(threads)), args, 0, st, hipEvent_t(ev0), hipEvent_t(ev1), 0);
    if (e != hipSuccess) {
        smallw::set_device_error(what, int(e));
        return SMALLW_EDEVICE;
    }
    return check_launch(what);
}

template <int D>
int launch_sweep(const smallw_plan* pl, const Params& a, hipStream_t st, void* ev0, void* ev1) {
    if (pl->prob.kv_dtype == SMALLW_KV_FP8_E4M3)
        return launch(sweep8_kernel<D>, pl->U, kSweepThreads, a, st, ev0, ev1,
                      "sweep kernel launch");
    if (pl->prob.kv_dtype == SMALLW_KV_MXFP4) {
        if constexpr (D == 64) return SMALLW_EUNSUPPORTED;  // the planner rejects it first
        else
        {
            const int T = (pl->R + 15) / 16;
            if (T == 5 || T == 6)
                return launch(sweep4_kernel<D, true>, pl->U, kSweepThreads, a, st, ev0, ev1,
                              "sweep kernel launch");
            return launch(sweep4_kernel<D, false>, pl->U, kSweepThreads, a, st, ev0, ev1,
                          "sweep kernel launch");
        }
    }
    if (pl->prob.v_layout == SMALLW_V_TOKEN_MAJOR)
        return launch(sweep_kernel<D, 4, true>, pl->U, kSweepThreads, a, st,
                      ev0, ev1, "sweep kernel launch");
    return launch(sweep_kernel<D, 4>, pl->U, kSweepThreads, a, st, ev0, ev1,
                  "sweep kernel launch");
}

template <int D>
int launch_combine(const smallw_plan* pl, const Params& a, hipStream_t st, void* ev1) {
    const int64_t blocks =
        int64_t(pl->prob.num_reqs) * pl->prob.num_kv_heads * ((pl->R + 15) / 16) * (D / 32);
    // no request with more than half a batch of splits: skip the empty slots'
    // loads (measured: draft block 6.2 -> 5.5 us; at 34 splits no gain)
    int smax = 0;
    for (int32_t sp : pl->splits) smax = sp > smax ? sp : smax;
    if (smax <= 32)
        return launch(combine_kernel<D, true>, blocks, kThreads, a, st, nullptr, ev1,
                      "combine kernel launch");
    return launch(combine_kernel<D, false>, blocks, kThreads, a, st, nullptr, ev1,
                  "combine kernel launch");
}

int record(void* ev, hipStream_t st) {
    if (!ev) return SMALLW_OK;
    const hipError_t e = hipEventRecord(hipEvent_t(ev), st);
    if (e != hipSuccess) {
        smallw::set_device_error("hipEventRecord", int(e));
        return SMALLW_EDEVICE;
    }
    return SMALLW_OK;
}

}  // namespace

extern "C" {

int small_w_attention_plan(const smallw_problem* problem, const int32_t* seq_lens_host,
                           smallw_plan** out) {
    if (!problem || !out) return SMALLW_EINVAL;
    *out = nullptr;
    smallw_problem pr = *problem;
    if (pr.num_cus < 0) return SMALLW_EINVAL;
    if (pr.num_cus == 0) {
        int dev = 0, n = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || n <= 0) {
            smallw::set_device_error("compute-unit query", int(e));
            return SMALLW_EDEVICE;
        }
        pr.num_cus = n;
    }
    return smallw::build_plan(pr, seq_lens_host, out);
}

int small_w_attention_run_events(const smallw_plan* pl, const void* q, const void* k_pool,
                                 const void* v_pool, const void* k_scale,
                                 const void* v_scale, const int32_t* block_table,
                                 const int32_t* seq_lens, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* ev_start, void* ev_sweep_done, void* ev_end) {
    if (!pl || !q || !k_pool || !v_pool || !block_table || !seq_lens || !out || !lse)
        return SMALLW_EINVAL;
    const bool scaled = pl->prob.kv_dtype != SMALLW_KV_BF16;
    if (scaled && (!k_scale || !v_scale)) return SMALLW_EINVAL;
    if (pl->ws_bytes > 0) {
        if (!workspace || workspace_bytes < pl->ws_bytes) return SMALLW_EWORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SMALLW_EWORKSPACE;
    }
    Params a;
    memset(&a, 0, sizeof a);
    fill_params(a, pl);
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint8_t*>(k_pool);
    a.v = static_cast<const uint8_t*>(v_pool);
    a.k_scale = static_cast<const float*>(k_scale);  // MXFP4: E8M0 bytes, read as such
    a.v_scale = static_cast<const float*>(v_scale);
    a.bt = block_table;
    a.seq = seq_lens;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    if (pl->ws_bytes > 0) {
        a.part_o = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + pl->part_o_off);
        a.part_rec = reinterpret_cast<float2*>(static_cast<uint8_t*>(workspace) + pl->part_rec_off);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the sweep's end timestamp goes to ev_sweep_done, and to ev_end too when
    // there is no combine (then a marker copies it if both were asked for)
    void* sweep_stop = pl->combine ? ev_sweep_done : (ev_sweep_done ? ev_sweep_done : ev_end);
    int rc;
    switch (pl->prob.head_dim) {
        case 64: rc = launch_sweep<64>(pl, a, st, ev_start, sweep_stop); break;
        case 128: rc = launch_sweep<128>(pl, a, st, ev_start, sweep_stop); break;
        case 256: rc = launch_sweep<256>(pl, a, st, ev_start, sweep_stop); break;
        default: return SMALLW_EUNSUPPORTED;
    }
    if (rc) return rc;
    if (!pl->combine) return (ev_sweep_done && ev_end) ? record(ev_end, st) : SMALLW_OK;
    switch (pl->prob.head_dim) {
        case 64: return launch_combine<64>(pl, a, st, ev_end);
        case 128: return launch_combine<128>(pl, a, st, ev_end);
        default: return launch_combine<256>(pl, a, st, ev_end);
    }
}

int small_w_attention_run(const smallw_plan* pl, const void* q, const void* k_pool,
                          const void* v_pool, const void* k_scale, const void* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return small_w_attention_run_events(pl, q, k_pool, v_pool, k_scale, v_scale, block_table,
                                        seq_lens, out, lse, workspace, workspace_bytes, stream,
                                        nullptr, nullptr, nullptr);
}

int small_w_attention_run_noalloc(const smallw_plan* pl, const void* q, const void* k_pool,
                                  const void* v_pool, const void* k_scale, const void* v_scale,
                                  const int32_t* block_table, const int32_t* seq_lens, void* out,
                                  float* lse, void* stream) {
    if (!pl) return SMALLW_EINVAL;
    if (pl->ws_bytes > SMALLW_NOALLOC_SCRATCH_BYTES) return SMALLW_EWORKSPACE;
    void* ws = nullptr;
    if (pl->ws_bytes > 0) {
        ws = scratch_address();
        if (!ws) return SMALLW_EDEVICE;
    }
    return small_w_attention_run_events(pl, q, k_pool, v_pool, k_scale, v_scale, block_table,
                                        seq_lens, out, lse, ws, ws ? SMALLW_NOALLOC_SCRATCH_BYTES : 0,
                                        stream, nullptr, nullptr, nullptr);
}

int small_w_attention_trace_pages(const smallw_plan* pl, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* pages_out,
                                  size_t max_unit_pages, void* stream) {
    if (!pl || !block_table || !seq_lens || !pages_out || max_unit_pages == 0)
        return SMALLW_EINVAL;
    Params a;
    memset(&a, 0, sizeof a);
    fill_params(a, pl);
    a.bt = block_table;
    a.seq = seq_lens;
    const int blocks = (pl->U + 255) / 256;
    hipLaunchKernelGGL(trace_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       a, pages_out, int64_t(max_unit_pages));
    return check_launch("trace kernel launch");
}

int small_w_attention_check_pages(const smallw_plan* pl, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* bad_out, void* stream) {
    if (!pl || !block_table || !seq_lens || !bad_out) return SMALLW_EINVAL;
    Params a;
    memset(&a, 0, sizeof a);
    fill_params(a, pl);
    a.bt = block_table;
    a.seq = seq_lens;
    hipLaunchKernelGGL(check_kernel, dim3(pl->prob.num_reqs), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a, bad_out);
    return check_launch("check kernel launch");
}

const char* small_w_attention_strerror(int status) {
    switch (status) {
        case SMALLW_OK: return "ok";
        case SMALLW_EINVAL: return "invalid argument";
        case SMALLW_EUNSUPPORTED: return "unsupported problem (head_dim, window, rows, page size or request count)";
        case SMALLW_EWORKSPACE: return "workspace missing, misaligned or too small";
        case SMALLW_EDEVICE: return g_err[0] ? g_err : "HIP device error";
        case SMALLW_ENOMEM: return "host allocation failed";
        default: return "unknown status";
    }
}

}  // extern "C"
