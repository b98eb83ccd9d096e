/*
 * smallw.h -- small-window paged attention for speculative-decoding verify and
 * draft blocks on AMD Instinct MI355X (gfx950).
 *
 * One call computes softmax attention for a window of W = 1..16 query rows per
 * request against that request's paged KV cache, for P requests at once, and
 * reads every visible K/V byte once for all W rows and all query heads of a
 * KV group.
 *
 * Where the operation is defined:
 *  - "ChunkedSmallT re-streams full KV per query chunk (DFlash K>=8 verify at
 *    long context)", section Finding: the W = K+1 verify rows of a speculative
 *    step attend the visible key range; key splitting plus a reduce step merge
 *    the partial results.  Section Measurement: the call is timed per layer on
 *    a cold cache and its bandwidth is the KV bytes of one sweep / time.
 *  - "DFlash2 leaves the paged graph fast path at every c>1 ...", sections The
 *    route change and Scope: attention for P x (1+k) block rows only, against
 *    per-request paged context held in one shared pool, addressed by a batched
 *    block table and per-request sequence lengths; section The cost: draft
 *    block rows are non-causal and attend the request's entire span.
 *  - "perf(dflash): widen the verify window past the compact graph's four-row
 *    limit", section What changed: only seq_len entries are read, so stale
 *    slots past a request's length are never touched, and an unsupported width
 *    must be an error, not a silent refusal.
 *
 * Semantics (per request p with length L = seq_lens[p], window row i, query
 * head h, KV head kvh = h / (Hq/Hkv)):
 *   visible keys  j < L                       (causal == 0, draft block)
 *                 j <= L - W + i              (causal == 1, verify window:
 *                                              L counts the window's own rows,
 *                                              row i sits at position L-W+i)
 *                 and j >= h - N + 1 with window_left = N > 0, h the row's
 *                 last visible key ("DFlash2 leaves the paged graph fast path
 *                 ...", section The cost, notes that the draft path does not
 *                 apply a window and leaves it to a separate issue)
 *   s_j = scale * <q, k_j>;  out = softmax(s) . V;  lse = ln sum_j exp(s_j)
 *   A row with no visible key (only when L == 0) gets out = 0, lse = -inf.
 *
 * Device layouts (all row-major, caller-owned):
 *   q            bf16   [P][W][Hq][D]
 *   k_pool       [num_pages][Hkv][16][D]     bf16, or e4m3fn bytes
 *   v_pool       [num_pages][Hkv][D][16]     bf16, or e4m3fn bytes; each
 *                                            16-token page-head is stored
 *                                            transposed (d-major)
 *                [num_pages][Hkv][16][D]     bf16 with v_layout token-major
 *   k_scale      fp32 [num_pages][Hkv][16]   fp8 only: value = code * scale
 *   v_scale      fp32 [num_pages][Hkv][16]   fp8 only
 * MXFP4 pools (kv_dtype SMALLW_KV_MXFP4, head_dim 128 or 256) hold two E2M1
 * codes per byte, the even element in the low nibble:
 *   k_pool       uint8 [num_pages][Hkv][16][D/2]   byte i of token t: elements
 *                                                  2i, 2i+1 of its row
 *   v_pool       uint8 [num_pages][Hkv][D][8]      byte i of row d: element d
 *                                                  of tokens 2i, 2i+1
 *   k_scale      uint8 E8M0 [num_pages][Hkv][16][D/32]: byte b of token t
 *                scales elements 32b .. 32b+31 of that token's K row by
 *                2^(e-127)
 *   v_scale      uint8 E8M0 [num_pages][Hkv][D/32][16]: block-major like the
 *                transposed value page; byte [b][t] scales elements
 *                32b .. 32b+31 of token t's V row
 * ("ChunkedSmallT re-streams full KV per query chunk", section Measurement,
 * times a 4-bit KV cache; the format here is OCP MXFP4: E2M1 values
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, 32-element blocks, E8M0 scales.)
 *   block_table  int32 [P][max_pages_per_req]; entry n of row p is the pool
 *                page holding tokens [16n, 16n+16) of request p
 *   seq_lens     int32 [P], the lengths this call attends with.  The plan
 *                fixes only the split counts; the kernels recompute every
 *                page range from these device lengths.  So a plan (or a
 *                captured graph of a call) stays valid when lengths change
 *                between calls, provided each length still obeys the plan's
 *                host rules (0 <= L_p <= 16*max_pages_per_req; causal:
 *                L_p == 0 or L_p >= W) and its block-table row covers it.
 *                Split balance follows the plan's lengths.  The row-exact
 *                bitwise guarantee holds when they equal the device lengths.
 *   out          bf16   [P][W][Hq][D]
 *   lse          fp32   [P][W][Hq]   natural log
 * Pages are 16 tokens.  e4m3fn is the OCP 8-bit format (bias 7, max 448,
 * S.1111.111 = NaN, no infinities).
 *
 * Status codes: every call returns SMALLW_OK (0) or a negative code; no C++
 * exception crosses this interface.  All shape and range checks happen in
 * small_w_attention_plan on the host.  Block-table entries outside
 * [0, num_pages) are clamped on the device, so they cannot fault, but give
 * undefined numbers; small_w_attention_check_pages counts them.
 */
#ifndef SMALLW_H
#define SMALLW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMALLW_OK            0
#define SMALLW_EINVAL       (-1)  /* malformed argument (null, negative, inconsistent) */
#define SMALLW_EUNSUPPORTED (-2)  /* well-formed but outside what the kernels serve    */
#define SMALLW_EWORKSPACE   (-3)  /* workspace missing or smaller than required       */
#define SMALLW_EDEVICE      (-4)  /* a HIP call failed; see small_w_attention_strerror */
#define SMALLW_ENOMEM       (-5)  /* host allocation failed                            */

#define SMALLW_PAGE_SIZE     16
#define SMALLW_MAX_WINDOW    16
#define SMALLW_MAX_REQS      256
#define SMALLW_MAX_ROWS      128  /* W * (Hq / Hkv) */
/* device scratch the library holds per GPU for small_w_attention_run_noalloc */
#define SMALLW_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum { SMALLW_KV_BF16 = 0, SMALLW_KV_FP8_E4M3 = 1, SMALLW_KV_MXFP4 = 2 } smallw_kv_dtype;

/* How each 16-token page-head of the value pool is laid out.  D-major is the
 * default; token-major stores V like K (a 16 x D block, token rows of D
 * values), the layout a pool written token by token has. */
typedef enum { SMALLW_V_DMAJOR = 0, SMALLW_V_TOKEN_MAJOR = 1 } smallw_v_layout;

typedef struct smallw_problem {
    int32_t num_reqs;          /* P, 1..SMALLW_MAX_REQS                              */
    int32_t window;            /* W, 1..SMALLW_MAX_WINDOW                            */
    int32_t num_q_heads;       /* Hq >= 1                                            */
    int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0, W*Hq/Hkv <= 128           */
    int32_t head_dim;          /* D: 64, 128 or 256 (MXFP4: 128 or 256)              */
    int32_t page_size;         /* must be 16                                         */
    int32_t num_pages;         /* pool capacity in pages, >= 1                       */
    int32_t max_pages_per_req; /* block_table row stride, >= 1                       */
    int32_t causal;            /* 1 = verify window (tail mask), 0 = draft block     */
    int32_t kv_dtype;          /* smallw_kv_dtype                                    */
    float   scale;             /* softmax scale; <= 0 selects 1/sqrt(D)              */
    int32_t num_cus;           /* compute units to plan for; 0 = ask current device  */
    int32_t force_splits;      /* 0 = automatic; > 0 = this many key splits per
                                  request (capped at its page count)                 */
    int32_t split_pages;       /* 0 = automatic; > 0 = row-exact mode: every request
                                  is split at multiples of this many pages, counted
                                  from its first page, and every row is finished by
                                  the combine kernel, so a row's result depends only
                                  on its own query, keys and values: it is bitwise
                                  the same whatever W, the other rows and the other
                                  requests are (exclusive with force_splits)         */
    int32_t window_left;       /* 0 = none; N > 0 = sliding window: a row whose last
                                  visible key is at position h sees only the keys
                                  h-N+1 .. h (pages before the lowest row's window
                                  are not read at all)                               */
    int32_t v_layout;          /* smallw_v_layout; token-major needs kv_dtype bf16
                                  (SMALLW_EUNSUPPORTED otherwise)                   */
} smallw_problem;

typedef struct smallw_plan smallw_plan; /* opaque, host-only, immutable */

/*
 * Validate a problem and decide the split-K decomposition for one call.
 * Plan once per speculative step, then run it for every attention layer.
 *   seq_lens_host  host int32 [P]: L_p >= 0, L_p <= 16*max_pages_per_req, and
 *                  for causal calls L_p == 0 or L_p >= W.
 *   out            receives a new plan; release it with ..._plan_destroy.
 * Splits: n_p = ceil(L_p/16) pages, n_eff of them streamed (fewer with a
 * sliding window); slots = num_cus * (2 for a bf16 pool with D < 256, else 1)
 * (work units resident per compute unit); a round holds max(1, floor(slots /
 * Hkv)) splits.
 * S_p = 1 for an empty request, min(force_splits, n_eff) when forced, else
 * apportioned: every request starts at one split, and one more at a time goes
 * to the request with the most pages per split (n_eff / S_p; the lower index on
 * ties) that keeps 8 pages a split, until the splits reach the budget: one
 * round when P fits in it (no second round), else P plus one round.  This
 * makes the largest split as small as the budget allows.  Work unit
 * u = unit_off[p] + kvh*S_p + s covers pages [floor(s n/S), floor((s+1) n/S)).
 * Row-exact mode (split_pages = B > 0): S_p = max(1, ceil(n_p / B)) and split
 * s covers pages [s*B, min((s+1)*B, n_p)) (the last split takes every page up
 * to the device length).
 * Sliding window (window_left = N > 0): pages before n_lo = floor(max(0, h0 -
 * N + 1) / 16), h0 = L - W (causal) or L - 1, are skipped: the formulas above
 * apply to the n_p - n_lo pages from n_lo on (row-exact pieces stay on the
 * absolute grid of multiples of B; the first one starts at n_lo moved down to
 * a multiple of 2 pages (bf16) or 8 pages (e4m3, MXFP4) from its grid point, so
 * the pages one step of the sweep groups line up in every call).
 * Returns SMALLW_EINVAL / SMALLW_EUNSUPPORTED on bad input (nothing allocated),
 * SMALLW_EDEVICE if num_cus == 0 and the device query fails, SMALLW_ENOMEM.
 */
int small_w_attention_plan(const smallw_problem* problem, const int32_t* seq_lens_host,
                           smallw_plan** out);

/* Device workspace bytes small_w_attention_run needs (0 when no request is
 * split and the plan is not row-exact).  Holds per-split partial outputs and
 * log-sum-exps. */
size_t small_w_attention_workspace_bytes(const smallw_plan* plan);

/*
 * Enqueue the attention for one layer on `stream` (a hipStream_t; NULL = the
 * default stream).  Launches the split-K sweep kernel and, when any request
 * is split, the log-sum-exp combine kernel.  No host synchronisation and no
 * allocation, so the call can be captured in a HIP graph.  All pointers are
 * device pointers in the layouts above; k_scale / v_scale (fp32 for fp8,
 * E8M0 bytes for MXFP4) are required for those formats and ignored for
 * bf16.  workspace must be 256-byte aligned and hold
 * small_w_attention_workspace_bytes(plan) bytes (may be NULL when that is 0);
 * it is scratch owned by the caller and may be reused between calls on the
 * same stream.  A plan is immutable and may be shared by threads and streams;
 * calls that overlap (other streams) need their own workspace and outputs.
 * Returns SMALLW_EINVAL (null pointer / plan), SMALLW_EWORKSPACE, or
 * SMALLW_EDEVICE (launch failure).
 */
int small_w_attention_run(const smallw_plan* plan, const void* q, const void* k_pool,
                          const void* v_pool, const void* k_scale, const void* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * As small_w_attention_run, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  The split partials go to a scratch
 * array of SMALLW_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on
 * every GPU it runs on, from module load until the process ends; this call
 * allocates nothing, neither on the device nor through any library routine.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (other streams, concurrent threads) race and give undefined results;
 * serialise them, or use small_w_attention_run with separate workspaces.
 * Nothing in the scratch needs to start at any value: each call writes every
 * byte it reads.  Returns SMALLW_EWORKSPACE when the plan needs more than the
 * scratch holds (small_w_attention_workspace_bytes(plan) >
 * SMALLW_NOALLOC_SCRATCH_BYTES), otherwise as small_w_attention_run.
 */
int small_w_attention_run_noalloc(const smallw_plan* plan, const void* q, const void* k_pool,
                                  const void* v_pool, const void* k_scale, const void* v_scale,
                                  const int32_t* block_table, const int32_t* seq_lens, void* out,
                                  float* lse, void* stream);

/*
 * As small_w_attention_run, and additionally sets caller-created hipEvent_t
 * handles (created with timing enabled) from the kernel dispatches themselves:
 * ev_start takes the sweep kernel's start, ev_sweep_done its end, ev_end the
 * combine kernel's end (the sweep's end when no request is split).  Any event
 * may be NULL.  For timing the kernels in place, as a kernel profiler would.
 */
int small_w_attention_run_events(const smallw_plan* plan, const void* q, const void* k_pool,
                                 const void* v_pool, const void* k_scale,
                                 const void* v_scale, const int32_t* block_table,
                                 const int32_t* seq_lens, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* ev_start, void* ev_sweep_done, void* ev_end);

/*
 * Export the plan's integer decomposition into host int32 `buf` of `cap`
 * entries; *needed receives the entry count.  Layout:
 *   [P, Hkv, U, R]  R = W*Hq/Hkv rows per work unit
 *   S_p           x P
 *   unit_off      x (P+1)
 *   (p, kvh, s, page_begin, page_end) x U
 * Returns SMALLW_EINVAL if buf is too small (with *needed set).
 */
int small_w_attention_plan_export(const smallw_plan* plan, int32_t* buf, size_t cap,
                                  size_t* needed);

/*
 * Debug index export: on `stream`, write the physical pool page of every page
 * each work unit streams, in the order the sweep kernel streams them, using
 * the sweep kernel's own unit-decode and page-addressing device code.
 * pages_out is device int32 [U][max_unit_pages] (unused tail entries = -1);
 * max_unit_pages comes from small_w_attention_plan_max_unit_pages.
 */
int small_w_attention_trace_pages(const smallw_plan* plan, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* pages_out,
                                  size_t max_unit_pages, void* stream);

/*
 * Input check for callers that cannot vouch for their tables: on `stream`,
 * write bad_out[p] (device int32 [P]) = the number of block_table entries that
 * a call with this plan reads for request p and that lie outside
 * [0, num_pages), or -1 when seq_lens[p] breaks the device-length rules
 * (L < 0, L > 16 * max_pages_per_req, or causal with 0 < L < W).  The entries
 * read are those of the pages small_w_attention_trace_pages lists for p's
 * units: logical pages from the first one a row attends (moved down to the
 * row-exact grouping grid in row-exact mode with a sliding window) to
 * ceil(L / 16).  A run does not fault on bad entries (they are clamped) but
 * gives undefined numbers for that request; all zeros means every page the run
 * reads is a pool page.  The plan is only read; nothing is allocated; bad_out
 * is written by one kernel on `stream` (SMALLW_EDEVICE if the launch fails).
 */
int small_w_attention_check_pages(const smallw_plan* plan, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* bad_out, void* stream);

/* Largest page count of any work unit of the plan (host lengths). */
size_t small_w_attention_plan_max_unit_pages(const smallw_plan* plan);

/*
 * Paged KV append (the step right before a verify call): on `stream`, write the
 * W window tokens' K and V rows into their pool slots, using the plan's shapes.
 * "perf(dflash): widen the verify window past the compact graph's four-row
 * limit", section What changed: the window rows are written into the paged
 * cache, and slots past a request's length are overwritten later, never read.
 *   k_new, v_new  device bf16 [P][W][Hkv][D]: token i of request p sits at
 *                 position pos = L_p - W + i (requests with L_p < W - i skip it)
 *   k_pool, v_pool, k_scale, v_scale, block_table, seq_lens: as for
 *                 small_w_attention_run (scales required for e4m3 and MXFP4)
 * The K row goes to slot pos % 16 of page block_table[p][pos / 16], the V row
 * to the same slot of the transposed value page (row pos % 16 of the value
 * page when the plan's v_layout is token-major).  bf16 pools get the bits as
 * given.  e4m3 pools get, per (token, KV head) row, scale = amax|x| / 448 (1.0
 * for an all-zero row) and codes = round-to-nearest-even of x / scale on the
 * OCP e4m3fn grid, computed in fp32 with IEEE division.  MXFP4 pools get, per
 * 32-element block of a row, the E8M0 byte X + 127 with X = floor(log2 amax)
 * - 2 clamped to [-127, 127] (0 for an all-zero block) and codes = the E2M1
 * value nearest x / 2^X, ties to the even code, saturating at 6, with the sign
 * of x (OCP Microscaling Formats v1.0 conversion); only the window tokens'
 * nibbles of the shared value bytes change.  Rows of different tokens must map
 * to different slots.  Returns SMALLW_EINVAL (null pointer or
 * plan), SMALLW_EDEVICE (launch failure).
 */
int small_w_kv_append(const smallw_plan* plan, const void* k_new, const void* v_new,
                      void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                      const int32_t* block_table, const int32_t* seq_lens, void* stream);

/*
 * Bandwidth reference: on `stream`, read `bytes` of device memory at `buf` once
 * with 16-byte loads and nothing else (bytes a multiple of 16, buf 16-byte
 * aligned).  Its bytes / time is the practical HBM read ceiling that the
 * attention call's KV bandwidth is set against: "ChunkedSmallT re-streams full
 * KV per query chunk", section Measurement, rates the call by one sweep's K and
 * V bytes over its time on a cold cache.  sink: device uint32, written only for
 * one XOR value of the data (it keeps the loads alive).  ev_start / ev_end:
 * optional hipEvent_t handles set from the kernel dispatch itself.  Returns
 * SMALLW_EINVAL (null, unaligned or zero size) or SMALLW_EDEVICE.
 */
int small_w_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream,
                        void* ev_start, void* ev_end);

/* Release a plan (NULL is allowed). */
void small_w_attention_plan_destroy(smallw_plan* plan);

/* Static description of a status code; for SMALLW_EDEVICE, the last HIP
 * error seen by this library on the calling thread. */
const char* small_w_attention_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SMALLW_H */
