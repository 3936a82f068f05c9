// hc_prefill.hip -- the hyper-connection read for wide inputs (T > 25 tokens):
// prefill chunks and verify windows beyond the short-window kernel.
//
// The read is the one of "#315 hc: the multi-token hyper-connection read split
// finer" with the norm folded into the down projection ("#2488 sycl/A770",
// Summary item 4) and the up projection fused with gr_mix_r as in "#1370
// prefill: ... gr_mix_r as its epilogue", "What it does": gated (T x 10240
// fp32) never leaves registers.  Three launches per chunk of up to 8192 tokens:
//
//   P1 down:  part[sig][t][j] = sum_{k in split sig} W_down[j][k] * (R'[t][k] *
//             w_norm[k]) and ssq[sig][t] = sum_{k in sig} R'[t][k]^2 over S
//             column splits that lie inside the streams: S = 4 (whole streams)
//             for chunks of more than 8064 tokens without pending, 8 (stream
//             halves, 1280 columns) from 3969 tokens, 16 (quarters) for
//             chunks of 1025..3968 tokens, 32 (320 columns) for 385..1024 and
//             80 (128 columns) up to 384 tokens (splits_for).  Chunks of at
//             most 192 tokens run it on prefill_down_small (80 x NT
//             workgroups of 32- or 64-token tiles, every load at entry).
//   P2 lo:    rs[t][s] = 1/sqrt(sum of stream s's split ssq / 2560 + eps) and
//             lo[t][j] = sum_s rs[t][s] * (stream s's split partials), stored
//             in fp32 in the tiled layout P3 copies into LDS verbatim (P3
//             splits each value into its three bf16 pieces in registers).
//   P3 up+mix: the up projection (K = 320) on the matrix cores, then the mix
//             of the 4 streams with R' and the bf16 / fp16 images, all in
//             registers.  Chunks of at most 256 tokens: 16-column tiles
//             for one or two token tiles, 32-column ones for three or four
//             (prefill_upmix).  Longer chunks: 128 tokens x 64 columns x 4
//             streams per workgroup of 8 waves, persistent over its items
//             without pending (prefill_upmix3), one item per workgroup with
//             pending or for a ragged last 128 tokens (prefill_upmix2).
//
// gfx950 design:
// * Both matrix kernels run bf16 v_mfma_f32_16x16x32_bf16 with every fp32
//   activation split exactly into three bf16 pieces (hi + mid + lo3 == x), so
//   each product is exact and the result stays fp32-faithful.
// * Weight operands (and P3's lo tiles, and P1's raw activations) go from
//   memory straight into LDS (16 bytes a lane, global_load_lds_dwordx4 or
//   its buffer form) through rings: P1 loads its W_down panel one K step of
//   32 ahead and raw R (and pending) two or three steps ahead; the narrow
//   P3 runs a ring of three to five stages (two to four steps ahead), the
//   128-token ones a five-stage ring four steps ahead.  LDS is read with inline-asm
//   ds_read_b128 and every wait is explicit: the compiler, seeing an LDS read
//   that may alias a load still landing in LDS, would wait for ALL loads in
//   flight (vmcnt(0)) and serialise the ring.
// * Inside LDS a K step of a weight tile is a "panel": one row per matrix
//   row, four 16-byte chunks per row, chunk c of row r stored at slot
//   4 r + (c ^ ((r >> 1) & 3)).  LDS serves a 16-byte read to 8 lanes per
//   cycle; the 8 lanes that read one chunk column of 8 consecutive rows then
//   hit distinct bank groups (measured: the swizzle by r >> 2 instead left
//   ~45 % of LDS cycles in bank conflicts).
// * P1 takes a whole CU (12 waves, up to 157 KB of LDS: 8 matrix waves and 4
//   producer waves that load and convert); the 128-token P3 takes a whole CU
//   too (8 waves, 160 KB), the narrow one 4 waves and 48-64 KB.
// * XCD-aware grids (workgroup b runs on XCD b % 8): with 8 splits P1's XCD x
//   owns split x, so its 820 KB W_down slice stays in that XCD's L2; P3's XCD
//   x owns 5 of the 40 column groups (W_up slices, 820 KB) and walks the token
//   tiles, the 5 workgroups of one tile being dispatched together so its lo
//   tile is read once per XCD.
#include "hc_internal.h"

#include <type_traits>

#pragma clang fp contract(off)

namespace hc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(u32x4 a, u32x4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x == hi + mid + lo3 exactly (bf16 pieces; see the short-window kernel).
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo3)
{
    const uint32_t hb = __float_as_uint(x) & 0xffff0000u;
    const float r1 = x - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(mb);
    hi = hb >> 16;
    mid = mb >> 16;
    lo3 = __float_as_uint(r2) >> 16;
}

// ---- LDS access with explicit waits ----------------------------------------
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)p;  // the low 32 bits of a shared-aperture address are the LDS offset
}
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr)
{
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16_off(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}
__device__ __forceinline__ void ds_write16(uint32_t addr, u32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
// Waits for every LDS read of this wave; the values in `v` are then "produced
// here", so no use of them moves above the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&v)[N])
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm volatile("" : "+v"(v[i]));
}
__device__ __forceinline__ void pin(u32x4& v)
{
    asm volatile("" : "+v"(v));
}
// Waits until at most N LDS reads of this wave are in flight; the values
// named are then "produced here", so no use of them moves above the wait,
// and the scheduler moves no instruction across it.
template <int N, typename... V>
__device__ __forceinline__ void lgkm_wait(V&... v)
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt field");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
    (pin(v), ...);
}
// No memory access moves across this point.
__device__ __forceinline__ void order()
{
    asm volatile("" ::: "memory");
}
// Waits until at most VM of this wave's memory loads are in flight and its
// LDS accesses are done, then the workgroup barrier.
template <int VM>
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}
// The same, leaving the wave's LG most recent LDS reads in flight.
template <int VM, int LG>
__device__ __forceinline__ void ring_barrier_lg()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(%1)\n\ts_barrier" ::"n"(VM), "n"(LG) : "memory");
}
// A buffer resource over `base` (raw, 2 GB range): loads through it take a
// 32-bit byte offset per lane and a scalar one.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// 16 bytes per lane through a buffer resource into LDS (lane l's bytes at
// lds_wave_base + 16 l): the lane's byte offset `voff` and a scalar `soff`.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint4* lds_wave_base, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, soff, 0, 0);
}
// 16 bytes per lane from memory into LDS: lane l's bytes land at
// lds_wave_base + 16 l (the base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* g, uint4* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

// Slot (in 16-byte chunks) of chunk c (0..3) of row r in a panel.  LDS
// serves a 16-byte read to 8 lanes per cycle (128 bytes, 32 banks); the 8
// lanes reading chunk c of 8 consecutive rows (two rows per 128 bytes) then
// hit 8 distinct 16-byte bank groups.
__host__ __device__ constexpr int panel_slot(int r, int c)
{
    return 4 * r + (c ^ ((r >> 1) & 3));
}

// Slot (0..7) of chunk 0 of row r in a 128-byte line of 8 chunks: chunk c of
// row r is stored at slot c ^ swz8(r), so 16 lanes reading one chunk of 16
// consecutive rows hit distinct 16-byte bank groups.
__host__ __device__ constexpr int swz8(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}

constexpr int kTok = 64;                       // token tile of both matrix kernels
constexpr int kKs = 32;                        // K step: one MFMA depth
constexpr int kUpSteps = kRank / kKs;          // 10
constexpr int kUpCols = 64;                    // P3 output columns per tile
constexpr int kUpGroups = kWidth / kUpCols;    // 40 column groups
constexpr int kGroupsPerXcd = kUpGroups / 8;   // 5
constexpr int kLoTile = kTok * 8;              // fp32 lo of one (token tile, K step): 512 chunks (8 KB)

// ---------------------------------------------------------------------------
// P1: down projection partials and sums of squares.  Workgroup b: split
// b % S of width 10240 / S (stream halves or quarters; with S = 8 the split is
// the XCD's, with S = 16 each XCD owns two), token tile b / S of 128 tokens.
// The 12 waves specialise (wave w runs on SIMD w % 4, so each SIMD holds two
// matrix waves and one producer): the vector work of the producers overlaps
// the matrix cores instead of adding to them, and two matrix waves per SIMD
// keep its matrix core issuing.
//  * matrix waves 0-7: wave m computes rows 160 (m % 2) .. +159 for tokens
//    32 (m / 2) .. +31: MFMA A = W_down rows (10 blocks of 16), B = the y
//    panels of its two token blocks; it reads LDS and issues MFMAs only.
//  * producer waves 8-11: issue every load (the W_down panel of a step one step
//    ahead, raw R and pending three steps ahead, the split's w_norm once) and
//    turn the raw activations of the next step into y = R' * w_norm, split
//    exactly into three bf16 panels, with the tokens' sums of squares.
// LDS: 2 W_down slots (20 KB), 2 y slots (3 panels of 128 rows, 24 KB), raw
// slots of 128 rows x 32 floats for R and pending (16 KB each; 3 slots, or 2
// with pending, which then arrive two steps ahead), w_norm.
// Raw rows: chunk c of row r at slot c ^ swz8(r) of its 128-byte line.
// ---------------------------------------------------------------------------
constexpr int kDnTok = 128;
constexpr int kDnWaves = 12;
constexpr int kDnMatrixWaves = 8;
constexpr int kDnWChunks = kRank * 4;           // W_down panel: 1280 chunks (20 KB)
constexpr int kDnRawChunks = kDnTok * 8;        // raw R (or pending) of a step: 1024 chunks (16 KB)
constexpr int kDnYChunks = 3 * kDnTok * 4;      // y: 3 panels of 128 rows x 4 chunks (24 KB)

template <int S, bool HAS_P>
__global__ __launch_bounds__(kDnWaves * 64) void prefill_down(int T, const float* __restrict__ R,
                                                              const float* __restrict__ P,
                                                              const float* __restrict__ w_norm,
                                                              const uint16_t* __restrict__ W_down,
                                                              float* __restrict__ part, float* __restrict__ ssq)
{
    constexpr int SW = kD / S;              // columns of a split
    constexpr int NS = SW / kKs;            // K steps
    constexpr int RS = HAS_P ? 2 : 3;       // raw slots (pending doubles each; 3 would not fit in LDS)
    constexpr int kRawSet = (HAS_P ? 2 : 1) * kDnRawChunks;
    constexpr int kWOff = 0;
    constexpr int kYOff = 2 * kDnWChunks;
    constexpr int kRawOff = kYOff + 2 * kDnYChunks;
    constexpr int kNormOff = kRawOff + RS * kRawSet;
    constexpr int kLdsChunks = kNormOff + SW / 4;
    // raw-load wave instructions per step and producer wave (16 per array, 4
    // waves), and how many of them a step's closing wait may leave in flight
    constexpr int kRawLoads = (HAS_P ? 2 : 1) * (kDnRawChunks / 64) / 4;
    constexpr int kFly = RS == 3 ? kRawLoads : 0;
    static_assert(SW % kKs == 0 && NS >= 4, "tiling");
    static_assert(kLdsChunks * 16 <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint4 lds[kLdsChunks];

    const int b = blockIdx.x;
    const int sig = b % S;
    const int t0 = (b / S) * kDnTok;
    const int kbase = sig * SW;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const uint32_t lds0 = lds_addr(lds);

    if (wave >= kDnMatrixWaves) {
        // =========================== producer ===========================
        const int pw = wave - kDnMatrixWaves;
        // W_down panel: wave instruction q (0..19) fills panel rows 16 q .. +15
        // (lane l: row 16 q + l / 4, chunk (l & 3) ^ ((row >> 1) & 3)); wave pw
        // issues q = pw + 4 k, k < 5.
        const int dchunk = (lane & 3) ^ ((lane >> 3) & 3);
        const uint16_t* wd_lane = W_down + (size_t)(lane >> 2) * kD + kbase + 8 * dchunk;
        // raw: wave instruction q (0..15) fills rows 8 q .. 8 q + 7 (lane l: row
        // 8 q + l / 8, chunk (l & 7) ^ swz8(row)); wave pw issues q = pw + 4 k,
        // k < 4.  Rows past T re-read row T - 1 (their results are never stored).
        const float* rraw[4];
        const float* praw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = pw + 4 * k;
            const int row = 8 * q + (lane >> 3);
            const int tr = t0 + row < T ? t0 + row : T - 1;
            const int ch = (lane & 7) ^ swz8(row);
            rraw[k] = R + (size_t)tr * kD + kbase + 4 * ch;
            praw[k] = HAS_P ? P + (size_t)tr * kD + kbase + 4 * ch : nullptr;
        }
        auto issue_w = [&](int ks) {
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                const int q = pw + 4 * k;
                dma16(wd_lane + (size_t)(16 * q) * kD + kKs * ks, lds + kWOff + (ks & 1) * kDnWChunks + 64 * q);
            }
        };
        auto issue_raw = [&](int ks) {
            const int slot = ks % RS;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int q = pw + 4 * k;
                dma16(rraw[k] + kKs * ks, lds + kRawOff + slot * kRawSet + 64 * q);
                if (HAS_P)
                    dma16(praw[k] + kKs * ks, lds + kRawOff + slot * kRawSet + kDnRawChunks + 64 * q);
            }
        };
        // conversion role: token row cr = (64 pw + lane) / 2, columns 16 h .. 16 h + 15
        const int cr = (64 * pw + lane) >> 1, h = lane & 1;
        const bool tok_ok = t0 + cr < T;
        float ssacc = 0.f;
        auto convert = [&](int ks) {
            const uint32_t rb = lds0 + 16 * (kRawOff + (ks % RS) * kRawSet + 8 * cr);
            u32x4 v[12];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                v[c] = ds_read16(rb + 16 * ((4 * h + c) ^ swz8(cr)));
                if (HAS_P)
                    v[4 + c] = ds_read16(rb + 16 * kDnRawChunks + 16 * ((4 * h + c) ^ swz8(cr)));
                v[8 + c] = ds_read16(lds0 + 16 * (kNormOff + 8 * ks + 4 * h + c));  // w_norm[32 ks + 16 h + 4 c ..]
            }
            lds_wait(v);
            uint32_t hi[16], mi[16], lo[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = __uint_as_float(v[e >> 2][e & 3]);
                if (HAS_P)
                    x += __uint_as_float(v[4 + (e >> 2)][e & 3]);
                ssacc += x * x;
                split3(x * __uint_as_float(v[8 + (e >> 2)][e & 3]), hi[e], mi[e], lo[e]);
            }
            // panel chunks 2 h and 2 h + 1 of row cr, in each of the 3 panels
            const uint32_t yb = lds0 + 16 * (kYOff + (ks & 1) * kDnYChunks);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t a = yb + 16 * panel_slot(cr, 2 * h + c);
                const int e = 8 * c;
                ds_write16(a, u32x4{hi[e] | (hi[e + 1] << 16), hi[e + 2] | (hi[e + 3] << 16),
                                    hi[e + 4] | (hi[e + 5] << 16), hi[e + 6] | (hi[e + 7] << 16)});
                ds_write16(a + 16 * kDnTok * 4, u32x4{mi[e] | (mi[e + 1] << 16), mi[e + 2] | (mi[e + 3] << 16),
                                                      mi[e + 4] | (mi[e + 5] << 16), mi[e + 6] | (mi[e + 7] << 16)});
                ds_write16(a + 32 * kDnTok * 4, u32x4{lo[e] | (lo[e + 1] << 16), lo[e + 2] | (lo[e + 3] << 16),
                                                      lo[e + 4] | (lo[e + 5] << 16), lo[e + 6] | (lo[e + 7] << 16)});
            }
        };
        // Schedule: raw of step k is issued at step k - RS (prologue for the
        // first RS steps), W_down of step k at step k - 1; step k's raw is
        // converted during step k - 1.  With 3 raw slots the wait ending step j
        // may leave the raw issued at step j in flight (it is converted two
        // steps later); with 2 slots it is converted at the next step and every
        // wait drains.
        issue_w(0);
        // the split's w_norm: SW / 4 chunks, wave instructions pw, pw + 4, ..
#pragma unroll
        for (int k = 0; k < (SW / 4 + 255) / 256; ++k)
            if (64 * (pw + 4 * k) + lane < SW / 4)
                dma16(w_norm + kbase + 4 * (64 * (pw + 4 * k) + lane), lds + kNormOff + 64 * (pw + 4 * k));
#pragma unroll
        for (int k = 0; k < RS - 1; ++k)
            issue_raw(k);
        order();
        issue_raw(RS - 1);
        ring_barrier<kRawLoads>();      // B0: W(0), w_norm, raw(0..RS-2) landed
        convert(0);
        ring_barrier<kFly>();           // B1: y(0) staged (and raw(1) landed when RS == 2)
#pragma unroll 1
        for (int j = 0; j < NS; ++j) {  // barrier B(j + 2) ends step j
            if (j + 1 < NS)
                issue_w(j + 1);
            order();
            const bool more = j + RS < NS;
            if (more)
                issue_raw(j + RS);       // into the slot of step j (converted during step j - 1)
            if (j + 1 < NS)
                convert(j + 1);
            if (more)
                ring_barrier<kFly>();
            else
                ring_barrier<0>();
        }
        // sums of squares: lanes 2 i and 2 i + 1 hold the two halves of token cr
        const float ss = ssacc + __shfl_xor(ssacc, 1);
        if (h == 0 && tok_ok)
            ssq[(size_t)sig * T + t0 + cr] = ss;
        return;
    }

    // ============================= matrix =============================
    // wave m computes rows 160 (m % 2) .. +159 for tokens 32 (m / 2) .. +31:
    // per K step it reads 10 KB of W_down and 6 KB of y from LDS (a 16-token x
    // 320-row tile would read 23 KB), for the same 60 MFMAs
    const int m = wave;
    const int rh = m & 1, tq = m >> 1;
    const int n = lane & 15, g = lane >> 4;
    f32x4_t acc[10][2];
#pragma unroll
    for (int jb = 0; jb < 10; ++jb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            acc[jb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // operands: W_down row block 10 rh + jb = this lane's slot in block 0 plus
    // 1 KB per block; y of token 32 tq + 16 tb + n, chunk g, panel p (a 16-row
    // block further is 1 KB further: the panel swizzle repeats every 8 rows)
    const uint32_t aoff = 16 * panel_slot(n, g) + 10240 * rh;
    const uint32_t yoff = 16 * panel_slot(32 * tq + n, g);
    auto compute = [&](int ks) {
        const uint32_t wb = lds0 + 16 * (kWOff + (ks & 1) * kDnWChunks) + aoff;
        const uint32_t yb = lds0 + 16 * (kYOff + (ks & 1) * kDnYChunks) + yoff;
        u32x4 y[3][2];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            y[p][0] = ds_read16(yb + 16 * kDnTok * 4 * p);
            y[p][1] = ds_read16(yb + 16 * kDnTok * 4 * p + 1024);
        }
        u32x4 wa[5];
        wa[0] = ds_read16_off<0>(wb);
        wa[1] = ds_read16_off<1024>(wb);
        wa[2] = ds_read16_off<2048>(wb);
        wa[3] = ds_read16_off<3072>(wb);
        wa[4] = ds_read16_off<4096>(wb);
        asm volatile("s_waitcnt lgkmcnt(5)" ::: "memory");
#pragma unroll
        for (int p = 0; p < 3; ++p) {
            asm volatile("" : "+v"(y[p][0]));
            asm volatile("" : "+v"(y[p][1]));
        }
        // 2 groups of 5 row blocks: the second group's operands are read
        // while the first group's 30 MFMAs run
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            u32x4 wn[5];
            if (grp == 0) {
                const uint32_t wg = wb + 5120;
                wn[0] = ds_read16_off<0>(wg);
                wn[1] = ds_read16_off<1024>(wg);
                wn[2] = ds_read16_off<2048>(wg);
                wn[3] = ds_read16_off<3072>(wg);
                wn[4] = ds_read16_off<4096>(wg);
                asm volatile("s_waitcnt lgkmcnt(5)" ::: "memory");
            } else {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
#pragma unroll
            for (int jb = 0; jb < 5; ++jb)
                asm volatile("" : "+v"(wa[jb]));
#pragma unroll
            for (int p = 2; p >= 0; --p)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int jb = 0; jb < 5; ++jb)
                        acc[5 * grp + jb][tb] = mfma16(wa[jb], y[p][tb], acc[5 * grp + jb][tb]);
            if (grp == 0) {
#pragma unroll
                for (int jb = 0; jb < 5; ++jb)
                    wa[jb] = wn[jb];
            }
        }
    };
    ring_barrier<0>();  // B0
    ring_barrier<0>();  // B1: y(0) and W(0) in LDS
#pragma unroll 1
    for (int j = 0; j < NS; ++j) {
        compute(j);
        ring_barrier<0>();  // B(j + 2)
    }
    // partials: lane holds tokens t0 + 32 tq + 16 tb + n, rows 160 rh + 16 jb
    // + 4 g .. +3
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = t0 + 32 * tq + 16 * tb + n;
        if (t < T) {
            float* dst = part + ((size_t)sig * T + t) * kRank + 160 * rh + 4 * g;
#pragma unroll
            for (int jb = 0; jb < 10; ++jb)
                *reinterpret_cast<f32x4_t*>(dst + 16 * jb) = acc[jb][tb];
        }
    }
}

// ---------------------------------------------------------------------------
// P1 for short chunks (at most kSmMaxTok tokens; 80 splits of 128 columns).
// The 128-token kernel above needs one memory latency per K step and runs 80
// workgroups for such chunks; this one issues every load at entry and spreads
// the chunk over 80 x NT workgroups.  Workgroup b = 8 i + x (XCD x) takes
// split 10 x + i / NT and token tile i % NT of TT tokens: the NT tiles of a
// split are dispatched together on one XCD, so its 80 KB W_down slice comes
// from memory once.
//  * loads: the tile's R (+ pending) and w_norm columns into registers, then
//    the whole W_down slice (320 rows x 128 columns) into LDS as whole
//    128-byte lines, the first line of every row (K steps 0-1) before the
//    second (K steps 2-3): [2 lines][320 rows][8 chunks], chunk c of a line
//    at slot c ^ swz8(row);
//  * y = R' * w_norm split into 3 bf16 planes [3][TT tokens][16 chunks] in LDS
//    (chunk j of token r at line_pos16(r, j)) with the tokens' sums of
//    squares, while the slice lands;
//  * 8 waves of MFMAs: wave w takes tokens 16 (w % NTH) .. +15 and rows
//    RW (w / NTH) .. +RW-1 (NTH = TT / 16 token groups, RW = 320 NTH / 8),
//    A = W_down rows, B = one y plane per piece: K steps 0-1 once the first
//    lines have landed, 2-3 after the second; lane (n, g) ends with rows
//    4 g .. 4 g + 3 of each 16-row block for token n in three accumulators
//    and stores hi + (mid + lo3) as partial dots, block by block while the
//    next block's products run.
// ---------------------------------------------------------------------------
constexpr int kSmSplits = 80;
constexpr int kSmCols = kD / kSmSplits;     // 128
constexpr int kSmRowChunks = kSmCols / 8;   // 16 chunks of 8 bf16 per row
constexpr int kSmWChunks = kRank * kSmRowChunks;  // 5120 (80 KB)
constexpr int kSmMaxTok = 192;

// Position (in chunks) of chunk j (0..15) of row r in a block of 16-chunk
// rows: chunks are swizzled inside their 128-byte line and odd rows swap the
// two lines, so 8 lanes reading chunk j of 8 consecutive rows hit 8 distinct
// 16-byte bank groups.
__host__ __device__ constexpr int line_pos16(int r, int j)
{
    return 16 * r + 8 * ((j >> 3) ^ (r & 1)) + ((j & 7) ^ swz8(r));
}

template <int TT, bool HAS_P>
__global__ __launch_bounds__(512) void prefill_down_small(int T, const float* __restrict__ R,
                                                          const float* __restrict__ P,
                                                          const float* __restrict__ w_norm,
                                                          const uint16_t* __restrict__ W_down,
                                                          float* __restrict__ part, float* __restrict__ ssq)
{
    constexpr int NTH = TT / 16;           // token groups of 16
    constexpr int RW = kRank * NTH / 8;    // rows per wave
    constexpr int MB = RW / 16;            // 16-row blocks per wave
    constexpr int NPASS = TT * kSmRowChunks / 512;  // conversion items per thread
    constexpr int kYChunks = TT * kSmRowChunks;     // one y plane
    static_assert((TT == 32 || TT == 64) && RW % 16 == 0 && NPASS >= 1, "tiling");
    static_assert(kSmWChunks % (8 * 64) == 0, "W slice: whole wave instructions per wave");
    __shared__ __align__(16) uint4 lds[kSmWChunks + 3 * kYChunks];
    const uint32_t w_lds = lds_addr(lds), y_lds = w_lds + 16 * kSmWChunks;

    const int nt = gridDim.x / kSmSplits;
    const int b = blockIdx.x, x = b & 7, i = b >> 3;
    const int sig = 10 * x + i / nt, t0 = (i % nt) * TT;
    const int kbase = kSmCols * sig;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // (1) R (+ pending) and w_norm of item it = tid + 512 k: token it / 16,
    //     columns 8 (it % 16) .. +7 (tokens past T re-read token T - 1)
    float4 rv[NPASS][2], pv[NPASS][2], wv[2];
    const int c = tid & 15;
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
        const int tl = (tid >> 4) + 32 * k;
        const int t = t0 + tl < T ? t0 + tl : T - 1;
        const float* rp = R + (size_t)t * kD + kbase + 8 * c;
        rv[k][0] = *reinterpret_cast<const float4*>(rp);
        rv[k][1] = *reinterpret_cast<const float4*>(rp + 4);
        if constexpr (HAS_P) {
            const float* pp = P + (size_t)t * kD + kbase + 8 * c;
            pv[k][0] = *reinterpret_cast<const float4*>(pp);
            pv[k][1] = *reinterpret_cast<const float4*>(pp + 4);
        }
    }
    wv[0] = *reinterpret_cast<const float4*>(w_norm + kbase + 8 * c);
    wv[1] = *reinterpret_cast<const float4*>(w_norm + kbase + 8 * c + 4);
    // (2) the W_down slice: wave instruction q (0..79) fills LDS positions
    //     64 q .. 64 q + 63, i.e. line q / 40 of rows 8 (q % 40) .. +7; eight
    //     consecutive lanes fetch one whole line.  Each wave issues its five
    //     first-line instructions (k < 5) before its second-line ones.
    __builtin_amdgcn_sched_barrier(0);
    {
        const __amdgpu_buffer_rsrc_t wr = rsrc_of(W_down);
#pragma unroll
        for (int k = 0; k < kSmWChunks / 512; ++k) {
            const int q = wave + 8 * k;
            const int ln = q / 40, row = 8 * (q - 40 * ln) + (lane >> 3);
            const int j = 8 * ln + ((lane & 7) ^ swz8(row));
            bdma16(wr, lds + 64 * q, 2u * ((uint32_t)row * kD + kbase + 8 * j), 0);
        }
    }
    // (3) y planes and sums of squares (LDS stores as inline asm: the
    //     compiler would make them wait for the slice's loads)
    float ssk[NPASS];
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
        const int tl = (tid >> 4) + 32 * k;
        const float rr[8] = {rv[k][0].x, rv[k][0].y, rv[k][0].z, rv[k][0].w,
                             rv[k][1].x, rv[k][1].y, rv[k][1].z, rv[k][1].w};
        const float ww[8] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w};
        float pr[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (HAS_P) {
            const float q8[8] = {pv[k][0].x, pv[k][0].y, pv[k][0].z, pv[k][0].w,
                                 pv[k][1].x, pv[k][1].y, pv[k][1].z, pv[k][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pr[e] = q8[e];
        }
        float ss = 0.f;
        uint32_t hi[8], mi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = HAS_P ? rr[e] + pr[e] : rr[e];
            ss += xv * xv;
            split3(xv * ww[e], hi[e], mi[e], lo[e]);
        }
        const uint32_t a = y_lds + 16 * line_pos16(tl, c);
        ds_write16(a, u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)});
        ds_write16(a + 16 * kYChunks,
                   u32x4{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16)});
        ds_write16(a + 32 * kYChunks,
                   u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)});
        // the token's 16 lanes (one 16-lane row of the wave) combine theirs
        ss += __shfl_xor(ss, 8, 16);
        ss += __shfl_xor(ss, 4, 16);
        ss += __shfl_xor(ss, 2, 16);
        ss += __shfl_xor(ss, 1, 16);
        ssk[k] = ss;  // (stored at the end: no store may sit among the loads the waits count)
    }
    ring_barrier<kSmWChunks / 1024>();  // y planes and every wave's first lines in LDS

    // (4) products: wave w, tokens 16 th + n, rows RW rg + 16 mb + 4 g ..
    const int th = wave % NTH, rg = wave / NTH;
    const int n = lane & 15, g = lane >> 4;
    f32x4_t acc[MB][3];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
            acc[mb][pc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto w_at = [&](int row, int j) { return w_lds + 16 * ((j >> 3) * (kRank * 8) + 8 * row + ((j & 7) ^ swz8(row))); };
    auto y_at = [&](int pc, int j) { return y_lds + 16 * (pc * kYChunks + line_pos16(16 * th + n, j)); };
    // K steps 0-1 (the first lines)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int j = 4 * ks + g;
        u32x4 a[MB], bb[3];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            a[mb] = ds_read16(w_at(RW * rg + 16 * mb + n, j));
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
            bb[pc] = ds_read16(y_at(pc, j));
        lds_wait(a);
        lds_wait(bb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int pc = 0; pc < 3; ++pc)
                acc[mb][pc] = mfma16(a[mb], bb[pc], acc[mb][pc]);
    }
    ring_barrier<0>();  // every wave's second lines in LDS
    // K steps 2-3, block by block; the partial dots of the blocks before
    // block mb are stored (written through, sc1: they drain while other
    // workgroups compute instead of all at the end of the launch from the
    // L2s) while block mb's products run.  Two blocks that make up a token's
    // 128-byte line (blocks mb, mb + 1 with mb - ps even) are stored as whole
    // lines: lanes n and n ^ 8 (DPP row_ror:8) trade halves, so one store
    // instruction writes 8 tokens x 128 bytes instead of 16 tokens x 64.
    const int t = t0 + 16 * th + n;
    const __amdgpu_buffer_rsrc_t prs = rsrc_of(part);
    const uint32_t dst = 4u * (uint32_t)(((size_t)sig * T + (t < T ? t : 0)) * kRank + RW * rg + 4 * g);
    const int ta = t0 + 16 * th + (n & 7), tb = ta + 8;  // the tokens of a lane's two whole-line stores
    const uint32_t dsta = 4u * (uint32_t)(((size_t)sig * T + (ta < T ? ta : 0)) * kRank + RW * rg + 4 * g);
    const uint32_t dstb = 4u * (uint32_t)(((size_t)sig * T + (tb < T ? tb : 0)) * kRank + RW * rg + 4 * g);
    const int ps = ((RW * rg) >> 4) & 1;  // parity of the first block that starts a 128-byte line
    auto block_sum = [&](int mb) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = acc[mb][0][e] + (acc[mb][1][e] + acc[mb][2][e]);
        return v;
    };
    auto store_single = [&](int mb) {
        const f32x4_t v = block_sum(mb);
        if (t < T)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs, dst + 64u * mb, 0, 16 /* sc1 */);
    };
    auto store_pair = [&](int mb) {
        const f32x4_t va = block_sum(mb), vb = block_sum(mb + 1);
        const bool low = n < 8;
        f32x4_t s1, s2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = low ? vb[e] : va[e];  // the half the partner lane stores
            const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, true));
            s1[e] = low ? va[e] : y;  // token ta: block mb (lanes n < 8), block mb + 1 (n >= 8)
            s2[e] = low ? y : vb[e];  // token tb: likewise
        }
        const uint32_t half = low ? 0u : 64u;
        if (ta < T)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s1), prs, dsta + 64u * mb + half, 0, 16);
        if (tb < T)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s2), prs, dstb + 64u * mb + half, 0, 16);
    };
    // stores what block p completes: nothing if it starts a line (its partner
    // follows), the pair if it ends one, else the block alone
    auto flush = [&](int p) {
        const bool second = ((p - ps) & 1) != 0 && p >= 1;
        const bool first = ((p - ps) & 1) == 0 && p + 1 < MB;
        if (second)
            store_pair(p - 1);
        else if (!first)
            store_single(p);
    };
    u32x4 b2[2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
            b2[h][pc] = ds_read16(y_at(pc, 4 * (2 + h) + g));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        u32x4 a2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a2[h] = ds_read16(w_at(RW * rg + 16 * mb + n, 4 * (2 + h) + g));
        lds_wait(a2);
        if (mb == 0) {
            lds_wait(b2[0]);
            lds_wait(b2[1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int pc = 0; pc < 3; ++pc)
                acc[mb][pc] = mfma16(a2[h], b2[h][pc], acc[mb][pc]);
        if (mb > 0)
            flush(mb - 1);
    }
    flush(MB - 1);
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
        const int tl = (tid >> 4) + 32 * k;
        if (c == 0 && t0 + tl < T)
            ssq[(size_t)sig * T + t0 + tl] = ssk[k];
    }
}

// ---------------------------------------------------------------------------
// P2: lo = sum_s rs_s * stream partial (fp32), in the tiled layout P3 copies
// into LDS verbatim: for token tile u (64 tokens) and K step ks, 64 rows of 32
// floats (8 KB) at chunk (u * 10 + ks) * 512; chunk c of row r at slot
// c ^ swz8(r) of its 128-byte line.  Tokens of the last tile past T get zeros.
// ---------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(256) void prefill_lo(int T, int Tpad, const float* __restrict__ part,
                                                  const float* __restrict__ ssq, uint4* __restrict__ lo_tiled)
{
    constexpr int Q = S / 4;  // splits per stream
    auto store = [&](int t, int c4, const float (&lo)[4]) {
        const int tile = t / kTok, tl = t - tile * kTok;
        const int ks = c4 >> 3, c = c4 & 7;
        lo_tiled[(size_t)(tile * kUpSteps + ks) * kLoTile + 8 * tl + (c ^ swz8(tl))] =
            make_uint4(__float_as_uint(lo[0]), __float_as_uint(lo[1]), __float_as_uint(lo[2]), __float_as_uint(lo[3]));
    };
    if constexpr (S == 80) {
        // 80 splits (short chunks, latency-bound): one wave per (token, block
        // rb of 32 rank indices).  Lane (s, h, c) sums partials 10 h .. 10 h +
        // 9 of stream s for rank indices 4 (8 rb + c) .. +3, so the eight lanes
        // of a (stream, half) read one whole 128-byte line of each partial row;
        // the halves are combined, then the streams as (s0 + s1) + (s2 + s3).
        // (16 lanes per item reading half lines took 1.2 us longer at 64
        // tokens.)
        const int wv = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
        const int t = wv / (kRank / 32), rb = wv - t * (kRank / 32);
        if (t >= Tpad)  // (whole waves)
            return;
        const int ln = threadIdx.x & 63, c = ln & 7, h = (ln >> 3) & 1, s = ln >> 4;
        const int c4 = 8 * rb + c;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < T) {
            float ss = 0.f, sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < Q / 2; ++q) {
                const int sg = Q * s + (Q / 2) * h + q;
                ss += ssq[(size_t)sg * T + t];
                const float4 a = *reinterpret_cast<const float4*>(part + ((size_t)sg * T + t) * kRank + 4 * c4);
                sum[0] += a.x;
                sum[1] += a.y;
                sum[2] += a.z;
                sum[3] += a.w;
            }
            // h0 + h1, the same bits in both halves' lanes
            ss += __shfl_xor(ss, 8);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sum[e] += __shfl_xor(sum[e], 8);
            const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = sum[e] * rs;
        }
        float lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = v[e] + __shfl_xor(v[e], 16);
            lo[e] = a + __shfl_xor(a, 32);
        }
        if (ln < 8)
            store(t, c4, lo);
        return;
    }
    // 32 splits: four lanes per (token, chunk of 4 rank indices), lane s
    // summing the Q partials of stream s, the streams combined in registers.
    // Coarse splits (long chunks, bandwidth-bound): one lane sums all four
    // streams.
    constexpr int L = S >= 32 ? 4 : 1;
    const int idx = (blockIdx.x * 256 + threadIdx.x) / L;
    const int t = idx / (kRank / 4);
    const int c4 = idx - t * (kRank / 4);
    if (t >= Tpad)  // (whole lane groups: Tpad * 80 groups fill whole waves)
        return;
    float lo[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (L == 4) {
        const int s = threadIdx.x & 3;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < T) {
            float ss = 0.f, sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int sg = Q * s + q;
                ss += ssq[(size_t)sg * T + t];
                const float4 a = *reinterpret_cast<const float4*>(part + ((size_t)sg * T + t) * kRank + 4 * c4);
                sum[0] += a.x;
                sum[1] += a.y;
                sum[2] += a.z;
                sum[3] += a.w;
            }
            const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = sum[e] * rs;
        }
        // (v0 + v1) + (v2 + v3), the same bits in all four lanes
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = v[e] + __shfl_xor(v[e], 1);
            lo[e] = a + __shfl_xor(a, 2);
        }
        if ((threadIdx.x & 3) != 0)
            return;
    } else if (t < T) {
        float v[4][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float ss = 0.f, sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int sg = Q * s + q;
                ss += ssq[(size_t)sg * T + t];
                const float4 a = *reinterpret_cast<const float4*>(part + ((size_t)sg * T + t) * kRank + 4 * c4);
                sum[0] += a.x;
                sum[1] += a.y;
                sum[2] += a.z;
                sum[3] += a.w;
            }
            const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[s][e] = sum[e] * rs;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            lo[e] = (v[0][e] + v[1][e]) + (v[2][e] + v[3][e]);
    }
    store(t, c4, lo);
}

// ---------------------------------------------------------------------------
// P3 for chunks of at most 4 token tiles: up projection with the stream mix
// as its epilogue on tiles of 64 tokens x 16 CB columns x 4 streams, 160 / CB
// workgroups per token tile, each streaming a part of a 64-column W_up
// panel, so a short read loads W_up over most of the chip (CB = 1 for one or
// two token tiles, 2 for three or four).  Workgroup b: XCD x = b % 8, q = b /
// 8: token tile q / G, column group x + 8 (q % G), G = 20 / CB.  Wave w owns
// tokens 16 w .. 16 w + 15 of the tile: MFMA A = W_up rows (4 streams), B =
// lo of the wave's tokens, split in registers into its three bf16 pieces.  D
// then holds, in lane (n, g), token 16 w + n and columns 16 cb + 4 g .. +3 of
// every stream, so the mix is per lane.  LDS stage: the W_up panel (64 CB
// rows: row 16 CB s + j = W_up row s * 2560 + c0 + j, 4 CB KB), then the
// tile's lo block of the step (8 KB).  NS stages, loaded NS - 1 steps ahead
// (each step's work is short next to a memory latency): 3 ahead for a chunk
// of one token tile, 4 for two, 2 for three and 3 for four.  (Measured at 33
// and 64 tokens: all 10 steps loaded at entry is 1 us slower than 3 ahead.)
// ---------------------------------------------------------------------------

// Calls f(std::integral_constant<int, K>) for K = K0 .. K0 + N - 1.
template <int K0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (N > 0) {
        f(std::integral_constant<int, K0>{});
        static_for<K0 + 1, N - 1>(f);
    }
}

template <bool HAS_P, bool BF16_LO, int NS, int CB>
__global__ __launch_bounds__(256, 2) void prefill_upmix(int T, const uint4* __restrict__ lo_tiled,
                                                        const uint16_t* __restrict__ W_up,
                                                        const float* R,
                                                        const float* __restrict__ P,
                                                        float* __restrict__ out_mixed,
                                                        uint16_t* __restrict__ out_bf16,
                                                        uint16_t* __restrict__ out_fp16,
                                                        float* R_commit)
{
    constexpr int kCols = 16 * CB;                      // output columns of the tile
    constexpr int kGpx = kWidth / kCols / 8;            // column groups per XCD (20 / CB)
    constexpr int kUpWChunks = 4 * kCols * 4;           // W_up panel: 256 CB chunks
    constexpr int kUpStage = kUpWChunks + kLoTile;      // 256 CB + 512 chunks
    constexpr int kUpLoads = kUpStage / 64 / 4;         // wave instructions per stage and wave (2 + CB)
    constexpr int NB = 2 * CB;                          // panel blocks of two streams
    static_assert(NS >= 3 && NS <= kUpSteps && (CB == 1 || CB == 2), "stages, column blocks");
    __shared__ __align__(16) uint4 lds[NS * kUpStage];

    const int b = blockIdx.x;
    const int x = b & 7, q = b >> 3;
    const int tile = q / kGpx;
    const int cg = x + 8 * (q - tile * kGpx);
    const int t0 = tile * kTok, c0 = cg * kCols;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;

    // stage loads: W_up panel instruction i (0..15) fills rows 16 i .. 16 i + 15
    // (lane l: row 16 i + l / 4, chunk (l & 3) ^ ((row >> 1) & 3)); lo
    // instruction i (0..7) copies 1 KB of the lo block.  Wave w issues W_up
    // i = w + 4 k (k < 4) and lo i = w, w + 4.
    const int wchunk = (lane & 3) ^ ((lane >> 3) & 3);
    const uint16_t* wu_lane[CB];
#pragma unroll
    for (int k = 0; k < CB; ++k) {
        const int prow = 16 * (wave + 4 * k) + (lane >> 2);  // panel row = kCols s + j
        wu_lane[k] = W_up + (size_t)((prow / kCols) * kWidth + c0 + (prow % kCols)) * kRank + 8 * wchunk;
    }
    const uint4* lo_lane = lo_tiled + (size_t)tile * kUpSteps * kLoTile + lane;
    auto issue = [&](int ks, int slot) {
        uint4* sb = lds + slot * kUpStage;
#pragma unroll
        for (int k = 0; k < CB; ++k)
            dma16(wu_lane[k] + kKs * ks, sb + 64 * (wave + 4 * k));
#pragma unroll
        for (int k = 0; k < 2; ++k)
            dma16(lo_lane + (size_t)ks * kLoTile + 64 * (wave + 4 * k), sb + kUpWChunks + 64 * (wave + 4 * k));
    };

    f32x4_t acc[CB][4];  // [column block][stream]
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[cb][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t lds0 = lds_addr(lds);
    // W_up operand of (stream s, column block cb): panel row 64 s + 16 cb + n,
    // chunk g = this lane's slot in the first block plus 1 KB per block
    const uint32_t aoff = 16 * panel_slot(n, g);
    // lo of token 16 wave + n, floats 8 g .. 8 g + 7
    const int lrow = 16 * wave + n;
    const uint32_t lo_a = 16 * (kUpWChunks + 8 * lrow + ((2 * g) ^ swz8(lrow)));
    const uint32_t lo_b = 16 * (kUpWChunks + 8 * lrow + ((2 * g + 1) ^ swz8(lrow)));
    auto compute = [&](int slot) {
        const uint32_t sb = lds0 + 16 * slot * kUpStage;
        u32x4 lv[2];
        lv[0] = ds_read16(sb + lo_a);
        lv[1] = ds_read16(sb + lo_b);
        u32x4 wa[NB];
        const uint32_t wb = sb + aoff;
        static_for<0, NB>([&](auto kc) { constexpr int k = decltype(kc)::value; wa[k] = ds_read16_off<1024 * k>(wb); });
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NB) : "memory");
        asm volatile("" : "+v"(lv[0]), "+v"(lv[1]));
        uint32_t hi[8], mi[8] = {}, l3[8] = {};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (BF16_LO)  // the fast mode: lo rounded to bf16 (nearest even), one piece
                hi[e] = __builtin_bit_cast(uint16_t, (__bf16)__uint_as_float(lv[e >> 2][e & 3]));
            else
                split3(__uint_as_float(lv[e >> 2][e & 3]), hi[e], mi[e], l3[e]);
        }
        u32x4 y[3];
        y[0] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
        y[1] = u32x4{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16)};
        y[2] = u32x4{l3[0] | (l3[1] << 16), l3[2] | (l3[3] << 16), l3[4] | (l3[5] << 16), l3[6] | (l3[7] << 16)};
        // streams 0-1 (column blocks 0..3) then streams 2-3: the second half's
        // W_up operands are read while the first half's 24 MFMAs run
        u32x4 wn[NB];
        static_for<0, NB>([&](auto kc) { constexpr int k = decltype(kc)::value; wn[k] = ds_read16_off<1024 * (NB + k)>(wb); });
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NB) : "memory");
#pragma unroll
        for (int k = 0; k < NB; ++k)
            asm volatile("" : "+v"(wa[k]));
        // panel block index k = CB s + cb
#pragma unroll
        for (int p = BF16_LO ? 0 : 2; p >= 0; --p)
#pragma unroll
            for (int k = 0; k < NB; ++k)
                acc[k % CB][k / CB] = mfma16(wa[k], y[p], acc[k % CB][k / CB]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int k = 0; k < NB; ++k)
            asm volatile("" : "+v"(wn[k]));
#pragma unroll
        for (int p = BF16_LO ? 0 : 2; p >= 0; --p)
#pragma unroll
            for (int k = 0; k < NB; ++k)
                acc[k % CB][2 + k / CB] = mfma16(wn[k], y[p], acc[k % CB][2 + k / CB]);
    };

    // The epilogue's R: this lane's token, columns c0 + 16 cb + 4 g .. +3 of
    // every stream (tokens past T re-read token T - 1 and store nothing).
    // Its loads are issued right after the last stage's loads and are
    // counted in the waits that follow.
    constexpr int kRLoads = 4 * CB;
    const int t = t0 + lrow;
    const int tr = t < T ? t : T - 1;
    const float* rrow = R + (size_t)tr * kD + c0 + 4 * g;
    float4 rv[CB][4];  // [column block][stream]

    // Stage k goes into slot k % NS.  Stages 0 .. NS - 2 are issued first;
    // step ks waits for its stage (and for every wave to be done with step
    // ks - 1), issues stage ks + NS - 1 into the slot step ks - 1 used, then
    // runs its MFMAs.  After the last stage come the epilogue's R loads.
    auto load_r = [&]() {
        // Loads through a pointer the compiler cannot trace to the read-only
        // argument: such loads count as ordinary memory accesses and stay
        // between the surrounding asm statements, where the waits count them.
        typedef __attribute__((address_space(1))) const f32x4_t gf32x4;  // global memory
        gf32x4* rl = (gf32x4*)rrow;  // (an address-space cast: the loads stay global loads)
        asm volatile("" : "+v"(rl));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4_t v = rl[(s * kWidth + 16 * cb) / 4];
                rv[cb][s] = make_float4(v[0], v[1], v[2], v[3]);
            }
    };
    static_for<0, NS - 1>([&](auto kc) { constexpr int k = decltype(kc)::value; issue(k, k); });
    static_for<0, kUpSteps>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        // this wave's loads issued after stage ks when the step starts: the
        // stages up to `last`, and the R loads (issued at step kUpSteps - NS)
        constexpr int last = ks + NS - 2 < kUpSteps - 1 ? ks + NS - 2 : kUpSteps - 1;
        constexpr int fly = (last - ks) * kUpLoads + (ks > kUpSteps - NS ? kRLoads : 0);
        ring_barrier<fly>();
        if constexpr (ks + NS - 1 < kUpSteps) {
            order();
            issue(ks + NS - 1, (ks + NS - 1) % NS);
            if constexpr (ks + NS - 1 == kUpSteps - 1) {
                order();
                load_r();
            }
        }
        compute(ks % NS);
    });
    // gated = up (identity epilogue); mixed = sum_s gated_s * R'_s, then images.
    if (HAS_P) {
        const float* prow = P + (size_t)tr * kD + c0 + 4 * g;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 pv = *reinterpret_cast<const float4*>(prow + s * kWidth + 16 * cb);
                rv[cb][s].x += pv.x;
                rv[cb][s].y += pv.y;
                rv[cb][s].z += pv.z;
                rv[cb][s].w += pv.w;
            }
        // the pending write committed: R' of this lane's token and columns
        // back into R (no other workgroup reads them in this chunk, and the
        // down projection of the chunk has finished)
        if (R_commit && t < T) {
            float* crow = R_commit + (size_t)t * kD + c0 + 4 * g;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    *reinterpret_cast<float4*>(crow + s * kWidth + 16 * cb) = rv[cb][s];
        }
    }
    // lane (n, g) holds token t, columns c0 + 16 cb + 4 g .. +3 of every
    // stream; the 4 lanes of a token store 64 contiguous bytes per block
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const float r[4][4] = {{rv[cb][0].x, rv[cb][0].y, rv[cb][0].z, rv[cb][0].w},
                               {rv[cb][1].x, rv[cb][1].y, rv[cb][1].z, rv[cb][1].w},
                               {rv[cb][2].x, rv[cb][2].y, rv[cb][2].z, rv[cb][2].w},
                               {rv[cb][3].x, rv[cb][3].y, rv[cb][3].z, rv[cb][3].w}};
        float m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m[i] = (acc[cb][0][i] * r[0][i] + acc[cb][1][i] * r[1][i]) + (acc[cb][2][i] * r[2][i] + acc[cb][3][i] * r[3][i]);
        if (t < T) {
            const size_t o = (size_t)t * kWidth + c0 + 16 * cb + 4 * g;
            *reinterpret_cast<float4*>(out_mixed + o) = make_float4(m[0], m[1], m[2], m[3]);
            uint32_t bh[4], hh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bh[i] = __builtin_bit_cast(uint16_t, (__bf16)m[i]);
                hh[i] = __builtin_bit_cast(uint16_t, (_Float16)m[i]);
            }
            *reinterpret_cast<uint2*>(out_bf16 + o) = make_uint2(bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16));
            *reinterpret_cast<uint2*>(out_fp16 + o) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
        }
    }
}

// ---------------------------------------------------------------------------
// P3 for chunks of more than 4 token tiles: one workgroup of 8 waves per CU
// takes 128 tokens (two token tiles) x 64 columns.  Waves 0-3 compute the
// first token tile, waves 4-7 the second, as above, so each W_up panel in
// LDS serves 128 tokens.  The ring holds five stages of 32 KB (the W_up
// panel, then the two tiles' lo blocks) loaded four steps ahead.  A wave
// reads the lo and the first four W_up operands of step ks + 1 at the end of
// step ks (stage ks + 1 has landed everywhere by then), so its MFMAs start
// right after the barrier instead of behind a burst of 8 waves' reads.  The
// epilogue's R is loaded right after the last stage, four steps before use.
// ---------------------------------------------------------------------------
constexpr int kUp2Slots = 5;
constexpr int kUp2WChunks = 1024;                     // W_up panel of 64 columns x 4 streams
constexpr int kUp2Stage = kUp2WChunks + 2 * kLoTile;  // 2048 chunks (32 KB)
constexpr int kUp2Loads = kUp2Stage / 64 / 8;         // wave instructions per stage and wave (4)
constexpr int kUp2Waves = 8;
constexpr int kPersistGrid = 256;  // one workgroup per CU

// Loads a wave of prefill_upmix2 has issued after stage `st` by the end of
// step `step` (issue order: stages 0-3, then per step j stage j + 4 while it
// exists and two R loads for j < 8); a stage past the last needs no wait.
constexpr int up2_loads_after(int st, int step)
{
    if (st >= kUpSteps)
        return 16;  // (only R can still be in flight: at most its 16 loads)
    int n = 0;
    bool seen = false;
    for (int k = 0; k < 4; ++k) {  // prologue
        if (seen)
            n += kUp2Loads;
        if (k == st)
            seen = true;
    }
    for (int j = 0; j <= step; ++j) {
        if (j + 4 < kUpSteps) {
            if (seen)
                n += kUp2Loads;
            if (j + 4 == st)
                seen = true;
        }
        if (j < 8 && seen)
            n += 2;
    }
    return n;
}

template <bool HAS_P, bool BF16_LO>
__global__ __launch_bounds__(kUp2Waves * 64, 1) void prefill_upmix2(int T, int tiles, const uint4* __restrict__ lo_tiled,
                                                                    const uint16_t* __restrict__ W_up,
                                                                    const float* R,
                                                                    const float* __restrict__ P,
                                                                    float* __restrict__ out_mixed,
                                                                    uint16_t* __restrict__ out_bf16,
                                                                    uint16_t* __restrict__ out_fp16,
                                                                    float* R_commit)
{
    static_assert(kUpSteps == 10, "schedule");
    static_assert(kUp2Slots * kUp2Stage * 16 <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint4 lds[kUp2Slots * kUp2Stage];

    const int b = blockIdx.x;
    const int x = b & 7, q = b >> 3;
    const int pair = q / kGroupsPerXcd;
    const int cg = x + 8 * (q - pair * kGroupsPerXcd);
    const int t0 = pair * 2 * kTok, c0 = cg * kUpCols;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int hf = wave >> 2, wl = wave & 3;  // token tile of the pair, wave within it

    // stage loads: W_up panel instruction i (0..15) fills rows 16 i .. +15
    // (lane l: row 16 i + l / 4, chunk (l & 3) ^ ((row >> 1) & 3)), wave w
    // issues i = w and w + 8; lo: wave w copies 1 KB w of each tile's block
    // (a second tile past the chunk re-reads the first: its tokens store nothing)
    const int wchunk = (lane & 3) ^ ((lane >> 3) & 3);
    const uint16_t* wu_lane[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int prow = 16 * (wave + 8 * k) + (lane >> 2);  // panel row = 64 s + j
        wu_lane[k] = W_up + (size_t)((prow / kUpCols) * kWidth + c0 + (prow % kUpCols)) * kRank + 8 * wchunk;
    }
    const int tile1 = 2 * pair + 1 < tiles ? 2 * pair + 1 : 2 * pair;
    const uint4* lo_lane0 = lo_tiled + (size_t)(2 * pair) * kUpSteps * kLoTile + 64 * wave + lane;
    const uint4* lo_lane1 = lo_tiled + (size_t)tile1 * kUpSteps * kLoTile + 64 * wave + lane;
    auto issue = [&](int ks) {
        uint4* sb = lds + (ks % kUp2Slots) * kUp2Stage;
        dma16(wu_lane[0] + kKs * ks, sb + 64 * wave);
        dma16(wu_lane[1] + kKs * ks, sb + 64 * (wave + 8));
        dma16(lo_lane0 + (size_t)ks * kLoTile, sb + kUp2WChunks + 64 * wave);
        dma16(lo_lane1 + (size_t)ks * kLoTile, sb + kUp2WChunks + kLoTile + 64 * wave);
    };

    f32x4_t acc[4][4];  // [column block][stream]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[cb][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t lds0 = lds_addr(lds);
    // W_up operand of panel block k = 4 s + cb (stream s, column block cb):
    // this lane's slot in block 0 plus 1 KB per block
    const uint32_t aoff = 16 * panel_slot(n, g);
    // lo of token 16 wl + n of the wave's tile, floats 8 g .. 8 g + 7
    const int lrow = 16 * wl + n;
    const uint32_t lo_a = 16 * (kUp2WChunks + kLoTile * hf + 8 * lrow + ((2 * g) ^ swz8(lrow)));
    const uint32_t lo_b = 16 * (kUp2WChunks + kLoTile * hf + 8 * lrow + ((2 * g + 1) ^ swz8(lrow)));
    // the reads that open step ks: its lo and W_up blocks 0-3
    auto read_first = [&](int ks, u32x4 (&lv)[2], u32x4 (&w0)[4]) {
        const uint32_t sb = lds0 + 16 * (ks % kUp2Slots) * kUp2Stage;
        lv[0] = ds_read16(sb + lo_a);
        lv[1] = ds_read16(sb + lo_b);
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w0[k] = ds_read16_off<1024 * k>(sb + aoff); });
    };
    // step ks with its first reads done by read_first: the other 12 W_up
    // blocks stream in behind the MFMAs of the earlier ones; an accumulator's
    // pieces 2, 1, 0 are four MFMAs apart
    auto compute = [&](int ks, u32x4 (&lv)[2], u32x4 (&w0)[4]) {
        const uint32_t wb = lds0 + 16 * (ks % kUp2Slots) * kUp2Stage + aoff;
        u32x4 w1[4], w2[4], w3[4];
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w1[k] = ds_read16_off<1024 * (4 + k)>(wb); });
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w2[k] = ds_read16_off<1024 * (8 + k)>(wb); });
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w3[k] = ds_read16_off<1024 * (12 + k)>(wb); });
        lgkm_wait<12>(lv[0], lv[1], w0[0], w0[1], w0[2], w0[3]);
        uint32_t hi[8], mi[8] = {}, l3[8] = {};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (BF16_LO)  // the fast mode: lo rounded to bf16 (nearest even), one piece
                hi[e] = __builtin_bit_cast(uint16_t, (__bf16)__uint_as_float(lv[e >> 2][e & 3]));
            else
                split3(__uint_as_float(lv[e >> 2][e & 3]), hi[e], mi[e], l3[e]);
        }
        u32x4 y[3];
        y[0] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
        y[1] = u32x4{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16)};
        y[2] = u32x4{l3[0] | (l3[1] << 16), l3[2] | (l3[3] << 16), l3[4] | (l3[5] << 16), l3[6] | (l3[7] << 16)};
        auto group = [&](int s, u32x4 (&w)[4]) {  // stream s: panel blocks 4 s .. 4 s + 3
#pragma unroll
            for (int p = BF16_LO ? 0 : 2; p >= 0; --p)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[cb][s] = mfma16(w[cb], y[p], acc[cb][s]);
        };
        group(0, w0);
        lgkm_wait<8>(w1[0], w1[1], w1[2], w1[3]);
        group(1, w1);
        lgkm_wait<4>(w2[0], w2[1], w2[2], w2[3]);
        group(2, w2);
        lgkm_wait<0>(w3[0], w3[1], w3[2], w3[3]);
        group(3, w3);
        __builtin_amdgcn_sched_barrier(0);  // the step's MFMAs issue before the next step's reads
    };

    // the epilogue's R: this lane's token, columns c0 + 16 cb + 4 g .. +3 of
    // every stream (tokens past T re-read token T - 1 and store nothing)
    constexpr int kRLoads = 16;
    const int t = t0 + kTok * hf + lrow;
    const int tr = t < T ? t : T - 1;
    const float* rrow = R + (size_t)tr * kD + c0 + 4 * g;
    float4 rv[4][4];  // [column block][stream]
    typedef __attribute__((address_space(1))) const f32x4_t gf32x4;  // global memory
    gf32x4* rl = (gf32x4*)rrow;  // (loads through it stay between the asm statements)
    asm volatile("" : "+v"(rl));

    // Step ks issues stage ks + 4, then (steps 0-7) two of the 16 R loads:
    // issued all at once, R's 128 KB per workgroup would hold up the wave's
    // instruction stream for thousands of cycles (measured: the step that
    // issued them took 4-5 times as long as the others).  Loads complete in
    // issue order; the wait closing step ks needs stage ks + 2 landed, so it
    // leaves in flight what was issued after that stage.  Step ks ends by
    // reading step ks + 1's first operands.
    u32x4 lv[2], w0[4];
    static_for<0, 4>([&](auto kc) { issue(decltype(kc)::value); });
    ring_barrier<2 * kUp2Loads>();  // stages 0 and 1 landed everywhere
    read_first(0, lv, w0);
    static_for<0, kUpSteps>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 4 < kUpSteps)
            issue(ks + 4);
        order();
        if constexpr (ks < 8) {
#pragma unroll
            for (int i = 2 * ks; i < 2 * ks + 2; ++i) {
                const f32x4_t v = rl[((i & 3) * kWidth + 16 * (i >> 2)) / 4];
                rv[i >> 2][i & 3] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
        order();
        compute(ks, lv, w0);
        if constexpr (ks + 1 < kUpSteps) {
            read_first(ks + 1, lv, w0);
            ring_barrier_lg<up2_loads_after(ks + 2, ks), 6>();
        }
    });

    if (HAS_P) {
        const float* prow = P + (size_t)tr * kD + c0 + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 pv = *reinterpret_cast<const float4*>(prow + s * kWidth + 16 * cb);
                rv[cb][s].x += pv.x;
                rv[cb][s].y += pv.y;
                rv[cb][s].z += pv.z;
                rv[cb][s].w += pv.w;
            }
        // the pending write committed: R' of this lane's token and columns
        // back into R (no other workgroup reads them in this chunk, and the
        // down projection of the chunk has finished)
        if (R_commit && t < T) {
            float* crow = R_commit + (size_t)t * kD + c0 + 4 * g;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    *reinterpret_cast<float4*>(crow + s * kWidth + 16 * cb) = rv[cb][s];
        }
    }
    // The wave's 16 tokens x 64 columns of mixed go through 4 KB of LDS of its
    // own (in ring slot 0, which no wave reads after step 5) so that every
    // store instruction writes whole 128-byte lines: written in the MFMA
    // layout (chunk 4 cb + g of row n at slot (4 cb + g) ^ n), read back as 4
    // rows of 16 lanes x 16 bytes.
    const uint32_t tb = lds0 + 4096 * wave;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float r[4][4] = {{rv[cb][0].x, rv[cb][0].y, rv[cb][0].z, rv[cb][0].w},
                               {rv[cb][1].x, rv[cb][1].y, rv[cb][1].z, rv[cb][1].w},
                               {rv[cb][2].x, rv[cb][2].y, rv[cb][2].z, rv[cb][2].w},
                               {rv[cb][3].x, rv[cb][3].y, rv[cb][3].z, rv[cb][3].w}};
        float m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m[i] = (acc[cb][0][i] * r[0][i] + acc[cb][1][i] * r[1][i]) +
                   (acc[cb][2][i] * r[2][i] + acc[cb][3][i] * r[3][i]);
        ds_write16(tb + 256 * n + 16 * ((4 * cb + g) ^ n),
                   u32x4{__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3])});
    }
    u32x4 mv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = (lane >> 4) + 4 * k, ch = lane & 15;
        mv[k] = ds_read16(tb + 256 * row + 16 * (ch ^ row));
    }
    lds_wait(mv);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = (lane >> 4) + 4 * k, ch = lane & 15;
        const int tt = t0 + kTok * hf + 16 * wl + row;
        if (tt < T) {
            const size_t o = (size_t)tt * kWidth + c0 + 4 * ch;
            const float m[4] = {__uint_as_float(mv[k][0]), __uint_as_float(mv[k][1]), __uint_as_float(mv[k][2]),
                                __uint_as_float(mv[k][3])};
            *reinterpret_cast<float4*>(out_mixed + o) = make_float4(m[0], m[1], m[2], m[3]);
            uint32_t bh[4], hh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bh[i] = __builtin_bit_cast(uint16_t, (__bf16)m[i]);
                hh[i] = __builtin_bit_cast(uint16_t, (_Float16)m[i]);
            }
            *reinterpret_cast<uint2*>(out_bf16 + o) = make_uint2(bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16));
            *reinterpret_cast<uint2*>(out_fp16 + o) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
        }
    }
}

// ---------------------------------------------------------------------------
// P3 without pending, persistent: one workgroup of 8 waves per CU walks its
// (128-token pair, 64-column group) items b, b + grid, ...; items are the
// full token pairs of the chunk (a ragged last pair goes to prefill_upmix2).
// The stage stream runs on across items: the last four steps of an item
// load the first four stages of the next (or, after the last item, the
// current item's again, so every wait counts the same), so a workgroup pays
// the ring's fill latency once instead of once per item.  Per item the
// steps are those of prefill_upmix2; the mixed values go through ring slot
// 4 (stage 9's, free after the item's last step) on their way out.
// ---------------------------------------------------------------------------
template <bool BF16_LO>
__global__ __launch_bounds__(kUp2Waves * 64, 1) void prefill_upmix3(int T, int items, const uint4* __restrict__ lo_tiled,
                                                                    const uint16_t* __restrict__ W_up,
                                                                    const float* R,
                                                                    float* __restrict__ out_mixed,
                                                                    uint16_t* __restrict__ out_bf16,
                                                                    uint16_t* __restrict__ out_fp16)
{
    static_assert(kUpSteps == 10 && kUp2Slots == 5, "schedule");
    __shared__ __align__(16) uint4 lds[kUp2Slots * kUp2Stage];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const int hf = wave >> 2, wl = wave & 3;

    // stage loads (as in prefill_upmix2): per lane offsets, item bases added per item
    const int wchunk = (lane & 3) ^ ((lane >> 3) & 3);
    uint32_t wu_off[2];  // (elements)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int prow = 16 * (wave + 8 * k) + (lane >> 2);  // panel row = 64 s + j
        wu_off[k] = (uint32_t)((prow / kUpCols) * kWidth + (prow % kUpCols)) * kRank + 8 * wchunk;
    }
    const __amdgpu_buffer_rsrc_t rrs = rsrc_of(R);
    const int lo_off = 64 * wave + lane;
    struct Item {
        int t0, c0;  // first token (of the pair) and column
    };
    auto item_of = [&](int w) {
        const int x = w & 7, q = w >> 3;
        const int pair = q / kGroupsPerXcd;
        const int cg = x + 8 * (q - pair * kGroupsPerXcd);
        return Item{pair * 2 * kTok, cg * kUpCols};
    };
    // (buffer loads: the compiler counts them exactly in its own waits,
    // where global loads into LDS make it wait for everything)
    const __amdgpu_buffer_rsrc_t wrs = rsrc_of(W_up), lrs = rsrc_of(lo_tiled);
    auto issue = [&](const Item& it, int ks, int slot) {
        uint4* sb = lds + slot * kUp2Stage;
        const uint32_t wso = 2u * ((uint32_t)it.c0 * kRank + kKs * ks);
        const uint32_t lso = 16u * ((uint32_t)(it.t0 / kTok) * kUpSteps * kLoTile + ks * kLoTile);
        bdma16(wrs, sb + 64 * wave, 2u * wu_off[0], wso);
        bdma16(wrs, sb + 64 * (wave + 8), 2u * wu_off[1], wso);
        bdma16(lrs, sb + kUp2WChunks + 64 * wave, 16u * lo_off, lso);
        bdma16(lrs, sb + kUp2WChunks + kLoTile + 64 * wave, 16u * lo_off, lso + 16u * kUpSteps * kLoTile);
    };

    const uint32_t lds0 = lds_addr(lds);
    const uint32_t aoff = 16 * panel_slot(n, g);
    const int lrow = 16 * wl + n;
    const uint32_t lo_a = 16 * (kUp2WChunks + kLoTile * hf + 8 * lrow + ((2 * g) ^ swz8(lrow)));
    const uint32_t lo_b = 16 * (kUp2WChunks + kLoTile * hf + 8 * lrow + ((2 * g + 1) ^ swz8(lrow)));
    auto read_first = [&](int slot, u32x4 (&lv)[2], u32x4 (&w0)[4]) {
        const uint32_t sb = lds0 + 16 * slot * kUp2Stage;
        lv[0] = ds_read16(sb + lo_a);
        lv[1] = ds_read16(sb + lo_b);
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w0[k] = ds_read16_off<1024 * k>(sb + aoff); });
    };
    f32x4_t acc[4][4];  // [column block][stream]
    // the other 12 W_up blocks are read one stream group ahead of their MFMAs
    auto compute = [&](int slot, u32x4 (&lv)[2], u32x4 (&w0)[4]) {
        const uint32_t wb = lds0 + 16 * slot * kUp2Stage + aoff;
        u32x4 w1[4], w2[4], w3[4];
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w1[k] = ds_read16_off<1024 * (4 + k)>(wb); });
        lgkm_wait<4>(lv[0], lv[1], w0[0], w0[1], w0[2], w0[3]);
        uint32_t hi[8], mi[8] = {}, l3[8] = {};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (BF16_LO)  // the fast mode: lo rounded to bf16 (nearest even), one piece
                hi[e] = __builtin_bit_cast(uint16_t, (__bf16)__uint_as_float(lv[e >> 2][e & 3]));
            else
                split3(__uint_as_float(lv[e >> 2][e & 3]), hi[e], mi[e], l3[e]);
        }
        u32x4 y[3];
        y[0] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
        y[1] = u32x4{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16)};
        y[2] = u32x4{l3[0] | (l3[1] << 16), l3[2] | (l3[3] << 16), l3[4] | (l3[5] << 16), l3[6] | (l3[7] << 16)};
        auto group = [&](int s, u32x4 (&w)[4]) {
#pragma unroll
            for (int p = BF16_LO ? 0 : 2; p >= 0; --p)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[cb][s] = mfma16(w[cb], y[p], acc[cb][s]);
        };
        group(0, w0);
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w2[k] = ds_read16_off<1024 * (8 + k)>(wb); });
        lgkm_wait<4>(w1[0], w1[1], w1[2], w1[3]);
        group(1, w1);
        static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; w3[k] = ds_read16_off<1024 * (12 + k)>(wb); });
        lgkm_wait<4>(w2[0], w2[1], w2[2], w2[3]);
        group(2, w2);
        lgkm_wait<0>(w3[0], w3[1], w3[2], w3[3]);
        group(3, w3);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Issue order per item: step ks loads stage ks + 4 of the item (ks < 6)
    // or stage ks - 6 of the next (ks >= 6), then two R loads (ks < 8); the
    // item ends with its 12 store instructions (full pairs: every row
    // stores).  The wait closing step ks needs stage ks + 2 landed and leaves
    // in flight what was issued after it: 22, 24 (the previous item's stores
    // included), 14 .. 14, 12, and after the item's stores, 22.  Before the
    // first item 12 stores that write nothing (offsets past a 0-byte buffer
    // resource) stand in for a previous item's, so every item waits alike.
    constexpr int kStores = 12;
    u32x4 lv[2], w0[4];
    const int grid = gridDim.x;
    int w = blockIdx.x;
    Item cur = item_of(w);
    Item nxt = w + grid < items ? item_of(w + grid) : cur;
    static_for<0, 4>([&](auto kc) { constexpr int k = decltype(kc)::value; issue(cur, k, k); });
    order();
    {
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(out_mixed, 0, 0, 0x00020000);
#pragma unroll
        for (int k = 0; k < kStores; ++k) {
            __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4u * lane, 256u * k, 0);
            order();
        }
    }
    order();
    ring_barrier<2 * kUp2Loads + kStores>();  // stages 0 and 1 landed everywhere
    read_first(0, lv, w0);
    while (true) {
        const int t = cur.t0 + kTok * hf + lrow;  // every token of a full pair is < T
        const uint32_t roff = 4u * ((uint32_t)t * kD + cur.c0 + 4 * g);  // (bytes; R of a chunk is < 2 GB)
        float4 rv[4][4];  // [column block][stream]
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[cb][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        static_for<0, kUpSteps>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            if constexpr (ks + 4 < kUpSteps)
                issue(cur, ks + 4, (ks + 4) % kUp2Slots);
            else
                issue(nxt, ks - 6, (ks + 4) % kUp2Slots);
            order();
            if constexpr (ks < 8) {
#pragma unroll
                for (int j = 2 * ks; j < 2 * ks + 2; ++j) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rrs, roff, 4u * ((j & 3) * kWidth + 16 * (j >> 2)), 0);
                    rv[j >> 2][j & 3] = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                                                    __uint_as_float(v[3]));
                }
            }
            order();
            compute(ks % kUp2Slots, lv, w0);
            if constexpr (ks + 1 < kUpSteps) {
                read_first((ks + 1) % kUp2Slots, lv, w0);
                ring_barrier_lg<(ks < 2 ? 10 + 2 * ks + kStores : ks == 8 ? 12 : 14), 6>();
            }
        });
        // every wave is done with ring slot 4 (stage 9) before it takes the mixed values
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const uint32_t tb = lds0 + 16 * 4 * kUp2Stage + 4096 * wave;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const float r[4][4] = {{rv[cb][0].x, rv[cb][0].y, rv[cb][0].z, rv[cb][0].w},
                                   {rv[cb][1].x, rv[cb][1].y, rv[cb][1].z, rv[cb][1].w},
                                   {rv[cb][2].x, rv[cb][2].y, rv[cb][2].z, rv[cb][2].w},
                                   {rv[cb][3].x, rv[cb][3].y, rv[cb][3].z, rv[cb][3].w}};
            float m[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                m[e] = (acc[cb][0][e] * r[0][e] + acc[cb][1][e] * r[1][e]) +
                       (acc[cb][2][e] * r[2][e] + acc[cb][3][e] * r[3][e]);
            ds_write16(tb + 256 * n + 16 * ((4 * cb + g) ^ n),
                       u32x4{__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3])});
        }
        u32x4 mv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = (lane >> 4) + 4 * k, ch = lane & 15;
            mv[k] = ds_read16(tb + 256 * row + 16 * (ch ^ row));
        }
        lds_wait(mv);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = (lane >> 4) + 4 * k, ch = lane & 15;
            const int tt = cur.t0 + kTok * hf + 16 * wl + row;
            const size_t o = (size_t)tt * kWidth + cur.c0 + 4 * ch;
            const float m[4] = {__uint_as_float(mv[k][0]), __uint_as_float(mv[k][1]), __uint_as_float(mv[k][2]),
                                __uint_as_float(mv[k][3])};
            *reinterpret_cast<float4*>(out_mixed + o) = make_float4(m[0], m[1], m[2], m[3]);
            uint32_t bh[4], hh[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bh[e] = __builtin_bit_cast(uint16_t, (__bf16)m[e]);
                hh[e] = __builtin_bit_cast(uint16_t, (_Float16)m[e]);
            }
            *reinterpret_cast<uint2*>(out_bf16 + o) = make_uint2(bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16));
            *reinterpret_cast<uint2*>(out_fp16 + o) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
        }
        w += grid;
        if (w >= items)
            break;
        cur = nxt;
        nxt = w + grid < items ? item_of(w + grid) : cur;
        read_first(0, lv, w0);
        ring_barrier_lg<10 + kStores, 6>();  // the next item's stage 1 landed; slot 4 free again
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // (the last item's extra stage loads land before exit)
}

int tiles_of(int tokens)
{
    return (tokens + kTok - 1) / kTok;
}

// P1's split count.  A workgroup takes a whole CU (its LDS), so the grid
// should fill the chip once: chunks of 64 tiles (8192 tokens) without a
// pending write use whole streams (4 splits; with pending the raw slots of
// 2560-column splits do not fit in LDS), chunks of 32 tiles or more stream
// halves, longer-than-1024-token chunks stream quarters (144-496 workgroups);
// shorter chunks split K finer so that short reads still stream W_down over
// most of the chip: 32 splits (320 columns) for 4-8 tiles, 80 splits (128
// columns, the narrowest the ring takes: 4 K steps) for 1-3 tiles.  Fewer
// splits write and read fewer partials (4 x 8192 x 320 floats, 42 MB, for an
// 8192-token chunk against 84 MB as two chunks of stream halves).
int splits_for(int tokens, bool pending)
{
    const int tiles = (tokens + kDnTok - 1) / kDnTok;
    if (!pending && tiles * 4 >= 256)
        return 4;
    if (tiles * 8 >= 256)
        return 8;
    if (tiles > 8)
        return 16;
    if (tiles > 3)
        return 32;
    return 80;
}

template <int S>
void launch_lo(int Tc, int tiles, float* part, float* ssq, uint4* planes, hipStream_t stream)
{
    const int items = tiles * kTok * (kRank / 4);
    constexpr int lanes = S == 80 ? 8 : (S >= 32 ? 4 : 1);  // lanes per item (as in prefill_lo)
    hipLaunchKernelGGL(prefill_lo<S>, dim3((lanes * items + 255) / 256), dim3(256), 0, stream, Tc, tiles * kTok, part,
                       ssq, planes);
}

template <int S>
void launch_down_lo(int Tc, int tiles, const float* Rc, const float* Pc, const float* w_norm,
                    const uint16_t* W_down, float* part, float* ssq, uint4* planes, hipStream_t stream)
{
    if constexpr (S == kSmSplits) {
        if (Tc <= kSmMaxTok) {
            // short chunks: 32-token tiles up to 96 tokens, 64-token ones above
            const bool t32 = Tc <= 96;
            const dim3 grid(kSmSplits * ((Tc + (t32 ? 31 : 63)) / (t32 ? 32 : 64))), block(512);
            auto* dn = Pc ? (t32 ? prefill_down_small<32, true> : prefill_down_small<64, true>)
                          : (t32 ? prefill_down_small<32, false> : prefill_down_small<64, false>);
            hipLaunchKernelGGL(dn, grid, block, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
            return launch_lo<S>(Tc, tiles, part, ssq, planes, stream);
        }
    }
    const dim3 grid1(S * ((Tc + kDnTok - 1) / kDnTok)), block1(kDnWaves * 64);
    if constexpr (S >= 8) {  // (4 splits are never used with pending)
        if (Pc) {
            hipLaunchKernelGGL((prefill_down<S, true>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part,
                               ssq);
            return launch_lo<S>(Tc, tiles, part, ssq, planes, stream);
        }
    }
    hipLaunchKernelGGL((prefill_down<S, false>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
    launch_lo<S>(Tc, tiles, part, ssq, planes, stream);
}

// (split, token) slots of the partial array, enough for any chunk of up to
// `chunk` tokens, with or without pending
size_t part_slots(int chunk)
{
    size_t most = 0;
    for (int tc = chunk; tc > 0; tc -= kDnTok)  // splits_for changes only at tile boundaries
        for (int pending = 0; pending < 2; ++pending) {
            const size_t n = (size_t)splits_for(tc, pending != 0) * tc;
            most = most > n ? most : n;
        }
    return most;
}

}  // namespace

size_t prefill_scratch_bytes(int chunk)
{
    const size_t tpad = (size_t)tiles_of(chunk) * kTok;
    return sizeof(float) * part_slots(chunk) * (kRank + 1) + sizeof(float) * tpad * kRank + 512;
}

hipError_t launch_prefill(int64_t T, const float* R, const float* P, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit, bool bf16_lo,
                          void* scratch, int chunk, hipStream_t stream)
{
    const size_t slots = part_slots(chunk);
    float* part = static_cast<float*>(scratch);  // [S][Tc][320]
    float* ssq = part + slots * kRank;             // [S][Tc]
    uint4* planes = reinterpret_cast<uint4*>(      // tiled fp32 lo
        (reinterpret_cast<uintptr_t>(ssq + slots) + 255) & ~uintptr_t(255));
    for (int64_t c0 = 0; c0 < T; c0 += chunk) {
        const int Tc = (int)(T - c0 < chunk ? T - c0 : chunk);
        const size_t in_off = (size_t)c0 * kD, out_off = (size_t)c0 * kWidth;
        const float* Rc = R + in_off;
        const float* Pc = P ? P + in_off : nullptr;
        const int tiles = tiles_of(Tc);
        switch (splits_for(Tc, Pc != nullptr)) {
        case 4: launch_down_lo<4>(Tc, tiles, Rc, Pc, w_norm, W_down, part, ssq, planes, stream); break;
        case 8: launch_down_lo<8>(Tc, tiles, Rc, Pc, w_norm, W_down, part, ssq, planes, stream); break;
        case 16: launch_down_lo<16>(Tc, tiles, Rc, Pc, w_norm, W_down, part, ssq, planes, stream); break;
        case 32: launch_down_lo<32>(Tc, tiles, Rc, Pc, w_norm, W_down, part, ssq, planes, stream); break;
        default: launch_down_lo<80>(Tc, tiles, Rc, Pc, w_norm, W_down, part, ssq, planes, stream); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        float* Cc = R_commit && Pc ? R_commit + in_off : nullptr;
        const bool narrow = tiles <= 4;  // 16- or 32-column tiles (measured: better up to 256 tokens)
        if (narrow) {
            // column blocks and ring depth by chunk (measured best): 16 columns
            // with 4 stages for one token tile and 5 for two; 32 columns with 3
            // stages for three tiles and 4 for four
            auto pick = [&](auto ns, auto cb) {
                constexpr int NS = decltype(ns)::value, CB = decltype(cb)::value;
                return Pc ? (bf16_lo ? prefill_upmix<true, true, NS, CB> : prefill_upmix<true, false, NS, CB>)
                          : (bf16_lo ? prefill_upmix<false, true, NS, CB> : prefill_upmix<false, false, NS, CB>);
            };
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            using I3 = std::integral_constant<int, 3>;
            using I4 = std::integral_constant<int, 4>;
            using I5 = std::integral_constant<int, 5>;
            auto* up = tiles == 1 ? pick(I4{}, I1{}) : tiles == 2 ? pick(I5{}, I1{}) : tiles == 3 ? pick(I3{}, I2{}) : pick(I4{}, I2{});
            const int cb = tiles <= 2 ? 1 : 2;
            hipLaunchKernelGGL(up, dim3(8 * (kWidth / (16 * cb) / 8) * tiles), dim3(256), 0, stream, Tc, planes, W_up, Rc,
                               Pc, out_mixed + out_off, out_bf16 + out_off, out_fp16 + out_off, Cc);
        } else if (Pc) {
            auto* up = bf16_lo ? prefill_upmix2<true, true> : prefill_upmix2<true, false>;
            hipLaunchKernelGGL(up, dim3(8 * kGroupsPerXcd * ((tiles + 1) / 2)), dim3(kUp2Waves * 64), 0, stream, Tc,
                               tiles, planes, W_up, Rc, Pc, out_mixed + out_off, out_bf16 + out_off,
                               out_fp16 + out_off, Cc);
        } else {
            // full token pairs on the persistent kernel, a ragged last pair on its own
            const int pairs = Tc / (2 * kTok), items = 8 * kGroupsPerXcd * pairs;
            if (items > 0) {
                auto* up = bf16_lo ? prefill_upmix3<true> : prefill_upmix3<false>;
                hipLaunchKernelGGL(up, dim3(items < kPersistGrid ? items : kPersistGrid), dim3(kUp2Waves * 64), 0,
                                   stream, Tc, items, planes, W_up, Rc, out_mixed + out_off, out_bf16 + out_off,
                                   out_fp16 + out_off);
            }
            const int t_done = pairs * 2 * kTok;
            if (t_done < Tc) {
                const int rest = Tc - t_done;
                auto* up = bf16_lo ? prefill_upmix2<false, true> : prefill_upmix2<false, false>;
                hipLaunchKernelGGL(up, dim3(8 * kGroupsPerXcd), dim3(kUp2Waves * 64), 0, stream, rest,
                                   tiles_of(rest), planes + (size_t)(t_done / kTok) * kUpSteps * kLoTile, W_up,
                                   Rc + (size_t)t_done * kD, nullptr, out_mixed + out_off + (size_t)t_done * kWidth,
                                   out_bf16 + out_off + (size_t)t_done * kWidth,
                                   out_fp16 + out_off + (size_t)t_done * kWidth, nullptr);
            }
        }
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace hc
