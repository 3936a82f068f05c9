// hc_prefill.hip -- the hyper-connection read for wide inputs (T > 8 tokens):
// prefill chunks and long verify windows.
//
// The read is the one of "#315 hc: the multi-token hyper-connection read split
// finer" with the norm folded into the down projection ("#2488 sycl/A770",
// Summary item 4) and the up projection fused with gr_mix_r as in "#1370
// prefill: ... gr_mix_r as its epilogue", "What it does": gated (T x 10240
// fp32) never leaves registers.  Three launches per chunk of up to 4096 tokens:
//
//   P1 down:  part[sig][t][j] = sum_{k in split sig} W_down[j][k] * (R'[t][k] *
//             w_norm[k]) and ssq[sig][t] = sum_{k in sig} R'[t][k]^2, where the
//             8 splits are the halves of the 4 streams (1280 columns each).
//   P2 lo:    rs[t][s] = 1/sqrt(sum of stream s's two ssq / 2560 + eps) and
//             lo[t][j] = sum_s rs[t][s] * (stream s's two partials), stored as
//             three bf16 planes (an exact split of the fp32 value) in the
//             tiled layout P3 copies into LDS verbatim.
//   P3 up+mix: a tile of 64 tokens x 64 output columns x 4 streams: the up
//             projection (K = 320) on the matrix cores, then the mix of the 4
//             streams with R' and the bf16 / fp16 images, all in registers.
//
// gfx950 design:
// * Both matrix kernels run bf16 v_mfma_f32_16x16x32_bf16 with every fp32
//   activation split exactly into three bf16 pieces (hi + mid + lo3 == x), so
//   each product is exact and the result stays fp32-faithful.
// * Weight operands (and P3's lo planes) go from memory straight into LDS
//   (global_load_lds_dwordx4, 16 bytes a lane) through a two-stage ring, one K
//   step of 32 ahead of the matrix cores.  LDS is read with inline-asm
//   ds_read_b128 and every wait is explicit: the compiler, seeing an LDS read
//   that may alias a load still landing in LDS, would wait for ALL loads in
//   flight (vmcnt(0)) and serialise the ring.
// * Inside LDS a K step of a tile is a "panel": one row per matrix row, four
//   16-byte chunks per row, chunk c of row r stored at slot 4 r + (c ^ ((r >>
//   2) & 3)).  The 16 lanes that read one chunk column of 16 consecutive rows
//   then hit 16 distinct 16-byte bank groups.
// * Both kernels use 4 waves and 56-64 KB of LDS, so two workgroups share a
//   CU: one's epilogue (memory bound) overlaps the other's matrix work.
// * XCD-aware grids (workgroup b runs on XCD b % 8): P1's XCD x owns split x,
//   so its 820 KB W_down slice stays in that XCD's L2; P3's XCD x owns 5 of
//   the 40 column groups (W_up slices, 820 KB) and walks the token tiles, the 5
//   workgroups of one tile being dispatched together so its lo planes are read
//   once per XCD.
// * The chunk keeps a chunk's R (+ pending) within the 256 MB Infinity Cache
//   for its second read in P3.
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
// 16 bytes per lane from memory into LDS: lane l's bytes land at
// lds_wave_base + 16 l (the base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* g, uint4* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

// Slot (in 16-byte chunks) of chunk c (0..3) of row r in a panel.
__host__ __device__ constexpr int panel_slot(int r, int c)
{
    return 4 * r + (c ^ ((r >> 2) & 3));
}

constexpr int kTok = 64;                       // token tile of both matrix kernels
constexpr int kKs = 32;                        // K step: one MFMA depth
constexpr int kUpSteps = kRank / kKs;          // 10
constexpr int kUpCols = 64;                    // P3 output columns per tile
constexpr int kUpGroups = kWidth / kUpCols;    // 40 column groups
constexpr int kGroupsPerXcd = kUpGroups / 8;   // 5
constexpr int kPlaneChunks = kTok * 4;         // one plane panel of a token tile: 256 chunks (4 KB)
constexpr int kLoBlock = 3 * kPlaneChunks;     // the three planes of one (tile, K step): 12 KB

// ---------------------------------------------------------------------------
// P1: down projection partials and sums of squares.  Workgroup b: split
// b % S of width 10240 / S (stream halves or quarters; with S = 8 the split is
// the XCD's, with S = 16 each XCD owns two), token tile b / S of 128 tokens.
// Wave w owns tokens 16 w .. 16 w + 15 of the tile and computes all 320 rows
// for them: MFMA A = W_down rows (20 blocks of 16), B = that wave's y = R' *
// w_norm, split in registers into its three bf16 pieces (each wave converts
// only its own tokens, so no y panel is shared through LDS).
// Everything reaches LDS by direct loads: the W_down panel of a step one step
// ahead (2 slots), raw R and pending two steps ahead (3 slots), and the
// split's w_norm once.  No loaded value lives in registers across a step.
// Raw rows are 32 floats (8 chunks of 16 bytes); chunk c of row r sits at slot
// c ^ swz(r) of its 128-byte line, so 16 lanes reading one chunk of 16 rows
// hit distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int kDnTok = 128;
constexpr int kDnWaves = 8;
constexpr int kDnWChunks = kRank * 4;           // W_down panel: 1280 chunks (20 KB)
constexpr int kDnRawChunks = kDnTok * 8;        // raw R (or pending) of a step: 1024 chunks (16 KB)

__device__ __forceinline__ int swz8(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}

template <int S, bool HAS_P>
__global__ __launch_bounds__(kDnWaves * 64) void prefill_down(int T, const float* __restrict__ R,
                                                              const float* __restrict__ P,
                                                              const float* __restrict__ w_norm,
                                                              const uint16_t* __restrict__ W_down,
                                                              float* __restrict__ part, float* __restrict__ ssq)
{
    constexpr int SW = kD / S;              // columns of a split
    constexpr int NS = SW / kKs;            // K steps
    constexpr int kRawSlots = 3;
    constexpr int kRawSet = (HAS_P ? 2 : 1) * kDnRawChunks;
    // LDS (chunks): 2 W_down slots, 3 raw slots (R, then pending), w_norm
    constexpr int kWOff = 0;
    constexpr int kRawOff = 2 * kDnWChunks;
    constexpr int kNormOff = kRawOff + kRawSlots * kRawSet;
    constexpr int kLdsChunks = kNormOff + SW / 4;
    // raw-load wave instructions per step and wave (16 per array, 8 waves)
    constexpr int kRawLoads = (HAS_P ? 2 : 1) * (kDnRawChunks / 64) / kDnWaves;
    static_assert(kDnRawChunks % (64 * kDnWaves) == 0 && SW % kKs == 0 && NS >= 3, "tiling");
    __shared__ __align__(16) uint4 lds[kLdsChunks];

    const int b = blockIdx.x;
    const int sig = b % S;
    const int t0 = (b / S) * kDnTok;
    const int kbase = sig * SW;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const uint32_t lds0 = lds_addr(lds);

    // W_down panel: wave instruction q (0..19) fills panel rows 16 q .. 16 q + 15
    // (lane l: row 16 q + l / 4, chunk (l & 3) ^ ((row >> 2) & 3)); wave w
    // issues q = w, w + 8 and (w < 4) w + 16.
    const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint16_t* wd_lane = W_down + (size_t)(lane >> 2) * kD + kbase + 8 * dchunk;
    // raw R / pending: wave instruction q (0..15) fills rows 8 q .. 8 q + 7 (lane
    // l: row 8 q + l / 8, chunk (l & 7) ^ swz8(row)); wave w issues q = w, w + 8.
    // Rows past T re-read row T - 1 (their results are never stored).
    const float* rraw[2];
    const float* praw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = wave + 8 * k;
        const int row = 8 * q + (lane >> 3);
        const int tr = t0 + row < T ? t0 + row : T - 1;
        const int ch = (lane & 7) ^ swz8(row);
        rraw[k] = R + (size_t)tr * kD + kbase + 4 * ch;
        praw[k] = HAS_P ? P + (size_t)tr * kD + kbase + 4 * ch : nullptr;
    }
    auto issue_w = [&](int ks, int slot) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int q = wave + 8 * k;
            if (k < 2 || wave < 4)
                dma16(wd_lane + (size_t)(16 * q) * kD + kKs * ks, lds + kWOff + slot * kDnWChunks + 64 * q);
        }
    };
    auto issue_raw = [&](int ks, int slot) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = wave + 8 * k;
            dma16(rraw[k] + kKs * ks, lds + kRawOff + slot * kRawSet + 64 * q);
            if (HAS_P)
                dma16(praw[k] + kKs * ks, lds + kRawOff + slot * kRawSet + kDnRawChunks + 64 * q);
        }
    };

    f32x4_t acc[20];
#pragma unroll
    for (int jb = 0; jb < 20; ++jb)
        acc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ssacc = 0.f;

    // this lane's B operand: token 16 wave + n, columns 8 g .. 8 g + 7 of the step
    const int trow = 16 * wave + n;
    const bool tok_ok = t0 + trow < T;
    const uint32_t raw_a = 16 * (trow * 8 + ((2 * g) ^ swz8(trow)));
    const uint32_t raw_b = 16 * (trow * 8 + ((2 * g + 1) ^ swz8(trow)));
    // W_down operand of row block jb: panel slot of row 16 jb + n, chunk g,
    // i.e. this lane's slot in block 0 plus 1 KB per block
    const uint32_t aoff = 16 * panel_slot(n, g);

    auto compute = [&](int ks, int wslot, int rslot) {
        const uint32_t rb = lds0 + 16 * (kRawOff + rslot * kRawSet);
        u32x4 raw[6];
        raw[0] = ds_read16(rb + raw_a);
        raw[1] = ds_read16(rb + raw_b);
        if (HAS_P) {
            raw[2] = ds_read16(rb + 16 * kDnRawChunks + raw_a);
            raw[3] = ds_read16(rb + 16 * kDnRawChunks + raw_b);
        }
        const uint32_t nb = lds0 + 16 * (kNormOff + 2 * (4 * ks + g));  // w_norm[32 ks + 8 g ..]
        raw[4] = ds_read16(nb);
        raw[5] = ds_read16(nb + 16);
        const uint32_t wb = lds0 + 16 * (kWOff + wslot * kDnWChunks) + aoff;
        u32x4 wa[5];
        wa[0] = ds_read16_off<0>(wb);
        wa[1] = ds_read16_off<1024>(wb);
        wa[2] = ds_read16_off<2048>(wb);
        wa[3] = ds_read16_off<3072>(wb);
        wa[4] = ds_read16_off<4096>(wb);
        lds_wait(raw);
        // y = R' * w_norm, its square sum, and the exact 3-way split
        uint32_t hi[8], mi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = __uint_as_float(raw[e >> 2][e & 3]);
            if (HAS_P)
                x += __uint_as_float(raw[2 + (e >> 2)][e & 3]);
            x = tok_ok ? x : 0.f;
            ssacc += x * x;
            split3(x * __uint_as_float(raw[4 + (e >> 2)][e & 3]), hi[e], mi[e], lo[e]);
        }
        u32x4 y[3];
        y[0] = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
        y[1] = u32x4{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16)};
        y[2] = u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
        // 4 groups of 5 row blocks: the next group's W_down operands are read
        // while this group's 15 MFMAs run
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            u32x4 wn[5];
            if (grp < 3) {
                const uint32_t wg = wb + 5120 * (grp + 1);
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
                for (int jb = 0; jb < 5; ++jb)
                    acc[5 * grp + jb] = mfma16(wa[jb], y[p], acc[5 * grp + jb]);
            if (grp < 3) {
#pragma unroll
                for (int jb = 0; jb < 5; ++jb)
                    wa[jb] = wn[jb];
            }
        }
    };

    // Step ks: W_down of step ks + 1 is issued, then the raw activations of
    // step ks + 2, so the wait at the end of the step leaves exactly those in
    // flight; the matrix cores run step ks.
    issue_w(0, 0);
    if (64 * wave + lane < SW / 4)  // the split's w_norm, SW / 4 chunks
        dma16(w_norm + kbase + 4 * (64 * wave + lane), lds + kNormOff + 64 * wave);
    issue_raw(0, 0);
    order();
    issue_raw(1, 1);
    ring_barrier<kRawLoads>();
    int rs0 = 0;  // raw slot of step ks
#pragma unroll 1
    for (int ks = 0; ks < NS - 2; ++ks) {
        issue_w(ks + 1, (ks + 1) & 1);
        order();
        issue_raw(ks + 2, rs0 == 0 ? 2 : rs0 - 1);  // (ks + 2) % 3
        compute(ks, ks & 1, rs0);
        ring_barrier<kRawLoads>();
        rs0 = rs0 == 2 ? 0 : rs0 + 1;
    }
    issue_w(NS - 1, (NS - 1) & 1);
    compute(NS - 2, (NS - 2) & 1, rs0);
    ring_barrier<0>();
    compute(NS - 1, (NS - 1) & 1, rs0 == 2 ? 0 : rs0 + 1);

    // partials: lane holds token t0 + 16 wave + n, rows 16 jb + 4 g .. +3
    const int t = t0 + trow;
    if (tok_ok) {
        float* dst = part + ((size_t)sig * T + t) * kRank + 4 * g;
#pragma unroll
        for (int jb = 0; jb < 20; ++jb)
            *reinterpret_cast<f32x4_t*>(dst + 16 * jb) = acc[jb];
    }
    // sum of squares of the token: lanes n, n + 16, n + 32, n + 48
    const float s1 = ssacc + __shfl_xor(ssacc, 16);
    const float s2 = s1 + __shfl_xor(s1, 32);
    if (g == 0 && tok_ok)
        ssq[(size_t)sig * T + t] = s2;
}

// ---------------------------------------------------------------------------
// P2: lo = sum_s rs_s * stream partial, as three bf16 planes in the tiled
// layout: for token tile u and K step ks, the three plane panels of 64 rows
// (tokens) x 4 chunks, 12 KB contiguous at chunk ((u * 10 + ks) * 3) * 256.
// Tokens of the last tile past T get zeros.
// ---------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(256) void prefill_lo(int T, int Tpad, const float* __restrict__ part,
                                                  const float* __restrict__ ssq, uint4* __restrict__ planes)
{
    constexpr int Q = S / 4;  // splits per stream
    const int idx = blockIdx.x * 256 + threadIdx.x;  // (token, chunk of 8 rank indices)
    const int t = idx / (kRank / 8);
    const int c8 = idx - t * (kRank / 8);
    if (t >= Tpad)
        return;
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        lo[e] = 0.f;
    if (t < T) {
        float v[4][8];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float ss = 0.f, sum[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sum[e] = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int sg = Q * s + q;
                ss += ssq[(size_t)sg * T + t];
                const float* pp = part + ((size_t)sg * T + t) * kRank + 8 * c8;
                const float4 a0 = *reinterpret_cast<const float4*>(pp), a1 = *reinterpret_cast<const float4*>(pp + 4);
                const float pv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sum[e] += pv[e];
            }
            const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[s][e] = sum[e] * rs;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            lo[e] = (v[0][e] + v[1][e]) + (v[2][e] + v[3][e]);
    }
    uint32_t hi[8], mi[8], l3[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        split3(lo[e], hi[e], mi[e], l3[e]);
    const int tile = t / kTok, tl = t - tile * kTok;
    const int ks = c8 >> 2, c = c8 & 3;
    uint4* dst = planes + (size_t)(tile * kUpSteps + ks) * kLoBlock + panel_slot(tl, c);
    dst[0] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    dst[kPlaneChunks] = make_uint4(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16));
    dst[2 * kPlaneChunks] = make_uint4(l3[0] | (l3[1] << 16), l3[2] | (l3[3] << 16), l3[4] | (l3[5] << 16), l3[6] | (l3[7] << 16));
}

// ---------------------------------------------------------------------------
// P3: up projection with the stream mix as its epilogue.  Workgroup b: XCD
// x = b % 8, q = b / 8: token tile q / 5, column group x + 8 (q % 5) (64
// columns).  Wave w computes columns c0 + 16 w .. +15 of all 4 streams for
// all 64 tokens: MFMA A = W_up rows (one block per stream), B = lo planes (4
// token blocks x 3 pieces); D then holds, in lane (n, g), token 16 tb + n and
// columns 4 g .. 4 g + 3 of every stream, so the mix is per lane.
// LDS stage (28 KB): W_up panel (256 rows: row 64 s + j = W_up row
// s * 2560 + c0 + j, 16 KB), then the 3 lo panels (12 KB).
// ---------------------------------------------------------------------------
constexpr int kUpWChunks = 4 * kUpCols * 4;      // 1024
constexpr int kUpStage = kUpWChunks + kLoBlock;  // 1792 chunks

template <bool HAS_P>
__global__ __launch_bounds__(256, 2) void prefill_upmix(int T, const uint4* __restrict__ planes,
                                                        const uint16_t* __restrict__ W_up,
                                                        const float* __restrict__ R,
                                                        const float* __restrict__ P,
                                                        float* __restrict__ out_mixed,
                                                        uint16_t* __restrict__ out_bf16,
                                                        uint16_t* __restrict__ out_fp16)
{
    __shared__ __align__(16) uint4 lds[2 * kUpStage];

    const int b = blockIdx.x;
    const int x = b & 7, q = b >> 3;
    const int tile = q / kGroupsPerXcd;
    const int cg = x + 8 * (q - tile * kGroupsPerXcd);
    const int t0 = tile * kTok, c0 = cg * kUpCols;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;

    // stage loads: wave instruction i (0..27): i < 16 fills W_up panel rows
    // 16 i .. 16 i + 15 (lane l: row 16 i + l / 4, chunk (l & 3) ^ ((row >> 2) & 3));
    // i >= 16 copies 1 KB of the lo block.  Wave w issues i = w + 4 k.
    const int wchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const uint16_t* wu_lane[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int prow = 16 * (wave + 4 * k) + (lane >> 2);  // panel row = 64 s + j
        wu_lane[k] = W_up + (size_t)((prow >> 6) * kWidth + c0 + (prow & 63)) * kRank + 8 * wchunk;
    }
    const uint4* lo_lane = planes + (size_t)tile * kUpSteps * kLoBlock + lane;
    auto issue = [&](int ks, int stage) {
        uint4* sb = lds + stage * kUpStage;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            dma16(wu_lane[k] + kKs * ks, sb + 64 * (wave + 4 * k));
#pragma unroll
        for (int k = 4; k < 7; ++k) {
            const int i = wave + 4 * k - 16;  // 1 KB piece of the lo block, 0..11
            dma16(lo_lane + (size_t)ks * kLoBlock + 64 * i, sb + kUpWChunks + 64 * i);
        }
    };

    f32x4_t acc[4][4];  // [token block][stream]
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[tb][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t lds0 = lds_addr(lds);
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        aoff[s] = 16 * panel_slot(64 * s + 16 * wave + n, g);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
        boff[tb] = 16 * (kUpWChunks + panel_slot(16 * tb + n, g));
    auto compute = [&](int stage) {
        const uint32_t sb = lds0 + 16 * stage * kUpStage;
        u32x4 op[16];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            op[s] = ds_read16(sb + aoff[s]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                op[4 + 3 * tb + p] = ds_read16(sb + boff[tb] + 16 * kPlaneChunks * p);
        lds_wait(op);
#pragma unroll
        for (int p = 2; p >= 0; --p)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[tb][s] = mfma16(op[s], op[4 + 3 * tb + p], acc[tb][s]);
    };

    issue(0, 0);
    ring_barrier<0>();
#pragma unroll 1
    for (int ks = 0; ks < kUpSteps - 1; ++ks) {
        issue(ks + 1, (ks + 1) & 1);
        compute(ks & 1);
        ring_barrier<0>();
    }
    compute((kUpSteps - 1) & 1);

    // gated = up (identity epilogue); mixed = sum_s gated_s * R'_s, then images.
    // Every R (and pending) load is issued before the first use (tokens past
    // T re-read token T - 1 and store nothing).
    const int c = c0 + 16 * wave + 4 * g;
    float4 rv[4][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int t = t0 + 16 * tb + n < T ? t0 + 16 * tb + n : T - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            rv[tb][s] = *reinterpret_cast<const float4*>(R + (size_t)t * kD + s * kWidth + c);
    }
    if (HAS_P) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int t = t0 + 16 * tb + n < T ? t0 + 16 * tb + n : T - 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 pv = *reinterpret_cast<const float4*>(P + (size_t)t * kD + s * kWidth + c);
                rv[tb][s].x += pv.x;
                rv[tb][s].y += pv.y;
                rv[tb][s].z += pv.z;
                rv[tb][s].w += pv.w;
            }
        }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int t = t0 + 16 * tb + n;
        const float r[4][4] = {{rv[tb][0].x, rv[tb][0].y, rv[tb][0].z, rv[tb][0].w},
                               {rv[tb][1].x, rv[tb][1].y, rv[tb][1].z, rv[tb][1].w},
                               {rv[tb][2].x, rv[tb][2].y, rv[tb][2].z, rv[tb][2].w},
                               {rv[tb][3].x, rv[tb][3].y, rv[tb][3].z, rv[tb][3].w}};
        float m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m[i] = (acc[tb][0][i] * r[0][i] + acc[tb][1][i] * r[1][i]) +
                   (acc[tb][2][i] * r[2][i] + acc[tb][3][i] * r[3][i]);
        if (t < T) {
            const size_t o = (size_t)t * kWidth + c;
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

int tiles_of(int tokens)
{
    return (tokens + kTok - 1) / kTok;
}

// P1's split count: stream halves when that already gives a workgroup per
// CU, else stream quarters.
int splits_for(int tokens)
{
    return (tokens + kDnTok - 1) / kDnTok * 8 >= 256 ? 8 : 16;
}

// (split, token) slots of the partial array, enough for any chunk of up to
// `chunk` tokens
size_t part_slots(int chunk)
{
    size_t most = 0;
    for (int tc = chunk; tc > 0; tc -= kDnTok) {  // splits_for changes only at tile boundaries
        const size_t n = (size_t)splits_for(tc) * tc;
        most = most > n ? most : n;
    }
    return most;
}

}  // namespace

size_t prefill_scratch_bytes(int chunk)
{
    const size_t tpad = (size_t)tiles_of(chunk) * kTok;
    return sizeof(float) * part_slots(chunk) * (kRank + 1) + sizeof(uint16_t) * 3 * tpad * kRank + 512;
}

hipError_t launch_prefill(int64_t T, const float* R, const float* P, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, void* scratch, int chunk,
                          hipStream_t stream)
{
    const size_t slots = part_slots(chunk);
    float* part = static_cast<float*>(scratch);  // [S][Tc][320]
    float* ssq = part + slots * kRank;             // [S][Tc]
    uint4* planes = reinterpret_cast<uint4*>(      // tiled lo planes
        (reinterpret_cast<uintptr_t>(ssq + slots) + 255) & ~uintptr_t(255));
    for (int64_t c0 = 0; c0 < T; c0 += chunk) {
        const int Tc = (int)(T - c0 < chunk ? T - c0 : chunk);
        const size_t in_off = (size_t)c0 * kD, out_off = (size_t)c0 * kWidth;
        const float* Rc = R + in_off;
        const float* Pc = P ? P + in_off : nullptr;
        const int S = splits_for(Tc);
        const dim3 grid1(S * ((Tc + kDnTok - 1) / kDnTok)), block1(kDnWaves * 64);
        if (S == 8) {
            if (Pc)
                hipLaunchKernelGGL((prefill_down<8, true>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
            else
                hipLaunchKernelGGL((prefill_down<8, false>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
        } else {
            if (Pc)
                hipLaunchKernelGGL((prefill_down<16, true>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
            else
                hipLaunchKernelGGL((prefill_down<16, false>), grid1, block1, 0, stream, Tc, Rc, Pc, w_norm, W_down, part, ssq);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int tiles = tiles_of(Tc);
        const int items = tiles * kTok * (kRank / 8);
        if (S == 8)
            hipLaunchKernelGGL(prefill_lo<8>, dim3((items + 255) / 256), dim3(256), 0, stream, Tc, tiles * kTok, part, ssq, planes);
        else
            hipLaunchKernelGGL(prefill_lo<16>, dim3((items + 255) / 256), dim3(256), 0, stream, Tc, tiles * kTok, part, ssq, planes);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int grid3 = 8 * kGroupsPerXcd * tiles;
        if (Pc)
            hipLaunchKernelGGL(prefill_upmix<true>, dim3(grid3), dim3(256), 0, stream, Tc, planes, W_up, Rc, Pc,
                               out_mixed + out_off, out_bf16 + out_off, out_fp16 + out_off);
        else
            hipLaunchKernelGGL(prefill_upmix<false>, dim3(grid3), dim3(256), 0, stream, Tc, planes, W_up, Rc, Pc,
                               out_mixed + out_off, out_bf16 + out_off, out_fp16 + out_off);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace hc
