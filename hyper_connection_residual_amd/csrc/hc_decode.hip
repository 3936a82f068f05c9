// hc_decode.hip -- the hyper-connection read for short windows (T <= 8 tokens)
// as ONE kernel launch on gfx950.
//
// What it computes is the read of "#315 hc: the multi-token hyper-connection
// read split finer" (norm, down projection, up projection) with the norm folded
// into the column-sliced down projection as in "#2488 sycl/A770", Summary
// item 4 (each slice stages R' * w_norm unscaled with its sum of squares; the
// reduction applies each stream's rs to that stream's partial dots), the
// reduction computed once per output row (#2488 items 1 and 3), and the up
// projection followed by the identity epilogue and the 4-stream mix of
// "#1370 prefill", "What it does" (the 4 streams of one column are mixed in
// registers, then the BF16/FP16 images are written).
//
// gfx950 design (the pages' kernels were written for RDNA2, Turing, Ada and
// Arc; none of their mechanics is reused):
//
// * 256 workgroups x 8 waves: exactly one workgroup per CU, each streaming the
//   same 51 KB of weights: a 40-row x 320-column tile of W_down and the 40 W_up
//   rows of its 10 output columns (4 runs of 10 consecutive rows).
// * The tiles go straight from memory into LDS (global_load_lds_dwordx4), each
//   wave instruction fetching 8 whole 128-byte lines.  Measured on MI355X:
//   loading the same bytes in the matrix cores' operand layout (16 rows x 64
//   bytes per instruction, half lines) lands the last byte over 1 us later.
//   Inside LDS the 8 chunks of each line are XOR-swizzled by row, so the
//   operand reads of 16 rows hit distinct banks.
// * Every load is issued at entry: W_down first by waves 0-5, then (after a
//   barrier, so the CU's queue holds W_down ahead of it) W_up by waves 6-7.
//   A CU serves its vector memory requests in order across waves (measured: a
//   load that hits L2 in 0.08 us takes over 1 us while another wave of the CU
//   has cold loads outstanding), so nothing may be issued late.  Barriers are
//   raw s_barrier with an LDS wait only: the compiler's __syncthreads() also
//   waits for the LDS-bound loads still in flight.
// * Both projections run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
//   with tokens as the M dimension.  Each fp32 activation is split exactly into
//   three bf16 pieces (hi + mid + lo3 == x), so every product is exact and the
//   result stays fp32-faithful.  Each piece has its own accumulator (three
//   independent MFMA chains), and the K range is split over two waves.
// * Two hand-offs, no grid barrier.  XCD x owns lo rows [40 x, 40 x + 40):
//   its 32 workgroups publish partial dots into the XCD's L2, 20 of them each
//   reduce two rows (one XCD-local hop) and publish lo device-wide, and every
//   workgroup gathers all of lo (one device-wide hop).  Hand-off words are 64
//   bits holding the payload and the launch's generation number, written once
//   with one store; a consumer polls one sentinel word per producer (its last
//   store), then reads the data once and re-reads only words whose tag is
//   still old.  Every workgroup counts its launches in its own slot, so all of
//   them agree on the generation without host involvement (the launch is
//   graph-capture safe).  Every wait is bounded.
#include "hc_internal.h"

// No multiply-add contraction anywhere in this file: a butterfly sum must give
// every lane the same bits, and a fused multiply-add would add the lane's own
// unrounded product to its partner's rounded one.
#pragma clang fp contract(off)

// Instrumentation hook: empty in the library; a timing build may define it to
// record when workgroups pass the numbered points.
#ifndef HC_PROBE
#define HC_PROBE(point, cond) ((void)0)
#endif
// Counting hook: empty in the library; a timing build may record how many
// polling rounds each wait took (site: which wait).
#ifndef HC_COUNT
#define HC_COUNT(site, kind, value, cond) ((void)0)
#endif

namespace hc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr long long kWaitTicks = 5000000;  // 50 ms of the 100 MHz wall clock
constexpr int kTileRows = 40;               // rows of a weight tile
constexpr int kTileChunks = kRank / 8;      // 16-byte chunks per tile row (40)
constexpr int kTileInstr = kTileRows * kTileChunks / 64;  // wave instructions per tile (25)
constexpr int kUpCols = kWidth / kDecWGs;   // output columns per workgroup (10)
constexpr int kYRow = kDecCols + 8;         // padded LDS row of an activation plane (bf16)
constexpr int kLoRow = kRank + 8;           // padded LDS row of a lo plane (bf16)
constexpr int kStageItems = kDecCols / 4;   // float4 activation items per token (80)
// scratch layout (in 64-bit words from the base): partial dots, slice sums of
// squares, lo, then the 32-bit generation counters and the timeout counter
constexpr size_t kPartWords = (size_t)kDecXcds * kDecPerXcd * kDecRowsPerXcd * kDecMaxT;
constexpr size_t kSsqWords = (size_t)kDecXcds * kDecPerXcd * kDecMaxT;
constexpr size_t kLoWords = (size_t)kDecMaxT * kRank;

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// x == hi + mid + lo3 exactly, each a bf16 (returned as its 16-bit pattern).
// hi keeps the top 8 significant bits (truncation); the remainders are exact
// in fp32 and the last one has at most 8 significant bits.
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// Butterfly sums; every lane of the group ends with the same bits.
__device__ __forceinline__ float sum4(float v)
{
    v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    return v;
}
__device__ __forceinline__ float sum8(float v)
{
    v = sum4(v);
    v += dpp<0x141>(v);  // row_half_mirror: the other quad of the 8
    return v;
}

// Workgroup barrier that waits for this wave's LDS operations only.  Loads
// into LDS still in flight are waited for explicitly, by the waves that issued
// them, before the barrier after which their data is read.
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_all_loads()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Makes a loaded value "produced here": the compiler may not hoist its use
// (and the wait for its load) above this point, e.g. above a barrier.
__device__ __forceinline__ void pin(float& v)
{
    asm volatile("" : "+v"(v));
}
__device__ __forceinline__ void pin(uint32_t& v)
{
    asm volatile("" : "+v"(v));
}

// A hand-off word for every CU of the device: the store writes through to
// memory (agent scope).
__device__ __forceinline__ void st_word(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A hand-off word for the CUs of this XCD only: the store stays in the XCD's
// L2 instead of writing through to memory (about 4x faster).
__device__ __forceinline__ void st_word_xcd(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Two aligned hand-off words (16 bytes) read in one load at device coherence
// (sc1: the load skips the CU's L1; it finds a line another CU of this XCD
// left in the shared L2, and a line written from another XCD in memory).
// Each 8-byte word was written by one store.  `base` must be the same for the
// whole wave (it becomes a buffer descriptor in scalar registers); the
// per-lane position goes in `index` (in words, even).  A load that may hit the
// CU's L1 (sc0 or none) is not used for hand-offs: it can keep returning a
// stale line.
__device__ __forceinline__ uint4 ld_words2(const uint64_t* base, int index)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint64_t*>(base), 0, 0x7fffffff, 0x00020000);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, index * 8, 0, 16 /* sc1 */));
}
__device__ __forceinline__ uint64_t tag_f32(float v, uint32_t gen)
{
    return (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32);
}
__device__ __forceinline__ void note_timeout(uint32_t* timeouts)
{
    __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spins until the sentinel words of every lane that has them (index >= 0)
// carry `gen` in their high 32 bits.  Returns false after a timeout (counted
// once).
__device__ __forceinline__ bool wait_sentinels(const uint64_t* base, int sent, const uint64_t* base2, int sent2,
                                               uint32_t gen, long long t0, int lane, uint32_t* timeouts,
                                               int site)
{
    [[maybe_unused]] int rounds = 0;
    while (true) {
        ++rounds;
        bool ok = true;
        if (sent >= 0) {
            const uint4 a = ld_words2(base, sent & ~1);
            ok = ((sent & 1) ? a.w : a.y) == gen;
        }
        if (sent2 >= 0) {
            const uint4 a = ld_words2(base2, sent2 & ~1);
            ok = ok && ((sent2 & 1) ? a.w : a.y) == gen;
        }
        if (__all(ok)) {
            HC_COUNT(site, 0, rounds, lane == 0);
            return true;
        }
        if (wall_clock64() - t0 > kWaitTicks) {
            if (lane == 0)
                note_timeout(timeouts);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Reads the T consecutive words at base + idx (idx even) into v once their
// tags carry `gen`, re-reading until they all do.  `live` false: nothing is
// read (a timeout already happened).
template <int T>
__device__ __forceinline__ void read_words(const uint64_t* base, int idx, uint32_t gen, bool live, long long t0,
                                           int lane, float (&v)[T], uint32_t* timeouts, int site)
{
    constexpr int NP = (T + 1) / 2;
#pragma unroll
    for (int t = 0; t < T; ++t)
        v[t] = 0.f;
    bool done = !live;
    [[maybe_unused]] int rounds = 0;
    while (true) {
        ++rounds;
        if (!done) {
            bool ok = true;
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                const uint4 a = ld_words2(base, idx + 2 * q);
                ok = ok && a.y == gen && (2 * q + 1 >= T || a.w == gen);
                v[2 * q] = __uint_as_float(a.x);
                if (2 * q + 1 < T)
                    v[2 * q + 1] = __uint_as_float(a.z);
            }
            done = ok;
        }
        if (__all(done)) {
            HC_COUNT(site, 1, rounds, lane == 0);
            return;
        }
        if (wall_clock64() - t0 > kWaitTicks) {
            if (lane == 0)
                note_timeout(timeouts);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Chunk placement inside a tile line: the 8 chunks of a 128-byte line are
// stored XOR-swizzled by row, so 16 lanes reading the same chunk column of 16
// consecutive rows hit distinct 16-byte bank groups (with 32 or 64 banks).
__device__ __forceinline__ int swz(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}
// LDS position (in 16-byte chunks) of chunk j (0..39) of tile row `row`.
__device__ __forceinline__ int tile_pos(int row, int j)
{
    return row * kTileChunks + (j & ~7) + ((j & 7) ^ swz(row));
}
// Wave instruction q of a tile load: lane l fills LDS position p = 64 q + l,
// i.e. (row, line, slot); it fetches that row's chunk 8 line + (slot ^ swz).
// Eight consecutive lanes fetch one whole 128-byte line.
__device__ __forceinline__ void tile_lane(int q, int lane, int& row, int& j)
{
    const int p = 64 * q + lane;
    row = p / kTileChunks;
    const int rem = p - row * kTileChunks;
    j = (rem & ~7) + ((rem & 7) ^ swz(row));
}
// 16 bytes per lane from memory into LDS: lane l's bytes land at
// lds_wave_base + 16 l (the base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const uint16_t* g, uint4* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

// The arguments the first loads need come first: the library is built with
// kernel-argument preloading, so they arrive in SGPRs and no wave has to fetch
// them from memory (a fetch that queues behind the other CUs' weight traffic).
template <int T>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const uint16_t* __restrict__ W_down, const uint16_t* __restrict__ W_up, const float* __restrict__ R,
    const float* __restrict__ P, const float* __restrict__ w_norm, uint64_t* __restrict__ scratch,
    float* __restrict__ out_mixed, uint16_t* __restrict__ out_bf16, uint16_t* __restrict__ out_fp16)
{
    static_assert(T >= 1 && T <= kDecMaxT, "short-window kernel takes 1..8 tokens");
    static_assert(kTileRows * kTileChunks == 64 * kTileInstr, "tiles are whole wave instructions");
    static_assert(kDecRowsPerXcd == kTileRows && kUpCols * 4 == kTileRows && kUpCols * kDecWGs == kWidth,
                  "tiles of 40 rows");
    static_assert(kDecCols == 8 * kTileChunks && kWidth % kDecCols == 0, "a W_down tile lies in one stream");
    static_assert(kStageItems * kDecMaxT <= 2 * 384, "two staging passes of waves 0-5");
    static_assert(kTileRows * kDecMaxT <= 5 * 64, "five mix-operand passes of wave 6");
    __shared__ __align__(16) uint4 wdt[kTileRows * kTileChunks];  // W_down tile
    __shared__ __align__(16) uint4 wut[kTileRows * kTileChunks];  // W_up tile, row 10 s + r = column 10 b + r of stream s
    __shared__ __align__(16) uint16_t ypl[3][T][kYRow];            // y = R' * w_norm, 3 bf16 pieces
    __shared__ __align__(16) uint16_t lpl[3][T][kLoRow];           // lo, 3 bf16 pieces
    __shared__ float sspart[T][kStageItems];                      // per-item sums of squares
    __shared__ __align__(16) f32x4_t comb[3][64];                 // second K half of the accumulators
    __shared__ float rpl[T][kTileRows];                           // R' of this workgroup's columns

    DecodeScratch s;
    s.part = scratch;
    s.ssq = s.part + kPartWords;
    s.lo = s.ssq + kSsqWords;
    s.gen = reinterpret_cast<uint32_t*>(s.lo + kLoWords);
    s.timeouts = s.gen + kDecWGs;
    const int b = blockIdx.x;
    const int x = b & 7;   // XCD
    const int i = b >> 3;  // index inside the XCD, 0..31
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // MFMA column slot (B / D operand)
    const int g = lane >> 4;  // MFMA k-group (A / B operand) and D row group
    // this launch's generation: one more than the launches this workgroup has
    // seen.  Every lane loads the counter (no per-lane branch); the value is
    // used only after the weights have landed.
    uint32_t seen = __hip_atomic_load(&s.gen[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0 && __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) != x)
        note_timeout(s.timeouts);  // not on the XCD the hand-offs assume: results invalid
    HC_PROBE(0, threadIdx.x == 0);

    // ---- (1) loads.  Waves 0-5: the W_down tile (rows 40 x + row, columns
    //      320 i + 8 j ..), then the activations of columns [320 i, 320 i + 320).
    //      Loads issued before a barrier are unconditional (items past the end
    //      re-read item 0; a missing pending re-reads R): a conditional load
    //      makes the compiler merge registers, which waits for every load.
    const float* Pm = P ? P : R;
    float4 rv[2], pv[2], wv[2];
    if (wave < 6) {
        for (int q = wave; q < kTileInstr; q += 6) {
            int row, j;
            tile_lane(q, lane, row, j);
            dma16(W_down + (size_t)(kDecRowsPerXcd * x + row) * kD + kDecCols * i + 8 * j, wdt + 64 * q);
        }
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int it = threadIdx.x + 384 * pass;
            const int itc = it < kStageItems * T ? it : 0;
            const int at = itc / kStageItems, f = itc - at * kStageItems;
            const size_t o = (size_t)at * kD + kDecCols * i + 4 * f;
            rv[pass] = *reinterpret_cast<const float4*>(R + o);
            pv[pass] = *reinterpret_cast<const float4*>(Pm + o);
            wv[pass] = *reinterpret_cast<const float4*>(w_norm + kDecCols * i + 4 * f);
        }
    }
    wg_barrier();  // B0: every W_down request is queued ahead of the W_up ones
    // Waves 6-7: the W_up tile (rows s * 2560 + 10 b + r), then (wave 6) R and
    // pending of this workgroup's 40 columns for the mix.
    float mr[5], mp[5];
    if (wave >= 6) {
        for (int q = wave - 6; q < kTileInstr; q += 2) {
            int row, j;
            tile_lane(q, lane, row, j);
            const int k = (row / kUpCols) * kWidth + kUpCols * b + row % kUpCols;
            dma16(W_up + (size_t)k * kRank + 8 * j, wut + 64 * q);
        }
        if (wave == 6) {
#pragma unroll
            for (int pass = 0; pass < 5; ++pass) {
                const int it = lane + 64 * pass;  // (token, tile row)
                const int itc = it < kTileRows * T ? it : 0;
                const int at = itc / kTileRows, row = itc - at * kTileRows;
                const size_t o = (size_t)at * kD + (row / kUpCols) * kWidth + kUpCols * b + row % kUpCols;
                mr[pass] = R[o];
                mp[pass] = Pm[o];
            }
        }
    }

    // ---- (2) waves 0-5 stage y = R' * w_norm (unscaled: the norm is folded
    //      into the reduction), its sums of squares, and the exact 3-way split.
    if (wave < 6) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int it = threadIdx.x + 384 * pass;
            if (it < kStageItems * T) {
                const int at = it / kStageItems, f = it - at * kStageItems;
                const float r[4] = {P ? rv[pass].x + pv[pass].x : rv[pass].x, P ? rv[pass].y + pv[pass].y : rv[pass].y,
                                    P ? rv[pass].z + pv[pass].z : rv[pass].z, P ? rv[pass].w + pv[pass].w : rv[pass].w};
                const float w[4] = {wv[pass].x, wv[pass].y, wv[pass].z, wv[pass].w};
                float ss = 0.f;
                uint32_t hi[4], mi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ss += r[e] * r[e];
                    split3(r[e] * w[e], hi[e], mi[e], lo[e]);
                }
                sspart[at][f] = ss;
                const int col = 4 * f;
                *reinterpret_cast<uint2*>(&ypl[0][at][col]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2*>(&ypl[1][at][col]) = make_uint2(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16));
                *reinterpret_cast<uint2*>(&ypl[2][at][col]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
        wait_all_loads();  // this wave's part of the W_down tile is in LDS
    }
    wg_barrier();  // B1: activations staged, W_down tile complete
    HC_PROBE(1, threadIdx.x == 0);

    // ---- (3) down projection: wave w < 6 takes rows 16 (w % 3) .. +15 of the
    //      tile (block 2: rows 32..39, its upper 8 slots repeat them) over
    //      K steps 5 (w / 3) .. +4 of 32 columns.
    f32x4_t dacc = {0.f, 0.f, 0.f, 0.f};
    if (wave < 6) {
        const int nb = wave % 3, kh = wave / 3;
        const int row = nb < 2 ? 16 * nb + n : 32 + (n & 7);
        const int m = lane & 15;  // A row = token
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
        for (int qq = 0; qq < 5; ++qq) {
            const int q = 5 * kh + qq;
            const uint4 wb = wdt[tile_pos(row, 4 * q + g)];
            const int col = 32 * q + 8 * g;
            uint4 ah = make_uint4(0, 0, 0, 0), am = ah, al = ah;
            if (m < T) {
                ah = *reinterpret_cast<const uint4*>(&ypl[0][m][col]);
                am = *reinterpret_cast<const uint4*>(&ypl[1][m][col]);
                al = *reinterpret_cast<const uint4*>(&ypl[2][m][col]);
            }
            a0 = mfma16(ah, wb, a0);
            a1 = mfma16(am, wb, a1);
            a2 = mfma16(al, wb, a2);
        }
        dacc = a0 + (a1 + a2);
        if (kh == 1)
            comb[nb][lane] = dacc;
    }
    HC_PROBE(2, threadIdx.x == 0);
    wg_barrier();  // Bc1: second K halves in LDS
    pin(seen);
    const uint32_t gen = (uint32_t)__builtin_amdgcn_readfirstlane((int)seen) + 1u;

    if (wave < 3) {
        // ---- (4) partial dots of rows 16 nb + n, tokens 4 g + e, into the XCD's L2
        dacc = dacc + comb[wave][lane];
        const int row = 16 * wave + n;
        if (row < kTileRows) {
            uint64_t* dst = s.part + (((size_t)x * kDecPerXcd + i) * kTileRows + row) * kDecMaxT + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e < T)
                    st_word_xcd(dst + e, tag_f32(dacc[e], gen));
        }
    } else if (wave == 3) {
        // ---- (4') the slice's sum of squares per token: lane 8 t + p sums 10
        //      of token t's 80 item sums, then the 8 lanes combine theirs
        const int tt = lane >> 3, p = lane & 7;
        float ss = 0.f;
        if (tt < T) {
#pragma unroll
            for (int f = 0; f < 10; ++f)
                ss += sspart[tt][10 * p + f];
        }
        ss = sum8(ss);
        if (tt < T && p == 0)
            st_word_xcd(&s.ssq[((size_t)x * kDecPerXcd + i) * kDecMaxT + tt], tag_f32(ss, gen));
    }
    HC_PROBE(3, threadIdx.x == 0);

    if (wave == 7 && i < kDecReducers) {
        // ---- (5) hop 1: rows 40 x + 2 i + r (r = lane / 32) over the XCD's 32
        //      partials (lane % 32 = source workgroup), each stream's rs from
        //      its 8 slices' sums of squares, lo published device-wide.
        const int r = lane >> 5, src = lane & 31;
        const int row = 2 * i + r;
        const int pidx = ((x * kDecPerXcd + src) * kTileRows + row) * kDecMaxT;
        const int sidx = (x * kDecPerXcd + src) * kDecMaxT;
        const long long t0 = wall_clock64();
        const bool live = wait_sentinels(s.part, pidx + T - 1, s.ssq, sidx + T - 1, gen, t0, lane, s.timeouts, 0);
        float v[T], q[T];
        read_words<T>(s.part, pidx, gen, live, t0, lane, v, s.timeouts, 0);
        read_words<T>(s.ssq, sidx, gen, live, t0, lane, q, s.timeouts, 1);
        HC_PROBE(12, lane == 0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            // lanes 8 s .. 8 s + 7 (of each half) hold the slices of stream s
            const float ss = sum8(q[t]);
            const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
            const float y = sum8(v[t]) * rs;
            const float y01 = y + dpp<0x128>(y);         // row_ror:8: streams (0 + 1), (2 + 3)
            const float lo = y01 + __shfl_xor(y01, 16);  // (s0 + s1) + (s2 + s3)
            if (src == t)
                st_word(&s.lo[(size_t)t * kRank + kDecRowsPerXcd * x + row], tag_f32(lo, gen));
        }
        HC_PROBE(13, lane == 0);
    }

    if (wave == 6) {
        // ---- (6') R' = R + pending of this workgroup's columns, for the mix
#pragma unroll
        for (int pass = 0; pass < 5; ++pass) {
            const int it = lane + 64 * pass;
            pin(mr[pass]);
            pin(mp[pass]);
            if (it < kTileRows * T) {
                const int at = it / kTileRows, row = it - at * kTileRows;
                rpl[at][row] = P ? mr[pass] + mp[pass] : mr[pass];
            }
        }
    }
    wg_barrier();  // Bh: this workgroup's hop 1 is done before any hop-2 load
                   // (a CU serves loads in order: a hop-2 load behind which a
                   // hop-1 load waits would delay every consumer of this row)
    if (wave == 0) {
        // ---- (6) hop 2, first: wait for this XCD's 20 reducers (their odd
        //      row, last token).  The other XCDs run in step with this one, so
        //      their lo is then due too; polling only local words keeps the
        //      device-wide traffic to one bulk read per workgroup.
        const long long t0 = wall_clock64();
        const int sent = lane < kDecReducers ? (T - 1) * kRank + kDecRowsPerXcd * x + 2 * lane + 1 : -1;
        HC_PROBE(15, lane == 0);
        wait_sentinels(s.lo, sent, s.lo, -1, gen, t0, lane, s.timeouts, 2);  // (a timeout is counted; the reads below are bounded too)
        HC_PROBE(14, lane == 0);
    }
    wg_barrier();  // Bs
    if (wave < 4) {
        // ---- (6) hop 2, then: wave w reads lo rows [80 w, 80 w + 80) (XCDs
        //      2 w, 2 w + 1), two rows per slot, re-reading words whose tag is
        //      still old, and stages their 3 bf16 pieces
        constexpr int NS = (40 * T + 63) / 64;  // slots per lane
        const int rbase = 80 * wave;
        const long long t0 = wall_clock64();
        uint4 lw[NS];
        bool done[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            lw[k] = make_uint4(0, 0, 0, 0);
            done[k] = lane + 64 * k >= 40 * T;
        }
        [[maybe_unused]] int rounds = 0;
        while (true) {
            ++rounds;
            bool all = true;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int sl = lane + 64 * k;
                if (!done[k]) {
                    lw[k] = ld_words2(s.lo, (sl / 40) * kRank + rbase + 2 * (sl % 40));
                    done[k] = lw[k].y == gen && lw[k].w == gen;
                }
                all = all && done[k];
            }
            if (__all(all)) {
                HC_COUNT(2, 1, rounds, wave == 0 && lane == 0);
                break;
            }
            if (wall_clock64() - t0 > kWaitTicks) {
                if (lane == 0)
                    note_timeout(s.timeouts);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int sl = lane + 64 * k;
            if (sl < 40 * T) {
                const int tt = sl / 40;
                const int jr = rbase + 2 * (sl % 40);
                uint32_t h0, m0, l0, h1, m1, l1;
                split3(__uint_as_float(lw[k].x), h0, m0, l0);
                split3(__uint_as_float(lw[k].z), h1, m1, l1);
                *reinterpret_cast<uint32_t*>(&lpl[0][tt][jr]) = h0 | (h1 << 16);
                *reinterpret_cast<uint32_t*>(&lpl[1][tt][jr]) = m0 | (m1 << 16);
                *reinterpret_cast<uint32_t*>(&lpl[2][tt][jr]) = l0 | (l1 << 16);
            }
        }
        HC_PROBE(7, wave == 0 && lane == 0);
    }
    if (wave >= 6)
        wait_all_loads();  // the W_up tile is in LDS
    HC_PROBE(6, wave == 6 && lane == 0);
    wg_barrier();  // B2: lo staged, W_up tile complete
    HC_PROBE(8, threadIdx.x == 0);

    // ---- (7) up projection: wave w < 6 takes output columns 4 (w % 3) .. +3
    //      of this workgroup (block 2: columns 8, 9; its slots for the block's
    //      columns 2, 3 repeat them and store nothing) over K steps
    //      5 (w / 3) .. +4; slot n = 4 (column) + stream.
    const int u = wave % 3;
    const int cc = n >> 2, st = n & 3;
    const bool owner = 4 * u + cc < kUpCols;
    const int cr = owner ? 4 * u + cc : 4 * u + (cc & 1);  // column inside the workgroup's 10
    f32x4_t uacc = {0.f, 0.f, 0.f, 0.f};
    if (wave < 6) {
        const int kh = wave / 3;
        const int row = st * kUpCols + cr;
        const int m = lane & 15;
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
        for (int qq = 0; qq < 5; ++qq) {
            const int q = 5 * kh + qq;
            const uint4 wb = wut[tile_pos(row, 4 * q + g)];
            const int jc = 32 * q + 8 * g;
            uint4 ah = make_uint4(0, 0, 0, 0), am = ah, al = ah;
            if (m < T) {
                ah = *reinterpret_cast<const uint4*>(&lpl[0][m][jc]);
                am = *reinterpret_cast<const uint4*>(&lpl[1][m][jc]);
                al = *reinterpret_cast<const uint4*>(&lpl[2][m][jc]);
            }
            a0 = mfma16(ah, wb, a0);
            a1 = mfma16(am, wb, a1);
            a2 = mfma16(al, wb, a2);
        }
        uacc = a0 + (a1 + a2);
        if (kh == 1)
            comb[u][lane] = uacc;
    }
    wg_barrier();  // Bc2
    if (wave < 3) {
        // gated = up (identity epilogue); mix the 4 streams of the column
        uacc = uacc + comb[u][lane];
        const int c = kUpCols * b + cr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tt = 4 * g + e;
            const float rp = rpl[tt < T ? tt : 0][st * kUpCols + cr];
            const float mixed = sum4(uacc[e] * rp);  // (s0 + s1) + (s2 + s3)
            if (st == 0 && owner && tt < T) {
                const size_t o = (size_t)tt * kWidth + c;
                out_mixed[o] = mixed;
                out_bf16[o] = __builtin_bit_cast(uint16_t, (__bf16)mixed);
                out_fp16[o] = __builtin_bit_cast(uint16_t, (_Float16)mixed);
            }
        }
        HC_PROBE(9, wave == 0 && lane == 0);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&s.gen[b], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t decode_scratch_bytes()
{
    return sizeof(uint64_t) * (kPartWords + kSsqWords + kLoWords) + sizeof(uint32_t) * (kDecWGs + 64);
}

void decode_scratch_carve(void* base, DecodeScratch* s)
{
    s->part = static_cast<uint64_t*>(base);
    s->ssq = s->part + kPartWords;
    s->lo = s->ssq + kSsqWords;
    s->gen = reinterpret_cast<uint32_t*>(s->lo + kLoWords);
    s->timeouts = s->gen + kDecWGs;
}

hipError_t decode_resident_blocks(int* blocks_per_cu)
{
    // the largest-LDS instance bounds residency for every T
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void*>(&decode_kernel<kDecMaxT>), kDecThreads, 0);
}

hipError_t launch_decode(int T, const float* R, const float* P, const float* w_norm,
                         const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                         uint16_t* out_bf16, uint16_t* out_fp16, const DecodeScratch& s,
                         hipStream_t stream)
{
    uint64_t* scratch = s.part;  // the carve's base: the kernel derives the rest
    void* args[] = {&W_down, &W_up, &R, &P, &w_norm, &scratch, &out_mixed, &out_bf16, &out_fp16};
    const void* fn = nullptr;
    switch (T) {
    case 1: fn = reinterpret_cast<const void*>(&decode_kernel<1>); break;
    case 2: fn = reinterpret_cast<const void*>(&decode_kernel<2>); break;
    case 3: fn = reinterpret_cast<const void*>(&decode_kernel<3>); break;
    case 4: fn = reinterpret_cast<const void*>(&decode_kernel<4>); break;
    case 5: fn = reinterpret_cast<const void*>(&decode_kernel<5>); break;
    case 6: fn = reinterpret_cast<const void*>(&decode_kernel<6>); break;
    case 7: fn = reinterpret_cast<const void*>(&decode_kernel<7>); break;
    case 8: fn = reinterpret_cast<const void*>(&decode_kernel<8>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(kDecWGs), dim3(kDecThreads), args, 0, stream);
}

}  // namespace hc
