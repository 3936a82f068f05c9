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
// * 256 workgroups x 8 waves, one per CU, each streaming 51 KB of weights.  A
//   CU serves its vector memory requests in order across its waves (measured:
//   a load that hits L2 in 0.08 us takes over 1 us while another wave of the
//   CU has cold loads outstanding), so a CU that polls for a hand-off while
//   its own weight loads are in flight waits for all of them.  The workgroups
//   of each XCD therefore split in two roles that never overlap: 16 "down"
//   workgroups stream W_down, publish partial dots and end without waiting for
//   anything; 16 "up" workgroups stream W_up and do every wait after it has
//   landed.  Both halves issue all their loads at entry, so the whole 13 MB is
//   in flight at once.
// * The tiles go straight from memory into LDS (global_load_lds_dwordx4), each
//   wave instruction fetching 8 whole 128-byte lines.  Measured on MI355X:
//   loading the same bytes in the matrix cores' operand layout (16 rows x 64
//   bytes per instruction, half lines) lands the last byte over 1 us later.
//   Inside LDS the chunks of each row are swizzled so that the operand reads
//   of 16 rows hit distinct banks.  Barriers are raw s_barrier with an LDS
//   wait only: the compiler's __syncthreads() also waits for LDS-bound loads.
// * Both projections run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
//   with tokens as the M dimension.  Each fp32 activation is split exactly into
//   three bf16 pieces (hi + mid + lo3 == x), so every product is exact and the
//   result stays fp32-faithful.  Each piece has its own accumulator (three
//   independent MFMA chains).
// * Two hand-offs, no grid barrier.  XCD x owns lo rows [40 x, 40 x + 40): up
//   workgroups reduce the 16 partials of 3 rows each through the XCD's L2
//   (hop 1) and publish lo device-wide; every up workgroup gathers all of lo
//   (hop 2).  Hand-off words are 64 bits holding the payload and the launch's
//   generation number, written once with one store; a consumer polls the data
//   words themselves (device-coherent loads, which see a write-through store
//   from another XCD even when they started polling before it), with every
//   load of a polling round in flight at once.  Every workgroup counts its
//   launches in its own slot, so all of them agree on the generation without
//   host involvement (the launch is graph-capture safe).  Every wait is
//   bounded.
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
constexpr int kTileChunks = 3200;           // 16-byte chunks in either weight tile (51,200 bytes)
constexpr int kTileInstr = kTileChunks / 64;  // wave instructions per tile (50)
constexpr int kDnRowChunks = kDecDownCols / 8;  // chunks per W_down tile row (80)
constexpr int kUpRowChunks = kRank / 8;         // chunks per W_up tile row (40)
constexpr int kUpRows = 4 * kDecUpCols;         // W_up tile rows (80): row 20 s + r
constexpr int kStageItems = kDecDownCols / 4;   // float4 activation items per token (160)
constexpr int kYRow = kDecDownCols + 8;         // padded LDS row of an activation plane (bf16)
constexpr int kLoRow = kRank + 8;               // padded LDS row of a lo plane (bf16)
// Scratch layout (in 64-bit words from the base): partial dots, slice sums of
// squares, lo, then the 32-bit generation counters and the timeout counter.
// Every producer writes whole 128-byte lines (16 words), padding unused token
// slots: a line the XCD's L2 holds only in part is filled from memory when it
// is read, which costs a memory round trip (about 0.5 us while the weights
// stream) instead of an L2 hit.
//   part [8 xcd][16 down wg][40 rows][8 tokens]     (two rows per line)
//   ssq  [8 xcd][16 down wg][16]                    (tokens 0..7, then padding)
//   lo   [8 replica][8 xcd][16 reducer] blocks of 64 words, the first 32 being
//        [8 tokens][4 rows] (rows 3 u .. 3 u + 2, padding).  Each reducer writes
//        one replica per consumer XCD, and the blocks are spread 512 bytes
//        apart: every line is then read by the 16 up workgroups of one XCD,
//        spread over many memory channels, instead of by all 128 at once.
constexpr int kSsqLine = 16;
constexpr int kLoRows = 4;
constexpr int kLoBlock = 64;
constexpr size_t kPartWords = (size_t)kDecXcds * kDecDownPerXcd * kDecRowsPerXcd * kDecMaxT;
constexpr size_t kSsqWords = (size_t)kDecXcds * kDecDownPerXcd * kSsqLine;
constexpr size_t kLoWords = (size_t)kDecXcds * kDecXcds * 16 * kLoBlock;
// word index of (token t, reducer row r) of reducer (xs, us) in replica y
__host__ __device__ constexpr int lo_word(int y, int xs, int us, int t, int r)
{
    return ((y * kDecXcds + xs) * 16 + us) * kLoBlock + t * kLoRows + r;
}

// LDS bytes per role: the weight tile, then the role's planes
constexpr size_t down_lds(int T)
{
    return 16 * kTileChunks + 2 * 3 * T * kYRow + 4 * T * kStageItems + 6 * 2 * 64 * 16;
}
constexpr size_t up_lds(int T)
{
    return 16 * kTileChunks + 2 * 3 * T * kLoRow + 4 * T * kUpRows + (kDecUpCols / 4) * 2 * 64 * 16;
}
constexpr size_t lds_bytes(int T)
{
    return down_lds(T) > up_lds(T) ? down_lds(T) : up_lds(T);
}

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

// Short-window MFMA blocks put (piece, token) pairs on the 16 A rows: row
// p T + t holds piece p (0 hi, 1 mid, 2 lo3) of token t.  kChains: MFMA chains
// per block (1 when all 3 T rows fit, else 2: pieces 0-1, then piece 2 on rows
// 0..T-1).  kPackRows: the A rows chain 0 carries.
template <int T>
constexpr int kChains = 3 * T <= 16 ? 1 : 2;
template <int T>
constexpr int kPackRows = kChains<T> == 1 ? 3 * T : 2 * T;

// Product-block element (piece p, token t; column = the lane's n) of block w,
// from blocks stored in LDS as [block][chain][64 lanes] f32x4 (the MFMA's own
// register layout: row i of column n sits in lane n + 16 (i / 4), element i % 4).
template <int T>
__device__ __forceinline__ float packed_at(const float* cf, int w, int p, int t, int n)
{
    const int c = (kChains<T> == 2 && p == 2) ? 1 : 0;
    const int i = c ? t : p * T + t;
    return cf[((w * kChains<T> + c) * 64 + n + 16 * (i >> 2)) * 4 + (i & 3)];
}
// The three pieces' products of token t summed: hi + (mid + lo3).
template <int T>
__device__ __forceinline__ float piece_sum(const float* cf, int w, int t, int n)
{
    return packed_at<T>(cf, w, 0, t, n) + (packed_at<T>(cf, w, 1, t, n) + packed_at<T>(cf, w, 2, t, n));
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
    // An opaque copy of the (wave-uniform, scalar) base: the compiler can
    // neither merge two polling loads nor move one out of its loop (it does
    // not treat a memory clobber as reaching buffer loads).
    asm volatile("" : "+s"(base));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint64_t*>(base), 0, 0x7fffffff, 0x00020000);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, index * 8, 0, 16 /* sc1 */));
}
// Start of a polling round (a compiler barrier; each polling load's opaque
// base is what keeps the loads inside their loop).
__device__ __forceinline__ void new_round()
{
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint64_t tag_f32(float v, uint32_t gen)
{
    return (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32);
}
// Tag of a word handed over inside one XCD: the generation and the
// producer's dispatch rotation (see the kernel).
__device__ __forceinline__ uint32_t xcd_tag(uint32_t gen, uint32_t rot)
{
    return (gen << 3) | rot;
}
__device__ __forceinline__ void note_timeout(uint32_t* timeouts)
{
    __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads the T consecutive words at base1 + idx1 and at base2 + idx2 (both
// even) into v1 and v2, polling until every tag carries `gen`.  Each polling
// round issues all its loads before it looks at any of them, so a round costs
// one memory latency whatever T is.  Returns false after a timeout (counted
// once; the values read so far are then meaningless).
template <int T>
__device__ __forceinline__ bool poll_words(const uint64_t* base1, int idx1, const uint64_t* base2, int idx2,
                                           uint32_t gen, long long t0, int lane, float (&v1)[T], float (&v2)[T],
                                           uint32_t* timeouts, int site)
{
    constexpr int NP = (T + 1) / 2;
    [[maybe_unused]] int rounds = 0;
    while (true) {
        ++rounds;
        new_round();
        uint4 a[NP], c[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            a[q] = ld_words2(base1, idx1 + 2 * q);
            c[q] = ld_words2(base2, idx2 + 2 * q);
        }
        bool ok = true;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            ok = ok && a[q].y == gen && c[q].y == gen && (2 * q + 1 >= T || (a[q].w == gen && c[q].w == gen));
            v1[2 * q] = __uint_as_float(a[q].x);
            v2[2 * q] = __uint_as_float(c[q].x);
            if (2 * q + 1 < T) {
                v1[2 * q + 1] = __uint_as_float(a[q].z);
                v2[2 * q + 1] = __uint_as_float(c[q].z);
            }
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

// ---- weight tiles in LDS.  A tile row holds RC chunks of 16 bytes (RC / 8
// whole 128-byte lines).  The 8 chunks of a line are stored XOR-swizzled by
// row, and in 80-chunk rows (whose pitch is a multiple of 256 bytes) odd rows
// also swap neighbouring lines, so 16 lanes reading the same chunk column of
// 16 consecutive rows hit distinct 16-byte bank groups (with 32 or 64 banks).
__device__ __forceinline__ int swz(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}
template <int RC>
__device__ __forceinline__ int line_perm(int row, int m)
{
    return RC % 16 == 0 ? m ^ (row & 1) : m;
}
// LDS position (in chunks) of chunk j of tile row `row`.
template <int RC>
__device__ __forceinline__ int tile_pos(int row, int j)
{
    return row * RC + 8 * line_perm<RC>(row, j >> 3) + ((j & 7) ^ swz(row));
}
// Wave instruction q of a tile load: lane l fills LDS position p = 64 q + l,
// i.e. (row, line, slot); it fetches the chunk that belongs there.  Eight
// consecutive lanes fetch one whole 128-byte line.
template <int RC>
__device__ __forceinline__ void tile_lane(int q, int lane, int& row, int& j)
{
    const int p = 64 * q + lane;
    row = p / RC;
    const int rem = p - row * RC;
    j = 8 * line_perm<RC>(row, rem >> 3) + ((rem & 7) ^ swz(row));
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
    static_assert(kDecRowsPerXcd * kDnRowChunks == kTileChunks && kUpRows * kUpRowChunks == kTileChunks,
                  "both tiles are 3200 chunks");
    static_assert(kWidth % kDecDownCols == 0, "a W_down tile lies in one stream");
    static_assert(kDecXcds * kDecRowsPerXcd == kRank && kDecXcds * kDecUpPerXcd * kDecUpCols == kWidth, "cover");
    static_assert(kStageItems * kDecMaxT <= 3 * kDecThreads && kUpRows * kDecMaxT <= 2 * kDecThreads, "passes");
    static_assert(kDecReducers <= 16 && kDecRedRows <= 3 && kDecDownPerXcd == 16, "one reducer wave");
    __shared__ __align__(16) uint4 lds[lds_bytes(T) / 16];
    uint4* const tile = lds;  // the role's weight tile

    DecodeScratch s;
    s.part = scratch;
    s.ssq = s.part + kPartWords;
    s.lo = s.ssq + kSsqWords;
    s.gen = reinterpret_cast<uint32_t*>(s.lo + kLoWords);
    s.timeouts = s.gen + kDecWGs;
    const int b = blockIdx.x;
    const int x = b & 7;   // group (all its workgroups share one XCD)
    const int i = b >> 3;  // index inside the XCD, 0..31
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // MFMA column slot (B / D operand)
    const int g = lane >> 4;  // MFMA k-group (A / B operand) and D row group
    const int m = lane & 15;  // MFMA A row = token
    // this launch's generation: one more than the launches this workgroup has
    // seen.  Every lane loads the counter (no per-lane branch); the value is
    // used only after the weights have landed.
    uint32_t seen = __hip_atomic_load(&s.gen[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The dispatcher deals workgroups to the XCDs round robin, starting where
    // the previous dispatch stopped: workgroup b runs on XCD (b + r) % 8 with
    // one rotation r for the whole launch, so the workgroups of one group x
    // share an L2 whatever r is.  Each workgroup puts its own r into the tags
    // of the words it hands over inside its XCD, and a reducer accepts only
    // its own r: a producer that ran on another XCD shows up as an expired
    // (counted) wait, never as a silent stale read.
    const uint32_t rot = (__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) - (uint32_t)x) & 7u;
    HC_PROBE(0, threadIdx.x == 0);
    // Loads issued before the first wait are unconditional (items past the end
    // re-read item 0; a missing pending re-reads R): a conditional load makes
    // the compiler merge registers, which waits for every load.
    const float* Pm = P ? P : R;

    if (i < kDecDownPerXcd) {
        // =========================== down ===========================
        const int d = i;
        uint16_t* const ypl = reinterpret_cast<uint16_t*>(lds + kTileChunks);     // [3][T][kYRow]
        float* const sspart = reinterpret_cast<float*>(ypl + 3 * T * kYRow);       // [T][160]
        f32x4_t* const comb = reinterpret_cast<f32x4_t*>(sspart + T * kStageItems);  // [6][chains][64]

        // (1) the W_down tile: rows 40 x + row, columns 640 d + 8 j ..
        for (int q = wave; q < kTileInstr; q += 8) {
            int row, j;
            tile_lane<kDnRowChunks>(q, lane, row, j);
            dma16(W_down + (size_t)(kDecRowsPerXcd * x + row) * kD + kDecDownCols * d + 8 * j, tile + 64 * q);
        }
        // the activations of columns [640 d, 640 d + 640)
        float4 rv[3], pv[3], wv[3];
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int it = threadIdx.x + kDecThreads * pass;
            const int itc = it < kStageItems * T ? it : 0;
            const int at = itc / kStageItems, f = itc - at * kStageItems;
            const size_t o = (size_t)at * kD + kDecDownCols * d + 4 * f;
            rv[pass] = *reinterpret_cast<const float4*>(R + o);
            pv[pass] = *reinterpret_cast<const float4*>(Pm + o);
            wv[pass] = *reinterpret_cast<const float4*>(w_norm + kDecDownCols * d + 4 * f);
        }
        // (2) y = R' * w_norm (unscaled: the norm is folded into the
        //     reduction), its sums of squares, and the exact 3-way split
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int it = threadIdx.x + kDecThreads * pass;
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
                sspart[at * kStageItems + f] = ss;
                const int col = 4 * f;
                *reinterpret_cast<uint2*>(&ypl[(0 * T + at) * kYRow + col]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2*>(&ypl[(1 * T + at) * kYRow + col]) = make_uint2(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16));
                *reinterpret_cast<uint2*>(&ypl[(2 * T + at) * kYRow + col]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
        wait_all_loads();  // this wave's part of the tile is in LDS
        wg_barrier();      // B1: activations staged, W_down tile complete
        HC_PROBE(1, threadIdx.x == 0);
        pin(seen);
        const uint32_t gen = (uint32_t)__builtin_amdgcn_readfirstlane((int)seen) + 1u;

        // (3) down projection: wave w < 6 takes rows 16 (w % 3) .. +15 of the
        //     tile (block 2: rows 32..39, its upper 8 slots repeat them) over
        //     K steps 10 (w / 3) .. +9 of 32 columns.  A rows are (piece,
        //     token) pairs in the planes' own order (row p T + t: piece p of
        //     token t), so one chain of MFMAs carries all three pieces when
        //     3 T <= 16, two chains (pieces 0-1, then piece 2) otherwise.
        if (wave < 6) {
            const int nb = wave % 3, kh = wave / 3;
            const int row = nb < 2 ? 16 * nb + n : 32 + (n & 7);
            // all operands first (one LDS latency, not ten); A rows past the
            // pieces re-read row 0: they only feed D rows nobody reads
            const int r0 = m < kPackRows<T> ? m : 0;
            const int r1 = 2 * T + (m < T ? m : 0);
            uint4 wb[10], a0[10], a1[10];
#pragma unroll
            for (int qq = 0; qq < 10; ++qq) {
                const int q = 10 * kh + qq;
                const int col = 32 * q + 8 * g;
                wb[qq] = tile[tile_pos<kDnRowChunks>(row, 4 * q + g)];
                a0[qq] = *reinterpret_cast<const uint4*>(&ypl[r0 * kYRow + col]);
                if (kChains<T> == 2)
                    a1[qq] = *reinterpret_cast<const uint4*>(&ypl[r1 * kYRow + col]);
            }
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
            for (int qq = 0; qq < 10; ++qq) {
                acc0 = mfma16(a0[qq], wb[qq], acc0);
                if (kChains<T> == 2)
                    acc1 = mfma16(a1[qq], wb[qq], acc1);
            }
            comb[(wave * kChains<T>) * 64 + lane] = acc0;
            if (kChains<T> == 2)
                comb[(wave * kChains<T> + 1) * 64 + lane] = acc1;
        } else if (wave == 6) {
            // (3') meanwhile, the slice's sum of squares per token: lane 8 t + p
            //      sums 20 of token t's 160 item sums, then the 8 lanes combine theirs
            const int tt = lane >> 3, p = lane & 7;
            float ss = 0.f;
            if (tt < T) {
#pragma unroll
                for (int f = 0; f < 20; ++f)
                    ss += sspart[tt * kStageItems + 20 * p + f];
            }
            ss = sum8(ss);
            if (p < 2)  // words 0..7: tokens (0 past T); words 8..15: padding -- one whole line
                st_word_xcd(&s.ssq[((size_t)x * kDecDownPerXcd + d) * kSsqLine + 8 * p + tt],
                            tag_f32(p == 0 ? ss : 0.f, xcd_tag(gen, rot)));
        }
        HC_PROBE(2, threadIdx.x == 0);
        wg_barrier();  // Bc1: every product block in LDS

        if (wave < 6) {
            // (4) partial dots of rows 16 (w % 3) + n, token 4 (w / 3) + g,
            //     into the XCD's L2: per K half hi + (mid + lo3), then the two
            //     halves (all 8 token slots, whole lines; slots >= T hold 0)
            const float* cf = reinterpret_cast<const float*>(comb);
            const int nb = wave % 3, t = 4 * (wave / 3) + g;
            const int row = 16 * nb + n;
            if (row < kDecRowsPerXcd) {
                const float v = t < T ? piece_sum<T>(cf, nb, t, n) + piece_sum<T>(cf, nb + 3, t, n) : 0.f;
                st_word_xcd(s.part + (((size_t)x * kDecDownPerXcd + d) * kDecRowsPerXcd + row) * kDecMaxT + t,
                            tag_f32(v, xcd_tag(gen, rot)));
            }
        }
        HC_PROBE(3, threadIdx.x == 0);
        if (threadIdx.x == 0)
            __hip_atomic_store(&s.gen[b], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ============================= up =============================
    const int u = i - kDecDownPerXcd;
    const int c0 = kDecUpCols * (kDecUpPerXcd * x + u);  // first output column
    uint16_t* const lpl = reinterpret_cast<uint16_t*>(lds + kTileChunks);  // [3][T][kLoRow]
    float* const rpl = reinterpret_cast<float*>(lpl + 3 * T * kLoRow);      // [T][80]: R' of tile row 20 s + r
    f32x4_t* const ucomb = reinterpret_cast<f32x4_t*>(rpl + T * kUpRows);   // [5 waves][chains][64]

    // (1) the W_up tile: rows s * 2560 + c0 + r (tile row 20 s + r)
    for (int q = wave; q < kTileInstr; q += 8) {
        int row, j;
        tile_lane<kUpRowChunks>(q, lane, row, j);
        const int k = (row / kDecUpCols) * kWidth + c0 + row % kDecUpCols;
        dma16(W_up + (size_t)k * kRank + 8 * j, tile + 64 * q);
    }
    // (2) a reducer touches (plain loads, which keep the lines in this XCD's
    //     L2) the lines it will poll: the 16 producers' partial rows
    //     3 u .. 3 u + 2 and their sums of squares.  Polls then hit L2 and see
    //     a producer's store as soon as it lands, instead of each round
    //     fetching the line from memory.  (Only lines written inside this XCD
    //     are touched this way.)  The loaded value is consumed only after the
    //     weights have landed, so nothing waits for it before then.
    uint32_t touched = 0;
    if (wave == 0 && u < kDecReducers) {
        const int src = lane & 15, k = lane >> 4;  // k 0..2: partial lines, 3: sums of squares
        const int rowl = kDecRedRows * u + 2 * k < kDecRowsPerXcd ? kDecRedRows * u + 2 * k : kDecRowsPerXcd - 1;
        const uint64_t* line = k < 3 ? s.part + (((size_t)x * kDecDownPerXcd + src) * kDecRowsPerXcd + rowl) * kDecMaxT
                                     : s.ssq + ((size_t)x * kDecDownPerXcd + src) * kSsqLine;
        touched = *reinterpret_cast<const uint32_t*>(line);  // (not volatile: that would wait here)
    }
    // R and pending of the same 80 (stream, column) pairs, for the mix
    float mr[2], mp[2];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int it = threadIdx.x + kDecThreads * pass;
        const int itc = it < kUpRows * T ? it : 0;
        const int at = itc / kUpRows, row = itc - at * kUpRows;
        const size_t o = (size_t)at * kD + (row / kDecUpCols) * kWidth + c0 + row % kDecUpCols;
        mr[pass] = R[o];
        mp[pass] = Pm[o];
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int it = threadIdx.x + kDecThreads * pass;
        if (it < kUpRows * T)
            rpl[it] = P ? mr[pass] + mp[pass] : mr[pass];  // it = 80 t + row
    }
    wait_all_loads();  // every load of this CU has landed: from here on, hand-off loads run at cache latency
    asm volatile("" ::"v"(touched));
    wg_barrier();      // B1
    HC_PROBE(1, threadIdx.x == 0);
    pin(seen);
    const uint32_t gen = (uint32_t)__builtin_amdgcn_readfirstlane((int)seen) + 1u;

    if (wave == 0) {
        if (u < kDecReducers) {
            // (5) hop 1: lo rows 3 u .. 3 u + 2 of this XCD from its 16
            //     down workgroups' partials, each stream's rs from its 4
            //     slices' sums of squares; lo published device-wide.  Up to 4
            //     tokens, a lane group per row (rows in parallel, tokens in
            //     turn); from 5 tokens, a lane group per pair of tokens (one
            //     load per row per polling round, rows in turn).
            if constexpr (T <= 4) {
                // lane = src + 16 r: row 3 u + r (r < 3) of down workgroup src
                const int r = lane >> 4, src = lane & 15;
                const int row = kDecRedRows * u + r;
                const bool valid = r < kDecRedRows && row < kDecRowsPerXcd;
                const int rowc = valid ? row : kDecRedRows * u;  // (a row of this reducer, read and discarded)
                const int pidx = ((x * kDecDownPerXcd + src) * kDecRowsPerXcd + rowc) * kDecMaxT;
                const int sidx = (x * kDecDownPerXcd + src) * kSsqLine;
                const long long t0 = wall_clock64();
                float v[T], q[T];
                poll_words<T>(s.part, pidx, s.ssq, sidx, xcd_tag(gen, rot), t0, lane, v, q, s.timeouts, 0);
                HC_PROBE(12, lane == 0);
                float mine = 0.f;  // lo of row 3 u + r, token `src`
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    // lanes 4 s .. 4 s + 3 (of each 16) hold the slices of stream s
                    const float ss = sum4(q[t]);
                    const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
                    const float y = sum4(v[t]) * rs;
                    const float y01 = y + dpp<0x141>(y);      // row_half_mirror: (s0 + s1), (s2 + s3)
                    const float lo = y01 + dpp<0x140>(y01);   // row_mirror: (s0 + s1) + (s2 + s3)
                    if (src == t)
                        mine = lo;
                }
                // 32 words (2 whole lines) per replica: tokens 0..7 x rows 0..3 of
                // this reducer, 0 in the padding
                const uint64_t word = tag_f32(valid && src < T ? mine : 0.f, gen);
#pragma unroll
                for (int y = 0; y < kDecXcds; ++y)
                    if (src < kDecMaxT)
                        st_word(&s.lo[lo_word(y, x, u, src, r)], word);
            } else {
                // lane = src + 16 q: tokens 2 q, 2 q + 1 of down workgroup src
                // (a polling round is 3 row loads and 1 sum-of-squares load)
                const int src = lane & 15, q = lane >> 4;
                const int pbase = (x * kDecDownPerXcd + src) * kDecRowsPerXcd;
                int pidx[kDecRedRows];
#pragma unroll
                for (int rr = 0; rr < kDecRedRows; ++rr) {
                    const int row = kDecRedRows * u + rr;
                    pidx[rr] = (pbase + (row < kDecRowsPerXcd ? row : kDecRowsPerXcd - 1)) * kDecMaxT + 2 * q;
                }
                const int sidx = (x * kDecDownPerXcd + src) * kSsqLine + 2 * q;
                const uint32_t htag = xcd_tag(gen, rot);
                const long long t0 = wall_clock64();
                uint4 pw[kDecRedRows], sw;
                [[maybe_unused]] int rounds = 0;
                while (true) {
                    ++rounds;
                    new_round();
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr)
                        pw[rr] = ld_words2(s.part, pidx[rr]);
                    sw = ld_words2(s.ssq, sidx);
                    bool ok = sw.y == htag && sw.w == htag;
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr)
                        ok = ok && pw[rr].y == htag && pw[rr].w == htag;
                    if (__all(ok)) {
                        HC_COUNT(0, 0, rounds, lane == 0);
                        break;
                    }
                    if (wall_clock64() - t0 > kWaitTicks) {
                        if (lane == 0)
                            note_timeout(s.timeouts);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                HC_PROBE(12, lane == 0);
                float lo[kDecRedRows][2];  // [row][token 2 q + h], the same in all 16 lanes of q
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // lanes 4 s .. 4 s + 3 (of each 16) hold the slices of stream s
                    const float ss = sum4(__uint_as_float(h ? sw.z : sw.x));
                    const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr) {
                        const float y = sum4(__uint_as_float(h ? pw[rr].z : pw[rr].x)) * rs;
                        const float y01 = y + dpp<0x141>(y);     // row_half_mirror: (s0 + s1), (s2 + s3)
                        lo[rr][h] = y01 + dpp<0x140>(y01);       // row_mirror: (s0 + s1) + (s2 + s3)
                    }
                }
                // 32 words (2 whole lines) per replica: tokens 0..7 x rows 0..3 of
                // this reducer, 0 in the padding; lane src < 8 of q writes row
                // src / 2, token 2 q + src % 2
                const int rr = src >> 1, h = src & 1, tok = 2 * q + h;
                const float mine = rr == 0 ? lo[0][h] : rr == 1 ? lo[1][h] : lo[2][h];
                const bool valid = rr < kDecRedRows && kDecRedRows * u + rr < kDecRowsPerXcd && tok < T;
                const uint64_t word = tag_f32(valid ? mine : 0.f, gen);
#pragma unroll
                for (int y = 0; y < kDecXcds; ++y)
                    if (src < 8)
                        st_word(&s.lo[lo_word(y, x, u, tok, rr)], word);
            }
            HC_PROBE(13, lane == 0);
        }
    }
    wg_barrier();  // Bs
    {
        // (6) hop 2: wave w polls the lo words of XCD w's reducers (slot =
        //     reducer, token, pair of rows) until every tag is current, then
        //     stages the 3 bf16 pieces of each value.  (Waves start after this
        //     workgroup's own reducer is done, so their cold loads do not
        //     queue in front of its L2 polls.)
        constexpr int NSL = kDecReducers * T * 2;  // slots per wave
        constexpr int NS = (NSL + 63) / 64;        // slots per lane
        const long long t0 = wall_clock64();
        uint4 lw[NS];
        int widx[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int sl = lane + 64 * k < NSL ? lane + 64 * k : 0;  // (past the end: re-read slot 0)
            const int pair = sl & 1, rest = sl >> 1;
            const int tt = rest % T, us = rest / T;  // us: reducer 0 .. 13
            widx[k] = lo_word(x, wave, us, tt, 2 * pair);
        }
        [[maybe_unused]] int rounds = 0;
        while (true) {
            ++rounds;
            new_round();
#pragma unroll
            for (int k = 0; k < NS; ++k)
                lw[k] = ld_words2(s.lo, widx[k]);
            bool all = true;
#pragma unroll
            for (int k = 0; k < NS; ++k)
                all = all && lw[k].y == gen && lw[k].w == gen;
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
        HC_PROBE(14, wave == 0 && lane == 0);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int sl = lane + 64 * k;
            if (sl < NSL) {
                const int pair = sl & 1, rest = sl >> 1;
                const int tt = rest % T, us = rest / T;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rr = 2 * pair + h;               // row of the reducer, 0..3
                    const int rowl = kDecRedRows * us + rr;    // row of the XCD, 0..39
                    if (rr < kDecRedRows && rowl < kDecRowsPerXcd) {
                        const int jr = kDecRowsPerXcd * wave + rowl;
                        uint32_t hb, mb, lb;
                        split3(__uint_as_float(h ? lw[k].z : lw[k].x), hb, mb, lb);
                        lpl[(0 * T + tt) * kLoRow + jr] = (uint16_t)hb;
                        lpl[(1 * T + tt) * kLoRow + jr] = (uint16_t)mb;
                        lpl[(2 * T + tt) * kLoRow + jr] = (uint16_t)lb;
                    }
                }
            }
        }
        HC_PROBE(7, wave == 0 && lane == 0);
    }
    wg_barrier();  // B2: lo staged
    HC_PROBE(8, threadIdx.x == 0);

    if (wave < kDecUpCols / 4) {
        // (7) up projection: wave w < 5 takes output columns c0 + 4 w .. +3
        //     (slot n = 4 column + stream), all 10 K steps, A rows packed as
        //     in the down projection; gated = up (identity epilogue); then the
        //     mix of the 4 streams of a column
        const int cc = n >> 2, st = n & 3;
        const int row = st * kDecUpCols + 4 * wave + cc;
        const int r0 = m < kPackRows<T> ? m : 0;
        const int r1 = 2 * T + (m < T ? m : 0);
        uint4 wb[10], a0[10], a1[10];
#pragma unroll
        for (int q = 0; q < 10; ++q) {
            const int jc = 32 * q + 8 * g;
            wb[q] = tile[tile_pos<kUpRowChunks>(row, 4 * q + g)];
            a0[q] = *reinterpret_cast<const uint4*>(&lpl[r0 * kLoRow + jc]);
            if (kChains<T> == 2)
                a1[q] = *reinterpret_cast<const uint4*>(&lpl[r1 * kLoRow + jc]);
        }
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int q = 0; q < 10; ++q) {
            acc0 = mfma16(a0[q], wb[q], acc0);
            if (kChains<T> == 2)
                acc1 = mfma16(a1[q], wb[q], acc1);
        }
        // a token's pieces sit in other lanes: through this wave's own LDS block
        f32x4_t* const ub = ucomb + wave * kChains<T> * 64;
        ub[lane] = acc0;
        if (kChains<T> == 2)
            ub[64 + lane] = acc1;
        asm volatile("" ::: "memory");  // (LDS operations of one wave complete in order)
        const float* cf = reinterpret_cast<const float*>(ub);
        const int c = c0 + 4 * wave + cc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tt = 4 * g + e;
            const float up = tt < T ? piece_sum<T>(cf, 0, tt, n) : 0.f;
            const float rp = rpl[(tt < T ? tt : 0) * kUpRows + row];
            const float mixed = sum4(up * rp);  // (s0 + s1) + (s2 + s3)
            if (st == 0 && tt < T) {
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
