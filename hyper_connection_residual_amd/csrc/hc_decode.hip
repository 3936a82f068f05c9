// hc_decode.hip -- the hyper-connection read for short windows (T <= 32 tokens)
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
// * 256 workgroups x 8 waves, one per CU.  Each workgroup streams a 25.6 KB
//   tile of W_down (40 rows x 320 columns) at entry and a 25.6 KB tile of
//   W_up (10 output columns x 4 streams) later.  A CU serves its vector
//   memory requests in order across its waves (measured: a load that hits L2
//   in 0.08 us takes over 1 us while another wave of the CU has cold loads
//   outstanding), so a poll issued behind a tile waits for the whole tile.
//   Most workgroups issue their W_up tile as soon as their partial dots are
//   stored; the 14 per XCD that reduce partials (below) issue it after that
//   reduction, so their polls never queue behind it.  (Measured: issuing the
//   W_up tiles at entry makes the W_down tiles land 1 us later, since the
//   memory system shares its bandwidth between everything in flight; issuing
//   them before the reduction delays the reduction.  Both are slower.)
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
//   result stays fp32-faithful.  The pieces of all tokens share the MFMA's
//   rows.  Up to 8 tokens row 4 t + p holds piece p of token t (one chain of
//   MFMAs per 4 tokens): a token's three products then sit in one lane, which
//   sums them and mixes the streams in registers.  Above 8 tokens row p T + t
//   holds them (3 or 6 chains) and the products go through LDS.
// * Two hand-offs, no grid barrier.  XCD x owns lo rows [40 x, 40 x + 40): 14
//   of its 32 workgroups each reduce the 32 partials of 3 rows through the
//   XCD's L2 (hop 1, one wave; two above 8 tokens) and publish lo device-wide; every workgroup gathers all of lo
//   (hop 2).  Hand-off words are 64 bits holding the payload and the launch's
//   generation number, written once with one store; a consumer polls the data
//   words themselves (device-coherent loads, which see a write-through store
//   from another XCD even when they started polling before it), with every
//   load of a polling round in flight at once.  Every workgroup counts its
//   launches in its own slot, so all of them agree on the generation without
//   host involvement (the launch is graph-capture safe).  Every wait is
//   bounded, and an expired wait never yields silent results: a reducer whose
//   wait expired publishes NaN words marked as poison, and a workgroup whose
//   own wait expired or that received poison stores NaN for every output it
//   owns (and commits nothing).
#include "hc_internal.h"

// No multiply-add contraction anywhere in this file: a butterfly sum must give
// every lane the same bits, and a fused multiply-add would add the lane's own
// unrounded product to its partner's rounded one.
#pragma clang fp contract(off)

// Instrumentation hook: empty in the library.  The timing build (built with
// HC_PROBE_STAMPS, into a separate library) records, in wave 0 lane 0, the
// 100 MHz wall clock when the workgroup passes each numbered point, and
// stores the stamps at the kernel's end into a ring of 64 launches that
// hc_probe_stamps copies out.  Points: 0 entry, 1 W_down tile and
// activations landed (y staged), 2 down products done, 3 partial dots
// stored, 12 hop 1 polls done and 13 lo published (reducers), 14 hop 2 polls
// done, 7 lo staged, 8 W_up tile landed and lo complete, 9 outputs stored,
// 15 exit.
#if defined(HC_PROBE_STAMPS)
#define HC_PROBE(point, cond)                                       \
    do {                                                            \
        if ((cond) && threadIdx.x == 0)                             \
            probe_t[point] = (unsigned long long)wall_clock64();    \
    } while (0)
#elif !defined(HC_PROBE)
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTileChunks = 1600;           // 16-byte chunks in either weight tile (25,600 bytes)
constexpr int kTileInstr = kTileChunks / 64;  // wave instructions per tile (25)
constexpr int kRowChunks = kRank / 8;       // chunks per row of either tile (40: 320 bf16)
constexpr int kUpRows = 4 * kDecUpCols;     // W_up tile rows (40): row 4 c + s
constexpr int kStageItems = kDecDownCols / 4;  // float4 activation items per token (80)
constexpr int kYRow = kDecDownCols + 8;     // padded LDS row of an activation plane (bf16)
constexpr int kLoRow = kRank + 8;           // padded LDS row of a lo plane (bf16)
// Scratch layout (in 64-bit words from the base): partial dots, slice sums of
// squares, lo, then the 32-bit generation counters and the timeout counter.
// Every producer writes whole 128-byte lines (16 words), padding unused token
// slots: a line an L2 holds only in part is filled from memory before it is
// read or written through, which costs a memory round trip.
//   part [8 xcd][32 wg][40 rows][8 token slots]     (two rows per line), or
//        [8 xcd][32 wg][40 rows][16 token slots]    (above 8 tokens: one row per line), or
//        [8 xcd][32 wg][40 rows][32 token slots]    (above 16 tokens: two lines per row)
//   ssq  [8 xcd][32 wg][16]                         (tokens 0..7, then padding; or tokens 0..15),
//        or [8 xcd][32 wg][32]                      (above 16 tokens: tokens 0..31)
//   lo   [8 replica][8 xcd][16 reducer] blocks of 64 words, the first 32 being
//        [8 tokens][4 rows] (rows 3 u .. 3 u + 2, padding; above 8 tokens all
//        64 are [16 tokens][4 rows]; above 16 tokens the blocks hold 128
//        words, [32 tokens][4 rows]).  Each reducer writes
//        one replica per consumer XCD, and the blocks are spread 512 bytes
//        apart: every line is then read by the 32 workgroups of one XCD,
//        spread over many memory channels, instead of by all 256 at once.
//        (Measured: a [token][320 rows] layout, whose lines several reducers
//        write in part, makes hop 2 take 1-2 us longer.)
constexpr int kLoRows = 4;
// Per token count: the ssq words of one workgroup (one line, two above 16
// tokens), the words of a lo block (2 or 4 lines, 8 above 16 tokens).
template <int T>
constexpr int kSsqLine = T <= 16 ? 16 : 32;
template <int T>
constexpr int kLoBlock = T <= 16 ? 64 : 128;
constexpr size_t kPartWords = (size_t)kDecXcds * kDecWgPerXcd * kDecRowsPerXcd * kDecMaxT;
constexpr size_t kSsqWords = (size_t)kDecXcds * kDecWgPerXcd * kSsqLine<kDecMaxT>;
constexpr size_t kLoWords = (size_t)kDecXcds * kDecXcds * 16 * kLoBlock<kDecMaxT>;
// word index of (token t, reducer row r) of reducer (xs, us) in replica y
template <int T>
__host__ __device__ constexpr int lo_word(int y, int xs, int us, int t, int r)
{
    return ((y * kDecXcds + xs) * 16 + us) * kLoBlock<T> + t * kLoRows + r;
}

// Short-window MFMA blocks put (piece, token) pairs on the 16 A rows: row
// p T + t holds piece p (0 hi, 1 mid, 2 lo3) of token t.  kChains: MFMA chains
// per block (1 when all 3 T rows fit; up to 8 tokens 2: pieces 0-1, then
// piece 2; up to 16, 3: one per piece; beyond, 6: chain 2 p + h carries
// tokens 16 h .. 16 h + 15 of piece p).  kPackRows: the A rows chain 0 carries.
template <int T>
constexpr int kChains = 3 * T <= 16 ? 1 : (T <= 8 ? 2 : (T <= 16 ? 3 : 6));
template <int T>
constexpr int kPackRows = kChains<T> == 1 ? 3 * T : (kChains<T> == 2 ? 2 * T : (kChains<T> == 3 ? T : 16));
// First plane row (p T + t) and row count of chain c.
template <int T>
__host__ __device__ constexpr int chain_base(int c)
{
    return kChains<T> == 6 ? (c >> 1) * T + 16 * (c & 1) : (c == 0 ? 0 : (kChains<T> == 3 ? c * T : 2 * T));
}
template <int T>
__host__ __device__ constexpr int chain_rows(int c)
{
    return kChains<T> == 6 ? ((c & 1) ? T - 16 : 16) : (c == 0 ? kPackRows<T> : T);
}
// Up to 8 tokens the blocks take the quad layout instead: A row 4 t + p holds
// piece p of token t (row 4 t + 3 is never written and feeds a D row nobody
// reads), one chain per 4 tokens.  The D layout then puts a token's three
// pieces into one lane (row i of column n sits in lane n + 16 (i / 4), element
// i % 4), so pieces are summed and the streams mixed in registers, with no
// product block going through LDS.
template <int T>
constexpr bool kQuad = T <= 8;
template <int T>
constexpr int kQuadChains = (T + 3) / 4;
// Rows of a y or lo plane set and the row of (piece p, token t) in it.
template <int T>
constexpr int kPlaneRows = kQuad<T> ? 16 * kQuadChains<T> : 3 * T;
template <int T>
__host__ __device__ constexpr int plane_row(int p, int t)
{
    return kQuad<T> ? 4 * t + p : p * T + t;
}
// Chains' room in the LDS product blocks (at least 2, as laid out for 1..8 tokens).
template <int T>
constexpr int kCombChains = kChains<T> < 2 ? 2 : kChains<T>;
// Token slots of a partial-dot row in scratch: 8 (two rows per 128-byte
// line) up to 8 tokens, 16 (one row per line) up to 16, else 32 (two lines).
template <int T>
constexpr int kTokSlots = T <= 8 ? 8 : (T <= 16 ? 16 : 32);

// LDS map (bytes): both weight tiles, the y planes [kPlaneRows][kYRow] bf16,
// the token sums of squares of the items [T][80] fp32, the down product blocks
// [6][chains][64] f32x4, the lo planes [kPlaneRows][kLoRow] bf16, R' of the up
// tile's rows [T][40] fp32, the up product blocks [3][chains][64] f32x4 (up to
// 8 tokens the product blocks and R' are laid out but unused).
// Above 16 tokens, regions never live at once share memory (kShare): the W_up
// tile lands where the W_down tile was (it is issued after the down MFMAs),
// the lo planes overwrite the y planes, the up product blocks the down ones.
template <int T> constexpr bool kShare = T > 16;
template <int T> constexpr size_t kOffUTile = kShare<T> ? 0 : 16 * kTileChunks;
template <int T> constexpr size_t kOffY = kOffUTile<T> + 16 * kTileChunks;
template <int T> constexpr size_t kOffSs = kOffY<T> + 2 * kPlaneRows<T> * kYRow;
template <int T> constexpr size_t kOffComb = kOffSs<T> + 4 * T * kStageItems;
template <int T> constexpr size_t kOffLo = kShare<T> ? kOffY<T> : kOffComb<T> + 6 * kCombChains<T> * 64 * 16;
template <int T>
constexpr size_t kOffRp = kShare<T> ? kOffComb<T> + 6 * kCombChains<T> * 64 * 16 : kOffLo<T> + 2 * kPlaneRows<T> * kLoRow;
template <int T> constexpr size_t kOffUComb = kShare<T> ? kOffComb<T> : kOffRp<T> + 4 * T * kUpRows;
template <int T>
constexpr size_t kLdsBytes = kShare<T> ? kOffRp<T> + 4 * T * kUpRows : kOffUComb<T> + 3 * kCombChains<T> * 64 * 16;

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


// Product-block element (piece p, token t; column = the lane's n) of block w,
// from blocks stored in LDS as [block][chain][64 lanes] f32x4 (the MFMA's own
// register layout: row i of column n sits in lane n + 16 (i / 4), element i % 4).
template <int T>
__device__ __forceinline__ float packed_at(const float* cf, int w, int p, int t, int n)
{
    const int c = kChains<T> == 6 ? 2 * p + (t >> 4) : kChains<T> == 3 ? p : ((kChains<T> == 2 && p == 2) ? 1 : 0);
    const int i = kChains<T> == 6 ? (t & 15) : kChains<T> == 3 ? t : (c ? t : p * T + t);
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
// Generations count modulo 2^31; the top bit of a device-wide lo word's tag
// marks poison: its producer's bounded wait expired and its payload is NaN.
constexpr uint32_t kGenMask = 0x7fffffffu;
constexpr uint32_t kPoison = 0x80000000u;
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
    // (a separate 24-bit product: fused, the compiler makes it a 64-bit
    // multiply-add whose unused high addend may sit in a register still being
    // loaded, and waits for that load)
    unsigned prod = __umul24((unsigned)row, (unsigned)RC);
    asm("" : "+v"(prod));
    const int rem = p - (int)prod;
    j = 8 * line_perm<RC>(row, rem >> 3) + ((rem & 7) ^ swz(row));
}
// 16 bytes per lane from memory into LDS: lane l's bytes land at
// lds_wave_base + 16 l (the base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const uint16_t* g, uint4* lds_wave_base)
{
    __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}
// LDS stores written as inline asm, which the compiler does not see: it would
// make a C++ store into the LDS array wait for every load into LDS still in
// flight (the W_down tile), where these run while the tile lands.  Barriers
// wait for them (lgkmcnt).
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)p;  // the low 32 bits of a shared-aperture address are the LDS offset
}
__device__ __forceinline__ void ds_st16(const void* p, uint32_t v)
{
    asm volatile("ds_write_b16 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_st32(const void* p, uint32_t v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_st64(const void* p, u32x2_t v)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// The same through a buffer resource: `voff` is the lane's byte offset.  The
// compiler orders these with ordinary loads (a wait for a load issued before
// them leaves them in flight), where after global_load_lds it waits for all.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint4* lds_wave_base, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, 0, 0, 0);
}

// The arguments the first loads need come first: the library is built with
// kernel-argument preloading, so they arrive in SGPRs and no wave has to fetch
// them from memory (a fetch that queues behind the other CUs' weight traffic).
#if defined(HC_PROBE_STAMPS)
// [64 launches (generation mod 64)][256 workgroups][16 points]: wall-clock stamps
__device__ unsigned long long hc_probe_ring[64 * kDecWGs * 16];
#endif

template <int T>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const uint16_t* __restrict__ W_down, const uint16_t* __restrict__ W_up, const float* R,
    const float* __restrict__ P, const float* __restrict__ w_norm, uint64_t* __restrict__ scratch,
    float* __restrict__ out_mixed, uint16_t* __restrict__ out_bf16, uint16_t* __restrict__ out_fp16,
    float* R_commit, long long wait_ticks)
{
    static_assert(T >= 1 && T <= kDecMaxT && kDecMaxT == 32, "short-window kernel takes 1..32 tokens");
    static_assert(kDecRowsPerXcd * kRowChunks == kTileChunks && kUpRows * kRowChunks == kTileChunks,
                  "both tiles are 1600 chunks");
    static_assert(kWidth % kDecDownCols == 0 && kWidth / kDecDownCols == 8, "8 down tiles per stream");
    static_assert(kDecXcds * kDecRowsPerXcd == kRank && kDecWGs * kDecUpCols == kWidth, "cover");
    static_assert(kStageItems * kDecMaxT <= 5 * kDecThreads && kUpRows * kDecMaxT <= 3 * kDecThreads, "passes");
    static_assert(kDecReducers <= 16 && kDecRedRows == 3 && kDecWgPerXcd == 32, "reducer layout");
    static_assert(kLdsBytes<T> <= 160 * 1024, "LDS");
    __shared__ __align__(16) uint4 lds[kLdsBytes<T> / 16];
    uint4* const dtile = lds;                                                              // W_down tile
    uint4* const utile = lds + kOffUTile<T> / 16;                                          // W_up tile
    uint16_t* const ypl = reinterpret_cast<uint16_t*>(lds + kOffY<T> / 16);               // [3 T][kYRow]
    float* const sspart = reinterpret_cast<float*>(lds + kOffSs<T> / 16);                 // [T][80]
    f32x4_t* const comb = reinterpret_cast<f32x4_t*>(lds + kOffComb<T> / 16);             // [6][chains][64]
    uint16_t* const lpl = reinterpret_cast<uint16_t*>(lds + kOffLo<T> / 16);              // [3 T][kLoRow]
    float* const rpl = reinterpret_cast<float*>(lds + kOffRp<T> / 16);                    // [T][40]
    f32x4_t* const ucomb = reinterpret_cast<f32x4_t*>(lds + kOffUComb<T> / 16);           // [3][chains][64]
    // set by a wave whose hop-2 wait expired or that received poison: the
    // workgroup then stores NaN outputs and commits nothing
    __shared__ uint32_t poisoned_wg;

    DecodeScratch s;
    s.part = scratch;
    s.ssq = s.part + kPartWords;
    s.lo = s.ssq + kSsqWords;
    s.gen = reinterpret_cast<uint32_t*>(s.lo + kLoWords);
    s.timeouts = s.gen + kDecWGs;
    const int b = blockIdx.x;
    const int x = b & 7;   // group (all its workgroups share one XCD)
    const int i = b >> 3;  // index inside the group, 0..31
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // MFMA column slot (B / D operand)
    const int g = lane >> 4;  // MFMA k-group (A / B operand) and D row group
    const int m = lane & 15;  // MFMA A row
    const int k0 = kDecDownCols * i;                 // first W_down column (inside stream i / 8)
    const int c0 = kDecUpCols * (kDecWgPerXcd * x + i);  // first output column
    const bool reducer = i < kDecReducers;
    const int u = i;                                 // reducer index: rows 3 u .. 3 u + 2 of the group
    // this launch's generation: one more than the launches this workgroup has
    // seen.  Every lane loads the counter (no per-lane branch); the value is
    // used only after the W_down tile has landed.
    uint32_t seen = __hip_atomic_load(&s.gen[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The dispatcher deals workgroups to the XCDs round robin, starting where
    // the previous dispatch stopped: workgroup b runs on XCD (b + r) % 8 with
    // one rotation r for the whole launch, so the workgroups of one group x
    // share an L2 whatever r is.  Each workgroup puts its own r into the tags
    // of the words it hands over inside its XCD, and a reducer accepts only
    // its own r: a producer that ran on another XCD shows up as an expired
    // (counted) wait, never as a silent stale read.
    const uint32_t rot = (__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) - (uint32_t)x) & 7u;
#if defined(HC_PROBE_STAMPS)
    unsigned long long probe_t[16] = {};
#endif
    HC_PROBE(0, threadIdx.x == 0);
    if (threadIdx.x == 0)
        poisoned_wg = 0;  // (ordered before any setter by the barriers B1, Bc1, Bs)
    const float* const Pm = P ? P : R;  // (a missing pending re-reads R)

    // ---- Loads.  The poll-line touches, the activations of the W_down tile's
    //      columns and the tile come first; the W_up tile and R' of its rows are
    //      issued only after this workgroup's down work (and, for a reducer,
    //      after hop 1).  While loads into LDS are in flight the compiler makes
    //      every LDS access wait for them, and a CU answers a poll only after
    //      its own earlier loads: the second tile's loads must not overlap
    //      either.  Loads issued before the first wait are unconditional
    //      (items past the end re-read item 0): a conditional load makes the
    //      compiler merge registers, which waits.
    // (0) a reducer touches (plain loads, which keep the lines in this XCD's
    //     L2) the lines it will poll: the 32 producers' partial rows 3 u ..
    //     3 u + 2 and their sums of squares.  Polls then hit L2 and see a
    //     producer's store as soon as it lands, instead of each round
    //     fetching the line from memory.
    uint32_t touched = 0, touched2 = 0, touched3 = 0, touched4 = 0;
    if (wave == 0 && reducer) {
        const int src = lane & 31, k = lane >> 5;
        const size_t prow = ((size_t)x * kDecWgPerXcd + src) * kDecRowsPerXcd;
        if constexpr (T <= 8) {
            // k 0, 1: the lines of rows 3 u and 3 u + 2 (two rows per line)
            const int row = kDecRedRows * u + 2 * k < kDecRowsPerXcd ? kDecRedRows * u + 2 * k : kDecRowsPerXcd - 1;
            touched = *reinterpret_cast<const uint32_t*>(s.part + (prow + row) * kTokSlots<T>);
            touched2 = *reinterpret_cast<const uint32_t*>(s.ssq + ((size_t)x * kDecWgPerXcd + src) * kSsqLine<T>);
        } else if constexpr (T <= 16) {
            // one row per line: rows 3 u + k, then row 3 u + 2 (k = 0) or the
            // sums of squares (k = 1)
            const int r0 = kDecRedRows * u + k, r2 = kDecRedRows * u + 2;
            touched = *reinterpret_cast<const uint32_t*>(s.part + (prow + r0) * kTokSlots<T>);
            touched2 = *reinterpret_cast<const uint32_t*>(
                k == 0 ? s.part + (prow + (r2 < kDecRowsPerXcd ? r2 : kDecRowsPerXcd - 1)) * kTokSlots<T>
                       : s.ssq + ((size_t)x * kDecWgPerXcd + src) * kSsqLine<T>);
        } else {
            // two lines per row: k = 0 takes both lines of rows 3 u and
            // 3 u + 1, k = 1 those of row 3 u + 2 and of the sums of squares
            const int ra = kDecRedRows * u + 2 * k, rb = kDecRedRows * u + 1;
            const uint64_t* la = s.part + (prow + (ra < kDecRowsPerXcd ? ra : kDecRowsPerXcd - 1)) * kTokSlots<T>;
            const uint64_t* lb = k == 0 ? s.part + (prow + (rb < kDecRowsPerXcd ? rb : kDecRowsPerXcd - 1)) * kTokSlots<T>
                                        : s.ssq + ((size_t)x * kDecWgPerXcd + src) * kSsqLine<T>;
            touched = *reinterpret_cast<const uint32_t*>(la);
            touched2 = *reinterpret_cast<const uint32_t*>(la + 16);
            touched3 = *reinterpret_cast<const uint32_t*>(lb);
            touched4 = *reinterpret_cast<const uint32_t*>(lb + 16);
        }
    }
    // (1) the activations of columns [k0, k0 + 320), first: staging y waits
    //     only for them and runs while the W_down tile lands
    constexpr int kItems = kStageItems * T;
    constexpr int kPasses = (kItems + kDecThreads - 1) / kDecThreads;
    float4 rv[kPasses], pv[kPasses], wv[kPasses];
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int it = threadIdx.x + kDecThreads * pass;
        const int itc = it < kItems ? it : 0;
        const int at = itc / kStageItems, f = itc - at * kStageItems;
        const size_t o = (size_t)at * kD + k0 + 4 * f;
        rv[pass] = *reinterpret_cast<const float4*>(R + o);
        pv[pass] = *reinterpret_cast<const float4*>(Pm + o);
        wv[pass] = *reinterpret_cast<const float4*>(w_norm + k0 + 4 * f);
    }
    // (2) W_down tile: rows 40 x + row, columns k0 + 8 j .. (buffer loads
    //     into LDS, which the compiler counts like ordinary loads; the
    //     scheduling barrier keeps them behind the activations)
    __builtin_amdgcn_sched_barrier(0);
    {
        const __amdgpu_buffer_rsrc_t wdr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(W_down), 0, 0x7fffffff, 0x00020000);
        // instructions wave + 8 k: k < 3 in every wave, k = 3 in wave 0 only
        // (unrolled, and unconditional where possible: the compiler can then
        // count the loads issued after the activations)
        static_assert(kTileInstr == 25, "25 wave instructions per tile");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = wave + 8 * k;
            if (k < 3 || wave == 0) {
                int row, j;
                tile_lane<kRowChunks>(q, lane, row, j);
                bdma16(wdr, dtile + 64 * q, 2u * ((uint32_t)(kDecRowsPerXcd * x + row) * kD + k0 + 8 * j));
            }
        }
    }
    // (4) later: the W_up tile (tile row 4 c + s = W_up row s * 2560 + c0 + c;
    //     buffer loads into LDS, unrolled like the W_down tile's, which the
    //     compiler counts exactly where after global_load_lds it would wait
    //     for every load before the first use of a polled word) and R and
    //     pending of those 40 (stream, column) pairs, for the mix.
    //     Above 8 tokens thread j's pass pp holds item j + 512 pp = 40 t + row
    //     (staged through LDS); in the quad layout lane (n, g) of wave w < 3
    //     holds, in slot c, token 4 c + g of the tile row its up products
    //     land on (tokens past T re-read token 0).
    constexpr int kUpPasses = kQuad<T> ? kQuadChains<T> : (kUpRows * T + kDecThreads - 1) / kDecThreads;
    float mr[kUpPasses], mp[kUpPasses];
    const int up_row = wave < 2 ? 16 * wave + n : 32 + (n & 7);  // (quad layout, waves 0..2)
    auto issue_up = [&]() {
        const __amdgpu_buffer_rsrc_t wur = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(W_up), 0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = wave + 8 * k;
            if (k < 3 || wave == 0) {
                int row, j;
                tile_lane<kRowChunks>(q, lane, row, j);
                bdma16(wur, utile + 64 * q, 2u * ((uint32_t)((row & 3) * kWidth + c0 + (row >> 2)) * kRank + 8 * j));
            }
        }
        if constexpr (kQuad<T>) {
            if (wave < 3) {
#pragma unroll
                for (int c = 0; c < kUpPasses; ++c) {
                    const int t = 4 * c + g;
                    const size_t o = (size_t)(t < T ? t : 0) * kD + (up_row & 3) * kWidth + c0 + (up_row >> 2);
                    mr[c] = R[o];
                    mp[c] = Pm[o];
                }
            }
        } else {
#pragma unroll
            for (int pp = 0; pp < kUpPasses; ++pp) {
                const int it = threadIdx.x + kDecThreads * pp;
                const int itc = it < kUpRows * T ? it : 0;
                const int at = itc / kUpRows, row = itc - at * kUpRows;
                const size_t o = (size_t)at * kD + (row & 3) * kWidth + c0 + (row >> 2);
                mr[pp] = R[o];
                mp[pp] = Pm[o];
            }
        }
    };

    // (6) y = R' * w_norm (unscaled: the norm is folded into the reduction),
    //     its sums of squares, and the exact 3-way split
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int it = threadIdx.x + kDecThreads * pass;
        if (it < kItems) {
            const int at = it / kStageItems, f = it - at * kStageItems;
            float ss = 0.f;
            uint32_t hi[4], mi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float rvv[4] = {rv[pass].x, rv[pass].y, rv[pass].z, rv[pass].w};
                const float pvv[4] = {pv[pass].x, pv[pass].y, pv[pass].z, pv[pass].w};
                const float wvv[4] = {wv[pass].x, wv[pass].y, wv[pass].z, wv[pass].w};
                const float r = P ? rvv[e] + pvv[e] : rvv[e];
                ss += r * r;
                split3(r * wvv[e], hi[e], mi[e], lo[e]);
            }
            ds_st32(&sspart[at * kStageItems + f], __float_as_uint(ss));
            const int col = 4 * f;
            ds_st64(&ypl[plane_row<T>(0, at) * kYRow + col], u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)});
            ds_st64(&ypl[plane_row<T>(1, at) * kYRow + col], u32x2_t{mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16)});
            ds_st64(&ypl[plane_row<T>(2, at) * kYRow + col], u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)});
        }
    }
    wait_all_loads();  // this wave's part of the W_down tile is in LDS
    asm volatile("" ::"v"(touched), "v"(touched2), "v"(touched3), "v"(touched4));
    wg_barrier();      // B1: y staged, W_down tile complete
    HC_PROBE(1, threadIdx.x == 0);
    pin(seen);
    const uint32_t gen = ((uint32_t)__builtin_amdgcn_readfirstlane((int)seen) + 1u) & kGenMask;

    // (7) down projection.  Above 8 tokens wave w < 6 takes rows 16 (w % 3)
    //     .. +15 of the tile (block 2: rows 32..39, its upper 8 slots repeat
    //     them) over K steps 5 (w / 3) .. +4 of 32 columns.  A rows are
    //     (piece, token) pairs in the planes' own order (row p T + t: piece p
    //     of token t), so 2, 3 or 6 chains carry the pieces (kChains).  Up to
    //     8 tokens (quad layout) wave w < 3 takes rows 16 w .. +15 over all 10
    //     K steps, and lane (n, g) of chain c ends with the three pieces'
    //     products of token 4 c + g, row 16 w + n, in elements 0..2.
    if (wave < (kQuad<T> ? 3 : 6)) {
        if constexpr (kQuad<T>) {
            // (7q, 8q) products, then the partial dots straight into the
            //     XCD's L2: hi + (mid + lo3) per token, all 8 token slots
            //     (whole lines; slots >= T hold 0)
            constexpr int NC = kQuadChains<T>;
            const int row = wave < 2 ? 16 * wave + n : 32 + (n & 7);
            uint4 wb[10], a[NC][10];
#pragma unroll
            for (int q = 0; q < 10; ++q) {
                const int col = 32 * q + 8 * g;
                wb[q] = dtile[tile_pos<kRowChunks>(row, 4 * q + g)];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    a[c][q] = *reinterpret_cast<const uint4*>(&ypl[(16 * c + m) * kYRow + col]);
            }
            f32x4_t acc[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 10; ++q)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[c] = mfma16(a[c][q], wb[q], acc[c]);
            HC_PROBE(2, threadIdx.x == 0);
            if (wave < 2 || n < 8) {  // (block 2's upper slots are copies)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = 4 * h + g;
                    const f32x4_t d = acc[h < NC ? h : 0];
                    const float v = h < NC && t < T ? d[0] + (d[1] + d[2]) : 0.f;
                    st_word_xcd(s.part + (((size_t)x * kDecWgPerXcd + i) * kDecRowsPerXcd + row) * kTokSlots<T> + t,
                                tag_f32(v, xcd_tag(gen, rot)));
                }
            }
        } else {
            constexpr int NC = kChains<T>;
            const int nb = wave % 3, kh = wave / 3;
            const int row = nb < 2 ? 16 * nb + n : 32 + (n & 7);
            // all operands first (one LDS latency, not five); A rows past the
            // pieces re-read the chain's first row: they only feed D rows nobody reads
            int ar[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                ar[c] = chain_base<T>(c) + (m < chain_rows<T>(c) ? m : 0);
            uint4 wb[5], a[NC][5];
#pragma unroll
            for (int qq = 0; qq < 5; ++qq) {
                const int q = 5 * kh + qq;
                const int col = 32 * q + 8 * g;
                wb[qq] = dtile[tile_pos<kRowChunks>(row, 4 * q + g)];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    a[c][qq] = *reinterpret_cast<const uint4*>(&ypl[ar[c] * kYRow + col]);
            }
            f32x4_t acc[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qq = 0; qq < 5; ++qq)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[c] = mfma16(a[c][qq], wb[qq], acc[c]);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                comb[(wave * NC + c) * 64 + lane] = acc[c];
        }
    } else if (wave == 6 || (T > 16 && wave == 7)) {
        // (7') meanwhile, the slice's sum of squares per token: lane 8 t + p
        //      sums 10 of token t's 80 item sums, then the 8 lanes combine theirs
        if constexpr (T <= 8) {
            const int tt = lane >> 3, p = lane & 7;
            float ss = 0.f;
            if (tt < T) {
#pragma unroll
                for (int f = 0; f < kStageItems / 8; ++f)
                    ss += sspart[tt * kStageItems + (kStageItems / 8) * p + f];
            }
            ss = sum8(ss);
            if (p < 2)  // words 0..7: tokens (0 past T); words 8..15: padding -- one whole line
                st_word_xcd(&s.ssq[((size_t)x * kDecWgPerXcd + i) * kSsqLine<T> + 8 * p + tt],
                            tag_f32(p == 0 ? ss : 0.f, xcd_tag(gen, rot)));
        } else {
            // lane 4 t + p sums 20 of token t's 80 item sums, then the 4
            // lanes combine theirs; words 0..15: tokens (0 past T); above 16
            // tokens waves 6 and 7 share the work (lane 4 t + p of their 128),
            // words 0..31 (two lines, one per wave)
            const int l = threadIdx.x - 6 * 64, tt = l >> 2, p = l & 3;
            float ss = 0.f;
            if (tt < T) {
#pragma unroll
                for (int f = 0; f < kStageItems / 4; ++f)
                    ss += sspart[tt * kStageItems + (kStageItems / 4) * p + f];
            }
            ss = sum4(ss);
            if (p == 0)
                st_word_xcd(&s.ssq[((size_t)x * kDecWgPerXcd + i) * kSsqLine<T> + tt], tag_f32(ss, xcd_tag(gen, rot)));
        }
    }
    if constexpr (!kQuad<T>) {
        HC_PROBE(2, threadIdx.x == 0);
        wg_barrier();  // Bc1: every product block in LDS

        if (wave < 6) {
            // (8) partial dots of rows 16 (w % 3) + n, token 4 (w / 3) + g, into
            //     the XCD's L2: per K half hi + (mid + lo3), then the two halves
            //     (all 8 token slots, whole lines; slots >= T hold 0)
            //     (above 8 tokens each lane also takes tokens t + 8, t + 16, ...:
            //     16 or 32 slots)
            const float* cf = reinterpret_cast<const float*>(comb);
            const int nb = wave % 3, t = 4 * (wave / 3) + g;
            const int row = 16 * nb + n;
            if (row < kDecRowsPerXcd) {
#pragma unroll
                for (int h = 0; h < kTokSlots<T> / 8; ++h) {
                    const int th = t + 8 * h;
                    const float v = th < T ? piece_sum<T>(cf, nb, th, n) + piece_sum<T>(cf, nb + 3, th, n) : 0.f;
                    st_word_xcd(s.part + (((size_t)x * kDecWgPerXcd + i) * kDecRowsPerXcd + row) * kTokSlots<T> + th,
                                tag_f32(v, xcd_tag(gen, rot)));
                }
            }
        }
    }
    HC_PROBE(3, threadIdx.x == 0);

    if (!reducer)
        issue_up();

    // above 8 tokens two waves share hop 1 (each takes half the pair groups)
    constexpr int kHopWaves = T > 8 ? 2 : 1;
    if (wave < kHopWaves && reducer) {
        // (9) hop 1: lo rows 3 u .. 3 u + 2 of this group from its 32
        //     workgroups' partials, each stream's rs from its 8 slices' sums
        //     of squares; lo published device-wide.  Lane src + 16 k holds
        //     sources src (streams 0-1) and src + 16 (streams 2-3); within
        //     each 16 lanes, lanes 8 s' .. 8 s' + 7 hold the 8 slices of
        //     streams s' and s' + 2.  Up to 4 tokens, lane group k = row
        //     (rows in parallel, tokens in turn); from 5 tokens, k = pair of
        //     tokens (one load per row and source per polling round).
        const uint32_t htag = xcd_tag(gen, rot);
        const long long t0 = wall_clock64();
        const int src = lane & 15, k = lane >> 4;
        const int pa0 = (x * kDecWgPerXcd + src) * kDecRowsPerXcd, pb0 = pa0 + 16 * kDecRowsPerXcd;
        const int sa0 = (x * kDecWgPerXcd + src) * kSsqLine<T>, sb0 = sa0 + 16 * kSsqLine<T>;
        // lo of (stream pair sums) -> (s0 + s1) + (s2 + s3), the same in all 16 lanes
        auto combine = [](float pa, float pb, float qa, float qb) {
            const float rsa = rsqrtf(sum8(qa) * (1.0f / (float)kWidth) + kEps);
            const float rsb = rsqrtf(sum8(qb) * (1.0f / (float)kWidth) + kEps);
            const float ya = sum8(pa) * rsa, yb = sum8(pb) * rsb;
            const float za = ya + dpp<0x140>(ya);  // row_mirror: the other half's stream
            const float zb = yb + dpp<0x140>(yb);
            return za + zb;
        };
        if constexpr (T <= 4) {
            constexpr int NP = (T + 1) / 2;
            const int row = kDecRedRows * u + k;
            const bool valid = k < kDecRedRows && row < kDecRowsPerXcd;
            const int rowc = valid ? row : kDecRedRows * u;  // (a row of this reducer, read and discarded)
            const int pa = (pa0 + rowc) * kTokSlots<T>, pb = (pb0 + rowc) * kTokSlots<T>;
            uint4 wa_[NP], wb_[NP], qa_[NP], qb_[NP];
            [[maybe_unused]] int rounds = 0;
            bool expired = false;  // (wave-uniform: the clock is a scalar read)
            while (true) {
                ++rounds;
                new_round();
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    wa_[q] = ld_words2(s.part, pa + 2 * q);
                    wb_[q] = ld_words2(s.part, pb + 2 * q);
                    qa_[q] = ld_words2(s.ssq, sa0 + 2 * q);
                    qb_[q] = ld_words2(s.ssq, sb0 + 2 * q);
                }
                bool ok = true;
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    ok = ok & (wa_[q].y == htag) & (wb_[q].y == htag) & (qa_[q].y == htag) & (qb_[q].y == htag) &
                         (2 * q + 1 >= T || ((wa_[q].w == htag) & (wb_[q].w == htag) & (qa_[q].w == htag) &
                                             (qb_[q].w == htag)));
                if (__all(ok)) {
                    HC_COUNT(0, 0, rounds, lane == 0);
                    break;
                }
                if (wall_clock64() - t0 > wait_ticks) {
                    if (lane == 0)
                        note_timeout(s.timeouts);
                    expired = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            HC_PROBE(12, lane == 0);
            float mine = 0.f;  // lo of row 3 u + k, token `src`
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const bool hi = t & 1;
                const float lo = combine(__uint_as_float(hi ? wa_[t >> 1].z : wa_[t >> 1].x),
                                         __uint_as_float(hi ? wb_[t >> 1].z : wb_[t >> 1].x),
                                         __uint_as_float(hi ? qa_[t >> 1].z : qa_[t >> 1].x),
                                         __uint_as_float(hi ? qb_[t >> 1].z : qb_[t >> 1].x));
                if (src == t)
                    mine = lo;
            }
            // 32 words (2 whole lines) per replica: tokens 0..7 x rows 0..3 of
            // this reducer, 0 in the padding; lane src < 8 of group k writes
            // row k, token src
            const uint64_t word = expired ? tag_f32(__builtin_nanf(""), gen | kPoison)
                                          : tag_f32(valid && src < T ? mine : 0.f, gen);
#pragma unroll
            for (int y = 0; y < kDecXcds; ++y)
                if (src < 8)
                    st_word(&s.lo[lo_word<T>(y, x, u, src, k)], word);
        } else {
            // token pairs: lane group k takes pairs k + 4 q (q < NQ: tokens
            // 2 k + 8 q, 2 k + 8 q + 1), all 3 rows.  Only the pair groups
            // holding tokens are reduced (the slots past them are padding);
            // with two hop waves wave w takes groups NQ w + q, q < NQ, and a
            // group past the tokens re-reads the last one (no conditional
            // polling load) and publishes nothing.
            constexpr int NQT = (T + 7) / 8;                         // pair groups holding tokens
            constexpr int NQ = kHopWaves == 2 ? (NQT + 1) / 2 : NQT;  // pair groups of this wave
            const int qb = NQ * wave;                                // its first group
            int qo[NQ];                                    // word offsets of its groups
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                qo[q] = 8 * (qb + q < NQT ? qb + q : NQT - 1);
            int pidx[kDecRedRows];
#pragma unroll
            for (int rr = 0; rr < kDecRedRows; ++rr) {
                const int row = kDecRedRows * u + rr;
                pidx[rr] = (row < kDecRowsPerXcd ? row : kDecRowsPerXcd - 1) * kTokSlots<T> + 2 * k;
            }
            uint4 wa_[kDecRedRows][NQ], wb_[kDecRedRows][NQ], qa_[NQ], qb_[NQ];
            [[maybe_unused]] int rounds = 0;
            bool expired = false;  // (wave-uniform)
            while (true) {
                ++rounds;
                new_round();
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr) {
                        wa_[rr][q] = ld_words2(s.part, pa0 * kTokSlots<T> + pidx[rr] + qo[q]);
                        wb_[rr][q] = ld_words2(s.part, pb0 * kTokSlots<T> + pidx[rr] + qo[q]);
                    }
                    qa_[q] = ld_words2(s.ssq, sa0 + 2 * k + qo[q]);
                    qb_[q] = ld_words2(s.ssq, sb0 + 2 * k + qo[q]);
                }
                bool ok = true;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    ok = ok & (qa_[q].y == htag) & (qa_[q].w == htag) & (qb_[q].y == htag) & (qb_[q].w == htag);
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr)
                        ok = ok & (wa_[rr][q].y == htag) & (wa_[rr][q].w == htag) & (wb_[rr][q].y == htag) &
                             (wb_[rr][q].w == htag);
                }
                if (__all(ok)) {
                    HC_COUNT(0, 0, rounds, lane == 0);
                    break;
                }
                if (wall_clock64() - t0 > wait_ticks) {
                    if (lane == 0)
                        note_timeout(s.timeouts);
                    expired = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            HC_PROBE(12, lane == 0);
            float lo[kDecRedRows][NQ][2];  // [row][pair group][token], the same in all 16 lanes of k
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int rr = 0; rr < kDecRedRows; ++rr)
                        lo[rr][q][h] = combine(__uint_as_float(h ? wa_[rr][q].z : wa_[rr][q].x),
                                               __uint_as_float(h ? wb_[rr][q].z : wb_[rr][q].x),
                                               __uint_as_float(h ? qa_[q].z : qa_[q].x),
                                               __uint_as_float(h ? qb_[q].z : qb_[q].x));
            // lane src of group k writes row (src / 2) % 4 (row 3: padding),
            // token 2 k + src % 2 + 8 (qb + q) for q = src / 8 (+ 2 w: with
            // 3 or 4 pair groups in one wave each lane writes two words)
            constexpr int NW = NQ > 2 ? 2 : 1;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const int rr = (src >> 1) & 3, h = src & 1, q = (src >> 3) + 2 * w2, tok = 2 * k + h + 8 * (qb + q);
                float mine = 0.f;
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
                    for (int r3 = 0; r3 < kDecRedRows; ++r3)
                        mine = (qq == q && r3 == rr) ? (h ? lo[r3][qq][1] : lo[r3][qq][0]) : mine;
                const bool valid = rr < kDecRedRows && kDecRedRows * u + rr < kDecRowsPerXcd && tok < T;
                const uint64_t word = expired ? tag_f32(__builtin_nanf(""), gen | kPoison)
                                              : tag_f32(valid ? mine : 0.f, gen);
#pragma unroll
                for (int y = 0; y < kDecXcds; ++y)
                    if (q < NQ && qb + q < NQT)
                        st_word(&s.lo[lo_word<T>(y, x, u, tok, rr)], word);
            }
        }
        HC_PROBE(13, lane == 0);
    }
    wg_barrier();  // Bs: this workgroup's hop 1 done
    if (reducer)
        issue_up();
    {
        // (10) hop 2: wave w polls the lo words of XCD w's reducers (slot =
        //     reducer, token, pair of rows) until every tag is current, then
        //     stages the 3 bf16 pieces of each value (inline-asm LDS stores,
        //     which do not wait for the W_up tile still landing).  (Waves start after this
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
            widx[k] = lo_word<T>(x, wave, us, tt, 2 * pair);
        }
        [[maybe_unused]] int rounds = 0;
        bool bad = false;  // this wave's wait expired, or a word it got is poison
        while (true) {
            ++rounds;
            new_round();
#pragma unroll
            for (int k = 0; k < NS; ++k)
                lw[k] = ld_words2(s.lo, widx[k]);
            bool all = true;
#pragma unroll
            for (int k = 0; k < NS; ++k)
                all = all && (lw[k].y & kGenMask) == gen && (lw[k].w & kGenMask) == gen;
            if (__all(all)) {
                HC_COUNT(2, 1, rounds, wave == 0 && lane == 0);
                break;
            }
            if (wall_clock64() - t0 > wait_ticks) {
                if (lane == 0)
                    note_timeout(s.timeouts);
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        bool got_poison = false;
#pragma unroll
        for (int k = 0; k < NS; ++k)
            got_poison = got_poison || ((lw[k].y | lw[k].w) & kPoison) != 0;
        bad = bad || __any(got_poison);
        if (bad) {
            // NaN lo: the up projection then gives NaN for every token
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                lw[k].x = __float_as_uint(__builtin_nanf(""));
                lw[k].z = lw[k].x;
            }
            if (lane == 0)
                poisoned_wg = 1;
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
                        ds_st16(&lpl[plane_row<T>(0, tt) * kLoRow + jr], hb);
                        ds_st16(&lpl[plane_row<T>(1, tt) * kLoRow + jr], mb);
                        ds_st16(&lpl[plane_row<T>(2, tt) * kLoRow + jr], lb);
                    }
                }
            }
        }
        HC_PROBE(7, wave == 0 && lane == 0);
    }
    wait_all_loads();  // the W_up tile and R' have landed
    float rprime[kUpPasses];
#pragma unroll
    for (int pp = 0; pp < kUpPasses; ++pp) {
        rprime[pp] = P ? mr[pp] + mp[pp] : mr[pp];
        const int it = threadIdx.x + kDecThreads * pp;  // it = 40 t + row
        if (!kQuad<T> && it < kUpRows * T)
            rpl[it] = rprime[pp];
    }
    wg_barrier();  // B2: lo and R' staged, W_up tile complete
    HC_PROBE(8, threadIdx.x == 0);
    const bool poisoned = poisoned_wg != 0;
    // (10') the pending write committed: R' of this workgroup's 40 (stream,
    //      column) pairs back into R.  No read of these elements is left
    //      anywhere: every workgroup read them for its down part before it
    //      stored the partials that hop 2 has just waited for, and no other
    //      workgroup mixes these columns.  (After an expired wait that is not
    //      known: nothing is committed.)
    if constexpr (kQuad<T>) {
        // (each (stream, column, token) once: block 2's upper slots are copies)
        if (R_commit && P && !poisoned && wave < 3 && (wave < 2 || n < 8)) {
#pragma unroll
            for (int c = 0; c < kUpPasses; ++c)
                if (4 * c + g < T)
                    R_commit[(size_t)(4 * c + g) * kD + (up_row & 3) * kWidth + c0 + (up_row >> 2)] = rprime[c];
        }
    } else {
#pragma unroll
        for (int pp = 0; pp < kUpPasses; ++pp) {
            const int it = threadIdx.x + kDecThreads * pp;
            if (R_commit && P && !poisoned && it < kUpRows * T) {
                const int at = it / kUpRows, row = it - at * kUpRows;
                R_commit[(size_t)at * kD + (row & 3) * kWidth + c0 + (row >> 2)] = rprime[pp];
            }
        }
    }

    if constexpr (kQuad<T>) {
        if (wave < 3) {
            // (11q) up projection, quad layout: wave w takes tile rows 16 w ..
            //      +15 (slot n = 4 column + stream; block 2: rows 32..39, its
            //      upper 8 slots repeat them), all 10 K steps; lane (n, g) of
            //      chain c ends with the pieces of token 4 c + g in elements
            //      0..2: up = hi + (mid + lo3); gated = up (identity
            //      epilogue); then the mix of the 4 streams of a column
            //      ((s0 + s1) + (s2 + s3), across the lane quad)
            constexpr int NC = kQuadChains<T>;
            uint4 wb[10], a[NC][10];
#pragma unroll
            for (int q = 0; q < 10; ++q) {
                const int jc = 32 * q + 8 * g;
                wb[q] = utile[tile_pos<kRowChunks>(up_row, 4 * q + g)];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    a[c][q] = *reinterpret_cast<const uint4*>(&lpl[(16 * c + m) * kLoRow + jc]);
            }
            f32x4_t acc[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 10; ++q)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc[c] = mfma16(a[c][q], wb[q], acc[c]);
            const int col = c0 + (up_row >> 2);
            const bool owner = (n & 3) == 0 && (wave < 2 || n < 8);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int t = 4 * c + g;
                const float up = acc[c][0] + (acc[c][1] + acc[c][2]);
                const float mixed = poisoned ? __builtin_nanf("") : sum4(up * rprime[c]);
                if (owner && t < T) {
                    const size_t o = (size_t)t * kWidth + col;
                    out_mixed[o] = mixed;
                    out_bf16[o] = __builtin_bit_cast(uint16_t, (__bf16)mixed);
                    out_fp16[o] = __builtin_bit_cast(uint16_t, (_Float16)mixed);
                }
            }
            HC_PROBE(9, wave == 0 && lane == 0);
        }
    } else {
        constexpr bool kSplitUp = kChains<T> == 6;  // above 16 tokens: one token half per wave
        if (wave < (kSplitUp ? 6 : 3)) {
            // (11) up projection: wave w takes tile rows 16 rb .. +15, rb = w % 3
            //      (slot n = 4 column + stream; block 2: rows 32..39, its upper 8
            //      slots repeat them), all 10 K steps, A rows packed as in the down
            //      projection (above 16 tokens: waves 0-2 the chains of tokens
            //      0..15, waves 3-5 those of tokens 16..); gated = up (identity
            //      epilogue); then the mix of the 4 streams of a column
            constexpr int UC = kSplitUp ? 3 : kChains<T>;  // chains per wave
            const int rb = wave % 3, th = kSplitUp ? wave / 3 : 0;
            const int row = rb < 2 ? 16 * rb + n : 32 + (n & 7);
            const int st = n & 3;
            int ar[UC];
#pragma unroll
            for (int j = 0; j < UC; ++j) {
                const int c = kSplitUp ? 2 * j + th : j;
                ar[j] = chain_base<T>(c) + (m < chain_rows<T>(c) ? m : 0);
            }
            uint4 wb[10], a[UC][10];
#pragma unroll
            for (int q = 0; q < 10; ++q) {
                const int jc = 32 * q + 8 * g;
                wb[q] = utile[tile_pos<kRowChunks>(row, 4 * q + g)];
#pragma unroll
                for (int j = 0; j < UC; ++j)
                    a[j][q] = *reinterpret_cast<const uint4*>(&lpl[ar[j] * kLoRow + jc]);
            }
            f32x4_t acc[UC];
#pragma unroll
            for (int j = 0; j < UC; ++j)
                acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 10; ++q)
#pragma unroll
                for (int j = 0; j < UC; ++j)
                    acc[j] = mfma16(a[j][q], wb[q], acc[j]);
            // a token's pieces sit in other lanes: through this wave's own LDS block
            f32x4_t* const ub = ucomb + wave * UC * 64;
#pragma unroll
            for (int j = 0; j < UC; ++j)
                ub[64 * j + lane] = acc[j];
            asm volatile("" ::: "memory");  // (LDS operations of one wave complete in order)
            const float* cf = reinterpret_cast<const float*>(ub);
            const int c = c0 + (row >> 2);
            const bool owner = st == 0 && (rb < 2 || n < 8);  // (block 2's upper slots are copies)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i16 = 4 * g + e, tt = 16 * th + i16;
                // block j holds piece j of tokens 16 th + i16 (row i16 of the block)
                auto at = [&](int j) { return cf[(64 * j + n + 16 * (i16 >> 2)) * 4 + (i16 & 3)]; };
                const float up = tt < T ? (kSplitUp ? at(0) + (at(1) + at(2)) : piece_sum<T>(cf, 0, tt, n)) : 0.f;
                const float rp = rpl[(tt < T ? tt : 0) * kUpRows + row];
                const float mixed = poisoned ? __builtin_nanf("") : sum4(up * rp);  // (s0 + s1) + (s2 + s3)
                if (owner && tt < T) {
                    const size_t o = (size_t)tt * kWidth + c;
                    out_mixed[o] = mixed;
                    out_bf16[o] = __builtin_bit_cast(uint16_t, (__bf16)mixed);
                    out_fp16[o] = __builtin_bit_cast(uint16_t, (_Float16)mixed);
                }
            }
            HC_PROBE(9, wave == 0 && lane == 0);
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&s.gen[b], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#if defined(HC_PROBE_STAMPS)
    HC_PROBE(15, true);
    if (threadIdx.x == 0)
        for (int p = 0; p < 16; ++p)
            hc_probe_ring[((gen & 63) * kDecWGs + b) * 16 + p] = probe_t[p];
#endif
}

// The allocation-free reads' scratch: one short-window workspace in a
// file-scope device array, which every GPU the library runs on holds until
// the process ends.  Host code never uses its name as an address: set-up takes
// each device's own address of it with hipGetSymbolAddress.
constexpr size_t kScratchWords = kPartWords + kSsqWords + kLoWords + (kDecWGs + 64) / 2;
static __device__ __align__(256) uint64_t scratch[kScratchWords];
constexpr int kMaxDevices = 64;
void* g_noalloc_base[kMaxDevices] = {};  // per device: the array's address (set-up done)

}  // namespace

size_t decode_scratch_bytes()
{
    return sizeof(uint64_t) * (kPartWords + kSsqWords + kLoWords) + sizeof(uint32_t) * (kDecWGs + 64);
}

hipError_t noalloc_setup(int dev, hipStream_t stream)
{
    static_assert(sizeof(scratch) >= sizeof(uint64_t) * (kPartWords + kSsqWords + kLoWords) +
                                           sizeof(uint32_t) * (kDecWGs + 64), "scratch size");
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    if (g_noalloc_base[dev])
        return hipSuccess;
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    // the hand-off protocol needs every word and counter to start at zero
    e = hipMemsetAsync(p, 0, decode_scratch_bytes(), stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return e;
    g_noalloc_base[dev] = p;
    return hipSuccess;
}

bool noalloc_scratch(int dev, DecodeScratch* s)
{
    if (dev < 0 || dev >= kMaxDevices || !g_noalloc_base[dev])
        return false;
    decode_scratch_carve(g_noalloc_base[dev], s);
    return true;
}

void decode_scratch_carve(void* base, DecodeScratch* s)
{
    s->part = static_cast<uint64_t*>(base);
    s->ssq = s->part + kPartWords;
    s->lo = s->ssq + kSsqWords;
    s->gen = reinterpret_cast<uint32_t*>(s->lo + kLoWords);
    s->timeouts = s->gen + kDecWGs;
}

#if defined(HC_PROBE_STAMPS)
// Timing build only: copies the stamp ring (64 x 256 x 16 values) to host.
extern "C" __attribute__((visibility("default"))) int hc_probe_stamps(unsigned long long* host)
{
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(hc_probe_ring), sizeof(hc_probe_ring), 0,
                               hipMemcpyDeviceToHost) == hipSuccess ? 0 : 1;
}
#endif

hipError_t decode_resident_blocks(int* blocks_per_cu)
{
    // the largest-LDS instances (16 tokens without shared regions, 32 with)
    // bound residency for every T
    int a = 0, c = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &a, reinterpret_cast<const void*>(&decode_kernel<16>), kDecThreads, 0);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &c, reinterpret_cast<const void*>(&decode_kernel<kDecMaxT>), kDecThreads, 0);
    *blocks_per_cu = a < c ? a : c;
    return e;
}

hipError_t launch_decode(int T, const float* R, const float* P, const float* w_norm,
                         const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                         uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit,
                         const DecodeScratch& s, hipStream_t stream, long long wait_ticks)
{
    uint64_t* scratch = s.part;  // the carve's base: the kernel derives the rest
    void* args[] = {&W_down, &W_up, &R, &P, &w_norm, &scratch, &out_mixed, &out_bf16, &out_fp16, &R_commit,
                    &wait_ticks};
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
    case 9: fn = reinterpret_cast<const void*>(&decode_kernel<9>); break;
    case 10: fn = reinterpret_cast<const void*>(&decode_kernel<10>); break;
    case 11: fn = reinterpret_cast<const void*>(&decode_kernel<11>); break;
    case 12: fn = reinterpret_cast<const void*>(&decode_kernel<12>); break;
    case 13: fn = reinterpret_cast<const void*>(&decode_kernel<13>); break;
    case 14: fn = reinterpret_cast<const void*>(&decode_kernel<14>); break;
    case 15: fn = reinterpret_cast<const void*>(&decode_kernel<15>); break;
    case 16: fn = reinterpret_cast<const void*>(&decode_kernel<16>); break;
    case 17: fn = reinterpret_cast<const void*>(&decode_kernel<17>); break;
    case 18: fn = reinterpret_cast<const void*>(&decode_kernel<18>); break;
    case 19: fn = reinterpret_cast<const void*>(&decode_kernel<19>); break;
    case 20: fn = reinterpret_cast<const void*>(&decode_kernel<20>); break;
    case 21: fn = reinterpret_cast<const void*>(&decode_kernel<21>); break;
    case 22: fn = reinterpret_cast<const void*>(&decode_kernel<22>); break;
    case 23: fn = reinterpret_cast<const void*>(&decode_kernel<23>); break;
    case 24: fn = reinterpret_cast<const void*>(&decode_kernel<24>); break;
    case 25: fn = reinterpret_cast<const void*>(&decode_kernel<25>); break;
    case 26: fn = reinterpret_cast<const void*>(&decode_kernel<26>); break;
    case 27: fn = reinterpret_cast<const void*>(&decode_kernel<27>); break;
    case 28: fn = reinterpret_cast<const void*>(&decode_kernel<28>); break;
    case 29: fn = reinterpret_cast<const void*>(&decode_kernel<29>); break;
    case 30: fn = reinterpret_cast<const void*>(&decode_kernel<30>); break;
    case 31: fn = reinterpret_cast<const void*>(&decode_kernel<31>); break;
    case 32: fn = reinterpret_cast<const void*>(&decode_kernel<32>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(kDecWGs), dim3(kDecThreads), args, 0, stream);
}

}  // namespace hc
