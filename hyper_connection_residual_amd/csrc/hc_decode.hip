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
// "#1370 prefill", "What it does" (a lane holds one (token, column) pair of
// all 4 streams and mixes them in registers, then writes the BF16/FP16 images).
//
// gfx950 design (the pages' kernels were written for RDNA2, Turing, Ada and
// Arc; none of their mechanics is reused):
//
// * 256 workgroups x 8 waves: exactly one workgroup per CU, so no CU carries
//   twice the weight bytes of another (a shared CU is always the straggler
//   every other workgroup ends up waiting for).  Every lane issues its whole
//   share of the 13 MB of weights as 16-byte loads at once.
// * Both projections run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
//   with tokens as the M dimension.  Each fp32 activation is split exactly into
//   three bf16 pieces (hi + mid + lo3 == x), so every product is exact and the
//   result stays fp32-faithful.
// * No grid barrier.  Hand-offs between workgroups are 64-bit words holding
//   their payload and the launch's generation number, written once with one
//   store and polled by the consumer, which sees either the old tag or the
//   whole new word.  Every workgroup counts its launches in its own slot, so
//   all of them agree on the generation without host involvement (the launch
//   is graph-capture safe).  Every wait is bounded.
// * The reduction is shaped by the chip's 8 XCDs.  A hop between workgroups of
//   one XCD goes through that XCD's L2 (stores land in L2; loads skip the CU's
//   L1); a hop between XCDs goes through device memory and costs several
//   times more.  The chain is: slice partials -> XCD partial (local) -> every
//   XCD gathers the 8 XCD partials and forms lo itself (the one device-wide
//   hop) -> lo spread inside the XCD (local).  Each XCD's columns lie inside a
//   single stream, so each stream's rs is applied at the device-wide hop.
// * Waves specialise.  Waves 0-4 run the down projection (16 rows each) and
//   then the hops; waves 5-7 hold the W_up rows of this workgroup's output
//   columns and run the up projection and the mix.  Global loads complete in
//   issue order per wave, so keeping the up weights in other waves lets the
//   down waves poll without waiting for them.  The up waves issue their loads
//   once this workgroup's W_down chunks have landed, so the W_down stream that
//   the reduction waits on gets the bandwidth first; the up weights land
//   while the hops are in flight.
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

namespace hc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr long long kWaitTicks = 5000000;  // 50 ms of the 100 MHz wall clock
constexpr int kUpSplitCols = 1536;         // workgroups 0..127 own 12 columns each, the rest 8
constexpr int kYRow = kDecSliceCols + 8;   // padded LDS row of an activation plane (bf16)
constexpr int kLoRow = kRank + 8;          // padded LDS row of a lo plane (bf16)

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

__device__ __forceinline__ void st_word(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// One hand-off word for the CUs of this XCD only: the store stays in the XCD's
// L2 (sc0) instead of writing through to memory, which halves the hop.
__device__ __forceinline__ void st_word_xcd(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t tag_f32(float v, uint32_t gen)
{
    return (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32);
}
__device__ __forceinline__ void note_timeout(uint32_t* timeouts)
{
    __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls the T words at `base + idx` for the two slots of this lane until every
// lane's words carry `gen`; returns them as floats.  Slot 1 exists for lanes
// < 16 only (80 slots: 8 sources x 10 rows).
template <int T>
__device__ __forceinline__ void poll80(const uint64_t* base, const int idx[2], uint32_t gen, int lane,
                                       float (&v)[2][T], uint32_t* timeouts)
{
    constexpr int NP = (T + 1) / 2;
    bool done[2] = {false, lane >= 16};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int t = 0; t < T; ++t)
            v[k][t] = 0.f;
    const long long t0 = wall_clock64();
    while (true) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!done[k]) {
                bool ok = true;
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const uint4 a = ld_words2(base, idx[k] + 2 * q);
                    ok = ok && a.y == gen && (2 * q + 1 >= T || a.w == gen);
                    v[k][2 * q] = __uint_as_float(a.x);
                    if (2 * q + 1 < T)
                        v[k][2 * q + 1] = __uint_as_float(a.z);
                }
                done[k] = ok;
            }
        }
        if (__all(done[0] && done[1]))
            return;
        if (wall_clock64() - t0 > kWaitTicks) {
            if (lane == 0)
                note_timeout(timeouts);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Hop B (wave 0 of workgroup (x, i)): the XCD partial of rows 10 i .. 10 i + 9
// = the sum of the XCD's 8 slice partials, published device-wide.  Lane slot
// sl: slice sl % 8, row 10 i + sl / 8.  Workgroup i == 0 also publishes the
// XCD's sum of squares.
template <int T>
__device__ __forceinline__ void hop_xcd_partial(const DecodeScratch& s, int x, int i, uint32_t gen,
                                                int lane)
{
    float v[2][T];
    int idx[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int sl = lane + 64 * k;
        const int row = kDecRowsPerWG * i + ((sl >> 3) < kDecRowsPerWG ? (sl >> 3) : 0);
        idx[k] = ((x * 8 + (sl & 7)) * kRank + row) * kDecMaxT;
    }
    poll80<T>(s.xs_part, idx, gen, lane, v, s.timeouts);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int sl = lane + 64 * k;
        const int row = kDecRowsPerWG * i + (sl >> 3);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float sum = sum8(v[k][t]);  // slices 0..7 of the XCD, fixed order
            if ((k == 0 || lane < 16) && (lane & 7) == t)
                st_word(&s.g_part[((size_t)x * kRank + row) * kDecMaxT + t], tag_f32(sum, gen));
        }
    }
    if (i == 0 && lane < 8) {
        float ss[T];
        const long long t0 = wall_clock64();
        while (true) {
            bool ok = true;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint4 a = ld_words2(s.xs_ssq, (x * 8 + lane) * kDecMaxT + (t & ~1));
                const uint32_t tagw = (t & 1) ? a.w : a.y;
                ok = ok && tagw == gen;
                ss[t] = __uint_as_float((t & 1) ? a.z : a.x);
            }
            if (ok)
                break;
            if (wall_clock64() - t0 > kWaitTicks) {
                note_timeout(s.timeouts);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // lanes 0..7 hold the 8 slices; sum within the 8 (exec covers them all)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float sum = sum8(ss[t]);
            if (lane == t)
                st_word(&s.g_ssq[(size_t)x * kDecMaxT + t], tag_f32(sum, gen));
        }
    }
}

// Hop C (wave 1 of workgroup (x, i)): lo for rows 10 i .. 10 i + 9 from the 8
// XCD partials: XCDs 2s and 2s+1 hold stream s, whose rs comes from the two
// XCD sums of squares.  lo = (s0 + s1) + (s2 + s3), stored packed into this
// XCD's copy.  Lane slot sl: XCD sl % 8, row 10 i + sl / 8.
template <int T>
__device__ __forceinline__ void hop_lo(const DecodeScratch& s, int x, int i, uint32_t gen, int lane)
{
    float v[2][T], q[2][T];
    int idx[2], sidx[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int sl = lane + 64 * k;
        const int row = kDecRowsPerWG * i + ((sl >> 3) < kDecRowsPerWG ? (sl >> 3) : 0);
        idx[k] = ((sl & 7) * kRank + row) * kDecMaxT;
        sidx[k] = (sl & 7) * kDecMaxT;
    }
    poll80<T>(s.g_part, idx, gen, lane, v, s.timeouts);
    poll80<T>(s.g_ssq, sidx, gen, lane, q, s.timeouts);
    const uint32_t g16 = gen & 0xffffu;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int sl = lane + 64 * k;
        const int row = kDecRowsPerWG * i + (sl >> 3);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float p = v[k][t] + dpp<0xB1>(v[k][t]);  // the stream's two halves
            const float ss = q[k][t] + dpp<0xB1>(q[k][t]);
            float lo = p * rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
            lo += dpp<0x4E>(lo);   // (s0 + s1), (s2 + s3)
            lo += dpp<0x141>(lo);  // (s0 + s1) + (s2 + s3)
            if ((k == 0 || lane < 16) && (lane & 7) == t) {
                uint32_t h, m, l;
                split3(lo, h, m, l);
                const uint64_t word = (uint64_t)(h | (m << 16)) | ((uint64_t)(l | (g16 << 16)) << 32);
                st_word_xcd(&s.x_lo[((size_t)x * kDecMaxT + t) * kRank + row], word);
            }
        }
    }
}

template <int T>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(
    const float* __restrict__ R, const float* __restrict__ P, const float* __restrict__ w_norm,
    const uint16_t* __restrict__ W_down, const uint16_t* __restrict__ W_up,
    float* __restrict__ out_mixed, uint16_t* __restrict__ out_bf16, uint16_t* __restrict__ out_fp16,
    DecodeScratch s)
{
    static_assert(T >= 1 && T <= kDecMaxT, "short-window kernel takes 1..8 tokens");
    static_assert(40 * kDecMaxT <= 64 * kDecDownWaves, "one staging thread per token float4");
    static_assert(kDecXcds * 8 * kDecSliceCols == kD && 32 * kDecRowsPerWG == kRank, "tiling");
    __shared__ __align__(16) uint16_t ypl[3][T][kYRow];   // y = R' * w_norm, 3 bf16 pieces
    __shared__ float sspart[T][kDecSliceCols / 4];         // per-thread sums of squares
    __shared__ __align__(16) uint16_t lpl[3][T][kLoRow];  // lo, 3 bf16 pieces

    const int b = blockIdx.x;
    const int x = b & 7;       // XCD
    const int i = b >> 3;      // index inside the XCD, 0..31
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // MFMA column slot (B / D operand)
    const int g = lane >> 4;  // MFMA k-group (A / B operand) and D row group
    // this launch's generation: one more than the launches this workgroup has seen
    uint32_t seen = 0;
    if (lane == 0)
        seen = __hip_atomic_load(&s.gen[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t gen = (uint32_t)__builtin_amdgcn_readfirstlane((int)seen) + 1u;
    if (threadIdx.x == 0 && __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) != x)
        note_timeout(s.timeouts);  // not on the XCD the hand-offs assume: results invalid
    HC_PROBE(0, threadIdx.x == 0);

    if (wave < kDecDownWaves) {
        // ======================= down waves =======================
        const int hl = i >> 2;                              // slice inside the XCD
        const int rg = i & 3;                               // 80-row group
        const int kcol = (8 * x + hl) * kDecSliceCols;      // first flattened column (stream x / 2)
        const int rb = kDecDownWaves * rg + wave;           // this wave's 16-row block

        // (1) activations first (loads complete in issue order): one float4 of
        //     one token per thread
        const int at = threadIdx.x / (kDecSliceCols / 4);
        const int af = threadIdx.x % (kDecSliceCols / 4);
        float4 rv = make_float4(0.f, 0.f, 0.f, 0.f), pv = rv, wv = rv;
        if (at < T) {
            rv = reinterpret_cast<const float4*>(R + (size_t)at * kD + kcol)[af];
            if (P)
                pv = reinterpret_cast<const float4*>(P + (size_t)at * kD + kcol)[af];
            wv = reinterpret_cast<const float4*>(w_norm + kcol)[af];
        }
        // (2) this wave's W_down chunks: rows 16*rb + n, 5 blocks of 32 columns
        uint4 wd[5];
        {
            const uint4* src = reinterpret_cast<const uint4*>(
                W_down + (size_t)(16 * rb + n) * kD + kcol + 8 * g);
#pragma unroll
            for (int q = 0; q < 5; ++q)
                wd[q] = src[4 * q];
        }
        // (3) y = R' * w_norm (unscaled: the norm is folded into the reduction),
        //     sums of squares, and the exact 3-way split into LDS
        if (at < T) {
            const float r[4] = {rv.x + pv.x, rv.y + pv.y, rv.z + pv.z, rv.w + pv.w};
            const float w[4] = {wv.x, wv.y, wv.z, wv.w};
            float ss = 0.f;
            uint32_t hi[4], mi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ss += r[e] * r[e];
                split3(r[e] * w[e], hi[e], mi[e], lo[e]);
            }
            sspart[at][af] = ss;
            const int col = 4 * af;
            *reinterpret_cast<uint2*>(&ypl[0][at][col]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
            *reinterpret_cast<uint2*>(&ypl[1][at][col]) = make_uint2(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16));
            *reinterpret_cast<uint2*>(&ypl[2][at][col]) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
        __syncthreads();  // B1: activations staged
        HC_PROBE(1, threadIdx.x == 0);

        // (4) the slice's sums of squares (one workgroup per slice publishes)
        if (rg == 0 && wave == 0 && lane < T) {
            float ss = 0.f;
            for (int f = 0; f < kDecSliceCols / 4; ++f)
                ss += sspart[lane][f];
            st_word_xcd(&s.xs_ssq[((size_t)x * 8 + hl) * kDecMaxT + lane], tag_f32(ss, gen));
        }

        // (5) partial dots on the matrix cores: D[token][row] over the 160 columns
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        {
            const int m = lane & 15;  // A row = token
#pragma unroll
            for (int q = 0; q < 5; ++q) {
                const int col = 32 * q + 8 * g;
                uint4 ah = make_uint4(0, 0, 0, 0), am = ah, al = ah;
                if (m < T) {
                    ah = *reinterpret_cast<const uint4*>(&ypl[0][m][col]);
                    am = *reinterpret_cast<const uint4*>(&ypl[1][m][col]);
                    al = *reinterpret_cast<const uint4*>(&ypl[2][m][col]);
                }
                acc = mfma16(al, wd[q], acc);
                acc = mfma16(am, wd[q], acc);
                acc = mfma16(ah, wd[q], acc);
            }
        }
        HC_PROBE(2, threadIdx.x == 0);
        __syncthreads();  // B1b: this workgroup's W_down chunks have landed
        // D rows = tokens 4g..4g+3 of row 16*rb + n, into the XCD's slice partials
        {
            uint64_t* dst = s.xs_part + (((size_t)x * 8 + hl) * kRank + 16 * rb + n) * kDecMaxT + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e < T)
                    st_word_xcd(dst + e, tag_f32(acc[e], gen));
        }
        // the stores must reach L2 before this wave starts polling: a polling
        // loop of L2 hits can otherwise keep its own earlier stores queued
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        HC_PROBE(3, threadIdx.x == 0);

        // (6) the hops: wave 0 hop B, wave 1 hop C
        if (wave == 0)
            hop_xcd_partial<T>(s, x, i, gen, lane);
        if (wave == 1)
            hop_lo<T>(s, x, i, gen, lane);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        HC_PROBE(5, threadIdx.x == 0);

        // (7) hop D: waves 0, 2, 3, 4 stage lo (this XCD's copy) for rank
        //     indices [80 p, 80 p + 80), two per slot, into LDS
        if (wave != 1) {
            constexpr int NS = (40 * T + 63) / 64;  // slots per lane
            const int part_base = 80 * (wave == 0 ? 0 : wave - 1);
            const uint32_t g16 = gen & 0xffffu;
            const uint64_t* lo_x = s.x_lo + (size_t)x * kDecMaxT * kRank;  // uniform per wave
            uint64_t w0[NS], w1[NS];
            bool done[NS];
#pragma unroll
            for (int r = 0; r < NS; ++r)
                done[r] = lane + 64 * r >= 40 * T;
            const long long t0 = wall_clock64();
            while (true) {
                bool all = true;
#pragma unroll
                for (int r = 0; r < NS; ++r) {
                    const int sl = lane + 64 * r;
                    if (!done[r]) {
                        const uint4 v = ld_words2(lo_x, (sl / 40) * kRank + part_base + 2 * (sl % 40));
                        w0[r] = (uint64_t)v.x | ((uint64_t)v.y << 32);
                        w1[r] = (uint64_t)v.z | ((uint64_t)v.w << 32);
                        done[r] = (v.y >> 16) == g16 && (v.w >> 16) == g16;
                    }
                    all = all && done[r];
                }
                if (__all(all))
                    break;
                if (wall_clock64() - t0 > kWaitTicks) {
                    if (lane == 0)
                        note_timeout(s.timeouts);
                    break;
                }
                __builtin_amdgcn_s_sleep(4);
            }
            HC_PROBE(7, wave == 0 && lane == 0);
#pragma unroll
            for (int r = 0; r < NS; ++r) {
                const int sl = lane + 64 * r;
                if (sl < 40 * T) {
                    const int tt = sl / 40;
                    const int j = part_base + 2 * (sl % 40);
                    const uint32_t a0 = (uint32_t)w0[r], a1 = (uint32_t)w1[r];
                    const uint32_t b0 = (uint32_t)(w0[r] >> 32), b1 = (uint32_t)(w1[r] >> 32);
                    *reinterpret_cast<uint32_t*>(&lpl[0][tt][j]) = (a0 & 0xffffu) | (a1 << 16);
                    *reinterpret_cast<uint32_t*>(&lpl[1][tt][j]) = (a0 >> 16) | (a1 & 0xffff0000u);
                    *reinterpret_cast<uint32_t*>(&lpl[2][tt][j]) = (b0 & 0xffffu) | (b1 << 16);
                }
            }
        }
        __syncthreads();  // B2: lo staged
        if (wave == 0 && lane == 0)
            __hip_atomic_store(&s.gen[b], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // ======================= up waves =======================
        const int u = wave - kDecDownWaves;        // this wave's block of 4 output columns
        const int nblk = b < kUpSplitCols / 12 ? 3 : 2;
        const int c0 = b < kUpSplitCols / 12 ? 12 * b : kUpSplitCols + 8 * (b - kUpSplitCols / 12);
        const bool active = u < nblk;
        const int cc = n >> 2;                     // column inside the 4
        const int st = n & 3;                      // stream
        const int c = c0 + 4 * u + cc;
        const int k = st * kWidth + c;             // W_up row of this MFMA column slot

        __syncthreads();  // B1
        __syncthreads();  // B1b: W_down has landed here; now the up weights
        uint4 wu[10];
        float rp[4] = {0.f, 0.f, 0.f, 0.f};        // R' for the mix: tokens 4g+i, stream st, column c
        if (active) {
            const uint4* src = reinterpret_cast<const uint4*>(W_up + (size_t)k * kRank + 8 * g);
#pragma unroll
            for (int q = 0; q < 10; ++q)
                wu[q] = src[4 * q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = 4 * g + e;
                if (tt < T) {
                    float v = R[(size_t)tt * kD + k];
                    if (P)
                        v += P[(size_t)tt * kD + k];
                    rp[e] = v;
                }
            }
        }
        HC_PROBE(6, wave == kDecDownWaves && lane == 0);
        __syncthreads();  // B2: lo staged
        HC_PROBE(8, wave == kDecDownWaves && lane == 0);
        if (active) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            const int m = lane & 15;  // A row = token
#pragma unroll
            for (int q = 0; q < 10; ++q) {
                const int j = 32 * q + 8 * g;
                uint4 ah = make_uint4(0, 0, 0, 0), am = ah, al = ah;
                if (m < T) {
                    ah = *reinterpret_cast<const uint4*>(&lpl[0][m][j]);
                    am = *reinterpret_cast<const uint4*>(&lpl[1][m][j]);
                    al = *reinterpret_cast<const uint4*>(&lpl[2][m][j]);
                }
                acc = mfma16(al, wu[q], acc);
                acc = mfma16(am, wu[q], acc);
                acc = mfma16(ah, wu[q], acc);
            }
            // gated = up (identity epilogue); mix the 4 streams of column c
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float mixed = sum4(acc[e] * rp[e]);  // (s0 + s1) + (s2 + s3)
                const int tt = 4 * g + e;
                if (st == 0 && tt < T) {
                    const size_t o = (size_t)tt * kWidth + c;
                    out_mixed[o] = mixed;
                    out_bf16[o] = __builtin_bit_cast(uint16_t, (__bf16)mixed);
                    out_fp16[o] = __builtin_bit_cast(uint16_t, (_Float16)mixed);
                }
            }
        }
        HC_PROBE(9, wave == kDecDownWaves && lane == 0);
    }
}

}  // namespace

size_t decode_scratch_bytes()
{
    return sizeof(uint64_t) * ((size_t)kDecXcds * 8 * kRank * kDecMaxT + (size_t)kDecXcds * 8 * kDecMaxT +
                               (size_t)kDecXcds * kRank * kDecMaxT + (size_t)kDecXcds * kDecMaxT +
                               (size_t)kDecXcds * kDecMaxT * kRank) +
           sizeof(uint32_t) * (kDecWGs + 64);
}

void decode_scratch_carve(void* base, DecodeScratch* s)
{
    uint64_t* p = static_cast<uint64_t*>(base);
    s->xs_part = p;
    p += (size_t)kDecXcds * 8 * kRank * kDecMaxT;
    s->xs_ssq = p;
    p += (size_t)kDecXcds * 8 * kDecMaxT;
    s->g_part = p;
    p += (size_t)kDecXcds * kRank * kDecMaxT;
    s->g_ssq = p;
    p += (size_t)kDecXcds * kDecMaxT;
    s->x_lo = p;
    p += (size_t)kDecXcds * kDecMaxT * kRank;
    s->gen = reinterpret_cast<uint32_t*>(p);
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
    void* args[] = {&R, &P, &w_norm, &W_down, &W_up, &out_mixed, &out_bf16, &out_fp16,
                    const_cast<DecodeScratch*>(&s)};
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
