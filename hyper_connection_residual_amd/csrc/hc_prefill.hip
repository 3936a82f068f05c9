// hc_prefill.hip -- the hyper-connection read for wide inputs (T > 8 tokens):
// prefill chunks and long verify windows.
//
// The read is the one of "#315 hc: the multi-token hyper-connection read split
// finer" with the norm folded into the down projection ("#2488 sycl/A770",
// Summary item 4) and the up projection fused with gr_mix_r as in "#1370
// prefill: ... gr_mix_r as its epilogue", "What it does": gated (T x 10240
// fp32) never leaves registers and LDS.  Three launches per chunk of up to
// 4096 tokens:
//
//   P1 down:  part[sig][t][j] = sum_{k in split sig} W_down[j][k] * (R'[t][k] *
//             w_norm[k]) and ssq[sig][t] = sum_{k in sig} R'[t][k]^2, where a
//             split is one stream (or half of one).  Tile: 64 tokens x 320 rows,
//             K streamed 32 columns at a time through double-buffered LDS.
//   P2 lo:    rs[t][s] = 1/sqrt(sum_{sig in s} ssq / 2560 + eps) and lo[t][j] =
//             sum_s rs[t][s] * sum_{sig in s} part[sig][t][j], stored as three
//             bf16 planes (an exact split of the fp32 value).
//   P3 up+mix: a tile of 128 tokens x 32 output columns x 4 streams: the up
//             projection (K = 320) on the matrix cores, then the mix of the 4
//             streams with R' and the bf16 / fp16 images, written coalesced
//             after a transpose through LDS.
//
// gfx950 choices: bf16 v_mfma_f32_16x16x32_bf16 with every fp32 activation
// split exactly into three bf16 pieces (so products are exact and results stay
// fp32-faithful); workgroups sharing a W_down slice (P1) or a token tile (P3)
// are dealt to the same XCD so the shared operand is served from that XCD's
// L2; the chunk size keeps a chunk's R (+ pending) within the 256 MB Infinity
// Cache for its second read in P3.
#include "hc_internal.h"

#pragma clang fp contract(off)

namespace hc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c)
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum4(float v)
{
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    return v;
}

constexpr int kP1Tok = 64;               // P1 token tile
constexpr int kP1Row = 32 + 8;           // padded LDS row (bf16) of a 32-column step
constexpr int kP3Tok = 128;              // P3 token tile
constexpr int kP3Cols = 32;              // P3 output columns per tile
constexpr int kP3ColTiles = kWidth / kP3Cols;  // 80

// ---------------------------------------------------------------------------
// P1: down projection partials and sums of squares.
// ---------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(256) void prefill_down(int T, const float* __restrict__ R,
                                                    const float* __restrict__ P,
                                                    const float* __restrict__ w_norm,
                                                    const uint16_t* __restrict__ W_down,
                                                    float* __restrict__ part, float* __restrict__ ssq)
{
    constexpr int KW = kWidth / S;  // columns of one split
    constexpr int KSTEPS = KW / 32;
    __shared__ __align__(16) uint16_t ypl[2][3][kP1Tok][kP1Row];

    const int bid = blockIdx.x;
    const int x = bid & 7;  // XCD: every workgroup of one split on one or two XCDs
    int sig, tile;
    if (S == 2) {
        sig = x;
        tile = bid >> 3;
    } else {
        sig = x & 3;
        tile = (bid >> 3) * 2 + (x >> 2);
    }
    const int t0 = tile * kP1Tok;
    if (t0 >= T)
        return;
    const int kbase = (sig / S) * kWidth + (sig % S) * KW;  // first flattened column

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    // staging role: token row r, 8 columns c8
    const int r = tid >> 2, c8 = (tid & 3) * 8;
    const int tr = t0 + r;
    const bool row_ok = tr < T;

    float ssacc = 0.f;
    float4 sr0, sr1, sp0, sp1, sw0, sw1;
    auto load_stage = [&](int ks) {
        const int k = kbase + ks * 32 + c8;
        sw0 = *reinterpret_cast<const float4*>(w_norm + k);
        sw1 = *reinterpret_cast<const float4*>(w_norm + k + 4);
        if (row_ok) {
            sr0 = *reinterpret_cast<const float4*>(R + (size_t)tr * kD + k);
            sr1 = *reinterpret_cast<const float4*>(R + (size_t)tr * kD + k + 4);
            if (P) {
                sp0 = *reinterpret_cast<const float4*>(P + (size_t)tr * kD + k);
                sp1 = *reinterpret_cast<const float4*>(P + (size_t)tr * kD + k + 4);
            }
        }
    };
    auto store_stage = [&](int buf) {
        uint32_t hi[8], mi[8], lo[8];
        if (row_ok) {
            float v[8] = {sr0.x, sr0.y, sr0.z, sr0.w, sr1.x, sr1.y, sr1.z, sr1.w};
            if (P) {
                v[0] += sp0.x; v[1] += sp0.y; v[2] += sp0.z; v[3] += sp0.w;
                v[4] += sp1.x; v[5] += sp1.y; v[6] += sp1.z; v[7] += sp1.w;
            }
            const float w[8] = {sw0.x, sw0.y, sw0.z, sw0.w, sw1.x, sw1.y, sw1.z, sw1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ssacc += v[e] * v[e];
                split3(v[e] * w[e], hi[e], mi[e], lo[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hi[e] = mi[e] = lo[e] = 0;
        }
        *reinterpret_cast<uint4*>(&ypl[buf][0][r][c8]) =
            make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
        *reinterpret_cast<uint4*>(&ypl[buf][1][r][c8]) =
            make_uint4(mi[0] | (mi[1] << 16), mi[2] | (mi[3] << 16), mi[4] | (mi[5] << 16), mi[6] | (mi[7] << 16));
        *reinterpret_cast<uint4*>(&ypl[buf][2][r][c8]) =
            make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
    };
    // this wave's rows: 16 * (5 wave + nb) + n
    const uint16_t* wrow[5];
#pragma unroll
    for (int nb = 0; nb < 5; ++nb)
        wrow[nb] = W_down + (size_t)(16 * (5 * wave + nb) + n) * kD + kbase + 8 * g;
    uint4 wb[5], wn[5];
    auto load_b = [&](int ks, uint4 (&dst)[5]) {
#pragma unroll
        for (int nb = 0; nb < 5; ++nb)
            dst[nb] = *reinterpret_cast<const uint4*>(wrow[nb] + ks * 32);
    };

    f32x4_t acc[4][5];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 5; ++nb)
            acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_stage(0);
    load_b(0, wb);
    store_stage(0);
    __syncthreads();
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int buf = ks & 1;
        const bool more = ks + 1 < KSTEPS;
        if (more) {
            load_stage(ks + 1);
            load_b(ks + 1, wn);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int m = 16 * mb + (lane & 15);
            const uint4 ah = *reinterpret_cast<const uint4*>(&ypl[buf][0][m][8 * g]);
            const uint4 am = *reinterpret_cast<const uint4*>(&ypl[buf][1][m][8 * g]);
            const uint4 al = *reinterpret_cast<const uint4*>(&ypl[buf][2][m][8 * g]);
#pragma unroll
            for (int nb = 0; nb < 5; ++nb) {
                acc[mb][nb] = mfma16(al, wb[nb], acc[mb][nb]);
                acc[mb][nb] = mfma16(am, wb[nb], acc[mb][nb]);
                acc[mb][nb] = mfma16(ah, wb[nb], acc[mb][nb]);
            }
        }
        if (more) {
            store_stage(buf ^ 1);
#pragma unroll
            for (int nb = 0; nb < 5; ++nb)
                wb[nb] = wn[nb];
        }
        __syncthreads();
    }

    // partials: D rows = tokens 16 mb + 4 g + i, columns = rows of W_down
    float* pdst = part + (size_t)sig * T * kRank;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * mb + 4 * g + i;
            if (t < T)
#pragma unroll
                for (int nb = 0; nb < 5; ++nb)
                    pdst[(size_t)t * kRank + 16 * (5 * wave + nb) + n] = acc[mb][nb][i];
        }
    // sums of squares: the 4 staging threads of a token row are one quad
    const float ss = sum4(ssacc);
    if ((tid & 3) == 0 && row_ok)
        ssq[(size_t)sig * T + tr] = ss;
}

// ---------------------------------------------------------------------------
// P2: lo = sum_s rs_s * stream partial, as three bf16 planes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_lo(int T, int S, const float* __restrict__ part,
                                                  const float* __restrict__ ssq,
                                                  uint16_t* __restrict__ planes)
{
    const int idx = blockIdx.x * 256 + threadIdx.x;  // (token, pair of rank indices)
    const int t = idx / (kRank / 2);
    if (t >= T)
        return;
    const int j = 2 * (idx % (kRank / 2));
    float v0[4], v1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float ss = 0.f, p0 = 0.f, p1 = 0.f;
        for (int q = 0; q < S; ++q) {
            const int sig = s * S + q;
            ss += ssq[(size_t)sig * T + t];
            const float2 pv = *reinterpret_cast<const float2*>(part + ((size_t)sig * T + t) * kRank + j);
            p0 += pv.x;
            p1 += pv.y;
        }
        const float rs = rsqrtf(ss * (1.0f / (float)kWidth) + kEps);
        v0[s] = p0 * rs;
        v1[s] = p1 * rs;
    }
    const float lo0 = (v0[0] + v0[1]) + (v0[2] + v0[3]);
    const float lo1 = (v1[0] + v1[1]) + (v1[2] + v1[3]);
    uint32_t h0, m0, l0, h1, m1, l1;
    split3(lo0, h0, m0, l0);
    split3(lo1, h1, m1, l1);
    const size_t o = (size_t)t * kRank + j;
    const size_t plane = (size_t)T * kRank;
    *reinterpret_cast<uint32_t*>(planes + o) = h0 | (h1 << 16);
    *reinterpret_cast<uint32_t*>(planes + plane + o) = m0 | (m1 << 16);
    *reinterpret_cast<uint32_t*>(planes + 2 * plane + o) = l0 | (l1 << 16);
}

// ---------------------------------------------------------------------------
// P3: up projection with the stream mix as its epilogue.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_upmix(int T, const uint16_t* __restrict__ planes,
                                                     const uint16_t* __restrict__ W_up,
                                                     const float* __restrict__ R,
                                                     const float* __restrict__ P,
                                                     float* __restrict__ out_mixed,
                                                     uint16_t* __restrict__ out_bf16,
                                                     uint16_t* __restrict__ out_fp16)
{
    __shared__ __align__(16) float upt[kP3Tok][4][kP3Cols + 4];  // up, transposed for the mix

    const int bid = blockIdx.x;
    const int x = bid & 7, jj = bid >> 3;  // a token tile's workgroups share an XCD
    const int tile = x + 8 * (jj / kP3ColTiles);
    const int t0 = tile * kP3Tok;
    if (t0 >= T)
        return;
    const int c0 = (jj % kP3ColTiles) * kP3Cols;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const size_t plane = (size_t)T * kRank;

    // A rows: tokens t0 + 32 wave + 16 mb + (lane & 15)
    const uint16_t* arow[2];
    bool aok[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int t = t0 + 32 * wave + 16 * mb + (lane & 15);
        aok[mb] = t < T;
        arow[mb] = planes + (size_t)(aok[mb] ? t : 0) * kRank + 8 * g;
    }
    // B rows: MFMA column slot n of block nb = column c0 + 4 nb + n / 4, stream n % 4
    const uint16_t* brow[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
        brow[nb] = W_up + (size_t)((n & 3) * kWidth + c0 + 4 * nb + (n >> 2)) * kRank + 8 * g;

    uint4 a[2][3], an[2][3], b[8], bn[8];
    auto load_ab = [&](int q, uint4 (&ad)[2][3], uint4 (&bd)[8]) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                ad[mb][p] = aok[mb] ? *reinterpret_cast<const uint4*>(arow[mb] + p * plane + 32 * q)
                                    : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
            bd[nb] = *reinterpret_cast<const uint4*>(brow[nb] + 32 * q);
    };

    f32x4_t acc[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
            acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_ab(0, a, b);
#pragma unroll 1
    for (int q = 0; q < kRank / 32; ++q) {
        const bool more = q + 1 < kRank / 32;
        if (more)
            load_ab(q + 1, an, bn);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                acc[mb][nb] = mfma16(a[mb][2], b[nb], acc[mb][nb]);
                acc[mb][nb] = mfma16(a[mb][1], b[nb], acc[mb][nb]);
                acc[mb][nb] = mfma16(a[mb][0], b[nb], acc[mb][nb]);
            }
        if (more) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    a[mb][p] = an[mb][p];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
                b[nb] = bn[nb];
        }
    }

    // gated = up (identity epilogue): transpose through LDS as [token][stream][column]
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                upt[32 * wave + 16 * mb + 4 * g + i][n & 3][4 * nb + (n >> 2)] = acc[mb][nb][i];
    __syncthreads();

    // mix: each item = one token and 4 consecutive columns
#pragma unroll
    for (int it = 0; it < kP3Tok * (kP3Cols / 4) / 256; ++it) {
        const int item = tid + 256 * it;
        const int tl = item / (kP3Cols / 4);
        const int cg = 4 * (item % (kP3Cols / 4));
        const int t = t0 + tl;
        if (t >= T)
            continue;
        const int c = c0 + cg;
        float4 m[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float4 rv = *reinterpret_cast<const float4*>(R + (size_t)t * kD + s * kWidth + c);
            if (P) {
                const float4 pv = *reinterpret_cast<const float4*>(P + (size_t)t * kD + s * kWidth + c);
                rv.x += pv.x;
                rv.y += pv.y;
                rv.z += pv.z;
                rv.w += pv.w;
            }
            const float4 u = *reinterpret_cast<const float4*>(&upt[tl][s][cg]);
            m[s] = make_float4(u.x * rv.x, u.y * rv.y, u.z * rv.z, u.w * rv.w);
        }
        const float4 mixed = make_float4((m[0].x + m[1].x) + (m[2].x + m[3].x),
                                         (m[0].y + m[1].y) + (m[2].y + m[3].y),
                                         (m[0].z + m[1].z) + (m[2].z + m[3].z),
                                         (m[0].w + m[1].w) + (m[2].w + m[3].w));
        const size_t o = (size_t)t * kWidth + c;
        *reinterpret_cast<float4*>(out_mixed + o) = mixed;
        const uint16_t b0 = __builtin_bit_cast(uint16_t, (__bf16)mixed.x);
        const uint16_t b1 = __builtin_bit_cast(uint16_t, (__bf16)mixed.y);
        const uint16_t b2 = __builtin_bit_cast(uint16_t, (__bf16)mixed.z);
        const uint16_t b3 = __builtin_bit_cast(uint16_t, (__bf16)mixed.w);
        *reinterpret_cast<uint2*>(out_bf16 + o) = make_uint2(b0 | ((uint32_t)b1 << 16), b2 | ((uint32_t)b3 << 16));
        const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)mixed.x);
        const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)mixed.y);
        const uint16_t h2 = __builtin_bit_cast(uint16_t, (_Float16)mixed.z);
        const uint16_t h3 = __builtin_bit_cast(uint16_t, (_Float16)mixed.w);
        *reinterpret_cast<uint2*>(out_fp16 + o) = make_uint2(h0 | ((uint32_t)h1 << 16), h2 | ((uint32_t)h3 << 16));
    }
}

}  // namespace

size_t prefill_scratch_bytes(int chunk)
{
    // S = 2 at most: 8 splits of partials and sums of squares, 3 lo planes
    return sizeof(float) * ((size_t)8 * chunk * kRank + (size_t)8 * chunk) +
           sizeof(uint16_t) * (size_t)3 * chunk * kRank + 256;
}

hipError_t launch_prefill(int64_t T, const float* R, const float* P, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, void* scratch, int chunk,
                          hipStream_t stream)
{
    float* part = static_cast<float*>(scratch);
    float* ssq = part + (size_t)8 * chunk * kRank;
    uint16_t* planes = reinterpret_cast<uint16_t*>(ssq + (size_t)8 * chunk);
    for (int64_t c0 = 0; c0 < T; c0 += chunk) {
        const int Tc = (int)(T - c0 < chunk ? T - c0 : chunk);
        const size_t in_off = (size_t)c0 * kD, out_off = (size_t)c0 * kWidth;
        const float* Rc = R + in_off;
        const float* Pc = P ? P + in_off : nullptr;
        const int tiles1 = (Tc + kP1Tok - 1) / kP1Tok;
        // one split per stream when that already fills the chip, else two
        const int S = tiles1 * 4 >= 256 ? 1 : 2;
        if (S == 1) {
            const int grid = 8 * ((tiles1 + 1) / 2);
            hipLaunchKernelGGL(prefill_down<1>, dim3(grid), dim3(256), 0, stream, Tc, Rc, Pc, w_norm,
                               W_down, part, ssq);
        } else {
            hipLaunchKernelGGL(prefill_down<2>, dim3(8 * tiles1), dim3(256), 0, stream, Tc, Rc, Pc,
                               w_norm, W_down, part, ssq);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int items = Tc * (kRank / 2);
        hipLaunchKernelGGL(prefill_lo, dim3((items + 255) / 256), dim3(256), 0, stream, Tc, S, part, ssq,
                           planes);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int tiles3 = (Tc + kP3Tok - 1) / kP3Tok;
        const int grid3 = 8 * kP3ColTiles * ((tiles3 + 7) / 8);
        hipLaunchKernelGGL(prefill_upmix, dim3(grid3), dim3(256), 0, stream, Tc, planes, W_up, Rc, Pc,
                           out_mixed + out_off, out_bf16 + out_off, out_fp16 + out_off);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace hc
