// hc_internal.h -- shapes, scratch layout and launcher declarations shared by
// the host library (hc_api.hip) and the HIP kernels.  Library-internal.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace hc {

constexpr int kStreams = 4;
constexpr int kWidth = 2560;
constexpr int kD = kStreams * kWidth;  // 10240: the flattened stream axis, k = s*2560 + c
constexpr int kRank = 320;
constexpr float kEps = 1e-6f;

// ---------------------------------------------------------------------------
// Short-window path (T <= kDecMaxT): one launch of kDecWGs workgroups, one
// per CU, each of 8 waves.  Workgroup b runs on XCD x = b % 8 (the dispatcher
// deals workgroups to the 8 XCDs round robin; the kernel checks it).  XCD x
// owns columns [1280 x, 1280 x + 1280) of W_down (half of stream x / 2) and
// output columns chosen per workgroup.
//   down waves 0-4:  workgroup (x, i = b / 8) computes slice hl = i / 4
//     (160 columns) for rows 80 (i % 4) .. +79, 16 rows per wave;
//   hop B (inside the XCD, through its L2): wave 0 of workgroup (x, i) sums
//     the XCD's 8 slices for rows 10 i .. 10 i + 9 and publishes that XCD
//     partial to device memory;
//   hop C (across XCDs): wave 1 of workgroup (x, i) gathers the 8 XCD
//     partials of rows 10 i .. 10 i + 9, applies each stream's rs and forms
//     lo for those rows -- every XCD computes all of lo itself;
//   hop D (inside the XCD): waves 0, 2, 3, 4 stage all of lo into LDS;
//   up waves 5-7: W_up rows of 12 (workgroups 0..127) or 8 output columns,
//     all 4 streams, then the stream mix.
// Hand-off words are 64 bits: payload plus the launch's generation number,
// written once with one store and polled by the consumer.
// ---------------------------------------------------------------------------
constexpr int kDecMaxT = 8;
constexpr int kDecWGs = 256;
constexpr int kDecThreads = 512;
constexpr int kDecDownWaves = 5;
constexpr int kDecXcds = 8;
constexpr int kDecSliceCols = 160;  // 8 slices per XCD, 64 in all
constexpr int kDecRowsPerWG = 10;   // rows of lo each workgroup reduces (32 x 10 = 320)

struct DecodeScratch {
    uint64_t* xs_part;   // [8 xcd][8 slice][kRank][kDecMaxT]: slice partials (XCD-local)
    uint64_t* xs_ssq;    // [8 xcd][8 slice][kDecMaxT]: slice sums of squares (XCD-local)
    uint64_t* g_part;    // [8 xcd][kRank][kDecMaxT]: XCD partials (device-wide)
    uint64_t* g_ssq;     // [8 xcd][kDecMaxT]: XCD sums of squares (device-wide)
    uint64_t* x_lo;      // [8 xcd][kDecMaxT][kRank]: lo, bf16 hi | mid << 16 | lo3 << 32 | (gen & 0xffff) << 48 (XCD-local)
    uint32_t* gen;       // [kDecWGs]: launches completed by each workgroup
    uint32_t* timeouts;  // [1]: expired bounded waits and misplaced workgroups
};

size_t decode_scratch_bytes();
void decode_scratch_carve(void* base, DecodeScratch* s);

// Workgroups of the short-window kernel that fit on one CU at once.
hipError_t decode_resident_blocks(int* blocks_per_cu);

hipError_t launch_decode(int T, const float* R, const float* P, const float* w_norm,
                         const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                         uint16_t* out_bf16, uint16_t* out_fp16, const DecodeScratch& s,
                         hipStream_t stream);

// ---------------------------------------------------------------------------
// Wide path (T > kDecMaxT): three launches per chunk of up to kPrefillChunk
// tokens (down partials, lo planes, up projection with the mix epilogue).
// ---------------------------------------------------------------------------
constexpr int kPrefillChunk = 4096;

size_t prefill_scratch_bytes(int chunk);

hipError_t launch_prefill(int64_t T, const float* R, const float* P, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, void* scratch, int chunk,
                          hipStream_t stream);

}  // namespace hc
