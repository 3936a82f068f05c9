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
// per CU, each of 8 waves.  Workgroup b belongs to group x = b % 8, i = b / 8;
// the dispatcher deals workgroups to the 8 XCDs round robin, so the 32
// workgroups of a group share one XCD and its L2 (the kernel checks it).
// Every workgroup takes two tiles of 25.6 KB, loaded in this order:
//   down: W_down rows [40 x, 40 x + 40) x columns [320 i, 320 i + 320)
//     (inside stream i / 8); its partial dots and the slice's sum of squares
//     go into the XCD's L2;
//   up: the W_up rows of output columns [10 (32 x + i), +10), all 4 streams.
// Workgroups i < 14 of each group then reduce 3 of its 40 rows over the 32
// partials (hop 1, inside the XCD) and publish lo device-wide; every
// workgroup gathers all of lo (hop 2), runs the up projection and the mix.
// Weight tiles are loaded straight into LDS as whole cache lines.  Hand-off
// words are 64 bits: payload plus a tag, written once with one store and
// polled by the consumer.
// ---------------------------------------------------------------------------
constexpr int kDecMaxT = 32;
// hc_read and its variants run the short-window kernel up to this many
// tokens and the wide path above: from 26 tokens the wide path is the faster
// one (measured back to back at 26 / 28 / 30 / 32 tokens: 14.8 / 15.0 /
// 15.0 / 15.2 us against 15.2 / 15.6 / 16.0 / 16.1 us; at 25 they tie).
// The kernel itself takes up to kDecMaxT (hc_read_noalloc and the start-up
// check run it up to 32).
constexpr int kShortReadMaxT = 25;
constexpr int kDecWGs = 256;
constexpr int kDecThreads = 512;
constexpr int kDecXcds = 8;
constexpr int kDecWgPerXcd = kDecWGs / kDecXcds;                 // 32 workgroups per XCD
constexpr int kDecRowsPerXcd = kRank / kDecXcds;                 // 40 lo rows per XCD
constexpr int kDecDownCols = kD / kDecWgPerXcd;                  // 320 W_down columns per workgroup
constexpr int kDecUpCols = kWidth / kDecWGs;                     // 10 output columns per workgroup
constexpr int kDecRedRows = 3;                                   // lo rows each reducing workgroup reduces
constexpr int kDecReducers = (kDecRowsPerXcd + kDecRedRows - 1) / kDecRedRows;  // 14 per XCD

struct DecodeScratch {
    uint64_t* part;      // [8 xcd][32 wg][40 rows][8 or 16 token slots]: partial dots (XCD-local)
    uint64_t* ssq;       // [8 xcd][32 wg][16]: column-slice sums of squares (XCD-local)
    uint64_t* lo;        // [kDecMaxT][kRank]: lo (device-wide)
    uint32_t* gen;       // [kDecWGs]: launches completed by each workgroup
    uint32_t* timeouts;  // [1]: expired bounded waits (a workgroup off its group's XCD expires one)
};

size_t decode_scratch_bytes();
void decode_scratch_carve(void* base, DecodeScratch* s);

// Allocation-free reads: set-up (once per device, with that device current,
// outside graph capture) takes the device's address of a file-scope device
// array holding one short-window workspace and clears it on `stream`;
// noalloc_scratch then carves that workspace (false before set-up).
hipError_t noalloc_setup(int dev, hipStream_t stream);
bool noalloc_scratch(int dev, DecodeScratch* s);

// Workgroups of the short-window kernel that fit on one CU at once.
hipError_t decode_resident_blocks(int* blocks_per_cu);

// Every bounded wait of the short-window kernel gives up after this many ticks
// of the 100 MHz wall clock (50 ms), counts one expired wait and goes on.
constexpr long long kDecWaitTicks = 5000000;

// R_commit: NULL, or R itself, which then receives R' = R + P (with P given).
// wait_ticks: the bounded waits' limit (kDecWaitTicks; the start-up check may
// pass a smaller one).
hipError_t launch_decode(int T, const float* R, const float* P, const float* w_norm,
                         const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                         uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit,
                         const DecodeScratch& s, hipStream_t stream, long long wait_ticks = kDecWaitTicks);

// ---------------------------------------------------------------------------
// Wide path (T > kDecMaxT): three launches per chunk of up to kPrefillChunk
// tokens (down partials, lo planes, up projection with the mix epilogue).
// ---------------------------------------------------------------------------
constexpr int kPrefillChunk = 8192;

size_t prefill_scratch_bytes(int chunk);

// bf16_lo: the up projection takes lo rounded to bf16 (hc_read_bf16_lo).
hipError_t launch_prefill(int64_t T, const float* R, const float* P, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit, bool bf16_lo,
                          void* scratch, int chunk, hipStream_t stream);

// ---------------------------------------------------------------------------
// Measurement reference: one launch of the short-window kernel's shape that
// streams `bytes` (a multiple of 16, at least 16) from src into LDS and writes
// one word per workgroup to sink[256].
// ---------------------------------------------------------------------------
hipError_t launch_stream(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace hc
