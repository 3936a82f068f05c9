/*
 * hc.h -- C ABI of the hyper-connection read on AMD Instinct MI355X (gfx950).
 *
 * The read, per token t (the pages: "#315 hc: the multi-token hyper-connection
 * read split finer", "What changes" and "Exactness"; "#1370 prefill: opt-in
 * STRATA_HC_UPMIX=1 on CUDA", "Why" and "What it does"; "#2226
 * STRATA_HC_PERSIST=1", Summary; "#2488 sycl/A770", Summary items 1-5):
 *
 *   R'[t,s,c]  = fl32(R[t,s,c] + pending[t,s,c])      (pending may be absent)
 *   rs[t,s]    = 1 / sqrt(mean_c R'[t,s,c]^2 + eps)    per token and stream
 *   xn[t,k]    = R'[t,s,c] * w_norm[s,c] * rs[t,s]     k = s*2560 + c
 *   lo[t,j]    = sum_k W_down[j,k] * xn[t,k]           down 10240 -> 320
 *   up[t,k]    = sum_j W_up[k,j] * lo[t,j]             up 320 -> 10240
 *   gated      = up                                    (identity epilogue)
 *   mixed[t,c] = sum_{s<4} gated[t, s*2560+c] * R'[t,s,c]
 *   out_bf16, out_fp16 = round-to-nearest-even images of the fp32 mixed
 *
 * with 4 streams, width 2560, rank 320 and eps = 1e-6.  Accumulation is fp32
 * (the GPU keeps every activation fp32-exact: bf16 matrix-core products use an
 * exact three-way bf16 split of each fp32 activation); results agree with the
 * exact value to about 1e-7 of max|mixed| and are bitwise reproducible run to
 * run on the same device.
 *
 * Memory: every pointer argument is a DEVICE pointer (hipMalloc memory or any
 * device-accessible allocation), row-major, contiguous, 16-byte aligned.  The
 * caller owns all of them; hc_read and hc_read_bf16_lo only read R,
 * pending, w_norm, W_down and W_up and only write the three outputs
 * (hc_read_commit also writes R).  Outputs must not overlap any input or
 * each other.
 *
 * Execution: asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream).  No host synchronization; results are visible to later work on the
 * same stream.  The library keeps a scratch workspace per (device, stream):
 * 3.7 MB for the short-window kernel, allocated on the first call on that
 * stream, and a fixed 95 MB for the wide path, allocated on the stream's
 * first wide read; later calls allocate nothing.  Workspaces are found by
 * the stream's handle value: call hc_release_stream before destroying a
 * stream that ran reads (otherwise its workspace lives until hc_release, and
 * a later stream that HIP gives the same handle takes it over, which is safe
 * once the old stream's work has finished).  Calls on different streams never
 * share scratch.  Calls on ONE stream are ordered by the stream and are safe.
 * Short-window reads (hc_read and its variants up to 25 tokens, hc_read_noalloc
 * up to 32) use every CU of the device and must not run at
 * the same time: the library orders them across streams.  A short-window
 * read on another stream than the device's last one waits for that last
 * read: through an event recorded right after it if there is one, else by
 * synchronizing the device.  Events are recorded only while streams
 * alternate: a switch of stream turns recording on (+3.5 us per read), and 64
 * reads in a row on one stream turn it off again.  The library never calls
 * HIP on a stream other than the one a call passes.  Under graph capture the
 * library does not order: the caller orders the replays of a graph.
 *
 * Errors: argument checks (T < 1, a null required pointer, misalignment, a
 * device that is not gfx950) happen before anything is enqueued and leave the
 * outputs untouched.  A failed kernel launch returns
 * HC_ERR_LAUNCH (hc_last_hip_error() gives the hipError_t).  Device faults
 * surface at the caller's next synchronization, as in HIP.  The single-launch
 * short-window kernel waits on data from other workgroups with a bounded wait
 * (50 ms).  If such a wait ever expires (the workgroups could not all be
 * resident at once, e.g. another process or a long kernel on another stream
 * held CUs), the read cannot produce its result; the call has already
 * returned, so the kernel marks it in the outputs instead: every output value
 * the affected workgroups own (all of them, once a reducer's wait expired) is
 * stored as NaN, in out_mixed and in both images, hc_read_commit leaves those
 * workgroups' part of R uncommitted, and hc_timeouts() counts the expired
 * waits.  Outputs are therefore either the read's result or NaN, never silently
 * wrong.  HC_WAIT_TICKS (ticks of the 100 MHz clock) lowers that limit for
 * ordinary reads (0: every wait gives up at its first miss), which tests use
 * to force the case.
 */
#ifndef HC_H
#define HC_H

#include <stdint.h>

#if defined(__GNUC__)
#define HC_API __attribute__((visibility("default")))
#else
#define HC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by hc_read and the other calls. */
#define HC_OK 0
#define HC_ERR_ARG 1     /* T < 1, or a required pointer is NULL */
#define HC_ERR_ALIGN 2   /* a pointer is not 16-byte aligned */
#define HC_ERR_DEVICE 3  /* the current device is not gfx950, or a HIP query failed */
#define HC_ERR_NOMEM 4   /* the scratch workspace could not be allocated */
#define HC_ERR_LAUNCH 5  /* a kernel launch failed (see hc_last_hip_error) */
#define HC_ERR_SIZE 6    /* T above 32 for hc_read_noalloc */
#define HC_ERR_STATE 7   /* hc_read_noalloc before its set-up on the device */

/* Dimensions of the read. */
#define HC_STREAMS 4
#define HC_WIDTH 2560
#define HC_RANK 320

/*
 * hc_read -- one hyper-connection read of T tokens.
 *
 *   T          number of tokens, >= 1
 *   R          const float  [T][4][2560]   residual streams
 *   pending    const float  [T][4][2560]   pending write added to R first, or
 *              NULL for none (the norm and the mix both see R' = R + pending)
 *   w_norm     const float  [4][2560]      RMS-norm weights
 *   W_down     const uint16_t [320][10240] bf16 bit patterns
 *   W_up       const uint16_t [10240][320] bf16 bit patterns
 *   out_mixed  float    [T][2560]          mixed output (fp32)
 *   out_bf16   uint16_t [T][2560]          bf16 bits, RNE of out_mixed
 *   out_fp16   uint16_t [T][2560]          IEEE binary16 bits, RNE of out_mixed
 *              (subnormals kept, overflow to +-inf)
 *   stream     hipStream_t to run on (NULL = default stream)
 *
 * T <= 25 runs one launch of the short-window (verify-window) kernel; larger
 * T runs the wide (prefill) path, which is the faster one from 26 tokens.  The short-window kernel is
 * used only where its start-up check passed (see hc_short_window_on);
 * elsewhere every T runs the wide path.  Every valid T is handled; there is no
 * fallback to return.
 * The first call on a device runs that check (a few milliseconds, with
 * synchronisation), and the first call on each stream allocates its
 * workspace: neither may be under graph capture.
 * Returns HC_OK or an HC_ERR_* code.
 */
HC_API int hc_read(int64_t T, const float* R, const float* pending, const float* w_norm,
            const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
            uint16_t* out_bf16, uint16_t* out_fp16, void* stream);

/*
 * hc_read_commit -- hc_read, and the pending write committed: R[t][s][c]
 * becomes R'[t][s][c] = fl32(R + pending), the pending-updated residual the
 * read itself applies first ("#2488 sycl/A770: faster hyper-connection read",
 * Summary item 4; "#315 hc: the multi-token hyper-connection read split
 * finer", Exactness: reads with and without the pending write).  The pages
 * only apply the pending write inside the read; writing it back is this
 * library's extension, so that the engine needs no separate residual update.
 *
 * Arguments as for hc_read, except that R is read and then overwritten in
 * place (caller-owned, [T][4][2560] fp32).  The outputs are the ones hc_read
 * gives for the same inputs, bit for bit.  With pending == NULL there is
 * nothing to commit and R is left untouched.  R must not overlap pending,
 * w_norm, the weights or the outputs.  If the call returns an error, R may
 * hold a mix of old and committed values.
 * Returns HC_OK or an HC_ERR_* code.
 */
HC_API int hc_read_commit(int64_t T, float* R, const float* pending, const float* w_norm,
                   const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                   uint16_t* out_bf16, uint16_t* out_fp16, void* stream);

/*
 * hc_read_bf16_lo -- hc_read with the pages' prefill numerics on the wide
 * path: the up projection takes lo rounded to bf16 (nearest even) and runs
 * one bf16 matrix product with fp32 accumulation, as the fused up + mix of
 * "#1370 prefill: opt-in STRATA_HC_UPMIX=1 on CUDA", What it does (BF16 mma
 * with FP32 accumulation), instead of the exact three-piece split of lo.  The
 * norm, the down projection and lo itself are unchanged, and windows of up to
 * 25 tokens (the short-window kernel) give hc_read's result.
 * Its contract is an error bound, not hc_read's 2e-6: every mixed value is
 * within 2^-8 * sum_s |R'[t][s][c]| * sum_j |W_up[s*2560+c][j]| * |lo[t][j]|
 * of the exact read (the bf16 rounding of each lo value), plus hc_read's
 * fp32 budget.  Arguments, layouts and errors as for hc_read.
 */
HC_API int hc_read_bf16_lo(int64_t T, const float* R, const float* pending, const float* w_norm,
                    const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                    uint16_t* out_bf16, uint16_t* out_fp16, void* stream);

/*
 * hc_read_noalloc -- hc_read for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It never calls hipMalloc, hipFree or any other allocating
 * routine: the hand-off scratch of the short-window kernel lives in a
 * file-scope device array of 3.7 MB that each GPU the library runs on holds
 * until the process ends, and every allocation-free read of a device shares
 * it.  Arguments and layouts are hc_read's; the caller still passes inputs
 * and outputs.  Up to 25 tokens the results are hc_read's bits (the same
 * kernel); from 26 to 32 tokens it runs the short-window kernel where hc_read
 * takes the wide path, and the two agree within hc_read's 2e-6.
 *
 * Limit: T <= 32 (one short-window launch); a larger T returns HC_ERR_SIZE
 * and enqueues nothing.  Set-up: the device's start-up check (the first
 * hc_short_window_on or read on the device, outside graph capture) takes the
 * array's address, clears it and creates the ordering event; before that, or
 * where the check turned the short-window kernel off, the call returns
 * HC_ERR_STATE.  Allocation-free reads are ordered across streams like
 * short-window reads; replays of captured graphs that hold them must not
 * overlap on one GPU (they would race on the shared array).  The array keeps
 * the last call's contents.  Errors as for hc_read, plus HC_ERR_SIZE and
 * HC_ERR_STATE; expired waits are counted by hc_timeouts on any stream.
 */
HC_API int hc_read_noalloc(int64_t T, const float* R, const float* pending, const float* w_norm,
                           const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                           uint16_t* out_bf16, uint16_t* out_fp16, void* stream);

/*
 * hc_short_window_on -- *on = 1 if the current device reads short windows
 * with the short-window kernel (hc_read up to 25 tokens, hc_read_noalloc up
 * to 32), 0 if every read takes the wide path.  The
 * kernel's hand-offs need its 256 workgroups resident together and placed on
 * the XCDs the way it expects; once per device (on the first call of any
 * entry point that reads) the library reads windows of 1, 5, 9, 17 and 32
 * tokens (one per code path of the kernel) through it and through the wide
 * path and keeps it only if every workgroup fits, no bounded wait expired,
 * every output is finite and each pair of outputs agrees to 4e-6 of its
 * largest value.  The
 * pages' reads check themselves the same way, once per card, bit for bit
 * against the plain variant ("#315 hc: the multi-token hyper-connection read
 * split finer", Exactness).  One line per device goes to stderr unless
 * HC_LOG=0; HC_SELFCHECK_WAIT_TICKS lowers the bounded waits' limit for the
 * check (ticks of the 100 MHz clock), which forces the fallback.  Runs the
 * check on the default stream if it has not run yet (not under capture).
 * Returns HC_OK or an HC_ERR_* code.
 */
HC_API int hc_short_window_on(int* on);

/* Text for a status code (static storage; never NULL). */
HC_API const char* hc_status_string(int status);

/* The hipError_t behind the last HC_ERR_LAUNCH / HC_ERR_DEVICE / HC_ERR_NOMEM
 * on this host thread (0 if none). */
HC_API int hc_last_hip_error(void);

/* The read's dimensions: streams, width, rank and eps (any pointer may be NULL). */
HC_API void hc_dims(int* n, int* C, int* r, float* eps);

/*
 * hc_timeouts -- number of expired bounded waits recorded in the workspace of
 * (current device, stream) and by the current device's allocation-free reads
 * since the last call, then resets them to zero (the reads concerned stored
 * NaN outputs; see Errors above).
 * Synchronizes `stream`.  *count receives 0 when the stream has no workspace.
 * Returns HC_OK or an HC_ERR_* code.
 */
HC_API int hc_timeouts(void* stream, uint32_t* count);

/*
 * hc_stream_read -- a measurement reference, not part of the read: one launch
 * of the short-window kernel's shape (256 workgroups of 512 threads, one per
 * CU) that streams `bytes` of `src` from memory into LDS with the whole-line
 * loads its weight tiles use and computes nothing.  Its duration is the
 * floor for a single launch moving that many bytes, against which the read's
 * duration (13,148,160 weight bytes, "#2070 sm_75: a hyper-connection up
 * kernel", the 13 MB of BF16 weights per read) is compared.
 *
 *   src     const device buffer of `bytes` bytes, 16-byte aligned
 *   bytes   a multiple of 16, >= 16
 *   sink    uint32_t[256] device buffer, 16-byte aligned: one word per
 *           workgroup (keeps the loads live; its contents mean nothing)
 *   stream  hipStream_t to run on (NULL = default stream)
 *
 * Asynchronous; allocates nothing.  Returns HC_OK, HC_ERR_ARG (null pointer,
 * bytes < 16 or not a multiple of 16), HC_ERR_ALIGN, HC_ERR_DEVICE or
 * HC_ERR_LAUNCH.
 */
HC_API int hc_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * hc_release_stream -- free the workspace of (current device, stream), after
 * synchronizing that stream.  Call it before destroying a stream that ran
 * reads, or the workspace stays allocated until hc_release.  Later calls on
 * the stream allocate again.  Returns HC_OK (also when the stream has no
 * workspace) or an HC_ERR_* code.
 */
HC_API int hc_release_stream(void* stream);

/* Free every workspace the library holds on every device (synchronizes each
 * device that has one).  Later calls allocate again. */
HC_API void hc_release(void);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
