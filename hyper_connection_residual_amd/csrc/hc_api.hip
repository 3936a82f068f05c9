// hc_api.hip -- host side of the C ABI declared in include/hc.h: argument
// checks, per-(device, stream) scratch workspaces, the start-up check of the
// short-window kernel, and dispatch to the short-window (one launch, up to 25
// tokens from hc_read, up to 32 from hc_read_noalloc) and wide (prefill)
// kernels.
#include "hc.h"
#include "hc_internal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace {

thread_local int g_last_hip_error = 0;

struct Workspace {
    int device = 0;
    hipStream_t stream = nullptr;  // (used only while the caller's stream is live: calls on it, hc_release_stream)
    void* dec_base = nullptr;
    hc::DecodeScratch dec{};
    void* wide_base = nullptr;
    size_t wide_bytes = 0;
};

std::mutex g_mutex;
// Workspaces by (device, stream handle value).  A stream that HIP creates with
// the handle of a destroyed one (its memory can be reused only once the old
// stream's work has finished) takes over that workspace; hc_release_stream
// frees a workspace before its stream is destroyed.
std::map<std::pair<int, uintptr_t>, Workspace*> g_workspaces;
std::map<int, bool> g_device_ok;
// Result of the start-up check of the short-window kernel per device (absent:
// not run yet).  Guarded by g_check_mutex, which is taken before g_mutex.
std::mutex g_check_mutex;
std::map<int, bool> g_short_window;
// Short-window launches of one device are ordered across streams.  Each needs
// all 256 of its workgroups resident at once (one per CU); two running at the
// same time could each get only part of the chip, and both would then wait
// until their bounded waits expire.  Per device: which stream made the last
// short-window launch (its handle value, only compared, never passed to HIP).
// A launch on another stream than the last one waits for the last launch:
// through an event recorded right after it, if there is one, else by
// synchronizing the device.  Events are recorded only while streams
// alternate: a switch turns recording on, and 64 launches in a row on one
// stream turn it off again, since an event per read costs +3.5 us (measured
// for a read followed by other work) and a stream's reads are ordered by the
// stream itself.  No handle of another stream is ever used.  Guarded by
// g_mutex.
constexpr int kQuietLaunches = 64;
struct ShortOrder {
    hipEvent_t done = nullptr;
    uintptr_t last = 0;     // stream handle value of the last launch
    bool used = false;      // a launch has been ordered on this device
    bool recording = false; // an event follows every launch
    bool recorded = false;  // `done` covers the last launch
    int quiet = 0;          // launches on the last stream since the last switch
};
std::map<int, ShortOrder> g_short_order;

int record(hipError_t e, int status)
{
    g_last_hip_error = static_cast<int>(e);
    return status;
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// The key of a stream: its handle value (never dereferenced).
uintptr_t stream_key(hipStream_t stream)
{
    return reinterpret_cast<uintptr_t>(stream);
}

// The bounded waits' limit of ordinary reads: HC_WAIT_TICKS (ticks of the
// 100 MHz clock) if set, else 50 ms.  Read once.
long long read_wait_ticks()
{
    static const long long ticks = [] {
        const char* v = std::getenv("HC_WAIT_TICKS");
        return v ? std::atoll(v) : hc::kDecWaitTicks;
    }();
    return ticks;
}

// The current device must be a gfx950 part.
int current_device(int* dev)
{
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_device_ok.find(*dev);
    if (it == g_device_ok.end()) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, *dev);
        if (e != hipSuccess)
            return record(e, HC_ERR_DEVICE);
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_device_ok.emplace(*dev, ok).first;
    }
    return it->second ? HC_OK : record(hipSuccess, HC_ERR_DEVICE);
}

// The workspace of (dev, stream); created (and zeroed on the stream) on first use.
int workspace(int dev, hipStream_t stream, Workspace** out)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    auto key = std::make_pair(dev, stream_key(stream));
    auto it = g_workspaces.find(key);
    if (it != g_workspaces.end()) {
        *out = it->second;
        return HC_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    if (cap != hipStreamCaptureStatusNone)  // the first call on a stream allocates: not under capture
        return record(hipErrorStreamCaptureUnsupported, HC_ERR_NOMEM);
    Workspace* ws = new Workspace();
    ws->device = dev;
    ws->stream = stream;
    const size_t bytes = hc::decode_scratch_bytes();
    e = hipMalloc(&ws->dec_base, bytes);
    if (e != hipSuccess) {
        delete ws;
        return record(e, HC_ERR_NOMEM);
    }
    e = hipMemsetAsync(ws->dec_base, 0, bytes, stream);
    if (e != hipSuccess) {
        (void)hipFree(ws->dec_base);
        delete ws;
        return record(e, HC_ERR_NOMEM);
    }
    hc::decode_scratch_carve(ws->dec_base, &ws->dec);
    g_workspaces.emplace(key, ws);
    *out = ws;
    return HC_OK;
}

// The wide path's scratch, allocated on its first use on this stream.
int wide_workspace(Workspace* ws)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    if (ws->wide_base)
        return HC_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(ws->stream, &cap);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    if (cap != hipStreamCaptureStatusNone)
        return record(hipErrorStreamCaptureUnsupported, HC_ERR_NOMEM);
    const size_t bytes = hc::prefill_scratch_bytes(hc::kPrefillChunk);
    e = hipMalloc(&ws->wide_base, bytes);
    if (e != hipSuccess) {
        ws->wide_base = nullptr;
        return record(e, HC_ERR_NOMEM);
    }
    ws->wide_bytes = bytes;
    return HC_OK;
}

bool log_enabled()
{
    const char* v = std::getenv("HC_LOG");
    return !(v && v[0] == '0' && v[1] == 0);
}

// Deterministic check inputs: values uniform in [-a, a) from a 32-bit
// xorshift, and bf16 bit patterns of such values (round to nearest even).
struct CheckRng {
    uint32_t x = 2463534242u;
    float next(float a)
    {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        return a * (2.0f * (float)(x >> 8) * (1.0f / 16777216.0f) - 1.0f);
    }
    uint16_t bf16(float a)
    {
        const float f = next(a);
        uint32_t u;
        std::memcpy(&u, &f, 4);
        return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
};

// The start-up check of the short-window kernel on one device (the pages'
// kernels check themselves once per card and fall back to the plain kernel
// on any disagreement: "#315 hc: the multi-token hyper-connection read split
// finer", Exactness).  Its hand-offs need all 256 workgroups resident at once
// and the dispatcher's placement of workgroups on XCDs; the check reads one
// window per code path of the kernel (1, 5, 9, 17 and 32 tokens, with
// pending: one, two, three and six MFMA chains; hop 1 on rows, on token pairs
// and on two waves; shared LDS regions) once through it and once through the
// wide path (which needs neither) and keeps it only if (a) every workgroup
// fits, (b) no bounded wait expired and (c) each pair of outputs agrees to
// 4e-6 of its largest value (each is within 2e-6 of the exact read).
// Otherwise every read takes the wide path.  The bounded
// waits' limit can be lowered with HC_SELFCHECK_WAIT_TICKS (ticks of the 100
// MHz clock) to force the fallback.  One line per device goes to stderr
// (HC_LOG=0 silences it).
int run_short_window_check(int dev, Workspace* ws, bool* on, char* why, size_t why_len)
{
    *on = false;
    int per_cu = 0;
    hipError_t e = hc::decode_resident_blocks(&per_cu);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    if (per_cu * cus < hc::kDecWGs) {
        std::snprintf(why, why_len, "%d workgroups per CU x %d CUs cannot hold %d", per_cu, cus, hc::kDecWGs);
        return HC_OK;
    }
    int st = wide_workspace(ws);
    if (st != HC_OK)
        return st;
    constexpr int kChecks[] = {1, 5, 9, 17, 32};
    constexpr int TM = hc::kDecMaxT;
    const size_t nin = (size_t)TM * hc::kD, nw = (size_t)hc::kRank * hc::kD, nout = (size_t)TM * hc::kWidth;
    CheckRng rng;
    std::vector<float> R(nin), P(nin), w(hc::kD);
    std::vector<uint16_t> Wd(nw), Wu(nw);
    for (auto& v : R) v = rng.next(1.7f);
    for (auto& v : P) v = rng.next(0.17f);
    for (auto& v : w) v = 1.0f + rng.next(0.17f);
    for (auto& v : Wd) v = rng.bf16(0.035f);
    for (auto& v : Wu) v = rng.bf16(0.035f);
    const size_t bytes = 4 * (2 * nin + hc::kD) + 2 * (2 * nw) + 2 * (4 * nout + 4 * nout);
    char* buf = nullptr;
    e = hipMalloc(&buf, bytes);
    if (e != hipSuccess)
        return record(e, HC_ERR_NOMEM);
    float* dR = reinterpret_cast<float*>(buf);
    float* dP = dR + nin;
    float* dw = dP + nin;
    uint16_t* dWd = reinterpret_cast<uint16_t*>(dw + hc::kD);
    uint16_t* dWu = dWd + nw;
    float* m1 = reinterpret_cast<float*>(dWu + nw);
    float* m2 = m1 + nout;
    uint16_t* img = reinterpret_cast<uint16_t*>(m2 + nout);  // 4 images of nout
    uint32_t expired = 0;
    std::vector<float> a(nout), b(nout);
    const char* env = std::getenv("HC_SELFCHECK_WAIT_TICKS");
    const long long ticks = env ? std::atoll(env) : hc::kDecWaitTicks;
    hipStream_t hs = ws->stream;
    e = hipMemcpyAsync(dR, R.data(), 4 * nin, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(dP, P.data(), 4 * nin, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(dw, w.data(), 4 * hc::kD, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(dWd, Wd.data(), 2 * nw, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemcpyAsync(dWu, Wu.data(), 2 * nw, hipMemcpyHostToDevice, hs);
    if (e == hipSuccess) e = hipMemsetAsync(ws->dec.timeouts, 0, sizeof(uint32_t), hs);
    double worst = 0.0;
    bool finite = true;
    int worst_T = 0;
    for (int T : kChecks) {
        const size_t no = (size_t)T * hc::kWidth;
        if (e == hipSuccess)
            e = hc::launch_decode(T, dR, dP, dw, dWd, dWu, m1, img, img + nout, nullptr, ws->dec, hs, ticks);
        if (e == hipSuccess)
            e = hc::launch_prefill(T, dR, dP, dw, dWd, dWu, m2, img + 2 * nout, img + 3 * nout, nullptr, false,
                                   ws->wide_base, hc::kPrefillChunk, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(a.data(), m1, 4 * no, hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(b.data(), m2, 4 * no, hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess)
            break;
        double dmax = 0.0, vmax = 0.0;
        for (size_t i = 0; i < no; ++i) {
            finite = finite && std::isfinite(a[i]) && std::isfinite(b[i]);
            dmax = std::fmax(dmax, std::fabs((double)a[i] - (double)b[i]));
            vmax = std::fmax(vmax, std::fabs((double)b[i]));
        }
        const double rel = vmax > 0.0 ? dmax / vmax : dmax;
        if (!(rel <= worst) || worst_T == 0) {
            worst = rel;
            worst_T = T;
        }
    }
    if (e == hipSuccess) e = hipMemcpyAsync(&expired, ws->dec.timeouts, sizeof(uint32_t), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess) e = hipMemsetAsync(ws->dec.timeouts, 0, sizeof(uint32_t), hs);
    if (e == hipSuccess) e = hipStreamSynchronize(hs);
    const hipError_t ef = hipFree(buf);
    if (e != hipSuccess || ef != hipSuccess)
        return record(e != hipSuccess ? e : ef, HC_ERR_DEVICE);
    *on = expired == 0 && finite && worst <= 4e-6;
    std::snprintf(why, why_len, "%u expired waits, %s, agrees with the wide path to %.1e (worst at %d tokens)",
                  expired, finite ? "all finite" : "NOT all finite", worst, worst_T);
    return HC_OK;
}

// Whether short windows use the short-window kernel on `dev`;
// the check runs on the first call for the device.
int short_window_on(int dev, Workspace* ws, bool* on)
{
    std::lock_guard<std::mutex> lock(g_check_mutex);
    auto it = g_short_window.find(dev);
    if (it != g_short_window.end()) {
        *on = it->second;
        return HC_OK;
    }
    char why[200] = "";
    const int st = run_short_window_check(dev, ws, on, why, sizeof why);
    if (st != HC_OK)
        return st;
    if (*on) {
        // set-up of the allocation-free reads on this device: the address of
        // their static scratch (cleared) and the cross-stream order's event,
        // so that hc_read_noalloc never allocates
        hipError_t e = hc::noalloc_setup(dev, ws->stream);
        if (e != hipSuccess)
            return record(e, HC_ERR_DEVICE);
        std::lock_guard<std::mutex> lock(g_mutex);
        ShortOrder& so = g_short_order[dev];
        if (!so.done && (e = hipEventCreateWithFlags(&so.done, hipEventDisableTiming)) != hipSuccess) {
            so.done = nullptr;
            return record(e, HC_ERR_DEVICE);
        }
    }
    g_short_window.emplace(dev, *on);
    if (log_enabled())
        std::fprintf(stderr, "hc: device %d: the short-window read is %s (start-up check: %s)%s\n", dev,
                     *on ? "on" : "OFF", why, *on ? "" : "; every read takes the wide path");
    return HC_OK;
}

// One launch of the short-window kernel on `hs`, after the last short-window
// launch on any other stream of this device (not under graph capture: the
// caller orders the replays of a graph).
hipError_t launch_short_window(int dev, hipStream_t hs, int T, const float* R, const float* pending,
                               const float* w_norm, const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                               uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit, const hc::DecodeScratch& scr)
{
    const uintptr_t id = stream_key(hs);
    std::lock_guard<std::mutex> lock(g_mutex);
    ShortOrder& so = g_short_order[dev];
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(hs, &cap);
    if (e != hipSuccess)
        return e;
    const bool order = cap == hipStreamCaptureStatusNone;
    if (order && so.used && id != so.last) {
        // a switch: after the last launch on the other stream
        e = so.recorded ? hipStreamWaitEvent(hs, so.done, 0) : hipDeviceSynchronize();
        if (e != hipSuccess)
            return e;
        so.recording = true;
        so.quiet = 0;
    } else if (order && so.recording && ++so.quiet >= kQuietLaunches) {
        so.recording = false;  // one stream again: its own order suffices
    }
    e = hc::launch_decode(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, R_commit, scr, hs,
                          read_wait_ticks());
    if (e != hipSuccess)
        return e;
    if (order) {
        so.recorded = false;
        if (so.recording) {
            if (!so.done) {
                e = hipEventCreateWithFlags(&so.done, hipEventDisableTiming);
                if (e != hipSuccess) {
                    so.done = nullptr;
                    return e;
                }
            }
            e = hipEventRecord(so.done, hs);
            if (e != hipSuccess)
                return e;
            so.recorded = true;
        }
        so.last = id;
        so.used = true;
    }
    return hipSuccess;
}

// The read of hc_read, hc_read_commit and hc_read_bf16_lo; R_commit is NULL
// or R; bf16_lo selects the fast numerics of the wide path.
int read_impl(int64_t T, const float* R, const float* pending, const float* w_norm, const uint16_t* W_down,
              const uint16_t* W_up, float* out_mixed, uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit,
              void* stream, bool bf16_lo = false)
{
    if (T < 1 || !R || !w_norm || !W_down || !W_up || !out_mixed || !out_bf16 || !out_fp16)
        return HC_ERR_ARG;
    if (!aligned16(R) || (pending && !aligned16(pending)) || !aligned16(w_norm) ||
        !aligned16(W_down) || !aligned16(W_up) || !aligned16(out_mixed) ||
        !aligned16(out_bf16) || !aligned16(out_fp16))
        return HC_ERR_ALIGN;
    if (!pending)
        R_commit = nullptr;  // nothing to commit
    int dev = 0;
    int st = current_device(&dev);
    if (st != HC_OK)
        return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    Workspace* ws = nullptr;
    st = workspace(dev, hs, &ws);
    if (st != HC_OK)
        return st;
    bool short_ok = false;
    st = short_window_on(dev, ws, &short_ok);
    if (st != HC_OK)
        return st;

    if (T <= hc::kShortReadMaxT && short_ok) {
        hipError_t e = launch_short_window(dev, hs, static_cast<int>(T), R, pending, w_norm, W_down, W_up,
                                           out_mixed, out_bf16, out_fp16, R_commit, ws->dec);
        return e == hipSuccess ? HC_OK : record(e, HC_ERR_LAUNCH);
    }
    st = wide_workspace(ws);
    if (st != HC_OK)
        return st;
    hipError_t e = hc::launch_prefill(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, R_commit,
                                      bf16_lo, ws->wide_base, hc::kPrefillChunk, hs);
    return e == hipSuccess ? HC_OK : record(e, HC_ERR_LAUNCH);
}

}  // namespace

extern "C" {

HC_API int hc_read(int64_t T, const float* R, const float* pending, const float* w_norm,
                   const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                   uint16_t* out_bf16, uint16_t* out_fp16, void* stream)
{
    return read_impl(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, nullptr, stream);
}

HC_API int hc_read_commit(int64_t T, float* R, const float* pending, const float* w_norm,
                          const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                          uint16_t* out_bf16, uint16_t* out_fp16, void* stream)
{
    return read_impl(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, R, stream);
}

HC_API int hc_read_bf16_lo(int64_t T, const float* R, const float* pending, const float* w_norm,
                           const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                           uint16_t* out_bf16, uint16_t* out_fp16, void* stream)
{
    return read_impl(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, nullptr, stream, true);
}

HC_API int hc_read_noalloc(int64_t T, const float* R, const float* pending, const float* w_norm,
                           const uint16_t* W_down, const uint16_t* W_up, float* out_mixed,
                           uint16_t* out_bf16, uint16_t* out_fp16, void* stream)
{
    if (T < 1 || !R || !w_norm || !W_down || !W_up || !out_mixed || !out_bf16 || !out_fp16)
        return HC_ERR_ARG;
    if (T > hc::kDecMaxT)
        return HC_ERR_SIZE;
    if (!aligned16(R) || (pending && !aligned16(pending)) || !aligned16(w_norm) ||
        !aligned16(W_down) || !aligned16(W_up) || !aligned16(out_mixed) ||
        !aligned16(out_bf16) || !aligned16(out_fp16))
        return HC_ERR_ALIGN;
    int dev = 0;
    int st = current_device(&dev);
    if (st != HC_OK)
        return st;
    {
        // set up by the device's start-up check, which must have kept the
        // short-window kernel (the wide path needs allocated scratch)
        std::lock_guard<std::mutex> lock(g_check_mutex);
        auto it = g_short_window.find(dev);
        if (it == g_short_window.end() || !it->second)
            return HC_ERR_STATE;
    }
    hc::DecodeScratch scr;
    if (!hc::noalloc_scratch(dev, &scr))
        return HC_ERR_STATE;
    const hipError_t e = launch_short_window(dev, static_cast<hipStream_t>(stream), static_cast<int>(T), R, pending,
                                             w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, nullptr, scr);
    return e == hipSuccess ? HC_OK : record(e, HC_ERR_LAUNCH);
}

HC_API int hc_short_window_on(int* on)
{
    if (!on)
        return HC_ERR_ARG;
    *on = 0;
    int dev = 0;
    int st = current_device(&dev);
    if (st != HC_OK)
        return st;
    Workspace* ws = nullptr;
    st = workspace(dev, nullptr, &ws);
    if (st != HC_OK)
        return st;
    bool b = false;
    st = short_window_on(dev, ws, &b);
    if (st != HC_OK)
        return st;
    *on = b ? 1 : 0;
    return HC_OK;
}

HC_API const char* hc_status_string(int status)
{
    switch (status) {
    case HC_OK: return "ok";
    case HC_ERR_ARG: return "invalid argument (T < 1 or a required pointer is NULL)";
    case HC_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case HC_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU or could not be queried";
    case HC_ERR_NOMEM: return "the scratch workspace could not be allocated (or the first call on a stream was under graph capture)";
    case HC_ERR_LAUNCH: return "a kernel launch failed";
    case HC_ERR_SIZE: return "T is above 32, the most hc_read_noalloc takes";
    case HC_ERR_STATE: return "allocation-free reads are not set up on this device (call hc_short_window_on first, "
                              "outside graph capture; they need the short-window kernel on)";
    default: return "unknown status";
    }
}

HC_API int hc_last_hip_error(void)
{
    return g_last_hip_error;
}

HC_API void hc_dims(int* n, int* C, int* r, float* eps)
{
    if (n)
        *n = hc::kStreams;
    if (C)
        *C = hc::kWidth;
    if (r)
        *r = hc::kRank;
    if (eps)
        *eps = hc::kEps;
}

HC_API int hc_timeouts(void* stream, uint32_t* count)
{
    if (!count)
        return HC_ERR_ARG;
    *count = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint32_t* counters[2] = {nullptr, nullptr};
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_workspaces.find(std::make_pair(dev, stream_key(hs)));
        if (it != g_workspaces.end())
            counters[0] = it->second->dec.timeouts;
    }
    hc::DecodeScratch na;
    if (hc::noalloc_scratch(dev, &na))
        counters[1] = na.timeouts;  // the allocation-free reads of this device
    uint32_t v[2] = {0, 0};
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
        if (!counters[i])
            continue;
        e = hipMemcpyAsync(&v[i], counters[i], sizeof(uint32_t), hipMemcpyDeviceToHost, hs);
        if (e == hipSuccess)
            e = hipMemsetAsync(counters[i], 0, sizeof(uint32_t), hs);
    }
    if (e == hipSuccess)
        e = hipStreamSynchronize(hs);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    *count = v[0] + v[1];
    return HC_OK;
}

HC_API int hc_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream)
{
    if (!src || !sink || bytes < 16 || bytes % 16 != 0)
        return HC_ERR_ARG;
    if (!aligned16(src) || !aligned16(sink))
        return HC_ERR_ALIGN;
    int dev = 0;
    int st = current_device(&dev);
    if (st != HC_OK)
        return st;
    const hipError_t e = hc::launch_stream(src, bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HC_OK : record(e, HC_ERR_LAUNCH);
}

HC_API int hc_release_stream(void* stream)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_workspaces.find(std::make_pair(dev, stream_key(hs)));
    if (it == g_workspaces.end())
        return HC_OK;
    Workspace* ws = it->second;
    e = hipStreamSynchronize(hs);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    if (ws->dec_base)
        (void)hipFree(ws->dec_base);
    if (ws->wide_base)
        (void)hipFree(ws->wide_base);
    delete ws;
    g_workspaces.erase(it);
    return HC_OK;
}

HC_API void hc_release(void)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_workspaces) {
        Workspace* ws = kv.second;
        (void)hipSetDevice(ws->device);
        (void)hipDeviceSynchronize();
        if (ws->dec_base)
            (void)hipFree(ws->dec_base);
        if (ws->wide_base)
            (void)hipFree(ws->wide_base);
        delete ws;
    }
    g_workspaces.clear();
    for (auto& kv : g_short_order) {
        if (kv.second.done) {
            (void)hipSetDevice(kv.first);
            (void)hipEventDestroy(kv.second.done);
        }
    }
    g_short_order.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
