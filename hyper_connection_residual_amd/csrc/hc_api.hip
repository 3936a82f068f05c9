// hc_api.hip -- host side of the C ABI declared in include/hc.h: argument
// checks, per-(device, stream) scratch workspaces, and dispatch to the
// short-window (T <= 8) and wide (prefill) kernels.
#include "hc.h"
#include "hc_internal.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace {

thread_local int g_last_hip_error = 0;

struct Workspace {
    int device = 0;
    hipStream_t stream = nullptr;
    void* dec_base = nullptr;
    hc::DecodeScratch dec{};
    void* wide_base = nullptr;
    size_t wide_bytes = 0;
};

std::mutex g_mutex;
std::map<std::pair<int, hipStream_t>, Workspace*> g_workspaces;
std::map<int, bool> g_device_ok;

int record(hipError_t e, int status)
{
    g_last_hip_error = static_cast<int>(e);
    return status;
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
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
        bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        if (ok) {
            // every workgroup of the short-window kernel must be resident at once
            int per_cu = 0;
            e = hc::decode_resident_blocks(&per_cu);
            if (e != hipSuccess)
                return record(e, HC_ERR_DEVICE);
            ok = per_cu * prop.multiProcessorCount >= hc::kDecWGs;
        }
        it = g_device_ok.emplace(*dev, ok).first;
    }
    return it->second ? HC_OK : record(hipSuccess, HC_ERR_DEVICE);
}

// The workspace of (dev, stream); created (and zeroed on the stream) on first use.
int workspace(int dev, hipStream_t stream, Workspace** out)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    auto key = std::make_pair(dev, stream);
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

// The read of hc_read and hc_read_commit; R_commit is NULL or R.
int read_impl(int64_t T, const float* R, const float* pending, const float* w_norm, const uint16_t* W_down,
              const uint16_t* W_up, float* out_mixed, uint16_t* out_bf16, uint16_t* out_fp16, float* R_commit,
              void* stream)
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

    if (T <= hc::kDecSplitMaxT) {
        // A short window: one launch per range of at most 8 consecutive tokens
        // (ranges of near-equal size).  Every token's read is independent of
        // the others, so the split changes no result.
        const int n = static_cast<int>((T + hc::kDecMaxT - 1) / hc::kDecMaxT);
        int t0 = 0;
        for (int c = 0; c < n; ++c) {
            const int left = static_cast<int>(T) - t0, chunks = n - c;
            const int tc = (left + chunks - 1) / chunks;
            const size_t in = static_cast<size_t>(t0) * hc::kD, out = static_cast<size_t>(t0) * hc::kWidth;
            hipError_t e = hc::launch_decode(tc, R + in, pending ? pending + in : nullptr, w_norm, W_down, W_up,
                                             out_mixed + out, out_bf16 + out, out_fp16 + out,
                                             R_commit ? R_commit + in : nullptr, ws->dec, hs);
            if (e != hipSuccess)
                return record(e, HC_ERR_LAUNCH);
            t0 += tc;
        }
        return HC_OK;
    }
    st = wide_workspace(ws);
    if (st != HC_OK)
        return st;
    hipError_t e = hc::launch_prefill(T, R, pending, w_norm, W_down, W_up, out_mixed, out_bf16, out_fp16, R_commit,
                                      ws->wide_base, hc::kPrefillChunk, hs);
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

HC_API const char* hc_status_string(int status)
{
    switch (status) {
    case HC_OK: return "ok";
    case HC_ERR_ARG: return "invalid argument (T < 1 or a required pointer is NULL)";
    case HC_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case HC_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU or could not be queried";
    case HC_ERR_NOMEM: return "the scratch workspace could not be allocated (or the first call on a stream was under graph capture)";
    case HC_ERR_LAUNCH: return "a kernel launch failed";
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
    Workspace* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_workspaces.find(std::make_pair(dev, hs));
        if (it == g_workspaces.end())
            return HC_OK;
        ws = it->second;
    }
    uint32_t v = 0;
    e = hipMemcpyAsync(&v, ws->dec.timeouts, sizeof(v), hipMemcpyDeviceToHost, hs);
    if (e == hipSuccess)
        e = hipMemsetAsync(ws->dec.timeouts, 0, sizeof(uint32_t), hs);
    if (e == hipSuccess)
        e = hipStreamSynchronize(hs);
    if (e != hipSuccess)
        return record(e, HC_ERR_DEVICE);
    *count = v;
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
    (void)hipSetDevice(cur);
}

}  // extern "C"
