// ds_api.hip -- host side of the C ABI declared in include/ds_sample.h.
//
// Validates every argument before anything is enqueued, splits a call into
// launches of at most 64 requests (their per-request parameters travel by value in
// the kernel argument segment, so no host-to-device copy precedes a launch), and
// picks the path: one wavefront per cell when the row fits in registers;
// otherwise a parts kernel (one workgroup per vocabulary part of a row) and a
// merge kernel (one per row), in batches of rows that fit the handle's record
// workspace.  ds_sample_device_params is the fixed-shape variant whose
// per-request parameters stay in device memory, for graph replay.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "ds_kernels.h"
#include "ds_sample.h"

struct ds_sampler {
    int device;
    // streaming-kernel workspace: one partial record per (row, vocabulary part)
    ds::PartRec* ws_part;
    // threshold windows and their key buffers for win_rows rows per launch
    // (vocabularies on the streaming path only; nullptr otherwise)
    ds::WinRec* ws_win;
    uint32_t* ws_keys;
    int64_t win_rows;
    int32_t vocab;
    int32_t dtype;
    int32_t max_rows;
    int64_t max_positions;
    int32_t max_requests;
    int32_t top_k;
    int32_t vocab_chunks;
    uint32_t flags;
    float z0;
    int32_t cus;  // compute units of the device
};

// Workspace of ds_sample_static: the streaming kernels' per-(row, part) records,
// one copy per device for the life of the process (512 KB).  Host code never
// passes this name to a kernel: it is a host-side stand-in, and the device
// address of each device's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) ds::PartRec scratch[ds::kWorkParts];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Standard normal quantile by bisection on erfc (host, once per handle).
double normal_quantile(double p) {
    double lo = -10.0, hi = 10.0;
    for (int i = 0; i < 200; ++i) {
        const double mid = 0.5 * (lo + hi);
        const double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
        if (cdf < p)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {  // dev < 0: stay on the current device
        err = hipGetDevice(&prev);
        if (err == hipSuccess && dev >= 0 && prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The row fits the wave-per-cell kernel's registers.
bool small_fits(const ds_sampler* s) {
    const bool bf16 = s->dtype == DS_DTYPE_BF16;
    const int ns = ds::small_slots_needed(bf16, s->vocab);
    return ns <= (bf16 ? ds::kSmallMaxSlotsBf16 : ds::kSmallMaxSlotsF32);
}

bool use_small_kernel(const ds_sampler* s) { return !(s->flags & DS_FLAG_FORCE_FALLBACK) && small_fits(s); }

// What a sampling call needs from its sampler: a handle's settings and limits,
// or the arguments of the handle-free entry point.
struct SamplerCfg {
    int32_t vocab, dtype, top_k, vocab_chunks;
    uint32_t flags;
    float z0;
    int32_t max_rows, max_requests;
    int64_t max_positions;
    int device;  // -1: the calling thread's current device
    // threshold windows of the streaming path (none: nullptr, 0 rows)
    ds::WinRec* win;
    uint32_t* keys;
    int64_t win_rows;
};

SamplerCfg cfg_of(const ds_sampler* s) {
    return SamplerCfg{s->vocab,    s->dtype,        s->top_k,         s->vocab_chunks, s->flags,
                      s->z0,       s->max_rows,     s->max_requests,  s->max_positions, s->device,
                      s->ws_win,   s->ws_keys,      s->win_rows};
}

// Parts per chunk and rows per streaming launch, and the window buffers it
// uses.  With the threshold output and window buffers the parts kernel that
// takes the window runs (smaller workgroups, so more parts of a row), and a
// launch holds as many rows as the buffers do (and the records allow).
int64_t stream_layout(ds::SampleArgs& a, bool bf16, int32_t vocab, int32_t chunks, int64_t cells, ds::WinRec* win,
                      uint32_t* keys, int64_t win_rows) {
    const bool use_win = a.thresholds && !a.force_fallback && win && keys && win_rows > 0;
    a.w.ppc = ds::row_parts_per_chunk(bf16, vocab, chunks, cells, use_win);
    a.w.nparts = a.w.ppc * chunks;
    int64_t slots = ds::kWorkParts / a.w.nparts;
    a.w.win = use_win ? win : nullptr;
    a.w.keys = use_win ? keys : nullptr;
    if (use_win && slots > win_rows) slots = win_rows;
    return slots;
}

// First pivot of the wave-per-cell kernel's exact threshold search: the normal
// quantile whose upper tail holds a little more than top_k of V ids.
float pivot_quantile(int32_t top_k, int32_t vocab) {
    double q0 = 1.25 * (double)top_k / vocab + 2.0 / std::sqrt((double)vocab);
    if (q0 > 0.5) q0 = 0.5;
    return (float)normal_quantile(1.0 - q0);
}

// Argument checks shared by ds_sample_create and ds_sample_static.
int check_sampler_settings(int32_t vocab, int32_t dtype, int32_t top_k, int32_t vocab_chunks, uint32_t flags) {
    if (vocab < 1) return fail(DS_ERR_INVALID_ARG, "vocab must be >= 1 (got %d)", vocab);
    if (dtype != DS_DTYPE_F32 && dtype != DS_DTYPE_BF16)
        return fail(DS_ERR_INVALID_ARG, "dtype must be DS_DTYPE_F32 or DS_DTYPE_BF16 (got %d)", dtype);
    if (top_k < 0 || top_k > vocab) return fail(DS_ERR_INVALID_ARG, "top_k must be in [0, vocab]");
    const int32_t max_chunks = vocab < 1024 ? vocab : 1024;
    if (vocab_chunks < 1 || vocab_chunks > max_chunks)
        return fail(DS_ERR_INVALID_ARG, "vocab_chunks must be in [1, %d]", max_chunks);
    if (flags & ~(uint32_t)(DS_FLAG_FORCE_FALLBACK | DS_FLAG_COMPACT_U))
        return fail(DS_ERR_INVALID_ARG, "unknown flags");
    return DS_OK;
}

// Limits of ds_sample_device_params: one wave reads every request's length,
// and 64 clamped lengths must sum below 2^31.
constexpr int32_t kDevParamsMaxRequests = ds::kWave;
constexpr int64_t kDevParamsMaxPositions = int64_t(1) << 24;

// The device-parameter kernels over every cell of the fixed [num_rows, d.P]
// layout: the wave-per-cell kernel, or the streaming pair in batches that fit
// the workspace (padding cells leave at once).
int launch_dev_params(ds_sampler* s, ds::SampleArgs& a, const ds::DevReq& d, int32_t num_rows,
                             hipStream_t st) {
    const bool bf16 = s->dtype == DS_DTYPE_BF16;
    const int64_t positions = d.P;
    if (use_small_kernel(s)) {
        const hipError_t e = ds::launch_sample_small_dev(bf16, a, d, st);
        if (e != hipSuccess) return hip_fail(e, "sampler kernel launch");
        return DS_OK;
    }
    // the streaming kernels over every cell of the fixed layout, in batches that
    // fit the workspace; padding cells leave at once
    const int64_t cells = (int64_t)num_rows * positions;
    const int64_t slots = stream_layout(a, bf16, s->vocab, s->vocab_chunks, cells, s->ws_win, s->ws_keys, s->win_rows);
    for (int64_t c0 = 0; c0 < cells; c0 += slots) {
        a.w.cell_base = c0;
        a.w.ncells = (int32_t)(cells - c0 < slots ? cells - c0 : slots);
        const hipError_t e = ds::launch_sample_row_dev(bf16, a, d, st);
        if (e != hipSuccess) return hip_fail(e, "sampler kernel launch");
    }
    return DS_OK;
}

}  // namespace

extern "C" {

const char* ds_last_error(void) { return g_err.c_str(); }

int ds_version(void) { return 300; }

int ds_sample_create(ds_sampler** out, int device, int32_t vocab, int32_t dtype, int32_t max_rows,
                     int64_t max_positions, int32_t max_requests, int32_t top_k,
                     int32_t vocab_chunks, uint32_t flags) {
    g_err.clear();
    if (!out) return fail(DS_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (vocab < 1) return fail(DS_ERR_INVALID_ARG, "vocab must be >= 1 (got %d)", vocab);
    if (dtype != DS_DTYPE_F32 && dtype != DS_DTYPE_BF16)
        return fail(DS_ERR_INVALID_ARG, "dtype must be DS_DTYPE_F32 or DS_DTYPE_BF16 (got %d)", dtype);
    if (max_rows < 1) return fail(DS_ERR_INVALID_ARG, "max_rows must be >= 1");
    if (max_positions < 1) return fail(DS_ERR_INVALID_ARG, "max_positions must be >= 1");
    if (max_requests < 1) return fail(DS_ERR_INVALID_ARG, "max_requests must be >= 1");
    if ((int64_t)max_rows * max_positions > (int64_t)INT32_MAX)
        return fail(DS_ERR_INVALID_ARG, "max_rows * max_positions exceeds 2^31 - 1 cells");
    {
        const int rc = check_sampler_settings(vocab, dtype, top_k, vocab_chunks, flags);
        if (rc != DS_OK) return rc;
    }
    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= ndev) return fail(DS_ERR_INVALID_ARG, "device %d out of range", device);

    ds_sampler* s = new (std::nothrow) ds_sampler();
    if (s) {
        s->ws_part = nullptr;
        s->ws_win = nullptr;
        s->ws_keys = nullptr;
        s->win_rows = 0;
    }
    if (!s) return fail(DS_ERR_NO_MEMORY, "host allocation failed");
    s->device = device;
    s->vocab = vocab;
    s->dtype = dtype;
    s->max_rows = max_rows;
    s->max_positions = max_positions;
    s->max_requests = max_requests;
    s->top_k = top_k ? top_k : (vocab + 9) / 10;
    s->vocab_chunks = vocab_chunks;
    s->flags = flags;
    s->z0 = pivot_quantile(s->top_k, vocab);
    {
        DeviceGuard dg(device);
        if (dg.err != hipSuccess) {
            delete s;
            return hip_fail(dg.err, "hipSetDevice");
        }
        if (hipDeviceGetAttribute(&s->cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || s->cus < 1)
            s->cus = 1;
        const hipError_t e1 = hipMalloc(&s->ws_part, sizeof(ds::PartRec) * ds::kWorkParts);
        if (e1 != hipSuccess) {
            delete s;
            return fail(DS_ERR_NO_MEMORY, "device workspace allocation failed");
        }
        if (!small_fits(s)) {
            // the streaming path's threshold windows: a record and a key buffer
            // (64 KB) per row of a launch, at most kWinRows rows (128 MB)
            const int64_t cells = (int64_t)max_rows * max_positions;
            s->win_rows = cells < ds::kWinRows ? cells : ds::kWinRows;
            const hipError_t e2 = hipMalloc(&s->ws_win, sizeof(ds::WinRec) * s->win_rows);
            const hipError_t e3 =
                e2 == hipSuccess ? hipMalloc(&s->ws_keys, sizeof(uint32_t) * ds::kWinKeysPerRow * s->win_rows)
                                 : e2;
            if (e2 != hipSuccess || e3 != hipSuccess) {
                (void)hipFree(s->ws_win);
                (void)hipFree(s->ws_part);
                delete s;
                return fail(DS_ERR_NO_MEMORY, "device workspace allocation failed");
            }
        }
    }
    *out = s;
    return DS_OK;
}

void ds_sample_destroy(ds_sampler* s) {
    if (!s) return;
    DeviceGuard dg(s->device);
    (void)hipFree(s->ws_part);
    (void)hipFree(s->ws_win);
    (void)hipFree(s->ws_keys);
    delete s;
}

}  // extern "C"

namespace {

// ds_sample's checks and launches, for a handle's settings or the handle-free
// entry point's; ws is the streaming kernels' record workspace.
// What a valid call asks for, found by check_call.
struct CallShape {
    int64_t P, Pu;   // positions, and positions whose requests read u
    bool need_u, compact_u, small, bf16;
};

// Every argument check of a sampling call, before anything touches the device.
int check_call(const SamplerCfg& s, const int64_t* request_ids, const void* c_logits, const void* u_logits,
               const int32_t* seq_lens, const int32_t* iterations, const float* guidance_scale, const float* temperature,
               int32_t num_requests, int32_t num_rows, const int32_t* tokens_out, const float* logprobs_out,
               const float* threshold_out, CallShape& sh) {
    if (!request_ids || !seq_lens || !iterations || !guidance_scale || !temperature)
        return fail(DS_ERR_INVALID_ARG, "a per-request host array is NULL");
    if (!c_logits || !tokens_out || !logprobs_out)
        return fail(DS_ERR_INVALID_ARG, "c_logits, tokens_out and logprobs_out must be non-NULL");
    if (num_requests < 1 || num_requests > s.max_requests)
        return fail(DS_ERR_CAPACITY, "num_requests %d outside [1, %d]", num_requests, s.max_requests);
    if (num_rows < 1 || num_rows > s.max_rows)
        return fail(DS_ERR_CAPACITY, "num_rows %d outside [1, %d]", num_rows, s.max_rows);
    const uintptr_t es = s.dtype == DS_DTYPE_BF16 ? 2 : 4;
    if (!aligned(c_logits, es)) return fail(DS_ERR_INVALID_ARG, "c_logits is not %d-byte aligned", (int)es);
    if (!aligned(tokens_out, 4) || !aligned(logprobs_out, 4) || (threshold_out && !aligned(threshold_out, 4)))
        return fail(DS_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
    int64_t P = 0, Pu = 0;
    bool need_u = false;
    for (int32_t r = 0; r < num_requests; ++r) {
        if (seq_lens[r] < 0) return fail(DS_ERR_INVALID_ARG, "seq_lens[%d] = %d < 0", r, seq_lens[r]);
        if (!std::isfinite(guidance_scale[r]))
            return fail(DS_ERR_INVALID_ARG, "guidance_scale[%d] is not finite", r);
        if (!(temperature[r] >= 0.0f) || !std::isfinite(temperature[r]))
            return fail(DS_ERR_INVALID_ARG, "temperature[%d] must be finite and >= 0", r);
        need_u |= guidance_scale[r] != 0.0f;
        P += seq_lens[r];
        if (guidance_scale[r] != 0.0f) Pu += seq_lens[r];
    }
    const bool compact_u = (s.flags & DS_FLAG_COMPACT_U) != 0;
    if (P > s.max_positions)
        return fail(DS_ERR_CAPACITY, "sum(seq_lens) = %lld exceeds max_positions %lld", (long long)P,
                    (long long)s.max_positions);
    if ((int64_t)num_rows * P > (int64_t)INT32_MAX)
        return fail(DS_ERR_CAPACITY, "num_rows * sum(seq_lens) exceeds 2^31 - 1 cells");
    if (need_u && !u_logits)
        return fail(DS_ERR_INVALID_ARG, "u_logits is NULL but a request has guidance_scale != 0");
    if (need_u) {
        if (!aligned(u_logits, es)) return fail(DS_ERR_INVALID_ARG, "u_logits is not %d-byte aligned", (int)es);
        if ((((uintptr_t)u_logits - (uintptr_t)c_logits) & 15u) != 0)
            return fail(DS_ERR_UNSUPPORTED, "u_logits and c_logits must have the same address modulo 16 bytes");
    }
    const bool bf16 = s.dtype == DS_DTYPE_BF16;
    const bool small = !(s.flags & DS_FLAG_FORCE_FALLBACK) &&
                       ds::small_slots_needed(bf16, s.vocab) <= (bf16 ? ds::kSmallMaxSlotsBf16 : ds::kSmallMaxSlotsF32);
    if (compact_u && need_u && !small && ((int64_t)s.vocab * (int64_t)es) % 16 != 0)
        return fail(DS_ERR_UNSUPPORTED, "a compacted u layout needs V * %d bytes to be a multiple of 16 here", (int)es);
    sh = CallShape{P, Pu, need_u, compact_u, small, bf16};
    return DS_OK;
}

int sample_call(const SamplerCfg& s, ds::PartRec* ws, const int64_t* request_ids, const void* c_logits,
                const void* u_logits, const int32_t* seq_lens, const int32_t* iterations, const float* guidance_scale,
                const float* temperature, int32_t num_requests, int32_t num_rows, uint64_t seed, int32_t* tokens_out,
                float* logprobs_out, float* threshold_out, void* stream) {
    CallShape sh;
    {
        const int rc = check_call(s, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale, temperature,
                                  num_requests, num_rows, tokens_out, logprobs_out, threshold_out, sh);
        if (rc != DS_OK) return rc;
    }
    const int64_t P = sh.P, Pu = sh.Pu;
    const bool need_u = sh.need_u, compact_u = sh.compact_u, small = sh.small, bf16 = sh.bf16;
    if (P == 0) return DS_OK;

    DeviceGuard dg(s.device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    hipStream_t st = (hipStream_t)stream;

    ds::SampleArgs a;
    a.c = c_logits;
    a.u = need_u ? u_logits : nullptr;
    a.V = s.vocab;
    a.rows = num_rows;
    a.top_k = s.top_k;
    a.vocab_chunks = s.vocab_chunks;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.z0 = s.z0;
    a.force_fallback = (s.flags & DS_FLAG_FORCE_FALLBACK) ? 1 : 0;
    a.tokens = tokens_out;
    a.logprobs = logprobs_out;
    a.thresholds = threshold_out;
    a.w = ds::RowWork{ws, 0, 0, 0, 0, nullptr, nullptr};

    // one launch per group of up to 64 non-empty requests (contiguous positions)
    int32_t r = 0;
    int64_t pos = 0, upos = 0;  // packed position of the launch; next compacted u position
    while (r < num_requests) {
        ds::ReqTable rq;
        std::memset(&rq, 0, sizeof rq);
        rq.P = (int32_t)P;
        rq.Pu = (int32_t)(compact_u ? Pu : P);
        while (r < num_requests && seq_lens[r] == 0) ++r;
        if (r >= num_requests) break;
        rq.pos0 = (int32_t)pos;
        int32_t n = 0, rel = 0;
        while (r < num_requests && n < ds::kMaxReqPerLaunch) {
            if (seq_lens[r] > 0) {
                rq.offs[n] = rel;
                ds::ReqParams& q = rq.req[n];
                q.start = rel;
                q.scale = guidance_scale[r];
                q.tau = temperature[r];
                // IEEE division, correctly rounded like the kernels' 1.0f / tau
                q.inv_tau = temperature[r] > 0.0f ? 1.0f / temperature[r] : 0.0f;
                // u position of the request's first cell: its own position, or the
                // next compacted one (requests with guidance 0 read no u)
                q.uoff = compact_u ? (int32_t)upos : (int32_t)(pos + rel);
                if (compact_u && guidance_scale[r] != 0.0f) upos += seq_lens[r];
                q.row_iter_hi = (uint32_t)iterations[r] << 16;
                q.rid = (uint32_t)request_ids[r];
                rel += seq_lens[r];
                ++n;
            }
            ++r;
        }
        rq.n = n;
        rq.offs[n] = rel;
        rq.npos = rel;
        // u can be loaded before the request lookup when every request reads it
        // at its own position
        rq.all_guided = compact_u ? 0 : 1;
        for (int32_t i = 0; i < n; ++i) rq.all_guided &= rq.req[i].scale != 0.0f ? 1 : 0;
        if (small) {
            const hipError_t e = ds::launch_sample_small(bf16, a, rq, st);
            if (e != hipSuccess) return hip_fail(e, "sampler kernel launch");
        } else {
            // the streaming kernel: cells in batches that fit the workspace
            const int64_t cells = (int64_t)num_rows * rel;
            const int64_t slots = stream_layout(a, bf16, s.vocab, s.vocab_chunks, cells, s.win, s.keys, s.win_rows);
            for (int64_t c0 = 0; c0 < cells; c0 += slots) {
                a.w.cell_base = c0;
                a.w.ncells = (int32_t)(cells - c0 < slots ? cells - c0 : slots);
                const hipError_t e = ds::launch_sample_row(bf16, a, rq, st);
                if (e != hipSuccess) return hip_fail(e, "sampler kernel launch");
            }
        }
        pos += rel;
    }
    return DS_OK;
}

// The static scratch of ds_sample_static on each device, found once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
ds::PartRec* g_scratch_ptr[kMaxDevices];

}  // namespace

extern "C" {

int ds_sample(ds_sampler* s, const int64_t* request_ids, const void* c_logits, const void* u_logits,
              const int32_t* seq_lens, const int32_t* iterations, const float* guidance_scale,
              const float* temperature, int32_t num_requests, int32_t num_rows, uint64_t seed,
              int32_t* tokens_out, float* logprobs_out, float* threshold_out, void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    return sample_call(cfg_of(s), s->ws_part, request_ids, c_logits, u_logits, seq_lens, iterations,
                       guidance_scale, temperature, num_requests, num_rows, seed, tokens_out, logprobs_out,
                       threshold_out, stream);
}

int ds_sample_static(int32_t vocab, int32_t dtype, int32_t top_k, int32_t vocab_chunks, uint32_t flags,
                     const int64_t* request_ids, const void* c_logits, const void* u_logits, const int32_t* seq_lens,
                     const int32_t* iterations, const float* guidance_scale, const float* temperature,
                     int32_t num_requests, int32_t num_rows, uint64_t seed, int32_t* tokens_out, float* logprobs_out,
                     float* threshold_out, void* stream) {
    g_err.clear();
    {
        const int rc = check_sampler_settings(vocab, dtype, top_k, vocab_chunks, flags);
        if (rc != DS_OK) return rc;
    }
    // settings of a handle without its limits (the cell count must fit 31 bits);
    // the first pivot quantile depends only on (top_k, vocab), so the last one is
    // kept per thread
    const int32_t k = top_k ? top_k : (vocab + 9) / 10;
    thread_local int32_t z_k = -1, z_v = -1;
    thread_local float z0 = 0.0f;
    if (z_k != k || z_v != vocab) {
        z0 = pivot_quantile(k, vocab);
        z_k = k;
        z_v = vocab;
    }
    // no threshold windows, and no memory beyond the static records
    const SamplerCfg cfg{vocab, dtype, k, vocab_chunks, flags, z0, INT32_MAX, INT32_MAX, INT32_MAX, -1,
                         nullptr, nullptr, 0};
    // every argument is checked before the device is asked anything
    {
        CallShape sh;
        const int rc = check_call(cfg, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale,
                                  temperature, num_requests, num_rows, tokens_out, logprobs_out, threshold_out, sh);
        if (rc != DS_OK || sh.P == 0) return rc;
    }
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DS_ERR_UNSUPPORTED, "device %d beyond the first %d", dev, kMaxDevices);
    ds::PartRec* ws = nullptr;
    {
        // the device copy of `scratch` of this device: its address, looked up once
        // with this device current (the array's name is not a device address in
        // host code)
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void* p = nullptr;
            const hipError_t e2 = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e2 != hipSuccess || !p) return hip_fail(e2 != hipSuccess ? e2 : hipErrorInvalidSymbol,
                                                        "hipGetSymbolAddress(scratch)");
            g_scratch_ptr[dev] = static_cast<ds::PartRec*>(p);
        }
        ws = g_scratch_ptr[dev];
    }
    return sample_call(cfg, ws, request_ids, c_logits, u_logits, seq_lens, iterations, guidance_scale, temperature,
                       num_requests, num_rows, seed, tokens_out, logprobs_out, threshold_out, stream);
}

int ds_sample_device_params(ds_sampler* s, const int64_t* request_ids, const void* c_logits, const void* u_logits,
                            const int32_t* seq_lens, const int32_t* iterations, const float* guidance_scale,
                            const float* temperature, int32_t num_requests, int32_t num_rows, int64_t positions,
                            uint64_t seed, int32_t* tokens_out, float* logprobs_out, float* threshold_out,
                            void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    if (!request_ids || !seq_lens || !iterations || !guidance_scale || !temperature)
        return fail(DS_ERR_INVALID_ARG, "a per-request device array is NULL");
    if (!c_logits || !tokens_out || !logprobs_out)
        return fail(DS_ERR_INVALID_ARG, "c_logits, tokens_out and logprobs_out must be non-NULL");
    if (num_requests < 1 || num_requests > s->max_requests || num_requests > kDevParamsMaxRequests)
        return fail(DS_ERR_CAPACITY, "num_requests %d outside [1, %d]", num_requests,
                    s->max_requests < kDevParamsMaxRequests ? s->max_requests : kDevParamsMaxRequests);
    if (num_rows < 1 || num_rows > s->max_rows)
        return fail(DS_ERR_CAPACITY, "num_rows %d outside [1, %d]", num_rows, s->max_rows);
    if (positions < 1 || positions > s->max_positions || positions > kDevParamsMaxPositions)
        return fail(DS_ERR_CAPACITY, "positions %lld outside [1, %lld]", (long long)positions,
                    (long long)(s->max_positions < kDevParamsMaxPositions ? s->max_positions : kDevParamsMaxPositions));
    const uintptr_t es = s->dtype == DS_DTYPE_BF16 ? 2 : 4;
    if (!aligned(c_logits, es)) return fail(DS_ERR_INVALID_ARG, "c_logits is not %d-byte aligned", (int)es);
    if (u_logits) {
        if (!aligned(u_logits, es)) return fail(DS_ERR_INVALID_ARG, "u_logits is not %d-byte aligned", (int)es);
        if ((((uintptr_t)u_logits - (uintptr_t)c_logits) & 15u) != 0)
            return fail(DS_ERR_UNSUPPORTED, "u_logits and c_logits must have the same address modulo 16 bytes");
    }
    if (!aligned(tokens_out, 4) || !aligned(logprobs_out, 4) || (threshold_out && !aligned(threshold_out, 4)))
        return fail(DS_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
    if (s->flags & DS_FLAG_COMPACT_U)
        return fail(DS_ERR_UNSUPPORTED, "ds_sample_device_params does not take the compacted u layout");
    if (!aligned(request_ids, 8) || !aligned(seq_lens, 4) || !aligned(iterations, 4) || !aligned(guidance_scale, 4) ||
        !aligned(temperature, 4))
        return fail(DS_ERR_INVALID_ARG, "per-request device arrays must be aligned to their element size");

    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    ds::SampleArgs a;
    a.c = c_logits;
    a.u = u_logits;
    a.V = s->vocab;
    a.rows = num_rows;
    a.top_k = s->top_k;
    a.vocab_chunks = s->vocab_chunks;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.z0 = s->z0;
    a.force_fallback = (s->flags & DS_FLAG_FORCE_FALLBACK) ? 1 : 0;
    a.tokens = tokens_out;
    a.logprobs = logprobs_out;
    a.thresholds = threshold_out;
    a.w = ds::RowWork{s->ws_part, 0, 0, 0, 0, nullptr, nullptr};
    ds::DevReq d;
    d.request_ids = request_ids;
    d.seq_lens = seq_lens;
    d.iterations = iterations;
    d.guidance = guidance_scale;
    d.temperature = temperature;
    d.n = num_requests;
    d.P = (int32_t)positions;
    d.one_per_request = 0;
    return launch_dev_params(s, a, d, num_rows, (hipStream_t)stream);
}

int ds_greedy_lse(ds_sampler* s, const void* logits, int64_t n_rows, int32_t* token_out, float* lse_out,
                  float* logprob_out, float* triples_out, void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    if (n_rows < 0) return fail(DS_ERR_INVALID_ARG, "n_rows must be >= 0");
    if (n_rows > (int64_t)s->max_rows * s->max_positions)
        return fail(DS_ERR_CAPACITY, "n_rows %lld exceeds max_rows * max_positions", (long long)n_rows);
    if (n_rows == 0) return DS_OK;
    if (!logits || !token_out || !lse_out || !logprob_out)
        return fail(DS_ERR_INVALID_ARG, "logits, token_out, lse_out and logprob_out must be non-NULL");
    const uintptr_t es = s->dtype == DS_DTYPE_BF16 ? 2 : 4;
    if (!aligned(logits, es)) return fail(DS_ERR_INVALID_ARG, "logits is not %d-byte aligned", (int)es);
    if (!aligned(token_out, 4) || !aligned(lse_out, 4) || !aligned(logprob_out, 4) ||
        (triples_out && !aligned(triples_out, 4)))
        return fail(DS_ERR_INVALID_ARG, "outputs must be 4-byte aligned");

    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    ds::GreedyArgs a;
    a.x = logits;
    a.n_rows = n_rows;
    a.V = s->vocab;
    a.vocab_chunks = s->vocab_chunks;
    a.token = token_out;
    a.lse = lse_out;
    a.logprob = logprob_out;
    a.triples = triples_out;
    const bool bf16 = s->dtype == DS_DTYPE_BF16;
    a.w = ds::RowWork{s->ws_part, 0, 0, 0, 0, nullptr, nullptr};
    // Rows that fill every compute unit (whole rounds of one row per unit, or
    // enough rounds that the last partial one costs little) take one workgroup
    // per row and no second kernel; otherwise rows are split into parts.
    const int64_t rounds = (n_rows + s->cus - 1) / s->cus;
    if (!(s->flags & DS_FLAG_FORCE_FALLBACK) && n_rows >= s->cus && n_rows * 10 >= rounds * s->cus * 9 &&
        ds::greedy_rows_fits(bf16, s->vocab, s->vocab_chunks, logits)) {
        const hipError_t e = ds::launch_greedy_rows(bf16, a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "greedy kernel launch");
        return DS_OK;
    }
    a.w.ppc = ds::row_parts_per_chunk(bf16, s->vocab, s->vocab_chunks, n_rows, false);
    a.w.nparts = a.w.ppc * s->vocab_chunks;
    const int64_t slots = ds::kWorkParts / a.w.nparts;
    for (int64_t c0 = 0; c0 < n_rows; c0 += slots) {
        a.w.cell_base = c0;
        a.w.ncells = (int32_t)(n_rows - c0 < slots ? n_rows - c0 : slots);
        const hipError_t e = ds::launch_greedy_lse(bf16, a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "greedy kernel launch");
    }
    return DS_OK;
}


// The pointer checks of the repetition penalty's arguments.
static int check_penalty_args(const ds_sampler* s, const void* logits, const uint32_t* seen_mask, const float* penalty) {
    if (!logits || !seen_mask || !penalty)
        return fail(DS_ERR_INVALID_ARG, "logits, seen_mask and penalty must be non-NULL");
    const uintptr_t es = s->dtype == DS_DTYPE_BF16 ? 2 : 4;
    if (!aligned(logits, es)) return fail(DS_ERR_INVALID_ARG, "logits is not %d-byte aligned", (int)es);
    if (!aligned(seen_mask, 4) || !aligned(penalty, 4))
        return fail(DS_ERR_INVALID_ARG, "seen_mask and penalty must be 4-byte aligned");
    return DS_OK;
}

int ds_repetition_penalty(ds_sampler* s, void* logits, int64_t n_rows, const uint32_t* seen_mask,
                          const float* penalty, void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    if (n_rows < 0) return fail(DS_ERR_INVALID_ARG, "n_rows must be >= 0");
    if (n_rows > (int64_t)s->max_rows * s->max_positions)
        return fail(DS_ERR_CAPACITY, "n_rows %lld exceeds max_rows * max_positions", (long long)n_rows);
    if (n_rows == 0) return DS_OK;
    {
        const int rc = check_penalty_args(s, logits, seen_mask, penalty);
        if (rc != DS_OK) return rc;
    }

    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    ds::PenaltyArgs a;
    a.logits = logits;
    a.seen = seen_mask;
    a.penalty = penalty;
    a.n_rows = n_rows;
    a.V = s->vocab;
    a.W = (s->vocab + 31) / 32;
    const hipError_t e = ds::launch_repetition_penalty(s->dtype == DS_DTYPE_BF16, a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "penalty kernel launch");
    return DS_OK;
}

int ds_sample_ar(ds_sampler* s, const int64_t* request_ids, void* logits, const uint32_t* seen_mask,
                 const float* penalty, const int32_t* iterations, const float* temperature, int32_t num_requests,
                 uint64_t seed, int32_t* tokens_out, float* logprobs_out, void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    if (num_requests < 1 || num_requests > s->max_requests || num_requests > s->max_positions ||
        num_requests > kDevParamsMaxPositions)
        return fail(DS_ERR_CAPACITY, "num_requests %d outside [1, min(max_requests, max_positions)]", num_requests);
    if (!request_ids || !iterations || !temperature)
        return fail(DS_ERR_INVALID_ARG, "a per-request device array is NULL");
    if (!logits || !tokens_out || !logprobs_out)
        return fail(DS_ERR_INVALID_ARG, "logits, tokens_out and logprobs_out must be non-NULL");
    if (!aligned(request_ids, 8) || !aligned(iterations, 4) || !aligned(temperature, 4))
        return fail(DS_ERR_INVALID_ARG, "per-request device arrays must be aligned to their element size");
    if (!aligned(tokens_out, 4) || !aligned(logprobs_out, 4))
        return fail(DS_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
    const bool pen = seen_mask || penalty;
    if (pen) {
        const int rc = check_penalty_args(s, logits, seen_mask, penalty);
        if (rc != DS_OK) return rc;
    } else {
        const uintptr_t es = s->dtype == DS_DTYPE_BF16 ? 2 : 4;
        if (!aligned(logits, es)) return fail(DS_ERR_INVALID_ARG, "logits is not %d-byte aligned", (int)es);
    }
    // The wave-per-cell kernel takes the penalised rows from the penalty kernel,
    // run first on the stream; the streaming parts penalise their own ids.
    const bool small = use_small_kernel(s);
    if (pen && small) {
        const int rc = ds_repetition_penalty(s, logits, num_requests, seen_mask, penalty, stream);
        if (rc != DS_OK) return rc;
    }

    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    ds::SampleArgs a;
    a.c = logits;
    a.u = nullptr;
    a.V = s->vocab;
    a.rows = 1;
    a.top_k = s->top_k;
    a.vocab_chunks = s->vocab_chunks;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.z0 = s->z0;
    a.force_fallback = (s->flags & DS_FLAG_FORCE_FALLBACK) ? 1 : 0;
    a.tokens = tokens_out;
    a.logprobs = logprobs_out;
    a.thresholds = nullptr;
    a.w = ds::RowWork{s->ws_part, 0, 0, 0, 0, nullptr, nullptr};
    ds::DevReq d;
    d.request_ids = request_ids;
    d.seq_lens = nullptr;
    d.iterations = iterations;
    d.guidance = nullptr;  // no u: every guidance scale is 0
    d.temperature = temperature;
    d.n = num_requests;
    d.P = num_requests;
    d.one_per_request = 1;
    if (pen && !small) {
        a.seen = seen_mask;
        a.penalty = penalty;
        a.W = (s->vocab + 31) / 32;
    }
    return launch_dev_params(s, a, d, 1, (hipStream_t)stream);
}

int ds_reveal_topk(ds_sampler* s, const float* scores, int32_t num_rows, const int32_t* seq_lens,
                   const int32_t* reveal_counts, int32_t num_requests, int32_t* index_out, float* score_out,
                   void* stream) {
    g_err.clear();
    if (!s) return fail(DS_ERR_INVALID_ARG, "sampler is NULL");
    if (num_requests < 1) return fail(DS_ERR_INVALID_ARG, "num_requests must be >= 1");
    if (num_requests > s->max_requests)
        return fail(DS_ERR_CAPACITY, "num_requests %d exceeds max_requests %d", num_requests, s->max_requests);
    if (num_rows < 1) return fail(DS_ERR_INVALID_ARG, "num_rows must be >= 1");
    if (num_rows > s->max_rows)
        return fail(DS_ERR_CAPACITY, "num_rows %d exceeds max_rows %d", num_rows, s->max_rows);
    if (!seq_lens || !reveal_counts) return fail(DS_ERR_INVALID_ARG, "seq_lens and reveal_counts must be non-NULL");
    int64_t P = 0, total = 0;
    for (int32_t r = 0; r < num_requests; ++r) {
        if (seq_lens[r] < 0) return fail(DS_ERR_INVALID_ARG, "seq_lens[%d] = %d is negative", r, seq_lens[r]);
        const int64_t n = (int64_t)num_rows * seq_lens[r];
        if (n > INT32_MAX) return fail(DS_ERR_UNSUPPORTED, "request %d has more than 2^31 - 1 cells", r);
        if (reveal_counts[r] < 0 || reveal_counts[r] > n)
            return fail(DS_ERR_INVALID_ARG, "reveal_counts[%d] = %d is outside [0, %lld]", r, reveal_counts[r],
                        (long long)n);
        if (reveal_counts[r] > ds::kRevealCap)
            return fail(DS_ERR_UNSUPPORTED, "reveal_counts[%d] = %d exceeds %d", r, reveal_counts[r],
                        ds::kRevealCap);
        P += seq_lens[r];
        total += reveal_counts[r];
    }
    if (P > s->max_positions)
        return fail(DS_ERR_CAPACITY, "sum(seq_lens) %lld exceeds max_positions %lld", (long long)P,
                    (long long)s->max_positions);
    if (total == 0) return DS_OK;
    if (!scores || !index_out) return fail(DS_ERR_INVALID_ARG, "scores and index_out must be non-NULL");
    if (!aligned(scores, 4) || !aligned(index_out, 4) || (score_out && !aligned(score_out, 4)))
        return fail(DS_ERR_INVALID_ARG, "scores and outputs must be 4-byte aligned");

    DeviceGuard dg(s->device);
    if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
    ds::RevealArgs a;
    a.scores = scores;
    a.P = P;
    a.C = num_rows;
    a.index_out = index_out;
    a.score_out = score_out;
    // one launch per group of up to 64 requests, each with its table by value
    int64_t off = 0, out = 0;
    for (int32_t r0 = 0; r0 < num_requests; r0 += ds::kMaxRevealPerLaunch) {
        ds::RevealTable rt;
        rt.n = 0;
        for (int32_t r = r0; r < num_requests && rt.n < ds::kMaxRevealPerLaunch; ++r) {
            rt.T[rt.n] = seq_lens[r];
            rt.k[rt.n] = reveal_counts[r];
            rt.off[rt.n] = off;
            rt.out[rt.n] = out;
            ++rt.n;
            off += seq_lens[r];
            out += reveal_counts[r];
        }
        const hipError_t e = ds::launch_reveal_topk(a, rt, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "reveal kernel launch");
    }
    return DS_OK;
}

int ds_read_probe(const void* x, int64_t n_rows, int64_t row_bytes, int32_t threads, uint32_t* sink, void* stream) {
    g_err.clear();
    if (!x || !sink) return fail(DS_ERR_INVALID_ARG, "x and sink must be non-NULL");
    if (!aligned(x, 16) || !aligned(sink, 4)) return fail(DS_ERR_INVALID_ARG, "x must be 16-byte and sink 4-byte aligned");
    if (n_rows < 1 || n_rows > INT32_MAX) return fail(DS_ERR_INVALID_ARG, "n_rows must be in [1, 2^31 - 1]");
    if (row_bytes < 16 || row_bytes % 16 != 0)
        return fail(DS_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
    if (threads != 256 && threads != 512 && threads != 1024)
        return fail(DS_ERR_INVALID_ARG, "threads must be 256, 512 or 1024");
    const hipError_t e = ds::launch_read_probe(x, n_rows, row_bytes / 16, threads, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return DS_OK;
}

}  // extern "C"
