// C ABI of the W8A16 GEMM: argument checks, plan, workspace, launch.
//
// The entry point mirrors `w8a16_gemm_pipelined_m32_strided` on the page
// "w8a16_gemm_pipelined_m32.rs": the same operands and strides, the same
// rejections in the same order, and an asynchronous launch on the caller's
// stream with no synchronisation.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"
#include "plan.h"

namespace w8a16 {

namespace {

// Split-K workspace and arrival counters of one (device, stream).  The
// counters are zeroed once at allocation; every kernel that uses them
// leaves them at zero again.
struct Workspace {
    float *ws = nullptr;
    uint64_t ws_bytes = 0;
    uint32_t *counters = nullptr;
    uint32_t counter_count = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers replaced by larger ones.  They are never freed: a HIP graph
// captured with an earlier, smaller plan on that stream keeps their
// addresses and may still be replayed.
std::vector<void *> g_retired;

std::mutex g_cu_mutex;
std::map<int, uint32_t> g_cu_count;

int hip_fail(hipError_t e, const char *what)
{
    char buf[256];
    snprintf(buf, sizeof buf, "w8a16_gemm: %s failed: %s", what, hipGetErrorString(e));
    return fail(W8A16_ERR_HIP, buf);
}

// ---- diagnostics ---------------------------------------------------------
// W8A16_LOG (print each distinct launch and its plan once) and
// W8A16_DEBUG_SYNC (wait for the stream after each launch and report a
// failed kernel), read once per process.  Unset, empty or "0" is off, "1"
// is on; any other value fails every enqueuing call with W8A16_ERR_ENV.
struct Levers {
    int status = W8A16_OK;
    bool log = false;
    bool debug_sync = false;
    char msg[160] = "";
};

Levers read_levers()
{
    Levers l;
    const char *names[2] = {"W8A16_LOG", "W8A16_DEBUG_SYNC"};
    bool *flags[2] = {&l.log, &l.debug_sync};
    for (int i = 0; i < 2; ++i) {
        const char *v = std::getenv(names[i]);
        if (!v || !*v || std::strcmp(v, "0") == 0)
            continue;
        if (std::strcmp(v, "1") == 0) {
            *flags[i] = true;
            continue;
        }
        l.status = W8A16_ERR_ENV;
        snprintf(l.msg, sizeof l.msg, "%s='%.48s' must be 0 or 1", names[i], v);
        break;
    }
    return l;
}

const Levers &levers()
{
    static const Levers l = read_levers();
    return l;
}

int check_levers(const char *entry)
{
    const Levers &l = levers();
    if (l.status == W8A16_OK)
        return W8A16_OK;
    char buf[224];
    snprintf(buf, sizeof buf, "%s: %s", entry, l.msg);
    return fail(l.status, buf);
}

const char *kernel_name(uint32_t kernel)
{
    switch (kernel) {
    case W8A16_KERNEL_STREAM: return "stream";
    case W8A16_KERNEL_TILE: return "tile";
    case W8A16_KERNEL_RING: return "ring";
    case W8A16_KERNEL_W8A8: return "w8a8";
    case W8A16_KERNEL_W4A4: return "w4a4";
    case W8A16_KERNEL_W4A4_PS: return "w4a4-persistent";
    default: return "?";
    }
}

std::mutex g_log_mutex;
std::set<std::string> g_logged;   // lines already printed (at most 4096 kept)

void log_line(const char *line)
{
    std::lock_guard<std::mutex> lock(g_log_mutex);
    if (g_logged.size() >= 4096 || !g_logged.insert(line).second)
        return;
    std::fputs(line, stderr);
}

// Under W8A16_LOG=1: the launch of `entry` with plan `p`; `why` is the
// planner's reason, or null for a caller's plan.
void log_plan(const char *entry, uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t &p,
              const char *why)
{
    if (!levers().log)
        return;
    char line[640];
    snprintf(line, sizeof line,
             "w8a16: %s m=%u n=%u k=%u: kernel=%s tile=%ux%u splits=%u (%u K steps each) "
             "waves=%u depth=%u stage_steps=%u a_depth=%u flags=0x%x grid=%u block=%u "
             "lds=%u workspace=%llu: %s\n",
             entry, m, n, k, kernel_name(p.kernel), 16 * p.m_blocks, 16 * p.n_blocks,
             p.splits, p.steps_per_split, p.waves, p.depth, p.stage_steps, p.a_depth, p.flags,
             p.grid, p.block, p.lds_bytes, (unsigned long long)p.workspace_bytes,
             why ? why : "caller's plan");
    log_line(line);
}

// Success epilogue of a call that enqueued work: clears the last error and,
// under W8A16_DEBUG_SYNC=1, waits for the stream (unless it is being
// captured, when nothing has run yet) and reports a failed kernel.
int launched(hipStream_t stream)
{
    if (levers().debug_sync) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        if (cs == hipStreamCaptureStatusNone) {
            e = hipStreamSynchronize(stream);
            if (e == hipSuccess)
                e = hipGetLastError();
            if (e != hipSuccess)
                return hip_fail(e, "kernel (checked under W8A16_DEBUG_SYNC)");
        }
    }
    set_last_error("");
    return W8A16_OK;
}

int device_cu_count(int dev, uint32_t *out)
{
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    auto it = g_cu_count.find(dev);
    if (it != g_cu_count.end()) {
        *out = it->second;
        return W8A16_OK;
    }
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute");
    g_cu_count[dev] = (uint32_t)cus;
    *out = (uint32_t)cus;
    return W8A16_OK;
}

// Workspace for `plan` on (dev, stream), grown if needed.  Growth allocates
// new buffers and keeps the old ones alive (calls still in flight, and
// graphs captured earlier, use them), so it needs no synchronisation.  It
// cannot happen while the stream is being captured into a graph: that
// returns W8A16_ERR_WORKSPACE and enqueues nothing.
int get_workspace(int dev, hipStream_t stream, const w8a16_plan_t &plan, Workspace *out)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[std::make_pair(dev, stream)];
    const bool grow_ws = plan.workspace_bytes > w.ws_bytes;
    const bool grow_ctr = plan.counter_count > w.counter_count;
    if (grow_ws || grow_ctr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone) {
            char buf[256];
            snprintf(buf, sizeof buf,
                     "w8a16_gemm: this plan needs %llu bytes of split-K workspace and %u "
                     "counters on a stream being captured, which has %llu and %u; make one "
                     "call with this plan (or a larger one) on the stream before capturing",
                     (unsigned long long)plan.workspace_bytes, plan.counter_count,
                     (unsigned long long)w.ws_bytes, w.counter_count);
            return fail(W8A16_ERR_WORKSPACE, buf);
        }
    }
    hipError_t e;
    if (grow_ws) {
        float *nws = nullptr;
        e = hipMalloc(reinterpret_cast<void **>(&nws), plan.workspace_bytes);
        if (e != hipSuccess)
            return hip_fail(e, "hipMalloc(workspace)");
        if (w.ws)
            g_retired.push_back(w.ws);
        w.ws = nws;
        w.ws_bytes = plan.workspace_bytes;
    }
    if (grow_ctr) {
        uint32_t *nc = nullptr;
        const size_t bytes = (size_t)plan.counter_count * sizeof(uint32_t);
        e = hipMalloc(reinterpret_cast<void **>(&nc), bytes);
        if (e != hipSuccess)
            return hip_fail(e, "hipMalloc(counters)");
        e = hipMemsetAsync(nc, 0, bytes, stream);
        if (e != hipSuccess) {
            (void)hipFree(nc);
            return hip_fail(e, "hipMemsetAsync(counters)");
        }
        if (w.counters)
            g_retired.push_back(w.counters);
        w.counters = nc;
        w.counter_count = plan.counter_count;
    }
    *out = w;
    return W8A16_OK;
}

// ---- scratch of w8a16_gemm_noalloc ---------------------------------------
// One static device array per GPU (each device holds its own copy of the
// code object's globals): FP32 split-K partials, then the arrival counters.
// In host code `scratch` names a host-side stand-in, not device memory; its
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchPartialBytes = (size_t)W8A16_NOALLOC_WORKSPACE_BYTES;
constexpr size_t kScratchCounterWords = (size_t)W8A16_NOALLOC_COUNTERS;
static __device__ __align__(256) uint8_t scratch[kScratchPartialBytes +
                                                 kScratchCounterWords * sizeof(uint32_t)];

__global__ __launch_bounds__(256) void w8a16_zero_words_kernel(uint32_t *p, uint32_t words)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < words)
        p[i] = 0u;
}

std::mutex g_scratch_mutex;
std::map<int, uint8_t *> g_scratch;   // device address of `scratch`, per device

// Device address of this device's scratch, looked up on the first call on
// the device (the current device), which also clears the counters with a
// fill kernel on `stream` (a kernel rather than a memset node, so that a
// graph capturing this first call records a plain kernel).  The counters
// start at zero and every kernel that uses them leaves them at zero.
int device_scratch(int dev, hipStream_t stream, uint8_t **out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *out = it->second;
        return W8A16_OK;
    }
    uint8_t *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&ptr), HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
    const uint32_t words = (uint32_t)kScratchCounterWords;
    hipLaunchKernelGGL(w8a16_zero_words_kernel, dim3((words + 255u) / 256u), dim3(256), 0,
                       stream, reinterpret_cast<uint32_t *>(ptr + kScratchPartialBytes), words);
    e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "scratch counter clear");
    g_scratch[dev] = ptr;
    *out = ptr;
    return W8A16_OK;
}

int check_call(const void *a, uint32_t a_row_stride, const void *w_fp8,
               const float *block_scale, void *c, uint32_t c_row_stride, uint32_t m,
               uint32_t n, uint32_t k)
{
    int st = check_args(m, n, k, a_row_stride, c_row_stride);
    if (st != W8A16_OK)
        return st;
    if (!a || !w_fp8 || !block_scale || !c)
        return fail(W8A16_ERR_NULL_PTR,
                    "w8a16_gemm: a, w_fp8, block_scale and c must be non-null");
    return W8A16_OK;
}

// Enqueue the plan's kernels.  `fixed`: the split-K workspace to use (the
// no-alloc entry's scratch); null takes the (device, stream) workspace.
int run(const char *entry, const char *why, const void *a, uint32_t a_row_stride,
        const void *w_fp8, const float *block_scale, void *c, uint32_t c_row_stride,
        uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t &plan, hipStream_t stream,
        const Workspace *fixed = nullptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    Workspace wsp;
    if (plan.splits > 1) {
        if (fixed) {
            wsp = *fixed;
        } else {
            int st = get_workspace(dev, stream, plan, &wsp);
            if (st != W8A16_OK)
                return st;
        }
    }
    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.a = static_cast<const uint8_t *>(a);
    g.w = static_cast<const uint8_t *>(w_fp8);
    g.scale = block_scale;
    g.c = static_cast<uint8_t *>(c);
    g.ws = wsp.ws;
    g.counters = wsp.counters;
    g.a_stride = a_row_stride;
    g.c_stride = c_row_stride;
    g.m = m;
    g.n = n;
    g.k = k;
    g.m_tiles = plan.m_tiles;
    g.n_tiles = plan.n_tiles;
    g.splits = plan.splits;
    g.steps_per_split = plan.steps_per_split;
    if (plan.kernel == W8A16_KERNEL_STREAM)
        e = launch_stream(g, plan, stream);
    else if (plan.kernel == W8A16_KERNEL_RING)
        e = launch_ring(g, plan, stream);
    else if (plan.n_blocks == kWideNBlocks)
        e = launch_wide(g, plan, stream);
    else
        e = plan.m_blocks == 4 ? launch_tile_m64(g, plan, stream)
                               : launch_tile_m128(g, plan, stream);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    log_plan(entry, m, n, k, plan, why);
    return launched(stream);
}

}  // namespace

}  // namespace w8a16

extern "C" {

int w8a16_gemm(const void *a, uint32_t a_row_stride, const void *w_fp8,
               const float *block_scale, void *c, uint32_t c_row_stride, uint32_t m,
               uint32_t n, uint32_t k, void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_gemm");
    if (st != W8A16_OK)
        return st;
    st = check_call(a, a_row_stride, w_fp8, block_scale, c, c_row_stride, m, n, k);
    if (st != W8A16_OK)
        return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    uint32_t cus = 0;
    st = device_cu_count(dev, &cus);
    if (st != W8A16_OK)
        return st;
    w8a16_plan_t plan;
    st = make_plan(m, n, k, cus, &plan);
    if (st != W8A16_OK)
        return st;
    return run("w8a16_gemm", plan_reason(), a, a_row_stride, w_fp8, block_scale, c,
               c_row_stride, m, n, k, plan, static_cast<hipStream_t>(stream));
}

int w8a16_gemm_planned(const void *a, uint32_t a_row_stride, const void *w_fp8,
                       const float *block_scale, void *c, uint32_t c_row_stride,
                       uint32_t m, uint32_t n, uint32_t k, const w8a16_plan_t *plan,
                       void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_gemm_planned");
    if (st != W8A16_OK)
        return st;
    st = check_call(a, a_row_stride, w_fp8, block_scale, c, c_row_stride, m, n, k);
    if (st != W8A16_OK)
        return st;
    if (!plan)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_gemm_planned: null plan");
    w8a16_plan_t p = *plan;
    st = plan_finalize(m, n, k, &p);
    if (st != W8A16_OK)
        return st;
    if (p.kernel == W8A16_KERNEL_W8A8)
        return fail(W8A16_ERR_BAD_PLAN, "w8a16_gemm_planned: the W8A8 kernel takes FP8 "
                                        "activations (w8a16_gemm_w8a8_planned)");
    return run("w8a16_gemm_planned", nullptr, a, a_row_stride, w_fp8, block_scale, c,
               c_row_stride, m, n, k, p, static_cast<hipStream_t>(stream));
}

int w8a16_gemm_noalloc(const void *a, uint32_t a_row_stride, const void *w_fp8,
                       const float *block_scale, void *c, uint32_t c_row_stride, uint32_t m,
                       uint32_t n, uint32_t k, void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_gemm_noalloc");
    if (st != W8A16_OK)
        return st;
    st = check_call(a, a_row_stride, w_fp8, block_scale, c, c_row_stride, m, n, k);
    if (st != W8A16_OK)
        return fail_with_name(st, "w8a16_gemm_noalloc");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    uint32_t cus = 0;
    st = device_cu_count(dev, &cus);
    if (st != W8A16_OK)
        return st;
    w8a16_plan_t plan;
    st = make_plan(m, n, k, cus, &plan);
    if (st != W8A16_OK)
        return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (plan.splits == 1)
        return run("w8a16_gemm_noalloc", plan_reason(), a, a_row_stride, w_fp8, block_scale,
                   c, c_row_stride, m, n, k, plan, hs);
    if (plan.workspace_bytes > kScratchPartialBytes || plan.counter_count > kScratchCounterWords) {
        char buf[256];
        snprintf(buf, sizeof buf,
                 "w8a16_gemm_noalloc: the plan for m=%u n=%u k=%u needs %llu bytes of split-K "
                 "partials and %u counter words; the scratch holds %llu and %llu",
                 m, n, k, (unsigned long long)plan.workspace_bytes, plan.counter_count,
                 (unsigned long long)kScratchPartialBytes,
                 (unsigned long long)kScratchCounterWords);
        return fail(W8A16_ERR_WORKSPACE, buf);
    }
    uint8_t *ptr = nullptr;
    st = device_scratch(dev, hs, &ptr);
    if (st != W8A16_OK)
        return st;
    Workspace wsp;
    wsp.ws = reinterpret_cast<float *>(ptr);
    wsp.ws_bytes = kScratchPartialBytes;
    wsp.counters = reinterpret_cast<uint32_t *>(ptr + kScratchPartialBytes);
    wsp.counter_count = (uint32_t)kScratchCounterWords;
    return run("w8a16_gemm_noalloc", plan_reason(), a, a_row_stride, w_fp8, block_scale, c,
               c_row_stride, m, n, k, plan, hs, &wsp);
}

int w8a16_act_quant_fp8(const void *a, uint32_t a_row_stride, void *q, uint32_t q_row_stride,
                        float *scales, uint32_t m, uint32_t k, void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_act_quant_fp8");
    if (st != W8A16_OK)
        return st;
    // m, k, the A pitch and its alignment as w8a16_gemm checks them (n = 1
    // stands for the absent output width), then the code pitch.
    st = check_args(m, 1, k, a_row_stride, 1);
    if (st != W8A16_OK)
        return fail_with_name(st, "w8a16_act_quant_fp8");
    char buf[192];
    if (q_row_stride < k) {
        snprintf(buf, sizeof buf,
                 "w8a16_act_quant_fp8: q_row_stride=%u must cover k=%u", q_row_stride, k);
        return fail(W8A16_ERR_PITCH_TOO_SHORT, buf);
    }
    if (q_row_stride % 16 != 0) {
        snprintf(buf, sizeof buf,
                 "w8a16_act_quant_fp8: q_row_stride=%u must keep rows 16B-aligned "
                 "(multiple of 16)", q_row_stride);
        return fail(W8A16_ERR_A_STRIDE_ALIGN, buf);
    }
    if (!a || !q || !scales)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_act_quant_fp8: a, q and scales must be non-null");
    QuantArgs qa;
    qa.a = static_cast<const uint8_t *>(a);
    qa.q = static_cast<uint8_t *>(q);
    qa.scales = scales;
    qa.a_stride = a_row_stride;
    qa.q_stride = q_row_stride;
    qa.m = m;
    qa.k = k;
    hipError_t e = launch_act_quant(qa, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    if (levers().log) {
        snprintf(buf, sizeof buf,
                 "w8a16: w8a16_act_quant_fp8 m=%u k=%u: per-token FP8 quantizer, one group of "
                 "128 K elements per scale\n", m, k);
        log_line(buf);
    }
    return launched(static_cast<hipStream_t>(stream));
}

int w8a16_gemm_w8a8_planned(const void *qa, uint32_t qa_row_stride, const float *a_scales,
                            const void *w_fp8, const float *block_scale, void *c,
                            uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k,
                            const w8a16_plan_t *plan, void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_gemm_w8a8");
    if (st != W8A16_OK)
        return st;
    st = check_call(qa, qa_row_stride, w_fp8, block_scale, c, c_row_stride, m, n, k);
    if (st != W8A16_OK)
        return st;
    if (qa_row_stride % 16 != 0) {
        char buf[160];
        snprintf(buf, sizeof buf,
                 "w8a16_gemm_w8a8: qa_row_stride=%u must keep FP8 rows 16B-aligned "
                 "(multiple of 16)", qa_row_stride);
        return fail(W8A16_ERR_A_STRIDE_ALIGN, buf);
    }
    if (!a_scales)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_gemm_w8a8: a_scales must be non-null");
    w8a16_plan_t p;
    if (plan) {
        p = *plan;
        st = plan_finalize(m, n, k, &p);
        if (st != W8A16_OK)
            return st;
        if (p.kernel != W8A16_KERNEL_W8A8)
            return fail(W8A16_ERR_BAD_PLAN, "w8a16_gemm_w8a8: plan kernel must be "
                                            "W8A16_KERNEL_W8A8");
    } else {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return hip_fail(e, "hipGetDevice");
        uint32_t cus = 0;
        st = device_cu_count(dev, &cus);
        if (st != W8A16_OK)
            return st;
        st = make_plan_w8a8(m, n, k, cus, &p);
        if (st != W8A16_OK)
            return st;
    }
    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.a = static_cast<const uint8_t *>(qa);
    g.w = static_cast<const uint8_t *>(w_fp8);
    g.scale = block_scale;
    g.c = static_cast<uint8_t *>(c);
    g.a_stride = qa_row_stride;
    g.c_stride = c_row_stride;
    g.m = m;
    g.n = n;
    g.k = k;
    g.m_tiles = p.m_tiles;
    g.n_tiles = p.n_tiles;
    g.splits = 1;
    g.steps_per_split = k / kKStep;
    hipError_t e = launch_w8a8(g, a_scales, p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    log_plan(plan ? "w8a16_gemm_w8a8_planned" : "w8a16_gemm_w8a8", m, n, k, p,
             plan ? nullptr : plan_reason());
    return launched(static_cast<hipStream_t>(stream));
}

int w8a16_gemm_w8a8(const void *qa, uint32_t qa_row_stride, const float *a_scales,
                    const void *w_fp8, const float *block_scale, void *c,
                    uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    return w8a16_gemm_w8a8_planned(qa, qa_row_stride, a_scales, w_fp8, block_scale, c,
                                   c_row_stride, m, n, k, nullptr, stream);
}

int w8a16_gemm_w4a4_planned(const void *a, uint32_t a_row_stride, const uint8_t *a_scale,
                            const void *w_fp4, const uint8_t *w_scale, void *c,
                            uint32_t c_row_stride, uint32_t m, uint32_t n, uint32_t k,
                            const w8a16_plan_t *plan, void *stream)
{
    using namespace w8a16;
    int st = check_levers("w8a16_gemm_w4a4");
    if (st != W8A16_OK)
        return st;
    st = check_args_w4a4(m, n, k, a_row_stride, c_row_stride);
    if (st != W8A16_OK)
        return st;
    if (!a || !a_scale || !w_fp4 || !w_scale || !c)
        return fail(W8A16_ERR_NULL_PTR,
                    "w8a16_gemm_w4a4: a, a_scale, w_fp4, w_scale and c must be non-null");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    w8a16_plan_t p;
    if (plan) {
        p = *plan;
        st = plan_finalize(m, n, k, &p);
        if (st != W8A16_OK)
            return st;
        if (p.kernel != W8A16_KERNEL_W4A4 && p.kernel != W8A16_KERNEL_W4A4_PS)
            return fail(W8A16_ERR_BAD_PLAN, "w8a16_gemm_w4a4: plan kernel must be "
                                            "W8A16_KERNEL_W4A4 or W8A16_KERNEL_W4A4_PS");
    } else {
        uint32_t cus = 0;
        st = device_cu_count(dev, &cus);
        if (st != W8A16_OK)
            return st;
        st = make_plan_w4a4(m, n, k, cus, &p);
        if (st != W8A16_OK)
            return st;
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    MxArgs g;
    std::memset(&g, 0, sizeof g);
    g.a = static_cast<const uint8_t *>(a);
    g.a_scale = a_scale;
    g.w = static_cast<const uint8_t *>(w_fp4);
    g.w_scale = w_scale;
    g.c = static_cast<uint8_t *>(c);
    g.a_stride = a_row_stride / 2u;
    g.c_stride = c_row_stride;
    g.m = m;
    g.n = n;
    g.k = k;
    g.m_tiles = p.m_tiles;
    g.n_tiles = p.n_tiles;
    g.tiles_base = (n + 15u) / 16u / p.grid;
    g.tiles_extra = (n + 15u) / 16u % p.grid;
    e = launch_w4a4(g, p, hs);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    log_plan(plan ? "w8a16_gemm_w4a4_planned" : "w8a16_gemm_w4a4", m, n, k, p,
             plan ? nullptr : plan_reason());
    return launched(hs);
}

int w8a16_gemm_w4a4(const void *a, uint32_t a_row_stride, const uint8_t *a_scale,
                    const void *w_fp4, const uint8_t *w_scale, void *c, uint32_t c_row_stride,
                    uint32_t m, uint32_t n, uint32_t k, void *stream)
{
    return w8a16_gemm_w4a4_planned(a, a_row_stride, a_scale, w_fp4, w_scale, c, c_row_stride,
                                   m, n, k, nullptr, stream);
}

int w8a16_gemm_batched(const w8a16_gemm_desc_t *descs, uint32_t count, void *stream)
{
    using namespace w8a16;
    if (check_levers("w8a16_gemm_batched") != W8A16_OK)
        return W8A16_ERR_ENV;
    if (!descs)
        return fail(W8A16_ERR_NULL_PTR, "w8a16_gemm_batched: null descriptors");
    if (count < 1 || count > W8A16_MAX_BATCH) {
        char buf[128];
        snprintf(buf, sizeof buf, "w8a16_gemm_batched: count=%u must be in 1..%u", count,
                 (unsigned)W8A16_MAX_BATCH);
        return fail(W8A16_ERR_BAD_PLAN, buf);
    }
    for (uint32_t i = 0; i < count; ++i) {
        const w8a16_gemm_desc_t &d = descs[i];
        int st = check_call(d.a, d.a_row_stride, d.w_fp8, d.block_scale, d.c, d.c_row_stride,
                            d.m, d.n, d.k);
        if (st != W8A16_OK)
            return fail_at(st, i);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    uint32_t cus = 0;
    int st = device_cu_count(dev, &cus);
    if (st != W8A16_OK)
        return st;
    w8a16_plan_t plan;
    st = plan_batched(descs, count, cus, &plan);
    if (st != W8A16_OK)
        return st;
    BatchArgs b;
    std::memset(&b, 0, sizeof b);
    b.count = count;
    uint32_t start = 0;
    for (uint32_t i = 0; i < count; ++i) {
        const w8a16_gemm_desc_t &d = descs[i];
        GemmArgs &g = b.g[i];
        g.a = static_cast<const uint8_t *>(d.a);
        g.w = static_cast<const uint8_t *>(d.w_fp8);
        g.scale = d.block_scale;
        g.c = static_cast<uint8_t *>(d.c);
        g.ws = nullptr;
        g.counters = nullptr;
        g.a_stride = d.a_row_stride;
        g.c_stride = d.c_row_stride;
        g.m = d.m;
        g.n = d.n;
        g.k = d.k;
        g.m_tiles = (d.m + 16 * plan.m_blocks - 1) / (16 * plan.m_blocks);
        g.n_tiles = (d.n + 16 * plan.n_blocks - 1) / (16 * plan.n_blocks);
        g.splits = 1;
        g.steps_per_split = d.k / kKStep;
        b.start[i] = start;
        start += g.m_tiles * g.n_tiles;
    }
    if (start != plan.grid)
        return fail(W8A16_ERR_BAD_PLAN, "w8a16_gemm_batched: inconsistent grid");
    e = launch_stream_batched(b, plan, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    if (levers().log) {
        char entry[64];
        snprintf(entry, sizeof entry, "w8a16_gemm_batched (%u problems, the first)", count);
        log_plan(entry, descs[0].m, descs[0].n, descs[0].k, plan, plan_reason());
    }
    return launched(static_cast<hipStream_t>(stream));
}

}  // extern "C"
