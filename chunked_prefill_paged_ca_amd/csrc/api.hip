// api.hip -- the C ABI entry points: context, workspace, metadata upload, validation, dispatch.
//
// Host runtime around the kernels.  A step's plan is plain host data; the first device call
// that sees a new plan generation copies its metadata once (pinned staging -> device, async on
// the caller's stream), and later calls with the same generation reuse the device copy.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "internal.h"

namespace ca {

namespace {
thread_local std::string t_last_error;
}

void set_error(const std::string& msg) { t_last_error = msg; }
void clear_error() { t_last_error.clear(); }

}  // namespace ca

using ca::DevPlan;
using ca::Shape;

namespace ca {
// Size of the static scratch array of ca_mixed_attention_noalloc.
constexpr size_t kScratchBytes = size_t(64) << 20;
}  // namespace ca

// Workspace of ca_mixed_attention_noalloc: the step's metadata and split-KV partials.  One copy
// per device, held from the library's first use on that device until the process ends, shared
// by every no-alloc call on the device.  Host code never names it in device work: its device
// address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) char scratch[ca::kScratchBytes];

namespace {

// Device address of `scratch` per device, looked up once per device (with that device current).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int device, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

namespace {

// Device buffer grown on demand.  Growth waits for the stream first, because kernels enqueued
// earlier may still read the old allocation.
struct DevBuf {
    void* ptr = nullptr;
    size_t bytes = 0;
    hipError_t reserve(size_t want, hipStream_t stream) {
        if (want <= bytes) return hipSuccess;
        if (ptr) {
            hipError_t e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return e;
            e = hipFree(ptr);
            if (e != hipSuccess) return e;
            ptr = nullptr;
            bytes = 0;
        }
        // doubling with a 1 MiB floor: a serving loop whose plans grow over time reallocates
        // (a stream synchronisation plus hipFree/hipMalloc) only a few times
        size_t cap = want * 2 > (size_t(1) << 20) ? want * 2 : (size_t(1) << 20);
        hipError_t e = hipMalloc(&ptr, cap);
        if (e != hipSuccess) { ptr = nullptr; return e; }
        bytes = cap;
        return hipSuccess;
    }
    void release() {
        if (ptr) (void)hipFree(ptr);
        ptr = nullptr;
        bytes = 0;
    }
};

// Copies the staged metadata into device memory.  The staging slots are pinned, device-mapped,
// coherent host memory, so a kernel can read them directly: the upload then runs on the compute
// queue in stream order, with no copy-engine hand-off between it and the kernels that read it.
__global__ void __launch_bounds__(256) upload_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] = src[i];
}

// Ring of pinned host staging slots.  A slot is reused only after the launch that read it (the
// upload kernel, or an append launch that copies the slot itself) has completed, so the host
// never overwrites bytes the device still needs.  Completion is reported by the attention launch
// that follows the reader on the same stream: its first thread stores the slot's generation into
// `done` (pinned host memory) as it starts, which by stream order is after the reader finished.
// No event goes into the stream (an event is a marker that delays the next kernel by a few
// microseconds).  A slot whose reader was followed by no reporting launch (a different stream,
// no attention call) is waited for with a device synchronisation when the ring comes back to it.
struct Staging {
    static constexpr int kSlots = 8;
    void* host[kSlots] = {};
    void* dev[kSlots] = {};  // the same memory as the device addresses it
    size_t cap[kSlots] = {};
    uint32_t* done_host = nullptr;  // [kSlots]: generation of the slot's last reader known finished
    uint32_t* done_dev = nullptr;   // the same memory as the device addresses it
    uint32_t gen[kSlots] = {};      // generation of the slot's current contents
    bool busy[kSlots] = {};         // a reader was enqueued and is not known to have finished
    bool reported[kSlots] = {};     // a launch that reports the reader's end was enqueued after it
    int last = -1;                  // the slot of the latest reader, not yet reported
    hipStream_t last_stream = nullptr;
    int next = 0;

    // Every slot is allocated here, at context creation, with kInitialBytes (enough for the
    // metadata of a step of several thousand sequences and ~250 K pages), so that a steady
    // stream of steps never allocates: a slot grows (doubling) only for a plan larger than that.
    static constexpr size_t kInitialBytes = size_t(2) << 20;
    hipError_t init() {
        hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&done_host), kSlots * sizeof(uint32_t),
                                     hipHostMallocMapped | hipHostMallocCoherent);
        if (e != hipSuccess) { done_host = nullptr; return e; }
        for (int i = 0; i < kSlots; ++i) done_host[i] = 0;
        e = hipHostGetDevicePointer(reinterpret_cast<void**>(&done_dev), done_host, 0);
        if (e != hipSuccess) return e;
        for (int i = 0; i < kSlots; ++i) {
            e = grow(i, kInitialBytes);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    hipError_t grow(int i, size_t want) {
        if (host[i]) (void)hipHostFree(host[i]);
        host[i] = nullptr;
        dev[i] = nullptr;
        cap[i] = 0;
        hipError_t e = hipHostMalloc(&host[i], want, hipHostMallocMapped | hipHostMallocCoherent);
        if (e != hipSuccess) { host[i] = nullptr; return e; }
        e = hipHostGetDevicePointer(&dev[i], host[i], 0);
        if (e != hipSuccess) {
            (void)hipHostFree(host[i]);
            host[i] = nullptr;
            dev[i] = nullptr;
            return e;
        }
        cap[i] = want;
        return hipSuccess;
    }
    // Wait until the last reader of slot i has finished.
    hipError_t wait_done(int i) {
        if (!busy[i]) return hipSuccess;
        if (reported[i]) {
            // the reporting launch is in the stream after the reader: its store arrives as the
            // stream gets there (after a second, wait for the device and look once more)
            const auto t0 = std::chrono::steady_clock::now();
            while (__atomic_load_n(&done_host[i], __ATOMIC_ACQUIRE) != gen[i]) {
                if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(1)) {
                    hipError_t e = hipDeviceSynchronize();
                    if (e != hipSuccess) return e;
                    if (__atomic_load_n(&done_host[i], __ATOMIC_ACQUIRE) != gen[i]) return hipErrorUnknown;
                    break;
                }
                std::this_thread::yield();
            }
        } else {
            hipError_t e = hipDeviceSynchronize();  // no report follows the reader
            if (e != hipSuccess) return e;
            if (last == i) last = -1;
        }
        busy[i] = false;
        reported[i] = false;
        return hipSuccess;
    }
    // The next slot of the ring, once the upload that last read it has completed.  With
    // may_grow false a plan larger than the slot is refused (*slot = -1) instead of allocating.
    hipError_t acquire(size_t bytes, int* slot, bool may_grow = true) {
        *slot = -1;
        const int i = next;
        if (cap[i] < bytes && !may_grow) return hipSuccess;
        next = (next + 1) % kSlots;
        hipError_t e = wait_done(i);
        if (e != hipSuccess) return e;
        ++gen[i];
        if (cap[i] < bytes) {
            hipError_t e = grow(i, bytes * 2);  // doubling, see DevBuf
            if (e != hipSuccess) return e;
        }
        *slot = i;
        return hipSuccess;
    }
    // bytes: a multiple of 16 within the slot's capacity
    hipError_t upload(int slot, void* dst, size_t bytes, hipStream_t stream,
                      const ca::LaunchEvents& timing) {
        const int64_t n = static_cast<int64_t>(bytes / 16);
        const int64_t blocks = (n + 255) / 256;
        const dim3 grid(static_cast<unsigned>(blocks < 256 ? (blocks > 0 ? blocks : 1) : 256));
        hipExtLaunchKernelGGL(upload_kernel, grid, dim3(256), 0, stream, timing.start, timing.stop, 0,
                              static_cast<const uint4*>(dev[slot]), static_cast<uint4*>(dst), n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return mark_read(slot, stream);
    }
    // After the launch that reads `slot` has been enqueued on `stream` (the upload kernel, or an
    // append launch that copies the slot itself).
    hipError_t mark_read(int slot, hipStream_t stream) {
        busy[slot] = true;
        reported[slot] = false;
        last = slot;
        last_stream = stream;
        return hipSuccess;
    }
    // For an attention launch about to be enqueued on `stream`: the report it should store (the
    // latest reader's slot, when that reader was enqueued on the same stream), in p.
    int report_into(ca::DevPlan& p, hipStream_t stream) const {
        p.done_flag = nullptr;
        p.done_value = 0;
        if (last < 0 || last_stream != stream) return -1;
        p.done_flag = done_dev + last;
        p.done_value = gen[last];
        return last;
    }
    // The launch carrying slot's report has been enqueued.
    void reported_by_launch(int slot) {
        if (slot < 0) return;
        reported[slot] = true;
        if (last == slot) last = -1;
    }
    void release() {
        bool any = false;
        for (int i = 0; i < kSlots; ++i) any = any || busy[i];
        if (any) (void)hipDeviceSynchronize();
        for (int i = 0; i < kSlots; ++i) {
            if (host[i]) (void)hipHostFree(host[i]);
            host[i] = nullptr;
            dev[i] = nullptr;
            busy[i] = reported[i] = false;
        }
        if (done_host) (void)hipHostFree(done_host);
        done_host = nullptr;
        done_dev = nullptr;
        last = -1;
    }
};

}  // namespace

// Work lists of one attention call, built on the host from the plan: decode splits and their
// merges, chunk workgroups and their merges (split = decode shares, csplit = keys per chunk
// split).
struct WorkKey {
    uint64_t generation = 0;
    int32_t hq = 0, hkv = 0, d = 0, split = 0, csplit = 0;
    double theta = 0.0;
    bool operator==(const WorkKey& o) const {
        return generation == o.generation && hq == o.hq && hkv == o.hkv && d == o.d &&
               split == o.split && csplit == o.csplit && theta == o.theta;
    }
};

struct DevWork {
    const int4* dec_items = nullptr;          // two int4 per decode item
    const int32_t* dec_wave_items = nullptr;  // [num_dec_waves + 1] first item of each wave
    const int4* merges = nullptr;
    const int4* chunk_items = nullptr;   // two int4 per workgroup
    const int4* chunk_groups = nullptr;  // two int4 per multi-split row block
    int32_t num_dec_items = 0, num_dec_waves = 0, num_merges = 0, num_slots = 0;
    int32_t dec_wgs = 0;  // decode workgroups of the attention launch
    int32_t dec_wpg = 0;  // decode wavefronts per decode workgroup
    int32_t num_chunk_items = 0, num_chunk_groups = 0, num_chunk_slots = 0;
    int32_t num_chunk_workers = 0;  // chunk workgroups of the attention launch
    int32_t num_chunk_static = 0;   // of those, the ones that start with the launch
    bool chunk_queue_mode = false;  // workers take items from queues (else one item each)
};

// Event pairs around the library's own launches (ca_profile_enable).
struct Profiler {
    struct Rec {
        const char* name;
        hipEvent_t a, b;
    };
    int mask = 0;  // CA_PROFILE_* kinds being timed (0: off)
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    hipEvent_t get(bool may_create = true) {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        if (!may_create) return nullptr;
        // Timing events carry no system-scope fence: they only stamp times and are never used
        // to make device memory visible to the host (a fenced event writes back and invalidates
        // the caches around the timed launch, a few microseconds each time).
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        ++created;
        return e;
    }
    // Create events ahead of use (when timing is switched on), so that timed launches draw them
    // from the pool instead of creating them between steps.
    static constexpr size_t kReserve = 512;  // 256 timed launches between two reads
    size_t created = 0;
    void reserve() {
        while (created < kReserve) {
            hipEvent_t e = nullptr;
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
            pool.push_back(e);
            ++created;
        }
    }
    void release() {
        for (auto& r : pending) {
            (void)hipEventDestroy(r.a);
            (void)hipEventDestroy(r.b);
        }
        for (auto e : pool) (void)hipEventDestroy(e);
        pending.clear();
        pool.clear();
        created = 0;
    }
};

// Timing of one library call when profiling is on: a start/stop event pair handed to the
// launcher, which attaches it to the call's kernels (LaunchEvents).  commit() after a successful
// launch files the record; otherwise the events go back to the pool unrecorded.
struct Timed {
    Profiler& pf;
    const char* name;
    ca::LaunchEvents ev{};
    bool committed = false;
    // may_create false: events only from the pool created ahead (ca_profile_enable); an empty
    // pool leaves the launch untimed
    Timed(Profiler& p, const char* n, int kind, bool may_create = true) : pf(p), name(n) {
        if ((pf.mask & kind) && pf.pending.size() < 65536) {
            ev.start = pf.get(may_create);
            ev.stop = pf.get(may_create);
            if (!ev.start || !ev.stop) {
                if (ev.start) pf.pool.push_back(ev.start);
                if (ev.stop) pf.pool.push_back(ev.stop);
                ev = ca::LaunchEvents{};
            }
        }
    }
    void commit() {
        if (ev.start) {
            pf.pending.push_back({name, ev.start, ev.stop});
            committed = true;
        }
    }
    ~Timed() {
        if (ev.start && !committed) {
            pf.pool.push_back(ev.start);
            pf.pool.push_back(ev.stop);
        }
    }
};

// Decode wavefronts per decode workgroup (one workgroup per CU, so one decode wave per SIMD).
// Measured on the part (same box, attention launch): the Mistral-7B and LLaMA2-70B steps take
// the same time with 4 or 8 decode waves per CU (the HBM stream rate does not depend on it); the
// chunk-heavy Yi-34B step is 4 % faster with 4.  A per-wave timeline also showed that a SIMD's
// older wave gets most of the SIMD's share of the memory pipe (equal shares ended 40 % apart
// with 8 waves per CU).
constexpr int32_t kDecodeWavesPerWg = 4;

struct ca_ctx {
    int device = 0;
    Profiler prof;
    Staging staging;
    DevBuf meta_buf;        // one upload per step: plan metadata, then the work lists
    // two sets of chunk work-queue counters, used by turns: the attention launch claims from
    // set queue_parity and zeroes the other, which the next queue-mode launch uses
    int* queue = nullptr;
    int32_t queue_parity = 0;
    DevPlan dplan{};
    const double* inv_freq = nullptr;  // [d / 2] rotary inverse frequencies of the current shape
    // one device table of inverse frequencies per (head dim, rotary base), filled once and kept
    // (a table may still be read by an earlier launch when another shape comes along)
    std::map<std::pair<int32_t, double>, void*> freq_tables;
    // Set by prepare(..., defer = true): the step's metadata sits in staging slot `defer_slot`
    // (defer_bytes) and has not been copied to meta_buf yet; hrow_pos / hrow_page are its per-row
    // arrays as the device sees the staging.  The next append launch copies it.
    int defer_slot = -1;
    size_t defer_bytes = 0;
    const int32_t* hrow_pos = nullptr;
    const int32_t* hrow_page = nullptr;
    DevBuf partial_buf;     // fp32 split-KV partials of the generic path
    WorkKey work_key{};     // what meta_buf holds (generation 0: nothing)
    DevWork dwork{};
    DevBuf dec_acc_buf;     // fp32 [slots][G][d]
    DevBuf dec_ml_buf;      // float2 [slots][G]
    DevBuf chk_acc_buf;     // fp32 [slots][cols][d]
    DevBuf chk_ml_buf;      // float2 [slots][cols]
    int32_t num_cus = 0;
    int32_t attn_wgs_per_cu[2] = {0, 0};  // d = 64, d = 128 (queried on first use)
    int32_t dec_wgs_override = 0;  // CA_DECODE_WGS: decode workgroups of an attention launch, 0 = auto
    int32_t dec_wpg = kDecodeWavesPerWg;  // CA_DECODE_WAVES: decode wavefronts per workgroup
    bool split_attention = false;  // CA_SPLIT_ATTENTION=1: decode and chunk as two launches
    int32_t csplit_override = 0;  // CA_CHUNK_SPLIT (keys per chunk split), 0 = automatic
    ca::Linear* linear = nullptr;  // hipBLASLt state of ca_qkv_projection (created on first use)
    DevBuf proj_part;              // fp32 K-split partials of the tiled projection
    int32_t proj_tile[3] = {0, 0, 0};  // CA_PROJECTION_TILE=bm,bn,split: tile shape of the tiled projection
    bool projection_library = false;  // CA_PROJECTION_LIBRARY=1: the library GEMM for every T
    // CA_DEBUG_VALIDATE=1: the append also checks that no two scheduled tokens write the same
    // (page, slot) (a sort of the step's write targets on the host).
    bool debug_validate = false;
    int32_t work_max_page = -1;     // largest page id of the plan meta_buf holds
    bool work_targets_checked = false;  // its write targets were checked
    // split partials of the current step (the growable buffers, or the static scratch array)
    float* dacc = nullptr;
    float2* dml = nullptr;
    float* cacc = nullptr;
    float2* cml = nullptr;
    void* scratch = nullptr;  // device address of the static scratch array on this ctx's device
    size_t meta_end = 0;      // bytes of the scratch the current metadata takes
    // host-side work lists of prepare(), kept so that a steady stream of steps reuses them
    std::vector<int4> items, merges, citems, groups, clist;
    std::vector<int32_t> corder;
    std::vector<int64_t> share_bounds;  // decode share boundaries of the last work lists
    int32_t chunk_workers = 0, chunk_static = 0;  // the chunk workers of the last work lists
    bool chunk_queue_mode = false;
    std::vector<int32_t> wave_items;
};

namespace {

ca_status device_error(const char* what, hipError_t e) {
    ca::set_error(std::string(what) + ": " + hipGetErrorString(e));
    return CA_ERR_DEVICE;
}

// Guard that makes ctx->device current for the duration of a call and restores the caller's.
struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

bool aligned16(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
    return true;
}

ca_status check_plan(const ca_plan* plan) {
    if (!plan) { ca::set_error("null plan"); return CA_ERR_INVALID_ARG; }
    if (plan->num_seqs < 0 || plan->num_tokens < 0 || plan->num_pages < 0 ||
        plan->num_decodes < 0 || plan->num_decodes > plan->num_seqs) {
        ca::set_error("plan counts are inconsistent");
        return CA_ERR_INVALID_ARG;
    }
    if (plan->num_seqs > 0 && (!plan->qo_indptr || !plan->kv_page_indptr ||
                               !plan->kv_last_page_len || !plan->kv_page_indices)) {
        ca::set_error("plan arrays are null");
        return CA_ERR_INVALID_ARG;
    }
    return CA_OK;
}

ca_status check_desc(const ca_attn_desc* d, const ca_plan* plan, Shape* sh) {
    if (!d) { ca::set_error("null descriptor"); return CA_ERR_INVALID_ARG; }
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0) {
        ca::set_error("num_q_heads must be a positive multiple of num_kv_heads");
        return CA_ERR_INVALID_ARG;
    }
    if (d->page_size <= 0 || d->page_size != plan->page_size) {
        ca::set_error("descriptor page_size must match the plan's");
        return CA_ERR_INVALID_ARG;
    }
    if (d->dtype != CA_BF16 && d->dtype != CA_FP32) {
        ca::set_error("unknown dtype");
        return CA_ERR_INVALID_ARG;
    }
    if (d->head_dim != 64 && d->head_dim != 128) {
        ca::set_error("head_dim must be 64 or 128");
        return CA_ERR_UNSUPPORTED;
    }
    if (d->page_size != 16) {
        ca::set_error("page_size must be 16");
        return CA_ERR_UNSUPPORTED;
    }
    if (!(d->sm_scale >= 0.0f) || !std::isfinite(d->sm_scale) || !(d->rope_theta >= 0.0f)) {
        ca::set_error("sm_scale and rope_theta must be finite and >= 0");
        return CA_ERR_INVALID_ARG;
    }
    sh->hq = d->num_q_heads;
    sh->hkv = d->num_kv_heads;
    sh->d = d->head_dim;
    sh->P = d->page_size;
    sh->scale = d->sm_scale > 0.0f ? d->sm_scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
    sh->theta = d->rope_theta > 0.0f ? static_cast<double>(d->rope_theta) : 10000.0;
    sh->dtype = d->dtype;
    return CA_OK;
}

// Host-side consistency of the plan arrays against the pool (they are read by the kernels, so
// every index is checked here before a launch).  *max_page receives the largest page id the plan
// names.  With write_targets, the (page, slot) every scheduled token is appended to must also be
// unique over the whole step: two sequences (or two positions of one sequence) that would write
// the same slot are a block-table error the append kernel cannot see -- its workgroups would race
// on that slot -- and the block table must stay consistent across appends (pinghaoyang.com.cn
// "Sarathi-Serve 完全拆解", section "先验证数值与状态正确性").
// The structural part: counts, indptr totals, per-sequence lengths.
ca_status validate_plan_structure(const ca_plan* plan) {
    const int32_t ns = plan->num_seqs;
    const int32_t P = plan->page_size;
    if (ns == 0) return CA_OK;
    if (P <= 0) {
        ca::set_error("plan page_size must be > 0");
        return CA_ERR_INVALID_ARG;
    }
    if (plan->qo_indptr[0] != 0 || plan->kv_page_indptr[0] != 0) {
        ca::set_error("indptr arrays must start at 0");
        return CA_ERR_INVALID_ARG;
    }
    for (int32_t s = 0; s < ns; ++s) {
        const int32_t q = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t last = plan->kv_last_page_len[s];
        if (q < 1 || np < 1 || last < 1 || last > P) {
            ca::set_error("sequence " + std::to_string(s) + ": empty rows/pages or bad last-page length");
            return CA_ERR_INVALID_ARG;
        }
        const int64_t kv_len = static_cast<int64_t>(np - 1) * P + last;
        if (kv_len < q) {
            ca::set_error("sequence " + std::to_string(s) + ": more rows than keys");
            return CA_ERR_INVALID_ARG;
        }
        if (s < plan->num_decodes && q != 1) {
            ca::set_error("decode sequence " + std::to_string(s) + " must have exactly one row");
            return CA_ERR_INVALID_ARG;
        }
    }
    if (plan->qo_indptr[ns] != plan->num_tokens || plan->kv_page_indptr[ns] != plan->num_pages) {
        ca::set_error("indptr totals disagree with num_tokens / num_pages");
        return CA_ERR_INVALID_ARG;
    }
    return CA_OK;
}

// The page ids against the pool, in one branch-free pass (it vectorises) that also copies them to
// `copy` when given (the staging slot: one read of the ids instead of two); the offending id is
// looked for only when the range is out of the pool.  *max_page: the largest id.
ca_status check_page_range(const ca_plan* plan, int64_t pool, int32_t* copy, int32_t* max_page) {
    int32_t lo = 0x7fffffff, top = -1;
    const int32_t* ids = plan->kv_page_indices;
    const int32_t n = plan->num_pages;
    if (copy) {
        for (int32_t j = 0; j < n; ++j) {
            const int32_t v = ids[j];
            copy[j] = v;
            lo = v < lo ? v : lo;
            top = v > top ? v : top;
        }
    } else {
        for (int32_t j = 0; j < n; ++j) {
            const int32_t v = ids[j];
            lo = v < lo ? v : lo;
            top = v > top ? v : top;
        }
    }
    *max_page = top;
    if (n > 0 && (lo < 0 || top >= pool)) {
        for (int32_t j = 0; j < n; ++j) {
            if (ids[j] < 0 || ids[j] >= pool) {
                ca::set_error("page index " + std::to_string(ids[j]) + " outside the pool");
                return CA_ERR_INVALID_ARG;
            }
        }
    }
    return CA_OK;
}

// The (page, slot) write targets of the step's tokens are unique (see validate_plan_arrays).
ca_status check_write_targets(const ca_plan* plan) {
    const int32_t ns = plan->num_seqs;
    const int32_t P = plan->page_size;
    std::vector<std::pair<int64_t, int32_t>> t;  // (page * P + slot, sequence)
    t.reserve(static_cast<size_t>(plan->num_tokens));
    for (int32_t s = 0; s < ns; ++s) {
        const int32_t q = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
        const int32_t p0 = plan->kv_page_indptr[s];
        const int32_t kv_len = (plan->kv_page_indptr[s + 1] - p0 - 1) * P + plan->kv_last_page_len[s];
        for (int32_t pos = kv_len - q; pos < kv_len; ++pos)
            t.emplace_back(static_cast<int64_t>(plan->kv_page_indices[p0 + pos / P]) * P + pos % P, s);
    }
    std::sort(t.begin(), t.end());
    for (size_t i = 1; i < t.size(); ++i) {
        if (t[i].first == t[i - 1].first) {
            ca::set_error("sequences " + std::to_string(t[i - 1].second) + " and " +
                          std::to_string(t[i].second) + " both append to page " +
                          std::to_string(t[i].first / P) + " slot " + std::to_string(t[i].first % P));
            return CA_ERR_INVALID_ARG;
        }
    }
    return CA_OK;
}

ca_status validate_plan_arrays(const ca_plan* plan, int64_t pool, bool write_targets,
                               int32_t* max_page) {
    *max_page = -1;
    if (plan->num_seqs == 0) return CA_OK;
    ca_status st = validate_plan_structure(plan);
    if (st == CA_OK) st = check_page_range(plan, pool, nullptr, max_page);
    if (st == CA_OK && write_targets) st = check_write_targets(plan);
    return st;
}

// Share of the CUs the decode rows get when they share the attention launch with chunk rows:
// each part in proportion to the CU-time it needs -- the decode stream the whole device for
// dec_us (its K/V bytes at kDecodeStreamBps), the chunk rows kChunkBlockUs per 32-key block of a
// column block -- within [kMinDecodeShare, kMaxDecodeShare].  Measured on the part (4 decode waves
// per workgroup, sweeps of the decode workgroups on several boxes): the Mistral-7B step is
// fastest at 3/4 of the CUs and the LLaMA2-70B step at 5/8-3/4 (both decode-heavy: the proportion
// is ~0.8 and clamps to 3/4), the chunk-heavy Yi-34B step at 5/16-3/8 (proportion ~0.26), where it
// ran 580-588 us against 595-642 us at 3/4 and fell off a cliff below 5/16 (the decode stream
// becomes the tail).
constexpr double kMaxDecodeShare = 0.75;
constexpr double kMinDecodeShare = 0.3125;
constexpr double kDecodeStreamBps = 6.3e12;  // decode K/V read rate the estimates assume
double chunk_block_us(const Shape& sh) { return sh.d == 128 ? 1.3 : 0.67; }

// Decode K/V stream time (us) and chunk CU-time (CU-us) of a plan, as the launch-shaping rules
// estimate them.
void mixed_work(const ca_plan* plan, const Shape& sh, double* dec_us, double* chunk_cu_us) {
    const int32_t G = sh.hq / sh.hkv;
    const int32_t cols = ca::chunk_cols_per_block();
    int64_t dec_keys = 0, chunk_keys = 0;
    for (int32_t s = 0; s < plan->num_seqs; ++s) {
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
        if (s < plan->num_decodes) {
            dec_keys += kv_len;
            continue;
        }
        const int32_t q_len = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
        for (int32_t cb = 0; cb < q_len * G; cb += cols) {
            const int32_t last = (cb + cols < q_len * G ? cb + cols : q_len * G) - 1;
            chunk_keys += kv_len - q_len + last / G + 1;
        }
    }
    *dec_us = static_cast<double>(dec_keys) * sh.hkv * sh.d * 4 / kDecodeStreamBps * 1e6;  // K + V, bf16
    *chunk_cu_us = static_cast<double>(chunk_keys) * sh.hkv / 32 * chunk_block_us(sh);
}

double mixed_decode_share(const ca_ctx* ctx, const ca_plan* plan, const Shape& sh) {
    double dec_us = 0, chunk_cu_us = 0;
    mixed_work(plan, sh, &dec_us, &chunk_cu_us);
    const double dec_cu_us = dec_us * ctx->num_cus;
    if (dec_cu_us <= 0) return kMaxDecodeShare;
    const double f = dec_cu_us / (dec_cu_us + chunk_cu_us);
    return f < kMinDecodeShare ? kMinDecodeShare : (f > kMaxDecodeShare ? kMaxDecodeShare : f);
}

// Decode workgroups of the attention launch and decode shares.  The 32-key blocks of every
// (decode row, kv head), laid end to end, are cut into one equal share per decode wavefront, so a
// single round of waves streams the whole decode K/V with no tail.  Alone (no chunk rows, or the
// two parts launched separately) decode takes every workgroup slot of the device; in a mixed
// launch it takes mixed_decode_share of them (rounded to whole XCD rounds of 8) and the chunk
// workgroups run beside it.  CA_DECODE_WGS sets the count of a mixed launch instead.  Returns
// the share count; *wgs gets the decode workgroups.
int32_t decode_shares(ca_ctx* ctx, const ca_plan* plan, const Shape& sh, int32_t* wgs) {
    int64_t blocks = 0;
    for (int32_t s = 0; s < plan->num_decodes; ++s) {
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
        blocks += (kv_len + 31) / 32;
    }
    blocks *= sh.hkv;
    int32_t& per_cu = ctx->attn_wgs_per_cu[sh.d == 128 ? 1 : 0];
    if (per_cu == 0) per_cu = ca::attention_wgs_per_cu(sh.d);
    const int32_t slots = ctx->num_cus * per_cu;
    const bool mixed = plan->num_seqs > plan->num_decodes && !ctx->split_attention;
    int32_t n = slots;
    if (mixed) {
        n = ctx->dec_wgs_override > 0 ? ctx->dec_wgs_override
                                      : static_cast<int32_t>(slots * mixed_decode_share(ctx, plan, sh));
        n = (n + 7) / 8 * 8;
        if (n > slots) n = slots;
    } else if (ctx->dec_wgs_override > 0) {
        n = ctx->dec_wgs_override < slots ? ctx->dec_wgs_override : slots;
    }
    const int32_t per_wg = ctx->dec_wpg;
    const int64_t W = static_cast<int64_t>(n) * per_wg;
    const int32_t shares = static_cast<int32_t>(W < blocks ? W : blocks);
    *wgs = shares > 0 ? (shares + per_wg - 1) / per_wg : 0;
    if (mixed) *wgs = (*wgs + 7) / 8 * 8;  // keep the chunk workgroups' XCD order
    return shares;
}

// Keys per chunk split: a row block whose visible keys exceed this is cut into several
// workgroups (merged afterwards) so that a step with few chunk rows still covers the CUs.
int32_t chunk_split_keys(const ca_ctx* ctx, const ca_plan* plan, const Shape& sh,
                         int32_t override_keys) {
    const int32_t G = sh.hq / sh.hkv;
    const int32_t cols_per_block = ca::chunk_cols_per_block();
    if (override_keys > 0) {
        int32_t longest = 0;
        for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
            const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
            const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
            if (kv_len > longest) longest = kv_len;
        }
        int32_t L = override_keys > (longest + 63) / 64 ? override_keys : (longest + 63) / 64;
        L = ((L + 31) / 32) * 32;
        return L < ca::chunk_max_split_keys() ? L : ca::chunk_max_split_keys() / 32 * 32;
    }
    int64_t work = 0;  // sum over column blocks of visible keys (x kv heads)
    int64_t blocks = 0;  // column blocks (x kv heads): the chunk workgroups if no row block is split
    int32_t widest = 0;  // most keys one column block sees
    for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
        const int32_t q_len = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
        const int32_t ncols = q_len * G;
        for (int32_t cb = 0; cb < ncols; cb += cols_per_block) {
            const int32_t last = (cb + cols_per_block < ncols ? cb + cols_per_block : ncols) - 1;
            const int32_t keys = kv_len - q_len + last / G + 1;
            work += static_cast<int64_t>(keys) * sh.hkv;
            blocks += sh.hkv;
            if (keys > widest) widest = keys;
        }
    }
    // When the chunk rows have the device to themselves (no decode rows in the launch), unsplit
    // row blocks that already fill most of it in one round, with key ranges of about the same
    // length, stay whole: splitting them only adds partials, a longer merge and each extra
    // workgroup's pipeline fill.  Measured on the part (Yi-34B chunk alone: 212 blocks of ~16 K
    // keys on 256 CUs): whole blocks 424-470 us with a 5 us merge, against 461-495 us with a
    // 31 us merge when cut into ~1 K workgroups.  Beside decode rows the chunk workgroups start
    // on a quarter of the CUs and take over the rest as the decode drains, and there the smaller
    // pieces rebalance onto the freed CUs: same fused time within the box-to-box spread.
    const bool beside_decode = plan->num_decodes > 0 && !ctx->split_attention;
    if (!beside_decode) {
        const int32_t known = ctx->attn_wgs_per_cu[sh.d == 128 ? 1 : 0];
        const int64_t slots = static_cast<int64_t>(ctx->num_cus) * (known > 0 ? known : 1);
        const int64_t cap = ca::chunk_max_split_keys() / 32 * 32;
        const bool one_round = blocks > 0 && 4 * blocks >= 3 * slots && blocks <= slots;
        const bool even = 4 * static_cast<int64_t>(widest) * blocks <= 5 * work;  // widest <= 1.25 x mean
        if (one_round && even && widest <= cap) return ((widest + 31) / 32) * 32;
    }
    // Otherwise aim at ~1 K workgroups (one per CU at a time, several rounds), each with at least
    // kMinSplitKeys keys as long as that still leaves one workgroup per CU (512 at least): a
    // shorter split spends too much of its time filling the stage pipeline and writing its 128 KB
    // of partials, while too few workgroups leave CUs idle.  Measured on the part (Llama-13B
    // 8192-token prompt, whole prompt at chunk size c): the 1280-key floor against 512 took c =
    // 128 / 256 / 512 / 1024 from 2848 / 1878 / 1418 / 1092 us to 2580 / 1628 / 1213 / 1023 us
    // (2048 was slower again for small c); applied without the one-per-CU bound it made the
    // Mistral-7B chunks launched alone (64 row blocks of ~1.8 K keys) 27 -> 45 us.
    constexpr int64_t kMinSplitKeys = 1280;
    const int64_t target = 1024;
    const int32_t known_cu = ctx->attn_wgs_per_cu[sh.d == 128 ? 1 : 0];
    const int64_t wg_slots = static_cast<int64_t>(ctx->num_cus) * (known_cu > 0 ? known_cu : 1);
    const int64_t per_slot = (work + wg_slots - 1) / wg_slots;
    int64_t L = (work + target - 1) / target;
    const int64_t floor_keys = per_slot < kMinSplitKeys ? per_slot : kMinSplitKeys;
    if (L < floor_keys) L = floor_keys;
    if (L < 512) L = 512;
    // When decode rows share the launch they set its length (their K/V stream), and the chunk
    // workgroups run beside them on the CUs the decode rows leave free.  If all the chunk work
    // fits there within that time, splitting a row block only adds its partials' round trip
    // through HBM and the merge: keep each block whole, as long as its workgroup still ends well
    // inside the decode time.  (The estimates are mixed_work's.)
    const bool fused = plan->num_decodes > 0 && plan->num_seqs > plan->num_decodes && !ctx->split_attention;
    if (fused) {
        double dec_us = 0, chunk_cu_us = 0;
        mixed_work(plan, sh, &dec_us, &chunk_cu_us);
        const double chunk_cus = ctx->num_cus * (1.0 - mixed_decode_share(ctx, plan, sh));
        if (chunk_cu_us <= 0.75 * chunk_cus * dec_us) {
            int32_t longest = 0;
            for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
                const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
                const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
                if (kv_len > longest) longest = kv_len;
            }
            const int64_t whole = static_cast<int64_t>(0.9 * dec_us / chunk_block_us(sh)) * 32;
            const int64_t keep = longest < whole ? longest : whole;
            if (keep > L) L = keep;
        } else {
            // More chunk work than the chunk CUs finish within the decode stream: it spills onto
            // the decode CUs as those drain (queue mode).  Splits of up to ~0.4 of the decode
            // time keep the partials (HBM traffic beside the decode stream, and merge work) few
            // while the queues still even out the end.  Measured on the part (LLaMA2-70B step,
            // ~950 us of decode): splits of 3200 / 4800 / 6400 / 9600 / 14400 / 21000 keys gave
            // 1119 / 1087 / 1041 / 1025 / 1053 / 1246 us (1173 us at the ~1.8 K-key default).
            const int64_t spill = static_cast<int64_t>(0.4 * dec_us / chunk_block_us(sh)) * 32;
            if (spill > L) L = spill;
        }
    }
    // With the device to themselves, a split length that leaves a few more items than workgroup
    // slots runs those few as a second round of the same length: lengthen the splits (by up to
    // twice) until one round holds every item.
    if (!beside_decode) {
        auto items_at = [&](int64_t len) {
            int64_t n = 0;
            for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
                const int32_t q_len = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
                const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
                const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
                const int32_t ncols = q_len * G;
                for (int32_t cb = 0; cb < ncols; cb += cols_per_block) {
                    const int32_t last = (cb + cols_per_block < ncols ? cb + cols_per_block : ncols) - 1;
                    n += (kv_len - q_len + last / G + 1 + len - 1) / len;
                }
            }
            return n * sh.hkv;
        };
        const int64_t L32 = ((L + 31) / 32) * 32;
        const int64_t n0 = items_at(L32);
        const int64_t cap = ca::chunk_max_split_keys() / 32 * 32;
        if (n0 > wg_slots && n0 < 2 * wg_slots) {
            for (int64_t L2 = L32 + 32; L2 <= 2 * L32 && L2 <= cap; L2 += 32) {
                if (items_at(L2) <= wg_slots) {
                    L = L2;
                    break;
                }
            }
        }
    }
    // the split merge handles at most 64 splits of one row block
    int32_t longest = 0;
    for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
        if (kv_len > longest) longest = kv_len;
    }
    if (L * 64 < longest) L = (longest + 63) / 64;
    L = ((L + 31) / 32) * 32;
    const int64_t cap = ca::chunk_max_split_keys() / 32 * 32;
    return static_cast<int32_t>(L < cap ? L : cap);
}

// Reorder workgroup records so that consecutive records (same sequence and kv head, hence the
// same K/V pages) are dispatched to the same XCD: workgroups go round-robin over the 8 XCDs, so
// record i is placed at grid slot (i % per) * 8 + i / per.  Returns the padded grid size; pad
// slots are marked with seq = -1.
template <int N>
int32_t xcd_order(const std::vector<int4>& in, std::vector<int4>& out) {
    const int32_t n = static_cast<int32_t>(in.size()) / N;
    const int32_t per = (n + 7) / 8;
    const int32_t grid = per * 8;
    out.assign(static_cast<size_t>(grid) * N, make_int4(-1, 0, 0, 0));
    for (int32_t i = 0; i < n; ++i) {
        const int32_t slot = (i % per) * 8 + i / per;
        for (int k = 0; k < N; ++k) out[static_cast<size_t>(slot) * N + k] = in[static_cast<size_t>(i) * N + k];
    }
    return grid;
}

// Make the plan's metadata and, for the MFMA path, its work lists resident on the device.
// Everything goes in ONE upload (pinned staging, copied by a kernel on the caller's stream):
//   [qo_indptr | kv_page_indptr | kv_last_page_len | kv_page_indices | row_seq | row_pos |
//    row_page | pad to 16 B][rotary inverse frequencies, fp64]
//   [decode items | first item of each decode wave | decode merges | chunk items | chunk merges]
// keyed by (plan generation, shape, split sizes), so the append and the attention of one step
// share it and a repeated call with the same plan uploads nothing.
// The rotary inverse frequencies theta^(-2i/d) of this shape, fp64, as a device table (built on
// the host once per (d, theta) and kept for the context's lifetime).
ca_status ensure_freq(ca_ctx* ctx, const Shape& sh) {
    const std::pair<int32_t, double> key(sh.d, static_cast<double>(sh.theta));
    auto it = ctx->freq_tables.find(key);
    if (it == ctx->freq_tables.end()) {
        std::vector<double> f(static_cast<size_t>(sh.d / 2));
        for (int32_t i = 0; i < sh.d / 2; ++i)
            f[static_cast<size_t>(i)] = std::pow(static_cast<double>(sh.theta), -2.0 * static_cast<double>(i) / static_cast<double>(sh.d));
        void* p = nullptr;
        hipError_t e = hipMalloc(&p, f.size() * sizeof(double));
        if (e != hipSuccess) return device_error("rotary table allocation", e);
        e = hipMemcpy(p, f.data(), f.size() * sizeof(double), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return device_error("rotary table copy", e);
        }
        it = ctx->freq_tables.emplace(key, p).first;
    }
    ctx->inv_freq = static_cast<const double*>(it->second);
    return CA_OK;
}

// The step's work lists on the host, into ctx's reused vectors: decode items in `split` equal
// shares (with their merges) and chunk workgroups of at most `csplit` keys (with their merges).
// *slots / *cslots receive the partial slots the decode and chunk splits need.
void build_lists(ca_ctx* ctx, const ca_plan* plan, const Shape& sh, bool mfma, int32_t split,
                 int32_t csplit, int32_t dec_wgs, int32_t* slots_out, int32_t* cslots_out) {
    const int G = sh.hq / sh.hkv;
    std::vector<int4>& items = ctx->items;
    std::vector<int4>& merges = ctx->merges;
    std::vector<int4>& citems = ctx->citems;
    std::vector<int4>& groups = ctx->groups;
    std::vector<int32_t>& wave_items = ctx->wave_items;
    items.clear();
    merges.clear();
    citems.clear();
    groups.clear();
    wave_items.clear();
    int32_t slots = 0, cslots = 0;
    if (mfma) {
        // decode: share w holds blocks [B w / W, B (w + 1) / W) of the B blocks of all
        // (decode row, kv head) pairs in order; each pair's run inside a share is one item, and
        // a pair cut over several shares gets one partial slot per piece and a merge
        const int32_t W = split;
        const int64_t B = [&] {
            int64_t b = 0;
            for (int32_t s = 0; s < plan->num_decodes; ++s) {
                const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
                b += ((np - 1) * plan->page_size + plan->kv_last_page_len[s] + 31) / 32;
            }
            return b * sh.hkv;
        }();
        // share boundaries B w / W, built incrementally (no division per share)
        std::vector<int64_t>& bounds = ctx->share_bounds;
        bounds.resize(static_cast<size_t>(W) + 2);
        {
            const int64_t q = W > 0 ? B / W : 0, r = W > 0 ? B % W : 0;
            int64_t b = 0, acc = 0;
            for (int32_t k = 0; k <= W; ++k) {
                bounds[static_cast<size_t>(k)] = b;
                b += q;
                acc += r;
                if (acc >= W) { acc -= W; ++b; }
            }
            bounds[static_cast<size_t>(W) + 1] = B;  // never reached: the walk stops at share W
        }
        const int64_t* bnd = bounds.data();
        wave_items.assign(static_cast<size_t>(W) + 1, 0);
        int32_t* wi = wave_items.data();
        // at most one item per (row, kv head) pair plus one per share boundary, and one merge per
        // pair: the lists are sized once and written through pointers
        const size_t max_items = static_cast<size_t>(plan->num_decodes) * sh.hkv + static_cast<size_t>(W) + 1;
        items.resize(2 * max_items);
        merges.resize(static_cast<size_t>(plan->num_decodes) * sh.hkv);
        int4* it = items.data();
        int4* mg = merges.data();
        int32_t n_it = 0;
        int64_t off = 0;
        int32_t w = 0;
        int64_t next_bound = bnd[1];
        for (int32_t s = 0; s < plan->num_decodes; ++s) {
            const int32_t p0 = plan->kv_page_indptr[s];
            const int32_t np = plan->kv_page_indptr[s + 1] - p0;
            const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
            const int64_t nb = (kv_len + 31) / 32;
            const int32_t row = plan->qo_indptr[s];
            for (int32_t g = 0; g < sh.hkv; ++g) {
                const int64_t end = off + nb;
                const int32_t first = n_it;
                for (int64_t lo = off; lo < end;) {
                    while (next_bound <= lo) {
                        wi[++w] = n_it;
                        next_bound = bnd[w + 1];
                    }
                    const int64_t hi = end < next_bound ? end : next_bound;
                    const int32_t kb = static_cast<int32_t>(32 * (lo - off));
                    const int32_t ke = static_cast<int32_t>(32 * (hi - off) < kv_len ? 32 * (hi - off) : kv_len);
                    it[2 * n_it] = make_int4(g, kb, ke, -1);
                    it[2 * n_it + 1] = make_int4(row, p0, np, 0);
                    ++n_it;
                    lo = hi;
                }
                const int32_t pieces = n_it - first;
                if (pieces > 1) {
                    *mg++ = make_int4(row, g, slots, pieces);
                    for (int32_t i = 0; i < pieces; ++i) it[2 * (first + i)].w = slots++;
                }
                off = end;
            }
        }
        while (w < W) wi[++w] = n_it;
        items.resize(2 * static_cast<size_t>(n_it));
        merges.resize(static_cast<size_t>(mg - merges.data()));
        // chunks: one workgroup per (sequence, kv head, block of 256 columns, split of Lc keys);
        // a column is one (row, q head) pair, numbered row * G + head
        const int32_t Lc = csplit;
        // A column block's split i covers keys [i Lc, (i + 1) Lc), the last one the remainder.
        // In queue mode (below) a block whose remainder would be longer than Lt = Lc / 4 gets a
        // last piece of Lt keys instead and its other pieces share the rest evenly (each at most
        // the split cap): the queues hand out the short pieces last, so the launch ends on a
        // round of short items rather than on whichever full-length items started last.
        const int32_t Lt = ((Lc / 4 + 31) / 32) * 32;
        const int32_t cap = ca::chunk_max_split_keys() / 32 * 32;
        auto piece = [&](int32_t key_end, int32_t nsplit, bool short_tail, int32_t i, int32_t* kb, int32_t* ke) {
            if (!short_tail) {
                *kb = i * Lc;
                *ke = (*kb + Lc < key_end) ? *kb + Lc : key_end;
                return;
            }
            const int32_t ts = (key_end - Lt) / 32 * 32;  // the short piece's first key
            auto at = [&](int32_t j) { return static_cast<int32_t>(static_cast<int64_t>(ts / 32) * j / (nsplit - 1)) * 32; };
            *kb = i < nsplit - 1 ? at(i) : ts;
            *ke = i < nsplit - 1 ? at(i + 1) : key_end;
        };
        auto has_short_tail = [&](int32_t key_end, int32_t nsplit) {
            if (nsplit < 2) return false;
            const int32_t r = key_end - (nsplit - 1) * Lc;
            const int32_t ts = (key_end - Lt) / 32 * 32;
            return r > Lt && ts / (nsplit - 1) + 32 <= cap;
        };
        const int32_t cols_per_block = ca::chunk_cols_per_block();
        // How the attention launch's chunk workers take the items (attn_mixed.hip).  If every
        // item fits on the workgroup slots free when the launch starts, one worker per item
        // (direct mode), the list in XCD order.  Otherwise one persistent worker per workgroup
        // slot of the device (queue mode): the workers on the slots the decode workgroups leave
        // start at once, the others as the decode drains, and each takes items until none is
        // left.  Measured on the part (Yi-34B step, 1096 items): with one workgroup per item the
        // in-order dispatcher left a tenth of the chunk CUs idle behind busy XCDs and the launch
        // ended on ~100 us of straggling full-length items; queue mode took the fused launch
        // 588 -> 559 us (LLaMA2-70B step 1222 -> 1172 us, Llama-13B one-shot prompt 773 ->
        // 716 us, its last 256-row chunk 77 -> 67 us).
        const int32_t per_cu = ctx->attn_wgs_per_cu[sh.d == 128 ? 1 : 0];
        const int32_t wslots = ctx->num_cus * (per_cu > 0 ? per_cu : 1);
        const bool fused = dec_wgs > 0 && plan->num_decodes > 0 && !ctx->split_attention;
        const int32_t early = fused ? (wslots > dec_wgs ? wslots - dec_wgs : 0) : wslots;
        int64_t n_items = 0;
        for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
            const int32_t q_len = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
            const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
            const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
            const int32_t ncols = q_len * G;
            for (int32_t cb = 0; cb < ncols; cb += cols_per_block) {
                const int32_t last = (cb + cols_per_block < ncols ? cb + cols_per_block : ncols) - 1;
                n_items += (kv_len - q_len + last / G + 1 + Lc - 1) / Lc;
            }
        }
        n_items *= sh.hkv;
        const bool queue_mode = n_items > early;
        std::vector<int4>& clist = ctx->clist;
        clist.clear();
        for (int32_t s = plan->num_decodes; s < plan->num_seqs; ++s) {
            const int32_t q_len = plan->qo_indptr[s + 1] - plan->qo_indptr[s];
            const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
            const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
            const int32_t ncols = q_len * G;
            // Records go key range by key range (all column blocks of split 0, then of split 1,
            // ...), so the workgroups that one XCD runs side by side read the same pages and
            // share them in its L2; each column block's partial slots stay contiguous.
            const int32_t nblocks = (ncols + cols_per_block - 1) / cols_per_block;
            for (int32_t g = 0; g < sh.hkv; ++g) {
                int32_t max_split = 0;
                const int32_t slot0 = cslots;
                for (int32_t b = 0; b < nblocks; ++b) {
                    const int32_t cb = b * cols_per_block;
                    const int32_t last = (cb + cols_per_block < ncols ? cb + cols_per_block : ncols) - 1;
                    const int32_t key_end = kv_len - q_len + last / G + 1;  // last row's position + 1
                    const int32_t nsplit = (key_end + Lc - 1) / Lc;
                    if (nsplit > max_split) max_split = nsplit;
                    if (nsplit > 1) {
                        groups.push_back(make_int4(s, g, cb, cslots));
                        groups.push_back(make_int4(nsplit, plan->qo_indptr[s], q_len, 0));
                        cslots += nsplit;
                    }
                }
                for (int32_t i = 0; i < max_split; ++i) {
                    int32_t slot = slot0;
                    for (int32_t b = 0; b < nblocks; ++b) {
                        const int32_t cb = b * cols_per_block;
                        const int32_t last = (cb + cols_per_block < ncols ? cb + cols_per_block : ncols) - 1;
                        const int32_t key_end = kv_len - q_len + last / G + 1;
                        const int32_t nsplit = (key_end + Lc - 1) / Lc;
                        if (i < nsplit) {
                            int32_t kb, ke;
                            piece(key_end, nsplit, queue_mode && has_short_tail(key_end, nsplit), i, &kb, &ke);
                            clist.push_back(make_int4(s, g, cb, nsplit == 1 ? -1 : slot + i));
                            clist.push_back(make_int4(kb, ke, 0, 0));
                        }
                        if (nsplit > 1) slot += nsplit;
                    }
                }
            }
        }
        // Queue mode: the list forms eight queues, one per XCD (queue x: the x-th eighth of
        // the list), each with its longer items first and the rest in list order (key range by
        // key range), so that the last items taken are the short pieces.
        const size_t n = clist.size() / 2;
        if (n == 0) {
            citems.clear();
            ctx->chunk_workers = ctx->chunk_static = 0;
            ctx->chunk_queue_mode = false;
        } else if (!queue_mode) {
            const int32_t grid = xcd_order<2>(clist, citems);
            ctx->chunk_workers = grid;
            ctx->chunk_static = grid;
            ctx->chunk_queue_mode = false;
        } else {
            const size_t per = (n + 7) / 8;
            citems.resize(clist.size());
            std::vector<int32_t>& order = ctx->corder;
            for (size_t x0 = 0; x0 < n; x0 += per) {
                const size_t x1 = x0 + per < n ? x0 + per : n;
                order.resize(x1 - x0);
                for (size_t i = x0; i < x1; ++i) order[i - x0] = static_cast<int32_t>(i);
                std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
                    return clist[2 * a + 1].y - clist[2 * a + 1].x > clist[2 * b + 1].y - clist[2 * b + 1].x;
                });
                for (size_t i = x0; i < x1; ++i) {
                    citems[2 * i] = clist[2 * order[i - x0]];
                    citems[2 * i + 1] = clist[2 * order[i - x0] + 1];
                }
            }
            ctx->chunk_workers = wslots;
            ctx->chunk_static = early;
            ctx->chunk_queue_mode = true;
        }
    }

    *slots_out = slots;
    *cslots_out = cslots;
}

// Where prepare() puts a step's device data: the context's growable buffers, or (no_alloc) the
// library's static scratch array, carved in 256-byte aligned pieces.
constexpr size_t kScratchAlign = 256;
size_t align_up(size_t x) { return (x + kScratchAlign - 1) / kScratchAlign * kScratchAlign; }

// defer: leave the metadata in its staging slot (ctx->defer_slot) for the append launch that
// follows to copy; otherwise copy it now with the upload kernel.  writes: the caller appends to
// the cache (with CA_DEBUG_VALIDATE its write targets are checked).
//
// no_alloc (ca_mixed_attention_noalloc): nothing is allocated.  The metadata goes through a
// staging slot allocated at ca_create (a plan too large for it is refused) into the static
// scratch array, followed by the split partials; when the chunk partials would not fit, the
// chunk key splits are made longer (fewer partial slots) until they do, and a plan whose
// metadata and decode partials alone exceed the scratch is refused.  The cache of device
// metadata is bypassed (every call uploads) and invalidated, so the growable buffers' copy is
// rebuilt by the next ordinary call.
ca_status prepare(ca_ctx* ctx, const ca_plan* plan, const Shape& sh, int64_t pool,
                  hipStream_t stream, bool defer = false, bool writes = false,
                  bool no_alloc = false) {
    const int G = sh.hq / sh.hkv;
    int32_t dec_wgs = 0;
    const bool mfma = sh.dtype == CA_BF16 && G <= 16;
    WorkKey key{plan->generation, sh.hq, sh.hkv, sh.d,
                mfma ? decode_shares(ctx, plan, sh, &dec_wgs) : -1,
                mfma ? chunk_split_keys(ctx, plan, sh, ctx->csplit_override) : -1, sh.theta};
    const bool check_targets = writes && ctx->debug_validate;
    if (!no_alloc && plan->generation != 0 && key == ctx->work_key) {
        // the plan was validated when it was first seen, but against that call's pool: its pages
        // must also lie in this call's
        if (ctx->work_max_page >= pool) {
            ca::set_error("page index " + std::to_string(ctx->work_max_page) + " outside the pool");
            return CA_ERR_INVALID_ARG;
        }
        if (check_targets && !ctx->work_targets_checked) {
            int32_t top = -1;
            ca_status st = validate_plan_arrays(plan, pool, true, &top);
            if (st != CA_OK) return st;
            ctx->work_targets_checked = true;
        }
        return CA_OK;
    }
    // structure first (the work lists below rely on it); the page ids are range-checked as they
    // are copied into the staging slot
    int32_t max_page = -1;
    ca_status st = plan->num_seqs > 0 ? validate_plan_structure(plan) : CA_OK;
    if (st == CA_OK && check_targets && plan->num_seqs > 0) st = check_write_targets(plan);
    if (st != CA_OK) return st;
    ctx->work_key = WorkKey{};  // meta_buf is about to change; nothing matches until it is whole
    ctx->defer_slot = -1;
    if (!no_alloc) {  // the attention alone never reads the rotary table
        st = ensure_freq(ctx, sh);
        if (st != CA_OK) return st;
    }

    int32_t slots = 0, cslots = 0;
    build_lists(ctx, plan, sh, mfma, key.split, key.csplit, dec_wgs, &slots, &cslots);
    const std::vector<int4>& items = ctx->items;
    const std::vector<int4>& merges = ctx->merges;
    const std::vector<int4>& citems = ctx->citems;
    const std::vector<int4>& groups = ctx->groups;
    const std::vector<int32_t>& wave_items = ctx->wave_items;
    // partial workspace of the MFMA path: decode [slots][G][d] + [slots][G], chunk
    // [cslots][cols][d] + [cslots][cols] (fp32 and float2)
    auto partial_bytes = [&](int32_t ds, int32_t cs) {
        if (!mfma) return size_t(0);
        const size_t d_ = static_cast<size_t>(ds > 0 ? ds : 1), c_ = static_cast<size_t>(cs > 0 ? cs : 1) * ca::chunk_cols_per_block();
        return align_up(d_ * G * sh.d * sizeof(float)) + align_up(d_ * G * sizeof(float2)) +
               align_up(c_ * sh.d * sizeof(float)) + align_up(c_ * sizeof(float2));
    };
    const int32_t ns = plan->num_seqs;
    const int32_t T = plan->num_tokens;
    const size_t plan_ints = static_cast<size_t>(ns + 1) * 2 + ns + plan->num_pages + 3 * static_cast<size_t>(T);
    const size_t off_items = (plan_ints * sizeof(int32_t) + 15) / 16 * 16;
    // staged layout after the plan arrays: decode items | first item of each decode wave (padded
    // to 16 bytes) | decode merges | chunk items | chunk merges
    auto meta_bytes = [&]() {
        return (off_items + items.size() * sizeof(int4) + (wave_items.size() + 3) / 4 * 4 * sizeof(int32_t) +
                merges.size() * sizeof(int4) + citems.size() * sizeof(int4) + groups.size() * sizeof(int4) +
                16 + 15) / 16 * 16;
    };
    size_t bytes = meta_bytes();
    char* meta_dst = nullptr;
    char* part_base = nullptr;
    hipError_t e = hipSuccess;
    if (no_alloc) {
        if (!ctx->scratch) { ca::set_error("scratch array unavailable"); return CA_ERR_INTERNAL; }
        // fewer, longer chunk splits until metadata and partials fit (a split never exceeds the
        // longest range one chunk workgroup may cover)
        const int32_t cap_keys = ca::chunk_max_split_keys() / 32 * 32;
        int32_t Lc = key.csplit;
        while (mfma && cslots > 0 && align_up(bytes) + partial_bytes(slots, cslots) > ca::kScratchBytes &&
               Lc < cap_keys) {
            Lc = Lc * 2 < cap_keys ? Lc * 2 : cap_keys;
            build_lists(ctx, plan, sh, mfma, key.split, Lc, dec_wgs, &slots, &cslots);
            bytes = meta_bytes();
        }
        if (align_up(bytes) + partial_bytes(slots, cslots) > ca::kScratchBytes) {
            ca::set_error("ca_mixed_attention_noalloc: the step needs " +
                          std::to_string(align_up(bytes) + partial_bytes(slots, cslots)) +
                          " bytes of workspace, more than the " + std::to_string(ca::kScratchBytes) +
                          "-byte scratch array");
            return CA_ERR_CAPACITY;
        }
        meta_dst = static_cast<char*>(ctx->scratch);
        part_base = meta_dst + align_up(bytes);
    } else {
        e = ctx->meta_buf.reserve(bytes, stream);
        if (e != hipSuccess) return device_error("metadata allocation", e);
        meta_dst = static_cast<char*>(ctx->meta_buf.ptr);
    }
    const size_t off_waves = off_items + items.size() * sizeof(int4);
    const size_t off_merge = off_waves + (wave_items.size() + 3) / 4 * 4 * sizeof(int32_t);
    const size_t off_citem = off_merge + merges.size() * sizeof(int4);
    const size_t off_group = off_citem + citems.size() * sizeof(int4);
    int slot = 0;
    e = ctx->staging.acquire(bytes, &slot, /*may_grow=*/!no_alloc);
    if (e != hipSuccess) return device_error("staging allocation", e);
    if (slot < 0) {
        ca::set_error("ca_mixed_attention_noalloc: the step's metadata (" + std::to_string(bytes) +
                      " bytes) exceeds a staging slot");
        return CA_ERR_CAPACITY;
    }
    char* h = static_cast<char*>(ctx->staging.host[slot]);
    int32_t* hp = reinterpret_cast<int32_t*>(h);
    std::memcpy(hp, plan->qo_indptr, sizeof(int32_t) * (ns + 1));
    std::memcpy(hp + (ns + 1), plan->kv_page_indptr, sizeof(int32_t) * (ns + 1));
    std::memcpy(hp + 2 * (ns + 1), plan->kv_last_page_len, sizeof(int32_t) * ns);
    st = check_page_range(plan, pool, hp + 2 * (ns + 1) + ns, &max_page);
    if (st != CA_OK) return st;
    // per row: its sequence, absolute position and destination page (the slot is pos % P)
    int32_t* hrow = hp + 2 * (ns + 1) + ns + plan->num_pages;
    int32_t* hpos = hrow + T;
    int32_t* hpage = hpos + T;
    for (int32_t s = 0; s < ns; ++s) {
        const int32_t q0 = plan->qo_indptr[s], q_len = plan->qo_indptr[s + 1] - q0;
        const int32_t p0 = plan->kv_page_indptr[s];
        const int32_t kv_len = (plan->kv_page_indptr[s + 1] - p0 - 1) * plan->page_size + plan->kv_last_page_len[s];
        for (int32_t i = 0; i < q_len; ++i) {
            const int32_t pos = kv_len - q_len + i;
            hrow[q0 + i] = s;
            hpos[q0 + i] = pos;
            hpage[q0 + i] = plan->kv_page_indices[p0 + pos / plan->page_size];
        }
    }
    std::memcpy(h + off_items, items.data(), items.size() * sizeof(int4));
    std::memcpy(h + off_waves, wave_items.data(), wave_items.size() * sizeof(int32_t));
    std::memcpy(h + off_merge, merges.data(), merges.size() * sizeof(int4));
    std::memcpy(h + off_citem, citems.data(), citems.size() * sizeof(int4));
    std::memcpy(h + off_group, groups.data(), groups.size() * sizeof(int4));
    const size_t row_pos_off = (static_cast<size_t>(2) * (ns + 1) + ns + plan->num_pages + T) * sizeof(int32_t);
    if (defer) {
        ctx->defer_slot = slot;
        ctx->defer_bytes = bytes;
        const char* hd = static_cast<const char*>(ctx->staging.dev[slot]);
        ctx->hrow_pos = reinterpret_cast<const int32_t*>(hd + row_pos_off);
        ctx->hrow_page = ctx->hrow_pos + T;
    } else {
        Timed t(ctx->prof, "upload", CA_PROFILE_UPLOAD, !no_alloc);
        e = ctx->staging.upload(slot, meta_dst, bytes, stream, t.ev);
        if (e == hipSuccess) t.commit();
        if (e != hipSuccess) {
            ctx->work_key = WorkKey{};
            return device_error("metadata upload", e);
        }
    }

    const char* d = meta_dst;
    const int32_t* dp = reinterpret_cast<const int32_t*>(d);
    ctx->dplan.qo_indptr = dp;
    ctx->dplan.kv_page_indptr = dp + (ns + 1);
    ctx->dplan.kv_last_page_len = dp + 2 * (ns + 1);
    ctx->dplan.kv_page_indices = dp + 2 * (ns + 1) + ns;
    ctx->dplan.row_seq = dp + 2 * (ns + 1) + ns + plan->num_pages;
    ctx->dplan.row_pos = ctx->dplan.row_seq + T;
    ctx->dplan.row_page = ctx->dplan.row_pos + T;
    ctx->dplan.num_seqs = ns;
    ctx->dplan.num_decodes = plan->num_decodes;
    ctx->dplan.num_tokens = plan->num_tokens;
    ctx->dplan.num_pages = plan->num_pages;
    ctx->dplan.page_size = plan->page_size;
    DevWork& w = ctx->dwork;
    w.dec_items = reinterpret_cast<const int4*>(d + off_items);
    w.dec_wave_items = reinterpret_cast<const int32_t*>(d + off_waves);
    w.merges = reinterpret_cast<const int4*>(d + off_merge);
    w.chunk_items = reinterpret_cast<const int4*>(d + off_citem);
    w.chunk_groups = reinterpret_cast<const int4*>(d + off_group);
    w.num_dec_items = static_cast<int32_t>(items.size() / 2);
    w.num_dec_waves = wave_items.empty() ? 0 : static_cast<int32_t>(wave_items.size()) - 1;
    w.dec_wgs = dec_wgs;
    w.dec_wpg = ctx->dec_wpg;
    w.num_merges = static_cast<int32_t>(merges.size());
    w.num_slots = slots;
    w.num_chunk_items = static_cast<int32_t>(citems.size() / 2);
    w.num_chunk_workers = ctx->chunk_workers;
    w.num_chunk_static = ctx->chunk_static;
    w.chunk_queue_mode = ctx->chunk_queue_mode;
    w.num_chunk_groups = static_cast<int32_t>(groups.size() / 2);
    w.num_chunk_slots = cslots;
    if (mfma) {
        const size_t dslots = static_cast<size_t>(slots > 0 ? slots : 1);
        const size_t cslots_sz = static_cast<size_t>(cslots > 0 ? cslots : 1) * ca::chunk_cols_per_block();
        if (no_alloc) {
            char* q = part_base;
            ctx->dacc = reinterpret_cast<float*>(q);
            q += align_up(dslots * G * sh.d * sizeof(float));
            ctx->dml = reinterpret_cast<float2*>(q);
            q += align_up(dslots * G * sizeof(float2));
            ctx->cacc = reinterpret_cast<float*>(q);
            q += align_up(cslots_sz * sh.d * sizeof(float));
            ctx->cml = reinterpret_cast<float2*>(q);
        } else {
            e = ctx->dec_acc_buf.reserve(dslots * G * sh.d * sizeof(float), stream);
            if (e == hipSuccess) e = ctx->dec_ml_buf.reserve(dslots * G * sizeof(float2), stream);
            if (e == hipSuccess) e = ctx->chk_acc_buf.reserve(cslots_sz * sh.d * sizeof(float), stream);
            if (e == hipSuccess) e = ctx->chk_ml_buf.reserve(cslots_sz * sizeof(float2), stream);
            if (e != hipSuccess) return device_error("partial allocation", e);
            ctx->dacc = static_cast<float*>(ctx->dec_acc_buf.ptr);
            ctx->dml = static_cast<float2*>(ctx->dec_ml_buf.ptr);
            ctx->cacc = static_cast<float*>(ctx->chk_acc_buf.ptr);
            ctx->cml = static_cast<float2*>(ctx->chk_ml_buf.ptr);
        }
    }
    ctx->meta_end = align_up(bytes);  // scratch bytes the metadata takes (no_alloc)
    if (no_alloc) return CA_OK;        // the scratch copy is not cached
    ctx->work_key = key;
    ctx->work_max_page = max_page;
    ctx->work_targets_checked = check_targets;
    return CA_OK;
}

}  // namespace

extern "C" {

ca_status ca_create(int device, ca_ctx** out) {
    ca::clear_error();
    if (!out) { ca::set_error("ca_create: null out"); return CA_ERR_INVALID_ARG; }
    *out = nullptr;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return device_error("hipGetDeviceCount", e);
    if (device < 0 || device >= count) { ca::set_error("ca_create: no such device"); return CA_ERR_INVALID_ARG; }
    DeviceGuard g(device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    ca_ctx* ctx = new ca_ctx();
    ctx->device = device;
    if (const char* env = std::getenv("CA_DECODE_WGS")) ctx->dec_wgs_override = std::atoi(env);
    if (const char* env = std::getenv("CA_SPLIT_ATTENTION")) ctx->split_attention = std::atoi(env) != 0;
    if (const char* env = std::getenv("CA_DECODE_WAVES")) {
        const int v = std::atoi(env);
        if (v >= 1 && v <= ca::attention_decode_waves_per_wg()) ctx->dec_wpg = v;
    }
    e = hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess || ctx->num_cus <= 0) {
        delete ctx;
        return device_error("hipDeviceGetAttribute(multiprocessor count)", e != hipSuccess ? e : hipErrorInvalidValue);
    }
    if (const char* env = std::getenv("CA_CHUNK_SPLIT")) ctx->csplit_override = std::atoi(env);
    if (const char* env = std::getenv("CA_PROJECTION_LIBRARY")) ctx->projection_library = std::atoi(env) != 0;
    if (const char* env = std::getenv("CA_DEBUG_VALIDATE")) ctx->debug_validate = std::atoi(env) != 0;
    if (const char* env = std::getenv("CA_PROJECTION_TILE")) {
        int bm = 0, bn = 0, sp = 0;
        if (std::sscanf(env, "%d,%d,%d", &bm, &bn, &sp) == 3) {
            ctx->proj_tile[0] = bm;
            ctx->proj_tile[1] = bn;
            ctx->proj_tile[2] = sp;
        }
    }
    e = ctx->staging.init();
    if (e != hipSuccess) {
        ctx->staging.release();
        delete ctx;
        return device_error("staging allocation", e);
    }
    e = scratch_address(device, &ctx->scratch);
    if (e != hipSuccess) {
        ctx->staging.release();
        delete ctx;
        return device_error("hipGetSymbolAddress(scratch)", e);
    }
    // both sets of chunk work-queue counters start at zero; each attention launch zeroes the set
    // it hands to the next one
    e = hipMalloc(&ctx->queue, 2 * ca::kQueueInts * sizeof(int));
    if (e == hipSuccess) e = hipMemset(ctx->queue, 0, 2 * ca::kQueueInts * sizeof(int));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        if (ctx->queue) (void)hipFree(ctx->queue);
        ctx->staging.release();
        delete ctx;
        return device_error("work-queue allocation", e);
    }
    *out = ctx;
    return CA_OK;
}

ca_status ca_destroy(ca_ctx* ctx) {
    ca::clear_error();
    if (!ctx) return CA_OK;
    DeviceGuard g(ctx->device);
    ctx->staging.release();
    ctx->meta_buf.release();
    ctx->partial_buf.release();
    ctx->proj_part.release();
    ctx->dec_acc_buf.release();
    ctx->dec_ml_buf.release();
    ctx->chk_acc_buf.release();
    ctx->chk_ml_buf.release();
    ctx->prof.release();
    if (ctx->queue) (void)hipFree(ctx->queue);
    for (auto& kv : ctx->freq_tables) (void)hipFree(kv.second);
    ca::linear_release(ctx->linear);
    delete ctx;
    return CA_OK;
}

}  // extern "C"

namespace {

// ca_append_kv_rope and ca_append_kv_rope_packed: q rows q_row elements apart, k and v rows
// kv_row apart.
ca_status append_impl(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan, const void* q_in,
                      void* q_out, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, int64_t num_pool_pages, void* hip_stream, int64_t q_row,
                      int64_t kv_row) {
    if (!ctx) { ca::set_error("null ctx"); return CA_ERR_INVALID_ARG; }
    ca_status st = check_plan(plan);
    if (st != CA_OK) return st;
    Shape sh{};
    st = check_desc(desc, plan, &sh);
    if (st != CA_OK) return st;
    if (num_pool_pages <= 0) { ca::set_error("num_pool_pages must be > 0"); return CA_ERR_INVALID_ARG; }
    if (plan->num_tokens == 0) return CA_OK;
    if (!q_in || !q_out || !k_new || !v_new || !k_cache || !v_cache) {
        ca::set_error("ca_append_kv_rope: null buffer");
        return CA_ERR_INVALID_ARG;
    }
    if (!aligned16({q_in, q_out, k_new, v_new, k_cache, v_cache})) {
        ca::set_error("ca_append_kv_rope: device buffers must be 16-byte aligned");
        return CA_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    st = prepare(ctx, plan, sh, num_pool_pages, stream, /*defer=*/true, /*writes=*/true);
    if (st != CA_OK) return st;
    // A fresh plan's metadata is still in its staging slot: this launch also copies it to device
    // memory (for the attention launch after it), and reads its own per-row values from the
    // staging.  A plan already on the device (append called again) takes the device copy.
    const int slot = ctx->defer_slot;
    const bool copy = slot >= 0;
    hipError_t e;
    {
        Timed t(ctx->prof, "append_rope", CA_PROFILE_APPEND);
        e = ca::launch_append_rope(ctx->dplan, sh, copy ? ctx->hrow_pos : ctx->dplan.row_pos,
                                   copy ? ctx->hrow_page : ctx->dplan.row_page, ctx->inv_freq, q_in,
                                   q_out, k_new, v_new, k_cache, v_cache,
                                   q_row < 0 ? int64_t(sh.hq) * sh.d : q_row,
                                   kv_row < 0 ? int64_t(sh.hkv) * sh.d : kv_row,
                                   copy ? ctx->staging.dev[slot] : nullptr, copy ? ctx->meta_buf.ptr : nullptr,
                                   copy ? static_cast<int64_t>(ctx->defer_bytes / 16) : 0, ctx->num_cus, stream,
                                   t.ev);
        if (e == hipSuccess) t.commit();
    }
    ctx->defer_slot = -1;
    if (e == hipSuccess && copy) e = ctx->staging.mark_read(slot, stream);
    if (e != hipSuccess) {
        if (copy) ctx->work_key = WorkKey{};  // the metadata never reached the device
        return device_error("append_rope launch", e);
    }
    return CA_OK;
}

}  // namespace

extern "C" {

ca_status ca_append_kv_rope(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                            const void* q_in, void* q_out, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int64_t num_pool_pages,
                            void* hip_stream) {
    ca::clear_error();
    return append_impl(ctx, desc, plan, q_in, q_out, k_new, v_new, k_cache, v_cache, num_pool_pages,
                       hip_stream, -1, -1);
}

ca_status ca_append_kv_rope_packed(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                                   const void* qkv, void* q_out, void* k_cache, void* v_cache,
                                   int64_t num_pool_pages, void* hip_stream) {
    ca::clear_error();
    if (!desc || !qkv) { ca::set_error("ca_append_kv_rope_packed: null argument"); return CA_ERR_INVALID_ARG; }
    const int64_t d = desc->head_dim, hq = desc->num_q_heads, hkv = desc->num_kv_heads;
    const int64_t eb = desc->dtype == CA_BF16 ? 2 : 4;
    const int64_t row = (hq + 2 * hkv) * d;
    const char* base = static_cast<const char*>(qkv);
    return append_impl(ctx, desc, plan, base, q_out, base + hq * d * eb, base + (hq + hkv) * d * eb,
                       k_cache, v_cache, num_pool_pages, hip_stream, row, row);
}

ca_status ca_qkv_projection(ca_ctx* ctx, const ca_attn_desc* desc, int32_t num_tokens,
                            int32_t hidden, const void* x, const void* w, void* qkv,
                            void* hip_stream) {
    ca::clear_error();
    if (!ctx || !desc) { ca::set_error("ca_qkv_projection: null argument"); return CA_ERR_INVALID_ARG; }
    if (desc->dtype != CA_BF16) { ca::set_error("ca_qkv_projection: bf16 only"); return CA_ERR_UNSUPPORTED; }
    if (num_tokens < 0 || hidden <= 0 || desc->num_q_heads <= 0 || desc->num_kv_heads <= 0 ||
        desc->head_dim <= 0 || hidden % 8 != 0) {
        ca::set_error("ca_qkv_projection: need num_tokens >= 0, hidden > 0 and a multiple of 8, heads > 0");
        return CA_ERR_INVALID_ARG;
    }
    if (num_tokens == 0) return CA_OK;
    if (!x || !w || !qkv) { ca::set_error("ca_qkv_projection: null buffer"); return CA_ERR_INVALID_ARG; }
    if (!aligned16({x, w, qkv})) {
        ca::set_error("ca_qkv_projection: device buffers must be 16-byte aligned");
        return CA_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const int64_t N = static_cast<int64_t>(desc->num_q_heads + 2 * desc->num_kv_heads) * desc->head_dim;
    std::string err;
    Timed t(ctx->prof, "qkv_projection", CA_PROFILE_PROJECTION);
    // few tokens: the weight-streaming kernel (bound by reading the weights once); otherwise,
    // or with CA_PROJECTION_LIBRARY=1, the library GEMM
    if (!ctx->projection_library && ca::skinny_projection_fits(num_tokens, hidden, N)) {
        const hipError_t e = ca::launch_skinny_projection(num_tokens, hidden, N, x, w, qkv, stream, t.ev);
        if (e != hipSuccess) return device_error("ca_qkv_projection", e);
        t.commit();
        return CA_OK;
    }
    // beyond 16 tokens: the tiled MFMA kernel (hidden and N multiples of 64)
    const ca::TiledPlan pl = ctx->projection_library ? ca::TiledPlan{}
                                                     : ca::plan_tiled_projection(num_tokens, hidden, N, ctx->num_cus);
    if (pl.ok) {
        ca::TiledPlan use = pl;
        if (ctx->proj_tile[0] > 0) {  // a forced shape, if the kernel has it and it divides the problem
            use.bm = ctx->proj_tile[0];
            use.bn = ctx->proj_tile[1];
            use.nsplit = ctx->proj_tile[2];
            if (!ca::tiled_shape_fits(use, num_tokens, hidden, N)) {
                ca::set_error("ca_qkv_projection: CA_PROJECTION_TILE does not fit this product");
                return CA_ERR_INVALID_ARG;
            }
        }
        hipError_t e = ctx->proj_part.reserve(ca::tiled_partial_bytes(use, num_tokens, N), stream);
        if (e != hipSuccess) return device_error("projection partial allocation", e);
        e = ca::launch_tiled_projection(use, num_tokens, hidden, N, x, w, qkv,
                                        static_cast<float*>(ctx->proj_part.ptr), stream, t.ev);
        if (e != hipSuccess) return device_error("ca_qkv_projection", e);
        t.commit();
        return CA_OK;
    }
    if (t.ev.start) (void)hipEventRecord(t.ev.start, stream);
    if (!ca::linear_bf16(ctx->linear, num_tokens, hidden, N, x, w, qkv, stream, &err)) {
        ca::set_error("ca_qkv_projection: " + err);
        return CA_ERR_DEVICE;
    }
    if (t.ev.stop && hipEventRecord(t.ev.stop, stream) == hipSuccess) t.commit();
    return CA_OK;
}

}  // extern "C"

namespace {

// ca_mixed_attention and ca_mixed_attention_noalloc (no_alloc: workspace in the static scratch
// array, nothing allocated; see prepare()).
ca_status attention_impl(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                         const void* q, const void* k_cache, const void* v_cache,
                         int64_t num_pool_pages, void* o, float* lse, void* hip_stream,
                         bool no_alloc) {
    if (!ctx) { ca::set_error("null ctx"); return CA_ERR_INVALID_ARG; }
    ca_status st = check_plan(plan);
    if (st != CA_OK) return st;
    Shape sh{};
    st = check_desc(desc, plan, &sh);
    if (st != CA_OK) return st;
    if (num_pool_pages <= 0) { ca::set_error("num_pool_pages must be > 0"); return CA_ERR_INVALID_ARG; }
    if (plan->num_tokens == 0) return CA_OK;
    if (!q || !k_cache || !v_cache || !o) {
        ca::set_error("ca_mixed_attention: null buffer");
        return CA_ERR_INVALID_ARG;
    }
    if (!aligned16({q, k_cache, v_cache, o}) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) {
        ca::set_error("ca_mixed_attention: device buffers must be 16-byte aligned (lse 4-byte)");
        return CA_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    st = prepare(ctx, plan, sh, num_pool_pages, stream, /*defer=*/false, /*writes=*/false, no_alloc);
    if (st != CA_OK) return st;

    const int G = sh.hq / sh.hkv;
    // the first attention launch reports that the staging slot of the launch before it may be
    // refilled (see Staging)
    const int report = ctx->staging.report_into(ctx->dplan, stream);
    struct ClearReport {
        ca::DevPlan& p;
        ~ClearReport() { p.done_flag = nullptr; }
    } clear_report{ctx->dplan};
    if (sh.dtype == CA_BF16 && G <= 16) {
        const DevWork& w = ctx->dwork;
        float* cacc = ctx->cacc;
        float2* cml = ctx->cml;
        float* dacc = ctx->dacc;
        float2* dml = ctx->dml;
        hipError_t e = hipSuccess;
        // One launch holds both kinds of work (attn_mixed.hip): decode workgroups stream the
        // decode K/V on part of the CUs while chunk workgroups run on the rest.  (Two launches on
        // two streams were measured and rejected: decode waves occupied every CU, the chunk
        // workgroups only started where a CU drained completely, and the fork/join events
        // stalled the host between steps.)  CA_SPLIT_ATTENTION=1 runs the parts as two launches
        // of the same kernel, each over the whole device, to time them separately.
        // the queue counter set of this launch, and the one it zeroes for the next queue-mode launch
        auto queue_set = [&](int k) { return ctx->queue + ((ctx->queue_parity + k) & 1) * ca::kQueueInts; };
        auto launched_queue = [&](bool queue_mode) { if (queue_mode) ctx->queue_parity ^= 1; };
        if (!ctx->split_attention) {
            Timed t(ctx->prof, "attention", CA_PROFILE_ATTENTION, !no_alloc);
            e = ca::launch_attention(ctx->dplan, sh, w.dec_wgs, w.dec_wpg, w.dec_items, w.dec_wave_items,
                                     w.num_dec_waves, w.chunk_items, w.num_chunk_items,
                                     w.num_chunk_workers, w.num_chunk_static, w.chunk_queue_mode,
                                     queue_set(0), queue_set(1), q, k_cache, v_cache, dacc, dml, cacc,
                                     cml, o, lse, stream, t.ev);
            if (e == hipSuccess) {
                t.commit();
                launched_queue(w.chunk_queue_mode && w.num_chunk_items > 0);
            }
        } else {
            if (w.num_chunk_items > 0) {
                Timed t(ctx->prof, "chunk", CA_PROFILE_ATTENTION, !no_alloc);
                e = ca::launch_attention(ctx->dplan, sh, 0, w.dec_wpg, w.dec_items, w.dec_wave_items, 0,
                                         w.chunk_items, w.num_chunk_items, w.num_chunk_workers,
                                         w.num_chunk_static, w.chunk_queue_mode, queue_set(0), queue_set(1),
                                         q, k_cache, v_cache, dacc, dml, cacc, cml, o, lse, stream,
                                         t.ev);
                if (e == hipSuccess) {
                    t.commit();
                    launched_queue(w.chunk_queue_mode);
                }
            }
            if (e == hipSuccess && w.num_dec_waves > 0) {
                Timed t(ctx->prof, "decode", CA_PROFILE_ATTENTION, !no_alloc);
                e = ca::launch_attention(ctx->dplan, sh, w.dec_wgs, w.dec_wpg, w.dec_items, w.dec_wave_items,
                                         w.num_dec_waves, w.chunk_items, 0, 0, 0, false, queue_set(0),
                                         queue_set(1), q, k_cache, v_cache, dacc, dml, cacc, cml, o,
                                         lse, stream, t.ev);
                if (e == hipSuccess) t.commit();
            }
        }
        const bool launched = (w.num_dec_waves > 0 && w.dec_wgs > 0) ||
                              (w.num_chunk_items > 0 && w.num_chunk_workers > 0);
        if (e == hipSuccess && launched) ctx->staging.reported_by_launch(report);
        if (e == hipSuccess && (w.num_merges > 0 || w.num_chunk_groups > 0)) {
            Timed t(ctx->prof, "merge", CA_PROFILE_MERGE, !no_alloc);
            e = ca::launch_merge(ctx->dplan, sh, w.merges, w.num_merges, dacc, dml, w.chunk_groups,
                                 w.num_chunk_groups, cacc, cml, o, lse, stream, t.ev);
            if (e == hipSuccess) t.commit();
        }
        if (e != hipSuccess) return device_error("attention launch", e);
        return CA_OK;
    }
    // fp32 storage, or groups wider than one MFMA tile: the plain kernel serves every row
    const int nsplit = 8;
    const size_t floats = ca::generic_partial_floats(plan->num_tokens, sh, nsplit);
    float* partial = nullptr;
    hipError_t e = hipSuccess;
    if (no_alloc) {
        if (ctx->meta_end + floats * sizeof(float) > ca::kScratchBytes) {
            ca::set_error("ca_mixed_attention_noalloc: the step needs " +
                          std::to_string(ctx->meta_end + floats * sizeof(float)) +
                          " bytes of workspace, more than the " + std::to_string(ca::kScratchBytes) +
                          "-byte scratch array");
            return CA_ERR_CAPACITY;
        }
        partial = reinterpret_cast<float*>(static_cast<char*>(ctx->scratch) + ctx->meta_end);
    } else {
        e = ctx->partial_buf.reserve(floats * sizeof(float), stream);
        if (e != hipSuccess) return device_error("partials allocation", e);
        partial = static_cast<float*>(ctx->partial_buf.ptr);
    }
    {
        Timed t(ctx->prof, "generic", CA_PROFILE_ATTENTION, !no_alloc);
        e = ca::launch_attention_generic(ctx->dplan, sh, 0, q, k_cache, v_cache, o, lse,
                                         partial, nsplit, stream,
                                         t.ev);
        if (e == hipSuccess) t.commit();
        if (e == hipSuccess) ctx->staging.reported_by_launch(report);
    }
    if (e != hipSuccess) return device_error("attention launch", e);
    return CA_OK;
}

}  // namespace

extern "C" {

ca_status ca_mixed_attention(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                             const void* q, const void* k_cache, const void* v_cache,
                             int64_t num_pool_pages, void* o, float* lse, void* hip_stream) {
    ca::clear_error();
    return attention_impl(ctx, desc, plan, q, k_cache, v_cache, num_pool_pages, o, lse, hip_stream,
                          false);
}

ca_status ca_mixed_attention_noalloc(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                                     const void* q, const void* k_cache, const void* v_cache,
                                     int64_t num_pool_pages, void* o, float* lse,
                                     void* hip_stream) {
    ca::clear_error();
    return attention_impl(ctx, desc, plan, q, k_cache, v_cache, num_pool_pages, o, lse, hip_stream,
                          true);
}

ca_status ca_plan_validate(const ca_plan* plan, int64_t num_pool_pages, int32_t flags) {
    ca::clear_error();
    ca_status st = check_plan(plan);
    if (st != CA_OK) return st;
    if (num_pool_pages <= 0) { ca::set_error("num_pool_pages must be > 0"); return CA_ERR_INVALID_ARG; }
    if (flags & ~CA_VALIDATE_WRITE_TARGETS) { ca::set_error("ca_plan_validate: unknown flags"); return CA_ERR_INVALID_ARG; }
    int32_t top = -1;
    return validate_plan_arrays(plan, num_pool_pages, (flags & CA_VALIDATE_WRITE_TARGETS) != 0, &top);
}

ca_status ca_profile_enable(ca_ctx* ctx, int enable) {
    ca::clear_error();
    if (!ctx) { ca::set_error("null ctx"); return CA_ERR_INVALID_ARG; }
    if (enable < 0 || enable > 63) { ca::set_error("ca_profile_enable: unknown flags"); return CA_ERR_INVALID_ARG; }
    ctx->prof.mask = (enable & CA_PROFILE_ALL) ? 0x3e : enable;
    if (ctx->prof.mask) {
        DeviceGuard g(ctx->device);
        if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
        ctx->prof.reserve();
    }
    return CA_OK;
}

ca_status ca_profile_read(ca_ctx* ctx, ca_profile_record* out, int32_t cap, int32_t* count) {
    ca::clear_error();
    if (!ctx || !count || (cap > 0 && !out) || cap < 0) { ca::set_error("ca_profile_read: bad arguments"); return CA_ERR_INVALID_ARG; }
    DeviceGuard g(ctx->device);
    int32_t n = 0;
    ca_status st = CA_OK;
    for (auto& r : ctx->prof.pending) {
        if (n < cap) {
            float ms = 0.0f;
            hipError_t e = hipEventSynchronize(r.b);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
            if (e != hipSuccess && st == CA_OK) st = device_error("ca_profile_read", e);
            out[n].kernel = r.name;
            out[n].ms = ms;
            ++n;
        }
        ctx->prof.pool.push_back(r.a);
        ctx->prof.pool.push_back(r.b);
    }
    ctx->prof.pending.clear();
    *count = n;
    return st;
}

const char* ca_status_string(ca_status s) {
    switch (s) {
        case CA_OK: return "ok";
        case CA_ERR_INVALID_ARG: return "invalid argument";
        case CA_ERR_NO_PAGES: return "no free KV slot for a decode";
        case CA_ERR_CAPACITY: return "plan arrays too small";
        case CA_ERR_UNSUPPORTED: return "unsupported shape";
        case CA_ERR_DEVICE: return "HIP device error";
        case CA_ERR_INTERNAL: return "internal consistency check failed";
    }
    return "unknown status";
}

const char* ca_last_error(void) { return ca::t_last_error.c_str(); }

}  // extern "C"
