// api.hip -- the C ABI entry points: context, workspace, metadata upload, validation, dispatch.
//
// Host runtime around the kernels.  A step's plan is plain host data; the first device call
// that sees a new plan generation copies its metadata once (pinned staging -> device, async on
// the caller's stream), and later calls with the same generation reuse the device copy.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
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
        size_t cap = want + want / 4 + 4096;
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

// Ring of pinned host staging slots.  A slot is reused only after the copy that read it has
// completed (its event), so the host never overwrites bytes an async copy still needs.
struct Staging {
    static constexpr int kSlots = 4;
    void* host[kSlots] = {};
    size_t cap[kSlots] = {};
    hipEvent_t ev[kSlots] = {};
    bool pending[kSlots] = {};
    int next = 0;

    hipError_t init() {
        for (int i = 0; i < kSlots; ++i) {
            hipError_t e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    hipError_t acquire(size_t bytes, int* slot) {
        int i = next;
        next = (next + 1) % kSlots;
        if (pending[i]) {
            hipError_t e = hipEventSynchronize(ev[i]);
            if (e != hipSuccess) return e;
            pending[i] = false;
        }
        if (cap[i] < bytes) {
            if (host[i]) (void)hipHostFree(host[i]);
            host[i] = nullptr;
            cap[i] = 0;
            size_t want = bytes + bytes / 4 + 4096;
            hipError_t e = hipHostMalloc(&host[i], want, hipHostMallocDefault);
            if (e != hipSuccess) { host[i] = nullptr; return e; }
            cap[i] = want;
        }
        *slot = i;
        return hipSuccess;
    }
    hipError_t copy(int slot, void* dst, size_t bytes, hipStream_t stream) {
        hipError_t e = hipMemcpyAsync(dst, host[slot], bytes, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return e;
        e = hipEventRecord(ev[slot], stream);
        if (e != hipSuccess) return e;
        pending[slot] = true;
        return hipSuccess;
    }
    void release() {
        for (int i = 0; i < kSlots; ++i) {
            if (pending[i]) (void)hipEventSynchronize(ev[i]);
            if (host[i]) (void)hipHostFree(host[i]);
            if (ev[i]) (void)hipEventDestroy(ev[i]);
            host[i] = nullptr;
            ev[i] = nullptr;
        }
    }
};

}  // namespace

// Work lists of one attention call, built on the host from the plan (decode splits, merges).
struct WorkKey {
    uint64_t generation = 0;
    int32_t hq = 0, hkv = 0, d = 0, split = 0;
    bool operator==(const WorkKey& o) const {
        return generation == o.generation && hq == o.hq && hkv == o.hkv && d == o.d && split == o.split;
    }
};

struct DevWork {
    const int4* dec_items = nullptr;
    const int32_t* dec_out = nullptr;
    const int4* merges = nullptr;
    int32_t num_dec_items = 0, num_merges = 0, num_slots = 0;
};

struct ca_ctx {
    int device = 0;
    Staging staging;
    DevBuf plan_buf;        // int32: qo_indptr | kv_page_indptr | kv_last_page_len | kv_page_indices
    uint64_t plan_generation = 0;
    DevPlan dplan{};
    DevBuf partial_buf;     // fp32 split-KV partials of the generic path
    DevBuf work_buf;        // decode items | item outputs | merges
    WorkKey work_key{};
    DevWork dwork{};
    DevBuf dec_acc_buf;     // fp32 [slots][G][d]
    DevBuf dec_ml_buf;      // float2 [slots][G]
    int32_t split_override = 0;  // CA_DECODE_SPLIT (keys per decode split), 0 = automatic
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
// every index is checked here before a launch).
ca_status validate_plan_arrays(const ca_plan* plan, int64_t pool) {
    const int32_t ns = plan->num_seqs;
    const int32_t P = plan->page_size;
    if (ns == 0) return CA_OK;
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
    for (int32_t j = 0; j < plan->num_pages; ++j) {
        if (plan->kv_page_indices[j] < 0 || plan->kv_page_indices[j] >= pool) {
            ca::set_error("page index " + std::to_string(plan->kv_page_indices[j]) + " outside the pool");
            return CA_ERR_INVALID_ARG;
        }
    }
    return CA_OK;
}

// Copy the plan's metadata to the device unless this generation is already there.
ca_status upload_plan(ca_ctx* ctx, const ca_plan* plan, int64_t pool, hipStream_t stream) {
    if (plan->generation != 0 && plan->generation == ctx->plan_generation) return CA_OK;
    ca_status st = validate_plan_arrays(plan, pool);
    if (st != CA_OK) return st;
    const int32_t ns = plan->num_seqs;
    const size_t n_ints = static_cast<size_t>(ns + 1) * 2 + ns + plan->num_pages;
    const size_t bytes = n_ints * sizeof(int32_t);
    hipError_t e = ctx->plan_buf.reserve(bytes, stream);
    if (e != hipSuccess) return device_error("plan metadata allocation", e);
    int slot = 0;
    e = ctx->staging.acquire(bytes, &slot);
    if (e != hipSuccess) return device_error("staging allocation", e);
    int32_t* h = static_cast<int32_t*>(ctx->staging.host[slot]);
    std::memcpy(h, plan->qo_indptr, sizeof(int32_t) * (ns + 1));
    std::memcpy(h + (ns + 1), plan->kv_page_indptr, sizeof(int32_t) * (ns + 1));
    std::memcpy(h + 2 * (ns + 1), plan->kv_last_page_len, sizeof(int32_t) * ns);
    if (plan->num_pages)
        std::memcpy(h + 2 * (ns + 1) + ns, plan->kv_page_indices, sizeof(int32_t) * plan->num_pages);
    e = ctx->staging.copy(slot, ctx->plan_buf.ptr, bytes, stream);
    if (e != hipSuccess) return device_error("plan metadata copy", e);
    const int32_t* d = static_cast<const int32_t*>(ctx->plan_buf.ptr);
    ctx->dplan.qo_indptr = d;
    ctx->dplan.kv_page_indptr = d + (ns + 1);
    ctx->dplan.kv_last_page_len = d + 2 * (ns + 1);
    ctx->dplan.kv_page_indices = d + 2 * (ns + 1) + ns;
    ctx->dplan.num_seqs = ns;
    ctx->dplan.num_decodes = plan->num_decodes;
    ctx->dplan.num_tokens = plan->num_tokens;
    ctx->dplan.num_pages = plan->num_pages;
    ctx->dplan.page_size = plan->page_size;
    ctx->plan_generation = plan->generation;
    return CA_OK;
}

// Keys per decode split: enough work items to cover every CU several times over, in whole
// 32-key blocks, and long enough that the partial (G x (d + 2) floats) stays a few percent of
// the K/V bytes the split reads.
int32_t decode_split_keys(const ca_plan* plan, const Shape& sh, int32_t override_keys) {
    if (override_keys > 0) return ((override_keys + 31) / 32) * 32;
    int64_t total = 0;
    for (int32_t s = 0; s < plan->num_decodes; ++s) {
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        total += static_cast<int64_t>(np - 1) * plan->page_size + plan->kv_last_page_len[s];
    }
    total *= sh.hkv;
    const int64_t target_items = 6144;
    int64_t L = (total + target_items - 1) / target_items;
    L = ((L + 31) / 32) * 32;
    if (L < 256) L = 256;
    if (L > 4096) L = 4096;
    return static_cast<int32_t>(L);
}

// Build (or reuse) the decode work list of this plan and shape and copy it to the device.
ca_status prepare_decode_work(ca_ctx* ctx, const ca_plan* plan, const Shape& sh,
                              hipStream_t stream) {
    WorkKey key{plan->generation, sh.hq, sh.hkv, sh.d, decode_split_keys(plan, sh, ctx->split_override)};
    if (plan->generation != 0 && key == ctx->work_key) return CA_OK;
    const int32_t L = key.split;
    std::vector<int4> items;
    std::vector<int32_t> outs;
    std::vector<int4> merges;
    int32_t slots = 0;
    for (int32_t s = 0; s < plan->num_decodes; ++s) {
        const int32_t np = plan->kv_page_indptr[s + 1] - plan->kv_page_indptr[s];
        const int32_t kv_len = (np - 1) * plan->page_size + plan->kv_last_page_len[s];
        const int32_t nsplit = (kv_len + L - 1) / L;
        for (int32_t g = 0; g < sh.hkv; ++g) {
            if (nsplit == 1) {
                items.push_back(make_int4(s, g, 0, kv_len));
                outs.push_back(-1);
                continue;
            }
            merges.push_back(make_int4(s, g, slots, nsplit));
            for (int32_t i = 0; i < nsplit; ++i) {
                const int32_t b = i * L, e = (b + L < kv_len) ? b + L : kv_len;
                items.push_back(make_int4(s, g, b, e));
                outs.push_back(slots++);
            }
        }
    }
    const size_t n_items = items.size(), n_merges = merges.size();
    const size_t out_words = (n_items + 3) / 4 * 4;
    const size_t bytes = n_items * sizeof(int4) + out_words * sizeof(int32_t) + n_merges * sizeof(int4) + 16;
    hipError_t e = ctx->work_buf.reserve(bytes, stream);
    if (e != hipSuccess) return device_error("work list allocation", e);
    int slot = 0;
    e = ctx->staging.acquire(bytes, &slot);
    if (e != hipSuccess) return device_error("staging allocation", e);
    char* h = static_cast<char*>(ctx->staging.host[slot]);
    std::memcpy(h, items.data(), n_items * sizeof(int4));
    std::memcpy(h + n_items * sizeof(int4), outs.data(), n_items * sizeof(int32_t));
    std::memcpy(h + n_items * sizeof(int4) + out_words * sizeof(int32_t), merges.data(), n_merges * sizeof(int4));
    e = ctx->staging.copy(slot, ctx->work_buf.ptr, bytes, stream);
    if (e != hipSuccess) return device_error("work list copy", e);
    const char* d = static_cast<const char*>(ctx->work_buf.ptr);
    ctx->dwork.dec_items = reinterpret_cast<const int4*>(d);
    ctx->dwork.dec_out = reinterpret_cast<const int32_t*>(d + n_items * sizeof(int4));
    ctx->dwork.merges = reinterpret_cast<const int4*>(d + n_items * sizeof(int4) + out_words * sizeof(int32_t));
    ctx->dwork.num_dec_items = static_cast<int32_t>(n_items);
    ctx->dwork.num_merges = static_cast<int32_t>(n_merges);
    ctx->dwork.num_slots = slots;
    const int G = sh.hq / sh.hkv;
    e = ctx->dec_acc_buf.reserve(static_cast<size_t>(slots > 0 ? slots : 1) * G * sh.d * sizeof(float), stream);
    if (e != hipSuccess) return device_error("decode partial allocation", e);
    e = ctx->dec_ml_buf.reserve(static_cast<size_t>(slots > 0 ? slots : 1) * G * sizeof(float2), stream);
    if (e != hipSuccess) return device_error("decode partial allocation", e);
    ctx->work_key = key;
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
    if (const char* env = std::getenv("CA_DECODE_SPLIT")) ctx->split_override = std::atoi(env);
    e = ctx->staging.init();
    if (e != hipSuccess) {
        ctx->staging.release();
        delete ctx;
        return device_error("hipEventCreate", e);
    }
    *out = ctx;
    return CA_OK;
}

ca_status ca_destroy(ca_ctx* ctx) {
    ca::clear_error();
    if (!ctx) return CA_OK;
    DeviceGuard g(ctx->device);
    ctx->staging.release();
    ctx->plan_buf.release();
    ctx->partial_buf.release();
    ctx->work_buf.release();
    ctx->dec_acc_buf.release();
    ctx->dec_ml_buf.release();
    delete ctx;
    return CA_OK;
}

ca_status ca_append_kv_rope(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                            const void* q_in, void* q_out, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int64_t num_pool_pages,
                            void* hip_stream) {
    ca::clear_error();
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
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    st = upload_plan(ctx, plan, num_pool_pages, stream);
    if (st != CA_OK) return st;
    hipError_t e = ca::launch_append_rope(ctx->dplan, sh, q_in, q_out, k_new, v_new, k_cache,
                                          v_cache, stream);
    if (e != hipSuccess) return device_error("append_rope launch", e);
    return CA_OK;
}

ca_status ca_mixed_attention(ca_ctx* ctx, const ca_attn_desc* desc, const ca_plan* plan,
                             const void* q, const void* k_cache, const void* v_cache,
                             int64_t num_pool_pages, void* o, float* lse, void* hip_stream) {
    ca::clear_error();
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
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess) return device_error("hipSetDevice", g.err);
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    st = upload_plan(ctx, plan, num_pool_pages, stream);
    if (st != CA_OK) return st;

    const int G = sh.hq / sh.hkv;
    const bool mfma_path = sh.dtype == CA_BF16 && G <= 16;
    int32_t generic_row0 = 0;
    if (mfma_path && plan->num_decodes > 0) {
        st = prepare_decode_work(ctx, plan, sh, stream);
        if (st != CA_OK) return st;
        hipError_t e = ca::launch_decode(ctx->dplan, sh, ctx->dwork.dec_items, ctx->dwork.dec_out,
                                         ctx->dwork.num_dec_items, ctx->dwork.merges,
                                         ctx->dwork.num_merges, q, k_cache, v_cache,
                                         static_cast<float*>(ctx->dec_acc_buf.ptr),
                                         static_cast<float2*>(ctx->dec_ml_buf.ptr),
                                         o, lse, stream);
        if (e != hipSuccess) return device_error("decode attention launch", e);
        generic_row0 = plan->qo_indptr[plan->num_decodes];
    }
    if (generic_row0 < plan->num_tokens) {
        const int nsplit = 8;
        const size_t floats = ca::generic_partial_floats(plan->num_tokens, sh, nsplit);
        hipError_t e = ctx->partial_buf.reserve(floats * sizeof(float), stream);
        if (e != hipSuccess) return device_error("partials allocation", e);
        e = ca::launch_attention_generic(ctx->dplan, sh, generic_row0, q, k_cache, v_cache, o, lse,
                                         static_cast<float*>(ctx->partial_buf.ptr), nsplit, stream);
        if (e != hipSuccess) return device_error("attention launch", e);
    }
    return CA_OK;
}

const char* ca_status_string(ca_status s) {
    switch (s) {
        case CA_OK: return "ok";
        case CA_ERR_INVALID_ARG: return "invalid argument";
        case CA_ERR_NO_PAGES: return "no free KV slot for a decode";
        case CA_ERR_CAPACITY: return "plan arrays too small";
        case CA_ERR_UNSUPPORTED: return "unsupported shape";
        case CA_ERR_DEVICE: return "HIP device error";
    }
    return "unknown status";
}

const char* ca_last_error(void) { return ca::t_last_error.c_str(); }

}  // extern "C"
