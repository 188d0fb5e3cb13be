// pa_vkv.hip -- KV storage on HIP virtual memory, one contiguous virtual
// range per request slot, with physical pages mapped as sequences grow.
//
// This is the vAttention design: virtual address space is reserved up front
// for every (layer, K/V) buffer of max_batch x max_context tokens, request
// slot r owns the sub-range starting at r * request_bytes, and physical pages
// are created and mapped into a slot's range only when its sequence needs
// them.  Kernels then see an ordinary contiguous tensor per request: no block
// table.  [論文解説: vAttention, 技術的詳細 › CUDA Virtual Memory Management
//  APIの活用; 仮想メモリの事前予約; リクエスト単位のKVキャッシュインデキシング;
//  Demand Paging vs Pre-allocation (deferred reclamation)]
//
// Inside a request's range the tokens are stored in the library's block
// format (16-token tiles per kv head), so the decode kernels run unchanged
// with "physical block = slot * stride + logical block" instead of a table
// lookup.  The HIP calls used: hipMemAddressReserve, hipMemCreate,
// hipMemMap, hipMemSetAccess, hipMemUnmap, hipMemRelease, hipMemAddressFree.
#include <chrono>
#include <stdio.h>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

struct pa_vkv {
    int layers = 0, max_batch = 0, max_ctx = 0, Hkv = 0, D = 0, dtype = 0, elem = 0, device = 0;
    int64_t page = 0;           // bytes per physical page
    int64_t block_bytes = 0;    // one 16-token block of all kv heads
    int64_t request_bytes = 0;  // stride between request slots (a whole number of pages)
    int req_stride = 0;         // the same in blocks
    int pages_per_req = 0;
    std::vector<char *> bufs;   // 2 * layers reserved ranges: K then V of each layer
    std::vector<int> mapped_pages;                         // [max_batch]
    std::vector<char> in_use;                              // [max_batch]
    std::vector<hipMemGenericAllocationHandle_t> handles;  // [2 * layers][max_batch][pages]
    int *d_mapped = nullptr;    // device int32 [max_batch]: tokens backed by memory
    double create_us = 0, map_us = 0;
    int64_t pages_created = 0;
};

namespace {

int fail(int status, const char *msg) { return pa::api_fail(status, msg); }
int hfail(hipError_t e, const char *where) {
    (void)hipGetLastError();
    return pa::api_hip_fail(e, where);
}

int elem_of(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_F16 || dtype == PA_BF16) ? 2 : 0; }

hipMemAllocationProp page_prop(int device) {
    hipMemAllocationProp prop{};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = device;
    return prop;
}

hipMemGenericAllocationHandle_t &handle_at(pa_vkv *v, int buf, int r, int p) {
    return v->handles[((size_t)buf * v->max_batch + r) * v->pages_per_req + p];
}

int tokens_backed(const pa_vkv *v, int pages) {
    const int64_t blocks = (int64_t)pages * v->page / v->block_bytes;
    const int64_t t = blocks * 16;
    return (int)(t < v->max_ctx ? t : v->max_ctx);
}

// Unmap and release pages [from, mapped) of slot r in every buffer.
int unmap_slot(pa_vkv *v, int r, int from) {
    for (size_t b = 0; b < v->bufs.size(); ++b) {
        for (int p = from; p < v->mapped_pages[r]; ++p) {
            char *addr = v->bufs[b] + r * v->request_bytes + (int64_t)p * v->page;
            hipError_t e = hipMemUnmap(addr, v->page);
            if (e != hipSuccess) return hfail(e, "pa_vkv: hipMemUnmap");
            e = hipMemRelease(handle_at(v, (int)b, r, p));
            if (e != hipSuccess) return hfail(e, "pa_vkv: hipMemRelease");
            handle_at(v, (int)b, r, p) = hipMemGenericAllocationHandle_t{};
        }
    }
    v->mapped_pages[r] = from;
    return PA_OK;
}

int upload_mapped(pa_vkv *v) {
    std::vector<int> t(v->max_batch);
    for (int r = 0; r < v->max_batch; ++r) t[r] = tokens_backed(v, v->mapped_pages[r]);
    hipError_t e = hipMemcpy(v->d_mapped, t.data(), t.size() * sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hfail(e, "pa_vkv: hipMemcpy");
    return PA_OK;
}

void teardown(pa_vkv *v) {
    for (int r = 0; r < v->max_batch && !v->handles.empty(); ++r) (void)unmap_slot(v, r, 0);
    for (char *b : v->bufs)
        if (b) (void)hipMemAddressFree(b, (size_t)v->max_batch * v->request_bytes);
    if (v->d_mapped) (void)hipFree(v->d_mapped);
    (void)hipGetLastError();
    delete v;
}

}  // namespace

// Page allocations one storage may hold at most (see pa_vkv_create).
constexpr int64_t kMaxPages = 24576;

int pa_vkv_create(int num_layers, int max_batch, int max_context_len, int num_kv_heads,
                  int head_dim, int dtype, int64_t page_bytes, pa_vkv **out) {
    if (!out) return fail(PA_ERR_INVALID_ARG, "pa_vkv_create: null handle pointer");
    *out = nullptr;
    const int e = elem_of(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "pa_vkv_create: unknown dtype");
    if (num_layers <= 0 || max_batch <= 0 || max_context_len <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || page_bytes < 0)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_create: sizes must be positive");
    if (max_context_len % 16 != 0 || head_dim % (16 / e) != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_create: max_context_len must be a multiple of "
                    "16 and head_dim of 16 bytes");
    const int64_t block_bytes = 16LL * num_kv_heads * head_dim * e;
    const int64_t S = (int64_t)(max_context_len / 16) * block_bytes;
    if ((int64_t)max_batch * S > ((int64_t)1 << 42))
        return fail(PA_ERR_UNSUPPORTED, "pa_vkv_create: more than 4 TiB per buffer");

    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hfail(err, "pa_vkv_create: hipGetDevice");
    int vmm = 0;
    err = hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, dev);
    if (err != hipSuccess) return hfail(err, "pa_vkv_create: hipDeviceGetAttribute");
    if (!vmm) return fail(PA_ERR_UNSUPPORTED, "pa_vkv_create: no virtual memory management");
    const hipMemAllocationProp prop = page_prop(dev);
    size_t gran = 0, recommended = 0;
    err = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum);
    if (err != hipSuccess || gran == 0) return hfail(err, "pa_vkv_create: granularity");
    err = hipMemGetAllocationGranularity(&recommended, &prop,
                                         hipMemAllocationGranularityRecommended);
    if (err != hipSuccess || recommended == 0 || recommended % gran != 0) {
        (void)hipGetLastError();
        recommended = gran;
    }
    // MI355X reports 4 KiB; mapping costs tens of microseconds per page
    // whatever its size, so the default page is at least 2 MiB
    int64_t def_page = (int64_t)recommended;
    while (def_page < (2 << 20)) def_page *= 2;
    const int64_t page = page_bytes ? page_bytes : def_page;
    if (page % (int64_t)gran != 0)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_create: page_bytes is not a multiple of the "
                    "device's allocation granularity");
    const int64_t req_bytes = (S + page - 1) / page * page;
    if (req_bytes % block_bytes != 0 || req_bytes / block_bytes > 0x7fffffff / max_batch)
        return fail(PA_ERR_UNSUPPORTED, "pa_vkv_create: pages and 16-token blocks do not tile "
                    "a request's range");
    // Every page is a physical allocation of its own (hipMemCreate), and the
    // runtime holds at most ~32K of them per process (on MI355X with ROCm
    // 7.2 the 32,757th fails, whatever the page size and free memory).  The
    // storage may map a page in every slot of every buffer, so refuse page
    // sizes whose worst case passes kMaxPages, and name one that fits.
    const int64_t worst = 2LL * num_layers * max_batch * (req_bytes / page);
    if (worst > kMaxPages) {
        int64_t fit = (int64_t)gran;
        while (2LL * num_layers * max_batch * ((S + fit - 1) / fit) > kMaxPages) fit *= 2;
        char msg[320];
        snprintf(msg, sizeof msg,
                 "pa_vkv_create: %lld-byte pages need up to %lld page allocations (2 x %d "
                 "layers x %d slots x %lld pages), past the %lld this library allows per "
                 "storage (the runtime holds about 32K per process); use pages of at least "
                 "%lld bytes",
                 (long long)page, (long long)worst, num_layers, max_batch,
                 (long long)(req_bytes / page), (long long)kMaxPages, (long long)fit);
        return fail(PA_ERR_UNSUPPORTED, msg);
    }

    pa_vkv *v = new pa_vkv;
    v->layers = num_layers;
    v->max_batch = max_batch;
    v->max_ctx = max_context_len;
    v->Hkv = num_kv_heads;
    v->D = head_dim;
    v->dtype = dtype;
    v->elem = e;
    v->device = dev;
    v->page = page;
    v->block_bytes = block_bytes;
    v->request_bytes = req_bytes;
    v->req_stride = (int)(req_bytes / block_bytes);
    v->pages_per_req = (int)(req_bytes / page);
    v->mapped_pages.assign(max_batch, 0);
    v->in_use.assign(max_batch, 0);
    v->handles.assign((size_t)2 * num_layers * max_batch * v->pages_per_req,
                      hipMemGenericAllocationHandle_t{});
    const size_t buf_bytes = (size_t)max_batch * req_bytes;
    for (int b = 0; b < 2 * num_layers; ++b) {
        void *p = nullptr;
        err = hipMemAddressReserve(&p, buf_bytes, (size_t)page, nullptr, 0);
        if (err != hipSuccess) {
            teardown(v);
            return hfail(err, "pa_vkv_create: hipMemAddressReserve");
        }
        v->bufs.push_back((char *)p);
    }
    err = hipMalloc((void **)&v->d_mapped, sizeof(int) * max_batch);
    if (err != hipSuccess) {
        teardown(v);
        return fail(PA_ERR_NO_MEMORY, "pa_vkv_create: hipMalloc of the mapped-token array");
    }
    const int rc = upload_mapped(v);
    if (rc != PA_OK) {
        teardown(v);
        return rc;
    }
    *out = v;
    return PA_OK;
}

int pa_vkv_info(const pa_vkv *v, int64_t *page_bytes, int64_t *request_stride_blocks,
                int64_t *mapped_bytes, double *create_us_per_page, double *map_us_per_page) {
    if (!v) return fail(PA_ERR_INVALID_ARG, "pa_vkv_info: null handle");
    int64_t pages = 0;
    for (int r = 0; r < v->max_batch; ++r) pages += v->mapped_pages[r];
    if (page_bytes) *page_bytes = v->page;
    if (request_stride_blocks) *request_stride_blocks = v->req_stride;
    if (mapped_bytes) *mapped_bytes = pages * (int64_t)v->bufs.size() * v->page;
    const double n = v->pages_created ? (double)v->pages_created : 1.0;
    if (create_us_per_page) *create_us_per_page = v->create_us / n;
    if (map_us_per_page) *map_us_per_page = v->map_us / n;
    return PA_OK;
}

int pa_vkv_layer(const pa_vkv *v, int layer, void **k_cache, void **v_cache) {
    if (!v || !k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "pa_vkv_layer: null pointer");
    if (layer < 0 || layer >= v->layers)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_layer: layer out of range");
    *k_cache = v->bufs[2 * layer];
    *v_cache = v->bufs[2 * layer + 1];
    return PA_OK;
}

int pa_vkv_alloc_reqid(pa_vkv *v, int *req_id) {
    if (!v || !req_id) return fail(PA_ERR_INVALID_ARG, "pa_vkv_alloc_reqid: null pointer");
    // a free slot whose pages are still mapped first (deferred reclamation)
    int best = -1;
    for (int r = 0; r < v->max_batch; ++r)
        if (!v->in_use[r] && (best < 0 || v->mapped_pages[r] > v->mapped_pages[best])) best = r;
    if (best < 0) return fail(PA_ERR_NO_MEMORY, "pa_vkv_alloc_reqid: every slot is in use");
    v->in_use[best] = 1;
    *req_id = best;
    return PA_OK;
}

int pa_vkv_free_reqid(pa_vkv *v, int req_id) {
    if (!v) return fail(PA_ERR_INVALID_ARG, "pa_vkv_free_reqid: null handle");
    if (req_id < 0 || req_id >= v->max_batch || !v->in_use[req_id])
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_free_reqid: slot not in use");
    v->in_use[req_id] = 0;  // its pages stay mapped until pa_vkv_reclaim
    return PA_OK;
}

int pa_vkv_step(pa_vkv *v, const int32_t *seq_lens) {
    if (!v || !seq_lens) return fail(PA_ERR_INVALID_ARG, "pa_vkv_step: null pointer");
    for (int r = 0; r < v->max_batch; ++r)
        if (seq_lens[r] < 0 || seq_lens[r] > v->max_ctx)
            return fail(PA_ERR_INVALID_ARG, "pa_vkv_step: a length is outside [0, max_context]");
    hipError_t err = hipSetDevice(v->device);
    if (err != hipSuccess) return hfail(err, "pa_vkv_step: hipSetDevice");
    const hipMemAllocationProp prop = page_prop(v->device);
    hipMemAccessDesc access{};
    access.location.type = hipMemLocationTypeDevice;
    access.location.id = v->device;
    access.flags = hipMemAccessFlagsProtReadWrite;
    bool grew = false;
    for (int r = 0; r < v->max_batch; ++r) {
        const int64_t need_bytes = (int64_t)((seq_lens[r] + 15) / 16) * v->block_bytes;
        const int need = (int)((need_bytes + v->page - 1) / v->page);
        while (v->mapped_pages[r] < need) {
            const int p = v->mapped_pages[r];
            for (size_t b = 0; b < v->bufs.size(); ++b) {
                char *addr = v->bufs[b] + r * v->request_bytes + (int64_t)p * v->page;
                hipMemGenericAllocationHandle_t h{};
                const auto t0 = std::chrono::steady_clock::now();
                err = hipMemCreate(&h, (size_t)v->page, &prop, 0);
                const auto t1 = std::chrono::steady_clock::now();
                if (err != hipSuccess) {
                    (void)hipGetLastError();
                    // undo this page in the buffers done so far, then report
                    for (size_t c = 0; c < b; ++c) {
                        char *a2 = v->bufs[c] + r * v->request_bytes + (int64_t)p * v->page;
                        (void)hipMemUnmap(a2, v->page);
                        (void)hipMemRelease(handle_at(v, (int)c, r, p));
                    }
                    if (grew) (void)upload_mapped(v);
                    char msg[200];
                    snprintf(msg, sizeof msg,
                             "pa_vkv_step: hipMemCreate failed after %lld pages (out of device "
                             "memory, or of the runtime's ~32K allocations per process)",
                             (long long)v->pages_created);
                    return fail(PA_ERR_NO_MEMORY, msg);
                }
                err = hipMemMap(addr, (size_t)v->page, 0, h, 0);
                if (err == hipSuccess) err = hipMemSetAccess(addr, (size_t)v->page, &access, 1);
                const auto t2 = std::chrono::steady_clock::now();
                if (err != hipSuccess) {
                    (void)hipMemUnmap(addr, v->page);
                    (void)hipMemRelease(h);
                    for (size_t c = 0; c < b; ++c) {
                        char *a2 = v->bufs[c] + r * v->request_bytes + (int64_t)p * v->page;
                        (void)hipMemUnmap(a2, v->page);
                        (void)hipMemRelease(handle_at(v, (int)c, r, p));
                    }
                    if (grew) (void)upload_mapped(v);
                    return hfail(err, "pa_vkv_step: hipMemMap / hipMemSetAccess");
                }
                handle_at(v, (int)b, r, p) = h;
                v->create_us += std::chrono::duration<double, std::micro>(t1 - t0).count();
                v->map_us += std::chrono::duration<double, std::micro>(t2 - t1).count();
                ++v->pages_created;
            }
            ++v->mapped_pages[r];
            grew = true;
        }
    }
    return grew ? upload_mapped(v) : PA_OK;
}

int pa_vkv_reclaim(pa_vkv *v) {
    if (!v) return fail(PA_ERR_INVALID_ARG, "pa_vkv_reclaim: null handle");
    hipError_t err = hipSetDevice(v->device);
    if (err == hipSuccess) err = hipDeviceSynchronize();  // no kernel may still use the pages
    if (err != hipSuccess) return hfail(err, "pa_vkv_reclaim: hipDeviceSynchronize");
    for (int r = 0; r < v->max_batch; ++r) {
        if (v->in_use[r] || v->mapped_pages[r] == 0) continue;
        const int rc = unmap_slot(v, r, 0);
        if (rc != PA_OK) return rc;
    }
    return upload_mapped(v);
}

int pa_vkv_destroy(pa_vkv *v) {
    if (!v) return PA_OK;
    hipError_t err = hipSetDevice(v->device);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err != hipSuccess) return hfail(err, "pa_vkv_destroy: hipDeviceSynchronize");
    teardown(v);
    return PA_OK;
}

int pa_vkv_write_kv(const pa_vkv *v, int layer, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, int64_t num_tokens, void *stream) {
    if (!v) return fail(PA_ERR_INVALID_ARG, "pa_vkv_write_kv: null handle");
    if (layer < 0 || layer >= v->layers)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_write_kv: layer out of range");
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_vkv_write_kv: num_tokens < 0");
    if (num_tokens == 0) return PA_OK;
    if (!k_new || !v_new || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_write_kv: null pointer");
    if (((uintptr_t)k_new & 15u) || ((uintptr_t)v_new & 15u) || ((uintptr_t)slot_mapping & 7u))
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_write_kv: data pointers must be 16-byte aligned");
    const int64_t NB = (int64_t)v->max_batch * v->req_stride;
    const int NC = v->D * v->elem / 16;
    if (NC > 256 || (num_tokens + (256 / NC) - 1) / (256 / NC) * v->Hkv > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "pa_vkv_write_kv: too many tokens for one launch");
    hipError_t err = pa::launch_write_kv(k_new, v_new, v->bufs[2 * layer], v->bufs[2 * layer + 1],
                                         slot_mapping, num_tokens, v->Hkv, v->D, 16, NB, v->elem,
                                         (hipStream_t)stream, v->d_mapped, v->req_stride,
                                         v->max_batch);
    if (err != hipSuccess) return hfail(err, "pa_vkv_write_kv launch");
    return PA_OK;
}

int pa_vkv_decode(const pa_vkv *v, int layer, const void *q, const int32_t *req_ids,
                  const int32_t *context_lens, float scale, void *out, int num_seqs,
                  int num_heads, int partition_tokens, void *stream) {
    if (!v) return fail(PA_ERR_INVALID_ARG, "pa_vkv_decode: null handle");
    if (layer < 0 || layer >= v->layers)
        return fail(PA_ERR_INVALID_ARG, "pa_vkv_decode: layer out of range");
    pa::Contiguous c{req_ids, v->d_mapped, v->req_stride, v->max_batch};
    return pa::decode_impl(q, v->bufs[2 * layer], v->bufs[2 * layer + 1], nullptr, context_lens,
                           scale, out, num_seqs, num_heads, v->Hkv, v->D, 16, v->max_ctx / 16,
                           (int64_t)v->max_batch * v->req_stride, v->dtype, partition_tokens, 0,
                           stream, &c);
}
