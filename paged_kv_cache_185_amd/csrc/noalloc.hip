// pa_decode_noalloc: paged decode whose split partials and completion counters
// live in a fixed device array of this library instead of a caller workspace,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` is a file-scope device variable of kNoAllocScratchBytes,
// one copy per GPU, held until the process ends.  Its name is a host-side
// stand-in in host code: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels.  Layout: the decode workspace layout of pa_decode
// (completion counters in the first 64 KiB, then the partials).  The counters
// are cleared by a fill kernel at set-up and every call leaves the ones it used
// at zero, so calls of any shape can follow one another.  Calls that overlap in
// time on one GPU share the array and race.
#include <mutex>
#include <string>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int64_t n_words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

pa_status fail(pa_status st, const std::string& msg) {
    set_error("pa_decode_noalloc: " + msg);
    return st;
}

// The current device's scratch address; at the first call on a device, look it
// up and clear the counter region with a kernel on `stream`.
pa_status device_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        const int64_t words = (int64_t)kDecodeCounterBytes / 4;
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           (uint32_t*)ptr, words);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("scratch clear: ") + hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" size_t pa_decode_noalloc_scratch_bytes(void) { return pa::kNoAllocScratchBytes; }

extern "C" pa_status pa_decode_noalloc(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                                       const float* q, float* out, const int32_t* block_tables,
                                       const int32_t* kv_lens, const int32_t* block_tables_host,
                                       const int32_t* kv_lens_host, int32_t n_seqs, int32_t max_pages,
                                       int32_t n_q_heads, float scale, int32_t partition_tokens,
                                       pa_stream stream) {
    using namespace pa;
    if (!desc) return fail(PA_ERR_INVALID, "desc is null");
    if (n_seqs > 0 && desc->n_kv_heads > 0 && (int64_t)n_seqs * desc->n_kv_heads > (int64_t)kDecodeCounterBytes / 4)
        return fail(PA_ERR_UNSUPPORTED, "n_seqs * n_kv_heads above 16384 (the scratch counter region)");
    const size_t need = pa_decode_workspace_bytes(desc, n_seqs, n_q_heads, max_pages, kv_lens_host,
                                                  partition_tokens);
    if (need > kNoAllocScratchBytes)
        return fail(PA_ERR_WORKSPACE, "the split partials need " + std::to_string(need) +
                                          " bytes, more than the fixed scratch of " +
                                          std::to_string(kNoAllocScratchBytes) +
                                          " bytes (use pa_decode with a workspace)");
    // a call that launches nothing, or needs no partials, does not touch the scratch
    void* ws = nullptr;
    if (n_seqs > 0 && need > 0) {
        pa_status st = device_scratch((hipStream_t)stream, &ws);
        if (st != PA_OK) return st;
    }
    return run_decode(desc, k_cache, v_cache, q, out, block_tables, kv_lens, block_tables_host, kv_lens_host,
                      n_seqs, max_pages, n_q_heads, scale, partition_tokens, ws, ws ? kNoAllocScratchBytes : 0, stream);
}
