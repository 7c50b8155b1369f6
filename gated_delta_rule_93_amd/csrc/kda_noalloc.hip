// kda_noalloc.hip -- kda_fwd for callers that cannot allocate device memory.
//
// kda_fwd_noalloc runs the prefill of kda_fwd with the library's own fixed device scratch in place
// of a caller-supplied workspace: a file-scope device array of kScratchBytes per GPU, held from the
// library's first use of it on that GPU until the process ends.  It calls no allocator: the
// array's device address is looked up once per device (hipGetSymbolAddress) and kept.  The chunks
// run in windows as large as the scratch holds (see kda_fwd), so any sequence length fits;
// sizes whose smallest window does not fit are refused before anything is launched.
//
// Every call on one GPU uses that GPU's one array and leaves its contents there.  Nothing in it
// needs to start at zero: each window's records are written before they are read, and the
// carried states are written by a sequence's first window before later windows read them.  Calls
// that overlap on one GPU (on different streams, or from different host threads without ordering
// between their streams) race on the array.
#include <atomic>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on the first call there.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

kda_status_t kda_fwd_noalloc(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                             int N, const void *q, const void *k, const void *v, const float *g, const float *beta,
                             float scale, const float *initial_state, float *final_state, void *o,
                             hipStream_t stream) {
    // Every argument of kda_fwd is checked first (with a stand-in workspace that is never
    // dereferenced and large enough for any size), then sizes whose smallest window does not fit
    // the scratch are refused, all before the scratch is looked up or anything is launched.
    void *const stand_in = reinterpret_cast<void *>((uintptr_t)256);
    const kda_status_t st = kda::fwd_check_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta,
                                                initial_state, final_state, o, stand_in, SIZE_MAX);
    if (st != KDA_OK) return st;
    const size_t need = kda_fwd_workspace_min_bytes(io, B, T, H, d_k, d_v, N, cu_seqlens != nullptr,
                                                    final_state != nullptr);
    if (need > kScratchBytes) return KDA_ERR_TOO_LARGE;
    if ((long)N * H == 0) return KDA_OK;
    void *ws = scratch_ptr();
    if (!ws) return KDA_ERR_LAUNCH;
    return kda_fwd(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, scale, initial_state, final_state, o, ws,
                   kScratchBytes, stream);
}

}  // extern "C"
