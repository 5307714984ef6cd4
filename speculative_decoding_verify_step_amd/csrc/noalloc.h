// noalloc.h -- spec_verify_step_noalloc: the greedy verify step for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Included at the end of
// spec_verify.hip (it uses that file's planning and launch code).
//
// The step's workspace -- the same buffers a context allocates at init, sized
// for the call's batch, without those of sampled verification and drafting --
// is carved from one file-scope device array, `scratch`, of
// NOALLOC_SCRATCH_BYTES.  The loader gives every GPU its own copy of the array,
// which it keeps until the process ends; its address on a device is looked up
// once (hipGetSymbolAddress, with that device current) and only that address
// is used from the host -- the array's name in host code is a host-side
// stand-in, not a device address.  Every call on a GPU shares that GPU's
// array, so calls that overlap in time on one GPU race.  The array keeps the
// last call's contents; each call rewrites the rotary table and clears the
// error word with kernels before the step (no memset, so the call can be
// captured into a graph).

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];   // device address of `scratch`, per device
bool g_scratch_checked[NOALLOC_MAX_DEVICES];

// Device address of this device's `scratch` (looked up on the first call).
int noalloc_scratch(int dev, char** out)
{
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(SV_ERR_UNSUPPORTED, "device index too large");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_checked[dev]) {
        int d = 0;
        int rc = check_device(&d);
        if (rc) return rc;
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SV_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
        g_scratch_checked[dev] = true;
    }
    *out = (char*)g_scratch_ptr[dev];
    return SV_OK;
}

// Rotary table (cos, sin) of pos * theta^(-2i/D) computed in double, stored
// fp32 -- the values the context's init computes on the host.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* rope, int cap, int half, float theta,
                                                         int D)
{
    const long n = (long)cap * half;
    for (long idx = blockIdx.x * 256L + threadIdx.x; idx < n; idx += (long)gridDim.x * 256) {
        const int p = (int)(idx / half), i = (int)(idx % half);
        const double ang = (double)p * pow((double)theta, -2.0 * i / D);
        rope[idx] = make_float2((float)cos(ang), (float)sin(ang));
    }
}

__global__ __launch_bounds__(64) void zero_word_kernel(unsigned* w)
{
    if (threadIdx.x == 0) *w = 0u;
}

}  // namespace

extern "C" int spec_verify_step_noalloc(const spec_verify_config* cfg, const spec_verify_weights* w,
                                        void* k_cache, void* v_cache, const int32_t* committed,
                                        const int32_t* drafts, const int32_t* ctx_in,
                                        int32_t* ctx_out, int batch, int32_t* accepted,
                                        int32_t* next_tok, uint32_t* error_word, void* stream)
{
    if (!cfg) return fail(SV_ERR_INVALID_ARG, "null config");
    int rc = validate_config(*cfg);
    if (rc) return rc;
    if (cfg->kv_page_size)
        return fail(SV_ERR_UNSUPPORTED, "paged caches need a context (spec_verify_set_kv_pages)");
    if (batch < 1 || batch > cfg->max_batch) return fail(SV_ERR_INVALID_ARG, "batch outside [1, max_batch]");
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    char* base = nullptr;
    rc = noalloc_scratch(dev, &base);
    if (rc) return rc;
    spec_verify_ctx c;     // planning only; its buffers are pieces of `scratch`
    rc = plan_context(&c, *cfg, dev);
    if (rc) return rc;
    size_t used = 0;
    carve_workspace(&c, batch, false, [&](size_t bytes) -> void* {
        const size_t at = (used + 255) & ~(size_t)255;
        used = at + bytes;
        return used <= NOALLOC_SCRATCH_BYTES ? base + at : base;   // sizes still counted past the end
    });
    if (used > NOALLOC_SCRATCH_BYTES)
        return fail(SV_ERR_UNSUPPORTED, "the step needs " + std::to_string(used) +
                                            " bytes of workspace; the no-alloc scratch holds " +
                                            std::to_string(NOALLOC_SCRATCH_BYTES));
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipSetDevice(dev));
    {
        const long n = (long)cfg->kv_capacity * (cfg->head_dim / 2);
        const unsigned blocks = (unsigned)std::min<long>((n + 255) / 256, 2048);
        rope_table_kernel<<<blocks, 256, 0, s>>>(c.rope, cfg->kv_capacity, cfg->head_dim / 2,
                                                 cfg->rope_theta, cfg->head_dim);
    }
    if (error_word) c.err_word = error_word;   // the caller's word collects the bits
    else zero_word_kernel<<<1, 64, 0, s>>>(c.err_word);
    HIP_TRY(hipGetLastError());
    return step_impl(&c, w, k_cache, v_cache, committed, drafts, ctx_in, ctx_out, batch, accepted,
                     next_tok, stream, nullptr);
}
