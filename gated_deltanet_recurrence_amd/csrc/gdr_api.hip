// C ABI of libgdr.so: argument validation on the host, kernel selection and
// launch on the caller's stream. The operations and argument contracts are
// documented in include/gdr.h.
#include <mutex>

#include "gdr.h"
#include "gdr_common.h"

// Scratch of gdr_chunk_noalloc: one array per GPU, held until the process
// ends. In host code its name is only a stand-in for the device symbol; its
// device address is resolved per device with hipGetSymbolAddress and only
// that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device, once resolved

// Device address of `scratch` on the current device, resolved on first use.
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return p == nullptr || ((uintptr_t)p & 3u) == 0; }

// Either beta (and optionally g), or the fused gates: the logits, a, A_log and
// dt_bias together, with neither beta nor g.
gdr_status check_gates(const void *beta, const void *logits, const float *g, const void *ga, const float *A_log,
                       const float *dt_bias)
{
    if (!logits && !ga) return beta ? GDR_OK : GDR_ERR_NULL;
    if (beta || g) return GDR_ERR_SHAPE;
    if (!logits || !ga || !A_log || !dt_bias) return GDR_ERR_NULL;
    return GDR_OK;
}

// The epilogue's z and w come together; eps must be a number >= 0.
gdr_status check_norm(const void *z, const float *w, float eps)
{
    if (!z && !w) return GDR_OK;
    if (!z || !w) return GDR_ERR_NULL;
    if (!(eps >= 0.f)) return GDR_ERR_SHAPE;
    return GDR_OK;
}

gdr_status from_launch(hipError_t e, bool supported)
{
    if (!supported) return GDR_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH;
}

// The epilogue as a separate pass over out, after the call's main kernels
// (same stream).
template <typename Args>
hipError_t launch_norm_pass(const Args *a, void *stream, bool *ok)
{
    gdr::NormParams n;
    n.out = a->out; n.z = a->norm_z; n.w = a->norm_w; n.lens = a->actual_seq_lengths; n.eps = a->norm_eps;
    n.B = a->B; n.Nv = a->Nv; n.S = a->S; n.Dv = a->Dv;
    return gdr::launch_norm(a->dtype, n, (hipStream_t)stream, ok);
}

// Shared checks of the two conv calls: sizes, then the pointers every call needs.
template <typename Args>
gdr_status check_conv(const Args *a, int max_S)
{
    if (a->dtype != GDR_F32 && a->dtype != GDR_BF16 && a->dtype != GDR_F16) return GDR_ERR_DTYPE;
    if (a->B < 0 || a->S < 1 || a->S > max_S || a->Nk < 1 || a->Nv < 1 || a->Dk < 1 || a->Dv < 1 ||
        a->Nv % a->Nk != 0 || a->Dk % 2 != 0 || a->Dv % 2 != 0 || a->K < 1 || a->K > 8)
        return GDR_ERR_SHAPE;
    if (a->B == 0) return GDR_OK;
    if (!a->x || !a->weight || !a->q || !a->k || !a->v) return GDR_ERR_NULL;
    const int64_t C = 2LL * a->Nk * a->Dk + (int64_t)a->Nv * a->Dv;
    // 32-bit channel and grid arithmetic; 64-bit element offsets
    // 32-bit byte offsets within one sequence's inputs and one head's plane
    // (the prefill reads whole token blocks of at most 64, up to S + 63)
    if (C > (1LL << 30) || a->B > 65535 || ((int64_t)a->S + 64) * C * (a->dtype == GDR_F32 ? 4 : 2) > 0x7fffffffLL)
        return GDR_ERR_UNSUPPORTED;
    if (!aligned16(a->x) || !aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned4(a->weight) ||
        !aligned4(a->bias))
        return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

template <typename Args>
void conv_params(const Args *a, gdr::ConvParams &p)
{
    p.x = a->x; p.w = a->weight; p.bias = a->bias;
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.B = a->B; p.S = a->S; p.Nk = a->Nk; p.Nv = a->Nv; p.Dk = a->Dk; p.Dv = a->Dv; p.K = a->K;
    p.init = nullptr; p.fin = nullptr; p.pool = nullptr;
    p.lens = nullptr; p.idx = nullptr; p.nacc = nullptr; p.slots = 0;
}

}  // namespace

extern "C" {

int32_t gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_string(gdr_status s)
{
    switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL: return "a required pointer is NULL";
    case GDR_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case GDR_ERR_DTYPE: return "unknown element type";
    case GDR_ERR_UNSUPPORTED: return "no kernel for these head sizes, chunk size or alignment";
    case GDR_ERR_LAUNCH: return "kernel launch failed";
    case GDR_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the allocation-free entry point holds";
    }
    return "unknown status";
}

gdr_status gdr_decode(const gdr_decode_args *a, void *stream)
{
    if (!a) return GDR_ERR_NULL;
    if (a->dtype != GDR_F32 && a->dtype != GDR_BF16 && a->dtype != GDR_F16) return GDR_ERR_DTYPE;
    if (a->B < 0 || a->S < 1 || a->S > 8 || a->Nk < 1 || a->Nv < 1 || a->Dk < 1 || a->Dv < 1 ||
        a->num_slots < 1 || a->Nv % a->Nk != 0)
        return GDR_ERR_SHAPE;
    if (a->num_state_indices != (int64_t)a->B * a->S) return GDR_ERR_SHAPE;
    if (a->B == 0) return GDR_OK;
    if (!a->q || !a->k || !a->v || !a->state_pool || !a->out || !a->actual_seq_lengths ||
        !a->ssm_state_indices)
        return GDR_ERR_NULL;
    const gdr_status gs = check_gates(a->beta, a->beta_logits, a->g, a->gate_a, a->A_log, a->dt_bias);
    if (gs != GDR_OK) return gs;
    const gdr_status ns = check_norm(a->norm_z, a->norm_w, a->norm_eps);
    if (ns != GDR_OK) return ns;
    if ((int64_t)a->B * a->Nv * 2 > 0x7fffffffLL) return GDR_ERR_UNSUPPORTED;
    if (a->norm_z && !gdr::norm_supported(a->Dv, a->B, a->Nv, a->S)) return GDR_ERR_UNSUPPORTED;
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->state_pool) ||
        !aligned16(a->out) || !aligned16(a->gk) || !aligned16(a->norm_z) || !aligned16(a->norm_w) ||
        !aligned4(a->beta) || !aligned4(a->beta_logits) ||
        !aligned4(a->gate_a) || !aligned4(a->g) || !aligned4(a->A_log) || !aligned4(a->dt_bias))
        return GDR_ERR_UNSUPPORTED;

    gdr::DecodeParams p;
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.beta = a->beta ? a->beta : a->beta_logits;
    p.beta_logit = a->beta ? 0 : 1;
    p.g = a->g; p.gk = a->gk;
    p.gate_a = a->gate_a; p.A_log = a->A_log; p.dt_bias = a->dt_bias;
    p.qk_norm = a->use_qk_l2norm != 0;
    p.pool = a->state_pool;
    p.lens = a->actual_seq_lengths; p.idx = a->ssm_state_indices; p.nacc = a->num_accepted_tokens;
    p.out = a->out;
    p.scale = a->scale_value;
    p.B = a->B; p.Nk = a->Nk; p.Nv = a->Nv; p.S = a->S; p.slots = a->num_slots;
    p.norm_z = a->norm_z; p.norm_w = a->norm_w; p.norm_eps = a->norm_eps;
    bool ok = false, norm_done = false;
    hipError_t e = gdr::launch_decode(a->dtype, a->Dk, a->Dv, p, (hipStream_t)stream, &ok, &norm_done);
    if (e == hipSuccess && ok && a->norm_z && !norm_done) e = launch_norm_pass(a, stream, &ok);
    return from_launch(e, ok);
}

int64_t gdr_chunk_workspace_size(const gdr_chunk_args *a)
{
    if (!a) return -1;
    if (a->B < 0 || a->S < 0 || a->Nv < 1) return 0;
    return gdr::chunk_workspace_bytes(a->dtype, a->Dk, a->Dv, a->chunk_size, a->B, a->Nv, a->S);
}

}  // extern "C"

namespace {

// gdr_chunk and gdr_chunk_noalloc: the same validation and launch; the
// scratch is the caller's workspace, or (noalloc) the library's array.
gdr_status chunk_call(const gdr_chunk_args *a, void *stream, bool noalloc)
{
    if (!a) return GDR_ERR_NULL;
    if (a->dtype != GDR_F32 && a->dtype != GDR_BF16 && a->dtype != GDR_F16) return GDR_ERR_DTYPE;
    if (a->B < 0 || a->S < 0 || a->Nk < 1 || a->Nv < 1 || a->Dk < 1 || a->Dv < 1 ||
        a->chunk_size < 1 || a->Nv % a->Nk != 0)
        return GDR_ERR_SHAPE;
    if (a->B == 0) return GDR_OK;
    if (!a->q || !a->k || !a->v || !a->out || !a->final_state) return GDR_ERR_NULL;
    const gdr_status gs = check_gates(a->beta, a->beta_logits, a->g, a->gate_a, a->A_log, a->dt_bias);
    if (gs != GDR_OK) return gs;
    const gdr_status ns = check_norm(a->norm_z, a->norm_w, a->norm_eps);
    if (ns != GDR_OK) return ns;
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out) ||
        !aligned16(a->initial_state) || !aligned16(a->final_state) || (!noalloc && !aligned16(a->workspace)) ||
        !aligned16(a->norm_z) || !aligned16(a->norm_w) ||
        !aligned4(a->beta) || !aligned4(a->beta_logits) || !aligned4(a->gate_a) || !aligned4(a->g) ||
        !aligned4(a->A_log) || !aligned4(a->dt_bias))
        return GDR_ERR_UNSUPPORTED;
    // 32-bit offsets inside the kernels: one head plane and the chunk count.
    if ((int64_t)a->S * a->Dk * 4 > 0x7fffffffLL || (int64_t)a->S * a->Dv * 4 > 0x7fffffffLL ||
        (int64_t)a->B * a->Nv * (a->S / a->chunk_size + 1) > 0x7ffffff0LL)
        return GDR_ERR_UNSUPPORTED;
    if (a->norm_z && !gdr::norm_supported(a->Dv, a->B, a->Nv, a->S)) return GDR_ERR_UNSUPPORTED;
    const int64_t need = gdr_chunk_workspace_size(a);
    void *work = a->workspace;
    if (noalloc) {
        if (need > GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERR_SCRATCH_LIMIT;
        work = nullptr;
        if (need > 0 && scratch_address(&work) != hipSuccess) return GDR_ERR_LAUNCH;
    } else {
        if (need > 0 && !a->workspace) return GDR_ERR_NULL;
        if (need > a->workspace_bytes) return GDR_ERR_SHAPE;
    }

    gdr::ChunkParams p;
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.beta = a->beta ? a->beta : a->beta_logits;
    p.beta_logit = a->beta ? 0 : 1;
    p.g = a->g;
    p.gate_a = a->gate_a; p.A_log = a->A_log; p.dt_bias = a->dt_bias;
    p.qk_norm = a->use_qk_l2norm != 0;
    p.init = a->initial_state;
    p.lens = a->actual_seq_lengths;
    p.out = a->out;
    p.fin = a->final_state;
    p.work = work;
    p.scale = a->scale_value;
    p.B = a->B; p.Nk = a->Nk; p.Nv = a->Nv; p.S = a->S;
    bool ok = false;
    hipError_t e = gdr::launch_chunk(a->dtype, a->Dk, a->Dv, a->chunk_size, p, (hipStream_t)stream, &ok);
    if (e == hipSuccess && ok && a->norm_z) e = launch_norm_pass(a, stream, &ok);
    return from_launch(e, ok);
}

}  // namespace

extern "C" {

gdr_status gdr_chunk(const gdr_chunk_args *a, void *stream) { return chunk_call(a, stream, false); }

gdr_status gdr_chunk_noalloc(const gdr_chunk_args *a, void *stream) { return chunk_call(a, stream, true); }

gdr_status gdr_conv_prefill(const gdr_conv_prefill_args *a, void *stream)
{
    if (!a) return GDR_ERR_NULL;
    const gdr_status cs = check_conv(a, 0x7fffffff);
    if (cs != GDR_OK || a->B == 0) return cs;
    if (!aligned16(a->initial_state) || !aligned16(a->final_state)) return GDR_ERR_UNSUPPORTED;
    if ((a->S + 63) / 64 > 65535) return GDR_ERR_UNSUPPORTED;
    gdr::ConvParams p;
    conv_params(a, p);
    p.init = a->initial_state; p.fin = a->final_state; p.lens = a->actual_seq_lengths;
    bool ok = false;
    hipError_t e = gdr::launch_conv_prefill(a->dtype, p, (hipStream_t)stream, &ok);
    return from_launch(e, ok);
}

gdr_status gdr_conv_decode(const gdr_conv_decode_args *a, void *stream)
{
    if (!a) return GDR_ERR_NULL;
    if (a->num_slots < 1 && a->B > 0) return GDR_ERR_SHAPE;
    if (a->num_state_indices != (int64_t)a->B * a->S) return GDR_ERR_SHAPE;
    const gdr_status cs = check_conv(a, 8);
    if (cs != GDR_OK || a->B == 0) return cs;
    if (!a->state_pool || !a->actual_seq_lengths || !a->ssm_state_indices) return GDR_ERR_NULL;
    if (!aligned16(a->state_pool)) return GDR_ERR_UNSUPPORTED;
    gdr::ConvParams p;
    conv_params(a, p);
    p.pool = a->state_pool; p.lens = a->actual_seq_lengths; p.idx = a->ssm_state_indices;
    p.nacc = a->num_accepted_tokens; p.slots = a->num_slots;
    bool ok = false;
    hipError_t e = gdr::launch_conv_decode(a->dtype, p, (hipStream_t)stream, &ok);
    return from_launch(e, ok);
}

}  // extern "C"
