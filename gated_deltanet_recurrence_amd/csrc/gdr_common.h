// Internal declarations shared by the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Kernel-side view of a decode call (all device pointers; sizes validated on the host).
// beta points at beta or, when beta_logit is set, at the gate logits b; gate_a
// (dtype), A_log and dt_bias (float32) are set when g is formed in the kernel.
struct DecodeParams {
    const void *q, *k, *v, *beta;
    const float *g, *gk;
    void *pool;
    const int32_t *lens, *idx, *nacc;
    void *out;
    const void *gate_a;
    const float *A_log, *dt_bias;
    float scale;
    int32_t B, Nk, Nv, S, slots;
    int32_t beta_logit;
    int32_t qk_norm;     // q and k replaced by x / sqrt(sum(x^2) + 1e-6) in the kernel
    // Gated RMSNorm epilogue (norm_z NULL: none): z in dtype, w float32.
    const void *norm_z;
    const float *norm_w;
    float norm_eps;
};

// Kernel-side view of a chunked prefill call.
// Gates as in DecodeParams.
struct ChunkParams {
    const void *q, *k, *v, *beta;
    const float *g;
    const void *init;
    const int32_t *lens;
    void *out;
    void *fin;
    void *work;        // caller's workspace (per-chunk T blocks of the matrix-core path)
    const void *gate_a;
    const float *A_log, *dt_bias;
    float scale;
    int32_t B, Nk, Nv, S;
    int32_t beta_logit;
    int32_t qk_norm;     // as in DecodeParams
};

// The gated RMSNorm epilogue as a pass of its own over the rows of out
// (B, Nv, S, Dv): rows t < clamp(lens[b], 0, S) (all S when lens is NULL) are
// replaced in place; the others are left alone.
struct NormParams {
    void *out;
    const void *z;
    const float *w;
    const int32_t *lens;
    float eps;
    int32_t B, Nv, S, Dv;
};

// Bytes of workspace the chunk launcher needs for these sizes (0: none).
int64_t chunk_workspace_bytes(int dtype, int Dk, int Dv, int C, int B, int Nv, int S);

// Launchers: return hipSuccess or the launch error. dtype: 0 = f32, 1 = bf16.
// Depthwise causal conv1d + SiLU with the q/k/v split (prefill: init/fin per
// sequence; decode: pool with the recurrence's slot rule).
struct ConvParams {
    const void *x;
    const float *w, *bias;
    const void *init;
    void *fin;
    void *pool;
    const int32_t *lens, *idx, *nacc;
    void *q, *k, *v;
    int32_t B, S, Nk, Nv, Dk, Dv, K, slots;
};
hipError_t launch_conv_prefill(int dtype, const ConvParams &p, hipStream_t s, bool *supported);
hipError_t launch_conv_decode(int dtype, const ConvParams &p, hipStream_t s, bool *supported);

// launch_decode sets *norm_done when the chosen kernel applied the epilogue itself.
hipError_t launch_decode(int dtype, int Dk, int Dv, const DecodeParams &p, hipStream_t s, bool *supported,
                         bool *norm_done);
hipError_t launch_chunk(int dtype, int Dk, int Dv, int C, const ChunkParams &p, hipStream_t s, bool *supported);
hipError_t launch_norm(int dtype, const NormParams &p, hipStream_t s, bool *supported);
// Whether launch_norm can take these sizes (checked before a call enqueues anything).
bool norm_supported(int Dv, int B, int Nv, int S);

// ---------------------------------------------------------------------------
// Element access helpers (device). The 16-bit I/O formats are bf16 (8-bit
// significand, float32's range) and IEEE fp16 (11-bit significand). Their
// values travel as raw 16-bit patterns, two to a 32-bit word (the first in
// the low half); widening to float32 is exact, narrowing rounds to nearest
// even through the hardware converters.
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;   // bf16 storage (bit pattern)
typedef _Float16 f16_t;    // fp16 storage

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats narrowed by one v_cvt_pk_bf16_f32 (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// The two 16-bit formats behind one interface, for the kernels written for
// either: lo / hi widen the elements of a word, pack narrows two floats into
// one, dot2 is the hardware two-term dot product (exact products, float32
// sum: v_dot2_f32_bf16 / v_dot2_f32_f16), to / from convert one element.
struct BF16 {
    typedef bf16_t T;
    typedef __bf16 E;
    static constexpr int dtype = 1;
    static __device__ __forceinline__ float lo(uint32_t u) { return bf16_lo(u); }
    static __device__ __forceinline__ float hi(uint32_t u) { return bf16_hi(u); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
    }
    static __device__ __forceinline__ float to(uint32_t bits) { return __uint_as_float(bits << 16); }
    static __device__ __forceinline__ uint16_t from(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};
struct F16 {
    typedef f16_t T;
    typedef _Float16 E;
    static constexpr int dtype = 2;
    static __device__ __forceinline__ float lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)u); }
    static __device__ __forceinline__ float hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }
    static __device__ __forceinline__ uint32_t pack(float a, float b)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
    }
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
    {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
    }
    static __device__ __forceinline__ float to(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }
    static __device__ __forceinline__ uint16_t from(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};
// Trait of a storage type.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> { typedef BF16 type; };
template <> struct Elem<f16_t> { typedef F16 type; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

// Fused gates (the Gated DeltaNet blog post's layer code; inferencelayer
// deltanet.rs, module header and its softplus): beta = sigmoid(b) and
// g = -exp(A_log) softplus(a + dt_bias), in float32.
__device__ __forceinline__ float gate_sigmoid(float b) { return 1.f / (1.f + __expf(-b)); }
// ln(1 + e^x); beyond |x| = 20 one of the two terms is below float32
// resolution and the result is x or e^x.
__device__ __forceinline__ float gate_softplus(float x)
{
    return x > 20.f ? x : (x < -20.f ? __expf(x) : __logf(1.f + __expf(x)));
}
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias)
{
    return -__expf(A_log) * gate_softplus(a + dt_bias);
}
// In-kernel q/k normalisation: 1 / sqrt(|x|^2 + 1e-6) (the blog post's l2norm;
// deltanet.rs l2norm, eps inside the square root).
constexpr float QK_NORM_EPS = 1e-6f;
__device__ __forceinline__ float qk_rnorm(float sumsq) { return rsqrtf(sumsq + QK_NORM_EPS); }

// Gated RMSNorm epilogue (inferencelayer deltanet.rs, the per-head gated
// RMSNorm): o_j w_j silu(z_j) / sqrt(mean(o^2) + eps), silu(x) = x / (1 + e^-x).
// An all-zero row stays zero: its factor is taken as 0 when mean + eps is 0.
__device__ __forceinline__ float norm_silu(float z) { return z / (1.f + __expf(-z)); }
__device__ __forceinline__ float norm_rinv(float sumsq, int Dv, float eps)
{
    const float m = sumsq / (float)Dv + eps;
    return m > 0.f ? 1.f / sqrtf(m) : 0.f;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x)
{
    __bf16 y = (__bf16)x;
    return __builtin_bit_cast(uint16_t, y);
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (_Float16)x; }

// Loads N consecutive elements (N * sizeof(T) in {4, 8, 16} bytes, aligned) as floats.
template <typename T, int N> struct VecIO;

template <> struct VecIO<float, 4> {
    static __device__ __forceinline__ void load(const float *p, float *o)
    {
        float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *o)
    {
        *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
    }
};
template <> struct VecIO<float, 2> {
    static __device__ __forceinline__ void load(const float *p, float *o)
    {
        float2 v = *reinterpret_cast<const float2 *>(p);
        o[0] = v.x; o[1] = v.y;
    }
    static __device__ __forceinline__ void store(float *p, const float *o)
    {
        *reinterpret_cast<float2 *>(p) = make_float2(o[0], o[1]);
    }
};
template <> struct VecIO<float, 1> {
    static __device__ __forceinline__ void load(const float *p, float *o) { o[0] = *p; }
    static __device__ __forceinline__ void store(float *p, const float *o) { *p = o[0]; }
};
// 16-bit elements (bf16 or fp16), through their trait.
template <typename T, int N, typename EL = typename Elem<T>::type> struct VecIO16;
template <typename T, typename EL> struct VecIO16<T, 8, EL> {
    static __device__ __forceinline__ void load(const T *p, float *o)
    {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        o[0] = EL::lo(v.x); o[1] = EL::hi(v.x); o[2] = EL::lo(v.y); o[3] = EL::hi(v.y);
        o[4] = EL::lo(v.z); o[5] = EL::hi(v.z); o[6] = EL::lo(v.w); o[7] = EL::hi(v.w);
    }
    static __device__ __forceinline__ void store(T *p, const float *o)
    {
        *reinterpret_cast<uint4 *>(p) = make_uint4(EL::pack(o[0], o[1]), EL::pack(o[2], o[3]),
                                                   EL::pack(o[4], o[5]), EL::pack(o[6], o[7]));
    }
};
template <typename T, typename EL> struct VecIO16<T, 4, EL> {
    static __device__ __forceinline__ void load(const T *p, float *o)
    {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        o[0] = EL::lo(v.x); o[1] = EL::hi(v.x); o[2] = EL::lo(v.y); o[3] = EL::hi(v.y);
    }
    static __device__ __forceinline__ void store(T *p, const float *o)
    {
        *reinterpret_cast<uint2 *>(p) = make_uint2(EL::pack(o[0], o[1]), EL::pack(o[2], o[3]));
    }
};
template <typename T, typename EL> struct VecIO16<T, 2, EL> {
    static __device__ __forceinline__ void load(const T *p, float *o)
    {
        uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        o[0] = EL::lo(v); o[1] = EL::hi(v);
    }
    static __device__ __forceinline__ void store(T *p, const float *o)
    {
        *reinterpret_cast<uint32_t *>(p) = EL::pack(o[0], o[1]);
    }
};
template <typename T, typename EL> struct VecIO16<T, 1, EL> {
    static __device__ __forceinline__ void load(const T *p, float *o) { o[0] = to_f32(*p); }
    static __device__ __forceinline__ void store(T *p, const float *o) { *p = from_f32<T>(o[0]); }
};
template <int N> struct VecIO<bf16_t, N> : VecIO16<bf16_t, N> {};
template <int N> struct VecIO<f16_t, N> : VecIO16<f16_t, N> {};

// Loads N consecutive elements with the widest aligned vector loads that fit
// (N is a power of two; the address is aligned to min(N, 16 / sizeof(T)) elements).
template <typename T, int N>
__device__ __forceinline__ void load_run(const T *p, float *o)
{
    constexpr int W0 = 16 / (int)sizeof(T);
    constexpr int W = N < W0 ? N : W0;
#pragma unroll
    for (int i = 0; i < N; i += W) VecIO<T, W>::load(p + i, o + i);
}

// Read-only int32 input that no kernel writes during a call (lengths, slot
// indices, accepted counts): read through the constant address space so a
// wave-uniform index becomes a scalar load, which does not queue behind the
// wave's outstanding vector loads and stores.
typedef const __attribute__((address_space(4))) int32_t *cint_ptr;
__device__ __forceinline__ int32_t ld_const(const int32_t *p, size_t i)
{
    return ((cint_ptr)p)[i];
}

// Cache policy of the decode kernels' state traffic: the state pool is read
// once and written once per call, in whole 128-byte lines, so both its loads
// and its stores are non-temporal (the nt bit, the aux argument of the buffer
// intrinsics) and stream past the caches. Measured on the decode step
// workload (per call): 30.6 us with neither, 28.8 us with nt loads only,
// 31.8 us with nt stores only, 26.2 us with both. Stores that cover only part
// of a line (the prefill's 8-byte output pieces) keep the default policy:
// non-temporal, they cost the chunked prefill 10 us.
constexpr int STREAM = 2;

// Wave-uniform value in a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace gdr
