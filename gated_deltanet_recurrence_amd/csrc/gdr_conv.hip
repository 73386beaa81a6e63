// Depthwise causal conv1d + SiLU ahead of the recurrence, with the split of
// its channels into q, k and v.
//
// Operation (the Gated DeltaNet blog post's layer code: causal_conv1d_fn and
// causal_conv1d_update with the SiLU activation, then the split of the fused
// projection; inferencelayer deltanet.rs: the conv ring of its step and chunk
// code and DN_CONV), per channel c of the C = 2 Nk Dk + Nv Dv channels:
//   y_t[c] = silu(bias[c] + sum_j w[c, j] x_{t-K+1+j}[c]),  taps oldest first,
// with the inputs before the first token taken from the carried state (the
// last K - 1 inputs, oldest first). y goes straight into the BNSD q, k, v the
// recurrence kernels read, so the conv, the activation, the split and the
// transpose are one pass over HBM.
//
// One thread per pair of adjacent channels (Dk and Dv are even, so a pair
// never straddles a head): 4-byte (bf16) or 8-byte (float) accesses, adjacent
// threads on adjacent pairs. Sums in float32.
#include "gdr_common.h"

namespace gdr {

namespace {

constexpr int CONV_THREADS = 256;
constexpr int CONV_TB = 32;    // tokens per prefill workgroup
constexpr int CONV_AHEAD = 16; // input loads issued ahead of their use

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_rsrc(const void *p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// Two adjacent channels: loads through a bounded buffer resource (byte offset
// off; reads past the bound return zeros, so they need no branch), stores
// through a plain pointer, since the destination plane differs between lanes
// on either side of a head boundary and a buffer resource must be uniform over
// the wave. store_nt carries the non-temporal hint, for the prefill's
// outputs: each is written once and read by a later kernel, and together
// they outgrow the L2.
template <typename T> struct Pair2;
template <typename T> struct Pair16 {
    typedef typename Elem<T>::type EL;
    static __device__ __forceinline__ float2 load(__amdgpu_buffer_rsrc_t r, int off)
    {
        const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        return make_float2(EL::lo(u), EL::hi(u));
    }
    static __device__ __forceinline__ void store(T *p, float2 v) { *reinterpret_cast<uint32_t *>(p) = EL::pack(v.x, v.y); }
    static __device__ __forceinline__ void store_nt(T *p, float2 v)
    {
        __builtin_nontemporal_store(EL::pack(v.x, v.y), reinterpret_cast<uint32_t *>(p));
    }
    static __device__ __forceinline__ float one(const T *p) { return to_f32(*p); }
    static __device__ __forceinline__ void put(T *p, float v) { *p = from_f32<T>(v); }
};
template <> struct Pair2<bf16_t> : Pair16<bf16_t> {};
template <> struct Pair2<f16_t> : Pair16<f16_t> {};
template <> struct Pair2<float> {
    static __device__ __forceinline__ float2 load(__amdgpu_buffer_rsrc_t r, int off)
    {
        const u32x2_t u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_float2(__uint_as_float(u.x), __uint_as_float(u.y));
    }
    static __device__ __forceinline__ void store(float *p, float2 v) { *reinterpret_cast<float2 *>(p) = v; }
    static __device__ __forceinline__ void store_nt(float *p, float2 v)
    {
        __builtin_nontemporal_store(u32x2_t{__float_as_uint(v.x), __float_as_uint(v.y)}, reinterpret_cast<u32x2_t *>(p));
    }
    static __device__ __forceinline__ float one(const float *p) { return *p; }
    static __device__ __forceinline__ void put(float *p, float v) { *p = v; }
};

// Where channel pair (c, c + 1) of sequence b goes in q, k or v: the head's
// plane of S rows of D elements, and the column d within a row.
template <typename T>
__device__ __forceinline__ T *split_dst(const ConvParams &p, int b, int c, int &D, int &d)
{
    const int nq = p.Nk * p.Dk;
    if (c < nq) {
        D = p.Dk;
        d = c % p.Dk;
        return static_cast<T *>(p.q) + ((size_t)b * p.Nk + c / p.Dk) * p.S * p.Dk;
    }
    if (c < 2 * nq) {
        c -= nq;
        D = p.Dk;
        d = c % p.Dk;
        return static_cast<T *>(p.k) + ((size_t)b * p.Nk + c / p.Dk) * p.S * p.Dk;
    }
    c -= 2 * nq;
    D = p.Dv;
    d = c % p.Dv;
    return static_cast<T *>(p.v) + ((size_t)b * p.Nv + c / p.Dv) * p.S * p.Dv;
}

// u sigmoid(u) with the hardware reciprocal (within 1 ulp) in place of a
// division: 1 + e^-u is at least 1, and an infinite one gives u * 0.
__device__ __forceinline__ float conv_silu(float u) { return u * __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

// One token: window win[0..K-2] (oldest first) and input xin; returns y and
// shifts xin into the window.
template <int K>
__device__ __forceinline__ float2 conv_step(float2 (&win)[K > 1 ? K - 1 : 1], float2 xin, const float (&w0)[K],
                                            const float (&w1)[K], float2 bv)
{
    float2 acc = make_float2(fmaf(w0[K - 1], xin.x, bv.x), fmaf(w1[K - 1], xin.y, bv.y));
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
        acc.x = fmaf(w0[j], win[j].x, acc.x);
        acc.y = fmaf(w1[j], win[j].y, acc.y);
    }
#pragma unroll
    for (int j = 0; j + 2 < K; ++j) win[j] = win[j + 1];
    if constexpr (K > 1) win[K - 2] = xin;
    return make_float2(conv_silu(acc.x), conv_silu(acc.y));
}

template <int K>
__device__ __forceinline__ void conv_weights(const ConvParams &p, int c, float (&w0)[K], float (&w1)[K], float2 &bv)
{
#pragma unroll
    for (int j = 0; j < K; ++j) {
        w0[j] = p.w[(size_t)c * K + j];
        w1[j] = p.w[(size_t)(c + 1) * K + j];
    }
    bv = p.bias ? make_float2(p.bias[c], p.bias[c + 1]) : make_float2(0.f, 0.f);
}

// Workgroup (channel pairs x, token block y, sequence z). Inputs are read
// through a resource bounded by the sequence's valid tokens: every token of
// the block is loaded ahead with no branch, and stored (zeros at t >= L) when
// it lies in the plane's S rows.
template <typename T, int K>
__global__ __launch_bounds__(CONV_THREADS) void conv_prefill_kernel(ConvParams p)
{
    constexpr int KW = K > 1 ? K - 1 : 1;
    constexpr int E = sizeof(T);
    const int C = 2 * p.Nk * p.Dk + p.Nv * p.Dv;
    const int c = 2 * (blockIdx.x * CONV_THREADS + threadIdx.x);
    if (c >= C) return;
    const int b = blockIdx.z, t0 = blockIdx.y * CONV_TB;
    int L = p.lens ? ld_const(p.lens, b) : p.S;
    L = L < 0 ? 0 : (L > p.S ? p.S : L);
    const T *xb = static_cast<const T *>(p.x) + (size_t)b * p.S * C;
    const auto xrs = conv_rsrc(xb, (int64_t)L * C * E);
    const T *init = p.init ? static_cast<const T *>(p.init) + ((size_t)b * C + c) * (K - 1) : nullptr;
    // input of token tau (tau < 0: the carried state; zeros without one)
    auto input = [&](int tau) __attribute__((always_inline)) {
        if (tau >= 0) return Pair2<T>::load(xrs, (tau * C + c) * E);
        if (!init) return make_float2(0.f, 0.f);
        return make_float2(Pair2<T>::one(init + tau + K - 1), Pair2<T>::one(init + (K - 1) + tau + K - 1));
    };
    float w0[K], w1[K];
    float2 bv;
    conv_weights<K>(p, c, w0, w1, bv);
    int D, d;
    T *const out = split_dst<T>(p, b, c, D, d) + d;
    float2 win[KW];
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) win[j] = input(t0 - (K - 1) + j);
    // Two batches of CONV_AHEAD tokens in flight: the next one's loads are
    // issued before the current one is computed.
    float2 xs[2][CONV_AHEAD];
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i) xs[0][i] = Pair2<T>::load(xrs, ((t0 + i) * C + c) * E);
#pragma unroll
    for (int nb = 0; nb < CONV_TB / CONV_AHEAD; ++nb) {
        const int ta = t0 + nb * CONV_AHEAD;
        if (nb + 1 < CONV_TB / CONV_AHEAD) {
#pragma unroll
            for (int i = 0; i < CONV_AHEAD; ++i) xs[(nb + 1) & 1][i] = Pair2<T>::load(xrs, ((ta + CONV_AHEAD + i) * C + c) * E);
        }
#pragma unroll
        for (int i = 0; i < CONV_AHEAD; ++i) {
            float2 y = conv_step<K>(win, xs[nb & 1][i], w0, w1, bv);
            if (ta + i >= L) y = make_float2(0.f, 0.f);   // rows past the length: exact zeros
            if (ta + i < p.S) Pair2<T>::store_nt(out + (size_t)(ta + i) * D, y);
        }
    }
    // The final state (the last K - 1 inputs) is written by the first token
    // block, after its reads of the initial state, so it may alias it.
    if (p.fin && blockIdx.y == 0 && K > 1) {
        float2 f[KW];
#pragma unroll
        for (int j = 0; j + 1 < K; ++j) f[j] = input(L - (K - 1) + j);
        T *fin = static_cast<T *>(p.fin) + ((size_t)b * C + c) * (K - 1);
#pragma unroll
        for (int j = 0; j + 1 < K; ++j) {
            Pair2<T>::put(fin + j, f[j].x);
            Pair2<T>::put(fin + (K - 1) + j, f[j].y);
        }
    }
}

// Workgroup (channel pairs x, sequence y); the S <= 8 inputs are loaded first
// (zeros past the valid tokens), then the tokens are applied in order, the
// state carried in registers and stored after every valid token whose slot
// the next token does not overwrite.
template <typename T, int K>
__global__ __launch_bounds__(CONV_THREADS) void conv_decode_kernel(ConvParams p)
{
    constexpr int KW = K > 1 ? K - 1 : 1;
    constexpr int E = sizeof(T);
    const int C = 2 * p.Nk * p.Dk + p.Nv * p.Dv;
    const int c = 2 * (blockIdx.x * CONV_THREADS + threadIdx.x);
    if (c >= C) return;
    const int b = blockIdx.y, S = p.S;
    int L = ld_const(p.lens, b);
    L = L < 0 ? 0 : (L > S ? S : L);
    const int n = p.nacc ? ld_const(p.nacc, b) : L;
    int r = -1;
    if (L > 0 && n >= 1 && n <= S) r = ld_const(p.idx, (size_t)b * S + n - 1);
    if (r < 0 || r >= p.slots) L = 0;   // skipped: zeros, no slot touched
    const auto xrs = conv_rsrc(static_cast<const T *>(p.x) + (size_t)b * S * C, (int64_t)L * C * E);
    float2 xs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xs[t] = Pair2<T>::load(xrs, (t * C + c) * E);
    T *pool = static_cast<T *>(p.pool);
    float w0[K], w1[K];
    float2 bv;
    conv_weights<K>(p, c, w0, w1, bv);
    int D, d;
    T *const out = split_dst<T>(p, b, c, D, d) + d;
    float2 win[KW];
    if (L > 0) {
        const T *src = pool + ((size_t)r * C + c) * (K - 1);
#pragma unroll
        for (int j = 0; j + 1 < K; ++j) win[j] = make_float2(Pair2<T>::one(src + j), Pair2<T>::one(src + (K - 1) + j));
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t >= S) break;
        if (t >= L) {
            Pair2<T>::store(out + (size_t)t * D, make_float2(0.f, 0.f));
            continue;
        }
        Pair2<T>::store(out + (size_t)t * D, conv_step<K>(win, xs[t], w0, w1, bv));
        const int s = ld_const(p.idx, (size_t)b * S + t);
        const bool again = t + 1 < L && ld_const(p.idx, (size_t)b * S + t + 1) == s;
        if (K > 1 && s >= 0 && s < p.slots && !again) {
            T *dst = pool + ((size_t)s * C + c) * (K - 1);
#pragma unroll
            for (int j = 0; j + 1 < K; ++j) {
                Pair2<T>::put(dst + j, win[j].x);
                Pair2<T>::put(dst + (K - 1) + j, win[j].y);
            }
        }
    }
}

template <template <typename, int> class Kern, typename T>
const void *conv_fn(int K)
{
    switch (K) {
    case 1: return (const void *)Kern<T, 1>::fn;
    case 2: return (const void *)Kern<T, 2>::fn;
    case 3: return (const void *)Kern<T, 3>::fn;
    case 4: return (const void *)Kern<T, 4>::fn;
    case 5: return (const void *)Kern<T, 5>::fn;
    case 6: return (const void *)Kern<T, 6>::fn;
    case 7: return (const void *)Kern<T, 7>::fn;
    case 8: return (const void *)Kern<T, 8>::fn;
    }
    return nullptr;
}
template <typename T, int K> struct PrefillK { static constexpr auto fn = conv_prefill_kernel<T, K>; };
template <typename T, int K> struct DecodeK { static constexpr auto fn = conv_decode_kernel<T, K>; };

}  // namespace

hipError_t launch_conv_prefill(int dtype, const ConvParams &p, hipStream_t s, bool *supported)
{
    const int C = 2 * p.Nk * p.Dk + p.Nv * p.Dv;
    const void *fn = dtype == 1 ? conv_fn<PrefillK, bf16_t>(p.K)
                                : (dtype == 2 ? conv_fn<PrefillK, f16_t>(p.K) : conv_fn<PrefillK, float>(p.K));
    *supported = fn != nullptr;
    if (!fn) return hipSuccess;
    ConvParams pc = p;
    void *args[] = {&pc};
    const dim3 grid((unsigned)((C / 2 + CONV_THREADS - 1) / CONV_THREADS), (unsigned)((p.S + CONV_TB - 1) / CONV_TB),
                    (unsigned)p.B);
    return hipLaunchKernel(fn, grid, dim3(CONV_THREADS), args, 0, s);
}

hipError_t launch_conv_decode(int dtype, const ConvParams &p, hipStream_t s, bool *supported)
{
    const int C = 2 * p.Nk * p.Dk + p.Nv * p.Dv;
    const void *fn = dtype == 1 ? conv_fn<DecodeK, bf16_t>(p.K)
                                : (dtype == 2 ? conv_fn<DecodeK, f16_t>(p.K) : conv_fn<DecodeK, float>(p.K));
    *supported = fn != nullptr;
    if (!fn) return hipSuccess;
    ConvParams pc = p;
    void *args[] = {&pc};
    const dim3 grid((unsigned)((C / 2 + CONV_THREADS - 1) / CONV_THREADS), (unsigned)p.B);
    return hipLaunchKernel(fn, grid, dim3(CONV_THREADS), args, 0, s);
}

}  // namespace gdr
