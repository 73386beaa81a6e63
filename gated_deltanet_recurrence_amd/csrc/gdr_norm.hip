// Gated RMSNorm output epilogue as a pass of its own, for the paths that do
// not apply it inside their kernels (the prefill kernels, whose rows of Dv
// columns are split between workgroups, and the general decode kernel).
//
// Operation (inferencelayer deltanet.rs: module header, and the per-head gated
// RMSNorm of its step and chunk code and of DN_STEP / DN_CHUNK), per output row
// o of Dv columns:  o_j w_j silu(z_j) / sqrt(mean(o^2) + eps).
#include "gdr_common.h"

namespace gdr {

namespace {

constexpr int NORM_WAVES = 4;   // waves per workgroup
constexpr int NORM_NB = 4;      // batches of rows per wave, loaded together

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Sum over aligned groups of LPR lanes (2, 4, 8 or 16) inside a 16-lane row,
// in every lane of the group: pair swap, quad swap, mirrored half, mirrored row.
template <int LPR>
__device__ __forceinline__ float group_sum(float x)
{
    x = dpp_add<0xB1>(x);                          // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) x = dpp_add<0x4E>(x);  // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) x = dpp_add<0x141>(x); // row_half_mirror
    if constexpr (LPR >= 16) x = dpp_add<0x140>(x); // row_mirror
    return x;
}

// Eight adjacent elements of a row (16 bytes in bf16, 32 in float).
template <typename T> struct Oct;
template <typename T> struct Oct16 {
    typedef typename Elem<T>::type EL;
    static __device__ __forceinline__ void load(const T *p, float *x)
    {
        const u32x4_t u = *reinterpret_cast<const u32x4_t *>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[2 * i] = EL::lo(w[i]); x[2 * i + 1] = EL::hi(w[i]); }
    }
    static __device__ __forceinline__ void store(T *p, const float *x)
    {
        *reinterpret_cast<u32x4_t *>(p) = u32x4_t{EL::pack(x[0], x[1]), EL::pack(x[2], x[3]),
                                                  EL::pack(x[4], x[5]), EL::pack(x[6], x[7])};
    }
};
template <> struct Oct<bf16_t> : Oct16<bf16_t> {};
template <> struct Oct<f16_t> : Oct16<f16_t> {};
template <> struct Oct<float> {
    static __device__ __forceinline__ void load(const float *p, float *x)
    {
        const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *x)
    {
        reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
};

// Workgroup = (value head (b, h), block of rows), nblk blocks per head. A row
// of DV columns is held by LPR = DV / 8 consecutive lanes, 8 columns each, so
// a wave covers 64 / LPR rows per batch and NORM_NB batches.
template <typename T, int DV>
__global__ __launch_bounds__(64 * NORM_WAVES) void norm_kernel(NormParams p, int nblk)
{
    constexpr int LPR = DV / 8, RPB = 64 / LPR, RPW = RPB * NORM_NB;
    const int lane = threadIdx.x & 63;
    const int wv = uniform(threadIdx.x >> 6);
    const int vh = (int)(blockIdx.x / (unsigned)nblk), tb = (int)(blockIdx.x % (unsigned)nblk);
    const int b = vh / p.Nv;
    int L = p.lens ? ld_const(p.lens, b) : p.S;
    L = L < 0 ? 0 : (L > p.S ? p.S : L);
    const int t0 = (tb * NORM_WAVES + wv) * RPW;
    if (t0 >= L) return;   // rows past the length stay as written (zeros)
    const int rb = lane / LPR, c = 8 * (lane % LPR);
    T *o = static_cast<T *>(p.out) + ((size_t)vh * p.S + t0 + rb) * DV + c;
    const T *z = static_cast<const T *>(p.z) + ((size_t)vh * p.S + t0 + rb) * DV + c;
    float w[8];
    Oct<float>::load(p.w + c, w);
    float ov[NORM_NB][8], zv[NORM_NB][8];
#pragma unroll
    for (int n = 0; n < NORM_NB; ++n) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[n][i] = zv[n][i] = 0.f;
        if (t0 + n * RPB + rb < L) {
            Oct<T>::load(o + n * RPB * DV, ov[n]);
            Oct<T>::load(z + n * RPB * DV, zv[n]);
        }
    }
#pragma unroll
    for (int n = 0; n < NORM_NB; ++n) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(ov[n][i], ov[n][i], ss);
        const float r = norm_rinv(group_sum<LPR>(ss), DV, p.eps);
        if (t0 + n * RPB + rb < L) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = ov[n][i] * r * w[i] * norm_silu(zv[n][i]);
            Oct<T>::store(o + n * RPB * DV, y);
        }
    }
}

// Rows covered by one workgroup.
int norm_rows_per_block(int Dv) { return NORM_WAVES * NORM_NB * (64 / (Dv / 8)); }

}  // namespace

bool norm_supported(int Dv, int B, int Nv, int S)
{
    if (Dv != 16 && Dv != 32 && Dv != 64 && Dv != 128) return false;
    const int rpb = norm_rows_per_block(Dv);
    return (int64_t)B * Nv * ((S + rpb - 1) / rpb) < 0x7fffffffLL;
}

hipError_t launch_norm(int dtype, const NormParams &p, hipStream_t s, bool *supported)
{
    *supported = norm_supported(p.Dv, p.B, p.Nv, p.S);
    if (!*supported) return hipSuccess;
    const int rpb = norm_rows_per_block(p.Dv);
    int nblk = (p.S + rpb - 1) / rpb;
    const int64_t nwg = (int64_t)p.B * p.Nv * nblk;
    if (nwg == 0) return hipSuccess;
    NormParams pc = p;
    void *args[] = {&pc, &nblk};
    const dim3 grid((unsigned)nwg), block(64 * NORM_WAVES);
    const void *fn = nullptr;
#define GDR_NORM_CASE(D_)                                                                          \
    if (p.Dv == D_)                                                                                \
        fn = dtype == 1 ? (const void *)norm_kernel<bf16_t, D_>                                    \
                        : (dtype == 2 ? (const void *)norm_kernel<f16_t, D_> : (const void *)norm_kernel<float, D_>);
    GDR_NORM_CASE(16) GDR_NORM_CASE(32) GDR_NORM_CASE(64) GDR_NORM_CASE(128)
#undef GDR_NORM_CASE
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace gdr
