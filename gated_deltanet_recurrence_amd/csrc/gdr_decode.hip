// Recurrent decode of the Gated Delta Rule on gfx950.
//
// Operation (lite_boost.ops.recurrent_gated_delta_rule, MindSpore Lite API
// page, algorithm and parameter sections): for each sequence b and value head
// h, starting from the pool slot selected through ssm_state_indices, apply
// the valid tokens in order — decay (exp(g), and exp(gk[i]) on row i), memory
// read kv = S^T k, delta write S += k (beta (v - kv))^T, output scale * S^T q —
// and store the state after each valid token into that token's slot.
//
// Design: the work is bound by streaming the state (Dk*Dv elements read and
// written once per call), so each wavefront owns one column tile of one
// (b, h) state and keeps it in registers, in float32, across all tokens of
// the call. The tile is TV columns wide: each lane holds VEC consecutive
// columns (one 16-byte load for bf16) of RPL consecutive rows. The lanes that
// share a column group sit next to each other (row group = low lane bits), so
// the two reductions over the key dimension (S^T k and S^T q) are a per-lane
// sum over its rows followed by an all-reduce inside a 16-lane DPP row
// (rotations by 8, 4, 2, 1), with no trip through the LDS crossbar. The
// columns of S evolve independently, so tiles need no exchange. Per call and
// head the state is read once and written once per distinct consecutive write
// slot; q/k/v/beta/g/gk/out are the only other traffic.
#include "gdr_common.h"

namespace gdr {

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over each aligned group of G consecutive lanes; every lane of the group
// receives the total. G <= 16 stays inside one DPP row.
template <int G>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (G >= 16) {
        x += dpp<0x128>(x);   // row_ror:8
        x += dpp<0x124>(x);   // row_ror:4
        x += dpp<0x122>(x);   // row_ror:2
        x += dpp<0x121>(x);   // row_ror:1
        if constexpr (G >= 32) x += __shfl_xor(x, 16);
        if constexpr (G >= 64) x += __shfl_xor(x, 32);
    } else if constexpr (G == 8) {
        x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
        x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
        x += dpp<0x141>(x);   // row_half_mirror
    } else if constexpr (G == 4) {
        x += dpp<0xB1>(x);
        x += dpp<0x4E>(x);
    } else if constexpr (G == 2) {
        x += dpp<0xB1>(x);
    }
    return x;
}

template <typename T, int DK, int DV, int TV, int VEC>
__global__ __launch_bounds__(128) void decode_kernel(DecodeParams p)
{
    static_assert(DV % TV == 0 && TV % VEC == 0, "tile shape");
    constexpr int CG = TV / VEC;   // lanes across the tile's columns
    static_assert(64 % CG == 0, "column groups must divide the wave");
    constexpr int RG = 64 / CG;    // lanes across the rows
    static_assert(DK % RG == 0, "rows must split evenly over lanes");
    constexpr int RPL = DK / RG;   // rows per lane
    constexpr int NT = DV / TV;    // column tiles per head

    const int lane = threadIdx.x & 63;
    const int wave = uniform(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const int Nv = p.Nv, S = p.S;
    if (wave >= p.B * Nv * NT) return;
    const int tile = wave % NT;
    const int h = (wave / NT) % Nv;
    const int b = wave / (NT * Nv);
    const int kh = h / (Nv / p.Nk);

    const int rg = lane % RG, cg = lane / RG;
    const int col = tile * TV + cg * VEC;
    const int row0 = rg * RPL;

    const T *q = static_cast<const T *>(p.q);
    const T *k = static_cast<const T *>(p.k);
    const T *v = static_cast<const T *>(p.v);
    const T *beta = static_cast<const T *>(p.beta);
    T *pool = static_cast<T *>(p.pool);
    T *out = static_cast<T *>(p.out);

    const size_t vh = (size_t)b * Nv + h;                  // (b, h) row of v / beta / g / out
    const size_t qkh = (size_t)b * p.Nk + kh;              // (b, kh) row of q / k

    // Integer resolution: lengths clamped, accepted count, read slot.
    int L = ld_const(p.lens, b);
    L = L < 0 ? 0 : (L > S ? S : L);
    const int n = p.nacc ? ld_const(p.nacc, b) : L;
    int r = -1;
    if (L > 0 && n >= 1 && n <= S) r = ld_const(p.idx, (size_t)b * S + n - 1);
    const bool active = r >= 0 && r < p.slots;

    float zero[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) zero[c] = 0.f;
    if (!active) {
        if (rg == 0)
            for (int t = 0; t < S; ++t) VecIO<T, VEC>::store(out + (vh * S + t) * DV + col, zero);
        return;
    }

    // The state tile, float32 in registers for the whole call.
    float st[RPL][VEC];
    {
        const T *sp = pool + ((size_t)r * Nv + h) * DK * DV + (size_t)row0 * DV + col;
#pragma unroll
        for (int i = 0; i < RPL; ++i) VecIO<T, VEC>::load(sp + (size_t)i * DV, st[i]);
    }

    for (int t = 0; t < L; ++t) {
        float kr[RPL], qr[RPL], vv[VEC];
        const size_t qkoff = (qkh * S + t) * DK + row0;
        load_run<T, RPL>(k + qkoff, kr);
        load_run<T, RPL>(q + qkoff, qr);
        VecIO<T, VEC>::load(v + (vh * S + t) * DV + col, vv);
        const float bt = to_f32(beta[vh * S + t]);

        // Decay: the whole state by exp(g), row i additionally by exp(gk[i]).
        const float a = p.g ? __expf(p.g[vh * S + t]) : 1.f;
        if (p.gk) {
            float gkr[RPL];
            load_run<float, RPL>(p.gk + (vh * S + t) * DK + row0, gkr);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float f = a * __expf(gkr[i]);
#pragma unroll
                for (int c = 0; c < VEC; ++c) st[i][c] *= f;
            }
        } else if (p.g) {
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int c = 0; c < VEC; ++c) st[i][c] *= a;
        }

        // Memory read kv = S^T k over the key dimension.
        float kv[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) s = fmaf(st[i][c], kr[i], s);
            kv[c] = s;
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) kv[c] = group_sum<RG>(kv[c]);

        // Delta write S += k (beta (v - kv))^T, and the output S^T q.
        float o[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const float d = bt * (vv[c] - kv[c]);
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                st[i][c] = fmaf(kr[i], d, st[i][c]);
                s = fmaf(st[i][c], qr[i], s);
            }
            o[c] = s;
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) o[c] = group_sum<RG>(o[c]);
        if (rg == 0) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) o[c] *= p.scale;
            VecIO<T, VEC>::store(out + (vh * S + t) * DV + col, o);
        }

        // Store the state into this token's slot unless the next token
        // overwrites the same slot.
        const int w = ld_const(p.idx, (size_t)b * S + t);
        const bool last = (t == L - 1) || (ld_const(p.idx, (size_t)b * S + t + 1) != w);
        if (last && w >= 0 && w < p.slots) {
            T *sp = pool + ((size_t)w * Nv + h) * DK * DV + (size_t)row0 * DV + col;
#pragma unroll
            for (int i = 0; i < RPL; ++i) VecIO<T, VEC>::store(sp + (size_t)i * DV, st[i]);
        }
    }
    if (rg == 0)
        for (int t = L; t < S; ++t) VecIO<T, VEC>::store(out + (vh * S + t) * DV + col, zero);
}

// Tile and vector width per (type, Dk, Dv): 16-byte row segments where the
// tile holds enough elements, a 32-column tile at most (measured fastest on
// MI355X among 16/32/64-column tiles and 1-8 waves per workgroup).
template <typename T, int DK, int DV>
static hipError_t launch_one(const DecodeParams &p, hipStream_t s)
{
    constexpr int TV_MAX = 32;
    constexpr int TV = DV > TV_MAX ? TV_MAX : DV;
    constexpr int VMAX = 16 / (int)sizeof(T);
    constexpr int PER_LANE = DK * TV / 64;
    constexpr int VEC0 = PER_LANE < VMAX ? PER_LANE : VMAX;
    constexpr int VEC = VEC0 > TV ? TV : VEC0;
    constexpr int NT = DV / TV;
    const long long waves = (long long)p.B * p.Nv * NT;
    const int wpb = 2;
    const dim3 grid((unsigned)((waves + wpb - 1) / wpb)), block(64 * wpb);
    DecodeParams pc = p;
    void *args[] = {&pc};
    return hipLaunchKernel((const void *)decode_kernel<T, DK, DV, TV, VEC>, grid, block, args, 0, s);
}

template <typename T>
static hipError_t launch_typed(int Dk, int Dv, const DecodeParams &p, hipStream_t s, bool *ok)
{
    *ok = true;
#define GDR_DEC_CASE(DK_, DV_) \
    if (Dk == DK_ && Dv == DV_) return launch_one<T, DK_, DV_>(p, s);
#define GDR_DEC_ROW(DK_) GDR_DEC_CASE(DK_, 16) GDR_DEC_CASE(DK_, 32) GDR_DEC_CASE(DK_, 64) GDR_DEC_CASE(DK_, 128)
    GDR_DEC_ROW(16)
    GDR_DEC_ROW(32)
    GDR_DEC_ROW(64)
    GDR_DEC_ROW(128)
#undef GDR_DEC_ROW
#undef GDR_DEC_CASE
    *ok = false;
    return hipSuccess;
}

hipError_t launch_decode(int dtype, int Dk, int Dv, const DecodeParams &p, hipStream_t s, bool *supported)
{
    if (dtype == 1) return launch_typed<bf16_t>(Dk, Dv, p, s, supported);
    return launch_typed<float>(Dk, Dv, p, s, supported);
}

}  // namespace gdr
