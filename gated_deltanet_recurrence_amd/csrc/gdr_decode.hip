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
// columns (one 16-byte load for 16-bit types) of RPL consecutive rows. The lanes that
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
        if (p.qk_norm) {
            // q and k to x / sqrt(|x|^2 + eps): the rows of a column group sit
            // in RG consecutive lanes.
            float kk = 0.f, qq = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                kk = fmaf(kr[i], kr[i], kk);
                qq = fmaf(qr[i], qr[i], qq);
            }
            const float rk = qk_rnorm(group_sum<RG>(kk)), rq = qk_rnorm(group_sum<RG>(qq));
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                kr[i] *= rk;
                qr[i] *= rq;
            }
        }
        const float braw = to_f32(beta[vh * S + t]);
        const float bt = p.beta_logit ? gate_sigmoid(braw) : braw;

        // Decay: the whole state by exp(g), row i additionally by exp(gk[i]).
        const float a = p.g ? __expf(p.g[vh * S + t])
                            : (p.gate_a ? __expf(gate_g(to_f32(static_cast<const T *>(p.gate_a)[vh * S + t]), p.A_log[h],
                                                        p.dt_bias[h]))
                                        : 1.f);
        if (p.gk) {
            float gkr[RPL];
            load_run<float, RPL>(p.gk + (vh * S + t) * DK + row0, gkr);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float f = a * __expf(gkr[i]);
#pragma unroll
                for (int c = 0; c < VEC; ++c) st[i][c] *= f;
            }
        } else if (p.g || p.gate_a) {
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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Decode step with one token per sequence (S = 1), 16-bit I/O (bf16 or fp16),
// Dk = Dv = 128.
//
// A workgroup of four wavefronts updates one head at a time and walks the
// heads g, g + G, g + 2G, ... (G workgroups, persistent: three per CU). Wave j
// owns the 32 rows [32j, 32j + 32) of the head's 128 x 128 state; lane l of it
// holds columns 8 (l % 16) .. + 7 of the eight consecutive rows
// 32j + 8 (l / 16) + i, so each load or store instruction of the wave moves
// four whole 256-byte rows. The column sums S^T (D k) and S^T (D q) are
// reduced over the wave's four lane rows with the cross-row lane swaps
// (v_permlane32_swap / v_permlane16_swap), then over the four waves through
// LDS with one barrier per head. All loads of the next head (state, k, q, v,
// gk) are in flight while the current head is updated and stored; its scalars
// are read one head earlier still. Every load goes through a buffer resource
// whose size is zero when there is nothing to read, so no load sits under a
// branch.
//
// Layout, measured on the decode step workload (2048 heads): eight waves per
// head (four rows per lane), one workgroup per CU and the loads of two heads
// ahead in flight took 25.7 us; four waves per head, three workgroups per CU
// and one head ahead 24.5-24.7 us (two or four workgroups per CU: 25.8 and
// 25.2 us; workgroup counts that leave CUs unevenly loaded: 26.7-28.0 us).
//
// With one token the output needs no pass over the updated state:
//   S' = D S + k delta^T,  D = diag(exp(g) exp(gk_i)),  delta = beta (v - S^T D k)
//   o  = scale S'^T q = scale (S^T (D q) + delta (k . q))
namespace s1 {
constexpr int DK = 128, DV = 128;
#ifndef GDR_S1_NW
#define GDR_S1_NW 4
#endif
constexpr int NW = GDR_S1_NW;         // waves per head (workgroup size 64 NW)
constexpr int RW = DK / NW;           // rows per wave
constexpr int NI = RW / 4;            // rows per lane, one per instruction
static_assert(NI == 4 || NI == 8, "4 or 8 rows per lane");
constexpr int PER_CU = 3;             // persistent workgroups per CU
#ifndef GDR_S1_NB
#define GDR_S1_NB 2
#endif
constexpr int NB = GDR_S1_NB;         // heads whose loads are in flight
}  // namespace s1

// Scalars of a head, read through the scalar cache ahead of use: beta (or its
// logit) and, with fused gates, a as 16-bit pairs; A_log and dt_bias of the head.
struct S1Scal { int32_t len, nacc, idx, beta2, g, alog = 0, dtb = 0; };
// One head's loads and resolution (r < 0: nothing to do).
struct S1Head {
    int b, h, r;
    float beta, g;
    u32x4_t st[s1::NI];   // 8 16-bit columns of each of the lane's rows
    u32x2_t k, q;         // the lane's first 4 rows of k and q (16-bit)
    u32x2_t k2, q2;       // rows 4-7 with 8 rows per lane
    u32x4_t v;            // the lane's 8 columns of v (16-bit)
    u32x4_t gk[s1::NI / 4];   // the lane's rows of gk (f32)
    uint32_t z;           // the epilogue's z at the lane's two output columns (16-bit)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
// Gated RMSNorm epilogue on the output row held by one wave, two columns per
// lane (o0, o1 at the columns of z's two halves, weights w0, w1): the sum of
// squares over the 16 lanes of a row (quad swaps, then the mirrored half and
// row), then over the four rows.
template <typename EL>
__device__ __forceinline__ uint32_t norm_pair(float o0, float o1, uint32_t z, float w0, float w1, float eps);

// Sum over the four 16-lane rows of a wave, in every lane.
__device__ __forceinline__ float rows_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename EL>
__device__ __forceinline__ uint32_t norm_pair(float o0, float o1, uint32_t z, float w0, float w1, float eps)
{
    float x = o0 * o0 + o1 * o1;
    x = dpp_add<0xB1, 0xf>(x);    // quad_perm [1,0,3,2]
    x = dpp_add<0x4E, 0xf>(x);    // quad_perm [2,3,0,1]
    x = dpp_add<0x141, 0xf>(x);   // row_half_mirror
    x = dpp_add<0x140, 0xf>(x);   // row_mirror
    const float r = norm_rinv(rows_sum(x), 128, eps);
    return EL::pack(o0 * r * w0 * norm_silu(EL::lo(z)), o1 * r * w1 * norm_silu(EL::hi(z)));
}

// Transposing reduction over the four 16-lane rows: given per-lane partials
// x0..x3, returns in lane row r the total over the rows of x_r.
__device__ __forceinline__ float rows_reduce4(float x0, float x1, float x2, float x3)
{
    // rows (0, 1, 2, 3) of a: x0 over rows {0,2}, {1,3}; x2 likewise
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x2), false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x1), __float_as_uint(x3), false, false);
    const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float C = __uint_as_float(c[0]) + __uint_as_float(c[1]);
    const auto d = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(C), false, false);
    return __uint_as_float(d[0]) + __uint_as_float(d[1]);
}

// Broadcast of each 16-lane row's value: y[r] holds row r's x in every row.
__device__ __forceinline__ void rows_gather(float x, float y[4])
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const auto e = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    const auto o = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
    y[0] = __uint_as_float(e[0]);
    y[2] = __uint_as_float(e[1]);
    y[1] = __uint_as_float(o[0]);
    y[3] = __uint_as_float(o[1]);
}

__device__ __forceinline__ void s1_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// GK: per-key decay gk given. FG: fused gates, beta and g formed in the
// kernel from the logits and the raw gate input a. QN: q and k normalised in
// the kernel. NRM: gated RMSNorm epilogue on the outputs (norm_pair).
template <typename EL, bool GK, bool FG, bool QN, bool NRM>
__global__ __launch_bounds__(64 * s1::NW) __attribute__((amdgpu_waves_per_eu(s1::PER_CU * s1::NW / 4)))
void decode_s1_kernel(DecodeParams p, int nheads)
{
    using namespace s1;
    __shared__ float4 red[2][NW][64];
    __shared__ float4 redkq[2][NW];   // k . q, |k|^2, |q|^2 of each wave's rows

    const int lane = threadIdx.x & 63;
    const int j = uniform(threadIdx.x >> 6);
    const int G = gridDim.x;
    const int Nv = p.Nv, rep = p.Nv / p.Nk;
    const int lr = lane >> 4, cg = lane & 15;
    const int row0 = j * RW + lr * NI;   // the lane's first row

    const uint16_t *q = static_cast<const uint16_t *>(p.q);
    const uint16_t *k = static_cast<const uint16_t *>(p.k);
    const uint16_t *v = static_cast<const uint16_t *>(p.v);
    uint16_t *pool = static_cast<uint16_t *>(p.pool);
    uint16_t *out = static_cast<uint16_t *>(p.out);
    // Gated RMSNorm epilogue (NRM): z of each head's row, w of the lane's columns.
    const uint16_t *zsrc = static_cast<const uint16_t *>(p.norm_z);
    float nw0 = 0.f, nw1 = 0.f;
    if constexpr (NRM) {
        const u32x2_t nwv = __builtin_amdgcn_raw_buffer_load_b64(brsrc(p.norm_w, DV * 4), (cg * 8 + lr * 2) * 4, 0, 0);
        nw0 = __uint_as_float(nwv.x);
        nw1 = __uint_as_float(nwv.y);
    }
    // Optional inputs are read from a valid stand-in address and discarded,
    // so no load sits under a branch.
    const int32_t *nacc_src = p.nacc ? p.nacc : p.lens;
    const int32_t *g_src = FG ? static_cast<const int32_t *>(p.gate_a) : (p.g ? reinterpret_cast<const int32_t *>(p.g) : p.lens);
    const int32_t *beta_src = static_cast<const int32_t *>(p.beta);

    auto scal = [&](int hd) __attribute__((always_inline)) {
        const int hc = hd < nheads ? hd : nheads - 1;
        const int b = hc / Nv, h = hc % Nv;
        const int vh = b * Nv + h;
        S1Scal c;
        c.len = ld_const(p.lens, b);
        c.nacc = ld_const(nacc_src, b);
        c.idx = ld_const(p.idx, b);
        c.beta2 = ld_const(beta_src, vh >> 1);
        c.g = ld_const(g_src, FG ? vh >> 1 : (p.g ? vh : 0));
        if constexpr (FG) {
            c.alog = ld_const(reinterpret_cast<const int32_t *>(p.A_log), h);
            c.dtb = ld_const(reinterpret_cast<const int32_t *>(p.dt_bias), h);
        }
        return c;
    };
    // Resolves a head from its scalars and issues all of its loads.
    auto load = [&](S1Head &H, const S1Scal &c, int hd) __attribute__((always_inline)) {
        const int hc = hd < nheads ? hd : nheads - 1;
        H.b = hc / Nv;
        H.h = hc % Nv;
        const int vh = H.b * Nv + H.h;
        const int L = c.len < 0 ? 0 : (c.len > 1 ? 1 : c.len);
        const int n = p.nacc ? c.nacc : L;
        const int r = (hd < nheads && L == 1 && n == 1) ? c.idx : -1;
        H.r = (r >= 0 && r < p.slots) ? r : -1;
        const float braw = EL::to((uint32_t)c.beta2 >> (16 * (vh & 1)));
        H.beta = FG ? gate_sigmoid(braw) : braw;
        if constexpr (FG)
            H.g = gate_g(EL::to((uint32_t)c.g >> (16 * (vh & 1))), __int_as_float(c.alog), __int_as_float(c.dtb));
        else
            H.g = p.g ? __int_as_float(c.g) : 0.f;
        const bool on = H.r >= 0;
        const auto srs = brsrc(pool + ((size_t)(on ? H.r : 0) * Nv + H.h) * DK * DV, on ? DK * DV * 2 : 0);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            H.st[i] = __builtin_amdgcn_raw_buffer_load_b128(srs, ((row0 + i) * DV + cg * 8) * 2, 0, STREAM);
        const size_t qk = (size_t)H.b * p.Nk + H.h / rep;
        const int tb = on ? DK * 2 : 0;
        if constexpr (NI == 4) {
            H.k = __builtin_amdgcn_raw_buffer_load_b64(brsrc(k + qk * DK, tb), row0 * 2, 0, 0);
            H.q = __builtin_amdgcn_raw_buffer_load_b64(brsrc(q + qk * DK, tb), row0 * 2, 0, 0);
        } else {
            const u32x4_t k4 = __builtin_amdgcn_raw_buffer_load_b128(brsrc(k + qk * DK, tb), row0 * 2, 0, 0);
            const u32x4_t q4 = __builtin_amdgcn_raw_buffer_load_b128(brsrc(q + qk * DK, tb), row0 * 2, 0, 0);
            H.k = u32x2_t{k4.x, k4.y};
            H.k2 = u32x2_t{k4.z, k4.w};
            H.q = u32x2_t{q4.x, q4.y};
            H.q2 = u32x2_t{q4.z, q4.w};
        }
        H.v = __builtin_amdgcn_raw_buffer_load_b128(brsrc(v + (size_t)vh * DV, on ? DV * 2 : 0), cg * 16, 0, 0);
        if constexpr (GK)
#pragma unroll
            for (int n = 0; n < NI / 4; ++n)
                H.gk[n] = __builtin_amdgcn_raw_buffer_load_b128(brsrc(p.gk + (size_t)vh * DK, on ? DK * 4 : 0), (row0 + 4 * n) * 4, 0, 0);
        if constexpr (NRM)
            H.z = __builtin_amdgcn_raw_buffer_load_b32(brsrc(zsrc + (size_t)vh * DV, on ? DV * 2 : 0), (cg * 8 + lr * 2) * 2, 0, 0);
    };
    // A skipped head still waits for its (empty) loads, so that every path
    // leaves the register sets settled: otherwise the compiler has to wait
    // for them where the paths meet, before the next prefetch is issued.
    auto settle = [&](const S1Head &H) __attribute__((always_inline)) {
        uint32_t x = H.k.x ^ H.q.x ^ H.v.x;
        if constexpr (NRM) x ^= H.z;
#pragma unroll
        for (int i = 0; i < NI; ++i) x ^= H.st[i].x ^ H.st[i].w;
        if constexpr (GK) x ^= H.gk[0].x;
        asm volatile("" ::"v"(x));
    };
    // Output columns of this lane in the writing wave: 8 cg + 2 lr, + 1.
    auto out_ptr = [&](const S1Head &H) __attribute__((always_inline)) {
        return reinterpret_cast<uint32_t *>(out + ((size_t)H.b * Nv + H.h) * DV + cg * 8 + lr * 2);
    };
    int par = 0;
    auto compute = [&](const S1Head &H) __attribute__((always_inline)) {
        if (H.r < 0) {
            settle(H);
            if (j == 0) *out_ptr(H) = 0u;
            return;
        }
        const float a = __expf(H.g);
        float dd[NI];
        if constexpr (GK) {
#pragma unroll
            for (int n = 0; n < NI / 4; ++n) {
                dd[4 * n] = a * __expf(__uint_as_float(H.gk[n].x));
                dd[4 * n + 1] = a * __expf(__uint_as_float(H.gk[n].y));
                dd[4 * n + 2] = a * __expf(__uint_as_float(H.gk[n].z));
                dd[4 * n + 3] = a * __expf(__uint_as_float(H.gk[n].w));
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) dd[i] = a;
        }
        // k and q of the lane's rows, as 16-bit pairs (rows 2pr, 2pr + 1)
        uint32_t kp[NI / 2], qp[NI / 2];
        kp[0] = H.k.x; kp[1] = H.k.y; qp[0] = H.q.x; qp[1] = H.q.y;
        if constexpr (NI == 8) { kp[2] = H.k2.x; kp[3] = H.k2.y; qp[2] = H.q2.x; qp[3] = H.q2.y; }
        float kr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) kr[i] = (i & 1) ? EL::hi(kp[i >> 1]) : EL::lo(kp[i >> 1]);
        // Partial S^T (D k) and S^T (D q) over the lane's rows.
        uint32_t sw[NI][4];
        float kv[8], sq[8], kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { kv[c] = 0.f; sq[c] = 0.f; }
#pragma unroll
        for (int i = 0; i < NI; ++i) { sw[i][0] = H.st[i].x; sw[i][1] = H.st[i].y; sw[i][2] = H.st[i].z; sw[i][3] = H.st[i].w; }
        if constexpr (GK) {
            float qr[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) qr[i] = (i & 1) ? EL::hi(qp[i >> 1]) : EL::lo(qp[i >> 1]);
            float dk[NI], dq[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                dk[i] = dd[i] * kr[i];
                dq[i] = dd[i] * qr[i];
                kq = fmaf(kr[i], qr[i], kq);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float s = (c & 1) ? EL::hi(sw[i][c >> 1]) : EL::lo(sw[i][c >> 1]);
                    kv[c] = fmaf(s, dk[i], kv[c]);
                    sq[c] = fmaf(s, dq[i], sq[c]);
                }
        } else {
            // One decay for all rows: the sums run over 16-bit pairs of rows
            // (v_dot2_f32_bf16 / v_dot2_f32_f16, exact products) and take
            // exp(g) afterwards.
#pragma unroll
            for (int pr = 0; pr < NI / 2; ++pr) {
                const uint32_t kb = kp[pr], qb = qp[pr];
                kq = EL::dot2(kb, qb, kq);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // (S[2pr][2u], S[2pr+1][2u]) and (S[2pr][2u+1], S[2pr+1][2u+1])
                    const uint32_t lo = __builtin_amdgcn_perm(sw[2 * pr + 1][u], sw[2 * pr][u], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(sw[2 * pr + 1][u], sw[2 * pr][u], 0x07060302u);
                    kv[2 * u] = EL::dot2(lo, kb, kv[2 * u]);
                    sq[2 * u] = EL::dot2(lo, qb, sq[2 * u]);
                    kv[2 * u + 1] = EL::dot2(hi, kb, kv[2 * u + 1]);
                    sq[2 * u + 1] = EL::dot2(hi, qb, sq[2 * u + 1]);
                }
            }
        }
        // Over the wave: lane row r keeps the totals of columns 8 cg + 2r, + 1.
        float4 t;
        t.x = rows_reduce4(kv[0], kv[2], kv[4], kv[6]);
        t.y = rows_reduce4(kv[1], kv[3], kv[5], kv[7]);
        t.z = rows_reduce4(sq[0], sq[2], sq[4], sq[6]);
        t.w = rows_reduce4(sq[1], sq[3], sq[5], sq[7]);
        kq = rows_sum(kq);
        // |k|^2 and |q|^2 for the in-kernel normalisation.
        float kk = 0.f, qq = 0.f;
        if constexpr (QN) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float qi = (i & 1) ? EL::hi(qp[i >> 1]) : EL::lo(qp[i >> 1]);
                kk = fmaf(kr[i], kr[i], kk);
                qq = fmaf(qi, qi, qq);
            }
            kk = rows_sum(kk);
            qq = rows_sum(qq);
        }
        // Over the workgroup.
        red[par][j][lane] = t;
        if (lane == 0) {
            if constexpr (QN)
                redkq[par][j] = float4{kq, kk, qq, 0.f};
            else
                redkq[par][j].x = kq;
        }
        s1_barrier();
        float4 u = red[par][0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float4 x = red[par][w][lane];
            u.x += x.x; u.y += x.y; u.z += x.z; u.w += x.w;
        }
        float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if constexpr (QN) {
                const float4 x = redkq[par][w];
                z.x += x.x; z.y += x.y; z.z += x.z;
            } else {
                z.x += redkq[par][w].x;
            }
        }
        kq = z.x;
        par ^= 1;
        if constexpr (!GK) { u.x *= a; u.y *= a; u.z *= a; u.w *= a; }
        // With normalised q and k, the sums scale by 1/|k| and 1/|q|, and the
        // update takes k/|k|.
        float rk = 1.f;
        if constexpr (QN) {
            rk = qk_rnorm(z.y);
            const float rq = qk_rnorm(z.z);
            u.x *= rk; u.y *= rk; u.z *= rq; u.w *= rq;
            kq *= rk * rq;
        }
        // delta of this lane row's two columns, then of all eight.
        const uint32_t vw = lr == 0 ? H.v.x : lr == 1 ? H.v.y : lr == 2 ? H.v.z : H.v.w;
        const float d0 = H.beta * (EL::lo(vw) - u.x), d1 = H.beta * (EL::hi(vw) - u.y);
        if (j == 0) {
            const float o0 = p.scale * fmaf(d0, kq, u.z), o1 = p.scale * fmaf(d1, kq, u.w);
            if constexpr (NRM)
                *out_ptr(H) = norm_pair<EL>(o0, o1, H.z, nw0, nw1, p.norm_eps);
            else
                *out_ptr(H) = EL::pack(o0, o1);
        }
        float e0[4], e1[4], dl[8];
        rows_gather(d0, e0);
        rows_gather(d1, e1);
#pragma unroll
        for (int r = 0; r < 4; ++r) { dl[2 * r] = e0[r] * rk; dl[2 * r + 1] = e1[r] * rk; }
        // S' = D S + k delta^T, stored at once.
        const auto srs = brsrc(pool + ((size_t)H.r * Nv + H.h) * DK * DV, DK * DV * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            // The packed words are widened afresh rather than kept widened
            // across the reductions.
            asm volatile("" : "+v"(sw[i][0]), "+v"(sw[i][1]), "+v"(sw[i][2]), "+v"(sw[i][3]));
            uint32_t ow[4];
#pragma unroll
            for (int c = 0; c < 8; c += 2)
                ow[c >> 1] = EL::pack(fmaf(EL::lo(sw[i][c >> 1]), dd[i], kr[i] * dl[c]),
                                         fmaf(EL::hi(sw[i][c >> 1]), dd[i], kr[i] * dl[c + 1]));
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{ow[0], ow[1], ow[2], ow[3]}, srs, ((row0 + i) * DV + cg * 8) * 2, 0, STREAM);
        }
    };

    // The loads of the heads up to hd + (NB - 1) G are in flight while head
    // hd is computed, and the scalars of the head after them; the NB register
    // sets rotate. The scheduling barriers keep each wait for scalars clear
    // of the scalar loads issued after it.
    S1Head H[NB];
    S1Scal C[NB];
    int hd = blockIdx.x;
#pragma unroll
    for (int m = 0; m + 1 < NB; ++m) {
        C[m] = scal(hd + m * G);
        load(H[m], C[m], hd + m * G);
    }
    C[NB - 1] = scal(hd + (NB - 1) * G);
    auto step = [&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        constexpr int f = (m + NB - 1) % NB;
        load(H[f], C[f], hd + (NB - 1) * G);
        __builtin_amdgcn_sched_barrier(0);
        C[m] = scal(hd + NB * G);
        __builtin_amdgcn_sched_barrier(0);
        compute(H[m]);
        hd += G;
        return hd >= nheads;
    };
    while (true) {
        if (step(std::integral_constant<int, 0>{})) break;
        if (step(std::integral_constant<int, 1>{})) break;
        if constexpr (NB > 2) { if (step(std::integral_constant<int, 2 % NB>{})) break; }
        if constexpr (NB > 3) { if (step(std::integral_constant<int, 3 % NB>{})) break; }
    }
}

// Decode calls of two to eight tokens per sequence (speculative steps), bf16 or fp16,
// Dk = Dv = 128. One workgroup of four wavefronts per (b, h): wave j owns the
// 32 rows [32j, 32j + 32) of the state, lane l the columns 8 (l % 16) .. + 7
// of the eight consecutive rows 32j + 8 (l / 16) + i, so that each load or
// store instruction of a wave moves four whole 256-byte rows. The state stays
// in float32 registers across the tokens. Per token, with the decayed state
// S' = D S (D = diag(exp(g) exp(gk_i))):
//   the column sums S'^T k and S'^T q, over the wave's four lane rows by lane
//   swaps and over the four waves through LDS (one barrier);
//   delta = beta (v - S'^T k),  o = scale (S'^T q + delta (k . q));
//   S <- S' + k delta^T, stored when the next token does not overwrite the
//   same slot.
// The next token's inputs are in flight while a token is computed; several
// workgroups per CU cover each other's barrier waits.
namespace mt {
constexpr int DK = 128, DV = 128;
constexpr int NW = 4;            // waves per head (workgroup size 256)
constexpr int RW = DK / NW;      // 32 rows per wave
constexpr int NI = RW / 4;       // 8 rows per lane
}  // namespace mt

// One token's inputs as a lane holds them.
struct MTTok {
    u32x4_t k, q;        // the lane's 8 rows of k and q (16-bit)
    u32x4_t v;           // the lane's 8 columns of v (16-bit)
    u32x4_t gk0, gk1;    // the lane's 8 rows of gk (f32)
    uint32_t beta, g;    // 16-bit in the low half (beta or its logit; a); g as f32 bits
    uint32_t z;          // the epilogue's z at the lane's two output columns (16-bit)
    int w;               // the token's write slot
};

template <typename EL, bool GK, bool FG, bool QN, bool NRM>
__global__ __launch_bounds__(64 * mt::NW) __attribute__((amdgpu_waves_per_eu((GK && (FG || QN)) || NRM ? 3 : 4))) void decode_mt_kernel(DecodeParams p)
{
    using namespace mt;
    __shared__ float4 red[2][NW][64];
    __shared__ float4 redkq[2][NW];   // k . q, |k|^2, |q|^2 of each wave's rows

    const int lane = threadIdx.x & 63;
    const int j = uniform(threadIdx.x >> 6);
    const int lr = lane >> 4, cg = lane & 15;
    const int row0 = j * RW + lr * NI;   // the lane's first row
    const int Nv = p.Nv, S = p.S, rep = p.Nv / p.Nk;
    const int b = blockIdx.x / Nv, h = blockIdx.x % Nv;
    const size_t vh = (size_t)b * Nv + h, qk = (size_t)b * p.Nk + h / rep;

    int L = ld_const(p.lens, b);
    L = L < 0 ? 0 : (L > S ? S : L);
    const int n = p.nacc ? ld_const(p.nacc, b) : L;
    int r = -1;
    if (L > 0 && n >= 1 && n <= S) r = ld_const(p.idx, (size_t)b * S + n - 1);
    // Output words of this lane in wave 0: columns 8 cg + 2 lr, + 1 of each token.
    uint32_t *optr = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.out) + vh * S * DV + cg * 8 + lr * 2);
    if (r < 0 || r >= p.slots) {
        if (j == 0)
            for (int t = 0; t < S; ++t) optr[t * (DV / 2)] = 0u;
        return;
    }

    // Token inputs through buffer resources bounded by the valid tokens: the
    // prefetch past the last one reads zeros.
    const auto krs = brsrc(static_cast<const uint16_t *>(p.k) + qk * S * DK, L * DK * 2);
    const auto qrs = brsrc(static_cast<const uint16_t *>(p.q) + qk * S * DK, L * DK * 2);
    const auto vrs = brsrc(static_cast<const uint16_t *>(p.v) + vh * S * DV, L * DV * 2);
    const auto brs = brsrc(static_cast<const uint16_t *>(p.beta) + vh * S, L * 2);
    // g (float32), or with fused gates the raw a (16-bit)
    const auto grs = FG ? brsrc(static_cast<const uint16_t *>(p.gate_a) + vh * S, L * 2)
                        : brsrc(p.g ? p.g + vh * S : nullptr, p.g ? L * 4 : 0);
    const float alog = FG ? __int_as_float(ld_const(reinterpret_cast<const int32_t *>(p.A_log), h)) : 0.f;
    const float dtb = FG ? __int_as_float(ld_const(reinterpret_cast<const int32_t *>(p.dt_bias), h)) : 0.f;
    const auto gkrs = brsrc(GK ? p.gk + vh * S * DK : nullptr, GK ? L * DK * 4 : 0);
    // Gated RMSNorm epilogue (NRM): z of each token's row, w of the lane's columns.
    const auto zrs = brsrc(NRM ? static_cast<const uint16_t *>(p.norm_z) + vh * S * DV : nullptr, NRM ? L * DV * 2 : 0);
    float nw0 = 0.f, nw1 = 0.f;
    if constexpr (NRM) {
        const u32x2_t nwv = __builtin_amdgcn_raw_buffer_load_b64(brsrc(p.norm_w, DV * 4), (cg * 8 + lr * 2) * 4, 0, 0);
        nw0 = __uint_as_float(nwv.x);
        nw1 = __uint_as_float(nwv.y);
    }
    auto ld_tok = [&](MTTok &T, int t) __attribute__((always_inline)) {
        T.k = __builtin_amdgcn_raw_buffer_load_b128(krs, (t * DK + row0) * 2, 0, 0);
        T.q = __builtin_amdgcn_raw_buffer_load_b128(qrs, (t * DK + row0) * 2, 0, 0);
        T.v = __builtin_amdgcn_raw_buffer_load_b128(vrs, (t * DV + cg * 8) * 2, 0, 0);
        if constexpr (GK) {
            T.gk0 = __builtin_amdgcn_raw_buffer_load_b128(gkrs, (t * DK + row0) * 4, 0, 0);
            T.gk1 = __builtin_amdgcn_raw_buffer_load_b128(gkrs, (t * DK + row0) * 4 + 16, 0, 0);
        }
        T.beta = __builtin_amdgcn_raw_buffer_load_b16(brs, t * 2, 0, 0);
        if constexpr (FG)
            T.g = __builtin_amdgcn_raw_buffer_load_b16(grs, t * 2, 0, 0);
        else
            T.g = __builtin_amdgcn_raw_buffer_load_b32(grs, t * 4, 0, 0);
        if constexpr (NRM) T.z = __builtin_amdgcn_raw_buffer_load_b32(zrs, (t * DV + cg * 8 + lr * 2) * 2, 0, 0);
        T.w = ld_const(p.idx, (size_t)b * S + (t < S ? t : S - 1));
    };

    MTTok cur, nxt;
    ld_tok(cur, 0);
    float st[NI][8];
    {
        const auto srs = brsrc(static_cast<const uint16_t *>(p.pool) + ((size_t)r * Nv + h) * DK * DV, DK * DV * 2);
        u32x4_t sw[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) sw[i] = __builtin_amdgcn_raw_buffer_load_b128(srs, ((row0 + i) * DV + cg * 8) * 2, 0, STREAM);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t w4[4] = {sw[i].x, sw[i].y, sw[i].z, sw[i].w};
#pragma unroll
            for (int c = 0; c < 8; ++c) st[i][c] = (c & 1) ? EL::hi(w4[c >> 1]) : EL::lo(w4[c >> 1]);
        }
    }
    uint16_t *pool = static_cast<uint16_t *>(p.pool);
    int par = 0;
    for (int t = 0; t < L; ++t) {
        ld_tok(nxt, t + 1);
        const float a = FG ? __expf(gate_g(EL::to(cur.g), alog, dtb))
                           : (p.g ? __expf(__uint_as_float(cur.g)) : 1.f);
        float dd[NI], kr[NI], qr[NI];
        {
            const uint32_t kw[4] = {cur.k.x, cur.k.y, cur.k.z, cur.k.w}, qw[4] = {cur.q.x, cur.q.y, cur.q.z, cur.q.w};
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kr[i] = (i & 1) ? EL::hi(kw[i >> 1]) : EL::lo(kw[i >> 1]);
                qr[i] = (i & 1) ? EL::hi(qw[i >> 1]) : EL::lo(qw[i >> 1]);
            }
            if constexpr (GK) {
                const uint32_t gw[8] = {cur.gk0.x, cur.gk0.y, cur.gk0.z, cur.gk0.w, cur.gk1.x, cur.gk1.y, cur.gk1.z, cur.gk1.w};
#pragma unroll
                for (int i = 0; i < NI; ++i) dd[i] = a * __expf(__uint_as_float(gw[i]));
            } else {
#pragma unroll
                for (int i = 0; i < NI; ++i) dd[i] = a;
            }
        }
        // Decay, then the partial column sums S'^T k, S'^T q and k . q over
        // the lane's rows.
        float kv[8], sq[8], kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { kv[c] = 0.f; sq[c] = 0.f; }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            kq = fmaf(kr[i], qr[i], kq);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st[i][c] *= dd[i];
                kv[c] = fmaf(st[i][c], kr[i], kv[c]);
                sq[c] = fmaf(st[i][c], qr[i], sq[c]);
            }
        }
        // Over the wave: lane row r keeps the totals of columns 8 cg + 2r, + 1.
        float4 tt;
        tt.x = rows_reduce4(kv[0], kv[2], kv[4], kv[6]);
        tt.y = rows_reduce4(kv[1], kv[3], kv[5], kv[7]);
        tt.z = rows_reduce4(sq[0], sq[2], sq[4], sq[6]);
        tt.w = rows_reduce4(sq[1], sq[3], sq[5], sq[7]);
        kq = rows_sum(kq);
        float kk = 0.f, qq = 0.f;   // |k|^2, |q|^2 for the in-kernel normalisation
        if constexpr (QN) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kk = fmaf(kr[i], kr[i], kk);
                qq = fmaf(qr[i], qr[i], qq);
            }
            kk = rows_sum(kk);
            qq = rows_sum(qq);
        }
        // Over the workgroup. The two buffers alternate by token: a wave can
        // write the next token's sums only after every wave has passed this
        // token's barrier, so after every read of the other buffer.
        red[par][j][lane] = tt;
        if (lane == 0) {
            if constexpr (QN)
                redkq[par][j] = float4{kq, kk, qq, 0.f};
            else
                redkq[par][j].x = kq;
        }
        s1_barrier();
        float4 u = red[par][0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float4 x = red[par][w][lane];
            u.x += x.x; u.y += x.y; u.z += x.z; u.w += x.w;
        }
        float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            if constexpr (QN) {
                const float4 x = redkq[par][w];
                z.x += x.x; z.y += x.y; z.z += x.z;
            } else {
                z.x += redkq[par][w].x;
            }
        }
        kq = z.x;
        par ^= 1;
        // With normalised q and k the sums scale by 1/|k| and 1/|q|, and the
        // update takes k/|k|.
        float rk = 1.f;
        if constexpr (QN) {
            rk = qk_rnorm(z.y);
            const float rq = qk_rnorm(z.z);
            u.x *= rk; u.y *= rk; u.z *= rq; u.w *= rq;
            kq *= rk * rq;
        }
        const float beta = FG ? gate_sigmoid(EL::to(cur.beta)) : EL::to(cur.beta);
        const uint32_t vw = lr == 0 ? cur.v.x : lr == 1 ? cur.v.y : lr == 2 ? cur.v.z : cur.v.w;
        const float d0 = beta * (EL::lo(vw) - u.x), d1 = beta * (EL::hi(vw) - u.y);
        if (j == 0) {
            const float o0 = p.scale * fmaf(d0, kq, u.z), o1 = p.scale * fmaf(d1, kq, u.w);
            if constexpr (NRM)
                optr[t * (DV / 2)] = norm_pair<EL>(o0, o1, cur.z, nw0, nw1, p.norm_eps);
            else
                optr[t * (DV / 2)] = EL::pack(o0, o1);
        }
        float e0[4], e1[4], dl[8];
        rows_gather(d0, e0);
        rows_gather(d1, e1);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) { dl[2 * q4] = e0[q4] * rk; dl[2 * q4 + 1] = e1[q4] * rk; }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) st[i][c] = fmaf(kr[i], dl[c], st[i][c]);
        // The state after this token, unless the next token overwrites the
        // same slot.
        const int w = cur.w;
        const bool last = (t == L - 1) || (nxt.w != w);
        if (last && w >= 0 && w < p.slots) {
            const auto wrs = brsrc(pool + ((size_t)w * Nv + h) * DK * DV, DK * DV * 2);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                uint32_t ow[4];
#pragma unroll
                for (int c = 0; c < 8; c += 2) ow[c >> 1] = EL::pack(st[i][c], st[i][c + 1]);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{ow[0], ow[1], ow[2], ow[3]}, wrs, ((row0 + i) * DV + cg * 8) * 2, 0, STREAM);
            }
        }
        cur = nxt;
    }
    if (j == 0)
        for (int t = L; t < S; ++t) optr[t * (DV / 2)] = 0u;
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

// The compiled variant for a call: per-key gate, fused gates, q/k
// normalisation, epilogue.
template <typename EL>
static const void *s1_kernel(const DecodeParams &p)
{
    static const void *const fns[16] = {
        (const void *)decode_s1_kernel<EL, false, false, false, false>, (const void *)decode_s1_kernel<EL, true, false, false, false>,
        (const void *)decode_s1_kernel<EL, false, true, false, false>, (const void *)decode_s1_kernel<EL, true, true, false, false>,
        (const void *)decode_s1_kernel<EL, false, false, true, false>, (const void *)decode_s1_kernel<EL, true, false, true, false>,
        (const void *)decode_s1_kernel<EL, false, true, true, false>, (const void *)decode_s1_kernel<EL, true, true, true, false>,
        (const void *)decode_s1_kernel<EL, false, false, false, true>, (const void *)decode_s1_kernel<EL, true, false, false, true>,
        (const void *)decode_s1_kernel<EL, false, true, false, true>, (const void *)decode_s1_kernel<EL, true, true, false, true>,
        (const void *)decode_s1_kernel<EL, false, false, true, true>, (const void *)decode_s1_kernel<EL, true, false, true, true>,
        (const void *)decode_s1_kernel<EL, false, true, true, true>, (const void *)decode_s1_kernel<EL, true, true, true, true>};
    return fns[(p.gk ? 1 : 0) + (p.gate_a ? 2 : 0) + (p.qk_norm ? 4 : 0) + (p.norm_z ? 8 : 0)];
}
template <typename EL>
static const void *mt_kernel(const DecodeParams &p)
{
    static const void *const fns[16] = {
        (const void *)decode_mt_kernel<EL, false, false, false, false>, (const void *)decode_mt_kernel<EL, true, false, false, false>,
        (const void *)decode_mt_kernel<EL, false, true, false, false>, (const void *)decode_mt_kernel<EL, true, true, false, false>,
        (const void *)decode_mt_kernel<EL, false, false, true, false>, (const void *)decode_mt_kernel<EL, true, false, true, false>,
        (const void *)decode_mt_kernel<EL, false, true, true, false>, (const void *)decode_mt_kernel<EL, true, true, true, false>,
        (const void *)decode_mt_kernel<EL, false, false, false, true>, (const void *)decode_mt_kernel<EL, true, false, false, true>,
        (const void *)decode_mt_kernel<EL, false, true, false, true>, (const void *)decode_mt_kernel<EL, true, true, false, true>,
        (const void *)decode_mt_kernel<EL, false, false, true, true>, (const void *)decode_mt_kernel<EL, true, false, true, true>,
        (const void *)decode_mt_kernel<EL, false, true, true, true>, (const void *)decode_mt_kernel<EL, true, true, true, true>};
    return fns[(p.gk ? 1 : 0) + (p.gate_a ? 2 : 0) + (p.qk_norm ? 4 : 0) + (p.norm_z ? 8 : 0)];
}

hipError_t launch_decode(int dtype, int Dk, int Dv, const DecodeParams &p, hipStream_t s, bool *supported,
                         bool *norm_done)
{
    *norm_done = false;
    // decode_s1_kernel reads beta (and a) of two heads as one 32-bit word, so
    // it takes an even number of heads; odd counts go to decode_mt_kernel,
    // whose bounded 16-bit loads never read past the last head.
    if (dtype != 0 && p.S == 1 && Dk == s1::DK && Dv == s1::DV && ((int64_t)p.B * p.Nv) % 2 == 0) {
        *supported = true;
        *norm_done = true;
        const int nheads = p.B * p.Nv;
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
        const int groups = s1::PER_CU * ncu;
        const dim3 grid((unsigned)(nheads < groups ? nheads : groups)), block(64 * s1::NW);
        DecodeParams pc = p;
        int nh = nheads;
        void *args[] = {&pc, &nh};
        const void *fn = dtype == 1 ? s1_kernel<BF16>(p) : s1_kernel<F16>(p);
        return hipLaunchKernel(fn, grid, block, args, 0, s);
    }
    if (dtype != 0 && Dk == mt::DK && Dv == mt::DV) {
        *supported = true;
        *norm_done = true;
        DecodeParams pc = p;
        void *args[] = {&pc};
        const void *fn = dtype == 1 ? mt_kernel<BF16>(p) : mt_kernel<F16>(p);
        return hipLaunchKernel(fn, dim3((unsigned)(p.B * p.Nv)), dim3(64 * mt::NW), args, 0, s);
    }
    if (dtype == 1) return launch_typed<bf16_t>(Dk, Dv, p, s, supported);
    if (dtype == 2) return launch_typed<f16_t>(Dk, Dv, p, s, supported);
    return launch_typed<float>(Dk, Dv, p, s, supported);
}

}  // namespace gdr
