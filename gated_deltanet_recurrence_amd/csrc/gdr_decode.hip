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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Decode step with one token per sequence (S = 1), bf16, Dk = Dv = 128: the
// state stream as a persistent, software-pipelined walk. Each wavefront owns
// the 32-column tiles w, w + G, w + 2G, ... of all (b, h) states and keeps
// the loads of the next tile in flight while it updates and stores the
// current one (two register sets, alternating). Every load goes through a
// buffer resource whose size is zero when the tile has nothing to read (a
// skipped sequence, or past the last tile), so loads never sit under a branch
// and never make the wave wait before their data is used.
//
// With one token the output needs no pass over the updated state:
//   S' = D S + k delta^T,  D = diag(exp(g) exp(gk_i)),  delta = beta (v - S^T D k)
//   o  = scale S'^T q = scale (S^T (D q) + delta (k . q))
// so S^T (D k) and S^T (D q) come from one pass over S and the store of S'
// follows the update directly.
namespace s1 {
constexpr int DK = 128, DV = 128, TV = 32, VEC = 8;
constexpr int CG = TV / VEC;    // 4 column groups of 8 columns
constexpr int RG = 64 / CG;     // 16 lanes across the rows
constexpr int RPL = DK / RG;    // 8 rows per lane
constexpr int NT = DV / TV;     // 4 tiles per head
constexpr int WPB = 4;          // wavefronts per workgroup
constexpr int WAVES = 2048;     // persistent wavefronts (8 per CU)
}  // namespace s1

// Per-tile values read through the scalar cache, one half-step before use.
struct S1Scal { int32_t len, nacc, idx, beta2, g; };
// Per-tile values after resolution, and the vector registers of its loads.
struct S1Tile { int b, h, ct, r; float beta, g; };
struct S1Regs {
    u32x4_t st[s1::RPL];   // state rows, 8 bf16 columns each
    u32x4_t k, q, v;       // k, q rows of this lane; v columns of this lane (bf16)
    u32x4_t gk[2];         // per-key gate of this lane's rows (f32)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

template <bool GK>
__global__ __launch_bounds__(256) void decode_s1_kernel(DecodeParams p, int ntiles)
{
    using namespace s1;
    const int lane = threadIdx.x & 63;
    const int w = uniform(blockIdx.x * WPB + (threadIdx.x >> 6));
    const int G = uniform(gridDim.x * WPB);
    const int Nv = p.Nv, rep = p.Nv / p.Nk;
    const int rg = lane % RG, cg = lane / RG;
    const int row0 = rg * RPL;

    const bf16_t *q = static_cast<const bf16_t *>(p.q);
    const bf16_t *k = static_cast<const bf16_t *>(p.k);
    const bf16_t *v = static_cast<const bf16_t *>(p.v);
    bf16_t *pool = static_cast<bf16_t *>(p.pool);
    bf16_t *out = static_cast<bf16_t *>(p.out);
    // Optional inputs are read from a valid stand-in address and discarded,
    // so no load sits under a branch.
    const int32_t *nacc_src = p.nacc ? p.nacc : p.lens;
    const int32_t *g_src = p.g ? reinterpret_cast<const int32_t *>(p.g) : p.lens;
    const int32_t *beta_src = static_cast<const int32_t *>(p.beta);

    auto coords = [&](int tile, int &b, int &h, int &ct) __attribute__((always_inline)) {
        const int tt = tile < ntiles ? tile : 0;
        ct = tt % NT;
        const int bh = tt / NT;
        h = bh % Nv;
        b = bh / Nv;
    };
    // Issues the scalar loads of a tile (they complete while the wave works).
    auto scal = [&](int tile) __attribute__((always_inline)) {
        int b, h, ct;
        coords(tile, b, h, ct);
        const size_t vh = (size_t)b * Nv + h;
        S1Scal c;
        c.len = ld_const(p.lens, b);
        c.nacc = ld_const(nacc_src, b);
        c.idx = ld_const(p.idx, b);
        c.beta2 = ld_const(beta_src, vh >> 1);
        c.g = ld_const(g_src, p.g ? vh : 0);
        return c;
    };
    // Resolves a tile from its scalars and issues its vector loads.
    auto vec = [&](S1Regs &R, S1Tile &t, const S1Scal &c, int tile) __attribute__((always_inline)) {
        coords(tile, t.b, t.h, t.ct);
        const size_t vh = (size_t)t.b * Nv + t.h;
        const int L = c.len < 0 ? 0 : (c.len > 1 ? 1 : c.len);
        const int n = p.nacc ? c.nacc : L;
        const int r = (tile < ntiles && L == 1 && n == 1) ? c.idx : -1;
        t.r = (r >= 0 && r < p.slots) ? r : -1;
        t.beta = __uint_as_float(((uint32_t)c.beta2 >> (16 * (int)(vh & 1))) << 16);
        t.g = p.g ? __int_as_float(c.g) : 0.f;
        const bool on = t.r >= 0;
        const size_t qk = (size_t)t.b * p.Nk + t.h / rep;
        const int col = t.ct * TV;
        const auto srs = brsrc(pool + ((size_t)(on ? t.r : 0) * Nv + t.h) * DK * DV + col, on ? (DK * DV - col) * 2 : 0);
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            R.st[i] = __builtin_amdgcn_raw_buffer_load_b128(srs, ((row0 + i) * DV + cg * VEC) * 2, 0, 0);
        const int tb = on ? DK * 2 : 0;
        R.k = __builtin_amdgcn_raw_buffer_load_b128(brsrc(k + qk * DK, tb), row0 * 2, 0, 0);
        R.q = __builtin_amdgcn_raw_buffer_load_b128(brsrc(q + qk * DK, tb), row0 * 2, 0, 0);
        R.v = __builtin_amdgcn_raw_buffer_load_b128(brsrc(v + vh * DV + col, on ? (DV - col) * 2 : 0), cg * VEC * 2, 0, 0);
        if constexpr (GK) {
            const auto grs = brsrc(p.gk + vh * DK, on ? DK * 4 : 0);
            R.gk[0] = __builtin_amdgcn_raw_buffer_load_b128(grs, row0 * 4, 0, 0);
            R.gk[1] = __builtin_amdgcn_raw_buffer_load_b128(grs, row0 * 4 + 16, 0, 0);
        }
    };
    // A tile that is skipped still waits for its (empty) loads, so that every
    // path leaves the register set settled: otherwise the compiler has to wait
    // for it where the paths meet, before the next prefetch is issued.
    auto settle = [&](const S1Regs &R) __attribute__((always_inline)) {
        uint32_t x = R.k.x ^ R.q.x ^ R.v.x;
#pragma unroll
        for (int i = 0; i < RPL; ++i) x ^= R.st[i].x ^ R.st[i].w;
        if constexpr (GK) x ^= R.gk[0].x ^ R.gk[1].x;
        asm volatile("" ::"v"(x));
    };
    auto compute = [&](const S1Regs &R, const S1Tile &t, int tile) __attribute__((always_inline)) {
        if (tile >= ntiles) {
            settle(R);
            return;
        }
        const size_t vh = (size_t)t.b * Nv + t.h;
        const int col = t.ct * TV + cg * VEC;
        bf16_t *op = out + vh * DV + col;
        if (t.r < 0) {
            settle(R);
            if (rg == 0) *reinterpret_cast<u32x4_t *>(op) = u32x4_t{0u, 0u, 0u, 0u};
            return;
        }
        // D = exp(g) exp(gk_i)
        const float a = __expf(t.g);
        const uint32_t kw[4] = {R.k.x, R.k.y, R.k.z, R.k.w}, qw[4] = {R.q.x, R.q.y, R.q.z, R.q.w};
        float dd[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) dd[i] = a;
        if constexpr (GK) {
            const uint32_t gw[8] = {R.gk[0].x, R.gk[0].y, R.gk[0].z, R.gk[0].w, R.gk[1].x, R.gk[1].y, R.gk[1].z, R.gk[1].w};
#pragma unroll
            for (int i = 0; i < RPL; ++i) dd[i] = a * __expf(__uint_as_float(gw[i]));
        }
        float kr[RPL], dk[RPL], dq[RPL], kq = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float ki = (i & 1) ? bf16_hi(kw[i >> 1]) : bf16_lo(kw[i >> 1]);
            const float qi = (i & 1) ? bf16_hi(qw[i >> 1]) : bf16_lo(qw[i >> 1]);
            kr[i] = ki;
            dk[i] = dd[i] * ki;
            dq[i] = dd[i] * qi;
            kq = fmaf(ki, qi, kq);
        }
        // One pass over S: S^T (D k) and S^T (D q) for this lane's columns.
        float st[RPL][VEC];
        float kv[VEC], sq[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) { kv[c] = 0.f; sq[c] = 0.f; }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const uint32_t sw[4] = {R.st[i].x, R.st[i].y, R.st[i].z, R.st[i].w};
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                st[i][c] = (c & 1) ? bf16_hi(sw[c >> 1]) : bf16_lo(sw[c >> 1]);
                kv[c] = fmaf(st[i][c], dk[i], kv[c]);
                sq[c] = fmaf(st[i][c], dq[i], sq[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) { kv[c] = group_sum<RG>(kv[c]); sq[c] = group_sum<RG>(sq[c]); }
        kq = group_sum<RG>(kq);
        // delta, the updated state (stored at once), then the output.
        const uint32_t vw[4] = {R.v.x, R.v.y, R.v.z, R.v.w};
        float dl[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) dl[c] = t.beta * (((c & 1) ? bf16_hi(vw[c >> 1]) : bf16_lo(vw[c >> 1])) - kv[c]);
        const auto srs = brsrc(pool + ((size_t)t.r * Nv + t.h) * DK * DV + t.ct * TV, (DK * DV - t.ct * TV) * 2);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            uint32_t ow[4];
#pragma unroll
            for (int c = 0; c < VEC; c += 2)
                ow[c >> 1] = pack_bf16x2(fmaf(st[i][c], dd[i], kr[i] * dl[c]), fmaf(st[i][c + 1], dd[i], kr[i] * dl[c + 1]));
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{ow[0], ow[1], ow[2], ow[3]}, srs, ((row0 + i) * DV + cg * VEC) * 2, 0, 0);
        }
        if (rg == 0) {
            uint32_t ow[4];
#pragma unroll
            for (int c = 0; c < VEC; c += 2)
                ow[c >> 1] = pack_bf16x2(p.scale * fmaf(dl[c], kq, sq[c]), p.scale * fmaf(dl[c + 1], kq, sq[c + 1]));
            *reinterpret_cast<u32x4_t *>(op) = u32x4_t{ow[0], ow[1], ow[2], ow[3]};
        }
    };

    // Half-step for tile i (register set X): consume the scalars of tile
    // i + G (issued one half-step earlier) and issue its vector loads into the
    // other set; then issue the scalars of tile i + 2G; then compute tile i.
    // The scheduling barriers keep each wait for scalars clear of the loads
    // issued after it.
    S1Regs A, B;
    S1Tile tA, tB;
    S1Scal cX, cY;
    int tile = w;
    cX = scal(tile);
    vec(A, tA, cX, tile);
    cY = scal(tile + G);
    while (true) {
        vec(B, tB, cY, tile + G);
        __builtin_amdgcn_sched_barrier(0);
        cX = scal(tile + 2 * G);
        __builtin_amdgcn_sched_barrier(0);
        compute(A, tA, tile);
        tile += G;
        if (tile >= ntiles) break;
        vec(A, tA, cX, tile + G);
        __builtin_amdgcn_sched_barrier(0);
        cY = scal(tile + 2 * G);
        __builtin_amdgcn_sched_barrier(0);
        compute(B, tB, tile);
        tile += G;
        if (tile >= ntiles) break;
    }
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
    if (dtype == 1 && p.S == 1 && Dk == s1::DK && Dv == s1::DV) {
        *supported = true;
        const int ntiles = p.B * p.Nv * s1::NT;
        const int waves = ntiles < s1::WAVES ? ntiles : s1::WAVES;
        const dim3 grid((unsigned)((waves + s1::WPB - 1) / s1::WPB)), block(64 * s1::WPB);
        DecodeParams pc = p;
        int nt = ntiles;
        void *args[] = {&pc, &nt};
        const void *fn = p.gk ? (const void *)decode_s1_kernel<true> : (const void *)decode_s1_kernel<false>;
        return hipLaunchKernel(fn, grid, block, args, 0, s);
    }
    if (dtype == 1) return launch_typed<bf16_t>(Dk, Dv, p, s, supported);
    return launch_typed<float>(Dk, Dv, p, s, supported);
}

}  // namespace gdr
