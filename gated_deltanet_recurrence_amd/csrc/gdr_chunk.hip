// Chunked prefill of the Gated Delta Rule on gfx950.
//
// Operation (lite_boost.ops.chunk_gated_delta_rule, MindSpore Lite API page,
// formula and parameters; the Gated DeltaNet blog post,
// torch_chunk_gated_delta_rule, steps 1-8; inferencelayer deltanet.rs,
// core_chunk derivation). For one sequence, one value head and one chunk of
// C tokens entering with state S0, with gamma the in-chunk cumulative log
// decay (zeros when g is absent):
//
//   A[r,i] = beta_r (k_r . k_i) exp(gamma_r - gamma_i)       i <  r   (else 0)
//   P[r,i] =        (q_r . k_i) exp(gamma_r - gamma_i)       i <= r   (else 0)
//   T      = (I + A)^-1                                      unit lower triangular
//   X      = diag(beta) (V - diag(exp(gamma)) K S0)
//   Vnew   = T X                                            what each token writes
//   O      = scale (diag(exp(gamma)) Q S0 + P Vnew)
//   S      = exp(gamma_last) S0 + (diag(exp(gamma_last - gamma)) K)^T Vnew
//
// Decay ratios are formed from differences of log decays, never as products
// of exp(gamma) and exp(-gamma). Tokens past the valid length of a partial
// chunk enter as identity steps (k = q = v = beta = 0, g = 0) by selection,
// so padded inputs are never read; their outputs are written as exact zeros.
//
// Two kernels:
//  * chunk_mfma_kernel — bf16 I/O, Dk = Dv = 128, C = 64. One workgroup of
//    four wavefronts per (sequence, value head, 64-column tile of Dv); the
//    columns of S evolve independently, so each tile carries its own slice of
//    the state through all chunks in float32 MFMA accumulators. All dense
//    products run on v_mfma_f32_16x16x32_bf16 with bf16 operands staged in LDS
//    in the layout each operand needs (16-byte reads). T is built per chunk:
//    each 16x16 diagonal block as the finite product
//    (I - A)(I + A^2)(I + A^4)(I + A^8) (A is nilpotent of index 16), computed
//    in registers with v_mfma_f32_16x16x16_bf16 (a result's register layout
//    is directly the right-hand operand layout, and its transpose the
//    left-hand one), then the off-diagonal blocks by block forward
//    substitution, T_ij = -T_ii sum_{j<=m<i} A_im T_mj, one block diagonal at
//    a time.
//  * chunk_f32_kernel — float32 I/O, small heads. The same chunk algorithm in
//    plain float32 arithmetic; T by row-wise forward substitution.
#include <atomic>

#include "gdr_common.h"

namespace gdr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mma32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(bf16x4_t a, bf16x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4_t to_bf4(f32x4_t x)
{
    bf16x4_t r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ f32x4_t zero4()
{
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
namespace mk {
constexpr int C = 64;        // chunk length
constexpr int DK = 128;      // key head size
constexpr int DV = 128;      // value head size
constexpr int DVT = 64;      // value columns per workgroup
constexpr int NT = DV / DVT; // column tiles per head
constexpr int LDK = DK + 8;  // padded row stride (elements) of 128-wide bf16 rows
constexpr int LDC = C + 8;   // padded row stride of 64-wide bf16 rows
constexpr int LDA = C + 4;   // padded row stride of the float32 A matrix
// LDS carve-up (bytes)
constexpr int OFF_K = 0;                              // K rows          [C][LDK]   bf16
constexpr int OFF_Q = OFF_K + C * LDK * 2;            // Q rows          [C][LDK]   bf16
constexpr int OFF_KT = OFF_Q + C * LDK * 2;           // decayed K^T     [DK][LDC]  bf16
constexpr int OFF_V = OFF_KT + DK * LDC * 2;          // V tile rows     [C][LDC]   bf16
constexpr int OFF_ST = OFF_V + C * LDC * 2;           // S^T tile        [DVT][LDK] bf16
constexpr int OFF_XT = OFF_ST + DVT * LDK * 2;        // X^T             [DVT][LDC] bf16
constexpr int OFF_VNT = OFF_XT + DVT * LDC * 2;       // Vnew^T          [DVT][LDC] bf16
constexpr int OFF_T = OFF_VNT + DVT * LDC * 2;        // T rows          [C][LDC]   bf16
constexpr int OFF_P = OFF_T + C * LDC * 2;            // P rows          [C][LDC]   bf16
constexpr int OFF_A = OFF_P + C * LDC * 2;            // A rows          [C][LDA]   f32
constexpr int OFF_TD = OFF_A + C * LDA * 4;           // T block dumps   [3][4][64] f32x4
constexpr int OFF_BG = OFF_TD + 3 * 4 * 64 * 16;      // beta, g         [2][C]     f32
constexpr int LDS_BYTES = OFF_BG + 2 * C * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
}  // namespace mk

__global__ __launch_bounds__(256) void chunk_mfma_kernel(ChunkParams p, int units)
{
    using namespace mk;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16 *Ks = reinterpret_cast<__bf16 *>(smem + OFF_K);
    __bf16 *Qs = reinterpret_cast<__bf16 *>(smem + OFF_Q);
    __bf16 *KTs = reinterpret_cast<__bf16 *>(smem + OFF_KT);
    __bf16 *Vs = reinterpret_cast<__bf16 *>(smem + OFF_V);
    __bf16 *STs = reinterpret_cast<__bf16 *>(smem + OFF_ST);
    __bf16 *XTs = reinterpret_cast<__bf16 *>(smem + OFF_XT);
    __bf16 *VNTs = reinterpret_cast<__bf16 *>(smem + OFF_VNT);
    __bf16 *Ts = reinterpret_cast<__bf16 *>(smem + OFF_T);
    __bf16 *Ps = reinterpret_cast<__bf16 *>(smem + OFF_P);
    float *As = reinterpret_cast<float *>(smem + OFF_A);
    f32x4_t *TD = reinterpret_cast<f32x4_t *>(smem + OFF_TD);
    float *betas = reinterpret_cast<float *>(smem + OFF_BG);
    float *gs = betas + C;

    // Workgroup -> unit. Workgroups are dealt round-robin to the 8 XCDs, so
    // consecutive units (the value heads and column tiles that share one
    // (b, key head) and therefore the same q/k) go to one XCD and its L2.
    const int nwg = gridDim.x;
    const int u = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    if (u >= units) return;
    const int Nk = p.Nk, Nv = p.Nv, S = p.S;
    const int rep = Nv / Nk;
    const int tile = u % NT;
    const int hr = (u / NT) % rep;
    const int bk = u / (NT * rep);
    const int kh = bk % Nk;
    const int b = bk / Nk;
    const int h = kh * rep + hr;
    const int col0 = tile * DVT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int n = lane & 15;   // column within a 16x16 tile
    const int g4 = lane >> 4;  // 4-row group within a 16x16 tile

    int L = p.lens ? p.lens[b] : S;
    L = L < 0 ? 0 : (L > S ? S : L);

    const bf16_t *qb = static_cast<const bf16_t *>(p.q) + ((size_t)b * Nk + kh) * S * DK;
    const bf16_t *kb = static_cast<const bf16_t *>(p.k) + ((size_t)b * Nk + kh) * S * DK;
    const bf16_t *vb = static_cast<const bf16_t *>(p.v) + ((size_t)b * Nv + h) * S * DV + col0;
    const bf16_t *betab = static_cast<const bf16_t *>(p.beta) + ((size_t)b * Nv + h) * S;
    const float *gb = p.g ? p.g + ((size_t)b * Nv + h) * S : nullptr;
    bf16_t *ob = static_cast<bf16_t *>(p.out) + ((size_t)b * Nv + h) * S * DV + col0;
    const bf16_t *ib = p.init ? static_cast<const bf16_t *>(p.init) + ((size_t)b * Nv + h) * DK * DV + col0 : nullptr;
    bf16_t *fb = static_cast<bf16_t *>(p.fin) + ((size_t)b * Nv + h) * DK * DV + col0;

    // State slice owned by this wave: key rows [32w, 32w + 32) x the tile's
    // DVT columns, as 2 x 4 MFMA accumulator tiles: st[rt][ct][i] holds
    // S[32w + 16rt + 4*g4 + i][16ct + n].
    f32x4_t st[2][DVT / 16];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < DVT / 16; ++ct) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dk = 32 * w + 16 * rt + 4 * g4 + i;
                st[rt][ct][i] = ib ? to_f32(ib[(size_t)dk * DV + 16 * ct + n]) : 0.f;
            }
        }

    // T's blocks above the diagonal stay zero for the whole kernel.
    for (int e = tid; e < C * LDC; e += 256) Ts[e] = (__bf16)0.f;

    // S^T (bf16) for the first chunk's products.
    auto write_st = [&]() {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct)
                *reinterpret_cast<bf16x4_t *>(STs + (16 * ct + n) * LDK + 32 * w + 16 * rt + 4 * g4) = to_bf4(st[rt][ct]);
    };
    write_st();

    const int nchunks = (L + C - 1) / C;
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int nval = min(C, L - t0);

        // ---- load the chunk (rows past the valid length become zeros) ----
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int id = tid + 256 * m;
            const int row = id >> 4, cv = (id & 15) * 8;
            uint4 kv4 = make_uint4(0, 0, 0, 0), qv4 = make_uint4(0, 0, 0, 0);
            if (row < nval) {
                kv4 = *reinterpret_cast<const uint4 *>(kb + (size_t)(t0 + row) * DK + cv);
                qv4 = *reinterpret_cast<const uint4 *>(qb + (size_t)(t0 + row) * DK + cv);
            }
            *reinterpret_cast<uint4 *>(Ks + row * LDK + cv) = kv4;
            *reinterpret_cast<uint4 *>(Qs + row * LDK + cv) = qv4;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int id = tid + 256 * m;
            const int row = id >> 3, cv = (id & 7) * 8;
            uint4 v4 = make_uint4(0, 0, 0, 0);
            if (row < nval) v4 = *reinterpret_cast<const uint4 *>(vb + (size_t)(t0 + row) * DV + cv);
            *reinterpret_cast<uint4 *>(Vs + row * LDC + cv) = v4;
        }
        if (tid < C) {
            betas[tid] = tid < nval ? to_f32(betab[t0 + tid]) : 0.f;
            gs[tid] = (gb && tid < nval) ? gb[t0 + tid] : 0.f;
        }
        __syncthreads();

        // ---- in-chunk cumulative log decay (every wave, lane t = token t) ----
        float gam = gs[lane];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(gam, d);
            if (lane >= d) gam += y;
        }
        const float gamC = __shfl(gam, 63);
        const float bet = betas[lane];

        // ---- decayed K^T: KT[dk][t] = exp(gamC - gam_t) K[t][dk] ----
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int id = tid + 256 * m;           // 512 items: 32 token pairs x 16 key groups
            const int tp = (id & 31) * 2, dg = (id >> 5) * 8;
            const float e0 = __expf(gamC - __shfl(gam, tp));
            const float e1 = __expf(gamC - __shfl(gam, tp + 1));
            const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t *>(Ks + tp * LDK + dg);
            const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t *>(Ks + (tp + 1) * LDK + dg);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __bf16 pr[2];
                pr[0] = (__bf16)((float)k0[i] * e0);
                pr[1] = (__bf16)((float)k1[i] * e1);
                *reinterpret_cast<uint32_t *>(KTs + (dg + i) * LDC + tp) = *reinterpret_cast<uint32_t *>(pr);
            }
        }

        // Per-lane row / column decay factors for this wave's 16-row block.
        float gr[4], br[4], egr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * g4 + i;
            gr[i] = __shfl(gam, r);
            br[i] = __shfl(bet, r);
            egr[i] = __expf(gr[i]);
        }

        // ---- Gram products: K K^T and Q K^T for row block w ----
        f32x4_t gk[4], gq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) { gk[j] = zero4(); gq[j] = zero4(); }
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            const bf16x8_t ak = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * w + n) * LDK + 32 * s + 8 * g4);
            const bf16x8_t aq = *reinterpret_cast<const bf16x8_t *>(Qs + (16 * w + n) * LDK + 32 * s + 8 * g4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_t bk = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * j + n) * LDK + 32 * s + 8 * g4);
                gk[j] = mma32(ak, bk, gk[j]);
                gq[j] = mma32(aq, bk, gq[j]);
            }
        }
        // Masks and decays: A (strict lower, beta-weighted), P (lower incl. diagonal).
        f32x4_t adiag = zero4(), adiagT = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cidx = 16 * j + n;
            const float gc = __shfl(gam, cidx);
            const float bc = __shfl(bet, cidx);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g4 + i;
                const float dec = (cidx <= r) ? __expf(gr[i] - gc) : 0.f;
                Ps[r * LDC + cidx] = (__bf16)(dec * gq[j][i]);
                const float a = (cidx < r) ? br[i] * dec * gk[j][i] : 0.f;
                if (j < w) As[r * LDA + cidx] = a;
                if (j == w) {
                    adiag[i] = a;
                    // transpose of the diagonal block: A[c][r] = beta_c exp(gam_c - gam_r) (k_c . k_r)
                    adiagT[i] = (r < cidx) ? bc * __expf(gc - gr[i]) * gk[j][i] : 0.f;
                }
            }
        }

        // ---- T_ww = (I + A_ww)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) ----
        // In the 16x16 accumulator layout a lane holds X[4*g4 + i][n]; that is
        // the right-hand operand layout of X and the left-hand operand layout
        // of X^T, so mma16(lay(X^T), lay(Y)) = lay(X Y).
        f32x4_t tww, twwT;
        {
            f32x4_t eye;
#pragma unroll
            for (int i = 0; i < 4; ++i) eye[i] = (4 * g4 + i == n) ? 1.f : 0.f;
            const bf16x4_t a = to_bf4(adiag), at = to_bf4(adiagT);
            const f32x4_t a2 = mma16(at, a, zero4());
            const f32x4_t a2t = mma16(a, at, zero4());
            const bf16x4_t a2b = to_bf4(a2), a2tb = to_bf4(a2t);
            const f32x4_t a4 = mma16(a2tb, a2b, zero4());
            const f32x4_t a4t = mma16(a2b, a2tb, zero4());
            const bf16x4_t a4b = to_bf4(a4), a4tb = to_bf4(a4t);
            const f32x4_t a8 = mma16(a4tb, a4b, zero4());
            const bf16x4_t x1t = to_bf4(eye - adiagT), y1 = to_bf4(eye + a2);
            const f32x4_t b1 = mma16(x1t, y1, zero4());          // (I - A)(I + A^2)
            const f32x4_t b1t = mma16(y1, x1t, zero4());         // its transpose
            const bf16x4_t b1tb = to_bf4(b1t), y2 = to_bf4(eye + a4);
            const f32x4_t b2t = mma16(y2, b1tb, zero4());        // ((I-A)(I+A^2)(I+A^4))^T
            const bf16x4_t b2tb = to_bf4(b2t), y3 = to_bf4(eye + a8);
            tww = mma16(b2tb, y3, zero4());
            twwT = mma16(y3, b2tb, zero4());
            (void)b1;
        }
        const bf16x4_t twwTb = to_bf4(twwT);
        TD[(0 * 4 + w) * 64 + lane] = tww;
#pragma unroll
        for (int i = 0; i < 4; ++i) Ts[(16 * w + 4 * g4 + i) * LDC + 16 * w + n] = (__bf16)tww[i];
        __syncthreads();

        // ---- off-diagonal blocks of T, one block diagonal per step ----
        // A-operand of A_wm: lane holds A[16w + n][16m + 4*g4 .. +3].
        auto a_op = [&](int m) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(As + (16 * w + n) * LDA + 16 * m + 4 * g4);
            return to_bf4(v);
        };
        if (w >= 1) {   // T_{w,w-1} = -T_ww A_{w,w-1} T_{w-1,w-1}
            const f32x4_t mwm = mma16(a_op(w - 1), to_bf4(TD[(0 * 4 + w - 1) * 64 + lane]), zero4());
            const f32x4_t t1 = -mma16(twwTb, to_bf4(mwm), zero4());
            TD[(1 * 4 + w) * 64 + lane] = t1;
#pragma unroll
            for (int i = 0; i < 4; ++i) Ts[(16 * w + 4 * g4 + i) * LDC + 16 * (w - 1) + n] = (__bf16)t1[i];
        }
        __syncthreads();
        if (w >= 2) {   // T_{w,w-2} = -T_ww (A_{w,w-2} T_{w-2,w-2} + A_{w,w-1} T_{w-1,w-2})
            f32x4_t mwm = mma16(a_op(w - 2), to_bf4(TD[(0 * 4 + w - 2) * 64 + lane]), zero4());
            mwm = mma16(a_op(w - 1), to_bf4(TD[(1 * 4 + w - 1) * 64 + lane]), mwm);
            const f32x4_t t2 = -mma16(twwTb, to_bf4(mwm), zero4());
            TD[(2 * 4 + w) * 64 + lane] = t2;
#pragma unroll
            for (int i = 0; i < 4; ++i) Ts[(16 * w + 4 * g4 + i) * LDC + 16 * (w - 2) + n] = (__bf16)t2[i];
        }
        __syncthreads();
        if (w == 3) {   // T_30 = -T_33 (A_30 T_00 + A_31 T_10 + A_32 T_20)
            f32x4_t mwm = mma16(a_op(0), to_bf4(TD[(0 * 4 + 0) * 64 + lane]), zero4());
            mwm = mma16(a_op(1), to_bf4(TD[(1 * 4 + 1) * 64 + lane]), mwm);
            mwm = mma16(a_op(2), to_bf4(TD[(2 * 4 + 2) * 64 + lane]), mwm);
            const f32x4_t t3 = -mma16(twwTb, to_bf4(mwm), zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) Ts[(16 * w + 4 * g4 + i) * LDC + n] = (__bf16)t3[i];
        }

        // ---- K S and Q S for row block w; X = beta (V - exp(gam) K S) ----
        f32x4_t yq[DVT / 16];
#pragma unroll
        for (int ct = 0; ct < DVT / 16; ++ct) {
            f32x4_t yk = zero4();
            yq[ct] = zero4();
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const bf16x8_t ak = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * w + n) * LDK + 32 * s + 8 * g4);
                const bf16x8_t aq = *reinterpret_cast<const bf16x8_t *>(Qs + (16 * w + n) * LDK + 32 * s + 8 * g4);
                const bf16x8_t bs = *reinterpret_cast<const bf16x8_t *>(STs + (16 * ct + n) * LDK + 32 * s + 8 * g4);
                yk = mma32(ak, bs, yk);
                yq[ct] = mma32(aq, bs, yq[ct]);
            }
            f32x4_t x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g4 + i;
                const float vv = (float)Vs[r * LDC + 16 * ct + n];
                x[i] = br[i] * (vv - egr[i] * yk[i]);
            }
            *reinterpret_cast<bf16x4_t *>(XTs + (16 * ct + n) * LDC + 16 * w + 4 * g4) = to_bf4(x);
        }
        __syncthreads();

        // ---- Vnew = T X (rows of block w need T columns < 16(w+1)) ----
        const int ksteps = w >= 2 ? 2 : 1;
#pragma unroll
        for (int ct = 0; ct < DVT / 16; ++ct) {
            f32x4_t vn = zero4();
            for (int s = 0; s < ksteps; ++s) {
                const bf16x8_t at = *reinterpret_cast<const bf16x8_t *>(Ts + (16 * w + n) * LDC + 32 * s + 8 * g4);
                const bf16x8_t bx = *reinterpret_cast<const bf16x8_t *>(XTs + (16 * ct + n) * LDC + 32 * s + 8 * g4);
                vn = mma32(at, bx, vn);
            }
            *reinterpret_cast<bf16x4_t *>(VNTs + (16 * ct + n) * LDC + 16 * w + 4 * g4) = to_bf4(vn);
        }
        __syncthreads();

        // ---- O = scale (exp(gam) Q S + P Vnew), rows of block w ----
#pragma unroll
        for (int ct = 0; ct < DVT / 16; ++ct) {
            f32x4_t o = zero4();
            for (int s = 0; s < ksteps; ++s) {
                const bf16x8_t ap = *reinterpret_cast<const bf16x8_t *>(Ps + (16 * w + n) * LDC + 32 * s + 8 * g4);
                const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(VNTs + (16 * ct + n) * LDC + 32 * s + 8 * g4);
                o = mma32(ap, bv, o);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g4 + i;
                const int t = t0 + r;
                if (t < S) {
                    const float val = r < nval ? p.scale * (egr[i] * yq[ct][i] + o[i]) : 0.f;
                    ob[(size_t)t * DV + 16 * ct + n] = from_f32<bf16_t>(val);
                }
            }
        }

        // ---- S <- exp(gamC) S + (decayed K)^T Vnew, key rows [32w, 32w+32) ----
        const float egC = __expf(gamC);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct) {
                f32x4_t acc = st[rt][ct] * egC;
#pragma unroll
                for (int s = 0; s < C / 32; ++s) {
                    const bf16x8_t ak = *reinterpret_cast<const bf16x8_t *>(KTs + (32 * w + 16 * rt + n) * LDC + 32 * s + 8 * g4);
                    const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(VNTs + (16 * ct + n) * LDC + 32 * s + 8 * g4);
                    acc = mma32(ak, bv, acc);
                }
                st[rt][ct] = acc;
            }
        write_st();
        __syncthreads();
    }

    // Final state of this tile, then zeros for every output row past the
    // last processed chunk.
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < DVT / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dk = 32 * w + 16 * rt + 4 * g4 + i;
                fb[(size_t)dk * DV + 16 * ct + n] = from_f32<bf16_t>(st[rt][ct][i]);
            }
    const int tz = nchunks * C;
    for (int id = tid; id < (S - tz) * (DVT / 8); id += 256) {
        const int row = tz + id / (DVT / 8), cv = (id % (DVT / 8)) * 8;
        *reinterpret_cast<uint4 *>(ob + (size_t)row * DV + cv) = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// float32 kernel for small heads (D <= 64): the same chunk algorithm in plain
// float32 arithmetic, one workgroup per (sequence, value head).
// ---------------------------------------------------------------------------
template <int D, int C>
__global__ __launch_bounds__(256) void chunk_f32_kernel(ChunkParams p)
{
    constexpr int LD = D + 1;
    constexpr int LC = C + 1;
    __shared__ float Kc[C * LD], Qc[C * LD], Vc[C * LD], X[C * LD], S[D * LD], A[C * LC], P[C * LC], T[C * LC];
    __shared__ float gam[C], bet[C];

    const int tid = threadIdx.x;
    const int Nk = p.Nk, Nv = p.Nv, Sl = p.S;
    const int h = blockIdx.x % Nv, b = blockIdx.x / Nv;
    const int kh = h / (Nv / Nk);
    int L = p.lens ? p.lens[b] : Sl;
    L = L < 0 ? 0 : (L > Sl ? Sl : L);
    const float *qb = static_cast<const float *>(p.q) + ((size_t)b * Nk + kh) * Sl * D;
    const float *kb = static_cast<const float *>(p.k) + ((size_t)b * Nk + kh) * Sl * D;
    const float *vb = static_cast<const float *>(p.v) + ((size_t)b * Nv + h) * Sl * D;
    const float *betab = static_cast<const float *>(p.beta) + ((size_t)b * Nv + h) * Sl;
    const float *gb = p.g ? p.g + ((size_t)b * Nv + h) * Sl : nullptr;
    float *ob = static_cast<float *>(p.out) + ((size_t)b * Nv + h) * Sl * D;
    const float *ib = p.init ? static_cast<const float *>(p.init) + ((size_t)b * Nv + h) * D * D : nullptr;
    float *fb = static_cast<float *>(p.fin) + ((size_t)b * Nv + h) * D * D;

    for (int e = tid; e < D * D; e += 256) S[(e / D) * LD + e % D] = ib ? ib[e] : 0.f;
    __syncthreads();

    const int nchunks = (L + C - 1) / C;
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C, nval = min(C, L - t0);
        for (int e = tid; e < C * D; e += 256) {
            const int r = e / D, j = e % D;
            const bool ok = r < nval;
            Kc[r * LD + j] = ok ? kb[(size_t)(t0 + r) * D + j] : 0.f;
            Qc[r * LD + j] = ok ? qb[(size_t)(t0 + r) * D + j] : 0.f;
            Vc[r * LD + j] = ok ? vb[(size_t)(t0 + r) * D + j] : 0.f;
        }
        if (tid < C) bet[tid] = tid < nval ? betab[t0 + tid] : 0.f;
        if (tid == 0) {
            float a = 0.f;
            for (int r = 0; r < C; ++r) {
                a += (gb && r < nval) ? gb[t0 + r] : 0.f;
                gam[r] = a;
            }
        }
        __syncthreads();
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, i = e % C;
            float kk = 0.f, qk = 0.f;
            for (int d = 0; d < D; ++d) {
                kk = fmaf(Kc[r * LD + d], Kc[i * LD + d], kk);
                qk = fmaf(Qc[r * LD + d], Kc[i * LD + d], qk);
            }
            const float dec = i <= r ? __expf(gam[r] - gam[i]) : 0.f;
            A[r * LC + i] = i < r ? bet[r] * dec * kk : 0.f;
            P[r * LC + i] = dec * qk;
            T[r * LC + i] = (r == i) ? 1.f : 0.f;
        }
        __syncthreads();
        // T = (I + A)^-1 by forward substitution, one row at a time.
        for (int r = 1; r < C; ++r) {
            for (int i = tid; i < r; i += 256) {
                float s = -A[r * LC + i];
                for (int m = i + 1; m < r; ++m) s = fmaf(-A[r * LC + m], T[m * LC + i], s);
                T[r * LC + i] = s;
            }
            __syncthreads();
        }
        // X = beta (V - exp(gam) K S); Q S is formed with the outputs, before
        // the state update.
        for (int e = tid; e < C * D; e += 256) {
            const int r = e / D, j = e % D;
            float ks = 0.f;
            for (int d = 0; d < D; ++d) ks = fmaf(Kc[r * LD + d], S[d * LD + j], ks);
            X[r * LD + j] = bet[r] * (Vc[r * LD + j] - __expf(gam[r]) * ks);
        }
        __syncthreads();
        // Vnew = T X (in Vc), then outputs and the state update.
        for (int e = tid; e < C * D; e += 256) {
            const int r = e / D, j = e % D;
            float s = 0.f;
            for (int i = 0; i <= r; ++i) s = fmaf(T[r * LC + i], X[i * LD + j], s);
            Vc[r * LD + j] = s;
        }
        __syncthreads();
        for (int e = tid; e < C * D; e += 256) {
            const int r = e / D, j = e % D;
            if (t0 + r >= Sl) continue;
            float qs = 0.f, pv = 0.f;
            for (int d = 0; d < D; ++d) qs = fmaf(Qc[r * LD + d], S[d * LD + j], qs);
            for (int i = 0; i <= r; ++i) pv = fmaf(P[r * LC + i], Vc[i * LD + j], pv);
            ob[(size_t)(t0 + r) * D + j] = r < nval ? p.scale * (__expf(gam[r]) * qs + pv) : 0.f;
        }
        __syncthreads();
        const float eC = __expf(gam[C - 1]);
        for (int e = tid; e < D * D; e += 256) {
            const int d = e / D, j = e % D;
            float s = S[d * LD + j] * eC;
            for (int i = 0; i < C; ++i) s = fmaf(__expf(gam[C - 1] - gam[i]) * Kc[i * LD + d], Vc[i * LD + j], s);
            S[d * LD + j] = s;
        }
        __syncthreads();
    }
    for (int e = tid; e < D * D; e += 256) fb[e] = S[(e / D) * LD + e % D];
    for (int e = nchunks * C * D + tid; e < Sl * D; e += 256) ob[e] = 0.f;
}

hipError_t launch_chunk(int dtype, int Dk, int Dv, int C, const ChunkParams &p, hipStream_t s, bool *supported)
{
    *supported = true;
    ChunkParams pc = p;
    if (dtype == 1) {
        if (Dk == mk::DK && Dv == mk::DV && C == mk::C) {
            const int units = p.B * p.Nv * mk::NT;
            const int nwg = (units + 7) / 8 * 8;
            int u = units;
            void *args[] = {&pc, &u};
            // Raise the dynamic-LDS limit once per process (first launch).
            static std::atomic<int> attr_done{0};
            if (!attr_done.load(std::memory_order_acquire)) {
                hipError_t e = hipFuncSetAttribute((const void *)chunk_mfma_kernel,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, mk::LDS_BYTES);
                if (e != hipSuccess) return e;
                attr_done.store(1, std::memory_order_release);
            }
            return hipLaunchKernel((const void *)chunk_mfma_kernel, dim3(nwg), dim3(256), args, mk::LDS_BYTES, s);
        }
        *supported = false;
        return hipSuccess;
    }
    void *args[] = {&pc};
    const dim3 grid((unsigned)(p.B * p.Nv)), block(256);
#define GDR_F32_CASE(D_, C_) \
    if (Dk == D_ && Dv == D_ && C == C_) return hipLaunchKernel((const void *)chunk_f32_kernel<D_, C_>, grid, block, args, 0, s);
    GDR_F32_CASE(16, 16) GDR_F32_CASE(16, 32) GDR_F32_CASE(16, 64)
    GDR_F32_CASE(32, 16) GDR_F32_CASE(32, 32) GDR_F32_CASE(32, 64)
    GDR_F32_CASE(64, 16) GDR_F32_CASE(64, 32)
#undef GDR_F32_CASE
    *supported = false;
    return hipSuccess;
}

}  // namespace gdr
