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
//   X      = diag(beta) (V - diag(exp(gamma)) K S0)
//   Vnew   = (I + A)^-1 X                                   what each token writes
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
//    eight wavefronts per (sequence, value head, 64-column tile of Dv); the
//    columns of S evolve independently, so each tile carries its own slice of
//    the state through all chunks in float32 MFMA accumulators. All dense
//    products run on v_mfma_f32_16x16x32_bf16 with bf16 operands staged in LDS
//    in the layout each operand needs (16-byte reads). T is never formed:
//    each 16x16 diagonal block of (I + A) is inverted as the finite product
//    (I - A)(I + A^2)(I + A^4)(I + A^8) (A is nilpotent of index 16) in
//    registers with v_mfma_f32_16x16x16_bf16 (a result's register layout is
//    directly the right-hand operand layout, and its transpose the left-hand
//    one), and (I + A) Vnew = X is solved by block forward substitution.
//  * chunk_f32_kernel — float32 I/O, small heads. The same chunk algorithm in
//    plain float32 arithmetic; T by row-wise forward substitution.
#include <atomic>

#include "gdr_common.h"

namespace gdr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
constexpr int NTHR = 512;    // 4 prep wavefronts + 4 chain wavefronts
// LDS carve-up (bytes)
constexpr int OFF_K = 0;                              // K rows          [C][LDK]   bf16
constexpr int OFF_Q = OFF_K + C * LDK * 2;            // Q rows          [C][LDK]   bf16
constexpr int OFF_KT = OFF_Q + C * LDK * 2;           // decayed K^T     [DK][LDC]  bf16
constexpr int OFF_V = OFF_KT + DK * LDC * 2;          // V tile rows     [C][LDC]   bf16
constexpr int OFF_ST = OFF_V + C * LDC * 2;           // S^T tile        [DVT][LDK] bf16
constexpr int OFF_XT = OFF_ST + DVT * LDK * 2;        // X^T; then output rows [DVT][LDC] bf16
constexpr int OFF_VNT = OFF_XT + DVT * LDC * 2;       // Vnew^T          [DVT][LDC] bf16
constexpr int OFF_P = OFF_VNT + DVT * LDC * 2;        // P rows          [C][LDC]   bf16
constexpr int OFF_A = OFF_P + C * LDC * 2;            // A rows          [C][LDA]   f32
constexpr int OFF_TD = OFF_A + C * LDA * 4;           // transposed diagonal inverse blocks [4][64] f32x4
constexpr int OFF_BG = OFF_TD + 4 * 64 * 16;          // beta, g         [2][C]     f32
constexpr int LDS_BYTES = OFF_BG + 2 * C * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
}  // namespace mk

// One chunk step, three phases separated by workgroup barriers:
//  1. prep waves (0-3): Gram products K K^T (row block w) and Q K^T (row block
//     3 - w, which balances the triangular work), the masks that turn them
//     into A and P, and the inverse T_ww of the diagonal block (I + A_ww);
//     chain waves (4-7): K S and Q S for row block w, X, and the decayed K^T.
//  2. chain wave w solves (I + A) Vnew = X for column tile w by block forward
//     substitution, Vnew_i = T_ii (X_i - sum_{j<i} A_ij Vnew_j), in registers;
//     prep waves write their share of the next chunk (loaded a whole step
//     earlier) into LDS and start the loads of the chunk after it.
//  3. chain waves: outputs, staged through LDS for 16-byte stores;
//     prep waves: the state update, held in their float32 accumulators.
// The two roles share every SIMD (wave i runs on SIMD i mod 4), so one role's
// waits overlap the other's matrix work. Every product loop reads each
// 16x32 operand fragment from LDS once and reuses it across output tiles.
__global__ __launch_bounds__(mk::NTHR) void chunk_mfma_kernel(ChunkParams p, int units)
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
    const int wv = uniform(tid >> 6);
    const bool prep = wv < 4;
    const int w = wv & 3;
    const int n = lane & 15;   // column within a 16x16 tile
    const int g4 = lane >> 4;  // 4-row group within a 16x16 tile

    int L = p.lens ? ld_const(p.lens, b) : S;
    L = L < 0 ? 0 : (L > S ? S : L);

    const bf16_t *qb = static_cast<const bf16_t *>(p.q) + ((size_t)b * Nk + kh) * S * DK;
    const bf16_t *kb = static_cast<const bf16_t *>(p.k) + ((size_t)b * Nk + kh) * S * DK;
    const bf16_t *vb = static_cast<const bf16_t *>(p.v) + ((size_t)b * Nv + h) * S * DV + col0;
    const bf16_t *betab = static_cast<const bf16_t *>(p.beta) + ((size_t)b * Nv + h) * S;
    const float *gb = p.g ? p.g + ((size_t)b * Nv + h) * S : nullptr;
    bf16_t *ob = static_cast<bf16_t *>(p.out) + ((size_t)b * Nv + h) * S * DV + col0;
    const bf16_t *ib = p.init ? static_cast<const bf16_t *>(p.init) + ((size_t)b * Nv + h) * DK * DV + col0 : nullptr;
    bf16_t *fb = static_cast<bf16_t *>(p.fin) + ((size_t)b * Nv + h) * DK * DV + col0;
    const int nchunks = (L + C - 1) / C;

    // The upper blocks of P stay zero for the whole kernel.
    for (int e = tid; e < C * LDC; e += NTHR) Ps[e] = (__bf16)0.f;

    // State slice of prep wave w: key rows [32w, 32w + 32) x the tile's DVT
    // columns as 2 x 4 accumulator tiles, st[rt][ct][i] = S[32w+16rt+4g4+i][16ct+n].
    f32x4_t st[2][DVT / 16];
    auto write_st = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct)
                *reinterpret_cast<bf16x4_t *>(STs + (16 * ct + n) * LDK + 32 * w + 16 * rt + 4 * g4) = to_bf4(st[rt][ct]);
    };
    if (prep) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int dk = 32 * w + 16 * rt + 4 * g4 + i;
                    st[rt][ct][i] = ib ? to_f32(ib[(size_t)dk * DV + 16 * ct + n]) : 0.f;
                }
        write_st();
    }

    // Chunk inputs in flight, loaded by the prep waves (256 threads): this
    // thread's 16-byte pieces of K, Q (4 each) and V (2), and one raw beta / g
    // value (converted when staged). Rows past the valid length load as zeros.
    constexpr int NPR = 256;
    u32x4_t rk[4], rq[4], rv[2];
    uint32_t rbg = 0;
    auto issue = [&](int c) __attribute__((always_inline)) {
        const int t0 = c * C, nv = min(C, L - t0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int id = tid + NPR * m;             // 1024 pieces: 64 rows x 16
            const int row = id >> 4, cv = (id & 15) * 8;
            rk[m] = u32x4_t{0u, 0u, 0u, 0u};
            rq[m] = u32x4_t{0u, 0u, 0u, 0u};
            if (row < nv) {
                rk[m] = *reinterpret_cast<const u32x4_t *>(kb + (size_t)(t0 + row) * DK + cv);
                rq[m] = *reinterpret_cast<const u32x4_t *>(qb + (size_t)(t0 + row) * DK + cv);
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int id = tid + NPR * m;             // 512 pieces: 64 rows x 8
            const int row = id >> 3, cv = (id & 7) * 8;
            rv[m] = u32x4_t{0u, 0u, 0u, 0u};
            if (row < nv) rv[m] = *reinterpret_cast<const u32x4_t *>(vb + (size_t)(t0 + row) * DV + cv);
        }
        rbg = 0;
        if (tid < C) {
            if (tid < nv) rbg = betab[t0 + tid];
        } else if (tid < 2 * C) {
            if (gb && tid - C < nv) rbg = reinterpret_cast<const uint32_t *>(gb)[t0 + tid - C];
        }
    };
    auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int id = tid + NPR * m;
            const int row = id >> 4, cv = (id & 15) * 8;
            *reinterpret_cast<u32x4_t *>(Ks + row * LDK + cv) = rk[m];
            *reinterpret_cast<u32x4_t *>(Qs + row * LDK + cv) = rq[m];
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int id = tid + NPR * m;
            *reinterpret_cast<u32x4_t *>(Vs + (id >> 3) * LDC + (id & 7) * 8) = rv[m];
        }
        if (tid < C) betas[tid] = __uint_as_float(rbg << 16);         // bf16 -> f32
        else if (tid < 2 * C) betas[tid] = __uint_as_float(rbg);      // betas[C + t] is g[t]
    };

    if (prep && nchunks > 0) {
        issue(0);
        stage();
        if (nchunks > 1) issue(1);
    }
    __syncthreads();

    // The two roles run separate loops with the same three barriers per
    // chunk (barriers count waves, so they meet); this keeps each role's
    // registers to its own.
    if (prep) {
        for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int nval = min(C, L - t0);

        // ---- in-chunk cumulative log decay (every wave, lane t = token t) ----
        float gam = gs[lane];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(gam, d);
            if (lane >= d) gam += y;
        }
        const float gamC = __shfl(gam, 63);
        const float bet = betas[lane];

            {
            // Gram K K^T for row block w (tiles j <= w) and Q K^T for row block
            // wq = 3 - w (tiles j <= wq); both use the K rows of block j as the
            // right-hand operand, read once per k-step.
            const int wq = 3 - w;
            f32x4_t gk[4], gq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) { gk[j] = zero4(); gq[j] = zero4(); }
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const bf16x8_t ak = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * w + n) * LDK + 32 * s + 8 * g4);
                const bf16x8_t aq = *reinterpret_cast<const bf16x8_t *>(Qs + (16 * wq + n) * LDK + 32 * s + 8 * g4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j > w && j > wq) continue;
                    const bf16x8_t bk = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * j + n) * LDK + 32 * s + 8 * g4);
                    if (j <= w) gk[j] = mma32(ak, bk, gk[j]);
                    if (j <= wq) gq[j] = mma32(aq, bk, gq[j]);
                }
            }
            float gr[4], br[4], gqr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gr[i] = __shfl(gam, 16 * w + 4 * g4 + i);
                br[i] = __shfl(bet, 16 * w + 4 * g4 + i);
                gqr[i] = __shfl(gam, 16 * wq + 4 * g4 + i);
            }
            f32x4_t adiag = zero4(), adiagT = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cidx = 16 * j + n;
                const float gc = __shfl(gam, cidx);
                const float bc = __shfl(bet, cidx);
                if (j <= w) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * w + 4 * g4 + i;
                        const float a = (cidx < r) ? br[i] * __expf(gr[i] - gc) * gk[j][i] : 0.f;
                        if (j < w) As[r * LDA + cidx] = a;
                        else {
                            adiag[i] = a;
                            // transpose of the diagonal block: A[c][r] = beta_c exp(gam_c - gam_r) (k_c . k_r)
                            adiagT[i] = (r < cidx) ? bc * __expf(gc - gr[i]) * gk[j][i] : 0.f;
                        }
                    }
                }
                if (j <= wq) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * wq + 4 * g4 + i;
                        Ps[r * LDC + cidx] = (__bf16)((cidx <= r) ? __expf(gqr[i] - gc) * gq[j][i] : 0.f);
                    }
                }
            }
            // T_ww = (I + A_ww)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8). In the
            // 16x16 accumulator layout a lane holds X[4*g4 + i][n]; that is the
            // right-hand operand layout of X and the left-hand operand layout of
            // X^T, so mma16(lay(X^T), lay(Y)) = lay(X Y). The substitution needs
            // T_ww as a left-hand operand, i.e. lay(T_ww^T).
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
            const f32x4_t b1t = mma16(y1, x1t, zero4());         // ((I - A)(I + A^2))^T
            const bf16x4_t b1tb = to_bf4(b1t), y2 = to_bf4(eye + a4);
            const f32x4_t b2t = mma16(y2, b1tb, zero4());        // ((I-A)(I+A^2)(I+A^4))^T
            const bf16x4_t b2tb = to_bf4(b2t), y3 = to_bf4(eye + a8);
            TD[w * 64 + lane] = mma16(y3, b2tb, zero4());        // lay(T_ww^T)
            }
            __syncthreads();
            {
            if (c + 1 < nchunks) stage();
            if (c + 2 < nchunks) issue(c + 2);
            }
            __syncthreads();
            {
            // S <- exp(gamC) S + (decayed K)^T Vnew, key rows [32w, 32w+32).
            const float egC = __expf(gamC);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < DVT / 16; ++ct) st[rt][ct] *= egC;
#pragma unroll
            for (int s = 0; s < C / 32; ++s) {
                bf16x8_t ak[2], bv[DVT / 16];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    ak[rt] = *reinterpret_cast<const bf16x8_t *>(KTs + (32 * w + 16 * rt + n) * LDC + 32 * s + 8 * g4);
#pragma unroll
                for (int ct = 0; ct < DVT / 16; ++ct)
                    bv[ct] = *reinterpret_cast<const bf16x8_t *>(VNTs + (16 * ct + n) * LDC + 32 * s + 8 * g4);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ct = 0; ct < DVT / 16; ++ct) st[rt][ct] = mma32(ak[rt], bv[ct], st[rt][ct]);
            }
            write_st();
            }
            __syncthreads();
        }
    } else {
        f32x4_t yq[DVT / 16];   // exp(gam) Q S for the output
        for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C;
        const int nval = min(C, L - t0);

        // ---- in-chunk cumulative log decay (every wave, lane t = token t) ----
        float gam = gs[lane];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(gam, d);
            if (lane >= d) gam += y;
        }
        const float gamC = __shfl(gam, 63);
        const float bet = betas[lane];

            {
            // K S and Q S for row block w; X = beta (V - exp(gam) K S).
            float brr[4], egr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * g4 + i;
                brr[i] = __shfl(bet, r);
                egr[i] = __expf(__shfl(gam, r));
            }
            f32x4_t yk[DVT / 16];
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct) { yk[ct] = zero4(); yq[ct] = zero4(); }
#pragma unroll
            for (int s = 0; s < DK / 32; ++s) {
                const bf16x8_t ak = *reinterpret_cast<const bf16x8_t *>(Ks + (16 * w + n) * LDK + 32 * s + 8 * g4);
                const bf16x8_t aq = *reinterpret_cast<const bf16x8_t *>(Qs + (16 * w + n) * LDK + 32 * s + 8 * g4);
#pragma unroll
                for (int ct = 0; ct < DVT / 16; ++ct) {
                    const bf16x8_t bs = *reinterpret_cast<const bf16x8_t *>(STs + (16 * ct + n) * LDK + 32 * s + 8 * g4);
                    yk[ct] = mma32(ak, bs, yk[ct]);
                    yq[ct] = mma32(aq, bs, yq[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct) {
                f32x4_t x;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * w + 4 * g4 + i;
                    const float vv = (float)Vs[r * LDC + 16 * ct + n];
                    x[i] = brr[i] * (vv - egr[i] * yk[ct][i]);
                    yq[ct][i] *= egr[i];
                }
                *reinterpret_cast<bf16x4_t *>(XTs + (16 * ct + n) * LDC + 16 * w + 4 * g4) = to_bf4(x);
            }
            // decayed K^T: KT[dk][t] = exp(gamC - gam_t) K[t][dk] (256 chain threads, 512 items)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int id = (tid - 256) + 256 * m;   // 32 token pairs x 16 key groups
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
            }
            __syncthreads();
            {
            // (I + A) Vnew = X for column tile ct = w, row block by row block:
            // Vnew_i = T_ii (X_i - sum_{j<i} A_ij Vnew_j). Left-hand operand
            // of -A_ij: lane holds -A[16i + n][16j + 4*g4 .. +3].
            const int ct = w;
            auto naop = [&](int i, int j) __attribute__((always_inline)) {
                return to_bf4(-*reinterpret_cast<const f32x4_t *>(As + (16 * i + n) * LDA + 16 * j + 4 * g4));
            };
            bf16x4_t vnb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x4_t xb = *reinterpret_cast<const bf16x4_t *>(XTs + (16 * ct + n) * LDC + 16 * i + 4 * g4);
                f32x4_t acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = (float)xb[e];
#pragma unroll
                for (int j = 0; j < i; ++j) acc = mma16(naop(i, j), vnb[j], acc);
                const f32x4_t vn = mma16(to_bf4(TD[i * 64 + lane]), to_bf4(acc), zero4());
                vnb[i] = to_bf4(vn);
                *reinterpret_cast<bf16x4_t *>(VNTs + (16 * ct + n) * LDC + 16 * i + 4 * g4) = vnb[i];
            }
            }
            __syncthreads();
            {
            // O = scale (exp(gam) Q S + P Vnew) for row block w, staged through
            // this wave's part of the X^T buffer as rows, then stored 16 bytes
            // at a time.
            const int ks = w >= 2 ? 2 : 1;
            f32x4_t o[DVT / 16];
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct) o[ct] = yq[ct];
            for (int s = 0; s < ks; ++s) {
                const bf16x8_t ap = *reinterpret_cast<const bf16x8_t *>(Ps + (16 * w + n) * LDC + 32 * s + 8 * g4);
#pragma unroll
                for (int ct = 0; ct < DVT / 16; ++ct) {
                    const bf16x8_t bv = *reinterpret_cast<const bf16x8_t *>(VNTs + (16 * ct + n) * LDC + 32 * s + 8 * g4);
                    o[ct] = mma32(ap, bv, o[ct]);
                }
            }
            __bf16 *Os = XTs;   // rows [16w, 16w + 16) of a [C][LDC] row-major view
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * w + 4 * g4 + i;
                    Os[r * LDC + 16 * ct + n] = (__bf16)(r < nval ? p.scale * o[ct][i] : 0.f);
                }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int id = lane + 64 * m;             // 16 rows x 8 pieces
                const int r = 16 * w + (id >> 3), cv = (id & 7) * 8;
                if (t0 + r < S)
                    *reinterpret_cast<uint4 *>(ob + (size_t)(t0 + r) * DV + cv) =
                        *reinterpret_cast<const uint4 *>(Os + r * LDC + cv);
            }
            }
            __syncthreads();
        }
    }

    // Final state of this tile, then zeros for every output row past the
    // last processed chunk.
    if (prep) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < DVT / 16; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int dk = 32 * w + 16 * rt + 4 * g4 + i;
                    fb[(size_t)dk * DV + 16 * ct + n] = from_f32<bf16_t>(st[rt][ct][i]);
                }
    }
    const int tz = nchunks * C;
    for (int id = tid; id < (S - tz) * (DVT / 8); id += NTHR) {
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
            return hipLaunchKernel((const void *)chunk_mfma_kernel, dim3(nwg), dim3(mk::NTHR), args, mk::LDS_BYTES, s);
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
