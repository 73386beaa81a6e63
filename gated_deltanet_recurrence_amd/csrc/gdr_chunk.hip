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
// Kernels:
//  * chunk_t_kernel + chunk_mfma_kernel — bf16 or fp16 I/O, Dk = Dv = 128, C = 64.
//    chunk_t_kernel forms T = (I + A)^-1 of every chunk of every sequence in
//    parallel (it depends on k, beta and g only) into the caller's workspace,
//    and writes the output rows of chunks wholly past a sequence's length as
//    zeros; chunk_mfma_kernel then makes one pass over the chunks per
//    (sequence, value head, half or whole of Dv), carrying its slice of the
//    state in float32 matrix-core accumulators. All dense products run on
//    v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x16_f16 for fp16 I/O) with
//    operands in the I/O format.
//  * chunk_f32_kernel — float32 I/O, small heads. The same chunk algorithm in
//    plain float32 arithmetic; T by row-wise forward substitution.
#include <atomic>
#include <type_traits>

#include "gdr_common.h"

namespace gdr {

// Eight 16-bit elements, the operand of one MFMA k-step: bf16, or fp16 bit
// patterns (reinterpreted where the fp16 MFMA takes them).
typedef __bf16 e16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_bf16. Lane l (h = l / 32) supplies row l % 32 of the
// left operand and column l % 32 of the right one, each as 8 consecutive
// k-values starting at 8h; the result gives lane l column l % 32, register q
// holding row 8(q / 4) + 4h + q % 4.
// v_mfma_f32_32x32x16_f16 has the same shape and lane layout.
template <typename EL> __device__ __forceinline__ f32x16_t mfma32(e16x8_t a, e16x8_t b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mfma32<BF16>(e16x8_t a, e16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mfma32<F16>(e16x8_t a, e16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t zero16()
{
    f32x16_t z;
#pragma unroll
    for (int q = 0; q < 16; ++q) z[q] = 0.f;
    return z;
}
// Row of result register q for a lane in half hh of the wave.
__device__ __forceinline__ int drow(int q, int hh) { return 8 * (q >> 2) + 4 * hh + (q & 3); }

// Registers 8s..8s+7 of a 32x32 result D(X), rounded to bf16, are the
// operand of k-step s when the contraction runs over the rows of X: the right
// operand of X and the left operand of X^T. This fixes the order in which a
// k-step visits its 16 contraction indices: storage slot 8h + e holds index
// 4h + e % 4 + 8(e / 4), i.e. bits 2 and 3 of the index are swapped ("k-order").
// Every operand tile in LDS is kept in k-order along its contraction axis, so
// each lane reads or writes one 16-byte piece per k-step.
template <typename EL>
__device__ __forceinline__ e16x8_t op8(const f32x16_t &d, int s)
{
    const u32x4_t w = {EL::pack(d[8 * s], d[8 * s + 1]), EL::pack(d[8 * s + 2], d[8 * s + 3]),
                       EL::pack(d[8 * s + 4], d[8 * s + 5]), EL::pack(d[8 * s + 6], d[8 * s + 7])};
    return __builtin_bit_cast(e16x8_t, w);
}
// Eight floats narrowed into one operand.
template <typename EL>
__device__ __forceinline__ e16x8_t pack8(const float (&x)[8])
{
    const u32x4_t w = {EL::pack(x[0], x[1]), EL::pack(x[2], x[3]), EL::pack(x[4], x[5]), EL::pack(x[6], x[7])};
    return __builtin_bit_cast(e16x8_t, w);
}
// D(X Y) + c over a 32-long contraction, from D(X^T) and D(Y).
template <typename EL>
__device__ __forceinline__ f32x16_t prod(const f32x16_t &dxt, const f32x16_t &dy, f32x16_t c)
{
    c = mfma32<EL>(op8<EL>(dxt, 0), op8<EL>(dy, 0), c);
    return mfma32<EL>(op8<EL>(dxt, 1), op8<EL>(dy, 1), c);
}

// Byte offset of 16-byte piece u of row r in a tile of 256- or 128-byte rows.
// The XOR swizzle spreads the 16 rows read by a half-wave over all 16 bank
// groups, so operand reads and result writes are free of bank conflicts.
__device__ __forceinline__ int sw256(int r, int u) { return (r << 8) + ((u ^ (r & 15)) << 4); }
__device__ __forceinline__ int sw128(int r, int u) { return (r << 7) + ((u ^ ((r >> 1) & 7)) << 4); }
// Swizzles of the tiles that are also read transposed (ldT below), whose
// reads touch 4 consecutive rows x 4 consecutive pieces: consecutive rows
// are sent to different 64-byte bank groups, while any 16 consecutive rows
// (256-byte rows) still fall on 16 different piece positions.
__device__ __forceinline__ int sw256t(int r, int u) { return (r << 8) + ((u ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4); }
__device__ __forceinline__ int sw128t(int r, int u) { return (r << 7) + ((u ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))) << 4); }

__device__ __forceinline__ e16x8_t ld8(const unsigned char *base, int off)
{
    return *reinterpret_cast<const e16x8_t *>(base + off);
}
__device__ __forceinline__ void st8(unsigned char *base, int off, e16x8_t v)
{
    *reinterpret_cast<e16x8_t *>(base + off) = v;
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t *lds_i16x4_ptr;

// Operand of k-step ks for a product that contracts over the ROWS of a
// row-major bf16 tile kept with k-order column pieces (row pitch 256 or 128
// bytes, swizzled by sw256t / sw128t): lane l takes column 32cb + (l & 31) and
// rows 16ks + 4(l >> 5) + {0..3, 8..11} (k-order), i.e. the left operand of
// the tile's transpose or its right operand. Two LDS transpose reads
// (ds_read_b64_tr_b16): inside each 16-lane group, result lane i gets element
// i % 4 of the 4 elements named by source lanes 4j + i / 4 (j = 0..3), so
// source lane m names row T(m / 4) and columns c + 4(m % 4) .. + 3.
template <int PITCH>
__device__ __forceinline__ e16x8_t ldT(const unsigned char *base, int cb, int ks, int lane)
{
    const int g = lane >> 4, m = lane & 15;
    const int row = 16 * ks + 4 * (g >> 1) + (m >> 2);
    const int c0 = 32 * cb + 16 * (g & 1) + 4 * (m & 3);
    const int piece = 2 * (c0 >> 4) + ((c0 >> 2) & 1);
    const int half = 8 * ((c0 >> 3) & 1);
    const int o1 = (PITCH == 256 ? sw256t(row, piece) : sw128t(row, piece)) + half;
    const int o2 = (PITCH == 256 ? sw256t(row + 8, piece) : sw128t(row + 8, piece)) + half;
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(base + o1));
    const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(base + o2));
    return __builtin_bit_cast(e16x8_t, i16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
}

// Left operand n (0-5) of a product with T diag(fac), from a chunk's T kept as
// chunk_t_kernel writes it (block j, k-step s in result-register order). The
// nonzero (row block, token k-step) pairs of T are n = (0,0), (0,1), (1,0),
// (1,1), (1,2), (1,3), held as (j, s) = (0,0), (0,1), (2,0), (2,1), (1,0),
// (1,1) (j: 0 = T_00, 1 = T_11, 2 = T_10); the lane's elements e are tokens
// 16 k2 + 4hh + (e & 3) + 8(e >> 2).
__device__ __forceinline__ int t_operand_offset(int n, int lane)
{
    const int j = n < 2 ? 0 : (n < 4 ? 2 : 1), s = n & 1;
    return ((2 * j + s) * 64 + lane) * 16;
}
// NEG: the operand of -T diag(fac), the sign taken by the multiply.
template <typename EL, bool NEG = false>
__device__ __forceinline__ e16x8_t t_operand(const unsigned char *tbase, int n, const float *fac, int lane)
{
    const int k2 = n < 2 ? n : n - 2;
    const u32x4_t t4 = *reinterpret_cast<const u32x4_t *>(tbase + t_operand_offset(n, lane));
    const int i0 = 16 * k2 + 4 * (lane >> 5);
    const float4 f0 = *reinterpret_cast<const float4 *>(fac + i0), f1 = *reinterpret_cast<const float4 *>(fac + i0 + 8);
    const float fe[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    const uint32_t w4[4] = {t4.x, t4.y, t4.z, t4.w};
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = ((e & 1) ? EL::hi(w4[e >> 1]) : EL::lo(w4[e >> 1])) * (NEG ? -fe[e] : fe[e]);
    return pack8<EL>(r);
}

namespace mk {
constexpr int C = 64;          // chunk length
constexpr int DK = 128;        // key head size
constexpr int DV = 128;        // value head size
constexpr int NTHR = 512;      // 8 wavefronts: prep waves, then chain waves
// Operand set of one chunk (double-buffered: the chain consumes chunk c while
// the prep waves build chunk c + 1). Byte offsets within a set:
constexpr int S_Q = 0;         // Q rows, features in k-order             [64][256 B]
constexpr int S_KT = 16384;    // K rows, features in k-order             [64][256 B] (read transposed)
constexpr int S_W = 32768;     // -W rows, features in k-order            [64][256 B]
constexpr int S_P = 49152;     // P rows, tokens in k-order               [64][128 B]
constexpr int S_VT = 57344;    // V rows (NT = 1: diag(beta) V), columns in k-order [64][2 DVT B] (read transposed)
// The rest depends on NT, the column tiles per head.
template <int NT> struct Tile {
    static constexpr int DVT = DV / NT;          // value columns per workgroup
    static constexpr int NCHAIN = DVT / 32;      // chain wavefronts, 32 state columns each
    static constexpr int NPREP = 8 - NCHAIN;     // wavefronts building the chunk operands
    static constexpr int S_T = S_VT + 64 * 2 * DVT;          // T as chunk_t_kernel wrote it [6][64][16 B]
    static constexpr int S_TB = S_T + 6144;                  // NT = 2: T diag(beta), same order
    static constexpr int S_VEC = NT == 2 ? S_TB + 6144 : S_T + 6144;
    // S_VEC: scale exp(gamma_t) (0 past the length) [64], exp(gamma_C - gamma_t) [64], exp(gamma_C)
    static constexpr int SET_BYTES = S_VEC + 1024;
    // Prep-only buffers.
    static constexpr int P_BG = 2 * SET_BYTES;  // beta, gamma log2(e), beta exp(gamma) [3][64] of the chunk being built
    static constexpr int P_FLAG = P_BG + 768;   // arrival counters of the prep waves
    static constexpr int LDS_BYTES = P_FLAG + 64;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace mk

// Synchronisation inside the workgroup orders LDS only. Waves never pass
// data through global memory, so a barrier or counter must not wait for the
// prefetch loads or output stores in flight (a workgroup-scope fence would).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the totals of rows 0 and 0-1 carried into later rows.
__device__ __forceinline__ float wave_prefix_sum(float x)
{
    x += dpp_f<0x111, 0xf>(x);   // row_shr:1
    x += dpp_f<0x112, 0xf>(x);   // row_shr:2
    x += dpp_f<0x114, 0xf>(x);   // row_shr:4
    x += dpp_f<0x118, 0xf>(x);   // row_shr:8
    x += dpp_f<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_f<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// In-kernel q/k normalisation of rows that lie in consecutive lanes, each lane
// holding `n` bf16 elements of the row (8 lanes x 16 or 16 lanes x 8): the
// sum of squares over the row's lanes, then x / sqrt(sum + eps), back to bf16.
template <int LANES>
__device__ __forceinline__ float row_lanes_sum(float x)
{
    static_assert(LANES == 8 || LANES == 16, "row width");
    x += dpp_f<0xB1, 0xf>(x);    // quad_perm [1,0,3,2]
    x += dpp_f<0x4E, 0xf>(x);    // quad_perm [2,3,0,1]
    x += dpp_f<0x141, 0xf>(x);   // row_half_mirror: the 8-lane half
    if constexpr (LANES == 16) x += dpp_f<0x140, 0xf>(x);   // row_mirror: the other half
    return x;
}
template <typename EL, int LANES, int W>
__device__ __forceinline__ void normalise_row(u32x4_t (&x)[W])
{
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const uint32_t a[4] = {x[w].x, x[w].y, x[w].z, x[w].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss = fmaf(EL::lo(a[e]), EL::lo(a[e]), ss);
            ss = fmaf(EL::hi(a[e]), EL::hi(a[e]), ss);
        }
    }
    const float r = qk_rnorm(row_lanes_sum<LANES>(ss));
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const uint32_t a[4] = {x[w].x, x[w].y, x[w].z, x[w].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = EL::pack(EL::lo(a[e]) * r, EL::hi(a[e]) * r);
        x[w] = u32x4_t{o[0], o[1], o[2], o[3]};
    }
}

// 16 consecutive elements (pieces a, b) into k-order: slots 0-3 and 12-15
// stay, slots 4-7 take elements 8-11, slots 8-11 elements 4-7.
__device__ __forceinline__ u32x4_t korder_lo(u32x4_t a, u32x4_t b) { return u32x4_t{a.x, a.y, b.x, b.y}; }
__device__ __forceinline__ u32x4_t korder_hi(u32x4_t a, u32x4_t b) { return u32x4_t{a.z, a.w, b.z, b.w}; }

// Arrival counters (LDS) that order the prep waves among themselves without
// holding up the chain waves. Counters only grow; a wave waits for the count
// that the current chunk's arrivals reach. LDS operations of one wave complete
// in order, so a wave's writes are visible once its increment is.
__device__ __forceinline__ void arrive(uint32_t *f, int lane)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(f, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_for(uint32_t *f, uint32_t target)
{
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}

// T = (I + A)^-1 of every chunk, ahead of the pass over the chunks: T depends
// on k, beta and g of its chunk only, never on the state, so all chunks of
// all sequences are independent. One wavefront per (sequence, value head,
// chunk), with no exchange between wavefronts.
//
// The solve is blocked forward substitution, which stays accurate however
// close the keys of a chunk are to one another (repeated tokens give equal
// keys); T itself is bounded there, but series forms of the inverse are not.
//   1. Gram blocks G_00, G_11 (K_d K_d^T) and G_10 (K_1 K_0^T) on the matrix
//      cores; A = strict_lower(diag(beta) K K^T * exp(gamma_r - gamma_i)).
//   2. The four 16x16 diagonal blocks D_B = (I + A_BB)^-1 by forward
//      substitution in float32, all four at once, one per 16-lane row of the
//      wave: lane r of row B holds row r of A_BB and of D_B. Step m
//      broadcasts row m of D_B (final by then) across the row and subtracts
//      A[r, m] times it from every row r; rows r <= m have A[r, m] = 0.
//   3. Two block merges. For a lower triangular matrix of two diagonal
//      blocks with inverses D_0, D_1 and off-diagonal block A_10, the inverse
//      has T_10 = -D_1 A_10 D_0 (block forward substitution), exactly. First
//      inside each 32-block (16x16 blocks), then over the whole chunk:
//      T_10 = -T_11 A_10 T_00 (32x32 blocks), on the matrix cores.
// T is stored in result-register order, so that every store is 1 KB
// contiguous: per chunk, block j (0: T_00, 1: T_11, 2: T_10) and k-step s hold
// op8 of D(T_j^T): row r = c32 of the block holds columns (k-order piece
// 2s + hh) at ((2j + s) * 64 + lane) * 16 bytes, 6 KB per chunk. The block
// T_01 = 0 is neither written nor read.
namespace tk {
constexpr int WAVES = 4;                  // independent wavefronts per workgroup
constexpr int CHUNK_ELEMS = 3 * 32 * 32;  // workspace elements per chunk: T_00, T_11, T_10 (T_01 = 0)
}  // namespace tk

// Value of lane m of the caller's 16-lane row, in every lane of the row
// (DPP row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + M, 0xf, 0xf, true));
}
// Steps M..14 of the forward substitution: x holds the lane's row of the
// block's inverse, na the negated row of its strictly lower A.
template <int M>
__device__ __forceinline__ void fsub16(float (&x)[16], const float (&na)[16])
{
    if constexpr (M < 15) {
#pragma unroll
        for (int j = 0; j <= M; ++j) x[j] = fmaf(na[M], row_bcast<M>(x[j]), x[j]);
        fsub16<M + 1>(x, na);
    }
}

template <typename EL>
__global__ __launch_bounds__(64 * tk::WAVES) __attribute__((amdgpu_waves_per_eu(3, 3))) void chunk_t_kernel(ChunkParams p, int nchk, int units)
{
    using namespace mk;
    // A few floats per wave: beta and gamma log2(e) of the chunk's tokens; and
    // per wave one 32-row half of the chunk's K, passed through LDS so that
    // the loads read whole rows.
    __shared__ __align__(16) float bgs[tk::WAVES][128];
    __shared__ __align__(16) unsigned char kst[tk::WAVES][32 * 256];
    const int Nk = p.Nk, Nv = p.Nv, S = p.S;
    const int rep = Nv / Nk;
    const int lane = threadIdx.x & 63, wl = uniform(threadIdx.x >> 6);
    const int hh = lane >> 5, c32 = lane & 31;
    // Unit order: value heads of one key head, then chunks, then (b, key
    // head): the waves of a workgroup share k through the cache.
    const int u = blockIdx.x * tk::WAVES + wl;
    if (u >= units) return;
    const int hr = u % rep;
    const int c = (u / rep) % nchk;
    const int bk = u / (rep * nchk);
    const int kh = bk % Nk, b = bk / Nk;
    const int h = kh * rep + hr;
    int L = p.lens ? ld_const(p.lens, b) : S;
    L = L < 0 ? 0 : (L > S ? S : L);
    const int t0 = c * C;
    if (t0 >= L) {
        // A chunk wholly past the length has no T. Its output rows are
        // padding, written here as zeros (the pass over the chunks writes the
        // rows of the chunks it processes): 64 rows of 256 bytes, rows past S
        // dropped by the buffer bound.
        const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<uint16_t *>(p.out) + ((size_t)b * Nv + h) * S * DV, (short)0, S * DV * 2, 0x00020000);
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int id = 64 * i + lane;
            __builtin_amdgcn_raw_buffer_store_b128(z, ors, ((t0 + (id >> 4)) * DV + 8 * (id & 15)) * 2, 0, 0);
        }
        return;
    }

    // K operands: row 32d + c32 of the chunk; k-step ks takes features
    // 16ks + 8hh .. + 7. The Gram blocks contract over the features, so any
    // order serves as long as both operands share it. Rows past L read as zeros.
    // The chunk's 16 KB are read as 16 whole-row loads (1 KB, 4 rows each) and
    // turned into operands through this wave's LDS half tile, one half at a
    // time (a wave's LDS accesses complete in order, so no barrier is needed).
    const uint16_t *kb = static_cast<const uint16_t *>(p.k) + ((size_t)b * Nk + kh) * S * DK;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, L * DK * 2, 0x00020000);
    u32x4_t kr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, t0 * DK * 2 + i * 1024 + lane * 16, 0, 0);
    if (p.qk_norm) {
        // Each load holds 4 whole rows, 16 lanes per row.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            u32x4_t one[1] = {kr[i]};
            normalise_row<EL, 16>(one);
            kr[i] = one[0];
        }
    }
    e16x8_t kf[2][8];
    unsigned char *kt = kst[wl];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4_t *>(kt + sw256(4 * i + (lane >> 4), lane & 15)) = kr[8 * d + i];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kf[d][ks] = ld8(kt, sw256(c32, 2 * ks + hh));
    }
    // beta and the in-chunk cumulative log decay (lane t = token t0 + t).
    {
        const size_t vh = (size_t)b * Nv + h;
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(static_cast<const uint16_t *>(p.beta) + vh * S), (short)0, L * 2, 0x00020000);
        // g, or with fused gates the raw input a (16-bit).
        const bool fg = p.gate_a != nullptr;
        const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
            fg ? (void *)(static_cast<const uint16_t *>(p.gate_a) + vh * S) : (void *)(p.g ? p.g + vh * S : nullptr),
            (short)0, fg ? L * 2 : (p.g ? L * 4 : 0), 0x00020000);
        const uint32_t rb = __builtin_amdgcn_raw_buffer_load_b16(brs, (t0 + lane) * 2, 0, 0);
        const uint32_t rg = fg ? __builtin_amdgcn_raw_buffer_load_b16(grs, (t0 + lane) * 2, 0, 0)
                               : __builtin_amdgcn_raw_buffer_load_b32(grs, (t0 + lane) * 4, 0, 0);
        float beta = EL::to(rb), g = __uint_as_float(rg);
        if (fg) {
            // Tokens past the length are identity steps: beta = g = 0.
            const bool valid = t0 + lane < L;
            beta = valid ? gate_sigmoid(beta) : 0.f;
            g = valid ? gate_g(EL::to(rg), p.A_log[h], p.dt_bias[h]) : 0.f;
        }
        bgs[wl][lane] = beta;
        bgs[wl][64 + lane] = wave_prefix_sum(g) * 1.44269504088896340736f;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's own writes, read below
    }
    const float *bg = bgs[wl], *gv = bgs[wl] + 64;
    // beta / gamma of the rows a lane holds in a result tile: rows 8m + 4hh + i
    // of the 32-row block starting at r0.
    auto rows4 = [&](const float *v, int r0, float *o) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 x = *reinterpret_cast<const float4 *>(v + r0 + 8 * m + 4 * hh);
            o[4 * m] = x.x; o[4 * m + 1] = x.y; o[4 * m + 2] = x.z; o[4 * m + 3] = x.w;
        }
    };

    f32x16_t G0 = zero16(), G1 = zero16(), G10 = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        G0 = mfma32<EL>(kf[0][ks], kf[0][ks], G0);
        G1 = mfma32<EL>(kf[1][ks], kf[1][ks], G1);
        G10 = mfma32<EL>(kf[1][ks], kf[0][ks], G10);
    }

    // Off-diagonal 16x16 block of each 32-block d (its rows 16-31 against
    // columns 0-15) as the left operand of k-step 1: registers 8-15 of D(A_dd)
    // in the lanes of columns 0-15, zero elsewhere.
    e16x8_t aoff[2];
    {
        float br[16], gr[16];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            rows4(bg, 32 * d, br);
            rows4(gv, 32 * d, gr);
            const float gc = gv[32 * d + c32];
            const f32x16_t &G = d ? G1 : G0;
            // -inf as the exponent, not a select of the product: the select
            // compiles to one branch per element, each with its own wait.
            float a8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a8[e] = br[8 + e] * __builtin_amdgcn_exp2f(c32 < 16 ? gr[8 + e] - gc : -INFINITY) * G[8 + e];
            aoff[d] = pack8<EL>(a8);
        }
    }

    // Rows of the 16x16 diagonal blocks, one per lane: after the swap, lane
    // 32d + c holds row c of G_dd (symmetric), its columns drow(q, 0) in x0
    // and drow(q, 1) in x1. Lane l is row r = l % 16 of block B = l / 16.
    const int B = lane >> 4, r = lane & 15, sb = B & 1;
    float x[16];
    {
        float na[16];
        float x0[16], x1[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(G0[q]), __float_as_uint(G1[q]), false, false);
            x0[q] = __uint_as_float(s[0]);
            x1[q] = __uint_as_float(s[1]);
        }
        // Column j of the block is column 16 sb + j of the 32-block: register
        // 8 sb + 4 (j / 8) + j % 4 of x0 (j % 8 < 4) or x1.
        const float brow = bg[16 * B + r], grow = gv[16 * B + r];
        float gcol[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gv + 16 * B + 4 * m);
            gcol[4 * m] = g4.x; gcol[4 * m + 1] = g4.y; gcol[4 * m + 2] = g4.z; gcol[4 * m + 3] = g4.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            // A select of values, not of arrays: a runtime choice between x0
            // and x1 keeps them out of registers (the compiler then places
            // them in LDS, 32 KB per workgroup, which also halves occupancy).
            const int qa = 4 * (j >> 3) + (j & 3);
            const float lo = ((j >> 2) & 1) ? x1[qa] : x0[qa];
            const float hi = ((j >> 2) & 1) ? x1[8 + qa] : x0[8 + qa];
            const float gjr = sb ? hi : lo;
            // Exponent selected before exp2: past the diagonal it could overflow.
            const float ex = __builtin_amdgcn_exp2f(j < r ? grow - gcol[j] : -INFINITY);
            na[j] = -(brow * ex * gjr);
            x[j] = j == r ? 1.f : 0.f;
        }
        fsub16<0>(x, na);
    }
    // D(D_dd^T) for the 32-block d (block diagonal of the two 16x16
    // inverses): lane (hh, c32) holds row c32 at columns drow(q, hh). Each
    // lane forms the hh = 0 and hh = 1 halves of its own row, and the swap
    // sends them to the lanes of 32-block 0 (R0) and 1 (R1).
    f32x16_t R0, R1;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const bool own = (q >> 3) == sb;
        const float p0 = own ? x[8 * ((q >> 2) & 1) + (q & 3)] : 0.f;
        const float p1 = own ? x[8 * ((q >> 2) & 1) + 4 + (q & 3)] : 0.f;
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
        R0[q] = __uint_as_float(s[0]);
        R1[q] = __uint_as_float(s[1]);
    }
    e16x8_t eye[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float one[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) one[e] = (16 * s + 4 * hh + (e & 3) + 8 * (e >> 2)) == c32 ? 1.f : 0.f;
        eye[s] = pack8<EL>(one);
    }
    // Merge inside each 32-block: T_dd^T = D_dd^T - D_dd^T Aoff^T D_dd^T.
    // Y = Aoff^T D_dd^T has nonzero rows 0-15 only (k-step 0 of the next
    // product), Aoff nonzero rows 16-31 only (k-step 1 of this one); the left
    // factor D_dd (not transposed) comes from D_dd^T and the identity.
    auto merge16 = [&](f32x16_t &R, const e16x8_t &ao) __attribute__((always_inline)) {
        const f32x16_t Y = mfma32<EL>(ao, op8<EL>(R, 1), zero16());
        const f32x16_t E = -mfma32<EL>(op8<EL>(R, 0), eye[0], zero16());
        R = mfma32<EL>(op8<EL>(E, 0), op8<EL>(Y, 0), R);
    };
    merge16(R0, aoff[0]);
    merge16(R1, aoff[1]);

    // A_10 (rows 32-63 of A against columns 0-31; no mask needed).
    {
        float br1[16], gr1[16];
        rows4(bg, 32, br1);
        rows4(gv, 32, gr1);
        const float gi = gv[c32];
#pragma unroll
        for (int q = 0; q < 16; ++q) G10[q] *= br1[q] * __builtin_amdgcn_exp2f(gr1[q] - gi);
    }
    unsigned char *tw = static_cast<unsigned char *>(p.work) + (((size_t)b * Nv + h) * nchk + c) * tk::CHUNK_ELEMS * 2;
    // k-step s of block j, in register order.
    auto put = [&](int j, int s, e16x8_t v) __attribute__((always_inline)) {
        *reinterpret_cast<e16x8_t *>(tw + ((2 * j + s) * 64 + lane) * 16) = v;
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        put(0, s, op8<EL>(R0, s));
        put(1, s, op8<EL>(R1, s));
    }
    // T_10^T = -T_00^T A_10^T T_11^T, with D(T_00) from D(T_00^T) and the identity.
    const f32x16_t Z = -prod<EL>(G10, R1, zero16());
    f32x16_t T0 = mfma32<EL>(op8<EL>(R0, 0), eye[0], zero16());
    T0 = mfma32<EL>(op8<EL>(R0, 1), eye[1], T0);
    const f32x16_t T10 = prod<EL>(T0, Z, zero16());
#pragma unroll
    for (int s = 0; s < 2; ++s) put(2, s, op8<EL>(T10, s));
}

// The chunk step, split so that only two products depend on the state:
//
//   W = T diag(beta exp(gamma)) K,  U = T diag(beta) V,  T = (I + A)^-1
//   Vnew = U - W S0
//   O^T  = (S0^T Q^T) diag(exp(gamma)) + Vnew^T P^T          (scaled on store)
//   S    = exp(gamma_C) S0 + K^T diag(exp(gamma_C - gamma)) Vnew
//
// The columns of S evolve independently, so a head's state may be split by
// columns between workgroups. One workgroup per (sequence, value head, tile
// of DV / NT columns): NT = 2 while the column halves of all heads fit one
// workgroup per CU; NT = 1 (whole heads) beyond that, so that the
// state-independent work of a chunk is done once per head rather than once
// per tile.
//
// Chain waves (the last DVT / 32) each own 32 state columns in float32 result
// registers and, for chunk c, also form U for their columns (it does not
// depend on the state, so it fills gaps in the products' dependency chains);
// their operands never leave registers except W, Q, P, K^T, V and T, read
// from the chunk's operand set.
// Prep waves build the operand set of chunk c + 1 meanwhile.
//   NT = 2, six prep waves: they stage K, Q and V in k-order and T as
//   chunk_t_kernel wrote it; waves 0, 1, 4 form the three nonzero blocks of P,
//   waves 0 and 1 then T diag(beta), U's left operand; waves 2, 3, 5 form -W
//   by 32 features (wave 5 two blocks; waves 2 and 3 share their SIMDs with
//   the chain waves).
//   NT = 1, four prep waves, each sharing its SIMD with a chain wave: all four
//   stage K, Q and the rows of diag(beta) V, so that T itself is U's left
//   operand (T diag(beta) would not fit in LDS beside 128-column V tiles);
//   wave 3 stages T and forms the per-token factors; waves 0-2 form the three
//   blocks of P, and every wave one 32-feature block of -W.
// Products that contract over tokens read K and V through LDS transpose
// reads of the staged rows, so neither is ever transposed explicitly.
// Chain and prep meet once per chunk at a workgroup barrier.

// Rows 8m + 4hh + i (m, i = 0..3) of the 32-row block starting at r0 of a
// per-token vector: the rows that a lane holds in a 32x32 result.
__device__ __forceinline__ void lane_rows(const float *v, int r0, int hh, float *o)
{
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float4 x = *reinterpret_cast<const float4 *>(v + r0 + 8 * m + 4 * hh);
        o[4 * m] = x.x; o[4 * m + 1] = x.y; o[4 * m + 2] = x.z; o[4 * m + 3] = x.w;
    }
}

// P block (tokens r in 32-block rbq, keys i in 32-block ibq), written as rows
// r: scale exp(gamma_r - gamma_i) q_r . k_i for i <= r, else 0. gv holds
// gamma log2(e) per token.
template <typename EL, bool ND>
__device__ __forceinline__ void p_block(unsigned char *set, const float *gv, float scale, int rbq, int ibq, int lane)
{
    const int hh = lane >> 5, c32 = lane & 31;
    f32x16_t G = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        G = mfma32<EL>(ld8(set, mk::S_KT + sw256t(32 * ibq + c32, 2 * ks + hh)),
                       ld8(set, mk::S_Q + sw256(32 * rbq + c32, 2 * ks + hh)), G);
    const int r = 32 * rbq + c32;
    if constexpr (ND) {
#pragma unroll
        for (int q = 0; q < 16; ++q) G[q] = 32 * ibq + drow(q, hh) <= r ? scale * G[q] : 0.f;
    } else {
        const float gq = gv[r];
        float gi[16];
        lane_rows(gv, 32 * ibq, hh, gi);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = 32 * ibq + drow(q, hh);
            G[q] = i <= r ? scale * __builtin_amdgcn_exp2f(gq - gi[q]) * G[q] : 0.f;
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) st8(set, mk::S_P + sw128(r, 2 * (2 * ibq + s) + hh), op8<EL>(G, s));
}

// -W for the 32 features of block fbk, written as -W rows: -W^T = K^T (-T'^T)
// with tp the six operands of -T' = -T diag(beta exp(gamma)).
template <typename EL>
__device__ __forceinline__ void w_block(unsigned char *set, const e16x8_t (&tp)[6], int fbk, int lane)
{
    const int hh = lane >> 5, c32 = lane & 31;
    e16x8_t ak[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) ak[k2] = ldT<256>(set + mk::S_KT, fbk, k2, lane);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        f32x16_t d = zero16();
#pragma unroll
        for (int k2 = 0; k2 < 2 * rb + 2; ++k2) d = mfma32<EL>(ak[k2], tp[rb == 0 ? k2 : 2 + k2], d);
#pragma unroll
        for (int s = 0; s < 2; ++s) st8(set, mk::S_W + sw256(32 * rb + c32, 2 * (2 * fbk + s) + hh), op8<EL>(d, s));
    }
}

// Per-token factors of a chunk (lane t = token t), from the raw beta (or its
// logit) and g (or a) as loaded: gamma is the in-chunk cumulative log decay,
// kept as gamma log2(e) for exp2. bg gets beta, gamma log2(e) and
// beta exp(gamma); vec (in the operand set) the output, update and state
// decays (nothing without decay: the chain then uses none).
template <typename EL, bool FG, bool ND>
__device__ __forceinline__ void token_factors(float *bg, float *vec, uint32_t rb, uint32_t rg, int nv, float scale,
                                              float a_log, float dt_b, int lane)
{
    float beta = EL::to(rb);
    if constexpr (ND) {
        // Outputs need no per-row factor either: rows past the length have
        // zero q.
        bg[lane] = beta;
        bg[64 + lane] = 0.f;
        bg[128 + lane] = beta;
    } else {
        float g = __uint_as_float(rg);
        if constexpr (FG) {
            // Fused gates; tokens past the length are identity steps.
            beta = lane < nv ? gate_sigmoid(beta) : 0.f;
            g = lane < nv ? gate_g(EL::to(rg), a_log, dt_b) : 0.f;
        }
        const float gam2 = wave_prefix_sum(g) * 1.44269504088896340736f;
        const float gamC2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam2), 63));
        const float eg = __builtin_amdgcn_exp2f(gam2);
        bg[lane] = beta;
        bg[64 + lane] = gam2;
        bg[128 + lane] = beta * eg;
        vec[lane] = lane < nv ? scale * eg : 0.f;
        vec[64 + lane] = __builtin_amdgcn_exp2f(gamC2 - gam2);
        if (lane == 0) vec[128] = __builtin_amdgcn_exp2f(gamC2);
    }
}

// FG: fused gates (raw a and beta logits in place of g and beta).
// ND: no decay (g absent, alpha = 1): every decay factor is 1, and the
// multiplies by them are left out.
// NT: column tiles per head (1 or 2).
template <typename EL, bool FG, bool ND, int NT>
__global__ __launch_bounds__(mk::NTHR) void chunk_mfma_kernel(ChunkParams p, int units)
{
    using namespace mk;
    using TL = Tile<NT>;
    constexpr int DVT = TL::DVT, NPREP = TL::NPREP, S_T = TL::S_T, S_VEC = TL::S_VEC, SET_BYTES = TL::SET_BYTES;
    // U's left operand: T diag(beta) (NT = 2), or T with diag(beta) V staged (NT = 1).
    constexpr int S_TU = NT == 2 ? TL::S_TB : TL::S_T;
    extern __shared__ __align__(16) unsigned char smem[];

    // Workgroup -> unit. Workgroups are dealt round-robin to the 8 XCDs, and
    // each XCD starts its workgroups in order as its CUs free up. The units of
    // one (b, key head) — its column tiles and value heads, which share q and
    // k — form a group kept on one XCD and its L2; consecutive groups go to
    // consecutive XCDs, so that every XCD gets an even share of long and short
    // sequences (handing each XCD a contiguous range of sequences instead made
    // the varlen prefill workload 1.7x longer than its average per XCD).
    const int Nk = p.Nk, Nv = p.Nv, S = p.S;
    const int G = NT * (Nv / Nk);
    const int xcd = blockIdx.x % 8, n = blockIdx.x / 8;
    const int u = (8 * (n / G) + xcd) * G + n % G;
    if (u >= units) return;
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
    const int hh = lane >> 5;    // half of the wave
    const int c32 = lane & 31;   // row / column of a 32x32 operand or result

    int L = p.lens ? ld_const(p.lens, b) : S;
    L = L < 0 ? 0 : (L > S ? S : L);
    const int nchunks = (L + C - 1) / C;

    const uint16_t *qb = static_cast<const uint16_t *>(p.q) + ((size_t)b * Nk + kh) * S * DK;
    const uint16_t *kb = static_cast<const uint16_t *>(p.k) + ((size_t)b * Nk + kh) * S * DK;
    const uint16_t *vb = static_cast<const uint16_t *>(p.v) + ((size_t)b * Nv + h) * S * DV + col0;
    const uint16_t *betab = static_cast<const uint16_t *>(p.beta) + ((size_t)b * Nv + h) * S;
    // g (float32), or with fused gates the raw input a (16-bit)
    constexpr bool fg = FG;
    const void *gb = fg ? (const void *)(static_cast<const uint16_t *>(p.gate_a) + ((size_t)b * Nv + h) * S)
                        : (const void *)(p.g ? p.g + ((size_t)b * Nv + h) * S : nullptr);
    // The fused gates' per-head parameters, read once: inside the chunk loop
    // the stores to the outputs keep the compiler from hoisting them.
    const float a_log = fg ? p.A_log[h] : 0.f, dt_b = fg ? p.dt_bias[h] : 0.f;
    uint16_t *ob = static_cast<uint16_t *>(p.out) + ((size_t)b * Nv + h) * S * DV + col0;
    const uint16_t *ib = p.init ? static_cast<const uint16_t *>(p.init) + ((size_t)b * Nv + h) * DK * DV + col0 : nullptr;
    uint16_t *fb = static_cast<uint16_t *>(p.fin) + ((size_t)b * Nv + h) * DK * DV + col0;

    uint32_t *flags = reinterpret_cast<uint32_t *>(smem + TL::P_FLAG);
    if (tid < 4) flags[tid] = 0u;
    lds_barrier();

    if (wv >= NPREP) {
        // ------------------------------ chain ------------------------------
        const int cw = wv - NPREP;   // state columns [32cw, 32cw + 32) of the tile
        // With column halves the recurrence is the critical path: its
        // instructions win issue arbitration against the prep waves sharing
        // the SIMD. With whole heads every SIMD holds a chain wave and a prep
        // wave, the two paths are about as long, and equal priority measured
        // best (varlen prefill pass 1330 us, against 1411 with the chain
        // raised by one and 1429 by two).
        if constexpr (NT == 2) __builtin_amdgcn_s_setprio(2);
        // Outputs go through a buffer resource bounded by this head's output
        // plane: stores of rows past S fall outside it and are dropped by the
        // hardware bounds check, with no branch in the loop.
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(ob, (short)0, (S * DV - col0) * 2, 0x00020000);
        f32x16_t st[4];              // st[f][q] = S[32f + drow(q)][32cw + c32]
        {
            // All 64 loads in flight at once: a buffer resource of size 0
            // when there is no initial state reads zeros, with no branch.
            const __amdgpu_buffer_rsrc_t irs =
                __builtin_amdgcn_make_buffer_rsrc((void *)ib, (short)0, ib ? (DK * DV - col0) * 2 : 0, 0x00020000);
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    st[f][q] = EL::to((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                        irs, ((32 * f + drow(q, hh)) * DV + 32 * cw + c32) * 2, 0, 0));
        }
        if (nchunks > 0) lds_barrier();   // operand set of chunk 0 is ready
        for (int c = 0; c < nchunks; ++c) {
            const unsigned char *set = smem + (c & 1) * SET_BYTES;
            const int t0 = c * C;

            e16x8_t sop[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) sop[ks] = op8<EL>(st[ks >> 1], ks & 1);

            // U = T diag(beta) V for this wave's columns (it does not depend on
            // the state), then Vnew = U - W S0 and S0^T Q^T, one pass over the
            // 128 features.
            f32x16_t vn[2], ot[2], uu[2];
            {
                e16x8_t bv[4];
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) bv[k2] = ldT<2 * DVT>(set + S_VT, cw, k2, lane);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    ot[rb] = zero16();
                    vn[rb] = zero16();
                    uu[rb] = zero16();
#pragma unroll
                    for (int k2 = 0; k2 < 2 * rb + 2; ++k2)
                        uu[rb] = mfma32<EL>(ld8(set + S_TU, t_operand_offset(rb == 0 ? k2 : 2 + k2, lane)), bv[k2], uu[rb]);
                }
            }
            {
                e16x8_t opd[2][4];
                auto ldk = [&](int ks, e16x8_t *o) __attribute__((always_inline)) {
                    o[0] = ld8(set, S_W + sw256(c32, 2 * ks + hh));
                    o[1] = ld8(set, S_W + sw256(32 + c32, 2 * ks + hh));
                    o[2] = ld8(set, S_Q + sw256(c32, 2 * ks + hh));
                    o[3] = ld8(set, S_Q + sw256(32 + c32, 2 * ks + hh));
                };
                ldk(0, opd[0]);
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    if (ks + 1 < 8) ldk(ks + 1, opd[(ks + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    const e16x8_t *o = opd[ks & 1];
                    vn[0] = mfma32<EL>(o[0], sop[ks], vn[0]);
                    vn[1] = mfma32<EL>(o[1], sop[ks], vn[1]);
                    ot[0] = mfma32<EL>(sop[ks], o[2], ot[0]);
                    ot[1] = mfma32<EL>(sop[ks], o[3], ot[1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) vn[rb] += uu[rb];
            const float *vec = reinterpret_cast<const float *>(set + S_VEC);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) ot[tb] *= ND ? p.scale : vec[32 * tb + c32];

            // Vnew as the left operand of Vnew^T, and decayed as the right
            // operand of the state update.
            e16x8_t vna[4], vnb[4];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                if constexpr (ND) {
                    vna[2 * rb] = vnb[2 * rb] = op8<EL>(vn[rb], 0);
                    vna[2 * rb + 1] = vnb[2 * rb + 1] = op8<EL>(vn[rb], 1);
                    continue;
                }
                f32x16_t dv;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float4 d4 = *reinterpret_cast<const float4 *>(vec + 64 + 32 * rb + 8 * m + 4 * hh);
                    dv[4 * m + 0] = vn[rb][4 * m + 0] * d4.x;
                    dv[4 * m + 1] = vn[rb][4 * m + 1] * d4.y;
                    dv[4 * m + 2] = vn[rb][4 * m + 2] * d4.z;
                    dv[4 * m + 3] = vn[rb][4 * m + 3] * d4.w;
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    vna[2 * rb + s] = op8<EL>(vn[rb], s);
                    vnb[2 * rb + s] = op8<EL>(dv, s);
                }
            }
            // O^T += Vnew^T P^T (P is lower triangular by 32-blocks).
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int k2 = 0; k2 < 2 * tb + 2; ++k2)
                    ot[tb] = mfma32<EL>(vna[k2], ld8(set, S_P + sw128(32 * tb + c32, 2 * k2 + hh)), ot[tb]);
            // Outputs: lane holds 4 consecutive columns of one token per group.
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int r = 32 * tb + c32;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x2_t o = {EL::pack(ot[tb][4 * m], ot[tb][4 * m + 1]), EL::pack(ot[tb][4 * m + 2], ot[tb][4 * m + 3])};
                    __builtin_amdgcn_raw_buffer_store_b64(o, orsrc,
                                                          ((t0 + r) * DV + 32 * cw + 8 * m + 4 * hh) * 2, 0, 0);
                }
            }
            // S <- exp(gamma_C) S0 + K^T (decayed Vnew).
            if constexpr (!ND) {
                const float egC = vec[128];
#pragma unroll
                for (int f = 0; f < 4; ++f) st[f] *= egC;
            }
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2)
                    st[f] = mfma32<EL>(ldT<256>(set + S_KT, f, k2, lane), vnb[k2], st[f]);
            lds_barrier();
        }
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                fb[(size_t)(32 * f + drow(q, hh)) * DV + 32 * cw + c32] = EL::from(st[f][q]);
    } else {
        // ------------------------------- prep ------------------------------

        // Inputs are read through buffer resources bounded by the sequence's
        // valid length: rows past it come back as zeros from the hardware
        // bounds check (identity steps). Loads need no branch, and are issued
        // even past the last chunk, so the loaded registers never meet control
        // flow that would make the compiler wait for them on the spot.
        const int Lk = L * DK * 2, Lv = (L * DV - col0) * 2;
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, Lk, 0x00020000);
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void *)qb, (short)0, Lk, 0x00020000);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, Lv, 0x00020000);
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc((void *)betab, (short)0, L * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t grs =
            __builtin_amdgcn_make_buffer_rsrc((void *)gb, (short)0, gb ? L * (fg ? 2 : 4) : 0, 0x00020000);
        // T of this head's chunks (written by chunk_t_kernel), bounded by the
        // chunks that exist; a chunk's 6 KB are copied as they are into its
        // operand set.
        const int nchk = (S + C - 1) / C;
        const uint16_t *twb = static_cast<const uint16_t *>(p.work) + ((size_t)b * Nv + h) * nchk * tk::CHUNK_ELEMS;
        const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc((void *)twb, (short)0, nchunks * tk::CHUNK_ELEMS * 2, 0x00020000);
        float *bg = reinterpret_cast<float *>(smem + TL::P_BG);
        const float *gv = bg + 64, *fv = bg + 128;

        // K and Q rows of a chunk into k-ordered tiles: a row of 256 bytes spans
        // 8 consecutive lanes, 32 bytes each; lane id of the 256 staging lanes.
        auto stage_kq = [&](unsigned char *set, u32x4_t (&ra)[8], int id0) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int id = id0 + 256 * m, row = id >> 3, grp = id & 7;
                if (p.qk_norm) {
                    u32x4_t kx[2] = {ra[2 * m], ra[2 * m + 1]}, qx[2] = {ra[4 + 2 * m], ra[5 + 2 * m]};
                    normalise_row<EL, 8>(kx);
                    normalise_row<EL, 8>(qx);
                    ra[2 * m] = kx[0]; ra[2 * m + 1] = kx[1];
                    ra[4 + 2 * m] = qx[0]; ra[5 + 2 * m] = qx[1];
                }
                *reinterpret_cast<u32x4_t *>(set + S_KT + sw256t(row, 2 * grp)) = korder_lo(ra[2 * m], ra[2 * m + 1]);
                *reinterpret_cast<u32x4_t *>(set + S_KT + sw256t(row, 2 * grp + 1)) = korder_hi(ra[2 * m], ra[2 * m + 1]);
                *reinterpret_cast<u32x4_t *>(set + S_Q + sw256(row, 2 * grp)) = korder_lo(ra[4 + 2 * m], ra[5 + 2 * m]);
                *reinterpret_cast<u32x4_t *>(set + S_Q + sw256(row, 2 * grp + 1)) = korder_hi(ra[4 + 2 * m], ra[5 + 2 * m]);
            }
        };
        auto issue_kq = [&](u32x4_t (&ra)[8], int id0, int t0) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int id = id0 + 256 * m, row = id >> 3, grp = id & 7;
                const int off = ((t0 + row) * DK + 16 * grp) * 2;
                ra[2 * m] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
                ra[2 * m + 1] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 16, 0, 0);
                ra[4 + 2 * m] = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
                ra[5 + 2 * m] = __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 16, 0, 0);
            }
        };
        auto issue_factors = [&](uint32_t &rb, uint32_t &rg, int t0) __attribute__((always_inline)) {
            rb = __builtin_amdgcn_raw_buffer_load_b16(brs, (t0 + lane) * 2, 0, 0);
            if constexpr (!ND)
                rg = fg ? __builtin_amdgcn_raw_buffer_load_b16(grs, (t0 + lane) * 2, 0, 0)
                        : __builtin_amdgcn_raw_buffer_load_b32(grs, (t0 + lane) * 4, 0, 0);
        };

        if constexpr (NT == 2) {
            // Chunk inputs in flight: waves 2-5 hold 2 x 32 bytes of K and of Q,
            // waves 0-1 2 x 32 bytes of V and 3 x 16 bytes of T, wave 1 one beta
            // and one g.
            u32x4_t ra[8], rt[3], traw[3];
            uint32_t rb = 0, rg = 0;
            const int ltid = wv >= 2 ? tid - 128 : tid;   // 0-255 for K/Q, 0-127 for V
            auto issue = [&](auto R, int cn) __attribute__((always_inline)) {
                constexpr int W = decltype(R)::value;
                const int t0 = cn * C;
                if constexpr (W >= 2) {
                    issue_kq(ra, ltid, t0);
                } else {
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const int id = ltid + 128 * m, row = id >> 2, grp = id & 3;
                        const int off = ((t0 + row) * DV + 16 * grp) * 2;
                        ra[2 * m] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
                        ra[2 * m + 1] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off + 16, 0, 0);
                    }
#pragma unroll
                    for (int n = 0; n < 3; ++n)
                        rt[n] = __builtin_amdgcn_raw_buffer_load_b128(trs, cn * tk::CHUNK_ELEMS * 2 + (ltid + 128 * n) * 16, 0, 0);
                    if constexpr (W == 1) issue_factors(rb, rg, t0);
                }
            };

            auto prep = [&](auto R, int cn) __attribute__((always_inline)) {
                constexpr int W = decltype(R)::value;
                unsigned char *set = smem + (cn & 1) * SET_BYTES;
                const uint32_t ncall = (uint32_t)cn + 1u;

                // ---- stage chunk cn (K and Q rows, V rows, T) ----
                if constexpr (W >= 2) {
                    stage_kq(set, ra, ltid);
                } else {
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const int id = ltid + 128 * m, row = id >> 2, grp = id & 3;
                        *reinterpret_cast<u32x4_t *>(set + S_VT + sw128t(row, 2 * grp)) = korder_lo(ra[2 * m], ra[2 * m + 1]);
                        *reinterpret_cast<u32x4_t *>(set + S_VT + sw128t(row, 2 * grp + 1)) = korder_hi(ra[2 * m], ra[2 * m + 1]);
                    }
#pragma unroll
                    for (int n = 0; n < 3; ++n) {
                        *reinterpret_cast<u32x4_t *>(set + S_T + (ltid + 128 * n) * 16) = rt[n];
                        traw[n] = rt[n];
                    }
                    if constexpr (W == 1)
                        token_factors<EL, FG, ND>(bg, reinterpret_cast<float *>(set + S_VEC), rb, rg, min(C, L - cn * C),
                                                  p.scale, a_log, dt_b, lane);
                }
                issue(R, cn + 1);
                arrive(flags + 0, lane);
                wait_for(flags + 0, 6u * ncall);

                if constexpr (W == 0 || W == 1 || W == 4)
                    p_block<EL, ND>(set, gv, p.scale, W == 0 ? 0 : 1, W == 4 ? 1 : 0, lane);
                if constexpr (W < 2) {
                    // T diag(beta) for the chain's U, from this lane's three pieces
                    // of T (block j = n, k-step s = W: tokens 16 k2 + 4hh + {0..3,
                    // 8..11} with k2 = s, or 2 + s in T_11).
#pragma unroll
                    for (int n = 0; n < 3; ++n) {
                        const int i0 = 16 * (n == 1 ? 2 + W : W) + 4 * hh;
                        const float4 f0 = *reinterpret_cast<const float4 *>(bg + i0), f1 = *reinterpret_cast<const float4 *>(bg + i0 + 8);
                        const float fe[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
                        const uint32_t w4[4] = {traw[n].x, traw[n].y, traw[n].z, traw[n].w};
                        float r[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) r[e] = ((e & 1) ? EL::hi(w4[e >> 1]) : EL::lo(w4[e >> 1])) * fe[e];
                        st8(set, TL::S_TB + (ltid + 128 * n) * 16, pack8<EL>(r));
                    }
                }
                if constexpr (W == 2 || W == 3 || W == 5) {
                    // -W by 32 features: blocks 2 and 3 on waves 2 and 3, blocks
                    // 0 and 1 on wave 5.
                    e16x8_t tp[6];
#pragma unroll
                    for (int n = 0; n < 6; ++n) tp[n] = t_operand<EL, true>(set + S_T, n, fv, lane);
                    if constexpr (W == 5) {
                        w_block<EL>(set, tp, 0, lane);
                        w_block<EL>(set, tp, 1, lane);
                    } else {
                        w_block<EL>(set, tp, W, lane);
                    }
                }
            };

            // Each role runs its own copy of the loop, so that it keeps only its
            // own addresses and values live.
            auto run = [&](auto R) __attribute__((always_inline)) {
                if (nchunks > 0) {
                    issue(R, 0);
                    prep(R, 0);
                    lds_barrier();
                    for (int c = 0; c + 1 < nchunks; ++c) {
                        prep(R, c + 1);
                        lds_barrier();
                    }
                    lds_barrier();   // the chain's last chunk
                }
            };
            switch (wv) {
            case 0: run(std::integral_constant<int, 0>{}); break;
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 4: run(std::integral_constant<int, 4>{}); break;
            default: run(std::integral_constant<int, 5>{}); break;
            }
        } else {
            // Whole rows, four prep waves. Chunk inputs in flight: every lane
            // holds 2 x 32 bytes each of K, Q and V and the betas of its two V
            // rows; waves 0-2 also two 16-byte pieces of T, wave 3 one beta
            // and one g for the per-token factors. The K, Q and V loads of the
            // next chunk are issued as soon as these are staged, ahead of the
            // smaller jobs, so that they have a whole chunk period to land.
            u32x4_t ra[8], rv[4], rt[2];
            uint32_t rbv[2] = {0u, 0u}, rb = 0, rg = 0;
            auto issue_rows = [&](int cn) __attribute__((always_inline)) {
                const int t0 = cn * C;
                issue_kq(ra, tid, t0);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int id = tid + 256 * m, row = id >> 3, grp = id & 7;
                    const int off = ((t0 + row) * DV + 16 * grp) * 2;
                    rv[2 * m] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
                    rv[2 * m + 1] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off + 16, 0, 0);
                    rbv[m] = __builtin_amdgcn_raw_buffer_load_b16(brs, (t0 + row) * 2, 0, 0);
                }
            };
            auto issue_aux = [&](auto R, int cn) __attribute__((always_inline)) {
                constexpr int W = decltype(R)::value;
                if constexpr (W < 3) {
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        rt[n] = __builtin_amdgcn_raw_buffer_load_b128(trs, cn * tk::CHUNK_ELEMS * 2 + (tid + 192 * n) * 16, 0, 0);
                } else {
                    issue_factors(rb, rg, cn * C);
                }
            };
            auto issue = [&](auto R, int cn) __attribute__((always_inline)) {
                issue_rows(cn);
                issue_aux(R, cn);
            };

            auto prep = [&](auto R, int cn) __attribute__((always_inline)) {
                constexpr int W = decltype(R)::value;
                unsigned char *set = smem + (cn & 1) * SET_BYTES;
                const uint32_t ncall = (uint32_t)cn + 1u;

                // ---- stage chunk cn (K and Q rows, diag(beta) V rows, T) ----
                stage_kq(set, ra, tid);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    // Rows past the length are zero whatever their beta.
                    const int id = tid + 256 * m, row = id >> 3, grp = id & 7;
                    float bt = EL::to(rbv[m]);
                    if constexpr (FG) bt = gate_sigmoid(bt);
                    uint32_t w[8] = {rv[2 * m].x, rv[2 * m].y, rv[2 * m].z, rv[2 * m].w,
                                     rv[2 * m + 1].x, rv[2 * m + 1].y, rv[2 * m + 1].z, rv[2 * m + 1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = EL::pack(EL::lo(w[e]) * bt, EL::hi(w[e]) * bt);
                    const u32x4_t a = {w[0], w[1], w[2], w[3]}, c = {w[4], w[5], w[6], w[7]};
                    *reinterpret_cast<u32x4_t *>(set + S_VT + sw256t(row, 2 * grp)) = korder_lo(a, c);
                    *reinterpret_cast<u32x4_t *>(set + S_VT + sw256t(row, 2 * grp + 1)) = korder_hi(a, c);
                }
                issue_rows(cn + 1);
                if constexpr (W < 3) {
#pragma unroll
                    for (int n = 0; n < 2; ++n) *reinterpret_cast<u32x4_t *>(set + S_T + (tid + 192 * n) * 16) = rt[n];
                } else {
                    token_factors<EL, FG, ND>(bg, reinterpret_cast<float *>(set + S_VEC), rb, rg, min(C, L - cn * C),
                                              p.scale, a_log, dt_b, lane);
                }
                issue_aux(R, cn + 1);
                arrive(flags + 0, lane);
                wait_for(flags + 0, 4u * ncall);

                if constexpr (W < 3) p_block<EL, ND>(set, gv, p.scale, W == 0 ? 0 : 1, W == 2 ? 1 : 0, lane);
                e16x8_t tp[6];
#pragma unroll
                for (int n = 0; n < 6; ++n) tp[n] = t_operand<EL, true>(set + S_T, n, fv, lane);
                w_block<EL>(set, tp, W, lane);
            };

            auto run = [&](auto R) __attribute__((always_inline)) {
                if (nchunks > 0) {
                    issue(R, 0);
                    prep(R, 0);
                    lds_barrier();
                    for (int c = 0; c + 1 < nchunks; ++c) {
                        prep(R, c + 1);
                        lds_barrier();
                    }
                    lds_barrier();   // the chain's last chunk
                }
            };
            switch (wv) {
            case 0: run(std::integral_constant<int, 0>{}); break;
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            default: run(std::integral_constant<int, 3>{}); break;
            }
        }
    }
    // Output rows of the chunks past the last one processed are padding,
    // zeroed by chunk_t_kernel.
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
    // fused gates: beta holds the logits, and g comes from a
    const float *gab = p.gate_a ? static_cast<const float *>(p.gate_a) + ((size_t)b * Nv + h) * Sl : nullptr;
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
        if (tid < C) bet[tid] = tid < nval ? (p.beta_logit ? gate_sigmoid(betab[t0 + tid]) : betab[t0 + tid]) : 0.f;
        if (tid == 0) {
            float a = 0.f;
            for (int r = 0; r < C; ++r) {
                if (r < nval) a += gab ? gate_g(gab[t0 + r], p.A_log[h], p.dt_bias[h]) : (gb ? gb[t0 + r] : 0.f);
                gam[r] = a;
            }
        }
        __syncthreads();
        if (p.qk_norm) {
            // k and q rows to x / sqrt(|x|^2 + eps); padded rows stay zero.
            for (int r = tid; r < 2 * C; r += 256) {
                float *row = (r < C ? Kc : Qc) + (r % C) * LD;
                float ss = 0.f;
                for (int d = 0; d < D; ++d) ss = fmaf(row[d], row[d], ss);
                const float rn = qk_rnorm(ss);
                for (int d = 0; d < D; ++d) row[d] *= rn;
            }
            __syncthreads();
        }
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

// The 16-bit matrix-core path takes chunk sizes 16, 32 and 64 and computes in
// chunks of 64: the chunk size is a blocking of the same recurrence, and the
// result differs only in rounding.
static bool mfma_chunk_size(int C) { return C == 16 || C == 32 || C == mk::C; }

int64_t chunk_workspace_bytes(int dtype, int Dk, int Dv, int C, int B, int Nv, int S)
{
    if ((dtype == 1 || dtype == 2) && Dk == mk::DK && Dv == mk::DV && mfma_chunk_size(C))
        return (int64_t)B * Nv * ((S + mk::C - 1) / mk::C) * tk::CHUNK_ELEMS * 2;
    return 0;
}

// The matrix-core kernel for an element format (0 bf16, 1 fp16), a form (0
// plain, 1 fused gates, 2 no decay) and NT column tiles per head.
static const void *mfma_variant(int half, int form, int nt)
{
#define GDR_MFMA_FORMS(EL_, NT_)                                                                                 \
    (form == 1 ? (const void *)chunk_mfma_kernel<EL_, true, false, NT_>                                          \
               : (form == 2 ? (const void *)chunk_mfma_kernel<EL_, false, true, NT_> : (const void *)chunk_mfma_kernel<EL_, false, false, NT_>))
    if (half) return nt == 1 ? GDR_MFMA_FORMS(F16, 1) : GDR_MFMA_FORMS(F16, 2);
    return nt == 1 ? GDR_MFMA_FORMS(BF16, 1) : GDR_MFMA_FORMS(BF16, 2);
#undef GDR_MFMA_FORMS
}

hipError_t launch_chunk(int dtype, int Dk, int Dv, int C, const ChunkParams &p, hipStream_t s, bool *supported)
{
    *supported = true;
    ChunkParams pc = p;
    if (dtype == 1 || dtype == 2) {
        if (Dk == mk::DK && Dv == mk::DV && mfma_chunk_size(C)) {
            const bool half = dtype == 2;
            // T of every chunk first, then the pass over the chunks.
            int nchk = (p.S + mk::C - 1) / mk::C;
            int tunits = p.B * p.Nv * nchk;
            if (tunits > 0) {
                void *targs[] = {&pc, &nchk, &tunits};
                const hipError_t e = hipLaunchKernel(half ? (const void *)chunk_t_kernel<F16> : (const void *)chunk_t_kernel<BF16>,
                                                     dim3((tunits + tk::WAVES - 1) / tk::WAVES), dim3(64 * tk::WAVES),
                                                     targs, 0, s);
                if (e != hipSuccess) return e;
            }
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
            // Column halves (NT = 2) while they fit one workgroup per CU, else
            // whole heads (NT = 1): a whole-head workgroup takes about 1.7x as
            // long per chunk as a half-head one, but does the work of two
            // (measured: 187.6 against 213.2 us at 128 heads of 4096 tokens,
            // 292.4 against 231.2 us at 160, 718.8 against 581.5 us at 512).
            int ncu = 0;
            if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
            const int nt = 2LL * p.B * p.Nv > ncu ? 1 : 2;
            const int units = p.B * p.Nv * nt;
            const int G = nt * (p.Nv / p.Nk);   // units of one (b, key head), kept on one XCD
            const int nwg = (units + 8 * G - 1) / (8 * G) * (8 * G);
            int u = units;
            void *args[] = {&pc, &u};
            // Raise the dynamic-LDS limit once per device (its first launch
            // there). The only state the library keeps: one bit per device,
            // set after the attribute is in place; racing first calls both
            // set it, which is harmless.
            static std::atomic<uint64_t> attr_done{0};
            const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
            if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
                for (int t = 0; t < 12; ++t) {
                    hipError_t e = hipFuncSetAttribute(mfma_variant(t & 1, (t >> 1) % 3, t < 6 ? 1 : 2),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, t < 6 ? mk::Tile<1>::LDS_BYTES
                                                                                                        : mk::Tile<2>::LDS_BYTES);
                    if (e != hipSuccess) return e;
                }
                attr_done.fetch_or(bit, std::memory_order_acq_rel);
            }
            const int form = pc.gate_a ? 1 : (!pc.g ? 2 : 0);
            return hipLaunchKernel(mfma_variant(half, form, nt), dim3(nwg), dim3(mk::NTHR), args,
                                   nt == 1 ? mk::Tile<1>::LDS_BYTES : mk::Tile<2>::LDS_BYTES, s);
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
