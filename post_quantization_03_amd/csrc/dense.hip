// Dense linear algebra on MFMA for gfx950: a batched GEMM (fp32 and fp64 matrix cores), a blocked
// Cholesky factorisation, a triangular inverse, and the two ABI calls built on them:
//   kq_cholinv  - damped factor R of H^{-1} (GPTQ's Cholesky form of the inverse Hessian), factorised
//                 in fp64 and rounded to fp32
//   kq_hg_sqrt  - principal square root of H_G and its inverse (output side of bidirectional
//                 incoherence processing), by the scaled Denman-Beavers iteration in fp64.
#include <cmath>

#include "kq_internal.h"

namespace kq {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef double d4v __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;
// Accumulator layouts differ: fp32 16x16x4 keeps rows 4*(l/16)+r in lane l, fp64 16x16x4 keeps
// rows 4*r + l/16 (both with column l%16); checked with a one-wave probe on gfx950.
template <>
struct Mfma<float> {
    typedef f4v acc_t;
    __device__ static inline acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline int row(int lane, int r) { return 4 * (lane >> 4) + r; }
};
template <>
struct Mfma<double> {
    typedef d4v acc_t;
    __device__ static inline acc_t mma(double a, double b, acc_t c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    __device__ static inline int row(int lane, int r) { return 4 * r + (lane >> 4); }
};

template <typename T>
struct alignas(16) V16 {
    T v[16 / sizeof(T)];
};

constexpr int GBM = 128, GBN = 128;
// LDS row pad (elements): makes the row stride 16 banks modulo 32 for both element sizes, so the
// four 16-lane groups of an operand read (rows kr..kr+3) fall on alternate bank halves.
template <typename T>
constexpr int gpad() { return sizeof(T) == 8 ? 8 : 16; }

// ===================================================================================== GEMM kernel
// 256 threads = 4 waves in a 2 x 2 arrangement; each wave owns a 64 x 64 block of C as 4 x 4
// MFMA 16x16 tiles (K = 4 per instruction). K is staged through LDS in 16-deep slices,
// double-buffered with one barrier per slice. Each operand keeps in LDS the contiguity it has in
// memory, so that the slice stores are whole 16-byte vectors: an operand contiguous along M (or N)
// is stored k-major ([k][m], rows padded by gpad so the 16-lane groups of an MFMA operand read hit
// disjoint banks); an operand contiguous along K (A not transposed) is stored m-major ([m][k], row
// stride BK + 4 = 20 floats: 20 m mod 64 is distinct for 16 consecutive m). MFMA operand layout
// (16x16x4): lane l holds A[l%16][l/16] and B[l/16][l%16]; the 4 accumulator registers hold column
// l%16 of C in the rows given by Mfma<T>::row.
template <typename T>
constexpr int gemm_bk() { return sizeof(T) == 8 ? 16 : 16; }

template <typename T, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs<T> g) {
    if (g.skip && *g.skip) return;
    constexpr int BK = gemm_bk<T>();
    constexpr int VN = 16 / sizeof(T);
    constexpr int VPR = BK / VN;                  // 16-byte vectors per tile row (k direction)
    constexpr int NV = GBM * BK / VN / 256;       // vectors per thread per operand
    // A: [BK][GBM + pad] when contiguous along M (TA), else [GBM][BK + 4] (one layout unused)
    constexpr int AKM = TA ? BK : GBM, AMN = TA ? GBM + gpad<T>() : BK + 16 / (int)sizeof(T);
    __shared__ __align__(16) T As[2][AKM][AMN];
    __shared__ __align__(16) T Bs[2][BK][GBN + gpad<T>()];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Tile order: work-groups are dealt round-robin to the 8 XCDs, so the linear id is remapped so
    // that each XCD works on a contiguous range of tiles (neighbouring tiles share A / B panels in
    // that XCD's L2). Triangular products launch only the stored triangle (1-D grid).
    int64_t tm, tn;
    {
        const int64_t nx = (g.N + GBN - 1) / GBN;
        const int64_t L = g.tri ? (int64_t)gridDim.x : (int64_t)gridDim.x * gridDim.y;
        int64_t lid = g.tri ? (int64_t)blockIdx.x : (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        if (L % 8 == 0) lid = (lid % 8) * (L / 8) + lid / 8;
        if (g.tri) {
            int64_t r = (int64_t)((sqrt(8.0 * (double)lid + 1.0) - 1.0) * 0.5);
            while (r * (r + 1) / 2 > lid) r--;
            while ((r + 1) * (r + 2) / 2 <= lid) r++;
            const int64_t c = lid - r * (r + 1) / 2;
            if (g.tri == 1) { tm = r; tn = c; } else { tm = c; tn = r; }
        } else {
            tm = lid / nx;
            tn = lid % nx;
        }
    }
    const int64_t m0 = tm * GBM, n0 = tn * GBN;
    if (tm == g.skip_tile || tn == g.skip_tile) return;
    const int64_t z = blockIdx.z, z1 = z / g.nb2, z2 = z % g.nb2;
    const T* __restrict__ A = g.A + z1 * g.sA1 + z2 * g.sA2;
    const T* __restrict__ B = g.B + z1 * g.sB1 + z2 * g.sB2;
    T* C = g.C + z1 * g.sC1 + z2 * g.sC2;
    const int8_t* rs = g.rsign ? g.rsign + z1 * g.sR1 + z2 * g.sR2 : nullptr;
    const int8_t* cs = g.csign ? g.csign + z1 * g.sS1 + z2 * g.sS2 : nullptr;
    const int64_t M = g.M, N = g.N;
    int64_t kb = 0, ke = g.K;
    if (g.kmode & 1) kb = kb > m0 ? kb : m0;
    if (g.kmode & 2) kb = kb > n0 ? kb : n0;
    if (g.kmode & 4) ke = ke < m0 + GBM ? ke : m0 + GBM;
    if (g.kmode & 8) ke = ke < n0 + GBN ? ke : n0 + GBN;
    kb = (kb / BK) * BK;

    typename Mfma<T>::acc_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = typename Mfma<T>::acc_t{0, 0, 0, 0};

    const int wm = wave >> 1, wn = wave & 1;
    T ra[NV][VN], rb[NV][VN];
    const bool fullMN = (m0 + GBM <= M) && (n0 + GBN <= N);

    auto gload = [&](int64_t k0) {
        const bool full = VEC && fullMN && (k0 + BK <= ke);
#pragma unroll
        for (int q = 0; q < NV; q++) {
            const int v = tid + 256 * q;
            // ---- A
            {
                int64_t gm, gk;
                if (!TA) { gm = m0 + v / VPR; gk = k0 + (v % VPR) * VN; }
                else { gk = k0 + v / (GBM / VN); gm = m0 + (v % (GBM / VN)) * VN; }
                const T* p = TA ? A + gk * g.lda + gm : A + gm * g.lda + gk;
                if (full) {
                    V16<T> t = *reinterpret_cast<const V16<T>*>(p);
#pragma unroll
                    for (int e = 0; e < VN; e++) ra[q][e] = t.v[e];
                } else {
#pragma unroll
                    for (int e = 0; e < VN; e++) {
                        bool in = TA ? (gk < ke && gm + e < M) : (gm < M && gk + e < ke);
                        ra[q][e] = in ? p[e] : T(0);
                    }
                }
            }
            // ---- B
            {
                int64_t gn, gk;
                if (TB) { gn = n0 + v / VPR; gk = k0 + (v % VPR) * VN; }
                else { gk = k0 + v / (GBN / VN); gn = n0 + (v % (GBN / VN)) * VN; }
                const T* p = TB ? B + gn * g.ldb + gk : B + gk * g.ldb + gn;
                if (full) {
                    V16<T> t = *reinterpret_cast<const V16<T>*>(p);
#pragma unroll
                    for (int e = 0; e < VN; e++) rb[q][e] = t.v[e];
                } else {
#pragma unroll
                    for (int e = 0; e < VN; e++) {
                        bool in = TB ? (gn < N && gk + e < ke) : (gk < ke && gn + e < N);
                        rb[q][e] = in ? p[e] : T(0);
                    }
                }
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NV; q++) {
            const int v = tid + 256 * q;
            if (!TA) {
                V16<T> t;
#pragma unroll
                for (int e = 0; e < VN; e++) t.v[e] = ra[q][e];
                *reinterpret_cast<V16<T>*>(&As[buf][v / VPR][(v % VPR) * VN]) = t;
            } else {
#pragma unroll
                for (int e = 0; e < VN; e++) As[buf][v / (GBM / VN)][(v % (GBM / VN)) * VN + e] = ra[q][e];
            }
            if (TB) {
#pragma unroll
                for (int e = 0; e < VN; e++) Bs[buf][(v % VPR) * VN + e][v / VPR] = rb[q][e];
            } else {
#pragma unroll
                for (int e = 0; e < VN; e++) Bs[buf][v / (GBN / VN)][(v % (GBN / VN)) * VN + e] = rb[q][e];
            }
        }
    };

    if (kb < ke) {
        gload(kb);
        sstore(0);
        __syncthreads();
        int buf = 0;
        for (int64_t k0 = kb; k0 < ke; k0 += BK) {
            const bool more = k0 + BK < ke;
            if (more) gload(k0 + BK);
#pragma unroll
            for (int kk = 0; kk < BK; kk += 4) {
                T a[4], b[4];
                const int kr = kk + (lane >> 4);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    a[i] = TA ? As[buf][kr][wm * 64 + 16 * i + (lane & 15)] : As[buf][wm * 64 + 16 * i + (lane & 15)][kr];
#pragma unroll
                for (int j = 0; j < 4; j++) b[j] = Bs[buf][kr][wn * 64 + 16 * j + (lane & 15)];
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++) acc[i][j] = Mfma<T>::mma(a[i], b[j], acc[i][j]);
            }
            if (more) sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    // epilogue in four chunks of 16 values per lane: all loads of C for a chunk are issued before
    // any of them is used, so the read-modify-write pays one memory latency per chunk
    const int64_t nl = n0 + wn * 64 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        T cv[4][4];
        int64_t mr[4];
#pragma unroll
        for (int r = 0; r < 4; r++) mr[r] = m0 + wm * 64 + 16 * i + Mfma<T>::row(lane, r);
        if (g.beta != T(0)) {
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int64_t n = nl + 16 * j;
                    cv[j][r] = (mr[r] < M && n < N) ? C[mr[r] * g.ldc + n] : T(0);
                }
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t m = mr[r], n = nl + 16 * j;
                if (m >= M || n >= N) continue;
                if (g.tri == 1 && n > m) continue;
                if (g.tri == 2 && m > n) continue;
                T v = g.alpha * acc[i][j][r];
                if (rs) v *= T(rs[m]);
                if (cs) v *= T(cs[n]);
                if (g.beta != T(0)) v += g.beta * cv[j][r];
                C[m * g.ldc + n] = v;
            }
    }
}

// fp32, neither operand transposed, rows of A and B in 16-byte vectors, K a multiple of 16, every tile
// launched (no triangle, K range or skipped tile): the same 128 x 128 tile, waves, MFMA sequence and
// epilogue as gemm_kernel, so each element of C is bit-identical to it, scheduled for throughput:
//  * the next K slice is loaded into registers before the current slice's products and stored to LDS
//    after them; the loads are ordinary (not read-only) loads held in place by a compiler barrier, so the
//    compiler can neither sink them next to their LDS stores nor spill them (the last slice reloads
//    itself, keeping the loop free of branches);
//  * at most 128 VGPRs (no accumulation registers), so with 38 KB of LDS four work-groups share a compute
//    unit;
//  * tiles in groups of 8 tile rows swept column by column inside each XCD's contiguous range, so a
//    group's A and B panels stay in that XCD's L2 while it works on them.
// Ragged M and N (N a multiple of 4) load clamped rows and columns and store only inside C.
// Measured on MI355X against gemm_kernel: 28672 x 7680 x 512 at 129 instead of 94 TFLOP/s, 4096^3 at
// 135 instead of 106, 28672 x 384 x 128 in 38 instead of 72 us.
constexpr int GF_BK = 16, GF_GROUP = 8;
__global__ __launch_bounds__(256, 2) void gemm_f32_nn_kernel(GemmArgs<float> g) {
    if (g.skip && *g.skip) return;
    __shared__ __align__(16) float As[2][GBM][GF_BK + 4];
    __shared__ __align__(16) float Bs[2][GF_BK][GBN + 16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t nx = (N + GBN - 1) / GBN, ny = (M + GBM - 1) / GBM, L = nx * ny;
    int64_t lid = blockIdx.x;
    if (L % 8 == 0) lid = (lid % 8) * (L / 8) + lid / 8;
    const int64_t grp = lid / (GF_GROUP * nx), r0 = grp * GF_GROUP;
    const int64_t rows = (ny - r0) < GF_GROUP ? (ny - r0) : GF_GROUP;
    const int64_t in = lid - grp * GF_GROUP * nx;
    const int64_t m0 = (r0 + in % rows) * GBM, n0 = (in / rows) * GBN;
    const int64_t z = blockIdx.z, z1 = z / g.nb2, z2 = z % g.nb2;
    const float* A = g.A + z1 * g.sA1 + z2 * g.sA2;
    const float* B = g.B + z1 * g.sB1 + z2 * g.sB2;
    float* C = g.C + z1 * g.sC1 + z2 * g.sC2;
    const int8_t* rs = g.rsign ? g.rsign + z1 * g.sR1 + z2 * g.sR2 : nullptr;
    const int8_t* cs = g.csign ? g.csign + z1 * g.sS1 + z2 * g.sS2 : nullptr;

    f4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f4v{0, 0, 0, 0};
    const int wm = wave >> 1, wn = wave & 1;
    // thread's vectors (q = 0, 1; v = tid + 256 q): A row v / 4, k (v % 4) * 4; B k v / 32, n (v % 32) * 4
    const float* pa[2];
    const float* pb[2];
    int sa[2], sb[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int v = tid + 256 * q;
        int64_t m = m0 + v / 4, n = n0 + (v % 32) * 4;
        m = m < M ? m : M - 1;
        n = n < N ? n : N - 4;
        pa[q] = A + m * g.lda + (v % 4) * 4;
        pb[q] = B + (int64_t)(v / 32) * g.ldb + n;
        sa[q] = (v / 4) * (GF_BK + 4) + (v % 4) * 4;
        sb[q] = (v / 32) * (GBN + 16) + (v % 32) * 4;
    }
    f4v ra[2], rb[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        ra[q] = *reinterpret_cast<const f4v*>(pa[q]);
        rb[q] = *reinterpret_cast<const f4v*>(pb[q]);
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
        *reinterpret_cast<f4v*>(&As[0][0][0] + sa[q]) = ra[q];
        *reinterpret_cast<f4v*>(&Bs[0][0][0] + sb[q]) = rb[q];
    }
    __syncthreads();
    int buf = 0;
    for (int64_t k0 = 0; k0 < K; k0 += GF_BK) {
        const int64_t kn = (k0 + GF_BK < K) ? k0 + GF_BK : k0;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            ra[q] = *reinterpret_cast<const f4v*>(pa[q] + kn);
            rb[q] = *reinterpret_cast<const f4v*>(pb[q] + kn * g.ldb);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < GF_BK; kk += 4) {
            float a[4], b[4];
            const int kr = kk + (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = As[buf][wm * 64 + 16 * i + (lane & 15)][kr];
#pragma unroll
            for (int j = 0; j < 4; j++) b[j] = Bs[buf][kr][wn * 64 + 16 * j + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = Mfma<float>::mma(a[i], b[j], acc[i][j]);
        }
        float* an = &As[buf ^ 1][0][0];
        float* bn = &Bs[buf ^ 1][0][0];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            *reinterpret_cast<f4v*>(an + sa[q]) = ra[q];
            *reinterpret_cast<f4v*>(bn + sb[q]) = rb[q];
        }
        __syncthreads();
        buf ^= 1;
    }

    // epilogue as in gemm_kernel: per chunk of 16 values, the loads of C first, then the stores
    const int64_t nl = n0 + wn * 64 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float cv[4][4];
        int64_t mr[4];
#pragma unroll
        for (int r = 0; r < 4; r++) mr[r] = m0 + wm * 64 + 16 * i + Mfma<float>::row(lane, r);
        if (g.beta != 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int64_t n = nl + 16 * j;
                    cv[j][r] = (mr[r] < M && n < N) ? C[mr[r] * g.ldc + n] : 0.0f;
                }
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t m = mr[r], n = nl + 16 * j;
                if (m >= M || n >= N) continue;
                float v = g.alpha * acc[i][j][r];
                if (rs) v *= float(rs[m]);
                if (cs) v *= float(cs[n]);
                if (g.beta != 0.0f) v += g.beta * cv[j][r];
                C[m * g.ldc + n] = v;
            }
    }
}

template <typename T>
kq_status gemm(const GemmArgs<T>& g, bool ta, bool tb, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return KQ_OK;
    if (g.focus >= 0 || g.skip_tile2 >= 0) return fail(KQ_EUNSUPPORTED, "gemm: tile focus is fp64-only");
    if constexpr (sizeof(T) == 4) {
        const bool fast = !ta && !tb && !g.tri && !g.kmode && g.skip_tile < 0 && g.K > 0 && g.K % GF_BK == 0 &&
                          g.N % 4 == 0 && aligned16(g.A) && aligned16(g.B) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
                          g.sA1 % 4 == 0 && g.sA2 % 4 == 0 && g.sB1 % 4 == 0 && g.sB2 % 4 == 0;
        if (fast) {
            const int64_t tiles = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
            if (tiles * 256 > 4294967295LL || g.nb1 * g.nb2 > 65535) return fail(KQ_ESHAPE, "gemm grid too large");
            hipLaunchKernelGGL(gemm_f32_nn_kernel, dim3((unsigned)tiles, 1, (unsigned)(g.nb1 * g.nb2)), dim3(256), 0,
                               st, reinterpret_cast<const GemmArgs<float>&>(g));
            return check_launch("gemm_f32_nn");
        }
    }
    constexpr int VN = 16 / sizeof(T);
    const bool vec = aligned16(g.A) && aligned16(g.B) && g.lda % VN == 0 && g.ldb % VN == 0 &&
                     g.sA1 % VN == 0 && g.sA2 % VN == 0 && g.sB1 % VN == 0 && g.sB2 % VN == 0;
    const int64_t nx = (g.N + GBN - 1) / GBN, ny = (g.M + GBM - 1) / GBM;
    if (g.tri && nx != ny) return fail(KQ_ESHAPE, "gemm: triangular products need a square tile grid");
    dim3 grid((unsigned)(g.tri ? nx * (nx + 1) / 2 : nx), (unsigned)(g.tri ? 1 : ny), (unsigned)(g.nb1 * g.nb2));
    if (grid.y > 65535 || grid.z > 65535) return fail(KQ_ESHAPE, "gemm grid too large");
#define KQ_GEMM_LAUNCH(TA_, TB_, V_) hipLaunchKernelGGL((gemm_kernel<T, TA_, TB_, V_>), grid, dim3(256), 0, st, g)
    if (vec) {
        if (!ta && !tb) KQ_GEMM_LAUNCH(false, false, true);
        else if (!ta && tb) KQ_GEMM_LAUNCH(false, true, true);
        else if (ta && !tb) KQ_GEMM_LAUNCH(true, false, true);
        else KQ_GEMM_LAUNCH(true, true, true);
    } else {
        if (!ta && !tb) KQ_GEMM_LAUNCH(false, false, false);
        else if (!ta && tb) KQ_GEMM_LAUNCH(false, true, false);
        else if (ta && !tb) KQ_GEMM_LAUNCH(true, false, false);
        else KQ_GEMM_LAUNCH(true, true, false);
    }
#undef KQ_GEMM_LAUNCH
    return check_launch("gemm");
}
template kq_status gemm<float>(const GemmArgs<float>&, bool, bool, hipStream_t);

// ================================================================================ fp64 GEMM (VALU)
// On gfx950 the fp64 matrix-core instruction (16x16x4) sustains about 36 TFLOP/s even in a
// dependency-free loop, while the fp64 vector FMA pipe sustains about 59 (both measured on MI355X with
// one-kernel probes), so fp64 products run on vector FMAs. 256 threads own a BM x BN tile of C; thread
// (tr, tc) = (tid / 16, tid % 16) keeps a register tile of rows h * BM/2 + tr * RG + i and columns
// h * BN/2 + 32 p + 2 tc + e (h = 0, 1; RG = BM/32; CG = BN/32 columns per half as CG/2 pairs p, e = 0, 1).
// Operands are staged k-major in LDS (double-buffered 16-deep K slices, one barrier per slice) and read
// as 16-byte vectors; the lanes of a wave that share a row group read the same A address (broadcast),
// and the 16 column groups read one contiguous 256-byte run of B per instruction (column pairs 32
// apart: four adjacent columns per thread would put the lanes 32 bytes apart, a two-way bank conflict). Tile order, triangular launch, K restriction and epilogue follow the MFMA
// kernel above.
template <int BM, int BN, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(256) void dgemm_valu_kernel(GemmArgs<double> g) {
    // The launch itself is the signal: this kernel starts only after the kernels before it on its queue
    // have completed. The store releases at device scope, pairing with the waiter's acquire, and comes
    // before the skip test so that a waiter is always released.
    if (g.signal && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        __hip_atomic_store(g.signal, g.signal_value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (g.skip && *g.skip) return;
    constexpr int BK = 16, PAD = 2;  // row stride 130 doubles: the transposing stores of a slice spread over the banks
    constexpr int RG = BM / 32, CG = BN / 32;
    constexpr int VPR = BK / 2;                  // 16-byte vectors per tile row (k direction)
    constexpr int NVA = BM * BK / 2 / 256, NVB = BN * BK / 2 / 256;
    static_assert(NVA >= 1 && NVB >= 1 && RG % 2 == 0 && CG % 2 == 0, "tile shape");
    __shared__ __align__(16) double As[2][BK][BM + PAD];
    __shared__ __align__(16) double Bs[2][BK][BN + PAD];
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    int64_t tm, tn;
    if (g.focus >= 0) {
        // lower triangle: the BM-tile rows of the 128-wide row `focus` (tiles (i, 0..i)), then its
        // BM-tile columns below them
        constexpr int64_t R = 128 / BM;
        const int64_t ntm = (g.M + BM - 1) / BM, f0 = g.focus * R;
        const int64_t rf = ntm - f0 < R ? ntm - f0 : R;
        int64_t lid = blockIdx.x;
        tm = -1;
        tn = 0;
        for (int64_t q = 0; q < rf && tm < 0; q++) {
            if (lid <= f0 + q) { tm = f0 + q; tn = lid; }
            else lid -= f0 + q + 1;
        }
        if (tm < 0) { tm = f0 + rf + lid / rf; tn = f0 + lid % rf; }
    } else if (BM == BN && g.kmode && !g.tri && (!(g.kmode & 10) || !(g.kmode & 5))) {
        // K ranges that depend on the tile (triangular operands) along one of the tile indices: tiles go
        // out longest K first, in the launch order itself (consecutive ids reach the 8 XCDs in turn, so
        // each XCD receives every 8th tile of that order and its share differs from the others' by at
        // most one tile). A K range set by the tile column runs down the columns (all rows of a column
        // share one B panel and one K range); one set by the tile row runs along the rows.
        const int64_t nx = (g.N + BN - 1) / BN, ny = (g.M + BM - 1) / BM;
        const int64_t lid = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        if (g.kmode & 10) {
            tm = lid % ny;
            tn = (g.kmode & 8) ? nx - 1 - lid / ny : lid / ny;
        } else {
            tn = lid % nx;
            tm = (g.kmode & 4) ? ny - 1 - lid / nx : lid / nx;
        }
    } else {
        const int64_t nx = (g.N + BN - 1) / BN;
        const int64_t L = g.tri ? (int64_t)gridDim.x : (int64_t)gridDim.x * gridDim.y;
        int64_t lid = g.tri ? (int64_t)blockIdx.x : (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        // Work-groups go to the 8 XCDs round-robin by id: give XCD x a contiguous run of tiles
        // (a bijection for any L; runs differ in length by at most one), so that tiles sharing a row
        // panel of A meet in one XCD's L2.
        {
            const int64_t x = lid % 8, q = lid / 8, base = L / 8, rem = L % 8;
            lid = x * base + (x < rem ? x : rem) + q;
        }
        if constexpr (BM != BN) {
            tm = lid / nx;  // row-block tiles (own_rows): never triangular
            tn = lid % nx;
        } else if (g.tri) {
            int64_t r = (int64_t)((sqrt(8.0 * (double)lid + 1.0) - 1.0) * 0.5);
            while (r * (r + 1) / 2 > lid) r--;
            while ((r + 1) * (r + 2) / 2 <= lid) r++;
            int64_t c = lid - r * (r + 1) / 2;
            if (g.compact) {
                // the grid enumerates the triangle without the skipped 128-wide rows and columns
                // (BM = BN = 128 here): map the reduced indices back, skipped indices ascending
                const int64_t s1 = g.skip_tile, s2 = g.skip_tile2;
                const int64_t lo = (s1 >= 0 && (s2 < 0 || s1 <= s2)) ? s1 : s2;
                const int64_t hi = (lo == s1) ? s2 : s1;
                if (lo >= 0) { r += r >= lo; c += c >= lo; }
                if (hi >= 0 && hi != lo) { r += r >= hi; c += c >= hi; }
            }
            if (g.tri == 1) { tm = r; tn = c; } else { tm = c; tn = r; }
        } else {
            tm = lid / nx;
            tn = lid % nx;
        }
    }
    // the tile indices are uniform over the work-group: keep them (and what derives from them) in
    // scalar registers, which leaves the vector registers to the accumulators and operands
    tm = (int64_t)__builtin_amdgcn_readfirstlane((int)tm);
    tn = (int64_t)__builtin_amdgcn_readfirstlane((int)tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    if (g.skip_tile >= 0 && ((m0 >> 7) == g.skip_tile || (n0 >> 7) == g.skip_tile)) return;
    if (g.skip_tile2 >= 0 && ((m0 >> 7) == g.skip_tile2 || (n0 >> 7) == g.skip_tile2)) return;
    const int64_t z = blockIdx.z, z1 = z / g.nb2, z2 = z % g.nb2;
    const double* __restrict__ A = g.A + z1 * g.sA1 + z2 * g.sA2;
    const double* __restrict__ B = g.B + z1 * g.sB1 + z2 * g.sB2;
    double* C = g.C + z1 * g.sC1 + z2 * g.sC2;
    const int8_t* rs = g.rsign ? g.rsign + z1 * g.sR1 + z2 * g.sR2 : nullptr;
    const int8_t* cs = g.csign ? g.csign + z1 * g.sS1 + z2 * g.sS2 : nullptr;
    const int64_t M = g.M, N = g.N;
    int64_t kb = 0, ke = g.K;
    if (g.kmode & 1) kb = kb > m0 ? kb : m0;
    if (g.kmode & 2) kb = kb > n0 ? kb : n0;
    if (g.kmode & 4) ke = ke < m0 + BM ? ke : m0 + BM;
    if (g.kmode & 8) ke = ke < n0 + BN ? ke : n0 + BN;
    kb = (kb / BK) * BK;

    double acc[2][RG][2][CG];
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < RG; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < CG; j++) acc[hi][i][hj][j] = 0.0;

    double ra[NVA][2], rb[NVB][2];
    const bool fullMN = (m0 + BM <= M) && (n0 + BN <= N);
    const bool cvec = ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && ((g.ldc & 1) == 0);
    const bool vec_epi = cvec && fullMN && !rs && !cs && (g.tri == 0 || tm != tn);
    // C - A B accumulated from -C: the tile's read of C comes first (work-groups alternate, by their
    // place in their XCD's run, between reading C first and last)
    const bool pre = g.stagger && vec_epi && g.alpha == -1.0 && g.beta == 1.0 &&
                     ((blockIdx.x >> 3) & 1) && kb < ke;
    if (pre) {
#pragma unroll
        for (int hi = 0; hi < 2; hi++)
#pragma unroll
            for (int i = 0; i < RG; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < CG; j += 2) {
                        const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                        const V16<double> t = *reinterpret_cast<const V16<double>*>(C + m * g.ldc + n);
                        acc[hi][i][hj][j] = -t.v[0];
                        acc[hi][i][hj][j + 1] = -t.v[1];
                    }
    }
    auto gload = [&](int64_t k0) {
        const bool full = VEC && fullMN && (k0 + BK <= ke);
#pragma unroll
        for (int q = 0; q < NVA; q++) {
            const int v = tid + 256 * q;
            int64_t gm, gk;
            if (!TA) { gm = m0 + v / VPR; gk = k0 + (v % VPR) * 2; }
            else { gk = k0 + v / (BM / 2); gm = m0 + (v % (BM / 2)) * 2; }
            const double* p = TA ? A + gk * g.lda + gm : A + gm * g.lda + gk;
            if (full) {
                const V16<double> t = *reinterpret_cast<const V16<double>*>(p);
                ra[q][0] = t.v[0]; ra[q][1] = t.v[1];
            } else {
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const bool in = TA ? (gk < ke && gm + e < M) : (gm < M && gk + e < ke);
                    ra[q][e] = in ? p[e] : 0.0;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NVB; q++) {
            const int v = tid + 256 * q;
            int64_t gn, gk;
            if (TB) { gn = n0 + v / VPR; gk = k0 + (v % VPR) * 2; }
            else { gk = k0 + v / (BN / 2); gn = n0 + (v % (BN / 2)) * 2; }
            const double* p = TB ? B + gn * g.ldb + gk : B + gk * g.ldb + gn;
            if (full) {
                const V16<double> t = *reinterpret_cast<const V16<double>*>(p);
                rb[q][0] = t.v[0]; rb[q][1] = t.v[1];
            } else {
#pragma unroll
                for (int e = 0; e < 2; e++) {
                    const bool in = TB ? (gn < N && gk + e < ke) : (gk < ke && gn + e < N);
                    rb[q][e] = in ? p[e] : 0.0;
                }
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NVA; q++) {
            const int v = tid + 256 * q;
            if (!TA) {
                As[buf][(v % VPR) * 2][v / VPR] = ra[q][0];
                As[buf][(v % VPR) * 2 + 1][v / VPR] = ra[q][1];
            } else {
                *reinterpret_cast<V16<double>*>(&As[buf][v / (BM / 2)][(v % (BM / 2)) * 2]) = V16<double>{{ra[q][0], ra[q][1]}};
            }
        }
#pragma unroll
        for (int q = 0; q < NVB; q++) {
            const int v = tid + 256 * q;
            if (TB) {
                Bs[buf][(v % VPR) * 2][v / VPR] = rb[q][0];
                Bs[buf][(v % VPR) * 2 + 1][v / VPR] = rb[q][1];
            } else {
                *reinterpret_cast<V16<double>*>(&Bs[buf][v / (BN / 2)][(v % (BN / 2)) * 2]) = V16<double>{{rb[q][0], rb[q][1]}};
            }
        }
    };

    if (kb < ke) {
        // A K range that starts at the tile (and ends where its neighbours' do) is walked from its end
        // down: tiles that share an operand panel then read each slice of it at about the same time
        const int64_t nsl = (ke - kb + BK - 1) / BK;
        const bool krev = (g.kmode & 3) && !(g.kmode & 12);
        const int64_t dk = krev ? -BK : BK;
        int64_t k0 = krev ? kb + (nsl - 1) * BK : kb;
        gload(k0);
        sstore(0);
        __syncthreads();
        int buf = 0;
        for (int64_t sl = 0; sl < nsl; sl++, k0 += dk) {
            const bool more = sl + 1 < nsl;
            if (more) gload(k0 + dk);
#pragma unroll 2
            for (int kk = 0; kk < BK; kk++) {
                double a[2][RG], b[2][CG];
#pragma unroll
                for (int h = 0; h < 2; h++) {
#pragma unroll
                    for (int i = 0; i < RG; i += 2) {
                        const V16<double> t = *reinterpret_cast<const V16<double>*>(&As[buf][kk][h * (BM / 2) + tr * RG + i]);
                        a[h][i] = t.v[0]; a[h][i + 1] = t.v[1];
                    }
#pragma unroll
                    for (int j = 0; j < CG; j += 2) {
                        const V16<double> t = *reinterpret_cast<const V16<double>*>(&Bs[buf][kk][h * (BN / 2) + (j >> 1) * 32 + 2 * tc]);
                        b[h][j] = t.v[0]; b[h][j + 1] = t.v[1];
                    }
                }
#pragma unroll
                for (int hi = 0; hi < 2; hi++)
#pragma unroll
                    for (int i = 0; i < RG; i++)
#pragma unroll
                        for (int hj = 0; hj < 2; hj++)
#pragma unroll
                            for (int j = 0; j < CG; j++) acc[hi][i][hj][j] = fma(a[hi][i], b[hj][j], acc[hi][i][hj][j]);
            }
            if (more) sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    // Epilogue. Full tiles that lie inside the stored triangle, without sign vectors, take 16-byte
    // loads and stores of C; every other tile goes element by element with the bounds checks.
    if (pre) {
        // acc = A B - C: store -acc
#pragma unroll
        for (int hi = 0; hi < 2; hi++)
#pragma unroll
            for (int i = 0; i < RG; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < CG; j += 2) {
                        const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                        *reinterpret_cast<V16<double>*>(C + m * g.ldc + n) =
                            V16<double>{{-acc[hi][i][hj][j], -acc[hi][i][hj][j + 1]}};
                    }
        return;
    }
    if (vec_epi) {
        const double alpha = g.alpha, beta = g.beta;
#pragma unroll
        for (int hi = 0; hi < 2; hi++) {
            V16<double> cv[RG][2][CG / 2];
            if (beta != 0.0) {
#pragma unroll
                for (int i = 0; i < RG; i++)
#pragma unroll
                    for (int hj = 0; hj < 2; hj++)
#pragma unroll
                        for (int j = 0; j < CG; j += 2) {
                            const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                            cv[i][hj][j / 2] = *reinterpret_cast<const V16<double>*>(C + m * g.ldc + n);
                        }
            }
#pragma unroll
            for (int i = 0; i < RG; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < CG; j += 2) {
                        const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                        V16<double> v;
                        v.v[0] = alpha * acc[hi][i][hj][j];
                        v.v[1] = alpha * acc[hi][i][hj][j + 1];
                        if (beta != 0.0) {
                            v.v[0] = fma(beta, cv[i][hj][j / 2].v[0], v.v[0]);
                            v.v[1] = fma(beta, cv[i][hj][j / 2].v[1], v.v[1]);
                        }
                        *reinterpret_cast<V16<double>*>(C + m * g.ldc + n) = v;
                    }
        }
        return;
    }
#pragma unroll
    for (int hi = 0; hi < 2; hi++) {
        double cv[RG][2][CG];
        if (g.beta != 0.0) {
#pragma unroll
            for (int i = 0; i < RG; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < CG; j++) {
                        const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                        cv[i][hj][j] = (m < M && n < N) ? C[m * g.ldc + n] : 0.0;
                    }
        }
#pragma unroll
        for (int i = 0; i < RG; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < CG; j++) {
                    const int64_t m = m0 + hi * (BM / 2) + tr * RG + i, n = n0 + hj * (BN / 2) + (j >> 1) * 32 + 2 * tc + (j & 1);
                    if (m >= M || n >= N) continue;
                    if (g.tri == 1 && n > m) continue;
                    if (g.tri == 2 && m > n) continue;
                    double v = g.alpha * acc[hi][i][hj][j];
                    if (rs) v *= (double)rs[m];
                    if (cs) v *= (double)cs[n];
                    if (g.beta != 0.0) v += g.beta * cv[i][hj][j];
                    C[m * g.ldc + n] = v;
                }
    }
}

template <int BM, int BN>
static void dgemm_launch(const GemmArgs<double>& g0, bool ta, bool tb, bool vec, hipStream_t st) {
    GemmArgs<double> g = g0;
    const int64_t nx = (g.N + BN - 1) / BN, ny = (g.M + BM - 1) / BM;
    int64_t gx = g.tri ? nx * (nx + 1) / 2 : nx;
    g.compact = 0;
    if (BM == 128 && BN == 128 && g.tri && g.focus < 0) {
        // leave the skipped tile rows and columns out of the grid: the work-groups that would only
        // return would otherwise count against each XCD's share of the chip
        const int64_t s1 = g.skip_tile, s2 = g.skip_tile2;
        const int64_t ns = (s1 >= 0 && s1 < nx) + (s2 >= 0 && s2 < nx && s2 != s1);
        if (ns > 0) {
            if (s1 >= nx) g.skip_tile = -1;
            if (s2 >= nx || s2 == s1) g.skip_tile2 = -1;
            const int64_t nr = nx - ns;
            gx = nr * (nr + 1) / 2;
            g.compact = 1;
            if (gx == 0) return;
        }
    }
    if (g.focus >= 0) {  // tiles of the focus rows, then the focus columns below them
        const int64_t R = 128 / BM, f0 = g.focus * R, rf = ny - f0 < R ? ny - f0 : R;
        gx = 0;
        for (int64_t q = 0; q < rf; q++) gx += f0 + q + 1;
        gx += rf * (ny - f0 - rf);
    }
    const dim3 grid((unsigned)gx, (unsigned)(g.tri ? 1 : ny), (unsigned)(g.nb1 * g.nb2));
#define KQ_DG(TA_, TB_, V_) hipLaunchKernelGGL((dgemm_valu_kernel<BM, BN, TA_, TB_, V_>), grid, dim3(256), 0, st, g)
    if (vec) {
        if (!ta && !tb) KQ_DG(false, false, true);
        else if (!ta && tb) KQ_DG(false, true, true);
        else if (ta && !tb) KQ_DG(true, false, true);
        else KQ_DG(true, true, true);
    } else {
        if (!ta && !tb) KQ_DG(false, false, false);
        else if (!ta && tb) KQ_DG(false, true, false);
        else if (ta && !tb) KQ_DG(true, false, false);
        else KQ_DG(true, true, false);
    }
#undef KQ_DG
}

// 128 x 128 tiles when they fill the chip (256 compute units), 64 x 64 otherwise.
template <>
kq_status gemm<double>(const GemmArgs<double>& g, bool ta, bool tb, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return KQ_OK;
    const bool vec = aligned16(g.A) && aligned16(g.B) && g.lda % 2 == 0 && g.ldb % 2 == 0 && g.sA1 % 2 == 0 &&
                     g.sA2 % 2 == 0 && g.sB1 % 2 == 0 && g.sB2 % 2 == 0;
    const int64_t batch = g.nb1 * g.nb2;
    if (batch > 65535) return fail(KQ_ESHAPE, "gemm: batch too large");
    const int64_t nx = (g.N + 127) / 128, ny = (g.M + 127) / 128;
    if (g.tri && nx != ny) return fail(KQ_ESHAPE, "gemm: triangular products need a square tile grid");
    if (g.focus >= 0 && (g.tri != 1 || g.focus >= nx)) return fail(KQ_EINVAL, "gemm: bad tile focus");
    const int64_t tiles = (g.tri ? nx * (nx + 1) / 2 : nx * ny) * batch;
    const bool big = tiles >= 256 && g.focus < 0;
    const int64_t ty = big ? ny : (g.M + 63) / 64;
    if (!g.tri && ty > 65535) return fail(KQ_ESHAPE, "gemm grid too large");
    if (g.tri && ((g.N + 63) / 64) != ((g.M + 63) / 64)) return fail(KQ_ESHAPE, "gemm: triangular products need a square tile grid");
    if (g.own_rows) {
        if (g.tri || g.focus >= 0 || g.N > 128) return fail(KQ_EINVAL, "gemm: row-block tiles need N <= 128");
        dgemm_launch<64, 128>(g, ta, tb, vec, st);
    } else if (big) dgemm_launch<128, 128>(g, ta, tb, vec, st);
    else dgemm_launch<64, 64>(g, ta, tb, vec, st);
    return check_launch("dgemm");
}

// ========================================================================================= helpers
template <typename T>
__global__ void fill_kernel(T* p, size_t count, T value, const int* skip) {
    if (skip && *skip) return;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < count; e += (size_t)gridDim.x * blockDim.x)
        p[e] = value;
}

template <typename T>
kq_status fill(T* p, size_t count, T value, hipStream_t st, const int* skip) {
    if (!count) return KQ_OK;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, p, count, value, skip);
    return check_launch("fill");
}
template kq_status fill<float>(float*, size_t, float, hipStream_t, const int*);
template kq_status fill<double>(double*, size_t, double, hipStream_t, const int*);
template kq_status fill<int>(int*, size_t, int, hipStream_t, const int*);
template kq_status fill<uint32_t>(uint32_t*, size_t, uint32_t, hipStream_t, const int*);

// ============================================================================== Cholesky, blocked
template <>
int potrf_nb<float>() { return 128; }
template <>
int potrf_nb<double>() { return 128; }

// One work-group per batch item factors the NB x NB diagonal block at (k0, k0) in LDS (16-column
// sub-panels: a single wave factors the sub-panel with shuffles, then all threads apply the rank-16
// update with 4 x 4 register micro-tiles), writes L back to A, and writes L^{-1} (computed in LDS
// by forward substitution on 16 x 16 diagonal sub-blocks and recursive doubling
// X21 = -X22 L21 X11) to X. Rows beyond n are padded with the identity.
template <typename T, int NB>
__global__ __launch_bounds__(256) void potrf_diag_kernel(T* A, int64_t lda, int64_t sA, T* X, int64_t ldx, int64_t sX,
                                                         int64_t n, int64_t k0, int32_t* info, int64_t info_stride,
                                                         double* logdet, const int* skip) {
    if (skip && *skip) return;
    constexpr int LD = NB + 1;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* L = reinterpret_cast<T*>(smem_raw);
    T* Xs = L + NB * LD;
    __shared__ int failed, fail_idx;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t z = blockIdx.x;
    A += z * sA + k0 * lda + k0;
    X += z * sX + k0 * ldx + k0;
    const int nbe = (int)((n - k0) < NB ? (n - k0) : NB);
    for (int e = tid; e < NB * NB; e += 256) {
        const int r = e / NB, c = e % NB;
        T v;
        if (r < nbe && c < nbe) v = (c <= r) ? A[(int64_t)r * lda + c] : T(0);
        else v = (r == c) ? T(1) : T(0);
        L[r * LD + c] = v;
        Xs[r * LD + c] = T(0);
    }
    if (tid == 0) { failed = 0; fail_idx = 0; }
    __syncthreads();

    for (int c0 = 0; c0 < NB; c0 += 16) {
        if (wave == 0) {
            T val[2][16];
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int r = c0 + lane + 64 * t;
#pragma unroll
                for (int cc = 0; cc < 16; cc++) val[t][cc] = (r < NB) ? L[r * LD + c0 + cc] : T(0);
            }
#pragma unroll
            for (int cc = 0; cc < 16; cc++) {
                const T piv = __shfl(val[0][cc], cc);
                const bool bad = !(piv > T(0));
                if (bad && lane == 0 && !failed) { failed = 1; fail_idx = c0 + cc; }
                const T d = sqrt(bad ? T(1) : piv);
                const T inv = T(1) / d;
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const int r = c0 + lane + 64 * t;
                    if (r == c0 + cc) val[t][cc] = d;
                    else if (r > c0 + cc) val[t][cc] *= inv;
                }
#pragma unroll
                for (int c2 = cc + 1; c2 < 16; c2++) {
                    const T l2 = __shfl(val[0][cc], c2);
#pragma unroll
                    for (int t = 0; t < 2; t++) {
                        const int r = c0 + lane + 64 * t;
                        if (r >= c0 + c2) val[t][c2] -= val[t][cc] * l2;
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int r = c0 + lane + 64 * t;
                if (r < NB) {
#pragma unroll
                    for (int cc = 0; cc < 16; cc++)
                        if (r >= c0 + cc) L[r * LD + c0 + cc] = val[t][cc];
                }
            }
        }
        __syncthreads();
        const int base = c0 + 16, rem = NB - base;
        if (rem > 0) {
            const int mt = rem / 4;  // micro-tiles per side (rem is a multiple of 16)
            for (int e = tid; e < mt * mt; e += 256) {
                const int br = e / mt, bc = e % mt;
                if (bc > br) continue;
                const int r = base + 4 * br, c = base + 4 * bc;
                T s[4][4] = {};
#pragma unroll
                for (int t = 0; t < 16; t++) {
                    T a[4], b[4];
#pragma unroll
                    for (int u = 0; u < 4; u++) { a[u] = L[(r + u) * LD + c0 + t]; b[u] = L[(c + u) * LD + c0 + t]; }
#pragma unroll
                    for (int u = 0; u < 4; u++)
#pragma unroll
                        for (int w = 0; w < 4; w++) s[u][w] += a[u] * b[w];
                }
#pragma unroll
                for (int u = 0; u < 4; u++)
#pragma unroll
                    for (int w = 0; w < 4; w++)
                        if (c + w <= r + u) L[(r + u) * LD + c + w] -= s[u][w];
            }
        }
        __syncthreads();
    }

    // ---- L^{-1}: 16 x 16 diagonal sub-blocks by forward substitution (one thread per column)
    if (tid < NB) {
        const int b = tid >> 4, c = tid & 15, bs = 16 * b;
        T x[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            T s = (r == c) ? T(1) : T(0);
#pragma unroll
            for (int t = 0; t < r; t++) s -= L[(bs + r) * LD + bs + t] * x[t];
            x[r] = (r >= c) ? s / L[(bs + r) * LD + bs + r] : T(0);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) Xs[(bs + r) * LD + bs + c] = x[r];
    }
    __syncthreads();
    // ---- recursive doubling: X21 = -X22 (L21 X11), temporaries in the (zero) upper block
    for (int s = 16; s < NB; s *= 2) {
        const int np = NB / (2 * s), cnt = np * s * s;
        for (int e = tid; e < cnt; e += 256) {
            const int p = e / (s * s), rr = (e / s) % s, cc = e % s, r0 = 2 * p * s;
            T a = 0;
            for (int k = cc; k < s; k++) a += L[(r0 + s + rr) * LD + r0 + k] * Xs[(r0 + k) * LD + r0 + cc];
            Xs[(r0 + rr) * LD + r0 + s + cc] = a;
        }
        __syncthreads();
        for (int e = tid; e < cnt; e += 256) {
            const int p = e / (s * s), rr = (e / s) % s, cc = e % s, r0 = 2 * p * s;
            T a = 0;
            for (int k = 0; k <= rr; k++) a += Xs[(r0 + s + rr) * LD + r0 + s + k] * Xs[(r0 + k) * LD + r0 + s + cc];
            Xs[(r0 + s + rr) * LD + r0 + cc] = -a;
        }
        __syncthreads();
        for (int e = tid; e < cnt; e += 256) {
            const int p = e / (s * s), rr = (e / s) % s, cc = e % s, r0 = 2 * p * s;
            Xs[(r0 + rr) * LD + r0 + s + cc] = T(0);
        }
        __syncthreads();
    }

    for (int e = tid; e < nbe * nbe; e += 256) {
        const int r = e / nbe, c = e % nbe;
        if (c <= r) {
            A[(int64_t)r * lda + c] = L[r * LD + c];
            X[(int64_t)r * ldx + c] = Xs[r * LD + c];
        }
    }
    if (tid == 0) {
        if (logdet) {
            double s = 0;
            for (int r = 0; r < nbe; r++) s += log((double)L[r * LD + r]);
            logdet[z] += s;
        }
        if (failed && info && fail_idx < nbe && info[z * info_stride] == 0)
            info[z * info_stride] = (int32_t)(k0 + fail_idx + 1);
    }
}

template <typename T, int NB>
static kq_status launch_diag(T* A, int64_t lda, int64_t sA, T* X, int64_t ldx, int64_t sX, int64_t n, int64_t k0,
                             int64_t batch, int32_t* info, int64_t info_stride, double* logdet, const int* skip,
                             hipStream_t st) {
    const size_t smem = size_t(2) * NB * (NB + 1) * sizeof(T);
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(&potrf_diag_kernel<T, NB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        attr = true;
    }
    hipLaunchKernelGGL((potrf_diag_kernel<T, NB>), dim3((unsigned)batch), dim3(256), smem, st, A, lda, sA, X, ldx, sX,
                       n, k0, info, info_stride, logdet, skip);
    return check_launch("potrf_diag");
}

template <typename T>
kq_status potrf_batched(T* A, int64_t lda, int64_t sA, T* X, int64_t ldx, int64_t sX, int64_t n, int64_t batch,
                        int32_t* info, int64_t info_stride, double* logdet, const int* skip, hipStream_t st,
                        double* scr) {
    const int NB = potrf_nb<T>();
    if (batch > 65535) return fail(KQ_ESHAPE, "potrf batch too large");
    for (int64_t k0 = 0; k0 < n; k0 += NB) {
        const int64_t nbe = (n - k0) < NB ? (n - k0) : NB, k1 = k0 + nbe;
        if (sizeof(T) == 4)
            KQ_TRY((launch_diag<T, 128>(A, lda, sA, X, ldx, sX, n, k0, batch, info, info_stride, logdet, skip, st)));
        else if (!logdet)
            KQ_TRY(chol_inv_diag128(reinterpret_cast<double*>(A), lda, sA, reinterpret_cast<double*>(X), ldx, sX, n,
                                    k0, batch, scr, info, info_stride, skip, st));
        else
            return fail(KQ_EUNSUPPORTED, "potrf: fp64 log-determinant not supported");
        if (k1 >= n) break;
        // panel: A[k1:, k0:k1] <- A[k1:, k0:k1] X_kk^T in place, so each work-group must own whole
        // rows of the panel (it reads only the rows it writes): 128-wide column tiles
        GemmArgs<T> p = gemm_args<T>(n - k1, nbe, nbe, A + k1 * lda + k0, lda, X + k0 * ldx + k0, ldx,
                                     A + k1 * lda + k0, lda, T(1), T(0));
        p.nb1 = batch; p.sA1 = sA; p.sB1 = sX; p.sC1 = sA; p.skip = skip; p.own_rows = 1;
        KQ_TRY(gemm<T>(p, false, true, st));
        // trailing: A[k1:, k1:] -= P P^T (lower triangle)
        GemmArgs<T> u = gemm_args<T>(n - k1, n - k1, nbe, A + k1 * lda + k0, lda, A + k1 * lda + k0, lda,
                                     A + k1 * lda + k1, lda, T(-1), T(1));
        u.nb1 = batch; u.sA1 = sA; u.sB1 = sA; u.sC1 = sA; u.tri = 1; u.skip = skip;
        KQ_TRY(gemm<T>(u, false, true, st));
    }
    return KQ_OK;
}
template kq_status potrf_batched<float>(float*, int64_t, int64_t, float*, int64_t, int64_t, int64_t, int64_t, int32_t*,
                                        int64_t, double*, const int*, hipStream_t, double*);
template kq_status potrf_batched<double>(double*, int64_t, int64_t, double*, int64_t, int64_t, int64_t, int64_t,
                                         int32_t*, int64_t, double*, const int*, hipStream_t, double*);

template <typename T>
kq_status trtri_batched(const T* L, int64_t ldl, int64_t sL, T* X, int64_t ldx, int64_t sX, int64_t n, int64_t batch,
                        T* Tscr, const int* skip, hipStream_t st) {
    const int64_t NB = potrf_nb<T>();
    const int64_t sT = n * n / 2 + NB * NB;
    for (int64_t s = NB; s < n; s *= 2) {
        const int64_t np = n / (2 * s);
        const int64_t r0r = np * 2 * s, s2r = n - r0r - s;  // ragged pair (if s2r > 0)
        for (int pass = 0; pass < 2; pass++) {
            const int64_t cnt = pass == 0 ? np : (s2r > 0 ? 1 : 0);
            if (!cnt) continue;
            const int64_t r0 = pass == 0 ? 0 : r0r, s2 = pass == 0 ? s : s2r;
            // T = L21 X11
            GemmArgs<T> a = gemm_args<T>(s2, s, s, L + (r0 + s) * ldl + r0, ldl, X + r0 * ldx + r0, ldx,
                                         Tscr + (pass == 0 ? 0 : np * s * s), s, T(1), T(0));
            a.nb1 = batch; a.nb2 = cnt; a.sA1 = sL; a.sA2 = 2 * s * (ldl + 1); a.sB1 = sX; a.sB2 = 2 * s * (ldx + 1);
            a.sC1 = sT; a.sC2 = s * s; a.kmode = 2; a.skip = skip;
            KQ_TRY(gemm<T>(a, false, false, st));
            // X21 = -X22 T
            GemmArgs<T> b = gemm_args<T>(s2, s, s2, X + (r0 + s) * ldx + (r0 + s), ldx, Tscr + (pass == 0 ? 0 : np * s * s),
                                         s, X + (r0 + s) * ldx + r0, ldx, T(-1), T(0));
            b.nb1 = batch; b.nb2 = cnt; b.sA1 = sX; b.sA2 = 2 * s * (ldx + 1); b.sB1 = sT; b.sB2 = s * s;
            b.sC1 = sX; b.sC2 = 2 * s * (ldx + 1); b.kmode = 4; b.skip = skip;
            KQ_TRY(gemm<T>(b, false, false, st));
        }
    }
    return KQ_OK;
}
template kq_status trtri_batched<float>(const float*, int64_t, int64_t, float*, int64_t, int64_t, int64_t, int64_t,
                                        float*, const int*, hipStream_t);
template kq_status trtri_batched<double>(const double*, int64_t, int64_t, double*, int64_t, int64_t, int64_t, int64_t,
                                         double*, const int*, hipStream_t);

}  // namespace kq

using namespace kq;

// ==================================================================================== kq_cholinv
// lambda = damp * mean(diag H) in fp64 with a fixed reduction order (one work-group).
__global__ void damp_kernel(const double* H, int64_t n, int64_t ldh, double damp, double* lam, int32_t* info) {
    __shared__ double part[256];
    double s = 0;
    for (int64_t r = threadIdx.x; r < n; r += 256) s += H[r * ldh + r];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *lam = damp * part[0] / (double)n;
        *info = 0;
    }
}

// Hr[a][b] = H[n-1-a][n-1-b] + lambda [a == b] in fp64, lower triangle only (read from H's lower
// triangle: H[n-1-b][n-1-a]). 64 x 64 tiles of Hr through LDS, so that the reads run along rows of H
// and the writes along rows of Hr; tiles above the diagonal return at once.
__global__ __launch_bounds__(256) void reverse_damped_kernel(const double* H, int64_t n, int64_t ldh, const double* lam,
                                                             double* Hr) {
    __shared__ double t[64][65];
    const int64_t a0 = (int64_t)blockIdx.y * 64, b0 = (int64_t)blockIdx.x * 64;
    if (b0 > a0) return;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t a = a0 + 63 - tx;  // lane tx reads column n-1-a of H: consecutive lanes, consecutive columns
    for (int j = ty; j < 64; j += 4) {
        const int64_t b = b0 + j;
        if (a < n && b < n && b <= a) t[63 - tx][j] = H[(n - 1 - b) * ldh + (n - 1 - a)];
    }
    __syncthreads();
    const double l = *lam;
    for (int i = ty; i < 64; i += 4) {
        const int64_t ar = a0 + i, b = b0 + tx;
        if (ar < n && b <= ar) Hr[ar * n + b] = t[i][tx] + (ar == b ? l : 0.0);
    }
}

// R[a][b] = X[n-1-a][n-1-b] for a <= b (rounded to fp32), 0 below the diagonal. For n a multiple of 4
// (and R 16-byte aligned) each thread takes four consecutive b: one 16-byte store of R, two 16-byte
// loads of X.
__global__ void reverse_upper_kernel(const double* X, int64_t n, float* R) {
    const int64_t a = blockIdx.y;
    if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(R) & 15) == 0) {
        const double* xr = X + (n - 1 - a) * n;
        for (int64_t b = 4 * (blockIdx.x * 256 + threadIdx.x); b < n; b += (int64_t)gridDim.x * 1024) {
            float4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (b + 3 >= a) {
                const double2 hi = *reinterpret_cast<const double2*>(xr + (n - 2 - b));   // columns n-2-b, n-1-b
                const double2 lo = *reinterpret_cast<const double2*>(xr + (n - 4 - b));   // columns n-4-b, n-3-b
                v.x = b >= a ? (float)hi.y : 0.0f;
                v.y = b + 1 >= a ? (float)hi.x : 0.0f;
                v.z = b + 2 >= a ? (float)lo.y : 0.0f;
                v.w = (float)lo.x;
            }
            *reinterpret_cast<float4*>(R + a * n + b) = v;
        }
        return;
    }
    for (int64_t b = blockIdx.x * 256 + threadIdx.x; b < n; b += (int64_t)gridDim.x * 256)
        R[a * n + b] = (b >= a) ? (float)X[(n - 1 - a) * n + (n - 1 - b)] : 0.0f;
}

// Lower Cholesky of one n x n fp64 matrix A (lda = n, lower triangle) with the inverses of its 128-wide
// diagonal blocks in X, blocked in two levels: the columns of a W-wide panel are factored by 128-wide
// steps whose rank-128 updates reach only the panel's own columns (all rows below), and the matrix right
// of the panel then receives the whole panel in one update with K = W. Most of the n^3/3 FLOP thus run
// in deep-K products instead of rank-128 ones (W = n: one panel, every update rank-128).
// For even n each step's update inside the panel is one launch with the sweep of the next diagonal
// block (chol_step_fused): the sweep, which needs one compute unit for ~75 us, runs beside the update
// instead of after it. Only the first block of a panel is swept alone, after the panel's big update.
// Measured on MI355X (before the fused steps): layer steps with widths 13824 and 8192 took 2.2 and 1.5
// ms less with panels than with one step of look-ahead (the diagonal block factored on a side queue
// beside the trailing update: its kernel needs a whole compute unit and waited for one while the update
// filled the chip). Panel widths measured on MI355X: 2048 took less than 512, 1024 and 4096 on the
// widths 13824 and 8192 (damped factor 53.4 and 17.5 ms with 1024-wide panels, 52.7 and 17.0 with
// 2048); below 6144 panels took longer than the single 128-wide steps.
constexpr int64_t PANEL_W = 2048, PANELS_FROM = 6144;
static kq_status potrf_panels(double* A, int64_t n, int64_t W, double* X, int32_t* info, double* scr, hipStream_t st) {
    constexpr int64_t NB = 128;
    const bool fuse = (n & 1) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
    bool swept = false;  // the diagonal block at k0 was swept by the fused step before it
    for (int64_t J0 = 0; J0 < n; J0 += W) {
        const int64_t J1 = J0 + W < n ? J0 + W : n;
        for (int64_t k0 = J0; k0 < J1; k0 += NB) {
            const int64_t k1 = k0 + NB < J1 ? k0 + NB : J1;
            if (swept) KQ_TRY(chol_extract_diag128(A, n, X, n, n, k0, scr, st));
            else KQ_TRY(chol_inv_diag128(A, n, 0, X, n, 0, n, k0, 1, scr, info, 0, nullptr, st));
            swept = false;
            if (k1 >= n) break;
            // A[k1:, k0:k1] <- A[k1:, k0:k1] X_kk^T in place (each work-group owns whole rows)
            GemmArgs<double> p = gemm_args<double>(n - k1, k1 - k0, k1 - k0, A + k1 * n + k0, n, X + k0 * n + k0, n,
                                                   A + k1 * n + k0, n, 1.0, 0.0);
            p.own_rows = 1;
            KQ_TRY(gemm<double>(p, false, true, st));
            // the rest of the panel: A[k1:, k1:J1] -= L[k1:, k0:k1] L[k1:J1, k0:k1]^T
            if (k1 < J1 && fuse) {
                KQ_TRY(chol_step_fused(A, n, n, k0, J1, scr, info, st));
                swept = true;
            } else if (k1 < J1) {
                // (the part of its diagonal block above the diagonal is written too; only lower
                // triangles are ever read)
                GemmArgs<double> u = gemm_args<double>(n - k1, J1 - k1, k1 - k0, A + k1 * n + k0, n, A + k1 * n + k0, n,
                                                       A + k1 * n + k1, n, -1.0, 1.0);
                KQ_TRY(gemm<double>(u, false, true, st));
            }
        }
        // right of the panel: A[J1:, J1:] -= L[J1:, J0:J1] L[J1:, J0:J1]^T (lower)
        if (J1 < n) {
            GemmArgs<double> u = gemm_args<double>(n - J1, n - J1, J1 - J0, A + J1 * n + J0, n, A + J1 * n + J0, n,
                                                   A + J1 * n + J1, n, -1.0, 1.0);
            u.tri = 1;
            KQ_TRY(gemm<double>(u, false, true, st));
        }
    }
    return KQ_OK;
}

static void cholinv_layout(Sizer& z, int64_t n) {
    z.take<double>(1);
    z.take<double>((size_t)n * n);
    z.take<double>((size_t)n * n);
    z.take<double>((size_t)(n * n / 2 + 128 * 128));
    z.take<double>((size_t)chol_scratch_doubles());
}

size_t cholinv_ws(int64_t n) {
    Sizer z;
    cholinv_layout(z, n);
    return z.used;
}

extern "C" kq_status kq_cholinv(const double* HX, int64_t n, int64_t ldh, double damp, float* R, int32_t* info,
                                void* ws, size_t ws_bytes, kq_stream stream) {
    if (!HX || !R || !info) return fail(KQ_EINVAL, "kq_cholinv: null pointer");
    if (n <= 0 || ldh < n) return fail(KQ_ESHAPE, "kq_cholinv: bad size n=%lld ldh=%lld", (long long)n, (long long)ldh);
    if (!(damp >= 0.0)) return fail(KQ_EINVAL, "kq_cholinv: damp must be >= 0");
    if (ws_bytes < cholinv_ws(n) || !ws) return fail(KQ_EWORKSPACE, "kq_cholinv: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    double* lam = ar.take<double>(1);
    double* Hr = ar.take<double>((size_t)n * n);
    double* X = ar.take<double>((size_t)n * n);
    double* Tscr = ar.take<double>((size_t)(n * n / 2 + 128 * 128));
    double* Cscr = ar.take<double>((size_t)chol_scratch_doubles());
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, HX, n, ldh, damp, lam, info);
    KQ_TRY(check_launch("damp"));
    dim3 g2((unsigned)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), (unsigned)n);
    if (n > 65535) return fail(KQ_ESHAPE, "kq_cholinv: n too large");
    const unsigned nt64 = (unsigned)((n + 63) / 64);
    hipLaunchKernelGGL(reverse_damped_kernel, dim3(nt64, nt64), dim3(256), 0, st, HX, n, ldh, lam, Hr);
    KQ_TRY(check_launch("reverse"));
    // X needs no clearing: the diagonal-block steps write whole 128-wide blocks (zero above the
    // diagonal), the triangular inverse whole blocks below them, and nothing reads above them
    if (n >= PANELS_FROM) KQ_TRY(potrf_panels(Hr, n, PANEL_W, X, info, Cscr, st));
    else if (n % 2 == 0) KQ_TRY(potrf_panels(Hr, n, n, X, info, Cscr, st));
    else KQ_TRY(potrf_batched<double>(Hr, n, 0, X, n, 0, n, 1, info, 0, nullptr, nullptr, st, Cscr));
    KQ_TRY(trtri_batched<double>(Hr, n, 0, X, n, 0, n, 1, Tscr, nullptr, st));
    hipLaunchKernelGGL(reverse_upper_kernel, g2, dim3(256), 0, st, X, n, R);
    return check_launch("reverse_upper");
}

