// Symmetric block Gauss-Jordan sweep (fp64) and the principal square root of H_G built on it.
//
// kq_hg_sqrt: S = H_G^{1/2} (principal) and S^{-1} for the output side of bidirectional incoherence
// processing (KronQ review page, Method (1)). Scaled Denman-Beavers iteration
//     Y_0 = A, Z_0 = I,  Y_{k+1} = (mu_k Y_k + Z_k^{-1} / mu_k) / 2,  Z_{k+1} = (mu_k Z_k + Y_k^{-1} / mu_k) / 2
// In the eigenbasis of A both iterates follow the scalar Newton sign step x <- (mu x + 1/(mu x)) / 2
// on x_0 = sqrt(lambda). The scale uses rigorous spectral bounds lambda_max <= ||A||_F and
// lambda_min >= 1 / ||A^{-1}||_F: with the x-interval [a, b], mu = 1/sqrt(ab) maps it to
// [1, (sqrt(b/a) + sqrt(a/b)) / 2], so the interval width after every step is known in closed form
// and the iteration stops once it is below 1e-10 (about 7 steps for cond(A) = 4e9).
//
// The SPD inverses come from a lower-triangle block sweep with 128-wide pivots: per pivot block k
// the panel C = A[:, k] is gathered (symmetric), the pivot P = C[k] is inverted in registers of one
// work-group, T = C P^{-1} and A_RR -= T C^T (fp64 MFMA GEMM, lower triangle, pivot tiles skipped),
// then T and -P^{-1} are scattered back. After all pivots A holds -A^{-1}. Y and Z of every block are
// one batch.
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "kq_internal.h"

namespace kq {

constexpr int GJ_NB = 128;
constexpr int GJ_RT = 32;  // rows per gather/scatter work-group

// Panel C[r][c] = A(r, k0 + c) of the symmetric matrix stored in its lower triangle; c >= nbk -> 0.
// Rows p0 <= r < p1 (the previous pivot block, whose column block has not been written back yet)
// come from that step's T instead: A(r, k0 + c) = Tp[k0 + c][r - p0].
__global__ __launch_bounds__(256) void gj_gather_kernel(const double* __restrict__ A, int64_t n, int64_t lda, int64_t sA,
                                                        int64_t k0, int nbk, double* __restrict__ C, int64_t sC,
                                                        const double* __restrict__ Tp, int64_t p0, int64_t p1,
                                                        const int* skip) {
    if (skip && *skip) return;
    __shared__ double tile[GJ_RT][GJ_NB + 1];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * GJ_RT, z = blockIdx.y;
    A += z * sA;
    C += z * sC;
    const int64_t k1 = k0 + nbk;
    if (Tp && r0 >= p0 && r0 + GJ_RT <= p1) {
        Tp += z * sC;
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int c = e / GJ_RT, rr = e % GJ_RT;
            tile[rr][c] = c < nbk ? Tp[(k0 + c) * GJ_NB + (r0 - p0) + rr] : 0.0;
        }
        __syncthreads();
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int rr = e / GJ_NB, c = e % GJ_NB;
            C[(r0 + rr) * GJ_NB + c] = tile[rr][c];
        }
    } else if (r0 >= k1) {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int64_t r = r0 + e / GJ_NB;
            const int c = e % GJ_NB;
            if (r < n) C[r * GJ_NB + c] = c < nbk ? A[r * lda + k0 + c] : 0.0;
        }
    } else if (r0 + GJ_RT <= k0) {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int c = e / GJ_RT, rr = e % GJ_RT;
            tile[rr][c] = c < nbk ? A[(k0 + c) * lda + r0 + rr] : 0.0;
        }
        __syncthreads();
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int rr = e / GJ_NB, c = e % GJ_NB;
            C[(r0 + rr) * GJ_NB + c] = tile[rr][c];
        }
    } else {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int64_t r = r0 + e / GJ_NB;
            const int c = e % GJ_NB;
            if (r >= n) continue;
            double v = 0.0;
            if (c < nbk) {
                const int64_t q = k0 + c;
                v = r >= q ? A[r * lda + q] : A[q * lda + r];
            }
            C[r * GJ_NB + c] = v;
        }
    }
}

// Step k's update of tile row and column f = k + 1, fused with the gather of panel f (n a multiple
// of 128, so every block is 128 wide). Work-groups take 64 x 64 tiles of the lower triangle in row
// block f (tiles (i, 0..i) of its two 64-row tiles) and in column block f below it, as the tile
// focus of the fp64 GEMM does, and apply A_tile -= T_k[rows] C_k[cols]^T with the whole K = 128 of
// both operands staged in LDS at once, and the tile of A read alongside (one load latency instead of
// one per 16-deep slice; the sums run over k in the same order). Each new value is also written to the panel of step f: at
// (row, col - 128 f) when the column is in block f, and transposed, through LDS, when the row is.
// Tiles in column block k are left out (that block is written back from T_k), and four more
// work-groups per item copy panel rows of block k from T_k: A(r, 128 f + c) = T_k[128 f + c][r - 128 k].
constexpr int GF_T = 64, GF_K = GJ_NB, GF_LD = GF_K + 2;  // tile edge; K staged in LDS; LDS row stride
struct alignas(16) GfPair {
    double v[2];
};
constexpr size_t GF_SMEM = size_t(2) * GF_T * GF_LD * sizeof(double);
static_assert(GF_SMEM >= GF_T * (GF_T + 1) * sizeof(double) && GF_SMEM >= 32 * (GJ_NB + 1) * sizeof(double),
              "the transposing and copying stages reuse the operand LDS");

__host__ __device__ inline int64_t gf_tiles(int64_t n, int64_t k) {  // focus tiles of step k per item
    const int64_t f0 = 2 * (k + 1), ny = n / GF_T;
    return (f0 + 1) + (f0 + 2) + 2 * (ny - f0 - 2);
}

__global__ __launch_bounds__(256) void gj_focus_gather_kernel(double* __restrict__ A, int64_t n, int64_t lda,
                                                              int64_t sA, const double* __restrict__ Tk,
                                                              const double* __restrict__ Ck, int64_t sC, int64_t k,
                                                              double* __restrict__ Cf, const int* skip) {
    if (skip && *skip) return;
    extern __shared__ __align__(16) double gf_sm[];
    double* As = gf_sm;
    double* Bs = gf_sm + GF_T * GF_LD;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    const int64_t z = blockIdx.z, f = k + 1, k0f = f * GJ_NB, p0 = k * GJ_NB;
    A += z * sA;
    Tk += z * sC;
    Ck += z * sC;
    Cf += z * sC;
    const int64_t nf = gf_tiles(n, k);
    int64_t lid = blockIdx.x;
    if (lid >= nf) {  // panel rows p0 + 32 w .. + 31 from T_k
        const int64_t r0 = p0 + 32 * (lid - nf);
        double (*tile)[GJ_NB + 1] = reinterpret_cast<double (*)[GJ_NB + 1]>(gf_sm);
        for (int e = tid; e < 32 * GJ_NB; e += 256) {
            const int c = e / 32, rr = e % 32;
            tile[rr][c] = Tk[(k0f + c) * GJ_NB + (r0 - p0) + rr];
        }
        __syncthreads();
        for (int e = tid; e < 32 * GJ_NB; e += 256) {
            const int rr = e / GJ_NB, c = e % GJ_NB;
            Cf[(r0 + rr) * GJ_NB + c] = tile[rr][c];
        }
        return;
    }
    const int64_t f0 = 2 * f;
    int64_t tm = -1, tn = 0;
    for (int64_t q = 0; q < 2 && tm < 0; q++) {
        if (lid <= f0 + q) { tm = f0 + q; tn = lid; }
        else lid -= f0 + q + 1;
    }
    if (tm < 0) { tm = f0 + 2 + lid / 2; tn = f0 + lid % 2; }
    if ((tn >> 1) == k) return;
    tm = (int64_t)__builtin_amdgcn_readfirstlane((int)tm);
    tn = (int64_t)__builtin_amdgcn_readfirstlane((int)tn);
    const int64_t m0 = tm * GF_T, n0 = tn * GF_T;
    // both operand tiles (64 rows x 128) into LDS, row-major in 16-byte pieces (coalesced, no bank
    // conflicts), and this thread's 16 entries of the tile of A into registers meanwhile
    double cin[2][2][2][2];
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++) {
                const int64_t m = m0 + hi * 32 + 2 * tr + i, c = n0 + hj * 32 + 2 * tc;
                const GfPair t = *reinterpret_cast<const GfPair*>(&A[m * lda + c]);
                cin[hi][i][hj][0] = t.v[0]; cin[hi][i][hj][1] = t.v[1];
            }
#pragma unroll 4
    for (int q = 0; q < GF_T * GF_K / 2 / 256; q++) {
        const int v = tid + 256 * q, r = v / (GF_K / 2), c2 = (v % (GF_K / 2)) * 2;
        *reinterpret_cast<GfPair*>(&As[r * GF_LD + c2]) = *reinterpret_cast<const GfPair*>(&Tk[(m0 + r) * GJ_NB + c2]);
        *reinterpret_cast<GfPair*>(&Bs[r * GF_LD + c2]) = *reinterpret_cast<const GfPair*>(&Ck[(n0 + r) * GJ_NB + c2]);
    }
    __syncthreads();
    // thread (tr, tc): rows h * 32 + 2 tr + i, columns h * 32 + 2 tc + j of the tile
    double acc[2][2][2][2];
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < 2; j++) acc[hi][i][hj][j] = 0.0;
#pragma unroll 4
    for (int kk = 0; kk < GF_K; kk += 2) {
        double a[2][2][2], b[2][2][2];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const GfPair ta = *reinterpret_cast<const GfPair*>(&As[(h * 32 + 2 * tr + i) * GF_LD + kk]);
                const GfPair tb = *reinterpret_cast<const GfPair*>(&Bs[(h * 32 + 2 * tc + i) * GF_LD + kk]);
                a[h][i][0] = ta.v[0]; a[h][i][1] = ta.v[1];
                b[h][i][0] = tb.v[0]; b[h][i][1] = tb.v[1];
            }
#pragma unroll
        for (int e = 0; e < 2; e++)
#pragma unroll
            for (int hi = 0; hi < 2; hi++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int hj = 0; hj < 2; hj++)
#pragma unroll
                        for (int j = 0; j < 2; j++)
                            acc[hi][i][hj][j] = fma(a[hi][i][e], b[hj][j][e], acc[hi][i][hj][j]);
    }
    // A = A - acc on the stored (lower) triangle; panel entries of column block f directly
    const bool col_f = (n0 >> 7) == f, row_f = (m0 >> 7) == f;
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int64_t m = m0 + hi * 32 + 2 * tr + i, c = n0 + hj * 32 + 2 * tc + j;
                    if (c > m) continue;
                    const double v = fma(1.0, cin[hi][i][hj][j], -acc[hi][i][hj][j]);
                    A[m * lda + c] = v;
                    if (col_f) Cf[m * GJ_NB + (c - k0f)] = v;
                    acc[hi][i][hj][j] = v;
                }
    if (!row_f) return;
    // row block f: the panel takes the transpose, staged through LDS
    __syncthreads();
    double (*L)[GF_T + 1] = reinterpret_cast<double (*)[GF_T + 1]>(gf_sm);
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < 2; j++) L[hj * 32 + 2 * tc + j][hi * 32 + 2 * tr + i] = acc[hi][i][hj][j];
    __syncthreads();
    for (int e = tid; e < GF_T * GF_T; e += 256) {
        const int cl = e / GF_T, ml = e % GF_T;
        if (n0 + cl > m0 + ml) continue;
        Cf[(n0 + cl) * GJ_NB + (m0 - k0f + ml)] = L[cl][ml];
    }
}

// Work-group barrier that orders LDS only: global stores issued before it may still be in flight
// (nothing in the work-group reads them back).
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders a wave's LDS writes before its later LDS reads of other lanes' data: the hardware runs a
// wave's LDS operations in order, so only the compiler has to be kept from reordering them.
__device__ inline void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 1/p to full fp64 precision: hardware reciprocal estimate refined by two Newton steps.
__device__ inline double recip64(double p) {
    double r = __builtin_amdgcn_rcp(p);
    r = fma(r, fma(-p, r, 1.0), r);
    return fma(r, fma(-p, r, 1.0), r);
}

// Tm = (A_RJ - E_RJ) D^{-1} for a thread's four rows R = 4tr..4tr+3 in the register sweeps below. The 16
// lanes of a DPP row share tr: lane tc forms the element (rr, q) = (tc & 3, tc >> 2) from the shifted
// pivot rows (A_R. - E_R. = A_.R - E_.R by symmetry) and column q of D^{-1}, and a row broadcast hands
// every lane all sixteen (Tm[rr][q] sits in lane 4q + rr). Same sums, in the same order, as each
// thread forming all sixteen itself, for a quarter of the LDS reads and FMAs.
template <int L>
__device__ __forceinline__ double row_lane(double v) {
    return __builtin_amdgcn_mov_dpp(v, 0x150 + L, 0xF, 0xF, false);
}
template <int... L>
__device__ __forceinline__ void tm_gather(double v, double (&Tm)[4][4], std::integer_sequence<int, L...>) {
    ((Tm[L & 3][L >> 2] = row_lane<L>(v)), ...);
}
__device__ __forceinline__ void pivot_tm(const double (*rowb)[GJ_NB], const double (*dinv)[4], int tr, int tc,
                                         double (&Tm)[4][4]) {
    const int rr = tc & 3, qq = tc >> 2;
    double t = 0.0;
#pragma unroll
    for (int q2 = 0; q2 < 4; q2++) t = fma(rowb[q2][4 * tr + rr], dinv[q2][qq], t);
    tm_gather(t, Tm, std::make_integer_sequence<int, 16>{});
}

// Pinv = P^{-1} for the nbk x nbk SPD pivot P = C[k0 : k0 + nbk][0 : nbk] (identity-padded to 128) by
// a Gauss-Jordan sweep held in registers: 512 threads, thread (tr, tc) owns rows 4tr..4tr+3 and
// columns 32p + 2tc + e (p = 0..3, e = 0, 1; two waves per SIMD). Pivots are taken four at a time (J = 4jb..4jb+3, pivot
// block D = A_JJ) with the symmetric sweep
//     A_RR -= A_RJ D^{-1} A_JR,  A_RJ <- A_RJ D^{-1},  A_JR <- D^{-1} A_JR,  A_JJ <- -D^{-1},
// which keeps A symmetric. All four cases are one rank-4 update A -= (A_.J - E_.J) D^{-1} (A_J. - E_J.)
// (E the identity) followed by A_JJ -= 2I, so every thread runs the same code: it reads the shifted
// pivot rows A_J. - E_J. and D^{-1} from LDS, takes its column factor from those rows by symmetry and
// updates its tile. The next step's pivot rows are written by their owners right after their update,
// and one of those threads reads the next 4 x 4 pivot block back from them, inverts it and writes
// D^{-1}, so one barrier per step separates the steps (LDS double-buffered).
// The block is first scaled to unit diagonal (A = S P S, S = diag(P)^{-1/2}); every pivot block of
// the sweep is then a Schur complement with entries of magnitude <= 1, so the identity shifts cancel
// nothing larger than the result. After the last step the registers hold -A^{-1}, and
// P^{-1} = S A^{-1} S.
constexpr int GJ_PIV_THREADS = 512;

// D (4 x 4, SPD) -> D^{-1} in place by unpivoted Gauss-Jordan; returns 1 + the first non-positive
// pivot (that pivot is replaced by 1), else 0.
__device__ inline int inv4_spd(double D[4][4]) {
    int bad = 0;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        double p = D[t][t];
        if (!(p > 0.0)) {
            bad = bad ? bad : t + 1;
            p = 1.0;
        }
        const double ip = recip64(p);
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int q2 = 0; q2 < 4; q2++)
                if (q != t && q2 != t) D[q][q2] = fma(-D[q][t] * ip, D[t][q2], D[q][q2]);
#pragma unroll
        for (int q = 0; q < 4; q++)
            if (q != t) { D[q][t] *= -ip; D[t][q] *= ip; }
        D[t][t] = ip;
    }
    return bad;
}

// With `ready` set the kernel is launched ahead of the kernel that writes its pivot block: it first
// waits, in a bounded loop, until ready[0] reaches `ready_at` (stored by the first work-group of the
// next kernel on that queue, which starts only once that kernel has completed and released its
// writes), then acquires at device scope before reading the block. A wait that runs out (only when
// the device runs kernels one at a time) sets ready[1], which ends every later wait of the same call
// at once, and info = -1; the block is inverted as found. `ready` belongs to one call (its workspace):
// the host reads ready[1] after the call's first step and redoes that call with queue waits.
constexpr int GJ_WAIT_POLLS = 1 << 20;  // at most about a second of polling
// The limit can be lowered through the environment (KQ_SWEEP_WAIT_POLLS, read on each sweep; from the
// Denman-Beavers step KQ_SWEEP_WAIT_FROM_STEP on, 0 by default), so that a test can make the wait run
// out on purpose, in the first step or in a later one, and check what the call does then.
static int gj_wait_polls(int step) {
    const char* e = std::getenv("KQ_SWEEP_WAIT_POLLS");
    const char* f = std::getenv("KQ_SWEEP_WAIT_FROM_STEP");
    const long v = e ? std::strtol(e, nullptr, 10) : 0;
    const long from = f ? std::strtol(f, nullptr, 10) : 0;
    return v > 0 && v < GJ_WAIT_POLLS && step >= from ? (int)v : GJ_WAIT_POLLS;
}
// Early-launched pivots occupy one compute unit per item while they wait: only for small batches,
// so that the kernels they wait for always find compute units.
constexpr int64_t GJ_EARLY_PIVOT_MAX = 16;


__global__ __launch_bounds__(GJ_PIV_THREADS) void gj_pivot_kernel(const double* __restrict__ C, int64_t sC,
                                                                  int64_t k0, int nbk, double* __restrict__ Pinv,
                                                                  int32_t* info, const int* skip,
                                                                  const uint64_t* ready, uint64_t ready_at,
                                                                  int max_polls) {
    if (skip && *skip) return;
    __shared__ __align__(16) double rowb[2][4][GJ_NB];
    __shared__ __align__(16) double dinv[2][4][4];
    __shared__ int bad_s;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    if (ready) {
        if (tid == 0) {
            int polls = 0;
            while (__hip_atomic_load(&ready[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < ready_at &&
                   __hip_atomic_load(&ready[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
                   ++polls < max_polls)
                __builtin_amdgcn_s_sleep(2);
            if (__hip_atomic_load(&ready[0], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < ready_at) {
                // the counter never came (the device ran the queues one kernel at a time, as under
                // some profilers): mark it for the host, which redoes the work with queue waits
                __hip_atomic_store(const_cast<uint64_t*>(&ready[1]), (uint64_t)1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (info) info[blockIdx.x] = -1;
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    // column cc of the thread's tile: four pairs, 32 apart, so that the 16 column groups of a wave
    // read one contiguous 256-byte run per 16-byte LDS read (four adjacent columns per thread would
    // put the lanes 32 bytes apart: a two-way bank conflict)
    auto col = [&](int cc) { return (cc >> 1) * 32 + 2 * tc + (cc & 1); };
    const int64_t z = blockIdx.x;
    const double* P = C + z * sC + k0 * GJ_NB;
    double sr[4], sc[8];
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
        const int r = 4 * tr + rr;
        const double p = r < nbk ? P[r * GJ_NB + r] : 1.0;
        sr[rr] = p > 0.0 ? 1.0 / sqrt(p) : 1.0;
    }
#pragma unroll
    for (int cc = 0; cc < 8; cc++) {
        const int c = col(cc);
        const double p = c < nbk ? P[c * GJ_NB + c] : 1.0;
        sc[cc] = p > 0.0 ? 1.0 / sqrt(p) : 1.0;
    }
    double a[4][8];
#pragma unroll
    for (int rr = 0; rr < 4; rr++)
#pragma unroll
        for (int cc = 0; cc < 8; cc++) {
            const int r = 4 * tr + rr, c = col(cc);
            a[rr][cc] = (r < nbk && c < nbk) ? P[r * GJ_NB + c] * sr[rr] * sc[cc] : (r == c ? 1.0 : 0.0);
        }
    // Publish the shifted pivot rows of step j (owners: tr == j) and D_j^{-1} (the owner of the
    // diagonal block: tr == j, tc == j / 2).
    auto publish = [&](int j) {
        if (tr == j) {
            const int buf = j & 1;
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) rowb[buf][q][col(cc)] = a[q][cc] - (col(cc) == 4 * j + q ? 1.0 : 0.0);
            // the pivot block spans two lanes: one lane reads it back from the rows just published
            // (LDS operations of a wave complete in order; the wave barrier keeps the compiler from
            // moving the reads above the writes)
            wave_lds_order();
            if (tc == 0) {
                double D[4][4];
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int q2 = 0; q2 < 4; q2++) D[q][q2] = rowb[buf][q][4 * j + q2] + (q == q2 ? 1.0 : 0.0);
                const int b = inv4_spd(D);
                if (b && bad_s == 0) bad_s = 4 * j + b;
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int q2 = 0; q2 < 4; q2++) dinv[buf][q][q2] = D[q][q2];
            }
        }
    };
    if (tid == 0) bad_s = 0;
    __syncthreads();
    publish(0);
    __syncthreads();
    for (int jb = 0; jb < 32; jb++) {
        const int buf = jb & 1;
        double Tm[4][4];
        pivot_tm(rowb[buf], dinv[buf], tr, tc, Tm);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            double rv[8];
#pragma unroll
            for (int cc = 0; cc < 8; cc++) rv[cc] = rowb[buf][q][col(cc)];
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) a[rr][cc] = fma(-Tm[rr][q], rv[cc], a[rr][cc]);
        }
        if (tr == jb) {
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++)
                    if (col(cc) == 4 * jb + q) a[q][cc] -= 2.0;
        }
        if (jb + 1 < 32) publish(jb + 1);
        __syncthreads();
    }
    // the swept block holds -A^{-1}
    double* out = Pinv + z * GJ_NB * GJ_NB;
#pragma unroll
    for (int rr = 0; rr < 4; rr++)
#pragma unroll
        for (int cc = 0; cc < 8; cc++) out[(4 * tr + rr) * GJ_NB + col(cc)] = -a[rr][cc] * sr[rr] * sc[cc];
    if (tid == 0 && bad_s && info && info[z] == 0) info[z] = (int32_t)(k0 + bad_s);
}

// D (4 x 4 SPD) = L L^T: L lower with positive diagonal, and Li = L^{-1} (lower). A non-positive
// pivot is replaced by 1 (the caller reports it through inv4_spd's flag).
__device__ inline void chol4_spd(const double D[4][4], double L[4][4], double Li[4][4]) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
        double sdiag = D[c][c];
#pragma unroll
        for (int k = 0; k < c; k++) sdiag = fma(-L[c][k], L[c][k], sdiag);
        const double d = sqrt(sdiag > 0.0 ? sdiag : 1.0), inv = recip64(d);
        L[c][c] = d;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            if (r <= c) { if (r < c) L[r][c] = 0.0; continue; }
            double t = D[r][c];
#pragma unroll
            for (int k = 0; k < c; k++) t = fma(-L[r][k], L[c][k], t);
            L[r][c] = t * inv;
        }
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const double ir = recip64(L[r][r]);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            if (c > r) { Li[r][c] = 0.0; continue; }
            if (c == r) { Li[r][r] = ir; continue; }
            double t = 0.0;
#pragma unroll
            for (int k = 0; k < r; k++)
                if (k >= c) t = fma(L[r][k], Li[k][c], t);
            Li[r][c] = -t * ir;
        }
    }
}

// Cholesky factor and its inverse of the nb x nb SPD diagonal block at (k0, k0) of a matrix stored in
// its lower triangle: L (lower) over the block's lower triangle, X = L^{-1} (lower) into X's block
// (whose upper part the caller has zeroed). Two kernels:
//  chol_sweep128_kernel: the register sweep of gj_pivot_kernel on the unit-diagonal-scaled block
//    A = S P S, which after the 4-pivot step J holds -(A_{0:J,0:J})^{-1} in the swept rows. It saves,
//    per step, the pre-step (identity-shifted) pivot rows, the post-step rows J and the 4 x 4
//    factor L_JJ = chol(D) to a scratch area;
//  chol_extract128_kernel: from those, in parallel,
//    columns J of L:    L_JJ, and L_RJ = A_RJ L_JJ^{-T} (A_RJ the pre-step column, equal to the
//                       pre-step row by symmetry),
//    rows J of L^{-1}:  (L^{-1})_{J,0:J} = L_JJ^T M_{J,0:J} with M = (A_{0:J,0:J})^{-1}, because
//                       M = L^{-T} L^{-1} on the leading block and (L^{-1})_JJ = L_JJ^{-1};
//    and undoes the scaling: L_P = S^{-1} L_A, L_P^{-1} = L_A^{-1} S.
// Scratch per item: CHOL_SCR doubles.
constexpr int64_t CHOL_SCR = 2 * 32 * 4 * GJ_NB + 32 * 16 + GJ_NB;
constexpr int CHOL_EXTRACT_SPLIT = 8;  // work-groups per item of the extraction

// The sweep of chol_sweep128_kernel on a block whose entries (unscaled; thread (tr, tc) holds rows
// 4tr..4tr+3 and columns col(cc) as in gj_pivot_kernel) are already in registers; dg(r) returns the
// unscaled diagonal entry r < nbk. Writes the scratch of the item and, for a non-positive pivot,
// info[info_slot] (if still 0).
template <typename Diag>
__device__ __forceinline__ void chol_sweep128_body(double (&a)[4][8], Diag dg, int nbk, double* __restrict__ scr,
                                                   int32_t* info, int64_t info_slot, int64_t k0) {
    __shared__ __align__(16) double rowb[2][4][GJ_NB];
    __shared__ __align__(16) double dinv[2][4][4];
    __shared__ int bad_s;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    auto col = [&](int cc) { return (cc >> 1) * 32 + 2 * tc + (cc & 1); };  // as in gj_pivot_kernel
    double* pre = scr;                       // [32][4][128]
    double* post = scr + 32 * 4 * GJ_NB;     // [32][4][128]
    double* lj = scr + 2 * 32 * 4 * GJ_NB;   // [32][4][4]
    double* sqs = lj + 32 * 16;              // [128] sqrt of the block's diagonal (the scaling)
    double sr[4], sc[8];
#pragma unroll
    for (int rr = 0; rr < 4; rr++) {
        const int r = 4 * tr + rr;
        const double p = r < nbk ? dg(r) : 1.0;
        sr[rr] = p > 0.0 ? 1.0 / sqrt(p) : 1.0;
        if (tc == 0) sqs[r] = p > 0.0 ? sqrt(p) : 1.0;
    }
#pragma unroll
    for (int cc = 0; cc < 8; cc++) {
        const int c = col(cc);
        const double p = c < nbk ? dg(c) : 1.0;
        sc[cc] = p > 0.0 ? 1.0 / sqrt(p) : 1.0;
    }
#pragma unroll
    for (int rr = 0; rr < 4; rr++)
#pragma unroll
        for (int cc = 0; cc < 8; cc++) {
            const int r = 4 * tr + rr, c = col(cc);
            a[rr][cc] = (r < nbk && c < nbk) ? a[rr][cc] * sr[rr] * sc[cc] : (r == c ? 1.0 : 0.0);
        }
    auto publish = [&](int j) {
        if (tr == j) {
            const int buf = j & 1;
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) rowb[buf][q][col(cc)] = a[q][cc] - (col(cc) == 4 * j + q ? 1.0 : 0.0);
            wave_lds_order();  // the pivot block is read back from the published rows, as in gj_pivot_kernel
            if (tc == 0) {
                double D[4][4], Lc[4][4], Li[4][4];
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int q2 = 0; q2 < 4; q2++) D[q][q2] = rowb[buf][q][4 * j + q2] + (q == q2 ? 1.0 : 0.0);
                chol4_spd(D, Lc, Li);
                const int b = inv4_spd(D);
                if (b && bad_s == 0) bad_s = 4 * j + b;
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int q2 = 0; q2 < 4; q2++) {
                        dinv[buf][q][q2] = D[q][q2];
                        lj[j * 16 + q * 4 + q2] = Lc[q][q2];
                    }
            }
        }
    };
    if (tid == 0) bad_s = 0;
    __syncthreads();
    publish(0);
    __syncthreads();
    for (int jb = 0; jb < 32; jb++) {
        const int buf = jb & 1;
        pre[jb * 4 * GJ_NB + tid] = (&rowb[buf][0][0])[tid];  // 512 = 4 x 128 values, one per thread
        double Tm[4][4];
        pivot_tm(rowb[buf], dinv[buf], tr, tc, Tm);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            double rv[8];
#pragma unroll
            for (int cc = 0; cc < 8; cc++) rv[cc] = rowb[buf][q][col(cc)];
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) a[rr][cc] = fma(-Tm[rr][q], rv[cc], a[rr][cc]);
        }
        if (tr == jb) {
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++)
                    if (col(cc) == 4 * jb + q) a[q][cc] -= 2.0;
        }
        if (tr == jb) {
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) post[(jb * 4 + q) * GJ_NB + col(cc)] = a[q][cc];
        }
        if (jb + 1 < 32) publish(jb + 1);
        lds_barrier();
    }
    if (tid == 0 && bad_s && bad_s <= nbk && info && info[info_slot] == 0) info[info_slot] = (int32_t)(k0 + bad_s);
}

__global__ __launch_bounds__(GJ_PIV_THREADS) void chol_sweep128_kernel(const double* __restrict__ A, int64_t lda,
                                                                       int64_t sA, int64_t n, int64_t k0,
                                                                       double* __restrict__ scr, int32_t* info,
                                                                       int64_t info_stride, const int* skip) {
    if (skip && *skip) return;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    auto col = [&](int cc) { return (cc >> 1) * 32 + 2 * tc + (cc & 1); };
    const int64_t z = blockIdx.x;
    A += z * sA + k0 * lda + k0;
    const int nbk = (int)((n - k0) < GJ_NB ? (n - k0) : GJ_NB);
    auto Aget = [&](int r, int c) { return c <= r ? A[(int64_t)r * lda + c] : A[(int64_t)c * lda + r]; };
    double a[4][8];
#pragma unroll
    for (int rr = 0; rr < 4; rr++)
#pragma unroll
        for (int cc = 0; cc < 8; cc++) {
            const int r = 4 * tr + rr, c = col(cc);
            a[rr][cc] = (r < nbk && c < nbk) ? Aget(r, c) : 0.0;
        }
    chol_sweep128_body(a, [&](int r) { return A[(int64_t)r * lda + r]; }, nbk, scr + z * CHOL_SCR, info,
                       z * info_stride, k0);
}

__global__ __launch_bounds__(512) void chol_extract128_kernel(double* __restrict__ A, int64_t lda, int64_t sA,
                                                              double* __restrict__ X, int64_t ldx, int64_t sX,
                                                              int64_t n, int64_t k0, const double* __restrict__ scr,
                                                              const int* skip) {
    if (skip && *skip) return;
    __shared__ double sq[GJ_NB];    // sqrt(P_rr)
    __shared__ double ljs[32][4][4], ljit[32][4][4];  // L_JJ and L_JJ^{-T}
    const int tid = threadIdx.x;
    const int64_t z = blockIdx.x;
    A += z * sA + k0 * lda + k0;
    X += z * sX + k0 * ldx + k0;
    scr += z * CHOL_SCR;
    const double* pre = scr;
    const double* post = scr + 32 * 4 * GJ_NB;
    const double* lj = scr + 2 * 32 * 4 * GJ_NB;
    const double* sqs = lj + 32 * 16;
    const int nbk = (int)((n - k0) < GJ_NB ? (n - k0) : GJ_NB);
    // the scaling comes from the sweep's scratch, not from A's diagonal, which the work-groups of
    // this item overwrite (they split the entries below: blockIdx.y of gridDim.y)
    if (tid < GJ_NB) sq[tid] = sqs[tid];
    if (tid < 32) {
        double L[4][4], Li[4][4];
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int q2 = 0; q2 < 4; q2++) L[q][q2] = lj[tid * 16 + q * 4 + q2];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const double ir = 1.0 / L[r][r];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                if (c > r) { Li[r][c] = 0.0; continue; }
                if (c == r) { Li[r][r] = ir; continue; }
                double t = 0.0;
#pragma unroll
                for (int k = 0; k < r; k++)
                    if (k >= c) t = fma(L[r][k], Li[k][c], t);
                Li[r][c] = -t * ir;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int q2 = 0; q2 < 4; q2++) {
                ljs[tid][q][q2] = L[q][q2];
                ljit[tid][q][q2] = Li[q2][q];
            }
    }
    __syncthreads();
    const int e0 = (int)blockIdx.y * 512 + tid, es = (int)gridDim.y * 512;
    // L: entry (r, 4 jb + q) for r >= 4 jb
    for (int e = e0; e < GJ_NB * 32; e += es) {
        const int r = e >> 5, jb = e & 31, j0 = 4 * jb;
        if (r < j0 || r >= nbk) continue;
        if (r < j0 + 4) {
            const int q = r - j0;
            for (int q2 = 0; q2 <= q; q2++)
                if (j0 + q2 < nbk) A[(int64_t)r * lda + j0 + q2] = ljs[jb][q][q2] * sq[r];
        } else {
            double cv[4];
#pragma unroll
            for (int q2 = 0; q2 < 4; q2++) cv[q2] = pre[(jb * 4 + q2) * GJ_NB + r];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                double t = 0.0;
#pragma unroll
                for (int q2 = 0; q2 < 4; q2++) t = fma(cv[q2], ljit[jb][q2][q], t);
                if (j0 + q < nbk) A[(int64_t)r * lda + j0 + q] = t * sq[r];
            }
        }
    }
    // X = L^{-1}: entry (4 jb + q, c) for c < 4 jb + 4, zero right of that in the block
    for (int e = e0; e < GJ_NB * GJ_NB; e += es) {
        const int r = e >> 7, c = e & 127, jb = r >> 2, q = r & 3;
        if (r >= nbk || c >= nbk) continue;
        if (c > 4 * jb + 3) {
            X[(int64_t)r * ldx + c] = 0.0;
            continue;
        }
        double t = 0.0;
#pragma unroll
        for (int q2 = 0; q2 < 4; q2++) t = fma(ljs[jb][q2][q], post[(jb * 4 + q2) * GJ_NB + c], t);
        X[(int64_t)r * ldx + c] = -t / sq[c];
    }
}

// ------------------------------------------------------------------------- fused Cholesky step
// One launch per step of the blocked lower Cholesky of a single matrix (row-major, lda even) that runs
// the factorization of the next 128-wide diagonal block beside the update of the columns below it, so
// that the one-work-group sweep no longer waits for the whole update:
//   work-group 0: D = A[k1:k1+nb, k1:k1+nb] - L_k L_k^T, with L_k = A[k1:k1+nb, k0:k1] the rows of the
//     columns just factored, formed in the sweep's register layout (L_k^T staged in LDS), then the sweep
//     of chol_sweep128_kernel on D, whose scratch chol_extract128_kernel turns into L and L^{-1};
//   every other work-group: two 256-thread halves, each one 128 x 128 tile (tm, tn), tn <= tm, of
//     A[k1:n, k1:J1] -= L L^T (L = A[k1:n, k0:k1]) other than the diagonal block, with 8 x 8 register
//     tiles and 16-deep slices double-buffered in LDS.
// Tiles above the diagonal are left out (only lower triangles are read), and the diagonal block keeps
// its old entries in A (the extraction overwrites its lower triangle with the factor).
constexpr int CS_BK = 16, CS_LD = GJ_NB + 2;
constexpr size_t CS_SMEM = size_t(2) * 2 * 2 * CS_BK * CS_LD * sizeof(double);  // 2 halves x (A, B) x 2 buffers
static_assert(CS_SMEM >= size_t(GJ_NB) * CS_LD * sizeof(double), "the staged L_k^T fits the tile buffers");
typedef double cs_d2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(512) void chol_step_kernel(double* A, int64_t lda, int64_t n, int64_t k0, int64_t J1,
                                                        int64_t ntiles, int64_t Nt, double* __restrict__ scr,
                                                        int32_t* info) {
    extern __shared__ __align__(16) unsigned char cs_raw[];
    double* lds = reinterpret_cast<double*>(cs_raw);
    const int tid = threadIdx.x;
    const int64_t k1 = k0 + GJ_NB, M = n - k1, N = J1 - k1;
    const double* L = A + k1 * lda + k0;
    double* C = A + k1 * lda + k1;
    if (blockIdx.x == 0) {
        __shared__ double dg[GJ_NB];
        const int tr = tid >> 4, tc = tid & 15;
        auto col = [&](int cc) { return (cc >> 1) * 32 + 2 * tc + (cc & 1); };
        const int nb = (int)(M < GJ_NB ? M : GJ_NB);
        for (int v = tid; v < GJ_NB * GJ_NB / 2; v += 512) {  // lds[k][r] = L_k[r][k]
            const int r = v >> 6, kp = (v & 63) * 2;
            cs_d2 t = {0.0, 0.0};
            if (r < nb) t = *reinterpret_cast<const cs_d2*>(L + (int64_t)r * lda + kp);
            lds[kp * CS_LD + r] = t.x;
            lds[(kp + 1) * CS_LD + r] = t.y;
        }
        double a[4][8];
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
#pragma unroll
            for (int cc = 0; cc < 8; cc++) {
                const int r = 4 * tr + rr, c = col(cc);
                a[rr][cc] = (r < nb && c < nb) ? (c <= r ? C[(int64_t)r * lda + c] : C[(int64_t)c * lda + r]) : 0.0;
            }
        __syncthreads();
        for (int k = 0; k < GJ_NB; k++) {
            const double* lr = lds + k * CS_LD;
            const cs_d2 p01 = *reinterpret_cast<const cs_d2*>(lr + 4 * tr);
            const cs_d2 p23 = *reinterpret_cast<const cs_d2*>(lr + 4 * tr + 2);
            const double pr[4] = {p01.x, p01.y, p23.x, p23.y};
            double pc[8];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const cs_d2 q = *reinterpret_cast<const cs_d2*>(lr + g * 32 + 2 * tc);
                pc[2 * g] = q.x;
                pc[2 * g + 1] = q.y;
            }
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
#pragma unroll
                for (int cc = 0; cc < 8; cc++) a[rr][cc] = fma(-pr[rr], pc[cc], a[rr][cc]);
        }
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
#pragma unroll
            for (int cc = 0; cc < 8; cc++)
                if (4 * tr + rr == col(cc)) dg[4 * tr + rr] = a[rr][cc];
        __syncthreads();
        chol_sweep128_body(a, [&](int r) { return dg[r]; }, nb, scr, info, 0, k1);
        return;
    }
    // ---- update tiles: tile list = the triangle of tile rows 0..Nt-1, then the rows below it
    const int h = __builtin_amdgcn_readfirstlane(tid >> 8), t = tid & 255, tr = t >> 4, tc = t & 15;
    int64_t idx = 1 + 2 * ((int64_t)blockIdx.x - 1) + h;
    const bool live = idx < ntiles;
    if (!live) idx = ntiles - 1;  // a real tile: its loads stay in bounds, nothing is stored
    int64_t tm, tn;
    const int64_t T = Nt * (Nt + 1) / 2;
    if (idx < T) {
        tm = (int64_t)((sqrt(8.0 * (double)idx + 1.0) - 1.0) * 0.5);
        while (tm * (tm + 1) / 2 > idx) tm--;
        while ((tm + 1) * (tm + 2) / 2 <= idx) tm++;
        tn = idx - tm * (tm + 1) / 2;
    } else {
        tm = Nt + (idx - T) / Nt;
        tn = (idx - T) % Nt;
    }
    tm = (int64_t)__builtin_amdgcn_readfirstlane((int)tm);
    tn = (int64_t)__builtin_amdgcn_readfirstlane((int)tn);
    const int64_t m0 = tm * GJ_NB, n0 = tn * GJ_NB;
    double* As = lds + h * (2 * 2 * CS_BK * CS_LD);  // [buf][k][m]
    double* Bs = As + 2 * CS_BK * CS_LD;
    double acc[2][4][2][4];
#pragma unroll
    for (int hi = 0; hi < 2; hi++)
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int hj = 0; hj < 2; hj++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[hi][i][hj][j] = 0.0;
    cs_d2 ra[4], rb[4];
    const bool rows_in = m0 + GJ_NB <= M && n0 + GJ_NB <= M;  // uniform: no per-row checks on the loads
    auto gload = [&](int kk0) {
        if (rows_in) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int v = t + 256 * q, row = v >> 3, kp = (v & 7) * 2;
                ra[q] = *reinterpret_cast<const cs_d2*>(L + (m0 + row) * lda + kk0 + kp);
                rb[q] = *reinterpret_cast<const cs_d2*>(L + (n0 + row) * lda + kk0 + kp);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int v = t + 256 * q, row = v >> 3, kp = (v & 7) * 2;
                const int64_t gm = m0 + row, gn = n0 + row;
                ra[q] = gm < M ? *reinterpret_cast<const cs_d2*>(L + gm * lda + kk0 + kp) : cs_d2{0.0, 0.0};
                rb[q] = gn < M ? *reinterpret_cast<const cs_d2*>(L + gn * lda + kk0 + kp) : cs_d2{0.0, 0.0};
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int v = t + 256 * q, row = v >> 3, kp = (v & 7) * 2;
            As[(buf * CS_BK + kp) * CS_LD + row] = ra[q].x;
            As[(buf * CS_BK + kp + 1) * CS_LD + row] = ra[q].y;
            Bs[(buf * CS_BK + kp) * CS_LD + row] = rb[q].x;
            Bs[(buf * CS_BK + kp + 1) * CS_LD + row] = rb[q].y;
        }
    };
    gload(0);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int kk0 = 0; kk0 < GJ_NB; kk0 += CS_BK) {
        const bool more = kk0 + CS_BK < GJ_NB;
        if (more) gload(kk0 + CS_BK);
#pragma unroll 2
        for (int kk = 0; kk < CS_BK; kk++) {
            const double* ar = As + (buf * CS_BK + kk) * CS_LD;
            const double* br = Bs + (buf * CS_BK + kk) * CS_LD;
            double av[2][4], bv[2][4];
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const cs_d2 x = *reinterpret_cast<const cs_d2*>(ar + hh * 64 + tr * 4 + i);
                    av[hh][i] = x.x;
                    av[hh][i + 1] = x.y;
                }
#pragma unroll
                for (int j = 0; j < 4; j += 2) {
                    const cs_d2 x = *reinterpret_cast<const cs_d2*>(br + hh * 64 + (j >> 1) * 32 + 2 * tc);
                    bv[hh][j] = x.x;
                    bv[hh][j + 1] = x.y;
                }
            }
#pragma unroll
            for (int hi = 0; hi < 2; hi++)
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int hj = 0; hj < 2; hj++)
#pragma unroll
                        for (int j = 0; j < 4; j++) acc[hi][i][hj][j] = fma(av[hi][i], bv[hj][j], acc[hi][i][hj][j]);
        }
        if (more) sstore(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    if (!live) return;
    const bool full = m0 + GJ_NB <= M && n0 + GJ_NB <= N;
    // C -= acc, half a tile at a time: every load of C is issued before the first store (the stores
    // could alias later loads, so interleaved they would wait for each other)
#pragma unroll
    for (int hi = 0; hi < 2; hi++) {
        if (full) {
            cs_d2 cv[4][2][2];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        const int64_t m = m0 + hi * 64 + tr * 4 + i, c = n0 + hj * 64 + (j >> 1) * 32 + 2 * tc;
                        cv[i][hj][j >> 1] = *reinterpret_cast<const cs_d2*>(C + m * lda + c);
                    }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        const int64_t m = m0 + hi * 64 + tr * 4 + i, c = n0 + hj * 64 + (j >> 1) * 32 + 2 * tc;
                        cs_d2 v = cv[i][hj][j >> 1];
                        v.x -= acc[hi][i][hj][j];
                        v.y -= acc[hi][i][hj][j + 1];
                        *reinterpret_cast<cs_d2*>(C + m * lda + c) = v;
                    }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int hj = 0; hj < 2; hj++)
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        const int64_t m = m0 + hi * 64 + tr * 4 + i, c = n0 + hj * 64 + (j >> 1) * 32 + 2 * tc;
                        double* p = C + m * lda + c;
                        if (m < M) {
                            if (c < N) p[0] -= acc[hi][i][hj][j];
                            if (c + 1 < N) p[1] -= acc[hi][i][hj][j + 1];
                        }
                    }
        }
    }
}


}  // namespace kq

kq_status kq::chol_inv_diag128(double* A, int64_t lda, int64_t sA, double* X, int64_t ldx, int64_t sX, int64_t n,
                               int64_t k0, int64_t batch, double* scr, int32_t* info, int64_t info_stride,
                               const int* skip, hipStream_t st) {
    if (batch > 65535) return fail(KQ_ESHAPE, "chol_inv_diag128: batch too large");
    if (!scr) return fail(KQ_EWORKSPACE, "chol_inv_diag128: no scratch");
    hipLaunchKernelGGL(chol_sweep128_kernel, dim3((unsigned)batch), dim3(GJ_PIV_THREADS), 0, st, A, lda, sA, n, k0, scr,
                       info, info_stride, skip);
    KQ_TRY(check_launch("chol_sweep128"));
    hipLaunchKernelGGL(chol_extract128_kernel, dim3((unsigned)batch, CHOL_EXTRACT_SPLIT), dim3(512), 0, st, A, lda, sA, X,
                       ldx, sX, n, k0, scr, skip);
    return check_launch("chol_extract128");
}

int64_t kq::chol_scratch_doubles() { return CHOL_SCR; }

kq_status kq::chol_step_fused(double* A, int64_t lda, int64_t n, int64_t k0, int64_t J1, double* scr, int32_t* info,
                              hipStream_t st) {
    const int64_t k1 = k0 + GJ_NB;
    if (k1 >= J1 || J1 > n || (lda & 1) || (reinterpret_cast<uintptr_t>(A) & 15) || !scr)
        return fail(KQ_EINVAL, "chol_step_fused: bad step");
    const int64_t Mt = (n - k1 + GJ_NB - 1) / GJ_NB, Nt = (J1 - k1 + GJ_NB - 1) / GJ_NB;
    const int64_t ntiles = Nt * (Nt + 1) / 2 + (Mt - Nt) * Nt;
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&chol_step_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)CS_SMEM);
        attr = true;
    }
    hipLaunchKernelGGL(chol_step_kernel, dim3((unsigned)(1 + ntiles / 2)), dim3(512), CS_SMEM, st, A, lda, n, k0, J1,
                       ntiles, Nt, scr, info);
    return check_launch("chol_step");
}

kq_status kq::chol_extract_diag128(double* A, int64_t lda, double* X, int64_t ldx, int64_t n, int64_t k0, double* scr,
                                   hipStream_t st) {
    hipLaunchKernelGGL(chol_extract128_kernel, dim3(1, CHOL_EXTRACT_SPLIT), dim3(512), 0, st, A, lda, (int64_t)0, X, ldx,
                       (int64_t)0, n, k0, scr, nullptr);
    return check_launch("chol_extract128");
}

namespace kq {

// A(r, k0 + c) <- T[r][c] for r outside the pivot block (lower-triangle position), and the pivot
// block <- -Pinv (lower triangle).
__global__ __launch_bounds__(256) void gj_scatter_kernel(double* __restrict__ A, int64_t n, int64_t lda, int64_t sA,
                                                         int64_t k0, int nbk, const double* __restrict__ T, int64_t sT,
                                                         const double* __restrict__ Pinv, const int* skip) {
    if (skip && *skip) return;
    __shared__ double tile[GJ_RT][GJ_NB + 1];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * GJ_RT, z = blockIdx.y;
    A += z * sA;
    T += z * sT;
    Pinv += z * GJ_NB * GJ_NB;
    const int64_t k1 = k0 + nbk;
    if (r0 >= k1) {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int64_t r = r0 + e / GJ_NB;
            const int c = e % GJ_NB;
            if (r < n && c < nbk) A[r * lda + k0 + c] = T[r * GJ_NB + c];
        }
    } else if (r0 + GJ_RT <= k0) {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int rr = e / GJ_NB, c = e % GJ_NB;
            tile[rr][c] = T[(r0 + rr) * GJ_NB + c];
        }
        __syncthreads();
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int c = e / GJ_RT, rr = e % GJ_RT;
            if (c < nbk) A[(k0 + c) * lda + r0 + rr] = tile[rr][c];
        }
    } else {
        for (int e = tid; e < GJ_RT * GJ_NB; e += 256) {
            const int64_t r = r0 + e / GJ_NB;
            const int c = e % GJ_NB;
            if (r >= n || c >= nbk) continue;
            const int64_t q = k0 + c;
            if (r >= k0 && r < k1) {
                if (c <= r - k0) A[r * lda + q] = -Pinv[(r - k0) * GJ_NB + c];
            } else if (r > q) {
                A[r * lda + q] = T[r * GJ_NB + c];
            } else {
                A[q * lda + r] = T[r * GJ_NB + c];
            }
        }
    }
}

// Queues of a device for the pipelined sweep (default priority): `side` runs the pivot chain,
// `main` the wide rank-128 updates. Events order both with the caller's stream; the mutex keeps the
// event sequence of one call intact when several host threads enqueue at once. The events only order
// work of the one device, so they take a device-scope release (no system-scope fence when recorded).
// The queues and events are created on a device's first sweep and kept until the process ends; they
// hold no data of any call.
struct SweepQueues {
    hipStream_t side = nullptr, main = nullptr;
    hipEvent_t ev[9] = {};
    bool gf_lds = false;        // the fused gather's LDS size has been allowed on this device
    bool ok = false;
};
static std::mutex g_sweep_mu;
static SweepQueues g_sweep[64];

// Hand-over state of one call's sweeps. `ready` lives in the call's workspace and is zeroed on the
// caller's stream when the call starts: [0] is a counter that only grows within the call (one store
// per signalled step, value `signalled`, kept on the host), which pivot kernels launched early wait
// on; [1] is set by a pivot whose wait ran out. `early` selects the device-side hand-over; without
// it the queues wait on events.
struct SweepSync {
    uint64_t* ready = nullptr;
    uint64_t signalled = 0;
    bool early = true;
    int step = 0;               // Denman-Beavers step of the sweep being enqueued
};

static kq_status sweep_queues(SweepQueues** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(KQ_EHIP, "sweep queues: no device");
    SweepQueues& q = g_sweep[dev];
    if (!q.ok) {
        if (hipStreamCreateWithFlags(&q.side, hipStreamNonBlocking) != hipSuccess ||
            hipStreamCreateWithFlags(&q.main, hipStreamNonBlocking) != hipSuccess)
            return fail(KQ_EHIP, "sweep queues: stream creation failed");
        for (hipEvent_t& e : q.ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
                return fail(KQ_EHIP, "sweep queues: event creation failed");
        q.ok = true;
    }
    *out = &q;
    return KQ_OK;
}

#define KQ_HIP(expr)                                                                    \
    do {                                                                                \
        if ((expr) != hipSuccess) return fail(KQ_EHIP, "%s failed", #expr);            \
    } while (0)

// A <- -A^{-1} for a batch of SPD matrices stored in their lower triangles (n x n, leading dimension
// lda, item stride sA). Scratch (two of each, alternating by pivot): panels C and T
// (batch x n x 128) and Pinv (batch x 128 x 128).
//
// Pipeline per pivot step k. The pivot block k + 1 depends on step k's update only through tile row
// and column k + 1, so:
//   main queue: update those tiles (tile (k + 1, k) excepted) and gather panel k + 1, taking tile
//               (k + 1, k) from T_k; then apply the rest of step k's update A_RR -= T_k C_k^T (every
//               tile outside rows and columns k, k + 1);
//   side queue: invert pivot k + 1, write T_k and -Pinv_k back into row and column k, form
//               T_{k+1} = C_{k+1} Pinv_{k+1}, concurrently with the main queue's wide update.
// The pivot's work-groups need a whole compute unit each (202 VGPRs x 8 waves), so they must be
// dispatched before the wide update's tiles fill the chip. With whole 128-wide blocks and a small
// batch the pivot kernel is launched as soon as the side queue reaches it and waits on the device
// for a counter that the main queue's wide update sets as it starts, right after the gather (a
// bounded wait; no queue wait or extra launch sits on that path). Otherwise the side queue waits for an event after the gather, and the wide
// update for an event the side queue records once past that wait, and the write-back runs on the
// main queue meanwhile. The queues touch disjoint tiles and alternate the panel buffers; step k + 1
// on the main queue waits for the side queue's T_{k+1} and write-back of step k. The caller's
// stream waits for both at the end.
static kq_status gj_inverse_batched(double* A, int64_t n, int64_t lda, int64_t sA, int64_t batch, double* const C[2],
                                    double* const T[2], double* const Pinv[2], int32_t* info, const int* skip,
                                    SweepSync* sync, hipStream_t st) {
    if (batch > 65535) return fail(KQ_ESHAPE, "sweep batch too large");
    const int64_t sC = n * GJ_NB;
    const int64_t nt = (n + GJ_NB - 1) / GJ_NB;
    const dim3 gr((unsigned)((n + GJ_RT - 1) / GJ_RT), (unsigned)batch);
    std::lock_guard<std::mutex> lock(g_sweep_mu);
    SweepQueues* q = nullptr;
    KQ_TRY(sweep_queues(&q));
    hipStream_t sb = q->side, sm = q->main;
    hipEvent_t ev0 = q->ev[0], evG[2] = {q->ev[1], q->ev[2]}, evB[2] = {q->ev[3], q->ev[4]}, evM = q->ev[5],
               evS[2] = {q->ev[7], q->ev[8]};
    auto nb_of = [&](int64_t k) { return (int)((n - k * GJ_NB) < GJ_NB ? (n - k * GJ_NB) : GJ_NB); };
    auto gather = [&](int64_t k, hipStream_t qg) -> kq_status {
        const int b = (int)(k & 1), nbk = nb_of(k);
        const int64_t k0 = k * GJ_NB;
        const double* Tp = k > 0 ? T[b ^ 1] : nullptr;
        const int64_t p0 = k > 0 ? k0 - GJ_NB : 0;
        hipLaunchKernelGGL(gj_gather_kernel, gr, dim3(256), 0, qg, A, n, lda, sA, k0, nbk, C[b], sC, Tp, p0, k0, skip);
        return check_launch("gj_gather");
    };
    const int polls = gj_wait_polls(sync ? sync->step : 0);
    // side queue: Pinv_k (waiting on the device counter for `ready_at` when given), T_k = C_k Pinv_k
    auto pivot = [&](int64_t k, uint64_t ready_at) -> kq_status {
        const int b = (int)(k & 1), nbk = nb_of(k);
        hipLaunchKernelGGL(gj_pivot_kernel, dim3((unsigned)batch), dim3(GJ_PIV_THREADS), 0, sb, C[b], sC, k * GJ_NB,
                           nbk, Pinv[b], info, skip, ready_at ? sync->ready : nullptr, ready_at, polls);
        return check_launch("gj_pivot");
    };
    auto tprod = [&](int64_t k) -> kq_status {
        const int b = (int)(k & 1), nbk = nb_of(k);
        GemmArgs<double> t = gemm_args<double>(n, nbk, nbk, C[b], GJ_NB, Pinv[b], GJ_NB, T[b], GJ_NB, 1.0, 0.0);
        t.nb1 = batch; t.sA1 = sC; t.sB1 = GJ_NB * GJ_NB; t.sC1 = sC; t.skip = skip;
        return gemm<double>(t, false, false, sb);
    };
    auto scatter = [&](int64_t k, hipStream_t qs) -> kq_status {
        const int b = (int)(k & 1);
        hipLaunchKernelGGL(gj_scatter_kernel, gr, dim3(256), 0, qs, A, n, lda, sA, k * GJ_NB, nb_of(k), T[b], sC,
                           Pinv[b], skip);
        return check_launch("gj_scatter");
    };
    // main queue: every tile outside rows/columns k, k + 1; with ready_at, the launch also releases
    // the device counter (it starts only after the gather before it has completed)
    auto wide_update = [&](int64_t k, uint64_t ready_at) -> kq_status {
        const int b = (int)(k & 1);
        GemmArgs<double> u = gemm_args<double>(n, n, nb_of(k), T[b], GJ_NB, C[b], GJ_NB, A, lda, -1.0, 1.0);
        u.nb1 = batch; u.sA1 = sC; u.sB1 = sC; u.sC1 = sA; u.tri = 1; u.skip = skip; u.skip_tile = k;
        u.skip_tile2 = k + 1 < nt ? k + 1 : -1;
        u.stagger = 1;
        if (ready_at) { u.signal = sync->ready; u.signal_value = ready_at; }
        return gemm<double>(u, false, true, sm);
    };
    // whole 128-wide blocks: the row and column update of the next pivot and its gather are one kernel
    const bool fused = n % GJ_NB == 0 && lda % 2 == 0 && sA % 2 == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
    if (fused && !q->gf_lds) {
        KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&gj_focus_gather_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)GF_SMEM));
        q->gf_lds = true;
    }
    auto focus_gather = [&](int64_t k) -> kq_status {  // main queue: step k on tile row/column k + 1, panel k + 1
        const int cur = (int)(k & 1);
        hipLaunchKernelGGL(gj_focus_gather_kernel, dim3((unsigned)(gf_tiles(n, k) + 4), 1, (unsigned)batch), dim3(256),
                           GF_SMEM, sm, A, n, lda, sA, T[cur], C[cur], sC, k, C[cur ^ 1], skip);
        return check_launch("gj_focus_gather");
    };
    KQ_HIP(hipEventRecord(ev0, st));
    KQ_HIP(hipStreamWaitEvent(sb, ev0, 0));
    KQ_TRY(gather(0, sb));
    KQ_TRY(pivot(0, 0));
    KQ_TRY(tprod(0));
    KQ_HIP(hipEventRecord(evB[0], sb));
    if (fused && batch <= GJ_EARLY_PIVOT_MAX && sync && sync->early && sync->ready) {
        // Step k: main queue: (T_k and the write-back of step k - 1 done) the fused row/column update
        // and gather, then the wide update, whose start releases the counter. Side queue: pivot k + 1,
        // launched at once so its work-groups hold their compute units before the wide update is
        // dispatched; it waits on the device for the counter, so no queue wait sits between the
        // gather and the pivot or between the pivot and the wide update. The write-back of step k
        // (rows and columns k, outside the wide update and the gather) goes just before the pivot,
        // T_{k+1} after it.
        for (int64_t k = 0; k < nt; k++) {
            const int cur = (int)(k & 1), nxt = cur ^ 1;
            KQ_HIP(hipStreamWaitEvent(sm, evB[cur], 0));
            uint64_t ready_at = 0;
            if (k + 1 < nt) {
                KQ_TRY(focus_gather(k));
                ready_at = ++sync->signalled;
                // the wide update's launch releases the counter: enqueue it before the pivot that waits
                KQ_TRY(wide_update(k, ready_at));
            } else if (nt > 1) {
                KQ_TRY(wide_update(k, 0));
            }
            // the write-back first, while the previous wide update drains and before this one fills
            // the chip, then the pivot, so that only T_{k+1} runs beside the update
            KQ_TRY(scatter(k, sb));
            if (k + 1 < nt) {
                KQ_TRY(pivot(k + 1, ready_at));
                KQ_TRY(tprod(k + 1));
            }
            KQ_HIP(hipEventRecord(evB[nxt], sb));
        }
    } else {
        for (int64_t k = 0; k < nt; k++) {
            const int cur = (int)(k & 1), nxt = cur ^ 1, nbk = nb_of(k);
            // main queue (step k - 1's update already behind it in order): T_k ready
            KQ_HIP(hipStreamWaitEvent(sm, evB[cur], 0));
            if (k + 1 < nt && fused) {
                KQ_TRY(focus_gather(k));
            } else if (k + 1 < nt) {
                GemmArgs<double> u = gemm_args<double>(n, n, nbk, T[cur], GJ_NB, C[cur], GJ_NB, A, lda, -1.0, 1.0);
                u.nb1 = batch; u.sA1 = sC; u.sB1 = sC; u.sC1 = sA; u.tri = 1; u.skip = skip; u.skip_tile = k;
                u.focus = k + 1;
                KQ_TRY(gemm<double>(u, false, true, sm));
                KQ_TRY(gather(k + 1, sm));
            }
            KQ_HIP(hipEventRecord(evG[cur], sm));
            // side queue: pivot k + 1; evS marks that it has passed its wait
            KQ_HIP(hipStreamWaitEvent(sb, evG[cur], 0));
            KQ_HIP(hipEventRecord(evS[cur], sb));
            if (k + 1 < nt) {
                KQ_TRY(pivot(k + 1, 0));
                KQ_TRY(tprod(k + 1));
            }
            KQ_HIP(hipEventRecord(evB[nxt], sb));
            // main queue: write step k back while the side queue takes its wait (rows and columns k
            // are outside both the update and the gather), then the rest of step k's update
            KQ_TRY(scatter(k, sm));
            KQ_HIP(hipStreamWaitEvent(sm, evS[cur], 0));
            if (nt > 1) KQ_TRY(wide_update(k, 0));
        }
    }
    KQ_HIP(hipEventRecord(evM, sm));
    KQ_HIP(hipStreamWaitEvent(st, evM, 0));
    KQ_HIP(hipStreamWaitEvent(st, evB[nt & 1], 0));
    return KQ_OK;
}

// ---------------------------------------------------------------------------------- DB kernels
// With x-interval bound b after a step, the eigenvalues of Y are within about (b - 1) of those of
// A^{1/2} (relative); 1e-8 is well below the fp32 rounding of the stored S. The bound recursion
// reaches it within 7 steps for any cond(A) <= 1e16 even with the loose norm bounds; a matrix that
// has not converged after those steps is reported through info (= o + 1).
constexpr int DB_MAXIT = 7;
constexpr double DB_TOL = 1e-8;
// Last step. After step k every eigenvalue of Z_k Y_k is x^2 with x in [1, b_k], and the Newton-Schulz
// step Y <- Y (3I - Z Y) / 2 = Y + Y E / 2, E = I - Z Y (and Z <- Z + E Z / 2) maps x = 1 + e to
// 1 - 1.5 e^2 - 0.5 e^3: from b - 1 <= DB_NS_MAX it lands within DB_TOL, as a Denman-Beavers step
// would, for one fp64 product (E, lower triangle) and one fp32 product per output instead of two SPD
// inverses. E is formed in fp64 from the fp64 iterates (it is the small difference of I and Z Y);
// the correction Y E / 2, some 1e-4 of Y, needs only fp32: its rounding error is ~1e-11 of Y.
constexpr double DB_NS_MAX = 8e-5;
constexpr int NORM_PARTS = 512;  // at most this many partial sums per matrix (one per work-group)

// Y_0 = H_G in fp64 (also into NI, where the first step's sweep inverts it in place), Z_0 = I, and the
// call's words cleared: flags, the caller's info, the sweep's hand-over counter and the pivots' info.
// It is the call's first kernel, and everything that reads those words runs after it on this queue or
// on queues forked from it (each separate clearing launch had to wait for a compute unit while the
// work already on the chip drained).
template <typename T>
__global__ void db_init_kernel(const T* HG, int64_t n, int64_t nbk, double* YZ, double* NI, int* flags,
                               int32_t* info, uint64_t* ready, int32_t* finfo, int64_t items) {
    const int64_t nn = n * n;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < nbk * nn; e += (int64_t)gridDim.x * 256) {
        const int64_t b = e / nn, rc = e % nn, r = rc / n, c = rc % n;
        const double h = (double)HG[b * nn + rc];
        YZ[e] = h;
        NI[e] = h;
        YZ[(nbk + b) * nn + rc] = (r == c) ? 1.0 : 0.0;
    }
    if (blockIdx.x == 0) {
        if (threadIdx.x < 4) flags[threadIdx.x] = 0;
        if (threadIdx.x < 2) ready[threadIdx.x] = 0;
        if (threadIdx.x == 0) *info = 0;
        for (int64_t k = threadIdx.x; k < items; k += 256) finfo[k] = 0;
    }
}

// Partial sums of the squared Frobenius norm of symmetric matrices stored in their lower triangles;
// part[z][p]. Runs only while flags[1] (iterations done) == it_only (or always when it_only < 0).
__global__ void sym_norm_part_kernel(const double* A, int64_t n, int64_t sA, double* part, const int* flags,
                                     int it_only) {
    if (it_only >= 0 && (flags[0] || flags[1] != it_only)) return;
    __shared__ double sp[256];
    const int64_t z = blockIdx.y;
    const int p = blockIdx.x;
    const double* M = A + z * sA;
    double acc = 0;
    for (int64_t r = p; r < n; r += gridDim.x) {
        for (int64_t c = threadIdx.x; c <= r; c += 256) {
            const double v = M[r * n + c];
            acc += (c == r ? 1.0 : 2.0) * v * v;
        }
    }
    sp[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sp[threadIdx.x] += sp[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[z * NORM_PARTS + p] = sp[0];
}

// Per block b: the scale mu_b of this step and the bound of the next x-interval [1, bnd_b].
// flags[1] == 0: x in [sqrt(lo), sqrt(hi)], hi = ||A||_F, lo = 1 / ||A^{-1}||_F.
__global__ void db_scale_kernel(const double* nrmA, const double* nrmInv, int64_t nbk, int parts, double* mu,
                                double* bnd, const int* flags) {
    if (flags[0]) return;
    for (int64_t b = blockIdx.x * 256 + threadIdx.x; b < nbk; b += (int64_t)gridDim.x * 256) {
        double sA = 0, sI = 0;
        if (flags[1] == 0) {
            for (int p = 0; p < parts; p++) { sA += nrmA[b * NORM_PARTS + p]; sI += nrmInv[b * NORM_PARTS + p]; }
            const double hi = sqrt(sA), lo = 1.0 / sqrt(sI);
            const double r = sqrt(hi / lo);                  // x-interval ratio
            mu[b] = 1.0 / sqrt(sqrt(hi * lo));
            bnd[b] = 0.5 * (sqrt(r) + 1.0 / sqrt(r));
        } else {
            const double bb = bnd[b];
            mu[b] = 1.0 / sqrt(bb);
            bnd[b] = 0.5 * (sqrt(bb) + 1.0 / sqrt(bb));
        }
    }
}

// Y <- (mu Y + Zinv / mu) / 2, Z <- (mu Z + Yinv / mu) / 2; NINV holds -inverses (lower triangles).
// Lower triangles read and written (the upper ones are filled once, after the last step); per-work-
// group partial sums of ||dY||^2 and ||Y||^2. The new Y and Z also go to NINV's lower triangles (each
// element is read there first, by the same thread), which is where the next step's sweep inverts them
// in place.
constexpr int DB_UPD_BLOCKS = 1024;
__global__ void db_update_kernel(double* YZ, double* NINV, const double* mu, int64_t n, int64_t nbk, double* part,
                                 const int* flags) {
    if (flags[0]) return;
    const bool first = flags[1] == 0;
    __shared__ double sd[256], sn[256];
    const int64_t nn = n * n, tri = n * (n + 1) / 2;
    double acc_d = 0, acc_n = 0;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < nbk * tri; e += (int64_t)gridDim.x * 256) {
        const int64_t b = e / tri;
        const int64_t t = e % tri;
        int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
        while (r * (r + 1) / 2 > t) r--;
        while ((r + 1) * (r + 2) / 2 <= t) r++;
        const int64_t c = t - r * (r + 1) / 2;
        const double m = mu[b];
        double* Y = YZ + b * nn;
        double* Z = YZ + (nbk + b) * nn;
        // Z_0 = I: the first step needs no inverse of Z
        const double yi = -NINV[b * nn + r * n + c];
        const double zi = first ? (r == c ? 1.0 : 0.0) : -NINV[(nbk + b) * nn + r * n + c];
        const double y = Y[r * n + c], zz = Z[r * n + c];
        const double yn = 0.5 * (m * y + zi / m);
        const double zn = 0.5 * (m * zz + yi / m);
        const double w = (r == c) ? 1.0 : 2.0;
        acc_d += w * (yn - y) * (yn - y);
        acc_n += w * yn * yn;
        Y[r * n + c] = yn;
        Z[r * n + c] = zn;
        NINV[b * nn + r * n + c] = yn;
        NINV[(nbk + b) * nn + r * n + c] = zn;
    }
    sd[threadIdx.x] = acc_d;
    sn[threadIdx.x] = acc_n;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            sd[threadIdx.x] += sd[threadIdx.x + w];
            sn[threadIdx.x] += sn[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = sd[0];
        part[2 * blockIdx.x + 1] = sn[0];
    }
}

// flags[0]: done, flags[1]: steps taken. Done when every block's interval bound is within DB_TOL of
// 1; a failed pivot or a non-finite value stops the iteration and is reported through info.
__global__ void db_converge_kernel(const double* part, const double* bnd, int64_t nbk, int* flags,
                                   const int32_t* finfo, int64_t nitems, int32_t* info) {
    if (flags[0]) return;
    // the update's partial sums, strided over the 64 lanes and then added in lane order (fixed order)
    __shared__ double sd[64], sn[64];
    double d = 0, nn = 0;
    for (int b = threadIdx.x; b < DB_UPD_BLOCKS; b += 64) { d += part[2 * b]; nn += part[2 * b + 1]; }
    sd[threadIdx.x] = d;
    sn[threadIdx.x] = nn;
    __syncthreads();
    if (threadIdx.x != 0) return;
    d = 0;
    nn = 0;
    for (int l = 0; l < 64; l++) { d += sd[l]; nn += sn[l]; }
    double bmax = 0;
    for (int64_t b = 0; b < nbk; b++) bmax = fmax(bmax, bnd[b] - 1.0);
    int32_t bad = 0;
    for (int64_t k = 0; k < nitems; k++)
        if (finfo[k] != 0) { bad = finfo[k]; break; }
    flags[1] += 1;
    const double rel = sqrt(d / nn);
    if (bad) { *info = bad; flags[0] = 1; return; }
    if (!(rel == rel) || !(nn > 0) || !(bmax == bmax)) { *info = 1; flags[0] = 1; return; }
    if (bmax < DB_TOL) flags[0] = 1;
}

// The number of steps the iteration takes (the first included), from the interval bounds after the
// first step by the recursion of db_scale_kernel (the same fp64 operations; a non-finite bound
// counts one step), and the other words the host reads after that step: out[0] = steps, out[1] =
// flags[0] (stopped: converged or failed), out[2] = 1 if a device-side wait of the sweep ran out,
// out[3] = 1 if after steps - 1 steps every block's bound is within DB_NS_MAX of 1 (the last step can
// be the Newton-Schulz step).
__global__ __launch_bounds__(256) void db_plan_kernel(const double* bnd, int64_t nbk, const int* flags,
                                                      const uint64_t* ready, int* out) {
    __shared__ int sk[256];
    int need = 1;
    for (int64_t b = threadIdx.x; b < nbk; b += 256) {
        double bb = bnd[b];
        int k = 1;
        while (bb - 1.0 >= DB_TOL && k < DB_MAXIT) {
            bb = 0.5 * (sqrt(bb) + 1.0 / sqrt(bb));
            k++;
        }
        need = need > k ? need : k;
    }
    sk[threadIdx.x] = need;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sk[threadIdx.x] = sk[threadIdx.x] > sk[threadIdx.x + w] ? sk[threadIdx.x] : sk[threadIdx.x + w];
        __syncthreads();
    }
    __syncthreads();
    const int total = sk[0];
    __syncthreads();
    // the bound of every block after total - 1 steps
    int ok = 1;
    for (int64_t b = threadIdx.x; b < nbk; b += 256) {
        double bb = bnd[b];
        for (int k = 1; k < total - 1; k++) bb = 0.5 * (sqrt(bb) + 1.0 / sqrt(bb));
        if (!(bb - 1.0 <= DB_NS_MAX)) ok = 0;
    }
    sk[threadIdx.x] = ok;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sk[threadIdx.x] = sk[threadIdx.x] < sk[threadIdx.x + w] ? sk[threadIdx.x] : sk[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = total;
        out[1] = flags[0];
        out[2] = ready[1] != 0 ? 1 : 0;
        out[3] = total >= 2 && sk[0] ? 1 : 0;
    }
}

// E = I in the lower triangles of nbk n x n matrices (the Newton-Schulz step's C before -= Z Y).
__global__ void ns_eye_kernel(double* E, int64_t n, int64_t nbk, const int* flags) {
    if (flags[0]) return;
    const int64_t nn = n * n;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < nbk * nn; e += (int64_t)gridDim.x * 256) {
        const int64_t rc = e % nn;
        E[e] = (rc / n == rc % n) ? 1.0 : 0.0;
    }
}

// fp32 operands and outputs of the Newton-Schulz step: Yf = S = Y, Zf = Si = Z (when Si is given),
// Ef = E mirrored from its lower triangle. S and Si receive the correction next, in place.
__global__ void ns_convert_kernel(const double* YZ, const double* E, int64_t n, int64_t nbk, float* Yf, float* Zf,
                                  float* Ef, float* S, float* Si) {
    const int64_t nn = n * n;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < nbk * nn; e += (int64_t)gridDim.x * 256) {
        const int64_t b = e / nn, rc = e % nn, r = rc / n, c = rc % n;
        const float y = (float)YZ[e];
        Yf[e] = y;
        S[e] = y;
        Ef[e] = (float)E[b * nn + (r >= c ? r * n + c : c * n + r)];
        if (Si) {
            const float z = (float)YZ[nbk * nn + e];
            Zf[e] = z;
            Si[e] = z;
        }
    }
}

__global__ void ns_done_kernel(int* flags) {
    if (threadIdx.x == 0 && !flags[0]) flags[0] = 1;
}

__global__ void db_final_kernel(const int* flags, int32_t* info, int32_t code) {
    if (threadIdx.x == 0 && !flags[0] && *info == 0) *info = code;
}

__global__ void db_out_kernel(const double* YZ, int64_t n, int64_t nbk, float* S, float* Si) {
    const int64_t nn = n * n;
    for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < nbk * nn; e += (int64_t)gridDim.x * 256) {
        S[e] = (float)YZ[e];
        if (Si) Si[e] = (float)YZ[nbk * nn + e];
    }
}

// Upper triangles of `items` symmetric n x n matrices from their lower ones, through 32 x 32 LDS tiles
// so that both the reads and the transposed writes are coalesced. Grid (tiles, tiles, items); tile
// (I, J) with I >= J reads block (I, J) and writes its transpose into block (J, I).
__global__ __launch_bounds__(256) void mirror_lower_batched_kernel(double* M, int64_t n) {
    const int64_t I = blockIdx.x, J = blockIdx.y;
    if (J > I) return;
    __shared__ double t[32][33];
    M += (int64_t)blockIdx.z * n * n;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int yy = ty; yy < 32; yy += 8) {
        const int64_t r = I * 32 + yy, c = J * 32 + tx;
        t[yy][tx] = (r < n && c < n) ? M[r * n + c] : 0.0;
    }
    __syncthreads();
    for (int yy = ty; yy < 32; yy += 8) {
        const int64_t r = J * 32 + yy, c = I * 32 + tx;  // upper element (r, c) = lower (c, r)
        if (r < n && c < n && c > r) M[r * n + c] = t[tx][yy];
    }
}

__global__ void hg_diag_kernel(const float* h, int64_t o, float* S, float* Si, int32_t* info) {
    for (int64_t r = blockIdx.x * 256 + threadIdx.x; r < o; r += (int64_t)gridDim.x * 256) {
        const float v = h[r];
        if (!(v > 0.0f)) atomicCAS(info, 0, (int32_t)(r + 1));  // tests only check info > 0
        const float sq = sqrtf(v > 0.0f ? v : 1.0f);
        S[r] = sq;
        if (Si) Si[r] = 1.0f / sq;
    }
}

template <typename Ar>
static void hg_layout(Ar& a, int64_t n, int64_t nbk) {
    const size_t nn = (size_t)n * n, items = 2 * (size_t)nbk;
    a.template take<double>(items * nn);                     // YZ
    a.template take<double>(items * nn);                     // sweep buffer (-inverses)
    for (int b = 0; b < 2; b++) {
        a.template take<double>(items * n * GJ_NB);          // C
        a.template take<double>(items * n * GJ_NB);          // T
        a.template take<double>(items * GJ_NB * GJ_NB);      // Pinv
    }
    a.template take<double>((size_t)nbk * NORM_PARTS);       // ||A||_F^2 parts
    a.template take<double>(items * NORM_PARTS);             // ||A^{-1}||_F^2 parts
    a.template take<double>(nbk);                            // mu
    a.template take<double>(nbk);                            // interval bound
    a.template take<int32_t>(items);                         // per-item info
    a.template take<double>(2 * DB_UPD_BLOCKS);              // partial sums
    a.template take<int>(4);                                 // flags
    a.template take<uint64_t>(2);                            // sweep hand-over counter and ran-out word
    a.template take<int>(4);                                 // words read back after the first step
    a.template take<float>((size_t)nbk * nn);                // E in fp32 (Newton-Schulz step)
}

// Host side of the square root's one readback: pinned memory, which the copy engine writes
// directly (no staging through a runtime buffer). One 16-byte buffer per host thread, allocated on
// the thread's first call and kept until the process ends.
static kq_status plan_host(int** out) {
    thread_local int* buf = nullptr;
    if (!buf) {
        void* p = nullptr;
        if (hipHostMalloc(&p, 4 * sizeof(int), hipHostMallocPortable) != hipSuccess || !p)
            return fail(KQ_EHIP, "square root: pinned host buffer for the readback");
        buf = static_cast<int*>(p);
    }
    *out = buf;
    return KQ_OK;
}

}  // namespace kq

using namespace kq;

size_t hg_sqrt_ws(kq_hg_form form, int64_t o, int64_t blk) {
    if (form == KQ_HG_DIAG) return 0;
    const int64_t n = form == KQ_HG_FULL ? o : blk, nbk = form == KQ_HG_FULL ? 1 : o / blk;
    Sizer z;
    hg_layout(z, n, nbk);
    return z.used;
}

// Denman-Beavers square root of nbk SPD n x n matrices (fp32 HGf or fp64 HGd, exactly one given);
// on return the workspace holds Y = A^{1/2} (items 0 .. nbk-1) and Z = A^{-1/2} (items nbk ..) in
// fp64 at *Y64 (Z at *Y64 + nbk n^2). info: 0, or o_info + 1 when the iteration did not converge
// or a matrix is not positive definite. With fp32 outputs S (and Si, may be null) given, the last
// step may be the Newton-Schulz step, which writes S and Si itself: *written is then true (and the
// fp64 iterates hold the step before it).
static kq_status db_sqrt(const float* HGf, const double* HGd, int64_t n, int64_t nbk, int32_t o_info, int32_t* info,
                         void* ws, size_t ws_bytes, double** Y64, hipStream_t st, bool early = true,
                         float* S = nullptr, float* Si = nullptr, bool* written = nullptr) {
    if (written) *written = false;
    Arena ar(ws, ws_bytes);
    const size_t nn = (size_t)n * n, items = 2 * (size_t)nbk;
    double* YZ = ar.take<double>(items * nn);
    double* NI = ar.take<double>(items * nn);
    double *C[2], *T[2], *Pinv[2];
    for (int b = 0; b < 2; b++) {
        C[b] = ar.take<double>(items * n * GJ_NB);
        T[b] = ar.take<double>(items * n * GJ_NB);
        Pinv[b] = ar.take<double>(items * GJ_NB * GJ_NB);
    }
    double* nrmA = ar.take<double>((size_t)nbk * NORM_PARTS);
    double* nrmI = ar.take<double>(items * NORM_PARTS);
    double* mu = ar.take<double>(nbk);
    double* bnd = ar.take<double>(nbk);
    int32_t* finfo = ar.take<int32_t>(items);
    double* part = ar.take<double>(2 * DB_UPD_BLOCKS);
    int* flags = ar.take<int>(4);
    uint64_t* ready = ar.take<uint64_t>(2);
    int* plan = ar.take<int>(4);
    float* Ef = ar.take<float>((size_t)nbk * nn);
    const int* done = flags;
    bool ns = false;
    SweepSync sync;
    sync.ready = ready;
    sync.early = early;

    const unsigned eb = (unsigned)((nbk * nn + 255) / 256 < 4096 ? (nbk * nn + 255) / 256 : 4096);
    if (HGd)
        hipLaunchKernelGGL(db_init_kernel<double>, dim3(eb), dim3(256), 0, st, HGd, n, nbk, YZ, NI, flags, info, ready,
                           finfo, (int64_t)items);
    else
        hipLaunchKernelGGL(db_init_kernel<float>, dim3(eb), dim3(256), 0, st, HGf, n, nbk, YZ, NI, flags, info, ready,
                           finfo, (int64_t)items);
    KQ_TRY(check_launch("db_init"));
    const int parts = (int)(n < NORM_PARTS ? n : NORM_PARTS);  // row-strided partial sums of ||.||_F^2
    hipLaunchKernelGGL(sym_norm_part_kernel, dim3(parts, (unsigned)nbk), dim3(256), 0, st, YZ, n, (int64_t)nn, nrmA,
                       flags, -1);
    KQ_TRY(check_launch("db_norm"));
    int nsteps = DB_MAXIT;
    for (int it = 0; it < nsteps; it++) {
        // the first step inverts Y_0 = A only (Z_0 = I); later steps find Y and Z in NI already
        // (written there by the previous step's update)
        const size_t inv_items = it == 0 ? (size_t)nbk : items;
        sync.step = it;
        KQ_TRY(gj_inverse_batched(NI, n, n, (int64_t)nn, (int64_t)inv_items, C, T, Pinv, finfo, done, &sync, st));
        // ||A^{-1}||_F of Y_0 = A (first step only; NI holds -A^{-1})
        hipLaunchKernelGGL(sym_norm_part_kernel, dim3(parts, (unsigned)nbk), dim3(256), 0, st, NI, n, (int64_t)nn,
                           nrmI, flags, 0);
        KQ_TRY(check_launch("db_norm_inv"));
        hipLaunchKernelGGL(db_scale_kernel, dim3((unsigned)((nbk + 255) / 256)), dim3(256), 0, st, nrmA, nrmI, nbk, parts, mu,
                           bnd, flags);
        KQ_TRY(check_launch("db_scale"));
        hipLaunchKernelGGL(db_update_kernel, dim3(DB_UPD_BLOCKS), dim3(256), 0, st, YZ, NI, mu, n, nbk, part, flags);
        KQ_TRY(check_launch("db_update"));
        hipLaunchKernelGGL(db_converge_kernel, dim3(1), dim3(64), 0, st, part, bnd, nbk, flags, finfo, (int64_t)items,
                           info);
        KQ_TRY(check_launch("db_converge"));
        if (it == 0) {
            // After the first step the interval bound of every block is known, and the later bounds
            // follow from it in closed form: the device counts the steps they imply, the host reads
            // that count back and launches exactly those steps, instead of sweeps that would only skip.
            int* hp = nullptr;
            KQ_TRY(plan_host(&hp));
            hipLaunchKernelGGL(db_plan_kernel, dim3(1), dim3(256), 0, st, bnd, nbk, flags, ready, plan);
            KQ_TRY(check_launch("db_plan"));
            KQ_HIP(hipMemcpyAsync(hp, plan, 4 * sizeof(int), hipMemcpyDeviceToHost, st));
            KQ_HIP(hipStreamSynchronize(st));
            const int need = hp[0], stopped = hp[1], ran_out = hp[2];
            if (ran_out) {
                // the device ran the sweep's queues one kernel at a time: redo this call with queue
                // waits (nothing is kept for later calls)
                KQ_TRY(db_sqrt(HGf, HGd, n, nbk, o_info, info, ws, ws_bytes, Y64, st, false, S, Si, written));
                set_error("notice: a device-side wait of the square root's sweep ran out; the call was redone "
                          "with queue waits");
                return KQ_OK;
            }
            if (stopped) break;  // converged after one step, or stopped on an error (info set)
            nsteps = need;
            if (S && hp[3]) {
                ns = true;
                nsteps = need - 1;
            }
        }
    }
    {
        const unsigned tiles = (unsigned)((n + 31) / 32);
        if (items > 65535) return fail(KQ_ESHAPE, "square root: too many blocks");
        hipLaunchKernelGGL(mirror_lower_batched_kernel, dim3(tiles, tiles, (unsigned)items), dim3(256), 0, st, YZ, n);
        KQ_TRY(check_launch("db_mirror"));
    }
    *Y64 = YZ;
    if (ns) {
        // the Newton-Schulz step (skipped on the device when the iteration stopped on an error: S and
        // Si are then the last iterates, and info is set). E (fp64) in NI's first half, Y and Z in
        // fp32 in its second half.
        double* E = NI;
        float* Yf = reinterpret_cast<float*>(NI + nbk * nn);
        float* Zf = Yf + nbk * nn;
        double* Y = YZ;
        double* Z = YZ + nbk * nn;
        hipLaunchKernelGGL(ns_eye_kernel, dim3(eb), dim3(256), 0, st, E, n, nbk, flags);
        KQ_TRY(check_launch("ns_eye"));
        GemmArgs<double> ge = gemm_args<double>(n, n, n, Z, n, Y, n, E, n, -1.0, 1.0);  // E = I - Z Y (Y = Y^T)
        ge.tri = 1; ge.nb1 = nbk; ge.sA1 = (int64_t)nn; ge.sB1 = (int64_t)nn; ge.sC1 = (int64_t)nn; ge.skip = flags;
        KQ_TRY(gemm<double>(ge, false, true, st));
        hipLaunchKernelGGL(ns_convert_kernel, dim3(eb), dim3(256), 0, st, YZ, E, n, nbk, Yf, Zf, Ef, S, Si);
        KQ_TRY(check_launch("ns_convert"));
        GemmArgs<float> gy = gemm_args<float>(n, n, n, Yf, n, Ef, n, S, n, 0.5f, 1.0f);  // S = Y + Y E / 2
        gy.nb1 = nbk; gy.sA1 = (int64_t)nn; gy.sB1 = (int64_t)nn; gy.sC1 = (int64_t)nn; gy.skip = flags;
        KQ_TRY(gemm<float>(gy, false, false, st));
        if (Si) {
            GemmArgs<float> gz = gemm_args<float>(n, n, n, Ef, n, Zf, n, Si, n, 0.5f, 1.0f);  // Si = Z + E Z / 2
            gz.nb1 = nbk; gz.sA1 = (int64_t)nn; gz.sB1 = (int64_t)nn; gz.sC1 = (int64_t)nn; gz.skip = flags;
            KQ_TRY(gemm<float>(gz, false, false, st));
        }
        hipLaunchKernelGGL(ns_done_kernel, dim3(1), dim3(64), 0, st, flags);
        KQ_TRY(check_launch("ns_done"));
        if (written) *written = true;
    }
    hipLaunchKernelGGL(db_final_kernel, dim3(1), dim3(64), 0, st, flags, info, o_info + 1);
    return check_launch("db_final");
}

// The square root reads its first step back to the host, so a stream under graph capture is refused
// before anything is enqueued.
kq_status kq::refuse_capture(hipStream_t st, const char* who) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return fail(KQ_EHIP, "%s: stream capture query failed", who);
    if (cs != hipStreamCaptureStatusNone)
        return fail(KQ_EINVAL, "%s: the stream is capturing a graph; this call reads back from the device", who);
    return KQ_OK;
}

kq_status kq::spd_sqrt_f64(const double* A, int64_t n, int32_t* info, void* ws, size_t ws_bytes, double** Y64,
                           hipStream_t st) {
    if (!ws || ws_bytes < hg_sqrt_ws(KQ_HG_FULL, n, 0)) return fail(KQ_EWORKSPACE, "square root: workspace too small");
    if (n > 65535 * (int64_t)GJ_RT) return fail(KQ_ESHAPE, "square root: too large");
    return db_sqrt(nullptr, A, n, 1, (int32_t)n, info, ws, ws_bytes, Y64, st);
}

extern "C" kq_status kq_hg_sqrt(const float* HG, kq_hg_form form, int64_t o, int64_t blk, float* S, float* Sinv,
                                int32_t* info, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!HG || !S || !info) return fail(KQ_EINVAL, "kq_hg_sqrt: null pointer");
    if (o <= 0) return fail(KQ_ESHAPE, "kq_hg_sqrt: o must be positive");
    hipStream_t st = hs(stream);
    if (form == KQ_HG_DIAG) {
        KQ_TRY(fill<int>(reinterpret_cast<int*>(info), 1, 0, st));
        const unsigned blocks = (unsigned)((o + 255) / 256 < 1024 ? (o + 255) / 256 : 1024);
        hipLaunchKernelGGL(hg_diag_kernel, dim3(blocks), dim3(256), 0, st, HG, o, S, Sinv, info);
        return check_launch("hg_diag");
    }
    if (form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "kq_hg_sqrt: bad form");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "kq_hg_sqrt: o must be a multiple of blk");
    const int64_t n = form == KQ_HG_FULL ? o : blk, nbk = form == KQ_HG_FULL ? 1 : o / blk;
    if (n > 65535 * (int64_t)GJ_RT) return fail(KQ_ESHAPE, "kq_hg_sqrt: too large");
    if (!ws || ws_bytes < hg_sqrt_ws(form, o, blk)) return fail(KQ_EWORKSPACE, "kq_hg_sqrt: workspace too small");
    KQ_TRY(refuse_capture(st, "kq_hg_sqrt"));
    set_error("");
    double* YZ = nullptr;
    bool written = false;
    KQ_TRY(db_sqrt(HG, nullptr, n, nbk, (int32_t)o, info, ws, ws_bytes, &YZ, st, true, S, Sinv, &written));
    if (written) return KQ_OK;
    const size_t nn = (size_t)n * n;
    const unsigned eb = (unsigned)((nbk * nn + 255) / 256 < 4096 ? (nbk * nn + 255) / 256 : 4096);
    hipLaunchKernelGGL(db_out_kernel, dim3(eb), dim3(256), 0, st, YZ, n, nbk, S, Sinv);
    return check_launch("db_out");
}
