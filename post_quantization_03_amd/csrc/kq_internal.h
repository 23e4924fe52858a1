// Internal declarations shared by the HIP sources of libkq (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "../../include/kq.h"

namespace kq {

// ------------------------------------------------------------------------------------------ errors
void set_error(const char* fmt, ...);
kq_status fail(kq_status st, const char* fmt, ...);
kq_status check_launch(const char* what);

#define KQ_TRY(expr)                         \
    do {                                     \
        kq_status _st = (expr);              \
        if (_st != KQ_OK) return _st;        \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t hs(kq_stream s) { return reinterpret_cast<hipStream_t>(s); }

// --------------------------------------------------------------------------------------- workspace
// Bump allocator over the caller's workspace. Every slice is 256-byte aligned.
struct Arena {
    char* base;
    size_t cap, used;
    Arena(void* b, size_t c) : base(static_cast<char*>(b)), cap(c), used(0) {}
    template <typename T>
    T* take(size_t count) {
        size_t off = (used + 255) & ~size_t(255);
        used = off + count * sizeof(T);
        return (base && used <= cap) ? reinterpret_cast<T*>(base + off) : nullptr;
    }
    bool ok() const { return used <= cap; }
};

// Sizes only (no pointers): the same code path as Arena, used by kq_workspace_bytes.
struct Sizer {
    size_t used = 0;
    template <typename T>
    void take(size_t count) { used = ((used + 255) & ~size_t(255)) + count * sizeof(T); }
};

// -------------------------------------------------------------------------------------------- GEMM
// C = alpha * op(A) op(B) [* rowsign[m]] [* colsign[n]] + beta * C on MFMA, row-major operands.
// op(A) is M x K (A stored M x K, or K x M when ta), op(B) is K x N (B stored K x N, or N x K when
// tb). Two batch levels: z = z1 * nb2 + z2, operand offset z1 * s?1 + z2 * s?2.
// tri: 0 full, 1 store only m >= n (lower), 2 store only m <= n (upper); only tiles touching the
// stored triangle are launched (M and N must give the same tile count). kmode restricts the K range per tile to skip structural zeros
// of triangular operands: bit0 k >= m0, bit1 k >= n0, bit2 k < m0 + 128, bit3 k < n0 + 128.
template <typename T>
struct GemmArgs {
    int64_t M, N, K;
    const T* A; int64_t lda, sA1, sA2;
    const T* B; int64_t ldb, sB1, sB2;
    T* C; int64_t ldc, sC1, sC2;
    int64_t nb1, nb2;
    T alpha, beta;
    const int8_t* rsign; int64_t sR1, sR2;
    const int8_t* csign; int64_t sS1, sS2;
    int tri, kmode;
    const int* skip;   // device flag: when nonzero every work-group returns at once (may be null)
    int64_t skip_tile; // tile row and tile column (128-wide) to leave untouched (-1: none)
    int64_t skip_tile2;// a second one (-1: none)
    int64_t focus;     // fp64 lower-triangular products only: launch just the 128-wide tile row and
                       // column `focus` (-1: all tiles)
    int compact;       // set by the fp64 launcher: the grid omits the skipped tile rows and columns
    int own_rows;      // fp64, N <= 128: one work-group per block of C rows, so that C may overwrite A
                       // (every work-group reads only the rows of A that it writes)
    int stagger;       // fp64, alpha = -1 and beta = 1: every other work-group reads its tile of C before
                       // the product instead of after it, so the tiles' reads of C spread over the launch
    uint64_t* signal;  // fp64: when set, the first work-group stores signal_value there as the launch
    uint64_t signal_value;  // starts (after the kernels before it on the queue have completed)
};

template <typename T>
GemmArgs<T> gemm_args(int64_t M, int64_t N, int64_t K, const T* A, int64_t lda, const T* B, int64_t ldb, T* C,
                      int64_t ldc, T alpha, T beta) {
    GemmArgs<T> g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
    g.nb1 = 1; g.nb2 = 1; g.alpha = alpha; g.beta = beta; g.skip_tile = -1; g.skip_tile2 = -1; g.focus = -1;
    return g;
}

template <typename T>
kq_status gemm(const GemmArgs<T>& g, bool ta, bool tb, hipStream_t st);

// ------------------------------------------------------------------------------- SPD toolkit
// Batched in-place lower Cholesky of n x n matrices A (item stride sA) with the inverses of the
// diagonal blocks written to X (item stride sX; fp32: X must be zero beforehand, fp64: the whole 128-wide
// diagonal blocks are written, zero above the diagonal), logdet[z] += sum log L_ii
// (may be null), info[z] set to 1 + index of the first failing pivot (may be null).
template <typename T>
kq_status potrf_batched(T* A, int64_t lda, int64_t sA, T* X, int64_t ldx, int64_t sX, int64_t n, int64_t batch,
                        int32_t* info, int64_t info_stride, double* logdet, const int* skip, hipStream_t st,
                        double* scr = nullptr);
// X <- L^{-1} (lower) given L (lower, strictly below the diagonal blocks) and X holding the
// inverses of the diagonal blocks (from potrf_batched). T scratch: batch * n * n / 4 elements.
template <typename T>
kq_status trtri_batched(const T* L, int64_t ldl, int64_t sL, T* X, int64_t ldx, int64_t sX, int64_t n,
                        int64_t batch, T* Tscr, const int* skip, hipStream_t st);
template <typename T>
int potrf_nb();
// fp64 diagonal-block step of potrf_batched: Cholesky factor L (lower, over the block) and L^{-1}
// (into X's block) of the 128 x 128 block at (k0, k0), by a register-resident sweep.
// scr: batch * chol_scratch_doubles() doubles.
kq_status chol_inv_diag128(double* A, int64_t lda, int64_t sA, double* X, int64_t ldx, int64_t sX, int64_t n,
                           int64_t k0, int64_t batch, double* scr, int32_t* info, int64_t info_stride,
                           const int* skip, hipStream_t st);
int64_t chol_scratch_doubles();
// One step k0 of a single matrix's blocked Cholesky (128-wide blocks, lda even, A 16-byte aligned): the
// update A[k1:n, k1:J1] -= L L^T by the columns k0..k1 = k0 + 128 just factored (lower tiles only, the
// diagonal block k1 left as it was) together with the sweep of that diagonal block, updated, into scr
// (k1 < J1 <= n). chol_extract_diag128 then writes its factor into A and its inverse into X.
kq_status chol_step_fused(double* A, int64_t lda, int64_t n, int64_t k0, int64_t J1, double* scr, int32_t* info,
                          hipStream_t st);
kq_status chol_extract_diag128(double* A, int64_t lda, double* X, int64_t ldx, int64_t n, int64_t k0, double* scr,
                               hipStream_t st);

// Square root of one SPD n x n fp64 matrix A by the scaled Denman-Beavers iteration (the same
// iteration as kq_hg_sqrt). On return *Y64 points into ws: A^{1/2} (n x n) followed by A^{-1/2}.
// info: 0, or n + 1 if A is not positive definite or the iteration did not converge.
// ws: hg_sqrt_ws(KQ_HG_FULL, n, 0) bytes.
kq_status spd_sqrt_f64(const double* A, int64_t n, int32_t* info, void* ws, size_t ws_bytes, double** Y64,
                       hipStream_t st);

// KQ_EINVAL when `st` is capturing a HIP graph (for calls that read back from the device).
kq_status refuse_capture(hipStream_t st, const char* who);

// ------------------------------------------------------------------------------------ helpers
template <typename T>
kq_status fill(T* p, size_t count, T value, hipStream_t st, const int* skip = nullptr);

}  // namespace kq

// workspace size of kq_hg_sqrt (defined with it)
size_t hg_sqrt_ws(kq_hg_form form, int64_t o, int64_t blk);
