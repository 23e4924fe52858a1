// Preparation of the output-side curvature H_G and the K-FAC layer loss.
//
// * kq_hg_extract: the fp32 storage forms (full, 128-block diagonal, diagonal) of an fp64
//   covariance accumulated by kq_hessian_accum from gradient rows (H_G = G^T G / n streams through
//   the same accumulation as H_X).
// * kq_hg_lowrank: a low-rank-plus-isotropic approximation of H_G = G^T G / n built from G alone
//   (the o x o matrix is never accumulated), and its square root and inverse square root in closed
//   form. KronQ review page, Limitations (2) and Sparks: H_G is held as a full d_out x d_out matrix
//   during the bidirectional preprocessing, and how much survives low-rank or blockwise
//   approximations is left open. With Q an orthonormal basis of range(H^{q+1} Omega) (randomised
//   range finder with q power steps on the caller's Gaussian Omega, o x k), B = Q^T H Q and
//   sigma = (tr H - tr B) / (o - k),
//       H^ = Q B Q^T + sigma (I - Q Q^T)
//   keeps H on the captured subspace, is isotropic on its complement and has the trace of H (so the
//   sensitivity tr(H_G) tr(H_X) is unchanged). Its root follows from B's:
//       H^{1/2} = sqrt(sigma) I + Q (B^{1/2} - sqrt(sigma) I) Q^T, H^{-1/2} likewise,
//   so the o x o Denman-Beavers iteration is replaced by one on k x k.
// * kq_kfac_loss: tr(H_G dW H_X dW^T) with dW = W^ - W in the original coordinates (KronQ review
//   page, Background: the Kronecker-factored Hessian H ~ H_X (x) H_G of one layer).
#include "kq_internal.h"

namespace kq {

constexpr int SQ_PARTS = 256;

__global__ void widen_rows_kernel(const float* __restrict__ src, int64_t ld, int64_t rows, int64_t cols,
                                  double* __restrict__ dst) {
    const int64_t total = rows * cols;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
        dst[e] = (double)src[(e / cols) * ld + e % cols];
}

// part[b] = sum of squares over a fixed strided share of A (fixed order within the block)
__global__ void sumsq_part_kernel(const double* __restrict__ A, int64_t count, double* __restrict__ part) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < count; e += (int64_t)SQ_PARTS * 256) s += A[e] * A[e];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// tr H = sum(part) / n, sigma = (tr H - tr B) / (o - k); flags[0] = 1 when sigma is not positive
__global__ void lowrank_sigma_kernel(const double* __restrict__ part, double inv_n, const double* __restrict__ B,
                                     int64_t k, int64_t o, double* __restrict__ sig, int* flags) {
    __shared__ double red[256];
    double a = 0.0, b = 0.0;
    for (int p = threadIdx.x; p < SQ_PARTS; p += 256) a += part[p];
    for (int64_t j = threadIdx.x; j < k; j += 256) b += B[j * k + j];
    red[threadIdx.x] = a;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const double trH = red[0] * inv_n;
    __syncthreads();
    red[threadIdx.x] = b;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double s = (trH - red[0]) / (double)(o - k);
        sig[0] = s;
        sig[1] = trH;
        flags[0] = (s > 0.0) ? 0 : 1;
    }
}

// diagonal shift of a k x k matrix by -c, with c = sqrt(sigma) (mode 0), 1/sqrt(sigma) (mode 1) or
// sigma (mode 2)
__device__ __forceinline__ double sigma_term(const double* sig, int mode) {
    const double s = sig[0] > 0.0 ? sig[0] : 0.0;
    return mode == 0 ? sqrt(s) : mode == 1 ? (s > 0.0 ? 1.0 / sqrt(s) : 0.0) : s;
}

__global__ void shift_diag_kernel(const double* __restrict__ A, int64_t k, const double* __restrict__ sig, int mode,
                                  double* __restrict__ out) {
    const double c = sigma_term(sig, mode);
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < k * k; e += (int64_t)gridDim.x * 256)
        out[e] = A[e] - ((e / k == e % k) ? c : 0.0);
}

// out (fp32, o x o) = M + c I
__global__ void add_diag_out_kernel(const double* __restrict__ M, int64_t o, const double* __restrict__ sig, int mode,
                                    float* __restrict__ out) {
    const double c = sigma_term(sig, mode);
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < o * o; e += (int64_t)gridDim.x * 256)
        out[e] = (float)(M[e] + ((e / o == e % o) ? c : 0.0));
}

// info: 0; 1 the range basis lost rank (a Cholesky pivot of Y^T Y failed); 2 sigma <= 0; 3 B's
// square root failed
__global__ void lowrank_info_kernel(const int32_t* __restrict__ pinfo, int npinfo, const int* __restrict__ flags,
                                    const int32_t* __restrict__ dbinfo, int32_t* __restrict__ info) {
    if (threadIdx.x != 0) return;
    int32_t v = 0;
    for (int j = 0; j < npinfo; j++)
        if (pinfo[j]) v = 1;
    if (!v && flags[0]) v = 2;
    if (!v && *dbinfo) v = 3;
    *info = v;
}

// H_G storage forms from an fp64 covariance
__global__ void hg_extract_kernel(const double* __restrict__ H, int64_t o, int64_t ldh, int form, int64_t blk,
                                  float* __restrict__ HG) {
    const int64_t total = form == KQ_HG_FULL ? o * o : form == KQ_HG_BLOCK ? o * blk : o;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        int64_t r, c;
        if (form == KQ_HG_FULL) {
            r = e / o; c = e % o;
        } else if (form == KQ_HG_BLOCK) {
            const int64_t b = e / (blk * blk), rc = e % (blk * blk);
            r = b * blk + rc / blk; c = b * blk + rc % blk;
        } else {
            r = e; c = e;
        }
        HG[e] = (float)H[r * ldh + c];
    }
}

// D = What - W in fp64 (W fp32 or bf16)
__global__ void diff_f64_kernel(const void* __restrict__ W, int wbf16, int64_t ldw, const float* __restrict__ What,
                                int64_t ldq, int64_t o, int64_t i, double* __restrict__ D) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < o * i; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / i, c = e % i;
        const double w = wbf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(W)[r * ldw + c] << 16)
                               : (double)static_cast<const float*>(W)[r * ldw + c];
        D[e] = (double)What[r * ldq + c] - w;
    }
}

// B = H_G D for the diagonal (row scale) form; the block and full forms use the fp64 GEMM on HG64
__global__ void hg_rows_kernel(const float* __restrict__ h, const double* __restrict__ D, int64_t o, int64_t i,
                               double* __restrict__ B) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < o * i; e += (int64_t)gridDim.x * 256)
        B[e] = (double)h[e / i] * D[e];
}

// part[b] = sum over a fixed share of A * B (elementwise)
__global__ void dot_part_kernel(const double* __restrict__ A, const double* __restrict__ B, int64_t count,
                                double* __restrict__ part) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < count; e += (int64_t)SQ_PARTS * 256) s += A[e] * B[e];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ void sum_parts_kernel(const double* __restrict__ part, double* __restrict__ out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int p = threadIdx.x; p < SQ_PARTS; p += 256) s += part[p];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

__global__ void copy_pair_kernel(const double* __restrict__ src, double* __restrict__ dst) {
    if (threadIdx.x < 2) dst[threadIdx.x] = src[threadIdx.x];
}

static unsigned grid_for(int64_t count) {
    const int64_t b = (count + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

// Q (o x k) = an orthonormal basis of range(Y) by two Cholesky-QR passes (Y^T Y = L L^T, Y <- Y L^{-T})
static kq_status orth(const double* Y, double* Q, double* Ytmp, int64_t o, int64_t k, double* C, double* X,
                      double* Tscr, double* cscr, int32_t* pinfo, hipStream_t st) {
    const double* cur = Y;
    for (int pass = 0; pass < 2; pass++) {
        GemmArgs<double> c = gemm_args<double>(k, k, o, cur, k, cur, k, C, k, 1.0, 0.0);
        KQ_TRY(gemm<double>(c, true, false, st));
        KQ_TRY(fill<double>(X, (size_t)k * k, 0.0, st));
        KQ_TRY(potrf_batched<double>(C, k, k * k, X, k, k * k, k, 1, pinfo + pass, 0, nullptr, nullptr, st, cscr));
        KQ_TRY(trtri_batched<double>(C, k, k * k, X, k, k * k, k, 1, Tscr, nullptr, st));
        double* dst = pass == 0 ? Ytmp : Q;
        GemmArgs<double> q = gemm_args<double>(o, k, k, cur, k, X, k, dst, k, 1.0, 0.0);
        KQ_TRY(gemm<double>(q, false, true, st));
        cur = dst;
    }
    return KQ_OK;
}

}  // namespace kq

using namespace kq;

static void lowrank_layout(Sizer& z, int64_t n, int64_t o, int64_t k) {
    z.take<double>((size_t)n * o);              // G in fp64
    z.take<double>((size_t)o * k);              // Omega, then Y
    z.take<double>((size_t)n * k);              // G Q
    z.take<double>((size_t)o * k);              // Y scratch
    z.take<double>((size_t)o * k);              // Q
    z.take<double>((size_t)k * k);              // C
    z.take<double>((size_t)k * k);              // X = L^{-1}
    z.take<double>((size_t)(k * k / 2 + 128 * 128));
    z.take<double>((size_t)chol_scratch_doubles());
    z.take<double>((size_t)k * k);              // B
    z.take<double>((size_t)k * k);              // core
    z.take<double>((size_t)o * k);              // Q core
    z.take<double>((size_t)o * o);              // o x o product
    z.take<double>(SQ_PARTS);
    z.take<double>(2);                          // sigma, tr H
    z.take<int32_t>(32);                        // Cholesky infos
    z.take<int32_t>(1);                         // square-root info
    z.take<int>(4);                             // flags
    z.take<char>(hg_sqrt_ws(KQ_HG_FULL, k, 0)); // k x k square root
}

size_t hg_lowrank_ws(int64_t n, int64_t o, int64_t k) {
    if (n <= 0 || o <= 0 || k <= 0) return 0;
    Sizer z;
    lowrank_layout(z, n, o, k);
    return z.used;
}

extern "C" kq_status kq_hg_lowrank(const float* G, int64_t n, int64_t o, int64_t ldg, int64_t k, int q,
                                   const float* omega, float* S, float* Sinv, float* HGhat, double* sigma,
                                   int32_t* info, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!G || !omega || !S || !info) return fail(KQ_EINVAL, "kq_hg_lowrank: null pointer");
    if (n <= 0 || o <= 1 || ldg < o) return fail(KQ_ESHAPE, "kq_hg_lowrank: bad sizes");
    if (k <= 0 || k >= o || k > n) return fail(KQ_ESHAPE, "kq_hg_lowrank: rank must satisfy 0 < k < o and k <= n");
    if (q < 0 || q > 15) return fail(KQ_EINVAL, "kq_hg_lowrank: power steps must be in 0..15");
    if (!ws || ws_bytes < hg_lowrank_ws(n, o, k)) return fail(KQ_EWORKSPACE, "kq_hg_lowrank: workspace too small");
    hipStream_t st = hs(stream);
    KQ_TRY(refuse_capture(st, "kq_hg_lowrank"));
    Arena ar(ws, ws_bytes);
    double* Gd = ar.take<double>((size_t)n * o);
    double* Y = ar.take<double>((size_t)o * k);
    double* GQ = ar.take<double>((size_t)n * k);
    double* Yt = ar.take<double>((size_t)o * k);
    double* Q = ar.take<double>((size_t)o * k);
    double* C = ar.take<double>((size_t)k * k);
    double* X = ar.take<double>((size_t)k * k);
    double* Tscr = ar.take<double>((size_t)(k * k / 2 + 128 * 128));
    double* cscr = ar.take<double>((size_t)chol_scratch_doubles());
    double* B = ar.take<double>((size_t)k * k);
    double* core = ar.take<double>((size_t)k * k);
    double* QC = ar.take<double>((size_t)o * k);
    double* OO = ar.take<double>((size_t)o * o);
    double* part = ar.take<double>(SQ_PARTS);
    double* sig = ar.take<double>(2);
    int32_t* pinfo = ar.take<int32_t>(32);
    int32_t* dbinfo = ar.take<int32_t>(1);
    int* flags = ar.take<int>(4);
    const size_t sq_bytes = hg_sqrt_ws(KQ_HG_FULL, k, 0);
    void* sqws = ar.take<char>(sq_bytes);
    const double inv_n = 1.0 / (double)n;

    KQ_TRY(fill<int>(reinterpret_cast<int*>(pinfo), 32, 0, st));
    hipLaunchKernelGGL(widen_rows_kernel, dim3(grid_for(n * o)), dim3(256), 0, st, G, ldg, n, o, Gd);
    KQ_TRY(check_launch("lowrank widen G"));
    hipLaunchKernelGGL(sumsq_part_kernel, dim3(SQ_PARTS), dim3(256), 0, st, Gd, n * o, part);
    KQ_TRY(check_launch("lowrank trace"));
    hipLaunchKernelGGL(widen_rows_kernel, dim3(grid_for(o * k)), dim3(256), 0, st, omega, k, o, k, Yt);
    KQ_TRY(check_launch("lowrank widen omega"));
    // range finder: Y = H Omega = G^T (G Omega) / n, then q power steps Y = H Q
    const double* basis = Yt;
    for (int p = 0; p <= q; p++) {
        GemmArgs<double> a = gemm_args<double>(n, k, o, Gd, o, basis, k, GQ, k, 1.0, 0.0);
        KQ_TRY(gemm<double>(a, false, false, st));
        GemmArgs<double> b = gemm_args<double>(o, k, n, Gd, o, GQ, k, Y, k, inv_n, 0.0);
        KQ_TRY(gemm<double>(b, true, false, st));
        KQ_TRY(orth(Y, Q, Yt, o, k, C, X, Tscr, cscr, pinfo + 2 * p, st));
        basis = Q;
    }
    // B = Q^T H Q = (G Q)^T (G Q) / n
    GemmArgs<double> a = gemm_args<double>(n, k, o, Gd, o, Q, k, GQ, k, 1.0, 0.0);
    KQ_TRY(gemm<double>(a, false, false, st));
    GemmArgs<double> b = gemm_args<double>(k, k, n, GQ, k, GQ, k, B, k, inv_n, 0.0);
    KQ_TRY(gemm<double>(b, true, false, st));
    hipLaunchKernelGGL(lowrank_sigma_kernel, dim3(1), dim3(256), 0, st, part, inv_n, B, k, o, sig, flags);
    KQ_TRY(check_launch("lowrank sigma"));
    if (sigma) {
        hipLaunchKernelGGL(copy_pair_kernel, dim3(1), dim3(64), 0, st, sig, sigma);
        KQ_TRY(check_launch("lowrank sigma out"));
    }
    // B^{1/2} and B^{-1/2}
    double* YZ = nullptr;
    KQ_TRY(spd_sqrt_f64(B, k, dbinfo, sqws, sq_bytes, &YZ, st));
    // S = sqrt(sigma) I + Q (B^{1/2} - sqrt(sigma) I) Q^T; S^{-1} with B^{-1/2} and 1/sqrt(sigma);
    // H^ = sigma I + Q (B - sigma I) Q^T
    const double* src[3] = {YZ, YZ + (size_t)k * k, B};
    float* dst[3] = {S, Sinv, HGhat};
    for (int m = 0; m < 3; m++) {
        if (!dst[m]) continue;
        hipLaunchKernelGGL(shift_diag_kernel, dim3(grid_for(k * k)), dim3(256), 0, st, src[m], k, sig, m, core);
        KQ_TRY(check_launch("lowrank core"));
        GemmArgs<double> c1 = gemm_args<double>(o, k, k, Q, k, core, k, QC, k, 1.0, 0.0);
        KQ_TRY(gemm<double>(c1, false, false, st));
        GemmArgs<double> c2 = gemm_args<double>(o, o, k, QC, k, Q, k, OO, o, 1.0, 0.0);
        KQ_TRY(gemm<double>(c2, false, true, st));
        hipLaunchKernelGGL(add_diag_out_kernel, dim3(grid_for(o * o)), dim3(256), 0, st, OO, o, sig, m, dst[m]);
        KQ_TRY(check_launch("lowrank out"));
    }
    hipLaunchKernelGGL(lowrank_info_kernel, dim3(1), dim3(64), 0, st, pinfo, 2 * (q + 1), flags, dbinfo, info);
    return check_launch("lowrank info");
}

extern "C" kq_status kq_hg_extract(const double* H, int64_t o, int64_t ldh, kq_hg_form form, int64_t blk, float* HG,
                                   kq_stream stream) {
    if (!H || !HG) return fail(KQ_EINVAL, "kq_hg_extract: null pointer");
    if (o <= 0 || ldh < o) return fail(KQ_ESHAPE, "kq_hg_extract: bad sizes");
    if (form != KQ_HG_DIAG && form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "kq_hg_extract: form");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "kq_hg_extract: bad block size");
    hipStream_t st = hs(stream);
    const int64_t total = form == KQ_HG_FULL ? o * o : form == KQ_HG_BLOCK ? o * blk : o;
    hipLaunchKernelGGL(hg_extract_kernel, dim3(grid_for(total)), dim3(256), 0, st, H, o, ldh, (int)form, blk, HG);
    return check_launch("hg_extract");
}

size_t kfac_loss_ws(int64_t o, int64_t i, kq_hg_form form, int64_t blk) {
    Sizer z;
    z.take<double>((size_t)o * i);   // dW
    z.take<double>((size_t)o * i);   // dW H_X
    z.take<double>((size_t)o * i);   // H_G dW
    const size_t hg = form == KQ_HG_FULL ? (size_t)o * o : form == KQ_HG_BLOCK ? (size_t)o * blk : 0;
    z.take<double>(hg);
    z.take<double>(SQ_PARTS);
    return z.used;
}

extern "C" kq_status kq_kfac_loss(const void* W, kq_dtype wdt, int64_t ldw, const float* What, int64_t ldq, int64_t o,
                                  int64_t i, const double* HX, int64_t ldh, const float* HG, kq_hg_form form,
                                  int64_t blk, double* loss, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!W || !What || !HX || !HG || !loss) return fail(KQ_EINVAL, "kq_kfac_loss: null pointer");
    if (o <= 0 || i <= 0 || ldw < i || ldq < i || ldh < i) return fail(KQ_ESHAPE, "kq_kfac_loss: bad sizes");
    if (wdt != KQ_F32 && wdt != KQ_BF16) return fail(KQ_EINVAL, "kq_kfac_loss: W must be fp32 or bf16");
    if (form != KQ_HG_DIAG && form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "kq_kfac_loss: form");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "kq_kfac_loss: bad block size");
    if (!ws || ws_bytes < kfac_loss_ws(o, i, form, blk)) return fail(KQ_EWORKSPACE, "kq_kfac_loss: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    double* D = ar.take<double>((size_t)o * i);
    double* A = ar.take<double>((size_t)o * i);
    double* Bm = ar.take<double>((size_t)o * i);
    const size_t hgn = form == KQ_HG_FULL ? (size_t)o * o : form == KQ_HG_BLOCK ? (size_t)o * blk : 0;
    double* H64 = ar.take<double>(hgn);
    double* part = ar.take<double>(SQ_PARTS);
    hipLaunchKernelGGL(diff_f64_kernel, dim3(grid_for(o * i)), dim3(256), 0, st, W, wdt == KQ_BF16 ? 1 : 0, ldw, What,
                       ldq, o, i, D);
    KQ_TRY(check_launch("kfac diff"));
    // A = dW H_X
    GemmArgs<double> ga = gemm_args<double>(o, i, i, D, i, HX, ldh, A, i, 1.0, 0.0);
    KQ_TRY(gemm<double>(ga, false, false, st));
    // Bm = H_G dW
    if (form == KQ_HG_DIAG) {
        hipLaunchKernelGGL(hg_rows_kernel, dim3(grid_for(o * i)), dim3(256), 0, st, HG, D, o, i, Bm);
        KQ_TRY(check_launch("kfac hg rows"));
    } else {
        const int64_t cols = form == KQ_HG_FULL ? o : blk;   // full: o x o; block: o rows of blk
        hipLaunchKernelGGL(widen_rows_kernel, dim3(grid_for((int64_t)hgn)), dim3(256), 0, st, HG, cols, o, cols, H64);
        KQ_TRY(check_launch("kfac widen hg"));
        if (form == KQ_HG_FULL) {
            GemmArgs<double> gb = gemm_args<double>(o, i, o, H64, o, D, i, Bm, i, 1.0, 0.0);
            KQ_TRY(gemm<double>(gb, false, false, st));
        } else {
            GemmArgs<double> gb = gemm_args<double>(blk, i, blk, H64, blk, D, i, Bm, i, 1.0, 0.0);
            gb.nb1 = o / blk; gb.sA1 = blk * blk; gb.sB1 = blk * i; gb.sC1 = blk * i;
            KQ_TRY(gemm<double>(gb, false, false, st));
        }
    }
    hipLaunchKernelGGL(dot_part_kernel, dim3(SQ_PARTS), dim3(256), 0, st, A, Bm, o * i, part);
    KQ_TRY(check_launch("kfac dot"));
    hipLaunchKernelGGL(sum_parts_kernel, dim3(1), dim3(256), 0, st, part, loss);
    return check_launch("kfac sum");
}

// ------------------------------------------------------------------------------ block column order
// Trace-sorted block order (H_Z-PTQ page, Weight scales and rounding: before the sweep the block
// rows and columns are sorted so that blocks with larger curvature traces are quantized first, as
// GPTQ's act-order does for columns). order[k] = the block with the k-th largest trace of its
// diagonal of H (ties: lower block index first); order[nb + b] = the position of block b.
__global__ void block_order_kernel(const double* __restrict__ H, int64_t ldh, int64_t nb, int64_t width,
                                   int32_t* __restrict__ order) {
    extern __shared__ double tr[];
    for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
        double s = 0.0;
        for (int64_t c = 0; c < width; c++) s += H[(b * width + c) * ldh + b * width + c];
        tr[b] = s;
    }
    __syncthreads();
    for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
        int64_t rank = 0;
        for (int64_t a = 0; a < nb; a++) rank += (tr[a] > tr[b]) || (tr[a] == tr[b] && a < b);
        order[rank] = (int32_t)b;
        order[nb + b] = (int32_t)rank;
    }
}

// Column blocks (axis 0) or row blocks (axis 1) of a rows x cols matrix: out block k = in block
// perm[k] (pass the second half of kq_block_order's output to undo its first half).
template <typename T>
__global__ void permute_blocks_kernel(const T* __restrict__ in, int64_t ldi, T* __restrict__ out, int64_t ldo,
                                      int64_t rows, int64_t cols, int64_t width, int axis, const int32_t* __restrict__ perm) {
    const int64_t total = rows * cols;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / cols, c = e % cols;
        const int64_t idx = axis == 0 ? c : r;            // position along the permuted axis (output)
        const int64_t src = (int64_t)perm[idx / width] * width + idx % width;
        out[r * ldo + c] = axis == 0 ? in[r * ldi + src] : in[src * ldi + c];
    }
}

extern "C" kq_status kq_block_order(const double* H, int64_t i, int64_t ldh, int64_t width, int32_t* order,
                                    kq_stream stream) {
    if (!H || !order) return fail(KQ_EINVAL, "kq_block_order: null pointer");
    if (i <= 0 || width <= 0 || i % width || ldh < i) return fail(KQ_ESHAPE, "kq_block_order: bad sizes");
    const int64_t nb = i / width;
    if (nb > 4096) return fail(KQ_ESHAPE, "kq_block_order: at most 4096 blocks");
    hipStream_t st = hs(stream);
    hipLaunchKernelGGL(block_order_kernel, dim3(1), dim3(256), (size_t)nb * sizeof(double), st, H, ldh, nb, width, order);
    return check_launch("block_order");
}

extern "C" kq_status kq_permute_blocks(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t rows, int64_t cols,
                                       int64_t width, int axis, int elem_bytes, const int32_t* perm,
                                       kq_stream stream) {
    if (!in || !out || !perm) return fail(KQ_EINVAL, "kq_permute_blocks: null pointer");
    if (in == out) return fail(KQ_EINVAL, "kq_permute_blocks: in and out must differ");
    if (rows <= 0 || cols <= 0 || width <= 0 || ldi < cols || ldo < cols) return fail(KQ_ESHAPE, "kq_permute_blocks: bad sizes");
    if ((axis == 0 && cols % width) || (axis == 1 && rows % width) || (axis != 0 && axis != 1))
        return fail(KQ_ESHAPE, "kq_permute_blocks: the permuted extent must be a multiple of width");
    hipStream_t st = hs(stream);
    const int64_t total = rows * cols;
    const unsigned g = grid_for(total);
    if (elem_bytes == 4)
        hipLaunchKernelGGL(permute_blocks_kernel<uint32_t>, dim3(g), dim3(256), 0, st, static_cast<const uint32_t*>(in),
                           ldi, static_cast<uint32_t*>(out), ldo, rows, cols, width, axis, perm);
    else if (elem_bytes == 8)
        hipLaunchKernelGGL(permute_blocks_kernel<uint64_t>, dim3(g), dim3(256), 0, st, static_cast<const uint64_t*>(in),
                           ldi, static_cast<uint64_t*>(out), ldo, rows, cols, width, axis, perm);
    else
        return fail(KQ_EINVAL, "kq_permute_blocks: elements must be 4 or 8 bytes");
    return check_launch("permute_blocks");
}

// ------------------------------------------------------------------------------ input drift
// GPTAQ-style correction of the input drift (KronQ review page, Prior limitations: GPTAQ corrects for
// the drift of a layer's input caused by quantizing earlier layers, still with H_X only; the
// solver's formula is not on the pages). Reading used here: with X the full-precision inputs and
// X~ the drifted ones, || W^ X~^T - W X^T ||^2 = || (W^ - W*) X~^T ||^2 + const for
//     W* = W C (H~ + lambda I)^{-1},  C = X^T X~ / n,  H~ = X~^T X~ / n
// (exact for lambda = 0; with lambda the ridge solution), so the drift moves the target from W to W*
// and the unchanged sweep then runs on (W*, H~).

__global__ void widen_any_kernel(const void* __restrict__ src, int bf16, int64_t ld, int64_t rows, int64_t cols,
                                 double* __restrict__ dst) {
    const int64_t total = rows * cols;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / cols, c = e % cols;
        dst[e] = bf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(src)[r * ld + c] << 16)
                      : (double)static_cast<const float*>(src)[r * ld + c];
    }
}

__global__ void narrow_kernel(const double* __restrict__ src, int64_t rows, int64_t cols, float* __restrict__ dst,
                              int64_t ldd) {
    const int64_t total = rows * cols;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
        dst[(e / cols) * ldd + e % cols] = (float)src[e];
}

constexpr int64_t XC_CHUNK = 8192;   // token rows widened per step

size_t cross_ws(int64_t n, int64_t d) {
    const int64_t c = n < XC_CHUNK ? n : XC_CHUNK;
    Sizer z;
    z.take<double>((size_t)c * d);
    z.take<double>((size_t)c * d);
    return z.used;
}

extern "C" kq_status kq_cross_accum(const void* A, const void* B, kq_dtype dt, int64_t n, int64_t d, int64_t lda,
                                    int64_t ldb, double alpha, double beta, double* C, void* ws, size_t ws_bytes,
                                    kq_stream stream) {
    if (!A || !B || !C) return fail(KQ_EINVAL, "kq_cross_accum: null pointer");
    if (n <= 0 || d <= 0 || lda < d || ldb < d) return fail(KQ_ESHAPE, "kq_cross_accum: bad sizes");
    if (dt != KQ_F32 && dt != KQ_BF16) return fail(KQ_EINVAL, "kq_cross_accum: inputs must be fp32 or bf16");
    if (!ws || ws_bytes < cross_ws(n, d)) return fail(KQ_EWORKSPACE, "kq_cross_accum: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    const int64_t chunk = n < XC_CHUNK ? n : XC_CHUNK;
    double* Ad = ar.take<double>((size_t)chunk * d);
    double* Bd = ar.take<double>((size_t)chunk * d);
    const int bf = dt == KQ_BF16 ? 1 : 0;
    const size_t es = bf ? 2 : 4;
    for (int64_t r0 = 0; r0 < n; r0 += chunk) {
        const int64_t m = n - r0 < chunk ? n - r0 : chunk;
        hipLaunchKernelGGL(widen_any_kernel, dim3(grid_for(m * d)), dim3(256), 0, st,
                           static_cast<const char*>(A) + (size_t)r0 * lda * es, bf, lda, m, d, Ad);
        hipLaunchKernelGGL(widen_any_kernel, dim3(grid_for(m * d)), dim3(256), 0, st,
                           static_cast<const char*>(B) + (size_t)r0 * ldb * es, bf, ldb, m, d, Bd);
        KQ_TRY(check_launch("cross widen"));
        // C = alpha A^T B + (first chunk: beta, then 1) C
        GemmArgs<double> g = gemm_args<double>(d, d, m, Ad, d, Bd, d, C, d, alpha, r0 == 0 ? beta : 1.0);
        KQ_TRY(gemm<double>(g, true, false, st));
    }
    return KQ_OK;
}

size_t drift_ws(int64_t o, int64_t i) {
    Sizer z;
    z.take<double>((size_t)o * i);   // W
    z.take<double>((size_t)o * i);   // W C
    z.take<double>((size_t)o * i);   // (W C) R^T
    z.take<double>((size_t)i * i);   // R
    return z.used;
}

extern "C" kq_status kq_drift_target(const void* W, kq_dtype wdt, int64_t ldw, int64_t o, int64_t i, const double* C,
                                     int64_t ldc, const float* R, int64_t ldr, float* Wt, int64_t ldt, void* ws,
                                     size_t ws_bytes, kq_stream stream) {
    if (!W || !C || !R || !Wt) return fail(KQ_EINVAL, "kq_drift_target: null pointer");
    if (o <= 0 || i <= 0 || ldw < i || ldc < i || ldr < i || ldt < i) return fail(KQ_ESHAPE, "kq_drift_target: bad sizes");
    if (wdt != KQ_F32 && wdt != KQ_BF16) return fail(KQ_EINVAL, "kq_drift_target: W must be fp32 or bf16");
    if (!ws || ws_bytes < drift_ws(o, i)) return fail(KQ_EWORKSPACE, "kq_drift_target: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    double* Wd = ar.take<double>((size_t)o * i);
    double* T1 = ar.take<double>((size_t)o * i);
    double* T2 = ar.take<double>((size_t)o * i);
    double* Rd = ar.take<double>((size_t)i * i);
    hipLaunchKernelGGL(widen_any_kernel, dim3(grid_for(o * i)), dim3(256), 0, st, W, wdt == KQ_BF16 ? 1 : 0, ldw, o, i, Wd);
    hipLaunchKernelGGL(widen_rows_kernel, dim3(grid_for(i * i)), dim3(256), 0, st, R, ldr, i, i, Rd);
    KQ_TRY(check_launch("drift widen"));
    // W* = ((W C) R^T) R with (H~ + lambda I)^{-1} = R^T R
    GemmArgs<double> a = gemm_args<double>(o, i, i, Wd, i, C, ldc, T1, i, 1.0, 0.0);
    KQ_TRY(gemm<double>(a, false, false, st));
    GemmArgs<double> b = gemm_args<double>(o, i, i, T1, i, Rd, i, T2, i, 1.0, 0.0);
    KQ_TRY(gemm<double>(b, false, true, st));
    GemmArgs<double> c = gemm_args<double>(o, i, i, T2, i, Rd, i, T1, i, 1.0, 0.0);
    KQ_TRY(gemm<double>(c, false, false, st));
    hipLaunchKernelGGL(narrow_kernel, dim3(grid_for(o * i)), dim3(256), 0, st, T1, o, i, Wt, ldt);
    return check_launch("drift narrow");
}
