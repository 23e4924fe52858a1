// H_X accumulation H <- beta H + alpha X^T X (KronQ review page, Background: the input activation
// covariance used as the layer-Hessian proxy).
//
// H is kept in fp64: the damped factor R of H^{-1} is as sensitive to H as cond(H) makes it, and
// rounding H to fp32 alone moves the sweep's pre-rounding values by up to ~2e-4 grid steps on the
// 4096-wide layers (cond ~2e5 after damping).
// bf16 X: bf16 x bf16 products are exact, so the gfx950 bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16) form exact products; each 64-token stage runs two instructions into an
// fp32 accumulator that starts at zero, and the stage's 64-product sum is added into fp64
// registers, so two fp32 roundings per 64 tokens enter the result. Only the lower-triangle
// 128 x 128 tiles of H are computed; a fixed split over tokens with a fixed-order fp64 reduction
// keeps the result deterministic, and both triangles are written.
// fp32 X: the fp64 MFMA GEMM on the widened values (small workloads only).
#include "kq_internal.h"

namespace kq {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

constexpr int SY_T = 128;   // output tile
constexpr int SY_K = 64;    // tokens per LDS sub-tile (and per fp32 chain flushed into fp64)
constexpr int SY_H = 2;     // sub-tiles per stage: a stage loads SY_H * SY_K tokens

struct alignas(16) U4 {
    uint32_t w[4];
};

// Tile t of the lower triangle (row-major over tm >= tn) -> (tm, tn).
__device__ inline void tri_decode(int t, int& tm, int& tn) {
    int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (r * (r + 1) / 2 > t) r--;
    while ((r + 1) * (r + 2) / 2 <= t) r++;
    tm = r;
    tn = t - r * (r + 1) / 2;
}

// LDS tile [128 rows][64 k] bf16, rows of 128 bytes made of eight 16-byte chunks; chunk c of row m is
// stored at position c ^ (m & 7) ^ ((m >> 3) & 7): the 16 consecutive rows read by an MFMA operand
// and the rows 8 apart written by one store instruction of the loaders both spread over the banks.
__device__ inline int lds_off(int m, int c) { return m * SY_K + ((c ^ (m & 7) ^ ((m >> 3) & 7)) << 3); }

// 512 threads = 8 waves; wave w owns rows 32 (w / 2) .. + 31 and columns 64 (w % 2) .. + 63 of the
// tile (2 x 4 MFMA tiles). Threads 0..255 stage X through registers into LDS (an 8 x 8 transpose of
// 16-bit values per thread), double-buffered with one barrier per 128-token stage: the loads of the
// next stage are issued before the current stage's products and have both 64-token halves of them to
// arrive in (with 64-token stages the waves spent about half their time waiting). 128 KB of LDS.
constexpr int SY_THREADS = 512;
constexpr size_t SY_SMEM = size_t(2) * 2 * SY_H * SY_T * SY_K * sizeof(uint16_t);
__global__ __launch_bounds__(SY_THREADS) void syrk_bf16_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t d,
                                                               int64_t ldx, int64_t tok_per_split, double alpha,
                                                               double beta, double* __restrict__ H,
                                                               double* __restrict__ part, int ntiles) {
    extern __shared__ __align__(16) uint16_t sy_lds[];
    // [buffer][half][SY_T * SY_K], A then B
    auto As = [&](int buf, int h) { return sy_lds + (size_t)(buf * SY_H + h) * SY_T * SY_K; };
    auto Bs = [&](int buf, int h) { return sy_lds + (size_t)((2 + buf) * SY_H + h) * SY_T * SY_K; };
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x, split = blockIdx.y;
    int tm, tn;
    tri_decode(tile, tm, tn);
    const int64_t m0 = (int64_t)tm * SY_T, n0 = (int64_t)tn * SY_T;
    const int64_t kb = (int64_t)split * tok_per_split;
    const int64_t ke = (kb + tok_per_split < n) ? kb + tok_per_split : n;

    // loader role (threads 0..255): 0..127 stage the row block (A), 128..255 the column block (B)
    const bool loader = tid < 256;
    const int op = (tid >> 7) & 1, p = tid & 127, kg = p >> 4, mc = p & 15;
    const int64_t cbase = (op ? n0 : m0) + 8 * mc;
    const bool fullc = cbase + 8 <= d;
    U4 v[SY_H][8];

    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int jj = 0; jj < SY_H * 8; jj++) {
            const int h = jj >> 3, j = jj & 7;
            const int64_t k = k0 + SY_K * h + 8 * kg + j;
            const uint16_t* src = X + k * ldx + cbase;
            if (k < ke && fullc) {
                v[h][j] = *reinterpret_cast<const U4*>(src);
            } else {
                uint16_t tmp[8];
#pragma unroll
                for (int e = 0; e < 8; e++) tmp[e] = (k < ke && cbase + e < d) ? src[e] : (uint16_t)0;
#pragma unroll
                for (int q = 0; q < 4; q++) v[h][j].w[q] = (uint32_t)tmp[2 * q] | ((uint32_t)tmp[2 * q + 1] << 16);
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < SY_H; h++) {
            // 8 x 8 transpose of 16-bit elements: out[mm] holds k = 0..7 of column 8*mc + mm
            U4 out[8];
#pragma unroll
            for (int q = 0; q < 4; q++) {
#pragma unroll
                for (int jp = 0; jp < 4; jp++) {
                    const uint32_t x = v[h][2 * jp].w[q], y = v[h][2 * jp + 1].w[q];
                    out[2 * q].w[jp] = (x & 0xFFFFu) | (y << 16);
                    out[2 * q + 1].w[jp] = (x >> 16) | (y & 0xFFFF0000u);
                }
            }
            uint16_t* dst = op ? Bs(buf, h) : As(buf, h);
#pragma unroll
            for (int mm = 0; mm < 8; mm++) {
                const int m = 8 * mc + mm;
                *reinterpret_cast<U4*>(dst + lds_off(m, kg)) = out[mm];
            }
        }
    };

    double acc[2][4][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[i][j][r] = 0.0;
    const int wm = wave >> 1, wn = wave & 1;

    if (kb < ke) {
        if (loader) {
            gload(kb);
            sstore(0);
        }
        __syncthreads();
        int buf = 0;
        for (int64_t k0 = kb; k0 < ke; k0 += SY_H * SY_K) {
            const bool more = k0 + SY_H * SY_K < ke;
            if (more && loader) gload(k0 + SY_H * SY_K);
#pragma unroll
            for (int h = 0; h < SY_H; h++) {
                if (h > 0 && k0 + SY_K * h >= ke) break;   // a last half past the split's end
                const uint16_t* Ah = As(buf, h);
                const uint16_t* Bh = Bs(buf, h);
                f4v pacc[2][4];
#pragma unroll
                for (int s = 0; s < 2; s++) {
                    bf8v a[2], b[4];
                    const int c = 4 * s + (lane >> 4);
#pragma unroll
                    for (int i = 0; i < 2; i++) {
                        const int m = wm * 32 + 16 * i + (lane & 15);
                        a[i] = *reinterpret_cast<const bf8v*>(Ah + lds_off(m, c));
                    }
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int nn = wn * 64 + 16 * j + (lane & 15);
                        b[j] = *reinterpret_cast<const bf8v*>(Bh + lds_off(nn, c));
                    }
#pragma unroll
                    for (int i = 0; i < 2; i++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            pacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j],
                                                                                 s ? pacc[i][j] : f4v{0, 0, 0, 0}, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
#pragma unroll
                        for (int r = 0; r < 4; r++) acc[i][j][r] += (double)pacc[i][j][r];
            }
            if (more && loader) sstore(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    if (part) {
        double* out = part + ((int64_t)split * ntiles + tile) * (SY_T * SY_T);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int mm = wm * 32 + 16 * i + 4 * (lane >> 4) + r, nn = wn * 64 + 16 * j + (lane & 15);
                    out[mm * SY_T + nn] = acc[i][j][r];
                }
    } else {
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int64_t m = m0 + wm * 32 + 16 * i + 4 * (lane >> 4) + r;
                    const int64_t c = n0 + wn * 64 + 16 * j + (lane & 15);
                    if (m >= d || c >= d || c > m) continue;
                    double val = alpha * acc[i][j][r];
                    if (beta != 0.0) val += beta * H[m * d + c];
                    H[m * d + c] = val;
                    H[c * d + m] = val;
                }
    }
}

// Sum the token splits in order, scale, and write both triangles.
__global__ void syrk_reduce_kernel(const double* __restrict__ part, int nsplit, int ntiles, int64_t d, double alpha,
                                   double beta, double* __restrict__ H) {
    const int tile = blockIdx.x;
    int tm, tn;
    tri_decode(tile, tm, tn);
    for (int e = threadIdx.x; e < SY_T * SY_T; e += blockDim.x) {
        const int mm = e / SY_T, nn = e % SY_T;
        const int64_t m = (int64_t)tm * SY_T + mm, c = (int64_t)tn * SY_T + nn;
        if (m >= d || c >= d || c > m) continue;
        double s = 0.0;
        for (int k = 0; k < nsplit; k++) s += part[((int64_t)k * ntiles + tile) * (SY_T * SY_T) + e];
        double val = alpha * s;
        if (beta != 0.0) val += beta * H[m * d + c];
        H[m * d + c] = val;
        H[c * d + m] = val;
    }
}

__global__ void mirror_lower_kernel(double* H, int64_t d) {
    const int64_t r = blockIdx.y;
    for (int64_t c = r + 1 + blockIdx.x * 256 + threadIdx.x; c < d; c += (int64_t)gridDim.x * 256) H[r * d + c] = H[c * d + r];
}

__global__ void scale_kernel(double* H, int64_t count, double beta) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256)
        H[e] = beta == 0.0 ? 0.0 : beta * H[e];
}

// fp32 X widened to fp64 (exact), for the fp64 GEMM path.
__global__ void widen_kernel(const float* __restrict__ X, int64_t n, int64_t d, int64_t ldx, double* __restrict__ Y) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < n * d; e += (int64_t)gridDim.x * 256)
        Y[e] = (double)X[(e / d) * ldx + e % d];
}

static void syrk_plan(int64_t n, int64_t d, int& ntiles, int& nsplit, int64_t& tps) {
    const int64_t nt = (d + SY_T - 1) / SY_T;
    ntiles = (int)(nt * (nt + 1) / 2);
    int64_t s = (2048 + ntiles - 1) / ntiles;
    const int64_t smax = (n + 1023) / 1024;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    tps = ((n + s - 1) / s + SY_H * SY_K - 1) / (SY_H * SY_K) * (SY_H * SY_K);
    nsplit = (int)((n + tps - 1) / tps);
    if (nsplit < 1) nsplit = 1;
}

}  // namespace kq

using namespace kq;

size_t hessian_ws(int64_t n, int64_t d, kq_dtype xdt) {
    if (n <= 0) return 0;
    if (xdt != KQ_BF16) return (size_t)n * d * sizeof(double) + 256;
    int ntiles, nsplit;
    int64_t tps;
    syrk_plan(n, d, ntiles, nsplit, tps);
    if (nsplit <= 1) return 0;
    return (size_t)nsplit * ntiles * SY_T * SY_T * sizeof(double) + 256;
}

extern "C" kq_status kq_hessian_accum(const void* X, kq_dtype xdt, int64_t n, int64_t d, int64_t ldx, double alpha,
                                      double beta, double* H, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!H) return fail(KQ_EINVAL, "kq_hessian_accum: null H");
    if (d <= 0 || n < 0) return fail(KQ_ESHAPE, "kq_hessian_accum: bad sizes");
    if (xdt != KQ_F32 && xdt != KQ_BF16) return fail(KQ_EINVAL, "kq_hessian_accum: bad dtype");
    if (!aligned16(H)) return fail(KQ_EINVAL, "kq_hessian_accum: H must be 16-byte aligned");
    hipStream_t st = hs(stream);
    if (n == 0) {
        unsigned b = (unsigned)((d * d + 255) / 256 < 4096 ? (d * d + 255) / 256 : 4096);
        hipLaunchKernelGGL(scale_kernel, dim3(b), dim3(256), 0, st, H, d * d, beta);
        return check_launch("hessian scale");
    }
    if (!X) return fail(KQ_EINVAL, "kq_hessian_accum: null X");
    if (ldx < d) return fail(KQ_ESHAPE, "kq_hessian_accum: ldx < d");
    if (!aligned16(X) || (xdt == KQ_BF16 ? ldx % 8 : ldx % 4))
        return fail(KQ_EINVAL, "kq_hessian_accum: X must be 16-byte aligned with ldx a multiple of 16 bytes");
    if (d > 65535) return fail(KQ_ESHAPE, "kq_hessian_accum: d too large");
    if (xdt == KQ_F32) {
        if (!ws || ws_bytes < hessian_ws(n, d, xdt)) return fail(KQ_EWORKSPACE, "kq_hessian_accum: workspace too small");
        double* Y = reinterpret_cast<double*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
        unsigned b = (unsigned)((n * d + 255) / 256 < 8192 ? (n * d + 255) / 256 : 8192);
        hipLaunchKernelGGL(widen_kernel, dim3(b), dim3(256), 0, st, static_cast<const float*>(X), n, d, ldx, Y);
        KQ_TRY(check_launch("hessian widen"));
        GemmArgs<double> g = gemm_args<double>(d, d, n, Y, d, Y, d, H, d, alpha, beta);
        g.tri = 1;
        KQ_TRY(gemm<double>(g, true, false, st));
        dim3 gm((unsigned)((d + 255) / 256 < 64 ? (d + 255) / 256 : 64), (unsigned)d);
        hipLaunchKernelGGL(mirror_lower_kernel, gm, dim3(256), 0, st, H, d);
        return check_launch("hessian mirror");
    }
    int ntiles, nsplit;
    int64_t tps;
    syrk_plan(n, d, ntiles, nsplit, tps);
    double* part = nullptr;
    if (nsplit > 1) {
        if (!ws || ws_bytes < hessian_ws(n, d, xdt)) return fail(KQ_EWORKSPACE, "kq_hessian_accum: workspace too small");
        part = reinterpret_cast<double*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
    }
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&syrk_bf16_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)SY_SMEM);
        attr = true;
    }
    hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)ntiles, (unsigned)nsplit), dim3(SY_THREADS), SY_SMEM, st,
                       static_cast<const uint16_t*>(X), n, d, ldx, tps, alpha, beta, H, part, ntiles);
    KQ_TRY(check_launch("syrk_bf16"));
    if (nsplit > 1) {
        hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)ntiles), dim3(256), 0, st, part, nsplit, ntiles, d, alpha,
                           beta, H);
        KQ_TRY(check_launch("syrk_reduce"));
    }
    return KQ_OK;
}
