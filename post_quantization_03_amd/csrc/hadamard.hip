// Random-sign Hadamard rotations of bidirectional incoherence processing (KronQ review page, Method
// (1) and "Where this paper sits": the input-side QuIP/QuIP# Hadamard rotation, extended to the
// output side after the H_G^{1/2} factor).
//
// H_d = P_m (x) H_{2^k} for d = m 2^k: Sylvester's H_{2^k} acts on every contiguous 2^k chunk of an
// index, and a Paley type-I matrix P_m (order q + 1 over GF(q), q = 3 mod 4) mixes the m chunks.
//  - along rows (contiguous): one work-group per row keeps the row in LDS and runs radix-4/radix-2
//    butterflies; sign and scale are fused into the load and the store;
//  - along columns (the output axis of row-major W, and the second side of H_X): "digit passes"
//    load a D x 64 tile of rows that differ in one base-D digit of the row index into LDS and
//    transform along it, so every pass streams the matrix once with 256-byte row segments;
//  - the P_m factor is a dense +-1 contraction, run on the fp32 MFMA GEMM (P is generated on the
//    device from the finite-field quadratic character).
#include <cmath>
#include <mutex>

#include "kq_internal.h"

namespace kq {

// ------------------------------------------------------------------------------ finite fields
struct Field {
    int q = 0, p = 0, e = 0, c0 = 0, c1 = 0, c2 = 0;  // GF(p^e); e = 3: modulus t^3 + c2 t^2 + c1 t + c0
};

static bool is_prime(int64_t n) {
    if (n < 2) return false;
    for (int64_t f = 2; f * f <= n; f++)
        if (n % f == 0) return false;
    return true;
}

static bool field_for(int64_t q, Field& f) {
    if (q % 4 != 3) return false;
    if (is_prime(q) && q < 46341) { f.q = (int)q; f.p = (int)q; f.e = 1; return true; }
    if (q == 27) { f.q = 27; f.p = 3; f.e = 3; f.c0 = 2; f.c1 = 2; f.c2 = 0; return true; }
    if (q == 343) { f.q = 343; f.p = 7; f.e = 3; f.c0 = 5; f.c1 = 0; f.c2 = 0; return true; }
    return false;
}

// d = m * p2 with m the smallest order (odd part of d) * 2^a that is 1 or q + 1 for a supported q.
static bool hadamard_split(int64_t d, int64_t& m, int64_t& p2, Field& f) {
    if (d <= 0) return false;
    const int64_t two = d & (-d), odd = d / two;
    for (int64_t a = 1; a <= two; a *= 2) {
        const int64_t mm = odd * a;
        if (mm == 1) { m = 1; p2 = d; f = Field{}; return true; }
        if (field_for(mm - 1, f)) { m = mm; p2 = d / mm; return true; }
    }
    return false;
}

__device__ inline void gf_mul3(const int* a, const int* b, int* out, int p, int c0, int c1, int c2) {
    int t[5] = {0, 0, 0, 0, 0};
    for (int i = 0; i < 3; i++)
        for (int j = 0; j < 3; j++) t[i + j] = (t[i + j] + a[i] * b[j]) % p;
    for (int deg = 4; deg >= 3; deg--) {
        const int c = t[deg];
        if (!c) continue;
        t[deg] = 0;
        t[deg - 1] = ((t[deg - 1] - c * c2) % p + p) % p;
        t[deg - 2] = ((t[deg - 2] - c * c1) % p + p) % p;
        t[deg - 3] = ((t[deg - 3] - c * c0) % p + p) % p;
    }
    out[0] = t[0]; out[1] = t[1]; out[2] = t[2];
}

// Quadratic character of element index x (base-p digits) of GF(q): x^((q-1)/2) is 1 or -1.
__device__ inline int gf_chi(int x, Field f) {
    if (x == 0) return 0;
    const int ex = (f.q - 1) / 2;
    if (f.e == 1) {
        int64_t r = 1, b = x, k = ex;
        while (k) {
            if (k & 1) r = (r * b) % f.q;
            b = (b * b) % f.q;
            k >>= 1;
        }
        return r == 1 ? 1 : -1;
    }
    int base[3] = {x % f.p, (x / f.p) % f.p, x / (f.p * f.p)};
    int r[3] = {1, 0, 0};
    int k = ex;
    while (k) {
        if (k & 1) gf_mul3(r, base, r, f.p, f.c0, f.c1, f.c2);
        gf_mul3(base, base, base, f.p, f.c0, f.c1, f.c2);
        k >>= 1;
    }
    return (r[0] == 1 && r[1] == 0 && r[2] == 0) ? 1 : -1;
}

__device__ inline int gf_sub(int a, int b, Field f) {
    if (f.e == 1) return ((a - b) % f.q + f.q) % f.q;
    int out = 0, place = 1;
    for (int i = 0; i < 3; i++) {
        out += (((a % f.p) - (b % f.p) + f.p) % f.p) * place;
        a /= f.p;
        b /= f.p;
        place *= f.p;
    }
    return out;
}

// P = I + [[0, 1^T], [-1, Q]] with Q_ab = chi(a - b); writes P (or P^T) as an m x m fp32 matrix.
template <typename T>
__global__ void paley_kernel(T* P, int m, Field f, int transpose) {
    for (int e = blockIdx.x * 256 + threadIdx.x; e < m * m; e += gridDim.x * 256) {
        int a = e / m, b = e % m;
        if (transpose) { int t = a; a = b; b = t; }
        int v;
        if (a == 0) v = (b == 0) ? 1 : 1;
        else if (b == 0) v = -1;
        else v = gf_chi(gf_sub(a - 1, b - 1, f), f) + (a == b ? 1 : 0);
        P[e] = (T)v;
    }
}

// ------------------------------------------------------------------------------ row transform
// IN: 0 = bf16 bits, 1 = fp32, 2 = fp64. T: arithmetic and output type (fp32 or fp64).
// Work-group b transforms the seg columns [s0, s0 + seg) of row r (r = b / (d / seg), s0 = (b % (d /
// seg)) * seg): the whole row when p2 = d, else a run of whole 2^lp2 chunks, so that the LDS tile stays
// small and many work-groups share a compute unit. Loads are issued eight vectors at a time.
template <int IN, typename T>
__global__ __launch_bounds__(256) void fwht_rows_kernel(const void* __restrict__ in, int64_t ldin, T* __restrict__ out,
                                                        int64_t ldout, int64_t d, int64_t seg, int lp2,
                                                        const int8_t* __restrict__ pre, const int8_t* __restrict__ post,
                                                        T scale, const float* __restrict__ post_scale) {
    extern __shared__ __align__(16) unsigned char xr_raw[];
    T* xr = reinterpret_cast<T*>(xr_raw);
    const int64_t nseg = d / seg;
    const int64_t r = blockIdx.x / nseg, s0 = (blockIdx.x % nseg) * seg;
    const int tid = threadIdx.x;
#pragma unroll 8
    for (int64_t c = 4 * tid; c < seg; c += 1024) {
        const int64_t gc = s0 + c;
        T v[4];
        if (IN == 0) {
            const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(in) + r * ldin + gc);
            v[0] = (T)__uint_as_float(u.x << 16);
            v[1] = (T)__uint_as_float(u.x & 0xFFFF0000u);
            v[2] = (T)__uint_as_float(u.y << 16);
            v[3] = (T)__uint_as_float(u.y & 0xFFFF0000u);
        } else if (IN == 1) {
            const float4 u = *reinterpret_cast<const float4*>(static_cast<const float*>(in) + r * ldin + gc);
            v[0] = (T)u.x; v[1] = (T)u.y; v[2] = (T)u.z; v[3] = (T)u.w;
        } else {
            const double* src = static_cast<const double*>(in) + r * ldin + gc;
            const double2 u0 = *reinterpret_cast<const double2*>(src);
            const double2 u1 = *reinterpret_cast<const double2*>(src + 2);
            v[0] = (T)u0.x; v[1] = (T)u0.y; v[2] = (T)u1.x; v[3] = (T)u1.y;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) xr[c + e] = pre ? v[e] * (T)pre[gc + e] : v[e];
    }
    __syncthreads();
    const int64_t p2 = int64_t(1) << lp2;
    int lh = 0;
    while ((int64_t(1) << lh) < p2) {
        const int64_t h = int64_t(1) << lh;
        if (2 * h < p2) {
            for (int64_t g = tid; g < seg / 4; g += 256) {
                const int64_t j = ((g >> lh) << (lh + 2)) + (g & (h - 1));
                const T a0 = xr[j], a1 = xr[j + h], a2 = xr[j + 2 * h], a3 = xr[j + 3 * h];
                const T b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
                xr[j] = b0 + b2;
                xr[j + h] = b1 + b3;
                xr[j + 2 * h] = b0 - b2;
                xr[j + 3 * h] = b1 - b3;
            }
            lh += 2;
        } else {
            for (int64_t g = tid; g < seg / 2; g += 256) {
                const int64_t j = ((g >> lh) << (lh + 1)) + (g & (h - 1));
                const T a0 = xr[j], a1 = xr[j + h];
                xr[j] = a0 + a1;
                xr[j + h] = a0 - a1;
            }
            lh += 1;
        }
        __syncthreads();
    }
    T* dst = out + r * ldout + s0;
#pragma unroll 4
    for (int64_t c = 4 * tid; c < seg; c += 1024) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            T v = post ? xr[c + e] * scale * (T)post[s0 + c + e] : xr[c + e] * scale;
            if (post_scale) v *= (T)post_scale[s0 + c + e];
            dst[c + e] = v;
        }
    }
}

// --------------------------------------------------------------------------- column digit pass
// Rows r = (hi * D + t) * S + lo, t = 0..D-1, transformed along t for 64 columns per work-group.
template <typename T, int NL>
__global__ __launch_bounds__(256) void fwht_cols_kernel(const T* __restrict__ in, int64_t ldin, T* __restrict__ out,
                                                        int64_t ldout, int64_t ncols, int lD, int64_t S,
                                                        const float* __restrict__ pre_scale,
                                                        const int8_t* __restrict__ pre_sign,
                                                        const float* __restrict__ post_scale,
                                                        const int8_t* __restrict__ post_sign, T scale) {
    extern __shared__ __align__(16) unsigned char xc_raw[];
    T* xc = reinterpret_cast<T*>(xc_raw);
    const int D = 1 << lD;
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64, lo = blockIdx.y, hi = blockIdx.z;
    const int c = tid & 63;
    const bool cin = c0 + c < ncols;
    // every load of the thread is issued before the first LDS store (D <= 4 NL rows)
    T v[NL];
#pragma unroll
    for (int q = 0; q < NL; q++) {
        const int t = (tid >> 6) + 4 * q;
        if (t < D) v[q] = cin ? in[((hi * D + t) * S + lo) * ldin + c0 + c] : T(0);
    }
#pragma unroll
    for (int q = 0; q < NL; q++) {
        const int t = (tid >> 6) + 4 * q;
        if (t < D) {
            const int64_t r = (hi * D + t) * S + lo;
            T x = v[q];
            if (pre_scale) x *= (T)pre_scale[r];
            if (pre_sign) x *= (T)pre_sign[r];
            xc[t * 64 + c] = x;
        }
    }
    __syncthreads();
    int lh = 0;
    while (lh < lD) {
        const int h = 1 << lh;
        if (lh + 1 < lD) {
            for (int g = tid >> 6; g < D / 4; g += 4) {
                const int j = ((g >> lh) << (lh + 2)) + (g & (h - 1));
                const T a0 = xc[j * 64 + c], a1 = xc[(j + h) * 64 + c], a2 = xc[(j + 2 * h) * 64 + c],
                        a3 = xc[(j + 3 * h) * 64 + c];
                const T b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
                xc[j * 64 + c] = b0 + b2;
                xc[(j + h) * 64 + c] = b1 + b3;
                xc[(j + 2 * h) * 64 + c] = b0 - b2;
                xc[(j + 3 * h) * 64 + c] = b1 - b3;
            }
            lh += 2;
        } else {
            for (int g = tid >> 6; g < D / 2; g += 4) {
                const int j = ((g >> lh) << (lh + 1)) + (g & (h - 1));
                const T a0 = xc[j * 64 + c], a1 = xc[(j + h) * 64 + c];
                xc[j * 64 + c] = a0 + a1;
                xc[(j + h) * 64 + c] = a0 - a1;
            }
            lh += 1;
        }
        __syncthreads();
    }
    if (!cin) return;
    for (int t = tid >> 6; t < D; t += 4) {
        const int64_t r = (hi * D + t) * S + lo;
        T v = xc[t * 64 + c] * scale;
        if (post_scale) v *= (T)post_scale[r];
        if (post_sign) v *= (T)post_sign[r];
        out[r * ldout + c0 + c] = v;
    }
}

// ------------------------------------------------------------------------------- host helpers
// in_kind: 0 bf16, 1 fp32, 2 fp64.
template <typename T>
static kq_status rows_transform(const void* in, int in_kind, int64_t ldin, T* out, int64_t ldout, int64_t R, int64_t d,
                                int64_t p2, const int8_t* pre, const int8_t* post, T scale, hipStream_t st,
                                const float* post_scale = nullptr) {
    if (R <= 0) return KQ_OK;
    int lp2 = 0;
    while ((int64_t(1) << lp2) < p2) lp2++;
    // columns per work-group: the whole row, or (several chunks of p2) the most whole chunks, a divisor
    // of the chunk count, within 2048 columns
    int64_t seg = d;
    if (p2 < d) {
        const int64_t m = d / p2;
        int64_t g = 1;
        for (int64_t c = 1; c <= m && c * p2 <= 2048; c++)
            if (m % c == 0 && (c * p2) % 4 == 0) g = c;
        seg = (g * p2) % 4 == 0 ? g * p2 : d;
    }
    const size_t smem = (size_t)seg * sizeof(T);
    if (smem > 160 * 1024) return fail(KQ_ESHAPE, "row transform: row of %lld elements does not fit in LDS", (long long)d);
    if (R * (d / seg) > 2147483647) return fail(KQ_ESHAPE, "row transform: too many rows");
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(&fwht_rows_kernel<0, T>), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        hipFuncSetAttribute(reinterpret_cast<const void*>(&fwht_rows_kernel<1, T>), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        hipFuncSetAttribute(reinterpret_cast<const void*>(&fwht_rows_kernel<2, T>), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr = true;
    }
    const dim3 grid((unsigned)(R * (d / seg)));
    if (in_kind == 0)
        hipLaunchKernelGGL((fwht_rows_kernel<0, T>), grid, dim3(256), smem, st, in, ldin, out, ldout, d, seg, lp2, pre, post, scale, post_scale);
    else if (in_kind == 1)
        hipLaunchKernelGGL((fwht_rows_kernel<1, T>), grid, dim3(256), smem, st, in, ldin, out, ldout, d, seg, lp2, pre, post, scale, post_scale);
    else
        hipLaunchKernelGGL((fwht_rows_kernel<2, T>), grid, dim3(256), smem, st, in, ldin, out, ldout, d, seg, lp2, pre, post, scale, post_scale);
    return check_launch("fwht_rows");
}

struct ColOps {
    const float* pre_scale = nullptr;
    const int8_t* pre_sign = nullptr;
    const float* post_scale = nullptr;
    const int8_t* post_sign = nullptr;
    double scale = 1.0;
};

// Sylvester transform along the row index within every chunk of p2 rows (R = m * p2 rows), as a
// sequence of digit passes of at most 2^8 (fp32) or 2^7 (fp64) rows each, so a pass's tile stays
// within 64 KB of LDS. The first pass reads `in`, later passes work in place on `out`.
// Pre-multipliers go to the first pass, post-multipliers and the scale to the last.
template <typename T>
static kq_status cols_transform(const T* in, int64_t ldin, T* out, int64_t ldout, int64_t R, int64_t ncols, int64_t p2,
                                const ColOps& ops, hipStream_t st) {
    const int maxbits = sizeof(T) == 8 ? 7 : 8;
    int k = 0;
    while ((int64_t(1) << k) < p2) k++;
    int npass = (k + maxbits - 1) / maxbits;
    if (npass == 0) npass = 1;
    int64_t S = 1;
    int done = 0;
    for (int ps = 0; ps < npass; ps++) {
        const int lD = (k - done) / (npass - ps);
        const int D = 1 << lD;
        const bool first = ps == 0, last = ps == npass - 1;
        const size_t smem = (size_t)D * 64 * sizeof(T);
        dim3 grid((unsigned)((ncols + 63) / 64), (unsigned)S, (unsigned)(R / ((int64_t)D * S)));
        if (S > 65535 || R / ((int64_t)D * S) > 65535) return fail(KQ_ESHAPE, "column transform grid too large");
#define KQ_FC(NL_) hipLaunchKernelGGL((fwht_cols_kernel<T, NL_>), grid, dim3(256), smem, st, first ? in : out,               \
                                   first ? ldin : ldout, out, ldout, ncols, lD, S, first ? ops.pre_scale : nullptr,     \
                                   first ? ops.pre_sign : nullptr, last ? ops.post_scale : nullptr,                     \
                                   last ? ops.post_sign : nullptr, (T)(last ? ops.scale : 1.0))
        if (D <= 16) KQ_FC(4);
        else if (D <= 64) KQ_FC(16);
        else if (D <= 128) KQ_FC(32);
        else KQ_FC(64);
#undef KQ_FC
        KQ_TRY(check_launch("fwht_cols"));
        S *= D;
        done += lD;
    }
    return KQ_OK;
}

template <typename T>
static kq_status make_paley(T* P, int64_t m, const Field& f, bool transpose, hipStream_t st) {
    const unsigned blocks = (unsigned)((m * m + 255) / 256 < 1024 ? (m * m + 255) / 256 : 1024);
    hipLaunchKernelGGL(paley_kernel<T>, dim3(blocks), dim3(256), 0, st, P, (int)m, f, transpose ? 1 : 0);
    return check_launch("paley");
}

// Paley mix of small order (m <= PM_MAX) in fp32, at HBM rate: every column vector (r, c), r < R,
// c < C, has its m entries at in + r ldr_in + b gs_in + c (b < m); out gets alpha P times it at the
// same places of out. A thread takes four adjacent vectors: m 16-byte loads, m^2 4-wide FMAs with P
// from LDS, m 16-byte stores (a GEMM with K = m < 16 runs on the general tiles at a fraction of this).
constexpr int PM_MAX = 32;
typedef float pm_f4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void paley_mix_kernel(const float* __restrict__ P, int m, const float* __restrict__ in,
                                                        int64_t ldr_in, int64_t gs_in, float* __restrict__ out,
                                                        int64_t ldr_out, int64_t gs_out, int64_t R, int64_t C,
                                                        float alpha) {
    __shared__ float Ps[PM_MAX * PM_MAX];
    for (int e = threadIdx.x; e < m * m; e += 256) Ps[e] = P[e];
    __syncthreads();
    const int64_t cq = C / 4, tot = R * cq;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < tot; v += (int64_t)gridDim.x * 256) {
        const int64_t r = v / cq, c = (v - r * cq) * 4;
        const float* src = in + r * ldr_in + c;
        pm_f4 x[PM_MAX];
#pragma unroll
        for (int b = 0; b < PM_MAX; b++)
            if (b < m) x[b] = *reinterpret_cast<const pm_f4*>(src + b * gs_in);
        float* dst = out + r * ldr_out + c;
        for (int a = 0; a < m; a++) {
            pm_f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < PM_MAX; b++)
                if (b < m) acc += Ps[a * m + b] * x[b];
            *reinterpret_cast<pm_f4*>(dst + a * gs_out) = alpha * acc;
        }
    }
}

static bool paley_mix_ok(int64_t m, int64_t C, const void* in, const void* out, int64_t ldr_in, int64_t gs_in,
                         int64_t ldr_out, int64_t gs_out) {
    return m >= 2 && m <= PM_MAX && C % 4 == 0 && aligned16(in) && aligned16(out) && ldr_in % 4 == 0 &&
           gs_in % 4 == 0 && ldr_out % 4 == 0 && gs_out % 4 == 0;
}

static kq_status paley_mix(const float* P, int64_t m, const float* in, int64_t ldr_in, int64_t gs_in, float* out,
                           int64_t ldr_out, int64_t gs_out, int64_t R, int64_t C, float alpha, hipStream_t st) {
    const int64_t tot = R * (C / 4);
    if (tot <= 0) return KQ_OK;
    const int64_t wg = (tot + 255) / 256;
    hipLaunchKernelGGL(paley_mix_kernel, dim3((unsigned)(wg < 65536 ? wg : 65536)), dim3(256), 0, st, P, (int)m, in,
                       ldr_in, gs_in, out, ldr_out, gs_out, R, C, alpha);
    return check_launch("paley_mix");
}

// out_r = alpha * P in_r for every row r, each row seen as an m x p2 matrix (row mix of chunks).
template <typename T>
static kq_status paley_rows(const T* P, const T* in, int64_t ldin, T* out, int64_t ldout, int64_t R, int64_t m,
                            int64_t p2, T alpha, hipStream_t st) {
    if constexpr (sizeof(T) == 4)
        if (paley_mix_ok(m, p2, in, out, ldin, p2, ldout, p2))
            return paley_mix(P, m, in, ldin, p2, out, ldout, p2, R, p2, alpha, st);
    for (int64_t r0 = 0; r0 < R; r0 += 65535) {
        const int64_t cnt = (R - r0) < 65535 ? (R - r0) : 65535;
        GemmArgs<T> g = gemm_args<T>(m, p2, m, P, m, in + r0 * ldin, p2, out + r0 * ldout, p2, alpha, T(0));
        g.nb1 = cnt; g.sA1 = 0; g.sB1 = ldin; g.sC1 = ldout;
        KQ_TRY(gemm<T>(g, false, false, st));
    }
    return KQ_OK;
}

// out = alpha * (P (x) I_{p2}) in along the row index (rows grouped in m chunks of p2 rows).
template <typename T>
static kq_status paley_cols(const T* P, const T* in, int64_t ldin, T* out, int64_t ldout, int64_t m, int64_t p2,
                            int64_t ncols, T alpha, hipStream_t st) {
    if constexpr (sizeof(T) == 4)
        if (paley_mix_ok(m, ncols, in, out, ldin, p2 * ldin, ldout, p2 * ldout))
            return paley_mix(P, m, in, ldin, p2 * ldin, out, ldout, p2 * ldout, p2, ncols, alpha, st);
    if (ldin == ncols && ldout == ncols) {
        GemmArgs<T> g = gemm_args<T>(m, p2 * ncols, m, P, m, in, p2 * ncols, out, p2 * ncols, alpha, T(0));
        return gemm<T>(g, false, false, st);
    }
    GemmArgs<T> g = gemm_args<T>(m, ncols, m, P, m, in, p2 * ldin, out, p2 * ldout, alpha, T(0));
    g.nb1 = p2; g.sA1 = 0; g.sB1 = ldin; g.sC1 = ldout;
    return gemm<T>(g, false, false, st);
}

}  // namespace kq

using namespace kq;

extern "C" int64_t kq_hadamard_order(int64_t d, int64_t* pow2) {
    int64_t m, p2;
    Field f;
    if (!hadamard_split(d, m, p2, f)) return 0;
    if (pow2) *pow2 = p2;
    return m;
}

size_t rotate_in_ws(int64_t o, int64_t i) {
    int64_t m, p2;
    Field f;
    if (!hadamard_split(i, m, p2, f)) return 0;
    Sizer z;
    z.take<float>((size_t)m * m);
    z.take<double>((size_t)m * m);
    if (m > 1) z.take<double>((size_t)(o > i ? o : i) * i);
    return z.used;
}

extern "C" kq_status kq_rotate_in(const void* Win, kq_dtype wdt, int64_t ldwin, float* Wout, int64_t ldw, int64_t o,
                                  int64_t i, double* HX, const int8_t* sign_in, void* ws, size_t ws_bytes,
                                  kq_stream stream) {
    if (!sign_in || (o > 0 && (!Win || !Wout))) return fail(KQ_EINVAL, "kq_rotate_in: null pointer");
    if (o < 0 || i <= 0 || (o > 0 && (ldwin < i || ldw < i))) return fail(KQ_ESHAPE, "kq_rotate_in: bad sizes");
    if (wdt != KQ_F32 && wdt != KQ_BF16) return fail(KQ_EINVAL, "kq_rotate_in: bad dtype");
    if (i % 4 || ldwin % 4 || ldw % 4 || (Win && !aligned16(Win)) || (Wout && !aligned16(Wout)) || (HX && !aligned16(HX)))
        return fail(KQ_EINVAL, "kq_rotate_in: i, leading dimensions and pointers must be 16-byte multiples");
    int64_t m, p2;
    Field f;
    if (!hadamard_split(i, m, p2, f)) return fail(KQ_EUNSUPPORTED, "kq_rotate_in: no Hadamard order for i=%lld", (long long)i);
    if (ws_bytes < rotate_in_ws(o, i) || (m > 1 && !ws)) return fail(KQ_EWORKSPACE, "kq_rotate_in: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    float* P = ar.take<float>((size_t)m * m);
    double* Pd = ar.take<double>((size_t)m * m);
    double* T = m > 1 ? ar.take<double>((size_t)(o > i ? o : i) * i) : nullptr;
    const double inv = 1.0 / std::sqrt((double)i);
    // W' = W U: rows w -> H (s * w) / sqrt(i)   (fp32)
    if (o > 0) {
        if (m == 1) {
            KQ_TRY(rows_transform<float>(Win, wdt == KQ_BF16 ? 0 : 1, ldwin, Wout, ldw, o, i, p2, sign_in, nullptr,
                                         (float)inv, st));
        } else {
            float* Tf = reinterpret_cast<float*>(T);
            KQ_TRY(make_paley<float>(P, m, f, false, st));
            KQ_TRY(rows_transform<float>(Win, wdt == KQ_BF16 ? 0 : 1, ldwin, Tf, i, o, i, p2, sign_in, nullptr, 1.0f, st));
            KQ_TRY(paley_rows<float>(P, Tf, i, Wout, ldw, o, m, p2, (float)inv, st));
        }
    }
    // H_X' = U^T H_X U: rows, then columns   (fp64)
    if (HX) {
        if (m == 1) {
            KQ_TRY(rows_transform<double>(HX, 2, i, HX, i, i, i, p2, sign_in, nullptr, inv, st));
            ColOps ops;
            ops.pre_sign = sign_in;
            ops.scale = inv;
            KQ_TRY(cols_transform<double>(HX, i, HX, i, i, i, p2, ops, st));
        } else {
            KQ_TRY(make_paley<double>(Pd, m, f, false, st));
            KQ_TRY(rows_transform<double>(HX, 2, i, HX, i, i, i, p2, sign_in, nullptr, 1.0, st));
            KQ_TRY(paley_rows<double>(Pd, HX, i, T, i, i, m, p2, inv, st));
            ColOps ops;
            ops.pre_sign = sign_in;
            KQ_TRY(cols_transform<double>(T, i, T, i, i, i, p2, ops, st));
            KQ_TRY(paley_cols<double>(Pd, T, i, HX, i, m, p2, i, inv, st));
        }
    }
    return KQ_OK;
}

size_t rotate_out_ws(int64_t o, int64_t i, kq_hg_form form) {
    int64_t m, p2;
    Field f;
    if (!hadamard_split(o, m, p2, f)) return 0;
    Sizer z;
    z.take<float>((size_t)m * m);
    if (m > 1 || form != KQ_HG_DIAG) z.take<float>((size_t)o * i);
    return z.used;
}

extern "C" kq_status kq_rotate_out(float* W, int64_t o, int64_t i, int64_t ldw, const float* S, kq_hg_form form,
                                   int64_t blk, const int8_t* sign_out, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!W || !S || !sign_out) return fail(KQ_EINVAL, "kq_rotate_out: null pointer");
    if (o <= 0 || i <= 0 || ldw < i) return fail(KQ_ESHAPE, "kq_rotate_out: bad sizes");
    if (i % 4 || ldw % 4 || !aligned16(W) || !aligned16(S)) return fail(KQ_EINVAL, "kq_rotate_out: alignment");
    if (form != KQ_HG_DIAG && form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "kq_rotate_out: bad form");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk || blk % 4)) return fail(KQ_ESHAPE, "kq_rotate_out: bad block size");
    int64_t m, p2;
    Field f;
    if (!hadamard_split(o, m, p2, f)) return fail(KQ_EUNSUPPORTED, "kq_rotate_out: no Hadamard order for o=%lld", (long long)o);
    if (ws_bytes < rotate_out_ws(o, i, form) || (rotate_out_ws(o, i, form) && !ws))
        return fail(KQ_EWORKSPACE, "kq_rotate_out: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    float* P = ar.take<float>((size_t)m * m);
    float* T = (m > 1 || form != KQ_HG_DIAG) ? ar.take<float>((size_t)o * i) : nullptr;
    const float inv = (float)(1.0 / std::sqrt((double)o));
    if (m > 1) KQ_TRY(make_paley<float>(P, m, f, false, st));
    ColOps ops;
    const float* src = W;
    int64_t ldsrc = ldw;
    if (form == KQ_HG_DIAG) {
        ops.pre_scale = S;
        ops.pre_sign = sign_out;
    } else {
        // T = D_t S W
        if (form == KQ_HG_FULL) {
            GemmArgs<float> g = gemm_args<float>(o, i, o, S, o, W, ldw, T, i, 1.0f, 0.0f);
            g.rsign = sign_out;
            KQ_TRY(gemm<float>(g, false, false, st));
        } else {
            GemmArgs<float> g = gemm_args<float>(blk, i, blk, S, blk, W, ldw, T, i, 1.0f, 0.0f);
            g.nb1 = o / blk; g.sA1 = blk * blk; g.sB1 = blk * ldw; g.sC1 = blk * i;
            g.rsign = sign_out; g.sR1 = blk;
            KQ_TRY(gemm<float>(g, false, false, st));
        }
        src = T;
        ldsrc = i;
    }
    if (m == 1) {
        ops.scale = inv;
        return cols_transform<float>(src, ldsrc, W, ldw, o, i, p2, ops, st);
    }
    // FWHT of the chunks into T (in place when T already holds D_t S W), then the Paley mix into W
    KQ_TRY(cols_transform<float>(src, ldsrc, T, i, o, i, p2, ops, st));
    return paley_cols<float>(P, T, i, W, ldw, m, p2, i, inv, st);
}

size_t unrotate_ws(int64_t o, int64_t i, kq_hg_form form) {
    int64_t mo, po, mi, pi;
    Field f;
    if (!hadamard_split(o, mo, po, f) || !hadamard_split(i, mi, pi, f)) return 0;
    Sizer z;
    z.take<float>((size_t)mo * mo);
    z.take<float>((size_t)mi * mi);
    z.take<float>((size_t)o * i);
    z.take<float>((size_t)o * i);
    (void)form;
    return z.used;
}

extern "C" kq_status kq_unrotate(const float* Q, int64_t o, int64_t i, int64_t ldq, const int8_t* sign_in,
                                 const int8_t* sign_out, const float* Sinv, kq_hg_form form, int64_t blk, float* What,
                                 int64_t ldw, void* ws, size_t ws_bytes, kq_stream stream) {
    if (!Q || !sign_in || !sign_out || !Sinv || !What) return fail(KQ_EINVAL, "kq_unrotate: null pointer");
    if (o <= 0 || i <= 0 || ldq < i || ldw < i) return fail(KQ_ESHAPE, "kq_unrotate: bad sizes");
    if (i % 4 || ldq % 4 || ldw % 4 || !aligned16(Q) || !aligned16(What)) return fail(KQ_EINVAL, "kq_unrotate: alignment");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "kq_unrotate: bad block size");
    int64_t mo, po, mi, pi;
    Field fo, fi;
    if (!hadamard_split(o, mo, po, fo) || !hadamard_split(i, mi, pi, fi))
        return fail(KQ_EUNSUPPORTED, "kq_unrotate: no Hadamard order");
    if (!ws || ws_bytes < unrotate_ws(o, i, form)) return fail(KQ_EWORKSPACE, "kq_unrotate: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    float* Po = ar.take<float>((size_t)mo * mo);
    float* Pi = ar.take<float>((size_t)mi * mi);
    float* T1 = ar.take<float>((size_t)o * i);
    float* T2 = ar.take<float>((size_t)o * i);
    // A = D_t H_o^T Q / sqrt(o) ; H_o^T = P_o^T (x) H
    ColOps ops;
    ops.post_sign = sign_out;
    ops.scale = 1.0 / std::sqrt((double)o);
    if (form == KQ_HG_DIAG) ops.post_scale = Sinv;
    if (mo > 1) {
        KQ_TRY(make_paley<float>(Po, mo, fo, true, st));
        KQ_TRY(paley_cols<float>(Po, Q, ldq, T1, i, mo, po, i, 1.0f, st));
        KQ_TRY(cols_transform<float>(T1, i, T1, i, o, i, po, ops, st));
    } else {
        KQ_TRY(cols_transform<float>(Q, ldq, T1, i, o, i, po, ops, st));
    }
    float* cur = T1;
    if (form != KQ_HG_DIAG) {
        if (form == KQ_HG_FULL) {
            GemmArgs<float> g = gemm_args<float>(o, i, o, Sinv, o, T1, i, T2, i, 1.0f, 0.0f);
            KQ_TRY(gemm<float>(g, false, false, st));
        } else {
            GemmArgs<float> g = gemm_args<float>(blk, i, blk, Sinv, blk, T1, i, T2, i, 1.0f, 0.0f);
            g.nb1 = o / blk; g.sA1 = blk * blk; g.sB1 = blk * i; g.sC1 = blk * i;
            KQ_TRY(gemm<float>(g, false, false, st));
        }
        cur = T2;
    }
    // rows a -> s * (H_i^T a) / sqrt(i)
    const float inv_i = (float)(1.0 / std::sqrt((double)i));
    if (mi > 1) {
        float* other = (cur == T1) ? T2 : T1;
        KQ_TRY(make_paley<float>(Pi, mi, fi, true, st));
        KQ_TRY(paley_rows<float>(Pi, cur, i, other, i, o, mi, pi, 1.0f, st));
        cur = other;
    }
    return rows_transform<float>(cur, 1, i, What, ldw, o, i, pi, nullptr, sign_in, inv_i, st);
}

// ------------------------------------------------------------------------- few long vectors
// out_r = post_scale * post * scale * ((P (x) H_p2) (pre * in_r)) for a handful of rows r of length
// d = m p2, spread over many workgroups (one row per workgroup would leave the chip idle). The
// Sylvester part factors along the index c = hi * VT_BL + lo as H_{p2/VT_BL} (x) H_{VT_BL}: the
// block pass transforms lo inside LDS, the stride pass transforms hi in registers, and the Paley
// pass mixes the m chunks of p2 (each output element is one row of P against a column of chunks).
namespace kq {

constexpr int VT_BL = 512;      // block of the first pass (two elements per thread)
constexpr int VT_MAXL = 64;     // longest stride pass: p2 <= VT_BL * VT_MAXL

struct VecOps {
    const int8_t* pre = nullptr;
    const int8_t* post = nullptr;
    const float* post_scale = nullptr;
    float scale = 1.0f;
};

__device__ __forceinline__ float vt_post(float v, int64_t idx, const VecOps& op) {
    v *= op.scale;
    if (op.post) v *= (float)op.post[idx];
    if (op.post_scale) v *= op.post_scale[idx];
    return v;
}

// Sylvester transform of `bl` consecutive elements (bl = min(p2, VT_BL), a power of two)
__global__ __launch_bounds__(256) void vt_block_kernel(const float* __restrict__ in, int64_t ldin, float* __restrict__ out,
                                                       int64_t ldout, int bl, int lbl, VecOps op, int last) {
    __shared__ float sh[VT_BL];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.y, base = (int64_t)blockIdx.x * bl;
    const float* src = in + r * ldin + base;
    for (int e = tid; e < bl; e += 256) sh[e] = op.pre ? src[e] * (float)op.pre[base + e] : src[e];
    __syncthreads();
    for (int l = 0; l < lbl; l++) {
        const int h = 1 << l;
        for (int g = tid; g < bl / 2; g += 256) {
            const int j = ((g >> l) << (l + 1)) + (g & (h - 1));
            const float a = sh[j], b = sh[j + h];
            sh[j] = a + b;
            sh[j + h] = a - b;
        }
        __syncthreads();
    }
    float* dst = out + r * ldout + base;
    for (int e = tid; e < bl; e += 256) dst[e] = last ? vt_post(sh[e], base + e, op) : sh[e];
}

// Sylvester transform along hi (length L = p2 / VT_BL) for every (chunk, lo) column, in registers
template <int L>
__global__ __launch_bounds__(256) void vt_stride_kernel(const float* __restrict__ in, int64_t ldin, float* __restrict__ out,
                                                        int64_t ldout, int64_t d, int64_t p2, VecOps op, int last) {
    const int64_t r = blockIdx.y;
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;    // chunk * VT_BL + lo
    if (col >= d / L) return;
    const int64_t chunk = col / VT_BL, lo = col % VT_BL;
    const int64_t b0 = chunk * p2 + lo;
    float v[L];
#pragma unroll
    for (int k = 0; k < L; k++) v[k] = in[r * ldin + b0 + (int64_t)k * VT_BL];
#pragma unroll
    for (int h = 1; h < L; h <<= 1)
#pragma unroll
        for (int k = 0; k < L; k++)
            if ((k & h) == 0) {
                const float a = v[k], b = v[k + h];
                v[k] = a + b;
                v[k + h] = a - b;
            }
#pragma unroll
    for (int k = 0; k < L; k++) {
        const int64_t idx = b0 + (int64_t)k * VT_BL;
        out[r * ldout + idx] = last ? vt_post(v[k], idx, op) : v[k];
    }
}

// out[j p2 + c] = post(sum_a P[j][a] in[a p2 + c])
__global__ __launch_bounds__(256) void vt_paley_kernel(const float* __restrict__ P, int m, const float* __restrict__ in,
                                                       int64_t ldin, float* __restrict__ out, int64_t ldout, int64_t p2,
                                                       VecOps op) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int j = blockIdx.y;
    const int64_t r = blockIdx.z;
    if (c >= p2) return;
    const float* src = in + r * ldin + c;
    const float* prow = P + (int64_t)j * m;
    // four independent partial sums (a mod 4) keep several loads in flight
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int a = 0;
    for (; a + 4 <= m; a += 4) {
#pragma unroll
        for (int q = 0; q < 4; q++) acc[q] = fmaf(prow[a + q], src[(int64_t)(a + q) * p2], acc[q]);
    }
    for (; a < m; a++) acc[a & 3] = fmaf(prow[a], src[(int64_t)a * p2], acc[a & 3]);
    const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const int64_t idx = (int64_t)j * p2 + c;
    out[r * ldout + idx] = vt_post(sum, idx, op);
}

// R rows (R <= 65535) of length d = m p2 (p2 a power of two, p2 <= VT_BL * VT_MAXL); tmp: R x d
// scratch (leading dimension d), may not alias in or out; out may alias in.
static kq_status vec_transform(const float* in, int64_t ldin, float* out, int64_t ldout, int64_t R, int64_t m, int64_t p2,
                               const float* P, const VecOps& op, float* tmp, hipStream_t st) {
    const int64_t d = m * p2;
    if (R <= 0) return KQ_OK;
    if (R > 65535 || p2 > (int64_t)VT_BL * VT_MAXL || m > 65535) return fail(KQ_ESHAPE, "vector transform: too large");
    const int bl = (int)(p2 < VT_BL ? p2 : VT_BL);
    int lbl = 0;
    while ((1 << lbl) < bl) lbl++;
    const int64_t L = p2 / bl;
    // pass results go to tmp or out so that the last pass writes out
    const int passes = 1 + (L > 1) + (m > 1);
    VecOps first = op, mid;
    first.post = nullptr; first.post_scale = nullptr; first.scale = 1.0f;
    mid.scale = 1.0f;
    int done = 0;
    auto dst_of = [&](int k) { return (passes - k) % 2 == 1 ? out : tmp; };   // the last pass writes out
    auto ld_of = [&](float* p) { return p == out ? ldout : d; };
    const float* cur = in;
    int64_t ldc = ldin;
    {
        float* dst = dst_of(done);
        const bool last = ++done == passes;
        VecOps o1 = first;
        if (last) { o1.post = op.post; o1.post_scale = op.post_scale; o1.scale = op.scale; }
        hipLaunchKernelGGL(vt_block_kernel, dim3((unsigned)(d / bl), (unsigned)R), dim3(256), 0, st, cur, ldc, dst,
                           ld_of(dst), bl, lbl, o1, last ? 1 : 0);
        KQ_TRY(check_launch("vt_block"));
        cur = dst; ldc = ld_of(dst);
    }
    if (L > 1) {
        float* dst = dst_of(done);
        const bool last = ++done == passes;
        const VecOps o2 = last ? op : mid;
        const dim3 grid((unsigned)((d / L + 255) / 256), (unsigned)R);
        switch (L) {
#define KQ_VT_STRIDE(n) case n: hipLaunchKernelGGL((vt_stride_kernel<n>), grid, dim3(256), 0, st, cur, ldc, dst, ld_of(dst), d, p2, o2, last ? 1 : 0); break;
            KQ_VT_STRIDE(2) KQ_VT_STRIDE(4) KQ_VT_STRIDE(8) KQ_VT_STRIDE(16) KQ_VT_STRIDE(32) KQ_VT_STRIDE(64)
#undef KQ_VT_STRIDE
            default: return fail(KQ_ESHAPE, "vector transform: bad stride length");
        }
        KQ_TRY(check_launch("vt_stride"));
        cur = dst; ldc = ld_of(dst);
    }
    if (m > 1) {
        float* dst = dst_of(done);
        ++done;
        const dim3 grid((unsigned)((p2 + 255) / 256), (unsigned)m, (unsigned)R);
        hipLaunchKernelGGL(vt_paley_kernel, grid, dim3(256), 0, st, P, (int)m, cur, ldc, dst, ld_of(dst), p2, op);
        KQ_TRY(check_launch("vt_paley"));
    }
    return KQ_OK;
}

}  // namespace kq

// ------------------------------------------------------------------------- inference-side matvec
namespace kq {
kq_status dequant_gemv(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i, int bits,
                       int group, const float* X, int64_t ldx, int64_t nt, float* Zt, int64_t ldz, float* Zp,
                       hipStream_t st);
size_t dequant_ws(int64_t o, int64_t i, int64_t nt);
kq_status sinv_gemv(const float* A, int64_t o, int64_t blk, const float* Zt, int64_t ldz, int64_t nt, float* Y,
                    int64_t ldy, hipStream_t st);
}  // namespace kq

size_t matvec_ws(int64_t o, int64_t i, int64_t nt, kq_hg_form form) {
    int64_t mo, po, mi, pi;
    Field fo, fi;
    if (!hadamard_split(o, mo, po, fo) || !hadamard_split(i, mi, pi, fi) || nt <= 0) return 0;
    Sizer z;
    z.take<float>((size_t)mo * mo);
    z.take<float>((size_t)mi * mi);
    z.take<float>((size_t)nt * i);   // X'
    z.take<float>((size_t)nt * i);   // Paley scratch
    z.take<float>((size_t)nt * o);   // Z^T
    z.take<float>((size_t)nt * o);   // Paley scratch
    z.take<float>((size_t)nt * o);   // V^T z
    z.take<char>(dequant_ws(o, i, nt));
    (void)form;
    return z.used;
}

// Host checks of kq_matvec_quantized's arguments (shared with its scratch-array variant); `who` names
// the entry point in the error text.
static kq_status matvec_validate(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i,
                                 int bits, int group, const int8_t* sign_in, const int8_t* sign_out, const float* Sinv,
                                 kq_hg_form form, int64_t blk, const float* X, int64_t ldx, int64_t nt, const float* Y,
                                 int64_t ldy, const char* who) {
    if (!codes || !scale || !offset || !sign_in || !sign_out || !Sinv || !X || !Y)
        return fail(KQ_EINVAL, "%s: null pointer", who);
    if (o <= 0 || i <= 0 || nt <= 0 || nt > 65535 || ldx < i || ldy < o)
        return fail(KQ_ESHAPE, "%s: bad sizes", who);
    if (bits < 2 || bits > 8) return fail(KQ_EUNSUPPORTED, "%s: bits", who);
    if (group != 0 && (group % 32 || i % group)) return fail(KQ_EUNSUPPORTED, "%s: group", who);
    if (i % 32 || (i * bits) % 32) return fail(KQ_ESHAPE, "%s: i must be a multiple of 32", who);
    if (ldx % 4 || !aligned16(X)) return fail(KQ_EINVAL, "%s: X alignment", who);
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "%s: bad block size", who);
    if (form != KQ_HG_DIAG && form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "%s: form", who);
    int64_t mo, po, mi, pi;
    Field fo, fi;
    if (!hadamard_split(o, mo, po, fo) || !hadamard_split(i, mi, pi, fi))
        return fail(KQ_EUNSUPPORTED, "%s: no Hadamard order", who);
    if (o % 4) return fail(KQ_ESHAPE, "%s: o must be a multiple of 4", who);
    return KQ_OK;
}

// The product itself, on a workspace of at least matvec_ws(o, i, nt, form) bytes. Every scratch slice
// it uses is written before it is read, so nothing in the workspace has to start at zero.
static kq_status matvec_run(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i,
                            int bits, int group, const int8_t* sign_in, const int8_t* sign_out, const float* Sinv,
                            kq_hg_form form, int64_t blk, const float* X, int64_t ldx, int64_t nt, float* Y,
                            int64_t ldy, void* ws, size_t ws_bytes, hipStream_t st) {
    int64_t mo, po, mi, pi;
    Field fo, fi;
    hadamard_split(o, mo, po, fo);
    hadamard_split(i, mi, pi, fi);
    Arena ar(ws, ws_bytes);
    float* Po = ar.take<float>((size_t)mo * mo);
    float* Pi = ar.take<float>((size_t)mi * mi);
    float* Xr = ar.take<float>((size_t)nt * i);
    float* Xt = ar.take<float>((size_t)nt * i);
    float* Zt = ar.take<float>((size_t)nt * o);
    float* T1 = ar.take<float>((size_t)nt * o);
    float* T2 = ar.take<float>((size_t)nt * o);
    const size_t zp_bytes = dequant_ws(o, i, nt);
    float* Zp = zp_bytes ? reinterpret_cast<float*>(ar.take<char>(zp_bytes)) : nullptr;
    // x' = U^T x: every token row x -> H_i (s * x) / sqrt(i)
    VecOps xin;
    xin.pre = sign_in;
    xin.scale = (float)(1.0 / std::sqrt((double)i));
    if (mi > 1) KQ_TRY(make_paley<float>(Pi, mi, fi, false, st));
    KQ_TRY(vec_transform(X, ldx, Xr, i, nt, mi, pi, Pi, xin, Xt, st));
    // z^T = x'^T Q''^T from the packed codes, one row of length o per token
    KQ_TRY(dequant_gemv(codes, scale, offset, o, i, bits, group, Xr, i, nt, Zt, o, Zp, st));
    // V^T z = t * (H_o^T z) / sqrt(o) along each token row, H_o^T = P_o^T (x) H; a diagonal S^{-1}
    // is folded into the same pass and written straight to Y
    VecOps vout;
    vout.post = sign_out;
    vout.scale = (float)(1.0 / std::sqrt((double)o));
    if (form == KQ_HG_DIAG) vout.post_scale = Sinv;
    if (mo > 1) KQ_TRY(make_paley<float>(Po, mo, fo, true, st));
    if (form == KQ_HG_DIAG) return vec_transform(Zt, o, Y, ldy, nt, mo, po, Po, vout, T1, st);
    KQ_TRY(vec_transform(Zt, o, T2, o, nt, mo, po, Po, vout, T1, st));
    const int64_t b = form == KQ_HG_FULL ? o : blk;
    if (sinv_gemv(Sinv, o, b, T2, o, nt, Y, ldy, st) == KQ_OK) return KQ_OK;   // up to 8 tokens
    // y_t = S^{-1} v_t for every token: Y = V S^{-T} (blockwise for the block form)
    GemmArgs<float> g = gemm_args<float>(nt, b, b, T2, o, Sinv, b, Y, ldy, 1.0f, 0.0f);
    if (form == KQ_HG_BLOCK) {
        g.nb1 = o / blk; g.sA1 = blk; g.sB1 = blk * blk; g.sC1 = blk;
    }
    return gemm<float>(g, false, true, st);
}

extern "C" kq_status kq_matvec_quantized(const uint32_t* codes, const float* scale, const float* offset, int64_t o,
                                         int64_t i, int bits, int group, const int8_t* sign_in, const int8_t* sign_out,
                                         const float* Sinv, kq_hg_form form, int64_t blk, const float* X, int64_t ldx,
                                         int64_t nt, float* Y, int64_t ldy, void* ws, size_t ws_bytes,
                                         kq_stream stream) {
    KQ_TRY(matvec_validate(codes, scale, offset, o, i, bits, group, sign_in, sign_out, Sinv, form, blk, X, ldx, nt, Y,
                           ldy, "kq_matvec_quantized"));
    if (!ws || ws_bytes < matvec_ws(o, i, nt, form)) return fail(KQ_EWORKSPACE, "kq_matvec_quantized: workspace too small");
    return matvec_run(codes, scale, offset, o, i, bits, group, sign_in, sign_out, Sinv, form, blk, X, ldx, nt, Y, ldy, ws,
                      ws_bytes, hs(stream));
}

// ------------------------------------------------------------------ the product without a workspace
// Scratch of kq_matvec_quantized_static: one array per device, part of the library's code object, held
// by every device the library runs on until the process ends. Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol): its device address is fetched once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr, and that address is what the kernels get.
static __device__ __align__(256) unsigned char scratch[KQ_MATVEC_STATIC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static kq_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(KQ_EHIP, "kq_matvec_quantized_static: no current device");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KQ_EHIP, "kq_matvec_quantized_static: scratch address: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KQ_OK;
}

extern "C" kq_status kq_matvec_quantized_static(const uint32_t* codes, const float* scale, const float* offset,
                                                int64_t o, int64_t i, int bits, int group, const int8_t* sign_in,
                                                const int8_t* sign_out, const float* Sinv, kq_hg_form form,
                                                int64_t blk, const float* X, int64_t ldx, int64_t nt, float* Y,
                                                int64_t ldy, kq_stream stream) {
    KQ_TRY(matvec_validate(codes, scale, offset, o, i, bits, group, sign_in, sign_out, Sinv, form, blk, X, ldx, nt, Y,
                           ldy, "kq_matvec_quantized_static"));
    const size_t need = matvec_ws(o, i, nt, form);
    if (need > (size_t)KQ_MATVEC_STATIC_SCRATCH_BYTES)
        return fail(KQ_EWORKSPACE,
                    "kq_matvec_quantized_static: o = %lld, i = %lld, %lld tokens need %zu scratch bytes, more than the "
                    "library's fixed %zu; use kq_matvec_quantized with a workspace, or fewer tokens per call",
                    (long long)o, (long long)i, (long long)nt, need, (size_t)KQ_MATVEC_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    KQ_TRY(scratch_address(&ws));
    return matvec_run(codes, scale, offset, o, i, bits, group, sign_in, sign_out, Sinv, form, blk, X, ldx, nt, Y, ldy, ws,
                      (size_t)KQ_MATVEC_STATIC_SCRATCH_BYTES, hs(stream));
}
