// Packed-code dequantizing matrix-vector product for the inference-side reversion y = W^ x with
// W^ = S^{-1} V^T Q'' U^T (KronQ review page, Limitations (3): at inference the orthogonal
// transforms are reverted online at Theta(d log d) per layer, with a fused kernel keeping the cost
// close to that of the weight matvec). This file holds the middle step Z = Q'' X'^T on the packed
// codes; the transforms are in hadamard.hip.
//
// Q''[r][c] = mu[r][g] + s[r][g] q[r][c] with g = c / group (one group per row when group = 0) and
// q the b-bit codes in the LSB-first bit stream of uint32 words, each row starting on a word
// boundary. 32 consecutive codes are exactly b words, so one lane owns one such chunk with no word
// shared between lanes. A chunk never straddles a group (group is a multiple of 32), so
//     z[r][t] = sum_chunks ( s[r][g] sum_{c in chunk} q[r][c] x'[t][c] + mu[r][g] sum_{c in chunk} x'[t][c] ).
//
// Work split: a workgroup of 8 wavefronts takes 32 rows (4 per wavefront) and one slice of KC
// columns; the slice of x' (NT tokens) is staged once in LDS in a chunk-blocked layout, together
// with its 32-column sums. Each lane decodes its chunk for its wavefront's 4 rows and reuses every
// x' value it reads for all 4. The codes dominate the HBM traffic (b/8 bytes per weight), so the
// kernel is HBM-bound while decode work per code stays at ~1.5 VALU operations: for b dividing 8
// the fields of one byte position are isolated with one shift and mask per word and converted by
// the byte-select conversions; for the other widths a field is a bit-field extract (a funnel shift
// when it straddles two words). Partial sums over slices go to a workspace and are added by a
// second small kernel, in a fixed order.
#include "kq_internal.h"

namespace kq {

constexpr int DQ_R = 4;                 // rows per wavefront
constexpr int DQ_WAVES = 8;             // wavefronts per workgroup of the dequantizing product
constexpr int DQ_THREADS = 64 * DQ_WAVES;
constexpr int DQ_ROWS_WG = DQ_WAVES * DQ_R;
constexpr int SG_ROWS_WG = 4 * DQ_R;    // rows per workgroup of the S^{-1} product (4 wavefronts)
constexpr int DQ_LDS_FLOATS = 16384;    // x' slice capacity (64 KiB): NT * KC <= this

template <int B>
struct CodeMask {
    // the b-bit mask repeated in every byte (only meaningful when b divides 8)
    static constexpr uint32_t rep = B == 8 ? 0xFFFFFFFFu : (((1u << B) - 1u) * 0x01010101u);
};

// field j (0..31) of a chunk held in B words; j is a compile-time constant after unrolling
template <int B>
__device__ __forceinline__ float code_at(const uint32_t (&w)[B], int j) {
    const int bit = j * B, wi = bit >> 5, sh = bit & 31;
    if constexpr (8 % B == 0) {
        uint32_t m = (w[wi] >> (sh & 7)) & CodeMask<B>::rep;
        // keep m opaque so the conversion below stays a byte-select conversion of the masked word
        // (one VALU operation per code) instead of being folded into a bit-field extract plus a
        // conversion
        asm("" : "+v"(m));
        return (float)((m >> (sh & 24)) & 0xFFu);
    } else {
        uint32_t v;
        if (sh + B > 32) v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
        else v = w[wi] >> sh;
        return (float)(v & ((1u << B) - 1u));
    }
}

// sum over the 8 lanes of an aligned group (quad swaps, then the half-row mirror); every lane of
// the group ends with the same value
__device__ __forceinline__ float sum8(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // 7 - lane
    return v;
}

template <int B, int NT>
__global__ __launch_bounds__(DQ_THREADS) void dequant_gemv_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ scale,
                                                           const float* __restrict__ offset, int64_t o, int64_t i,
                                                           int G, int64_t KC, const float* __restrict__ X, int64_t ldx,
                                                           int nt, float* __restrict__ Z, int64_t zsr, int64_t zst,
                                                           int64_t zslice) {
    extern __shared__ __align__(16) float dq_sm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * KC;      // slices of one row group are dispatched together
    const int kc = (int)((i - col0) < KC ? (i - col0) : KC);   // multiple of 32
    const int nch = kc >> 5;
    float* xs = dq_sm;                          // [NT][kc] chunk-blocked
    float* ps = dq_sm + (size_t)NT * KC;        // [NT][nch] 32-column sums

    const int64_t ng = i / G;
    const int64_t wpr = i * B / 32;
    const int64_t r0 = ((int64_t)blockIdx.y * DQ_WAVES + wave) * DQ_R;
    const uint32_t* crow[DQ_R];
    int64_t prow[DQ_R];
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++) {
        int64_t r = r0 + rr < o ? r0 + rr : o - 1;     // clamp loads; stores are masked
        r = r < 0 ? 0 : r;
        crow[rr] = codes + r * wpr + (col0 >> 5) * B;
        prow[rr] = r * ng;
    }
    // the first chunk's codes are requested before the x' slice is staged
    uint32_t wn[DQ_R][B];
    if (lane < nch) {
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
            for (int k = 0; k < B; k++) wn[rr][k] = __builtin_nontemporal_load(crow[rr] + lane * B + k);
    }

    // stage x' (zero rows past nt) as float4s over the flattened (token, column) range with 8 loads
    // in flight per thread, and the 32-column sums (8 consecutive threads hold one chunk of one
    // token: nc4 is a multiple of 8)
    const int nc4 = kc >> 2, tot4 = NT * nc4;
    for (int b0 = 0; b0 < tot4; b0 += 8 * DQ_THREADS) {
        float4 v[8];
        int tt[8], cc[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = b0 + u * DQ_THREADS + tid;
            tt[u] = e / nc4;
            cc[u] = e - tt[u] * nc4;
            v[u] = (e < tot4 && tt[u] < nt) ? *reinterpret_cast<const float4*>(X + (int64_t)tt[u] * ldx + col0 + 4 * cc[u])
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = b0 + u * DQ_THREADS + tid;
            const float cs = sum8((v[u].x + v[u].y) + (v[u].z + v[u].w));
            if (e < tot4) {
                const int c4 = cc[u], t = tt[u];
                const int ch = c4 >> 3, jb = (c4 & 7) >> 1, jj = (c4 & 1) * 4;
                *reinterpret_cast<float4*>(xs + t * kc + jb * (nch * 8) + ch * 8 + jj) = v[u];
                if ((c4 & 7) == 0) ps[t * nch + ch] = cs;
            }
        }
    }
    __syncthreads();
    if (r0 >= o) return;

    float acc[DQ_R][NT];
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rr][t] = 0.0f;

    for (int ch = lane; ch < nch; ch += 64) {
        uint32_t w[DQ_R][B];
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
            for (int k = 0; k < B; k++) w[rr][k] = wn[rr][k];
        const int chn = ch + 64;
        if (chn < nch) {
#pragma unroll
            for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
                for (int k = 0; k < B; k++) wn[rr][k] = __builtin_nontemporal_load(crow[rr] + chn * B + k);
        }
        const int64_t g = (col0 + ch * 32) / G;
        float sv[DQ_R], mv[DQ_R];
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++) {
            sv[rr] = scale[prow[rr] + g];
            mv[rr] = offset[prow[rr] + g];
        }
        float dot[DQ_R][NT];
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
            for (int t = 0; t < NT; t++) dot[rr][t] = 0.0f;
#pragma unroll
        for (int jb = 0; jb < 4; jb++) {
            float xv[NT][8];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float4* p = reinterpret_cast<const float4*>(xs + t * kc + jb * (nch * 8) + ch * 8);
                const float4 a = p[0], b = p[1];
                xv[t][0] = a.x; xv[t][1] = a.y; xv[t][2] = a.z; xv[t][3] = a.w;
                xv[t][4] = b.x; xv[t][5] = b.y; xv[t][6] = b.z; xv[t][7] = b.w;
            }
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
#pragma unroll
                for (int rr = 0; rr < DQ_R; rr++) {
                    const float q = code_at<B>(w[rr], jb * 8 + jj);
#pragma unroll
                    for (int t = 0; t < NT; t++) dot[rr][t] = fmaf(q, xv[t][jj], dot[rr][t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float cs = ps[t * nch + ch];
#pragma unroll
            for (int rr = 0; rr < DQ_R; rr++) acc[rr][t] = fmaf(sv[rr], dot[rr][t], fmaf(mv[rr], cs, acc[rr][t]));
        }
    }
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            float v = acc[rr][t];
#pragma unroll
            for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
            acc[rr][t] = v;
        }
    }
    if (lane == 0) {
        float* zb = Z + (int64_t)blockIdx.x * zslice;
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++) {
            if (r0 + rr >= o) break;
#pragma unroll
            for (int t = 0; t < NT; t++)
                if (t < nt) zb[(r0 + rr) * zsr + t * zst] = acc[rr][t];
        }
    }
}

// Zt[t][r] = sum_k Zp[k][r][t], k = 0 .. ks-1 in order
__global__ void dequant_reduce_kernel(const float* __restrict__ Zp, int64_t slice, int ks, int64_t o, int nt,
                                      int64_t ldp, float* __restrict__ Zt, int64_t ldz) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < o * nt; e += (int64_t)gridDim.x * 256) {
        const int64_t t = e / o, r = e % o;
        float s = 0.0f;
        for (int k = 0; k < ks; k++) s += Zp[k * slice + r * ldp + t];
        Zt[t * ldz + r] = s;
    }
}

// Y[t][r] = sum_k A_r[k] Zt[t][kb + k] over the diagonal block that holds row r: the full matrix
// (blk = o) or a block-diagonal one (o / blk blocks of blk x blk stored one after another). One
// wavefront per 4 rows (blk is a multiple of 4, so they share a block), lanes along k with float4
// loads of A and of the token rows; HBM-bound on A.
template <int NT>
__global__ __launch_bounds__(256) void sinv_gemv_kernel(const float* __restrict__ A, int64_t o, int64_t blk,
                                                        const float* __restrict__ Zt, int64_t ldz, int nt,
                                                        float* __restrict__ Y, int64_t ldy) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * DQ_R;
    if (r0 >= o) return;
    const int64_t b = r0 / blk, kb = b * blk;
    const float4* arow[DQ_R];
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++) {
        const int64_t r = r0 + rr < o ? r0 + rr : o - 1;
        arow[rr] = reinterpret_cast<const float4*>(A + b * blk * blk + (r - kb) * blk);
    }
    const float4* zrow[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) zrow[t] = reinterpret_cast<const float4*>(Zt + (int64_t)(t < nt ? t : 0) * ldz + kb);
    float acc[DQ_R][NT];
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rr][t] = 0.0f;
    const int64_t n4 = blk >> 2;
#pragma unroll 2
    for (int64_t k4 = lane; k4 < n4; k4 += 64) {
        float4 a[DQ_R], z[NT];
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++) a[rr] = arow[rr][k4];
#pragma unroll
        for (int t = 0; t < NT; t++) z[t] = zrow[t][k4];
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
            for (int t = 0; t < NT; t++)
                acc[rr][t] = fmaf(a[rr].w, z[t].w, fmaf(a[rr].z, z[t].z, fmaf(a[rr].y, z[t].y, fmaf(a[rr].x, z[t].x, acc[rr][t]))));
    }
#pragma unroll
    for (int rr = 0; rr < DQ_R; rr++)
#pragma unroll
        for (int t = 0; t < NT; t++) {
            float v = acc[rr][t];
#pragma unroll
            for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
            acc[rr][t] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int rr = 0; rr < DQ_R; rr++) {
            if (r0 + rr >= o) break;
#pragma unroll
            for (int t = 0; t < NT; t++)
                if (t < nt) Y[t * ldy + r0 + rr] = acc[rr][t];
        }
    }
}

// Y (nt x o, leading dimension ldy) = the token rows of Zt (nt x o, leading dimension ldz) times
// S^{-T}, i.e. y_t = S^{-1} z_t, for up to 8 tokens; S^{-1} full (blk = o) or block-diagonal.
// Returns KQ_EUNSUPPORTED when the shape does not suit the kernel (nt > 8, blk or ldz not a multiple
// of 4, unaligned operands) so that the caller uses the general GEMM.
kq_status sinv_gemv(const float* A, int64_t o, int64_t blk, const float* Zt, int64_t ldz, int64_t nt, float* Y,
                    int64_t ldy, hipStream_t st) {
    if (nt > 8 || nt <= 0 || blk % 4 || ldz % 4 || o % blk || reinterpret_cast<uintptr_t>(A) % 16 ||
        reinterpret_cast<uintptr_t>(Zt) % 16)
        return KQ_EUNSUPPORTED;
    const dim3 grid((unsigned)((o + SG_ROWS_WG - 1) / SG_ROWS_WG));
    const int n = (int)nt;
    if (n == 1) hipLaunchKernelGGL((sinv_gemv_kernel<1>), grid, dim3(256), 0, st, A, o, blk, Zt, ldz, n, Y, ldy);
    else if (n == 2) hipLaunchKernelGGL((sinv_gemv_kernel<2>), grid, dim3(256), 0, st, A, o, blk, Zt, ldz, n, Y, ldy);
    else if (n <= 4) hipLaunchKernelGGL((sinv_gemv_kernel<4>), grid, dim3(256), 0, st, A, o, blk, Zt, ldz, n, Y, ldy);
    else hipLaunchKernelGGL((sinv_gemv_kernel<8>), grid, dim3(256), 0, st, A, o, blk, Zt, ldz, n, Y, ldy);
    return check_launch("sinv_gemv");
}

// Slice width for NT tokens per pass: at most the LDS capacity, and narrow enough to give about
// 512 workgroups (16 wavefronts per CU) while every lane of a wavefront still owns a chunk
// (KC >= 2048).
static int64_t dq_slice(int64_t o, int64_t i, int NT) {
    const int64_t kcmax = DQ_LDS_FLOATS / NT;
    const int64_t rows = (o + DQ_ROWS_WG - 1) / DQ_ROWS_WG;
    int64_t ks = (i + kcmax - 1) / kcmax;
    while (rows * ks < 512 && i / (ks + 1) >= 2048) ks++;
    int64_t kc = (i + ks - 1) / ks;
    kc = (kc + 31) / 32 * 32;
    return kc;
}

static size_t dequant_ws_valu(int64_t o, int64_t i, int64_t nt) {
    int64_t ks = 1;
    for (int NT = 1; NT <= 8; NT *= 2) {
        if (NT > 1 && NT / 2 >= nt) break;
        const int64_t kc = dq_slice(o, i, NT);
        const int64_t k = (i + kc - 1) / kc;
        ks = k > ks ? k : ks;
    }
    return ks > 1 ? (size_t)ks * o * 8 * sizeof(float) : 0;
}

template <int B, int NT>
static void dq_launch(dim3 grid, size_t smem, hipStream_t st, const uint32_t* codes, const float* scale,
                      const float* offset, int64_t o, int64_t i, int G, int64_t KC, const float* X, int64_t ldx,
                      int nt, float* Z, int64_t zsr, int64_t zst, int64_t zslice) {
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(&dequant_gemv_kernel<B, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        attr = true;
    }
    hipLaunchKernelGGL((dequant_gemv_kernel<B, NT>), grid, dim3(DQ_THREADS), smem, st, codes, scale, offset, o, i, G, KC, X,
                       ldx, nt, Z, zsr, zst, zslice);
}

template <int B>
static kq_status dq_dispatch(int NT, dim3 grid, size_t smem, hipStream_t st, const uint32_t* codes,
                             const float* scale, const float* offset, int64_t o, int64_t i, int G, int64_t KC,
                             const float* X, int64_t ldx, int nt, float* Z, int64_t zsr, int64_t zst, int64_t zslice) {
    switch (NT) {
        case 1: dq_launch<B, 1>(grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        case 2: dq_launch<B, 2>(grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        case 4: dq_launch<B, 4>(grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        default: dq_launch<B, 8>(grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
    }
    return check_launch("dequant_gemv");
}

// ----------------------------------------------------------------------- matrix-core variant
// The same product on the int8 matrix cores (v_mfma_i32_16x16x64_i8), for groups that are a multiple
// of 128 columns (or one group per row). Codes are exact int8 operands; each token's x' is scaled
// by a power of two so that |x'| < 2^22 and split into three balanced base-256 digits (int8 limbs,
// 22 bits, about fp32's precision), so every partial product is exact and the int32 sums are
// exact; the three limb sums are recombined in fp32 once per group and scaled by the group's s,
// while mu multiplies the group's float sums of x'. One instruction covers 16 rows x 64 codes x 16
// tokens, so 1 to 16 tokens cost the same.
//
// Layout. A row's 128-code window is split among the four lane groups g of the operand layout:
// group g owns codes 32 g .. 32 g + 31 (exactly `B` words, loaded by one lane), and instruction j
// (0, 1) of the window takes codes 16 j .. 16 j + 15 of each group's chunk. The 16 codes sit in the
// A operand's 16 bytes in an order chosen per width so that unpacking is a few masks (slot()), and
// the staged limbs of x' use the same byte order, so the instruction pairs every code with its own
// column (the instruction sums A(lane i + 16 g)[b] * B(lane j + 16 g)[b] over g and b).
typedef int dm_v4i __attribute__((ext_vector_type(4)));

constexpr int DM_T = 16;            // tokens per pass
constexpr int DM_NW = 8;            // 128-column windows per slice (slices of at most 1024 columns)
constexpr int DM_ROWS = 64;         // rows per row block (4 wavefronts x 16)

// byte slot (4 * register + byte) of code c (0..15) of an instruction's 16 codes
template <int B>
__device__ __forceinline__ int dm_slot(int c) {
    if constexpr (B == 2) return 4 * (c & 3) + (c >> 2);
    else if constexpr (B == 4) return 4 * (2 * (c >> 3) + (c & 1)) + ((c & 7) >> 1);
    else return c;
}

// the code held in byte slot s (the inverse of dm_slot)
template <int B>
__device__ __forceinline__ int dm_code(int s) {
    if constexpr (B == 2) return 4 * (s & 3) + (s >> 2);
    else if constexpr (B == 4) return 8 * ((s >> 2) >> 1) + 2 * (s & 3) + ((s >> 2) & 1);
    else return s;
}

// A operand of instruction j from the lane's `B` words (codes 16 j .. 16 j + 15 of its chunk)
template <int B>
__device__ __forceinline__ dm_v4i dm_unpack(const uint32_t (&w)[B], int j) {
    dm_v4i a;
    if constexpr (B == 2) {
        const uint32_t x = w[j];
        a[0] = (int)(x & 0x03030303u);
        a[1] = (int)((x >> 2) & 0x03030303u);
        a[2] = (int)((x >> 4) & 0x03030303u);
        a[3] = (int)((x >> 6) & 0x03030303u);
    } else if constexpr (B == 4) {
        const uint32_t x0 = w[2 * j], x1 = w[2 * j + 1];
        a[0] = (int)(x0 & 0x0F0F0F0Fu);
        a[1] = (int)((x0 >> 4) & 0x0F0F0F0Fu);
        a[2] = (int)(x1 & 0x0F0F0F0Fu);
        a[3] = (int)((x1 >> 4) & 0x0F0F0F0Fu);
    } else if constexpr (B == 8) {
#pragma unroll
        for (int r = 0; r < 4; r++) a[r] = (int)(w[4 * j + r] ^ 0x80808080u);   // q - 128 as int8
    } else {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int bit = (16 * j + 4 * r + b) * B, wi = bit >> 5, sh = bit & 31;
                uint32_t q = (sh + B > 32) ? __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) : (w[wi] >> sh);
                v |= (q & ((1u << B) - 1u)) << (8 * b);
            }
            a[r] = (int)v;
        }
    }
    return a;
}

template <int B, int NTS, int RB>
__global__ __launch_bounds__(256) void dequant_mfma_kernel(const uint32_t* __restrict__ codes, const float* __restrict__ scale,
                                                           const float* __restrict__ offset, int64_t o, int64_t i,
                                                           int64_t G, int64_t KC, const float* __restrict__ X,
                                                           int64_t ldx, int nt, float* __restrict__ Z, int64_t zsr,
                                                           int64_t zst, int64_t zslice) {
    extern __shared__ __align__(16) unsigned char dm_sm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * KC;
    const int kc = (int)((i - col0) < KC ? (i - col0) : KC);    // multiple of 128
    const int nwin = kc >> 7, nch = kc >> 5, cpt = (int)(KC >> 5);
    unsigned char* limbs = dm_sm;                                              // [KC/128][4][2][3][NTS][16]
    unsigned char* zero16 = dm_sm + (size_t)KC * 3 * NTS;                      // 16 zero bytes
    float* ps = reinterpret_cast<float*>(zero16 + 16);                         // [NTS][KC/32] chunk sums
    float* tinv = ps + (size_t)NTS * cpt;                                      // [NTS] 2^-e_t
    unsigned int* tmax = reinterpret_cast<unsigned int*>(tinv + NTS);          // [NTS] max |x'| bits

    // the wavefront's codes (every window of the slice) and its first group's grid parameters are
    // requested before the staging, so their latency overlaps it
    const int64_t ng = i / G;
    const int64_t wpr = i * B / 32;
    const int tl = lane & 15, lg = lane >> 4;                 // token (output column) / lane group
    const int64_t rw0 = ((int64_t)blockIdx.y * 4 + wave) * (16 * RB);
    const bool wlive = rw0 < o;
    const uint32_t* cb[RB];
#pragma unroll
    for (int k = 0; k < RB; k++) {
        const int64_t r = rw0 + 16 * k + tl;
        cb[k] = codes + (r < o ? r : o - 1) * wpr + ((col0 >> 5) + lg) * B;
    }
    uint32_t wall[DM_NW][RB][B];
#pragma unroll
    for (int W = 0; W < DM_NW; W++)
#pragma unroll
        for (int k = 0; k < RB; k++)
#pragma unroll
            for (int q = 0; q < B; q++)
                wall[W][k][q] = (wlive && W < nwin) ? __builtin_nontemporal_load(cb[k] + W * 4 * B + q) : 0u;
    int64_t prow[RB][4];
#pragma unroll
    for (int k = 0; k < RB; k++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = rw0 + 16 * k + 4 * lg + r;
            prow[k][r] = (row < o ? row : o - 1) * ng;
        }
    float svn[RB][4], mvn[RB][4];
    {
        const int64_t g0 = col0 / G;
#pragma unroll
        for (int k = 0; k < RB; k++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                svn[k][r] = scale[prow[k][r] + g0];
                mvn[k][r] = offset[prow[k][r] + g0];
            }
    }

    // stage x' over (token, 32-column chunk) pairs, at most two per thread, kept in registers: chunk
    // sums and each token's max |x'| (an integer max of non-negative float bits, order-free), then
    // the int8 limbs, each (instruction, limb) fragment of 16 bytes assembled and stored at once
    if (tid < NTS) tmax[tid] = 0u;
    if (tid < 4) reinterpret_cast<uint32_t*>(zero16)[tid] = 0u;
    __syncthreads();
    float v[2][32];
#pragma unroll
    for (int pp = 0; pp < 2; pp++) {
        const int p = tid + 256 * pp;
        const int t = p / nch, ch = p - t * nch;
        float sacc = 0.0f, mx = 0.0f;
        const bool on = p < NTS * nch && t < nt;
        const float* xr = X + (int64_t)(on ? t : 0) * ldx + col0 + 32 * (on ? ch : 0);
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const float4 x4 = on ? *reinterpret_cast<const float4*>(xr + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
            v[pp][4 * q] = x4.x; v[pp][4 * q + 1] = x4.y; v[pp][4 * q + 2] = x4.z; v[pp][4 * q + 3] = x4.w;
            sacc += (x4.x + x4.y) + (x4.z + x4.w);
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x4.x), fabsf(x4.y)), fmaxf(fabsf(x4.z), fabsf(x4.w))));
        }
        if (p < NTS * nch) {
            ps[t * cpt + ch] = sacc;
            atomicMax(&tmax[t], __float_as_uint(mx));
        }
    }
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < 2; pp++) {
        const int p = tid + 256 * pp;
        if (p >= NTS * nch) continue;
        const int t = p / nch, ch = p - t * nch;
        const int W = ch >> 2, g = ch & 3;
        unsigned char* base0 = limbs + ((((size_t)W * 4 + g) * 2) * 3) * (NTS * 16) + t * 16;
        const float mx = __uint_as_float(tmax[t]);
        const int e = mx > 0.0f ? 21 - ilogbf(mx) : 0;       // |x'| 2^e < 2^22
        if (ch == 0) tinv[t] = ldexpf(1.0f, -e);
        const float f = ldexpf(1.0f, e);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            int u[16];
#pragma unroll
            for (int c = 0; c < 16; c++) u[c] = (int)rintf(v[pp][16 * j + c] * f);
            unsigned char* base = base0 + (size_t)j * 3 * (NTS * 16);
#pragma unroll
            for (int l3 = 2; l3 >= 0; l3--) {
                // digit l3 of every code (l3 = 2 the lowest), then remove it
                int dg[16];
#pragma unroll
                for (int c = 0; c < 16; c++) {
                    dg[c] = l3 == 0 ? u[c] : ((u[c] + 128) & 255) - 128;
                    u[c] = (u[c] - dg[c]) >> 8;
                }
                uint32_t wd[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    uint32_t x = 0;
#pragma unroll
                    for (int bb = 0; bb < 4; bb++) x |= ((uint32_t)dg[dm_code<B>(4 * r + bb)] & 0xFFu) << (8 * bb);
                    wd[r] = x;
                }
                *reinterpret_cast<uint4*>(base + l3 * (NTS * 16)) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
        }
    }
    __syncthreads();
    if (!wlive) return;

    // main loop: one read of the x' fragments per instruction serves the wavefront's RB row blocks
    const float tinv_t = tl < NTS ? tinv[tl] : 0.0f;
    float zf[RB][4];
    dm_v4i acc[RB][3];
#pragma unroll
    for (int k = 0; k < RB; k++) {
#pragma unroll
        for (int r = 0; r < 4; r++) zf[k][r] = 0.0f;
#pragma unroll
        for (int l3 = 0; l3 < 3; l3++) acc[k][l3] = dm_v4i{0, 0, 0, 0};
    }
    int run0 = 0;     // first window of the open group run
#pragma unroll
    for (int W = 0; W < DM_NW; W++) {
        if (W >= nwin) break;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            dm_v4i bv[3];
#pragma unroll
            for (int l3 = 0; l3 < 3; l3++) {
                const unsigned char* src = tl < NTS
                    ? limbs + ((((size_t)W * 4 + lg) * 2 + j) * 3 + l3) * (NTS * 16) + tl * 16 : zero16;
                bv[l3] = *reinterpret_cast<const dm_v4i*>(src);
            }
#pragma unroll
            for (int k = 0; k < RB; k++) {
                const dm_v4i a = dm_unpack<B>(wall[W][k], j);
#pragma unroll
                for (int l3 = 0; l3 < 3; l3++) acc[k][l3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bv[l3], acc[k][l3], 0, 0, 0);
            }
        }
        const int64_t cend = col0 + (int64_t)(W + 1) * 128;
        if (cend % G == 0 || W + 1 == nwin) {
            // close the run: windows run0 .. W of one group (its s and mu were requested ahead)
            float gsum = 0.0f;
            if (tl < NTS)
                for (int ch = 4 * run0; ch < 4 * (W + 1); ch++) gsum += ps[tl * cpt + ch];
            const bool more = W + 1 < nwin;
            const int64_t gn = cend / G;          // the next group, if the slice goes on
#pragma unroll
            for (int k = 0; k < RB; k++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float sv = svn[k][r], mv = mvn[k][r];
                    if (more) {
                        svn[k][r] = scale[prow[k][r] + gn];
                        mvn[k][r] = offset[prow[k][r] + gn];
                    }
                    const float dot = fmaf((float)acc[k][0][r], 65536.0f, fmaf((float)acc[k][1][r], 256.0f, (float)acc[k][2][r]));
                    const float mo = B == 8 ? fmaf(128.0f, sv, mv) : mv;
                    zf[k][r] = fmaf(sv, dot * tinv_t, fmaf(mo, gsum, zf[k][r]));
                }
#pragma unroll
                for (int l3 = 0; l3 < 3; l3++) acc[k][l3] = dm_v4i{0, 0, 0, 0};
            }
            run0 = W + 1;
        }
    }
    if (tl < nt) {
        float* zb = Z + (int64_t)blockIdx.x * zslice;
#pragma unroll
        for (int k = 0; k < RB; k++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t row = rw0 + 16 * k + 4 * lg + r;
                if (row < o) zb[row * zsr + tl * zst] = zf[k][r];
            }
    }
}

static bool dm_eligible(int64_t i, int G) { return i % 128 == 0 && G % 128 == 0; }

// tokens staged per pass for nt tokens
static int dm_nts(int64_t nt) { return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : nt <= 8 ? 8 : 16; }

static size_t dm_smem(int64_t KC, int NTS) {
    return (size_t)KC * 3 * NTS + 16 + ((size_t)NTS * (KC / 32) + 2 * NTS) * sizeof(float);
}

// Slice width: 1024 columns (all of a slice's codes fit in a lane's registers), narrowed to 256 at
// most while the grid has fewer than 512 workgroups; one block of 16 rows per wavefront.
static void dm_plan(int64_t o, int64_t i, int NTS, int64_t& KC, int64_t& ks, int& RB) {
    KC = 128 * DM_NW;
    RB = 1;
    (void)NTS;
    auto wgs = [&](int64_t kc) { return ((o + 63) / 64) * ((i + kc - 1) / kc); };
    while (wgs(KC) < 512 && KC > 256) KC /= 2;
    ks = (i + KC - 1) / KC;
}

template <int B, int NTS>
static void dm_launch_rb(int RB, dim3 grid, size_t smem, hipStream_t st, const uint32_t* codes, const float* scale,
                         const float* offset, int64_t o, int64_t i, int64_t G, int64_t KC, const float* X, int64_t ldx,
                         int nt, float* Z, int64_t zsr, int64_t zst, int64_t zslice) {
    (void)RB;   // one block of 16 rows per wavefront (dm_plan)
    static bool attr = false;
    if (!attr) {
        hipFuncSetAttribute(reinterpret_cast<const void*>(&dequant_mfma_kernel<B, NTS, 1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 72 * 1024);
        attr = true;
    }
    hipLaunchKernelGGL((dequant_mfma_kernel<B, NTS, 1>), grid, dim3(256), smem, st, codes, scale, offset, o, i, G, KC,
                       X, ldx, nt, Z, zsr, zst, zslice);
}

template <int B>
static void dm_launch(int NTS, int RB, dim3 grid, size_t smem, hipStream_t st, const uint32_t* codes,
                      const float* scale, const float* offset, int64_t o, int64_t i, int64_t G, int64_t KC,
                      const float* X, int64_t ldx, int nt, float* Z, int64_t zsr, int64_t zst, int64_t zslice) {
    switch (NTS) {
        case 1: dm_launch_rb<B, 1>(RB, grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        case 2: dm_launch_rb<B, 2>(RB, grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        case 4: dm_launch_rb<B, 4>(RB, grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        case 8: dm_launch_rb<B, 8>(RB, grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
        default: dm_launch_rb<B, 16>(RB, grid, smem, st, codes, scale, offset, o, i, G, KC, X, ldx, nt, Z, zsr, zst, zslice); break;
    }
}

static kq_status dequant_mfma(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i,
                              int bits, int G, const float* X, int64_t ldx, int64_t nt, float* Zt, int64_t ldz,
                              float* Zp, hipStream_t st) {
    for (int64_t t0 = 0; t0 < nt; t0 += DM_T) {
        const int cnt = (int)((nt - t0) < DM_T ? (nt - t0) : DM_T);
        const int NTS = dm_nts(cnt);
        int64_t KC, ks;
        int RB;
        dm_plan(o, i, NTS, KC, ks, RB);
        if (ks > 1 && !Zp) return fail(KQ_EWORKSPACE, "dequant_gemv: slice workspace missing");
        const int64_t rgroups = (o + 64LL * RB - 1) / (64LL * RB);
        if (rgroups > 65535) return fail(KQ_ESHAPE, "dequant_gemv: too many rows");
        const dim3 grid((unsigned)ks, (unsigned)rgroups);
        const size_t smem = dm_smem(KC, NTS);
        const int64_t zslice = o * DM_T;
        float* dst = ks > 1 ? Zp : Zt + t0 * ldz;
        const int64_t zsr = ks > 1 ? DM_T : 1, zst = ks > 1 ? 1 : ldz;
        const float* Xp = X + t0 * ldx;
#define KQ_DM(b) case b: dm_launch<b>(NTS, RB, grid, smem, st, codes, scale, offset, o, i, (int64_t)G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
        switch (bits) {
            KQ_DM(2) KQ_DM(3) KQ_DM(4) KQ_DM(5) KQ_DM(6) KQ_DM(7) KQ_DM(8)
            default: return fail(KQ_EUNSUPPORTED, "dequant_gemv: bits");
        }
#undef KQ_DM
        KQ_TRY(check_launch("dequant_mfma"));
        if (ks > 1) {
            const int64_t n = o * cnt;
            const unsigned b = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
            hipLaunchKernelGGL(dequant_reduce_kernel, dim3(b), dim3(256), 0, st, Zp, zslice, (int)ks, o, cnt,
                               (int64_t)DM_T, Zt + t0 * ldz, ldz);
            KQ_TRY(check_launch("dequant_reduce"));
        }
    }
    return KQ_OK;
}

// slice partials of either kernel (the larger of the two plans, so any group size fits)
size_t dequant_ws(int64_t o, int64_t i, int64_t nt) {
    size_t m = 0;
    for (int NTS = 1; NTS <= 16; NTS *= 2) {
        if (NTS > 1 && NTS / 2 >= nt) break;
        int64_t KC, ks;
        int RB;
        dm_plan(o, i, NTS, KC, ks, RB);
        const size_t mm = ks > 1 ? (size_t)ks * o * DM_T * sizeof(float) : 0;
        m = mm > m ? mm : m;
    }
    const size_t v = dequant_ws_valu(o, i, nt);
    return m > v ? m : v;
}

// Zt (nt x o, leading dimension ldz) = X Q''^T for the nt token rows of X (leading dimension ldx);
// Zp: workspace of dequant_ws(o, i, nt) bytes (may be null when that is 0).
kq_status dequant_gemv(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i, int bits,
                       int group, const float* X, int64_t ldx, int64_t nt, float* Zt, int64_t ldz, float* Zp,
                       hipStream_t st) {
    const int G = group ? group : (int)i;
    if (G % 32 || i % G || i % 32) return fail(KQ_EUNSUPPORTED, "dequant_gemv: group must be a multiple of 32");
    if (bits < 2 || bits > 8) return fail(KQ_EUNSUPPORTED, "dequant_gemv: bits must be in 2..8");
    if (o <= 0 || nt <= 0 || (o + DQ_ROWS_WG - 1) / DQ_ROWS_WG > 65535) return fail(KQ_ESHAPE, "dequant_gemv: bad sizes");
    if (ldx % 4 || reinterpret_cast<uintptr_t>(X) % 16) return fail(KQ_EINVAL, "dequant_gemv: x' rows must be 16-byte aligned");
    // the matrix-core kernel for token blocks of more than 4 (measured: at 1 token the VALU kernel is
    // about twice as fast on the C2-C4 layer shapes, at 8 tokens the matrix-core one up to 2.2x)
    if (dm_eligible(i, G) && nt > 4) return dequant_mfma(codes, scale, offset, o, i, bits, G, X, ldx, nt, Zt, ldz, Zp, st);
    for (int64_t t0 = 0; t0 < nt; t0 += 8) {
        const int cnt = (int)((nt - t0) < 8 ? (nt - t0) : 8);
        const int NT = cnt == 1 ? 1 : cnt == 2 ? 2 : cnt <= 4 ? 4 : 8;
        const int64_t KC = dq_slice(o, i, NT);
        const int64_t ks = (i + KC - 1) / KC;
        if (ks > 1 && !Zp) return fail(KQ_EWORKSPACE, "dequant_gemv: slice workspace missing");
        const dim3 grid((unsigned)ks, (unsigned)((o + DQ_ROWS_WG - 1) / DQ_ROWS_WG));
        const size_t smem = ((size_t)NT * KC + (size_t)NT * (KC / 32)) * sizeof(float);
        float* dst = ks > 1 ? Zp : Zt + t0 * ldz;
        const int64_t zsr = ks > 1 ? 8 : 1, zst = ks > 1 ? 1 : ldz;
        const int64_t zslice = o * 8;
        const float* Xp = X + t0 * ldx;
        kq_status s = KQ_OK;
        switch (bits) {
            case 2: s = dq_dispatch<2>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            case 3: s = dq_dispatch<3>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            case 4: s = dq_dispatch<4>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            case 5: s = dq_dispatch<5>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            case 6: s = dq_dispatch<6>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            case 7: s = dq_dispatch<7>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
            default: s = dq_dispatch<8>(NT, grid, smem, st, codes, scale, offset, o, i, G, KC, Xp, ldx, cnt, dst, zsr, zst, zslice); break;
        }
        KQ_TRY(s);
        if (ks > 1) {
            const int64_t n = o * cnt;
            const unsigned b = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
            hipLaunchKernelGGL(dequant_reduce_kernel, dim3(b), dim3(256), 0, st, Zp, zslice, (int)ks, o, cnt, (int64_t)8,
                               Zt + t0 * ldz, ldz);
            KQ_TRY(check_launch("dequant_reduce"));
        }
    }
    return KQ_OK;
}

}  // namespace kq
