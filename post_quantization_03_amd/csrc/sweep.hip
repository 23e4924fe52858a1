// GPTQ column sweep (KronQ review page, Prior limitations / Goal: the column-wise OBS update with H_X
// only, left unchanged by KronQ), the layer loss used for verification, and the sensitivity score
// tr(H_G) tr(H_X) (review page, Method (2)).
//
// Sweep layout. Columns are processed in blocks of 128. Inside a block every row is owned by a group
// of 16 lanes of one wavefront; lane q holds the 8 columns q, q + 16, ..., q + 112 in registers, so
// the columns still to be updated stay spread over all 16 lanes as the sweep advances. For column j
// the owning lane's value is broadcast within the 16-lane group, every lane rounds it to the grid
// (same arithmetic on every lane, so no second broadcast), and updates its own later columns with
// the row j of the block's R (staged once per work-group in LDS). The lazy trailing updates
// W[:, b1:] -= E R[b0:b1, b1:] run on the fp32 MFMA GEMM, in two levels (see SW_SB).
#include <cmath>
#include <mutex>

#include "kq_internal.h"

namespace kq {

constexpr int SW_B = 128;         // column block
constexpr int SW_ROWS = 16;       // rows per work-group (16 lanes each)

// Candidate range factor m of nsearch: spread evenly over [1/2, 1] (Hessian-aware scale search).
__device__ __forceinline__ float search_alpha(int m, int nsearch) {
    return nsearch > 1 ? 0.5f + 0.5f * (float)m / (float)(nsearch - 1) : 1.0f;
}

// Per-row grid over the whole row before the sweep (group = 0): offset = min, scale = (max-min)/L.
__global__ __launch_bounds__(256) void row_grid_kernel(const float* __restrict__ W, int64_t i, int64_t ldw, float L,
                                                       float* __restrict__ scale, float* __restrict__ offset) {
    __shared__ float smin[256], smax[256];
    const int64_t r = blockIdx.x;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t c = threadIdx.x; c < i; c += 256) {
        const float v = W[r * ldw + c];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    smin[threadIdx.x] = mn;
    smax[threadIdx.x] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            smin[threadIdx.x] = fminf(smin[threadIdx.x], smin[threadIdx.x + w]);
            smax[threadIdx.x] = fmaxf(smax[threadIdx.x], smax[threadIdx.x + w]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        offset[r] = smin[0];
        scale[r] = (smax[0] - smin[0]) / L;
    }
}

// Per-row Hessian-aware grid (group = 0): the [min, max] range shrunk about its midpoint by the
// factor (of nsearch in [1/2, 1]) with the smallest rounding error weighted by 1 / R_cc^2 (first
// minimum). The row and the weights sit in LDS (8 i bytes); per candidate every thread sums its
// columns, the wavefronts reduce by shuffles and the four partials are added in a fixed order by
// every thread, so all threads take the same decision.
__global__ __launch_bounds__(256) void row_grid_search_kernel(const float* __restrict__ W, int64_t i, int64_t ldw,
                                                              float L, float* __restrict__ scale,
                                                              float* __restrict__ offset, const float* __restrict__ R,
                                                              int64_t ldr, int nsearch) {
    extern __shared__ __align__(16) float rg_sm[];
    float* vrow = rg_sm;            // i
    float* wgt = rg_sm + i;         // i
    __shared__ float part[2][4];
    __shared__ float smin[4], smax[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = blockIdx.x;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t c = tid; c < i; c += 256) {
        const float v = W[r * ldw + c];
        const float rc = R[c * ldr + c];
        vrow[c] = v;
        wgt[c] = 1.0f / (rc * rc);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, m, 64));
        mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    if (lane == 0) { smin[wave] = mn; smax[wave] = mx; }
    __syncthreads();
    mn = fminf(fminf(smin[0], smin[1]), fminf(smin[2], smin[3]));
    mx = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
    if (!(mx > mn)) {
        if (tid == 0) { offset[r] = mn; scale[r] = (mx - mn) / L; }
        return;
    }
    const float c = 0.5f * (mn + mx), h = 0.5f * (mx - mn);
    float best = INFINITY, ba = 1.0f;
    for (int m = 0; m < nsearch; m++) {
        const float a = search_alpha(m, nsearch);
        const float sa = 2.0f * a * h / L, ma = c - a * h, ia = 1.0f / sa;
        float err = 0.0f;
        for (int64_t col = tid; col < i; col += 256) {
            const float v = vrow[col];
            const float qf = fminf(fmaxf(rintf((v - ma) * ia), 0.0f), L);
            const float dv = v - fmaf(sa, qf, ma);
            err = fmaf(dv * dv, wgt[col], err);
        }
#pragma unroll
        for (int k = 32; k > 0; k >>= 1) err += __shfl_xor(err, k, 64);
        if (lane == 0) part[m & 1][wave] = err;
        __syncthreads();
        const float tot = (part[m & 1][0] + part[m & 1][1]) + (part[m & 1][2] + part[m & 1][3]);
        if (tot < best) { best = tot; ba = a; }
    }
    if (tid == 0) {
        offset[r] = c - ba * h;
        scale[r] = 2.0f * ba * h / L;
    }
}

// Value of lane `src` of each 16-lane row, broadcast to the whole row (DPP row_newbcast: a VALU move,
// no LDS round trip). `src` must fold to a constant after unrolling.
__device__ inline float row_bcast(float x, int src) {
    const int xi = __float_as_int(x);
    int r;
    switch (src) {
#define KQ_BC(n) case n: r = __builtin_amdgcn_update_dpp(0, xi, 0x150 + n, 0xF, 0xF, false); break;
        KQ_BC(0) KQ_BC(1) KQ_BC(2) KQ_BC(3) KQ_BC(4) KQ_BC(5) KQ_BC(6) KQ_BC(7)
        KQ_BC(8) KQ_BC(9) KQ_BC(10) KQ_BC(11) KQ_BC(12) KQ_BC(13) KQ_BC(14)
        default: r = __builtin_amdgcn_update_dpp(0, xi, 0x150 + 15, 0xF, 0xF, false); break;
#undef KQ_BC
    }
    return __int_as_float(r);
}

template <int G, bool SEARCH>
__global__ __launch_bounds__(256) void sweep_block_kernel(float* __restrict__ W, int64_t o, int64_t i, int64_t ldw,
                                                          const float* __restrict__ R, int64_t ldr, int64_t b0,
                                                          int bits, uint32_t* __restrict__ codes,
                                                          float* __restrict__ scale, float* __restrict__ offset,
                                                          float* __restrict__ row_loss, float* __restrict__ E,
                                                          int64_t lde, int first, int nsearch) {
    extern __shared__ __align__(16) float sm[];
    float* Rb = sm;                        // 128 x 128
    float* rdiag = sm + SW_B * SW_B;       // 128 reciprocals of R_jj
    uint8_t* cl = reinterpret_cast<uint8_t*>(rdiag + SW_B);  // 16 rows x 128 codes
    const int tid = threadIdx.x;
    for (int e = tid; e < SW_B * SW_B / 4; e += 256) {
        const int a = e / (SW_B / 4), c4 = (e % (SW_B / 4)) * 4;
        const float4 v = *reinterpret_cast<const float4*>(R + (b0 + a) * ldr + b0 + c4);
        *reinterpret_cast<float4*>(Rb + a * SW_B + c4) = v;
    }
    __syncthreads();
    if (tid < SW_B) rdiag[tid] = 1.0f / Rb[tid * SW_B + tid];
    __syncthreads();

    const int q = tid & 15, rl = tid >> 4;
    const int64_t row = (int64_t)blockIdx.x * SW_ROWS + rl;
    const bool live = row < o;
    const int64_t rr = live ? row : 0;
    const float L = (float)((1 << bits) - 1);
    const int ng = G ? (int)(i / G) : 1;
    float* wrow = W + rr * ldw + b0;
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) v[u] = live ? wrow[16 * u + q] : 0.0f;
    float mu = 0.0f, s = 0.0f, invs = 0.0f;
    if (G == 0) {
        mu = offset[rr];
        s = scale[rr];
        invs = s > 0.0f ? 1.0f / s : 0.0f;
    }
    int code[8];
    float eown[8];
    float loss = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; u++) { code[u] = 0; eown[u] = 0.0f; }

    // Two unrolled levels, so every column index below is a constant. The reciprocals of R_jj for the
    // 16 columns of a lane group and the lane's entries of R row j + 1 are loaded one step ahead,
    // so the per-column chain (broadcast, round, error, update) waits on no LDS access.
    const int cq = q;  // lane's column within each 16-column group
    float rnext[8];
#pragma unroll
    for (int u = 0; u < 8; u++) rnext[u] = Rb[16 * u + cq];  // row 0
#pragma unroll
    for (int uj = 0; uj < SW_B / 16; uj++) {
        float rd[16];
#pragma unroll
        for (int t = 0; t < 16; t++) rd[t] = rdiag[16 * uj + t];
#pragma unroll
        for (int qj = 0; qj < 16; qj++) {
            const int j = 16 * uj + qj;
            float rcur[8];
#pragma unroll
            for (int u = 0; u < 8; u++) rcur[u] = rnext[u];
            if (j + 1 < SW_B) {
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (16 * u + 15 > j + 1) rnext[u] = Rb[(j + 1) * SW_B + 16 * u + cq];
            }
            if (G > 0 && (j % (G > 0 ? G : 1)) == 0) {
                float mn = INFINITY, mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    if (16 * u + 15 < j || 16 * u >= j + G) continue;
                    const int col = 16 * u + cq;
                    if (col >= j && col < j + G) { mn = fminf(mn, v[u]); mx = fmaxf(mx, v[u]); }
                }
#pragma unroll
                for (int w = 8; w > 0; w >>= 1) {
                    mn = fminf(mn, __shfl_xor(mn, w, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, w, 16));
                }
                mu = mn;
                s = (mx - mn) / L;
                if (SEARCH && nsearch > 0 && mx > mn) {
                    // Hessian-aware grid: the range shrunk about its midpoint by the factor (of nsearch
                    // in [1/2, 1]) with the smallest rounding error weighted by 1 / R_cc^2; the row's
                    // total is taken from lane 0 of the 16 so that every lane makes the same choice
                    const float c = 0.5f * (mn + mx), h = 0.5f * (mx - mn);
                    float wd[8];
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const float rr_ = rdiag[16 * u + cq];
                        wd[u] = rr_ * rr_;
                    }
                    float best = INFINITY, ba = 1.0f;
                    for (int m = 0; m < nsearch; m++) {
                        const float a = search_alpha(m, nsearch);
                        const float sa = 2.0f * a * h / L, ma = c - a * h, ia = 1.0f / sa;
                        float err = 0.0f;
#pragma unroll
                        for (int u = 0; u < 8; u++) {
                            if (16 * u + 15 < j || 16 * u >= j + G) continue;
                            const int col = 16 * u + cq;
                            if (col >= j && col < j + G) {
                                const float qf = fminf(fmaxf(rintf((v[u] - ma) * ia), 0.0f), L);
                                const float dv = v[u] - fmaf(sa, qf, ma);
                                err = fmaf(dv * dv, wd[u], err);
                            }
                        }
#pragma unroll
                        for (int w = 8; w > 0; w >>= 1) err += __shfl_xor(err, w, 16);
                        err = row_bcast(err, 0);
                        if (err < best) { best = err; ba = a; }
                    }
                    mu = c - ba * h;
                    s = 2.0f * ba * h / L;
                }
                invs = s > 0.0f ? 1.0f / s : 0.0f;
                if (live && cq == 0) {
                    const int64_t gidx = (b0 + j) / (G > 0 ? G : 1);
                    offset[rr * ng + gidx] = mu;
                    scale[rr * ng + gidx] = s;
                }
            }
            const float w = row_bcast(v[uj], qj);
            const float uu = (w - mu) * invs;
            const float qf = fminf(fmaxf(rintf(uu), 0.0f), L);
            const float deq = fmaf(s, qf, mu);
            const float e = (w - deq) * rd[qj];
            loss = fmaf(e, e, loss);
            const bool own = (cq == qj);
            code[uj] = own ? (int)qf : code[uj];
            eown[uj] = own ? e : eown[uj];
            // columns of group uj: the owner takes the rounded value, later columns the update
            v[uj] = own ? deq : (cq > qj ? fmaf(-e, rcur[uj], v[uj]) : v[uj]);
#pragma unroll
            for (int u = uj + 1; u < 8; u++) v[u] = fmaf(-e, rcur[u], v[u]);
        }
    }

    // outputs: w^ back into W, scaled errors into E, codes packed per row, loss
    if (live) {
#pragma unroll
        for (int u = 0; u < 8; u++) {
            wrow[16 * u + q] = v[u];
            E[rr * lde + 16 * u + q] = eown[u];
        }
        if (q == 0 && row_loss) row_loss[rr] = (first ? 0.0f : row_loss[rr]) + loss;
    }
#pragma unroll
    for (int u = 0; u < 8; u++) cl[rl * SW_B + 16 * u + q] = (uint8_t)code[u];
    __syncthreads();
    const int nw = 4 * bits;   // words per row per block
    const int64_t wpr = i * bits / 32;
    if (live) {
        for (int wd = q; wd < nw; wd += 16) {
            uint32_t word = 0;
            for (int p = 0; p < 32; p++) {
                const int B = 32 * wd + p, col = B / bits, t = B % bits;
                word |= (uint32_t)((cl[rl * SW_B + col] >> t) & 1) << p;
            }
            codes[rr * wpr + (b0 / 32) * bits + wd] = word;
        }
    }
}

}  // namespace kq

using namespace kq;

// Lazy updates in two levels: inside a super-block of SW_SB columns each block's errors update the
// rest of the super-block (K = 128); at the super-block's end the trailing columns receive one
// update with K = SW_SB, so most of the trailing-update FLOP run in deep-K GEMMs. Measured on MI355X
// against 256 and 512 (and 2048 with 2048-wide factor panels): 1024 took the least time on the
// 28672 x 8192, 5120 x 13824 and 4096 x 4096 layers (quantize phase 22.0, 14.3, 1.82 ms with 512).
constexpr int SW_SB = 1024;

size_t quantize_ws(int64_t o) {
    Sizer z;
    z.take<float>((size_t)o * SW_SB);
    return z.used;
}

// Rows are independent once R is fixed, so a tall sweep runs on up to SW_PARTS row panels at once: the
// first on the caller's stream, the others on side queues of the library, forked from and joined back
// into the caller's stream by events. One panel's latency-bound 128-step block sweeps then run beside
// another's trailing-update GEMMs. The queues (default priority) and events are created on a device's
// first such call and kept until the process ends; they carry no data between calls, and the mutex
// keeps one call's event sequence intact against other host threads.
// Measured on the layer shapes here: with 28672 rows the four panels cut the phase by a tenth; with
// 4096 and 5120 rows they lengthen it (the queues share the device's few hardware queues, and the
// smaller launches lose more to their tails), so panels start at 16384 rows.
constexpr int SW_PARTS = 4;
constexpr int64_t SW_PART_MIN_ROWS = 4096;   // rows per panel at least
constexpr int64_t SW_PANELS_FROM = 16384;    // fewer rows: one panel
struct SweepPartQueues {
    hipStream_t side[SW_PARTS - 1] = {};
    hipEvent_t fork = nullptr, join[SW_PARTS - 1] = {};
    bool ok = false;
};
static std::mutex g_sp_mu;
static SweepPartQueues g_sp[64];

static kq_status sweep_part_queues(SweepPartQueues** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(KQ_EHIP, "sweep queues: no device");
    SweepPartQueues& q = g_sp[dev];
    if (!q.ok) {
        const unsigned fl = hipEventDisableTiming | hipEventDisableSystemFence;
        if (hipEventCreateWithFlags(&q.fork, fl) != hipSuccess) return fail(KQ_EHIP, "sweep queues: event creation failed");
        for (int k = 0; k < SW_PARTS - 1; k++) {
            if (hipStreamCreateWithFlags(&q.side[k], hipStreamNonBlocking) != hipSuccess)
                return fail(KQ_EHIP, "sweep queues: stream creation failed");
            if (hipEventCreateWithFlags(&q.join[k], fl) != hipSuccess)
                return fail(KQ_EHIP, "sweep queues: event creation failed");
        }
        q.ok = true;
    }
    *out = &q;
    return KQ_OK;
}

// The column-block sweep of rows [0, o) of W (and of the row-indexed outputs passed with them) on one
// queue: per 128-column block the block kernel, then the lazy trailing updates in two levels.
static kq_status sweep_rows(float* W, int64_t o, int64_t i, int64_t ldw, const float* R, int64_t ldr, int bits,
                            int group, int candidates, uint32_t* codes, float* scale, float* offset, float* row_loss,
                            float* E, size_t smem, hipStream_t st) {
    const dim3 grid((unsigned)((o + SW_ROWS - 1) / SW_ROWS));
    for (int64_t s0 = 0; s0 < i; s0 += SW_SB) {
        const int64_t s1 = s0 + SW_SB < i ? s0 + SW_SB : i;
        for (int64_t b0 = s0; b0 < s1; b0 += SW_B) {
            const int first = b0 == 0;
            float* Eb = E + (b0 - s0);
#define KQ_SW(g, srch) hipLaunchKernelGGL((sweep_block_kernel<g, srch>), grid, dim3(256), smem, st, W, o, i, ldw, R, ldr, b0, bits, codes, scale, offset, row_loss, Eb, (int64_t)SW_SB, first, candidates)
#define KQ_SW2(g) if (candidates > 0) KQ_SW(g, true); else KQ_SW(g, false);
            switch (group) {
                case 0: KQ_SW2(0) break;
                case 16: KQ_SW2(16) break;
                case 32: KQ_SW2(32) break;
                case 64: KQ_SW2(64) break;
                default: KQ_SW2(128) break;
            }
#undef KQ_SW2
#undef KQ_SW
            KQ_TRY(check_launch("sweep_block"));
            // the rest of the super-block: W[:, b1:s1] -= E_b R[b0:b1, b1:s1]
            const int64_t b1 = b0 + SW_B;
            if (b1 < s1) {
                GemmArgs<float> g = gemm_args<float>(o, s1 - b1, SW_B, Eb, SW_SB, R + b0 * ldr + b1, ldr, W + b1, ldw,
                                                     -1.0f, 1.0f);
                KQ_TRY(gemm<float>(g, false, false, st));
            }
        }
        // columns after the super-block: W[:, s1:] -= E R[s0:s1, s1:]
        if (s1 < i) {
            GemmArgs<float> g = gemm_args<float>(o, i - s1, s1 - s0, E, SW_SB, R + s0 * ldr + s1, ldr, W + s1, ldw,
                                                 -1.0f, 1.0f);
            KQ_TRY(gemm<float>(g, false, false, st));
        }
    }
    return KQ_OK;
}

#define KQ_HIPS(expr)                                                                   \
    do {                                                                                \
        if ((expr) != hipSuccess) return fail(KQ_EHIP, "%s failed", #expr);            \
    } while (0)

extern "C" kq_status kq_quantize_layer_search(float* W, int64_t o, int64_t i, int64_t ldw, const float* R, int64_t ldr,
                                              int bits, int group, int block, int candidates, uint32_t* codes,
                                              float* scale, float* offset, float* row_loss, void* ws, size_t ws_bytes,
                                              kq_stream stream) {
    if (!W || !R || !codes || !scale || !offset) return fail(KQ_EINVAL, "kq_quantize_layer: null pointer");
    if (candidates < 0 || candidates > 4096) return fail(KQ_EINVAL, "kq_quantize_layer: candidates must be in 0..4096");
    if (o <= 0 || i <= 0 || ldw < i || ldr < i) return fail(KQ_ESHAPE, "kq_quantize_layer: bad sizes");
    if (bits < 2 || bits > 8) return fail(KQ_EUNSUPPORTED, "kq_quantize_layer: bits must be in 2..8");
    if (block != SW_B) return fail(KQ_EUNSUPPORTED, "kq_quantize_layer: block must be 128");
    if (i % SW_B) return fail(KQ_ESHAPE, "kq_quantize_layer: i must be a multiple of 128");
    if (!(group == 0 || group == 16 || group == 32 || group == 64 || group == 128))
        return fail(KQ_EUNSUPPORTED, "kq_quantize_layer: group must be 0, 16, 32, 64 or 128");
    if ((i * bits) % 32) return fail(KQ_ESHAPE, "kq_quantize_layer: i*bits must be a multiple of 32");
    if (ldw % 4 || ldr % 4 || !aligned16(W) || !aligned16(R)) return fail(KQ_EINVAL, "kq_quantize_layer: alignment");
    if (!ws || ws_bytes < quantize_ws(o)) return fail(KQ_EWORKSPACE, "kq_quantize_layer: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    float* E = ar.take<float>((size_t)o * SW_SB);
    if (o > 2147483647LL * SW_ROWS) return fail(KQ_ESHAPE, "kq_quantize_layer: o too large");
    const float L = (float)((1 << bits) - 1);
    if (group == 0) {
        if (candidates > 0) {
            const size_t rsm = (size_t)2 * i * sizeof(float);
            if (rsm > 150 * 1024) return fail(KQ_ESHAPE, "kq_quantize_layer: rows too long for the per-row grid search");
            static bool rattr = false;
            if (!rattr) {
                hipFuncSetAttribute(reinterpret_cast<const void*>(&row_grid_search_kernel),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
                rattr = true;
            }
            hipLaunchKernelGGL(row_grid_search_kernel, dim3((unsigned)o), dim3(256), rsm, st, W, i, ldw, L, scale, offset,
                               R, ldr, candidates);
        } else {
            hipLaunchKernelGGL(row_grid_kernel, dim3((unsigned)o), dim3(256), 0, st, W, i, ldw, L, scale, offset);
        }
        KQ_TRY(check_launch("row_grid"));
    }
    const size_t smem = (SW_B * SW_B + SW_B) * sizeof(float) + SW_ROWS * SW_B;
    static bool attr = false;
    if (!attr) {
#define KQ_SW_ATTR(g) \
        hipFuncSetAttribute(reinterpret_cast<const void*>(&sweep_block_kernel<g, false>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem); \
        hipFuncSetAttribute(reinterpret_cast<const void*>(&sweep_block_kernel<g, true>), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        KQ_SW_ATTR(0) KQ_SW_ATTR(16) KQ_SW_ATTR(32) KQ_SW_ATTR(64) KQ_SW_ATTR(128)
#undef KQ_SW_ATTR
        attr = true;
    }
    // row panels: the last ones may be shorter; every panel a multiple of the work-group's 16 rows
    int parts = o < SW_PANELS_FROM ? 1 : (int)(o / SW_PART_MIN_ROWS);
    parts = parts < 1 ? 1 : (parts > SW_PARTS ? SW_PARTS : parts);
    const int64_t per = ((o + parts - 1) / parts + SW_ROWS - 1) / SW_ROWS * SW_ROWS;
    const int64_t ng = group ? i / group : 1, wpr = i * bits / 32;
    auto part = [&](int64_t r0, hipStream_t q) {
        const int64_t rows = (o - r0) < per ? (o - r0) : per;
        return sweep_rows(W + r0 * ldw, rows, i, ldw, R, ldr, bits, group, candidates, codes + r0 * wpr,
                          scale + r0 * ng, offset + r0 * ng, row_loss ? row_loss + r0 : nullptr, E + r0 * SW_SB, smem,
                          q);
    };
    if (parts == 1) return part(0, st);
    std::lock_guard<std::mutex> lock(g_sp_mu);
    SweepPartQueues* pq = nullptr;
    KQ_TRY(sweep_part_queues(&pq));
    KQ_HIPS(hipEventRecord(pq->fork, st));
    int used = 0;
    for (int64_t r0 = per; r0 < o && used < SW_PARTS - 1; r0 += per, used++) {
        KQ_HIPS(hipStreamWaitEvent(pq->side[used], pq->fork, 0));
        KQ_TRY(part(r0, pq->side[used]));
        KQ_HIPS(hipEventRecord(pq->join[used], pq->side[used]));
    }
    KQ_TRY(part(0, st));
    for (int k = 0; k < used; k++) KQ_HIPS(hipStreamWaitEvent(st, pq->join[k], 0));
    return KQ_OK;
}
#undef KQ_HIPS

extern "C" kq_status kq_quantize_layer(float* W, int64_t o, int64_t i, int64_t ldw, const float* R, int64_t ldr, int bits,
                                       int group, int block, uint32_t* codes, float* scale, float* offset,
                                       float* row_loss, void* ws, size_t ws_bytes, kq_stream stream) {
    return kq_quantize_layer_search(W, o, i, ldw, R, ldr, bits, group, block, 0, codes, scale, offset, row_loss, ws,
                                    ws_bytes, stream);
}

// ----------------------------------------------------------------------------------- sensitivity
__global__ void sensitivity_kernel(const double* HX, int64_t i, int64_t ldh, const float* HG, int form, int64_t o,
                                   int64_t blk, double* score) {
    __shared__ double sx[256], sg[256];
    double ax = 0, ag = 0;
    for (int64_t r = threadIdx.x; r < i; r += 256) ax += HX[r * ldh + r];
    for (int64_t r = threadIdx.x; r < o; r += 256) {
        if (form == KQ_HG_DIAG) ag += (double)HG[r];
        else if (form == KQ_HG_FULL) ag += (double)HG[r * o + r];
        else ag += (double)HG[(r / blk) * blk * blk + (r % blk) * blk + (r % blk)];
    }
    sx[threadIdx.x] = ax;
    sg[threadIdx.x] = ag;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            sx[threadIdx.x] += sx[threadIdx.x + w];
            sg[threadIdx.x] += sg[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) *score = sx[0] * sg[0];
}

extern "C" kq_status kq_sensitivity(const double* HX, int64_t i, int64_t ldh, const float* HG, kq_hg_form form, int64_t o,
                                    int64_t blk, double* score, kq_stream stream) {
    if (!HX || !HG || !score) return fail(KQ_EINVAL, "kq_sensitivity: null pointer");
    if (i <= 0 || o <= 0 || ldh < i) return fail(KQ_ESHAPE, "kq_sensitivity: bad sizes");
    if (form != KQ_HG_DIAG && form != KQ_HG_BLOCK && form != KQ_HG_FULL) return fail(KQ_EINVAL, "kq_sensitivity: bad form");
    if (form == KQ_HG_BLOCK && (blk <= 0 || o % blk)) return fail(KQ_ESHAPE, "kq_sensitivity: bad block size");
    hipLaunchKernelGGL(sensitivity_kernel, dim3(1), dim3(256), 0, hs(stream), HX, i, ldh, HG, (int)form, o, blk, score);
    return check_launch("sensitivity");
}

// ------------------------------------------------------------------------------------ layer loss
__global__ void diff_kernel(const float* Q, const float* W2, int64_t o, int64_t i, int64_t ldw, float* D) {
    const int64_t tot = o * i;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < tot; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / i, c = e % i;
        D[e] = Q[r * ldw + c] - W2[r * ldw + c];
    }
}

// row_loss[r] = sum_c D[r][c] G[r][c] in fp64 (one work-group per row), then the total in row order.
__global__ void rowdot_kernel(const float* D, const float* G, int64_t i, double* out) {
    __shared__ double sp[256];
    const int64_t r = blockIdx.x;
    double a = 0;
    for (int64_t c = threadIdx.x; c < i; c += 256) a += (double)D[r * i + c] * (double)G[r * i + c];
    sp[threadIdx.x] = a;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sp[threadIdx.x] += sp[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[r] = sp[0];
}

__global__ void sum_rows_kernel(const double* rl, int64_t o, double* total) {
    __shared__ double sp[256];
    double a = 0;
    for (int64_t r = threadIdx.x; r < o; r += 256) a += rl[r];
    sp[threadIdx.x] = a;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sp[threadIdx.x] += sp[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *total = sp[0];
}

__global__ void narrow_kernel(const double* H, int64_t n, int64_t ldh, float* Hf) {
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < n * n; e += (int64_t)gridDim.x * 256)
        Hf[e] = (float)H[(e / n) * ldh + e % n];
}

size_t loss_ws(int64_t o, int64_t i) {
    Sizer z;
    z.take<float>((size_t)o * i);
    z.take<float>((size_t)o * i);
    z.take<double>((size_t)o);
    z.take<float>((size_t)i * i);
    return z.used;
}

extern "C" kq_status kq_layer_loss(const float* W2, const float* Q, int64_t o, int64_t i, int64_t ldw, const double* HX2,
                                   int64_t ldh, double* row_loss, double* loss, void* ws, size_t ws_bytes,
                                   kq_stream stream) {
    if (!W2 || !Q || !HX2 || !loss) return fail(KQ_EINVAL, "kq_layer_loss: null pointer");
    if (o <= 0 || i <= 0 || ldw < i || ldh < i) return fail(KQ_ESHAPE, "kq_layer_loss: bad sizes");
    if (!ws || ws_bytes < loss_ws(o, i)) return fail(KQ_EWORKSPACE, "kq_layer_loss: workspace too small");
    hipStream_t st = hs(stream);
    Arena ar(ws, ws_bytes);
    float* D = ar.take<float>((size_t)o * i);
    float* G = ar.take<float>((size_t)o * i);
    double* rl = ar.take<double>((size_t)o);
    float* Hf = ar.take<float>((size_t)i * i);
    if (row_loss) rl = row_loss;
    unsigned b = (unsigned)((o * i + 255) / 256 < 8192 ? (o * i + 255) / 256 : 8192);
    hipLaunchKernelGGL(diff_kernel, dim3(b), dim3(256), 0, st, Q, W2, o, i, ldw, D);
    KQ_TRY(check_launch("loss diff"));
    const unsigned hb = (unsigned)((i * i + 255) / 256 < 8192 ? (i * i + 255) / 256 : 8192);
    hipLaunchKernelGGL(narrow_kernel, dim3(hb), dim3(256), 0, st, HX2, i, ldh, Hf);
    KQ_TRY(check_launch("loss narrow"));
    GemmArgs<float> g = gemm_args<float>(o, i, i, D, i, Hf, i, G, i, 1.0f, 0.0f);
    KQ_TRY(gemm<float>(g, false, false, st));
    hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)o), dim3(256), 0, st, D, G, i, rl);
    KQ_TRY(check_launch("loss rowdot"));
    hipLaunchKernelGGL(sum_rows_kernel, dim3(1), dim3(256), 0, st, rl, o, loss);
    return check_launch("loss sum");
}
