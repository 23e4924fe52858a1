// Error reporting, workspace sizing and version of the C ABI.
#include <cmath>
#include <cstdarg>
#include <cstring>
#include <vector>

#include "kq_internal.h"

size_t cholinv_ws(int64_t n);
size_t hg_sqrt_ws(kq_hg_form form, int64_t o, int64_t blk);
size_t hessian_ws(int64_t n, int64_t d, kq_dtype xdt);
size_t rotate_in_ws(int64_t o, int64_t i);
size_t rotate_out_ws(int64_t o, int64_t i, kq_hg_form form);
size_t unrotate_ws(int64_t o, int64_t i, kq_hg_form form);
size_t quantize_ws(int64_t o);
size_t loss_ws(int64_t o, int64_t i);
size_t matvec_ws(int64_t o, int64_t i, int64_t nt, kq_hg_form form);
size_t hg_lowrank_ws(int64_t n, int64_t o, int64_t k);
size_t kfac_loss_ws(int64_t o, int64_t i, kq_hg_form form, int64_t blk);
size_t cross_ws(int64_t n, int64_t d);
size_t drift_ws(int64_t o, int64_t i);

namespace kq {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

kq_status fail(kq_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kq_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KQ_EHIP, "%s: %s", what, hipGetErrorString(e));
    return KQ_OK;
}

}  // namespace kq

extern "C" const char* kq_last_error(void) { return kq::g_err; }

extern "C" const char* kq_strerror(kq_status s) {
    switch (s) {
        case KQ_OK: return "ok";
        case KQ_EINVAL: return "invalid argument";
        case KQ_ESHAPE: return "invalid or unsupported shape";
        case KQ_ENOTPD: return "matrix not positive definite";
        case KQ_EUNSUPPORTED: return "unsupported configuration";
        case KQ_EHIP: return "HIP error";
        case KQ_EWORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

extern "C" int kq_version(void) { return 1; }

extern "C" size_t kq_workspace_bytes(kq_op op, int64_t o, int64_t i, int64_t n, kq_dtype xdt, int bits, int group,
                                     kq_hg_form form, int64_t blk) {
    (void)bits;
    (void)group;
    switch (op) {
        case KQ_OP_HESSIAN: return hessian_ws(n, i, xdt);
        case KQ_OP_ROTATE_IN: return rotate_in_ws(o, i);
        case KQ_OP_HG_SQRT: return hg_sqrt_ws(form, o, blk);
        case KQ_OP_ROTATE_OUT: return rotate_out_ws(o, i, form);
        case KQ_OP_CHOLINV: return cholinv_ws(i);
        case KQ_OP_QUANTIZE: return quantize_ws(o);
        case KQ_OP_UNROTATE: return unrotate_ws(o, i, form);
        case KQ_OP_LOSS: return loss_ws(o, i);
        case KQ_OP_MATVEC: return matvec_ws(o, i, n, form);
        case KQ_OP_HG_LOWRANK: return hg_lowrank_ws(n, o, i);
        case KQ_OP_KFAC_LOSS: return kfac_loss_ws(o, i, form, blk);
        case KQ_OP_CROSS: return cross_ws(n, i);
        case KQ_OP_DRIFT: return drift_ws(o, i);
    }
    return 0;
}

extern "C" kq_status kq_allocate_bits(const double* scores, const int64_t* sizes, int64_t count, double budget,
                                      int bmin, int bmax, int32_t* bits) {
    if (!scores || !sizes || !bits) return kq::fail(KQ_EINVAL, "kq_allocate_bits: null pointer");
    if (count <= 0 || bmin < 1 || bmax < bmin || bmax > 16) return kq::fail(KQ_EINVAL, "kq_allocate_bits: bad arguments");
    double total = 0.0;
    for (int64_t l = 0; l < count; l++) {
        if (!(sizes[l] > 0) || !(scores[l] >= 0.0)) return kq::fail(KQ_EINVAL, "kq_allocate_bits: bad size or score");
        total += (double)sizes[l];
        bits[l] = bmin;
    }
    auto unit = [](int b) { const double r = std::ldexp(1.0, b) - 1.0; return 1.0 / (r * r); };
    const double cap = budget * total;
    double used = (double)bmin * total;
    for (;;) {
        int64_t best = -1;
        double best_gain = -1.0;
        for (int64_t l = 0; l < count; l++) {
            if (bits[l] >= bmax || used + (double)sizes[l] > cap) continue;
            const double gain = scores[l] * (unit(bits[l]) - unit(bits[l] + 1)) / (double)sizes[l];
            if (gain > best_gain) { best = l; best_gain = gain; }
        }
        if (best < 0) return KQ_OK;
        bits[best] += 1;
        used += (double)sizes[best];
    }
}
