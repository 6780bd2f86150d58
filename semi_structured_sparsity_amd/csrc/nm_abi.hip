// nm_abi.hip -- the extern "C" entry points declared in include/nm_mask.h.
//
// Each entry point validates its arguments on the host, derives the fp32 launch constants
// (A = kappa*log2(e)/tau, B = 1/tau, C = kappa/tau, computed in double and rounded once), and
// launches one kernel on the caller's stream.  No HIP call is made before validation passes,
// so every argument error is reported without touching the device.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/nm_mask.h"
#include "nm_kernels.hpp"

namespace {

bool supported_nm(int32_t n, int32_t m) { return (m == 4 || m == 8) && n >= 1 && n < m; }

int32_t binom_host(int32_t m, int32_t n) {
    int64_t c = 1;
    for (int32_t i = 0; i < n; ++i) c = c * (m - i) / (i + 1);
    return (int32_t)c;
}

int32_t index_bits(int32_t m) { return m <= 4 ? 2 : 3; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest flat thread count a launch may need: the grid's x dimension is at most 2^31 - 1
// blocks of 256 threads.
constexpr int64_t kMaxThreads = ((int64_t)1 << 31) * 256 - 256;

// Shape checks shared by all entry points; on success *groups = rows*cols/m and *K = C(m,n).
nm_status check_shape(const nm_shape* s, int64_t* groups, int32_t* K) {
    if (!s) return NM_EINVAL;
    if (s->rows < 0 || s->cols < 0) return NM_EINVAL;
    if (!supported_nm(s->n, s->m)) return NM_EUNSUPPORTED;
    if (s->wtype != NM_F32 && s->wtype != NM_BF16) return NM_EUNSUPPORTED;
    if (s->cols % s->m != 0) return NM_EINVAL;
    *K = binom_host(s->m, s->n);
    if (s->rows > 0 && s->cols > INT64_MAX / 16 / s->rows) return NM_EINVAL;
    const int64_t g = s->rows * (s->cols / s->m);
    if (g > INT64_MAX / 8 / *K) return NM_EINVAL;  // logit byte offsets stay in int64
    if (g > kMaxThreads) return NM_EINVAL;         // one group or more per thread
    *groups = g;
    return NM_OK;
}

nm_status check_sample(const nm_sample* smp, float* A, float* B, float* C) {
    if (!smp) return NM_EINVAL;
    const double kappa = smp->kappa, tau = smp->tau;
    if (!(isfinite(kappa) && kappa >= 0.0)) return NM_EINVAL;
    if (!(isfinite(tau) && tau > 0.0)) return NM_EINVAL;
    const double log2e = 1.4426950408889634074;
    *A = (float)(kappa * log2e / tau);
    *B = (float)(1.0 / tau);
    *C = (float)(kappa / tau);
    if (!isfinite(*A) || !isfinite(*B) || !isfinite(*C)) return NM_EINVAL;
    return NM_OK;
}

nm::NoiseKey noise_key(const nm_sample* smp) {
    return nm::NoiseKey{(uint32_t)smp->seed, (uint32_t)(smp->seed >> 32), (uint32_t)smp->offset,
                        (uint32_t)(smp->offset >> 32)};
}

nm::MonitorArgs monitor_args(const nm_shape* shape, const nm_sample* sample, const void* w, const float* logits,
                             void* w_masked, const uint8_t* prev_sample, uint8_t* sample_idx, double* stats,
                             void* workspace, int64_t groups, float A, float B) {
    const nm::MonitorLayout L = nm::monitor_layout(shape->n, shape->m, groups);
    const float A0 = (float)((double)sample->kappa * 1.4426950408889634074);
    return nm::MonitorArgs{nm::FwdArgs{w, logits, w_masked, groups, A, B, noise_key(sample)},
                           prev_sample,
                           sample_idx,
                           static_cast<unsigned long long*>(workspace),
                           ldexp(1.0, L.frac_bits),
                           ldexp(1.0, -L.frac_bits),
                           stats,
                           A0};
}

nm_status launched(hipError_t e) { return e == hipSuccess ? NM_OK : NM_EHIP; }

}  // namespace

// ------------------------------------------------------------------------------------------
// nm_mask_forward_monitor_static: the monitored forward with its per-block partial sums in a
// fixed device array instead of a caller workspace.  In host code the array's name only stands
// for the symbol: its device address (one per GPU, each GPU holds its own copy) is looked up
// with hipGetSymbolAddress once per device, with that device current, and only that address is
// handed to the kernels.

static __device__ __align__(256) unsigned char scratch[NM_MONITOR_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until looked up

nm_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return NM_EHIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return NM_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NM_OK;
}

}  // namespace

extern "C" {

int32_t nm_num_candidates(int32_t n, int32_t m) { return supported_nm(n, m) ? binom_host(m, n) : -1; }

nm_status nm_candidate_table(int32_t n, int32_t m, uint8_t* out_bits) {
    if (!supported_nm(n, m)) return NM_EUNSUPPORTED;
    if (!out_bits) return NM_EINVAL;
    // lexicographic order of the ascending kept-position lists
    int32_t k = 0;
    for (int32_t r = (1 << m) - 1; r >= 0; --r) {
        if (__builtin_popcount((unsigned)r) != n) continue;
        uint32_t bits = 0;
        for (int32_t j = 0; j < m; ++j)
            if (r >> (m - 1 - j) & 1) bits |= 1u << j;
        out_bits[k++] = (uint8_t)bits;
    }
    return NM_OK;
}

int64_t nm_packed_value_elems(const nm_shape* s) {
    int64_t g;
    int32_t K;
    if (check_shape(s, &g, &K) != NM_OK) return -1;
    return g * s->n;
}

int64_t nm_index_words_per_row(const nm_shape* s) {
    int64_t g;
    int32_t K;
    if (check_shape(s, &g, &K) != NM_OK) return -1;
    const int64_t bits = s->cols / s->m * s->n * index_bits(s->m);
    return (bits + 31) / 32;
}

int64_t nm_packed_index_words(const nm_shape* s) {
    const int64_t wpr = nm_index_words_per_row(s);
    return wpr < 0 ? -1 : wpr * s->rows;
}

const char* nm_status_str(int32_t st) {
    switch (st) {
    case NM_OK: return "ok";
    case NM_EINVAL: return "invalid argument";
    case NM_EALIGN: return "pointer not 16-byte aligned";
    case NM_EUNSUPPORTED: return "unsupported n:m or element type";
    case NM_EHIP: return "HIP launch failed";
    case NM_ESCRATCH: return "shape needs more scratch memory than the static array holds";
    default: return "unknown status";
    }
}

nm_status nm_mask_forward(const nm_shape* shape, const nm_sample* sample, const void* w,
                          const float* logits, void* w_masked, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !w_masked) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(w_masked)) return NM_EALIGN;
    nm::FwdArgs a{w, logits, w_masked, groups, A, B, noise_key(sample)};
    return launched(nm::launch_forward(shape->n, shape->m, shape->wtype, a, false, (hipStream_t)stream));
}

// The monitored forward with its partial sums in the static array (see `scratch` above).
nm_status nm_mask_forward_monitor_static(const nm_shape* shape, const nm_sample* sample, const void* w,
                                         const float* logits, void* w_masked, const uint8_t* prev_sample,
                                         uint8_t* sample_idx, double* stats, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !w_masked || !stats) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(w_masked) || !aligned16(stats)) return NM_EALIGN;
    if (nm::monitor_layout(shape->n, shape->m, groups).bytes > NM_MONITOR_SCRATCH_BYTES) return NM_ESCRATCH;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != NM_OK) return st;
    const nm::MonitorArgs a = monitor_args(shape, sample, w, logits, w_masked, prev_sample, sample_idx, stats, ws,
                                           groups, A, B);
    return launched(nm::launch_forward_monitor(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

int64_t nm_monitor_workspace_bytes(const nm_shape* shape) {
    int64_t groups;
    int32_t K;
    if (check_shape(shape, &groups, &K) != NM_OK) return -1;
    return nm::monitor_layout(shape->n, shape->m, groups).bytes;
}

nm_status nm_mask_forward_offset_dev(const nm_shape* shape, const nm_sample* sample,
                                     const uint64_t* offset_dev, const void* w, const float* logits,
                                     void* w_masked, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!offset_dev || !w || !logits || !w_masked) return NM_EINVAL;
    if (((uintptr_t)offset_dev & 7u) != 0 || !aligned16(w) || !aligned16(logits) || !aligned16(w_masked))
        return NM_EALIGN;
    nm::FwdArgs a{w, logits, w_masked, groups, A, B, noise_key(sample), nullptr, nullptr, nullptr, offset_dev};
    return launched(nm::launch_forward(shape->n, shape->m, shape->wtype, a, false, (hipStream_t)stream));
}

nm_status nm_mask_backward_offset_dev(const nm_shape* shape, const nm_sample* sample,
                                      const uint64_t* offset_dev, const void* w, const float* logits,
                                      const void* grad_w_masked, float* grad_logits, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!offset_dev || !w || !logits || !grad_w_masked || !grad_logits) return NM_EINVAL;
    if (((uintptr_t)offset_dev & 7u) != 0 || !aligned16(w) || !aligned16(logits) ||
        !aligned16(grad_w_masked) || !aligned16(grad_logits))
        return NM_EALIGN;
    nm::BwdArgs a{w, logits, grad_w_masked, grad_logits, groups, A, B, C, noise_key(sample), 0.0f, offset_dev};
    return launched(nm::launch_backward(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_mask_forward_monitor(const nm_shape* shape, const nm_sample* sample, const void* w,
                                  const float* logits, void* w_masked, const uint8_t* prev_sample,
                                  uint8_t* sample_idx, double* stats, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !w_masked || !stats || !workspace) return NM_EINVAL;
    if (workspace_bytes < nm::monitor_layout(shape->n, shape->m, groups).bytes) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(w_masked) || !aligned16(stats) ||
        !aligned16(workspace))
        return NM_EALIGN;
    const nm::MonitorArgs a = monitor_args(shape, sample, w, logits, w_masked, prev_sample, sample_idx, stats,
                                           workspace, groups, A, B);
    return launched(nm::launch_forward_monitor(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_debug_soft_mask(const nm_shape* shape, const nm_sample* sample, const float* logits,
                             float* soft_mask, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!logits || !soft_mask) return NM_EINVAL;
    if (!aligned16(logits) || !aligned16(soft_mask)) return NM_EALIGN;
    nm::FwdArgs a{nullptr, logits, soft_mask, groups, A, B, noise_key(sample)};
    return launched(nm::launch_forward(shape->n, shape->m, shape->wtype, a, true, (hipStream_t)stream));
}

nm_status nm_mask_backward(const nm_shape* shape, const nm_sample* sample, const void* w,
                           const float* logits, const void* grad_w_masked, float* grad_logits,
                           void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !grad_w_masked || !grad_logits) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(grad_w_masked) || !aligned16(grad_logits))
        return NM_EALIGN;
    nm::BwdArgs a{w, logits, grad_w_masked, grad_logits, groups, A, B, C, noise_key(sample)};
    return launched(nm::launch_backward(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_mask_backward_wreg(const nm_shape* shape, const nm_sample* sample, float lambda,
                                const void* w, const float* logits, const void* grad_w_masked,
                                float* grad_logits, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    const float lam2 = 2.0f * lambda;
    if (!isfinite(lambda) || !isfinite(lam2)) return NM_EINVAL;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !grad_logits) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(grad_logits) ||
        (grad_w_masked && !aligned16(grad_w_masked)))
        return NM_EALIGN;
    nm::BwdArgs a{w, logits, grad_w_masked, grad_logits, groups, A, B, C, noise_key(sample), lam2};
    return launched(nm::launch_backward_wreg(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_mask_harden_pack(const nm_shape* shape, const void* w, const float* logits, void* values,
                              uint32_t* indices, uint8_t* hard_idx, void* stream) {
    int64_t groups;
    int32_t K;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !values || !indices) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(values) || !aligned16(indices) ||
        (hard_idx && !aligned16(hard_idx)))
        return NM_EALIGN;
    const int64_t gpr = shape->cols / shape->m, wb = shape->wtype == NM_BF16 ? 2 : 4;
    const bool aligned = (shape->cols * wb) % 16 == 0 && (gpr * K * 4) % 16 == 0 &&
                         (gpr * shape->n * wb) % 16 == 0;
    nm::PackArgs a{w, logits, values, indices, hard_idx, shape->rows, gpr,
                   nm_index_words_per_row(shape), aligned ? 1 : 0, gpr % 16 == 0 ? 1 : 0};
    return launched(nm::launch_pack(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_mask_forward_pack(const nm_shape* shape, const nm_sample* sample, const void* w,
                               const float* logits, void* w_masked, void* values, uint32_t* indices,
                               uint8_t* hard_idx, void* stream) {
    int64_t groups;
    int32_t K;
    float A, B, C;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if ((st = check_sample(sample, &A, &B, &C)) != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!w || !logits || !w_masked || !values || !indices) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits) || !aligned16(w_masked) || !aligned16(values) ||
        !aligned16(indices) || (hard_idx && !aligned16(hard_idx)))
        return NM_EALIGN;
    const int64_t gpr = shape->cols / shape->m;
    if (shape->n == 2 && shape->m == 4 && gpr % 8 == 0) {
        nm::FwdArgs a{w, logits, w_masked, groups, A, B, noise_key(sample), values, indices, hard_idx};
        return launched(nm::launch_forward_pack(shape->wtype, a, (hipStream_t)stream));
    }
    // other shapes: the two passes one after the other, with the same results
    if ((st = nm_mask_forward(shape, sample, w, logits, w_masked, stream)) != NM_OK) return st;
    return nm_mask_harden_pack(shape, w, logits, values, indices, hard_idx, stream);
}

nm_status nm_unpack(const nm_shape* shape, const void* values, const uint32_t* indices, void* w_dense,
                    void* stream) {
    int64_t groups;
    int32_t K;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if (groups == 0) return NM_OK;
    if (!values || !indices || !w_dense) return NM_EINVAL;
    if (!aligned16(values) || !aligned16(indices) || !aligned16(w_dense)) return NM_EALIGN;
    const int64_t gpr = shape->cols / shape->m, wb = shape->wtype == NM_BF16 ? 2 : 4;
    const bool aligned = (shape->cols * wb) % 16 == 0 && (gpr * shape->n * wb) % 16 == 0;
    nm::UnpackArgs a{values, indices, w_dense, shape->rows, gpr, nm_index_words_per_row(shape),
                     aligned ? 1 : 0};
    return launched(nm::launch_unpack(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

nm_status nm_prior_init(const nm_shape* shape, float alpha, const void* w, float* logits,
                        uint8_t* prior_idx, void* stream) {
    int64_t groups;
    int32_t K;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if (!isfinite(alpha)) return NM_EINVAL;
    if (groups == 0) return NM_OK;
    if (!w || !logits) return NM_EINVAL;
    if (!aligned16(w) || !aligned16(logits)) return NM_EALIGN;
    nm::PriorArgs a{w, logits, prior_idx, groups, alpha};
    return launched(nm::launch_prior(shape->n, shape->m, shape->wtype, a, (hipStream_t)stream));
}

namespace {

// Size checks of the product without pointers: NM_OK and *empty when nothing is to be done.
nm_status spmm_sizes(const nm_shape* w_shape, int64_t tokens, bool* empty) {
    int64_t groups;
    int32_t K;
    const nm_status st = check_shape(w_shape, &groups, &K);
    if (st != NM_OK) return st;
    if (tokens < 0) return NM_EINVAL;
    if (w_shape->n != 2 || w_shape->m != 4 || w_shape->wtype != NM_BF16) return NM_EUNSUPPORTED;
    const int64_t out = w_shape->rows, in = w_shape->cols;
    *empty = out == 0 || tokens == 0;
    if (*empty) return NM_OK;
    if (in == 0 || in % 64 != 0 || out % 4 != 0) return NM_EUNSUPPORTED;
    if (tokens > INT64_MAX / 4 / (in > out ? in : out)) return NM_EINVAL;
    return NM_OK;
}

// Checks of the product's sizes and pointers shared by its two entry points; on success *a is
// filled (and the call launches nothing if *empty).
nm_status spmm_args(const nm_shape* w_shape, const void* values, const uint32_t* indices, const void* x,
                    int64_t tokens, void* y, int32_t ytype, nm::SpmmArgs* a, bool* empty) {
    nm_status st = spmm_sizes(w_shape, tokens, empty);
    if (st != NM_OK) return st;
    if (ytype != NM_F32 && ytype != NM_BF16) return NM_EINVAL;
    if (*empty) return NM_OK;
    const int64_t out = w_shape->rows, in = w_shape->cols;
    if (((out + 255) / 256 + 8) * ((tokens + 255) / 256 + 4) > (int64_t)INT32_MAX) return NM_EINVAL;  // one block per tile
    if (!values || !indices || !x || !y) return NM_EINVAL;
    if (!aligned16(values) || !aligned16(indices) || !aligned16(x) || !aligned16(y)) return NM_EALIGN;
    *a = nm::SpmmArgs{static_cast<const uint16_t*>(values), indices, static_cast<const uint16_t*>(x), y,
                      out, in, tokens, in / 2, in / 32, in, out, ytype == NM_F32 ? 0 : 1};
    return NM_OK;
}

}  // namespace

nm_status nm_sparse_matmul(const nm_shape* w_shape, const void* values, const uint32_t* indices,
                           const void* x, int64_t tokens, void* y, int32_t ytype, void* stream) {
    nm::SpmmArgs a;
    bool empty = false;
    const nm_status st = spmm_args(w_shape, values, indices, x, tokens, y, ytype, &a, &empty);
    if (st != NM_OK || empty) return st;
    return launched(nm::launch_spmm24(a, nullptr, 0, (hipStream_t)stream));
}

int64_t nm_sparse_matmul_workspace_bytes(const nm_shape* w_shape, int64_t tokens) {
    bool empty = false;
    if (spmm_sizes(w_shape, tokens, &empty) != NM_OK) return -1;
    return empty ? 0 : nm::spmm_workspace_bytes(w_shape->rows, w_shape->cols, tokens);
}

nm_status nm_sparse_matmul_plan(const nm_shape* w_shape, int64_t tokens, int32_t with_workspace, int32_t* tile,
                                int32_t* parts) {
    if (!tile || !parts) return NM_EINVAL;
    bool empty = false;
    const nm_status st = spmm_sizes(w_shape, tokens, &empty);
    if (st != NM_OK) return st;
    if (empty) {
        *tile = -1;
        *parts = 0;
        return NM_OK;
    }
    const nm::SpmmPlan pl = nm::spmm_plan(w_shape->rows, w_shape->cols, tokens, nm::spmm_cus(), with_workspace != 0);
    *tile = pl.tile;
    *parts = pl.parts;
    return NM_OK;
}

nm_status nm_sparse_matmul_ws(const nm_shape* w_shape, const void* values, const uint32_t* indices,
                              const void* x, int64_t tokens, void* y, int32_t ytype, void* workspace,
                              int64_t workspace_bytes, void* stream) {
    nm::SpmmArgs a;
    bool empty = false;
    const nm_status st = spmm_args(w_shape, values, indices, x, tokens, y, ytype, &a, &empty);
    if (st != NM_OK || empty) return st;
    const int64_t need = nm::spmm_workspace_bytes(a.out, a.in, tokens);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return NM_EINVAL;
        if (!aligned16(workspace)) return NM_EALIGN;
    }
    return launched(nm::launch_spmm24(a, need > 0 ? static_cast<float*>(workspace) : nullptr, workspace_bytes,
                                      (hipStream_t)stream));
}

nm_status nm_debug_noise(const nm_shape* shape, const nm_sample* sample, uint32_t* words, void* stream) {
    int64_t groups;
    int32_t K;
    nm_status st = check_shape(shape, &groups, &K);
    if (st != NM_OK) return st;
    if (!sample) return NM_EINVAL;
    if (groups == 0) return NM_OK;
    if (!words) return NM_EINVAL;
    if (!aligned16(words)) return NM_EALIGN;
    nm::NoiseArgs a{words, groups * K, noise_key(sample)};
    return launched(nm::launch_debug_noise(a, (hipStream_t)stream));
}

nm_status nm_debug_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0 || bytes / 16 > kMaxThreads) return NM_EINVAL;
    if (bytes == 0) return NM_OK;
    if (!src || !dst) return NM_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return NM_EALIGN;
    return launched(nm::launch_debug_copy(src, dst, bytes / 16, (hipStream_t)stream));
}

nm_status nm_debug_gumbel_log2(const uint32_t* words, float* h, int64_t count, void* stream) {
    if (count < 0 || count > kMaxThreads) return NM_EINVAL;
    if (count == 0) return NM_OK;
    if (!words || !h) return NM_EINVAL;
    if (!aligned16(words) || !aligned16(h)) return NM_EALIGN;
    nm::GumbelArgs a{words, h, count};
    return launched(nm::launch_debug_gumbel(a, (hipStream_t)stream));
}

}  // extern "C"
