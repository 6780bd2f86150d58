// nm_kernels.hpp -- kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nm {

// Philox key (the seed) and counter high half (the offset) of one launch.
struct NoiseKey {
    uint32_t k0, k1;      // seed lo, hi
    uint32_t off0, off1;  // offset lo, hi
};

// The noise key of a launch: the offset is the launch argument, or, when offset_dev is given,
// the 64-bit value it points to, read when the kernel runs (a graph replayed once per training
// step then samples fresh noise at each step).  The pointer is uniform: one scalar load.
__device__ __forceinline__ NoiseKey step_key(const NoiseKey& nk, const uint64_t* offset_dev) {
    if (!offset_dev) return nk;
    const uint64_t off = *offset_dev;
    return NoiseKey{nk.k0, nk.k1, (uint32_t)off, (uint32_t)(off >> 32)};
}

struct FwdArgs {
    const void* w;
    const float* logits;
    void* out;           // w_masked (wtype) or soft mask (fp32)
    int64_t groups;      // rows * cols / m
    float A, B;          // kappa*log2(e)/tau, 1/tau
    NoiseKey nk;
    // forward + pack in one pass (launch_forward_pack): the packed form of the hard mask
    void* values;
    uint32_t* indices;
    uint8_t* hard;       // may be null
    const uint64_t* offset_dev;  // may be null: the offset then comes from nk
};

// Workspace of the monitored forward: a 64-ary tree over the blocks of the launch, two 64-bit
// words (p_max sum, L1 sum) per node of every level above the blocks.  The words are zero
// between calls: each call's last arrival at a node sets that node back to zero.
struct MonitorLayout {
    int64_t blocks;   // blocks of the launch (the tree's leaves)
    int64_t words;    // words of all levels
    int64_t bytes;    // workspace size (at least 16)
    int frac_bits;    // F: the p_max sums are kept as integers in units of 2^-F
};
MonitorLayout monitor_layout(int n, int m, int64_t groups);

struct MonitorArgs {
    FwdArgs f;           // the forward's arguments (f.out = w_masked)
    const uint8_t* prev; // previous step's sampled candidates, may be null
    uint8_t* sample;     // this step's sampled candidates, may be null
    unsigned long long* tree;  // the tree's words, level by level
    double pscale, pinv;       // 2^F and 2^-F
    double* stats;       // [2]: sum of p_max, sum of l1
    float A0;            // kappa*log2(e)
};

struct BwdArgs {
    const void* w;
    const float* logits;
    const void* grad;    // null: regulariser only (launch_backward_wreg)
    float* dlogits;
    int64_t groups;
    float A, B, C;       // C = kappa/tau
    NoiseKey nk;
    float lam2;          // 2 * lambda of the weight regulariser (launch_backward_wreg only)
    const uint64_t* offset_dev;  // may be null: the offset then comes from nk
};

struct PackArgs {
    const void* w;
    const float* logits;
    void* values;
    uint32_t* indices;
    uint8_t* hard;       // may be null
    int64_t rows, gpr;   // groups per row
    int64_t words_per_row;
    int32_t aligned;         // rows of w, logits and values start on 16-byte boundaries
    int32_t hard_aligned;    // rows of hard start on 16-byte boundaries
};

struct UnpackArgs {
    const void* values;
    const uint32_t* indices;
    void* dense;
    int64_t rows, gpr, words_per_row;
    int32_t aligned;         // rows of values and dense start on 16-byte boundaries
};

struct PriorArgs {
    const void* w;
    float* logits;
    uint8_t* idx;        // may be null
    int64_t groups;
    float alpha;
};

struct NoiseArgs {
    uint32_t* words;
    int64_t slots;       // groups * K
    NoiseKey nk;
};

struct GumbelArgs {
    const uint32_t* words;
    float* h;
    int64_t count;
};

// Product with packed 2:4 bf16 weights: Y [tokens, out] = X [tokens, in] * W^T, W [out, in].
struct SpmmArgs {
    const uint16_t* values;    // [out, in/2] bf16 bits
    const uint32_t* indices;   // [out, in/32]
    const uint16_t* x;         // [tokens, in] bf16 bits
    void* y;                   // [tokens, out] fp32 (ytype 0) or bf16 (ytype 1)
    int64_t out, in, tokens;
    int64_t vstride, istride, xstride, ystride;  // row strides in elements
    int32_t ytype;
};

// Product plan: the kernel (tile 0: row streaming, 1-4 tokens; 16: the 16-row kernel; 64, 128
// or 256: the tile of W rows x tokens per block) and the parts its k range is split into.
struct SpmmPlan {
    int tile, parts;
};
SpmmPlan spmm_plan(int64_t out, int64_t in, int64_t tokens, int cus, bool allow_split);
int spmm_cus();  // compute units of the current device (256 if it cannot be asked)
// fp32 workspace the product needs on the current device: 4 * parts * tokens * out, or 0
int64_t spmm_workspace_bytes(int64_t out, int64_t in, int64_t tokens);
// ws may be null (no k split); otherwise ws_bytes of 16-byte aligned device memory
hipError_t launch_spmm24(const SpmmArgs& a, float* ws, int64_t ws_bytes, hipStream_t s);

hipError_t launch_forward(int n, int m, int wtype, const FwdArgs& a, bool soft_mask, hipStream_t s);
// 2:4 only, rows whose index bits fill whole words (cols/4 a multiple of 8)
hipError_t launch_forward_pack(int wtype, const FwdArgs& a, hipStream_t s);
hipError_t launch_backward(int n, int m, int wtype, const BwdArgs& a, hipStream_t s);
hipError_t launch_backward_wreg(int n, int m, int wtype, const BwdArgs& a, hipStream_t s);
hipError_t launch_pack(int n, int m, int wtype, const PackArgs& a, hipStream_t s);
hipError_t launch_unpack(int n, int m, int wtype, const UnpackArgs& a, hipStream_t s);
hipError_t launch_forward_monitor(int n, int m, int wtype, const MonitorArgs& a, hipStream_t s);
hipError_t launch_prior(int n, int m, int wtype, const PriorArgs& a, hipStream_t s);
hipError_t launch_debug_noise(const NoiseArgs& a, hipStream_t s);
hipError_t launch_debug_copy(const void* src, void* dst, int64_t vecs, hipStream_t s);
hipError_t launch_debug_gumbel(const GumbelArgs& a, hipStream_t s);
int groups_per_thread(int n, int m);

}  // namespace nm
