// Float64 re-run of one (row, query head) whose bf16 output holds a NaN or an infinity.
//
// TensorFold pull request #1123, "What this changes", non-finite bullet and the review that
// follows it: a non-finite output re-runs its own row and head (never a whole block) in
// float64, so that non-finite outputs take float64's class. fp32 can disagree with float64
// in two ways the fast kernels cannot avoid: a weight float64 keeps (e^-200) underflows to
// 0 in fp32 next to an infinite value (0 * inf = NaN instead of inf), and in a shared MFMA
// tile a key a row does not see still meets that row's P = 0 (0 * inf). float64 can only be
// non-finite where fp32 is, so re-running exactly the non-finite (row, head)s is enough.
//
// One workgroup of D threads per (row, head), D = head dim: scores in float64 as plain
// dim-order sums of exact bf16 -> f64 products, max, exp, l = sum p, x_d = sum p v_d / l,
// keys outside [lo, last] (or in unselected blocks) never touched, sums started at +0, one
// rounding to bf16; a (row, head) with no key gives 0 / 0 = NaN.
#pragma once

#include "wa_common.h"

namespace wa {

// float64 -> bf16 bits, round to nearest even, signed underflow, overflow to inf: first to
// float32 with round-to-odd (truncate, then set the last bit if inexact), whose 16 spare
// bits make the second rounding, float32 -> bf16 nearest-even, exact.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
    if (x != x) return 0x7FC0u;
    float f = __double2float_rz(x);
    if ((double)f != x && !isinf(x)) f = __uint_as_float(__float_as_uint(f) | 1u);
    return f32_to_bf16_rne(f);
}

__device__ __forceinline__ bool bf16_nonfinite(uint16_t b) { return (b & 0x7F80u) == 0x7F80u; }

// Block-wide: does any of the D outputs of this (row, head) hold a NaN or an infinity?
template <int D>
__device__ __forceinline__ bool any_nonfinite(const uint16_t* out) {
    return __syncthreads_or(bf16_nonfinite(out[threadIdx.x]));
}

// The float64 re-run. q: the head's query row; kb, vb: key/value base of the key head
// (slot 0); sslot: slot stride; keys lo..last, key j in slot j mod ring; with a block mask
// (bm, words; nullptr: none) only the keys of selected 64-key blocks.
template <int D>
__device__ void rerun_f64(const uint16_t* q, const uint16_t* kb, const uint16_t* vb,
                          int64_t sslot, int ring, int lo, int last, float scale, uint16_t* out,
                          const uint32_t* bm = nullptr, int words = 0) {
    auto sel = [&](int j) { return bm == nullptr || block_selected(bm, words, j / kSparseBlock); };
    __shared__ double qs[D];
    __shared__ double ps[D];
    __shared__ double red[D];
    // threads D .. blockDim - 1 (a workgroup wider than D) take part in the barriers only
    const int t = threadIdx.x;
    const bool act = t < D;
    if (act) qs[t] = (double)bf16_to_f32(q[t]);
    __syncthreads();
    const double c = (double)scale;
    auto score = [&](int j) {
        const uint16_t* kr = kb + (int64_t)(j % ring) * sslot;
        double s = 0.0;
        for (int e = 0; e < D; ++e) s += qs[e] * (double)bf16_to_f32(kr[e]);
        return c * s;
    };
    // pass 1: the maximum score (a NaN score reaches the output through its weight)
    double mx = -INFINITY;
    if (act)
        for (int j = lo + t; j <= last; j += D)
            if (sel(j)) mx = fmax(mx, score(j));
    if (act) red[t] = mx;
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
        if (t < w) red[t] = fmax(red[t], red[t + w]);
        __syncthreads();
    }
    const double m = red[0];
    __syncthreads();
    // pass 2: weights of D keys at a time, then every thread folds its dim over them
    double l = 0.0, x = 0.0;
    for (int base = lo; base <= last; base += D) {
        const int j = base + t;
        double p = 0.0;
        if (act && j <= last && sel(j)) p = exp(score(j) - m);
        if (act) ps[t] = p;
        l += p;
        __syncthreads();
        const int nk = act ? min(D, last - base + 1) : 0;
        for (int i = 0; i < nk; ++i) {
            const int jj = base + i;
            if (sel(jj)) x += ps[i] * (double)bf16_to_f32(vb[(int64_t)(jj % ring) * sslot + t]);
        }
        __syncthreads();
    }
    if (act) red[t] = l;
    __syncthreads();
    for (int w = D / 2; w > 0; w >>= 1) {
        if (t < w) red[t] = red[t] + red[t + w];
        __syncthreads();
    }
    const double lsum = 0.0 + red[0];
    if (act) out[t] = (uint16_t)f64_to_bf16_rne((0.0 + x) / lsum);
}

}  // namespace wa
