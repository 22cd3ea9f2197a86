// Split-KV decode for windowed GQA attention on gfx950: chunk partials and the ordered merge.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Decode bullet. Keys are split into 256-key chunks at absolute key
// positions; one workgroup per (row, key head, chunk) computes fp32 scores for the G query
// heads of the key head, the chunk max m_c, p = expf(s - m_c), l_c = sum p and
// o_c = sum p v with p kept in fp32; a second kernel merges the chunks of a row in chunk
// order. Chunks holding none of a row's keys are never launched into the merge, so the
// split depends only on key positions.
//
// gfx950 mapping (wave64):
//   scores  v_mfma_f32_16x16x32_bf16 with the chunk's keys on M and the group's query heads
//           on N (up to 16); bf16 x bf16 products are exact in fp32, the sums are fp32. K
//           rows go straight from HBM/L2 into the MFMA operand registers (128 contiguous
//           bytes per lane); each wave scores 64 keys.
//   softmax one wave per query head: 4 keys per lane, wave butterflies for max and sum.
//   P.V     fp32 on the VALU: NRUN key runs of 256/NRUN consecutive keys; D/8 lanes per
//           run, 8 dims a lane; each run is an fma chain in key order; runs are summed in
//           run order through LDS.
//   grid    one workgroup per (row, key head, chunk), ordered so that each XCD works on the
//           rows of a few key heads and their rings stay in its L2.
#include "wa_common.h"
#include "rerun_f64.h"

// Tuning switches (defaults chosen by measurement on MI355X):
//   WA_DECODE_ORDER   0: XCD-grouped (key head, row, chunk) order; 1: (row, chunk, key head)
//   WA_DECODE_VEARLY  1: issue the V loads before the score MFMAs wait for K
//   WA_DECODE_KT      16-key K tiles in flight together per wave (4 tiles per wave)
//   WA_DECODE_VB      batches the V loads of a key run are split into (register budget)
#ifndef WA_DECODE_ORDER
#define WA_DECODE_ORDER 0
#endif
#ifndef WA_DECODE_VEARLY
#define WA_DECODE_VEARLY 0
#endif
#ifndef WA_DECODE_KT
#define WA_DECODE_KT 2
#endif
#ifndef WA_DECODE_VB
#define WA_DECODE_VB 2
#endif

namespace wa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    f[0] = lo_bf16(w.x); f[1] = hi_bf16(w.x);
    f[2] = lo_bf16(w.y); f[3] = hi_bf16(w.y);
    f[4] = lo_bf16(w.z); f[5] = hi_bf16(w.z);
    f[6] = lo_bf16(w.w); f[7] = hi_bf16(w.w);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, xor_shfl(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += xor_shfl(x, m);
    return x;
}

// Row bounds shared by the partial kernel and the merge: the same clamps on both sides.
struct RowSpan {
    int pos, lo, c_lo, c_hi;
};

__device__ __forceinline__ RowSpan row_span(const int32_t* pos_of_row, int r, int max_pos,
                                            int window) {
    RowSpan s;
    int p = pos_of_row[r];
    p = p < 0 ? 0 : (p > max_pos ? max_pos : p);
    s.pos = p;
    s.lo = window > 0 ? max(0, p - window + 1) : 0;
    s.c_lo = s.lo / kChunk;
    s.c_hi = p / kChunk;
    return s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
union Pack8 {
    bf16x8 v;
    uint4 u;
};

// Linear workgroup id -> logical id such that each XCD (8 on MI355X, ids dealt out
// round-robin) runs a contiguous range of logical ids.
__device__ __forceinline__ int xcd_logical(int L, int total) {
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, extra = total & 7;
    return (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
}

template <int D, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_part_kernel(DecodeArgs a) {
    constexpr int KSTEPS = D / 32;       // MFMA k-steps over the head dim
    constexpr int LPK = D / 8;           // lanes per key run row in P.V (8 dims a lane)
    constexpr int NRUN = kThreads / LPK; // P.V key runs
    constexpr int RUNLEN = kChunk / NRUN;
    constexpr int GH = GMAX < 4 ? GMAX : 4;   // heads per LDS reduction pass
    constexpr int NB = WA_DECODE_VB;          // V prefetch batches per run (register budget)
    constexpr int BL = RUNLEN / NB;           // keys per batch

    __shared__ float sc[GMAX][kChunk];
    __shared__ float red[NRUN][GH][D];

#if WA_DECODE_ORDER == 0
    // logical order (key head, row, chunk slot): an XCD holds the rows of a few key heads
    const int total = gridDim.x;
    const int logical = xcd_logical(blockIdx.x, total);
    const int per_g = a.rows * a.C;
    const int g = logical / per_g;
    const int r = (logical % per_g) / a.C;
    const int kslot = logical % a.C;
#else
    // order (row, chunk slot, key head), key heads adjacent, no XCD remap
    const int logical = blockIdx.x;
    const int g = logical % a.hkv;
    const int kslot = (logical / a.hkv) % a.C;
    const int r = logical / (a.hkv * a.C);
#endif

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = a.hq / a.hkv;

    const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
    const int c = rs.c_lo + kslot;
    if (c > rs.c_hi) return;
    int t = a.stream_of_row[r];
    t = t < 0 ? 0 : (t >= a.streams ? a.streams - 1 : t);
    const int j0 = max(rs.lo, c * kChunk);
    const int j1 = min(rs.pos, c * kChunk + kChunk - 1);
    const int nk = j1 - j0 + 1;           // visible keys in this chunk, >= 1
    const int kbase = j0 - c * kChunk;    // chunk-relative index of the first visible key

    const uint16_t* kbase_ptr = a.k + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
    const uint16_t* vbase_ptr = a.v + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
    // ring slot of chunk-relative key kk: one modulo per workgroup, then a conditional
    // subtraction (a ring of at least one chunk wraps at most once inside a chunk)
    const int sb = (c * kChunk) % a.ring;
    const bool big_ring = a.ring >= kChunk;
    auto slot_of = [&](int kk) {
        const int s = sb + kk;
        return big_ring ? (s >= a.ring ? s - a.ring : s) : s % a.ring;
    };

    // ---- start this thread's V loads for P.V now, so their latency hides behind the
    // softmax: run `run` covers chunk keys run*RUNLEN .. +RUNLEN-1, 8 dims per lane
    const int run = tid / LPK;
    const int dl = tid % LPK;
    const int r0 = max(run * RUNLEN, kbase);
    const int r1 = min(run * RUNLEN + RUNLEN, kbase + nk);
    uint4 vr[BL];
    // whole-run loads: every key of a run that holds a visible key is fetched (its slot is
    // inside the ring), keys outside [r0, r1) are skipped in the sums below
    auto load_batch = [&](int b) {
        if (r0 < r1) {
#pragma unroll
            for (int i = 0; i < BL; ++i) {
                const int slot = slot_of(run * RUNLEN + b * BL + i);
                vr[i] = *reinterpret_cast<const uint4*>(vbase_ptr + (int64_t)slot * a.kv_sslot + dl * 8);
            }
        }
    };
#if WA_DECODE_VEARLY
    load_batch(0);
#endif

    // ---- scores on MFMA: S^T (16 keys x 16 heads) = K (16 x 32 dims) . q^T, fp32 accumulate.
    // bf16 x bf16 products are exact in fp32; only the sum is rounded. Lane l feeds key
    // l % 16 of the tile and dims 32*ks + 8*(l/16) + 0..7 at k-step ks (the four lanes of a
    // key read 64 contiguous bytes per instruction; the q operand uses the same dims); the
    // result lane holds head l % 16 and keys 4*(l/16) + 0..3 of the tile. Wave w scores
    // chunk keys 64w .. 64w+63.
    {
        const int n = lane & 15, kg = lane >> 4;
        Pack8 qb[KSTEPS];
        // lanes of heads >= G read head G-1 and their scores are never used
        const uint16_t* qp = a.q + (int64_t)r * a.q_srow + (int64_t)(g * G + min(n, G - 1)) * a.q_shead + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qb[ks].u = *reinterpret_cast<const uint4*>(qp + 32 * ks);
        const int kw0 = 64 * wave;                        // chunk-relative first key of the wave
        if (kw0 < kbase + nk && kw0 + 63 >= kbase) {
            constexpr int KT = WA_DECODE_KT;              // 16-key tiles whose K is in flight together
#pragma unroll
            for (int u0 = 0; u0 < 4; u0 += KT) {
                Pack8 kb[KT][KSTEPS];
#pragma unroll
                for (int u = 0; u < KT; ++u) {
                    const int slot = slot_of(kw0 + 16 * (u0 + u) + n);
                    const uint16_t* kp = kbase_ptr + (int64_t)slot * a.kv_sslot + 8 * kg;
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks) kb[u][ks].u = *reinterpret_cast<const uint4*>(kp + 32 * ks);
                }
#pragma unroll
                for (int u = 0; u < KT; ++u) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KSTEPS; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[u][ks].v, qb[ks].v, acc, 0, 0, 0);
                    if (n < G) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int kk = kw0 + 16 * (u0 + u) + 4 * kg + i;
                            if (kk >= kbase && kk < kbase + nk) sc[n][kk] = a.scale * acc[i];
                        }
                    }
                }
            }
        }
    }

#if !WA_DECODE_VEARLY
    load_batch(0);
#endif
    __syncthreads();
    // ---- chunk softmax: m_c, p = expf(s - m_c), l_c, one wave per head ----
    for (int h = wave; h < G; h += 4) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = lane + 64 * i;
            if (kk < nk) mx = fmaxf(mx, sc[h][kbase + kk]);
        }
        mx = wave_max(mx);
        const float mu = (mx == -INFINITY) ? 0.f : mx;   // all scores -inf: weights 0
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = lane + 64 * i;
            if (kk < nk) {
                const float p = expf(sc[h][kbase + kk] - mu);
                sc[h][kbase + kk] = p;
                sum += p;
            }
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            const int64_t pi = ((int64_t)r * a.hq + g * G + h) * a.C + kslot;
            a.m[pi] = mx;
            a.l[pi] = sum;
        }
    }
    __syncthreads();

    // ---- P.V: NRUN runs of consecutive keys, fma chains in key order ----
    float acc[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    const bool run_full = r0 == run * RUNLEN && r1 == run * RUNLEN + RUNLEN;
    auto fold_key = [&](int i, int kk) {
        const uint4 w = vr[i];
        const float vf[8] = {lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y),
                             lo_bf16(w.z), hi_bf16(w.z), lo_bf16(w.w), hi_bf16(w.w)};
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h < G) {
                const float p = sc[h][kk];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (b > 0) load_batch(b);
        if (run_full) {
#pragma unroll
            for (int i = 0; i < BL; ++i) fold_key(i, run * RUNLEN + b * BL + i);
        } else if (r0 < r1) {
#pragma unroll
            for (int i = 0; i < BL; ++i) {
                const int kk = run * RUNLEN + b * BL + i;
                if (kk >= r0 && kk < r1) fold_key(i, kk);
            }
        }
    }
    // sum the runs in run order, GH heads per pass
#pragma unroll
    for (int hp = 0; hp < GMAX; hp += GH) {
        if (hp >= G) break;
#pragma unroll
        for (int hh = 0; hh < GH; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[run][hh][dl * 8 + e] = acc[hp + hh][e];
        __syncthreads();
        for (int i = tid; i < GH * D; i += kThreads) {
            const int hh = i / D, e = i % D;
            if (hp + hh < G) {
                float s = red[0][hh][e];
#pragma unroll
                for (int q = 1; q < NRUN; ++q) s += red[q][hh][e];
                a.o[(((int64_t)r * a.hq + g * G + hp + hh) * a.C + kslot) * D + e] = s;
            }
        }
        __syncthreads();
    }
}

// Ordered merge: M = max m_c over the row's chunks, a_c = expf(m_c - M), out = bf16(sum a_c o_c /
// sum a_c l_c), both sums fma chains in chunk order. One wave per (row, query head): lane c
// holds chunk c's (m, l), lane i dims DL*i .. DL*i + DL - 1. (row, head)s with a non-finite
// output are listed and, when the caller passed q/K/V, re-run in float64 afterwards by the
// whole workgroup.
constexpr int kMergePairs = 4;     // = waves of a D = 256 workgroup; D = 128 loops twice

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
    constexpr int W = D / 64;             // waves
    constexpr int DL = D / 64;            // dims per lane
    __shared__ int flagged[kMergePairs];
    __shared__ int nflag;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t npairs = (int64_t)a.rows * a.hq;
    const int64_t first = (int64_t)blockIdx.x * kMergePairs;
    if (t == 0) nflag = 0;
    __syncthreads();
    for (int i = wave; i < kMergePairs; i += W) {
        const int64_t pr = first + i;
        if (pr >= npairs) break;
        const int r = (int)(pr / a.hq), h = (int)(pr % a.hq);
        const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
        int n = rs.c_hi - rs.c_lo + 1;
        n = n > a.C ? a.C : n;
        const int64_t pi = pr * a.C;      // (r * hq + h) * C
        float M = -INFINITY;
        for (int cb = 0; cb < n; cb += 64)
            M = fmaxf(M, cb + lane < n ? a.m[pi + cb + lane] : -INFINITY);
        M = wave_max(M);
        float num[DL], den = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) num[e] = 0.f;
        const float* op = a.o + pi * D + DL * lane;
        for (int cb = 0; cb < n; cb += 64) {
            const bool in = cb + lane < n;
            const float ac = expf((in ? a.m[pi + cb + lane] : -INFINITY) - M);
            const float lc = in ? a.l[pi + cb + lane] : 0.f;
            const int ce = min(n - cb, 64);
            // eight chunks' o loads in flight at a time, then their fmas in chunk order
            for (int cg = 0; cg < ce; cg += 8) {
                float o[8][DL];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (cg + j < ce) {
                        const float* oc = op + (int64_t)(cb + cg + j) * D;
                        if constexpr (DL == 4) {
                            const float4 v = *reinterpret_cast<const float4*>(oc);
                            o[j][0] = v.x; o[j][1] = v.y; o[j][2] = v.z; o[j][3] = v.w;
                        } else {
                            const float2 v = *reinterpret_cast<const float2*>(oc);
                            o[j][0] = v.x; o[j][1] = v.y;
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (cg + j < ce) {
                        const float ac_c = __shfl(ac, cg + j, 64);
                        const float l_c = __shfl(lc, cg + j, 64);
#pragma unroll
                        for (int e = 0; e < DL; ++e) num[e] = fmaf(ac_c, o[j][e], num[e]);
                        den = fmaf(ac_c, l_c, den);
                    }
                }
            }
        }
        uint16_t* orow = a.out + (int64_t)r * a.o_srow + (int64_t)h * a.o_shead;
        bool bad = false;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            const uint32_t b = f32_to_bf16_rne(num[e] / den);
            orow[DL * lane + e] = (uint16_t)b;
            bad = bad || bf16_nonfinite((uint16_t)b);
        }
        if (a.rerun && __any(bad) && lane == 0) flagged[atomicAdd(&nflag, 1)] = i;
    }
    __syncthreads();
    const int nf = nflag;
    for (int f = 0; f < nf; ++f) {
        const int64_t pr = first + flagged[f];
        const int r = (int)(pr / a.hq), h = (int)(pr % a.hq);
        const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
        int t_ = a.stream_of_row[r];
        t_ = t_ < 0 ? 0 : (t_ >= a.streams ? a.streams - 1 : t_);
        const int g = h / (a.hq / a.hkv);
        const int64_t kv = (int64_t)t_ * a.kv_sstream + (int64_t)g * a.kv_shead;
        uint16_t* orow = a.out + (int64_t)r * a.o_srow + (int64_t)h * a.o_shead;
        rerun_f64<D>(a.q + (int64_t)r * a.q_srow + (int64_t)h * a.q_shead, a.k + kv, a.v + kv,
                     a.kv_sslot, a.ring, rs.lo, rs.pos, a.scale, orow);
        __syncthreads();
    }
}

template <int D>
hipError_t launch_part_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    dim3 grid(a.C * a.hkv * a.rows);
    if (G <= 1) hipLaunchKernelGGL((decode_part_kernel<D, 1>), grid, dim3(kThreads), 0, s, a);
    else if (G <= 2) hipLaunchKernelGGL((decode_part_kernel<D, 2>), grid, dim3(kThreads), 0, s, a);
    else if (G <= 4) hipLaunchKernelGGL((decode_part_kernel<D, 4>), grid, dim3(kThreads), 0, s, a);
    else if (G <= 8) hipLaunchKernelGGL((decode_part_kernel<D, 8>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_part_kernel<D, 16>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_part(const DecodeArgs& a, hipStream_t s) {
    return a.d == 256 ? launch_part_d<256>(a, s) : launch_part_d<128>(a, s);
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(((int64_t)a.rows * a.hq + kMergePairs - 1) / kMergePairs));
    if (a.d == 256) hipLaunchKernelGGL((merge_kernel<256>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace wa
