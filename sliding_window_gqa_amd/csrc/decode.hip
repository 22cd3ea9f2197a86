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
//   scores  D/8 lanes per key, each lane an fma chain over 8 consecutive dims of the key
//           (one 16-byte load), then a xor butterfly across those lanes; 64/(D/8) keys per
//           wave instruction, coalesced 16-byte loads of each key row.
//   softmax one wave per query head: 4 keys per lane, wave butterflies for max and sum.
//   P.V     NRUN key runs of 256/NRUN consecutive keys; D/8 lanes per run, 8 dims a lane;
//           each run is an fma chain in key order; runs are summed in run order through LDS.
#include "wa_common.h"

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

template <int D, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_part_kernel(DecodeArgs a) {
    constexpr int LPK = D / 8;           // lanes per key in the score pass
    constexpr int KPW = 64 / LPK;        // keys per wave instruction
    constexpr int NRUN = kThreads / LPK; // P.V key runs
    constexpr int RUNLEN = kChunk / NRUN;
    constexpr int GH = GMAX < 4 ? GMAX : 4;   // heads per LDS reduction pass

    __shared__ float qs[GMAX][D];
    __shared__ float sc[GMAX][kChunk];
    __shared__ float red[NRUN][GH][D];

    const int kslot = blockIdx.x;
    const int g = blockIdx.y;
    const int r = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = a.hq / a.hkv;

    const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
    const int c = rs.c_lo + kslot;
    if (c > rs.c_hi || kslot >= a.C) return;
    int t = a.stream_of_row[r];
    t = t < 0 ? 0 : (t >= a.streams ? a.streams - 1 : t);
    const int j0 = max(rs.lo, c * kChunk);
    const int j1 = min(rs.pos, c * kChunk + kChunk - 1);
    const int nk = j1 - j0 + 1;           // visible keys in this chunk, >= 1
    const int kbase = j0 - c * kChunk;    // chunk-relative index of the first visible key

    const uint16_t* kbase_ptr = a.k + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
    const uint16_t* vbase_ptr = a.v + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;

    // q of the group's heads, widened to fp32
    for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, e = i % D;
        qs[h][e] = bf16_to_f32(a.q[(int64_t)r * a.q_srow + (int64_t)(g * G + h) * a.q_shead + e]);
    }
    __syncthreads();

    // ---- scores: s = scale * (q . k) for the visible keys ----
    {
        const int sub = lane / LPK;          // key within the wave instruction
        const int dl = lane % LPK;           // 8-dim slice of the key
        float qf[GMAX][8];
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[h][e] = (h < G) ? qs[h][dl * 8 + e] : 0.f;
        for (int base = wave * KPW; base < nk; base += 4 * KPW) {
            const int kk = base + sub;
            const bool valid = kk < nk;
            const int j = j0 + (valid ? kk : 0);
            const int slot = j % a.ring;
            float kf[8];
            load8(kbase_ptr + (int64_t)slot * a.kv_sslot + dl * 8, kf);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h < G) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = fmaf(qf[h][e], kf[e], s);
#pragma unroll
                    for (int m = 1; m < LPK; m <<= 1) s += xor_shfl(s, m);
                    if (valid && dl == 0) sc[h][kbase + kk] = a.scale * s;
                }
            }
        }
    }
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
    const int run = tid / LPK;
    const int dl = tid % LPK;
    float acc[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    {
        const int r0 = max(run * RUNLEN, kbase);
        const int r1 = min(run * RUNLEN + RUNLEN, kbase + nk);
        for (int kk = r0; kk < r1; ++kk) {
            const int slot = (c * kChunk + kk) % a.ring;
            float vf[8];
            load8(vbase_ptr + (int64_t)slot * a.kv_sslot + dl * 8, vf);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h < G) {
                    const float p = sc[h][kk];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
                }
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

// One workgroup per (row, query head); one thread per output dim.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
    const int r = blockIdx.x;
    const int h = blockIdx.y;
    const int e = threadIdx.x;
    const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
    int n = rs.c_hi - rs.c_lo + 1;
    n = n > a.C ? a.C : n;
    const int64_t pi = ((int64_t)r * a.hq + h) * a.C;
    float M = -INFINITY;
    for (int c = 0; c < n; ++c) M = fmaxf(M, a.m[pi + c]);
    float num = 0.f, den = 0.f;
    for (int c = 0; c < n; ++c) {
        const float ac = expf(a.m[pi + c] - M);
        num = fmaf(ac, a.o[(pi + c) * D + e], num);
        den = fmaf(ac, a.l[pi + c], den);
    }
    a.out[(int64_t)r * a.o_srow + (int64_t)h * a.o_shead + e] = (uint16_t)f32_to_bf16_rne(num / den);
}

template <int D>
hipError_t launch_part_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    dim3 grid(a.C, a.hkv, a.rows);
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
    dim3 grid(a.rows, a.hq);
    if (a.d == 256) hipLaunchKernelGGL((merge_kernel<256>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace wa
