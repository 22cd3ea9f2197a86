// Split-KV decode for windowed GQA attention on gfx950: chunk partials and the ordered merge.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Decode bullet. Keys are split into 256-key chunks at absolute key
// positions; for each (row, key head, chunk) the G query heads of the key head get fp32
// scores, the chunk max m_c, p = expf(s - m_c), l_c = sum p and o_c = sum p v with p kept in
// fp32; the chunks of a row are then merged in chunk order. Chunks holding none of a row's
// keys take no part, so the split depends only on key positions.
//
// gfx950 mapping (wave64, 256 threads): the chunk's keys form NRUN runs of consecutive keys,
// each run owned by D/8 lanes holding 8 dims apiece, for K and V alike. Every load
// instruction of a wave then reads whole 512-byte key rows (two keys per instruction at
// d = 256), the pattern that streams HBM best on this part.
//   scores  per lane: 8-dim partial dot products with v_dot2_f32_bf16 (bf16 pairs, fp32
//           accumulate), then a transposing sum over the run's lanes (DPP quad permutes and
//           row mirrors, a swizzle for the 16-lane step) that leaves each key's score in one
//           lane: 8 keys per reduction up to four query heads a key head, 16 beyond; no
//           partial sum kept longer than needed.
//   softmax one wave per query head: 4 keys per lane, wave butterflies for max and sum.
//   P.V     fp32 on the VALU: each run is an fma chain in key order over its keys, 8 dims a
//           lane; the runs are summed in run order through LDS.
//   loads   K and V arrive in units of 8 keys (8 x 16 bytes per lane) for large grids, at
//           most 64 registers so that eight workgroups share a CU, or of 16 or 32 keys (fewer
//           round trips) for small grids, through one register buffer that is
//           refilled with the next unit as soon as it is consumed; a second buffer (twice the
//           loads in flight) streamed slower.
//   kernels decode_kernel<.., false, ..>: one workgroup per (row, key head, chunk), partials
//           to memory, then merge_kernel; decode_kernel<.., true, 8>: for large batches of
//           rows that do not share rings, one workgroup per (row, key head) walks the row's
//           chunks and merges them itself.
//           All run the same per-chunk arithmetic (the load unit sets only the loads in
//           flight) and the same merge arithmetic, so a row's bits do not depend on which one
//           ran it (nor on the batch, the slot or the ring size).
//   grid    workgroup ids remapped so that each XCD works on the rows of a few key heads and
//           their rings stay in its L2.
//
// This file: the merge kernel and the launchers; the chunk kernel is in decode_impl.h and
// decode_inst.hip instantiates it.
#include "decode_impl.h"

namespace wa {

hipError_t launch_decode_kernel_128_1(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_128_2(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_128_4(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_128_8(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_128_16(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_256_1(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_256_2(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_256_4(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_256_8(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_kernel_256_16(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_128_1(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_128_2(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_128_4(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_128_8(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_128_16(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_256_1(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_256_2(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_256_4(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_256_8(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_small_256_16(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_whole_256_1(const DecodeArgs&, unsigned, hipStream_t);
hipError_t launch_decode_whole_256_2(const DecodeArgs&, unsigned, hipStream_t);

namespace {

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
        const int64_t pi = pr * a.C;      // (r * hq + h) * C
        const float* op = a.o + pi * D + DL * lane;
        // eight chunks' o at a time, chunk c0 + j from chunk c0 (j < cnt)
        auto load8 = [&](float (&o)[8][DL], int c0, int cnt) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < cnt) {
                    const float* oc = op + (int64_t)(c0 + j) * D;
                    if constexpr (DL == 4) {
                        const float4 v = *reinterpret_cast<const float4*>(oc);
                        o[j][0] = v.x; o[j][1] = v.y; o[j][2] = v.z; o[j][3] = v.w;
                    } else {
                        const float2 v = *reinterpret_cast<const float2*>(oc);
                        o[j][0] = v.x; o[j][1] = v.y;
                    }
                }
            }
        };
        // the pair's first 64 chunk slots' (m, l) and first eight slots' o are all requested
        // before the row's position is known (slots past the row's chunk count hold stale
        // values and are never used), so the common row takes one memory round trip, not two
        float o[8][DL];
        load8(o, 0, min(a.C, 8));
        const bool inC = lane < a.C;
        const float mC = inC ? a.m[pi + lane] : -INFINITY;
        const float lC = inC ? a.l[pi + lane] : 0.f;
        const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
        int n = rs.c_hi - rs.c_lo + 1;
        n = n > a.C ? a.C : n;
        const bool in0 = lane < n;
        const float m0 = in0 ? mC : -INFINITY;
        const float l0 = in0 ? lC : 0.f;
        float M = fmaxf(-INFINITY, m0);
        for (int cb = 64; cb < n; cb += 64)
            M = fmaxf(M, cb + lane < n ? a.m[pi + cb + lane] : -INFINITY);
        M = wave_max(M);
        float num[DL], den = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) num[e] = 0.f;
        for (int cb = 0; cb < n; cb += 64) {
            const bool in = cb + lane < n;
            const float ac = WA_CONTROL == 3 ? (in ? 1.f : 0.f)
                                             : expf((cb == 0 ? m0 : (in ? a.m[pi + cb + lane] : -INFINITY)) - M);
            const float lc = cb == 0 ? l0 : (in ? a.l[pi + cb + lane] : 0.f);
            const int ce = min(n - cb, 64);
            // eight chunks' o loads in flight at a time, then their fmas in chunk order
            for (int cg = 0; cg < ce; cg += 8) {
                if (cb + cg > 0) load8(o, cb + cg, ce - cg);
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
            const uint32_t b = merge_round(num[e] / den);
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

// Chunk grids below this many workgroups (under four a CU) load 16- or 32-key units (fewer
// round trips per chunk); larger grids load 8-key units, which fit eight workgroups a CU.
// The arithmetic is the same.
constexpr unsigned kSmallGrid = 1024;

template <int D>
hipError_t launch_part_d(const DecodeArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const unsigned grid = (unsigned)(a.C * a.hkv * a.rows);
    if (grid < kSmallGrid) {
        if (D == 256) {
            if (G <= 1) return launch_decode_small_256_1(a, grid, s);
            if (G <= 2) return launch_decode_small_256_2(a, grid, s);
            if (G <= 4) return launch_decode_small_256_4(a, grid, s);
            if (G <= 8) return launch_decode_small_256_8(a, grid, s);
            return launch_decode_small_256_16(a, grid, s);
        }
        if (G <= 1) return launch_decode_small_128_1(a, grid, s);
        if (G <= 2) return launch_decode_small_128_2(a, grid, s);
        if (G <= 4) return launch_decode_small_128_4(a, grid, s);
        if (G <= 8) return launch_decode_small_128_8(a, grid, s);
        return launch_decode_small_128_16(a, grid, s);
    }
    if (D == 256) {
        if (G <= 1) return launch_decode_kernel_256_1(a, grid, s);
        if (G <= 2) return launch_decode_kernel_256_2(a, grid, s);
        if (G <= 4) return launch_decode_kernel_256_4(a, grid, s);
        if (G <= 8) return launch_decode_kernel_256_8(a, grid, s);
        return launch_decode_kernel_256_16(a, grid, s);
    }
    if (G <= 1) return launch_decode_kernel_128_1(a, grid, s);
    if (G <= 2) return launch_decode_kernel_128_2(a, grid, s);
    if (G <= 4) return launch_decode_kernel_128_4(a, grid, s);
    if (G <= 8) return launch_decode_kernel_128_8(a, grid, s);
    return launch_decode_kernel_128_16(a, grid, s);
}

// Whole rows for large batches of rows that do not share rings; rows sharing rings read
// their keys from L2 and run faster as chunk workgroups (more of them in flight per CU).
bool decode_whole_rows(const DecodeArgs& a) {
    const int G = a.hq / a.hkv;
    return a.d == 256 && G <= 2 && a.C <= kRowCMax && (int64_t)a.rows * a.hkv >= kRowMinWG &&
           a.streams >= a.rows && a.ring >= kChunk && (a.ring & 15) == 0;
}

}  // namespace

bool decode_extent_ok(int64_t ring, int64_t kv_sslot, int d) {
    return (ring - 1) * kv_sslot * 2 + 2 * d < 0x7FFFFFFF;
}

hipError_t launch_decode_part(const DecodeArgs& a, hipStream_t s) {
    return a.d == 256 ? launch_part_d<256>(a, s) : launch_part_d<128>(a, s);
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((unsigned)(((int64_t)a.rows * a.hq + kMergePairs - 1) / kMergePairs));
    if (a.d == 256) hipLaunchKernelGGL((merge_kernel<256>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (decode_whole_rows(a)) {
        const unsigned grid = (unsigned)((int64_t)a.rows * a.hkv);
        return a.hq == a.hkv ? launch_decode_whole_256_1(a, grid, s) : launch_decode_whole_256_2(a, grid, s);
    }
    hipError_t e = launch_decode_part(a, s);
    if (e != hipSuccess) return e;
    return launch_merge(a, s);
}

}  // namespace wa

