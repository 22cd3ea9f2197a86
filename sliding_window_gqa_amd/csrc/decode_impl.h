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
// This header holds the chunk kernel; decode_inst.hip instantiates it once per (head dim,
// query heads per key head, form), and decode.hip holds the merge kernel and the launchers.
#pragma once

#include "wa_common.h"
#include "rerun_f64.h"

namespace wa {

namespace {

constexpr int kThreads = 256;
constexpr int kRowCMax = 8;                // most chunks per row in the whole-row kernel
constexpr int kRowMinWG = 256;             // smaller batches use the chunk-partial kernel
constexpr int kBufferWord3 = 0x00020000;   // buffer descriptor word 3: raw 32-bit data format
constexpr int kLoadNonTemporal = 2;        // cache-policy bit of a buffer load: nt (streaming)

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
    s.lo = window > 0 ? max(0, p - window + 1 - (WA_CONTROL == 1)) : 0;
    s.c_lo = s.lo / kChunk;
    s.c_hi = p / kChunk;
    return s;
}

// The merge's final rounding (nearest-even; toward zero in control build 4).
__device__ __forceinline__ uint32_t merge_round(float x) {
    if constexpr (WA_CONTROL == 4) return (x != x) ? 0x7FC0u : (__float_as_uint(x) >> 16);
    return f32_to_bf16_rne(x);
}

// Linear workgroup id -> logical id such that each XCD (8 on MI355X, ids dealt out
// round-robin) runs a contiguous range of logical ids.
__device__ __forceinline__ int xcd_logical(int L, int total) {
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, extra = total & 7;
    return (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a compile-time index for the written-out unit steps
template <int N>
struct Int {
    static constexpr int value = N;
};

// 2-element bf16 dot product accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// The partner lane of a reduction step inside a group of 32 lanes; partners differ in bit
// log2(M) of the lane index: xor for M = 1, 2 (quad permutes), the mirror image inside 8 and
// 16 lanes for M = 4, 8 (row half-mirror, row mirror), xor 16 through the swizzle unit.
template <int M>
__device__ __forceinline__ float partner(float x) {
    const int i = __float_as_int(x);
    int r;
    if constexpr (M == 1) r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);
    else if constexpr (M == 2) r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);
    else if constexpr (M == 4) r = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true);
    else if constexpr (M == 8) r = __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, true);
    else r = __builtin_amdgcn_ds_swizzle(i, 0x401F);
    return __int_as_float(r);
}

// One step of the transposing sum: of 2N values (keys) a lane keeps the half selected by
// bit M of its index, adding the partner's copy of that half.
template <int M, int N>
__device__ __forceinline__ void halve(const float (&in)[2 * N], float (&out)[N], int dl) {
    const bool up = (dl & M) != 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float keep = up ? in[N + j] : in[j];
        const float send = up ? in[j] : in[N + j];
        out[j] = keep + partner<M>(send);
    }
}

// Sum over the LPK lanes of a run of TK per-lane partials v[i] (key i of a TK-key unit, TK =
// 8 or 16). TK = 16: lane dl ends with the full sum of key dl >> 1 (LPK = 32; lanes dl and
// dl ^ 1 agree) or key dl (LPK = 16). TK = 8: key dl >> 2 (LPK = 32; lanes dl .. dl ^ 3
// agree) or key dl >> 1 (LPK = 16; lanes dl and dl ^ 1 agree). A fixed tree: the bits of a
// key never depend on the data.
template <int LPK, int TK>
__device__ __forceinline__ float unit_sum(const float (&v)[TK], int dl) {
    static_assert(LPK == 32 || LPK == 16, "8 dims a lane at d = 128 or 256");
    if constexpr (TK == 16) {
        float a8[8], a4[4], a2[2], a1[1];
        if constexpr (LPK == 32) {
            halve<16, 8>(v, a8, dl);
            halve<8, 4>(a8, a4, dl);
            halve<4, 2>(a4, a2, dl);
            halve<2, 1>(a2, a1, dl);
            return a1[0] + partner<1>(a1[0]);
        } else {
            halve<8, 8>(v, a8, dl);
            halve<4, 4>(a8, a4, dl);
            halve<2, 2>(a4, a2, dl);
            halve<1, 1>(a2, a1, dl);
            return a1[0];
        }
    } else {
        static_assert(TK == 8, "units of 8 or 16 keys");
        float a4[4], a2[2], a1[1];
        if constexpr (LPK == 32) {
            halve<16, 4>(v, a4, dl);
            halve<8, 2>(a4, a2, dl);
            halve<4, 1>(a2, a1, dl);
            const float s = a1[0] + partner<2>(a1[0]);
            return s + partner<1>(s);
        } else {
            halve<8, 4>(v, a4, dl);
            halve<4, 2>(a4, a2, dl);
            halve<2, 1>(a2, a1, dl);
            return a1[0] + partner<1>(a1[0]);
        }
    }
}

template <int D, int GMAX, bool WHOLE, int UK>
__global__ __launch_bounds__(kThreads, WHOLE || GMAX > 8 ? 2
                                      : UK == 8 ? (GMAX <= 2 ? 8 : 4)
                                      : UK == 16 ? (GMAX <= 2 ? 4 : 3) : 2) void decode_kernel(DecodeArgs a) {
    constexpr int LPK = D / 8;               // lanes per key: 8 dims a lane
    constexpr int NRUN = kThreads / LPK;     // runs of consecutive keys per chunk
    constexpr int RUNLEN = kChunk / NRUN;    // keys per run
    // TK-key units of the lane tree and the fma chains: 8 keys up to four query heads a key
    // head, 16 beyond (fewer live partials a head); UK-key load units, UK >= TK
    constexpr int TK = GMAX <= 4 ? 8 : 16;
    constexpr int NU = RUNLEN / TK;          // tree units per run
    constexpr int NL = RUNLEN / UK;          // load units per run, for K and for V
    constexpr int HU = UK / TK;              // tree units per load unit
    constexpr int GH = GMAX < 4 ? GMAX : 4;  // heads per LDS reduction pass
    constexpr int CM = WHOLE ? kRowCMax : 1;
    static_assert(!WHOLE || (D == 256 && GMAX <= 2), "whole rows: d = 256, at most two query heads per key head");
    static_assert(RUNLEN == 16 || RUNLEN == 32, "runs of 16 or 32 keys");
    static_assert((UK == 8 || UK == 16 || UK == 32) && UK >= TK && UK <= RUNLEN,
                  "load units of 8, 16 or 32 keys, whole tree units within a run");

    __shared__ float sc[GMAX][kChunk];
    __shared__ float red[NRUN][GH][D];
    __shared__ __attribute__((aligned(16))) uint16_t qs[GMAX][D];
    __shared__ float part[CM][WHOLE ? GMAX : 1][WHOLE ? D : 1];
    __shared__ float cm[CM][GMAX];
    __shared__ float cl[CM][GMAX];

    const int logical = xcd_logical(blockIdx.x, gridDim.x);
    int g, r, kslot = 0;
    if constexpr (WHOLE) {
        // logical order (key head, row)
        g = logical / a.rows;
        r = logical % a.rows;
    } else {
        // logical order (key head, row, chunk slot)
        const int per_g = a.rows * a.C;
        g = logical / per_g;
        r = (logical % per_g) / a.C;
        kslot = logical % a.C;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = a.hq / a.hkv;

    const RowSpan rs = row_span(a.pos_of_row, r, a.max_pos, a.window);
    const int nchunks = rs.c_hi - rs.c_lo + 1;
    int k0, nch;
    if constexpr (WHOLE) {
        k0 = 0;
        nch = min(nchunks, min(a.C, kRowCMax));
    } else {
        if (kslot >= nchunks) return;
        k0 = kslot;
        nch = 1;
    }
    int t = a.stream_of_row[r];
    t = t < 0 ? 0 : (t >= a.streams ? a.streams - 1 : t);
    const uint16_t* kbase_ptr = a.k + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
    const uint16_t* vbase_ptr = a.v + (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
    // Buffer loads from the key head's ring: base and extent in scalar registers, a 32-bit
    // lane offset, and anything past the extent reads as zero. The host checks that the
    // ring's byte span fits in 31 bits.
    const uint32_t sslot_b = (uint32_t)a.kv_sslot * 2u;
    const int extent = (int)((uint32_t)(a.ring - 1) * sslot_b + 2u * D);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase_ptr, (short)0, extent, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase_ptr, (short)0, extent, kBufferWord3);
    // Whole rows are read once (their rings are not shared): non-temporal loads keep them from
    // displacing other data in the caches (the 64-stream decode: 102 -> 94 us). Chunk
    // workgroups keep the default policy, as rows sharing a ring re-read its keys from L2.
    auto ld16 = [](__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff, (int)soff,
                                                                               WHOLE ? kLoadNonTemporal : 0));
    };
    // A load unit is UK (8, 16 or 32) keys starting at an absolute position that is a
    // multiple of UK; in a ring whose length is a multiple of UK such a unit never wraps, so
    // its keys are one lane offset plus the key step i * slot bytes in the instruction's
    // scalar offset (the whole-row kernel's rings are multiples of 16, its units 8 keys).
    const bool aligned = WHOLE || (a.ring & (UK - 1)) == 0;
    const bool big_ring = WHOLE || a.ring >= kChunk;

    struct Chunk {
        int kbase, nk, sb;
    };
    auto chunk_at = [&](int k) {
        const int c = rs.c_lo + k;
        const int j0 = max(rs.lo, c * kChunk);
        const int j1 = min(rs.pos, c * kChunk + kChunk - 1);
        Chunk ch;
        ch.nk = j1 - j0 + 1;              // visible keys in the chunk, >= 1
        ch.kbase = j0 - c * kChunk;       // chunk-relative index of the first visible key
        ch.sb = (c * kChunk) % a.ring;
        return ch;
    };
    // ring slot of chunk-relative key kk (a ring of at least one chunk wraps at most once
    // inside a chunk)
    auto slot_of = [&](const Chunk& ch, int kk) {
        const int s = ch.sb + kk;
        return big_ring ? (s >= a.ring ? s - a.ring : s) : s % a.ring;
    };

    // this thread's run and dims: keys run*RUNLEN .. +RUNLEN-1, dims 8 dl .. 8 dl + 7
    const int run = tid / LPK;
    const int dl = tid % LPK;

    // the query heads of the key head, staged in LDS (heads >= G repeat head G-1, unused)
    for (int i = tid; i < GMAX * D / 8; i += kThreads) {
        const int h = i / (D / 8), c = i % (D / 8);
        const uint16_t* qp = a.q + (int64_t)r * a.q_srow + (int64_t)(g * G + min(h, G - 1)) * a.q_shead + 8 * c;
        *reinterpret_cast<uint4*>(&qs[h][8 * c]) = *reinterpret_cast<const uint4*>(qp);
    }
    __syncthreads();

    // Load unit u of a chunk: u < NL are K units, u >= NL V units; unit b of either covers
    // keys run*RUNLEN + UK b .. + UK - 1 of the run and fills the register buffer, which is
    // refilled with the next unit as soon as the unit has been consumed. Every unit issues its
    // UK loads (a run with no visible key reads the head's first row instead), so the loads in
    // flight are fixed and every wait covers exactly the unit about to be consumed. Keys of a
    // run outside the row's range are fetched (their slots are in the ring) and ignored. The
    // load unit sets only how many loads a wave has in flight, never the arithmetic, which
    // works on TK-key tree units: 8-key load units let eight workgroups share a CU (more waves
    // to cover the L2 latency of shared keys), 16-key ones cut the round trips of a small grid.
    struct Unit {
        uint32_t vo;     // lane offset of the unit's first key (aligned rings)
        int s0;          // ring slot of the unit's first key
        bool on;         // the run holds a visible key (else the loads read the first slots)
        bool isv;
    };
    auto unit_of = [&](const Chunk& ch, int u, bool want) {
        Unit un;
        un.isv = u >= NL;
        const int b = un.isv ? u - NL : u;
        const int r0 = max(run * RUNLEN, ch.kbase);
        const int r1 = min(run * RUNLEN + RUNLEN, ch.kbase + ch.nk);
        un.on = want && r0 < r1;
        un.s0 = un.on ? slot_of(ch, run * RUNLEN + UK * b) : 0;
        un.vo = (uint32_t)un.s0 * sslot_b + 16u * dl;
        return un;
    };
    auto load_key = [&](const Unit& un, int i) {
        const __amdgpu_buffer_rsrc_t rsrc = un.isv ? vrs : krs;
        if (aligned) return ld16(rsrc, un.vo, (uint32_t)i * sslot_b);
        int sl = un.s0 + i;
        sl = big_ring ? (sl >= a.ring ? sl - a.ring : sl) : sl % a.ring;
        return ld16(rsrc, (uint32_t)sl * sslot_b + 16u * dl, 0u);
    };
    auto issue = [&](const Chunk& ch, int u, bool want, uint4 (&B)[UK]) __attribute__((always_inline)) {
        const Unit un = unit_of(ch, u, want);
#pragma unroll
        for (int i = 0; i < UK; ++i) B[i] = load_key(un, i);
    };
    // (The per-unit lambdas are always inlined: at 16 query heads a key head the compiler
    // otherwise left the head loops rolled and kept the accumulators in scratch memory.)
    // Scores of the run's tree unit b (buffer entries o .. o + TK - 1): s = scale * (q . k)
    // for every head of the group, into sc.
    auto consume_k = [&](const Chunk& ch, int b, const uint4 (&B)[UK], int o) __attribute__((always_inline)) {
        const int key = TK == 16 ? (LPK == 32 ? (dl >> 1) : dl) : (LPK == 32 ? (dl >> 2) : (dl >> 1));
        const bool writer = TK == 16 ? (LPK == 32 ? (dl & 1) == 0 : true)
                                     : (LPK == 32 ? (dl & 3) == 0 : (dl & 1) == 0);
        const int kk = run * RUNLEN + TK * b + key;
        const bool vis = writer && kk >= ch.kbase && kk < ch.kbase + ch.nk;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h < G) {
                const uint4 qv = *reinterpret_cast<const uint4*>(&qs[h][8 * dl]);
                float v[TK];
#pragma unroll
                for (int i = 0; i < TK; ++i) {
                    float s = dot2(qv.x, B[o + i].x, 0.f);
                    s = dot2(qv.y, B[o + i].y, s);
                    s = dot2(qv.z, B[o + i].z, s);
                    v[i] = dot2(qv.w, B[o + i].w, s);
                }
                const float s = unit_sum<LPK, TK>(v, dl);
                if (vis) sc[h][kk] = a.scale * s;
            }
        }
    };
    float acc[GMAX][8];
    auto fold_key = [&](const uint4& w, int kk) __attribute__((always_inline)) {
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
    // P.V of the run's tree unit b (buffer entries o .. o + TK - 1): fma chains in key order
    // over the run's visible keys
    auto consume_v = [&](const Chunk& ch, int b, const uint4 (&B)[UK], int o) __attribute__((always_inline)) {
        const int r0 = max(run * RUNLEN, ch.kbase);
        const int r1 = min(run * RUNLEN + RUNLEN, ch.kbase + ch.nk);
        if (r0 == run * RUNLEN && r1 == run * RUNLEN + RUNLEN) {
#pragma unroll
            for (int i = 0; i < TK; ++i) fold_key(B[o + i], run * RUNLEN + TK * b + i);
        } else if (r0 < r1) {
#pragma unroll
            for (int i = 0; i < TK; ++i) {
                const int kk = run * RUNLEN + TK * b + i;
                if (kk >= r0 && kk < r1) fold_key(B[o + i], kk);
            }
        }
    };

    // one register buffer (two, double the loads in flight, measured slower on this part's
    // memory system)
    uint4 X[UK];
    Chunk cur = chunk_at(k0);
    issue(cur, 0, true, X);
    for (int k = k0; k < k0 + nch; ++k) {
        const int ks = k - k0;                   // chunk slot within this workgroup
        const bool more = k + 1 < k0 + nch;
        const Chunk nxt = chunk_at(more ? k + 1 : k);
        // ---- scores; each consumed unit frees the buffer for the next: K units, then the
        // first V unit
        // (the tree units are written out, not looped over: in a loop the compiler kept more
        // registers live and spilled at eight or more query heads a key head)
        auto kstep = [&](auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            if constexpr (b < NU) {
                consume_k(cur, b, X, TK * (b % HU));
                if constexpr (b % HU == HU - 1) issue(cur, b / HU + 1, true, X);
            }
        };
        kstep(Int<0>{});
        kstep(Int<1>{});
        kstep(Int<2>{});
        kstep(Int<3>{});
        __syncthreads();
        // ---- chunk softmax: m_c, p = expf(s - m_c), l_c, one wave per head
        for (int h = wave; h < G; h += 4) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = lane + 64 * i;
                if (kk < cur.nk) mx = fmaxf(mx, sc[h][cur.kbase + kk]);
            }
            mx = wave_max(mx);
            const float mu = (mx == -INFINITY) ? 0.f : mx;   // all scores -inf: weights 0
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = lane + 64 * i;
                if (kk < cur.nk) {
                    const float p = expf(sc[h][cur.kbase + kk] - mu);
                    sc[h][cur.kbase + kk] = p;
                    sum += p;
                }
            }
            sum = wave_sum(sum);
            if (lane == 0) {
                if constexpr (WHOLE) {
                    cm[ks][h] = mx;
                    cl[ks][h] = sum;
                } else {
                    const int64_t pi = ((int64_t)r * a.hq + g * G + h) * a.C + kslot;
                    a.m[pi] = mx;
                    a.l[pi] = sum;
                }
            }
        }
        __syncthreads();
        // ---- P.V; the freed buffer takes the remaining V units, then the next chunk's first
        // K unit
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
        auto vstep = [&](auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            if constexpr (b < NU) {
                consume_v(cur, b, X, TK * (b % HU));
                if constexpr (b % HU == HU - 1) {
                    if constexpr (b / HU + 1 < NL) issue(cur, NL + b / HU + 1, true, X);
                    else if (WHOLE) issue(nxt, 0, more, X);
                }
            }
        };
        vstep(Int<0>{});
        vstep(Int<1>{});
        vstep(Int<2>{});
        vstep(Int<3>{});
        // ---- runs summed in run order, GH heads per pass
#pragma unroll
        for (int hp = 0; hp < GMAX; hp += GH) {
            if (hp < G) {
#pragma unroll
                for (int hh = 0; hh < GH; ++hh)
#pragma unroll
                    for (int e = 0; e < 8; ++e) red[run][hh][dl * 8 + e] = acc[hp + hh][e];
                __syncthreads();
#pragma unroll
                for (int i = tid; i < GH * D; i += kThreads) {
                    const int hh = i / D, e = i % D;
                    if (hp + hh < G) {
                        float s = red[0][hh][e];
#pragma unroll
                        for (int q = 1; q < NRUN; ++q) s += red[q][hh][e];
                        if constexpr (WHOLE) part[ks][hp + hh][e] = s;
                        else a.o[(((int64_t)r * a.hq + g * G + hp + hh) * a.C + kslot) * D + e] = s;
                    }
                }
                if (!WHOLE || GMAX > GH) __syncthreads();
            }
        }
        cur = nxt;
    }
    if constexpr (WHOLE) {
        __syncthreads();
        // merge in chunk order (merge_kernel's arithmetic), and the chunk partials to the
        // workspace in the layout wa_merge reads; thread tid holds dim tid of every head
        __shared__ int bad[GMAX];
        if (tid < GMAX) bad[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) {
            if (hh < G) {
                const int h = g * G + hh;
                const int64_t pi = ((int64_t)r * a.hq + h) * a.C;
                float M = -INFINITY;
                for (int k = 0; k < nch; ++k) M = fmaxf(M, cm[k][hh]);
                float num = 0.f, den = 0.f;
                for (int k = 0; k < nch; ++k) {
                    const float ac = WA_CONTROL == 3 ? 1.f : expf(cm[k][hh] - M);
                    const float o = part[k][hh][tid];
                    num = fmaf(ac, o, num);
                    den = fmaf(ac, cl[k][hh], den);
                    a.o[(pi + k) * D + tid] = o;
                }
                if (tid < nch) {
                    a.m[pi + tid] = cm[tid][hh];
                    a.l[pi + tid] = cl[tid][hh];
                }
                const uint32_t bits = merge_round(num / den);
                a.out[(int64_t)r * a.o_srow + (int64_t)h * a.o_shead + tid] = (uint16_t)bits;
                if (bf16_nonfinite((uint16_t)bits)) bad[hh] = 1;
            }
        }
        __syncthreads();
        if (!a.rerun) return;
#pragma unroll
        for (int hh = 0; hh < GMAX; ++hh) {
            if (hh < G && bad[hh]) {
                const int h = g * G + hh;
                const int64_t kv = (int64_t)t * a.kv_sstream + (int64_t)g * a.kv_shead;
                rerun_f64<D>(a.q + (int64_t)r * a.q_srow + (int64_t)h * a.q_shead, a.k + kv, a.v + kv,
                             a.kv_sslot, a.ring, rs.lo, rs.pos, a.scale,
                             a.out + (int64_t)r * a.o_srow + (int64_t)h * a.o_shead);
                __syncthreads();
            }
        }
    }
}

// Launch of decode_kernel<D, GMAX, WHOLE, UK> on `grid` workgroups (defined by the file that
// instantiates it).
template <int D, int GMAX, bool WHOLE, int UK>
hipError_t launch_chunk_kernel(const DecodeArgs& a, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((decode_kernel<D, GMAX, WHOLE, UK>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace wa
