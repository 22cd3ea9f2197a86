// Dense prompt rows at head dim 256 on gfx950: the quarter-tile kernel.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Prompt, Window.p32 and promptRows(..., hi) bullets, as in
// prompt_impl.h: each row i sees keys [lo_i, last_i], keys come in tiles at absolute
// positions, every tile folds into a running (m, l, O) with one rescale, P enters P.V as one
// bf16, as bf16(P) + bf16(P - bf16(P)) (p32), or as three bf16 parts.
//
// Design (own): a workgroup holds 32 (row, query head) pairs of one key head and eight waves,
// two per SIMD. Wave w takes the keys 16 (w % 4) .. + 15 (its quarter) of the even tiles
// (absolute index) of the block's key range (w < 4) or of the odd ones (w >= 4), with a
// running (m, l, O) of its
// own; the two waves of a SIMD work on different tiles, so one's softmax runs while the
// other's matrix products do. After the last tile the eight states are merged in LDS, in
// wave order (M = max m_w, a_w = 2^(m_w - M), den = sum a_w l_w, out = bf16(sum (a_w / den)
// O_w), the sums fma chains in w order), half of the dims at a time. So every row is finished inside its workgroup: no fp32
// partials leave the CU and no merge kernel follows; a (row, head) whose bf16 output is not
// finite is re-run in float64 by the same workgroup (rerun_f64.h), so no check kernel
// follows either. A row's bits depend only on its key range and the absolute tile grid (a
// quarter holding none of the row's keys leaves that row's state exactly unchanged), never on
// how the prompt is cut into calls.
//   * S^T of a quarter (16 keys x 32 pairs) is two v_mfma_f32_16x16x32_bf16 chains (pairs
//     0..15 and 16..31) over eight 32-dim steps; K fragments are 16-byte LDS reads of the
//     wave's own rows, the Q^T operand 16-byte reads of the block's q, stored once in LDS;
//   * one v_permlane16_swap per accumulator register moves the scores into the layout of
//     the P^T operand of v_mfma_f32_32x32x16_bf16: lane l then holds pair l % 32 and keys
//     8 (l / 32) .. + 7 of the quarter, so the mask, the row maximum (one v_permlane32_swap
//     between the two lane halves), the exponentials and the O rescale are lane-local;
//   * O^T += V^T P^T over the quarter's 16 keys: eight 32-dim blocks, NP MFMAs each, V^T from
//     the transposing LDS read (ds_read_b64_tr_b16);
//   * each wave loads only its own 16 rows of K and V (no barrier in the walk) into one
//     stage per tile parity, by LDS-direct loads with explicit waits: V^T is read first, the
//     next quarter's V streams in during the score products and its K during P.V; 16-byte
//     chunks swizzled against bank conflicts, ring wrap as in the 128-pair kernel;
//   * workgroup ids are remapped so that each XCD walks a contiguous range of (key head,
//     block of pairs), keeping a key head's K/V stream in its L2.
// Against the 128-pair kernel this spreads one block of pairs over all four SIMDs of a CU
// (a quarter of the per-tile work on each), at four times the K/V bytes per pair moved from
// L2 into LDS.
#pragma once

#include "prompt_impl.h"

namespace wa {

namespace {

constexpr int kQuarterPairs = 32;     // (row, head) pairs per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt operands (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// vector-memory count at most 24, 16, 8 or 0, the other counters not waited for
constexpr int kWaitVm24 = 0x4000 | 0x0F78;
constexpr int kWaitVm16 = 0x4000 | 0x0F70;
constexpr int kWaitVm8 = 0x0F78;
constexpr int kWaitVm0 = 0x0F70;


constexpr int kOctWaves = 8;           // waves of a quarter-tile workgroup (two per SIMD)
constexpr int kOctThreads = 64 * kOctWaves;

template <int NP>
__global__ __launch_bounds__(kOctThreads, 1) void prompt_quarter_kernel(PromptArgs a, int nblk) {
    constexpr int D = 256;
    constexpr int KS = D / 32;             // 32-dim steps of S^T
    constexpr int DBLK = D / 32;           // 32-dim blocks of O^T
    constexpr int RB = 2 * D;              // bytes per K/V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPK = 1024 / RB;         // rows per 1 KiB wave load
    constexpr int TILE_B = BN * RB;        // bytes of one K (or V) tile
    constexpr int QL = 16 * RB / 1024;     // wave loads per quarter (each of K and V)
    static_assert(QL == KS && QL == DBLK, "one V load per score step, one K load per O block");
    // one stage per tile parity (K and V: 32 KiB each); wave w owns rows 16 (w % 4) .. + 15
    // of its parity's stage. After the walk these four arrays hold the O of the merge.
    __shared__ __attribute__((aligned(1024))) char Ks[2][TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs[2][TILE_B];
    // Q^T operand: pair p's 256 dims in 512 bytes, 16-byte chunk c at c ^ (p & 15)
    __shared__ __attribute__((aligned(1024))) char Qs[kQuarterPairs * RB];
    __shared__ float red_m[kOctWaves][kQuarterPairs];
    __shared__ float red_l[kOctWaves][kQuarterPairs];
    __shared__ int bad[kQuarterPairs];     // pairs whose bf16 output holds a NaN or an infinity

    // XCD x (ids dealt out to the 8 XCDs in turn) takes a contiguous share of the logical
    // ids (key head, block of pairs)
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int per = total >> 3, extra = total & 7;
    const int logical = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
    const int g = logical / nblk;          // key head
    const int blk = logical % nblk;        // block of pairs

    const int tid = threadIdx.x;
    if (tid < kQuarterPairs) bad[tid] = 0;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: quarter addresses
    const int qw = wave & 3;               // quarter of the tile
    const int par = wave >> 2;             // tile parity
    const int h = lane >> 5;               // lane half: keys 8h .. 8h + 7 of a quarter
    const int col = lane & 31;             // pair of the P^T / O^T layout
    const int c16 = lane & 15, q4 = lane >> 4;
    const int G = a.hq / a.hkv;

    const int pair = blk * kQuarterPairs + col;
    const int row = pair / G;
    const int head = g * G + pair % G;
    const bool valid = row < a.n;

    // the block's key range: lo is non-decreasing in the row, so the first valid row gives
    // kmin; kmax is the largest last key of a valid pair
    const int row_first = blk * kQuarterPairs / G;
    if (row_first >= a.n) return;          // no valid pair in this workgroup (uniform)
    const int kmin = prompt_lo(a, row_first);
    // every valid row's last key is at least its own position, so the last valid row's
    // position is a lower bound of the block's last key kmax (known before hi is)
    const int kmax_low = a.p0 + min(a.n - 1, (blk * kQuarterPairs + kQuarterPairs - 1) / G);
    const int t0 = kmin / BN;

    const uint16_t* kg = a.k + (int64_t)g * a.kv_shead;
    const uint16_t* vg = a.v + (int64_t)g * a.kv_shead;

    // Tile loads: a wave loads only its own quarter, QL 1 KiB wave loads each of K and V (RPK
    // rows of CPR chunks). A quarter with every key inside [kmin, kmax] and no ring wrap goes
    // by buffer loads from a descriptor on its first slot (no records: zeros); an edge quarter
    // key by key, clamped into [kmin, kmax] (keys outside a pair's range are masked) and
    // wrapped into the ring. Every quarter issues QL loads each.
    const int ld_row = lane / CPR, ld_p = lane % CPR;
    uint32_t lane_off[QL];
#pragma unroll
    for (int i = 0; i < QL; ++i) {
        const int r = RPK * i + ld_row;                  // row within the quarter
        const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
        lane_off[i] = (uint32_t)(r * a.kv_sslot + 8 * c) * 2u;
    }
    const int quarter_extent = (int)((uint32_t)(15 * a.kv_sslot) * 2u + 2u * D);
    char* const kst = Ks[par] + 16 * RB * qw;              // this wave's rows of its stage
    char* const vst = Vs[par] + 16 * RB * qw;
    const uint32_t mk = lds_addr(kst), mv = lds_addr(vst);
    // quarter of tile `tile` whose first key sits in ring slot sq (element offset so)
    auto is_fast = [&](int tile, int sq, int kcap) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * qw;
        return qb >= kmin && qb + 15 <= kcap && sq + 16 <= a.ring;
    };
    auto qdesc = [&](const uint16_t* src, int64_t so, bool use) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(src + so), (short)0, use ? quarter_extent : 0, 0x00020000);
    };
    // key qb + r clamped into [kmin, kcap] and wrapped into the ring, counted from the
    // quarter's first key clamped into that range (every clamped key lies 0 .. 15 keys after
    // it: one wrap at most in a ring of at least 16 slots)
    auto issue_edge = [&](const uint16_t* src, int tile, uint32_t m0, int kcap) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * qw;
        const int qbc = min(max(qb, kmin), kcap);
        const int sqc = ring_slot(a, qbc);
#pragma unroll
        for (int i = 0; i < QL; ++i) {
            const int r = RPK * i + ld_row;
            const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
            const int jc = min(max(qb + r, kmin), kcap);
            int slot = sqc + (jc - qbc);
            if (a.ring >= 16) slot = slot >= a.ring ? slot - a.ring : slot;
            else slot = jc % a.ring;
            lds_dma_global16(src + (int64_t)slot * a.kv_sslot + 8 * c, m0 + 1024 * i);
        }
    };
    auto issue_whole = [&](const uint16_t* src, int tile, int sq, int64_t so, uint32_t m0, int kcap) __attribute__((always_inline)) {
        if (is_fast(tile, sq, kcap)) {
            const __amdgpu_buffer_rsrc_t rs = qdesc(src, so, true);
#pragma unroll
            for (int i = 0; i < QL; ++i) lds_dma_buffer16(rs, lane_off[i], m0 + 1024 * i);
        } else {
            issue_edge(src, tile, m0, kcap);
        }
    };

    // This wave's first quarter goes out before hi is known when it lies wholly below kmax_low
    // (so no key of it is clamped at the top, and kmax >= kmax_low means it meets the range);
    // hi's latency, the tile's and q's then overlap.
    const int ta0 = t0 + ((par - t0) & 1);
    const int qb0 = ta0 * BN + 16 * qw;
    const bool early = qb0 + 15 >= kmin && qb0 + 15 <= kmax_low;
    if (early) {
        const int sq0 = ring_slot(a, qb0);
        issue_whole(vg, ta0, sq0, (int64_t)sq0 * a.kv_sslot, mv, kmax_low);
        issue_whole(kg, ta0, sq0, (int64_t)sq0 * a.kv_sslot, mk, kmax_low);
    }
    // the block's q, requested now (stored into LDS before the walk)
    uint4 qv[kQuarterPairs * CPR / kOctThreads];
#pragma unroll
    for (int k = 0; k < kQuarterPairs * CPR / kOctThreads; ++k) {
        const int i = tid + kOctThreads * k;
        const int p = i / CPR, c = i % CPR;
        const int pr = blk * kQuarterPairs + p;
        const int qrow = pr / G;
        qv[k] = *reinterpret_cast<const uint4*>(
            a.q + (int64_t)(qrow < a.n ? qrow : 0) * a.q_srow + (int64_t)(g * G + pr % G) * a.q_shead + 8 * c);
    }
    const int big = 0x7FFFFFFF;
    int lo = big, last = -1;               // empty range for padding pairs
    if (valid) prompt_span(a, row, lo, last);
    // every wave holds the same 32 pairs, so these are the workgroup's values as well; kept in
    // scalar registers so that the tile addresses and descriptors derived from them are too
    const int kmax = __builtin_amdgcn_readfirstlane(wave_max_i(last));
    const int loall = __builtin_amdgcn_readfirstlane(wave_max_i(valid ? lo : -1));
    const int lastall = __builtin_amdgcn_readfirstlane(wave_min_i(valid ? last : big));
    const int t1 = kmax / BN;

    // this wave's tiles: those of its parity (absolute tile index, so that a row's bits do not
    // depend on where a call's first block starts) that its quarter meets (keys of the
    // block's range), a contiguous run ta, ta + 2, .., tz
    auto meets = [&](int tile) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * qw;
        return qb <= kmax && qb + 15 >= kmin;
    };
    auto is_full = [&](int tile) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * qw;
        return qb >= loall && qb + 15 <= lastall;
    };
    int ta = ta0;
    if (ta <= t1 && !meets(ta)) ta += 2;
    int tz = t1 - ((t1 - par) & 1);                    // last tile of this parity
    if (tz >= ta && !meets(tz)) tz -= 2;
    const bool work = ta <= tz;
    // ring slot and element offset of the wave's current quarter, advanced two tiles at a
    // time (one wrap in a ring of at least 128 slots, a loop in a shorter one)
    int cs = ring_slot(a, ta * BN + 16 * qw);
    int64_t cso = (int64_t)cs * a.kv_sslot;
    const int64_t step_elems = (int64_t)(2 * BN) * a.kv_sslot, ring_elems = (int64_t)a.ring * a.kv_sslot;
    auto advance = [&](int& sq, int64_t& so) __attribute__((always_inline)) {
        sq += 2 * BN;
        so += step_elems;
        while (sq >= a.ring) {
            sq -= a.ring;
            so -= ring_elems;
        }
    };
    if (work && !(early && ta == ta0)) {  // the first quarter, if not out already: V, then K
        issue_whole(vg, ta, cs, cso, mv, kmax);
        issue_whole(kg, ta, cs, cso, mk, kmax);
    }

    // the block's q into LDS (a padding pair takes row 0's q: its range is empty, so every key
    // is masked); a negative scale is carried by q's sign (exact), so the exponent factor is
    // positive
    {
        const uint32_t sgn = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int k = 0; k < kQuarterPairs * CPR / kOctThreads; ++k) {
            const int i = tid + kOctThreads * k;
            const int p = i / CPR, c = i % CPR;
            *reinterpret_cast<uint4*>(Qs + p * RB + 16 * ((c & ~15) | ((c & 15) ^ (p & 15)))) =
                make_uint4(qv[k].x ^ sgn, qv[k].y ^ sgn, qv[k].z ^ sgn, qv[k].w ^ sgn);
        }
    }
    __syncthreads();

    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;  // m in log2 units (scaled score)
    const float cexp = fabsf(a.scale) * kLog2e;

    // LDS read offsets, fixed for the walk (the second half of a row's chunks, 256 bytes on).
    // K (A operand of 16x16x32): own row 16 qw + l % 16, logical chunk 4 ks + l / 16.
    // Q^T (B operand): pair 16 nb + l % 16 (nb: 16 pairs, 8 KiB on), the same chunk.
    // V^T (A operand of 32x32x16) by the transposing read: 16-lane group q = lane / 16,
    // j = lane % 16 reads row 16 qw + 8h + 4u + j / 4 at dims 32 db + 16 (q & 1) + 4 (j & 3)
    // + 0..3; the two reads (u = 0, 1) give lane l dim 32 db + l % 32 at keys 8h + 0..7.
    int koff[KS / 2], qoff[KS / 2], voff[2][DBLK / 2];
    {
        const int kr = 16 * qw + c16;
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
            const int c = 4 * ks + q4;
            koff[ks] = kr * RB + 16 * (c ^ swz(kr));
            qoff[ks] = c16 * RB + 16 * (c ^ c16);
        }
        const int j16 = lane & 15, cg = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int vr = 16 * qw + 8 * h + 4 * u + (j16 >> 2);
#pragma unroll
            for (int db = 0; db < DBLK / 2; ++db) {
                const int c = 4 * db + cg;
                voff[u][db] = vr * RB + 16 * (c ^ swz(vr)) + 8 * (j16 & 1);
            }
        }
    }

    // The walk: one quarter a tile. In flight at a quarter's start: its V (QL loads, plus QL
    // for an edge quarter), then its K (the same). V^T is read first; the next quarter's V
    // goes out during the score products (one load after each 32-dim step), its K during P.V
    // (one after each 32-dim block); descriptors with no records unless on the fast path,
    // edge quarters key by key after them.
    for (int tile = ta; work; tile += 2) {
        const bool more = tile + 2 <= tz;
        int ns = cs;
        int64_t nso = cso;
        advance(ns, nso);
        const bool nfast = more && is_fast(tile + 2, ns, kmax);

        lds_dma_wait_vm8();                // this quarter's V (its K may still be in flight)
        uint2 vx[DBLK][2];
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                vx[db][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16_ptr)(Vs[par] + voff[u][db & 3] + (db >> 2) * 256)));
        lds_wait_reads();                  // V^T read: the stage may be refilled
        lds_dma_wait_vm0();                // this quarter's K
        // S^T = K Q^T, 16 keys x 32 pairs; the next quarter's V in between
        f32x4 s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[nb][r] = 0.f;
        {
            const __amdgpu_buffer_rsrc_t nrv = qdesc(vg, nso, nfast);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Pack8 kf, qa, qb;
                const int ko = koff[ks & 3] + (ks >> 2) * 256, qo = qoff[ks & 3] + (ks >> 2) * 256;
                kf.u = *reinterpret_cast<const uint4*>(Ks[par] + ko);
                qa.u = *reinterpret_cast<const uint4*>(Qs + qo);
                qb.u = *reinterpret_cast<const uint4*>(Qs + 16 * RB + qo);
                s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.v, qa.v, s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.v, qb.v, s[1], 0, 0, 0);
                lds_dma_buffer16(nrv, lane_off[ks], mv + 1024 * ks);
            }
            if (more && !nfast) issue_edge(vg, tile + 2, mv, kmax);
        }
        lds_wait_reads();                  // K read: the stage may be refilled
        // to the P^T layout: lane l = 32a + 16b + c holds pair 16b + c; its keys 8a + i come
        // from lane 32a + c (register s[b][i]) and keys 8a + 4 + i from lane 32a + 16 + c
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0][i]), __float_as_uint(s[1][i]), false, false);
            x[i] = __uint_as_float(r[0]);
            x[4 + i] = __uint_as_float(r[1]);
        }
        // online softmax over the quarter's keys 16 qw + 8h + 0..7 of this lane's pair
        if (!is_full(tile)) {
            const int kb = tile * BN + 16 * qw + 8 * h;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (kb + j < lo || kb + j > last) x[j] = -INFINITY;
        }
        float smax = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) smax = fmaxf(smax, x[j]);
        smax = pair_max(smax);
        // lazy maximum (moves only by more than kLazy in log2 units, so p <= 2^kLazy)
        const float m_cand = fmaxf(m_run, smax * cexp);
        const bool grow = m_cand > m_run + kLazy;
        const float m_new = grow ? m_cand : m_run;
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(x[j], cexp, -mu));
            x[j] = p;
            psum += p;
        }
        // O and l are still zero while m is -inf: only rows with earlier keys rescale
        if (__any(grow && m_run != -INFINITY)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mu) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        l_run += psum;
        m_run = m_new;
        // NP bf16 parts of P: part k is the bf16 rounding of P minus parts 0..k-1
        Pack8 phi, pmid, plo;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p0 = x[2 * u], p1 = x[2 * u + 1];
            phi.w[u] = cvt_pk_bf16(p0, p1);
            if (NP == 2 && WA_CONTROL == 6) pmid.w[u] = 0u;
            else if (NP >= 2) {
                const float e0 = p0 - lo_bf16(phi.w[u]), e1 = p1 - hi_bf16(phi.w[u]);
                pmid.w[u] = cvt_pk_bf16(e0, e1);
                if (NP == 3) plo.w[u] = cvt_pk_bf16(e0 - lo_bf16(pmid.w[u]), e1 - hi_bf16(pmid.w[u]));
            }
        }
        {
            const __amdgpu_buffer_rsrc_t nrk = qdesc(kg, nso, nfast);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                Pack8 av;
                av.w[0] = vx[db][0].x;
                av.w[1] = vx[db][0].y;
                av.w[2] = vx[db][1].x;
                av.w[3] = vx[db][1].y;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, phi.v, oacc[db], 0, 0, 0);
                if (NP >= 2) oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, pmid.v, oacc[db], 0, 0, 0);
                if (NP == 3) oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, plo.v, oacc[db], 0, 0, 0);
                lds_dma_buffer16(nrk, lane_off[db], mk + 1024 * db);
            }
            if (more && !nfast) issue_edge(kg, tile + 2, mk, kmax);
        }
        if (!more) break;
        cs = ns;
        cso = nso;
    }

    // Merge of the eight states, in two halves of the dims (the eight O would not fit in LDS
    // at once). For half hh every wave stores its O of dims 128 hh .. + 127 (32 pairs x 512
    // bytes, 16-byte chunk c of pair col at c ^ (col & 15)) into the half of stage array w % 4
    // numbered w / 4, and its (m, l) into red_*; then wave w produces dims 128 hh + 16 w ..
    // + 15 of every pair: M = max m_v, a_v = 2^(m_v - M), den = sum a_v l_v, out =
    // bf16(sum (a_v / den) O_v), the sums fma chains in wave order. A (row, head) with a
    // non-finite value is flagged, not stored, and re-run below.
    const float l_tot = pair_sum(l_run);
    auto arrs = [&](int j) __attribute__((always_inline)) {
        return j == 0 ? Ks[0] : j == 1 ? Vs[0] : j == 2 ? Ks[1] : Vs[1];
    };
    auto region = [&](int w) __attribute__((always_inline)) { return arrs(w & 3) + (TILE_B / 2) * (w >> 2); };
    auto o_chunk = [&](const char* base, int c) __attribute__((always_inline)) {
        return reinterpret_cast<const float4*>(base + col * 512 + 16 * ((c & ~15) | ((c & 15) ^ (col & 15))));
    };
    __builtin_amdgcn_s_waitcnt(0);
    if (h == 0) { red_m[wave][col] = m_run; red_l[wave][col] = l_tot; }
    __syncthreads();                       // every wave is done with the stages
    float ac[kOctWaves];
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kOctWaves; ++w) M = fmaxf(M, red_m[w][col]);
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kOctWaves; ++w) {
            const float mw = red_m[w][col];
            ac[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            den = fmaf(ac[w], red_l[w][col], den);
        }
        // one division a lane instead of one per value (den = 0, a row without keys, gives
        // NaN and a float64 re-run, as 0 / 0 would)
        const float rden = 1.f / den;
#pragma unroll
        for (int w = 0; w < kOctWaves; ++w) ac[w] *= rden;
    }
    uint2 res[2][2];
    uint32_t expo = 0;                     // OR of the exponent fields: all ones = not finite
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        // O^T layout: register 4k + i of block db holds dims 32 db + 8k + 4h + i
        char* const mine = region(wave);
#pragma unroll
        for (int db = 4 * hh; db < 4 * hh + 4; ++db)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int c = ((32 * db + 8 * k + 4 * h) & 127) >> 2;
                *reinterpret_cast<float4*>(mine + col * 512 + 16 * ((c & ~15) | ((c & 15) ^ (col & 15)))) =
                    make_float4(oacc[db][4 * k], oacc[db][4 * k + 1], oacc[db][4 * k + 2], oacc[db][4 * k + 3]);
            }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = 4 * wave + 2 * h + i;              // dims 128 hh + 4c .. + 3
            float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < kOctWaves; ++w) {
                const float4 o = *o_chunk(region(w), c);
                num.x = fmaf(ac[w], o.x, num.x);
                num.y = fmaf(ac[w], o.y, num.y);
                num.z = fmaf(ac[w], o.z, num.z);
                num.w = fmaf(ac[w], o.w, num.w);
            }
            res[hh][i].x = cvt_pk_bf16(num.x, num.y);
            res[hh][i].y = cvt_pk_bf16(num.z, num.w);
            const uint32_t e0 = res[hh][i].x & 0x7F807F80u, e1 = res[hh][i].y & 0x7F807F80u;
            expo |= ((e0 & 0x7F80u) == 0x7F80u) | ((e0 >> 16) == 0x7F80u) |
                    ((e1 & 0x7F80u) == 0x7F80u) | ((e1 >> 16) == 0x7F80u);
        }
        __syncthreads();                   // the regions are read before the next half's stores
    }
    if (valid && expo) bad[col] = 1;
    __syncthreads();
    if (valid && !bad[col]) {
        uint16_t* op = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead + 16 * wave + 8 * h;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 2; ++i) *reinterpret_cast<uint2*>(op + 128 * hh + 4 * i) = res[hh][i];
    }
    // a (row, head) whose output holds a NaN or an infinity is re-run alone in float64 by the
    // whole workgroup; the flag is read from LDS by every thread, so the branch is uniform
    for (int p = 0; p < kQuarterPairs; ++p) {
        if (!bad[p]) continue;
        const int pr = blk * kQuarterPairs + p;
        const int r = pr / G, hd = g * G + pr % G;
        int rlo, rlast;
        prompt_span(a, r, rlo, rlast);
        const int64_t kv = (int64_t)g * a.kv_shead;
        rerun_f64<D>(a.q + (int64_t)r * a.q_srow + (int64_t)hd * a.q_shead, a.k + kv, a.v + kv,
                     a.kv_sslot, a.ring, rlo, rlast, a.scale,
                     a.out + (int64_t)r * a.o_srow + (int64_t)hd * a.o_shead);
        __syncthreads();
    }
}

// Launch of the quarter-tile kernel: grid = key heads x blocks of 32 pairs.
template <int NP>
hipError_t launch_quarter(const PromptArgs& b, hipStream_t s) {
    const int G = b.hq / b.hkv;
    const int nblk = (int)(((int64_t)b.n * G + kQuarterPairs - 1) / kQuarterPairs);
    hipLaunchKernelGGL((prompt_quarter_kernel<NP>), dim3((unsigned)(nblk * b.hkv)), dim3(kOctThreads), 0, s, b, nblk);
    return hipGetLastError();
}

}  // namespace
}  // namespace wa
