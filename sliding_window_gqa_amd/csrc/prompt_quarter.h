// Dense prompt rows at head dim 256 on gfx950: the quarter-tile kernel.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Prompt, Window.p32 and promptRows(..., hi) bullets, as in
// prompt_impl.h: each row i sees keys [lo_i, last_i], keys come in tiles at absolute
// positions, every tile folds into a running (m, l, O) with one rescale, P enters P.V as one
// bf16, as bf16(P) + bf16(P - bf16(P)) (p32), or as three bf16 parts.
//
// Design (own): a workgroup holds 32 (row, query head) pairs of one key head and four waves,
// one per SIMD. All four waves hold the same 32 pairs; they share every 64-key K/V tile in
// LDS and wave w takes the keys 16w .. 16w + 15 of each tile (its quarter), with a running
// (m, l, O) of its own over its quarters. After the last tile the four states are merged in
// LDS in wave order: M = max m_w, a_w = 2^(m_w - M), den = sum a_w l_w, out =
// bf16(sum (a_w / den) O_w), the sums fma chains in w order. So every row is finished inside its workgroup: no fp32
// partials leave the CU and no merge kernel follows; a (row, head) whose bf16 output is not
// finite is re-run in float64 by the same workgroup (rerun_f64.h), so no check kernel
// follows either. A row's bits depend only on its key
// range and the absolute tile grid (a quarter holding none of the row's keys leaves that
// row's state exactly unchanged), never on how the prompt is cut into calls.
//   * S^T of a quarter (16 keys x 32 pairs) is two v_mfma_f32_16x16x32_bf16 chains (pairs
//     0..15 and 16..31) over eight 32-dim steps; K fragments are 16-byte LDS reads, the Q^T
//     operand stays in registers for the whole walk;
//   * one v_permlane16_swap per accumulator register moves the scores into the layout of
//     the P^T operand of v_mfma_f32_32x32x16_bf16: lane l then holds pair l % 32 and keys
//     8 (l / 32) .. + 7 of the quarter, so the mask, the row maximum (one v_permlane32_swap
//     between the two lane halves), the exponentials and the O rescale are lane-local, as in
//     the 128-pair kernel;
//   * O^T += V^T P^T over the quarter's 16 keys: eight 32-dim blocks, NP MFMAs each, V^T from
//     the transposing LDS read (ds_read_b64_tr_b16);
//   * tiles are fetched by buffer loads straight into double-buffered LDS (one barrier a
//     tile), with the 16-byte-chunk swizzle and the ring wrap of the 128-pair kernel;
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

template <int NP>
__global__ __launch_bounds__(kThreads, 1) void prompt_quarter_kernel(PromptArgs a, int nblk) {
    constexpr int D = 256;
    constexpr int KS = D / 32;             // 32-dim steps of S^T
    constexpr int DBLK = D / 32;           // 32-dim blocks of O^T
    constexpr int RB = 2 * D;              // bytes per K/V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPK = 1024 / RB;         // rows per 1 KiB wave load
    constexpr int TILE_B = BN * RB;        // bytes of one K (or V) tile
    // two stages of K and V tiles (distinct arrays: the compiler can tell the direct-to-LDS
    // loads into one stage from the reads of the other); after the walk wave w's O goes to
    // array w (32 pairs x 256 dims x 4 bytes = one tile)
    __shared__ __attribute__((aligned(1024))) char Ks0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Ks1[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs1[TILE_B];
    __shared__ float red_m[kWaves][kQuarterPairs];
    __shared__ float red_l[kWaves][kQuarterPairs];
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
    const int h = lane >> 5;               // lane half: keys 8h .. 8h + 7 of a quarter
    const int col = lane & 31;             // pair of the P^T / O^T layout
    const int G = a.hq / a.hkv;

    const int pair = blk * kQuarterPairs + col;
    const int row = pair / G;
    const int head = g * G + pair % G;
    const bool valid = row < a.n;

    // The block's key range before hi is known: lo is non-decreasing in the row, so the first
    // valid row gives kmin; every valid row's last key is at least its own position, so the
    // last valid row's position is a lower bound of kmax.
    const int row_first = blk * kQuarterPairs / G;
    const int row_last = min(a.n - 1, (blk * kQuarterPairs + kQuarterPairs - 1) / G);
    const bool any_valid = row_first < a.n;
    const int kmin = prompt_lo(a, row_first);
    const int kmax_low = a.p0 + row_last;

    const uint16_t* kg = a.k + (int64_t)g * a.kv_shead;
    const uint16_t* vg = a.v + (int64_t)g * a.kv_shead;

    // Tile loads: wave w loads only its own quarter, rows 16w .. 16w + 15 of K and V (the rows
    // no other wave reads), as QL 1 KiB wave loads each (RPK rows of CPR chunks), K's before
    // V's. A quarter with every key inside [kmin, kcap] and no ring wrap goes by buffer loads
    // from a descriptor on its first slot; an edge quarter key by key, clamped into
    // [kmin, kcap] (keys the ring holds; keys outside a row's range are masked) and wrapped
    // into the ring.
    constexpr int QL = 16 * RB / 1024;     // wave loads per quarter (each of K and V)
    const int ld_row = lane / CPR, ld_p = lane % CPR;
    uint32_t lane_off[QL];
#pragma unroll
    for (int i = 0; i < QL; ++i) {
        const int r = RPK * i + ld_row;                  // row within the quarter
        const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
        lane_off[i] = (uint32_t)(r * a.kv_sslot + 8 * c) * 2u;
    }
    const int quarter_extent = (int)((uint32_t)(15 * a.kv_sslot) * 2u + 2u * D);
    struct QLoad {
        bool fast;
        __amdgpu_buffer_rsrc_t rk, rv;
        int qb, sq, kcap;
        char* kd;
        char* vd;
    };
    // a quarter whose first key's ring slot sq and element offset so = sq * kv_sslot are known
    auto prep_at = [&](int tile, int sq, int64_t so, char* kdst, char* vdst, int kcap) __attribute__((always_inline)) {
        QLoad L;
        L.qb = tile * BN + 16 * wave;
        L.sq = sq;
        L.kcap = kcap;
        L.kd = kdst + 16 * RB * wave;
        L.vd = vdst + 16 * RB * wave;
        L.fast = L.qb >= kmin && L.qb + 15 <= kcap && L.sq + 16 <= a.ring;
        L.rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kg + so), (short)0, quarter_extent, 0x00020000);
        L.rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vg + so), (short)0, quarter_extent, 0x00020000);
        return L;
    };
    auto prep = [&](int tile, char* kdst, char* vdst, int kcap) __attribute__((always_inline)) {
        const int sq = ring_slot(a, tile * BN + 16 * wave);
        return prep_at(tile, sq, (int64_t)sq * a.kv_sslot, kdst, vdst, kcap);
    };
    // wave load i of K (v = false) or V (v = true) of a prepared quarter
    auto part = [&](const QLoad& L, int i, bool v) __attribute__((always_inline)) {
        char* const dst = (v ? L.vd : L.kd) + 1024 * i;
        if (L.fast) {
            buffer_to_lds16(v ? L.rv : L.rk, dst, lane_off[i]);
            return;
        }
        const int r = RPK * i + ld_row;
        const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
        const int jc = min(max(L.qb + r, kmin), L.kcap);
        // jc - qb < 16: a ring of at least 16 slots wraps at most once inside a quarter, a
        // shorter ring may wrap several times
        int slot = L.sq + (jc - L.qb);
        if (a.ring >= 16) slot = slot >= a.ring ? slot - a.ring : slot;
        else slot = jc % a.ring;
        __builtin_amdgcn_global_load_lds((v ? vg : kg) + (int64_t)slot * a.kv_sslot + 8 * c,
                                         (lds_void_ptr)dst, 16, 0, 0);
    };
    static_assert(QL == KS && QL == DBLK, "one K load per score step, one V load per O block");
    auto issue_all = [&](const QLoad& L) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < QL; ++i) part(L, i, false);
#pragma unroll
        for (int i = 0; i < QL; ++i) part(L, i, true);
    };

    // hi (if any) is loaded first, then this wave's first quarter when it lies below kmax_low
    // (so it needs no hi), then q: the three latencies overlap
    const int big = 0x7FFFFFFF;
    int lo = big, last = -1;               // empty range for padding pairs
    if (valid) prompt_span(a, row, lo, last);
    const int t0 = kmin / BN;
    const int qb0 = t0 * BN + 16 * wave;
    const bool early = any_valid && qb0 + 15 >= kmin && qb0 + 15 <= kmax_low;
    if (early) issue_all(prep(t0, Ks0, Vs0, kmax_low));

    // Q^T operand of the 16x16x32 products: lane l holds pair 16 nb + l % 16 at dims
    // 32 ks + 8 (l / 16) + 0..7; a padding pair takes row 0's q (its column of S^T is never
    // used: its range is empty, so every key is masked)
    Pack8 qreg[2][KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int pr = blk * kQuarterPairs + 16 * nb + (lane & 15);
        const int qrow = pr / G;
        const uint16_t* qp = a.q + (int64_t)(qrow < a.n ? qrow : 0) * a.q_srow +
                             (int64_t)(g * G + pr % G) * a.q_shead + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[nb][ks].u = *reinterpret_cast<const uint4*>(qp + 32 * ks);
    }

    // every wave holds the same 32 pairs, so these are the workgroup's values as well; they
    // are the same on every lane, and kept in scalar registers so that the tile addresses and
    // buffer descriptors derived from them are scalar too
    const int kmax = __builtin_amdgcn_readfirstlane(wave_max_i(last));
    if (!any_valid) return;                // no valid pair in this workgroup (uniform, no loads)
    const int loall = __builtin_amdgcn_readfirstlane(wave_max_i(valid ? lo : -1));
    const int lastall = __builtin_amdgcn_readfirstlane(wave_min_i(valid ? last : big));
    const int t1 = kmax / BN;

    // this wave's quarter of a tile: does it meet the workgroup's keys, and does every valid
    // pair see all of it (no mask)?
    auto meets = [&](int tile) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        return qb <= kmax && qb + 15 >= kmin;
    };
    auto is_full = [&](int tile) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        return qb >= loall && qb + 15 <= lastall;
    };
    if (!early && meets(t0)) issue_all(prep(t0, Ks0, Vs0, kmax));

    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;  // m in log2 units (scaled score)
    const float cexp = fabsf(a.scale) * kLog2e;

    // LDS read offsets within a tile, fixed for the walk.
    // K (A operand of 16x16x32): row 16 wave + l % 16, logical chunk 4 ks + l / 16.
    int koff[KS];
    {
        const int kr = 16 * wave + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 4 * ks + (lane >> 4);
            koff[ks] = kr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(kr)));
        }
    }
    // V^T (A operand of 32x32x16) by the transposing read: 16-lane group q = lane / 16,
    // j = lane % 16 reads row 16 wave + 8h + 4u + j / 4 at dims 32 db + 16 (q & 1) + 4 (j & 3)
    // + 0..3; the two reads (u = 0, 1) give lane l dim 32 db + l % 32 at keys 8h + 0..7.
    int voff[2][DBLK];
    {
        const int j16 = lane & 15, cg = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int vr = 16 * wave + 8 * h + 4 * u + (j16 >> 2);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const int c = 4 * db + cg;
                voff[u][db] = vr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(vr))) + 8 * (j16 & 1);
            }
        }
    }

    // one quarter: S^T, softmax, O^T += V^T P^T. On entry this quarter's QL K and QL V loads
    // may be in flight (K's first) and nothing after them. The next quarter's loads are
    // issued inside, one after each 32-dim step of the score products (K) and one after each
    // 32-dim block of P.V (V): the load path takes one at a time while the products run,
    // instead of the wave stalling on a batch. nxt: the next quarter is on the fast path.
    auto quarter = [&](bool nxt, int64_t nso, int tile, const char* kt, const char* vt, char* knext, char* vnext)
        __attribute__((always_inline)) {
        // descriptors of the next quarter's K and V (element offset nso of its first slot):
        // with no records when it is not on the fast path (those loads then touch no memory),
        // so that every quarter issues the same loads at the same places and waits the same way
        const int nrec = nxt ? quarter_extent : 0;
        const __amdgpu_buffer_rsrc_t nrk = __builtin_amdgcn_make_buffer_rsrc((void*)(kg + nso), (short)0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t nrv = __builtin_amdgcn_make_buffer_rsrc((void*)(vg + nso), (short)0, nrec, 0x00020000);
        char* const nkd = knext + 16 * RB * wave;
        char* const nvd = vnext + 16 * RB * wave;
        __builtin_amdgcn_s_waitcnt(kWaitVm8);          // this quarter's K (its V may fly)
        // S^T = K Q^T, 16 keys x 32 pairs; K fragments two steps ahead
        f32x4 s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[nb][r] = 0.f;
        Pack8 ka[2];
        ka[0].u = *reinterpret_cast<const uint4*>(kt + koff[0]);
        ka[1].u = *reinterpret_cast<const uint4*>(kt + koff[1]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const Pack8 cur = ka[ks & 1];
            if (ks + 2 < KS) ka[ks & 1].u = *reinterpret_cast<const uint4*>(kt + koff[ks + 2]);
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.v, qreg[0][ks].v, s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.v, qreg[1][ks].v, s[1], 0, 0, 0);
            buffer_to_lds16(nrk, nkd + 1024 * ks, lane_off[ks]);   // next quarter's K
        }
        // keep that order: the first two K reads, then per step two products, the next K read
        // and one load of the next quarter
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm8);          // this quarter's V
        uint2 vx[DBLK][2];
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                vx[db][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16_ptr)(vt + voff[u][db])));
        // to the P^T layout: lane l = 32a + 16b + c holds pair 16b + c; its keys 8a + i come
        // from lane 32a + c (register s[b][i]) and keys 8a + 4 + i from lane 32a + 16 + c
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0][i]), __float_as_uint(s[1][i]), false, false);
            x[i] = __uint_as_float(r[0]);
            x[4 + i] = __uint_as_float(r[1]);
        }
        // online softmax over the quarter's keys 16w + 8h + 0..7 of this lane's pair
        if (!is_full(tile)) {
            const int kb = tile * BN + 16 * wave + 8 * h;
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
            buffer_to_lds16(nrv, nvd + 1024 * db, lane_off[db]);   // next quarter's V
        }
        // keep that order: per 32-dim block its NP products, then one load of the next quarter
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            __builtin_amdgcn_sched_group_barrier(0x008, NP, 1);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
        }
    };

    // one tile of this wave (no barrier: a wave reads only the rows it loaded itself): the
    // quarter loads the next quarter on the fast path itself; an edge next quarter (the ends
    // of the range, a ring wrap), or the next quarter of a tile this wave skips, is issued
    // whole afterwards
    //
    // ns, nso: ring slot and element offset of this wave's quarter of the tile after the
    // current one, advanced a tile at a time (one wrap per tile in a ring of at least 64
    // slots, a loop in a shorter one) instead of a remainder and a product per tile
    int ns = ring_slot(a, (t0 + 1) * BN + 16 * wave);
    int64_t nso = (int64_t)ns * a.kv_sslot;
    const int64_t tile_elems = (int64_t)BN * a.kv_sslot, ring_elems = (int64_t)a.ring * a.kv_sslot;
    auto step = [&](int tile, const char* kt, const char* vt, char* knext, char* vnext, bool more) {
        const bool nxt = more && meets(tile + 1);
        const bool fast = nxt && prep_at(tile + 1, ns, nso, knext, vnext, kmax).fast;
        const bool here = meets(tile);
        if (here) quarter(fast, nso, tile, kt, vt, knext, vnext);
        if (nxt && !(here && fast)) issue_all(prep_at(tile + 1, ns, nso, knext, vnext, kmax));
        ns += BN;
        nso += tile_elems;
        while (ns >= a.ring) {
            ns -= a.ring;
            nso -= ring_elems;
        }
    };

    if (a.scale < 0.f) {
        // a negative scale is carried by q's sign (exact), so the exponent factor is positive
        // (a branch, so that a positive scale does not wait for the q loads here)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qreg[nb][ks].u.x ^= 0x80008000u; qreg[nb][ks].u.y ^= 0x80008000u;
                qreg[nb][ks].u.z ^= 0x80008000u; qreg[nb][ks].u.w ^= 0x80008000u;
            }
    }
    for (int t = t0; t <= t1; t += 2) {
        step(t, Ks0, Vs0, Ks1, Vs1, t + 1 <= t1);
        if (t + 1 <= t1) step(t + 1, Ks1, Vs1, Ks0, Vs0, t + 2 <= t1);
    }
    // merge of the four quarters' states. A wave's own rows of the four stage arrays (rows
    // 16w .. 16w + 15 of every tile, 8 KiB in each) are touched by no other wave and hold
    // exactly its O: once its own loads have landed it stores O there without waiting for
    // the other waves, dims 64j .. 64j + 63 into array j (pair-major, 256 bytes a pair, the
    // 16-byte chunk c of pair p at c ^ (p & 15)), and (m, l) into red_*.
    const float l_tot = pair_sum(l_run);
    char* const arrs[kWaves] = {Ks0, Vs0, Ks1, Vs1};
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * h;        // dims d0 .. d0 + 3
            const int c = (d0 & 63) >> 2;                   // chunk within the 64-dim block
            float* ob = reinterpret_cast<float*>(arrs[d0 >> 6] + 16 * RB * wave) + col * 64;
            *reinterpret_cast<float4*>(ob + 4 * (c ^ (col & 15))) =
                make_float4(oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]);
        }
    if (h == 0) { red_m[wave][col] = m_run; red_l[wave][col] = l_tot; }
    lds_barrier();
    // wave w produces dims 64w + 32h + 0..31 of pair col from array w; a (row, head) with a
    // non-finite value is flagged before any of its values is stored, and re-run below instead
    const char* const mine = wave == 0 ? Ks0 : wave == 1 ? Vs0 : wave == 2 ? Ks1 : Vs1;
    uint2 res[8];
    if (valid) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][col]);
        float ac[kWaves], den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = red_m[w][col];
            ac[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            den = fmaf(ac[w], red_l[w][col], den);
        }
        // out = sum_w (a_w / den) O_w: one division a lane instead of one per value (den = 0,
        // a row without keys, gives NaN and a float64 re-run, as 0 / 0 would)
        const float rden = 1.f / den;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ac[w] *= rden;
        uint32_t expo = 0;                 // OR of the exponent fields: all ones = not finite
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * h + i;                         // dims 64 wave + 4c .. + 3
            float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float4 o = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(mine + 16 * RB * w) + col * 64 + 4 * (c ^ (col & 15)));
                num.x = fmaf(ac[w], o.x, num.x);
                num.y = fmaf(ac[w], o.y, num.y);
                num.z = fmaf(ac[w], o.z, num.z);
                num.w = fmaf(ac[w], o.w, num.w);
            }
            res[i].x = cvt_pk_bf16(num.x, num.y);
            res[i].y = cvt_pk_bf16(num.z, num.w);
            const uint32_t e0 = res[i].x & 0x7F807F80u, e1 = res[i].y & 0x7F807F80u;
            expo |= ((e0 & 0x7F80u) == 0x7F80u) | ((e0 >> 16) == 0x7F80u) |
                    ((e1 & 0x7F80u) == 0x7F80u) | ((e1 >> 16) == 0x7F80u);
        }
        if (expo) bad[col] = 1;
    }
    lds_barrier();
    if (valid && !bad[col]) {
        uint16_t* op = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead + 64 * wave + 32 * h;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint2*>(op + 4 * i) = res[i];
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
    hipLaunchKernelGGL((prompt_quarter_kernel<NP>), dim3((unsigned)(nblk * b.hkv)), dim3(kThreads), 0, s, b, nblk);
    return hipGetLastError();
}

}  // namespace
}  // namespace wa
