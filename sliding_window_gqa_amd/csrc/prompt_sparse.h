// Block-sparse prompt rows at head dim 256 on gfx950: the row-group kernel.
//
// Method: TensorFold pull request #1622, "What this changes": each row sees the keys of its
// range [lo_i, last_i] (the window and hi of pull request #1123, "window_attention at head
// dim 256", promptRows(..., hi)) that lie in a 64-key block the row selected; an fp32 online
// softmax walks the union of the selected blocks of the rows sharing a key head's tile, with
// per-row block masks and causal ends, and the parts of a row are merged in order. P enters
// P.V as one bf16, as bf16(P) + bf16(P - bf16(P)) (p32) or as three bf16 parts.
//
// Design (own): a workgroup holds up to 16 (row, query head) columns of one key head -- whole
// rows when a key head has at most 16 query heads (12 heads of one row: 12 columns), so the
// columns share one row's selection and the walk has no union of other rows' blocks to
// carry -- and one 4096-key segment at absolute positions (64 blocks, two mask words). Its
// four waves, one a SIMD, all hold the same columns; wave w takes keys 16w .. 16w + 15 of
// every selected block (its quarter) with a running (m, l, O) of its own, loading only its
// own 16 rows of K and V (double-buffered, no barrier in the walk).
//   * S^T of a quarter (16 keys x 16 columns) is one v_mfma_f32_16x16x32_bf16 product over
//     eight 32-dim steps (two chains, even and odd steps, added at the end); its
//     accumulator layout (lane l: keys 4 (l / 16) + i of column l % 16) is exactly the
//     B operand of v_mfma_f32_16x16x16bf16_1k, so P goes to P.V without a shuffle;
//   * the column's row maximum and sum span the four lanes l % 16 + 16k: one
//     v_permlane16_swap and one v_permlane32_swap step;
//   * O^T += V^T P^T: sixteen 16-dim blocks, NP products each, V^T by the transposing LDS
//     read (ds_read_b64_tr_b16); O^T holds 64 registers a lane;
//   * the next quarter's loads go out one after each score step (K) and one after every
//     other 16-dim block of P.V (V), as in prompt_quarter.h;
//   * after the walk the four states are merged in LDS in wave order (M = max m_w,
//     a_w = 2^(m_w - M), l = sum a_w l_w, o = sum a_w O_w) and written as the segment's fp32
//     partial (m in log2 units), which prompt_merge_kernel combines over the segments in
//     order, with the float64 re-run of non-finite rows. A segment holding none of a row's
//     selected keys writes no partial for it (the merge applies the same rule).
// A row's bits depend only on its range, its selection, the absolute block and segment grid
// and the quarter split, never on the other rows of its call or on how the prompt is cut.
#pragma once

#include "prompt_quarter.h"

namespace wa {

namespace {

constexpr int kRowCols = 16;           // (row, head) columns per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int ctz64(uint64_t x) { return __builtin_ctzll(x); }

template <int NP>
__global__ __launch_bounds__(kThreads, 1) void prompt_rows_kernel(PromptArgs a, int nrg, int nhg, int nseg) {
    constexpr int D = 256;
    constexpr int KS = D / 32;             // 32-dim steps of S^T
    constexpr int DB = D / 16;             // 16-dim blocks of O^T
    constexpr int RB = 2 * D;              // bytes per K/V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPK = 1024 / RB;         // rows per 1 KiB wave load
    constexpr int TILE_B = BN * RB;        // bytes of one K (or V) tile
    constexpr int QL = 16 * RB / 1024;     // wave loads per quarter (each of K and V)
    constexpr int SEGB = kSparseSeg / kSparseBlock;   // blocks a segment (one or two mask words)
    static_assert(SEGB == 32 || SEGB == 64, "a segment is one or two whole mask words");
    static_assert(QL == KS && 2 * QL == DB, "one K load per score step, one V load per two O blocks");
    // two stages of K and V; wave w owns rows 16w .. 16w + 15 of each (8 KiB an array)
    __shared__ __attribute__((aligned(1024))) char Ks0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Ks1[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs1[TILE_B];
    __shared__ float red_m[kWaves][kRowCols];
    __shared__ float red_l[kWaves][kRowCols];

    // XCD x takes a contiguous share of the logical ids (key head, segment, row group, head
    // group): an XCD's workgroups read one head's K and V over one segment (4096 keys, 4 MiB
    // at d = 256), which its L2 can hold while their selections revisit it
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int per = total >> 3, extra = total & 7;
    int logical = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
    const int hgi = logical % nhg;
    logical /= nhg;
    const int rg = logical % nrg;
    logical /= nrg;
    const int sidx = logical % nseg;
    const int g = logical / nseg;          // key head

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15;             // column of the 16x16 layouts
    const int q4 = lane >> 4;              // lane group: keys 4 q4 .. 4 q4 + 3 of a quarter
    const int G = a.hq / a.hkv;
    const int HG = G <= kRowCols ? G : kRowCols;         // heads a row contributes
    const int RG = G <= kRowCols ? kRowCols / G : 1;     // rows a workgroup holds

    const int row = rg * RG + c16 / HG;
    const int hin = hgi * kRowCols + c16 % HG;
    const bool valid = c16 < RG * HG && row < a.n && hin < G;
    const int head = g * G + (hin < G ? hin : 0);

    const int big = 0x7FFFFFFF;
    int lo = big, last = -1;
    if (valid) prompt_span(a, row, lo, last);
    const int kmin0 = __builtin_amdgcn_readfirstlane(wave_min_i(lo));
    const int kmax0 = __builtin_amdgcn_readfirstlane(wave_max_i(last));
    if (kmax0 < kmin0) return;             // no valid column (uniform: all waves alike)
    // this workgroup's segment of the key range, at absolute positions
    const int seg = kmin0 / kSparseSeg + sidx;
    const int kmin = max(kmin0, seg * kSparseSeg);
    const int kmax = min(kmax0, seg * kSparseSeg + kSparseSeg - 1);
    if (kmax < kmin) return;
    // this lane's row: its selected blocks of the segment that meet its range (bit i = block
    // SEGB seg + i); the walk takes the union over the columns
    uint64_t eff = 0;
    if (valid) {
        const uint32_t* brow = a.bm + (int64_t)row * a.bm_srow;
        const int w0 = SEGB / 32 * seg;
        const uint32_t lw = w0 < a.bm_words ? brow[w0] : 0u;
        const uint32_t hw = SEGB == 64 && w0 + 1 < a.bm_words ? brow[w0 + 1] : 0u;
        eff = ((uint64_t)hw << 32) | lw;
        const int b_lo = lo / kSparseBlock - SEGB * seg, b_hi = last / kSparseBlock - SEGB * seg;
        if (b_hi < 0 || b_lo > SEGB - 1) eff = 0;
        else {
            if (b_lo > 0) eff &= ~0ull << b_lo;
            if (b_hi < 63) eff &= ~0ull >> (63 - b_hi);
        }
    }
    uint32_t ulo = (uint32_t)eff, uhi = (uint32_t)(eff >> 32);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        ulo |= (uint32_t)__shfl_xor((int)ulo, m, 64);
        uhi |= (uint32_t)__shfl_xor((int)uhi, m, 64);
    }
    const uint64_t tiles = ((uint64_t)__builtin_amdgcn_readfirstlane(uhi) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane(ulo);
    if (tiles == 0) return;                // no column selected a block here (uniform)
    const int tb0 = SEGB * seg;            // absolute index of the segment's first block

    const uint16_t* kg = a.k + (int64_t)g * a.kv_shead;
    const uint16_t* vg = a.v + (int64_t)g * a.kv_shead;

    // quarter loads (own rows), as in prompt_quarter.h
    const int ld_row = lane / CPR, ld_p = lane % CPR;
    uint32_t lane_off[QL];
#pragma unroll
    for (int i = 0; i < QL; ++i) {
        const int r = RPK * i + ld_row;
        const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
        lane_off[i] = (uint32_t)(r * a.kv_sslot + 8 * c) * 2u;
    }
    const int quarter_extent = (int)((uint32_t)(15 * a.kv_sslot) * 2u + 2u * D);
    auto is_fast = [&](int tile) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        return qb >= kmin && qb + 15 <= kmax && qb % a.ring + 16 <= a.ring;
    };
    auto qdesc = [&](int tile, const uint16_t* src, bool use) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        const int sq = qb % a.ring;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(src + (int64_t)sq * a.kv_sslot), (short)0,
                                                 use && is_fast(tile) ? quarter_extent : 0, 0x00020000);
    };
    // a whole quarter, key by key (clamped into [kmin, kmax], wrapped into the ring), K's first.
    // A selected tile may hold quarters wholly below kmin or above kmax; the slot is counted
    // from the quarter's first key clamped into [kmin, kmax], so that every clamped key lies
    // 0 .. 15 keys after it (one wrap at most in a ring of at least 16 slots).
    auto issue_edge = [&](int tile, char* kdst, char* vdst) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        const int qbc = min(max(qb, kmin), kmax);
        const int sqc = qbc % a.ring;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int i = 0; i < QL; ++i) {
                const int r = RPK * i + ld_row;
                const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
                const int jc = min(max(qb + r, kmin), kmax);
                int slot = sqc + (jc - qbc);
                if (a.ring >= 16) slot = slot >= a.ring ? slot - a.ring : slot;
                else slot = jc % a.ring;
                const uint16_t* src = half ? vg : kg;
                char* dst = (half ? vdst : kdst) + 16 * RB * wave + 1024 * i;
                __builtin_amdgcn_global_load_lds(src + (int64_t)slot * a.kv_sslot + 8 * c,
                                                 (lds_void_ptr)dst, 16, 0, 0);
            }
    };
    auto issue_fast = [&](int tile, char* kdst, char* vdst) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rk = qdesc(tile, kg, true), rv = qdesc(tile, vg, true);
#pragma unroll
        for (int i = 0; i < QL; ++i) buffer_to_lds16(rk, kdst + 16 * RB * wave + 1024 * i, lane_off[i]);
#pragma unroll
        for (int i = 0; i < QL; ++i) buffer_to_lds16(rv, vdst + 16 * RB * wave + 1024 * i, lane_off[i]);
    };
    auto issue_whole = [&](int tile, char* kdst, char* vdst) __attribute__((always_inline)) {
        if (is_fast(tile)) issue_fast(tile, kdst, vdst);
        else issue_edge(tile, kdst, vdst);
    };

    uint64_t rem = tiles;
    int cur = tb0 + ctz64(rem);
    rem &= rem - 1;
    issue_whole(cur, Ks0, Vs0);

    // Q^T operand of the score product: lane l holds column l % 16 at dims 32 ks + 8 (l / 16)
    // + 0..7 (a padding column takes a valid row's q; its scores are never used)
    Pack8 qreg[KS];
    {
        const uint16_t* qp = a.q + (int64_t)(valid ? row : 0) * a.q_srow + (int64_t)head * a.q_shead + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks].u = *reinterpret_cast<const uint4*>(qp + 32 * ks);
    }
    if (a.scale < 0.f) {
        // a negative scale is carried by q's sign (exact), so the exponent factor is positive
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks].u.x ^= 0x80008000u; qreg[ks].u.y ^= 0x80008000u;
            qreg[ks].u.z ^= 0x80008000u; qreg[ks].u.w ^= 0x80008000u;
        }
    }

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;  // m in log2 units (scaled score)
    const float cexp = fabsf(a.scale) * kLog2e;

    // LDS read offsets within a tile. K (A operand of 16x16x32): row 16 wave + l % 16, logical
    // chunk 4 ks + l / 16. V^T (A operand of 16x16x16) by the transposing read: 16-lane group
    // q4 reads rows 16 wave + 4 q4 + j / 4 at dims 16 db + 4 (j & 3) + 0..3 (j = lane % 16),
    // which gives lane l dim 16 db + l % 16 at keys 4 q4 + 0..3.
    int koff[KS], voff[DB];
    {
        const int kr = 16 * wave + c16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 4 * ks + q4;
            koff[ks] = kr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(kr)));
        }
        const int vr = 16 * wave + 4 * q4 + (c16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int c = 2 * db + ((c16 & 3) >> 1);
            voff[db] = vr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(vr))) + 8 * (c16 & 1);
        }
    }

    // max and sum over the four lanes l % 16 + 16 k of a column (the same bits on all four)
    auto col_max = [](float x) __attribute__((always_inline)) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return pair_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
    };
    auto col_sum = [](float x) __attribute__((always_inline)) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
    };

    // one quarter of block `tile` from stages kt / vt; the next quarter's loads (descriptors
    // with no records unless it is on the fast path) go out in between; waits as in
    // prompt_quarter.h: this quarter's K with all but the last QL loads landed, its V with all
    // but the next quarter's QL K loads
    auto quarter = [&](int tile, bool nxt, int ntile, const char* kt, const char* vt, char* kn, char* vn)
        __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t nrk = qdesc(ntile, kg, nxt), nrv = qdesc(ntile, vg, nxt);
        char* const nkd = kn + 16 * RB * wave;
        char* const nvd = vn + 16 * RB * wave;
        __builtin_amdgcn_s_waitcnt(kWaitVm8);
        f32x4 s0, s1;
#pragma unroll
        for (int r = 0; r < 4; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
        Pack8 ka[2];
        ka[0].u = *reinterpret_cast<const uint4*>(kt + koff[0]);
        ka[1].u = *reinterpret_cast<const uint4*>(kt + koff[1]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const Pack8 c = ka[ks & 1];
            if (ks + 2 < KS) ka[ks & 1].u = *reinterpret_cast<const uint4*>(kt + koff[ks + 2]);
            if (ks & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.v, qreg[ks].v, s1, 0, 0, 0);
            else s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.v, qreg[ks].v, s0, 0, 0, 0);
            buffer_to_lds16(nrk, nkd + 1024 * ks, lane_off[ks]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm8);          // this quarter's V
        uint2 vx[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
            vx[db] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16_ptr)(vt + voff[db])));
        // online softmax over keys 16w + 4 q4 + 0..3 of this lane's column
        float x[4];
        const int kb = tile * BN + 16 * wave + 4 * q4;
        const bool sel = (eff >> (tile - tb0)) & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = s0[i] + s1[i];
            if (!sel || kb + i < lo || kb + i > last) x[i] = -INFINITY;
        }
        const float smax = col_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float m_cand = fmaxf(m_run, smax * cexp);
        const bool grow = m_cand > m_run + kLazy;
        const float m_new = grow ? m_cand : m_run;
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(x[i], cexp, -mu));
            x[i] = p;
            psum += p;
        }
        if (__any(grow && m_run != -INFINITY)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mu) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
        }
        l_run += psum;
        m_run = m_new;
        // NP bf16 parts of P (B operand: keys 4 q4 + 0..3 of column l % 16)
        uint2 phi, pmid, plo;
        {
            phi.x = cvt_pk_bf16(x[0], x[1]);
            phi.y = cvt_pk_bf16(x[2], x[3]);
            if (NP == 2 && WA_CONTROL == 6) { pmid.x = 0u; pmid.y = 0u; }
            else if (NP >= 2) {
                const float e0 = x[0] - lo_bf16(phi.x), e1 = x[1] - hi_bf16(phi.x);
                const float e2 = x[2] - lo_bf16(phi.y), e3 = x[3] - hi_bf16(phi.y);
                pmid.x = cvt_pk_bf16(e0, e1);
                pmid.y = cvt_pk_bf16(e2, e3);
                if (NP == 3) {
                    plo.x = cvt_pk_bf16(e0 - lo_bf16(pmid.x), e1 - hi_bf16(pmid.x));
                    plo.y = cvt_pk_bf16(e2 - lo_bf16(pmid.y), e3 - hi_bf16(pmid.y));
                }
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const s16x4 av = __builtin_bit_cast(s16x4, vx[db]);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, phi), oacc[db], 0, 0, 0);
            if (NP >= 2)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, pmid), oacc[db], 0, 0, 0);
            if (NP == 3)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, plo), oacc[db], 0, 0, 0);
            if (db & 1) buffer_to_lds16(nrv, nvd + 1024 * (db >> 1), lane_off[db >> 1]);
        }
#pragma unroll
        for (int db = 0; db < DB; db += 2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * NP, 1);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
        }
    };

    // walk the selected blocks in ascending order, two at a time over fixed stage arrays
    auto step = [&](const char* kt, const char* vt, char* kn, char* vn) __attribute__((always_inline)) {
        const bool more = rem != 0;
        const int nxt = more ? tb0 + ctz64(rem) : cur;
        const bool fast = more && is_fast(nxt);
        quarter(cur, fast, nxt, kt, vt, kn, vn);
        if (more && !fast) issue_edge(nxt, kn, vn);
        rem &= rem - 1;
        cur = nxt;
        return more;
    };
    for (;;) {
        if (!step(Ks0, Vs0, Ks1, Vs1)) break;
        if (!step(Ks1, Vs1, Ks0, Vs0)) break;
    }

    // merge of the four quarters' states: wave w stores its O into its own rows of Ks0 (dims
    // 0..127) and Vs0 (dims 128..255), column-major rows of 128 floats, the 16-byte chunk c of
    // column p at c ^ (p & 15)
    const float l_tot = col_sum(l_run);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d0 = 16 * db + 4 * q4;                  // dims d0 .. d0 + 3
        const int c = (d0 & 127) >> 2;
        float* ob = reinterpret_cast<float*>((d0 < 128 ? Ks0 : Vs0) + 16 * RB * wave) + c16 * 128;
        *reinterpret_cast<float4*>(ob + 4 * (c ^ c16)) =
            make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    }
    if (q4 == 0) { red_m[wave][c16] = m_run; red_l[wave][c16] = l_tot; }
    lds_barrier();
    // wave w combines dims 64w + 16 q4 + 0..15 of column c16 and writes the segment's partial
    // of a column whose row has selected keys here
    if (!valid || eff == 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][c16]);
    float ac[kWaves], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float mw = red_m[w][c16];
        ac[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        lsum = fmaf(ac[w], red_l[w][c16], lsum);
    }
    const int pos = __builtin_amdgcn_readfirstlane(wave);
    const char* const half = pos < 2 ? Ks0 : Vs0;         // dims 64w.. lie in this array
    const int64_t pi = ((int64_t)row * a.hq + head) * a.Cp + (seg - lo / kSparseSeg);
    if (q4 == 0) { a.pm[pi] = M; a.pl[pi] = lsum; }
    float* op = a.po + pi * D + 64 * wave + 16 * q4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = ((64 * wave + 16 * q4) & 127) / 4 + i;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float4 v = *reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(half + 16 * RB * w) + c16 * 128 + 4 * (c ^ c16));
            o.x = fmaf(ac[w], v.x, o.x);
            o.y = fmaf(ac[w], v.y, o.y);
            o.z = fmaf(ac[w], v.z, o.z);
            o.w = fmaf(ac[w], v.w, o.w);
        }
        *reinterpret_cast<float4*>(op + 4 * i) = o;
    }
}

// Launch of the row-group kernel for a block-sparse prompt at d = 256 (the caller's args with
// the segment chunking): grid = key heads x row groups x head groups x segments.
template <int NP>
hipError_t launch_rows(const PromptArgs& b, hipStream_t s) {
    const int G = b.hq / b.hkv;
    const int RG = G <= kRowCols ? kRowCols / G : 1;
    const int nhg = G <= kRowCols ? 1 : (G + kRowCols - 1) / kRowCols;
    const int nrg = (b.n + RG - 1) / RG;
    const int nseg = b.nchunk;
    const int64_t grid = (int64_t)b.hkv * nrg * nhg * nseg;
    hipLaunchKernelGGL((prompt_rows_kernel<NP>), dim3((unsigned)grid), dim3(kThreads), 0, s, b, nrg, nhg, nseg);
    return hipGetLastError();
}

}  // namespace
}  // namespace wa
