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
// every selected block (its quarter) with a running (m, l, O) of its own, and walks the
// selected blocks two at a time (a and b; b absent at an odd end):
//   * K goes into LDS (one stage a block) by buffer_load ... lds and is read back in the
//     score product's operand layout (lane l: key l % 16 of the quarter, dims 32 ks +
//     8 (l / 16) + 0..7); the next step's K loads go out once the score products have read
//     this step's, one after each 16-dim block of P.V;
//   * S^T of a quarter (16 keys x 16 columns) is one chain of eight v_mfma_f32_16x16x32_bf16
//     products; lane l then holds keys 4 (l / 16) + i of column l % 16 for both blocks, and
//     those eight values, a's four then b's four, are exactly the B operand (32 keys) of a
//     v_mfma_f32_16x16x32_bf16 P.V product whose A operand puts the same keys in the same
//     order: the transposing LDS reads (ds_read_b64_tr_b16) of the two blocks' V, side by side;
//   * V goes into LDS the same way (the transposing reads need it there), the next step's V
//     among the score products; each wave loads only its own 16 rows of every block, so the
//     walk needs no barrier;
//   * the column's row maximum and sum span the four lanes l % 16 + 16k: one
//     v_permlane16_swap and one v_permlane32_swap step;
//   * after the walk the four states are merged in LDS in wave order (M = max m_w,
//     a_w = 2^(m_w - M), l = sum a_w l_w, o = sum a_w O_w) and written as the segment's fp32
//     partial (m in log2 units), which prompt_merge_kernel combines over the segments in
//     order, with the float64 re-run of non-finite rows. A segment holding none of a row's
//     selected keys writes no partial for it (the merge applies the same rule).
// A row's bits depend only on its range, its selection, the absolute block and segment grid
// and the quarter split and pairing of the walk, never on the other rows of its call or on how
// the prompt is cut: the pairing is that of the row's own selection when the workgroup holds
// one row; with several rows (few query heads a key head) a block another row selected can
// change the pairing, within the tolerance of the fp32 sums.
#pragma once

#include "prompt_quarter.h"

namespace wa {

namespace {

constexpr int kRowCols = 16;           // (row, head) columns per workgroup

__device__ __forceinline__ int ctz64(uint64_t x) { return __builtin_ctzll(x); }

template <int NP>
__global__ __launch_bounds__(kThreads, 1) void prompt_rows_kernel(PromptArgs a, int nrg, int nhg, int nseg) {
    constexpr int D = 256;
    constexpr int KS = D / 32;             // 32-dim steps of S^T
    constexpr int DB = D / 16;             // 16-dim blocks of O^T
    constexpr int RB = 2 * D;              // bytes per V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPK = 1024 / RB;         // rows per 1 KiB wave load
    constexpr int TILE_B = BN * RB;        // bytes of one K (or V) tile
    constexpr int QL = 16 * RB / 1024;     // wave loads per quarter (each of K and V)
    constexpr int SEGB = kSparseSeg / kSparseBlock;   // blocks a segment (one or two mask words)
    static_assert(SEGB == 32 || SEGB == 64, "a segment is one or two whole mask words");
    static_assert(2 * QL == DB, "one V load after each 16-dim block of P.V (two quarters a step)");
    // K and V of the two blocks of a step, one stage each: block a in Ks[0] / Vs[0], b in
    // Ks[1] / Vs[1]; wave w owns rows 16w .. 16w + 15 of each (8 KiB an array)
    __shared__ __attribute__((aligned(1024))) char Ks[2][TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs[2][TILE_B];
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

    // Loads of a quarter (own 16 rows of block `tile`, K or V, into `dst`): 16 bytes a lane
    // straight into LDS (buffer_load ... lds / global_load_lds, issued by the lds_dma_* helpers
    // so that the waits below are the only ones on them: the compiler would otherwise make every
    // LDS read wait for all such loads in flight). A quarter with every key inside [kmin, kmax]
    // and no ring wrap goes by buffer loads from a descriptor on its first slot (no records:
    // zeros, for an absent block), an edge quarter key by key. Every quarter issues QL loads.
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
        return qb >= kmin && qb + 15 <= kmax && ring_slot(a, qb) + 16 <= a.ring;
    };
    auto qdesc = [&](const uint16_t* src, int tile, bool use) __attribute__((always_inline)) {
        const int sq = ring_slot(a, tile * BN + 16 * wave);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(src + (int64_t)sq * a.kv_sslot), (short)0,
                                                 use ? quarter_extent : 0, 0x00020000);
    };
    auto lds_base = [&](const char* dst) __attribute__((always_inline)) { return lds_addr(dst + 16 * RB * wave); };
    // a quarter key by key: key qb + r clamped into [kmin, kmax] and wrapped into the ring,
    // counted from the quarter's first key clamped into that range (every clamped key lies
    // 0 .. 15 keys after it: one wrap at most in a ring of at least 16 slots; a selected block
    // may hold quarters wholly below kmin or above kmax)
    auto issue_edge = [&](const uint16_t* src, int tile, const char* dst) __attribute__((always_inline)) {
        const int qb = tile * BN + 16 * wave;
        const int qbc = min(max(qb, kmin), kmax);
        const int sqc = ring_slot(a, qbc);
        int slot[QL];
#pragma unroll
        for (int i = 0; i < QL; ++i) slot[i] = sqc + (min(max(qb + RPK * i + ld_row, kmin), kmax) - qbc);
        if (a.ring >= 16) {
#pragma unroll
            for (int i = 0; i < QL; ++i) slot[i] = slot[i] >= a.ring ? slot[i] - a.ring : slot[i];
        } else {
#pragma unroll
            for (int i = 0; i < QL; ++i) slot[i] = min(max(qb + RPK * i + ld_row, kmin), kmax) % a.ring;
        }
        const uint32_t m0 = lds_base(dst);
#pragma unroll
        for (int i = 0; i < QL; ++i) {
            const int r = RPK * i + ld_row;
            const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
            lds_dma_global16(src + (int64_t)slot[i] * a.kv_sslot + 8 * c, m0 + 1024 * i);
        }
    };
    // a whole quarter now (`use` false: zeros)
    auto issue_quarter = [&](const uint16_t* src, int tile, bool use, const char* dst) __attribute__((always_inline)) {
        if (use && !is_fast(tile)) {
            issue_edge(src, tile, dst);
        } else {
            const __amdgpu_buffer_rsrc_t rs = qdesc(src, tile, use);
            const uint32_t m0 = lds_base(dst);
#pragma unroll
            for (int i = 0; i < QL; ++i) lds_dma_buffer16(rs, lane_off[i], m0 + 1024 * i);
        }
    };

    // the walk's first step: blocks a and b (b absent: zeros for its K and V, its scores masked)
    uint64_t rem = tiles;
    auto take = [&]() __attribute__((always_inline)) {
        const int t = tb0 + ctz64(rem);
        rem &= rem - 1;
        return t;
    };
    int ta = take();
    bool hb = rem != 0;
    int tb = hb ? take() : ta;
    issue_quarter(vg, ta, true, Vs[0]);
    issue_quarter(vg, tb, hb, Vs[1]);
    issue_quarter(kg, ta, true, Ks[0]);
    issue_quarter(kg, tb, hb, Ks[1]);

    // Q^T operand of the score product: lane l holds column l % 16 at dims 32 ks + 8 (l / 16)
    // + 0..7 (a padding column takes a valid row's q; its scores are never used)
    Pack8 qreg[KS];
    {
        const uint16_t* qp = a.q + (int64_t)(valid ? row : 0) * a.q_srow + (int64_t)head * a.q_shead + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks].u = *reinterpret_cast<const uint4*>(qp + 32 * ks);
    }
    // every load so far has landed: from here on the walk's own waits are the only ones
    __builtin_amdgcn_s_waitcnt(0);
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

    // LDS read offsets within a block's array. K (A operand of 16x16x32): row 16 wave + l % 16,
    // logical chunk 4 ks + l / 16. V^T (A operand of P.V) by the transposing read: 16-lane group
    // q4 reads rows 16 wave + 4 q4 + j / 4 at dims 16 db + 4 (j & 3) + 0..3 (j = lane % 16),
    // which gives lane l dim 16 db + l % 16 at keys 4 q4 + 0..3; blocks db and db + 8 differ by
    // 256 bytes
    int koff[KS], voff[DB / 2];
    {
        const int kr = 16 * wave + c16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 4 * ks + q4;
            koff[ks] = kr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(kr)));
        }
        const int vr = 16 * wave + 4 * q4 + (c16 >> 2);
#pragma unroll
        for (int db = 0; db < DB / 2; ++db) {
            const int c = 2 * db + ((c16 & 3) >> 1);
            voff[db] = vr * RB + 16 * (c ^ swz(vr)) + 8 * (c16 & 1);
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

    // One step over blocks (ta, tb). In flight at its start: this step's V (QL loads a quarter,
    // plus QL for each edge quarter), then its K (the same). V^T is read first, so that the
    // next step's V streams in while the score products run (one load after each of them;
    // descriptors with no records unless on the fast path, edge quarters key by key after
    // them); the next step's K goes out once the score products have read this step's, one
    // load after each 16-dim block of P.V (edge quarters after it).
    for (;;) {
        lds_dma_wait_vm16();               // this step's V (its K may still be in flight)
        uint2 vta[DB], vtb[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int off = voff[db & 7] + (db >> 3) * 256;
            vta[db] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vs[0] + off)));
            vtb[db] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vs[1] + off)));
        }
        lds_wait_reads();                  // V^T read: its stage may be refilled
        lds_dma_wait_vm0();                // this step's K
        const bool more = rem != 0;
        const int na = more ? take() : ta;
        const bool nhb = rem != 0;
        const int nb = nhb ? take() : na;
        const bool fva = more && is_fast(na), fvb = nhb && is_fast(nb);
        f32x4 sa, sb;
#pragma unroll
        for (int r = 0; r < 4; ++r) { sa[r] = 0.f; sb[r] = 0.f; }
        {
            const __amdgpu_buffer_rsrc_t rva = qdesc(vg, na, fva), rvb = qdesc(vg, nb, fvb);
            const uint32_t mva = lds_base(Vs[0]), mvb = lds_base(Vs[1]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Pack8 ka, kb;
                ka.u = *reinterpret_cast<const uint4*>(Ks[0] + koff[ks]);
                kb.u = *reinterpret_cast<const uint4*>(Ks[1] + koff[ks]);
                sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.v, qreg[ks].v, sa, 0, 0, 0);
                lds_dma_buffer16(rva, lane_off[ks], mva + 1024 * ks);
                sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb.v, qreg[ks].v, sb, 0, 0, 0);
                lds_dma_buffer16(rvb, lane_off[ks], mvb + 1024 * ks);
            }
            if (more && !fva) issue_edge(vg, na, Vs[0]);
            if (nhb && !fvb) issue_edge(vg, nb, Vs[1]);
            lds_wait_reads();              // K read: its stage may be refilled
        }
        // online softmax over keys 16w + 4 q4 + 0..3 of blocks a (x[0..3]) and b (x[4..7])
        float x[8];
        {
            const int kba = ta * BN + 16 * wave + 4 * q4, kbb = tb * BN + 16 * wave + 4 * q4;
            const bool sela = (eff >> (ta - tb0)) & 1;
            const bool selb = hb && ((eff >> (tb - tb0)) & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = (sela & (kba + i >= lo) & (kba + i <= last)) ? sa[i] : -INFINITY;
                x[4 + i] = (selb & (kbb + i >= lo) & (kbb + i <= last)) ? sb[i] : -INFINITY;
            }
        }
        const float smax = col_max(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
        const float m_cand = fmaxf(m_run, smax * cexp);
        const bool grow = m_cand > m_run + kLazy;
        const float m_new = grow ? m_cand : m_run;
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
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
        // NP bf16 parts of P: the B operand, keys a 4 q4 + 0..3 then b 4 q4 + 0..3 of column l % 16
        uint32_t wh[4], wm[4], wl[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            wh[h] = cvt_pk_bf16(x[2 * h], x[2 * h + 1]);
            wm[h] = wl[h] = 0u;
            if (NP >= 2 && !(NP == 2 && WA_CONTROL == 6)) {
                const float e0 = x[2 * h] - lo_bf16(wh[h]), e1 = x[2 * h + 1] - hi_bf16(wh[h]);
                wm[h] = cvt_pk_bf16(e0, e1);
                if (NP == 3) wl[h] = cvt_pk_bf16(e0 - lo_bf16(wm[h]), e1 - hi_bf16(wm[h]));
            }
        }
        Pack8 ph, pm, pl;
        ph.u = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        pm.u = make_uint4(wm[0], wm[1], wm[2], wm[3]);
        pl.u = make_uint4(wl[0], wl[1], wl[2], wl[3]);
        const bool fka = more && is_fast(na), fkb = nhb && is_fast(nb);
        const __amdgpu_buffer_rsrc_t rka = qdesc(kg, na, fka), rkb = qdesc(kg, nb, fkb);
        const uint32_t mka = lds_base(Ks[0]), mkb = lds_base(Ks[1]);
        // O^T += V^T P^T: per 16-dim block, the two blocks' V^T side by side as one 32-key operand
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            Pack8 av;
            av.u = make_uint4(vta[db].x, vta[db].y, vtb[db].x, vtb[db].y);
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, ph.v, oacc[db], 0, 0, 0);
            if (NP >= 2) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, pm.v, oacc[db], 0, 0, 0);
            if (NP == 3) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, pl.v, oacc[db], 0, 0, 0);
            if (db < QL) lds_dma_buffer16(rka, lane_off[db], mka + 1024 * db);
            else lds_dma_buffer16(rkb, lane_off[db - QL], mkb + 1024 * (db - QL));
        }
        if (more && !fka) issue_edge(kg, na, Ks[0]);
        if (nhb && !fkb) issue_edge(kg, nb, Ks[1]);
        if (!more) break;
        ta = na;
        tb = nb;
        hb = nhb;
    }

    // merge of the four quarters' states: wave w stores its O into its own rows of Ks[0] (dims
    // 0..127) and Ks[1] (dims 128..255), column-major rows of 128 floats, the 16-byte chunk c of
    // column p at c ^ (p & 15)
    const float l_tot = col_sum(l_run);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d0 = 16 * db + 4 * q4;                  // dims d0 .. d0 + 3
        const int c = (d0 & 127) >> 2;
        float* ob = reinterpret_cast<float*>(Ks[d0 < 128 ? 0 : 1] + 16 * RB * wave) + c16 * 128;
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
    const char* const half = Ks[wave < 2 ? 0 : 1];        // dims 64w.. lie in this array
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
