// Prompt rows of windowed GQA attention on gfx950: MFMA tiled online softmax.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Prompt, Window.p32 and promptRows(..., hi) bullets. Each row i sees
// keys [lo_i, last_i]; keys come in tiles at absolute positions; every tile folds into the
// running (m, l, O) of a row with one rescale; P enters P.V as one bf16 or, with p32, as
// bf16(P) followed by bf16(P - bf16(P)). A third mode carries P as three bf16 parts
// (hi, mid, lo: each part the bf16 rounding of what the earlier parts leave), whose sum is
// fp32's P exactly, so that P.V has fp32-accurate products on the bf16 matrix cores; this
// is the three-part 16-bit split of TensorFold pull request #1622 (review answer, "What
// changed"), applied to P. q needs no split here: it arrives as bf16, so its products with
// k are already exact and the scale multiplies the fp32 sum.
// A tile that holds none of a row's keys leaves that row's state exactly unchanged
// (alpha = 1, P = 0), so a row's bits depend only on its own key range and the absolute
// tile grid, never on how the prompt is cut into calls.
//
// gfx950 design (own, not the page's tensor-core layout):
//   * a workgroup holds 4 waves; each wave owns 32 (row, query head) pairs of one key head,
//     so the G query heads of a key head share every K/V tile (GQA folded into the MFMA N
//     dimension, rows x heads);
//   * v_mfma_f32_32x32x16_bf16 computes S^T = K Q^T (keys x pairs) and O^T += V^T P^T
//     (dims x pairs). With the transposed products every lane holds a single pair (lane % 32)
//     in all of S, P and O, so the row max, the rescale and the sum are lane-local plus one
//     exchange between the two lane halves;
//   * K and V tiles go from memory straight into LDS ([key][dim], 16-byte chunks swizzled),
//     by buffer loads with a per-tile descriptor on interior tiles; K fragments are 16-byte
//     LDS reads, V^T fragments come from the transposing LDS read (ds_read_b64_tr_b16); the
//     tiles are double buffered, the next tile's loads are in flight while the current tile
//     computes, and there is one barrier per tile; unsplit dense prompts at d = 128 walk the
//     tiles software-pipelined (tile t + 1's score MFMAs are issued before tile t's softmax,
//     K is fetched two tiles ahead and V one), with each tile's arithmetic unchanged;
//   * the K rows of a tile are fed to the first MFMA in a permuted order so that the S^T
//     accumulator registers of a lane are, eight at a time, exactly the B operand (P^T) the
//     P.V MFMA needs for eight consecutive keys: no shuffles between the two products;
//   * tiles inside every pair's window skip the mask; tiles outside a wave's key range are
//     skipped by that wave; the running maximum is lazy (it moves only when a tile's maximum
//     exceeds it by more than 2^8 in probability), so the O rescale runs on few tiles;
//   * the workgroup index is remapped so that each XCD (8 on MI355X, workgroups dealt out
//     round-robin) works through a contiguous range of (key head, row block) tiles, keeping
//     a key head's K/V stream in that XCD's L2;
// This kernel serves prompts at d = 128 (dense, windowed or not, and block-sparse); prompts at
// d = 256 take the quarter-tile kernel (prompt_quarter.h, dense) or the row-group kernel
// (prompt_sparse.h, block-sparse).
//
// This header holds the kernels; prompt_inst.hip instantiates them once per (head dim, parts
// of P), so that they compile in parallel, and prompt.hip holds the launcher.
#pragma once

#include "wa_common.h"
#include "rerun_f64.h"

namespace wa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPairs = 32 * kWaves;   // (row, head) pairs per workgroup
static_assert(kPairs == kPromptPairs, "the launcher sizes the grid with kPromptPairs");
constexpr int BN = 64;                // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;          // running-max slack in log2 units (p <= 256)

union Pack8 {
    bf16x8 v;
    uint4 u;
    uint32_t w[4];
};

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// M-index i of the S^T tile (0..31) -> key within the 32-key half-tile. Lane half h holds
// M-indices 8a + 4h + b (a, b in 0..3); this order makes its registers 8s..8s+7 the keys
// 16s + 8h + 0..7.
__device__ __forceinline__ int sigma(int i) {
    const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// First key of prompt row `row`: the window anchored on the row's own position (non-
// decreasing in the row).
__device__ __forceinline__ int prompt_lo(const PromptArgs& a, int row) {
    return a.window > 0 ? max(0, a.p0 + row - a.window + 1 - (WA_CONTROL == 2)) : 0;
}

// Key range [lo, last] of prompt row `row` (a valid row): the window anchored on the row's
// own position, the last key hi[row] clamped into [p0 + row, p0 + n - 1] or the position.
__device__ __forceinline__ void prompt_span(const PromptArgs& a, int row, int& lo, int& last) {
    const int p = a.p0 + row;
    lo = prompt_lo(a, row);
    last = p;
    if (a.hi && WA_CONTROL != 5) {
        const int hv = a.hi[row];
        last = hv < p ? p : (hv > a.p0 + a.n - 1 ? a.p0 + a.n - 1 : hv);
    }
}

// Both lane halves of a pair combined, on every lane, without an LDS round trip: the
// half-swap (v_permlane32_swap) leaves lanes l and l ^ 32 holding each other's value in one of
// its two results, and max / sum of the two results is the pair's (the same order of operands
// on both halves, so both lanes get the same bits).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = min(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = max(x, __shfl_xor(x, m, 64));
    return x;
}

// Chunk swizzle of the LDS tiles: 16-byte chunk c of row r sits at position
// c ^ swz(r) (low four bits). It makes the K reads of the S^T product (16 rows with
// distinct low bits) and the transposing V reads (4 consecutive rows x 4 chunks) fall on
// distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// 16 bytes per lane from a buffer descriptor straight into LDS (buffer_load_dwordx4 ... lds):
// lane i's bytes land at dst + 16 i.
// LDS loads issued as inline assembly (they write LDS only, no register): the compiler does not
// track them, so each wait on them is written out (lds_dma_wait_*, s_waitcnt before the results
// are read). M0 holds the wave's LDS destination; lane i's 16 bytes land at M0 + 16 i.
// Volatile statements keep their order among themselves; the waits below also order every
// memory access around them, so an LDS read and the load that refills its stage stay on either
// side of a wait.
__device__ __forceinline__ void lds_dma_buffer16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(m0), "s"(rsrc));
}
__device__ __forceinline__ void lds_dma_global16(const void* src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0));
}
// all but the last 16 (8) vector-memory loads have landed; all have
__device__ __forceinline__ void lds_dma_wait_vm16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }
__device__ __forceinline__ void lds_dma_wait_vm8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ void lds_dma_wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// every LDS read issued so far has returned
__device__ __forceinline__ void lds_wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// LDS address of a shared-memory pointer, uniform over the wave
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void_ptr)p);
}

// the same from a wave-uniform base address plus a 32-bit lane offset (global_load_lds, saddr
// form)
__device__ __forceinline__ void lds_dma_global16_s(const void* base, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(m0));
}

// Workgroup barrier that waits for this wave's LDS (and scalar) operations only: global loads
// still in flight stay in flight across it (__syncthreads would wait for them as well). The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int NP>
__global__ __launch_bounds__(kThreads, 2) void prompt_kernel(PromptArgs a, int nblk) {
    static_assert(D == 128, "prompts at d = 256 take prompt_quarter.h (dense) or prompt_sparse.h (block-sparse)");
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int RB = 2 * D;              // bytes per K/V row in LDS
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPK = 1024 / RB;         // rows per 1 KiB wave load
    constexpr int NQ = BN * RB / 1024;     // 1 KiB wave loads per tile (each of K and V)
    constexpr int TILE_B = BN * RB;        // bytes of one K (or V) tile
    // two stages of K and V tiles, as four distinct arrays so that the compiler can tell
    // the direct-to-LDS loads into one stage from the reads of the other
    __shared__ __attribute__((aligned(1024))) char Ks0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs0[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Ks1[TILE_B];
    __shared__ __attribute__((aligned(1024))) char Vs1[TILE_B];
    __shared__ int red_i[2][kWaves];
    __shared__ uint32_t red_sel[kWaves];

    // XCD-aware remap of the linear workgroup index (the hardware deals ids out to the 8 XCDs
    // in turn): XCD x takes a contiguous share of the logical ids (key head, block of pairs,
    // chunk), so one head's K/V stream stays in its L2.
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int per = total >> 3, extra = total & 7;
    const int logical = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
    const int cidx = logical % a.nchunk;    // key chunk of the workgroup's range (split mode)
    const int gb = logical / a.nchunk;
    const int g = gb / nblk;                // key head
    const int blk = gb % nblk;              // block of pairs

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;                // lane half
    const int col = lane & 31;              // pair within the wave
    const int G = a.hq / a.hkv;

    const int pair = blk * kPairs + wave * 32 + col;
    const int row = pair / G;
    const int head = g * G + pair % G;
    const bool valid = row < a.n;

    // Q^T operand: this lane's pair, dims 16*ks + 8*h + 0..7, loaded first and waited for at
    // the first barrier (zeros for a padding pair)
    Pack8 qreg[KSTEPS];
    {
        const uint16_t* qp = a.q + (int64_t)row * a.q_srow + (int64_t)head * a.q_shead + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (valid) qreg[ks].u = *reinterpret_cast<const uint4*>(qp + 16 * ks);
            else qreg[ks].u = make_uint4(0, 0, 0, 0);
        }
    }

    const int big = 0x7FFFFFFF;
    int lo = big, last = -1;                // empty range for padding pairs
    if (valid) prompt_span(a, row, lo, last);
    // key range of this wave, the range all its valid pairs see, and the workgroup range
    const int w_kmin = wave_min_i(lo);
    const int w_kmax = wave_max_i(last);
    const int w_loall = wave_max_i(valid ? lo : -1);
    const int w_lastall = wave_min_i(valid ? last : big);
    if (lane == 0) { red_i[0][wave] = w_kmin; red_i[1][wave] = w_kmax; }
    __syncthreads();
    int kmin = red_i[0][0], kmax = red_i[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) { kmin = min(kmin, red_i[0][w]); kmax = max(kmax, red_i[1][w]); }
    if (kmax < kmin) return;                // no valid pair in this workgroup
    // split mode: this workgroup takes the key chunk cidx of its range, at absolute
    // positions, and writes per-chunk partials that a merge combines in chunk order
    const bool split = a.nchunk > 1 || a.bm != nullptr;
    const int chunk = kmin / kPromptChunk + cidx;
    if (split) {
        kmin = max(kmin, chunk * kPromptChunk);
        kmax = min(kmax, chunk * kPromptChunk + kPromptChunk - 1);
        if (kmax < kmin) return;
    }
    const int t0 = kmin / BN, t1 = kmax / BN;

    // Block-sparse prompts (always split, so t1 - t0 < 6): bit i of `eff` says that tile
    // t0 + i is selected by this lane's row and meets its key range; the workgroup walks
    // only the union of its rows' tiles, a wave computes only its own union, and a lane
    // masks the tiles its row did not select.
    const bool sparse = a.bm != nullptr;
    uint32_t eff = 0, w_any = 0, w_every = 0, tiles = 0;
    if (sparse) {
        if (valid) {
            const uint32_t* brow = a.bm + (int64_t)row * a.bm_srow;
            for (int b = t0; b <= t1; ++b)
                if (block_selected(brow, a.bm_words, b) && BN * b <= last && BN * b + BN - 1 >= lo)
                    eff |= 1u << (b - t0);
        }
        w_any = eff;                        // tiles some lane of the wave needs
        w_every = valid ? eff : ~0u;        // tiles every valid lane of the wave selected
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            w_any |= (uint32_t)__shfl_xor((int)w_any, m, 64);
            w_every &= (uint32_t)__shfl_xor((int)w_every, m, 64);
        }
        if (lane == 0) red_sel[wave] = w_any;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tiles |= red_sel[w];
        if (tiles == 0) return;             // none of the workgroup's rows selected a tile here
    }
    // the i-th tile the workgroup walks, and how many
    auto tile_at = [&](int i) {
        if (!sparse) return t0 + i;
        uint32_t x = tiles;
        for (int k = 0; k < i; ++k) x &= x - 1;
        return x ? t0 + __builtin_ctz(x) : t1;     // past the last tile: a placeholder, unused
    };
    const int ntiles = sparse ? __builtin_popcount(tiles) : t1 - t0 + 1;

    // A negative scale is carried by q's sign (exact), so the exponent factor is positive and
    // the row maximum of the raw scores gives the maximum of the scaled ones.
    {
        const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qreg[ks].u.x ^= flip; qreg[ks].u.y ^= flip; qreg[ks].u.z ^= flip; qreg[ks].u.w ^= flip;
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;   // m in log2 units (scaled score)
    const float cexp = fabsf(a.scale) * kLog2e;

    const uint16_t* kg = a.k + (int64_t)g * a.kv_shead;
    const uint16_t* vg = a.v + (int64_t)g * a.kv_shead;

    // LDS read offsets (bytes within a tile), fixed for the whole key loop.
    // K for S^T: row 32*mb + sigma(col), logical chunk 2*ks + h.
    const int krow = sigma(col);
    int koff[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int c = 2 * ks + h;
        koff[ks] = krow * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(krow)));
    }
    // V for O^T via the transposing read: 16-lane group q = lane / 16, j = lane % 16 reads
    // row 16*s + 8*h + 4*u + j/4 at dims 32*db + 16*(q & 1) + 4*(j & 3) + 0..3.
    const int j16 = lane & 15, cg = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    int voff[2][DBLK];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int vr = 8 * h + 4 * u + (j16 >> 2);      // row within a 16-key step (s = 0)
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int c = 4 * db + cg;
            voff[u][db] = vr * RB + 16 * ((c & ~15) | ((c & 15) ^ swz(vr))) + 8 * (j16 & 1);
        }
    }

    // One wave load moves 1 KiB: RPK rows of CPR chunks; lane -> (row, stored chunk p),
    // fetching logical chunk p ^ swz(row) of key base + row (clamped into [kmin, kmax], so
    // every fetched key is one the ring holds; keys outside every window are masked).
    const int ld_row = lane / CPR, ld_p = lane % CPR;
    // Interior tiles (every key inside [kmin, kmax], no ring wrap inside the tile) take the
    // fast path: buffer loads straight into LDS from a descriptor whose base is the tile's
    // first slot (two scalar adds per tile), with the lane offsets computed once here.
    // Edge tiles clamp each key into [kmin, kmax] and wrap it per lane.
    uint32_t lane_off[NQ / kWaves];
#pragma unroll
    for (int i = 0; i < NQ / kWaves; ++i) {
        const int q = wave + kWaves * i;
        const int r = RPK * q + ld_row;
        const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
        lane_off[i] = (uint32_t)(r * a.kv_sslot + 8 * c) * 2u;
    }
    const int tile_extent = (int)((uint32_t)((BN - 1) * a.kv_sslot) * 2u + 2u * D);
    // LDS addresses of the four stages and the wave index, uniform (for the load's M0)
    const uint32_t mK0 = lds_addr(Ks0), mK1 = lds_addr(Ks1), mV0 = lds_addr(Vs0), mV1 = lds_addr(Vs1);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    auto mstage = [&](const char* p) __attribute__((always_inline)) {
        return p == Ks0 ? mK0 : p == Ks1 ? mK1 : p == Vs0 ? mV0 : mV1;
    };
    // loads of one tile of K (or V) into an LDS stage
    auto issue_half = [&](int tile, char* dst, const uint16_t* src) __attribute__((always_inline)) {
        const uint32_t mdst = mstage(dst);
        const int base = tile * BN;
        const int sbase = ring_slot(a, base);
        if (base >= kmin && base + BN - 1 <= kmax && sbase + BN <= a.ring) {
            const int64_t toff = (int64_t)sbase * a.kv_sslot;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + toff), (short)0, tile_extent, 0x00020000);
#pragma unroll
            for (int i = 0; i < NQ / kWaves; ++i) lds_dma_buffer16(rs, lane_off[i], mdst + 1024u * (uwave + kWaves * i));
            return;
        }
#pragma unroll
        for (int i = 0; i < NQ / kWaves; ++i) {
            const int q = wave + kWaves * i;
            const int r = RPK * q + ld_row;
            const int c = (ld_p & ~15) | ((ld_p & 15) ^ swz(r));
            const int jc = min(max(base + r, kmin), kmax);
            // jc - base < 64: a ring of at least one tile wraps at most once inside the tile,
            // a shorter ring (a small window over a short cache) may wrap several times
            int slot = sbase + (jc - base);
            if (a.ring >= BN) slot = slot >= a.ring ? slot - a.ring : slot;
            else slot = jc % a.ring;
            const int64_t off = (int64_t)slot * a.kv_sslot + 8 * c;
            lds_dma_global16_s(src, (uint32_t)(off * 2), mdst + 1024u * (uwave + kWaves * i));
        }
    };
    auto issue_tile = [&](int tile, char* kdst, char* vdst) __attribute__((always_inline)) {
        issue_half(tile, kdst, kg);
        issue_half(tile, vdst, vg);
    };

    // S^T of one tile into sacc (this wave's pairs; the tile must meet the wave's range)
    auto scores = [&](const char* kt, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
        // S^T = K Q^T for two 32-key halves
        // the two 32-key halves alternate, so each LDS read has two MFMAs to hide behind
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
        // K fragments are read two k-steps ahead of their MFMAs
        Pack8 ka[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            ka[ks][0].u = *reinterpret_cast<const uint4*>(kt + koff[ks]);
            ka[ks][1].u = *reinterpret_cast<const uint4*>(kt + 32 * RB + koff[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const Pack8 a0 = ka[ks & 1][0], a1 = ka[ks & 1][1];
            if (ks + 2 < KSTEPS) {
                ka[ks & 1][0].u = *reinterpret_cast<const uint4*>(kt + koff[ks + 2]);
                ka[ks & 1][1].u = *reinterpret_cast<const uint4*>(kt + 32 * RB + koff[ks + 2]);
            }
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0.v, qreg[ks].v, sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1.v, qreg[ks].v, sacc[1], 0, 0, 0);
        }
        // keep the reads two k-steps ahead in the instruction order: 4 reads, then
        // (2 MFMAs, 2 reads) pairs, then the last 4 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks + 2 < KSTEPS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    };
    // softmax of one tile's S^T (mask, lazy running maximum, exponentials, row sum, O rescale)
    // and its P.V into O
    // softmax head of one tile: mask (unless every pair sees the whole tile), the tile's
    // maximum against the lazy running maximum, p = 2^(t - m) into sacc, and the row sum
    struct Soft {
        float m_new, mu, psum;
        bool grow;
    };
    auto is_full = [&](int tile) __attribute__((always_inline)) {
        const int base = tile * BN;
        const uint32_t tbit = sparse ? 1u << (tile - t0) : 0u;
        return base >= w_loall && base + BN - 1 <= w_lastall && (!sparse || (w_every & tbit));
    };
    auto soft_head = [&](int tile, f32x16 (&sacc)[2], bool full) __attribute__((always_inline)) {
        const int base = tile * BN;
        const uint32_t tbit = sparse ? 1u << (tile - t0) : 0u;
        // online softmax; t = s * scale * log2(e) is formed inside the exponent's fma
        const bool lsel = !sparse || (eff & tbit);
        if (!full) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kpos = base + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
                    if (kpos < lo || kpos > last || !lsel) sacc[mb][r] = -INFINITY;
                }
        }
        float smax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[mb][r]);
        smax = pair_max(smax);
        // lazy maximum: m moves only when the tile's maximum exceeds it by more than
        // kLazy (log2 units), so p <= 2^kLazy and most tiles need no rescale of O
        Soft sf;
        const float m_cand = fmaxf(m_run, smax * cexp);
        sf.grow = m_cand > m_run + kLazy;
        sf.m_new = sf.grow ? m_cand : m_run;
        sf.mu = (sf.m_new == -INFINITY) ? 0.f : sf.m_new;
        sf.psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r], cexp, -sf.mu));
                sacc[mb][r] = p;
                sf.psum += p;
            }
        return sf;
    };
    // softmax tail and P.V: O rescale when the maximum moved, l and m, then O += P V
    auto soft_tail = [&](const Soft& sf, f32x16 (&sacc)[2], const char* vt) __attribute__((always_inline)) {
        const bool grow = sf.grow;
        const float mu = sf.mu, psum = sf.psum, m_new = sf.m_new;
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

        // O^T += V^T P^T, four 16-key steps; V^T comes from the transposing LDS read, one step
        // ahead of its MFMAs (two register stages of V^T fragments)
        uint2 vx[2][DBLK][2];
        auto read_v = [&](int s, uint2 (&dst)[DBLK][2]) __attribute__((always_inline)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    dst[db][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_ptr)(vt + 16 * s * RB + voff[u][db])));
        };
        read_v(0, vx[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s + 1 < 4) read_v(s + 1, vx[(s + 1) & 1]);
            const int mb = s >> 1, r0 = (s & 1) * 8;
            // NP bf16 parts of P: part k is the bf16 rounding of P minus parts 0..k-1 (each
            // difference exact in fp32)
            Pack8 phi, pmid, plo;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = sacc[mb][r0 + 2 * u], p1 = sacc[mb][r0 + 2 * u + 1];
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
                av.w[0] = vx[s & 1][db][0].x;
                av.w[1] = vx[s & 1][db][0].y;
                av.w[2] = vx[s & 1][db][1].x;
                av.w[3] = vx[s & 1][db][1].y;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, phi.v, oacc[db], 0, 0, 0);
                if (NP >= 2)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, pmid.v, oacc[db], 0, 0, 0);
                if (NP == 3)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, plo.v, oacc[db], 0, 0, 0);
            }
        }
    };
    auto finish = [&](int tile, f32x16 (&sacc)[2], const char* vt) __attribute__((always_inline)) {
        const Soft sf = soft_head(tile, sacc, is_full(tile));
        soft_tail(sf, sacc, vt);
    };
    // does the tile meet this wave's key range (and, sparse, its rows' selection)?
    auto meets = [&](int tile) __attribute__((always_inline)) {
        const int base = tile * BN;
        const uint32_t tbit = sparse ? 1u << (tile - t0) : 0u;
        return base <= w_kmax && base + BN - 1 >= w_kmin && (!sparse || (w_any & tbit));
    };

    // one tile: start the next tile's loads into the other stage, compute on this stage,
    // then wait for the loads and meet at the barrier
    auto step = [&](int tile, const char* kt, const char* vt, char* knext, char* vnext, bool more,
                    int next) {
        if (more) issue_tile(next, knext, vnext);
        if (meets(tile)) {
            f32x16 sacc[2];
            scores(kt, sacc);
            finish(tile, sacc, vt);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // unsplit dense prompts (the long ones) walk their tiles software-pipelined
    const bool piped = !split && !sparse;
    if (piped) {
        // A software-pipelined walk. While tile t's
        // softmax runs on the VALU, tile t + 1's scores are already on the matrix cores; K is
        // fetched two tiles ahead and V one. K(t) and V(t) sit in stage (t - t0) & 1. The
        // arithmetic of every tile is step's, so the bits are the same.
        f32x16 sa[2], sb[2];
        // iteration t: K(t + 2) replaces K(t) (its scores were taken last iteration), V(t + 1)
        // replaces V(t - 1); then scores(t + 1) and finish(t)
        auto iter = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2], char* kc, const char* kn,
                        const char* vc, char* vn) __attribute__((always_inline)) {
            if (t + 2 <= t1) issue_half(t + 2, kc, kg);
            if (t + 1 <= t1) issue_half(t + 1, vn, vg);
            if (t + 1 <= t1 && meets(t + 1)) scores(kn, nxt);
            if (meets(t)) finish(t, cur, vc);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        issue_half(t0, Ks0, kg);
        issue_half(t0, Vs0, vg);
        if (t0 + 1 <= t1) issue_half(t0 + 1, Ks1, kg);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (meets(t0)) scores(Ks0, sa);
        __syncthreads();                    // K(t0) read by every wave before K(t0 + 2) lands
        for (int t = t0; t <= t1; t += 2) {
            iter(t, sa, sb, Ks0, Ks1, Vs0, Vs1);
            if (t + 1 <= t1) iter(t + 1, sb, sa, Ks1, Ks0, Vs1, Vs0);
        }
    } else {
        issue_tile(tile_at(0), Ks0, Vs0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int i = 0; i < ntiles; i += 2) {
            step(tile_at(i), Ks0, Vs0, Ks1, Vs1, i + 1 < ntiles, tile_at(i + 1));
            if (i + 1 < ntiles) step(tile_at(i + 1), Ks1, Vs1, Ks0, Vs0, i + 2 < ntiles, tile_at(i + 2));
        }
    }

    // epilogue: O / l, one rounding to bf16; in split mode the chunk's (m, l, O) partial
    const float l_tot = pair_sum(l_run);
    if (split) {
        // the partial of a chunk holding at least one of the row's keys (sparse: of its
        // selected blocks); the merge reads exactly these
        if (valid && lo <= chunk * kPromptChunk + kPromptChunk - 1 && last >= chunk * kPromptChunk &&
            (!sparse || eff != 0)) {
            const int64_t pi = ((int64_t)row * a.hq + head) * a.Cp + (chunk - lo / kPromptChunk);
            if (h == 0) { a.pm[pi] = m_run; a.pl[pi] = l_tot; }
            float* op = a.po + pi * D;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d0 = 32 * db + 8 * q4 + 4 * h;
                    *reinterpret_cast<float4*>(op + d0) =
                        make_float4(oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]);
                }
        }
        return;
    }
    if (valid) {
        uint16_t* op = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = 32 * db + 8 * q4 + 4 * h;
                uint2 w;
                w.x = pack_bf16x2(oacc[db][4 * q4 + 0] / l_tot, oacc[db][4 * q4 + 1] / l_tot);
                w.y = pack_bf16x2(oacc[db][4 * q4 + 2] / l_tot, oacc[db][4 * q4 + 3] / l_tot);
                *reinterpret_cast<uint2*>(op + d0) = w;
            }
    }
}

// Merge of the split prompt's chunk partials: M = max m_c over the chunks of the row's range,
// a_c = 2^(m_c - M) (m is in log2 units), out = bf16(sum a_c o_c / sum a_c l_c), both sums
// fma chains in chunk order. One wave per (row, head): lane c holds chunk c's (m, l), lane i
// dims DL*i .. DL*i + DL - 1. (row, head)s with a non-finite output are listed and re-run in
// float64 afterwards by the whole workgroup.
constexpr int kMergePairs = 4;     // = waves of a D = 256 workgroup; D = 128 loops twice

template <int D>
__global__ __launch_bounds__(D) void prompt_merge_kernel(PromptArgs a) {
    constexpr int W = D / 64;             // waves
    constexpr int DL = D / 64;            // dims per lane
    __shared__ int flagged[kMergePairs];
    __shared__ int nflag;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t npairs = (int64_t)a.n * a.hq;
    const int64_t first = (int64_t)blockIdx.x * kMergePairs;
    if (t == 0) nflag = 0;
    __syncthreads();
    for (int i = wave; i < kMergePairs; i += W) {
        const int64_t pr = first + i;
        if (pr >= npairs) break;
        const int row = (int)(pr / a.hq), head = (int)(pr % a.hq);
        int lo, last;
        prompt_span(a, row, lo, last);
        const int CK = a.chunk_keys;
        int nc = last / CK - lo / CK + 1;
        nc = nc > a.Cp ? a.Cp : nc;
        const int64_t pi = pr * a.Cp;     // (row * hq + head) * Cp
        // Does chunk c (of the row's range) hold one of the row's keys? Every chunk of a
        // dense range does; a sparse row's chunk only through a selected block that meets
        // [lo, last] -- the rule the prompt kernel writes partials by.
        const uint32_t* brow = a.bm ? a.bm + (int64_t)row * a.bm_srow : nullptr;
        // The blocks that meet [lo, last] are lo / 64 .. last / 64; the chunk's share of them,
        // b0 .. b1, is tested a mask word at a time.
        auto present = [&](int c) {
            if (c >= nc) return false;
            if (!brow) return true;
            const int nb = CK / kSparseBlock;
            const int c0 = (lo / CK + c) * nb;
            const int b0 = max(c0, lo / kSparseBlock), b1 = min(c0 + nb - 1, last / kSparseBlock);
            for (int w = b0 >> 5; w <= (b1 >> 5) && w < a.bm_words; ++w) {
                const int s = max(b0 - 32 * w, 0), e = min(b1 - 32 * w, 31);
                if (s <= e && (brow[w] & (0xFFFFFFFFu >> (31 - e)) & (0xFFFFFFFFu << s))) return true;
            }
            return false;
        };
        const float* op = a.po + pi * D + DL * lane;
        // eight chunks' o at a time, chunk c0 + j from chunk c0 (j < cnt, present ones)
        auto load8 = [&](float (&o)[8][DL], int c0, int cnt, uint64_t inmask) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < cnt && ((inmask >> j) & 1)) {
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
        // chunks in blocks of 64, lane c of a block holding chunk (m, l); the first block's
        // (m, l) and its first eight chunks' o are requested together with the mask words
        // that tell which are present (slots of absent chunks hold stale values, never used)
        float o[8][DL];
        load8(o, 0, min(nc, 8), ~0ull);
        const bool inr = lane < nc;
        const float mr = inr ? a.pm[pi + lane] : -INFINITY;
        const float lr = inr ? a.pl[pi + lane] : 0.f;
        const bool in0 = present(lane);
        const uint64_t inmask0 = __ballot(in0);
        const float m0 = in0 ? mr : -INFINITY;
        const float l0 = in0 ? lr : 0.f;
        float M = fmaxf(-INFINITY, m0);
        for (int cb = 64; cb < nc; cb += 64)
            M = fmaxf(M, present(cb + lane) ? a.pm[pi + cb + lane] : -INFINITY);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
        float num[DL], den = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) num[e] = 0.f;
        for (int cb = 0; cb < nc; cb += 64) {
            const bool in = cb == 0 ? in0 : present(cb + lane);
            const float ac = __builtin_amdgcn_exp2f((cb == 0 ? m0 : (in ? a.pm[pi + cb + lane] : -INFINITY)) - M);
            const float lc = cb == 0 ? l0 : (in ? a.pl[pi + cb + lane] : 0.f);
            const uint64_t inmask = cb == 0 ? inmask0 : __ballot(in);
            const int ce = min(nc - cb, 64);
            // eight chunks' o loads in flight at a time, then their fmas in chunk order
            for (int cg = 0; cg < ce; cg += 8) {
                if (cb + cg > 0) load8(o, cb + cg, ce - cg, inmask >> cg);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (cg + j < ce && ((inmask >> (cg + j)) & 1)) {
                        const float ac_c = __shfl(ac, cg + j, 64);
                        const float l_c = __shfl(lc, cg + j, 64);
#pragma unroll
                        for (int e = 0; e < DL; ++e) num[e] = fmaf(ac_c, o[j][e], num[e]);
                        den = fmaf(ac_c, l_c, den);
                    }
                }
            }
        }
        uint16_t* orow = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead;
        uint32_t b[DL];
        bool bad = false;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            b[e] = f32_to_bf16_rne(num[e] / den);
            bad = bad || bf16_nonfinite((uint16_t)b[e]);
        }
        if constexpr (DL == 4) {
            *reinterpret_cast<uint2*>(orow + DL * lane) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
        } else {
            *reinterpret_cast<uint32_t*>(orow + DL * lane) = b[0] | (b[1] << 16);
        }
        if (__any(bad) && lane == 0) flagged[atomicAdd(&nflag, 1)] = i;
    }
    __syncthreads();
    const int nf = nflag;
    for (int f = 0; f < nf; ++f) {
        const int64_t pr = first + flagged[f];
        const int row = (int)(pr / a.hq), head = (int)(pr % a.hq);
        int lo, last;
        prompt_span(a, row, lo, last);
        uint16_t* orow = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead;
        const int64_t kv = (int64_t)(head / (a.hq / a.hkv)) * a.kv_shead;
        rerun_f64<D>(a.q + (int64_t)row * a.q_srow + (int64_t)head * a.q_shead, a.k + kv, a.v + kv,
                     a.kv_sslot, a.ring, lo, last, a.scale, orow,
                     a.bm ? a.bm + (int64_t)row * a.bm_srow : nullptr, a.bm_words);
        __syncthreads();
    }
}

// Unsplit prompts: find the (row, head)s whose bf16 output holds a NaN or an infinity and
// re-run each of them alone in float64; every other (row, head) is only read. A workgroup
// scans kCheckPairs consecutive (row, head)s, 4 bf16 a lane, then re-runs the flagged ones
// one after the other with all its threads.
constexpr int kCheckPairs = 64;

template <int D>
__global__ __launch_bounds__(D) void prompt_check_kernel(PromptArgs a) {
    constexpr int TPP = D / 4;            // lanes per (row, head): 4 bf16 each
    constexpr int PPI = D / TPP;          // (row, head)s per pass of the workgroup
    __shared__ int flagged[kCheckPairs];
    __shared__ int nflag;
    const int t = threadIdx.x;
    const int64_t npairs = (int64_t)a.n * a.hq;
    const int64_t first = (int64_t)blockIdx.x * kCheckPairs;
    if (t == 0) nflag = 0;
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < kCheckPairs / PPI; ++it) {
        const int local = it * PPI + t / TPP;
        const int64_t pr = first + local;
        bool bad = false;
        if (pr < npairs) {
            const int row = (int)(pr / a.hq), head = (int)(pr % a.hq);
            const uint2 w = *reinterpret_cast<const uint2*>(
                a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead + 4 * (t % TPP));
            bad = bf16_nonfinite(w.x & 0xFFFFu) || bf16_nonfinite(w.x >> 16) ||
                  bf16_nonfinite(w.y & 0xFFFFu) || bf16_nonfinite(w.y >> 16);
        }
        // OR over the TPP lanes of each (row, head); TPP divides the wave
        const unsigned long long b = __ballot(bad);
        const int sub = (t & 63) / TPP;
        const unsigned long long m = TPP == 64 ? ~0ull : (((1ull << TPP) - 1) << (sub * TPP));
        if ((b & m) != 0 && t % TPP == 0) flagged[atomicAdd(&nflag, 1)] = local;
    }
    __syncthreads();
    const int nf = nflag;
    for (int i = 0; i < nf; ++i) {
        const int64_t pr = first + flagged[i];
        const int row = (int)(pr / a.hq), head = (int)(pr % a.hq);
        uint16_t* orow = a.out + (int64_t)row * a.o_srow + (int64_t)head * a.o_shead;
        int lo, last;
        prompt_span(a, row, lo, last);
        const int64_t kv = (int64_t)(head / (a.hq / a.hkv)) * a.kv_shead;
        rerun_f64<D>(a.q + (int64_t)row * a.q_srow + (int64_t)head * a.q_shead, a.k + kv, a.v + kv,
                     a.kv_sslot, a.ring, lo, last, a.scale, orow);
        __syncthreads();
    }
}

// Launch of the main kernel <D, NP> on a grid of `grid` workgroups (defined by the file that
// instantiates it).
template <int D, int NP>
hipError_t launch_main(const PromptArgs& b, int nblk, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((prompt_kernel<D, NP>), dim3(grid), dim3(kThreads), 0, s, b, nblk);
    return hipGetLastError();
}

// The kernel after the main one: the chunk merge of split prompts, else the non-finite check.
template <int D>
hipError_t launch_post(const PromptArgs& a, hipStream_t s) {
    const int64_t npairs = (int64_t)a.n * a.hq;
    if (a.nchunk > 1 || a.bm)
        hipLaunchKernelGGL((prompt_merge_kernel<D>), dim3((unsigned)((npairs + kMergePairs - 1) / kMergePairs)),
                           dim3(D), 0, s, a);
    else
        hipLaunchKernelGGL((prompt_check_kernel<D>), dim3((unsigned)((npairs + kCheckPairs - 1) / kCheckPairs)),
                           dim3(D), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace wa
