// Prompt rows of windowed GQA attention on gfx950: MFMA tiled online softmax.
//
// Method: TensorFold pull request #1123, "window_attention at head dim 256", section
// "What this changes", Prompt, Window.p32 and promptRows(..., hi) bullets. Each row i sees
// keys [lo_i, last_i]; keys come in tiles at absolute positions; every tile folds into the
// running (m, l, O) of a row with one rescale; P enters P.V as one bf16 or, with p32, as
// bf16(P) followed by bf16(P - bf16(P)). A tile that holds none of a row's keys leaves that
// row's state exactly unchanged (alpha = 1, P = 0), so a row's bits depend only on its own
// key range and the absolute tile grid, never on how the prompt is cut into calls.
//
// gfx950 design (own, not the page's tensor-core layout):
//   * a workgroup holds 4 waves; each wave owns 32 (row, query head) pairs of one key head,
//     so the G query heads of a key head share every K/V tile (GQA folded into the MFMA N
//     dimension, rows x heads);
//   * v_mfma_f32_32x32x16_bf16 computes S^T = K Q^T (keys x pairs) and O^T += V^T P^T
//     (dims x pairs). With the transposed products every lane holds a single pair (lane % 32)
//     in all of S, P and O, so the row max, the rescale and the sum are lane-local plus one
//     exchange between the two lane halves;
//   * K tiles sit in LDS as [key][dim]; V tiles are transposed on their way into LDS
//     ([dim][key]) so both MFMA operands are 16-byte LDS reads; the tiles are double
//     buffered, the next tile's global loads are in flight while the current tile computes,
//     and there is one barrier per tile;
//   * the K rows of a tile are fed to the first MFMA in a permuted order so that the S^T
//     accumulator registers of a lane are, eight at a time, exactly the B operand (P^T) the
//     P.V MFMA needs for eight consecutive keys: no shuffles between the two products;
//   * tiles inside every pair's window skip the mask; tiles outside a wave's key range are
//     skipped by that wave; the O rescale is skipped when no row's maximum moved;
//   * the workgroup index is remapped so that each XCD (8 on MI355X, workgroups dealt out
//     round-robin) works through a contiguous range of (key head, row block) tiles, keeping
//     a key head's K/V stream in that XCD's L2.
#include "wa_common.h"

namespace wa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPairs = 32 * kWaves;   // (row, head) pairs per workgroup
constexpr int BN = 64;                // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

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

template <int D>
struct TileRegs {
    static constexpr int KV = BN * D / 8 / kThreads;   // 16-byte K chunks per thread
    static constexpr int VV = BN * D / 8 / kThreads;   // 16-byte V chunks per thread
    uint4 k[KV];
    uint4 v[VV];
};

template <int D, bool P32>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 1) void prompt_kernel(PromptArgs a, int nblk) {
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int KS = D + 8;      // K tile row stride (elements)
    constexpr int VS = BN + 8;     // V^T tile row stride (elements)
    constexpr int DC = D / 8;      // 16-byte chunks per key row
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t VT[2][D * VS];
    __shared__ int red_i[2][kWaves];

    // XCD-aware remap of the linear workgroup index
    const int total = gridDim.x;
    const int L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, extra = total & 7;
    const int logical = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + idx;
    const int g = logical / nblk;           // key head
    const int blk = logical % nblk;         // block of pairs

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

    const int big = 0x7FFFFFFF;
    int lo = big, last = -1;                // empty range for padding pairs
    if (valid) {
        const int p = a.p0 + row;
        lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
        last = p;
        if (a.hi) {
            int hv = a.hi[row];
            hv = hv < p ? p : (hv > a.p0 + a.n - 1 ? a.p0 + a.n - 1 : hv);
            last = hv;
        }
    }
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

    // Q^T operand: this lane's pair, dims 16*ks + 8*h + 0..7
    // A negative scale is carried by q's sign (exact), so the exponent factor is positive
    // and the row maximum of the raw scores gives the maximum of the scaled ones.
    Pack8 qreg[KSTEPS];
    {
        const uint16_t* qp = a.q + (int64_t)row * a.q_srow + (int64_t)head * a.q_shead + 8 * h;
        const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if (valid) qreg[ks].u = *reinterpret_cast<const uint4*>(qp + 16 * ks);
            else qreg[ks].u = make_uint4(0, 0, 0, 0);
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
    const int krow = sigma(col);            // K row this lane feeds to the S^T MFMA

    // this thread's share of a tile load: K row chunks (coalesced rows), V 4-key groups
    const int k_dc = tid % DC, k_kk0 = tid / DC;          // K: key k_kk0 + it*(kThreads/DC)
    constexpr int KSTRIDE = kThreads / DC;
    const int v_dc = tid % DC, v_kq0 = tid / DC;          // V: keys 4*(v_kq0 + it*KSTRIDE) + 0..3

    auto load_tile = [&](int tile, TileRegs<D>& r) {
        const int base = tile * BN;
        int sbase = base % a.ring;
#pragma unroll
        for (int it = 0; it < TileRegs<D>::KV; ++it) {
            const int kk = k_kk0 + it * KSTRIDE;
            const int j = base + kk;
            int s = sbase + kk;
            s = s >= a.ring ? s - a.ring : s;
            r.k[it] = make_uint4(0, 0, 0, 0);
            if (j >= kmin && j <= kmax)
                r.k[it] = *reinterpret_cast<const uint4*>(kg + (int64_t)s * a.kv_sslot + k_dc * 8);
        }
#pragma unroll
        for (int it = 0; it < TileRegs<D>::VV; ++it) {
            const int kk = 4 * v_kq0 + (it / 4) * 4 * KSTRIDE + (it % 4);
            const int j = base + kk;
            int s = sbase + kk;
            s = s >= a.ring ? s - a.ring : s;
            r.v[it] = make_uint4(0, 0, 0, 0);
            if (j >= kmin && j <= kmax)
                r.v[it] = *reinterpret_cast<const uint4*>(vg + (int64_t)s * a.kv_sslot + v_dc * 8);
        }
    };
    auto store_tile = [&](int buf, const TileRegs<D>& r) {
#pragma unroll
        for (int it = 0; it < TileRegs<D>::KV; ++it) {
            const int kk = k_kk0 + it * KSTRIDE;
            *reinterpret_cast<uint4*>(&Ks[buf][kk * KS + k_dc * 8]) = r.k[it];
        }
#pragma unroll
        for (int grp = 0; grp < TileRegs<D>::VV / 4; ++grp) {
            const int kk = 4 * v_kq0 + grp * 4 * KSTRIDE;
            const uint4* x = &r.v[grp * 4];
            const uint32_t w0[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
            const uint32_t w1[4] = {x[1].x, x[1].y, x[1].z, x[1].w};
            const uint32_t w2[4] = {x[2].x, x[2].y, x[2].z, x[2].w};
            const uint32_t w3[4] = {x[3].x, x[3].y, x[3].z, x[3].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // dims 2e and 2e+1 of keys kk..kk+3
                uint2 lo2, hi2;
                lo2.x = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
                lo2.y = __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u);
                hi2.x = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
                hi2.y = __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u);
                *reinterpret_cast<uint2*>(&VT[buf][(v_dc * 8 + 2 * e) * VS + kk]) = lo2;
                *reinterpret_cast<uint2*>(&VT[buf][(v_dc * 8 + 2 * e + 1) * VS + kk]) = hi2;
            }
        }
    };

    const int t0 = kmin / BN, t1 = kmax / BN;
    TileRegs<D> pre;
    load_tile(t0, pre);
    store_tile(0, pre);
    __syncthreads();

    for (int tile = t0; tile <= t1; ++tile) {
        const int buf = (tile - t0) & 1;
        const int base = tile * BN;
        const bool more = tile < t1;
        if (more) load_tile(tile + 1, pre);

        // this wave computes only if the tile meets its key range
        if (base <= w_kmax && base + BN - 1 >= w_kmin) {
            // S^T = K Q^T for two 32-key halves
            f32x16 sacc[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.f;
                const uint16_t* kp = &Ks[buf][(32 * mb + krow) * KS + 8 * h];
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    Pack8 av;
                    av.u = *reinterpret_cast<const uint4*>(kp + 16 * ks);
                    sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, qreg[ks].v, sacc[mb], 0, 0, 0);
                }
            }

            // online softmax; t = s * scale * log2(e) is formed inside the exponent's fma
            const bool full = base >= w_loall && base + BN - 1 <= w_lastall;
            if (!full) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kpos = base + 32 * mb + 16 * (r >> 3) + 8 * h + (r & 7);
                        if (kpos < lo || kpos > last) sacc[mb][r] = -INFINITY;
                    }
            }
            float smax = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[mb][r]);
            smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
            const float m_new = fmaxf(m_run, smax * cexp);
            const float mu = (m_new == -INFINITY) ? 0.f : m_new;
            float psum = 0.f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][r], cexp, -mu));
                    sacc[mb][r] = p;
                    psum += p;
                }
            if (__any(m_new != m_run)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            l_run += psum;
            m_run = m_new;

            // O^T += V^T P^T, four 16-key steps
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int mb = s >> 1, r0 = (s & 1) * 8;
                Pack8 phi, plo;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float p0 = sacc[mb][r0 + 2 * u], p1 = sacc[mb][r0 + 2 * u + 1];
                    phi.w[u] = cvt_pk_bf16(p0, p1);
                    if (P32) plo.w[u] = cvt_pk_bf16(p0 - lo_bf16(phi.w[u]), p1 - hi_bf16(phi.w[u]));
                }
#pragma unroll
                for (int db = 0; db < DBLK; ++db) {
                    Pack8 av;
                    av.u = *reinterpret_cast<const uint4*>(&VT[buf][(32 * db + col) * VS + 16 * s + 8 * h]);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, phi.v, oacc[db], 0, 0, 0);
                    if (P32)
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av.v, plo.v, oacc[db], 0, 0, 0);
                }
            }
        }
        if (more) store_tile(buf ^ 1, pre);
        __syncthreads();
    }

    // epilogue: O / l, one rounding to bf16
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
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

template <int D>
hipError_t launch_d(const PromptArgs& a, hipStream_t s) {
    const int G = a.hq / a.hkv;
    const int nblk = (int)(((int64_t)a.n * G + kPairs - 1) / kPairs);
    dim3 grid(nblk * a.hkv);
    if (a.p32) hipLaunchKernelGGL((prompt_kernel<D, true>), grid, dim3(kThreads), 0, s, a, nblk);
    else hipLaunchKernelGGL((prompt_kernel<D, false>), grid, dim3(kThreads), 0, s, a, nblk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prompt(const PromptArgs& a, hipStream_t s) {
    return a.d == 256 ? launch_d<256>(a, s) : launch_d<128>(a, s);
}

}  // namespace wa
